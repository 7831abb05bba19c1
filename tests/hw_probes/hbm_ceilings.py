"""Attainable HBM rates of simple streaming kernels on this GPU
(tests/hw_probes/jas_hw_probes.hip, stream_mix): copy (1 read, 1 write),
2 reads and 1 write (the softmax backward's mix) and read-only, 16-byte
nontemporal accesses, 1 GiB per array, over a few grid sizes and chunks in
flight per thread.  Prints each configuration and the best of each mix.
A measurement that the softmax kernels' rates are read against, not a test.
"""
import ctypes
import os

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjas_hw_probes.so")
MIXES = {0: ("copy (1R+1W)", 2), 1: ("2R+1W", 3), 2: ("read only", 1)}


def main():
    L = ctypes.CDLL(LIB)
    L.probe_stream_mix.restype = ctypes.c_int
    L.probe_stream_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    b = torch.full((n // 4,), 2, dtype=torch.int32, device="cuda")
    d = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    best = {}
    for mix, (name, arrays) in MIXES.items():
        for blocks in (1024, 2048, 4096):
            for chunks in (1, 2, 4):
                args = (a.data_ptr(), b.data_ptr(), d.data_ptr(), n // 16, mix, chunks, blocks, sp)
                assert L.probe_stream_mix(*args) == 0
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(10):
                    L.probe_stream_mix(*args)
                e1.record(st)
                torch.cuda.synchronize()
                gbs = arrays * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
                best[name] = max(best.get(name, 0.0), gbs)
                print(f"{name:13s} grid {blocks:5d} chunks {chunks}: {gbs:7.1f} GB/s", flush=True)
    for name, gbs in best.items():
        print(f"best {name}: {gbs:.1f} GB/s", flush=True)


if __name__ == "__main__":
    main()
