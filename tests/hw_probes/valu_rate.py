"""Issue rate of v_exp_f32 and v_mul_f32 on the GPU (tests/hw_probes/
jas_hw_probes.hip, valu_rate): 8 independent chains per lane, 4096
workgroups of 256 threads, registers only.  Prints lane-operations per
SIMD per cycle at the MI355X clock of 2.4 GHz (1024 SIMDs).  A
measurement behind the fused attention kernel's VALU budget, not a test.
"""
import ctypes
import os

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjas_hw_probes.so")


def main():
    L = ctypes.CDLL(LIB)
    L.probe_valu_rate.restype = ctypes.c_int
    L.probe_valu_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    blocks, iters = 4096, 2000
    out = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    for op, name in ((0, "v_exp_f32"), (1, "v_mul_f32")):
        assert L.probe_valu_rate(out.data_ptr(), blocks, op, 10, ctypes.c_void_p(st.cuda_stream)) == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        L.probe_valu_rate(out.data_ptr(), blocks, op, iters, ctypes.c_void_p(st.cuda_stream))
        b.record(st)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        ops = blocks * 256 * iters * 128
        rate = ops / (1024 * ms * 1e-3 * 2.4e9)
        print(f"{name}: {ms:.3f} ms, {rate:.2f} lane-operations per SIMD per cycle "
              f"({64 / rate:.1f} cycles per wave64 instruction)", flush=True)


if __name__ == "__main__":
    main()
