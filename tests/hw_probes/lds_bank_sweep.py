"""Time the LDS read probe (tests/hw_probes/jas_hw_probes.hip, lds_read) over
row strides, to find the strides at which a 16-byte read by lanes spread
over 16 rows is free of bank conflicts on gfx950.  Run it under
`rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS` for the conflict counts;
alone it prints each pattern's time from HIP events.  A measurement, not a
test: the attention kernel's LDS row strides are chosen from its result.
"""
import ctypes
import os
import sys

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjas_hw_probes.so")
PATTERNS = [(rs, 16) for rs in range(16, 400, 16)] + [(272, 32), (288, 64), (80, 32)]


def main():
    L = ctypes.CDLL(LIB)
    L.probe_lds_read.restype = ctypes.c_int
    L.probe_lds_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
    blocks, iters = 1024, 2000
    out = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    for rs, gs in PATTERNS:
        if L.probe_lds_read(out.data_ptr(), blocks, rs, gs, 10, ctypes.c_void_p(st.cuda_stream)):
            sys.exit("probe_lds_read rejected its arguments")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        L.probe_lds_read(out.data_ptr(), blocks, rs, gs, iters, ctypes.c_void_p(st.cuda_stream))
        b.record(st)
        torch.cuda.synchronize()
        print(f"row stride {rs:4d} B ({rs % 64:2d} mod 64), group stride {gs:3d} B: "
              f"{a.elapsed_time(b) * 1e3:8.1f} us", flush=True)


if __name__ == "__main__":
    main()
