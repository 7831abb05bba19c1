"""Benchmark: fixed-order row softmax forward + backward on one MI355X.

Default workload: joint image+text attention scores, bf16 [1, 24, 4352, 4352]
(4,096 image + 256 text keys per row, 104,448 rows), per-batch text-padding
mask, forward then backward on the forward's P.  One step = jas_fwd +
jas_bwd over the whole tensor, inputs resident in HBM.

Reported: algorithmic bytes moved per second (fwd reads scores and writes P,
bwd reads P and dP and writes dS: 5 x 2 bytes per element) and rows/s,
per-kernel HIP-event durations, the roofline fraction of the dominant kernel
against MI355X's 8 TB/s, and the CPU oracle timed on a bounded sample of the
same rows on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c2|c5]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "fwd+bwd softmax HBM GB/s and rows/s (bf16, 4,352 keys) vs 8 TB/s roofline"

WORKLOADS = {
    # name: (description, B, H, S, N, dtype, mask, sink, causal, backward)
    "c3": ("joint image+text attention scores bf16 [1,24,4352,4352], per-batch text padding mask, fwd+bwd",
           1, 24, 4352, 4352, "bf16", True, False, False, True),
    "c2": ("bf16 scores 16384 rows x 4352 keys, N(0,1) with x8 outliers on 0.1%, fwd only",
           1, 1, 16384, 4352, "bf16", False, False, False, False),
    "c5": ("causal self-attention scores bf16 [1,32,8192,8192] + per-head sink, fwd+bwd",
           1, 32, 8192, 8192, "bf16", False, True, True, True),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-check", action="store_true", help="skip the parity check before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU oracle sample")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(wl, dev):
    import torch
    import synth
    _, B, H, S, N, dt, has_mask, has_sink, causal, _ = WORKLOADS[wl]
    mask = sink = g = None
    if wl == "c3":
        s, mask, g, _ = synth.c3_inputs(seed=3, device=dev, B=B, H=H, S=S, N=N)
        mask = mask.view(B, 1, 1, N)
    elif wl == "c2":
        s = synth.c2_scores(seed=2, device=dev, rows=S, N=N)
    else:
        s, sink, g = synth.c5_inputs(seed=5, device=dev, B=B, H=H, S=S)
    return s, mask, sink, g


def check_parity(wl, s, mask, sink, g):
    """Sampled rows against the oracle before timing (forward within 1 bf16
    ulp; backward stage-isolated on the oracle's P, bit-exact)."""
    import torch
    import deterministic_attention_softmax_amd as jas
    import oracle
    import synth
    _, B, H, S, N, _, _, _, _, backward = WORKLOADS[wl]
    rows = B * H * S
    idx = np.unique(np.random.default_rng(7).choice(rows, 32, replace=False))
    it = torch.as_tensor(idx, device=s.device)
    P, ps = jas.fwd(s, mask=mask, sink=sink)
    s_rows = synth.to_numpy_bits(s.reshape(-1, N).index_select(0, it))
    m_rows = None
    if mask is not None:
        m_rows = np.ascontiguousarray(mask.reshape(B, N).cpu().numpy()[idx // (H * S)])
    sig = None if sink is None else np.ascontiguousarray(sink.cpu().numpy()[(idx // S) % H])
    k = len(idx)
    P_o, ps_o = oracle.fwd(s_rows.reshape(1, k, 1, N), 1, k, 1, N, mask=m_rows,
                           mask_strides=(0, N, 0), sink=sig)
    P_g = synth.to_numpy_bits(P.reshape(-1, N).index_select(0, it)).reshape(P_o.shape)
    ulp = int(np.max(np.abs(P_g.astype(np.int32) - P_o.astype(np.int32))))
    assert ulp <= 1, f"forward parity: {ulp} bf16 ulp"
    if not backward:
        return {"fwd_max_ulp": ulp}
    # backward on the oracle's P at the sampled rows
    P.reshape(-1, N).index_copy_(0, it, synth.from_numpy_bits(P_o.reshape(k, N), s.device))
    if ps is not None:
        ps[it] = torch.from_numpy(ps_o).to(s.device)
    dS, _ = jas.bwd(P, g, p_sink=ps)
    g_rows = synth.to_numpy_bits(g.reshape(-1, N).index_select(0, it))
    dS_o, _ = oracle.bwd(P_o, g_rows.reshape(P_o.shape), 1, k, 1, N,
                         p_sink=None if ps is None else ps_o)
    dS_g = synth.to_numpy_bits(dS.reshape(-1, N).index_select(0, it)).reshape(dS_o.shape)
    assert np.array_equal(dS_g, dS_o), "backward parity: dS not bit-exact"
    return {"fwd_max_ulp": ulp, "bwd_bitexact": True}


def cpu_baseline(wl, s, mask, sink, g, target_s):
    """The oracle, as it stands, on a bounded sample of the same rows."""
    import oracle
    import synth
    _, B, H, S, N, _, _, _, _, backward = WORKLOADS[wl]
    threads = oracle.default_threads()
    esz = 2

    def run(k):
        rows = np.arange(k)
        s_rows = synth.to_numpy_bits(s.reshape(-1, N)[:k])
        m_rows = None if mask is None else np.ascontiguousarray(
            mask.reshape(B, N).cpu().numpy()[rows // (H * S)])
        sig = None if sink is None else np.ascontiguousarray(sink.cpu().numpy()[(rows // S) % H])
        g_rows = synth.to_numpy_bits(g.reshape(-1, N)[:k]) if backward else None
        t0 = time.perf_counter()
        P, ps = oracle.fwd(s_rows.reshape(1, k, 1, N), 1, k, 1, N, mask=m_rows,
                           mask_strides=(0, N, 0), sink=sig, threads=threads)
        if backward:
            oracle.bwd(P, g_rows.reshape(P.shape), 1, k, 1, N, p_sink=ps, threads=threads)
        return time.perf_counter() - t0

    k0 = min(256, B * H * S)
    t0 = run(k0)
    k = int(min(B * H * S, max(k0, k0 * target_s / max(t0, 1e-3))))
    t = run(k)
    per_elem = (5 if backward else 2) * esz
    return {
        "value": round(k * N * per_elem / t / 1e9, 4), "unit": "GB/s",
        "rows_per_s": round(k / t, 1), "cores": threads, "kind": "oracle",
        "sample": f"first {k} rows of the same workload ({k * N} elements), "
                  f"{'fwd+bwd' if backward else 'fwd'}, {t:.1f} s wall",
    }


def copy_ceiling(nbytes, stream, steps=10):
    """A plain 16-byte copy of `nbytes` (the dominant kernel's bytes: half
    read, half written) with the test-only probe kernel, if it is built: the
    attainable read+write bandwidth on this machine."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "tests", "hw_probes", "libjas_hw_probes.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.probe_copy16.restype = ctypes.c_int
    L.probe_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    n16 = max(1, nbytes // 32)
    src = torch.empty(n16 * 16, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for nt in (0, 1):
        for _ in range(3):
            L.probe_copy16(src.data_ptr(), dst.data_ptr(), n16, nt, 0, stream.cuda_stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            L.probe_copy16(src.data_ptr(), dst.data_ptr(), n16, nt, 0, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out["nontemporal" if nt else "plain"] = round(2 * n16 * 16 / (ms * 1e-3) / 1e9, 1)
    return {"unit": "GB/s", "bytes": 2 * n16 * 16, **out}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import deterministic_attention_softmax_amd as jas
    jas.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    wl = args.workload
    desc, B, H, S, N, dt, has_mask, has_sink, causal, backward = WORKLOADS[wl]
    rows, E = B * H * S, B * H * S * N
    esz = 2
    log(f"workload {wl}: {desc}")
    s, mask, sink, g = make_inputs(wl, dev)
    torch.cuda.synchronize()

    check = None
    if not args.no_check:
        check = check_parity(wl, s, mask, sink, g)
        log(f"parity check: {check}")

    P = torch.empty_like(s)
    dS = torch.empty_like(s) if backward else None
    ps = torch.empty(rows, dtype=torch.float32, device=dev) if has_sink else None
    dsk = torch.empty(H, dtype=torch.float32, device=dev) if has_sink else None
    ws = torch.empty(max(4, rows * 4 + 256), dtype=torch.uint8, device=dev) if has_sink else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        jas.fwd(s, mask=mask, sink=sink, out=P, p_sink=ps)
        if ev:
            ev[1].record(stream)
        if backward:
            jas.bwd(P, g, p_sink=ps, out=dS, d_sink=dsk, workspace=ws)
        if ev:
            ev[2].record(stream)

    # bring clocks and page mappings to steady state (untimed, before the
    # warmup steps proper)
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    bwd_ms = np.array([b.elapsed_time(c) for _, b, c in evs]) if backward else np.zeros(1)
    step_ms = wall * 1e3 / args.steps

    fwd_bytes = 2 * esz * E + (E // N * 4 if has_sink else 0)
    bwd_bytes = 3 * esz * E + (E // N * 12 if has_sink else 0) if backward else 0
    total_bytes = fwd_bytes + bwd_bytes
    gbs = total_bytes / (step_ms * 1e-3) / 1e9
    fwd_gbs = fwd_bytes / (fwd_ms.mean() * 1e-3) / 1e9
    bwd_gbs = bwd_bytes / (bwd_ms.mean() * 1e-3) / 1e9 if backward else None
    dom = ("jas bwd", bwd_gbs, bwd_bytes, bwd_ms.mean()) if backward else \
          ("jas fwd", fwd_gbs, fwd_bytes, fwd_ms.mean())
    log(f"fwd {fwd_ms.mean():.3f} ms ({fwd_gbs:.0f} GB/s)" +
        (f", bwd {bwd_ms.mean():.3f} ms ({bwd_gbs:.0f} GB/s)" if backward else "") +
        f", step {step_ms:.3f} ms")

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": desc, "batch": B, "heads": H, "q_rows": S, "keys": N,
                   "rows": rows, "mask": has_mask, "sink": has_sink, "backward": backward},
        "rows_per_s": round(rows / (step_ms * 1e-3), 1),
        "fwd_ms": round(float(fwd_ms.mean()), 4), "fwd_gbs": round(fwd_gbs, 1),
        "bwd_ms": round(float(bwd_ms.mean()), 4) if backward else None,
        "bwd_gbs": round(bwd_gbs, 1) if backward else None,
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": round(dom[1], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom[1] / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": dom[2],
                     "avg_launch_ms": round(float(dom[3]), 4)},
        "parity": check,
    }
    out["copy_ceiling"] = copy_ceiling(dom[2], stream)
    if out["copy_ceiling"]:
        best = max(out["copy_ceiling"]["plain"], out["copy_ceiling"]["nontemporal"])
        out["roofline"]["frac_of_copy"] = round(dom[1] / best, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(wl, s, mask, sink, g, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
