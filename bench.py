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

Other workloads: joint4352_keylen (the padding as key lengths, padded keys
not read), rows4352 (forward only), causal8192 (causal scores, -inf above the
diagonal, read like any other key), causal8192_skip (the same scores with
the causal flag: nothing above the diagonal is read) and long65536 (rows of
65,536 keys through the streaming kernels).  With keys excluded,
the algorithmic bytes count the scores and P of the visible keys only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30  # timed steps touch at least this many bytes of buffers
METRIC = "fwd+bwd softmax HBM GB/s and rows/s (bf16, 4,352 keys) vs 8 TB/s roofline"

WORKLOADS = {
    # name: (description, B, H, S, N, dtype, mask, sink, exclusion, backward); exclusion is
    # None (every key read), "causal" (JAS_FLAG_CAUSAL) or "key_len" (JAS_FLAG_KEY_LEN)
    "joint4352": ("joint image+text attention scores bf16 [1,24,4352,4352], per-batch text padding mask, fwd+bwd",
           1, 24, 4352, 4352, "bf16", True, False, None, True),
    "joint4352_keylen": ("joint image+text attention scores bf16 [1,24,4352,4352], text padding as per-batch "
                         "key lengths (keys past them not read), fwd+bwd",
           1, 24, 4352, 4352, "bf16", False, False, "key_len", True),
    "rows4352": ("bf16 scores 16384 rows x 4352 keys, N(0,1) with x8 outliers on 0.1%, fwd only",
           1, 1, 16384, 4352, "bf16", False, False, None, False),
    "causal8192": ("causal self-attention scores bf16 [1,32,8192,8192] + per-head sink, -inf scores above "
                   "the diagonal read like any other, fwd+bwd",
           1, 32, 8192, 8192, "bf16", False, True, None, True),
    "causal8192_skip": ("causal self-attention scores bf16 [1,32,8192,8192] + per-head sink, causal flag "
                        "(scores and P above the diagonal not read), fwd+bwd",
           1, 32, 8192, 8192, "bf16", False, True, "causal", True),
    "long65536": ("long-context rows bf16 [1,16,512,65536] (512 queries at the end of 65,536 keys), "
                  "causal flag, streaming kernels, fwd+bwd",
           1, 16, 512, 65536, "bf16", False, False, "causal", True),
}


# fused attention forward (jas_attn_fwd): name: (description, B, H, Hkv, S, N, D, mask, causal, sink)
ATTN_WORKLOADS = {
    "attn4352": ("fused attention forward bf16 q/k/v [1,24,4352,128] (joint image+text shape), "
                 "per-batch text padding mask", 1, 24, 24, 4352, 4352, 128, True, False, False),
    "attn8192_causal": ("fused attention forward bf16 q/k/v [1,32,8192,128], causal flag, "
                        "per-head sink", 1, 32, 32, 8192, 8192, 128, False, True, True),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0

# Seeds of every synthetic input, recorded in each result line.  One seed
# draws a workload's scores, mask and dP (synth/ derives the streams from it);
# the parity check's row sample has its own.
SEEDS = {"joint4352": 3, "joint4352_keylen": 3, "rows4352": 2, "causal8192": 5,
         "causal8192_skip": 5, "long65536": 7}
ATTN_SEEDS = {"q": 81, "k": 82, "v": 83, "sink": 84, "mask": 3}
CHECK_SEED = 7


def row_kends(wl, key_len):
    """Visible keys of every row (int64 [B*H*S]): the causal condition
    key <= N - S + q and the batch entry's key length, clamped to [0, N]."""
    _, B, H, S, N, _, _, _, excl, _ = WORKLOADS[wl]
    k = np.full((B, H, S), N, np.int64)
    if excl == "causal":
        k = np.minimum(k, (np.arange(S) + (N - S) + 1)[None, None, :])
    if excl == "key_len":
        k = np.minimum(k, np.asarray(key_len, np.int64)[:, None, None])
    return np.clip(k, 0, N).reshape(-1)


CSRC = os.path.join(ROOT, "deterministic_attention_softmax_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """sha256 over the sources of the row-softmax kernels and of the host
    code that picks their instance and geometry (every .h / .hip / .cpp file
    of csrc/ except the fused attention's jas_attn.hip and jas_attn.h, in
    name order): a traffic record is only used while it still matches."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip", ".cpp")) and name not in ("jas_attn.hip", "jas_attn.h"):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def attn_source_hash():
    """sha256 over the fused attention's sources (jas_attn.hip, the headers
    it includes and the host code that picks its launch), for its traffic
    records."""
    import hashlib
    h = hashlib.sha256()
    for name in ("jas_attn.hip", "jas_attn.h", "jas_internal.h", "jas_kernels.h", "jas_api.cpp"):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_attn_traffic(wl):
    """HBM bytes per fused attention call from the committed PMC record, or
    None when there is none or the sources changed since."""
    path = traffic_record_path(wl)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("attn_source_sha256") != attn_source_hash():
        return None
    return int(rec["call"]["hbm_bytes_per_call"])


def traffic_record_path(wl):
    return os.path.join(PROFILES, f"pmc_traffic_jas_{wl}.json")


def load_traffic(wl, kernel):
    """HBM bytes per launch of `kernel` ("fwd"/"bwd") from the committed PMC
    record, or None when there is none or the kernels changed since."""
    path = traffic_record_path(wl)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["hbm_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="joint4352",
                    choices=sorted(WORKLOADS) + sorted(ATTN_WORKLOADS))
    ap.add_argument("--no-check", action="store_true", help="skip the parity check before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--attn-query-blocks", type=int, default=0, choices=(0, 1, 2),
                    help="fused attention: 16-query blocks per wavefront (0 = library default)")
    ap.add_argument("--json-out", metavar="PATH", help="also write the result line to PATH")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarise rocprofv3 output under DIR (trace/, fetch/, write/) into profiles/")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(wl, dev):
    import torch
    import synth
    _, B, H, S, N, dt, has_mask, has_sink, excl, _ = WORKLOADS[wl]
    mask = sink = g = key_len = None
    seed = SEEDS[wl]
    if wl.startswith("joint4352"):
        s, mask, g, pads = synth.joint_attention_bf16(seed=seed, device=dev, B=B, H=H, S=S, N=N)
        mask = mask.view(B, 1, 1, N)
        if excl == "key_len":
            mask = None
            key_len = torch.tensor([N - p for p in pads], dtype=torch.int32, device=dev)
    elif wl == "rows4352":
        s = synth.rows_with_outliers_bf16(seed=seed, device=dev, rows=S, N=N)
    elif wl == "long65536":
        s, g = synth.long_context_bf16(seed=seed, device=dev, B=B, H=H, S=S, N=N)
    else:
        s, sink, g = synth.causal_sink_bf16(seed=seed, device=dev, B=B, H=H, S=S)
    return s, mask, sink, g, key_len


def oracle_row_mask(wl, mask, kend, idx):
    """fp32 [k, N] additive mask for rows `idx` handed to the oracle as
    independent rows: the workload's mask row plus -inf past the row's
    visible keys (the oracle treats an excluded key exactly as a -inf one)."""
    _, B, H, S, N, _, _, _, excl, _ = WORKLOADS[wl]
    m = np.zeros((len(idx), N), np.float32)
    if mask is not None:
        m += mask.reshape(B, N).cpu().numpy()[idx // (H * S)]
    if excl is not None:
        m[np.arange(N)[None, :] >= kend[idx][:, None]] = -np.inf
    return m


def check_parity(wl, s, mask, sink, g, key_len):
    """Sampled rows against the oracle before timing (forward within 1 bf16
    ulp; backward stage-isolated on the oracle's P, bit-exact)."""
    import torch
    import deterministic_attention_softmax_amd as jas
    import oracle
    import synth
    _, B, H, S, N, _, _, _, excl, backward = WORKLOADS[wl]
    causal = excl == "causal"
    rows = B * H * S
    kend = row_kends(wl, None if key_len is None else key_len.cpu().numpy())
    idx = np.unique(np.random.default_rng(CHECK_SEED).choice(rows, 32, replace=False))
    it = torch.as_tensor(idx, device=s.device)
    P, ps = jas.fwd(s, mask=mask, sink=sink, causal=causal, key_len=key_len)
    s_rows = synth.to_numpy_bits(s.reshape(-1, N).index_select(0, it))
    m_rows = oracle_row_mask(wl, mask, kend, idx) if (mask is not None or excl) else None
    sig = None if sink is None else np.ascontiguousarray(sink.cpu().numpy()[(idx // S) % H])
    k = len(idx)
    P_o, ps_o = oracle.fwd(s_rows.reshape(1, k, 1, N), 1, k, 1, N, mask=m_rows,
                           mask_strides=(0, N, 0), sink=sig)
    P_g = synth.to_numpy_bits(P.reshape(-1, N).index_select(0, it)).reshape(P_o.shape)
    ulp = int(np.max(np.abs(P_g.astype(np.int32) - P_o.astype(np.int32))))
    assert ulp <= 1, f"forward parity: {ulp} bf16 ulp"
    if not backward:
        return {"fwd_max_ulp": ulp}
    # backward on the oracle's P at the sampled rows (+0 past the visible keys)
    P.reshape(-1, N).index_copy_(0, it, synth.from_numpy_bits(P_o.reshape(k, N), s.device))
    if ps is not None:
        ps[it] = torch.from_numpy(ps_o).to(s.device)
    dS, _ = jas.bwd(P, g, p_sink=ps, causal=causal, key_len=key_len)
    g_rows = synth.to_numpy_bits(g.reshape(-1, N).index_select(0, it))
    dS_o, _ = oracle.bwd(P_o, g_rows.reshape(P_o.shape), 1, k, 1, N,
                         p_sink=None if ps is None else ps_o)
    dS_g = synth.to_numpy_bits(dS.reshape(-1, N).index_select(0, it)).reshape(dS_o.shape)
    assert np.array_equal(dS_g, dS_o), "backward parity: dS not bit-exact"
    return {"fwd_max_ulp": ulp, "bwd_bitexact": True}


def check_invariance(wl, run0, set0, s, mask, sink, g, key_len, ps, dsk):
    """Byte identity before timing (RL-Kernel PR #240, Acceptance Criteria:
    bitwise batch invariance; RL-Kernel PR #453, Benchmark: bytes checked
    before timing).  The outputs of the prepared calls the timed steps make
    are compared with: the same calls again (repeat), the binding's wrapper
    calls (wrapper), a grid capped at 997 workgroups that loop over the rows
    (capped_grid), and one head's rows computed as their own call of batch
    1 x 1 head (sub_batch)."""
    import torch
    import deterministic_attention_softmax_amd as jas
    _, B, H, S, N, _, _, _, excl, backward = WORKLOADS[wl]
    causal = excl == "causal"
    rf, rb = run0
    _, _, P, dS = set0

    def snap():
        torch.cuda.synchronize()
        return (P.clone(), dS.clone() if backward else None,
                None if ps is None else ps.clone(), None if dsk is None else dsk.clone())

    def same(x, y):
        return x is None and y is None or torch.equal(x.view(torch.uint8), y.view(torch.uint8))

    def agree(ref, got, sel=slice(None)):
        return all(same(None if r is None else r[sel], None if t is None else t[sel])
                   for r, t in zip(ref, got))

    def wrapped(launch=None, si=s, gi=g, sk=sink):
        r = jas.fwd(si, mask=mask, sink=sk, causal=causal, key_len=key_len, launch=launch)
        Pw, psw = r[0], r[1]
        dSw = dskw = None
        if backward:
            dSw, dskw = jas.bwd(Pw, gi, p_sink=psw, causal=causal, key_len=key_len, launch=launch)
        torch.cuda.synchronize()
        return Pw, dSw, psw, dskw

    rf()
    if backward:
        rb()
    ref = snap()
    rf()
    if backward:
        rb()
    res = {"repeat": agree(ref, snap())}
    res["wrapper"] = agree(ref, wrapped())
    res["capped_grid"] = agree(ref, wrapped(launch=(0, 0, 0, 997, 0)))
    h0 = H // 2  # one head of the B = 1 workloads: its rows, in order, as a call of its own
    one = wrapped(si=s[:, h0:h0 + 1].contiguous(), gi=g[:, h0:h0 + 1].contiguous() if backward else None,
                  sk=None if sink is None else sink[h0:h0 + 1].contiguous())
    sub = (ref[0][:, h0:h0 + 1], None if ref[1] is None else ref[1][:, h0:h0 + 1],
           None if ref[2] is None else ref[2].view(B, H, S)[:, h0:h0 + 1].reshape(-1),
           None if ref[3] is None else ref[3][h0:h0 + 1])
    res["sub_batch"] = B == 1 and all(
        same(None if a is None else a.contiguous(), b) for a, b in zip(sub, one))
    assert all(res.values()), f"outputs not byte-identical: {res}"
    return res


def cpu_baseline(wl, s, mask, sink, g, key_len, target_s):
    """The oracle, as it stands, on a bounded sample of the same rows: k rows
    spread evenly over the whole tensor, each handed to the oracle as its own
    batch entry (its mask row, and its visible length as that entry's key
    length when keys are excluded), one oracle call per head so that each
    call has one sink logit."""
    import oracle
    import synth
    _, B, H, S, N, _, _, _, excl, backward = WORKLOADS[wl]
    affinity, share, share_from = host_cpus()
    threads = max(1, min(affinity, share))
    esz = 2
    kend = row_kends(wl, None if key_len is None else key_len.cpu().numpy())
    m_all = None if mask is None else mask.reshape(B, N).cpu().numpy()
    sk_all = None if sink is None else sink.cpu().numpy()
    s2, g2 = s.reshape(-1, N), (g.reshape(-1, N) if backward else None)

    def run(k, threads=threads):
        rows = np.unique(np.linspace(0, B * H * S - 1, k).round().astype(np.int64))
        heads = (rows // S) % H
        t = 0.0
        for h in np.unique(heads):
            r = rows[heads == h]
            n = len(r)
            it = torch_index(r, s.device)
            s_rows = synth.to_numpy_bits(s2.index_select(0, it))
            g_rows = synth.to_numpy_bits(g2.index_select(0, it)) if backward else None
            m_rows = None if m_all is None else np.ascontiguousarray(m_all[r // (H * S)])
            sig = None if sk_all is None else sk_all[h:h + 1]
            kl = None if excl is None else np.ascontiguousarray(kend[r].astype(np.int32))
            t0 = time.perf_counter()
            P, ps = oracle.fwd(s_rows.reshape(n, 1, 1, N), n, 1, 1, N, mask=m_rows,
                               mask_strides=(N, 0, 0), sink=sig, threads=threads, key_len=kl)
            if backward:
                oracle.bwd(P, g_rows.reshape(P.shape), n, 1, 1, N, p_sink=ps, threads=threads,
                           key_len=kl)
            t += time.perf_counter() - t0
        vis = int(kend[rows].sum())
        nbytes = esz * (vis + len(rows) * N) + (esz * (vis + 2 * len(rows) * N) if backward else 0)
        return t, len(rows), nbytes

    k0 = min(512, B * H * S)
    t0, _, _ = run(k0)
    k = int(min(B * H * S, max(k0, k0 * target_s / max(t0, 1e-3))))
    t, k, nbytes = run(k)
    # the same oracle on one thread, on a sample of about a fifth of the time
    t1p, _, _ = run(k0, threads=1)
    k1 = int(min(B * H * S, max(k0, k0 * (target_s / 5) / max(t1p, 1e-3))))
    t1, k1, nbytes1 = run(k1, threads=1)
    return {
        "value": round(nbytes / t / 1e9, 4), "unit": "GB/s",
        "rows_per_s": round(k / t, 1), "cores": threads, "kind": "oracle",
        "affinity_cores": affinity, "cpu_share": share, "cpu_share_from": share_from,
        "sample": f"{k} rows spread evenly over the whole workload ({k * N} elements), "
                  f"{'fwd+bwd' if backward else 'fwd'}, {t:.1f} s of oracle time",
        "cpu_model": cpu_model(),
        "one_thread": {"value": round(nbytes1 / t1 / 1e9, 4), "unit": "GB/s",
                       "rows_per_s": round(k1 / t1, 1),
                       "sample": f"{k1} rows spread evenly, {t1:.1f} s of oracle time"},
    }


def host_cpus():
    """(cores in this process's affinity mask, the CPU share granted to the
    process, where that share comes from).  The share is the cgroup's CPU
    quota when one is set, else OMP_NUM_THREADS, else the affinity count:
    on a shared host the affinity mask can list every core of the machine
    while the job is granted only a slice of them, and threads beyond the
    slice only queue."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            return affinity, max(1, int(int(quota) // int(period))), "cgroup cpu.max"
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        return affinity, int(omp), "OMP_NUM_THREADS"
    return affinity, affinity, "affinity"


def cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def torch_index(idx, device):
    import torch
    return torch.as_tensor(idx, device=device)


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "tests", "hw_probes", "libjas_hw_probes.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.probe_copy16.restype = ctypes.c_int
    L.probe_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    L.probe_read2_write1.restype = ctypes.c_int
    L.probe_read2_write1.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return L


def _time_launch(launch, stream, steps):
    import torch
    for _ in range(3):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def copy_ceiling(nbytes, stream, steps=10):
    """Attainable rates of simple 16-byte streams moving `nbytes` (the
    dominant kernel's bytes) with the test-only probe kernels, if built: a
    copy (one read, one write per word: the forward's mix; also the
    calibration point of the HBM byte counters) and two reads with one
    write (the backward's mix), each with normal and nontemporal cache
    policy and at several grid sizes; the best of each is reported.  Like the
    timed steps, successive launches rotate over enough buffer sets to touch
    ROTATE_BYTES, so a small stream is not served from the Infinity Cache."""
    import torch
    L = _probe_lib()
    if L is None:
        return None
    out = {"unit": "GB/s"}
    sets = max(1, -(-ROTATE_BYTES // max(1, nbytes)))
    out["buffer_sets"] = sets

    def rotating(launch_on):  # launch_on(i) launches on buffer set i
        k = [0]

        def launch():
            launch_on(k[0] % sets)
            k[0] += 1
        return launch

    def grids(n16):  # persistent grids, and one workgroup per 1,024 words (a whole pass)
        return sorted({1024, 2048, 8192, 16384, max(1, -(-n16 // 1024))})

    n16 = max(1, nbytes // 32)
    src = [torch.empty(n16 * 16, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    dst = [torch.empty_like(x) for x in src]
    for nt in (0, 1):
        best = 0.0
        for blocks in grids(n16):
            ms = _time_launch(rotating(lambda i: L.probe_copy16(src[i].data_ptr(), dst[i].data_ptr(),
                                                                n16, nt, blocks, stream.cuda_stream)),
                              stream, max(steps, sets))
            best = max(best, 2 * n16 * 16 / (ms * 1e-3) / 1e9)
        out["nontemporal" if nt else "plain"] = round(best, 1)
    out["bytes"] = 2 * n16 * 16
    del src, dst
    n16 = max(1, nbytes // 48)
    a = [torch.empty(n16 * 16, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    b = [torch.empty_like(x) for x in a]
    d = [torch.empty_like(x) for x in a]
    best = 0.0
    for nt in (0, 1):
        for blocks in grids(n16):
            ms = _time_launch(rotating(lambda i: L.probe_read2_write1(
                a[i].data_ptr(), b[i].data_ptr(), d[i].data_ptr(), n16, nt, blocks, stream.cuda_stream)),
                stream, max(steps, sets))
            best = max(best, 3 * n16 * 16 / (ms * 1e-3) / 1e9)
    out["r2w1"] = round(best, 1)
    out["r2w1_bytes"] = 3 * n16 * 16
    return out


def _kernel_kind(name):
    if "fwd_kernel" in name or "fwd_stream_kernel" in name:
        return "fwd"
    if "bwd_kernel" in name or "bwd_stream_kernel" in name:
        return "bwd"
    if "dsink_kernel" in name:
        return "dsink"
    if "copy16<true>" in name:
        return "copy_nt"
    if "copy16<false>" in name:
        return "copy"
    return None


def summarize_profiles(prof_dir, wl):
    """Write profiles/kernel_trace_jas_<wl>.md and pmc_traffic_jas_<wl>.{md,json}
    from rocprofv3 CSV output (see the commands recorded in them)."""
    import csv
    desc = WORKLOADS[wl][0]
    os.makedirs(PROFILES, exist_ok=True)
    trace = os.path.join(prof_dir, "trace", f"{wl}_kernel_stats.csv")
    bench_log = os.path.join(prof_dir, "trace", "bench_line.json")
    rows = list(csv.DictReader(open(trace)))
    line = json.load(open(bench_log)) if os.path.exists(bench_log) else None
    out = [f"# rocprofv3 kernel trace: jas kernels, workload {wl}", "",
           f"Workload: {desc}.", "",
           "Command (repository root, MI355X, ROCm 7.2):", "",
           "```",
           f"rocprofv3 --kernel-trace --stats --output-format csv -d {prof_dir}/trace -o {wl} -- "
           f"python3 bench.py --workload {wl} --steps 10 --warmup 3 --no-cpu-baseline "
           f"--json-out {prof_dir}/trace/bench_line.json",
           "```", "",
           "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    avg = {}
    for r in rows:
        kind = _kernel_kind(r["Name"])
        if kind is None:
            continue
        name = re.sub(r"\([^()]*\)$", "", r["Name"]).replace("void ", "")
        a = float(r["AverageNs"]) / 1e3
        avg[kind] = a
        out.append(f"| `{name}` | {r['Calls']} | {a:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} |")
    if line:
        out += ["", "The same run's bench.py line (HIP events on the launch stream):", "",
                f"- fwd average {line['fwd_ms'] * 1e3:.1f} us ({line['fwd_gbs']} GB/s)"]
        if line.get("bwd_ms"):
            out.append(f"- bwd average {line['bwd_ms'] * 1e3:.1f} us ({line['bwd_gbs']} GB/s)")
        out.append(f"- fwd+bwd {line['value']} GB/s, {line['ms_per_step']} ms per step")
    open(os.path.join(PROFILES, f"kernel_trace_jas_{wl}.md"), "w").write("\n".join(out) + "\n")

    # PMC: FETCH_SIZE / WRITE_SIZE in KiB per dispatch, calibrated on the copy
    # kernel of known size that bench.py runs in the same process
    counters = {}
    for cname, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        path = os.path.join(prof_dir, sub, f"{wl}_counter_collection.csv")
        for r in csv.DictReader(open(path)):
            kind = _kernel_kind(r["Kernel_Name"])
            if kind is None or r["Counter_Name"] != cname:
                continue
            counters.setdefault((kind, cname), []).append(float(r["Counter_Value"]) * 1024.0)
    line_pmc = json.load(open(os.path.join(prof_dir, "fetch", "bench_line.json")))
    copy_bytes = line_pmc["copy_ceiling"]["bytes"] / 2  # read = written = half the moved bytes
    fac = {c: copy_bytes / np.mean(counters[("copy", c)]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    E = WORKLOADS[wl][1] * WORKLOADS[wl][2] * WORKLOADS[wl][3] * WORKLOADS[wl][4]
    V = int(line_pmc["config"].get("visible_keys", E))  # keys read of scores / P
    alg = {"fwd": (2 * V, 2 * E), "bwd": (2 * V + 2 * E, 2 * E)}
    rec = {"workload": wl, "kernel_source_sha256": kernel_source_hash(),
           "calibration": {"copy_bytes_read": copy_bytes, "copy_bytes_written": copy_bytes,
                           "fetch_factor": round(fac["FETCH_SIZE"], 4),
                           "write_factor": round(fac["WRITE_SIZE"], 4)},
           "kernels": {}}
    md = [f"# rocprofv3 HBM traffic: jas kernels, workload {wl}", "",
          f"Workload: {desc}.", "", "Commands (repository root):", "", "```"]
    for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        md.append(f"rocprofv3 --pmc {c} --output-format csv -d {prof_dir}/{sub} -o {wl} -- "
                  f"python3 bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --no-check "
                  f"--json-out {prof_dir}/{sub}/bench_line.json")
    md += [f"python3 bench.py --workload {wl} --summarize-profiles {prof_dir}", "```", "",
           "Counters are KiB per dispatch.  Each is scaled by what it reads for the 16-byte copy "
           f"kernel of known size in the same process ({copy_bytes / 1e6:.1f} MB read and written): "
           f"FETCH_SIZE x {fac['FETCH_SIZE']:.4f}, WRITE_SIZE x {fac['WRITE_SIZE']:.4f}.", "",
           "| kernel | dispatches | HBM read MB | HBM written MB | algorithmic read MB | "
           "algorithmic written MB | traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
    for kind in ("fwd", "bwd"):
        if (kind, "FETCH_SIZE") not in counters:
            continue
        rd = float(np.mean(counters[(kind, "FETCH_SIZE")])) * fac["FETCH_SIZE"]
        wr = float(np.mean(counters[(kind, "WRITE_SIZE")])) * fac["WRITE_SIZE"]
        ar, aw = alg[kind]
        rec["kernels"][kind] = {"hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr),
                                "hbm_bytes_per_launch": int(rd + wr),
                                "algorithmic_bytes_per_launch": ar + aw}
        md.append(f"| jas {kind} | {len(counters[(kind, 'FETCH_SIZE')])} | {rd / 1e6:.1f} | "
                  f"{wr / 1e6:.1f} | {ar / 1e6:.1f} | {aw / 1e6:.1f} | {(rd + wr) / (ar + aw):.4f} |")
    md += ["", "Algorithmic bytes: forward reads the scores and writes P (2 bytes each per "
           "element), backward reads P and dP and writes dS; with keys excluded, scores and P "
           f"count on the {V} visible keys only; the per-row sink values (4 bytes "
           "per row, written and read as one scattered word per row) and the mask row are not "
           "counted there and show as the small excess.", "",
           f"Kernel source sha256 at measurement: `{rec['kernel_source_sha256']}`; bench.py "
           "reports these bytes as `roofline.traffic` only while the source still hashes to it."]
    open(os.path.join(PROFILES, f"pmc_traffic_jas_{wl}.md"), "w").write("\n".join(md) + "\n")
    json.dump(rec, open(traffic_record_path(wl), "w"), indent=1)
    print("\n".join(out + [""] + md))


def attn_flops(B, H, S, N, D, causal):
    """Useful FLOPs of attention forward: 2*S*N*D for QK and as many for PV
    per (batch, head), over the visible (query, key) pairs."""
    pairs = S * N
    if causal:
        q = np.arange(S)
        pairs = int(np.clip(q + (N - S) + 1, 0, N).sum())
    return 4.0 * B * H * pairs * D


def bench_attention(args):
    import torch
    import deterministic_attention_softmax_amd as jas
    import oracle
    import synth
    jas.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    wl = args.workload
    desc, B, H, Hkv, S, N, D, has_mask, causal, has_sink = ATTN_WORKLOADS[wl]
    log(f"workload {wl}: {desc}")
    q = synth.normal((B, H, S, D), 1.0, ATTN_SEEDS["q"], dev, torch.bfloat16)
    k = synth.normal((B, Hkv, N, D), 1.0, ATTN_SEEDS["k"], dev, torch.bfloat16)
    v = synth.normal((B, Hkv, N, D), 1.0, ATTN_SEEDS["v"], dev, torch.bfloat16)
    mask = sink = None
    if has_mask:
        _, mask, _, _ = synth.joint_attention_bf16(seed=ATTN_SEEDS["mask"], device="cpu", B=B, H=1,
                                                   S=1, N=N)
        mask = mask.to(dev).view(B, 1, 1, N)
    if has_sink:
        sink = synth.normal((H,), 1.0, ATTN_SEEDS["sink"], dev)
    scale = 1.0 / np.sqrt(D)
    out = torch.empty_like(q)
    d = jas.make_attn_desc(B, H, Hkv, S, N, D, jas.JAS_DTYPE_BF16, 0, scale)

    # rotated buffer sets (copies of the same inputs), as in the softmax bench:
    # consecutive calls do not find each other's q, k, v and out in the
    # Infinity Cache (within one call K and V are shared by design)
    set_bytes = 2 * (2 * q.numel() + 2 * k.numel())
    nsets = max(1, -(-ROTATE_BYTES // set_bytes))
    sets = [(q, k, v, out)] + [(q.clone(), k.clone(), v.clone(), torch.empty_like(q))
                               for _ in range(nsets - 1)]
    nstep = [0]
    # each set's call prepared once (checks, descriptor, outputs): a timed
    # step is one jas_attn_fwd_ex call
    runs = [jas.attn_fwd_prepared(qi, ki, vi, scale=scale, mask=mask,
                                  mask_strides=None if mask is None else (N, 0, 0), sink=sink,
                                  causal=causal, want_lse=True, out=oi,
                                  query_blocks=args.attn_query_blocks) for qi, ki, vi, oi in sets]

    def step():
        run, res = runs[nstep[0] % nsets]
        nstep[0] += 1
        run()
        return res

    check = None
    if not args.no_check:
        r = step()  # the first set: q, k, v themselves
        torch.cuda.synchronize()
        qi = np.sort(np.random.default_rng(CHECK_SEED).choice(S, 2, replace=False))
        if causal:
            qi = np.array([S - 2, S - 1])  # the sub-call keeps the causal offset of the last rows
        it = torch.as_tensor(qi, device=dev)
        qs = q[:, :, it].contiguous()
        o = oracle.attn_fwd(synth.to_numpy_bits(qs), synth.to_numpy_bits(k), synth.to_numpy_bits(v),
                            np.float32(scale), mask=None if mask is None else mask.cpu().numpy(),
                            mask_strides=(N, 0, 0), causal=causal,
                            sink=None if sink is None else sink.cpu().numpy())
        got = (synth.to_numpy_bits(r["out"][:, :, it]).astype(np.uint32) << 16).view(np.float32)
        want = (o["out"].astype(np.uint32) << 16).view(np.float32)
        rel = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want), 1e-3)
        check = {"sampled_queries": int(len(qi) * B * H), "out_max_rel": float(rel.max())}
        assert check["out_max_rel"] < 2.0 ** -6, f"attention parity: {check}"
        log(f"parity check: {check}")
    stream = torch.cuda.current_stream()
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    # per-call durations: HIP events on the launch stream around `steps`
    # back-to-back calls, five times; the duration per call of each of the five
    ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / args.steps)
    ms = np.array(ms)
    flops = attn_flops(B, H, S, N, D, causal)
    tflops = flops / (step_ms * 1e-3) / 1e12
    ktf = flops / (ms.mean() * 1e-3) / 1e12
    log(f"attention {ms.mean():.3f} ms per call, {ktf:.0f} TFLOP/s")
    res = {
        "metric": "fused attention forward TFLOP/s (useful 4*B*H*pairs*D) vs MFMA bf16 dense peak",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "batch": B, "heads": H, "kv_heads": Hkv, "q_len": S,
                   "kv_len": N, "head_dim": D, "mask": has_mask, "causal": causal,
                   "sink": has_sink, "useful_flops": flops,
                   "query_blocks_per_wave": args.attn_query_blocks or "library default"},
        "seed": {**ATTN_SEEDS, "parity_rows": CHECK_SEED},
        "buffer_sets": nsets,
        "roofline": {"bound": "mfma", "kernel": "jas_attn_fwd (fused kernel)",
                     "achieved": round(ktf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ktf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_attn_traffic(wl),
                     "flops_per_launch": flops, "avg_launch_ms": round(float(ms.mean()), 4),
                     "median_launch_ms": round(float(np.median(ms)), 4)},
        "parity": check,
        # the copy kernel the PMC traffic records are calibrated on (1 GiB moved)
        "copy_ceiling": copy_ceiling(1 << 30, stream),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        kq = 1
        t = 0.0
        k_np, v_np = synth.to_numpy_bits(k), synth.to_numpy_bits(v)
        m_np = None if mask is None else mask.cpu().numpy()
        s_np = None if sink is None else sink.cpu().numpy()
        while True:
            q_np = synth.to_numpy_bits(q[:, :, S - kq:].contiguous())
            t0 = time.perf_counter()
            oracle.attn_fwd(q_np, k_np, v_np, np.float32(scale), mask=m_np,
                            mask_strides=(N, 0, 0), causal=causal, sink=s_np,
                            threads=max(1, min(host_cpus()[:2])))
            t = time.perf_counter() - t0
            if t > args.cpu_seconds / 4 or kq >= S:
                break
            kq = min(S, kq * 4)
        # the last kq queries keep their causal offset (key <= N - S + q)
        qq = np.arange(S - kq, S)
        pairs = int(np.clip(qq + (N - S) + 1, 0, N).sum()) if causal else kq * N
        f = 4.0 * B * H * pairs * D
        affinity, share, share_from = host_cpus()
        res["cpu_baseline"] = {"value": round(f / t / 1e12, 6), "unit": "TFLOP/s",
                               "cores": max(1, min(affinity, share)), "kind": "oracle",
                               "affinity_cores": affinity, "cpu_share": share,
                               "cpu_share_from": share_from,
                               "sample": f"the last {kq} queries of every head ({B * H * kq} rows "
                                         f"x {N} keys), {t:.1f} s",
                               "cpu_model": cpu_model()}
    print(json.dumps(res), flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        json.dump(res, open(args.json_out, "w"))


ATTN_PMC_SETS = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_ANY",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VMEM SQ_INST_LEVEL_VMEM "
    "SQ_LDS_ADDR_CONFLICT SQ_CYCLES",
]


def summarize_attn_profiles(prof_dir, wl):
    """Write profiles/kernel_trace_jas_<wl>.md from rocprofv3 output under
    prof_dir: the kernel trace (trace/) and, when present, the two SQ counter
    passes (pmc1/, pmc2/) of the fused attention kernel."""
    import csv
    desc, B, H, Hkv, S, N, D, has_mask, causal, has_sink = ATTN_WORKLOADS[wl]
    os.makedirs(PROFILES, exist_ok=True)
    rows = list(csv.DictReader(open(os.path.join(prof_dir, "trace", f"{wl}_kernel_stats.csv"))))
    line_path = os.path.join(prof_dir, "trace", "bench_line.json")
    line = json.load(open(line_path)) if os.path.exists(line_path) else None
    out = [f"# rocprofv3 kernel trace: jas fused attention, workload {wl}", "",
           f"Workload: {desc}.", "", "Commands (repository root, MI355X, ROCm 7.2):", "", "```",
           f"rocprofv3 --kernel-trace --stats --output-format csv -d {prof_dir}/trace -o {wl} -- "
           f"python3 bench.py --workload {wl} --steps 10 --warmup 3 --no-cpu-baseline "
           f"--json-out {prof_dir}/trace/bench_line.json"]
    for i, cs in enumerate(ATTN_PMC_SETS, 1):
        out.append(f"rocprofv3 --pmc {cs} --output-format csv -d {prof_dir}/pmc{i} -o {wl} -- "
                   f"python3 bench.py --workload {wl} --steps 2 --warmup 1 --no-check --no-cpu-baseline")
    out += [f"python3 bench.py --workload {wl} --summarize-profiles {prof_dir}", "```", "",
            "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    flops = attn_flops(B, H, S, N, D, causal)
    avg_attn = None
    for r in rows:
        n = r["Name"]
        if "attn_fwd_kernel" not in n:
            continue
        name = re.sub(r"\([^()]*\)$", "", n).replace("void ", "")
        a = float(r["AverageNs"]) / 1e3
        if "attn_fwd_kernel" in n:
            avg_attn = a
        out.append(f"| `{name}` | {r['Calls']} | {a:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} |")
    if avg_attn:
        out += ["", f"Fused kernel alone: {flops / (avg_attn * 1e-6) / 1e12:.0f} TFLOP/s of useful "
                f"attention FLOPs ({flops:.4g} per call; the kernel also recomputes QK once)."]
    if line:
        out += ["", "The same run's bench.py line (HIP events around the whole call): "
                f"{line['roofline']['avg_launch_ms'] * 1e3:.1f} us, {line['value']} TFLOP/s."]
    counters = {}
    for i in (1, 2):
        path = os.path.join(prof_dir, f"pmc{i}", f"{wl}_counter_collection.csv")
        if not os.path.exists(path):
            continue
        for r in csv.DictReader(open(path)):
            if "attn_fwd_kernel" in r["Kernel_Name"]:
                counters.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if counters:
        m = {c: float(np.mean(v)) for c, v in counters.items()}
        out += ["", "SQ counters of the fused kernel (mean per dispatch, chip totals):", "",
                "| counter | value |", "|---|---|"]
        out += [f"| {c} | {m[c]:.4g} |" for c in sorted(m)]
        if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m:
            out += ["", f"VALU instructions per MFMA: {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f}."]
        if "SQ_ACTIVE_INST_VALU" in m and "SQ_WAVE_CYCLES" in m:
            out.append(f"VALU-active share of wave cycles: "
                       f"{m['SQ_ACTIVE_INST_VALU'] / m['SQ_WAVE_CYCLES']:.3f}; waiting share: "
                       f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}.")
    open(os.path.join(PROFILES, f"kernel_trace_jas_{wl}.md"), "w").write("\n".join(out) + "\n")
    print("\n".join(out))
    if os.path.isdir(os.path.join(prof_dir, "fetch")) and os.path.isdir(os.path.join(prof_dir, "write")):
        summarize_attn_traffic(prof_dir, wl)


def summarize_attn_traffic(prof_dir, wl):
    """profiles/pmc_traffic_jas_<wl>.{md,json}: HBM bytes per fused attention
    call (the fused kernel, which reads V in place) from FETCH_SIZE /
    WRITE_SIZE, calibrated on the copy kernel bench.py runs in the same
    process."""
    import csv
    desc, B, H, Hkv, S, N, D, has_mask, causal, has_sink = ATTN_WORKLOADS[wl]

    def kind(name):
        if "attn_fwd_kernel" in name:
            return "attn"
        if "copy16<false>" in name:
            return "copy"
        return None

    counters = {}
    for cname, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        for r in csv.DictReader(open(os.path.join(prof_dir, sub, f"{wl}_counter_collection.csv"))):
            k = kind(r["Kernel_Name"])
            if k is not None and r["Counter_Name"] == cname:
                counters.setdefault((k, cname), []).append(float(r["Counter_Value"]) * 1024.0)
    line = json.load(open(os.path.join(prof_dir, "fetch", "bench_line.json")))
    copy_bytes = line["copy_ceiling"]["bytes"] / 2
    fac = {c: copy_bytes / np.mean(counters[("copy", c)]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    # algorithmic bytes of one call: q, k, v read and out written once each
    alg_r = 2 * (B * H * S * D + 2 * B * Hkv * N * D)
    alg_w = 2 * B * H * S * D
    rec = {"workload": wl, "attn_source_sha256": attn_source_hash(),
           "calibration": {"copy_bytes_read": copy_bytes, "copy_bytes_written": copy_bytes,
                           "fetch_factor": round(fac["FETCH_SIZE"], 4),
                           "write_factor": round(fac["WRITE_SIZE"], 4)},
           "kernels": {}}
    md = [f"# rocprofv3 HBM traffic: jas fused attention, workload {wl}", "",
          f"Workload: {desc}.", "", "Commands (repository root):", "", "```"]
    for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        md.append(f"rocprofv3 --pmc {c} --output-format csv -d {prof_dir}/{sub} -o {wl} -- "
                  f"python3 bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --no-check "
                  f"--json-out {prof_dir}/{sub}/bench_line.json")
    md += [f"python3 bench.py --workload {wl} --summarize-profiles {prof_dir}", "```", "",
           "Counters are KiB per dispatch, scaled by what each reads for the 16-byte copy kernel of "
           f"known size in the same process ({copy_bytes / 1e6:.1f} MB read and written): "
           f"FETCH_SIZE x {fac['FETCH_SIZE']:.4f}, WRITE_SIZE x {fac['WRITE_SIZE']:.4f}.", "",
           "| kernel | dispatches | HBM read MB | HBM written MB |", "|---|---|---|---|"]
    tot_r = tot_w = 0.0
    for k in ("attn",):
        rd = float(np.mean(counters[(k, "FETCH_SIZE")])) * fac["FETCH_SIZE"]
        wr = float(np.mean(counters[(k, "WRITE_SIZE")])) * fac["WRITE_SIZE"]
        tot_r, tot_w = tot_r + rd, tot_w + wr
        rec["kernels"][k] = {"hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr)}
        md.append(f"| fused attention | "
                  f"{len(counters[(k, 'FETCH_SIZE')])} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
    rec["call"] = {"hbm_bytes_per_call": int(tot_r + tot_w), "algorithmic_bytes_per_call": alg_r + alg_w}
    md += ["", f"Per call: {tot_r / 1e6:.1f} MB read and {tot_w / 1e6:.1f} MB written, against "
           f"{alg_r / 1e6:.1f} MB and {alg_w / 1e6:.1f} MB of algorithmic bytes (q, k and v read once, "
           f"out written once; mask, lse and sink values not counted): "
           f"{(tot_r + tot_w) / (alg_r + alg_w):.3f} x.  The excess is K and V read by more than one "
           "XCD (each XCD's L2 holds its own copy).", "",
           f"Attention source sha256 at measurement: `{rec['attn_source_sha256']}`; bench.py reports "
           "the per-call bytes as `roofline.traffic` only while the sources still hash to it."]
    open(os.path.join(PROFILES, f"pmc_traffic_jas_{wl}.md"), "w").write("\n".join(md) + "\n")
    json.dump(rec, open(traffic_record_path(wl), "w"), indent=1)
    print("\n".join(md))


def main():
    args = parse()
    if args.summarize_profiles:
        if args.workload in ATTN_WORKLOADS:
            summarize_attn_profiles(args.summarize_profiles, args.workload)
        else:
            summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload in ATTN_WORKLOADS:
        bench_attention(args)
        return
    import torch
    import deterministic_attention_softmax_amd as jas
    jas.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    wl = args.workload
    desc, B, H, S, N, dt, has_mask, has_sink, excl, backward = WORKLOADS[wl]
    causal = excl == "causal"
    rows, E = B * H * S, B * H * S * N
    esz = 2
    log(f"workload {wl}: {desc}")
    s, mask, sink, g, key_len = make_inputs(wl, dev)
    torch.cuda.synchronize()
    # keys each row reads (scores in the forward, P in the backward)
    V = int(row_kends(wl, None if key_len is None else key_len.cpu().numpy()).sum())

    check = None
    if not args.no_check:
        check = check_parity(wl, s, mask, sink, g, key_len)
        log(f"parity check: {check}")

    # Buffer sets rotated from step to step so that the timed steps touch at
    # least ROTATE_BYTES: a workload smaller than the 256 MB Infinity Cache
    # would otherwise be served from it on repeated steps.  Extra sets hold
    # copies of the same inputs.
    set_bytes = s.numel() * esz * (4 if backward else 2)
    nsets = max(1, -(-ROTATE_BYTES // set_bytes))
    sets = [(s, g, torch.empty_like(s), torch.empty_like(s) if backward else None)]
    for _ in range(nsets - 1):
        sets.append((s.clone(), g.clone() if backward else None, torch.empty_like(s),
                     torch.empty_like(s) if backward else None))
    ps = torch.empty(rows, dtype=torch.float32, device=dev) if has_sink else None
    dsk = torch.empty(H, dtype=torch.float32, device=dev) if has_sink else None
    ws = torch.empty(max(4, rows * 4 + 256), dtype=torch.uint8, device=dev) if has_sink else None
    stream = torch.cuda.current_stream()
    nstep = [0]

    # The steps call jas_fwd / jas_bwd directly, with the descriptors and
    # pointers of each buffer set built and checked once by the binding
    # (fwd_prepared / bwd_prepared): no Python wrapper work between launches.
    runs = []
    for si, gi, P, dS in sets:
        rf, _ = jas.fwd_prepared(si, mask=mask, sink=sink, out=P, p_sink=ps, causal=causal,
                                 key_len=key_len)
        rb = None
        if backward:
            rb, _ = jas.bwd_prepared(P, gi, p_sink=ps, out=dS, d_sink=dsk, workspace=ws,
                                     causal=causal, key_len=key_len)
        runs.append((rf, rb))
    invariance = None
    if not args.no_check:
        invariance = check_invariance(wl, runs[0], sets[0], s, mask, sink, g, key_len, ps, dsk)
        log(f"invariance check: {invariance}")

    def step():
        rf, rb = runs[nstep[0] % nsets]
        nstep[0] += 1
        rf()
        if backward:
            rb()

    # bring clocks and page mappings to steady state (untimed, before the
    # warmup steps proper)
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps: one C call per kernel launch, nothing else between
    # them, so the host enqueues ahead of the device and the wall time is
    # the device's.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    # Per-kernel durations: HIP events on the launch stream around K
    # back-to-back launches of one direction (over the same buffer sets),
    # five times; the duration per launch of each of the five.  No event
    # sits between two launches, so a short kernel is not charged for the
    # event records.
    def kernel_ms(which, reps=5):
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                runs[i % nsets][which]()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / args.steps)
        return np.array(out)
    fwd_ms = kernel_ms(0)
    bwd_ms = kernel_ms(1) if backward else np.zeros(1)

    fwd_bytes = esz * (V + E) + (rows * 4 if has_sink else 0)
    bwd_bytes = esz * (V + 2 * E) + (rows * 12 if has_sink else 0) if backward else 0
    total_bytes = fwd_bytes + bwd_bytes
    gbs = total_bytes / (step_ms * 1e-3) / 1e9
    fwd_gbs = fwd_bytes / (fwd_ms.mean() * 1e-3) / 1e9
    bwd_gbs = bwd_bytes / (bwd_ms.mean() * 1e-3) / 1e9 if backward else None
    dom = ("jas bwd", bwd_gbs, bwd_bytes, bwd_ms) if backward else \
          ("jas fwd", fwd_gbs, fwd_bytes, fwd_ms)
    log(f"fwd {fwd_ms.mean():.4f} ms (median {np.median(fwd_ms):.4f}, {fwd_gbs:.0f} GB/s)" +
        (f", bwd {bwd_ms.mean():.4f} ms (median {np.median(bwd_ms):.4f}, {bwd_gbs:.0f} GB/s)"
         if backward else "") + f", step {step_ms:.4f} ms")

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": desc, "batch": B, "heads": H, "q_rows": S, "keys": N,
                   "rows": rows, "mask": has_mask, "sink": has_sink, "exclusion": excl,
                   "visible_keys": V, "backward": backward},
        "rows_per_s": round(rows / (step_ms * 1e-3), 1),
        "seed": {"inputs": SEEDS[wl], "parity_rows": CHECK_SEED},
        "buffer_sets": nsets,
        "fwd_ms": round(float(fwd_ms.mean()), 4), "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "fwd_gbs": round(fwd_gbs, 1),
        "bwd_ms": round(float(bwd_ms.mean()), 4) if backward else None,
        "bwd_ms_median": round(float(np.median(bwd_ms)), 4) if backward else None,
        "bwd_gbs": round(bwd_gbs, 1) if backward else None,
        "kernel_times": "HIP events on the launch stream around `steps` back-to-back launches of "
                        "one direction, 5 repetitions after the timed steps: mean and median of the "
                        "5 per-launch durations",
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": round(dom[1], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom[1] / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(wl, "bwd" if backward else "fwd"),
                     "bytes_per_launch": dom[2], "avg_launch_ms": round(float(dom[3].mean()), 4),
                     "median_launch_ms": round(float(np.median(dom[3])), 4)},
        "parity": check,
        "invariance": invariance,
    }
    out["copy_ceiling"] = copy_ceiling(dom[2], stream)
    if out["copy_ceiling"]:
        # like for like: the forward's one read and one write against the
        # copy, the backward's two reads and one write against that stream
        cc = out["copy_ceiling"]
        best = cc["r2w1"] if backward else max(cc["plain"], cc["nontemporal"])
        out["roofline"]["frac_of_copy"] = round(dom[1] / best, 4)
        out["roofline"]["copy_mix"] = "2R+1W" if backward else "1R+1W"
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(wl, s, mask, sink, g, key_len, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        json.dump(out, open(args.json_out, "w"))


if __name__ == "__main__":
    main()
