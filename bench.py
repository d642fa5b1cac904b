"""Benchmark of the fused exact-attention path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward (O and lse) and the recompute backward (dQ, dK, dV) of
B=1, H=32, N=8192, d=128, causal, bf16 attention with inputs resident in HBM.

    python bench.py [--steps K] [--warmup W] [--passes fwd|fwdbwd] [--no-cpu-baseline] [--no-extras]
                    [--workload headline|window512|varlen|blocksparse|io|decode|configs] [--n N]

The default (headline) workload is the one above.  `window512` runs the same
shape with a causal sliding window of 512 keys (local attention, through the
packed-sequence entry points with one sequence); `varlen` runs a packed batch
of 16 causal sequences of seeded lengths between 256 and 4096 (32 heads,
d=128, bf16).  `blocksparse` runs the headline shape with a seeded per-head
mask of 128 x 128 blocks, half of them active (attn_fwd_blocksparse /
attn_bwd_blocksparse).  `io` times the fused forward against the unfused three-pass
forward (B=1, H=8, N=--n, d=128, bf16, causal) and runs one plain 1 GiB device
copy; run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives each kernel's
memory traffic, the copy serving as the counters' calibration.  `configs`
times the forward (and the backward where there is one) of each of the five
problem configurations.  Prints one JSON line.  Throughput is algorithmic FLOP/s: forward
4*d*pairs, backward 10*d*pairs (five d-deep products per unmasked pair,
the score recomputation included), pairs = N(N+1)/2 per head when causal.
Kernel durations come from HIP events recorded on the stream the library
launches on (torch's current stream).

The headline run also reports, outside the timed region, (i) the instruction
rates of the part measured by the rate_probe executable (v_exp_f32, fp32 FMA
and bf16 MFMA per CU per shader cycle) with the time those rates put under
the passes' exponentials, and (ii) the shader clock (rocm-smi) and the
socket power (amd-smi) sampled while each pass runs back to back for a few
seconds, beside the package power cap: the part lowers its clock to hold
the cap under sustained load.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense 16-bit MFMA FLOP/clk/CU
WORKLOAD_INDEX = 3         # B=1 H=32 N=8192 d=128 bf16 causal, forward + backward
METRIC = "fused attention fwd/bwd TFLOP/s and % MFMA peak, N=8192 d=128 causal bf16"

# HBM bytes per launch of the headline kernels, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of `bench.py --no-cpu-baseline
# --steps 3 --warmup 1`, scaled by what the same counters read for a plain 1 GiB
# device copy (FETCH_SIZE reads half the copied bytes: factor 2.0; WRITE_SIZE
# reads them exactly: factor 1.0).  The figures hold only for the kernel
# code and device compile flags they were taken on, whose digest
# (kernel_code_digest) is stored beside them; for any other code the traffic
# is reported as null.
TRAFFIC_SOURCES = ("attn_device.h", "attn_launch.h", "attn_fwd.hip", "attn_fwd_loop.inc", "attn_bwd.hip",
                   "attn_dq_loop.inc", "attn_dkdv_loop.inc")
TRAFFIC = {
    "sha256": "6701e0780a1bf1c66278d61609f855b02c80a01a216633ac343ec58223d26cbe",
    "fwd": 295856551,             # attn_fwd_kernel: fetch 2 x 111187.1 KiB + write 66560.0 KiB
    "bwd": 488129917 + 405581125,  # attn_bwd_dq_kernel (2 x 205075.5 + 66560.0 KiB) + attn_bwd_dkdv_kernel (2 x 132508.7 + 131072.0 KiB)
}


def kernel_code_digest():
    """SHA-256 of the device compile flags and the kernel sources with comments
    and whitespace removed: a change to the code or its flags changes it, a
    change to a comment does not."""
    import hashlib
    import re
    from io_aware_exact_06_amd import build as _build
    h = hashlib.sha256()
    h.update(" ".join(f for f in _build.COMMON if not f.startswith("-I")).encode())
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "io_aware_exact_06_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(which):
    return TRAFFIC[which] if kernel_code_digest() == TRAFFIC["sha256"] else None


def run_rate_probe():
    """Instruction rates from the rate_probe executable (None if it is absent or fails)."""
    exe = os.path.join(ROOT, "io_aware_exact_06_amd", "rate_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (OSError, ValueError, IndexError, subprocess.TimeoutExpired):
        return None


def sample_sclk(run_for, seconds=2.5, samples=3):
    """Shader clock (MHz, rocm-smi) and socket power (W, amd-smi) read while
    run_for() keeps the GPU busy.

    run_for(n) enqueues n passes; enough are queued for `seconds`, and both are
    sampled `samples` times while they run.  Returns (clocks, powers), each a
    list of samples or None.
    """
    import torch
    try:
        t0 = time.perf_counter()
        run_for(10)
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / 10
        run_for(max(10, int(seconds / max(per, 1e-5))))
        clk, pwr = [], []
        for _ in range(samples):
            time.sleep(seconds / (3 * samples + 1))
            r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
            m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)Mhz\)", r.stdout)
            if m:
                clk.append(int(m.group(1)))
            try:
                r = subprocess.run(["amd-smi", "metric", "--power"], capture_output=True, text=True, timeout=20)
                m = re.search(r"SOCKET_POWER:\s*(\d+)", r.stdout)
                if m:
                    pwr.append(int(m.group(1)))
            except (OSError, subprocess.TimeoutExpired):
                pass
        torch.cuda.synchronize()
        return clk or None, pwr or None
    except (OSError, subprocess.TimeoutExpired):
        torch.cuda.synchronize()
        return None, None


def power_cap_w():
    """The package power cap (W) rocm-smi reports, or None."""
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True, timeout=20)
        m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", r.stdout)
        return float(m.group(1)) if m else None
    except (OSError, subprocess.TimeoutExpired):
        return None


def flops(w, passes):
    pairs = w.pairs_per_head() * w.B * w.H
    f = 4.0 * w.d * pairs
    b = 10.0 * w.d * pairs
    return f, (b if "bwd" in passes else 0.0)


def cpu_baseline(w, inp, scale, passes, budget_s=10.0):
    """The fp64 oracle on the host's cores, on whole heads of the workload.

    Heads (b=0, h=0), (b=0, h=1), ... are run one after another (forward, then
    backward when timed) until about `budget_s` seconds of oracle work have
    been spent; the rate uses the same FLOP count as the GPU.
    """
    import oracle
    pairs = w.pairs_per_head()
    per_head = 4.0 * w.d * pairs + (10.0 * w.d * pairs if "bwd" in passes else 0.0)
    total_t, heads = 0.0, 0
    for h in range(w.B * w.H):
        b, hh = divmod(h, w.H)
        q, k, v = (inp[n][b, hh].double().numpy()[None] for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, w.causal, scale)
        if "bwd" in passes:
            oracle.bwd(q, k, v, inp["dout"][b, hh].double().numpy()[None], w.causal, scale)
        total_t += time.perf_counter() - t0
        heads += 1
        if total_t >= budget_s:
            break
    what = "forward + backward" if "bwd" in passes else "forward"
    return {"value": per_head * heads / total_t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d of %d heads of the workload (N=%d, d=%d, causal=%s), %s, %.1f s"
                      % (heads, w.B * w.H, w.N, w.d, w.causal, what, total_t),
            "cpu": cpu_model()}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), else what platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def pairs_window(n, wl):
    """Unmasked pairs of one causal head of length n whose rows see at most wl + 1 keys."""
    w = wl + 1
    return (w * (w + 1)) // 2 + max(0, n - w) * w if n > w else n * (n + 1) // 2


class Packed:
    """A packed-sequence workload timed through attn_fwd_varlen / attn_bwd_varlen."""

    def __init__(self, name, lengths, H, d, dtype, causal, window, seed):
        import numpy as np
        import torch

        from io_aware_exact_06_amd.inputs import default_scale, make_inputs
        self.name, self.H, self.d, self.dtype, self.causal, self.window = name, H, d, dtype, causal, window
        self.lengths = [int(x) for x in lengths]
        total = sum(self.lengths)
        inp = make_inputs(1, H, total, d, dtype, seed, with_dout=True)
        dev = torch.device("cuda:0")
        self.q, self.k, self.v, self.do = (inp[n][0].to(dev) for n in ("q", "k", "v", "dout"))
        cu = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)
        self.cu = torch.from_numpy(cu).to(dev)
        self.scale = default_scale(d)
        self.maxlen = max(self.lengths)
        wl = window[0]
        self.pairs = sum(pairs_window(n, wl) if wl >= 0 else n * (n + 1) // 2 for n in self.lengths) * H

    def run(self, attn, bwd, ev=None):
        if ev is not None:
            ev[0].record()
        o, lse = attn.fwd_varlen(self.q, self.k, self.v, self.cu, self.cu, self.maxlen, self.causal, self.scale,
                                 self.window)
        if ev is not None:
            ev[1].record()
        if bwd:
            attn.bwd_varlen(self.q, self.k, self.v, o, self.do, lse, self.cu, self.cu, self.maxlen, self.maxlen,
                            self.causal, self.scale, self.window)
            if ev is not None:
                ev[2].record()
        return o, lse


def bench_packed(args, workload):
    """Time a packed workload; print its JSON line (same fields as the headline line)."""
    import numpy as np
    import torch

    from io_aware_exact_06_amd import attn
    if workload == "window512":
        wk = Packed("fwdbwd_B1_H32_N8192_d128_bf16_causal_window512", [8192], 32, 128, "bf16", True, (511, -1),
                    1003)
    else:
        rng = np.random.default_rng(2024)
        wk = Packed("fwdbwd_H32_varlen16_256to4096_d128_bf16_causal", rng.integers(256, 4097, size=16), 32, 128,
                    "bf16", True, (-1, -1), 1004)
    bwd = "bwd" in args.passes
    for _ in range(args.warmup):
        wk.run(attn, bwd)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        o, lse = wk.run(attn, bwd, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs] if bwd else [0.0]
    ff = 4.0 * wk.d * wk.pairs
    fb = 10.0 * wk.d * wk.pairs if bwd else 0.0
    f_tf = ff / (sum(fwd_ms) / len(fwd_ms) * 1e-3) / 1e12
    b_tf = fb / (sum(bwd_ms) / len(bwd_ms) * 1e-3) / 1e12 if bwd else None
    ms_step = wall * 1e3 / args.steps
    out = {
        "metric": METRIC, "value": round((ff + fb) / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wk.dtype,
        "data": "synthetic: iid N(0,1) fp32 rounded to bf16",
        "config": {"workload": wk.name, "H": wk.H, "d": wk.d, "lengths": wk.lengths, "causal": wk.causal,
                   "window": list(wk.window), "passes": args.passes, "unmasked_pairs": wk.pairs},
        "fwd": {"avg_ms": round(sum(fwd_ms) / len(fwd_ms), 4), "tflops": round(f_tf, 2),
                "pct_peak": round(100 * f_tf / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(b_tf if bwd else f_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round((b_tf if bwd else f_tf) / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "kernel": "attn_bwd_varlen pass" if bwd else "attn_fwd_kernel (packed)"},
        "outputs_finite": bool(torch.isfinite(o).all()),
    }
    if bwd:
        out["bwd"] = {"avg_ms": round(sum(bwd_ms) / len(bwd_ms), 4), "tflops": round(b_tf, 2),
                      "pct_peak": round(100 * b_tf / PEAK_BF16_TFLOPS, 2)}
    print(json.dumps(out), flush=True)


def bench_decode(args):
    """Decode shape: 32 sequences of one query row each against 8192 cached keys
    (32 heads, d = 128, bf16, causal with rows aligned to the end of the keys)
    through attn_fwd_varlen.  The pass reads every K and V row once, so the
    roof is HBM bandwidth; the line reports the compulsory bytes (Q, K, V, O,
    lse) per second against 8 TB/s."""
    import numpy as np
    import torch

    from io_aware_exact_06_amd import attn
    from io_aware_exact_06_amd.inputs import default_scale, make_inputs
    nseq, nk, H, d = 32, 8192, 32, 128
    lq, lk = [1] * nseq, [nk] * nseq
    dev = torch.device("cuda:0")
    a = make_inputs(1, H, sum(lq), d, "bf16", 1006)
    b = make_inputs(1, H, sum(lk), d, "bf16", 1007)
    q = a["q"][0].to(dev)
    k, v = b["k"][0].to(dev), b["v"][0].to(dev)
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)).to(dev)
    cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)).to(dev)
    scale = default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty((H, sum(lq)), dtype=torch.float32, device=dev)

    def run():
        attn.fwd_varlen(q, k, v, cu_q, cu_k, max(lq), True, scale, o=o, lse=lse)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        run()
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    avg = sum(ms) / len(ms)
    nbytes = 2 * H * d * (sum(lq) * 2 + sum(lk) * 2) + 4 * H * sum(lq)  # Q, O, K, V (16-bit) + lse
    gbs = nbytes / (avg * 1e-3) / 1e9
    out = {
        "metric": "decode attention forward HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: iid N(0,1) fp32 rounded to bf16, seeds 1006, 1007",
        "config": {"workload": "fwd_decode32_nq1_nk8192_H32_d128_bf16_causal", "sequences": nseq, "nq": 1,
                   "nk": nk, "H": H, "d": d, "causal": True, "passes": "fwd"},
        "fwd": {"avg_ms": round(avg, 4), "min_ms": round(min(ms), 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None, "kernel": "attn_fwd_kernel (packed)",
                     "compulsory_bytes": nbytes},
        "outputs_finite": bool(torch.isfinite(o).all() and torch.isfinite(lse).all()),
    }
    print(json.dumps(out), flush=True)


def bench_blocksparse(args):
    """Headline shape with a per-head 50% random block mask (seed 2025), causal."""
    import numpy as np
    import torch

    from io_aware_exact_06_amd import attn
    from io_aware_exact_06_amd.inputs import default_scale, make_inputs
    B, H, N, d = 1, 32, 8192, 128
    nb = N // attn.MASK_BLOCK
    rng = np.random.default_rng(2025)
    mask = (rng.random((H, nb, nb)) < 0.5).astype(np.uint8)
    mask[:, np.arange(nb), np.arange(nb)] = 1  # every row keeps its diagonal block
    # visible (query, key) pairs: active blocks, causal inside the diagonal blocks
    tri = attn.MASK_BLOCK * (attn.MASK_BLOCK + 1) // 2
    full = attn.MASK_BLOCK * attn.MASK_BLOCK
    low = np.tril(np.ones((nb, nb), bool), -1)
    pairs = int(sum(mask[h][low].sum() * full + np.trace(mask[h]) * tri for h in range(H)))
    inp = make_inputs(B, H, N, d, "bf16", 1003, with_dout=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    m = torch.from_numpy(mask).to(dev)
    scale = default_scale(d)
    bwd = "bwd" in args.passes

    def run(ev=None):
        if ev is not None:
            ev[0].record()
        o, lse = attn.fwd_blocksparse(q, k, v, m, True, scale)
        if ev is not None:
            ev[1].record()
        if bwd:
            attn.bwd_blocksparse(q, k, v, o, do, lse, m, True, scale)
            if ev is not None:
                ev[2].record()
        return o

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        o = run(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps if bwd else 0.0
    f_tf = 4.0 * d * pairs / (fwd_ms * 1e-3) / 1e12
    b_tf = 10.0 * d * pairs / (bwd_ms * 1e-3) / 1e12 if bwd else None
    ms_step = wall * 1e3 / args.steps
    out = {
        "metric": METRIC, "value": round((4.0 + (10.0 if bwd else 0.0)) * d * pairs / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic: iid N(0,1) fp32 rounded to bf16, seed 1003; mask seed 2025",
        "config": {"workload": "fwdbwd_B1_H32_N8192_d128_bf16_causal_blocksparse50", "B": B, "H": H, "N": N,
                   "d": d, "causal": True, "mask_block": attn.MASK_BLOCK,
                   "active_blocks": int(mask.sum()), "visible_pairs": pairs, "passes": args.passes},
        "fwd": {"avg_ms": round(fwd_ms, 4), "tflops": round(f_tf, 2), "pct_peak": round(100 * f_tf / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(b_tf if bwd else f_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round((b_tf if bwd else f_tf) / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_bwd_blocksparse pass" if bwd else "attn_fwd_kernel (block mask)"},
        "outputs_finite": bool(torch.isfinite(o).all()),
    }
    if bwd:
        out["bwd"] = {"avg_ms": round(bwd_ms, 4), "tflops": round(b_tf, 2),
                      "pct_peak": round(100 * b_tf / PEAK_BF16_TFLOPS, 2)}
    print(json.dumps(out), flush=True)


def bench_io(args):
    """Fused vs unfused forward at one sequence length, plus a calibration copy."""
    import torch

    from io_aware_exact_06_amd import attn
    from io_aware_exact_06_amd.inputs import default_scale, make_inputs
    B, H, N, d = 1, 8, args.n, 128
    inp = make_inputs(B, H, N, d, "bf16", 1005)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    scale = default_scale(d)
    ws = torch.empty(attn.attn_fwd_unfused_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
    res = {}
    for name, fn in (("fused", lambda: attn.fwd(q, k, v, True, scale)),
                     ("unfused", lambda: attn.fwd_unfused(q, k, v, True, scale, workspace=ws))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            o, lse = fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"avg_ms": round(e0.elapsed_time(e1) / args.steps, 4), "finite": bool(torch.isfinite(o).all())}
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)  # calibration: exactly 1 GiB read and 1 GiB written
    torch.cuda.synchronize()
    pairs = N * (N + 1) // 2 * B * H
    compulsory = 4 * B * H * N * d * 2 + B * H * N * 4
    print(json.dumps({"workload": "io_B1_H8_N%d_d128_bf16_causal" % N, "N": N, "unmasked_pairs": pairs,
                      "compulsory_bytes_fused": compulsory,
                      "intermediate_bytes_unfused": B * H * N * N * (4 + 2), "fused": res["fused"],
                      "unfused": res["unfused"], "calibration_copy_bytes": 1 << 30}), flush=True)


# Work per unmasked (query, key) pair of each pass as the kernels execute it,
# counted from their inner loops (unmasked tiles, per lane and score element):
#   fwd: two d-deep products (4 d MFMA FLOP); one v_exp_f32; about 4 other
#        vector instructions (scale-and-subtract FMA, running-sum add, half a
#        16-bit pack, half a dot2 adding the rounded weights, half a three-input
#        maximum, plus the maximum's NaN quieting);
#   bwd: seven d-deep products (14 d MFMA FLOP: S, dP, dQ in the dQ kernel; S,
#        dP, dV, dK in the dK/dV kernel); two v_exp_f32 (one per kernel);
#        about 5.5 other vector instructions (dQ kernel: the FMA, the product
#        P (dP - D) -- the dP accumulator starts from -D -- and half a pack;
#        dK/dV kernel: the same plus a second half pack).
KERNEL_WORK = {"fwd": {"mfma_flop_per_d": 4.0, "exp": 1.0, "valu": 4.0},
               "bwd": {"mfma_flop_per_d": 14.0, "exp": 2.0, "valu": 5.5}}


def floors(pairs, d, pass_, rates):
    """Time floors (ms) of one pass from the measured instruction rates (each at
    the clock its probe ran at): the matrix cores on the executed MFMA work, and
    the vector unit on the exponentials plus the other vector instructions
    (both issue through the vector pipe, so their times add)."""
    kw = KERNEL_WORK[pass_]
    cus = rates["cus"]
    mfma_rate = rates["mfma_bf16_flop_per_clk_per_cu"] * cus * rates["mfma_mhz"] * 1e6
    exp_rate = rates["exp_per_clk_per_cu"] * cus * rates["exp_mhz"] * 1e6
    fma_rate = rates["fma_f32_per_clk_per_cu"] * cus * rates["fma_mhz"] * 1e6
    t_mfma = pairs * kw["mfma_flop_per_d"] * d / mfma_rate * 1e3
    t_exp = pairs * kw["exp"] / exp_rate * 1e3
    t_vec = t_exp + pairs * kw["valu"] / fma_rate * 1e3
    return {"mfma_floor_ms": round(t_mfma, 5), "exp_floor_ms": round(t_exp, 5), "vector_floor_ms": round(t_vec, 5)}


def roof_row(prefix, pairs, d, pass_, ms, rates):
    """Floors of a pass, the binding one and the fraction of it achieved."""
    if not rates:
        return {}
    f = floors(pairs, d, pass_, rates)
    bound = "mfma" if f["mfma_floor_ms"] >= f["vector_floor_ms"] else "vector"
    fl = max(f["mfma_floor_ms"], f["vector_floor_ms"])
    out = {prefix + "_" + k: v for k, v in f.items()}
    out[prefix + "_bound"] = bound
    out[prefix + "_frac_of_bound"] = round(fl / ms, 4)
    return out


def bench_configs(args):
    """Every problem configuration of the workload list, forward (and backward
    where the configuration has one), timed with HIP events on the launch
    stream; one JSON line with a row per configuration.  The small ones are
    launch- or latency-bound and are reported, not held to the matrix roof."""
    import torch

    from io_aware_exact_06_amd import attn
    from io_aware_exact_06_amd.inputs import WORKLOADS, default_scale, workload_inputs

    rates = None if args.no_extras else run_rate_probe()  # before this process touches the GPU
    dev = torch.device("cuda:0")
    rows = []
    for idx, w in enumerate(WORKLOADS):
        inp = workload_inputs(idx)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        scale = default_scale(w.d)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        ff = 4.0 * w.d * w.pairs_per_head() * w.B * w.H
        reps = max(args.steps, 200 if ff < 5e10 else 0)
        fwd = lambda: attn.fwd(q, k, v, w.causal, scale, o=o, lse=lse)
        for _ in range(args.warmup):
            fwd()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            fwd()
        e[1].record()
        torch.cuda.synchronize()
        f_ms = e[0].elapsed_time(e[1]) / reps
        pairs = w.pairs_per_head() * w.B * w.H
        row = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
               "causal": w.causal, "fwd_ms": round(f_ms, 5), "fwd_tflops": round(ff / f_ms / 1e9, 2),
               "fwd_pct_peak": round(100 * ff / f_ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
        row.update(roof_row("fwd", pairs, w.d, "fwd", f_ms, rates))
        if w.backward:
            do = inp["dout"].to(dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            ws = torch.empty(max(1, attn.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d)), dtype=torch.uint8,
                             device=dev)
            fb = 10.0 * w.d * w.pairs_per_head() * w.B * w.H
            bwd = lambda: attn.bwd(q, k, v, o, do, lse, w.causal, scale, dq=dq, dk=dk, dv=dv, workspace=ws)
            for _ in range(args.warmup):
                bwd()
            e[0].record()
            for _ in range(args.steps):
                bwd()
            e[1].record()
            torch.cuda.synchronize()
            b_ms = e[0].elapsed_time(e[1]) / args.steps
            row.update({"bwd_ms": round(b_ms, 5), "bwd_tflops": round(fb / b_ms / 1e9, 2),
                        "bwd_pct_peak": round(100 * fb / b_ms / 1e9 / PEAK_BF16_TFLOPS, 2)})
            row.update(roof_row("bwd", pairs, w.d, "bwd", b_ms, rates))
        rows.append(row)
        del q, k, v, o, lse
    print(json.dumps({"metric": "fused attention fwd/bwd TFLOP/s per configuration", "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "peak": PEAK_BF16_TFLOPS,
                      "rates": rates, "kernel_work_per_pair": KERNEL_WORK,
                      "data": "synthetic: the configurations' seeded inputs", "configs": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--passes", choices=["fwd", "fwdbwd"], default="fwdbwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the instruction-rate probe and the clock sampling (profiling runs)")
    ap.add_argument("--workload", choices=["headline", "window512", "varlen", "blocksparse", "io", "decode",
                                           "configs"],
                    default="headline")
    ap.add_argument("--n", type=int, default=4096, help="sequence length of the io workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from io_aware_exact_06_amd import attn
    from io_aware_exact_06_amd.inputs import WORKLOADS, default_scale, workload_inputs

    if not os.path.exists(attn.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if args.workload == "io":
        bench_io(args)
        return
    if args.workload == "blocksparse":
        bench_blocksparse(args)
        return
    if args.workload == "decode":
        bench_decode(args)
        return
    if args.workload == "configs":
        bench_configs(args)
        return
    if args.workload != "headline":
        bench_packed(args, args.workload)
        return

    rates = None if args.no_extras else run_rate_probe()  # before this process touches the GPU
    w = WORKLOADS[WORKLOAD_INDEX]
    scale = default_scale(w.d)
    inp = workload_inputs(WORKLOAD_INDEX)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(1, attn.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d)), dtype=torch.uint8, device=dev)
    bwd = "bwd" in args.passes

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        attn.fwd(q, k, v, w.causal, scale, o=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if bwd:
            attn.bwd(q, k, v, o, do, lse, w.causal, scale, dq=dq, dk=dk, dv=dv, workspace=ws)
            if ev is not None:
                ev[2].record()

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

    fwd_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    bwd_ms = sorted(e[1].elapsed_time(e[2]) for e in evs) if bwd else [0.0]
    med = lambda a: a[len(a) // 2]
    finite = bool(torch.isfinite(o).all() and torch.isfinite(lse).all())
    if bwd:
        finite = finite and bool(torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all())
    ff, fb = flops(w, args.passes)
    ms_step = wall * 1e3 / args.steps
    f_tf = ff / (sum(fwd_ms) / len(fwd_ms) * 1e-3) / 1e12
    b_tf = fb / (sum(bwd_ms) / len(bwd_ms) * 1e-3) / 1e12 if bwd else None
    value = (ff + fb) / (ms_step * 1e-3) / 1e12
    # Dominant work: the backward pass (attn_bwd_dq_kernel then attn_bwd_dkdv_kernel,
    # timed together by the events around one attn_bwd call) when it runs, else the forward.
    fwd_roof = {"bound": "mfma", "achieved": round(f_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(f_tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("fwd"),
                "kernel": "attn_fwd_kernel",
                "avg_ms": round(sum(fwd_ms) / len(fwd_ms), 4)}
    if bwd:
        dom = {"kernel": "attn_bwd pass: attn_bwd_dq_kernel + attn_bwd_dkdv_kernel",
               "achieved": b_tf, "avg_ms": sum(bwd_ms) / len(bwd_ms), "traffic": measured_traffic("bwd")}
    else:
        dom = {"kernel": "attn_fwd_kernel", "achieved": f_tf, "avg_ms": sum(fwd_ms) / len(fwd_ms),
               "traffic": measured_traffic("fwd")}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) fp32 rounded to bf16, seed 1003",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "dtype": w.dtype, "passes": args.passes},
        "fwd": {"median_ms": round(med(fwd_ms), 4), "min_ms": round(fwd_ms[0], 4),
                "tflops": round(f_tf, 2), "pct_peak": round(100 * f_tf / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(dom["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom["achieved"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": dom["traffic"], "kernel": dom["kernel"], "avg_ms": round(dom["avg_ms"], 4)},
        "roofline_fwd": fwd_roof,
        "outputs_finite": finite,
    }
    if bwd:
        out["bwd"] = {"median_ms": round(med(bwd_ms), 4), "min_ms": round(bwd_ms[0], 4),
                      "tflops": round(b_tf, 2), "pct_peak": round(100 * b_tf / PEAK_BF16_TFLOPS, 2)}
    # Floors of each pass from the measured instruction rates: the matrix cores
    # on the executed MFMA work, the vector unit on the exponentials and other
    # vector instructions per pair (KERNEL_WORK), each at its probe's clock.
    if rates:
        pairs = w.pairs_per_head() * w.B * w.H
        out["rates"] = dict(rates)
        out["floors"] = {"fwd": roof_row("fwd", pairs, w.d, "fwd", sum(fwd_ms) / len(fwd_ms), rates)}
        if bwd:
            out["floors"]["bwd"] = roof_row("bwd", pairs, w.d, "bwd", sum(bwd_ms) / len(bwd_ms), rates)
    fwd_only = lambda n: [attn.fwd(q, k, v, w.causal, scale, o=o, lse=lse) for _ in range(n)]
    bwd_only = lambda n: [attn.bwd(q, k, v, o, do, lse, w.causal, scale, dq=dq, dk=dk, dv=dv, workspace=ws)
                          for _ in range(n)]
    if not args.no_extras:
        fc, fp = sample_sclk(fwd_only)
        bc, bp = sample_sclk(bwd_only) if bwd else (None, None)
        out["sclk_mhz_sustained"] = {"fwd": fc, "bwd": bc}
        out["socket_power_w"] = {"fwd": fp, "bwd": bp, "cap": power_cap_w()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, scale, args.passes)
    print(json.dumps(out), flush=True)
    if not finite:
        sys.exit(1)


if __name__ == "__main__":
    main()
