"""Benchmark of the fused per-state norm + FC on one MI355X.

One step = one call of the fused step (row statistics, normalisation, the
FC contraction, epilogue) over one batch of synthetic tokens already
resident in HBM.  Default workload: the 8B-shaped decode batch, d = 4096,
M = 64 tokens (8 sequences x 8 draft tokens), LayerNorm with affine
gamma/beta and an FC bias; W [12288, 4096] bf16 is 96 MiB.

The headline entry point is eagle31_fuse_folded: the norm parameters are
folded into the FC once per weight set by eagle31_fold_prepare (the fold the
EAGLE 3.1 explainer describes; its one-time cost is reported beside the
line, outside the timed region), and every step is one launch that streams
the folded weight.  eagle31_fuse on the stored W is measured too.

Cold cache: R copies of (W, hidden states, out) are rotated so the footprint
is at least 512 MiB, twice the 256 MB MALL; every step reads a W that is not
cache-resident, as a serving loop that streams many layers would.

Prints ONE JSON line.  `value` is tokens/s over the K timed steps; the
`roofline` object reports the decode kernel's algorithmic bytes per launch
over its average launch duration (HIP events on the launch stream) against
the 8 TB/s HBM peak; `cpu_baseline` times the fp64 oracle on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 1024 * 1024
METRIC = "fused norm+FC tokens/s; % HBM peak (decode M) / % bf16 MFMA peak (prefill)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--M", type=int, default=64, help="tokens of the headline decode step")
    p.add_argument("--no-sweep", action="store_true", help="skip the per-M decode sweep")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    p.add_argument("--only", choices=["decode", "decode_folded", "prefill", "rowstats", "copy", "postnorm", "postnorm_decode",
                                             "embedcat", "verify", "rows"], default=None,
                   help="run a single leg (used under rocprofv3)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def measured_traffic(M):
    """HBM bytes per launch of the decode kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, calibrated), or None when that
    summary is for another token count or the kernel's sources have changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "gemv_cols_d4096_M64_layernorm.md")
    if M != 64 or not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
    if rec is None:
        return None
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for src in rec["sources"]:
        with open(os.path.join(root, src), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["sha256"] else None


def alg_bytes(d, M, norm, has_beta, has_bias):
    """W + three hidden states + out + bf16 parameter vectors, each once."""
    nvec = 0
    if norm == 1:
        nvec = 3 + (3 if has_beta else 0)
    elif norm == 2:
        nvec = 3
    return 3 * d * d * 2 + 3 * M * d * 2 + M * d * 2 + (nvec + (1 if has_bias else 0)) * d * 2


def flops(d, M):
    return 2 * M * 3 * d * d


def to_dev(bits):
    """bfloat16 bit patterns (numpy uint16) -> device tensor."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


class Rotation:
    """R device copies of one problem instance (same values, distinct memory)."""

    def __init__(self, inp, R, torch, with_W=True):
        self.sets = []
        base_h = [to_dev(x) for x in inp.h]
        base_W = to_dev(inp.W) if with_W else None
        for r in range(R):
            h = [x.clone() for x in base_h] if r else base_h
            W = (base_W.clone() if r else base_W) if with_W else None
            out = torch.empty((inp.M, inp.d), dtype=torch.bfloat16, device="cuda")
            self.sets.append((h, W, out))
        self.gamma = [to_dev(x) for x in inp.gamma]
        self.beta = None if inp.beta is None else [to_dev(x) for x in inp.beta]
        self.bias = None if inp.bias is None else to_dev(inp.bias)


def time_loop(torch, fn, R, steps, warmup, per_call_events=False):
    for i in range(warmup):
        fn(i % R)
    torch.cuda.synchronize()
    if per_call_events:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            fn(i % R)
            ev[i][1].record()
        torch.cuda.synchronize()
        durs = [a.elapsed_time(b) * 1e3 for a, b in ev]  # microseconds
        return durs
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        fn(i % R)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return t0.elapsed_time(t1) * 1e-3, wall


_INPUTS = {}


def cached_inputs(synth, cfg, M):
    key = (cfg, M)
    if key not in _INPUTS:
        if len(_INPUTS) >= 2:
            _INPUTS.clear()
        _INPUTS[key] = synth.make_inputs(cfg, M)
    return _INPUTS[key]


def rotation_count(footprint):
    return max(2, -(-2 * MALL_BYTES // footprint))


def folded_bytes(d, M):
    """W' + three hidden states + out + u [3, d] and c [d] (float32), each once."""
    return 3 * d * d * 2 + 3 * M * d * 2 + M * d * 2 + 4 * d * 4


def decode_leg(torch, pkg, synth, M, steps, warmup, entry="folded", repeats=5):
    """Config-2 decode batch of M tokens through one entry point, cold-cache
    rotation; median of `repeats` timed loops plus per-call HIP events."""
    w = synth.CONFIGS[2]
    inp = cached_inputs(synth, 2, 64).rows(M)
    kind, eps = w.norms[0]
    foot = 3 * inp.d * inp.d * 2 + 4 * M * inp.d * 2
    R = rotation_count(foot)
    rot = Rotation(inp, R, torch)
    fold_us = None
    if entry == "folded":
        prepared = [pkg.fold_prepare(kind, rot.gamma, rot.beta, W, rot.bias) for (_, W, _) in rot.sets]
        # one fold per weight set, timed warm (outputs from the caching allocator)
        W0 = rot.sets[0][1]
        for _ in range(2):
            pkg.fold_prepare(kind, rot.gamma, rot.beta, W0, rot.bias)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            pkg.fold_prepare(kind, rot.gamma, rot.beta, W0, rot.bias)
        e1.record()
        torch.cuda.synchronize()
        fold_us = e0.elapsed_time(e1) / 10 * 1e3
        for k in range(R):  # the folded calls never read the stored W
            h, _, out = rot.sets[k]
            rot.sets[k] = (h, None, out)
        torch.cuda.empty_cache()

        def fn(i):
            h, _, out = rot.sets[i]
            wf, u, c = prepared[i]
            pkg.fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c, out)

        nbytes = folded_bytes(inp.d, M)
    else:
        def fn(i):
            h, W, out = rot.sets[i]
            pkg.fuse(h[0], h[1], h[2], kind, eps, rot.gamma, rot.beta, W, rot.bias, out)

        nbytes = alg_bytes(inp.d, M, kind, inp.beta is not None, inp.bias is not None)

    totals = []
    for _ in range(repeats):
        t, wall = time_loop(torch, fn, R, steps, warmup)
        totals.append(t)
    t_med = statistics.median(totals)
    durs = time_loop(torch, fn, R, steps, warmup, per_call_events=True)
    res = dict(M=M, d=inp.d, R=R, entry=entry, seconds=t_med, seconds_all=totals, steps=steps,
               us_per_step=t_med / steps * 1e6, event_us_mean=statistics.mean(durs),
               event_us_median=statistics.median(durs), bytes=nbytes, fold_prepare_us=fold_us,
               inp=inp, kind=kind, eps=eps)
    del rot
    torch.cuda.empty_cache()
    return res


def prefill_leg(torch, pkg, synth, cfg, M, kind, eps, steps, warmup, folded=False, repeats=5):
    """One workload through eagle31_fuse (stored W) or eagle31_fuse_folded
    (weight folded beforehand), cold-cache rotation; reports tokens/s and the
    fraction of both peaks (HBM with the entry point's algorithmic bytes,
    MFMA with 2 M 3d d flops)."""
    # a smaller M is the prefix of the workload's largest M
    inp = cached_inputs(synth, cfg, synth.CONFIGS[cfg].max_M).rows(M)
    foot = 3 * inp.d * inp.d * 2 + 4 * M * inp.d * 2
    R = 2 if foot >= MALL_BYTES else rotation_count(foot)
    rot = Rotation(inp, R, torch)
    if folded:
        prepared = [pkg.fold_prepare(kind, rot.gamma, rot.beta, W, rot.bias) for (_, W, _) in rot.sets]

    def fn(i):
        h, W, out = rot.sets[i]
        if folded:
            wf, u, c = prepared[i]
            pkg.fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c, out)
        else:
            pkg.fuse(h[0], h[1], h[2], kind, eps, rot.gamma, rot.beta, W, rot.bias, out)

    times = []
    for _ in range(repeats):
        t, _ = time_loop(torch, fn, R, steps, warmup)
        times.append(t / steps)
    per = statistics.median(times)
    nbytes = folded_bytes(inp.d, M) if folded else alg_bytes(inp.d, M, kind, inp.beta is not None,
                                                              inp.bias is not None)
    res = dict(workload=synth.CONFIGS[cfg].name, d=inp.d, M=M, norm=synth.workloads.NORM_NAMES[kind],
               variant="folded" if folded else "plain", steps=steps, repeats=repeats,
               ms_per_step=per * 1e3, ms_p10=min(times) * 1e3, ms_p90=max(times) * 1e3, tokens_per_s=M / per,
               hbm_frac=nbytes / per / 1e9 / HBM_PEAK_GBS,
               mfma_frac=flops(inp.d, M) / per / 1e12 / BF16_PEAK_TFLOPS,
               tflops=flops(inp.d, M) / per / 1e12)
    del rot
    torch.cuda.empty_cache()
    return res


def rows_leg(torch, pkg, synth, cfg, M, n_src, kind, eps, steps, warmup, mode):
    """eagle31_fuse_folded_rows against the dense eagle31_fuse_folded on one
    workload: `dense` reads three contiguous [M, d] states into [M, d];
    `strided` reads them as column blocks of one [M, 3d] buffer and writes the
    right half of an [M, 2d] drafter-input buffer; `indexed` gathers M rows
    (seeded, any order, repeats) of an [n_src, 3d] buffer into the same
    half-buffer.  Cold-cache rotation of every buffer and of W'; the bytes are
    the folded step's (plus the index list)."""
    import numpy as np
    inp = synth.make_inputs(cfg, n_src if mode == "indexed" else M)
    d = inp.d
    rows = inp.M
    foot = 3 * d * d * 2 + 3 * rows * d * 2 + 2 * M * d * 2
    R = 2 if foot >= MALL_BYTES else rotation_count(foot)
    base_W = to_dev(inp.W)
    gamma = [to_dev(x) for x in inp.gamma]
    beta = None if inp.beta is None else [to_dev(x) for x in inp.beta]
    bias = None if inp.bias is None else to_dev(inp.bias)
    idx = None
    if mode == "indexed":
        idx = torch.from_numpy(np.random.default_rng(M).integers(0, n_src, size=M).astype(np.int32)).to("cuda")
    sets = []
    for r in range(R):
        wf, u, c = pkg.fold_prepare(kind, gamma, beta, base_W if r == 0 else base_W.clone(), bias)
        if mode == "dense":
            h = [to_dev(x) for x in inp.h]
            out = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
        else:
            buf = torch.empty((rows, 3 * d), dtype=torch.bfloat16, device="cuda")
            for k in range(3):
                buf[:, k * d:(k + 1) * d] = to_dev(inp.h[k])
            h = [buf[:, k * d:(k + 1) * d] for k in range(3)]
            out = torch.empty((M, 2 * d), dtype=torch.bfloat16, device="cuda")[:, d:]
        sets.append((h, (wf, u, c), out))
    del base_W
    torch.cuda.empty_cache()

    def fn(i):
        h, (wf, u, c), out = sets[i]
        if mode == "dense":
            pkg.fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c, out)
        else:
            pkg.fuse_folded_rows(h[0], h[1], h[2], kind, eps, wf, u, c, row_index=idx, out=out)

    times = []
    for _ in range(3):
        t, _ = time_loop(torch, fn, R, steps, warmup)
        times.append(t / steps)
    per = statistics.median(times)
    nbytes = folded_bytes(d, M) + (M * 4 if idx is not None else 0)
    res = dict(mode=mode, workload=synth.CONFIGS[cfg].name, d=d, M=M, n_src=rows, R=R, steps=steps,
               us_per_call=round(per * 1e6, 3), us_p10=round(min(times) * 1e6, 3), us_p90=round(max(times) * 1e6, 3),
               hbm_frac=round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4),
               mfma_frac=round(flops(d, M) / per / 1e12 / BF16_PEAK_TFLOPS, 4))
    del sets
    torch.cuda.empty_cache()
    return res


def rows_legs(torch, pkg, synth, prefill=True):
    out = [rows_leg(torch, pkg, synth, 2, 64, 256, 1, 1e-5, 200, 20, mode) for mode in ("dense", "strided", "indexed")]
    if prefill:
        out += [rows_leg(torch, pkg, synth, 5, 4096, 4096, 1, 1e-5, 20, 5, mode)
                for mode in ("dense", "strided", "indexed")]
    return out


def postnorm_leg(torch, pkg, synth, cfg, M, kind, eps, steps, warmup):
    """eagle31_norm_output (post-norm feedback) on one workload's hidden-state
    shape: x read once, out written once, gamma and beta read once per call;
    cold-cache rotation over distinct copies of x and out."""
    inp = synth.make_inputs(cfg, M, with_weights=False)
    d = inp.d
    R = 2 if 2 * M * d * 2 >= MALL_BYTES else rotation_count(2 * M * d * 2)
    x0 = to_dev(inp.h[2])
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    outs = [torch.empty_like(x0) for _ in range(R)]
    g, b = to_dev(inp.gamma[2]), to_dev(inp.beta[2])
    name = synth.workloads.NORM_NAMES[kind]

    def fn(i):
        pkg.norm_output(xs[i], name, eps, g, b if kind == 1 else None, out=outs[i])

    t, _ = time_loop(torch, fn, R, steps, warmup)
    per = t / steps
    nbytes = 2 * M * d * 2 + (2 if kind == 1 else 1) * d * 2
    res = dict(entry="eagle31_norm_output", kernel="norm_rows_kernel", workload=synth.CONFIGS[cfg].name, d=d, M=M,
               norm=name, steps=steps, R=R, us_per_call=round(per * 1e6, 3), bytes_per_call=nbytes,
               gbs=round(nbytes / per / 1e9, 1), hbm_frac=round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4))
    del xs, outs
    torch.cuda.empty_cache()
    return res


def embedcat_leg(torch, pkg, synth, M, d, steps, warmup, vocab=32000):
    """eagle31_embed_concat on one workload's shape: an embedding row and a
    fused row read, a [2d] row written per token; cold copies rotated."""
    import numpy as np
    tokens, embed, fused = synth.make_embed_inputs(M, d, vocab, seed=3)
    foot = 3 * M * d * 2
    R = 2 if foot >= MALL_BYTES else rotation_count(foot)
    tok = torch.from_numpy(np.ascontiguousarray(tokens)).to("cuda")
    emb = to_dev(embed)
    f0 = to_dev(fused)
    fs = [f0] + [f0.clone() for _ in range(R - 1)]
    outs = [torch.empty((M, 2 * d), dtype=torch.bfloat16, device="cuda") for _ in range(R)]

    def fn(i):
        pkg.embed_concat(tok, emb, fs[i], out=outs[i])

    t, _ = time_loop(torch, fn, R, steps, warmup)
    per = t / steps
    nbytes = 4 * M * d * 2 + 4 * M  # embedding rows + fused rows read, [M, 2d] written, token ids
    res = dict(entry="eagle31_embed_concat", kernel="embed_concat_kernel", d=d, M=M, vocab=vocab, steps=steps, R=R,
               us_per_call=round(per * 1e6, 3), bytes_per_call=nbytes, gbs=round(nbytes / per / 1e9, 1),
               hbm_frac=round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4))
    del fs, outs, emb
    torch.cuda.empty_cache()
    return res


def verify_leg(torch, pkg, synth, V, B=64, N=4, steps=100, warmup=10):
    """eagle31_verify_accept on B sequences x N drafts over a V-token
    vocabulary.  The step must read, per sequence, the rows it samples from:
    q_j and p_j (2 V floats) after a rejection, q_N (V floats) when every
    draft is kept; plus the draft positions' p and q values, the drafts and the
    uniforms.  Those bytes over the call time give the HBM fraction.  Copies of
    the inputs are rotated so the sampled rows are not cache-resident."""
    import numpy as np
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=V, spread=0.5)
    per_set = (p.nbytes + q.nbytes)
    n_o = None
    sets = []
    base = [torch.from_numpy(x).to("cuda") for x in (p, q, draft, u_acc, u_res)]
    n_acc, nxt = pkg.verify_accept(*base)
    torch.cuda.synchronize()
    n_o = n_acc.cpu().numpy()
    rows_read = int(np.sum(np.where(n_o < N, 2, 1)))
    bytes_alg = rows_read * V * 4 + B * N * (4 + 4 + 4 + 4) + B * 4 + 2 * B * 4
    R = max(2, -(-2 * MALL_BYTES // max(1, rows_read * V * 4)))
    R = min(R, max(2, int(6e9 // per_set)))
    for r in range(R):
        sets.append(base if r == 0 else [x.clone() for x in base])
    outs = [(torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"))
            for _ in range(R)]

    def fn(i):
        s = sets[i]
        pkg.verify_accept(*s, n_accepted=outs[i][0], next_token=outs[i][1])

    times = []
    for _ in range(5):
        t, _ = time_loop(torch, fn, R, steps, warmup)
        times.append(t / steps)
    per = statistics.median(times)
    res = dict(entry="eagle31_verify_accept", kernel="verify_kernel", B=B, N=N, V=V, R=R, steps=steps,
               us_per_call=round(per * 1e6, 3), us_p10=round(sorted(times)[0] * 1e6, 3),
               us_p90=round(sorted(times)[-1] * 1e6, 3), kept_mean=round(float(n_o.mean()), 3),
               bytes_per_call=bytes_alg, gbs=round(bytes_alg / per / 1e9, 1),
               hbm_frac=round(bytes_alg / per / 1e9 / HBM_PEAK_GBS, 4))
    del sets, outs, base
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_leg(inp, kind, eps, budget_s, what="the full decode batch"):
    """The fp64 oracle as it stands, on preconverted float64 arrays, repeated
    until about budget_s seconds of host work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    H = [oracle.decode_bf16(h) for h in inp.h]
    g = [oracle.decode_bf16(x) for x in inp.gamma]
    b = None if inp.beta is None else [oracle.decode_bf16(x) for x in inp.beta]
    W = oracle.decode_bf16(inp.W)
    bias = None if inp.bias is None else oracle.decode_bf16(inp.bias)
    oracle.fuse(H, kind, eps, g, b, W, bias)  # warm BLAS
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.fuse(H, kind, eps, g, b, W, bias)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 10000:
            break
    return dict(value=inp.M * n / el, unit="tokens/s", cores=threads, kind="oracle", cpu_model=cpu_model(),
                sample=f"{n} oracle calls of {what} (d={inp.d}, M={inp.M}) on float64 "
                       f"arrays, {el:.1f} s; BLAS threads {threads}")


def copy_leg(torch, nbytes=1 << 30, steps=20):
    """A plain device copy of known size (counter calibration reference)."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    bb = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        bb.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        bb.copy_(a)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return dict(bytes_per_copy=nbytes, gbs=2 * nbytes * steps / el / 1e9)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the fused step is row independent, and how it would shard over "
              "several GPUs is described, not measured. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import eagle_draft_feature_amd as pkg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkg.lib()

    if args.only == "copy":
        print(json.dumps(copy_leg(torch)))
        return
    if args.only == "prefill":
        print(json.dumps(prefill_leg(torch, pkg, synth, 4, 32768, 1, 1e-5, max(3, args.steps), args.warmup, folded=True,
                                     repeats=1 if args.steps < 10 else 5)))
        return
    if args.only == "verify":
        print(json.dumps([verify_leg(torch, pkg, synth, V) for V in (32000, 128256, 151936)]))
        return
    if args.only == "rows":
        print(json.dumps(rows_legs(torch, pkg, synth)))
        return
    if args.only == "embedcat":
        print(json.dumps([embedcat_leg(torch, pkg, synth, 64, 4096, max(50, args.steps), args.warmup),
                          embedcat_leg(torch, pkg, synth, 32768, 7168, 20, 5)]))
        return
    if args.only == "postnorm_decode":
        print(json.dumps(postnorm_leg(torch, pkg, synth, 2, 64, 1, 1e-5, max(50, args.steps), args.warmup)))
        return
    if args.only == "postnorm":
        print(json.dumps(postnorm_leg(torch, pkg, synth, 4, 32768, 1, 1e-5, max(5, args.steps), args.warmup)))
        return
    if args.only == "rowstats":
        inp = synth.make_inputs(4, with_weights=False)
        h = [to_dev(x) for x in inp.h]
        for _ in range(args.warmup):
            pkg.row_stats(h[0], h[1], h[2], 1, 1e-5)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            pkg.row_stats(h[0], h[1], h[2], 1, 1e-5)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        print(json.dumps(dict(rowstats_us=el * 1e6, gbs=3 * inp.M * inp.d * 2 / el / 1e9)))
        return

    if args.only in ("decode", "decode_folded"):
        r = decode_leg(torch, pkg, synth, args.M, args.steps, args.warmup,
                       entry="folded" if args.only == "decode_folded" else "plain", repeats=3)
        r["tokens_per_s"] = args.M / (r["seconds"] / r["steps"])
        r["hbm_frac"] = r["bytes"] / (r["seconds"] / r["steps"]) / 1e9 / HBM_PEAK_GBS
        print(json.dumps({k: v for k, v in r.items() if k != "inp"}))
        return
    dec = decode_leg(torch, pkg, synth, args.M, args.steps, args.warmup, entry="folded")

    value = args.M * dec["steps"] / dec["seconds"]
    # one launch per call: HIP events around the timed region / launches
    kern_us = dec["seconds"] / dec["steps"] * 1e6
    achieved = dec["bytes"] / (kern_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(args.M),
                    kernel="gemvn_kernel (eagle31_fuse_folded, column split, up to 128 tokens)",
                    bytes_per_launch=dec["bytes"], launch_us_mean=round(kern_us, 3),
                    launch_us_mean_single_events=round(dec["event_us_mean"], 3))

    sweep = []
    if not args.no_sweep:
        for entry, Ms in (("folded", (1, 4, 8, 16, 32, 64)), ("plain", (1, 16, 64))):
            for M in Ms:
                r = dec if (entry == "folded" and M == args.M) else decode_leg(
                    torch, pkg, synth, M, args.steps, args.warmup, entry=entry, repeats=3)
                per = r["seconds"] / r["steps"]
                sweep.append(dict(entry=entry, M=M, us_per_step=round(per * 1e6, 3),
                                  tokens_per_s=round(M / per, 1),
                                  hbm_frac=round(r["bytes"] / per / 1e9 / HBM_PEAK_GBS, 4),
                                  event_us_mean=round(r["event_us_mean"], 3)))

    prefill = []
    others = []
    if not args.no_prefill:
        prefill.append(prefill_leg(torch, pkg, synth, 4, 32768, 1, 1e-5, 20, 3, folded=False))
        prefill.append(prefill_leg(torch, pkg, synth, 4, 32768, 1, 1e-5, 20, 3, folded=True))
        prefill.append(prefill_leg(torch, pkg, synth, 5, 4096, 1, 1e-5, 30, 5, folded=False))
        prefill.append(prefill_leg(torch, pkg, synth, 5, 4096, 1, 1e-5, 30, 5, folded=True))
        # the other sizes of the draft-tree and chunked-prefill workloads
        # (reported against both peaks; the graded bars are the lines above)
        for M in (64, 128, 256):
            for folded in (True, False):
                others.append(prefill_leg(torch, pkg, synth, 3, M, 2, 1e-6, 200, 20, folded=folded))
        for kind, eps in ((1, 1e-5), (2, 1e-6)):
            for M in (512, 2048, 4093) + ((4096,) if kind == 2 else ()):
                others.append(prefill_leg(torch, pkg, synth, 5, M, kind, eps, 30 if M < 4000 else 20, 5,
                                          folded=True))

    # the post-norm feedback of the drafter output (a next step of the path),
    # at the decode batch's and the prefill batch's shapes
    postnorm = [postnorm_leg(torch, pkg, synth, 2, 64, 1, 1e-5, 400, 50)]
    if not args.no_prefill:
        postnorm.append(postnorm_leg(torch, pkg, synth, 4, 32768, 1, 1e-5, 20, 5))

    # the drafter-input concatenation (embedding of the last token, then the
    # fused feature) at the decode and prefill shapes
    embedcat = [embedcat_leg(torch, pkg, synth, 64, 4096, 400, 50)]
    if not args.no_prefill:
        embedcat.append(embedcat_leg(torch, pkg, synth, 32768, 7168, 20, 5))

    # the verify / accept step over the vocabulary (a next step of the path)
    verify = [verify_leg(torch, pkg, synth, V) for V in (32000, 128256, 151936)]

    # strided / indexed hidden-state inputs against the dense entry point
    rows = rows_legs(torch, pkg, synth, prefill=not args.no_prefill)

    cpu = None
    cpu_prefill = None
    if not args.no_cpu:
        cpu = cpu_baseline_leg(dec["inp"], dec["kind"], dec["eps"], args.cpu_seconds)
        if not args.no_prefill:
            # a bounded sample of the long-context prefill workload: its first 512 rows
            pf = cached_inputs(synth, 4, synth.CONFIGS[4].max_M).rows(512)
            cpu_prefill = cpu_baseline_leg(pf, 1, 1e-5, args.cpu_seconds,
                                           what="the first 512 rows of the long-context prefill workload")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["seconds"] / dec["steps"] * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_ln_d4096", "d": dec["d"], "M": args.M, "norm": "layernorm",
                   "eps": dec["eps"], "W": [3 * dec["d"], dec["d"]], "bias": True,
                   "cold_cache_rotation": dec["R"], "entry_point": "eagle31_fuse_folded",
                   "weights": "folded once per weight set by eagle31_fold_prepare (outside the timed region)",
                   "fold_prepare_us": round(dec["fold_prepare_us"], 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_prefill": cpu_prefill,
        "decode_sweep": sweep,
        "prefill": prefill,
        "other_workloads": others,
        "postnorm": postnorm,
        "embed_concat": embedcat,
        "verify": verify,
        "rows": rows,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
