"""Benchmark of the deterministic-reduction hot path on one MI355X.

One step = one pass of every operation on the path over one batch of
seeded synthetic input shaped like an 8B-class model (hidden 4096, MLP 14336,
vocabulary 151936), batch 256:
  rmsnorm      inv_rmsnorm           x[256,4096] bf16 -> fp32
  shrink       det_splitk_gemm       X[256,4096] A[4096,64], 8 slices
  shrink_atom  atomic_splitk_gemm    the same product, fp32 atomics (control)
  cast         detred_f32_to_bf16    shrink output -> bf16
  expand       det_splitk_gemm       [256,64] B[64,4096]
  dense        det_splitk_gemm       X[256,4096] W[4096,14336]
  tp_shards    tree_tp_shards_gemm   X[512,8192] W[8192,8192]: 8 virtual shards'
                                     subtree roots (what each rank computes)
  tp_combine   tree_combine_f32      the top 3 tree levels over the 8 roots
                                     (what the cross-rank reduction computes)
  log_softmax_mean inv_log_softmax_mean logits[256,151936] fp32: log_softmax
                                     and the row mean in one pass over the
                                     logits (the bits of inv_log_softmax and
                                     inv_mean, which are checked against it)
Every operation runs in libdetred's HIP kernels.  The step's three
independent chains (dense -> log_softmax_mean; the tree-TP pair; rmsnorm,
the LoRA shrink/control/cast/expand) run on three streams of default
priority, forked from and joined to the main stream with events; the same
ops issued serially on one stream are timed too (ms_per_step_serial).
`value` is the deterministic GEMM work of a step (shrink, expand, dense,
tree-TP) divided by the step time.  Each operation is also timed alone
with HIP events on the stream it runs on; the slowest one gets the roofline
object.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from invariant_reduction_amd import detred, inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

B = 256          # batch rows of the step
H = 4096         # hidden size
R = 64           # LoRA rank
F = 14336        # MLP width
V = 151936       # vocabulary
TP_M, TP_K, TP_N, TP_T = 512, 8192, 8192, 8

WORKLOAD = ("hot_path_8b_b256: rmsnorm[256,4096]; lora shrink X[256,4096]A[4096,64] det split-K=8 "
            "(+atomic control); bf16 cast; expand [256,64]B[64,4096]; dense X[256,4096]W[4096,14336]; "
            "tree-TP X[512,8192]W[8192,8192] T=8; log_softmax+mean logits[256,151936] (one pass)")

PROFILES = os.path.join(ROOT, "profiles")


def d16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


class Workload:
    """Device-resident inputs, outputs and workspaces of one step."""

    def __init__(self, dev, seed=0):
        self.dev = dev
        x, g = inputs.rmsnorm_inputs(B, H, seed)
        X, A, Bm = inputs.lora_inputs(B, H, R, seed)
        _, W = inputs.dense_inputs(B, H, F, seed)
        Xt, Wt = inputs.dense_inputs(TP_M, TP_K, TP_N, seed)
        lg = inputs.logits_inputs(B, V, seed)
        self.host = dict(x=x, g=g, X=X, A=A, B=Bm, W=W, Xt=Xt, Wt=Wt, lg=lg)
        f32 = torch.float32
        self.x, self.g = d16(x, dev), d16(g, dev)
        self.X, self.A, self.B, self.W = d16(X, dev), d16(A, dev), d16(Bm, dev), d16(W, dev)
        self.Xt, self.Wt = d16(Xt, dev), d16(Wt, dev)
        self.lg = torch.from_numpy(lg).to(dev)
        self.y_rms = torch.empty((B, H), dtype=f32, device=dev)
        self.y_shr = torch.empty((B, R), dtype=f32, device=dev)
        self.y_atm = torch.empty((B, R), dtype=f32, device=dev)
        self.y_b16 = torch.empty((B, R), dtype=torch.int16, device=dev)
        self.y_exp = torch.empty((B, H), dtype=f32, device=dev)
        self.y_dns = torch.empty((B, F), dtype=f32, device=dev)
        self.y_tp = torch.empty((TP_M, TP_N), dtype=f32, device=dev)
        self.y_lsm = torch.empty((B, V), dtype=f32, device=dev)
        self.y_mean = torch.empty((B,), dtype=f32, device=dev)
        self.ws_shr = detred.workspace(B, R, H, 8, dev)
        self.p_tp = torch.empty((TP_T, TP_M, TP_N), dtype=f32, device=dev)
        self.ws_dns = detred.workspace(B, F, H, 0, dev)

    def ops(self, streams):
        """(name, launch, det-GEMM flops, algorithmic bytes, lane) in step
        order.  Algorithmic bytes count inputs and the final output once;
        split partials and shard buffers are not credited (tp_shards: X, W
        and one [M,N] result).  Each launch re-issues a C call whose arguments were
        marshalled once, on streams[lane].  Lanes are independent chains:
        0 dense -> log_softmax_mean; 1 the tree-TP pair; 2 rmsnorm, the
        LoRA shrink/control/cast/expand."""
        gb = 2  # bytes per bf16

        def P(lane, fn, *args):
            return detred.prepare(fn, *args, stream=streams[lane])
        return [
            ("rmsnorm", P(2, detred.inv_rmsnorm, self.x, self.g, self.y_rms, 1e-6),
             0, B * H * gb + H * gb + B * H * 4, 2),
            ("shrink", P(2, detred.det_splitk_gemm, self.X, self.A, self.y_shr, 8, self.ws_shr),
             2 * B * H * R, B * H * gb + H * R * gb + B * R * 4, 2),
            ("shrink_atom", P(2, detred.atomic_splitk_gemm, self.X, self.A, self.y_atm, 8),
             0, B * H * gb + H * R * gb + B * R * 4, 2),
            ("cast", P(2, detred.detred_f32_to_bf16, self.y_shr, self.y_b16),
             0, B * R * 4 + B * R * gb, 2),
            ("expand", P(2, detred.det_splitk_gemm, self.y_b16, self.B, self.y_exp, 0),
             2 * B * R * H, B * R * gb + R * H * gb + B * H * 4, 2),
            ("dense", P(0, detred.det_splitk_gemm, self.X, self.W, self.y_dns, 0, self.ws_dns),
             2 * B * H * F, B * H * gb + H * F * gb + B * F * 4, 0),
            ("tp_shards", P(1, detred.tree_tp_shards_gemm, self.Xt, self.Wt, self.p_tp, TP_T),
             2 * TP_M * TP_K * TP_N, TP_M * TP_K * gb + TP_K * TP_N * gb + TP_M * TP_N * 4, 1),
            ("tp_combine", P(1, detred.tree_combine_f32, self.p_tp, self.y_tp),
             0, TP_T * TP_M * TP_N * 4 + TP_M * TP_N * 4, 1),
            ("log_softmax_mean", P(0, detred.inv_log_softmax_mean, self.lg, self.y_lsm,
                                   self.y_mean),
             0, 2 * B * V * 4 + B * 4, 0),
        ]


class Step:
    """One step: the ops issued in order, each on its lane's stream; the
    side streams wait for the main stream before their first op and the
    main stream waits for them after their last (events, no host sync)."""

    def __init__(self, ops, streams):
        self.ops = ops
        self.streams = streams
        self.fork = torch.cuda.Event()
        self.join = [torch.cuda.Event() for _ in streams]

    def __call__(self):
        main = self.streams[0]
        if len(self.streams) > 1:
            self.fork.record(main)
            for s in self.streams[1:]:
                s.wait_event(self.fork)
        for op in self.ops:
            op[1]()
        if len(self.streams) > 1:
            for s, e in zip(self.streams[1:], self.join[1:]):
                e.record(s)
                main.wait_event(e)


def time_steps(step, steps, stream):
    """Whole-region time of `steps` passes, bracketed by one HIP event pair
    on the main stream (which joins every side stream each step)."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_ops(ops, steps, stream):
    """Per-launch durations: a HIP event pair around every launch of a
    pass of `steps` serial steps (every op on `stream`, one at a time)."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        for i, op in enumerate(ops):
            ev[s][i][0].record(stream)
            op[1]()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    return [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)] for i in range(len(ops))]


def median_time_us(fn, reps, stream, warm=20):
    for _ in range(warm):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
    return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]


def cold_time_us(fn, reps, stream, flush):
    """Median of reps calls, each after a read of `flush` (a 512 MiB
    buffer, twice the MALL, written once beforehand so that its lines are
    clean), so the call's operands come from HBM and no write-back of
    dirty lines overlaps it."""
    fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for a, b in evs:
            flush.sum()
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
    return ts[len(ts) // 2]


def latency_ratios(dev, stream):
    """Deterministic split-K=8 vs atomic split-K=8 (zero fill included) vs
    unsplit, on the LoRA shrink shapes; interleaved, medians of 200."""
    out = {}
    for (M, K, r) in [(16, 512, 16), (256, 4096, 64), (256, 4096, 16), (1, 4096, 64)]:
        X, A, _ = inputs.lora_inputs(M, K, r, 0)
        Xd, Ad = d16(X, dev), d16(A, dev)
        Y = torch.empty((M, r), dtype=torch.float32, device=dev)
        ws = detred.workspace(M, r, K, 8, dev)
        fns = {
            "det8": detred.prepare(detred.det_splitk_gemm, Xd, Ad, Y, 8, ws),
            "atomic8": detred.prepare(detred.atomic_splitk_gemm, Xd, Ad, Y, 8),
            "unsplit": detred.prepare(detred.det_splitk_gemm, Xd, Ad, Y, 1),
        }
        med = {k: [] for k in fns}
        for _ in range(3):  # interleave the variants
            for k, fn in fns.items():
                med[k].append(median_time_us(fn, 200, stream)[0])
        m = {k: statistics.median(v) for k, v in med.items()}
        out["%dx%dx%d" % (M, r, K)] = {
            "det8_us": round(m["det8"], 2), "atomic8_us": round(m["atomic8"], 2),
            "unsplit_us": round(m["unsplit"], 2),
            "det_over_atomic": round(m["det8"] / m["atomic8"], 4),
            "det_over_unsplit": round(m["det8"] / m["unsplit"], 4),
        }
    return out


def invariance(wl, dev):
    """Rows of the step's outputs compared bitwise with reference runs: the
    reference is split 1 / one shard at the full batch; the others are the
    step's own outputs (8 slices, 8 shards), batch prefixes, single rows and
    the replays of the timed steps (checked by the caller)."""
    same = total = 0

    def cmp(a, b):
        nonlocal same, total
        a = a.view(torch.int32).reshape(a.shape[0], -1)
        b = b.view(torch.int32).reshape(b.shape[0], -1)
        eq = torch.all(a == b, dim=1)
        same += int(eq.sum())
        total += eq.numel()

    f32 = torch.float32
    # shrink: split 8 (step) vs unsplit, prefixes and single rows
    ref = torch.empty((B, R), dtype=f32, device=dev)
    detred.det_splitk_gemm(wl.X, wl.A, ref, 1)
    cmp(wl.y_shr, ref)
    for M in (1, 17, 128, 255):
        y = torch.empty((M, R), dtype=f32, device=dev)
        detred.det_splitk_gemm(wl.X[:M], wl.A, y, 8, detred.workspace(M, R, H, 8, dev))
        cmp(y, ref[:M])
    for j in (5, 200):
        y = torch.empty((1, R), dtype=f32, device=dev)
        detred.det_splitk_gemm(wl.X[j:j + 1], wl.A, y, 8, detred.workspace(1, R, H, 8, dev))
        cmp(y, ref[j:j + 1])
    # dense: prefixes, split 4 vs policy
    for M in (1, 16, 128):
        y = torch.empty((M, F), dtype=f32, device=dev)
        detred.det_splitk_gemm(wl.X[:M], wl.W, y, 0, detred.workspace(M, F, H, 0, dev))
        cmp(y, wl.y_dns[:M])
    y = torch.empty((B, F), dtype=f32, device=dev)
    detred.det_splitk_gemm(wl.X, wl.W, y, 4, detred.workspace(B, F, H, 4, dev))
    cmp(y, wl.y_dns)
    # tree-TP: T = 1, 2, 4 vs the step's T = 8
    for T in (1, 2, 4):
        y = torch.empty((TP_M, TP_N), dtype=f32, device=dev)
        detred.tree_tp_gemm(wl.Xt, wl.Wt, y, T, detred.workspace(TP_M, TP_N, TP_K, T, dev))
        cmp(y, wl.y_tp)
    # row ops: prefixes
    for Bp in (1, 16):
        y = torch.empty((Bp, H), dtype=f32, device=dev)
        detred.inv_rmsnorm(wl.x[:Bp], wl.g, y, 1e-6)
        cmp(y, wl.y_rms[:Bp])
        y = torch.empty((Bp, V), dtype=f32, device=dev)
        detred.inv_log_softmax(wl.lg[:Bp], y)
        cmp(y, wl.y_lsm[:Bp])
        y = torch.empty((Bp,), dtype=f32, device=dev)
        detred.inv_mean(wl.lg[:Bp], y)
        cmp(y, wl.y_mean[:Bp])
    torch.cuda.synchronize()
    return same, total


def tp_breakdown(wl, dev, stream):
    """tree_tp per shard count, the shard kernel alone at its share shape,
    and the combine alone (medians, microseconds)."""
    out = {}
    for T in (1, 2, 4, 8):
        ws = detred.workspace(TP_M, TP_N, TP_K, T, dev)
        y = torch.empty((TP_M, TP_N), dtype=torch.float32, device=dev)
        out["T%d_us" % T] = round(median_time_us(
            detred.prepare(detred.tree_tp_gemm, wl.Xt, wl.Wt, y, T, ws), 20, stream, warm=3)[0], 1)
    Kt = TP_K // TP_T
    Xs = wl.Xt[:, :Kt].contiguous()
    Ws = wl.Wt[:Kt].contiguous()
    P = torch.empty((TP_T, TP_M, TP_N), dtype=torch.float32, device=dev)
    out["shard_share_shape_us"] = round(median_time_us(
        detred.prepare(detred.tree_tp_shard_gemm, Xs, Ws, P[0], TP_T), 20, stream, warm=3)[0], 1)
    y = torch.empty((TP_M, TP_N), dtype=torch.float32, device=dev)
    out["combine_T8_us"] = round(median_time_us(
        detred.prepare(detred.tree_combine_f32, P, y), 20, stream, warm=3)[0], 1)
    return out


def divergence(dev, stream):
    """Replay divergence of det vs atomic split-K=8 over 100 replays on the
    LoRA shrink shapes: the share of replays 1..99 that differ anywhere from
    replay 0, the number of distinct outputs among the 100, and the mean
    fraction of elements that differ from replay 0."""
    out = {}
    for (M, K, r) in [(16, 512, 16), (256, 4096, 64)]:
        X, A, _ = inputs.lora_inputs(M, K, r, 0)
        Xd, Ad = d16(X, dev), d16(A, dev)
        Y = torch.empty((M, r), dtype=torch.float32, device=dev)
        ws = detred.workspace(M, r, K, 8, dev)
        res = {}
        for name, fn in (("det8", detred.prepare(detred.det_splitk_gemm, Xd, Ad, Y, 8, ws)),
                         ("atomic8", detred.prepare(detred.atomic_splitk_gemm, Xd, Ad, Y, 8))):
            outs = []
            for _ in range(100):
                fn()
                outs.append(Y.view(torch.int32).clone())
            torch.cuda.synchronize()
            ref = outs[0]
            differ = [int((o != ref).sum()) for o in outs[1:]]
            hashes = {hashlib.sha256(o.cpu().numpy().tobytes()).hexdigest() for o in outs}
            res[name] = {"replays_differing_pct": round(100.0 * sum(d > 0 for d in differ) / 99, 2),
                         "distinct_outputs": len(hashes),
                         "mean_elements_differing_pct": round(100.0 * sum(differ) / 99 / ref.numel(), 3)}
        out["%dx%dx%d" % (M, r, K)] = res
    return out


def extensions(dev, stream):
    """The next-row operations, timed alone (median/p10/p90 of 50 launches):
    the one-call LoRA layer (hidden 4096, rank 64, batch 256), addmm with a
    bias row into a bf16 output on the dense shape, the dense product and
    the tree-TP shard roots with their weights in the linear-layer layout,
    decode attention with the fixed 256-position KV split, and bf16
    RMSNorm."""
    out = {}
    gb = 2

    def record(name, fn, flops, nbytes):
        med, p10, p90 = median_time_us(fn, 50, stream, warm=5)
        st = {"median_us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
              "gbs": round(nbytes / (med * 1e-6) / 1e9, 1)}
        if flops:
            st["tflops"] = round(flops / (med * 1e-6) / 1e12, 2)
        if flops and flops / nbytes >= RIDGE:
            st["roofline"] = {"bound": "mfma", "frac": round(flops / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        else:
            st["roofline"] = {"bound": "hbm", "frac": round(nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        st["algorithmic_bytes"] = nbytes
        out[name] = st

    X, W, A, Bm = inputs.lora_layer_inputs(B, H, H, R, 0)
    Xd, Wd, Ad, Bd = (d16(t, dev) for t in (X, W, A, Bm))
    Y = torch.empty((B, H), dtype=torch.int16, device=dev)
    ws = detred.lora_workspace(B, H, H, R, dev)
    record("lora_layer_%dx%dx%d_r%d" % (B, H, H, R),
           detred.prepare(detred.det_lora_forward, Xd, Wd, Ad, Bd, Y, 2.0, ws),
           2 * B * H * H + 2 * B * H * R + 2 * B * R * H,
           B * H * gb + H * H * gb + H * R * gb + R * H * gb + B * H * gb)
    _, Wdn = inputs.dense_inputs(B, H, F, 0)
    Wdd = d16(Wdn, dev)
    Xdd = d16(inputs.dense_inputs(B, H, F, 0)[0], dev)
    bias = torch.from_numpy(inputs.bias_inputs(F, 0)).to(dev)
    Yb = torch.empty((B, F), dtype=torch.int16, device=dev)
    record("addmm_bias_bf16_%dx%dx%d" % (B, F, H),
           detred.prepare(detred.det_splitk_addmm, Xdd, Wdd, Yb, bias, 1.0, 1.0, 0,
                          detred.workspace(B, F, H, 0, dev)),
           2 * B * H * F, B * H * gb + H * F * gb + F * 4 + B * F * gb)
    # the dense product with its weight stored as a linear layer keeps it
    # ([out, in] = [14336, 4096], K contiguous; the same values): the
    # transposed-weight kernels read both operands with ds_read_b128
    Wtd = Wdd.t().contiguous()
    Yd = torch.empty((B, F), dtype=torch.float32, device=dev)
    record("dense_linear_weight_%dx%dx%d" % (B, F, H),
           detred.prepare(detred.det_splitk_gemm, Xdd, Wtd.t(), Yd, 0,
                          detred.workspace(B, F, H, 0, dev)),
           2 * B * H * F, B * H * gb + H * F * gb + B * F * 4)
    del Wtd
    # the shard roots of the tree-TP product with the weight of a
    # row-parallel linear layer ([8192, 8192] = [out, in], K contiguous)
    Xt, Wt = inputs.dense_inputs(TP_M, TP_K, TP_N, 0)
    Xtd, Wtt = d16(Xt, dev), d16(Wt, dev).t().contiguous()
    Pt = torch.empty((TP_T, TP_M, TP_N), dtype=torch.float32, device=dev)
    record("tp_shards_linear_weight_%dx%dx%d_t%d" % (TP_M, TP_N, TP_K, TP_T),
           detred.prepare(detred.tree_tp_shards_gemm, Xtd, Wtt.t(), Pt, TP_T),
           2 * TP_M * TP_K * TP_N, TP_M * TP_K * gb + TP_K * TP_N * gb + TP_M * TP_N * 4)
    del Wtt, Pt
    # decode attention: 8B-class GQA (32 query heads, 8 KV heads, head dim
    # 128), 64 sequences of 4096 cached positions; the 1 GiB cache is drawn
    # on the device from a seeded generator
    AB, AHq, AHkv, AD, AL = 64, 32, 8, 128, 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    qa = torch.randn((AB, AHq, AD), device=dev, generator=gen).to(torch.bfloat16)
    ka = torch.randn((AB, AHkv, AL, AD), device=dev, generator=gen).to(torch.bfloat16)
    va = torch.randn((AB, AHkv, AL, AD), device=dev, generator=gen).to(torch.bfloat16)
    la = torch.full((AB,), AL, dtype=torch.int32, device=dev)
    oa = torch.empty((AB, AHq, AD), dtype=torch.float32, device=dev)
    wsa = detred.attention_workspace(AB, AHq, AD, AL, dev)
    record("decode_attention_b%d_hq%d_hkv%d_d%d_len%d" % (AB, AHq, AHkv, AD, AL),
           detred.prepare(detred.inv_decode_attention, qa, ka, va, la, oa, AD ** -0.5, wsa),
           4 * AB * AHq * AL * AD, 2 * AB * AHkv * AL * AD * gb + AB * AHq * AD * (gb + 4))
    del qa, ka, va
    x, g = inputs.rmsnorm_inputs(B, H, 0)
    yr = torch.empty((B, H), dtype=torch.int16, device=dev)
    record("rmsnorm_bf16_%dx%d" % (B, H),
           detred.prepare(detred.inv_rmsnorm_bf16, d16(x, dev), d16(g, dev), yr, 1e-6),
           0, B * H * gb + H * gb + B * H * gb)
    return out


def config_sweep(dev, stream):
    """The measurement table of the configurations: each call timed alone
    (median of 20 after 3 warm-ups, HIP events), with its roofline time
    max(flop / 2.5 PF/s, algorithmic bytes / 8 TB/s) and the fraction
    roofline / measured.  Inputs are drawn on the device from seeded
    generators with the configurations' distributions."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    gb = 2
    out = {}
    flush = torch.ones((128 << 20,), dtype=torch.float32, device=dev)

    def bf(shape, std):
        return (torch.randn(shape, device=dev, generator=gen) * std).to(torch.bfloat16)

    def rec(name, fn, flops, nbytes):
        med = median_time_us(fn, 20, stream, warm=3)[0]
        cold = cold_time_us(fn, 10, stream, flush)
        roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        out[name] = {"us": round(med, 2), "us_cold": round(cold, 2), "roofline_us": round(roof, 2),
                     "bound": "mfma" if flops / max(nbytes, 1) >= RIDGE else "hbm",
                     "frac": round(roof / med, 4), "frac_cold": round(roof / cold, 4)}

    # LoRA shrink (det split-K = 8) and expand, M x r
    for r in (16, 64):
        A = bf((H, r), 0.02)
        Bm = bf((r, H), 0.02)
        for M in (1, 8, 64, 256):
            X = bf((M, H), 1.0)
            Y = torch.empty((M, r), dtype=torch.float32, device=dev)
            rec("shrink_m%d_r%d" % (M, r),
                detred.prepare(detred.det_splitk_gemm, X, A, Y, 8, detred.workspace(M, r, H, 8, dev)),
                2 * M * H * r, M * H * gb + H * r * gb + M * r * 4)
            Z = torch.empty((M, H), dtype=torch.float32, device=dev)
            Yb = bf((M, r), 1.0)
            rec("expand_m%d_r%d" % (M, r), detred.prepare(detred.det_splitk_gemm, Yb, Bm, Z, 0),
                2 * M * r * H, M * r * gb + r * H * gb + M * H * 4)
    # dense X[M,4096] W[4096,14336], automatic split
    W = bf((H, F), 0.02)
    for M in (1, 16, 128, 1024, 4096):
        X = bf((M, H), 1.0)
        Y = torch.empty((M, F), dtype=torch.float32, device=dev)
        rec("dense_m%d" % M, detred.prepare(detred.det_splitk_gemm, X, W, Y, 0,
                                            detred.workspace(M, F, H, 0, dev)),
            2 * M * H * F, M * H * gb + H * F * gb + M * F * 4)
    del W
    # tree-TP X[512,8192] W[8192,8192], both phases
    Xt, Wt = bf((TP_M, TP_K), 1.0), bf((TP_K, TP_N), 0.02)
    Yt = torch.empty((TP_M, TP_N), dtype=torch.float32, device=dev)
    for T in (1, 2, 4, 8):
        rec("tree_tp_T%d" % T, detred.prepare(detred.tree_tp_gemm, Xt, Wt, Yt, T,
                                             detred.workspace(TP_M, TP_N, TP_K, T, dev)),
            2 * TP_M * TP_K * TP_N, TP_M * TP_K * gb + TP_K * TP_N * gb + TP_M * TP_N * 4)
    del Xt, Wt
    # row ops
    g = (1.0 + 0.1 * torch.randn((H,), device=dev, generator=gen)).to(torch.bfloat16)
    for Bn in (1, 16, 256, 4096):
        x = bf((Bn, H), 1.0)
        y = torch.empty((Bn, H), dtype=torch.float32, device=dev)
        rec("rmsnorm_b%d" % Bn, detred.prepare(detred.inv_rmsnorm, x, g, y, 1e-6),
            0, Bn * H * gb + H * gb + Bn * H * 4)
    for Bn in (256, 4096):
        lg = torch.randn((Bn, V), device=dev, generator=gen) * 3.0
        ys = torch.empty_like(lg)
        rec("log_softmax_b%d" % Bn, detred.prepare(detred.inv_log_softmax, lg, ys), 0, 2 * Bn * V * 4)
        del ys
        ym = torch.empty((Bn,), dtype=torch.float32, device=dev)
        rec("mean_b%d" % Bn, detred.prepare(detred.inv_mean, lg, ym), 0, Bn * V * 4 + Bn * 4)
        ys = torch.empty_like(lg)
        rec("log_softmax_mean_b%d" % Bn,
            detred.prepare(detred.inv_log_softmax_mean, lg, ys, ym), 0, 2 * Bn * V * 4 + Bn * 4)
        del ys
        del lg
    return out


def source_hash():
    """Hash of the kernel sources, to tell whether committed counter data
    were taken on the kernels that run now."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_reduction_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_op):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("ops", {}).get(kernel_op)


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands, on the host cores: one full step of the same
    workload (every row of every operation), repeated until min_seconds."""
    import oracle
    h = wl.host
    flops = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.rmsnorm(h["x"], h["g"], 1e-6)
        y, _ = oracle.gemm(h["X"], h["A"], with_magnitude=False)
        yb = oracle.f32_to_bf16(y.astype(np.float32))
        oracle.gemm(yb, h["B"], with_magnitude=False)
        oracle.gemm(h["X"], h["W"], with_magnitude=False)
        oracle.gemm(h["Xt"], h["Wt"], with_magnitude=False)
        oracle.log_softmax(h["lg"])
        oracle.mean(h["lg"])
        flops += 2 * B * H * R * 2 + 2 * B * H * F + 2 * TP_M * TP_K * TP_N
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": "%d full step(s) of the same workload in fp64 (all rows of shrink, expand, "
                      "dense, tree-TP, rmsnorm, log_softmax, mean); %.1f s" % (reps, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="only the timed steps (for profiler runs): no ratios, "
                         "invariance checks, breakdown or CPU baseline")
    ap.add_argument("--serial", action="store_true",
                    help="issue every op on the main stream (no overlap between kernels, "
                         "so a profiler's per-kernel durations match the per-op timings)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    detred.lib()
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print("bench: generating inputs", file=sys.stderr, flush=True)
    wl = Workload(dev)
    # the step's three independent chains on three streams (default
    # priority), and the same ops all on the main stream for the serial
    # step and the per-op timings
    lanes = [stream, torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    if args.serial:
        lanes = [stream]
    ops = wl.ops(lanes * 3 if args.serial else lanes)
    serial_ops = wl.ops([stream, stream, stream])
    step = Step(ops, lanes)
    serial = Step(serial_ops, [stream])
    for _ in range(args.warmup):
        step()
        serial()
    torch.cuda.synchronize()
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)

    total_ms = time_steps(step, args.steps, stream)
    ms_per_step = total_ms / args.steps
    ms_serial = time_steps(serial, args.steps, stream) / args.steps
    per_op = time_ops(serial_ops, args.steps, stream)
    det_flops = sum(op[2] for op in ops)
    value = det_flops / (ms_per_step * 1e-3) / 1e12

    op_stats = {}
    for (name, _, fl, by, _), ts in zip(ops, per_op):
        avg = sum(ts) / len(ts)
        srt = sorted(ts)
        st = {"avg_us": round(avg * 1000, 2), "median_us": round(statistics.median(ts) * 1000, 2),
              "p10_us": round(srt[len(srt) // 10] * 1000, 2),
              "p90_us": round(srt[(9 * len(srt)) // 10] * 1000, 2)}
        if fl:
            st["tflops"] = round(fl / (avg * 1e-3) / 1e12, 2)
        st["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
        op_stats[name] = st
    dom_i = max(range(len(ops)), key=lambda i: sum(per_op[i]))
    dname, _, dfl, dby, _ = ops[dom_i]
    davg_s = sum(per_op[dom_i]) / len(per_op[dom_i]) * 1e-3
    if dfl and dfl / dby >= RIDGE:
        roof = {"bound": "mfma", "achieved": round(dfl / davg_s / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dby / davg_s / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dname)
    roof["kernel"] = dname

    ratios = tp = div = ext = sweep = None
    same = total = 0
    if not args.quick:
        print("bench: latency ratios, invariance, tree-TP breakdown", file=sys.stderr, flush=True)
        ratios = latency_ratios(dev, stream)
        same, total = invariance(wl, dev)
        tp = tp_breakdown(wl, dev, stream)
        div = divergence(dev, stream)
        print("bench: next-row operations", file=sys.stderr, flush=True)
        ext = extensions(dev, stream)
        print("bench: configuration sweep", file=sys.stderr, flush=True)
        sweep = config_sweep(dev, stream)

    # replays: every deterministic output is reproduced bit for bit; the
    # atomic control is counted
    ref = {k: getattr(wl, k).clone() for k in ("y_shr", "y_dns", "y_tp", "y_lsm", "y_mean", "y_rms")}
    atom0 = None
    det_same = atom_diff = 0
    for r in range(20):
        step()
        torch.cuda.synchronize()
        det_same += all(torch.equal(getattr(wl, k).view(torch.int32), v.view(torch.int32))
                        for k, v in ref.items())
        a = wl.y_atm.clone()
        if atom0 is None:
            atom0 = a
        else:
            atom_diff += not torch.equal(a.view(torch.int32), atom0.view(torch.int32))

    cpu = None
    if not args.no_cpu_baseline and not args.quick:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    line = {
        "metric": "det split-K GEMM TFLOP/s & latency vs atomic; % rows bit-invariant across M/TP",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_serial": round(ms_serial, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/N(0,0.02)/N(1,0.1)/N(0,3) inputs of the 8B-like shapes)",
        "config": {"workload": WORKLOAD, "global_batch": B, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ops": op_stats,
        "det_vs_atomic": ratios,
        "replay_divergence": div,
        "extensions": ext,
        "configs": sweep,
        "tree_tp_breakdown": tp,
        "bit_invariant_rows_pct": round(100.0 * same / max(total, 1), 4),
        "bit_invariant_rows_checked": total,
        "det_replays_identical": "%d/20" % det_same,
        "atomic_replays_differing": "%d/19" % atom_diff,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
