#!/usr/bin/env python3
"""Benchmark of the Sparse-BitNet BitLinear hot path on one MI355X.

Prints ONE JSON line.  The headline (`value`) is decode GB/s at 6:8 on the
Qwen2.5-0.5B-shaped workload: one token through a 24-layer stack of the
layer's seven BitLinear projections (q 896->896, k/v 896->128, o 896->896,
gate/up 896->4864, down 4864->896), i.e. 168 GEMVs per step, run as one
grouped launch pair (activation quantisation, then contraction).  Attention,
norms and the other glue are out of scope, so every projection gets its own
synthetic N(0,1) input; the grouping is labelled in `config`.  The packed
weights rotate over a pool of distinct device copies larger than twice the
256 MB Infinity Cache, so every step streams its weights from HBM.

Extra sections (same JSON line): the 6:8-over-8:8 speedup on the same
kernels, per-projection single-call latency, the prefill step of the
Qwen2.5-1.5B shape (mask recompute + pack + int8 GEMM), a BitNet-2B4T block
training step (7 BitLinears fwd + dual-STE bwd), and the CPU oracle timed on
a bounded sample of the decode workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # dense int8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA, published

QWEN05_LAYER = [  # (name, n_out, k)
    ("q", 896, 896), ("k", 128, 896), ("v", 128, 896), ("o", 896, 896),
    ("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864),
]
QWEN05_LAYERS = 24
QWEN15_PREFILL = [("gate", 8960, 1536), ("up", 8960, 1536), ("down", 1536, 8960)]
BITNET2B_BLOCK = [
    ("q", 2560, 2560), ("k", 640, 2560), ("v", 640, 2560), ("o", 2560, 2560),
    ("gate", 6912, 2560), ("up", 6912, 2560), ("down", 2560, 6912),
]


# HBM bytes of one launch of the grouped decode contraction (6:8), from two
# rocprofv3 --pmc runs of `bench.py --quick` (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, mean of 66 dispatches), scaled by what the same
# counters read for a plain 256 MiB device copy (FETCH_SIZE 131084 KiB per
# copy -> x2.0; WRITE_SIZE 262144 KiB -> x1.0).  Valid only for the kernel
# sources it was taken on (their SHA-256 below); otherwise reported as null.
DECODE_TRAFFIC = {
    "sources": ["sparse_linear_layers_group_amd/csrc/gemv.hip",
                "sparse_linear_layers_group_amd/csrc/common.h",
                "sparse_linear_layers_group_amd/csrc/launch.h"],
    "sha256": "15dd177c999cbbe3ef9470b5e52b62aadb3a75990f1a7daba7ed02302f01b6f8",
    "fetch_kib": 39918.6, "fetch_scale": 2.0,
    "write_kib": 1188.0, "write_scale": 1.0,
}


def decode_traffic_bytes():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != DECODE_TRAFFIC["sha256"]:
        return None
    t = DECODE_TRAFFIC
    return round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (no extra sections)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (reference for the HBM byte counters)")
    ap.add_argument("--library-reference", action="store_true",
                    help="only time the vendor library's dense GEMMs (torch -> hipBLASLt) at the "
                         "prefill and backward shapes, as context for the roofline fractions")
    return ap.parse_args()


def library_reference(torch, reps=10):
    """Dense bf16 and int8 GEMMs of the vendor library at the shapes this
    path contracts (C[M x N] = A[M x K] B[N x K]^T), timed like the kernels.
    Context only: nothing of the path runs through them."""
    shapes = [("prefill gate/up", 2048, 8960, 1536), ("prefill down", 2048, 1536, 8960),
              ("bwd dX gate", 4096, 2560, 6912), ("bwd dW gate", 6912, 2560, 4096)]
    out = []
    for name, M, N, K in shapes:
        a = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(N, K, dtype=torch.bfloat16, device="cuda")
        ai = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        bi = torch.randint(-1, 2, (N, K), dtype=torch.int8, device="cuda")
        row = {"shape": name, "M": M, "N": N, "K": K}
        for kind, f, peak in (("bf16", lambda: a @ b.t(), BF16_PEAK_TFLOPS),
                              ("int8", lambda: torch._int_mm(ai, bi.t()), INT8_PEAK_TOPS)):
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            with Timer(torch) as t:
                for _ in range(reps):
                    f()
            tops = 2 * M * N * K / (t.ms() / reps * 1e-3) / 1e12
            row[kind] = {"us": round(1000 * t.ms() / reps, 1), "tops": round(tops, 1),
                         "frac": round(tops / peak, 4)}
        out.append(row)
    print(json.dumps({"library_reference": out}), flush=True)


def copy_calibration(torch, reps=5):
    """Plain device-to-device copies of a known size: under rocprofv3 --pmc
    their FETCH_SIZE / WRITE_SIZE per dispatch give the scale from counter
    units to bytes (each copy reads and writes 256 MiB)."""
    n = 256 * 2 ** 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "dispatches": reps}}), flush=True)


def packed_bytes(n_out, k, n, m):
    from sparse_linear_layers_group_amd import bitlinear as bl
    return bl.bitlinear_packed_bytes(n_out, k, n, m)


class Timer:
    """HIP events on torch's current stream (the stream the library's
    kernels are launched on)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()

    def ms(self):
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


# --------------------------------------------------------------- decode
def build_decode(torch, bl, n, m, tokens=1):
    """Weights of one Qwen2.5-0.5B-shaped layer (synthetic N(0, 0.02)),
    quantised and packed on the GPU, replicated into a rotating pool of
    distinct device buffers; one grouped plan per pool copy."""
    from sparse_linear_layers_group_amd import synth
    from sparse_linear_layers_group_amd.layer import BitLinearWeight, bf16_tensor

    packs = []
    for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
        lw = BitLinearWeight(n_out, k, n, m)
        lw.quantize(bf16_tensor(synth.weights(n_out, k, seed=0, config=2, layer=li)))
        packs.append(lw)
    torch.cuda.synchronize()
    stack_bytes = QWEN05_LAYERS * sum(p.packed.numel() for p in packs)
    copies = max(2, -(-2 * 256 * 2 ** 20 // stack_bytes) + 0)  # > 2x the 256 MB cache
    # activations: distinct synthetic inputs per (layer, projection), shared by pool copies
    xs, ys, xqs, scs = [], [], [], []
    for L in range(QWEN05_LAYERS):
        for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
            xs.append(bf16_tensor(synth.activations(tokens, k, seed=1 + L, config=2, layer=li)))
            ys.append(torch.empty(tokens * n_out, dtype=torch.float32, device="cuda"))
            xqs.append(torch.empty(tokens * k, dtype=torch.int8, device="cuda"))
            scs.append(torch.empty(tokens, dtype=torch.float32, device="cuda"))
    plans, keep = [], []
    for c in range(copies):
        entries = []
        for L in range(QWEN05_LAYERS):
            for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
                buf = packs[li].packed.clone()  # a distinct copy at its own address
                keep.append(buf)
                i = L * len(QWEN05_LAYER) + li
                entries.append(dict(X=xs[i], packed=buf, gamma=packs[li].gamma, Y=ys[i], xq=xqs[i],
                                    x_scale=scs[i], k=k, n_out=n_out))
        items = bl.make_fwd_items(entries, tokens)
        nbytes = bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens)
        plan = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
        plans.append(plan)
    torch.cuda.synchronize()
    per_step = {
        "packed": QWEN05_LAYERS * sum(p.packed.numel() for p in packs),
        "x_bf16": QWEN05_LAYERS * sum(2 * tokens * k for _, _, k in QWEN05_LAYER),
        "x_int8": QWEN05_LAYERS * sum(tokens * k for _, _, k in QWEN05_LAYER),
        "y": QWEN05_LAYERS * sum(4 * tokens * n for _, n, _ in QWEN05_LAYER),
    }
    return dict(packs=packs, plans=plans, keep=keep, copies=copies, per_step=per_step,
                pool_bytes=copies * stack_bytes, ys=ys)


def time_decode(torch, bl, d, n, m, steps, warmup):
    plans = d["plans"]
    for i in range(warmup):
        bl.bitlinear_fwd_group(plans[i % len(plans)], n, m, 3)
    torch.cuda.synchronize()
    # whole steps, back to back
    with Timer(torch) as t_all:
        for i in range(steps):
            bl.bitlinear_fwd_group(plans[i % len(plans)], n, m, 3)
    ms_total = t_all.ms()
    # the contraction kernel alone, per launch (events around each launch)
    evs = []
    for i in range(steps):
        bl.bitlinear_fwd_group(plans[i % len(plans)], n, m, 1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        bl.bitlinear_fwd_group(plans[i % len(plans)], n, m, 2)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    gemv_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    # the contraction alone, back to back (activations quantised once per plan)
    for p in plans:
        bl.bitlinear_fwd_group(p, n, m, 1)
    with Timer(torch) as t_b2b:
        for i in range(steps):
            bl.bitlinear_fwd_group(plans[i % len(plans)], n, m, 2)
    return ms_total / steps, gemv_ms, t_b2b.ms() / steps


def single_call_latency(torch, bl, d, iters=200):
    """Per-projection bitlinear_fwd latency at 1 token (weights rotating over
    the pool copies, so each call streams from HBM)."""
    from sparse_linear_layers_group_amd import synth
    from sparse_linear_layers_group_amd.layer import bf16_tensor
    out = {}
    nproj = len(QWEN05_LAYER)
    for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
        lw = d["packs"][li]
        X = bf16_tensor(synth.activations(1, k, seed=5, config=2, layer=li))
        bufs = lw.fwd_buffers(1)
        copies = [d["keep"][j] for j in range(li, len(d["keep"]), nproj)]
        for i in range(20):
            bl.bitlinear_fwd(X, 1, k, copies[i % len(copies)], n_out, lw.n, lw.m, lw.gamma, bufs["Y"],
                             bufs["xq"], bufs["x_scale"], ws=bufs["ws"])
        torch.cuda.synchronize()
        with Timer(torch) as t:
            for i in range(iters):
                bl.bitlinear_fwd(X, 1, k, copies[i % len(copies)], n_out, lw.n, lw.m, lw.gamma,
                                 bufs["Y"], bufs["xq"], bufs["x_scale"], ws=bufs["ws"])
        out[name] = round(1000.0 * t.ms() / iters, 2)
    return out


def verify_decode_sample(torch, d, n, m):
    """Sampled check of the grouped results against the oracle (one layer)."""
    import numpy as np
    import oracle
    from sparse_linear_layers_group_amd import synth
    bl_plan = d["plans"][0]
    from sparse_linear_layers_group_amd import bitlinear as bl
    bl.bitlinear_fwd_group(bl_plan, n, m, 3)
    torch.cuda.synchronize()
    worst = 0.0
    for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
        W = synth.weights(n_out, k, seed=0, config=2, layer=li)
        X = synth.activations(1, k, seed=1, config=2, layer=li)  # layer L = 0
        mb = oracle.mask(W, n, m)
        g = oracle.gamma(W)
        T = oracle.ternary(W, mb, g)
        xq, sc = oracle.act_quant(X)
        _, Yref = oracle.fwd(xq, sc, T, g)
        Y = d["ys"][li].cpu().numpy().astype(np.float64)
        err = np.abs(Y - Yref[0])
        ok = np.all(err <= 1e-5 * np.abs(Yref[0]))
        if not ok:
            raise RuntimeError(f"decode result mismatch on {name}")
        worst = max(worst, float(np.max(err / np.maximum(np.abs(Yref[0]), 1e-30))))
    return worst


# --------------------------------------------------------------- prefill / train
def prefill_step(torch, bl, n, m, tokens=2048, iters=10):
    """Qwen2.5-1.5B-shaped prefill: per step, mask recompute + pack of gate,
    up and down (one grouped plan), activation quantisation, int8 GEMMs."""
    from sparse_linear_layers_group_amd import synth
    from sparse_linear_layers_group_amd.layer import BitLinearWeight, QuantGroup, bf16_tensor
    Ws, lws, bufs = [], [], []
    for li, (name, n_out, k) in enumerate(QWEN15_PREFILL):
        Ws.append(bf16_tensor(synth.weights(n_out, k, seed=0, config=3, layer=li)))
        lws.append(BitLinearWeight(n_out, k, n, m))
        bufs.append(lws[-1].fwd_buffers(tokens))
    X1 = bf16_tensor(synth.activations(tokens, 1536, seed=0, config=3, layer=0))
    X2 = bf16_tensor(synth.activations(tokens, 8960, seed=0, config=3, layer=2))
    xs = [X1, X1, X2]

    qg = QuantGroup(list(zip(lws, Ws)))  # plan built once; each step: three launches

    def quant():
        qg.run()

    def act():
        bl.bitlinear_act_quant(X1, tokens, 1536, bufs[0]["xq"], bufs[0]["x_scale"])
        bl.bitlinear_act_quant(X2, tokens, 8960, bufs[2]["xq"], bufs[2]["x_scale"])

    def gemm():
        for i, lw in enumerate(lws):
            src = bufs[0] if i == 1 else bufs[i]
            bl.bitlinear_contract(src["xq"], src["x_scale"], tokens, lw.k, lw.packed, lw.n_out, n, m,
                                  lw.gamma, bufs[i]["Y"], ws=bufs[i]["ws"])

    for f in (quant, act, gemm):
        f()
    torch.cuda.synchronize()
    res = {}
    for name, f in (("mask_pack_ms", quant), ("act_quant_ms", act), ("gemm_ms", gemm)):
        with Timer(torch) as t:
            for _ in range(iters):
                f()
        res[name] = t.ms() / iters
    ops = sum(2 * tokens * n_out * k for _, n_out, k in QWEN15_PREFILL)
    wts = sum(n_out * k for _, n_out, k in QWEN15_PREFILL)
    res["gemm_tops_issued"] = ops / (res["gemm_ms"] * 1e-3) / 1e12
    res["gemm_tops_algorithmic"] = res["gemm_tops_issued"] * n / m
    res["gemm_frac_int8_peak"] = res["gemm_tops_issued"] / INT8_PEAK_TOPS
    # mask + pack: reads W twice (mask pass, pack pass) + mask write/read + packed write
    mp_bytes = wts * (2 + 2 + 0.125 + 0.125) + sum(packed_bytes(n_out, k, n, m) for _, n_out, k in QWEN15_PREFILL)
    res["mask_pack_gbs"] = mp_bytes / (res["mask_pack_ms"] * 1e-3) / 1e9
    res["step_ms"] = res["mask_pack_ms"] + res["act_quant_ms"] + res["gemm_ms"]
    return {k2: round(v, 4) for k2, v in res.items()}


def train_step(torch, bl, n, m, tokens=4096, iters=3):
    """BitNet-b1.58-2B4T-shaped block: all 7 BitLinears, per step mask +
    pack (one grouped plan), forward (int8 MFMA), dual-STE backward (bf16
    MFMA) and the latent-weight update (plain gradient step on binary32
    latent weights, writing the bf16 W the next step's mask reads).  The
    feed-forward is chained: squared-ReLU gating of the gate/up outputs
    forms the down projection's int8 input, and its backward turns the down
    projection's dX into the gate/up dY."""
    from sparse_linear_layers_group_amd import synth
    from sparse_linear_layers_group_amd.layer import BitLinearWeight, LatentWeights, QuantGroup, bf16_tensor
    hid = 2560
    Ws, lws, fb, dys, gx, gw = [], [], [], [], [], []
    for li, (name, n_out, k) in enumerate(BITNET2B_BLOCK):
        Ws.append(bf16_tensor(synth.weights(n_out, k, seed=0, config=5, layer=li)))
        lws.append(BitLinearWeight(n_out, k, n, m))
        fb.append(lws[-1].fwd_buffers(tokens))
        dys.append(bf16_tensor(synth.grad_output(tokens, n_out, seed=0, config=5, layer=li)))
        gx.append(torch.empty(tokens * k, dtype=torch.float32, device="cuda"))
        gw.append(torch.empty(n_out * k, dtype=torch.float32, device="cuda"))
    # q/k/v and gate/up read the same block input, quantised once;
    # attention and norms are out of scope, so o gets its own synthetic
    # input; down reads the gating of gate and up
    X = bf16_tensor(synth.activations(tokens, hid, seed=0, config=5, layer=0))
    Xo = bf16_tensor(synth.activations(tokens, hid, seed=0, config=5, layer=3))
    src = [0, 0, 0, 3, 0, 0, 6]  # which layer's x_q buffer each layer reads
    ffn = 6912

    qg = QuantGroup(list(zip(lws, Ws)))  # plan built once; each step: three launches

    def quant():
        qg.run()

    def contract(i):
        lw, a = lws[i], fb[src[i]]
        bl.bitlinear_contract(a["xq"], a["x_scale"], tokens, lw.k, lw.packed, lw.n_out, n, m,
                              lw.gamma, fb[i]["Y"], ws=fb[i]["ws"])

    def fwd():
        for i, x in ((0, X), (3, Xo)):
            bl.bitlinear_act_quant(x, tokens, lws[i].k, fb[i]["xq"], fb[i]["x_scale"])
        for i in range(6):
            contract(i)
        bl.bitlinear_relu2_gate(fb[4]["Y"], fb[5]["Y"], tokens, ffn, None, fb[6]["xq"], fb[6]["x_scale"])
        contract(6)

    # one backward workspace, sized for the largest layer (calls run in order on one stream)
    bws = torch.empty(max(bl.bitlinear_bwd_workspace_bytes(tokens, lw.k, lw.n_out) for lw in lws),
                      dtype=torch.uint8, device="cuda")

    def bwd_layer(i):
        lw, a = lws[i], fb[src[i]]
        bl.bitlinear_bwd(dys[i], a["xq"], a["x_scale"], lw.packed, lw.gamma, tokens, lw.k,
                         lw.n_out, n, m, gx[i], gw[i], ws=bws)

    def bwd():
        bwd_layer(6)  # down (synthetic dY), then the gating backward: dY of gate and up
        bl.bitlinear_relu2_gate_bwd(gx[6], fb[4]["Y"], fb[5]["Y"], tokens * ffn, dys[4], dys[5])
        for i in (4, 5, 3, 0, 1, 2):
            bwd_layer(i)

    # binary32 latent weights; the update writes the bf16 W the plan reads
    lats = [LatentWeights(W) for W in Ws]
    assert all(lat.W.data_ptr() == W.data_ptr() for lat, W in zip(lats, Ws))

    def update():
        for i, lat in enumerate(lats):
            lat.update(gw[i], 1e-3)

    for f in (quant, fwd, bwd, update):
        f()
    torch.cuda.synchronize()
    res = {}
    for name, f in (("mask_pack_ms", quant), ("fwd_ms", fwd), ("bwd_ms", bwd), ("update_ms", update)):
        with Timer(torch) as t:
            for _ in range(iters):
                f()
        res[name] = t.ms() / iters
    mac = sum(tokens * n_out * k for _, n_out, k in BITNET2B_BLOCK)
    res["fwd_tops_issued"] = 2 * mac / (res["fwd_ms"] * 1e-3) / 1e12
    res["bwd_tflops_issued"] = 4 * mac / (res["bwd_ms"] * 1e-3) / 1e12
    res["bwd_frac_bf16_peak"] = res["bwd_tflops_issued"] / BF16_PEAK_TFLOPS
    wts = sum(n_out * k for _, n_out, k in BITNET2B_BLOCK)
    res["update_gbs"] = wts * 14 / (res["update_ms"] * 1e-3) / 1e9  # 4+4 read, 4+2 written per weight
    res["step_ms"] = res["mask_pack_ms"] + res["fwd_ms"] + res["bwd_ms"] + res["update_ms"]
    return {k2: round(v, 4) for k2, v in res.items()}


# --------------------------------------------------------------- CPU baseline
def cpu_baseline(n, m, budget_s=10.0):
    """The oracle (plain C, binary64/exact integer) on a bounded sample of the
    decode workload: repeated single-token forwards of the seven projections
    of one Qwen2.5-0.5B-shaped layer, from int8 codes prepared once."""
    import oracle
    from sparse_linear_layers_group_amd import synth
    codes = []
    for li, (name, n_out, k) in enumerate(QWEN05_LAYER):
        W = synth.weights(n_out, k, seed=0, config=2, layer=li)
        mb = oracle.mask(W, n, m)
        g = oracle.gamma(W)
        codes.append((oracle.ternary(W, mb, g), g, k))
    xs = [synth.activations(1, k, seed=1, config=2, layer=li) for li, (_, _, k) in enumerate(QWEN05_LAYER)]
    layer_bytes = sum(packed_bytes(n_out, k, n, m) + 2 * k + 4 * n_out for _, n_out, k in QWEN05_LAYER)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for (T, g, k), X in zip(codes, xs):
            xq, sc = oracle.act_quant(X)
            oracle.fwd(xq, sc, T, g, threads=1, want_acc=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(layer_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} single-token forwards of one Qwen2.5-0.5B-shaped layer (7 projections, {n}:{m}), "
                      f"act-quant + int64 contraction + binary64 epilogue from int8 codes, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.library_reference:
        library_reference(torch)
        return
    from sparse_linear_layers_group_amd import bitlinear as bl
    if not os.path.exists(bl.LIB_PATH):
        from sparse_linear_layers_group_amd import build
        build.build()
    bl.lib()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name}, {props.multi_processor_count} CUs")

    t_setup = time.perf_counter()
    d68 = build_decode(torch, bl, 6, 8)
    log(f"decode pool: {d68['copies']} copies, {d68['pool_bytes'] / 2**20:.0f} MiB ({time.perf_counter() - t_setup:.1f} s)")
    worst = verify_decode_sample(torch, d68, 6, 8)
    step_ms, gemv_ms, gemv_b2b_ms = time_decode(torch, bl, d68, 6, 8, args.steps, args.warmup)
    ps = d68["per_step"]
    step_bytes = ps["packed"] + ps["x_bf16"] + ps["y"]
    value = step_bytes / (step_ms * 1e-3) / 1e9
    gemv_bytes = ps["packed"] + ps["x_int8"] + ps["y"]
    # kernel time: back-to-back contraction launches (events on the launch
    # stream around the batch); per-launch event pairs add ~2-3 us of event
    # overhead and are reported beside it
    achieved = gemv_bytes / (gemv_b2b_ms * 1e-3) / 1e9
    log(f"decode 6:8: step {step_ms * 1000:.1f} us, {value:.0f} GB/s; contraction {gemv_b2b_ms * 1000:.1f} us, {achieved:.0f} GB/s")

    out = {
        "metric": "6:8 BitLinear GB/s (decode) & int8 TOPS (prefill), % roofline, speedup vs 8:8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Qwen2.5-0.5B-shaped decode, 1 token, 6:8: q 896->896, k/v 896->128, o 896->896, "
                        "gate/up 896->4864, down 4864->896 BitLinear GEMVs x 24 layers = 168 GEMVs per step, "
                        "grouped into one activation-quant launch + one contraction launch",
            "grouped": True,
            "layers_per_step": QWEN05_LAYERS,
            "tokens": 1,
            "pattern": "6:8",
            "weight_pool_MiB": round(d68["pool_bytes"] / 2 ** 20, 1),
            "bytes_per_step": step_bytes,
        },
        "roofline": {
            "kernel": "gemv_group_kernel<6> (grouped decode contraction)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": decode_traffic_bytes(),
            "kernel_us": round(gemv_b2b_ms * 1000, 3),
            "kernel_us_event_pairs": round(gemv_ms * 1000, 3),
            "algorithmic_bytes_per_launch": gemv_bytes,
        },
        "check": {"decode_vs_oracle_max_rel_err": worst},
    }
    if not args.quick:
        d88 = build_decode(torch, bl, 8, 8)
        s88, _, g88 = time_decode(torch, bl, d88, 8, 8, args.steps, args.warmup)
        out["vs_8_8"] = {
            "step_speedup": round(s88 / step_ms, 4),
            "contraction_speedup": round(g88 / gemv_b2b_ms, 4),
            "bytes_ratio": round(d88["per_step"]["packed"] / ps["packed"], 4),
            "step_ms_8_8": round(s88, 5),
            "contraction_us_8_8": round(g88 * 1000, 3),
            "contraction_gbs_8_8": round((d88["per_step"]["packed"] + ps["x_int8"] + ps["y"]) / (g88 * 1e-3) / 1e9, 2),
        }
        log(f"decode 8:8: step {s88 * 1000:.1f} us, contraction {g88 * 1000:.1f} us")
        out["single_call_us"] = single_call_latency(torch, bl, d68)
        p88 = d88["per_step"]["packed"]
        del d88
        # the same decode step at the other patterns the pages sweep (8:8
        # down to 2:8; 2:4 for reference): packed bytes and measured times
        sweep = {}
        for n, m in ((4, 8), (3, 8), (2, 8), (2, 4)):
            dn = build_decode(torch, bl, n, m)
            sn, _, gn = time_decode(torch, bl, dn, n, m, args.steps, args.warmup)
            pk = dn["per_step"]["packed"]
            sweep[f"{n}:{m}"] = {
                "step_us": round(sn * 1000, 3),
                "contraction_us": round(gn * 1000, 3),
                "packed_bytes_per_step": pk,
                "bytes_ratio_vs_8_8": round(p88 / pk, 4),
                "step_speedup_vs_8_8": round(s88 / sn, 4),
                "contraction_speedup_vs_8_8": round(g88 / gn, 4),
            }
            log(f"decode {n}:{m}: step {sn * 1000:.1f} us, contraction {gn * 1000:.1f} us")
            del dn
        out["decode_nm_sweep"] = sweep
        log("prefill ...")
        out["prefill_qwen15_6_8"] = prefill_step(torch, bl, 6, 8)
        out["prefill_qwen15_8_8"] = prefill_step(torch, bl, 8, 8)
        log("train step ...")
        out["train_bitnet2b_6_8"] = train_step(torch, bl, 6, 8)
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(6, 8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
