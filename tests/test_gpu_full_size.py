"""GPU parity at the full sizes of the measured workloads, through the C ABI.

Weight paths (mask, gamma, codes, packed bytes) are compared in full; the
large contractions are compared at sampled (token, row) pairs that the
oracle computes one by one, plus the four output corners.  The launch
configurations are the ones bench.py times (grouped decode plan, prefill
kernel, split-k where it applies, backward through its workspace)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl
from sparse_linear_layers_group_amd import synth
from sparse_linear_layers_group_amd.layer import BitLinearWeight, bf16_tensor

import _gpu_helpers as H

pytestmark = pytest.mark.gpu

QWEN05 = [(896, 896), (128, 896), (128, 896), (896, 896), (4864, 896), (4864, 896), (896, 4864)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    H.ensure_built()


def test_qwen05_decode_layer_grouped():
    """Qwen2.5-0.5B-shaped decode, 1 token: the seven projections of two
    layers in one grouped plan, every output against the oracle."""
    weights = []
    for li, (n_out, k) in enumerate(QWEN05):
        W = synth.weights(n_out, k, seed=0, config=2, layer=li)
        weights.append(H.check_weight_path(W, 6, 8))
    entries, refs = [], []
    for L in range(2):
        for li, (n_out, k) in enumerate(QWEN05):
            lw, T, g = weights[li]
            X = synth.activations(1, k, seed=1 + L, config=2, layer=li)
            xq, sc = oracle.act_quant(X)
            _, Yref = oracle.fwd(xq, sc, T, g)
            entries.append(dict(X=bf16_tensor(X), packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                                Y=torch.full((n_out,), float("nan"), device="cuda"),
                                xq=torch.empty(k, dtype=torch.int8, device="cuda"),
                                x_scale=torch.empty(1, dtype=torch.float32, device="cuda")))
            refs.append((xq, sc, Yref))
    items = bl.make_fwd_items(entries, 1)
    plan = torch.empty(bl.bitlinear_fwd_group_plan_bytes(items, len(entries), 1), dtype=torch.uint8,
                       device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), 1, 6, 8, plan)
    bl.bitlinear_fwd_group(plan, 6, 8, 3)
    torch.cuda.synchronize()
    for e, (xq, sc, Yref) in zip(entries, refs):
        assert np.array_equal(e["xq"].cpu().numpy(), xq[0])
        assert np.array_equal(e["x_scale"].cpu().numpy(), sc.astype(np.float32))
        H.assert_y_close(e["Y"].cpu().numpy().astype(np.float64), Yref[0])


@pytest.mark.parametrize("n_out,k", [(8960, 1536), (1536, 8960)])
def test_qwen15_prefill_full_size(n_out, k):
    """Qwen2.5-1.5B-shaped prefill at 2048 tokens, 6:8: gate/up and down."""
    W = synth.weights(n_out, k, seed=0, config=3, layer=0 if n_out > k else 2)
    X = synth.activations(2048, k, seed=0, config=3, layer=0 if n_out > k else 2)
    lw, T, g = H.check_weight_path(W, 6, 8)
    H.check_forward_sampled(lw, T, g, X, seed=n_out)


@pytest.mark.parametrize("n,m", [(8, 8), (6, 8), (4, 8), (2, 4), (2, 8)])
@pytest.mark.parametrize("n_out,k", [(11008, 2048), (2048, 11008)])
def test_qwen3b_sweep_full_size(n_out, k, n, m):
    """Qwen2.5-3B-shaped sweep: both shapes, every pattern, token counts
    1, 16 (decode kernel), 512 and 4096 (prefill kernel)."""
    W = synth.weights(n_out, k, seed=0, config=4, layer=0 if n_out > k else 1)
    lw, T, g = H.check_weight_path(W, n, m)
    for tokens in (1, 16, 512, 4096):
        X = synth.activations(tokens, k, seed=tokens, config=4, layer=0 if n_out > k else 1)
        H.check_forward_sampled(lw, T, g, X, pairs=2048, seed=tokens + n)


def _abs_bits(bits):
    return (bits & np.uint16(0x7FFF)).astype(np.uint16)


BITNET2B = [  # (name, n_out, k, input layer) -- q/k/v and gate/up share the block input
    ("q", 2560, 2560, 0), ("k", 640, 2560, 0), ("v", 640, 2560, 0), ("o", 2560, 2560, 3),
    ("gate", 6912, 2560, 0), ("up", 6912, 2560, 0), ("down", 2560, 6912, 6),
]


@pytest.mark.parametrize("li", range(len(BITNET2B)), ids=[b[0] for b in BITNET2B])
def test_bitnet2b_forward_full_size(li):
    """BitNet-b1.58-2B4T-shaped block, 4096 tokens, 6:8: each of the seven
    layers' weight path in full (bit-exact) and its forward at sampled
    (token, row) pairs and the corners (acc bit-exact, Y within 1e-5)."""
    name, n_out, k, src = BITNET2B[li]
    W = synth.weights(n_out, k, seed=0, config=5, layer=li)
    X = synth.activations(4096, k, seed=0, config=5, layer=src)
    lw, T, g = H.check_weight_path(W, 6, 8)
    H.check_forward_sampled(lw, T, g, X, pairs=4096, seed=li)


def _tile_pairs(rng, M, N, tile=128, extra=2048):
    """One random element in every tile x tile block of an M x N output,
    `extra` uniform draws and the four corners."""
    I, J = np.meshgrid(np.arange(0, M, tile), np.arange(0, N, tile), indexing="ij")
    I, J = I.ravel(), J.ravel()
    r = I + rng.integers(0, np.minimum(tile, M - I))
    c = J + rng.integers(0, np.minimum(tile, N - J))
    r = np.concatenate([r, rng.integers(0, M, extra), [0, 0, M - 1, M - 1]])
    c = np.concatenate([c, rng.integers(0, N, extra), [0, N - 1, 0, N - 1]])
    return r, c


def _lines(rng, M, N, nrows=3, ncols=3):
    """Every element of a few whole rows (the first, the last, random ones)
    and of a few whole columns of an M x N output."""
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, nrows - 2)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, ncols - 2)]))
    r = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), cols.size)])
    c = np.concatenate([np.tile(np.arange(N), rows.size), np.repeat(cols, M)])
    return r, c


def _rss(A, B, i_idx, j_idx, chunk=512):
    """sqrt(sum_k (A[i, k] B[k, j])^2) for each pair (i, j): the size of a
    random-sign sum's rounding error, used to tell which reference values
    are large enough for an elementwise relative check."""
    out = np.empty(i_idx.size)
    for s in range(0, i_idx.size, chunk):
        a = A[i_idx[s:s + chunk]]
        b = B[:, j_idx[s:s + chunk]].T
        out[s:s + chunk] = np.sqrt(np.sum((a * b) ** 2, axis=1))
    return out


def _check_grad(got, ref, absprod, rss, elem_bound, frob_rel, rel_where):
    """Elementwise error within the worst-case rounding bound; Frobenius
    error of the sampled set within frob_rel of its reference norm; and
    relative error within frob_rel wherever |ref| >= rel_where * rss."""
    err = np.abs(got - ref)
    worst = np.max(err / np.maximum(elem_bound * absprod + 2.0 ** -23 * np.abs(ref), 1e-300))
    assert worst <= 1.0, f"elementwise error / bound {worst}"
    fr = np.linalg.norm(err) / np.linalg.norm(ref)
    assert fr <= frob_rel, f"Frobenius relative error {fr}"
    big = np.abs(ref) >= rel_where * rss
    assert big.sum() >= 64
    rel = np.max(err[big] / np.abs(ref[big]))
    assert rel <= frob_rel, f"relative error where |ref| is large {rel}"
    return fr, rel


@pytest.mark.parametrize("n_out,k", [(6912, 2560), (2560, 6912), (640, 2560), (2560, 2560)])
def test_bitnet2b_backward_full_size(n_out, k):
    """BitNet-b1.58-2B4T-shaped layers at 4096 tokens, 6:8: dX and dW
    against the oracle at one element of every 128 x 128 output tile, 2048
    more random elements, the corners, and whole rows and columns.

    dX = gamma dY codes: both factors are exact in bf16, so the only error
    is binary32 accumulation, bounded by n_out 2^-24 times the sum of
    absolute products; sampled-set Frobenius and large-element relative
    error within 1e-4.  dW = (dY s)^T x_q: dY s is rounded to bf16 (relative
    2^-8 per term) and accumulated in binary32, so the bound is (2^-8 +
    tokens 2^-24) times the sum of absolute products; Frobenius and
    large-element relative error within 1e-2, the bar for the bf16
    backward products (each split-k range of the k/v dW contributes to
    every element, so a lost range fails the Frobenius check)."""
    tokens = 4096
    W = synth.weights(n_out, k, seed=0, config=5, layer=0)
    X = synth.activations(tokens, k, seed=0, config=5, layer=0)
    dY = synth.grad_output(tokens, n_out, seed=0, config=5, layer=0)
    lw, T, g = H.check_weight_path(W, 6, 8)
    bufs = lw.fwd(bf16_tensor(X), tokens)
    torch.cuda.synchronize()
    xq, sc = oracle.act_quant(X)
    assert np.array_equal(bufs["xq"].cpu().numpy().reshape(tokens, k), xq)
    assert np.array_equal(bufs["x_scale"].cpu().numpy(), sc.astype(np.float32))
    dX, dW = lw.bwd(bf16_tensor(dY), bufs["xq"], bufs["x_scale"], tokens)
    torch.cuda.synchronize()
    dX = dX.cpu().numpy().reshape(tokens, k).astype(np.float64)
    dW = dW.cpu().numpy().reshape(n_out, k).astype(np.float64)
    dYf = synth.bf16_bits_to_f32(dY).astype(np.float64)
    rng = np.random.default_rng(n_out + k)

    t1, c1 = _tile_pairs(rng, tokens, k)
    t2, c2 = _lines(rng, tokens, k)
    t_idx, c_idx = np.concatenate([t1, t2]), np.concatenate([c1, c2])
    ref = oracle.bwd_dx_pairs(dY, T, g, t_idx, c_idx)
    absprod = oracle.bwd_dx_pairs(_abs_bits(dY), np.abs(T), g, t_idx, c_idx)
    rss = g * _rss(dYf, T.astype(np.float64), t_idx, c_idx)
    _check_grad(dX[t_idx, c_idx], ref, absprod, rss, n_out * 2.0 ** -24, 1e-4, 1.0)

    r1, c1 = _tile_pairs(rng, n_out, k)
    r2, c2 = _lines(rng, n_out, k)
    r_idx, c_idx = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    ref = oracle.bwd_dw_pairs(dY, xq, sc, r_idx, c_idx)
    absprod = oracle.bwd_dw_pairs(_abs_bits(dY), np.abs(xq), sc, r_idx, c_idx)
    rss = _rss((dYf * sc[:, None]).T, xq.astype(np.float64), r_idx, c_idx)
    _check_grad(dW[r_idx, c_idx], ref, absprod, rss, 2.0 ** -8 + tokens * 2.0 ** -24, 1e-2, 2.0)
