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


@pytest.mark.parametrize("n_out,k", [(6912, 2560), (2560, 6912), (640, 2560)])
def test_bitnet2b_backward_full_size(n_out, k):
    """BitNet-b1.58-2B4T-shaped layers at 4096 tokens, 6:8: dX and dW at
    sampled elements against the oracle, within the bf16-product bound
    (each compared element within 1e-2 of its sum of absolute products)."""
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
    rng = np.random.default_rng(n_out + k)
    npair = 2048
    t_idx = np.concatenate([rng.integers(0, tokens, npair), [0, tokens - 1]])
    c_idx = np.concatenate([rng.integers(0, k, npair), [0, k - 1]])
    ref = oracle.bwd_dx_pairs(dY, T, g, t_idx, c_idx)
    bound = oracle.bwd_dx_pairs(_abs_bits(dY), np.abs(T), g, t_idx, c_idx)
    err = np.abs(dX[t_idx, c_idx] - ref)
    assert np.all(err <= 1e-2 * bound + 1e-30), f"dX max err/bound {np.max(err / np.maximum(bound, 1e-30))}"
    r_idx = np.concatenate([rng.integers(0, n_out, npair), [0, n_out - 1]])
    c_idx = np.concatenate([rng.integers(0, k, npair), [k - 1, 0]])
    ref = oracle.bwd_dw_pairs(dY, xq, sc, r_idx, c_idx)
    bound = oracle.bwd_dw_pairs(_abs_bits(dY), np.abs(xq), sc, r_idx, c_idx)
    err = np.abs(dW[r_idx, c_idx] - ref)
    assert np.all(err <= 1e-2 * bound + 1e-30), f"dW max err/bound {np.max(err / np.maximum(bound, 1e-30))}"
