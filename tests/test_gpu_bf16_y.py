"""GPU parity of the bf16 Y epilogue (bitlinear_fwd_bf16,
bitlinear_contract_bf16) through the C ABI: bf16 outputs bit-identical to
the oracle's bf16 forward (the binary32 epilogue rounded once more to the
nearest bf16, ties to even) at decode and prefill sizes, ragged and split
along k; at the full Qwen2.5-1.5B prefill size, bit-identical to the binary32
call's Y rounded to bf16 and within one bf16 rounding of the oracle's
binary64 Y on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl
from sparse_linear_layers_group_amd import synth
from sparse_linear_layers_group_amd.layer import bf16_tensor

import _gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    H.ensure_built()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _ws(tokens, k, n_out):
    nws = bl.bitlinear_fwd_workspace_bytes(tokens, k, n_out)
    return torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4)])
@pytest.mark.parametrize("tokens,n_out,k", [(1, 200, 1152), (5, 40, 384), (16, 896, 4864),
                                            (100, 200, 1152), (77, 1000, 640), (300, 200, 2432)])
def test_bf16_y_matches_oracle(tokens, n_out, k, n, m):
    W = synth.weights(n_out, k, seed=tokens + n_out)
    X = synth.activations(tokens, k, seed=k + tokens)
    lw, T, g = H.check_weight_path(W, n, m)
    xq_ref, sc_ref = oracle.act_quant(X)
    Yref = oracle.fwd_bf16(xq_ref, sc_ref, T, g)
    xq = torch.empty(tokens * k, dtype=torch.int8, device="cuda")
    sc = torch.empty(tokens, dtype=torch.float32, device="cuda")
    Yb = torch.full((tokens * n_out,), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = _ws(tokens, k, n_out)
    bl.bitlinear_fwd_bf16(bf16_tensor(X), tokens, k, lw.packed, n_out, n, m, lw.gamma, Yb, xq, sc, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy().reshape(xq_ref.shape), xq_ref)
    got = _bits(Yb).reshape(Yref.shape)
    assert np.array_equal(got, Yref), f"{np.count_nonzero(got != Yref)} bf16 outputs differ"
    # the contraction alone, twice on one workspace (split-k counters return to zero)
    Yc = torch.empty_like(Yb)
    ws2 = _ws(tokens, k, n_out)
    for _ in range(2):
        Yc.fill_(float("nan"))
        bl.bitlinear_contract_bf16(xq, sc, tokens, k, lw.packed, n_out, n, m, lw.gamma, Yc, ws=ws2)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(Yc).reshape(Yref.shape), Yref)


def test_bf16_y_full_size_prefill_qwen15():
    """Qwen2.5-1.5B down projection at 2048 tokens (the split-k prefill
    launch): bf16 Y equals the binary32 Y of bitlinear_fwd rounded to bf16,
    everywhere; sampled outputs within one bf16 rounding of the oracle."""
    n_out, k, tokens = 1536, 8960, 2048
    W = synth.weights(n_out, k, seed=0, config=3, layer=2)
    X = synth.activations(tokens, k, seed=0, config=3, layer=2)
    lw, T, g = H.check_weight_path(W, 6, 8)
    Xd = bf16_tensor(X)
    xq = torch.empty(tokens * k, dtype=torch.int8, device="cuda")
    sc = torch.empty(tokens, dtype=torch.float32, device="cuda")
    Y = torch.empty(tokens * n_out, dtype=torch.float32, device="cuda")
    Yb = torch.empty(tokens * n_out, dtype=torch.bfloat16, device="cuda")
    bl.bitlinear_fwd(Xd, tokens, k, lw.packed, n_out, 6, 8, lw.gamma, Y, xq, sc, ws=_ws(tokens, k, n_out))
    bl.bitlinear_fwd_bf16(Xd, tokens, k, lw.packed, n_out, 6, 8, lw.gamma, Yb, xq, sc, ws=_ws(tokens, k, n_out))
    torch.cuda.synchronize()
    # binary32 -> nearest bf16, ties to even (finite values), on the host
    u = Y.cpu().numpy().view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(_bits(Yb), want)
    rng = np.random.default_rng(5)
    ti = rng.integers(0, tokens, 2048)
    ri = rng.integers(0, n_out, 2048)
    xq_h = xq.cpu().numpy().reshape(tokens, k)
    sc_h = sc.cpu().numpy().astype(np.float64)
    _, Y64 = oracle.fwd_pairs(xq_h, sc_h, T, g, ti, ri)
    got = Yb.float().cpu().numpy().reshape(tokens, n_out)[ti, ri].astype(np.float64)
    assert np.all(np.abs(got - Y64) <= 2.0 ** -8 * np.abs(Y64) + 1e-30)
