"""bitlinear_contract_group: layers that read the same activations in
shared launches.  Each layer's Y (binary32 or bf16) must equal its own
bitlinear_contract / bitlinear_contract_bf16 call bit for bit (the int32
sums are exact in any order), and at small sizes the oracle's Y within the
forward's bar (1e-5 relative, exact zeros where the accumulator is zero;
bf16 Y bit-identical to the oracle's rounding)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl
from sparse_linear_layers_group_amd import synth
from sparse_linear_layers_group_amd.layer import bf16_tensor

import _gpu_helpers as H

pytestmark = pytest.mark.gpu


def _case(shapes, bf16, tokens, k, n, m, seed, with_oracle):
    X = synth.activations(tokens, k, seed=seed)
    xq = torch.empty(tokens * k, dtype=torch.int8, device="cuda")
    sc = torch.empty(tokens, dtype=torch.float32, device="cuda")
    bl.bitlinear_act_quant(bf16_tensor(X), tokens, k, xq, sc)
    layers, entries = [], []
    for i, n_out in enumerate(shapes):
        Wb = synth.weights(n_out, k, seed=seed + 1 + i)
        if with_oracle:
            lw, T, g = H.check_weight_path(Wb, n, m)
        else:
            lw, _, _ = H.quantize_on_gpu(Wb, n, m, want_wq=False)
            T = g = None
        e = dict(packed=lw.packed, gamma=lw.gamma, n_out=n_out)
        if bf16[i]:
            e["Y_bf16"] = torch.full((tokens * n_out,), 0x7fc0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        else:
            e["Y"] = torch.full((tokens * n_out,), float("nan"), dtype=torch.float32, device="cuda")
        layers.append((lw, T, g))
        entries.append(e)
    items = bl.make_contract_items(entries, tokens)
    nws = bl.bitlinear_contract_group_workspace_bytes(items, len(entries), tokens, k)
    ws = torch.zeros(max(nws, 256), dtype=torch.uint8, device="cuda")
    bl.bitlinear_contract_group(items, len(entries), xq, sc, tokens, k, n, m, ws=ws, ws_bytes=nws)
    torch.cuda.synchronize()
    return X, xq, sc, layers, entries


def _own_call(lw, e, xq, sc, tokens, k, n, m):
    nws = bl.bitlinear_fwd_workspace_bytes(tokens, k, lw.n_out)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None
    if "Y_bf16" in e:
        Y = torch.empty(tokens * lw.n_out, dtype=torch.bfloat16, device="cuda")
        bl.bitlinear_contract_bf16(xq, sc, tokens, k, lw.packed, lw.n_out, n, m, lw.gamma, Y, ws=ws)
    else:
        Y = torch.empty(tokens * lw.n_out, dtype=torch.float32, device="cuda")
        bl.bitlinear_contract(xq, sc, tokens, k, lw.packed, lw.n_out, n, m, lw.gamma, Y, ws=ws)
    torch.cuda.synchronize()
    return Y


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 8)])
@pytest.mark.parametrize("tokens", [5, 300])
def test_contract_group_matches_oracle_and_own_calls(n, m, tokens):
    """Ragged layers (a partial strip, a partial 256-row block), binary32 and
    bf16 outputs mixed, at decode (5) and prefill (300) token counts."""
    k = 384
    shapes, bf16 = [136, 320, 64], [False, True, False]
    X, xq, sc, layers, entries = _case(shapes, bf16, tokens, k, n, m, seed=tokens + n, with_oracle=True)
    xq_ref, sc_ref = oracle.act_quant(X)
    for (lw, T, g), e in zip(layers, entries):
        got = e.get("Y", e.get("Y_bf16"))
        if "Y_bf16" in e:
            want = oracle.fwd_bf16(xq_ref, sc_ref, T, g)
            assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16).reshape(want.shape), want)
        else:
            acc_ref, Y_ref = oracle.fwd(xq_ref, sc_ref, T, g)
            H.assert_y_close(got.cpu().numpy().reshape(Y_ref.shape).astype(np.float64), Y_ref, acc_ref)
        assert np.array_equal(_bits(got), _bits(_own_call(lw, e, xq, sc, tokens, k, n, m)))


@pytest.mark.parametrize("shapes", [
    [2560, 640, 640],   # BitNet-2B4T q, k, v
    [6912, 6912],       # BitNet-2B4T gate, up
])
def test_contract_group_bitnet_shapes_match_own_calls(shapes):
    """The groupings the training step uses, at 4096 tokens: bit-identical
    to each layer's own call (which splits k for some shapes)."""
    tokens, k = 4096, 2560
    X, xq, sc, layers, entries = _case(shapes, [False] * len(shapes), tokens, k, 6, 8, seed=11,
                                       with_oracle=False)
    for (lw, _, _), e in zip(layers, entries):
        assert np.array_equal(_bits(e["Y"]), _bits(_own_call(lw, e, xq, sc, tokens, k, 6, 8)))


def test_contract_group_more_layers_than_one_launch():
    """Nine layers take two launches (at most eight layers per launch)."""
    tokens, k = 100, 256
    shapes = [64 * (i + 1) for i in range(9)]
    X, xq, sc, layers, entries = _case(shapes, [i % 2 == 1 for i in range(9)], tokens, k, 6, 8, seed=3,
                                       with_oracle=False)
    for (lw, _, _), e in zip(layers, entries):
        got = e.get("Y", e.get("Y_bf16"))
        assert np.array_equal(_bits(got), _bits(_own_call(lw, e, xq, sc, tokens, k, 6, 8)))


def test_contract_group_reruns_bit_identical():
    """Two calls on the same inputs give the same bits (no order-dependent
    sums anywhere in the grouped launches)."""
    tokens, k = 520, 512
    shapes = [1040, 320, 64]
    X, xq, sc, layers, entries = _case(shapes, [False, True, False], tokens, k, 6, 8, seed=17, with_oracle=False)
    first = [_bits(e.get("Y", e.get("Y_bf16"))).copy() for e in entries]
    items = bl.make_contract_items(entries, tokens)
    bl.bitlinear_contract_group(items, len(entries), xq, sc, tokens, k, 6, 8)
    torch.cuda.synchronize()
    for f, e in zip(first, entries):
        assert np.array_equal(f, _bits(e.get("Y", e.get("Y_bf16"))))
