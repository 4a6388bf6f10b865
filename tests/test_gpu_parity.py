"""GPU parity: the HIP path through the C ABI against the oracle, on seeded
inputs.  Masks, gamma, ternary codes, packed bytes, int8 activations, scales
and int32 accumulators must match bit for bit; Y within 1e-5 relative;
dX / dW within the bf16-product tolerance (see _gpu_helpers)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl
from sparse_linear_layers_group_amd import synth
from sparse_linear_layers_group_amd.layer import (BitLinearWeight, LatentWeights, QuantGroup, bf16_bits,
                                                   bf16_tensor, dense_to_sparse)

import _gpu_helpers as H

pytestmark = pytest.mark.gpu

PATTERNS = [(8, 8), (6, 8), (4, 8), (2, 4), (3, 8), (2, 8)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    H.ensure_built()


def test_tiny_config_forward_6_8():
    """W bf16 [128 x 256] ~ N(0, 0.02), X bf16 [8 x 256] ~ N(0, 1), 6:8, seed 0."""
    W = synth.weights(128, 256, seed=0, config=1)
    X = synth.activations(8, 256, seed=0, config=1)
    lw, T, g = H.check_weight_path(W, 6, 8)
    H.check_forward(lw, T, g, X)


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("n_out,k", [(48, 256), (40, 384), (200, 896), (16, 128)])
def test_weight_path(n, m, n_out, k):
    H.check_weight_path(synth.weights(n_out, k, seed=n_out + k + n), n, m)


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("n_out,k,tokens", [
    (48, 256, 1), (40, 384, 5), (160, 896, 16),   # decode kernel, ragged tiles
    (64, 640, 17), (200, 384, 130), (136, 1152, 260),  # prefill kernel, ragged tiles
])
def test_forward_parity(n, m, n_out, k, tokens):
    seed = 7 * n_out + k + tokens + n
    W = synth.weights(n_out, k, seed=seed)
    X = synth.activations(tokens, k, seed=seed)
    lw, T, g = H.check_weight_path(W, n, m)
    H.check_forward(lw, T, g, X)


@pytest.mark.parametrize("n_out,k", [(32, 128), (2048, 11008), (11008, 256), (896, 4864)])
def test_decode_split_k_and_tall_shapes(n_out, k):
    """Few row tiles with long k split the k range across wavefronts; the
    partial sums meet by integer atomics, so results stay exact."""
    W = synth.weights(n_out, k, seed=k)
    lw, T, g = H.check_weight_path(W, 6, 8)
    for tokens in (1, 3, 16):
        H.check_forward(lw, T, g, synth.activations(tokens, k, seed=tokens))


def test_decode_and_prefill_kernels_agree():
    """tokens <= 16 runs the decode kernel, more tokens the prefill kernel:
    the rows they share are identical."""
    W = synth.weights(96, 512, seed=3)
    X = synth.activations(40, 512, seed=3)
    lw, T, g = H.check_weight_path(W, 6, 8)
    big = lw.fwd(bf16_tensor(X), 40)
    small = lw.fwd(bf16_tensor(X[:16]), 16)
    torch.cuda.synchronize()
    a = big["Y"].cpu().numpy().reshape(40, 96)[:16]
    b = small["Y"].cpu().numpy().reshape(16, 96)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("n_out,k,tokens", [(48, 256, 7), (64, 384, 130), (128, 256, 64)])
def test_backward_parity(n, m, n_out, k, tokens):
    seed = 3 * n_out + k + tokens + m
    W = synth.weights(n_out, k, seed=seed)
    X = synth.activations(tokens, k, seed=seed)
    dY = synth.grad_output(tokens, n_out, seed=seed)
    lw, T, g = H.check_weight_path(W, n, m)
    bufs, xq, sc = H.check_forward(lw, T, g, X)
    dX, dW = lw.bwd(bf16_tensor(dY), bufs["xq"], bufs["x_scale"], tokens)
    torch.cuda.synchronize()
    dyv = np.abs(synth.bf16_bits_to_f32(dY).astype(np.float64))
    ref_dx = oracle.bwd_dx(dY, T, g)
    H.assert_grad_close(dX.cpu().numpy().reshape(ref_dx.shape).astype(np.float64), ref_dx,
                        g * (dyv @ np.abs(T).astype(np.float64)))
    ref_dw = oracle.bwd_dw(dY, xq, sc)
    H.assert_grad_close(dW.cpu().numpy().reshape(ref_dw.shape).astype(np.float64), ref_dw,
                        dyv.T @ (np.abs(xq) * sc[:, None]))


@pytest.mark.parametrize("n_out,k,tokens", [(2048, 256, 64), (128, 256, 4096), (640, 384, 2100)])
def test_backward_split_along_k(n_out, k, tokens):
    """Products with few output tiles and a deep contraction are cut along k
    into binary32 partial tiles (dX of a 64-token batch over 2048 rows, dW
    of a 4096-token batch, a ragged last range): same tolerance against the
    oracle, and bit-identical on a rerun (the partials are summed in a
    fixed order)."""
    test_backward_parity(6, 8, n_out, k, tokens)
    W = synth.weights(n_out, k, seed=9)
    lw, _, _ = H.quantize_on_gpu(W, 6, 8, want_wq=False)
    X = synth.activations(tokens, k, seed=9)
    dY = bf16_tensor(synth.grad_output(tokens, n_out, seed=9))
    bufs = lw.fwd(bf16_tensor(X), tokens)
    ws = lw.bwd_workspace(tokens)
    a = lw.bwd(dY, bufs["xq"], bufs["x_scale"], tokens, ws=ws)
    b = lw.bwd(dY, bufs["xq"], bufs["x_scale"], tokens, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_gamma_exact_for_out_of_window_magnitudes():
    """Magnitudes >= 2 and bf16 subnormals take the rare accumulation path;
    gamma must still be the exact sum rounded once."""
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 0x7F80, size=(64, 256), dtype=np.uint16)  # every finite magnitude
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)
    bits[:8] = rng.integers(1, 0x80, size=(8, 256), dtype=np.uint16)  # subnormals
    for n, m in PATTERNS:
        H.check_weight_path(bits, n, m)
    H.check_weight_path(bits, 6, 8, gamma_over=bl.BL_GAMMA_MASKED)


def test_gamma_exact_over_many_workgroups():
    """Enough 8-groups for the largest mask grid (1024 workgroups, two
    passes each, a short last range), with magnitudes of every exponent
    and signed zeros scattered so that many wavefronts mix groups on the
    window path with groups on the exact per-element path."""
    W = synth.weights(2304, 4096, seed=23)
    rng = np.random.default_rng(23)
    pos = rng.choice(W.size, size=3000, replace=False)
    flat = W.reshape(-1)
    flat[pos] = rng.integers(1, 0x7F80, size=pos.size, dtype=np.uint16)
    flat[pos[::2]] |= 0x8000
    zeros = rng.choice(W.size, size=2000, replace=False)  # +0 and -0 among in-window groups
    flat[zeros] = np.where(np.arange(zeros.size) % 2 == 0, 0, 0x8000).astype(np.uint16)
    assert bl.bitlinear_workspace_bytes(2304, 4096) == 1024 * (32 + 2048)
    H.check_weight_path(W, 6, 8)


def test_masked_gamma_ablation():
    W = synth.weights(96, 512, seed=17)
    lw, T, g = H.check_weight_path(W, 6, 8, gamma_over=bl.BL_GAMMA_MASKED)
    H.check_forward(lw, T, g, synth.activations(9, 512, seed=17))


def test_degenerate_inputs():
    # all-zero weights: gamma 0, no codes, zero output
    W = np.zeros((32, 256), np.uint16)
    lw, T, g = H.check_weight_path(W, 6, 8)
    assert g == 0.0 and not T.any()
    X = synth.activations(4, 256, seed=1)
    bufs, _, _ = H.check_forward(lw, T, g, X)
    assert not bufs["Y"].cpu().numpy().any()
    # zero token rows and signed zeros
    W = synth.weights(64, 256, seed=2)
    X = synth.activations(20, 256, seed=2)
    X[3] = 0
    X[5] = 0x8000
    lw, T, g = H.check_weight_path(W, 6, 8)
    bufs, xq, sc = H.check_forward(lw, T, g, X)
    assert sc[3] == 0 and sc[5] == 0
    lw.fwd(bf16_tensor(X[:0]), 0)  # zero tokens: a no-op


def test_zero_tokens_backward_gives_zero_dw():
    W = synth.weights(64, 256, seed=9)
    lw, T, g = H.check_weight_path(W, 6, 8)
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")[:0]
    dW = torch.full((64 * 256,), 7.0, dtype=torch.float32, device="cuda")
    bl.bitlinear_bwd(dummy, None, None, lw.packed, lw.gamma, 0, 256, 64, 6, 8, None, dW)
    torch.cuda.synchronize()
    assert not dW.cpu().numpy().any()


def test_repeat_runs_are_bit_identical():
    W = synth.weights(256, 1024, seed=5)
    X = synth.activations(33, 1024, seed=5)
    dY = synth.grad_output(33, 256, seed=5)
    outs = []
    for _ in range(2):
        lw = BitLinearWeight(256, 1024, 6, 8)
        lw.quantize(bf16_tensor(W))
        b = lw.fwd(bf16_tensor(X), 33)
        dX, dW = lw.bwd(bf16_tensor(dY), b["xq"], b["x_scale"], 33)
        b1 = lw.fwd(bf16_tensor(X[:1]), 1)
        torch.cuda.synchronize()
        outs.append([lw.gamma.cpu().numpy(), lw.packed.cpu().numpy(), b["Y"].cpu().numpy(),
                     dX.cpu().numpy(), dW.cpu().numpy(), b1["Y"].cpu().numpy()])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_host_errors_with_device_buffers():
    lw = BitLinearWeight(64, 256, 6, 8)
    W = bf16_tensor(synth.weights(64, 256))
    with pytest.raises(bl.BitLinearError) as e:
        bl.bitlinear_quantize_mask(W, 64, 256, 6, 8, 0, lw.mask, None, lw.gamma, lw.ws, ws_bytes=16)
    assert e.value.status == bl.BL_EWORKSPACE
    with pytest.raises(bl.BitLinearError) as e:
        bl.bitlinear_pack(W, lw.mask, lw.gamma, 64, 256, 6, 8, lw.packed, packed_bytes=100)
    assert e.value.status == bl.BL_ESHAPE


@pytest.mark.parametrize("tokens", [1, 5, 16])
@pytest.mark.parametrize("n,m", [(6, 8), (8, 8), (2, 4), (2, 8)])
def test_grouped_decode_matches_oracle(tokens, n, m):
    """One plan, several GEMVs of different shapes (including a ragged row
    tile and a partial 512-wide k super-tile), two launches."""
    shapes = [(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)]
    entries, refs = [], []
    for i, (n_out, k) in enumerate(shapes):
        W = synth.weights(n_out, k, seed=100 + i)
        X = synth.activations(tokens, k, seed=200 + i)
        lw, T, g = H.check_weight_path(W, n, m)
        xq, sc = oracle.act_quant(X)
        _, Yref = oracle.fwd(xq, sc, T, g)
        e = dict(X=bf16_tensor(X), packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                 Y=torch.full((tokens * n_out,), float("nan"), dtype=torch.float32, device="cuda"),
                 xq=torch.empty(tokens * k, dtype=torch.int8, device="cuda"),
                 x_scale=torch.empty(tokens, dtype=torch.float32, device="cuda"), lw=lw)
        entries.append(e)
        refs.append((xq, sc, Yref))
    items = bl.make_fwd_items(entries, tokens)
    nbytes = bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens)
    plan = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
    for stages in ((3,), (1, 2)):
        for e in entries:
            e["Y"].fill_(float("nan"))
        for s in stages:
            bl.bitlinear_fwd_group(plan, n, m, s)
        torch.cuda.synchronize()
        for e, (xq, sc, Yref) in zip(entries, refs):
            assert np.array_equal(e["xq"].cpu().numpy().reshape(xq.shape), xq)
            assert np.array_equal(e["x_scale"].cpu().numpy(), sc.astype(np.float32))
            H.assert_y_close(e["Y"].cpu().numpy().reshape(Yref.shape).astype(np.float64), Yref)


@pytest.mark.parametrize("tokens,shapes", [
    # one strip per workgroup, ranges cut inside a 38-block strip, idle
    # wavefronts (k = 128, 256)
    (1, [(896, 4864), (64, 128), (128, 256), (200, 1152), (72, 640)]),
    (16, [(896, 4864), (64, 128), (128, 256), (200, 1152), (72, 640)]),
    # many strips per workgroup: the 0.5B feed-forward shapes
    (1, [(4864, 896), (896, 4864), (4864, 896), (896, 896)]),
    # ~31 one-block strips per workgroup at 16 tokens
    (16, [(64000, 128)] * 8),
])
def test_grouped_decode_matches_single_calls(tokens, shapes):
    """Grouped decode: every Y bit-identical to a single bitlinear_contract
    call on the same int8 activations, and to the oracle within the decode
    tolerance on a sample of rows."""
    n, m = 6, 8
    entries, singles = [], []
    for i, (n_out, k) in enumerate(shapes):
        W = synth.weights(n_out, k, seed=500 + i)
        X = synth.activations(tokens, k, seed=600 + i)
        lw = BitLinearWeight(n_out, k, n, m)
        lw.quantize(bf16_tensor(W))
        e = dict(X=bf16_tensor(X), packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                 Y=torch.full((tokens * n_out,), float("nan"), dtype=torch.float32, device="cuda"),
                 xq=torch.empty(tokens * k, dtype=torch.int8, device="cuda"),
                 x_scale=torch.empty(tokens, dtype=torch.float32, device="cuda"), lw=lw, W=W, Xb=X)
        entries.append(e)
    items = bl.make_fwd_items(entries, tokens)
    plan = torch.empty(bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens), dtype=torch.uint8,
                       device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
    for rep in range(2):  # the plan is reused
        for e in entries:
            e["Y"].fill_(float("nan"))
        bl.bitlinear_fwd_group(plan, n, m, 3)
        torch.cuda.synchronize()
        for i, e in enumerate(entries):
            Ys = torch.empty_like(e["Y"])
            nws = bl.bitlinear_fwd_workspace_bytes(tokens, e["k"], e["n_out"])
            ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None
            bl.bitlinear_contract(e["xq"], e["x_scale"], tokens, e["k"], e["lw"].packed, e["n_out"], n, m,
                                  e["lw"].gamma, Ys, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(e["Y"].cpu().numpy().view(np.uint32), Ys.cpu().numpy().view(np.uint32)), i
    # the oracle on a sample of rows of the first item (gamma over all rows)
    e = entries[0]
    rows = np.arange(0, e["n_out"], max(1, e["n_out"] // 97))
    xq, sc = oracle.act_quant(e["Xb"])
    assert np.array_equal(e["xq"].cpu().numpy().reshape(xq.shape), xq)
    g = oracle.gamma(e["W"])
    Wr = np.ascontiguousarray(e["W"][rows])
    T = oracle.ternary(Wr, oracle.mask(Wr, n, m), g)
    acc_ref, Yref = oracle.fwd(xq, sc, T, g)
    Y = e["Y"].cpu().numpy().reshape(tokens, e["n_out"])[:, rows]
    H.assert_y_close(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("n_out,k,tokens", [(200, 2432, 300), (512, 1024, 17), (1536, 8960, 1024)])
def test_prefill_split_k(n_out, k, tokens):
    """Layers with few output tiles split their k blocks over two
    workgroups (uneven parts: 19 blocks as 9 + 10; 35 + 35 for the
    Qwen2.5-1.5B down projection at 1024 tokens); the int32 sums must still
    be exact and repeat calls must reuse the workspace."""
    nws = bl.bitlinear_fwd_workspace_bytes(tokens, k, n_out)
    assert nws > 0, "shape should take the split-k path"
    W = synth.weights(n_out, k, seed=41)
    X = synth.activations(tokens, k, seed=41)
    lw, T, g = H.check_weight_path(W, 6, 8)
    if tokens * n_out <= 600_000:
        bufs, _, _ = H.check_forward(lw, T, g, X)
    else:
        bufs = H.check_forward_sampled(lw, T, g, X, seed=41)
    Y0 = bufs["Y"].cpu().numpy().copy()
    lw.fwd(bf16_tensor(X), tokens, bufs=bufs)
    torch.cuda.synchronize()
    assert np.array_equal(bufs["Y"].cpu().numpy(), Y0)


@pytest.mark.parametrize("tokens", [1, 16, 100])
def test_act_quant_plus_contract_equals_fwd(tokens):
    W = synth.weights(2048, 1024, seed=31)
    X = synth.activations(tokens, 1024, seed=31)
    lw, T, g = H.check_weight_path(W, 6, 8)
    ref = lw.fwd(bf16_tensor(X), tokens)
    xq = torch.empty(tokens * 1024, dtype=torch.int8, device="cuda")
    sc = torch.empty(tokens, dtype=torch.float32, device="cuda")
    Y = torch.empty(tokens * 2048, dtype=torch.float32, device="cuda")
    nws = bl.bitlinear_fwd_workspace_bytes(tokens, 1024, 2048)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None
    bl.bitlinear_act_quant(bf16_tensor(X), tokens, 1024, xq, sc)
    for _ in range(3):  # every call returns the split-k counters to zero
        bl.bitlinear_contract(xq, sc, tokens, 1024, lw.packed, 2048, 6, 8, lw.gamma, Y, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy(), ref["Y"].cpu().numpy())
    if ws is not None:
        # decode: the whole workspace; prefill: the ticket block in front of
        # the partial tiles (one counter per 256 x 64 tile and wavefront)
        tiles = -(-2048 // 256) * -(-tokens // 64)
        n_zero = nws if tokens <= 16 else -(-tiles * 16 // 256) * 256
        assert not ws[:n_zero].cpu().numpy().any()
    assert np.array_equal(xq.cpu().numpy(), ref["xq"].cpu().numpy())


@pytest.mark.parametrize("plan_nm,run_nm", [((6, 8), (8, 8)), ((2, 8), (6, 8)), ((8, 8), (2, 4))])
def test_grouped_decode_rejects_other_pattern(plan_nm, run_nm):
    """A grouped contraction run with an N:M pattern whose sign-slot count
    differs from the plan's reads no packed byte and sets every output of
    every item to NaN; the plan then still runs correctly with its own
    pattern."""
    tokens = 2
    shapes = [(200, 1152), (48, 256), (896, 4864)]
    n, m = plan_nm
    entries, refs = [], []
    for i, (n_out, k) in enumerate(shapes):
        W = synth.weights(n_out, k, seed=300 + i)
        X = synth.activations(tokens, k, seed=400 + i)
        lw, T, g = H.check_weight_path(W, n, m)
        xq, sc = oracle.act_quant(X)
        _, Yref = oracle.fwd(xq, sc, T, g)
        entries.append(dict(X=bf16_tensor(X), packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                            Y=torch.zeros(tokens * n_out, dtype=torch.float32, device="cuda"),
                            xq=torch.empty(tokens * k, dtype=torch.int8, device="cuda"),
                            x_scale=torch.empty(tokens, dtype=torch.float32, device="cuda"), lw=lw))
        refs.append(Yref)
    items = bl.make_fwd_items(entries, tokens)
    plan = torch.empty(bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens), dtype=torch.uint8,
                       device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
    bl.bitlinear_fwd_group(plan, run_nm[0], run_nm[1], 3)
    torch.cuda.synchronize()
    for e in entries:
        assert torch.isnan(e["Y"]).all()
    bl.bitlinear_fwd_group(plan, n, m, 3)
    torch.cuda.synchronize()
    for e, Yref in zip(entries, refs):
        H.assert_y_close(e["Y"].cpu().numpy().reshape(Yref.shape).astype(np.float64), Yref)


def test_group_plan_validation():
    lw = BitLinearWeight(64, 256, 6, 8)
    e = dict(X=torch.zeros(256, dtype=torch.bfloat16, device="cuda"), packed=lw.packed, gamma=lw.gamma,
             Y=torch.zeros(64, dtype=torch.float32, device="cuda"),
             xq=torch.zeros(256, dtype=torch.int8, device="cuda"),
             x_scale=torch.zeros(1, dtype=torch.float32, device="cuda"), k=256, n_out=64)
    items = bl.make_fwd_items([e], 1)
    plan = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bl.BitLinearError) as err:
        bl.bitlinear_fwd_group_plan(items, 1, 1, 6, 8, plan)
    assert err.value.status == bl.BL_EWORKSPACE
    assert bl.bitlinear_fwd_group_plan_bytes(items, 1, 17) == 0  # decode only: <= 16 tokens


@pytest.mark.parametrize("n,m,gamma_over", [(6, 8, 0), (8, 8, 0), (2, 4, 0), (4, 8, 1), (3, 8, 0), (2, 8, 1)])
def test_grouped_quantisation_matches_oracle(n, m, gamma_over):
    """Grouped mask + gamma + pack of ragged layers in one plan: every mask,
    gamma and packed byte bit-identical to the oracle, run twice (the plan
    is reused and the shared workspace needs no clearing between runs)."""
    shapes = [(48, 256), (200, 896), (16, 128), (896, 896), (128, 2432), (40, 384)]
    pairs, refs = [], []
    for i, (n_out, k) in enumerate(shapes):
        Wbits = synth.weights(n_out, k, seed=40 + i)
        mb = oracle.mask(Wbits, n, m)
        g = oracle.gamma(Wbits, gamma_over == bl.BL_GAMMA_MASKED, mb)
        P = oracle.pack(oracle.ternary(Wbits, mb, g), H.S_OF[(n, m)])
        pairs.append((BitLinearWeight(n_out, k, n, m, gamma_over), bf16_tensor(Wbits)))
        refs.append((mb, g, P))
    qg = QuantGroup(pairs)
    for rep in range(2):
        for lw, _ in pairs:
            lw.mask.fill_(0xA5)
            lw.packed.fill_(0x5A)
            lw.gamma.fill_(float("nan"))
        qg.run()
        torch.cuda.synchronize()
        for (lw, _), (mb, g, P) in zip(pairs, refs):
            assert np.array_equal(lw.mask.cpu().numpy().reshape(mb.shape), mb), (rep, lw.n_out, lw.k)
            assert H.f64_bits(lw.gamma.cpu().numpy()[0]) == H.f64_bits(g), (rep, lw.n_out, lw.k)
            assert np.array_equal(lw.packed.cpu().numpy(), P), (rep, lw.n_out, lw.k)


def test_grouped_quantisation_full_size_matches_single_calls():
    """A Qwen2.5-1.5B-shaped block (q, k, v, o, gate, up, down) in one plan:
    bit-identical to the single-layer calls, which the weight-path tests
    pin to the oracle; gamma also against the oracle, with magnitudes of
    every exponent planted so workgroups take the rare accumulation path."""
    shapes = [(1536, 1536), (256, 1536), (256, 1536), (1536, 1536), (8960, 1536), (8960, 1536),
              (1536, 8960)]
    rng = np.random.default_rng(77)
    pairs, singles, gref = [], [], []
    for i, (n_out, k) in enumerate(shapes):
        Wbits = synth.weights(n_out, k, seed=0, config=3, layer=i)
        flat = Wbits.reshape(-1)
        pos = rng.choice(flat.size, size=500, replace=False)
        flat[pos] = rng.integers(1, 0x7F80, size=pos.size, dtype=np.uint16)
        W = bf16_tensor(Wbits)
        single = BitLinearWeight(n_out, k, 6, 8)
        single.quantize(W)
        pairs.append((BitLinearWeight(n_out, k, 6, 8), W))
        singles.append(single)
        gref.append(oracle.gamma(Wbits, False, None))
    qg = QuantGroup(pairs)
    qg.run()
    torch.cuda.synchronize()
    for (lw, _), s, g in zip(pairs, singles, gref):
        assert torch.equal(lw.mask, s.mask), (lw.n_out, lw.k)
        assert torch.equal(lw.packed, s.packed), (lw.n_out, lw.k)
        assert H.f64_bits(lw.gamma.cpu().numpy()[0]) == H.f64_bits(s.gamma.cpu().numpy()[0]) == H.f64_bits(g)


def test_grouped_quantisation_plan_checks():
    lw = BitLinearWeight(64, 256, 6, 8)
    W = torch.zeros(64 * 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        QuantGroup([(lw, W), (BitLinearWeight(64, 256, 8, 8), W)])
    qg = QuantGroup([(lw, W)])
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_quant_group_plan(qg.items, 1, 6, 8, 0, qg.ws[:0], qg.plan)
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_quant_group_plan(qg.items, 1, 6, 8, 0, qg.ws, qg.plan[:16])
    # a run with another pattern or gamma mode than the plan's writes no
    # mask or packed byte and turns gamma into NaN, so the stale codes show
    for n_run, m_run, go_run in ((2, 8, 0), (6, 8, 1), (4, 8, 0)):
        lw.mask.fill_(0x33)
        lw.packed.fill_(0x44)
        lw.gamma.fill_(7.0)
        bl.bitlinear_quant_group(qg.plan, n_run, m_run, go_run)
        torch.cuda.synchronize()
        assert (lw.mask == 0x33).all() and (lw.packed == 0x44).all()
        assert np.isnan(lw.gamma.item()), (n_run, m_run, go_run)
    # and everything formed with that gamma is NaN
    X = bf16_tensor(synth.activations(4, 256, seed=3))
    bufs = lw.fwd(X, 4)
    torch.cuda.synchronize()
    assert torch.isnan(bufs["Y"]).all()
    qg.run()
    torch.cuda.synchronize()
    Z = np.zeros((64, 256), np.uint16)
    mb = oracle.mask(Z, 6, 8)  # all magnitudes equal: the lower indices are kept
    assert lw.gamma.cpu().item() == 0.0
    assert np.array_equal(lw.mask.cpu().numpy().reshape(mb.shape), mb)
    assert np.array_equal(lw.packed.cpu().numpy(), oracle.pack(oracle.ternary(Z, mb, 0.0), 6))


def _near_half_way_rows(rng, rows, k):
    """Rows whose quotients 127 x / a sit on or within 2^-11 of half-integers
    (exact ties included), for random bf16 maxima a, plus rows whose maximum
    is tiny (subnormal, and the smallest magnitudes around 2^-100)."""
    out = np.zeros((rows, k), np.uint16)
    for r in range(rows):
        if r == rows - 1:
            a_bits = 0x0040  # subnormal maximum
        elif r == rows - 2:
            a_bits = 0x0D80  # 2^-100
        elif r == rows - 3:
            a_bits = 0x0D7F  # just below 2^-100
        else:
            a_bits = int(rng.integers(0x3000, 0x4C00))  # about 2^-31 .. 2^25
        mags = np.arange(1, a_bits + 1, dtype=np.uint32).astype(np.uint16)
        vals = synth.bf16_bits_to_f32(mags).astype(np.float64)
        a = vals[-1]
        q = 127.0 * vals / a
        near = np.abs(np.abs(q - np.floor(q)) - 0.5) <= 2.0 ** -11
        pick = mags[near]
        if pick.size == 0 or a_bits < 0x0080:
            pick = mags
        sel = rng.choice(pick, size=k - 1, replace=True)
        sel = sel | (rng.integers(0, 2, size=k - 1).astype(np.uint16) << 15)
        out[r, 0] = a_bits | (0x8000 if r % 2 else 0)
        out[r, 1:] = sel
    return out


@pytest.mark.parametrize("rows,k", [(40, 1024), (9, 8960)])
def test_act_quant_near_half_way_quotients(rows, k):
    """The activation codes are round-half-even of the exact quotient,
    including quotients on or next to half-integers (taken exactly), and
    rows whose maximum is below 2^-100 (division path)."""
    rng = np.random.default_rng(rows + k)
    X = _near_half_way_rows(rng, rows, k)
    xq_ref, sc_ref = oracle.act_quant(X)
    xq = torch.empty(rows * k, dtype=torch.int8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    bl.bitlinear_act_quant(bf16_tensor(X), rows, k, xq, sc)
    torch.cuda.synchronize()
    got = xq.cpu().numpy().reshape(rows, k)
    assert np.array_equal(got, xq_ref), f"x_q differs at {np.argwhere(got != xq_ref)[:5]}"
    assert np.array_equal(sc.cpu().numpy(), sc_ref.astype(np.float32))


@pytest.mark.parametrize("count", [8, 3 * 2048 + 8, 256 * 4864])
def test_latent_update_matches_oracle(count):
    """binary32 latent weights after one gradient step and their bf16 copy:
    bit-exact against the oracle, with half-way cases planted up front."""
    rng = np.random.default_rng(count)
    w = (rng.standard_normal(count) * 0.02).astype(np.float32)
    g = (rng.standard_normal(count) * 1e-2).astype(np.float32)
    lr = np.float32(0.25)
    if count >= 8:  # w - lr*g exactly half-way between two binary32 / bf16 values
        w[:4] = [1.0 + 2.0 ** -23, 1.0 + 2.0 ** -22, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]
        g[:4] = [2.0 ** -22, 2.0 ** -22, 0.0, 0.0]
    ref_w, ref_b = oracle.latent_update(w, g, lr)
    Wm = torch.from_numpy(w.copy()).cuda()
    Wb = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    bl.bitlinear_latent_update(Wm, torch.from_numpy(g).cuda(), count, float(lr), Wb)
    torch.cuda.synchronize()
    assert np.array_equal(Wm.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    assert np.array_equal(Wb.view(torch.int16).cpu().numpy().view(np.uint16), ref_b)


def test_dense_to_sparse_training_steps():
    """Four training steps of one layer, dense (8:8) for two then 6:8: each
    step's mask, gamma and packed bytes from the current latent weights,
    the forward, and the latent update (with this step's dW) match the
    oracle on the same inputs; dW within the bf16-product tolerance."""
    n_out, k, tokens, lr = 64, 256, 32, 0.5
    lat = LatentWeights(bf16_tensor(synth.weights(n_out, k, seed=50)))
    for step in range(4):
        n, m = dense_to_sparse(step, 2, 6, 8)
        Wbits = bf16_bits(lat.W).reshape(n_out, k)
        lw, T, g = H.check_weight_path(Wbits, n, m)
        X = synth.activations(tokens, k, seed=60 + step)
        bufs, xq, sc = H.check_forward(lw, T, g, X)
        dY = synth.grad_output(tokens, n_out, seed=70 + step)
        _, dW = lw.bwd(bf16_tensor(dY), bufs["xq"], bufs["x_scale"], tokens, dX=False)
        torch.cuda.synchronize()
        dW_ref = oracle.bwd_dw_pairs(dY, xq, sc, np.repeat(np.arange(n_out), k), np.tile(np.arange(k), n_out))
        got = dW.cpu().numpy().astype(np.float64)
        bound = oracle.bwd_dw_pairs((dY & np.uint16(0x7FFF)).astype(np.uint16), np.abs(xq), sc,
                                    np.repeat(np.arange(n_out), k), np.tile(np.arange(k), n_out))
        assert np.all(np.abs(got - dW_ref) <= 1e-2 * bound + 1e-30)
        master_before = lat.master.cpu().numpy()
        ref_w, ref_b = oracle.latent_update(master_before, dW.cpu().numpy(), lr)
        lat.update(dW, lr)
        torch.cuda.synchronize()
        assert np.array_equal(lat.master.cpu().numpy().reshape(-1).view(np.uint32), ref_w.view(np.uint32)), step
        assert np.array_equal(bf16_bits(lat.W).reshape(-1), ref_b), step


@pytest.mark.parametrize("tokens,n", [(37, 6912), (5, 9216), (1, 128)])
def test_relu2_gate_matches_oracle(tokens, n):
    """Squared-ReLU gating: h (bf16), and the down projection's x_q and
    x_scale formed from it, bit-exact against the oracle (gating, then the
    oracle's activation quantisation of h); rows wider than the registers
    hold take the recomputing path."""
    rng = np.random.default_rng(tokens * n)
    G = rng.standard_normal((tokens, n)).astype(np.float32)
    U = rng.standard_normal((tokens, n)).astype(np.float32)
    G[0, :16] = [0.0, -0.0, -1.0, 2.0, 1e-30, -1e-30, 3.0, 0.5] * 2
    H_ref = oracle.relu2_gate(G, U)
    xq_ref, sc_ref = oracle.act_quant(H_ref)
    Gd, Ud = torch.from_numpy(G).cuda(), torch.from_numpy(U).cuda()
    H = torch.empty(tokens * n, dtype=torch.bfloat16, device="cuda")
    xq = torch.empty(tokens * n, dtype=torch.int8, device="cuda")
    sc = torch.empty(tokens, dtype=torch.float32, device="cuda")
    bl.bitlinear_relu2_gate(Gd, Ud, tokens, n, H, xq, sc)
    xq2 = torch.empty_like(xq)
    sc2 = torch.empty_like(sc)
    bl.bitlinear_relu2_gate(Gd, Ud, tokens, n, None, xq2, sc2)  # without H
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(H).reshape(tokens, n), H_ref)
    assert np.array_equal(xq.cpu().numpy().reshape(tokens, n), xq_ref)
    assert np.array_equal(sc.cpu().numpy(), sc_ref.astype(np.float32))
    assert torch.equal(xq, xq2) and torch.equal(sc, sc2)


@pytest.mark.parametrize("count", [8, 2048 * 3 + 8, 4096 * 6912])
def test_relu2_gate_bwd_matches_oracle(count):
    rng = np.random.default_rng(count)
    d = rng.standard_normal(count).astype(np.float32)
    g = rng.standard_normal(count).astype(np.float32)
    u = rng.standard_normal(count).astype(np.float32)
    dg_ref, du_ref = oracle.relu2_gate_bwd(d, g, u)
    dG = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    dU = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    bl.bitlinear_relu2_gate_bwd(torch.from_numpy(d).cuda(), torch.from_numpy(g).cuda(),
                                torch.from_numpy(u).cuda(), count, dG, dU)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(dG), dg_ref)
    assert np.array_equal(bf16_bits(dU), du_ref)


def _group_entries(shapes, tokens, n, m, seed):
    entries = []
    for i, (n_out, k) in enumerate(shapes):
        W = synth.weights(n_out, k, seed=seed + i)
        X = synth.activations(tokens, k, seed=seed + 100 + i)
        lw = BitLinearWeight(n_out, k, n, m)
        lw.quantize(bf16_tensor(W))
        entries.append(dict(X=bf16_tensor(X), packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                            Y=torch.full((tokens * n_out,), float("nan"), dtype=torch.float32, device="cuda"),
                            xq=torch.zeros(tokens * k, dtype=torch.int8, device="cuda"),
                            x_scale=torch.zeros(tokens, dtype=torch.float32, device="cuda"), lw=lw))
    return entries


@pytest.mark.parametrize("tokens,shapes", [
    (1, [(896, 896), (128, 896), (128, 896), (896, 896), (4864, 896), (4864, 896), (896, 4864)] * 2),
    (1, [(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)]),
    (5, [(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)]),
    (8, [(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)]),
    (1, [(11008, 2048)] * 4 + [(2048, 11008)] * 2),
    # 5 rows of 11 segments (ten of 1024 values and one of 768): 55 of the
    # workgroup's 64 absmax slots, each row's maximum over 11 of them
    (5, [(128, 11008), (64, 256)]),
])
def test_grouped_decode_fused_matches_two_launches(tokens, shapes, n=6, m=8):
    """Stage 4 (activation quantisation inside the contraction launch):
    Y, x_q and x_scale bit-identical to stage 3 (two launches)."""
    entries = _group_entries(shapes, tokens, n, m, seed=700)
    items = bl.make_fwd_items(entries, tokens)
    assert bl.bitlinear_fwd_group_plan_fuses(items, len(entries), tokens, n, m)
    plan = torch.empty(bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens), dtype=torch.uint8,
                       device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
    bl.bitlinear_fwd_group(plan, n, m, 3)
    torch.cuda.synchronize()
    ref = [(e["Y"].cpu().numpy().copy(), e["xq"].cpu().numpy().copy(), e["x_scale"].cpu().numpy().copy())
           for e in entries]
    for rep in range(2):
        for e in entries:
            e["Y"].fill_(float("nan"))
            e["xq"].zero_()
            e["x_scale"].zero_()
        bl.bitlinear_fwd_group(plan, n, m, 4)
        torch.cuda.synchronize()
        for i, (e, (Y, xq, sc)) in enumerate(zip(entries, ref)):
            assert np.array_equal(e["Y"].cpu().numpy().view(np.uint32), Y.view(np.uint32)), i
            assert np.array_equal(e["xq"].cpu().numpy(), xq), i
            assert np.array_equal(e["x_scale"].cpu().numpy().view(np.uint32), sc.view(np.uint32)), i


@pytest.mark.parametrize("n,m", [(8, 8), (2, 8), (2, 4)])
def test_grouped_decode_fused_other_patterns(n, m):
    """Stage 4 at the other sign-slot counts (S = 8, 2, 4): bit-identical to
    stage 3 at 1 and 3 tokens."""
    shapes = [(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)]
    for tokens in (1, 3):
        test_grouped_decode_fused_matches_two_launches(tokens, shapes, n, m)


@pytest.mark.parametrize("tokens", [16, 6])
def test_grouped_decode_fused_run_of_unfused_plan_is_nan(tokens):
    """A plan whose workgroups' activation rows do not fit LDS (16 tokens of
    an 11008-wide item) or need more than the 64 segment slots (6 tokens:
    66 segments, 66 KB of codes) cannot run stage 4: every Y becomes NaN,
    and the plan then still runs as two launches."""
    n, m = 6, 8
    entries = _group_entries([(128, 11008), (64, 256)], tokens, n, m, seed=900)
    items = bl.make_fwd_items(entries, tokens)
    assert not bl.bitlinear_fwd_group_plan_fuses(items, len(entries), tokens, n, m)
    plan = torch.empty(bl.bitlinear_fwd_group_plan_bytes(items, len(entries), tokens), dtype=torch.uint8,
                       device="cuda")
    bl.bitlinear_fwd_group_plan(items, len(entries), tokens, n, m, plan)
    for e in entries:
        e["Y"].zero_()
    bl.bitlinear_fwd_group(plan, n, m, 4)
    torch.cuda.synchronize()
    for e in entries:
        assert torch.isnan(e["Y"]).all()
    bl.bitlinear_fwd_group(plan, n, m, 3)
    torch.cuda.synchronize()
    for e in entries:
        X = e["X"].view(torch.int16).cpu().numpy().view(np.uint16).reshape(tokens, e["k"])
        xq, sc = oracle.act_quant(X)
        assert np.array_equal(e["xq"].cpu().numpy().reshape(xq.shape), xq)
        assert not torch.isnan(e["Y"]).any()
