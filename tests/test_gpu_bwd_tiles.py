"""The backward products on 256 x 128 and 256 x 256 workgroup tiles (LDS
DMA, wavefronts of 128 x 64) against the 128 x 128 tiles and the oracle.
Every tile size contracts k in the same order through the same MFMA
instruction, so dX and dW must agree bit for bit; ragged shapes cover rows
and columns past the tile edges and contraction depths that end inside a
32-wide LDS stage."""
import numpy as np
import pytest
import torch

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl
from sparse_linear_layers_group_amd import synth
from sparse_linear_layers_group_amd.layer import bf16_tensor

import _gpu_helpers as H

pytestmark = pytest.mark.gpu


def _grads(lw, dY, bufs, tokens, tiles):
    bl.bitlinear_bwd_tiles(tiles)
    try:
        dX, dW = lw.bwd(dY, bufs["xq"], bufs["x_scale"], tokens)
        torch.cuda.synchronize()
    finally:
        bl.bitlinear_bwd_tiles(0)
    return dX.cpu().numpy(), dW.cpu().numpy()


@pytest.mark.parametrize("n_out,k,tokens", [
    (272, 384, 300),    # every edge ragged; dX depth 272 ends half way into a stage
    (48, 256, 7),       # one tile, mostly past the edges
    (512, 1024, 520),   # whole 256 x 128 tiles plus a ragged token edge
    (1040, 640, 256),   # several tiles both ways, dW depth 256
])
def test_bwd_256_row_tiles_match_128_tiles_and_oracle(n_out, k, tokens):
    seed = n_out + 7 * k + tokens
    W = synth.weights(n_out, k, seed=seed)
    X = synth.activations(tokens, k, seed=seed)
    dYb = synth.grad_output(tokens, n_out, seed=seed)
    lw, T, g = H.check_weight_path(W, 6, 8)
    bufs, xq, sc = H.check_forward(lw, T, g, X)
    dY = bf16_tensor(dYb)
    dx128, dw128 = _grads(lw, dY, bufs, tokens, 1)
    for kind in (2, 3):
        dx256, dw256 = _grads(lw, dY, bufs, tokens, kind)
        assert np.array_equal(dx256.view(np.uint32), dx128.view(np.uint32)), kind
        assert np.array_equal(dw256.view(np.uint32), dw128.view(np.uint32)), kind
    dyv = np.abs(synth.bf16_bits_to_f32(dYb).astype(np.float64))
    ref_dx = oracle.bwd_dx(dYb, T, g)
    H.assert_grad_close(dx256.reshape(ref_dx.shape).astype(np.float64), ref_dx,
                        g * (dyv @ np.abs(T).astype(np.float64)))
    ref_dw = oracle.bwd_dw(dYb, xq, sc)
    H.assert_grad_close(dw256.reshape(ref_dw.shape).astype(np.float64), ref_dw,
                        dyv.T @ (np.abs(xq) * sc[:, None]))


def test_bwd_tiles_rejects_other_sizes():
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_bwd_tiles(4)
    bl.bitlinear_bwd_tiles(0)


def _splits(M, N, K):
    """bitlinear_bwd's split rule: at most 128 tiles of 128 x 128 and k >= 2048."""
    tiles = -(-M // 128) * -(-N // 128)
    return tiles <= 128 and K >= 2048


def _group_case(shapes, tokens, outputs, seed, inputs=None):
    """Layers with synthetic weights, activations and output gradients, their
    per-layer bitlinear_bwd results, and the grouped call's.  Layers with the
    same entry in `inputs` take the same activations and pass the same x_q
    and s_t tensors (as layers fed one input do)."""
    layers, entries, fed = [], [], {}
    for i, (n_out, k) in enumerate(shapes):
        W = synth.weights(n_out, k, seed=seed + i)
        src = i if inputs is None else inputs[i]
        dYb = synth.grad_output(tokens, n_out, seed=seed + 90 + i)
        lw, _, _ = H.quantize_on_gpu(W, 6, 8, want_wq=False)
        if src not in fed:
            fed[src] = lw.fwd(bf16_tensor(synth.activations(tokens, k, seed=seed + 50 + src)), tokens)
        bufs = fed[src]
        dY = bf16_tensor(dYb)
        want_dx, want_dw = outputs[i]
        ref = lw.bwd(dY, bufs["xq"], bufs["x_scale"], tokens, dX=want_dx, dW=want_dw)
        e = dict(dY=dY, xq=bufs["xq"], x_scale=bufs["x_scale"], packed=lw.packed, gamma=lw.gamma, k=k, n_out=n_out,
                 dX=torch.full((tokens * k,), float("nan"), device="cuda") if want_dx else None,
                 dW=torch.full((n_out * k,), float("nan"), device="cuda") if want_dw else None)
        layers.append((n_out, k, ref))
        entries.append(e)
    items = bl.make_bwd_items(entries, tokens)
    ws = torch.empty(max(bl.bitlinear_bwd_group_workspace_bytes(items, len(entries), tokens), 256),
                     dtype=torch.uint8, device="cuda")
    bl.bitlinear_bwd_group(items, len(entries), tokens, 6, 8, ws)
    torch.cuda.synchronize()
    return layers, entries


@pytest.mark.parametrize("shapes,tokens,outputs,inputs", [
    # ragged layers, some outputs skipped
    ([(272, 384), (48, 256), (512, 1024), (1040, 640)], 300,
     [(True, True), (True, False), (False, True), (True, True)], None),
    # ragged layers fed one input (one prepared x_q), one fed another
    ([(272, 384), (48, 384), (512, 384), (1040, 640)], 300,
     [(True, True), (False, True), (True, True), (True, True)], [0, 0, 0, 1]),
    # BitNet-2B4T q, k, v (one input), o at 4096 tokens (the k and v dW are
    # split along k by per-layer calls)
    ([(2560, 2560), (640, 2560), (640, 2560), (2560, 2560)], 4096, [(True, True)] * 4, [0, 0, 0, 1]),
    # BitNet-2B4T gate and up (one input) and down's dW alone, as the
    # training step groups them after down's dX and the gating backward
    ([(6912, 2560), (6912, 2560), (2560, 6912)], 4096, [(True, True), (True, True), (False, True)],
     [0, 0, 1]),
])
def test_bwd_group_matches_per_layer_calls(shapes, tokens, outputs, inputs):
    """bitlinear_bwd_group against bitlinear_bwd on each layer: bit for bit,
    except products the per-layer call splits along k, which agree to
    binary32 rounding (relative Frobenius difference below 1e-5)."""
    layers, entries = _group_case(shapes, tokens, outputs, seed=tokens + len(shapes), inputs=inputs)
    for (n_out, k, ref), e in zip(layers, entries):
        for name, got, want, split in (("dX", e["dX"], ref[0], _splits(tokens, k, n_out)),
                                       ("dW", e["dW"], ref[1], _splits(n_out, k, -(-tokens // 64) * 64))):
            if got is None:
                continue
            g, w = got.cpu().numpy(), want.cpu().numpy()
            if split:
                d = np.linalg.norm((g - w).astype(np.float64)) / np.linalg.norm(w.astype(np.float64))
                assert d < 1e-5, (name, n_out, k, d)
            else:
                assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), (name, n_out, k)


def test_bwd_group_many_items():
    """Nine layers: 22 conversion tasks (two conversion launches of at most
    16 tasks) and 17 products (two product launches of at most 16), four of
    the layers sharing one input; bit-identical to per-layer calls except
    split products."""
    shapes = [(64, 256), (128, 384), (48, 256), (256, 640), (192, 256), (80, 512), (320, 256), (64, 384),
              (112, 768)]  # (n_out, k); the layers fed input 0 share k = 256
    outputs = [(True, True)] * 8 + [(True, False)]
    inputs = [0, 1, 0, 2, 0, 3, 0, 4, 5]
    tokens = 200
    layers, entries = _group_case(shapes, tokens, outputs, seed=91, inputs=inputs)
    for (n_out, k, ref), e in zip(layers, entries):
        for name, got, want, split in (("dX", e["dX"], ref[0], _splits(tokens, k, n_out)),
                                       ("dW", e["dW"], ref[1], _splits(n_out, k, -(-tokens // 64) * 64))):
            if got is None:
                continue
            g, w = got.cpu().numpy(), want.cpu().numpy()
            if split:
                d = np.linalg.norm((g - w).astype(np.float64)) / np.linalg.norm(w.astype(np.float64))
                assert d < 1e-5, (name, n_out, k, d)
            else:
                assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), (name, n_out, k)


def test_bwd_group_reruns_bit_identical():
    """A second grouped call on the same inputs (the same workspace reused)
    gives the same bits."""
    shapes, tokens = [(272, 384), (48, 384), (512, 384)], 300
    layers, entries = _group_case(shapes, tokens, [(True, True)] * 3, seed=23, inputs=[0, 0, 0])
    first = [(e["dX"].cpu().numpy().copy(), e["dW"].cpu().numpy().copy()) for e in entries]
    items = bl.make_bwd_items(entries, tokens)
    ws = torch.empty(max(bl.bitlinear_bwd_group_workspace_bytes(items, len(entries), tokens), 256),
                     dtype=torch.uint8, device="cuda")
    bl.bitlinear_bwd_group(items, len(entries), tokens, 6, 8, ws)
    torch.cuda.synchronize()
    for (dx, dw), e in zip(first, entries):
        assert np.array_equal(dx.view(np.uint32), e["dX"].cpu().numpy().view(np.uint32))
        assert np.array_equal(dw.view(np.uint32), e["dW"].cpu().numpy().view(np.uint32))


def test_bwd_group_no_tokens_zeroes_dw():
    """No tokens: every requested dW becomes zeros, no workspace needed."""
    entries = []
    for n_out, k in ((128, 256), (64, 384)):
        lw, _, _ = H.quantize_on_gpu(synth.weights(n_out, k, seed=n_out), 6, 8, want_wq=False)
        entries.append(dict(dY=torch.empty(0, dtype=torch.bfloat16, device="cuda"), packed=lw.packed,
                            gamma=lw.gamma, k=k, n_out=n_out,
                            dW=torch.full((n_out * k,), float("nan"), device="cuda")))
    items = bl.make_bwd_items(entries, 0)
    bl.bitlinear_bwd_group(items, len(entries), 0, 6, 8)
    torch.cuda.synchronize()
    for e in entries:
        assert torch.count_nonzero(e["dW"]).item() == 0


@pytest.mark.parametrize("n_out,k,tokens,want_dw", [
    (272, 384, 300, True), (48, 256, 70, False),     # ragged
    (2560, 6912, 4096, True),                          # BitNet-2B4T down at 4096 tokens
])
def test_bwd_relu2_gate_matches_separate_calls(n_out, k, tokens, want_dw):
    """The down projection's backward with the gating backward fused into
    its dX epilogue: dG, dU and dW bit-identical to bitlinear_bwd followed
    by bitlinear_relu2_gate_bwd, on every tile choice."""
    lw, _, _ = H.quantize_on_gpu(synth.weights(n_out, k, seed=k + tokens), 6, 8, want_wq=False)
    bufs = lw.fwd(bf16_tensor(synth.activations(tokens, k, seed=tokens)), tokens)
    dY = bf16_tensor(synth.grad_output(tokens, n_out, seed=n_out))
    gen = torch.Generator(device="cuda").manual_seed(tokens)
    G = torch.randn(tokens * k, device="cuda", generator=gen)
    U = torch.randn(tokens * k, device="cuda", generator=gen)
    ws = torch.empty(bl.bitlinear_bwd_workspace_bytes(tokens, k, n_out), dtype=torch.uint8, device="cuda")
    dX = torch.empty(tokens * k, dtype=torch.float32, device="cuda")
    dW_ref = torch.empty(n_out * k, dtype=torch.float32, device="cuda")
    bl.bitlinear_bwd(dY, bufs["xq"], bufs["x_scale"], lw.packed, lw.gamma, tokens, k, n_out, 6, 8, dX, dW_ref, ws=ws)
    dG_ref = torch.empty(tokens * k, dtype=torch.bfloat16, device="cuda")
    dU_ref = torch.empty(tokens * k, dtype=torch.bfloat16, device="cuda")
    bl.bitlinear_relu2_gate_bwd(dX, G, U, tokens * k, dG_ref, dU_ref)
    torch.cuda.synchronize()
    for tiles in (0, 1, 2, 3):
        bl.bitlinear_bwd_tiles(tiles)
        try:
            dG = torch.full((tokens * k,), 0x7fc0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            dU = torch.full((tokens * k,), 0x7fc0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            dW = torch.full((n_out * k,), float("nan"), device="cuda") if want_dw else None
            bl.bitlinear_bwd_relu2_gate(dY, bufs["xq"], bufs["x_scale"], lw.packed, lw.gamma, tokens, k, n_out, 6, 8,
                                        G, U, dG, dU, dW, ws=ws)
            torch.cuda.synchronize()
        finally:
            bl.bitlinear_bwd_tiles(0)
        assert torch.equal(dG.view(torch.int16), dG_ref.view(torch.int16)), tiles
        assert torch.equal(dU.view(torch.int16), dU_ref.view(torch.int16)), tiles
        if want_dw:
            assert np.array_equal(dW.cpu().numpy().view(np.uint32), dW_ref.cpu().numpy().view(np.uint32)), tiles


@pytest.mark.gpu
@pytest.mark.parametrize("shapes,tokens,outputs,inputs", [
    ([(272, 384), (48, 384), (512, 384), (1040, 640)], 300,
     [(True, True), (False, True), (True, True), (True, True)], [0, 0, 0, 1]),
    ([(2560, 2560), (640, 2560), (640, 2560)], 4096, [(True, True)] * 3, [0, 0, 0]),
])
def test_bwd_group_phases_match_one_call(shapes, tokens, outputs, inputs):
    """BL_BWD_PREPARE on a second stream, then BL_BWD_FINISH on the current
    one after an event, on a workspace that starts as garbage: dX and dW
    equal the one-call grouped backward's bit for bit."""
    layers, entries = _group_case(shapes, tokens, outputs, seed=7 * tokens + len(shapes), inputs=inputs)
    fresh = [dict(e, dX=None if e["dX"] is None else torch.full_like(e["dX"], float("nan")),
                  dW=None if e["dW"] is None else torch.full_like(e["dW"], float("nan"))) for e in entries]
    items = bl.make_bwd_items(fresh, tokens)
    need = bl.bitlinear_bwd_group_workspace_bytes(items, len(fresh), tokens)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.bitlinear_bwd_group_phase(items, len(fresh), tokens, 6, 8, bl.BL_BWD_PREPARE, ws,
                                     stream=side.cuda_stream)
    done = torch.cuda.Event()
    done.record(side)
    torch.cuda.current_stream().wait_event(done)
    bl.bitlinear_bwd_group_phase(items, len(fresh), tokens, 6, 8, bl.BL_BWD_FINISH, ws)
    torch.cuda.synchronize()
    for e, f in zip(entries, fresh):
        for name in ("dX", "dW"):
            if e[name] is None:
                continue
            assert np.array_equal(f[name].cpu().numpy().view(np.uint32), e[name].cpu().numpy().view(np.uint32)), name
