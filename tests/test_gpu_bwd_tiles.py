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
