"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle
checks.  This module holds no arithmetic of the method itself: it only draws
normal samples and rounds them to bf16 bit patterns.

Recipe (one stream per tensor):
  rng = numpy.random.Generator(PCG64(SeedSequence([seed, config, layer, tensor])))
  v   = rng.standard_normal(shape) (binary64) * std
  bits = bf16 bit pattern of v, rounded to nearest-even to binary32 and then
         to nearest-even to bf16 with explicit integer operations.

The distributions follow the workloads the pages describe (latent weights of
a pretrained-scale LLM and unit-scale activations): W ~ N(0, 0.02^2),
X ~ N(0, 1), dY ~ N(0, 1).
"""
import numpy as np

W_STD = 0.02
X_STD = 1.0
DY_STD = 1.0

# tensor ids inside a layer's seed sequence
TENSOR_W, TENSOR_X, TENSOR_DY = 0, 1, 2


def f32_to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even) -> uint16 bits.
    NaN/Inf never occur for the finite normal draws used here."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std, seed=0, config=0, layer=0, tensor=0) -> np.ndarray:
    ss = np.random.SeedSequence([int(seed), int(config), int(layer), int(tensor)])
    rng = np.random.Generator(np.random.PCG64(ss))
    v = rng.standard_normal(size=shape, dtype=np.float64) * std
    return f32_to_bf16_bits(v.astype(np.float32))


def weights(n_out, k, seed=0, config=0, layer=0):
    return normal_bf16((n_out, k), W_STD, seed, config, layer, TENSOR_W)


def activations(tokens, k, seed=0, config=0, layer=0):
    return normal_bf16((tokens, k), X_STD, seed, config, layer, TENSOR_X)


def grad_output(tokens, n_out, seed=0, config=0, layer=0):
    return normal_bf16((tokens, n_out), DY_STD, seed, config, layer, TENSOR_DY)
