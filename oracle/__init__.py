"""CPU oracle for the Sparse-BitNet BitLinear path -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and it shares no code with them.

The arithmetic lives in oracle.c (plain C, binary64 / exact integers); this
module only marshals numpy arrays through ctypes.  Each wrapper names the
step it computes; the definitions and the readings of the pages are stated
in oracle.c next to the code.

bf16 tensors are passed as numpy uint16 arrays of raw bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_mask": (None, [_vp, _i64, _i64, _int, _int, _vp]),
        "oracle_gamma": (_dbl, [_vp, _i64, _i64, _int, _vp]),
        "oracle_ternary": (None, [_vp, _vp, _dbl, _i64, _i64, _vp]),
        "oracle_act_quant": (None, [_vp, _i64, _i64, _vp, _vp]),
        "oracle_fwd": (_int, [_vp, _vp, _vp, _dbl, _i64, _i64, _i64, _vp, _vp, _int]),
        "oracle_fwd_pairs": (None, [_vp, _vp, _vp, _dbl, _i64, _vp, _vp, _i64, _vp, _vp]),
        "oracle_fwd_bf16": (_int, [_vp, _vp, _vp, _dbl, _i64, _i64, _i64, _vp]),
        "oracle_bwd_dx": (None, [_vp, _vp, _dbl, _i64, _i64, _i64, _vp, _int]),
        "oracle_bwd_dw": (None, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _int]),
        "oracle_bwd_dx_pairs": (None, [_vp, _vp, _dbl, _i64, _i64, _vp, _vp, _i64, _vp]),
        "oracle_bwd_dw_pairs": (None, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
        "oracle_s_of": (_int, [_int, _int]),
        "oracle_packed_bytes": (_i64, [_i64, _i64, _int]),
        "oracle_pack": (_int, [_vp, _i64, _i64, _int, _vp]),
        "oracle_unpack": (None, [_vp, _i64, _i64, _int, _vp]),
        "oracle_sp24_packed_bytes": (_i64, [_i64, _i64]),
        "oracle_pack_sp24": (_int, [_vp, _i64, _i64, _vp]),
        "oracle_unpack_sp24": (None, [_vp, _i64, _i64, _vp]),
        "oracle_latent_update": (None, [_vp, _vp, _i64, ctypes.c_float, _vp]),
        "oracle_relu2_gate": (None, [_vp, _vp, _i64, _vp]),
        "oracle_relu2_gate_bwd": (None, [_vp, _vp, _vp, _i64, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def mask(W, n, m):
    """N:M mask of latent W (uint16 bf16 bits, [n_out, k]) -> uint8 [n_out, k/8]."""
    W = _c(W, np.uint16)
    n_out, k = W.shape
    out = np.zeros((n_out, k // 8), dtype=np.uint8)
    _load().oracle_mask(_p(W), n_out, k, n, m, _p(out))
    return out


def gamma(W, over_masked=False, mask_bits=None):
    """Absmean scale: exact sum of |W| rounded once to binary64, over count."""
    W = _c(W, np.uint16)
    n_out, k = W.shape
    mb = _c(mask_bits if mask_bits is not None else np.zeros((n_out, k // 8), np.uint8), np.uint8)
    return _load().oracle_gamma(_p(W), n_out, k, int(bool(over_masked)), _p(mb))


def ternary(W, mask_bits, g):
    """Masked ternary codes int8 [n_out, k] in {-1, 0, 1}."""
    W = _c(W, np.uint16)
    mb = _c(mask_bits, np.uint8)
    n_out, k = W.shape
    out = np.zeros((n_out, k), dtype=np.int8)
    _load().oracle_ternary(_p(W), _p(mb), float(g), n_out, k, _p(out))
    return out


def act_quant(X):
    """Per-token absmax int8 quantisation -> (x_q int8 [T, k], scale float64 [T])."""
    X = _c(X, np.uint16)
    tokens, k = X.shape
    xq = np.zeros((tokens, k), dtype=np.int8)
    sc = np.zeros(tokens, dtype=np.float64)
    _load().oracle_act_quant(_p(X), tokens, k, _p(xq), _p(sc))
    return xq, sc


def fwd(xq, scale, T, g, threads=1, want_acc=True, want_y=True):
    """Contraction + epilogue -> (acc int32 [T, n] or None, Y float64 [T, n] or None)."""
    xq = _c(xq, np.int8)
    scale = _c(scale, np.float64)
    T = _c(T, np.int8)
    tokens, k = xq.shape
    n_out = T.shape[0]
    acc = np.zeros((tokens, n_out), dtype=np.int32) if want_acc else None
    Y = np.zeros((tokens, n_out), dtype=np.float64) if want_y else None
    ovf = _load().oracle_fwd(_p(xq), _p(scale), _p(T), float(g), tokens, k, n_out,
                             _p(acc) if acc is not None else None,
                             _p(Y) if Y is not None else None, int(threads))
    if ovf:
        raise OverflowError("an accumulator left the int32 range")
    return acc, Y


def fwd_bf16(xq, scale, T, g):
    """Contraction + epilogue with bf16 outputs -> uint16 [T, n] bf16 bits."""
    xq = _c(xq, np.int8)
    scale = _c(scale, np.float64)
    T = _c(T, np.int8)
    tokens, k = xq.shape
    n_out = T.shape[0]
    Y = np.zeros((tokens, n_out), dtype=np.uint16)
    if _load().oracle_fwd_bf16(_p(xq), _p(scale), _p(T), float(g), tokens, k, n_out, _p(Y)):
        raise OverflowError("an accumulator left the int32 range")
    return Y


def fwd_pairs(xq, scale, T, g, t_idx, n_idx):
    """Selected outputs: (acc int64 [P], Y float64 [P]) at the (t, n) pairs."""
    xq = _c(xq, np.int8)
    scale = _c(scale, np.float64)
    T = _c(T, np.int8)
    t_idx = _c(t_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    cnt = t_idx.size
    acc = np.zeros(cnt, dtype=np.int64)
    Y = np.zeros(cnt, dtype=np.float64)
    _load().oracle_fwd_pairs(_p(xq), _p(scale), _p(T), float(g), xq.shape[1],
                             _p(t_idx), _p(n_idx), cnt, _p(acc), _p(Y))
    return acc, Y


def bwd_dx(dY, T, g, threads=1):
    """dX = gamma * dY @ T  (binary64) -> float64 [T, k]."""
    dY = _c(dY, np.uint16)
    T = _c(T, np.int8)
    tokens, n_out = dY.shape
    k = T.shape[1]
    out = np.zeros((tokens, k), dtype=np.float64)
    _load().oracle_bwd_dx(_p(dY), _p(T), float(g), tokens, k, n_out, _p(out), int(threads))
    return out


def bwd_dw(dY, xq, scale, threads=1):
    """dW = (dY)^T @ (x_q * s)  (binary64) -> float64 [n_out, k], dense."""
    dY = _c(dY, np.uint16)
    xq = _c(xq, np.int8)
    scale = _c(scale, np.float64)
    tokens, n_out = dY.shape
    k = xq.shape[1]
    out = np.zeros((n_out, k), dtype=np.float64)
    _load().oracle_bwd_dw(_p(dY), _p(xq), _p(scale), tokens, k, n_out, _p(out), int(threads))
    return out


def bwd_dx_pairs(dY, T, g, t_idx, c_idx):
    dY = _c(dY, np.uint16)
    T = _c(T, np.int8)
    t_idx = _c(t_idx, np.int64)
    c_idx = _c(c_idx, np.int64)
    out = np.zeros(t_idx.size, dtype=np.float64)
    _load().oracle_bwd_dx_pairs(_p(dY), _p(T), float(g), T.shape[1], T.shape[0],
                                _p(t_idx), _p(c_idx), t_idx.size, _p(out))
    return out


def bwd_dw_pairs(dY, xq, scale, r_idx, c_idx):
    dY = _c(dY, np.uint16)
    xq = _c(xq, np.int8)
    scale = _c(scale, np.float64)
    r_idx = _c(r_idx, np.int64)
    c_idx = _c(c_idx, np.int64)
    out = np.zeros(r_idx.size, dtype=np.float64)
    _load().oracle_bwd_dw_pairs(_p(dY), _p(xq), _p(scale), xq.shape[0], xq.shape[1],
                                dY.shape[1], _p(r_idx), _p(c_idx), r_idx.size, _p(out))
    return out


def s_of(n, m):
    """Sign slots per 8-group in the packed format (-1 if N:M unsupported)."""
    return _load().oracle_s_of(int(n), int(m))


def packed_bytes(n_out, k, s):
    return _load().oracle_packed_bytes(int(n_out), int(k), int(s))


def pack(T, s):
    """Packed bytes (uint8 [packed_bytes]) of ternary codes T [n_out, k]."""
    T = _c(T, np.int8)
    n_out, k = T.shape
    out = np.zeros(packed_bytes(n_out, k, s), dtype=np.uint8)
    if _load().oracle_pack(_p(T), n_out, k, int(s), _p(out)) != 0:
        raise ValueError("a group holds more nonzeros than the format allows")
    return out


def unpack(packed, n_out, k, s):
    packed = _c(packed, np.uint8)
    T = np.zeros((n_out, k), dtype=np.int8)
    _load().oracle_unpack(_p(packed), int(n_out), int(k), int(s), _p(T))
    return T


def sp24_packed_bytes(n_out, k):
    return _load().oracle_sp24_packed_bytes(int(n_out), int(k))


def pack_sp24(T):
    """2:4 codes T [n_out, k] in the sparse-operand + index layout (uint8)."""
    T = _c(T, np.int8)
    n_out, k = T.shape
    out = np.zeros(sp24_packed_bytes(n_out, k), dtype=np.uint8)
    if _load().oracle_pack_sp24(_p(T), n_out, k, _p(out)) != 0:
        raise ValueError("a quad holds more than two nonzero codes")
    return out


def unpack_sp24(packed, n_out, k):
    packed = _c(packed, np.uint8)
    T = np.zeros((n_out, k), dtype=np.int8)
    _load().oracle_unpack_sp24(_p(packed), int(n_out), int(k), _p(T))
    return T


def forward_all(W, X, n, m, over_masked=False, threads=1):
    """The whole forward path in the order the steps run: mask, gamma,
    ternary, activation quantisation, contraction and epilogue."""
    mb = mask(W, n, m)
    g = gamma(W, over_masked, mb)
    T = ternary(W, mb, g)
    xq, sc = act_quant(X)
    acc, Y = fwd(xq, sc, T, g, threads=threads)
    return {"mask": mb, "gamma": g, "T": T, "xq": xq, "scale": sc, "acc": acc, "Y": Y}


def latent_update(w_master, dw, lr):
    """Plain gradient step on binary32 latent weights -> (new binary32
    weights, their bf16 bit patterns); the inputs are not modified."""
    wm = np.array(w_master, dtype=np.float32, copy=True).reshape(-1)
    g = _c(np.asarray(dw, dtype=np.float32).reshape(-1), np.float32)
    out = np.zeros(wm.size, dtype=np.uint16)
    _load().oracle_latent_update(_p(wm), _p(g), wm.size, float(np.float32(lr)), _p(out))
    return wm, out


def relu2_gate(G, U):
    """Squared-ReLU gating -> bf16 bit patterns of h (same shape as G)."""
    g = _c(G, np.float32)
    u = _c(U, np.float32)
    h = np.zeros(g.shape, dtype=np.uint16)
    _load().oracle_relu2_gate(_p(g), _p(u), g.size, _p(h))
    return h


def relu2_gate_bwd(dH, G, U):
    """Its backward -> (dG, dU) as bf16 bit patterns."""
    d = _c(dH, np.float32)
    g = _c(G, np.float32)
    u = _c(U, np.float32)
    dg = np.zeros(g.shape, dtype=np.uint16)
    du = np.zeros(g.shape, dtype=np.uint16)
    _load().oracle_relu2_gate_bwd(_p(d), _p(g), _p(u), g.size, _p(dg), _p(du))
    return dg, du
