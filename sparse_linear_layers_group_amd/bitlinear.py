"""Thin Python binding of libbitlinear.so (C ABI in include/bitlinear.h).

Argument marshalling only: each function has the C entry point's name and
argument order, takes torch tensors where the C call takes device pointers,
checks dtype / device / contiguity / size, and passes raw pointers and the
caller's HIP stream (default: torch's current stream).  Every step of the
computation runs in the HIP library; if the library is not built, loading
fails with an error -- there is no fallback path.
"""
import ctypes
import os
import re

import numpy as np

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BITLINEAR_LIB") or os.path.join(_HERE, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "bitlinear.h")

BL_OK, BL_EINVAL, BL_ESHAPE, BL_EUNSUPPORTED, BL_EWORKSPACE, BL_EHIP = range(6)
BL_GAMMA_DENSE, BL_GAMMA_MASKED = 0, 1


class BitLinearError(RuntimeError):
    def __init__(self, status, where, detail):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_lib = None
_i64, _int, _sz, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "bitlinear_packed_bytes": (_sz, [_i64, _i64, _int, _int]),
    "bitlinear_workspace_bytes": (_sz, [_i64, _i64]),
    "bitlinear_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_quantize_mask": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_pack": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "bitlinear_fwd": (_int, [_vp, _i64, _i64, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_bwd_tiles": (_int, [_int]),
    "bitlinear_bwd_relu2_gate": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _sz, _vp]),
    "bitlinear_bwd_group_workspace_bytes": (_sz, [_vp, _int, _i64]),
    "bitlinear_bwd_group": (_int, [_vp, _int, _i64, _int, _int, _vp, _sz, _vp]),
    "bitlinear_bwd_group_phase": (_int, [_vp, _int, _i64, _int, _int, _int, _vp, _sz, _vp]),
    "bitlinear_contract_group_workspace_bytes": (_sz, [_vp, _int, _i64, _i64]),
    "bitlinear_contract_group": (_int, [_vp, _int, _vp, _vp, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "bitlinear_fwd_noalloc": (_int, [_vp, _i64, _i64, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "bitlinear_sp24_packed_bytes": (_sz, [_i64, _i64]),
    "bitlinear_sp24_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_pack_sp24": (_int, [_vp, _vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "bitlinear_contract_sp24": (_int, [_vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_act_quant": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "bitlinear_contract": (_int, [_vp, _vp, _i64, _i64, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_fwd_bf16": (_int, [_vp, _i64, _i64, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_contract_bf16": (_int, [_vp, _vp, _i64, _i64, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bitlinear_fwd_group_plan_bytes": (_sz, [_vp, _int, _i64]),
    "bitlinear_fwd_group_plan": (_int, [_vp, _int, _i64, _int, _int, _vp, _sz, _vp]),
    "bitlinear_fwd_group_plan_host": (_int, [_vp, _int, _i64, _int, _int, _vp, _sz]),
    "bitlinear_fwd_group_plan_fuses": (_int, [_vp, _int, _i64, _int, _int]),
    "bitlinear_fwd_group": (_int, [_vp, _int, _int, _int, _vp]),
    "bitlinear_quant_group_workspace_bytes": (_sz, [_vp, _int]),
    "bitlinear_quant_group_plan_bytes": (_sz, [_vp, _int]),
    "bitlinear_quant_group_plan": (_int, [_vp, _int, _int, _int, _int, _vp, _sz, _vp, _sz, _vp]),
    "bitlinear_quant_group": (_int, [_vp, _int, _int, _int, _vp]),
    "bitlinear_latent_update": (_int, [_vp, _vp, _i64, ctypes.c_float, _vp, _vp]),
    "bitlinear_relu2_gate": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bitlinear_relu2_gate_bwd": (_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "bitlinear_status_string": (ctypes.c_char_p, [_int]),
    "bitlinear_last_error": (ctypes.c_char_p, []),
}


def header_functions():
    """Names of the functions include/bitlinear.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def lib():
    """Load libbitlinear.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m sparse_linear_layers_group_amd.build")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t, dtypes, numel, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _check(status, where):
    if status != BL_OK:
        detail = lib().bitlinear_last_error().decode() or lib().bitlinear_status_string(status).decode()
        raise BitLinearError(status, where, detail)


def bitlinear_status_string(status):
    return lib().bitlinear_status_string(int(status)).decode()


def bitlinear_last_error():
    return lib().bitlinear_last_error().decode()


def bitlinear_packed_bytes(n_out, k, n, m):
    return int(lib().bitlinear_packed_bytes(int(n_out), int(k), int(n), int(m)))


def bitlinear_workspace_bytes(n_out, k):
    return int(lib().bitlinear_workspace_bytes(int(n_out), int(k)))


def bitlinear_fwd_workspace_bytes(tokens, k, n_out):
    return int(lib().bitlinear_fwd_workspace_bytes(int(tokens), int(k), int(n_out)))


def bitlinear_quantize_mask(W, n_out, k, n, m, gamma_over, mask, wq, gamma, ws, ws_bytes=None,
                            stream=None):
    st = lib().bitlinear_quantize_mask(
        _ptr(W, _BF16, n_out * k, "W"), n_out, k, n, m, gamma_over,
        _ptr(mask, (torch.uint8,), n_out * (k // 8), "mask"),
        _ptr(wq, (torch.int8,), n_out * k, "wq", optional=True),
        _ptr(gamma, (torch.float64,), 1, "gamma"),
        _ptr(ws, (torch.uint8,), None, "ws"),
        ws.numel() if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_quantize_mask")


def bitlinear_pack(W, mask, gamma, n_out, k, n, m, packed, packed_bytes=None, stream=None):
    st = lib().bitlinear_pack(
        _ptr(W, _BF16, n_out * k, "W"), _ptr(mask, (torch.uint8,), n_out * (k // 8), "mask"),
        _ptr(gamma, (torch.float64,), 1, "gamma"), n_out, k, n, m,
        _ptr(packed, (torch.uint8,), None, "packed"),
        packed.numel() if packed_bytes is None else int(packed_bytes), _stream(stream))
    _check(st, "bitlinear_pack")


def bitlinear_fwd(X, tokens, k, packed, n_out, n, m, gamma, Y, xq, x_scale, acc=None, ws=None,
                  ws_bytes=None, stream=None):
    st = lib().bitlinear_fwd(
        _ptr(X, _BF16, tokens * k, "X"), tokens, k, _ptr(packed, (torch.uint8,), None, "packed"),
        n_out, n, m, _ptr(gamma, (torch.float64,), 1, "gamma"),
        _ptr(Y, (torch.float32,), tokens * n_out, "Y"), _ptr(xq, (torch.int8,), tokens * k, "xq"),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes),
        _stream(stream))
    _check(st, "bitlinear_fwd")


def bitlinear_fwd_bf16(X, tokens, k, packed, n_out, n, m, gamma, Y, xq, x_scale, acc=None, ws=None,
                       ws_bytes=None, stream=None):
    """bitlinear_fwd with bf16 Y (a bfloat16 tensor of tokens * n_out)."""
    st = lib().bitlinear_fwd_bf16(
        _ptr(X, _BF16, tokens * k, "X"), tokens, k, _ptr(packed, (torch.uint8,), None, "packed"),
        n_out, n, m, _ptr(gamma, (torch.float64,), 1, "gamma"),
        _ptr(Y, _BF16, tokens * n_out, "Y"), _ptr(xq, (torch.int8,), tokens * k, "xq"),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes),
        _stream(stream))
    _check(st, "bitlinear_fwd_bf16")


def bitlinear_fwd_noalloc(X, tokens, k, packed, n_out, n, m, gamma, Y, xq, x_scale, acc=None, stream=None):
    st = lib().bitlinear_fwd_noalloc(
        _ptr(X, _BF16, tokens * k, "X"), tokens, k, _ptr(packed, (torch.uint8,), None, "packed"),
        n_out, n, m, _ptr(gamma, (torch.float64,), 1, "gamma"),
        _ptr(Y, (torch.float32,), tokens * n_out, "Y"), _ptr(xq, (torch.int8,), tokens * k, "xq"),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True), _stream(stream))
    _check(st, "bitlinear_fwd_noalloc")


def bitlinear_sp24_packed_bytes(n_out, k):
    return int(lib().bitlinear_sp24_packed_bytes(int(n_out), int(k)))


def bitlinear_sp24_workspace_bytes(tokens, k, n_out):
    return int(lib().bitlinear_sp24_workspace_bytes(int(tokens), int(k), int(n_out)))


def bitlinear_pack_sp24(W, mask, gamma, n_out, k, packed, packed_bytes=None, stream=None):
    st = lib().bitlinear_pack_sp24(
        _ptr(W, _BF16, n_out * k, "W"), _ptr(mask, (torch.uint8,), n_out * (k // 8), "mask"),
        _ptr(gamma, (torch.float64,), 1, "gamma"), n_out, k, _ptr(packed, (torch.uint8,), None, "packed"),
        packed.numel() if packed_bytes is None else int(packed_bytes), _stream(stream))
    _check(st, "bitlinear_pack_sp24")


def bitlinear_contract_sp24(xq, x_scale, tokens, k, packed, n_out, gamma, Y, acc=None, ws=None, ws_bytes=None,
                            stream=None):
    st = lib().bitlinear_contract_sp24(
        _ptr(xq, (torch.int8,), tokens * k, "xq"), _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        tokens, k, _ptr(packed, (torch.uint8,), None, "packed"), n_out, _ptr(gamma, (torch.float64,), 1, "gamma"),
        _ptr(Y, (torch.float32,), tokens * n_out, "Y"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_contract_sp24")


def bitlinear_bwd_workspace_bytes(tokens, k, n_out):
    return int(lib().bitlinear_bwd_workspace_bytes(int(tokens), int(k), int(n_out)))


def bitlinear_bwd(dY, xq, x_scale, packed, gamma, tokens, k, n_out, n, m, dX, dW, ws=None,
                  ws_bytes=None, stream=None):
    st = lib().bitlinear_bwd(
        _ptr(dY, _BF16, tokens * n_out, "dY"), _ptr(xq, (torch.int8,), tokens * k, "xq", optional=True),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale", optional=True),
        _ptr(packed, (torch.uint8,), None, "packed", optional=True),
        _ptr(gamma, (torch.float64,), 1, "gamma", optional=True), tokens, k, n_out, n, m,
        _ptr(dX, (torch.float32,), tokens * k, "dX", optional=True),
        _ptr(dW, (torch.float32,), n_out * k, "dW", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes),
        _stream(stream))
    _check(st, "bitlinear_bwd")


class bitlinear_bwd_item(ctypes.Structure):
    """Mirror of the C struct bitlinear_bwd_item (device pointers as ints)."""
    _fields_ = [("dY", _vp), ("xq", _vp), ("x_scale", _vp), ("packed", _vp), ("gamma", _vp),
                ("dX", _vp), ("dW", _vp), ("k", _i64), ("n_out", _i64)]


def make_bwd_items(entries, tokens):
    """entries: dicts with tensors dY, xq, x_scale, packed, gamma, dX (or None),
    dW (or None) and ints k, n_out."""
    arr = (bitlinear_bwd_item * len(entries))()
    for i, e in enumerate(entries):
        k, n_out = int(e["k"]), int(e["n_out"])
        arr[i] = bitlinear_bwd_item(
            _ptr(e["dY"], _BF16, tokens * n_out, "dY"), _ptr(e.get("xq"), (torch.int8,), tokens * k, "xq", optional=True),
            _ptr(e.get("x_scale"), (torch.float32,), tokens, "x_scale", optional=True),
            _ptr(e.get("packed"), (torch.uint8,), None, "packed", optional=True),
            _ptr(e.get("gamma"), (torch.float64,), 1, "gamma", optional=True),
            _ptr(e.get("dX"), (torch.float32,), tokens * k, "dX", optional=True),
            _ptr(e.get("dW"), (torch.float32,), n_out * k, "dW", optional=True), k, n_out)
    return arr


def bitlinear_bwd_group_workspace_bytes(items, count, tokens):
    return int(lib().bitlinear_bwd_group_workspace_bytes(items, int(count), int(tokens)))


def bitlinear_bwd_group(items, count, tokens, n, m, ws=None, ws_bytes=None, stream=None):
    st = lib().bitlinear_bwd_group(items, int(count), int(tokens), n, m,
                                   _ptr(ws, (torch.uint8,), None, "ws", optional=True),
                                   (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes),
                                   _stream(stream))
    _check(st, "bitlinear_bwd_group")


BL_BWD_PREPARE = 1
BL_BWD_FINISH = 2


def bitlinear_bwd_group_phase(items, count, tokens, n, m, phase, ws=None, ws_bytes=None, stream=None):
    """One half of bitlinear_bwd_group: BL_BWD_PREPARE converts the codes and
    x_q into ws, BL_BWD_FINISH converts dY and runs the products."""
    st = lib().bitlinear_bwd_group_phase(items, int(count), int(tokens), n, m, int(phase),
                                         _ptr(ws, (torch.uint8,), None, "ws", optional=True),
                                         (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes),
                                         _stream(stream))
    _check(st, "bitlinear_bwd_group_phase")


def bitlinear_bwd_relu2_gate(dY, xq, x_scale, packed, gamma, tokens, k, n_out, n, m, G, U, dG, dU, dW=None,
                             ws=None, ws_bytes=None, stream=None):
    """The down projection's backward with the squared-ReLU gating backward
    fused into its dX epilogue: dG, dU (bfloat16, tokens * k) and dW."""
    st = lib().bitlinear_bwd_relu2_gate(
        _ptr(dY, _BF16, tokens * n_out, "dY"), _ptr(xq, (torch.int8,), tokens * k, "xq", optional=True),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale", optional=True),
        _ptr(packed, (torch.uint8,), None, "packed"), _ptr(gamma, (torch.float64,), 1, "gamma"),
        tokens, k, n_out, n, m, _ptr(G, (torch.float32,), tokens * k, "G"), _ptr(U, (torch.float32,), tokens * k, "U"),
        _ptr(dG, _BF16, tokens * k, "dG"), _ptr(dU, _BF16, tokens * k, "dU"),
        _ptr(dW, (torch.float32,), n_out * k, "dW", optional=True), _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_bwd_relu2_gate")


def bitlinear_bwd_tiles(tiles):
    """Fix the backward products' tiles (0: chosen per launch, 1: 128 x 128,
    2: 256 x 128, 3: 256 x 256)."""
    _check(lib().bitlinear_bwd_tiles(int(tiles)), "bitlinear_bwd_tiles")


def bitlinear_latent_update(W_master, dW, count, lr, W, stream=None):
    st = lib().bitlinear_latent_update(
        _ptr(W_master, (torch.float32,), count, "W_master"), _ptr(dW, (torch.float32,), count, "dW"),
        int(count), float(lr), _ptr(W, _BF16, count, "W"), _stream(stream))
    _check(st, "bitlinear_latent_update")


def bitlinear_relu2_gate(G, U, tokens, n, H, xq, x_scale, stream=None):
    st = lib().bitlinear_relu2_gate(
        _ptr(G, (torch.float32,), tokens * n, "G"), _ptr(U, (torch.float32,), tokens * n, "U"), tokens, n,
        _ptr(H, _BF16, tokens * n, "H", optional=True), _ptr(xq, (torch.int8,), tokens * n, "xq"),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale"), _stream(stream))
    _check(st, "bitlinear_relu2_gate")


def bitlinear_relu2_gate_bwd(dH, G, U, count, dG, dU, stream=None):
    st = lib().bitlinear_relu2_gate_bwd(
        _ptr(dH, (torch.float32,), count, "dH"), _ptr(G, (torch.float32,), count, "G"),
        _ptr(U, (torch.float32,), count, "U"), int(count), _ptr(dG, _BF16, count, "dG"),
        _ptr(dU, _BF16, count, "dU"), _stream(stream))
    _check(st, "bitlinear_relu2_gate_bwd")


def bitlinear_act_quant(X, tokens, k, xq, x_scale, stream=None):
    st = lib().bitlinear_act_quant(_ptr(X, _BF16, tokens * k, "X"), tokens, k,
                                   _ptr(xq, (torch.int8,), tokens * k, "xq"),
                                   _ptr(x_scale, (torch.float32,), tokens, "x_scale"), _stream(stream))
    _check(st, "bitlinear_act_quant")


def bitlinear_contract(xq, x_scale, tokens, k, packed, n_out, n, m, gamma, Y, acc=None, ws=None,
                       ws_bytes=None, stream=None):
    st = lib().bitlinear_contract(
        _ptr(xq, (torch.int8,), tokens * k, "xq"), _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        tokens, k, _ptr(packed, (torch.uint8,), None, "packed"), n_out, n, m,
        _ptr(gamma, (torch.float64,), 1, "gamma"), _ptr(Y, (torch.float32,), tokens * n_out, "Y"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_contract")


class bitlinear_contract_item(ctypes.Structure):
    """Mirror of the C struct bitlinear_contract_item (device pointers as ints)."""
    _fields_ = [("packed", _vp), ("gamma", _vp), ("Y", _vp), ("Y_bf16", _vp), ("n_out", _i64)]


def make_contract_items(entries, tokens):
    """entries: dicts with tensors packed, gamma, Y (float32) or Y_bf16
    (bfloat16), and int n_out."""
    arr = (bitlinear_contract_item * len(entries))()
    for i, e in enumerate(entries):
        n_out = int(e["n_out"])
        arr[i] = bitlinear_contract_item(
            _ptr(e["packed"], (torch.uint8,), None, "packed"), _ptr(e["gamma"], (torch.float64,), 1, "gamma"),
            _ptr(e.get("Y"), (torch.float32,), tokens * n_out, "Y", optional=True),
            _ptr(e.get("Y_bf16"), _BF16, tokens * n_out, "Y_bf16", optional=True), n_out)
    return arr


def bitlinear_contract_group_workspace_bytes(items, count, tokens, k):
    return int(lib().bitlinear_contract_group_workspace_bytes(items, int(count), int(tokens), int(k)))


def bitlinear_contract_group(items, count, xq, x_scale, tokens, k, n, m, ws=None, ws_bytes=None, stream=None):
    st = lib().bitlinear_contract_group(
        items, int(count), _ptr(xq, (torch.int8,), tokens * k, "xq"),
        _ptr(x_scale, (torch.float32,), tokens, "x_scale"), int(tokens), int(k), n, m,
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_contract_group")


def bitlinear_contract_bf16(xq, x_scale, tokens, k, packed, n_out, n, m, gamma, Y, acc=None, ws=None,
                            ws_bytes=None, stream=None):
    """bitlinear_contract with bf16 Y (a bfloat16 tensor of tokens * n_out)."""
    st = lib().bitlinear_contract_bf16(
        _ptr(xq, (torch.int8,), tokens * k, "xq"), _ptr(x_scale, (torch.float32,), tokens, "x_scale"),
        tokens, k, _ptr(packed, (torch.uint8,), None, "packed"), n_out, n, m,
        _ptr(gamma, (torch.float64,), 1, "gamma"), _ptr(Y, _BF16, tokens * n_out, "Y"),
        _ptr(acc, (torch.int32,), tokens * n_out, "acc", optional=True),
        _ptr(ws, (torch.uint8,), None, "ws", optional=True),
        (ws.numel() if ws is not None else 0) if ws_bytes is None else int(ws_bytes), _stream(stream))
    _check(st, "bitlinear_contract_bf16")


class bitlinear_fwd_item(ctypes.Structure):
    """Mirror of the C struct bitlinear_fwd_item (device pointers as ints)."""
    _fields_ = [("X", _vp), ("packed", _vp), ("gamma", _vp), ("Y", _vp), ("xq", _vp),
                ("x_scale", _vp), ("k", _i64), ("n_out", _i64)]


def make_fwd_items(entries, tokens):
    """entries: dicts with tensors X, packed, gamma, Y, xq, x_scale and ints k, n_out."""
    arr = (bitlinear_fwd_item * len(entries))()
    for i, e in enumerate(entries):
        k, n_out = int(e["k"]), int(e["n_out"])
        arr[i] = bitlinear_fwd_item(
            _ptr(e["X"], _BF16, tokens * k, "X"), _ptr(e["packed"], (torch.uint8,), None, "packed"),
            _ptr(e["gamma"], (torch.float64,), 1, "gamma"),
            _ptr(e["Y"], (torch.float32,), tokens * n_out, "Y"), _ptr(e["xq"], (torch.int8,), tokens * k, "xq"),
            _ptr(e["x_scale"], (torch.float32,), tokens, "x_scale"), k, n_out)
    return arr


def bitlinear_fwd_group_plan_bytes(items, count, tokens):
    return int(lib().bitlinear_fwd_group_plan_bytes(items, int(count), int(tokens)))


def bitlinear_fwd_group_plan(items, count, tokens, n, m, plan, plan_bytes=None, stream=None):
    st = lib().bitlinear_fwd_group_plan(items, int(count), int(tokens), n, m,
                                        _ptr(plan, (torch.uint8,), None, "plan"),
                                        plan.numel() if plan_bytes is None else int(plan_bytes),
                                        _stream(stream))
    _check(st, "bitlinear_fwd_group_plan")


def bitlinear_fwd_group_plan_host(items, count, tokens, n, m, image):
    """The plan image into a host numpy uint8 array (no device call)."""
    if not (isinstance(image, np.ndarray) and image.dtype == np.uint8 and image.flags["C_CONTIGUOUS"]):
        raise TypeError("image must be a C-contiguous numpy uint8 array")
    st = lib().bitlinear_fwd_group_plan_host(items, int(count), int(tokens), n, m,
                                             image.ctypes.data_as(ctypes.c_void_p), image.nbytes)
    _check(st, "bitlinear_fwd_group_plan_host")


def bitlinear_fwd_group_plan_fuses(items, count, tokens, n, m):
    """True when the plan for these items can run stage 4 (one launch)."""
    st = lib().bitlinear_fwd_group_plan_fuses(items, int(count), int(tokens), n, m)
    if st < 0:
        _check(-st, "bitlinear_fwd_group_plan_fuses")
    return st == 1


def bitlinear_fwd_group(plan, n, m, stages=3, stream=None):
    st = lib().bitlinear_fwd_group(_ptr(plan, (torch.uint8,), None, "plan"), n, m, int(stages),
                                   _stream(stream))
    _check(st, "bitlinear_fwd_group")


class bitlinear_quant_item(ctypes.Structure):
    """Mirror of the C struct bitlinear_quant_item (device pointers as ints)."""
    _fields_ = [("W", _vp), ("mask", _vp), ("gamma", _vp), ("packed", _vp), ("n_out", _i64), ("k", _i64)]


def make_quant_items(entries, n, m):
    """entries: dicts with tensors W, mask, gamma, packed and ints n_out, k."""
    arr = (bitlinear_quant_item * len(entries))()
    for i, e in enumerate(entries):
        n_out, k = int(e["n_out"]), int(e["k"])
        arr[i] = bitlinear_quant_item(
            _ptr(e["W"], _BF16, n_out * k, "W"), _ptr(e["mask"], (torch.uint8,), n_out * (k // 8), "mask"),
            _ptr(e["gamma"], (torch.float64,), 1, "gamma"),
            _ptr(e["packed"], (torch.uint8,), bitlinear_packed_bytes(n_out, k, n, m), "packed"), n_out, k)
    return arr


def bitlinear_quant_group_workspace_bytes(items, count):
    return int(lib().bitlinear_quant_group_workspace_bytes(items, int(count)))


def bitlinear_quant_group_plan_bytes(items, count):
    return int(lib().bitlinear_quant_group_plan_bytes(items, int(count)))


def bitlinear_quant_group_plan(items, count, n, m, gamma_over, ws, plan, ws_bytes=None, plan_bytes=None,
                               stream=None):
    st = lib().bitlinear_quant_group_plan(
        items, int(count), n, m, gamma_over, _ptr(ws, (torch.uint8,), None, "ws"),
        ws.numel() if ws_bytes is None else int(ws_bytes), _ptr(plan, (torch.uint8,), None, "plan"),
        plan.numel() if plan_bytes is None else int(plan_bytes), _stream(stream))
    _check(st, "bitlinear_quant_group_plan")


def bitlinear_quant_group(plan, n, m, gamma_over, stream=None):
    st = lib().bitlinear_quant_group(_ptr(plan, (torch.uint8,), None, "plan"), n, m, gamma_over,
                                     _stream(stream))
    _check(st, "bitlinear_quant_group")
