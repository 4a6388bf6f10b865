"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/bitlinear.h declares, computes sizes like the format
definition, and rejects bad arguments before enqueueing anything."""
import ctypes
import os

import pytest

import oracle
from sparse_linear_layers_group_amd import bitlinear as bl


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bl.LIB_PATH):
        from sparse_linear_layers_group_amd import build
        build.build()
    return bl.lib()


def test_exports_every_declared_function(L):
    names = bl.header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), f"{name} declared in bitlinear.h but not exported"


@pytest.mark.parametrize("n,m", [(8, 8), (6, 8), (4, 8), (2, 4), (3, 8), (2, 8)])
@pytest.mark.parametrize("n_out,k", [(128, 256), (896, 896), (40, 384), (11008, 2048), (1, 128)])
def test_packed_bytes_matches_format_definition(L, n, m, n_out, k):
    assert bl.bitlinear_packed_bytes(n_out, k, n, m) == oracle.packed_bytes(n_out, k, oracle.s_of(n, m))


def test_packed_bytes_rejects(L):
    assert bl.bitlinear_packed_bytes(128, 100, 6, 8) == 0
    assert bl.bitlinear_packed_bytes(0, 256, 6, 8) == 0
    assert bl.bitlinear_packed_bytes(128, 256, 5, 8) == 0
    assert bl.bitlinear_packed_bytes(1 << 20, 1 << 12, 6, 8) == 0  # n_out*k >= 2^31


def test_tiny_config_packed_size(L):
    # [128 x 256] at 6:8: 8 row tiles x 16 rows x 2 blocks x 28 bytes
    assert bl.bitlinear_packed_bytes(128, 256, 6, 8) == 7168


A = 4096  # an aligned, never dereferenced address


def call_qm(L, **kw):
    a = dict(W=A, n_out=128, k=256, n=6, m=8, go=0, mask=A, wq=None, gamma=A, ws=A,
             ws_bytes=bl.bitlinear_workspace_bytes(128, 256))
    a.update(kw)
    return L.bitlinear_quantize_mask(a["W"], a["n_out"], a["k"], a["n"], a["m"], a["go"], a["mask"],
                                     a["wq"], a["gamma"], a["ws"], a["ws_bytes"], None)


def test_quantize_mask_validation(L):
    assert call_qm(L, n=5) == bl.BL_EUNSUPPORTED
    assert "5:8" in bl.bitlinear_last_error()
    assert call_qm(L, m=16, n=8) == bl.BL_EUNSUPPORTED
    assert call_qm(L, k=100) == bl.BL_ESHAPE
    assert call_qm(L, k=0) == bl.BL_ESHAPE
    assert call_qm(L, n_out=0) == bl.BL_ESHAPE
    assert call_qm(L, W=None) == bl.BL_EINVAL
    assert call_qm(L, W=A + 2) == bl.BL_EINVAL
    assert call_qm(L, mask=None) == bl.BL_EINVAL
    assert call_qm(L, wq=A + 1) == bl.BL_EINVAL
    assert call_qm(L, gamma=A + 4) == bl.BL_EINVAL
    assert call_qm(L, go=2) == bl.BL_EINVAL
    assert call_qm(L, ws=None) == bl.BL_EWORKSPACE
    assert call_qm(L, ws_bytes=8) == bl.BL_EWORKSPACE


def test_pack_validation(L):
    nb = bl.bitlinear_packed_bytes(128, 256, 6, 8)
    assert L.bitlinear_pack(A, A, A, 128, 256, 6, 8, A, nb - 4, None) == bl.BL_ESHAPE
    assert L.bitlinear_pack(A, A, A, 128, 256, 6, 8, None, nb, None) == bl.BL_EINVAL
    assert L.bitlinear_pack(A, A, A, 128, 256, 5, 8, A, nb, None) == bl.BL_EUNSUPPORTED


def test_fwd_validation(L):
    f = L.bitlinear_fwd
    assert f(A, -1, 256, A, 128, 6, 8, A, A, A, A, None, A, 1 << 20, None) == bl.BL_ESHAPE
    assert f(A, 4, 250, A, 128, 6, 8, A, A, A, A, None, A, 1 << 20, None) == bl.BL_ESHAPE
    assert f(None, 4, 256, A, 128, 6, 8, A, A, A, A, None, A, 1 << 20, None) == bl.BL_EINVAL
    assert f(A, 4, 256, A, 128, 6, 8, A, A, None, A, None, A, 1 << 20, None) == bl.BL_EINVAL
    assert f(A, 4, 256, A, 128, 6, 8, A, A, A, A, A + 8, A, 1 << 20, None) == bl.BL_EINVAL
    need = bl.bitlinear_fwd_workspace_bytes(4, 256, 128)
    if need:
        assert f(A, 4, 256, A, 128, 6, 8, A, A, A, A, None, None, 0, None) == bl.BL_EWORKSPACE
    # zero tokens is a valid no-op that touches nothing
    assert f(None, 0, 256, None, 128, 6, 8, None, None, None, None, None, None, 0, None) == bl.BL_OK


def test_bwd_validation(L):
    b = L.bitlinear_bwd
    assert b(A, A, A, A, A, 4, 256, 120, 6, 8, A, A, None, 0, None) == bl.BL_ESHAPE  # n_out % 16
    assert b(A, A, A, A, A, 4, 256, 128, 6, 8, A + 4, None, None, 0, None) == bl.BL_EINVAL
    need = bl.bitlinear_bwd_workspace_bytes(4, 256, 128)
    assert need == L.bitlinear_bwd_workspace_bytes(4, 256, 128) > 0
    assert bl.bitlinear_bwd_workspace_bytes(4, 256, 120) == 0  # n_out % 16
    assert b(A, A, A, A, A, 4, 256, 128, 6, 8, A, None, None, 0, None) == bl.BL_EWORKSPACE
    assert b(A, A, A, A, A, 4, 256, 128, 6, 8, A, None, A, need - 1, None) == bl.BL_EWORKSPACE
    assert b(None, A, A, A, A, 4, 256, 128, 6, 8, A, None, A, need, None) == bl.BL_EINVAL
    assert b(A, A, A, A, A, 4, 256, 128, 6, 8, None, None, None, 0, None) == bl.BL_OK  # nothing asked


def test_bwd_checks_every_input_before_the_first_launch(L):
    """With dX and dW both requested, a bad input of dW (NULL or misaligned
    x_q or x_scale) is reported before the dX kernels are queued: on a host
    without a GPU a launch would have returned BL_EHIP instead."""
    b = L.bitlinear_bwd
    need = bl.bitlinear_bwd_workspace_bytes(4, 256, 128)
    assert b(A, None, A, A, A, 4, 256, 128, 6, 8, A, A, A, need, None) == bl.BL_EINVAL
    assert "xq" in bl.bitlinear_last_error()
    assert b(A, A, A + 2, A, A, 4, 256, 128, 6, 8, A, A, A, need, None) == bl.BL_EINVAL
    assert "x_scale" in bl.bitlinear_last_error()
    assert b(A, A, A, None, A, 4, 256, 128, 6, 8, A, A, A, need, None) == bl.BL_EINVAL
    assert b(A, A, A, A, A + 4, 4, 256, 128, 6, 8, A, A, A, need, None) == bl.BL_EINVAL


def test_unsupported_pattern_message_lists_every_pattern(L):
    assert call_qm(L, n=5) == bl.BL_EUNSUPPORTED
    msg = bl.bitlinear_last_error()
    for p in ("8:8", "6:8", "4:8", "3:8", "2:8", "2:4"):
        assert p in msg


def test_fwd_noalloc_validation(L):
    """The allocation-free forward validates like bitlinear_fwd and rejects a
    forward whose workspace exceeds its static scratch before touching any
    device state."""
    f = L.bitlinear_fwd_noalloc
    assert f(A, 4, 250, A, 128, 6, 8, A, A, A, A, None, None) == bl.BL_ESHAPE
    assert f(A, 4, 256, A, 128, 5, 8, A, A, A, A, None, None) == bl.BL_EUNSUPPORTED
    assert f(None, 0, 256, None, 128, 6, 8, None, None, None, None, None, None) == bl.BL_OK
    assert bl.bitlinear_fwd_workspace_bytes(1024, 1024, 1536) > 8 << 20
    assert f(A, 1024, 1024, A, 1536, 6, 8, A, A, A, A, None, None) == bl.BL_EWORKSPACE
    assert "static scratch" in bl.bitlinear_last_error()


@pytest.mark.parametrize("n_out,k", [(128, 256), (40, 384), (11008, 2048), (1, 128)])
def test_sp24_sizes_match_layout_definition(L, n_out, k):
    assert bl.bitlinear_sp24_packed_bytes(n_out, k) == oracle.sp24_packed_bytes(n_out, k)


def test_sp24_validation(L):
    assert bl.bitlinear_sp24_packed_bytes(128, 100) == 0
    nb = bl.bitlinear_sp24_packed_bytes(128, 256)
    p = L.bitlinear_pack_sp24
    assert p(A, A, A, 128, 256, A, nb - 16, None) == bl.BL_ESHAPE
    assert p(A, None, A, 128, 256, A, nb, None) == bl.BL_EINVAL
    assert p(A, A, A, 128, 250, A, nb, None) == bl.BL_ESHAPE
    c = L.bitlinear_contract_sp24
    assert c(A, A, 4, 250, A, 128, A, A, None, None, 0, None) == bl.BL_ESHAPE
    assert c(None, A, 4, 256, A, 128, A, A, None, None, 0, None) == bl.BL_EINVAL
    assert c(None, None, 0, 256, None, 128, None, None, None, None, 0, None) == bl.BL_OK
    need = bl.bitlinear_sp24_workspace_bytes(512, 1024, 1536)
    assert need > 0
    assert c(A, A, 512, 1024, A, 1536, A, A, None, None, 0, None) == bl.BL_EWORKSPACE


def test_status_strings(L):
    for s in range(6):
        assert bl.bitlinear_status_string(s)
    assert bl.bitlinear_status_string(99) == "unknown status"


def test_launch_without_device_reports_hip_error(L):
    """On a host without a GPU a fully valid call reaches the launch and
    returns BL_EHIP with the runtime's message, instead of crashing."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present: fake pointers must not reach a real launch")
    except ImportError:
        pass
    nb = bl.bitlinear_packed_bytes(128, 256, 6, 8)
    st = L.bitlinear_pack(A, A, A, 128, 256, 6, 8, A, nb, None)
    assert st == bl.BL_EHIP
    assert bl.bitlinear_last_error()


def _qitems(shapes, over=None):
    arr = (bl.bitlinear_quant_item * len(shapes))()
    for i, (n_out, k) in enumerate(shapes):
        f = dict(W=A, mask=A, gamma=A, packed=A, n_out=n_out, k=k)
        f.update((over or {}).get(i, {}))
        arr[i] = bl.bitlinear_quant_item(f["W"], f["mask"], f["gamma"], f["packed"], f["n_out"], f["k"])
    return arr


def test_quant_group_sizes(L):
    """The grouped workspace is one 256-byte aligned region per item, each at
    least the single call's workspace; bad shapes give 0."""
    shapes = [(896, 896), (128, 896), (4864, 896), (896, 4864)]
    items = _qitems(shapes)
    ws = bl.bitlinear_quant_group_workspace_bytes(items, len(shapes))
    single = [bl.bitlinear_workspace_bytes(n_out, k) for n_out, k in shapes]
    assert ws == sum((s + 255) // 256 * 256 for s in single)
    plan = bl.bitlinear_quant_group_plan_bytes(items, len(shapes))
    assert plan > 64 + 128 * len(shapes)
    assert bl.bitlinear_quant_group_workspace_bytes(_qitems([(128, 100)]), 1) == 0
    assert bl.bitlinear_quant_group_plan_bytes(items, 0) == 0
    assert bl.bitlinear_quant_group_plan_bytes(None, 1) == 0


def test_quant_group_validation(L):
    shapes = [(128, 256), (256, 128)]
    items = _qitems(shapes)
    ws = bl.bitlinear_quant_group_workspace_bytes(items, 2)
    pb = bl.bitlinear_quant_group_plan_bytes(items, 2)
    f = L.bitlinear_quant_group_plan
    assert f(items, 2, 5, 8, 0, A, ws, A, pb, None) == bl.BL_EUNSUPPORTED
    assert f(items, 2, 6, 8, 2, A, ws, A, pb, None) == bl.BL_EINVAL
    assert f(items, 0, 6, 8, 0, A, ws, A, pb, None) == bl.BL_ESHAPE
    assert f(None, 2, 6, 8, 0, A, ws, A, pb, None) == bl.BL_EINVAL
    assert f(_qitems([(128, 256), (128, 100)]), 2, 6, 8, 0, A, ws, A, pb, None) == bl.BL_ESHAPE
    assert "item 1" in bl.bitlinear_last_error()
    assert f(_qitems(shapes, {1: dict(W=A + 2)}), 2, 6, 8, 0, A, ws, A, pb, None) == bl.BL_EINVAL
    assert f(_qitems(shapes, {0: dict(packed=None)}), 2, 6, 8, 0, A, ws, A, pb, None) == bl.BL_EINVAL
    assert f(_qitems(shapes, {0: dict(gamma=A + 4)}), 2, 6, 8, 0, A, ws, A, pb, None) == bl.BL_EINVAL
    assert f(items, 2, 6, 8, 0, A, ws - 1, A, pb, None) == bl.BL_EWORKSPACE
    assert f(items, 2, 6, 8, 0, None, ws, A, pb, None) == bl.BL_EWORKSPACE
    assert f(items, 2, 6, 8, 0, A, ws, A, pb - 1, None) == bl.BL_EWORKSPACE
    assert f(items, 2, 6, 8, 0, A, ws, None, pb, None) == bl.BL_EINVAL
    g = L.bitlinear_quant_group
    assert g(A, 6, 8, 3, None) == bl.BL_EINVAL
    assert g(None, 6, 8, 0, None) == bl.BL_EINVAL
    assert g(A, 7, 8, 0, None) == bl.BL_EUNSUPPORTED


def test_latent_update_validation(L):
    f = L.bitlinear_latent_update
    assert f(A, A, 12, 0.1, A, None) == bl.BL_ESHAPE   # not a multiple of 8
    assert f(A, A, -8, 0.1, A, None) == bl.BL_ESHAPE
    assert f(None, A, 16, 0.1, A, None) == bl.BL_EINVAL
    assert f(A, A + 4, 16, 0.1, A, None) == bl.BL_EINVAL
    assert f(A, A, 16, 0.1, None, None) == bl.BL_EINVAL
    assert f(None, None, 0, 0.1, None, None) == bl.BL_OK  # no-op


def test_relu2_gate_validation(L):
    f = L.bitlinear_relu2_gate
    assert f(A, A, 4, 100, None, A, A, None) == bl.BL_ESHAPE   # n % 128
    assert f(A, A, -1, 256, None, A, A, None) == bl.BL_ESHAPE
    assert f(None, A, 4, 256, None, A, A, None) == bl.BL_EINVAL
    assert f(A, A, 4, 256, A + 2, A, A, None) == bl.BL_EINVAL  # misaligned H
    assert f(A, A, 4, 256, None, A, A + 2, None) == bl.BL_EINVAL
    assert f(None, None, 0, 256, None, None, None, None) == bl.BL_OK
    b = L.bitlinear_relu2_gate_bwd
    assert b(A, A, A, 12, A, A, None) == bl.BL_ESHAPE
    assert b(A, A, A, 16, None, A, None) == bl.BL_EINVAL
    assert b(None, None, None, 0, None, None, None) == bl.BL_OK


def test_bf16_outputs_reject_null_y(L):
    """The bf16-output calls check Y first, with every other pointer valid-looking."""
    fake = ctypes.c_void_p(1 << 20)
    st = L.bitlinear_contract_bf16(fake, fake, 1, 128, fake, 64, 6, 8, fake, None, None, None, 0, None)
    assert st == bl.BL_EINVAL
    st = L.bitlinear_fwd_bf16(fake, 1, 128, fake, 64, 6, 8, fake, None, fake, fake, None, None, 0, None)
    assert st == bl.BL_EINVAL


def test_group_stages_validated(L):
    fake = ctypes.c_void_p(1 << 20)
    for stages in (0, 5, -1):
        assert L.bitlinear_fwd_group(fake, 6, 8, stages, None) == bl.BL_EINVAL


def _bwd_items(specs):
    """specs: (k, n_out, dX?, dW?) with stand-in aligned device addresses."""
    arr = (bl.bitlinear_bwd_item * len(specs))()
    for i, (k, n_out, want_dx, want_dw) in enumerate(specs):
        arr[i] = bl.bitlinear_bwd_item(A, A, A, A, A, A if want_dx else None, A if want_dw else None, k, n_out)
    return arr


def test_bwd_group_sizes(L):
    """The grouped workspace is the sum of every item's operand region (no
    split partials), and 0 for an invalid item."""
    items = _bwd_items([(256, 128, True, True), (2560, 640, True, True), (384, 272, False, True)])
    total = bl.bitlinear_bwd_group_workspace_bytes(items, 3, 300)
    parts = [bl.bitlinear_bwd_group_workspace_bytes(_bwd_items([s]), 1, 300)
             for s in [(256, 128, True, True), (2560, 640, True, True), (384, 272, False, True)]]
    assert total == sum(parts) > 0
    assert all(p % 256 == 0 and p <= bl.bitlinear_bwd_workspace_bytes(300, k, n)
               for p, (k, n, _, _) in zip(parts, [(256, 128, 0, 0), (2560, 640, 0, 0), (384, 272, 0, 0)]))
    assert bl.bitlinear_bwd_group_workspace_bytes(_bwd_items([(256, 120, True, True)]), 1, 4) == 0
    assert bl.bitlinear_bwd_group_workspace_bytes(items, 0, 4) == 0


def test_bwd_group_validation(L):
    """Every item is checked before anything is enqueued (on a host without
    a GPU a launch would have returned BL_EHIP), and the error names the
    item."""
    g = L.bitlinear_bwd_group
    good = _bwd_items([(256, 128, True, True), (384, 272, True, True)])
    need = bl.bitlinear_bwd_group_workspace_bytes(good, 2, 4)
    assert g(None, 1, 4, 6, 8, A, need, None) == bl.BL_EINVAL
    assert g(good, 0, 4, 6, 8, A, need, None) == bl.BL_ESHAPE
    assert g(good, 2, -1, 6, 8, A, need, None) == bl.BL_ESHAPE
    assert g(good, 2, 4, 5, 8, A, need, None) == bl.BL_EUNSUPPORTED
    assert g(good, 2, 4, 6, 8, A, need - 1, None) == bl.BL_EWORKSPACE
    assert g(good, 2, 4, 6, 8, None, 0, None) == bl.BL_EWORKSPACE
    assert g(good, 2, 4, 6, 8, A + 16, need, None) == bl.BL_EINVAL  # ws alignment
    bad = _bwd_items([(256, 128, True, True), (384, 120, True, True)])  # n_out % 16
    assert g(bad, 2, 4, 6, 8, A, need, None) == bl.BL_ESHAPE
    assert "item 1" in bl.bitlinear_last_error()
    bad = _bwd_items([(256, 128, True, True), (384, 272, False, True)])
    bad[1].xq = None  # dW needs x_q
    assert g(bad, 2, 4, 6, 8, A, need, None) == bl.BL_EINVAL
    assert "item 1" in bl.bitlinear_last_error() and "xq" in bl.bitlinear_last_error()
    bad = _bwd_items([(256, 128, True, True)])
    bad[0].packed = None  # dX needs the packed codes
    assert g(bad, 1, 4, 6, 8, A, need, None) == bl.BL_EINVAL
    none = _bwd_items([(256, 128, False, False)])
    assert g(none, 1, 4, 6, 8, None, 0, None) == bl.BL_OK  # nothing asked: nothing runs


def _contract_items(specs):
    """specs: (n_out, Y?, Y_bf16?) with stand-in aligned device addresses."""
    arr = (bl.bitlinear_contract_item * len(specs))()
    for i, (n_out, y, yb) in enumerate(specs):
        arr[i] = bl.bitlinear_contract_item(A, A, A if y else None, A if yb else None, n_out)
    return arr


def test_contract_group_sizes(L):
    """No workspace above 16 tokens; at most 16 tokens the largest of the
    items' decode workspaces (they run in turn on one); 0 for a bad shape."""
    items = _contract_items([(896, True, False), (128, True, False), (4864, False, True)])
    assert bl.bitlinear_contract_group_workspace_bytes(items, 3, 64, 896) == 0
    for tokens in (1, 16):
        want = max(bl.bitlinear_fwd_workspace_bytes(tokens, 896, n) for n in (896, 128, 4864))
        assert bl.bitlinear_contract_group_workspace_bytes(items, 3, tokens, 896) == want
    assert bl.bitlinear_contract_group_workspace_bytes(items, 3, 64, 100) == 0  # k % 128
    assert bl.bitlinear_contract_group_workspace_bytes(items, 0, 64, 896) == 0


def test_contract_group_validation(L):
    """Every item is checked before anything is enqueued, and the error
    names the item."""
    g = L.bitlinear_contract_group
    good = _contract_items([(896, True, False), (128, False, True)])
    assert g(None, 1, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_EINVAL
    assert g(good, 0, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_ESHAPE
    assert g(good, 2, A, A, 64, 896, 5, 8, None, 0, None) == bl.BL_EUNSUPPORTED
    assert g(good, 2, A, A, 64, 100, 6, 8, None, 0, None) == bl.BL_ESHAPE
    assert g(good, 2, A, A, -1, 896, 6, 8, None, 0, None) == bl.BL_ESHAPE
    both = _contract_items([(896, True, False), (128, True, True)])
    assert g(both, 2, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_EINVAL
    assert "item 1" in bl.bitlinear_last_error()
    neither = _contract_items([(896, False, False)])
    assert g(neither, 1, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_EINVAL
    bad = _contract_items([(896, True, False), (0, True, False)])
    assert g(bad, 2, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_ESHAPE
    assert "item 1" in bl.bitlinear_last_error()
    bad = _contract_items([(896, True, False)])
    bad[0].gamma = A + 4  # gamma needs 8-byte alignment
    assert g(bad, 1, A, A, 64, 896, 6, 8, None, 0, None) == bl.BL_EINVAL
    assert g(good, 2, None, A, 64, 896, 6, 8, None, 0, None) == bl.BL_EINVAL  # xq
    need = bl.bitlinear_contract_group_workspace_bytes(good, 2, 4, 896)
    assert need > 0
    assert g(good, 2, A, A, 4, 896, 6, 8, None, 0, None) == bl.BL_EWORKSPACE
    assert g(good, 2, A, A, 0, 896, 6, 8, None, 0, None) == bl.BL_OK  # no tokens: nothing runs


def test_bwd_group_phase_validation(L):
    """The phased grouped backward takes BL_BWD_PREPARE, BL_BWD_FINISH or both,
    validates like the one-call form, and with no tokens the preparing half
    enqueues nothing."""
    g = L.bitlinear_bwd_group_phase
    good = _bwd_items([(256, 128, True, True), (384, 272, True, True)])
    need = bl.bitlinear_bwd_group_workspace_bytes(good, 2, 4)
    for phase in (0, 4, -1):
        assert g(good, 2, 4, 6, 8, phase, A, need, None) == bl.BL_EINVAL
        assert "phase" in bl.bitlinear_last_error()
    for phase in (bl.BL_BWD_PREPARE, bl.BL_BWD_FINISH, bl.BL_BWD_PREPARE | bl.BL_BWD_FINISH):
        assert g(good, 2, 4, 6, 8, phase, A, need - 1, None) == bl.BL_EWORKSPACE
        assert g(good, 2, 4, 5, 8, phase, A, need, None) == bl.BL_EUNSUPPORTED
        bad = _bwd_items([(256, 128, True, True), (384, 120, True, True)])
        assert g(bad, 2, 4, 6, 8, phase, A, need, None) == bl.BL_ESHAPE
        assert "item 1" in bl.bitlinear_last_error()
    assert g(good, 2, 0, 6, 8, bl.BL_BWD_PREPARE, None, 0, None) == bl.BL_OK
