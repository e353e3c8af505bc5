"""C ABI checks that need no GPU: the library loads, exports every function
include/haste.h declares, and rejects bad arguments on the host before any
HIP call (so these run on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

from group_shared_fixed_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "haste.h")

OK, NULL, DIM, UNSUP, ALIGN, WS = 0, -1, -2, -3, -4, -5
P = ctypes.c_void_p
A = P(0x100000)          # 16-byte aligned fake device pointer (never dereferenced)
MIS = P(0x100008)        # misaligned fake pointer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(haste_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hb.LIB_PATH):
        pytest.fail("libhaste.so is not built (run __graft_entry__.build())")
    return hb.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), f"libhaste.so does not export {n}"
        assert n in hb.SIGNATURES, f"binding has no signature for {n}"


def test_version_and_status_strings(L):
    assert b"gfx950" in L.haste_version()
    for code in range(-7, 1):
        assert L.haste_status_string(code)
    assert L.haste_status_string(5) == b"unknown status"


def test_workspace_size(L):
    # feature-major copy of h: H * round_up(B, 32) * 2 bytes, 256-aligned
    assert L.haste_workspace_size(0, 128, 768, 93748, 32, 64, 0) == 768 * 128 * 2
    assert L.haste_workspace_size(0, 100, 768, 10, 32, 64, 0) == 768 * 128 * 2
    # atomic dh: only the 256-byte status word
    assert L.haste_workspace_size(2, 128, 768, 10, 32, 64, 0) == 256
    # deterministic dh: status word, one hand-off flag per workgroup, the partials
    # (32-row tiles at G = 32, F = 64: 4 batch tiles x 64 label chunks)
    det = L.haste_workspace_size(2, 128, 768, 10, 32, 64, 1)
    assert det == 256 + 1024 + 64 * 4 * 32 * 768 * 4
    assert L.haste_workspace_size(4, 128, 768, 10, 32, 64, 1) == 768 * 128 * 2 + det
    assert L.haste_workspace_size(4, 128, 768, 10, 32, 64, 0) == 256 + 768 * 128 * 2
    # the G = 1 baseline's feature gradient has no turn waits, so no status word
    assert L.haste_workspace_size(7, 128, 768, 10, 1, 64, 0) == 0
    assert L.haste_workspace_size(99, 128, 768, 10, 32, 64, 0) == 0


def test_section_interface_names(L):
    """haste_bwd_h_workspace_size and the fused pass's workspace op."""
    for mode in (0, 1):
        for (B, H, K, G, F) in ((128, 768, 93748, 32, 64), (256, 768, 41888, 16, 128), (50, 1024, 9, 64, 32)):
            assert L.haste_bwd_h_workspace_size(B, H, K, G, F, mode) == L.haste_workspace_size(2, B, H, K, G, F, mode)
            assert L.haste_workspace_size(8, B, H, K, G, F, mode) == L.haste_workspace_size(4, B, H, K, G, F, mode) + 256


def _fbb(L, h=A, idx=A, W=A, rp=A, col=A, scale=0.5, dW=A, dh=A, loss=A, mode=1, ws=A, wsb=1 << 30,
         B=128, H=768, K=100, G=32, F=64):
    return L.haste_fwd_bce_bwd(h, idx, W, rp, col, scale, dW, dh, loss, mode, ws, wsb, B, H, K, G, F, None)


def test_fwd_bce_bwd_rejects(L):
    assert _fbb(L, h=None) == NULL
    assert _fbb(L, W=None) == NULL
    assert _fbb(L, dW=None) == NULL
    assert _fbb(L, dh=None) == NULL
    assert _fbb(L, rp=None) == NULL
    assert _fbb(L, B=0) == DIM
    assert _fbb(L, scale=0.0) == DIM
    assert _fbb(L, G=8) == UNSUP
    assert _fbb(L, B=257) == UNSUP                   # label cursors cover 256 rows
    assert _fbb(L, mode=2) == UNSUP
    assert _fbb(L, loss=MIS) == ALIGN
    assert _fbb(L, dW=MIS) == ALIGN
    assert _fbb(L, ws=None) == WS
    need = L.haste_workspace_size(8, 128, 768, 100, 32, 64, 1)
    assert _fbb(L, wsb=need - 256) == WS              # the fp64 loss accumulator is missing
    assert _fbb(L, ws=P(0x100010)) == WS


def _sbf(L, h=A, idx=A, W=A, rp=A, col=A, scale=0.5, dW=A, dh=A, loss=None, mode=1, ws=A, wsb=1 << 30,
         B=128, H=768, K=100, G=32, F=64):
    return L.haste_step_bf16dw(h, idx, W, rp, col, scale, dW, dh, loss, B, H, K, G, F, mode, ws, wsb, None, None)


def test_step_bf16dw_rejects(L):
    assert _sbf(L, W=None) == NULL
    assert _sbf(L, dW=None) == NULL
    assert _sbf(L, dh=None) == NULL
    assert _sbf(L, h=None) == NULL
    assert _sbf(L, B=0) == DIM
    assert _sbf(L, scale=-1.0) == DIM
    assert _sbf(L, G=8) == UNSUP
    assert _sbf(L, F=48) == UNSUP
    assert _sbf(L, mode=2) == UNSUP
    assert _sbf(L, dW=MIS) == ALIGN
    assert _sbf(L, ws=None) == WS
    need = L.haste_workspace_size(4, 128, 768, 100, 32, 64, 1)
    assert _sbf(L, wsb=need - 256) == WS


def test_hT_offsets_stay_32_bit(L):
    """Shapes whose feature-major copy of h would pass 2^31 bytes (32-bit
    gather offsets) or need more than 65535 transpose workgroups are refused."""
    assert _fwd(L, B=1 << 20, H=1024) == UNSUP                   # exactly 2^31 bytes
    assert _fwd(L, B=(1 << 21) + 32, H=64, F=64) == UNSUP        # Bp / 32 > 65535
    assert L.haste_bwd_w(A, A, A, A, 1 << 20, 1024, 100, 32, 64, A, 1 << 40, None) == UNSUP


def test_label_emb_rejects(L):
    def acc(h=A, rp=A, col=A, nnz=10, B=4, H=64, Lb=100, S=A, n=A, ws=A, wsb=1 << 30):
        return L.haste_label_emb_accumulate(h, rp, col, nnz, B, H, Lb, S, n, ws, wsb, None)
    assert acc(h=None) == NULL
    assert acc(col=None) == NULL
    assert acc(S=None) == NULL
    assert acc(B=0) == DIM
    assert acc(nnz=-1) == DIM
    assert acc(H=60) == UNSUP                      # H % 8
    assert acc(H=2048) == UNSUP
    assert acc(S=MIS) == ALIGN
    assert acc(ws=None) == WS
    assert acc(wsb=16) == WS
    assert L.haste_label_emb_workspace_size(5000) == 8192 * 8 + 20224
    assert L.haste_label_emb_finalize(None, A, 10, 64, A, None) == NULL
    assert L.haste_label_emb_finalize(A, A, 10, 12, A, None) == UNSUP
    assert L.haste_label_emb_finalize(A, A, 0, 64, A, None) == DIM
    assert L.haste_label_emb_finalize(A, A, 10, 64, MIS, None) == ALIGN


def test_workspace_status_rejects(L):
    out = ctypes.c_int32(0)
    assert L.haste_workspace_status(None, ctypes.byref(out), None) == NULL
    assert L.haste_workspace_status(P(0x100000), None, None) == NULL
    assert L.haste_workspace_status(P(0x100010), ctypes.byref(out), None) == WS


def _fwd(L, h=A, idx=A, W=A, Z=A, B=128, H=768, K=100, G=32, F=64, ws=A, wsb=1 << 30):
    return L.haste_fwd(h, idx, W, Z, B, H, K, G, F, ws, wsb, None)


def test_fwd_rejects(L):
    assert _fwd(L, h=None) == NULL
    assert _fwd(L, Z=None) == NULL
    assert _fwd(L, B=0) == DIM
    assert _fwd(L, K=-1) == DIM
    assert _fwd(L, F=64, H=32) == DIM                 # F distinct columns out of H
    assert _fwd(L, G=8) == UNSUP
    assert _fwd(L, G=1) == UNSUP                      # G = 1 is the haste_fixed_* path
    assert _fwd(L, F=48) == UNSUP
    assert _fwd(L, H=2048) == UNSUP
    assert _fwd(L, K=(1 << 31) // 32) == UNSUP        # L = K*G must fit int32 label ids
    assert _fwd(L, W=MIS) == ALIGN
    assert _fwd(L, Z=MIS) == ALIGN
    assert _fwd(L, ws=None) == WS
    assert _fwd(L, wsb=100) == WS
    assert _fwd(L, ws=P(0x100010)) == WS             # not 256-aligned


def test_bwd_rejects(L):
    assert L.haste_bwd_w(A, A, None, A, 128, 768, 10, 32, 64, A, 1 << 30, None) == NULL
    assert L.haste_bwd_w(A, A, A, A, 128, 768, 10, 32, 96, A, 1 << 30, None) == UNSUP
    assert L.haste_bwd_h(A, A, A, None, 128, 768, 10, 32, 64, 0, None, 0, None) == NULL
    assert L.haste_bwd_h(A, A, A, A, 128, 768, 10, 32, 64, 2, None, 0, None) == UNSUP   # bad mode
    assert L.haste_bwd_h(A, A, A, A, 128, 768, 10, 32, 64, 1, None, 0, None) == WS      # det needs ws
    assert L.haste_bwd_h(A, A, MIS, A, 128, 768, 10, 32, 64, 0, None, 0, None) == ALIGN


def test_label_paths_reject(L):
    f = L.haste_fwd_bce
    assert f(A, A, A, None, A, 1.0, A, None, None, 128, 768, 10, 32, 64, A, 1 << 30, None) == NULL
    assert f(A, A, A, A, A, 1.0, None, None, None, 128, 768, 10, 32, 64, A, 1 << 30, None) == NULL
    assert f(A, A, A, A, A, 1.0, A, None, None, 300, 768, 10, 32, 64, A, 1 << 30, None) == UNSUP   # B > 256
    assert f(A, A, A, A, A, 0.0, A, None, None, 128, 768, 10, 32, 64, A, 1 << 30, None) == DIM    # scale
    assert f(A, A, A, A, A, 1.0, A, MIS, None, 128, 768, 10, 32, 64, A, 1 << 30, None) == ALIGN   # Z
    s = L.haste_step
    assert s(A, A, A, A, A, 1.0, None, A, None, None, 128, 768, 10, 32, 64, 0, A, 1 << 30, None) == NULL
    assert s(A, A, A, A, A, 1.0, A, A, None, None, 128, 768, 10, 32, 64, 5, A, 1 << 30, None) == UNSUP
    assert s(A, A, A, A, A, 1.0, A, A, None, None, 128, 768, 10, 32, 64, 1, A, 1000, None) == WS


def test_fixed_rejects(L):
    assert L.haste_fixed_fwd(A, None, A, A, 128, 768, 1000, 64, A, 1 << 30, None) == NULL
    assert L.haste_fixed_fwd(A, A, A, A, 128, 768, 1000, 80, A, 1 << 30, None) == UNSUP
    assert L.haste_fixed_bwd_w(A, A, A, A, 128, 768, 0, 64, A, 1 << 30, None) == DIM
    assert L.haste_fixed_bwd_h(A, A, A, A, 128, 768, 1000, 64, 1, None, 0, None) == WS


def test_order_slots_rejects(L):
    assert L.haste_order_slots(None, A, A, 10, 32, 64, None) == NULL
    assert L.haste_order_slots(A, A, A, 0, 32, 64, None) == DIM
    assert L.haste_order_slots(A, A, A, 10, 0, 64, None) == DIM
    assert L.haste_order_slots(A, A, A, 10, 8, 64, None) == UNSUP
    assert L.haste_order_slots(A, A, A, 10, 32, 48, None) == UNSUP
    assert L.haste_order_slots(A, A, A, 10, 32, 256, None) == UNSUP
    assert L.haste_order_slots(A, A, A, (2**31) // 32, 32, 64, None) == UNSUP
    assert L.haste_order_slots(MIS, A, A, 10, 32, 64, None) == ALIGN
    assert L.haste_order_slots(A, MIS, None, 10, 32, 64, None) == ALIGN


def test_validate_rejects(L):
    assert L.haste_validate_idx(None, 10, 64, 768, A, None) == NULL
    assert L.haste_validate_idx(A, 0, 64, 768, A, None) == DIM
    assert L.haste_validate_labels(A, A, 0, 10, A, None) == DIM


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(hb.HasteError):
        hb.lib(str(tmp_path / "nope.so"))


def test_head_and_joint_reject(L):
    ws_h = L.haste_head_workspace_size(128, 768, 89088)
    assert ws_h > 128 * 89088 * 4 and ws_h % 256 == 0
    assert L.haste_head_workspace_size(0, 768, 10) == 0

    def head(h=A, W=A, rp=A, col=A, s=0.5, dW=A, dh=A, Z=None, loss=None, B=16, H=64, Lh=10, ws=A,
             wsb=1 << 30):
        return L.haste_head_step(h, W, rp, col, ctypes.c_float(s), dW, dh, Z, loss, B, H, Lh, ws, wsb, None)

    assert head(h=None) == NULL
    assert head(dh=None) == NULL
    assert head(B=0) == DIM
    assert head(s=0.0) == DIM
    assert head(W=MIS) == ALIGN
    assert head(ws=None) == WS
    assert head(wsb=16) == WS

    def joint(idx=A, Wt=A, st=0.5, sh=0.5, G=32, F=64, mode=0, wsb=1 << 30):
        return L.haste_joint_step(A, idx, Wt, A, A, A, A, A, ctypes.c_float(st), ctypes.c_float(sh), A, A, A, None,
                                  16, 768, 10, G, F, 100, mode, A, wsb, None)

    assert joint(idx=None) == NULL
    assert joint(st=0.0) == DIM
    assert joint(G=8) == UNSUP
    assert joint(mode=5) == UNSUP
    assert joint(Wt=MIS) == ALIGN
    assert joint(wsb=16) == WS


def test_rewire_rejects(L):
    B, H, K, G, F = 64, 256, 10, 32, 64
    need = L.haste_rewire_workspace_size(B, H, K, G, F)
    assert need == 256 * 64 * 2 + ((K * H * 4 + 255) // 256) * 256

    def rw(h=A, idx=A, idx_out=P(0x900000), W=A, W_out=P(0xA00000), n=4, B=B, H=H, G=G, F=F, ws=A,
           wsb=1 << 30):
        return L.haste_rewire(h, A, idx, W, n, idx_out, W_out, None, None, B, H, K, G, F, ws, wsb, None)

    assert rw(h=None) == NULL
    assert rw(n=-1) == DIM
    assert rw(n=F + 1) == DIM
    assert rw(B=257) == UNSUP
    assert rw(G=8) == UNSUP
    assert rw(W=MIS) == ALIGN
    assert rw(idx_out=P(0x100000 + 256)) == DIM    # overlaps idx without being idx
    assert rw(ws=None) == WS


def test_w8_reject(L):
    assert L.haste_quantize_w8(None, A, A, 10, 32, 64, None) == NULL
    assert L.haste_quantize_w8(A, A, A, 0, 32, 64, None) == DIM
    assert L.haste_quantize_w8(A, A, A, 10, 8, 64, None) == UNSUP
    assert L.haste_quantize_w8(A, MIS, A, 10, 32, 64, None) == ALIGN
    assert L.haste_fwd_w8(A, A, None, A, A, 128, 768, 10, 32, 64, A, 1 << 30, None) == NULL
    assert L.haste_fwd_w8(A, A, A, None, A, 128, 768, 10, 32, 64, A, 1 << 30, None) == NULL
    assert L.haste_fwd_w8(A, A, MIS, A, A, 128, 768, 10, 32, 64, A, 1 << 30, None) == ALIGN
    assert L.haste_step_w8(A, A, A, A, A, A, ctypes.c_float(0.5), A, A, None, None, 300, 768, 10, 32, 64, 0, A,
                           1 << 30, None) == UNSUP          # B above the label-driven limit
    assert L.haste_step_w8(A, A, None, A, A, A, ctypes.c_float(0.5), A, A, None, None, 128, 768, 10, 32, 64, 0, A,
                           1 << 30, None) == NULL


def test_grouping_reject(L):
    assert L.haste_kmeans_assign_workspace_size(0, 10, 64, 0) == 0
    assert L.haste_group_workspace_size(1000, 0) == 0
    assert L.haste_kmeans_assign(None, None, 100, 100, A, 10, 64, A, None, A, 1 << 30, None) == NULL
    assert L.haste_kmeans_assign(A, None, 50, 100, A, 10, 64, A, None, A, 1 << 30, None) == DIM   # rows NULL: n = L
    assert L.haste_kmeans_assign(A, None, 100, 100, A, 10, 60, A, None, A, 1 << 30, None) == UNSUP  # H % 8
    assert L.haste_kmeans_assign(A, None, 100, 100, A, 200, 64, A, None, A, 1 << 30, None) == UNSUP  # C > L
    assert L.haste_kmeans_assign(A, None, 100, 100, A, 10, 64, A, None, A, 16, None) == WS
    assert L.haste_kmeans_update(A, A, A, 0, 100, 10, 64, A, A, A, A, 1 << 30, None) == DIM
    assert L.haste_kmeans_update(A, A, A, 10, 100, 10, 64, MIS, A, A, A, 1 << 30, None) == ALIGN
    assert L.haste_kmeans_init(A, None, 100, 10, 64, A, A, A, None) == NULL
    assert L.haste_group_greedy(A, A, 100, 10, 64, 32, A, A, 1 << 30, None) == DIM      # L % G
    assert L.haste_group_greedy(A, A, 128, 10, 64, 128, A, A, 1 << 30, None) == DIM     # G > 64
    assert L.haste_group_greedy(A, A, 128, 10, 64, 32, A, A, 16, None) == WS
