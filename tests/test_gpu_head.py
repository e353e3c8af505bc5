"""GPU parity of the head-tail split: the dense head pass (haste_head_step)
and the joint head + tail pass (haste_joint_step) against the fp64 CPU
oracle, called through the C ABI.  Small and ragged shapes compare every
output; the full 3M split compares the whole head, sampled rows of dh and
sampled groups of the tail's dW."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import get_workload, make_inputs, normal_bf16, zipf_labels

pytestmark = pytest.mark.gpu

# (B, H, L_head): one label, a ragged label count (BCE tail stores), label
# counts that are multiples of 8 (16-byte stores, and the matrix-core
# feature-gradient kernel, here with two 128-row blocks and a partial
# column block), batches around 128, and label counts past one or several
# feature-gradient chunks of 1024 labels
# B <= 128, H % 64 == 0 and L % 8 == 0 take the fused logits + BCE kernel
# (e.g. (64, 128, 256), (128, 768, 2048), (64, 256, 5000), (37, 192, 200));
# the others the rocBLAS logits and the separate BCE kernel
HEAD_CASES = [(1, 16, 1), (5, 40, 13), (64, 128, 256), (37, 96, 73), (130, 264, 1001), (128, 768, 2048),
              (64, 256, 5000), (130, 200, 1000), (3, 8, 8), (37, 192, 200), (1, 64, 8)]


def _head_inputs(B, H, L, seed):
    h = normal_bf16(B * H, 1.0, seed, 1).reshape(B, H)
    W = normal_bf16(L * H, float(1.0 / np.sqrt(H)), seed, 7).reshape(L, H)
    rp, col = zipf_labels(B, L, min(4, L), seed)
    return h, W, rp, col


@pytest.mark.parametrize("shape", HEAD_CASES, ids=[f"b{b}_h{h}_l{l}" for b, h, l in HEAD_CASES])
def test_head_step(shape):
    B, H, L = shape
    say(f"  head_step B={B} H={H} L={L}")
    h, W, rp, col = _head_inputs(B, H, L, 30 + L)
    s = 1.0 / B
    out = hs.head_step(to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(rp), to_dev_i32(col), s, want_Z=True,
                       want_loss=True)
    ref = O.oracle_head_step(h, W, rp, col, s)
    assert_parity(to_host(out["Z"]), ref["Z"], "head Z")
    assert_parity(to_host(out["dW"]), ref["dW"], "head dW")
    assert_parity(to_host(out["dh"]), ref["dh"], "head dh")
    loss = float(to_host(out["loss"])[0])
    say(f"    loss {loss:.9g} vs {ref['loss']:.9g}")
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])


@pytest.mark.parametrize("L", [777, 776])
def test_head_step_repeatable_and_optional_outputs(L):
    B, H = 96, 256
    h, W, rp, col = _head_inputs(B, H, L, 41)
    d = [to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(rp), to_dev_i32(col)]
    a = hs.head_step(*d, 1.0 / B, want_Z=True, want_loss=True)
    b = hs.head_step(*d, 1.0 / B)
    for k in ("dW", "dh"):
        assert (to_host(a[k]).view(np.uint32) == to_host(b[k]).view(np.uint32)).all(), f"head {k} not repeatable"


def _joint(w, d, mode, st, sh, want_loss=True):
    return hs.joint_step(to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_i32(d["y_rowptr"]),
                         to_dev_i32(d["y_col"]), to_dev_bf16(d["W_head"]), to_dev_i32(d["yh_rowptr"]),
                         to_dev_i32(d["yh_col"]), st, sh, w.G, mode=mode, want_loss=want_loss)


@pytest.mark.parametrize("mode", ["atomic", "det"])
def test_joint_step_small(mode):
    w = get_workload("ht_small")
    d = make_inputs(w, dZ=False, w_head=True)
    st, sh = 1.0 / w.B, 0.5 / w.B
    say(f"  joint_step ht_small [{mode}]")
    out = _joint(w, d, mode, st, sh)
    ref = O.oracle_joint_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["W_head"], d["yh_rowptr"],
                              d["yh_col"], st, sh, w.G)
    assert_parity(to_host(out["dW_tail"]), ref["dW_tail"], "joint dW_tail")
    assert_parity(to_host(out["dW_head"]), ref["dW_head"], "joint dW_head")
    assert_parity(to_host(out["dh"]), ref["dh"], "joint dh")
    loss = float(to_host(out["loss"])[0])
    say(f"    loss {loss:.9g} vs {ref['loss']:.9g}")
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    if mode == "det":
        again = _joint(w, d, mode, st, sh)
        assert (to_host(again["dh"]).view(np.uint32) == to_host(out["dh"]).view(np.uint32)).all(), \
            "joint dh not bitwise repeatable in deterministic mode"


def test_joint_equals_tail_plus_head():
    """dh of the joint pass is the tail's dh plus the head's, in that order."""
    w = get_workload("ht_small")
    d = make_inputs(w, dZ=False, w_head=True)
    s = 1.0 / w.B
    out = _joint(w, d, "det", s, s, want_loss=False)
    hd, idx, Wt = to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"])
    t = hs.step(hd, idx, Wt, to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"]), s, w.G, mode="det")
    hh = hs.head_step(hd, to_dev_bf16(d["W_head"]), to_dev_i32(d["yh_rowptr"]), to_dev_i32(d["yh_col"]), s)
    for k_joint, k_part, part in (("dW_tail", "dW", t), ("dW_head", "dW", hh)):
        assert (to_host(out[k_joint]).view(np.uint32) == to_host(part[k_part]).view(np.uint32)).all(), k_joint
    # the head pass adds its product onto the tail's dh as one fp32 addition
    want = to_host(t["dh"]) + to_host(hh["dh"])
    assert (to_host(out["dh"]).view(np.uint32) == want.view(np.uint32)).all(), "joint dh != tail dh + head dh"


def _rows_labels(rowptr, col, rows):
    rp, cols = [0], []
    for b in rows:
        c = col[rowptr[b]:rowptr[b + 1]]
        cols.append(c)
        rp.append(rp[-1] + c.size)
    return np.array(rp, np.int32), (np.concatenate(cols).astype(np.int32) if rp[-1] else np.zeros(0, np.int32))


def _group_labels(rowptr, col, lo, hi):
    rp, cols = [0], []
    for b in range(rowptr.size - 1):
        c = col[rowptr[b]:rowptr[b + 1]]
        c = c[(c >= lo) & (c < hi)] - lo
        cols.append(c)
        rp.append(rp[-1] + c.size)
    return np.array(rp, np.int32), (np.concatenate(cols).astype(np.int32) if rp[-1] else np.zeros(0, np.int32))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_joint_step_fullsize_sampled():
    """The 3M head-tail split (89,088 head labels, 2,910,848 tail labels at
    G = 32, F = 64, H = 768, B = 128) in the benchmark's launch
    configuration: the whole head against the oracle, dh on sampled rows,
    the tail's dW on sampled groups."""
    w = get_workload("ht3m_tail_shaped")
    say(f"  generating {w.name} with its head")
    d = make_inputs(w, dZ=False, w_head=True)
    B, G, K = w.B, w.G, w.K
    s = 1.0 / B
    say("  joint_step [det]")
    out = _joint(w, d, "det", s, s)
    dW_head = to_host(out["dW_head"])
    dW_tail = to_host(out["dW_tail"])
    dh = to_host(out["dh"])
    del out
    say("  oracle head (full)")
    ref_h = O.oracle_head_step(d["h"], d["W_head"], d["yh_rowptr"], d["yh_col"], s)
    assert_parity(dW_head, ref_h["dW"], "dW_head")
    rows = sorted({0, 1, B // 2, B - 1})
    rp, col = _rows_labels(d["y_rowptr"], d["y_col"], rows)
    say(f"  oracle tail on rows {rows}")
    ref_t = O.oracle_step(np.ascontiguousarray(d["h"][rows]), d["idx"], d["W"], rp, col, s, G, want_dW=False)
    assert_parity(dh[rows], ref_t["dh"] + ref_h["dh"][rows], "dh rows")
    for k0 in (0, K // 2, K - 48):
        k1 = k0 + 48
        rpg, colg = _group_labels(d["y_rowptr"], d["y_col"], k0 * G, k1 * G)
        ref = O.oracle_step(d["h"], np.ascontiguousarray(d["idx"][k0:k1]), np.ascontiguousarray(d["W"][k0 * G:k1 * G]),
                            rpg, colg, s, G, want_dh=False)
        assert_parity(dW_tail[k0 * G:k1 * G], ref["dW"], f"dW_tail groups [{k0},{k1})")
