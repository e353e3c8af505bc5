"""GPU parity of the bank-balanced slot order (haste_order_slots) against the
CPU oracle, through the C ABI: the reordered index rows, the moved weight
columns and the permutation are integer work and must match bit-exactly.
The layer run on reordered index sets must still match the oracle, and its
dh must equal (to the parity tolerance) that of the original order."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_exact, assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import get_workload, make_inputs, normal_bf16, sorted_subsets

pytestmark = pytest.mark.gpu

# (K, G, F, H, seed)
CASES = [
    (1, 16, 32, 64, 1),
    (5, 32, 64, 768, 2),
    (1000, 32, 64, 768, 3),
    (333, 16, 128, 768, 4),
    (77, 64, 64, 1024, 5),
    (64, 64, 128, 256, 6),
    (17, 16, 32, 32, 7),          # F = H: every column present
    (9, 32, 128, 130, 8),
]


@pytest.mark.parametrize("K,G,F,H,seed", CASES)
def test_order_slots_bit_exact(K, G, F, H, seed):
    say(f"order_slots K={K} G={G} F={F} H={H}")
    idx = sorted_subsets(K, F, H, seed, 0)
    if seed % 2:
        rng = np.random.default_rng(seed)
        idx = np.stack([r[rng.permutation(F)] for r in idx]).astype(np.int32)   # any given order
    W = normal_bf16(K * G * F, 0.5, seed, 2).reshape(K * G, F)
    want_idx, want_W, want_perm = O.oracle_order_slots(idx, W, G)
    di, dw = to_dev_i32(idx), to_dev_bf16(W)
    perm = hs.order_slots(di, dw, G, perm=True)
    assert_exact(to_host(di), want_idx, "idx")
    assert_exact(to_host(dw), want_W, "W")
    assert_exact(to_host(perm), want_perm, "perm")
    # index rows alone (W not given), no permutation output
    di2 = to_dev_i32(idx)
    assert hs.order_slots(di2) is None
    assert_exact(to_host(di2), want_idx, "idx alone")
    assert hs.validate_idx(di, H) == 0


def test_layer_on_ordered_slots_matches_oracle():
    d = make_inputs(get_workload("tiny_4k"))
    G, H = 16, d["h"].shape[1]
    B = d["h"].shape[0]
    scale = 1.0 / B
    h, idx, W = to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"])
    rp, col = to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"])
    base = {k: to_host(v) for k, v in hs.step(h, idx, W, rp, col, scale, G, mode="det", want_Z=True).items()
            if v is not None}
    perm = hs.order_slots(idx, W, G, perm=True)
    # the reference orders the generator's arrays itself; the GPU's order must equal it
    idx_o, W_o, p = O.oracle_order_slots(d["idx"], d["W"], G)
    p = p.astype(np.int64)
    assert_exact(to_host(idx), idx_o, "ordered idx")
    assert_exact(to_host(W), W_o, "ordered W")
    assert_exact(to_host(perm), p, "perm")
    ref = O.oracle_step(d["h"], idx_o, W_o, d["y_rowptr"], d["y_col"], scale, G)
    for mode in ("det", "atomic"):
        out = {k: to_host(v) for k, v in hs.step(h, idx, W, rp, col, scale, G, mode=mode).items() if v is not None}
        assert_parity(out["dh"], ref["dh"], f"dh ordered {mode}")
        assert_parity(out["dW"], ref["dW"], f"dW ordered {mode}")
        assert_parity(out["dh"], base["dh"], f"dh ordered vs original {mode}")
        assert_parity(out["dW"], np.take_along_axis(base["dW"], np.repeat(p, G, 0), 1),
                      f"dW ordered vs original permuted {mode}")
    z = to_host(hs.fwd(h, idx, W, G))
    assert_parity(z, O.oracle_fwd(d["h"], idx_o, W_o, G), "Z ordered")
    assert_parity(z, base["Z"], "Z ordered vs original")


def test_order_slots_full_size_sampled():
    w = get_workload("amazon3m_shaped")
    idx = sorted_subsets(w.K, w.F, w.H, w.seed_no, 0)
    di = to_dev_i32(idx)
    perm = hs.order_slots(di, perm=True)
    got, gp = to_host(di), to_host(perm)
    rows = np.random.default_rng(11).choice(w.K, 1500, replace=False)
    rows = np.concatenate([rows, [0, w.K - 1]])
    want, _, wp = O.oracle_order_slots(idx[rows])
    assert_exact(got[rows], want, "3M idx sampled rows")
    assert_exact(gp[rows], wp, "3M perm sampled rows")
    assert hs.validate_idx(di, w.H) == 0


def test_any_slot_order_every_call():
    """Index rows in an arbitrary order (W's columns moved along): forward,
    dW, dh (both modes) and the fused pass match the oracle on the same
    permuted inputs, and rewiring yields the same sets and weights as it does
    from sorted rows."""
    B, H, K, G, F = 77, 300, 40, 32, 64
    rng = np.random.default_rng(41)
    idx = sorted_subsets(K, F, H, 12, 0)
    W = normal_bf16(K * G * F, 0.5, 12, 2).reshape(K * G, F)
    h = normal_bf16(B * H, 1.0, 12, 1).reshape(B, H)
    dZ = normal_bf16(B * K * G, 1.0, 12, 3).reshape(B, K * G)
    sig = np.stack([rng.permutation(F) for _ in range(K)])
    idx_p = np.ascontiguousarray(np.take_along_axis(idx, sig, 1)).astype(np.int32)
    W_p = np.ascontiguousarray(np.take_along_axis(W, np.repeat(sig, G, 0), 1))
    # two distinct positive labels per sample, sorted (CSR)
    col = np.concatenate([np.sort(rng.choice(K * G, 2, replace=False)) for _ in range(B)]).astype(np.int32)
    rp = np.arange(0, 2 * B + 1, 2, dtype=np.int32)
    dh_, dp = to_dev_bf16(h), to_dev_i32(idx_p)
    dw_, dz_ = to_dev_bf16(W_p), to_dev_bf16(dZ)
    assert hs.validate_idx(dp, H) == 0
    assert_parity(to_host(hs.fwd(dh_, dp, dw_, G)), O.oracle_fwd(h, idx_p, W_p, G), "Z, shuffled slots")
    assert_parity(to_host(hs.bwd_w(dh_, dp, dz_, G)), O.oracle_bwd_w(h, idx_p, dZ, G), "dW, shuffled slots")
    ref_dh = O.oracle_bwd_h(dZ, idx_p, W_p, G, H)
    for mode in ("det", "atomic"):
        assert_parity(to_host(hs.bwd_h(dz_, dp, dw_, G, H, mode=mode)), ref_dh, f"dh {mode}, shuffled slots")
    ref = O.oracle_step(h, idx_p, W_p, rp, col, 1.0 / B, G)
    out = hs.step(dh_, dp, dw_, to_dev_i32(rp), to_dev_i32(col), 1.0 / B, G, mode="det")
    assert_parity(to_host(out["dW"]), ref["dW"], "step dW, shuffled slots")
    assert_parity(to_host(out["dh"]), ref["dh"], "step dh, shuffled slots")
    # rewiring: small-integer inputs make every score exact, so the selection
    # is the same whatever the order of the input row
    hi = (rng.integers(-3, 4, size=(B, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    zi = (rng.integers(-3, 4, size=(B, K * G)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wi = (rng.integers(-3, 4, size=(K * G, F)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wi_p = np.ascontiguousarray(np.take_along_axis(wi, np.repeat(sig, G, 0), 1))
    r_sorted = hs.rewire(to_dev_bf16(hi), to_dev_bf16(zi), to_dev_i32(idx), to_dev_bf16(wi), G, 9)
    r_shuf = hs.rewire(to_dev_bf16(hi), to_dev_bf16(zi), to_dev_i32(idx_p), to_dev_bf16(wi_p), G, 9)
    assert_exact(to_host(r_shuf["idx"]), to_host(r_sorted["idx"]), "rewired index rows")
    assert_exact(to_host(r_shuf["W"]), to_host(r_sorted["W"]), "rewired weights")
    want_idx, want_W, _, _ = O.oracle_rewire(hi, zi, idx_p, wi_p, 9, G)
    assert_exact(to_host(r_shuf["idx"]), want_idx, "rewired index rows vs oracle")
    assert_exact(to_host(r_shuf["W"]), want_W, "rewired weights vs oracle")
