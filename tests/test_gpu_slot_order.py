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
