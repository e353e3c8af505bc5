"""GPU parity on seeded random shapes, as a third layer beside the hand-picked
cases of test_gpu_parity.py: every G and F the library supports, any H from
F to 1024 (odd ones included), batches of 1 to 256 rows and 1 to 300
groups, each shape running every layer call through the C ABI against the
fp64 oracle at the same bar (relative L2 2e-3, max abs 1e-2; loss to 1e-5
relative)."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import normal_bf16, sorted_subsets
from test_gpu_parity import labels_mixed

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([16, 32, 64]))
        F = int(rng.choice([32, 64, 128]))
        H = int(rng.integers(F, 1025))
        B = int(rng.integers(1, 257))
        K = int(rng.integers(1, 301))
        out.append((B, H, K, G, F))
    return out


SHAPES = _shapes()


def _inputs(B, H, K, G, F, seed):
    L = K * G
    d = {
        "h": normal_bf16(B * H, 1.0, seed, 1).reshape(B, H),
        "W": normal_bf16(L * F, float(1 / np.sqrt(F)), seed, 2).reshape(L, F),
        "dZ": normal_bf16(B * L, 1.0, seed, 3).reshape(B, L),
        "idx": sorted_subsets(K, F, H, seed, 0),
    }
    d["y_rowptr"], d["y_col"] = labels_mixed(B, L, seed)
    return d


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_H{s[1]}_K{s[2]}_G{s[3]}_F{s[4]}" for s in SHAPES])
def test_every_call_on_a_random_shape(shape):
    B, H, K, G, F = shape
    seed = 700 + SHAPES.index(shape)
    say(f"  random shape B={B} H={H} K={K} G={G} F={F}")
    d = _inputs(B, H, K, G, F, seed)
    s = 1.0 / B
    h, idx, W, dZ = to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_bf16(d["dZ"])
    rp = to_dev_i32(d["y_rowptr"])
    col = to_dev_i32(d["y_col"] if d["y_col"].size else np.zeros(4, np.int32))

    assert_parity(to_host(hs.fwd(h, idx, W, G)), O.oracle_fwd(d["h"], d["idx"], d["W"], G), "Z")
    assert_parity(to_host(hs.bwd_w(h, idx, dZ, G)), O.oracle_bwd_w(d["h"], d["idx"], d["dZ"], G), "dW")
    ref_dh = O.oracle_bwd_h(d["dZ"], d["idx"], d["W"], G, H)
    for mode in ("atomic", "det"):
        assert_parity(to_host(hs.bwd_h(dZ, idx, W, G, H, mode=mode)), ref_dh, f"dh[{mode}]")

    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], s, G)
    for mode in ("atomic", "det"):
        out = hs.step(h, idx, W, rp, col, s, G, mode=mode, want_Z=True, want_loss=True)
        assert_parity(to_host(out["Z"]), ref["Z"], f"step Z[{mode}]")
        assert_parity(to_host(out["dW"]), ref["dW"], f"step dW[{mode}]")
        assert_parity(to_host(out["dh"]), ref["dh"], f"step dh[{mode}]")
        lg = float(to_host(out["loss"])[0])
        assert abs(lg - ref["loss"]) <= 1e-5 * abs(ref["loss"]), (lg, ref["loss"])
    out = hs.step(h, idx, W, rp, col, s, G, mode="det", dw_bf16=True)
    dw16 = to_host(out["dW"])
    assert_parity((dw16.astype(np.uint32) << 16).view(np.float32), ref["dW"], "step bf16 dW")
    assert_parity(to_host(out["dh"]), ref["dh"], "step dh (bf16 dW pass)")
