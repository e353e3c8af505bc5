"""haste_step_noalloc (the fused pass on the library's per-GPU scratch array,
no workspace, no allocation) against haste_step through the C ABI: two calls
in a row, the second with a smaller input, in both dh modes; deterministic
results bitwise equal, atomic ones within the parity tolerance; the small
case also against the oracle; shapes past the array's size refused."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_exact, assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import normal_bf16, sorted_subsets, zipf_labels

pytestmark = pytest.mark.gpu

# (B, H, K, G, F): a 640K-label pass with the 3M shape's row tiles (25 MB of
# deterministic partials), then a small ragged one
LARGE = (128, 768, 20000, 32, 64)
SMALL = (45, 200, 37, 16, 64)


def inputs(shape, seed):
    B, H, K, G, F = shape
    L = K * G
    d = {"h": normal_bf16(B * H, 1.0, seed, 1).reshape(B, H),
         "W": normal_bf16(L * F, float(1 / np.sqrt(F)), seed, 2).reshape(L, F),
         "idx": sorted_subsets(K, F, H, seed, 0)}
    d["y_rowptr"], d["y_col"] = zipf_labels(B, L, 5, seed)
    return d


def dev(d):
    return (to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_i32(d["y_rowptr"]),
            to_dev_i32(d["y_col"]))


def run_both(shape, d, mode):
    B, H, K, G, F = shape
    h, idx, W, rp, col = dev(d)
    s = 1.0 / B
    ref = hs.step(h, idx, W, rp, col, s, G, mode=mode, want_Z=True, want_loss=True)
    got = hs.step_noalloc(h, idx, W, rp, col, s, G, mode=mode, want_Z=True, want_loss=True)
    return {k: to_host(v) for k, v in ref.items()}, {k: to_host(v) for k, v in got.items()}


@pytest.mark.parametrize("mode", ["det", "atomic"])
def test_noalloc_matches_step_two_calls(mode):
    for i, (shape, seed) in enumerate(((LARGE, 31), (SMALL, 32))):
        say(f"  noalloc[{mode}] call {i + 1} {shape}")
        d = inputs(shape, seed)
        ref, got = run_both(shape, d, mode)
        # dW, Z and the loss come from the same forward kernel in both calls
        assert_exact(got["dW"], ref["dW"], "dW")
        assert_exact(got["Z"], ref["Z"], "Z")
        if mode == "det":
            assert_exact(got["dh"], ref["dh"], "dh")
            assert got["loss"][0] == ref["loss"][0]
        else:
            assert_parity(got["dh"], ref["dh"], "dh vs haste_step")
            assert abs(got["loss"][0] - ref["loss"][0]) <= 1e-9 * abs(ref["loss"][0])
        if shape == SMALL:
            B, H, K, G, F = shape
            o = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], 1.0 / B, G)
            assert_parity(got["dW"], o["dW"], "dW vs oracle")
            assert_parity(got["dh"], o["dh"], "dh vs oracle")
            assert abs(got["loss"][0] - o["loss"]) <= 1e-5 * abs(o["loss"])


def test_noalloc_refuses_shapes_past_its_scratch():
    import torch
    B, H, K, G, F = 256, 1024, 64, 32, 64    # 16-row tiles: 33.6 MB of deterministic partials
    need = hs.workspace_size("step", B, H, K, G, F, "det")
    assert need > 32 << 20
    dv = torch.device("cuda:0")
    h = torch.zeros(B, H, dtype=torch.bfloat16, device=dv)
    idx = torch.zeros(K, F, dtype=torch.int32, device=dv)
    W = torch.zeros(K * G, F, dtype=torch.bfloat16, device=dv)
    rp = torch.zeros(B + 1, dtype=torch.int32, device=dv)
    col = torch.zeros(4, dtype=torch.int32, device=dv)
    with pytest.raises(hs.binding.HasteError) as e:
        hs.step_noalloc(h, idx, W, rp, col, 1.0 / B, G, mode="det")
    assert e.value.code == -5
    # the atomic mode needs no partials: the same shape fits
    assert hs.workspace_size("step", B, H, K, G, F, "atomic") <= 32 << 20
