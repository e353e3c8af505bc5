"""The feature-gradient status word: every call that runs the grouped dh
kernels leaves 0 in the first 4 bytes of its workspace after a correct run,
and a turn wait that gives up (forced from the host with a zero wait bound,
so every kernel still runs to its end) is reported, never silent."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import normal_bf16, sorted_subsets, zipf_labels

pytestmark = pytest.mark.gpu

# (B, H, K, G, F): the 32-row kernel with a turn counter per 16-row half
# (G = 32, F = 64) and per 8-row quarter (G = 16, F = 128), and the 16-row
# kernel (H > 768)
SHAPES = [(77, 768, 900, 32, 64), (45, 640, 400, 16, 128), (50, 1024, 300, 16, 64)]


def inputs(B, H, K, G, F, seed):
    L = K * G
    d = {"h": normal_bf16(B * H, 1.0, seed, 1).reshape(B, H),
         "W": normal_bf16(L * F, float(1 / np.sqrt(F)), seed, 2).reshape(L, F),
         "dZ": normal_bf16(B * L, 1.0, seed, 3).reshape(B, L),
         "idx": sorted_subsets(K, F, H, seed, 0)}
    d["y_rowptr"], d["y_col"] = zipf_labels(B, L, 5, seed)
    return d


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", ["atomic", "det"])
def test_status_word_zero_after_correct_runs(shape, mode):
    import torch
    B, H, K, G, F = shape
    say(f"  status ok {mode} {shape}")
    d = inputs(B, H, K, G, F, 11)
    h, idx, W, dZ = to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_bf16(d["dZ"])
    rp, col = to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"])
    ws = torch.empty(hs.workspace_size("step", B, H, K, G, F, mode), dtype=torch.uint8, device=h.device)
    ws.fill_(0xAB)                       # stale contents must not leak into the word
    hs.binding.CHECK_DH_STATUS = False
    try:
        dh = hs.bwd_h(dZ, idx, W, G, H, mode=mode, workspace=ws)
        assert hs.binding.workspace_status(ws) == 0
        assert_parity(to_host(dh), O.oracle_bwd_h(d["dZ"], d["idx"], d["W"], G, H), f"dh[{mode}]")
        ws.fill_(0xAB)
        hs.step(h, idx, W, rp, col, 1.0 / B, G, mode=mode, workspace=ws)
        assert hs.binding.workspace_status(ws) == 0
    finally:
        hs.binding.CHECK_DH_STATUS = True


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", ["atomic", "det"])
def test_turn_wait_give_up_is_reported(shape, mode):
    """Wait bound 0: no wave gets its turn, every update is skipped, the kernels
    end normally and the status word says so; the checked binding raises."""
    import torch
    B, H, K, G, F = shape
    say(f"  status forced {mode} {shape}")
    d = inputs(B, H, K, G, F, 12)
    h, idx, W, dZ = to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_bf16(d["dZ"])
    rp, col = to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"])
    ws = torch.empty(hs.workspace_size("step", B, H, K, G, F, mode), dtype=torch.uint8, device=h.device)
    hs.binding.test_set_turn_spins(0)
    try:
        with pytest.raises(hs.binding.HandoffError):
            hs.bwd_h(dZ, idx, W, G, H, mode=mode, workspace=ws)
        assert hs.binding.workspace_status(ws) == 1
        with pytest.raises(hs.binding.HandoffError):
            hs.step(h, idx, W, rp, col, 1.0 / B, G, mode=mode, workspace=ws)
        assert hs.binding.workspace_status(ws) == 1
    finally:
        hs.binding.test_set_turn_spins(-1)
    # default bound again: the same workspace reports a clean run
    dh = hs.bwd_h(dZ, idx, W, G, H, mode=mode, workspace=ws)
    assert hs.binding.workspace_status(ws) == 0
    assert_parity(to_host(dh), O.oracle_bwd_h(d["dZ"], d["idx"], d["W"], G, H), f"dh[{mode}]")
