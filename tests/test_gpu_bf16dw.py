"""GPU checks of the fused pass with a bf16 weight gradient
(haste_step_bf16dw), through the C ABI.  Its dW must be, bit for bit, the
bf16 rounding (to nearest even) of haste_step's fp32 dW on the same inputs,
and its dh and loss those of haste_step.  Against the fp64 oracle it meets
the parity bar on every shape: the storage rounding alone gives dW a
relative L2 error of about 1.65e-3 (half a bf16 unit in the last place at
most per entry), under the 2e-3 bar, because the dZ that forms it is split
into bf16 hi + lo parts and the fp32 sum is rounded once."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_host
from oracle import oracle as O
from synthetic import get_workload, make_inputs
from test_gpu_parity import case, dev_inputs

pytestmark = pytest.mark.gpu

# the tile paths of the forward kernel: dW staged per group (G x (F + 4)
# floats fit) and per 16-label tile (wide tiles), chunk pairs (B 97..128),
# one chunk, padded batches
SHAPES = ["tiny_4k", "g32_f64_b77", "g64_f64_b64", "g16_f128_b256", "g32_f128_b96", "g64_f32_b33",
          "g32_f32_b1", "g32_f64_many_b128", "g64_f128_b45"]


def _rne_bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", SHAPES)
@pytest.mark.parametrize("mode", ["det", "atomic"])
def test_bf16_dw_is_the_rounded_fp32_dw(name, mode):
    d = case(name)
    say(f"bf16 dW {name} {mode}")
    h, idx, W, dZ, rp, col = dev_inputs(d)
    G, s = d["G"], d["scale"]
    ref = hs.step(h, idx, W, rp, col, s, G, mode="det" if mode == "det" else "atomic", want_loss=True)
    out = hs.step(h, idx, W, rp, col, s, G, mode=mode, want_loss=True, dw_bf16=True)
    dw32, dw16 = to_host(ref["dW"]), to_host(out["dW"])
    assert dw16.dtype == np.uint16 and dw16.shape == dw32.shape
    want = _rne_bf16_bits(dw32)
    bad = np.count_nonzero(dw16 != want)
    assert bad == 0, f"{bad} dW entries are not the rounded fp32 dW"
    if mode == "det":
        assert np.array_equal(to_host(out["dh"]).view(np.uint32), to_host(ref["dh"]).view(np.uint32))
    else:
        assert np.allclose(to_host(out["dh"]), to_host(ref["dh"]), rtol=1e-5, atol=1e-6)
    assert abs(to_host(out["loss"])[0] - to_host(ref["loss"])[0]) <= 1e-12 * abs(to_host(ref["loss"])[0]) + 1e-12
    oref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], s, G)
    dwf = (dw16.astype(np.uint32) << 16).view(np.float32)
    assert_parity(dwf, oref["dW"], f"bf16 dW vs oracle {name} {mode}")
    assert_parity(to_host(out["dh"]), oref["dh"], f"dh vs oracle {name} {mode}")


def test_bf16_dw_refuses_logits_output():
    d = case("tiny_4k")
    h, idx, W, dZ, rp, col = dev_inputs(d)
    with pytest.raises(ValueError):
        hs.step(h, idx, W, rp, col, d["scale"], d["G"], want_Z=True, dw_bf16=True)


def test_bf16_dw_full_3m():
    """The Amazon-3M shape: every dW entry the rounded fp32 value (compared on
    the device), dh bitwise that of the fp32-dW pass."""
    import torch
    w = get_workload("amazon3m_shaped")
    d = make_inputs(w, dZ=False)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    h, idx, W, rp, col = bf(d["h"]), i32(d["idx"]), bf(d["W"]), i32(d["y_rowptr"]), i32(d["y_col"])
    ref = hs.step(h, idx, W, rp, col, 1.0 / w.B, w.G, mode="det")
    out = hs.step(h, idx, W, rp, col, 1.0 / w.B, w.G, mode="det", dw_bf16=True)
    torch.cuda.synchronize()
    want = ref["dW"].to(torch.bfloat16)
    bad = int((out["dW"].view(torch.int16) != want.view(torch.int16)).sum().item())
    assert bad == 0, f"{bad} of {want.numel()} dW entries differ from the rounded fp32 dW"
    assert torch.equal(out["dh"].view(torch.int32), ref["dh"].view(torch.int32))
