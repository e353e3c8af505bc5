"""GPU parity of the FP8-weight variants: haste_quantize_w8 bit-exact
against the oracle's E4M3 codec and group exponents; haste_fwd_w8 and
haste_step_w8 bitwise equal to haste_fwd / haste_step on the dequantized
(exact bf16) weights, and within the layer's tolerance of the fp64 oracle
run on those weights."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import bf16_bits, get_workload, make_inputs, normal_bf16, sorted_subsets, zipf_labels

pytestmark = pytest.mark.gpu

# (B, H, K, G, F): the 32-row and 16-row feature-gradient kernels, every G and F
CASES = [(64, 256, 37, 16, 32), (77, 768, 29, 32, 64), (128, 768, 300, 32, 64), (64, 768, 21, 64, 64),
         (256, 768, 13, 16, 128), (96, 512, 11, 32, 128), (33, 96, 17, 64, 32), (45, 200, 9, 64, 128)]


def _weights(K, G, F, seed):
    """Weights whose groups span many binades, with an all-zero group, a
    group of tiny values and exact E4M3 ties after scaling."""
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.integers(-20, 20, size=K)
    w = rng.normal(size=(K * G, F)) * np.repeat(mag, G)[:, None]
    w[:G] = 0.0
    if K > 2:
        w[G:2 * G] *= 2.0 ** -110
        w[2 * G, 0] = 448.0 * 2.0 ** 3                       # the group maximum, exactly 448 * 2^3
        w[2 * G, 1:9] = np.array([1.0625, 1.1875, 3.25, -0.15625, 2 ** -6, 2 ** -9, 1.5 * 2 ** -9, 2.5 * 2 ** -9]) * 8
    return bf16_bits(w.astype(np.float32))


@pytest.mark.parametrize("G,F", [(16, 32), (16, 128), (32, 64), (64, 64), (64, 128)])
def test_quantize_w8_bit_exact(G, F):
    K = 23
    W = _weights(K, G, F, 70 + G + F)
    W8, e = hs.quantize_w8(to_dev_bf16(W), G)
    ref8, refe = O.oracle_quantize_w8(W, G)
    assert (to_host(e) == refe).all(), f"group exponents differ: {to_host(e)} vs {refe}"
    got = to_host(W8)
    bad = np.argwhere(got != ref8)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def _case_inputs(B, H, K, G, F, seed):
    h = normal_bf16(B * H, 1.0, seed, 1).reshape(B, H)
    W = normal_bf16(K * G * F, float(1.0 / np.sqrt(F)), seed, 2).reshape(K * G, F)
    idx = sorted_subsets(K, F, H, seed, 0)
    rp, col = zipf_labels(B, K * G, min(5, K * G), seed)
    return h, W, idx, rp, col


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}_h{c[1]}_k{c[2]}_g{c[3]}_f{c[4]}" for c in CASES])
def test_step_w8(case):
    B, H, K, G, F = case
    say(f"  step_w8 B={B} H={H} K={K} G={G} F={F}")
    h, W, idx, rp, col = _case_inputs(B, H, K, G, F, 80 + K)
    W8, e = O.oracle_quantize_w8(W, G)
    Wq = O.oracle_dequantize_w8(W8, e, G)                  # the weights the FP8 variant computes with
    hd, idd, rpd, cold = to_dev_bf16(h), to_dev_i32(idx), to_dev_i32(rp), to_dev_i32(col)
    W8d, ed = __import__("torch").from_numpy(W8).to(hd.device), to_dev_i32(e)
    s = 1.0 / B
    a = hs.step_w8(hd, idd, W8d, ed, rpd, cold, s, G, mode="det", want_Z=True, want_loss=True)
    b = hs.step(hd, idd, to_dev_bf16(Wq), rpd, cold, s, G, mode="det", want_Z=True, want_loss=True)
    for k in ("Z", "dW", "dh"):
        assert (to_host(a[k]).view(np.uint32) == to_host(b[k]).view(np.uint32)).all(), f"{k} differs from bf16 step"
    ref = O.oracle_step(h, idx, Wq, rp, col, s, G)
    assert_parity(to_host(a["Z"]), ref["Z"], "Z")
    assert_parity(to_host(a["dW"]), ref["dW"], "dW")
    assert_parity(to_host(a["dh"]), ref["dh"], "dh")
    loss = float(to_host(a["loss"])[0])
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    # atomic mode and the forward alone
    c = hs.step_w8(hd, idd, W8d, ed, rpd, cold, s, G, mode="atomic")
    assert_parity(to_host(c["dh"]), ref["dh"], "dh atomic")
    Z = hs.fwd_w8(hd, idd, W8d, ed, G)
    assert (to_host(Z).view(np.uint32) == to_host(hs.fwd(hd, idd, to_dev_bf16(Wq), G)).view(np.uint32)).all()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_step_w8_fullsize():
    """Amazon-3M shape in the benchmark's configuration: quantized on the GPU
    (codes checked on sampled group slices), then the FP8 step bitwise equal
    to the bf16 step on the dequantized weights, and against the oracle on
    sampled rows and groups."""
    import torch

    w = get_workload("amazon3m_shaped")
    say(f"  generating {w.name}")
    d = make_inputs(w, dZ=False)
    B, G, K = w.B, w.G, w.K
    hd, idd = to_dev_bf16(d["h"]), to_dev_i32(d["idx"])
    W8, e = hs.quantize_w8(to_dev_bf16(d["W"]), G)
    W8h, eh = to_host(W8), to_host(e)
    for k0 in (0, K // 2, K - 64):
        k1 = k0 + 64
        r8, re = O.oracle_quantize_w8(np.ascontiguousarray(d["W"][k0 * G:k1 * G]), G)
        assert (W8h[k0 * G:k1 * G] == r8).all() and (eh[k0:k1] == re).all(), f"codes of groups [{k0},{k1})"
    Wq = O.oracle_dequantize_w8(W8h, eh, G)
    rpd, cold = to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"])
    s = 1.0 / B
    a = hs.step_w8(hd, idd, W8, e, rpd, cold, s, G, mode="det")
    dW, dh = to_host(a["dW"]), to_host(a["dh"])
    del a
    b = hs.step(hd, idd, to_dev_bf16(Wq), rpd, cold, s, G, mode="det")
    assert (dW.view(np.uint32) == to_host(b["dW"]).view(np.uint32)).all(), "dW differs from the bf16 step"
    assert (dh.view(np.uint32) == to_host(b["dh"]).view(np.uint32)).all(), "dh differs from the bf16 step"
    del b
    torch.cuda.empty_cache()
    rows = [0, B // 2, B - 1]
    rp, cols = [0], []
    for r in rows:
        c = d["y_col"][d["y_rowptr"][r]:d["y_rowptr"][r + 1]]
        cols.append(c)
        rp.append(rp[-1] + c.size)
    ref = O.oracle_step(np.ascontiguousarray(d["h"][rows]), d["idx"], Wq, np.array(rp, np.int32),
                        np.concatenate(cols).astype(np.int32), s, G, want_dW=False)
    assert_parity(dh[rows], ref["dh"], "dh rows")
