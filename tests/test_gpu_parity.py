"""GPU parity: every libhaste entry point against the fp64 CPU oracle, called
through the C ABI (ctypes binding), at sizes that span several tiles and a
ragged batch tail, plus bit-exact index probes and determinism."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import (assert_exact, assert_parity, dev, say, to_dev_bf16, to_dev_i32, to_host)
from oracle import oracle as O
from synthetic import bf16_bits, normal_bf16, sorted_subsets, zipf_labels

pytestmark = pytest.mark.gpu

# name: (B, H, K, G, F)
CASES = {
    "tiny_4k": (64, 256, 256, 16, 32),
    "g16_f64_b45": (45, 200, 37, 16, 64),
    "g32_f64_b77": (77, 768, 29, 32, 64),
    "g64_f64_b64": (64, 768, 21, 64, 64),
    "g16_f128_b256": (256, 768, 13, 16, 128),
    "g32_f128_b96": (96, 512, 11, 32, 128),
    "g64_f32_b33": (33, 96, 17, 64, 32),
    "g32_f32_b1": (1, 64, 9, 32, 32),
    "g32_f64_h1024": (50, 1024, 10, 32, 64),
    # many groups per label chunk: every wave of a dh workgroup gets several
    # groups, so the ordered accumulation and the one-ahead prefetch run
    "g16_f32_many": (64, 256, 4096, 16, 32),
    "g16_f64_many_b40": (40, 512, 3000, 16, 64),
    "g32_f64_many_b100": (100, 768, 3000, 32, 64),
    "g64_f64_many_b70": (70, 768, 1500, 64, 64),
    "g16_f128_many_b130": (130, 768, 1200, 16, 128),
    # batches of 97..128 rows (four 32-row chunks) with small tiles: the
    # fused step without optional outputs runs its chunks in pairs there
    "g32_f64_many_b128": (128, 768, 2000, 32, 64),
    "g16_f64_many_b120": (120, 512, 2500, 16, 64),
    "g32_f32_b97": (97, 256, 300, 32, 32),
    "g16_f32_b128": (128, 128, 40, 16, 32),
    # G = 64 with F = 128: the 16-row feature-gradient kernel with its
    # largest static LDS, first launched at a small H
    "g64_f128_b45": (45, 200, 9, 64, 128),
    # the 32-row feature-gradient kernel with seven waves (G = 16, F = 128)
    # and with six (G = 64, F = 64), each at a small H and a ragged last tile
    "g16_f128_h200_b45": (45, 200, 23, 16, 128),
    "g64_f64_h96_b33": (33, 96, 19, 64, 64),
}

_cache = {}


def labels_mixed(B, L, seed):
    """CSR labels with empty rows, Zipf rows and one row dense in one group."""
    rng = np.random.default_rng(seed)
    rp, cz = zipf_labels(B, L, min(5, L), seed)
    rows = []
    for b in range(B):
        if b % 7 == 3:
            rows.append(np.zeros(0, np.int32))
        elif b % 11 == 5:
            k = rng.integers(0, max(1, L // 16))
            rows.append(np.arange(16 * k, min(L, 16 * k + 16), dtype=np.int32))
        else:
            rows.append(cz[rp[b]:rp[b + 1]])
    rowptr = np.zeros(B + 1, np.int32)
    rowptr[1:] = np.cumsum([r.size for r in rows])
    col = np.concatenate(rows).astype(np.int32) if rowptr[-1] else np.zeros(0, np.int32)
    return rowptr, col


def case(name):
    if name in _cache:
        return _cache[name]
    B, H, K, G, F = CASES[name]
    seed = 100 + sorted(CASES).index(name)
    L = K * G
    d = {
        "B": B, "H": H, "K": K, "G": G, "F": F, "L": L,
        "h": normal_bf16(B * H, 1.0, seed, 1).reshape(B, H),
        "W": normal_bf16(L * F, float(1 / np.sqrt(F)), seed, 2).reshape(L, F),
        "dZ": normal_bf16(B * L, 1.0, seed, 3).reshape(B, L),
        "idx": sorted_subsets(K, F, H, seed, 0),
    }
    d["y_rowptr"], d["y_col"] = labels_mixed(B, L, seed)
    d["scale"] = 1.0 / B
    _cache[name] = d
    return d


def dev_inputs(d):
    return (to_dev_bf16(d["h"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), to_dev_bf16(d["dZ"]),
            to_dev_i32(d["y_rowptr"]), to_dev_i32(d["y_col"] if d["y_col"].size else np.zeros(4, np.int32)))


@pytest.mark.parametrize("name", list(CASES))
def test_fwd(name):
    d = case(name)
    say(f"  fwd {name} {CASES[name]}")
    h, idx, W, _, _, _ = dev_inputs(d)
    Z = to_host(hs.fwd(h, idx, W, d["G"]))
    assert_parity(Z, O.oracle_fwd(d["h"], d["idx"], d["W"], d["G"]), "Z")


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_w(name):
    d = case(name)
    say(f"  bwd_w {name} {CASES[name]}")
    h, idx, _, dZ, _, _ = dev_inputs(d)
    dW = to_host(hs.bwd_w(h, idx, dZ, d["G"]))
    assert_parity(dW, O.oracle_bwd_w(d["h"], d["idx"], d["dZ"], d["G"]), "dW")


@pytest.mark.parametrize("mode", ["atomic", "det"])
@pytest.mark.parametrize("name", list(CASES))
def test_bwd_h(name, mode):
    d = case(name)
    say(f"  bwd_h[{mode}] {name} {CASES[name]}")
    _, idx, W, dZ, _, _ = dev_inputs(d)
    dh = to_host(hs.bwd_h(dZ, idx, W, d["G"], d["H"], mode=mode))
    assert_parity(dh, O.oracle_bwd_h(d["dZ"], d["idx"], d["W"], d["G"], d["H"]), f"dh[{mode}]")


@pytest.mark.parametrize("name", list(CASES))
def test_fwd_bce(name):
    d = case(name)
    say(f"  fwd_bce {name} {CASES[name]}")
    h, idx, W, _, rp, col = dev_inputs(d)
    dZ, Z, loss = hs.fwd_bce(h, idx, W, rp, col, d["scale"], d["G"], want_Z=True, want_loss=True)
    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["scale"], d["G"],
                        want_dW=False, want_dh=False)
    assert_parity(to_host(Z), ref["Z"], "Z")
    dz = to_host(dZ).astype(np.uint32) << 16
    assert_parity(dz.view(np.float32), ref["dZ"], "dZ(bf16)")
    lg = float(to_host(loss)[0])
    say(f"    loss gpu={lg:.9g} oracle={ref['loss']:.9g}")
    assert abs(lg - ref["loss"]) <= 1e-5 * abs(ref["loss"])


@pytest.mark.parametrize("name", ["tiny_4k", "g32_f64_b77", "g32_f64_many_b128", "g16_f64_many_b120", "g32_f32_b97",
                                  "g16_f32_b128", "g16_f128_b256"])
def test_fwd_bce_without_optional_outputs(name):
    d = case(name)
    say(f"  fwd_bce(no Z, no loss) {name} {CASES[name]}")
    h, idx, W, _, rp, col = dev_inputs(d)
    dZ, Z, loss = hs.fwd_bce(h, idx, W, rp, col, d["scale"], d["G"])
    assert Z is None and loss is None
    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["scale"], d["G"],
                        want_dW=False, want_dh=False)
    dz = to_host(dZ).astype(np.uint32) << 16
    assert_parity(dz.view(np.float32), ref["dZ"], "dZ(bf16)")


@pytest.mark.parametrize("mode", ["atomic", "det"])
@pytest.mark.parametrize("name", list(CASES))
def test_step(name, mode):
    d = case(name)
    say(f"  step[{mode}] {name} {CASES[name]}")
    h, idx, W, _, rp, col = dev_inputs(d)
    out = hs.step(h, idx, W, rp, col, d["scale"], d["G"], mode=mode, want_Z=True, want_loss=True)
    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["scale"], d["G"])
    assert_parity(to_host(out["Z"]), ref["Z"], "Z")
    assert_parity(to_host(out["dW"]), ref["dW"], "dW")
    assert_parity(to_host(out["dh"]), ref["dh"], f"dh[{mode}]")
    lg = float(to_host(out["loss"])[0])
    assert abs(lg - ref["loss"]) <= 1e-5 * abs(ref["loss"])


@pytest.mark.parametrize("name", ["tiny_4k", "g32_f64_b77", "g16_f128_b256", "g32_f64_many_b128",
                                  "g16_f64_many_b120", "g32_f32_b97", "g16_f32_b128", "g32_f64_many_b100"])
def test_step_without_optional_outputs(name):
    d = case(name)
    say(f"  step(no Z, no loss) {name}")
    h, idx, W, _, rp, col = dev_inputs(d)
    out = hs.step(h, idx, W, rp, col, d["scale"], d["G"], mode="det")
    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["scale"], d["G"])
    assert_parity(to_host(out["dW"]), ref["dW"], "dW")
    assert_parity(to_host(out["dh"]), ref["dh"], "dh")


# ------------------------------------------------------------ G = 1 baseline

# f64_h1024: the G = 1 dh accumulator (16 x (1024 + 4) fp32) passes the
# default 64 KB of dynamic LDS
# f32_h131: an odd H, so the accumulator flush wraps rows at every step
FIXED = {"f32": (64, 256, 700, 32), "f64_b77": (77, 768, 333, 64), "f128_b256": (256, 768, 150, 128),
         "f64_b1": (1, 96, 65, 64), "f64_h1024": (40, 1024, 200, 64), "f32_h131": (37, 131, 90, 32)}


@pytest.mark.parametrize("mode", ["atomic", "det"])
@pytest.mark.parametrize("name", list(FIXED))
def test_fixed(name, mode):
    B, H, L, F = FIXED[name]
    seed = 300 + sorted(FIXED).index(name)
    say(f"  fixed[{mode}] {name} {FIXED[name]}")
    hb = normal_bf16(B * H, 1.0, seed, 1).reshape(B, H)
    Wb = normal_bf16(L * F, float(1 / np.sqrt(F)), seed, 2).reshape(L, F)
    dZb = normal_bf16(B * L, 1.0, seed, 3).reshape(B, L)
    idx1 = sorted_subsets(L, F, H, seed, 6)
    h, W, dZ, ix = to_dev_bf16(hb), to_dev_bf16(Wb), to_dev_bf16(dZb), to_dev_i32(idx1)
    assert_parity(to_host(hs.fixed_fwd(h, ix, W)), O.oracle_fwd(hb, idx1, Wb, 1), "Z")
    assert_parity(to_host(hs.fixed_bwd_w(h, ix, dZ)), O.oracle_bwd_w(hb, idx1, dZb, 1), "dW")
    assert_parity(to_host(hs.fixed_bwd_h(dZ, ix, W, H, mode=mode)), O.oracle_bwd_h(dZb, idx1, Wb, 1, H),
                  f"dh[{mode}]")


# ------------------------------------------------------ exact index handling

def test_one_hot_probes_bit_exact():
    """h = one-hot column j: Z[:, l] is exactly W[l, f] where I_k[f] = j."""
    B, H, K, G, F = 40, 768, 23, 32, 64
    idxn = sorted_subsets(K, F, H, 77, 0)
    Wb = normal_bf16(K * G * F, 0.125, 77, 2).reshape(K * G, F)
    one = bf16_bits(np.array([1.0], np.float32))[0]
    idx, W = to_dev_i32(idxn), to_dev_bf16(Wb)
    for j in (0, int(idxn[5, 7]), H - 1):
        say(f"  one-hot column {j}")
        hb = np.zeros((B, H), np.uint16)
        hb[:, j] = one
        Z = to_host(hs.fwd(to_dev_bf16(hb), idx, W, G))
        assert_exact(Z, O.oracle_fwd(hb, idxn, Wb, G), f"one-hot Z col {j}")
    rng = np.random.default_rng(3)
    hb = bf16_bits(rng.integers(-4, 5, (B, H)).astype(np.float32))
    for (b, l) in ((0, 0), (B - 1, K * G - 1), (17, 300)):
        say(f"  one-hot dZ[{b},{l}]")
        dZb = np.zeros((B, K * G), np.uint16)
        dZb[b, l] = one
        dZ = to_dev_bf16(dZb)
        assert_exact(to_host(hs.bwd_w(to_dev_bf16(hb), idx, dZ, G)), O.oracle_bwd_w(hb, idxn, dZb, G),
                     "one-hot dW")
        for mode in ("atomic", "det"):
            assert_exact(to_host(hs.bwd_h(dZ, idx, W, G, H, mode=mode)), O.oracle_bwd_h(dZb, idxn, Wb, G, H),
                         f"one-hot dh[{mode}]")


@pytest.mark.parametrize("G,F", [(16, 128), (32, 64), (64, 64)])
def test_all_ones_integer_exact(G, F):
    """h = W = dZ = 1: every fp32 partial sum is an exact integer, so both dh
    modes must equal G * count(j) bit for bit (a lost update or a race would
    show as a wrong integer)."""
    B, H, K = 72, 768, 2000
    say(f"  all-ones G={G} F={F} K={K}")
    idxn = sorted_subsets(K, F, H, 78, 0)
    one = bf16_bits(np.array([1.0], np.float32))[0]
    h = to_dev_bf16(np.full((B, H), one, np.uint16))
    W = to_dev_bf16(np.full((K * G, F), one, np.uint16))
    dZ = to_dev_bf16(np.full((B, K * G), one, np.uint16))
    idx = to_dev_i32(idxn)
    cnt = np.bincount(idxn.ravel(), minlength=H).astype(np.float64)
    assert_exact(to_host(hs.fwd(h, idx, W, G)), np.full((B, K * G), F), "Z")
    assert_exact(to_host(hs.bwd_w(h, idx, dZ, G)), np.full((K * G, F), B), "dW")
    for mode in ("atomic", "det"):
        assert_exact(to_host(hs.bwd_h(dZ, idx, W, G, H, mode=mode)), np.tile(G * cnt, (B, 1)), f"dh[{mode}]")


@pytest.mark.parametrize("mode", ["atomic", "det"])
@pytest.mark.parametrize("name", ["tiny_4k", "g32_f64_many_b128", "g16_f128_many_b130", "g64_f64_h96_b33",
                                  "g32_f64_h1024"])
def test_fwd_bce_bwd(name, mode):
    """haste_fwd_bce_bwd (the interface table's argument order, fp32 loss):
    dW and dh against the oracle, bitwise equal to haste_step's in
    deterministic mode, the loss within 1e-5 of the oracle's."""
    d = case(name)
    say(f"  fwd_bce_bwd[{mode}] {name} {CASES[name]}")
    h, idx, W, _, rp, col = dev_inputs(d)
    out = hs.fwd_bce_bwd(h, idx, W, rp, col, d["scale"], d["G"], mode=mode, want_loss=True)
    ref = O.oracle_step(d["h"], d["idx"], d["W"], d["y_rowptr"], d["y_col"], d["scale"], d["G"])
    dW, dh = to_host(out["dW"]), to_host(out["dh"])
    assert_parity(dW, ref["dW"], "dW")
    assert_parity(dh, ref["dh"], f"dh[{mode}]")
    lg = float(to_host(out["loss"])[0])
    assert abs(lg - ref["loss"]) <= 1e-5 * abs(ref["loss"]), (lg, ref["loss"])
    if mode == "det":
        # same kernels as haste_step with a loss (the loss-carrying epilogue
        # forms sigmoid from e^-|z|, so dZ, and hence dW, differ in the last
        # bits from the pass without one)
        st = hs.step(h, idx, W, rp, col, d["scale"], d["G"], mode="det", want_loss=True)
        assert (to_host(st["dW"]).view(np.uint32) == dW.view(np.uint32)).all()
        assert (to_host(st["dh"]).view(np.uint32) == dh.view(np.uint32)).all()


def test_deterministic_mode_repeats_bitwise():
    d = case("g32_f64_b77")
    h, idx, W, dZ, rp, col = dev_inputs(d)
    a = [to_host(hs.bwd_h(dZ, idx, W, d["G"], d["H"], mode="det")) for _ in range(5)]
    s = [to_host(hs.step(h, idx, W, rp, col, d["scale"], d["G"], mode="det")["dh"]) for _ in range(5)]
    for i in range(1, 5):
        assert (a[i].view(np.uint32) == a[0].view(np.uint32)).all(), "bwd_h det not bitwise repeatable"
        assert (s[i].view(np.uint32) == s[0].view(np.uint32)).all(), "step det not bitwise repeatable"


def test_validators():
    import torch
    H = 100
    idxn = sorted_subsets(50, 32, H, 5, 0)
    assert hs.validate_idx(to_dev_i32(idxn), H) == 0
    bad = idxn.copy()
    bad[3, 4] = H          # out of range
    bad[10, 0], bad[10, 1] = bad[10, 1], bad[10, 0]   # unsorted: a valid set
    bad[20, 6] = bad[20, 5]                            # duplicate
    bad[30, 7] = -1                                    # negative
    assert hs.validate_idx(to_dev_i32(bad), H) == 3
    # F = 128 (two passes of a wave): a repeat across the passes, a shuffled row
    idx2 = sorted_subsets(9, 128, 768, 6, 0)
    idx2[4] = idx2[4][np.random.default_rng(3).permutation(128)]
    assert hs.validate_idx(to_dev_i32(idx2), 768) == 0
    idx2[2, 127] = idx2[2, 3]
    idx2[7, 64] = idx2[7, 63]
    assert hs.validate_idx(to_dev_i32(idx2), 768) == 2
    rp = np.array([0, 2, 2, 5], np.int32)
    col = np.array([1, 9, 0, 4, 7], np.int32)
    assert hs.validate_labels(to_dev_i32(rp), to_dev_i32(col), 10) == 0
    col2 = np.array([9, 1, 0, 4, 12], np.int32)
    assert hs.validate_labels(to_dev_i32(rp), to_dev_i32(col2), 10) == 2
    torch.cuda.synchronize()
