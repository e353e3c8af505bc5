"""GPU parity of the group-level rewiring (haste_rewire) against the CPU
oracle, through the C ABI.  The scores are fp32 on the GPU and fp64 in the
oracle; the selection is integer work, so it is checked bit-exactly by
running the oracle's selection on the GPU's own scores, and against the
oracle's end-to-end result wherever the oracle's decision is not a near
tie.  Integer-valued inputs make every score exact in fp32, which checks
the tie-breaking bit-exactly end to end."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import bf16_bits, get_workload, make_inputs, normal_bf16, sorted_subsets

pytestmark = pytest.mark.gpu

# (B, H, K, G, F, n_swap)
CASES = [
    (64, 256, 37, 16, 32, 5),
    (45, 200, 11, 32, 64, 13),
    (128, 768, 29, 32, 64, 8),
    (77, 768, 9, 64, 64, 64),
    (256, 768, 13, 16, 128, 20),
    (1, 64, 7, 32, 32, 3),
    (160, 1024, 5, 64, 128, 100),
    (33, 96, 17, 64, 32, 0),
    (96, 130, 21, 16, 128, 1),
]


def _inputs(B, H, K, G, F, seed):
    h = normal_bf16(B * H, 1.0, seed, 1).reshape(B, H)
    W = normal_bf16(K * G * F, 0.5, seed, 2).reshape(K * G, F)
    dZ = normal_bf16(B * K * G, 1.0, seed, 3).reshape(B, K * G)
    idx = sorted_subsets(K, F, H, seed, 0)
    return h, dZ, idx, W


def _margin_ok(idx, grow, prune, n, k, rel=1e-4):
    """True when the oracle's drop and grow decisions for group k are not
    near ties (the fp32 scores of the GPU could order them differently)."""
    F = idx.shape[1]
    if n == 0:
        return True
    p = np.sort(prune[k])
    if n < F and p[n] - p[n - 1] <= rel * max(abs(p[n]), 1e-30):
        return False
    order = np.argsort(prune[k], kind="stable")
    kept = set(int(c) for c in idx[k][order[n:]])
    cand = np.array([grow[k, j] for j in range(grow.shape[1]) if j not in kept])
    c = np.sort(cand)[::-1]
    if n < c.size and c[n - 1] - c[n] <= rel * max(abs(c[n - 1]), 1e-30):
        return False
    return True


def _host(out):
    return {k: to_host(v) for k, v in out.items() if v is not None}


def _check(h, dZ, idx, W, G, n, out, what, exact_scores=False):
    """out: host arrays idx, W, grow, prune from the GPU."""
    grow, prune = O.oracle_rewire_scores(h, dZ, idx, W, G)
    g_gpu = out["grow"].astype(np.float64)
    p_gpu = out["prune"].astype(np.float64)
    if exact_scores:
        assert (g_gpu == grow).all() and (p_gpu == prune).all(), f"{what}: integer scores not exact"
    else:
        assert_parity(g_gpu, grow, f"{what} grow", rel=1e-5, mabs=1e-3 * max(1.0, float(np.abs(grow).max())))
        assert_parity(p_gpu, prune, f"{what} prune", rel=1e-6, mabs=1e-4)
    i_gpu, w_gpu = out["idx"], out["W"]
    # the selection, bit-exact, from the GPU's own scores
    i_sel, w_sel = O.oracle_rewire_select(idx, W, g_gpu, p_gpu, n, G)
    assert (i_gpu == i_sel).all(), f"{what}: index rows differ from the selection on the GPU scores"
    assert (w_gpu == w_sel).all(), f"{what}: weights differ from the selection on the GPU scores"
    # end to end against the oracle's own scores, away from near ties
    i_ref, w_ref = O.oracle_rewire_select(idx, W, grow, prune, n, G)
    K = idx.shape[0]
    clear = [k for k in range(K) if _margin_ok(idx, grow, prune, n, k)]
    say(f"    {what}: {len(clear)}/{K} groups without a near tie")
    for k in clear:
        assert (i_gpu[k] == i_ref[k]).all(), f"{what}: group {k} index row"
        assert (w_gpu[k * G:(k + 1) * G] == w_ref[k * G:(k + 1) * G]).all(), f"{what}: group {k} weights"
    # invariants that hold for every group
    assert (np.diff(i_gpu, axis=1) > 0).all() and i_gpu.min() >= 0 and i_gpu.max() < h.shape[1]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}_h{c[1]}_k{c[2]}_g{c[3]}_f{c[4]}_n{c[5]}" for c in CASES])
def test_rewire(case):
    B, H, K, G, F, n = case
    say(f"  rewire B={B} H={H} K={K} G={G} F={F} n={n}")
    h, dZ, idx, W = _inputs(B, H, K, G, F, 40 + K)
    out = _host(hs.rewire(to_dev_bf16(h), to_dev_bf16(dZ), to_dev_i32(idx), to_dev_bf16(W), G, n,
                          want_scores=True))
    _check(h, dZ, idx, W, G, n, out, "rewire")


@pytest.mark.parametrize("G,F", [(16, 32), (32, 64), (64, 128)])
def test_rewire_integer_inputs_exact(G, F):
    """Small-integer h, dZ, W: every score is an exact fp32 integer, so
    scores, ties and the whole result match the oracle bit for bit."""
    B, H, K, n = 70, 300, 19, F // 4
    rng = np.random.default_rng(50 + G)
    h = bf16_bits(rng.integers(-2, 3, size=(B, H)).astype(np.float32))
    dZ = bf16_bits(rng.integers(-1, 2, size=(B, K * G)).astype(np.float32))
    W = bf16_bits(rng.integers(-2, 3, size=(K * G, F)).astype(np.float32))
    idx = sorted_subsets(K, F, H, 50 + G, 0)
    out = _host(hs.rewire(to_dev_bf16(h), to_dev_bf16(dZ), to_dev_i32(idx), to_dev_bf16(W), G, n,
                          want_scores=True))
    _check(h, dZ, idx, W, G, n, out, "integer", exact_scores=True)
    i_ref, w_ref = O.oracle_rewire_select(idx, W, *O.oracle_rewire_scores(h, dZ, idx, W, G), n, G)
    assert (out["idx"] == i_ref).all() and (out["W"] == w_ref).all()


def test_rewire_in_place_and_repeatable():
    B, H, K, G, F, n = 100, 768, 40, 32, 64, 16
    h, dZ, idx, W = _inputs(B, H, K, G, F, 60)
    hd, dzd = to_dev_bf16(h), to_dev_bf16(dZ)
    a = hs.rewire(hd, dzd, to_dev_i32(idx), to_dev_bf16(W), G, n, want_scores=True)
    b = hs.rewire(hd, dzd, to_dev_i32(idx), to_dev_bf16(W), G, n, want_scores=True)
    assert (to_host(a["grow"]).view(np.uint32) == to_host(b["grow"]).view(np.uint32)).all(), "grow not repeatable"
    idx_d, W_d = to_dev_i32(idx), to_dev_bf16(W)
    c = hs.rewire(hd, dzd, idx_d, W_d, G, n, idx_out=idx_d, W_out=W_d)
    assert c["idx"].data_ptr() == idx_d.data_ptr()
    assert (to_host(idx_d) == to_host(a["idx"])).all(), "in-place index rows differ"
    assert (to_host(W_d) == to_host(a["W"])).all(), "in-place weights differ"


def test_rewire_rejects_bad_arguments():
    B, H, K, G, F = 8, 64, 3, 16, 32
    h, dZ, idx, W = _inputs(B, H, K, G, F, 61)
    hd, dzd, idd, Wd = to_dev_bf16(h), to_dev_bf16(dZ), to_dev_i32(idx), to_dev_bf16(W)
    for n in (-1, F + 1):
        with pytest.raises(hs.HasteError):
            hs.rewire(hd, dzd, idd, Wd, G, n)
    # an output that overlaps its input without being the same range
    import torch
    big = torch.empty(K * F + 8, dtype=torch.int32, device=idd.device)
    big[:K * F] = idd.view(-1)
    with pytest.raises(hs.HasteError):
        hs.rewire(hd, dzd, big[:K * F].view(K, F), Wd, G, 2, idx_out=big[4:4 + K * F].view(K, F))


def _slice_labels(d, k0, k1, G):
    return np.ascontiguousarray(d["dZ"][:, k0 * G:k1 * G])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_rewire_fullsize_sampled():
    """The Amazon-3M shape (K = 93,748 groups of G = 32, F = 64, H = 768,
    B = 128) with n_swap = 16, in the benchmark's configuration: scores and
    the selection on sampled group slices against the oracle."""
    w = get_workload("amazon3m_shaped")
    say(f"  generating {w.name}")
    d = make_inputs(w, dZ=True, labels=False)
    G, K, n = w.G, w.K, 16
    out = _host(hs.rewire(to_dev_bf16(d["h"]), to_dev_bf16(d["dZ"]), to_dev_i32(d["idx"]), to_dev_bf16(d["W"]), G,
                          n, want_scores=True))
    for k0 in (0, K // 2, K - 48):
        k1 = k0 + 48
        idx = np.ascontiguousarray(d["idx"][k0:k1])
        W = np.ascontiguousarray(d["W"][k0 * G:k1 * G])
        sub = {"grow": out["grow"][k0:k1], "prune": out["prune"][k0:k1], "idx": out["idx"][k0:k1],
               "W": out["W"][k0 * G:k1 * G]}
        _check(d["h"], _slice_labels(d, k0, k1, G), idx, W, G, n, sub, f"groups [{k0},{k1})")

