"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin_* function takes a loaded oracle library (ctypes) and raises
AssertionError when the oracle disagrees with the fact it checks.  The pins
are used twice: once on the real oracle (test_oracle_pins.py) and once on
copies of the oracle with a planted mistake (test_oracle_mutants.py), which
must each fail at least one pin.

What pins what:
  hand examples (tests/golden)  fwd, bwd_w, bwd_h, bce, loss: values computed by hand
  dense special case F=H        fwd, bwd_w, bwd_h == numpy matmul
  brute-force masked dense      fwd, bwd_w, bwd_h via an L x H matrix with zeros
  one-hot probes                index handling, exact
  all-ones integer case         closed forms Z=F, dW=B, dh=G*count(j)
  finite differences            bwd_w, bwd_h == exact differences of <dZ, fwd>
  permutation invariance        group order and slot order conventions
  torch autograd                dZ, dW, dh, loss == autograd of forward+BCE
  BCE closed form (W = 0)       dZ = s(1/2 - Y), loss = s*B*L*ln 2
  G=1 special case              per-label fixed fan-in dot products
  head == tail oracle at F = H  dense head (numpy) == group-shared oracle (C) with I_k = [0, H)
  head BCE closed form (W = 0)  head dZ, dW, dh = 0, loss
  joint torch autograd          joint head + tail dW_tail, dW_head, dh, loss == autograd
                                of both branches' BCE with separate scales
  rewire scores via autograd    grow score == |dense gradient| (torch autograd) summed per group,
                                prune score == |W| summed per group (plain loops)
  rewire brute force            drop / grow sets == the best n-subsets found by enumeration
  rewire special cases          n = 0 identity, all-slots swap, ties, a planted strongest column
  E4M3 codec vs torch           decode of all 256 codes and encode of random, midpoint and
                                subnormal values == torch.float8_e4m3fn (a library routine)
  E4M3 hand values              codes of 1, 448, 2^-9, -2, ties to even
  FP8 group scales              e_k minimal, dequantized weights exact in bf16, within the
                                format's rounding bound of W, and encoding back to their codes
  k-means assignment            brute-force loops over centres, ties to the lowest centre
  k-means update                Sculley's per-sample rule (loops) == the closed form; full-batch
                                steps from zero counts never lower the objective (Lloyd)
  greedy grouping               planted clumps recovered exactly; partition and leftover rules
  slot order                    hand-worked rows (tests/golden); every row a permutation with W's
                                columns moved along; repeated keys per run == the lower bound
                                sum_v max(0, count_v - F/8), which brute force over all splits of
                                16 slots into two runs confirms is the least possible
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import oracle as O
from synthetic import bf16_bits, bf16_value, normal_bf16, sorted_subsets

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EXACT = 0.0


def _f(bits):
    return bf16_value(bits).astype(np.float64)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    ok = err <= atol + rtol * np.abs(b)
    assert ok.all(), f"{what}: max abs err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"


def _rand_case(B, H, K, G, F, seed):
    h = normal_bf16(B * H, 1.0, seed, 1).reshape(B, H)
    W = normal_bf16(K * G * F, 0.5, seed, 2).reshape(K * G, F)
    dZ = normal_bf16(B * K * G, 1.0, seed, 3).reshape(B, K * G)
    idx = sorted_subsets(K, F, H, seed, 0)
    return h, idx, W, dZ


def _small_int_bf16(shape, rng, lo=-3, hi=4):
    return bf16_bits(rng.integers(lo, hi, size=shape).astype(np.float32))


# --------------------------------------------------------------------------

def pin_hand_example(lib):
    with open(os.path.join(GOLDEN, "hand_example_b2_h4_k2_g2_f2.json")) as fh:
        g = json.load(fh)
    s = g["shape"]
    h = bf16_bits(np.array(g["h"], np.float32))
    W = bf16_bits(np.array(g["W"], np.float32))
    dZ = bf16_bits(np.array(g["dZ"], np.float32))
    idx = np.array(g["idx"], np.int32)
    Z = O.oracle_fwd(h, idx, W, s["G"], lib=lib)
    dW = O.oracle_bwd_w(h, idx, dZ, s["G"], lib=lib)
    dh = O.oracle_bwd_h(dZ, idx, W, s["G"], s["H"], lib=lib)
    _close(Z, g["Z"], 0, EXACT, "hand Z")
    _close(dW, g["dW"], 0, EXACT, "hand dW")
    _close(dh, g["dh"], 0, EXACT, "hand dh")


def pin_bce_hand_example(lib):
    with open(os.path.join(GOLDEN, "bce_hand_example_b2_l2.json")) as fh:
        g = json.load(fh)
    Z = np.array(g["Z"], np.float64)
    dZ, loss = O.oracle_bce(Z, np.array(g["y_rowptr"], np.int32), np.array(g["y_col"], np.int32),
                            g["scale"], lib=lib)
    _close(dZ, g["dZ"], 1e-14, 1e-15, "bce hand dZ")
    assert abs(loss - g["loss"]) < 1e-12, f"bce hand loss {loss} vs {g['loss']}"


def pin_dense_special_case(lib):
    """F = H and every I_k = [0, H): the layer is a dense linear map."""
    B, H, K, G = 5, 24, 3, 4
    F = H
    h, _, W, dZ = _rand_case(B, H, K, G, F, 11)
    idx = np.tile(np.arange(H, dtype=np.int32), (K, 1))
    hf, Wf, dZf = _f(h), _f(W), _f(dZ)
    _close(O.oracle_fwd(h, idx, W, G, lib=lib), hf @ Wf.T, what="dense Z")
    _close(O.oracle_bwd_w(h, idx, dZ, G, lib=lib), dZf.T @ hf, what="dense dW")
    _close(O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib), dZf @ Wf, what="dense dh")


def pin_brute_force_masked_dense(lib):
    """Materialise the sparse layer as an L x H matrix and use matmul."""
    B, H, K, G, F = 6, 40, 5, 3, 7
    h, idx, W, dZ = _rand_case(B, H, K, G, F, 12)
    L = K * G
    hf, Wf, dZf = _f(h), _f(W), _f(dZ)
    Wd = np.zeros((L, H))
    M = np.zeros((L, H), dtype=np.int64)
    for l in range(L):
        for f in range(F):
            Wd[l, idx[l // G, f]] = Wf[l, f]
            M[l, idx[l // G, f]] += 1
    assert (M.sum(1) == F).all() and (M <= 1).all()
    for k in range(K):
        assert (M[k * G:(k + 1) * G] == M[k * G]).all()
    dWd = dZf.T @ hf
    dW_ref = np.array([[dWd[l, idx[l // G, f]] for f in range(F)] for l in range(L)])
    _close(O.oracle_fwd(h, idx, W, G, lib=lib), hf @ Wd.T, what="brute Z")
    _close(O.oracle_bwd_w(h, idx, dZ, G, lib=lib), dW_ref, what="brute dW")
    _close(O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib), dZf @ Wd, what="brute dh")


def pin_one_hot_probes(lib):
    """A one-hot feature column or gradient entry selects single products."""
    B, H, K, G, F = 4, 32, 6, 2, 5
    _, idx, W, _ = _rand_case(B, H, K, G, F, 13)
    L = K * G
    Wf = _f(W)
    one = bf16_bits(np.array([1.0], np.float32))[0]
    for j in (0, 7, H - 1):
        h = np.zeros((B, H), np.uint16)
        h[:, j] = one
        Z = O.oracle_fwd(h, idx, W, G, lib=lib)
        exp = np.zeros((B, L))
        for l in range(L):
            hit = np.nonzero(idx[l // G] == j)[0]
            if hit.size:
                exp[:, l] = Wf[l, hit[0]]
        _close(Z, exp, 0, EXACT, f"one-hot Z j={j}")
    rng = np.random.default_rng(5)
    h = _small_int_bf16((B, H), rng)
    hf = _f(h)
    for (b, l) in ((0, 0), (B - 1, L - 1), (2, 5)):
        dZ = np.zeros((B, L), np.uint16)
        dZ[b, l] = one
        k = l // G
        dW = O.oracle_bwd_w(h, idx, dZ, G, lib=lib)
        expw = np.zeros((L, F))
        expw[l] = hf[b, idx[k]]
        _close(dW, expw, 0, EXACT, f"one-hot dW {(b, l)}")
        dh = O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib)
        exph = np.zeros((B, H))
        exph[b, idx[k]] = Wf[l]
        _close(dh, exph, 0, EXACT, f"one-hot dh {(b, l)}")


def pin_all_ones(lib):
    """h = W = dZ = 1: Z = F, dW = B, dh[b, j] = G * #{k : j in I_k}."""
    B, H, K, G, F = 3, 50, 9, 4, 6
    _, idx, _, _ = _rand_case(B, H, K, G, F, 14)
    L = K * G
    one = bf16_bits(np.array([1.0], np.float32))[0]
    h = np.full((B, H), one, np.uint16)
    W = np.full((L, F), one, np.uint16)
    dZ = np.full((B, L), one, np.uint16)
    cnt = np.bincount(idx.ravel(), minlength=H).astype(np.float64)
    _close(O.oracle_fwd(h, idx, W, G, lib=lib), np.full((B, L), F), 0, EXACT, "ones Z")
    _close(O.oracle_bwd_w(h, idx, dZ, G, lib=lib), np.full((L, F), B), 0, EXACT, "ones dW")
    _close(O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib), np.tile(G * cnt, (B, 1)), 0, EXACT, "ones dh")


def pin_finite_differences(lib):
    """S(h, W) = <dZ, fwd(h, W)> is bilinear, so S(h + e_bj) - S(h) = dh[b, j]
    and S(W + e_lf) - S(W) = dW[l, f] exactly (integer-valued inputs, fp64)."""
    B, H, K, G, F = 3, 20, 4, 3, 5
    rng = np.random.default_rng(6)
    _, idx, _, _ = _rand_case(B, H, K, G, F, 15)
    L = K * G
    h = _small_int_bf16((B, H), rng)
    W = _small_int_bf16((L, F), rng)
    dZ = _small_int_bf16((B, L), rng)
    dZf = _f(dZ)

    def S(hh, WW):
        return float((dZf * O.oracle_fwd(hh, idx, WW, G, lib=lib)).sum())

    base = S(h, W)
    dh = O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib)
    dW = O.oracle_bwd_w(h, idx, dZ, G, lib=lib)
    for (b, j) in ((0, int(idx[0, 0])), (B - 1, int(idx[K - 1, F - 1])), (1, int(idx[2, 2]))):
        h2 = h.copy()
        h2[b, j] = bf16_bits(np.array([_f(h[b:b + 1, j:j + 1])[0, 0] + 1.0], np.float32))[0]
        assert S(h2, W) - base == dh[b, j], f"fd dh[{b},{j}]"
    for (l, f) in ((0, 0), (L - 1, F - 1), (4, 3)):
        W2 = W.copy()
        W2[l, f] = bf16_bits(np.array([_f(W[l:l + 1, f:f + 1])[0, 0] + 1.0], np.float32))[0]
        assert S(h, W2) - base == dW[l, f], f"fd dW[{l},{f}]"


def pin_permutation_invariance(lib):
    B, H, K, G, F = 4, 30, 5, 3, 6
    h, idx, W, dZ = _rand_case(B, H, K, G, F, 16)
    L = K * G
    rng = np.random.default_rng(7)
    Z = O.oracle_fwd(h, idx, W, G, lib=lib)
    dW = O.oracle_bwd_w(h, idx, dZ, G, lib=lib)
    dh = O.oracle_bwd_h(dZ, idx, W, G, H, lib=lib)
    # group order
    p = rng.permutation(K)
    lp = (p[:, None] * G + np.arange(G)[None, :]).ravel()
    idx2 = np.ascontiguousarray(idx[p])
    W2 = np.ascontiguousarray(W[lp])
    dZ2 = np.ascontiguousarray(dZ[:, lp])
    _close(O.oracle_fwd(h, idx2, W2, G, lib=lib), Z[:, lp], what="perm-group Z")
    _close(O.oracle_bwd_w(h, idx2, dZ2, G, lib=lib), dW[lp], what="perm-group dW")
    _close(O.oracle_bwd_h(dZ2, idx2, W2, G, H, lib=lib), dh, what="perm-group dh")
    # slot order inside each group (index row and the G weight rows together)
    sig = np.stack([rng.permutation(F) for _ in range(K)])
    idx3 = np.ascontiguousarray(np.take_along_axis(idx, sig, 1))
    W3 = np.ascontiguousarray(np.take_along_axis(W, np.repeat(sig, G, 0), 1))
    _close(O.oracle_fwd(h, idx3, W3, G, lib=lib), Z, what="perm-slot Z")
    _close(O.oracle_bwd_w(h, idx3, dZ, G, lib=lib), np.take_along_axis(dW, np.repeat(sig, G, 0), 1),
           what="perm-slot dW")
    _close(O.oracle_bwd_h(dZ, idx3, W3, G, H, lib=lib), dh, what="perm-slot dh")


def pin_bce_zero_weights(lib):
    """W = 0 gives Z = 0, sigmoid = 1/2, dZ = s(1/2 - Y), loss = s*B*L*ln 2."""
    B, H, K, G, F = 4, 16, 3, 4, 5
    h, idx, _, _ = _rand_case(B, H, K, G, F, 17)
    L = K * G
    W = np.zeros((L, F), np.uint16)
    rowptr = np.array([0, 2, 2, 5, 6], np.int32)
    col = np.array([1, 7, 0, 3, 11, 5], np.int32)
    s = 1.0 / B
    r = O.oracle_step(h, idx, W, rowptr, col, s, G, lib=lib)
    Y = np.zeros((B, L))
    for b in range(B):
        Y[b, col[rowptr[b]:rowptr[b + 1]]] = 1
    _close(r["Z"], np.zeros((B, L)), 0, EXACT, "bce0 Z")
    _close(r["dZ"], s * (0.5 - Y), 0, EXACT, "bce0 dZ")
    assert abs(r["loss"] - s * B * L * math.log(2.0)) < 1e-12, "bce0 loss"


def pin_torch_autograd(lib):
    """dZ, dW, dh and the loss equal torch autograd of forward + BCE (fp64, CPU)."""
    import torch

    B, H, K, G, F = 5, 36, 6, 4, 8
    h, idx, W, _ = _rand_case(B, H, K, G, F, 18)
    L = K * G
    rowptr = np.array([0, 3, 4, 4, 7, 9], np.int32)
    col = np.array([0, 5, 23, 9, 1, 2, 17, 8, 20], np.int32)
    s = 1.0 / B
    r = O.oracle_step(h, idx, W, rowptr, col, s, G, lib=lib)
    ht = torch.tensor(_f(h), requires_grad=True)
    Wt = torch.tensor(_f(W), requires_grad=True)
    it = torch.tensor(idx.astype(np.int64))
    Hg = ht[:, it]                                        # B x K x F
    Zt = torch.einsum("bkf,kgf->bkg", Hg, Wt.reshape(K, G, F)).reshape(B, L)
    Zt.retain_grad()
    Y = torch.zeros(B, L, dtype=torch.float64)
    for b in range(B):
        Y[b, torch.tensor(col[rowptr[b]:rowptr[b + 1]].astype(np.int64))] = 1
    loss = torch.nn.functional.binary_cross_entropy_with_logits(Zt, Y, reduction="sum") * s
    loss.backward()
    _close(r["Z"], Zt.detach().numpy(), 1e-12, 1e-12, "autograd Z")
    _close(r["dZ"], Zt.grad.numpy(), 1e-10, 1e-14, "autograd dZ")
    _close(r["dW"], Wt.grad.numpy(), 1e-10, 1e-13, "autograd dW")
    _close(r["dh"], ht.grad.numpy(), 1e-10, 1e-13, "autograd dh")
    assert abs(r["loss"] - loss.item()) < 1e-10 * abs(loss.item()), "autograd loss"


def pin_g1_per_label(lib):
    """G = 1: every label has its own index set; z = per-label dot product."""
    B, H, L, F = 4, 25, 9, 6
    h = normal_bf16(B * H, 1.0, 19, 1).reshape(B, H)
    W = normal_bf16(L * F, 0.5, 19, 2).reshape(L, F)
    dZ = normal_bf16(B * L, 1.0, 19, 3).reshape(B, L)
    idx1 = sorted_subsets(L, F, H, 19, 6)
    hf, Wf, dZf = _f(h), _f(W), _f(dZ)
    gathered = hf[:, idx1]                                  # B x L x F
    Z_ref = np.einsum("blf,lf->bl", gathered, Wf)
    dW_ref = np.einsum("bl,blf->lf", dZf, gathered)
    dh_ref = np.zeros((B, H))
    for b in range(B):
        np.add.at(dh_ref[b], idx1.ravel(), (dZf[b][:, None] * Wf).ravel())
    _close(O.oracle_fwd(h, idx1, W, 1, lib=lib), Z_ref, what="G1 Z")
    _close(O.oracle_bwd_w(h, idx1, dZ, 1, lib=lib), dW_ref, what="G1 dW")
    _close(O.oracle_bwd_h(dZ, idx1, W, 1, H, lib=lib), dh_ref, what="G1 dh")


def _labels_dense(rowptr, col, B, L):
    Y = np.zeros((B, L))
    for b in range(B):
        Y[b, col[rowptr[b]:rowptr[b + 1]]] = 1
    return Y


def pin_head_dense_equals_tail_oracle(lib):
    """The dense head is the group-shared layer with F = H and every I_k =
    [0, H): the numpy head oracle equals the C oracle on that layer."""
    B, H, K, G = 6, 10, 3, 4
    L = K * G
    h = normal_bf16(B * H, 1.0, 21, 1).reshape(B, H)
    W = normal_bf16(L * H, 0.5, 21, 2).reshape(L, H)
    rowptr = np.array([0, 2, 3, 3, 6, 8, 9], np.int32)
    col = np.array([0, 11, 4, 1, 2, 7, 5, 9, 3], np.int32)
    s = 1.0 / B
    idx = np.tile(np.arange(H, dtype=np.int32), (K, 1))
    t = O.oracle_step(h, idx, W, rowptr, col, s, G, lib=lib)
    hd = O.oracle_head_step(h, W, rowptr, col, s, lib=lib)
    for k in ("Z", "dZ", "dW", "dh"):
        _close(hd[k], t[k], what=f"head vs tail oracle {k}")
    assert abs(hd["loss"] - t["loss"]) <= 1e-12 * abs(t["loss"]), "head vs tail oracle loss"


def pin_head_zero_weights(lib):
    """W_head = 0: Z = 0, dZ = s(1/2 - Y), dW = dZ^T h, dh = 0, loss = s*B*L*ln 2."""
    B, H, L = 5, 7, 9
    h = normal_bf16(B * H, 1.0, 22, 1).reshape(B, H)
    W = np.zeros((L, H), np.uint16)
    rowptr = np.array([0, 1, 4, 4, 5, 7], np.int32)
    col = np.array([8, 0, 3, 5, 2, 1, 8], np.int32)
    s = 0.25
    r = O.oracle_head_step(h, W, rowptr, col, s, lib=lib)
    Y = _labels_dense(rowptr, col, B, L)
    dZ = s * (0.5 - Y)
    _close(r["Z"], np.zeros((B, L)), 0, EXACT, "head0 Z")
    _close(r["dZ"], dZ, 0, EXACT, "head0 dZ")
    _close(r["dh"], np.zeros((B, H)), 0, EXACT, "head0 dh")
    hf = _f(h)
    dW = np.array([[sum(dZ[b, l] * hf[b, j] for b in range(B)) for j in range(H)] for l in range(L)])
    _close(r["dW"], dW, 1e-14, 1e-15, "head0 dW")
    assert abs(r["loss"] - s * B * L * math.log(2.0)) < 1e-12, "head0 loss"


def pin_joint_torch_autograd(lib):
    """Joint head + tail pass == torch autograd (fp64, CPU) of
    s_t BCE(tail logits, Y_t) + s_h BCE(h W_head^T, Y_h), with the tail as a
    masked dense L x H matrix (distinct scales pin which branch gets which)."""
    import torch

    B, H, K, G, F, Lh = 5, 20, 4, 3, 6, 7
    Lt = K * G
    h, idx, Wt, _ = _rand_case(B, H, K, G, F, 23)
    Wh = normal_bf16(Lh * H, 0.5, 23, 7).reshape(Lh, H)
    yt_rp = np.array([0, 2, 2, 3, 5, 6], np.int32)
    yt_col = np.array([1, 10, 4, 0, 11, 6], np.int32)
    yh_rp = np.array([0, 1, 3, 3, 4, 6], np.int32)
    yh_col = np.array([6, 0, 2, 5, 1, 3], np.int32)
    st, sh = 0.2, 0.35
    r = O.oracle_joint_step(h, idx, Wt, yt_rp, yt_col, Wh, yh_rp, yh_col, st, sh, G, lib=lib)
    ht = torch.tensor(_f(h), requires_grad=True)
    Wd = torch.zeros(Lt, H, dtype=torch.float64)
    for l in range(Lt):
        Wd[l, torch.tensor(idx[l // G].astype(np.int64))] = torch.tensor(_f(Wt)[l])
    Wd.requires_grad_(True)
    Wht = torch.tensor(_f(Wh), requires_grad=True)
    Yt = torch.tensor(_labels_dense(yt_rp, yt_col, B, Lt))
    Yh = torch.tensor(_labels_dense(yh_rp, yh_col, B, Lh))
    bce = torch.nn.functional.binary_cross_entropy_with_logits
    loss = st * bce(ht @ Wd.T, Yt, reduction="sum") + sh * bce(ht @ Wht.T, Yh, reduction="sum")
    loss.backward()
    dWt_ref = np.stack([Wd.grad.numpy()[l, idx[l // G]] for l in range(Lt)])
    _close(r["dW_tail"], dWt_ref, 1e-10, 1e-13, "joint dW_tail")
    _close(r["dW_head"], Wht.grad.numpy(), 1e-10, 1e-13, "joint dW_head")
    _close(r["dh"], ht.grad.numpy(), 1e-10, 1e-13, "joint dh")
    assert abs(r["loss"] - loss.item()) < 1e-10 * abs(loss.item()), "joint loss"


def pin_rewire_scores_autograd(lib):
    """grow[k, j] = sum over the group's labels of |d<dZ, h W_dense^T>/dW_dense[l, j]|
    with the gradient from torch autograd on a dense L x H weight matrix;
    prune[k, f] = sum over the group's labels of |W[l, f]| by plain loops."""
    import torch

    B, H, K, G, F = 6, 14, 3, 4, 5
    h, idx, W, dZ = _rand_case(B, H, K, G, F, 24)
    grow, prune = O.oracle_rewire_scores(h, dZ, idx, W, G)
    Wd = torch.zeros(K * G, H, dtype=torch.float64, requires_grad=True)
    S = (torch.tensor(_f(dZ)) * (torch.tensor(_f(h)) @ Wd.T)).sum()
    S.backward()
    g = Wd.grad.numpy()
    want = np.array([[sum(abs(g[k * G + i, j]) for i in range(G)) for j in range(H)] for k in range(K)])
    _close(grow, want, 1e-12, 1e-13, "rewire grow score")
    wf = _f(W)
    want_p = np.array([[sum(abs(wf[k * G + i, f]) for i in range(G)) for f in range(F)] for k in range(K)])
    _close(prune, want_p, 0, EXACT, "rewire prune score")


def pin_rewire_brute_force(lib):
    """With distinct scores the dropped slots are the n-subset of I_k with
    the smallest total prune score and the grown columns the n-subset of the
    non-kept columns with the largest total grow score (enumerated)."""
    import itertools

    rng = np.random.default_rng(25)
    K, G, F, H = 6, 2, 4, 9
    for n in (1, 2, 3, 4):
        idx = np.stack([np.sort(rng.choice(H, F, replace=False)) for _ in range(K)]).astype(np.int32)
        W = bf16_bits(rng.normal(size=(K * G, F)).astype(np.float32))
        prune = rng.permutation(K * F).reshape(K, F).astype(np.float64)
        grow = rng.permutation(K * H).reshape(K, H).astype(np.float64)
        # make a dropped column the strongest grower in group 0: it must come back
        f_low = int(np.argmin(prune[0]))
        grow[0, idx[0, f_low]] = 10.0 * K * H
        idx_new, W_new = O.oracle_rewire_select(idx, W, grow, prune, n, G)
        for k in range(K):
            cols = list(idx[k])
            drop = min(itertools.combinations(range(F), n), key=lambda c: sum(prune[k, f] for f in c))
            kept = [cols[f] for f in range(F) if f not in drop]
            cand = [j for j in range(H) if j not in kept]
            add = max(itertools.combinations(cand, n), key=lambda c: sum(grow[k, j] for j in c))
            want = sorted(kept + list(add))
            assert list(idx_new[k]) == want, f"rewire brute force n={n} k={k}: {list(idx_new[k])} vs {want}"
            for f_new, c in enumerate(want):
                src = W[k * G:(k + 1) * G, cols.index(c)] if c in kept else np.zeros(G, np.uint16)
                assert (W_new[k * G:(k + 1) * G, f_new] == src).all(), f"rewire weights n={n} k={k} col {c}"
        assert idx[0, f_low] in idx_new[0], "a dropped column with the top grow score must be regrown"


def pin_rewire_special_cases(lib):
    """n = 0 changes nothing; n = F with H = F regrows every column at zero
    weight; equal scores drop and grow the lowest column ids; a planted
    feature/gradient pair makes one column the strongest grower."""
    B, H, K, G, F = 5, 12, 3, 4, 4
    h, idx, W, dZ = _rand_case(B, H, K, G, F, 26)
    i0, w0, _, _ = O.oracle_rewire(h, dZ, idx, W, 0, G)
    assert (i0 == idx).all() and (w0 == W).all(), "n = 0 must be the identity"
    # H = F: the only candidates are the dropped columns themselves
    idx_d = np.tile(np.arange(F, dtype=np.int32), (K, 1))
    hd = h[:, :F].copy()
    i1, w1, _, _ = O.oracle_rewire(hd, dZ, idx_d, W, F, G)
    assert (i1 == idx_d).all() and (w1 == 0).all(), "full swap at H = F"
    # ties: equal prune and grow scores everywhere
    prune = np.ones((K, F))
    grow = np.ones((K, H))
    i2, w2 = O.oracle_rewire_select(idx, W, grow, prune, 2, G)
    for k in range(K):
        kept = sorted(idx[k])[2:]
        add = [j for j in range(H) if j not in kept][:2]
        assert list(i2[k]) == sorted(kept + add), f"tie-break, group {k}"
    # planted case: only label 1 of group 1 has a gradient, and only through
    # feature column j*, which group 1 does not use; slot 2 of group 1 has
    # the smallest weights
    jstar = [j for j in range(H) if j not in idx[1]][0]
    hp = np.zeros((B, H), np.uint16)
    hp[:, jstar] = bf16_bits(np.full(B, 2.0, np.float32))
    hp[:, (jstar + 1) % H] = bf16_bits(np.full(B, 0.5, np.float32))
    dZp = np.zeros_like(dZ)
    dZp[:, 1 * G + 1] = bf16_bits(np.linspace(0.5, 1.5, B).astype(np.float32))
    Wp = bf16_bits(np.full((K * G, F), 1.0, np.float32))
    Wp[1 * G:2 * G, 2] = bf16_bits(np.full(G, 0.125, np.float32))
    i3, w3, grow3, _ = O.oracle_rewire(hp, dZp, idx, Wp, 1, G)
    assert abs(grow3[1, jstar] - 2.0 * np.linspace(0.5, 1.5, B).astype(np.float32).astype(np.float64).sum()) < 1e-9
    want = sorted([c for f, c in enumerate(idx[1]) if f != 2] + [jstar])
    assert list(i3[1]) == want, "planted strongest column must replace the weakest slot"
    f_new = want.index(jstar)
    assert (w3[G:2 * G, f_new] == 0).all() and (w3[G:2 * G] != 0).sum() == G * (F - 1)


def pin_e4m3_codec_torch(lib):
    """The E4M3 codec against torch's float8_e4m3fn conversion (CPU)."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "E4M3 NaN codes"
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]), "E4M3 decode"
    rng = np.random.default_rng(27)
    finite = np.sort(np.unique(got[fin & (got >= 0)]))
    mids = (finite[1:] + finite[:-1]) / 2                      # exact ties
    vals = np.concatenate([
        rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000), rng.normal(0, 2.0 ** -7, 2000),
        mids, -mids, finite, -finite, [0.0, -0.0, 448.0, -448.0],
    ]).astype(np.float32).astype(np.float64)                   # fp32-exact inputs
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    enc = O.e4m3_encode(vals)
    bad = np.nonzero(enc != want)[0]
    assert bad.size == 0, f"E4M3 encode: {bad.size} differ, e.g. {vals[bad[:3]]} -> {enc[bad[:3]]} vs {want[bad[:3]]}"


def pin_e4m3_hand_values(lib):
    """1 = 0x38, 448 = 0x7E, 2^-9 = 0x01, 2^-6 = 0x08, -2 = 0xC0, 0 = 0x00;
    1.0625 lies halfway between 1 (0x38) and 1.125 (0x39): the even code
    0x38; 1.1875 halfway between 0x39 and 0x3A (1.25): 0x3A."""
    vals = np.array([1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -2.0, 0.0, 1.0625, 1.1875])
    want = np.array([0x38, 0x7E, 0x01, 0x08, 0xC0, 0x00, 0x38, 0x3A], np.uint8)
    assert np.array_equal(O.e4m3_encode(vals), want), "E4M3 hand values"
    assert np.array_equal(O.e4m3_decode(want[:6]), vals[:6]), "E4M3 hand decode"


def pin_w8_group_scales(lib):
    """e_k is the smallest integer with max|W_k| 2^-e_k <= 448; the
    dequantized weights are exact bf16 values within the E4M3 rounding bound
    of W (relative 2^-4 in the normal range, 2^(e_k-10) absolute below)."""
    K, G, F = 40, 16, 32
    rng = np.random.default_rng(28)
    mag = 2.0 ** rng.integers(-12, 12, size=K)
    W = bf16_bits((rng.normal(size=(K * G, F)) * np.repeat(mag, G)[:, None]).astype(np.float32))
    W[:G] = 0                                                  # an all-zero group
    W8, e = O.oracle_quantize_w8(W, G)
    wf = _f(W)
    mx = np.abs(wf).reshape(K, -1).max(axis=1)
    for k in range(K):
        if mx[k] == 0:
            assert e[k] == 0
            continue
        assert mx[k] * 2.0 ** -int(e[k]) <= 448.0 < mx[k] * 2.0 ** -(int(e[k]) - 1), f"group {k} exponent"
    deq = _f(O.oracle_dequantize_w8(W8, e, G))
    sc = np.repeat(2.0 ** e.astype(np.float64), G)[:, None]
    normal = np.abs(wf) >= 2.0 ** -6 * sc
    err = np.abs(deq - wf)
    assert (err[normal] <= 2.0 ** -4 * np.abs(wf[normal])).all(), "normal-range rounding bound"
    assert (err[~normal] <= (2.0 ** -10 * sc + 0 * wf)[~normal]).all(), "subnormal-range rounding bound"
    # with the same exponents the dequantized weights encode back to the same codes
    again = O.e4m3_encode(deq / sc)
    assert (again == W8).all(), "codes do not round-trip"


def pin_kmeans_assign_brute_force(lib):
    """a[l] is the centre with the largest dot product, found by plain loops;
    a repeated centre row must lose to its first copy."""
    rng = np.random.default_rng(29)
    L, C, H = 30, 7, 6
    E = bf16_bits(rng.integers(-3, 4, size=(L, H)).astype(np.float32))
    M = bf16_bits(rng.integers(-3, 4, size=(C, H)).astype(np.float32))
    M[5] = M[2]                                     # exact ties between centres 2 and 5
    a, smax = O.oracle_kmeans_assign(E, M)
    ef, mf = _f(E), _f(M)
    for l in range(L):
        best, bc = None, -1
        for c in range(C):
            d = sum(ef[l, j] * mf[c, j] for j in range(H))
            if best is None or d > best:
                best, bc = d, c
        assert a[l] == bc and smax[l] == best, f"label {l}: {a[l]} vs {bc}"


def pin_kmeans_update(lib):
    """The closed-form update equals Sculley's per-sample rule run as loops
    (v += 1; mu += (x - mu) / v, in batch order), then normalised; and
    full-batch steps from zero counts (spherical Lloyd) never lower
    sum_l <E_l, mu_a(l)>."""
    rng = np.random.default_rng(30)
    L, C, H = 60, 5, 8
    E = bf16_bits(rng.normal(size=(L, H)).astype(np.float32))
    ef = _f(E)
    Mc = ef[[3, 17, 29, 41, 55]].copy()
    v = np.array([0, 4, 1, 0, 9])
    batch = np.sort(rng.choice(L, size=25, replace=False)).astype(np.int32)
    a_b = rng.integers(0, C - 1, size=25).astype(np.int32)        # centre C-1 gets nothing
    got, v_got = O.oracle_kmeans_update(E, batch, a_b, Mc, v)
    mu, cnt = Mc.copy(), v.copy()
    touched = set()
    for x, c in zip(batch, a_b):
        cnt[c] += 1
        mu[c] = mu[c] + (ef[x] - mu[c]) / cnt[c]
        touched.add(int(c))
    for c in touched:
        mu[c] = mu[c] / np.sqrt(sum(t * t for t in mu[c]))
    _close(got, mu, 1e-12, 1e-12, "k-means update vs per-sample rule")
    assert (v_got == cnt).all(), "k-means counts"
    # spherical Lloyd steps: objective non-decreasing
    M = bf16_bits(ef[[0, 10, 20, 30, 40]].astype(np.float32))
    Mc = _f(M)
    prev = -np.inf
    for _ in range(6):
        a, _ = O.oracle_kmeans_assign(E, bf16_bits(Mc.astype(np.float32)))
        Mc, _ = O.oracle_kmeans_update(E, np.arange(L, dtype=np.int32), a, Mc, np.zeros(C, np.int64))
        obj = float(sum(ef[l] @ Mc[a[l]] for l in range(L)))
        assert obj >= prev - 1e-9, f"objective fell: {obj} < {prev}"
        prev = obj


def pin_group_greedy(lib):
    """Planted clumps: inside each cluster, clumps of G identical unit
    vectors, orthogonal to each other, plus a few labels orthogonal to
    everything with ids above every clump member (so no seed is one of
    them); the greedy groups must be exactly the clumps (members in
    increasing id), clusters in order, then the leftovers in (cluster, id)
    order cut into groups of G."""
    rng = np.random.default_rng(31)
    G, H = 4, 32
    clumps = {0: 2, 1: 1, 2: 3}                    # clumps per cluster
    extra = {0: 1, 1: 3, 2: 0}                     # leftovers per cluster
    n = sum(G * k + extra[c] for c, k in clumps.items())
    n_pad = (-n) % G                               # a fourth cluster of leftovers only
    L = n + n_pad
    n_clump = G * sum(clumps.values())
    # label ids in the order the loop below takes them: clump members get a
    # shuffle of the low ids, leftovers a shuffle of the high ids
    low, high = rng.permutation(n_clump), n_clump + rng.permutation(L - n_clump)
    ids, il, ih = [], 0, 0
    for c in range(3):
        ids += list(low[il:il + G * clumps[c]])
        il += G * clumps[c]
        ids += list(high[ih:ih + extra[c]])
        ih += extra[c]
    ids += list(high[ih:])
    ids = np.array(ids)
    E = np.zeros((L, H), np.float32)
    a = np.zeros(L, np.int32)
    axis = 0
    pos = 0
    want_groups, left = [], []
    for c in range(3):
        for _ in range(clumps[c]):
            members = ids[pos:pos + G]
            pos += G
            E[members, axis] = 1.0
            axis += 1
            a[members] = c
            want_groups.append((c, sorted(int(x) for x in members)))
        for _ in range(extra[c]):
            x = ids[pos]
            pos += 1
            E[x, axis] = 1.0
            axis += 1
            a[x] = c
            left.append((c, int(x)))
    for _ in range(n_pad):
        x = ids[pos]
        pos += 1
        E[x, axis] = 1.0
        axis += 1
        a[x] = 3
        left.append((3, int(x)))
    perm = O.oracle_group_greedy(bf16_bits(E), a, 4, G)
    assert sorted(perm.tolist()) == list(range(L)), "not a permutation"
    greedy = [g for _, g in sorted(want_groups, key=lambda t: (t[0], t[1][0]))]
    lo = [x for _, x in sorted(left)]
    want = [x for g in greedy for x in g] + lo
    assert perm.tolist() == want, "planted clumps not recovered"
    # random embeddings: a partition whose greedy groups stay inside one cluster
    L2, C2 = 96, 5
    E2 = bf16_bits(rng.normal(size=(L2, H)).astype(np.float32))
    a2 = rng.integers(0, C2, size=L2).astype(np.int32)
    p2 = O.oracle_group_greedy(E2, a2, C2, G)
    assert sorted(p2.tolist()) == list(range(L2))
    n_greedy = sum(int((a2 == c).sum()) // G for c in range(C2))
    for k in range(n_greedy):
        g = p2[k * G:(k + 1) * G]
        assert len(set(a2[g].tolist())) == 1 and list(g) == sorted(g), f"greedy group {k}"
    rest = p2[n_greedy * G:].tolist()
    assert rest == sorted(rest, key=lambda x: (a2[x], x)), "leftovers not in (cluster, id) order"
    for c in range(C2):
        assert sum(1 for x in rest if a2[x] == c) == int((a2 == c).sum()) % G, f"leftovers of cluster {c}"


def _csr(rows):
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([x for r in rows for x in r], np.int32)
    return rp, col


def pin_label_emb_hand_example(lib):
    """One-hot features: sample features e_0, e_0, e_1, e_2 (H = 4); label 0 is
    positive for samples 0, 1, 2 -> sum (2, 1, 0, 0) -> (2, 1, 0, 0) / sqrt 5;
    label 1 for sample 3 only -> e_2; label 2 for none -> 0; label 3 for
    samples 2 and 3 -> (0, 1, 1, 0) / sqrt 2."""
    H, L = 4, 4
    hf = np.zeros((4, H), np.float32)
    hf[0, 0] = hf[1, 0] = hf[2, 1] = hf[3, 2] = 1.0
    rp, col = _csr([[0], [0], [0, 3], [1, 3]])
    E, S, n = O.oracle_label_emb([(bf16_bits(hf), rp, col)], L, H)
    want = np.array([[2, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 0], [0, 1, 1, 0]], np.float64)
    _close(S, want, what="sums")
    assert n.tolist() == [3, 1, 0, 2]
    r5, r2 = 1 / np.sqrt(5), 1 / np.sqrt(2)
    want_e = np.array([[2 * r5, r5, 0, 0], [0, 0, 1, 0], [0, 0, 0, 0], [0, r2, r2, 0]])
    # bf16 keeps 8 significant bits
    _close(_f(E), want_e, rtol=2 ** -8, atol=0, what="embeddings")
    assert (E[2] == 0).all()


def pin_label_emb_dense_product(lib):
    """The sums are Y^T h for the dense 0/1 label matrix Y (a matrix product,
    per batch, added over batches); the counts its column sums; every
    embedding of a label with positives has unit norm up to bf16 rounding and
    points along its sum."""
    rng = np.random.default_rng(41)
    L, H = 30, 24
    batches, Ssum, nsum = [], np.zeros((L, H)), np.zeros(L)
    for B in (17, 9, 1):
        h = bf16_bits(rng.normal(size=(B, H)).astype(np.float32))
        rows = [sorted(rng.choice(L - 3, size=rng.integers(0, 6), replace=False).tolist()) for _ in range(B)]
        rp, col = _csr(rows)
        Y = np.zeros((B, L))
        for b, r in enumerate(rows):
            Y[b, r] = 1.0
        Ssum += Y.T @ _f(h)
        nsum += Y.sum(axis=0)
        batches.append((h, rp, col))
    E, S, n = O.oracle_label_emb(batches, L, H)
    _close(S, Ssum, what="sums vs Y^T h")
    assert (n == nsum).all()
    Ef = _f(E)
    has = nsum > 0
    assert (Ef[~has] == 0).all(), "labels without positives must get 0"
    norms = np.linalg.norm(Ef[has], axis=1)
    assert np.all(np.abs(norms - 1) < 2 ** -7), norms
    cos = (Ef[has] * S[has]).sum(axis=1) / (norms * np.linalg.norm(S[has], axis=1))
    assert np.all(cos > 1 - 2 ** -12)


def pin_label_emb_invariances(lib):
    """Splitting a batch, scaling every feature by 2 (exact in bf16) or adding
    a copy of every sample leaves the embeddings bit for bit; sums scale and
    counts double as they must."""
    rng = np.random.default_rng(42)
    L, H, B = 20, 16, 24
    h = bf16_bits(rng.normal(size=(B, H)).astype(np.float32))
    rows = [sorted(rng.choice(L, size=rng.integers(0, 5), replace=False).tolist()) for _ in range(B)]
    rp, col = _csr(rows)
    E1, S1, n1 = O.oracle_label_emb([(h, rp, col)], L, H)
    parts = []
    for lo, hi in ((0, 7), (7, 8), (8, B)):
        r2, c2 = _csr(rows[lo:hi])
        parts.append((np.ascontiguousarray(h[lo:hi]), r2, c2))
    E2, S2, n2 = O.oracle_label_emb(parts, L, H)
    assert (E1 == E2).all() and (n1 == n2).all()
    _close(S1, S2, what="split batches")
    h2 = bf16_bits((2 * _f(h)).astype(np.float32))
    E3, S3, _ = O.oracle_label_emb([(h2, rp, col)], L, H)
    assert (E3 == E1).all()
    _close(S3, 2 * S1, what="doubled features")
    E4, S4, n4 = O.oracle_label_emb([(h, rp, col), (h, rp, col)], L, H)
    assert (E4 == E1).all() and (n4 == 2 * n1).all()
    _close(S4, 2 * S1, what="repeated batch")
    one = np.flatnonzero(n1 == 1)
    for l in one[:5]:
        b = [i for i, r in enumerate(rows) if l in r][0]
        u = _f(h[b]) / np.linalg.norm(_f(h[b]))
        assert (E1[l] == O.f64_to_bf16_bits(u)).all(), "a single positive gives its own direction"
    # direct rounding: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3 * 2^-8 rounds up to 1 + 2^-6 ... checked on the bit patterns
    r = O.f64_to_bf16_bits(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -9), 0.0]))
    assert r.tolist() == [0x3F80, 0x3F82, 0xBF80, 0x0000], [hex(x) for x in r]


def _run_repeats(row, F):
    """Slots of each run of 8 whose bank key (j >> 1) mod 8 repeats an earlier
    slot of the same run, summed over the runs."""
    keys = [(int(j) >> 1) & 7 for j in row]
    return sum(8 - len(set(keys[r:r + 8])) for r in range(0, F, 8))


def pin_slot_order_hand_examples(lib):
    with open(os.path.join(GOLDEN, "slot_order_hand_examples.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        idx = np.array([c["idx"]], np.int32)
        idx_new, _, perm = O.oracle_order_slots(idx)
        assert list(perm[0]) == c["perm"], f"slot order perm {list(perm[0])} vs {c['perm']}"
        assert list(idx_new[0]) == c["idx_new"], f"slot order idx {list(idx_new[0])} vs {c['idx_new']}"


def pin_slot_order_properties(lib):
    rng = np.random.default_rng(21)
    for F, H, G in ((16, 40, 3), (32, 256, 2), (64, 768, 4), (128, 768, 2), (128, 1024, 1)):
        K = 40
        idx = sorted_subsets(K, F, H, 9, F)
        W = rng.integers(0, 1 << 16, size=(K * G, F), dtype=np.uint16)
        idx_new, W_new, perm = O.oracle_order_slots(idx, W, G)
        for k in range(K):
            assert sorted(perm[k]) == list(range(F)), "slot order: not a permutation"
            assert (idx_new[k] == idx[k][perm[k]]).all(), "slot order: index row not permuted by perm"
            for g in range(G):
                assert (W_new[k * G + g] == W[k * G + g][perm[k]]).all(), "slot order: W column left behind"
            counts = np.bincount((idx[k] >> 1) & 7, minlength=8)
            bound = int(np.maximum(counts - F // 8, 0).sum())
            assert _run_repeats(idx_new[k], F) == bound, f"slot order F={F} k={k}: repeats above the bound"
    # brute force: no split of 16 slots into two runs of 8 repeats fewer keys
    import itertools
    for seed in range(6):
        row = sorted_subsets(1, 16, 48, 30 + seed, 16)[0]
        best = min(_run_repeats([row[i] for i in a] + [row[i] for i in range(16) if i not in a], 16)
                   for a in itertools.combinations(range(16), 8) if 0 in a)
        idx_new, _, _ = O.oracle_order_slots(row[None, :])
        assert _run_repeats(idx_new[0], 16) == best, f"slot order brute force seed {seed}"


ALL_PINS = [
    pin_hand_example,
    pin_bce_hand_example,
    pin_dense_special_case,
    pin_brute_force_masked_dense,
    pin_one_hot_probes,
    pin_all_ones,
    pin_finite_differences,
    pin_permutation_invariance,
    pin_bce_zero_weights,
    pin_torch_autograd,
    pin_g1_per_label,
    pin_head_dense_equals_tail_oracle,
    pin_head_zero_weights,
    pin_joint_torch_autograd,
    pin_rewire_scores_autograd,
    pin_rewire_brute_force,
    pin_rewire_special_cases,
    pin_e4m3_codec_torch,
    pin_e4m3_hand_values,
    pin_w8_group_scales,
    pin_kmeans_assign_brute_force,
    pin_kmeans_update,
    pin_group_greedy,
    pin_label_emb_hand_example,
    pin_label_emb_dense_product,
    pin_label_emb_invariances,
    pin_slot_order_hand_examples,
    pin_slot_order_properties,
]
