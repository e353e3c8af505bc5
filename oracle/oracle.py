"""ctypes wrapper of liboracle.so (built from haste_oracle.c with gcc), and
the dense head of the head-tail split in numpy fp64.

Test infrastructure only: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it, never the product path.  Every function
takes numpy arrays: bf16 tensors as uint16 bit patterns, index sets and
labels as int32, and returns fp64 numpy arrays.  Shapes are checked here; the
C code assumes them.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "haste_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, IEEE fp64, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if absent) and declare the C signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    for name in ("oracle_fwd", "oracle_bwd_w", "oracle_bwd_w_f64", "oracle_bwd_h", "oracle_bwd_h_f64"):
        getattr(lib, name).argtypes = [P, P, P, P, I, I, I, I, I]
        getattr(lib, name).restype = None
    lib.oracle_bce.argtypes = [P, I, I, P, P, ctypes.c_double, P, P]
    lib.oracle_bce.restype = None
    lib.oracle_step.argtypes = [P, P, P, P, P, ctypes.c_double, P, P, P, P, P, I, I, I, I, I]
    lib.oracle_step.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(name, a, dtype, shape):
    if a.dtype != dtype or not a.flags.c_contiguous or tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected C-contiguous {np.dtype(dtype)} {tuple(shape)}, "
                         f"got {a.dtype} {a.shape}")


def _dims(idx, G, h=None, B=None, H=None):
    K, F = idx.shape
    return K, F, K * G


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def oracle_fwd(h, idx, W, G, lib=None):
    """Z (B x L fp64) = forward logits."""
    lib = lib or load()
    B, H = h.shape
    K, F, L = _dims(idx, G)
    _check("h", h, np.uint16, (B, H)); _check("idx", idx, np.int32, (K, F)); _check("W", W, np.uint16, (L, F))
    Z = np.empty((B, L), dtype=np.float64)
    lib.oracle_fwd(_p(h), _p(idx), _p(W), _p(Z), B, H, K, G, F)
    return Z


def oracle_bwd_w(h, idx, dZ, G, lib=None):
    """dW (L x F fp64).  dZ is bf16 bits (uint16) or fp64."""
    lib = lib or load()
    B, H = h.shape
    K, F, L = _dims(idx, G)
    _check("h", h, np.uint16, (B, H)); _check("idx", idx, np.int32, (K, F))
    dW = np.empty((L, F), dtype=np.float64)
    if dZ.dtype == np.float64:
        _check("dZ", dZ, np.float64, (B, L))
        lib.oracle_bwd_w_f64(_p(h), _p(idx), _p(dZ), _p(dW), B, H, K, G, F)
    else:
        _check("dZ", dZ, np.uint16, (B, L))
        lib.oracle_bwd_w(_p(h), _p(idx), _p(dZ), _p(dW), B, H, K, G, F)
    return dW


def oracle_bwd_h(dZ, idx, W, G, H, lib=None):
    """dh (B x H fp64).  dZ is bf16 bits (uint16) or fp64."""
    lib = lib or load()
    B = dZ.shape[0]
    K, F, L = _dims(idx, G)
    _check("idx", idx, np.int32, (K, F)); _check("W", W, np.uint16, (L, F))
    dh = np.empty((B, H), dtype=np.float64)
    if dZ.dtype == np.float64:
        _check("dZ", dZ, np.float64, (B, L))
        lib.oracle_bwd_h_f64(_p(dZ), _p(idx), _p(W), _p(dh), B, H, K, G, F)
    else:
        _check("dZ", dZ, np.uint16, (B, L))
        lib.oracle_bwd_h(_p(dZ), _p(idx), _p(W), _p(dh), B, H, K, G, F)
    return dh


def oracle_bce(Z, y_rowptr, y_col, scale, lib=None):
    """(dZ fp64 B x L, loss float) of BCE(sigmoid(Z), Y) with Y from CSR."""
    lib = lib or load()
    B, L = Z.shape
    _check("Z", Z, np.float64, (B, L))
    _check("y_rowptr", y_rowptr, np.int32, (B + 1,))
    _check("y_col", y_col, np.int32, (int(y_rowptr[-1]),))
    if y_col.size and (y_col.min() < 0 or y_col.max() >= L):
        raise ValueError("label id out of range")
    dZ = np.empty((B, L), dtype=np.float64)
    loss = np.zeros(1, dtype=np.float64)
    lib.oracle_bce(_p(Z), B, L, _p(y_rowptr), _p(y_col), float(scale), _p(dZ), _p(loss))
    return dZ, float(loss[0])


def oracle_step(h, idx, W, y_rowptr, y_col, scale, G, want_dW=True, want_dh=True, lib=None):
    """Full training pass: returns dict with Z, dZ (fp64), dW, dh, loss."""
    lib = lib or load()
    B, H = h.shape
    K, F, L = _dims(idx, G)
    _check("h", h, np.uint16, (B, H)); _check("idx", idx, np.int32, (K, F)); _check("W", W, np.uint16, (L, F))
    _check("y_rowptr", y_rowptr, np.int32, (B + 1,))
    _check("y_col", y_col, np.int32, (int(y_rowptr[-1]),))
    if y_col.size and (y_col.min() < 0 or y_col.max() >= L):
        raise ValueError("label id out of range")
    Z = np.empty((B, L), dtype=np.float64)
    dZ = np.empty((B, L), dtype=np.float64)
    dW = np.empty((L, F), dtype=np.float64) if want_dW else None
    dh = np.empty((B, H), dtype=np.float64) if want_dh else None
    loss = np.zeros(1, dtype=np.float64)
    lib.oracle_step(_p(h), _p(idx), _p(W), _p(y_rowptr), _p(y_col), float(scale),
                    _p(Z), _p(dZ), _p(dW), _p(dh), _p(loss), B, H, K, G, F)
    return {"Z": Z, "dZ": dZ, "dW": dW, "dh": dh, "loss": float(loss[0])}


def _bf16_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_head_step(h, W_head, y_rowptr, y_col, scale, lib=None):
    """Dense head of the head-tail split (HASTE notes, "Head-tail split":
    every head label sees all H features; the BCE objective covers head and
    tail labels alike).  Z = h W_head^T, dZ and the loss from oracle_bce,
    dW = dZ^T h, dh = dZ W_head; numpy fp64 products.  Returns dict with Z,
    dZ, dW (L_head x H), dh (B x H), loss."""
    B, H = h.shape
    L = W_head.shape[0]
    _check("h", h, np.uint16, (B, H)); _check("W_head", W_head, np.uint16, (L, H))
    hf, Wf = _bf16_f64(h), _bf16_f64(W_head)
    Z = np.ascontiguousarray(hf @ Wf.T)
    dZ, loss = oracle_bce(Z, y_rowptr, y_col, scale, lib=lib)
    return {"Z": Z, "dZ": dZ, "dW": dZ.T @ hf, "dh": dZ @ Wf, "loss": loss}


def oracle_joint_step(h, idx, W_tail, yt_rowptr, yt_col, W_head, yh_rowptr, yh_col, scale_tail, scale_head, G,
                      lib=None):
    """Head + tail training pass on shared features h (HASTE notes,
    "Head-tail split"): the tail's oracle_step and the head's
    oracle_head_step; the feature gradient and the loss of the joint
    objective are the sums of the two branches'.  Returns dict with dW_tail,
    dW_head, dh, loss and the per-branch results under "tail" and "head"."""
    t = oracle_step(h, idx, W_tail, yt_rowptr, yt_col, scale_tail, G, lib=lib)
    hd = oracle_head_step(h, W_head, yh_rowptr, yh_col, scale_head, lib=lib)
    return {"dW_tail": t["dW"], "dW_head": hd["dW"], "dh": t["dh"] + hd["dh"], "loss": t["loss"] + hd["loss"],
            "tail": t, "head": hd}


def oracle_rewire_scores(h, dZ, idx, W, G):
    """Scores of the group-level rewiring step (HASTE notes, "loss /
    training strategy": RigL-style dynamic sparse training periodically
    reselects each group's index set I_k, keeping |I_k| = F; the algorithm
    itself is not printed, so this follows RigL with the group as the unit).
      grow[k, j]  = sum_g | sum_b dZ[b, kG+g] h[b, j] |   (K x H): the size of
                    the dense loss gradient the group's labels would have on
                    feature column j (RigL's growth criterion, summed over G)
      prune[k, f] = sum_g | W[kG+g, f] |                  (K x F): the weight
                    magnitude of slot f (RigL's drop criterion, summed over G)
    dZ is bf16 bits (B x L); fp64 results."""
    B, H = h.shape
    K, F = idx.shape
    L = K * G
    _check("h", h, np.uint16, (B, H)); _check("dZ", dZ, np.uint16, (B, L))
    _check("idx", idx, np.int32, (K, F)); _check("W", W, np.uint16, (L, F))
    hf, dzf, wf = _bf16_f64(h), _bf16_f64(dZ), _bf16_f64(W)
    grow = np.empty((K, H))
    for k in range(K):
        dense_grad = dzf[:, k * G:(k + 1) * G].T @ hf          # G x H
        grow[k] = np.abs(dense_grad).sum(axis=0)
    prune = np.abs(wf).reshape(K, G, F).sum(axis=1)
    return grow, prune


def oracle_rewire_select(idx, W, grow, prune, n_swap, G):
    """The discrete rewiring phase for every group k, given its scores:
      1. drop the n_swap slots with the smallest prune score (equal scores:
         the lower column id is dropped first);
      2. grow the n_swap columns with the largest grow score among the
         columns not kept (a dropped column may come back; equal scores:
         the lower column id first);
      3. the new I_k is the kept and grown columns in increasing order; a
         kept column keeps its weights (its W column moves with it), a grown
         column starts at weight zero.
    Returns (idx_new K x F int32, W_new L x F bf16 bits)."""
    K, F = idx.shape
    H = grow.shape[1]
    if not 0 <= n_swap <= F:
        raise ValueError("need 0 <= n_swap <= F")
    idx_new = np.empty_like(idx)
    W_new = np.zeros_like(W)
    for k in range(K):
        cols = [int(c) for c in idx[k]]
        by_weight = sorted(range(F), key=lambda f: (prune[k, f], cols[f]))
        dropped = set(by_weight[:n_swap])
        kept = {cols[f]: f for f in range(F) if f not in dropped}
        candidates = [j for j in range(H) if j not in kept]
        grown = sorted(candidates, key=lambda j: (-grow[k, j], j))[:n_swap]
        new_cols = sorted(list(kept) + grown)
        idx_new[k] = new_cols
        for f_new, c in enumerate(new_cols):
            if c in kept:
                W_new[k * G:(k + 1) * G, f_new] = W[k * G:(k + 1) * G, kept[c]]
    return idx_new, W_new


def oracle_rewire(h, dZ, idx, W, n_swap, G):
    """Scores, then the selection: (idx_new, W_new, grow, prune)."""
    grow, prune = oracle_rewire_scores(h, dZ, idx, W, G)
    idx_new, W_new = oracle_rewire_select(idx, W, grow, prune, n_swap, G)
    return idx_new, W_new, grow, prune


# ---------------------------------------------------------------- FP8 weights
#
# HASTE notes, "limitations": combining the layer with FP8 quantisation is
# the named next step.  The reading here: W is stored as OCP FP8 E4M3 codes
# (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities, the
# all-ones magnitude is NaN, largest finite 448) with one power-of-two scale
# 2^e_k per label group; the layer then computes exactly what the bf16 layer
# computes on the dequantized weights.

def e4m3_decode(codes):
    """E4M3 codes (uint8) -> fp64 values, from the format's definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.ldexp(1.0, e - 10))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """fp64 values with |x| <= 448 -> E4M3 codes (uint8), rounded to nearest
    with ties to the even code.  Normal range (|x| >= 2^-6): 3 fraction bits
    of |x| = q 2^(E-3), q in [8, 16], code = 8 (E + 6) + q (q = 16 carries into
    the next binade); below it, n = |x| 2^9 rounded, code = n."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0) or np.any(np.isnan(a)):
        raise ValueError("value outside the E4M3 range")
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^ex, f in [0.5, 1)
    E = ex - 1                                           # a = 1.xxx 2^E
    normal = a >= 2.0 ** -6
    q = np.rint(np.ldexp(a, 3 - E))                      # exact scaling, rint = ties to even
    code_n = 8 * (E + 6) + q
    code_s = np.rint(np.ldexp(a, 9))
    code = np.where(normal, code_n, code_s).astype(np.int64)
    code |= np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def w8_group_exponent(W, G):
    """Per group k, the smallest integer e_k with max |W_k| 2^-e_k <= 448
    (0 for an all-zero group), clamped to [-120, 120]."""
    K = W.shape[0] // G
    mx = np.abs(_bf16_f64(W)).reshape(K, -1).max(axis=1)
    e = np.zeros(K, dtype=np.int64)
    nz = mx > 0
    e[nz] = np.ceil(np.log2(mx[nz] / 448.0)).astype(np.int64)
    # log2 of an exact ratio: confirm the integer against the condition itself
    for k in np.nonzero(nz)[0]:
        while np.ldexp(mx[k], -int(e[k])) > 448.0:
            e[k] += 1
        while np.ldexp(mx[k], -(int(e[k]) - 1)) <= 448.0:
            e[k] -= 1
    return np.clip(e, -120, 120).astype(np.int32)


def oracle_quantize_w8(W, G):
    """bf16 W (L x F bits) -> (W8 L x F uint8 E4M3 codes, wexp K int32):
    code = encode(W 2^-e_k) for the labels of group k."""
    L, F = W.shape
    _check("W", W, np.uint16, (L, F))
    wexp = w8_group_exponent(W, G)
    scaled = _bf16_f64(W) * np.ldexp(1.0, -np.repeat(wexp, G).astype(np.int64))[:, None]
    return e4m3_encode(scaled), wexp


def oracle_dequantize_w8(W8, wexp, G):
    """(W8, wexp) -> bf16 bits of decode(code) 2^e_k (exact in bf16)."""
    vals = e4m3_decode(W8) * np.ldexp(1.0, np.repeat(wexp, G).astype(np.int64))[:, None]
    f32 = vals.astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if not np.array_equal(back, vals):
        raise ValueError("dequantized weight not exact in bf16")
    return bits


# ------------------------------------------------------------ label grouping
#
# HASTE notes, "group-shared fixed fan-in": labels are grouped by embedding
# similarity, approximately, in two stages: mini-batch spherical k-means into
# C ~ L / (beta G) coarse clusters, then, inside each cluster, greedy groups
# of a seed and its G - 1 nearest neighbours.  Embeddings are given (L x H
# bf16); similarity is the dot product (the cosine for unit vectors).

def oracle_kmeans_assign(E, M):
    """a[l] = argmax_c <E_l, M_c> (the lowest c among equal maxima) and the
    maximum s[l]; E (L x H) and M (C x H) are bf16 bits."""
    Ef, Mf = _bf16_f64(E), _bf16_f64(M)
    S = Ef @ Mf.T
    a = np.argmax(S, axis=1)                       # first maximum = lowest c
    return a.astype(np.int32), S[np.arange(S.shape[0]), a]


def oracle_kmeans_update(E, batch, a_batch, Mc, v):
    """One mini-batch step of spherical k-means: Sculley's mini-batch update
    (each batch member x of centre c moves it by (x - mu_c) / v_c after
    v_c += 1, i.e. mu_c becomes the running mean of everything assigned to it
    so far), then the centre is projected back onto the unit sphere.  Centres
    without batch members are left as they are.  Mc: C x H fp64, v: C counts.
    Returns (Mc_new, v_new)."""
    Ef = _bf16_f64(E)
    Mc = np.array(Mc, dtype=np.float64, copy=True)
    v = np.array(v, dtype=np.int64, copy=True)
    for c in np.unique(a_batch):
        members = np.asarray(batch)[np.asarray(a_batch) == c]
        m = members.size
        mu = (v[c] * Mc[c] + Ef[members].sum(axis=0)) / (v[c] + m)
        v[c] += m
        Mc[c] = mu / np.linalg.norm(mu)
    return Mc, v


def oracle_group_greedy(E, a, C, G):
    """Groups of exactly G labels from cluster assignments a (L,) in [0, C):
    inside each cluster (members in increasing label id), while at least G
    members are ungrouped, the lowest-id ungrouped member is the seed and the
    G - 1 ungrouped members with the largest <E_seed, E_x> (lower id on
    ties) join it; a group lists its members in increasing id.  Clusters are
    taken in increasing id; the members left over (fewer than G per cluster)
    are then concatenated in (cluster, id) order and cut into consecutive
    groups of G.  Returns perm (L,) int32: group k = perm[kG : (k+1)G].
    L must be a multiple of G."""
    L = E.shape[0]
    if L % G:
        raise ValueError("L must be a multiple of G")
    Ef = _bf16_f64(E)
    groups, leftovers = [], []
    for c in range(C):
        free = [int(x) for x in np.nonzero(np.asarray(a) == c)[0]]      # increasing id
        while len(free) >= G:
            seed = free[0]
            rest = free[1:]
            sims = Ef[rest] @ Ef[seed]
            order = sorted(range(len(rest)), key=lambda i: (-sims[i], rest[i]))[:G - 1]
            chosen = sorted([seed] + [rest[i] for i in order])
            groups.append(chosen)
            taken = set(chosen)
            free = [x for x in free if x not in taken]
        leftovers.extend(free)
    for i in range(0, len(leftovers), G):
        groups.append(leftovers[i:i + G])
    return np.array([x for g in groups for x in g], dtype=np.int32)


# ------------------------------------------------------------ label embeddings
#
# HASTE notes, "group-shared fixed fan-in": the grouping works on label
# embeddings, a label's embedding being the normalized mean of the encoder
# features of the samples that have the label as a positive.  Over a
# dataset given as batches of features h (B x H bf16) and 0/1 labels (CSR,
# ids in [0, L)), the oracle keeps per label the fp64 sum of those features
# and the number of positives; the direction of the mean is the direction
# of the sum.

def oracle_label_emb_accumulate(S, n, h, y_rowptr, y_col):
    """Adds one batch in place: for every sample b and every positive label
    l of b, S[l] += h[b] and n[l] += 1.  S: L x H fp64, n: L int64.
    Returns (S, n)."""
    hf = _bf16_f64(h)
    rp = np.asarray(y_rowptr, dtype=np.int64)
    col = np.asarray(y_col, dtype=np.int64)
    for b in range(hf.shape[0]):
        for p in range(rp[b], rp[b + 1]):
            S[col[p]] += hf[b]
            n[col[p]] += 1
    return S, n


def f64_to_bf16_bits(x):
    """Round fp64 values to the nearest bf16, ties to even (directly, without
    an fp32 step); returns the 16-bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                               # x = m 2^e, 0.5 <= |m| < 1
    q = np.rint(np.ldexp(m, 8))                      # 8 significant bits, ties to even
    r = np.ldexp(q, e - 8).astype(np.float32)        # exact in fp32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def oracle_label_emb_finalize(S, n):
    """e_l = S_l / |S_l|, rounded to bf16 (L x H bits); 0 for a label without
    positives or with a zero sum."""
    S = np.asarray(S, dtype=np.float64)
    norm = np.sqrt((S * S).sum(axis=1))
    ok = (np.asarray(n) > 0) & (norm > 0)
    E = np.zeros_like(S)
    E[ok] = S[ok] / norm[ok, None]
    return f64_to_bf16_bits(E)


def oracle_label_emb(batches, L, H):
    """Embeddings from a list of (h, y_rowptr, y_col) batches: (E bits, S, n)."""
    S = np.zeros((L, H), dtype=np.float64)
    n = np.zeros(L, dtype=np.int64)
    for h, rp, col in batches:
        oracle_label_emb_accumulate(S, n, h, rp, col)
    return oracle_label_emb_finalize(S, n), S, n


# ------------------------------------------------------------------ slot order
#
# HASTE notes, "group-shared fixed fan-in": a group is defined by its index
# set I_k.  The slot f at which a column sits carries no meaning as long as
# column f of W_k moves with it, since every product of the layer sums over
# the slots.  The library can therefore store each group's slots in an order
# chosen for its feature-gradient accumulator.  That accumulator keeps the
# rows of feature column j in bank group (j >> 1) mod 8, and one of its
# read-add-write instructions covers a run of 8 consecutive slots, so the
# columns of a run should have distinct keys (j >> 1) mod 8.  The order,
# group by group (F a multiple of 8, R = F / 8 runs):
#   1. sort the F slots by key, equal keys in slot order;
#   2. deal the sorted slots over the runs in turn: the p-th slot of the
#      sorted list becomes new slot 8 (p mod R) + (p div R).
# A key held by at most R slots then lands in distinct runs.

def oracle_order_slots(idx, W=None, G=None):
    """(idx_new, W_new, perm) with perm[k, s] the old slot of new slot s:
    idx_new[k, s] = idx[k, perm[k, s]] and, when W (L x F bf16 bits, L = K G)
    is given, W_new[k G + g, s] = W[k G + g, perm[k, s]] (else W_new is None)."""
    idx = np.asarray(idx)
    K, F = idx.shape
    if F % 8 != 0:
        raise ValueError("F must be a multiple of 8")
    R = F // 8
    perm = np.empty((K, F), dtype=np.int32)
    for k in range(K):
        keys = [(int(idx[k, f]) >> 1) & 7 for f in range(F)]
        order = sorted(range(F), key=lambda f: (keys[f], f))
        for p, f in enumerate(order):
            perm[k, 8 * (p % R) + p // R] = f
    idx_new = np.take_along_axis(idx, perm, axis=1).astype(np.int32)
    W_new = None
    if W is not None:
        _check("W", W, np.uint16, (K * G, F))
        W_new = np.take_along_axis(W, np.repeat(perm, G, axis=0), axis=1)
    return idx_new, W_new, perm
