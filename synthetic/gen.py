"""Seeded input generators (no layer arithmetic lives here).

Every tensor is drawn from ``np.random.SeedSequence([seed_no, tensor_no,
chunk])`` so the result does not depend on the number of worker threads.
Tensor numbers: 0 group index sets, 1 features h, 2 weights W, 3 upstream
gradient dZ, 4 label-rank permutation, 5 positive labels, 6 per-label index
sets of the G=1 fixed fan-in baseline, 7 dense-head weights, 8 label
embeddings, 9 their topics, 10 k-means draws (initial centres, mini-batches).

bf16 values are carried as their uint16 bit patterns, rounded from float32
to nearest with ties to even.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

T_IDX, T_H, T_W, T_DZ, T_PERM, T_POS, T_IDX1, T_WHEAD, T_EMB, T_EMBTOPIC, T_KM = range(11)

_CHUNK = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed_no: int, tensor_no: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed_no, tensor_no, chunk]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any((u & 0x7F800000) == 0x7F800000):
        raise ValueError("bf16_bits: NaN/Inf inputs are not generated here")
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_value(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(n: int, std: float, seed_no: int, tensor_no: int) -> np.ndarray:
    """n draws of N(0, std^2), rounded to bf16 bit patterns."""
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _rng(seed_no, tensor_no, c).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = bf16_bits(x)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def sorted_subsets(rows: int, F: int, H: int, seed_no: int, tensor_no: int = T_IDX) -> np.ndarray:
    """rows x F int32: each row an F-subset of [0, H) drawn uniformly without
    replacement, sorted ascending.

    Draw H random 53-bit keys per row, keep the F columns with the smallest
    keys (a uniformly random F-subset), then sort the kept column ids.
    """
    if not (0 < F <= H <= 1024):
        raise ValueError("need 0 < F <= H <= 1024")
    out = np.empty((rows, F), dtype=np.int32)
    per = max(1, _CHUNK // H)
    nchunks = (rows + per - 1) // per
    col = np.arange(H, dtype=np.uint64)

    def work(c):
        lo, hi = c * per, min(rows, (c + 1) * per)
        keys = _rng(seed_no, tensor_no, c).integers(0, 2**63, size=(hi - lo, H), dtype=np.int64)
        keys = ((keys.view(np.uint64) >> np.uint64(10)) << np.uint64(10)) | col
        if F < H:
            keys = np.partition(keys, F - 1, axis=1)[:, :F]
        out[lo:hi] = np.sort((keys & np.uint64(1023)).astype(np.int32), axis=1)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _zipf_draws(B: int, L: int, m: int, seed_no: int, s: float):
    """Per sample, m distinct Zipf(s) ranks in [0, L) (0 = most frequent),
    and the seeded permutation that maps rank r to label id perm[r]."""
    if m > L:
        raise ValueError("m > L")
    ranks = np.arange(1, L + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    perm = _rng(seed_no, T_PERM).permutation(L).astype(np.int64)
    rng = _rng(seed_no, T_POS)
    draws = np.empty((B, m), dtype=np.int64)
    for b in range(B):
        chosen: list[int] = []
        seen: set[int] = set()
        while len(chosen) < m:
            u = rng.random(2 * m)
            r = np.minimum(np.searchsorted(cdf, u, side="right"), L - 1)
            for x in r.tolist():
                if x not in seen:
                    seen.add(x)
                    chosen.append(x)
                    if len(chosen) == m:
                        break
        draws[b] = chosen
    return draws, perm


def _csr(rows: list) -> tuple:
    rowptr = np.zeros(len(rows) + 1, dtype=np.int64)
    rowptr[1:] = np.cumsum([r.size for r in rows])
    col = np.concatenate(rows).astype(np.int32) if rows and rowptr[-1] else np.zeros(0, np.int32)
    return rowptr.astype(np.int32), col


def zipf_labels(B: int, L: int, m: int, seed_no: int, s: float = 1.1):
    """0/1 label matrix B x L as CSR (rowptr int32 [B+1], col int32 [B*m]).

    Every sample gets exactly m distinct labels.  A label is drawn by rank r
    from a Zipf(s) law truncated at L (p(r) proportional to r^-s, inverse-CDF
    sampling), duplicates are redrawn, and rank r maps to label id perm[r-1]
    for a seeded permutation perm of [0, L).  Column ids are sorted within a
    row.
    """
    draws, perm = _zipf_draws(B, L, m, seed_no, s)
    return _csr([np.sort(perm[d]) for d in draws])


def head_tail_labels(B: int, L: int, L_head: int, m: int, seed_no: int, s: float = 1.1):
    """The labels of zipf_labels(B, L, m, seed_no, s) split into a head (the
    L_head most frequent ranks, label ids perm[0 .. L_head-1]) and a tail
    (the other L - L_head ids).  Each part is renumbered in increasing order
    of the original id.  Returns (head_rowptr, head_col, tail_rowptr,
    tail_col), CSR with sorted ids per row."""
    if not 0 < L_head < L:
        raise ValueError("need 0 < L_head < L")
    draws, perm = _zipf_draws(B, L, m, seed_no, s)
    is_head = np.zeros(L, dtype=bool)
    is_head[perm[:L_head]] = True
    head_id = np.cumsum(is_head) - 1
    tail_id = np.cumsum(~is_head) - 1
    hrows, trows = [], []
    for d in draws:
        ids = np.sort(perm[d])
        hd = is_head[ids]
        hrows.append(head_id[ids[hd]])
        trows.append(tail_id[ids[~hd]])
    return (*_csr(hrows), *_csr(trows))


def make_inputs(w, *, dZ: bool = True, labels: bool = True, idx1: bool = False, w_head: bool = False) -> dict:
    """All inputs of one workload `w` (a synthetic.configs.Workload).

    Returns a dict of numpy arrays: idx (K x F int32), h (B x H bf16 bits),
    W (L x F bf16 bits), optionally dZ (B x L bf16 bits), y_rowptr / y_col
    (CSR 0/1 labels) and idx1 (L x F int32 per-label index sets for the G=1
    baseline).  For the tail workload of a head-tail split (w.head_labels >
    0) the labels are drawn over the full label space and split: y_* are the
    tail's, yh_* the head's; w_head adds the head's weights W_head
    (head_labels x H bf16 bits, N(0, 1/H)).
    """
    out = {
        "idx": sorted_subsets(w.K, w.F, w.H, w.seed_no, T_IDX),
        "h": normal_bf16(w.B * w.H, 1.0, w.seed_no, T_H).reshape(w.B, w.H),
        "W": normal_bf16(w.L * w.F, float(1.0 / np.sqrt(w.F)), w.seed_no, T_W).reshape(w.L, w.F),
    }
    if dZ:
        out["dZ"] = normal_bf16(w.B * w.L, 1.0, w.seed_no, T_DZ).reshape(w.B, w.L)
    if labels and w.head_labels:
        # tail workload of a head-tail split: labels drawn over the full
        # label space, the tail's part as y_*, the head's as yh_*
        out["yh_rowptr"], out["yh_col"], out["y_rowptr"], out["y_col"] = head_tail_labels(
            w.B, w.L + w.head_labels, w.head_labels, w.m, w.seed_no, w.zipf_s)
    elif labels:
        out["y_rowptr"], out["y_col"] = zipf_labels(w.B, w.L, w.m, w.seed_no, w.zipf_s)
    if w_head:
        if not w.head_labels:
            raise ValueError(f"{w.name} has no dense head")
        out["W_head"] = normal_bf16(w.head_labels * w.H, float(1.0 / np.sqrt(w.H)), w.seed_no,
                                    T_WHEAD).reshape(w.head_labels, w.H)
    if idx1:
        out["idx1"] = sorted_subsets(w.L, w.F, w.H, w.seed_no, T_IDX1)
    return out


def label_embeddings(L: int, H: int, topics: int, noise: float, seed_no: int) -> np.ndarray:
    """L x H bf16 bits: unit vectors normalize(t_{c(l)} + noise * n_l) with
    `topics` random unit topic directions t, c(l) uniform, n_l ~ N(0, I/H)."""
    rng_t = _rng(seed_no, T_EMBTOPIC)
    T = rng_t.normal(size=(topics, H))
    T /= np.linalg.norm(T, axis=1, keepdims=True)
    c = rng_t.integers(0, topics, size=L)
    out = np.empty((L, H), dtype=np.uint16)
    step = max(1, _CHUNK // H)

    def work(i):
        lo, hi = i * step, min(L, (i + 1) * step)
        x = T[c[lo:hi]] + noise * _rng(seed_no, T_EMB, i).normal(size=(hi - lo, H)) / np.sqrt(H)
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        out[lo:hi] = bf16_bits(x.astype(np.float32))

    nchunks = (L + step - 1) // step
    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def kmeans_draws(L: int, C: int, batch: int, iters: int, seed_no: int):
    """The random choices of mini-batch k-means, drawn here and passed to both
    implementations: C distinct initial centre labels and `iters` mini-batches
    of `batch` distinct labels each."""
    rng = _rng(seed_no, T_KM)
    init = np.sort(rng.choice(L, size=C, replace=False)).astype(np.int32)
    batches = [np.sort(rng.choice(L, size=batch, replace=False)).astype(np.int32) for _ in range(iters)]
    return init, batches
