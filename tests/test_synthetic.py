"""Seeded input generators: determinism and the properties the layer assumes."""

import numpy as np
import torch

from synthetic import (bf16_bits, bf16_value, get_workload, make_inputs, normal_bf16,
                       sorted_subsets, zipf_labels)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16_bits(x) == ref).all()
    assert (bf16_value(ref) == torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()).all()


def test_sorted_subsets_properties_and_determinism():
    a = sorted_subsets(3000, 64, 768, 3)
    b = sorted_subsets(3000, 64, 768, 3)
    assert (a == b).all() and a.dtype == np.int32
    assert (np.diff(a, axis=1) > 0).all() and a.min() >= 0 and a.max() < 768
    # uniform marginals: every column is chosen with probability F/H
    cnt = np.bincount(a.ravel(), minlength=768) / 3000
    assert abs(cnt.mean() - 64 / 768) < 1e-12 and cnt.std() < 0.02
    full = sorted_subsets(5, 32, 32, 1)
    assert (full == np.arange(32)).all()


def test_normal_bf16_chunk_independent_of_threads():
    x = normal_bf16(5_000_000, 0.125, 7, 2)
    y = normal_bf16(5_000_000, 0.125, 7, 2)
    assert (x == y).all()
    v = bf16_value(x).astype(np.float64)
    assert abs(v.std() - 0.125) < 1e-3 and abs(v.mean()) < 1e-3


def test_zipf_labels_csr():
    rowptr, col = zipf_labels(64, 100000, 36, 3)
    assert rowptr[0] == 0 and (np.diff(rowptr) == 36).all() and col.size == 64 * 36
    for b in range(64):
        r = col[rowptr[b]:rowptr[b + 1]]
        assert (np.diff(r) > 0).all() and r.min() >= 0 and r.max() < 100000
    # a heavy head: the most frequent label appears in most samples
    assert np.bincount(col).max() > 40


def test_make_inputs_tiny_shapes():
    w = get_workload("tiny_4k")
    d = make_inputs(w, idx1=True)
    assert d["idx"].shape == (w.K, w.F) and d["h"].shape == (w.B, w.H)
    assert d["W"].shape == (w.L, w.F) and d["dZ"].shape == (w.B, w.L)
    assert d["idx1"].shape == (w.L, w.F) and d["y_rowptr"].shape == (w.B + 1,)
