"""GPU parity of the label embeddings (haste_label_emb_accumulate /
haste_label_emb_finalize) against the fp64 oracle, through the C ABI:
per-label sums and counts over several batches, the bf16 embeddings within
one bf16 rounding step, labels without positives exactly 0, integer-valued
features summed exactly, bitwise repeats, an empty batch, and a label with
thousands of positives in one batch (multi-block sort)."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import bf16_bits, normal_bf16, zipf_labels

pytestmark = pytest.mark.gpu


def run_gpu(batches, L, H):
    import torch
    dev = torch.device("cuda:0")
    S = torch.zeros(L, H, dtype=torch.float32, device=dev)
    n = torch.zeros(L, dtype=torch.int32, device=dev)
    for h, rp, col in batches:
        c = to_dev_i32(col if col.size else np.zeros(4, np.int32))
        hs.label_emb_accumulate(to_dev_bf16(h), to_dev_i32(rp), c, S, n, nnz=int(rp[-1]))
    E = hs.label_emb_finalize(S, n)
    return to_host(E), to_host(S), to_host(n)


def check(batches, L, H, exact_sums=False):
    E, S, n = run_gpu(batches, L, H)
    Eo, So, no = O.oracle_label_emb(batches, L, H)
    assert (n == no).all(), "counts differ"
    if exact_sums:
        assert (S.astype(np.float64) == So).all(), "integer sums differ"
    else:
        err = np.abs(S - So).max()
        say(f"    sums: max abs err {err:.2e} (|S| up to {np.abs(So).max():.1f})")
        assert err <= 1e-5 * max(1.0, np.abs(So).max())
    ef, eo = O._bf16_f64(E), O._bf16_f64(Eo)
    none = no == 0
    assert (E[none] == 0).all(), "labels without positives must be 0"
    # within one bf16 rounding step of the oracle's directly rounded values,
    # plus what the fp32 sums' rounding moves a unit vector (|dS| / |S| < 1e-6)
    d = np.abs(ef - eo)
    bound = 2.0 ** -7 * np.abs(eo) + 1e-5             # one step is 2^-7 |x| at the bottom of a binade
    assert (d <= bound).all(), f"embeddings differ by more than one bf16 step: worst {(d - bound).max():.2e}"
    same = (E == Eo).mean()
    say(f"    {100 * same:.3f} % of embedding values bit-equal to the oracle's")
    return E, S


@pytest.mark.parametrize("L,H,bs", [(5000, 64, (128, 1, 77)), (3000, 768, (256, 100)), (2000, 1024, (64, 64, 9)),
                                    (700, 200, (33,))])
def test_label_emb_random(L, H, bs):
    say(f"  label emb L={L} H={H} batches={bs}")
    batches = []
    for i, B in enumerate(bs):
        h = normal_bf16(B * H, 1.0, 500 + i, 1).reshape(B, H)
        rp, col = zipf_labels(B, L, min(9, L), 600 + i)
        batches.append((h, rp, col))
    check(batches, L, H)


def test_label_emb_integer_exact_and_repeat():
    rng = np.random.default_rng(7)
    L, H = 1500, 96
    batches = []
    for i, B in enumerate((200, 50)):
        h = bf16_bits(rng.integers(-3, 4, size=(B, H)).astype(np.float32))
        rp, col = zipf_labels(B, L, 12, 700 + i)
        batches.append((h, rp, col))
    E1, S1 = check(batches, L, H, exact_sums=True)
    E2, S2, _ = run_gpu(batches, L, H)
    assert (S1.view(np.uint32) == S2.view(np.uint32)).all() and (E1 == E2).all(), "not bitwise repeatable"


def test_label_emb_empty_batch_and_dense_label():
    """An empty batch changes nothing; a label positive for all 3000 samples
    of a batch (nnz past one 2048-key sort block)."""
    L, H, B = 64, 128, 3000
    h = normal_bf16(B * H, 1.0, 801, 1).reshape(B, H)
    rows = [[7] + ([20 + b % 30] if b % 3 == 0 else []) for b in range(B)]
    rp = np.zeros(B + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([x for r in rows for x in r], np.int32)
    empty = (normal_bf16(5 * H, 1.0, 802, 1).reshape(5, H), np.zeros(6, np.int32), np.zeros(0, np.int32))
    check([empty, (h, rp, col), empty], L, H)
