"""Workload shapes for the group-shared fixed fan-in tail layer.

The shapes stand in for the extreme multi-label datasets the HASTE paper
trains on (HASTE, "Main results" table: Amazon-670K, Amazon-3M,
LF-Paper2Keywords-8.6M).  None of those datasets is used: every tensor is
drawn from seeded distributions with the label count, hidden width H=768 of a
BERT-base encoder ("Limitations" section) and the positives per sample given
below.  `seed_no` keys numpy's SeedSequence so each workload draws its own
independent stream.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    seed_no: int
    L: int          # labels
    G: int          # labels per group (shared fan-in index set)
    H: int          # feature width that index sets draw from
    F: int          # fan-in per label (= |I_k|)
    B: int          # batch
    m: int          # positive labels per sample (0/1 label matrix row weight)
    zipf_s: float = 1.1
    head_labels: int = 0   # > 0: this is the tail of a head-tail split with this many head labels

    @property
    def K(self) -> int:
        return self.L // self.G

    def useful_flops_per_contraction(self) -> int:
        """2*B*L*F: one multiply-add per (sample, label, fan-in slot)."""
        return 2 * self.B * self.L * self.F


WORKLOADS = {
    # Small case the oracle finishes in well under a second.
    "tiny_4k": Workload("tiny_4k", 1, L=4096, G=16, H=256, F=32, B=64, m=5),
    # Amazon-670K-shaped: 670,208 = 16 * 41,888 labels.
    "amazon670k_shaped": Workload("amazon670k_shaped", 2, L=670_208, G=16, H=768, F=128, B=256, m=5),
    # Amazon-3M-shaped: 2,999,936 = 32 * 93,748 labels, ~36 positives/sample.
    "amazon3m_shaped": Workload("amazon3m_shaped", 3, L=2_999_936, G=32, H=768, F=64, B=128, m=36),
    # LF-Paper2Keywords-8.6M-shaped: 8,601,600 = 64 * 134,400 labels.
    "lfpaper8600k_shaped": Workload("lfpaper8600k_shaped", 4, L=8_601_600, G=64, H=768, F=64, B=64, m=5),
    # Sparse tail of a 3M label space after moving the 3 % most frequent
    # labels (89,088) to a dense head: 2,910,848 tail labels, divisible by
    # 16, 32 and 64.  G here is the default of the G sweep.  The ~36
    # positives per sample are drawn over all 2,999,936 labels and split.
    "ht3m_tail_shaped": Workload("ht3m_tail_shaped", 5, L=2_910_848, G=32, H=768, F=64, B=128, m=36,
                                 head_labels=89_088),
    # Small head-tail split for parity tests: 1,504 tail labels (G = 16,
    # F = 32) and a 73-label dense head over H = 96 features.
    "ht_small": Workload("ht_small", 6, L=1_504, G=16, H=96, F=32, B=37, m=9, head_labels=73),
}

HT3M_FULL_LABELS = 2_999_936
HT3M_HEAD_LABELS = 89_088


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        d = dict(w.__dict__)
        d.update(overrides)
        w = Workload(**d)
    return w
