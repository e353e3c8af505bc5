"""GPU parity of the semantic label grouping (haste_kmeans_assign,
haste_kmeans_init, haste_kmeans_update, haste_group_greedy) against the CPU
oracle, through the C ABI.  Integer-valued embeddings make every dot
product exact in fp32, so assignments, ties and groups are checked bit for
bit; on unit-vector embeddings the floating-point results are checked
within tolerance and the decisions wherever the oracle's are not near ties."""

import numpy as np
import pytest

import group_shared_fixed_amd as hs
from gpu_util import assert_parity, say, to_dev_bf16, to_dev_i32, to_host
from oracle import oracle as O
from synthetic import bf16_bits, kmeans_draws, label_embeddings

pytestmark = pytest.mark.gpu


def _int_emb(L, H, seed, lo=-2, hi=3):
    return bf16_bits(np.random.default_rng(seed).integers(lo, hi, size=(L, H)).astype(np.float32))


def assert_assign_valid(a, S, eps, what):
    """Every assignment takes a centre whose score is within eps of the row's
    best (the oracle's pick up to a near tie)."""
    rows = np.arange(S.shape[0])
    gap = S.max(axis=1) - S[rows, a]
    bad = np.nonzero(gap > eps)[0]
    assert bad.size == 0, f"{what}: {bad.size} assignments miss the best score by > {eps}, first {bad[:5]}"


def assert_greedy_valid(E, a, C, G, perm, clusters, eps):
    """Replays the greedy rule on the given clusters with the GPU's own picks:
    within a cluster the groups come in order, each lists its members in
    increasing id, its seed is the lowest-id member not yet grouped (exact),
    and each of the other G - 1 members is an ungrouped member of the cluster
    whose similarity with the seed is within eps of the (G - 1)-th largest
    among the ungrouped candidates (the oracle's pick up to a near tie).  The
    leftovers of all clusters follow the greedy groups in (cluster, id) order
    when every cluster is replayed."""
    Ef = O._bf16_f64(E)
    L = E.shape[0]
    sizes = np.bincount(a, minlength=C)
    n_c = sizes // G
    gbase = np.concatenate([[0], np.cumsum(n_c)[:-1]]).astype(np.int64)
    near = 0
    leftovers = {}
    for c in clusters:
        members = np.nonzero(a == c)[0]
        free = np.ones(L, bool)
        for k in range(int(n_c[c])):
            g = perm[(gbase[c] + k) * G:(gbase[c] + k + 1) * G]
            assert list(g) == sorted(g), f"cluster {c} group {k} not in increasing id"
            assert (a[g] == c).all(), f"cluster {c} group {k} takes a label of another cluster"
            assert free[g].all(), f"cluster {c} group {k} reuses a grouped label"
            cand = members[free[members]]
            seed = cand[0]
            assert seed in g, f"cluster {c} group {k}: seed {seed} missing"
            others = cand[1:]
            sim = Ef[others] @ Ef[seed]
            t = np.sort(sim)[::-1][G - 2]
            picked = np.isin(others, g)
            assert picked.sum() == G - 1
            worst = sim[picked].min()
            assert worst >= t - eps, f"cluster {c} group {k}: a pick {t - worst:.3e} below the (G-1)-th best"
            near += int(worst < t)
            free[g] = False
        leftovers[c] = members[free[members]]
    if len(clusters) == C:
        rest = np.concatenate([leftovers[c] for c in range(C)])
        assert np.array_equal(perm[int(n_c.sum()) * G:], rest), "leftovers not in (cluster, id) order"
    return near


@pytest.mark.parametrize("L,C,H", [(3000, 37, 64), (513, 5, 8), (4096, 300, 128), (2600, 700, 200),
                                   # one label and one centre; H at its maximum; five centre tiles
                                   (1, 1, 8), (300, 2, 1024), (5000, 1200, 128)])
def test_kmeans_assign_integer_exact(L, C, H):
    E = _int_emb(L, H, 90 + C)
    M = _int_emb(C, H, 91 + C)
    M[C - 1] = M[0]                                # tied centres: the lower one wins
    a, s = hs.kmeans_assign(to_dev_bf16(E), to_dev_bf16(M), want_score=True)
    ra, rs = O.oracle_kmeans_assign(E, M)
    assert (to_host(a) == ra).all(), "assignments differ"
    assert (to_host(s).astype(np.float64) == rs).all(), "scores differ"
    rows = np.sort(np.random.default_rng(C).choice(L, size=max(L // 3, 1), replace=False)).astype(np.int32)
    a2, _ = hs.kmeans_assign(to_dev_bf16(E), to_dev_bf16(M), rows=to_dev_i32(rows))
    assert (to_host(a2) == ra[rows]).all(), "assignments of a row subset differ"


def test_kmeans_assign_unit_vectors():
    L, C, H = 6000, 64, 128
    E = label_embeddings(L, H, 40, 0.8, 92)
    init, _ = kmeans_draws(L, C, 16, 1, 92)
    M = np.ascontiguousarray(E[init])
    a, s = hs.kmeans_assign(to_dev_bf16(E), to_dev_bf16(M), want_score=True)
    a, s = to_host(a), to_host(s)
    S = O._bf16_f64(E) @ O._bf16_f64(M).T
    best = S.max(axis=1)
    assert (np.abs(S[np.arange(L), a] - best) <= 1e-5).all(), "an assignment misses the maximum"
    assert_parity(s, best, "scores", rel=1e-6, mabs=1e-5)
    ra, _ = O.oracle_kmeans_assign(E, M)
    srt = np.sort(S, axis=1)
    clear = srt[:, -1] - srt[:, -2] > 1e-5
    assert (a[clear] == ra[clear]).all()
    say(f"    {clear.sum()}/{L} labels without a near tie")


def test_kmeans_update_steps():
    """Three mini-batch steps; each checked against the oracle step run from
    the GPU's own centres and counts (so fp32 rounding does not compound)."""
    import torch

    L, C, H = 5000, 40, 96
    E = label_embeddings(L, H, 30, 0.7, 93)
    init, batches = kmeans_draws(L, C, 700, 3, 93)
    Ed = to_dev_bf16(E)
    Mc, Mb, v = hs.kmeans_init(Ed, to_dev_i32(init))
    assert (to_host(Mb) == E[init]).all() and (to_host(v) == 0).all()
    assert (to_host(Mc) == O._bf16_f64(E[init]).astype(np.float32)).all()
    for it, b in enumerate(batches):
        Mc0, v0 = to_host(Mc).astype(np.float64), to_host(v).astype(np.int64)
        a, _ = hs.kmeans_assign(Ed, Mb, rows=to_dev_i32(b))
        a_h = to_host(a)
        Sb = O._bf16_f64(E[b]) @ O._bf16_f64(to_host(Mb)).T
        assert_assign_valid(a_h, Sb, 1e-5, f"batch assignments of step {it}")
        hs.kmeans_update(Ed, to_dev_i32(b), a, Mc, Mb, v)
        want, want_v = O.oracle_kmeans_update(E, b, a_h, Mc0, v0)
        got = to_host(Mc).astype(np.float64)
        assert_parity(got, want, f"centres after step {it}", rel=1e-5, mabs=1e-5)
        assert (to_host(v) == want_v).all(), "counts"
        untouched = np.setdiff1d(np.arange(C), np.unique(a_h))
        assert (got[untouched] == Mc0[untouched]).all(), "centres without members changed"
        mb = to_host(Mb)
        assert (mb == bf16_bits(to_host(Mc))).all(), "Mb is not the bf16 rounding of Mc"
    torch.cuda.synchronize()


@pytest.mark.parametrize("L,C,H,G,big", [(2048, 13, 64, 16, 0), (1536, 7, 32, 32, 0), (4096, 40, 128, 64, 0),
                                         (960, 1, 16, 16, 0),
                                         # clusters past 1,024 members keep their per-member
                                         # state in the workspace instead of LDS
                                         (4096, 3, 32, 16, 1), (6144, 4, 64, 32, 1), (8192, 2, 32, 64, 1),
                                         (2048, 1, 16, 32, 1)])
def test_group_greedy_integer_exact(L, C, H, G, big):
    E = _int_emb(L, H, 94 + G, -1, 2)
    rng = np.random.default_rng(95 + C)
    a = rng.integers(0, C, size=L).astype(np.int32)
    if big:
        a[rng.random(L) < 0.7] = 0                 # cluster 0 holds ~70 % of the labels
        assert (a == 0).sum() > 1024
    perm = to_host(hs.group_greedy(to_dev_bf16(E), to_dev_i32(a), C, G))
    want = O.oracle_group_greedy(E, a, C, G)
    assert sorted(perm.tolist()) == list(range(L)), "not a permutation"
    bad = np.nonzero(perm != want)[0]
    assert bad.size == 0, f"{bad.size} positions differ, first at {bad[:5]}"


def test_group_greedy_unit_vectors_and_repeat():
    L, C, H, G = 8192, 48, 128, 32
    E = label_embeddings(L, H, 48, 0.6, 96)
    init, _ = kmeans_draws(L, C, 16, 1, 96)
    a, _ = O.oracle_kmeans_assign(E, np.ascontiguousarray(E[init]))
    Ed, ad = to_dev_bf16(E), to_dev_i32(a)
    p1 = to_host(hs.group_greedy(Ed, ad, C, G))
    p2 = to_host(hs.group_greedy(Ed, ad, C, G))
    assert (p1 == p2).all(), "grouping not repeatable"
    assert sorted(p1.tolist()) == list(range(L))
    want = O.oracle_group_greedy(E, a, C, G)
    same = np.mean([(p1[k * G:(k + 1) * G] == want[k * G:(k + 1) * G]).all() for k in range(L // G)])
    say(f"    {100 * same:.2f} % of groups identical to the oracle's")
    near = assert_greedy_valid(E, a, C, G, p1, list(range(C)), 1e-4)
    say(f"    every group valid; {near} decided within a near tie")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_grouping_fullsize_sampled():
    """Amazon-3M label count, H = 768, G = 32, C = L / (4 G) = 23,437
    clusters: init, two mini-batch steps of 65,536 labels, the full
    assignment and the greedy groups; sampled labels' assignments and
    sampled clusters' groups against the oracle, the whole permutation's
    structure checked."""
    L, H, G = 2_999_936, 768, 32
    C = L // (4 * G)
    say("  generating 3M embeddings")
    E = label_embeddings(L, H, 4096, 0.6, 97)
    init, batches = kmeans_draws(L, C, 65536, 2, 97)
    Ed = to_dev_bf16(E)
    Mc, Mb, v = hs.kmeans_init(Ed, to_dev_i32(init))
    for b in batches:
        a_b, _ = hs.kmeans_assign(Ed, Mb, rows=to_dev_i32(b))
        hs.kmeans_update(Ed, to_dev_i32(b), a_b, Mc, Mb, v)
    a_d, s_d = hs.kmeans_assign(Ed, Mb, want_score=True)
    a, s = to_host(a_d), to_host(s_d)
    M = to_host(Mb)
    rng = np.random.default_rng(98)
    sample = rng.choice(L, size=256, replace=False)
    S = O._bf16_f64(E[sample]) @ O._bf16_f64(M).T
    assert (np.abs(S[np.arange(256), a[sample]] - S.max(axis=1)) <= 1e-4).all(), "sampled assignments"
    say("  greedy groups")
    perm = to_host(hs.group_greedy(Ed, a_d, C, G))
    assert np.array_equal(np.sort(perm), np.arange(L)), "not a permutation"
    sizes = np.bincount(a, minlength=C)
    n_c = sizes // G
    gbase = np.concatenate([[0], np.cumsum(n_c)[:-1]])
    for k in range(0, int(n_c.sum()), max(1, int(n_c.sum()) // 500)):
        g = perm[k * G:(k + 1) * G]
        assert len(set(a[g].tolist())) == 1 and list(g) == sorted(g), f"group {k}"
    agree = 0
    cl = [int(c) for c in rng.choice(C, size=40, replace=False) if n_c[c] > 0]
    for c in cl:
        members = np.nonzero(a == c)[0]
        pad = (-members.size) % G                  # a second, padding cluster keeps L % G == 0
        sub = np.concatenate([E[members], np.zeros((pad, H), np.uint16)])
        sub_a = np.concatenate([np.zeros(members.size, np.int32), np.ones(pad, np.int32)])
        local = O.oracle_group_greedy(sub, sub_a, 2, G)
        want = members[local[:n_c[c] * G]]
        got = perm[gbase[c] * G:(gbase[c] + n_c[c]) * G]
        agree += int(np.array_equal(got, want))
    say(f"    {agree}/{len(cl)} sampled clusters identical to the oracle's groups")
    near = assert_greedy_valid(E, a, C, G, perm, cl, 1e-4)
    say(f"    every sampled cluster's groups valid; {near} picks decided within a near tie")
