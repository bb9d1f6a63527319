"""Oracle selection and placement.

Selection: query-key affinity over compressed mid blocks, top-k
[digest 方法步骤详情 (3); arXiv "Compressed Mid Tokens"]. The block score is the
stated reading: mean over heads of <mean-pooled Q, mean-pooled block keys>/sqrt(128).
Placement: the selected blocks are re-aligned to continuous positions
[summary "Method"; arXiv "Incremental RoPE adjustment"].
"""
import math

import numpy as np
import pytest

import oracle as O
import pfgen


def test_planted_answer_is_recovered():
    cfg = pfgen.C0.replace(pool_blocks=24, top_k=5)
    chosen = [2, 7, 11, 19, 23]
    c = pfgen.planted_pool(cfg, 11, chosen)
    s = O.block_scores(c["q"], c["pool_k"], cfg.n_c)
    assert O.select_topk(s, 5) == chosen
    assert O.topk_gap(s, 5) > 1.0


def test_double_sum_definition_tiny():
    # phi_j = sum_h sum_i sum_{t in block j} q_i . k_t / sqrt(128), in loops; it
    # equals n_q * N_c * H * s_j, so it ranks blocks identically.
    rng = np.random.default_rng(12)
    n_q, n_c, M, H = 4, 3, 5, 2
    q = O.f64_to_bf16(rng.standard_normal((n_q, H, 128)))
    kp = O.f64_to_bf16(rng.standard_normal((M * n_c, H, 128)))
    Q, K = O.bf16_to_f64(q).tolist(), O.bf16_to_f64(kp).tolist()
    s = O.block_scores(q, kp, n_c)
    for j in range(M):
        phi = 0.0
        for h in range(H):
            for i in range(n_q):
                for t in range(j * n_c, (j + 1) * n_c):
                    phi += sum(a * b for a, b in zip(Q[i][h], K[t][h])) / math.sqrt(128)
        assert phi == pytest.approx(n_q * n_c * H * s[j], rel=1e-12, abs=1e-12)


def test_ties_go_to_lower_index():
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    pk = c["pool_k"].copy()
    s = O.block_scores(c["q"], pk, cfg.n_c)
    best = int(np.argmax(s))
    dup = (best + 5) % cfg.pool_blocks
    pk[dup * 8:(dup + 1) * 8] = pk[best * 8:(best + 1) * 8]
    s2 = O.block_scores(c["q"], pk, cfg.n_c)
    assert s2[best] == s2[dup]
    assert O.select_topk(s2, 1) == [min(best, dup)]
    assert O.select_topk([1.0, 2.0, 2.0, 0.5], 2) == [1, 2]
    assert O.select_topk([2.0, 2.0, 2.0, 2.0], 3) == [0, 1, 2]


def test_k_equals_m_and_order():
    s = [0.3, -1.0, 5.0, 0.2]
    assert O.select_topk(s, 4) == [0, 1, 2, 3]
    assert O.select_topk(s, 2) == [0, 2]         # ascending block order
    assert O.topk_gap(s, 4) == math.inf
    assert O.topk_gap(s, 2) == pytest.approx(0.1)


def test_acceptable_sets():
    s = [1.0, 0.9995, 0.5, 0.2]
    assert O.topk_acceptable([0], s, 1, 1e-3)
    assert O.topk_acceptable([1], s, 1, 1e-3)      # within the near-tie window
    assert not O.topk_acceptable([2], s, 1, 1e-3)
    assert not O.topk_acceptable([0, 0], s, 2, 1e-3)


def test_placement_closed_form_first_use():
    M, k, Bf, Sb = 40, 16, 4, 2
    tags = O.initial_pos_tags(M, Sb, Bf)
    assert list(tags[:3]) == [8, 12, 16]             # sink holds frames 0..7
    rng = np.random.default_rng(0)
    ids = sorted(rng.choice(M, k, replace=False).tolist())
    Fr = (Sb + M) * Bf
    d, t = O.placement_deltas(ids, tags, Fr, Bf)
    for r, b in enumerate(ids):
        assert d[r] == (M - k + r - b) * Bf          # closed form from the initial tags
        assert d[r] >= 0
    sel = t[ids]
    assert list(np.diff(sel)) == [Bf] * (k - 1) and sel[-1] + Bf == Fr
    # selecting the newest k blocks needs no shift
    d2, _ = O.placement_deltas(list(range(M - k, M)), tags, Fr, Bf)
    assert not d2.any()


def test_placement_repeated_keeps_tags_consistent():
    M, k, Bf, Sb = 12, 4, 4, 2
    tags0 = O.initial_pos_tags(M, Sb, Bf)
    tags = tags0.copy()
    total = np.zeros(M, np.int64)
    Fr = (Sb + M) * Bf
    rng = np.random.default_rng(1)
    saw_negative = False
    for _ in range(6):
        ids = sorted(rng.choice(M, k, replace=False).tolist())
        d, tags = O.placement_deltas(ids, tags, Fr, Bf)
        total[ids] += d
        saw_negative |= bool((d < 0).any())
    assert np.array_equal(tags0 + total, tags)       # a tag is its start plus every shift
    assert saw_negative                               # later steps can move blocks back


def test_rollin_block_needs_no_shift_when_selected_last():
    # the block that just left the recent window sits directly before the new
    # recent block: chosen in the last slot, its delta is zero; the other
    # selected blocks are placed exactly as without it
    M, Sb, Bf, k = 6, 2, 4, 3
    n_c, H = 2, 1
    rng = np.random.default_rng(3)
    pk = rng.integers(0, 1 << 16, (M * n_c, H, 128), dtype=np.uint16)
    tags = O.initial_pos_tags(M, Sb, Bf)
    fr = (Sb + M) * Bf
    blk = rng.integers(0, 1 << 16, (n_c, H, 128), dtype=np.uint16)
    pk2, pv2, tags2 = O.rollin(pk, pk, tags, blk, blk, fr)
    assert pk2.shape == ((M + 1) * n_c, H, 128) and np.array_equal(pk2[M * n_c:], blk)
    assert tags2.tolist() == tags.tolist() + [fr]
    d, t = O.placement_deltas([1, 4, M], tags2, fr + Bf, Bf)
    assert d[-1] == 0 and t[M] == fr
    d_ref, _ = O.placement_deltas([1, 4], tags, fr, Bf)
    assert d[:2].tolist() == d_ref.tolist()


def test_subsampled_scores_closed_forms():
    # queries repeated in runs of s rows: every s-th row has the same mean, so
    # the sub-sampled score equals the full one; odd heads all zero: the
    # half-heads score is exactly twice the full one (mean over half the heads)
    rng = np.random.default_rng(9)
    H, n_c, M, s = 4, 3, 5, 4
    base = rng.standard_normal((6, H, 128))
    q = O.f64_to_bf16(np.repeat(base, s, axis=0))
    pk = O.f64_to_bf16(rng.standard_normal((M * n_c, H, 128)))
    full = O.block_scores(q, pk, n_c)
    assert np.allclose(O.block_scores(q, pk, n_c, q_step=s), full, rtol=1e-12, atol=1e-15)
    q2 = O.bf16_to_f64(q).copy()
    q2[:, 1::2] = 0.0
    q2 = O.f64_to_bf16(q2)
    assert np.allclose(O.block_scores(q2, pk, n_c, head_step=2), 2 * O.block_scores(q2, pk, n_c), rtol=1e-12,
                       atol=1e-15)


# ---- baseline selectors ([digest] 实验结果; [arXiv] "FIFO vs. Dynamic Context Selection") ----

def test_splitmix64_published_outputs():
    # the first outputs of SplitMix64 seeded with 0, as its reference
    # implementation prints them; draw i of stream (0, 0) is output i
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [O.random_draw(0, 0, i) for i in (1, 2, 3)] == want


def _all_draw_sequences(n, k):
    import itertools
    return itertools.product(*[range(n - k + r + 1) for r in range(k)])


@pytest.mark.parametrize("n,k", [(6, 3), (5, 1), (7, 2), (4, 4)])
def test_floyd_sampling_is_exactly_uniform(n, k):
    # with every step's draw ranging over all of 0..j, each k-subset comes out
    # the same number of times: (n!/(n-k)!) / C(n, k) = k!
    from collections import Counter
    from math import comb, factorial
    counts = Counter()
    for seq in _all_draw_sequences(n, k):
        sub = O.floyd_sample(n, k, lambda r, j, seq=seq: seq[r])
        assert len(sub) == k and sub == sorted(set(sub)) and all(0 <= x < n for x in sub)
        counts[tuple(sub)] += 1
    assert len(counts) == comb(n, k)
    assert set(counts.values()) == {factorial(k)}


def test_floyd_planted_mistake_breaks_uniformity():
    # keeping t when it is already present (a lost sample) or drawing from
    # 0..j-1 both break the exact count
    from collections import Counter

    def floyd_wrong_range(n, k, draw):
        kept = set()
        for r in range(k):
            j = n - k + r
            t = draw(r, j) % j if j else 0
            kept.add(j if t in kept else t)
        return sorted(kept)
    counts = Counter(tuple(floyd_wrong_range(6, 3, lambda r, j, s=s: s[r])) for s in _all_draw_sequences(6, 3))
    assert len(set(counts.values())) > 1


def test_select_random_properties():
    M, k = 40, 16
    seen = np.zeros(M)
    for counter in range(3000):
        ids = O.select_random(M, k, 1234, counter)
        assert len(ids) == k and ids == sorted(set(ids)) and 0 <= ids[0] and ids[-1] < M
        seen[ids] += 1
    # each block is chosen with probability k/M: 1200 of 3000, sd ~ 26.8
    assert np.max(np.abs(seen - 3000 * k / M)) < 5 * np.sqrt(3000 * (k / M) * (1 - k / M))
    assert O.select_random(M, M, 7, 0) == list(range(M))
    assert O.select_random(M, k, 7, 0) != O.select_random(M, k, 7, 1)
    assert O.select_random(M, k, 7, 0) == O.select_random(M, k, 7, 0)


def test_select_fifo_keeps_the_newest_blocks():
    assert O.select_fifo(40, 16) == list(range(24, 40))
    assert O.select_fifo(16, 16) == list(range(16))
