"""GPU parity: pf_score_select and pf_selection_deltas against the oracle."""
import numpy as np
import pytest
import torch

import bounded_kv_cache_pf_amd as pf
import oracle as O
import pfgen
from gpu_util import dev, dev_i32, say

pytestmark = pytest.mark.gpu

FLAG_GAP = 1e-3


def _select(c, n_c, k):
    ids, scores = pf.pf_score_select(dev(c["q"]), dev(c["pool_k"]), n_c, k)
    return ids.cpu().numpy().tolist(), scores.cpu().numpy().astype(np.float64)


def _compare(c, n_c, k, require_unflagged=False):
    ref_s = O.block_scores(c["q"], c["pool_k"], n_c)
    ref_ids = O.select_topk(ref_s, k)
    gap = O.topk_gap(ref_s, k)
    ids, s = _select(c, n_c, k)
    err = float(np.max(np.abs(s - ref_s)))
    flagged = gap < FLAG_GAP
    say(f"  select: M={len(ref_s)} k={k} score max-abs err {err:.2e}, spread {np.ptp(ref_s):.3e}, "
        f"k/k+1 gap {gap:.3e}{' FLAGGED' if flagged else ''}")
    assert err <= 1e-5 + 1e-5 * float(np.max(np.abs(ref_s)))
    assert ids == sorted(ids) and len(set(ids)) == k
    # the ranking is exact at every size, near-ties included: the ids are the
    # top-k of the scores the call returned, by (-score, index)
    assert ids == O.select_topk(s, k)
    if require_unflagged:
        assert not flagged
    if flagged:
        assert O.topk_acceptable(ids, ref_s, k, FLAG_GAP)
    else:
        assert ids == ref_ids
    return ids, flagged


@pytest.mark.parametrize("cfg", [pfgen.C0, pfgen.C1, pfgen.C2, pfgen.C2Q], ids=lambda c: c.name)
def test_select_configs(cfg):
    say(f"test_select_configs {cfg.name}")
    for seed in (cfg.seed, cfg.seed + 1, cfg.seed + 2):
        _compare(pfgen.make(cfg, seed), cfg.n_c, cfg.top_k)


def test_select_planted_answer_full_size():
    say("test_select_planted_answer_full_size")
    cfg = pfgen.C2
    chosen = [0, 9, 17, 30, 41, 42, 43, 57, 60, 71, 88, 90, 99, 100, 114, 115]
    c = pfgen.planted_pool(cfg, 77, chosen, margin=4.0)
    ids, _ = _compare(c, cfg.n_c, 16, require_unflagged=True)
    assert ids == chosen


def test_select_ties_go_to_lower_index():
    say("test_select_ties_go_to_lower_index")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    s = O.block_scores(c["q"], c["pool_k"], cfg.n_c)
    order = np.argsort(-s, kind="stable")
    kth = int(order[15])                     # the last block that makes the top 16
    dup = int(order[-1])                     # the lowest-ranked block, outside the top 16
    n = cfg.n_c
    pk = c["pool_k"].copy()
    pk[dup * n:(dup + 1) * n] = pk[kth * n:(kth + 1) * n]
    c2 = dict(c, pool_k=pk)
    ids, scores = _select(c2, n, 16)
    assert scores[dup] == scores[kth]          # identical blocks, identical fp32 scores
    ref = O.select_topk(O.block_scores(c2["q"], pk, n), 16)
    assert ids == ref
    assert min(kth, dup) in ids and max(kth, dup) not in ids


def test_select_k_equals_m_and_limits():
    say("test_select_k_equals_m_and_limits")
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    ids, _ = _select(c, cfg.n_c, cfg.pool_blocks)
    assert ids == list(range(cfg.pool_blocks))
    # the largest pool and top-k the library accepts (tiny blocks keep it fast)
    rng = np.random.default_rng(21)
    q = O.f64_to_bf16(rng.standard_normal((300, 2, 128)) + rng.standard_normal((1, 2, 128)))
    pk = O.f64_to_bf16(rng.standard_normal((4096 * 2, 2, 128)) + np.repeat(rng.standard_normal((4096, 1, 2, 128)), 2, axis=1).reshape(-1, 2, 128))
    _compare({"q": q, "pool_k": pk}, 2, 256)
    _compare({"q": q, "pool_k": pk[:2 * 1000]}, 2, 1)


@pytest.mark.parametrize("heads,M", [(1, 24), (3, 24), (5, 24), (32, 24), (1, 300), (2, 700)])
def test_select_head_counts(heads, M):
    # one score thread per four columns, rounded up to whole waves: 1, 3 and 5
    # heads leave part of the last wave without columns. A one-layer call with
    # at most 512 blocks ranks in its last score workgroup, by counting when
    # the blocks fit one per thread and by sorting when they do not (1 head,
    # 300 blocks); 700 blocks take the separate top-k launch.
    say(f"test_select_head_counts heads={heads} M={M}")
    rng = np.random.default_rng(100 + heads + M)
    n_c = 20 if M < 100 else 4
    q = O.f64_to_bf16(rng.standard_normal((150, heads, 128)) + rng.standard_normal((1, heads, 128)))
    off = np.repeat(rng.standard_normal((M, 1, heads, 128)) * 0.5, n_c, axis=1).reshape(-1, heads, 128)
    pk = O.f64_to_bf16(rng.standard_normal((M * n_c, heads, 128)) + off)
    _compare({"q": q, "pool_k": pk}, n_c, 6)


def test_select_repeatable_bits():
    say("test_select_repeatable_bits")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    q, pk = dev(c["q"]), dev(c["pool_k"])
    a = pf.pf_score_select(q, pk, cfg.n_c, 16)[1].cpu().numpy()
    b = pf.pf_score_select(q, pk, cfg.n_c, 16)[1].cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("cfg", [pfgen.C1, pfgen.C2], ids=lambda c: c.name)
def test_deltas_match_oracle_over_steps(cfg):
    say(f"test_deltas_match_oracle_over_steps {cfg.name}")
    M, k, Bf = cfg.pool_blocks, cfg.top_k, cfg.block_frames
    tags = O.initial_pos_tags(M, cfg.sink_blocks, Bf)
    tags_dev = dev_i32(tags)
    Fr = (cfg.sink_blocks + M) * Bf
    rng = np.random.default_rng(cfg.seed)
    for step in range(5):
        ids = sorted(rng.choice(M, k, replace=False).tolist())
        d_ref, tags = O.placement_deltas(ids, tags, Fr, Bf)
        d = pf.pf_selection_deltas(dev_i32(ids), tags_dev, Fr, Bf)
        assert d.cpu().numpy().tolist() == d_ref.tolist()
        assert tags_dev.cpu().numpy().tolist() == tags.tolist()


def test_deltas_invalid_ids():
    say("test_deltas_invalid_ids")
    tags = dev_i32([8, 12, 4, 20])
    d = pf.pf_selection_deltas(dev_i32([-3, 2, 9]), tags, 24, 4)
    # r = 1: target 24 - (3 - 1) * 4 = 16, delta 16 - 4; out-of-range ids get 0
    assert d.cpu().numpy().tolist() == [0, 12, 0]
    assert tags.cpu().numpy().tolist() == [8, 12, 16, 20]


def test_select_batched_equals_single_calls():
    say("test_select_batched_equals_single_calls")
    cfg = pfgen.C2Q
    B = 3
    cs = [pfgen.make(cfg, cfg.seed + b) for b in range(B)]
    rows = cfg.pool_blocks * cfg.n_c
    q = dev(np.stack([c["q"] for c in cs]))
    slab = dev(np.stack([np.concatenate([c["pool_k"], c["pool_k"][:cfg.n_c]]) for c in cs]))  # one spare block
    ids, scores = pf.pf_score_select_batched(q, slab[:, :rows], cfg.n_c, cfg.top_k)
    ids, scores = ids.cpu().numpy(), scores.cpu().numpy()
    for b, c in enumerate(cs):
        i1, s1 = _select(c, cfg.n_c, cfg.top_k)
        assert ids[b].tolist() == i1
        assert np.array_equal(scores[b].view(np.uint32), s1.astype(np.float32).view(np.uint32))
        _compare(c, cfg.n_c, cfg.top_k)
    tags = torch.stack([dev_i32(O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks, cfg.block_frames))] * B)
    fr = (cfg.sink_blocks + cfg.pool_blocks) * cfg.block_frames
    d = pf.pf_selection_deltas_batched(dev_i32(ids), tags, fr, cfg.block_frames).cpu().numpy()
    for b in range(B):
        d_ref, t_ref = O.placement_deltas(ids[b].tolist(), O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks,
                                                                              cfg.block_frames), fr, cfg.block_frames)
        assert d[b].tolist() == d_ref.tolist()
        assert tags[b].cpu().numpy().tolist() == t_ref.tolist()


@pytest.mark.parametrize("steps", [(1, 1), (4, 2), (3, 5), (7, 1)])
def test_select_subsampled(steps):
    q_step, head_step = steps
    say(f"test_select_subsampled q_step={q_step} head_step={head_step}")
    cfg = pfgen.C2Q
    c = pfgen.make(cfg)
    ref_s = O.block_scores(c["q"], c["pool_k"], cfg.n_c, q_step=q_step, head_step=head_step)
    ids, s = pf.pf_score_select_sub(dev(c["q"]), dev(c["pool_k"]), cfg.n_c, cfg.top_k, q_step, head_step)
    ids, s = ids.cpu().numpy().tolist(), s.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(s - ref_s)))
    gap = O.topk_gap(ref_s, cfg.top_k)
    say(f"  score max-abs err {err:.2e}, k/k+1 gap {gap:.3e}")
    assert err <= 1e-5 + 1e-5 * float(np.max(np.abs(ref_s)))
    assert ids == O.select_topk(s, cfg.top_k)
    if gap >= FLAG_GAP:
        assert ids == O.select_topk(ref_s, cfg.top_k)
    else:
        assert O.topk_acceptable(ids, ref_s, cfg.top_k, FLAG_GAP)
    if steps == (1, 1):
        i1, s1 = _select(c, cfg.n_c, cfg.top_k)
        assert ids == i1 and np.array_equal(s.astype(np.float32).view(np.uint32), s1.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("cfg", [pfgen.C1, pfgen.C2Q, pfgen.C0], ids=lambda c: c.name)
def test_select_place_fused_equals_separate_calls(cfg):
    # the fused call gives the bits of pf_score_select + pf_selection_deltas,
    # over several steps in which the tags keep moving, and the oracle's ids/deltas
    say(f"test_select_place_fused_equals_separate_calls {cfg.name}")
    M, k, Bf = cfg.pool_blocks, cfg.top_k, cfg.block_frames
    fr = (cfg.sink_blocks + M) * Bf
    tags0 = O.initial_pos_tags(M, cfg.sink_blocks, Bf)
    t_fused, t_sep, t_ref = dev_i32(tags0), dev_i32(tags0), tags0
    for step in range(3):
        c = pfgen.make(cfg, cfg.seed + 40 + step)
        q, pk = dev(c["q"]), dev(c["pool_k"])
        ids_f, d_f, s_f = pf.pf_select_place(q, pk, cfg.n_c, k, t_fused, fr, Bf)
        ids_s, s_s = pf.pf_score_select(q, pk, cfg.n_c, k)
        d_s = pf.pf_selection_deltas(ids_s, t_sep, fr, Bf)
        assert ids_f.cpu().numpy().tolist() == ids_s.cpu().numpy().tolist()
        assert np.array_equal(s_f.cpu().numpy().view(np.uint32), s_s.cpu().numpy().view(np.uint32))
        assert d_f.cpu().numpy().tolist() == d_s.cpu().numpy().tolist()
        assert t_fused.cpu().numpy().tolist() == t_sep.cpu().numpy().tolist()
        ids, flagged = _compare(c, cfg.n_c, k)
        assert ids == ids_f.cpu().numpy().tolist()
        d_ref, t_ref = O.placement_deltas(ids, t_ref, fr, Bf)
        assert d_f.cpu().numpy().tolist() == d_ref.tolist()
        assert t_fused.cpu().numpy().tolist() == t_ref.tolist()


@pytest.mark.parametrize("B", [4, 6])
def test_select_place_batched_equals_single_calls(B):
    # 4 caches x 116 blocks rank in their last score workgroups; 6 caches
    # (696 score workgroups) take the separate top-k launch
    say(f"test_select_place_batched_equals_single_calls B={B}")
    cfg = pfgen.C2
    cs = [pfgen.make(cfg, cfg.seed + 60 + b) for b in range(B)]
    M, k, Bf = cfg.pool_blocks, cfg.top_k, cfg.block_frames
    fr = (cfg.sink_blocks + M) * Bf
    tags0 = O.initial_pos_tags(M, cfg.sink_blocks, Bf)
    q = dev(np.stack([c["q"] for c in cs]))
    pk = dev(np.stack([c["pool_k"] for c in cs]))
    tags = torch.stack([dev_i32(tags0)] * B)
    ids, d, s = pf.pf_select_place_batched(q, pk, cfg.n_c, k, tags, fr, Bf)
    for b, c in enumerate(cs):
        t1 = dev_i32(tags0)
        i1, d1, s1 = pf.pf_select_place(dev(c["q"]), dev(c["pool_k"]), cfg.n_c, k, t1, fr, Bf)
        assert ids[b].cpu().numpy().tolist() == i1.cpu().numpy().tolist()
        assert d[b].cpu().numpy().tolist() == d1.cpu().numpy().tolist()
        assert np.array_equal(s[b].cpu().numpy().view(np.uint32), s1.cpu().numpy().view(np.uint32))
        assert tags[b].cpu().numpy().tolist() == t1.cpu().numpy().tolist()
        assert ids[b].cpu().numpy().tolist() == O.select_topk(s[b].cpu().numpy().astype(np.float64), k)


def test_random_selector_matches_oracle_bit_exact():
    # the random-selection baseline: the same counter-based stream and Floyd
    # steps on both sides, so the ids agree exactly for every stream
    say("test_random_selector_matches_oracle_bit_exact")
    for n_blocks, k, seed in ((40, 16, 1234), (116, 16, 99), (10, 4, 0), (16, 16, 5), (4096, 256, 2 ** 63 + 17),
                              (1, 1, 3)):
        nb = 7
        got = pf.pf_select_random(n_blocks, k, seed, 1000, n_batch=nb).cpu().numpy()
        for b in range(nb):
            assert got[b].tolist() == O.select_random(n_blocks, k, seed, 1000 + b), (n_blocks, k, seed, b)
    one = pf.pf_select_random(40, 16, 1234, 1000).cpu().numpy().tolist()
    assert one == O.select_random(40, 16, 1234, 1000)
