"""GPU parity: pf_partition_attn against the oracle's softmax attention."""
import numpy as np
import pytest
import torch

import bounded_kv_cache_pf_amd as pf
import oracle as O
import pfgen
from gpu_util import MAX_ABS, MEAN_ABS, REL_L2, attn_errors, dev, dev_i32, host, say

pytestmark = pytest.mark.gpu


def _run(c, n_c, ids, want_lse=True, scale=0.0):
    mid = dev_i32(ids) if len(ids) else None
    o, lse = pf.pf_partition_attn(dev(c["q"]), dev(c["sink_k"]), dev(c["sink_v"]),
                                  dev(c["pool_k"]) if len(ids) else None,
                                  dev(c["pool_v"]) if len(ids) else None, n_c, mid,
                                  dev(c["recent_k"]), dev(c["recent_v"]), dev(c["cur_k"]), dev(c["cur_v"]),
                                  scale=scale, want_lse=want_lse)
    torch.cuda.synchronize()
    return host(o), (lse.cpu().numpy() if lse is not None else None)


def _compare(c, n_c, ids, rows=None, label=""):
    o, lse = _run(c, n_c, ids)
    ks, vs = O.partitions(c, n_c, ids)
    q = c["q"] if rows is None else c["q"][rows]
    ref, ref_lse = O.attn_partitioned(q, ks, vs)
    got = o if rows is None else o[rows]
    got_lse = lse if rows is None else lse[:, rows]
    mx, mean, rel = attn_errors(got, ref)
    lse_err = float(np.max(np.abs(got_lse - ref_lse)))
    say(f"  attn {label}: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e} lse {lse_err:.2e} "
        f"(|O| rms {np.sqrt(np.mean(ref ** 2)):.3e})")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2
    assert lse_err <= 1e-3
    return o


def _sample_rows(n_q, seed=0, extra=48):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, n_q // 2, n_q - 97, n_q - 96, n_q - 33, n_q - 32, n_q - 1]
    rows = set(r for r in fixed if 0 <= r < n_q) | set(rng.integers(0, n_q, extra).tolist())
    return np.array(sorted(rows))


def test_attn_c0_all_rows():
    say("test_attn_c0_all_rows")
    cfg = pfgen.C0
    for seed in (1000, 1001, 1002):
        c = pfgen.make(cfg, seed)
        ids = sorted(np.random.default_rng(seed).choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
        _compare(c, cfg.n_c, ids, label=f"C0 seed {seed}")


@pytest.mark.parametrize("cfg", [pfgen.C1, pfgen.C2], ids=lambda c: c.name)
def test_attn_full_size_sampled_rows(cfg):
    say(f"test_attn_full_size_sampled_rows {cfg.name}")
    c = pfgen.make(cfg)
    ids = sorted(np.random.default_rng(cfg.seed).choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
    _compare(c, cfg.n_c, ids, rows=_sample_rows(cfg.n), label=cfg.name)


def test_attn_default_layer_all_rows():
    # every one of the 6,240 x 12 query rows of the default layer against the
    # oracle (about 20 s of fp64 on the host), so full-size parity does not
    # rest on sampled rows alone
    say("test_attn_default_layer_all_rows")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    ids = sorted(np.random.default_rng(cfg.seed + 3).choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
    _compare(c, cfg.n_c, ids, label="C1 all rows")


def test_attn_sharp_scores():
    # Q x 8: score std ~4, a peaked softmax that exercises the running-max rescale
    say("test_attn_sharp_scores")
    cfg = pfgen.C1.replace(q_mult=8.0)
    c = pfgen.make(cfg)
    ids = list(range(0, 40, 3))[:16]
    _compare(c, cfg.n_c, ids, rows=_sample_rows(cfg.n, 1), label="C1 q*8")


def test_attn_ragged_shapes_and_empty_partitions():
    say("test_attn_ragged_shapes_and_empty_partitions")
    rng = np.random.default_rng(7)

    def bits(rows, H=3):
        return O.f64_to_bf16(rng.standard_normal((rows, H, 128)))
    base = dict(q=bits(200), sink_k=bits(77), sink_v=bits(77), pool_k=bits(9 * 13), pool_v=bits(9 * 13),
                recent_k=bits(65), recent_v=bits(65), cur_k=bits(200), cur_v=bits(200))
    _compare(base, 13, [8, 0, 4], label="ragged")                      # unsorted ids are fine
    e = dict(base, sink_k=bits(0), sink_v=bits(0))
    _compare(e, 13, [1, 2], label="no sink")
    _compare(base, 13, [], label="no mid")
    e = dict(base, sink_k=bits(0), sink_v=bits(0), recent_k=bits(0), recent_v=bits(0))
    _compare(e, 13, [3], label="mid + cur only")
    e = dict(base, q=bits(1), cur_k=bits(1), cur_v=bits(1), sink_k=bits(0), sink_v=bits(0),
             recent_k=bits(0), recent_v=bits(0))
    _compare(e, 13, [], label="one query, one key")


def test_attn_zero_queries_mean_of_values():
    say("test_attn_zero_queries_mean_of_values")
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    c["q"] = np.zeros_like(c["q"])
    ids = [0, 2, 4, 6]
    o, lse = _run(c, cfg.n_c, ids)
    ks, vs = O.partitions(c, cfg.n_c, ids)
    mean_v = O.bf16_to_f64(np.concatenate(vs)).mean(axis=0)
    assert np.max(np.abs(O.bf16_to_f64(o) - mean_v[None])) < 1e-3
    assert np.max(np.abs(lse - np.log(1056))) < 1e-4


def test_attn_invalid_ids_are_masked():
    say("test_attn_invalid_ids_are_masked")
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    o_bad, _ = _run(c, cfg.n_c, [1, -5, 3, 99])
    ks, vs = O.partitions(c, cfg.n_c, [1, 3])
    ref, _ = O.attn_partitioned(c["q"], ks, vs)
    mx, mean, rel = attn_errors(o_bad, ref)
    assert mx <= MAX_ABS and rel <= REL_L2


def test_attn_invalid_ids_in_whole_mid_tiles():
    # At C1 sizes 22 key tiles hold mid rows only; their loads resolve rows through the
    # ids. Two invalid ids fall inside such tiles: their rows are masked, as if absent.
    say("test_attn_invalid_ids_in_whole_mid_tiles")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    ids = list(range(0, 2 * cfg.top_k, 2))
    ids[3], ids[9] = -1, cfg.pool_blocks + 7
    valid = [i for i in ids if 0 <= i < cfg.pool_blocks]
    o, lse = _run(c, cfg.n_c, ids)
    rows = _sample_rows(cfg.n, 5, extra=16)
    ks, vs = O.partitions(c, cfg.n_c, valid)
    ref, ref_lse = O.attn_partitioned(c["q"][rows], ks, vs)
    mx, mean, rel = attn_errors(o[rows], ref)
    lse_err = float(np.max(np.abs(lse[:, rows] - ref_lse)))
    say(f"  attn C1 with 2 invalid ids: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e} lse {lse_err:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2
    assert lse_err <= 1e-3


def test_attn_gather_equals_copy():
    # reading the pool through ids == attending over the copied rows as a partition
    say("test_attn_gather_equals_copy")
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    ids = [7, 2, 5, 9]
    o1, _ = _run(c, cfg.n_c, ids)
    mid_k = O.gather_mid(c["pool_k"], cfg.n_c, ids)
    mid_v = O.gather_mid(c["pool_v"], cfg.n_c, ids)
    c2 = dict(c, sink_k=np.concatenate([c["sink_k"], mid_k]), sink_v=np.concatenate([c["sink_v"], mid_v]))
    o2, _ = _run(c2, cfg.n_c, [])
    assert np.array_equal(o1, o2)


def test_attn_unbounded_c4_sampled_rows():
    say("test_attn_unbounded_c4_sampled_rows (generating 748,800 keys)")
    cfg = pfgen.C4
    c = pfgen.make(cfg)
    _compare(c, cfg.n_c, [], rows=_sample_rows(cfg.n, 4, extra=8), label="C4 748,800 keys")


def _bits(rng, rows, H, scale=1.0):
    return O.f64_to_bf16(rng.standard_normal((rows, H, 128)) * scale)


@pytest.mark.parametrize("H", [1, 32])
def test_attn_head_count_limits(H):
    say(f"test_attn_head_count_limits H={H}")
    rng = np.random.default_rng(20 + H)
    n_q = 300 if H == 32 else 1000
    c = dict(q=_bits(rng, n_q, H), sink_k=_bits(rng, 130, H), sink_v=_bits(rng, 130, H),
             pool_k=_bits(rng, 6 * 11, H), pool_v=_bits(rng, 6 * 11, H), recent_k=_bits(rng, 70, H),
             recent_v=_bits(rng, 70, H), cur_k=_bits(rng, 90, H), cur_v=_bits(rng, 90, H))
    _compare(c, 11, [5, 1, 3], rows=_sample_rows(n_q, H), label=f"H={H}")


def test_attn_32_heads_whole_partition_and_mid_tiles():
    # 32 heads (row stride 8 KB) with partitions long enough that whole key tiles lie
    # inside the sink, inside the mid blocks and inside recent/current: every loader path
    say("test_attn_32_heads_whole_partition_and_mid_tiles")
    rng = np.random.default_rng(41)
    H, n_c, n_q = 32, 160, 300
    c = dict(q=_bits(rng, n_q, H), sink_k=_bits(rng, 640, H), sink_v=_bits(rng, 640, H),
             pool_k=_bits(rng, 6 * n_c, H), pool_v=_bits(rng, 6 * n_c, H), recent_k=_bits(rng, 300, H),
             recent_v=_bits(rng, 300, H), cur_k=_bits(rng, 400, H), cur_v=_bits(rng, 400, H))
    _compare(c, n_c, [4, 0, 5, 2], rows=_sample_rows(n_q, 41, extra=8), label="H=32, 1,980 keys")


def test_attn_max_selected_blocks_duplicates_and_scale():
    say("test_attn_max_selected_blocks_duplicates_and_scale")
    rng = np.random.default_rng(31)
    H, n_c = 2, 2
    c = dict(q=_bits(rng, 130, H), sink_k=_bits(rng, 5, H), sink_v=_bits(rng, 5, H),
             pool_k=_bits(rng, 1200 * n_c, H), pool_v=_bits(rng, 1200 * n_c, H), recent_k=_bits(rng, 3, H),
             recent_v=_bits(rng, 3, H), cur_k=_bits(rng, 7, H), cur_v=_bits(rng, 7, H))
    ids = rng.integers(0, 1200, 1024).tolist()          # PF_MAX_SELECTED ids, repeats allowed
    _compare(c, n_c, ids, label="1024 selected blocks with repeats")
    o, lse = _run(c, n_c, ids, scale=0.03)
    ks, vs = O.partitions(c, n_c, ids)
    # the oracle applies 1/sqrt(128); fold the requested scale into its queries
    qs = O.f64_to_bf16(O.bf16_to_f64(c["q"]) * (0.03 * np.sqrt(128.0)))
    ref, _ = O.attn_partitioned(qs, ks, vs)
    # the scaled queries were rounded to bf16 for the reference: allow that rounding
    mx, mean, rel = attn_errors(o, ref)
    say(f"  scale 0.03: max-abs {mx:.2e} rel-L2 {rel:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2


def test_attn_whole_rounds_and_tail_only_plans():
    # 256 units = exactly the resident workgroups (one round, no tail), and 240
    # units (no whole round: every unit runs whole in the tail slots)
    say("test_attn_whole_rounds_and_tail_only_plans")
    rng = np.random.default_rng(41)
    for H, n_q in ((32, 2048), (20, 3000)):
        c = dict(q=_bits(rng, n_q, H, 0.7), sink_k=_bits(rng, 256, H, 0.7), sink_v=_bits(rng, 256, H, 0.7),
                 pool_k=_bits(rng, 4 * 9, H, 0.7), pool_v=_bits(rng, 4 * 9, H, 0.7), recent_k=_bits(rng, 64, H, 0.7),
                 recent_v=_bits(rng, 64, H, 0.7), cur_k=_bits(rng, 100, H, 0.7), cur_v=_bits(rng, 100, H, 0.7))
        _compare(c, 9, [3, 0], rows=_sample_rows(n_q, H, extra=16), label=f"H={H} n_q={n_q}")


@pytest.mark.parametrize("n_q,H,n_keys", [(3136, 20, 4000), (1100, 7, 20000), (6300, 12, 6000), (100, 5, 3000)],
                         ids=["partial-units-in-round-and-tail", "two-kinds-7-and-6-segments",
                              "five-live-waves", "one-partial-unit-per-head"])
def test_attn_tail_plans_with_partial_query_units(n_q, H, n_keys):
    # n_q not a multiple of 256: each head's last query unit is partial and its
    # waves past n_q only load. With 256 resident workgroups these shapes put
    # partial units in a whole round and in a tail of their own (3136 x 20),
    # cut full and partial tail units into 7 and 6 key segments (1100 x 7),
    # give partial units five live waves (6300 x 12), and leave no full unit
    # (100 x 5); on any machine they cover partial units with 1..8 live waves
    say(f"test_attn_tail_plans_with_partial_query_units n_q={n_q} H={H} keys={n_keys}")
    rng = np.random.default_rng(n_q + H)
    n_c, ids = 100, [7, 2, 11, 4]
    n_sink, n_rec = 256, 300
    n_cur = n_keys - n_sink - n_rec - len(ids) * n_c
    c = dict(q=_bits(rng, n_q, H, 0.7), sink_k=_bits(rng, n_sink, H, 0.7), sink_v=_bits(rng, n_sink, H, 0.7),
             pool_k=_bits(rng, 12 * n_c, H, 0.7), pool_v=_bits(rng, 12 * n_c, H, 0.7),
             recent_k=_bits(rng, n_rec, H, 0.7), recent_v=_bits(rng, n_rec, H, 0.7),
             cur_k=_bits(rng, n_cur, H, 0.7), cur_v=_bits(rng, n_cur, H, 0.7))
    rows = _sample_rows(n_q, n_q, extra=24)
    rows = np.union1d(rows, np.arange(max(0, n_q - 40), n_q))
    _compare(c, n_c, ids, rows=rows, label=f"n_q={n_q} H={H} keys={n_keys}")


@pytest.mark.parametrize("boost", [20.0, 70.0])
def test_attn_late_dominant_keys(boost):
    # a few keys near the end of the context score `boost` nats above the rest:
    # the running max must move up by far more than the lazy-rescale slack
    # (70 nats = 101 in log2 units) after many tiles have been accumulated
    say(f"test_attn_late_dominant_keys boost {boost}")
    rng = np.random.default_rng(int(boost))
    H, n_q = 2, 300
    u = rng.standard_normal((H, 128))
    q = O.f64_to_bf16(u[None] + 0.1 * rng.standard_normal((n_q, H, 128)))
    qf = O.bf16_to_f64(q).mean(axis=0)                      # [H][128]
    cur = 0.3 * rng.standard_normal((400, H, 128))
    for key in (390, 391, 396):
        cur[key] = qf * (boost * np.sqrt(128.0) / np.sum(qf * qf, axis=1))[:, None]
    c = dict(q=q, sink_k=_bits(rng, 1000, H, 0.3), sink_v=_bits(rng, 1000, H),
             pool_k=_bits(rng, 4 * 20, H, 0.3), pool_v=_bits(rng, 4 * 20, H),
             recent_k=_bits(rng, 500, H, 0.3), recent_v=_bits(rng, 500, H),
             cur_k=O.f64_to_bf16(cur), cur_v=_bits(rng, 400, H))
    _compare(c, 20, [1, 3], label=f"late keys +{boost} nats")


def test_attn_and_select_on_a_side_stream_without_workspace():
    # the binding allocates the workspace and outputs while the kernels run on
    # a stream other than the current one; memory the current stream allocates
    # and overwrites right after the calls must not be the memory those kernels
    # still use
    say("test_attn_and_select_on_a_side_stream_without_workspace")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    ids = sorted(np.random.default_rng(5).choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
    t = {k: dev(v) for k, v in c.items()}
    mid = dev_i32(ids)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    need = pf.pf_partition_attn_workspace_bytes(cfg.n, cfg.heads, cfg.n_keys)
    assert need > 0
    o, lse = pf.pf_partition_attn(t["q"], t["sink_k"], t["sink_v"], t["pool_k"], t["pool_v"], cfg.n_c, mid,
                                  t["recent_k"], t["recent_v"], t["cur_k"], t["cur_v"], want_lse=True, stream=side)
    sel, scores = pf.pf_score_select(t["q"], t["pool_k"], cfg.n_c, cfg.top_k, stream=side)
    junk = [torch.full((need,), 255, dtype=torch.uint8, device="cuda") for _ in range(4)]
    junk += [torch.full(tuple(o.shape), -7, dtype=torch.int16, device="cuda") for _ in range(2)]
    side.synchronize()
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.n, 9, extra=16)
    ks, vs = O.partitions(c, cfg.n_c, ids)
    ref, ref_lse = O.attn_partitioned(c["q"][rows], ks, vs)
    mx, mean, rel = attn_errors(host(o)[rows], ref)
    say(f"  side stream: max-abs {mx:.3e} rel-L2 {rel:.3e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2
    assert float(np.max(np.abs(lse.cpu().numpy()[:, rows] - ref_lse))) <= 1e-3
    s_ref = O.block_scores(c["q"], c["pool_k"], cfg.n_c)
    got = sel.cpu().numpy().tolist()
    err = float(np.max(np.abs(scores.cpu().numpy().astype(np.float64) - s_ref)))
    assert err <= 1e-5 + 1e-5 * float(np.max(np.abs(s_ref)))
    if O.topk_gap(s_ref, cfg.top_k) < 1e-3:      # flagged: any set within the margin
        assert O.topk_acceptable(got, s_ref, cfg.top_k, 1e-3)
    else:
        assert got == O.select_topk(s_ref, cfg.top_k)
    del junk
