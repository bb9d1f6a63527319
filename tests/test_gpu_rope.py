"""GPU parity: pf_rope_shift against the oracle's temporal rotation."""
import numpy as np
import pytest
import torch

import bounded_kv_cache_pf_amd as pf
import oracle as O
import pfgen
from gpu_util import dev, dev_i32, host, say, ulp_diff

pytestmark = pytest.mark.gpu


def _check(pool_bits, n_c, ids, deltas, base=10000.0, block_ids_null=False):
    ref = O.rope_shift_blocks(pool_bits, n_c, ids, deltas, base)
    k = dev(pool_bits)
    pf.pf_rope_shift(k, n_c, dev_i32(deltas), None if block_ids_null else dev_i32(ids), base)
    got = host(k)
    assert np.array_equal(got[..., 44:], pool_bits[..., 44:]), "dims 44..127 must be untouched"
    ud = ulp_diff(got[..., :44], ref[..., :44])
    exact = float((ud == 0).mean())
    say(f"  rope: {len(ids)} blocks, max ulp {ud.max()}, exact fraction {exact:.6f}")
    assert ud.max() <= 1
    assert exact > 0.999
    return got


@pytest.mark.parametrize("cfg", [pfgen.C0, pfgen.C1, pfgen.C2], ids=lambda c: c.name)
def test_rope_shift_configs(cfg):
    say(f"test_rope_shift_configs {cfg.name}")
    c = pfgen.make(cfg)
    rng = np.random.default_rng(cfg.seed)
    ids = sorted(rng.choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
    if cfg.delta_range is not None:
        deltas = c["deltas"].tolist()
    else:
        tags = O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks, cfg.block_frames)
        deltas, _ = O.placement_deltas(ids, tags, (cfg.sink_blocks + cfg.pool_blocks) * cfg.block_frames,
                                       cfg.block_frames)
        deltas = deltas.tolist()
    got = _check(c["pool_k"], cfg.n_c, ids, deltas)
    untouched = np.ones(cfg.pool_blocks, bool)
    untouched[ids] = False
    rows = np.repeat(untouched, cfg.n_c)
    assert np.array_equal(got[rows], c["pool_k"][rows])


def test_rope_shift_negative_large_and_zero_deltas():
    say("test_rope_shift_negative_large_and_zero_deltas")
    rng = np.random.default_rng(3)
    pool = O.f64_to_bf16(rng.standard_normal((12 * 7, 3, 128)))
    _check(pool, 7, [0, 3, 5, 11], [-480, 0, 480, 100000])


def test_rope_shift_slab_mode_and_ragged_rows():
    # block_ids NULL: blocks 0..n_shift-1; one block of 12,480 rows is the sink slab
    say("test_rope_shift_slab_mode_and_ragged_rows")
    rng = np.random.default_rng(4)
    sink = O.f64_to_bf16(rng.standard_normal((12480, 12, 128)) / np.sqrt(2))
    _check(sink, 12480, [0], [8], block_ids_null=True)
    odd = O.f64_to_bf16(rng.standard_normal((5 * 131, 5, 128)))
    _check(odd, 131, [0, 1, 2], [3, -7, 11], block_ids_null=True)


def test_rope_shift_invalid_ids_are_skipped():
    say("test_rope_shift_invalid_ids_are_skipped")
    rng = np.random.default_rng(5)
    pool = O.f64_to_bf16(rng.standard_normal((10 * 8, 2, 128)))
    k = dev(pool)
    pf.pf_rope_shift(k, 8, dev_i32([5, 5, 5]), dev_i32([-1, 10, 1 << 30]))
    assert np.array_equal(host(k), pool)


def test_rope_shift_other_base():
    say("test_rope_shift_other_base")
    rng = np.random.default_rng(6)
    pool = O.f64_to_bf16(rng.standard_normal((6 * 16, 4, 128)))
    _check(pool, 16, [1, 4], [9, 33], base=500000.0)


def test_rope_shift_batched_equals_single_calls():
    say("test_rope_shift_batched_equals_single_calls")
    B, M, n_c, H, k = 5, 12, 7, 3, 4
    rng = np.random.default_rng(11)
    pools = O.f64_to_bf16(rng.standard_normal((B, M * n_c + 3, H, 128)))   # slabs with 3 spare rows
    ids = np.stack([np.sort(rng.choice(M, k, replace=False)) for _ in range(B)]).astype(np.int32)
    deltas = rng.integers(-200, 200, (B, k)).astype(np.int32)
    ids[2, 1] = M + 5                       # out of range: skipped
    deltas[3, 0] = 0                        # identity
    slab = dev(pools)
    view = slab[:, :M * n_c]
    pf.pf_rope_shift_batched(view, n_c, dev_i32(deltas), dev_i32(ids))
    got = host(slab)
    for b in range(B):
        one = dev(pools[b, :M * n_c])
        pf.pf_rope_shift(one, n_c, dev_i32(deltas[b]), dev_i32(ids[b]))
        assert np.array_equal(got[b, :M * n_c], host(one)), b
        ok = [i for i in ids[b].tolist() if 0 <= i < M]
        dl = [int(d) for i, d in zip(ids[b].tolist(), deltas[b].tolist()) if 0 <= i < M]
        ref = O.rope_shift_blocks(pools[b, :M * n_c], n_c, ok, dl)
        assert ulp_diff(got[b, :M * n_c], ref).max() <= 1
        assert np.array_equal(got[b, M * n_c:], pools[b, M * n_c:]), "rows past the view must not move"


def test_sink_shift_after_eviction_batched_over_layers():
    """The pages' eviction event: every layer's sink slab moves forward by
    delta = evicted blocks x B_f frames, in one batched call (block_ids NULL:
    the whole slab is one block)."""
    say("test_sink_shift_after_eviction_batched_over_layers")
    cfg = pfgen.C1
    L, n_evict = 3, 2
    rng = np.random.default_rng(12)
    sinks = O.f64_to_bf16(rng.standard_normal((L, cfg.n_sink, cfg.heads, 128)) / np.sqrt(2))
    pool = np.zeros((4 * cfg.n_c, cfg.heads, 128), dtype=np.uint16)
    tags = O.initial_pos_tags(4, cfg.sink_blocks, cfg.block_frames)
    ref = [O.evict_and_shift_sink(sinks[l], pool, pool, tags, n_evict, cfg.n_c, cfg.block_frames) for l in range(L)]
    k = dev(sinks)
    deltas = dev_i32([[ref[0]["delta"]]] * L)
    pf.pf_rope_shift_batched(k, cfg.n_sink, deltas)
    got = host(k)
    for l in range(L):
        ud = ulp_diff(got[l], ref[l]["sink_k"])
        say(f"  layer {l}: delta {ref[l]['delta']}, max ulp {ud.max()}, exact {(ud == 0).mean():.6f}")
        assert ud.max() <= 1 and (ud == 0).mean() > 0.999
