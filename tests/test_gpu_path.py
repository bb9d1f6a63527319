"""GPU parity of the whole layer-step path: select -> place -> shift -> attend.

Every stage's output is compared with the oracle's, which follows its own state
from the same seeded inputs.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bounded_kv_cache_pf_amd as pf
import oracle as O
import pfgen
from gpu_util import MAX_ABS, MEAN_ABS, REL_L2, attn_errors, dev, dev_i32, host, say, ulp_diff

pytestmark = pytest.mark.gpu


class DeviceLayer:
    """One layer's cache on the device plus its pool position tags."""

    def __init__(self, c, cfg):
        self.cfg = cfg
        self.t = {k: dev(v) for k, v in c.items() if k != "deltas"}
        self.tags = dev_i32(O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks, cfg.block_frames))

    def step(self, q=None):
        cfg, t = self.cfg, self.t
        q = t["q"] if q is None else q
        M = t["pool_k"].shape[0] // cfg.n_c
        ids, scores = pf.pf_score_select(q, t["pool_k"], cfg.n_c, cfg.top_k)
        fr = (cfg.sink_blocks + M) * cfg.block_frames
        deltas = pf.pf_selection_deltas(ids, self.tags, fr, cfg.block_frames)
        pf.pf_rope_shift(t["pool_k"], cfg.n_c, deltas, ids)
        o, lse = pf.pf_partition_attn(q, t["sink_k"], t["sink_v"], t["pool_k"], t["pool_v"], cfg.n_c, ids,
                                      t["recent_k"], t["recent_v"], t["cur_k"], t["cur_v"], want_lse=True)
        return ids, scores, deltas, o, lse


def check_step(label, cfg, c_ref, tags_ref, dl, out, rows):
    ids, scores, deltas, o, lse = out
    fr = (cfg.sink_blocks + c_ref["pool_k"].shape[0] // cfg.n_c) * cfg.block_frames
    ref = O.layer_step(c_ref, tags_ref, cfg.n_c, cfg.top_k, fr, cfg.block_frames, q_rows=rows)
    ids = ids.cpu().numpy().tolist()
    # exact ranking of the scores the call returned, near-ties included
    assert ids == O.select_topk(scores.cpu().numpy().astype(np.float64), cfg.top_k)
    flagged = ref["gap"] < 1e-3
    if ids != ref["ids"]:
        assert flagged and O.topk_acceptable(ids, ref["scores"], cfg.top_k, 1e-3), (ids, ref["ids"])
        say(f"  {label}: flagged near-tie chose another valid set; downstream not comparable")
        return None
    assert deltas.cpu().numpy().tolist() == ref["deltas"].tolist()
    assert dl.tags.cpu().numpy().tolist() == ref["tags"].tolist()
    ud = ulp_diff(host(dl.t["pool_k"]), ref["pool_k"])
    assert ud.max() <= 1, ud.max()
    mx, mean, rel = attn_errors(host(o)[rows], ref["o"])
    lse_err = float(np.max(np.abs(lse.cpu().numpy()[:, rows] - ref["lse"])))
    say(f"  {label}: ids ok (gap {ref['gap']:.2e}{' flagged' if flagged else ''}), pool max ulp {ud.max()}, "
        f"attn max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e} lse {lse_err:.1e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2 and lse_err <= 1e-3
    return ref


@pytest.mark.parametrize("cfg", [pfgen.C0, pfgen.C1, pfgen.C2, pfgen.C2Q], ids=lambda c: c.name)
def test_layer_step(cfg):
    say(f"test_layer_step {cfg.name}")
    if cfg is pfgen.C0:
        cfg = cfg.replace(delta_range=None)
    c = pfgen.make(cfg)
    c.pop("deltas", None)
    dl = DeviceLayer(c, cfg)
    rows = np.unique(np.r_[0, 33, 127, 128, cfg.n - 1, np.random.default_rng(0).integers(0, cfg.n, 24)])
    tags = O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks, cfg.block_frames)
    ref = check_step(cfg.name, cfg, c, tags, dl, dl.step(), rows)
    # a second step on the shifted pool with fresh queries: deltas can now be negative
    if ref is not None:
        rng = np.random.default_rng(cfg.seed + 5)
        q2 = pfgen.bf16_bits(rng.standard_normal((cfg.n, cfg.heads, 128)).astype(np.float32) * cfg.scale
                             + (rng.standard_normal((1, cfg.heads, 128)).astype(np.float32)
                                if cfg.query_offset_std else 0))
        c2 = dict(c, q=q2, pool_k=ref["pool_k"])
        check_step(cfg.name + " step 2", cfg, c2, ref["tags"], dl, dl.step(dev(q2)), rows)


def test_full_generation_step_c3():
    """30 layers x 4 denoising steps at the 116-block pool shapes, then the roll-in
    of one compressed block per layer and one step of the next block on the
    117-block pool. Selection, placement and the shift run batched over the
    layers; every layer's ids, deltas, tags and shifted pool are compared with
    the oracle at every step, and attention on sampled rows for three layers."""
    cfg = pfgen.C3
    L, S, M, n_c, k, Bf, H = cfg.layers, cfg.steps, cfg.pool_blocks, cfg.n_c, cfg.top_k, cfg.block_frames, cfg.heads
    Sb = cfg.sink_blocks
    attn_layers = (0, L // 2, L - 1)
    # unit edges, and the last (partial) 256-query unit of a head, whose waves
    # past the last query only load
    rows = np.unique(np.r_[0, 127, 128, 255, 256, cfg.n - 96, cfg.n - 33, cfg.n - 1,
                           np.random.default_rng(1).integers(0, cfg.n, 8)])
    say(f"test_full_generation_step_c3: {L} layers x {S} steps, pool {M} -> {M + 1}")

    pool_rows = (M + 1) * n_c
    pool_k_dev = torch.zeros((L, pool_rows, H, 128), dtype=torch.int16, device="cuda")
    pool_v_dev = torch.zeros_like(pool_k_dev)
    ref_pool_k, ref_pool_v, ref_tags, full = [], [], [], {}
    for l in range(L):
        c = pfgen.make_cache(cfg, pfgen.layer_seed(cfg, l))
        pool_k_dev[l, :M * n_c] = dev(c["pool_k"])
        pool_v_dev[l, :M * n_c] = dev(c["pool_v"])
        ref_pool_k.append(c["pool_k"])
        ref_pool_v.append(c["pool_v"])
        ref_tags.append(O.initial_pos_tags(M, Sb, Bf))
        if l in attn_layers:
            full[l] = {"host": c, "dev": {n: dev(c[n]) for n in ("sink_k", "sink_v", "recent_k", "recent_v",
                                                                   "cur_k", "cur_v")}}
    say("  caches ready")
    tags_dev = dev_i32(np.stack(ref_tags))
    diverged = set()

    def run_step(step, n_blocks, fr):
        qs = [pfgen.step_queries(cfg, l, step) for l in range(L)]
        q_dev = dev(np.stack(qs))
        view_k = pool_k_dev[:, :n_blocks * n_c]
        ids, sc = pf.pf_score_select_batched(q_dev, view_k, n_c, k)
        deltas = pf.pf_selection_deltas_batched(ids, tags_dev, fr, Bf)
        pf.pf_rope_shift_batched(view_k, n_c, deltas, ids)
        outs = {}
        for l in attn_layers:
            d = full[l]["dev"]
            outs[l] = pf.pf_partition_attn(q_dev[l], d["sink_k"], d["sink_v"], view_k[l],
                                           pool_v_dev[l, :n_blocks * n_c], n_c, ids[l], d["recent_k"],
                                           d["recent_v"], d["cur_k"], d["cur_v"])[0]
        ids_h, deltas_h, tags_h = ids.cpu().numpy(), deltas.cpu().numpy(), tags_dev.cpu().numpy()
        sc_h = sc.cpu().numpy().astype(np.float64)
        for l in range(L):   # exact ranking of each layer's returned scores
            assert ids_h[l].tolist() == O.select_topk(sc_h[l], k), (step, l)
        pools_h = {l: host(pool_k_dev[l, :n_blocks * n_c]) for l in range(L) if l not in diverged}
        o_h = {l: host(outs[l])[rows] for l in attn_layers}

        def check_layer(l):
            """Oracle step of layer l against the device results (runs in a worker thread)."""
            scores = O.block_scores(qs[l], ref_pool_k[l], n_c)
            ref_ids = O.select_topk(scores, k)
            gap = O.topk_gap(scores, k)
            res = {"flagged": gap < 1e-3, "diverged": False, "attn": None}
            if ids_h[l].tolist() != ref_ids:
                assert gap < 1e-3 and O.topk_acceptable(ids_h[l].tolist(), scores, k, 1e-3), (step, l)
                res["diverged"] = True
                return res
            d_ref, ref_tags[l] = O.placement_deltas(ref_ids, ref_tags[l], fr, Bf)
            assert deltas_h[l].tolist() == d_ref.tolist(), (step, l)
            assert tags_h[l].tolist() == ref_tags[l].tolist(), (step, l)
            ref_pool_k[l] = O.rope_shift_blocks(ref_pool_k[l], n_c, ref_ids, d_ref.tolist())
            got = pools_h[l]
            sel = np.zeros(n_blocks, bool)
            sel[ref_ids] = True
            sel = np.repeat(sel, n_c)
            assert ulp_diff(got[sel], ref_pool_k[l][sel]).max() <= 1, (step, l)
            assert np.array_equal(got[~sel], ref_pool_k[l][~sel]), (step, l)
            if l in attn_layers:
                cache = dict(full[l]["host"], q=qs[l], pool_k=ref_pool_k[l], pool_v=ref_pool_v[l])
                ks, vs = O.partitions(cache, n_c, ref_ids)
                o_ref, _ = O.attn_partitioned(qs[l][rows], ks, vs)
                res["attn"] = attn_errors(o_h[l], o_ref)
            return res

        live = [l for l in range(L) if l not in diverged]
        with ThreadPoolExecutor(max_workers=8) as ex:
            results = dict(zip(live, ex.map(check_layer, live)))
        worst = 0.0
        for l, r in results.items():
            if r["diverged"]:
                say(f"  step {step} layer {l}: flagged near-tie chose another valid set; layer no longer compared")
                diverged.add(l)
            if r["attn"] is not None:
                mx, mean, rel = r["attn"]
                worst = max(worst, mx)
                assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2, (step, l, mx, mean, rel)
        say(f"  step {step}: {L - len(diverged)} of {L} layers match the oracle (ids, deltas, tags, pool bits), "
            f"{sum(r['flagged'] for r in results.values())} flagged near-ties, "
            f"attention max-abs {worst:.2e} on layers {attn_layers}")

    fr = (Sb + M) * Bf
    for step in range(S):
        run_step(step, M, fr)
    # roll-in: the recent block leaves the window and joins the pool compressed
    blocks = [pfgen.rollin_block(cfg, l) for l in range(L)]
    tags_dev = torch.cat([tags_dev, torch.zeros((L, 1), dtype=torch.int32, device="cuda")], dim=1).contiguous()
    pf.pf_rollin_batched(pool_k_dev, pool_v_dev, tags_dev, M, dev(np.stack([b["k"] for b in blocks])),
                         dev(np.stack([b["v"] for b in blocks])), fr)
    for l, blk in enumerate(blocks):
        ref_pool_k[l], ref_pool_v[l], ref_tags[l] = O.rollin(ref_pool_k[l], ref_pool_v[l], ref_tags[l], blk["k"],
                                                             blk["v"], fr)
    assert tags_dev.cpu().numpy().tolist() == [t.tolist() for t in ref_tags]
    assert np.array_equal(host(pool_v_dev[:, M * n_c:]), np.stack([b["v"] for b in blocks]))
    say("  rolled in one block per layer")
    run_step(S, M + 1, fr + Bf)
    assert len(diverged) <= 2


def test_rollin_on_a_second_stream_during_attention():
    """The roll-in writes the slot after the pool's last block on its own stream
    while attention reads the earlier slots: both results are exact."""
    say("test_rollin_on_a_second_stream_during_attention")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    M, n_c = cfg.pool_blocks, cfg.n_c
    t = {k: dev(v) for k, v in c.items() if k != "deltas"}
    pk = torch.cat([t["pool_k"], torch.zeros_like(t["pool_k"][:n_c])]).contiguous()
    pv = torch.cat([t["pool_v"], torch.zeros_like(t["pool_v"][:n_c])]).contiguous()
    tags = dev_i32(np.r_[O.initial_pos_tags(M, cfg.sink_blocks, cfg.block_frames), -1])
    blk = pfgen.rollin_block(cfg, 0)
    bk, bv = dev(blk["k"]), dev(blk["v"])
    ids = dev_i32(list(range(0, 32, 2)))
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    o, _ = pf.pf_partition_attn(t["q"], t["sink_k"], t["sink_v"], pk[:M * n_c], pv[:M * n_c], n_c, ids,
                                t["recent_k"], t["recent_v"], t["cur_k"], t["cur_v"])
    with torch.cuda.stream(side):
        pf.pf_rollin(pk, pv, tags, M, bk, bv, 1234)
    torch.cuda.synchronize()
    assert np.array_equal(host(pk[M * n_c:]), blk["k"]) and np.array_equal(host(pv[M * n_c:]), blk["v"])
    assert np.array_equal(host(pk[:M * n_c]), c["pool_k"])
    assert tags.cpu().numpy().tolist()[M] == 1234
    rows = np.r_[0, 1, 1000, cfg.n - 1]
    ks, vs = O.partitions(c, n_c, list(range(0, 32, 2)))
    ref, _ = O.attn_partitioned(c["q"][rows], ks, vs)
    mx, mean, rel = attn_errors(host(o)[rows], ref)
    say(f"  attention alongside the roll-in: max-abs {mx:.2e} rel-L2 {rel:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2
