"""GPU parity of the whole layer-step path: select -> place -> shift -> attend.

Every stage's output is compared with the oracle's, which follows its own state
from the same seeded inputs.
"""
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
