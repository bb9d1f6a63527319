"""pf_partition_attn_noalloc (the entry point for callers that cannot
allocate) against pf_partition_attn on the same inputs: two calls in a row,
the second smaller, so the second runs on the scratch array the first left
behind."""
import numpy as np
import pytest
import torch

import bounded_kv_cache_pf_amd as pf
import oracle as O
import pfgen
from gpu_util import MAX_ABS, MEAN_ABS, REL_L2, attn_errors, dev, dev_i32, host, say

pytestmark = pytest.mark.gpu


def _inputs(c, ids):
    t = {k: dev(v) for k, v in c.items()}
    return (t["q"], t["sink_k"], t["sink_v"], t["pool_k"], t["pool_v"]), dev_i32(ids), \
        (t["recent_k"], t["recent_v"], t["cur_k"], t["cur_v"])


def _both(c, n_c, ids, label):
    (q, sk, sv, pk, pv), mid, rest = _inputs(c, ids)
    n_keys = sk.shape[0] + len(ids) * n_c + rest[0].shape[0] + rest[2].shape[0]
    need = pf.pf_partition_attn_workspace_bytes(q.shape[0], q.shape[1], n_keys)
    say(f"  {label}: {q.shape[0]} queries x {q.shape[1]} heads over {n_keys} keys, {need} bytes of partials")
    assert need > 0                                  # the shape uses the scratch array
    o_ref, lse_ref = pf.pf_partition_attn(q, sk, sv, pk, pv, n_c, mid, *rest, want_lse=True)
    o = torch.full_like(q, 0x7FBF)
    lse = torch.full((q.shape[1], q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    pf.pf_partition_attn_noalloc(q, sk, sv, pk, pv, n_c, mid, *rest, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
    return host(o)


def test_noalloc_equals_workspace_call_twice_second_smaller():
    say("test_noalloc_equals_workspace_call_twice_second_smaller")
    cfg = pfgen.C1
    c = pfgen.make(cfg)
    ids = sorted(np.random.default_rng(11).choice(cfg.pool_blocks, cfg.top_k, replace=False).tolist())
    o1 = _both(c, cfg.n_c, ids, "C1")
    rows = np.array([0, 1, 255, 256, 3000, 6143, 6144, 6239])
    ks, vs = O.partitions(c, cfg.n_c, ids)
    ref, _ = O.attn_partitioned(c["q"][rows], ks, vs)
    mx, mean, rel = attn_errors(o1[rows], ref)
    say(f"    oracle rows: max-abs {mx:.2e} rel-L2 {rel:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2

    rng = np.random.default_rng(12)
    H, n_c = 4, 20

    def bits(rows):
        return O.f64_to_bf16(rng.standard_normal((rows, H, 128)) * 0.7)
    small = dict(q=bits(1000), sink_k=bits(2500), sink_v=bits(2500), pool_k=bits(30 * n_c), pool_v=bits(30 * n_c),
                 recent_k=bits(1200), recent_v=bits(1200), cur_k=bits(1000), cur_v=bits(1000))
    sids = [2, 7, 11, 29]
    o2 = _both(small, n_c, sids, "smaller")
    ks, vs = O.partitions(small, n_c, sids)
    ref, _ = O.attn_partitioned(small["q"], ks, vs)
    mx, mean, rel = attn_errors(o2, ref)
    say(f"    oracle all rows: max-abs {mx:.2e} rel-L2 {rel:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2


def test_noalloc_refuses_without_output():
    q = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        pf.pf_partition_attn_noalloc(q, q, q, None, None, 8, None, None, None, q, q, o=None)
