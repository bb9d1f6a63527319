"""Oracle attention: two formulations, a library routine, closed forms.

Definition: softmax(Q K^T / sqrt(d_h)) V over the concatenated context
[digest 前置知识 KV缓存; arXiv "Bounded Attention Context"].
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import pfgen


def _bits(rng, shape, scale=1.0):
    return O.f64_to_bf16(rng.standard_normal(shape) * scale)


def _c0_parts(seed=1000):
    cfg = pfgen.C0
    c = pfgen.make(cfg, seed)
    ids = [1, 3, 6, 8]
    ks, vs = O.partitions(c, cfg.n_c, ids)
    return c, ks, vs


def test_partitioned_equals_bruteforce_c0():
    c, ks, vs = _c0_parts()
    o1, l1 = O.attn_bruteforce(c["q"], ks, vs)
    o2, l2 = O.attn_partitioned(c["q"], ks, vs)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


def _torch_sdpa(q_bits, ks, vs):
    q = torch.from_numpy(O.bf16_to_f64(q_bits)).permute(1, 0, 2)      # [H, n_q, D]
    k = torch.from_numpy(O.bf16_to_f64(np.concatenate(ks))).permute(1, 0, 2)
    v = torch.from_numpy(O.bf16_to_f64(np.concatenate(vs))).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    return o.permute(1, 0, 2).numpy()


def test_against_torch_sdpa_fp64():
    c, ks, vs = _c0_parts()
    o, _ = O.attn_partitioned(c["q"], ks, vs)
    assert np.max(np.abs(o - _torch_sdpa(c["q"], ks, vs))) < 1e-12


def test_loop_definition_tiny():
    # pure-Python loops over a 2-query, 5-key, 1-head case in three partitions
    rng = np.random.default_rng(2)
    q = _bits(rng, (2, 1, 128))
    ks = [_bits(rng, (2, 1, 128)), _bits(rng, (1, 1, 128)), _bits(rng, (2, 1, 128))]
    vs = [_bits(rng, (2, 1, 128)), _bits(rng, (1, 1, 128)), _bits(rng, (2, 1, 128))]
    K = [row for p in ks for row in O.bf16_to_f64(p)[:, 0, :].tolist()]
    V = [row for p in vs for row in O.bf16_to_f64(p)[:, 0, :].tolist()]
    Q = O.bf16_to_f64(q)[:, 0, :].tolist()
    o, _ = O.attn_partitioned(q, ks, vs)
    for i in range(2):
        logits = [sum(a * b for a, b in zip(Q[i], K[t])) / math.sqrt(128) for t in range(5)]
        w = [math.exp(x) for x in logits]
        z = sum(w)
        for d in range(128):
            ref = sum(w[t] * V[t][d] for t in range(5)) / z
            assert abs(o[i, 0, d] - ref) < 1e-12


def test_zero_queries_give_mean_of_values():
    c, ks, vs = _c0_parts()
    q0 = np.zeros_like(c["q"])
    o, lse = O.attn_partitioned(q0, ks, vs)
    mean_v = O.bf16_to_f64(np.concatenate(vs)).mean(axis=0)
    assert np.max(np.abs(o - mean_v[None])) < 1e-12
    assert np.max(np.abs(lse - math.log(1056))) < 1e-12


def test_boosted_key_dominates():
    rng = np.random.default_rng(8)
    H = 1
    q = np.zeros((1, H, 128))
    q[0, 0, 0] = 1.0
    keys = np.zeros((50, H, 128))
    keys[17, 0, 0] = 30.0 * math.sqrt(128)     # logit 30 against 0 for the rest
    vals = rng.standard_normal((50, H, 128))
    qb, kb, vb = O.f64_to_bf16(q), O.f64_to_bf16(keys), O.f64_to_bf16(vals)
    o, _ = O.attn_partitioned(qb, [kb[:20], kb[20:]], [vb[:20], vb[20:]])
    v17 = O.bf16_to_f64(vb[17])
    assert np.max(np.abs(o[0] - v17)) < 60 * math.exp(-30) * 10


def test_invariant_to_key_order_and_partitioning():
    c, ks, vs = _c0_parts()
    K, V = np.concatenate(ks), np.concatenate(vs)
    perm = np.random.default_rng(9).permutation(K.shape[0])
    K2, V2 = K[perm], V[perm]
    o1, _ = O.attn_partitioned(c["q"], ks, vs)
    o2, _ = O.attn_partitioned(c["q"], [K2[:100], K2[100:101], K2[101:]], [V2[:100], V2[100:101], V2[101:]])
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_mid_gather_uses_ids():
    cfg = pfgen.C0
    c = pfgen.make(cfg)
    mid = O.gather_mid(c["pool_k"], cfg.n_c, [6, 2])
    assert np.array_equal(mid[:8], c["pool_k"][48:56])
    assert np.array_equal(mid[8:], c["pool_k"][16:24])
    assert O.gather_mid(c["pool_k"], cfg.n_c, []).shape[0] == 0


def _mut_no_scale(q, ks, vs):
    return O.attn_partitioned(q, ks, vs, scale=1.0)


def _mut_drop_partition(q, ks, vs):
    return O.attn_partitioned(q, ks[:-1], vs[:-1])


def _mut_transposed_v(q, ks, vs):
    # V rows taken from the key array: a swapped operand
    return O.attn_partitioned(q, ks, ks)


def _mut_separate_softmax(q, ks, vs):
    # one softmax per partition, averaged, instead of one over the concatenation
    outs = [O.attn_bruteforce(q, [k], [v])[0] for k, v in zip(ks, vs) if k.shape[0]]
    return sum(outs) / len(outs), None


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_drop_partition, _mut_transposed_v,
                                    _mut_separate_softmax])
def test_planted_mistakes_fail_library_pin(mutant):
    c, ks, vs = _c0_parts()
    o, _ = mutant(c["q"], ks, vs)
    assert np.max(np.abs(o - _torch_sdpa(c["q"], ks, vs))) > 1e-3
