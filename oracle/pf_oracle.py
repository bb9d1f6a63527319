"""Plain CPU oracle for PackForcing's per-block context attention.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the bench's
CPU-baseline leg may import this module. The library never calls it, and it
shares no code with the HIP path: it reads the same bfloat16 bit arrays the GPU
reads, widens them to float64 and computes each step from its definition.

Sources (five web pages on PackForcing, arXiv 2603.25730):
  [digest]  "PackForcing：短视频训练即可实现长视频采样与长上下文推理"
            (paper.rainbus.top digest), sections 前置知识 (KV缓存, RoPE) and
            方法步骤详情 items (1)-(5).
  [arXiv]   "PackForcing: Short Video Training Suffices for Long Video Sampling
            and Long Context Inference" (arXiv HTML), paragraphs "KV Caching",
            "Sink Tokens", "Compressed Mid Tokens", "Recent & Current Tokens",
            "Bounded Attention Context", "The Position Misalignment Problem",
            "Incremental RoPE adjustment", "Implementation Details".
  [summary] openbayes English summary, "Method".
  The HR branch follows [arXiv] "HR Branch: Progressive 3D Convolution" and
  "Feature Fusion", and [digest] 前置知识 3D卷积.

Readings where the pages are silent:
  * RoPE frequencies: each axis a of width d_a uses theta_{a,j} = base^(-2j/d_a),
    j < d_a/2, base 10000 (RoFormer form); complex pairs are adjacent reals
    (2j, 2j+1); temporal pairs occupy dims 0..43, height 44..85, width 86..127.
  * Rotation sign: a shift by delta multiplies by e^{+i theta_t delta}, so a
    positive delta moves a key later in time.
  * Block score: s_j = mean over heads of <mean_i q_i, mean_{t in block j} k_t>
    / sqrt(128); top-k by (-s_j, j), so ties go to the lower block index; the
    ids come back sorted ascending.
  * Placement: the selected blocks, in chronological order, are laid end to end
    just before the recent block; delta is the block's target first frame minus
    the frame its keys currently encode.
  * Attention: one softmax over the concatenation sink || selected mid ||
    recent || current, no mask, scale 1/sqrt(128).

  * HR branch of the compressor: see its section below (kernel = stride, SiLU
    after each strided stage, a linear projection, bf16 storage per stage).

Parity unpinned (the pages do not fix these, so no test can pin them to the
pages): whether the scoring rule equals the paper's missing Sec. 3.5 rule, the
frequency base and pair layout of the paper's backbone, the placement rule, and
the HR branch's kernel sizes, widths and (trained) weights.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
# [digest] 前置知识 RoPE; [arXiv] "The Position Misalignment Problem":
# theta = [theta_t, theta_h, theta_w] allocated 44 + 42 + 42 = 128 dims per head.
T_DIMS, H_DIMS, W_DIMS = 44, 42, 42
ROPE_BASE = 10000.0


# ---------------------------------------------------------------------------
# bfloat16 storage
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> float64. Exact: bf16 is the top half of fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest, ties to even, in one rounding.

    bf16 keeps 8 significant bits. Write |x| = f * 2^e with f in [0.5, 1); the
    representable neighbours are multiples of 2^(e-8) (never finer than the
    subnormal quantum 2^-133). Dividing by a power of two is exact, and
    np.round rounds halves to even, so round(x / q) * q is the correctly rounded
    value; it has at most 8 significant bits, so the cast to float32 is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x / q) * q
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, x), r)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Token arithmetic  [arXiv] "KV Caching", "Compressed Mid Tokens",
# "Bounded Attention Context"; [digest] 方法步骤详情 (2), (5)
# ---------------------------------------------------------------------------

def tokens_per_block(block_frames: int, h: int, w: int) -> int:
    """n = B_f * h * w tokens per block after patchification."""
    return block_frames * h * w


def compressed_tokens(block_frames: int, h: int, w: int) -> int:
    """N_c = floor(B_f/2) * floor(h/4) * floor(w/4)."""
    return (block_frames // 2) * (h // 4) * (w // 4)


def context_size(n_sink_frames: int, n_mid: int, n_recent_frames: int,
                 block_frames: int, h: int, w: int) -> int:
    """|C| = (N_sink/B_f) n + N_mid N_c + (N_recent/B_f + 1) n."""
    n = tokens_per_block(block_frames, h, w)
    nc = compressed_tokens(block_frames, h, w)
    return (n_sink_frames // block_frames) * n + n_mid * nc + (n_recent_frames // block_frames + 1) * n


def kv_cache_bytes(tokens: int, layers: int, hidden: int, bytes_per_elem: int = 2) -> int:
    """K and V for every token, layer and hidden channel."""
    return tokens * layers * 2 * hidden * bytes_per_elem


# ---------------------------------------------------------------------------
# RoPE  [digest] 前置知识 RoPE; [arXiv] "The Position Misalignment Problem",
# "Incremental RoPE adjustment"; [digest] 方法步骤详情 (4)
# ---------------------------------------------------------------------------

def axis_freqs(axis_dims: int, base: float = ROPE_BASE) -> np.ndarray:
    j = np.arange(axis_dims // 2, dtype=np.float64)
    return base ** (-2.0 * j / axis_dims)


def _as_complex(k: np.ndarray) -> np.ndarray:
    return k[..., 0::2] + 1j * k[..., 1::2]


def _as_real(z: np.ndarray) -> np.ndarray:
    out = np.empty(z.shape[:-1] + (2 * z.shape[-1],), dtype=np.float64)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def rope_encode(k_raw: np.ndarray, p_t: float, p_h: float, p_w: float,
                base: float = ROPE_BASE) -> np.ndarray:
    """k^(p) = k_raw * e^{i theta p} with theta = [theta_t, theta_h, theta_w]."""
    ang = np.concatenate([axis_freqs(T_DIMS, base) * p_t,
                          axis_freqs(H_DIMS, base) * p_h,
                          axis_freqs(W_DIMS, base) * p_w])
    return _as_real(_as_complex(np.asarray(k_raw, np.float64)) * np.exp(1j * ang))


def rope_shift(k: np.ndarray, delta: float, base: float = ROPE_BASE) -> np.ndarray:
    """k' = k * e^{i(theta_t delta, 1_h, 1_w)}: rotate the 44 temporal dims only.

    The height and width entries are the identity rotation, so dims 44..127 are
    returned untouched.
    """
    k = np.array(k, dtype=np.float64, copy=True)
    zt = _as_complex(k[..., :T_DIMS]) * np.exp(1j * axis_freqs(T_DIMS, base) * delta)
    k[..., :T_DIMS] = _as_real(zt)
    return k


def rope_shift_blocks(pool_k_bits: np.ndarray, n_c: int, block_ids: Sequence[int],
                      deltas: Sequence[int], base: float = ROPE_BASE) -> np.ndarray:
    """Shift every row of each listed pool block by its delta; store as bf16.

    The pool is kept in bfloat16, so each shifted key is rounded back to bf16.
    A zero delta is the identity rotation and leaves the stored bits alone.
    Returns a new bit array; V is never rotated.
    """
    out = np.array(pool_k_bits, dtype=np.uint16, copy=True)
    for b, d in zip(block_ids, deltas):
        if int(d) == 0:
            continue
        rows = slice(int(b) * n_c, (int(b) + 1) * n_c)
        k = bf16_to_f64(out[rows])
        out[rows, ..., :T_DIMS] = f64_to_bf16(rope_shift(k, float(d), base)[..., :T_DIMS])
    return out


# ---------------------------------------------------------------------------
# Dynamic context selection  [digest] 方法步骤详情 (3); [arXiv] "Compressed Mid
# Tokens", "Implementation Details" (N_top = 16)
# ---------------------------------------------------------------------------

def block_scores(q_bits: np.ndarray, pool_k_bits: np.ndarray, n_c: int, q_step: int = 1,
                 head_step: int = 1) -> np.ndarray:
    """s_j = (1/H) sum_h <mean_i q_{i,h}, mean_{t in block j} k_{t,h}> / sqrt(128).

    q_step / head_step > 1: the pages' faster selection ([digest] 局限与改进:
    subsampled query tokens and half of the heads): only query rows 0, q_step,
    ... and heads 0, head_step, ... enter, and the means run over those.
    """
    q = bf16_to_f64(q_bits)[::q_step, ::head_step]          # [n_q', H', D]
    H = q.shape[1]
    k = bf16_to_f64(pool_k_bits)[:, ::head_step].reshape(-1, n_c, H, HEAD_DIM)
    q_mean = q.mean(axis=0)                       # [H, D]
    k_mean = k.mean(axis=1)                       # [M, H, D]
    per_head = np.einsum("hd,mhd->mh", q_mean, k_mean) / math.sqrt(HEAD_DIM)
    return per_head.mean(axis=1)


def select_topk(scores: Sequence[float], k: int) -> List[int]:
    """The k best blocks by (-score, index); returned in ascending block order."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def topk_gap(scores: Sequence[float], k: int) -> float:
    """Score gap between the k-th and (k+1)-th best blocks (inf when k == M)."""
    s = sorted((float(x) for x in scores), reverse=True)
    return math.inf if k >= len(s) else s[k - 1] - s[k]


def topk_acceptable(ids: Sequence[int], scores: Sequence[float], k: int, tol: float) -> bool:
    """A set G is acceptable when min_{g in G} s_g >= max_{b not in G} s_b - tol."""
    g = set(int(i) for i in ids)
    if len(g) != k or any(i < 0 or i >= len(scores) for i in g):
        return False
    rest = [scores[b] for b in range(len(scores)) if b not in g]
    if not rest:
        return True
    return min(scores[i] for i in g) >= max(rest) - tol


# ---------------------------------------------------------------------------
# Baseline selectors  [digest] 实验结果 (dynamic selection against FIFO and
# random selection); [arXiv] "FIFO vs. Dynamic Context Selection"
# ---------------------------------------------------------------------------
#
# Readings: FIFO keeps the k most recent pool blocks (the highest ids, since
# blocks enter the pool in arrival order). Random selection draws k distinct
# blocks uniformly; the pages name no generator, so the draws come from
# SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014) used as a counter-based stream, and the k-subset
# from Floyd's sampling algorithm (Bentley and Floyd, "A sample of
# brilliance", CACM 1987).

_M64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15


def splitmix64_mix(z: int) -> int:
    """The SplitMix64 output function of a 64-bit state."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def random_draw(seed: int, counter: int, i: int) -> int:
    """Draw i (1, 2, ...) of stream (seed, counter): SplitMix64 started from
    state seed + counter * 2^32 * gamma, i.e. mix(seed + (counter * 2^32 + i) * gamma)."""
    return splitmix64_mix((seed + ((counter << 32) + i) * SPLITMIX_GAMMA) & _M64)


def floyd_sample(n: int, k: int, draw) -> List[int]:
    """Floyd's algorithm: k distinct values of range(n), each k-subset equally
    likely when draw(r, j) is uniform on 0..j. Step r (r = 0..k-1) takes
    j = n - k + r and t = draw(r, j); it keeps t unless t was already kept,
    in which case it keeps j. Returned in ascending order."""
    kept = set()
    for r in range(k):
        j = n - k + r
        t = draw(r, j)
        kept.add(j if t in kept else t)
    return sorted(kept)


def select_random(n_blocks: int, k: int, seed: int, counter: int) -> List[int]:
    """k distinct pool blocks chosen at random (the random-selection baseline);
    step r maps draw r+1 to 0..j by the top 32 bits times (j+1), over 2^32."""
    return floyd_sample(n_blocks, k, lambda r, j: ((random_draw(seed, counter, r + 1) >> 32) * (j + 1)) >> 32)


def select_fifo(n_blocks: int, k: int) -> List[int]:
    """The FIFO baseline: the k most recent pool blocks."""
    return list(range(n_blocks - k, n_blocks))


# ---------------------------------------------------------------------------
# Placement of the selected blocks  [arXiv] "The Position Misalignment Problem",
# "Incremental RoPE adjustment"; [summary] "Method" (remaining tokens shifted to
# continuous indices)
# ---------------------------------------------------------------------------

def initial_pos_tags(n_blocks: int, sink_blocks: int, block_frames: int) -> np.ndarray:
    """Pool block m first holds frames starting at (sink_blocks + m) * B_f."""
    return ((sink_blocks + np.arange(n_blocks)) * block_frames).astype(np.int64)


def placement_deltas(ids: Sequence[int], pos_tags: np.ndarray, recent_first_frame: int,
                     block_frames: int) -> Tuple[np.ndarray, np.ndarray]:
    """Lay the selected blocks end to end just before the recent block.

    Block r of k (ascending) gets target T_r = F_recent - (k - r) * B_f and
    delta_r = T_r - P[id_r]; its tag becomes T_r. Returns (deltas, new tags).
    """
    k = len(ids)
    tags = np.array(pos_tags, dtype=np.int64, copy=True)
    deltas = np.zeros(k, dtype=np.int64)
    for r, b in enumerate(ids):
        target = recent_first_frame - (k - r) * block_frames
        deltas[r] = target - tags[b]
        tags[b] = target
    return deltas, tags


def rollin(pool_k: np.ndarray, pool_v: np.ndarray, pos_tags: np.ndarray, block_k: np.ndarray,
           block_v: np.ndarray, first_frame: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Append one compressed block to the mid pool.

    [arXiv] "Dual-Resolution Shifting Mechanism": a block that leaves the recent
    window enters the mid buffer as its compressed backup. Its keys still carry
    the positions they were encoded at, so its tag is the first frame the block
    held as the recent block. Returns (pool_k, pool_v, pos_tags), all new arrays.
    """
    return (np.concatenate([pool_k, block_k], axis=0), np.concatenate([pool_v, block_v], axis=0),
            np.append(np.asarray(pos_tags, dtype=np.int64), np.int64(first_frame)))


def evict_and_shift_sink(sink_k: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray, pos_tags: np.ndarray,
                         n_evict: int, n_c: int, block_frames: int,
                         base: float = ROPE_BASE) -> Dict[str, np.ndarray]:
    """Evict the n_evict oldest pool blocks and move the sink after them.

    [arXiv] "The Position Misalignment Problem": keeping the mid pool within its
    budget evicts its oldest compressed blocks, which opens a gap of
    delta = n_evict * B_f frames between the sink and the first surviving mid
    block. "Incremental RoPE adjustment": the sink keys are rotated forward by
    delta on the temporal axis only, so they again sit directly before the mid
    keys. Pool blocks are in arrival order (block 0 is the oldest). Returns the
    shifted sink (bf16 bits), the surviving pool K/V and tags, and delta.
    """
    delta = int(n_evict) * int(block_frames)
    rows = sink_k.shape[0]
    shifted = rope_shift_blocks(sink_k, rows, [0], [delta], base)
    cut = int(n_evict) * int(n_c)
    return {"sink_k": shifted, "pool_k": pool_k[cut:], "pool_v": pool_v[cut:],
            "tags": np.asarray(pos_tags, dtype=np.int64)[int(n_evict):], "delta": delta}


# ---------------------------------------------------------------------------
# Attention  [digest] 前置知识 KV缓存 (softmax(Q K^T / sqrt(d_h)) V), 方法步骤详情 (5);
# [arXiv] "Bounded Attention Context" (C = C_sink || C_mid || C_rc)
# ---------------------------------------------------------------------------

def gather_mid(pool_bits: np.ndarray, n_c: int, ids: Sequence[int]) -> np.ndarray:
    """Rows of the selected pool blocks, in the order of ids."""
    if len(ids) == 0:
        return pool_bits[:0]
    return np.concatenate([pool_bits[int(b) * n_c:(int(b) + 1) * n_c] for b in ids], axis=0)


def attn_bruteforce(q_bits: np.ndarray, k_parts: Sequence[np.ndarray], v_parts: Sequence[np.ndarray],
                    scale: float = 1.0 / math.sqrt(HEAD_DIM)) -> Tuple[np.ndarray, np.ndarray]:
    """Concatenate the partitions, then one softmax(Q K^T * scale) V per head.

    Returns O [n_q, H, D] and the natural-log LSE [H, n_q], in float64.
    """
    k_all = np.concatenate(k_parts, axis=0)
    v_all = np.concatenate(v_parts, axis=0)
    n_q, H, _ = q_bits.shape
    o = np.empty((n_q, H, HEAD_DIM))
    lse = np.empty((H, n_q))
    for h in range(H):
        q = bf16_to_f64(q_bits[:, h, :])
        k = bf16_to_f64(k_all[:, h, :])
        v = bf16_to_f64(v_all[:, h, :])
        s = (q @ k.T) * scale                              # [n_q, n_k]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[:, h, :] = (e / z) @ v
        lse[h] = (m + np.log(z))[:, 0]
    return o, lse


def attn_partitioned(q_bits: np.ndarray, k_parts: Sequence[np.ndarray], v_parts: Sequence[np.ndarray],
                     scale: float = 1.0 / math.sqrt(HEAD_DIM)) -> Tuple[np.ndarray, np.ndarray]:
    """Same softmax, assembled from per-partition statistics.

    For each partition p: m_p = max score, l_p = sum exp(s - m_p),
    U_p = sum exp(s - m_p) v. Then m = max_p m_p, l = sum_p e^{m_p - m} l_p and
    O = sum_p e^{m_p - m} U_p / l. Empty partitions are skipped.
    """
    n_q, H, D = q_bits.shape
    o = np.empty((n_q, H, D))
    lse = np.empty((H, n_q))
    parts = [(kp, vp) for kp, vp in zip(k_parts, v_parts) if kp.shape[0] > 0]
    for h in range(H):
        q = bf16_to_f64(q_bits[:, h, :])
        stats = []
        for kp, vp in parts:
            s = (q @ bf16_to_f64(kp[:, h, :]).T) * scale
            m_p = s.max(axis=1)
            e = np.exp(s - m_p[:, None])
            stats.append((m_p, e.sum(axis=1), e @ bf16_to_f64(vp[:, h, :])))
        m = np.max(np.stack([st[0] for st in stats]), axis=0)
        l = np.zeros(n_q)
        u = np.zeros((n_q, D))
        for m_p, l_p, u_p in stats:
            w = np.exp(m_p - m)
            l += w * l_p
            u += w[:, None] * u_p
        o[:, h, :] = u / l[:, None]
        lse[h] = m + np.log(l)
    return o, lse


def partitions(cache: Dict[str, np.ndarray], n_c: int, ids: Sequence[int]):
    """(K parts, V parts) of the bounded context in concatenation order."""
    ks = [cache["sink_k"], gather_mid(cache["pool_k"], n_c, ids), cache["recent_k"], cache["cur_k"]]
    vs = [cache["sink_v"], gather_mid(cache["pool_v"], n_c, ids), cache["recent_v"], cache["cur_v"]]
    return ks, vs


# ---------------------------------------------------------------------------
# One layer-step of the path: select -> place -> shift -> attend
# ---------------------------------------------------------------------------

def layer_step(cache: Dict[str, np.ndarray], pos_tags: np.ndarray, n_c: int, top_k: int,
               recent_first_frame: int, block_frames: int, q_rows=None,
               base: float = ROPE_BASE) -> Dict[str, object]:
    """Run the whole path on one layer; returns ids, deltas, new tags, shifted
    pool keys and the attention output (for all queries, or the rows given)."""
    scores = block_scores(cache["q"], cache["pool_k"], n_c)
    ids = select_topk(scores, top_k)
    deltas, tags = placement_deltas(ids, pos_tags, recent_first_frame, block_frames)
    pool_k = rope_shift_blocks(cache["pool_k"], n_c, ids, deltas, base)
    shifted = dict(cache, pool_k=pool_k)
    ks, vs = partitions(shifted, n_c, ids)
    q = cache["q"] if q_rows is None else cache["q"][q_rows]
    o, lse = attn_partitioned(q, ks, vs)
    return {"scores": scores, "ids": ids, "gap": topk_gap(scores, top_k), "deltas": deltas,
            "tags": tags, "pool_k": pool_k, "o": o, "lse": lse}


# ---------------------------------------------------------------------------
# HR branch of the compressor  [arXiv] "HR Branch: Progressive 3D Convolution"
# and "Feature Fusion" (N_c = floor(T/2) floor(H/8) floor(W/8)); [digest]
# 前置知识 3D卷积 and 方法步骤详情 (2)
# ---------------------------------------------------------------------------
#
# Readings where the pages are silent:
#  * each strided convolution has its kernel equal to its stride and no
#    padding, so every output position sees one disjoint input patch and every
#    dimension is floored, which is exactly what the N_c formula counts;
#  * SiLU follows each strided convolution; the final 1x1x1 projection to the
#    hidden width is linear;
#  * activations are stored channels-last, [B][T][H][W][C], as bfloat16 after
#    every stage (round-to-nearest-even of the exact value), the way a bf16
#    network keeps them; weights are [C_out][kt][kh][kw][C_in] bfloat16 and
#    biases float32;
#  * the compressed tokens are numbered t-major: token (t, h, w) is row
#    (t*H_out + h)*W_out + w.

HR_STAGE_KERNELS = ((2, 1, 1), (1, 2, 2), (1, 2, 2), (1, 2, 2))


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x), written so that neither branch overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, x / (1.0 + e), x * e / (1.0 + e))


def hr_conv_stage(x_bits: np.ndarray, w_bits: np.ndarray, bias, kernel, act: bool = True,
                  round_output: bool = True) -> np.ndarray:
    """One strided 3D convolution (kernel = stride, no padding) plus bias and,
    when act, SiLU. x_bits [B][T][H][W][C_in] and w_bits
    [C_out][kt][kh][kw][C_in] are bfloat16 bits; bias is [C_out] (or None).
    The output is [B][T//kt][H//kh][W//kw][C_out]: bfloat16 bits, or the exact
    float64 values when round_output is False."""
    x = bf16_to_f64(x_bits)
    kt, kh, kw = kernel
    B, T, H, W, C = x.shape
    w = bf16_to_f64(w_bits)
    c_out = w.shape[0]
    assert w.shape == (c_out, kt, kh, kw, C), (w.shape, kernel, C)
    To, Ho, Wo = T // kt, H // kh, W // kw
    x = x[:, :To * kt, :Ho * kh, :Wo * kw, :]
    # each output position's patch, flattened in (dt, dh, dw, c) order
    patches = x.reshape(B, To, kt, Ho, kh, Wo, kw, C).transpose(0, 1, 3, 5, 2, 4, 6, 7)
    patches = patches.reshape(B * To * Ho * Wo, kt * kh * kw * C)
    y = patches @ w.reshape(c_out, -1).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    if act:
        y = silu(y)
    y = y.reshape(B, To, Ho, Wo, c_out)
    return f64_to_bf16(y) if round_output else y


def hr_branch(z_bits: np.ndarray, stages, proj) -> np.ndarray:
    """The HR branch: the strided stages of HR_STAGE_KERNELS, each followed by
    SiLU, then the linear 1x1x1 projection. z_bits is the latent block
    [B][T][H][W][C] (bfloat16 bits); stages is a list of (w_bits, bias), one per
    kernel; proj is (w_bits [d][C_last], bias). Returns [B][N_c][d] bfloat16
    bits with N_c = (T//2) (H//8) (W//8) tokens numbered t-major."""
    x = z_bits
    for (w, b), k in zip(stages, HR_STAGE_KERNELS):
        x = hr_conv_stage(x, w, b, k, act=True)
    wp, bp = proj
    d = wp.shape[0]
    y = hr_conv_stage(x, wp.reshape(d, 1, 1, 1, -1), bp, (1, 1, 1), act=False)
    B, To, Ho, Wo, _ = y.shape
    return y.reshape(B, To * Ho * Wo, d)
