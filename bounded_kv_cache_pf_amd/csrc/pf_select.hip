// Dynamic context selection and placement.
//
// Scoring [PackForcing digest (paper.rainbus.top), 方法步骤详情 (3); arXiv HTML,
// "Compressed Mid Tokens"]: query-key affinity of every compressed mid block,
// then the top-k blocks. With pooled queries and pooled block keys,
//   s_j = (1/H) sum_h < mean_i q_{i,h}, mean_{t in j} k_{t,h} > / sqrt(128).
// Placement [arXiv HTML, "The Position Misalignment Problem", "Incremental RoPE
// adjustment"; openbayes summary, "Method"]: the selected blocks are laid end to
// end before the recent block and each one's temporal shift is returned.
//
// The scoring reads Q and the whole pool once (HBM-bound), in three or four
// launches on one stream; every launch covers a batch of independent caches
// (grid y):
//   1. colsum: every workgroup sums a segment of rows (a 64-row slice of Q, or a
//      slice of one pool block) column by column into fp32 partials;
//   2. qsum:   the Q partials are added per column, 16 interleaved runs of
//              segments combined in a fixed order;
//   3. score:  one workgroup per block adds its slices and dots with the Q sum;
//   4. topk:   one workgroup per cache ranks (score desc, index asc) the keys
//              in LDS, writes the first k ids in ascending order and, for the
//              fused select-and-place call, places them. A small call (one
//              layer) runs this in the last score workgroup of each cache
//              instead of a fourth launch.
// Every sum runs in a fixed order that does not depend on the batch, so
// identical blocks get identical scores, repeated calls give identical bits,
// and a batched call gives the bits of the single calls.
#include <math.h>

#include "pf_internal.h"

namespace {
typedef unsigned int u4v __attribute__((ext_vector_type(4)));   // for the streaming (non-temporal) loads

// Segments of the column sums, the same for every batch size, so a batched call
// adds in the order of the single calls. Q rows per colsum workgroup, and the
// pool slices aimed at per cache (at least one per block): one layer's call
// (6,240 queries, 40 blocks) gets 98 Q and 120 pool workgroups, about one per
// CU; a 116-block pool gets one slice per block, a third of the partial sums
// that the score kernel reads back before. Timed on one device against 32 /
// 256 and other pairs: 2.5 us faster for one layer, 11% faster for 30 caches
// batched.
constexpr int kQSegRows = 64;
constexpr int kTargetSegments = 96;
constexpr int kRowUnroll = 4;      // rows whose loads a colsum thread keeps in flight
constexpr int kQsumCols = 64;      // columns per qsum workgroup
constexpr int kQsumRuns = 16;      // interleaved runs of Q segments per column
constexpr int kFusedTopkMaxWorkgroups = 512;   // score launches up to this size also run the top-k

struct SelectPlan {
  int H, cw;          // heads, 16-byte column chunks per row (H*16)
  int rpar;           // row-parallel thread groups per colsum workgroup
  int64_t n_q;
  int nq_seg;         // Q segments
  int n_blocks, n_c;
  int ksub;           // slices per pool block
  int sub_rows;       // rows per slice (last slice may be shorter)
  int n_seg;          // segments per cache
  size_t cache_partials, cache_floats;   // floats per cache: partials, qsum, scores, a counter
  size_t bytes;
};

// q_step / head_step: score with query rows 0, q_step, 2 q_step, ... and heads
// 0, head_step, 2 head_step, ... only (1, 1: every query and head).
SelectPlan make_plan(int64_t n_q, int H, int n_blocks, int n_c, int n_batch, int q_step = 1, int head_step = 1) {
  SelectPlan p{};
  H = (H + head_step - 1) / head_step;           // heads that are scored
  n_q = (n_q + q_step - 1) / q_step;             // query rows that are scored
  p.H = H;
  p.cw = H * 16;
  p.rpar = 1024 / p.cw;
  if (p.rpar > 16) p.rpar = 16;
  if (p.rpar < 1) p.rpar = 1;
  p.n_q = n_q;
  p.nq_seg = static_cast<int>((n_q + kQSegRows - 1) / kQSegRows);
  p.n_blocks = n_blocks;
  p.n_c = n_c;
  int ksub = (kTargetSegments + n_blocks - 1) / n_blocks;
  if (ksub > n_c) ksub = n_c;
  if (ksub < 1) ksub = 1;
  p.sub_rows = (n_c + ksub - 1) / ksub;
  p.ksub = (n_c + p.sub_rows - 1) / p.sub_rows;
  p.n_seg = p.nq_seg + n_blocks * p.ksub;
  const size_t cols = static_cast<size_t>(H) * PF_HEAD_DIM;
  p.cache_partials = static_cast<size_t>(p.n_seg) * cols;
  p.cache_floats = p.cache_partials + cols + static_cast<size_t>(n_blocks) + 1;
  p.cache_floats = (p.cache_floats + 63) & ~static_cast<size_t>(63);   // 256-byte aligned per cache
  p.bytes = p.cache_floats * sizeof(float) * static_cast<size_t>(n_batch);
  return p;
}

// 1. Column sums of row segments. blockDim = (cw, rpar); thread (x, y) owns the
// 8 columns of chunk x and rows y, y+rpar, ... of its segment, added in row
// order (loads run kRowUnroll rows ahead). blockIdx.y is the cache. The scan
// reads every byte once, so its loads are marked non-temporal (streamed past
// the caches); that raises the achieved read bandwidth by about a tenth.
__global__ __launch_bounds__(1024) void colsum_kernel(const uint16_t* __restrict__ q, int64_t q_bstride,
                                                      const uint16_t* __restrict__ pool, int64_t pool_bstride,
                                                      float* __restrict__ ws, int64_t cache_floats, int64_t n_q,
                                                      int nq_seg, int n_c, int ksub, int sub_rows,
                                                      int64_t row_elems, int q_step, int head_step,
                                                      int64_t counter_off) {
  extern __shared__ float red[];   // [rpar][cw*8]
  const int cw = blockDim.x, rpar = blockDim.y;
  const int x = threadIdx.x, y = threadIdx.y;
  const int seg = blockIdx.x;
  const int64_t b = blockIdx.y;
  // the score launch counts its finished workgroups here (one counter per cache)
  if (seg == 0 && x == 0 && y == 0) reinterpret_cast<uint32_t*>(ws + b * cache_floats + counter_off)[0] = 0u;
  const uint16_t* base;
  int64_t rows, stride;   // rows of this segment, elements between them
  if (seg < nq_seg) {
    const int64_t r0 = static_cast<int64_t>(seg) * kQSegRows;   // in scored (sub-sampled) rows
    rows = n_q - r0 < kQSegRows ? n_q - r0 : kQSegRows;
    stride = row_elems * q_step;
    base = q + b * q_bstride + r0 * stride;
  } else {
    const int s = seg - nq_seg;
    const int blk = s / ksub, sub = s % ksub;
    const int r_in = sub * sub_rows;
    rows = n_c - r_in < sub_rows ? n_c - r_in : sub_rows;
    stride = row_elems;
    base = pool + b * pool_bstride + (static_cast<int64_t>(blk) * n_c + r_in) * row_elems;
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // column chunk x: 8 dims of scored head x/16 (head (x/16) * head_step of the row)
  const uint16_t* p = base + (x >> 4) * head_step * PF_HEAD_DIM + (x & 15) * 8;
  int64_t r = y;
  for (; r + (kRowUnroll - 1) * rpar < rows; r += kRowUnroll * rpar) {
    uint4 w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p + (r + u * rpar) * stride));
      w[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += pf::bf16_to_f32(static_cast<uint16_t>(ww[i] & 0xFFFFu));
        acc[2 * i + 1] += pf::bf16_to_f32(static_cast<uint16_t>(ww[i] >> 16));
      }
    }
  }
  for (; r < rows; r += rpar) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + r * stride);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += pf::bf16_to_f32(static_cast<uint16_t>(ww[i] & 0xFFFFu));
      acc[2 * i + 1] += pf::bf16_to_f32(static_cast<uint16_t>(ww[i] >> 16));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[(y * cw + x) * 8 + i] = acc[i];
  __syncthreads();
  if (y == 0) {
    for (int yy = 1; yy < rpar; ++yy)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += red[(yy * cw + x) * 8 + i];
    float* out = ws + b * cache_floats + static_cast<int64_t>(seg) * cw * 8 + x * 8;
    reinterpret_cast<float4*>(out)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(out)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// 2. Q sum. Thread (c, g) adds segments g, g+16, g+32, ... of column c in
// order; the 16 runs are then added in order g = 0..15.
__global__ __launch_bounds__(kQsumCols * kQsumRuns) void qsum_kernel(float* __restrict__ ws, int64_t cache_floats,
                                                                     int64_t qsum_off, int nq_seg, int cols) {
  __shared__ float red[kQsumRuns][kQsumCols];
  const int tc = threadIdx.x % kQsumCols;
  const int g = threadIdx.x / kQsumCols;
  const int c = blockIdx.x * kQsumCols + tc;
  float* cache = ws + static_cast<int64_t>(blockIdx.y) * cache_floats;
  float s = 0.f;
  if (c < cols) {
    // eight segments per pass, all loaded before the first add (a segment past
    // the last reads segment g and adds 0), so a pass costs one memory latency
    constexpr int kPass = 8;
    for (int i = g; i < nq_seg; i += kPass * kQsumRuns) {
      float v[kPass];
#pragma unroll
      for (int u = 0; u < kPass; ++u) {
        const int seg = i + u * kQsumRuns;
        v[u] = cache[static_cast<int64_t>(seg < nq_seg ? seg : g) * cols + c];
      }
#pragma unroll
      for (int u = 0; u < kPass; ++u) s += i + u * kQsumRuns < nq_seg ? v[u] : 0.f;
    }
  }
  red[g][tc] = s;
  __syncthreads();
  if (g == 0 && c < cols) {
    float t = red[0][tc];
#pragma unroll
    for (int j = 1; j < kQsumRuns; ++j) t += red[j][tc];
    cache[qsum_off + c] = t;
  }
}

// Ascending order of the key == descending score, then ascending index.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t idx) {
  if (s == 0.f) s = 0.f;   // -0 and +0 tie
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending float order
  return (static_cast<uint64_t>(~u) << 32) | idx;
}

// Placement of the r-th of k selected blocks (ascending ids): it goes to the
// r-th of k block slots that end right before the recent block; its shift is
// that slot's first frame minus the frame its keys encode now (the tag).
__device__ __forceinline__ void place_one(int32_t id, int r, int top_k, int32_t* tags, int n_blocks,
                                          int32_t recent_first_frame, int32_t block_frames, int32_t* delta) {
  if (id < 0 || id >= n_blocks) {
    *delta = 0;
    return;
  }
  const int32_t target = recent_first_frame - (top_k - r) * block_frames;
  *delta = target - tags[id];
  tags[id] = target;
}

// Top-k of one cache's scores by one workgroup: the k smallest rank keys. Up
// to one key per thread, a key's rank is the count of smaller keys (all keys
// differ, the index breaks ties); more blocks than threads are sorted
// (bitonic, in LDS).

// chosen[r] = index of the key of rank r, r < top_k
__device__ __forceinline__ void topk_by_rank(const float* scores, int n_blocks, int top_k, uint64_t* keys,
                                             uint32_t* chosen) {
  const int tid = static_cast<int>(threadIdx.x);
  uint64_t mine = ~0ull;
  if (tid < n_blocks) {
    mine = rank_key(scores[tid], static_cast<uint32_t>(tid));
    keys[tid] = mine;
  }
  __syncthreads();
  if (tid < n_blocks) {
    int rank = 0;
    for (int j = 0; j < n_blocks; ++j) rank += keys[j] < mine;
    if (rank < top_k) chosen[rank] = static_cast<uint32_t>(tid);
  }
}

__device__ __forceinline__ void topk_by_sort(const float* scores, int n_blocks, int top_k, uint64_t* keys,
                                             uint32_t* chosen) {
  int P = 1;
  while (P < n_blocks) P <<= 1;
  for (int i = threadIdx.x; i < P; i += blockDim.x)
    keys[i] = i < n_blocks ? rank_key(scores[i], static_cast<uint32_t>(i)) : ~0ull;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x0 = keys[i], x1 = keys[ixj];
          const bool up = (i & k) == 0;
          if ((x0 > x1) == up) {
            keys[i] = x1;
            keys[ixj] = x0;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < top_k; r += blockDim.x) chosen[r] = static_cast<uint32_t>(keys[r] & 0xFFFFFFFFu);
}


// The k smallest rank keys of one cache's scores (by the calling workgroup),
// written as ids in ascending order; with tags != nullptr those blocks are also
// placed. keys, chosen and sorted_ids are the workgroup's LDS arrays.
__device__ __forceinline__ void topk_write_place(const float* scores, int64_t b, int n_blocks, int top_k,
                                                 int32_t* ids_out, int32_t* tags, int32_t recent_first_frame,
                                                 int32_t block_frames, int32_t* deltas, uint64_t* keys,
                                                 uint32_t* chosen, int32_t* sorted_ids) {
  if (n_blocks <= static_cast<int>(blockDim.x))
    topk_by_rank(scores, n_blocks, top_k, keys, chosen);
  else
    topk_by_sort(scores, n_blocks, top_k, keys, chosen);
  __syncthreads();
  // ascending ids: each chosen id's position is the count of smaller chosen ids
  int32_t* ids = ids_out + b * top_k;
  for (int i = threadIdx.x; i < top_k; i += blockDim.x) {
    const uint32_t me = chosen[i];
    int rank = 0;
    for (int r = 0; r < top_k; ++r) rank += chosen[r] < me;
    ids[rank] = static_cast<int32_t>(me);
    sorted_ids[rank] = static_cast<int32_t>(me);
  }
  if (tags == nullptr) return;
  __syncthreads();
  for (int i = threadIdx.x; i < top_k; i += blockDim.x)
    place_one(sorted_ids[i], i, top_k, tags + b * n_blocks, n_blocks, recent_first_frame, block_frames,
              deltas + b * top_k + i);
}

// 3. Block score: one workgroup per pool block and cache, one thread per four
// columns (cols / 4 threads, rounded up to whole waves). A thread adds its
// columns' slices in slice order (every load issued before the first add),
// dots them with the Q sum in column order, and the threads' products are
// added by a fixed tree: within each wave by lane-distance halving, then the
// waves in order.
// kFused: the last workgroup of a cache to finish (a counter that the
// column-sum launch cleared) also runs that cache's top-k and placement. Each
// workgroup then publishes its score with a device-scope release, which
// writes back its L2: cheap for a few dozen workgroups (one layer's call),
// costly for thousands (a batched call), which launch topk_kernel instead.
template <bool kFused>
__global__ __launch_bounds__(1024) void score_kernel(float* __restrict__ ws, int64_t cache_floats, int64_t qsum_off,
                                                     int64_t scores_off, int64_t counter_off,
                                                     float* __restrict__ scores_out, int n_blocks, int nq_seg,
                                                     int ksub, int cols, float norm, int top_k,
                                                     int32_t* __restrict__ ids_out, int32_t* __restrict__ tags,
                                                     int32_t recent_first_frame, int32_t block_frames,
                                                     int32_t* __restrict__ deltas) {
  __shared__ float red[16];
  __shared__ uint64_t keys[kFused ? PF_MAX_BLOCKS : 1];
  __shared__ uint32_t chosen[kFused ? PF_MAX_TOPK : 1];
  __shared__ int32_t sorted_ids[kFused ? PF_MAX_TOPK : 1];
  __shared__ int is_last;
  const int blk = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.y;
  float* cache = ws + b * cache_floats;
  const float4* kp =
      reinterpret_cast<const float4*>(cache + (static_cast<int64_t>(nq_seg) + static_cast<int64_t>(blk) * ksub) * cols) + t;
  const int c4 = cols >> 2;
  float dot = 0.f;
  if (t < c4) {
    float4 ks = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    for (; s + 7 < ksub; s += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = kp[static_cast<int64_t>(s + u) * c4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ks.x += v[u].x; ks.y += v[u].y; ks.z += v[u].z; ks.w += v[u].w;
      }
    }
    for (; s < ksub; ++s) {
      const float4 v = kp[static_cast<int64_t>(s) * c4];
      ks.x += v.x; ks.y += v.y; ks.z += v.z; ks.w += v.w;
    }
    const float4 qv = reinterpret_cast<const float4*>(cache + qsum_off)[t];
    dot = qv.x * ks.x;
    dot += qv.y * ks.y;
    dot += qv.z * ks.z;
    dot += qv.w * ks.w;
  }
  // every lane of the (whole) waves takes part; lanes past the columns add 0
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) dot += __shfl_xor(dot, d);
  const int n_waves = (blockDim.x + 63) >> 6;
  if ((t & 63) == 0) red[t >> 6] = dot;
  __syncthreads();
  if (t == 0) {
    float total = red[0];
    for (int w = 1; w < n_waves; ++w) total += red[w];
    const float sc = total * norm;
    cache[scores_off + blk] = sc;
    if (scores_out) scores_out[b * n_blocks + blk] = sc;
    if constexpr (kFused) {
      // release the score, then count this workgroup
      __threadfence();
      const uint32_t done = atomicAdd(reinterpret_cast<uint32_t*>(cache + counter_off), 1u);
      is_last = done == static_cast<uint32_t>(n_blocks - 1);
    }
  }
  if constexpr (kFused) {
    __syncthreads();
    if (!is_last) return;
    __threadfence();   // acquire: every workgroup's score is visible from here
    topk_write_place(cache + scores_off, b, n_blocks, top_k, ids_out, tags, recent_first_frame, block_frames,
                     deltas, keys, chosen, sorted_ids);
  }
}

// 4. Top-k (batched calls): one workgroup per cache.
constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ ws, int64_t cache_floats,
                                                             int64_t scores_off, int n_blocks, int top_k,
                                                             int32_t* __restrict__ ids_out,
                                                             int32_t* __restrict__ tags, int32_t recent_first_frame,
                                                             int32_t block_frames, int32_t* __restrict__ deltas) {
  __shared__ uint64_t keys[PF_MAX_BLOCKS];
  __shared__ uint32_t chosen[PF_MAX_TOPK];
  __shared__ int32_t sorted_ids[PF_MAX_TOPK];
  const int64_t b = blockIdx.x;
  topk_write_place(ws + b * cache_floats + scores_off, b, n_blocks, top_k, ids_out, tags, recent_first_frame,
                   block_frames, deltas, keys, chosen, sorted_ids);
}

// Placement, one workgroup per cache.
__global__ __launch_bounds__(PF_MAX_TOPK) void deltas_kernel(const int32_t* __restrict__ ids, int top_k,
                                                             int32_t* __restrict__ tags, int n_blocks,
                                                             int32_t recent_first_frame, int32_t block_frames,
                                                             int32_t* __restrict__ deltas) {
  const int r = threadIdx.x;
  if (r >= top_k) return;
  const int64_t b = blockIdx.x;
  place_one(ids[b * top_k + r], r, top_k, tags + b * n_blocks, n_blocks, recent_first_frame, block_frames,
            deltas + b * top_k + r);
}

// Random-selection baseline [digest, 实验结果; arXiv HTML, "FIFO vs. Dynamic
// Context Selection"]: k distinct blocks by Floyd's sampling algorithm
// (Bentley and Floyd, CACM 1987) over a counter-based SplitMix64 stream
// (Steele, Lea and Flood, OOPSLA 2014). Draw i (1, 2, ...) of stream
// (seed, counter) is mix(seed + (counter * 2^32 + i) * gamma).
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One workgroup per cache b (stream counter + b). Thread 0 runs Floyd's steps
// with a membership bitmap in LDS; then thread r writes kept value r at its
// rank, so the ids come out ascending.
__global__ __launch_bounds__(PF_MAX_TOPK) void random_select_kernel(int n_blocks, int top_k, uint64_t seed,
                                                                     uint64_t counter, int32_t* __restrict__ ids_out) {
  __shared__ uint32_t member[PF_MAX_BLOCKS / 32];
  __shared__ int32_t kept[PF_MAX_TOPK];
  const int tid = static_cast<int>(threadIdx.x);
  const uint64_t c = counter + blockIdx.x;
  for (int i = tid; i < PF_MAX_BLOCKS / 32; i += blockDim.x) member[i] = 0u;
  __syncthreads();
  if (tid == 0) {
    for (int r = 0; r < top_k; ++r) {
      const uint32_t j = static_cast<uint32_t>(n_blocks - top_k + r);
      const uint64_t x = splitmix_mix(seed + ((c << 32) + static_cast<uint64_t>(r + 1)) * kGamma);
      const uint32_t t = static_cast<uint32_t>(((x >> 32) * (static_cast<uint64_t>(j) + 1)) >> 32);
      const bool seen = (member[t >> 5] >> (t & 31)) & 1u;
      const uint32_t v = seen ? j : t;
      member[v >> 5] |= 1u << (v & 31);
      kept[r] = static_cast<int32_t>(v);
    }
  }
  __syncthreads();
  if (tid < top_k) {
    const int32_t me = kept[tid];
    int rank = 0;
    for (int r = 0; r < top_k; ++r) rank += kept[r] < me;
    ids_out[static_cast<int64_t>(blockIdx.x) * top_k + rank] = me;
  }
}

bool valid_sizes(int64_t n_q, int n_heads, int n_blocks, int n_c, int n_batch) {
  return n_q >= 1 && n_heads >= 1 && n_heads <= PF_MAX_HEADS && n_blocks >= 1 && n_blocks <= PF_MAX_BLOCKS &&
         n_c >= 1 && n_batch >= 1 && n_batch <= PF_MAX_BATCH;
}

}  // namespace

extern "C" size_t pf_score_select_batched_workspace_bytes(int64_t n_q, int n_heads, int n_blocks, int n_c,
                                                          int n_batch) {
  if (!valid_sizes(n_q, n_heads, n_blocks, n_c, n_batch)) return 0;
  return make_plan(n_q, n_heads, n_blocks, n_c, n_batch).bytes;
}

extern "C" size_t pf_score_select_workspace_bytes(int64_t n_q, int n_heads, int n_blocks, int n_c) {
  return pf_score_select_batched_workspace_bytes(n_q, n_heads, n_blocks, n_c, 1);
}

namespace {

// tags == nullptr: selection only; otherwise the selected blocks are also
// placed (tags updated, deltas written) by the workgroup that selects them.
pf_status score_select(const pf_bf16* q, int64_t q_batch_stride, int64_t n_q, int n_heads, int q_step,
                       int head_step, const pf_bf16* pool_k, int64_t pool_batch_stride, int n_blocks, int n_c,
                       int top_k, int n_batch, int32_t* ids_out, float* scores_out, void* workspace,
                       size_t workspace_bytes, void* stream, int32_t* tags = nullptr,
                       int32_t recent_first_frame = 0, int32_t block_frames = 1, int32_t* deltas_out = nullptr) {
  PF_REQUIRE_PTR(q);
  PF_REQUIRE_PTR(pool_k);
  PF_REQUIRE_PTR(ids_out);
  PF_REQUIRE(n_q >= 1, PF_ERR_SHAPE, "n_q must be >= 1");
  PF_REQUIRE(n_c >= 1, PF_ERR_SHAPE, "n_c must be >= 1");
  PF_REQUIRE(n_heads >= 1 && n_heads <= PF_MAX_HEADS, PF_ERR_UNSUPPORTED,
             "n_heads must be in [1, %d] (got %d)", PF_MAX_HEADS, n_heads);
  PF_REQUIRE(n_blocks >= 1 && n_blocks <= PF_MAX_BLOCKS, PF_ERR_UNSUPPORTED,
             "n_blocks must be in [1, %d] (got %d)", PF_MAX_BLOCKS, n_blocks);
  PF_REQUIRE(top_k >= 1 && top_k <= n_blocks && top_k <= PF_MAX_TOPK, PF_ERR_RANGE,
             "top_k must be in [1, min(n_blocks, %d)] (got %d)", PF_MAX_TOPK, top_k);
  PF_REQUIRE(n_batch >= 1 && n_batch <= PF_MAX_BATCH, PF_ERR_RANGE, "n_batch must be in [1, %d] (got %d)",
             PF_MAX_BATCH, n_batch);
  PF_REQUIRE(n_q <= (int64_t{1} << 40), PF_ERR_UNSUPPORTED, "n_q too large");
  const int64_t row = static_cast<int64_t>(n_heads) * PF_HEAD_DIM;
  if (n_batch > 1) {
    PF_REQUIRE(q_batch_stride >= n_q * row, PF_ERR_SHAPE, "q_batch_stride (%lld) is smaller than one cache's Q",
               static_cast<long long>(q_batch_stride));
    PF_REQUIRE(pool_batch_stride >= static_cast<int64_t>(n_blocks) * n_c * row, PF_ERR_SHAPE,
               "pool_batch_stride (%lld) is smaller than one cache's pool", static_cast<long long>(pool_batch_stride));
    PF_REQUIRE(q_batch_stride % 8 == 0 && pool_batch_stride % 8 == 0, PF_ERR_MISALIGNED,
               "batch strides must be multiples of 8 elements (16 bytes)");
  }
  PF_REQUIRE_ALIGNED(q);
  PF_REQUIRE_ALIGNED(pool_k);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(ids_out) & 3u) == 0, PF_ERR_MISALIGNED, "ids_out is not 4-byte aligned");
  PF_REQUIRE((reinterpret_cast<uintptr_t>(scores_out) & 3u) == 0, PF_ERR_MISALIGNED,
             "scores_out is not 4-byte aligned");
  PF_REQUIRE(q_step >= 1 && head_step >= 1 && head_step <= n_heads, PF_ERR_RANGE,
             "q_step must be >= 1 and head_step in [1, n_heads] (got %d, %d)", q_step, head_step);
  const SelectPlan p = make_plan(n_q, n_heads, n_blocks, n_c, n_batch, q_step, head_step);
  PF_REQUIRE(workspace != nullptr, PF_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", p.bytes);
  PF_REQUIRE(workspace_bytes >= p.bytes, PF_ERR_WORKSPACE, "workspace has %zu bytes, need %zu",
             workspace_bytes, p.bytes);
  PF_REQUIRE_ALIGNED(workspace);
  PF_REQUIRE(static_cast<int64_t>(p.nq_seg) + static_cast<int64_t>(n_blocks) * p.ksub < 0x7FFFFFFF,
             PF_ERR_UNSUPPORTED, "too many segments");

  hipStream_t st = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  const int cols = p.H * PF_HEAD_DIM;   // scored heads only
  const int64_t cf = static_cast<int64_t>(p.cache_floats);
  const int64_t qsum_off = static_cast<int64_t>(p.cache_partials);
  const int64_t scores_off = qsum_off + cols;
  const int64_t counter_off = scores_off + n_blocks;
  const int64_t qs = n_batch > 1 ? q_batch_stride : 0;
  const int64_t ps = n_batch > 1 ? pool_batch_stride : 0;

  const size_t lds = static_cast<size_t>(p.rpar) * p.cw * 8 * sizeof(float);
  hipLaunchKernelGGL(colsum_kernel, dim3(p.n_seg, n_batch), dim3(p.cw, p.rpar), lds, st,
                     reinterpret_cast<const uint16_t*>(q), qs, reinterpret_cast<const uint16_t*>(pool_k), ps, ws,
                     cf, p.n_q, p.nq_seg, n_c, p.ksub, p.sub_rows, static_cast<int64_t>(n_heads) * PF_HEAD_DIM,
                     q_step, head_step, counter_off);
  pf_status s = pf::launch_status("pf_score_select (colsum)");
  if (s != PF_OK) return s;
  hipLaunchKernelGGL(qsum_kernel, dim3((cols + kQsumCols - 1) / kQsumCols, n_batch), dim3(kQsumCols * kQsumRuns), 0,
                     st, ws, cf, qsum_off, p.nq_seg, cols);
  s = pf::launch_status("pf_score_select (qsum)");
  if (s != PF_OK) return s;
  const double norm = 1.0 / (static_cast<double>(p.n_q) * n_c * p.H * sqrt(static_cast<double>(PF_HEAD_DIM)));
  const dim3 score_threads((cols / 4 + 63) / 64 * 64);
  if (static_cast<int64_t>(n_blocks) * n_batch <= kFusedTopkMaxWorkgroups) {
    hipLaunchKernelGGL(score_kernel<true>, dim3(n_blocks, n_batch), score_threads, 0, st, ws, cf, qsum_off,
                       scores_off, counter_off, scores_out, n_blocks, p.nq_seg, p.ksub, cols,
                       static_cast<float>(norm), top_k, ids_out, tags, recent_first_frame, block_frames, deltas_out);
    return pf::launch_status("pf_score_select (score, top-k)");
  }
  hipLaunchKernelGGL(score_kernel<false>, dim3(n_blocks, n_batch), score_threads, 0, st, ws, cf, qsum_off,
                     scores_off, counter_off, scores_out, n_blocks, p.nq_seg, p.ksub, cols, static_cast<float>(norm),
                     top_k, ids_out, tags, recent_first_frame, block_frames, deltas_out);
  s = pf::launch_status("pf_score_select (score)");
  if (s != PF_OK) return s;
  hipLaunchKernelGGL(topk_kernel, dim3(n_batch), dim3(kTopkThreads), 0, st, ws, cf, scores_off, n_blocks, top_k,
                     ids_out, tags, recent_first_frame, block_frames, deltas_out);
  return pf::launch_status("pf_score_select (top-k)");
}

}  // namespace

extern "C" pf_status pf_score_select_batched(const pf_bf16* q, int64_t q_batch_stride, int64_t n_q, int n_heads,
                                             const pf_bf16* pool_k, int64_t pool_batch_stride, int n_blocks,
                                             int n_c, int top_k, int n_batch, int32_t* ids_out,
                                             float* scores_out, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  return score_select(q, q_batch_stride, n_q, n_heads, 1, 1, pool_k, pool_batch_stride, n_blocks, n_c, top_k,
                      n_batch, ids_out, scores_out, workspace, workspace_bytes, stream);
}

extern "C" pf_status pf_score_select(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* pool_k,
                                     int n_blocks, int n_c, int top_k, int32_t* ids_out, float* scores_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return score_select(q, 0, n_q, n_heads, 1, 1, pool_k, 0, n_blocks, n_c, top_k, 1, ids_out, scores_out,
                      workspace, workspace_bytes, stream);
}

extern "C" size_t pf_score_select_sub_workspace_bytes(int64_t n_q, int n_heads, int q_step, int head_step,
                                                      int n_blocks, int n_c) {
  if (!valid_sizes(n_q, n_heads, n_blocks, n_c, 1) || q_step < 1 || head_step < 1 || head_step > n_heads) return 0;
  return make_plan(n_q, n_heads, n_blocks, n_c, 1, q_step, head_step).bytes;
}

extern "C" pf_status pf_score_select_sub(const pf_bf16* q, int64_t n_q, int n_heads, int q_step, int head_step,
                                         const pf_bf16* pool_k, int n_blocks, int n_c, int top_k, int32_t* ids_out,
                                         float* scores_out, void* workspace, size_t workspace_bytes, void* stream) {
  return score_select(q, 0, n_q, n_heads, q_step, head_step, pool_k, 0, n_blocks, n_c, top_k, 1, ids_out,
                      scores_out, workspace, workspace_bytes, stream);
}

extern "C" pf_status pf_select_place_batched(const pf_bf16* q, int64_t q_batch_stride, int64_t n_q, int n_heads,
                                             const pf_bf16* pool_k, int64_t pool_batch_stride, int n_blocks,
                                             int n_c, int top_k, int32_t* pos_tags, int32_t recent_first_frame,
                                             int32_t block_frames, int n_batch, int32_t* ids_out,
                                             int32_t* deltas_out, float* scores_out, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  PF_REQUIRE_PTR(pos_tags);
  PF_REQUIRE_PTR(deltas_out);
  PF_REQUIRE(block_frames >= 1, PF_ERR_RANGE, "block_frames must be >= 1");
  PF_REQUIRE(((reinterpret_cast<uintptr_t>(pos_tags) | reinterpret_cast<uintptr_t>(deltas_out)) & 3u) == 0,
             PF_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
  return score_select(q, q_batch_stride, n_q, n_heads, 1, 1, pool_k, pool_batch_stride, n_blocks, n_c, top_k,
                      n_batch, ids_out, scores_out, workspace, workspace_bytes, stream, pos_tags,
                      recent_first_frame, block_frames, deltas_out);
}

extern "C" pf_status pf_select_place(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* pool_k,
                                     int n_blocks, int n_c, int top_k, int32_t* pos_tags,
                                     int32_t recent_first_frame, int32_t block_frames, int32_t* ids_out,
                                     int32_t* deltas_out, float* scores_out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return pf_select_place_batched(q, 0, n_q, n_heads, pool_k, 0, n_blocks, n_c, top_k, pos_tags, recent_first_frame,
                                 block_frames, 1, ids_out, deltas_out, scores_out, workspace, workspace_bytes,
                                 stream);
}

extern "C" pf_status pf_selection_deltas_batched(const int32_t* ids, int top_k, int32_t* pos_tags, int n_blocks,
                                                 int32_t recent_first_frame, int32_t block_frames, int n_batch,
                                                 int32_t* deltas_out, void* stream) {
  PF_REQUIRE_PTR(ids);
  PF_REQUIRE_PTR(pos_tags);
  PF_REQUIRE_PTR(deltas_out);
  PF_REQUIRE(n_blocks >= 1, PF_ERR_SHAPE, "n_blocks must be >= 1");
  PF_REQUIRE(top_k >= 1 && top_k <= PF_MAX_TOPK && top_k <= n_blocks, PF_ERR_RANGE,
             "top_k must be in [1, min(n_blocks, %d)] (got %d)", PF_MAX_TOPK, top_k);
  PF_REQUIRE(block_frames >= 1, PF_ERR_RANGE, "block_frames must be >= 1");
  PF_REQUIRE(n_batch >= 1 && n_batch <= PF_MAX_BATCH, PF_ERR_RANGE, "n_batch must be in [1, %d] (got %d)",
             PF_MAX_BATCH, n_batch);
  PF_REQUIRE(((reinterpret_cast<uintptr_t>(ids) | reinterpret_cast<uintptr_t>(pos_tags) |
               reinterpret_cast<uintptr_t>(deltas_out)) & 3u) == 0,
             PF_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
  hipLaunchKernelGGL(deltas_kernel, dim3(n_batch), dim3(PF_MAX_TOPK), 0, static_cast<hipStream_t>(stream), ids,
                     top_k, pos_tags, n_blocks, recent_first_frame, block_frames, deltas_out);
  return pf::launch_status("pf_selection_deltas");
}

extern "C" pf_status pf_selection_deltas(const int32_t* ids, int top_k, int32_t* pos_tags, int n_blocks,
                                         int32_t recent_first_frame, int32_t block_frames, int32_t* deltas_out,
                                         void* stream) {
  return pf_selection_deltas_batched(ids, top_k, pos_tags, n_blocks, recent_first_frame, block_frames, 1,
                                     deltas_out, stream);
}

extern "C" pf_status pf_select_random(int n_blocks, int top_k, uint64_t seed, uint64_t counter, int n_batch,
                                      int32_t* ids_out, void* stream) {
  PF_REQUIRE_PTR(ids_out);
  PF_REQUIRE(n_blocks >= 1 && n_blocks <= PF_MAX_BLOCKS, PF_ERR_UNSUPPORTED,
             "n_blocks must be in [1, %d] (got %d)", PF_MAX_BLOCKS, n_blocks);
  PF_REQUIRE(top_k >= 1 && top_k <= n_blocks && top_k <= PF_MAX_TOPK, PF_ERR_RANGE,
             "top_k must be in [1, min(n_blocks, %d)] (got %d)", PF_MAX_TOPK, top_k);
  PF_REQUIRE(n_batch >= 1 && n_batch <= PF_MAX_BATCH, PF_ERR_RANGE, "n_batch must be in [1, %d] (got %d)",
             PF_MAX_BATCH, n_batch);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(ids_out) & 3u) == 0, PF_ERR_MISALIGNED, "ids_out is not 4-byte aligned");
  hipLaunchKernelGGL(random_select_kernel, dim3(n_batch), dim3(PF_MAX_TOPK), 0, static_cast<hipStream_t>(stream),
                     n_blocks, top_k, seed, counter, ids_out);
  return pf::launch_status("pf_select_random");
}
