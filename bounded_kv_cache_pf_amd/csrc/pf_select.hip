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
// The scoring reads Q and the whole pool once (HBM-bound), in four launches on
// one stream:
//   1. colsum: every workgroup sums a segment of rows (a 64-row slice of Q, or a
//      slice of one pool block) column by column into fp32 partials;
//   2. qsum:   the Q partials are added in segment order;
//   3. score:  one workgroup per block adds its slices and dots with the Q sum;
//   4. topk:   one workgroup bitonic-sorts (score desc, index asc) keys in LDS
//              and writes the first k ids in ascending order.
// Every sum runs in a fixed order, so identical blocks get identical scores
// and repeated calls give identical bits.
#include <math.h>

#include "pf_internal.h"

namespace {

constexpr int kQSegRows = 64;      // rows of Q per colsum workgroup
constexpr int kTargetSegments = 512;

struct SelectPlan {
  int H, cw;          // heads, 16-byte column chunks per row (H*16)
  int rpar;           // row-parallel thread groups per colsum workgroup
  int64_t n_q;
  int nq_seg;         // Q segments
  int n_blocks, n_c;
  int ksub;           // slices per pool block
  int sub_rows;       // rows per slice (last slice may be shorter)
  size_t off_partials, off_qsum, off_scores, bytes;
};

SelectPlan make_plan(int64_t n_q, int H, int n_blocks, int n_c) {
  SelectPlan p{};
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
  const size_t cols = static_cast<size_t>(H) * PF_HEAD_DIM;
  const size_t n_seg = static_cast<size_t>(p.nq_seg) + static_cast<size_t>(n_blocks) * p.ksub;
  p.off_partials = 0;
  p.off_qsum = n_seg * cols * sizeof(float);
  p.off_scores = p.off_qsum + cols * sizeof(float);
  p.bytes = p.off_scores + static_cast<size_t>(n_blocks) * sizeof(float);
  p.bytes = (p.bytes + 255) & ~static_cast<size_t>(255);
  return p;
}

// 1. Column sums of row segments. blockDim = (cw, rpar); thread (x, y) owns the
// 8 columns of chunk x and rows y, y+rpar, ... of its segment.
__global__ void colsum_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool,
                              float* __restrict__ partials, int64_t n_q, int nq_seg, int n_c,
                              int ksub, int sub_rows) {
  extern __shared__ float red[];   // [rpar][cw*8]
  const int cw = blockDim.x, rpar = blockDim.y;
  const int x = threadIdx.x, y = threadIdx.y;
  const int seg = blockIdx.x;
  const uint16_t* base;
  int64_t rows;
  if (seg < nq_seg) {
    const int64_t r0 = static_cast<int64_t>(seg) * kQSegRows;
    rows = n_q - r0 < kQSegRows ? n_q - r0 : kQSegRows;
    base = q + r0 * cw * 8;
  } else {
    const int s = seg - nq_seg;
    const int blk = s / ksub, sub = s % ksub;
    const int r_in = sub * sub_rows;
    rows = n_c - r_in < sub_rows ? n_c - r_in : sub_rows;
    base = pool + (static_cast<int64_t>(blk) * n_c + r_in) * cw * 8;
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t stride = static_cast<int64_t>(cw) * 8;
  for (int64_t r = y; r < rows; r += rpar) {
    const uint4 w = *reinterpret_cast<const uint4*>(base + r * stride + x * 8);
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
    float* out = partials + static_cast<int64_t>(seg) * stride + x * 8;
    reinterpret_cast<float4*>(out)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(out)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// 2. Q sum: column c = sum over Q segments, in segment order.
__global__ __launch_bounds__(256) void qsum_kernel(const float* __restrict__ partials, float* __restrict__ qsum,
                                                   int nq_seg, int cols) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int i = 0; i < nq_seg; ++i) s += partials[static_cast<int64_t>(i) * cols + c];
  qsum[c] = s;
}

// 3. Block score: one workgroup per pool block.
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ partials, const float* __restrict__ qsum,
                                                    float* __restrict__ scores, float* __restrict__ scores_out,
                                                    int nq_seg, int ksub, int cols, float norm) {
  __shared__ float red[256];
  const int blk = blockIdx.x;
  const float* kp = partials + (static_cast<int64_t>(nq_seg) + static_cast<int64_t>(blk) * ksub) * cols;
  float dot = 0.f;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    float ks = 0.f;
    for (int s = 0; s < ksub; ++s) ks += kp[static_cast<int64_t>(s) * cols + c];
    dot += qsum[c] * ks;
  }
  red[threadIdx.x] = dot;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float s = red[0] * norm;
    scores[blk] = s;
    if (scores_out) scores_out[blk] = s;
  }
}

// Ascending order of the key == descending score, then ascending index.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t idx) {
  if (s == 0.f) s = 0.f;   // -0 and +0 tie
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending float order
  return (static_cast<uint64_t>(~u) << 32) | idx;
}

// 4. Top-k: bitonic sort of up to PF_MAX_BLOCKS keys in LDS, one workgroup.
constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int n_blocks,
                                                             int top_k, int32_t* __restrict__ ids_out) {
  __shared__ uint64_t keys[PF_MAX_BLOCKS];
  __shared__ uint32_t chosen[PF_MAX_TOPK];
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
          const uint64_t a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < top_k) chosen[threadIdx.x] = static_cast<uint32_t>(keys[threadIdx.x] & 0xFFFFFFFFu);
  __syncthreads();
  if (threadIdx.x < top_k) {
    const uint32_t me = chosen[threadIdx.x];
    int rank = 0;
    for (int r = 0; r < top_k; ++r) rank += chosen[r] < me;
    ids_out[rank] = static_cast<int32_t>(me);
  }
}

__global__ __launch_bounds__(PF_MAX_TOPK) void deltas_kernel(const int32_t* __restrict__ ids, int top_k,
                                                             int32_t* __restrict__ tags, int n_blocks,
                                                             int32_t recent_first_frame, int32_t block_frames,
                                                             int32_t* __restrict__ deltas) {
  const int r = threadIdx.x;
  if (r >= top_k) return;
  const int32_t id = ids[r];
  if (id < 0 || id >= n_blocks) {
    deltas[r] = 0;
    return;
  }
  const int32_t target = recent_first_frame - (top_k - r) * block_frames;
  deltas[r] = target - tags[id];
  tags[id] = target;
}

}  // namespace

extern "C" size_t pf_score_select_workspace_bytes(int64_t n_q, int n_heads, int n_blocks, int n_c) {
  if (n_q < 1 || n_heads < 1 || n_heads > PF_MAX_HEADS || n_blocks < 1 || n_blocks > PF_MAX_BLOCKS || n_c < 1)
    return 0;
  return make_plan(n_q, n_heads, n_blocks, n_c).bytes;
}

extern "C" pf_status pf_score_select(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* pool_k,
                                     int n_blocks, int n_c, int top_k, int32_t* ids_out, float* scores_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
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
  PF_REQUIRE(n_q <= (int64_t{1} << 40), PF_ERR_UNSUPPORTED, "n_q too large");
  PF_REQUIRE_ALIGNED(q);
  PF_REQUIRE_ALIGNED(pool_k);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(ids_out) & 3u) == 0, PF_ERR_MISALIGNED, "ids_out is not 4-byte aligned");
  PF_REQUIRE((reinterpret_cast<uintptr_t>(scores_out) & 3u) == 0, PF_ERR_MISALIGNED,
             "scores_out is not 4-byte aligned");
  const SelectPlan p = make_plan(n_q, n_heads, n_blocks, n_c);
  PF_REQUIRE(workspace != nullptr, PF_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", p.bytes);
  PF_REQUIRE(workspace_bytes >= p.bytes, PF_ERR_WORKSPACE, "workspace has %zu bytes, need %zu",
             workspace_bytes, p.bytes);
  PF_REQUIRE_ALIGNED(workspace);
  PF_REQUIRE(static_cast<int64_t>(p.nq_seg) + static_cast<int64_t>(n_blocks) * p.ksub < 0x7FFFFFFF,
             PF_ERR_UNSUPPORTED, "too many segments");

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* partials = reinterpret_cast<float*>(ws + p.off_partials);
  float* qsum = reinterpret_cast<float*>(ws + p.off_qsum);
  float* scores = reinterpret_cast<float*>(ws + p.off_scores);
  const int cols = n_heads * PF_HEAD_DIM;
  const int n_seg = p.nq_seg + n_blocks * p.ksub;

  const size_t lds = static_cast<size_t>(p.rpar) * p.cw * 8 * sizeof(float);
  hipLaunchKernelGGL(colsum_kernel, dim3(n_seg), dim3(p.cw, p.rpar), lds, st,
                     reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(pool_k), partials,
                     n_q, p.nq_seg, n_c, p.ksub, p.sub_rows);
  pf_status s = pf::launch_status("pf_score_select (colsum)");
  if (s != PF_OK) return s;
  hipLaunchKernelGGL(qsum_kernel, dim3((cols + 255) / 256), dim3(256), 0, st, partials, qsum, p.nq_seg, cols);
  s = pf::launch_status("pf_score_select (qsum)");
  if (s != PF_OK) return s;
  const double norm = 1.0 / (static_cast<double>(n_q) * n_c * n_heads * sqrt(static_cast<double>(PF_HEAD_DIM)));
  hipLaunchKernelGGL(score_kernel, dim3(n_blocks), dim3(256), 0, st, partials, qsum, scores, scores_out,
                     p.nq_seg, p.ksub, cols, static_cast<float>(norm));
  s = pf::launch_status("pf_score_select (score)");
  if (s != PF_OK) return s;
  hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kTopkThreads), 0, st, scores, n_blocks, top_k, ids_out);
  return pf::launch_status("pf_score_select (topk)");
}

extern "C" pf_status pf_selection_deltas(const int32_t* ids, int top_k, int32_t* pos_tags, int n_blocks,
                                         int32_t recent_first_frame, int32_t block_frames, int32_t* deltas_out,
                                         void* stream) {
  PF_REQUIRE_PTR(ids);
  PF_REQUIRE_PTR(pos_tags);
  PF_REQUIRE_PTR(deltas_out);
  PF_REQUIRE(n_blocks >= 1, PF_ERR_SHAPE, "n_blocks must be >= 1");
  PF_REQUIRE(top_k >= 1 && top_k <= PF_MAX_TOPK && top_k <= n_blocks, PF_ERR_RANGE,
             "top_k must be in [1, min(n_blocks, %d)] (got %d)", PF_MAX_TOPK, top_k);
  PF_REQUIRE(block_frames >= 1, PF_ERR_RANGE, "block_frames must be >= 1");
  PF_REQUIRE(((reinterpret_cast<uintptr_t>(ids) | reinterpret_cast<uintptr_t>(pos_tags) |
               reinterpret_cast<uintptr_t>(deltas_out)) & 3u) == 0,
             PF_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
  hipLaunchKernelGGL(deltas_kernel, dim3(1), dim3(PF_MAX_TOPK), 0, static_cast<hipStream_t>(stream), ids, top_k,
                     pos_tags, n_blocks, recent_first_frame, block_frames, deltas_out);
  return pf::launch_status("pf_selection_deltas");
}
