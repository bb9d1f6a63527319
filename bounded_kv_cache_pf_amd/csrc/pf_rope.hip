// Incremental temporal RoPE shift, in place on bf16 keys.
//
// PackForcing digest (paper.rainbus.top), 前置知识 RoPE and 方法步骤详情 (4);
// arXiv HTML, "Incremental RoPE adjustment": a cached key already carries
// e^{i theta p}; multiplying by e^{i theta_t delta} moves it to p + delta on the
// temporal axis while the height and width rotations stay the identity.
//
// The rotation runs in fp64 and is rounded once to bf16, so the stored key is
// the correctly rounded rotation of the stored input.
//
// HBM-bound: each row-head reads and writes the 88 bytes of its 44 temporal
// dims. Eight lanes serve one row-head, 16 bytes each (dims 8c..8c+7), so a
// wave touches eight 256-byte row-heads with full-width vector accesses. Lanes
// 0..4 rotate dims 0..39 and lane 5 dims 40..43; lane 5 writes dims 44..47 and
// lanes 6 and 7 dims 48..63 back with their own bits, so every store covers
// the row-head's whole first 128-byte line: the caches then never merge a
// partly written line with the old contents from memory.
// Each lane's loads are issued before the workgroup computes its fp64 cos/sin
// table, so the table's latency hides under the memory latency.
#include <math.h>

#include "pf_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRowHead = 8;
constexpr int kRowHeadsPerPass = kThreads / kLanesPerRowHead;  // 32
// Row-heads per lane: four keep 64 KB of each large launch in flight per
// workgroup; a small launch (one layer's selected blocks) takes two, twice the
// workgroups, each with a shorter chain of loads, rotations and stores
// (1.2 us faster for one layer, 10% slower on 30 layers' blocks).
constexpr int kPassesLarge = 4;
constexpr int kPassesSmall = 2;
constexpr int64_t kSmallLaunchRowHeads = int64_t{1} << 17;
constexpr int kPairs = PF_TEMPORAL_DIMS / 2;                   // 22

// fp64 -> bf16 with a single round-to-nearest-even. The hardware fp64 -> fp32
// conversion rounds to nearest; a second rounding to bf16 can only go wrong
// when the fp32 value sits exactly on a bf16 midpoint while the fp64 value
// does not, and then nudging it one fp32 step toward the fp64 value settles
// the tie on the correct side.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const float r = static_cast<float>(d);
  uint32_t rb = __float_as_uint(r);
  if ((rb & 0xFFFFu) == 0x8000u && static_cast<double>(r) != d) rb += fabs(d) > fabs(static_cast<double>(r)) ? 1u : 0xFFFFFFFFu;
  if ((rb & 0x7F800000u) == 0x7F800000u) return rb >> 16;   // inf stays inf
  return (rb + 0x7FFFu + ((rb >> 16) & 1u)) >> 16;
}

// (x + iy) * (c + is) in fp64, stored back as a bf16 pair.
__device__ __forceinline__ void rotate_pair(uint32_t& packed, double c, double s) {
  const double x = pf::bf16_to_f32(static_cast<uint16_t>(packed & 0xFFFFu));
  const double y = pf::bf16_to_f32(static_cast<uint16_t>(packed >> 16));
  const double xr = x * c - y * s;
  const double yr = x * s + y * c;
  packed = f64_to_bf16_rne(xr) | (f64_to_bf16_rne(yr) << 16);
}

template <int kPasses>
__global__ __launch_bounds__(kThreads) void rope_shift_kernel(
    uint16_t* __restrict__ k, int64_t k_bstride, int64_t row_heads_per_block, int64_t n_blocks,
    const int32_t* __restrict__ block_ids, const int32_t* __restrict__ deltas, int n_shift, double base) {
  const int64_t entry = static_cast<int64_t>(blockIdx.z) * n_shift + blockIdx.y;
  const int64_t blk = block_ids ? static_cast<int64_t>(block_ids[entry]) : blockIdx.y;
  const int delta = deltas[entry];
  if (blk < 0 || blk >= n_blocks || delta == 0) return;   // delta 0 is the identity

  const int sub = threadIdx.x % kLanesPerRowHead;
  const int local = threadIdx.x / kLanesPerRowHead;
  uint16_t* blk_base = k + blockIdx.z * k_bstride + blk * row_heads_per_block * PF_HEAD_DIM;
  constexpr int kRowHeadsPerBlock = kRowHeadsPerPass * kPasses;
  const int64_t rh0 = static_cast<int64_t>(blockIdx.x) * kRowHeadsPerBlock + local;
  // all loads first (kPasses row-heads in flight per lane), then rotate and store
  uint4 w[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int64_t rh = rh0 + pass * kRowHeadsPerPass;
    w[pass] = make_uint4(0, 0, 0, 0);
    if (rh < row_heads_per_block) {
      const uint16_t* p = blk_base + rh * PF_HEAD_DIM + sub * 8;
      w[pass] = *reinterpret_cast<const uint4*>(p);
    }
  }
  __shared__ double cs[kPairs], sn[kPairs];
  if (threadIdx.x < kPairs) {
    const double theta = pow(base, -2.0 * threadIdx.x / PF_TEMPORAL_DIMS);
    sincos(theta * static_cast<double>(delta), &sn[threadIdx.x], &cs[threadIdx.x]);
  }
  __syncthreads();

#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int64_t rh = rh0 + pass * kRowHeadsPerPass;
    if (rh >= row_heads_per_block) break;
    uint16_t* p = blk_base + rh * PF_HEAD_DIM + sub * 8;
    if (sub < 5) {
      const int j = sub * 4;
      rotate_pair(w[pass].x, cs[j + 0], sn[j + 0]);
      rotate_pair(w[pass].y, cs[j + 1], sn[j + 1]);
      rotate_pair(w[pass].z, cs[j + 2], sn[j + 2]);
      rotate_pair(w[pass].w, cs[j + 3], sn[j + 3]);
      *reinterpret_cast<uint4*>(p) = w[pass];
    } else if (sub == 5) {
      rotate_pair(w[pass].x, cs[20], sn[20]);
      rotate_pair(w[pass].y, cs[21], sn[21]);
      *reinterpret_cast<uint4*>(p) = w[pass];
    } else {
      *reinterpret_cast<uint4*>(p) = w[pass];
    }
  }
}

}  // namespace

extern "C" pf_status pf_rope_shift_batched(pf_bf16* k, int64_t k_batch_stride, int n_heads, int64_t rows_per_block,
                                           int64_t n_blocks, const int32_t* block_ids, const int32_t* deltas,
                                           int n_shift, int n_batch, double rope_base, void* stream) {
  PF_REQUIRE(n_shift >= 0, PF_ERR_RANGE, "n_shift must be >= 0 (got %d)", n_shift);
  PF_REQUIRE(n_heads >= 1 && n_heads <= PF_MAX_HEADS, PF_ERR_UNSUPPORTED,
             "n_heads must be in [1, %d] (got %d)", PF_MAX_HEADS, n_heads);
  PF_REQUIRE(rows_per_block >= 1, PF_ERR_SHAPE, "rows_per_block must be >= 1");
  PF_REQUIRE(n_blocks >= 1, PF_ERR_SHAPE, "n_blocks must be >= 1");
  PF_REQUIRE(rope_base > 1.0, PF_ERR_RANGE, "rope_base must be > 1");
  PF_REQUIRE(n_batch >= 1 && n_batch <= PF_MAX_BATCH, PF_ERR_RANGE, "n_batch must be in [1, %d] (got %d)",
             PF_MAX_BATCH, n_batch);
  if (block_ids == nullptr)
    PF_REQUIRE(n_shift <= n_blocks, PF_ERR_RANGE, "n_shift (%d) exceeds n_blocks without block_ids", n_shift);
  PF_REQUIRE(n_shift <= 65535, PF_ERR_UNSUPPORTED, "n_shift must be <= 65535");
  if (n_batch > 1) {
    PF_REQUIRE(k_batch_stride >= rows_per_block * n_blocks * n_heads * PF_HEAD_DIM, PF_ERR_SHAPE,
               "k_batch_stride (%lld) is smaller than one cache's keys", static_cast<long long>(k_batch_stride));
    PF_REQUIRE(k_batch_stride % 8 == 0, PF_ERR_MISALIGNED, "k_batch_stride must be a multiple of 8 elements");
  }
  if (n_shift == 0) return pf::ok();
  PF_REQUIRE_PTR(k);
  PF_REQUIRE_PTR(deltas);
  PF_REQUIRE_ALIGNED(k);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(deltas) & 3u) == 0, PF_ERR_MISALIGNED, "deltas is not 4-byte aligned");
  PF_REQUIRE((reinterpret_cast<uintptr_t>(block_ids) & 3u) == 0, PF_ERR_MISALIGNED, "block_ids is not 4-byte aligned");

  const int64_t rh_per_block = rows_per_block * n_heads;
  const bool small = rh_per_block * n_shift * n_batch <= kSmallLaunchRowHeads;
  const int64_t per_wg = kRowHeadsPerPass * (small ? kPassesSmall : kPassesLarge);
  const int64_t gx = (rh_per_block + per_wg - 1) / per_wg;
  PF_REQUIRE(gx <= 0x7FFFFFFF, PF_ERR_UNSUPPORTED, "block too large");
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(n_shift), static_cast<unsigned>(n_batch));
  if (small)
    hipLaunchKernelGGL(rope_shift_kernel<kPassesSmall>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<uint16_t*>(k), n_batch > 1 ? k_batch_stride : 0, rh_per_block, n_blocks,
                       block_ids, deltas, n_shift, rope_base);
  else
    hipLaunchKernelGGL(rope_shift_kernel<kPassesLarge>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<uint16_t*>(k), n_batch > 1 ? k_batch_stride : 0, rh_per_block, n_blocks,
                       block_ids, deltas, n_shift, rope_base);
  return pf::launch_status("pf_rope_shift");
}

extern "C" pf_status pf_rope_shift(pf_bf16* k, int n_heads, int64_t rows_per_block, int64_t n_blocks,
                                   const int32_t* block_ids, const int32_t* deltas, int n_shift,
                                   double rope_base, void* stream) {
  return pf_rope_shift_batched(k, 0, n_heads, rows_per_block, n_blocks, block_ids, deltas, n_shift, 1, rope_base,
                               stream);
}
