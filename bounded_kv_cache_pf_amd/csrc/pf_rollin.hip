// Roll-in of one compressed block into the mid pool.
//
// PackForcing arXiv HTML, "Dual-Resolution Shifting Mechanism": while a block
// is generated, a reduced-resolution backup of its keys and values is kept;
// when the block leaves the recent window the backup joins the mid buffer.
// Its keys still carry the positions they were encoded at, so the pool slot's
// position tag becomes the first frame the block held.
//
// A plain device copy (HBM-bound, 16-byte vector accesses) plus one tag
// write; it is meant to run on a stream of its own, overlapped with the
// attention of the next block, which never reads the slot being filled.
#include "pf_internal.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void rollin_kernel(uint4* __restrict__ pool_k, uint4* __restrict__ pool_v,
                                                          int64_t pool_bstride16, const uint4* __restrict__ blk_k,
                                                          const uint4* __restrict__ blk_v, int64_t blk_bstride16,
                                                          int64_t n16, int32_t* __restrict__ tags, int tags_bstride,
                                                          int slot, int32_t first_frame) {
  const int64_t b = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n16) {
    pool_k[b * pool_bstride16 + i] = blk_k[b * blk_bstride16 + i];
    pool_v[b * pool_bstride16 + i] = blk_v[b * blk_bstride16 + i];
  }
  if (i == 0 && tags != nullptr) tags[b * tags_bstride + slot] = first_frame;
}

}  // namespace

extern "C" pf_status pf_rollin_batched(pf_bf16* pool_k, pf_bf16* pool_v, int64_t pool_batch_stride,
                                       int32_t* pos_tags, int tags_batch_stride, int n_heads, int n_c, int slot,
                                       const pf_bf16* block_k, const pf_bf16* block_v, int64_t block_batch_stride,
                                       int32_t first_frame, int n_batch, void* stream) {
  PF_REQUIRE_PTR(pool_k);
  PF_REQUIRE_PTR(pool_v);
  PF_REQUIRE_PTR(block_k);
  PF_REQUIRE_PTR(block_v);
  PF_REQUIRE(n_heads >= 1 && n_heads <= PF_MAX_HEADS, PF_ERR_UNSUPPORTED, "n_heads must be in [1, %d] (got %d)",
             PF_MAX_HEADS, n_heads);
  PF_REQUIRE(n_c >= 1, PF_ERR_SHAPE, "n_c must be >= 1");
  PF_REQUIRE(slot >= 0, PF_ERR_RANGE, "slot must be >= 0 (got %d)", slot);
  PF_REQUIRE(n_batch >= 1 && n_batch <= PF_MAX_BATCH, PF_ERR_RANGE, "n_batch must be in [1, %d] (got %d)",
             PF_MAX_BATCH, n_batch);
  const int64_t blk_elems = static_cast<int64_t>(n_c) * n_heads * PF_HEAD_DIM;
  if (n_batch > 1) {
    PF_REQUIRE(pool_batch_stride >= (static_cast<int64_t>(slot) + 1) * blk_elems, PF_ERR_SHAPE,
               "pool_batch_stride (%lld) does not hold slot %d", static_cast<long long>(pool_batch_stride), slot);
    PF_REQUIRE(block_batch_stride >= blk_elems, PF_ERR_SHAPE, "block_batch_stride is smaller than one block");
    PF_REQUIRE(pool_batch_stride % 8 == 0 && block_batch_stride % 8 == 0, PF_ERR_MISALIGNED,
               "batch strides must be multiples of 8 elements");
    if (pos_tags != nullptr)
      PF_REQUIRE(tags_batch_stride > slot, PF_ERR_SHAPE, "tags_batch_stride must exceed slot");
  }
  PF_REQUIRE_ALIGNED(pool_k);
  PF_REQUIRE_ALIGNED(pool_v);
  PF_REQUIRE_ALIGNED(block_k);
  PF_REQUIRE_ALIGNED(block_v);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(pos_tags) & 3u) == 0, PF_ERR_MISALIGNED, "pos_tags is not 4-byte aligned");
  const int64_t n16 = blk_elems / 8;   // 128 dims per head: always a whole number of 16-byte vectors
  const int64_t gx = (n16 + kThreads - 1) / kThreads;
  PF_REQUIRE(gx <= 0x7FFFFFFF, PF_ERR_UNSUPPORTED, "block too large");
  uint4* pk = reinterpret_cast<uint4*>(pool_k) + static_cast<int64_t>(slot) * n16;
  uint4* pv = reinterpret_cast<uint4*>(pool_v) + static_cast<int64_t>(slot) * n16;
  hipLaunchKernelGGL(rollin_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(n_batch)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), pk, pv, n_batch > 1 ? pool_batch_stride / 8 : 0,
                     reinterpret_cast<const uint4*>(block_k), reinterpret_cast<const uint4*>(block_v),
                     n_batch > 1 ? block_batch_stride / 8 : 0, n16, pos_tags, n_batch > 1 ? tags_batch_stride : 0,
                     slot, first_frame);
  return pf::launch_status("pf_rollin");
}

extern "C" pf_status pf_rollin(pf_bf16* pool_k, pf_bf16* pool_v, int32_t* pos_tags, int n_heads, int n_c, int slot,
                               const pf_bf16* block_k, const pf_bf16* block_v, int32_t first_frame, void* stream) {
  return pf_rollin_batched(pool_k, pool_v, 0, pos_tags, 0, n_heads, n_c, slot, block_k, block_v, 0, first_frame, 1,
                           stream);
}
