// Partition attention over the bounded three-partition context.
//
// PackForcing digest (paper.rainbus.top), 前置知识 KV缓存 and 方法步骤详情 (5);
// arXiv HTML, "Bounded Attention Context": the current block's queries attend,
// with a single softmax, over sink || selected mid blocks || recent || current.
// The selected mid blocks are read where they sit in the pool, through the id
// list; nothing is concatenated in memory.
//
// Design (gfx950, wave64, bf16 MFMA 32x32x16 with fp32 accumulation):
//  * A workgroup of 4 waves owns 128 queries of one head; each wave owns 32.
//  * Keys stream in tiles of 64 through LDS (double-buffered, loaded with
//    16-byte global loads, rows resolved per partition). K and V stay row-major
//    in LDS; the PV product reads V with the gfx950 transposing LDS read.
//  * The score tile is computed transposed, S^T = K Q^T, so each lane holds one
//    query's scores in registers: row max / row sum are per-lane (plus one swap
//    between the two half-waves for the max), and the probabilities are already
//    in the B-operand layout of O^T = V^T P^T.
//  * Online softmax in the log2 domain (scale * log2 e folded into one FMA).
//  * Workgroups are numbered so that each XCD (workgroup id mod 8) walks a
//    contiguous range of (head, query tile) pairs: tiles that share K/V share
//    that XCD's L2.
#include <math.h>

#include "pf_internal.h"

namespace {

using pf::bf16x8;
using pf::floatx16;
using pf::short4v;

constexpr int D = PF_HEAD_DIM;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;       // queries per workgroup
constexpr int kBN = 64;                // keys per tile
constexpr int kStride = D + 16;        // LDS row stride in bf16 (288 bytes): conflict-free reads
constexpr int kTileElems = kBN * kStride;
constexpr int kXcds = 8;

struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const uint16_t* k_rec;
  const uint16_t* v_rec;
  const uint16_t* k_cur;
  const uint16_t* v_cur;
  const int32_t* mid_ids;
  int64_t n_q;
  int32_t H;
  int32_t n_c;
  int32_t n_sel;
  int32_t n_blocks;
  int32_t e_sink, e_mid, e_rec, e_cur;   // cumulative ends of the partitions (e_cur = key count)
  int32_t num_qtiles;
  int32_t total_tiles;
  float scale_log2;
};

// Source row of virtual key kk for head h; returns false for keys that do not
// exist (past the end, or inside a mid block whose id is out of range).
__device__ __forceinline__ bool resolve_key(const AttnArgs& a, const int32_t* ids_lds, int32_t kk,
                                            const uint16_t*& kp, const uint16_t*& vp, int64_t& off) {
  int64_t row;
  if (kk < a.e_sink) {
    kp = a.k_sink; vp = a.v_sink; row = kk;
  } else if (kk < a.e_mid) {
    const int32_t x = kk - a.e_sink;
    const int32_t b = x / a.n_c;
    const int32_t id = ids_lds[b];
    if (id < 0 || id >= a.n_blocks) return false;
    kp = a.k_pool; vp = a.v_pool; row = static_cast<int64_t>(id) * a.n_c + (x - b * a.n_c);
  } else if (kk < a.e_rec) {
    kp = a.k_rec; vp = a.v_rec; row = kk - a.e_mid;
  } else if (kk < a.e_cur) {
    kp = a.k_cur; vp = a.v_cur; row = kk - a.e_rec;
  } else {
    return false;
  }
  off = row * a.H * D;
  return true;
}

struct TileRegs {
  uint4 k[4];
  uint4 v[4];
  bool valid[4];
};

// Thread t moves 16-byte chunk (t & 15) of tile rows (t >> 4) + 16 i, i < 4.
__device__ __forceinline__ void load_tile(const AttnArgs& a, const int32_t* ids_lds, int h, int32_t k0,
                                          TileRegs& r) {
  const int t = threadIdx.x;
  const int col = (t & 15) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 4) + 16 * i;
    const uint16_t* kp;
    const uint16_t* vp;
    int64_t off;
    r.valid[i] = resolve_key(a, ids_lds, k0 + row, kp, vp, off);
    if (r.valid[i]) {
      off += static_cast<int64_t>(h) * D + col;
      r.k[i] = *reinterpret_cast<const uint4*>(kp + off);
      r.v[i] = *reinterpret_cast<const uint4*>(vp + off);
    } else {
      r.k[i] = make_uint4(0, 0, 0, 0);
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* ks, uint16_t* vs, uint8_t* kbad) {
  const int t = threadIdx.x;
  const int col = (t & 15) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 4) + 16 * i;
    *reinterpret_cast<uint4*>(ks + row * kStride + col) = r.k[i];
    *reinterpret_cast<uint4*>(vs + row * kStride + col) = r.v[i];
    if ((t & 15) == 0) kbad[row] = r.valid[i] ? 0 : 1;
  }
}

__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ short4v lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

__global__ __launch_bounds__(kThreads, 1) void partition_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kTileElems];
  __shared__ uint8_t kbad[2][kBN];
  __shared__ int32_t ids_lds[PF_MAX_SELECTED];
  __shared__ int any_bad_id;

  // XCD-aware numbering: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles (head-major, then query tile).
  const int b = blockIdx.x;
  const int per = a.total_tiles / kXcds, rem = a.total_tiles % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int h = logical / a.num_qtiles;
  const int64_t q0 = static_cast<int64_t>(logical % a.num_qtiles) * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;      // half-wave
  const int l32 = lane & 31;

  if (tid == 0) any_bad_id = 0;
  __syncthreads();
  for (int i = tid; i < a.n_sel; i += kThreads) {
    const int32_t id = a.mid_ids[i];
    ids_lds[i] = id;
    if (id < 0 || id >= a.n_blocks) any_bad_id = 1;
  }
  __syncthreads();
  const bool bad_ids = any_bad_id != 0;

  // Q^T operand: lane holds query (q0 + 32 wave + l32), dims 16 st + 8 g .. +7.
  const int64_t qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < a.n_q;
  bf16x8 qf[8];
  {
    const uint16_t* qp = a.q + (qvalid ? qrow : 0) * a.H * D + static_cast<int64_t>(h) * D + 8 * g;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * st);
      if (!qvalid) v = bf16x8{};
      qf[st] = v;
    }
  }

  floatx16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = floatx16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int32_t n_keys = a.e_cur;
  const int n_tiles = (n_keys + kBN - 1) / kBN;

  TileRegs regs;
  load_tile(a, ids_lds, h, 0, regs);
  store_tile(regs, ks[0], vs[0], kbad[0]);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int32_t k0 = it * kBN;
    const bool has_next = it + 1 < n_tiles;
    if (has_next) load_tile(a, ids_lds, h, k0 + kBN, regs);

    const uint16_t* kt = ks[buf];
    const uint16_t* vt = vs[buf];

    // ---- S^T = K Q^T for two 32-key blocks ----
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      const uint16_t* kr = kt + (kb * 32 + l32) * kStride + 8 * g;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kr + 16 * st), qf[st], s[kb], 0, 0, 0);
    }

    // ---- mask keys that do not exist ----
    const bool need_mask = (k0 + kBN > n_keys) || (bad_ids && k0 < a.e_mid && k0 + kBN > a.e_sink);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (kbad[buf][key]) s[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(fmaf(s[kb][i], a.scale_log2, -m_use));
        s[kb][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    // ---- P^T as the B operand: chunk c covers keys 16c .. 16c+15 ----
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[c][t] = static_cast<__bf16>(s[c >> 1][8 * (c & 1) + t]);

    // ---- O^T += V^T P^T ----
    // Transposing read: lane (row 16c + 4g + (lane&15)/4, col 32db + 16((lane>>4)&1) + 4(lane&3))
    // delivers dims 32db + l32 for keys 16c + 4g + 0..3 (and +8 for the second read).
    const int vrow = 4 * g + ((lane & 15) >> 2);
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vp = vt + (16 * c + vrow) * kStride + 32 * db + vcol;
        const short4v lo = lds_read_tr(vp);
        const short4v hi = lds_read_tr(vp + 8 * kStride);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], acc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile(regs, ks[buf ^ 1], vs[buf ^ 1], kbad[buf ^ 1]);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* op = a.o + qrow * a.H * D + static_cast<int64_t>(h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int dim = 32 * db + 8 * qd + 4 * g;
        uint2 w;
        w.x = pf::pack_bf16x2(acc[db][4 * qd + 0] * inv, acc[db][4 * qd + 1] * inv);
        w.y = pf::pack_bf16x2(acc[db][4 * qd + 2] * inv, acc[db][4 * qd + 3] * inv);
        *reinterpret_cast<uint2*>(op + dim) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<int64_t>(h) * a.n_q + qrow] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

bool is_aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" size_t pf_partition_attn_workspace_bytes(int64_t n_q, int n_heads, int64_t n_keys) {
  (void)n_q;
  (void)n_heads;
  (void)n_keys;
  return 0;
}

extern "C" pf_status pf_partition_attn(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* sink_k,
                                       const pf_bf16* sink_v, int64_t n_sink, const pf_bf16* pool_k,
                                       const pf_bf16* pool_v, int n_blocks, int n_c, const int32_t* mid_ids,
                                       int n_sel, const pf_bf16* recent_k, const pf_bf16* recent_v,
                                       int64_t n_recent, const pf_bf16* cur_k, const pf_bf16* cur_v, int64_t n_cur,
                                       float scale, pf_bf16* o, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  PF_REQUIRE_PTR(q);
  PF_REQUIRE_PTR(o);
  PF_REQUIRE_ALIGNED(q);
  PF_REQUIRE_ALIGNED(o);
  PF_REQUIRE(n_q >= 1, PF_ERR_SHAPE, "n_q must be >= 1");
  PF_REQUIRE(n_heads >= 1 && n_heads <= PF_MAX_HEADS, PF_ERR_UNSUPPORTED,
             "n_heads must be in [1, %d] (got %d)", PF_MAX_HEADS, n_heads);
  PF_REQUIRE(n_sink >= 0 && n_recent >= 0 && n_cur >= 0, PF_ERR_SHAPE, "partition row counts must be >= 0");
  PF_REQUIRE(n_sel >= 0 && n_sel <= PF_MAX_SELECTED, PF_ERR_RANGE, "n_sel must be in [0, %d] (got %d)",
             PF_MAX_SELECTED, n_sel);
  if (n_sink > 0) {
    PF_REQUIRE_PTR(sink_k);
    PF_REQUIRE_PTR(sink_v);
    PF_REQUIRE_ALIGNED(sink_k);
    PF_REQUIRE_ALIGNED(sink_v);
  }
  if (n_recent > 0) {
    PF_REQUIRE_PTR(recent_k);
    PF_REQUIRE_PTR(recent_v);
    PF_REQUIRE_ALIGNED(recent_k);
    PF_REQUIRE_ALIGNED(recent_v);
  }
  if (n_cur > 0) {
    PF_REQUIRE_PTR(cur_k);
    PF_REQUIRE_PTR(cur_v);
    PF_REQUIRE_ALIGNED(cur_k);
    PF_REQUIRE_ALIGNED(cur_v);
  }
  if (n_sel > 0) {
    PF_REQUIRE_PTR(pool_k);
    PF_REQUIRE_PTR(pool_v);
    PF_REQUIRE_PTR(mid_ids);
    PF_REQUIRE_ALIGNED(pool_k);
    PF_REQUIRE_ALIGNED(pool_v);
    PF_REQUIRE(is_aligned4(mid_ids), PF_ERR_MISALIGNED, "mid_ids is not 4-byte aligned");
    PF_REQUIRE(n_c >= 1, PF_ERR_SHAPE, "n_c must be >= 1 when n_sel > 0");
    PF_REQUIRE(n_blocks >= 1 && n_sel <= n_blocks, PF_ERR_RANGE, "n_sel (%d) must be <= n_blocks (%d)", n_sel,
               n_blocks);
  }
  PF_REQUIRE(is_aligned4(lse), PF_ERR_MISALIGNED, "lse is not 4-byte aligned");
  const int64_t n_mid = n_sel > 0 ? static_cast<int64_t>(n_sel) * n_c : 0;
  const int64_t n_keys = n_sink + n_mid + n_recent + n_cur;
  PF_REQUIRE(n_keys >= 1, PF_ERR_SHAPE, "the context has no keys");
  PF_REQUIRE(n_keys < (int64_t{1} << 31) - kBN, PF_ERR_UNSUPPORTED, "too many keys (%lld)",
             static_cast<long long>(n_keys));
  const int64_t num_qtiles = (n_q + kBM - 1) / kBM;
  const int64_t total = num_qtiles * n_heads;
  PF_REQUIRE(total < 0x7FFFFFFF, PF_ERR_UNSUPPORTED, "too many query tiles");

  AttnArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.o = reinterpret_cast<uint16_t*>(o);
  a.lse = lse;
  a.k_sink = reinterpret_cast<const uint16_t*>(sink_k);
  a.v_sink = reinterpret_cast<const uint16_t*>(sink_v);
  a.k_pool = reinterpret_cast<const uint16_t*>(pool_k);
  a.v_pool = reinterpret_cast<const uint16_t*>(pool_v);
  a.k_rec = reinterpret_cast<const uint16_t*>(recent_k);
  a.v_rec = reinterpret_cast<const uint16_t*>(recent_v);
  a.k_cur = reinterpret_cast<const uint16_t*>(cur_k);
  a.v_cur = reinterpret_cast<const uint16_t*>(cur_v);
  a.mid_ids = mid_ids;
  a.n_q = n_q;
  a.H = n_heads;
  a.n_c = n_sel > 0 ? n_c : 1;
  a.n_sel = n_sel;
  a.n_blocks = n_blocks;
  a.e_sink = static_cast<int32_t>(n_sink);
  a.e_mid = static_cast<int32_t>(n_sink + n_mid);
  a.e_rec = static_cast<int32_t>(n_sink + n_mid + n_recent);
  a.e_cur = static_cast<int32_t>(n_keys);
  a.num_qtiles = static_cast<int32_t>(num_qtiles);
  a.total_tiles = static_cast<int32_t>(total);
  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(D));
  a.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  hipLaunchKernelGGL(partition_attn_kernel, dim3(static_cast<unsigned>(total)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return pf::launch_status("pf_partition_attn");
}
