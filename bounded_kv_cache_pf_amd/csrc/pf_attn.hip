// Partition attention over the bounded three-partition context.
//
// PackForcing digest (paper.rainbus.top), 前置知识 KV缓存 and 方法步骤详情 (5);
// arXiv HTML, "Bounded Attention Context": the current block's queries attend,
// with a single softmax, over sink || selected mid blocks || recent || current.
// The selected mid blocks are read where they sit in the pool, through the id
// list; nothing is concatenated in memory.
//
// Design (gfx950, wave64, bf16 MFMA 32x32x16 with fp32 accumulation):
//  * A workgroup of 8 waves owns a unit = 256 queries of one head; each wave
//    owns 32 queries and two waves share each SIMD, so one wave's softmax
//    overlaps the other's matrix products. Every K/V tile brought into LDS
//    feeds 256 queries.
//  * The MFMA operands read from LDS run kRing-1 MFMAs ahead of their use
//    (an operand ring), so no MFMA waits on the LDS latency of its own read.
//  * Keys stream in tiles of 128 straight from global memory into LDS (raw
//    buffer loads, 16 bytes per lane, no register staging), double buffered.
//    Each 256-byte LDS row holds one key's 128 dims with its 16-byte chunks
//    XOR-swizzled by the row, so the K reads (16 bytes per lane) and the
//    transposing V reads (8 bytes per lane) hit distinct banks. The next
//    tile's loads are spread over the current tile's QK MFMAs when the tile
//    lies in one partition or holds mid keys only; a tile across a partition
//    boundary resolves each row and loads in one burst.
//  * The score tile is computed transposed, S^T = K Q^T, so each lane holds
//    half of one query's 128 scores and the other half-wave the rest: the row
//    max needs one swap between half-waves, the row sum none, and the
//    probabilities are already in the B-operand layout of O^T = V^T P^T. V is
//    read with the gfx950 transposing LDS read.
//  * Online softmax in the log2 domain, with a fast path: a tile's scores are
//    exponentiated against the running max without searching for the tile's
//    own max. Only a row's first tile, a tile with masked keys, or a tile whose
//    row sum passes 2^64 (a score far above the running max) takes the exact
//    path: its scores are recomputed from LDS, the max is searched, and the
//    running max is raised when the tile's max exceeds it by more than 2^8
//    (then O is rescaled; a wave-uniform branch). Probabilities and O stay
//    far inside the fp32 and bf16 range either way.
//  * Scheduling: with G resident workgroups and U units, the first
//    floor(U/G) rounds give every workgroup whole units, numbered so that each
//    XCD walks consecutive units of one head in lockstep (shared K/V in its
//    L2). The units of full query tiles come first and the heads' last,
//    partial query tiles after them, so the partial ones fall in the tail.
//    The R remaining units are cut into key segments, one segment count per
//    kind of unit (full or partial), chosen so that the segments end close
//    together: a wave whose 32 queries all lie past the last query only loads
//    its share of each tile, which makes a partial unit with at most four live
//    waves cheaper per tile. Neighbouring workgroups take the same segment of
//    different full units, so they too read the same keys together; the
//    partial units (one per head, none sharing keys) are spread over all
//    XCDs. Segments write unnormalised partial results that a small merge
//    kernel combines. This removes the tail round of idle CUs.
#include <math.h>

#include <mutex>

#include "pf_internal.h"

namespace {

using pf::bf16x8;
using pf::floatx16;
using pf::short4v;

constexpr int D = PF_HEAD_DIM;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;         // queries per unit
constexpr int kBN = 128;                 // keys per tile
constexpr int kNB = kBN / 32;            // 32-key blocks per tile
constexpr int kRowsPerWave = kBN / kWaves;   // tile rows each wave loads
constexpr int kLoadsPerWave = kRowsPerWave / 4;   // four rows (1 KB) per load instruction
constexpr int kOcc = 1;                  // workgroups per CU the kernel is built for
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;    // log2 units: p may grow to 2^8 before a rescale
constexpr float kPsumLimit = 0x1p64f;     // fast-path row sums above this take the exact path
constexpr int kMinTailTiles = 16;        // shortest run of key tiles worth a partial
constexpr size_t kPartFloats = static_cast<size_t>(kBM) * D + 2 * kBM;   // U, m, l
constexpr size_t kPartBytes = kPartFloats * 4;

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
  const uint16_t* k_safe;   // a row that exists, loaded for masked keys
  const uint16_t* v_safe;
  const int32_t* mid_ids;
  float* part;              // partial results of split units (workspace)
  int64_t n_q;
  int64_t row_stride;       // H * 128
  int32_t H;
  int32_t n_c;
  int32_t n_sel;
  int32_t n_blocks;
  int32_t e_sink, e_mid, e_rec, e_cur;   // cumulative ends of the partitions (e_cur = key count)
  int32_t units;            // query units (ceil(n_q / kBM) per head) x H
  int32_t n_kt;             // key tiles per unit
  int32_t G;                // workgroups in the grid
  int32_t rounds;           // rounds of whole units
  int32_t nfull;            // query units per head with kBM real queries
  int32_t tail_f, tail_p;   // tail units with kBM real queries / with fewer
  int32_t seg_f, seg_p;     // key segments per tail unit of each kind (1: it runs whole)
  float scale_log2;
  float inv_nc;             // 1 / n_c
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS row r stores its 16-byte chunk j at position j ^ swz(r). swz is a
// bijection of r mod 16, so 16 consecutive rows read at one logical chunk hit
// 16 distinct chunks (the K reads), and the 4-row x 4-chunk footprint of a
// transposing V read lands on 16 distinct chunks as well.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Tiles are loaded with raw buffer loads straight into LDS (16 bytes per
// lane, no register staging). Word 3 of a gfx9-family buffer descriptor:
// 32-bit data format, everything else zero. Offsets are 32-bit, so each
// descriptor starts near the rows it serves (a tile's first row in its
// partition; the pool, whose rows the ids scatter, from its start).
constexpr int kRsrcWord3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const uint16_t* p, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, static_cast<int>(n), kRsrcWord3);
}

// One 1 KB load: 64 lanes x 16 bytes from descriptor r at byte offset voff
// into four consecutive 256-byte LDS rows starting at lds.
__device__ __forceinline__ void dma16(rsrc_t r, uint16_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Tile layout in LDS: wave w fills rows kRowsPerWave*w .., four rows (1 KB)
// per load; lane L lands on row kRowsPerWave*w + 4i + L/16 at physical chunk
// L%16, so it fetches logical chunk (L%16) ^ swz(row).
__device__ __forceinline__ int tile_row(int wave_u, int lane, int i) {
  return kRowsPerWave * wave_u + 4 * i + (lane >> 4);
}
__device__ __forceinline__ int chunk_bytes(int lane, int row) { return ((lane & 15) ^ swz(row)) << 4; }

// A tile whose loads can be spread over the MFMAs: one descriptor pair and
// this lane's byte offset for each of the wave's loads.
struct TileSrc {
  rsrc_t k, v;
  int voff[kLoadsPerWave];
};

// x / n_c for a mid key's offset x (0 <= x < n_sel * n_c, so the quotient is
// below PF_MAX_SELECTED): an fp32 estimate is within one of the quotient, and
// one correction step fixes it. (Integer division has no instruction here.)
__device__ __forceinline__ int32_t mid_block(int32_t x, int32_t n_c, float inv_nc) {
  int32_t q = static_cast<int32_t>(static_cast<float>(x) * inv_nc);
  const int32_t r = x - q * n_c;
  if (r < 0)
    --q;
  else if (r >= n_c)
    ++q;
  return q;
}

// Tile inside one contiguous partition (sink, recent or current).
__device__ __forceinline__ bool contiguous_tile(const AttnArgs& a, int h, int32_t kt, int wave_u, int lane,
                                                TileSrc& t) {
  const int32_t k0 = kt * kBN;
  const uint16_t* kb;
  const uint16_t* vb;
  int32_t r0, rows;
  if (k0 + kBN <= a.e_sink) {
    kb = a.k_sink; vb = a.v_sink; r0 = k0; rows = a.e_sink;
  } else if (k0 >= a.e_mid && k0 + kBN <= a.e_rec) {
    kb = a.k_rec; vb = a.v_rec; r0 = k0 - a.e_mid; rows = a.e_rec - a.e_mid;
  } else if (k0 >= a.e_rec && k0 + kBN <= a.e_cur) {
    kb = a.k_cur; vb = a.v_cur; r0 = k0 - a.e_rec; rows = a.e_cur - a.e_rec;
  } else {
    return false;
  }
  const int64_t off = static_cast<int64_t>(r0) * a.row_stride + h * D;
  const int64_t bytes = (static_cast<int64_t>(rows - r0) * a.row_stride - h * D) * 2;
  t.k = make_rsrc(kb + off, bytes);
  t.v = make_rsrc(vb + off, bytes);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = tile_row(wave_u, lane, i);
    t.voff[i] = static_cast<int>(row * a.row_stride * 2) + chunk_bytes(lane, row);
  }
  return true;
}

// Tile of mid keys only: rows of the selected pool blocks, found through the
// ids. Rows of an invalid id read pool row 0 and are flagged in kbad.
__device__ __forceinline__ bool mid_tile(const AttnArgs& a, const int32_t* ids_lds, int h, int32_t kt, int wave_u,
                                         int lane, uint8_t* kbad, TileSrc& t) {
  const int32_t k0 = kt * kBN;
  if (k0 < a.e_sink || k0 + kBN > a.e_mid) return false;
  const int64_t hb = static_cast<int64_t>(h) * D;
  const int64_t bytes = (static_cast<int64_t>(a.n_blocks) * a.n_c * a.row_stride - hb) * 2;
  t.k = make_rsrc(a.k_pool + hb, bytes);
  t.v = make_rsrc(a.v_pool + hb, bytes);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = tile_row(wave_u, lane, i);
    const int32_t x = k0 + row - a.e_sink;
    const int32_t b = mid_block(x, a.n_c, a.inv_nc);
    const int32_t id = ids_lds[b];
    const bool ok = id >= 0 && id < a.n_blocks;
    const int64_t prow = ok ? static_cast<int64_t>(id) * a.n_c + (x - b * a.n_c) : 0;
    t.voff[i] = static_cast<int>(prow * a.row_stride * 2) + chunk_bytes(lane, row);
    if ((lane & 15) == 0) kbad[row] = ok ? 0 : 1;
  }
  return true;
}

// Load j (0 .. 2*kLoadsPerWave-1: the K loads, then the V loads) of this
// wave's share of a spreadable tile.
__device__ __forceinline__ void load_part(const TileSrc& t, int j, uint16_t* ks, uint16_t* vs, int wave_u) {
  const int i = j % kLoadsPerWave;
  const int lds_row = kRowsPerWave * wave_u + 4 * i;
  if (j < kLoadsPerWave)
    dma16(t.k, ks + lds_row * D, t.voff[i]);
  else
    dma16(t.v, vs + lds_row * D, t.voff[i]);
}

// Any tile, row by row: each lane resolves its key to a partition and a row
// there (mid keys through the ids; keys past the end and rows of an invalid id
// read the safe row and are flagged in kbad). One load per partition present
// among a load's lanes, masked to those lanes. Used for the tiles that
// straddle a partition boundary or run past the last key.
__device__ __forceinline__ void load_general(const AttnArgs& a, const int32_t* ids_lds, int h, int32_t kt,
                                             uint16_t* ks, uint16_t* vs, uint8_t* kbad, int wave_u, int lane) {
  const int32_t k0 = kt * kBN;
  const int64_t hb = static_cast<int64_t>(h) * D;
  const int64_t rs = a.row_stride;
  // first row of each contiguous partition the descriptors start at
  const int32_t b_sink = k0;
  const int32_t b_rec = (k0 > a.e_mid ? k0 : a.e_mid) - a.e_mid;
  const int32_t b_cur = (k0 > a.e_rec ? k0 : a.e_rec) - a.e_rec;
  int part[kLoadsPerWave], voff[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = tile_row(wave_u, lane, i);
    const int32_t kk = k0 + row;
    int pt = 4;
    int64_t prow = 0;
    if (kk < a.e_sink) {
      pt = 0; prow = kk - b_sink;
    } else if (kk < a.e_mid) {
      const int32_t x = kk - a.e_sink;
      const int32_t b = mid_block(x, a.n_c, a.inv_nc);
      const int32_t id = ids_lds[b];
      if (id >= 0 && id < a.n_blocks) {
        pt = 1; prow = static_cast<int64_t>(id) * a.n_c + (x - b * a.n_c);
      }
    } else if (kk < a.e_rec) {
      pt = 2; prow = kk - a.e_mid - b_rec;
    } else if (kk < a.e_cur) {
      pt = 3; prow = kk - a.e_rec - b_cur;
    }
    part[i] = pt;
    voff[i] = static_cast<int>(prow * rs * 2) + chunk_bytes(lane, row);
    if ((lane & 15) == 0) kbad[row] = pt == 4 ? 1 : 0;
  }
#pragma unroll
  for (int pt = 0; pt < 5; ++pt) {
    const uint16_t* kb = pt == 0 ? a.k_sink : pt == 1 ? a.k_pool : pt == 2 ? a.k_rec : pt == 3 ? a.k_cur : a.k_safe;
    const uint16_t* vb = pt == 0 ? a.v_sink : pt == 1 ? a.v_pool : pt == 2 ? a.v_rec : pt == 3 ? a.v_cur : a.v_safe;
    const int64_t first = pt == 0 ? b_sink : pt == 2 ? b_rec : pt == 3 ? b_cur : 0;
    const int64_t rows = pt == 0   ? a.e_sink
                         : pt == 1 ? static_cast<int64_t>(a.n_blocks) * a.n_c
                         : pt == 2 ? a.e_rec - a.e_mid
                         : pt == 3 ? a.e_cur - a.e_rec
                                   : 1;
    const int64_t off = first * rs + hb;
    const int64_t bytes = ((rows - first) * rs - hb) * 2;
    const rsrc_t rk = make_rsrc(kb + off, bytes);
    const rsrc_t rv = make_rsrc(vb + off, bytes);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      if (__builtin_amdgcn_ballot_w64(part[i] == pt) == 0) continue;
      if (part[i] == pt) {
        const int lds_row = kRowsPerWave * wave_u + 4 * i;
        dma16(rk, ks + lds_row * D, voff[i]);
        dma16(rv, vs + lds_row * D, voff[i]);
      }
    }
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

__device__ __forceinline__ short4v lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

// Operand ring of a run of N MFMAs whose operands take RPO LDS reads each:
// keep the reads of the first kRing-1 operands, then MFMA i followed by the
// reads of operand i+kRing-1, in that order in the final schedule.
constexpr int kRing = 3;

// With DM > 0, a vector-memory load follows every DM-th MFMA as well.
template <int N, int RPO, int DM, int I>
__device__ __forceinline__ void sched_ring_step() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + kRing - 1 < N) __builtin_amdgcn_sched_group_barrier(0x100, RPO, 0);
    if constexpr (DM > 0 && I % DM == DM - 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    sched_ring_step<N, RPO, DM, I + 1>();
  }
}

template <int N, int RPO, int DM = 0>
__device__ __forceinline__ void sched_ring() {
  __builtin_amdgcn_sched_group_barrier(0x100, (kRing - 1) * RPO, 0);
  sched_ring_step<N, RPO, DM, 0>();
}

struct Smem {
  uint16_t ks[2][kBN * D];
  uint16_t vs[2][kBN * D];
  uint8_t kbad[2][kBN];
  int32_t ids[PF_MAX_SELECTED];
  int any_bad_id;
};

// Units are numbered head-major over the full query units of every head
// first, then the last, partial unit of each head (when n_q is not a
// multiple of kBM), so that the partial units, which cost less, fall in the
// tail where they get their own segment count.
__device__ __forceinline__ void unit_coords(const AttnArgs& a, int unit, int& h, int64_t& q0) {
  const int full = a.H * a.nfull;
  if (unit < full) {
    h = unit / a.nfull;
    q0 = static_cast<int64_t>(unit - h * a.nfull) * kBM;
  } else {
    h = unit - full;
    q0 = static_cast<int64_t>(a.nfull) * kBM;
  }
}

// One unit (head h, queries q0 .. q0+kBM-1) over key tiles [kt0, kt1).
// direct: the run covers the whole unit -> write O (and LSE); otherwise write
// the unnormalised partial U, m (log2 domain) and l to partial slot `slot`.
__device__ __forceinline__ void run_unit(const AttnArgs& a, Smem& sm, int h, int64_t q0, int kt0, int kt1,
                                         bool direct, int64_t slot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // Q^T operand: query q0 + 32 wave + l32, dims 16 st + 8 g .. +7.
  const int64_t qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < a.n_q;
  // a wave whose queries all lie past n_q only loads its share of each tile
  const bool live = q0 + 32 * wave_u < a.n_q;
  bf16x8 qf[8];
  {
    const uint16_t* qp = a.q + (qvalid ? qrow : 0) * a.row_stride + static_cast<int64_t>(h) * D + 8 * g;
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

  // Per-lane LDS offsets (elements), loop invariant.
  // K (A operand of S^T): row kb*32 + l32, logical chunk 2st + g.
  int k_off[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) k_off[st] = l32 * D + (((2 * st + g) ^ swz(l32)) << 3);
  // V (transposing read): row 16c + 4g + (lane&15)/4 (+8 for the second read),
  // logical elements 32db + 16dh + 4(lane&3) = chunk 4db + 2dh + (lane&3)/2, half lane&1.
  const int v_r = 4 * g + ((lane & 15) >> 2);
  const int v_x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_h = 4 * (lane & 1);
  int v_lo[4], v_hi[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    v_lo[db] = v_r * D + (((4 * db + v_x) ^ swz(v_r)) << 3) + v_h;
    v_hi[db] = (v_r + 8) * D + (((4 * db + v_x) ^ swz(v_r + 8)) << 3) + v_h;
  }
  {
    TileSrc t;
    if (contiguous_tile(a, h, kt0, wave_u, lane, t) || mid_tile(a, sm.ids, h, kt0, wave_u, lane, sm.kbad[0], t)) {
#pragma unroll
      for (int j = 0; j < 2 * kLoadsPerWave; ++j) load_part(t, j, sm.ks[0], sm.vs[0], wave_u);
    } else {
      load_general(a, sm.ids, h, kt0, sm.ks[0], sm.vs[0], sm.kbad[0], wave_u, lane);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const bool bad_ids = sm.any_bad_id != 0;
  // One key tile. The tile's buffers and the next tile's are distinct, and
  // saying so (restrict) lets the compiler see that the LDS reads of this
  // tile do not wait for the loads of the next one in flight.
  auto step = [&](int32_t kt, const uint16_t* __restrict__ kt_lds, const uint16_t* __restrict__ vt_lds,
                  const uint8_t* __restrict__ kbad_cur, uint16_t* __restrict__ k_next,
                  uint16_t* __restrict__ v_next, uint8_t* __restrict__ kbad_next) {
    const int32_t k0 = kt * kBN;
    // Next tile: inside one partition its loads are spread over the QK MFMAs
    // below (in a burst they would stall the issuing waves behind the
    // vector-memory address queue); a tile across a boundary loads here.
    TileSrc nt;
    bool spread = false;
    if (kt + 1 < kt1) {
      spread = contiguous_tile(a, h, kt + 1, wave_u, lane, nt) ||
               mid_tile(a, sm.ids, h, kt + 1, wave_u, lane, kbad_next, nt);
      if (!spread) load_general(a, sm.ids, h, kt + 1, k_next, v_next, kbad_next, wave_u, lane);
    }
    if (!live) {
      if (spread) {
#pragma unroll
        for (int j = 0; j < 2 * kLoadsPerWave; ++j) load_part(nt, j, k_next, v_next, wave_u);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      return;
    }

    // ---- S^T = K Q^T for kNB 32-key blocks ----
    // operand i: dims 16st.. (st = i/kNB) of key block kb = i%kNB, so the kNB
    // accumulator chains alternate; operand i+kRing-1 is read while MFMA i issues
    floatx16 s[kNB];
    auto qk = [&]() {
      auto load_k = [&](int i) { return *reinterpret_cast<const bf16x8*>(kt_lds + (i % kNB) * 32 * D + k_off[i / kNB]); };
      bf16x8 op[kRing];
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) op[r] = load_k(r);
#pragma unroll
      for (int i = 0; i < 8 * kNB; ++i) {
        if (i + kRing - 1 < 8 * kNB) op[(i + kRing - 1) % kRing] = load_k(i + kRing - 1);
        s[i % kNB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % kRing], qf[i / kNB], i < kNB ? floatx16{} : s[i % kNB],
                                                           0, 0, 0);
      }
      sched_ring<8 * kNB, 1>();
    };
    if (spread) {
      // the same products with the next tile's loads, one per kDm MFMAs
      constexpr int kDm = 8 * kNB / (2 * kLoadsPerWave);
      auto load_k = [&](int i) { return *reinterpret_cast<const bf16x8*>(kt_lds + (i % kNB) * 32 * D + k_off[i / kNB]); };
      bf16x8 op[kRing];
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) op[r] = load_k(r);
#pragma unroll
      for (int i = 0; i < 8 * kNB; ++i) {
        if (i + kRing - 1 < 8 * kNB) op[(i + kRing - 1) % kRing] = load_k(i + kRing - 1);
        s[i % kNB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % kRing], qf[i / kNB], i < kNB ? floatx16{} : s[i % kNB],
                                                           0, 0, 0);
        if (i % kDm == kDm - 1) load_part(nt, i / kDm, k_next, v_next, wave_u);
      }
      sched_ring<8 * kNB, 1, kDm>();
    } else {
      qk();
    }

    // ---- online softmax (log2 domain, lazy rescale) ----
    // Fast path: exponentiate against the running max without looking for the
    // tile's max; the tile only needs the exact path (mask, max, rescale) when
    // it has masked keys, is a row's first tile, or a probability grew past
    // 2^64 (seen in the row sum), and then its scores are recomputed from LDS.
    const bool need_mask = (k0 + kBN > a.e_cur) || (bad_ids && k0 < a.e_mid && k0 + kBN > a.e_sink);
    bool slow = need_mask || __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    float psum = 0.f;
    if (!slow) {
#pragma unroll
      for (int kb = 0; kb < kNB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -m_run));
          s[kb][i] = p;
          psum += p;
        }
      slow = __builtin_amdgcn_ballot_w64(!(psum <= kPsumLimit)) != 0;
      if (slow) qk();
    }
    if (slow) {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < kNB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (kbad_cur[key]) s[kb][i] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int kb = 1; kb < kNB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = half_swap_max(mx) * a.scale_log2;
      const bool grow = mx > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < kNB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -m_use));
          s[kb][i] = p;
          psum += p;
        }
    }
    l_run += psum;

    // ---- P^T as the B operand: chunk c covers keys 16c .. 16c+15 ----
    bf16x8 pb[2 * kNB];
#pragma unroll
    for (int c = 0; c < 2 * kNB; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[c][t] = static_cast<__bf16>(s[c >> 1][8 * (c & 1) + t]);

    // ---- O^T += V^T P^T ----
    // operand i: keys 16c.. (c = i/4), dims 32db.. (db = i%4): four chains
    {
      auto load_v = [&](int i) {
        const short4v lo = lds_read_tr(vt_lds + 16 * (i >> 2) * D + v_lo[i & 3]);
        const short4v hi = lds_read_tr(vt_lds + 16 * (i >> 2) * D + v_hi[i & 3]);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 op[kRing];
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) op[r] = load_v(r);
#pragma unroll
      for (int i = 0; i < 8 * kNB; ++i) {
        if (i + kRing - 1 < 8 * kNB) op[(i + kRing - 1) % kRing] = load_v(i + kRing - 1);
        acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % kRing], pb[i >> 2], acc[i & 3], 0, 0, 0);
      }
      sched_ring<8 * kNB, 2>();
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int32_t kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    step(kt, sm.ks[buf], sm.vs[buf], sm.kbad[buf], sm.ks[buf ^ 1], sm.vs[buf ^ 1], sm.kbad[buf ^ 1]);
  }

  const float l_tot = half_swap_sum(l_run);
  if (direct) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
      uint16_t* op = a.o + qrow * a.row_stride + static_cast<int64_t>(h) * D;
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
      // log2 of l by the hardware log (v_log_f32 is base 2); LSE in natural log
      if (a.lse != nullptr && g == 0)
        a.lse[static_cast<int64_t>(h) * a.n_q + qrow] =
            l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  } else {
    // partial slot: U [256 queries][128 dims], then m [256], l [256]
    float* base = a.part + slot * static_cast<int64_t>(kPartFloats);
    const int ql = wave * 32 + l32;
    float* up = base + static_cast<int64_t>(ql) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int dim = 32 * db + 8 * qd + 4 * g;
        *reinterpret_cast<float4*>(up + dim) =
            make_float4(acc[db][4 * qd + 0], acc[db][4 * qd + 1], acc[db][4 * qd + 2], acc[db][4 * qd + 3]);
      }
    if (g == 0) {
      base[kBM * D + ql] = m_run;
      base[kBM * D + kBM + ql] = l_tot;
    }
  }
}

// Workgroup g runs on XCD g % 8; XCD x gets the consecutive slots x*G/8 .. .
__device__ __forceinline__ int xcd_slot(int g, int G) {
  return (G % kXcds == 0) ? (g % kXcds) * (G / kXcds) + g / kXcds : g;
}

__global__ __launch_bounds__(kThreads, kOcc) void partition_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const int tid = threadIdx.x;
  if (tid == 0) sm.any_bad_id = 0;
  __syncthreads();
  for (int i = tid; i < a.n_sel; i += kThreads) {
    const int32_t id = a.mid_ids[i];
    sm.ids[i] = id;
    if (id < 0 || id >= a.n_blocks) sm.any_bad_id = 1;
  }
  __syncthreads();

  const int slot = xcd_slot(blockIdx.x, a.G);
  for (int r = 0; r < a.rounds; ++r) {
    const int unit = r * a.G + slot;
    if (unit >= a.units) break;
    int h;
    int64_t q0;
    unit_coords(a, unit, h, q0);
    run_unit(a, sm, h, q0, 0, a.n_kt, true, 0);
  }
  // Tail items: the segments of the full tail units (n_f of them, segment-
  // major: item k is segment k / tail_f of unit k % tail_f), then those of the
  // partial ones (n_p). Item k of the full kind writes partial slot k, item k
  // of the partial kind slot n_f + k. The items are laid out in one sequence
  // with the partial ones spread evenly among the full ones, and each XCD
  // takes a run of consecutive positions: neighbouring workgroups take the
  // same segment of different full units and share those keys in their XCD's
  // L2, while the partial units, each alone with its keys, are spread over
  // all XCDs.
  const int n_f = a.seg_f * a.tail_f;
  const int n_p = a.seg_p * a.tail_p;
  const int n_items = n_f + n_p;
  int pos = -1;
  if (a.G % kXcds == 0) {
    const int per = a.G / kXcds;
    const int x = slot / per;
    const int j = slot - x * per;
    const int lo = static_cast<int>(static_cast<int64_t>(x) * n_items / kXcds);
    const int hi = static_cast<int>(static_cast<int64_t>(x + 1) * n_items / kXcds);
    if (j < hi - lo) pos = lo + j;
  } else if (slot < n_items) {
    pos = slot;
  }
  if (pos >= 0) {
    const int p0 = static_cast<int>(static_cast<int64_t>(pos) * n_p / n_items);
    const int p1 = static_cast<int>(static_cast<int64_t>(pos + 1) * n_p / n_items);
    int seg, tu, nseg, buf;
    if (p1 > p0) {
      seg = p0 / a.tail_p;
      tu = a.tail_f + p0 - seg * a.tail_p;
      nseg = a.seg_p;
      buf = n_f + p0;
    } else {
      const int k = pos - p0;
      seg = k / a.tail_f;
      tu = k - seg * a.tail_f;
      nseg = a.seg_f;
      buf = k;
    }
    const int kt0 = static_cast<int>(static_cast<int64_t>(seg) * a.n_kt / nseg);
    const int kt1 = static_cast<int>(static_cast<int64_t>(seg + 1) * a.n_kt / nseg);
    int h;
    int64_t q0;
    unit_coords(a, a.units - a.tail_f - a.tail_p + tu, h, q0);
    run_unit(a, sm, h, q0, kt0, kt1, nseg == 1, buf);
  }
}

// Merge the segments of cut units. Workgroup (tu, y) takes queries
// 32y .. 32y+31 of tail unit tu, whose segment c wrote partial slot
// first + c * stride; eight threads share a query, 16 dims each.
constexpr int kMergeQueries = 32;

__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int tu = blockIdx.x;
  const bool kind_f = tu < a.tail_f;
  const int nseg = kind_f ? a.seg_f : a.seg_p;
  if (nseg <= 1) return;
  const int64_t first = kind_f ? tu : static_cast<int64_t>(a.seg_f) * a.tail_f + (tu - a.tail_f);
  const int64_t stride = kind_f ? a.tail_f : a.tail_p;
  int h;
  int64_t q0;
  unit_coords(a, a.units - a.tail_f - a.tail_p + tu, h, q0);
  const int ql = blockIdx.y * kMergeQueries + (threadIdx.x >> 3);
  const int d0 = (threadIdx.x & 7) * 16;
  const int64_t qrow = q0 + ql;
  float m = -INFINITY;
  for (int c = 0; c < nseg; ++c) m = fmaxf(m, a.part[(first + c * stride) * kPartFloats + kBM * D + ql]);
  const float m_use = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = 0.f;
  for (int c = 0; c < nseg; ++c) {
    const float* base = a.part + (first + c * stride) * kPartFloats;
    const float w = __builtin_amdgcn_exp2f(base[kBM * D + ql] - m_use);
    l += w * base[kBM * D + kBM + ql];
    const float* up = base + static_cast<int64_t>(ql) * D + d0;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(up + i);
      u[i] += w * v.x;
      u[i + 1] += w * v.y;
      u[i + 2] += w * v.z;
      u[i + 3] += w * v.w;
    }
  }
  if (qrow >= a.n_q) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* op = a.o + qrow * a.row_stride + static_cast<int64_t>(h) * D + d0;
#pragma unroll
  for (int i = 0; i < 16; i += 8) {
    uint4 w;
    w.x = pf::pack_bf16x2(u[i] * inv, u[i + 1] * inv);
    w.y = pf::pack_bf16x2(u[i + 2] * inv, u[i + 3] * inv);
    w.z = pf::pack_bf16x2(u[i + 4] * inv, u[i + 5] * inv);
    w.w = pf::pack_bf16x2(u[i + 6] * inv, u[i + 7] * inv);
    *reinterpret_cast<uint4*>(op + i) = w;
  }
  if (a.lse != nullptr && d0 == 0)
    a.lse[static_cast<int64_t>(h) * a.n_q + qrow] =
        l > 0.f ? (m_use + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
}

// ---- launch plan ----

struct Plan {
  int64_t units = 0, n_kt = 0;
  int grid = 0, G = 0, rounds = 0, nfull = 0, tail_f = 0, tail_p = 0, seg_f = 0, seg_p = 0;
  size_t ws_bytes = 0;
};

int resident_workgroups() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, partition_attn_kernel, kThreads, 0) != hipSuccess ||
        per <= 0)
      per = 1;
    cached[dev] = cus * per;
  }
  return cached[dev];
}

// Cost of a key tile for a unit whose live waves each have a SIMD to
// themselves (at most 4 of its 8 waves hold queries), relative to a unit whose
// SIMDs each run two live waves. Measured on the default layer's shape (3 live
// waves): cutting those units into 4 segments instead of 5 did not lengthen
// the tail, so such a tile costs at most about 2/3 of a full one.
constexpr double kLoneWaveCost = 0.75;

// Rounds of whole units first; a remainder under 3/4 of the machine is cut
// into key segments (each at least kMinTailTiles tiles), otherwise it runs as
// one more round of whole units. The tail holds up to two kinds of unit: full
// ones, and the partial last units of the heads, which cost less per tile
// when at most four of their waves hold queries. Each kind gets one segment
// count; the dearer kind (longest segment x cost) gets one more segment per
// unit while the machine holds them, so the slots end close to together.
Plan make_plan(int64_t n_q, int H, int64_t n_keys, int resident) {
  Plan p;
  p.nfull = static_cast<int>(n_q / kBM);
  const int64_t rest = n_q - static_cast<int64_t>(p.nfull) * kBM;
  p.units = (static_cast<int64_t>(p.nfull) + (rest > 0 ? 1 : 0)) * H;
  p.n_kt = (n_keys + kBN - 1) / kBN;
  const int64_t full = p.units / resident;
  const int64_t rem = p.units - full * resident;
  p.rounds = static_cast<int>(full);
  if (rem > 0 && (rem * 4 < static_cast<int64_t>(resident) * 3 || full == 0)) {
    const int64_t partial_units = rest > 0 ? H : 0;
    p.tail_p = static_cast<int>(rem < partial_units ? rem : partial_units);
    p.tail_f = static_cast<int>(rem - p.tail_p);
    const double cost_p = (rest + 31) / 32 <= 4 ? kLoneWaveCost : 1.0;
    int64_t max_seg = p.n_kt / kMinTailTiles;
    if (max_seg < 1) max_seg = 1;
    p.seg_f = p.tail_f > 0 ? 1 : 0;
    p.seg_p = p.tail_p > 0 ? 1 : 0;
    int64_t used = rem;
    for (;;) {
      const double len_f = p.tail_f > 0 ? static_cast<double>(p.n_kt) / p.seg_f : 0.0;
      const double len_p = p.tail_p > 0 ? cost_p * static_cast<double>(p.n_kt) / p.seg_p : 0.0;
      const bool inc_f = p.tail_f > 0 && len_f >= len_p;
      const bool inc_p = p.tail_p > 0 && len_p >= len_f;
      const int64_t need = (inc_f ? p.tail_f : 0) + (inc_p ? p.tail_p : 0);
      if (used + need > resident) break;
      if ((inc_f && p.seg_f + 1 > max_seg) || (inc_p && p.seg_p + 1 > max_seg)) break;
      p.seg_f += inc_f ? 1 : 0;
      p.seg_p += inc_p ? 1 : 0;
      used += need;
    }
    const int64_t slots = static_cast<int64_t>(p.seg_f) * p.tail_f + static_cast<int64_t>(p.seg_p) * p.tail_p;
    p.ws_bytes = (p.seg_f > 1 || p.seg_p > 1) ? static_cast<size_t>(slots) * kPartBytes : 0;
    p.grid = full > 0 ? resident : static_cast<int>(slots);
  } else {
    if (rem > 0) p.rounds += 1;
    p.grid = full > 0 ? resident : static_cast<int>(rem);
  }
  p.G = p.grid;
  return p;
}

bool is_aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" size_t pf_partition_attn_workspace_bytes(int64_t n_q, int n_heads, int64_t n_keys) {
  if (n_q < 1 || n_heads < 1 || n_heads > PF_MAX_HEADS || n_keys < 1) return 0;
  return make_plan(n_q, n_heads, n_keys, resident_workgroups()).ws_bytes;
}

namespace {

// The partial results of split units live in the caller's workspace, or, for
// pf_partition_attn_noalloc, in this fixed device array (one per GPU, for the
// life of the process). Host code never names the array in a launch: it
// passes the device address that hipGetSymbolAddress returns for the current
// device.
constexpr size_t kScratchBytes = size_t{40} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

pf_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pf::fail(PF_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return pf::fail(PF_ERR_UNSUPPORTED, "device %d is beyond the 64 this library tracks", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || p == nullptr)
      return pf::fail(PF_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g));
    addr[dev] = p;
  }
  *out = addr[dev];
  return PF_OK;
}

// Validation and launch shared by both entry points. With `use_scratch`, the
// partials go to the device's scratch array instead of `workspace`.
pf_status attn_call(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* sink_k, const pf_bf16* sink_v,
                    int64_t n_sink, const pf_bf16* pool_k, const pf_bf16* pool_v, int n_blocks, int n_c,
                    const int32_t* mid_ids, int n_sel, const pf_bf16* recent_k, const pf_bf16* recent_v,
                    int64_t n_recent, const pf_bf16* cur_k, const pf_bf16* cur_v, int64_t n_cur, float scale,
                    pf_bf16* o, float* lse, void* workspace, size_t workspace_bytes, bool use_scratch,
                    void* stream) {
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
  // pool rows are addressed with 32-bit byte offsets from the pool's start
  const int64_t pool_rows = n_sel > 0 ? static_cast<int64_t>(n_blocks) * n_c : 0;
  PF_REQUIRE(pool_rows * n_heads * D * 2 < (int64_t{1} << 31), PF_ERR_UNSUPPORTED,
             "the pool holds 2 GiB or more of K (or V)");
  const int64_t num_qtiles = (n_q + kBM - 1) / kBM;
  PF_REQUIRE(num_qtiles * n_heads < 0x7FFFFFFF, PF_ERR_UNSUPPORTED, "too many query tiles");

  const Plan p = make_plan(n_q, n_heads, n_keys, resident_workgroups());
  if (use_scratch) {
    PF_REQUIRE(p.ws_bytes <= kScratchBytes, PF_ERR_UNSUPPORTED,
               "this shape needs %zu bytes of partials, beyond the %zu-byte scratch array", p.ws_bytes,
               kScratchBytes);
    if (p.ws_bytes > 0) {
      const pf_status s = scratch_address(&workspace);
      if (s != PF_OK) return s;
    }
  } else if (p.ws_bytes > 0) {
    PF_REQUIRE(workspace != nullptr, PF_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", p.ws_bytes);
    PF_REQUIRE(workspace_bytes >= p.ws_bytes, PF_ERR_WORKSPACE, "workspace has %zu bytes, need %zu",
               workspace_bytes, p.ws_bytes);
    PF_REQUIRE_ALIGNED(workspace);
  }

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
  // masked keys load a row that exists (their scores are discarded)
  if (n_sink > 0) {
    a.k_safe = a.k_sink; a.v_safe = a.v_sink;
  } else if (n_recent > 0) {
    a.k_safe = a.k_rec; a.v_safe = a.v_rec;
  } else if (n_cur > 0) {
    a.k_safe = a.k_cur; a.v_safe = a.v_cur;
  } else {
    a.k_safe = a.k_pool; a.v_safe = a.v_pool;
  }
  a.mid_ids = mid_ids;
  a.part = static_cast<float*>(workspace);
  a.n_q = n_q;
  a.row_stride = static_cast<int64_t>(n_heads) * D;
  a.H = n_heads;
  a.n_c = n_sel > 0 ? n_c : 1;
  a.inv_nc = 1.0f / static_cast<float>(a.n_c);
  a.n_sel = n_sel;
  a.n_blocks = n_blocks;
  a.e_sink = static_cast<int32_t>(n_sink);
  a.e_mid = static_cast<int32_t>(n_sink + n_mid);
  a.e_rec = static_cast<int32_t>(n_sink + n_mid + n_recent);
  a.e_cur = static_cast<int32_t>(n_keys);
  a.units = static_cast<int32_t>(p.units);
  a.n_kt = static_cast<int32_t>(p.n_kt);
  a.G = p.G;
  a.rounds = p.rounds;
  a.nfull = p.nfull;
  a.tail_f = p.tail_f;
  a.tail_p = p.tail_p;
  a.seg_f = p.seg_f;
  a.seg_p = p.seg_p;
  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(D));
  a.scale_log2 = static_cast<float>(sc * 1.4426950408889634);

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(partition_attn_kernel, dim3(p.grid), dim3(kThreads), 0, st, a);
  pf_status s = pf::launch_status("pf_partition_attn");
  if (s != PF_OK || (p.seg_f <= 1 && p.seg_p <= 1)) return s;
  hipLaunchKernelGGL(merge_kernel, dim3(p.tail_f + p.tail_p, kBM / kMergeQueries), dim3(256), 0, st, a);
  return pf::launch_status("pf_partition_attn (merge)");
}

}  // namespace

extern "C" pf_status pf_partition_attn(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* sink_k,
                                       const pf_bf16* sink_v, int64_t n_sink, const pf_bf16* pool_k,
                                       const pf_bf16* pool_v, int n_blocks, int n_c, const int32_t* mid_ids,
                                       int n_sel, const pf_bf16* recent_k, const pf_bf16* recent_v,
                                       int64_t n_recent, const pf_bf16* cur_k, const pf_bf16* cur_v, int64_t n_cur,
                                       float scale, pf_bf16* o, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return attn_call(q, n_q, n_heads, sink_k, sink_v, n_sink, pool_k, pool_v, n_blocks, n_c, mid_ids, n_sel, recent_k,
                   recent_v, n_recent, cur_k, cur_v, n_cur, scale, o, lse, workspace, workspace_bytes, false, stream);
}

extern "C" pf_status pf_partition_attn_noalloc(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* sink_k,
                                               const pf_bf16* sink_v, int64_t n_sink, const pf_bf16* pool_k,
                                               const pf_bf16* pool_v, int n_blocks, int n_c,
                                               const int32_t* mid_ids, int n_sel, const pf_bf16* recent_k,
                                               const pf_bf16* recent_v, int64_t n_recent, const pf_bf16* cur_k,
                                               const pf_bf16* cur_v, int64_t n_cur, float scale, pf_bf16* o,
                                               float* lse, void* stream) {
  return attn_call(q, n_q, n_heads, sink_k, sink_v, n_sink, pool_k, pool_v, n_blocks, n_c, mid_ids, n_sel, recent_k,
                   recent_v, n_recent, cur_k, cur_v, n_cur, scale, o, lse, nullptr, 0, true, stream);
}
