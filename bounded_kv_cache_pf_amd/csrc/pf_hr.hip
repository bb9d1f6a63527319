// HR branch of the compressor: strided 3D convolutions with SiLU, then a
// linear 1x1x1 projection to the hidden width.
//
// PackForcing arXiv HTML, "HR Branch: Progressive 3D Convolution": the branch
// works on the VAE latent of a block, halves time once and space three times
// (a 2x8x8 = 128x volume reduction) with SiLU after every strided stage, and
// projects to the hidden width d = 1536; "Feature Fusion" gives the token
// count N_c = floor(T/2) floor(H/8) floor(W/8) (182 for a 4 x 60 x 104 latent).
// Digest (paper.rainbus.top), 前置知识 3D卷积.
//
// Each stage's kernel equals its stride (no padding), so one output position
// reads one disjoint input patch and the stage is a plain GEMM over patches:
//   y[m][n] = act(bias[n] + sum_k W[n][k] * X[m][k]),
// with m = (b, t, h, w) an output position, k = (dt, dh, dw, c) a patch
// element. Activations are channels-last bf16, [B][T][H][W][C], so a run of
// 16 consecutive k (C_in is a multiple of 16) is 32 contiguous bytes of one
// input position: the patch matrix X is never built, each MFMA operand is read
// straight from the activation tensor (an implicit GEMM).
//
// Design (gfx950, wave64, MFMA 32x32x16 bf16, fp32 accumulation):
//  * C_in a multiple of 64 (every stage but the first): a workgroup of 4
//    waves owns 128 channels x 128 positions. K advances in chunks of 64
//    elements, one 128-byte run of every weight row and patch row, moved into
//    LDS by global_load_lds (8 whole rows per instruction, double-buffered,
//    16-byte chunks XOR-swizzled by row); each wave computes a 64 x 64
//    sub-tile from LDS fragments.
//  * Otherwise (the 16-channel latent): one wave per workgroup, operands read
//    straight from global memory in the MFMA layout, eight K steps in flight.
//    Its 64 x 64 wave tile drops to 32 x 32 when K is only a few steps deep.
//  * Both use the transposed product D^T = W X^T and stage the output tile
//    through LDS, so the stores write whole rows of channels.
//  * Deep, narrow stages (few positions, K up to 4096) split K over up to 8
//    workgroups that write fp32 partials; a second kernel sums them in a fixed
//    order, adds the bias and applies SiLU. Results are bit-reproducible.
//  * Each XCD gets a contiguous slice of the larger operand (positions or
//    channels) and all of the smaller, so the smaller stays in its L2.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "pf_internal.h"

namespace {

using pf::bf16x8;
using pf::floatx16;

constexpr int kMaxSplit = 8;    // K splits of one stage
constexpr int kXcds = 8;
constexpr int kTargetWaves = 2048;
constexpr int kDepth = 8;       // K steps of operands in flight per wave
// split K only while the fp32 partials written and re-read stay under this
// multiple of the bytes the stage reads anyway (weights + activations)
constexpr double kPartialBudget = 2.0;

struct ConvArgs {
  const uint16_t* x;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  float* part;          // [n_split][M][c_out] when n_split > 1
  int32_t M;            // output positions (batch included), below 2^31
  int32_t T, H, W, c_in;
  int32_t kt, kh, kw;
  int32_t To, Ho, Wo;
  int32_t c_out, K;
  int32_t act;
  int32_t m_tiles, n_tiles, n_split, k_chunk;
  int32_t m_slow;       // 1: position tiles are the slow index (activations larger than weights)
  int32_t G;            // workgroups in the grid
};

__device__ __forceinline__ float silu(float v) {
  // v * sigmoid(v); exp2 overflows to +inf for very negative v, giving -0
  return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f));
}

// Workgroup g runs on XCD g % 8: give XCD x the consecutive logical ids
// x*G/8 .. so that neighbours (same weight slice) share an L2.
__device__ __forceinline__ int logical_id(int g, int G) {
  return (G % kXcds == 0) ? (g % kXcds) * (G / kXcds) + g / kXcds : g;
}

// One wave owns NI x 32 output channels and NJ x 32 positions (NI * NJ MFMA
// tiles): 2 x 2 normally, 1 x 1 for reductions only a few steps deep.
template <int NI, int NJ>
__global__ __launch_bounds__(64) void hr_conv_kernel(ConvArgs a) {
  const int lane = threadIdx.x;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  // logical id -> tile. The operand with more bytes is the slow index, so each
  // XCD covers one contiguous slice of it and all of the smaller operand.
  const int L = logical_id(blockIdx.x, a.G);
  const int s = L / (a.m_tiles * a.n_tiles);
  const int t = L - s * (a.m_tiles * a.n_tiles);
  const int mt = a.m_slow ? t / a.n_tiles : t % a.m_tiles;
  const int nt = a.m_slow ? t % a.n_tiles : t / a.m_tiles;
  const int n0 = nt * 32 * NI;
  const int m0 = mt * 32 * NJ;
  const int k_begin = s * a.k_chunk;
  const int k_end = min(a.K, k_begin + a.k_chunk);

  // A operand (weights): channel n0 + 32i + l32, k = k0 + 8g .. +7
  const uint16_t* wr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = min(n0 + 32 * i + l32, a.c_out - 1);
    wr[i] = a.w + static_cast<int64_t>(n) * a.K + 8 * g;
  }
  // B operand (patches): position m0 + 32j + l32 (32-bit: the host keeps M
  // below 2^31); element offset of its patch origin
  int64_t xo[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t m = static_cast<uint32_t>(min(m0 + 32 * j + l32, a.M - 1));
    const uint32_t wo = m % static_cast<uint32_t>(a.Wo);
    uint32_t r = m / static_cast<uint32_t>(a.Wo);
    const uint32_t ho = r % static_cast<uint32_t>(a.Ho);
    r /= static_cast<uint32_t>(a.Ho);
    const uint32_t to = r % static_cast<uint32_t>(a.To);
    const uint32_t b = r / static_cast<uint32_t>(a.To);
    xo[j] = (((static_cast<int64_t>(b) * a.T + to * a.kt) * a.H + ho * a.kh) * a.W + wo * a.kw) * a.c_in + 8 * g;
  }
  // element offset of patch segment seg = (dt, dh, dw) from the patch origin
  auto seg_off = [&](int seg) -> int64_t {
    const int dw = seg % a.kw;
    const int dh = (seg / a.kw) % a.kh;
    const int dt = seg / (a.kw * a.kh);
    return ((static_cast<int64_t>(dt) * a.H + dh) * a.W + dw) * a.c_in;
  };

  floatx16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx16{};

  // K loop with a ring of kDepth steps of operands in flight: step st's
  // fragments sit in ring slot st % kDepth and are loaded kDepth-1 steps
  // before its MFMAs, which hides the L2 latency even when a wave has the SIMD
  // to itself. The load cursor (all wave-uniform) walks (segment, channel)
  // without division and stops on the last step, so loads past the end repeat
  // it and every load and MFMA of the main loop is unconditional.
  const int kb0 = __builtin_amdgcn_readfirstlane(k_begin);
  const int n_steps = __builtin_amdgcn_readfirstlane(max(0, (k_end - k_begin) / 16));
  const int k_last = kb0 + 16 * (n_steps - 1);
  int cur_k = kb0;
  int cur_seg = kb0 / a.c_in;
  int cur_ci = kb0 - cur_seg * a.c_in;
  int64_t cur_base = seg_off(cur_seg);
  bf16x8 ra[kDepth][NI], rb[kDepth][NJ];
  auto load_slot = [&](bf16x8 (&av)[NI], bf16x8 (&bv)[NJ]) {
    const int64_t off = cur_base + cur_ci;
#pragma unroll
    for (int i = 0; i < NI; ++i) av[i] = *reinterpret_cast<const bf16x8*>(wr[i] + cur_k);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[j] = *reinterpret_cast<const bf16x8*>(a.x + xo[j] + off);
    if (cur_k < k_last) {
      cur_k += 16;
      cur_ci += 16;
      if (cur_ci == a.c_in) {
        cur_ci = 0;
        ++cur_seg;
        cur_base = seg_off(cur_seg);
      }
    }
  };
  auto mfma_slot = [&](const bf16x8 (&av)[NI], const bf16x8 (&bv)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  };
  if (n_steps > 0) {
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (d < n_steps) load_slot(ra[d], rb[d]);
    const int n_main = n_steps - n_steps % kDepth;
    for (int sb = 0; sb < n_main; sb += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load_slot(ra[(d + kDepth - 1) % kDepth], rb[(d + kDepth - 1) % kDepth]);
        mfma_slot(ra[d], rb[d]);
      }
    }
    // the last n_steps % kDepth steps are already in slots 0 ..
    const int n_tail = n_steps - n_main;
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (d < n_tail) mfma_slot(ra[d], rb[d]);
  }

  // D^T register r of lane l: channel 8(r/4) + 4(l/32) + r%4 of the 32-block,
  // position l%32. The tile goes through LDS ([position][channel], rows
  // padded against bank conflicts) so that global stores write whole rows.
  constexpr int kCols = 32 * NI, kStride = 32 * NI + 4;
  __shared__ __attribute__((aligned(16))) float tile[32 * NJ * kStride];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * i + 8 * q + 4 * g;
        *reinterpret_cast<float4*>(&tile[(32 * j + l32) * kStride + nl]) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  __syncthreads();
  if (a.n_split == 1) {
    // kCols/8 lanes per position, 8 channels (16 bytes of bf16) each
    constexpr int kLanesPerRow = kCols / 8, kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
    for (int pass = 0; pass < 32 * NJ / kRowsPerPass; ++pass) {
      const int pl = kRowsPerPass * pass + lane / kLanesPerRow;
      const int nl = 8 * (lane % kLanesPerRow);
      const int m = m0 + pl;
      const int n = n0 + nl;
      if (m >= a.M || n >= a.c_out) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = tile[pl * kStride + nl + e] + (a.bias != nullptr ? a.bias[n + e] : 0.f);
        if (a.act) v[e] = silu(v[e]);
      }
      uint4 pk;
      pk.x = pf::pack_bf16x2(v[0], v[1]);
      pk.y = pf::pack_bf16x2(v[2], v[3]);
      pk.z = pf::pack_bf16x2(v[4], v[5]);
      pk.w = pf::pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(a.y + static_cast<int64_t>(m) * a.c_out + n) = pk;
    }
  } else {
    // kCols/4 lanes per position, 4 channels (16 bytes of fp32) each
    constexpr int kLanesPerRow = kCols / 4, kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
    for (int pass = 0; pass < 32 * NJ / kRowsPerPass; ++pass) {
      const int pl = kRowsPerPass * pass + lane / kLanesPerRow;
      const int nl = 4 * (lane % kLanesPerRow);
      const int m = m0 + pl;
      const int n = n0 + nl;
      if (m >= a.M || n >= a.c_out) continue;
      *reinterpret_cast<float4*>(a.part + (static_cast<int64_t>(s) * a.M + m) * a.c_out + n) =
          *reinterpret_cast<const float4*>(&tile[pl * kStride + nl]);
    }
  }
}

// Workgroup-tiled variant for C_in a multiple of 64: a workgroup of 4 waves
// owns 128 channels x 128 positions. Each 64-element K chunk of its 128
// weight rows and 128 patch rows (128 contiguous bytes per row) moves into LDS
// with global_load_lds, eight whole rows per instruction, double-buffered;
// the 16-byte chunks of a row are XOR-swizzled by the row so the MFMA
// fragment reads spread over the banks. Each wave computes 64 x 64 of the
// tile from LDS.
constexpr int kBT = 128;   // workgroup tile: channels and positions
constexpr int kBK = 64;    // K elements per chunk

struct LdsTiles {
  uint16_t a[2][kBT * kBK];
  uint16_t b[2][kBT * kBK];
};
constexpr int kOutStride = kBT + 4;   // fp32 row of the staged output tile
constexpr size_t kLdsBytes =
    sizeof(LdsTiles) > kBT * kOutStride * sizeof(float) ? sizeof(LdsTiles) : kBT * kOutStride * sizeof(float);

typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(256) void hr_conv_lds_kernel(ConvArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[kLdsBytes];
  LdsTiles& sm = *reinterpret_cast<LdsTiles*>(lds_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int L = logical_id(blockIdx.x, a.G);
  const int s = L / (a.m_tiles * a.n_tiles);
  const int t = L - s * (a.m_tiles * a.n_tiles);
  const int mt = a.m_slow ? t / a.n_tiles : t % a.m_tiles;
  const int nt = a.m_slow ? t % a.n_tiles : t / a.m_tiles;
  const int n0 = nt * kBT;
  const int m0 = mt * kBT;
  const int k_begin = __builtin_amdgcn_readfirstlane(s * a.k_chunk);
  const int k_end = __builtin_amdgcn_readfirstlane(min(a.K, k_begin + a.k_chunk));
  const int n_chunks = max(0, (k_end - k_begin) / kBK);

  // loader: wave w fills rows 32w .. 32w+31 of both tiles, 8 rows (1 KB) per
  // instruction; lane L lands on row 32w + 8i + L/8 at physical chunk L%8 and
  // fetches logical chunk (L%8) ^ (row & 7)
  const uint16_t* wsrc[4];
  int64_t xsrc[4];
  int lchunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    lchunk[i] = 8 * ((lane & 7) ^ (row & 7));
    const int n = min(n0 + row, a.c_out - 1);
    wsrc[i] = a.w + static_cast<int64_t>(n) * a.K + lchunk[i];
    const uint32_t m = static_cast<uint32_t>(min(m0 + row, a.M - 1));
    const uint32_t wo = m % static_cast<uint32_t>(a.Wo);
    uint32_t r = m / static_cast<uint32_t>(a.Wo);
    const uint32_t ho = r % static_cast<uint32_t>(a.Ho);
    r /= static_cast<uint32_t>(a.Ho);
    const uint32_t to = r % static_cast<uint32_t>(a.To);
    const uint32_t b = r / static_cast<uint32_t>(a.To);
    xsrc[i] = (((static_cast<int64_t>(b) * a.T + to * a.kt) * a.H + ho * a.kh) * a.W + wo * a.kw) * a.c_in + lchunk[i];
  }
  auto seg_off = [&](int seg) -> int64_t {
    const int dw = seg % a.kw;
    const int dh = (seg / a.kw) % a.kh;
    const int dt = seg / (a.kw * a.kh);
    return ((static_cast<int64_t>(dt) * a.H + dh) * a.W + dw) * a.c_in;
  };
  // chunk cursor (wave-uniform): K element, channel within the segment, segment offset
  int cur_k = k_begin;
  int cur_seg = k_begin / a.c_in;
  int cur_ci = k_begin - cur_seg * a.c_in;
  int64_t cur_base = seg_off(cur_seg);
  auto issue = [&](int buf) {
    const int64_t xoff = cur_base + cur_ci;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row0 = 32 * wave + 8 * i;
      __builtin_amdgcn_global_load_lds(wsrc[i] + cur_k, (lds_void*)(sm.a[buf] + row0 * kBK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.x + xsrc[i] + xoff, (lds_void*)(sm.b[buf] + row0 * kBK), 16, 0, 0);
    }
    cur_k += kBK;
    cur_ci += kBK;
    if (cur_ci == a.c_in) {
      cur_ci = 0;
      ++cur_seg;
      cur_base = seg_off(cur_seg);
    }
  };

  // compute: wave (wn, wm) = (w & 1, w >> 1) owns channels 64wn.., positions 64wm..
  const int wn = wave & 1, wm = wave >> 1;
  int a_off[2][4], b_off[2][4];   // element offsets of the fragments in a tile, per (block, k-step)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ra = 64 * wn + 32 * i + l32;
      const int rb = 64 * wm + 32 * i + l32;
      a_off[i][ks] = ra * kBK + 8 * ((2 * ks + g) ^ (ra & 7));
      b_off[i][ks] = rb * kBK + 8 * ((2 * ks + g) ^ (rb & 7));
    }
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  if (n_chunks > 0) {
    issue(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      const int buf = c & 1;
      if (c + 1 < n_chunks) issue(buf ^ 1);
      const uint16_t* ta = sm.a[buf];
      const uint16_t* tb = sm.b[buf];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = *reinterpret_cast<const bf16x8*>(ta + a_off[i][ks]);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(tb + b_off[j][ks]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // stage the tile in LDS as fp32 [position][channel] (the operand tiles are
  // no longer read: every wave passed the last barrier), then write whole rows
  float* tile = reinterpret_cast<float*>(lds_raw);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 64 * wn + 32 * i + 8 * q + 4 * g;
        const int pl = 64 * wm + 32 * j + l32;
        *reinterpret_cast<float4*>(&tile[pl * kOutStride + nl]) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  __syncthreads();
  if (a.n_split == 1) {
    // 16 threads per position, 8 channels (16 bytes of bf16) each: 16 positions per pass
#pragma unroll
    for (int pass = 0; pass < kBT / 16; ++pass) {
      const int pl = 16 * pass + (tid >> 4);
      const int nl = 8 * (tid & 15);
      const int m = m0 + pl;
      const int n = n0 + nl;
      if (m >= a.M || n >= a.c_out) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = tile[pl * kOutStride + nl + e] + (a.bias != nullptr ? a.bias[n + e] : 0.f);
        if (a.act) v[e] = silu(v[e]);
      }
      uint4 pk;
      pk.x = pf::pack_bf16x2(v[0], v[1]);
      pk.y = pf::pack_bf16x2(v[2], v[3]);
      pk.z = pf::pack_bf16x2(v[4], v[5]);
      pk.w = pf::pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(a.y + static_cast<int64_t>(m) * a.c_out + n) = pk;
    }
  } else {
    // 32 threads per position, 4 channels (16 bytes of fp32) each: 8 positions per pass
#pragma unroll
    for (int pass = 0; pass < kBT / 8; ++pass) {
      const int pl = 8 * pass + (tid >> 5);
      const int nl = 4 * (tid & 31);
      const int m = m0 + pl;
      const int n = n0 + nl;
      if (m >= a.M || n >= a.c_out) continue;
      *reinterpret_cast<float4*>(a.part + (static_cast<int64_t>(s) * a.M + m) * a.c_out + n) =
          *reinterpret_cast<const float4*>(&tile[pl * kOutStride + nl]);
    }
  }
}

// Sum the K-split partials in split order, add the bias, apply SiLU, round.
__global__ __launch_bounds__(256) void hr_reduce_kernel(ConvArgs a) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // 4 channels each
  const int64_t total4 = static_cast<int64_t>(a.M) * a.c_out / 4;
  if (i4 >= total4) return;
  const int64_t e0 = 4 * i4;
  const int n = static_cast<int>(e0 % a.c_out);
  float4 sum = *reinterpret_cast<const float4*>(a.part + e0);
  for (int s = 1; s < a.n_split; ++s) {
    const float4 p =
        *reinterpret_cast<const float4*>(a.part + static_cast<int64_t>(s) * a.M * a.c_out + e0);
    sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w;
  }
  float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] += a.bias != nullptr ? a.bias[n + e] : 0.f;
    if (a.act) v[e] = silu(v[e]);
  }
  uint2 pk;
  pk.x = pf::pack_bf16x2(v[0], v[1]);
  pk.y = pf::pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(a.y + e0) = pk;
}

struct ConvPlan {
  int64_t M = 0;
  int To = 0, Ho = 0, Wo = 0, K = 0;
  int ni = 2, nj = 2;   // wave tile: 32 ni channels x 32 nj positions
  bool lds = false;     // workgroup-tiled kernel (C_in a multiple of 64)
  int m_tiles = 0, n_tiles = 0, n_split = 1, k_chunk = 0, G = 0;
  size_t ws_bytes = 0;
};

// CUs of the current device, looked up once per device
int multiprocessors() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

ConvPlan make_conv_plan(int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw, int c_out) {
  ConvPlan p;
  p.To = T / kt;
  p.Ho = H / kh;
  p.Wo = W / kw;
  p.M = static_cast<int64_t>(n_batch) * p.To * p.Ho * p.Wo;
  p.K = kt * kh * kw * c_in;
  const int64_t target = static_cast<int64_t>(kTargetWaves) * multiprocessors() / 256;
  const double reads = 2.0 * (static_cast<double>(c_out) * p.K + static_cast<double>(p.M) * p.K);
  const double part_per_split = 4.0 * static_cast<double>(p.M) * c_out;
  int64_t tiles = 0;
  int split = 1;
  p.lds = c_in % kBK == 0;
  if (p.lds) {
    // 128 x 128 workgroup tiles (4 waves), K in chunks of 64
    p.m_tiles = static_cast<int>((p.M + kBT - 1) / kBT);
    p.n_tiles = (c_out + kBT - 1) / kBT;
    tiles = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
    const int chunks = p.K / kBK;
    while (split < kMaxSplit && 4 * tiles * split * 2 <= target && chunks / (split * 2) >= 4 &&
           part_per_split * split * 2 <= kPartialBudget * reads)
      split *= 2;
    p.k_chunk = ((chunks + split - 1) / split) * kBK;
  } else {
    // 64 x 64 wave tiles (each fragment feeds two MFMAs) unless the reduction
    // is only a few steps deep; then the operand reuse is worth less than more waves
    p.ni = p.nj = (p.K / 16 <= 4) ? 1 : 2;
    p.m_tiles = static_cast<int>((p.M + 32 * p.nj - 1) / (32 * p.nj));
    p.n_tiles = (c_out + 32 * p.ni - 1) / (32 * p.ni);
    tiles = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
    const int steps = p.K / 16;
    // split K while the grid holds fewer waves than the target, every split
    // keeps at least 2 * kDepth steps of 16 and the partials stay in budget
    while (split < kMaxSplit && tiles * split * 2 <= target && steps / (split * 2) >= 2 * kDepth &&
           part_per_split * split * 2 <= kPartialBudget * reads)
      split *= 2;
    p.k_chunk = ((steps + split - 1) / split) * 16;
  }
  p.n_split = (p.K + p.k_chunk - 1) / p.k_chunk;
  p.G = static_cast<int>(tiles * p.n_split);
  p.ws_bytes = p.n_split > 1 ? static_cast<size_t>(p.n_split) * p.M * c_out * sizeof(float) : 0;
  return p;
}

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

pf_status check_conv(const pf_bf16* x, int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw,
                     const pf_bf16* w, const float* bias, int c_out, const pf_bf16* y) {
  PF_REQUIRE_PTR(x);
  PF_REQUIRE_PTR(w);
  PF_REQUIRE_PTR(y);
  PF_REQUIRE_ALIGNED(x);
  PF_REQUIRE_ALIGNED(w);
  PF_REQUIRE_ALIGNED(y);
  PF_REQUIRE((reinterpret_cast<uintptr_t>(bias) & 3u) == 0, PF_ERR_MISALIGNED, "bias is not 4-byte aligned");
  PF_REQUIRE(n_batch >= 1, PF_ERR_SHAPE, "n_batch must be >= 1");
  PF_REQUIRE(kt >= 1 && kh >= 1 && kw >= 1 && kt * kh * kw <= 64, PF_ERR_UNSUPPORTED,
             "kernel %dx%dx%d: each side >= 1, at most 64 taps", kt, kh, kw);
  PF_REQUIRE(T >= kt && H >= kh && W >= kw, PF_ERR_SHAPE,
             "input %dx%dx%d is smaller than the kernel %dx%dx%d", T, H, W, kt, kh, kw);
  PF_REQUIRE(c_in >= 16 && c_in % 16 == 0 && c_in <= 65536, PF_ERR_UNSUPPORTED,
             "c_in must be a multiple of 16 in [16, 65536] (got %d)", c_in);
  PF_REQUIRE(c_out >= 16 && c_out % 16 == 0 && c_out <= 65536, PF_ERR_UNSUPPORTED,
             "c_out must be a multiple of 16 in [16, 65536] (got %d)", c_out);
  const int64_t M = static_cast<int64_t>(n_batch) * (T / kt) * (H / kh) * (W / kw);
  PF_REQUIRE(static_cast<int64_t>(n_batch) * T * H * W * c_in < (int64_t{1} << 40), PF_ERR_UNSUPPORTED,
             "input too large");
  PF_REQUIRE(M < (int64_t{1} << 31) - 64 && (M + 31) / 32 * ((c_out + 31) / 32) * kMaxSplit < 0x7FFFFFFF,
             PF_ERR_UNSUPPORTED, "too many output positions");
  return PF_OK;
}

pf_status launch_conv(const pf_bf16* x, int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw,
                      const pf_bf16* w, const float* bias, int c_out, int act, pf_bf16* y, void* workspace,
                      size_t workspace_bytes, hipStream_t st, const char* what) {
  const ConvPlan p = make_conv_plan(n_batch, T, H, W, c_in, kt, kh, kw, c_out);
  if (p.ws_bytes > 0) {
    PF_REQUIRE(workspace != nullptr, PF_ERR_WORKSPACE, "%s: workspace is NULL (need %zu bytes)", what, p.ws_bytes);
    PF_REQUIRE(workspace_bytes >= p.ws_bytes, PF_ERR_WORKSPACE, "%s: workspace has %zu bytes, need %zu", what,
               workspace_bytes, p.ws_bytes);
    PF_REQUIRE_ALIGNED(workspace);
  }
  ConvArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.w = reinterpret_cast<const uint16_t*>(w);
  a.bias = bias;
  a.y = reinterpret_cast<uint16_t*>(y);
  a.part = static_cast<float*>(workspace);
  a.M = static_cast<int32_t>(p.M);
  a.T = T; a.H = H; a.W = W; a.c_in = c_in;
  a.kt = kt; a.kh = kh; a.kw = kw;
  a.To = p.To; a.Ho = p.Ho; a.Wo = p.Wo;
  a.c_out = c_out;
  a.K = p.K;
  a.act = act ? 1 : 0;
  a.m_tiles = p.m_tiles;
  a.n_tiles = p.n_tiles;
  a.n_split = p.n_split;
  a.k_chunk = p.k_chunk;
  a.G = p.G;
  // activations (positions x K) against weights (channels x K)
  a.m_slow = p.M > c_out ? 1 : 0;
  if (p.lds)
    hipLaunchKernelGGL(hr_conv_lds_kernel, dim3(p.G), dim3(256), 0, st, a);
  else if (p.ni == 2 && p.nj == 2)
    hipLaunchKernelGGL((hr_conv_kernel<2, 2>), dim3(p.G), dim3(64), 0, st, a);
  else if (p.ni == 2)
    hipLaunchKernelGGL((hr_conv_kernel<2, 1>), dim3(p.G), dim3(64), 0, st, a);
  else if (p.nj == 2)
    hipLaunchKernelGGL((hr_conv_kernel<1, 2>), dim3(p.G), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((hr_conv_kernel<1, 1>), dim3(p.G), dim3(64), 0, st, a);
  pf_status s = pf::launch_status(what);
  if (s != PF_OK || p.n_split == 1) return s;
  const int64_t total4 = p.M * c_out / 4;
  hipLaunchKernelGGL(hr_reduce_kernel, dim3(static_cast<unsigned>((total4 + 255) / 256)), dim3(256), 0, st, a);
  return pf::launch_status(what);
}

// intermediate activations of the branch: two ping-pong buffers, then the
// split-K partials of the largest stage
struct BranchPlan {
  size_t act_bytes = 0, part_bytes = 0, ws_bytes = 0;
};

BranchPlan make_branch_plan(int n_batch, int T, int H, int W, int c_in, const int* widths, int hidden) {
  BranchPlan bp;
  int t = T, h = H, w = W, c = c_in;
  for (int s = 0; s < PF_HR_STAGES; ++s) {
    const int kt = s == 0 ? 2 : 1, k = s == 0 ? 1 : 2;
    const ConvPlan p = make_conv_plan(n_batch, t, h, w, c, kt, k, k, widths[s]);
    t /= kt; h /= k; w /= k;
    bp.act_bytes = std::max(bp.act_bytes, round_up(static_cast<size_t>(p.M) * widths[s] * 2));
    bp.part_bytes = std::max(bp.part_bytes, round_up(p.ws_bytes));
    c = widths[s];
  }
  const ConvPlan p = make_conv_plan(n_batch, t, h, w, c, 1, 1, 1, hidden);
  bp.part_bytes = std::max(bp.part_bytes, round_up(p.ws_bytes));
  bp.ws_bytes = 2 * bp.act_bytes + bp.part_bytes;
  return bp;
}

}  // namespace

extern "C" size_t pf_hr_conv_workspace_bytes(int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw,
                                             int c_out) {
  if (n_batch < 1 || kt < 1 || kh < 1 || kw < 1 || T < kt || H < kh || W < kw || c_in < 16 || c_out < 16) return 0;
  return make_conv_plan(n_batch, T, H, W, c_in, kt, kh, kw, c_out).ws_bytes;
}

extern "C" pf_status pf_hr_conv(const pf_bf16* x, int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw,
                                const pf_bf16* w, const float* bias, int c_out, int act, pf_bf16* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const pf_status v = check_conv(x, n_batch, T, H, W, c_in, kt, kh, kw, w, bias, c_out, y);
  if (v != PF_OK) return v;
  return launch_conv(x, n_batch, T, H, W, c_in, kt, kh, kw, w, bias, c_out, act, y, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream), "pf_hr_conv");
}

extern "C" size_t pf_hr_branch_workspace_bytes(int n_batch, int T, int H, int W, int c_in, const int* widths,
                                               int hidden) {
  if (widths == nullptr || n_batch < 1 || T < 2 || H < 8 || W < 8 || c_in < 16 || hidden < 16) return 0;
  for (int s = 0; s < PF_HR_STAGES; ++s)
    if (widths[s] < 16) return 0;
  return make_branch_plan(n_batch, T, H, W, c_in, widths, hidden).ws_bytes;
}

extern "C" int64_t pf_hr_branch_out_tokens(int T, int H, int W) {
  if (T < 2 || H < 8 || W < 8) return 0;
  int t = T, h = H, w = W;
  for (int s = 0; s < PF_HR_STAGES; ++s) {
    const int kt = s == 0 ? 2 : 1, k = s == 0 ? 1 : 2;
    t /= kt; h /= k; w /= k;
  }
  return static_cast<int64_t>(t) * h * w;
}

extern "C" pf_status pf_hr_branch(const pf_bf16* z, int n_batch, int T, int H, int W, int c_in,
                                  const pf_bf16* const* stage_w, const float* const* stage_b, const int* widths,
                                  const pf_bf16* proj_w, const float* proj_b, int hidden, pf_bf16* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  PF_REQUIRE_PTR(stage_w);
  PF_REQUIRE_PTR(stage_b);
  PF_REQUIRE_PTR(widths);
  PF_REQUIRE(T >= 2 && H >= 8 && W >= 8, PF_ERR_SHAPE,
             "the latent block must be at least 2 x 8 x 8 (got %d x %d x %d)", T, H, W);
  // validate every stage before anything is enqueued
  {
    int t = T, h = H, w = W, c = c_in;
    for (int s = 0; s < PF_HR_STAGES; ++s) {
      const int kt = s == 0 ? 2 : 1, k = s == 0 ? 1 : 2;
      const pf_status v = check_conv(z, n_batch, t, h, w, c, kt, k, k, stage_w[s], stage_b[s], widths[s], out);
      if (v != PF_OK) return v;
      t /= kt; h /= k; w /= k;
      c = widths[s];
    }
    const pf_status v = check_conv(z, n_batch, t, h, w, c, 1, 1, 1, proj_w, proj_b, hidden, out);
    if (v != PF_OK) return v;
  }
  const BranchPlan bp = make_branch_plan(n_batch, T, H, W, c_in, widths, hidden);
  PF_REQUIRE(workspace != nullptr, PF_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", bp.ws_bytes);
  PF_REQUIRE(workspace_bytes >= bp.ws_bytes, PF_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes,
             bp.ws_bytes);
  PF_REQUIRE_ALIGNED(workspace);

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  pf_bf16* act[2] = {reinterpret_cast<pf_bf16*>(ws), reinterpret_cast<pf_bf16*>(ws + bp.act_bytes)};
  void* part = ws + 2 * bp.act_bytes;
  const pf_bf16* x = z;
  int t = T, h = H, w = W, c = c_in;
  for (int s = 0; s < PF_HR_STAGES; ++s) {
    const int kt = s == 0 ? 2 : 1, k = s == 0 ? 1 : 2;
    const pf_status r = launch_conv(x, n_batch, t, h, w, c, kt, k, k, stage_w[s], stage_b[s], widths[s], 1,
                                    act[s & 1], part, bp.part_bytes, st, "pf_hr_branch");
    if (r != PF_OK) return r;
    x = act[s & 1];
    t /= kt; h /= k; w /= k;
    c = widths[s];
  }
  return launch_conv(x, n_batch, t, h, w, c, 1, 1, 1, proj_w, proj_b, hidden, 0, out, part, bp.part_bytes, st,
                     "pf_hr_branch");
}
