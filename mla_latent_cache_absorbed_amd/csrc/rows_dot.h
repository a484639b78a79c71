// rows_dot.h -- the few-row form of the skinny products x W^T used after
// and before the decode step (oproj.hip: the output projection and the
// query latent; rope_proj.hip: the stages with RoPE).
//
// With one or a few rows of x the product is a stream of W and nothing
// else.  The MFMA kernel of oproj.hip then needs slices of k to fill the
// compute units, and with them fp32 partial sums and a second launch that
// adds them up.  Here each wave takes two adjacent output features over
// the whole of k, so a single launch leaves finished sums and the caller's
// epilogue (bf16 rounding, RoPE, a paged destination) runs in the same
// kernel.  The compute units fill because the wave count is half the
// feature count (2560 waves for W^O at DeepSeek-V2 width).
//
// With one or two rows, every wave reads x from L2 beside its weights.
// Three or four rows of x, read that way, are 1.5-2 times the weight
// bytes (the query side's second stage ran slower than on the MFMA
// kernel), so then a work-group (four waves, eight features) first copies
// x into LDS, when it fits in kRowsDotMaxLdsBytes, and x leaves L2 once
// per work-group; its first weight loads are issued before that copy.
// Larger x takes the MFMA kernel.  (The LDS copy is no gain with one or
// two rows: for W^O at one row the copy and its barrier before the weight
// stream made the product 8 % slower than reading x from L2.)
//
// Lane l covers k positions 512 s + 8 l .. + 7 of step s: one 16-byte load
// per feature row each step, so every load instruction of a wave reads
// 1 KB of contiguous memory, and one 16-byte read per row of x.  The
// products run on v_dot2_f32_bf16, which adds two bf16 products (exact in
// fp32) to an fp32 accumulator: four per 16-byte pair.  The 64 lanes' sums
// then meet in a fixed xor butterfly, so the result does not depend on
// timing.  Each step's global loads are issued kDepth steps (4 or 8) before
// its products.
#pragma once

#include "common.h"

namespace mla {

// Rows up to which the one-launch form runs; more rows take the MFMA kernel
// with slices of k.
constexpr int kRowsDotMaxRows = 4;
// k must be a multiple of this (one step of the 64 lanes, 8 values each).
constexpr int kRowsDotK = 512;
constexpr int kRowsDotWaves = 4;     // waves per work-group
constexpr int kRowsDotFeatures = 2;  // adjacent output features per wave
constexpr int kRowsDotPerGroup = kRowsDotWaves * kRowsDotFeatures;
// Steps of global loads in flight per wave: 4, or 8 for one row of x with
// k >= 8192 (W^O at one row: 35.3 -> 33.9 us; with two rows, or with
// fewer steps than 16, the deeper ring measured slower: its registers
// cost waves, its first loads re-read the last step when k is short).
constexpr int kRowsDotDepth = 4;
constexpr int kRowsDotDeepDepth = 8;
__host__ __device__ inline bool rows_dot_deep(int rows, int k) { return rows == 1 && k >= 16 * kRowsDotK; }
// Waves that share one feature pair, each taking every kSplit-th step of
// k: 4 (the whole work-group) when the features are few (n < 1024: the
// cache append's 576), so that a wave's chain of dependent loads is a
// quarter as long; else 1.  The partial sums meet in LDS in wave order.
// (Cache append at 2 and 4 rows: 10.6 -> 9.6 and 12.0 -> 10.9 us; the
// query latent's 1536 features measured 0.5 us slower split.)
__host__ __device__ inline int rows_dot_split(int n, int k) {
  return n < 1024 && k / kRowsDotK >= kRowsDotWaves ? kRowsDotWaves : 1;
}
// Largest x a work-group holds in LDS (rows * k bf16 values): four
// work-groups per CU.
constexpr size_t kRowsDotMaxLdsBytes = 40 * 1024;
// Rows up to which every wave reads x from L2.
constexpr int kRowsDotMaxL2Rows = 2;

// Whether x [rows][k] goes through LDS.
__host__ __device__ inline bool rows_dot_x_in_lds(int rows, int k) {
  return rows > kRowsDotMaxL2Rows && (size_t)rows * k * 2 <= kRowsDotMaxLdsBytes;
}
// Whether the one-launch form takes rows x [rows][k] against n output
// features (bf16 storage assumed).
__host__ __device__ inline bool rows_dot_applies(int rows, int k, int n) {
  return rows >= 1 && rows <= kRowsDotMaxRows && k % kRowsDotK == 0 && n % kRowsDotPerGroup == 0 &&
         (rows_dot_x_in_lds(rows, k) || rows <= kRowsDotMaxL2Rows);
}
// LDS bytes of a work-group.
inline size_t rows_dot_lds_bytes(int rows, int k) { return rows_dot_x_in_lds(rows, k) ? (size_t)rows * k * 2 : 0; }

// Eight bf16 products of a and b added to c.  Each element is copied out
// of its vector before the bit cast: a bit cast of the subscript
// expression itself compiles to element 0 every time.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float c) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t aq = a[q], bq = b[q];
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aq), __builtin_bit_cast(bf16x2, bq), c, false);
  }
  return c;
}

// out[f][r] = sum over k of wf[k] x[r][k] for the two feature rows w0, w1
// (k contiguous values each) and the rows r < kR of x ([rows][k]); every
// lane receives every sum.  A row r >= rows reads row 0 instead and its
// sums are to be dropped.  kDepth: kRowsDotDeepDepth when rows_dot_deep
// (and kSplit is 1), else kRowsDotDepth.  kSplit = rows_dot_split(n, k):
// the waves w with the same w / kSplit share w0, w1, wave w taking the
// steps w % kSplit, w % kSplit + kSplit, ...; the return value says
// whether this wave holds the finished sums (one wave per pair).  kLds
// (= rows_dot_x_in_lds(rows, k)) or kSplit > 1: called by all threads of
// the work-group (kRowsDotWaves waves), with xs the work-group's LDS of
// rows_dot_lds_bytes(rows, k) bytes for kLds; one barrier for each.
// Otherwise xs is unused and the waves run independently.  pre() runs once
// the first steps' loads are out (work of the caller's epilogue that does
// not depend on the sums).
template <int kR, bool kLds, int kDepth, int kSplit, typename Pre>
__device__ __forceinline__ bool rows_dot(const uint16_t* x, int rows, int k, const uint16_t* w0, const uint16_t* w1,
                                         uint16_t* xs, float (&out)[kRowsDotFeatures][kR], Pre pre) {
  static_assert(kSplit == 1 || kSplit == kRowsDotWaves, "a feature pair takes one wave or the whole work-group");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % kSplit;
  const int steps = (k / kRowsDotK - part + kSplit - 1) / kSplit;  // this wave's steps (>= 1)
  constexpr size_t kStride = (size_t)kRowsDotK * kSplit;           // elements between them
  const int e0 = kRowsDotK * part + 8 * lane;
  const uint16_t* wp[kRowsDotFeatures] = {w0 + e0, w1 + e0};
  const uint16_t* xg[kR];  // x rows in global memory (not kLds)
#pragma unroll
  for (int r = 0; r < kR; ++r) xg[r] = x + (size_t)(r < rows ? r : 0) * k + e0;

  u32x4 wv[kDepth][kRowsDotFeatures];
  u32x4 xv[kLds ? 1 : kDepth][kR];
  auto load = [&](int slot, int s) {
#pragma unroll
    for (int f = 0; f < kRowsDotFeatures; ++f)
      wv[slot][f] = *reinterpret_cast<const u32x4*>(wp[f] + kStride * s);
    if constexpr (!kLds) {
#pragma unroll
      for (int r = 0; r < kR; ++r) xv[slot][r] = *reinterpret_cast<const u32x4*>(xg[r] + kStride * s);
    }
  };
  // the first steps' loads go out before the copy of x (a step past the
  // end re-reads the last one: the loads stay unconditional)
#pragma unroll
  for (int u = 0; u < kDepth; ++u) load(u, u < steps ? u : steps - 1);
  pre();  // the caller's work that does not need the sums, under those loads

  const uint16_t* xr[kR];  // x rows in LDS (kLds)
  if constexpr (kLds) {
    const int pieces = rows * k / 8;  // 16-byte pieces of x
    for (int i = threadIdx.x; i < pieces; i += kRowsDotWaves * 64)
      *reinterpret_cast<u32x4*>(xs + 8 * i) = *reinterpret_cast<const u32x4*>(x + 8 * (size_t)i);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kR; ++r) xr[r] = xs + (r < rows ? r : 0) * k + e0;
  }

  float acc[kRowsDotFeatures][kR];
#pragma unroll
  for (int f = 0; f < kRowsDotFeatures; ++f)
#pragma unroll
    for (int r = 0; r < kR; ++r) acc[f][r] = 0.f;
  auto dot = [&](int slot, int s) {
    u32x4 xs_v[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      if constexpr (kLds)
        xs_v[r] = *reinterpret_cast<const u32x4*>(xr[r] + kStride * s);
      else
        xs_v[r] = xv[slot][r];
    }
#pragma unroll
    for (int f = 0; f < kRowsDotFeatures; ++f)
#pragma unroll
      for (int r = 0; r < kR; ++r) acc[f][r] = dot8_bf16(wv[slot][f], xs_v[r], acc[f][r]);
  };
  // every round but the last has all its steps; the last has 1 .. depth
  const int last = (steps - 1) / kDepth * kDepth;
  for (int s = 0; s < last; s += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      dot(u, s + u);
      const int next = s + u + kDepth;
      load(u, next < steps ? next : steps - 1);  // unconditional: the compiler's waits stay exact
      // keep each slot's refill right behind its products (the scheduler
      // would sink all refills to the end of the round, so that a wave
      // waited out a whole load latency in every round)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < kDepth; ++u)
    if (last + u < steps) dot(u, last + u);

#pragma unroll
  for (int f = 0; f < kRowsDotFeatures; ++f)
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float v = acc[f][r];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v = xor_sum(v, m);
      out[f][r] = v;
    }
  if constexpr (kSplit > 1) {
    __shared__ float red[kRowsDotWaves][kRowsDotFeatures][kR];
    if (lane == 0) {
#pragma unroll
      for (int f = 0; f < kRowsDotFeatures; ++f)
#pragma unroll
        for (int r = 0; r < kR; ++r) red[wave][f][r] = out[f][r];
    }
    __syncthreads();
    if (part != 0) return false;
#pragma unroll
    for (int f = 0; f < kRowsDotFeatures; ++f)
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float v = red[wave][f][r];
#pragma unroll
        for (int j = 1; j < kSplit; ++j) v += red[wave + j][f][r];
        out[f][r] = v;
      }
  }
  return true;
}

// The sums of row `lane` (lanes 0 .. kR - 1), for the lane that stores it.
template <int kR>
__device__ __forceinline__ void rows_dot_pick(const float (&s)[kRowsDotFeatures][kR], int lane, float& v0,
                                              float& v1) {
  v0 = s[0][0];
  v1 = s[1][0];
#pragma unroll
  for (int r = 1; r < kR; ++r)
    if (lane == r) {
      v0 = s[0][r];
      v1 = s[1][r];
    }
}

}  // namespace mla
