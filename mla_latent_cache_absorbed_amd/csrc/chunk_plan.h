// chunk_plan.h -- how the context of every sequence of a call is cut into
// chunks (fast path), computed on the device from the context lengths so
// that ragged batches get chunks of one common length: a long sequence gets
// more chunks, a short one fewer, and every work-group streams about the
// same number of tiles.
//
// Chunks are numbered globally: sequence b owns chunks first_b .. first_b +
// n_b - 1 with n_b = ceil(L_b / C) (L_b clamped to [0, max_len]) and first_b
// the prefix sum of n over the sequences before b.  The split kernel's
// work-group for chunk g finds its sequence by a scan; the finish kernel
// finds the chunks of its rows the same way.  Every wave computes the same
// wave-uniform result from the same loads, so no LDS exchange is needed.
#pragma once

#include "common.h"

namespace mla {
namespace chunks {

constexpr int kAlign = 32;  // tokens: chunks are whole tiles

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int max_len) {
  return clamp_len(lens[b], max_len);
}

// The clamped context lengths, read once: lane l keeps that of sequence l;
// sequences from 64 on (a rare batch size) are read again where needed.
struct Lens {
  const int32_t* lens;
  int batch, max_len, mine;
  __device__ __forceinline__ Lens(const int32_t* p, int batch_, int max_len_, int lane)
      : lens(p), batch(batch_), max_len(max_len_), mine(lane < batch_ ? seq_len(p, lane, max_len_) : 0) {}
  // with context_lens[lane] already loaded (unclamped)
  __device__ __forceinline__ Lens(const int32_t* p, int batch_, int max_len_, int lane, int raw)
      : lens(p), batch(batch_), max_len(max_len_), mine(lane < batch_ ? clamp_len(raw, max_len_) : 0) {}
  // Sum over the sequences of fn(length): lane l takes sequences l, l + 64,
  // ... (the first from the register), then the wave adds up.
  template <typename Fn>
  __device__ __forceinline__ int sum(Fn fn, int lane) const;
};

__device__ __forceinline__ int wave_sum(int v);
__device__ __forceinline__ int wave_max(int v);

template <typename Fn>
__device__ __forceinline__ int Lens::sum(Fn fn, int lane) const {
  int acc = lane < batch ? fn(mine) : 0;
  for (int b = lane + 64; b < batch; b += 64) acc += fn(seq_len(lens, b, max_len));
  return wave_sum(acc);
}

// Cross-lane steps on the VALU (DPP and the gfx950 permlane swaps), not
// through LDS: a plan is a chain of a few dozen of them.
//   dpp_perm: lane l receives v from the lane that the DPP control selects
//   (all sources valid for the controls used here).
template <int kCtrl>
__device__ __forceinline__ int dpp_perm(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
//   dpp_shift: the same with lanes whose source is outside the row (or
//   whose row the mask leaves out) receiving 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_shift(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xF, false);
}

// op over the 64 lanes, in every lane: lane pairs l ^ 1, l ^ 2 (quad
// permutations), the two quads of each 8 (row half mirror), the two 8s of
// each row of 16 (row mirror), then rows l ^ 16 and l ^ 32 (permlane swaps).
template <typename Op>
__device__ __forceinline__ int wave_reduce(int v, Op op) {
  v = op(v, dpp_perm<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_perm<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_perm<0x141>(v));  // row_half_mirror
  v = op(v, dpp_perm<0x140>(v));  // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = op((int)a[0], (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return op((int)c[0], (int)c[1]);
}

__device__ __forceinline__ int wave_sum(int v) {
  return wave_reduce(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ int wave_max(int v) {
  return wave_reduce(v, [](int x, int y) { return x > y ? x : y; });
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each
// row of 16, then the last lane of row 0 (2) into row 1 (3), and lane 31
// into rows 2 and 3.
__device__ __forceinline__ int wave_scan(int v) {
  v += dpp_shift<0x111, 0xF>(v);  // row_shr:1
  v += dpp_shift<0x112, 0xF>(v);  // row_shr:2
  v += dpp_shift<0x114, 0xF>(v);  // row_shr:4
  v += dpp_shift<0x118, 0xF>(v);  // row_shr:8
  v += dpp_shift<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_shift<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Value of v in lane `src` (uniform), in every lane.
__device__ __forceinline__ int lane_int(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Chunks of all sequences for chunk length c (wave-uniform).
__device__ __forceinline__ int count_chunks(const Lens& L, int c, int lane) {
  return L.sum([c](int len) { return ceil_div(len, c); }, lane);
}

// The chunk length of the call: about the shortest whole-tile length in
// [min_len, max_chunk] whose chunk count stays within target, found by
// correcting the evenly divided length for the rounding of each sequence up
// to whole chunks; target > batch guarantees the last try.
__device__ __forceinline__ int chunk_len(const Lens& L, int target, int min_len, int max_chunk, int lane) {
  const int batch = L.batch;
  const int total = L.sum([](int len) { return len; }, lane);
  auto len_for = [&](int parts) {
    int c = ceil_div(ceil_div(total, parts > 0 ? parts : 1), kAlign) * kAlign;
    return c < min_len ? min_len : (c > max_chunk ? max_chunk : c);
  };
  int parts = target;
  for (int k = 0; k < 3; ++k) {
    const int c = len_for(parts);
    const int n = count_chunks(L, c, lane);
    if (n <= target || c == max_chunk) return c;
    parts -= n - target;  // the chunks that rounding added
    if (parts < 1) break;
  }
  // n_b <= L_b / c + 1 for every b, so n <= total / c + batch <= target
  return len_for(target - batch);
}

// Sequence and chunk-within-sequence of global chunk g, or b = -1 when the
// call has fewer chunks.
__device__ __forceinline__ void locate(const Lens& L, int c, int g, int lane, int& b_out, int& j_out) {
  b_out = -1;
  j_out = 0;
  int first = 0;
  for (int b0 = 0; b0 < L.batch; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < L.batch ? ceil_div(b0 == 0 ? L.mine : seq_len(L.lens, b, L.max_len), c) : 0;
    const int incl = wave_scan(n);
    const int start = first + incl - n;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(b < L.batch && g >= start && g < start + n);
    if (hit != 0) {
      const int src = __builtin_ctzll(hit);
      b_out = b0 + src;
      j_out = g - lane_int(start, src);
      return;
    }
    first += lane_int(incl, 63);
  }
}

}  // namespace chunks
}  // namespace mla
