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

template <typename Fn>
__device__ __forceinline__ int Lens::sum(Fn fn, int lane) const {
  int acc = lane < batch ? fn(mine) : 0;
  for (int b = lane + 64; b < batch; b += 64) acc += fn(seq_len(lens, b, max_len));
  return wave_sum(acc);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

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
    const int incl = wave_scan(n, lane);
    const int start = first + incl - n;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(b < L.batch && g >= start && g < start + n);
    if (hit != 0) {
      const int src = __builtin_ctzll(hit);
      b_out = b0 + src;
      j_out = g - __shfl(start, src, 64);
      return;
    }
    first += __shfl(incl, 63, 64);
  }
}

}  // namespace chunks
}  // namespace mla
