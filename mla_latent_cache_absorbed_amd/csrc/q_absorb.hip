// q_absorb.hip -- query absorption: q_abs[r, i, :] = W_UK[i]^T q[r, i, :].
//
// Moves the key up-projection from every cached token onto the one new
// query (the bilinear identity a^T M b = (M^T a)^T b, "Mathematical
// Prerequisites for DeepSeek-V2" section 6; the absorbed query of "MLA, dim
// by dim" section 5.1 and the q^A of "From Vanilla Transformers to Modern
// LLMs ... Part 3" section 3.e.2).  Cost per query row: 2 h d_h d_c FLOPs,
// independent of the context length.
//
// Fast path (bf16, d_h = 128): one work-group per (head, 64 latent columns).
// W_UK[i] streams from HBM once (16 KB per group); it is the dominant cost
// for small batches, so the kernel is built around one coalesced pass over
// the weight.  The contraction runs on 16x16x32 bf16 MFMA with the latent
// column as M, the query row as N and d_h as K.  W_UK is stored
// [h][d_h][d_c] (column index fastest), so the K-contiguous operand the
// MFMA wants is W^T; the tile is transposed once through LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDh = 128;          // d_h of the fast path (MFMA K)
constexpr int kCols = 64;         // latent columns per work-group
constexpr int kWtStride = kDh + 8;  // LDS row stride (elements) of W^T tile

__global__ __launch_bounds__(256) void q_absorb_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_abs, int rows, int h, int d_c) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kCols * kWtStride];

  const int head = blockIdx.x;
  const int c0 = blockIdx.y * kCols;
  const int tid = threadIdx.x;

  // Stage W_UK[head][:, c0:c0+64] as W^T (column-major for the MFMA).
  // Chunk ch covers 8 consecutive columns of one row k: 8 threads read one
  // 128-byte row segment, so each wave touches 8 full cache lines.
  const uint16_t* wsrc = w_uk + (size_t)head * kDh * d_c + c0;
#pragma unroll
  for (int j = 0; j < (kDh * kCols / 8) / 256; ++j) {
    const int ch = tid + 256 * j;
    const int k = ch >> 3, cc = ch & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(wsrc + (size_t)k * d_c + 8 * cc);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t x = static_cast<uint16_t>(w4[e >> 1] >> (16 * (e & 1)));
      wt[(8 * cc + e) * kWtStride + k] = x;
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int col = 16 * wave + l16;  // this lane's M row (latent column)

  bf16x8 a[kDh / 32];
#pragma unroll
  for (int s = 0; s < kDh / 32; ++s)
    a[s] = as_bf16x8(*reinterpret_cast<const uint4*>(&wt[col * kWtStride + 32 * s + 8 * g]));

  for (int rb = 0; rb < rows; rb += 16) {
    const int r = rb + l16;  // this lane's N column (query row)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* qrow = q + ((size_t)r * h + head) * kDh;
#pragma unroll
    for (int s = 0; s < kDh / 32; ++s) {
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (r < rows) bv = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g);
      acc = mfma16x16x32(a[s], as_bf16x8(bv), acc);
    }
    if (r < rows) {
      // D[4g + j][l16] = q_abs[r][head][c0 + 16 wave + 4g + j]
      uint2 packed;
      packed.x = pack_bf16x2(acc[0], acc[1]);
      packed.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(q_abs + ((size_t)r * h + head) * d_c + c0 + 16 * wave + 4 * g) = packed;
    }
  }
}

}  // namespace

hipError_t launch_q_absorb_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  dim3 grid(a.h, a.d_c / kCols);
  launch_kernel(q_absorb_bf16_kernel, grid, dim3(256), s,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.w_uk),
                     static_cast<uint16_t*>(a.q_abs), rows, a.h, a.d_c);
  return hipGetLastError();
}

}  // namespace mla
