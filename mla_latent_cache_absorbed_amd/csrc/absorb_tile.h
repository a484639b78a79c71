// absorb_tile.h -- query absorption on one 128 x 128 slice of W_UK[i]:
//   q_abs[r, i, c0 : c0 + 128] = W_UK[i][:, c0 : c0 + 128]^T q[r, i, :]
// for every query row r (the bilinear identity a^T M b = (M^T a)^T b moves
// the key up-projection from every cached token onto the one query,
// "Mathematical Prerequisites for DeepSeek-V2" section 6; the absorbed
// query of "MLA, dim by dim" section 5.1 and the q^A of "From Vanilla
// Transformers to Modern LLMs ... Part 3" section 3.e.2).  Fast path only:
// bf16, d_h = 128.
//
// Four waves handle one slice.  The slice (32 KB) comes into LDS by direct
// global->LDS DMA in its stored [d_h][d_c] order, so W_UK streams from HBM
// exactly once; the contraction runs on 16x16x32 bf16 MFMA with the latent
// column as M, the query row as N and d_h as K.  The K-contiguous A operand
// the MFMA wants is W^T; the transposing LDS read ds_read_b64_tr_b16
// produces it from the row-major tile (within 16 lanes, lane i receives
// element i & 3 of the 8-byte chunk addressed by lane 4e + (i >> 2), for
// e = 0..3).
#pragma once

#include "common.h"

namespace mla {
namespace absorb {

constexpr int kDh = 128;              // d_h (MFMA K)
constexpr int kCols = 128;            // latent columns per slice
constexpr int kRowBytes = kCols * 2;  // 256 B of one W row in the tile
constexpr int kTileBytes = kDh * kRowBytes;  // 32 KB

// XOR on the 16-byte chunk index (0..15) of tile row k.  The transposing
// reads of one 32-lane half touch 8 rows (k = 0-3 and 8-11 of its 32-row
// slab) at the same two adjacent chunks; this sends them to 8 distinct
// chunk pairs, i.e. to all 64 banks.
__device__ __forceinline__ int w_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// Wave wt (0..3) of the four copies rows 32 wt .. 32 wt + 31 of
// W_UK[i][:, c0 : c0 + 128] (w_head = W_UK[i], row-major [d_h][d_c]) into
// the tile at LDS address tile_lds: eight DMAs of four 256-byte rows.
__device__ __forceinline__ void load_tile(uint32_t tile_lds, const uint16_t* w_head, int c0, int d_c,
                                          int wt, int lane) {
  const int rsub = lane >> 4, l16 = lane & 15;  // row within the DMA, chunk
  const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(w_head + c0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k0 = 32 * wt + 4 * j;
    const int k = k0 + rsub;
    const uint32_t voff = (uint32_t)rsub * (uint32_t)(d_c * 2) + 16u * (uint32_t)(l16 ^ w_swz(k));
    lds_dma16(wsrc + (size_t)k0 * d_c * 2, voff, tile_lds + (uint32_t)k0 * kRowBytes);
  }
}

// Wave wt's two 16-column M tiles of the slice in LDS, for every query row:
// q_abs[r][head][c0 + 32 wt .. + 31] (q and q_abs row-major [R][h][...]).
__device__ __forceinline__ void compute_tile(const AS3 uint8_t* tile, const uint16_t* __restrict__ q,
                                             uint16_t* __restrict__ q_abs, int head, int c0, int rows,
                                             int h, int d_c, int wt, int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  // A operands, 4 K steps per M tile: lane j of 16-lane group g addresses
  // row 8g + (j >> 2) (+4 for the upper half of the step) and columns
  // 4 (j & 3) .. + 3 of its M tile
  bf16x8 a[2][kDh / 32];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int byte = 2 * (16 * (2 * wt + mt) + 4 * (l16 & 3));  // first column, within the row
#pragma unroll
    for (int s = 0; s < kDh / 32; ++s) {
      u16x4 half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k = 32 * s + 8 * g + 4 * hh + (l16 >> 2);
        const AS3 uint8_t* p = tile + k * kRowBytes + 16 * ((byte >> 4) ^ w_swz(k)) + (byte & 15);
        half[hh] = __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 tr_vec*)p));
      }
      const u16x8 v = {half[0][0], half[0][1], half[0][2], half[0][3],
                       half[1][0], half[1][1], half[1][2], half[1][3]};
      a[mt][s] = as_bf16x8(v);
    }
  }

  for (int rb = 0; rb < rows; rb += 16) {
    const int r = rb + l16;  // this lane's N column (query row)
    const uint16_t* qrow = q + ((size_t)r * h + head) * kDh;
    bf16x8 bq[kDh / 32];
#pragma unroll
    for (int s = 0; s < kDh / 32; ++s) {
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (r < rows) bv = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g);
      bq[s] = as_bf16x8(bv);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kDh / 32; ++s) acc = mfma16x16x32(a[mt][s], bq[s], acc);
      if (r < rows) {
        // D[4g + j][l16] = q_abs[r][head][c0 + 16 (2 wt + mt) + 4g + j]
        uint2 packed;
        packed.x = pack_bf16x2(acc[0], acc[1]);
        packed.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(q_abs + ((size_t)r * h + head) * d_c + c0 + 16 * (2 * wt + mt) + 4 * g) =
            packed;
      }
    }
  }
}

}  // namespace absorb
}  // namespace mla
