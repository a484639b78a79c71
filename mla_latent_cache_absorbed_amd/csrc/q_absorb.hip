// q_absorb.hip -- query absorption: q_abs[r, i, :] = W_UK[i]^T q[r, i, :].
//
// Moves the key up-projection from every cached token onto the one new
// query (the bilinear identity a^T M b = (M^T a)^T b, "Mathematical
// Prerequisites for DeepSeek-V2" section 6; the absorbed query of "MLA, dim
// by dim" section 5.1 and the q^A of "From Vanilla Transformers to Modern
// LLMs ... Part 3" section 3.e.2).  Cost per query row: 2 h d_h d_c FLOPs,
// independent of the context length.
//
// Fast path (bf16, d_h = 128): one work-group per (head, 128 latent
// columns).  W_UK[i] streams from HBM exactly once (32 KB per group) by
// direct global->LDS DMA in its stored [d_h][d_c] order; the contraction
// runs on 16x16x32 bf16 MFMA with the latent column as M, the query row as N
// and d_h as K.  The K-contiguous A operand the MFMA wants is W^T; the
// transposing LDS read ds_read_b64_tr_b16 produces it from the row-major
// tile (within 16 lanes, lane i receives element i & 3 of the 8-byte chunk
// addressed by lane 4e + (i >> 2), for e = 0..3).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDh = 128;             // d_h of the fast path (MFMA K)
constexpr int kCols = 128;           // latent columns per work-group
constexpr int kRowBytes = kCols * 2;  // 256 B of one W row in the tile
constexpr int kThreads = 256;

#define AS3 __attribute__((address_space(3)))
typedef short tr_vec __attribute__((vector_size(8)));

// XOR on the 16-byte chunk index (0..15) of tile row k.  The transposing
// reads of one 32-lane half touch 8 rows (k = 0-3 and 8-11 of its 32-row
// slab) at the same two adjacent chunks; this sends them to 8 distinct
// chunk pairs, i.e. to all 64 banks.
__device__ __forceinline__ int w_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// One wave-wide DMA of 64 x 16 bytes: lane l reads sbase + voff and writes
// lds_base + 16 l (M0 holds the LDS base; saved and restored around it).
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}

__global__ __launch_bounds__(kThreads) void q_absorb_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_abs, int rows, int h, int d_c) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDh * kRowBytes];  // 32 KB

  const int head = blockIdx.x;
  const int c0 = blockIdx.y * kCols;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;

  // ---- W_UK[head][:, c0 : c0 + 128] into LDS, row-major, swizzled: wave w
  //      copies rows 32w .. 32w + 31, four 256-byte rows per DMA ----
  {
    const uint32_t tile_base = (uint32_t)(uintptr_t)((AS3 uint8_t*)tile);
    const int rsub = lane >> 4;  // row within the DMA
    const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(w_uk + (size_t)head * kDh * d_c + c0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k0 = 32 * wave + 4 * j;
      const int k = k0 + rsub;
      const uint32_t voff = (uint32_t)rsub * (uint32_t)(d_c * 2) + 16u * (uint32_t)(l16 ^ w_swz(k));
      lds_dma16(wsrc + (size_t)k0 * d_c * 2, voff, tile_base + (uint32_t)k0 * kRowBytes);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- A operands: this wave's two 16-column M tiles, 4 K steps each ----
  // lane j of 16-lane group g addresses row 8g + (j >> 2) (+4 for the upper
  // half of the step) and columns 4 (j & 3) .. + 3 of its M tile
  bf16x8 a[2][kDh / 32];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int col = 16 * (2 * wave + mt) + 4 * (l16 & 3);  // first of 4 columns
#pragma unroll
    for (int s = 0; s < kDh / 32; ++s) {
      u16x4 half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k = 32 * s + 8 * g + 4 * hh + (l16 >> 2);
        const int byte = col * 2;  // within the row
        const AS3 uint8_t* p = (const AS3 uint8_t*)tile + k * kRowBytes +
                               16 * ((byte >> 4) ^ w_swz(k)) + (byte & 15);
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
        // D[4g + j][l16] = q_abs[r][head][c0 + 16 (2 wave + mt) + 4g + j]
        uint2 packed;
        packed.x = pack_bf16x2(acc[0], acc[1]);
        packed.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(q_abs + ((size_t)r * h + head) * d_c + c0 + 16 * (2 * wave + mt) + 4 * g) =
            packed;
      }
    }
  }
}

}  // namespace

hipError_t launch_q_absorb_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  dim3 grid(a.h, a.d_c / kCols);
  launch_kernel(q_absorb_bf16_kernel, grid, dim3(kThreads), s,
                static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.w_uk),
                static_cast<uint16_t*>(a.q_abs), rows, a.h, a.d_c);
  return hipGetLastError();
}

}  // namespace mla
