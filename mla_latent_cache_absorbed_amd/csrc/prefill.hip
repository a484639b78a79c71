// prefill.hip -- attention over a whole prompt (prefill), in the order the
// pages derive for it: rebuild the per-head keys and values from the latent
// cache, then causal attention over d_h + d_r dimensions.
//
// For a prompt of T tokens with latents c_t (d_c), shared rotated RoPE keys
// k_R,t (d_r), queries q_t,i (d_h) and RoPE queries q_R,t,i (d_r):
//   k_t,i = W_UK[i] c_t,  v_t,i = W_UV[i] c_t                  (rebuild)
//   s(t, u) = scale ([q_t,i; q_R,t,i] . [k_u,i; k_R,u]),  u <= t (causal)
//   o_t,i = sum_u softmax_u(s(t, u)) v_u,i
// ("MLA, dim by dim" section 4.1: with T queries the quadratic score term
// should contract over d_k, so K and V are rebuilt first and the absorbed
// order of decode is the wrong one here; section 5.1 for the decoupled
// RoPE part; "Multi-Head Latent Attention: ..." section "MLA: Low-Rank
// Key-Value Joint Compression" for k = W^UK c).
//
// gfx950 design (bf16 storage, fp32 accumulation)
// - Rebuild: K_all [T][h d_h] = C [T][d_c] W_UK^T, the same for V: one
//   MFMA GEMM kernel, 128 x 128 output tiles per work-group (four waves of
//   64 x 64, 32x32x16 MFMA), k = d_c staged in 64-wide slices through LDS by
//   direct DMA (two stages, 16-byte chunks XOR-swizzled by row), the tile
//   written back through LDS so that each lane stores 16 contiguous bytes.
// - Attention: one work-group per (head, 128 queries), four waves of 32
//   queries sharing each 32-key tile of K (d_h), K_R (d_r) and V (d_h) in an
//   LDS ring of three stages filled by DMA.  Scores are computed transposed,
//   S^T = K Q^T (keys as M, queries as N, 192 as K) with the wave's queries
//   held in registers, so each lane owns one query's 16 scores of the tile:
//   the online softmax is per lane (the two lanes of a query combine with
//   one cross-half swap), and the accumulator O^T = V^T P^T (d_h as M) is
//   rescaled per lane.  P^T feeds the next MFMA straight from the score
//   registers: its key order (lane half g holds keys 4g..4g+3 and
//   8+4g..8+4g+3 of each 16) is matched by two transposing LDS reads of V
//   (ds_read_b64_tr_b16) per operand.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kThreads = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Rebuild GEMM: out[t][n] = sum_c x[t][c] w[n][c]
// ---------------------------------------------------------------------------
constexpr int kGemmTile = 128;
constexpr int kGemmK = 64;                    // k slice per LDS stage
constexpr int kGemmRowBytes = kGemmK * 2;     // 128 bytes per staged row
constexpr int kGemmTileBytes = kGemmTile * kGemmRowBytes;  // 16 KB per operand

struct GemmArgs {
  const uint16_t* x;       // [rows][k]
  const uint16_t* w[2];    // [n][k] each (grid z picks one)
  uint16_t* out[2];        // [rows][n] each
  int rows, k, n;
};

// 16-byte chunk c of staged row r (128 bytes) is stored at chunk
// c ^ ((r >> 1) & 7): two rows share each 256-byte bank period, so the 16
// rows one operand read serves at a time land in 16 different slots.
__device__ __forceinline__ int gemm_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ uint32_t gemm_off(int r, int c) { return (uint32_t)r * kGemmRowBytes + 16u * (uint32_t)(c ^ gemm_swz(r)); }

__global__ __launch_bounds__(kThreads) void kv_rebuild_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kGemmTileBytes];  // [stage][x | w]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int t0 = blockIdx.y * kGemmTile, n0 = blockIdx.x * kGemmTile;
  const int wm = wave >> 1, wn = wave & 1;  // the wave's 64 x 64 quarter
  const uint16_t* wsrc = a.w[blockIdx.z];
  uint16_t* dst = a.out[blockIdx.z];

  // DMA: one instruction fills 8 staged rows of 128 bytes (lane l writes
  // slot l % 8 of row l / 8, which holds chunk (l % 8) ^ gemm_swz(row): the
  // lane reads that chunk); a stage is 16 instructions per operand, 8 per wave
  const uint32_t lds_base = (uint32_t)(uintptr_t)((AS3 uint8_t*)lds);
  auto issue = [&](int stage, int kk) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int op = q >> 2;                   // 0: x rows, 1: w rows
      const int grp = 4 * wave + (q & 3);      // 8-row group of the tile
      const int r = 8 * grp + (lane >> 3);     // staged row 0..127
      const int base = op == 0 ? t0 : n0;
      const int lim = op == 0 ? a.rows : a.n;
      const int rr = base + r < lim ? r : lim - 1 - base;  // rows past the end repeat the last (never stored)
      const uint32_t voff = ((uint32_t)rr * (uint32_t)a.k + 8u * (uint32_t)((lane & 7) ^ gemm_swz(r))) * 2u;
      const uint16_t* sbase = (op == 0 ? a.x + (size_t)t0 * a.k : wsrc + (size_t)n0 * a.k) + kk;
      lds_dma16(sbase, voff, lds_base + (uint32_t)((stage * 2 + op) * kGemmTileBytes + grp * 8 * kGemmRowBytes));
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int slices = a.k / kGemmK;
  issue(0, 0);
  for (int sl = 0; sl < slices; ++sl) {
    const int st = sl & 1;
    wait_vm0();
    __syncthreads();  // slice sl is in stage st; everyone is done with stage st ^ 1
    if (sl + 1 < slices) issue(st ^ 1, (sl + 1) * kGemmK);
    const AS3 uint8_t* xs = (const AS3 uint8_t*)lds[st][0];
    const AS3 uint8_t* ws = (const AS3 uint8_t*)lds[st][1];
#pragma unroll
    for (int ks = 0; ks < kGemmK / 16; ++ks) {
      // k chunk of this lane: 2 ks + hi (16-byte chunks of the 128-byte row)
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + l32;
        av[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(xs + gemm_off(r, 2 * ks + hi)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 64 * wn + 32 * j + l32;
        bv[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(ws + gemm_off(r, 2 * ks + hi)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
    }
  }
  __syncthreads();  // the staging buffers are free
  // D[m][n] of block (i, j): lane l holds n = l32 (column), m = 8 (e / 4) +
  // 4 hi + e % 4 (row).  Write the 128 x 128 bf16 tile row-major into LDS
  // (256-byte rows, 16-byte chunks swizzled by row), then store 16 bytes per
  // lane: rows of the tile are contiguous 256-byte runs of the output.
  uint8_t* tile = &lds[0][0][0];  // 32 KB: 128 rows x 256 bytes
  auto tile_off = [](int r, int col) -> uint32_t {
    return (uint32_t)r * 256u + 16u * (uint32_t)(((col >> 3) ^ (r & 15))) + 2u * (uint32_t)(col & 7);
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        const int col = 64 * wn + 32 * j + l32;
        *reinterpret_cast<AS3 uint16_t*>((AS3 uint8_t*)tile + tile_off(r, col)) = f32_to_bf16(acc[i][j][e]);
      }
  __syncthreads();
  // 128 rows x 16 chunks = 2048 chunks, 8 per thread
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = q * kThreads + tid;
    const int r = idx >> 4, c = idx & 15;
    const int gr = t0 + r, gc = n0 + 8 * c;
    if (gr >= a.rows || gc >= a.n) continue;
    const u32x4 v = *reinterpret_cast<const AS3 u32x4*>((AS3 uint8_t*)tile + (uint32_t)r * 256u +
                                                         16u * (uint32_t)(c ^ (r & 15)));
    *reinterpret_cast<u32x4*>(dst + (size_t)gr * a.n + gc) = v;
  }
}

// ---------------------------------------------------------------------------
// Causal attention over the rebuilt keys and values (d_h = 128, d_r = 64)
// ---------------------------------------------------------------------------
constexpr int kDh = 128;
constexpr int kDr = 64;
constexpr int kKeyTile = 32;
constexpr int kQueries = 128;                      // per work-group (4 waves x 32)
constexpr int kStages = 3;
constexpr int kKBytes = kKeyTile * kDh * 2;        // 8 KB: 32 rows of 256 bytes
constexpr int kRBytes = kKeyTile * kDr * 2;        // 4 KB: 32 rows of 128 bytes
constexpr int kVBytes = kKeyTile * kDh * 2;        // 8 KB
constexpr int kStageBytes = kKBytes + kRBytes + kVBytes;
constexpr int kAttnDmas = (kKBytes + kRBytes + kVBytes) / 1024 / 4;  // per wave per tile: 5
constexpr float kRescaleSlack = 8.0f;              // log2 units a weight may exceed 1 by

struct AttnArgs {
  const uint16_t* k_all;  // [T][h][d_h]
  const uint16_t* v_all;  // [T][h][d_h]
  const uint16_t* kr;     // [T][d_r]
  const uint16_t* q;      // [T][h][d_h]
  const uint16_t* qr;     // [T][h][d_r]
  void* out;              // [T][h][d_h]
  int T, h, qblocks, out_bf16;
  float scale_log2;
};

// LDS layouts of a stage (16-byte chunks XOR-swizzled by row):
// K rows (256 B): chunk c of row r at c ^ (r & 15)      (score operand reads)
// K_R rows (128 B): chunk c at c ^ ((r >> 1) & 7) (two rows per bank period)
// V rows (256 B): chunk c at c ^ (4 (r & 3))             (transposing reads)
__device__ __forceinline__ uint32_t k_off(int r, int c) { return (uint32_t)r * 256u + 16u * (uint32_t)(c ^ (r & 15)); }
__device__ __forceinline__ uint32_t r_off(int r, int c) { return (uint32_t)r * 128u + 16u * (uint32_t)(c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ uint32_t v_off(int r, int col) {
  return (uint32_t)r * 256u + 16u * (uint32_t)((col >> 3) ^ (4 * (r & 3))) + 8u * (uint32_t)((col >> 2) & 1);
}

__global__ __launch_bounds__(kThreads, 2) void prefill_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages][kStageBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  // all query blocks of a head on one XCD (block index mod 8), the longest
  // (latest) blocks first
  const int id = blockIdx.x;
  const int rest = id >> 3;
  const int head = (rest / a.qblocks) * 8 + (id & 7);
  if (head >= a.h) return;
  const int qblk = a.qblocks - 1 - rest % a.qblocks;
  const int qb = qblk * kQueries;
  const int qw = qb + 32 * wave;                       // this wave's first query
  const int kend = min(a.T, qb + kQueries);            // keys the block needs: 0 .. kend - 1
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
  // tiles this wave computes (none when all its queries lie past the prompt)
  const int my_tiles = qw >= a.T ? 0 : min(ntiles, (min(a.T, qw + 32) + kKeyTile - 1) / kKeyTile);
  const size_t hd = (size_t)a.h * kDh;

  // queries: B operand of S^T = K Q^T, lane = query qw + l32, dims 16 s + 8 hi
  bf16x8 qv[12];
  {
    const int qq = min(qw + l32, a.T - 1);
    const uint16_t* qp = a.q + (size_t)qq * hd + (size_t)head * kDh + 8 * hi;
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * s));
    const uint16_t* qrp = a.qr + ((size_t)qq * a.h + head) * kDr + 8 * hi;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[8 + s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrp + 16 * s));
    // Consume the query registers here: the compiler then waits for these
    // loads once, before the loop.  (Its waits for them inside the loop
    // count the tile DMAs too, which it cannot see, and so made every tile
    // wait for the DMAs just issued for tile it + 2.)
#pragma unroll
    for (int s = 0; s < 12; ++s) asm volatile("" ::"v"(qv[s]));
  }

  // tile DMAs: per tile 8 KB of K (8 instructions of 4 rows), 4 KB of K_R (4
  // of 8 rows), 8 KB of V (8 of 4 rows): 20, five per wave
  const uint32_t ring_base = (uint32_t)(uintptr_t)((AS3 uint8_t*)ring);
  auto dma = [&](int tile) {
    const int stage = tile % kStages;
    const int k0 = tile * kKeyTile;
#pragma unroll
    for (int u = 0; u < kAttnDmas; ++u) {
      const int d = 5 * wave + u;  // 0..19: K 0..7, K_R 8..11, V 12..19
      if (d < 8 || d >= 12) {
        const bool isv = d >= 12;
        const int grp = isv ? d - 12 : d;        // 4-row group
        const int r = 4 * grp + (lane >> 4);     // tile row 0..31
        const int key = min(k0 + r, a.T - 1);    // keys past the end repeat the last (masked)
        const int c = (lane & 15) ^ (isv ? 4 * (r & 3) : (r & 15));  // chunk this lane's slot holds
        // uniform base at the tile's first key, so the lane offsets stay small
        const uint16_t* base = (isv ? a.v_all : a.k_all) + (size_t)k0 * hd + (size_t)head * kDh;
        const uint32_t voff = (uint32_t)((size_t)(key - k0) * hd * 2) + 16u * (uint32_t)c;
        lds_dma16(base, voff, ring_base + (uint32_t)(stage * kStageBytes + (isv ? kKBytes + kRBytes : 0) + grp * 1024));
      } else {
        const int grp = d - 8;                   // 8-row group
        const int r = 8 * grp + (lane >> 3);
        const int key = min(k0 + r, a.T - 1);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        const uint32_t voff = (uint32_t)(key - k0) * (kDr * 2) + 16u * (uint32_t)c;
        lds_dma16(a.kr + (size_t)k0 * kDr, voff, ring_base + (uint32_t)(stage * kStageBytes + kKBytes + grp * 1024));
      }
    }
  };
  dma(0);
  if (ntiles > 1) dma(1);

  f32x16 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // transposing-read addresses (lane group q = lane / 16, a16 = lane % 16):
  // keys 16 ks + 4 (q / 2) + a16 / 4 (+ 8), dims 32 mb + 16 (q % 2) + 4 (a16 % 4)
  const int q4 = lane >> 4, a16 = lane & 15;
  const int tr_row = 4 * (q4 >> 1) + (a16 >> 2);
  const int tr_col = 16 * (q4 & 1) + 4 * (a16 & 3);

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else wait_vm0();
    static_assert(kAttnDmas == 5, "the wait above counts one tile of a wave's DMAs");
    __syncthreads();  // tile it is in LDS; tile it - 1's stage is free
    if (it + 2 < ntiles) dma(it + 2);
    if (it >= my_tiles) continue;  // keys past this wave's last query
    const AS3 uint8_t* st = (const AS3 uint8_t*)ring + (it % kStages) * kStageBytes;
    // ---- S^T[key][query] over 128 content + 64 RoPE dims ----
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      const AS3 uint8_t* src = s < 8 ? st + k_off(l32, 2 * s + hi) : st + kKBytes + r_off(l32, 2 * (s - 8) + hi);
      sc = mfma32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(src)), qv[s], sc);
    }
    // ---- online softmax of the lane's query (base 2) ----
    const int k0 = it * kKeyTile;
    float tmax = -INFINITY;
    if (k0 + kKeyTile > qw || k0 + kKeyTile > a.T) {  // the wave's diagonal tile, or the prompt's last
      const int query = qw + l32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 8 * (j >> 2) + 4 * hi + (j & 3);
        const float v = (key <= query && key < a.T) ? sc[j] * a.scale_log2 : -INFINITY;
        sc[j] = v;
        tmax = fmaxf(tmax, v);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sc[j] *= a.scale_log2;
        tmax = fmaxf(tmax, sc[j]);
      }
    }
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if (tmax > m_run + kRescaleSlack) {  // the reference moves (always on the first tile)
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - tmax);
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < 4; ++m) o[m] *= alpha;
      m_run = tmax;
    }
    bf16x8 pb[2];
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = __builtin_amdgcn_exp2f(sc[8 * ks + e] - m_run);
      pb[ks] = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 two = {pb[ks][e], pb[ks][e + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(two, one, l_run, false);
      }
    }
    // ---- O^T[dv][query] += V^T[dv][keys] P^T[keys][query] ----
    const AS3 uint8_t* vs = st + kKBytes + kRBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r0 = 16 * ks + tr_row, col = 32 * mb + tr_col;
        const u16x4 lo = __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 tr_vec*)(vs + v_off(r0, col))));
        const u16x4 up = __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 tr_vec*)(vs + v_off(r0 + 8, col))));
        const u16x8 av = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        o[mb] = mfma32x32x16(as_bf16x8(av), pb[ks], o[mb]);
      }
  }

  // ---- normalise and store: lane holds dims 32 mb + 8 (j / 4) + 4 hi + j % 4 of its query ----
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int query = qw + l32;
    if (query < a.T) {
      const size_t row = (size_t)query * hd + (size_t)head * kDh;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * mb + 8 * g + 4 * hi;
          const f32x4 v = {o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv, o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv};
          if (a.out_bf16)
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row + dim) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          else
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row + dim) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Plain kernels: any dims, either storage type
// ---------------------------------------------------------------------------
// out[t][n] = sum_c x[t][c] w[n][c] (fp32 sum)
template <typename T>
__global__ __launch_bounds__(kThreads) void rebuild_general_kernel(const T* x, const T* w, T* out, int rows, int k,
                                                                   int n) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)rows * n) return;
  const int t = (int)(i / n), c = (int)(i % n);
  float acc = 0.f;
  for (int m = 0; m < k; ++m) acc = __builtin_fmaf(load_as_f32(x + (size_t)t * k, m), load_as_f32(w + (size_t)c * k, m), acc);
  store_from_f32(out, i, acc);
}

// One thread per (query, head): two passes over its visible keys (maximum,
// then weights and the weighted value sum), fp32.
template <typename T, typename Tout>
__global__ __launch_bounds__(kThreads) void attn_general_kernel(const T* k_all, const T* v_all, const T* kr, const T* q,
                                                                const T* qr, Tout* out, int Tn, int h, int d_h, int d_r,
                                                                float scale) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)Tn * h) return;
  const int t = (int)(i / h), head = (int)(i % h);
  const size_t hd = (size_t)h * d_h;
  auto score = [&](int u) {
    float s = 0.f;
    for (int d = 0; d < d_h; ++d)
      s = __builtin_fmaf(load_as_f32(q, (size_t)t * hd + (size_t)head * d_h + d), load_as_f32(k_all, (size_t)u * hd + (size_t)head * d_h + d), s);
    for (int d = 0; d < d_r; ++d)
      s = __builtin_fmaf(load_as_f32(qr, ((size_t)t * h + head) * d_r + d), load_as_f32(kr, (size_t)u * d_r + d), s);
    return s * scale;
  };
  float mx = -INFINITY;
  for (int u = 0; u <= t; ++u) mx = fmaxf(mx, score(u));
  for (int d = 0; d < d_h; ++d) {  // one output dim per pass (small shapes only)
    float acc = 0.f, l = 0.f;
    for (int u = 0; u <= t; ++u) {
      const float p = expf(score(u) - mx);
      l += p;
      acc = __builtin_fmaf(p, load_as_f32(v_all, (size_t)u * hd + (size_t)head * d_h + d), acc);
    }
    store_from_f32(out, (size_t)t * hd + (size_t)head * d_h + d, acc / l);
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

bool prefill_fast(int d_c, int d_r, int d_h, bool bf16) {
  return bf16 && d_h == kDh && d_r == kDr && d_c % kGemmK == 0;
}

size_t prefill_workspace_bytes(int T, int h, int d_h, bool bf16) {
  return 2 * align256((size_t)T * h * d_h * (bf16 ? 2 : 4));
}

hipError_t launch_prefill(const PrefillLaunch& p, const LaunchCtx& s) {
  if (p.T == 0) return hipSuccess;
  const size_t kv = align256((size_t)p.T * p.h * p.d_h * (p.bf16 ? 2 : 4));
  void* k_all = p.work;
  void* v_all = static_cast<uint8_t*>(p.work) + kv;
  const int n = p.h * p.d_h;
  if (prefill_fast(p.d_c, p.d_r, p.d_h, p.bf16)) {
    GemmArgs g;
    g.x = static_cast<const uint16_t*>(p.latent);
    g.w[0] = static_cast<const uint16_t*>(p.w_uk);
    g.w[1] = static_cast<const uint16_t*>(p.w_uv);
    g.out[0] = static_cast<uint16_t*>(k_all);
    g.out[1] = static_cast<uint16_t*>(v_all);
    g.rows = p.T;
    g.k = p.d_c;
    g.n = n;
    launch_kernel(kv_rebuild_kernel, dim3((n + kGemmTile - 1) / kGemmTile, (p.T + kGemmTile - 1) / kGemmTile, 2),
                  dim3(kThreads), s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnArgs a;
    a.k_all = static_cast<const uint16_t*>(k_all);
    a.v_all = static_cast<const uint16_t*>(v_all);
    a.kr = static_cast<const uint16_t*>(p.rope);
    a.q = static_cast<const uint16_t*>(p.q);
    a.qr = static_cast<const uint16_t*>(p.q_r);
    a.out = p.out;
    a.T = p.T;
    a.h = p.h;
    a.qblocks = (p.T + kQueries - 1) / kQueries;
    a.out_bf16 = p.out_bf16;
    a.scale_log2 = p.scale * kLog2e;
    const int groups = ((p.h + 7) / 8) * 8 * a.qblocks;
    launch_kernel(prefill_attn_kernel, dim3(groups), dim3(kThreads), s, a);
    return hipGetLastError();
  }
  const dim3 rgrid((unsigned)(((size_t)p.T * n + kThreads - 1) / kThreads));
  const dim3 agrid((unsigned)(((size_t)p.T * p.h + kThreads - 1) / kThreads));
  if (p.bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(p.latent);
    launch_kernel(rebuild_general_kernel<uint16_t>, rgrid, dim3(kThreads), s, x, static_cast<const uint16_t*>(p.w_uk),
                  static_cast<uint16_t*>(k_all), p.T, p.d_c, n);
    launch_kernel(rebuild_general_kernel<uint16_t>, rgrid, dim3(kThreads), s, x, static_cast<const uint16_t*>(p.w_uv),
                  static_cast<uint16_t*>(v_all), p.T, p.d_c, n);
    auto args = [&](auto* out) {
      launch_kernel(attn_general_kernel<uint16_t, std::remove_pointer_t<decltype(out)>>, agrid, dim3(kThreads), s,
                    static_cast<const uint16_t*>(k_all), static_cast<const uint16_t*>(v_all),
                    static_cast<const uint16_t*>(p.rope), static_cast<const uint16_t*>(p.q),
                    static_cast<const uint16_t*>(p.q_r), out, p.T, p.h, p.d_h, p.d_r, p.scale);
    };
    if (p.out_bf16) args(static_cast<uint16_t*>(p.out));
    else args(static_cast<float*>(p.out));
  } else {
    const float* x = static_cast<const float*>(p.latent);
    launch_kernel(rebuild_general_kernel<float>, rgrid, dim3(kThreads), s, x, static_cast<const float*>(p.w_uk),
                  static_cast<float*>(k_all), p.T, p.d_c, n);
    launch_kernel(rebuild_general_kernel<float>, rgrid, dim3(kThreads), s, x, static_cast<const float*>(p.w_uv),
                  static_cast<float*>(v_all), p.T, p.d_c, n);
    auto args = [&](auto* out) {
      launch_kernel(attn_general_kernel<float, std::remove_pointer_t<decltype(out)>>, agrid, dim3(kThreads), s,
                    static_cast<const float*>(k_all), static_cast<const float*>(v_all),
                    static_cast<const float*>(p.rope), static_cast<const float*>(p.q),
                    static_cast<const float*>(p.q_r), out, p.T, p.h, p.d_h, p.d_r, p.scale);
    };
    if (p.out_bf16) args(static_cast<uint16_t*>(p.out));
    else args(static_cast<float*>(p.out));
  }
  return hipGetLastError();
}

}  // namespace mla
