// finish.hip -- split combine and W_UV up-projection in one pass (fast path).
//
// For query row r and head i the split kernel left one normalised latent
// o_s (bf16, [R][S][h][512]) and one base-2 log-sum-exp lse_s (fp32) per
// context chunk s.  This kernel forms
//   c_bar = sum_s w_s o_s / sum_s w_s,   w_s = 2^(lse_s - m)
// for any reference m (here running maxima, merged at the end)
// (the softmax over the whole visible context evaluated chunk by chunk: the
// chunks partition the token axis, so the merge is exact up to rounding;
// "MLA, dim by dim" section 5.2) and then
//   o[r, i, :] = W_UV[i] c_bar
// (the value up-projection applied once per head, by linearity,
// "Mathematical Prerequisites for DeepSeek-V2" section 7; "From Vanilla
// Transformers to Modern LLMs ... Part 3" section 3.g).  Chunks with
// lse = -inf (nothing visible) weigh 0 and their result is never used.
//
// One work-group per (head, 64 output rows): W_UV[i] rows stream from HBM
// once, straight into the MFMA A operand (rows of W as M, d_c as K), while
// c_bar of 16 query rows at a time is built in LDS from the chunk results
// (one 1 KB row per chunk, 16-byte loads) and read back as the B operand.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDh = 128;
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 64;  // chunk groups of the combine

#define AS3 __attribute__((address_space(3)))

// Physical 16-byte chunk of logical chunk c in c_bar row `row` (< 16): the
// XOR spreads the B-operand reads (16 rows, one chunk each) over the banks.
__device__ __forceinline__ int cb_chunk(int row, int c) { return c ^ row; }

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void finish_bf16_kernel(const uint16_t* __restrict__ part_o,
                                                               const float* __restrict__ part_lse,
                                                               const uint16_t* __restrict__ w_uv,
                                                               void* __restrict__ out, int rows,
                                                               int splits, int h) {
  __shared__ __attribute__((aligned(16))) u32x4 cb[16][kDc / 8];  // c_bar rows, bf16
  __shared__ f32x4 part_acc[kGroups - 1][64][2];
  __shared__ float part_w[kGroups - 1][64];
  __shared__ float red[kThreads / 64];

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int a_base = 64 * blockIdx.y + 16 * wave;  // this wave's 16 output rows

  constexpr int kUnroll = 16;              // chunks in flight per lane
  const size_t stride = (size_t)h * kDc;   // elements of one chunk's results
  // One batch of the merge: the lse and the 8 features of this lane of the
  // chunks s0, s0 + 4, ... of row r (chunks past the end read as empty).
  auto load_batch = [&](int r, int s0, float* l, uint4* v) {
    const float* lse = part_lse + (size_t)r * splits * h + head;
    const uint16_t* src = part_o + ((size_t)r * splits * h + head) * kDc + 8 * lane;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + kGroups * u;
      if (s < splits) {  // uniform per wave
        l[u] = lse[(size_t)s * h];
        v[u] = *reinterpret_cast<const uint4*>(src + s * stride);
      } else {
        l[u] = -INFINITY;
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // The first batch goes out before the weight rows: loads complete in
  // order, so the merge then need not wait for the weight stream.
  float l_first[kUnroll];
  uint4 v_first[kUnroll];
  if (rows <= 0) return;  // (the host launches no empty batch)
  load_batch(0, wave, l_first, v_first);

  // W_UV[head] rows a_base .. a_base + 15 as the A operand: lane (g, l16)
  // holds row l16, d_c elements 32 s + 8 g .. + 7 for step s.
  const uint16_t* wrow = w_uv + ((size_t)head * kDh + a_base + l16) * kDc;
  bf16x8 wa[kDc / 32];
#pragma unroll
  for (int s = 0; s < kDc / 32; ++s)
    wa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(wrow + 32 * s + 8 * g));

  for (int rb = 0; rb < rows; rb += 16) {
    const int nr = min(16, rows - rb);
    // ---- combine: c_bar of rows rb .. rb + nr - 1 into LDS ----
    for (int rr = 0; rr < nr; ++rr) {
      const int r = rb + rr;
      // lane covers features 8 lane .. 8 lane + 7; wave `wave` takes every
      // 4th chunk with its own running maximum, the four are merged below
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f, mx = -INFINITY;
      for (int s0 = wave; s0 < splits; s0 += kGroups * kUnroll) {
        float l[kUnroll];
        uint4 v[kUnroll];
        if (r == 0 && s0 == wave) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            l[u] = l_first[u];
            v[u] = v_first[u];
          }
        } else {
          load_batch(r, s0, l, v);
        }
        float bmx = l[0];  // the same in every lane (one head)
#pragma unroll
        for (int u = 1; u < kUnroll; ++u) bmx = fmaxf(bmx, l[u]);
        if (bmx > mx) {  // raise the reference of what is summed so far
          const float f = mx == -INFINITY ? 0.f : exp2f(mx - bmx);
          acc0 *= f;
          acc1 *= f;
          wsum *= f;
          mx = bmx;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          // an empty chunk (lse = -inf) weighs 0 and its (unwritten) result
          // is dropped by the selects
          const float w = l[u] == -INFINITY ? 0.f : exp2f(l[u] - mx);
          const bool use = w != 0.f;
          const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = w * bf16_to_f32(static_cast<uint16_t>(x[e]));
            const float hi = w * bf16_to_f32(static_cast<uint16_t>(x[e] >> 16));
            if (e < 2) {
              acc0[2 * e] += use ? lo : 0.f;
              acc0[2 * e + 1] += use ? hi : 0.f;
            } else {
              acc1[2 * e - 4] += use ? lo : 0.f;
              acc1[2 * e - 3] += use ? hi : 0.f;
            }
          }
          wsum += w;
        }
      }
      if (wave > 0) {
        part_acc[wave - 1][lane][0] = acc0;
        part_acc[wave - 1][lane][1] = acc1;
        part_w[wave - 1][lane] = wsum;
        if (lane == 0) red[wave] = mx;
      }
      __syncthreads();
      if (wave == 0) {
        float mall = mx;
#pragma unroll
        for (int k = 1; k < kGroups; ++k) mall = fmaxf(mall, red[k]);
        const float f0 = mx == -INFINITY ? 0.f : exp2f(mx - mall);
        acc0 *= f0;
        acc1 *= f0;
        wsum *= f0;
#pragma unroll
        for (int k = 0; k < kGroups - 1; ++k) {
          const float mk = red[k + 1];
          const float fk = mk == -INFINITY ? 0.f : exp2f(mk - mall);
          acc0 += fk * part_acc[k][lane][0];
          acc1 += fk * part_acc[k][lane][1];
          wsum += fk * part_w[k][lane];
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        acc0 *= inv;
        acc1 *= inv;
        cb[rr][cb_chunk(rr, lane)] = u32x4{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                                           pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
      }
      __syncthreads();  // red, part_acc reusable; cb row written
    }

    // ---- up-projection of the block: D[a][r] = sum_c W_UV[a][c] c_bar[r][c] ----
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDc / 32; ++s) {
      u32x4 bv = {0u, 0u, 0u, 0u};
      if (l16 < nr) bv = cb[l16][cb_chunk(l16, 4 * s + g)];
      acc = mfma16x16x32(wa[s], __builtin_bit_cast(bf16x8, bv), acc);
    }
    const int r = rb + l16;
    if (l16 < nr) {
      // D[4g + j][l16] = o[r][head][a_base + 4g + j]
      const size_t o = ((size_t)r * h + head) * kDh + a_base + 4 * g;
      if (kBf16Out) {
        uint2 packed;
        packed.x = pack_bf16x2(acc[0], acc[1]);
        packed.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = packed;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + o) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    __syncthreads();  // cb is rewritten by the next block of rows
  }
}

}  // namespace

hipError_t launch_finish_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  const dim3 grid(a.h, kDh / 64);
  const uint16_t* po = static_cast<const uint16_t*>(a.part_o);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_uv);
  if (a.out_bf16)
    launch_kernel(finish_bf16_kernel<true>, grid, dim3(kThreads), s, po, a.part_lse, w, a.out, rows,
                  a.splits, a.h);
  else
    launch_kernel(finish_bf16_kernel<false>, grid, dim3(kThreads), s, po, a.part_lse, w, a.out, rows,
                  a.splits, a.h);
  return hipGetLastError();
}

}  // namespace mla
