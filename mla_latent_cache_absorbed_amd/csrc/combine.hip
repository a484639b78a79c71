// combine.hip -- merge the per-chunk results of the split kernel.
//
// Chunk s of a query row produced a normalised latent o_s (bf16 on the
// fast path, fp32 on the general path) and a base-2 log-sum-exp lse_s of its
// scores (fp32).  The full-context weighted latent is
//   c_bar = sum_s w_s o_s,  w_s = 2^(lse_s - LSE),  LSE = log2 sum_s 2^lse_s,
// which equals sum_t p_t C[t] over the whole visible context (the softmax of
// "MLA, dim by dim" section 5.2 evaluated chunk by chunk; chunks partition
// the token axis, so the merge is exact up to rounding).  Empty chunks carry
// lse = -inf and weight 0.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// General path: fp32 partials, any d_c.
template <bool kBf16Out>
__global__ __launch_bounds__(128) void combine_general_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_lse,
                                                              void* __restrict__ c_bar, int splits,
                                                              int h, int d_c) {
  const int row_head = blockIdx.x;  // r * h + head
  const int r = row_head / h, head = row_head % h;
  const float* lse = part_lse + (size_t)r * splits * h + head;

  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, lse[(size_t)s * h]);

  for (int f = threadIdx.x; f < d_c; f += blockDim.x) {
    float acc = 0.f, wsum = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float l = lse[(size_t)s * h];
      if (l == -INFINITY) continue;
      const float w = exp2f(l - mx);
      wsum += w;
      acc += w * part_o[(((size_t)r * splits + s) * h + head) * d_c + f];
    }
    const float v = wsum > 0.f ? acc / wsum : 0.f;
    const size_t o = (size_t)row_head * d_c + f;
    if (kBf16Out) static_cast<uint16_t*>(c_bar)[o] = f32_to_bf16(v);
    else static_cast<float*>(c_bar)[o] = v;
  }
}

// Fast path: bf16 partials, d_c = 512, bf16 output.  The split kernel
// stores each chunk result in the order its registers hold it, so that every
// store instruction writes 512 contiguous bytes:
//   [row][chunk][h / 16 head blocks][32 feature blocks][64 lanes][4]
// where lane = 16 ((f % 16) / 4) + head % 16 and the last index is f % 4,
// for feature f = 16 (feature block) + 4 ((f % 16) / 4) + f % 4.  The result
// of a chunk with lse = -inf is undefined and never read.
//
// Block (row, head block, feature block): 64 lanes x 4 groups that take
// every 4th chunk, merged through LDS.
constexpr int kFastDc = 512;

__global__ __launch_bounds__(256) void combine_fast_kernel(const uint16_t* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           uint16_t* __restrict__ c_bar,
                                                           int splits, int h) {
  __shared__ float mx_part[16][16];  // [split subset][head]
  __shared__ f32x4 acc_part[3][64];
  __shared__ float wsum_part[3][64];
  const int hblocks = h / 16;
  const int r = blockIdx.x / hblocks, hb = blockIdx.x % hblocks, fb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 6, l16 = lane & 15;
  const float* lse = part_lse + (size_t)r * splits * h + hb * 16;

  {  // largest chunk lse of each of the 16 heads
    const int i = tid & 15, k = tid >> 4;
    float m = -INFINITY;
    for (int s = k; s < splits; s += 16) m = fmaxf(m, lse[(size_t)s * h + i]);
    mx_part[k][i] = m;
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) mx = fmaxf(mx, mx_part[k][l16]);

  const size_t split_stride = (size_t)h * kFastDc;  // elements per chunk
  const uint16_t* src = part_o + (size_t)r * splits * split_stride +
                        (((size_t)hb * (kFastDc / 16) + fb) * 64 + lane) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  // Four chunks per step, all loads first so that they are in flight
  // together.  An empty chunk's result is read but never used: its weight
  // is 0 and the select below drops the (possibly non-finite) product.
  constexpr int kUnroll = 4;
  for (int s0 = grp; s0 < splits; s0 += 4 * kUnroll) {
    float l[kUnroll];
    uint2 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + 4 * u;
      if (s < splits) {  // uniform per wave
        l[u] = lse[(size_t)s * h + l16];
        v[u] = *reinterpret_cast<const uint2*>(src + s * split_stride);
      } else {
        l[u] = -INFINITY;
        v[u] = make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = l[u] == -INFINITY ? 0.f : exp2f(l[u] - mx);
      const bool use = w != 0.f;
      const float x0 = w * bf16_to_f32(static_cast<uint16_t>(v[u].x));
      const float x1 = w * bf16_to_f32(static_cast<uint16_t>(v[u].x >> 16));
      const float x2 = w * bf16_to_f32(static_cast<uint16_t>(v[u].y));
      const float x3 = w * bf16_to_f32(static_cast<uint16_t>(v[u].y >> 16));
      acc[0] += use ? x0 : 0.f;
      acc[1] += use ? x1 : 0.f;
      acc[2] += use ? x2 : 0.f;
      acc[3] += use ? x3 : 0.f;
      wsum += w;
    }
  }
  if (grp > 0) {
    acc_part[grp - 1][lane] = acc;
    wsum_part[grp - 1][lane] = wsum;
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      acc += acc_part[k][lane];
      wsum += wsum_part[k][lane];
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int head = hb * 16 + l16;
    const int f0 = fb * 16 + 4 * (lane >> 4);
    *reinterpret_cast<uint2*>(c_bar + ((size_t)r * h + head) * kFastDc + f0) =
        make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool fast, const LaunchCtx& s) {
  const int blocks = a.batch * a.n_q * a.h;
  if (fast)
    launch_kernel(combine_fast_kernel, dim3(a.batch * a.n_q * (a.h / 16), kFastDc / 16), dim3(256), s,
                       static_cast<const uint16_t*>(a.part_o), a.part_lse,
                       static_cast<uint16_t*>(a.c_bar), a.splits, a.h);
  else
    launch_kernel(combine_general_kernel<false>, dim3(blocks), dim3(128), s,
                       static_cast<const float*>(a.part_o), a.part_lse, a.c_bar, a.splits, a.h,
                       a.d_c);
  return hipGetLastError();
}

}  // namespace mla
