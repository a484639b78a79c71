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

// Fast path: bf16 partials, d_c = 512, bf16 output.  Block (row*h + head,
// half of the features): 64 threads per 4-feature group column x 4 groups
// that take every 4th split, merged through LDS at the end.
constexpr int kFastDc = 512;

__global__ __launch_bounds__(256) void combine_fast_kernel(const uint16_t* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           uint16_t* __restrict__ c_bar,
                                                           int splits, int h) {
  __shared__ float red[256];
  __shared__ f32x4 acc_part[3][64];
  __shared__ float wsum_part[3];
  const int row_head = blockIdx.x;
  const int r = row_head / h, head = row_head % h;
  const int tid = threadIdx.x, fq = tid & 63, grp = tid >> 6;
  const float* lse = part_lse + (size_t)r * splits * h + head;

  float mx = -INFINITY;
  for (int s = tid; s < splits; s += 256) mx = fmaxf(mx, lse[(size_t)s * h]);
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];

  const int f0 = blockIdx.y * (kFastDc / 2) + 4 * fq;
  const uint16_t* src = part_o + ((size_t)r * splits * h + head) * kFastDc + f0;
  const size_t split_stride = (size_t)h * kFastDc;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll 4
  for (int s = grp; s < splits; s += 4) {
    const float l = lse[(size_t)s * h];
    const float w = l == -INFINITY ? 0.f : exp2f(l - mx);
    const uint2 v = *reinterpret_cast<const uint2*>(src + s * split_stride);
    wsum += w;
    acc[0] += w * bf16_to_f32(static_cast<uint16_t>(v.x));
    acc[1] += w * bf16_to_f32(static_cast<uint16_t>(v.x >> 16));
    acc[2] += w * bf16_to_f32(static_cast<uint16_t>(v.y));
    acc[3] += w * bf16_to_f32(static_cast<uint16_t>(v.y >> 16));
  }
  if (grp > 0) {
    acc_part[grp - 1][fq] = acc;
    if (fq == 0) wsum_part[grp - 1] = wsum;
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) acc += acc_part[k][fq];
    const float total = wsum + wsum_part[0] + wsum_part[1] + wsum_part[2];
    const float inv = total > 0.f ? 1.f / total : 0.f;
    *reinterpret_cast<uint2*>(c_bar + (size_t)row_head * kFastDc + f0) =
        make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool fast, const LaunchCtx& s) {
  const int blocks = a.batch * a.n_q * a.h;
  if (fast)
    launch_kernel(combine_fast_kernel, dim3(blocks, 2), dim3(256), s,
                       static_cast<const uint16_t*>(a.part_o), a.part_lse,
                       static_cast<uint16_t*>(a.c_bar), a.splits, a.h);
  else
    launch_kernel(combine_general_kernel<false>, dim3(blocks), dim3(128), s,
                       static_cast<const float*>(a.part_o), a.part_lse, a.c_bar, a.splits, a.h,
                       a.d_c);
  return hipGetLastError();
}

}  // namespace mla
