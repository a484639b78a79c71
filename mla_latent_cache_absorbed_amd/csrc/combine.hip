// combine.hip -- merge the per-chunk results of the split kernel.
//
// Chunk s of a query row produced a normalised latent o_s and a base-2
// log-sum-exp lse_s of its scores.  The full-context weighted latent is
//   c_bar = sum_s w_s o_s,  w_s = 2^(lse_s - LSE),  LSE = log2 sum_s 2^lse_s,
// which equals sum_t p_t C[t] over the whole visible context (the softmax of
// "MLA, dim by dim" section 5.2 evaluated chunk by chunk; chunks partition
// the token axis, so the merge is exact up to rounding).  Empty chunks carry
// lse = -inf and weight 0.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

template <bool kBf16Out>
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      void* __restrict__ c_bar, int splits, int h,
                                                      int d_c) {
  const int row_head = blockIdx.x;  // r * h + head
  const int r = row_head / h, head = row_head % h;
  const float* lse = part_lse + (size_t)r * splits * h + head;

  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, lse[(size_t)s * h]);

  for (int f0 = 4 * threadIdx.x; f0 < d_c; f0 += 4 * blockDim.x) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    const int nf = min(4, d_c - f0);
    for (int s = 0; s < splits; ++s) {
      const float l = lse[(size_t)s * h];
      if (l == -INFINITY) continue;
      const float w = exp2f(l - mx);
      wsum += w;
      const float* src = part_o + (((size_t)r * splits + s) * h + head) * d_c + f0;
      if (nf == 4 && (d_c & 3) == 0) {
        const float4 v = *reinterpret_cast<const float4*>(src);
        acc[0] += w * v.x; acc[1] += w * v.y; acc[2] += w * v.z; acc[3] += w * v.w;
      } else {
        for (int e = 0; e < nf; ++e) acc[e] += w * src[e];
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const size_t o = (size_t)row_head * d_c + f0;
    if (kBf16Out) {
      uint16_t* dst = static_cast<uint16_t*>(c_bar);
      for (int e = 0; e < nf; ++e) dst[o + e] = f32_to_bf16(acc[e] * inv);
    } else {
      float* dst = static_cast<float*>(c_bar);
      for (int e = 0; e < nf; ++e) dst[o + e] = acc[e] * inv;
    }
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool cbar_bf16, hipStream_t s) {
  const int blocks = a.batch * a.n_q * a.h;
  if (cbar_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(128), 0, s, a.part_o, a.part_lse,
                       a.c_bar, a.splits, a.h, a.d_c);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(128), 0, s, a.part_o, a.part_lse,
                       a.c_bar, a.splits, a.h, a.d_c);
  return hipGetLastError();
}

}  // namespace mla
