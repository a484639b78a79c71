// combine.hip -- merge the per-chunk results of the general split kernel
// (the fast path merges them inside finish.hip).
//
// Chunk s of a query row produced a normalised latent o_s (fp32) and a
// base-2 log-sum-exp lse_s of its scores (fp32).  The full-context weighted latent is
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

}  // namespace

hipError_t launch_combine_general(const DecodeArgs& a, const LaunchCtx& s) {
  const int blocks = a.batch * a.n_q * a.h;
  launch_kernel(combine_general_kernel<false>, dim3(blocks), dim3(128), s,
                static_cast<const float*>(a.part_o), a.part_lse, a.c_bar, a.splits, a.h, a.d_c);
  return hipGetLastError();
}

}  // namespace mla
