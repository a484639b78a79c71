// up_project.hip -- value up-projection: o[r, i, :] = W_UV[i] c_bar[r, i, :].
//
// Applied once per head to the softmax-weighted latent instead of once per
// cached token (linearity, "Mathematical Prerequisites for DeepSeek-V2"
// section 7; "MLA, dim by dim" section 4.2, value chain; "From Vanilla
// Transformers to Modern LLMs ... Part 3" section 3.g).  Cost per query row:
// 2 h d_c d_h FLOPs; the weight (h d_h d_c values) streams from HBM once.
//
// Fast path (bf16, d_c = 512, d_h = 128): one work-group per (head, 64
// output rows).  W_UV[i] is stored [d_h][d_c] with d_c fastest, which is
// already the K-contiguous A operand of a 16x16x32 MFMA (rows of W as M,
// query rows as N), so each lane streams its operand straight from HBM.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDh = 128;

template <bool kBf16Out>
__global__ __launch_bounds__(256) void up_project_bf16_kernel(const uint16_t* __restrict__ w_uv,
                                                              const uint16_t* __restrict__ c_bar,
                                                              void* __restrict__ out, int rows,
                                                              int h) {
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int a_base = 64 * blockIdx.y + 16 * wave;  // this wave's 16 output rows

  const uint16_t* wrow = w_uv + ((size_t)head * kDh + a_base + l16) * kDc;
  bf16x8 wa[kDc / 32];
#pragma unroll
  for (int s = 0; s < kDc / 32; ++s)
    wa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(wrow + 32 * s + 8 * g));

  for (int rb = 0; rb < rows; rb += 16) {
    const int r = rb + l16;
    const uint16_t* crow = c_bar + ((size_t)r * h + head) * kDc;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDc / 32; ++s) {
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (r < rows) bv = *reinterpret_cast<const uint4*>(crow + 32 * s + 8 * g);
      acc = mfma16x16x32(wa[s], as_bf16x8(bv), acc);
    }
    if (r < rows) {
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
  }
}

}  // namespace

hipError_t launch_up_project_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  dim3 grid(a.h, kDh / 64);
  if (a.out_bf16)
    launch_kernel(up_project_bf16_kernel<true>, grid, dim3(256), s,
                       static_cast<const uint16_t*>(a.w_uv), static_cast<const uint16_t*>(a.c_bar),
                       a.out, rows, a.h);
  else
    launch_kernel(up_project_bf16_kernel<false>, grid, dim3(256), s,
                       static_cast<const uint16_t*>(a.w_uv), static_cast<const uint16_t*>(a.c_bar),
                       a.out, rows, a.h);
  return hipGetLastError();
}

}  // namespace mla
