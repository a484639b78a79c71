// q_absorb.hip -- query absorption: q_abs[r, i, :] = W_UK[i]^T q[r, i, :],
// as a kernel of its own (fast path).
//
// Moves the key up-projection from every cached token onto the one new
// query (the bilinear identity, "Mathematical Prerequisites for DeepSeek-V2"
// section 6; the absorbed query of "MLA, dim by dim" section 5.1).  Cost per
// query row: 2 h d_h d_c FLOPs, independent of the context length.
//
// One work-group of four waves per (head, 128 latent columns): the slice of
// W_UK[i] streams from HBM once into LDS and meets every query row there
// (absorb_tile.h).
#include "absorb_tile.h"
#include "kernels.h"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void q_absorb_bf16_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_abs, int rows,
                                                            int h, int d_c) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[absorb::kTileBytes];  // 32 KB

  const int head = blockIdx.x;
  const int c0 = blockIdx.y * absorb::kCols;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  absorb::load_tile((uint32_t)(uintptr_t)((AS3 uint8_t*)tile), w_uk + (size_t)head * absorb::kDh * d_c, c0,
                    d_c, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  absorb::compute_tile((const AS3 uint8_t*)tile, q, q_abs, head, c0, rows, h, d_c, wave, lane);
}

}  // namespace

hipError_t launch_q_absorb_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  dim3 grid(a.h, a.d_c / absorb::kCols);
  launch_kernel(q_absorb_bf16_kernel, grid, dim3(256), s, static_cast<const uint16_t*>(a.q),
                static_cast<const uint16_t*>(a.w_uk), static_cast<uint16_t*>(a.q_abs), rows, a.h, a.d_c);
  return hipGetLastError();
}

}  // namespace mla
