// kernels.h -- internal launch interface between the host plan and the
// gfx950 kernels.  Not part of the public C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Everything the four steps of one decode call need, already validated.
struct DecodeArgs {
  int batch, n_q, h, d_c, d_r, d_h;
  int page_size, max_pages, num_pages, max_len;
  int splits;      // chunks per sequence (S) of a fixed chunking
  int chunk_len;   // tokens per chunk of a fixed chunking
  // Fast path: chunk results are stored per global chunk, [chunks][n_q][h]
  // [d_c].  planned = 0: chunk g is chunk g % splits of sequence g / splits
  // (chunks = batch * splits).  planned = 1: the chunk length and every
  // sequence's chunks come from the context lengths on the device
  // (chunk_plan.h: about plan_target chunks in all, lengths within
  // [plan_min_chunk, plan_max_chunk]); chunks bounds their number.
  int planned = 0;
  int chunks = 0;
  int plan_target = 0, plan_min_chunk = 0, plan_max_chunk = 0;
  int in_bf16;     // storage type of q, q_r, caches, weights
  int out_bf16;    // storage type of o
  float scale_log2;  // softmax scale * log2(e)

  const void* q;
  const void* q_r;
  const void* latent_pool;
  const void* rope_pool;
  const int32_t* page_table;
  const int32_t* context_lens;
  const void* w_uk;
  const void* w_uv;
  void* out;

  // workspace carve-up
  void* q_abs;      // [R][h][d_c]      bf16 (fast path) or f32 (general path)
  void* part_o;     // chunk results already normalised: bf16 [chunks][n_q][h]
                    // [d_c] (fast path) or f32 [R][S][h][d_c] (general path)
  float* part_lse;  // f32 base-2 log-sum-exp of each chunk result, same order
  void* c_bar;      // [R][h][d_c]      f32 (general path only)
};

// Where a kernel is launched.  With both events set, the launch records
// the kernel's own start and end (the dispatch's timestamps) into them, so
// that per-kernel times exclude the gaps between launches.
struct LaunchCtx {
  hipStream_t stream = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, dim3 grid, dim3 block, const LaunchCtx& c, Args... args) {
  if (c.start && c.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, c.stream, c.start, c.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, c.stream, args...);
}

// Heads handled by one work-group of the fast split kernel.
constexpr int kFastHeadsPerGroup = 64;
// Tokens staged per LDS tile in the fast split kernel.
constexpr int kFastTile = 32;
// Largest chunk (in tiles) the fast split kernel accepts: it keeps the pool
// row of every tile of its chunk in LDS.
constexpr int kMaxFastChunkTiles = 1024;

// Fast path: bf16 storage, d_c = 512, d_r = 64, d_h = 128, h % 64 == 0,
// page_size % 32 == 0.
hipError_t launch_q_absorb_bf16(const DecodeArgs& a, const LaunchCtx& s);
hipError_t launch_split_attn_bf16(const DecodeArgs& a, const LaunchCtx& s);
// Chunk merge and W_UV up-projection in one kernel.
hipError_t launch_finish_bf16(const DecodeArgs& a, const LaunchCtx& s);

// General path: any dims (d_c <= 1024), f32 or bf16 storage, f32 math.
hipError_t launch_q_absorb_general(const DecodeArgs& a, const LaunchCtx& s);
hipError_t launch_split_attn_general(const DecodeArgs& a, const LaunchCtx& s);
hipError_t launch_up_project_general(const DecodeArgs& a, const LaunchCtx& s);

// Log-sum-exp merge of the f32 chunk results into c_bar (general path).
hipError_t launch_combine_general(const DecodeArgs& a, const LaunchCtx& s);

}  // namespace mla
