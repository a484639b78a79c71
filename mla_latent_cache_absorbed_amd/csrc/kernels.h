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
inline void launch_kernel_lds(Kernel kernel, dim3 grid, dim3 block, size_t lds_bytes, const LaunchCtx& c,
                              Args... args) {
  if (c.start && c.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, c.stream, c.start, c.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, c.stream, args...);
}

template <typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, dim3 grid, dim3 block, const LaunchCtx& c, Args... args) {
  launch_kernel_lds(kernel, grid, block, 0, c, args...);
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

// Output projection u = [o_1; ...; o_h] W^O of `rows` query rows (oproj.hip).
struct OprojLaunch {
  const void* o;  // [rows][k], k = h d_h
  const void* w;  // [d][k] (W^O transposed)
  void* part;     // fp32 slice partials (oproj_workspace_bytes), may be null when that is 0
  void* u;        // [rows][d]
  int rows = 0, k = 0, d = 0;
  bool in_bf16 = true, out_bf16 = true;
};
// The MFMA kernels apply (bf16 storage, d % 64 == 0, k % 512 == 0).
bool oproj_fast_applies(int k, int d, bool bf16);
// Slices of k (a power of two) the MFMA kernels split the product into.
int oproj_splits(int rows, int k, int d);
// fp32 partial bytes the launch needs in OprojLaunch::part (0: none).
size_t oproj_workspace_bytes(int rows, int k, int d, bool bf16);
hipError_t launch_oproj(const OprojLaunch& p, const LaunchCtx& s);
// The same MFMA product on x [rows][k] (bf16) and the stacked weights
// [w0 ([d0][k]); w1 ([d - d0][k])], both bf16 with d0 and d multiples of 64
// (and oproj_fast_applies(k, d, true)): writes the fp32 slice partials
// [oproj_splits(rows, k, d)][rows][d] into part, for a caller's own finish.
hipError_t launch_proj_partial(const void* x, const void* w0, const void* w1, int rows, int k, int d, int d0,
                               float* part, const LaunchCtx& s);

// The cache append of a step (rope_proj.hip): c = W_DKV x and
// k_R = RoPE(W_KR x, pos) of each new token into its pool rows.
struct AppendLaunch {
  const void* x;      // [rows][d_model]
  const void* w_dkv;  // [d_c][d_model]
  const void* w_kr;   // [d_r][d_model]
  int rows = 0, d_model = 0, d_c = 0, d_r = 0;
  const int32_t* seq;         // [rows]
  const int32_t* pos;         // [rows]
  const int32_t* page_table;  // [batch][max_pages]
  int max_pages = 0, page_size = 0, num_pages = 0;
  void* latent_pool;  // [num_pages][page_size][d_c]
  void* rope_pool;    // [num_pages][page_size][d_r]
  const double* theta;  // [d_r / 2] RoPE frequencies, or null: base^(-2j/d_r)
  double base = 10000.0;
  bool bf16 = true;
  void* work;  // cache_append_workspace_bytes
};
bool cache_append_fast(int d_model, int d_c, int d_r, bool bf16);
size_t cache_append_workspace_bytes(int rows, int d_model, int d_c, int d_r, bool bf16);
hipError_t launch_cache_append(const AppendLaunch& p, const LaunchCtx& s);

// The query side of a step (rope_proj.hip): c_Q = W_DQ x, q_i = W_UQ[i] c_Q,
// q_R,i = RoPE(W_QR[i] c_Q, pos).
struct QueryLaunch {
  const void* x;     // [rows][d_model]
  const void* w_dq;  // [d_qc][d_model]
  const void* w_uq;  // [h d_h][d_qc]
  const void* w_qr;  // [h d_r][d_qc]
  int rows = 0, d_model = 0, d_qc = 0, h = 0, d_h = 0, d_r = 0;
  const int32_t* pos;  // [rows]
  void* q;             // [rows][h][d_h]
  void* q_r;           // [rows][h][d_r]
  const double* theta;
  double base = 10000.0;
  bool bf16 = true;
  void* work;  // query_project_workspace_bytes: c_Q, then the fp32 partials
};
size_t query_project_workspace_bytes(int rows, int d_model, int d_qc, int h, int d_h, int d_r, bool bf16);
hipError_t launch_query_project(const QueryLaunch& p, const LaunchCtx& s);

// The cache append and the query side of the same rows (rope_proj.hip; x,
// rows, pos, theta and the workspace are the same in both): up to four
// rows the first stages share one launch, [W_DKV; W_KR; W_DQ] x, so that x
// and the launch are paid once; otherwise the two calls in turn.
bool token_project_fused(int rows, int d_model, int d_c, int d_r, int d_qc, int h, int d_h, bool bf16);
size_t token_project_workspace_bytes(int rows, int d_model, int d_c, int d_r, int d_qc, int h, int d_h, bool bf16);
hipError_t launch_token_project(const AppendLaunch& ap, const QueryLaunch& qp, const LaunchCtx& s);

// Prefill attention over a prompt of T tokens (prefill.hip): K and V rebuilt
// from the latents, then causal attention over d_h + d_r dims.
struct PrefillLaunch {
  const void* latent;  // [T][d_c]
  const void* rope;    // [T][d_r] (rotated)
  const void* q;       // [T][h][d_h]
  const void* q_r;     // [T][h][d_r]
  const void* w_uk;    // [h][d_h][d_c]
  const void* w_uv;    // [h][d_h][d_c]
  void* out;           // [T][h][d_h]
  int T = 0, h = 0, d_c = 0, d_r = 0, d_h = 0;
  float scale = 0.f;
  bool bf16 = true, out_bf16 = true;
  void* work;  // prefill_workspace_bytes: K then V, [T][h][d_h] each
};
bool prefill_fast(int d_c, int d_r, int d_h, bool bf16);
size_t prefill_workspace_bytes(int T, int h, int d_h, bool bf16);
hipError_t launch_prefill(const PrefillLaunch& p, const LaunchCtx& s);

}  // namespace mla
