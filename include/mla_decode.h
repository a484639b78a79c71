/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) absorbed-weight MLA decode
 * library, libmla_decode.so.
 *
 * One decode step of Multi-head Latent Attention over a compressed KV cache,
 * in absorbed-weight form ("MLA, dim by dim", sections 4.2 and 5.2; "From
 * Vanilla Transformers to Modern LLMs ... Part 3", sections 3.e.2, 3.g, 3.o
 * and 3.p; "Multi-Head Latent Attention: Low-Rank KV Compression, Decoupled
 * RoPE, and Matrix Absorption", section "Matrix Absorption").  For query row
 * r = (sequence b, new token m) and head i:
 *
 *   q_abs   = W_UK[i]^T q[r,i]                                   (absorb)
 *   s_t     = scale * (q_abs . C_b[t] + q_R[r,i] . K_R,b[t])     (score)
 *   p       = softmax over the visible tokens t = 0 .. L_b - n_q + m
 *   c_bar   = sum_t p_t C_b[t]                                   (latent sum)
 *   o[r,i]  = W_UV[i] c_bar                                      (up-project)
 *
 * Per-head keys and values are never formed.  C_b is the latent cache of
 * sequence b (d_c values per token) and K_R,b the shared RoPE key cache (d_r
 * values per token, already rotated, one key for all heads).  The context is
 * split into chunks that are reduced separately and merged with a
 * log-sum-exp combine.
 *
 * Conventions
 *   - All device buffers are caller-owned (typically torch tensors); the
 *     library owns only the opaque host-side plan.  `run` never allocates,
 *     frees or synchronises: it enqueues its kernels on the caller's stream
 *     (three on the bf16 fast path, where the merge and the up-projection
 *     are one kernel; four on the general path) and returns.
 *   - Layouts are dense row-major with the listed shapes.  Weights act on
 *     column vectors: k = W_UK[i] c, with W[i] a d_h x d_c matrix.
 *   - `context_lens[b]` counts every cached token of sequence b, including
 *     its n_q new tokens; new token m of sequence b attends to tokens
 *     0 .. L_b - n_q + m (a causal diagonal over the last n_q tokens).
 *   - Token t of sequence b is row t % page_size of pool page
 *     page_table[b][t / page_size].  A contiguous cache is a pool whose
 *     table lists its pages in order.
 *   - Shapes must satisfy the dimension-compatibility rule of matrix
 *     products ("Mathematical Prerequisites for DeepSeek-V2", section 1);
 *     violations are reported before any launch.
 *
 * Errors: every entry point returns a status; negative values are failures.
 * Argument errors are found on the host before any work is enqueued and
 * leave the stream untouched.  A failed launch returns MLA_ERR_HIP.  Faults
 * inside a kernel surface at the caller's next synchronisation.  The text of
 * the last failure on the calling thread is available from
 * mla_decode_last_error().
 *
 * Device-side safety: page ids are clamped into [0, num_pages) and lengths
 * into [0, max_context_len] inside the kernels, so malformed device-side
 * tables give wrong numbers but never an out-of-bounds access.  This is why
 * `run` takes the pool's page count (num_pages) beside the problem's own
 * arguments.
 *
 * Thread safety: a plan is immutable after mla_decode_create, except for
 * its optional timing record: `run` takes the next timing slot with an
 * atomic increment.  Concurrent runs on one plan (from several threads, on
 * several streams) are legal when their workspaces (and outputs) are
 * distinct.  mla_decode_enable_timing, mla_decode_read_timing(_runs) and
 * mla_decode_destroy must not overlap any other call on the same plan.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mla_decode_plan* mla_decode_t; /* opaque; owned by the library */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* a null pointer, a non-positive size, a bad enum */
  MLA_ERR_UNSUPPORTED = -2, /* valid request this build does not implement    */
  MLA_ERR_WORKSPACE = -3,   /* workspace smaller than mla_decode_workspace_size */
  MLA_ERR_HIP = -4,         /* the HIP runtime reported an error               */
  MLA_ERR_NOMEM = -5        /* host allocation of the plan failed              */
} mla_status_t;

typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_F32 = 1 } mla_dtype_t;

typedef struct {
  int32_t h;                 /* query heads                                     */
  int32_t d_c;               /* latent width (KV compression dimension)         */
  int32_t d_r;               /* decoupled RoPE width (0 allowed on the f32 path)*/
  int32_t d_h;               /* per-head width of q, keys, values and o         */
  int32_t dtype;             /* mla_dtype_t of q, q_r, caches and weights       */
  int32_t out_dtype;         /* mla_dtype_t of o; -1 = same as dtype            */
  int32_t page_size;         /* tokens per cache page                           */
  int32_t max_batch;         /* largest batch a run may pass                    */
  int32_t max_q_per_seq;     /* largest n_q a run may pass                      */
  int32_t max_pages_per_seq; /* row stride of page_table                        */
  int32_t num_splits;        /* 0 = automatic; > 0 forces the chunk count       */
  float scale;               /* 0 = 1/sqrt(d_h + d_r)                           */
} mla_decode_config_t;

/* Validates the configuration and builds a plan (host only, no device work).
 * The dimensions are those of the pages' problem statement: h heads, latent
 * width d_c, decoupled RoPE width d_r and per-head width d_h ("MLA, dim by
 * dim" section 5.2, the per-head query, key and value shapes); a shape that
 * no kernel can take is refused here ("Mathematical Prerequisites for
 * DeepSeek-V2" section 1, the dimension-compatibility rule of products).
 * On success *out_plan owns a plan to release with mla_decode_destroy. */
mla_status_t mla_decode_create(const mla_decode_config_t* cfg, mla_decode_t* out_plan);

/* Bytes of device workspace `run` needs for this batch shape (0 on an
 * invalid request; the reason is in mla_decode_last_error()).  The
 * workspace holds the absorbed queries (W_UK[i]^T q, "Mathematical
 * Prerequisites for DeepSeek-V2" section 6) and the per-chunk partial
 * results and log-sum-exps (and, on the general path, the merged latents). */
size_t mla_decode_workspace_size(mla_decode_t plan, int32_t batch, int32_t n_q,
                                 int32_t max_context_len);

/* Chunking the plan would use for this batch shape: number of chunks per
 * sequence and tokens per chunk.  Host only; lets callers and tests see the
 * split decision.  (0, 0) means that the chunking is decided on the device
 * from the context lengths: on the bf16 fast path with several sequences and
 * no forced count, one chunk length is chosen for the call so that the
 * chunks of all sequences (a long sequence gets more, a short one fewer)
 * fill the GPU evenly. */
mla_status_t mla_decode_split_plan(mla_decode_t plan, int32_t batch, int32_t n_q,
                                   int32_t max_context_len, int32_t* num_splits,
                                   int32_t* chunk_len);

/* Enqueues one decode step on `stream` (a hipStream_t; NULL = the null
 * stream): the absorbed-weight decode of "MLA, dim by dim" section 5.2 (the
 * cached decode chains: scores against the latent and the shared RoPE key
 * cache, softmax over the visible tokens, latent sum, up-projection) and
 * "From Vanilla Transformers to Modern LLMs ... Part 3" sections 3.e.2 to
 * 3.p.  The arguments are that problem's: queries q and q_R, the latent and
 * RoPE caches (here paged), W_UK, W_UV and the context lengths.  Every
 * pointer is device memory:
 *   q            [batch][n_q][h][d_h]         dtype
 *   q_r          [batch][n_q][h][d_r]         dtype, already rotated
 *   latent_pool  [num_pages][page_size][d_c]  dtype
 *   rope_pool    [num_pages][page_size][d_r]  dtype, already rotated
 *   page_table   [batch][max_pages_per_seq]   int32
 *   context_lens [batch]                      int32, each in [n_q, max_context_len]
 *   w_uk, w_uv   [h][d_h][d_c]                dtype
 *   out          [batch][n_q][h][d_h]         out_dtype (written)
 *   workspace    >= mla_decode_workspace_size(plan, batch, n_q, max_context_len)
 *                bytes, 256-byte aligned, contents need not be initialised.
 * max_context_len bounds every context_lens entry and must fit the table:
 * max_context_len <= max_pages_per_seq * page_size. */
mla_status_t mla_decode_run(mla_decode_t plan, int32_t batch, int32_t n_q,
                            int32_t max_context_len, int32_t num_pages,
                            const void* q, const void* q_r,
                            const void* latent_pool, const void* rope_pool,
                            const int32_t* page_table, const int32_t* context_lens,
                            const void* w_uk, const void* w_uv, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * decode step as mla_decode_run, same arguments minus the workspace, with
 * the workspace taken from a static array in the library's device code
 * (64 MiB per GPU, held until the process ends; its device address is
 * looked up once per device).  It calls no hipMalloc, hipFree or other
 * allocating routine.  A call whose workspace (mla_decode_workspace_size)
 * exceeds 64 MiB is refused with MLA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU uses that GPU's one array: calls that
 * overlap on a GPU (other streams, other threads, other plans) race and
 * must be serialised by the caller.  Nothing in the array needs to start
 * at zero: every byte a step reads was written earlier in the same step. */
mla_status_t mla_decode_run_static(mla_decode_t plan, int32_t batch, int32_t n_q,
                                   int32_t max_context_len, int32_t num_pages,
                                   const void* q, const void* q_r,
                                   const void* latent_pool, const void* rope_pool,
                                   const int32_t* page_table, const int32_t* context_lens,
                                   const void* w_uk, const void* w_uv, void* out, void* stream);

/* Per-kernel timing (instrumentation, off by default; not part of the
 * method).  With max_runs > 0
 * every later `run` on this plan launches each of its kernels (absorb,
 * split, combine, up-project) with a start and a stop HIP event that the
 * dispatch itself fills in (the kernel's own begin and end, as a profiler
 * sees them, not the gaps between launches), for up to max_runs runs;
 * max_runs = 0 turns it off.
 * Creates the events on the current device; allocates no device memory. */
mla_status_t mla_decode_enable_timing(mla_decode_t plan, int32_t max_runs);

/* Waits for the recorded events, writes the summed milliseconds of each of
 * the four steps over the recorded runs into ms[0..3] and the number of runs
 * into *runs, then starts a new recording.  On the bf16 fast path the chunk
 * merge and the up-projection run as one kernel, reported in ms[2]; ms[3]
 * is then 0. */
mla_status_t mla_decode_read_timing(mla_decode_t plan, float* ms, int32_t* runs);

/* Per-run variant of mla_decode_read_timing: writes the milliseconds of
 * each of the four steps of each recorded run, ms[4 r + k] for run r <
 * *runs <= max_runs (a step the path does not launch reads 0), then starts
 * a new recording. */
mla_status_t mla_decode_read_timing_runs(mla_decode_t plan, float* ms, int32_t max_runs,
                                         int32_t* runs);

/* The output projection that follows the decode step: for each of `rows`
 * query rows, the h head outputs of `run` (o[r][i][:], d_h values each) are
 * concatenated head after head into k = h * d_h values and multiplied by
 * W^O, u[r] = [o[r][0]; ...; o[r][h-1]] W^O ("From Vanilla Transformers to
 * Modern LLMs ... Part 3" sections 3.h and 3.p; the W^O product of the
 * "Matrix Absorption" section of "Multi-Head Latent Attention: Low-Rank KV
 * Compression, Decoupled RoPE, and Matrix Absorption").  Every pointer is
 * device memory:
 *   o    [rows][k]        dtype (the output of `run`, [batch][n_q][h][d_h],
 *                          is this with rows = batch * n_q)
 *   w_o  [d_model][k]     dtype: W^O transposed (each output feature's k
 *                          weights contiguous; the pages' W^O is k x d_model)
 *   u    [rows][d_model]  out_dtype (-1 = dtype)
 *   workspace             mla_oproj_workspace_size bytes (fp32 partial sums
 *                          over slices of k; 0 bytes, and NULL allowed, when
 *                          it returns 0), 256-byte aligned, caller-owned
 * bf16 storage with d_model % 64 == 0 and k % 512 == 0 runs with fp32
 * accumulation (16-byte aligned o, w_o and u required): up to four rows in
 * one launch with bf16 dot products and no workspace (x within 40 KB for
 * three or four rows), more rows on MFMA over slices of k; other shapes
 * and fp32 storage on a plain fp32 kernel.  The result does not depend on
 * timing (partials are summed in a fixed order).  Enqueued on `stream`
 * (a hipStream_t, NULL = the null stream); no allocation, no
 * synchronisation.  Argument errors return a negative status before any
 * launch, with text from mla_decode_last_error(). */
size_t mla_oproj_workspace_size(int32_t rows, int32_t k, int32_t d_model, int32_t dtype);
mla_status_t mla_oproj_run(int32_t rows, int32_t k, int32_t d_model, int32_t dtype, int32_t out_dtype,
                           const void* o, const void* w_o, void* u, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The cache append of one decode step, before `run` reads the cache: for
 * each of `rows` new tokens, with hidden state x[r] (d_model values),
 * sequence seq[r] and position pos[r] (0-based), the latent
 * c = W_DKV x[r] and the decoupled RoPE key k_R = RoPE(W_KR x[r], pos[r])
 * are written into row pos % page_size of page
 * page_table[seq][pos / page_size] of latent_pool and rope_pool
 * ("Multi-Head Latent Attention: Low-Rank KV Compression, Decoupled RoPE,
 * and Matrix Absorption", section "MLA: Low-Rank Key-Value Joint
 * Compression"; "MLA, dim by dim" section 5.2, the shared RoPE key cached
 * after rotation; "From Vanilla Transformers to Modern LLMs ... Part 3"
 * sections 3.b and 3.k).  RoPE turns adjacent pairs (y_2j, y_2j+1) by the
 * angle pos * theta_j, theta_j = rope_theta[j] when rope_theta (device,
 * d_r / 2 doubles) is given, else rope_base^(-2 j / d_r) ("MLA, dim by
 * dim", RoPE paragraph of section 4); angles are formed in fp64.  Device
 * memory, all in `dtype` unless noted:
 *   x        [rows][d_model]
 *   w_dkv    [d_c][d_model]   (acting on column vectors: c = W_DKV x)
 *   w_kr     [d_r][d_model]
 *   seq, pos [rows] int32;  page_table [batch][max_pages_per_seq] int32
 *   latent_pool [num_pages][page_size][d_c], rope_pool [num_pages][page_size][d_r]
 *   workspace   mla_cache_append_workspace_size bytes (NULL when 0), 256-byte aligned
 * A row whose position or page lies outside the table or the pool is not
 * written.  bf16 with d_model % 512 == 0 and d_c, d_r multiples of 64 runs
 * the fast kernels (16-byte aligned tensors): up to four rows one launch
 * with no workspace, more rows MFMA over slices of k; other shapes and
 * fp32 on a plain kernel.  Rows that write the same pool row race.  Enqueued on `stream`;
 * no allocation, no synchronisation; argument errors return a negative
 * status before any launch. */
size_t mla_cache_append_workspace_size(int32_t rows, int32_t d_model, int32_t d_c, int32_t d_r, int32_t dtype);
mla_status_t mla_cache_append_run(int32_t rows, int32_t d_model, int32_t d_c, int32_t d_r, int32_t dtype,
                                  const void* x, const void* w_dkv, const void* w_kr,
                                  const int32_t* seq, const int32_t* pos, const int32_t* page_table,
                                  int32_t max_pages_per_seq, int32_t page_size, int32_t num_pages,
                                  void* latent_pool, void* rope_pool, const double* rope_theta,
                                  double rope_base, void* workspace, size_t workspace_bytes, void* stream);

/* The query side of one decode step: for each of `rows` query rows with
 * hidden state x[r] and position pos[r], the query latent c_Q = W_DQ x
 * (d_qc values), then per head i the content query q[r][i] = W_UQ[i] c_Q
 * and the RoPE query q_r[r][i] = RoPE(W_QR[i] c_Q, pos[r]) (the query
 * down-projection and per-head up-projections of "Multi-Head Latent
 * Attention: ..."; "MLA, dim by dim" section 4.3, in the order
 * (x W_DQ) W_UQ, and 5.2; "From Vanilla Transformers ..." sections 3.d and
 * 3.l) -- the q and q_r that `run` takes.  Device memory in `dtype`:
 *   x [rows][d_model]; w_dq [d_qc][d_model]; w_uq [h][d_h][d_qc];
 *   w_qr [h][d_r][d_qc]; pos [rows] int32;
 *   q [rows][h][d_h]; q_r [rows][h][d_r];
 *   workspace mla_query_project_workspace_size bytes, 256-byte aligned
 *   (c_Q, kept in dtype -- bf16 rounds it to nearest even as the next
 *   product's operand -- and fp32 partial sums).
 * RoPE as for mla_cache_append_run.  bf16 with d_model and d_qc multiples of
 * 512 and d_qc, h * d_h, h * d_r multiples of 64 runs the fast kernels (one
 * launch per stage up to four rows, MFMA over slices of k beyond); other
 * shapes and fp32 on plain kernels.  Enqueued on `stream`; no allocation, no
 * synchronisation; argument errors return a negative status before any
 * launch. */
size_t mla_query_project_workspace_size(int32_t rows, int32_t d_model, int32_t d_qc, int32_t h, int32_t d_h,
                                        int32_t d_r, int32_t dtype);
mla_status_t mla_query_project_run(int32_t rows, int32_t d_model, int32_t d_qc, int32_t h, int32_t d_h,
                                   int32_t d_r, int32_t dtype, const void* x, const void* w_dq,
                                   const void* w_uq, const void* w_qr, const int32_t* pos, void* q,
                                   void* q_r, const double* rope_theta, double rope_base, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Both projections of the current tokens in one call: the cache append of
 * mla_cache_append_run and the query side of mla_query_project_run for
 * the same rows, hidden states x and positions pos (the latent, the RoPE
 * key and the query latent all read x: "Multi-Head Latent Attention: ...",
 * sections "MLA: Low-Rank Key-Value Joint Compression" and on the query
 * compression; "MLA, dim by dim" sections 4.3 and 5.2).  Arguments as in
 * those two calls (one rope_theta / rope_base for keys and queries);
 * workspace mla_token_project_workspace_size bytes, 256-byte aligned.  Up
 * to four rows of bf16 with the fast shapes, the first stages share one
 * launch ([W_DKV; W_KR; W_DQ] x) and the call makes two launches in all;
 * otherwise it runs the two calls in turn, with the same results.  Rows
 * whose page lies outside the table or the pool are not written to the
 * pools; their queries are.  Enqueued on `stream`; no allocation, no
 * synchronisation; argument errors return a negative status before any
 * launch. */
size_t mla_token_project_workspace_size(int32_t rows, int32_t d_model, int32_t d_c, int32_t d_r, int32_t d_qc,
                                        int32_t h, int32_t d_h, int32_t dtype);
mla_status_t mla_token_project_run(int32_t rows, int32_t d_model, int32_t d_c, int32_t d_r, int32_t d_qc,
                                   int32_t h, int32_t d_h, int32_t dtype, const void* x, const void* w_dkv,
                                   const void* w_kr, const void* w_dq, const void* w_uq, const void* w_qr,
                                   const int32_t* seq, const int32_t* pos, const int32_t* page_table,
                                   int32_t max_pages_per_seq, int32_t page_size, int32_t num_pages,
                                   void* latent_pool, void* rope_pool, void* q, void* q_r,
                                   const double* rope_theta, double rope_base, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Prefill: attention over a whole prompt of T tokens, each attending to
 * itself and the tokens before it, in the order the pages derive for many
 * queries ("MLA, dim by dim" section 4.1): the per-head keys and values are
 * rebuilt from the latents, k_t,i = W_UK[i] c_t and v_t,i = W_UV[i] c_t,
 * and the scores contract over d_h + d_r dimensions,
 * s(t, u) = scale [q_t,i; q_R,t,i] . [k_u,i; k_R,u] for u <= t, then
 * o_t,i = sum_u softmax(s) v_u,i (section 5.1 of the same page for the
 * decoupled RoPE part).  scale 0 = 1 / sqrt(d_h + d_r).  Device memory in
 * `dtype` (out in out_dtype, -1 = dtype):
 *   latent [T][d_c]; rope [T][d_r] (already rotated); q [T][h][d_h];
 *   q_r [T][h][d_r]; w_uk, w_uv [h][d_h][d_c]; out [T][h][d_h];
 *   workspace mla_prefill_workspace_size bytes, 256-byte aligned (the
 *   rebuilt K and V, [T][h][d_h] each, in dtype).
 * bf16 with d_h = 128, d_r = 64 and d_c % 64 == 0 runs on MFMA (16-byte
 * aligned tensors); other shapes and fp32 on plain kernels (meant for small
 * problems).  Enqueued on `stream`; no allocation, no synchronisation;
 * argument errors return a negative status before any launch. */
size_t mla_prefill_workspace_size(int32_t T, int32_t h, int32_t d_h, int32_t dtype);
mla_status_t mla_prefill_run(int32_t T, int32_t h, int32_t d_c, int32_t d_r, int32_t d_h, int32_t dtype,
                             int32_t out_dtype, float scale, const void* latent, const void* rope,
                             const void* q, const void* q_r, const void* w_uk, const void* w_uv, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Releases a plan.  NULL is accepted and ignored. */
void mla_decode_destroy(mla_decode_t plan);

/* Text of the last failure on the calling thread ("" when none). */
const char* mla_decode_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
