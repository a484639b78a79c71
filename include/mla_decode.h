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
 * tables give wrong numbers but never an out-of-bounds access.
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
 * On success *out_plan owns a plan to release with mla_decode_destroy. */
mla_status_t mla_decode_create(const mla_decode_config_t* cfg, mla_decode_t* out_plan);

/* Bytes of device workspace `run` needs for this batch shape (0 on an
 * invalid request; the reason is in mla_decode_last_error()).  The
 * workspace holds the absorbed queries and the per-chunk partial results
 * and log-sum-exps (and, on the general path, the merged latents). */
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
 * stream).  Every pointer is device memory:
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

/* Per-kernel timing (instrumentation, off by default).  With max_runs > 0
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

/* Releases a plan.  NULL is accepted and ignored. */
void mla_decode_destroy(mla_decode_t plan);

/* Text of the last failure on the calling thread ("" when none). */
const char* mla_decode_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
