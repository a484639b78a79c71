// decode.cpp -- host side of the C ABI in include/mla_decode.h.
//
// Validates configurations and calls, chooses how the context is split into
// chunks (or that the kernels plan it from the context lengths), carves the
// caller's workspace, and enqueues the kernels on the caller's stream: three
// on the bf16 fast path, four on the general path.  It never allocates device
// memory and never synchronises.
#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"

constexpr int kKernels = 4;  // absorb, split, combine, up-project
constexpr int kEventsPerRun = 2 * kKernels;

struct mla_decode_plan {
  mla_decode_config_t cfg;
  int out_dtype;   // resolved (never -1)
  bool fast;       // bf16 MFMA kernels apply
  float scale;     // resolved softmax scale
  int num_cus;     // compute units the split heuristic fills
  // optional per-kernel timing: a start and a stop event per kernel per
  // recorded run, filled in by the launches themselves
  std::vector<hipEvent_t> events;
  int timing_capacity = 0;
  int timing_runs = 0;
};

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

// A chunk is never shorter than this many tokens unless the context is:
// each chunk writes h * d_c * 4 bytes of partial result, which must stay
// small next to the chunk's own cache bytes ((d_c + d_r) * 2 per token).
constexpr int kMinChunkTokens = 128;
// Work-groups per CU the split kernel is sized for.
constexpr int kGroupsPerCu = 1;

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

bool fast_path_applies(const mla_decode_config_t& c) {
  return c.dtype == MLA_DTYPE_BF16 && c.d_c == 512 && c.d_r == 64 && c.d_h == 128 &&
         c.h % mla::kFastHeadsPerGroup == 0 && c.page_size % mla::kFastTile == 0;
}

int query_num_cus() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return 256;  // MI355X
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

struct Split {
  int splits, chunk_len;  // fixed chunking: chunks per sequence, tokens per chunk
  // fast path: chunk results are stored per global chunk; `planned`: the
  // chunking is decided on the device from the context lengths (about
  // `target` chunks in all), `chunks` bounds their number
  bool planned = false;
  int chunks = 0, target = 0;
};

// Longest chunk of a planned chunking (the fast split kernel's tile table).
constexpr int kMaxPlannedChunk = mla::kMaxFastChunkTiles * mla::kFastTile;

// Chunks per sequence: enough work-groups to fill the CUs, but chunks no
// shorter than kMinChunkTokens; a forced count from the config wins.
Split plan_splits(const mla_decode_plan& p, int batch, int n_q, int max_len) {
  const int gran = p.fast ? mla::kFastTile : 1;
  const int groups_per_chunk = n_q * (p.fast ? p.cfg.h / mla::kFastHeadsPerGroup : p.cfg.h);
  int s;
  if (p.cfg.num_splits > 0) {
    s = p.cfg.num_splits;
  } else {
    const int target = kGroupsPerCu * p.num_cus;
    const int want = ceil_div(target, (long long)std::max(1, batch) * groups_per_chunk);
    const int cap = std::max(1, ceil_div(max_len, kMinChunkTokens));
    s = std::min(std::max(want, 1), cap);
  }
  s = std::min(std::max(s, 1), std::max(1, ceil_div(max_len, gran)));
  if (p.fast)  // the fast split kernel keeps at most kMaxFastChunkTiles tiles per chunk
    s = std::max(s, ceil_div(max_len, (long long)mla::kMaxFastChunkTiles * mla::kFastTile));
  Split r;
  r.chunk_len = ceil_div(ceil_div(max_len, s), gran) * gran;
  r.splits = std::max(1, ceil_div(max_len, r.chunk_len));
  r.chunks = batch * r.splits;
  // Several sequences of unknown (possibly very different) lengths: one
  // chunk length for the call, chosen on the device from the actual lengths
  // so that every work-group gets about the same number of tiles.  Worth its
  // extra dependent load (the lengths before the page table, and again in
  // the merge) when a sequence gets more than two chunks on average; with
  // fewer, the fixed chunking keeps the work-groups of equal-length
  // sequences just as even.
  if (p.fast && p.cfg.num_splits == 0 && batch > 1) {
    const int target = std::max(1, kGroupsPerCu * p.num_cus / groups_per_chunk);
    if (target > 2 * batch) {
      r.planned = true;
      r.target = target;
      // the device's choice keeps the count within the target, unless the
      // chunk length reaches its maximum (then n <= total / max + batch)
      r.chunks = std::max(target, batch + ceil_div((long long)batch * max_len, kMaxPlannedChunk));
    }
  }
  return r;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t q_abs, part_o, part_lse, c_bar, total;
};

Layout layout_for(const mla_decode_plan& p, int batch, int n_q, const Split& sp) {
  const size_t R = (size_t)batch * n_q, h = p.cfg.h, d_c = p.cfg.d_c;
  const size_t inter = p.fast ? 2 : 4;  // bytes per q_abs / partial / c_bar element
  // chunk results: [chunks][n_q] rows on the fast path, [R][S] otherwise
  const size_t parts = p.fast ? (size_t)sp.chunks * n_q : R * sp.splits;
  Layout l;
  l.q_abs = 0;
  l.part_o = l.q_abs + align256(R * h * d_c * inter);
  l.part_lse = l.part_o + align256(parts * h * d_c * inter);
  l.c_bar = l.part_lse + align256(parts * h * 4);
  // the fast path merges the chunks straight into the up-projection
  l.total = l.c_bar + (p.fast ? 0 : align256(R * h * d_c * inter));
  return l;
}

mla_status_t check_shape(const mla_decode_plan* p, int32_t batch, int32_t n_q,
                         int32_t max_context_len) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  const mla_decode_config_t& c = p->cfg;
  if (batch < 0 || batch > c.max_batch)
    return fail(MLA_ERR_INVALID_ARG, "batch %d outside [0, max_batch=%d]", batch, c.max_batch);
  if (n_q < 1 || n_q > c.max_q_per_seq)
    return fail(MLA_ERR_INVALID_ARG, "n_q %d outside [1, max_q_per_seq=%d]", n_q, c.max_q_per_seq);
  const long long cap = (long long)c.max_pages_per_seq * c.page_size;
  if (max_context_len < n_q || max_context_len > cap)
    return fail(MLA_ERR_INVALID_ARG,
                "max_context_len %d outside [n_q=%d, max_pages_per_seq*page_size=%lld]",
                max_context_len, n_q, cap);
  return MLA_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

extern "C" {

mla_status_t mla_decode_create(const mla_decode_config_t* cfg, mla_decode_t* out_plan) {
  g_last_error.clear();
  if (!cfg || !out_plan) return fail(MLA_ERR_INVALID_ARG, "cfg and out_plan must not be NULL");
  *out_plan = nullptr;
  const mla_decode_config_t& c = *cfg;
  if (c.h < 1 || c.d_c < 1 || c.d_h < 1 || c.d_r < 0)
    return fail(MLA_ERR_INVALID_ARG, "dimensions must be positive (h=%d d_c=%d d_r=%d d_h=%d)",
                c.h, c.d_c, c.d_r, c.d_h);
  if (c.dtype != MLA_DTYPE_BF16 && c.dtype != MLA_DTYPE_F32)
    return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", c.dtype);
  if (c.out_dtype != -1 && c.out_dtype != MLA_DTYPE_BF16 && c.out_dtype != MLA_DTYPE_F32)
    return fail(MLA_ERR_INVALID_ARG, "unknown out_dtype %d", c.out_dtype);
  if (c.page_size < 1 || c.max_batch < 1 || c.max_q_per_seq < 1 || c.max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARG,
                "page_size, max_batch, max_q_per_seq and max_pages_per_seq must be >= 1");
  if (c.num_splits < 0) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (!(c.scale >= 0.f) || std::isinf(c.scale))
    return fail(MLA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if ((long long)c.max_pages_per_seq * c.page_size > (1LL << 30))
    return fail(MLA_ERR_UNSUPPORTED, "context capacity above 2^30 tokens");
  const bool fast = fast_path_applies(c);
  if (!fast && c.d_c > 1024)
    return fail(MLA_ERR_UNSUPPORTED, "d_c=%d: only d_c <= 1024 is built outside the "
                "(h%%64, 512, 64, 128) bf16 shape", c.d_c);

  mla_decode_plan* p = new (std::nothrow) mla_decode_plan;
  if (!p) return fail(MLA_ERR_NOMEM, "out of host memory");
  p->cfg = c;
  p->out_dtype = c.out_dtype == -1 ? c.dtype : c.out_dtype;
  p->fast = fast;
  p->scale = c.scale > 0.f ? c.scale : 1.0f / std::sqrt((float)(c.d_h + c.d_r));
  p->num_cus = query_num_cus();
  *out_plan = p;
  return MLA_OK;
}

size_t mla_decode_workspace_size(mla_decode_t plan, int32_t batch, int32_t n_q,
                                 int32_t max_context_len) {
  if (check_shape(plan, batch, n_q, max_context_len) != MLA_OK) return 0;
  if (batch == 0) return 0;
  const Split s = plan_splits(*plan, batch, n_q, max_context_len);
  return layout_for(*plan, batch, n_q, s).total;
}

mla_status_t mla_decode_split_plan(mla_decode_t plan, int32_t batch, int32_t n_q,
                                   int32_t max_context_len, int32_t* num_splits,
                                   int32_t* chunk_len) {
  mla_status_t st = check_shape(plan, batch, n_q, max_context_len);
  if (st != MLA_OK) return st;
  if (!num_splits || !chunk_len) return fail(MLA_ERR_INVALID_ARG, "output pointers are NULL");
  const Split s = plan_splits(*plan, batch, n_q, max_context_len);
  *num_splits = s.planned ? 0 : s.splits;
  *chunk_len = s.planned ? 0 : s.chunk_len;
  return MLA_OK;
}

mla_status_t mla_decode_run(mla_decode_t plan, int32_t batch, int32_t n_q,
                            int32_t max_context_len, int32_t num_pages, const void* q,
                            const void* q_r, const void* latent_pool, const void* rope_pool,
                            const int32_t* page_table, const int32_t* context_lens,
                            const void* w_uk, const void* w_uv, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status_t st = check_shape(plan, batch, n_q, max_context_len);
  if (st != MLA_OK) return st;
  if (batch == 0) return MLA_OK;  // nothing to do
  const mla_decode_plan& p = *plan;
  const mla_decode_config_t& c = p.cfg;
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (!q || !latent_pool || !page_table || !context_lens || !w_uk || !w_uv || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (c.d_r > 0 && (!q_r || !rope_pool))
    return fail(MLA_ERR_INVALID_ARG, "q_r and rope_pool are required when d_r > 0");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (p.fast) {
    const void* vec[] = {q, q_r, latent_pool, rope_pool, w_uk, w_uv, out};
    for (const void* v : vec)
      if (!aligned(v, 16))
        return fail(MLA_ERR_INVALID_ARG, "bf16 kernels need 16-byte aligned tensors");
  } else {
    const size_t el = c.dtype == MLA_DTYPE_BF16 ? 2 : 4;
    const void* vec[] = {q, latent_pool, w_uk, w_uv};
    for (const void* v : vec)
      if (!aligned(v, el)) return fail(MLA_ERR_INVALID_ARG, "misaligned tensor");
  }
  if (!aligned(page_table, 4) || !aligned(context_lens, 4))
    return fail(MLA_ERR_INVALID_ARG, "page_table and context_lens must be 4-byte aligned");

  const Split s = plan_splits(p, batch, n_q, max_context_len);
  const Layout l = layout_for(p, batch, n_q, s);
  if (workspace_bytes < l.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, l.total);

  mla::DecodeArgs a;
  a.batch = batch;
  a.n_q = n_q;
  a.h = c.h;
  a.d_c = c.d_c;
  a.d_r = c.d_r;
  a.d_h = c.d_h;
  a.page_size = c.page_size;
  a.max_pages = c.max_pages_per_seq;
  a.num_pages = num_pages;
  a.max_len = max_context_len;
  a.splits = s.splits;
  a.chunk_len = s.chunk_len;
  a.planned = s.planned;
  a.chunks = s.chunks;
  a.plan_target = s.target;
  a.plan_min_chunk = kMinChunkTokens;
  a.plan_max_chunk = kMaxPlannedChunk;
  a.in_bf16 = c.dtype == MLA_DTYPE_BF16;
  a.out_bf16 = p.out_dtype == MLA_DTYPE_BF16;
  a.scale_log2 = p.scale * 1.4426950408889634f;  // exp(x) = 2^(x log2 e)
  a.q = q;
  a.q_r = q_r;
  a.latent_pool = latent_pool;
  a.rope_pool = rope_pool;
  a.page_table = page_table;
  a.context_lens = context_lens;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.q_abs = ws + l.q_abs;
  a.part_o = ws + l.part_o;
  a.part_lse = reinterpret_cast<float*>(ws + l.part_lse);
  a.c_bar = ws + l.c_bar;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = nullptr;
  if (plan->timing_runs < plan->timing_capacity)
    ev = &plan->events[(size_t)plan->timing_runs++ * kEventsPerRun];
  for (int k = 0; k < kKernels; ++k) {
    mla::LaunchCtx c;
    c.stream = hs;
    if (ev) {
      c.start = ev[2 * k];
      c.stop = ev[2 * k + 1];
    }
    hipError_t e;
    switch (k) {
      case 0: e = p.fast ? mla::launch_q_absorb_bf16(a, c) : mla::launch_q_absorb_general(a, c); break;
      case 1: e = p.fast ? mla::launch_split_attn_bf16(a, c) : mla::launch_split_attn_general(a, c); break;
      case 2: e = p.fast ? mla::launch_finish_bf16(a, c) : mla::launch_combine_general(a, c); break;
      default:
        if (p.fast) continue;  // folded into the finish kernel
        e = mla::launch_up_project_general(a, c);
        break;
    }
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return MLA_OK;
}

mla_status_t mla_decode_enable_timing(mla_decode_t plan, int32_t max_runs) {
  g_last_error.clear();
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  if (max_runs < 0 || max_runs > (1 << 16))
    return fail(MLA_ERR_INVALID_ARG, "max_runs %d outside [0, 65536]", max_runs);
  for (hipEvent_t e : plan->events) (void)hipEventDestroy(e);
  plan->events.clear();
  plan->timing_capacity = 0;
  plan->timing_runs = 0;
  const size_t n = (size_t)max_runs * kEventsPerRun;
  plan->events.reserve(n);
  for (size_t i = 0; i < n; ++i) {
    hipEvent_t e;
    hipError_t st = hipEventCreate(&e);
    if (st != hipSuccess) {
      for (hipEvent_t x : plan->events) (void)hipEventDestroy(x);
      plan->events.clear();
      return fail(MLA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(st));
    }
    plan->events.push_back(e);
  }
  plan->timing_capacity = max_runs;
  return MLA_OK;
}

mla_status_t mla_decode_read_timing(mla_decode_t plan, float* ms, int32_t* runs) {
  g_last_error.clear();
  if (!plan || !ms || !runs) return fail(MLA_ERR_INVALID_ARG, "NULL argument");
  for (int k = 0; k < kKernels; ++k) ms[k] = 0.f;
  const int n = plan->timing_runs;
  if (n > 0) {
    // the stop event of the last kernel the plan launches
    const int last = plan->fast ? 2 : 3;
    hipError_t st = hipEventSynchronize(plan->events[(size_t)(n - 1) * kEventsPerRun + 2 * last + 1]);
    if (st != hipSuccess) return fail(MLA_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(st));
  }
  for (int r = 0; r < n; ++r) {
    const hipEvent_t* ev = &plan->events[(size_t)r * kEventsPerRun];
    for (int k = 0; k < kKernels; ++k) {
      if (plan->fast && k == 3) continue;  // no separate up-projection kernel
      float t = 0.f;
      hipError_t st = hipEventElapsedTime(&t, ev[2 * k], ev[2 * k + 1]);
      if (st != hipSuccess) return fail(MLA_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(st));
      ms[k] += t;
    }
  }
  *runs = n;
  plan->timing_runs = 0;
  return MLA_OK;
}

void mla_decode_destroy(mla_decode_t plan) {
  if (!plan) return;
  for (hipEvent_t e : plan->events) (void)hipEventDestroy(e);
  delete plan;
}

const char* mla_decode_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
