// rope_proj.hip -- the current token's projections, the steps before the
// decode path: what the cache and the query of a step are made from.
//
// Cache append: for each new token, with hidden state x (d_model values),
// the latent c = W_DKV x (d_c) and the decoupled RoPE key
// k_R = RoPE(W_KR x, t) (d_r) go into row t % page_size of page
// page_table[seq][t / page_size] of the latent and RoPE pools
// ("Multi-Head Latent Attention: Low-Rank KV Compression, Decoupled RoPE,
// and Matrix Absorption", section "MLA: Low-Rank Key-Value Joint
// Compression"; "MLA, dim by dim" section 5.2, the shared RoPE key cached
// after rotation; "From Vanilla Transformers to Modern LLMs ... Part 3"
// sections 3.b and 3.k).
//
// Query side: the query latent c_Q = W_DQ x (d_qc), then per head the
// content query q_i = W_UQ[i] c_Q (d_h) and the RoPE query
// q_R,i = RoPE(W_QR[i] c_Q, t) (d_r), in the order (x W_DQ) W_UQ of "MLA,
// dim by dim" section 4.3 (the same page's section 5.2 and "From Vanilla
// Transformers ..." sections 3.d and 3.l).  The outputs are the q and q_R
// that the decode step takes.
//
// RoPE rotates adjacent pairs (y_2j, y_2j+1) = (x_2j cos - x_2j+1 sin,
// x_2j+1 cos + x_2j sin) by the angle t theta_j, theta_j = base^(-2j/d_r)
// unless the caller gives the frequencies ("MLA, dim by dim", the RoPE
// paragraph of section 4).  Angles are formed and reduced in fp64 (t theta
// reaches 10^5 radians at long contexts, where fp32 would keep two digits).
//
// gfx950 design: both are skinny products (a few rows against weights of
// 5.9 MB for the cache append, 15.7 + 75.5 MB for the query side at
// DeepSeek-V2 widths) and run on the output projection's MFMA split-k
// kernel (oproj.hip) with the two weights of a stage stacked as one
// ([W_DKV; W_KR], [W_UQ; W_QR]); a finish kernel here sums its fp32 slice
// partials in slice order, applies RoPE to the second weight's features
// and writes bf16 to the pools (cache append) or to q and q_R (query side).
// Up to kRowsDotMaxRows rows (with x within 64 KB) a stage is one launch
// instead: one wave per two adjacent output features over the whole of k
// (rows_dot.h), with the RoPE pair and the store in the same kernel.  Other shapes and fp32
// storage run one plain kernel per stage.
#include "common.h"
#include "kernels.h"
#include "rows_dot.h"

namespace mla {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double rope_theta(const double* theta, double base, int j, int d_r) {
  return theta ? theta[j] : pow(base, -2.0 * j / d_r);
}

// Destination of one row: its element offsets in the two outputs (dense
// [rows][n0] / [rows][n1], or the pool row of the token), or false when a
// paged row's page lies outside the table or the pool (nothing is written).
struct Dest {
  void* out0;
  void* out1;
  const int32_t* seq;         // paged only
  const int32_t* page_table;  // paged only: [batch][max_pages]
  int max_pages, page_size, num_pages;
  bool paged;
};

__device__ __forceinline__ bool dest_row(const Dest& d, int r, int t, size_t& row) {
  if (!d.paged) {
    row = (size_t)r;
    return true;
  }
  if (t < 0) return false;
  const int j = t / d.page_size;
  if (j >= d.max_pages) return false;
  const int page = d.page_table[(size_t)d.seq[r] * d.max_pages + j];
  if (page < 0 || page >= d.num_pages) return false;
  row = (size_t)page * d.page_size + (size_t)(t % d.page_size);
  return true;
}

struct FinishArgs {
  const float* part;  // [splits][rows][n0 + n1]
  int splits, rows, n0, n1, d_r;
  const int32_t* pos;
  const double* theta;
  double base;
  Dest dst;
};

// Four consecutive features of one row per thread: the slice sum in slice
// order, RoPE on the second weight's features (two adjacent pairs), bf16.
__global__ __launch_bounds__(kThreads) void rope_finish_kernel(FinishArgs a) {
  const int n = a.n0 + a.n1;
  const int quads = n / 4;
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)a.rows * quads) return;
  const int r = (int)(i / quads), f = 4 * (int)(i % quads);
  const size_t stride = (size_t)a.rows * n;
  const float* p = a.part + (size_t)r * n + f;
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  for (int s = 1; s < a.splits; ++s) v += *reinterpret_cast<const f32x4*>(p + s * stride);
  const int t = a.pos[r];
  size_t row;
  if (!dest_row(a.dst, r, t, row)) return;
  uint16_t* out;
  if (f < a.n0) {
    out = static_cast<uint16_t*>(a.dst.out0) + row * a.n0 + f;
  } else {
    const int g = f - a.n0;
    const int j0 = (g % a.d_r) / 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      double sn, cs;
      sincos((double)t * rope_theta(a.theta, a.base, j0 + q, a.d_r), &sn, &cs);
      const float c = (float)cs, s = (float)sn;
      const float x0 = v[2 * q], x1 = v[2 * q + 1];
      v[2 * q] = x0 * c - x1 * s;
      v[2 * q + 1] = x1 * c + x0 * s;
    }
    out = static_cast<uint16_t*>(a.dst.out1) + row * a.n1 + g;
  }
  *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Up to kR rows: output features n, n + 1 of the stacked weights
// [w0; w1; w2] over the whole of k (n even, so a RoPE pair stays together),
// by one wave or by the work-group's kSplit waves; lane r of the wave with
// the sums finishes row r.  w0 and w1 go to the destination (RoPE on w1);
// w2, when n2 > 0, goes plainly to a dense [rows][n2] output (the query
// latent when the cache append and the query side's first stage share one
// launch).
struct RowsArgs {
  const uint16_t* x;   // [rows][k]
  const uint16_t* w0;  // [n0][k]
  const uint16_t* w1;  // [n1][k]
  const uint16_t* w2;  // [n2][k]
  int rows, k, n0, n1, n2, d_r;
  const int32_t* pos;
  const double* theta;
  double base;
  Dest dst;
  uint16_t* out2;      // [rows][n2]
};

template <int kR, bool kLds, int kDepth, int kSplit>
__global__ __launch_bounds__(kRowsDotWaves * 64) void rope_rows_kernel(RowsArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t x_lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // < n0 + n1 + n2: the grid is (n0 + n1 + n2) / (8 / kSplit)
  const int n = kRowsDotFeatures * (blockIdx.x * (kRowsDotWaves / kSplit) + wave / kSplit);
  const int n01 = a.n0 + a.n1;
  const uint16_t* w = n < a.n0 ? a.w0 + (size_t)n * a.k
                      : n < n01 ? a.w1 + (size_t)(n - a.n0) * a.k
                                : a.w2 + (size_t)(n - n01) * a.k;
  // the row's position is loaded ahead of the weights, and a RoPE pair's
  // angle (fp64 pow and sincos: ~1 us of latency) is worked out while the
  // first weight loads are in flight
  const int t = lane < a.rows ? a.pos[lane] : 0;
  float c = 1.f, si = 0.f;
  auto angle = [&] {
    if (n >= a.n0 && n < n01 && lane < a.rows) {
      double sn, cs;
      sincos((double)t * rope_theta(a.theta, a.base, ((n - a.n0) % a.d_r) / 2, a.d_r), &sn, &cs);
      c = (float)cs;
      si = (float)sn;
    }
  };
  float sums[kRowsDotFeatures][kR];
  if (!rows_dot<kR, kLds, kDepth, kSplit>(a.x, a.rows, a.k, w, w + a.k, x_lds, sums, angle)) return;
  if (lane >= a.rows) return;
  float v0, v1;
  rows_dot_pick<kR>(sums, lane, v0, v1);
  if (n >= n01) {  // the third weight: plain, dense rows
    *reinterpret_cast<uint32_t*>(a.out2 + (size_t)lane * a.n2 + (n - n01)) = pack_bf16x2(v0, v1);
    return;
  }
  size_t row;
  if (!dest_row(a.dst, lane, t, row)) return;
  uint16_t* out;
  if (n < a.n0) {
    out = static_cast<uint16_t*>(a.dst.out0) + row * a.n0 + n;
  } else {
    const float x0 = v0, x1 = v1;
    v0 = x0 * c - x1 * si;
    v1 = x1 * c + x0 * si;
    out = static_cast<uint16_t*>(a.dst.out1) + row * a.n1 + (n - a.n0);
  }
  *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(v0, v1);
}

// Any shape and either storage type: one thread per output feature of the
// first weight, or per RoPE pair of the second, fp32 dot products over k.
template <typename T>
__global__ __launch_bounds__(kThreads) void proj_rope_general_kernel(const T* x, const T* w0, const T* w1, int rows,
                                                                     int k, int n0, int n1, int d_r,
                                                                     const int32_t* pos, const double* theta,
                                                                     double base, Dest dst) {
  const int units = n0 + n1 / 2;
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)rows * units) return;
  const int r = (int)(i / units), u = (int)(i % units);
  const int t = pos[r];
  size_t row;
  if (!dest_row(dst, r, t, row)) return;
  const T* xr = x + (size_t)r * k;
  auto dot = [&](const T* wrow) {
    float acc = 0.f;
    for (int m = 0; m < k; ++m) acc = __builtin_fmaf(load_as_f32(xr, m), load_as_f32(wrow, m), acc);
    return acc;
  };
  if (u < n0) {
    store_from_f32(static_cast<T*>(dst.out0), row * n0 + u, dot(w0 + (size_t)u * k));
    return;
  }
  const int g = 2 * (u - n0);  // first feature of the pair in the second weight
  const float x0 = dot(w1 + (size_t)g * k), x1 = dot(w1 + (size_t)(g + 1) * k);
  double sn, cs;
  sincos((double)t * rope_theta(theta, base, (g % d_r) / 2, d_r), &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  store_from_f32(static_cast<T*>(dst.out1), row * n1 + g, x0 * c - x1 * s);
  store_from_f32(static_cast<T*>(dst.out1), row * n1 + g + 1, x1 * c + x0 * s);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The few-row kernel on [w0; w1; w2] (w2 optional: n2 = 0).
hipError_t launch_rows(const void* x, const void* w0, const void* w1, const void* w2, int rows, int k, int n0, int n1,
                       int n2, int d_r, const int32_t* pos, const double* theta, double base, const Dest& dst,
                       void* out2, const LaunchCtx& s) {
  RowsArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w0 = static_cast<const uint16_t*>(w0);
  a.w1 = static_cast<const uint16_t*>(w1);
  a.w2 = static_cast<const uint16_t*>(w2);
  a.rows = rows;
  a.k = k;
  a.n0 = n0;
  a.n1 = n1;
  a.n2 = n2;
  a.d_r = d_r;
  a.pos = pos;
  a.theta = theta;
  a.base = base;
  a.dst = dst;
  a.out2 = static_cast<uint16_t*>(out2);
  const int split = rows_dot_split(n0 + n1 + n2, k);
  const dim3 grid((n0 + n1 + n2) / (kRowsDotPerGroup / split)), block(kRowsDotWaves * 64);
  const size_t lds = rows_dot_lds_bytes(rows, k);
  constexpr int kD = kRowsDotDepth, kW = kRowsDotWaves;
  if (split > 1) {  // few features: the work-group's waves split k
    if (lds > 0)
      launch_kernel_lds(rope_rows_kernel<4, true, kD, kW>, grid, block, lds, s, a);
    else if (rows == 1)
      launch_kernel(rope_rows_kernel<1, false, kD, kW>, grid, block, s, a);
    else
      launch_kernel(rope_rows_kernel<2, false, kD, kW>, grid, block, s, a);
  } else if (lds > 0) {  // three or four rows of x, staged in LDS
    launch_kernel_lds(rope_rows_kernel<4, true, kD, 1>, grid, block, lds, s, a);
  } else if (rows_dot_deep(rows, k)) {  // one or two rows of x, read from L2
    launch_kernel(rope_rows_kernel<1, false, kRowsDotDeepDepth, 1>, grid, block, s, a);
  } else if (rows == 1) {
    launch_kernel(rope_rows_kernel<1, false, kD, 1>, grid, block, s, a);
  } else {
    launch_kernel(rope_rows_kernel<2, false, kD, 1>, grid, block, s, a);
  }
  return hipGetLastError();
}

// One projection stage with RoPE on the second weight: the few-row kernel,
// or MFMA partials plus the finish kernel, or the plain kernel.
hipError_t run_stage(const void* x, const void* w0, const void* w1, int rows, int k, int n0, int n1, int d_r,
                     const int32_t* pos, const double* theta, double base, const Dest& dst, bool bf16, bool fast,
                     float* part, const LaunchCtx& s) {
  if (fast && rows_dot_applies(rows, k, n0 + n1))
    return launch_rows(x, w0, w1, nullptr, rows, k, n0, n1, 0, d_r, pos, theta, base, dst, nullptr, s);
  if (fast) {
    hipError_t e = launch_proj_partial(x, w0, w1, rows, k, n0 + n1, n0, part, s);
    if (e != hipSuccess) return e;
    FinishArgs a;
    a.part = part;
    a.splits = oproj_splits(rows, k, n0 + n1);
    a.rows = rows;
    a.n0 = n0;
    a.n1 = n1;
    a.d_r = d_r;
    a.pos = pos;
    a.theta = theta;
    a.base = base;
    a.dst = dst;
    const size_t threads = (size_t)rows * (n0 + n1) / 4;
    launch_kernel(rope_finish_kernel, dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads), s, a);
    return hipGetLastError();
  }
  const size_t threads = (size_t)rows * (n0 + n1 / 2);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  if (bf16)
    launch_kernel(proj_rope_general_kernel<uint16_t>, grid, dim3(kThreads), s, static_cast<const uint16_t*>(x),
                  static_cast<const uint16_t*>(w0), static_cast<const uint16_t*>(w1), rows, k, n0, n1, d_r, pos,
                  theta, base, dst);
  else
    launch_kernel(proj_rope_general_kernel<float>, grid, dim3(kThreads), s, static_cast<const float*>(x),
                  static_cast<const float*>(w0), static_cast<const float*>(w1), rows, k, n0, n1, d_r, pos, theta,
                  base, dst);
  return hipGetLastError();
}

bool stage_fast(int k, int n0, int n1, int d_r, bool bf16) {
  return bf16 && n0 % 64 == 0 && n1 % 64 == 0 && d_r % 4 == 0 && oproj_fast_applies(k, n0 + n1, true);
}

size_t stage_part_bytes(int rows, int k, int n, bool fast) {
  return fast && !rows_dot_applies(rows, k, n) ? (size_t)oproj_splits(rows, k, n) * rows * n * sizeof(float) : 0;
}

}  // namespace

bool cache_append_fast(int d_model, int d_c, int d_r, bool bf16) { return stage_fast(d_model, d_c, d_r, d_r, bf16); }

size_t cache_append_workspace_bytes(int rows, int d_model, int d_c, int d_r, bool bf16) {
  return stage_part_bytes(rows, d_model, d_c + d_r, cache_append_fast(d_model, d_c, d_r, bf16));
}

hipError_t launch_cache_append(const AppendLaunch& p, const LaunchCtx& s) {
  if (p.rows == 0) return hipSuccess;
  Dest dst;
  dst.out0 = p.latent_pool;
  dst.out1 = p.rope_pool;
  dst.seq = p.seq;
  dst.page_table = p.page_table;
  dst.max_pages = p.max_pages;
  dst.page_size = p.page_size;
  dst.num_pages = p.num_pages;
  dst.paged = true;
  return run_stage(p.x, p.w_dkv, p.w_kr, p.rows, p.d_model, p.d_c, p.d_r, p.d_r, p.pos, p.theta, p.base, dst,
                   p.bf16, cache_append_fast(p.d_model, p.d_c, p.d_r, p.bf16), static_cast<float*>(p.work), s);
}

size_t query_project_workspace_bytes(int rows, int d_model, int d_qc, int h, int d_h, int d_r, bool bf16) {
  const size_t cq = align256((size_t)rows * d_qc * (bf16 ? 2 : 4));
  const size_t s1 = oproj_workspace_bytes(rows, d_model, d_qc, bf16);
  const size_t s2 = stage_part_bytes(rows, d_qc, h * (d_h + d_r), stage_fast(d_qc, h * d_h, h * d_r, d_r, bf16));
  return cq + (s1 > s2 ? s1 : s2);
}

hipError_t launch_query_project(const QueryLaunch& p, const LaunchCtx& s) {
  if (p.rows == 0) return hipSuccess;
  // stage 1: c_Q = W_DQ x, kept in the storage type (bf16: rounded to nearest
  // even, the next product's MFMA operand)
  uint8_t* work = static_cast<uint8_t*>(p.work);
  void* cq = work;
  void* part = work + align256((size_t)p.rows * p.d_qc * (p.bf16 ? 2 : 4));
  OprojLaunch o;
  o.o = p.x;
  o.w = p.w_dq;
  o.part = part;
  o.u = cq;
  o.rows = p.rows;
  o.k = p.d_model;
  o.d = p.d_qc;
  o.in_bf16 = p.bf16;
  o.out_bf16 = p.bf16;
  hipError_t e = launch_oproj(o, s);
  if (e != hipSuccess) return e;
  // stage 2: [q; q_R] = [W_UQ; W_QR] c_Q, RoPE on q_R per head
  Dest dst;
  dst.out0 = p.q;
  dst.out1 = p.q_r;
  dst.seq = nullptr;
  dst.page_table = nullptr;
  dst.max_pages = dst.page_size = dst.num_pages = 0;
  dst.paged = false;
  const int n0 = p.h * p.d_h, n1 = p.h * p.d_r;
  return run_stage(cq, p.w_uq, p.w_qr, p.rows, p.d_qc, n0, n1, p.d_r, p.pos, p.theta, p.base, dst, p.bf16,
                   stage_fast(p.d_qc, n0, n1, p.d_r, p.bf16), static_cast<float*>(part), s);
}

bool token_project_fused(int rows, int d_model, int d_c, int d_r, int d_qc, int h, int d_h, bool bf16) {
  return cache_append_fast(d_model, d_c, d_r, bf16) && stage_fast(d_qc, h * d_h, h * d_r, d_r, bf16) &&
         d_qc % 64 == 0 && rows_dot_applies(rows, d_model, d_c + d_r + d_qc) &&
         rows_dot_applies(rows, d_qc, h * (d_h + d_r));
}

size_t token_project_workspace_bytes(int rows, int d_model, int d_c, int d_r, int d_qc, int h, int d_h, bool bf16) {
  if (token_project_fused(rows, d_model, d_c, d_r, d_qc, h, d_h, bf16)) return align256((size_t)rows * d_qc * 2);
  const size_t a = cache_append_workspace_bytes(rows, d_model, d_c, d_r, bf16);
  const size_t q = query_project_workspace_bytes(rows, d_model, d_qc, h, d_h, d_r, bf16);
  return a > q ? a : q;
}

hipError_t launch_token_project(const AppendLaunch& ap, const QueryLaunch& qp, const LaunchCtx& s) {
  if (ap.rows == 0) return hipSuccess;
  if (!token_project_fused(ap.rows, ap.d_model, ap.d_c, ap.d_r, qp.d_qc, qp.h, qp.d_h, ap.bf16)) {
    const hipError_t e = launch_cache_append(ap, s);  // the workspace is free again when it ends
    return e != hipSuccess ? e : launch_query_project(qp, s);
  }
  // stage 1: the latent and RoPE key into the pools, c_Q (bf16) into the workspace
  Dest pool;
  pool.out0 = ap.latent_pool;
  pool.out1 = ap.rope_pool;
  pool.seq = ap.seq;
  pool.page_table = ap.page_table;
  pool.max_pages = ap.max_pages;
  pool.page_size = ap.page_size;
  pool.num_pages = ap.num_pages;
  pool.paged = true;
  void* cq = qp.work;
  hipError_t e = launch_rows(ap.x, ap.w_dkv, ap.w_kr, qp.w_dq, ap.rows, ap.d_model, ap.d_c, ap.d_r, qp.d_qc, ap.d_r,
                             ap.pos, ap.theta, ap.base, pool, cq, s);
  if (e != hipSuccess) return e;
  // stage 2: [q; q_R] = [W_UQ; W_QR] c_Q, as in launch_query_project
  Dest dst;
  dst.out0 = qp.q;
  dst.out1 = qp.q_r;
  dst.seq = nullptr;
  dst.page_table = nullptr;
  dst.max_pages = dst.page_size = dst.num_pages = 0;
  dst.paged = false;
  return launch_rows(cq, qp.w_uq, qp.w_qr, nullptr, qp.rows, qp.d_qc, qp.h * qp.d_h, qp.h * qp.d_r, 0, qp.d_r, qp.pos,
                     qp.theta, qp.base, dst, nullptr, s);
}

}  // namespace mla
