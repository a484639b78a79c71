// oproj.hip -- the output projection that follows the decode step.
//
// For each query row r the h head outputs o_{r,1} .. o_{r,h} (d_h values
// each, as the decode step writes them) are concatenated head after head
// into k = h d_h values and multiplied by the output projection W^O, a
// k x d matrix: u_r = [o_{r,1}; ...; o_{r,h}] W^O ("From Vanilla
// Transformers to Modern LLMs ... Part 3" sections 3.h and 3.p; the W^O
// product of the "Matrix Absorption" section of "Multi-Head Latent
// Attention: Low-Rank KV Compression, Decoupled RoPE, and Matrix
// Absorption").  W^O is stored transposed, [d][k], so that each output
// feature's k weights are contiguous.
//
// gfx950 design (bf16 storage, fp32 accumulation)
// - A decode step has few query rows (1..64 here) against a weight of
//   k d values (16384 x 5120 bf16 = 168 MB at DeepSeek-V2 width): the
//   product streams W^O from HBM once and is bound by that stream.  W^O is
//   not merged into W_UV (the pages' W^OUV): per head that is a d_c x d
//   matrix, h d_c d values in all (671 MB at DeepSeek-V2 width) instead of
//   h d_h d, four times the bytes for this bandwidth-bound step.
// - Work-group = 64 output features x one slice of k x up to 64 rows.
//   Its four waves split the slice four ways and each covers all 64
//   features (four 16-feature MFMA blocks) and all rows (up to four 16-row
//   blocks) of its quarter, so every weight and every o value is read by
//   exactly one wave: W^O goes straight from HBM into MFMA A operands
//   (16 bytes per lane, 64 contiguous bytes per feature row per load), o
//   (a few MB at most, L2-resident) into B operands.  Loads run kDepth
//   k-steps ahead of the MFMAs.
// - The four waves' partial tiles are summed through LDS in wave order.
//   With one slice the sum is the result; with S > 1 slices each
//   work-group writes an fp32 partial and a second kernel sums the S
//   partials of each output in slice order, so the result does not depend
//   on timing.  S is chosen so that the grid has at least 1024 work-groups.
// - Up to kRowsDotMaxRows rows (with x within 64 KB), one launch without
//   slices instead: one wave per two output features over the whole of k
//   (rows_dot.h), no partials.
// - Shapes outside d % 64 == 0 and k % 512 == 0, and fp32 storage, take a
//   plain kernel: one thread per output, an fp32 dot product over k.
#include "common.h"
#include "kernels.h"
#include "rows_dot.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kFeatures = 64;  // output features per work-group
constexpr int kNb = kFeatures / 16;
constexpr int kRowsPerGroup = 64;
// k-steps of loads in flight per wave: four, or two with four 16-row
// blocks (so that a wave stays within 256 registers and two work-groups
// share a CU); either divides a wave's steps, a multiple of four
constexpr int kMaxDepth = 4;
template <int kRb>
constexpr int depth_for() { return kRb >= 4 ? 2 : kMaxDepth; }

struct OprojArgs {
  const uint16_t* o;   // [rows][k]
  const uint16_t* w;   // [d0][k]: output features 0 .. d0 - 1
  const uint16_t* w1;  // [d - d0][k]: output features d0 .. d - 1 (a second stacked weight)
  float* part;         // [splits][rows][d] (splits > 1, or always with write_part)
  void* u;             // [rows][d]
  int rows, k, d, d0, splits, out_bf16, write_part;
};

template <int kRb>  // 16-row blocks per work-group (1, 2 or 4)
__global__ __launch_bounds__(kThreads) void oproj_partial_kernel(OprojArgs a) {
  constexpr int kDepth = depth_for<kRb>();
  __shared__ __attribute__((aligned(16))) f32x4 red[kWaves][kNb][kRb][64];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kFeatures;
  const int slice = blockIdx.y;
  const int r0 = blockIdx.z * kRowsPerGroup;
  const int kw = a.k / (a.splits * kWaves);  // k values of this wave (a multiple of 32 kDepth)
  const int k0 = (slice * kWaves + wave) * kw;

  // A operand of feature block j, k-step s: W[n0 + 16 j + l16][k0 + 32 s + 8 g .. + 7]
  // (a work-group's 64 features lie in one of the two stacked weights)
  const uint16_t* wp = n0 < a.d0 ? a.w + (size_t)(n0 + l16) * a.k + k0 + 8 * g
                                 : a.w1 + (size_t)(n0 - a.d0 + l16) * a.k + k0 + 8 * g;
  const size_t wj = (size_t)16 * a.k;  // next feature block
  // B operand of row block rb: o[r0 + 16 rb + l16][k0 + 32 s + 8 g .. + 7]; a
  // row past the end reads row r0 instead (its results are never stored)
  const uint16_t* op[kRb];
#pragma unroll
  for (int rb = 0; rb < kRb; ++rb) {
    const int row = r0 + 16 * rb + l16;
    op[rb] = a.o + (size_t)(row < a.rows ? row : r0) * a.k + k0 + 8 * g;
  }

  f32x4 acc[kNb][kRb];
#pragma unroll
  for (int j = 0; j < kNb; ++j)
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb) acc[j][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wa[kDepth][kNb], ob[kDepth][kRb];
  auto load = [&](int slot, int s) {
#pragma unroll
    for (int j = 0; j < kNb; ++j)
      wa[slot][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wp + j * wj + 32 * s));
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb)
      ob[slot][rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op[rb] + 32 * s));
  };
  const int steps = kw / 32;
#pragma unroll
  for (int u = 0; u < kDepth; ++u) load(u, u);
  for (int s = 0; s < steps; s += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
#pragma unroll
      for (int j = 0; j < kNb; ++j)
#pragma unroll
        for (int rb = 0; rb < kRb; ++rb) acc[j][rb] = mfma16x16x32(wa[u][j], ob[u][rb], acc[j][rb]);
      if (s + u + kDepth < steps) load(u, s + u + kDepth);
    }
  }

  // the four waves' partial tiles, summed in wave order: wave w takes
  // feature block w.  D[4 g + e][l16] of block (j, rb) is feature
  // n0 + 16 j + 4 g + e of row r0 + 16 rb + l16.
#pragma unroll
  for (int j = 0; j < kNb; ++j)
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb) red[wave][j][rb][lane] = acc[j][rb];
  __syncthreads();
  const int j = wave;
  const int n = n0 + 16 * j + 4 * g;
#pragma unroll
  for (int rb = 0; rb < kRb; ++rb) {
    f32x4 v = red[0][j][rb][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[w][j][rb][lane];
    const int row = r0 + 16 * rb + l16;
    if (row >= a.rows) continue;
    const size_t idx = (size_t)row * a.d + n;
    if (a.splits > 1 || a.write_part) {
      *reinterpret_cast<f32x4*>(a.part + (size_t)slice * a.rows * a.d + idx) = v;
    } else if (a.out_bf16) {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.u) + idx) = u32x2{pack_bf16x2(v[0], v[1]),
                                                                          pack_bf16x2(v[2], v[3])};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.u) + idx) = v;
    }
  }
}

// Up to kR rows (rows_dot_applies): output features n, n + 1 over the whole
// of k, by one wave or by the work-group's kSplit waves; lane r of the wave
// with the sums stores row r.
template <int kR, bool kLds, int kDepth, int kSplit>
__global__ __launch_bounds__(kRowsDotWaves * 64) void oproj_rows_kernel(OprojArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t x_lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // < d: the grid is d / (8 / kSplit)
  const int n = kRowsDotFeatures * (blockIdx.x * (kRowsDotWaves / kSplit) + wave / kSplit);
  const uint16_t* w = a.w + (size_t)n * a.k;
  float s[kRowsDotFeatures][kR];
  if (!rows_dot<kR, kLds, kDepth, kSplit>(a.o, a.rows, a.k, w, w + a.k, x_lds, s, [] {})) return;
  if (lane >= a.rows) return;
  float v0, v1;
  rows_dot_pick<kR>(s, lane, v0, v1);
  const size_t idx = (size_t)lane * a.d + n;
  if (a.out_bf16)
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.u) + idx) = pack_bf16x2(v0, v1);
  else
    *reinterpret_cast<f32x2*>(static_cast<float*>(a.u) + idx) = f32x2{v0, v1};
}

// u = sum over the S slices of the partials, in slice order; four
// consecutive outputs per thread (d % 64 == 0).
__global__ __launch_bounds__(kThreads) void oproj_reduce_kernel(OprojArgs a) {
  const size_t total4 = (size_t)a.rows * a.d / 4;
  const size_t i4 = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i4 >= total4) return;
  const size_t stride = (size_t)a.rows * a.d;
  f32x4 v = *reinterpret_cast<const f32x4*>(a.part + 4 * i4);
  for (int s = 1; s < a.splits; ++s) v += *reinterpret_cast<const f32x4*>(a.part + s * stride + 4 * i4);
  if (a.out_bf16)
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.u) + 4 * i4) = u32x2{pack_bf16x2(v[0], v[1]),
                                                                          pack_bf16x2(v[2], v[3])};
  else
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.u) + 4 * i4) = v;
}

// Any shape and storage type: one thread per output u[r][n], the fp32 sum
// over k in increasing order.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void oproj_general_kernel(const Tin* o, const Tin* w, Tout* u, int rows,
                                                                 int k, int d) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)rows * d) return;
  const int r = (int)(i / d), n = (int)(i % d);
  const Tin* orow = o + (size_t)r * k;
  const Tin* wrow = w + (size_t)n * k;
  float acc = 0.f;
  for (int x = 0; x < k; ++x) acc = __builtin_fmaf(load_as_f32(orow, x), load_as_f32(wrow, x), acc);
  store_from_f32(u, i, acc);
}

int splits_for(int rows, int k, int d) {
  const int groups = (d / kFeatures) * ((rows + kRowsPerGroup - 1) / kRowsPerGroup);
  // The smallest slice count that gives at least 1024 work-groups (16 slices
  // at k = 16384, d = 5120: 1, 32 and 64 rows ran 2-8 % faster than with 8
  // slices, and 32 slices slower again), else the most there can be; every
  // wave keeps whole unrolled k-steps, so the count divides k / 512.
  const int units = k / (kWaves * 32 * kMaxDepth);
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && groups * s >= 1024) return s;
  return units;
}

// The MFMA partial kernel on x [rows][k] times the stacked weights [w0
// ([d0][k]); w1 ([d - d0][k])]^T; `used` receives the arguments it ran with.
hipError_t launch_partial(const void* x, const void* w0, const void* w1, int rows, int k, int d, int d0,
                                 float* part, bool write_part, void* u, bool out_bf16, const LaunchCtx& s,
                                 OprojArgs* used) {
  OprojArgs a;
  a.o = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w0);
  a.w1 = static_cast<const uint16_t*>(w1);
  a.part = part;
  a.u = u;
  a.rows = rows;
  a.k = k;
  a.d = d;
  a.d0 = d0;
  a.splits = splits_for(rows, k, d);
  a.out_bf16 = out_bf16;
  a.write_part = write_part;
  const dim3 grid(d / kFeatures, a.splits, (rows + kRowsPerGroup - 1) / kRowsPerGroup);
  if (rows <= 16)
    launch_kernel(oproj_partial_kernel<1>, grid, dim3(kThreads), s, a);
  else if (rows <= 32)
    launch_kernel(oproj_partial_kernel<2>, grid, dim3(kThreads), s, a);
  else
    launch_kernel(oproj_partial_kernel<4>, grid, dim3(kThreads), s, a);
  if (used) *used = a;
  return hipGetLastError();
}

}  // namespace

static_assert((kWaves * 32 * kMaxDepth) % kRowsDotK == 0, "the few-row kernel steps through k in 512s");

bool oproj_fast_applies(int k, int d, bool bf16) { return bf16 && d % kFeatures == 0 && k % (kWaves * 32 * kMaxDepth) == 0; }


hipError_t launch_oproj(const OprojLaunch& p, const LaunchCtx& s) {
  if (p.rows == 0) return hipSuccess;
  if (!oproj_fast_applies(p.k, p.d, p.in_bf16)) {
    const dim3 grid((unsigned)(((size_t)p.rows * p.d + kThreads - 1) / kThreads));
    if (p.in_bf16 && p.out_bf16)
      launch_kernel(oproj_general_kernel<uint16_t, uint16_t>, grid, dim3(kThreads), s,
                    static_cast<const uint16_t*>(p.o), static_cast<const uint16_t*>(p.w),
                    static_cast<uint16_t*>(p.u), p.rows, p.k, p.d);
    else if (p.in_bf16)
      launch_kernel(oproj_general_kernel<uint16_t, float>, grid, dim3(kThreads), s,
                    static_cast<const uint16_t*>(p.o), static_cast<const uint16_t*>(p.w),
                    static_cast<float*>(p.u), p.rows, p.k, p.d);
    else if (p.out_bf16)
      launch_kernel(oproj_general_kernel<float, uint16_t>, grid, dim3(kThreads), s,
                    static_cast<const float*>(p.o), static_cast<const float*>(p.w),
                    static_cast<uint16_t*>(p.u), p.rows, p.k, p.d);
    else
      launch_kernel(oproj_general_kernel<float, float>, grid, dim3(kThreads), s, static_cast<const float*>(p.o),
                    static_cast<const float*>(p.w), static_cast<float*>(p.u), p.rows, p.k, p.d);
    return hipGetLastError();
  }
  OprojArgs a;
  if (rows_dot_applies(p.rows, p.k, p.d)) {
    a.o = static_cast<const uint16_t*>(p.o);
    a.w = static_cast<const uint16_t*>(p.w);
    a.w1 = nullptr;
    a.part = nullptr;
    a.u = p.u;
    a.rows = p.rows;
    a.k = p.k;
    a.d = p.d;
    a.d0 = p.d;
    a.splits = 1;
    a.out_bf16 = p.out_bf16;
    a.write_part = 0;
    const int split = rows_dot_split(p.d, p.k);
    const dim3 grid(p.d / (kRowsDotPerGroup / split)), block(kRowsDotWaves * 64);
    const size_t lds = rows_dot_lds_bytes(p.rows, p.k);
    constexpr int kD = kRowsDotDepth, kW = kRowsDotWaves;
    if (split > 1) {  // few features: the work-group's waves split k
      if (lds > 0)
        launch_kernel_lds(oproj_rows_kernel<4, true, kD, kW>, grid, block, lds, s, a);
      else if (p.rows == 1)
        launch_kernel(oproj_rows_kernel<1, false, kD, kW>, grid, block, s, a);
      else
        launch_kernel(oproj_rows_kernel<2, false, kD, kW>, grid, block, s, a);
    } else if (lds > 0) {  // three or four rows of x, staged in LDS
      launch_kernel_lds(oproj_rows_kernel<4, true, kD, 1>, grid, block, lds, s, a);
    } else if (rows_dot_deep(p.rows, p.k)) {  // one or two rows of x, read from L2
      launch_kernel(oproj_rows_kernel<1, false, kRowsDotDeepDepth, 1>, grid, block, s, a);
    } else if (p.rows == 1) {
      launch_kernel(oproj_rows_kernel<1, false, kD, 1>, grid, block, s, a);
    } else {
      launch_kernel(oproj_rows_kernel<2, false, kD, 1>, grid, block, s, a);
    }
    return hipGetLastError();
  }
  const hipError_t e = launch_partial(p.o, p.w, nullptr, p.rows, p.k, p.d, p.d, static_cast<float*>(p.part), false,
                                      p.u, p.out_bf16, s, &a);
  if (e != hipSuccess) return e;
  if (a.splits > 1) {
    const size_t total4 = (size_t)p.rows * p.d / 4;
    launch_kernel(oproj_reduce_kernel, dim3((unsigned)((total4 + kThreads - 1) / kThreads)), dim3(kThreads), s, a);
  }
  return hipGetLastError();
}

int oproj_splits(int rows, int k, int d) { return splits_for(rows, k, d); }

hipError_t launch_proj_partial(const void* x, const void* w0, const void* w1, int rows, int k, int d, int d0,
                               float* part, const LaunchCtx& s) {
  return launch_partial(x, w0, w1, rows, k, d, d0, part, true, nullptr, false, s, nullptr);
}

size_t oproj_workspace_bytes(int rows, int k, int d, bool bf16) {
  if (!oproj_fast_applies(k, d, bf16) || rows_dot_applies(rows, k, d)) return 0;
  const int s = oproj_splits(rows, k, d);
  return s > 1 ? (size_t)s * rows * d * sizeof(float) : 0;
}

}  // namespace mla
