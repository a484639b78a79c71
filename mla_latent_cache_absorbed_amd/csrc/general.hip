// general.hip -- the decode step for arbitrary dimensions, fp32 arithmetic.
//
// Same four steps and same chunked online softmax as the fast path, written
// for any (h, d_c <= 1024, d_r, d_h) and either storage type, with every
// product and sum in fp32 (this is the fp32 mode: nothing drops below fp32).
// It serves small or unusual shapes, where the work is launch-bound and a
// simple mapping costs nothing that matters.
//
//   absorb:  q_abs[r,i,c] = sum_k q[r,i,k] W_UK[i][k][c]
//            ("Mathematical Prerequisites for DeepSeek-V2" section 6)
//   split:   per (row, head, chunk) online softmax of
//            scale * (q_abs . C[t] + q_R . K_R[t]) and sum_t p_t C[t]
//            ("MLA, dim by dim" section 5.2, cached-decode chains)
//   up:      o[r,i,a] = sum_c W_UV[i][a][c] c_bar[r,i,c]
//            ("Mathematical Prerequisites for DeepSeek-V2" section 7)
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kMaxPerLane = 16;  // d_c <= 64 * 16

template <typename T>
__global__ __launch_bounds__(256) void absorb_general_kernel(const T* __restrict__ q,
                                                             const T* __restrict__ w_uk,
                                                             float* __restrict__ q_abs, int rows,
                                                             int h, int d_c, int d_h) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)rows * h * d_c;
  if (idx >= total) return;
  const int c = (int)(idx % d_c);
  const size_t rh = idx / d_c;  // r * h + i
  const int i = (int)(rh % h);
  float acc = 0.f;
  for (int k = 0; k < d_h; ++k)
    acc += load_as_f32(q, rh * d_h + k) * load_as_f32(w_uk, ((size_t)i * d_h + k) * d_c + c);
  q_abs[idx] = acc;
}

template <typename T>
__global__ __launch_bounds__(64) void split_general_kernel(DecodeArgs a) {
  const int split = blockIdx.x, head = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x;
  const int b = r / a.n_q, m = r % a.n_q;
  const T* lat = static_cast<const T*>(a.latent_pool);
  const T* rop = static_cast<const T*>(a.rope_pool);
  const T* qr = static_cast<const T*>(a.q_r) + ((size_t)r * a.h + head) * a.d_r;
  const float* qa = static_cast<const float*>(a.q_abs) + ((size_t)r * a.h + head) * a.d_c;

  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int vis = L - a.n_q + m + 1;  // query m sees tokens 0 .. L - n_q + m
  vis = vis < 0 ? 0 : vis;
  const int t0 = split * a.chunk_len;
  const int t1 = min(t0 + a.chunk_len, vis);

  float acc[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) acc[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = t0; t < t1; ++t) {
    int pg = a.page_table[(size_t)b * a.max_pages + t / a.page_size];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    const size_t row = (size_t)pg * a.page_size + t % a.page_size;
    const T* crow = lat + row * a.d_c;
    const T* krow = rop + row * a.d_r;
    float part = 0.f;
    for (int f = lane; f < a.d_c; f += 64) part += qa[f] * load_as_f32(crow, f);
    for (int f = lane; f < a.d_r; f += 64) part += load_as_f32(qr, f) * load_as_f32(krow, f);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) part = xor_sum(part, mask);
    const float s2 = part * a.scale_log2;
    const float m_new = fmaxf(m_run, s2);
    const float alpha = exp2f(m_run - m_new);
    const float pw = exp2f(s2 - m_new);
    l_run = l_run * alpha + pw;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int f = lane + 64 * j;
      if (f < a.d_c) acc[j] = acc[j] * alpha + pw * load_as_f32(crow, f);
    }
    m_run = m_new;
  }

  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* po = static_cast<float*>(a.part_o) + (((size_t)r * a.splits + split) * a.h + head) * a.d_c;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int f = lane + 64 * j;
    if (f < a.d_c) po[f] = acc[j] * inv;
  }
  if (lane == 0)
    a.part_lse[((size_t)r * a.splits + split) * a.h + head] =
        l_run > 0.f ? m_run + log2f(l_run) : -INFINITY;
}

template <typename T, typename TOut>
__global__ __launch_bounds__(256) void up_general_kernel(const T* __restrict__ w_uv,
                                                         const float* __restrict__ c_bar,
                                                         TOut* __restrict__ out, int rows, int h,
                                                         int d_c, int d_h) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)rows * h * d_h;
  if (idx >= total) return;
  const int a_row = (int)(idx % d_h);
  const size_t rh = idx / d_h;
  const int i = (int)(rh % h);
  const T* w = w_uv + ((size_t)i * d_h + a_row) * d_c;
  const float* c = c_bar + rh * d_c;
  float acc = 0.f;
  for (int f = 0; f < d_c; ++f) acc += load_as_f32(w, f) * c[f];
  store_from_f32(out, idx, acc);
}

inline unsigned blocks_for(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_q_absorb_general(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  const size_t n = (size_t)rows * a.h * a.d_c;
  if (a.in_bf16)
    launch_kernel(absorb_general_kernel<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.w_uk),
                       static_cast<float*>(a.q_abs), rows, a.h, a.d_c, a.d_h);
  else
    launch_kernel(absorb_general_kernel<float>, dim3(blocks_for(n, 256)), dim3(256), s,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.w_uk),
                       static_cast<float*>(a.q_abs), rows, a.h, a.d_c, a.d_h);
  return hipGetLastError();
}

hipError_t launch_split_attn_general(const DecodeArgs& a, const LaunchCtx& s) {
  dim3 grid(a.splits, a.h, a.batch * a.n_q);
  if (a.in_bf16)
    launch_kernel(split_general_kernel<uint16_t>, grid, dim3(64), s, a);
  else
    launch_kernel(split_general_kernel<float>, grid, dim3(64), s, a);
  return hipGetLastError();
}

hipError_t launch_up_project_general(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  const size_t n = (size_t)rows * a.h * a.d_h;
  const dim3 grid(blocks_for(n, 256)), block(256);
  const float* cb = static_cast<const float*>(a.c_bar);
  if (a.in_bf16) {
    const uint16_t* w = static_cast<const uint16_t*>(a.w_uv);
    if (a.out_bf16)
      launch_kernel((up_general_kernel<uint16_t, uint16_t>), grid, block, s, w, cb,
                         static_cast<uint16_t*>(a.out), rows, a.h, a.d_c, a.d_h);
    else
      launch_kernel((up_general_kernel<uint16_t, float>), grid, block, s, w, cb,
                         static_cast<float*>(a.out), rows, a.h, a.d_c, a.d_h);
  } else {
    const float* w = static_cast<const float*>(a.w_uv);
    if (a.out_bf16)
      launch_kernel((up_general_kernel<float, uint16_t>), grid, block, s, w, cb,
                         static_cast<uint16_t*>(a.out), rows, a.h, a.d_c, a.d_h);
    else
      launch_kernel((up_general_kernel<float, float>), grid, block, s, w, cb,
                         static_cast<float*>(a.out), rows, a.h, a.d_c, a.d_h);
  }
  return hipGetLastError();
}

}  // namespace mla
