// split_attn.hip -- the cache-reading hot loop of absorbed MLA decode.
//
// For one query row r, one chunk [t0, t1) of the context and a group of
// 64 heads, computes over the chunk
//   s_t   = scale * (q_abs . C[t] + q_R . K_R[t])        (score)
//   p_t   = exp(s_t - m) with the running max m           (online softmax)
//   acc   = sum_t p_t C[t],  l = sum_t p_t                (latent accumulation)
// and writes the chunk's normalised latent acc / l and its base-2
// log-sum-exp.  The cache is contracted last for the scores and first for
// the values, which is the cheapest association for a single query ("MLA,
// dim by dim" section 4.2 and the cached-decode chains of section 5.2; the
// concatenated content + RoPE dot product of "Mathematical Prerequisites for
// DeepSeek-V2" section 9; one scale on the summed score as in "From Vanilla
// Transformers to Modern LLMs ... Part 3" section 3.o).  Per cached token
// and query row this is 4 h d_c + 2 h d_r + h FLOPs over d_c + d_r cached
// values ("MLA, dim by dim", FLOPs table of section 5.2).
//
// gfx950 design
// - 256 threads = 4 wave64s; each wave owns 16 heads.  Every 32-token tile
//   of latent + RoPE rows is read from HBM once per work-group with 16-byte
//   loads (8 lanes per 128-byte line) and staged in LDS, where all 64 heads
//   reuse it.
// - Scores: S^T[token][head] = KV[token][:] . Q[head][:] on 16x16x32 bf16
//   MFMA, tokens as M, heads as N, K over the 576 latent + RoPE features.
//   The absorbed query (bf16) stays in registers for the whole chunk.
// - With heads as N, each lane holds one head's scores for 8 tokens, so the
//   running max and the rescale of the accumulator are per-lane values; the
//   tile maximum needs two cross-lane steps.
// - Latent accumulation: O^T[feature][head] += C^T[feature][token] .
//   P^T[token][head], features as M (32 blocks of 16), heads as N, tokens as
//   K.  The probabilities come straight out of the score accumulators in the
//   B-operand layout (the k order is permuted identically on both sides), so
//   no shuffle is needed.  The A operand needs the tile feature-major; it is
//   written to LDS a second time, transposed, with a 4-token XOR swizzle so
//   that both the transposing writes and the 8-byte MFMA reads spread over
//   the LDS banks.
// - The accumulator (64 heads x 512 features, fp32) lives in registers: 128
//   per lane; with the query operands that needs one wave per SIMD (one
//   work-group per CU), so the 512-entry register file is available.
// - Work-groups that read the same chunk (other heads, other query tokens of
//   the same sequence) get block indices congruent mod 8, so they run on one
//   XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDkv = kDc + kDr;
constexpr int kTile = kFastTile;          // 32 tokens
constexpr int kWaves = kFastHeadsPerGroup / 16;
constexpr int kThreads = 64 * kWaves;     // 256
constexpr int kKvStride = kDkv + 8;       // token-major row, elements (1168 B)
constexpr int kCtStride = kTile + 8;      // feature-major row, elements (80 B)
constexpr int kLdsKv = kTile * kKvStride;
constexpr int kLdsCt = kDc * kCtStride;
constexpr int kLdsBytes = (kLdsKv + kLdsCt) * 2;
constexpr int kLatChunks = kTile * kDc / 8 / kThreads;  // 16-byte chunks per thread (8)

static_assert(kThreads == 256, "load mapping assumes 256 threads");
static_assert(kTile * kDr / 8 == kThreads, "one RoPE chunk per thread");

struct SplitArgs {
  const uint16_t* q_abs;        // [R][h][512]
  const uint16_t* q_r;          // [R][h][64]
  const uint16_t* latent_pool;  // [P][page][512]
  const uint16_t* rope_pool;    // [P][page][64]
  const int32_t* page_table;    // [B][max_pages]
  const int32_t* context_lens;  // [B]
  float* part_o;                // [R][S][h][512]
  float* part_lse;              // [R][S][h]
  int batch, n_q, h, head_groups, splits, chunk_len;
  int page_size, max_pages, num_pages, max_len;
  float scale_log2;
};

__device__ __forceinline__ int page_of(const SplitArgs& p, int b, int t) {
  int pg = p.page_table[(size_t)b * p.max_pages + t / p.page_size];
  pg = pg < 0 ? 0 : pg;
  return pg >= p.num_pages ? p.num_pages - 1 : pg;
}

__global__ __launch_bounds__(kThreads, 1) void split_attn_bf16_kernel(SplitArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* kv = lds;           // [32][kKvStride]   token-major latent | rope
  uint16_t* ct = lds + kLdsKv;  // [512][kCtStride]  feature-major latent, swizzled

  // ---- which (sequence, chunk, query token, head group) this group owns ----
  const int sharers = p.n_q * p.head_groups;
  const int x = blockIdx.x;
  const int rest = x >> 3;
  const int unit = (rest / sharers) * 8 + (x & 7);
  if (unit >= p.batch * p.splits) return;
  const int k = rest % sharers;
  const int b = unit / p.splits, split = unit % p.splits;
  const int m = k / p.head_groups, hgi = k % p.head_groups;
  const int r = b * p.n_q + m;

  int L = p.context_lens[b];
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  int vis = L - p.n_q + m + 1;  // query m sees tokens 0 .. L - n_q + m
  vis = vis < 0 ? 0 : vis;
  const int t0 = split * p.chunk_len;
  const int t1 = min(t0 + p.chunk_len, vis);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int head = hgi * kFastHeadsPerGroup + 16 * wave + l16;

  float* po = p.part_o + (((size_t)r * p.splits + split) * p.h + head) * kDc;
  float* pl = p.part_lse + ((size_t)r * p.splits + split) * p.h + head;

  if (t0 >= t1) {  // nothing visible in this chunk for this query row
#pragma unroll 4
    for (int fb = 0; fb < kDc / 16; ++fb)
      *reinterpret_cast<float4*>(po + fb * 16 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g == 0) *pl = -INFINITY;
    return;
  }

  // ---- absorbed query and RoPE query: MFMA B operands, kept in registers ----
  bf16x8 qa[kDc / 32], qr[kDr / 32];
  {
    const uint16_t* qa_row = p.q_abs + ((size_t)r * p.h + head) * kDc;
    const uint16_t* qr_row = p.q_r + ((size_t)r * p.h + head) * kDr;
#pragma unroll
    for (int s = 0; s < kDc / 32; ++s)
      qa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qa_row + 32 * s + 8 * g));
#pragma unroll
    for (int s = 0; s < kDr / 32; ++s)
      qr[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qr_row + 32 * s + 8 * g));
  }

  f32x4 acc[kDc / 16];
#pragma unroll
  for (int fb = 0; fb < kDc / 16; ++fb) acc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- load mapping: latent chunk j of this thread = token lt, features
  //      8 (lpc + 8 j) .. +7; RoPE chunk = token rt, features 8 rc .. +7 ----
  const int lt = (lane >> 3) + 8 * wave;
  const int lpc = lane & 7;
  const int rt = tid >> 3, rc = tid & 7;

  // Global -> LDS staging of one tile, in two halves so that at most five
  // 16-byte loads per thread are in flight (the accumulator and the query
  // already hold most of the register file).  The other work-group on the
  // CU computes while this one waits on HBM.
  auto load_stage = [&](int ts) {
    const int gt = ts + lt;
    const bool lat_ok = gt < t1;
    const uint16_t* src = p.latent_pool;
    if (lat_ok) {
      const int pg = page_of(p, b, gt);
      src += ((size_t)pg * p.page_size + gt % p.page_size) * kDc + 8 * lpc;
    }
    const int gr = ts + rt;
    uint4 rope = make_uint4(0, 0, 0, 0);
    if (gr < t1) {
      const int pg = page_of(p, b, gr);
      rope = *reinterpret_cast<const uint4*>(p.rope_pool + ((size_t)pg * p.page_size + gr % p.page_size) * kDr + 8 * rc);
    }
    // element (feature f, token t) of the transposed copy sits at
    // ct[f][t ^ 4 sigma(f)], sigma(f) = (f >> 3) & 7 = lpc for this thread
    const int tcol = lt ^ (4 * lpc);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 lat[kLatChunks / 2];
#pragma unroll
      for (int j = 0; j < kLatChunks / 2; ++j)
        lat[j] = lat_ok ? *reinterpret_cast<const uint4*>(src + 64 * (j + half * kLatChunks / 2))
                        : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kLatChunks / 2; ++j) {
        const int pc = lpc + 8 * (j + half * kLatChunks / 2);
        *reinterpret_cast<uint4*>(&kv[lt * kKvStride + 8 * pc]) = lat[j];
        const uint32_t w4[4] = {lat[j].x, lat[j].y, lat[j].z, lat[j].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          ct[(8 * pc + e) * kCtStride + tcol] = static_cast<uint16_t>(w4[e >> 1] >> (16 * (e & 1)));
      }
    }
    *reinterpret_cast<uint4*>(&kv[rt * kKvStride + kDc + 8 * rc]) = rope;
  };

  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  for (int it = 0; it < ntiles; ++it) {
    const int ts = t0 + it * kTile;
    __syncthreads();  // every wave is done with the previous tile
    load_stage(ts);
    __syncthreads();

    // ---- scores: S^T[tb*16 + 4g + j][head] ----
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < kDkv / 32; ++s) {
      const bf16x8 bq = s < kDc / 32 ? qa[s] : qr[s - kDc / 32];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&kv[(tb * 16 + l16) * kKvStride + 32 * s + 8 * g]));
        sacc[tb] = mfma16x16x32(av, bq, sacc[tb]);
      }
      // keep only a few operand loads in flight (register budget)
      if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax (base 2), per lane = per head ----
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = ts + tb * 16 + 4 * g + j;
        const float v = t < t1 ? sacc[tb][j] * p.scale_log2 : -INFINITY;
        sv[tb * 4 + j] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    uint32_t pk[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint16_t b0 = f32_to_bf16(exp2f(sv[e] - m_use));
      const uint16_t b1 = f32_to_bf16(exp2f(sv[e + 1] - m_use));
      psum += bf16_to_f32(b0) + bf16_to_f32(b1);  // normalise by the weights the MFMA sees
      pk[e >> 1] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));

    // ---- latent accumulation: O^T[f][head] += C^T[f][tokens] . P^T[tokens][head] ----
#pragma unroll
    for (int fb = 0; fb < kDc / 16; ++fb) {
      const int f = fb * 16 + l16;
      const int sig = (f >> 3) & 7;
      const uint16_t* row = &ct[f * kCtStride];
      const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * (g ^ sig));
      const uint2 hi = *reinterpret_cast<const uint2*>(row + 4 * ((4 + g) ^ sig));
      acc[fb] *= alpha;
      acc[fb] = mfma16x16x32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[fb]);
      if ((fb & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- normalise and write this chunk's result ----
  float l_tot = xor_sum(l_run, 16);
  l_tot = xor_sum(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int fb = 0; fb < kDc / 16; ++fb)
    *reinterpret_cast<float4*>(po + fb * 16 + 4 * g) =
        make_float4(acc[fb][0] * inv, acc[fb][1] * inv, acc[fb][2] * inv, acc[fb][3] * inv);
  if (g == 0) *pl = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
}

}  // namespace

hipError_t launch_split_attn_bf16(const DecodeArgs& a, hipStream_t s) {
  // more than 64 KB of dynamic LDS has to be requested once per process
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(split_attn_bf16_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return attr;
  SplitArgs p;
  p.q_abs = static_cast<const uint16_t*>(a.q_abs);
  p.q_r = static_cast<const uint16_t*>(a.q_r);
  p.latent_pool = static_cast<const uint16_t*>(a.latent_pool);
  p.rope_pool = static_cast<const uint16_t*>(a.rope_pool);
  p.page_table = a.page_table;
  p.context_lens = a.context_lens;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.batch = a.batch;
  p.n_q = a.n_q;
  p.h = a.h;
  p.head_groups = a.h / kFastHeadsPerGroup;
  p.splits = a.splits;
  p.chunk_len = a.chunk_len;
  p.page_size = a.page_size;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.max_len = a.max_len;
  p.scale_log2 = a.scale_log2;
  const int units = a.batch * a.splits;
  const int groups = ((units + 7) / 8) * 8 * a.n_q * p.head_groups;
  hipLaunchKernelGGL(split_attn_bf16_kernel, dim3(groups), dim3(kThreads), kLdsBytes, s, p);
  return hipGetLastError();
}

}  // namespace mla
