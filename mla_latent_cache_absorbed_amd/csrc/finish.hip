// finish.hip -- split combine and W_UV up-projection in one pass (fast path).
//
// For query row r and head i the split kernel left one normalised latent
// o_s (bf16, [R][S][h][512]) and one base-2 log-sum-exp lse_s (fp32) per
// context chunk s.  This kernel forms
//   c_bar = sum_s w_s o_s / sum_s w_s,   w_s = 2^(lse_s - m)
// for any reference m (here the maximum, or running maxima merged at the
// end) (the softmax over the whole visible context evaluated chunk by
// chunk: the chunks partition the token axis, so the merge is exact up to
// rounding; "MLA, dim by dim" section 5.2) and then
//   o[r, i, :] = W_UV[i] c_bar
// (the value up-projection applied once per head, by linearity,
// "Mathematical Prerequisites for DeepSeek-V2" section 7; "From Vanilla
// Transformers to Modern LLMs ... Part 3" section 3.g).  Chunks with
// lse = -inf (nothing visible) weigh 0 and their result is never used.
//
// One work-group per (head, 64 rows of W_UV[i], 16 query rows): the W_UV
// rows stream from HBM straight into the MFMA A operand (rows of W as M, d_c
// as K) while c_bar of the 16 query rows is built in LDS from the chunk
// results (one 1 KB row per chunk, 16-byte loads) and read back as the B
// operand.  Work-groups of one head get block indices congruent mod 8, so
// they run on one XCD and the W_UV rows and chunk results that several of
// them read come from its L2.  Two ways to merge:
// - few chunks (S <= 16): each wave merges whole query rows on its own,
//   every (row, chunk) load of a batch in flight at once;
// - many chunks: all four waves merge one row, each with every fourth chunk
//   and its own running maximum, and the four partial sums meet in LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDh = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBlock = 16;  // query rows per work-group (the MFMA N)
constexpr int kBatch = 16;     // chunk loads in flight per lane

// Physical 16-byte chunk of logical chunk c in c_bar row `row` (< 16): the
// XOR spreads the B-operand reads (16 rows, one chunk each) over the banks.
__device__ __forceinline__ int cb_chunk(int row, int c) { return c ^ row; }

struct MergeShared {
  u32x4 cb[kRowBlock][kDc / 8];  // c_bar rows (bf16), chunk-swizzled
  f32x4 part_acc[kWaves - 1][64][2];
  float part_w[kWaves - 1][64];
  float red[kWaves];
};

// Weighted sum of one batch of chunk results into (acc0, acc1, wsum) with
// weights 2^(l - mx); empty chunks (l = -inf) weigh 0 and their (unwritten)
// results are dropped by the selects.
template <int kN>
__device__ __forceinline__ void accumulate(const float* l, const uint4* v, float mx, f32x4& acc0,
                                           f32x4& acc1, float& wsum) {
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    const float w = l[u] == -INFINITY ? 0.f : exp2f(l[u] - mx);
    const bool use = w != 0.f;
    const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = w * bf16_to_f32(static_cast<uint16_t>(x[e]));
      const float hi = w * bf16_to_f32(static_cast<uint16_t>(x[e] >> 16));
      if (e < 2) {
        acc0[2 * e] += use ? lo : 0.f;
        acc0[2 * e + 1] += use ? hi : 0.f;
      } else {
        acc1[2 * e - 4] += use ? lo : 0.f;
        acc1[2 * e - 3] += use ? hi : 0.f;
      }
    }
    wsum += w;
  }
}

__device__ __forceinline__ u32x4 pack_row(f32x4 acc0, f32x4 acc1, float wsum) {
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  return u32x4{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
               pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
}

// kSlots > 0: each wave merges 16 / kSlots whole rows per batch, kSlots
// chunk slots per row (kSlots >= S, a power of two).  kSlots == 0: the
// four waves share each row's chunks.
template <bool kBf16Out, int kSlots>
__global__ __launch_bounds__(kThreads) void finish_bf16_kernel(const uint16_t* __restrict__ part_o,
                                                               const float* __restrict__ part_lse,
                                                               const uint16_t* __restrict__ w_uv,
                                                               void* __restrict__ out, int rows,
                                                               int splits, int h) {
  __shared__ __attribute__((aligned(16))) MergeShared sh;

  // blockIdx.x = head + h * (W_UV half + 2 * row block): congruent mod 8
  // for one head when h % 8 == 0
  const int head = blockIdx.x % h;
  const int rest = blockIdx.x / h;
  const int a_base = 64 * (rest & 1);
  const int rb = kRowBlock * (rest >> 1);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int nr = min(kRowBlock, rows - rb);
  if (nr <= 0) return;  // (the host launches no empty block)

  const size_t stride = (size_t)h * kDc;  // elements of one chunk's results
  // lse and this lane's 8 features of chunk s of row r (row < rows, s < splits)
  auto lse_at = [&](int r, int s) { return part_lse[((size_t)r * splits + s) * h + head]; };
  auto res_at = [&](int r, int s) {
    return *reinterpret_cast<const uint4*>(part_o + ((size_t)r * splits * h + head) * kDc + s * stride +
                                           8 * lane);
  };

  // ---- first batch of chunk loads, ahead of the weight rows (loads
  //      complete in order, so the merge need not wait for the weights) ----
  constexpr int kRowsPerBatch = kSlots > 0 ? kBatch / kSlots : 1;
  float l_first[kBatch];
  uint4 v_first[kBatch];
  auto load_rows = [&](int row0, float* l, uint4* v) {  // kSlots > 0: rows row0 .. + kRowsPerBatch - 1
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int rr = row0 + u / (kSlots > 0 ? kSlots : 1), s = u % (kSlots > 0 ? kSlots : 1);
      if (rr < nr && s < splits) {  // uniform per wave
        l[u] = lse_at(rb + rr, s);
        v[u] = res_at(rb + rr, s);
      } else {
        l[u] = -INFINITY;
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_chunks = [&](int r, int s0, float* l, uint4* v) {  // kSlots == 0: chunks s0, s0 + 4, ...
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + kWaves * u;
      if (s < splits) {  // uniform per wave
        l[u] = lse_at(r, s);
        v[u] = res_at(r, s);
      } else {
        l[u] = -INFINITY;
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  if (kSlots > 0)
    load_rows(wave * kRowsPerBatch, l_first, v_first);
  else
    load_chunks(rb, wave, l_first, v_first);

  // W_UV[head] rows a_base + 16 wave .. + 15 as the A operand: lane (g, l16)
  // holds row l16, d_c elements 32 s + 8 g .. + 7 for step s.
  const uint16_t* wrow = w_uv + ((size_t)head * kDh + a_base + 16 * wave + l16) * kDc;
  bf16x8 wa[kDc / 32];
#pragma unroll
  for (int s = 0; s < kDc / 32; ++s)
    wa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(wrow + 32 * s + 8 * g));
  // keep the weight loads here, in flight during the merge (the scheduler
  // would otherwise move them after the merge arithmetic)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- combine: c_bar of rows rb .. rb + nr - 1 into LDS ----
  // The prefetched batch is merged on a code path of its own: joined with
  // the path of a fresh batch, the compiler would wait for every load in
  // flight (the weight rows included) before either.
  if (kSlots > 0) {
    constexpr int kS = kSlots > 0 ? kSlots : 1;
    auto merge_rows = [&](int row0, const float* l, const uint4* v) {
#pragma unroll
      for (int ri = 0; ri < kRowsPerBatch; ++ri) {
        const int rr = row0 + ri;
        const float* lr = l + ri * kS;
        const uint4* vr = v + ri * kS;
        float mx = lr[0];  // the same in every lane (one head)
#pragma unroll
        for (int s = 1; s < kS; ++s) mx = fmaxf(mx, lr[s]);
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        float wsum = 0.f;
        accumulate<kS>(lr, vr, mx, acc0, acc1, wsum);
        if (rr < nr) sh.cb[rr][cb_chunk(rr, lane)] = pack_row(acc0, acc1, wsum);
      }
    };
    int row0 = wave * kRowsPerBatch;
    if (row0 < nr) {
      merge_rows(row0, l_first, v_first);
      for (row0 += kWaves * kRowsPerBatch; row0 < nr; row0 += kWaves * kRowsPerBatch) {
        float l[kBatch];
        uint4 v[kBatch];
        load_rows(row0, l, v);
        merge_rows(row0, l, v);
      }
    }
    __syncthreads();  // every c_bar row written
  } else {
    // one row: lane covers features 8 lane .. 8 lane + 7; wave `wave` takes
    // every 4th chunk with its own running maximum, the four are merged
    // through LDS; the first row (prefetched batch) is peeled off the loop
    auto merge_row = [&](int rr, bool prefetched) {
      const int r = rb + rr;
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f, mx = -INFINITY;
      auto merge_chunks = [&](const float* l, const uint4* v) {
        float bmx = l[0];
#pragma unroll
        for (int u = 1; u < kBatch; ++u) bmx = fmaxf(bmx, l[u]);
        if (bmx > mx) {  // raise the reference of what is summed so far
          const float f = mx == -INFINITY ? 0.f : exp2f(mx - bmx);
          acc0 *= f;
          acc1 *= f;
          wsum *= f;
          mx = bmx;
        }
        accumulate<kBatch>(l, v, mx, acc0, acc1, wsum);
      };
      if (prefetched) {
        merge_chunks(l_first, v_first);
      } else {
        float l[kBatch];
        uint4 v[kBatch];
        load_chunks(r, wave, l, v);
        merge_chunks(l, v);
      }
      for (int s0 = wave + kWaves * kBatch; s0 < splits; s0 += kWaves * kBatch) {
        float l[kBatch];
        uint4 v[kBatch];
        load_chunks(r, s0, l, v);
        merge_chunks(l, v);
      }
      if (wave > 0) {
        sh.part_acc[wave - 1][lane][0] = acc0;
        sh.part_acc[wave - 1][lane][1] = acc1;
        sh.part_w[wave - 1][lane] = wsum;
        if (lane == 0) sh.red[wave] = mx;
      }
      __syncthreads();
      if (wave == 0) {
        float mall = mx;
#pragma unroll
        for (int k = 1; k < kWaves; ++k) mall = fmaxf(mall, sh.red[k]);
        const float f0 = mx == -INFINITY ? 0.f : exp2f(mx - mall);
        acc0 *= f0;
        acc1 *= f0;
        wsum *= f0;
#pragma unroll
        for (int k = 0; k < kWaves - 1; ++k) {
          const float mk = sh.red[k + 1];
          const float fk = mk == -INFINITY ? 0.f : exp2f(mk - mall);
          acc0 += fk * sh.part_acc[k][lane][0];
          acc1 += fk * sh.part_acc[k][lane][1];
          wsum += fk * sh.part_w[k][lane];
        }
        sh.cb[rr][cb_chunk(rr, lane)] = pack_row(acc0, acc1, wsum);
      }
      __syncthreads();  // red, part_acc reusable; cb row written
    };
    merge_row(0, true);
    for (int rr = 1; rr < nr; ++rr) merge_row(rr, false);
  }

  // ---- up-projection of the block: D[a][r] = sum_c W_UV[a][c] c_bar[r][c] ----
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kDc / 32; ++s) {
    u32x4 bv = {0u, 0u, 0u, 0u};
    if (l16 < nr) bv = sh.cb[l16][cb_chunk(l16, 4 * s + g)];
    acc = mfma16x16x32(wa[s], __builtin_bit_cast(bf16x8, bv), acc);
  }
  if (l16 < nr) {
    // D[4g + j][l16] = o[rb + l16][head][a_base + 16 wave + 4g + j]
    const size_t o = ((size_t)(rb + l16) * h + head) * kDh + a_base + 16 * wave + 4 * g;
    if (kBf16Out) {
      uint2 packed;
      packed.x = pack_bf16x2(acc[0], acc[1]);
      packed.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = packed;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + o) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

template <bool kBf16Out>
void launch_slots(const DecodeArgs& a, const LaunchCtx& s, dim3 grid, int rows) {
  const uint16_t* po = static_cast<const uint16_t*>(a.part_o);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_uv);
  const int S = a.splits;
#define MLA_FINISH(k) \
  launch_kernel(finish_bf16_kernel<kBf16Out, k>, grid, dim3(kThreads), s, po, a.part_lse, w, a.out, rows, S, a.h)
  if (S <= 1) MLA_FINISH(1);
  else if (S <= 2) MLA_FINISH(2);
  else if (S <= 4) MLA_FINISH(4);
  else if (S <= 8) MLA_FINISH(8);
  else if (S <= 16) MLA_FINISH(16);
  else MLA_FINISH(0);
#undef MLA_FINISH
}

}  // namespace

hipError_t launch_finish_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  const int rows = a.batch * a.n_q;
  const dim3 grid(a.h * 2 * ((rows + kRowBlock - 1) / kRowBlock));
  if (a.out_bf16)
    launch_slots<true>(a, s, grid, rows);
  else
    launch_slots<false>(a, s, grid, rows);
  return hipGetLastError();
}

}  // namespace mla
