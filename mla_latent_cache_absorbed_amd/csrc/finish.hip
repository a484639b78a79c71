// finish.hip -- split combine and W_UV up-projection in one pass (fast path).
//
// For query row r and head i the split kernel left one normalised latent
// o_s (bf16) and one base-2 log-sum-exp lse_s (fp32) per context chunk s of
// the row's sequence.  This kernel forms
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
// The chunk results of query row r = (sequence b, token m) are those of
// chunks first_b .. first_b + n_b - 1, stored [chunk][n_q][h][d_c] (lse
// [chunk][n_q][h]): with a fixed chunking first_b = S b and n_b = S; with the
// chunking planned from the context lengths (chunk_plan.h) the same device
// computation that placed the split kernel's work-groups gives them.
//
// One work-group per (head, 64 rows of W_UV[i], 16 query rows): the W_UV
// rows stream from HBM straight into the MFMA A operand (rows of W as M, d_c
// as K) while c_bar of the 16 query rows is built in LDS from the chunk
// results (one 1 KB row per chunk, 16-byte loads) and read back as the B
// operand.  Work-groups of one head get block indices congruent mod 8, so
// they run on one XCD and the W_UV rows and chunk results that several of
// them read come from its L2.  Two ways to merge:
// - few chunks (S <= 16) and at least four rows: each wave merges whole
//   query rows on its own, every (row, chunk) load of a batch in flight at
//   once;
// - otherwise all four waves merge one row, each with every fourth chunk
//   and its own running maximum, and the four partial sums meet in LDS.
#include "chunk_plan.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDh = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBlock = 16;  // query rows per work-group (the MFMA N)
constexpr int kMaxItems = 32;  // chunk results in flight per lane, at most

// Physical 16-byte chunk of logical chunk c in c_bar row `row` (< 16): the
// XOR spreads the B-operand reads (16 rows, one chunk each) over the banks.
__device__ __forceinline__ int cb_chunk(int row, int c) { return c ^ row; }

struct MergeShared {
  u32x4 cb[kRowBlock][kDc / 8];  // c_bar rows (bf16), chunk-swizzled
  f32x4 part_acc[kWaves - 1][64][2];
  float part_w[kWaves - 1][64];
  float red[kWaves];
  int row_first[kRowBlock];  // planned chunking: first chunk of each row
  int row_count[kRowBlock];  // and its number of chunks
  int max_count;
};

struct FinishArgs {
  const uint16_t* part_o;
  const float* part_lse;
  const uint16_t* w_uv;
  void* out;
  const int32_t* context_lens;
  int rows, n_q, h, batch, max_len;
  int slots;  // > 0: fixed chunking, `slots` chunks per sequence; 0: planned
  int plan_target, plan_min, plan_max;  // planned chunking (chunk_plan.h)
};

// Where the chunk results of the rows of one block are: lse index of chunk 0
// of row rb + rr (this head), the index step from one chunk to the next, and
// the row's number of chunks, for the fixed chunking or the planned one.
// (The planned tables are read through LDS pointers: a generic pointer
// would make the compiler wait for every global load in flight.)
template <bool kPlanned>
struct RowMap {
  const AS3 int* first;  // planned: row_first, row_count in LDS
  const AS3 int* count_;
  int rb, head, n_q, h, slots;
  __device__ __forceinline__ size_t base(int rr) const {
    const int r = rb + rr, b = r / n_q, m = r - b * n_q;
    const int g0 = kPlanned ? first[rr] : b * slots;
    return ((size_t)g0 * n_q + m) * h + head;
  }
  __device__ __forceinline__ size_t step() const { return (size_t)n_q * h; }
  __device__ __forceinline__ int count(int rr) const { return kPlanned ? count_[rr] : slots; }
};

// 2^x on the hardware exp2 (one instruction; a result below 2^-126 flushes
// to 0, a weight far too small to matter next to the largest, which is 1).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of v in lane u (u uniform), as a scalar.
__device__ __forceinline__ float lane_value(float v, int u) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), u));
}

// Weighted sum of one batch of chunk results into (acc0, acc1, wsum) with
// weights 2^(l - mx): the lse of item u is in lane first + u of lv (one
// load per batch instead of one per chunk), its 8 features of this lane in
// v[u].  Empty chunks (l = -inf) weigh 0 and their (unwritten) results are
// dropped by the selects.
template <int kN>
__device__ __forceinline__ void accumulate(float lv, int first, const uint4* v, float mx, f32x4& acc0,
                                           f32x4& acc1, float& wsum) {
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    const float l = lane_value(lv, first + u);
    const float w = l == -INFINITY ? 0.f : exp2_hw(l - mx);
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

// The block's merge and up-projection.  kSlots > 0: each wave merges
// 16 / kSlots whole rows per batch, kSlots chunk slots per row (kSlots >= any
// row's chunk count, a power of two).  kSlots == 0: the four waves share each
// row's chunks.
// W_UV[head] rows a_base + 16 wave .. + 15 as the A operand: lane (g, l16)
// holds row l16, d_c elements 32 s + 8 g .. + 7 for step s.
__device__ __forceinline__ void load_weights(const FinishArgs& f, int head, int a_base, int wave, int lane,
                                             bf16x8* wa) {
  const uint16_t* wrow = f.w_uv + ((size_t)head * kDh + a_base + 16 * wave + (lane & 15)) * kDc;
#pragma unroll
  for (int s = 0; s < kDc / 32; ++s)
    wa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(wrow + 32 * s + 8 * (lane >> 4)));
  // keep the weight loads here, in flight during what follows (the
  // scheduler would otherwise move them after the merge arithmetic)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// kPreloaded: the caller has loaded the weight rows into wa already.
// kBatch: chunk loads in flight per lane when the waves share a row.
template <bool kBf16Out, int kSlots, bool kPreloaded, int kBatch, typename Map>
__device__ __forceinline__ void finish_rows(const FinishArgs& f, MergeShared& sh, const Map& rm, int head,
                                            int a_base, int rb, int nr, int wave, int lane, bf16x8* wa) {
  const int h = f.h;
  const int g = lane >> 4, l16 = lane & 15;
  // lse index of chunk 0 of row rb + l, in lane l < nr: each row's base is
  // worked out once, by its own lane (its division by n_q, repeated per
  // load, had delayed the loads' issue).  It fits an int: the chunk
  // results it indexes take 1 KB each.
  const int lane_base = lane < nr ? static_cast<int>(rm.base(lane)) : 0;
  auto base_of = [&](int rr) { return __builtin_amdgcn_readlane(lane_base, rr); };  // rr wave-uniform
  // lse of chunk s of row rb + rr (s < count(rr)); a row's chunk results
  // are `res_step` elements apart from chunk 0 at row_res(rr) (a
  // wave-uniform address; each lane adds its 16-byte offset as a 32-bit
  // vector offset, so that every load is a scalar base plus a vector offset
  // and no 64-bit address is kept per load)
  const size_t lse_step = rm.step();
  const size_t res_step = lse_step * kDc;
  const uint32_t lane_off = 16u * (uint32_t)lane;
  // An item past its row's chunks weighs 0 (its lse is -inf) and its value
  // is dropped by the merge's selects: it loads the row's last chunk again
  // (a row without chunks: the first kilobyte of W_UV) instead of branching
  // around the load, so that no zero-fill joins a loaded register and
  // forces a wait.
  struct RowRes {
    const uint8_t* first;  // chunk 0 of the row (wave-uniform)
    int last;              // its last chunk, clamped to 0
  };
  auto row_res = [&](int rr, int n) {
    return n > 0 ? RowRes{reinterpret_cast<const uint8_t*>(f.part_o + (size_t)base_of(rr) * kDc), n - 1}
                 : RowRes{reinterpret_cast<const uint8_t*>(f.w_uv), 0};
  };
  auto res_at = [&](const RowRes& row, int s) {
    return *reinterpret_cast<const uint4*>(row.first + (size_t)min(s, row.last) * (res_step * 2) + lane_off);
  };

  // ---- first batch of chunk loads, ahead of the weight rows (loads
  //      complete in order, so the merge need not wait for the weights) ----
  // few chunks: each wave merges whole rows, its 4 of the block's 16 in one
  // batch of (row, chunk) items (up to 8 chunk slots: at most 32 items), or
  // 2 rows per batch with 16 slots; many chunks: kBatch chunks of a row per
  // batch.  Item u's lse is loaded by lane u (one load for the batch), its
  // result by every lane (8 features each).
  constexpr int kRowsPerBatch = kSlots > 0 ? (kSlots <= 8 ? kRowBlock / kWaves : kMaxItems / kSlots) : 1;
  constexpr int kS = kSlots > 0 ? kSlots : 1;
  constexpr int kItems = kSlots > 0 ? kRowsPerBatch * kSlots : kBatch;
  static_assert(kItems <= kMaxItems, "one batch's results fit the registers");
  float l_first;
  uint4 v_first[kItems];
  auto load_rows = [&](int row0, float& lv, uint4* v) {  // kSlots > 0: rows row0 .. + kRowsPerBatch - 1
    {
      const int rr = row0 + lane / kS, s = lane % kS;
      const int base = __shfl(lane_base, rr < nr ? rr : 0, 64);
      lv = -INFINITY;
      if (lane < kItems && rr < nr) {
        if (s < rm.count(rr)) lv = f.part_lse[(size_t)base + (size_t)s * lse_step];
      }
    }
    RowRes row[kRowsPerBatch];
#pragma unroll
    for (int ri = 0; ri < kRowsPerBatch; ++ri) {
      const int rr = row0 + ri;
      row[ri] = row_res(rr, rr < nr ? rm.count(rr) : 0);
    }
#pragma unroll
    for (int u = 0; u < kItems; ++u) v[u] = res_at(row[u / kS], u % kS);
  };
  auto load_chunks = [&](int rr, int s0, float& lv, uint4* v) {  // kSlots == 0: chunks s0, s0 + 4, ...
    const int n = rm.count(rr);
    {
      const int s = s0 + kWaves * lane;
      lv = -INFINITY;
      if (lane < kBatch && s < n) lv = f.part_lse[(size_t)base_of(rr) + (size_t)s * lse_step];
    }
    const RowRes row = row_res(rr, n);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = res_at(row, s0 + kWaves * u);
  };
  if (kSlots > 0)
    load_rows(wave * kRowsPerBatch, l_first, v_first);
  else
    load_chunks(0, wave, l_first, v_first);

  if (!kPreloaded) load_weights(f, head, a_base, wave, lane, wa);

  // ---- combine: c_bar of rows rb .. rb + nr - 1 into LDS ----
  // The prefetched batch is merged on a code path of its own: joined with
  // the path of a fresh batch, the compiler would wait for every load in
  // flight (the weight rows included) before either.
  if (kSlots > 0) {
    auto merge_rows = [&](int row0, float lv, const uint4* v) {
#pragma unroll
      for (int ri = 0; ri < kRowsPerBatch; ++ri) {
        const int rr = row0 + ri;
        float mx = lane_value(lv, ri * kS);
#pragma unroll
        for (int s = 1; s < kS; ++s) mx = fmaxf(mx, lane_value(lv, ri * kS + s));
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        float wsum = 0.f;
        accumulate<kS>(lv, ri * kS, v + ri * kS, mx, acc0, acc1, wsum);
        if (rr < nr) sh.cb[rr][cb_chunk(rr, lane)] = pack_row(acc0, acc1, wsum);
      }
    };
    int row0 = wave * kRowsPerBatch;
    if (row0 < nr) {
      merge_rows(row0, l_first, v_first);
      for (row0 += kWaves * kRowsPerBatch; row0 < nr; row0 += kWaves * kRowsPerBatch) {
        float lv;
        uint4 v[kItems];
        load_rows(row0, lv, v);
        merge_rows(row0, lv, v);
      }
    }
    __syncthreads();  // every c_bar row written
  } else {
    // one row: lane covers features 8 lane .. 8 lane + 7; wave `wave` takes
    // every 4th chunk with its own running maximum, the four are merged
    // through LDS; the first row (prefetched batch) is peeled off the loop
    auto merge_row = [&](int rr, bool prefetched) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f, mx = -INFINITY;
      auto merge_chunks = [&](float lv, const uint4* v) {
        float bmx = lane_value(lv, 0);
#pragma unroll
        for (int u = 1; u < kBatch; ++u) bmx = fmaxf(bmx, lane_value(lv, u));
        if (bmx > mx) {  // raise the reference of what is summed so far
          const float f = mx == -INFINITY ? 0.f : exp2_hw(mx - bmx);
          acc0 *= f;
          acc1 *= f;
          wsum *= f;
          mx = bmx;
        }
        accumulate<kBatch>(lv, 0, v, mx, acc0, acc1, wsum);
      };
      if (prefetched) {
        merge_chunks(l_first, v_first);
      } else {
        float lv;
        uint4 v[kBatch];
        load_chunks(rr, wave, lv, v);
        merge_chunks(lv, v);
      }
      for (int s0 = wave + kWaves * kBatch; s0 < rm.count(rr); s0 += kWaves * kBatch) {
        float lv;
        uint4 v[kBatch];
        load_chunks(rr, s0, lv, v);
        merge_chunks(lv, v);
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
        const float f0 = mx == -INFINITY ? 0.f : exp2_hw(mx - mall);
        acc0 *= f0;
        acc1 *= f0;
        wsum *= f0;
#pragma unroll
        for (int k = 0; k < kWaves - 1; ++k) {
          const float mk = sh.red[k + 1];
          const float fk = mk == -INFINITY ? 0.f : exp2_hw(mk - mall);
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
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(f.out) + o) = packed;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(f.out) + o) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// kSlots >= 0: the merge variant for a fixed chunking, kBatch chunks in
// flight per lane when the waves share a row.  kSlots < 0: planned
// chunking, the variant chosen per work-group from the chunk counts of its
// rows, with the weight rows loaded while those are worked out; the
// variants kept here (up to 8 chunk slots per row, or 8 chunks in flight
// when the waves share a row) leave room for three work-groups per CU.
template <bool kBf16Out, int kSlots, int kBatch>
__global__ __launch_bounds__(kThreads) void finish_bf16_kernel(FinishArgs f) {
  __shared__ __attribute__((aligned(16))) MergeShared sh;

  // every kernel argument in registers before the first branch (else the
  // pointers come in a second scalar load after it, one more memory
  // latency before the first loads issue)
  asm volatile("" ::"s"(f.part_o), "s"(f.part_lse), "s"(f.w_uv), "s"(f.out), "s"(f.context_lens), "s"(f.max_len),
               "s"(f.slots), "s"(f.plan_target), "s"(f.plan_min), "s"(f.plan_max));
  // blockIdx.x = head + h * (W_UV half + 2 * row block): congruent mod 8
  // for one head when h % 8 == 0
  const int head = blockIdx.x % f.h;
  const int rest = blockIdx.x / f.h;
  const int a_base = 64 * (rest & 1);
  const int rb = kRowBlock * (rest >> 1);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nr = min(kRowBlock, f.rows - rb);
  if (nr <= 0) return;  // (the host launches no empty block)
  bf16x8 wa[kDc / 32];

  if constexpr (kSlots >= 0) {
    const RowMap<false> rm{nullptr, nullptr, rb, head, f.n_q, f.h, f.slots};
    finish_rows<kBf16Out, (kSlots >= 0 ? kSlots : 0), false, kBatch>(f, sh, rm, head, a_base, rb, nr, wave,
                                                                     lane, wa);
  } else {
    // the lengths go out first, the weight rows behind them (loads
    // complete in order), then the first chunk and count of every row
    int my_len = 0;
    if (wave == 0 && lane < f.batch) my_len = f.context_lens[lane];
    load_weights(f, head, a_base, wave, lane, wa);
    if (wave == 0) {
      const chunks::Lens lens(f.context_lens, f.batch, f.max_len, lane, my_len);
      const int c = chunks::chunk_len(lens, f.plan_target, f.plan_min, f.plan_max, lane);
      const int my_b = lane < nr ? (rb + lane) / f.n_q : -1;
      int my_first = 0, my_count = 0, first = 0;
      for (int b0 = 0; b0 < f.batch; b0 += 64) {
        const int b = b0 + lane;
        const int n = b < f.batch ? chunks::ceil_div(b0 == 0 ? lens.mine : chunks::seq_len(f.context_lens, b, f.max_len), c) : 0;
        const int incl = chunks::wave_scan(n);
        const int start = first + incl - n;
        const int src = my_b - b0;
        const int s_start = __shfl(start, src & 63, 64), s_n = __shfl(n, src & 63, 64);
        if (src >= 0 && src < 64) {
          my_first = s_start;
          my_count = s_n;
        }
        first += chunks::lane_int(incl, 63);
      }
      const int mx = chunks::wave_max(lane < nr ? my_count : 0);
      if (lane < nr) {
        sh.row_first[lane] = my_first;
        sh.row_count[lane] = my_count;
      }
      if (lane == 0) sh.max_count = mx;
    }
    __syncthreads();
    const RowMap<true> rm{(const AS3 int*)sh.row_first, (const AS3 int*)sh.row_count, rb, head, f.n_q, f.h, 0};
    const int n = *(const AS3 int*)&sh.max_count;
    if (nr < kWaves && n > 1) finish_rows<kBf16Out, 0, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
    else if (n <= 1) finish_rows<kBf16Out, 1, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
    else if (n <= 2) finish_rows<kBf16Out, 2, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
    else if (n <= 4) finish_rows<kBf16Out, 4, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
    else if (n <= 8) finish_rows<kBf16Out, 8, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
    else finish_rows<kBf16Out, 0, true, 8>(f, sh, rm, head, a_base, rb, nr, wave, lane, wa);
  }
}

template <bool kBf16Out>
void launch_slots(const DecodeArgs& a, const LaunchCtx& s, dim3 grid, int rows) {
  FinishArgs f;
  f.part_o = static_cast<const uint16_t*>(a.part_o);
  f.part_lse = a.part_lse;
  f.w_uv = static_cast<const uint16_t*>(a.w_uv);
  f.out = a.out;
  f.context_lens = a.context_lens;
  f.rows = rows;
  f.n_q = a.n_q;
  f.h = a.h;
  f.batch = a.batch;
  f.max_len = a.max_len;
  f.slots = a.planned ? 0 : a.splits;
  f.plan_target = a.plan_target;
  f.plan_min = a.plan_min_chunk;
  f.plan_max = a.plan_max_chunk;
  const int S = a.splits;
#define MLA_FINISH(k, n) launch_kernel(finish_bf16_kernel<kBf16Out, k, n>, grid, dim3(kThreads), s, f)
  if (a.planned) MLA_FINISH(-1, 8);
  else if (S <= 1) MLA_FINISH(1, 16);
  else if (rows >= kWaves && S <= 16) {  // every wave merges rows of its own
    if (S <= 2) MLA_FINISH(2, 16);
    else if (S <= 4) MLA_FINISH(4, 16);
    else if (S <= 8) MLA_FINISH(8, 16);
    else MLA_FINISH(16, 16);
  } else if (S <= kWaves * 8) MLA_FINISH(0, 8);  // the waves share each row
  else MLA_FINISH(0, 16);
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
