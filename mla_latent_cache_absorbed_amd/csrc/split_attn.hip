// split_attn.hip -- the cache-reading hot loop of absorbed MLA decode.
//
// For one query row r, one chunk [t0, t1) of the context and a group of
// 64 heads, computes over the chunk
//   s_t   = scale * (q_abs . C[t] + q_R . K_R[t])        (score)
//   p_t   = exp(s_t - m) with a running reference m      (online softmax)
//   acc   = sum_t p_t C[t],  l = sum_t p_t                (latent accumulation)
// and writes the chunk's normalised latent acc / l (bf16) and its base-2
// log-sum-exp (fp32).  The cache is contracted last for the scores and
// first for the values, which is the cheapest association for a single
// query ("MLA, dim by dim" section 4.2 and the cached-decode chains of
// section 5.2; the concatenated content + RoPE dot product of "Mathematical
// Prerequisites for DeepSeek-V2" section 9; one scale on the summed score as
// in "From Vanilla Transformers to Modern LLMs ... Part 3" section 3.o).
// Per cached token and query row this is 4 h d_c + 2 h d_r + h FLOPs over
// d_c + d_r cached values ("MLA, dim by dim", FLOPs of section 5.2).
//
// gfx950 design
// - 768 threads = 12 wave64s, three per SIMD, in two roles:
//     score waves 0-3 (one 16-head block each): scores of tile k on
//       16x16x32 bf16 MFMA, the online softmax, and the bf16 probabilities
//       P(k) published to LDS (plus per-head rescale factors when the
//       reference moves);
//     accumulate waves 4-11 (64 latent features each, all 64 heads): issue
//       the tile DMAs and fold P(k-1) into the fp32 latent accumulator
//       against tile k-1; every latent operand they read feeds four MFMAs,
//       one per head block.
//   Each SIMD runs one score wave and two accumulate waves, so one wave's
//   LDS and DMA latency is covered by the others' MFMAs, and every wave fits
//   in 168 registers (with two waves per SIMD, 128 features per accumulate
//   wave, the loop ran 3-7 % slower at T = 32K..128K).  One work-group
//   barrier per tile orders everything.
// - The chunk streams in 32-token tiles through a ring of four LDS stages
//   filled by direct global->LDS DMA (global_load_lds_dwordx4): no staging
//   registers; tiles k+1 and k+2 are in flight while the score waves read
//   tile k and the accumulate waves tile k-1.  A DMA instruction holds its
//   wave at issue while the CU's fetch path is busy, so the accumulate
//   waves issue a tile's DMAs first in each iteration, while the score
//   waves' MFMAs run.  A tile never straddles a cache page (pages are
//   multiples of 32 tokens), so each tile is one contiguous run of 32
//   latent rows and 32 RoPE rows in the pool; every tile's pool row is
//   looked up once at the start.
// - Prologue: the group's absorbed-query rows (64 x 1 KB, plus their RoPE
//   parts) come into the two ring stages that tiles 2 and 3 will use, by
//   DMA in whole rows, and the score waves read their operands from there;
//   the first barrier waits for tile 0 only.
// - The tile stays token-major in LDS with its 16-byte chunks XOR-swizzled
//   per row, so that both read patterns below are free of bank conflicts.
// - Scores: S^T[token][head] = KV[token][:] . Q[head][:], tokens as M, heads
//   as N, K over the 576 latent + RoPE features.  The absorbed query (bf16)
//   stays in registers for the whole chunk.  With heads as N each lane holds
//   one head's scores for 8 tokens, so softmax state is per lane and a tile
//   maximum needs two cross-lane swaps.
// - Latent accumulation: O^T[feature][head] += C^T[feature][token] .
//   P^T[token][head], features as M, heads as N, tokens as K.  The
//   feature-major A operand comes straight from the token-major tile through
//   the transposing LDS read ds_read_b64_tr_b16 (within 16 lanes, lane i
//   receives element i & 3 of the 8-byte chunk addressed by lane 4e + (i >> 2),
//   for e = 0..3).  P comes out of the score accumulators already in the
//   matching B-operand order, so it crosses LDS as one 16-byte store and load
//   per lane and head block.
// - The chunk result is transposed to head-major order through the (by then
//   free) LDS ring, so that every wave stores whole 1 KB head rows, with
//   non-temporal stores.
// - Work-groups that read the same chunk (other heads, other query tokens of
//   the same sequence) get block indices congruent mod 8, so they run on one
//   XCD and share its L2.
// - Chunks are numbered over the whole batch (one work-group per chunk,
//   query token and head group) and their results stored [chunk][n_q][h]
//   [d_c].  Either every sequence has the same number of chunks, or the
//   chunk length is planned from the context lengths (chunk_plan.h) and
//   each work-group finds its sequence and chunk by a scan of the lengths,
//   so that ragged batches keep every work-group about equally long.
#include "chunk_plan.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDkv = kDc + kDr;
constexpr int kTile = kFastTile;                  // 32 tokens
constexpr int kBlocks = kFastHeadsPerGroup / 16;  // 16-head blocks per group (4)
constexpr int kWaves = 12;
constexpr int kThreads = 64 * kWaves;
constexpr int kAccWaves = 8;
constexpr int kAccFeatureBlocks = kDc / 16 / kAccWaves;  // 16-feature blocks per accumulate wave
constexpr int kStages = 4;                        // LDS ring depth
constexpr int kLatBytes = kTile * kDc * 2;        // 32 KB: 32 rows of 1 KB
constexpr int kRopeBytes = kTile * kDr * 2;       // 4 KB: 32 rows of 128 B
constexpr int kStageBytes = kLatBytes + kRopeBytes;
// Tile DMAs per accumulate wave: 4 latent rows (one DMA each) and 4 RoPE
// rows (one DMA with half the lanes).
constexpr int kLatRowsPerWave = kTile / kAccWaves;   // 4
constexpr int kRopeRowsPerWave = kTile / kAccWaves;  // 4
constexpr int kAccDmas = kLatRowsPerWave + 1;        // 5

// LDS operand reads kept in flight, in pairs (lgkmcnt counts at most 15)
constexpr int kScoreReadsAhead = 4;
constexpr int kAccReadsAhead = 6;

static_assert(kBlocks == 4 && kTile == 32, "load mapping assumes 4 head blocks and 32-token tiles");

// The absorbed query of the group (64 rows of 1 KB, then 64 RoPE rows of
// 128 B) passes through ring stages kQStage.. during the prologue.
constexpr int kQStage = 2;
constexpr int kQLatBytes = kFastHeadsPerGroup * kDc * 2;
static_assert(kQLatBytes + kFastHeadsPerGroup * kDr * 2 <= (kStages - kQStage) * kStageBytes,
              "the query fits into the ring stages that the prologue leaves free");
// Largest factor (as a power of two) by which a weight may exceed 1 before
// the reference maximum moves; 2^8 keeps every sum far from fp32 overflow.
constexpr float kRescaleSlack = 8.0f;

struct SplitArgs {
  const uint16_t* q_abs;        // [R][h][512]
  const uint16_t* q_r;          // [R][h][64]
  const uint16_t* latent_pool;  // [P][page][512]
  const uint16_t* rope_pool;    // [P][page][64]
  const int32_t* page_table;    // [B][max_pages]
  const int32_t* context_lens;  // [B]
  uint16_t* part_o;             // [chunks][n_q][h][512] bf16
  float* part_lse;              // [chunks][n_q][h]
  int batch, n_q, h, head_groups, splits, chunk_len;
  int planned, chunks, plan_target, plan_min, plan_max;  // chunk numbering (kernels.h)
  int page_size, max_pages, num_pages, max_len;
  float scale_log2;
};

// Swizzle (an XOR on the 16-byte chunk index) of latent row r of a tile;
// only r mod 16 matters.  A linear map of the row bits, chosen so that both
// read patterns below are free of LDS bank conflicts on gfx950, as measured
// with the SQ_LDS_BANK_CONFLICT counter: the score operand reads (16 rows,
// one chunk each, 16 bytes per lane) and the transposing reads (8 rows, two
// adjacent chunks, 8 bytes per lane).  Row bits 0, 1, 2 go to chunk bits
// 3, 2, 1 and row bit 3 flips chunk bits 0 and 1.
__device__ __forceinline__ int lat_swz(int r) {
  return (((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1)) ^ (((r >> 3) & 1) * 3);
}
// Same for the 8 chunks of a 128-byte RoPE row.
__device__ __forceinline__ int rope_swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// The four lanes l, l^16, l^32, l^48 hold the same head (different tokens):
// reduce across them with the gfx950 cross-row swaps instead of LDS
// permutes.  permlane16_swap(x, x) leaves {x[l], x[l^16]} in the two
// results (in some order) and permlane32_swap(x, x) {x[l], x[l^32]}.
__device__ __forceinline__ float max_over_token_lanes(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_token_lanes(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Work-group barrier that orders LDS accesses (this wave's LDS stores have
// completed) but leaves outstanding global->LDS DMAs and global stores
// alone: DMAs are waited for explicitly with vmcnt, so the next tiles stay
// in flight across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk result, head-major in the (then free) tile ring: head row of 1 KB,
// its 16-byte chunks XOR-swizzled by head bits 0-3 and the two 8-byte
// halves of each chunk by head bit 3.  An accumulate-wave write stores
// 8 bytes (4 features) per lane for 16 heads; with both swizzles every 16
// lanes of it hit 16 different 8-byte bank pairs of a 128-byte line (the
// earlier 32-byte swizzle alone left 4 per line: a 4-way conflict, 12
// extra cycles per write instruction by the SQ_LDS_BANK_CONFLICT counter).
// A reader of whole chunks swaps the halves back when head bit 3 is set.
__device__ __forceinline__ uint32_t result_offset(int head, int feature) {
  return (uint32_t)head * (kDc * 2) + 16u * (uint32_t)((feature >> 3) ^ (head & 15)) +
         8u * (uint32_t)(((feature >> 2) & 1) ^ ((head >> 3) & 1)) + 2u * (feature & 3);
}

struct Shared {
  uint8_t ring[kStages * kStageBytes];  // the tile ring (token-major, swizzled)
  u32x4 prob[2][kBlocks][64];           // P(k) per 16-head block, in B-operand order
  float alpha[2][kBlocks * 16];         // rescale factor per head when flagged
  u32x4 rescale[2];                     // per 16-head block: accumulator must be rescaled
  float inv_l[kBlocks * 16];            // 1 / sum of weights, per head, at the end
  int tile_row[kMaxFastChunkTiles];     // pool row of each tile's first token
};
static_assert(sizeof(Shared) <= 160 * 1024, "LDS budget");

__global__ __launch_bounds__(kThreads, 1) void split_attn_bf16_kernel(SplitArgs p) {
  __shared__ __attribute__((aligned(16))) Shared sh;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;

  // every kernel argument in registers before the first branch (else the
  // pointers, in another 64-byte line of the argument block, come in a
  // second scalar load after it: one more memory latency)
  asm volatile("" ::"s"(p.q_abs), "s"(p.q_r), "s"(p.latent_pool), "s"(p.rope_pool), "s"(p.page_table),
               "s"(p.context_lens), "s"(p.part_o), "s"(p.part_lse));
  // ---- which (global chunk, query token, head group) this group owns ----
  const int sharers = p.n_q * p.head_groups;
  const int x = blockIdx.x;
  const int rest = x >> 3;
  const int unit = (rest / sharers) * 8 + (x & 7);  // global chunk
  if (unit >= p.chunks) return;
  const int k = rest % sharers;
  const int m = k / p.head_groups, hgi = k % p.head_groups;
  int b, chunk, clen;  // sequence, chunk within it, chunk length
  if (p.planned) {  // from the context lengths (every wave alike)
    const chunks::Lens lens(p.context_lens, p.batch, p.max_len, lane);
    clen = chunks::chunk_len(lens, p.plan_target, p.plan_min, p.plan_max, lane);
    chunks::locate(lens, clen, unit, lane, b, chunk);
    // (wave-uniform values: keep them in scalar registers for the DMAs)
    clen = __builtin_amdgcn_readfirstlane(clen);
    b = __builtin_amdgcn_readfirstlane(b);
    chunk = __builtin_amdgcn_readfirstlane(chunk);
    if (b < 0) return;  // the call has fewer chunks
  } else {
    b = unit / p.splits;
    chunk = unit % p.splits;
    clen = p.chunk_len;
  }
  const int r = b * p.n_q + m;
  const int t0 = chunk * clen;
  const bool scorer = wave < kWaves - kAccWaves;

  // Pool row of the tile starting at token ts of sequence b (tiles past the
  // table clamp to its last entry; they are never used).
  const int32_t* pt_row = p.page_table + (size_t)b * p.max_pages;
  auto tile_pool_row = [&](int ts) {
    int j = ts / p.page_size;
    j = j < p.max_pages ? j : p.max_pages - 1;
    int pg = pt_row[j];
    pg = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
    return pg * p.page_size + ts % p.page_size;
  };
  // Pool rows of tiles 2.. of the chunk into LDS (every tile that can hold a
  // visible token; all threads share the work, before the first barrier).
  auto fill_tile_rows = [&]() {
    const int bound = min(clen, max(p.max_len - t0, 0));
    const int ntiles_max = (bound + kTile - 1) / kTile;
    for (int i = 2 + tid; i < ntiles_max; i += kThreads) sh.tile_row[i] = tile_pool_row(t0 + i * kTile);
  };
  // Last visible token + 1 of this chunk for query m (tokens 0 .. L - n_q + m).
  auto chunk_end = [&](int L) {
    L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
    const int vis = max(L - p.n_q + m + 1, 0);
    return min(t0 + clen, vis);
  };
  const size_t res_row = ((size_t)unit * p.n_q + m) * p.h + hgi * kFastHeadsPerGroup;  // [chunk][m][head]
  float* pl = p.part_lse + res_row;

  // The chunk result leaves LDS one 1 KB head row per wave instruction:
  // [chunk][n_q][h][d_c] bf16, each wave storing 8 of the 64 heads.
  auto store_result = [&]() {
    uint16_t* po = p.part_o + res_row * kDc;
#pragma unroll
    for (int k2 = 0; k2 < (kFastHeadsPerGroup + kWaves - 1) / kWaves; ++k2) {
      const int head = wave + kWaves * k2;
      if (head >= kFastHeadsPerGroup) break;
      // features 8 lane .. 8 lane + 7: one chunk, its halves swapped for
      // head bit 3
      const u32x4 c = *reinterpret_cast<const AS3 u32x4*>((AS3 uint8_t*)sh.ring + head * (kDc * 2) +
                                                          16 * (lane ^ (head & 15)));
      const u32x4 v = (head & 8) ? u32x4{c[2], c[3], c[0], c[1]} : c;
      // non-temporal: the results stream out to memory rather than wait as
      // dirty L2 lines for the write-back at the end of the kernel
      // (2-3 % shorter kernel at T=4K..128K)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(po + (size_t)head * kDc + 8 * lane));
    }
  };

  // Tile i -> stage i % kStages.  Accumulate wave a copies latent rows
  // 4a..4a+3 of each tile (one 1 KB row per DMA) and RoPE rows 4a..4a+3 (one
  // DMA, lanes 0-31); row0 is the pool row of the tile's first token.  Rows past the end
  // of the chunk repeat the tile's first row, so the LDS never holds
  // non-finite garbage; their probabilities are exactly 0.  All address
  // arithmetic is scalar except the lane offsets.
  const uint32_t ring_base = (uint32_t)(uintptr_t)((AS3 uint8_t*)sh.ring);
  const int dma_wave = wave - (kWaves - kAccWaves);  // accumulate wave index
  const int rope_row = kRopeRowsPerWave * dma_wave + ((lane >> 3) & (kRopeRowsPerWave - 1));
  const uint32_t rope_chunk = 16u * (uint32_t)((lane & 7) ^ rope_swz(rope_row));
  const uint32_t rope_voff = (uint32_t)rope_row * (kDr * 2) + rope_chunk;
  // DMA number `part` of this wave for tile i (parts 0-3: latent rows,
  // part 4: the RoPE rows); t1 ends the chunk.
  auto dma = [&](int i, int row0, int t1, int part, const uint32_t* lat_voff) {
    const int nvalid = min(kTile, t1 - (t0 + i * kTile));
    const uint32_t sb = ring_base + (uint32_t)((i % kStages) * kStageBytes);
    if (part < kLatRowsPerWave) {
      const int rr = kLatRowsPerWave * dma_wave + part;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(p.latent_pool) +
                           ((size_t)row0 + (rr < nvalid ? rr : 0)) * (kDc * 2);
      lds_dma16(src, lat_voff[part], sb + rr * (kDc * 2));
    } else {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(p.rope_pool) + (size_t)row0 * (kDr * 2);
      const uint32_t voff = rope_row < nvalid ? rope_voff : rope_chunk;
      if (lane < 8 * kRopeRowsPerWave) lds_dma16(src, voff, sb + kLatBytes + kRopeRowsPerWave * dma_wave * (kDr * 2));
    }
  };

  // Iteration it (0..ntiles): score waves handle tile it, accumulate waves
  // tile it - 1; both roles pass the same ntiles + 2 barriers after the
  // prologue's.  P(k) and the rescale flags of tile k live in slot k & 1:
  // written by the score waves between barriers k and k + 1, read by the
  // accumulate waves between barriers k + 1 and k + 2, and overwritten
  // (tile k + 2) only after that.  The accumulate waves issue tile it + 2
  // between barriers it and it + 1 (before folding tile it - 1), into the
  // stage that tile it - 2 (finished before barrier it) occupied, and wait
  // for their share of tile it + 1 before barrier it + 1.  Each role keeps
  // all of its state inside its own branch, so that nothing of one role is
  // live across the other's loop.
  if (scorer) {
    // ---- prologue: this wave's 16 absorbed-query rows (and their RoPE
    //      parts) come into ring stages 2-3 by DMA, whole 1 KB rows per
    //      instruction, with the tile-row swizzles; the length and the other
    //      tiles' pool rows go out behind them ----
    const int blk = wave;  // head block within the group
    const int head0 = hgi * kFastHeadsPerGroup + 16 * blk;  // first head of the block
    const uint32_t q_lds = ring_base + (uint32_t)(kQStage * kStageBytes);
    {
      const uint8_t* qa_src = reinterpret_cast<const uint8_t*>(p.q_abs + ((size_t)r * p.h + head0) * kDc);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        lds_dma16(qa_src + (size_t)j * (kDc * 2), 16u * (uint32_t)(lane ^ lat_swz(j)),
                  q_lds + (uint32_t)(16 * blk + j) * (kDc * 2));
      const uint8_t* qr_src = reinterpret_cast<const uint8_t*>(p.q_r + ((size_t)r * p.h + head0) * kDr);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int row = 8 * d + (lane >> 3);  // head within the block
        lds_dma16(qr_src + (size_t)(8 * d) * (kDr * 2),
                  (uint32_t)(lane >> 3) * (kDr * 2) + 16u * (uint32_t)((lane & 7) ^ rope_swz(row)),
                  q_lds + (uint32_t)kQLatBytes + (uint32_t)(16 * blk + 8 * d) * (kDr * 2));
      }
    }
    const int L = p.context_lens[b];
    fill_tile_rows();
    const int t1 = chunk_end(L);
    if (t0 >= t1) {  // nothing visible: lse = -inf, the chunk result is never read
      if (g == 0) pl[16 * blk + l16] = -INFINITY;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA outlives the work-group
      return;
    }
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;

    // score reads: row l16 (+16 tb), chunk 4s + g -> (4s) ^ c1_x with
    // c1_x = g ^ lat_swz(l16) < 16, i.e. base[s & 3] + 256 (s >> 2); the
    // query rows of the block sit in the same layout
    const int c1_x = g ^ lat_swz(l16);
    const int rope_x = g ^ rope_swz(l16);
    uint32_t c1_base[4], rope_base[2];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) c1_base[k2] = l16 * (kDc * 2) + 16 * ((4 * k2) ^ c1_x);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) rope_base[k2] = kLatBytes + l16 * (kDr * 2) + 16 * ((4 * k2) ^ rope_x);

    // this wave's DMAs have landed: the query operands into registers, read
    // before the barrier after which stage 2 takes tile 2
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const AS3 uint8_t* q_blk = (const AS3 uint8_t*)sh.ring + kQStage * kStageBytes + 16 * blk * (kDc * 2);
    const AS3 uint8_t* qr_blk = (const AS3 uint8_t*)sh.ring + kQStage * kStageBytes + kQLatBytes +
                                16 * blk * (kDr * 2) - kLatBytes;
    bf16x8 qa[kDc / 32], qr[kDr / 32];
#pragma unroll
    for (int s = 0; s < kDc / 32; ++s)
      qa[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(q_blk + c1_base[s & 3] + 256 * (s >> 2)));
#pragma unroll
    for (int s = 0; s < kDr / 32; ++s)
      qr[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(qr_blk + rope_base[s]));
    // Consume the query registers here, so that the compiler's own waits for
    // them stay out of the loop.
#pragma unroll
    for (int s = 0; s < kDc / 32; ++s) asm volatile("" :: "v"(qa[s]));
#pragma unroll
    for (int s = 0; s < kDr / 32; ++s) asm volatile("" :: "v"(qr[s]));
    __syncthreads();  // tile_row is visible, the first tiles are in LDS, the query is read

    float m_run = -INFINITY, l_run = 0.f;  // reference maximum, per-lane partial weight sum
    for (int it = 0; it < ntiles; ++it) {
      block_barrier();
      const int ts = t0 + it * kTile;
      const AS3 uint8_t* stage = (const AS3 uint8_t*)sh.ring + (it % kStages) * kStageBytes;

      // ---- scores: S^T[tb*16 + 4g + j][head], operands kAhead steps ahead ----
      auto score_operand = [&](int s, int tb) -> bf16x8 {
        const AS3 uint8_t* src = s < kDc / 32
            ? stage + c1_base[s & 3] + 256 * (s >> 2) + tb * 16 * (kDc * 2)
            : stage + rope_base[s - kDc / 32] + tb * 16 * (kDr * 2);
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const AS3 u32x4*>(src));
      };
      constexpr int kAhead = kScoreReadsAhead;
      constexpr int kSteps = kDkv / 32;
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 opq[kAhead + 1][2];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) {
        opq[s][0] = score_operand(s, 0);
        opq[s][1] = score_operand(s, 1);
      }
      // The scheduling fences keep each read kAhead steps ahead of its use
      // (the scheduler would otherwise sink reads next to their MFMAs and
      // expose the full LDS latency on every step).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        if (s + kAhead < kSteps) {
          opq[(s + kAhead) % (kAhead + 1)][0] = score_operand(s + kAhead, 0);
          opq[(s + kAhead) % (kAhead + 1)][1] = score_operand(s + kAhead, 1);
        }
        const bf16x8 bq = s < kDc / 32 ? qa[s] : qr[s - kDc / 32];
        sacc[0] = mfma16x16x32(opq[s % (kAhead + 1)][0], bq, sacc[0]);
        sacc[1] = mfma16x16x32(opq[s % (kAhead + 1)][1], bq, sacc[1]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax (base 2), per lane = per head ----
      // m_run is a reference maximum, not necessarily the exact running
      // max: it moves only when a score exceeds it by more than
      // kRescaleSlack, so weights stay below 2^kRescaleSlack and most tiles
      // need no rescale.  The final division by l makes the result
      // independent of the reference.
      const int slot = it & 1;
      if (ts + kTile > t1) {  // the chunk's last tile: tokens past t1 weigh 0
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ts + tb * 16 + 4 * g + j >= t1) sacc[tb][j] = -INFINITY;
      }
      // Scaled scores (base 2); the product is a canonical float, so the
      // maxima below need no NaN quieting.
      f32x4 ss[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) ss[tb] = sacc[tb] * p.scale_log2;
      // This lane's maximum over its 8 tokens.  Some head's tile maximum
      // exceeds its reference by more than the slack exactly when some
      // lane's does, so the cross-lane reduction runs only on the tiles
      // where a reference moves (the first, and rarely after it).
      const float lmax = fmaxf(fmaxf(fmaxf(ss[0][0], ss[0][1]), fmaxf(ss[0][2], ss[0][3])),
                               fmaxf(fmaxf(ss[1][0], ss[1][1]), fmaxf(ss[1][2], ss[1][3])));
      if (__builtin_amdgcn_ballot_w64(lmax > m_run + kRescaleSlack) != 0) {  // wave-uniform
        const float tmax = max_over_token_lanes(lmax);  // the head's tile maximum
        const float m_new = fmaxf(m_run, tmax);
        // nothing has been accumulated before the first tile: no rescale
        const int flag = m_run != -INFINITY;
        if (flag) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          if (g == 0) sh.alpha[slot][16 * blk + l16] = alpha;
        }
        if (lane == 0) sh.rescale[slot][blk] = flag;
        m_run = m_new;
      } else if (lane == 0) {
        sh.rescale[slot][blk] = 0;
      }
      f32x8 pf;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pf[tb * 4 + j] = __builtin_amdgcn_exp2f(ss[tb][j] - m_run);
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);  // round to nearest even
      sh.prob[slot][blk][lane] = __builtin_bit_cast(u32x4, pb);
      // sum of the weights the MFMA sees (bf16), two per dot2
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 two = {pb[e], pb[e + 1]};
        psum = __builtin_amdgcn_fdot2_f32_bf16(two, one, psum, false);
      }
      l_run += psum;
    }
    block_barrier();  // iteration ntiles: the accumulate waves fold the last tile
    const float l_tot = sum_over_token_lanes(l_run);
    if (g == 0) {
      pl[16 * blk + l16] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
      sh.inv_l[16 * blk + l16] = l_tot > 0.f ? 1.f / l_tot : 0.f;
    }
    block_barrier();  // inv_l is visible
    block_barrier();  // the accumulate waves have written the result into LDS
    store_result();
    return;
  }

  // ---- accumulate waves: issue the tile DMAs; fold features
  //      [128 a, 128 a + 128) of all 64 heads ----
  const int a = wave - (kWaves - kAccWaves);
  // prologue: the length and the first two tiles' pool rows (scalar loads)
  // go out together with the other tiles' pool rows
  const int L = p.context_lens[b];
  const int row_a = tile_pool_row(t0);
  const int row_b = tile_pool_row(t0 + kTile);
  fill_tile_rows();
  uint32_t lat_voff[kLatRowsPerWave];
#pragma unroll
  for (int j = 0; j < kLatRowsPerWave; ++j)
    lat_voff[j] = 16u * (uint32_t)(lane ^ lat_swz(kLatRowsPerWave * a + j));
  const int t1 = chunk_end(L);
  if (t0 >= t1) return;  // the score waves write lse = -inf
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;  // <= kMaxFastChunkTiles (host-checked)

#pragma unroll
  for (int part = 0; part < kAccDmas; ++part) dma(0, row_a, t1, part, lat_voff);
  if (ntiles > 1) {
#pragma unroll
    for (int part = 0; part < kAccDmas; ++part) dma(1, row_b, t1, part, lat_voff);
  }
  // tile 0 has landed (tile 1 may still be in flight: the loop waits for
  // it before barrier 1)
  if (ntiles > 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // tile_row is visible, tile 0 is in LDS

  // transposing reads: row 4g + e (+16 for the upper 16 tokens), chunk
  // 2 fb + (q >> 1), half q & 1 -> base[fb & 7] + 256 (fb >> 3)
  const int tr_row = 4 * g + (l16 >> 2);
  const int tr_x = ((l16 & 3) >> 1) ^ lat_swz(tr_row);
  uint32_t tr_base[8];
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) tr_base[k2] = tr_row * (kDc * 2) + 16 * ((2 * k2) ^ tr_x) + 8 * (l16 & 1);

  f32x4 acc[kAccFeatureBlocks][kBlocks];
#pragma unroll
  for (int fb = 0; fb < kAccFeatureBlocks; ++fb)
#pragma unroll
    for (int hb = 0; hb < kBlocks; ++hb) acc[fb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it <= ntiles; ++it) {
    if (it < ntiles) {  // this wave's DMAs of tile it have landed
      if (it + 1 < ntiles) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      static_assert(kAccDmas == 5, "the vmcnt above counts one tile of an accumulate wave's DMAs");
    }
    block_barrier();
    const bool more = it + 2 < ntiles;  // tile it + 2 goes out during this iteration
    const int row_next = more ? __builtin_amdgcn_readfirstlane(sh.tile_row[it + 2]) : 0;
    if (it == 0) {
      if (more) {
#pragma unroll
        for (int part = 0; part < kAccDmas; ++part) dma(2, row_next, t1, part, lat_voff);
      }
      continue;
    }
    // Tile it + 2 goes out before the fold: a DMA holds its wave at issue
    // while the CU's fetch path is busy, and here that time overlaps the
    // score waves' MFMAs (issued after the fold, it delayed the barrier by
    // the whole hold: 4-9 % longer loop at T = 32K..128K and in MTP).
    if (more) {
#pragma unroll
      for (int part = 0; part < kAccDmas; ++part) dma(it + 2, row_next, t1, part, lat_voff);
    }
    const int j = it - 1;  // tile folded in this iteration
    const int slot = j & 1;
    const AS3 uint8_t* stage = (const AS3 uint8_t*)sh.ring + (j % kStages) * kStageBytes;
    auto latent_operand = [&](int fbl) -> bf16x8 {
      const int fb = kAccFeatureBlocks * a + fbl;  // feature block of the tile
      const AS3 uint8_t* a0 = stage + tr_base[fb & 7] + 256 * (fb >> 3);
      const u16x4 lo = __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 tr_vec*)a0));
      const u16x4 hi = __builtin_bit_cast(
          u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 tr_vec*)(a0 + 16 * (kDc * 2))));
      const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return as_bf16x8(v);
    };
    // The four rescale flags, P(j) and the first latent operands go out
    // together and the MFMAs follow.
    const u32x4 flags = sh.rescale[slot];
    bf16x8 pb[kBlocks];
#pragma unroll
    for (int hb = 0; hb < kBlocks; ++hb) pb[hb] = __builtin_bit_cast(bf16x8, sh.prob[slot][hb][lane]);
    constexpr int kAhead = kAccReadsAhead;
    bf16x8 opq[kAhead + 1];
#pragma unroll
    for (int fb = 0; fb < kAhead; ++fb) opq[fb] = latent_operand(fb);
    if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) {  // the reference maximum moved (rare)
#pragma unroll
      for (int hb = 0; hb < kBlocks; ++hb) {
        if (flags[hb] != 0) {
          const float alpha = sh.alpha[slot][16 * hb + l16];
#pragma unroll
          for (int fb = 0; fb < kAccFeatureBlocks; ++fb) acc[fb][hb] *= alpha;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead (as for the scores)

    // ---- O^T[f][head] += C^T[f][tokens] . P^T[tokens][head] ----
#pragma unroll
    for (int fb = 0; fb < kAccFeatureBlocks; ++fb) {
      if (fb + kAhead < kAccFeatureBlocks) opq[(fb + kAhead) % (kAhead + 1)] = latent_operand(fb + kAhead);
#pragma unroll
      for (int hb = 0; hb < kBlocks; ++hb)
        acc[fb][hb] = mfma16x16x32(opq[fb % (kAhead + 1)], pb[hb], acc[fb][hb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  block_barrier();  // pairs with the score waves' barrier after their lse
  // normalised result (bf16) into LDS, head-major, then out by all waves;
  // head 16 hb + l16 differs from head l16 by hb * 16 rows (the swizzle
  // depends on the head mod 16 only), an immediate offset
  uint32_t w_ofs[kAccFeatureBlocks];
#pragma unroll
  for (int fbl = 0; fbl < kAccFeatureBlocks; ++fbl)
    w_ofs[fbl] = result_offset(l16, 16 * (kAccFeatureBlocks * a + fbl) + 4 * g);  // D[4g + j][l16]
#pragma unroll
  for (int hb = 0; hb < kBlocks; ++hb) {
    const float inv = sh.inv_l[16 * hb + l16];
#pragma unroll
    for (int fbl = 0; fbl < kAccFeatureBlocks; ++fbl) {
      const f32x4 v = acc[fbl][hb] * inv;
      *reinterpret_cast<AS3 u32x2*>((AS3 uint8_t*)sh.ring + w_ofs[fbl] + hb * 16 * (kDc * 2)) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  block_barrier();
  store_result();
}

}  // namespace

hipError_t launch_split_attn_bf16(const DecodeArgs& a, const LaunchCtx& s) {
  SplitArgs p;
  p.q_abs = static_cast<const uint16_t*>(a.q_abs);
  p.q_r = static_cast<const uint16_t*>(a.q_r);
  p.latent_pool = static_cast<const uint16_t*>(a.latent_pool);
  p.rope_pool = static_cast<const uint16_t*>(a.rope_pool);
  p.page_table = a.page_table;
  p.context_lens = a.context_lens;
  p.part_o = static_cast<uint16_t*>(a.part_o);
  p.part_lse = a.part_lse;
  p.batch = a.batch;
  p.n_q = a.n_q;
  p.h = a.h;
  p.head_groups = a.h / kFastHeadsPerGroup;
  p.splits = a.splits;
  p.chunk_len = a.chunk_len;
  p.planned = a.planned;
  p.chunks = a.chunks;
  p.plan_target = a.plan_target;
  p.plan_min = a.plan_min_chunk;
  p.plan_max = a.plan_max_chunk;
  p.page_size = a.page_size;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.max_len = a.max_len;
  p.scale_log2 = a.scale_log2;
  const int groups = ((a.chunks + 7) / 8) * 8 * a.n_q * p.head_groups;
  launch_kernel(split_attn_bf16_kernel, dim3(groups), dim3(kThreads), s, p);
  return hipGetLastError();
}

}  // namespace mla
