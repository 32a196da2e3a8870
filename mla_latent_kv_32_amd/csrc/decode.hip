// Absorbed MLA decode over a paged latent cache, gfx950.
//
// Every head scores the same cached row [c_KV | rotated k_R] (576 values), so
// a workgroup streams each 32-token block of a sequence from HBM into LDS once
// and all of its heads (up to 128) consume it there.  The decoding-stage MQA
// form of MLA (Su, "The Ultimate Tug-of-War Between Cache and Performance",
// MLA Part 3, eq:mla-mqa); one loaded latent serves every head (Riju,
// "Multi-Head Latent Attention vs GQA vs MQA", "Arithmetic intensity changes
// under absorption").
//
// Work split (8 waves, 128 heads): waves pair up on 32 heads.
//   scores   each wave owns 16 heads: S^T[tok, head] = K[tok, 0:576] . Q^T
//            (v_mfma_f32_16x16x32_bf16), then the online softmax of its heads
//            (fp32, exp2, lazily rescaled) and P rounded to bf16
//   exchange both waves of a pair publish P (bf16, 1 KB per wave) and the
//            per-head rescale factors through LDS
//   values   O^T[col, head] += V^T[col, tok] . P^T[tok, head] for the pair's 32
//            heads (v_mfma_f32_32x32x16_bf16), V = K[:, 0:512]; wave h of the
//            pair owns columns [256 h, 256 h + 256)
// The 32x32x16 value product reads one 1 KB operand tile per 16384 MACs, half
// of what 16-head value products need, at the same register footprint (72
// query + 128 accumulator VGPRs per wave), and no score or softmax work is
// duplicated.
//
// Schedule: waves w and w + 4 share a SIMD.  Waves 0..3 (group X) and 4..7
// (group Y) run half a block apart, so one group's score MFMAs and softmax
// overlap the other group's value MFMAs.  Two workgroup barriers per block
// serve both groups: for X they are "block ready" and "P exchanged", for Y the
// other way round.
//
// Data movement: 16-byte global->LDS DMA copies (global_load_lds_dwordx4),
// one 1 KB latent row per wave-wide copy, into a ring of four 36 KB slots;
// copies of a block are issued 2.5 blocks ahead of their first use.  Chunks
// are XOR-swizzled per row so that the row-wise score reads (ds_read_b128) and
// the transposed value reads (ds_read_b64_tr_b16) spread over the LDS banks;
// the value operand is read transposed straight out of the same tile.
//
// Split-KV: a sequence may be cut into chunks of split_tokens; each chunk
// writes (o / l in bf16, lse in fp32) partials and a combine kernel merges
// them with log-sum-exp weights in fp32.  Chunks of one sequence are placed on
// one XCD so that its L2 serves the query to all of them.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int TB = 32;                          // tokens per block
constexpr int LAT_BYTES = DC * 2;               // 1024: latent part of a row
constexpr int ROPE_BYTES = DR * 2;              // 128: rotary part of a row
constexpr int SLOT_LAT = TB * LAT_BYTES;        // 32768
constexpr int SLOT_BYTES = SLOT_LAT + TB * ROPE_BYTES;   // 36864
constexpr int NSLOT = 4;
constexpr int NDMA = TB + TB * ROPE_BYTES / 1024;        // 36 wave-wide copies per block
constexpr int KSTEPS = DROW / 32;               // 18 score k-steps of 32 dims
constexpr int KLAT = DC / 32;                   // the first 16 of them are latent
constexpr int CB = DC / 64;                     // 8 value column blocks of 32 per wave
constexpr int PX_BYTES = 8 * 32 * 8;            // P of a pair: [token quartet][head][4 tokens] bf16
constexpr int AX_BYTES = 32 * 4;                // per-head fp32 factors of a pair
constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_SLACK = 8.0f;           // log2 units a stale max may lag
constexpr int STAGE_BYTES = TB * FP8_ROW_BYTES;  // 20992: a block of packed fp8 rows
constexpr int FP8_SCALE_OFF = DC + ROPE_BYTES;   // 640: the four group scales of a packed row

// LDS slot layout for a block of 32 tokens:
//   [0, 32 KB)      latent rows, 1024 B each; 16-byte chunk c of row r sits at
//                   chunk position c ^ fl(r) (XOR inside aligned 16-chunk groups)
//   [32 KB, 36 KB)  rotary keys, 128 B each; chunk c of row r at c ^ fr(r)
// LDS bank groups on gfx950 (measured lane pair by lane pair with the
// bank-conflict counter): a 128-bit read is served 16 lanes at a time, the
// groups being the 4-lane clusters q = l / 4 in {0, 3, 5, 6}, {1, 2, 4, 7},
// {8, 11, 13, 14}, {9, 10, 12, 15}; a 64-bit write 16 consecutive lanes at a
// time.  A 16-byte chunk's bank quad is its position mod 16 (rows are 1 KB).
//   - score reads (lane l: row l % 16, chunk 4 ks + l / 16): group {0,3,5,6}
//     holds rows {0-3, 12-15} at chunk c and rows {4-11} at chunk c + 1, so
//     fl must be a bijection on r & 15 whose values on rows 4..11 are closed
//     under ^ 1;
//   - value reads: 4 aligned rows, each at one aligned 4-chunk group, need
//     bits 2..3 of fl distinct over 4 aligned rows.
// fl(r) = 4 (r & 3) + h[(r >> 2) & 3] with h = (2, 0, 1, 3) satisfies both
// (and fl(r + 4) = fl(r) ^ 2 for r % 8 < 4).  For the 128-byte rotary rows
// (two per 256-byte bank period) fr(r) = (r >> 1) & 7 spreads every read group
// over distinct (r & 1, position) pairs.
__device__ __forceinline__ int fl(int r) { return ((r & 3) << 2) | ((0xD2 >> (2 * ((r >> 2) & 3))) & 3); }
__device__ __forceinline__ int fr(int r) { return (r >> 1) & 7; }

// Pairwise reductions across lanes l ^ 16 and l ^ 32 with the gfx950 lane
// swaps (VALU; no LDS traffic).  Both lanes of a pair get the same result.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maxima of scores that are finite or -inf: v_max3_f32 / v_max_f32 as
// written (the fmaxf form quiets signalling NaNs first, one extra
// instruction per operand).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The copy (DMA) side of a decoder: which rows of a block each of the NW
// copying waves moves.
template <int NW>
struct BlockCopier {
  static constexpr int NI = (NDMA + NW - 1) / NW;       // max DMA copies per wave per block
  static_assert((NSLOT - 1) * NI <= 63, "three blocks of copies must fit the vmcnt counter");

  // Copies this wave issues per block: copies n = wave, wave + NW, ... < 36.
  __device__ __forceinline__ static int copies(int wave) { return (NDMA - wave + NW - 1) / NW; }

  // Start the DMA of the 32-token block starting at tok0 into `slot`.  Copy
  // n < 32 moves latent row n (one 1 KB row per wave-wide instruction);
  // copies 32..35 move the rotary keys of 8 rows each.  Rows past `last`
  // re-read row `last` (finite data); their scores are masked.
  __device__ __forceinline__ static void issue(const uint8_t *cache, int phys, int tok0, int last,
                                               int wave, int lane, uint8_t *slot) {
    const uint8_t *base = cache + (static_cast<size_t>(phys) * PAGE + (tok0 & 32)) * ROW_BYTES;
    const uint32_t slot_lds = lds_addr(slot);
    // Opaque copy of the lane id: keeps the compiler from hoisting the
    // per-copy offsets out of the streaming loop into registers.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = wave + i * NW;
      if (i * NW + NW <= NDMA || n < NDMA) {
        if (n < TB) {
          // row min(n, last) through a scalar base; lane offset (lane ^ fl(n)) * 16
          dma16_s(static_cast<uint32_t>((ln ^ fl(n)) << 4), base + min(n, last) * ROW_BYTES,
                  __builtin_amdgcn_readfirstlane(slot_lds + n * LAT_BYTES));
        } else {
          const int rr = (n - TB) * 8 + (ln >> 3);
          const int r = min(rr, last);
          dma16_s(static_cast<uint32_t>(r * ROW_BYTES + LAT_BYTES + (((ln & 7) ^ fr(rr)) << 4)), base,
                  __builtin_amdgcn_readfirstlane(slot_lds + SLOT_LAT + (n - TB) * 1024));
        }
      }
    }
  }
};

// The copy side of the fp8 cache.  A packed row is [512 E4M3 codes | 64 bf16
// rotary values | 4 fp32 group scales] (656 bytes) and the 32 rows of a block
// are contiguous in the page, so each of the NC copying waves moves its own
// TB / NC rows as one contiguous byte range into a staging buffer, unchanged.
// The same wave later expands exactly those rows (convert8), so the copy and
// the expansion need no workgroup barrier between them.
template <int NC>
struct Fp8Copier {
  static constexpr int ROWS = TB / NC;                          // rows per copying wave
  static constexpr int CHUNKS = ROWS * FP8_ROW_BYTES / 16;      // 16-byte pieces per wave
  static constexpr int NI = (CHUNKS + 63) / 64;                 // wave-wide copies per block
  static constexpr int TAIL = CHUNKS - (NI - 1) * 64;           // active lanes of the last copy
  static_assert(ROWS * FP8_ROW_BYTES % 16 == 0 && 2 * NI <= 63, "copy ranges");

  // Rows past the end of the sequence are copied too (they lie inside the
  // page) and discarded by the expansion.
  __device__ __forceinline__ static void issue(const uint8_t *cache, int phys, int tok0, int wave, int lane,
                                               uint8_t *stage) {
    const uint8_t *src = cache + (static_cast<size_t>(phys) * PAGE + (tok0 & 32) + wave * ROWS) * FP8_ROW_BYTES;
    const uint32_t dst = lds_addr(stage + wave * ROWS * FP8_ROW_BYTES);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + 1 < NI || ln < TAIL)
        dma16_s(static_cast<uint32_t>((i * 64 + ln) * 16), src, __builtin_amdgcn_readfirstlane(dst + i * 1024));
    }
  }
};

// One wave: scores and softmax for 16 heads, values for its pair's 32 heads
// over half of the columns.
//   MFMA 16x16x32 bf16: A/B lane l: row/column l % 16, k = 8 (l / 16) + j;
//                       C register i: row 4 (l / 16) + i, column l % 16.
//   MFMA 32x32x16 bf16: A/B lane l: row/column l % 32, k = 8 (l / 32) + j;
//                       C register i: row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
template <int NW_>
struct DecoderPair {
  static constexpr int NW = NW_;
  static constexpr int HEADS = NW * 16;          // heads per workgroup
  // Copying waves.  A global->LDS copy stalls at issue while the memory pipe
  // is full, and a stalled wave issues no MFMAs; with 8 waves only group X
  // (which otherwise waits for group Y at the first barrier) copies.
  static constexpr int NC = NW == 8 ? 4 : NW;
  static constexpr int NI = BlockCopier<NC>::NI;
  static constexpr int NI8 = Fp8Copier<NC>::NI;

  const DecodeArgs &a;
  const int wave, half;                          // wave-uniform
  const int b, split;
  const int seq_len, t_begin, t_end;
  const int32_t *bt_row;                         // block-table row of the sequence
  uint8_t *px;                                   // LDS: this pair's P tile
  float *ax;                                     // LDS: this pair's per-head rescale factors
  float *fx;                                     // LDS: this pair's per-head 1 / l

  bf16x8 qf[KSTEPS];
  f32x16 o[CB];
  f32x4 s0, s1;               // scores of the block's two 16-token halves
  // Per scoring lane (head l % 16, tokens 4 (l / 16) + i and 16 + 4 (l / 16) + i):
  // m_run: running max of the head (log2 units); l_run: its share of the sum
  // of the bf16-rounded weights that multiply V; e_run: the same sum of the
  // unrounded weights (gives an lse free of the bf16 rounding of P).
  float m_run, l_run, e_run;

  __device__ DecoderPair(const DecodeArgs &args, uint8_t *px_, float *ax_, float *fx_, int b_, int split_, int S,
                         int t0, int t1)
      : a(args), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        half(__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 1)),
        b(b_), split(split_), seq_len(S), t_begin(t0), t_end(t1),
        bt_row(args.block_table + static_cast<size_t>(b_) * args.max_blocks),
        px(px_ + (threadIdx.x >> 7) * PX_BYTES), ax(ax_ + (threadIdx.x >> 7) * 32),
        fx(fx_ + (threadIdx.x >> 7) * 32) {}

  // Per-lane quantities are recomputed where they are used rather than held
  // in registers across the streaming loop; the opaque lane id keeps the
  // compiler from hoisting them back out of it.
  __device__ __forceinline__ static int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
  }
  // head scored by lane l, and the pair head a 32-wide lane layout maps to lane l
  __device__ __forceinline__ int score_head(int l) const { return blockIdx.y * HEADS + wave * 16 + (l & 15); }
  __device__ __forceinline__ int pair_head(int l) const { return blockIdx.y * HEADS + (wave >> 1) * 32 + (l & 31); }
  // End (exclusive token index) of what query row v sees in this chunk: the
  // chunk end for a single new token; with q_len new tokens, row v (token
  // j = v / heads) does not see the q_len - 1 - j newest ones.  vis_min: the
  // smallest of these over the rows (that of token 0).
  __device__ __forceinline__ int vis_end(int v) const {
    return a.q_len <= 1 ? t_end : min(t_end, seq_len - (a.q_len - 1) + v / a.heads);
  }
  __device__ __forceinline__ int vis_min() const {
    return a.q_len <= 1 ? t_end : min(t_end, seq_len - (a.q_len - 1));
  }

  // LDS byte offsets of the first read of each kind.  Every other read is one
  // of these XOR a compile-time constant plus an immediate: the XOR acts on
  // address bits that the base's remaining terms leave zero.
  //   latent score reads, k-step ks < 16: row r = l % 16 (+16), chunk 4 ks + g
  //   (g = l / 16) at position (4 (ks & 3) ^ (fl & 12)) + (g ^ (fl & 3)):
  //   k_base ^ 64 (ks & 3), + 256 (ks >> 2), + 16 KB for rows 16..31
  __device__ __forceinline__ static int k_base(int l) {
    const int r = l & 15, g = l >> 4, f = fl(r);
    return r * LAT_BYTES + (((f & 12) | (g ^ (f & 3))) << 4);
  }
  //   rotary score reads, k-steps 16, 17: chunk 4 (ks - 16) + g of row r, at
  //   position (4 (ks - 16) ^ (fr & 4)) + (g ^ (fr & 3)): kr_base ^ 64 (ks - 16),
  //   + 2 KB for rows 16..31
  __device__ __forceinline__ static int kr_base(int l) {
    const int r = l & 15, g = l >> 4, f = fr(r);
    return SLOT_LAT + r * ROPE_BYTES + (((f & 4) | (g ^ (f & 3))) << 4);
  }
  //   value reads (transposed, lane l supplies one address): row
  //   16 t + 8 (l / 32) + 4 hi + (l & 15) / 4, latent chunk of column block
  //   cb = 8 half + j: 4 cb + 2 ((l >> 4) & 1) + (l & 3) / 2, byte 8 (l & 1):
  //   v_base ^ 64 (j & 3), + 256 (j >> 2), + 16 KB t; the hi rows sit 4 rows
  //   further, where fl(row + 4) = fl(row) ^ 2: ^ 32, + 4 KB
  __device__ __forceinline__ int v_base(int l) const {
    const int row0 = 8 * (l >> 5) + ((l & 15) >> 2);
    const int fv = fl(row0);
    const int csub = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    return row0 * LAT_BYTES + half * 512 + (((fv & 12) | (csub ^ (fv & 3))) << 4) + 8 * (l & 1);
  }

  __device__ __forceinline__ void begin() {
    m_run = -FLT_MAX;         // finite: a row whose tokens are all masked keeps weights exp2(-inf) = 0
    l_run = 0.f;
    e_run = 0.f;
#pragma unroll
    for (int j = 0; j < CB; ++j) o[j] = f32x16{};
  }

  // Query fragments (16x16x32 B operand): lane (head l % 16, g = l / 16) holds
  // dims 32 ks + 8 g + [0, 8).
  __device__ __forceinline__ void load_q() {
    const int l = threadIdx.x & 63, head = score_head(l);
    const bool head_ok = head < a.H;
    const uint16_t *qp = a.q + (static_cast<size_t>(b) * a.H + (head_ok ? head : 0)) * DROW + (l >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 32);
      if (!head_ok) v = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __device__ __forceinline__ int copies() const { return wave < NC ? BlockCopier<NC>::copies(wave) : 0; }

  // Physical page of block blk: a scalar load from the block table, issued a
  // step before the copy that needs it so its latency stays off the LDS path.
  __device__ __forceinline__ int page_of(int blk) const {
    return ((const_i32 *)bt_row)[(t_begin + blk * TB) >> 6];
  }

  __device__ __forceinline__ void issue(int blk, int phys, uint8_t *slot) {
    const int tok0 = t_begin + blk * TB;
    if (wave < NC) BlockCopier<NC>::issue(a.cache, phys, tok0, min(TB, t_end - tok0) - 1, wave, threadIdx.x & 63, slot);
  }

  // fp8 cache: start the copy of block blk's packed rows into `stage`.
  __device__ __forceinline__ void issue8(int blk, int phys, uint8_t *stage) {
    if (wave < NC) Fp8Copier<NC>::issue(a.cache, phys, t_begin + blk * TB, wave, threadIdx.x & 63, stage);
  }

  // fp8 cache: expand this wave's rows of block blk from `stage` into the
  // bf16 slot layout the score and value reads expect.  Latent value j of a
  // row is code_j * scale[j / 128] formed in fp32 and rounded to bf16 (the
  // E4M3 code converts to fp32 exactly); the rotary part is copied.  Rows
  // past the end of the chunk become zeros, so their masked scores meet
  // finite values.  Lane l handles 16-byte output chunk l of each latent row.
  __device__ __forceinline__ void convert8(int blk, const uint8_t *stage, uint8_t *slot) {
    if (wave >= NC) return;
    constexpr int ROWS = Fp8Copier<NC>::ROWS;
    const int tok0 = t_begin + blk * TB;
    const int last = min(TB, t_end - tok0) - 1;
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      const int r = wave * ROWS + k;
      u32x4 out = u32x4{0, 0, 0, 0};
      if (r <= last) {
        const uint8_t *src = stage + r * FP8_ROW_BYTES;
        const u32x2 codes = *reinterpret_cast<const u32x2 *>(src + l * 8);
        const float sc = *reinterpret_cast<const float *>(src + FP8_SCALE_OFF + (l >> 4) * 4);
        bf16x8 v;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[h]), false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[h]), true);
          v[4 * h + 0] = to_bf16(lo[0] * sc);
          v[4 * h + 1] = to_bf16(lo[1] * sc);
          v[4 * h + 2] = to_bf16(hi[0] * sc);
          v[4 * h + 3] = to_bf16(hi[1] * sc);
        }
        out = __builtin_bit_cast(u32x4, v);
      }
      *reinterpret_cast<u32x4 *>(slot + r * LAT_BYTES + ((l ^ fl(r)) << 4)) = out;
    }
#pragma unroll
    for (int n0 = 0; n0 < ROWS * 8; n0 += 64) {
      const int n = n0 + l;
      const int r = wave * ROWS + (n >> 3), c = n & 7;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (r <= last) v = *reinterpret_cast<const u32x4 *>(stage + r * FP8_ROW_BYTES + DC + c * 16);
      *reinterpret_cast<u32x4 *>(slot + SLOT_LAT + r * ROPE_BYTES + ((c ^ fr(r)) << 4)) = v;
    }
  }

  // Scores of this wave's 16 heads for the block in `slot`, online softmax,
  // then P and the rescale factors published to the pair's exchange tiles.
  __device__ __forceinline__ void scores_softmax(const uint8_t *slot, int blk) {
    const int l = lane_id(), g = l >> 4;
    const int kb = k_base(l), krb = kr_base(l);
    // Operands stream through a ring PF k-steps deep so LDS latency overlaps
    // earlier MFMAs; the empty asm ties each MFMA operand to its place in the
    // ring (without it the scheduler sinks every read to just before its use).
    auto kread = [&](int ks, int hi) -> bf16x8 {
      const uint8_t *kp = ks < KLAT ? slot + (kb ^ ((ks & 3) * 64)) + (ks >> 2) * 256 + hi * 16 * LAT_BYTES
                                    : slot + (krb ^ ((ks - KLAT) * 64)) + hi * 16 * ROPE_BYTES;
      return *reinterpret_cast<const bf16x8 *>(kp);
    };
    constexpr int PF = 2;
    bf16x8 k0[KSTEPS], k1[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) {
      k0[ks] = kread(ks, 0);
      k1[ks] = kread(ks, 1);
    }
    s0 = f32x4{};
    s1 = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + PF < KSTEPS) {
        k0[ks + PF] = kread(ks + PF, 0);
        k1[ks + PF] = kread(ks + PF, 1);
      }
      asm volatile("" : "+v"(k0[ks]), "+v"(k1[ks]) : : "memory");
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[ks], qf[ks], s1, 0, 0, 0);
    }

    // ---- online softmax.  Scores stay unscaled: the scale c = softmax_scale *
    // log2(e) > 0 enters the running max (max(c s) = c max(s)) and the exponent
    // as one fma.
    const int tok0 = t_begin + blk * TB;
    const float c = a.scale_log2;
    if (tok0 + TB > vis_min()) [[unlikely]] {
      // last block of the chunk (tokens at or past t_end do not exist), or a
      // block holding new tokens that some multi-token rows do not see
      const int lim = vis_end(score_head(l)) - tok0 - 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= lim) s0[i] = -INFINITY;
        if (16 + i >= lim) s1[i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = max_xor32(max_xor16(mx)) * c;
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.0f;
    if (m_new > m_run + RESCALE_SLACK) {
      alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      e_run *= alpha;
      m_run = m_new;
    }
    bf16x4 p0, p1;
    float pe = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -m_run));
      const float f1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -m_run));
      pe += f0 + f1;
      p0[i] = to_bf16(f0);
      p1[i] = to_bf16(f1);
    }
    // sum of the rounded weights: bf16 pairs dotted with (1, 1)
    const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float ps = l_run;
    ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[0], p0[1]}, one2, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[2], p0[3]}, one2, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[0], p1[1]}, one2, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[2], p1[3]}, one2, ps, false);
    l_run = ps;
    e_run += pe;

    // ---- publish.  P tile of the pair: quartet k = token / 4, 8 bytes per
    // (quartet, pair head), P[token][head] at ((k * 32 + head) * 8 + 2 (token % 4)):
    // 16 consecutive lanes write 16 consecutive 8-byte slots.  This lane holds
    // quartets g (tokens 4 g + i) and 4 + g (tokens 16 + 4 g + i).
    const int ph = half * 16 + (l & 15);
    uint8_t *pw = px + (g * 32 + ph) * 8;
    *reinterpret_cast<bf16x4 *>(pw) = p0;
    *reinterpret_cast<bf16x4 *>(pw + 4 * 32 * 8) = p1;
    if (g == 0) ax[ph] = alpha;
  }

  // After the pair's P is visible: rescale if any of the pair's heads moved
  // its max, then the value product of the block in `slot`.
  __device__ __forceinline__ void values(const uint8_t *slot) {
    const int l = lane_id();
    const int vb = v_base(l);
    // B operand of token step t: lane (pair head l % 32, hb = l / 32) holds
    // tokens 16 t + 8 hb + [0, 8): quartets 4 t + 2 hb and 4 t + 2 hb + 1.
    auto pread = [&](int k) -> bf16x4 {
      return *reinterpret_cast<const bf16x4 *>(px + (k * 32 + (l & 31)) * 8);
    };
    const int q0 = 2 * (l >> 5);
    const bf16x4 p00 = pread(q0), p01 = pread(q0 + 1), p10 = pread(q0 + 4), p11 = pread(q0 + 5);
    const bf16x8 pb0 = __builtin_shufflevector(p00, p01, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 pb1 = __builtin_shufflevector(p10, p11, 0, 1, 2, 3, 4, 5, 6, 7);
    const float alpha = ax[l & 31];
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < CB; ++j) o[j] *= alpha;
    }
    // A operand: a transposed read returns 4 consecutive tokens of one column
    // per lane: "lo" covers tokens 16 t + 8 hb + [0, 4), "hi" the next 4.
    auto vread = [&](int n) -> bf16x8 {
      const int j = n & 7, t = n >> 3;
      const int x = vb ^ ((j & 3) * 64);
      const uint8_t *r0 = slot + x + (j >> 2) * 256 + t * 16 * LAT_BYTES;
      const uint8_t *r1 = slot + (x ^ 32) + (j >> 2) * 256 + t * 16 * LAT_BYTES + 4 * LAT_BYTES;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r1);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // n = 8 t + j: consecutive MFMAs go to different accumulators.
    constexpr int PV = 3;
    constexpr int NV = 2 * CB;
    bf16x8 vf[NV];
#pragma unroll
    for (int n = 0; n < PV; ++n) vf[n] = vread(n);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + PV < NV) vf[n + PV] = vread(n + PV);
      asm volatile("" : "+v"(vf[n]) : : "memory");
      o[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n], n < 8 ? pb0 : pb1, o[n & 7], 0, 0, 0);
    }
  }

  // Normalise and store.  The scoring lanes publish 1 / l of their heads
  // (to tiles of their own, as the partner wave may still be reading the
  // rescale factors) and write lse.  Lane (pair head l % 32, hb) holds
  // columns 32 (8 half + j) + 8 q + 4 hb + [0, 4) in registers 4 q .. 4 q + 3
  // of o[j]: stored directly, every instruction would scatter 16-byte pieces
  // over 32 rows.  The tile goes through LDS instead (`stage`, the free slot
  // ring: row = head of the workgroup, 1 KB, chunk c at position c ^ (row &
  // 15)), and each wave then writes 16 whole rows, 1 KB per instruction.
  // Every wave of the workgroup calls this once (it contains barriers).
  __device__ __forceinline__ void finish(uint8_t *stage) {
    const int l = threadIdx.x & 63;
    const float l_tot = sum_xor32(sum_xor16(l_run));
    const float e_tot = sum_xor32(sum_xor16(e_run));
    const int sh = score_head(l);
    // l_tot >= 1 unless the row saw no token of the chunk (a multi-token row
    // past its position): then o = 0 and lse = log 0 = -inf
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = (m_run + __log2f(e_tot)) * LN2;
    if (l < 16) {
      fx[half * 16 + l] = inv;
      if (sh < a.H) {
        if (a.direct) {
          if (a.lse) a.lse[static_cast<size_t>(b) * a.H + sh] = lse_v;
        } else {
          a.lse_part[(static_cast<size_t>(b) * a.n_splits + split) * a.H + sh] = lse_v;
        }
      }
    }
    barrier_lds();            // 1 / l visible; every wave is done with the slots
    const float scale = fx[l & 31];
    const int row = (wave >> 1) * 32 + (l & 31);
    uint8_t *srow = stage + row * LAT_BYTES + (l >> 5) * 8;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[j][4 * q + e] * scale);
        const int c = half * 32 + j * 4 + q;                  // 16-byte chunk of the row
        *reinterpret_cast<bf16x4 *>(srow + ((c ^ (row & 15)) << 4)) = v;
      }
    }
    barrier_lds();
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const int r = wave * 16 + k;
      const int head = blockIdx.y * HEADS + r;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * LAT_BYTES + ((l ^ (r & 15)) << 4));
      if (head < a.H) {
        uint16_t *dst = a.direct ? a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC
                                 : a.o_part + ((static_cast<size_t>(b) * a.n_splits + split) * a.H + head) * DC;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + l * 8));
      }
    }
  }
};

// One wave per SIMD: 4 waves of 32 heads each (128 heads per workgroup), 512
// registers per lane.  Both products use v_mfma_f32_32x32x16_bf16 with the
// heads as the 32-wide N dimension, so every 1 KB operand tile read from LDS
// feeds 32 heads, and no wave exchanges anything with another.
//   scores   S^T[row, head] = K[row, 0:576] . Q^T over 36 k-steps of 16 dims;
//            the query fragments (144 VGPRs) stay in registers
//   softmax  on the score accumulator: lane (head l % 32, hb = l / 32) holds
//            K-rows 8 (i / 4) + 4 hb + i % 4 of register i
//   values   O^T[col, head] += V^T[col, row] . P^T[row, head]; registers
//            8 t .. 8 t + 7 of the score accumulator, rounded to bf16, are the
//            B operand of token step t as they stand
//   16 column tiles x 16 registers of accumulators per lane (256 AGPRs).
// A single wave per SIMD issues at most one instruction per four cycles, and
// a 32x32x16 MFMA lasts eight of those issue slots, so the operand reads are
// laid out to need no address arithmetic: every read is a per-lane base
// register plus an immediate offset.
//
// Slot layout (one 32-token block): latent rows at a padded stride of
// 1040 bytes (the 16-byte pad puts row r's chunk c on bank quad (r + c) % 16),
// then the rotary keys, 128 bytes per row, chunk c of row r at c ^ fr(r).
// Token n of the block is stored in row n.  The MFMA's K-row m is token
// pi(m): with m = 16 t + 8 h + 4 b + d, pi(m) = 16 b + 4 d + 2 t + h.
//   - score reads: lane l reads row pi(l % 32), chunk 2 ks + l / 32; each
//     16-lane read group covers the residues of its 16 rows mod 16 once, so
//     no two lanes share a bank quad;
//   - value reads (transposed): the lo/hi reads of token step t cover rows
//     16 hb + 4 d + 2 t (+ 1 for hi), d = 0..3 -- four rows 4 apart, so the
//     4 x 4 chunks of 32 lanes fall on 16 distinct bank quads, and the rows
//     are exactly the K-rows of score registers 8 t .. 8 t + 7 in the order
//     the B operand expects.
// A stale running max may lag the true one by up to 32 (log2 units) before
// the value accumulators are rescaled: weights stay below 2^32 and sums of
// them below 2^51 times the largest latent value, far inside fp32, and the
// rescale (which touches all 256 accumulator registers) becomes rare.
constexpr float SOLO_SLACK = 32.0f;
constexpr int S_LROW = LAT_BYTES + 16;               // 1040
constexpr int S_LAT = TB * S_LROW;                   // 33280
constexpr int S_SLOT = S_LAT + TB * ROPE_BYTES;      // 37376
__device__ __forceinline__ int solo_pi(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m & 3) + 2 * ((m >> 4) & 1) + ((m >> 3) & 1);
}

struct DecoderSolo {
  static constexpr int NW = 4;
  static constexpr int HEADS = 128;
  static constexpr int NI = TB / NW + 1;           // copies per wave per block
  static constexpr int KS = DROW / 16;             // 36 score k-steps
  static constexpr int KSL = DC / 16;              // the first 32 are latent
  static constexpr int NT = DC / 32;               // 16 value column tiles
  static_assert(NI * NW == NDMA && 3 * NI <= 63, "every wave copies the same share of a block");
  static_assert(3 * (NI - 1) + 1 < 2 * (DC / 32), "every copy of a block is issued among its value MFMAs");

  const DecodeArgs &a;
  const int wave;
  const int b, split, grp;
  const int seq_len, t_begin, t_end;
  const int32_t *bt_row;

  bf16x8 qf[KS];
  f32x16 o[NT];
  // Per lane (head l % 32; lanes l and l + 32 share a head and hold the same
  // m_run): running max (log2 units), this lane's share of the sum of the
  // bf16-rounded weights and of the unrounded weights.
  float m_run, l_run, e_run;
  // Per-lane LDS offsets of the score (latent, rotary) and value operand
  // reads within a slot, formed once: recomputing them in every block cost
  // about 20 VALU instructions per block.
  int kb_, krb_, vb_;
  uint32_t voff_, roff_full_;   // full-block copy offsets (latent rows, rotary rows)

  __device__ DecoderSolo(const DecodeArgs &args, int b_, int split_, int grp_, int S, int t0, int t1)
      : a(args), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)), b(b_), split(split_), grp(grp_),
        seq_len(S), t_begin(t0), t_end(t1),
        bt_row(args.block_table + static_cast<size_t>(b_) * args.max_blocks) {}

  __device__ __forceinline__ static int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
  }
  __device__ __forceinline__ static int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
  }
  __device__ __forceinline__ int head_of(int l) const { return grp * HEADS + wave * 32 + (l & 31); }
  // Tokens of this chunk that the query row of lane l sees: all of them for
  // a single new token; with q_len new tokens, row v (token j = v / heads)
  // does not see the q_len - 1 - j newest ones.
  __device__ __forceinline__ int visible(int l) const {
    if (a.q_len <= 1) return t_end - t_begin;
    const int v = head_of(l);
    return min(t_end, seq_len - (a.q_len - 1) + v / a.heads) - t_begin;
  }
  // Mask limit for block blk: token 16 hb + n of the block is visible while
  // n < limit (lanes l and l + 32 hold the token halves hb = 0, 1).
  __device__ __forceinline__ int mask_limit(int l, int blk) const {
    return visible(l) - blk * TB - 16 * ((l >> 5) & 1);
  }

  __device__ __forceinline__ void begin() {
    m_run = -FLT_MAX;         // finite: a row whose tokens are all masked keeps weights exp2(-inf) = 0
    l_run = 0.f;
    e_run = 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) o[j] = f32x16{};
    const int l = lane_id();
    kb_ = k_base(l);
    krb_ = kr_base(l);
    vb_ = v_base(l);
    voff_ = static_cast<uint32_t>(l << 4);
    roff_full_ = rope_voff_full(l);
  }

  // Query through LDS.  Read straight into the MFMA layout, every query load
  // would touch 32 head rows (32 bytes of each), and the 36 loads of a wave
  // would fetch each 128-byte line four times.  Instead each wave copies its
  // 32 heads' rows (36 KB, contiguous in q) into LDS with whole-1 KB copies,
  // then reads its fragments from there.  Staging layout: 16-byte chunk c of
  // row r (head of the workgroup) at chunk position 72 (r - row0) +
  // (c ^ qs(r)), qs(r) = (r >> 1) & 7, so a fragment read (16 rows at one
  // chunk index) meets 16 distinct bank quads.  Rows past H re-read row
  // H - 1.  row0 is the first row the staging area holds (waves stage in two
  // halves of 64 rows, 73,728 bytes).
  static constexpr int Q_CHUNKS = DROW / 8;                     // 72 chunks of 16 bytes per row
  static constexpr int Q_WAVE_BYTES = 32 * DROW * 2;            // 36,864: one wave's heads
  static constexpr int Q_COPIES = Q_WAVE_BYTES / 1024;          // 36 copies per wave
  __device__ __forceinline__ static int qs(int r) { return (r >> 1) & 7; }
  __device__ __forceinline__ void load_q_lds(uint8_t *stage, int row0) {
    const int l = threadIdx.x & 63;
    const uint8_t *rows = reinterpret_cast<const uint8_t *>(a.q + (static_cast<size_t>(b) * a.H + grp * HEADS) * DROW);
    const int last = min(HEADS, a.H - grp * HEADS) - 1;
    const uint32_t dst = lds_addr(stage) + (wave * 32 - row0) * (DROW * 2);
#pragma unroll
    for (int k = 0; k < Q_COPIES; ++k) {
      const int pos = wave * (Q_WAVE_BYTES / 16) + 64 * k + l;   // chunk position of row 0-based staging
      const int r = pos / Q_CHUNKS, c = (pos - r * Q_CHUNKS) ^ qs(r);
      dma16_s(static_cast<uint32_t>(min(r, last) * (DROW * 2) + c * 16), rows,
              __builtin_amdgcn_readfirstlane(dst + 1024 * k));
    }
  }
  // Fragments from the staging area (after this wave's copies have landed).
  __device__ __forceinline__ void read_q_lds(const uint8_t *stage, int row0) {
    const int l = threadIdx.x & 63;
    const int r = wave * 32 + (l & 31), hb = l >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 2 * ks + hb;
      qf[ks] = *reinterpret_cast<const bf16x8 *>(stage + 16 * ((r - row0) * Q_CHUNKS + (c ^ qs(r))));
    }
  }


  __device__ __forceinline__ int page_of(int blk) const {
    return ((const_i32 *)bt_row)[(t_begin + blk * TB) >> 6];
  }

  // Copies of a block into its slot: wave w moves latent rows w + 4 k
  // (k = 0..7, one 1 KB row per wave-wide copy, to row w + 4 k of the slot)
  // and the rotary keys of rows 8 w .. 8 w + 7 (copy k = 8).  Rows past the
  // end of the chunk re-read its last row (finite data, masked scores).
  struct Copy {
    const uint8_t *base;       // first row of the block in its page
    uint32_t slot_lds;
    int last;                  // last valid row of the block
  };
  __device__ __forceinline__ Copy copy_of(int blk, int phys, uint8_t *slot) const {
    const int tok0 = t_begin + blk * TB;
    return Copy{a.cache + (static_cast<size_t>(phys) * PAGE + (tok0 & 32)) * ROW_BYTES, lds_addr(slot),
                min(TB, t_end - tok0) - 1};
  }
  // voff: this lane's byte offset in a latent row (16 * lane); roff: its
  // offset for the rotary copy (row min(8 w + l / 8, last), chunk l % 8 of
  // the rotary part, stored at chunk (l % 8) ^ fr(row)).
  __device__ __forceinline__ uint32_t rope_voff(const Copy &c, int l) const {
    const int rr = wave * 8 + (l >> 3);
    return static_cast<uint32_t>(min(rr, c.last) * ROW_BYTES + LAT_BYTES + (((l & 7) ^ fr(rr)) << 4));
  }
  __device__ __forceinline__ void copy(const Copy &c, int k, uint32_t voff, uint32_t roff) const {
    if (k < TB / NW) {
      const int n = wave + NW * k;
      dma16_s(voff, c.base + min(n, c.last) * ROW_BYTES, __builtin_amdgcn_readfirstlane(c.slot_lds + n * S_LROW));
    } else {
      dma16_s(roff, c.base, __builtin_amdgcn_readfirstlane(c.slot_lds + S_LAT + wave * 1024));
    }
  }
  __device__ __forceinline__ void issue(int blk, int phys, uint8_t *slot) const {
    const Copy c = copy_of(blk, phys, slot);
    const int l = lane_id();
    const uint32_t voff = static_cast<uint32_t>(l << 4), roff = rope_voff(c, l);
#pragma unroll
    for (int k = 0; k < NI; ++k) copy(c, k, voff, roff);
  }

  // Blocks with every row inside the chunk take a shorter copy: a buffer
  // resource based at this wave's first row of the block (row w), the row
  // offsets of copies k = 1..7 (4 k rows) and of the rotary copy (7 w rows)
  // in SGPRs set once per workgroup (a buffer load's SGPR offset moves the
  // global address only, not the LDS one), so a copy is an M0 update and the
  // load, where the clamped form forms each row's 64-bit address.
  struct FullCopy {
    i32x4 rsrc;           // raw buffer at row w of the block
    uint32_t m0_lat;      // LDS address of slot row w
    uint32_t m0_rope;     // LDS address of this wave's rotary rows in the slot
  };
  uint32_t soff_[NI];     // soff_[k]: 4 k rows (k < 8); soff_[8]: 7 w rows
  __device__ __forceinline__ static uint32_t sgpr_const(uint32_t x) {
    asm volatile("s_mov_b32 %0, %1" : "=s"(x) : "s"(x));
    return x;
  }
  __device__ __forceinline__ void init_full_copy() {
#pragma unroll
    for (int k = 1; k < NI - 1; ++k) soff_[k] = sgpr_const(k * NW * ROW_BYTES);
    soff_[NI - 1] = sgpr_const(__builtin_amdgcn_readfirstlane(7 * wave * ROW_BYTES));
  }
  __device__ __forceinline__ FullCopy full_copy_of(int blk, int phys, uint8_t *slot) const {
    const int tok0 = t_begin + blk * TB;
    const uint64_t p = reinterpret_cast<uint64_t>(a.cache) +
                       (static_cast<uint64_t>(phys) * PAGE + (tok0 & 32) + wave) * ROW_BYTES;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xFFFF));
    r[2] = -1;                    // num_records: no range check (offsets stay inside the page)
    r[3] = 0x00020000;            // raw buffer, 32-bit data format
    const uint32_t s = lds_addr(slot);
    return FullCopy{r, static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(s + wave * S_LROW)),
                    static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(s + S_LAT + wave * 1024))};
  }
  // Rotary copy offset of lane l relative to row w + 7 w = 8 w: row l / 8 of
  // the wave's eight, chunk l % 8 stored at chunk (l % 8) ^ fr(row).
  __device__ __forceinline__ uint32_t rope_voff_full(int l) const {
    const int j = l >> 3;
    return static_cast<uint32_t>(j * ROW_BYTES + LAT_BYTES + (((l & 7) ^ fr(wave * 8 + j)) << 4));
  }
  // M0 (the LDS address of a copy) is set one copy ahead: copy k issues its
  // load and then sets M0 for copy k + 1, so the MFMAs between two copies
  // stand in for the wait state an M0 write needs before an LDS DMA.  The
  // compiler itself never uses M0 in these kernels, so the value survives
  // between the statements.
  __device__ __forceinline__ void copy_full_m0(const FullCopy &f) const {
    asm volatile("s_mov_b32 m0, %0" : : "s"(f.m0_lat) : "memory", "m0");
  }
  __device__ __forceinline__ void copy_full(const FullCopy &f, int k, uint32_t voff, uint32_t roff) const {
    if (k == 0)
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_add_i32 m0, %2, %3"
                   : : "v"(voff), "s"(f.rsrc), "s"(f.m0_lat), "i"(NW * S_LROW) : "memory", "m0");
    else if (k < TB / NW - 1)
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds\n\ts_add_i32 m0, %3, %4"
                   : : "v"(voff), "s"(f.rsrc), "s"(soff_[k]), "s"(f.m0_lat), "i"((k + 1) * NW * S_LROW)
                   : "memory", "m0");
    else if (k == TB / NW - 1)
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds\n\ts_mov_b32 m0, %3"
                   : : "v"(voff), "s"(f.rsrc), "s"(soff_[k]), "s"(f.m0_rope) : "memory", "m0");
    else
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                   : : "v"(roff), "s"(f.rsrc), "s"(soff_[NI - 1]) : "memory", "m0");
  }

  // MFMAs are written out so that their order is the program order (the
  // loads between them are pinned by the memory clobber) and so that the
  // score accumulator stays in VGPRs (the builtin would take the accumulator
  // form, and the 256 value accumulators fill the AGPR file).  The score
  // accumulator lives in fixed registers (v[16:31]) so that the compiler
  // never copies it between two MFMAs of its chain.  The last MFMA of a chain
  // whose result compiler-generated code reads carries the result wait states
  // in the same asm statement: the compiler cannot see that an asm MFMA is
  // still writing its output.  "nop" adds the wait states a VALU write of an
  // operand needs right before an MFMA (the first MFMA after the softmax).
#define MLA_MFMA_WAIT "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
  __device__ __forceinline__ static void mfma_s(f32x16 &s, bf16x8 k, bf16x8 q, bool first, bool last) {
    if (first)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                   : "=&{v[16:31]}"(s) : "v"(k), "v"(q) : "memory");
    else if (!last)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+{v[16:31]}"(s) : "v"(k), "v"(q) : "memory");
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" MLA_MFMA_WAIT
                   : "+{v[16:31]}"(s) : "v"(k), "v"(q) : "memory");
  }
  // The same chain pinned to v[16:31] (PAR 0) or v[32:47] (PAR 1), with no
  // result wait states on its last MFMA: the phase loop alternates the two so
  // that a block's scores stay where the chain left them (no copy), and the
  // first read of them comes a value phase later.
  template <int PAR>
  __device__ __forceinline__ static void mfma_sp(f32x16 &s, bf16x8 k, bf16x8 q, bool first) {
    if (PAR == 0) {
      if (first)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                     : "=&{v[16:31]}"(s) : "v"(k), "v"(q) : "memory");
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{v[16:31]}"(s) : "v"(k), "v"(q) : "memory");
    } else {
      if (first)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                     : "=&{v[32:47]}"(s) : "v"(k), "v"(q) : "memory");
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{v[32:47]}"(s) : "v"(k), "v"(q) : "memory");
    }
  }
  __device__ __forceinline__ static void mfma_o(f32x16 &acc, bf16x8 v, bf16x8 p, bool nop, bool last) {
    if (nop)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p) : "memory");
    else if (!last)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p) : "memory");
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" MLA_MFMA_WAIT
                   : "+a"(acc) : "v"(v), "v"(p) : "memory");
  }
#undef MLA_MFMA_WAIT
  // Orders every later read of the value accumulators after the asm MFMAs
  // issued before it.
  __device__ __forceinline__ void fence_o() {
#pragma unroll
    for (int j = 0; j < NT; ++j) asm volatile("" : "+a"(o[j]) : : "memory");
  }

  // Score operand of k-step ks (A of S^T = K Q^T): lane l, K-row m = l % 32,
  // reads row pi(m), 16-byte chunk 2 ks + l / 32: k_base + 32 ks.  Rotary
  // k-steps (ks >= 32): chunk c = 2 (ks - 32) + l / 32 at c ^ fr(row):
  // kr_base ^ 32 (ks - 32).
  __device__ __forceinline__ static int k_base(int l) {
    return solo_pi(l & 31) * S_LROW + 16 * (l >> 5);
  }
  __device__ __forceinline__ static int kr_base(int l) {
    const int r = solo_pi(l & 31);
    return S_LAT + r * ROPE_BYTES + (((l >> 5) ^ fr(r)) << 4);
  }
  __device__ __forceinline__ static bf16x8 kread(const uint8_t *slot, int kb, int krb, int ks) {
    const uint8_t *p = ks < KSL ? slot + kb + 32 * ks : slot + (krb ^ ((ks - KSL) * 32));
    return *reinterpret_cast<const bf16x8 *>(p);
  }
  // Value operand n = 16 t + j (column tile j, token step t; A of
  // O^T += V^T P^T): a transposed read returns column 32 j + l % 32 of the
  // 4 rows supplied by the lane quads of its 16-lane group.  Lane l supplies
  // row 16 hb + 4 d + 2 t (d = (l & 15) / 4; + 1 for the hi read), chunk
  // 4 j + csub, csub = 2 ((l >> 4) & 1) + (l & 3) / 2, byte 8 (l & 1):
  // v_base + 2080 t + 64 j, hi + 1040.
  __device__ __forceinline__ static int v_base(int l) {
    const int row = 16 * (l >> 5) + 4 * ((l & 15) >> 2);
    const int csub = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    return row * S_LROW + 16 * csub + 8 * (l & 1);
  }
  __device__ __forceinline__ static bf16x8 vread(const uint8_t *slot, int vb, int n) {
    const int j = n & 15, t = n >> 4;
    const uint8_t *r0 = slot + vb + 2 * t * S_LROW + 64 * j;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + S_LROW));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // Online-softmax state of the block whose scores are in the score
  // accumulator.  Register i of lane (head, hb) holds the score of token
  // pi(8 (i / 4) + 4 hb + i % 4) = 16 hb + 4 (i % 4) + 2 (i / 8) + (i / 4) % 2.
  // The max update is branch-free (the lazy rescale of the value
  // accumulators by alpha happens before the next value product).
  struct Soft {
    float mx, alpha, pe;
    bf16x8 p[2];
  };
  // Step k (0..13) of the softmax of scores s; the steps are spread over the
  // value MFMAs of the previous block.
  __device__ __forceinline__ void soft_step(int k, f32x16 &s, Soft &st, bool mask, int lim) {
    const float c = a.scale_log2;
    if (k == 0) {
      if (mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (4 * (i & 3) + 2 * (i >> 3) + ((i >> 2) & 1) >= lim) s[i] = -INFINITY;
      }
      st.mx = vmax3(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], s[5]), vmax(s[6], s[7]));
    } else if (k == 1) {
      st.mx = vmax3(vmax3(st.mx, s[8], s[9]), vmax3(s[10], s[11], s[12]), vmax3(s[13], s[14], s[15]));
    } else if (k == 2) {
      const float m_new = vmax(m_run, vmax_xor32(st.mx) * c);
      const bool up = m_new > m_run + SOLO_SLACK;
      const float e = __builtin_amdgcn_exp2f(m_run - m_new);       // 0 on the first block (m_run = -FLT_MAX)
      st.alpha = up ? e : 1.0f;
      m_run = up ? m_new : m_run;
      l_run *= st.alpha;
      e_run *= st.alpha;
      st.pe = 0.f;
      // Each step's results are pinned where the step stands: the compiler
      // would otherwise sink the softmax past the rescale branch, out from
      // under the score MFMAs it is spread over.
      asm volatile("" : "+v"(m_run), "+v"(st.alpha), "+v"(l_run), "+v"(e_run));
    } else if (k < 11) {
      // two registers per step: 2 (k - 3), 2 (k - 3) + 1
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * (k - 3) + h;
        const float f = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_run));
        st.pe += f;
        st.p[i >> 3][i & 7] = to_bf16(f);
      }
      asm volatile("" : "+v"(st.pe), "+v"(st.p[(2 * (k - 3)) >> 3]));
    } else if (k < 13) {
      // sum of the rounded weights (bf16 pairs dotted with (1, 1))
      const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      const bf16x8 q = st.p[k - 11];
      float ps = l_run;
#pragma unroll
      for (int i = 0; i < 4; ++i) ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{q[2 * i], q[2 * i + 1]}, one2, ps, false);
      l_run = ps;
      if (k == 12) e_run += st.pe;
      asm volatile("" : "+v"(l_run), "+v"(e_run));
    }
  }
  // Scores of tokens at or past `lim` (mask_limit) set to -inf: the block
  // before the last one, for multi-token rows (a no-op otherwise).
  __device__ __forceinline__ void mask_scores(f32x16 &s, int lim) const {
    if (a.q_len <= 1) return;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (4 * (i & 3) + 2 * (i >> 3) + ((i >> 2) & 1) >= lim) s[i] = -INFINITY;
  }
  __device__ __forceinline__ void softmax_all(f32x16 &s, Soft &st, bool mask, int lim) {
#pragma unroll
    for (int k = 0; k < 13; ++k) soft_step(k, s, st, mask, lim);
  }
  // Rescale the value accumulators if any head of the wave moved its max.
  __device__ __forceinline__ void rescale(float alpha) {
    if (__ballot(alpha != 1.0f)) {
      // In place on the accumulator registers, one at a time (a vector
      // multiply of o would copy all 256 of them out of the AGPR file),
      // after the wait states of the value MFMAs that wrote them last.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          float t;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\t"
                       "v_accvgpr_write_b32 %0, %1"
                       : "+a"(o[j][k]), "=&v"(t) : "v"(alpha));
        }
      asm volatile("s_nop 7" ::: "memory");
    }
  }

  // One step of the pipeline, on blocks i (in `slot_v`, scores in s) and
  // i + 1 (in `slot_s`): the 36 score MFMAs of block i + 1 with the softmax of
  // block i spread over them (its steps between every second MFMA), the
  // rescale of the value accumulators for block i, then the 32 value MFMAs of
  // block i with the nine copies of `cp` (when COPY) spread over them.  s holds
  // block i + 1's scores on return.  first: block i is block 0 (the
  // accumulators are still zero).  Block i is never the last block of the
  // chunk; multi-token rows that do not see some of its tokens have them
  // masked beforehand (mask_scores).  Operands are read in order and used in
  // swapped pairs (MFMA slot 2m takes read 2m + 1, slot 2m + 1 read 2m), so a
  // single LDS wait before each pair covers both of its reads.
  // COPY: 0 no copies, 1 the clamped copies of `cp`, 2 the full-block
  // copies of `fc`.
  // PAR < 0: the new scores replace s (a copy out of the chain's registers);
  // PAR 0 / 1: they go to *s_out, left in the chain's registers (mfma_sp).
  template <int COPY, int PAR = -1>
  __device__ __forceinline__ void phase(const uint8_t *slot_s, const uint8_t *slot_v, f32x16 &s, bool first,
                                        const Copy &cp, const FullCopy &fc, f32x16 *s_out = nullptr) {
    const int l = lane_id();
    const int kb = kb_, krb = krb_;
    constexpr int RK = 4, RV = 4, NV = 2 * NT;
    bf16x8 kr[KS], vf[NV];
    f32x16 sn;
    Soft st;
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) kr[ks] = kread(slot_s, kb, krb, ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + RK < KS) kr[ks + RK] = kread(slot_s, kb, krb, ks + RK);
      if (PAR < 0) mfma_s(sn, kr[ks ^ 1], qf[ks ^ 1], ks == 0, ks == KS - 1);
      else mfma_sp<PAR>(sn, kr[ks ^ 1], qf[ks ^ 1], ks == 0);
      if ((ks & 1) == 0 && ks / 2 < 13) soft_step(ks / 2, s, st, false, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    rescale(first ? 1.0f : st.alpha);
    const int vb = vb_;
    uint32_t voff = 0, roff = 0;
    if (COPY == 1) {
      voff = static_cast<uint32_t>(opaque(l) << 4);
      roff = rope_voff(cp, l);
    }
    if (COPY == 2) {
      voff = voff_;
      roff = roff_full_;
      copy_full_m0(fc);
    }
#pragma unroll
    for (int n = 0; n < RV; ++n) vf[n] = vread(slot_v, vb, n);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + RV < NV) vf[n + RV] = vread(slot_v, vb, n + RV);
      mfma_o(o[(n ^ 1) & 15], vf[n ^ 1], st.p[(n ^ 1) >> 4], n == 0, false);
      if (COPY && n % 3 == 1 && n / 3 < NI) {                               // copies k = 0..8 at n = 3 k + 1
        if (COPY == 1) copy(cp, n / 3, voff, roff);
        else copy_full(fc, n / 3, voff, roff);
      }
    }
    if (PAR < 0) s = sn;
    else *s_out = sn;
  }

  // ---- fp8 cache.  A packed row is [512 E4M3 codes | 64 bf16 rotary values
  // | 4 fp32 group scales] (656 bytes) and the 32 rows of a block are
  // contiguous in the page.  Wave w copies rows 8 w .. 8 w + 7 of a block
  // unchanged into a staging buffer (5248 contiguous bytes, six wave-wide
  // copies) and later expands exactly those rows into the bf16 slot layout,
  // so copy and expansion need no workgroup barrier between them.
  static constexpr int ROWS8 = TB / NW;                            // rows per wave
  static constexpr int CH8 = ROWS8 * FP8_ROW_BYTES / 16;           // 328 16-byte pieces
  static constexpr int NI8 = (CH8 + 63) / 64;                      // 6 copies per wave per block
  static constexpr int TAIL8 = CH8 - (NI8 - 1) * 64;               // lanes of the last copy
  static_assert(ROWS8 * FP8_ROW_BYTES % 16 == 0 && 3 * NI8 <= 63, "fp8 copy ranges");
  __device__ __forceinline__ void copy8(int blk, int phys, uint8_t *stage, int k) const {
    const uint8_t *src = a.cache + (static_cast<size_t>(phys) * PAGE + ((t_begin + blk * TB) & 32) + wave * ROWS8) *
                                       FP8_ROW_BYTES;
    const int ln = lane_id();
    if (k + 1 < NI8 || ln < TAIL8)
      dma16_s(static_cast<uint32_t>((k * 64 + ln) * 16), src,
              __builtin_amdgcn_readfirstlane(lds_addr(stage + wave * ROWS8 * FP8_ROW_BYTES) + k * 1024));
  }
  __device__ __forceinline__ void issue8(int blk, int phys, uint8_t *stage) const {
#pragma unroll
    for (int k = 0; k < NI8; ++k) copy8(blk, phys, stage, k);
  }
  // Expand row k (0..7) of this wave's share of block blk from `stage` into
  // `slot`: latent value j = code_j * scale[j / 128], formed in fp32 (the
  // E4M3 code converts exactly) and rounded to bf16; lane l writes 16-byte
  // chunk l of the padded latent row.  Rows past the end of the chunk become
  // zeros (their scores are masked; zeros keep their products finite).
  __device__ __forceinline__ void expand8_row(int blk, const uint8_t *stage, uint8_t *slot, int k) const {
    const int l = lane_id();
    const int r = wave * ROWS8 + k;
    u32x4 out = u32x4{0, 0, 0, 0};
    if (t_begin + blk * TB + r < t_end) {
      const uint8_t *src = stage + r * FP8_ROW_BYTES;
      const u32x2 codes = *reinterpret_cast<const u32x2 *>(src + l * 8);
      const float sc = *reinterpret_cast<const float *>(src + FP8_SCALE_OFF + (l >> 4) * 4);
      bf16x8 v;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[h]), false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[h]), true);
        v[4 * h + 0] = to_bf16(lo[0] * sc);
        v[4 * h + 1] = to_bf16(lo[1] * sc);
        v[4 * h + 2] = to_bf16(hi[0] * sc);
        v[4 * h + 3] = to_bf16(hi[1] * sc);
      }
      out = __builtin_bit_cast(u32x4, v);
    }
    *reinterpret_cast<u32x4 *>(slot + r * S_LROW + l * 16) = out;
  }
  // The rotary parts of this wave's 8 rows: lane l copies chunk l % 8 of row
  // 8 w + l / 8 (stored at chunk (l % 8) ^ fr(row) of the rotary region).
  __device__ __forceinline__ void expand8_rope(int blk, const uint8_t *stage, uint8_t *slot) const {
    const int l = lane_id();
    const int r = wave * ROWS8 + (l >> 3), c = l & 7;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (t_begin + blk * TB + r < t_end) v = *reinterpret_cast<const u32x4 *>(stage + r * FP8_ROW_BYTES + DC + c * 16);
    *reinterpret_cast<u32x4 *>(slot + S_LAT + r * ROPE_BYTES + ((c ^ fr(r)) << 4)) = v;
  }
  __device__ __forceinline__ void expand8(int blk, const uint8_t *stage, uint8_t *slot) const {
#pragma unroll
    for (int k = 0; k < ROWS8; ++k) expand8_row(blk, stage, slot, k);
    expand8_rope(blk, stage, slot);
  }

  // fp8 pipeline step on blocks i (values, `slot_v`) and i + 1 (scores,
  // `slot_s`): part A as in phase(), with the copies of block i + 3 into
  // `stage_n` (COPY) spread over its first MFMAs; part B: the value MFMAs of
  // block i with [wait for this wave's copies of block i + 2] [expansion of
  // block i + 2 from `stage_e` into `slot_e`, a row every four MFMAs]
  // (EXPAND) spread over them.
  template <bool COPY, bool EXPAND>
  __device__ __forceinline__ void phase8(const uint8_t *slot_s, const uint8_t *slot_v, f32x16 &s, bool first,
                                         int blk_n, int phys_n, uint8_t *stage_n, int blk_e, const uint8_t *stage_e,
                                         uint8_t *slot_e) {
    const int l = lane_id();
    const int kb = k_base(l), krb = kr_base(l);
    constexpr int RK = 4, RV = 4, NV = 2 * NT;
    bf16x8 kr[KS], vf[NV];
    f32x16 sn;
    Soft st;
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) kr[ks] = kread(slot_s, kb, krb, ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + RK < KS) kr[ks + RK] = kread(slot_s, kb, krb, ks + RK);
      mfma_s(sn, kr[ks ^ 1], qf[ks ^ 1], ks == 0, ks == KS - 1);
      if ((ks & 1) == 0 && ks / 2 < 13) soft_step(ks / 2, s, st, false, 0);
      if (COPY && (ks & 1) == 1 && ks / 2 < NI8) copy8(blk_n, phys_n, stage_n, ks / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    rescale(first ? 1.0f : st.alpha);
    const int vb = v_base(l);
#pragma unroll
    for (int n = 0; n < RV; ++n) vf[n] = vread(slot_v, vb, n);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + RV < NV) vf[n + RV] = vread(slot_v, vb, n + RV);
      mfma_o(o[(n ^ 1) & 15], vf[n ^ 1], st.p[(n ^ 1) >> 4], n == 0, false);
      if (EXPAND) {
        if (n == 0) {
          if (COPY) wait_vmcnt<NI8>();
          else wait_vmcnt<0>();
        }
        if ((n & 3) == 1) expand8_row(blk_e, stage_e, slot_e, n >> 2);
        if (n == NV - 1) expand8_rope(blk_e, stage_e, slot_e);
      }
    }
    s = sn;
  }

  // Scores of the first block (no value product yet).
  __device__ __forceinline__ f32x16 scores(const uint8_t *slot) const {
    const int l = lane_id();
    const int kb = k_base(l), krb = kr_base(l);
    constexpr int RK = 4;
    bf16x8 kr[KS];
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) kr[ks] = kread(slot, kb, krb, ks);
    f32x16 s;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + RK < KS) kr[ks + RK] = kread(slot, kb, krb, ks + RK);
      mfma_s(s, kr[ks], qf[ks], ks == 0, ks == KS - 1);
    }
    return s;
  }

  // Value product of the last block alone.
  __device__ __forceinline__ void values(const uint8_t *slot, const bf16x8 (&pv)[2]) {
    const int l = lane_id();
    const int vb = v_base(l);
    constexpr int RV = 4, NV = 2 * NT;
    bf16x8 vf[NV];
#pragma unroll
    for (int n = 0; n < RV; ++n) vf[n] = vread(slot, vb, n);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + RV < NV) vf[n + RV] = vread(slot, vb, n + RV);
      mfma_o(o[n & 15], vf[n], pv[n >> 4], n == 0, n == NV - 1);
    }
  }

  // Normalise and store: lse by the lanes of the first half; the tile goes
  // through LDS (row = head of the workgroup, 16-byte chunk c at position
  // c ^ (row & 15)) so that each global store writes one whole 1 KB row.
  // Each wave reads back only the rows it wrote.  The rows are written once
  // and read once, by the combine: non-temporal stores (streaming cache
  // policy) shorten the kernel's end by about 1.6 us at 32 x 128 heads x 8
  // chunks (33.6 MB of partials).
  __device__ __forceinline__ void finish(uint8_t *stage) {
    const int l = threadIdx.x & 63;
    const float l_tot = sum_xor32(l_run);
    const float e_tot = sum_xor32(e_run);
    // l_tot >= 1 unless the row saw no token of the chunk (a multi-token row
    // past its position): then o = 0 and lse = log 0 = -inf
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = (m_run + __log2f(e_tot)) * LN2;
    const int head = head_of(l);
    if (l < 32 && head < a.H) {
      if (a.direct) {
        if (a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = lse_v;
      } else {
        a.lse_part[(static_cast<size_t>(b) * a.n_splits + split) * a.H + head] = lse_v;
      }
    }
    barrier_lds();            // every wave is done with the slots
    const int row = wave * 32 + (l & 31);
    uint8_t *srow = stage + row * LAT_BYTES + (l >> 5) * 8;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[j][4 * q + e] * inv);
        const int c = j * 4 + q;                            // 16-byte chunk of the row
        *reinterpret_cast<bf16x4 *>(srow + ((c ^ (row & 15)) << 4)) = v;
      }
    }
    asm volatile("" ::: "memory");   // a wave's LDS accesses complete in order
#pragma unroll 4
    for (int k = 0; k < 32; ++k) {
      const int r = wave * 32 + k;
      const int h = grp * HEADS + r;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * LAT_BYTES + ((l ^ (r & 15)) << 4));
      if (h < a.H) {
        uint16_t *dst = a.direct ? a.o_latent + (static_cast<size_t>(b) * a.H + h) * DC
                                 : a.o_part + ((static_cast<size_t>(b) * a.n_splits + split) * a.H + h) * DC;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + l * 8));
      }
    }
  }
};

// Wait until this wave's copies of block i have landed (copies of the next
// `ahead` blocks may still be in flight).
template <int NI, int AHEAD>
__device__ __forceinline__ void wait_block(bool full_share) {
  if (full_share) wait_vmcnt<AHEAD * NI>();
  else wait_vmcnt<AHEAD * (NI - 1)>();
}

#define MLA_WAIT_BLOCK(i)                                              \
  if ((i) + 2 < nblk) wait_block<D::NI, 2>(full_share);                \
  else if ((i) + 1 < nblk) wait_block<D::NI, 1>(full_share);           \
  else wait_vmcnt<0>();

// Group X, block i in slot CUR (block i + 3 goes into NXT, the slot of block
// i - 1): [wait copies of i] Ba [scores + softmax i] Bb [copy i + 3]
// [values i].
#define MLA_STEP_X(K, CUR, NXT)                                        \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    const int phys = i + 3 < nblk ? dec.page_of(i + 3) : 0;            \
    MLA_WAIT_BLOCK(i)                                                  \
    barrier_no_fence();                                                \
    dec.scores_softmax(CUR, i);                                        \
    barrier_lds();                                                     \
    if (i + 3 < nblk) dec.issue(i + 3, phys, NXT);                     \
    dec.values(CUR);                                                   \
  }

// Group Y, block i >= 1 in slot CUR (block i - 1 in PRV, which is also the
// slot block i + 3 is copied into): [wait copies of i] Ba [values i - 1] Bb
// [copy i + 3 into PRV] [scores + softmax i].  Ba publishes Y's P of i - 1.
#define MLA_STEP_Y(K, CUR, PRV)                                        \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    const int phys = i + 3 < nblk ? dec.page_of(i + 3) : 0;            \
    MLA_WAIT_BLOCK(i)                                                  \
    barrier_lds();                                                     \
    dec.values(PRV);                                                   \
    barrier_no_fence();                                                \
    if (i + 3 < nblk) dec.issue(i + 3, phys, PRV);                     \
    dec.scores_softmax(CUR, i);                                        \
  }

template <class D, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(D::NW * 64, D::NW * 64),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[NSLOT * SLOT_BYTES];
  uint8_t *const slot0 = ring, *const slot1 = ring + SLOT_BYTES, *const slot2 = ring + 2 * SLOT_BYTES,
                 *const slot3 = ring + 3 * SLOT_BYTES;
  static_assert(D::HEADS * LAT_BYTES <= NSLOT * SLOT_BYTES, "the output tile is staged in the slot ring");
  __shared__ __attribute__((aligned(16))) uint8_t px[D::NW / 2 * PX_BYTES];
  __shared__ __attribute__((aligned(16))) float ax[D::NW / 2 * 32];
  __shared__ __attribute__((aligned(16))) float fx[D::NW / 2 * 32];
  constexpr int NW = D::NW;

  // Chunk placement: workgroups are dealt to the 8 XCDs round-robin by id, so
  // id -> (XCD id % 8, position id / 8) is remapped to consecutive chunk
  // indices per XCD; the chunks of a sequence then share one L2.
  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int b = item / a.n_splits;
  const int split = item - b * a.n_splits;
  const int S = a.seq_lens[b];
  const int t_begin = split * a.split_tokens;
  const int t_end = min(S, t_begin + a.split_tokens);

  if (t_begin >= t_end) {
    // Nothing to attend.  A whole-sequence launch still owes its outputs
    // (empty sequence: zeros and lse = -inf); split chunks past the end of a
    // sequence are skipped by the combine kernel.
    if (a.direct) {
      const int t = threadIdx.x;
      const int head = blockIdx.y * D::HEADS + t / 4;       // 4 threads per head
      if (head < a.H) {
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % 4) * (DC / 4);
        for (int c = 0; c < DC / 4; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % 4 == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  // Page ids are read with scalar loads (the streaming loop's only vector
  // memory operations are its DMA copies, so vmcnt counts exactly those).
  D dec(a, px, ax, fx, b, split, S, t_begin, t_end);
  dec.begin();
  const int nblk = (t_end - t_begin + TB - 1) / TB;
  // Block 0's copies go out before the query loads so the two latencies
  // overlap; both are waited for here (the compiler, which does not see the
  // copies, would otherwise wait for everything at the first use of the
  // query), and blocks 1 and 2 follow, to land while block 0 is computed.
  dec.issue(0, dec.page_of(0), slot0);
  dec.load_q();
  wait_vmcnt<0>();
  if (nblk > 1) dec.issue(1, dec.page_of(1), slot1);
  if (nblk > 2) dec.issue(2, dec.page_of(2), slot2);
  const bool full_share = dec.copies() == D::NI;

  // Slot of block i: i % 4.  The slot of block i - 1 is rewritten (block
  // i + 3) only after the second barrier of block i, when both groups are
  // done with block i - 1.
  const bool group_y = NW == 8 && (threadIdx.x >> 8) != 0;
  if (!group_y) {
    for (int blk = 0; blk < nblk; blk += 4) {
      MLA_STEP_X(0, slot0, slot3)
      MLA_STEP_X(1, slot1, slot0)
      MLA_STEP_X(2, slot2, slot1)
      MLA_STEP_X(3, slot3, slot2)
    }
    barrier_no_fence();       // Y publishes its P of the last block
  } else {
    // block 0: nothing of Y's to finish yet
    {
      const int phys = nblk > 3 ? dec.page_of(3) : 0;
      barrier_lds();
      barrier_no_fence();
      if (nblk > 3) dec.issue(3, phys, slot3);
      dec.scores_softmax(slot0, 0);
    }
    for (int blk = 1; blk < nblk; blk += 4) {
      MLA_STEP_Y(0, slot1, slot0)
      MLA_STEP_Y(1, slot2, slot1)
      MLA_STEP_Y(2, slot3, slot2)
      MLA_STEP_Y(3, slot0, slot3)
    }
    barrier_lds();
    const int last = (nblk - 1) & 3;
    dec.values(last == 0 ? slot0 : (last == 1 ? slot1 : (last == 2 ? slot2 : slot3)));
  }
  dec.finish(ring);
}

#undef MLA_STEP_X
#undef MLA_STEP_Y
#undef MLA_WAIT_BLOCK

// One-wave-per-SIMD decoder.
// Prologue: the query rows go through the slot ring (whole-row copies, then
// the fragments) in two halves while blocks 0 and 1 are copied into the
// other half of the ring; then block 2.
// Iteration i (scores of block i already in s): [wait own copies of i + 1]
// barrier [scores i + 1 with the softmax of i] [rescale] [values i with the
// copies of i + 3 into the slot of i - 1]; the last block is peeled off the
// loop.  The barrier makes block i + 1 visible and certifies that every wave
// is done with block i - 1.  Slot of block i: (i + 2) % 4.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_solo_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[NSLOT * S_SLOT];
  static_assert(DecoderSolo::HEADS * LAT_BYTES <= NSLOT * S_SLOT, "the output tile is staged in the slot ring");
  static_assert(DecoderSolo::HEADS * DROW * 2 <= NSLOT * S_SLOT, "the query is staged in the slot ring");

  // One workgroup per (sequence, chunk, head group), the head groups of a
  // chunk numbered consecutively; workgroups are dealt to the 8 XCDs
  // round-robin by id, so id -> (XCD id % 8, position id / 8) is remapped to
  // consecutive indices per XCD: the chunks of a sequence, and the head
  // groups that read the same chunk, share one L2.
  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int groups = (a.H + DecoderSolo::HEADS - 1) / DecoderSolo::HEADS;
  const int grp = item % groups;
  item /= groups;
  const int b = item / a.n_splits;
  const int split = item - b * a.n_splits;
  const int S = a.seq_lens[b];
  const int t_begin = split * a.split_tokens;
  const int t_end = min(S, t_begin + a.split_tokens);

  if (t_begin >= t_end) {
    if (a.direct) {
      const int t = threadIdx.x;
      const int head = grp * DecoderSolo::HEADS + t / 2;      // 2 threads per head
      if (head < a.H) {
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % 2) * (DC / 2);
        for (int c = 0; c < DC / 2; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % 2 == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  constexpr int NI = DecoderSolo::NI;
  DecoderSolo dec(a, b, split, grp, S, t_begin, t_end);
  dec.begin();
  const int nblk = (t_end - t_begin + TB - 1) / TB;
  const bool ragged = (t_end - t_begin) % TB != 0 || a.q_len > 1;
  // Slot of block i: (i + 2) % 4, so that blocks 0 and 1 land in slots 2
  // and 3 while the query rows are staged in the first 73,728 bytes (slots
  // 0 and 1), in two halves: waves 0 and 1, then waves 2 and 3.
  auto slot = [&](int i) { return ring + ((i + 2) & (NSLOT - 1)) * S_SLOT; };
  const bool first_half = dec.wave < 2;
  if (first_half) dec.load_q_lds(ring, 0);
  dec.issue(0, dec.page_of(0), slot(0));
  if (nblk > 1) dec.issue(1, dec.page_of(1), slot(1));
  if (first_half) {
    if (nblk > 1) wait_vmcnt<2 * NI>();       // the query rows (copied before blocks 0, 1)
    else wait_vmcnt<NI>();
    dec.read_q_lds(ring, 0);
  }
  barrier_lds();              // waves 0 and 1 are done with the staging area
  if (!first_half) {
    dec.load_q_lds(ring, 2 * 32);
    wait_vmcnt<0>();          // the query rows, and blocks 0 and 1 (copied before them)
    dec.read_q_lds(ring, 2 * 32);
  }
  barrier_lds();              // the staging area (slots 0 and 1) is free
  if (nblk > 2) dec.issue(2, dec.page_of(2), slot(2));
  if (nblk > 2) wait_vmcnt<NI>();             // blocks 0 and 1
  else wait_vmcnt<0>();
  barrier_no_fence();         // blocks 0 and 1 visible
  f32x16 s = dec.scores(slot(0));
  int i = 0;
  // Only the chunk's last block can have rows past its end: the copies of
  // every other block take the full-block form.
  dec.init_full_copy();
  // two blocks per iteration, the scores alternating between the chain's two
  // register ranges (s: v[32:47], s1: v[16:31])
  f32x16 s1;
  for (; i + 5 < nblk; i += 2) {
    {
      const int phys = dec.page_of(i + 3);
      wait_vmcnt<NI>();
      barrier_no_fence();
      dec.phase<2, 0>(slot(i + 1), slot(i), s, i == 0, DecoderSolo::Copy{},
                      dec.full_copy_of(i + 3, phys, slot(i + 3)), &s1);
    }
    {
      const int phys = dec.page_of(i + 4);
      wait_vmcnt<NI>();
      barrier_no_fence();
      dec.phase<2, 1>(slot(i + 2), slot(i + 1), s1, false, DecoderSolo::Copy{},
                      dec.full_copy_of(i + 4, phys, slot(i + 4)), &s);
    }
  }
  for (; i + 4 < nblk; ++i) {
    const int phys = dec.page_of(i + 3);
    wait_vmcnt<NI>();
    barrier_no_fence();
    dec.phase<2>(slot(i + 1), slot(i), s, i == 0, DecoderSolo::Copy{}, dec.full_copy_of(i + 3, phys, slot(i + 3)));
  }
  if (i + 3 < nblk) {
    const int phys = dec.page_of(i + 3);
    wait_vmcnt<NI>();
    barrier_no_fence();
    dec.phase<1>(slot(i + 1), slot(i), s, i == 0, dec.copy_of(i + 3, phys, slot(i + 3)), DecoderSolo::FullCopy{});
    ++i;
  }
  for (; i + 1 < nblk; ++i) {
    if (i + 2 < nblk) wait_vmcnt<NI>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    dec.mask_scores(s, dec.mask_limit(DecoderSolo::lane_id(), i));
    dec.phase<0>(slot(i + 1), slot(i), s, i == 0, DecoderSolo::Copy{}, DecoderSolo::FullCopy{});
  }
  {
    DecoderSolo::Soft st;
    dec.softmax_all(s, st, ragged, dec.mask_limit(DecoderSolo::lane_id(), nblk - 1));
    dec.rescale(nblk == 1 ? 1.0f : st.alpha);
    dec.values(slot(nblk - 1), st.p);
  }
  dec.fence_o();
  dec.finish(ring);
}

// fp8 cache, one wave per SIMD.  Three bf16 slots (block i in slot i % 3)
// and two staging buffers of packed rows (block i in stage i % 2).
// Iteration i: barrier (block i + 1's expansion visible; every wave done with
// block i - 1, whose slot receives block i + 2) [scores i + 1 with the
// softmax of i and the copies of block i + 3 into the stage of block i + 1
// (expanded by this same wave one step earlier)] [rescale] [values i with:
// wait for this wave's copies of block i + 2, expansion of block i + 2].
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_solo_fp8_kernel(DecodeArgs a) {
  constexpr int RING = 3 * S_SLOT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RING + 2 * STAGE_BYTES];
  static_assert(DecoderSolo::HEADS * LAT_BYTES <= RING + 2 * STAGE_BYTES, "the output tile is staged in LDS");
  uint8_t *const stage0 = lds + RING;

  // One workgroup per (sequence, chunk, head group), the head groups of a
  // chunk numbered consecutively; workgroups are dealt to the 8 XCDs
  // round-robin by id, so id -> (XCD id % 8, position id / 8) is remapped to
  // consecutive indices per XCD: the chunks of a sequence, and the head
  // groups that read the same chunk, share one L2.
  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int groups = (a.H + DecoderSolo::HEADS - 1) / DecoderSolo::HEADS;
  const int grp = item % groups;
  item /= groups;
  const int b = item / a.n_splits;
  const int split = item - b * a.n_splits;
  const int S = a.seq_lens[b];
  const int t_begin = split * a.split_tokens;
  const int t_end = min(S, t_begin + a.split_tokens);

  if (t_begin >= t_end) {
    if (a.direct) {
      const int t = threadIdx.x;
      const int head = grp * DecoderSolo::HEADS + t / 2;      // 2 threads per head
      if (head < a.H) {
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % 2) * (DC / 2);
        for (int c = 0; c < DC / 2; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % 2 == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  DecoderSolo dec(a, b, split, grp, S, t_begin, t_end);
  dec.begin();
  const int nblk = (t_end - t_begin + TB - 1) / TB;
  const bool ragged = (t_end - t_begin) % TB != 0 || a.q_len > 1;
  auto slot = [&](int i) { return lds + (i % 3) * S_SLOT; };
  auto stage = [&](int i) { return stage0 + (i & 1) * STAGE_BYTES; };
  constexpr int NI8 = DecoderSolo::NI8;
  static_assert(2 * 32 * DROW * 2 <= 2 * S_SLOT, "half of the query rows fit the first two slots");
  // Blocks 0 and 1 go to their stages while the query rows are staged in the
  // first 73,728 bytes (slots 0 and 1) in two halves, as in the bf16 kernel;
  // then block 0 is expanded, block 2 requested into its stage and block 1
  // expanded.
  dec.issue8(0, dec.page_of(0), stage(0));
  if (nblk > 1) dec.issue8(1, dec.page_of(1), stage(1));
  if (dec.wave < 2) {
    dec.load_q_lds(lds, 0);
    wait_vmcnt<0>();          // the query rows, and blocks 0 and 1 (copied before them)
    dec.read_q_lds(lds, 0);
  }
  barrier_lds();              // waves 0 and 1 are done with the staging area
  if (dec.wave >= 2) {
    dec.load_q_lds(lds, 2 * 32);
    wait_vmcnt<0>();
    dec.read_q_lds(lds, 2 * 32);
  }
  barrier_lds();              // the staging area (slots 0 and 1) is free
  dec.expand8(0, stage(0), slot(0));
  if (nblk > 1) {
    if (nblk > 2) {
      dec.issue8(2, dec.page_of(2), stage(0));
      wait_vmcnt<NI8>();
    } else {
      wait_vmcnt<0>();
    }
    dec.expand8(1, stage(1), slot(1));
  }
  barrier_lds();              // blocks 0 and 1 visible
  f32x16 s = dec.scores(slot(0));
  int i = 0;
  for (; i + 3 < nblk; ++i) {
    const int phys = dec.page_of(i + 3);
    barrier_lds();
    dec.phase8<true, true>(slot(i + 1), slot(i), s, i == 0, i + 3, phys, stage(i + 3), i + 2, stage(i + 2),
                           slot(i + 2));
  }
  if (i + 2 < nblk) {
    barrier_lds();
    dec.mask_scores(s, dec.mask_limit(DecoderSolo::lane_id(), i));
    dec.phase8<false, true>(slot(i + 1), slot(i), s, i == 0, 0, 0, nullptr, i + 2, stage(i + 2), slot(i + 2));
    ++i;
  }
  if (i + 1 < nblk) {
    barrier_lds();
    dec.mask_scores(s, dec.mask_limit(DecoderSolo::lane_id(), i));
    dec.phase8<false, false>(slot(i + 1), slot(i), s, i == 0, 0, 0, nullptr, 0, nullptr, nullptr);
    ++i;
  }
  {
    DecoderSolo::Soft st;
    dec.softmax_all(s, st, ragged, dec.mask_limit(DecoderSolo::lane_id(), nblk - 1));
    dec.rescale(nblk == 1 ? 1.0f : st.alpha);
    dec.values(slot(nblk - 1), st.p);
  }
  dec.fence_o();
  dec.finish(lds);
}

// fp8 cache.  Packed rows are copied into a staging buffer one step ahead
// and expanded to bf16 into a ring of three slots one block before use; the
// score, softmax and value phases are those of the bf16 kernel.
//
// Group X, block i in slot CUR (block i + 1 goes into NXT, the slot of block
// i - 2): Ba [scores + softmax i] Bb [copy i + 2 into staging i % 2]
// [values i] [wait copy i + 1, expand i + 1].  Ba also publishes X's
// expansion of block i.
#define MLA_STEP_X8(K, CUR, NXT)                                       \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    const int phys = i + 2 < nblk ? dec.page_of(i + 2) : 0;            \
    barrier_lds();                                                     \
    dec.scores_softmax(CUR, i);                                        \
    barrier_lds();                                                     \
    if (i + 2 < nblk) dec.issue8(i + 2, phys, stage + (i & 1) * STAGE_BYTES); \
    dec.values(CUR);                                                   \
    if (i + 1 < nblk) {                                                \
      if (i + 2 < nblk) wait_vmcnt<D::NI8>();                          \
      else wait_vmcnt<0>();                                            \
      dec.convert8(i + 1, stage + ((i + 1) & 1) * STAGE_BYTES, NXT);   \
    }                                                                  \
  }

// Group Y, block i >= 1 in slot CUR, block i - 1 in PRV: Ba [values i - 1]
// Bb [scores + softmax i].
#define MLA_STEP_Y8(K, CUR, PRV)                                       \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    barrier_lds();                                                     \
    dec.values(PRV);                                                   \
    barrier_no_fence();                                                \
    dec.scores_softmax(CUR, i);                                        \
  }

template <class D, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(D::NW * 64, D::NW * 64),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void decode_fp8_kernel(DecodeArgs a) {
  constexpr int RING = 3 * SLOT_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RING + 2 * STAGE_BYTES];
  uint8_t *const slot0 = lds, *const slot1 = lds + SLOT_BYTES, *const slot2 = lds + 2 * SLOT_BYTES;
  uint8_t *const stage = lds + RING;
  static_assert(D::HEADS * LAT_BYTES <= RING + 2 * STAGE_BYTES, "the output tile is staged in LDS");
  __shared__ __attribute__((aligned(16))) uint8_t px[D::NW / 2 * PX_BYTES];
  __shared__ __attribute__((aligned(16))) float ax[D::NW / 2 * 32];
  __shared__ __attribute__((aligned(16))) float fx[D::NW / 2 * 32];
  constexpr int NW = D::NW;

  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int b = item / a.n_splits;
  const int split = item - b * a.n_splits;
  const int S = a.seq_lens[b];
  const int t_begin = split * a.split_tokens;
  const int t_end = min(S, t_begin + a.split_tokens);

  if (t_begin >= t_end) {
    if (a.direct) {
      const int t = threadIdx.x;
      const int head = blockIdx.y * D::HEADS + t / 4;
      if (head < a.H) {
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % 4) * (DC / 4);
        for (int c = 0; c < DC / 4; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % 4 == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  D dec(a, px, ax, fx, b, split, S, t_begin, t_end);
  dec.begin();
  const int nblk = (t_end - t_begin + TB - 1) / TB;
  dec.issue8(0, dec.page_of(0), stage);
  dec.load_q();
  wait_vmcnt<0>();
  if (nblk > 1) dec.issue8(1, dec.page_of(1), stage + STAGE_BYTES);
  dec.convert8(0, stage, slot0);

  // Slot of block i: i % 3.  Block i + 1 is expanded into the slot of block
  // i - 2 after the second barrier of block i, when both groups are done
  // with block i - 2.
  const bool group_y = NW == 8 && (threadIdx.x >> 8) != 0;
  if (!group_y) {
    for (int blk = 0; blk < nblk; blk += 3) {
      MLA_STEP_X8(0, slot0, slot1)
      MLA_STEP_X8(1, slot1, slot2)
      MLA_STEP_X8(2, slot2, slot0)
    }
    barrier_no_fence();       // Y publishes its P of the last block
  } else {
    barrier_lds();
    barrier_no_fence();
    dec.scores_softmax(slot0, 0);
    for (int blk = 1; blk < nblk; blk += 3) {
      MLA_STEP_Y8(0, slot1, slot0)
      MLA_STEP_Y8(1, slot2, slot1)
      MLA_STEP_Y8(2, slot0, slot2)
    }
    barrier_lds();
    const int last = (nblk - 1) % 3;
    dec.values(last == 0 ? slot0 : (last == 1 ? slot1 : slot2));
  }
  dec.finish(lds);
}

#undef MLA_STEP_X8
#undef MLA_STEP_Y8

// Merge split-KV partials: o = sum_c w_c o_c / sum_c w_c, w_c = exp(lse_c - L),
// L = max_c lse_c (the softmax regrouped over the chunks).  One workgroup
// per (sequence, head) with one wave per range of combine_range(n_splits)
// chunks: lanes hold 8 columns each, every wave requests its range's partial
// rows 16 at a time before the maximum lse is known (fp32 sums in chunk
// order), and wave 0 adds the range sums in order.  A long sequence's rows
// are thus read by up to 8 waves at once.
// A multi-token row merges the chunks that hold tokens it sees.
__global__ __launch_bounds__(512) void combine_kernel(DecodeArgs a) {
  __shared__ float red[7][9][64];            // range sums of waves 1..7: 8 columns and z per lane
  const int b = blockIdx.x, head = blockIdx.y;
  const int t = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  int S = a.seq_lens[b];
  if (a.q_len > 1) S = max(0, S - (a.q_len - 1) + head / a.heads);
  const int nv = (S + a.split_tokens - 1) / a.split_tokens;
  uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + t * 8;
  if (nv <= 0) {
    if (wave == 0) {
      *reinterpret_cast<u32x4 *>(dst) = u32x4{0, 0, 0, 0};
      if (t == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
    }
    return;
  }
  const size_t stride = static_cast<size_t>(a.H);
  const float *lp = a.lse_part + static_cast<size_t>(b) * a.n_splits * stride + head;
  const uint16_t *op = a.o_part + (static_cast<size_t>(b) * a.n_splits * stride + head) * DC + t * 8;
  const int R = combine_range(a.n_splits);
  const int c_begin = wave * R, c_end = min(nv, c_begin + R);
  // The partial rows of this wave's range (16 at a time) are requested
  // before the maximum, which only the weights need: one round trip.
  constexpr int BATCH = 16;
  float L = -INFINITY;
  float acc[8] = {};
  float z = 0.f;
  for (int c0 = c_begin; c0 < c_end; c0 += BATCH) {
    u32x4 v[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k)
      v[k] = c0 + k < c_end ? *reinterpret_cast<const u32x4 *>(op + (c0 + k) * stride * DC) : u32x4{0, 0, 0, 0};
    const float lw = t < BATCH && c0 + t < c_end ? lp[(c0 + t) * stride] : -INFINITY;   // lane k: chunk c0 + k
    if (c0 == c_begin) {
      for (int c = t; c < nv; c += 64) L = fmaxf(L, lp[c * stride]);
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) L = fmaxf(L, __shfl_xor(L, m));
    }
    const float wl = t < BATCH && c0 + t < c_end ? expf(lw - L) : 0.f;
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
      z += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * __uint_as_float(v[k][e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(v[k][e] & 0xFFFF0000u);
      }
    }
  }
  if (W > 1) {
    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave - 1][e][t] = acc[e];
      red[wave - 1][8][t] = z;
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < W && w * R < nv; ++w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += red[w - 1][e][t];
      z += red[w - 1][8][t];
    }
  }
  const float inv = 1.0f / z;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = to_bf16(acc[e] * inv);
  *reinterpret_cast<bf16x8 *>(dst) = out;
  if (t == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = L + logf(z);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int nw = decode_waves(a.H);
  const int hpw = decode_heads_per_wave(a.H);
  const int groups = (a.H + hpw * nw - 1) / (hpw * nw);
  dim3 grid(a.B * a.n_splits, groups);
  // one-wave-per-SIMD kernels: head groups folded into the x dimension
  const dim3 grid_solo(a.B * a.n_splits * groups, 1);
  if (a.kv_fp8 && nw == 8) {
    decode_solo_fp8_kernel<<<grid_solo, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  // H <= 64: two waves per SIMD (DecoderPair with 2 or 4 waves)
  if (a.kv_fp8) {
    if (nw == 2) decode_fp8_kernel<DecoderPair<2>, 1><<<grid, 128, 0, stream>>>(a);
    else decode_fp8_kernel<DecoderPair<4>, 1><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  if (nw == 8) {
    decode_solo_kernel<<<grid_solo, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  if (nw == 2) decode_bf16_kernel<DecoderPair<2>, 1><<<grid, 128, 0, stream>>>(a);
  else decode_bf16_kernel<DecoderPair<4>, 1><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  // one workgroup per (b, head), one wave per range of chunks
  const int R = combine_range(a.n_splits);
  const int waves = (a.n_splits + R - 1) / R;
  combine_kernel<<<dim3(a.B, a.H), 64 * waves, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
