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
// Work split: the waves of a workgroup form pairs; a pair owns 32 heads.
// Both waves of a pair see every token of a block, and each takes half of the
// contraction and half of the output:
//   scores   S^T[tok, head] = K[tok, dims] . Q^T[dims, head]   (v_mfma_f32_32x32x16_bf16)
//            wave h sums the 16-dim k-steps 2 ks + h, ks = 0..17 (latent and rotary)
//   exchange each wave adds its partner's fp32 partial through LDS; both then hold
//            the identical full scores and run the same online softmax (fp32, exp2,
//            lazily rescaled)
//   values   O^T[col, head] += V^T[col, tok] . P^T[tok, head], V = K[:, 0:512];
//            wave h owns columns [256 h, 256 h + 256)
// A 32x32x16 product reads one 1 KB operand tile per 16384 MACs, half of what a
// 16x16x32 product needs, so the pair layout halves the LDS bytes per MFMA for
// the same register footprint (72 query + 128 accumulator VGPRs per wave).
//
// Schedule: with 8 waves, waves w and w + 4 share a SIMD.  Waves 0..3 (group
// X) and 4..7 (group Y) run half a block apart, so one group's score MFMAs
// overlap the other group's softmax (VALU) instead of both groups idling the
// matrix core at the same time.  Two workgroup barriers per block serve both
// groups: for X they are "block ready" and "partials exchanged", for Y the
// other way round.
//
// Data movement: 16-byte global->LDS DMA copies (global_load_lds_dwordx4),
// one 1 KB latent row per wave-wide copy, into a ring of three 36 KB slots.  Chunks are XOR-swizzled per row
// so that the row-wise score reads (ds_read_b128) and the transposed value
// reads (ds_read_b64_tr_b16) spread over the LDS banks; the value operand is
// read transposed straight out of the same tile.
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
constexpr int NDMA = TB + TB * ROPE_BYTES / 1024;        // 36 wave-wide copies per block
constexpr int KS = DROW / 32;                   // 18 k-steps of 16 dims per wave
constexpr int KS_LAT = DC / 32;                 // the first 16 of them are latent
constexpr int CB = DC / 64;                     // 8 column blocks of 32 per wave
constexpr int XCH_BYTES = 32 * 32 * 4;          // one wave's partial score tile
constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_SLACK = 8.0f;           // log2 units a stale max may lag

// LDS slot layout for a block of 32 tokens:
//   [0, 32 KB)      latent rows, 1024 B each; 16-byte chunk c of row r sits at
//                   chunk position c ^ fl(r) (XOR inside aligned 16-chunk groups)
//   [32 KB, 36 KB)  rotary keys, 128 B each; chunk c of row r at c ^ fr(r)
// The LDS serves a 128-bit read to 16 consecutive lanes at a time and a
// transposed 64-bit read to lanes 0..31 and 32..63 (gfx950, measured per
// access pattern with the bank-conflict counter), so:
//   - score reads: lanes 16k..16k+15 read rows 16m..16m+15 at one chunk, so
//     fl must be a bijection on r & 15;
//   - value reads: 4 aligned rows, each at one aligned 4-chunk group, need
//     bits 2..3 of fl distinct over 4 aligned rows.
// fl(r) = 4 (r & 3) + ((r >> 2) & 3) satisfies both.  For the 128-byte rotary
// rows (two per 256-byte bank period) the 16 rows of a read must cover
// (r & 1, position) once each: fr(r) = (r >> 1) & 7.
__device__ __forceinline__ int fl(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int fr(int r) { return (r >> 1) & 7; }

// Maximum / sum across lanes l and l ^ 32 with the gfx950 lane swap (VALU).
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The copy (DMA) side of a decoder: which rows of a block each wave moves.
template <int NW>
struct BlockCopier {
  static constexpr int NI = (NDMA + NW - 1) / NW;       // max DMA copies per wave per block
  static_assert(2 * NI <= 63, "two blocks of copies must fit the vmcnt counter");

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

// One wave of a pair: 32 heads, half of the score contraction, half of the
// output columns.  MFMA 32x32x16 bf16 lane layouts (A/B: row or column l % 32,
// k = 8 (l / 32) + j; C: column l % 32, row 8 (i / 4) + 4 (l / 32) + i % 4).
template <int NW_>
struct DecoderPair {
  static constexpr int NW = NW_;
  static constexpr int HEADS = NW * 16;          // heads per workgroup
  static constexpr int NI = BlockCopier<NW>::NI;

  const DecodeArgs &a;
  const int wave, half;                          // wave-uniform
  const int b, split;
  const int t_begin, t_end;
  const int32_t *bt_row;                         // block-table row of the sequence
  uint8_t *xch;                                  // LDS exchange tiles, one per wave

  bf16x8 qf[KS];
  f32x16 o[CB];
  f32x16 s;                   // this wave's partial, then the full, scores of a block
  // m_run: running max (log2 units); l_run: sum of the bf16-rounded weights
  // that multiply V (normalises o consistently); e_run: the same sum of the
  // unrounded weights (gives an lse free of the bf16 rounding of P).  Each
  // lane holds the sums over its 16 tokens of a block; lanes l and l ^ 32
  // together cover the head.
  float m_run, l_run, e_run;

  __device__ DecoderPair(const DecodeArgs &args, uint8_t *xch_, int b_, int split_, int t0, int t1)
      : a(args), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        half(__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 1)),
        b(b_), split(split_), t_begin(t0), t_end(t1),
        bt_row(args.block_table + static_cast<size_t>(b_) * args.max_blocks), xch(xch_) {}

  // Per-lane quantities are recomputed where they are used rather than held
  // in registers across the streaming loop; the opaque lane id keeps the
  // compiler from hoisting them back out of it.
  __device__ __forceinline__ static int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
  }
  __device__ __forceinline__ int head_of(int l) const { return blockIdx.y * HEADS + (wave >> 1) * 32 + (l & 31); }

  // LDS byte offsets of the first read of each kind.  Every other read is one
  // of these XOR a compile-time constant plus an immediate: the XOR acts on
  // address bits that the base's remaining terms leave zero.
  //   latent score reads, k-step ks < 16: row r = l % 32, latent chunk
  //   2 (2 ks + half) + hb = 16 (ks >> 2) + (4 (ks & 3) + 2 half + hb), at
  //   position (4 (ks & 3) ^ (fl & 12)) + ((2 half + hb) ^ (fl & 3)):
  //   k_base ^ 64 (ks & 3), + 256 (ks >> 2)
  __device__ __forceinline__ int k_base(int l) const {
    const int r = l & 31, hb = l >> 5, f = fl(r);
    return r * LAT_BYTES + (((f & 12) | ((2 * half + hb) ^ (f & 3))) << 4);
  }
  //   rotary score reads, k-steps 16, 17: chunk 4 (ks - 16) + 2 half + hb of
  //   row r, at position (4 (ks - 16) ^ (fr & 4)) + ((2 half + hb) ^ (fr & 3)):
  //   kr_base ^ 64 (ks - 16)
  __device__ __forceinline__ int kr_base(int l) const {
    const int r = l & 31, hb = l >> 5, g = fr(r);
    return SLOT_LAT + r * ROPE_BYTES + (((g & 4) | ((2 * half + hb) ^ (g & 3))) << 4);
  }
  //   value reads (transposed, lane l supplies one address): row
  //   16 t + 8 hi + 4 (l / 32) + (l & 15) / 4, latent chunk of column block
  //   cb = 8 half + j: 4 cb + 2 ((l >> 4) & 1) + (l & 3) / 2, byte 8 (l & 1):
  //   v_base ^ 64 (j & 3), + 256 (j >> 2), + 16 KB t; the hi rows sit 8 rows
  //   further, where fl(row + 8) = fl(row) ^ 2: ^ 32, + 8 KB
  __device__ __forceinline__ int v_base(int l) const {
    const int row0 = 4 * (l >> 5) + ((l & 15) >> 2);
    const int fv = fl(row0);
    const int csub = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    return row0 * LAT_BYTES + half * 512 + (((fv & 12) | (csub ^ (fv & 3))) << 4) + 8 * (l & 1);
  }
  //   exchange tile: four 1 KB rows of 16 B per lane, lane chunk l ^ 8 (l / 32)
  __device__ __forceinline__ static int x_off(int l) { return (l ^ ((l >> 5) << 3)) << 4; }

  __device__ __forceinline__ void begin() {
    m_run = -INFINITY;
    l_run = 0.f;
    e_run = 0.f;
#pragma unroll
    for (int j = 0; j < CB; ++j) o[j] = f32x16{};
  }

  // Query fragments (MFMA B operand): lane (head, hb) holds dims
  // 16 (2 ks + half) + 8 hb + [0, 8).
  __device__ __forceinline__ void load_q() {
    const int l = threadIdx.x & 63, head = head_of(l);
    const bool head_ok = head < a.H;
    const uint16_t *qp = a.q + (static_cast<size_t>(b) * a.H + (head_ok ? head : 0)) * DROW + half * 16 + (l >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 32);
      if (!head_ok) v = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __device__ __forceinline__ int copies() const { return BlockCopier<NW>::copies(wave); }

  // Physical page of block blk: a scalar load from the block table, issued a
  // step before the copy that needs it so its latency stays off the LDS path.
  __device__ __forceinline__ int page_of(int blk) const {
    return ((const_i32 *)bt_row)[(t_begin + blk * TB) >> 6];
  }

  __device__ __forceinline__ void issue(int blk, int phys, uint8_t *slot) {
    const int tok0 = t_begin + blk * TB;
    BlockCopier<NW>::issue(a.cache, phys, tok0, min(TB, t_end - tok0) - 1, wave, threadIdx.x & 63, slot);
  }

  // Partial scores of the block in `slot` over this wave's 18 k-steps, then
  // published to the partner wave through this wave's exchange tile.
  __device__ __forceinline__ void scores(const uint8_t *slot) {
    const int l = lane_id();
    const int kb = k_base(l), krb = kr_base(l);

    // ---- partial scores over this wave's 18 k-steps.  Operands stream
    // through a ring PF k-steps deep so LDS latency overlaps earlier MFMAs;
    // the empty asm ties each MFMA operand to its place in the ring (without
    // it the scheduler sinks every read to just before its use).
    auto kread = [&](int ks) -> bf16x8 {
      const uint8_t *kp = ks < KS_LAT ? slot + (kb ^ ((ks & 3) * 64)) + (ks >> 2) * 256
                                      : slot + (krb ^ ((ks - KS_LAT) * 64));
      return *reinterpret_cast<const bf16x8 *>(kp);
    };
    constexpr int PF = 3;
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) kf[ks] = kread(ks);
    s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) kf[ks + PF] = kread(ks + PF);
      asm volatile("" : "+v"(kf[ks]) : : "memory");
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
    }

    uint8_t *mine = xch + wave * XCH_BYTES + x_off(l);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4 *>(mine + i * 1024) = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
  }

  // After the partner's partial is visible: full scores, online softmax and
  // the value product for the block in `slot` (block index blk).
  __device__ __forceinline__ void softmax_values(const uint8_t *slot, int blk) {
    const int tok0 = t_begin + blk * TB;
    const int l = lane_id(), hb = l >> 5;
    const int vb = v_base(l);
    // Both waves of the pair hold S_own + S_partner: the same fp32 sums, as
    // addition commutes.
    const uint8_t *theirs = xch + (wave ^ 1) * XCH_BYTES + x_off(l);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(theirs + i * 1024);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * i + e] += t[e];
    }

    // ---- online softmax: lane holds head l % 32 for tokens 8 (i / 4) + 4 hb + i % 4.
    // Scores stay unscaled; the scale c = softmax_scale * log2(e) > 0 enters
    // the running max (max(c s) = c max(s)) and the exponent as one fma.
    const float c = a.scale_log2;
    if (tok0 + TB > t_end) [[unlikely]] {
      // last block of the chunk: tokens at or past t_end do not exist
      const int lim = t_end - tok0 - 4 * hb;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + (i & 3) >= lim) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = max_xor32(mx) * c;
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run + RESCALE_SLACK)) {
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < CB; ++j) o[j] *= alpha;
      l_run *= alpha;
      e_run *= alpha;
      m_run = m_new;
    }
    // P as the MFMA B operand of token step t: k index 8 hb + j stands for
    // token 16 t + 8 (j / 4) + 4 hb + j % 4, i.e. score register 8 t + j.
    bf16x8 p[2];
    float pe = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_run));
      pe += pf;
      p[i >> 3][i & 7] = to_bf16(pf);
    }
    // sum of the rounded weights: bf16 pairs dotted with (1, 1)
    float ps = l_run;
    const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 pr = {p[i >> 2][2 * (i & 3)], p[i >> 2][2 * (i & 3) + 1]};
      ps = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps, false);
    }
    l_run = ps;
    e_run += pe;

    // ---- O^T[col, head] += V^T[col, token] P^T[token, head] over this wave's
    // 8 column blocks and the block's two 16-token steps.  A transposed read
    // returns 4 consecutive tokens of one column per lane: "lo" covers tokens
    // 16 t + 4 hb + [0, 4), "hi" the same 8 rows further.
    auto vread = [&](int n) -> bf16x8 {
      const int j = n >> 1, t = n & 1;
      const int x = vb ^ ((j & 3) * 64);
      const uint8_t *r0 = slot + x + (j >> 2) * 256 + t * 16 * LAT_BYTES;
      const uint8_t *r1 = slot + (x ^ 32) + (j >> 2) * 256 + t * 16 * LAT_BYTES + 8 * LAT_BYTES;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r1);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int PV = 2;
    constexpr int NV = 2 * CB;
    bf16x8 vf[NV];
#pragma unroll
    for (int n = 0; n < PV; ++n) vf[n] = vread(n);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + PV < NV) vf[n + PV] = vread(n + PV);
      asm volatile("" : "+v"(vf[n]) : : "memory");
      o[n >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n], p[n & 1], o[n >> 1], 0, 0, 0);
    }
  }

  // Lane (head l % 32, hb) holds columns 32 (8 half + j) + 8 q + 4 hb + [0, 4)
  // in registers 4 q .. 4 q + 3 of o[j].
  __device__ __forceinline__ void finish() {
    const float l_tot = sum_xor32(l_run);
    const float e_tot = sum_xor32(e_run);
    const float inv = 1.0f / l_tot;
    const float lse_v = (m_run + __log2f(e_tot)) * LN2;
    const int l = threadIdx.x & 63, hb = l >> 5, head = head_of(l);
    if (head >= a.H) return;
    uint16_t *dst;
    if (a.direct) {
      dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC;
      if (half == 0 && hb == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = lse_v;
    } else {
      const size_t row = (static_cast<size_t>(b) * a.n_splits + split) * a.H + head;
      dst = a.o_part + row * DC;
      if (half == 0 && hb == 0) a.lse_part[row] = lse_v;
    }
    dst += half * 256 + hb * 4;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[j][4 * q + e] * inv);
        *reinterpret_cast<bf16x4 *>(dst + j * 32 + q * 8) = v;
      }
    }
  }
};

// Wait until this wave's copies of block i have landed (copies of the next
// `ahead` blocks may still be in flight), then synchronise the workgroup.
template <int NI, int AHEAD>
__device__ __forceinline__ void wait_block(bool full_share) {
  if (full_share) wait_vmcnt<AHEAD * NI>();
  else wait_vmcnt<AHEAD * (NI - 1)>();
}

// Group X, block i in slot CUR: [wait copies of i] Ba [scores i] Bb [copy i + 2
// into NXT] [softmax + values i].
#define MLA_STEP_X(K, CUR, NXT)                                        \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    const int phys = i + 2 < nblk ? dec.page_of(i + 2) : 0;            \
    if (i + 1 < nblk) wait_block<D::NI, 1>(full_share);                \
    else wait_vmcnt<0>();                                              \
    barrier_no_fence();                                                \
    dec.scores(CUR);                                                   \
    barrier_lds();                                                     \
    if (i + 2 < nblk) dec.issue(i + 2, phys, NXT);                     \
    dec.softmax_values(CUR, i);                                        \
  }

// Group Y, block i >= 1 in slot CUR (block i - 1 in PRV, which is also the
// slot block i + 2 is copied into): [wait copies of i] Ba [softmax + values
// i - 1] Bb [copy i + 2 into PRV] [scores i].  Ba publishes Y's partials of
// i - 1.
#define MLA_STEP_Y(K, CUR, PRV)                                        \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    const int phys = i + 2 < nblk ? dec.page_of(i + 2) : 0;            \
    if (i + 1 < nblk) wait_block<D::NI, 1>(full_share);                \
    else wait_vmcnt<0>();                                              \
    barrier_lds();                                                     \
    dec.softmax_values(PRV, i - 1);                                    \
    barrier_no_fence();                                                \
    if (i + 2 < nblk) dec.issue(i + 2, phys, PRV);                     \
    dec.scores(CUR);                                                   \
  }

template <class D, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(D::NW * 64, D::NW * 64),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t slot0[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slot1[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slot2[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t xch[D::NW * XCH_BYTES];
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
  D dec(a, xch, b, split, t_begin, t_end);
  dec.begin();
  dec.load_q();
  wait_vmcnt<0>();            // query fragments landed before any copy is queued
  const bool full_share = dec.copies() == D::NI;

  const int nblk = (t_end - t_begin + TB - 1) / TB;
  dec.issue(0, dec.page_of(0), slot0);
  if (nblk > 1) dec.issue(1, dec.page_of(1), slot1);

  // Slot of block i: i % 3.  A slot is rewritten (block i + 3) only after the
  // second barrier of block i + 1, when both groups are done with block i.
  const bool group_y = NW == 8 && (threadIdx.x >> 8) != 0;
  if (!group_y) {
    for (int blk = 0; blk < nblk; blk += 3) {
      MLA_STEP_X(0, slot0, slot2)
      MLA_STEP_X(1, slot1, slot0)
      MLA_STEP_X(2, slot2, slot1)
    }
    barrier_no_fence();       // Y publishes its partials of the last block
  } else {
    // block 0: nothing of Y's to finish yet
    if (nblk > 1) wait_block<D::NI, 1>(full_share);
    else wait_vmcnt<0>();
    const int phys = nblk > 2 ? dec.page_of(2) : 0;
    barrier_lds();
    barrier_no_fence();
    if (nblk > 2) dec.issue(2, phys, slot2);
    dec.scores(slot0);
    for (int blk = 1; blk < nblk; blk += 3) {
      MLA_STEP_Y(0, slot1, slot0)
      MLA_STEP_Y(1, slot2, slot1)
      MLA_STEP_Y(2, slot0, slot2)
    }
    barrier_lds();
    const int last = nblk - 1;
    dec.softmax_values(last % 3 == 0 ? slot0 : (last % 3 == 1 ? slot1 : slot2), last);
  }
  dec.finish();
}

#undef MLA_STEP_X
#undef MLA_STEP_Y

// Merge split-KV partials: o = sum_c w_c o_c / sum_c w_c, w_c = exp(lse_c - L).
// One 64-lane group per (sequence, head), 8 columns per lane.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int t = threadIdx.x & 63;
  if (head >= a.H) return;
  const int S = a.seq_lens[b];
  const int nv = (S + a.split_tokens - 1) / a.split_tokens;
  uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + t * 8;
  if (nv <= 0) {
    *reinterpret_cast<u32x4 *>(dst) = u32x4{0, 0, 0, 0};
    if (t == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
    return;
  }
  const size_t stride = static_cast<size_t>(a.H);
  const float *lp = a.lse_part + static_cast<size_t>(b) * a.n_splits * stride + head;
  float L = -INFINITY;
  for (int c = 0; c < nv; ++c) L = fmaxf(L, lp[c * stride]);
  float acc[8] = {};
  float z = 0.f;
  const uint16_t *op = a.o_part + (static_cast<size_t>(b) * a.n_splits * stride + head) * DC + t * 8;
  for (int c = 0; c < nv; ++c) {
    const float w = expf(lp[c * stride] - L);
    z += w;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(op + c * stride * DC);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += w * __uint_as_float(v[e] & 0xFFFF0000u);
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
  switch (nw) {
    case 2: decode_bf16_kernel<DecoderPair<2>, 1><<<grid, 128, 0, stream>>>(a); break;
    case 4: decode_bf16_kernel<DecoderPair<4>, 1><<<grid, 256, 0, stream>>>(a); break;
    default: decode_bf16_kernel<DecoderPair<8>, 2><<<grid, 512, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  combine_kernel<<<dim3(a.B, (a.H + 3) / 4), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
