// Absorbed MLA decode over the fp8 latent cache with fp8 matrix products
// (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4), reading the E4M3 codes as
// stored instead of expanding them to bf16 first.
//
// The cache row keeps c_KV as E4M3 codes with one fp32 scale per 128-wide
// group, the rotary key in bf16 (Riju, "Multi-Head Latent Attention vs GQA vs
// MQA", "Interaction with quantisation and paging").  With k_t = [sc_t,g *
// code_t | kr_t] the scores and the weighted sum of the decoding-stage MQA
// form (Su, MLA Part 3, eq:mla-mqa) regroup by scale group g:
//   q . k_t  = sum_g sc_t,g (q_g . code_t,g) + q_R . kr_t
//   o_g      = sum_t (p_t sc_t,g) code_t,g
// so the codes enter both products unchanged, and each group's scale is
// applied to a per-group score accumulator (fp32, after the product) and
// folded into the weights of the value product.
//
// Operands in E4M3 carry 4 significant bits; one term each would leave the
// result several times outside the fp8-cache tolerance, so the query and the
// weights are each split into two E4M3 terms, x ~ hi + lo with hi = e4m3(x)
// and lo = e4m3(x - hi) (about 8 significant bits, close to bf16), and every
// product runs twice, hi and lo into one accumulator.  Power-of-two factors
// keep the terms inside the E4M3 range (the conversion does not saturate: an
// input beyond 448 becomes NaN) and are undone exactly by the MFMA's E8M0
// block scales:
//   query    per head: 2^a_h with max |q_h| 2^a_h in [128, 256); B scale
//            2^-a_h
//   weights  per block, head and group: B = p 2^k_h f_t,g, where 2^k_h
//            brings the head's largest weight of the block into [32, 64)
//            (so small weights stay clear of the E4M3 subnormals) and
//            f_t,g = sc_t,g 2^(1 - E_g) with 2^E_g <= max_t sc_t,g <
//            2^(E_g + 1), so f < 4 and B < 256; B scale 2^(E_g - 1 - k_h).
//            The score product of group g takes 2^(E_g - 1) as its A scale,
//            so that f_t,g turns its accumulator back into true units.
//
// Work split: one workgroup per (sequence, chunk, 128 heads), four waves,
// one per SIMD, 32 heads each; a block is one 64-token page, copied whole
// (41,984 contiguous bytes) into a ring of three LDS slots with 16-byte
// global->LDS copies.  Per block and wave:
//   scale table  the 64 tokens' group scales, their per-group maxima E_g and
//                f_t,g, written to this wave's own 1 KB table [g][token]
//   scores       S^T[token, head] for two 32-token halves: the rotary part
//                with 4 bf16 MFMAs (32x32x16), then per group 4 scaled fp8
//                MFMAs (2 k-steps of 64 codes x {hi, lo}) into a group
//                accumulator, added into the scores with f_t,g (fp32)
//   softmax      online, lazily rescaled, weights p = exp2(s - m) in fp32
//   values       per group: weights times f_t,g split into hi/lo E4M3 (the
//                B operand, 32 tokens per lane), then 4 column tiles x
//                {hi, lo} scaled fp8 MFMAs with the codes read transposed
//                (ds_read_b64_tr_b8) as the A operand
// The score accumulator's layout is the value product's B layout: lane
// (head n = l % 32, g = l / 32) holds the scores of tokens
// 32 h + 8 (i / 4) + 4 g + i % 4 in register i of half h, and byte
// p = 16 h + i of its value operand is that token's weight.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// LDS accesses at 32-bit LDS byte addresses: constant offsets fold into the
// instructions' immediate offset field (a generic pointer would be rebuilt
// from the aperture base at every access).
// A per-lane base the compiler cannot see into: it keeps base + constant
// as one register plus an immediate offset instead of precomputing (and
// spilling) each lane-dependent sum.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
template <class T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T *)(uintptr_t)addr;
}
template <class T>
__device__ __forceinline__ void lds_st(uint32_t addr, T v) {
  *(__attribute__((address_space(3))) T *)(uintptr_t)addr = v;
}

constexpr int TB8 = 64;                          // tokens per block: one page
constexpr int ROWB = FP8_ROW_BYTES;              // 656
constexpr int PAGE8 = TB8 * ROWB;                // 41,984
constexpr int ROW_PIECES = ROWB / 16;            // 41 16-byte pieces per row
constexpr int NW8 = 4;
constexpr int WPIECES = TB8 * ROW_PIECES / NW8;  // 656 pieces per wave per block
constexpr int NC8 = (WPIECES + 63) / 64;         // 11 copies per wave per block
constexpr int TAILC = WPIECES - (NC8 - 1) * 64;  // lanes of the last copy
constexpr int NSL = 3;
constexpr int TABLE_BYTES = 4 * TB8 * 4;         // fp32 [group][token]
constexpr int LDS8 = 128 * 1024;                 // the ring and tables; later the output tile
constexpr int QR_BYTES = 4 * 4 * 64 * 16;        // rotary query fragments: [wave][k-step][lane] 16 B
constexpr int SCALE_OFF = DC + DR * 2;           // 640: the group scales in a row
constexpr float SLACK8 = 6.0f;
constexpr float LN2_8 = 0.69314718055994530942f;
static_assert(NSL * PAGE8 + NW8 * TABLE_BYTES <= LDS8, "LDS budget");
static_assert(2 * NC8 <= 63 && TAILC > 0, "two blocks of copies fit the vmcnt counter");

__device__ __forceinline__ float max_swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Per-halfword maxima of a wave's 64 values (two unsigned 16-bit fields per
// word): lane swaps across l ^ 32 and l ^ 16, then rotations within each row
// of 16 lanes (DPP row_ror 8, 4, 2, 1) -- VALU only, no LDS round trips.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int pk_max_u16(int a, int b) {
  return __builtin_bit_cast(int, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ int wave_max_u16x2(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = pk_max_u16(static_cast<int>(r[0]), static_cast<int>(r[1]));
  r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = pk_max_u16(static_cast<int>(r[0]), static_cast<int>(r[1]));
  v = pk_max_u16(v, __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false));
  v = pk_max_u16(v, __builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false));
  v = pk_max_u16(v, __builtin_amdgcn_update_dpp(v, v, 0x122, 0xF, 0xF, false));
  v = pk_max_u16(v, __builtin_amdgcn_update_dpp(v, v, 0x121, 0xF, 0xF, false));
  return v;
}

// x -> (hi, lo) E4M3 pairs for 4 values, byte e of each word = value e.
struct TwoTerm {
  int hi, lo;
};
// The low word is written without a tied input (the builtin would first
// zero the register it then overwrites), the high word in place.
__device__ __forceinline__ int cvt_fp8_lo(float a, float b) {
  int r;
  asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ int cvt_fp8_hi(int r, float a, float b) {
  asm("v_cvt_pk_fp8_f32 %0, %1, %2 op_sel:[0,0,1]" : "+v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ TwoTerm split4(float x0, float x1, float x2, float x3) {
  const int hi = cvt_fp8_hi(cvt_fp8_lo(x0, x1), x2, x3);
  const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  const int lo = cvt_fp8_hi(cvt_fp8_lo(x0 - b01[0], x1 - b01[1]), x2 - b23[0], x3 - b23[1]);
  return TwoTerm{hi, lo};
}

struct DecoderF8 {
  static constexpr int HEADS = 128;

  const DecodeArgs &a;
  const int wave;
  const int b, split, grp;
  const int t_begin, t_end;
  const int32_t *bt_row;

  i32x8 qh[8], ql[8];      // latent query, two E4M3 terms, k-step ks: dims 64 ks + 32 g + [0, 32)
  uint32_t qr_lds;         // rotary query fragments in LDS, k-step ks at + 1024 ks: dims 16 ks + 8 g + [0, 8)
  int sb;                  // E8M0 of 2^-a_h
  f32x16 o[16];            // value accumulators, tile 4 g + c
  float m_run, l_run;

  __device__ DecoderF8(const DecodeArgs &args, int b_, int split_, int grp_, int t0, int t1)
      : a(args), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)), b(b_), split(split_), grp(grp_),
        t_begin(t0), t_end(t1), bt_row(args.block_table + static_cast<size_t>(b_) * args.max_blocks) {}

  __device__ __forceinline__ static int lane_id() { return threadIdx.x & 63; }
  __device__ __forceinline__ int head_of(int l) const { return grp * HEADS + wave * 32 + (l & 31); }

  __device__ __forceinline__ int page_of(int blk) const {
    return ((const_i32 *)bt_row)[(t_begin >> 6) + blk];
  }

  // Copies of block blk (one page) into `slot`: wave w moves 16-byte pieces
  // 656 w .. 656 w + 655 of the page, piece P of row P / 41 to slot offset
  // 16 P.  Rows past the end of the chunk re-read its last row (finite
  // data; their weights are zero).
  __device__ __forceinline__ void issue(int blk, uint32_t slot) const {
    const int tok0 = t_begin + blk * TB8;
    const int last = min(TB8, t_end - tok0) - 1;
    const uint8_t *base = a.cache + static_cast<size_t>(page_of(blk)) * PAGE8;
    // Opaque copy of the lane id: keeps the compiler from hoisting the
    // per-copy offsets out of the streaming loop into (spilled) registers.
    int l = lane_id();
    asm volatile("" : "+v"(l));
    const uint32_t dst = slot + wave * WPIECES * 16;
#pragma unroll
    for (int k = 0; k < NC8; ++k) {
      const int P = wave * WPIECES + 64 * k + l;
      int src = P;
      if (last < TB8 - 1) {
        const int row = P / ROW_PIECES;
        src = P + (row > last ? (last - row) * ROW_PIECES : 0);
      }
      if (k + 1 < NC8 || l < TAILC)
        dma16_s(static_cast<uint32_t>(src * 16), base, __builtin_amdgcn_readfirstlane(dst + k * 1024));
    }
  }

  // Query fragments straight from q: per head a power of two 2^a_h brings
  // max |q_lat| into [128, 256), then each value becomes hi + lo in E4M3.
  __device__ __forceinline__ void load_q(uint32_t qr_base) {
    const int l = lane_id(), g = l >> 5;
    const int head = head_of(l);
    const bool ok = head < a.H;
    const uint16_t *qp = a.q + (static_cast<size_t>(b) * a.H + (ok ? head : 0)) * DROW;
    u32x4 raw[8][4];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(qp + 64 * ks + 32 * g + 8 * j);
        raw[ks][j] = ok ? v : u32x4{0, 0, 0, 0};
      }
    qr_lds = qr_base + wave * 4096 + l * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qp + DC + 16 * ks + 8 * g);
      lds_st<u32x4>(qr_lds + 1024 * ks, ok ? v : u32x4{0, 0, 0, 0});
    }
    // max |q| as bf16 bits (non-negative bf16 patterns order as integers)
    uint32_t mx = 0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t v = raw[ks][j][d];
          mx = max(mx, max(v & 0x7FFFu, (v >> 16) & 0x7FFFu));
        }
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), 32)));
    const int eb = static_cast<int>(mx >> 7);               // biased exponent of max |q_h|
    const int e_h = eb == 0 ? 0 : max(eb - 127, -120);
    const int ah = 7 - e_h;
    sb = 127 - ah;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // bytes 4 k .. 4 k + 3: bf16 elements 4 k .. 4 k + 3 of the step
        const uint32_t w0 = raw[ks][k >> 1][2 * (k & 1)], w1 = raw[ks][k >> 1][2 * (k & 1) + 1];
        const float x0 = __builtin_ldexpf(__uint_as_float(w0 << 16), ah);
        const float x1 = __builtin_ldexpf(__uint_as_float(w0 & 0xFFFF0000u), ah);
        const float x2 = __builtin_ldexpf(__uint_as_float(w1 << 16), ah);
        const float x3 = __builtin_ldexpf(__uint_as_float(w1 & 0xFFFF0000u), ah);
        const TwoTerm t = split4(x0, x1, x2, x3);
        qh[ks][k] = t.hi;
        ql[ks][k] = t.lo;
      }
    }
  }

  __device__ __forceinline__ void begin() {
    m_run = -FLT_MAX;
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = f32x16{};
  }

  // Group scales of the block in `slot`: returns the E8M0 value of
  // 2^(E_g - 1) for each group and writes f_t,g to this wave's table.
  __device__ __forceinline__ void scale_table(uint32_t slot, uint32_t table, int (&s8)[4]) const {
    const int t = lane_id();
    const f32x4 sc = lds_ld<f32x4>(opaque_u32(slot + t * ROWB) + SCALE_OFF);
    int eb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) eb[g] = static_cast<int>((__float_as_uint(sc[g]) >> 23) & 0xFF);
    const int m01 = wave_max_u16x2(eb[0] | (eb[1] << 16));
    const int m23 = wave_max_u16x2(eb[2] | (eb[3] << 16));
    const int em[4] = {m01 & 0xFFFF, m01 >> 16, m23 & 0xFFFF, m23 >> 16};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int emax = max(__builtin_amdgcn_readfirstlane(em[g]), 1);   // biased E_g, normal range
      s8[g] = emax - 1;                                                 // 127 + E_g - 1
      lds_st<float>(table + 4 * (g * TB8 + t), __builtin_ldexpf(sc[g], 128 - emax));   // sc 2^(1 - E_g)
    }
  }

  // Score MFMAs, written out so that the score accumulator stays in fixed
  // VGPRs (v[16:31]) and the two group accumulators in v[32:47] / v[48:63]:
  // the compiler never copies them while an MFMA is still writing them (it
  // cannot see that an asm MFMA writes asynchronously).  A group chain's
  // result is read by VALU code only after the next chain has been issued
  // (four MFMAs of 16 passes behind it) or after explicit wait states.
  __device__ __forceinline__ static void mfma_rope(f32x16 &s, bf16x8 k, bf16x8 q, bool first) {
    if (first)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&{v[16:31]}"(s) : "v"(k), "v"(q));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{v[16:31]}"(s) : "v"(k), "v"(q));
  }
#define MLA_F8_GROUP_MFMA(NAME, REGS)                                                                      \
  __device__ __forceinline__ static void NAME(f32x16 &acc, const i32x8 &A, const i32x8 &B, int sa, int sbv,  \
                                              bool first) {                                                \
    if (first)                                                                                             \
      asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"    \
                   : "=&{" REGS "}"(acc) : "v"(A), "v"(B), "v"(sa), "v"(sbv));                             \
    else                                                                                                   \
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"              \
                   : "+{" REGS "}"(acc) : "v"(A), "v"(B), "v"(sa), "v"(sbv));                              \
  }
  MLA_F8_GROUP_MFMA(mfma_g0, "v[32:47]")
  MLA_F8_GROUP_MFMA(mfma_g1, "v[48:63]")
#undef MLA_F8_GROUP_MFMA

  // s[i] += f[g][token i] * acc[i] for half h (4 table reads of 4 tokens).
  __device__ __forceinline__ static void combine(f32x16 &s, const f32x16 &acc, uint32_t tg, int cg, int h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 f = lds_ld<f32x4>(tg + 4 * (cg * TB8 + 32 * h + 8 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * q + e] = __builtin_fmaf(f[e], acc[4 * q + e], s[4 * q + e]);
    }
  }

  // Scores of half h (tokens 32 h .. 32 h + 31) of the block in `slot`.
  // tg: this lane's table base (table + 16 g).
  // work(k), k = 0..7, runs after the MFMA pair of k-step k (VALU work of
  // another half that the MFMAs hide).
  template <class Work>
  __device__ __forceinline__ f32x16 scores(uint32_t slot, uint32_t tg, const int (&s8)[4], int h, Work &&work) const {
    const int l = lane_id(), m = l & 31, g = l >> 5;
    const uint32_t row = opaque_u32(slot + (32 * h + m) * ROWB + 32 * g);
    const uint32_t rrow = opaque_u32(slot + (32 * h + m) * ROWB + 16 * g);
    f32x16 s, acc0, acc1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kr = lds_ld<bf16x8>(rrow + DC + 32 * ks);
      const bf16x8 qk = lds_ld<bf16x8>(opaque_u32(qr_lds) + 1024 * ks);
      mfma_rope(s, kr, qk, ks == 0);
    }
    // codes of k-step ks + 1 are read before the MFMAs of k-step ks
    u32x4 c0 = lds_ld<u32x4>(row), c1 = lds_ld<u32x4>(row + 16);
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * cg + kk;
        const i32x8 A = __builtin_bit_cast(i32x8, __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7));
        if (ks + 1 < 8) {
          c0 = lds_ld<u32x4>(row + 64 * (ks + 1));
          c1 = lds_ld<u32x4>(row + 64 * (ks + 1) + 16);
        }
        asm volatile("" ::: "memory");
        if (cg & 1) {
          mfma_g1(acc1, A, qh[ks], s8[cg], sb, kk == 0);
          mfma_g1(acc1, A, ql[ks], s8[cg], sb, false);
        } else {
          mfma_g0(acc0, A, qh[ks], s8[cg], sb, kk == 0);
          mfma_g0(acc0, A, ql[ks], s8[cg], sb, false);
        }
        asm volatile("" ::: "memory");
        work(ks);
      }
      // the previous group's chain is four MFMAs behind: combine it
      if (cg == 1 || cg == 3) {
        asm volatile("" : "+{v[32:47]}"(acc0), "+{v[16:31]}"(s));
        combine(s, acc0, tg, cg - 1, h);
      } else if (cg == 2) {
        asm volatile("" : "+{v[48:63]}"(acc1), "+{v[16:31]}"(s));
        combine(s, acc1, tg, cg - 1, h);
      }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+{v[48:63]}"(acc1), "+{v[16:31]}"(s));
    combine(s, acc1, tg, 3, h);
    return s;
  }

  // Online softmax, one 32-token half at a time (lazily rescaled running
  // max m_run, log2 units).  Half 0's step k (0..7) runs between the score
  // MFMAs of half 1; half 1 then settles the block's k_h, which puts the
  // head's largest weight of the block in [32, 64): p 2^k_h replaces the
  // scores, l_run gathers the unscaled weights, and kmax keeps every B scale
  // 2^(E_g - 1 - k_h) inside the E8M0 range.
  struct Half0 {
    float mx;      // half 0's largest score (log2 units)
    float off;     // exponent offset of its weights: m_run - k0
    float ps;      // sum of its weights at scale 2^k0
    float alpha;   // rescale of the running sums at half 0
    int k0;
  };
  static __device__ __forceinline__ void mask_half(f32x16 &s, int lim, int h) {
    const int g = lane_id() >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (32 * h + 8 * (i >> 2) + 4 * g + (i & 3) >= lim) s[i] = -INFINITY;
  }
  template <bool MASK>
  __device__ __forceinline__ void soft0_step(int k, f32x16 &s0, Half0 &st, int lim, int kmax) {
    const float c = a.scale_log2;
    if (k == 0) {
      if (MASK) mask_half(s0, lim, 0);
      st.mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s0[4], s0[5]), fmaxf(s0[6], s0[7])));
      asm volatile("" : "+v"(st.mx));
    } else if (k == 1) {
      st.mx = fmaxf(st.mx, fmaxf(fmaxf(fmaxf(s0[8], s0[9]), fmaxf(s0[10], s0[11])),
                                 fmaxf(fmaxf(s0[12], s0[13]), fmaxf(s0[14], s0[15]))));
      st.mx = max_swap32(st.mx) * c;
      asm volatile("" : "+v"(st.mx));
    } else if (k == 2) {
      const float m_new = fmaxf(m_run, st.mx);
      const bool up = m_new > m_run + SLACK8;
      st.alpha = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = up ? m_new : m_run;
      // the half's largest weight is 2^d, d <= SLACK8: k0 = 5 - floor(d) >= -1
      st.k0 = min(5 - static_cast<int>(floorf(st.mx - m_run)), kmax);
      st.off = m_run - static_cast<float>(st.k0);
      st.ps = 0.f;
      asm volatile("" : "+v"(m_run), "+v"(st.alpha), "+v"(st.off), "+v"(st.k0));
    } else if (k < 7) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * (k - 3) + e;
        s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -st.off));
        st.ps += s0[i];
      }
      asm volatile("" : "+v"(st.ps));
    } else {
      l_run = l_run * st.alpha + __builtin_ldexpf(st.ps, -st.k0);
      asm volatile("" : "+v"(l_run));
    }
  }
  // Half 1 and the block's k_h (returned); rescales half 0's weights and the
  // value accumulators as needed.
  template <bool MASK>
  __device__ __forceinline__ int soft1(f32x16 &s0, f32x16 &s1, const Half0 &st, int lim, int kmax) {
    const float c = a.scale_log2;
    if (MASK) mask_half(s1, lim, 1);
    float mx = fmaxf(fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])), fmaxf(fmaxf(s1[4], s1[5]), fmaxf(s1[6], s1[7])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s1[8], s1[9]), fmaxf(s1[10], s1[11])),
                         fmaxf(fmaxf(s1[12], s1[13]), fmaxf(s1[14], s1[15]))));
    mx = max_swap32(mx) * c;
    const float m_new = fmaxf(m_run, mx);
    const bool up = m_new > m_run + SLACK8;
    const float alpha1 = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = up ? m_new : m_run;
    const int kh = min(5 - static_cast<int>(floorf(fmaxf(mx, st.mx) - m_run)), kmax);
    const float off = m_run - static_cast<float>(kh);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -off));
      ps += s1[i];
    }
    l_run = l_run * alpha1 + __builtin_ldexpf(ps, -kh);
    // half 0's weights from 2^k0 relative to the old running max to 2^k_h
    // relative to the new one
    const float f0 = __builtin_ldexpf(alpha1, kh - st.k0);
    if (__ballot(f0 != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s0[i] *= f0;
    }
    const float alpha = st.alpha * alpha1;
    if (__ballot(alpha != 1.0f)) {
      // in place on the accumulator registers, after the wait states of the
      // value MFMAs that wrote them last
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          float t;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\t"
                       "v_accvgpr_write_b32 %0, %1"
                       : "+a"(o[j][k]), "=&v"(t) : "v"(alpha));
        }
      asm volatile("s_nop 7" ::: "memory");
    }
    return kh;
  }

  // Value MFMA on an accumulator pinned to the AGPR file (the builtin would
  // let the compiler move the 256 accumulators through VGPRs).  Consecutive
  // MFMAs into the same accumulator need no wait states; readers of the
  // accumulators wait explicitly (rescale, fence_o).
  __device__ __forceinline__ static void mfma_pv(f32x16 &acc, const i32x8 &A, const i32x8 &B, int sa, int sbv,
                                                 bool nop) {
    if (nop)
      asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                   : "+a"(acc) : "v"(A), "v"(B), "v"(sa), "v"(sbv));
    else
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                   : "+a"(acc) : "v"(A), "v"(B), "v"(sa), "v"(sbv));
  }
  __device__ __forceinline__ void fence_o() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+a"(o[j]) : : "memory");
  }

  // Value product of the block in `slot` with weights p 2^k_h (in p0, p1).
  __device__ __forceinline__ void values(uint32_t slot, uint32_t tg, const int (&s8)[4], const f32x16 &p0,
                                         const f32x16 &p1, int kh) {
    const int l = lane_id(), g = l >> 5;
    // transposed-read base: lane pair (2 k, 2 k + 1) of each 16-lane group
    // supplies row k of the 8 x 16-byte tile: token 16 r + 8 (k / 4) + 4 g +
    // k % 4 for read r, bytes 64 (group & 1) + 8 (lane & 1) of the 32-column
    // tile's span
    const int k = (l & 15) >> 1;
    const int vrow = 8 * (k >> 2) + 4 * g + (k & 3);
    const uint32_t vb = opaque_u32(slot + vrow * ROWB + 64 * ((l >> 4) & 1) + 8 * (l & 1));
    // B operand of group cg, quarter c (words 2 c, 2 c + 1 of hi and lo):
    // weights of tokens 32 h + 8 q + 4 g + [0, 4), h = c / 2, q = 2 (c % 2) + [0, 2)
    auto build = [&](i32x8 &bh, i32x8 &bl, int cg, int c) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kw = 2 * c + k2, h = kw >> 2, q = kw & 3;
        const f32x4 f = lds_ld<f32x4>(tg + 4 * (cg * TB8 + 32 * h + 8 * q));
        const f32x16 &p = h ? p1 : p0;
        const TwoTerm t = split4(p[4 * q] * f[0], p[4 * q + 1] * f[1], p[4 * q + 2] * f[2], p[4 * q + 3] * f[3]);
        bh[kw] = t.hi;
        bl[kw] = t.lo;
      }
    };
    i32x8 bh[2], bl[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) build(bh[0], bl[0], 0, c);
    auto vread = [&](int cg, int c) {
      i32x8 A;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2 *)(uintptr_t)(vb + r * 16 * ROWB + 128 * cg + 16 * c));
        A[2 * r] = v[0];
        A[2 * r + 1] = v[1];
      }
      return A;
    };
    i32x8 An = vread(0, 0);
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x8 A = An;
        if (4 * cg + c + 1 < 16) An = vread((4 * cg + c + 1) >> 2, (c + 1) & 3);
        asm volatile("" ::: "memory");
        mfma_pv(o[4 * cg + c], A, bh[cg & 1], 127, s8[cg] - kh, c == 0);
        mfma_pv(o[4 * cg + c], A, bl[cg & 1], 127, s8[cg] - kh, false);
        // the next group's weights, a quarter per column tile, while these run
        if (cg < 3) build(bh[(cg + 1) & 1], bl[(cg + 1) & 1], cg + 1, c);
      }
    }
  }

  // lim: tokens of the block inside the chunk; MASK: lim may be below 64.
  template <bool MASK>
  __device__ __forceinline__ void block(uint32_t slot, uint32_t table, int lim) {
    int s8[4];
    scale_table(slot, table, s8);
    const uint32_t tg = opaque_u32(table + 16 * (lane_id() >> 5));
    const int kmax = min(min(s8[0], s8[1]), min(s8[2], s8[3]));
    f32x16 s0 = scores(slot, tg, s8, 0, [](int) {});
    Half0 st;
    f32x16 s1 = scores(slot, tg, s8, 1, [&](int k) { soft0_step<MASK>(k, s0, st, lim, kmax); });
    const int kh = soft1<MASK>(s0, s1, st, lim, kmax);
    values(slot, tg, s8, s0, s1, kh);
  }

  // Normalise and store through LDS (row = head of the workgroup, 1 KB of
  // bf16; 16-byte chunk C at position C ^ (row & 15)).  Register i of tile
  // 4 cg + c holds latent column 128 cg + 64 (i / 8) + 16 c + 8 ((i / 4) & 1)
  // + 4 g + i % 4.
  __device__ __forceinline__ void finish(uint8_t *stage) {
    const int l = lane_id(), g = l >> 5;
    const float l_tot = sum_swap32(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = (m_run + __log2f(l_tot)) * LN2_8;
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
    uint8_t *srow = stage + row * (DC * 2) + 8 * g;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[4 * cg + c][4 * q + e] * inv);
          const int C = 16 * cg + 8 * (q >> 1) + 2 * c + (q & 1);
          *reinterpret_cast<bf16x4 *>(srow + ((C ^ (row & 15)) << 4)) = v;
        }
    asm volatile("" ::: "memory");   // a wave's LDS accesses complete in order
#pragma unroll 4
    for (int kk = 0; kk < 32; ++kk) {
      const int r = wave * 32 + kk;
      const int h = grp * HEADS + r;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * (DC * 2) + ((l ^ (r & 15)) << 4));
      if (h < a.H) {
        uint16_t *dst = a.direct ? a.o_latent + (static_cast<size_t>(b) * a.H + h) * DC
                                 : a.o_part + ((static_cast<size_t>(b) * a.n_splits + split) * a.H + h) * DC;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + l * 8));
      }
    }
  }
};

// Iteration i: [wait this wave's copies of block i] barrier (block i
// visible; every wave done with block i - 1, whose slot receives block
// i + 2) [copies of block i + 2] [scale table, scores, softmax, values of
// block i].  Slot of block i: i % 3.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_fp8_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS8 + QR_BYTES];
  static_assert(DecoderF8::HEADS * DC * 2 <= LDS8, "the output tile is staged in LDS");

  // One workgroup per (sequence, chunk, head group); ids are remapped so
  // that consecutive items share an XCD (workgroups are dealt to the 8 XCDs
  // round-robin).
  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int groups = (a.H + DecoderF8::HEADS - 1) / DecoderF8::HEADS;
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
      const int head = grp * DecoderF8::HEADS + t / 2;        // 2 threads per head
      if (head < a.H) {
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % 2) * (DC / 2);
        for (int c = 0; c < DC / 2; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % 2 == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  DecoderF8 dec(a, b, split, grp, t_begin, t_end);
  const int nblk = (t_end - t_begin + TB8 - 1) / TB8;
  const uint32_t lds0 = lds_addr(lds);
  auto slot = [&](int i) { return lds0 + (i % NSL) * PAGE8; };
  const uint32_t table = lds0 + NSL * PAGE8 + dec.wave * TABLE_BYTES;
  dec.issue(0, slot(0));
  if (nblk > 1) dec.issue(1, slot(1));
  dec.begin();
  dec.load_q(lds0 + LDS8);
  for (int i = 0; i + 1 < nblk; ++i) {
    wait_vmcnt<NC8>();
    barrier_no_fence();
    if (i + 2 < nblk) dec.issue(i + 2, slot(i + 2));
    dec.block<false>(slot(i), table, TB8);
  }
  wait_vmcnt<0>();
  barrier_no_fence();
  dec.block<true>(slot(nblk - 1), table, t_end - (t_begin + (nblk - 1) * TB8));
  dec.fence_o();
  dec.finish(lds);
}

}  // namespace

hipError_t launch_decode_fp8_mfma(const DecodeArgs &a, hipStream_t stream) {
  if (!a.kv_fp8 || a.q_len > 1) return hipErrorInvalidValue;
  const int groups = (a.H + DecoderF8::HEADS - 1) / DecoderF8::HEADS;
  decode_fp8_mfma_kernel<<<dim3(a.B * a.n_splits * groups, 1), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
