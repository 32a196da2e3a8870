// Absorbed MLA decode over a paged latent cache, gfx950.
//
// Every head scores the same cached row [c_KV | rotated k_R] (576 values), so
// a workgroup streams each 32-token block of a sequence from HBM into LDS once
// and all of its heads (up to 128, 16 per wave, 8 waves) consume it there:
//   S^T[tok, head] = K[tok, 0:576] . Q^T[0:576, head]     MFMA 16x16x32 bf16
//   online softmax per head (fp32, exp2, lazily rescaled)
//   O^T[col, head] += V^T[col, tok] . P^T[tok, head]      MFMA, V = K[:, 0:512]
// The decoding-stage MQA form of MLA (Su, "The Ultimate Tug-of-War Between
// Cache and Performance", MLA Part 3, eq:mla-mqa); one loaded latent serves
// every head (Riju, "Multi-Head Latent Attention vs GQA vs MQA", "Arithmetic
// intensity changes under absorption").
//
// Data movement: 16-byte global->LDS DMA copies (global_load_lds_dwordx4),
// one 1 KB latent row per wave-wide copy, into a ring of four 36 KB slots:
// three blocks in flight while one is computed.  Chunks are XOR-swizzled per
// row so that the row-wise reads of the score product and the transposed
// reads (ds_read_b64_tr_b16) of the value product spread over the LDS banks.
// The value operand is read transposed straight out of the same tile: no
// second copy of V exists anywhere.
//
// Split-KV: a sequence may be cut into chunks of split_tokens; each chunk
// writes (o / l in bf16, lse in fp32) partials and a combine kernel merges
// them with log-sum-exp weights in fp32.
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
constexpr int KSTEPS = DROW / 32;               // 18 MFMA k-steps over 576
constexpr int KLAT = DC / 32;                   // 16 of them over the latent
constexpr int CBLKS = DC / 16;                  // 32 column blocks of O
constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_SLACK = 8.0f;           // log2 units a stale max may lag
constexpr int MAX_SPLIT_PAGES = MLA_MAX_SPLIT_TOKENS / PAGE;

// LDS slot layout for a block of 32 tokens:
//   [0, 32 KB)      latent rows, 1024 B each; 16-byte chunk c of row r sits at
//                   chunk position c ^ fl(r) (XOR inside aligned 16-chunk groups)
//   [32 KB, 36 KB)  rotary keys, 128 B each; chunk c of row r at c ^ (r & 7)
// fl is a bijection on 0..15 chosen so that (a) 16 consecutive rows reading the
// same chunk and (b) 4 aligned consecutive rows reading an aligned chunk pair
// (the transposed value reads) each touch distinct banks.
__device__ __forceinline__ int fl(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// 8-dim group of a 32-dim k-step that the 16-lane group g of a wave reads in
// the score product.  With lane groups 1 and 2 exchanged, the 16 lanes the LDS
// serves together in a 128-bit read hit 16 distinct bank quads (measured on
// gfx950: the identity order costs a 2-way conflict on every score read).
__device__ __forceinline__ int kgroup(int g) { return ((g & 1) << 1) | (g >> 1); }

// Pairwise reductions across lanes l ^ 16 and l ^ 32 with the gfx950 lane
// swaps (VALU; no LDS traffic).  Both lanes of a pair get the same result.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// The copy (DMA) side of a decoder: which rows of a block each wave moves.
template <int NW>
struct BlockCopier {
  static constexpr int NI = (NDMA + NW - 1) / NW;       // max DMA copies per wave per block
  static_assert(3 * NI <= 63, "three blocks of copies must fit the vmcnt counter");

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
    // per-copy address arithmetic out of the streaming loop into registers.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = wave + i * NW;
      if (i * NW + NW <= NDMA || n < NDMA) {
        if (n < TB) {
          const int r = min(n, last);
          dma16(base + r * ROW_BYTES + ((ln ^ fl(n)) << 4),
                __builtin_amdgcn_readfirstlane(slot_lds + n * LAT_BYTES));
        } else {
          const int rr = (n - TB) * 8 + (ln >> 3);
          const int r = min(rr, last);
          dma16(base + r * ROW_BYTES + LAT_BYTES + (((ln & 7) ^ (rr & 7)) << 4),
                __builtin_amdgcn_readfirstlane(slot_lds + SLOT_LAT + (n - TB) * 1024));
        }
      }
    }
  }
};

// 16 heads per wave: v_mfma_f32_16x16x32_bf16, two waves per SIMD.
template <int NW_>
struct DecoderW16 {
  static constexpr int NW = NW_;
  static constexpr int HPW = 16;
  static constexpr int NI = BlockCopier<NW>::NI;

  const DecodeArgs &a;
  const int lane, wave, g, r16;
  const int b, split, head;
  const bool head_ok;
  const int t_begin, t_end;
  const int32_t *pages;       // LDS copy of the chunk's page ids

  bf16x8 qf[KSTEPS];
  f32x4 o[CBLKS];
  // m_run: running max (log2 units); l_run: sum of the bf16-rounded weights
  // that multiply V (normalises o consistently); e_run: the same sum of the
  // unrounded weights (gives an lse free of the bf16 rounding of P).
  float m_run, l_run, e_run;
  // per-lane LDS byte offsets; every LDS read is one of these plus a constant
  int k_off[4];               // latent score reads, ks & 3
  int kr_off[2];              // rotary score reads, ks - 16
  int v_off[8];               // transposed value reads, cb & 7

  __device__ DecoderW16(const DecodeArgs &args, const int32_t *pages_, int b_, int split_, int t0, int t1)
      : a(args), lane(threadIdx.x & 63), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        g((threadIdx.x & 63) >> 4),
        r16(threadIdx.x & 15), b(b_), split(split_),
        head((blockIdx.y * NW + (threadIdx.x >> 6)) * HPW + (threadIdx.x & 15)),
        head_ok(((blockIdx.y * NW + (threadIdx.x >> 6)) * HPW + (threadIdx.x & 15)) < args.H),
        t_begin(t0), t_end(t1), pages(pages_) {}

  __device__ __forceinline__ void begin() {
    m_run = -INFINITY;
    l_run = 0.f;
    e_run = 0.f;
#pragma unroll
    for (int cb = 0; cb < CBLKS; ++cb) o[cb] = f32x4{};
    // score reads: row r16 (+16), latent chunk 4 ks + kg = 16 (ks >> 2) + (4 (ks & 3) + kg)
    const int kg = kgroup(g);
#pragma unroll
    for (int e = 0; e < 4; ++e) k_off[e] = r16 * LAT_BYTES + (((4 * e + kg) ^ fl(r16)) << 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) kr_off[e] = SLOT_LAT + r16 * ROPE_BYTES + (((4 * e + kg) ^ (r16 & 7)) << 4);
    // value reads: row trow (+16), latent chunk 2 cb + csub = 16 (cb >> 3) + (2 (cb & 7) + csub),
    // byte (r16 & 1) * 8 inside the chunk
    const int trow = g * 4 + (r16 >> 2);
    const int csub = (r16 & 3) >> 1;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v_off[e] = trow * LAT_BYTES + (((2 * e + csub) ^ fl(trow)) << 4) + (r16 & 1) * 8;
  }

  // Query fragments (MFMA B operand): lane (head, g) holds dims [32 ks + 8 kgroup(g), +8),
  // the same 8-dim group its score reads fetch from the cached rows.
  __device__ __forceinline__ void load_q() {
    const uint16_t *qp = a.q + (static_cast<size_t>(b) * a.H + (head_ok ? head : 0)) * DROW + kgroup(g) * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 32);
      if (!head_ok) v = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __device__ __forceinline__ int copies() const { return BlockCopier<NW>::copies(wave); }

  __device__ __forceinline__ void issue(int blk, uint8_t *slot) {
    const int tok0 = t_begin + blk * TB;
    const int phys = __builtin_amdgcn_readfirstlane(pages[(tok0 - t_begin) >> 6]);
    BlockCopier<NW>::issue(a.cache, phys, tok0, min(TB, t_end - tok0) - 1, wave, lane, slot);
  }

  __device__ __forceinline__ void compute(const uint8_t *slot, int blk) {
    const int tok0 = t_begin + blk * TB;

    // ---- scores S^T[token, head] for the two 16-token halves of the block
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint8_t *kp = ks < KLAT ? slot + k_off[ks & 3] + (ks >> 2) * 256 : slot + kr_off[ks - KLAT];
      const int second = ks < KLAT ? 16 * LAT_BYTES : 16 * ROPE_BYTES;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8 *>(kp);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8 *>(kp + second);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
    }

    // ---- online softmax: lane holds head r16 for tokens 4g+i and 16+4g+i
    float xs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = (i < 4 ? s0[i] : s1[i - 4]) * a.scale_log2;
    if (tok0 + TB > t_end) [[unlikely]] {
      // last block of the chunk: tokens at or past t_end do not exist
      const int lim = t_end - tok0 - g * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i >> 2) * 16 + (i & 3) >= lim) xs[i] = -INFINITY;
    }
    float mx = xs[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, xs[i]);
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run + RESCALE_SLACK)) {
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int cb = 0; cb < CBLKS; ++cb) o[cb] *= alpha;
      l_run *= alpha;
      e_run *= alpha;
      m_run = m_new;
    }
    bf16x8 p;
    float ps = 0.f, pe = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pf = __builtin_amdgcn_exp2f(xs[i] - m_run);
      const __bf16 pb = to_bf16(pf);
      pe += pf;
      ps += static_cast<float>(pb);
      p[i] = pb;
    }
    l_run += ps;
    e_run += pe;

    // ---- O^T[col, head] += V^T[col, token] P^T[token, head]
    // The MFMA k index 8g + j stands for token 4g + j (j < 4) and 16 + 4g + j - 4
    // (j >= 4): the order in which the score accumulators hold P.  Each
    // transposed read returns 4 tokens of one column per lane; lane
    // (16g + 4r + q) supplies the address of token row r, columns [4q, 4q+4)
    // of the 16-column block.
#pragma unroll
    for (int cb = 0; cb < CBLKS; ++cb) {
      const uint8_t *r0 = slot + v_off[cb & 7] + (cb >> 3) * 256;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + 16 * LAT_BYTES));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, p, o[cb], 0, 0, 0);
    }
  }

  // lane (head r16, g) holds columns 16 cb + 4 g + [0,4) of its head.
  __device__ __forceinline__ void finish() {
    const float l_tot = sum_xor32(sum_xor16(l_run));
    const float e_tot = sum_xor32(sum_xor16(e_run));
    const float inv = 1.0f / l_tot;
    const float lse_v = (m_run + __log2f(e_tot)) * LN2;
    if (!head_ok) return;
    if (a.direct) {
      uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + g * 4;
#pragma unroll
      for (int cb = 0; cb < CBLKS; ++cb) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[cb][e] * inv);
        *reinterpret_cast<bf16x4 *>(dst + cb * 16) = v;
      }
      if (g == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = lse_v;
    } else {
      const size_t row = (static_cast<size_t>(b) * a.n_splits + split) * a.H + head;
      uint16_t *dst = a.o_part + row * DC + g * 4;
#pragma unroll
      for (int cb = 0; cb < CBLKS; ++cb) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[cb][e] * inv);
        *reinterpret_cast<bf16x4 *>(dst + cb * 16) = v;
      }
      if (g == 0) a.lse_part[row] = lse_v;
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

#define MLA_DECODE_STEP(K, CUR, NXT)                                   \
  {                                                                    \
    const int i = blk + (K);                                           \
    if (i >= nblk) break;                                              \
    if (i + 2 < nblk) wait_block<D::NI, 2>(full_share);                \
    else if (i + 1 < nblk) wait_block<D::NI, 1>(full_share);           \
    else wait_vmcnt<0>();                                              \
    barrier_no_fence();                                                \
    if (i + 3 < nblk) dec.issue(i + 3, NXT);                           \
    dec.compute(CUR, i);                                               \
  }

template <class D, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(D::NW * 64, D::NW * 64),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t slot0[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slot1[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slot2[SLOT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slot3[SLOT_BYTES];
  __shared__ int32_t pages[MAX_SPLIT_PAGES];
  constexpr int NW = D::NW;

  const int item = blockIdx.x;
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
      const int per = NW * 64 / (D::HPW * NW);            // threads per head
      const int head = blockIdx.y * D::HPW * NW + t / per;
      if (head < a.H) {
        const int cols = DC / per;
        uint16_t *dst = a.o_latent + (static_cast<size_t>(b) * a.H + head) * DC + (t % per) * cols;
        for (int c = 0; c < cols; c += 8) *reinterpret_cast<u32x4 *>(dst + c) = u32x4{0, 0, 0, 0};
        if (t % per == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.H + head] = -INFINITY;
      }
    }
    return;
  }

  // Page ids of this chunk -> LDS, so the streaming loop issues no vector
  // loads besides its DMA copies (vmcnt then counts exactly those).
  {
    const int32_t *bt = a.block_table + static_cast<size_t>(b) * a.max_blocks + (t_begin >> 6);
    const int np = (t_end - t_begin + PAGE - 1) / PAGE;
    for (int i = threadIdx.x; i < np; i += NW * 64) pages[i] = bt[i];
  }
  __syncthreads();

  D dec(a, pages, b, split, t_begin, t_end);
  dec.begin();
  dec.load_q();
  wait_vmcnt<0>();            // query fragments landed before any copy is queued
  const bool full_share = dec.copies() == D::NI;

  const int nblk = (t_end - t_begin + TB - 1) / TB;
  dec.issue(0, slot0);
  if (nblk > 1) dec.issue(1, slot1);
  if (nblk > 2) dec.issue(2, slot2);

  for (int blk = 0; blk < nblk; blk += 4) {
    MLA_DECODE_STEP(0, slot0, slot3)
    MLA_DECODE_STEP(1, slot1, slot0)
    MLA_DECODE_STEP(2, slot2, slot1)
    MLA_DECODE_STEP(3, slot3, slot2)
  }
  dec.finish();
}

#undef MLA_DECODE_STEP

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
    case 2: decode_bf16_kernel<DecoderW16<2>, 1><<<grid, 128, 0, stream>>>(a); break;
    case 4: decode_bf16_kernel<DecoderW16<4>, 1><<<grid, 256, 0, stream>>>(a); break;
    default: decode_bf16_kernel<DecoderW16<8>, 2><<<grid, 512, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  combine_kernel<<<dim3(a.B, (a.H + 3) / 4), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
