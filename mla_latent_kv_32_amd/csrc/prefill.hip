// Prefill of whole prompts in the explicit (non-absorbed) form.
//
// For prompts the absorbed form would multiply the attention FLOPs by
// (576 + 512) / (192 + 128) = 3.4 (Su, "The Ultimate Tug-of-War Between Cache
// and Performance", Part 3: MHA form eq:mla-mha for training and prefill, the
// MQA form eq:mla-mqa for decoding; Riju, "Multi-Head Latent Attention vs GQA
// vs MQA", non-absorbed module).  So each head gets its own keys and values,
// rebuilt from the latent:
//   K^(h) = [c W_UK[h]^T | RoPE(k_pe)]   (192 wide; the rotary part shared)
//   V^(h) = c W_UV[h]                    (128 wide)
//   o_t^(h) = sum_{i <= t} softmax_i(scale [q_nope | RoPE(q_pe)]_t . K_i^(h)) V_i^(h)
// and the prompt's rows [c_t | RoPE(k_pe_t, t)] go to the paged latent cache
// for the decode steps that follow.  Token t of a prompt sits at position t.
//
// Precision.  The attention's operands -- the rotated query and key, the
// materialised K_nope and V, and the softmax weights P -- are IEEE half
// (fp16 MFMAs, fp32 accumulation): each is one rounding away from its fp32
// value, and half's 11-bit significand keeps the sum of those roundings
// inside 2e-3 + 2e-2 |o| where bf16's 8 bits do not (a row of a short
// prefix is a sum of a few O(1) terms).  q_nope arrives in bf16 and converts
// to half exactly.  Half is finite below 65520: per-head keys, values and
// queries must stay below that magnitude (unit-scale activations are five
// orders of magnitude inside it); P stays at most 2^8 by the lazy rescale.
//
// Launches: RoPE + cache rows; the two up-projections; causal attention.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {
namespace {

// ---- RoPE of the prompt tokens and their cache rows.  Workgroup (b, y)
// handles positions 8 y .. 8 y + 7 of prompt b: the angles of all eight
// tokens first (one thread per token and pair), then the query pairs of
// every head in 16-byte pieces (to the workspace, in fp16), the shared rotary
// key (to the workspace in fp16, for the attention) and the cache rows (bf16
// or fp8, as every cache row).
constexpr int ROPE_TOK = 8;

__global__ __launch_bounds__(256) void prefill_rope_kernel(PrefillArgs a) {
  __shared__ float cs[ROPE_TOK][DR / 2], sn[ROPE_TOK][DR / 2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t_begin = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - t_begin;
  const int P = a.prefix_lens ? a.prefix_lens[b] : 0;     // token j of the prompt sits at position P + j
  const int k_begin = a.cu_keys[b] + P;                    // its key index: k_begin + j
  const int p0 = blockIdx.y * ROPE_TOK;
  if (p0 >= L) return;
  const int ntok = min(ROPE_TOK, L - p0);
  {
    const int j = tid / (DR / 2), i = tid % (DR / 2);
    if (j < ntok) rope_cos_sin(a.inv_freq, P + p0 + j, i, cs[j][i], sn[j][i]);
  }
  if (a.prefix_lens) {
    // the prompt's own latents join the prefix's in the key array (exact in
    // bf16: a second term, if the rows have one, is zero)
    const int pieces = a.c_keys_w / 8;
    for (int idx = tid; idx < ntok * pieces; idx += blockDim.x) {
      const int j = idx / pieces, v = idx % pieces;
      const int kk = min(k_begin + p0 + j, a.T_keys - 1);
      const u32x4 val = v < DC / 8
          ? *reinterpret_cast<const u32x4 *>(a.c + (static_cast<size_t>(t_begin) + p0 + j) * DC + 8 * v)
          : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4 *>(a.c_gather + static_cast<size_t>(kk) * a.c_keys_w + 8 * v) = val;
    }
  }
  __syncthreads();
  const int H = a.H;
  constexpr int VEC = DR / 8;                          // 16-byte pieces of a rotary part
  for (int idx = tid; idx < ntok * H * VEC; idx += blockDim.x) {
    const int j = idx / (H * VEC), rem = idx % (H * VEC), h = rem / VEC, v = rem % VEC;
    const size_t off = ((static_cast<size_t>(t_begin) + p0 + j) * H + h) * DR + 8 * v;
    u32x4 pr = *reinterpret_cast<const u32x4 *>(a.q_pe + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = rope_rotate_pair_f16(pr[e], cs[j][4 * v + e], sn[j][4 * v + e]);
    *reinterpret_cast<u32x4 *>(a.q_rot + off) = pr;
  }
  if (tid < ntok * VEC) {
    const int j = tid / VEC, v = tid % VEC;
    const size_t off = (static_cast<size_t>(t_begin) + p0 + j) * DR + 8 * v;
    u32x4 pr = *reinterpret_cast<const u32x4 *>(a.k_pe + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = rope_rotate_pair_f16(pr[e], cs[j][4 * v + e], sn[j][4 * v + e]);
    const int kk = min(k_begin + p0 + j, a.T_keys - 1);
    *reinterpret_cast<u32x4 *>(a.k_rot + static_cast<size_t>(kk) * DR + 8 * v) = pr;
  }
  for (int j = 0; j < ntok; ++j) {
    const int pos = P + p0 + j;
    const size_t t = static_cast<size_t>(t_begin) + p0 + j;
    // (a position past the block-table row -- a prefix and chunk longer
    // than the row allows, which the caller must not pass -- is clamped to
    // the row's last page instead of reading past it)
    const int page = a.block_table[static_cast<size_t>(b) * a.max_blocks + min(pos / PAGE, a.max_blocks - 1)];
    store_cache_row(a.cache, a.kv_fp8, static_cast<size_t>(page) * PAGE + pos % PAGE, a.c + t * DC,
                    a.k_pe + t * DR, tid, cs[j], sn[j]);
  }
}

// ---- chunks: key offsets cu_keys[b] = sum_{b' < b} (P_b' + L_b'), one
// workgroup (contiguous ranges per thread, then a scan of the 256 range sums).
__global__ __launch_bounds__(256) void prefill_keys_scan_kernel(const int32_t *cu_seqlens, const int32_t *prefix,
                                                                int32_t *cu_keys, int B) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (B + 255) / 256, b0 = tid * per, b1 = min(B, b0 + per);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += prefix[b] + cu_seqlens[b + 1] - cu_seqlens[b];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    cu_keys[B] = run;
  }
  __syncthreads();
  int run = part[tid];
  for (int b = b0; b < b1; ++b) {
    cu_keys[b] = run;
    run += prefix[b] + cu_seqlens[b + 1] - cu_seqlens[b];
  }
}

// ---- chunks: the cached prefix rows into the key arrays.  Workgroup (b, y)
// handles prefix positions 8 y .. 8 y + 7 of prompt b: latent to c_gather
// (bf16 rows as stored; fp8 rows as two bf16 terms of code * group scale,
// hi = bf16(x) and lo = bf16(x - hi), within 2^-17 of x, so that rounding
// the dequantised latent before the up-projection -- where the per-head
// products could cancel far below its size -- costs nothing visible), the
// stored rotated key to k_rot in half.
__global__ __launch_bounds__(256) void prefill_gather_kernel(PrefillArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int P = a.prefix_lens[b];
  const int p0 = blockIdx.y * ROPE_TOK;
  if (p0 >= P) return;
  const int ntok = min(ROPE_TOK, P - p0);
  const int k_begin = a.cu_keys[b];
  const int j = tid >> 5, lane = tid & 31;                 // 32 threads per token
  if (j >= ntok) return;
  const int pos = p0 + j;
  const int page = a.block_table[static_cast<size_t>(b) * a.max_blocks + min(pos / PAGE, a.max_blocks - 1)];
  const size_t slot = static_cast<size_t>(page) * PAGE + pos % PAGE;
  const size_t kk = static_cast<size_t>(min(k_begin + pos, a.T_keys - 1));
  uint16_t *cdst = a.c_gather + kk * a.c_keys_w + 16 * lane;   // 16 latent values per thread
  const uint16_t *rope_src;
  if (a.kv_fp8) {
    const uint8_t *row = a.cache + slot * FP8_ROW_BYTES;
    const u32x4 codes = *reinterpret_cast<const u32x4 *>(row + 16 * lane);
    const float sc = *reinterpret_cast<const float *>(row + DC + 2 * DR + 4 * (lane >> 3));
    uint16_t hi16[16], lo16[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 c01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[w]), false);
      const f32x2 c23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[w]), true);
      const float x[4] = {c01[0] * sc, c01[1] * sc, c23[0] * sc, c23[1] * sc};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 h = to_bf16(x[e]);
        hi16[4 * w + e] = bf16_bits(h);
        lo16[4 * w + e] = bf16_bits(to_bf16(x[e] - static_cast<float>(h)));
      }
    }
    *reinterpret_cast<u32x4 *>(cdst) = *reinterpret_cast<const u32x4 *>(hi16);
    *reinterpret_cast<u32x4 *>(cdst + 8) = *reinterpret_cast<const u32x4 *>(hi16 + 8);
    *reinterpret_cast<u32x4 *>(cdst + DC) = *reinterpret_cast<const u32x4 *>(lo16);
    *reinterpret_cast<u32x4 *>(cdst + DC + 8) = *reinterpret_cast<const u32x4 *>(lo16 + 8);
    rope_src = reinterpret_cast<const uint16_t *>(row + DC);
  } else {
    const uint16_t *row = reinterpret_cast<const uint16_t *>(a.cache) + slot * DROW;
    *reinterpret_cast<u32x4 *>(cdst) = *reinterpret_cast<const u32x4 *>(row + 16 * lane);
    *reinterpret_cast<u32x4 *>(cdst + 8) = *reinterpret_cast<const u32x4 *>(row + 16 * lane + 8);
    rope_src = row + DC;
  }
  if (lane < DR / 8) {
    // bf16 -> half: exact for magnitudes in [2^-14, 65504]
    const u32x4 r = *reinterpret_cast<const u32x4 *>(rope_src + 8 * lane);
    u32x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo16 = f16_bits(__uint_as_float(r[e] << 16));
      const uint32_t hi16 = f16_bits(__uint_as_float(r[e] & 0xFFFF0000u));
      h[e] = lo16 | (hi16 << 16);
    }
    *reinterpret_cast<u32x4 *>(a.k_rot + kk * DR + 8 * lane) = h;
  }
}

// ---- per-head up-projection of the shared latent: out[t, h, :] =
// c[t, :] . W[h] (K = 512, N = 128; W = W_UK^T, read from W_UK [H, 128, 512]
// as stored, or W_UV [H, 512, 128]),
// bf16 operands, fp32 accumulation, written in fp16.  KDIM = 1024 takes rows
// [c_hi | c_lo] against [W; W]: out = c_hi W + c_lo W in one accumulation.
//
// The product is formed transposed, out^T[col, t] = W[h]^T[col, :] .
// c^T[:, t], so that the latent -- the operand every head shares -- is the
// MFMA's B operand and stays in registers for all the heads of a workgroup:
// wave w holds the latent rows of its MT 32-token tiles (the B fragments of
// every k-step, 256 accumulation registers) from the start, and only the
// weights stream through LDS.  Workgroup: 4 x 32 MT tokens (256 for K = 512,
// 128 for K = 1024) x a group of heads.  The weights of the group's heads run
// through a 6-stage ring of 64-row chunks (16 KB: 64 rows x 256 bytes,
// 16-byte piece c of row k at c ^ 4 (k & 3)), read transposed
// (ds_read_b64_tr_b16) as the A operand, each fragment feeding MT MFMAs.
// The accumulators of a head (32x32 tiles, registers: column 8 (i / 4) +
// 4 (l / 32) + i % 4 of the tile, token l % 32) leave as fp16: a swap
// between lanes l and l + 32 gives each lane 8 consecutive columns, each
// wave stages its own rows in LDS and stores them as whole 256-byte rows
// (stores of 32-byte row pieces straight from the registers took half as
// long again).  Compared with 256-token x 1-head tiles streaming both
// operands, the latent is read from L2 once per head group instead of once
// per head, and the weights once per 256 tokens.
constexpr int PJ_KC = 64;                           // weight rows per chunk
constexpr int PJ_CBYTES = PJ_KC * DV * 2;           // 16 KB
constexpr int PJ_NST = 6;                           // ring stages
constexpr int PJ_CPW = PJ_CBYTES / 1024 / 4;        // copies per wave per chunk: 4
static_assert((PJ_NST - 2) * PJ_CPW <= 63, "the chunks in flight fit the vmcnt counter");

__host__ __device__ constexpr int proj_tokens(int kdim) { return 4 * 32 * (1024 / kdim); }

// WCOL: the weights arrive column-major per head, [H, 128, 512] (W_UK as
// stored, row = output column), instead of [H, 512, 128] (W_UV): a chunk is
// then 128 column rows x 128 bytes (64 k), 16-byte piece p of column row r
// at position p ^ ((r >> 1) & 7), and the A operand is a plain 16-byte read
// (lane: column row l % 32 of the tile, k-piece 2 s + l / 32).
template <int KDIM, bool WCOL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void prefill_proj_kernel(const uint16_t *act, const uint16_t *w, uint16_t *out, int T, int H, int hpw) {
  constexpr int MT = 1024 / KDIM;                  // 32-token tiles per wave: 2 or 1
  constexpr int KS = KDIM / 16;                    // k-steps: 32 or 64
  constexpr int NCH = KDIM / PJ_KC;                // chunks per head: 8 or 16
  constexpr int TM = proj_tokens(KDIM);            // tokens per workgroup
  constexpr int NN = DV / 32;                      // column tiles: 4
  static_assert(MT * KS * 4 == 256, "the latent fragments fill the accumulation registers");
  constexpr int PJ_STORES = 8 * MT;                // whole-row stores per wave and head (4 rows each)
  __shared__ __attribute__((aligned(16))) uint8_t ring[PJ_NST * PJ_CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ostage[TM * DV * 2];   // the head's output rows

  // workgroups are dealt to the 8 XCDs round-robin: consecutive indices per
  // XCD, token tile fastest, so the workgroups of one XCD share a head group
  const int G = gridDim.x;
  const int item = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int tiles = (T + TM - 1) / TM;
  const int t0 = (item % tiles) * TM, h0 = (item / tiles) * hpw;
  const int nh = min(hpw, H - h0);
  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t *const otile = ostage + wave * (32 * MT * DV * 2);

  // the latent fragments: lat[m][ks] = c[t, 16 ks + 8 (l / 32) .. + 7] for
  // token t = t0 + 32 (MT wave + m) + l % 32 (rows past T re-read row T - 1)
  bf16x8 lat[MT][KS];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = min(t0 + 32 * (MT * wave + m) + (l & 31), T - 1);
    const uint16_t *row = act + static_cast<size_t>(t) * KDIM + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) lat[m][ks] = *reinterpret_cast<const bf16x8 *>(row + 16 * ks);
  }

  // chunk g of the group: head h0 + g / NCH, weight rows 64 (g % NCH) % 512;
  // copy k of wave w moves rows 16 w + 4 k .. + 3 (lane: row + l / 16, piece
  // (l % 16) ^ 4 (row & 3), stored at position l % 16); column-major
  // weights: column rows 32 w + 8 k .. + 7 (lane: row + l / 8, piece
  // (l % 8) ^ ((row >> 1) & 7), stored at position l % 8)
  const uint32_t ring_lds = lds_addr(ring);
  uint32_t cpo[PJ_CPW];
#pragma unroll
  for (int k = 0; k < PJ_CPW; ++k) {
    if (WCOL) {
      const int cr = 8 * (PJ_CPW * wave + k) + (l >> 3);
      cpo[k] = static_cast<uint32_t>(cr * (DC * 2) + 16 * ((l & 7) ^ ((cr >> 1) & 7)));
    } else {
      const int kr = 4 * (PJ_CPW * wave + k) + (l >> 4);
      cpo[k] = static_cast<uint32_t>(kr * (DV * 2) + 16 * ((l & 15) ^ (4 * (kr & 3))));
    }
  }
  const int total = nh * NCH;
  auto issue = [&](int g) {
    const int hh = g / NCH, c = g - hh * NCH;
    const uint8_t *src = reinterpret_cast<const uint8_t *>(w + static_cast<size_t>(h0 + hh) * DC * DV) +
                         static_cast<size_t>((c * PJ_KC) % DC) * (WCOL ? 2 : DV * 2);
    const uint32_t st = ring_lds + (g % PJ_NST) * PJ_CBYTES + wave * (PJ_CPW * 1024);
#pragma unroll
    for (int k = 0; k < PJ_CPW; ++k) dma16_s(cpo[k], src, st + k * 1024);
  };

  // transposed weight reads: lane 16 gq + q reads rows 8 (gq >> 1) + q / 4
  // (and + 4) of a k-step, columns 32 n + 16 (gq & 1) + 4 (q & 3) .. + 4
  const int gq = l >> 4, q = l & 15;
  const int krow = 8 * (gq >> 1) + (q >> 2);
  int b_off[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n)
    b_off[n] = krow * (DV * 2) + ((4 * (n ^ (krow & 3)) + 2 * (gq & 1) + ((q & 3) >> 1)) << 4) + (q & 1) * 8;
  // operand j = NN s + n of a chunk: k-step s, column tile n
  constexpr int NJ = (PJ_KC / 16) * NN;            // 16 per chunk
  constexpr int R = 3;                             // operands read ahead of their MFMAs
  // column-major weights: lane l reads column row 32 n + l % 32 (swizzle
  // f = ((l % 32) >> 1) & 7 whatever n), piece 2 s + l / 32 at position
  // (2 s + l / 32) ^ f; one offset per k-step, the column tile an immediate
  int c_off[PJ_KC / 16];
#pragma unroll
  for (int s4 = 0; s4 < PJ_KC / 16; ++s4)
    c_off[s4] = (l & 31) * (PJ_KC * 2) + (((2 * s4 + (l >> 5)) ^ (((l & 31) >> 1) & 7)) << 4);
  auto read_w = [&](const uint8_t *st, int j) {
    if (WCOL) return *reinterpret_cast<const bf16x8 *>(st + c_off[j / NN] + (j % NN) * 32 * (PJ_KC * 2));
    const uint8_t *b0 = st + b_off[j % NN] + 16 * (j / NN) * (DV * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)b0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(b0 + 4 * (DV * 2)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Ring: chunks 0 .. NST - 2 go out first; the barrier that publishes
  // chunk g + 1 sits in chunk g once its last operand read is issued (so the
  // reads of chunk g + 1's first R operands overlap chunk g's last MFMAs),
  // and it sends chunk g + NST - 1 into the slot of chunk g - 1, whose reads
  // every wave finished before the previous barrier.
#pragma unroll
  for (int g = 0; g < PJ_NST - 1; ++g)
    if (g < total) issue(g);
  if (PJ_NST - 2 < total) wait_vmcnt<(PJ_NST - 2) * PJ_CPW>();
  else wait_vmcnt<0>();
  barrier_no_fence();
  bf16x8 nxt[R];
#pragma unroll
  for (int j = 0; j < R; ++j) nxt[j] = read_w(ring, j);

  f32x16 acc[MT][NN];
  for (int hh = 0; hh < nh; ++hh) {
    // the chunks of a head unrolled: every k-step names its latent fragment
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int g = hh * NCH + c;
      const uint8_t *st = ring + (g % PJ_NST) * PJ_CBYTES;
      bf16x8 wv[NJ];
#pragma unroll
      for (int j = 0; j < R; ++j) wv[j] = nxt[j];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j + R < NJ) wv[j + R] = read_w(st, j + R);
        if (j == NJ - R && g + 1 < total) {
          // copies of chunks g + 2 .. g + NST - 2 may stay in flight, and in
          // the first NST - 2 chunks of a head also the previous head's
          // stores, which went out after the copies of chunk g + 1
          if (g + PJ_NST - 2 >= total) wait_vmcnt<0>();
          else if (c < PJ_NST - 2 && hh > 0) wait_vmcnt<(PJ_NST - 3) * PJ_CPW + PJ_STORES>();
          else wait_vmcnt<(PJ_NST - 3) * PJ_CPW>();
          barrier_no_fence();            // chunk g + 1 landed
          if (g + PJ_NST - 1 < total) issue(g + PJ_NST - 1);
          const uint8_t *st1 = ring + ((g + 1) % PJ_NST) * PJ_CBYTES;
#pragma unroll
          for (int jj = 0; jj < R; ++jj) nxt[jj] = read_w(st1, jj);
        }
        const int ks = c * (PJ_KC / 16) + j / NN, n = j % NN;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (ks == 0)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=&v"(acc[m][n]) : "v"(wv[j]), "a"(lat[m][ks]) : "memory");
          else
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+v"(acc[m][n]) : "v"(wv[j]), "a"(lat[m][ks]) : "memory");
        }
      }
    }
    {
      // the last MFMA's result wait states, then the head's tile out: each
      // wave stages its own rows in LDS (fp16, row = token, 16-byte piece x
      // at position x ^ (row & 15)) and stores them as whole rows.  Rows
      // past T hold row T - 1's values (their latent re-read row T - 1) and
      // are stored there again, so every lane stores and the number of
      // stores per head is fixed (the vmcnt waits above count them).
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      const int h = h0 + hh;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int r = 32 * m + (l & 31);
#pragma unroll
        for (int n = 0; n < NN; ++n) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            // registers 8 p .. 8 p + 7: columns 16 p + {0..3, 8..11} (l < 32)
            // or 16 p + {4..7, 12..15}; swap so that lane l < 32 holds
            // 16 p + 0..7 and lane l + 32 16 p + 8..15
            uint32_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = f16_bits(acc[m][n][8 * p + 2 * e]) | (static_cast<uint32_t>(f16_bits(acc[m][n][8 * p + 2 * e + 1])) << 16);
            const auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
            const int x = 4 * n + 2 * p + (l >> 5);
            *reinterpret_cast<u32x4 *>(otile + r * (DV * 2) + ((x ^ (r & 15)) << 4)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
          }
        }
      }
#pragma unroll
      for (int k = 0; k < PJ_STORES; ++k) {
        const int r = 4 * k + (l >> 4), x = l & 15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(otile + r * (DV * 2) + ((x ^ (r & 15)) << 4));
        const int t = min(t0 + 32 * MT * wave + r, T - 1);
        *reinterpret_cast<u32x4 *>(out + (static_cast<size_t>(t) * H + h) * DV + 8 * x) = v;
      }
    }
  }
}

// ---- causal attention, one head and 128 query rows per workgroup.
//
// Four waves of 32 query rows each; keys in blocks of 32, staged in LDS and
// shared by the four waves.  Both products are v_mfma_f32_32x32x16_f16 with
// the query rows as the 32-wide N dimension, the layout of the decode's
// one-wave-per-SIMD kernel:
//   scores   S^T[key, q] = K[key, 0:192] . Q^T over 12 k-steps; the query
//            fragments (48 VGPRs) stay in registers
//   softmax  on the score accumulator: lane (q row l % 32, hb = l / 32) holds
//            keys pi(8 (i / 4) + 4 hb + i % 4) of register i
//   values   O^T[d, q] += V^T[d, key] . P^T[key, q]; registers 8 t .. 8 t + 7
//            of the score accumulator, rounded to fp16, are the B operand of
//            key step t as they stand (keys stored in natural order, the
//            MFMA's K-row m reading key pi(m))
// A block is three XOR-swizzled regions filled by 16-byte global->LDS copies
// (20 per block, five per wave) into a ring of three buffers, two
// blocks in flight while one is used:
//   K latent part  32 rows x 256 B, piece c of row r at c ^ (r & 15)
//   K rotary part  32 rows x 128 B, piece c of row r at c ^ ((r >> 1) & 7)
//   V              32 rows x 256 B, piece c of row r at c ^ 4 ((r >> 2) & 3)
// so the score reads (rows pi(l % 32), whose residues mod 16 differ within
// each 16-lane group) and the transposed value reads (four rows 4 apart,
// four pieces) meet distinct bank quads.
constexpr int FA_Q = 128;                       // query rows per workgroup
constexpr int FA_KB = 32;                       // keys per block
constexpr int FA_KS = (DNOPE + DR) / 16;        // 12 score k-steps
constexpr int FA_KN = FA_KB * DNOPE * 2;        // 8 KB: latent part of K
constexpr int FA_KR = FA_KB * DR * 2;           // 4 KB: rotary part of K
constexpr int FA_VB = FA_KB * DV * 2;           // 8 KB: V
constexpr int FA_BUF = FA_KN + FA_KR + FA_VB;   // 20 KB per block
constexpr int FA_CPW = FA_BUF / 1024 / 4;       // 5 copies per wave per block
constexpr float FA_SLACK = 8.0f;                // lazy rescale margin (log2 units): P <= 2^8 in fp16
constexpr int FA_GRP = 8;                       // (prompt, head) pairs per scheduling group
constexpr int FA_NBUF = 3;                      // block ring (a fourth buffer measured no gain)
static_assert(FA_Q * DV * 2 <= FA_NBUF * FA_BUF, "the output tile is staged in the block ring");
static_assert(FA_NBUF == 3, "the block loop below is unrolled over three buffers");

__device__ __forceinline__ int fa_pi(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m & 3) + 2 * ((m >> 4) & 1) + ((m >> 3) & 1);
}
__device__ __forceinline__ float fa_max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fa_sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void prefill_attention_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[FA_NBUF * FA_BUF];
  // One workgroup per (prompt, head, query tile).  Workgroups are dealt to
  // the 8 XCDs round-robin by id, so id -> (XCD id % 8, position id / 8) is
  // remapped to consecutive items per XCD; the items run in groups of
  // FA_GRP (prompt, head) pairs, each group's tiles longest first (tile
  // major): the tiles that read the same heads' keys and values share one
  // L2 at about the same time, and every group, the last one included, ends
  // on its shortest tiles.
  const int tiles = (a.max_len + FA_Q - 1) / FA_Q;
  const int G = gridDim.x;
  int item = blockIdx.x;
  if ((G & 7) == 0) item = (item & 7) * (G >> 3) + (item >> 3);
  const int grp = item / (FA_GRP * tiles);
  const int gr = item - grp * (FA_GRP * tiles);
  const int gs = min(FA_GRP, a.B * a.H - grp * FA_GRP);       // pairs in this group
  const int tile = tiles - 1 - gr / gs;
  const int bh = grp * FA_GRP + gr % gs;
  const int b = bh / a.H, h = bh % a.H;
  const int t_begin = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - t_begin;
  const int q0 = tile * FA_Q;
  if (q0 >= L) return;
  // query row j of the prompt sits at position P + j and sees the keys at
  // positions 0 .. P + j (key k of the prompt: index k_begin + k)
  const int P = a.prefix_lens ? a.prefix_lens[b] : 0;
  const int k_begin = a.cu_keys[b];
  const int k_last = min(k_begin + P + L, a.T_keys) - 1;
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = l >> 5;
  const int qi = q0 + wave * 32 + (l & 31);                 // this lane's query row
  const int H = a.H;
  const int nkb = (min(P + L, P + q0 + FA_Q) + FA_KB - 1) / FA_KB;

  // block copies (20 per block, 1 KB each): wave w issues K latent copies
  // 2 w, 2 w + 1 (rows 4 j + l / 16, piece l % 16), K rotary copy w (rows
  // 8 w + l / 8, piece l % 8) and V copies 2 w, 2 w + 1 (rows 4 j + l / 16);
  // rows past the prompt re-read its last row (their scores are masked).
  // Per-lane source offsets from the block's first key row (the same for
  // every whole block), wave-uniform block bases.
  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kn_src = reinterpret_cast<const uint8_t *>(a.k_nope) + static_cast<size_t>(h) * (DNOPE * 2);
  const uint8_t *kr_src = reinterpret_cast<const uint8_t *>(a.k_rot);
  const uint8_t *v_src = reinterpret_cast<const uint8_t *>(a.v) + static_cast<size_t>(h) * (DV * 2);
  const uint32_t row_hd = static_cast<uint32_t>(H) * (DNOPE * 2);  // bytes between tokens, per-head arrays
  auto copy_off = [&](int k, int nrow) -> uint32_t {
    if (k < 2) {
      const int r = 4 * (2 * wave + k) + (l >> 4), c = (l & 15) ^ (r & 15);
      return static_cast<uint32_t>(min(r, nrow - 1)) * row_hd + 16 * c;
    }
    if (k == 2) {
      const int r = 8 * wave + (l >> 3), c = (l & 7) ^ ((r >> 1) & 7);
      return static_cast<uint32_t>(min(r, nrow - 1) * (DR * 2) + 16 * c);
    }
    const int r = 4 * (2 * wave + k - 3) + (l >> 4), c = (l & 15) ^ (4 * ((r >> 2) & 3));
    return static_cast<uint32_t>(min(r, nrow - 1)) * row_hd + 16 * c;
  };
  uint32_t cpo[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) cpo[k] = copy_off(k, FA_KB);
  auto issue = [&](int kb, int buf) {
    const uint32_t base = lds0 + buf * FA_BUF;
    const int tok0 = k_begin + kb * FA_KB;
    const uint8_t *kn = kn_src + static_cast<size_t>(tok0) * row_hd;
    const uint8_t *kr = kr_src + static_cast<size_t>(tok0) * (DR * 2);
    const uint8_t *vv = v_src + static_cast<size_t>(tok0) * row_hd;
    const uint32_t dst[5] = {base + (2 * wave) * 1024, base + (2 * wave + 1) * 1024, base + FA_KN + wave * 1024,
                             base + FA_KN + FA_KR + (2 * wave) * 1024, base + FA_KN + FA_KR + (2 * wave + 1) * 1024};
    if (tok0 + FA_KB - 1 <= k_last) {
#pragma unroll
      for (int k = 0; k < 5; ++k) dma16_s(cpo[k], k < 2 ? kn : k == 2 ? kr : vv, dst[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 5; ++k) dma16_s(copy_off(k, k_last - tok0 + 1), k < 2 ? kn : k == 2 ? kr : vv, dst[k]);
    }
  };

  // Query fragments: lane (q row, hb) holds dims 16 ks + 8 hb .. + 8.  The
  // wave's 32 rows are first copied whole into the (still unused) ring with
  // 16-byte global->LDS copies -- 4 q_nope rows (256 B) or 8 rotated rows
  // (128 B) per copy, so every request reads whole rows -- piece c of row r
  // at position c ^ (r & 15) (q_nope) or c ^ ((r >> 1) & 7) (rotated), then read
  // into the MFMA layout.  The bf16 q_nope converts to half (exact inside
  // half's range); the rotated part is already half.
  f16x8 qf[FA_KS];
  {
    constexpr int QN = 32 * DNOPE * 2, QR = 32 * DR * 2;           // 8 KB, 4 KB per wave
    static_assert(4 * (QN + QR) <= FA_NBUF * FA_BUF, "the query rows are staged in the block ring");
    const uint32_t qbase = lds0 + wave * (QN + QR);
    const int r0 = q0 + wave * 32;
    const uint8_t *qn = reinterpret_cast<const uint8_t *>(a.q_nope);
    const uint8_t *qr = reinterpret_cast<const uint8_t *>(a.q_rot);
#pragma unroll
    for (int k = 0; k < QN / 1024; ++k) {
      const int r = 4 * k + (l >> 4), c = (l & 15) ^ (r & 15);
      const size_t th = (static_cast<size_t>(t_begin) + min(r0 + r, L - 1)) * H + h;
      dma16(qn + th * (DNOPE * 2) + 16 * c, qbase + k * 1024);
    }
#pragma unroll
    for (int k = 0; k < QR / 1024; ++k) {
      const int r = 8 * k + (l >> 3), c = (l & 7) ^ ((r >> 1) & 7);
      const size_t th = (static_cast<size_t>(t_begin) + min(r0 + r, L - 1)) * H + h;
      dma16(qr + th * (DR * 2) + 16 * c, qbase + QN + k * 1024);
    }
    wait_vmcnt<0>();           // this wave's rows (each wave reads only its own)
    asm volatile("" ::: "memory");
    const int r = l & 31;
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) {
      if (ks < DNOPE / 16) {
        const int c = 2 * ks + hb;
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(lds + wave * (QN + QR) + r * (DNOPE * 2) + ((c ^ (r & 15)) << 4));
        f16x8 h8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h8[2 * e] = static_cast<_Float16>(__uint_as_float(raw[e] << 16));
          h8[2 * e + 1] = static_cast<_Float16>(__uint_as_float(raw[e] & 0xFFFF0000u));
        }
        qf[ks] = h8;
      } else {
        const int c = 2 * (ks - DNOPE / 16) + hb;
        qf[ks] = *reinterpret_cast<const f16x8 *>(lds + wave * (QN + QR) + QN + r * (DR * 2) + ((c ^ ((r >> 1) & 7)) << 4));
      }
    }
  }
  barrier_lds();               // every wave has its query fragments: the ring takes blocks now
  for (int i = 0; i < FA_NBUF - 1; ++i)
    if (i < nkb) issue(i, i);

  // per-lane read offsets within a block buffer
  const int m = fa_pi(l & 31);
  // K latent piece 2 ks + hb of row m at ((2 ks + hb) ^ (m & 15)): base ^ 32 ks
  const int kn_off = m * (DNOPE * 2) + 16 * ((m & 14) | (hb ^ (m & 1)));
  // K rotary piece 2 (ks - 8) + hb of row m at (... ^ ((m >> 1) & 7)): base ^ 32 (ks - 8)
  const int fr = (m >> 1) & 7;
  const int kr_off = FA_KN + m * (DR * 2) + 16 * ((fr & 6) | (hb ^ (fr & 1)));
  // V (transposed reads): lane supplies row 16 hb + 4 d + 2 t (+ 1 for hi),
  // piece 4 j + csub at (4 (j ^ d) + csub), byte 8 (l & 1)
  const int d = (l & 15) >> 2;
  const int csub = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
  const int v_off = FA_KN + FA_KR + (16 * hb + 4 * d) * (DV * 2) + 16 * csub + 8 * (l & 1);
  // the same per k-step and column tile, kept in registers so that a block
  // read is one LDS instruction with the buffer as its immediate offset
  int k_offs[FA_KS], v_offs[DV / 32];
#pragma unroll
  for (int ks = 0; ks < FA_KS; ++ks)
    k_offs[ks] = ks < DNOPE / 16 ? (kn_off ^ (32 * ks)) : (kr_off ^ (32 * (ks - DNOPE / 16)));
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) v_offs[j] = v_off + 64 * (j ^ d);

  f32x16 o[DV / 32];
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) o[j] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = a.scale_log2;

  // Block kb in buffer kb % FA_NBUF; the loop is unrolled FA_NBUF times so
  // that the buffer is a constant in every LDS address.
  auto block = [&](int kb, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    // block kb has landed once at most the copies of block kb + 1 (5 per
    // wave) are outstanding
    if (kb + 1 < nkb) wait_vmcnt<5>();
    else wait_vmcnt<0>();
    barrier_no_fence();        // block kb visible; every wave is done with block kb - 1
    if (kb + FA_NBUF - 1 < nkb) issue(kb + FA_NBUF - 1, (BUF + FA_NBUF - 1) % FA_NBUF);
    const uint8_t *buf = lds + BUF * FA_BUF;
    // scores: every key fragment of the block is read before the first
    // MFMA, so that the chain of 12 MFMAs waits for the LDS once
    f16x8 kf[FA_KS];
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) kf[ks] = *reinterpret_cast<const f16x8 *>(buf + k_offs[ks]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qf[ks], s, 0, 0, 0);
    // causal mask: key kb * 32 + tok(i) is visible to query qi while <= P + qi
    const int lim = P + qi - kb * FA_KB - 16 * hb;            // visible while tok - 16 hb <= lim
    if (kb * FA_KB + FA_KB - 1 > P + q0 + wave * 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (4 * (i & 3) + 2 * (i >> 3) + ((i >> 2) & 1) > lim) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    const float m_new = fmaxf(m_run, fa_max_xor32(mx) * c);
    float alpha = 1.0f;
    if (m_new > m_run + FA_SLACK) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
    }
    if (kb > 0 && __ballot(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) o[j] *= alpha;
    }
    f16x8 p[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      p[i >> 3][i & 7] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_run)));
    const f16x2 one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      l_run = __builtin_amdgcn_fdot2(f16x2{p[i >> 2][2 * (i & 3)], p[i >> 2][2 * (i & 3) + 1]}, one2, l_run, false);
    // values
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const uint8_t *r0 = buf + v_offs[j] + 2 * t * (DV * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + DV * 2));
        const f16x8 vf = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, p[t], o[j], 0, 0, 0);
      }
    }
  };

  for (int kb = 0; kb < nkb; kb += FA_NBUF) {
    block(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < nkb) block(kb + 1, std::integral_constant<int, 1>{});
    if (kb + 2 < nkb) block(kb + 2, std::integral_constant<int, 2>{});
  }

  // normalise; stage rows (query row = 32 wave + l % 32, 16-byte piece x at
  // position x ^ (row & 15)) and store whole 256-byte rows
  const float inv = 1.0f / fa_sum_xor32(l_run);
  const int row = wave * 32 + (l & 31);
  barrier_no_fence();          // every wave is done with the ring
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[j][4 * q + e] * inv);
      // columns 32 j + 8 q + 4 hb .. + 4: half of 16-byte piece 4 j + q
      const int x = 4 * j + q;
      *reinterpret_cast<bf16x4 *>(lds + row * (DV * 2) + ((x ^ (row & 15)) << 4) + 8 * hb) = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = wave * 32 + 4 * k + (l >> 4), x = l & 15;
    const int qr = q0 + r;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + r * (DV * 2) + ((x ^ (r & 15)) << 4));
    if (qr < L) *reinterpret_cast<u32x4 *>(a.o + ((static_cast<size_t>(t_begin) + qr) * H + h) * DV + 8 * x) = v;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a_in, hipStream_t stream) {
  if (a_in.max_len <= 0 || a_in.T <= 0) return hipSuccess;
  PrefillArgs a = a_in;
  hipError_t e;
  if (a.prefix_lens) {
    // chunks over a cached prefix: key offsets, the prefix rows, then as below
    // with the prompt's latents copied after its prefix's by the RoPE kernel
    a.cu_keys = a.cu_keys_ws;
    a.c_keys = a.c_gather;
    a.c_keys_w = a.kv_fp8 ? 2 * DC : DC;
    prefill_keys_scan_kernel<<<1, 256, 0, stream>>>(a.cu_seqlens, a.prefix_lens, a.cu_keys_ws, a.B);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.max_prefix > 0) {
      prefill_gather_kernel<<<dim3(a.B, (a.max_prefix + ROPE_TOK - 1) / ROPE_TOK), 256, 0, stream>>>(a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  } else {
    a.cu_keys = a.cu_seqlens;
    a.c_keys = a.c;
    a.c_keys_w = DC;
    a.T_keys = a.T;
  }
  prefill_rope_kernel<<<dim3(a.B, (a.max_len + ROPE_TOK - 1) / ROPE_TOK), 256, 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // heads per workgroup: enough workgroups for the 256 compute units, at
  // most 16 heads each
  const int ptiles = (a.T_keys + proj_tokens(a.c_keys_w) - 1) / proj_tokens(a.c_keys_w);
  const int hpw = std::max(1, std::min(16, a.H * ptiles / 256));
  const dim3 pgrid(ptiles * ((a.H + hpw - 1) / hpw));
  if (a.c_keys_w == 2 * DC) {
    prefill_proj_kernel<2 * DC, true><<<pgrid, 256, 0, stream>>>(a.c_keys, a.w_uk, a.k_nope, a.T_keys, a.H, hpw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prefill_proj_kernel<2 * DC, false><<<pgrid, 256, 0, stream>>>(a.c_keys, a.w_uv, a.v, a.T_keys, a.H, hpw);
  } else {
    prefill_proj_kernel<DC, true><<<pgrid, 256, 0, stream>>>(a.c_keys, a.w_uk, a.k_nope, a.T_keys, a.H, hpw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prefill_proj_kernel<DC, false><<<pgrid, 256, 0, stream>>>(a.c_keys, a.w_uv, a.v, a.T_keys, a.H, hpw);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long items = static_cast<long>((a.max_len + FA_Q - 1) / FA_Q) * a.H * a.B;
  if (items > 2147483647L) return hipErrorInvalidValue;
  prefill_attention_kernel<<<dim3(static_cast<unsigned>(items)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
