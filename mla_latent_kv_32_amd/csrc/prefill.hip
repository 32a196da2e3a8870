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
// Launches: RoPE + cache rows; W_UK transposed per head; the two
// up-projections; causal attention.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {
namespace {

// ---- RoPE of the prompt tokens and their cache rows.  Workgroup (b, y)
// handles positions 8 y .. 8 y + 7 of prompt b: the angles of all eight
// tokens first (one thread per token and pair), then the query pairs of
// every head in 16-byte pieces (to the workspace), the shared rotary key (to
// the workspace, for the attention) and the cache rows.
constexpr int ROPE_TOK = 8;

__global__ __launch_bounds__(256) void prefill_rope_kernel(PrefillArgs a) {
  __shared__ float cs[ROPE_TOK][DR / 2], sn[ROPE_TOK][DR / 2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t_begin = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - t_begin;
  const int p0 = blockIdx.y * ROPE_TOK;
  if (p0 >= L) return;
  const int ntok = min(ROPE_TOK, L - p0);
  {
    const int j = tid / (DR / 2), i = tid % (DR / 2);
    if (j < ntok) rope_cos_sin(a.inv_freq, p0 + j, i, cs[j][i], sn[j][i]);
  }
  __syncthreads();
  const int H = a.H;
  constexpr int VEC = DR / 8;                          // 16-byte pieces of a rotary part
  for (int idx = tid; idx < ntok * H * VEC; idx += blockDim.x) {
    const int j = idx / (H * VEC), rem = idx % (H * VEC), h = rem / VEC, v = rem % VEC;
    const size_t off = ((static_cast<size_t>(t_begin) + p0 + j) * H + h) * DR + 8 * v;
    u32x4 pr = *reinterpret_cast<const u32x4 *>(a.q_pe + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = rope_rotate_pair(pr[e], cs[j][4 * v + e], sn[j][4 * v + e]);
    *reinterpret_cast<u32x4 *>(a.q_rot + off) = pr;
  }
  if (tid < ntok * VEC) {
    const int j = tid / VEC, v = tid % VEC;
    const size_t off = (static_cast<size_t>(t_begin) + p0 + j) * DR + 8 * v;
    u32x4 pr = *reinterpret_cast<const u32x4 *>(a.k_pe + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = rope_rotate_pair(pr[e], cs[j][4 * v + e], sn[j][4 * v + e]);
    *reinterpret_cast<u32x4 *>(a.k_rot + off) = pr;
  }
  for (int j = 0; j < ntok; ++j) {
    const int pos = p0 + j;
    const size_t t = static_cast<size_t>(t_begin) + pos;
    const int page = a.block_table[static_cast<size_t>(b) * a.max_blocks + pos / PAGE];
    store_cache_row(a.cache, a.kv_fp8, static_cast<size_t>(page) * PAGE + pos % PAGE, a.c + t * DC,
                    a.k_pe + t * DR, tid, cs[j], sn[j]);
  }
}

// ---- W_UK[h] [128, 512] -> W_UK[h]^T [512, 128] (32 x 32 tiles through LDS)
__global__ __launch_bounds__(256) void transpose_wuk_kernel(const uint16_t *w, uint16_t *wt) {
  __shared__ uint16_t tile[32][33];
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * 32, h = blockIdx.z;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;           // 32 x 8
  const uint16_t *src = w + static_cast<size_t>(h) * DNOPE * DC;
  uint16_t *dst = wt + static_cast<size_t>(h) * DC * DNOPE;
  for (int r = ty; r < 32; r += 8) tile[r][tx] = src[static_cast<size_t>(n0 + r) * DC + k0 + tx];
  __syncthreads();
  for (int r = ty; r < 32; r += 8) dst[static_cast<size_t>(k0 + r) * DNOPE + n0 + tx] = tile[tx][r];
}

// ---- per-head up-projection of the shared latent: out[t, h, :] =
// c[t, :] . W[h] (K = 512, N = 128; W = W_UK^T or W_UV, both [H, 512, 128]).
//
// Workgroup: 256 tokens x one head; wave w owns tokens 64 w .. 64 w + 63 (two
// 32-row tiles) and all four 32-column tiles, so every weight fragment read
// from LDS feeds two MFMAs.  K runs in chunks of 32 through a 3-stage LDS
// ring fed by 16-byte global->LDS copies (two chunks in flight while one is
// multiplied).  A chunk: 256 rows x 64 bytes, 16-byte piece c of row r at
// position c ^ ((r >> 2) & 3), so a read of one piece of 16 consecutive rows
// meets 16 bank quads.  B chunk: 32 rows x 256 bytes, piece c of row k at
// c ^ 4 (k & 3), read transposed (ds_read_b64_tr_b16) as in the absorption
// GEMMs.  The output tile goes through the ring to whole-row stores.
constexpr int PJ_TM = 256;                      // tokens per workgroup
constexpr int PJ_MT = PJ_TM / 4 / 32;           // 32-row tiles per wave: 2
constexpr int PJ_KC = 32;                       // K per chunk
constexpr int PJ_NCH = DC / PJ_KC;              // 16 chunks
constexpr int PJ_ABYTES = PJ_TM * PJ_KC * 2;    // 16 KB
constexpr int PJ_BBYTES = PJ_KC * DV * 2;       // 8 KB
constexpr int PJ_STAGE = PJ_ABYTES + PJ_BBYTES;
constexpr int PJ_ACOPIES = PJ_ABYTES / 1024;    // 16 one-KB copies of A per chunk
constexpr int PJ_CPW = PJ_STAGE / 1024 / 4;     // copies per wave per chunk: 6
static_assert(PJ_STAGE % 4096 == 0, "a chunk splits evenly over the four waves");
static_assert(PJ_TM * DV * 2 <= 3 * PJ_STAGE, "the output tile is staged in the ring");

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void prefill_proj_kernel(const uint16_t *act, const uint16_t *w, uint16_t *out, int T, int H) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[3 * PJ_STAGE];
  const int h = blockIdx.y, t0 = blockIdx.x * PJ_TM;
  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t *wh = reinterpret_cast<const uint8_t *>(w + static_cast<size_t>(h) * DC * DV);
  const uint32_t ring_lds = lds_addr(ring);
  // copy j (0..23) of a chunk: j < 16 -> A rows 16 j .. 16 j + 15; else B
  // rows 4 (j - 16) .. + 3 (wave-uniform: j = 6 wave + k)
  auto issue = [&](int ch) {
    const uint32_t st = ring_lds + (ch % 3) * PJ_STAGE;
#pragma unroll
    for (int k = 0; k < PJ_CPW; ++k) {
      const int j = wave * PJ_CPW + k;
      if (j < PJ_ACOPIES) {
        const int r = 16 * j + (l >> 2), pos = l & 3;
        const int c = pos ^ ((r >> 2) & 3);
        const size_t t = static_cast<size_t>(min(t0 + r, T - 1));
        dma16(reinterpret_cast<const uint8_t *>(act) + t * (DC * 2) + ch * (PJ_KC * 2) + 16 * c,
              __builtin_amdgcn_readfirstlane(st + j * 1024));
      } else {
        const int kr = 4 * (j - PJ_ACOPIES) + (l >> 4), pos = l & 15;
        const int c = pos ^ (4 * (kr & 3));
        dma16(wh + static_cast<size_t>(ch * PJ_KC + kr) * (DV * 2) + 16 * c,
              __builtin_amdgcn_readfirstlane(st + PJ_ABYTES + (j - PJ_ACOPIES) * 1024));
      }
    }
  };
  f32x16 acc[PJ_MT][DV / 32];
#pragma unroll
  for (int m = 0; m < PJ_MT; ++m)
#pragma unroll
    for (int n = 0; n < DV / 32; ++n) acc[m][n] = f32x16{};
  // A read of tile m: row 64 wave + 32 m + l % 32, piece 2 s + l / 32 (k-step s of the chunk)
  const int ar0 = 32 * PJ_MT * wave + (l & 31);
  // B reads (transposed): lane 16 g + q reads rows 8 (g >> 1) + q / 4 (+ 4) of
  // a k-step, columns 32 n + 16 (g & 1) + 4 (q & 3) .. + 4
  const int g = l >> 4, q = l & 15;
  const int krow = 8 * (g >> 1) + (q >> 2);
  issue(0);
  issue(1);
  for (int ch = 0; ch < PJ_NCH; ++ch) {
    if (ch + 1 < PJ_NCH) wait_vmcnt<PJ_CPW>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    if (ch + 2 < PJ_NCH) issue(ch + 2);
    const uint8_t *st = ring + (ch % 3) * PJ_STAGE;
#pragma unroll
    for (int s = 0; s < PJ_KC / 16; ++s) {
      const int piece = 2 * s + (l >> 5);
      bf16x8 av[PJ_MT];
#pragma unroll
      for (int m = 0; m < PJ_MT; ++m) {
        const int ar = ar0 + 32 * m;
        av[m] = *reinterpret_cast<const bf16x8 *>(st + ar * (PJ_KC * 2) + ((piece ^ ((ar >> 2) & 3)) << 4));
      }
#pragma unroll
      for (int n = 0; n < DV / 32; ++n) {
        const int chunk = 4 * n + 2 * (g & 1) + ((q & 3) >> 1);
        const int k0 = 16 * s + krow, k1 = k0 + 4;
        const uint8_t *b0 = st + PJ_ABYTES + k0 * (DV * 2) + ((chunk ^ (4 * (k0 & 3))) << 4) + (q & 1) * 8;
        const uint8_t *b1 = st + PJ_ABYTES + k1 * (DV * 2) + ((chunk ^ (4 * (k1 & 3))) << 4) + (q & 1) * 8;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)b0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)b1);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int m = 0; m < PJ_MT; ++m) acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bv, acc[m][n], 0, 0, 0);
      }
    }
  }
  // stage: row = token, 16-byte piece x at position x ^ (row & 15); then whole rows
  __syncthreads();
  const int hb = l >> 5, r = l & 31;
#pragma unroll
  for (int m = 0; m < PJ_MT; ++m)
#pragma unroll
    for (int n = 0; n < DV / 32; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = ar0 - (l & 31) + 32 * m + (i >> 2) * 8 + hb * 4 + (i & 3), col = 32 * n + r;
        *reinterpret_cast<uint16_t *>(ring + row * (DV * 2) + (((col >> 3) ^ (row & 15)) << 4) + 2 * (col & 7)) =
            bf16_bits(to_bf16(acc[m][n][i]));
      }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PJ_TM * 16 / 256; ++k) {
    const int p = threadIdx.x + 256 * k, row = p >> 4, x = p & 15;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ring + row * (DV * 2) + ((x ^ (row & 15)) << 4));
    if (t0 + row < T)
      *reinterpret_cast<u32x4 *>(out + (static_cast<size_t>(t0 + row) * H + h) * DV + 8 * x) = v;
  }
}

// ---- causal attention, one head and 128 query rows per workgroup.
//
// Four waves of 32 query rows each; keys in blocks of 32, staged in LDS and
// shared by the four waves.  Both products are v_mfma_f32_32x32x16_bf16 with
// the query rows as the 32-wide N dimension, the layout of the decode's
// one-wave-per-SIMD kernel:
//   scores   S^T[key, q] = K[key, 0:192] . Q^T over 12 k-steps; the query
//            fragments (48 VGPRs) stay in registers
//   softmax  on the score accumulator: lane (q row l % 32, hb = l / 32) holds
//            keys pi(8 (i / 4) + 4 hb + i % 4) of register i
//   values   O^T[d, q] += V^T[d, key] . P^T[key, q]; registers 8 t .. 8 t + 7
//            of the score accumulator, rounded to bf16, are the B operand of
//            key step t as they stand (keys stored in natural order, the
//            MFMA's K-row m reading key pi(m))
// A block is three XOR-swizzled regions filled by 16-byte global->LDS copies
// (20 per block, five per wave) into a ring of three buffers, two blocks in
// flight while one is used:
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
constexpr float FA_SLACK = 16.0f;               // lazy rescale margin (log2 units)
static_assert(FA_Q * DV * 2 <= 3 * FA_BUF, "the output tile is staged in the block ring");

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
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * FA_BUF];
  // One workgroup per (prompt, head, query tile), the tiles of a (prompt,
  // head) numbered consecutively, longest first; workgroups are dealt to the
  // 8 XCDs round-robin by id, so id -> (XCD id % 8, position id / 8) is
  // remapped to consecutive items per XCD: the tiles that read the same
  // head's keys and values share one L2.
  const int tiles = (a.max_len + FA_Q - 1) / FA_Q;
  const int G = gridDim.x;
  int item = blockIdx.x;
  if ((G & 7) == 0) item = (item & 7) * (G >> 3) + (item >> 3);
  const int tile = tiles - 1 - item % tiles;
  const int bh = item / tiles;
  const int b = bh / a.H, h = bh % a.H;
  const int t_begin = a.cu_seqlens[b];
  const int L = a.cu_seqlens[b + 1] - t_begin;
  const int q0 = tile * FA_Q;
  if (q0 >= L) return;
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = l >> 5;
  const int qi = q0 + wave * 32 + (l & 31);                 // this lane's query row (position)
  const int H = a.H;
  const int nkb = (min(L, q0 + FA_Q) + FA_KB - 1) / FA_KB;

  // block copies (20 per block, 1 KB each): wave w issues K latent copies
  // 2 w, 2 w + 1 (rows 4 j + l / 16, piece l % 16), K rotary copy w (rows
  // 8 w + l / 8, piece l % 8) and V copies 2 w, 2 w + 1 (rows 4 j + l / 16);
  // rows past the prompt re-read its last row (their scores are masked).
  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kn_src = reinterpret_cast<const uint8_t *>(a.k_nope) + static_cast<size_t>(h) * (DNOPE * 2);
  const uint8_t *kr_src = reinterpret_cast<const uint8_t *>(a.k_rot);
  const uint8_t *v_src = reinterpret_cast<const uint8_t *>(a.v) + static_cast<size_t>(h) * (DV * 2);
  const size_t row_hd = static_cast<size_t>(H) * (DNOPE * 2);    // bytes between tokens, per-head arrays
  auto issue = [&](int kb) {
    const uint32_t base = lds0 + (kb % 3) * FA_BUF;
    const int tok0 = t_begin + kb * FA_KB, last = t_begin + L - 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 2 * wave + k, r = 4 * j + (l >> 4), c = (l & 15) ^ (r & 15);
      const size_t t = static_cast<size_t>(min(tok0 + r, last));
      dma16(kn_src + t * row_hd + 16 * c, __builtin_amdgcn_readfirstlane(base + j * 1024));
    }
    {
      const int r = 8 * wave + (l >> 3), c = (l & 7) ^ ((r >> 1) & 7);
      const size_t t = static_cast<size_t>(min(tok0 + r, last));
      dma16(kr_src + t * (DR * 2) + 16 * c, __builtin_amdgcn_readfirstlane(base + FA_KN + wave * 1024));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 2 * wave + k, r = 4 * j + (l >> 4), c = (l & 15) ^ (4 * ((r >> 2) & 3));
      const size_t t = static_cast<size_t>(min(tok0 + r, last));
      dma16(v_src + t * row_hd + 16 * c, __builtin_amdgcn_readfirstlane(base + FA_KN + FA_KR + j * 1024));
    }
  };

  // query fragments: lane (q row, hb) holds dims 16 ks + 8 hb .. + 8
  bf16x8 qf[FA_KS];
  {
    const size_t th = (static_cast<size_t>(t_begin) + min(qi, L - 1)) * H + h;
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) {
      const uint16_t *src = ks < DNOPE / 16 ? a.q_nope + th * DNOPE + 16 * ks + 8 * hb
                                            : a.q_rot + th * DR + 16 * (ks - DNOPE / 16) + 8 * hb;
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src));
    }
    // Wait for the query here, before any block copy is issued: the
    // compiler does not see the copies (inline asm) and would otherwise
    // place its waits for the query inside the loop, where they also wait
    // for the copies of the blocks ahead.
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

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

  f32x16 o[DV / 32];
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) o[j] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = a.scale_log2;

  issue(0);
  if (nkb > 1) issue(1);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) wait_vmcnt<FA_CPW>();
    else wait_vmcnt<0>();
    barrier_no_fence();        // block kb visible; every wave is done with block kb - 1
    if (kb + 2 < nkb) issue(kb + 2);
    const uint8_t *buf = lds + (kb % 3) * FA_BUF;
    // scores
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < FA_KS; ++ks) {
      const int off = ks < DNOPE / 16 ? (kn_off ^ (32 * ks)) : (kr_off ^ (32 * (ks - DNOPE / 16)));
      const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(buf + off);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr, qf[ks], s, 0, 0, 0);
    }
    // causal mask: key kb * 32 + tok(i) is visible to query qi while <= qi
    const int lim = qi - kb * FA_KB - 16 * hb;                // visible while tok - 16 hb <= lim
    if (kb * FA_KB + FA_KB - 1 > q0 + wave * 32) {
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
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) o[j] *= alpha;
    }
    bf16x8 p[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i >> 3][i & 7] = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_run)));
    const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[i >> 2][2 * (i & 3)], p[i >> 2][2 * (i & 3) + 1]}, one2,
                                              l_run, false);
    // values
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const uint8_t *r0 = buf + v_off + 2 * t * (DV * 2) + 64 * (j ^ d);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)r0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + DV * 2));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[t], o[j], 0, 0, 0);
      }
    }
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

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  if (a.max_len <= 0 || a.T <= 0) return hipSuccess;
  prefill_rope_kernel<<<dim3(a.B, (a.max_len + ROPE_TOK - 1) / ROPE_TOK), 256, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  transpose_wuk_kernel<<<dim3(DC / 32, DNOPE / 32, a.H), 256, 0, stream>>>(a.w_uk, a.w_ukt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 pgrid((a.T + PJ_TM - 1) / PJ_TM, a.H);
  prefill_proj_kernel<<<pgrid, 256, 0, stream>>>(a.c, a.w_ukt, a.k_nope, a.T, a.H);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prefill_proj_kernel<<<pgrid, 256, 0, stream>>>(a.c, a.w_uv, a.v, a.T, a.H);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long items = static_cast<long>((a.max_len + FA_Q - 1) / FA_Q) * a.H * a.B;
  if (items > 2147483647L) return hipErrorInvalidValue;
  prefill_attention_kernel<<<dim3(static_cast<unsigned>(items)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
