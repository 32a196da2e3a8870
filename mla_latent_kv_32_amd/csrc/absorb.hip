// Query and value absorption GEMMs (per head, batch as the MFMA M dimension).
//
//   q[b,h,0:512] = q_nope[b,h,0:128] . W_UK[h]      K = 128, N = 512
//   o[b,h,0:128] = o_lat[b,h,0:512]  . W_UV[h]      K = 512, N = 128
//
// The content score q_nope W_UK . c lets the cached latent stand in for the
// key; the value up-projection moves behind the latent-weighted sum (Su, "The
// Ultimate Tug-of-War Between Cache and Performance", MLA Part 1 identity and
// eq:mla-mqa; Riju, "Multi-Head Latent Attention vs GQA vs MQA", "Inside MLA:
// Absorption").  Applied sequentially to the projected query, never through a
// pre-merged matrix (Su, MLA additional notes 1-2).
//
// These are weight-streaming GEMMs (the weights dominate the bytes at decode
// batch sizes).  A workgroup owns one head and NT output columns: the weight
// tile W[h][0:K][n0:n0+NT] is copied into LDS once with 16-byte DMA copies and
// reused by every 32-row batch tile; each wave computes 32 columns with
// v_mfma_f32_32x32x16_bf16, taking the activations (A, K-contiguous) straight
// from global memory and the weight operand (B, K-strided) from LDS with the
// transposed read ds_read_b64_tr_b16.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {
namespace {

// Chunk swizzle of the weight tile: 16-byte chunk c of row k sits at chunk
// position c ^ wsw(k).  The 32 lanes served together by a transposed read
// touch rows k0..k0+3 and 4 consecutive chunks; the swizzle spreads them over
// all 64 banks (row pitch 256 B: XOR bits 2-3 with k & 3; 128 B: bit 2 with
// bit 1 of k, the odd rows already sitting in the other half of the banks).
template <int NT>
__device__ __forceinline__ int wsw(int k) {
  return NT == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

// Weight tile W[h][0:K][n0:n0+NT] -> LDS (row k, position p <- chunk
// p ^ wsw(k) of the row) with 16-byte DMA copies; the caller waits.
template <int K, int N, int NT>
__device__ __forceinline__ void absorb_load_weights(const uint16_t *w, int h, int n0, uint8_t *tile, int wave,
                                                    int lane) {
  constexpr int CPR = NT * 2 / 16;                      // 16-byte chunks per tile row
  constexpr int CHUNKS = K * CPR;
  constexpr int NWAVE = NT / 32;
  constexpr int PER_WAVE = CHUNKS / (64 * NWAVE);       // DMA copies per wave
  static_assert(CHUNKS % (64 * NWAVE) == 0, "tile must split evenly over the waves");
  const uint8_t *wg = reinterpret_cast<const uint8_t *>(w + (static_cast<size_t>(h) * K) * N + n0);
  const uint32_t tile_lds = lds_addr(tile);
#pragma unroll 4
  for (int i = 0; i < PER_WAVE; ++i) {
    const int base = (wave * PER_WAVE + i) * 64;
    const int p = base + lane;
    const int k = p / CPR;
    const int c = (p % CPR) ^ wsw<NT>(k);
    dma16(wg + static_cast<size_t>(k) * N * 2 + c * 16, __builtin_amdgcn_readfirstlane(tile_lds + base * 16));
  }
}

// Activations of batch tile b0 (A operand, K-contiguous): lane (row r, half
// hl) holds act[b0 + r, h, 16 kb + 8 hl .. + 8] for every k-step kb; rows
// past the batch read as zero.
template <int K>
__device__ __forceinline__ void absorb_load_act(const uint16_t *act, int B, int H, int h, int b0, int lane,
                                                u32x4 (&av)[K / 16]) {
  const int r = lane & 31, hl = lane >> 5;
  const bool aval = r < B - b0;
  const uint16_t *ap = act + (static_cast<size_t>(b0 + (aval ? r : 0)) * H + h) * K + hl * 8;
#pragma unroll
  for (int kb = 0; kb < K / 16; ++kb) {
    av[kb] = *reinterpret_cast<const u32x4 *>(ap + kb * 16);
    if (!aval) av[kb] = u32x4{0, 0, 0, 0};
  }
}

// out[b0 + row, h, n0 + 32 wave + col] for one batch tile: 32x32x16 MFMAs
// over the K-steps, the weight operand read transposed from the LDS tile
// (lane 16 g + q reads rows 8 (g >> 1) + q / 4 (+4 for the second read) of
// each 16-row k-step, columns 32 wave + 16 (g & 1) + 4 (q & 3) .. +4).
template <int K, int N, int NT>
__device__ __forceinline__ f32x16 absorb_mfma(const u32x4 (&av)[K / 16], const uint8_t *tile, int wave, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int krow = 8 * (g >> 1) + (q >> 2);
  const int chunk = 4 * wave + 2 * (g & 1) + ((q & 3) >> 1);
  const int boff0 = krow * (NT * 2) + ((chunk ^ wsw<NT>(krow)) << 4) + (q & 1) * 8;
  const int boff1 = (krow + 4) * (NT * 2) + ((chunk ^ wsw<NT>(krow + 4)) << 4) + (q & 1) * 8;
  f32x16 acc = {};
#pragma unroll 8
  for (int kb = 0; kb < K / 16; ++kb) {
    // rows kb*16 + ... : the swizzle depends on k & 3 / (k >> 1) & 1 only, which 16 kb keeps
    const uint8_t *t0 = tile + kb * 16 * (NT * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff1));
    const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[kb]), bv, acc, 0, 0, 0);
  }
  return acc;
}

template <int K, int N, int NT, int OUT_ROW>
__device__ __forceinline__ void absorb_tile(const u32x4 (&av)[K / 16], const uint8_t *tile, uint16_t *out, int B,
                                            int H, int h, int n0, int b0, int wave, int lane) {
  const f32x16 acc = absorb_mfma<K, N, NT>(av, tile, wave, lane);
  // row (batch) b0 + (i/4)*8 + 4*hl + i%4, column n0 + 32 wave + r
  const int r = lane & 31, hl = lane >> 5, rows = B - b0;
  const size_t ld_out = static_cast<size_t>(H) * OUT_ROW;
  uint16_t *op = out + static_cast<size_t>(b0) * ld_out + static_cast<size_t>(h) * OUT_ROW + n0 + wave * 32 + r;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
    if (row < rows) op[row * ld_out] = bf16_bits(to_bf16(acc[i]));
  }
}

// absorb_tile with the output tile (32 batch rows x NT columns, bf16) staged
// through LDS: every thread then stores two whole 16-byte pieces of a row
// instead of sixteen 2-byte values scattered over 16 rows.  `stage` holds
// 32 * NT bf16; the caller separates consecutive uses by a barrier.
template <int K, int N, int NT, int OUT_ROW>
__device__ __forceinline__ void absorb_tile_staged(const u32x4 (&av)[K / 16], const uint8_t *tile, uint16_t *stage,
                                                   uint16_t *out, int B, int H, int h, int n0, int b0, int wave,
                                                   int lane) {
  const f32x16 acc = absorb_mfma<K, N, NT>(av, tile, wave, lane);
  const int r = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
    stage[row * NT + wave * 32 + r] = bf16_bits(to_bf16(acc[i]));
  }
  __syncthreads();
  constexpr int PIECES = NT / 8;                       // 16-byte pieces per row
  const int t = threadIdx.x;                           // NT * 2 threads, 2 pieces each
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = t * 2 + k, row = p / PIECES, c = p % PIECES;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * NT + c * 8);
    if (row < B - b0)
      *reinterpret_cast<u32x4 *>(out + (static_cast<size_t>(b0 + row) * H + h) * OUT_ROW + n0 + c * 8) = v;
  }
}

template <int K, int N, int NT, int OUT_ROW>
__global__ __launch_bounds__(NT * 2) void absorb_kernel(const uint16_t *act, const uint16_t *w, uint16_t *out,
                                                        int B, int H) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[K * NT * 2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * NT;
  const int h = blockIdx.y;
  absorb_load_weights<K, N, NT>(w, h, n0, tile, wave, lane);
  wait_vmcnt<0>();
  __syncthreads();
  if constexpr (K <= 128) {
    for (int b0 = 0; b0 < B; b0 += 32) {
      u32x4 av[K / 16];
      absorb_load_act<K>(act, B, H, h, b0, lane, av);
      absorb_tile<K, N, NT, OUT_ROW>(av, tile, out, B, H, h, n0, b0, wave, lane);
    }
  } else {
    // long K: the activations stream through a ring of 8 k-steps instead of
    // being held whole (K / 16 x 4 registers would not fit beside the rest)
    constexpr int RA = 8;
    const int g = lane >> 4, q = lane & 15;
    const int krow = 8 * (g >> 1) + (q >> 2);
    const int chunk = 4 * wave + 2 * (g & 1) + ((q & 3) >> 1);
    const int boff0 = krow * (NT * 2) + ((chunk ^ wsw<NT>(krow)) << 4) + (q & 1) * 8;
    const int boff1 = (krow + 4) * (NT * 2) + ((chunk ^ wsw<NT>(krow + 4)) << 4) + (q & 1) * 8;
    const int r = lane & 31, hl = lane >> 5;
    for (int b0 = 0; b0 < B; b0 += 32) {
      const bool aval = r < B - b0;
      const uint16_t *ap = act + (static_cast<size_t>(b0 + (aval ? r : 0)) * H + h) * K + hl * 8;
      u32x4 ring[RA];
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) ring[kb] = *reinterpret_cast<const u32x4 *>(ap + kb * 16);
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < K / 16; ++kb) {
        u32x4 av = ring[kb % RA];
        if (kb + RA < K / 16) ring[kb % RA] = *reinterpret_cast<const u32x4 *>(ap + (kb + RA) * 16);
        if (!aval) av = u32x4{0, 0, 0, 0};
        const uint8_t *t0 = tile + kb * 16 * (NT * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff1));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bv, acc, 0, 0, 0);
      }
      const int rows = B - b0;
      const size_t ld_out = static_cast<size_t>(H) * OUT_ROW;
      uint16_t *op = out + static_cast<size_t>(b0) * ld_out + static_cast<size_t>(h) * OUT_ROW + n0 + wave * 32 + r;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
        if (row < rows) op[row * ld_out] = bf16_bits(to_bf16(acc[i]));
      }
    }
  }
}

// The query side of a decode step in one launch: q[:, :, 0:512] =
// q_nope . W_UK (the GEMM of absorb_kernel<128, 512, 128, 576>, grid rows
// 0..H-1: 4 column tiles per head) with the work of rope_append_kernel.
// Workgroup (x, h < H) turns the query pairs of head h for the sequences
// b = x (mod 4) while its weight tile is in flight: the first pair's operands
// (q_pe pair, length, frequency) are requested before the activations and the
// weight copies, and the vector-memory counter completes in order, so the
// angle and the rotation wait for those few loads only, not for the copies.
// The cache rows are appended by extra grid rows h >= H that copy no weights
// (workgroup (x, H + y) takes the sequences b = 4 y + x modulo their count).
// The arithmetic is that of the two separate launches, so the results are
// bit-identical to them.
__global__ __launch_bounds__(256) void query_kernel(const uint16_t *q_nope, const uint16_t *w_uk, RopeAppendArgs ra) {
  constexpr int K = DNOPE, N = DC, NT = 128;
  __shared__ __attribute__((aligned(16))) uint8_t tile[K * NT * 2];
  __shared__ __attribute__((aligned(16))) uint16_t stage[32 * NT];
  __shared__ float cs[DR / 2], sn[DR / 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * NT;
  const int h = blockIdx.y;
  const int B = ra.B, H = ra.H;

  if (h >= H) {
    // cache rows
    const int stride = gridDim.x * (gridDim.y - H);
    for (int b = (h - H) * gridDim.x + blockIdx.x; b < B; b += stride) {
      const int S = ra.seq_lens[b];
      if (S <= 0) continue;
      __syncthreads();   // cs / sn free again
      if (tid < DR / 2) rope_cos_sin(ra, rope_position(S), tid, cs[tid], sn[tid]);
      __syncthreads();
      append_row(ra, b, S, tid, cs, sn);
    }
    return;
  }

  // query rotary pairs: thread (j = tid / 32, pair i = tid % 32), sequences
  // b = x + 4 j + 32 m; the operands of m = 0 go out first
  const int i = tid & 31, bq = blockIdx.x + 4 * (tid >> 5);
  const double w = ra.inv_freq[i];
  uint32_t pr0 = 0;
  int s0 = 0;
  if (bq < B) {
    pr0 = rope_query_load(ra, bq, h, i);
    s0 = ra.seq_lens[bq];
  }
  u32x4 av[K / 16];
  absorb_load_act<K>(q_nope, B, H, h, 0, lane, av);
  absorb_load_weights<K, N, NT>(w_uk, h, n0, tile, wave, lane);
  // keeps the position arithmetic (and with it the wait for the length)
  // behind the copies
  asm volatile("" : "+v"(s0));
  if (bq < B) {
    float c, s;
    rope_cos_sin_at(w, rope_position(s0), c, s);
    rope_query_store(ra, bq, h, i, pr0, c, s);
    for (int b = bq + 32; b < B; b += 32) {
      const uint32_t pr = rope_query_load(ra, b, h, i);
      rope_cos_sin_at(w, rope_position(ra.seq_lens[b]), c, s);
      rope_query_store(ra, b, h, i, pr, c, s);
    }
  }

  wait_vmcnt<0>();
  __syncthreads();
  absorb_tile_staged<K, N, NT, DROW>(av, tile, stage, ra.q, B, H, h, n0, 0, wave, lane);
  for (int b0 = 32; b0 < B; b0 += 32) {
    absorb_load_act<K>(q_nope, B, H, h, b0, lane, av);
    __syncthreads();           // the previous tile's stores have read the stage
    absorb_tile_staged<K, N, NT, DROW>(av, tile, stage, ra.q, B, H, h, n0, b0, wave, lane);
  }
}

// Split-KV merge fused with the value up-projection.  Each workgroup owns one
// head h and keeps W_UV[h] (512 x 128 bf16, 128 KB) in LDS; the batch is cut
// into tiles of 16 sequences, and the tiles of a head are dealt out to
// COMBINE_TILE_SLOTS(B) workgroups (two for 17..32 sequences, so a 32-sequence
// batch fills 256 compute units).  Workgroups that share a head are numbered
// so that they run on the same XCD and the second W_UV read can hit its L2.
//
// Merge: wave w builds tile rows w and w + 8.  Lanes 32 j .. 32 j + 31 hold
// row j's chunk log-sum-exps (one pass for up to 32 chunks, loaded together
// with the sequence lengths), the row maximum is a 32-lane shuffle reduction,
// and the weights reach the accumulation as wave-uniform values; all partial
// rows of a batch of 8 chunks are loaded together, the first batch before
// the lengths and lse values have arrived and before the W_UV copies, so the
// merge does not wait behind them.  Each row sums its chunks in chunk order
// in batches of 8 with the arithmetic of combine_kernel, so o_latent and lse
// equal the separate merge bit for bit.  The merged bf16 rows go to an LDS
// tile (16-byte chunk c of row r at position c ^ (r & 15)) whose rows 16..31
// stay zero, and waves 0-3 multiply it by W_UV[h] with 32x32x16 MFMAs, 32
// output columns each (rows 16..31 of the product are discarded).
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void combine_absorb_out_kernel(CombineOutArgs a) {
  constexpr int K = DC, N = DV, NT = 128;
  constexpr int NWAVE = 8, ROWS = 16, RPW = ROWS / NWAVE;   // 2 tile rows per wave
  constexpr int LPR = 64 / RPW;                             // 32 lanes per row in the lse phase
  constexpr int VB = 8;                                     // chunks per load batch
  constexpr int CPR = NT * 2 / 16;                          // 16-byte chunks per W row
  constexpr int PER_WAVE = K * CPR / (64 * NWAVE);          // 16 DMA copies per wave
  __shared__ __attribute__((aligned(16))) uint8_t wt[K * NT * 2];     // 128 KB
  __shared__ __attribute__((aligned(16))) uint8_t at[32 * DC * 2];    //  32 KB

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slots = a.tile_slots;
  const int G = gridDim.x;
  const int L = blockIdx.x;
  const int item = (G & 7) == 0 ? (L & 7) * (G >> 3) + (L >> 3) : L;
  const int h = item / slots, slot = item % slots;

  // W_UV[h] -> LDS (row k, position p <- chunk p ^ wsw(k) of the row); issued
  // after the first tile's merge loads, so that those do not queue behind it
  const uint8_t *wg = reinterpret_cast<const uint8_t *>(a.w_uv + static_cast<size_t>(h) * K * N);
  const uint32_t wt_lds = lds_addr(wt);
  auto load_w = [&]() {
#pragma unroll 4
    for (int i = 0; i < PER_WAVE; ++i) {
      const int base = (wave * PER_WAVE + i) * 64;
      const int p = base + lane;
      const int k = p / CPR;
      const int c = (p % CPR) ^ wsw<NT>(k);
      dma16(wg + static_cast<size_t>(k) * N * 2 + c * 16, __builtin_amdgcn_readfirstlane(wt_lds + base * 16));
    }
  };
  // rows 16..31 of the A tile: zero for the whole kernel
  reinterpret_cast<u32x4 *>(at + ROWS * DC * 2)[threadIdx.x] = u32x4{0, 0, 0, 0};
  reinterpret_cast<u32x4 *>(at + ROWS * DC * 2)[threadIdx.x + 512] = u32x4{0, 0, 0, 0};

  // transposed B reads (waves 0-3), as in absorb_kernel
  const int g = lane >> 4, q = lane & 15;
  const int krow = 8 * (g >> 1) + (q >> 2);
  const int chunk = 4 * (wave & 3) + 2 * (g & 1) + ((q & 3) >> 1);
  const int boff0 = krow * (NT * 2) + ((chunk ^ wsw<NT>(krow)) << 4) + (q & 1) * 8;
  const int boff1 = (krow + 4) * (NT * 2) + ((chunk ^ wsw<NT>(krow + 4)) << 4) + (q & 1) * 8;
  const int r = lane & 31, hl = lane >> 5;
  const size_t stride = static_cast<size_t>(a.H);
  const int jl = lane / LPR, kl = lane % LPR;   // lse phase: row jl of this wave, chunk slot kl
  bool first = true;

  for (int b0 = slot * ROWS; b0 < a.B; b0 += slots * ROWS) {
    // ---- chunk counts and row maxima, lane-parallel.  The first LPR chunk
    // lse values are loaded alongside the sequence lengths (every chunk slot
    // below n_splits lies inside the workspace) and masked afterwards.
    const int bl = b0 + wave + NWAVE * jl;
    const float *lp_l = a.lse_part + static_cast<size_t>(bl < a.B ? bl : 0) * a.n_splits * stride + h;
    const float l0 = kl < a.n_splits ? lp_l[kl * stride] : -INFINITY;
    int nv_l = 0;
    if (bl < a.B) nv_l = max(0, (a.seq_lens[bl] + a.split_tokens - 1) / a.split_tokens);
    const uint16_t *op[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int b = b0 + wave + NWAVE * j;
      op[j] = a.o_part + (static_cast<size_t>(b < a.B ? b : 0) * a.n_splits * stride + h) * DC + lane * 8;
    }
    // The first batch of chunks of every row is requested before the lengths
    // are known (the chunks lie inside the workspace; those past a row's
    // count are zeroed after the load), then the W_UV tile on the first pass.
    u32x4 v0[RPW][VB];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int k = 0; k < VB; ++k)
        v0[j][k] = k < a.n_splits ? *reinterpret_cast<const u32x4 *>(op[j] + k * stride * DC) : u32x4{0, 0, 0, 0};
    if (first) load_w();
    float mx = kl < nv_l ? l0 : -INFINITY;
    for (int c = kl + LPR; c < nv_l; c += LPR) mx = fmaxf(mx, lp_l[c * stride]);
#pragma unroll
    for (int sh = 1; sh < LPR; sh <<= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
    int nv[RPW];
    float Lm[RPW];
    int ncmax = 0;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      nv[j] = __builtin_amdgcn_readlane(nv_l, LPR * j);
      Lm[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), LPR * j));
      ncmax = max(ncmax, nv[j]);
    }

    // ---- weighted sums in the order of combine_kernel: VB chunks of every
    // row per batch, each range of combine_range(n_splits) chunks summed in
    // chunk order from zero (accr, zr), the range sums added in range order
    // (acc, z) -- so the sums are the same
    float acc[RPW][8] = {};
    float z[RPW] = {};
    float accr[RPW][8] = {};
    float zr[RPW] = {};
    const int R = combine_range(a.n_splits);
    // add the range that started at chunk c (rows that have chunks there)
    auto flush = [&](int c) {
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        if (c < nv[j]) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] += accr[j][e];
          z[j] += zr[j];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) accr[j][e] = 0.f;
        zr[j] = 0.f;
      }
    };
    // lane LPR j + k: weight of chunk cb + k of row j
    float w_l = kl < nv_l ? expf(l0 - mx) : 0.f;
    auto accumulate = [&](const u32x4 (&v)[RPW][VB], int part) {
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
#pragma unroll
        for (int k = 0; k < VB; ++k) {
          const float wk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), LPR * j + part + k));
          zr[j] += wk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            accr[j][2 * e] += wk * __uint_as_float(v[j][k][e] << 16);
            accr[j][2 * e + 1] += wk * __uint_as_float(v[j][k][e] & 0xFFFF0000u);
          }
        }
      }
    };
    if (ncmax > 0) {
#pragma unroll
      for (int j = 0; j < RPW; ++j)
#pragma unroll
        for (int k = 0; k < VB; ++k)
          if (k >= nv[j]) v0[j][k] = u32x4{0, 0, 0, 0};
      accumulate(v0, 0);
    }
    for (int c0 = VB; c0 < ncmax; c0 += VB) {
      if (c0 % R == 0) flush(c0 - R);
      const int part = c0 & (LPR - 1);
      if (part == 0) {
        w_l = 0.f;
        if (c0 + kl < nv_l) w_l = expf(lp_l[(c0 + kl) * stride] - mx);
      }
      u32x4 v[RPW][VB];
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
#pragma unroll
        for (int k = 0; k < VB; ++k) {
          if (c0 + k < nv[j]) v[j][k] = *reinterpret_cast<const u32x4 *>(op[j] + (c0 + k) * stride * DC);
          else v[j][k] = u32x4{0, 0, 0, 0};
        }
      }
      accumulate(v, part);
    }
    if (ncmax > 0) flush((ncmax - 1) / R * R);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int row = wave + NWAVE * j;
      const int b = b0 + row;
      bf16x8 out = {};
      if (nv[j] > 0) {
        const float inv = 1.0f / z[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = to_bf16(acc[j][e] * inv);
      }
      if (b < a.B) {
        if (lane == 0 && a.lse)
          a.lse[static_cast<size_t>(b) * a.H + h] = nv[j] > 0 ? Lm[j] + logf(z[j]) : -INFINITY;
        if (a.o_latent)
          *reinterpret_cast<bf16x8 *>(a.o_latent + (static_cast<size_t>(b) * a.H + h) * DC + lane * 8) = out;
      }
      *reinterpret_cast<bf16x8 *>(at + row * DC * 2 + ((lane ^ (row & 15)) << 4)) = out;
    }
    if (first) wait_vmcnt<0>();         // this wave's W tile copies landed
    first = false;
    __syncthreads();

    // ---- o[b0 + row, h, 32 wave + r] = tile[row, :] . W_UV[h][:, 32 wave + r]
    if (wave < 4) {
      f32x16 d = {};
#pragma unroll 8
      for (int kb = 0; kb < K / 16; ++kb) {
        const int ck = 2 * kb + hl;                         // 16-byte chunk of tile row r
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(at + r * DC * 2 + ((ck ^ (r & 15)) << 4));
        const uint8_t *t0 = wt + kb * 16 * (NT * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff1));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, d, 0, 0, 0);
      }
      const int rows = min(ROWS, a.B - b0);
      const size_t ld_out = static_cast<size_t>(a.H) * DV;
      uint16_t *opo = a.o + static_cast<size_t>(b0) * ld_out + static_cast<size_t>(h) * DV + wave * 32 + r;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
        if (row < rows) opo[row * ld_out] = bf16_bits(to_bf16(d[i]));
      }
    }
    __syncthreads();                    // the tile is rebuilt for the next rows
  }
  // (every workgroup has at least one tile: slot < tiles)
}

}  // namespace

hipError_t launch_combine_absorb_out(const CombineOutArgs &args, hipStream_t stream) {
  // 16-sequence tiles dealt to enough workgroups per head to reach 256
  // workgroups, but never more than there are tiles
  CombineOutArgs a = args;
  const int tiles = (a.B + 15) / 16;
  a.tile_slots = std::max(1, std::min(tiles, (256 + a.H - 1) / a.H));
  combine_absorb_out_kernel<<<dim3(a.H * a.tile_slots), 512, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_absorb_q(const uint16_t *q_nope, const uint16_t *w_uk, uint16_t *q, int B, int H,
                           hipStream_t stream) {
  absorb_kernel<DNOPE, DC, 128, DROW><<<dim3(DC / 128, H), 256, 0, stream>>>(q_nope, w_uk, q, B, H);
  return hipGetLastError();
}

hipError_t launch_query(const uint16_t *q_nope, const uint16_t *w_uk, const RopeAppendArgs &ra, hipStream_t stream) {
  // H rows of 4 GEMM workgroups, then 1..8 rows of 4 append workgroups
  const int append_rows = std::max(1, std::min(8, (ra.B + 3) / 4));
  query_kernel<<<dim3(DC / 128, ra.H + append_rows), 256, 0, stream>>>(q_nope, w_uk, ra);
  return hipGetLastError();
}

hipError_t launch_absorb_out(const uint16_t *o_latent, const uint16_t *w_uv, uint16_t *o, int B, int H,
                             hipStream_t stream) {
  absorb_kernel<DC, DV, 64, DV><<<dim3(DV / 64, H), 128, 0, stream>>>(o_latent, w_uv, o, B, H);
  return hipGetLastError();
}

}  // namespace mla
