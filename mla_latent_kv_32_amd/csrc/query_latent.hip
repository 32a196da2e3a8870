// The decode query from the low-rank query latent, in one launch.
//
//   q_h[b]            = c'[b] . W_UQ[:, 192 h : 192 h + 192]     K = 1536, N = 192
//   q[b, h, 0:512]    = q_h[b, 0:128] . W_UK[h]                  K = 128,  N = 512
//   q[b, h, 512:576]  = RoPE(q_h[b, 128:192], S_b - 1)
//
// Queries pass through their own low-rank latent c' (Su, "The Ultimate
// Tug-of-War Between Cache and Performance", MLA Part 3; Riju, "Multi-Head
// Latent Attention vs GQA vs MQA", "Query compression is separate"), and the
// up-projection and W_UK are applied one after the other, never through a
// merged matrix (Su, MLA additional notes 1-2).  W_UQ's 192 output columns of
// head h are [nope | rope], head-major.
//
// A workgroup owns one head and 64 sequences.  W_UQ's 590 KB for the head
// stream through a four-stage LDS ring (three chunks in flight) in chunks of 64 rows (16-byte DMA
// copies, the sequences' latents alongside), 32x32x16 bf16 MFMAs with the
// sequences as M; the nope columns then go to LDS as two bf16 terms, W_UK[h]
// (128 KB) follows into LDS, and the second product runs there.  The rotary columns
// are turned in fp32 straight from the accumulators (the pair partner is the
// neighbouring lane) with cos/sin of the sequences' positions formed in fp64
// at the start.  Extra grid rows append the new tokens' cache rows, as in the
// other query kernels.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {
namespace {

constexpr int DQ = MLA_D_Q;                // 1536
constexpr int QH = DNOPE + DR;             // 192 columns of W_UQ per head
constexpr int MT = 64;                     // sequences per workgroup
constexpr int KC = 64;                     // W_UQ rows per streamed chunk
constexpr int NCH = DQ / KC;               // 24 chunks
constexpr int WROW = QH * 2;               // 384 bytes of a chunk row
constexpr int WCH = KC * WROW;             // 24,576 bytes of weights per chunk
constexpr int ACH = MT * KC * 2;           // 8,192 bytes of latents per chunk
constexpr int STAGE = WCH + ACH;           // 32,768
constexpr int NSTAGE = 4;
constexpr int WCOPIES = WCH / 1024;        // 24 weight copies per chunk
constexpr int CPW = STAGE / 1024 / 4;      // 8 copies per wave per chunk
constexpr int UK_BYTES = DNOPE * DC * 2;   // 131,072: W_UK[h]
constexpr int QN_OFF = UK_BYTES;           // the nope tile [64 x 128] bf16 after W_UK
static_assert(NSTAGE * STAGE <= UK_BYTES, "the ring fits below the nope tile");
static_assert(DQ % KC == 0 && WCH % 1024 == 0 && ACH % 1024 == 0, "chunk geometry");

// Swizzles (16-byte chunk c of row r stored at position c ^ s(r)):
//   W_UQ chunk rows (384 bytes, 24 chunks): 4 ((r >> 1) & 1) -- a transposed
//     read of rows r0..r0+3 and four chunks meets 16 bank quads;
//   latent chunk rows (128 bytes): (r >> 1) & 7 -- 16 rows at one chunk
//     meet 16 bank quads;
//   W_UK rows (1024 bytes): 4 (r & 3); nope tile rows (256 bytes): r & 15.
__device__ __forceinline__ int swz_wuq(int r) { return 4 * ((r >> 1) & 1); }
__device__ __forceinline__ int swz_lat(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_wuk(int r) { return 4 * (r & 3); }

// Transposed B read of a 16-row k-step (rows k0 + krow and k0 + krow + 4 of
// the lane), 32 columns starting at column 32 nt: 8 bf16 per lane.
template <int ROWB, int (*SWZ)(int)>
__device__ __forceinline__ bf16x8 read_b(const uint8_t *tile, int k0, int nt, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int krow = 8 * (g >> 1) + (q >> 2);
  const int chunk = 4 * nt + 2 * (g & 1) + ((q & 3) >> 1);
  const int r0 = k0 + krow, r1 = r0 + 4;
  const uint8_t *p0 = tile + r0 * ROWB + ((chunk ^ SWZ(r0)) << 4) + (q & 1) * 8;
  const uint8_t *p1 = tile + r1 * ROWB + ((chunk ^ SWZ(r1)) << 4) + (q & 1) * 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void query_latent_kernel(QueryLatentArgs qa) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[UK_BYTES + MT * DNOPE * 2];
  // cos/sin of the sequences' positions per rotary pair; once the rotary
  // columns are done, the same 16 KB hold the low part of the nope tile
  __shared__ __attribute__((aligned(16))) float csn[MT][DR / 2][2];
  static_assert(sizeof(csn) == MT * DNOPE * 2, "the low nope tile reuses the angle table");
  const RopeAppendArgs &ra = qa.ra;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int B = ra.B, H = ra.H;

  if (h >= H) {
    // cache rows of the new tokens (the start of csn serves as their angle table)
    float *cs = &csn[0][0][0], *sn = cs + DR / 2;
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

  const int b0 = blockIdx.x * MT;
  const int last_row = min(MT, B - b0) - 1;
  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *wsrc = reinterpret_cast<const uint8_t *>(qa.w_uq) + static_cast<size_t>(h) * WROW;
  const size_t wpitch = static_cast<size_t>(H) * WROW;
  const uint8_t *asrc = reinterpret_cast<const uint8_t *>(qa.c_q) + static_cast<size_t>(b0) * (DQ * 2);

  // copy j (0..31) of chunk ch: j < 24 -> weight pieces 64 j .. 64 j + 63
  // (row p / 24, position p % 24); else latent pieces (row p / 8, position
  // p % 8).  Wave w issues copies 8 w .. 8 w + 7.  Rows past the batch
  // re-read the last sequence.
  auto issue = [&](int ch) {
    const uint32_t st = lds0 + (ch % NSTAGE) * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int j = wave * CPW + i;
      if (j < WCOPIES) {
        const int p = 64 * j + lane, r = p / 24, pos = p - 24 * r;
        const int c = pos ^ swz_wuq(r);
        dma16(wsrc + (static_cast<size_t>(ch) * KC + r) * wpitch + c * 16, __builtin_amdgcn_readfirstlane(st + 1024 * j));
      } else {
        const int p = 64 * (j - WCOPIES) + lane, r = p >> 3, pos = p & 7;
        const int c = pos ^ swz_lat(r);
        dma16(asrc + static_cast<size_t>(min(r, last_row)) * (DQ * 2) + ch * (KC * 2) + c * 16,
              __builtin_amdgcn_readfirstlane(st + 1024 * j));
      }
    }
  };
  issue(0);
  issue(1);
  issue(2);

  // angles of the sequences' positions (fp64), while the first chunks land
  for (int e = tid; e < MT * (DR / 2); e += 256) {
    const int r = e / (DR / 2), i = e % (DR / 2);
    const int pos = b0 + r < B ? rope_position(ra.seq_lens[b0 + r]) : 0;
    rope_cos_sin(ra, pos, i, csn[r][i][0], csn[r][i][1]);
  }

  // ---- q_h = c' . W_UQ_h: wave w owns sequences 32 (w & 1) .. + 31 and
  // column tiles 3 (w >> 1) .. + 2 (waves 0, 1: nope columns 0..95; waves
  // 2, 3: nope 96..127 and the rotary columns)
  const int mw = wave & 1, nt0 = 3 * (wave >> 1);
  const int ar = 32 * mw + (lane & 31), hb = lane >> 5;
  f32x16 acc[3] = {};
  for (int ch = 0; ch < NCH; ++ch) {
    if (ch + 2 < NCH) wait_vmcnt<2 * CPW>();   // chunks ch + 1 and ch + 2 may still be in flight
    else if (ch + 1 < NCH) wait_vmcnt<CPW>();
    else wait_vmcnt<0>();
    barrier_no_fence();                       // chunk ch visible; every wave done with chunk ch - 1
    if (ch + 3 < NCH) issue(ch + 3);
    const uint8_t *st = lds + (ch % NSTAGE) * STAGE;
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      const int c = 2 * ks + hb;
      const bf16x8 av = *reinterpret_cast<const bf16x8 *>(st + WCH + ar * (KC * 2) + ((c ^ swz_lat(ar)) << 4));
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const bf16x8 bv = read_b<WROW, swz_wuq>(st, 16 * ks, nt0 + t, lane);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[t], 0, 0, 0);
      }
    }
  }
  __syncthreads();                            // every wave is done with the ring

  // W_UK[h] -> LDS [0, 128 KB): row k (1 KB), chunk c at c ^ swz_wuk(k)
  {
    const uint8_t *uk = reinterpret_cast<const uint8_t *>(qa.w_uk) + static_cast<size_t>(h) * UK_BYTES;
#pragma unroll 4
    for (int i = 0; i < UK_BYTES / 1024 / 4; ++i) {
      const int j = wave * (UK_BYTES / 1024 / 4) + i;        // 32 copies per wave, one 1 KB row each
      const int c = lane ^ swz_wuk(j);
      dma16(uk + static_cast<size_t>(j) * 1024 + c * 16, __builtin_amdgcn_readfirstlane(lds0 + 1024 * j));
    }
  }

  // The nope columns go to LDS as a sum of two bf16 tiles, hi = bf16(x) and
  // lo = bf16(x - hi) (row r, chunk c at c ^ (r & 15)): the second product
  // then sees q_nope to about 2^-17 relative instead of one bf16 rounding,
  // which alone would move q_lat elements by several 1e-3.  The rotary
  // columns are turned and stored.  Register i of tile t: row
  // 32 mw + 8 (i / 4) + 4 hb + i % 4, column 32 (nt0 + t) + lane % 32.
  uint8_t *qn = lds + QN_OFF;
  uint8_t *ql = reinterpret_cast<uint8_t *>(&csn[0][0][0]);
  auto qn_off = [](int row, int col) { return row * (DNOPE * 2) + (((col >> 3) ^ (row & 15)) << 4) + 2 * (col & 7); };
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int col = 32 * (nt0 + t) + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * mw + 8 * (i >> 2) + 4 * hb + (i & 3);
      const float x = acc[t][i];
      if (nt0 + t < DNOPE / 32) {
        *reinterpret_cast<uint16_t *>(qn + qn_off(row, col)) = bf16_bits(to_bf16(x));
      } else {
        const float y = __shfl_xor(x, 1);      // the pair partner (neighbouring column)
        const int pr = (col - DNOPE) >> 1;
        const float cs = csn[row][pr][0], sn = csn[row][pr][1];
        const float v = (col & 1) ? y * sn + x * cs : x * cs - y * sn;
        if (row <= last_row)
          ra.q[(static_cast<size_t>(b0 + row) * H + h) * DROW + DC + (col - DNOPE)] = bf16_bits(to_bf16(v));
      }
    }
  }
  __syncthreads();                            // the angle table is free
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (nt0 + t >= DNOPE / 32) continue;
    const int col = 32 * (nt0 + t) + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * mw + 8 * (i >> 2) + 4 * hb + (i & 3);
      const float x = acc[t][i];
      *reinterpret_cast<uint16_t *>(ql + qn_off(row, col)) = bf16_bits(to_bf16(x - bf16_round_f32(x)));
    }
  }
  wait_vmcnt<0>();                            // this wave's W_UK copies
  __syncthreads();                            // W_UK and both nope tiles visible

  // ---- q_lat = (hi + lo) . W_UK[h]: wave w owns columns 128 w .. 128 w + 127
  // (tiles 4 w .. 4 w + 3) of both 32-sequence halves
  f32x16 o[2][4] = {};
#pragma unroll
  for (int ks = 0; ks < DNOPE / 16; ++ks) {
    const int c = 2 * ks + hb;
    bf16x8 ah[2], al[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = 32 * m + (lane & 31);
      const int off = r * (DNOPE * 2) + ((c ^ (r & 15)) << 4);
      ah[m] = *reinterpret_cast<const bf16x8 *>(qn + off);
      al[m] = *reinterpret_cast<const bf16x8 *>(ql + off);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 bv = read_b<DC * 2, swz_wuk>(lds, 16 * ks, 4 * wave + t, lane);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        o[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[m], bv, o[m][t], 0, 0, 0);
        o[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[m], bv, o[m][t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = 32 * (4 * wave + t) + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * m + 8 * (i >> 2) + 4 * hb + (i & 3);
        if (row <= last_row) ra.q[(static_cast<size_t>(b0 + row) * H + h) * DROW + col] = bf16_bits(to_bf16(o[m][t][i]));
      }
    }
}

}  // namespace

hipError_t launch_query_latent(const QueryLatentArgs &qa, hipStream_t stream) {
  const int tiles = (qa.ra.B + MT - 1) / MT;
  const int append_rows = qa.ra.kv_new ? std::max(1, std::min(8, (qa.ra.B + tiles - 1) / tiles)) : 0;
  query_latent_kernel<<<dim3(tiles, qa.ra.H + append_rows), 256, 0, stream>>>(qa);
  return hipGetLastError();
}

}  // namespace mla
