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
#include "common.h"
#include "kernels.h"

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

template <int K, int N, int NT, int OUT_ROW>
__global__ __launch_bounds__(NT * 2) void absorb_kernel(const uint16_t *act, const uint16_t *w, uint16_t *out,
                                                        int B, int H) {
  constexpr int CPR = NT * 2 / 16;                      // 16-byte chunks per tile row
  constexpr int CHUNKS = K * CPR;
  constexpr int NWAVE = NT / 32;
  constexpr int PER_WAVE = CHUNKS / (64 * NWAVE);       // DMA copies per wave
  static_assert(CHUNKS % (64 * NWAVE) == 0, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t tile[K * NT * 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * NT;
  const int h = blockIdx.y;

  // ---- weight tile -> LDS (row k, position p <- chunk p ^ wsw(k) of the row)
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
  wait_vmcnt<0>();
  __syncthreads();

  // ---- per-lane LDS offsets of the transposed B reads (lane 16g + q reads
  // rows 8 (g >> 1) + q / 4 (+4 for the second read) of each 16-row k-step,
  // columns 32 wave + 16 (g & 1) + 4 (q & 3) .. +4)
  const int g = lane >> 4, q = lane & 15;
  const int krow = 8 * (g >> 1) + (q >> 2);
  const int chunk = 4 * wave + 2 * (g & 1) + ((q & 3) >> 1);
  const int boff0 = krow * (NT * 2) + ((chunk ^ wsw<NT>(krow)) << 4) + (q & 1) * 8;
  const int boff1 = (krow + 4) * (NT * 2) + ((chunk ^ wsw<NT>(krow + 4)) << 4) + (q & 1) * 8;

  const int r = lane & 31, hl = lane >> 5;
  const size_t ld_act = static_cast<size_t>(H) * K;
  const size_t ld_out = static_cast<size_t>(H) * OUT_ROW;
  for (int b0 = 0; b0 < B; b0 += 32) {
    const int rows = B - b0;
    const bool aval = r < rows;
    const uint16_t *ap = act + (static_cast<size_t>(b0 + (aval ? r : 0)) * H + h) * K + hl * 8;
    f32x16 acc = {};
#pragma unroll 8
    for (int kb = 0; kb < K / 16; ++kb) {
      u32x4 av = *reinterpret_cast<const u32x4 *>(ap + kb * 16);
      if (!aval) av = u32x4{0, 0, 0, 0};
      // rows kb*16 + ... : the swizzle depends on k & 3 / (k >> 1) & 1 only, which 16 kb keeps
      const uint8_t *t0 = tile + kb * 16 * (NT * 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t0 + boff1));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bv, acc, 0, 0, 0);
    }
    // row (batch) b0 + (i/4)*8 + 4*hl + i%4, column n0 + 32 wave + r
    uint16_t *op = out + static_cast<size_t>(b0) * ld_out + static_cast<size_t>(h) * OUT_ROW + n0 + wave * 32 + r;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
      if (row < rows) op[row * ld_out] = bf16_bits(to_bf16(acc[i]));
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t *q_nope, const uint16_t *w_uk, uint16_t *q, int B, int H,
                           hipStream_t stream) {
  absorb_kernel<DNOPE, DC, 128, DROW><<<dim3(DC / 128, H), 256, 0, stream>>>(q_nope, w_uk, q, B, H);
  return hipGetLastError();
}

hipError_t launch_absorb_out(const uint16_t *o_latent, const uint16_t *w_uv, uint16_t *o, int B, int H,
                             hipStream_t stream) {
  absorb_kernel<DC, DV, 64, DV><<<dim3(DV / 64, H), 128, 0, stream>>>(o_latent, w_uv, o, B, H);
  return hipGetLastError();
}

}  // namespace mla
