// Query and value absorption GEMMs (per-head, batch as the MFMA M dimension).
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
// Each wave produces one 32 (batch) x 32 (column) tile with
// v_mfma_f32_32x32x16_bf16: A rows are 16-byte loads of the activations, B
// columns are gathered from the row-major weight (consecutive lanes read
// consecutive columns, so each weight row segment is read once per tile).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

template <int K>
__device__ __forceinline__ f32x16 wave_tile(const uint16_t *A, size_t lda, int rows_valid,
                                            const uint16_t *Bm, int ldb) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hl = lane >> 5;
  const bool aval = r < rows_valid;
  const uint16_t *ap = A + (aval ? r : 0) * lda + hl * 8;
  const uint16_t *bp = Bm + static_cast<size_t>(hl * 8) * ldb + r;
  f32x16 acc = {};
#pragma unroll 4
  for (int kb = 0; kb < K / 16; ++kb) {
    u32x4 av = *reinterpret_cast<const u32x4 *>(ap + kb * 16);
    if (!aval) av = u32x4{0, 0, 0, 0};
    bf16x8 bv;
#pragma unroll
    for (int j = 0; j < 8; ++j) bv[j] = __builtin_bit_cast(__bf16, bp[static_cast<size_t>(kb * 16 + j) * ldb]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bv, acc, 0, 0, 0);
  }
  return acc;
}

// Store a 32x32 accumulator tile: row (batch) b0 + (i/4)*8 + 4*half + i%4, column lane%32.
__device__ __forceinline__ void store_tile(const f32x16 &acc, uint16_t *C, size_t ldc, int rows_valid) {
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = (i >> 2) * 8 + hl * 4 + (i & 3);
    if (row < rows_valid) C[row * ldc + (lane & 31)] = bf16_bits(to_bf16(acc[i]));
  }
}

// grid (DC/128, H, ceil(B/32)), 4 waves: wave w owns columns [128 x + 32 w, +32).
__global__ __launch_bounds__(256) void absorb_q_kernel(const uint16_t *q_nope, const uint16_t *w_uk,
                                                       uint16_t *q, int B, int H) {
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 128 + wave * 32;
  const int h = blockIdx.y;
  const int b0 = blockIdx.z * 32;
  const int rows = B - b0;
  const f32x16 acc = wave_tile<DNOPE>(q_nope + (static_cast<size_t>(b0) * H + h) * DNOPE,
                                      static_cast<size_t>(H) * DNOPE, rows,
                                      w_uk + static_cast<size_t>(h) * DNOPE * DC + n0, DC);
  store_tile(acc, q + (static_cast<size_t>(b0) * H + h) * DROW + n0, static_cast<size_t>(H) * DROW, rows);
}

// grid (1, H, ceil(B/32)), 4 waves: wave w owns output columns [32 w, +32).
__global__ __launch_bounds__(256) void absorb_out_kernel(const uint16_t *o_lat, const uint16_t *w_uv,
                                                         uint16_t *o, int B, int H) {
  const int wave = threadIdx.x >> 6;
  const int n0 = wave * 32;
  const int h = blockIdx.y;
  const int b0 = blockIdx.z * 32;
  const int rows = B - b0;
  const f32x16 acc = wave_tile<DC>(o_lat + (static_cast<size_t>(b0) * H + h) * DC,
                                   static_cast<size_t>(H) * DC, rows,
                                   w_uv + static_cast<size_t>(h) * DC * DV + n0, DV);
  store_tile(acc, o + (static_cast<size_t>(b0) * H + h) * DV + n0, static_cast<size_t>(H) * DV, rows);
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t *q_nope, const uint16_t *w_uk, uint16_t *q, int B, int H,
                           hipStream_t stream) {
  absorb_q_kernel<<<dim3(DC / 128, H, (B + 31) / 32), 256, 0, stream>>>(q_nope, w_uk, q, B, H);
  return hipGetLastError();
}

hipError_t launch_absorb_out(const uint16_t *o_latent, const uint16_t *w_uv, uint16_t *o, int B, int H,
                             hipStream_t stream) {
  absorb_out_kernel<<<dim3(1, H, (B + 31) / 32), 256, 0, stream>>>(o_latent, w_uv, o, B, H);
  return hipGetLastError();
}

}  // namespace mla
