// Decoupled RoPE for the new token and its append to the paged latent cache.
//
// The query's rotary part and the shared rotary key are turned by the token's
// position; the key is stored already rotated next to the latent, so decode
// never rotates cached rows again (Su, "The Ultimate Tug-of-War Between Cache
// and Performance", MLA Part 2; DL0107, "Multi-head Latent Attention MLA",
// decoupled RoPE paragraph).  Pairs are interleaved (v[2i], v[2i+1]) with
// frequency theta^(-2i/64) (Riju, "Multi-Head Latent Attention vs GQA vs MQA",
// rope function in "A latent KV projection in PyTorch").  Angles are formed
// and reduced in float64 (positions reach 32K and beyond; the 32 frequencies
// come from the host), the rotation runs in float32, results round to bf16.
//
// fp8 caches store the latent as OCP E4M3 codes with one fp32 scale per group
// of 128: scale = amax/448 (IEEE float32 division), code = round-to-nearest-
// even of c/scale, saturated at +-448.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

// float -> OCP E4M3 code, round to nearest even, saturating (no NaN inputs).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    // subnormals and zero: multiples of 2^-9; 8 * 2^-9 is the smallest normal
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    const uint32_t ua = __float_as_uint(a);
    int e = static_cast<int>(ua >> 23) - 127;          // -6 .. 8
    const uint32_t man = ua & 0x7FFFFFu;
    uint32_t m = man >> 20;                            // top 3 mantissa bits
    const uint32_t rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) { m = 0u; ++e; }
    code = (static_cast<uint32_t>(e + 7) << 3) | m;   // a <= 448 keeps this <= 0x7E
  }
  return code == 0u ? 0u : (code | sign);
}

// grid (B, ceil(H / 16)): each workgroup rotates the query pairs of 16 heads
// of one sequence (2 pairs per thread); workgroup (b, 0) also appends the row.
constexpr int HEADS_PER_WG = 16;

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  __shared__ float cs[DR / 2], sn[DR / 2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = a.seq_lens[b];
  const int pos = S > 0 ? S - 1 : 0;
  if (tid < DR / 2) {
    double sv, cv;
    sincos(static_cast<double>(pos) * a.inv_freq[tid], &sv, &cv);
    cs[tid] = static_cast<float>(cv);
    sn[tid] = static_cast<float>(sv);
  }
  __syncthreads();

  const int h0 = blockIdx.y * HEADS_PER_WG;
  for (int idx = tid; idx < HEADS_PER_WG * (DR / 2); idx += blockDim.x) {
    const int h = h0 + idx / (DR / 2), i = idx % (DR / 2);
    if (h >= a.H) break;
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    const uint32_t pr = *reinterpret_cast<const uint32_t *>(a.q_pe + bh * DR + 2 * i);
    const float x1 = bf16_to_f32(pr & 0xFFFFu), x2 = bf16_to_f32(pr >> 16);
    const float y1 = x1 * cs[i] - x2 * sn[i];
    const float y2 = x1 * sn[i] + x2 * cs[i];
    *reinterpret_cast<uint32_t *>(a.q + bh * DROW + DC + 2 * i) =
        static_cast<uint32_t>(bf16_bits(to_bf16(y1))) | (static_cast<uint32_t>(bf16_bits(to_bf16(y2))) << 16);
  }
  if (blockIdx.y != 0) return;
  if (S <= 0) return;

  const int page = a.block_table[static_cast<size_t>(b) * a.max_blocks + (pos / PAGE)];
  const uint16_t *src = a.kv_new + static_cast<size_t>(b) * DROW;
  const size_t slot = static_cast<size_t>(page) * PAGE + (pos % PAGE);
  uint8_t *row = a.cache + slot * (a.kv_fp8 ? FP8_ROW_BYTES : ROW_BYTES);
  const int rope_off = a.kv_fp8 ? DC : 2 * DC;   // byte offset of the rotary key in the row

  if (tid < DR / 2) {
    const uint32_t pr = *reinterpret_cast<const uint32_t *>(src + DC + 2 * tid);
    const float x1 = bf16_to_f32(pr & 0xFFFFu), x2 = bf16_to_f32(pr >> 16);
    const float y1 = x1 * cs[tid] - x2 * sn[tid];
    const float y2 = x1 * sn[tid] + x2 * cs[tid];
    *reinterpret_cast<uint32_t *>(row + rope_off + 4 * tid) =
        static_cast<uint32_t>(bf16_bits(to_bf16(y1))) | (static_cast<uint32_t>(bf16_bits(to_bf16(y2))) << 16);
  }
  if (!a.kv_fp8) {
    if (tid < DC / 8)
      *reinterpret_cast<u32x4 *>(row + tid * 16) = *reinterpret_cast<const u32x4 *>(src + tid * 8);
    return;
  }
  // fp8: wave g quantises latent group g (128 values, 2 per lane).
  const uint32_t pr = *reinterpret_cast<const uint32_t *>(src + 2 * tid);
  const float v0 = bf16_to_f32(pr & 0xFFFFu), v1 = bf16_to_f32(pr >> 16);
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
  const uint32_t c0 = e4m3_rne_sat(v0 / scale), c1 = e4m3_rne_sat(v1 / scale);
  *reinterpret_cast<uint16_t *>(row + 2 * tid) = static_cast<uint16_t>(c0 | (c1 << 8));
  if ((tid & 63) == 0) *reinterpret_cast<float *>(row + DC + 2 * DR + 4 * (tid >> 6)) = scale;
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs &a, hipStream_t stream) {
  rope_append_kernel<<<dim3(a.B, (a.H + HEADS_PER_WG - 1) / HEADS_PER_WG), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
