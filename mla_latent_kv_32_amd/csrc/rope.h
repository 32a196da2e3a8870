// Decoupled RoPE of the new token and its append to the paged latent cache:
// the device pieces shared by rope_append_kernel and the fused query kernel.
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
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

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

// Position of the token appended for a sequence of length S (row S - 1); an
// empty slot rotates at position 0 and appends nothing.
__device__ __forceinline__ int rope_position(int S) { return S > 0 ? S - 1 : 0; }

// cos and sin of pos * w for the frequency w of one pair (angle formed and
// reduced in float64).
__device__ __forceinline__ void rope_cos_sin_at(double w, int pos, float &c, float &s) {
  double sv, cv;
  sincos(static_cast<double>(pos) * w, &sv, &cv);
  c = static_cast<float>(cv);
  s = static_cast<float>(sv);
}
__device__ __forceinline__ void rope_cos_sin(const double *inv_freq, int pos, int i, float &c, float &s) {
  rope_cos_sin_at(inv_freq[i], pos, c, s);
}
__device__ __forceinline__ void rope_cos_sin(const RopeAppendArgs &a, int pos, int i, float &c, float &s) {
  rope_cos_sin(a.inv_freq, pos, i, c, s);
}

// One interleaved bf16 pair (packed low | high << 16) turned by the angle.
__device__ __forceinline__ uint32_t rope_rotate_pair(uint32_t pr, float c, float s) {
  const float x1 = bf16_to_f32(pr & 0xFFFFu), x2 = bf16_to_f32(pr >> 16);
  const float y1 = x1 * c - x2 * s;
  const float y2 = x1 * s + x2 * c;
  return static_cast<uint32_t>(bf16_bits(to_bf16(y1))) | (static_cast<uint32_t>(bf16_bits(to_bf16(y2))) << 16);
}

// The same rotation with the result rounded to IEEE half instead (the
// explicit-form prefill keeps its attention operands in fp16).
__device__ __forceinline__ uint32_t rope_rotate_pair_f16(uint32_t pr, float c, float s) {
  const float x1 = bf16_to_f32(pr & 0xFFFFu), x2 = bf16_to_f32(pr >> 16);
  const float y1 = x1 * c - x2 * s;
  const float y2 = x1 * s + x2 * c;
  return static_cast<uint32_t>(f16_bits(y1)) | (static_cast<uint32_t>(f16_bits(y2)) << 16);
}

// Query pair i of (b, h): q[b, h, 512 + 2i .. 512 + 2i + 1] = RoPE(q_pe[b, h]).
__device__ __forceinline__ uint32_t rope_query_load(const RopeAppendArgs &a, int b, int h, int i) {
  return *reinterpret_cast<const uint32_t *>(a.q_pe + (static_cast<size_t>(b) * a.H + h) * DR + 2 * i);
}
__device__ __forceinline__ void rope_query_store(const RopeAppendArgs &a, int b, int h, int i, uint32_t pr, float c,
                                                 float s) {
  *reinterpret_cast<uint32_t *>(a.q + (static_cast<size_t>(b) * a.H + h) * DROW + DC + 2 * i) =
      rope_rotate_pair(pr, c, s);
}
__device__ __forceinline__ void rope_query_pair(const RopeAppendArgs &a, int b, int h, int i, float c, float s) {
  rope_query_store(a, b, h, i, rope_query_load(a, b, h, i), c, s);
}

// Store one latent-cache row at slot `slot` of the pool (page * 64 + offset):
// the latent part `lat` (512 bf16) copied (bf16 pool) or quantised (fp8 pool:
// wave g quantises group g), the rotary key `kpe` (64 bf16, unrotated) turned
// by (cs[i], sn[i]) = angle of pair i at the token's position.  Called by all
// 256 threads of a workgroup.
__device__ __forceinline__ void store_cache_row(uint8_t *cache, int kv_fp8, size_t slot, const uint16_t *lat,
                                                const uint16_t *kpe, int tid, const float *cs, const float *sn) {
  uint8_t *row = cache + slot * (kv_fp8 ? FP8_ROW_BYTES : ROW_BYTES);
  const int rope_off = kv_fp8 ? DC : 2 * DC;     // byte offset of the rotary key in the row

  if (tid < DR / 2) {
    const uint32_t pr = *reinterpret_cast<const uint32_t *>(kpe + 2 * tid);
    *reinterpret_cast<uint32_t *>(row + rope_off + 4 * tid) = rope_rotate_pair(pr, cs[tid], sn[tid]);
  }
  if (!kv_fp8) {
    if (tid < DC / 8)
      *reinterpret_cast<u32x4 *>(row + tid * 16) = *reinterpret_cast<const u32x4 *>(lat + tid * 8);
    return;
  }
  // fp8: wave g quantises latent group g (128 values, 2 per lane).
  const uint32_t pr = *reinterpret_cast<const uint32_t *>(lat + 2 * tid);
  const float v0 = bf16_to_f32(pr & 0xFFFFu), v1 = bf16_to_f32(pr >> 16);
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
  const uint32_t c0 = e4m3_rne_sat(v0 / scale), c1 = e4m3_rne_sat(v1 / scale);
  *reinterpret_cast<uint16_t *>(row + 2 * tid) = static_cast<uint16_t>(c0 | (c1 << 8));
  if ((tid & 63) == 0) *reinterpret_cast<float *>(row + DC + 2 * DR + 4 * (tid >> 6)) = scale;
}

// Append the new token's row of sequence b (S = seq_lens[b] > 0) at position
// S - 1 from kv_new[b] = [latent | unrotated rotary key].
__device__ __forceinline__ void append_row(const RopeAppendArgs &a, int b, int S, int tid, const float *cs,
                                           const float *sn) {
  const int pos = rope_position(S);
  const int page = a.block_table[static_cast<size_t>(b) * a.max_blocks + (pos / PAGE)];
  const uint16_t *src = a.kv_new + static_cast<size_t>(b) * DROW;
  store_cache_row(a.cache, a.kv_fp8, static_cast<size_t>(page) * PAGE + (pos % PAGE), src, src + DC, tid, cs, sn);
}

}  // namespace mla
