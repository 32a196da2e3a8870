// Launch interfaces between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {


struct DecodeArgs {
  const uint16_t *q;            // [B, H, 576] bf16
  const uint8_t *cache;         // paged pool
  const int32_t *block_table;   // [B, max_blocks]
  const int32_t *seq_lens;      // [B]
  int max_blocks;
  int B, H;
  int split_tokens;             // multiple of 64
  int n_splits;                 // chunks per sequence in the grid
  int direct;                   // 1: one chunk, write o_latent / lse directly
  int kv_fp8;                   // 1: packed fp8 rows (656 bytes), else bf16 rows (1152 bytes)
  float scale_log2;             // softmax_scale * log2(e)
  // Multi-token decode: H = q_len * heads query rows per sequence, row
  // v = j * heads + h for new token j; row v sees the tokens t <
  // seq_len - (q_len - 1) + v / heads.  q_len <= 1 is the single-token case.
  int q_len;
  int heads;
  uint16_t *o_latent;           // [B, H, 512] bf16
  float *lse;                   // [B, H] or null
  uint16_t *o_part;             // [B, n_splits, H, 512] bf16 partial outputs
  float *lse_part;              // [B, n_splits, H] fp32
};

// Split-KV combine order.  A row's partials are summed in ranges of
// combine_range(n_splits) consecutive chunks -- each range in chunk order
// from zero, then the range sums in range order -- so that up to 8 waves can
// stream one row's chunks at once.  A multiple of 8 (the load batch), at
// least 16, and at most 8 ranges.  Every combine kernel follows this order,
// so the separate and the fused merges agree bit for bit.
__host__ __device__ inline int combine_range(int n_splits) {
  int r = (n_splits + 7) / 8;
  r = (r + 7) & ~7;
  return r < 16 ? 16 : r;
}

// Attention over each chunk; direct mode writes o_latent/lse, else partials.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// Log-sum-exp merge of the partials into o_latent/lse.
hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream);
// fp8 cache only, single new token: the same chunks and partials as
// launch_decode, with both products on fp8 MFMAs over the stored codes.
hipError_t launch_decode_fp8_mfma(const DecodeArgs &a, hipStream_t stream);

// Decode workgroup shape: 16 heads per wave (MFMA 16x16x32) and 2, 4 or 8
// waves per workgroup.  At least two waves share a block's copies so that
// three blocks in flight stay within the 6-bit vector-memory counter
// (3 x 18 copies per wave).
inline int decode_heads_per_wave(int) { return 16; }
inline int decode_waves(int H) { return H <= 32 ? 2 : (H <= 64 ? 4 : 8); }
inline int decode_head_groups(int H) {
  const int per = decode_heads_per_wave(H) * decode_waves(H);
  return (H + per - 1) / per;
}

// q[b,h,0:512] = q_nope[b,h,:] . W_UK[h]
hipError_t launch_absorb_q(const uint16_t *q_nope, const uint16_t *w_uk, uint16_t *q, int B, int H,
                           hipStream_t stream);
// o[b,h,:] = o_latent[b,h,:] . W_UV[h]
hipError_t launch_absorb_out(const uint16_t *o_latent, const uint16_t *w_uv, uint16_t *o, int B, int H,
                             hipStream_t stream);

// Split-KV combine fused with the value absorption (one workgroup per head).
struct CombineOutArgs {
  const uint16_t *o_part;       // [B, n_splits, H, 512] bf16
  const float *lse_part;        // [B, n_splits, H]
  const int32_t *seq_lens;
  int split_tokens, n_splits;
  const uint16_t *w_uv;         // [H, 512, 128]
  uint16_t *o;                  // [B, H, 128]
  uint16_t *o_latent;           // [B, H, 512] or null
  float *lse;                   // [B, H] or null
  int B, H;
  int tile_slots;               // workgroups per head (set by the launcher)
};
hipError_t launch_combine_absorb_out(const CombineOutArgs &a, hipStream_t stream);

struct RopeAppendArgs {
  const uint16_t *q_pe;         // [B, H, 64]
  const uint16_t *kv_new;       // [B, 576]
  const int32_t *seq_lens;
  const int32_t *block_table;
  int max_blocks;
  uint8_t *cache;
  int kv_fp8;
  double inv_freq[32];          // theta^(-2i/64), i = 0..31, formed on the host in float64
  uint16_t *q;                  // [B, H, 576]
  int B, H;
};

hipError_t launch_rope_append(const RopeAppendArgs &a, hipStream_t stream);

// The decode query from the query latent: q[:, :, 0:512] = (c' W_UQ_nope) . W_UK,
// q[:, :, 512:576] = RoPE(c' W_UQ_rope); ra.q_pe is unused, ra.kv_new null =
// no cache append.
struct QueryLatentArgs {
  const uint16_t *c_q;          // [B, 1536]
  const uint16_t *w_uq;         // [1536, H * 192], per head [nope 128 | rope 64]
  const uint16_t *w_uk;         // [H, 128, 512]
  RopeAppendArgs ra;
};
hipError_t launch_query_latent(const QueryLatentArgs &qa, hipStream_t stream);
// mla_absorb_q and mla_rope_append_cache in one launch (ra.q receives both parts).
hipError_t launch_query(const uint16_t *q_nope, const uint16_t *w_uk, const RopeAppendArgs &ra, hipStream_t stream);

// Explicit-form prefill of B packed prompts (T tokens in all, token-major,
// prompt b = tokens cu_seqlens[b] .. cu_seqlens[b + 1] - 1 at positions 0..).
struct PrefillArgs {
  const uint16_t *q_nope;       // [T, H, 128]
  const uint16_t *q_pe;         // [T, H, 64], unrotated
  const uint16_t *c;            // [T, 512] latents
  const uint16_t *k_pe;         // [T, 64], unrotated shared rotary key
  const uint16_t *w_uk;         // [H, 128, 512]
  const uint16_t *w_uv;         // [H, 512, 128]
  const int32_t *cu_seqlens;    // [B + 1]
  const int32_t *block_table;   // [B, max_blocks]
  int max_blocks;
  uint8_t *cache;
  int kv_fp8;
  double inv_freq[32];
  float scale_log2;             // softmax_scale * log2(e)
  int B, H, T, max_len;
  uint16_t *o;                  // [T, H, 128]
  // Chunks that continue a cached prefix: prompt b's P_b = prefix_lens[b]
  // rows are already in the cache and its tokens sit at positions P_b + j.
  // Keys (the prefix's and the prompt's own) are packed per prompt at
  // cu_keys[b] .. cu_keys[b + 1] - 1 of the key arrays.  Without a prefix
  // (prefix_lens null) cu_keys = cu_seqlens, c_keys = c and T_keys = T.
  const int32_t *prefix_lens;   // [B] or null
  const int32_t *cu_keys;       // [B + 1]
  const uint16_t *c_keys;       // [T_keys, c_keys_w] latents of every key (bf16)
  int c_keys_w;                 // 512, or 1024 = [hi | lo] bf16 terms (fp8 prefix rows)
  int T_keys, max_prefix;
  // workspace (attention operands in IEEE half)
  uint16_t *q_rot;              // [T, H, 64] fp16
  uint16_t *k_rot;              // [T_keys, 64] fp16
  uint16_t *k_nope;             // [T_keys, H, 128] fp16
  uint16_t *v;                  // [T_keys, H, 128] fp16
  uint16_t *c_gather;           // [T_keys, c_keys_w] bf16 (chunks only: c_keys points here)
  int32_t *cu_keys_ws;          // [B + 1] (chunks only: cu_keys points here)
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// Check of seq_lens / block_table against the host-side bounds.
struct ValidateArgs {
  const int32_t *seq_lens;      // [B]
  const int32_t *block_table;   // [B, max_blocks]
  int max_blocks, max_seq_len, num_blocks, B;
  int32_t *bad;                 // number of sequences breaking a rule
  int32_t *first_bad;           // smallest such b, -1 if none (or null)
};
hipError_t launch_validate_paging(const ValidateArgs &a, hipStream_t stream);

}  // namespace mla
