// C ABI of the MLA absorbed-decode library: argument validation, split
// planning and kernel launches on the caller's stream.  See include/mla.h for
// the contract of every entry point.
#include <math.h>
#include <stdint.h>

#include "mla.h"

#include <cmath>
#include <mutex>
#include "common.h"
#include "kernels.h"

// Fixed split-KV scratch of mla_decode_paged_noalloc (one copy per GPU).
// Host code never uses this name as an address: it is a host-side stand-in;
// the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMinSplitTokens = 256;   // smallest chunk the planner picks
constexpr int kDefaultCUs = 256;

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return kDefaultCUs;
  return cus;
}

int head_groups(int H) { return mla::decode_head_groups(H); }

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Chunk size giving roughly one workgroup per compute unit, never below
// kMinSplitTokens, a multiple of the page size.
int plan_split(int B, int H, int max_seq_len) {
  int full = round_up(max_seq_len > 0 ? max_seq_len : 1, MLA_BLOCK_SIZE);
  if (full > MLA_MAX_SPLIT_TOKENS) full = MLA_MAX_SPLIT_TOKENS;
  const long items = static_cast<long>(B) * head_groups(H);
  const int cus = device_cus();
  if (items >= cus) return full;
  const int n = static_cast<int>((cus + items - 1) / items);
  int split = round_up((max_seq_len + n - 1) / n, MLA_BLOCK_SIZE);
  if (split < kMinSplitTokens) split = kMinSplitTokens;
  return split < full ? split : full;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t workspace_for(int B, int H, int n_splits) {
  const size_t rows = static_cast<size_t>(B) * n_splits * H;
  return align256(rows * MLA_D_C * sizeof(uint16_t)) + align256(rows * sizeof(float));
}

int status_of(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported size or format";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_SCRATCH_TOO_SMALL: return "request exceeds the fixed scratch buffer";
    default: return "unknown status";
  }
}

int mla_abi_version(void) { return MLA_ABI_VERSION; }

int mla_absorb_q(const void *q_nope, const void *w_uk, void *q, int B, int H, int d_nope, int d_c,
                 int d_r, void *stream) {
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q) || B < 1 || H < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if (B > 65535 * 32 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (d_nope != MLA_D_NOPE || d_c != MLA_D_C || d_r != MLA_D_R) return MLA_ERR_UNSUPPORTED;
  return status_of(mla::launch_absorb_q(static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(w_uk),
                                        static_cast<uint16_t *>(q), B, H, static_cast<hipStream_t>(stream)));
}

namespace {

// Validation and argument block of mla_rope_append_cache; MLA_OK or an error.
int rope_args(const void *q_pe, const void *kv_new, const int32_t *seq_lens, const int32_t *block_table,
              int max_blocks_per_seq, void *kv_cache, int kv_dtype, int num_blocks, int block_size,
              float rope_theta, void *q, int B, int H, int d_c, int d_r, mla::RopeAppendArgs *a) {
  if (!aligned16(q_pe) || !aligned16(kv_new) || !aligned16(seq_lens) || !aligned16(block_table) ||
      !aligned16(kv_cache) || !aligned16(q) || B < 1 || H < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      !(rope_theta > 0.0f) || !isfinite(rope_theta))
    return MLA_ERR_INVALID_ARGUMENT;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARGUMENT;
  if (d_c != MLA_D_C || d_r != MLA_D_R || block_size != MLA_BLOCK_SIZE)
    return MLA_ERR_UNSUPPORTED;
  a->q_pe = static_cast<const uint16_t *>(q_pe);
  a->kv_new = static_cast<const uint16_t *>(kv_new);
  a->seq_lens = seq_lens;
  a->block_table = block_table;
  a->max_blocks = max_blocks_per_seq;
  a->cache = static_cast<uint8_t *>(kv_cache);
  a->kv_fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  for (int i = 0; i < MLA_D_R / 2; ++i)
    a->inv_freq[i] = std::pow(static_cast<double>(rope_theta), -(2.0 * i) / static_cast<double>(MLA_D_R));
  a->q = static_cast<uint16_t *>(q);
  a->B = B;
  a->H = H;
  return MLA_OK;
}

}  // namespace

int mla_rope_append_cache(const void *q_pe, const void *kv_new, const int32_t *seq_lens,
                          const int32_t *block_table, int max_blocks_per_seq, void *kv_cache, int kv_dtype,
                          int num_blocks, int block_size, float rope_theta, void *q, int B, int H, int d_c,
                          int d_r, void *stream) {
  mla::RopeAppendArgs a;
  const int st = rope_args(q_pe, kv_new, seq_lens, block_table, max_blocks_per_seq, kv_cache, kv_dtype, num_blocks,
                           block_size, rope_theta, q, B, H, d_c, d_r, &a);
  if (st != MLA_OK) return st;
  return status_of(mla::launch_rope_append(a, static_cast<hipStream_t>(stream)));
}

int mla_absorb_q_rope_append(const void *q_nope, const void *w_uk, const void *q_pe, const void *kv_new,
                             const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                             void *kv_cache, int kv_dtype, int num_blocks, int block_size, float rope_theta,
                             void *q, int B, int H, int d_nope, int d_c, int d_r, void *stream) {
  if (!aligned16(q_nope) || !aligned16(w_uk)) return MLA_ERR_INVALID_ARGUMENT;
  mla::RopeAppendArgs a;
  const int st = rope_args(q_pe, kv_new, seq_lens, block_table, max_blocks_per_seq, kv_cache, kv_dtype, num_blocks,
                           block_size, rope_theta, q, B, H, d_c, d_r, &a);
  if (st != MLA_OK) return st;
  if (B > 65535 * 32 || H > 65535 - 8) return MLA_ERR_UNSUPPORTED;   // grid rows: H + up to 8 append rows
  if (d_nope != MLA_D_NOPE) return MLA_ERR_UNSUPPORTED;
  return status_of(mla::launch_query(static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(w_uk), a,
                                     static_cast<hipStream_t>(stream)));
}

int mla_query_from_latent(const void *c_q, const void *w_uq, const void *w_uk, const void *kv_new,
                          const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                          void *kv_cache, int kv_dtype, int num_blocks, int block_size, float rope_theta,
                          void *q, int B, int H, int d_q, int d_nope, int d_c, int d_r, void *stream) {
  if (!aligned16(c_q) || !aligned16(w_uq) || !aligned16(w_uk) || !aligned16(seq_lens) || !aligned16(q) || B < 1 ||
      H < 1 || !(rope_theta > 0.0f) || !isfinite(rope_theta))
    return MLA_ERR_INVALID_ARGUMENT;
  if (d_q != MLA_D_Q || d_nope != MLA_D_NOPE || d_c != MLA_D_C || d_r != MLA_D_R) return MLA_ERR_UNSUPPORTED;
  if (H > 65535 - 8 || (B + 63) / 64 > 65535) return MLA_ERR_UNSUPPORTED;
  mla::QueryLatentArgs qa = {};
  if (kv_new != nullptr) {
    // rope_args validates the append's arguments; its q_pe slot is unused here (q stands in)
    const int st = rope_args(q, kv_new, seq_lens, block_table, max_blocks_per_seq, kv_cache, kv_dtype, num_blocks,
                             block_size, rope_theta, q, B, H, d_c, d_r, &qa.ra);
    if (st != MLA_OK) return st;
  } else {
    qa.ra.seq_lens = seq_lens;
    for (int i = 0; i < MLA_D_R / 2; ++i)
      qa.ra.inv_freq[i] = std::pow(static_cast<double>(rope_theta), -(2.0 * i) / static_cast<double>(MLA_D_R));
    qa.ra.q = static_cast<uint16_t *>(q);
    qa.ra.B = B;
    qa.ra.H = H;
  }
  qa.ra.q_pe = nullptr;
  qa.c_q = static_cast<const uint16_t *>(c_q);
  qa.w_uq = static_cast<const uint16_t *>(w_uq);
  qa.w_uk = static_cast<const uint16_t *>(w_uk);
  return status_of(mla::launch_query_latent(qa, static_cast<hipStream_t>(stream)));
}

int mla_validate_paging(const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                        int max_seq_len, int num_blocks, int block_size, int B, int32_t *bad,
                        int32_t *first_bad, void *stream) {
  if (seq_lens == nullptr || block_table == nullptr || bad == nullptr || B < 1 || max_blocks_per_seq < 1 ||
      max_seq_len < 0 || num_blocks < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  mla::ValidateArgs a;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.num_blocks = num_blocks;
  a.B = B;
  a.bad = bad;
  a.first_bad = first_bad;
  return status_of(mla::launch_validate_paging(a, static_cast<hipStream_t>(stream)));
}

int mla_decode_split_tokens(int B, int H, int max_seq_len) {
  if (B < 1 || H < 1 || max_seq_len < 0) return 0;
  return plan_split(B, H, max_seq_len);
}

size_t mla_decode_workspace_bytes(int B, int H, int max_seq_len, int split_tokens) {
  if (B < 1 || H < 1 || max_seq_len <= 0 || split_tokens < 0 || split_tokens % MLA_BLOCK_SIZE ||
      split_tokens > MLA_MAX_SPLIT_TOKENS)
    return 0;
  const int split = split_tokens ? split_tokens : plan_split(B, H, max_seq_len);
  return workspace_for(B, H, (max_seq_len + split - 1) / split);
}

}  // extern "C"

namespace {

enum class DecodeMode { Paged, Partial };

// Shared validation and argument set-up of mla_decode_paged / mla_decode_partial.
int prepare_decode(DecodeMode mode, const void *q, const void *kv_cache, int kv_dtype,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *seq_lens,
                   int max_seq_len, int num_blocks, int block_size, float softmax_scale, int split_tokens,
                   void *workspace, size_t workspace_bytes, void *o_latent, float *lse, int B, int H,
                   mla::DecodeArgs *a) {
  const bool paged = mode == DecodeMode::Paged;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(block_table) || !aligned16(seq_lens) ||
      (paged && !aligned16(o_latent)) || (lse != nullptr && !aligned16(lse)) || B < 1 || H < 1 ||
      max_blocks_per_seq < 1 || num_blocks < 1 || max_seq_len < 0 || !isfinite(softmax_scale) ||
      split_tokens < 0 || split_tokens % MLA_BLOCK_SIZE != 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARGUMENT;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long>(max_seq_len) > static_cast<long>(max_blocks_per_seq) * block_size)
    return MLA_ERR_INVALID_ARGUMENT;
  if (split_tokens > MLA_MAX_SPLIT_TOKENS) return MLA_ERR_UNSUPPORTED;
  const int split = split_tokens ? split_tokens : plan_split(B, H, max_seq_len);
  const int n_splits = max_seq_len > 0 ? (max_seq_len + split - 1) / split : 1;
  if (static_cast<long>(B) * n_splits * head_groups(H) > 2147483647L) return MLA_ERR_UNSUPPORTED;
  const bool direct = paged && n_splits == 1;
  const size_t need = direct ? 0 : workspace_for(B, H, n_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  a->q = static_cast<const uint16_t *>(q);
  a->cache = static_cast<const uint8_t *>(kv_cache);
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->max_blocks = max_blocks_per_seq;
  a->B = B;
  a->H = H;
  a->split_tokens = split;
  a->n_splits = n_splits;
  a->direct = direct ? 1 : 0;
  a->kv_fp8 = kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0;
  a->scale_log2 = softmax_scale * 1.44269504088896340736f;
  a->q_len = 1;
  a->heads = H;
  a->o_latent = static_cast<uint16_t *>(o_latent);
  a->lse = lse;
  const size_t rows = static_cast<size_t>(B) * n_splits * H;
  a->o_part = need ? static_cast<uint16_t *>(workspace) : nullptr;
  a->lse_part = need ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                                 align256(rows * MLA_D_C * sizeof(uint16_t)))
                     : nullptr;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_paged(const void *q, const void *kv_cache, int kv_dtype, const int32_t *block_table,
                     int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len, int num_blocks,
                     int block_size, float softmax_scale, int split_tokens, void *workspace,
                     size_t workspace_bytes, void *o_latent, float *lse, int B, int H, void *stream) {
  mla::DecodeArgs a;
  const int st = prepare_decode(DecodeMode::Paged, q, kv_cache, kv_dtype, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, num_blocks, block_size, softmax_scale, split_tokens,
                                workspace, workspace_bytes, o_latent, lse, B, H, &a);
  if (st != MLA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = mla::launch_decode(a, s);
  if (e != hipSuccess || a.direct) return status_of(e);
  return status_of(mla::launch_combine(a, s));
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_LAUNCH;
  if (dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_paged_noalloc(const void *q, const void *kv_cache, int kv_dtype, const int32_t *block_table,
                             int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len, int num_blocks,
                             int block_size, float softmax_scale, int split_tokens, void *o_latent, float *lse,
                             int B, int H, void *stream) {
  // The partials this request needs, against the fixed buffer (host arithmetic only).
  if (B >= 1 && H >= 1 && max_seq_len > 0 && split_tokens >= 0 && split_tokens % MLA_BLOCK_SIZE == 0 &&
      split_tokens <= MLA_MAX_SPLIT_TOKENS) {
    const int split = split_tokens ? split_tokens : plan_split(B, H, max_seq_len);
    const int n_splits = (max_seq_len + split - 1) / split;
    if (n_splits > 1 && workspace_for(B, H, n_splits) > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_TOO_SMALL;
  }
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  return mla_decode_paged(q, kv_cache, kv_dtype, block_table, max_blocks_per_seq, seq_lens, max_seq_len, num_blocks,
                          block_size, softmax_scale, split_tokens, ws, MLA_NOALLOC_SCRATCH_BYTES, o_latent, lse, B, H,
                          stream);
}

int mla_decode_paged_fp8_mfma(const void *q, const void *kv_cache, int kv_dtype, const int32_t *block_table,
                              int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len, int num_blocks,
                              int block_size, float softmax_scale, int split_tokens, void *workspace,
                              size_t workspace_bytes, void *o_latent, float *lse, int B, int H, void *stream) {
  mla::DecodeArgs a;
  const int st = prepare_decode(DecodeMode::Paged, q, kv_cache, kv_dtype, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, num_blocks, block_size, softmax_scale, split_tokens,
                                workspace, workspace_bytes, o_latent, lse, B, H, &a);
  if (st != MLA_OK) return st;
  if (!a.kv_fp8) return MLA_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = mla::launch_decode_fp8_mfma(a, s);
  if (e != hipSuccess || a.direct) return status_of(e);
  return status_of(mla::launch_combine(a, s));
}

int mla_decode_paged_multi(const void *q, const void *kv_cache, int kv_dtype, const int32_t *block_table,
                           int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len, int num_blocks,
                           int block_size, float softmax_scale, int split_tokens, void *workspace,
                           size_t workspace_bytes, void *o_latent, float *lse, int B, int H, int q_len,
                           void *stream) {
  if (q_len < 1 || H < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (q_len > MLA_MAX_Q_LEN || static_cast<long>(H) * q_len > 2147483647L) return MLA_ERR_UNSUPPORTED;
  const int rows = H * q_len;
  mla::DecodeArgs a;
  const int st = prepare_decode(DecodeMode::Paged, q, kv_cache, kv_dtype, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, num_blocks, block_size, softmax_scale, split_tokens,
                                workspace, workspace_bytes, o_latent, lse, B, rows, &a);
  if (st != MLA_OK) return st;
  a.q_len = q_len;
  a.heads = H;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = mla::launch_decode(a, s);
  if (e != hipSuccess || a.direct) return status_of(e);
  return status_of(mla::launch_combine(a, s));
}

int mla_decode_partial(const void *q, const void *kv_cache, int kv_dtype, const int32_t *block_table,
                       int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len, int num_blocks,
                       int block_size, float softmax_scale, int split_tokens, void *workspace,
                       size_t workspace_bytes, int B, int H, void *stream) {
  if (max_seq_len <= 0) return MLA_ERR_INVALID_ARGUMENT;
  mla::DecodeArgs a;
  const int st = prepare_decode(DecodeMode::Partial, q, kv_cache, kv_dtype, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, num_blocks, block_size, softmax_scale, split_tokens,
                                workspace, workspace_bytes, nullptr, nullptr, B, H, &a);
  if (st != MLA_OK) return st;
  return status_of(mla::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int mla_decode_combine(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens, int max_seq_len,
                       int split_tokens, void *o_latent, float *lse, int B, int H, void *stream) {
  if (!aligned16(workspace) || !aligned16(seq_lens) || !aligned16(o_latent) ||
      (lse != nullptr && !aligned16(lse)) || B < 1 || H < 1 || max_seq_len <= 0 || split_tokens < 0 ||
      split_tokens % MLA_BLOCK_SIZE != 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (split_tokens > MLA_MAX_SPLIT_TOKENS) return MLA_ERR_UNSUPPORTED;
  const int split = split_tokens ? split_tokens : plan_split(B, H, max_seq_len);
  const int n_splits = (max_seq_len + split - 1) / split;
  const size_t need = workspace_for(B, H, n_splits);
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
  mla::DecodeArgs a = {};
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = H;
  a.q_len = 1;
  a.heads = H;
  a.split_tokens = split;
  a.n_splits = n_splits;
  a.o_latent = static_cast<uint16_t *>(o_latent);
  a.lse = lse;
  const size_t rows = static_cast<size_t>(B) * n_splits * H;
  a.o_part = static_cast<uint16_t *>(const_cast<void *>(workspace));
  a.lse_part = reinterpret_cast<float *>(static_cast<uint8_t *>(const_cast<void *>(workspace)) +
                                         align256(rows * MLA_D_C * sizeof(uint16_t)));
  return status_of(mla::launch_combine(a, static_cast<hipStream_t>(stream)));
}

int mla_decode_combine_absorb_out(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens,
                                  int max_seq_len, int split_tokens, const void *w_uv, void *o, void *o_latent,
                                  float *lse, int B, int H, int d_c, int d_v, void *stream) {
  if (!aligned16(workspace) || !aligned16(seq_lens) || !aligned16(w_uv) || !aligned16(o) ||
      (o_latent != nullptr && !aligned16(o_latent)) || (lse != nullptr && !aligned16(lse)) || B < 1 || H < 1 ||
      max_seq_len <= 0 || split_tokens < 0 || split_tokens % MLA_BLOCK_SIZE != 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (split_tokens > MLA_MAX_SPLIT_TOKENS || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (d_c != MLA_D_C || d_v != MLA_D_V) return MLA_ERR_UNSUPPORTED;
  const int split = split_tokens ? split_tokens : plan_split(B, H, max_seq_len);
  const int n_splits = (max_seq_len + split - 1) / split;
  const size_t need = workspace_for(B, H, n_splits);
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
  mla::CombineOutArgs a = {};
  const size_t rows = static_cast<size_t>(B) * n_splits * H;
  a.o_part = static_cast<const uint16_t *>(workspace);
  a.lse_part = reinterpret_cast<const float *>(static_cast<const uint8_t *>(workspace) +
                                               align256(rows * MLA_D_C * sizeof(uint16_t)));
  a.seq_lens = seq_lens;
  a.split_tokens = split;
  a.n_splits = n_splits;
  a.w_uv = static_cast<const uint16_t *>(w_uv);
  a.o = static_cast<uint16_t *>(o);
  a.o_latent = static_cast<uint16_t *>(o_latent);
  a.lse = lse;
  a.B = B;
  a.H = H;
  return status_of(mla::launch_combine_absorb_out(a, static_cast<hipStream_t>(stream)));
}

size_t mla_prefill_workspace_bytes(int total_tokens, int H) {
  if (total_tokens < 1 || H < 1) return 0;
  const size_t T = static_cast<size_t>(total_tokens), h = static_cast<size_t>(H);
  return align256(T * h * MLA_D_R * 2) + align256(T * MLA_D_R * 2) + 2 * align256(T * h * MLA_D_NOPE * 2);
}

int mla_prefill(const void *q_nope, const void *q_pe, const void *c_kv, const void *k_pe, const void *w_uk,
                const void *w_uv, const int32_t *cu_seqlens, int B, int total_tokens, int max_seqlen, int H,
                float softmax_scale, float rope_theta, const int32_t *block_table, int max_blocks_per_seq,
                void *kv_cache, int kv_dtype, int num_blocks, int block_size, void *o, void *workspace,
                size_t workspace_bytes, void *stream) {
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(cu_seqlens) || !aligned16(block_table) || !aligned16(kv_cache) ||
      !aligned16(o) || B < 1 || H < 1 || total_tokens < 0 || max_seqlen < 0 || max_blocks_per_seq < 1 ||
      num_blocks < 1 || !isfinite(softmax_scale) || !(rope_theta > 0.0f) || !isfinite(rope_theta))
    return MLA_ERR_INVALID_ARGUMENT;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARGUMENT;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long>(max_seqlen) > static_cast<long>(max_blocks_per_seq) * block_size)
    return MLA_ERR_INVALID_ARGUMENT;
  if (B > 65535 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (total_tokens == 0 || max_seqlen == 0) return MLA_OK;
  const size_t need = mla_prefill_workspace_bytes(total_tokens, H);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  mla::PrefillArgs a = {};
  a.q_nope = static_cast<const uint16_t *>(q_nope);
  a.q_pe = static_cast<const uint16_t *>(q_pe);
  a.c = static_cast<const uint16_t *>(c_kv);
  a.k_pe = static_cast<const uint16_t *>(k_pe);
  a.w_uk = static_cast<const uint16_t *>(w_uk);
  a.w_uv = static_cast<const uint16_t *>(w_uv);
  a.cu_seqlens = cu_seqlens;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.cache = static_cast<uint8_t *>(kv_cache);
  a.kv_fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  for (int i = 0; i < MLA_D_R / 2; ++i)
    a.inv_freq[i] = std::pow(static_cast<double>(rope_theta), -(2.0 * i) / static_cast<double>(MLA_D_R));
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.B = B;
  a.H = H;
  a.T = total_tokens;
  a.max_len = max_seqlen;
  a.o = static_cast<uint16_t *>(o);
  const size_t T = static_cast<size_t>(total_tokens), h = static_cast<size_t>(H);
  uint8_t *p = static_cast<uint8_t *>(workspace);
  a.q_rot = reinterpret_cast<uint16_t *>(p);
  p += align256(T * h * MLA_D_R * 2);
  a.k_rot = reinterpret_cast<uint16_t *>(p);
  p += align256(T * MLA_D_R * 2);
  a.k_nope = reinterpret_cast<uint16_t *>(p);
  p += align256(T * h * MLA_D_NOPE * 2);
  a.v = reinterpret_cast<uint16_t *>(p);
  return status_of(mla::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

size_t mla_prefill_chunk_workspace_bytes(int total_tokens, int total_keys, int B, int H) {
  if (total_tokens < 1 || total_keys < total_tokens || B < 1 || H < 1) return 0;
  const size_t T = static_cast<size_t>(total_tokens), K = static_cast<size_t>(total_keys),
               h = static_cast<size_t>(H);
  return align256(T * h * MLA_D_R * 2) + align256(K * MLA_D_R * 2) + 2 * align256(K * h * MLA_D_NOPE * 2) +
         align256(K * 2 * MLA_D_C * 2) +
         align256((static_cast<size_t>(B) + 1) * sizeof(int32_t));
}

int mla_prefill_chunk(const void *q_nope, const void *q_pe, const void *c_kv, const void *k_pe, const void *w_uk,
                      const void *w_uv, const int32_t *cu_seqlens, const int32_t *prefix_lens, int B,
                      int total_tokens, int max_seqlen, int total_keys, int max_prefix, int H, float softmax_scale,
                      float rope_theta, const int32_t *block_table, int max_blocks_per_seq, void *kv_cache,
                      int kv_dtype, int num_blocks, int block_size, void *o, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(cu_seqlens) || !aligned16(prefix_lens) || !aligned16(block_table) ||
      !aligned16(kv_cache) || !aligned16(o) || B < 1 || H < 1 || total_tokens < 0 || max_seqlen < 0 ||
      max_prefix < 0 || total_keys < total_tokens || max_blocks_per_seq < 1 || num_blocks < 1 ||
      !isfinite(softmax_scale) || !(rope_theta > 0.0f) || !isfinite(rope_theta))
    return MLA_ERR_INVALID_ARGUMENT;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARGUMENT;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  const long cap = static_cast<long>(max_blocks_per_seq) * block_size;
  if (max_prefix > cap || max_seqlen > cap) return MLA_ERR_INVALID_ARGUMENT;
  if (B > 65535 || H > 65535 || total_keys > 2147483647 / MLA_D_C) return MLA_ERR_UNSUPPORTED;
  if (total_tokens == 0 || max_seqlen == 0) return MLA_OK;
  const size_t need = mla_prefill_chunk_workspace_bytes(total_tokens, total_keys, B, H);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  mla::PrefillArgs a = {};
  a.q_nope = static_cast<const uint16_t *>(q_nope);
  a.q_pe = static_cast<const uint16_t *>(q_pe);
  a.c = static_cast<const uint16_t *>(c_kv);
  a.k_pe = static_cast<const uint16_t *>(k_pe);
  a.w_uk = static_cast<const uint16_t *>(w_uk);
  a.w_uv = static_cast<const uint16_t *>(w_uv);
  a.cu_seqlens = cu_seqlens;
  a.prefix_lens = prefix_lens;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.cache = static_cast<uint8_t *>(kv_cache);
  a.kv_fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  for (int i = 0; i < MLA_D_R / 2; ++i)
    a.inv_freq[i] = std::pow(static_cast<double>(rope_theta), -(2.0 * i) / static_cast<double>(MLA_D_R));
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.B = B;
  a.H = H;
  a.T = total_tokens;
  a.max_len = max_seqlen;
  a.T_keys = total_keys;
  a.max_prefix = max_prefix;
  a.o = static_cast<uint16_t *>(o);
  const size_t T = static_cast<size_t>(total_tokens), K = static_cast<size_t>(total_keys),
               h = static_cast<size_t>(H);
  uint8_t *p = static_cast<uint8_t *>(workspace);
  a.q_rot = reinterpret_cast<uint16_t *>(p);
  p += align256(T * h * MLA_D_R * 2);
  a.k_rot = reinterpret_cast<uint16_t *>(p);
  p += align256(K * MLA_D_R * 2);
  a.k_nope = reinterpret_cast<uint16_t *>(p);
  p += align256(K * h * MLA_D_NOPE * 2);
  a.v = reinterpret_cast<uint16_t *>(p);
  p += align256(K * h * MLA_D_NOPE * 2);
  a.c_gather = reinterpret_cast<uint16_t *>(p);
  p += align256(K * 2 * MLA_D_C * 2);
  a.cu_keys_ws = reinterpret_cast<int32_t *>(p);
  return status_of(mla::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int mla_absorb_out(const void *o_latent, const void *w_uv, void *o, int B, int H, int d_c, int d_v,
                   void *stream) {
  if (!aligned16(o_latent) || !aligned16(w_uv) || !aligned16(o) || B < 1 || H < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if (B > 65535 * 32 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (d_c != MLA_D_C || d_v != MLA_D_V) return MLA_ERR_UNSUPPORTED;
  return status_of(mla::launch_absorb_out(static_cast<const uint16_t *>(o_latent),
                                          static_cast<const uint16_t *>(w_uv), static_cast<uint16_t *>(o), B, H,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
