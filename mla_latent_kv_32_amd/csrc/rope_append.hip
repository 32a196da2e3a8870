// Decoupled RoPE for the new token and its append to the paged latent cache
// (the arithmetic lives in rope.h; this file launches it on its own).
#include "rope.h"

namespace mla {
namespace {

// grid (B, ceil(H / 16)): each workgroup rotates the query pairs of 16 heads
// of one sequence (2 pairs per thread); workgroup (b, 0) also appends the row.
constexpr int HEADS_PER_WG = 16;

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  __shared__ float cs[DR / 2], sn[DR / 2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = a.seq_lens[b];
  if (tid < DR / 2) rope_cos_sin(a, rope_position(S), tid, cs[tid], sn[tid]);
  __syncthreads();

  const int h0 = blockIdx.y * HEADS_PER_WG;
  for (int idx = tid; idx < HEADS_PER_WG * (DR / 2); idx += blockDim.x) {
    const int h = h0 + idx / (DR / 2), i = idx % (DR / 2);
    if (h >= a.H) break;
    rope_query_pair(a, b, h, i, cs[i], sn[i]);
  }
  if (blockIdx.y != 0 || S <= 0) return;
  append_row(a, b, S, tid, cs, sn);
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs &a, hipStream_t stream) {
  rope_append_kernel<<<dim3(a.B, (a.H + HEADS_PER_WG - 1) / HEADS_PER_WG), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
