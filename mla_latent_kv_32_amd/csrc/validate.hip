// Check of the device-resident paging values that the decode, append and
// prefill calls trust (sequence lengths and block-table page ids).  The
// paged cache maps token t of sequence b to page block_table[b][t / 64],
// slot t % 64; a length past the caller's bound or a page id outside the
// pool would send those calls outside their buffers, so this call lets a
// caller check its tables before handing them over.
//
// One workgroup of 1024 threads: wave w takes sequences b = w, w + 16, ...;
// its lanes scan the pages in use, a ballot flags the sequence, and the
// per-wave counts and smallest flagged b are reduced through LDS.  No atomics
// and no memset: the two results are written by thread 0 at the end, so the
// call is safe inside a captured graph and gives the same result every time.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int VT_THREADS = 1024;
constexpr int VT_WAVES = VT_THREADS / 64;

__global__ __launch_bounds__(VT_THREADS) void validate_paging_kernel(ValidateArgs a) {
  __shared__ int bad_w[VT_WAVES], first_w[VT_WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int bad = 0, first = INT_MAX;
  for (int b = wave; b < a.B; b += VT_WAVES) {
    const int S = a.seq_lens[b];
    bool broken = S < 0 || S > a.max_seq_len || S > a.max_blocks * PAGE;
    if (!broken) {
      const int pages = (S + PAGE - 1) / PAGE;
      const int32_t *row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
      bool lane_bad = false;
      for (int j = lane; j < pages; j += 64) {
        const int p = row[j];
        lane_bad = lane_bad || p < 0 || p >= a.num_blocks;
      }
      broken = __ballot(lane_bad) != 0;
    }
    if (broken) {
      ++bad;
      first = min(first, b);
    }
  }
  if (lane == 0) {
    bad_w[wave] = bad;
    first_w[wave] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0, f = INT_MAX;
    for (int w = 0; w < VT_WAVES; ++w) {
      n += bad_w[w];
      f = min(f, first_w[w]);
    }
    *a.bad = n;
    if (a.first_bad) *a.first_bad = n > 0 ? f : -1;
  }
}

}  // namespace

hipError_t launch_validate_paging(const ValidateArgs &a, hipStream_t stream) {
  validate_paging_kernel<<<1, VT_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
