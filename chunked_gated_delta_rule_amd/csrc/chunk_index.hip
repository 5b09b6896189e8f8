// Device-built chunk-index table (FLA issue 1155, "[RFC] Graph capture support
// for prefill and training", section "Core design"): a fixed [nt_max, 2] table
// filled by a searchsorted over the per-sequence chunk offsets, with the
// sentinel (-1, -1) in every unused slot, so that chunk-sized grids can be
// launched at the static size nt_max and the host never reads cu_seqlens.
//
// One work-group of 1024 threads: per-sequence chunk counts, a block-wide
// exclusive scan into LDS, then one binary search per slot.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kIndexThreads = 1024;
constexpr int kMaxSeqs = 16384;  // (n_max + 1) offsets live in LDS

__global__ __launch_bounds__(kIndexThreads) void chunk_index_kernel(const int32_t *__restrict__ cu,
                                                                    int32_t n_max, int32_t nt_max,
                                                                    int32_t t_max,
                                                                    int32_t *__restrict__ table) {
  __shared__ int32_t co[kMaxSeqs + 1];
  __shared__ int32_t part[kIndexThreads];
  const int tid = threadIdx.x;
  const int per = (n_max + kIndexThreads - 1) / kIndexThreads;
  const int s0 = min(tid * per, n_max);
  const int s1 = min(s0 + per, n_max);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += seq_chunks(cu, s, t_max);
  part[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread totals.
  for (int off = 1; off < kIndexThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - local;  // exclusive offset of this thread's segment
  for (int s = s0; s < s1; ++s) {
    co[s] = run;
    run += seq_chunks(cu, s, t_max);
  }
  if (tid == kIndexThreads - 1) co[n_max] = part[kIndexThreads - 1];
  __syncthreads();
  const int total = co[n_max];
  for (int j = tid; j < nt_max; j += kIndexThreads) {
    int2 e = make_int2(-1, -1);
    if (j < total) {
      // last s with co[s] <= j (upper bound minus one); skips empty sequences
      int lo = 0, hi = n_max;  // invariant: co[lo] <= j < co[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (co[mid] <= j) lo = mid; else hi = mid;
      }
      e = make_int2(lo, j - co[lo]);
    }
    reinterpret_cast<int2 *>(table)[j] = e;
  }
}

}  // namespace

hipError_t launch_chunk_index(const int32_t *cu_seqlens, int32_t n_max, int32_t nt_max,
                              int32_t t_max, int32_t *table, hipStream_t stream, KernelEvents ev) {
  if (n_max > kMaxSeqs) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(kIndexThreads), 0, stream, ev.start,
                        ev.stop, 0, cu_seqlens, n_max, nt_max, t_max, table);
  return hipGetLastError();
}

}  // namespace gdn
