// Visiting order of the sequences for one step's attention calls: the
// longest prefix first. The attention work of a sequence grows with its
// prefix length; handing the longest ones out first keeps every compute
// unit busy until the end of a launch (longest-processing-time-first
// list scheduling).
#include <limits.h>

#include "focus_internal.hpp"

namespace focus {
namespace {

// Longest-prefix-first visiting order of the sequences; equal lengths keep
// the lower sequence first. Up to 256 sequences: one 1024-thread block;
// the four threads i, i + 256, i + 512, i + 768 each count, over a quarter
// of the lengths (broadcast from LDS, four per read), the sequences that go
// before sequence i; the four counts add up to its rank. Up to kMaxSort:
// bitonic sort of (P_b, ~b) in LDS by 1024 threads. Larger batches keep
// their natural order.
constexpr int kMaxSort = 16384;  // 64-bit keys: 128 KiB of the 160 KiB of LDS
constexpr int kRankMax = 256;

__global__ void __launch_bounds__(1024) lpt_rank_kernel(
    int batch, const int32_t* __restrict__ cu_prefix, int32_t* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) int len[kRankMax];
  __shared__ int part[4][kRankMax];
  const int tid = threadIdx.x;
  const int i = tid & (kRankMax - 1);       // the sequence ranked
  const int q = tid >> 8;                   // the quarter of the lengths
  const int n4 = (batch + 3) & ~3;
  // Padding up to a multiple of four never goes before a sequence, whatever
  // its length (a non-monotone cu_prefix can make a length negative): the
  // rank of sequence i counts only real sequences, so the ranks are a
  // permutation of 0 .. batch-1 and every store below stays inside order[].
  if (tid < n4) len[tid] = tid < batch ? cu_prefix[tid + 1] - cu_prefix[tid] : INT_MIN;
  __syncthreads();
  int rank = 0;
  if (i < batch) {
    const int mine = len[i];
    const int j1 = min(n4, 64 * (q + 1));
    // unrolled so that several LDS reads are in flight, not one at a time
#pragma unroll 4
    for (int j = 64 * q; j < j1; j += 4) {
      const int4 l4 = *reinterpret_cast<const int4*>(len + j);
      rank += (l4.x > mine) + (l4.x == mine && j < i);
      rank += (l4.y > mine) + (l4.y == mine && j + 1 < i);
      rank += (l4.z > mine) + (l4.z == mine && j + 2 < i);
      rank += (l4.w > mine) + (l4.w == mine && j + 3 < i);
    }
  }
  part[q][i] = rank;
  __syncthreads();
  if (tid < batch) order[part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid]] = tid;
}

__global__ void __launch_bounds__(1024) lpt_sort_kernel(
    int batch, const int32_t* __restrict__ cu_prefix, int32_t* __restrict__ order) {
  __shared__ uint64_t key[kMaxSort];
  const int tid = threadIdx.x;
  if (batch > kMaxSort) {
    for (int i = tid; i < batch; i += 1024) order[i] = i;
    return;
  }
  int n2 = 1;
  while (n2 < batch) n2 <<= 1;
  for (int i = tid; i < n2; i += 1024) {
    uint64_t k = 0;  // padding: below every real key
    if (i < batch) {
      // signed length with the sign bit flipped: unsigned order = signed order
      const uint32_t len = (uint32_t)(cu_prefix[i + 1] - cu_prefix[i]) ^ 0x80000000u;
      k = ((uint64_t)len << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t x = key[i], y = key[p];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            key[i] = y;
            key[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < batch; i += 1024)
    order[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)key[i]);
}

}  // namespace

size_t order_workspace_bytes(int batch) {
  return ((size_t)batch * sizeof(int32_t) + 255) & ~(size_t)255;
}

hipError_t launch_lpt_order(int batch, const int32_t* cu_prefix, int32_t* order,
                            hipStream_t s) {
  if (batch <= kRankMax) {
    hipLaunchKernelGGL(lpt_rank_kernel, dim3(1), dim3(1024), 0, s, batch, cu_prefix, order);
  } else {
    hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(1024), 0, s, batch, cu_prefix, order);
  }
  return hipGetLastError();
}

}  // namespace focus
