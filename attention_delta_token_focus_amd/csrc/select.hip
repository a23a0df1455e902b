// Importance delta, per-sequence top-K and stream compaction for gfx950.
//
// What is computed (Pith review page of "FOCUS: DLLMs Know How to Tame
// Their Compute Bound", arXiv 2601.23278, section "What carries the
// argument"; MaxPool kernel size in its Free-Parameter Ledger, Eq. 15; Eq. 3
// for the delta): per sequence, the per-head importances of layers 0 and 1
// are averaged over heads, max-filtered over block positions, subtracted
// (layer 1 minus layer 0), and the K_b positions with the largest delta are
// kept; the kept positions are then compacted into one index list with
// per-sequence offsets.
#include "focus_internal.hpp"

namespace focus {
namespace {

// Monotone map of a float onto uint32 (larger float -> larger code); -0 is
// folded onto +0 first so that equal values share a code.
__device__ __forceinline__ uint32_t order_code(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wavefront per sequence. Lane l holds block positions l and l + 64.
__global__ void __launch_bounds__(64) delta_topk_kernel(
    int B, int Hq, int radius, const float* __restrict__ imp0,
    const float* __restrict__ imp1, const int32_t* __restrict__ k_keep,
    uint8_t* __restrict__ keep, float* __restrict__ dI) {
  __shared__ float mean[2][128];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float inv_h = 1.0f / (float)Hq;
  const float* i0 = imp0 + (size_t)b * Hq * B;
  const float* i1 = imp1 + (size_t)b * Hq * B;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + 64 * s;
    if (j < B) {
      float a0 = 0.f, a1 = 0.f;
      for (int h = 0; h < Hq; ++h) {  // fixed head order
        a0 += i0[h * B + j];
        a1 += i1[h * B + j];
      }
      mean[0][j] = a0 * inv_h;
      mean[1][j] = a1 * inv_h;
    }
  }
  __syncthreads();

  // Sort keys: (order code of dI) << 32 | (~j), so that larger dI comes
  // first and, for equal dI, the lower position. Empty slots are 0, which
  // is below every real key.
  uint64_t key[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + 64 * s;
    key[s] = 0;
    if (j < B) {
      const int lo = max(0, j - radius), hi = min(B - 1, j + radius);
      float m0 = -INFINITY, m1 = -INFINITY;
      for (int t = lo; t <= hi; ++t) {
        m0 = fmaxf(m0, mean[0][t]);
        m1 = fmaxf(m1, mean[1][t]);
      }
      const float d = m1 - m0;
      if (dI != nullptr) dI[(size_t)b * B + j] = d;
      key[s] = ((uint64_t)order_code(d) << 32) | (uint32_t)(0xFFFFFFFFu - j);
    }
  }

  // Bitonic sort of the 128 slots (index i = lane + 64*slot) into
  // descending order.
  for (int k = 2; k <= 128; k <<= 1) {
    for (int st = k >> 1; st > 0; st >>= 1) {
      if (st == 64) {
        // partner is the other slot of the same lane; k == 128: descending
        const uint64_t hi = key[0] > key[1] ? key[0] : key[1];
        const uint64_t lo = key[0] > key[1] ? key[1] : key[0];
        key[0] = hi;
        key[1] = lo;
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int i = lane + 64 * s;
          const uint64_t other = __shfl_xor(key[s], st);
          const bool lower = (i & st) == 0;
          const bool desc = (i & k) == 0;
          const bool take_max = (lower == desc);
          const uint64_t mx = key[s] > other ? key[s] : other;
          const uint64_t mn = key[s] > other ? other : key[s];
          key[s] = take_max ? mx : mn;
        }
      }
    }
  }

  const int kb = min(max(k_keep[b], 0), B);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int p = lane + 64 * s;  // rank in descending order
    if (key[s] != 0) {
      const int j = (int)(0xFFFFFFFFu - (uint32_t)key[s]);
      keep[(size_t)b * B + j] = p < kb ? 1 : 0;
    }
  }
}

// One workgroup of 1024 threads walks the batch in chunks of 1024
// sequences: per-sequence counts, a workgroup exclusive scan (wavefront
// shuffles + LDS), then per sequence a ballot over the keep bytes whose
// mbcnt rank places each kept index.
__global__ void __launch_bounds__(1024) compact_kernel(
    int batch, int B, const uint8_t* __restrict__ keep,
    int32_t* __restrict__ idx, int32_t* __restrict__ cu_ret) {
  __shared__ int wsum[16];
  __shared__ int offs[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < batch; base += 1024) {
    const int b = base + tid;
    int cnt = 0;
    if (b < batch) {
      const uint8_t* kp = keep + (size_t)b * B;
      for (int j = 0; j < B; ++j) cnt += kp[j] != 0;
    }
    int x = cnt;  // inclusive scan within the wavefront
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const int y = __shfl_up(w, o);
        if (lane >= o) w += y;
      }
      if (lane < 16) wsum[lane] = w;
    }
    __syncthreads();
    const int excl = carry + (wave ? wsum[wave - 1] : 0) + x - cnt;
    if (b < batch) cu_ret[b] = excl;
    offs[tid] = excl;
    const int chunk_total = wsum[15];
    __syncthreads();
    for (int sb = wave * 64; sb < wave * 64 + 64; ++sb) {
      const int bb = base + sb;
      if (bb >= batch) break;
      int off = offs[sb];
      for (int j0 = 0; j0 < B; j0 += 64) {
        const int j = j0 + lane;
        const bool kept = j < B && keep[(size_t)bb * B + j] != 0;
        const uint64_t m = __ballot(kept);
        const int rank = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (kept) idx[off + rank] = bb * B + j;
        off += __popcll(m);
      }
    }
    carry += chunk_total;
    __syncthreads();
  }
  if (tid == 0) cu_ret[batch] = carry;
}

}  // namespace

hipError_t launch_delta_topk(int batch, int B, int Hq, int pool_k,
                             const float* imp0, const float* imp1,
                             const int32_t* k_keep, uint8_t* keep, float* dI,
                             hipStream_t s) {
  hipLaunchKernelGGL(delta_topk_kernel, dim3(batch), dim3(64), 0, s, B, Hq,
                     (pool_k - 1) / 2, imp0, imp1, k_keep, keep, dI);
  return hipGetLastError();
}

hipError_t launch_compact(int batch, int B, const uint8_t* keep, int32_t* idx,
                          int32_t* cu_ret, hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, s, batch, B, keep,
                     idx, cu_ret);
  return hipGetLastError();
}

}  // namespace focus
