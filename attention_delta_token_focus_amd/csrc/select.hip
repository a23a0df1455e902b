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

// Sum over heads of one block position for both layers, heads in
// ascending order; eight heads' loads are issued before any is added.
__device__ __forceinline__ void head_sums(const float* __restrict__ i0,
                                          const float* __restrict__ i1, int Hq,
                                          int B, int j, float& a0, float& a1) {
  a0 = 0.f;
  a1 = 0.f;
  int h = 0;
  for (; h + 8 <= Hq; h += 8) {
    float x0[8], x1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      x0[u] = i0[(h + u) * B + j];
      x1[u] = i1[(h + u) * B + j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 += x0[u];
      a1 += x1[u];
    }
  }
  for (; h < Hq; ++h) {
    a0 += i0[h * B + j];
    a1 += i1[h * B + j];
  }
}

// Bitonic sort of NS*64 slots (slot i = lane + 64*s) into descending
// order, with lane shuffles; slot pairs of one lane compare in registers.
template <int NS>
__device__ __forceinline__ void bitonic_desc(uint64_t (&key)[2], int lane) {
  constexpr int N = NS * 64;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int st = k >> 1; st > 0; st >>= 1) {
      if (st == 64) {
        // only when k == 128: descending merge of the two slots
        const uint64_t hi = key[0] > key[1] ? key[0] : key[1];
        const uint64_t lo = key[0] > key[1] ? key[1] : key[0];
        key[0] = hi;
        key[1] = lo;
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int i = lane + 64 * s;
          const uint64_t other = __shfl_xor(key[s], st);
          const bool take_max = ((i & st) == 0) == ((i & k) == 0);
          const uint64_t mx = key[s] > other ? key[s] : other;
          const uint64_t mn = key[s] > other ? other : key[s];
          key[s] = take_max ? mx : mn;
        }
      }
    }
  }
}

// Head mean, MaxPool1D, delta and top-K of sequence b by one wavefront
// (lane l holds block positions l and l + 64). Writes dI and keep; returns
// in `flags` the keep flag of every position, and the number kept.
//
// With `masked` given, only positions with masked[j] != 0 are candidates
// (at most K_b of them), and the retained set grows by the structural
// constraints selected in `rules`: each candidate's predecessor
// (kKeepPredecessor) and every masked position left of the rightmost
// candidate (kKeepMaskedPrefix). `cand`, when given, receives the
// candidate flags. Without a mask and rules this is plain top-K.
//
// With `yield_hist` given, the budget is not k_keep[b] but the dynamic
// budget K = min(|M|, max(1, ceil(alpha * max(y_b, n)))), n = the masked
// positions whose delta exceeds mean + population std of the deltas over
// the masked positions (0 if none is masked); it is written to k_used[b]
// when k_used is given. Sums are fixed-order wavefront reductions in fp32.
constexpr int kKeepPredecessor = 1;
constexpr int kKeepMaskedPrefix = 2;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int NS>
__device__ __forceinline__ void delta_topk_wave(
    int b, int B, int Hq, int radius, const float* __restrict__ imp0,
    const float* __restrict__ imp1, const uint8_t* __restrict__ masked,
    int rules, const int32_t* __restrict__ k_keep,
    const float* __restrict__ yield_hist, float alpha,
    int32_t* __restrict__ k_used, uint8_t* __restrict__ keep,
    uint8_t* __restrict__ cand, float* __restrict__ dI, float (*mean)[128],
    uint8_t* flags, int& n_kept) {
  const int lane = threadIdx.x;
  const float inv_h = 1.0f / (float)Hq;
  const float* i0 = imp0 + (size_t)b * Hq * B;
  const float* i1 = imp1 + (size_t)b * Hq * B;
  int kb = yield_hist != nullptr ? 0 : min(max(k_keep[b], 0), B);
  bool elig[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    elig[s] = j < B && (masked == nullptr || masked[(size_t)b * B + j] != 0);
    if (j < B) {
      float a0, a1;
      head_sums(i0, i1, Hq, B, j, a0, a1);
      mean[0][j] = a0 * inv_h;
      mean[1][j] = a1 * inv_h;
      flags[j] = 0;
    }
  }
  __syncthreads();

  // Sort keys: (order code of dI) << 32 | (~j), so that larger dI comes
  // first and, for equal dI, the lower position. Empty slots and positions
  // that are not candidates are 0, below every real key (~j is never 0).
  uint64_t key[2] = {0, 0};
  float dv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    dv[s] = 0.f;
    if (j < B) {
      const int lo = max(0, j - radius), hi = min(B - 1, j + radius);
      float m0 = -INFINITY, m1 = -INFINITY;
      for (int t = lo; t <= hi; ++t) {
        m0 = fmaxf(m0, mean[0][t]);
        m1 = fmaxf(m1, mean[1][t]);
      }
      const float d = m1 - m0;
      dv[s] = d;
      if (dI != nullptr) dI[(size_t)b * B + j] = d;
      if (elig[s]) key[s] = ((uint64_t)order_code(d) << 32) | (uint32_t)(0xFFFFFFFFu - j);
    }
  }
  if (yield_hist != nullptr) {
    // dynamic budget from the masked positions' delta statistics
    float sum = 0.f;
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (elig[s]) {
        sum += dv[s];
        ++cnt;
      }
    }
    sum = wave_sum(sum);
    cnt = wave_sum(cnt);
    if (cnt > 0) {
      const float mu = sum / (float)cnt;
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (elig[s]) ss += (dv[s] - mu) * (dv[s] - mu);
      }
      ss = wave_sum(ss);
      const float thr = mu + __builtin_sqrtf(ss / (float)cnt);
      int above = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) above += (elig[s] && dv[s] > thr) ? 1 : 0;
      above = wave_sum(above);
      const float want = __builtin_ceilf(alpha * fmaxf(yield_hist[b], (float)above));
      kb = min(cnt, max(1, (int)fminf(want, (float)B)));
    }
    if (k_used != nullptr && lane == 0) k_used[b] = kb;
  }
  bitonic_desc<NS>(key, lane);
  // Candidates: the first K_b ranks that hold a real key.
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int p = lane + 64 * s;  // rank in descending order
    if (key[s] != 0 && p < kb) flags[(int)(0xFFFFFFFFu - (uint32_t)key[s])] = 1;
  }
  __syncthreads();

  // Retained set from the candidate flags, position by position.
  int rightmost = -1;
  if (rules & kKeepMaskedPrefix) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = lane + 64 * s;
      if (j < B && flags[j] != 0) rightmost = max(rightmost, j);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rightmost = max(rightmost, __shfl_xor(rightmost, o));
  }
  uint8_t kept[NS];
  int cnt = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    kept[s] = 0;
    if (j < B) {
      const bool c = flags[j] != 0;
      bool k = c;
      if ((rules & kKeepPredecessor) && j + 1 < B && flags[j + 1] != 0) k = true;
      if (elig[s] && j < rightmost) k = true;
      kept[s] = k ? 1 : 0;
      cnt += kept[s];
      keep[(size_t)b * B + j] = kept[s];
      if (cand != nullptr) cand[(size_t)b * B + j] = c ? 1 : 0;
    }
  }
  __syncthreads();  // every lane has read the candidate flags
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    if (j < B) flags[j] = kept[s];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  n_kept = cnt;
  __syncthreads();
}

// One wavefront per sequence.
template <int NS>
__global__ void __launch_bounds__(64) delta_topk_kernel(
    int B, int Hq, int radius, const float* __restrict__ imp0,
    const float* __restrict__ imp1, const uint8_t* __restrict__ masked,
    int rules, const int32_t* __restrict__ k_keep,
    const float* __restrict__ yield_hist, float alpha, int32_t* __restrict__ k_used,
    uint8_t* __restrict__ keep, uint8_t* __restrict__ cand, float* __restrict__ dI) {
  __shared__ float mean[2][128];
  __shared__ uint8_t flags[128];
  int n_kept;
  delta_topk_wave<NS>(blockIdx.x, B, Hq, radius, imp0, imp1, masked, rules, k_keep,
                      yield_hist, alpha, k_used, keep, cand, dI, mean, flags, n_kept);
}

// Delta/top-K and compaction in one launch, one wavefront per sequence.
// The offset of sequence b is the sum of the clamped budgets of the
// sequences before it (top-K keeps exactly that many), summed by the wave
// itself; kept positions are ranked in ascending order with a ballot and
// mbcnt over the keep flags.
template <int NS>
__global__ void __launch_bounds__(64) select_kernel(
    int batch, int B, int Hq, int radius, const float* __restrict__ imp0,
    const float* __restrict__ imp1, const int32_t* __restrict__ k_keep,
    uint8_t* __restrict__ keep, float* __restrict__ dI,
    int32_t* __restrict__ idx, int32_t* __restrict__ cu_ret) {
  __shared__ float mean[2][128];
  __shared__ uint8_t flags[128];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int off = 0;
  // unrolled so that several budget loads are in flight (the host sends
  // batches above kFusedSelectMax to the two-launch path instead)
#pragma unroll 8
  for (int c = 0; c < b; c += 64) {
    const int i = c + lane;
    if (i < b) off += min(max(k_keep[i], 0), B);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o);
  int kb;
  delta_topk_wave<NS>(b, B, Hq, radius, imp0, imp1, nullptr, 0, k_keep, nullptr,
                      0.f, nullptr, keep, nullptr, dI, mean, flags, kb);
  int base = off;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    const bool kept = j < B && flags[j] != 0;
    const uint64_t m = __ballot(kept);
    const int rank = __builtin_amdgcn_mbcnt_hi(
        (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (kept) idx[base + rank] = b * B + j;
    base += __popcll(m);
  }
  if (lane == 0) {
    cu_ret[b] = off;
    if (b == batch - 1) cu_ret[batch] = off + kb;
  }
}

// One workgroup of 1024 threads walks the batch in chunks of 1024
// sequences. Thread t owns sequence base + t: it counts its kept bytes
// (16-byte loads when rows are 16-byte aligned) and the workgroup takes an
// exclusive scan of the counts (wavefront shuffles + LDS). Then each
// wavefront writes the kept indices of one sequence at a time, lane j for
// position j (its rank among the kept positions from a ballot), so that the
// indices of a sequence leave in one contiguous store, ascending.
template <bool VEC>
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
    const bool live = b < batch;
    int cnt = 0;
    if constexpr (VEC) {
      const int nv = B >> 4;
      const u32x4* kp = reinterpret_cast<const u32x4*>(keep + (size_t)b * B);
      u32x4 row[8];  // up to 128 keep bytes
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        row[v] = (live && v < nv) ? kp[v] : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = row[v][w];
          // bytes are 0/1 flags; count the non-zero ones
          const uint32_t nz = ((x | (x >> 1) | (x >> 2) | (x >> 3) | (x >> 4) |
                                (x >> 5) | (x >> 6) | (x >> 7)) & 0x01010101u);
          cnt += __popc(nz);
        }
      }
    } else if (live) {
      const uint8_t* kp = keep + (size_t)b * B;
#pragma unroll 8
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
    const int off = carry + (wave ? wsum[wave - 1] : 0) + x - cnt;
    const int chunk_total = wsum[15];
    offs[tid] = off;
    if (live) cu_ret[b] = off;
    __syncthreads();
    const int nseq = min(1024, batch - base);
    for (int s = wave; s < nseq; s += 16) {
      const int bs = base + s;
      const uint8_t* kp = keep + (size_t)bs * B;
      int o = offs[s];
      for (int j0 = 0; j0 < B; j0 += 64) {
        const int j = j0 + lane;
        const bool k = j < B && kp[j] != 0;
        const uint64_t m = __ballot(k);
        const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (k) idx[o + r] = bs * B + j;
        o += __popcll(m);
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
                             const uint8_t* masked, int rules,
                             const int32_t* k_keep, const float* yield_hist,
                             float alpha, int32_t* k_used, uint8_t* keep,
                             uint8_t* cand, float* dI, hipStream_t s) {
  if (B <= 64) {
    hipLaunchKernelGGL(delta_topk_kernel<1>, dim3(batch), dim3(64), 0, s, B, Hq,
                       (pool_k - 1) / 2, imp0, imp1, masked, rules, k_keep, yield_hist,
                       alpha, k_used, keep, cand, dI);
  } else {
    hipLaunchKernelGGL(delta_topk_kernel<2>, dim3(batch), dim3(64), 0, s, B, Hq,
                       (pool_k - 1) / 2, imp0, imp1, masked, rules, k_keep, yield_hist,
                       alpha, k_used, keep, cand, dI);
  }
  return hipGetLastError();
}

hipError_t launch_select(int batch, int B, int Hq, int pool_k,
                         const float* imp0, const float* imp1,
                         const int32_t* k_keep, uint8_t* keep, float* dI,
                         int32_t* idx, int32_t* cu_ret, hipStream_t s) {
  // Each wavefront of the fused kernel sums the budgets of all earlier
  // sequences (O(batch) per sequence); past kFusedSelectMax sequences the
  // two launches (O(batch) in total) are faster, with the same outputs.
  if (batch > kFusedSelectMax) {
    const hipError_t e = launch_delta_topk(batch, B, Hq, pool_k, imp0, imp1, nullptr, 0,
                                           k_keep, nullptr, 0.f, nullptr, keep, nullptr,
                                           dI, s);
    if (e != hipSuccess) return e;
    return launch_compact(batch, B, keep, idx, cu_ret, s);
  }
  if (B <= 64) {
    hipLaunchKernelGGL(select_kernel<1>, dim3(batch), dim3(64), 0, s, batch, B, Hq,
                       (pool_k - 1) / 2, imp0, imp1, k_keep, keep, dI, idx, cu_ret);
  } else {
    hipLaunchKernelGGL(select_kernel<2>, dim3(batch), dim3(64), 0, s, batch, B, Hq,
                       (pool_k - 1) / 2, imp0, imp1, k_keep, keep, dI, idx, cu_ret);
  }
  return hipGetLastError();
}

hipError_t launch_compact(int batch, int B, const uint8_t* keep, int32_t* idx,
                          int32_t* cu_ret, hipStream_t s) {
  // 16-byte row loads need 16-byte aligned rows (B a multiple of 16).
  if (B % 16 == 0 && (reinterpret_cast<uintptr_t>(keep) & 15u) == 0) {
    hipLaunchKernelGGL(compact_kernel<true>, dim3(1), dim3(1024), 0, s, batch, B,
                       keep, idx, cu_ret);
  } else {
    hipLaunchKernelGGL(compact_kernel<false>, dim3(1), dim3(1024), 0, s, batch, B,
                       keep, idx, cu_ret);
  }
  return hipGetLastError();
}

}  // namespace focus
