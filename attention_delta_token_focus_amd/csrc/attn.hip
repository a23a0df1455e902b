// Block attention with importance, and retained-query attention, for
// gfx950 (MI355X).
//
// What is computed (Pith review page of "FOCUS: DLLMs Know How to Tame
// Their Compute Bound", arXiv 2601.23278, section "What carries the
// argument"; row softmax as read in its Referee Report on Eq. 2): for each
// sequence and query head, every block query attends to the P_b prefix keys
// and to the block keys; the importance of block token j is the column sum
// of the softmax weights it receives from the block queries. The retained
// mode ("The pith": later layers run on the retained tokens only) attends
// gathered retained queries to the prefix plus the retained block keys.
//
// Design (MI355X-first):
//  * One workgroup per (sequence, KV head, chunk of query heads): the G
//    query heads sharing a KV head are stacked as up to 128 query rows, so
//    every K/V byte read from HBM feeds G*B rows of MFMA work.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query row for the
//    whole kernel (row max and row sum need only one cross-half exchange),
//    and the probabilities leave the accumulator already in the B-operand
//    layout of O^T = V^T P^T.
//  * K/V tiles of 64 keys are streamed HBM -> registers -> LDS, double
//    buffered, one barrier per tile. V is transposed on its way into LDS
//    with an XOR swizzle that keeps both the transposing writes and the
//    MFMA-operand reads free of bank conflicts.
//  * Online softmax in the log2 domain, scale applied in fp32 after the
//    MFMA. Importance is a second pass over the block keys only: once the
//    final row lse is known, exp2(s - lse) for the block columns is
//    recomputed from the block K tile (kept out of the main loop so the
//    importance needs the exact lse), written to LDS, and summed down the
//    columns in a fixed order (no atomics, bitwise deterministic).
#include "focus_internal.hpp"

namespace focus {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static constexpr int KM = 16;  // reduction depth of one instruction
  static constexpr int KL = 8;   // reduction values held by one lane
  typedef bf16x8 frag;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KM = 2;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// LDS geometry for one element type and head dim.
template <typename T, int D> struct Geo {
  static constexpr int ES = sizeof(T);
  static constexpr int CE = 16 / ES;               // elements per 16 B chunk
  static constexpr int CPR = D / CE;               // chunks per key row
  static constexpr int KPT = kTile * CPR / kThreads;  // keys per loader thread
  static constexpr int KPITCH = D + CE;            // K row pitch (elements)
  static constexpr bool SWZ = (ES == 2 && D == 128);
  static constexpr int VPITCH = SWZ ? kTile : kTile + CE;  // V^T row pitch
  static constexpr int KBUF = kTile * KPITCH * ES;  // bytes per K buffer
  static constexpr int VBUF = D * VPITCH * ES;      // bytes per V^T buffer
  static constexpr int PPITCH = kTile + 4;          // fp32 probability pitch
  static constexpr int PBUF = kRowsPerWG * PPITCH * 4;
  static constexpr int MAIN = 2 * KBUF + 2 * VBUF;
  static constexpr int SMEM = MAIN > KBUF + PBUF ? MAIN : KBUF + PBUF;
  static_assert(KPT >= 1 && KPT * kThreads == kTile * CPR, "loader shape");
};

// Element offset of V^T[d][key] inside one V^T buffer. For bf16 with
// d = 128 the 4-key groups are XOR-swizzled by a function of d that makes
// (a) the 16 lanes writing rows d = 8c + e (c = 0..15, fixed e) and
// (b) the 16 lanes reading rows d = 32t + m (m = 0..15) hit distinct
// 8-byte bank pairs.
template <typename T, int D>
__device__ __forceinline__ int vt_off(int d, int key) {
  using G = Geo<T, D>;
  if constexpr (G::SWZ) {
    const int sw = ((d >> 3) ^ ((d & 7) << 1)) & 15;
    return d * kTile + ((((key >> 2) ^ sw) << 2) | (key & 3));
  } else {
    return d * G::VPITCH + key;
  }
}

template <typename T>
__device__ __forceinline__ T to_elem(float x) {
  return static_cast<T>(x);
}

// Element e of a 16-byte chunk held as four dwords.
template <typename T>
__device__ __forceinline__ T chunk_elem(const u32x4& v, int e) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(v[e]);
  } else {
    const uint16_t bits = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    return __builtin_bit_cast(__bf16, bits);
  }
}

// Two workgroups per CU, except fp32 with head_dim 128: its fp32 operand
// and LDS tiles need more registers than two workgroups per CU leave
// (the compiler reaches one), so that instantiation asks for one.
template <bool RET, typename T, int D>
__global__ void __launch_bounds__(kThreads, (sizeof(T) == 4 && D == 128) ? 1 : 2)
    attn_kernel(const AttnArgs a) {
  using M = Mfma<T>;
  using G = Geo<T, D>;
  using frag = typename M::frag;
  constexpr int NS = D / M::KM;    // MFMA steps over head_dim for S^T
  constexpr int NDT = D / 32;      // 32-wide head_dim tiles of O^T
  constexpr int PVS = 16 / M::KL;  // MFMA steps per 32 keys for O^T

  __shared__ __attribute__((aligned(16))) char smem[G::SMEM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;    // query row inside the wave's 32-row block
  const int half = lane >> 5;

  int item, hc;
  attn_work_item(blockIdx.x, a.n_hc, &item, &hc);
  if (item >= a.batch * a.Hkv) return;  // grid padding, uniform per block
  const int g = item % a.Hkv;
  const int rank = item / a.Hkv;
  const int b = a.order != nullptr ? min(max(a.order[rank], 0), a.batch - 1) : rank;

  const int p0 = a.cu_prefix[b];
  // Paged prefix: a length past the sequence's page-table row (a broken
  // max_prefix promise) is cut there, so no entry of another row is read.
  const int plen = (a.page_table != nullptr)
      ? min(a.cu_prefix[b + 1] - p0, a.pages_per_seq * a.page_size)
      : a.cu_prefix[b + 1] - p0;
  int rbase, nq;
  if constexpr (RET) {
    rbase = a.cu_ret[b];
    nq = min(a.cu_ret[b + 1] - rbase, a.rph);  // a broken max_ret promise stays in bounds
    if (nq <= 0) return;  // uniform over the workgroup
  } else {
    rbase = b * a.B;
    nq = a.B;
  }
  const int nh = min(a.hpw, a.G - hc * a.hpw);
  const int r = wave * 32 + n;
  const int hl = r / a.rph;
  const int qi = r - hl * a.rph;
  const bool row_ok = (hl < nh) && (qi < nq);
  const int h = g * a.G + hc * a.hpw + hl;
  const bool wave_on = wave * 32 < nh * a.rph;
  int qrow = 0;
  if (row_ok) qrow = RET ? a.idx[rbase + qi] : rbase + qi;

  // Q^T as the B operand: lane (row n, half) holds k = half*KL .. +KL-1 of
  // each MFMA step.
  frag qf[NS];
  {
    const T* qp = static_cast<const T*>(a.q) + ((size_t)qrow * a.Hq + h) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (row_ok) {
        qf[s] = *reinterpret_cast<const frag*>(qp + s * M::KM + half * M::KL);
      } else {
        qf[s] = frag{};
      }
    }
  }

  const int npt = (plen + kTile - 1) / kTile;
  const int nbt = (nq + kTile - 1) / kTile;
  const int nt = npt + nbt;

  // Loader coordinates: chunk lc of keys lkg*KPT .. +KPT-1.
  const int lc = tid % G::CPR;
  const int lkg = tid / G::CPR;
  u32x4 kr[G::KPT], vr[G::KPT];

  auto tile_count = [&](int t) {
    return t < npt ? min(kTile, plen - t * kTile)
                   : min(kTile, nq - (t - npt) * kTile);
  };
  auto tile_row = [&](int t, int key) -> size_t {
    if (t < npt) {
      const int tok = t * kTile + key;
      if (a.page_table == nullptr) return (size_t)(p0 + tok);
      const int32_t* ptab = a.page_table + (size_t)b * a.pages_per_seq;
      return (size_t)ptab[tok / a.page_size] * a.page_size + tok % a.page_size;
    }
    const int j = (t - npt) * kTile + key;
    if constexpr (RET) return (size_t)a.idx[rbase + j];
    return (size_t)(rbase + j);
  };
  auto load_tile = [&](int t, bool with_v) {
    const int cnt = tile_count(t);
    const T* kb = static_cast<const T*>(t < npt ? a.k_cache : a.k_blk);
    const T* vb = static_cast<const T*>(t < npt ? a.v_cache : a.v_blk);
#pragma unroll
    for (int k = 0; k < G::KPT; ++k) {
      const int key = lkg * G::KPT + k;
      if (key < cnt) {
        const size_t off = (tile_row(t, key) * a.Hkv + g) * D + lc * G::CE;
        kr[k] = *reinterpret_cast<const u32x4*>(kb + off);
        if (with_v) vr[k] = *reinterpret_cast<const u32x4*>(vb + off);
      } else {
        kr[k] = u32x4{0, 0, 0, 0};
        vr[k] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf, bool with_v) {
    T* ks = reinterpret_cast<T*>(smem + buf * G::KBUF);
#pragma unroll
    for (int k = 0; k < G::KPT; ++k) {
      *reinterpret_cast<u32x4*>(ks + (lkg * G::KPT + k) * G::KPITCH +
                                lc * G::CE) = kr[k];
    }
    if (!with_v) return;
    T* vt = reinterpret_cast<T*>(smem + 2 * G::KBUF + buf * G::VBUF);
    if constexpr (G::SWZ && G::KPT == 4) {
      // 4 keys x 8 dims in registers -> 8 dims x 4 keys, 8-byte writes.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t x0 = vr[0][w], x1 = vr[1][w], x2 = vr[2][w], x3 = vr[3][w];
        uint32_t lo, hi;
        if (e & 1) {
          lo = (x0 >> 16) | (x1 & 0xFFFF0000u);
          hi = (x2 >> 16) | (x3 & 0xFFFF0000u);
        } else {
          lo = (x0 & 0xFFFFu) | (x1 << 16);
          hi = (x2 & 0xFFFFu) | (x3 << 16);
        }
        const int d = lc * 8 + e;
        *reinterpret_cast<u32x2*>(vt + vt_off<T, D>(d, lkg * 4)) =
            u32x2{lo, hi};
      }
    } else {
#pragma unroll
      for (int k = 0; k < G::KPT; ++k) {
#pragma unroll
        for (int e = 0; e < G::CE; ++e) {
          vt[vt_off<T, D>(lc * G::CE + e, lkg * G::KPT + k)] =
              chunk_elem<T>(vr[k], e);
        }
      }
    }
  };
  // S^T for the 64 keys of K buffer `buf`: sacc[kt][v] is the score of key
  // kt*32 + 8*(v/4) + 4*half + v%4 against this lane's query row.
  auto scores = [&](int buf, f32x16 (&sacc)[2]) {
    const T* ks = reinterpret_cast<const T*>(smem + buf * G::KBUF);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 acc = {};
      const T* krow = ks + (kt * 32 + n) * G::KPITCH + half * M::KL;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const frag af = *reinterpret_cast<const frag*>(krow + s * M::KM);
        acc = M::run(af, qf[s], acc);
      }
      sacc[kt] = acc;
    }
  };

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  float mrun = -INFINITY;  // running row max, log2 domain
  float lsum = 0.f;        // this lane's share of the row sum

  // Importance only (block mode with out = NULL): no V, no P V.
  const bool wo = a.out != nullptr;
  load_tile(0, wo);
  store_tile(0, wo);
  if (nt > 1) load_tile(1, wo);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (wave_on) {
      const int cnt = tile_count(t);
      f32x16 sacc[2];
      scores(buf, sacc);
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const float s = key < cnt ? sacc[kt][v] * a.sl2 : -INFINITY;
          sacc[kt][v] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun, mx);
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(sacc[kt][v] - mnew);
          sacc[kt][v] = p;
          ps += p;
        }
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

      const T* vt =
          reinterpret_cast<const T*>(smem + 2 * G::KBUF + buf * G::VBUF);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (!wo) break;
#pragma unroll
        for (int st = 0; st < PVS; ++st) {
          frag pb;
          if constexpr (M::KL == 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = to_elem<T>(sacc[kt][st * 8 + e]);
          } else {
            pb = sacc[kt][st];
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int d = dt * 32 + n;
            frag va;
            if constexpr (M::KL == 8) {
              const int k0 = kt * 32 + 16 * st + 4 * half;
              const bf16x4 lo =
                  *reinterpret_cast<const bf16x4*>(vt + vt_off<T, D>(d, k0));
              const bf16x4 hi =
                  *reinterpret_cast<const bf16x4*>(vt + vt_off<T, D>(d, k0 + 8));
              va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
              const int key = kt * 32 + 8 * (st >> 2) + 4 * half + (st & 3);
              va = vt[vt_off<T, D>(d, key)];
            }
            oacc[dt] = M::run(va, pb, oacc[dt]);
          }
        }
      }
    }
    if (t + 1 < nt) store_tile(buf ^ 1, wo);
    if (t + 2 < nt) load_tile(t + 2, wo);
    __syncthreads();
  }

  // Final row statistics (both halves of a row hold the same max).
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float lse2 = mrun + log2f(ltot);

  if (wave_on && row_ok) {
    const float inv = 1.0f / ltot;
    T* op = static_cast<T*>(a.out) + ((size_t)(rbase + qi) * a.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (!wo) break;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * half;
        if constexpr (sizeof(T) == 2) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = to_elem<T>(oacc[dt][4 * q4 + e] * inv);
          *reinterpret_cast<bf16x4*>(op + d0) = o;
        } else {
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = oacc[dt][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4*>(op + d0) = o;
        }
      }
    }
    if constexpr (!RET) {
      if (a.lse != nullptr && half == 0) {
        a.lse[((size_t)b * a.Hq + h) * a.B + qi] = lse2 * kLn2;
      }
    }
  }

  if constexpr (!RET) {
    // Pass 2: importance of the block columns from the final lse.
    float* pbuf = reinterpret_cast<float*>(smem + G::KBUF);
    for (int tb = 0; tb < nbt; ++tb) {
      const int t = npt + tb;
      const int cnt = tile_count(t);
      load_tile(t, false);
      store_tile(0, false);
      __syncthreads();
      if (wave_on) {
        f32x16 sacc[2];
        scores(0, sacc);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = kt * 32 + 8 * q4 + 4 * half + e;
              pv[e] = key < cnt ? __builtin_amdgcn_exp2f(
                                      sacc[kt][4 * q4 + e] * a.sl2 - lse2)
                                : 0.f;
            }
            *reinterpret_cast<f32x4*>(pbuf + r * G::PPITCH + kt * 32 + 8 * q4 +
                                      4 * half) = pv;
          }
        }
      }
      __syncthreads();
      for (int id = tid; id < nh * kTile; id += kThreads) {
        const int hh = id / kTile;
        const int key = id - hh * kTile;
        if (key < cnt) {
          float acc = 0.f;
          const float* col = pbuf + (hh * a.rph) * G::PPITCH + key;
          for (int i = 0; i < a.B; ++i) acc += col[i * G::PPITCH];
          const int hg = g * a.G + hc * a.hpw + hh;
          a.imp[((size_t)b * a.Hq + hg) * a.B + tb * kTile + key] = acc;
        }
      }
      __syncthreads();
    }
  }
}

template <bool RET>
hipError_t launch(Elem e, int d, int batch, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(attn_grid_size(batch * a.Hkv, a.n_hc));
  const dim3 block(kThreads);
  if (e == Elem::BF16 && d == 128) {
    hipLaunchKernelGGL((attn_kernel<RET, __bf16, 128>), grid, block, 0, s, a);
  } else if (e == Elem::BF16 && d == 64) {
    hipLaunchKernelGGL((attn_kernel<RET, __bf16, 64>), grid, block, 0, s, a);
  } else if (e == Elem::F32 && d == 128) {
    hipLaunchKernelGGL((attn_kernel<RET, float, 128>), grid, block, 0, s, a);
  } else if (e == Elem::F32 && d == 64) {
    hipLaunchKernelGGL((attn_kernel<RET, float, 64>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_attn(Elem e, int d, int batch, const AttnArgs& a,
                             hipStream_t s) {
  if (e == Elem::BF16 && d == 128) return launch_block_attn_bf16(batch, a, s);
  return launch<false>(e, d, batch, a, s);
}

hipError_t launch_retained_attn(Elem e, int d, int batch, const AttnArgs& a,
                                hipStream_t s) {
  if (e == Elem::BF16 && d == 128) return launch_retained_attn_bf16(batch, a, s);
  return launch<true>(e, d, batch, a, s);
}

}  // namespace focus
