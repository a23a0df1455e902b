// Block attention with importance, and retained-query attention: the bf16,
// head_dim 128 kernel tuned for gfx950 (MI355X).
//
// Same computation as the generic kernel in attn.hip (see there for the
// sources on the pages); this file only changes how the work is mapped on
// the chip:
//  * K/V tiles of 32 keys travel HBM -> LDS by direct-to-LDS loads
//    (buffer_load_dwordx4 ... lds for whole prefix tiles, addressed from a
//    scalar per-tile base; global_load_lds_dwordx4 for the rest) through a
//    ring of 4 stages: while tile t is computed, tile t + 1 is resident
//    and tiles t + 2 and t + 3 are in flight; no registers hold loads.
//    Completion is tracked by hand: each wave waits until its own loads for
//    the tile are done (vmcnt), then one barrier per tile publishes them.
//  * K rows sit in LDS with their 16-byte chunks XOR-swizzled by the row
//    (conflict-free ds_read_b128 operand reads). V stays key-major in LDS
//    and the O^T = V^T P^T operand is read with ds_read_b64_tr_b16, which
//    hands each lane 4 consecutive keys of one head-dim column. The LDS
//    serves 32 lanes of 8-byte reads per cycle; one such read touches 4 key
//    rows x 64 bytes, so V's 16-byte chunks are XOR-swizzled by
//    4 * (row mod 4), which spreads those 16 chunks over all banks.
//  * Online softmax with the scale folded into one FMA per score. The
//    running max starts at the first tile's max; the exponentials of a
//    later tile are taken against it before the tile's own max is known,
//    in place of the raw scores. Only when a lane's 16 of them sum to more
//    than 2^8 (or are not finite) is the max taken, from raw scores
//    recomputed out of the still-resident K tile, and O rescaled. The final
//    O / l and lse are exact whatever max was used, and no exponential
//    exceeds 2^8.
//  * Inside one wave the matrix core and the vector ALU overlap: the eight
//    score MFMAs of tile t + 1 are issued one at a time between the
//    exponentials of tile t (scheduling fences keep that order).
//  * The block keys are processed last and their raw scores stay in
//    registers, so the importance pass needs neither a reload nor a
//    recompute once the final lse is known (and those registers are free
//    during the prefix stream). Its column sums run in two fixed-order
//    levels over all threads (row segments, then the segments in order).
//  * Work items are visited longest prefix first (order from a one-block
//    rank count, or bitonic sort past 256 sequences, of the prefix
//    lengths), the KV heads of a sequence on neighbouring workgroups.
#include "focus_internal.hpp"

namespace focus {
namespace {

constexpr int TK = 32;          // keys per tile
// Ring depth, with O (K + V tiles, 16 KB a stage) and without (K only):
// four stages measured best for both (three to five were tried).
constexpr int NSTAGE = 4;
constexpr int NW = kThreads / 64;  // waves per workgroup (128 query rows)
constexpr int D = 128;
constexpr int ROWB = D * 2;     // bytes per key row (256)
constexpr int TILEB = TK * ROWB;        // 8 KB per K or V tile
constexpr int PPITCH = TK + 4;          // fp32 probability row pitch
// One ring stage holds a K tile and, when O is produced, a V tile.
template <bool WO> constexpr int stage_bytes() { return WO ? 2 * TILEB : TILEB; }
constexpr float kLn2 = 0.6931471805599453f;
// A lane's sum of the 16 exponentials of a tile above which the running
// max is recomputed (and O rescaled).
constexpr float kSumMax = 256.0f;
constexpr int kPageRegs = 4;    // paged prefix: registers of cached page entries
// s_waitcnt immediate for vmcnt(0) with expcnt / lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Cache policy of the direct-to-LDS K/V loads (POL, the instruction's
// cache-policy bits). With one head chunk per KV head each K/V row is read
// once per launch: nt (non-temporal), measured 7% faster for block and 10%
// for retained attention at B = 32 than the default policy. With several
// head chunks the chunks of an item stream the same rows close together on
// one XCD and L2 serves the repeats: the default policy from three chunks
// on, measured 3.6% faster for block attention at B = 128 (four chunks),
// the launch after it 2-3% slower (what the cached rows leave in L2); at
// B = 64 (two chunks) block attention gained nothing, so nt stays there.
// Retained attention at these budgets has one chunk (its full-budget form
// has the chunks of block attention).
constexpr int kPolicyNt = 2;       // cache-policy bits: nt
constexpr int kPolicyDefault = 0;

// A wave-uniform pointer, moved to scalar registers explicitly.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource at a tile's first byte (gfx9 word 3: 32-bit data
// format, no swizzle); lane offsets stay far below its 2 GiB range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, 0x7fffffff, 0x00020000);
}
template <int POL>
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, POL);
}

template <int POL>
__device__ __forceinline__ void dma16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, POL);
}

// 16 bytes of O to global memory with the sc1 and nt cache-policy bits (the
// compiler's non-temporal store sets nt alone). Measured on MI355X, same
// outputs: block attention about 1% faster at B = 32, 64 and 128 than with
// nt alone, retained attention unchanged; with sc1 alone block attention
// gained 2% but the next launch lost about as much (the writes drained
// during it), and write-back stores were 3% slower.
__device__ __forceinline__ void store_o16(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v) : "memory");
}

// Wait until at most `n` of this wave's vector-memory operations are
// outstanding, then barrier; n above 12 waits as for 12 (more than
// needed, never less). The memory clobber keeps the compiler from moving
// LDS accesses across it.
#define FOCUS_WB(N)                                                           \
  case N:                                                                     \
    asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
    break;
__device__ __forceinline__ void wait_and_barrier(int n) {
  switch (n < 0 ? 0 : (n > 12 ? 12 : n)) {
    FOCUS_WB(0) FOCUS_WB(1) FOCUS_WB(2) FOCUS_WB(3) FOCUS_WB(4) FOCUS_WB(5)
    FOCUS_WB(6) FOCUS_WB(7) FOCUS_WB(8) FOCUS_WB(9) FOCUS_WB(10) FOCUS_WB(11)
    default:
      FOCUS_WB(12)
  }
}
#undef FOCUS_WB

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)p));
}

// The sixteen V^T operand fragments of one 32-key tile: for head-dim tiles
// dt = 0..3 (addresses a0..a3) the keys at row offsets +0, +8 rows (f, the
// first 16 keys) and +16, +24 rows (h, the last 16), each read with
// ds_read_b64_tr_b16. The reads sit in one asm block that also waits for
// them (one LDS wait per tile), so no output register is ever left with a
// load in flight (and the compiler adds no wait of its own for the
// direct-to-LDS loads that may still be landing in other ring stages). The
// outputs are early-clobber: a read may land while a later read of the
// block has not yet taken its address, so no output may share a register
// with an address.
__device__ __forceinline__ void v_frags16(uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3, u32x2v (&f)[8], u32x2v (&h)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:0\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:0\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:0\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %12, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %13, %18 offset:6144\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
        "=&v"(f[6]), "=&v"(f[7]), "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]),
        "=&v"(h[4]), "=&v"(h[5]), "=&v"(h[6]), "=&v"(h[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Max / sum of a value over the lane pair (l, l ^ 32), without LDS:
// v_permlane32_swap exchanges the two 32-lane halves, so the pair of
// results holds both values in every lane.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of a lane's 16 exponentials, pairwise in a fixed order.
__device__ __forceinline__ float tile_sum(const f32x16& p) {
  float q8[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) q8[v] = p[2 * v] + p[2 * v + 1];
  return ((q8[0] + q8[1]) + (q8[2] + q8[3])) + ((q8[4] + q8[5]) + (q8[6] + q8[7]));
}

__device__ __forceinline__ bf16x8 cat8(u32x2v lo, u32x2v hi) {
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// WO: O is produced. Without it (importance only: block mode with out =
// NULL) no V is loaded and no P V product is formed; the K-only ring is half
// the size and three workgroups share a CU.
// PAGED: the prefix K/V live in pages (AttnArgs::page_table).
// Four waves per workgroup (NW); eight-wave workgroups of 256 rows (one per
// CU, 8-stage ring), which halve the workgroups that stream the same K/V
// when a KV head has more than 128 query rows, measured no faster at
// B = 64 / 128 or G = 8.
template <bool RET, int NBT, bool WO, bool PAGED, int POL>
__global__ void __launch_bounds__(NW * 64, WO ? 2 : 3)
    attn_bf16_kernel(const AttnArgs a) {
  constexpr int STAGEB = stage_bytes<WO>();
  constexpr int SMEM = NSTAGE * STAGEB;
  constexpr int NTHR = NW * 64;
  constexpr int SPW = 8 / NW;                // 4-row DMA slots per wave
  constexpr int OPS = (WO ? 2 : 1) * SPW;    // loads per wave per tile
  static_assert(NW * 32 * PPITCH * 4 + NTHR * 4 <= SMEM, "pass-2 buffers fit the ring");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
  const int lane = tid & 63;
  const int n = lane & 31;
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
  const int plen = PAGED
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

  // ---- loader geometry: lane covers row (4j + lane/16) of DMA slot j,
  // physical 16-byte chunk lane%16; wave w owns slots SPW*w .. SPW*w+SPW-1.
  const int lrow0 = 4 * SPW * wave + (lane >> 4);   // rows lrow0 + 4i
  const int pchunk = lane & 15;
  const int nbt = (nq + TK - 1) / TK;        // block tiles (<= NBT)
  const int npt = (plen + TK - 1) / TK;
  const int nt = nbt + npt;

  // Retained mode: the block rows this lane loads (gathered through idx),
  // resolved up front so that no index load sits between the streaming
  // loads. Block mode computes them from rbase.
  int brow[RET ? NBT : 1][SPW];
  if constexpr (RET) {
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        // rows past the end repeat the last row (masked)
        const int j = min(bt * TK + lrow0 + 4 * i, nq - 1);
        brow[bt][i] = bt < nbt ? a.idx[rbase + j] : 0;
      }
    }
  }

  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const char* kb = static_cast<const char*>(a.k_blk);
  const char* vb = static_cast<const char*>(a.v_blk);
  const size_t rowstride = (size_t)a.Hkv * ROWB;  // bytes between tokens
  const size_t goff = (size_t)g * ROWB;

  // Byte offsets of the two rows this lane loads in a prefix tile, relative
  // to the tile's first token: full tiles add one scalar base per tile.
  // (32 rows of at most kMaxHeads heads stay below 2^32 bytes.)
  uint32_t koff[SPW], voff[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int lr = lrow0 + 4 * i;
    const uint32_t rb = (uint32_t)(lr * rowstride + goff);
    koff[i] = rb + ((pchunk ^ (lr & 15)) << 4);
    voff[i] = rb + ((pchunk ^ ((lr & 3) << 2)) << 4);
  }

  // Paged prefix (PAGED): a cursor over the sequence's pages follows the
  // tiles, which are issued strictly in order; pages hold a multiple of 32
  // tokens, so a tile never straddles two pages. The page entries are held
  // in registers, lane l of register k holding entry pg_base + 64k + l, and
  // read with v_readlane: a scalar load of the page table in the loop would
  // make every later LDS wait a full lgkmcnt(0), stalling on that load.
  // Past 64 * kPageRegs pages the cache is refilled once the ring has
  // drained (one drain per 64 * kPageRegs pages).
  [[maybe_unused]] const int32_t* ptab = nullptr;
  [[maybe_unused]] int pg_tiles = 1, pg_count = 0, pg_i = 0, pg_t = 0, pg_base = 0;
  [[maybe_unused]] int pg_cache[kPageRegs];
  auto load_page_cache = [&](int base) {
#pragma unroll
    for (int k = 0; k < kPageRegs; ++k) {
      const int i = base + 64 * k + lane;
      pg_cache[k] = i < pg_count ? ptab[i] : 0;
    }
  };
  if constexpr (PAGED) {
    ptab = a.page_table + (size_t)b * a.pages_per_seq;
    pg_tiles = a.page_size / TK;
    pg_count = (plen + a.page_size - 1) / a.page_size;
    load_page_cache(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  // Row of the first token of prefix tile t (called once per prefix tile,
  // t = 0, 1, 2, ... in order).
  auto prefix_row0 = [&](int t) -> int64_t {
    if constexpr (!PAGED) {
      return (int64_t)p0 + t * TK;
    } else {
      int rel = pg_i - pg_base;
      if (rel >= 64 * kPageRegs) {
        // drain the ring, refill, and wait with the builtin so that the
        // compiler sees the refill complete (no wait of its own later)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        pg_base = pg_i;
        load_page_cache(pg_base);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        rel = 0;
      }
      int entry = 0;
#pragma unroll
      for (int k = 0; k < kPageRegs; ++k)
        if ((rel >> 6) == k) entry = __builtin_amdgcn_readlane(pg_cache[k], rel & 63);
      const int64_t r = (int64_t)entry * a.page_size + (int64_t)pg_t * TK;
      if (++pg_t == pg_tiles) {
        pg_t = 0;
        ++pg_i;
      }
      return r;
    }
  };

  // Tiles 0 .. npt-1 are the prefix, npt .. nt-1 the block.
  auto issue_tile = [&](int t) {
    char* st = smem + (t % NSTAGE) * STAGEB;
    if (t < npt) {
      const int64_t r0 = prefix_row0(t);
      if ((t + 1) * TK <= plen) {
        // full prefix tile
        const size_t tb = (size_t)r0 * rowstride;
        // A full tile is addressed as a buffer at the tile's first byte (the
        // 64-bit base in scalar registers) plus the lane's constant 32-bit
        // offset: no vector address arithmetic per load.
        const auto rk = tile_rsrc(uniform_ptr(kc + tb));
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
          char* dst = st + (SPW * wave + i) * 1024;
          dma16b<POL>(rk, koff[i], dst);
        }
        if constexpr (WO) {
          const auto rv = tile_rsrc(uniform_ptr(vc + tb));
#pragma unroll
          for (int i = 0; i < SPW; ++i) {
            char* dst = st + (SPW * wave + i) * 1024;
            dma16b<POL>(rv, voff[i], dst + TILEB);
          }
        }
        return;
      }
      // last, partial prefix tile: rows past the end repeat the last row
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int lr = lrow0 + 4 * i;          // row inside the tile
        const int64_t row = r0 + min(lr, plen - 1 - t * TK);
        // koff/voff hold lr * rowstride; take it back out in integers
        const ptrdiff_t shift = ((ptrdiff_t)row - lr) * (ptrdiff_t)rowstride;
        char* dst = st + (SPW * wave + i) * 1024;
        dma16<POL>(kc + (size_t)((ptrdiff_t)koff[i] + shift), dst);
        if constexpr (WO) dma16<POL>(vc + (size_t)((ptrdiff_t)voff[i] + shift), dst + TILEB);
      }
      return;
    }
    const int bt = t - npt;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int lr = lrow0 + 4 * i;          // row inside the tile
      int row;
      if constexpr (RET) {
        row = 0;
#pragma unroll
        for (int k = 0; k < NBT; ++k)
          if (k == bt) row = brow[k][i];
      } else {
        row = rbase + min(bt * TK + lr, nq - 1);
      }
      const ptrdiff_t shift = ((ptrdiff_t)row - lr) * (ptrdiff_t)rowstride;
      char* dst = st + (SPW * wave + i) * 1024;
      dma16<POL>(kb + (size_t)((ptrdiff_t)koff[i] + shift), dst);
      if constexpr (WO) dma16<POL>(vb + (size_t)((ptrdiff_t)voff[i] + shift), dst + TILEB);
    }
  };

  // Q^T operand: lane (row n, half) holds d = 16s + 8*half .. +7.
  bf16x8 qf[8];
  {
    const __bf16* qp = nullptr;
    if (row_ok) {
      const int qrow = RET ? a.idx[rbase + qi] : rbase + qi;
      qp = static_cast<const __bf16*>(a.q) + ((size_t)qrow * a.Hq + h) * D;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * half)
                     : bf16x8{};
  }

  // Prologue: tiles 0 .. NSTAGE-2 in flight. All index and Q loads are
  // consumed first so that vmcnt below counts ring loads only (the builtin,
  // so that the compiler knows they are complete too).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  for (int t = 0; t < NSTAGE - 1 && t < nt; ++t) issue_tile(t);

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  f32x16 sblk[NBT];
#pragma unroll
  for (int bt = 0; bt < NBT; ++bt) sblk[bt] = f32x16{};
  float mrun = -INFINITY;  // max used for the exponentials (log2 domain)
  float lsum = 0.f;        // this lane's share of the row sum
  const float c = a.sl2;

  // Per-lane LDS read offsets.
  const int krd = n * ROWB;                       // + ((2s+half)^(n&15))*16
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int ve = l16 >> 2, vq = l16 & 3;
  const int vh = grp >> 1;
  // V^T operand read: row (16*st + 8*x + 4*vh + ve), logical chunk
  // 4*dt + 2*(grp&1) + vq/2, swizzled by 4*ve, byte 8*(vq&1).
  const int vrow_base = 4 * vh + ve;
  const int vchunk_base = 2 * (grp & 1) + (vq >> 1);
  const int vbyte = 8 * (vq & 1);

  // S^T of one tile (raw scores, unmasked): lane (row n, half) gets keys
  // 8*(v/4) + 4*half + v%4, v = 0..15.
  auto qk = [&](int t) -> f32x16 {
    const char* ks = smem + (t % NSTAGE) * STAGEB;
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int ch = (2 * k + half) ^ (n & 15);
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(ks + krd + ch * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[k], acc, 0, 0, 0);
    }
    return acc;
  };
  auto tile_cnt = [&](int t) {
    return t < npt ? min(TK, plen - t * TK) : min(TK, nq - (t - npt) * TK);
  };
  // Keys past the tile's count get score -inf.
  auto mask_tile = [&](f32x16& s, int cnt) {
    if (cnt < TK) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + 4 * half + (v & 3);
        if (key >= cnt) s[v] = -INFINITY;
      }
    }
  };
  // Max of a row's scores in the log2 domain (both lanes of the row).
  auto row_max2 = [&](const f32x16& s) {
    const float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]);
    const float m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]);
    const float m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
    const float mm = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), s[15]));
    return pair_max(mm) * c;
  };

  // V^T fragment offsets inside a V tile, one per head-dim tile.
  uint32_t va_off[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    va_off[dt] = vrow_base * ROWB + (((4 * dt + vchunk_base) ^ (4 * ve)) << 4) + vbyte;

  // One tile of the software pipeline: the scores of tile t + 1 are issued
  // on the matrix cores (into s_nxt) while the vector units run the softmax
  // of tile t (s_cur) and its P V product. Tiles t and t + 1 are resident at
  // the top; the ring slot of tile t - 1 is then refilled with tile t + 3.
  // cap, when given, receives the masked raw scores of a block tile.
  auto tile_step = [&](int t, f32x16& s_cur, f32x16& s_nxt, f32x16* cap, bool more) {
    // tiles t and t + 1 resident; t + 2 .. t + NSTAGE - 2 may be in flight
    wait_and_barrier(OPS * max(0, min(t + NSTAGE - 2, nt - 1) - (t + 1)));
    if (t + NSTAGE - 1 < nt) issue_tile(t + NSTAGE - 1);
    if (!wave_on) return;

    f32x16& s = s_cur;
    const int cnt = tile_cnt(t);
    mask_tile(s, cnt);
    if (cap != nullptr) *cap = s;
    // Exponentials against the running max first, in place of the raw
    // scores; the max of this tile is only needed when their sum exceeds
    // kSumMax or is not finite. They are interleaved with the score MFMAs
    // of tile t + 1 (more: a tile follows), so that the vector ALU and the
    // matrix core of this wave work at the same time; the fences keep the
    // compiler from regrouping them.
    float q8[8];
    if (more) {
      const char* ks = smem + ((t + 1) % NSTAGE) * STAGEB;
      bf16x8 kf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int ch = (2 * k + half) ^ (n & 15);
        kf[k] = *reinterpret_cast<const bf16x8*>(ks + krd + ch * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc = {};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], acc, 0, 0, 0);
        s[2 * k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k], c, -mrun));
        s[2 * k + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k + 1], c, -mrun));
        q8[k] = s[2 * k] + s[2 * k + 1];
        __builtin_amdgcn_sched_barrier(0);
      }
      s_nxt = acc;
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], c, -mrun));
#pragma unroll
      for (int k = 0; k < 8; ++k) q8[k] = s[2 * k] + s[2 * k + 1];
    }
    float ts = ((q8[0] + q8[1]) + (q8[2] + q8[3])) + ((q8[4] + q8[5]) + (q8[6] + q8[7]));
    if (__any(!(ts <= kSumMax))) {
      // The raw scores were overwritten: a block tile kept them (cap);
      // otherwise tile t is still resident in the ring and they are
      // recomputed (the same MFMA chain, the same bits).
      f32x16 r;
      if (cap != nullptr) {
        r = *cap;
      } else {
        r = qk(t);
        mask_tile(r, cnt);
      }
      const float mnew = fmaxf(mrun, row_max2(r));
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
      if constexpr (WO) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(r[v], c, -mrun));
      ts = tile_sum(s);
    }
    lsum += ts;
    if constexpr (!WO) return;

    const uint32_t vbase = lds_addr(smem + (t % NSTAGE) * STAGEB + TILEB);
    u32x2v f0[8], f1[8];
    v_frags16(vbase + va_off[0], vbase + va_off[1], vbase + va_off[2],
              vbase + va_off[3], f0, f1);
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[e]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          cat8(f0[2 * dt], f0[2 * dt + 1]), pb, oacc[dt], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[8 + e]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          cat8(f1[2 * dt], f1[2 * dt + 1]), pb, oacc[dt], 0, 0, 0);
  };

  // Tile 0 must be in LDS before its scores; tiles 1.. may still land.
  wait_and_barrier(OPS * (min(nt, NSTAGE - 1) - 1));
  f32x16 sa = {}, sb = {};
  if (wave_on) {
    // The running max starts at the first tile's max, so that tile takes
    // the common path (same values as rescaling from -inf).
    sa = qk(0);
    mask_tile(sa, tile_cnt(0));
    mrun = row_max2(sa);
  }
  // Prefix tiles two at a time, so that the score registers alternate
  // instead of being copied between iterations; then the block tiles,
  // unrolled, each keeping its raw scores in registers of its own for the
  // importance pass (live only from here on).
  // (A wave with rows has nq >= 1, hence a block tile after every prefix
  // tile.)
  for (int t = 0; t < npt; t += 2) {
    tile_step(t, sa, sb, nullptr, true);
    if (t + 1 < npt) tile_step(t + 1, sb, sa, nullptr, true);
  }
  if (npt & 1) sa = sb;
#pragma unroll
  for (int bt = 0; bt < NBT; ++bt) {
    if (bt < nbt) {
      f32x16* cap = nullptr;
      if constexpr (!RET) cap = &sblk[bt];
      if (bt & 1)
        tile_step(npt + bt, sb, sa, cap, npt + bt + 1 < nt);
      else
        tile_step(npt + bt, sa, sb, cap, npt + bt + 1 < nt);
    }
  }

  const float ltot = pair_sum(lsum);
  const float lse2 = mrun + log2f(ltot);

  // The ring is idle from here on: the last tile waited for every load
  // (vmcnt(0)), so the barriers below need no vmcnt wait, and the O stores
  // come last, after the importance pass, so that nothing waits on them.
  if constexpr (!RET) {
    // Importance of the block columns: exp2(s*c - lse2) from the kept raw
    // block scores, summed down each column per head in a fixed order: with
    // fewer than NTHR (head, key) columns, every thread adds a segment of
    // rows of one column and one thread per column then adds the segments
    // in order (a column of B = 128 rows is 8 segments of 16, not one
    // chain of 128 LDS reads); otherwise each column has at most 16 rows
    // and one thread adds it.
    float* pbuf = reinterpret_cast<float*>(smem);
    float* part = pbuf + NW * 32 * PPITCH;           // segment sums, <= NTHR
    const int ncol = nh * TK;
    const int nseg = max(1, NTHR / ncol);
    const int seg = (a.B + nseg - 1) / nseg;
    for (int bt = 0; bt < nbt; ++bt) {
      const int cnt = min(TK, nq - bt * TK);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wave_on) {
        f32x16 sb = {};
#pragma unroll
        for (int k = 0; k < NBT; ++k)
          if (k == bt) sb = sblk[k];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[4 * q4 + e], c, -lse2));
          *reinterpret_cast<f32x4*>(pbuf + r * PPITCH + 8 * q4 + 4 * half) = pv;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (nseg == 1) {
        for (int cl = tid; cl < ncol; cl += NTHR) {
          const int hh = cl / TK;
          const int key = cl - hh * TK;
          if (key < cnt) {
            float acc = 0.f;
            const float* col = pbuf + (hh * a.rph) * PPITCH + key;
            for (int i = 0; i < a.B; ++i) acc += col[i * PPITCH];
            const int hg = g * a.G + hc * a.hpw + hh;
            a.imp[((size_t)b * a.Hq + hg) * a.B + bt * TK + key] = acc;
          }
        }
        continue;
      }
      if (tid < ncol * nseg) {
        const int sg = tid / ncol;
        const int cl = tid - sg * ncol;
        const int hh = cl / TK;
        const int key = cl - hh * TK;
        const int i1 = min(a.B, (sg + 1) * seg);
        const float* col = pbuf + (hh * a.rph) * PPITCH + key;
        float acc = 0.f;
#pragma unroll 8
        for (int i = sg * seg; i < i1; ++i) acc += col[i * PPITCH];
        part[tid] = acc;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (tid < ncol) {
        const int hh = tid / TK;
        const int key = tid - hh * TK;
        if (key < cnt) {
          float acc = 0.f;
          for (int sg = 0; sg < nseg; ++sg) acc += part[sg * ncol + tid];
          const int hg = g * a.G + hc * a.hpw + hh;
          a.imp[((size_t)b * a.Hq + hg) * a.B + bt * TK + key] = acc;
        }
      }
    }
    if (wave_on && row_ok && a.lse != nullptr && half == 0)
      a.lse[((size_t)b * a.Hq + h) * a.B + qi] = lse2 * kLn2;
  }

  if constexpr (WO) {
    // O through LDS: each wave stages its 32 rows x 128 values (row pitch
    // 272 bytes), then stores whole rows with 16-byte lanes, 4 rows of 256
    // bytes per instruction. The staging area
    // sits above the importance buffer; it overlaps the ring, so all waves
    // must be past their last P V reads first.
    constexpr int OP = 272;
    if constexpr (RET) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    static_assert(SMEM >= NW * 32 * OP + NW * 32 * PPITCH * 4 + NTHR * 4, "O staging fits");
    char* ost = smem + (SMEM - NW * 32 * OP) + wave * (32 * OP);
    if (wave_on) {
      const float inv = 1.0f / ltot;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(oacc[dt][4 * q4 + e] * inv);
          *reinterpret_cast<bf16x4*>(ost + n * OP + (dt * 32 + 8 * q4 + 4 * half) * 2) = o;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cidx = lane + 64 * k;           // 16-byte chunk of the wave's tile
        const int row = cidx >> 4, c16 = cidx & 15;
        const int rr = wave * 32 + row;
        const int hl2 = rr / a.rph;
        const int qi2 = rr - hl2 * a.rph;
        if (hl2 < nh && qi2 < nq) {
          const int h2 = g * a.G + hc * a.hpw + hl2;
          const int qrow = rbase + qi2;           // output row (retained: its slot)
          store_o16(static_cast<char*>(a.out) + ((size_t)qrow * a.Hq + h2) * (D * 2) + c16 * 16,
                    *reinterpret_cast<const u32x4*>(ost + row * OP + c16 * 16));
        }
      }
    }
  }
}

template <bool RET, bool WO, bool PAGED, int POL>
hipError_t launch_nbt(int nbt, int batch, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(attn_grid_size(batch * a.Hkv, a.n_hc)), block(NW * 64);
  switch (nbt) {
    case 1:
      hipLaunchKernelGGL((attn_bf16_kernel<RET, 1, WO, PAGED, POL>), grid, block, 0, s, a);
      break;
    case 2:
      hipLaunchKernelGGL((attn_bf16_kernel<RET, 2, WO, PAGED, POL>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((attn_bf16_kernel<RET, 4, WO, PAGED, POL>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

template <bool RET, bool WO>
hipError_t launch_layout(int nbt, int batch, const AttnArgs& a, hipStream_t s) {
  if (a.n_hc >= 3) {
    if (a.page_table != nullptr) return launch_nbt<RET, WO, true, kPolicyDefault>(nbt, batch, a, s);
    return launch_nbt<RET, WO, false, kPolicyDefault>(nbt, batch, a, s);
  }
  if (a.page_table != nullptr) return launch_nbt<RET, WO, true, kPolicyNt>(nbt, batch, a, s);
  return launch_nbt<RET, WO, false, kPolicyNt>(nbt, batch, a, s);
}

int block_tiles(int rows) {
  const int t = (rows + TK - 1) / TK;
  return t <= 1 ? 1 : (t <= 2 ? 2 : 4);
}

}  // namespace

hipError_t launch_block_attn_bf16(int batch, const AttnArgs& a, hipStream_t s) {
  if (a.out == nullptr) return launch_layout<false, false>(block_tiles(a.B), batch, a, s);
  return launch_layout<false, true>(block_tiles(a.B), batch, a, s);
}

hipError_t launch_retained_attn_bf16(int batch, const AttnArgs& a, hipStream_t s) {
  return launch_layout<true, true>(block_tiles(a.rph), batch, a, s);
}

}  // namespace focus
