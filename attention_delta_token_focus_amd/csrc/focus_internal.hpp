// Internal declarations shared by the libfocus translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace focus {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Key tile width of the attention kernels (keys per LDS tile).
constexpr int kTile = 64;
// Query rows per workgroup (4 waves x 32 rows, one 32x32 MFMA row block
// per wave).
constexpr int kRowsPerWG = 128;
constexpr int kThreads = 256;

struct AttnArgs {
  const void* q;
  const void* k_blk;
  const void* v_blk;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_prefix;
  const int32_t* idx;     // retained mode: gathered block rows
  const int32_t* cu_ret;  // retained mode: per-sequence row offsets
  const int32_t* order;   // visiting order of the sequences (may be null)
  int batch;              // number of sequences
  void* out;
  float* imp;             // block mode only
  float* lse;             // block mode only, may be null
  int B;                  // block size (rows per sequence in q/k_blk)
  int Hq, Hkv, G;         // G = Hq / Hkv
  int rph;                // query rows reserved per head in a workgroup
  int hpw;                // query heads per workgroup
  int n_hc;               // head chunks per KV head
  float sl2;              // softmax scale * log2(e)
  // Paged prefix KV (page_table non-null): k_cache / v_cache are pools of
  // pages of page_size tokens ([pages, page_size, Hkv, d]); token t of
  // sequence b sits in page page_table[b * pages_per_seq + t / page_size],
  // slot t % page_size. cu_prefix then only gives the lengths.
  const int32_t* page_table;
  int page_size;          // a multiple of 32
  int pages_per_seq;
};

// Heads per token are bounded so that a 32-token tile of one KV head spans
// less than 4 GiB and in-tile byte offsets fit 32 bits.
constexpr int kMaxHeads = 4096;

// Workgroups are dispatched to the 8 XCDs of an MI355X round-robin by
// block index, and each XCD has its own L2. The attention grid therefore
// keeps the n_hc query-head chunks of one (sequence, KV head) item -- which
// all stream the same K/V -- on one XCD: item i goes to XCD i % 8, and its
// chunks are consecutive in that XCD's dispatch order.
constexpr int kXcds = 8;

__host__ __device__ inline unsigned attn_grid_size(int items, int n_hc) {
  return (unsigned)((items + kXcds - 1) / kXcds) * kXcds * (unsigned)n_hc;
}

// Decodes a block index into (item, chunk); item >= items marks padding.
__device__ inline void attn_work_item(int blk, int n_hc, int* item, int* hc) {
  const int x = blk % kXcds;
  const int s = blk / kXcds;
  const int q = s / n_hc;
  *item = kXcds * q + x;
  *hc = s - q * n_hc;
}

enum class Elem { F32 = 0, BF16 = 1 };

// Launchers; return the launch status.
hipError_t launch_block_attn(Elem e, int d, int batch, const AttnArgs& a,
                             hipStream_t s);
hipError_t launch_retained_attn(Elem e, int d, int batch, const AttnArgs& a,
                                hipStream_t s);
// Tuned bf16 / head_dim 128 kernels (attn_bf16.hip).
hipError_t launch_block_attn_bf16(int batch, const AttnArgs& a, hipStream_t s);
hipError_t launch_retained_attn_bf16(int batch, const AttnArgs& a, hipStream_t s);
// Longest-prefix-first order of the sequences into `order` [batch]
// (schedule.hip).
hipError_t launch_lpt_order(int batch, const int32_t* cu_prefix, int32_t* order,
                            hipStream_t s);
size_t order_workspace_bytes(int batch);

hipError_t launch_delta_topk(int batch, int B, int Hq, int pool_k,
                             const float* imp0, const float* imp1,
                             const uint8_t* masked, int rules,
                             const int32_t* k_keep, const float* yield_hist,
                             float alpha, int32_t* k_used, uint8_t* keep,
                             uint8_t* cand, float* dI, hipStream_t s);
// Largest batch the fused delta/top-K + compaction kernel takes.
constexpr int kFusedSelectMax = 4096;
hipError_t launch_select(int batch, int B, int Hq, int pool_k,
                         const float* imp0, const float* imp1,
                         const int32_t* k_keep, uint8_t* keep, float* dI,
                         int32_t* idx, int32_t* cu_ret, hipStream_t s);
hipError_t launch_compact(int batch, int B, const uint8_t* keep, int32_t* idx,
                          int32_t* cu_ret, hipStream_t s);

}  // namespace focus
