// C ABI of libfocus: argument validation, launch geometry, error strings.
// Every entry point checks its host-visible arguments before enqueuing any
// work and never lets a C++ exception escape.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "focus.h"
#include "focus_internal.hpp"

// Device scratch of focus_block_attn_importance_noalloc: the visiting order
// that call writes before its attention launch (what the workspace holds
// for focus_block_attn_importance with order = NULL). Every GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code `scratch` is only a host-side handle: its device address
// comes from hipGetSymbolAddress (see noalloc_scratch below).
constexpr int kNoAllocMaxBatch = 65536;  // sequences (256 KiB of int32)
static __device__ __align__(256) int32_t scratch[kNoAllocMaxBatch];

namespace {

thread_local std::string tl_error;

focus_status fail(focus_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  tl_error = buf;
  return s;
}

focus_status ok() {
  tl_error.clear();
  return FOCUS_OK;
}

focus_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FOCUS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

#define REQUIRE_PTR(p)                                                       \
  do {                                                                       \
    if ((p) == nullptr)                                                      \
      return fail(FOCUS_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);          \
    if (!aligned16(p))                                                       \
      return fail(FOCUS_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, \
                  #p);                                                       \
  } while (0)

#define OPTIONAL_PTR(p)                                                      \
  do {                                                                       \
    if ((p) != nullptr && !aligned16(p))                                     \
      return fail(FOCUS_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, \
                  #p);                                                       \
  } while (0)

focus_status check_attn_shape(const char* fn, int dt, int batch, int B,
                              int Hq, int Hkv, int d, int max_prefix) {
  if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
  if (B < 1 || B > 128)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
  if (Hq < 1 || Hkv < 1)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d / Hkv %d < 1", fn, Hq, Hkv);
  if (Hq > focus::kMaxHeads)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d > %d", fn, Hq, focus::kMaxHeads);
  if (max_prefix < 0)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: max_prefix %d < 0", fn, max_prefix);
  if (Hq % Hkv != 0)
    return fail(FOCUS_ERR_UNSUPPORTED, "%s: Hq %d is not a multiple of Hkv %d",
                fn, Hq, Hkv);
  if (d != 64 && d != 128)
    return fail(FOCUS_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, d);
  if (dt != FOCUS_F32 && dt != FOCUS_BF16)
    return fail(FOCUS_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dt);
  return FOCUS_OK;
}

// Query heads stacked per workgroup: up to 128 rows of rph rows each.
void head_chunks(int G, int rph, int* hpw, int* n_hc) {
  int per = focus::kRowsPerWG / rph;
  if (per < 1) per = 1;
  if (per > G) per = G;
  *hpw = per;
  *n_hc = (G + per - 1) / per;
}

// Visiting order of the attention call: the caller's (from focus_schedule),
// else the longest-prefix-first one written into the workspace by a
// one-block kernel first. (Deriving it inside every attention workgroup was
// measured slower: it delays the start of each workgroup's K/V stream.)
hipError_t plan_order(int batch, const int32_t* cu_prefix, const int32_t* order,
                      void* workspace, focus::AttnArgs* a, hipStream_t s) {
  a->batch = batch;
  if (order != nullptr) {
    a->order = order;
    return hipSuccess;
  }
  int32_t* own = static_cast<int32_t*>(workspace);
  a->order = own;
  return focus::launch_lpt_order(batch, cu_prefix, own, s);
}

float log2_scale(float scale, int d) {
  const float s = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  return s * 1.4426950408889634f;
}

// Page-table arguments of the paged entry points (none for the packed
// layout).
struct Paging {
  const int32_t* table = nullptr;
  int page_size = 0;
  int pages_per_seq = 0;
};

focus_status check_paging(const char* fn, const Paging& pg, int max_prefix) {
  if (pg.page_size < 32 || pg.page_size % 32 != 0)
    return fail(FOCUS_ERR_UNSUPPORTED, "%s: page_size %d is not a positive multiple of 32",
                fn, pg.page_size);
  if (pg.pages_per_seq < 0 ||
      (int64_t)pg.pages_per_seq * pg.page_size < (int64_t)max_prefix)
    return fail(FOCUS_ERR_INVALID_ARG,
                "%s: pages_per_seq %d x page_size %d < max_prefix %d", fn,
                pg.pages_per_seq, pg.page_size, max_prefix);
  if (max_prefix > 0 && pg.table == nullptr)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: page_table is NULL", fn);
  if (pg.table != nullptr && !aligned16(pg.table))
    return fail(FOCUS_ERR_INVALID_ARG, "%s: page_table is not 16-byte aligned", fn);
  return FOCUS_OK;
}

// Device address of `scratch` on the device that `stream` belongs to,
// looked up once per device (with that device current) and cached.
constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
int32_t* scratch_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(void* stream, int32_t** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice((hipStream_t)stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

// static_scratch: the order goes to the library's own device scratch
// (focus_block_attn_importance_noalloc); workspace is then ignored.
focus_status block_attn_impl(
    const char* fn, focus_dtype dt, int batch, int B, int Hq, int Hkv, int d,
    float scale, const void* q, const void* k_blk, const void* v_blk,
    const void* k_cache, const void* v_cache, const Paging* pg,
    const int32_t* cu_prefix, const int32_t* order, int max_prefix, void* out,
    float* imp, float* lse, void* workspace, size_t workspace_bytes, void* stream,
    bool static_scratch = false) {
  try {
    focus_status st = check_attn_shape(fn, dt, batch, B, Hq, Hkv, d, max_prefix);
    if (st != FOCUS_OK) return st;
    if (pg != nullptr) {
      st = check_paging(fn, *pg, max_prefix);
      if (st != FOCUS_OK) return st;
    }
    REQUIRE_PTR(q);
    REQUIRE_PTR(k_blk);
    REQUIRE_PTR(cu_prefix);
    REQUIRE_PTR(imp);
    OPTIONAL_PTR(out);
    OPTIONAL_PTR(lse);
    OPTIONAL_PTR(order);
    OPTIONAL_PTR(workspace);
    // out == NULL: importance (and lse) only; the values are not read.
    if (out != nullptr) REQUIRE_PTR(v_blk);
    if (max_prefix > 0) {
      REQUIRE_PTR(k_cache);
      if (out != nullptr) REQUIRE_PTR(v_cache);
    }
    size_t need = 0;
    st = focus_block_attn_importance_workspace(batch, B, Hq, Hkv, d, max_prefix, &need);
    if (st != FOCUS_OK) return st;
    if (static_scratch) {
      if (batch > kNoAllocMaxBatch)
        return fail(FOCUS_ERR_WORKSPACE,
                    "%s: batch %d exceeds the static scratch (%d sequences)", fn, batch,
                    kNoAllocMaxBatch);
      int32_t* ptr = nullptr;
      const hipError_t he = noalloc_scratch(stream, &ptr);
      if (he != hipSuccess) return hip_status(he, "static scratch lookup");
      workspace = ptr;
      workspace_bytes = sizeof(int32_t) * (size_t)kNoAllocMaxBatch;
    }
    if (order != nullptr) need = 0;  // the workspace only holds our own order
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
      return fail(FOCUS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed",
                  fn, workspace_bytes, need);
    focus::AttnArgs a = {};
    a.q = q;
    a.k_blk = k_blk;
    a.v_blk = v_blk;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.cu_prefix = cu_prefix;
    a.out = out;
    a.imp = imp;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.rph = B;
    head_chunks(a.G, B, &a.hpw, &a.n_hc);
    a.sl2 = log2_scale(scale, d);
    if (pg != nullptr) {
      a.page_table = pg->table;
      a.page_size = pg->page_size;
      a.pages_per_seq = pg->pages_per_seq;
    }
    const focus::Elem e = dt == FOCUS_BF16 ? focus::Elem::BF16 : focus::Elem::F32;
    hipError_t he = plan_order(batch, cu_prefix, order, workspace, &a, (hipStream_t)stream);
    if (he != hipSuccess) return hip_status(he, "work-order launch");
    return hip_status(focus::launch_block_attn(e, d, batch, a, (hipStream_t)stream),
                      "block attention launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status retained_attn_impl(
    const char* fn, focus_dtype dt, int batch, int B, int Hq, int Hkv, int d,
    float scale, const void* q_src, const void* k_src, const void* v_src,
    const int32_t* idx, const int32_t* cu_ret, int n_ret, int max_ret,
    const void* k_cache, const void* v_cache, const Paging* pg,
    const int32_t* cu_prefix, const int32_t* order, int max_prefix, void* out,
    void* workspace, size_t workspace_bytes, void* stream) {
  try {
    focus_status st = check_attn_shape(fn, dt, batch, B, Hq, Hkv, d, max_prefix);
    if (st != FOCUS_OK) return st;
    if (pg != nullptr) {
      st = check_paging(fn, *pg, max_prefix);
      if (st != FOCUS_OK) return st;
    }
    if (n_ret < 0) return fail(FOCUS_ERR_INVALID_ARG, "%s: n_ret %d < 0", fn, n_ret);
    if (max_ret < 0 || max_ret > B)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: max_ret %d outside [0, B=%d]", fn,
                  max_ret, B);
    if (n_ret > 0 && max_ret == 0)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: max_ret is 0 but n_ret is %d", fn, n_ret);
    if (n_ret == 0) return ok();
    REQUIRE_PTR(q_src);
    REQUIRE_PTR(k_src);
    REQUIRE_PTR(v_src);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(cu_ret);
    REQUIRE_PTR(cu_prefix);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(order);
    OPTIONAL_PTR(workspace);
    if (max_prefix > 0) {
      REQUIRE_PTR(k_cache);
      REQUIRE_PTR(v_cache);
    }
    size_t need = 0;
    st = focus_retained_attn_workspace(batch, Hq, Hkv, d, max_prefix, n_ret,
                                       max_ret, &need);
    if (st != FOCUS_OK) return st;
    if (order != nullptr) need = 0;  // the workspace only holds our own order
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
      return fail(FOCUS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed",
                  fn, workspace_bytes, need);
    focus::AttnArgs a = {};
    a.q = q_src;
    a.k_blk = k_src;
    a.v_blk = v_src;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.cu_prefix = cu_prefix;
    a.idx = idx;
    a.cu_ret = cu_ret;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.rph = max_ret;
    head_chunks(a.G, max_ret, &a.hpw, &a.n_hc);
    a.sl2 = log2_scale(scale, d);
    if (pg != nullptr) {
      a.page_table = pg->table;
      a.page_size = pg->page_size;
      a.pages_per_seq = pg->pages_per_seq;
    }
    const focus::Elem e = dt == FOCUS_BF16 ? focus::Elem::BF16 : focus::Elem::F32;
    hipError_t he = plan_order(batch, cu_prefix, order, workspace, &a, (hipStream_t)stream);
    if (he != hipSuccess) return hip_status(he, "work-order launch");
    return hip_status(
        focus::launch_retained_attn(e, d, batch, a, (hipStream_t)stream),
        "retained attention launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

}  // namespace

extern "C" {

const char* focus_version(void) { return "libfocus 0.1.0 gfx950"; }

const char* focus_status_string(focus_status s) {
  switch (s) {
    case FOCUS_OK: return "FOCUS_OK";
    case FOCUS_ERR_INVALID_ARG: return "FOCUS_ERR_INVALID_ARG";
    case FOCUS_ERR_UNSUPPORTED: return "FOCUS_ERR_UNSUPPORTED";
    case FOCUS_ERR_WORKSPACE: return "FOCUS_ERR_WORKSPACE";
    case FOCUS_ERR_HIP: return "FOCUS_ERR_HIP";
  }
  return "FOCUS_ERR_UNKNOWN";
}

const char* focus_last_error(void) { return tl_error.c_str(); }

focus_status focus_schedule(int batch, const int32_t* cu_prefix, int32_t* order,
                            void* stream) {
  const char* fn = "focus_schedule";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (cu_prefix == nullptr || order == nullptr)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: cu_prefix and order must be non-NULL", fn);
    return hip_status(focus::launch_lpt_order(batch, cu_prefix, order, (hipStream_t)stream),
                      "schedule launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_block_attn_importance_workspace(int batch, int B, int Hq,
                                                   int Hkv, int d,
                                                   int max_prefix,
                                                   size_t* bytes) {
  const char* fn = "focus_block_attn_importance_workspace";
  if (bytes == nullptr) return fail(FOCUS_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  focus_status st = check_attn_shape(fn, FOCUS_BF16, batch, B, Hq, Hkv, d, max_prefix);
  if (st != FOCUS_OK) return st;
  *bytes = focus::order_workspace_bytes(batch);
  return ok();
}

focus_status focus_block_attn_importance(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk, const void* k_cache,
    const void* v_cache, const int32_t* cu_prefix, const int32_t* order,
    int max_prefix, void* out, float* imp, float* lse, void* workspace,
    size_t workspace_bytes, void* stream) {
  return block_attn_impl("focus_block_attn_importance", dt, batch, B, Hq, Hkv, d,
                         scale, q, k_blk, v_blk, k_cache, v_cache, nullptr,
                         cu_prefix, order, max_prefix, out, imp, lse, workspace,
                         workspace_bytes, stream);
}

focus_status focus_block_attn_importance_noalloc(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk, const void* k_cache,
    const void* v_cache, const int32_t* cu_prefix, int max_prefix, void* out,
    float* imp, float* lse, void* stream) {
  return block_attn_impl("focus_block_attn_importance_noalloc", dt, batch, B, Hq, Hkv,
                         d, scale, q, k_blk, v_blk, k_cache, v_cache, nullptr,
                         cu_prefix, nullptr, max_prefix, out, imp, lse, nullptr, 0,
                         stream, /*static_scratch=*/true);
}

focus_status focus_block_attn_importance_paged(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk, const void* k_pages,
    const void* v_pages, const int32_t* page_table, int page_size,
    int pages_per_seq, const int32_t* cu_prefix, const int32_t* order,
    int max_prefix, void* out, float* imp, float* lse, void* workspace,
    size_t workspace_bytes, void* stream) {
  Paging pg;
  pg.table = page_table;
  pg.page_size = page_size;
  pg.pages_per_seq = pages_per_seq;
  return block_attn_impl("focus_block_attn_importance_paged", dt, batch, B, Hq, Hkv,
                         d, scale, q, k_blk, v_blk, k_pages, v_pages, &pg, cu_prefix,
                         order, max_prefix, out, imp, lse, workspace, workspace_bytes,
                         stream);
}

focus_status focus_delta_topk(int batch, int B, int Hq, int pool_k,
                              const float* imp0, const float* imp1,
                              const int32_t* k_keep, uint8_t* keep, float* dI,
                              void* stream) {
  const char* fn = "focus_delta_topk";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (B < 1 || B > 128)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
    if (Hq < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d < 1", fn, Hq);
    if (pool_k < 1 || pool_k > 255 || pool_k % 2 == 0)
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: pool_k %d must be odd in [1, 255]",
                  fn, pool_k);
    REQUIRE_PTR(imp0);
    REQUIRE_PTR(imp1);
    if (k_keep == nullptr) return fail(FOCUS_ERR_INVALID_ARG, "%s: k_keep is NULL", fn);
    if (keep == nullptr) return fail(FOCUS_ERR_INVALID_ARG, "%s: keep is NULL", fn);
    return hip_status(focus::launch_delta_topk(batch, B, Hq, pool_k, imp0, imp1, nullptr,
                                               0, k_keep, nullptr, 0.f, nullptr, keep,
                                               nullptr, dI, (hipStream_t)stream),
                      "delta/top-K launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_select(int batch, int B, int Hq, int pool_k, const float* imp0,
                          const float* imp1, const int32_t* k_keep, uint8_t* keep,
                          float* dI, int32_t* idx, int32_t* cu_ret, void* stream) {
  const char* fn = "focus_select";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (B < 1 || B > 128)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
    if (Hq < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d < 1", fn, Hq);
    if (pool_k < 1 || pool_k > 255 || pool_k % 2 == 0)
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: pool_k %d must be odd in [1, 255]",
                  fn, pool_k);
    REQUIRE_PTR(imp0);
    REQUIRE_PTR(imp1);
    if (k_keep == nullptr || keep == nullptr || idx == nullptr || cu_ret == nullptr)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: k_keep, keep, idx and cu_ret must be non-NULL",
                  fn);
    return hip_status(focus::launch_select(batch, B, Hq, pool_k, imp0, imp1, k_keep, keep,
                                           dI, idx, cu_ret, (hipStream_t)stream),
                      "select launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_select_masked(int batch, int B, int Hq, int pool_k,
                                 const float* imp0, const float* imp1,
                                 const uint8_t* masked, const int32_t* k_keep,
                                 int rules, uint8_t* keep, uint8_t* cand, float* dI,
                                 int32_t* idx, int32_t* cu_ret, void* stream) {
  const char* fn = "focus_select_masked";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (B < 1 || B > 128)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
    if (Hq < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d < 1", fn, Hq);
    if (pool_k < 1 || pool_k > 255 || pool_k % 2 == 0)
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: pool_k %d must be odd in [1, 255]",
                  fn, pool_k);
    if (rules & ~(FOCUS_KEEP_PREDECESSOR | FOCUS_KEEP_MASKED_PREFIX))
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: unknown rule bits 0x%x", fn, rules);
    REQUIRE_PTR(imp0);
    REQUIRE_PTR(imp1);
    if (k_keep == nullptr || keep == nullptr)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: k_keep and keep must be non-NULL", fn);
    if ((idx == nullptr) != (cu_ret == nullptr))
      return fail(FOCUS_ERR_INVALID_ARG, "%s: idx and cu_ret must be both given or both NULL",
                  fn);
    hipError_t e = focus::launch_delta_topk(batch, B, Hq, pool_k, imp0, imp1, masked, rules,
                                            k_keep, nullptr, 0.f, nullptr, keep, cand, dI,
                                            (hipStream_t)stream);
    if (e != hipSuccess || idx == nullptr) return hip_status(e, "masked delta/top-K launch");
    return hip_status(focus::launch_compact(batch, B, keep, idx, cu_ret, (hipStream_t)stream),
                      "compaction launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_select_dynamic(int batch, int B, int Hq, int pool_k,
                                  const float* imp0, const float* imp1,
                                  const uint8_t* masked, const float* yield_hist,
                                  float alpha, int rules, int32_t* k_used,
                                  uint8_t* keep, uint8_t* cand, float* dI,
                                  int32_t* idx, int32_t* cu_ret, void* stream) {
  const char* fn = "focus_select_dynamic";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (B < 1 || B > 128)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
    if (Hq < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: Hq %d < 1", fn, Hq);
    if (pool_k < 1 || pool_k > 255 || pool_k % 2 == 0)
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: pool_k %d must be odd in [1, 255]",
                  fn, pool_k);
    if (rules & ~(FOCUS_KEEP_PREDECESSOR | FOCUS_KEEP_MASKED_PREFIX))
      return fail(FOCUS_ERR_UNSUPPORTED, "%s: unknown rule bits 0x%x", fn, rules);
    if (!(alpha > 0.f) || !(alpha < 1e6f))
      return fail(FOCUS_ERR_INVALID_ARG, "%s: alpha %g outside (0, 1e6)", fn, (double)alpha);
    REQUIRE_PTR(imp0);
    REQUIRE_PTR(imp1);
    if (yield_hist == nullptr || keep == nullptr)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: yield_hist and keep must be non-NULL", fn);
    if ((idx == nullptr) != (cu_ret == nullptr))
      return fail(FOCUS_ERR_INVALID_ARG, "%s: idx and cu_ret must be both given or both NULL",
                  fn);
    hipError_t e = focus::launch_delta_topk(batch, B, Hq, pool_k, imp0, imp1, masked, rules,
                                            nullptr, yield_hist, alpha, k_used, keep, cand,
                                            dI, (hipStream_t)stream);
    if (e != hipSuccess || idx == nullptr) return hip_status(e, "dynamic delta/top-K launch");
    return hip_status(focus::launch_compact(batch, B, keep, idx, cu_ret, (hipStream_t)stream),
                      "compaction launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_compact(int batch, int B, const uint8_t* keep, int32_t* idx,
                           int32_t* cu_ret, void* stream) {
  const char* fn = "focus_compact";
  try {
    if (batch < 1) return fail(FOCUS_ERR_INVALID_ARG, "%s: batch %d < 1", fn, batch);
    if (B < 1 || B > 128)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: B %d outside [1, 128]", fn, B);
    if (keep == nullptr || idx == nullptr || cu_ret == nullptr)
      return fail(FOCUS_ERR_INVALID_ARG, "%s: keep, idx and cu_ret must be non-NULL", fn);
    return hip_status(focus::launch_compact(batch, B, keep, idx, cu_ret,
                                            (hipStream_t)stream),
                      "compaction launch");
  } catch (...) {
    return fail(FOCUS_ERR_HIP, "%s: unexpected host exception", fn);
  }
}

focus_status focus_retained_attn_workspace(int batch, int Hq, int Hkv, int d,
                                           int max_prefix, int n_ret,
                                           int max_ret, size_t* bytes) {
  const char* fn = "focus_retained_attn_workspace";
  if (bytes == nullptr) return fail(FOCUS_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  focus_status st = check_attn_shape(fn, FOCUS_BF16, batch, 1, Hq, Hkv, d, max_prefix);
  if (st != FOCUS_OK) return st;
  if (n_ret < 0 || max_ret < 0)
    return fail(FOCUS_ERR_INVALID_ARG, "%s: n_ret %d / max_ret %d < 0", fn, n_ret, max_ret);
  *bytes = focus::order_workspace_bytes(batch);
  return ok();
}

focus_status focus_retained_attn(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q_src, const void* k_src, const void* v_src,
    const int32_t* idx, const int32_t* cu_ret, int n_ret, int max_ret,
    const void* k_cache, const void* v_cache, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  return retained_attn_impl("focus_retained_attn", dt, batch, B, Hq, Hkv, d, scale,
                            q_src, k_src, v_src, idx, cu_ret, n_ret, max_ret, k_cache,
                            v_cache, nullptr, cu_prefix, order, max_prefix, out,
                            workspace, workspace_bytes, stream);
}

focus_status focus_retained_attn_paged(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q_src, const void* k_src, const void* v_src,
    const int32_t* idx, const int32_t* cu_ret, int n_ret, int max_ret,
    const void* k_pages, const void* v_pages, const int32_t* page_table,
    int page_size, int pages_per_seq, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  Paging pg;
  pg.table = page_table;
  pg.page_size = page_size;
  pg.pages_per_seq = pages_per_seq;
  return retained_attn_impl("focus_retained_attn_paged", dt, batch, B, Hq, Hkv, d,
                            scale, q_src, k_src, v_src, idx, cu_ret, n_ret, max_ret,
                            k_pages, v_pages, &pg, cu_prefix, order, max_prefix, out,
                            workspace, workspace_bytes, stream);
}

}  // extern "C"
