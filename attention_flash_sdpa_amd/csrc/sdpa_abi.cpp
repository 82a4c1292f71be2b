// sdpa_abi.cpp -- the extern "C" front end declared in include/sdpa.h:
// validation, planning and kernel launch.  Nothing here allocates device
// memory or synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "sdpa_internal.h"

namespace sdpa {
const char* last_error_text();
}

using namespace sdpa;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute-unit count of the current device, cached per device id.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kDefaultCUs;
    cached[dev] = n;
  }
  return cached[dev];
}

// A forced form of the 16-bit prefill kernels (for tuning sweeps and tests):
// narrow1 / narrow2 = one wave per SIMD with one / two key ranges, occ2 = two
// waves per SIMD, split4 = its four-key-range form, kvsplit = narrow2 with
// the key range also split across workgroups, kvsplit1 = narrow1 split across
// workgroups; "" or "auto" = the
// planner's choice.  The environment variable SDPA_PREFILL_VARIANT sets the
// initial value, read once per process; sdpa_set_prefill_variant changes it.
int variant_code(const char* e) {
  if (e == nullptr || !*e || !strcmp(e, "auto")) return 0;
  if (!strcmp(e, "narrow1")) return 3;
  if (!strcmp(e, "narrow2")) return 4;
  if (!strcmp(e, "occ2")) return 5;
  if (!strcmp(e, "split4")) return 6;
  if (!strcmp(e, "kvsplit")) return 7;
  if (!strcmp(e, "kvsplit1")) return 8;
  return -1;
}

std::atomic<int> g_variant{-1};  // -1: the environment has not been read yet

int prefill_variant() {
  int v = g_variant.load(std::memory_order_relaxed);
  if (v < 0) {
    v = variant_code(getenv("SDPA_PREFILL_VARIANT"));
    if (v < 0) v = 0;
    int expected = -1;
    if (!g_variant.compare_exchange_strong(expected, v)) v = expected;
  }
  return v;
}

sdpa_status_t hip_status(int err, const char* what) {
  if (err == 0) return SDPA_OK;
  set_error("%s: %s", what, hipGetErrorString((hipError_t)err));
  return SDPA_ERR_HIP;
}

}  // namespace

extern "C" {

int sdpa_abi_version(void) { return SDPA_ABI_VERSION; }

const char* sdpa_status_string(int status) {
  switch (status) {
    case SDPA_OK: return "SDPA_OK";
    case SDPA_ERR_NULL_PTR: return "SDPA_ERR_NULL_PTR: a required pointer is NULL";
    case SDPA_ERR_BAD_SHAPE: return "SDPA_ERR_BAD_SHAPE: invalid problem shape";
    case SDPA_ERR_BAD_SCALE: return "SDPA_ERR_BAD_SCALE: scale or descale not finite or negative";
    case SDPA_ERR_UNSUPPORTED: return "SDPA_ERR_UNSUPPORTED: dtype / head-dim combination not supported";
    case SDPA_ERR_MISALIGNED: return "SDPA_ERR_MISALIGNED: data pointer not 16-byte aligned";
    case SDPA_ERR_WORKSPACE: return "SDPA_ERR_WORKSPACE: workspace missing or too small";
    case SDPA_ERR_HIP: return "SDPA_ERR_HIP: HIP runtime error";
    default: return "unknown sdpa status";
  }
}

const char* sdpa_last_error(void) { return last_error_text(); }

sdpa_status_t sdpa_set_prefill_variant(const char* name) {
  clear_error();
  const int v = variant_code(name);
  if (v < 0) {
    set_error("unknown prefill variant \"%s\"", name);
    return SDPA_ERR_UNSUPPORTED;
  }
  g_variant.store(v, std::memory_order_relaxed);
  return SDPA_OK;
}

sdpa_status_t sdpa_plan(const sdpa_problem_t* problem, int is_decode, int num_cus, int num_splits,
                        sdpa_plan_t* plan) {
  clear_error();
  if (problem == nullptr || plan == nullptr) {
    set_error("problem and plan must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  // a prefill plan is the one sdpa_prefill_fwd runs when given its workspace
  return make_plan(*problem, is_decode != 0, num_cus, num_splits, plan, is_decode ? 0 : prefill_variant(), false,
                   is_decode == 0);
}

sdpa_status_t sdpa_loop_counts(int q_len, int kv_len, int d_qk, int d_v, int block_q, int block_k,
                               int block_d, int block_v, int causal, sdpa_loop_counts_t* out) {
  clear_error();
  if (out == nullptr) {
    set_error("out must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  return loop_counts(q_len, kv_len, d_qk, d_v, block_q, block_k, block_d, block_v, causal != 0, out);
}

size_t sdpa_prefill_workspace_bytes(const sdpa_problem_t* problem) {
  if (problem == nullptr) return 0;
  sdpa_plan_t plan;
  if (make_plan(*problem, false, device_cus(), 0, &plan, prefill_variant(), false, true) != SDPA_OK) return 0;
  return (size_t)plan.workspace_bytes;
}

size_t sdpa_decode_workspace_bytes(const sdpa_problem_t* problem, int num_splits) {
  if (problem == nullptr) return 0;
  sdpa_plan_t plan;
  if (make_plan(*problem, true, device_cus(), num_splits, &plan) != SDPA_OK) return 0;
  return (size_t)plan.workspace_bytes;
}

// Fills the kernel arguments of a planned prefill and launches it; a plan
// split across workgroups (kv_splits > 1) keeps its partials in workspace and
// is followed by the combine.
static sdpa_status_t prefill_launch(const sdpa_problem_t& p, const sdpa_plan_t& plan, const void* q, const void* k,
                                    const void* v, void* o, float* lse, const void* k_cache, const void* v_cache,
                                    int32_t cache_len, int32_t cache_cap, void* stream, void* workspace = nullptr) {
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = p.batch;
  a.q_len = p.q_len;
  a.kv_len = p.kv_len;
  a.head_q = p.head_q;
  a.head_kv = p.head_kv;
  a.group = p.head_q / p.head_kv;
  a.heads_per_group = plan.heads_per_group;
  a.qtiles_per_group = plan.qtiles_per_group;
  a.q_tiles = plan.q_tiles;
  a.head_groups = (a.group + plan.heads_per_group - 1) / plan.heads_per_group;
  a.num_groups = plan.num_groups;
  a.s2 = (float)((double)p.scale * 1.4426950408889634 * (double)p.q_descale * (double)p.k_descale);
  a.v_descale = p.v_descale;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_len = cache_len;
  a.cache_cap = cache_cap;
  const int64_t rows = (int64_t)p.batch * p.q_len * p.head_q;
  if (plan.kv_splits > 1) {
    const uint64_t po = (uint64_t)rows * plan.kv_splits * p.d_v * 4;
    a.kv_splits = plan.kv_splits;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)((char*)workspace + ((po + 255) / 256) * 256);
  }
  sdpa_status_t st = hip_status(launch_prefill(a, plan, p.causal != 0, (ihipStream_t*)stream), "prefill launch");
  if (st != SDPA_OK || plan.kv_splits <= 1) return st;
  // the combine sees one row per (batch, query row, query head)
  DecodeArgs c{};
  c.o = o;
  c.lse = lse;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.batch = p.batch * p.q_len;
  c.head_q = p.head_q;
  c.num_splits = plan.kv_splits;
  c.v_descale = a.v_descale;
  c.lse_q_len = p.q_len;
  return hip_status(launch_split_combine(c, p.in_dtype, p.d_v, plan.combine_groups, (ihipStream_t*)stream),
                    "prefill combine launch");
}

sdpa_status_t sdpa_prefill_fwd(const sdpa_problem_t* problem, const void* q, const void* k, const void* v,
                               void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  const sdpa_problem_t& p = *problem;
  sdpa_plan_t plan;
  sdpa_status_t st = make_plan(p, false, device_cus(), 0, &plan, prefill_variant(), false, true);
  if (st != SDPA_OK) return st;
  if (p.batch == 0 || p.q_len == 0) return SDPA_OK;
  if (o == nullptr || q == nullptr || (p.kv_len > 0 && (k == nullptr || v == nullptr))) {
    set_error("q, k, v and o must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  const bool use_ws = plan.workspace_bytes > 0 && workspace != nullptr && workspace_bytes >= plan.workspace_bytes;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (use_ws && !aligned16(workspace)) ||
      ((uintptr_t)lse & 3u)) {
    set_error("q, k, v, o, workspace must be 16-byte aligned and lse 4-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  if (plan.workspace_bytes > 0 && !use_ws) {
    // no room for the partials: the same problem without the split
    st = make_plan(p, false, device_cus(), 0, &plan, prefill_variant(), false, false);
    if (st != SDPA_OK) return st;
  }
  return prefill_launch(p, plan, q, k, v, o, lse, nullptr, nullptr, 0, 0, stream, workspace);
}

size_t sdpa_prefill_cached_workspace_bytes(const sdpa_problem_t* problem, int32_t cache_len) {
  if (problem == nullptr || cache_len < 0 || problem->kv_len < 0 ||
      (int64_t)problem->kv_len + cache_len > INT32_MAX)
    return 0;
  sdpa_problem_t vp = *problem;
  vp.kv_len = cache_len + problem->kv_len;
  sdpa_plan_t plan;
  if (make_plan(vp, false, device_cus(), 0, &plan, prefill_variant(), cache_len > 0, true) != SDPA_OK) return 0;
  return (size_t)plan.workspace_bytes;
}

sdpa_status_t sdpa_prefill_cached_fwd(const sdpa_problem_t* problem, const void* q, const void* k_cache,
                                      const void* v_cache, int32_t cache_len, int32_t cache_cap, const void* k,
                                      const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  const sdpa_problem_t& p = *problem;
  if (cache_len < 0 || cache_cap < cache_len) {
    set_error("need 0 <= cache_len <= cache_cap (cache_len=%d, cache_cap=%d)", cache_len, cache_cap);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (p.causal && p.q_len > p.kv_len) {
    set_error("causal cached prefill needs q_len <= new keys (q_len=%d, kv_len=%d)", p.q_len, p.kv_len);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (p.kv_len < 0 || (int64_t)p.kv_len + cache_len > INT32_MAX) {
    set_error("cache_len + kv_len out of range (%d + %d)", cache_len, p.kv_len);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (cache_len == 0)  // nothing cached: the plain prefill
    return sdpa_prefill_fwd(problem, q, k, v, o, lse, workspace, workspace_bytes, stream);
  // one sequence of cache_len + kv_len keys for the planner and the kernel
  sdpa_problem_t vp = p;
  vp.kv_len = cache_len + p.kv_len;
  sdpa_plan_t plan;
  sdpa_status_t st = make_plan(vp, false, device_cus(), 0, &plan, prefill_variant(), true, true);
  if (st != SDPA_OK) return st;
  const bool use_ws = plan.workspace_bytes > 0 && workspace != nullptr && workspace_bytes >= plan.workspace_bytes;
  if (use_ws && !aligned16(workspace)) {
    set_error("workspace must be 16-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  if (plan.workspace_bytes > 0 && !use_ws) {
    // no room for the partials: the same problem without the split
    st = make_plan(vp, false, device_cus(), 0, &plan, prefill_variant(), true, false);
    if (st != SDPA_OK) return st;
  }
  if ((int64_t)cache_cap * p.head_kv * (p.d_qk > p.d_v ? p.d_qk : p.d_v) >= (int64_t)1 << 31) {
    set_error("one batch entry of the cache exceeds 2^31 elements (cache_cap=%d)", cache_cap);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (p.batch == 0 || p.q_len == 0) return SDPA_OK;
  if (o == nullptr || q == nullptr || k_cache == nullptr || v_cache == nullptr ||
      (p.kv_len > 0 && (k == nullptr || v == nullptr))) {
    set_error("q, k_cache, v_cache, k, v and o must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(k_cache) ||
      !aligned16(v_cache) || ((uintptr_t)lse & 3u)) {
    set_error("q, k, v, o, k_cache, v_cache must be 16-byte aligned and lse 4-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  return prefill_launch(vp, plan, q, k, v, o, lse, k_cache, v_cache, cache_len, cache_cap, stream, workspace);
}

sdpa_status_t sdpa_mask_convert(const uint8_t* mask, void* out, int64_t n, int32_t out_dtype, void* stream) {
  clear_error();
  if (n < 0) {
    set_error("n must not be negative (got %lld)", (long long)n);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (out_dtype != SDPA_F16 && out_dtype != SDPA_BF16) {
    set_error("mask conversion writes fp16 or bf16 (got out_dtype=%d)", out_dtype);
    return SDPA_ERR_UNSUPPORTED;
  }
  if (n == 0) return SDPA_OK;
  if (mask == nullptr || out == nullptr) {
    set_error("mask and out must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  if (!aligned16(mask) || !aligned16(out)) {
    set_error("mask and out must be 16-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  return hip_status(launch_mask_convert(mask, out, n, out_dtype, (ihipStream_t*)stream), "mask conversion launch");
}

sdpa_status_t sdpa_hbm_read_probe(const void* data, int64_t bytes, uint32_t* sink, void* stream) {
  clear_error();
  if (bytes < 0 || bytes % 16 != 0) {
    set_error("bytes must be a non-negative multiple of 16 (got %lld)", (long long)bytes);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (bytes == 0) return SDPA_OK;
  if (data == nullptr || sink == nullptr) {
    set_error("data and sink must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  if (!aligned16(data) || ((uintptr_t)sink & 3) != 0) {
    set_error("data must be 16-byte and sink 4-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  return hip_status(launch_hbm_read_probe(data, bytes, sink, (ihipStream_t*)stream), "read probe launch");
}

sdpa_status_t sdpa_prefill_masked_fwd(const sdpa_problem_t* problem, const void* q, const void* k, const void* v,
                                      const void* mask, int64_t mask_stride_b, int64_t mask_stride_h,
                                      int32_t mask_stride_row, void* o, float* lse, void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  const sdpa_problem_t& p = *problem;
  sdpa_plan_t plan;  // shape, head and scale checks shared with the plain prefill
  sdpa_status_t st = make_plan(p, false, device_cus(), 0, &plan);
  if (st != SDPA_OK) return st;
  if (p.in_dtype == SDPA_FP8_E4M3 || p.out_dtype != p.in_dtype || p.d_qk != p.d_v) {
    set_error("the masked prefill takes fp16/bf16 inputs with the same output type and d_qk == d_v "
              "(in=%d out=%d d_qk=%d d_v=%d)", p.in_dtype, p.out_dtype, p.d_qk, p.d_v);
    return SDPA_ERR_UNSUPPORTED;
  }
  const int64_t min_row = p.kv_len > 8 ? p.kv_len : 8;
  if (p.kv_len > 0 &&  // without keys the mask is never read
      (mask_stride_b < 0 || mask_stride_h < 0 || mask_stride_row < min_row || mask_stride_row % 8 != 0 ||
       mask_stride_b % 8 != 0 || mask_stride_h % 8 != 0)) {
    set_error("mask strides must be >= 0 and multiples of 8 elements, the row stride >= max(kv_len, 8) "
              "(b=%lld h=%lld row=%d kv_len=%d)", (long long)mask_stride_b, (long long)mask_stride_h,
              mask_stride_row, p.kv_len);
    return SDPA_ERR_BAD_SHAPE;
  }
  // the two-waves-per-SIMD shape (one key range, 64-key blocks, four waves)
  // with the bias added in its softmax
  st = make_plan(p, false, device_cus(), 0, &plan, 5);
  if (st != SDPA_OK) return st;
  if (p.batch == 0 || p.q_len == 0) return SDPA_OK;
  if (o == nullptr || q == nullptr || (p.kv_len > 0 && (k == nullptr || v == nullptr || mask == nullptr))) {
    set_error("q, k, v, mask and o must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(mask) ||
      ((uintptr_t)lse & 3u)) {
    set_error("q, k, v, mask, o must be 16-byte aligned and lse 4-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = p.batch;
  a.q_len = p.q_len;
  a.kv_len = p.kv_len;
  a.head_q = p.head_q;
  a.head_kv = p.head_kv;
  a.group = p.head_q / p.head_kv;
  a.heads_per_group = plan.heads_per_group;
  a.qtiles_per_group = plan.qtiles_per_group;
  a.q_tiles = plan.q_tiles;
  a.head_groups = (a.group + plan.heads_per_group - 1) / plan.heads_per_group;
  a.num_groups = plan.num_groups;
  a.s2 = (float)((double)p.scale * 1.4426950408889634);
  a.s_nat = p.scale;
  a.v_descale = 1.f;
  a.mask = mask;
  a.mask_sb = mask_stride_b;
  a.mask_sh = mask_stride_h;
  a.mask_row = mask_stride_row;
  return hip_status(launch_prefill_o2_bias(a, plan, p.causal != 0, (ihipStream_t*)stream), "masked prefill launch");
}

// Shared by the dense and the paged decode entry points; cache rows per
// page and the table are checked by the caller.
static sdpa_status_t decode_common(const sdpa_problem_t* problem, const void* q, const void* k, const void* v,
                                   void* o, float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                                   void* stream, const int32_t* seq_lens, const int32_t* page_table,
                                   int32_t num_pages, int32_t page_size, int32_t pages_per_seq) {
  const sdpa_problem_t& p = *problem;
  sdpa_plan_t plan;
  sdpa_status_t st = make_plan(p, true, device_cus(), num_splits, &plan);
  if (st != SDPA_OK) return st;
  if (p.batch == 0) return SDPA_OK;
  if (o == nullptr || q == nullptr || (p.kv_len > 0 && (k == nullptr || v == nullptr))) {
    set_error("q, k, v and o must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
      ((uintptr_t)lse & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)page_table & 3u)) {
    set_error("q, k, v, o, workspace must be 16-byte aligned and lse, seq_lens, page_table 4-byte aligned");
    return SDPA_ERR_MISALIGNED;
  }
  if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
    set_error("workspace of %llu bytes needed, %llu given", (unsigned long long)plan.workspace_bytes,
              (unsigned long long)workspace_bytes);
    return SDPA_ERR_WORKSPACE;
  }
  DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  const uint64_t po = (uint64_t)p.batch * p.head_q * plan.num_splits * p.d_v * 4;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ((po + 255) / 256) * 256);
  a.batch = p.batch;
  a.kv_len = p.kv_len;
  a.head_q = p.head_q;
  a.head_kv = p.head_kv;
  a.group = p.head_q / p.head_kv;
  a.num_splits = plan.num_splits;
  a.blocks_per_split = plan.blocks_per_split;
  a.split_waves = plan.num_splits;
  a.gtiles = (a.group + kDecodeMaxGroup - 1) / kDecodeMaxGroup;
  a.s2 = (float)((double)p.scale * 1.4426950408889634 * (double)p.q_descale * (double)p.k_descale);
  a.v_descale = p.v_descale;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  return hip_status(launch_decode(a, plan, (ihipStream_t*)stream), "decode launch");
}

sdpa_status_t sdpa_decode_fwd(const sdpa_problem_t* problem, const void* q, const void* k, const void* v,
                              void* o, float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                              void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  return decode_common(problem, q, k, v, o, lse, num_splits, workspace, workspace_bytes, stream, nullptr, nullptr,
                       0, 0, 0);
}

sdpa_status_t sdpa_decode_fwd_noalloc(const sdpa_problem_t* problem, const void* q, const void* k, const void* v,
                                      void* o, float* lse, int num_splits, void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  sdpa_plan_t plan;
  sdpa_status_t st = make_plan(*problem, true, device_cus(), num_splits, &plan);
  if (st != SDPA_OK) return st;
  if (plan.workspace_bytes > kNoAllocScratchBytes) {
    set_error("the split partials need %llu bytes, more than the %llu-byte static scratch of the no-allocation "
              "decode; use sdpa_decode_fwd with a workspace", (unsigned long long)plan.workspace_bytes,
              (unsigned long long)kNoAllocScratchBytes);
    return SDPA_ERR_WORKSPACE;
  }
  if (problem->batch == 0) return SDPA_OK;
  void* ws = nullptr;
  const int e = noalloc_scratch(&ws);
  if (e != 0) return hip_status(e, "static decode scratch lookup");
  return decode_common(problem, q, k, v, o, lse, num_splits, ws, kNoAllocScratchBytes, stream, nullptr, nullptr, 0,
                       0, 0);
}

sdpa_status_t sdpa_decode_paged_fwd(const sdpa_problem_t* problem, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t num_pages, int32_t page_size, int32_t pages_per_seq, void* o,
                                    float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  clear_error();
  if (problem == nullptr) {
    set_error("problem must not be NULL");
    return SDPA_ERR_NULL_PTR;
  }
  const sdpa_problem_t& p = *problem;
  if (page_table != nullptr && p.batch > 0 && p.kv_len > 0) {
    if (!(page_size == 8 || page_size == 16 || (page_size > 0 && page_size % kDecodeBlockK == 0))) {
      set_error("page_size must be 8, 16 or a positive multiple of %d (got %d)", kDecodeBlockK, page_size);
      return SDPA_ERR_BAD_SHAPE;
    }
    if (num_pages <= 0 || pages_per_seq <= 0 || (int64_t)pages_per_seq * page_size < p.kv_len) {
      set_error("need num_pages > 0 and pages_per_seq * page_size >= kv_len (num_pages=%d, pages_per_seq=%d, "
                "page_size=%d, kv_len=%d)", num_pages, pages_per_seq, page_size, p.kv_len);
      return SDPA_ERR_BAD_SHAPE;
    }
    if ((int64_t)num_pages * page_size > INT32_MAX || (int64_t)p.batch * pages_per_seq > INT32_MAX) {
      set_error("page pool or table too large (num_pages=%d, page_size=%d, pages_per_seq=%d)", num_pages,
                page_size, pages_per_seq);
      return SDPA_ERR_BAD_SHAPE;
    }
  }
  return decode_common(problem, q, k_cache, v_cache, o, lse, num_splits, workspace, workspace_bytes, stream,
                       seq_lens, page_table, num_pages, page_size, pages_per_seq);
}

}  // extern "C"
