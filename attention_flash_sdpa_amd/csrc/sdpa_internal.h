// sdpa_internal.h -- host-side interfaces between the C-ABI front end, the
// planner and the kernel launchers.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sdpa.h"

struct ihipStream_t;

namespace sdpa {

// Kernel instantiation ids chosen by the planner.
enum KernelId : int32_t {
  kPrefillF16D64 = 0,
  kPrefillBf16D64 = 1,
  kPrefillF16D128 = 2,
  kPrefillBf16D128 = 3,
  kPrefillFp8D192 = 4,
  kOccF16D64 = 12,  // 32-row kernel, two waves per SIMD (large grids)
  kOccBf16D64 = 13,
  kOccF16D128 = 14,
  kOccBf16D128 = 15,
  kDecodeF16D64 = 16,
  kDecodeBf16D64 = 17,
  kDecodeF16D128 = 18,
  kDecodeBf16D128 = 19,
  kSplitF16D64 = 24,  // 32-row kernel, 8 waves: 2 heads x 4 key ranges (small grids)
  kSplitBf16D64 = 25,
  kSplitF16D128 = 26,
  kSplitBf16D128 = 27,
};

constexpr int kRowsPerWave = 32;   // prefill: query rows per wave (MFMA N)
constexpr int kPrefillWaves = 4;   // prefill: waves per workgroup
constexpr int kPrefillBlockK = 64; // prefill: keys per K/V block
constexpr int kSplitWaves = 8;     // 4-range prefill: waves per workgroup
constexpr int kSplitRanges = 4;    // 4-range prefill: key ranges per workgroup
constexpr int kSplitBlockK = 32;   // 4-range prefill: keys per K/V block
constexpr int kDecodeBlockK = 32;  // decode: keys per K/V block
constexpr int kLdsPerCu = 160 * 1024;  // LDS bytes per CU (gfx950)
constexpr int kCombineRows = 4;    // decode combine: (batch, query head) rows per workgroup
constexpr int kDecodeMaxGroup = 16;  // decode: query heads per wave (MFMA N); larger groups take several waves
constexpr int kDecodeWaves = 4;    // decode: waves (= splits) per workgroup
constexpr int64_t kMaskMaxGroups = (int64_t)1 << 30;  // mask conversion: grid cap (beyond it, a grid-stride loop)
constexpr int kDefaultCUs = 256;
constexpr int kMinSplitBlocks = 4;  // prefill split across workgroups: K blocks per key range, at least
constexpr int kMinSplitSaving = 5;  // ... and mainloop iterations it saves per range, at least

// Validates the problem; fills *plan.  Writes a detail message through
// set_error() on failure.  Pure host code.
// variant: 0 = planner's choice, 3 / 4 = the one-wave-per-SIMD 32-row
// kernel with one / two key ranges per workgroup, 5 = the two-waves-per-SIMD
// 32-row kernel, 6 = its 8-wave, four-key-range form (tuning sweeps and tests
// only), 7 = variant 4 with the key range also split across workgroups
// (kv_splits >= 2), 8 = the same with one key range per workgroup.  cached: a cached-KV prefill (kv_len counts cache and new
// keys), which the 16-bit kernels implement (not the fp8 one).  kv_split:
// whether the plan may split key ranges across workgroups (the caller has a
// workspace for the partials).
sdpa_status_t make_plan(const sdpa_problem_t& p, bool is_decode, int num_cus, int num_splits,
                        sdpa_plan_t* plan, int variant = 0, bool cached = false, bool kv_split = false);

sdpa_status_t loop_counts(int q_len, int kv_len, int d_qk, int d_v, int block_q, int block_k, int block_d,
                          int block_v, bool causal, sdpa_loop_counts_t* out);

void set_error(const char* fmt, ...);
void clear_error();

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t batch, q_len, kv_len, head_q, head_kv, group;
  int32_t heads_per_group, qtiles_per_group, q_tiles, head_groups, num_groups;
  float s2;         // scale * log2(e) * q_descale * k_descale
  float v_descale;  // applied to the output (fp8 inputs), else 1
  // cached-KV prefill: keys 0 .. cache_len-1 come from k_cache / v_cache
  // ([batch, cache_cap, head_kv, d]), keys cache_len .. kv_len-1 from k / v
  // ([batch, kv_len - cache_len, head_kv, d]); unused otherwise
  const void* k_cache;
  const void* v_cache;
  int32_t cache_len, cache_cap;
  // additive bias (the masked prefill; NULL otherwise): the value for (b, h,
  // row i, key j) is mask[b*mask_sb + h*mask_sh + i*mask_row + j] in the
  // inputs' 16-bit type; mask_row is a multiple of 8 and >= max(kv_len, 8)
  const void* mask;
  int64_t mask_sb, mask_sh;
  int32_t mask_row;
  float s_nat;      // the softmax scale itself (natural-log domain)
  // key range split across kv_splits workgroups (one-wave kernel only): each
  // writes unnormalized fp32 partials of its rows to part_o [batch, q_len,
  // head_q, kv_splits, d_v] and (max in log2 domain, sum) to part_ml [...,
  // 2] instead of O and lse; 1 = no split, O and lse written directly
  int32_t kv_splits = 1;
  float* part_o = nullptr;
  float* part_ml = nullptr;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;    // [batch, head_q, splits, d_v]
  float* part_ml;   // [batch, head_q, splits, 2] = (max in log2 domain, sum)
  int32_t batch, kv_len, head_q, head_kv, group;
  int32_t num_splits, blocks_per_split, split_waves;
  int32_t gtiles;   // tiles of up to 16 query heads per KV head (the MFMA N dimension)
  float s2;
  float v_descale;
  // variable-length and paged key/value caches (both NULL: every sequence
  // holds kv_len keys in a dense [batch, kv_len, head_kv, d] cache)
  const int32_t* seq_lens;    // [batch] keys per sequence, or NULL
  const int32_t* page_table;  // [batch, pages_per_seq] physical page ids, or NULL
  int32_t num_pages, page_size, pages_per_seq;
  // combine only: query rows per (batch, head) lse row.  The combine's rows
  // are bh = b' * head_q + h over b' < batch; its lse goes to lse[bh] when
  // lse_q_len <= 1 (decode), else to the prefill layout [batch / lse_q_len,
  // head_q, lse_q_len] with b' = b * lse_q_len + i
  int32_t lse_q_len;
};

int launch_prefill(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream);
int launch_prefill_fp8(const PrefillArgs& a, int causal, ihipStream_t* stream);
int launch_prefill_o2(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream);
// the two-waves-per-SIMD kernel with the additive bias a.mask (masked prefill)
int launch_prefill_o2_bias(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream);
int launch_prefill_cached(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream);
// the one-wave kernel with its keys split across workgroups (plan.kv_splits >
// 1), dense (a.k_cache == NULL) or cached; partials only, the caller launches
// the combine
int launch_prefill_split(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream);
int launch_mask_convert(const uint8_t* in, void* out, int64_t n, int out_dtype, ihipStream_t* stream);
// HBM streaming-read probe (mask.hip): kProbeGroups workgroups
constexpr int kProbeGroups = 2048;
int launch_hbm_read_probe(const void* data, int64_t bytes, uint32_t* sink, ihipStream_t* stream);

int launch_decode(const DecodeArgs& a, const sdpa_plan_t& plan, ihipStream_t* stream);
// the decode combine kernel alone over `groups` workgroups (the prefill's
// split across workgroups), for 16-bit in_dtype and d_v 64 / 128
int launch_split_combine(const DecodeArgs& a, int in_dtype, int d_v, int groups, ihipStream_t* stream);

// The no-allocation decode keeps its split partials in a static device array
// of this size (per GPU); larger problems are refused.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
// Device address of that array on the current GPU (looked up on the first
// call per device, then cached).  Returns a hipError_t value (0 = success).
int noalloc_scratch(void** ptr);

}  // namespace sdpa
