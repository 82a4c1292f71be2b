// planner.cpp -- argument validation and the tile-config / launch planner.
// Pure host code: no HIP calls, testable without a GPU through sdpa_plan().
//
// The planner plays the role the pages give to host-side dispatch: the launcher
// selection keyed on dtype and head dim ("Xe SDPA Forward Mainloop", section
// "Who decides the instantiated mainloop?") and loop counts precomputed on the
// host ("xe2-sdp-kernels", section "Inner-loop rules").
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sdpa_bounds.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

thread_local char g_last_error[512];

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is16(int dt) { return dt == SDPA_F16 || dt == SDPA_BF16; }

int prefill_kernel_id(const sdpa_problem_t& p) {
  if (is16(p.in_dtype) && p.out_dtype == p.in_dtype && p.d_qk == p.d_v) {
    const bool bf = p.in_dtype == SDPA_BF16;
    if (p.d_qk == 64) return bf ? kPrefillBf16D64 : kPrefillF16D64;
    if (p.d_qk == 128) return bf ? kPrefillBf16D128 : kPrefillF16D128;
  }
  if (p.in_dtype == SDPA_FP8_E4M3 && p.d_qk == 192 && p.d_v == 128 && p.out_dtype == SDPA_BF16)
    return kPrefillFp8D192;
  return -1;
}

int decode_kernel_id(const sdpa_problem_t& p) {
  if (is16(p.in_dtype) && p.out_dtype == p.in_dtype && p.d_qk == p.d_v) {
    const bool bf = p.in_dtype == SDPA_BF16;
    if (p.d_qk == 64) return bf ? kDecodeBf16D64 : kDecodeF16D64;
    if (p.d_qk == 128) return bf ? kDecodeBf16D128 : kDecodeF16D128;
  }
  return -1;
}

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = 0; }

const char* last_error_text() { return g_last_error; }

sdpa_status_t make_plan(const sdpa_problem_t& p, bool is_decode, int num_cus, int num_splits,
                        sdpa_plan_t* plan, int variant, bool cached, bool kv_split) {
  memset(plan, 0, sizeof *plan);
  if (num_cus <= 0) num_cus = kDefaultCUs;
  if (p.batch < 0 || p.q_len < 0 || p.kv_len < 0) {
    set_error("negative size: batch=%d q_len=%d kv_len=%d", p.batch, p.q_len, p.kv_len);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (p.head_q <= 0 || p.head_kv <= 0 || p.head_q % p.head_kv != 0) {
    set_error("head_q=%d must be a positive multiple of head_kv=%d", p.head_q, p.head_kv);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (p.d_qk <= 0 || p.d_v <= 0) {
    set_error("head dims must be positive (d_qk=%d d_v=%d)", p.d_qk, p.d_v);
    return SDPA_ERR_BAD_SHAPE;
  }
  if (!isfinite(p.scale) || p.scale < 0.f) {
    set_error("scale must be finite and >= 0 (got %g)", (double)p.scale);
    return SDPA_ERR_BAD_SCALE;
  }
  const float ds[3] = {p.q_descale, p.k_descale, p.v_descale};
  for (float d : ds) {
    if (!isfinite(d) || d < 0.f) {
      set_error("descale factors must be finite and >= 0 (got %g)", (double)d);
      return SDPA_ERR_BAD_SCALE;
    }
    // dequantisation factors belong to fp8 inputs only: a 16-bit tensor holds
    // its values as they are, so any other factor would silently rescale them
    if (p.in_dtype != SDPA_FP8_E4M3 && d != 1.f) {
      set_error("descale factors must be 1 for fp16/bf16 inputs (got %g)", (double)d);
      return SDPA_ERR_BAD_SCALE;
    }
  }
  const int64_t G = p.head_q / p.head_kv;
  // element offsets inside one batch entry are 32-bit in the kernels
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)p.q_len * p.head_q * (p.d_qk > p.d_v ? p.d_qk : p.d_v) >= lim ||
      (int64_t)p.kv_len * p.head_kv * (p.d_qk > p.d_v ? p.d_qk : p.d_v) * 2 >= lim) {
    set_error("one batch entry exceeds 2^31 elements (q_len=%d kv_len=%d)", p.q_len, p.kv_len);
    return SDPA_ERR_BAD_SHAPE;
  }

  if (!is_decode) {
    int kid = prefill_kernel_id(p);
    if (cached && kid == kPrefillFp8D192) kid = -1;  // the fp8 kernel reads one K/V tensor
    if (kid < 0) {
      set_error("unsupported prefill (in_dtype=%d, out_dtype=%d, d_qk=%d, d_v=%d)", p.in_dtype, p.out_dtype,
                p.d_qk, p.d_v);
      return SDPA_ERR_UNSUPPORTED;
    }
    const int rows = kRowsPerWave;
    plan->kernel = kid;
    plan->waves_per_group = kPrefillWaves;
    plan->rows_per_wave = rows;
    plan->block_k = kPrefillBlockK;
    plan->stages = 2;
    plan->kv_blocks = (int32_t)ceil_div(p.kv_len, plan->block_k);
    // Pack query heads of one GQA group into the workgroup when the group
    // size allows it (K/V blocks in LDS are then shared by several heads);
    // otherwise stack consecutive query tiles of one head.  Short queries
    // pack heads even when the group size is not a multiple of the pack.
    auto shape = [&](int waves, int* hp_out, int* qt_out) -> int64_t {
      int hp;
      if (G % 4 == 0) hp = 4;
      else if (G % 2 == 0) hp = 2;
      else hp = 1;
      if (p.q_len <= rows) hp = (int)(G < waves ? G : waves);
      if (hp > waves) hp = waves;
      while (waves % hp) --hp;
      const int qtiles = waves / hp;
      *hp_out = hp;
      *qt_out = qtiles;
      return (int64_t)p.batch * p.head_kv * ceil_div(G, hp) * ceil_div(p.q_len, (int64_t)rows * qtiles);
    };
    int hp, qtiles, ks = 1;
    int64_t groups = shape(kPrefillWaves, &hp, &qtiles);
    // Too few workgroups to give every CU one: split the key range of each
    // workgroup in two halves, each streamed by half of its waves and merged
    // at the end, which doubles the workgroup count.
    bool split = kid != kPrefillFp8D192 && groups < num_cus && plan->kv_blocks >= 2;
    if (variant == 3 || variant == 5 || variant == 8) split = false;
    if (variant == 4 || variant == 7) split = kid != kPrefillFp8D192;
    if (split) {
      ks = 2;
      groups = shape(kPrefillWaves / 2, &hp, &qtiles);
    }
    // More workgroups than CUs: the two-waves-per-SIMD form keeps two of them
    // on every CU at once (the one-wave form would run in rounds).
    bool occ2 = kid != kPrefillFp8D192 && ks == 1 && groups > num_cus;
    if (variant == 3 || variant == 4 || variant == 7 || variant == 8) occ2 = false;
    if (variant == 5) occ2 = kid != kPrefillFp8D192;
    if (occ2) plan->kernel = kid - kPrefillF16D64 + kOccF16D64;
    // Four key ranges of 32-key blocks, two waves (heads or query tiles) per
    // range, 8 waves per workgroup at two waves per SIMD: the same grid as the
    // two-range split with twice the waves in flight.
    bool split4 = false;
    if (variant == 6) split4 = kid != kPrefillFp8D192;
    if (split4) {
      ks = kSplitRanges;
      groups = shape(kSplitWaves / kSplitRanges, &hp, &qtiles);
      plan->kernel = kid - kPrefillF16D64 + kSplitF16D64;
      plan->waves_per_group = kSplitWaves;
      plan->block_k = kSplitBlockK;
      plan->kv_blocks = (int32_t)ceil_div(p.kv_len, plan->block_k);
    }
    // Even the two-range split leaves more than half the CUs idle (short
    // queries over a long key sequence): split each tile's K blocks across
    // kvs workgroups as well, at most one workgroup per CU, no range shorter
    // than kMinSplitBlocks blocks.  They write fp32 partials that a second
    // kernel combines, which only pays when it multiplies the grid and
    // shortens the ranges by at least kMinSplitSaving iterations; the range
    // count is then evened out so that no range is left empty.
    // Short-query rows are few, so the partials stay small next to K/V.
    // Once split this way, one key range per workgroup (all four waves on
    // one K/V stream: four heads of a group, or four query tiles) with twice
    // the workgroups measured 0-8% faster than two ranges of two waves: each
    // block is loaded once for four waves instead of twice for two.
    int64_t kvs = 1;
    const int64_t rows_all = (int64_t)p.batch * p.q_len * p.head_q;
    auto auto_kvs = [&](int64_t g, int r) -> int64_t {  // g workgroups per split, r ranges each
      if (2 * g > num_cus) return 1;
      int64_t n = num_cus / g;  // whole rounds: no workgroup waits for a free CU
      const int64_t by_len = plan->kv_blocks / (r * kMinSplitBlocks);
      if (n > by_len) n = by_len;
      if (n < 2) return 1;
      const int64_t per = ceil_div(plan->kv_blocks, r * n);  // blocks per range
      n = ceil_div(plan->kv_blocks, r * per);
      // the combine costs about what four mainloop iterations do
      return ceil_div(plan->kv_blocks, r) - per < kMinSplitSaving ? 1 : n;
    };
    const bool one_wave = plan->kernel == kid && kid != kPrefillFp8D192 && (ks == 2 || variant == 8);
    if (kv_split && one_wave && groups > 0 && (variant == 0 || variant == 7 || variant == 8)) {
      if (variant == 7 || variant == 8) {
        // forced (tests): two ranges per workgroup (7) or one (8), at least
        // two workgroups, as many as the blocks allow, even when some of
        // their ranges then hold no block
        kvs = ceil_div(num_cus, groups);
        if (kvs > plan->kv_blocks) kvs = plan->kv_blocks;
        if (kvs < 2) kvs = 2;
      } else if ((kvs = auto_kvs(groups, ks)) > 1) {
        int hp1, qt1;
        const int64_t g1 = shape(kPrefillWaves, &hp1, &qt1);
        const int64_t kvs1 = auto_kvs(g1, 1);
        if (kvs1 > 1 && g1 * kvs1 >= groups * kvs) {
          ks = 1;
          groups = g1;
          hp = hp1;
          qtiles = qt1;
          kvs = kvs1;
        }
      }
      // partial and combine indices are 32-bit rows
      if (kvs > 1 && (rows_all * kvs * (p.d_v > 2 ? p.d_v : 2) >= lim || groups * kvs >= lim)) kvs = 1;
    }
    plan->num_splits = ks;
    plan->kv_splits = (int32_t)kvs;
    plan->heads_per_group = hp;
    plan->qtiles_per_group = qtiles;
    plan->block_q = rows * qtiles;
    plan->q_tiles = (int32_t)ceil_div(p.q_len, plan->block_q);
    if (groups * kvs >= lim) {
      set_error("grid too large (%lld workgroups)", (long long)(groups * kvs));
      return SDPA_ERR_BAD_SHAPE;
    }
    plan->num_groups = (int32_t)(groups * kvs);
    // mainloop iterations per key range: the kernels cut the K blocks of a
    // workgroup's query rows into ks * kvs ranges of ceil(n_blocks / (ks *
    // kvs)) blocks each, ks per workgroup; a workgroup whose first range
    // starts past the last block runs none
    if (p.batch > 0 && p.q_len > 0 && groups > 0) {
      const int64_t per_tile = groups / plan->q_tiles;  // workgroups sharing one query tile (per split)
      int32_t mx = 0, mn = INT32_MAX;
      int64_t sum = 0;
      for (int qt = 0; qt < plan->q_tiles; ++qt) {
        const int row0 = qt * plan->block_q;
        const int row_end = row0 + plan->block_q < p.q_len ? row0 + plan->block_q : p.q_len;
        const KBlockRange r = kblock_range(row0, row_end, p.q_len, p.kv_len, plan->block_k, p.causal != 0);
        const int64_t cnt = ceil_div(r.n_blocks, ks * kvs);
        for (int64_t s = 0; s < kvs; ++s) {
          const int32_t it = s * ks * cnt < r.n_blocks ? (int32_t)cnt : 0;
          mx = it > mx ? it : mx;
          mn = it < mn ? it : mn;
          sum += (int64_t)it * ks * per_tile;
        }
      }
      plan->range_iters_max = mx;
      plan->range_iters_min = mn;
      plan->range_iters_sum = sum;
    }
    const int esz = p.in_dtype == SDPA_FP8_E4M3 ? 1 : 2;
    plan->lds_bytes = (uint64_t)ks * plan->stages * plan->block_k * (p.d_qk + p.d_v) * esz;
    plan->workspace_bytes = 0;
    if (kvs > 1) {
      const uint64_t po = (uint64_t)rows_all * kvs * p.d_v * 4;
      plan->workspace_bytes = ((po + 255) / 256) * 256 + (uint64_t)rows_all * kvs * 2 * 4;
      plan->combine_groups = (int32_t)ceil_div(rows_all, kCombineRows);
    }
    return SDPA_OK;
  }

  // ---- split-KV decode ----------------------------------------------------
  if (p.q_len != 1) {
    set_error("decode needs q_len == 1 (got %d)", p.q_len);
    return SDPA_ERR_BAD_SHAPE;
  }
  const int kid = decode_kernel_id(p);
  if (kid < 0) {
    set_error("unsupported decode (in_dtype=%d, out_dtype=%d, d_qk=%d, d_v=%d)", p.in_dtype, p.out_dtype, p.d_qk,
              p.d_v);
    return SDPA_ERR_UNSUPPORTED;
  }
  if (num_splits < 0 || num_splits > 4096) {
    set_error("num_splits must be in [0, 4096] (got %d)", num_splits);
    return SDPA_ERR_BAD_SHAPE;
  }
  plan->kernel = kid;
  plan->waves_per_group = kDecodeWaves;
  plan->rows_per_wave = kDecodeMaxGroup;
  plan->heads_per_group = (int32_t)G;
  plan->qtiles_per_group = 1;
  plan->block_q = 1;
  plan->block_k = kDecodeBlockK;
  plan->stages = 2;
  plan->q_tiles = 1;
  plan->kv_blocks = (int32_t)ceil_div(p.kv_len, kDecodeBlockK);
  // one wave per (batch, KV head, tile of up to 16 query heads, split)
  const int64_t gtiles = ceil_div(G, kDecodeMaxGroup);
  const int64_t pairs = (int64_t)p.batch * p.head_kv * gtiles;
  int64_t S;
  if (num_splits > 0) {
    S = num_splits;
    plan->blocks_per_split = (int32_t)(plan->kv_blocks > 0 ? ceil_div(plan->kv_blocks, S) : 1);
  } else {
    // One round of workgroups, as many as fit on a CU at once (LDS-bound: the
    // double-buffered K/V blocks of its 4 waves), keeps every CU streaming; a
    // second round would start only as the first drains.  No split is shorter
    // than two blocks, so the per-split overhead (Q load, partial write,
    // combine) stays a few percent of the K/V bytes.
    const int64_t lds = (int64_t)kDecodeWaves * 2 * kDecodeBlockK * (p.d_qk + p.d_v) * 2;
    int64_t per_cu = kLdsPerCu / lds;
    if (per_cu < 1) per_cu = 1;
    if (per_cu > 2) per_cu = 2;  // at most two waves per SIMD
    const int64_t target = (int64_t)num_cus * kDecodeWaves * per_cu;
    S = pairs > 0 ? ceil_div(target, pairs) : 1;
    const int64_t max_s = plan->kv_blocks / 2 > 0 ? plan->kv_blocks / 2 : 1;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    plan->blocks_per_split = (int32_t)(plan->kv_blocks > 0 ? ceil_div(plan->kv_blocks, S) : 1);
    S = plan->kv_blocks > 0 ? ceil_div(plan->kv_blocks, plan->blocks_per_split) : 1;
  }
  plan->num_splits = (int32_t)S;
  const int64_t waves = pairs * S;
  if (waves >= lim) {
    set_error("grid too large (%lld waves)", (long long)waves);
    return SDPA_ERR_BAD_SHAPE;
  }
  // one workgroup per (batch, split, 4 adjacent (KV head, query-head tile) tasks)
  plan->num_groups = (int32_t)(p.batch * S * ceil_div((int64_t)p.head_kv * gtiles, kDecodeWaves));
  plan->combine_groups = (int32_t)ceil_div((int64_t)p.batch * p.head_q, kCombineRows);
  plan->lds_bytes = (uint64_t)kDecodeWaves * 2 * kDecodeBlockK * (p.d_qk + p.d_v) * 2;
  const uint64_t po = (uint64_t)p.batch * p.head_q * S * p.d_v * 4;
  const uint64_t pml = (uint64_t)p.batch * p.head_q * S * 2 * 4;
  plan->workspace_bytes = ((po + 255) / 256) * 256 + pml;
  return SDPA_OK;
}

sdpa_status_t loop_counts(int q_len, int kv_len, int d_qk, int d_v, int block_q, int block_k, int block_d,
                          int block_v, bool causal, sdpa_loop_counts_t* out) {
  memset(out, 0, sizeof *out);
  if (q_len < 0 || kv_len < 0 || d_qk <= 0 || d_v <= 0 || block_q <= 0 || block_k <= 0 || block_d <= 0 ||
      block_v <= 0) {
    set_error("loop counts need non-negative lengths and positive dims / tiles");
    return SDPA_ERR_BAD_SHAPE;
  }
  out->q_blocks = ceil_div(q_len, block_q);
  out->k_blocks = ceil_div(kv_len, block_k);
  out->d_loops = ceil_div(d_qk, block_d);
  out->vv_loops = ceil_div(d_v, block_v);
  for (int64_t qb = 0; qb < out->q_blocks; ++qb) {
    const int row0 = (int)(qb * block_q);
    const int row_end = row0 + block_q < q_len ? row0 + block_q : q_len;
    const KBlockRange r = kblock_range(row0, row_end, q_len, kv_len, block_k, causal);
    out->blocks_visited += r.n_blocks;
    out->blocks_masked += r.n_blocks - r.n_full;
  }
  out->qk_tiles = out->blocks_visited * out->d_loops;
  out->pv_tiles = out->blocks_visited * out->vv_loops;
  out->softmax_tiles = out->blocks_visited;
  return SDPA_OK;
}

}  // namespace sdpa
