/*
 * sdpa.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product-attention
 * forward library: a causal/full prefill mainloop (also over a cached prefix,
 * and with a full additive mask), a two-phase split-KV decode (also over
 * variable-length and paged caches) and a boolean-to-additive mask
 * conversion.  The attention calls compute
 *
 *     O = softmax(Q K^T * scale + mask) V
 *
 * with an online (blocked) softmax in fp32, as described on the page
 * "Xe SDPA Forward Mainloop -- Key Loops + Shapes" (sections "mainloop_body(K)",
 * "softmax() helper", "Full simplified pseudocode"), and the two-phase decode
 * named on the page "xe2-sdp-kernels" (section "Assets").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major, batch outermost (the GQA layouts of
 *    "xe2-sdp-kernels", section "GQA layout", with a leading batch):
 *        Q [batch, q_len, head_q, d_qk]
 *        K [batch, kv_len, head_kv, d_qk]
 *        V [batch, kv_len, head_kv, d_v]
 *        O [batch, q_len, head_q, d_v]
 *        lse (optional) [batch, head_q, q_len] fp32, natural-log sum-exp of the
 *        scaled visible scores; -inf for a row with no visible key.
 *    For decode q_len is 1, so Q is [batch, head_q, d_qk] and O is
 *    [batch, head_q, d_v].
 *  - GQA: query head h reads KV head h / (head_q / head_kv).
 *  - Causal (causal != 0) is aligned bottom-right: key j is visible to query i
 *    iff j <= i + kv_len - q_len.  A row with no visible key (q_len > kv_len,
 *    or kv_len == 0) yields O = 0 and lse = -inf, never NaN.
 *  - Data pointers are device addresses, 16-byte aligned, owned by the caller
 *    and left untouched except O, lse and the workspace.  The library never
 *    allocates, frees or synchronises: work is enqueued on `stream` (a
 *    hipStream_t passed as void*, NULL = the null stream) and results are
 *    ready when the stream reaches that point.
 *  - All validation happens before any launch; on an error nothing is
 *    enqueued.  Calls are stateless and thread-safe; sdpa_last_error() keeps
 *    a per-thread text for the last failing call.
 *  - Supported (in_dtype, d_qk, d_v): fp16/bf16 with d_qk == d_v in {64, 128};
 *    fp8 e4m3 (OCP "fn" variant, largest finite 448) with (192, 128).
 *    out_dtype is fp16 or bf16.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_ABI_VERSION 3

typedef enum {
  SDPA_F16 = 0,
  SDPA_BF16 = 1,
  SDPA_FP8_E4M3 = 2
} sdpa_dtype_t;

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                     */
  SDPA_ERR_BAD_SHAPE = 2,   /* negative size, head_q % head_kv != 0, decode
                               with q_len != 1, sizes overflowing 32-bit
                               element offsets per batch entry, ...          */
  SDPA_ERR_BAD_SCALE = 3,   /* scale or a descale not finite, or negative, or
                               a descale != 1 with fp16/bf16 inputs          */
  SDPA_ERR_UNSUPPORTED = 4, /* (dtype, d_qk, d_v) outside the supported set   */
  SDPA_ERR_MISALIGNED = 5,  /* a data pointer not 16-byte aligned             */
  SDPA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required        */
  SDPA_ERR_HIP = 7          /* the HIP runtime reported an error              */
} sdpa_status_t;

/* One attention problem.  scale multiplies Q K^T (callers usually pass
 * 1/sqrt(d_qk)); it is folded with log2(e) so that every exponential is a
 * base-2 exponential ("Xe SDPA Forward Mainloop", section "Arguments /
 * params").  q/k/v_descale are the per-tensor dequantisation factors of fp8
 * inputs (x = x_q * descale), host floats known when the inputs were
 * quantised; any value other than 1 with fp16/bf16 inputs is rejected with
 * SDPA_ERR_BAD_SCALE by every entry point. */
typedef struct sdpa_problem {
  int32_t batch;
  int32_t q_len;
  int32_t kv_len;
  int32_t head_q;
  int32_t head_kv;
  int32_t d_qk;
  int32_t d_v;
  int32_t in_dtype;  /* sdpa_dtype_t of Q, K and V */
  int32_t out_dtype; /* sdpa_dtype_t of O: SDPA_F16 or SDPA_BF16 */
  int32_t causal;    /* 0 = full, otherwise bottom-right causal */
  float scale;       /* finite, >= 0 */
  float q_descale;
  float k_descale;
  float v_descale;
} sdpa_problem_t;

/* Launch plan chosen by the host planner (pure host code, no GPU needed).
 * Every wave owns rows_per_wave query rows of one head; a workgroup holds
 * heads_per_group query heads of one KV group times qtiles_per_group
 * consecutive query tiles, so all its waves read the same K/V blocks. */
typedef struct sdpa_plan {
  int32_t kernel;           /* internal instantiation id                       */
  int32_t waves_per_group;  /* waves in one workgroup                           */
  int32_t rows_per_wave;    /* query rows per wave (MFMA N dimension)           */
  int32_t heads_per_group;  /* query heads sharing one workgroup                */
  int32_t qtiles_per_group; /* wave-sized query tiles per head per workgroup    */
  int32_t block_q;          /* query rows per head per workgroup                */
  int32_t block_k;          /* keys per K/V block (one mainloop iteration)      */
  int32_t stages;           /* K/V blocks resident in LDS (prefetch depth + 1)  */
  int32_t q_tiles;          /* workgroup-sized query tiles per head             */
  int32_t kv_blocks;        /* ceil(kv_len / block_k)                           */
  int32_t num_groups;       /* workgroups of the main kernel                    */
  int32_t num_splits;       /* decode: key-range splits per (batch, KV head);
                               prefill: key ranges per workgroup (1, 2 or 4), each
                               streamed by its own waves, merged at the end    */
  int32_t blocks_per_split; /* decode: K/V blocks per split                     */
  int32_t combine_groups;   /* decode, and prefill with kv_splits > 1:
                               workgroups of the combine kernel                */
  uint64_t lds_bytes;       /* LDS per workgroup of the main kernel             */
  uint64_t workspace_bytes; /* device workspace the call needs (prefill: for
                               the kv_splits > 1 plan; smaller runs unsplit)   */
  /* Prefill load balance (0 for decode).  Every key range of a workgroup runs
   * ceil(K blocks of its query rows / num_splits) mainloop iterations (the
   * causal K-block range of "Xe SDPA Forward Mainloop", section "Outer
   * K-block loop", cut into num_splits equal parts); with one workgroup per
   * CU the busiest range sets the launch time.  max / (sum / (num_groups *
   * num_splits)) is the imbalance factor (1 = even). */
  int64_t range_iters_sum;  /* iterations summed over all ranges of all groups  */
  int32_t range_iters_max;  /* iterations of the busiest range                  */
  int32_t range_iters_min;  /* iterations of the lightest range                 */
  /* Prefill: workgroups sharing one query tile's K blocks (1 = none).  With
   * kv_splits > 1 each of them takes num_splits of the tile's kv_splits *
   * num_splits equal key ranges ("Xe SDPA Forward Mainloop", section "Outer
   * K-block loop": a K-block subrange per work item), writes unnormalized
   * fp32 partial outputs with their running (max, sum) to the workspace, and
   * a second kernel merges the partials of every query row (combine_groups
   * workgroups), as the split-KV decode does.  num_groups counts all
   * workgroups, splits included. */
  int32_t kv_splits;
} sdpa_plan_t;

/* Tile-level loop counts of one attention head for a given tiling, in the
 * units the page "Xe SDPA Forward Mainloop -- Key Loops + Shapes" uses in its
 * section "Loop counts for seq_q=512, seq_k=512, head_dim=128": query blocks
 * of block_q rows, K blocks of block_k keys, QK MMA steps of block_d head-dim
 * columns and PV MMA steps of block_v value columns per K block.  For causal
 * problems only the K blocks a query block can see are visited (the planner's
 * and the kernels' shared loop bound). */
typedef struct sdpa_loop_counts {
  int64_t q_blocks;         /* ceil(q_len / block_q)                          */
  int64_t k_blocks;         /* ceil(kv_len / block_k)                         */
  int64_t d_loops;          /* ceil(d_qk / block_d) QK steps per K block      */
  int64_t vv_loops;         /* ceil(d_v / block_v) PV steps per K block       */
  int64_t blocks_visited;   /* K blocks visited, summed over query blocks     */
  int64_t blocks_masked;    /* of those, blocks that need the mask (peeled)   */
  int64_t qk_tiles;         /* blocks_visited * d_loops                       */
  int64_t pv_tiles;         /* blocks_visited * vv_loops                      */
  int64_t softmax_tiles;    /* blocks_visited ([block_q, block_k] tiles)      */
} sdpa_loop_counts_t;

/* Fills *out for one head (all sizes > 0 except q_len/kv_len >= 0).
 * Host-only. */
sdpa_status_t sdpa_loop_counts(int q_len, int kv_len, int d_qk, int d_v, int block_q, int block_k,
                               int block_d, int block_v, int causal, sdpa_loop_counts_t* out);

/* ABI version of the loaded library (SDPA_ABI_VERSION it was built with). */
int sdpa_abi_version(void);

/* Static text for a status code. */
const char* sdpa_status_string(int status);

/* Detail text of the last failing call on the calling thread ("" if none). */
const char* sdpa_last_error(void);

/* Forces one form of the 16-bit prefill kernels for every later call of this
 * process, for tuning sweeps and tests (the forms compute the same result):
 *   "narrow1" / "narrow2" : one wave per SIMD, one / two key ranges per
 *                           workgroup merged at the end;
 *   "occ2"                : two waves per SIMD, one key range;
 *   "split4"              : two waves per SIMD, four key ranges of 32-key blocks;
 *   "kvsplit"             : "narrow2" with the key range also split across
 *                           at least two workgroups (plan.kv_splits), even on
 *                           shapes where some ranges hold no key (sdpa_prefill_fwd
 *                           with a workspace only; other entry points run
 *                           "narrow2");
 *   "kvsplit1"            : the same with one key range per workgroup
 *                           ("narrow1" split across workgroups);
 *   "" / "auto" / NULL    : the planner's choice (the default).
 * The environment variable SDPA_PREFILL_VARIANT gives the initial value (read
 * once).  Unknown names return SDPA_ERR_UNSUPPORTED and change nothing.
 * Host-only; process-wide; do not change it while another thread plans or
 * launches a prefill. */
sdpa_status_t sdpa_set_prefill_variant(const char* name);

/* Validates a problem and fills the plan the entry points would use.
 * is_decode selects the split-KV decode path (q_len must be 1).  num_cus is
 * the compute-unit count to plan for (<= 0: 256, the MI355X count).
 * num_splits (decode only) forces a split count, 0 lets the planner choose.
 * Host-only: touches no GPU. */
sdpa_status_t sdpa_plan(const sdpa_problem_t* problem, int is_decode, int num_cus,
                        int num_splits, sdpa_plan_t* plan);

/* Device workspace bytes sdpa_prefill_fwd needs for the planned split of the
 * key range across workgroups (plan.kv_splits > 1): fp32 partial outputs
 * [batch, q_len, head_q, kv_splits, d_v] (rounded up to 256 bytes) followed
 * by partial (max, sum) pairs [batch, q_len, head_q, kv_splits, 2].  0 when
 * the plan does not split (most shapes: the split is planned only when the
 * problem has too few query tiles to occupy half the GPU) and for an invalid
 * problem. */
size_t sdpa_prefill_workspace_bytes(const sdpa_problem_t* problem);

/* Device workspace bytes sdpa_decode_fwd needs for num_splits (0 = the
 * planner's choice): fp32 partial outputs [batch, head_q, splits, d_v] and
 * partial (max, sum) pairs [batch, head_q, splits, 2].  Returns 0 for an
 * invalid problem. */
size_t sdpa_decode_workspace_bytes(const sdpa_problem_t* problem, int num_splits);

/* Prefill / general forward: one fused kernel.  Streams K/V blocks past each
 * resident Q tile ("Xe SDPA Forward Mainloop", sections "Outer K-block loop"
 * and "mainloop_body(K)"): S = Q K^T (MFMA, fp32 accumulate), mask on the
 * boundary blocks only, online softmax with exp2, P V (MFMA) into an fp32
 * accumulator, then O = acc / rowsum in the epilogue.
 *   q, k, v : device inputs in the layouts above, dtype problem->in_dtype
 *   o       : device output, dtype problem->out_dtype
 *   lse     : device fp32 [batch, head_q, q_len] or NULL
 *   workspace, workspace_bytes: caller-owned device scratch, 16-byte
 *             aligned, of sdpa_prefill_workspace_bytes() bytes, which the
 *             call overwrites (stream-ordered: calls that share one workspace
 *             must be ordered on one stream).  NULL / a smaller size runs the
 *             same problem without the cross-workgroup split (the result
 *             agrees to rounding; it may take longer); a workspace is never
 *             required.
 *   stream  : hipStream_t or NULL
 * batch == 0 or q_len == 0 is a successful no-op. */
sdpa_status_t sdpa_prefill_fwd(const sdpa_problem_t* problem, const void* q, const void* k,
                               const void* v, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Cached-KV (chunked) prefill: the chunk's q_len queries attend to a cached
 * prefix of cache_len keys followed by the chunk's own kv_len keys.  The
 * mainloop page ("Xe SDPA Forward Mainloop") takes its first
 * ceil(cache_len / block) K blocks from the cache and the rest from the new
 * tensors, indexed from the first new key (sections "Startup prefetch +
 * init", "Outer K-block loop" and the K prefetch of "mainloop_body(K)"),
 * and masks causally only the blocks that are not cache blocks (section
 * "mask branches").  So with causal != 0 every query sees every cached key
 * and query i sees new key j iff j <= i + kv_len - q_len; this needs
 * q_len <= kv_len (else SDPA_ERR_BAD_SHAPE).  The result equals
 * sdpa_prefill_fwd over the concatenated keys [cache | new].
 *   problem  : kv_len = the chunk's new keys; other fields as for prefill
 *   q        : [batch, q_len, head_q, d_qk]
 *   k_cache, v_cache : [batch, cache_cap, head_kv, d_qk|d_v], of which keys
 *              0 .. cache_len-1 are read (0 <= cache_len <= cache_cap); may
 *              be NULL when cache_len == 0 (then this is sdpa_prefill_fwd)
 *   k, v     : [batch, kv_len, head_kv, d_qk|d_v] (the chunk's own keys)
 *   o, lse   : as for sdpa_prefill_fwd
 *   workspace, workspace_bytes: as for sdpa_prefill_fwd, sized by
 *             sdpa_prefill_cached_workspace_bytes(problem, cache_len): a
 *             short chunk over a long cache spreads its keys over several
 *             workgroups; NULL / smaller runs it unsplit
 * 16-bit inputs only (fp16/bf16, d 64 or 128; fp8 gives
 * SDPA_ERR_UNSUPPORTED).  Errors as for sdpa_prefill_fwd. */
sdpa_status_t sdpa_prefill_cached_fwd(const sdpa_problem_t* problem, const void* q,
                                      const void* k_cache, const void* v_cache, int32_t cache_len,
                                      int32_t cache_cap, const void* k, const void* v, void* o,
                                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace bytes sdpa_prefill_cached_fwd uses for a chunk over
 * cache_len cached keys: the layout of sdpa_prefill_workspace_bytes for the
 * cache_len + kv_len keys of the whole sequence; 0 when the plan does not
 * split and for an invalid problem. */
size_t sdpa_prefill_cached_workspace_bytes(const sdpa_problem_t* problem, int32_t cache_len);

/* Boolean -> additive mask conversion, the memory-bound mask_convert kernel
 * of "xe2-sdp-kernels" (section "Performance testing"), producing the full
 * additive mask the mainloop's optional mask argument applies to the scores
 * ("Xe SDPA Forward Mainloop", section "Runtime args / params").  Element e
 * of out (out_dtype SDPA_F16 or SDPA_BF16) is +0 where mask[e] != 0 (the key
 * takes part) and -inf where mask[e] == 0; any layout, element for element.
 *   mask : device uint8 [n] (torch.bool storage qualifies), 16-byte aligned
 *   out  : device 16-bit [n], 16-byte aligned, written entirely
 * n == 0 is a no-op.  Enqueued on `stream`; nothing synchronises. */
sdpa_status_t sdpa_mask_convert(const uint8_t* mask, void* out, int64_t n, int32_t out_dtype,
                                void* stream);

/* Measurement helper, not part of the attention computation: the HBM
 * streaming-read rate that bounds the split-KV decode.  Loads every byte of
 * data once (16-byte non-temporal loads, a fixed grid of 2048 workgroups of
 * 256 threads) and folds it by XOR; a workgroup writes its fold to
 * sink[workgroup] only in the unlikely case that it equals 0x9e3779b9, so
 * timed over a buffer its traffic is the read of `bytes`.
 *   data  : device, 16-byte aligned, `bytes` readable bytes
 *   bytes : a multiple of 16 (0: no-op)
 *   sink  : device uint32 [2048], may be written
 * Enqueued on `stream`; nothing synchronises. */
sdpa_status_t sdpa_hbm_read_probe(const void* data, int64_t bytes, uint32_t* sink, void* stream);

/* Prefill with a full additive mask: O = softmax(Q K^T * scale + mask) V,
 * the mainloop's optional full mask ("Xe SDPA Forward Mainloop", section
 * "Runtime args / params") added to every score in its mask step (section
 * "Compact shape table", row "Mask"); with causal != 0 the bottom-right
 * causal rule applies as well.  A row whose scores are all -inf gets O = 0
 * and lse = -inf.
 *   q, k, v, o, lse : as for sdpa_prefill_fwd; fp16 or bf16 inputs with the
 *       same output type and d_qk == d_v in {64, 128}
 *   mask : device, the inputs' 16-bit type, 16-byte aligned; the value for
 *       (batch b, query head h, row i, key j) is at element
 *       b*mask_stride_b + h*mask_stride_h + i*mask_stride_row + j.  A stride
 *       of 0 broadcasts over batch or heads.  All strides are multiples of 8
 *       elements and mask_stride_row >= max(kv_len, 8): rows may be padded,
 *       and the padding is read but never used.  With kv_len == 0 the mask
 *       is not read (its pointer and strides are not checked); O = 0 and
 *       lse = -inf.
 * No workspace; errors as for sdpa_prefill_fwd. */
sdpa_status_t sdpa_prefill_masked_fwd(const sdpa_problem_t* problem, const void* q, const void* k,
                                      const void* v, const void* mask, int64_t mask_stride_b,
                                      int64_t mask_stride_h, int32_t mask_stride_row, void* o,
                                      float* lse, void* stream);

/* Two-phase split-KV decode ("xe2-sdp-kernels", section "Assets": production
 * decode, two-phase) for one new token per sequence (q_len == 1).
 * Phase 1: one workgroup per (batch, KV head, split) streams its key range
 * once for all head_q/head_kv query heads of the group and writes unnormalised
 * partial outputs with their running max and sum into the workspace.
 * Phase 2: one wavefront per (batch, query head), four per workgroup,
 * rescales and merges the splits (the same rescale the online softmax applies
 * between K blocks) and writes O (and lse).  Both kernels run on `stream`;
 * nothing synchronises.
 *   q : [batch, head_q, d_qk]; k, v : [batch, kv_len, head_kv, d_qk|d_v]
 *   o : [batch, head_q, d_v]; lse : [batch, head_q] fp32 or NULL
 *   num_splits : 0 = planner's choice, otherwise the split count to use
 *   workspace  : >= sdpa_decode_workspace_bytes(problem, num_splits) bytes,
 *                16-byte aligned; its contents on entry are ignored. */
sdpa_status_t sdpa_decode_fwd(const sdpa_problem_t* problem, const void* q, const void* k,
                              const void* v, void* o, float* lse, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/* sdpa_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a static device
 * array of 64 MiB held by the library on each GPU it runs on until the
 * process ends; its address is looked up on the first call per device.  The
 * call itself allocates and frees nothing.
 *   arguments as for sdpa_decode_fwd, less workspace / workspace_bytes.
 * A problem whose partials (sdpa_decode_workspace_bytes) exceed 64 MiB
 * returns SDPA_ERR_WORKSPACE before any launch.  Every call on one GPU uses
 * the same array, which keeps the last call's contents (nothing in it needs
 * clearing: each call writes every partial it reads): calls that overlap on
 * one GPU (two streams, or two threads) race and must be serialised by the
 * caller, e.g. on one stream. */
sdpa_status_t sdpa_decode_fwd_noalloc(const sdpa_problem_t* problem, const void* q, const void* k,
                                      const void* v, void* o, float* lse, int num_splits,
                                      void* stream);

/* Decode over variable-length and/or paged key/value caches.  The mainloop
 * page ("Xe SDPA Forward Mainloop", section "Runtime args / params") lists
 * an optional page table, page size and per-sequence page counts among its
 * runtime arguments, section "Helpers" a logical-to-physical K tile lookup,
 * and section "Launcher -> kernel" a variable-length mode; the pages fix no
 * layout, so this one is taken:
 *   page_table == NULL : k_cache, v_cache are dense [batch, kv_len, head_kv,
 *       d_qk|d_v] as for sdpa_decode_fwd (num_pages, page_size,
 *       pages_per_seq ignored).
 *   page_table != NULL : k_cache, v_cache are pools [num_pages, page_size,
 *       head_kv, d_qk|d_v]; page_table is device int32 [batch, pages_per_seq]
 *       and keys p*page_size .. (p+1)*page_size - 1 of sequence b sit in
 *       physical page page_table[b * pages_per_seq + p].  page_size must be 8,
 *       16 or a positive multiple of 32, pages_per_seq * page_size >= kv_len.
 *   seq_lens : device int32 [batch], sequence b attends to its first
 *       seq_lens[b] keys (clamped to [0, kv_len]; 0 gives O = 0 and
 *       lse = -inf), or NULL for kv_len keys each.
 * problem->kv_len is the longest sequence the call allows; split count and
 * workspace follow it exactly as for sdpa_decode_fwd (the same
 * sdpa_decode_workspace_bytes).  Only the table entries of pages holding a
 * sequence's first seq_lens[b] keys are read.  The table lives on the device
 * and is not checked on the host: an entry outside [0, num_pages) is never
 * dereferenced (page 0 is read in its place) and turns that sequence's O and
 * lse rows (all heads) into NaN.  Pointers 4-byte (tables) or 16-byte (data,
 * workspace) aligned; other arguments and errors as for sdpa_decode_fwd. */
sdpa_status_t sdpa_decode_paged_fwd(const sdpa_problem_t* problem, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t num_pages, int32_t page_size, int32_t pages_per_seq,
                                    void* o, float* lse, int num_splits, void* workspace,
                                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
