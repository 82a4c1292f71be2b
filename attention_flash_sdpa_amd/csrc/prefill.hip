// prefill.hip -- fused SDPA forward mainloop for gfx950 (16-bit inputs).
//
// Structure follows "Xe SDPA Forward Mainloop -- Key Loops + Shapes"
// (sections "Startup prefetch + init", "mainloop_body(K)", "softmax()
// helper", "Outer K-block loop"): a resident Q tile, K/V blocks streamed
// through a prefetch pipeline, S = Q K^T on the matrix cores, mask, online
// softmax with exp2 and a log2(e)-folded scale, and P V accumulated in fp32.
// The MI355X mapping:
//
//  * One workgroup = 4 wavefronts that all read the same K/V blocks: either
//    up to 4 query heads of one GQA group on the same 32 query rows, or
//    consecutive 32-row tiles of one head (the planner picks).
//  * Each wave computes S^T = K Q^T (the operand order the page's source
//    comment "S = K * Q" uses), so lane l and lane l^32 together hold all the
//    scores of query row l%32.  Row max / row sum are in-lane reductions plus
//    one permlane32 swap; the running max, sum and rescale factor stay in
//    registers of that lane.
//  * The probabilities are packed to 16 bits in place and used directly as the
//    B operand of O^T = V^T P^T, so P never leaves registers; O^T stays in
//    the MFMA accumulators and its rescale by 2^(m_old - m_new) is lane-local.
//  * Software pipeline: iteration j issues the QK MFMAs of block j+1 before
//    the softmax of block j, so the exp/VALU work of one block overlaps the
//    matrix-core work of the next, then runs the PV MFMAs of block j.  K and V
//    therefore have separate double buffers: K(j+2) and V(j+1) are loaded
//    during iteration j, each with a whole iteration to arrive.
//  * K/V blocks of 64 keys go global -> LDS with direct 16-byte-per-lane loads
//    (no register staging, scalar base address + per-lane offset) into rows
//    whose 16-byte slots are swizzled (swz_prefill) so that K fragment reads
//    (ds_read_b128) and transposed V fragment reads (ds_read_b64_tr_b16) are
//    free of bank conflicts.  Buffer parity is a compile-time parameter, so
//    every LDS read uses an immediate offset.
//  * The K loop is split on the block counts into a branch-free unmasked part
//    and a peeled masked tail ("xe2-sdp-kernels", section "Inner-loop
//    rules"): only the tail blocks evaluate the causal/remainder predicate.
#include "prefill_kernel.h"

namespace sdpa {

template <class T, int D, int KS>
static int launch_ks(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * kPrefillWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_kernel<T, D, D, true, KS, false>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, D, false, KS, false>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <class T, int D>
static int launch_one(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  return plan.num_splits == 2 ? launch_ks<T, D, 2>(a, causal, stream) : launch_ks<T, D, 1>(a, causal, stream);
}

int launch_prefill(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  // keys split across workgroups (dense or cached): prefill_split.hip
  if (plan.kv_splits > 1) return launch_prefill_split(a, plan, causal, stream);
  if (a.k_cache != nullptr) return launch_prefill_cached(a, plan, causal, stream);
  switch (plan.kernel) {
    case kPrefillF16D64: return launch_one<F16, 64>(a, plan, causal, stream);
    case kPrefillBf16D64: return launch_one<Bf16, 64>(a, plan, causal, stream);
    case kPrefillF16D128: return launch_one<F16, 128>(a, plan, causal, stream);
    case kPrefillBf16D128: return launch_one<Bf16, 128>(a, plan, causal, stream);
    case kPrefillFp8D192: return launch_prefill_fp8(a, causal, stream);
    case kOccF16D64:
    case kOccBf16D64:
    case kOccF16D128:
    case kOccBf16D128:
    case kSplitF16D64:
    case kSplitBf16D64:
    case kSplitF16D128:
    case kSplitBf16D128: return launch_prefill_o2(a, plan, causal, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace sdpa
