// prefill_o2.hip -- the 32-row prefill mainloop in its two-waves-per-SIMD
// form (at most 256 registers per wave, so two waves share each SIMD and hide
// each other's LDS, memory and barrier latencies).
//
// Same method and data layout as prefill.hip ("Xe SDPA Forward Mainloop --
// Key Loops + Shapes", sections "mainloop_body(K)", "softmax() helper" and
// "Outer K-block loop"): S^T = K Q^T on the matrix cores, the blocked online
// softmax with exp2 and the scale folded with log2(e), O^T += V^T P^T with P
// kept in registers, K/V blocks streamed into double-buffered, swizzled LDS
// by direct 16-byte loads, a branch-free unmasked loop and a peeled masked
// tail.  Two shapes are instantiated:
//
//  * NW = 4 waves, one key range, 64-key blocks: for grids with more
//    workgroups than CUs, where two workgroups share a CU;
//  * NW = 8 waves, KS = 4 key ranges, 32-key blocks: for small grids.  Two
//    query heads (or tiles) share each range's K/V stream, the four ranges
//    of the workgroup's key span run side by side and are merged through LDS
//    at the end with the split-softmax algebra of the two-phase decode
//    ("xe2-sdp-kernels", section "Assets", two-phase decode), which gives
//    every SIMD two waves where the one-range grid would give it one.
//
// The masked prefill runs the first shape with the full additive mask of
// the mainloop's optional mask argument ("Xe SDPA Forward Mainloop",
// section "Runtime args / params"), added to every score in the mask step
// (section "Compact shape table", row "Mask"): each lane loads the bias of
// its own scores (its query row, 4 keys per 8-byte load) straight into
// registers one block ahead, and the softmax forms scale*S + bias before the
// row max; causal and ragged limits apply on top in the masked blocks.
//
// Software pipeline: iteration j issues the QK MFMAs of block j+1 before the
// softmax of block j is finished, then runs the PV MFMAs of block j; K(j+2)
// and V(j+1) are loaded during iteration j.  Buffer parity is a compile-time
// parameter (the loop is unrolled by two), so every LDS read uses an
// immediate offset.
#include "prefill_o2_kernel.h"

namespace sdpa {

template <class T, int D, int NW, int KS, int BK>
static int launch_o2_t(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * NW);
  if (causal)
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, true, NW, KS, BK, false>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, false, NW, KS, BK, false>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_prefill_o2(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  switch (plan.kernel) {
    case kOccF16D64: return launch_o2_t<F16, 64, 4, 1, 64>(a, causal, stream);
    case kOccBf16D64: return launch_o2_t<Bf16, 64, 4, 1, 64>(a, causal, stream);
    case kOccF16D128: return launch_o2_t<F16, 128, 4, 1, 64>(a, causal, stream);
    case kOccBf16D128: return launch_o2_t<Bf16, 128, 4, 1, 64>(a, causal, stream);
    case kSplitF16D64: return launch_o2_t<F16, 64, 8, 4, 32>(a, causal, stream);
    case kSplitBf16D64: return launch_o2_t<Bf16, 64, 8, 4, 32>(a, causal, stream);
    case kSplitF16D128: return launch_o2_t<F16, 128, 8, 4, 32>(a, causal, stream);
    case kSplitBf16D128: return launch_o2_t<Bf16, 128, 8, 4, 32>(a, causal, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

template <class T, int D>
static int launch_o2_bias_t(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * 4);
  if (causal)
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, true, 4, 1, 64, false, true>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, false, 4, 1, 64, false, true>), grid, block, 0, (hipStream_t)stream,
                       a);
  return (int)hipGetLastError();
}

// The masked prefill: the one-range, four-wave shape with the additive bias.
int launch_prefill_o2_bias(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  switch (plan.kernel) {
    case kOccF16D64: return launch_o2_bias_t<F16, 64>(a, causal, stream);
    case kOccBf16D64: return launch_o2_bias_t<Bf16, 64>(a, causal, stream);
    case kOccF16D128: return launch_o2_bias_t<F16, 128>(a, causal, stream);
    case kOccBf16D128: return launch_o2_bias_t<Bf16, 128>(a, causal, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace sdpa
