// prefill_split.hip -- the KVSPLIT instantiations of the one-wave prefill
// kernel (prefill_kernel.h): a query tile's K blocks spread over kv_splits
// workgroups, each writing unnormalized fp32 partials and their (max, sum)
// to the caller's workspace, for dense keys and for a cached prefix + new
// keys.  The K-block subrange per work item is the causal tail's
// blk_k0..blk_k1 of "Xe SDPA Forward Mainloop" (section "Outer K-block
// loop"); the partials are merged by the split-KV decode's second phase
// (decode_combine_kernel, launched by the caller).  Compiled apart from
// prefill.hip and prefill_cached.hip so that the three sets of
// instantiations build in parallel.
#include "prefill_kernel.h"

namespace sdpa {

template <class T, int D, int KS, bool CACHED, bool ALIGN>
static int launch_split_form(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * kPrefillWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_kernel<T, D, D, true, KS, CACHED, ALIGN, true>), grid, block, 0, (hipStream_t)stream,
                       a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, D, false, KS, CACHED, ALIGN, true>), grid, block, 0,
                       (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <class T, int D, int KS>
static int launch_split_ks(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  if (a.k_cache == nullptr) return launch_split_form<T, D, KS, false, false>(a, causal, stream);
  // the scalar-base fills of the cached form, as in prefill_cached.hip
  constexpr int RSTEP = 512 / D;
  if (a.cache_len % RSTEP == 0 && a.kv_len % RSTEP == 0)
    return launch_split_form<T, D, KS, true, true>(a, causal, stream);
  return launch_split_form<T, D, KS, true, false>(a, causal, stream);
}

template <class T, int D>
static int launch_split_one(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  return plan.num_splits == 2 ? launch_split_ks<T, D, 2>(a, causal, stream)
                              : launch_split_ks<T, D, 1>(a, causal, stream);
}

int launch_prefill_split(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  if (plan.num_splits != 1 && plan.num_splits != 2) return (int)hipErrorInvalidValue;
  switch (plan.kernel) {  // the planner splits the one-wave 16-bit forms only
    case kPrefillF16D64: return launch_split_one<F16, 64>(a, plan, causal, stream);
    case kPrefillBf16D64: return launch_split_one<Bf16, 64>(a, plan, causal, stream);
    case kPrefillF16D128: return launch_split_one<F16, 128>(a, plan, causal, stream);
    case kPrefillBf16D128: return launch_split_one<Bf16, 128>(a, plan, causal, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace sdpa
