// prefill_cached.hip -- cached-KV (chunked) prefill instantiations of the
// one-wave and the two-waves-per-SIMD prefill kernels (prefill_kernel.h and
// prefill_o2_kernel.h with CACHED = true): the chunk's
// queries over a cached prefix followed by the chunk's own keys, the mode
// "Xe SDPA Forward Mainloop" runs with kblocks_cache > 0 (sections "Startup
// prefetch + init" and "Outer K-block loop").  Compiled apart from
// prefill.hip only so that the two sets of instantiations build in parallel.
#include "prefill_kernel.h"
#include "prefill_o2_kernel.h"

namespace sdpa {

template <class T, int D, int KS, bool ALIGN>
static void launch_cached_form(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * kPrefillWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_kernel<T, D, D, true, KS, true, ALIGN>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, D, false, KS, true, ALIGN>), grid, block, 0, (hipStream_t)stream, a);
}

// One fill instruction covers 1 KiB, i.e. 512 / D key rows; when the cache
// length and the key count are multiples of that, no instruction straddles
// the cache and the new keys, and the fills take a scalar base.
template <class T, int D, int KS>
static int launch_cached_ks(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  constexpr int RSTEP = 512 / D;
  if (a.cache_len % RSTEP == 0 && a.kv_len % RSTEP == 0)
    launch_cached_form<T, D, KS, true>(a, causal, stream);
  else
    launch_cached_form<T, D, KS, false>(a, causal, stream);
  return (int)hipGetLastError();
}

template <class T, int D>
static int launch_cached_one(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  return plan.num_splits == 2 ? launch_cached_ks<T, D, 2>(a, causal, stream)
                              : launch_cached_ks<T, D, 1>(a, causal, stream);
}

template <class T, int D, int NW, int KS, int BK>
static int launch_cached_o2(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * NW);
  if (causal)
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, true, NW, KS, BK, true>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_o2_kernel<T, D, D, false, NW, KS, BK, true>), grid, block, 0, (hipStream_t)stream,
                       a);
  return (int)hipGetLastError();
}

int launch_prefill_cached(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  switch (plan.kernel) {
    case kOccF16D64: return launch_cached_o2<F16, 64, 4, 1, 64>(a, causal, stream);
    case kOccBf16D64: return launch_cached_o2<Bf16, 64, 4, 1, 64>(a, causal, stream);
    case kOccF16D128: return launch_cached_o2<F16, 128, 4, 1, 64>(a, causal, stream);
    case kOccBf16D128: return launch_cached_o2<Bf16, 128, 4, 1, 64>(a, causal, stream);
    case kSplitF16D64: return launch_cached_o2<F16, 64, 8, 4, 32>(a, causal, stream);
    case kSplitBf16D64: return launch_cached_o2<Bf16, 64, 8, 4, 32>(a, causal, stream);
    case kSplitF16D128: return launch_cached_o2<F16, 128, 8, 4, 32>(a, causal, stream);
    case kSplitBf16D128: return launch_cached_o2<Bf16, 128, 8, 4, 32>(a, causal, stream);
    case kPrefillF16D64: return launch_cached_one<F16, 64>(a, plan, causal, stream);
    case kPrefillBf16D64: return launch_cached_one<Bf16, 64>(a, plan, causal, stream);
    case kPrefillF16D128: return launch_cached_one<F16, 128>(a, plan, causal, stream);
    case kPrefillBf16D128: return launch_cached_one<Bf16, 128>(a, plan, causal, stream);
    default: return (int)hipErrorInvalidValue;  // no wide or fp8 form reads a cache
  }
}

}  // namespace sdpa
