// sdpa_bounds.h -- the K-block range of one query block, shared by the host
// planner (loop counts, tests) and the kernels (their loop bounds), so both
// use one definition.
//
// Bottom-right causal visibility: key j is visible to query i iff
// j <= i + kv_len - q_len.  For query rows [row0, row_end) the blocks of
// block_k keys split into [0, n_full) -- every key visible to every row, no
// mask needed -- and [n_full, n_blocks) -- the peeled tail that needs the
// causal and/or remainder mask ("xe2-sdp-kernels", section "Inner-loop rules":
// separate the last iterations from the main loop instead of branching).
#pragma once

#ifdef __HIP__
#include <hip/hip_runtime.h>
#define SDPA_HD __host__ __device__ __forceinline__
#else
#define SDPA_HD inline
#endif

namespace sdpa {

struct KBlockRange {
  int n_blocks;  // blocks holding at least one key visible to some row
  int n_full;    // leading blocks whose keys are visible to every row
};

SDPA_HD int imin(int a, int b) { return a < b ? a : b; }
SDPA_HD int imax(int a, int b) { return a > b ? a : b; }

SDPA_HD KBlockRange kblock_range(int row0, int row_end, int q_len, int kv_len, int block_k, bool causal) {
  int kv_end = kv_len, kv_full = kv_len;
  if (causal) {
    const int off = kv_len - q_len;
    kv_end = imin(imax(row_end + off, 0), kv_len);   // keys visible to the last row
    kv_full = imin(imax(row0 + off + 1, 0), kv_len); // keys visible to the first row
  }
  KBlockRange r;
  r.n_blocks = (kv_end + block_k - 1) / block_k;
  r.n_full = imin(kv_full / block_k, r.n_blocks);
  return r;
}

}  // namespace sdpa
