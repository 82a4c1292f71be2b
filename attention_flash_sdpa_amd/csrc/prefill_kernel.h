// prefill_kernel.h -- the one-wave-per-SIMD prefill kernel template
// (prefill_kernel<T, D, DV, CAUSAL, KS, CACHED, CALIGN, KVSPLIT>), included by prefill.hip
// (dense keys) and prefill_cached.hip (cached prefix + new keys), which
// compile their instantiations in parallel.  The design is described at the
// top of prefill.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "sdpa_bounds.h"
#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

// LDS reads of slots [a, b]: one K fragment per Q K slot when there is a
// next block, two transposed V^T halves per P V slot.
template <int NQK, int NSLOT, bool NEXT>
__host__ __device__ constexpr int reads_in(int a, int b) {
  int c = 0;
  for (int m = a; m <= b; ++m) c += m < NQK ? (NEXT ? 1 : 0) : (m < NSLOT ? 2 : 0);
  return c;
}

template <class T, int D, int DV, bool CAUSAL, int KS, bool CACHED, bool CALIGN = false, bool KVSPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const PrefillArgs a) {
  constexpr int BK = kPrefillBlockK;
  constexpr int NWS = kPrefillWaves / KS;       // waves sharing one K/V stream
  constexpr int KROW = D * 2, VROW = DV * 2;    // LDS bytes per key row
  constexpr int KCPR = D / 8, VCPR = DV / 8;    // 16-byte slots per row
  constexpr int KBYTES = BK * KROW, VBYTES = BK * VROW;
  constexpr int K_INSTR = BK * KCPR / 64 / NWS; // 1 KiB direct loads per wave per block
  constexpr int V_INSTR = BK * VCPR / 64 / NWS;
  constexpr int NT = DV / 32;                   // O^T accumulator tiles
  constexpr int KSTEPS = D / 16;                // MFMA k-steps of S^T = K Q^T
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "block too small for the fill");
  static_assert(64 % KCPR == 0 && 64 % VCPR == 0, "one load covers whole key rows");
  static_assert(KS == 1 || KS == 2, "one or two key ranges per workgroup");
  // LDS per key range: K buffers 0/1, then V buffers 0/1
  constexpr uint32_t KBUF0 = 0, KBUF1 = KBYTES;
  constexpr uint32_t VBUF0 = 2 * KBYTES, VBUF1 = 2 * KBYTES + VBYTES;
  constexpr uint32_t RANGE_BYTES = 2 * KBYTES + 2 * VBYTES;

  __shared__ __attribute__((aligned(1024))) char smem[KS * RANGE_BYTES];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kr_i = wave / NWS;  // key range of this wave
  const int wis = wave % NWS;   // wave index within its key range
  const uint32_t lds0 = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem + kr_i * RANGE_BYTES;
  const int hl = lane >> 5;     // lane half
  const int l32 = lane & 31;

  // ---- work decode -------------------------------------------------------
  // KVSPLIT: kv_splits workgroups share one tile's K blocks (consecutive
  // after the remap, so on one XCD): workgroup ksp of them takes its KS key
  // ranges and writes partials (a form of its own, so that the other forms
  // keep their compile-time range arithmetic)
  const int nsp = KVSPLIT ? a.kv_splits : 1;
  int wg = remap_xcd(blockIdx.x, a.num_groups);
  const int ksp = nsp > 1 ? wg % nsp : 0;
  if (nsp > 1) wg /= nsp;
  int qt = wg % a.q_tiles;
  int rest = wg / a.q_tiles;
  const int hg = rest % a.head_groups;
  rest /= a.head_groups;
  const int g = rest % a.head_kv;
  const int b = rest / a.head_kv;
  if (CAUSAL) qt = a.q_tiles - 1 - qt;  // heaviest causal tiles first
  const int hp_i = wis % a.heads_per_group;
  const int qp_i = wis / a.heads_per_group;
  // heads_per_group need not divide the group size: waves past the group's
  // last head run the loop (uniform barriers) but store nothing
  const bool head_ok = hg * a.heads_per_group + hp_i < a.group;
  const int h = g * a.group + min(hg * a.heads_per_group + hp_i, a.group - 1);
  const int Sq = a.q_len, Sk = a.kv_len, off = Sk - Sq;
  const int wg_row0 = qt * (kRowsPerWave * a.qtiles_per_group);
  const int row0 = wg_row0 + kRowsPerWave * qp_i;
  const int wg_row_end = min(wg_row0 + kRowsPerWave * a.qtiles_per_group, Sq);

  // K blocks of the workgroup: [0, n_full) unmasked, [n_full, n_blocks) masked
  const KBlockRange kr = kblock_range(wg_row0, wg_row_end, Sq, Sk, BK, CAUSAL);
  const int n_blocks = kr.n_blocks;
  const int n_full = kr.n_full;

  const int qrow = row0 + l32;
  const bool row_ok = head_ok && qrow < Sq;
  typedef uint16_t elem_t;
  elem_t* __restrict__ optr = (elem_t*)a.o;
  // split across workgroups: this row's partial (row-major over (batch, query
  // row, query head), then split); formed where it is stored, so that
  // nothing of it stays live through the mainloop
  auto partial_row = [&]() __attribute__((always_inline)) -> size_t {
    return ((size_t)(b * Sq + qrow) * a.head_q + h) * nsp + ksp;
  };

  // Key ranges: the tile's n_blocks blocks are cut into R = KS * kv_splits
  // ranges of cnt = ceil(n_blocks / R) blocks; range r = ksp * KS + kr_i
  // takes blocks [r * cnt, (r + 1) * cnt).  Blocks past n_blocks lie past
  // every visible key and are masked entirely, so all ranges of a workgroup
  // run the same number of iterations.
  const int nr = KS * nsp;
  const int cnt = nr == 1 ? n_blocks : (n_blocks + nr - 1) / nr;
  const int kb0 = (ksp * KS + kr_i) * cnt;
  const int n_unmasked = min(max(n_full - kb0, 0), cnt);

  // no visible key for any row of this workgroup (or, split across
  // workgroups, none in its ranges): O = 0 and lse = -inf, or the empty
  // partial (max -inf, sum 0, zero output)
  if (n_blocks == 0 || ksp * KS * cnt >= n_blocks) {
    if (row_ok && kr_i == 0) {
      if (nsp > 1) {
        const size_t prow = partial_row();
        float* po = a.part_o + prow * DV;
        for (int c = hl * (DV / 2); c < (hl + 1) * (DV / 2); c += 4) *(f32x4_t*)(po + c) = f32x4_t{0, 0, 0, 0};
        if (hl == 0) *(f32x2_t*)(a.part_ml + 2 * prow) = f32x2_t{-INFINITY, 0.f};
      } else {
        elem_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
        for (int c = hl * (DV / 2); c < (hl + 1) * (DV / 2); c += 8) *(u32x4_t*)(orow + c) = u32x4_t{0, 0, 0, 0};
        if (a.lse != nullptr && hl == 0) a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = -INFINITY;
      }
    }
    return;
  }

  // ---- direct global -> LDS fills ------------------------------------------
  // Instruction i of this wave covers the 64 16-byte slots starting at slot
  // (wis*INSTR + i)*64; lane p holds slot P: row P / CPR, position P % CPR,
  // which receives chunk (P % CPR) ^ swizzle(row) of that key row.
  const char* kg = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * (D * 2);
  const char* vg = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * (DV * 2);
  const int kstride = a.head_kv * D * 2;  // bytes between consecutive keys
  const int vstride = a.head_kv * DV * 2;
  // Cached-KV prefill: the key sequence is the cached prefix followed by the
  // chunk's own keys (kv_len counts both), so the block walk and the masks
  // are those of one sequence of kv_len keys with bottom-right causality,
  // which on these keys leaves every cached key visible to every query (the
  // caller keeps q_len <= new keys).  Only the address of key t changes:
  // (t < cache_len ? cache : new - cache_len rows) + t * stride, chosen per
  // lane, so a block may straddle the two tensors.
  const int Sc = CACHED ? a.cache_len : 0;
  uint64_t kc_base = 0, vc_base = 0, kn_base = 0, vn_base = 0;
  if constexpr (CACHED) {
    const size_t new_rows = (size_t)(Sk - Sc);
    kc_base = (uint64_t)(uintptr_t)a.k_cache + ((size_t)b * a.cache_cap * a.head_kv + g) * (D * 2);
    vc_base = (uint64_t)(uintptr_t)a.v_cache + ((size_t)b * a.cache_cap * a.head_kv + g) * (DV * 2);
    kn_base = (uint64_t)(uintptr_t)a.k + (b * new_rows * a.head_kv + g) * (D * 2) - (uint64_t)Sc * kstride;
    vn_base = (uint64_t)(uintptr_t)a.v + (b * new_rows * a.head_kv + g) * (DV * 2) - (uint64_t)Sc * vstride;
  }
  // lane address of 16-byte chunk ch of key t (cached form only)
  auto cached_addr = [&](bool is_v, int t, uint32_t ch) __attribute__((always_inline)) -> uint64_t {
    const uint64_t base = t < Sc ? (is_v ? vc_base : kc_base) : (is_v ? vn_base : kn_base);
    return base + (uint64_t)(uint32_t)t * (uint32_t)(is_v ? vstride : kstride) + ch;
  };
  // per fill instruction: the lane's key row within the block and the byte
  // offset of its 16-byte chunk within the key row
  int krow[K_INSTR], vrow[V_INSTR];
  uint32_t kch[K_INSTR], vch[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int slot = (wis * K_INSTR + i) * 64 + lane, r = slot / KCPR;
    krow[i] = r;
    kch[i] = fill_chunk_prefill<KCPR>(slot) * 16;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = (wis * V_INSTR + i) * 64 + lane, r = slot / VCPR;
    vrow[i] = r;
    vch[i] = fill_chunk_prefill<VCPR>(slot) * 16;
  }
  const int last_key = Sk - 1;
  // lane byte offsets within a whole block, less the instruction offset
  // (i % 4) KiB that load i adds to both of its addresses (four loads share
  // one M0 value)
  uint32_t kfo[K_INSTR], vfo[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) kfo[i] = krow[i] * kstride + kch[i] - (i % 4) * 1024;
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) vfo[i] = vrow[i] * vstride + vch[i] - (i % 4) * 1024;
  // First key held by the LDS copy of block kb: its own start, except for a
  // block that would run past the last key, which is loaded as the last BK
  // keys instead (its keys before kb*BK, already processed, are masked).  So
  // every load is a whole block at a scalar base with fixed lane offsets.
  // With fewer than BK keys in all (one block) the rows past the end re-read
  // the last key and are masked.
  const bool whole_tail = Sk >= BK;
  auto row0_of = [&](int kb) __attribute__((always_inline)) -> int {
    return whole_tail ? min(kb * BK, Sk - BK) : kb * BK;
  };
  // one fill instruction i of block j of this range into LDS buffer buf
  auto fill_k1 = [&](int j, uint32_t buf, int i) __attribute__((always_inline)) {
    const int kb = kb0 + j;
    const uint32_t l = lds0 + buf + (wis * K_INSTR + i) * 1024;
    if constexpr (CACHED) {
      const int t = whole_tail ? row0_of(kb) + krow[i] : min(kb * BK + krow[i], last_key);
      global_to_lds_16((const void*)(uintptr_t)cached_addr(false, t, kch[i]), l);
    } else if (whole_tail)
      global_to_lds_16_sbase(kg + (size_t)row0_of(kb) * kstride, kfo[i] + (i % 4) * 1024, l);
    else
      global_to_lds_16_sbase(kg, (uint32_t)(min(kb * BK + krow[i], last_key) * kstride) + kch[i], l);
  };
  auto fill_v1 = [&](int j, uint32_t buf, int i) __attribute__((always_inline)) {
    const int kb = kb0 + j;
    const uint32_t l = lds0 + buf + (wis * V_INSTR + i) * 1024;
    if constexpr (CACHED) {
      const int t = whole_tail ? row0_of(kb) + vrow[i] : min(kb * BK + vrow[i], last_key);
      global_to_lds_16((const void*)(uintptr_t)cached_addr(true, t, vch[i]), l);
    } else if (whole_tail)
      global_to_lds_16_sbase(vg + (size_t)row0_of(kb) * vstride, vfo[i] + (i % 4) * 1024, l);
    else
      global_to_lds_16_sbase(vg, (uint32_t)(min(kb * BK + vrow[i], last_key) * vstride) + vch[i], l);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once, then K(0),
  // V(0) and K(1) (block 0 again when there is no block 1, into a buffer
  // nothing reads): all in flight at once, the first block's scores wait for
  // Q and K(0) only
  u32x4_t qf[KSTEPS];
  {
    const elem_t* qptr = (const elem_t*)a.q + ((size_t)(b * Sq + min(qrow, Sq - 1)) * a.head_q + h) * D + 8 * hl;
    static_for<KSTEPS>([&](auto s) __attribute__((always_inline)) {
      constexpr int S = decltype(s)::value;
      // the cached form computes its fill addresses lane by lane in the
      // prologue, and the register allocator then reuses registers of
      // untracked loads still in flight; it loads Q with tracked loads (the
      // compiler's own wait then also covers K(0), V(0) and K(1))
      if constexpr (CACHED)
        qf[S] = *(const u32x4_t*)((const char*)qptr + 32 * S);
      else
        global_load_16_untracked<32 * S>(qf[S], qptr);
    });
  }
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) fill_k1(0, KBUF0, i);
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) fill_v1(0, VBUF0, i);
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) fill_k1(min(1, cnt - 1), KBUF1, i);

  // ---- per-lane LDS read offsets -----------------------------------------
  // K fragment (A operand): key row l%32 (+32 for the second score tile),
  // head-dim slot 2*s + l/32.
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    koff[s] = lds0 + prefill_k_read<KCPR>(lane, s);
  // V^T fragment (A operand of O^T = V^T P^T) via ds_read_b64_tr_b16: lane
  // (group gq = l/16, s = l%16) addresses key row 4*(gq/2) + s/4 (+8 for the
  // second half, +16 per key chunk) at value columns 32t + 16*(gq%2) +
  // 4*(s%4).  The swizzle of rows r and r + 8 differs, so both halves get
  // offsets; +16 rows per key chunk leaves it unchanged.
  uint32_t voff[2][NT];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int t = 0; t < NT; ++t) voff[hf][t] = lds0 + prefill_vt_read<VCPR>(lane, hf, t);

  // ---- online softmax state ----------------------------------------------
  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -INFINITY;  // running max of s2*S for query l%32 (log2 domain)
  float l_run = 0.f;        // this lane's share of the running sum
  const float s2 = a.s2;
  f32x16_t sa[2], sb[2];    // score tiles of two consecutive blocks


  // Visible positions of block kb for this lane: register r of score tile t
  // holds key row0 + 4*hl + 32t + 8(r/4) + r%4, visible iff it is at least
  // kb*BK (not processed before) and at most the row's last visible key; the
  // position 32t + 8(r/4) + r%4 must lie in [lo, hi].
  struct Window {
    int lo, hi;
  };
  auto window = [&](int kb) __attribute__((always_inline)) -> Window {
    const int base = row0_of(kb) + 4 * hl;
    return Window{kb * BK - base, (CAUSAL ? min(Sk - 1, qrow + off) : Sk - 1) - base};
  };

  // Block row max (log2 domain, scale folded in).  In a masked block the
  // scores are replaced in place by s2*S or -inf.
  auto block_max = [&](int j, f32x16_t (&sc)[2], auto masked_tag) __attribute__((always_inline)) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (MASKED) {
      const Window w = window(kb0 + j);
      float bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = 32 * t + 8 * (r >> 2) + (r & 3);
          const float x = (pos >= w.lo && pos <= w.hi) ? sc[t][r] * s2 : -INFINITY;
          sc[t][r] = x;
          bmax = fmaxf(bmax, x);
        }
      return bmax;
    } else {
      float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = (t == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
      return mx * s2;
    }
  };

  // Row max across the lane pair and lazy rescale: the running max only moves
  // (and O, l are rescaled by 2^(m_old - m_new)) when some row's block max
  // exceeds it by more than kSlack; otherwise the stale max is kept, so
  // P <= 2^kSlack.  The final O / l is unchanged because l accumulates the
  // same P values.  Returns the subtrahend m of P = 2^(s2*S - m).
  auto update_max = [&](float bmax, auto masked_tag) __attribute__((always_inline)) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    bmax = pair_max(bmax);
    const float m_new = fmaxf(m_run, bmax);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kSlack)) {
      // rows that have seen no visible key keep m = -inf (masked blocks only)
      const float m_tgt = MASKED ? (m_new == -INFINITY ? 0.f : m_new) : m_new;
      const float alpha = fast_exp2(m_run - m_tgt);
      l_run *= alpha;
      mfma_acc_drain(acc);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
      m_run = m_new;
    }
    return MASKED ? (m_run == -INFINITY ? 0.f : m_run) : m_run;
  };

  // ---- one pipeline iteration, as a fixed sequence of MFMA slots ----------
  // Iteration j (PAR = j & 1): on entry the scores of block j are in
  // registers with their subtrahend m_sub, K(j+1) sits in K buffer 1-PAR and
  // V(j) in V buffer PAR, and every wave is past the reads of the previous
  // iteration.  It runs 2*KSTEPS QK slots (the scores
  // of block j+1, two 32-key tiles) followed by 4*NT PV slots (O^T += V^T P^T
  // of block j, four 16-key chunks).  Every slot issues one MFMA, the LDS
  // fragment reads of the slot kPD places ahead, one share of the vector work
  // and, every few slots, one of the direct loads of V(j+1) / K(j+2) into the
  // buffers the previous iteration freed.  The vector work is spread so that
  // it runs under the matrix core:
  //   QK slots:          exponentials of score tile 0 of block j and of the
  //                      first half of tile 1
  //   first half of PV:  exponentials of the rest of tile 1 (chunk 3, used
  //                      from the last quarter of the PV slots on)
  //   second half of PV: row max of block j+1
  // A scheduling fence closes each slot, so the order is the one written.
  constexpr int NQK = 2 * KSTEPS;               // QK slots
  constexpr int NPV = 4 * NT;                   // PV slots
  constexpr int NSLOT = NQK + NPV;
  constexpr int kPD = 4;                        // read-ahead distance (slots)
  constexpr int NDMA = K_INSTR + V_INSTR;
  // the direct loads go one per DSTRIDE slots; the split form streams its
  // keys from HBM (no other workgroup shares them), so it issues them in the
  // first slots and gives them the rest of the iteration to land
  constexpr int DSTRIDE = KVSPLIT ? 1 : (NSLOT / NDMA > 0 ? NSLOT / NDMA : 1);
  static_assert(NQK % 8 == 0 && NPV % 4 == 0, "slot counts");

  auto iteration = [&](int j, float m_sub, auto mcur_tag, auto mnext_tag, auto next_tag, auto par_tag)
      __attribute__((always_inline)) -> float {
    constexpr bool MCUR = decltype(mcur_tag)::value;
    constexpr bool MNEXT = decltype(mnext_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr uint32_t KB_NEXT = PAR ? KBUF0 : KBUF1;   // holds K(j+1)
    constexpr uint32_t KB_FREE = PAR ? KBUF1 : KBUF0;   // receives K(j+2)
    constexpr uint32_t VB_CUR = PAR ? VBUF1 : VBUF0;    // holds V(j)
    constexpr uint32_t VB_FREE = PAR ? VBUF0 : VBUF1;   // receives V(j+1)
    f32x16_t(&s_cur)[2] = PAR ? sb : sa;
    f32x16_t(&s_nxt)[2] = PAR ? sa : sb;

    // Direct loads of this iteration, V(j+1) then K(j+2), without branches:
    // an iteration with a next block implies more than BK keys, so every
    // load is a whole block (the tail block shifted, see row0_of); when there
    // is no block j+2 the K loads re-read block j+1 into the free buffer,
    // which nothing reads afterwards.
    const int kbv = kb0 + j + 1;
    const int kbk = kb0 + min(j + 2, cnt - 1);
    const int vrow0 = row0_of(kbv), krow0 = row0_of(kbk);
    const char* vsrc = vg + (size_t)vrow0 * vstride;
    const char* ksrc = kg + (size_t)krow0 * kstride;
    // cached form: the two candidate bases of each block (scalars)
    const uint64_t kcb = kc_base + (uint64_t)krow0 * kstride, knb = kn_base + (uint64_t)krow0 * kstride;
    const uint64_t vcb = vc_base + (uint64_t)vrow0 * vstride, vnb = vn_base + (uint64_t)vrow0 * vstride;
    const uint32_t vl = lds0 + VB_FREE + wis * V_INSTR * 1024;
    const uint32_t kl = lds0 + KB_FREE + wis * K_INSTR * 1024;
    auto dma = [&](auto i_tag) __attribute__((always_inline)) {
      constexpr int I = decltype(i_tag)::value;
      constexpr bool IS_V = I < V_INSTR;
      constexpr int i = IS_V ? I : I - V_INSTR;
      // load i goes to LDS (group base) + (i / 4) * 4 KiB + (i % 4) KiB; the
      // first load from each base waits for its SGPRs, the first of each
      // group of four for its M0 write, the rest for nothing
      constexpr int WAITS = i == 0 ? 5 : (i % 4 == 0 ? 1 : 0);
      if constexpr (CACHED && CALIGN) {
        // cache length and key count are multiples of the RSTEP rows one
        // load covers, so every load lies in one tensor: its base is a
        // scalar choice and the lane offsets are the dense form's
        constexpr int RSTEP = 64 / (IS_V ? VCPR : KCPR);
        const int first = (IS_V ? vrow0 : krow0) + (wis * (IS_V ? V_INSTR : K_INSTR) + i) * RSTEP;
        const uint64_t base = first < Sc ? (IS_V ? vcb : kcb) : (IS_V ? vnb : knb);
        global_to_lds_16_off<(i % 4) * 1024, WAITS>((const void*)(uintptr_t)base, IS_V ? vfo[i] : kfo[i],
                                                  (IS_V ? vl : kl) + (i / 4) * 4096);
      } else if constexpr (CACHED) {
        // per-lane addresses (the block may straddle cache and new keys).
        // The lane's key row in load i is row[0] + i * 64 / CPR, so whether
        // it is cached is one compare against a scalar bound; the address is
        // the block's cache or new base plus the lane offset kept for the
        // dense form (which already holds -OFF).
        constexpr int RSTEP = 64 / (IS_V ? VCPR : KCPR);
        const int lim = Sc - (IS_V ? vrow0 : krow0) - i * RSTEP;
        const bool in_cache = (IS_V ? vrow[0] : krow[0]) < lim;
        const uint64_t base = in_cache ? (IS_V ? vcb : kcb) : (IS_V ? vnb : knb);
        global_to_lds_16_voff<(i % 4) * 1024, (WAITS ? 1 : 0)>(
            (const void*)(uintptr_t)(base + (IS_V ? vfo[i] : kfo[i])), (IS_V ? vl : kl) + (i / 4) * 4096);
      } else if constexpr (IS_V)
        global_to_lds_16_off<(i % 4) * 1024, WAITS>(vsrc, vfo[i], vl + (i / 4) * 4096);
      else
        global_to_lds_16_off<(i % 4) * 1024, WAITS>(ksrc, kfo[i], kl + (i / 4) * 4096);
    };

    // visible window of block j+1 (masked flavour only)
    const Window w_next = window(kb0 + j + 1);

    u32x4_t kfr[NQK];    // K fragments, one per QK slot
    u32x4_t vfr[NPV];    // V^T fragments, one per PV slot
    u32x4_t pf[4];       // packed P of block j, one per 16-key chunk
    float bmax = -INFINITY;
    // LDS reads of slot N (issued kPD slots ahead of its MFMA)
    auto read = [&](auto n_tag) __attribute__((always_inline)) {
      constexpr int N = decltype(n_tag)::value;
      if constexpr (N < NQK) {
        if constexpr (NEXT) kfr[N] = ds_read_b128_at<KB_NEXT + (N % 2) * 32 * KROW>(koff[N / 2]);
      } else if constexpr (N < NSLOT) {
        constexpr int m = N - NQK, c = m / NT, t = m % NT;
        const u32x2_t lo = ds_read_tr16_at<VB_CUR + 16 * c * VROW>(voff[0][t]);
        const u32x2_t hi = ds_read_tr16_at<VB_CUR + 16 * c * VROW>(voff[1][t]);
        vfr[m] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      }
    };
    auto maxv = [&](int t, int r) __attribute__((always_inline)) {
      if constexpr (MNEXT) {
        const int pos = 32 * t + 8 * (r >> 2) + (r & 3);
        const float x = (pos >= w_next.lo && pos <= w_next.hi) ? s_nxt[t][r] * s2 : -INFINITY;
        s_nxt[t][r] = x;
        bmax = fmaxf(bmax, x);
      } else {
        bmax = fmaxf(bmax, s_nxt[t][r]);
      }
    };
    // exponentials of score tile TL, values [R0, R1): pairs are packed into
    // the PV operand of their 16-key chunk and added to the row sum
    float pend[2] = {0.f, 0.f};  // even value of a pair awaiting its partner
    auto exp_range = [&](auto tl_tag, auto r0_tag, auto r1_tag) __attribute__((always_inline)) {
      constexpr int TL = decltype(tl_tag)::value;
      constexpr int R0 = decltype(r0_tag)::value, R1 = decltype(r1_tag)::value;
#pragma unroll
      for (int r = R0; r < R1; ++r) {
        // exponent and exponential in one asm block that reads the score
        // where the MFMA left it (anchoring the work to this slot without
        // copying the score out of its tile first); the compiler keeps a wait
        // state between the block and the first use of its result, which the
        // exponential needs
        float p;
        if constexpr (MCUR)
          asm volatile("v_sub_f32 %0, %1, %2\n\tv_exp_f32 %0, %0" : "=&v"(p) : "v"(s_cur[TL][r]), "v"(m_sub));
        else
          asm volatile("v_fma_f32 %0, %1, %2, -%3\n\tv_exp_f32 %0, %0"
                       : "=&v"(p) : "v"(s_cur[TL][r]), "s"(s2), "v"(m_sub));
        if (r & 1) {
          uint32_t pk = pack2<T>(pend[TL], p);
          l_run += pend[TL] + p;  // row sum over the fp32 values
          asm volatile("" ::"v"(pk));  // computed in this slot; not tied, so it
                                        // can be formed in its operand register
          pf[2 * TL + (r >> 3)][(r & 7) >> 1] = pk;
        } else {
          pend[TL] = p;
          pin(pend[TL]);
        }
      }
      if constexpr (R1 > R0) pin(l_run);
    };
    auto slot = [&](auto n_tag) __attribute__((always_inline)) {
      constexpr int N = decltype(n_tag)::value;
      // one LDS wait per pair of slots: the even slot waits for its own and
      // the next slot's fragments (the reads of slots N+2 .. N+kPD may stay
      // in flight; slot N+1+kPD's read is issued later), the odd slot none
      constexpr int LGKM = N % 2 == 0 ? reads_in<NQK, NSLOT, NEXT>(N + 2, N + kPD) : -1;
      read(std::integral_constant<int, N + kPD>{});
      if constexpr (N < NQK) {
        if constexpr (NEXT) {
          if constexpr (N < 2)
            mfma_s_first<T, LGKM>(s_nxt[N % 2], kfr[N], qf[N / 2]);
          else
            mfma_s_acc<T, LGKM>(s_nxt[N % 2], kfr[N], qf[N / 2]);
        }
        // exponentials of tile 0 (all) and of the first half of tile 1
        exp_range(std::integral_constant<int, 0>{}, std::integral_constant<int, N * 16 / NQK>{},
                  std::integral_constant<int, (N + 1) * 16 / NQK>{});
        exp_range(std::integral_constant<int, 1>{}, std::integral_constant<int, N * 8 / NQK>{},
                  std::integral_constant<int, (N + 1) * 8 / NQK>{});
        if constexpr (NEXT && N == NQK - 1) mfma_s_drain(s_nxt);
      } else {
        constexpr int m = N - NQK, c = m / NT, t = m % NT;
        mfma_o_acc<T, LGKM>(acc[t], vfr[m], pf[c]);
        constexpr int H = NPV / 2;
        if constexpr (m < H) {
          // second half of tile 1 (chunk 3 is used from slot 3*NT on)
          exp_range(std::integral_constant<int, 1>{}, std::integral_constant<int, 8 + m * 8 / H>{},
                    std::integral_constant<int, 8 + (m + 1) * 8 / H>{});
        } else if constexpr (NEXT) {
          // row max of block j+1 over the remaining slots
          constexpr int q = m - H;
          pin(bmax);
#pragma unroll
          for (int e = q * 32 / H; e < (q + 1) * 32 / H; ++e) maxv(e / 16, e % 16);
          pin(bmax);
        }
      }
      if constexpr (NEXT && N % DSTRIDE == 0 && N / DSTRIDE < NDMA)
        dma(std::integral_constant<int, N / DSTRIDE>{});
    };

    __builtin_amdgcn_sched_barrier(0);
    static_for<kPD>([&](auto n) __attribute__((always_inline)) { read(n); });
    static_for<NSLOT>([&](auto n) __attribute__((always_inline)) { slot(n); });
    // the accumulators may be copied between registers at block boundaries:
    // let the last P V MFMAs finish first
    mfma_acc_drain(acc);
    __builtin_amdgcn_sched_barrier(0);

    float m_next = 0.f;
    if constexpr (NEXT) {
      m_next = update_max(MNEXT ? bmax : bmax * s2, mnext_tag);
      wait_vmcnt<0>();  // V(j+1), K(j+2) have landed
      __syncthreads();  // ... for every wave, which are all past this iteration
    }
    return m_next;
  };

  using Unmasked = std::false_type;
  using Masked = std::true_type;
  using Next = std::true_type;
  using Last = std::false_type;
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  float m_sub = 0.f;  // subtrahend of the block whose scores are in registers
  // Iterations [j0, j1) of one flavour, unrolled by two so that the score
  // tiles visibly alternate (block j in sa for even j, in sb for odd j).
  auto run = [&](int j0, int j1, auto mcur_tag, auto mnext_tag) __attribute__((always_inline)) {
    int j = j0;
    if (j < j1 && (j & 1)) {
      m_sub = iteration(j, m_sub, mcur_tag, mnext_tag, Next{}, Par1{});
      ++j;
    }
    for (; j + 1 < j1; j += 2) {
      m_sub = iteration(j, m_sub, mcur_tag, mnext_tag, Next{}, Par0{});
      m_sub = iteration(j + 1, m_sub, mcur_tag, mnext_tag, Next{}, Par1{});
    }
    if (j < j1) m_sub = iteration(j, m_sub, mcur_tag, mnext_tag, Next{}, Par0{});
  };

  // ---- K-block pipeline ---------------------------------------------------
  // prologue: once Q and K(0) have landed (V(0) and K(1) may still be in
  // flight), the scores and max of block 0
  if constexpr (CACHED)
    wait_vmcnt<V_INSTR + K_INSTR>();
  else
    wait_vmcnt_pin<V_INSTR + K_INSTR>(qf);
  qf[0] = row_ok ? qf[0] : u32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int s = 1; s < KSTEPS; ++s) qf[s] = row_ok ? qf[s] : u32x4_t{0, 0, 0, 0};
  __syncthreads();
  {
    constexpr int NQK0 = 2 * KSTEPS, PD = 4;
    u32x4_t kfr0[NQK0];
    auto rd = [&](auto n_tag) __attribute__((always_inline)) {
      constexpr int N = decltype(n_tag)::value;
      if constexpr (N < NQK0) kfr0[N] = ds_read_b128_at<KBUF0 + (N % 2) * 32 * KROW>(koff[N / 2]);
    };
    __builtin_amdgcn_sched_barrier(0);
    static_for<PD>([&](auto n) __attribute__((always_inline)) { rd(n); });
    static_for<NQK0>([&](auto n) __attribute__((always_inline)) {
      constexpr int N = decltype(n)::value;
      constexpr int LGKM = (NQK0 - 1 - N) < PD ? (NQK0 - 1 - N) : PD;
      rd(std::integral_constant<int, N + PD>{});
      if constexpr (N < 2)
        mfma_s_first<T, LGKM>(sa[N % 2], kfr0[N], qf[N / 2]);
      else
        mfma_s_acc<T, LGKM>(sa[N % 2], kfr0[N], qf[N / 2]);
    });
    mfma_s_drain(sa);
    __builtin_amdgcn_sched_barrier(0);
  }
  // first block: O and l are still zero, so the running max is simply set
  if (n_unmasked > 0) {
    m_run = pair_max(block_max(0, sa, Unmasked{}));
    m_sub = m_run;
  } else {
    m_run = pair_max(block_max(0, sa, Masked{}));
    m_sub = m_run == -INFINITY ? 0.f : m_run;
  }
  wait_vmcnt<0>();  // V(0), K(1)
  __syncthreads();  // and every wave is past its reads of K buffer 0

  // iterations with a next block: [0, cnt-1); block j is masked iff j >= u
  const int n_next = cnt - 1;
  const int u = n_unmasked;
  const int ju = min(max(u - 1, 0), n_next);  // last iteration with both blocks unmasked, + 1
  run(0, ju, Unmasked{}, Unmasked{});
  if (ju < n_next && ju < u) {   // block ju unmasked, block ju+1 masked
    if (ju & 1)
      m_sub = iteration(ju, m_sub, Unmasked{}, Masked{}, Next{}, Par1{});
    else
      m_sub = iteration(ju, m_sub, Unmasked{}, Masked{}, Next{}, Par0{});
    run(ju + 1, n_next, Masked{}, Masked{});
  } else {
    run(ju, n_next, Masked{}, Masked{});
  }
  // the last block (peeled)
  if (n_next < u) {
    if (n_next & 1)
      iteration(n_next, m_sub, Unmasked{}, Unmasked{}, Last{}, Par1{});
    else
      iteration(n_next, m_sub, Unmasked{}, Unmasked{}, Last{}, Par0{});
  } else {
    if (n_next & 1)
      iteration(n_next, m_sub, Masked{}, Masked{}, Last{}, Par1{});
    else
      iteration(n_next, m_sub, Masked{}, Masked{}, Last{}, Par0{});
  }

  mfma_acc_drain(acc);  // the last P V MFMAs have written the accumulators

  // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------
  // Value tiles [T0, T1) of this wave's rows.
  auto store = [&](auto t0_tag, auto t1_tag) __attribute__((always_inline)) {
    constexpr int T0 = decltype(t0_tag)::value, T1 = decltype(t1_tag)::value;
    const float l_tot = pair_sum(l_run);
    if (nsp > 1) {
      // split across workgroups: the unnormalized accumulators (register r
      // of tile t holds value column 32t + 8(r/4) + 4*hl + r%4) and (m, l)
      if (row_ok) {
        const size_t prow = partial_row();
        float* po = a.part_o + prow * DV + 4 * hl;
#pragma unroll
        for (int t = T0; t < T1; ++t)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(f32x4_t*)(po + 32 * t + 8 * q4) =
                f32x4_t{acc[t][4 * q4], acc[t][4 * q4 + 1], acc[t][4 * q4 + 2], acc[t][4 * q4 + 3]};
        if (hl == 0 && T0 == 0) *(f32x2_t*)(a.part_ml + 2 * prow) = f32x2_t{m_run, l_tot};
      }
      return;
    }
    const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
    u32x4_t runs[T1 - T0][2];
#pragma unroll
    for (int t = T0; t < T1; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x2_t w[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int r = 8 * p + 4 * k;
          w[k].x = pack2<T>(acc[t][r + 0] * inv, acc[t][r + 1] * inv);
          w[k].y = pack2<T>(acc[t][r + 2] * inv, acc[t][r + 3] * inv);
        }
        runs[t - T0][p] = pair_runs16(w[0], w[1]);
      }
    if (row_ok) {
      elem_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
#pragma unroll
      for (int t = T0; t < T1; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) *(u32x4_t*)(orow + 32 * t + 16 * p + 8 * hl) = runs[t - T0][p];
      if (a.lse != nullptr && hl == 0 && T0 == 0)
        a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  };

  if constexpr (KS == 1) {
    store(std::integral_constant<int, 0>{}, std::integral_constant<int, NT>{});
  } else {
    // ---- merge of the two key ranges through LDS ---------------------------
    // Each range finalizes half of the value tiles of its rows: range 0 tiles
    // [0, NT/2), range 1 [NT/2, NT).  A wave hands the other half of its
    // accumulators and its (m, l) to its partner wave (same rows, other range)
    // as 16-byte lane-major rows (conflict-free), then merges its own half.
    constexpr int H = NT / 2;
    constexpr int XROWS = H * 4 + 1;
    static_assert(2 * NWS * XROWS * 1024 <= sizeof(smem), "merge area");
    __syncthreads();  // every wave is past its last LDS read
    SDPA_LDS f32x4_t* xout = (SDPA_LDS f32x4_t*)((SDPA_LDS char*)smem) + (kr_i * NWS + wis) * XROWS * 64 + lane;
    SDPA_LDS f32x4_t* xin = (SDPA_LDS f32x4_t*)((SDPA_LDS char*)smem) + ((1 - kr_i) * NWS + wis) * XROWS * 64 + lane;
    auto hand_over = [&](auto t0_tag) __attribute__((always_inline)) {
      constexpr int T0 = decltype(t0_tag)::value;
#pragma unroll
      for (int t = 0; t < H; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xout[(t * 4 + q4) * 64] = f32x4_t{acc[T0 + t][4 * q4], acc[T0 + t][4 * q4 + 1], acc[T0 + t][4 * q4 + 2],
                                            acc[T0 + t][4 * q4 + 3]};
      xout[H * 4 * 64] = f32x4_t{m_run, l_run, 0.f, 0.f};
    };
    auto merge = [&](auto t0_tag) __attribute__((always_inline)) {
      constexpr int T0 = decltype(t0_tag)::value;
      const f32x4_t ml = xin[H * 4 * 64];
      const float m1 = ml[0], l1 = ml[1];
      const float mm = fmaxf(m_run, m1);
      const float w0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
      const float w1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
      l_run = l_run * w0 + l1 * w1;
      m_run = mm;
#pragma unroll
      for (int t = 0; t < H; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t o1 = xin[(t * 4 + q4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[T0 + t][4 * q4 + e] = acc[T0 + t][4 * q4 + e] * w0 + o1[e] * w1;
        }
    };
    using Lo = std::integral_constant<int, 0>;
    using Hi = std::integral_constant<int, H>;
    using End = std::integral_constant<int, NT>;
    if (kr_i == 0) hand_over(Hi{});
    else hand_over(Lo{});
    __syncthreads();
    if (kr_i == 0) {
      merge(Lo{});
      store(Lo{}, Hi{});
    } else {
      merge(Hi{});
      store(Hi{}, End{});
    }
  }
}

}  // namespace sdpa
