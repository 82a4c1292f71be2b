// prefill_o2_kernel.h -- the 32-row prefill mainloop in its two-waves-per-SIMD
// form (prefill_o2_kernel<T, D, DV, CAUSAL, NW, KS, BK, CACHED, BIAS>),
// included by prefill_o2.hip (dense keys, and with BIAS the full additive
// mask) and prefill_cached.hip (cached prefix + new keys).  The design is
// described at the top of prefill_o2.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "sdpa_bounds.h"
#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <class T, int D, int DV, bool CAUSAL, int NW, int KS, int BKT, bool CACHED, bool BIAS = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_o2_kernel(const PrefillArgs a) {
  constexpr int BK = BKT;                     // keys per block
  constexpr int NWS = NW / KS;                // waves sharing one K/V stream
  constexpr int NTL = BK / 32;                // 32-key score tiles per block
  constexpr int NCH = BK / 16;                // 16-key PV chunks per block
  constexpr int KROW = D * 2, VROW = DV * 2;  // LDS bytes per key row
  constexpr int KCPR = D / 8, VCPR = DV / 8;  // 16-byte slots per row
  constexpr int KBYTES = BK * KROW, VBYTES = BK * VROW;
  constexpr int K_INSTR = BK * KCPR / 64 / NWS;  // 1 KiB direct loads per wave per block
  constexpr int V_INSTR = BK * VCPR / 64 / NWS;
  constexpr int NT = DV / 32;                    // O^T accumulator tiles
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "block too small for the fill");
  static_assert(NW % KS == 0 && (BK == 32 || BK == 64), "shape");
  static_assert(!BIAS || (KS == 1 && !CACHED), "the bias form streams one dense key range");
  constexpr int ML = BIAS ? NTL * 2 : 0;         // 16-byte bias loads per lane per block
  // LDS per key range: K buffers 0/1, then V buffers 0/1
  constexpr uint32_t KBUF0 = 0, KBUF1 = KBYTES;
  constexpr uint32_t VBUF0 = 2 * KBYTES, VBUF1 = 2 * KBYTES + VBYTES;
  constexpr uint32_t RANGE_BYTES = 2 * KBYTES + 2 * VBYTES;

  __shared__ __attribute__((aligned(1024))) char smem[KS * RANGE_BYTES];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kr_i = KS == 1 ? 0 : wave / NWS;     // key range of this wave
  const int wis = KS == 1 ? wave : wave % NWS;  // wave index within its key range
  const uint32_t lds0 = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem + kr_i * RANGE_BYTES;
  const int hl = lane >> 5;  // lane half
  const int l32 = lane & 31;

  // ---- work decode -------------------------------------------------------
  int wg = remap_xcd(blockIdx.x, a.num_groups);
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

  if (n_blocks == 0) {  // no visible key for any row of this workgroup
    if (row_ok && kr_i == 0) {
      elem_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
      for (int c = hl * (DV / 2); c < (hl + 1) * (DV / 2); c += 8) *(u32x4_t*)(orow + c) = u32x4_t{0, 0, 0, 0};
      if (a.lse != nullptr && hl == 0) a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = -INFINITY;
    }
    return;
  }

  // Key range of this wave: range r takes blocks [r*cnt, (r+1)*cnt); blocks
  // past n_blocks (the end of the last ranges) are masked entirely, so every
  // range runs the same number of iterations.
  const int cnt = (n_blocks + KS - 1) / KS;
  const int kb0 = kr_i * cnt;
  const int n_unmasked = min(max(n_full - kb0, 0), cnt);

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once; the prologue
  // waits for them together with K(0) ----------------------------------------
  u32x4_t qf[D / 16];
  {
    const elem_t* qptr = (const elem_t*)a.q + ((size_t)(b * Sq + min(qrow, Sq - 1)) * a.head_q + h) * D + 8 * hl;
    static_for<D / 16>([&](auto s) __attribute__((always_inline)) {
      constexpr int S = decltype(s)::value;
      // the cached form computes its fill addresses lane by lane, which lets
      // the register allocator reuse registers of untracked loads still in
      // flight: it loads Q with tracked loads
      if constexpr (CACHED)
        qf[S] = *(const u32x4_t*)((const char*)qptr + 32 * S);
      else
        global_load_16_untracked<32 * S>(qf[S], qptr);
    });
  }

  // ---- additive bias (BIAS): the values of this lane's scores, straight from
  // memory into registers one block ahead.  Register r of score tile t holds
  // key kb*BK + 32t + 8(r/4) + 4*hl + r%4: four runs of four keys.  The lane
  // pair (l, l+32) loads them as 16-byte pieces of row qrow (clamped to the
  // last row): load p of tile t brings keys 32t + 16p + 8*hl .. +7, and
  // bias_runs() exchanges the halves the partner needs.  A start past the
  // row is clamped to its last eight elements, which only moves loads of
  // keys past kv_len (masked anyway) and keeps every read inside the row.
  // One register set: iteration j reads block j's values, then loads block
  // j+1's into the same registers, which the next iteration's K/V wait
  // covers (the compiler does not count these loads; an ISA scan checks that
  // nothing touches the registers before it).
  const elem_t* mrow = nullptr;
  if constexpr (BIAS)
    mrow = (const elem_t*)a.mask + (size_t)b * a.mask_sb + (size_t)h * a.mask_sh +
           (size_t)min(qrow, Sq - 1) * a.mask_row;
  u32x4_t mv[BIAS ? NTL * 2 : 1];
  auto load_bias = [&](int kb, u32x4_t (&m)[BIAS ? NTL * 2 : 1]) __attribute__((always_inline)) {
    if constexpr (BIAS) {
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          global_load_16_untracked<0>(m[2 * t + p], mrow + min(kb * BK + 32 * t + 16 * p + 8 * hl, a.mask_row - 8));
    }
  };
  const float s_nat = a.s_nat;

  // ---- direct global -> LDS fills ------------------------------------------
  // Instruction i of this wave covers the 64 16-byte slots starting at slot
  // (wis*INSTR + i)*64; lane p holds slot P: row P / CPR, position P % CPR,
  // which receives chunk (P % CPR) ^ swizzle(row) of that key row.
  const char* kg = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * (D * 2);
  const char* vg = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * (DV * 2);
  const int kstride = a.head_kv * D * 2;  // bytes between consecutive keys
  const int vstride = a.head_kv * DV * 2;
  uint32_t kfo[K_INSTR], vfo[V_INSTR];    // byte offsets within a whole block, less (i % 4) KiB
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int slot = (wis * K_INSTR + i) * 64 + lane, r = slot / KCPR;
    kfo[i] = r * kstride + fill_chunk_prefill<KCPR>(slot) * 16 - (i % 4) * 1024;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = (wis * V_INSTR + i) * 64 + lane, r = slot / VCPR;
    vfo[i] = r * vstride + fill_chunk_prefill<VCPR>(slot) * 16 - (i % 4) * 1024;
  }
  const int last_key = Sk - 1;
  // Cached-KV prefill: keys 0 .. cache_len-1 come from the cache tensors
  // (cache_cap rows per batch entry), the rest from the new tensors, whose
  // row 0 is key cache_len; the lane picks its key's tensor, so a block may
  // straddle the two (the block walk and masks are those of one sequence of
  // kv_len keys)
  const int Sc = CACHED ? a.cache_len : 0;
  uint64_t kc_base = 0, vc_base = 0, kn_base = 0, vn_base = 0;
  if constexpr (CACHED) {
    const size_t new_rows = (size_t)(Sk - Sc);
    kc_base = (uint64_t)(uintptr_t)a.k_cache + ((size_t)b * a.cache_cap * a.head_kv + g) * (D * 2);
    vc_base = (uint64_t)(uintptr_t)a.v_cache + ((size_t)b * a.cache_cap * a.head_kv + g) * (DV * 2);
    kn_base = (uint64_t)(uintptr_t)a.k + (b * new_rows * a.head_kv + g) * (D * 2) - (uint64_t)Sc * kstride;
    vn_base = (uint64_t)(uintptr_t)a.v + (b * new_rows * a.head_kv + g) * (DV * 2) - (uint64_t)Sc * vstride;
  }
  // A block is whole if all its BK keys exist; in a ragged block (the last
  // one, or one past the end) rows past the last key re-read it (masked).
  // cached form: the scalar base of a whole block inside one tensor, or 0
  // for a block that straddles the two (or runs past the last key)
  auto cached_base = [&](int kb, uint64_t cbase, uint64_t nbase, int stride) __attribute__((always_inline)) {
    const int k0 = kb * BK;
    if (k0 + BK <= Sc) return cbase + (uint64_t)(uint32_t)k0 * (uint32_t)stride;
    if (k0 >= Sc && k0 + BK <= Sk) return nbase + (uint64_t)(uint32_t)k0 * (uint32_t)stride;
    return (uint64_t)0;
  };
  auto fill_k = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t l = lds0 + buf + wis * K_INSTR * 1024;
    const uint64_t cb = CACHED ? cached_base(kb, kc_base, kn_base, kstride) : 0;
    if (CACHED && cb != 0) {
      static_for<K_INSTR>([&](auto i_tag) __attribute__((always_inline)) {
        constexpr int i = decltype(i_tag)::value;
        global_to_lds_16_off<(i % 4) * 1024, i == 0 ? 5 : (i % 4 == 0 ? 1 : 0)>((const void*)(uintptr_t)cb, kfo[i],
                                                                               l + (i / 4) * 4096);
      });
    } else if constexpr (CACHED) {
#pragma unroll
      for (int i = 0; i < K_INSTR; ++i) {
        const int slot = (wis * K_INSTR + i) * 64 + lane, r = slot / KCPR;
        const int key = min(kb * BK + r, last_key);
        const uint64_t base = key < Sc ? kc_base : kn_base;
        global_to_lds_16((const void*)(uintptr_t)(base + (uint64_t)(uint32_t)key * (uint32_t)kstride +
                                                  fill_chunk_prefill<KCPR>(slot) * 16),
                         l + i * 1024);
      }
    } else if ((kb + 1) * BK <= Sk) {
      const char* base = kg + (size_t)kb * BK * kstride;
      // four 1 KiB loads per M0 value, the instruction offset moving both
      // addresses (the lane offsets are stored less it)
      static_for<K_INSTR>([&](auto i_tag) __attribute__((always_inline)) {
        constexpr int i = decltype(i_tag)::value;
        global_to_lds_16_off<(i % 4) * 1024, i == 0 ? 5 : (i % 4 == 0 ? 1 : 0)>(base, kfo[i], l + (i / 4) * 4096);
      });
    } else {
#pragma unroll
      for (int i = 0; i < K_INSTR; ++i) {
        const int slot = (wis * K_INSTR + i) * 64 + lane, r = slot / KCPR;
        const int key = min(kb * BK + r, last_key);
        global_to_lds_16(kg + (size_t)key * kstride + fill_chunk_prefill<KCPR>(slot) * 16,
                         l + i * 1024);
      }
    }
  };
  auto fill_v = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t l = lds0 + buf + wis * V_INSTR * 1024;
    const uint64_t cb = CACHED ? cached_base(kb, vc_base, vn_base, vstride) : 0;
    if (CACHED && cb != 0) {
      static_for<V_INSTR>([&](auto i_tag) __attribute__((always_inline)) {
        constexpr int i = decltype(i_tag)::value;
        global_to_lds_16_off<(i % 4) * 1024, i == 0 ? 5 : (i % 4 == 0 ? 1 : 0)>((const void*)(uintptr_t)cb, vfo[i],
                                                                               l + (i / 4) * 4096);
      });
    } else if constexpr (CACHED) {
#pragma unroll
      for (int i = 0; i < V_INSTR; ++i) {
        const int slot = (wis * V_INSTR + i) * 64 + lane, r = slot / VCPR;
        const int key = min(kb * BK + r, last_key);
        const uint64_t base = key < Sc ? vc_base : vn_base;
        global_to_lds_16((const void*)(uintptr_t)(base + (uint64_t)(uint32_t)key * (uint32_t)vstride +
                                                  fill_chunk_prefill<VCPR>(slot) * 16),
                         l + i * 1024);
      }
    } else if ((kb + 1) * BK <= Sk) {
      const char* base = vg + (size_t)kb * BK * vstride;
      // four 1 KiB loads per M0 value, the instruction offset moving both
      // addresses (the lane offsets are stored less it)
      static_for<V_INSTR>([&](auto i_tag) __attribute__((always_inline)) {
        constexpr int i = decltype(i_tag)::value;
        global_to_lds_16_off<(i % 4) * 1024, i == 0 ? 5 : (i % 4 == 0 ? 1 : 0)>(base, vfo[i], l + (i / 4) * 4096);
      });
    } else {
#pragma unroll
      for (int i = 0; i < V_INSTR; ++i) {
        const int slot = (wis * V_INSTR + i) * 64 + lane, r = slot / VCPR;
        const int key = min(kb * BK + r, last_key);
        global_to_lds_16(vg + (size_t)key * vstride + fill_chunk_prefill<VCPR>(slot) * 16,
                         l + i * 1024);
      }
    }
  };

  // ---- per-lane LDS read offsets -----------------------------------------
  // K fragment (A operand): key row l%32 (+32 per score tile), head-dim slot
  // 2*s + l/32.
  uint32_t koff[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
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
  f32x16_t sa[NTL], sb[NTL];  // score tiles of two consecutive blocks

  // GEMM 1: S^T[key][query] of the block in K buffer KB
  auto qk = [&](auto kb_tag, f32x16_t (&sc)[NTL]) __attribute__((always_inline)) {
    constexpr uint32_t KB = decltype(kb_tag)::value;
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const u32x4_t kf = lds_read_b128(koff[s] + KB + 32 * t * KROW);
        sc[t] = mfma32x32x16<T>(kf, qf[s], sc[t]);
      }
  };

  // Softmax part 1: mask (tail blocks only), block row max, lazy rescale.
  // Returns the subtrahend m of P = 2^(s2*S - m).
  auto softmax_max = [&](int kb, f32x16_t (&sc)[NTL], const u32x4_t (&mv)[BIAS ? NTL * 2 : 1], auto masked_tag)
      __attribute__((always_inline)) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float bmax;
    if constexpr (BIAS) {
      // scores become scale*S + bias (natural-log domain) in place; the block
      // max is taken there and moved to the log2 domain of the running max
      const int lim = MASKED ? (CAUSAL ? min(Sk - 1, qrow + off) : Sk - 1) - (kb * BK + 4 * hl) : 0;
      bmax = -INFINITY;
      u32x2_t mb[NTL * 4];  // mb[4t + c]: the four keys 32t + 8c + 4*hl ..
#pragma unroll
      for (int i = 0; i < NTL * 2; ++i) bias_runs(mv[i], mb[2 * i], mb[2 * i + 1]);
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t w = (r & 2) ? mb[4 * t + (r >> 2)].y : mb[4 * t + (r >> 2)].x;
          float bias;
          if constexpr (T::is_bf16)
            bias = __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
          else
            bias = (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (w >> 16) : (w & 0xffffu)));
          float x = fmaf(sc[t][r], s_nat, bias);
          if constexpr (MASKED) x = (32 * t + 8 * (r >> 2) + (r & 3)) <= lim ? x : -INFINITY;
          sc[t][r] = x;
          bmax = fmaxf(bmax, x);
        }
      bmax *= kLog2e;
    } else if constexpr (MASKED) {
      // register r of tile t holds key kb*BK + 4*hl + 32t + 8(r/4) + r%4; it is
      // visible iff that key <= the row's last visible key
      const int lim = (CAUSAL ? min(Sk - 1, qrow + off) : Sk - 1) - (kb * BK + 4 * hl);
      bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (32 * t + 8 * (r >> 2) + (r & 3)) <= lim ? sc[t][r] * s2 : -INFINITY;
          sc[t][r] = x;
          bmax = fmaxf(bmax, x);
        }
    } else {
      float mx = sc[0][0];
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
      bmax = mx * s2;
    }
    bmax = pair_max(bmax);
    // Lazy rescale: the running max only moves (and O, l are rescaled by
    // 2^(m_old - m_new)) when some row's block max exceeds it by more than
    // kSlack; otherwise the stale max is kept, so P <= 2^kSlack.  The final
    // O / l is unchanged because l accumulates the same P values.
    const float m_new = fmaxf(m_run, bmax);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kSlack)) {
      // rows that have seen no visible key keep m = -inf (masked blocks only)
      // (with a bias, any block: a bias of -inf can remove every key of a row)
      const float m_tgt = MASKED || BIAS ? (m_new == -INFINITY ? 0.f : m_new) : m_new;
      const float alpha = fast_exp2(m_run - m_tgt);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
      m_run = m_new;
    }
    return MASKED || BIAS ? (m_run == -INFINITY ? 0.f : m_run) : m_run;
  };

  // Softmax part 2: P = 2^(s2*S - m) packed to 16 bits as the PV B operand;
  // the row sum is taken over the fp32 values before the packing.
  auto softmax_exp = [&](const f32x16_t (&sc)[NTL], float m_sub, u32x4_t (&pf)[NCH], auto masked_tag)
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0, p1;
        if constexpr (BIAS) {  // scores in the natural-log domain
          p0 = fast_exp2(fmaf(sc[t][r], kLog2e, -m_sub));
          p1 = fast_exp2(fmaf(sc[t][r + 1], kLog2e, -m_sub));
        } else if constexpr (MASKED) {
          p0 = fast_exp2(sc[t][r] - m_sub);
          p1 = fast_exp2(sc[t][r + 1] - m_sub);
        } else {
          p0 = fast_exp2(fmaf(sc[t][r], s2, -m_sub));
          p1 = fast_exp2(fmaf(sc[t][r + 1], s2, -m_sub));
        }
        const uint32_t pk = pack2<T>(p0, p1);
        pf[2 * t + (r >> 3)][(r & 7) >> 1] = pk;
        l_run += p0 + p1;  // row sum over the fp32 values
      }
  };

  // GEMM 2: O^T[dv][query] += V^T P^T from V buffer VB, 16 keys per MFMA
  auto pv = [&](auto vb_tag, const u32x4_t (&pf)[NCH]) __attribute__((always_inline)) {
    constexpr uint32_t VB = decltype(vb_tag)::value;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2_t lo = lds_read_tr16(voff[0][t] + VB + (16 * c) * VROW);
        const u32x2_t hi = lds_read_tr16(voff[1][t] + VB + (16 * c) * VROW);
        const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
        acc[t] = mfma32x32x16<T>(vf, pf[c], acc[t]);
      }
  };

  // One pipeline iteration j (PAR = j & 1, block kb0 + j): the scores of
  // block j are in registers, K(j+1) sits in K buffer 1-PAR and V(j) in V
  // buffer PAR.  It starts the loads of V(j+1) and K(j+2) into the buffers
  // freed by the previous iteration, computes the scores of block j+1, then
  // the softmax and P V of block j.
  auto iteration = [&](int j, auto masked_tag, auto next_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr uint32_t KB_NEXT = PAR ? KBUF0 : KBUF1;   // holds K(j+1)
    constexpr uint32_t KB_FREE = PAR ? KBUF1 : KBUF0;   // receives K(j+2)
    constexpr uint32_t VB_CUR = PAR ? VBUF1 : VBUF0;    // holds V(j)
    constexpr uint32_t VB_FREE = PAR ? VBUF0 : VBUF1;   // receives V(j+1)
    f32x16_t(&s_cur)[NTL] = PAR ? sb : sa;
    f32x16_t(&s_nxt)[NTL] = PAR ? sa : sb;
    wait_vmcnt<0>();  // K(j+1), V(j) (and the bias of block j) have landed
    if constexpr (BIAS) pin_regs(mv);
    // every wave's loads have landed, and every wave is past iteration j-1,
    // whose reads of K(j) and V(j-1) were the last of the buffers refilled here
    __syncthreads();
    if constexpr (NEXT) {
      fill_v(kb0 + j + 1, VB_FREE);
      if (j + 2 < cnt) fill_k(kb0 + j + 2, KB_FREE);
    }
    const float m_sub = softmax_max(kb0 + j, s_cur, mv, masked_tag);
    if constexpr (BIAS && NEXT) load_bias(kb0 + j + 1, mv);
    u32x4_t pf[NCH];
    // Phase fence, then the QK MFMAs of block j+1 interleaved with the
    // exponentials of block j: after each K fragment read and MFMA the wave
    // issues a few independent VALU instructions, which execute while the
    // matrix core works on that MFMA.
    __builtin_amdgcn_sched_barrier(0);
    // the matrix-core part of the block at raised issue priority: the other
    // wave on this SIMD, in its softmax, waits or barrier, yields to it
    __builtin_amdgcn_s_setprio(1);
    if constexpr (NEXT) qk(std::integral_constant<uint32_t, KB_NEXT>{}, s_nxt);
    softmax_exp(s_cur, m_sub, pf, masked_tag);
    if constexpr (NEXT) {
#pragma unroll
      for (int i = 0; i < NTL * D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // twelve VALU
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    pv(std::integral_constant<uint32_t, VB_CUR>{}, pf);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  // Iterations [j0, j1) of one flavour, unrolled by two so that the score
  // tiles visibly alternate (block j in sa for even j, in sb for odd j).
  auto run = [&](int j0, int j1, auto masked_tag, auto next_tag) __attribute__((always_inline)) {
    int j = j0;
    if (j < j1 && (j & 1)) iteration(j++, masked_tag, next_tag, Par1{});
    for (; j + 1 < j1; j += 2) {
      iteration(j, masked_tag, next_tag, Par0{});
      iteration(j + 1, masked_tag, next_tag, Par1{});
    }
    if (j < j1) iteration(j, masked_tag, next_tag, Par0{});
  };

  // ---- K-block pipeline ---------------------------------------------------
  using Unmasked = std::false_type;
  using Masked = std::true_type;
  using Next = std::true_type;
  using Last = std::false_type;
  // Q, K(0), V(0) and K(1) in flight at once (block 0 again when there is no
  // block 1, into a buffer nothing reads); the first scores wait for Q and
  // K(0) only
  fill_k(kb0, KBUF0);
  fill_v(kb0, VBUF0);
  fill_k(kb0 + min(1, cnt - 1), KBUF1);
  load_bias(kb0, mv);  // waited for by the first iteration
  if constexpr (CACHED)
    wait_vmcnt<K_INSTR + V_INSTR>();
  else
    wait_vmcnt_pin<K_INSTR + V_INSTR + ML>(qf);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = row_ok ? qf[s] : u32x4_t{0, 0, 0, 0};
  __syncthreads();
  qk(std::integral_constant<uint32_t, KBUF0>{}, sa);
  const int n_next = cnt - 1;  // iterations that have a next block
  const int j_mask = min(n_unmasked, n_next);
  run(0, j_mask, Unmasked{}, Next{});
  run(j_mask, n_next, Masked{}, Next{});
  // the last block (peeled): masked unless every key of it is visible to
  // every row, in which case the mask is a no-op
  if (n_next & 1)
    iteration(n_next, Masked{}, Last{}, Par1{});
  else
    iteration(n_next, Masked{}, Last{}, Par0{});

  // ---- merge of the key ranges (ranges 1.. -> LDS -> range 0) -------------
  if constexpr (KS > 1) {
    __syncthreads();  // every wave is past its last LDS read
    // per wave of ranges 1..KS-1: NT*16 accumulators + (m, l) per lane, as
    // 16-byte lane-major rows (conflict-free)
    constexpr int XROWS = NT * 4 + 1;
    static_assert((KS - 1) * NWS * XROWS * 1024 <= KS * RANGE_BYTES, "merge area");
    SDPA_LDS f32x4_t* xbase = (SDPA_LDS f32x4_t*)((SDPA_LDS char*)smem) + lane;
    if (kr_i > 0) {
      SDPA_LDS f32x4_t* xb = xbase + ((kr_i - 1) * NWS + wis) * XROWS * 64;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xb[(t * 4 + q4) * 64] = f32x4_t{acc[t][4 * q4], acc[t][4 * q4 + 1], acc[t][4 * q4 + 2], acc[t][4 * q4 + 3]};
      xb[NT * 4 * 64] = f32x4_t{m_run, l_run, 0.f, 0.f};
    }
    __syncthreads();
    if (kr_i > 0) return;
    float mr[KS], lr[KS];
    mr[0] = m_run;
    lr[0] = l_run;
    float mm = m_run;
#pragma unroll
    for (int r = 1; r < KS; ++r) {
      const f32x4_t ml = xbase[((r - 1) * NWS + wis) * XROWS * 64 + NT * 4 * 64];
      mr[r] = ml[0];
      lr[r] = ml[1];
      mm = fmaxf(mm, mr[r]);
    }
    float w[KS];
    l_run = 0.f;
#pragma unroll
    for (int r = 0; r < KS; ++r) {
      w[r] = mr[r] == -INFINITY ? 0.f : fast_exp2(mr[r] - mm);  // empty range: weight 0
      l_run += w[r] * lr[r];
    }
    m_run = mm;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][4 * q4 + e] *= w[0];
#pragma unroll
        for (int r = 1; r < KS; ++r) {
          const f32x4_t o = xbase[((r - 1) * NWS + wis) * XROWS * 64 + (t * 4 + q4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][4 * q4 + e] += w[r] * o[e];
        }
      }
  }

  // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
  u32x4_t runs[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x2_t w2[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = 8 * p + 4 * k;
        w2[k].x = pack2<T>(acc[t][r + 0] * inv, acc[t][r + 1] * inv);
        w2[k].y = pack2<T>(acc[t][r + 2] * inv, acc[t][r + 3] * inv);
      }
      runs[t][p] = pair_runs16(w2[0], w2[1]);
    }
  if (row_ok) {
    elem_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p) *(u32x4_t*)(orow + 32 * t + 16 * p + 8 * hl) = runs[t][p];
    if (a.lse != nullptr && hl == 0)
      a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace sdpa
