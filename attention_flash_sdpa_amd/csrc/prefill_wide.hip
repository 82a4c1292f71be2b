// prefill_wide.hip -- fused SDPA forward mainloop for gfx950 (16-bit inputs),
// 64 query rows per wavefront, one wavefront per SIMD.
//
// The same method as prefill.hip ("Xe SDPA Forward Mainloop -- Key Loops +
// Shapes", sections "mainloop_body(K)" and "softmax() helper"), laid out for
// large problems: each wave owns two 32-row query tiles, so every K and V^T
// fragment read from LDS feeds two MFMAs (one per query tile).  Blocks are 32
// keys, which keeps the score tiles of two blocks in registers.  That halves the LDS instructions per FLOP, which
// otherwise take about as long as the MFMAs themselves (the LDS pipe retires
// one quarter-wave per clock whatever the access width).  With one wave per
// SIMD the whole 512-entry register file is available: the O^T accumulators
// live in AGPRs, leaving room to keep several LDS fragments in flight and to
// overlap the QK MFMAs of block j+1 with the exponentials of block j.
#include <math.h>

#include <type_traits>

#include "sdpa_bounds.h"
#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <class T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_wide_kernel(const PrefillArgs a) {
  constexpr int BK = kWideBlockK;         // 32 keys per block: one key tile
  constexpr int KT = BK / 32;             // key tiles per block
  constexpr int NC = BK / 16;             // 16-key chunks per block (PV k-steps)
  constexpr int NW = kPrefillWaves;
  constexpr int ROWS = kWideRowsPerWave;  // 64 = two 32-row MFMA tiles
  constexpr int KROW = D * 2, VROW = DV * 2;
  constexpr int KCPR = D / 8, VCPR = DV / 8;
  constexpr int KBYTES = BK * KROW, VBYTES = BK * VROW;
  constexpr int K_INSTR = BK * KCPR / 64 / NW;
  constexpr int V_INSTR = BK * VCPR / 64 / NW;
  constexpr int NT = DV / 32;
  constexpr int KS = D / 16;  // k-steps of the QK MFMA
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "block too small for the fill");
  constexpr uint32_t KBUF0 = 0, KBUF1 = KBYTES;
  constexpr uint32_t VBUF0 = 2 * KBYTES, VBUF1 = 2 * KBYTES + VBYTES;

  __shared__ __attribute__((aligned(1024))) char smem[2 * KBYTES + 2 * VBYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem;

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // ---- work decode (as the 32-row kernel, with 64-row wave tiles) ---------
  int wg = remap_xcd(blockIdx.x, a.num_groups);
  int qt = wg % a.q_tiles;
  int rest = wg / a.q_tiles;
  const int hg = rest % a.head_groups;
  rest /= a.head_groups;
  const int g = rest % a.head_kv;
  const int b = rest / a.head_kv;
  if (CAUSAL) qt = a.q_tiles - 1 - qt;
  const int hp_i = wave % a.heads_per_group;
  const int qp_i = wave / a.heads_per_group;
  const bool head_ok = hg * a.heads_per_group + hp_i < a.group;
  const int h = g * a.group + min(hg * a.heads_per_group + hp_i, a.group - 1);
  const int Sq = a.q_len, Sk = a.kv_len, off = Sk - Sq;
  const int wg_row0 = qt * (ROWS * a.qtiles_per_group);
  const int row0 = wg_row0 + ROWS * qp_i;
  const int wg_row_end = min(wg_row0 + ROWS * a.qtiles_per_group, Sq);
  const KBlockRange kr = kblock_range(wg_row0, wg_row_end, Sq, Sk, BK, CAUSAL);
  const int n_blocks = kr.n_blocks;
  const int n_full = kr.n_full;

  int qrow[2];
  bool row_ok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    qrow[u] = row0 + 32 * u + l32;
    row_ok[u] = head_ok && qrow[u] < Sq;
  }
  uint16_t* __restrict__ optr = (uint16_t*)a.o;

  if (n_blocks == 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (row_ok[u]) {
        uint16_t* orow = optr + ((size_t)(b * Sq + qrow[u]) * a.head_q + h) * DV;
        for (int c = hl * (DV / 2); c < (hl + 1) * (DV / 2); c += 8) *(u32x4_t*)(orow + c) = u32x4_t{0, 0, 0, 0};
        if (a.lse != nullptr && hl == 0) a.lse[((size_t)b * a.head_q + h) * Sq + qrow[u]] = -INFINITY;
      }
    return;
  }

  // ---- Q fragments of both query tiles -----------------------------------
  u32x4_t qf[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint16_t* qptr =
        (const uint16_t*)a.q + ((size_t)(b * Sq + min(qrow[u], Sq - 1)) * a.head_q + h) * D + 8 * hl;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *(const u32x4_t*)(qptr + 16 * s);
      qf[u][s] = row_ok[u] ? v : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- direct global -> LDS fills (same layout as the 32-row kernel) -------
  const char* kg = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * (D * 2);
  const char* vg = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * (DV * 2);
  const int kstride = a.head_kv * D * 2;
  const int vstride = a.head_kv * DV * 2;
  uint32_t kfo[K_INSTR], vfo[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int slot = (wave * K_INSTR + i) * 64 + lane, r = slot / KCPR;
    kfo[i] = r * kstride + (((slot % KCPR) ^ (int)swz_prefill<KCPR>(r)) * 16) - (i % 4) * 1024;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = (wave * V_INSTR + i) * 64 + lane, r = slot / VCPR;
    vfo[i] = r * vstride + (((slot % VCPR) ^ (int)swz_prefill<VCPR>(r)) * 16) - (i % 4) * 1024;
  }
  const int last_key = Sk - 1;
  auto fill_k = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t l = lds0 + buf + wave * K_INSTR * 1024;
    if ((kb + 1) * BK <= Sk) {
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
        const int slot = (wave * K_INSTR + i) * 64 + lane, r = slot / KCPR;
        const int key = min(kb * BK + r, last_key);
        global_to_lds_16(kg + (size_t)key * kstride + (((slot % KCPR) ^ (int)swz_prefill<KCPR>(r)) * 16),
                         l + i * 1024);
      }
    }
  };
  auto fill_v = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t l = lds0 + buf + wave * V_INSTR * 1024;
    if ((kb + 1) * BK <= Sk) {
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
        const int slot = (wave * V_INSTR + i) * 64 + lane, r = slot / VCPR;
        const int key = min(kb * BK + r, last_key);
        global_to_lds_16(vg + (size_t)key * vstride + (((slot % VCPR) ^ (int)swz_prefill<VCPR>(r)) * 16),
                         l + i * 1024);
      }
    }
  };

  // ---- per-lane LDS read offsets (as the 32-row kernel) --------------------
  uint32_t koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    koff[s] = lds0 + l32 * KROW + ((((2 * s + hl)) ^ (int)swz_prefill<KCPR>(l32)) << 4);
  uint32_t voff[2][NT];
  {
    const int gq = lane >> 4, s = lane & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 8 * hf + 4 * (gq >> 1) + (s >> 2);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = 32 * t + 16 * (gq & 1) + 4 * (s & 3);
        voff[hf][t] = lds0 + r * VROW + ((((col >> 3) ^ (int)swz_prefill<VCPR>(r))) << 4) + ((col & 7) << 1);
      }
    }
  }

  // ---- state ----------------------------------------------------------------
  f32x16_t acc[2][NT];  // [query tile][value tile]
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][t][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float s2 = a.s2;
  f32x16_t sa[KT][2], sb[KT][2];  // [key tile][query tile] scores of two blocks

  // GEMM 1: each K fragment (one key tile, one k-step) feeds both query tiles
  auto qk = [&](auto kb_tag, f32x16_t (&sc)[KT][2]) __attribute__((always_inline)) {
    constexpr uint32_t KB = decltype(kb_tag)::value;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][u][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const u32x4_t kf = lds_read_b128(koff[s] + KB + 32 * kt * KROW);
        sc[kt][0] = mfma32x32x16<T>(kf, qf[0][s], sc[kt][0]);
        sc[kt][1] = mfma32x32x16<T>(kf, qf[1][s], sc[kt][1]);
      }
  };

  // mask (tail blocks), block row max of query tile u in the log2 domain
  auto block_max = [&](int kb, f32x16_t (&sc)[KT][2], int u, auto masked_tag) __attribute__((always_inline)) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float bmax;
    if constexpr (MASKED) {
      const int lim = (CAUSAL ? min(Sk - 1, qrow[u] + off) : Sk - 1) - (kb * BK + 4 * hl);
      bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (32 * kt + 8 * (r >> 2) + (r & 3)) <= lim ? sc[kt][u][r] * s2 : -INFINITY;
          sc[kt][u][r] = x;
          bmax = fmaxf(bmax, x);
        }
    } else {
      float mx = sc[0][u][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][u][r]);
      bmax = mx * s2;
    }
    return pair_max(bmax);
  };

  // row maxima of both query tiles, one lazy-rescale decision for the wave
  auto softmax_max = [&](int kb, f32x16_t (&sc)[KT][2], float (&m_sub)[2], auto masked_tag)
                         __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float m_new[2];
    bool need = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      m_new[u] = fmaxf(m_run[u], block_max(kb, sc, u, masked_tag));
      need |= m_new[u] > m_run[u] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float m_tgt = MASKED ? (m_new[u] == -INFINITY ? 0.f : m_new[u]) : m_new[u];
        const float alpha = fast_exp2(m_run[u] - m_tgt);
        l_run[u] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[u][t][r] *= alpha;
        m_run[u] = m_new[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) m_sub[u] = MASKED ? (m_run[u] == -INFINITY ? 0.f : m_run[u]) : m_run[u];
  };

  auto softmax_exp = [&](const f32x16_t (&sc)[KT][2], const float (&m_sub)[2], u32x4_t (&pf)[2][NC],
                         auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0, p1;
          if constexpr (MASKED) {
            p0 = fast_exp2(sc[kt][u][r] - m_sub[u]);
            p1 = fast_exp2(sc[kt][u][r + 1] - m_sub[u]);
          } else {
            p0 = fast_exp2(fmaf(sc[kt][u][r], s2, -m_sub[u]));
            p1 = fast_exp2(fmaf(sc[kt][u][r + 1], s2, -m_sub[u]));
          }
          const uint32_t pk = pack2<T>(p0, p1);
          pf[u][2 * kt + (r >> 3)][(r & 7) >> 1] = pk;
          l_run[u] = add_pair<T>(pk, l_run[u]);
        }
  };

  // GEMM 2: each V^T fragment feeds both query tiles
  auto pv = [&](auto vb_tag, const u32x4_t (&pf)[2][NC]) __attribute__((always_inline)) {
    constexpr uint32_t VB = decltype(vb_tag)::value;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2_t lo = lds_read_tr16(voff[0][t] + VB + (16 * c) * VROW);
        const u32x2_t hi = lds_read_tr16(voff[1][t] + VB + (16 * c) * VROW);
        const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
        acc[0][t] = mfma32x32x16<T>(vf, pf[0][c], acc[0][t]);
        acc[1][t] = mfma32x32x16<T>(vf, pf[1][c], acc[1][t]);
      }
  };

  // Issue order inside the QK + exp phase: four K fragment reads ahead, then
  // per fragment its two MFMAs, a slice of the exponential work (which runs
  // while the matrix core is busy) and the read of the fragment four ahead.
  auto schedule_qk_exp = [&]() __attribute__((always_inline)) {
    constexpr int NF = KT * KS;  // K fragments per block
    constexpr int AHEAD = 4;
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
      if (i + AHEAD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // PV phase: four V^T fragments (eight tr16 reads) ahead of their MFMAs
  auto schedule_pv = [&]() __attribute__((always_inline)) {
    constexpr int NF = NC * NT;  // V^T fragments per block
    constexpr int AHEAD = 4;
#pragma unroll
    for (int i = 0; i < 2 * AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i + AHEAD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  auto iteration = [&](int j, auto masked_tag, auto next_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr uint32_t KB_NEXT = PAR ? KBUF0 : KBUF1;
    constexpr uint32_t KB_FREE = PAR ? KBUF1 : KBUF0;
    constexpr uint32_t VB_CUR = PAR ? VBUF1 : VBUF0;
    constexpr uint32_t VB_FREE = PAR ? VBUF0 : VBUF1;
    f32x16_t(&s_cur)[KT][2] = PAR ? sb : sa;
    f32x16_t(&s_nxt)[KT][2] = PAR ? sa : sb;
    if constexpr (NEXT) {
      fill_v(j + 1, VB_FREE);
      if (j + 2 < n_blocks) {
        fill_k(j + 2, KB_FREE);
        wait_vmcnt<K_INSTR + V_INSTR>();
      } else {
        wait_vmcnt<V_INSTR>();
      }
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    float m_sub[2];
    softmax_max(j, s_cur, m_sub, masked_tag);
    u32x4_t pf[2][NC];
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) qk(std::integral_constant<uint32_t, KB_NEXT>{}, s_nxt);
    softmax_exp(s_cur, m_sub, pf, masked_tag);
    if constexpr (NEXT) schedule_qk_exp();
    __builtin_amdgcn_sched_barrier(0);
    pv(std::integral_constant<uint32_t, VB_CUR>{}, pf);
    schedule_pv();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) __syncthreads();
  };

  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  auto run = [&](int j0, int j1, auto masked_tag, auto next_tag) __attribute__((always_inline)) {
    int j = j0;
    if (j < j1 && (j & 1)) iteration(j++, masked_tag, next_tag, Par1{});
    for (; j + 1 < j1; j += 2) {
      iteration(j, masked_tag, next_tag, Par0{});
      iteration(j + 1, masked_tag, next_tag, Par1{});
    }
    if (j < j1) iteration(j, masked_tag, next_tag, Par0{});
  };

  using Unmasked = std::false_type;
  using Masked = std::true_type;
  using Next = std::true_type;
  using Last = std::false_type;
  fill_k(0, KBUF0);
  fill_v(0, VBUF0);
  if (n_blocks > 1) {
    fill_k(1, KBUF1);
    wait_vmcnt<K_INSTR + V_INSTR>();
  } else {
    wait_vmcnt<V_INSTR>();
  }
  __syncthreads();
  qk(std::integral_constant<uint32_t, KBUF0>{}, sa);
  __syncthreads();
  const int n_next = n_blocks - 1;
  const int j_mask = min(n_full, n_next);
  run(0, j_mask, Unmasked{}, Next{});
  run(j_mask, n_next, Masked{}, Next{});
  if (n_next & 1)
    iteration(n_next, Masked{}, Last{}, Par1{});
  else
    iteration(n_next, Masked{}, Last{}, Par0{});

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float l_tot = pair_sum(l_run[u]);
    const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
    if (row_ok[u]) {
      uint16_t* orow = optr + ((size_t)(b * Sq + qrow[u]) * a.head_q + h) * DV;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = 32 * t + 8 * q4 + 4 * hl;
          u32x2_t w;
          w.x = pack2<T>(acc[u][t][4 * q4 + 0] * inv, acc[u][t][4 * q4 + 1] * inv);
          w.y = pack2<T>(acc[u][t][4 * q4 + 2] * inv, acc[u][t][4 * q4 + 3] * inv);
          *(u32x2_t*)(orow + col) = w;
        }
      if (a.lse != nullptr && hl == 0)
        a.lse[((size_t)b * a.head_q + h) * Sq + qrow[u]] =
            l_tot > 0.f ? (m_run[u] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <class T, int D>
static int launch_wide_t(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * kPrefillWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_wide_kernel<T, D, D, true>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<T, D, D, false>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_prefill_wide(const PrefillArgs& a, const sdpa_plan_t& plan, int causal, ihipStream_t* stream) {
  switch (plan.kernel) {
    case kWideF16D64: return launch_wide_t<F16, 64>(a, causal, stream);
    case kWideBf16D64: return launch_wide_t<Bf16, 64>(a, causal, stream);
    case kWideF16D128: return launch_wide_t<F16, 128>(a, causal, stream);
    case kWideBf16D128: return launch_wide_t<Bf16, 128>(a, causal, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace sdpa
