// prefill_fp8.hip -- fused SDPA forward for OCP fp8 e4m3 inputs with
// d_qk = 192, d_v = 128 (the MLA-shaped prefill), bf16 output.
//
// Same mainloop as the 16-bit kernel ("Xe SDPA Forward Mainloop -- Key Loops +
// Shapes", sections "mainloop_body(K)" and "softmax() helper"): each wave owns
// 32 query rows, computes S^T = K Q^T, runs the online softmax in fp32 with
// exp2 and the scale folded with log2(e), and accumulates O^T += V^T P^T in
// fp32.  What changes for fp8:
//
//  * QK uses the 32x32x64 fp8 MFMA (three k-steps over 192 head dims, as in
//    the MLA op of the Modular MAX page, which streams K through 32x32x64 fp8
//    fragments).  The per-tensor dequantisation factors of Q and K are folded
//    into the softmax scale; the one of V is applied in the epilogue.
//  * P V runs in bf16: V fragments come out of LDS transposed with
//    ds_read_b64_tr_b8 (eight keys of one value column per lane, the 8-bit
//    transposed read the same page uses for its V fragments) and are widened
//    exactly to bf16; P is rounded to bf16 (relative error <= 2^-9 instead of
//    the 2^-4 of fp8, which would put short causal rows near the accuracy
//    bound), and the row sum is taken over those rounded values.
//  * K rows are 192 bytes, so each K block is kept in LDS as a 128-byte part
//    (dims 0..127) and a 64-byte part (dims 128..191), each with a
//    power-of-two swizzle that keeps the fragment reads free of bank
//    conflicts.
#include <math.h>

#include <type_traits>

#include "sdpa_bounds.h"
#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(const PrefillArgs a) {
  constexpr int D = 192, DV = 128;
  constexpr int BK = kPrefillBlockK;  // 64 keys per block
  constexpr int NW = kPrefillWaves;
  constexpr int KAROW = 128, KBROW = 64, VROW = 128;         // LDS bytes per key row
  constexpr int KABYTES = BK * KAROW, KBBYTES = BK * KBROW, VBYTES = BK * VROW;
  constexpr int STAGE = KABYTES + KBBYTES + VBYTES;          // 20 KiB
  constexpr int KA_INSTR = KABYTES / 1024 / NW;              // 2 per wave
  constexpr int KB_INSTR = KBBYTES / 1024 / NW;              // 1 per wave
  constexpr int V_INSTR = VBYTES / 1024 / NW;                // 2 per wave
  constexpr int NT = DV / 32;                                // O^T accumulator tiles
  static_assert(KA_INSTR * NW * 1024 == KABYTES && KB_INSTR * NW * 1024 == KBBYTES &&
                    V_INSTR * NW * 1024 == VBYTES,
                "block split into whole 1 KiB loads per wave");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem;

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // ---- work decode (same mapping as the 16-bit kernel) --------------------
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
  const int wg_row0 = qt * (kRowsPerWave * a.qtiles_per_group);
  const int row0 = wg_row0 + kRowsPerWave * qp_i;
  const int wg_row_end = min(wg_row0 + kRowsPerWave * a.qtiles_per_group, Sq);
  const KBlockRange kr = kblock_range(wg_row0, wg_row_end, Sq, Sk, BK, CAUSAL);
  const int n_blocks = kr.n_blocks;
  const int n_full = kr.n_full;

  const int qrow = row0 + l32;
  const bool row_ok = head_ok && qrow < Sq;
  uint16_t* __restrict__ optr = (uint16_t*)a.o;

  if (n_blocks == 0) {
    if (row_ok) {
      uint16_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
      for (int c = hl * (DV / 2); c < (hl + 1) * (DV / 2); c += 8) *(u32x4_t*)(orow + c) = u32x4_t{0, 0, 0, 0};
      if (a.lse != nullptr && hl == 0) a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = -INFINITY;
    }
    return;
  }

  // ---- Q fragments: B operand of the fp8 MFMA, 32 bytes per k-step --------
  i32x8_t qf[3];
  {
    const uint8_t* qptr = (const uint8_t*)a.q + ((size_t)(b * Sq + min(qrow, Sq - 1)) * a.head_q + h) * D + 32 * hl;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const u32x4_t lo = *(const u32x4_t*)(qptr + 64 * s);
      const u32x4_t hi = *(const u32x4_t*)(qptr + 64 * s + 16);
      i32x8_t v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      qf[s] = row_ok ? v : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // ---- direct global -> LDS fill ------------------------------------------
  const char* kg = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * D;
  const char* vg = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * DV;
  const int kstride = a.head_kv * D, vstride = a.head_kv * DV;  // bytes between keys
  int ka_row[KA_INSTR], ka_col[KA_INSTR], kb_row[KB_INSTR], kb_col[KB_INSTR], v_row[V_INSTR], v_col[V_INSTR];
#pragma unroll
  for (int i = 0; i < KA_INSTR; ++i) {
    const int slot = (wave * KA_INSTR + i) * 64 + lane, r = slot / 8;
    ka_row[i] = r;
    ka_col[i] = ((slot % 8) ^ (int)swz_prefill<8>(r)) * 16;
  }
#pragma unroll
  for (int i = 0; i < KB_INSTR; ++i) {
    const int slot = (wave * KB_INSTR + i) * 64 + lane, r = slot / 4;
    kb_row[i] = r;
    kb_col[i] = KAROW + ((slot % 4) ^ (int)swz_quarter(r)) * 16;  // dims 128.. of the row
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = (wave * V_INSTR + i) * 64 + lane, r = slot / 8;
    v_row[i] = r;
    v_col[i] = ((slot % 8) ^ (int)swz_prefill<8>(r)) * 16;
  }
  const int last_key = Sk - 1;
  auto issue_fill = [&](int kb, int stage) __attribute__((always_inline)) {
    const uint32_t base = lds0 + stage * STAGE;
#pragma unroll
    for (int i = 0; i < KA_INSTR; ++i)
      global_to_lds_16(kg + (size_t)min(kb * BK + ka_row[i], last_key) * kstride + ka_col[i],
                       base + (wave * KA_INSTR + i) * 1024);
#pragma unroll
    for (int i = 0; i < KB_INSTR; ++i)
      global_to_lds_16(kg + (size_t)min(kb * BK + kb_row[i], last_key) * kstride + kb_col[i],
                       base + KABYTES + (wave * KB_INSTR + i) * 1024);
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      global_to_lds_16(vg + (size_t)min(kb * BK + v_row[i], last_key) * vstride + v_col[i],
                       base + KABYTES + KBBYTES + (wave * V_INSTR + i) * 1024);
  };

  // ---- per-lane LDS read offsets -----------------------------------------
  // K fragment (A operand of 32x32x64): key row l%32 (+32 for the second
  // score tile), 32 bytes at dims 64s + 32*(l/32): chunks 2*(l/32) (+1) of
  // part A for s = 0, 1 (+4 for s = 1) and of part B for s = 2.
  uint32_t ka_off[2][2], kb_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      ka_off[s][c] = l32 * KAROW + (((4 * s + 2 * hl + c) ^ (int)swz_prefill<8>(l32)) << 4);
#pragma unroll
  for (int c = 0; c < 2; ++c) kb_off[c] = KABYTES + l32 * KBROW + (((2 * hl + c) ^ (int)swz_quarter(l32)) << 4);
  // V^T fragment (A operand of the bf16 32x32x16 MFMA) via ds_read_b64_tr_b8:
  // lane (group gq = l/16, s = l%16) addresses key row 8*(r/4) + 4*(gq/2) +
  // r%4 with r = s/2 (+16 per key chunk) and value bytes 32t + 16*(gq%2) +
  // 8*(s%2); its group partner lanes then hold 8 keys of one value column.
  uint32_t v_off[NT];
  {
    const int gq = lane >> 4, s = lane & 15;
    const int r = s >> 1;
    const int row = 8 * (r >> 2) + 4 * (gq >> 1) + (r & 3);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 32 * t + 16 * (gq & 1) + 8 * (s & 1);
      v_off[t] = KABYTES + KBBYTES + row * VROW + ((((col >> 4) ^ (int)swz_prefill<8>(row))) << 4) + (col & 15);
    }
  }

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float s2 = a.s2;

  auto block = [&](int kb, int stage, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint32_t base = lds0 + stage * STAGE;

    // GEMM 1 (fp8): S^T[key][query], three k-steps of 64 head dims
    f32x16_t sc[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[0][r] = 0.f;
      sc[1][r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        u32x4_t x0, x1;
        if (s < 2) {
          x0 = lds_read_b128(base + ka_off[s][0] + 32 * t * KAROW);
          x1 = lds_read_b128(base + ka_off[s][1] + 32 * t * KAROW);
        } else {
          x0 = lds_read_b128(base + kb_off[0] + 32 * t * KBROW);
          x1 = lds_read_b128(base + kb_off[1] + 32 * t * KBROW);
        }
        const i32x8_t kf = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sc[t] = mfma32x32x64_fp8(kf, qf[s], sc[t]);
      }
    }

    float bmax;
    if constexpr (MASKED) {
      const int lim = (CAUSAL ? min(Sk - 1, qrow + off) : Sk - 1) - (kb * BK + 4 * hl);
      bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (32 * t + 8 * (r >> 2) + (r & 3)) <= lim ? sc[t][r] * s2 : -INFINITY;
          sc[t][r] = x;
          bmax = fmaxf(bmax, x);
        }
    } else {
      float mx = sc[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
      bmax = mx * s2;
    }
    bmax = pair_max(bmax);
    const float m_new = fmaxf(m_run, bmax);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kSlack)) {
      const float m_tgt = MASKED ? (m_new == -INFINITY ? 0.f : m_new) : m_new;
      const float alpha = fast_exp2(m_run - m_tgt);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
      m_run = m_new;
    }
    const float m_sub = MASKED ? (m_run == -INFINITY ? 0.f : m_run) : m_run;

    u32x4_t pf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0, p1;
        if constexpr (MASKED) {
          p0 = fast_exp2(sc[t][r] - m_sub);
          p1 = fast_exp2(sc[t][r + 1] - m_sub);
        } else {
          p0 = fast_exp2(fmaf(sc[t][r], s2, -m_sub));
          p1 = fast_exp2(fmaf(sc[t][r + 1], s2, -m_sub));
        }
        const uint32_t pk = pack2<Bf16>(p0, p1);
        pf[2 * t + (r >> 3)][(r & 7) >> 1] = pk;
        l_run = add_pair<Bf16>(pk, l_run);
      }

    // GEMM 2 (bf16): O^T += V^T P^T, V widened from fp8 after the transposed read
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2_t v8 = lds_read_tr8(base + v_off[t] + (16 * c) * VROW);
        const u32x2_t lo = fp8x4_to_bf16x4(v8.x), hi = fp8x4_to_bf16x4(v8.y);
        const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
        acc[t] = mfma32x32x16<Bf16>(vf, pf[c], acc[t]);
      }
  };

  using Unmasked = std::false_type;
  using Masked = std::true_type;
  constexpr int FILL = KA_INSTR + KB_INSTR + V_INSTR;

  issue_fill(0, 0);
  int kb = 0;
  const int n_pref = n_blocks - 1;
  for (; kb < min(n_full, n_pref); ++kb) {
    issue_fill(kb + 1, (kb + 1) & 1);
    wait_vmcnt<FILL>();
    __syncthreads();
    block(kb, kb & 1, Unmasked{});
    __syncthreads();
  }
  for (; kb < n_pref; ++kb) {
    issue_fill(kb + 1, (kb + 1) & 1);
    wait_vmcnt<FILL>();
    __syncthreads();
    block(kb, kb & 1, Masked{});
    __syncthreads();
  }
  wait_vmcnt<0>();
  __syncthreads();
  block(kb, kb & 1, Masked{});

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
  if (row_ok) {
    uint16_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = 32 * t + 8 * q4 + 4 * hl;
        u32x2_t w;
        w.x = pack2<Bf16>(acc[t][4 * q4 + 0] * inv, acc[t][4 * q4 + 1] * inv);
        w.y = pack2<Bf16>(acc[t][4 * q4 + 2] * inv, acc[t][4 * q4 + 3] * inv);
        *(u32x2_t*)(orow + col) = w;
      }
    if (a.lse != nullptr && hl == 0)
      a.lse[((size_t)b * a.head_q + h) * Sq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

int launch_prefill_fp8(const PrefillArgs& a, int causal, ihipStream_t* stream) {
  dim3 grid(a.num_groups), block(64 * kPrefillWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_fp8_kernel<true>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_fp8_kernel<false>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace sdpa
