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
//  * P V runs at the fp8 rate on the blocks every row of the workgroup sees
//    whole: P is rounded to e4m3 (relative error <= 2^-4 per value) and meets
//    the V^T fragments as they come out of LDS, 32 keys per lane from four
//    ds_read_b64_tr_b8 reads (eight keys of one value column each, the 8-bit
//    transposed read the same page uses for its V fragments), in one
//    32x32x64 fp8 MFMA per value tile and block; the row sum is taken over
//    the unrounded fp32 P.  Masked blocks (the causal diagonal, the ragged
//    tail, the last block) run P V in bf16 instead, V widened exactly from
//    fp8 and P rounded to bf16 (relative error <= 2^-9), so rows with few
//    visible keys, whose output is an average of few P values, keep the
//    finer rounding.  The row sum is taken over the fp32 P in both cases.
//  * K rows are 192 bytes, so each K block is kept in LDS as a 128-byte part
//    (dims 0..127) and a 64-byte part (dims 128..191), each with a
//    power-of-two swizzle that keeps the fragment reads free of bank
//    conflicts.
//  * Software pipeline as in the two-waves-per-SIMD 16-bit kernel: iteration
//    j loads V(j+1) and K(j+2) into separate double buffers, issues the QK
//    MFMAs of block j+1 interleaved with the exponentials of block j, then
//    the P V MFMAs of block j; two waves per SIMD hide the rest.
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
  static_assert(KAROW == 128 && KBROW == 64 && VROW == 128, "row sizes of fp8_k*_read / fp8_vt_read");
  constexpr int KBYTES = KABYTES + KBBYTES;                  // 12 KiB per K block
  constexpr int KA_INSTR = KABYTES / 1024 / NW;              // 2 per wave
  constexpr int KB_INSTR = KBBYTES / 1024 / NW;              // 1 per wave
  constexpr int K_INSTR = KA_INSTR + KB_INSTR;
  constexpr int V_INSTR = VBYTES / 1024 / NW;                // 2 per wave
  constexpr int NT = DV / 32;                                // O^T accumulator tiles
  static_assert(KA_INSTR * NW * 1024 == KABYTES && KB_INSTR * NW * 1024 == KBBYTES &&
                    V_INSTR * NW * 1024 == VBYTES,
                "block split into whole 1 KiB loads per wave");
  // LDS: K buffers 0/1 (part A then part B), then V buffers 0/1
  constexpr uint32_t KBUF0 = 0, KBUF1 = KBYTES;
  constexpr uint32_t VBUF0 = 2 * KBYTES, VBUF1 = 2 * KBYTES + VBYTES;

  __shared__ __attribute__((aligned(1024))) char smem[2 * KBYTES + 2 * VBYTES];
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

  // ---- direct global -> LDS fills (rows past the last key re-read it) -----
  const char* kg = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * D;
  const char* vg = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * DV;
  const int kstride = a.head_kv * D, vstride = a.head_kv * DV;  // bytes between keys
  int ka_row[KA_INSTR], ka_col[KA_INSTR], kb_row[KB_INSTR], kb_col[KB_INSTR], v_row[V_INSTR], v_col[V_INSTR];
#pragma unroll
  for (int i = 0; i < KA_INSTR; ++i) {
    const int slot = (wave * KA_INSTR + i) * 64 + lane, r = slot / 8;
    ka_row[i] = r;
    ka_col[i] = fill_chunk_prefill<8>(slot) * 16;
  }
#pragma unroll
  for (int i = 0; i < KB_INSTR; ++i) {
    const int slot = (wave * KB_INSTR + i) * 64 + lane, r = slot / 4;
    kb_row[i] = r;
    kb_col[i] = KAROW + fill_chunk_quarter(slot) * 16;  // dims 128.. of the row
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = (wave * V_INSTR + i) * 64 + lane, r = slot / 8;
    v_row[i] = r;
    v_col[i] = fill_chunk_prefill<8>(slot) * 16;
  }
  const int last_key = Sk - 1;
  auto fill_k = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t base = lds0 + buf;
#pragma unroll
    for (int i = 0; i < KA_INSTR; ++i)
      global_to_lds_16(kg + (size_t)min(kb * BK + ka_row[i], last_key) * kstride + ka_col[i],
                       base + (wave * KA_INSTR + i) * 1024);
#pragma unroll
    for (int i = 0; i < KB_INSTR; ++i)
      global_to_lds_16(kg + (size_t)min(kb * BK + kb_row[i], last_key) * kstride + kb_col[i],
                       base + KABYTES + (wave * KB_INSTR + i) * 1024);
  };
  auto fill_v = [&](int kb, uint32_t buf) __attribute__((always_inline)) {
    const uint32_t base = lds0 + buf;
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      global_to_lds_16(vg + (size_t)min(kb * BK + v_row[i], last_key) * vstride + v_col[i],
                       base + (wave * V_INSTR + i) * 1024);
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
      ka_off[s][c] = lds0 + fp8_ka_read(lane, s, c);
#pragma unroll
  for (int c = 0; c < 2; ++c)
    kb_off[c] = lds0 + KABYTES + fp8_kb_read(lane, c);
  // V^T fragment (A operand of the bf16 32x32x16 MFMA) via ds_read_b64_tr_b8:
  // lane (group gq = l/16, s = l%16) addresses key row 8*(r/4) + 4*(gq/2) +
  // r%4 with r = s/2 (+16 per key chunk) and value bytes 32t + 16*(gq%2) +
  // 8*(s%2); its group partner lanes then hold 8 keys of one value column.
  uint32_t v_off[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) v_off[t] = lds0 + fp8_vt_read(lane, t);

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float s2 = a.s2;
  f32x16_t sa[2], sb[2];  // score tiles of two consecutive blocks

  // GEMM 1 (fp8): S^T[key][query] of the block in K buffer KB, three k-steps
  // of 64 head dims per 32-key score tile
  auto qk = [&](auto kb_tag, f32x16_t (&sc)[2]) __attribute__((always_inline)) {
    constexpr uint32_t KB = decltype(kb_tag)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[0][r] = 0.f;
      sc[1][r] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4_t x0, x1;
        if (s < 2) {
          x0 = lds_read_b128(ka_off[s][0] + KB + 32 * t * KAROW);
          x1 = lds_read_b128(ka_off[s][1] + KB + 32 * t * KAROW);
        } else {
          x0 = lds_read_b128(kb_off[0] + KB + 32 * t * KBROW);
          x1 = lds_read_b128(kb_off[1] + KB + 32 * t * KBROW);
        }
        const i32x8_t kf = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sc[t] = mfma32x32x64_fp8(kf, qf[s], sc[t]);
      }
  };

  // Softmax part 1: mask (tail blocks only), block row max, lazy rescale
  // (the running max only moves when it grows by more than kSlack, so
  // P <= 2^kSlack; O / l is unchanged because l sums the same P values).
  auto softmax_max = [&](int kb, f32x16_t (&sc)[2], auto masked_tag) __attribute__((always_inline)) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float bmax;
    if constexpr (MASKED) {
      // register r of tile t holds key kb*BK + 4*hl + 32t + 8(r/4) + r%4
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
    return MASKED ? (m_run == -INFINITY ? 0.f : m_run) : m_run;
  };

  // Softmax part 2: P = 2^(s2*S - m), its row sum taken over the fp32 values.
  // Masked blocks: rounded to bf16, four dwords per 16-key chunk c (the B
  // operand of the bf16 P V).  Unmasked blocks: rounded to e4m3, eight dwords
  // for the 64 keys of the block (the B operand of the fp8 P V): dword
  // 4t + r/4 holds registers r..r+3 (r % 4 == 0) of score tile t, i.e. bytes
  // 4(r/4%2).. of chunk 2t + r/8, the key order of the transposed V reads.
  auto softmax_exp = [&](const f32x16_t (&sc)[2], float m_sub, u32x4_t (&pf)[4], i32x8_t& pf8, auto masked_tag)
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (MASKED) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(sc[t][r] - m_sub);
          const float p1 = fast_exp2(sc[t][r + 1] - m_sub);
          pf[2 * t + (r >> 3)][(r & 7) >> 1] = pack2<Bf16>(p0, p1);
          l_run += p0 + p1;
        }
    } else {
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = fast_exp2(fmaf(sc[t][r], s2, -m_sub));
          const float p1 = fast_exp2(fmaf(sc[t][r + 1], s2, -m_sub));
          const float p2 = fast_exp2(fmaf(sc[t][r + 2], s2, -m_sub));
          const float p3 = fast_exp2(fmaf(sc[t][r + 3], s2, -m_sub));
          const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          pf8[4 * t + r / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
          la += p0 + p1;
          lb += p2 + p3;
        }
      l_run += la + lb;
    }
  };

  // GEMM 2, masked blocks (bf16): O^T += V^T P^T from V buffer VB, V widened
  // from fp8 after the transposed read
  auto pv = [&](auto vb_tag, const u32x4_t (&pf)[4]) __attribute__((always_inline)) {
    constexpr uint32_t VB = decltype(vb_tag)::value;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2_t v8 = lds_read_tr8(v_off[t] + VB + (16 * c) * VROW);
        const u32x2_t lo = fp8x4_to_bf16x4(v8.x), hi = fp8x4_to_bf16x4(v8.y);
        const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
        acc[t] = mfma32x32x16<Bf16>(vf, pf[c], acc[t]);
      }
  };
  // GEMM 2, unmasked blocks (fp8): one 32x32x64 MFMA per value tile over the
  // whole block; the V^T fragment is the four transposed reads of chunks
  // 0..3 (eight keys each, in the byte order of P's packing above)
  auto pv_fp8 = [&](auto vb_tag, const i32x8_t& pf8) __attribute__((always_inline)) {
    constexpr uint32_t VB = decltype(vb_tag)::value;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      i32x8_t vf;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2_t v8 = lds_read_tr8(v_off[t] + VB + (16 * c) * VROW);
        vf[2 * c] = (int)v8.x;
        vf[2 * c + 1] = (int)v8.y;
      }
      acc[t] = mfma32x32x64_fp8(vf, pf8, acc[t]);
    }
  };

  // One pipeline iteration j (PAR = j & 1): the scores of block j are in
  // registers, K(j+1) sits in K buffer 1-PAR and V(j) in V buffer PAR.  It
  // starts the loads of V(j+1) and K(j+2) into the buffers freed by the
  // previous iteration, computes the scores of block j+1 interleaved with the
  // exponentials of block j, then the P V of block j.
  auto iteration = [&](int j, auto masked_tag, auto next_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr uint32_t KB_NEXT = PAR ? KBUF0 : KBUF1;   // holds K(j+1)
    constexpr uint32_t KB_FREE = PAR ? KBUF1 : KBUF0;   // receives K(j+2)
    constexpr uint32_t VB_CUR = PAR ? VBUF1 : VBUF0;    // holds V(j)
    constexpr uint32_t VB_FREE = PAR ? VBUF0 : VBUF1;   // receives V(j+1)
    f32x16_t(&s_cur)[2] = PAR ? sb : sa;
    f32x16_t(&s_nxt)[2] = PAR ? sa : sb;
    wait_vmcnt<0>();  // K(j+1), V(j) have landed
    // every wave's loads have landed, and every wave is past iteration j-1,
    // whose reads of K(j) and V(j-1) were the last of the buffers refilled here
    __syncthreads();
    if constexpr (NEXT) {
      fill_v(j + 1, VB_FREE);
      if (j + 2 < n_blocks) fill_k(j + 2, KB_FREE);
    }
    constexpr bool MASKED = decltype(masked_tag)::value;
    const float m_sub = softmax_max(j, s_cur, masked_tag);
    u32x4_t pf[4];
    i32x8_t pf8;
    __builtin_amdgcn_sched_barrier(0);
    // the matrix-core part of the block at raised issue priority (as in the
    // two-wave 16-bit kernel)
    __builtin_amdgcn_s_setprio(1);
    if constexpr (NEXT) qk(std::integral_constant<uint32_t, KB_NEXT>{}, s_nxt);
    softmax_exp(s_cur, m_sub, pf, pf8, masked_tag);
    if constexpr (NEXT) {
      // per QK MFMA (64 cycles on the matrix core): its two K reads and a
      // share of the exponentials
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, MASKED ? 14 : 20, 0);  // VALU
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MASKED)
      pv(std::integral_constant<uint32_t, VB_CUR>{}, pf);
    else
      pv_fp8(std::integral_constant<uint32_t, VB_CUR>{}, pf8);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
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

  // ---- K-block pipeline ---------------------------------------------------
  using Unmasked = std::false_type;
  using Masked = std::true_type;
  using Next = std::true_type;
  using Last = std::false_type;
  fill_k(0, KBUF0);
  fill_v(0, VBUF0);
  if (n_blocks > 1) {
    fill_k(1, KBUF1);
    wait_vmcnt<K_INSTR + V_INSTR>();  // K(0) has landed
  } else {
    wait_vmcnt<V_INSTR>();
  }
  __syncthreads();
  qk(std::integral_constant<uint32_t, KBUF0>{}, sa);
  const int n_next = n_blocks - 1;  // iterations that have a next block
  const int j_mask = min(n_full, n_next);
  run(0, j_mask, Unmasked{}, Next{});
  run(j_mask, n_next, Masked{}, Next{});
  // the last block (peeled): masked unless every key of it is visible to
  // every row, in which case the mask is a no-op
  if (n_next & 1)
    iteration(n_next, Masked{}, Last{}, Par1{});
  else
    iteration(n_next, Masked{}, Last{}, Par0{});

  // ---- epilogue ------------------------------------------------------------
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
        w2[k].x = pack2<Bf16>(acc[t][r + 0] * inv, acc[t][r + 1] * inv);
        w2[k].y = pack2<Bf16>(acc[t][r + 2] * inv, acc[t][r + 3] * inv);
      }
      runs[t][p] = pair_runs16(w2[0], w2[1]);
    }
  if (row_ok) {
    uint16_t* orow = optr + ((size_t)(b * Sq + qrow) * a.head_q + h) * DV;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p) *(u32x4_t*)(orow + 32 * t + 16 * p + 8 * hl) = runs[t][p];
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
