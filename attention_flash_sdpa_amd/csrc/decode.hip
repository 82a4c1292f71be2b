// decode.hip -- two-phase split-KV decode for gfx950 (one new token per
// sequence, 16-bit inputs).
//
// The page "xe2-sdp-kernels" (section "Assets") names a two-phase production
// decode; the split itself is the K-block subrange [blk_k0, blk_k1) of
// "Xe SDPA Forward Mainloop" (section "Outer K-block loop"), and the merge is
// the online-softmax rescale of its "softmax() helper" applied across splits.
//
// Phase 1 (decode_split_kernel): one wavefront per (batch, KV head, split).
// The G = head_q / head_kv query heads of the group are the MFMA N dimension
// (16x16x32 MFMA, G <= 16), so every K/V byte is read from HBM exactly once
// for all heads of the group.  K fragments go straight from HBM into
// registers (they already have the A-operand layout: one key row per lane, 16
// contiguous bytes); V blocks go HBM -> LDS with direct loads and come back
// transposed with ds_read_b64_tr_b16.  Both are prefetched one 32-key block
// ahead, ping-ponging between two register sets and two LDS stages.  The wave
// writes its unnormalised partial output and its (max, sum) pair.
//
// Phase 2 (decode_combine_kernel): one wavefront per (batch, query head)
// merges the splits: M = max_s m_s, w_s = 2^(m_s - M), O = sum w_s O_s /
// sum w_s l_s (0 when nothing was visible), lse = ln2 * (M + log2 den).
#include <math.h>

#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <class T, int D, int DV>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a) {
  constexpr int BK = kDecodeBlockK;           // 32 keys per block (two 16-key tiles)
  constexpr int VROW = DV * 2;
  constexpr int VCPR = DV / 8;
  constexpr int VBYTES = BK * VROW;           // one V stage
  constexpr int V_INSTR = VBYTES / 1024;      // 1 KiB direct loads per block
  constexpr int KS = D / 32;                  // k-steps of the QK MFMA
  constexpr int NT = DV / 16;                 // O^T accumulator tiles
  constexpr int K_LOADS = 2 * KS;             // 16-byte K loads per lane per block
  static_assert(VCPR >= 8, "swizzle needs >= 8 slots per row");
  static_assert(V_INSTR * 1024 == VBYTES, "V block must be whole 1 KiB pieces");

  __shared__ __attribute__((aligned(1024))) char smem[kDecodeWaves * 2 * VBYTES];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds_w = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem + wave * 2 * VBYTES;

  const int S = a.num_splits;
  const int wid = blockIdx.x * kDecodeWaves + wave;
  if (wid >= a.batch * a.head_kv * S) return;  // no barriers in this kernel
  const int split = wid % S;
  const int g = (wid / S) % a.head_kv;
  const int b = wid / (S * a.head_kv);
  const int G = a.group;
  const int Sk = a.kv_len;
  const int k_begin = min(split * a.blocks_per_split * BK, Sk);
  const int k_end = min(k_begin + a.blocks_per_split * BK, Sk);
  const int nb = (k_end - k_begin + BK - 1) / BK;

  const int n16 = lane & 15;   // query head within the group (MFMA N index)
  const int gq = lane >> 4;    // lane group of 16
  const bool head_ok = n16 < G;
  const int h = g * G + min(n16, G - 1);

  // Q^T fragments (B operand of S^T = K Q^T): head n16, dims 32s + 8*gq .. +7
  u32x4_t qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)b * a.head_q + h) * D + 8 * gq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *(const u32x4_t*)(qp + 32 * s);
      qf[s] = head_ok ? v : u32x4_t{0, 0, 0, 0};
    }
  }

  const size_t row_k = (size_t)a.head_kv * D;   // elements between keys
  const size_t row_v = (size_t)a.head_kv * DV;
  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * Sk * a.head_kv + g) * D + 8 * gq;
  const char* vbase = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * (DV * 2);
  const int last_key = Sk - 1;

  // K fragment loads for block kb: lane reads key (tile*16 + n16), dims
  // 32s + 8*gq .. +7 (the A-operand layout of 16x16x32).
  auto load_k = [&](int kb, u32x4_t (&kf)[K_LOADS]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = min(kb + 16 * t + n16, last_key);
      const uint16_t* kp = kbase + (size_t)key * row_k;
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[t * KS + s] = *(const u32x4_t*)(kp + 32 * s);
    }
  };
  // V block kb into LDS stage: rows of DV values, 16-byte slots swizzled.
  int vrow[V_INSTR], vcol[V_INSTR];
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = i * 64 + lane;
    const int r = slot / VCPR;
    vrow[i] = r;
    vcol[i] = ((slot % VCPR) ^ (int)swz(r)) * 16;
  }
  auto load_v = [&](int kb, int stage) {
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i) {
      const int key = min(kb + vrow[i], last_key);
      global_to_lds_16(vbase + (size_t)key * row_v * 2 + vcol[i], lds_w + stage * VBYTES + i * 1024);
    }
  };
  // transposed V^T fragment offsets: lane (gq, s = l%16) addresses key row
  // 4*gq + s/4 (+16 for the second half) at value columns 16t + 4*(s%4)
  uint32_t voff[NT];
  {
    const int s = lane & 15;
    const int r = 4 * gq + (s >> 2);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * t + 4 * (s & 3);
      voff[t] = r * VROW + (((col >> 3) ^ (int)swz(r)) << 4) + ((col & 7) << 1);
    }
  }

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float s2 = a.s2;

  auto block = [&](int kb, int stage, const u32x4_t (&kf)[K_LOADS], bool prefetched, bool masked) {
    f32x4_t sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc[t] = mfma16x16x32<T>(kf[t * KS + s], qf[s], sc[t]);
    }
    // scores in the log2 domain; keys past the split end are masked (only in
    // the split's last block)
    float x[8];
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[t][r] * s2;
        if (masked) v = (kb + 16 * t + 4 * gq + r < k_end) ? v : -INFINITY;
        x[4 * t + r] = v;
        bmax = fmaxf(bmax, v);
      }
    bmax = fmaxf(bmax, xor_lane(bmax, 16));
    bmax = fmaxf(bmax, xor_lane(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_sub);
    m_run = m_new;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(x[i] - m_sub);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    // P^T as the B operand: k = 8*gq + j takes tile 0 register j (j < 4) and
    // tile 1 register j-4 (j >= 4)
    u32x4_t pf;
    pf.x = pack2<T>(p[0], p[1]);
    pf.y = pack2<T>(p[2], p[3]);
    pf.z = pack2<T>(p[4], p[5]);
    pf.w = pack2<T>(p[6], p[7]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    if (prefetched)
      wait_vmcnt<K_LOADS + V_INSTR>();
    else
      wait_vmcnt<0>();
    const uint32_t vs = lds_w + stage * VBYTES;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x2_t lo = lds_read_tr16(vs + voff[t]);
      const u32x2_t hi = lds_read_tr16(vs + voff[t] + 16 * VROW);
      const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
      acc[t] = mfma16x16x32<T>(vf, pf, acc[t]);
    }
  };

  if (nb > 0) {
    u32x4_t ka[K_LOADS], kb2[K_LOADS];
    load_k(k_begin, ka);
    load_v(k_begin, 0);
    for (int i = 0; i < nb; i += 2) {
      const int key0 = k_begin + i * BK;
      const bool has1 = i + 1 < nb;
      if (has1) {
        load_k(key0 + BK, kb2);
        load_v(key0 + BK, 1);
      }
      block(key0, 0, ka, has1, !has1);
      if (has1) {
        const bool has2 = i + 2 < nb;
        if (has2) {
          load_k(key0 + 2 * BK, ka);
          load_v(key0 + 2 * BK, 0);
        }
        block(key0 + BK, 1, kb2, has2, !has2);
      }
    }
  }

  // partial results: unnormalised O^T (lane holds head n16, values 16t + 4*gq + r)
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += xor_lane(l_tot, 32);
  if (head_ok) {
    const size_t pidx = ((size_t)b * a.head_q + h) * S + split;
    float* po = a.part_o + pidx * DV + 4 * gq;
#pragma unroll
    for (int t = 0; t < NT; ++t) *(f32x4_t*)(po + 16 * t) = acc[t];
    if (gq == 0) {
      a.part_ml[2 * pidx] = m_run;
      a.part_ml[2 * pidx + 1] = l_tot;
    }
  }
}

template <class T, int DV>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeArgs a) {
  const int bh = blockIdx.x;  // b * head_q + h
  const int lane = threadIdx.x;
  const int S = a.num_splits;
  const float* ml = a.part_ml + (size_t)bh * S * 2;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  const float m_sub = M == -INFINITY ? 0.f : M;
  float den = 0.f;
  constexpr int PER = DV / 64;
  float num[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) num[j] = 0.f;
  const float* po = a.part_o + (size_t)bh * S * DV;
  for (int s = 0; s < S; ++s) {
    const float w = fast_exp2(ml[2 * s] - m_sub);  // 0 for an empty split
    den += w * ml[2 * s + 1];
#pragma unroll
    for (int j = 0; j < PER; ++j) num[j] += w * po[(size_t)s * DV + lane + 64 * j];
  }
  const float inv = den > 0.f ? a.v_descale / den : 0.f;
  uint16_t* o = (uint16_t*)a.o + (size_t)bh * DV;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t w = pack2<T>(num[j] * inv, 0.f);
    o[lane + 64 * j] = (uint16_t)(w & 0xffff);
  }
  if (a.lse != nullptr && lane == 0) a.lse[bh] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

template <class T, int D>
static int launch_decode_t(const DecodeArgs& a, const sdpa_plan_t& plan, ihipStream_t* stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D, D>), dim3(plan.num_groups), dim3(64 * kDecodeWaves), 0,
                     (hipStream_t)stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(plan.combine_groups), dim3(64), 0, (hipStream_t)stream,
                     a);
  return (int)hipGetLastError();
}

int launch_decode(const DecodeArgs& a, const sdpa_plan_t& plan, ihipStream_t* stream) {
  switch (plan.kernel) {
    case kDecodeF16D64: return launch_decode_t<F16, 64>(a, plan, stream);
    case kDecodeBf16D64: return launch_decode_t<Bf16, 64>(a, plan, stream);
    case kDecodeF16D128: return launch_decode_t<F16, 128>(a, plan, stream);
    case kDecodeBf16D128: return launch_decode_t<Bf16, 128>(a, plan, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace sdpa
