// masked.hip -- prefill with a full additive mask for gfx950 (16-bit inputs).
//
// The mainloop's optional full mask ("Xe SDPA Forward Mainloop -- Key Loops
// + Shapes", section "Runtime args / params") is applied in its mask step
// (section "Compact shape table", row "Mask"): every score of the tile gets
// its mask value added before the online softmax, so every K block is a
// masked block.  O = softmax(Q K^T * scale + mask [+ causal]) V.
//
// Layout of the work: one wavefront = RT tiles of 16 query rows of one head;
// a workgroup = 4 such waves on consecutive rows of that head.  S^T = K Q^T
// on 16x16x32 MFMAs (a tile's 16 query rows are the N dimension), so lane
// (n16 = l % 16, gq = l / 16) holds the scores of row n16 of each tile for
// keys 16t + 4gq + r of each 16-key part t; row max and row sum reduce over
// the four gq lane groups.  Every K and V^T fragment read from LDS feeds the
// MFMAs of all RT tiles, which also gives the scheduler RT independent
// softmax chains per block.  Each wave streams its own K/V blocks of 32 keys
// into a wave-private double buffer in LDS with direct 16-byte loads (no
// barriers), and beside them the block's mask tiles: 16 rows x 32 keys x 2
// bytes = exactly one 1 KiB direct load per tile (lane l: row l / 4, keys
// 8 (l % 4) .. +7).  Each lane reads its 2 x 4 mask values per tile back with
// two ds_read_b64 and adds mask * log2(e) to the log2-domain scores.
#include <math.h>

#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <class T>
__device__ __forceinline__ float half_to_float(uint32_t bits16) {
  if constexpr (T::is_bf16)
    return __uint_as_float(bits16 << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <class T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_masked_kernel(const MaskedArgs a) {
  constexpr int RT = kMaskedRowTiles;         // 16-row tiles per wave
  constexpr int BK = kMaskedBlockK;           // 32 keys per block (two 16-key tiles)
  constexpr int KROW = D * 2, VROW = DV * 2;  // LDS bytes per key row
  constexpr int KCPR = D / 8, VCPR = DV / 8;  // 16-byte slots per row
  constexpr int KBYTES = BK * KROW, VBYTES = BK * VROW;
  constexpr int MBYTES = RT * 16 * BK * 2;    // mask tiles: RT x 16 rows x 32 keys
  constexpr int STAGE = KBYTES + VBYTES + MBYTES;
  constexpr int K_INSTR = KBYTES / 1024, V_INSTR = VBYTES / 1024;
  constexpr int KS = D / 32;                  // k-steps of the QK MFMA
  constexpr int NT = DV / 16;                 // O^T accumulator tiles
  static_assert(MBYTES == RT * 1024, "one direct load per mask tile");
  static_assert(K_INSTR * 1024 == KBYTES && V_INSTR * 1024 == VBYTES, "whole 1 KiB pieces");

  __shared__ __attribute__((aligned(1024))) char smem[kMaskedWaves * 2 * STAGE];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds_w = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem + wave * 2 * STAGE;

  const int Sq = a.q_len, Sk = a.kv_len, off = Sk - Sq;
  const int rt = blockIdx.x % a.row_tiles;
  const int bh = blockIdx.x / a.row_tiles;  // b * head_q + h
  const int h = bh % a.head_q;
  const int b = bh / a.head_q;
  const int g = h / a.group;
  const int row0 = (rt * kMaskedWaves + wave) * 16 * RT;
  if (row0 >= Sq) return;  // no barriers in this kernel

  const int n16 = lane & 15;  // query row within a tile (MFMA N index)
  const int gq = lane >> 4;   // lane group of 16
  int qrow[RT], row_end[RT];
  bool row_ok[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    qrow[u] = row0 + 16 * u + n16;
    row_ok[u] = qrow[u] < Sq;
    // keys [0, row_end) of this lane's row are visible before the mask
    row_end[u] = CAUSAL ? min(Sk, qrow[u] + off + 1) : Sk;
  }
  // keys the wave needs: all, or (causal) up to its last row's last visible key
  const int last_row = min(row0 + 16 * RT - 1, Sq - 1);
  const int k_end = CAUSAL ? min(Sk, max(last_row + off + 1, 0)) : Sk;
  const int nb = (k_end + BK - 1) / BK;

  // Q^T fragments (B operand of S^T = K Q^T): row qrow, dims 32s + 8gq .. +7
  u32x4_t qf[RT][KS];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const uint16_t* qp =
        (const uint16_t*)a.q + ((size_t)(b * Sq + min(qrow[u], Sq - 1)) * a.head_q + h) * D + 8 * gq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *(const u32x4_t*)(qp + 32 * s);
      qf[u][s] = row_ok[u] ? v : u32x4_t{0, 0, 0, 0};
    }
  }

  // direct fills: K/V rows as in the split-KV decode (16 or 8 lanes per key
  // row, swizzled slots), rows past the last key repeat it (masked later)
  const char* kbase = (const char*)a.k + ((size_t)b * Sk * a.head_kv + g) * KROW;
  const char* vbase = (const char*)a.v + ((size_t)b * Sk * a.head_kv + g) * VROW;
  const size_t kstride = (size_t)a.head_kv * KROW, vstride = (size_t)a.head_kv * VROW;
  int krow[K_INSTR], kcol[K_INSTR], vrow[V_INSTR], vcol[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int slot = i * 64 + lane, r = slot / KCPR;
    krow[i] = r;
    kcol[i] = ((slot % KCPR) ^ (int)swz_prefill<KCPR>(r)) * 16;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = i * 64 + lane, r = slot / VCPR;
    vrow[i] = r;
    vcol[i] = ((slot % VCPR) ^ (int)swz_decode<VCPR>(r)) * 16;
  }
  const int last_key = Sk - 1;
  // mask rows of this tile (rows past the end repeat the last row), lane's
  // 8-key chunk; a chunk is clamped to the padded row (row stride >= Sk,
  // a multiple of 8), so it never leaves the row: keys past Sk are masked
  const uint16_t* mbase = (const uint16_t*)a.mask + (size_t)b * a.mask_sb + (size_t)h * a.mask_sh;
  const uint16_t* mrow[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) mrow[u] = mbase + (size_t)min(row0 + 16 * u + (lane >> 2), Sq - 1) * a.mask_row;
  const int mcol = 8 * (lane & 3);
  auto issue_fill = [&](int key0, int stage) __attribute__((always_inline)) {
    const uint32_t kl = lds_w + stage * STAGE, vl = kl + KBYTES, ml = vl + VBYTES;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      global_to_lds_16(kbase + (size_t)min(key0 + krow[i], last_key) * kstride + kcol[i], kl + i * 1024);
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      global_to_lds_16(vbase + (size_t)min(key0 + vrow[i], last_key) * vstride + vcol[i], vl + i * 1024);
#pragma unroll
    for (int u = 0; u < RT; ++u) global_to_lds_16(mrow[u] + min(key0 + mcol, a.mask_row - 8), ml + u * 1024);
  };

  // K fragment (A operand): key row 16t + l%16, slot 4s + l/16
  uint32_t koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = n16 * KROW + (((4 * s + gq) ^ (int)swz_prefill<KCPR>(n16)) << 4);
  // V^T fragments via ds_read_b64_tr_b16 (as in the split-KV decode)
  uint32_t voff[2][NT];
  {
    const int s = lane & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 16 * hf + 4 * gq + (s >> 2);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = 16 * t + 4 * (s & 3);
        voff[hf][t] = r * VROW + (((col >> 3) ^ (int)swz_decode<VCPR>(r)) << 4) + ((col & 7) << 1);
      }
    }
  }
  // mask values of row n16, keys 16t + 4gq .. +3: 8 bytes at row * 64 + 32t + 8gq
  const uint32_t moff = n16 * (BK * 2) + 8 * gq;

  f32x4_t acc[RT][NT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[u][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }
  const float s2 = a.s2;

  auto block = [&](int key0, int stage) __attribute__((always_inline)) {
    const uint32_t ks = lds_w + stage * STAGE, vs = ks + KBYTES, ms = vs + VBYTES;
    f32x4_t sc[RT][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int u = 0; u < RT; ++u) sc[u][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4_t kf = lds_read_b128(ks + koff[s] + 16 * t * KROW);
#pragma unroll
        for (int u = 0; u < RT; ++u) sc[u][t] = mfma16x16x32<T>(kf, qf[u][s], sc[u][t]);
      }
    }
    u32x4_t pf[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      // log2-domain scores plus the mask; keys past the row's end are removed
      float x[8];
      float bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x2_t mv = *(SDPA_LDS const u32x2_t*)(uintptr_t)(ms + u * 1024 + moff + 32 * t);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t bits = (r < 2 ? mv.x : mv.y) >> (16 * (r & 1)) & 0xffffu;
          const float mval = half_to_float<T>(bits);
          const bool vis = key0 + 16 * t + 4 * gq + r < row_end[u];
          const float v = vis ? __builtin_fmaf(mval, kLog2e, sc[u][t][r] * s2) : -INFINITY;
          x[4 * t + r] = v;
          bmax = fmaxf(bmax, v);
        }
      }
      bmax = fmaxf(bmax, xor_lane(bmax, 16));
      bmax = fmaxf(bmax, xor_lane(bmax, 32));
      const float m_new = fmaxf(m_run[u], bmax);
      const float m_sub = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[u] - m_sub);
      m_run[u] = m_new;
      // P^T as the B operand: k = 8gq + j takes part 0 register j (j < 4)
      // and part 1 register j-4 (j >= 4)
      pf[u].x = pack2<T>(fast_exp2(x[0] - m_sub), fast_exp2(x[1] - m_sub));
      pf[u].y = pack2<T>(fast_exp2(x[2] - m_sub), fast_exp2(x[3] - m_sub));
      pf[u].z = pack2<T>(fast_exp2(x[4] - m_sub), fast_exp2(x[5] - m_sub));
      pf[u].w = pack2<T>(fast_exp2(x[6] - m_sub), fast_exp2(x[7] - m_sub));
      float psum = add_pair<T>(pf[u].x, 0.f);
      psum = add_pair<T>(pf[u].y, psum);
      psum = add_pair<T>(pf[u].z, psum);
      psum = add_pair<T>(pf[u].w, psum);
      l_run[u] = l_run[u] * alpha + psum;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[u][t] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x2_t lo = lds_read_tr16(vs + voff[0][t]);
      const u32x2_t hi = lds_read_tr16(vs + voff[1][t]);
      const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int u = 0; u < RT; ++u) acc[u][t] = mfma16x16x32<T>(vf, pf[u], acc[u][t]);
    }
  };

  // K/V/mask pipeline: block i+1 in flight while block i computes; the
  // direct loads are invisible to the compiler's wait counting, so every
  // wait is explicit (buffers private to the wave: no barrier)
  constexpr int PER_BLOCK = K_INSTR + V_INSTR + RT;
  if (nb > 0) {
    issue_fill(0, 0);
    int i = 0;
    for (; i < nb - 1; ++i) {
      issue_fill((i + 1) * BK, (i + 1) & 1);
      wait_vmcnt<PER_BLOCK>();
      block(i * BK, i & 1);
    }
    wait_vmcnt<0>();
    block(i * BK, i & 1);
  }

  // epilogue: O = O^T / l for row qrow (lane holds values 16t + 4gq + r)
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    float l_tot = l_run[u] + xor_lane(l_run[u], 16);
    l_tot += xor_lane(l_tot, 32);
    if (row_ok[u]) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = (uint16_t*)a.o + ((size_t)(b * Sq + qrow[u]) * a.head_q + h) * DV + 4 * gq;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *(u32x2_t*)(op + 16 * t) = u32x2_t{pack2<T>(acc[u][t][0] * inv, acc[u][t][1] * inv),
                                           pack2<T>(acc[u][t][2] * inv, acc[u][t][3] * inv)};
      if (a.lse != nullptr && gq == 0)
        a.lse[((size_t)b * a.head_q + h) * Sq + qrow[u]] =
            l_tot > 0.f ? (m_run[u] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <class T, int D>
static int launch_masked_t(const MaskedArgs& a, int causal, ihipStream_t* stream) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.head_q * a.row_tiles)), block(64 * kMaskedWaves);
  if (causal)
    hipLaunchKernelGGL((prefill_masked_kernel<T, D, D, true>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_masked_kernel<T, D, D, false>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_prefill_masked(const MaskedArgs& a, int in_dtype, int d, int causal, ihipStream_t* stream) {
  if (in_dtype == SDPA_BF16) return d == 64 ? launch_masked_t<Bf16, 64>(a, causal, stream)
                                            : launch_masked_t<Bf16, 128>(a, causal, stream);
  return d == 64 ? launch_masked_t<F16, 64>(a, causal, stream) : launch_masked_t<F16, 128>(a, causal, stream);
}

}  // namespace sdpa
