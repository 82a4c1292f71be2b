// decode.hip -- two-phase split-KV decode for gfx950 (one new token per
// sequence, 16-bit inputs).
//
// The page "xe2-sdp-kernels" (section "Assets") names a two-phase production
// decode; the split itself is the K-block subrange [blk_k0, blk_k1) of
// "Xe SDPA Forward Mainloop" (section "Outer K-block loop"), and the merge is
// the online-softmax rescale of its "softmax() helper" applied across splits.
//
// Phase 1 (decode_split_kernel): one wavefront per (batch, KV head, split);
// a workgroup holds 4 adjacent KV heads of one split so that its loads of a
// key are contiguous.  The G = head_q / head_kv query heads of the group are
// the MFMA N dimension (16x16x32 MFMA), so every K/V byte is read from HBM
// exactly once for all heads of the group ("xe2-sdp-kernels", section "GQA
// layout", which puts no bound on the group size).  A group of more than 16
// query heads takes one wave per 16-head tile, adjacent in the workgroup, so
// the tiles' reads of the same keys meet in L2.  K and V blocks of 32
// keys go HBM -> LDS with direct 16-byte loads (whole key rows per 16 lanes),
// one block ahead, into two wave-private stages; K fragments come back with
// ds_read_b128 and V^T fragments with ds_read_b64_tr_b16, both swizzled to
// avoid bank conflicts.  The wave writes its unnormalised partial output and
// its (max, sum) pair.
//
// Phase 2 (decode_combine_kernel): one wavefront per (batch, query head)
// merges the splits: M = max_s m_s, w_s = 2^(m_s - M), O = sum w_s O_s /
// sum w_s l_s (0 when nothing was visible), lse = ln2 * (M + log2 den).
// The prefill split across workgroups reuses it with one row per (batch,
// query row, query head) (launch_split_combine).
//
// Variable-length and paged caches (the mainloop's optional paged-KV
// arguments and its logical-to-physical K tile helper, "Xe SDPA Forward
// Mainloop", sections "Runtime args / params" and "Helpers"; its variable-
// length launch mode, section "Launcher -> kernel"): sequence b holds
// seq_lens[b] keys, and with a page table its keys p*page_size ..
// (p+1)*page_size - 1 sit in physical page page_table[b][p] of a
// [num_pages, page_size, head_kv, d] pool.  A page size that is a multiple
// of the 32-key block puts every block in one page (one table entry, a scalar
// base); pages of 8 or 16 keys split a block over 4 or 2 pages, and each lane
// takes its key row's page.  Table entries come from a register that holds
// 64 of the split's entries (one per lane).  An entry outside [0, num_pages)
// is never dereferenced: page 0 is read in its place and the affected rows
// come out NaN.
#include <math.h>

#include <mutex>

#include "sdpa_device.h"
#include "sdpa_internal.h"

namespace sdpa {

template <class T, int D, int DV, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a) {
  constexpr int BK = kDecodeBlockK;           // 32 keys per block (two 16-key tiles)
  constexpr int KROW = D * 2, VROW = DV * 2;  // LDS bytes per key row
  constexpr int KCPR = D / 8, VCPR = DV / 8;  // 16-byte slots per row
  constexpr int KBYTES = BK * KROW, VBYTES = BK * VROW;
  constexpr int STAGE = KBYTES + VBYTES;      // one K/V block of one wave
  constexpr int K_INSTR = KBYTES / 1024, V_INSTR = VBYTES / 1024;  // 1 KiB direct loads
  constexpr int KS = D / 32;                  // k-steps of the QK MFMA
  constexpr int NT = DV / 16;                 // O^T accumulator tiles
  static_assert(K_INSTR * 1024 == KBYTES && V_INSTR * 1024 == VBYTES, "whole 1 KiB pieces");

  __shared__ __attribute__((aligned(1024))) char smem[kDecodeWaves * 2 * STAGE];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds_w = (uint32_t)(uintptr_t)(SDPA_LDS char*)smem + wave * 2 * STAGE;

  // workgroup = (batch, split, 4 adjacent wave tasks); a wave task is one KV
  // head and one tile of up to 16 of its query heads (the MFMA N dimension):
  // task t covers KV head t / gtiles, query heads 16 * (t % gtiles) .. +15 of
  // its group.  Tiles of one KV head are adjacent, so a workgroup's loads of a
  // key are contiguous (4 head rows) or repeat one row, served by L2.
  const int S = a.num_splits;
  const int tasks = a.head_kv * a.gtiles;
  const int hgroups = (tasks + kDecodeWaves - 1) / kDecodeWaves;
  const int hgi = blockIdx.x % hgroups;
  const int split = (blockIdx.x / hgroups) % S;
  const int b = blockIdx.x / (hgroups * S);
  const int task = hgi * kDecodeWaves + wave;
  if (task >= tasks) return;  // no barriers in this kernel
  const int g = task / a.gtiles;
  const int h0 = 16 * (task - g * a.gtiles);   // first query head of the tile within the group
  const int G = min(a.group - h0, 16);          // query heads of this tile
  const int Sk = a.kv_len;
  // this sequence's keys: kv_len, or its own length clamped to [0, kv_len]
  const int seq_len = a.seq_lens == nullptr ? Sk : min(max(a.seq_lens[b], 0), Sk);
  const int k_begin = min(split * a.blocks_per_split * BK, seq_len);
  const int k_end = min(k_begin + a.blocks_per_split * BK, seq_len);
  const int nb = (k_end - k_begin + BK - 1) / BK;

  const int n16 = lane & 15;   // query head within the group (MFMA N index)
  const int gq = lane >> 4;    // lane group of 16
  const bool head_ok = n16 < G;
  const int h = g * a.group + h0 + min(n16, G - 1);

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

  // direct global -> LDS fill of one block: instruction i covers rows
  // [i*1024/ROW, ...), lane p the 16-byte slot p % CPR of its row, which holds
  // chunk slot ^ swizzle(row) -- so 16 (or 8) lanes read one whole key row
  // (dense: row 0 of sequence b; paged: row 0 of the pool, page p starting at
  // row p * page_size -- the rows of one page follow each other as in a
  // dense sequence)
  const size_t seq_rows = PAGED ? 0 : (size_t)b * Sk;
  const char* kbase = (const char*)a.k + (seq_rows * a.head_kv + g) * KROW;
  const char* vbase = (const char*)a.v + (seq_rows * a.head_kv + g) * VROW;
  const size_t kstride = (size_t)a.head_kv * KROW, vstride = (size_t)a.head_kv * VROW;
  int krow[K_INSTR], kcol[K_INSTR], vrow[V_INSTR], vcol[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int slot = i * 64 + lane, r = slot / KCPR;
    krow[i] = r;
    kcol[i] = fill_chunk_decode_k<KCPR>(slot) * 16;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int slot = i * 64 + lane, r = slot / VCPR;
    vrow[i] = r;
    vcol[i] = fill_chunk_decode<VCPR>(slot) * 16;
  }
  const int last_key = seq_len - 1;

  // paged: table entries of pages pt_first .. pt_first + 63 of this sequence
  // (lane i holds entry pt_first + i, clamped to the table row), the page and
  // row within it of the next block to fill, and whether any entry used was
  // out of range.  Fills run in key order, so the cursor just advances.
  int pt_first = 0, pt_page = 0, pt_row = 0;
  int pt_vals = 0;
  bool pt_bad = false;
  const int32_t* pt = PAGED ? a.page_table + (size_t)b * a.pages_per_seq : nullptr;
  // pages of fewer than BK keys: a block covers nsub = BK / page_size whole
  // pages (blocks start at multiples of BK, so pt_row stays 0)
  const int nsub = PAGED && a.page_size < BK ? BK / a.page_size : 1;
  const int sub_shift = nsub == 4 ? 3 : 4;  // log2 of the keys per page (8 or 16)
  if constexpr (PAGED) {
    if (nb > 0) {
      pt_page = k_begin / a.page_size;
      pt_row = k_begin - pt_page * a.page_size;
      pt_first = pt_page;
      pt_vals = pt[min(pt_first + lane, a.pages_per_seq - 1)];
    }
  }

  auto issue_fill = [&](int key0, int stage) __attribute__((always_inline)) {
    const uint32_t kl = lds_w + stage * STAGE, vl = kl + KBYTES;
    // rows past the sequence end repeat its last key (masked later); they stay
    // in the block's page because blocks start at multiples of 32 keys
    const int lim = last_key - key0;
    size_t row0 = (size_t)key0;
    if constexpr (PAGED) {
      if (pt_page - pt_first + nsub > 64) {  // next 64 entries (long splits only)
        pt_first = pt_page;
        pt_vals = (int)global_load_dword_sync(pt + min(pt_first + lane, a.pages_per_seq - 1));
      }
      if (nsub > 1) {
        // small pages: entries of the block's pages that hold a key of the
        // sequence (rows past its end are clamped to its last key, so the
        // others are never used and may hold anything)
        int ph[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool used = j < nsub && (j << sub_shift) <= lim;
          int e = __builtin_amdgcn_readlane(pt_vals, pt_page - pt_first + (used ? j : 0));
          if ((uint32_t)e >= (uint32_t)a.num_pages) {
            pt_bad = pt_bad || used;
            e = 0;
          }
          ph[j] = e;
        }
        pt_page += nsub;
        auto addr = [&](const char* base, int r, size_t stride, int col) __attribute__((always_inline)) {
          const int j = r >> sub_shift;
          const int e = j == 0 ? ph[0] : (j == 1 ? ph[1] : (j == 2 ? ph[2] : ph[3]));
          const size_t row = (size_t)e * a.page_size + (r & ((1 << sub_shift) - 1));
          return base + row * stride + col;
        };
#pragma unroll
        for (int i = 0; i < K_INSTR; ++i)
          global_to_lds_16_nt(addr(kbase, min(krow[i], lim), kstride, kcol[i]), kl + i * 1024);
#pragma unroll
        for (int i = 0; i < V_INSTR; ++i)
          global_to_lds_16_nt(addr(vbase, min(vrow[i], lim), vstride, vcol[i]), vl + i * 1024);
        return;
      }
      int phys = __builtin_amdgcn_readlane(pt_vals, pt_page - pt_first);
      if ((uint32_t)phys >= (uint32_t)a.num_pages) {
        pt_bad = true;
        phys = 0;
      }
      row0 = (size_t)phys * a.page_size + pt_row;
      pt_row += BK;
      if (pt_row == a.page_size) {
        pt_row = 0;
        ++pt_page;
      }
    }
    const char* kb = kbase + row0 * kstride;
    const char* vb = vbase + row0 * vstride;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      global_to_lds_16_nt(kb + (size_t)min(krow[i], lim) * kstride + kcol[i], kl + i * 1024);
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      global_to_lds_16_nt(vb + (size_t)min(vrow[i], lim) * vstride + vcol[i], vl + i * 1024);
  };

  // K fragment (A operand of 16x16x32): key row 16t + l%16, slot 4s + l/16
  uint32_t koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = decode_k_read<KCPR>(lane, s);
  // V^T fragment offsets for ds_read_b64_tr_b16: lane (gq, s = l%16) addresses
  // key row 4*gq + s/4 (+16 for the second half) at value columns 16t + 4*(s%4)
  uint32_t voff[2][NT];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int t = 0; t < NT; ++t) voff[hf][t] = decode_vt_read<VCPR>(lane, hf, t);

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float s2 = a.s2;

  auto block = [&](int key0, int stage, bool masked) __attribute__((always_inline)) {
    const uint32_t ks = lds_w + stage * STAGE, vs = ks + KBYTES;
    f32x4_t sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc[t] = mfma16x16x32<T>(lds_read_b128(ks + koff[s] + 16 * t * KROW), qf[s], sc[t]);
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
        if (masked) v = (key0 + 16 * t + 4 * gq + r < k_end) ? v : -INFINITY;
        x[4 * t + r] = v;
        bmax = fmaxf(bmax, v);
      }
    bmax = pair_max(pair16_max(bmax));
    const float m_new = fmaxf(m_run, bmax);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_sub);
    m_run = m_new;
    // P^T as the B operand: k = 8*gq + j takes tile 0 register j (j < 4) and
    // tile 1 register j-4 (j >= 4)
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(x[i] - m_sub);
    u32x4_t pf;
    pf.x = pack2<T>(p[0], p[1]);
    pf.y = pack2<T>(p[2], p[3]);
    pf.z = pack2<T>(p[4], p[5]);
    pf.w = pack2<T>(p[6], p[7]);
    const float psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));  // over the fp32 P
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x2_t lo = lds_read_tr16(vs + voff[0][t]);
      const u32x2_t hi = lds_read_tr16(vs + voff[1][t]);
      const u32x4_t vf = {lo.x, lo.y, hi.x, hi.y};
      acc[t] = mfma16x16x32<T>(vf, pf, acc[t]);
    }
  };

  // K/V pipeline: block i+1 is in flight while block i computes.  All loads
  // are direct-to-LDS and invisible to the compiler's wait counting, so every
  // wait below is explicit; the buffers are private to the wave (no barrier).
  if (nb > 0) {
    issue_fill(k_begin, 0);
    int i = 0;
    for (; i < nb - 1; ++i) {
      issue_fill(k_begin + (i + 1) * BK, (i + 1) & 1);
      wait_vmcnt<K_INSTR + V_INSTR>();
      block(k_begin + i * BK, i & 1, false);
    }
    wait_vmcnt<0>();
    block(k_begin + i * BK, i & 1, true);  // last block: keys past k_end masked
  }

  // partial results: unnormalised O^T (lane holds head n16, values 16t + 4*gq + r)
  float l_tot = pair_sum(pair16_sum(l_run));
  if constexpr (PAGED) {
    if (pt_bad) {  // a page-table entry was out of range: poison the rows
      l_tot = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{l_tot, l_tot, l_tot, l_tot};
    }
  }
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

// splits combined from registers in one pass (more use the looped path)
constexpr int kCombineFast = 32;

// lse position of combine row bh = b' * head_q + h: bh itself for decode;
// for the prefill's rows b' = b * lse_q_len + i, [b, h, i] of [batch, head_q,
// q_len]
__device__ inline size_t combine_lse_index(const DecodeArgs& a, int bh) {
  if (a.lse_q_len <= 1) return (size_t)bh;
  const int h = bh % a.head_q, bq = bh / a.head_q;
  return ((size_t)(bq / a.lse_q_len) * a.head_q + h) * a.lse_q_len + bq % a.lse_q_len;
}

template <class T, int DV>
__global__ __launch_bounds__(64 * kCombineRows) void decode_combine_kernel(const DecodeArgs a) {
  constexpr int PER = DV / 64;   // value columns per lane (contiguous)
  constexpr int CH = 16;         // splits whose partials are loaded together
  typedef float vec_t __attribute__((ext_vector_type(PER)));
  // one wave per (batch, query head) row, kCombineRows rows per workgroup
  const int bh = blockIdx.x * kCombineRows + (threadIdx.x >> 6);  // b * head_q + h
  const int lane = threadIdx.x & 63;
  if (bh >= a.batch * a.head_q) return;  // no barriers in this kernel
  const int S = a.num_splits;
  const float* ml = a.part_ml + (size_t)bh * S * 2;
  const float* po = a.part_o + (size_t)bh * S * DV + PER * lane;

  if (S <= kCombineFast) {
    // Every lane loads all (m, l) pairs (one cache line, broadcast) and its
    // columns of every partial row at once, then combines in registers: no
    // cross-lane reduction, one memory round trip.
    f32x2_t mlv[kCombineFast];
    vec_t vals[kCombineFast];
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) mlv[u] = u < S ? *(const f32x2_t*)(ml + 2 * u) : f32x2_t{-INFINITY, 0.f};
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) vals[u] = u < S ? *(const vec_t*)(po + (size_t)u * DV) : (vec_t)0.f;
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) M = fmaxf(M, mlv[u][0]);
    const float m_sub = M == -INFINITY ? 0.f : M;
    float den = 0.f;
    vec_t num = (vec_t)0.f;
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) {
      const float mu = mlv[u][0], lu = mlv[u][1];
      const float w = u < S ? fast_exp2(mu - m_sub) : 0.f;  // 0 for an empty split (m = -inf)
      den += w * lu;
      num += w * vals[u];
    }
    const float inv = den > 0.f ? a.v_descale / den : 0.f;
    uint16_t* o = (uint16_t*)a.o + (size_t)bh * DV + PER * lane;
    if constexpr (PER == 2) {
      *(uint32_t*)o = pack2<T>(num[0] * inv, num[1] * inv);
    } else {
      o[0] = (uint16_t)(pack2<T>(num[0] * inv, 0.f) & 0xffff);
    }
    if (a.lse != nullptr && lane == 0)
      a.lse[combine_lse_index(a, bh)] = den == 0.f ? -INFINITY : (M + log2f(den)) * kLn2;
    return;
  }

  // many splits: global max over splits (lane s covers splits s, s+64, ...)
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, xor_lane(M, d));
  const float m_sub = M == -INFINITY ? 0.f : M;

  // weighted sums: one split weight per lane, CH partial rows loaded at once
  float den = 0.f;
  vec_t num = (vec_t)0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f;
    if (s < S) {
      w = fast_exp2(ml[2 * s] - m_sub);  // 0 for an empty split (m = -inf)
      den += w * ml[2 * s + 1];
    }
    const int n = min(64, S - s0);
    for (int c0 = 0; c0 < n; c0 += CH) {
      vec_t vals[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u)
        vals[u] = c0 + u < n ? *(const vec_t*)(po + (size_t)(s0 + c0 + u) * DV) : (vec_t)0.f;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(c0 + u, 63)));
        num += (c0 + u < n ? wu : 0.f) * vals[u];
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) den += xor_lane(den, d);

  const float inv = den > 0.f ? a.v_descale / den : 0.f;
  uint16_t* o = (uint16_t*)a.o + (size_t)bh * DV + PER * lane;
  if constexpr (PER == 2) {
    *(uint32_t*)o = pack2<T>(num[0] * inv, num[1] * inv);
  } else {
    o[0] = (uint16_t)(pack2<T>(num[0] * inv, 0.f) & 0xffff);
  }
  if (a.lse != nullptr && lane == 0)
      a.lse[combine_lse_index(a, bh)] = den == 0.f ? -INFINITY : (M + log2f(den)) * kLn2;
}

// ---- scratch of the no-allocation decode entry point -----------------------
// Split partials of sdpa_decode_fwd_noalloc live in this file-scope array, one
// copy per GPU the library runs on, held until the process ends.  In host code
// `scratch` only names a host-side stand-in: its device address on the current
// GPU comes from hipGetSymbolAddress, fetched once per device and kept.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

template <class T, int D>
static int launch_decode_t(const DecodeArgs& a, const sdpa_plan_t& plan, ihipStream_t* stream) {
  if (a.page_table != nullptr)
    hipLaunchKernelGGL((decode_split_kernel<T, D, D, true>), dim3(plan.num_groups), dim3(64 * kDecodeWaves), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, D, false>), dim3(plan.num_groups), dim3(64 * kDecodeWaves), 0,
                       (hipStream_t)stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(plan.combine_groups), dim3(64 * kCombineRows), 0, (hipStream_t)stream,
                     a);
  return (int)hipGetLastError();
}

int launch_split_combine(const DecodeArgs& a, int in_dtype, int d_v, int groups, ihipStream_t* stream) {
  const dim3 grid(groups), block(64 * kCombineRows);
  const bool bf = in_dtype == SDPA_BF16;
  if (in_dtype != SDPA_BF16 && in_dtype != SDPA_F16) return (int)hipErrorInvalidValue;
  if (d_v == 64) {
    if (bf) hipLaunchKernelGGL((decode_combine_kernel<Bf16, 64>), grid, block, 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((decode_combine_kernel<F16, 64>), grid, block, 0, (hipStream_t)stream, a);
  } else if (d_v == 128) {
    if (bf) hipLaunchKernelGGL((decode_combine_kernel<Bf16, 128>), grid, block, 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((decode_combine_kernel<F16, 128>), grid, block, 0, (hipStream_t)stream, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
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
