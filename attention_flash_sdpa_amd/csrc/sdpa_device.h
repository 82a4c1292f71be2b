// sdpa_device.h -- gfx950 device primitives shared by the attention kernels:
// MFMA wrappers, cross-lane row reductions, packing of probabilities into MFMA
// operands, direct global->LDS loads and the LDS swizzle.
//
// MFMA operand layouts used throughout (CDNA4, 64-lane wavefronts):
//   32x32x16 (bf16/f16):  A[m][k]: lane l holds m = l%32, k = 8*(l/32) + j
//                         B[k][n]: lane l holds n = l%32, k = 8*(l/32) + j
//                         C[m][n]: lane l, register r holds n = l%32,
//                                  m = 8*(r/4) + 4*(l/32) + r%4
//   16x16x32 (bf16/f16):  A: m = l%16, k = 8*(l/16) + j; B: n = l%16, same k;
//                         C: n = l%16, m = 4*(l/16) + r
//   32x32x64 (fp8 e4m3):  as 32x32x16 with 32 k-contiguous bytes per lane.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element r
// (r = 0..3) from the 8-byte row addressed by group lane 4r + i/4, at
// position i%4 -- a 4x16 -> 16x4 transpose of 16-bit elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lds_layout.h"

namespace sdpa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));


#define SDPA_LDS __attribute__((address_space(3)))

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (compile-time
// unrolled; every index is a constant expression inside f).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Largest growth (log2 units) of a row max tolerated before O and l are
// rescaled: probabilities then stay <= 2^8, far inside fp16/bf16 range.
constexpr float kSlack = 8.0f;

// Spreads consecutive logical workgroup ids over one XCD: hardware dispatches
// workgroup i to XCD i % 8, so logical ids [x*n/8, (x+1)*n/8) (which share
// K/V heads) are served by XCD x and its L2.
__device__ __forceinline__ int remap_xcd(int i, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = i & 7, j = i >> 3;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Element-type tags of the 16-bit inputs.
struct Bf16 {
  static constexpr bool is_bf16 = true;
};
struct F16 {
  static constexpr bool is_bf16 = false;
};

// 32x32x16 MFMA on 8 packed 16-bit elements per lane (bit patterns in u32x4).
template <class T>
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (T::is_bf16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---- hand-ordered building blocks of the prefill mainloop ----------------
// The mainloop issues its LDS fragment reads and its MFMAs from inline
// assembly so that their order, and with it the read-ahead distance, is the
// one written; the compiler keeps register allocation and the vector math in
// between.  Everything the compiler would otherwise insert for these
// instructions is explicit here:
//  * the LDS wait: each MFMA waits until at most LGKM LDS reads of this wave
//    are in flight (LDS reads complete in order, so the reads issued after
//    the one it needs may stay outstanding);
//  * no wait states before an MFMA for its A/B inputs: the Q K inputs come
//    from LDS or from registers written long before, and the slot schedule
//    packs each 16-key chunk of P at least a slot ahead of its P V MFMAs
//    (a vector write followed within two wait states by an MFMA read of the
//    same register would need them; an ISA scan of every built MFMA checks
//    that none occurs);
//  * mfma_acc_drain(): >= 18 wait states after the last P V MFMA before any
//    other instruction touches the accumulators.
template <int OFF>
__device__ __forceinline__ u32x4_t ds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// c = A B (C = 0) / c += A B, scores in VGPRs
template <class T, int LGKM>
__device__ __forceinline__ void mfma_s_first(f32x16_t& c, u32x4_t a, u32x4_t b) {
  static_assert(LGKM >= -1 && LGKM <= 15, "lgkmcnt range (-1: no wait)");
  if constexpr (T::is_bf16)
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                   : "=&v"(c) : "v"(a), "v"(b), "i"(LGKM));
  else
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0"
                   : "=&v"(c) : "v"(a), "v"(b), "i"(LGKM));
}
template <class T, int LGKM>
__device__ __forceinline__ void mfma_s_acc(f32x16_t& c, u32x4_t a, u32x4_t b) {
  static_assert(LGKM >= -1 && LGKM <= 15, "lgkmcnt range (-1: no wait)");
  if constexpr (T::is_bf16)
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+v"(c) : "v"(a), "v"(b), "i"(LGKM));
  else
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                   : "+v"(c) : "v"(a), "v"(b), "i"(LGKM));
}

// acc += A B with the accumulators in AGPRs (touched only by the matrix core
// inside the loop, which leaves the VGPRs to scores, fragments and softmax)
template <class T, int LGKM>
__device__ __forceinline__ void mfma_o_acc(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  static_assert(LGKM >= -1 && LGKM <= 15, "lgkmcnt range (-1: no wait)");
  if constexpr (T::is_bf16)
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(acc) : "v"(a), "v"(b), "i"(LGKM));
  else
    if constexpr (LGKM < 0)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                   : "+a"(acc) : "v"(a), "v"(b), "i"(LGKM));
}

template <int NT>
__device__ __forceinline__ void mfma_acc_drain(f32x16_t (&acc)[NT]) {
  if constexpr (NT == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]));
}

// >= 18 wait states after the last Q K MFMA of a block before any other
// instruction reads the two score tiles it wrote
__device__ __forceinline__ void mfma_s_drain(f32x16_t (&sc)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sc[0]), "+v"(sc[1]));
}

// Ties a value to this point of the instruction order: instructions that use
// the pinned value come after it, and (pinned at the end of a step) its
// producers come before it.  Emits nothing.
template <class V>
__device__ __forceinline__ void pin(V& v) {
  asm volatile("" : "+v"(v));
}

template <class T>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (T::is_bf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}


// Packs two fp32 values into one dword of 16-bit elements, round to nearest
// even (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <class T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  if constexpr (T::is_bf16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 32x32x64 MFMA on OCP fp8 e4m3 operands (32 bytes per lane), unit block
// scales (E8M0 exponent 127 = 2^0).
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four e4m3 bytes (one dword) widened exactly to four bf16 values (two dwords).
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap(a, b) swaps
// the upper half of a with the lower half of b, so with a = b = x the returned
// pair is (own, partner) in lanes 0-31 and (partner, own) in lanes 32-63: the
// max / sum of the pair is the same in both halves.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// O leaves the 32x32 accumulator layout in 4-column pieces: in a value tile,
// lane l holds columns 8j + 4(l/32) .. +3 of row l%32 (j = 0..3).  Two
// half-wave swaps turn the pieces j = 2p (w_even) and 2p+1 (w_odd) of the lane
// pair (l, l+32) into one 8-column run per lane, columns 16p + 8(l/32) .. +7,
// for one 16-byte store: v_permlane32_swap(a, b) exchanges lanes 32-63 of a
// with lanes 0-31 of b.
__device__ __forceinline__ u32x4_t pair_runs16(u32x2_t w_even, u32x2_t w_odd) {
  const auto sx = __builtin_amdgcn_permlane32_swap(w_even.x, w_odd.x, false, false);
  const auto sy = __builtin_amdgcn_permlane32_swap(w_even.y, w_odd.y, false, false);
  return u32x4_t{sx[0], sy[0], sx[1], sy[1]};
}

// The inverse of pair_runs16 for loads: the lane pair (l, l+32) loaded 16
// bytes each, lane l keys k0 .. k0+7 and lane l+32 keys k0+8 .. k0+15 of one
// row (two 16-bit keys per dword); afterwards each lane holds its own four of
// each 8-key run, lane l keys k0 .. +3 (lo) and k0+8 .. +3 (hi), lane l+32
// keys k0+4 .. +3 (lo) and k0+12 .. +3 (hi).
__device__ __forceinline__ void bias_runs(const u32x4_t& v, u32x2_t& lo, u32x2_t& hi) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  lo = u32x2_t{s0[0], s1[0]};
  hi = u32x2_t{s0[1], s1[1]};
}

// The same over the lane pair (l, l ^ 16): v_permlane16_swap(a, b) swaps the
// odd 16-lane rows of a with the even rows of b, so with a = b = x the pair
// is (own, partner) in even rows and (partner, own) in odd rows.
__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Butterfly over lanes with the given xor distance (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float x, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Transposed 8-byte LDS read (see the layout note at the top of the file).
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t byte_addr) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS s16x4_t*)(uintptr_t)byte_addr);
  return __builtin_bit_cast(u32x2_t, v);
}

// Transposed 8-byte LDS read of 8-bit elements: within each 16-lane group,
// lane i receives byte r (r = 0..7) of the 8-byte row addressed by group lane
// 2r + i/8, at position i%8 -- an 8x16 -> 16x8 byte transpose.
__device__ __forceinline__ u32x2_t lds_read_tr8(uint32_t byte_addr) {
  i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SDPA_LDS i32x2_t*)(uintptr_t)byte_addr);
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t byte_addr) {
  return *(SDPA_LDS const u32x4_t*)(uintptr_t)byte_addr;
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds_base + 16*i (lds_base is wavefront-uniform and goes through M0).
// Written as inline assembly so that the compiler's wait-count insertion does
// not see an LDS write here and force a full drain (vmcnt(0)) before every
// later LDS read; completion is tracked explicitly with wait_vmcnt<N>() and a
// workgroup barrier before the data is read.
//
// Hazards: the compiler does not see inside the asm, so the wait states the
// load needs after its inputs are written are inserted here -- one after an
// SALU write of M0 (s_nop 0), five after a VALU write (v_readfirstlane) of
// the SGPR base used by the scalar-base form below (s_nop 4).
__device__ __forceinline__ void global_to_lds_16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// As global_to_lds_16 with the non-temporal hint: for data read once (the
// decode's stream of K/V), which then does not displace reused lines.
__device__ __forceinline__ void global_to_lds_16_nt(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// As global_to_lds_16 with a wavefront-uniform 64-bit base in SGPRs and a
// per-lane 32-bit byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void global_to_lds_16_sbase(const void* sbase, uint32_t voffset, uint32_t lds_base) {
  // the base is uniform by construction; readfirstlane makes that explicit
  // for the compiler so the operand lands in SGPRs
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voffset), "s"(u), "{m0}"(lds_base) : "memory");
}

// 16-byte global load into a VGPR quad, issued from asm so that the
// compiler's wait-count tracking does not see it: it can then be issued
// ahead of direct-to-LDS loads and waited for with a vmcnt that leaves those
// in flight (the compiler would otherwise wait for all of them before the
// first use).  Its result is read only after a vmcnt wait that covers it and
// a pin of the registers (wait_vmcnt_pin<N>(), or wait_vmcnt<N>() then
// pin_regs()); an ISA scan checks that nothing touches them before the wait.
template <int OFF>
__device__ __forceinline__ void global_load_16_untracked(u32x4_t& d, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=&v"(d) : "v"(p), "i"(OFF) : "memory");
}

// As global_to_lds_16_off with a per-lane 64-bit address (the lane's address
// less OFF) instead of a scalar base: used where the lanes of one load read
// from different tensors.  A vector address carries no SGPR hazard, so only
// an M0 write needs its wait state (WAITS 1), else none (WAITS 0).
template <int OFF, int WAITS>
__device__ __forceinline__ void global_to_lds_16_voff(const void* addr, uint32_t m0_base) {
  static_assert(OFF >= 0 && OFF < 4096 && (WAITS == 0 || WAITS == 1), "offset / wait states");
  if constexpr (WAITS == 1)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(addr), "{m0}"(m0_base), "i"(OFF)
                 : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, off offset:%2" ::"v"(addr), "{m0}"(m0_base), "i"(OFF) : "memory");
}

// One dword load that waits for every outstanding vector-memory load of the
// wave (including untracked direct-to-LDS ones) before returning.  Meant for
// rare loads inside an explicitly counted load pipeline: a compiler-tracked
// load there would make the compiler wait on every path through the loop,
// this waits only where it runs.
__device__ __forceinline__ uint32_t global_load_dword_sync(const void* p) {
  uint32_t d;
  asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=&v"(d) : "v"(p) : "memory");
  return d;
}

// As global_to_lds_16_sbase, for a later load from the same base: the base
// SGPRs were written (by the first load's v_readfirstlane) at least five
// instructions earlier, so only the M0 write needs its wait state.
__device__ __forceinline__ void global_to_lds_16_sbase_next(const void* sbase, uint32_t voffset, uint32_t lds_base) {
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voffset), "s"(u), "{m0}"(lds_base) : "memory");
}

// Direct 16-byte load from base + voffset + OFF into LDS at m0_base + OFF
// (+16 per lane): the instruction's offset field applies to both addresses,
// so up to four consecutive 1 KiB loads share one M0 value.  WAITS is the
// wait states issued first: 5 after the v_readfirstlane that writes a new
// base, 1 after an M0 write, 0 when neither changed since the previous load.
template <int OFF, int WAITS>
__device__ __forceinline__ void global_to_lds_16_off(const void* sbase, uint32_t voffset, uint32_t m0_base) {
  static_assert(OFF >= 0 && OFF < 4096 && (WAITS == 0 || WAITS == 1 || WAITS == 5), "offset / wait states");
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  if constexpr (WAITS == 5)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voffset), "s"(u), "{m0}"(m0_base),
                 "i"(OFF) : "memory");
  else if constexpr (WAITS == 1)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voffset), "s"(u), "{m0}"(m0_base),
                 "i"(OFF) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voffset), "s"(u), "{m0}"(m0_base), "i"(OFF)
                 : "memory");
}

// Waits until at most N vector-memory operations of this wave are in flight,
// then marks the registers of d as written here, so no use of them can be
// scheduled before the wait.
template <int N, int K, class V>
__device__ __forceinline__ void wait_vmcnt_pin(V (&d)[K]) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" : "+v"(d[k]));
}

// Marks the registers of d as written here (after an explicit wait that
// covers their untracked loads), so no use of them moves above it.
template <int K, class V>
__device__ __forceinline__ void pin_regs(V (&d)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" : "+v"(d[k]));
}

// Waits until at most n vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace sdpa
