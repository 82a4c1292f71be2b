// lds_layout.h -- where the K/V blocks sit in LDS and which bytes each lane's
// fragment reads address.  Plain integer functions, compiled for the device
// (the kernels) and for the host (the CPU model of the LDS banks in the
// tests), so both use one definition.
//
// Fills.  A block is filled by direct global->LDS loads of 16 bytes per lane,
// 64 lanes per instruction, to consecutive LDS slots: slot s (byte 16*s of the
// block) belongs to row s / SLOTS (SLOTS = row bytes / 16) and holds that
// row's 16-byte chunk (s % SLOTS) ^ f(row).  So chunk c of row r sits at
// 16-byte position c ^ f(r) of the row (the XOR is its own inverse).
//
// Banks.  The LDS has 64 banks of 4 bytes.  A ds_read_b64 (plain or
// transposed) is served 32 consecutive lanes at a time.  A ds_read_b128 is
// served 16 lanes at a time, in the groups {0-3, 12-15, 20-23, 24-27} and
// {4-7, 8-11, 16-19, 28-31} of each half-wave (measured with the LDS
// bank-conflict counter on MI355X).  A read is conflict-free when each group
// addresses 64 distinct banks, i.e. distinct 16- (or 8-) byte positions of a
// 256-byte bank line.  The swizzles f below are chosen for the read patterns
// that follow them.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#include <hip/hip_runtime.h>
#define SDPA_LAYOUT_FN __host__ __device__ __forceinline__ constexpr
#else
#define SDPA_LAYOUT_FN inline constexpr
#endif

namespace sdpa {

// ---- swizzles ---------------------------------------------------------------
// Prefill rows (SLOTS = 16 or 8), read as
//  * K fragments (ds_read_b128): 16 consecutive rows at one chunk;
//  * V^T fragments (ds_read_b64_tr_b16): 4 consecutive rows x 4 chunks per
//    half-wave.
// With 16 slots per 256-byte row, f swaps the two 2-bit fields of r % 16; with
// 8 slots (two rows per bank line) f applies the 3-bit analogue to r / 2.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t swz_prefill(uint32_t r) {
  static_assert(SLOTS == 16 || SLOTS == 8, "row of 128 or 256 bytes");
  if constexpr (SLOTS == 16) return ((r & 3u) << 2) | ((r >> 2) & 3u);
  const uint32_t x = r >> 1;
  return ((x & 1u) << 2) | ((x >> 1) & 3u);
}

// 64-byte rows (4 slots, four rows per bank line), read as 16 consecutive rows
// at one chunk: f = (r / 4) % 4 spreads them over the 16 positions.
SDPA_LAYOUT_FN uint32_t swz_quarter(uint32_t r) { return (r >> 2) & 3u; }

// Decode K fragments (16x16x32 MFMA, ds_read_b128): lane l reads row l % 16 at
// chunk 4s + l / 16, so a 16-lane group holds rows {0-3, 12-15} at one chunk
// and rows {4-11} at the next (or the reverse).  With 16 slots f keeps the
// prefill form in bits 2-3 and puts bit 3 of r in bit 1, which separates the
// two row sets; with 8 slots f = (r / 2) % 8.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t swz_decode_k(uint32_t r) {
  static_assert(SLOTS == 16 || SLOTS == 8, "row of 128 or 256 bytes");
  if constexpr (SLOTS == 16) return ((r & 3u) << 2) | ((r >> 2) & 2u);
  return (r >> 1) & 7u;
}

// Decode V^T fragments (16x16x32 MFMA, ds_read_b64_tr_b16): each half-wave
// reads 8 consecutive rows x 2 adjacent chunks.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t swz_decode(uint32_t r) {
  static_assert(SLOTS == 16 || SLOTS == 8, "row of 128 or 256 bytes");
  if constexpr (SLOTS == 16) return (r & 7u) << 1;
  return ((r >> 1) & 3u) << 1;
}

// ---- fills: the row chunk that block slot `slot` holds ----------------------
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t fill_chunk_prefill(uint32_t slot) {
  return (slot % SLOTS) ^ swz_prefill<SLOTS>(slot / SLOTS);
}
SDPA_LAYOUT_FN uint32_t fill_chunk_quarter(uint32_t slot) { return (slot % 4u) ^ swz_quarter(slot / 4u); }
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t fill_chunk_decode_k(uint32_t slot) {
  return (slot % SLOTS) ^ swz_decode_k<SLOTS>(slot / SLOTS);
}
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t fill_chunk_decode(uint32_t slot) {
  return (slot % SLOTS) ^ swz_decode<SLOTS>(slot / SLOTS);
}

// ---- fragment reads: byte offset within the block ---------------------------
// 16-bit prefill, 32x32x16 K fragment (A operand of S^T = K Q^T, ds_read_b128)
// for k-step s: key row l % 32, head-dim chunk 2s + l / 32.  Score tile t adds
// 32 rows (32 * row bytes), which leaves the swizzle unchanged.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t prefill_k_read(uint32_t lane, uint32_t s) {
  const uint32_t r = lane & 31u;
  return r * SLOTS * 16u + (((2u * s + (lane >> 5)) ^ swz_prefill<SLOTS>(r)) << 4);
}

// 16-bit prefill, V^T fragment (A operand of O^T = V^T P^T) by
// ds_read_b64_tr_b16, half hf, value tile t: lane (group gq = l/16, s = l%16)
// addresses key row 8hf + 4(gq/2) + s/4 at value columns 32t + 16(gq%2) +
// 4(s%4) .. +3.  Key chunk c adds 16 rows, which leaves the swizzle unchanged.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t prefill_vt_read(uint32_t lane, uint32_t hf, uint32_t t) {
  const uint32_t gq = lane >> 4, s = lane & 15u;
  const uint32_t r = 8u * hf + 4u * (gq >> 1) + (s >> 2);
  const uint32_t col = 32u * t + 16u * (gq & 1u) + 4u * (s & 3u);
  return r * SLOTS * 16u + (((col >> 3) ^ swz_prefill<SLOTS>(r)) << 4) + ((col & 7u) << 1);
}

// fp8 prefill (d_qk 192 as a 128-byte part A and a 64-byte part B per key,
// d_v 128).  K fragment of the 32x32x64 MFMA, k-step s of part A (s = 0, 1) or
// of part B, 16-byte half c: key row l % 32, chunk 4s + 2(l/32) + c of part A
// or 2(l/32) + c of part B.
SDPA_LAYOUT_FN uint32_t fp8_ka_read(uint32_t lane, uint32_t s, uint32_t c) {
  const uint32_t r = lane & 31u;
  return r * 128u + (((4u * s + 2u * (lane >> 5) + c) ^ swz_prefill<8>(r)) << 4);
}
SDPA_LAYOUT_FN uint32_t fp8_kb_read(uint32_t lane, uint32_t c) {
  const uint32_t r = lane & 31u;
  return r * 64u + (((2u * (lane >> 5) + c) ^ swz_quarter(r)) << 4);
}
// fp8 V^T fragment by ds_read_b64_tr_b8, value tile t: lane (gq = l/16,
// s = l%16) addresses key row 8(r/4) + 4(gq/2) + r%4 with r = s/2 at value
// bytes 32t + 16(gq%2) + 8(s%2) .. +7.  Key chunk c adds 16 rows.
SDPA_LAYOUT_FN uint32_t fp8_vt_read(uint32_t lane, uint32_t t) {
  const uint32_t gq = lane >> 4, s = lane & 15u, r = s >> 1;
  const uint32_t row = 8u * (r >> 2) + 4u * (gq >> 1) + (r & 3u);
  const uint32_t col = 32u * t + 16u * (gq & 1u) + 8u * (s & 1u);
  return row * 128u + (((col >> 4) ^ swz_prefill<8>(row)) << 4) + (col & 15u);
}

// Decode, 16x16x32 K fragment (ds_read_b128) for k-step s: key row l % 16,
// chunk 4s + l / 16.  Score tile t adds 16 rows.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t decode_k_read(uint32_t lane, uint32_t s) {
  const uint32_t r = lane & 15u;
  return r * SLOTS * 16u + (((4u * s + (lane >> 4)) ^ swz_decode_k<SLOTS>(r)) << 4);
}
// Decode V^T fragment by ds_read_b64_tr_b16, half hf, value tile t: lane
// (gq = l/16, s = l%16) addresses key row 16hf + 4gq + s/4 at value columns
// 16t + 4(s%4) .. +3.
template <int SLOTS>
SDPA_LAYOUT_FN uint32_t decode_vt_read(uint32_t lane, uint32_t hf, uint32_t t) {
  const uint32_t gq = lane >> 4, s = lane & 15u;
  const uint32_t r = 16u * hf + 4u * gq + (s >> 2);
  const uint32_t col = 16u * t + 4u * (s & 3u);
  return r * SLOTS * 16u + (((col >> 3) ^ swz_decode<SLOTS>(r)) << 4) + ((col & 7u) << 1);
}

}  // namespace sdpa

#undef SDPA_LAYOUT_FN
