// Device-side building blocks shared by the grouped 4-bit GEMM kernels (gfx950).
//
//  * 16x16x32 MFMA wrappers (fp16 operands for NF4, bf16 for MXFP4; fp32 accumulate)
//  * the NF4 table and its v_perm lookup (4-bit code -> fp16 in registers)
//  * MXFP4 decode through the gfx950 scaled fp4 -> bf16 conversion
//  * bf16 -> fp16 activation conversion with the fp16 range check
//  * the in-workgroup prefix sum of `sizes` and the work-unit lookup
//
// The method these kernels implement ("grouped-nf4-gemm 0.33.1", opening
// description): 4-bit codes go through a 16-value table, are multiplied by their
// block scale, products are summed in fp32 and results are rounded to bf16; one
// launch covers every routed expert.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geg_launch.hpp"

namespace geg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));


// Device error word bits (mirrors GEG_DEVERR_* in include/geg.h).
constexpr uint32_t kErrNegativeSize = 0x1u;
constexpr uint32_t kErrSizesExceedM = 0x2u;
constexpr uint32_t kErrFp16Range = 0x4u;
constexpr uint32_t kErrBadExpertId = 0x8u;
constexpr uint32_t kErrNonFinite = 0x10u;   // W4A8: an activation is inf or NaN

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value {hi, lo}.
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ------------------------------------------------------------------ MFMA
// D(16x16, fp32) += A(16x32) . B(32x16). Lane l supplies A row (l % 16) and B
// column (l % 16), each with 8 contraction slots in group (l / 16); it receives
// D column (l % 16), rows 4*(l/16) .. +3. Only the pairing of A and B slots
// matters for the result, so the kernels may assign any k to a slot as long as
// A and B agree.
template <Fmt F>
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c);
template <>
__device__ __forceinline__ f32x4 mfma16<NF4>(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<MXFP4>(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ NF4 table
// NormalFloat-4 values, index 0..15, as fp32 bit patterns (QLoRA, Dettmers et al.
// 2023, appendix E; the table bitsandbytes stores for its 4-bit layout).
__device__ __forceinline__ float nf4_value(int i) {
  constexpr uint32_t bits[16] = {
      0xBF800000u, 0xBF3239B1u, 0xBF066B30u, 0xBECA32A0u, 0xBE91A24Du, 0xBE3D353Fu,
      0xBDBA7871u, 0x00000000u, 0x3DA2FAFFu, 0x3E24CAE3u, 0x3E7C04DDu, 0x3EAD033Au,
      0x3EE1A4B8u, 0x3F1007ABu, 0x3F3913B3u, 0x3F800000u};
  return __builtin_bit_cast(float, bits[i]);
}

// A 16-entry table of 16-bit values arranged for byte lookups with v_perm:
// lo[q] holds the low bytes of entries 4q..4q+3, hi[q] their high bytes.
struct Lut16 {
  uint32_t lo[4];
  uint32_t hi[4];
};

// Build the lookup table from 16 fp16 values packed two per dword (entry 2i in
// the low half of p[i]).
__device__ __forceinline__ Lut16 lut_from_pairs(const uint32_t p[8]) {
  Lut16 t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// fp32 product T * scale. The empty asm keeps the product in a register as an
// fp32 value: without it the compiler fuses multiply and fp16 conversion into a
// mixed-precision fma with a +0 addend, which turns a -0.0 product into +0.0.
__device__ __forceinline__ float nf4_times(int i, float scale) {
  float v = nf4_value(i) * scale;
  asm("" : "+v"(v));
  return v;
}

// Quarter j (entries 4j .. 4j+3) of the table of fp16 T[i] * scale (fp32
// product, one rounding to nearest even): fills lo[j] and hi[j].
__device__ __forceinline__ void nf4_scaled_lut_quarter(float scale, int j, Lut16& t) {
  uint32_t p[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f16x2 v;
    v[0] = (_Float16)nf4_times(4 * j + 2 * i, scale);
    v[1] = (_Float16)nf4_times(4 * j + 2 * i + 1, scale);
    p[i] = __builtin_bit_cast(uint32_t, v);
  }
  t.lo[j] = perm(p[1], p[0], 0x06040200u);
  t.hi[j] = perm(p[1], p[0], 0x07050301u);
}

// {fp16(ta * s), fp16(tb * s)}: exact product, one rounding to nearest even,
// one mixed-precision fma per value (the +0 addend can turn a -0.0 product into
// +0.0, which no sum of products can tell apart).
__device__ __forceinline__ uint32_t f16x2_times(float ta, float tb, float s) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "=v"(d) : "s"(ta), "v"(s));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(d) : "s"(tb), "v"(s));
  return d;
}

// The same quarter with f16x2_times (two VALU instructions per pair instead of
// three). For the GEMM kernels, whose decoded weights only enter sums.
__device__ __forceinline__ void nf4_scaled_lut_quarter_mix(float scale, int j, Lut16& t) {
  uint32_t p[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    p[i] = f16x2_times(nf4_value(4 * j + 2 * i), nf4_value(4 * j + 2 * i + 1), scale);
  t.lo[j] = perm(p[1], p[0], 0x06040200u);
  t.hi[j] = perm(p[1], p[0], 0x07050301u);
}

// fp16 of T[i] * scale for i = 0..15 (fp32 product, one rounding to nearest even).
__device__ __forceinline__ Lut16 nf4_scaled_lut(float scale) {
  Lut16 t;
#pragma unroll
  for (int j = 0; j < 4; ++j) nf4_scaled_lut_quarter(scale, j, t);
  return t;
}

// Look up four 4-bit indices (one per byte): s7 = idx & 7 per byte and
// sel = 0x03020100 | 4 * (bit 3 of each byte). Returns the low bytes and the
// high bytes of the four entries.
__device__ __forceinline__ void lut_lookup4(const Lut16& t, uint32_t s7, uint32_t sel,
                                            uint32_t& lo, uint32_t& hi) {
  lo = perm(perm(t.lo[3], t.lo[2], s7), perm(t.lo[1], t.lo[0], s7), sel);
  hi = perm(perm(t.hi[3], t.hi[2], s7), perm(t.hi[1], t.hi[0], s7), sel);
}

// Decode 8 NF4 codes from one dword of packed bytes (byte b holds k = 2b in its
// high nibble and k = 2b+1 in its low nibble) into 8 fp16 values in the slot
// order k = [0, 2, 4, 6, 1, 3, 5, 7] (the NF4 slot order): out[0] = {k0, k2},
// out[1] = {k4, k6}, out[2] = {k1, k3}, out[3] = {k5, k7}.
// The even-k half of nf4_decode8: {k0, k2}, {k4, k6} (high nibbles).
__device__ __forceinline__ u32x2 nf4_decode8_even(const Lut16& t, uint32_t x) {
  const uint32_t s7e = (x >> 4) & 0x07070707u;
  const uint32_t sele = ((x >> 5) & 0x04040404u) | 0x03020100u;
  uint32_t lo, hi;
  lut_lookup4(t, s7e, sele, lo, hi);
  return u32x2{perm(hi, lo, 0x05010400u), perm(hi, lo, 0x07030602u)};
}

// The odd-k half of nf4_decode8: {k1, k3}, {k5, k7} (low nibbles).
__device__ __forceinline__ u32x2 nf4_decode8_odd(const Lut16& t, uint32_t x) {
  const uint32_t s7o = x & 0x07070707u;
  const uint32_t selo = ((x >> 1) & 0x04040404u) | 0x03020100u;
  uint32_t lo, hi;
  lut_lookup4(t, s7o, selo, lo, hi);
  return u32x2{perm(hi, lo, 0x05010400u), perm(hi, lo, 0x07030602u)};
}

__device__ __forceinline__ u32x4 nf4_decode8(const Lut16& t, uint32_t x) {
  const u32x2 e = nf4_decode8_even(t, x);
  const u32x2 o = nf4_decode8_odd(t, x);
  return u32x4{e[0], e[1], o[0], o[1]};
}

// The same with the selector constants passed in registers (m4 = 0x04040404,
// base = 0x03020100, made opaque by the caller): the mask and the merge then fold
// into one and-or per four codes.
__device__ __forceinline__ u32x4 nf4_decode8(const Lut16& t, uint32_t x, uint32_t m4, uint32_t base) {
  uint32_t lo, hi;
  lut_lookup4(t, (x >> 4) & 0x07070707u, ((x >> 5) & m4) | base, lo, hi);
  const uint32_t e0 = perm(hi, lo, 0x05010400u), e1 = perm(hi, lo, 0x07030602u);
  lut_lookup4(t, x & 0x07070707u, ((x >> 1) & m4) | base, lo, hi);
  return u32x4{e0, e1, perm(hi, lo, 0x05010400u), perm(hi, lo, 0x07030602u)};
}

// Selector constants for the and-or form above, hidden from constant folding.
__device__ __forceinline__ void nf4_selector_consts(uint32_t& m4, uint32_t& base) {
  m4 = 0x04040404u;
  base = 0x03020100u;
  asm volatile("" : "+v"(base));
  asm volatile("" : "+s"(m4));
}

// ------------------------------------------------------------------ NF4 byte table (LDS)
// The decode-class kernels look codes up a byte at a time in LDS instead of in
// registers. Entry v (a code byte) is the fp16 pair {T[v >> 4], T[v & 15]}, i.e.
// the weights k = 2b and 2b + 1 of byte b in natural order. The 256 entries are
// stored C times, interleaved (copy c of entry v is word C v + c), and lane l
// reads copy l % C. LDS serves a 32-bit read 32 lanes at a time, so with C = 32
// or 64 the lanes of one pass hit 32 different banks whatever the codes: a
// lookup is one conflict-free read. Its byte address {4 (l % C), code byte} is
// one v_perm for C = 64 (a 64 KiB table) and a bit-field extract plus a
// shift-or for C = 32 (32 KiB). About 0.5 or 1 vector instruction per code
// against about 3 for the register table.
template <int C>
constexpr int nf4_byte_lut_words() { return 256 * C; }
constexpr int kNf4ByteLutWords = 256 * 64;

// Fill the table (every thread of an NT-thread workgroup takes part; the caller
// places a barrier before the first lookup). Word quad q = NT i + t holds copies
// 4 (q % (C / 4)) .. +3 of entry q / (C / 4); consecutive threads fill
// consecutive quads, so the stores are conflict-free.
template <int C = 64, int NT = kThreads>
__device__ __forceinline__ void nf4_byte_lut_fill(uint32_t* lut) {
  static_assert(C == 32 || C == 64, "32 or 64 copies");
  constexpr int Q = C / 4;                    // quads per entry
  constexpr int kQuads = 256 * Q;
  static_assert(NT % (16 * Q) == 0 && kQuads % NT == 0, "threads must tile the entries evenly");
  constexpr int R = NT / (16 * Q);            // high-nibble values per pass
  const int t = threadIdx.x;
  // entry of quad NT i + t: (NT i + t) / Q = 16 R i + t / Q, so its low nibble is
  // (t / Q) % 16 and its high nibble R i + t / (16 Q)
  const int lo = (t / Q) & 15, sub = t / (16 * Q);
  _Float16 lv = (_Float16)0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (lo == j) lv = (_Float16)nf4_value(j);
  const uint32_t high_half = (uint32_t)__builtin_bit_cast(uint16_t, lv) << 16;
#pragma unroll
  for (int i = 0; i < kQuads / NT; ++i) {
    uint32_t low_half = __builtin_bit_cast(uint16_t, (_Float16)nf4_value(R * i));
#pragma unroll
    for (int r = 1; r < R; ++r)
      if (sub == r) low_half = __builtin_bit_cast(uint16_t, (_Float16)nf4_value(R * i + r));
    const uint32_t v = high_half | low_half;
    *reinterpret_cast<u32x4*>(lut + 4 * (NT * i + t)) = u32x4{v, v, v, v};
  }
}

// Byte offset of the lane's copy (kept in the low bits of the address).
template <int C = 64>
__device__ __forceinline__ uint32_t nf4_byte_lut_lane(int lane) { return 4u * (uint32_t)(lane % C); }

// Decode 8 NF4 codes from one dword of packed bytes (byte b holds k = 2b in its
// high nibble and k = 2b+1 in its low nibble) to 8 fp16 values in natural k
// order: out[b] = {k 2b, k 2b+1}.
template <int C = 64>
__device__ __forceinline__ u32x4 nf4_byte_lut_decode8(const uint32_t* lut, uint32_t x, uint32_t lane_off) {
  u32x4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t addr;
    if constexpr (C == 64)
      addr = perm(x, lane_off, 0x0C0C0400u | ((uint32_t)b << 8));   // {lane_off, byte b of x, 0, 0}
    else
      addr = (__builtin_amdgcn_ubfe(x, 8 * b, 8) << 7) | lane_off;  // 128 * code byte + 4 (lane % 32)
    r[b] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr);
  }
  return r;
}

// ------------------------------------------------------------------ MXFP4 decode
// e8m0 byte -> fp32 scale 2^(x-127): normal for 1..254, 2^-127 (subnormal) for 0,
// NaN for 255.
__device__ __forceinline__ float e8m0_to_f32(uint32_t x) {
  uint32_t bits = x == 0 ? 0x00400000u : (x == 255 ? 0x7FC00000u : (x << 23));
  return __builtin_bit_cast(float, bits);
}

// Decode 8 e2m1 codes (byte b: k = 2b in the low nibble, 2b+1 in the high nibble)
// to bf16 times `scale`, natural k order, with the gfx950 scaled fp4 conversion.
__device__ __forceinline__ u32x4 mxfp4_decode8(uint32_t x, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 3));
  return r;
}

// ------------------------------------------------------------------ activations
// 8 bf16 (4 dwords, natural order) -> 8 fp16 in the NF4 slot order, round to nearest
// even (exact for 2^-14 <= |x| <= 65504). `range` accumulates |h| per half as
// integers so that an overflow to inf can be flagged afterwards.
__device__ __forceinline__ u32x4 bf16x8_to_f16_slots(const u32x4& x, uint32_t& range) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, x[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, x[i] & 0xFFFF0000u);
  }
  constexpr int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h;
    h[0] = (_Float16)v[order[2 * i]];
    h[1] = (_Float16)v[order[2 * i + 1]];
    r[i] = __builtin_bit_cast(uint32_t, h);
    u16x2 m = __builtin_bit_cast(u16x2, r[i] & 0x7FFF7FFFu);
    u16x2 acc = __builtin_bit_cast(u16x2, range);
    range = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(acc, m));
  }
  return r;
}

// Same, natural order (used where the other operand keeps natural order).
__device__ __forceinline__ u32x4 bf16x8_to_f16(const u32x4& x, uint32_t& range) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h;
    h[0] = (_Float16)__builtin_bit_cast(float, x[i] << 16);
    h[1] = (_Float16)__builtin_bit_cast(float, x[i] & 0xFFFF0000u);
    r[i] = __builtin_bit_cast(uint32_t, h);
    u16x2 m = __builtin_bit_cast(u16x2, r[i] & 0x7FFF7FFFu);
    u16x2 acc = __builtin_bit_cast(u16x2, range);
    range = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(acc, m));
  }
  return r;
}

// 4 bf16 (2 dwords) -> 4 fp16, natural order, with the same range tracking.
__device__ __forceinline__ u32x2 bf16x4_to_f16(const u32x2& x, uint32_t& range) {
  const u32x4 r = bf16x8_to_f16(u32x4{x[0], x[1], 0u, 0u}, range);
  return u32x2{r[0], r[1]};
}

// Gated unit of the fused expert block: silu(g) * u with silu(x) = x / (1 + e^-x),
// in fp32 with the hardware exponential and reciprocal (about 1 ulp each; the
// result is rounded to bf16). e^-x overflowing to inf for very negative g gives
// a reciprocal of 0 and a result of -0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// The value held by the neighbouring lane (l ^ 1): a DPP quad permutation.
__device__ __forceinline__ float lane_pair_swap(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ bool range_overflowed(uint32_t range) {
  return (range & 0xFFFFu) >= 0x7C00u || (range >> 16) >= 0x7C00u;
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 h;
  h[0] = (__bf16)a;
  h[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// ------------------------------------------------------------------ routing plan
// Each workgroup rebuilds, in LDS, the exclusive prefix sum of the per-expert row
// counts ("grouped-nf4-gemm releases", v0.2.6: rows are grouped by expert and
// sizes[e] counts expert e's rows) and a prefix sum of work units per expert.
// Negative sizes count as 0 and offsets are clamped to M, so no unit ever
// touches a row outside [0, M); both conditions are flagged in the error word.
// 8 consecutive fp32 values of a row (two 16-byte buffer loads; `ok` false or a
// record past the end reads zeros) as two bf16x8 MFMA operands: hi = bf16(v) and
// lo = bf16(v - hi), about 16 significant bits together (v multiplied by
// scale, then by 2^sexp, first).
struct Split8 {
  u32x4 hi, lo;
};
__device__ __forceinline__ Split8 load8_split(const __amdgpu_buffer_rsrc_t& R, uint32_t elem_off, bool ok,
                                              float scale = 1.0f, int sexp = 0) {
  const uint32_t b = (elem_off * 4u) | ((uint32_t)!ok << 31);   // bit 31: past every record
  const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(R, b, 0, 0);
  const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(R, b + 16u, 0, 0);
  Split8 s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v0 = __builtin_amdgcn_ldexpf(scale * __uint_as_float(i < 2 ? p[2 * i] : q[2 * i - 4]), sexp);
    const float v1 = __builtin_amdgcn_ldexpf(scale * __uint_as_float(i < 2 ? p[2 * i + 1] : q[2 * i - 3]), sexp);
    const uint32_t h = pack_bf16x2(v0, v1);
    s.hi[i] = h;
    s.lo[i] = pack_bf16x2(v0 - __uint_as_float(h << 16), v1 - __uint_as_float(h & 0xFFFF0000u));
  }
  return s;
}

struct Plan {
  int32_t off[kMaxExperts + 1];    // clamped row offsets
  int32_t upre[kMaxExperts + 1];   // exclusive prefix of work units
};

// Inclusive prefix sum over the 64 lanes of a wavefront, with unsigned adds
// that saturate at 2^32 - 1. DPP row shifts by 1, 2, 4 and 8 scan each row of 16
// lanes; row broadcast 15 then adds row 0's total to row 1 and row 2's to row 3,
// and row broadcast 31 adds the total of rows 0-1 to rows 2-3. Lanes whose
// source is outside the row (or rows the mask leaves out) add 0.
__device__ __forceinline__ uint32_t wave_scan_sat(uint32_t v) {
  auto step = [](uint32_t x, uint32_t t) { return __builtin_elementwise_add_sat(x, t); };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

struct NoOverlap {
  __device__ void operator()() const {}
};

// Fill plan.off / plan.upre (wavefront 0 scans 64 experts at a time, the other
// wavefronts wait at the barrier). `units(size)` gives the number of work units
// of an expert with `size` (clamped) rows. `overlap()` runs on every thread while
// the first 64 sizes are in flight (a kernel's LDS set-up, say). Returns the
// total number of units. Row counts are clamped to M + 1 <= 2^31 before the
// scan, so the saturating 32-bit sums are exact up to the point where they pass
// M, and offsets are clamped to M after it.
// `off` and `upre` each hold E + 1 entries in LDS.
template <typename UnitFn, typename Overlap = NoOverlap>
__device__ int32_t build_plan(int32_t* off, int32_t* upre, const int32_t* __restrict__ sizes, int E,
                              int64_t M, uint32_t* err_word, UnitFn units, Overlap overlap = Overlap{}) {
  const int t = threadIdx.x;
  int32_t first = 0;
  if (t < 64 && t < E) first = sizes[t];
  overlap();
  if (t < 64) {
    const int lane = t;
    const uint32_t m = (uint32_t)M;
    uint32_t run = 0, urun = 0, err = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int32_t raw = base == 0 ? first : (e < E ? sizes[e] : 0);
      if (raw < 0) {
        err |= kErrNegativeSize;
        raw = 0;
      }
      const uint32_t s = min((uint32_t)raw, m + 1u);
      const uint32_t incl = __builtin_elementwise_add_sat(wave_scan_sat(s), run);
      const uint32_t lo = min(incl - s, m), hi = min(incl, m);
      const uint32_t uc = e < E ? (uint32_t)units((int32_t)(hi - lo)) : 0u;
      const uint32_t uincl = wave_scan_sat(uc) + urun;
      if (e < E) {
        off[e] = (int32_t)lo;
        upre[e] = (int32_t)(uincl - uc);
      }
      run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      urun = (uint32_t)__builtin_amdgcn_readlane((int)uincl, 63);
    }
    if (lane == 0) {
      off[E] = (int32_t)min(run, m);
      upre[E] = (int32_t)urun;
      if (run > m) err |= kErrSizesExceedM;
    }
    if (err) atomicOr(err_word, err);
  }
  __syncthreads();
  return upre[E];
}

// Two work lists in one scan: units(size, c) gives expert e's units of class c
// (0 or 1); upre0 / upre1 receive the exclusive prefix of each class over the
// experts. The tiled kernel runs every class-0 unit before any class-1 unit.
// Returns the class-0 total; upre1[E] holds the class-1 total.
template <typename UnitFn>
__device__ int32_t build_plan2(int32_t* off, int32_t* upre0, int32_t* upre1, const int32_t* __restrict__ sizes,
                               int E, int64_t M, uint32_t* err_word, UnitFn units) {
  const int t = threadIdx.x;
  if (t < 64) {
    const int lane = t;
    const uint32_t m = (uint32_t)M;
    uint32_t run = 0, urun0 = 0, urun1 = 0, err = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int32_t raw = e < E ? sizes[e] : 0;
      if (raw < 0) {
        err |= kErrNegativeSize;
        raw = 0;
      }
      const uint32_t s = min((uint32_t)raw, m + 1u);
      const uint32_t incl = __builtin_elementwise_add_sat(wave_scan_sat(s), run);
      const uint32_t lo = min(incl - s, m), hi = min(incl, m);
      const uint32_t u0 = e < E ? (uint32_t)units((int32_t)(hi - lo), 0) : 0u;
      const uint32_t u1 = e < E ? (uint32_t)units((int32_t)(hi - lo), 1) : 0u;
      const uint32_t i0 = wave_scan_sat(u0) + urun0;
      const uint32_t i1 = wave_scan_sat(u1) + urun1;
      if (e < E) {
        off[e] = (int32_t)lo;
        upre0[e] = (int32_t)(i0 - u0);
        upre1[e] = (int32_t)(i1 - u1);
      }
      run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      urun0 = (uint32_t)__builtin_amdgcn_readlane((int)i0, 63);
      urun1 = (uint32_t)__builtin_amdgcn_readlane((int)i1, 63);
    }
    if (lane == 0) {
      off[E] = (int32_t)min(run, m);
      upre0[E] = (int32_t)urun0;
      upre1[E] = (int32_t)urun1;
      if (run > m) err |= kErrSizesExceedM;
    }
    if (err) atomicOr(err_word, err);
  }
  __syncthreads();
  return upre0[E];
}

template <typename UnitFn, typename Overlap = NoOverlap>
__device__ int32_t build_plan(Plan& p, const int32_t* __restrict__ sizes, int E, int64_t M,
                              uint32_t* err_word, UnitFn units, Overlap overlap = Overlap{}) {
  return build_plan(p.off, p.upre, sizes, E, M, err_word, units, overlap);
}

// Expert owning work unit u (uniform over the wavefront, which must be whole):
// the largest e with upre[e] <= u. upre is nondecreasing with upre[0] = 0, so
// that e is the number of e' in [1, E) with upre[e'] <= u, counted 64 experts per
// ballot (experts with no units share the next expert's upre and are passed).
__device__ __forceinline__ int find_expert(const int32_t* upre, int E, int32_t u) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int base = 1; base < E; base += 64) {
    const int e = base + lane;
    const bool le = e < E && upre[e] <= u;
    const uint64_t b = __ballot(le);
    cnt += __builtin_popcountll(b);
    if (b != ~0ull) break;   // the rest lie past u
  }
  return cnt;
}

__device__ __forceinline__ int find_expert(const Plan& p, int E, int32_t u) { return find_expert(p.upre, E, u); }

}  // namespace geg
