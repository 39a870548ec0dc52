// Tiled (prefill-shape) path of the grouped 4-bit GEMM.
//
// One persistent launch walks every 256x256 output tile of every expert that has
// more rows than the skinny path takes. Per 64-wide K stage a workgroup stages
// its activation tile (NF4: from the row-scaled fp16 copy a prior pass made) and decodes
// its 256 weight rows once into LDS: codes through the 16-value table, times the
// block scale, so the decode is shared by all 256 rows of the tile
// ("grouped-nf4-gemm 0.33.1", opening description: table decode in registers,
// blockwise scaling, fp32 accumulation, bf16 epilogue, no dequantised copy of an
// expert in memory). Eight wavefronts (two per SIMD) each own a 128x64 block of
// the tile and run 8x4 16x16x32 MFMAs per 32 k.
//
// Pipeline: LDS holds two stages. A stage runs as 16 groups of 4 MFMAs; each
// group also issues one LDS operand read three groups ahead and one slice of the
// next stage's staging work (activation rows into the other buffer, or weight
// decode), so LDS latency and VALU work hide under the MFMAs. Raw activations
// are loaded one stage ahead and raw codes two stages ahead, into registers. A
// barrier after the staging groups publishes the next buffer, which lets the
// last groups read the next stage's first operands early.
// LDS rows are 128 B (64 halves) with the 16-byte chunk index XOR-swizzled by
// the row, which makes both the row-wise stores and the MFMA operand reads
// (16 rows, one chunk each) free of bank conflicts.
//
// Tiles are assigned XCD-aware: workgroup b runs on XCD b % 8, and each XCD
// takes a contiguous run of tiles (same expert and row block, neighbouring column
// blocks), so an activation block is fetched into one XCD's L2 and reused there.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int BM = 256;  // rows (routed tokens) per tile
constexpr int BN = 256;  // columns (weight rows) per tile
constexpr int BK = 64;   // k per stage
constexpr int kXcds = 8;
constexpr int kTileThreads = 512;
constexpr int kTileWaves = kTileThreads / 64;
constexpr int kEpiLd = 64 + 8;  // epilogue row stride in halves (144 B)
constexpr int kLdB = BN + 16;   // dgrad weight-tile row stride in halves (544 B)

// LDS of one workgroup: two stages of activation and weight tiles, or the
// epilogue's result blocks. Forward weight tiles hold 256 weight rows of 64 k;
// dgrad weight tiles hold the stage's 64 weight rows (the contraction) of 256
// output columns, both as written by the staging threads.
template <bool DG>
union TileLds {
  struct {
    uint16_t a[2][BM * BK];
    uint16_t b[2][DG ? BK * kLdB : BN * BK];
  };
  uint16_t epi[kTileWaves][128 * kEpiLd];  // per-wavefront bf16 result block
};

// Half-element offset of 16-byte chunk `chunk` (0..7) of LDS row `row` (rows are
// 128 B). A 16-byte LDS read serves two 8-lane groups per clock over the 64
// banks (lane groups {0,3}, {1,2}, {4,7} and {5,6}, measured with the bank
// conflict counter); with the chunk XORed by row % 8, the two groups of an MFMA
// operand read (rows r..r+7 at chunk c, rows r+8..r+15 at chunk c^1, or the
// reverse) cover all 16 bank quads, so operand reads run at the full 256 B per
// clock. Row-wise stores (8 lanes per clock) stay conflict-free too. Rows 16
// apart differ by a fixed offset (one address register per operand stream).
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

// dgrad weight tile: rows of 256 output columns plus 16 halves of padding
// (544 B), one per weight row of the stage (contraction slot s, 0..63) at row
// position dg_pos(s). The MFMA operand needs the transpose (8 contraction rows of
// one output column per lane), which gfx950's transposing LDS read provides:
// within each 16-lane group, lane L reads 8 bytes, and lane i receives element
// i % 4 of the reads of lanes 4 j + i / 4, j = 0..3 (measured). So lane L of a
// group reads slot s0 + L / 4 at columns c0 + 4 (L % 4); lane i then holds
// column c0 + i of slots s0..s0+3. A 32-lane pass reads slots 8 g + 4 h + i
// (g = 0, 1; i = 0..3) of one column block: dg_pos swaps bits 2 and 3 of the
// slot so that they are 8 consecutive positions, which the 544-byte stride
// spreads over the 8 disjoint 32-byte bank groups; column blocks and substeps
// are plain offsets. (The 16-byte stores of 16 consecutive slots meet 2-way.)
__device__ __forceinline__ int dg_pos(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

// dgrad output column of MFMA column c (0..15) within a 16-column block: NF4
// stages each 8-column chunk in the slot order [0, 2, 4, 6, 1, 3, 5, 7].
__device__ __forceinline__ int dg_col(int c) { return (c & 8) | ((c & 3) << 1) | ((c >> 2) & 1); }

// Where a tile's operands come from. Loads go through buffer resources whose
// record count bounds every access: rows past the expert's last row and weight
// rows past N read as zeros, and a load switched off (count 0) reads nothing.
struct TileSrc {
  const void* a;              // activation rows of the tile
  const void* w;              // packed codes of the tile's weight rows
  const void* s;              // their scales
  int32_t na, nw, ns;         // bytes readable from each
  uint32_t a_off;             // this lane's activation byte offset (row, chunk) at stage 0
  uint32_t a_rows8;           // bytes between activation rows 8 apart
  uint32_t w_off;             // this thread's code byte offset at stage 0
  uint32_t w_step;            // code bytes per stage
  uint32_t s_off;             // this thread's scale byte offset at stage 0
  uint32_t s_step;            // scale bytes per stage
};

__device__ __forceinline__ int32_t clamp_bytes(int64_t bytes) {
  return bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes;
}

// Raw (undecoded) stage data held in registers between its global load and its
// LDS store: activations are single-buffered, codes double-buffered (they come
// from HBM and get two stages of latency; activations are mostly L2 hits).
struct RawA {
  u32x4 v[4];      // rows 32w + 8i + lane/8, 8 bf16 at chunk lane%8
};
struct RawB {
  u32x4 c;         // 32 codes of weight row t/2, k in [k0 + 32 (t%2), +32)
  float s;         // NF4: absmax of the row's 64-block; MXFP4: e8m0 byte of the 32-block
};

// Operand sources of the tile (expert e, rows row0.., output columns o0..),
// starting at contraction stage st0 (a piece of a split tile: every base moves
// st0 stages on and every window ends where the tile's does, so the piece reads
// like a tile of the remaining contraction).
// Forward: out = A . W^T contracts over K; thread t stages codes of weight row t/2
// (32 k per stage half t%2). dgrad: dX = dY . W contracts over N; thread t stages
// weight row n = t%64 of the stage's 64, columns o0 + 32 (t/64) .. +32.
template <Fmt F, bool DG>
__device__ __forceinline__ TileSrc tile_src(const GemmArgs& g, int e, int64_t row0, int rows,
                                            int64_t o0, int wave, int lane, int st0) {
  const int64_t K = g.K, N = g.N;
  const int64_t C = DG ? N : K;   // contraction length = activation row length
  const int64_t k0 = (int64_t)st0 * BK;
  TileSrc t;
  // NF4 reads the fp16 copy of the activations (already in the NF4 slot order).
  t.a = (F == NF4 ? g.a16 : g.a) + row0 * C + k0;
  t.na = clamp_bytes((int64_t)rows * C * 2 - k0 * 2);
  t.a_off = (uint32_t)(((32 * wave + (lane >> 3)) * C + 8 * (lane & 7)) * 2);
  t.a_rows8 = (uint32_t)(8 * C * 2);
  const int tid = threadIdx.x;
  if constexpr (DG) {
    // stage st0 starts at weight row k0
    t.w = g.wq + (int64_t)e * N * (K >> 1) + k0 * (K >> 1);
    t.nw = clamp_bytes((N - k0) * (K >> 1));
    const int n = tid & 63, kc = tid >> 6;
    const int64_t kcol = o0 + 32 * kc;    // past K: never stored
    t.w_off = (uint32_t)(n * (K >> 1) + (kcol >> 1));
    t.w_step = (uint32_t)(BK * (K >> 1));
    if constexpr (F == NF4) {
      t.s = reinterpret_cast<const float*>(g.scales) + ((int64_t)e * N + k0) * (K >> 6);
      t.ns = clamp_bytes((N - k0) * (K >> 6) * 4);
      t.s_off = (uint32_t)((n * (K >> 6) + (kcol >> 6)) * 4);
      t.s_step = (uint32_t)(BK * (K >> 6) * 4);
    } else {
      // the thread's 32 columns are exactly one 32-block of the weight row
      t.s = reinterpret_cast<const uint8_t*>(g.scales) + ((int64_t)e * N + k0) * (K >> 5);
      t.ns = clamp_bytes((N - k0) * (K >> 5));
      t.s_off = (uint32_t)(n * (K >> 5) + (kcol >> 5));
      t.s_step = (uint32_t)(BK * (K >> 5));
    }
  } else {
    // stage st0 starts k0 into every weight row (st0 scales of a 64-block each,
    // or 2 st0 of a 32-block)
    const int64_t nrows = min<int64_t>(BN, N - o0);
    const int64_t wrow0 = (int64_t)e * N + o0;
    t.w = g.wq + wrow0 * (K >> 1) + (k0 >> 1);
    t.nw = clamp_bytes(nrows * (K >> 1) - (k0 >> 1));
    if constexpr (F == NF4) {
      t.s = reinterpret_cast<const float*>(g.scales) + wrow0 * (K >> 6) + st0;
      t.ns = clamp_bytes((nrows * (K >> 6) - st0) * 4);
    } else {
      t.s = reinterpret_cast<const uint8_t*>(g.scales) + wrow0 * (K >> 5) + 2 * (int64_t)st0;
      t.ns = clamp_bytes(nrows * (K >> 5) - 2 * (int64_t)st0);
    }
    t.w_off = (uint32_t)((tid >> 1) * (K >> 1) + 16 * (tid & 1));
    t.w_step = BK / 2;
    t.s_off = (uint32_t)(F == NF4 ? (tid >> 1) * (K >> 6) * 4 : (tid >> 1) * (K >> 5) + (tid & 1));
    t.s_step = F == NF4 ? 4 : 2;
  }
  return t;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_on(const void* base, int32_t n, bool on) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, on ? n : 0, 0x00020000);
}

// Activations of stage st, coalesced: 8 lanes cover one row's 128 bytes; piece
// i holds rows 8 i + lane/8 of the wavefront's 32.
__device__ __forceinline__ void load_a(RawA& r, const TileSrc& t, int st, bool on) {
  const __amdgpu_buffer_rsrc_t R = rsrc_on(t.a, t.na, on);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(R, t.a_off, (uint32_t)st * (BK * 2) + (uint32_t)i * t.a_rows8, 0);
}

// Piece i of load_a alone (one load per MFMA group keeps the vector memory
// path from bunching up).
__device__ __forceinline__ void load_a_piece(RawA& r, int i, const TileSrc& t, int st, bool on) {
  r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_on(t.a, t.na, on), t.a_off,
                                                 (uint32_t)st * (BK * 2) + (uint32_t)i * t.a_rows8, 0);
}

template <Fmt F>
__device__ __forceinline__ void load_b(RawB& r, const TileSrc& t, int st, bool on) {
  r.c = __builtin_amdgcn_raw_buffer_load_b128(rsrc_on(t.w, t.nw, on), t.w_off, (uint32_t)st * t.w_step, 0);
  const __amdgpu_buffer_rsrc_t S = rsrc_on(t.s, t.ns, on);
  if constexpr (F == NF4)
    r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(S, t.s_off, (uint32_t)st * t.s_step, 0));
  else
    r.s = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(S, t.s_off, (uint32_t)st * t.s_step, 0));
}

// One row chunk of raw activations -> LDS. With TAIL, chunks past the
// contraction length C are zeroed (NF4 forward has C % 64 == 0; MXFP4 can have a
// 32-wide tail and dgrad an 8-aligned one).
template <Fmt F, bool DG, bool TAIL>
__device__ __forceinline__ void store_a_piece(const RawA& r, int i, uint16_t* As, int64_t k0,
                                              int64_t C, int wave, int lane) {
  const int chunk = lane & 7;
  const int row = 32 * wave + 8 * i + (lane >> 3);
  u32x4 v = r.v[i];
  if constexpr (TAIL) v = k0 + 8 * chunk < C ? v : u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(&As[swz(row, chunk)]) = v;
}

// Decode state of a thread's weight row for one stage: the NF4 table scaled by
// the block's absmax, or the MXFP4 block scale (0 for a 32-wide piece past K).
template <Fmt F> struct BDec;
template <> struct BDec<NF4> { Lut16 lut; };
template <> struct BDec<MXFP4> { float sc; };

// Part j (0..3) of the decode state of stage k0 from the raw scale: NF4 builds
// table entries 4j .. 4j+3; MXFP4 converts the block scale at j = 0.
// dgrad (MXFP4): the thread's columns are one 32-block; columns past K are
// never stored and weight rows past N read zero codes and a zero scale byte.
template <Fmt F, bool DG = false>
__device__ __forceinline__ void b_setup(BDec<F>& d, int j, const RawB& r, int64_t k0, int64_t K) {
  if constexpr (F == NF4) {
    nf4_scaled_lut_quarter_mix(r.s, j, d.lut);
  } else if (j == 0) {
    const bool ok = DG || k0 + 32 * (threadIdx.x & 1) < K;
    d.sc = ok ? e8m0_to_f32(__builtin_bit_cast(uint32_t, r.s)) : 0.f;
  }
}

// NF4 slot of contraction offset j (0..7) within an 8-chunk: the activations of
// the NF4 path are stored in slot order [0, 2, 4, 6, 1, 3, 5, 7].
__device__ __forceinline__ int nf4_slot(int j) { return (j >> 1) | ((j & 1) << 2); }

// Four NF4 codes in flight (the even-k or the odd-k half of an 8-code piece):
// their v_perm selectors and the low bytes of their table entries. Byte b of
// the packed dword holds k = 2b in its high nibble and k = 2b + 1 in its low one.
struct NF4Half {
  uint32_t s7;   // index & 7 per byte
  uint32_t sel;  // 0x03020100 | 4 * (bit 3 of the index) per byte
  uint32_t lo;
};

// `m4` = 0x04040404 and `base` = 0x03020100, kept in registers so that the mask
// and the merge fold into one and-or.
template <bool EVEN>
__device__ __forceinline__ void nf4_half_select(uint32_t x, uint32_t m4, uint32_t base, NF4Half& h) {
  if constexpr (EVEN) {
    h.s7 = (x >> 4) & 0x07070707u;
    h.sel = ((x >> 5) & m4) | base;
  } else {
    h.s7 = x & 0x07070707u;
    h.sel = ((x >> 1) & m4) | base;
  }
}

__device__ __forceinline__ void nf4_half_lo(const Lut16& t, NF4Half& h) {
  h.lo = perm(perm(t.lo[3], t.lo[2], h.s7), perm(t.lo[1], t.lo[0], h.s7), h.sel);
}

// High bytes, then the four fp16 values as two slot-ordered pairs.
__device__ __forceinline__ u32x2 nf4_half_out(const Lut16& t, const NF4Half& h) {
  const uint32_t hi = perm(perm(t.hi[3], t.hi[2], h.s7), perm(t.hi[1], t.hi[0], h.s7), h.sel);
  return u32x2{perm(hi, h.lo, 0x05010400u), perm(hi, h.lo, 0x07030602u)};
}

// Staging step r (0..2) of the thread's weight piece q (its 8 codes r.c[q]):
// NF4 r = 0 selects the even-k codes and looks up their low bytes, r = 1
// finishes them and selects the odd-k codes, r = 2 finishes the piece and stores
// it; MXFP4 decodes and stores the whole piece at r = 0. Each step is 7-8 VALU
// instructions, so that two steps fit under the four MFMAs of a group.
// Forward: row t/2, chunk 4 (t%2) + q, one 16-byte store in slot order. dgrad:
// the codes are output columns 32 (t/64) + 8 q + j of weight row n = t%64, one
// 16-byte store into chunk 4 (t/64) + q of the weight row's LDS row `brow` (the
// row's contraction slot).
template <Fmt F, bool DG>
__device__ __forceinline__ void b_step(int q, int r, const RawB& rb, const BDec<F>& d, NF4Half& h,
                                       u32x2& even, uint16_t* Bs, int brow, uint32_t m4,
                                       uint32_t base) {
  const int t = threadIdx.x;
  const int bo = DG ? dg_pos(brow) * kLdB + (4 * (t >> 6) + q) * 8 : swz(t >> 1, 4 * (t & 1) + q);
  if constexpr (F == NF4) {
    const uint32_t x = rb.c[q];
    if (r == 0) {
      nf4_half_select<true>(x, m4, base, h);
      nf4_half_lo(d.lut, h);
    } else if (r == 1) {
      even = nf4_half_out(d.lut, h);
      nf4_half_select<false>(x, m4, base, h);
    } else {
      nf4_half_lo(d.lut, h);
      const u32x2 odd = nf4_half_out(d.lut, h);
      *reinterpret_cast<u32x4*>(&Bs[bo]) = u32x4{even[0], even[1], odd[0], odd[1]};
    }
  } else if (r == 0) {
    *reinterpret_cast<u32x4*>(&Bs[bo]) = mxfp4_decode8(rb.c[q], d.sc);   // k = 8q + j, natural order
  }
}

__device__ __forceinline__ u32x4 lds_frag(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ u32x2 lds_tr4(lds_u16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// A wavefront's weight-operand read offsets (halves, from a stage buffer).
// Forward: the fragment of substep s and column block j is one 16-byte read at
// off ^ 32 s + 16 j rows. dgrad: two transposing reads (contraction slots
// 8 g + 0..3 and 8 g + 4..7 of the substep, g = lane / 16) per column block j,
// at off[h] + 16 j (+ 32 rows in substep 1).
template <bool DG> struct BRd { uint32_t off; };
template <> struct BRd<true> { uint32_t off[2]; };

template <bool DG>
__device__ __forceinline__ u32x4 b_frag(const uint16_t* Bbuf, const BRd<DG>& br, int sub, int j) {
  if constexpr (DG) {
    lds_u16* p = (lds_u16*)const_cast<uint16_t*>(Bbuf);   // the stage buffer, as an LDS address
    const u32x2 lo = lds_tr4(p + br.off[0] + (sub * (32 * kLdB) + 16 * j));
    const u32x2 hi = lds_tr4(p + br.off[1] + (sub * (32 * kLdB) + 16 * j));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return lds_frag(Bbuf + (sub ? br.off ^ 32u : br.off) + 16 * BK * j);
  }
}

// Accumulator layout. With the weight fragment as the instruction's first
// operand and the activation fragment as its second (TR), block (i, j) comes out
// transposed: lane l holds row 16 i + l % 16, columns 16 j + 4 (l / 16) + q,
// q = 0..3, i.e. four adjacent outputs of one row (one row exponent, one 8-byte
// LDS write). The NF4 dgrad keeps the other order (lane l: rows
// 16 i + 4 (l / 16) + q, column 16 j + l % 16), because its MFMA columns are in
// the NF4 slot order and four adjacent ones are not adjacent outputs.
template <Fmt F, bool DG>
constexpr bool kTr = !(DG && F == NF4);

// The 4 MFMAs of one 16-row A fragment with the substep's 4 B fragments.
template <Fmt F, bool TR>
__device__ __forceinline__ void mfma_row(const u32x4& a, const u32x4 (&b)[4], f32x4 (&acc)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = TR ? mfma16<F>(b[j], a, acc[j]) : mfma16<F>(a, b[j], acc[j]);
}

// Operand registers carried from one stage into the next: the first substep's
// B fragments and its first three A fragments, read ahead of the stage.
struct Ops {
  u32x4 b[4];
  u32x4 a[3];
};

// One 64-k stage of the tile's main loop, in 16 groups of (up to) 4 MFMAs:
// groups 0-7 run substep 0 (k 0..31 of the stage), groups 8-15 substep 1. Each
// group issues its LDS operand read three groups ahead of use and a slice of the
// staging work, spread so that no group holds more than about two VALU
// instructions per MFMA: the MFMA pipe hides that much VALU work of the same
// wavefront, while a denser burst stalls it.
//   groups 0-3    store the next stage's activation rows (from registers)
//   groups 0-1    finish the next stage's decode table (entries 8-15)
//   groups 2-13   decode and store the next stage's weights, piece q in groups
//                 2 + 3q .. 4 + 3q
//   barrier Y after group 13 publishes the next stage's buffers; groups 14-15
//   read its first operands ahead and build the first half of the table of the
//   stage after it (entries 0-7, from the raw scale already in registers)
// Y is the stage's only barrier: every read of the current buffers is issued by
// group 12 and has completed when a wavefront passes Y, so the next stage's
// staging may overwrite them as soon as all wavefronts are past it.
// H = number of the wavefront's 64-row halves that hold rows of the expert.
template <Fmt F, bool DG, bool TAIL, int H, int P>
__device__ __forceinline__ void tile_stage(TileLds<DG>& L, const TileSrc& src, int64_t C, int64_t K,
                                           int st, int nst, int wave, int lane, int brow,
                                           RawA& ra, RawB (&rb)[2], BDec<F>& dec, Ops& ops,
                                           f32x4 (&acc)[8][4], uint32_t aoff, const BRd<DG>& br,
                                           uint32_t m4, uint32_t base) {
  constexpr int cur = P, nxt = P ^ 1;   // st % 2 == P
  const int64_t k1 = (int64_t)(st + 1) * BK;
  // Substep 1 reads chunk 4 + c where substep 0 reads chunk c: the swizzled
  // chunk differs in bit 2, i.e. the half offset differs in bit 5.
  const uint16_t* A0 = L.a[cur] + aoff;
  const uint16_t* A1 = L.a[cur] + (aoff ^ 32u);
  const uint16_t* An = L.a[nxt] + aoff;
  constexpr int NI = 4 * H;                   // A fragments per substep
  u32x4 af[16];      // A fragment of group g (substep g / 8, rows 16 (g % 8))
  u32x4 b1[4];
  NF4Half h;
  u32x2 even;
#pragma unroll
  for (int i = 0; i < 3; ++i) af[i] = ops.a[i];

#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const int sub = g >> 3, i = g & 7;
    // operand reads: A fragment of group g + 3 (if it has MFMAs), B of substep 1
    // at group 4, the next stage's first operands after barrier Y
    {
      const int g3 = g + 3, i3 = g3 & 7;
      if (g3 < 16 && i3 < NI) af[g3] = lds_frag((g3 < 8 ? A0 : A1) + 16 * BK * i3);
    }
    if (NI > 0 && g == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) b1[j] = b_frag<DG>(L.b[cur], br, 1, j);
    }
    if (NI > 0 && g == 14) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ops.b[j] = b_frag<DG>(L.b[nxt], br, 0, j);
    }
    if (g == 14 && NI > 0) ops.a[0] = lds_frag(An);
    if (g == 15 && NI > 1) ops.a[1] = lds_frag(An + 16 * BK);
    if (g == 15 && NI > 2) ops.a[2] = lds_frag(An + 32 * BK);
    if (i < NI) mfma_row<F, kTr<F, DG>>(af[g], sub ? b1 : ops.b, acc[i]);
    // staging of the next stage (on the last stage it writes stale data into the
    // free buffer, which nothing reads; this keeps the groups free of branches)
    if (g < 4) {
      store_a_piece<F, DG, TAIL>(ra, g, L.a[nxt], k1, C, wave, lane);
      load_a_piece(ra, g, src, st + 2, st + 2 < nst);
    }
    if (g == 0 || g == 1) b_setup<F, DG>(dec, g + 2, rb[P ^ 1], k1, K);
    if (g >= 2 && g < 14) {
      b_step<F, DG>((g - 2) / 3, (g - 2) % 3, rb[P ^ 1], dec, h, even, L.b[nxt], brow, m4, base);
      if (g == 13) load_b<F>(rb[P ^ 1], src, st + 3, st + 3 < nst);
    }
    if (g == 13) __syncthreads();   // Y: the next stage's buffers are complete
    if (g == 14 || g == 15) b_setup<F, DG>(dec, g - 14, rb[P], k1 + BK, K);
    // one MFMA, then up to two VALU instructions, four times
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The first loads of a tile (stage 0's activations and codes, stage 1's codes,
// the NF4 row exponents), issued ahead of its prologue: the tiled kernel issues
// them right after the previous tile's K loop, so that their latency passes
// under that tile's epilogue.
template <Fmt F>
__device__ __forceinline__ void tile_prefetch(const TileSrc& src, int nst, const int32_t* rexp, int rows,
                                              RawA& ra, RawB (&rb)[2], int32_t& rxv) {
  rxv = 0;
  if constexpr (F == NF4) {
    // rows past the expert read 0
    const __amdgpu_buffer_rsrc_t RX =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(rexp), (short)0, rows * 4, 0x00020000);
    if (threadIdx.x < BM) rxv = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(RX, threadIdx.x * 4u, 0, 0);
  }
  load_a(ra, src, 0, true);
  load_b<F>(rb[0], src, 0, true);
  load_b<F>(rb[1], src, 1, nst > 1);
}

// Main loop over the K stages of one tile (H = the wavefront's active 64-row
// halves; every wavefront runs the same barriers whatever its H).
template <Fmt F, bool DG, bool TAIL, int H>
__device__ __forceinline__ void run_tile_h(TileLds<DG>& L, const TileSrc& src, int64_t C, int64_t K,
                                           int wave, int lane, f32x4 (&acc)[8][4], RawA& ra,
                                           RawB (&rb)[2], int32_t rxv, int32_t* rx) {
  const int wm = wave >> 2, wn = wave & 3;
  const int r16 = lane & 15;
  const uint32_t aoff = (uint32_t)swz(128 * wm + r16, lane >> 4);
  BRd<DG> br;
  if constexpr (DG) {
    const int g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      br.off[h] = (uint32_t)(dg_pos(8 * g + 4 * h + (r16 >> 2)) * kLdB + 64 * wn + 4 * (r16 & 3));
  } else {
    br.off = (uint32_t)swz(64 * wn + r16, lane >> 4);
  }
  // dgrad staging row: the weight row's contraction slot (NF4 slot order, or
  // natural order for MXFP4's bf16 operands)
  const int brow = F == NF4 ? ((threadIdx.x & 63) & ~7) + nf4_slot(threadIdx.x & 7) : (threadIdx.x & 63);
  const int nst = (int)((C + BK - 1) / BK);
  uint32_t m4 = 0x04040404u, base = 0x03020100u;
  asm volatile("" : "+v"(base));
  asm volatile("" : "+s"(m4));
  BDec<F> dec;
  Ops ops;
  // Prologue: stage 0 into buffer 0 from the registers tile_prefetch filled
  // (during the previous tile's epilogue); raw data of stages 1 (activations)
  // and 1, 2 (codes) in flight; the first half of stage 1's decode state. NF4:
  // the tile's row exponents go to LDS for the epilogue.
#pragma unroll
  for (int q = 0; q < 4; ++q) store_a_piece<F, DG, TAIL>(ra, q, L.a[0], 0, C, wave, lane);
  if constexpr (F == NF4)
    if (threadIdx.x < BM) rx[threadIdx.x] = rxv;
  {
    NF4Half h;
    u32x2 even;
#pragma unroll
    for (int j = 0; j < 4; ++j) b_setup<F, DG>(dec, j, rb[0], 0, K);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 3; ++r) b_step<F, DG>(q, r, rb[0], dec, h, even, L.b[0], brow, m4, base);
  }
  load_a(ra, src, 1, nst > 1);
  load_b<F>(rb[0], src, 2, nst > 2);
  b_setup<F, DG>(dec, 0, rb[1], BK, K);
  b_setup<F, DG>(dec, 1, rb[1], BK, K);
  __syncthreads();
  if constexpr (H > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ops.b[j] = b_frag<DG>(L.b[0], br, 0, j);
#pragma unroll
    for (int i = 0; i < 3; ++i) ops.a[i] = lds_frag(L.a[0] + aoff + 16 * BK * i);
  }
  for (int st = 0; st < nst; st += 2) {
    tile_stage<F, DG, TAIL, H, 0>(L, src, C, K, st, nst, wave, lane, brow, ra, rb, dec, ops, acc, aoff, br, m4, base);
    if (st + 1 < nst)
      tile_stage<F, DG, TAIL, H, 1>(L, src, C, K, st + 1, nst, wave, lane, brow, ra, rb, dec, ops, acc, aoff, br,
                                    m4, base);
  }
  __syncthreads();   // the epilogue reuses the stage buffers
}

// Forward (DG = false): out[M, N] = a . W^T per expert. dgrad (DG = true):
// out[M, K] = dY . W per expert (NF4: `a16` holds dY as fp16 in the slot order;
// MXFP4 reads the bf16 dY directly).
// TAIL: the contraction length is not a multiple of 64, so the last stage's
// activation chunks past it must be zeroed (MXFP4 K, dgrad N).
//
// Work order. An expert's rows split into full 256-row blocks and a remainder
// block. A tile's cost follows the MFMA work of its 64-row halves while its
// weight decode is the same for any row count, so a remainder of up to 128 rows
// costs half a full tile or less. Class 0 (every full block, and remainders of
// more than 128 rows) comes first, expert by expert; class 1 (the smaller
// remainders) follows, so the persistent rounds end on the cheapest tiles
// instead of leaving whole tiles for a last, mostly idle round.
// Work units of an expert with s rows: class 0 (c = 0) and class 1 (c = 1) tiles.
__device__ __forceinline__ int32_t tile_units(int32_t s, int c, int32_t thresh, int n_tiles) {
  if (s <= thresh) return 0;
  const int32_t full = s / BM, rem = s % BM;
  if (c == 0) return (full + (rem > BM / 2 ? 1 : 0)) * n_tiles;
  return rem > 0 && rem <= BM / 2 ? n_tiles : 0;
}

// Split of the last round. The class-1 tiles follow the class-0 ones round by
// round; the r of them that are left over for a last, partial round would run
// there on r CUs while the rest idle, so each of those r is split into S pieces
// of consecutive contraction stages (S <= smax, S r <= G). The first `unsplit`
// class-1 tiles run whole; S = 1 when nothing is split.
struct TailPlan {
  int32_t unsplit;
  int S;
};
__device__ __forceinline__ TailPlan tail_plan(int32_t total0, int32_t total1, int G, int smax, int nst) {
  const TailPlan none{total1, 1};
  if (smax <= 1 || total1 <= 0) return none;
  const int32_t free_slots = (G - total0 % G) % G;
  if (total1 <= free_slots) return none;
  const int32_t r = (total1 - free_slots) % G;
  if (r == 0) return none;
  const int S = min(min(smax, nst), min(G / r, kMaxTailPieces / r));
  return S > 1 ? TailPlan{total1 - r, S} : none;
}

template <Fmt F, bool DG, bool TAIL>
__global__ __launch_bounds__(kTileThreads, 1) void tile_kernel(GemmArgs g) {
  __shared__ int32_t p_off[kMaxExperts + 1];
  __shared__ int32_t p_u0[kMaxExperts + 1];
  __shared__ int32_t p_u1[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) TileLds<DG> L;
  __shared__ __attribute__((aligned(16))) int32_t rx[F == NF4 ? BM : 1];   // NF4 row exponents of the tile

  const int64_t C = DG ? g.N : g.K;   // contraction length
  const int64_t O = DG ? g.K : g.N;   // output width
  const int n_tiles = (int)((O + BN - 1) / BN);
  const int nst = (int)((C + BK - 1) / BK);
  const int32_t thresh = g.thresh;
  const int32_t total0 = build_plan2(p_off, p_u0, p_u1, g.sizes, g.E, g.M, g.err, [&](int32_t s, int c) -> int32_t {
    return tile_units(s, c, thresh, n_tiles);
  });
  const int32_t total1 = p_u1[g.E];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // XCD-aware order: round r hands XCD x the tiles r*G + x*(G/8) .. + G/8 - 1.
  const int G = gridDim.x;
  const int per_xcd = G / kXcds;
  const int slot = (G % kXcds == 0) ? (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds
                                    : blockIdx.x;
  const TailPlan tp = tail_plan(total0, total1, G, g.tail_split, nst);
  const int S = tp.S;
  const int32_t total = total0 + tp.unsplit + (total1 - tp.unsplit) * S;

  // Unit u: its expert, rows, output columns and contraction range.
  struct Unit {
    int e, piece, st0;
    bool split;
    int32_t w;   // split units: partial-sum slot
    int64_t row0, n0, Cp, Kp;
    int rows;
  };
  auto decode_unit = [&](int32_t u) -> Unit {
    Unit t;
    int mt, nt;
    t.piece = 0;
    t.split = false;
    t.w = 0;
    if (u < total0) {
      t.e = find_expert(p_u0, g.E, u);
      const int32_t lu = u - p_u0[t.e];
      mt = lu / n_tiles;
      nt = lu % n_tiles;
    } else {
      int32_t t1 = u - total0;
      if (t1 >= tp.unsplit) {
        t.split = true;
        t.w = t1 - tp.unsplit;
        t.piece = t.w % S;
        t1 = tp.unsplit + t.w / S;
      }
      t.e = find_expert(p_u1, g.E, t1);
      mt = (p_off[t.e + 1] - p_off[t.e]) / BM;   // the remainder block
      nt = t1 - p_u1[t.e];
    }
    t.row0 = (int64_t)p_off[t.e] + (int64_t)mt * BM;
    t.rows = min(BM, (int)(p_off[t.e + 1] - t.row0));
    t.n0 = (int64_t)nt * BN;
    // A piece reads like a tile of a shorter contraction: stages piece nst / S ..
    // (piece + 1) nst / S - 1, the last piece running to the end (with the
    // contraction's own tail).
    t.st0 = t.split ? t.piece * nst / S : 0;
    t.Cp = !t.split ? C
           : t.piece == S - 1 ? C - (int64_t)t.st0 * BK
                              : (int64_t)((t.piece + 1) * nst / S - t.st0) * BK;
    t.Kp = DG ? g.K : t.Cp;
    return t;
  };
  auto unit_src = [&](const Unit& t) { return tile_src<F, DG>(g, t.e, t.row0, t.rows, t.n0, wave, lane, t.st0); };
  auto prefetch = [&](const Unit& t, const TileSrc& src, RawA& ra, RawB (&rb)[2], int32_t& rxv) {
    tile_prefetch<F>(src, (int)((t.Cp + BK - 1) / BK), F == NF4 ? g.rexp + t.row0 : g.sizes, t.rows, ra, rb, rxv);
  };

  // NF4 forward: the first loads of the next unit go out between this unit's K
  // loop and its epilogue (the other instantiations issue them at the start of
  // the unit: there the extra live registers cost spills in the stage loop).
  constexpr bool kPf = F == NF4 && !DG;
  RawA ra;
  RawB rb[2];
  int32_t rxv = 0;
  Unit cu{}, nu{};
  TileSrc src{}, nsrc{};
  int32_t u = slot;
  if (kPf && u < total) {
    cu = decode_unit(u);
    src = unit_src(cu);
    prefetch(cu, src, ra, rb, rxv);
  }
  auto advance = [&] {
    if constexpr (kPf) {
      cu = nu;
      src = nsrc;
    }
  };
  for (; u < total; u += G, advance()) {
    if constexpr (!kPf) {
      cu = decode_unit(u);
      src = unit_src(cu);
      prefetch(cu, src, ra, rb, rxv);
    }
    const int e = cu.e, piece = cu.piece;
    const bool split = cu.split;
    const int32_t w = cu.w;
    const int64_t row0 = cu.row0, n0 = cu.n0;
    const int rows = cu.rows;

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int vrows = __builtin_amdgcn_readfirstlane(rows - 128 * wm);
    if (vrows > 64)
      run_tile_h<F, DG, TAIL, 2>(L, src, cu.Cp, cu.Kp, wave, lane, acc, ra, rb, rxv, rx);
    else if (vrows > 0)
      run_tile_h<F, DG, TAIL, 1>(L, src, cu.Cp, cu.Kp, wave, lane, acc, ra, rb, rxv, rx);
    else
      run_tile_h<F, DG, TAIL, 0>(L, src, cu.Cp, cu.Kp, wave, lane, acc, ra, rb, rxv, rx);
    if (kPf && u + G < total) {
      nu = decode_unit(u + G);
      nsrc = unit_src(nu);
      prefetch(nu, nsrc, ra, rb, rxv);
    }

    // NF4: the fp16 operand rows were multiplied by 2^-rexp[row] (exact), so each
    // result is multiplied by 2^rexp[row] (exact) where it is read out for its
    // bf16 rounding, and the adapter delta joins the accumulators at the same
    // 2^-rexp[row] scale. Rows past the expert read exponent 0 and are never
    // stored. MXFP4 operands are not scaled.
    auto rowexp = [&](int r) -> int {   // r: row of the wavefront's 128-row block
      if constexpr (F == NF4) return rx[128 * wm + r];
      return 0;
    };
    auto unscale = [](float v, int ex) -> float {
      if constexpr (F == NF4) return __builtin_amdgcn_ldexpf(v, ex);
      return v;
    };

    // Epilogue through LDS: each wavefront writes its 128x64 block as bf16
    // (row-major, rows padded to 144 B) over the idle stage buffers, then stores
    // whole 16-byte row pieces. acc[i][j][q] is row 16i + lane%16, column
    // 16j + 4(lane/16) + q of the block (kTr), or row 16i + 4(lane/16) + q,
    // column 16j + lane%16 (NF4 dgrad); every write offset is a constant from
    // the lane's base.
    if (g.lora_r > 0 && rows > 128 * wm && piece == 0) {   // a split tile adds the delta once
      // Low-rank adapter delta into the accumulators before their bf16 rounding:
      // block (i, j) += s U[rows 16 i .., 32 of r] Q[columns 16 j .., 32 of r]^T,
      // the fp32 operands split into bf16 pairs (hi x hi + hi x lo + lo x hi; s
      // applied to U before the split). Rows past the expert and columns past
      // the output width read zeros.
      const int r = g.lora_r;
      const int r16 = lane & 15, kg = lane >> 4;
      const int64_t qcols = min<int64_t>(64, O - n0 - 64 * wn);
      const __amdgpu_buffer_rsrc_t RU = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(g.lora_u + (row0 + 128 * wm) * r), (short)0, (rows - 128 * wm) * r * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t RQ = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(g.lora_q + ((int64_t)e * O + n0 + 64 * wn) * r), (short)0,
          (int32_t)(qcols > 0 ? qcols * r * 4 : 0), 0x00020000);
      for (int j0 = 0; j0 < r; j0 += 32) {
        const int jj = j0 + 8 * kg;
        const bool ok = jj < r;
        Split8 bq[4];
        // NF4 dgrad: MFMA column c of a block is output column dg_col(c)
        const int qc = (DG && F == NF4) ? dg_col(r16) : r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[j] = load8_split(RQ, (uint32_t)((16 * j + qc) * r + jj), ok);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const Split8 au = load8_split(RU, (uint32_t)((16 * i + r16) * r + jj), ok, g.lora_s,
                                        -rowexp(16 * i + r16));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // the same operand order as the main loop, so the layouts agree
            if constexpr (kTr<F, DG>) {
              acc[i][j] = mfma16<MXFP4>(bq[j].hi, au.hi, acc[i][j]);
              acc[i][j] = mfma16<MXFP4>(bq[j].lo, au.hi, acc[i][j]);
              acc[i][j] = mfma16<MXFP4>(bq[j].hi, au.lo, acc[i][j]);
            } else {
              acc[i][j] = mfma16<MXFP4>(au.hi, bq[j].hi, acc[i][j]);
              acc[i][j] = mfma16<MXFP4>(au.hi, bq[j].lo, acc[i][j]);
              acc[i][j] = mfma16<MXFP4>(au.lo, bq[j].hi, acc[i][j]);
            }
          }
        }
      }
    }
    if (split) {
      // fp32 partial sums of this piece (rows < 128: wave row 0 only), output
      // columns in final order, row factor 2^rexp already applied; the fixup
      // launch adds the S pieces in order. The barrier after it keeps the next
      // tile's prologue from rewriting the row exponents while they are read.
      if (wm == 0) {
        float* P = g.tail_part + (int64_t)w * kTailPieceFloats;
        if constexpr (kTr<F, DG>) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 16 * i + (lane & 15);
            const int ex = rowexp(r);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f32x4 v;
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = unscale(acc[i][j][q], ex);
              *reinterpret_cast<f32x4*>(&P[r * BN + 64 * wn + 16 * j + 4 * (lane >> 4)]) = v;
            }
          }
        } else {
          const int c16 = dg_col(lane & 15);
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 16 * i + 4 * (lane >> 4) + q;
              const int ex = rowexp(r);
#pragma unroll
              for (int j = 0; j < 4; ++j) P[r * BN + 64 * wn + 16 * j + c16] = unscale(acc[i][j][q], ex);
            }
        }
      }
      __syncthreads();
      continue;
    }
    uint16_t* E = L.epi[wave];
    auto bf16x2 = [](float x, float y) -> uint32_t {
      return (uint32_t)to_bf16(x) | ((uint32_t)to_bf16(y) << 16);
    };
    if (!DG && g.glu) {
      // Fused expert block: columns 2c, 2c+1 are the gate and up of unit c, so a
      // lane's four adjacent columns (transposed layout) are units
      // 8 j + 2 (l / 16) and the next one of its row, written as one bf16 pair.
      // The wavefront's 128 x 32 unit block goes through LDS like the plain
      // epilogue.
      uint16_t* base = E + (lane & 15) * kEpiLd + 2 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ex = rowexp(16 * i + (lane & 15));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = unscale(acc[i][j][q], ex);
          *reinterpret_cast<uint32_t*>(base + (16 * i) * kEpiLd + 8 * j) =
              bf16x2(swiglu(v[0], v[1]), swiglu(v[2], v[3]));
        }
      }
      // each wavefront reads back only its own block: LDS keeps a wavefront's
      // accesses in order, so no workgroup barrier is needed here
      __builtin_amdgcn_wave_barrier();
      const int chunk = lane & 3;
      const int64_t O2 = O >> 1;
      const int64_t col = (n0 >> 1) + 32 * wn + 8 * chunk;
      const bool vec = (O2 & 7) == 0 && col + 8 <= O2;
      const uint16_t* src = E + (lane >> 2) * kEpiLd + 8 * chunk;
      for (int rr = 0; rr < 128; rr += 16) {
        const int lr = 128 * wm + rr + (lane >> 2);
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + rr * kEpiLd);
        if (lr < rows && col < O2) {
          uint16_t* dst = g.out + (row0 + lr) * O2 + col;
          if (vec) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (col + x < O2) dst[x] = (uint16_t)(v[x >> 1] >> (16 * (x & 1)));
          }
        }
      }
      __syncthreads();   // the stage buffers are reused by the next tile
      continue;
    }
    if constexpr (kTr<F, DG>) {
      // four adjacent outputs of one row per block: one 8-byte write
      uint16_t* base = E + (lane & 15) * kEpiLd + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ex = rowexp(16 * i + (lane & 15));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x2*>(base + (16 * i) * kEpiLd + 16 * j) =
              u32x2{bf16x2(unscale(acc[i][j][0], ex), unscale(acc[i][j][1], ex)),
                    bf16x2(unscale(acc[i][j][2], ex), unscale(acc[i][j][3], ex))};
      }
    } else {
      uint16_t* base = E + (4 * (lane >> 4)) * kEpiLd + dg_col(lane & 15);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ex = rowexp(16 * i + 4 * (lane >> 4) + q);
#pragma unroll
          for (int j = 0; j < 4; ++j) base[(16 * i + q) * kEpiLd + 16 * j] = to_bf16(unscale(acc[i][j][q], ex));
        }
    }
    __builtin_amdgcn_wave_barrier();   // own block only (as in the gated epilogue)
    {
      const int chunk = lane & 7;
      const int64_t col = n0 + 64 * wn + 8 * chunk;
      const bool vec = (O & 7) == 0 && col + 8 <= O;
      const uint16_t* src = E + (lane >> 3) * kEpiLd + 8 * chunk;
      for (int rr = 0; rr < 128; rr += 8) {
        const int lr = 128 * wm + rr + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + rr * kEpiLd);
        if (lr < rows) {
          uint16_t* dst = g.out + (row0 + lr) * O + col;
          if (vec) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (col + x < O) dst[x] = (uint16_t)(v[x >> 1] >> (16 * (x & 1)));
          }
        }
      }
    }
    __syncthreads();  // the stage buffers are reused by the next tile
  }
}

// Split class-1 tiles (see tile_kernel): out = bf16 of the S pieces' partial
// sums added in piece order; with the gated epilogue, of silu(gate) * up over
// the column pairs (2c, 2c + 1). Recomputes the tiled kernel's plan and split
// from the same arguments and grid; exits when no tile was split.
__global__ __launch_bounds__(kThreads) void tile_fixup_kernel(GemmArgs g, int dgrad, int tile_grid) {
  __shared__ int32_t p_off[kMaxExperts + 1];
  __shared__ int32_t p_u0[kMaxExperts + 1];
  __shared__ int32_t p_u1[kMaxExperts + 1];
  const int64_t C = dgrad ? g.N : g.K;
  const int64_t O = dgrad ? g.K : g.N;
  const int n_tiles = (int)((O + BN - 1) / BN);
  const int nst = (int)((C + BK - 1) / BK);
  const int32_t thresh = g.thresh;
  const int32_t total0 = build_plan2(p_off, p_u0, p_u1, g.sizes, g.E, g.M, g.err, [&](int32_t s, int c) -> int32_t {
    return tile_units(s, c, thresh, n_tiles);
  });
  const int32_t total1 = p_u1[g.E];
  const TailPlan tp = tail_plan(total0, total1, tile_grid, g.tail_split, nst);
  const int S = tp.S;
  if (S <= 1) return;
  const bool glu = !dgrad && g.glu;
  // Work items: 8 rows of one split tile; thread t sums columns 8 (t % 32) .. +8
  // of row t / 32, with the 2 S float4 loads of its pieces in flight together.
  const int32_t items = (total1 - tp.unsplit) * (BM / 2 / 8);
  const int tr = threadIdx.x >> 5, tc = 8 * (threadIdx.x & 31);
  for (int32_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int32_t x = it / (BM / 2 / 8);
    const int r = 8 * (it % (BM / 2 / 8)) + tr;
    const int32_t t1 = tp.unsplit + x;
    const int e = find_expert(p_u1, g.E, t1);
    const int64_t row0 = (int64_t)p_off[e] + (int64_t)((p_off[e + 1] - p_off[e]) / BM) * BM;
    const int rows = (int)(p_off[e + 1] - row0);
    if (r >= rows) continue;
    const int64_t n0 = (int64_t)(t1 - p_u1[e]) * BN;
    const float* P = g.tail_part + (int64_t)x * S * kTailPieceFloats + r * BN + tc;
    f32x4 v0 = *reinterpret_cast<const f32x4*>(P), v1 = *reinterpret_cast<const f32x4*>(P + 4);
    for (int s = 1; s < S; ++s) {
      v0 += *reinterpret_cast<const f32x4*>(P + s * kTailPieceFloats);
      v1 += *reinterpret_cast<const f32x4*>(P + s * kTailPieceFloats + 4);
    }
    if (glu) {
      // columns (2c, 2c + 1) = (gate, up) of unit c: 4 units per thread
      const int64_t O2 = O >> 1;
      const int64_t col = (n0 + tc) >> 1;
      uint16_t* dst = g.out + (row0 + r) * O2 + col;
      const float u[4] = {swiglu(v0[0], v0[1]), swiglu(v0[2], v0[3]), swiglu(v1[0], v1[1]), swiglu(v1[2], v1[3])};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (col + k < O2) dst[k] = to_bf16(u[k]);
    } else {
      const int64_t col = n0 + tc;
      uint16_t* dst = g.out + (row0 + r) * O + col;
      const float u[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if ((O & 7) == 0 && col + 8 <= O) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (uint32_t)to_bf16(u[2 * k]) | ((uint32_t)to_bf16(u[2 * k + 1]) << 16);
        *reinterpret_cast<u32x4*>(dst) = w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (col + k < O) dst[k] = to_bf16(u[k]);
      }
    }
  }
}

}  // namespace

hipError_t launch_tile_fixup(const GemmArgs& g, bool dgrad, int tile_grid, hipStream_t s) {
  // at most tile_grid split tiles of 16 work items each; two workgroups per CU
  const int grid = std::max(1, 2 * tile_grid);
  hipLaunchKernelGGL(tile_fixup_kernel, dim3(grid), dim3(kThreads), 0, s, g, dgrad ? 1 : 0, tile_grid);
  return hipGetLastError();
}

template <Fmt F, bool DG, bool TAIL>
hipError_t launch_tile_t(const GemmArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL((tile_kernel<F, DG, TAIL>), dim3(grid), dim3(kTileThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_tile(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == NF4) return launch_tile_t<NF4, false, false>(g, grid, s);
  if (g.K % BK) return launch_tile_t<MXFP4, false, true>(g, grid, s);
  return launch_tile_t<MXFP4, false, false>(g, grid, s);
}

hipError_t launch_tile_dgrad(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == MXFP4) {
    if (g.N % BK) return launch_tile_t<MXFP4, true, true>(g, grid, s);
    return launch_tile_t<MXFP4, true, false>(g, grid, s);
  }
  if (g.N % BK) return launch_tile_t<NF4, true, true>(g, grid, s);
  return launch_tile_t<NF4, true, false>(g, grid, s);
}

}  // namespace geg
