// Tiled (prefill-shape) path of the grouped 4-bit GEMM.
//
// One persistent launch walks every 256x256 output tile of every expert that has
// more rows than the skinny path takes. Per 64-wide K stage a workgroup stages
// its activation tile (NF4: from the fp16 copy a prior pass made) and decodes
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
constexpr int kLdT = 80;        // dgrad weight rows in LDS: 64 halves + 16 pad (160 B)

// LDS of one workgroup: two stages of activation and weight tiles, or the
// epilogue's result blocks. The dgrad weight tile is written transposed (one
// contraction index per lane, scattered over 256 rows), so its rows are padded
// instead of swizzled (a 160-byte stride keeps the operand reads conflict-free).
template <bool DG>
union TileLds {
  struct {
    uint16_t a[2][BM * BK];
    uint16_t b[2][BN * (DG ? kLdT : BK)];
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

// Weight-tile offset of (row, chunk): swizzled rows for the forward pass, padded
// rows for dgrad.
template <bool DG>
__device__ __forceinline__ int bpos(int row, int chunk) {
  return DG ? row * kLdT + chunk * 8 : swz(row, chunk);
}

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

// Operand sources of the tile (expert e, rows row0.., output columns o0..).
// Forward: out = A . W^T contracts over K; thread t stages codes of weight row t/2
// (32 k per stage half t%2). dgrad: dX = dY . W contracts over N; thread t stages
// weight row n = t%64 of the stage's 64, columns o0 + 32 (t/64) .. +32.
template <Fmt F, bool DG>
__device__ __forceinline__ TileSrc tile_src(const GemmArgs& g, int e, int64_t row0, int rows,
                                            int64_t o0, int wave, int lane) {
  const int64_t K = g.K, N = g.N;
  const int64_t C = DG ? N : K;   // contraction length = activation row length
  TileSrc t;
  // NF4 reads the fp16 copy of the activations (already in the NF4 slot order).
  t.a = (F == NF4 ? g.a16 : g.a) + row0 * C;
  t.na = clamp_bytes((int64_t)rows * C * 2);
  t.a_off = (uint32_t)(((32 * wave + (lane >> 3)) * C + 8 * (lane & 7)) * 2);
  t.a_rows8 = (uint32_t)(8 * C * 2);
  const int tid = threadIdx.x;
  if constexpr (DG) {
    t.w = g.wq + (int64_t)e * N * (K >> 1);
    t.nw = clamp_bytes(N * (K >> 1));
    const int n = tid & 63, kc = tid >> 6;
    const int64_t kcol = o0 + 32 * kc;    // past K: never stored
    t.w_off = (uint32_t)(n * (K >> 1) + (kcol >> 1));
    t.w_step = (uint32_t)(BK * (K >> 1));
    if constexpr (F == NF4) {
      t.s = reinterpret_cast<const float*>(g.scales) + (int64_t)e * N * (K >> 6);
      t.ns = clamp_bytes(N * (K >> 6) * 4);
      t.s_off = (uint32_t)((n * (K >> 6) + (kcol >> 6)) * 4);
      t.s_step = (uint32_t)(BK * (K >> 6) * 4);
    } else {
      // the thread's 32 columns are exactly one 32-block of the weight row
      t.s = reinterpret_cast<const uint8_t*>(g.scales) + (int64_t)e * N * (K >> 5);
      t.ns = clamp_bytes(N * (K >> 5));
      t.s_off = (uint32_t)(n * (K >> 5) + (kcol >> 5));
      t.s_step = (uint32_t)(BK * (K >> 5));
    }
  } else {
    const int64_t nrows = min<int64_t>(BN, N - o0);
    const int64_t wrow0 = (int64_t)e * N + o0;
    t.w = g.wq + wrow0 * (K >> 1);
    t.nw = clamp_bytes(nrows * (K >> 1));
    if constexpr (F == NF4) {
      t.s = reinterpret_cast<const float*>(g.scales) + wrow0 * (K >> 6);
      t.ns = clamp_bytes(nrows * (K >> 6) * 4);
    } else {
      t.s = reinterpret_cast<const uint8_t*>(g.scales) + wrow0 * (K >> 5);
      t.ns = clamp_bytes(nrows * (K >> 5));
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

// dgrad: the four values of a half go to LDS rows k = 32 (t/64) + 8 q + 2 i + odd
// (i = 0..3) at the thread's column `bcol` (2-byte stores).
__device__ __forceinline__ void dg_store_half(uint16_t* Bs, int q, int odd, int bcol, u32x2 v) {
  uint16_t* p = Bs + (32 * (threadIdx.x >> 6) + 8 * q + odd) * kLdT + bcol;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[2 * i * kLdT] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
}

// Staging step r (0..2) of the thread's weight piece q (its 8 codes r.c[q]):
// NF4 r = 0 selects the even-k codes and looks up their low bytes, r = 1
// finishes them and selects the odd-k codes, r = 2 finishes the piece and stores
// it; MXFP4 decodes and stores the whole piece at r = 0. Each step is 7-8 VALU
// instructions, so that two steps fit under the four MFMAs of a group.
// Forward: row t/2, chunk 4 (t%2) + q, one 16-byte store in slot order. dgrad:
// the codes are columns k = 32 (t/64) + 8 q + j of weight row n = t%64; each
// value goes to LDS row k at the slot of n.
template <Fmt F, bool DG>
__device__ __forceinline__ void b_step(int q, int r, const RawB& rb, const BDec<F>& d, NF4Half& h,
                                       u32x2& even, uint16_t* Bs, int bcol, uint32_t m4,
                                       uint32_t base) {
  const int t = threadIdx.x;
  if constexpr (F == NF4) {
    const uint32_t x = rb.c[q];
    if (r == 0) {
      nf4_half_select<true>(x, m4, base, h);
      nf4_half_lo(d.lut, h);
    } else if (r == 1) {
      even = nf4_half_out(d.lut, h);
      if constexpr (DG) dg_store_half(Bs, q, 0, bcol, even);
      nf4_half_select<false>(x, m4, base, h);
    } else {
      nf4_half_lo(d.lut, h);
      const u32x2 odd = nf4_half_out(d.lut, h);
      if constexpr (DG)
        dg_store_half(Bs, q, 1, bcol, odd);
      else
        *reinterpret_cast<u32x4*>(&Bs[swz(t >> 1, 4 * (t & 1) + q)]) = u32x4{even[0], even[1], odd[0], odd[1]};
    }
  } else if (r == 0) {
    const u32x4 v = mxfp4_decode8(rb.c[q], d.sc);   // k = 8q + j, natural order
    if constexpr (DG) {
      // column n of rows k = 32 (t/64) + 8 q + j (2-byte stores)
      uint16_t* p = Bs + (32 * (t >> 6) + 8 * q) * kLdT + bcol;
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j * kLdT] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
    } else {
      *reinterpret_cast<u32x4*>(&Bs[swz(t >> 1, 4 * (t & 1) + q)]) = v;
    }
  }
}

__device__ __forceinline__ u32x4 lds_frag(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// The 4 MFMAs of one 16-row A fragment with the substep's 4 B fragments.
template <Fmt F>
__device__ __forceinline__ void mfma_row(const u32x4& a, const u32x4 (&b)[4], f32x4 (&acc)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = mfma16<F>(a, b[j], acc[j]);
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
//   barrier X at the end frees the current buffers.
// H = number of the wavefront's 64-row halves that hold rows of the expert.
template <Fmt F, bool DG, bool TAIL, int H, int P>
__device__ __forceinline__ void tile_stage(TileLds<DG>& L, const TileSrc& src, int64_t C, int64_t K,
                                           int st, int nst, int wave, int lane, int bcol,
                                           RawA& ra, RawB (&rb)[2], BDec<F>& dec, Ops& ops,
                                           f32x4 (&acc)[8][4], uint32_t aoff, uint32_t boff,
                                           uint32_t m4, uint32_t base) {
  constexpr int cur = P, nxt = P ^ 1;   // st % 2 == P
  const int64_t k1 = (int64_t)(st + 1) * BK;
  // Substep 1 reads chunk 4 + c where substep 0 reads chunk c: the swizzled
  // chunk differs in bit 2, i.e. the half offset differs in bit 5 (the padded
  // dgrad weight rows are plainly 32 halves further).
  const uint16_t* A0 = L.a[cur] + aoff;
  const uint16_t* A1 = L.a[cur] + (aoff ^ 32u);
  const uint16_t* B1 = L.b[cur] + (DG ? boff + 32u : boff ^ 32u);
  const uint16_t* An = L.a[nxt] + aoff;
  const uint16_t* Bn = L.b[nxt] + boff;
  constexpr int BR = 16 * (DG ? kLdT : BK);   // B fragment stride (16 rows)
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
      for (int j = 0; j < 4; ++j) b1[j] = lds_frag(B1 + BR * j);
    }
    if (NI > 0 && g == 14) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ops.b[j] = lds_frag(Bn + BR * j);
    }
    if (g == 14 && NI > 0) ops.a[0] = lds_frag(An);
    if (g == 15 && NI > 1) ops.a[1] = lds_frag(An + 16 * BK);
    if (g == 15 && NI > 2) ops.a[2] = lds_frag(An + 32 * BK);
    if (i < NI) mfma_row<F>(af[g], sub ? b1 : ops.b, acc[i]);
    // staging of the next stage (on the last stage it writes stale data into the
    // free buffer, which nothing reads; this keeps the groups free of branches)
    if (g < 4) {
      store_a_piece<F, DG, TAIL>(ra, g, L.a[nxt], k1, C, wave, lane);
      load_a_piece(ra, g, src, st + 2, st + 2 < nst);
    }
    if (g == 0 || g == 1) b_setup<F, DG>(dec, g + 2, rb[P ^ 1], k1, K);
    if (g >= 2 && g < 14) {
      b_step<F, DG>((g - 2) / 3, (g - 2) % 3, rb[P ^ 1], dec, h, even, L.b[nxt], bcol, m4, base);
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
  // X: every wavefront is done with the current buffers.
  __syncthreads();
}

// Main loop over the K stages of one tile (H = the wavefront's active 64-row
// halves; every wavefront runs the same barriers whatever its H).
template <Fmt F, bool DG, bool TAIL, int H>
__device__ __forceinline__ void run_tile_h(TileLds<DG>& L, const TileSrc& src, int64_t C, int64_t K,
                                           int wave, int lane, f32x4 (&acc)[8][4]) {
  const int wm = wave >> 2, wn = wave & 3;
  const int r16 = lane & 15;
  const uint32_t aoff = (uint32_t)swz(128 * wm + r16, lane >> 4);
  const uint32_t boff = (uint32_t)bpos<DG>(64 * wn + r16, lane >> 4);
  // dgrad staging column: the weight row's contraction slot (NF4 slot order, or
  // natural order for MXFP4's bf16 operands)
  const int bcol = F == NF4 ? ((threadIdx.x & 63) & ~7) + nf4_slot(threadIdx.x & 7) : (threadIdx.x & 63);
  constexpr int BR = 16 * (DG ? kLdT : BK);
  const int nst = (int)((C + BK - 1) / BK);
  uint32_t m4 = 0x04040404u, base = 0x03020100u;
  asm volatile("" : "+v"(base));
  asm volatile("" : "+s"(m4));
  RawA ra;
  RawB rb[2];
  BDec<F> dec;
  Ops ops;
  // Prologue: stage 0 into buffer 0; raw data of stages 1 (activations) and
  // 1, 2 (codes) in flight; the first half of stage 1's decode state.
  load_a(ra, src, 0, true);
  load_b<F>(rb[0], src, 0, true);
  load_b<F>(rb[1], src, 1, nst > 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_a_piece<F, DG, TAIL>(ra, q, L.a[0], 0, C, wave, lane);
  {
    NF4Half h;
    u32x2 even;
#pragma unroll
    for (int j = 0; j < 4; ++j) b_setup<F, DG>(dec, j, rb[0], 0, K);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 3; ++r) b_step<F, DG>(q, r, rb[0], dec, h, even, L.b[0], bcol, m4, base);
  }
  load_a(ra, src, 1, nst > 1);
  load_b<F>(rb[0], src, 2, nst > 2);
  b_setup<F, DG>(dec, 0, rb[1], BK, K);
  b_setup<F, DG>(dec, 1, rb[1], BK, K);
  __syncthreads();
  if constexpr (H > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ops.b[j] = lds_frag(L.b[0] + boff + BR * j);
#pragma unroll
    for (int i = 0; i < 3; ++i) ops.a[i] = lds_frag(L.a[0] + aoff + 16 * BK * i);
  }
  for (int st = 0; st < nst; st += 2) {
    tile_stage<F, DG, TAIL, H, 0>(L, src, C, K, st, nst, wave, lane, bcol, ra, rb, dec, ops, acc, aoff, boff, m4, base);
    if (st + 1 < nst)
      tile_stage<F, DG, TAIL, H, 1>(L, src, C, K, st + 1, nst, wave, lane, bcol, ra, rb, dec, ops, acc, aoff, boff,
                                    m4, base);
  }
}

// Forward (DG = false): out[M, N] = a . W^T per expert. dgrad (DG = true):
// out[M, K] = dY . W per expert (NF4: `a16` holds dY as fp16 in the slot order;
// MXFP4 reads the bf16 dY directly).
// TAIL: the contraction length is not a multiple of 64, so the last stage's
// activation chunks past it must be zeroed (MXFP4 K, dgrad N).
template <Fmt F, bool DG, bool TAIL>
__global__ __launch_bounds__(kTileThreads, 1) void tile_kernel(GemmArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) TileLds<DG> L;

  const int64_t C = DG ? g.N : g.K;   // contraction length
  const int64_t O = DG ? g.K : g.N;   // output width
  const int n_tiles = (int)((O + BN - 1) / BN);
  const int32_t thresh = g.thresh;
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    if (s <= thresh) return 0;
    return ((s + BM - 1) / BM) * n_tiles;
  });

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // XCD-aware order: round r hands XCD x the tiles r*G + x*(G/8) .. + G/8 - 1.
  const int G = gridDim.x;
  const int per_xcd = G / kXcds;
  const int slot = (G % kXcds == 0) ? (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds
                                    : blockIdx.x;

  for (int32_t base = 0; base < total; base += G) {
    const int32_t u = base + slot;
    if (u >= total) break;
    const int e = find_expert(plan, g.E, u);
    const int32_t lu = u - plan.upre[e];
    const int mt = lu / n_tiles, nt = lu % n_tiles;
    const int64_t row0 = (int64_t)plan.off[e] + (int64_t)mt * BM;
    const int rows = min(BM, (int)(plan.off[e + 1] - row0));
    const int64_t n0 = (int64_t)nt * BN;

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const TileSrc src = tile_src<F, DG>(g, e, row0, rows, n0, wave, lane);
    const int vrows = __builtin_amdgcn_readfirstlane(rows - 128 * wm);
    if (vrows > 64)
      run_tile_h<F, DG, TAIL, 2>(L, src, C, g.K, wave, lane, acc);
    else if (vrows > 0)
      run_tile_h<F, DG, TAIL, 1>(L, src, C, g.K, wave, lane, acc);
    else
      run_tile_h<F, DG, TAIL, 0>(L, src, C, g.K, wave, lane, acc);

    // Epilogue through LDS: each wavefront writes its 128x64 block as bf16
    // (row-major, rows padded to 144 B) over the idle stage buffers, then stores
    // whole 16-byte row pieces. acc[i][j][q] is row 16i + 4(lane/16) + q,
    // column 16j + lane%16 of the block; every write offset is a constant from
    // the lane's base.
    if (g.lora_r > 0 && rows > 128 * wm) {
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
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[j] = load8_split(RQ, (uint32_t)((16 * j + r16) * r + jj), ok);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const Split8 au = load8_split(RU, (uint32_t)((16 * i + r16) * r + jj), ok, g.lora_s);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = mfma16<MXFP4>(au.hi, bq[j].hi, acc[i][j]);
            acc[i][j] = mfma16<MXFP4>(au.hi, bq[j].lo, acc[i][j]);
            acc[i][j] = mfma16<MXFP4>(au.lo, bq[j].hi, acc[i][j]);
          }
        }
      }
    }
    uint16_t* E = L.epi[wave];
    if (!DG && g.glu) {
      // Fused expert block: columns 2c, 2c+1 (lanes l, l ^ 1) are the gate and
      // up of unit c. Each lane of a pair computes two of the four rows' units:
      // the even lane rows q = 0, 1, the odd lane rows q = 2, 3, trading the
      // missing halves with its neighbour. The wavefront's 128 x 32 unit block
      // goes through LDS like the plain epilogue.
      const bool odd = lane & 1;
      uint16_t* base = E + (4 * (lane >> 4) + (odd ? 2 : 0)) * kEpiLd + ((lane & 15) >> 1);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = acc[i][j];
          const float r0 = lane_pair_swap(odd ? v[0] : v[2]);
          const float r1 = lane_pair_swap(odd ? v[1] : v[3]);
          const float a0 = odd ? swiglu(r0, v[2]) : swiglu(v[0], r0);
          const float a1 = odd ? swiglu(r1, v[3]) : swiglu(v[1], r1);
          base[(16 * i) * kEpiLd + 8 * j] = to_bf16(a0);
          base[(16 * i + 1) * kEpiLd + 8 * j] = to_bf16(a1);
        }
      __syncthreads();
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
    {
      uint16_t* base = E + (4 * (lane >> 4)) * kEpiLd + (lane & 15);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) base[(16 * i + q) * kEpiLd + 16 * j] = to_bf16(acc[i][j][q]);
    }
    __syncthreads();
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

}  // namespace

hipError_t launch_tile(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == NF4)
    hipLaunchKernelGGL((tile_kernel<NF4, false, false>), dim3(grid), dim3(kTileThreads), 0, s, g);
  else if (g.K % BK)
    hipLaunchKernelGGL((tile_kernel<MXFP4, false, true>), dim3(grid), dim3(kTileThreads), 0, s, g);
  else
    hipLaunchKernelGGL((tile_kernel<MXFP4, false, false>), dim3(grid), dim3(kTileThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_tile_dgrad(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == MXFP4) {
    if (g.N % BK)
      hipLaunchKernelGGL((tile_kernel<MXFP4, true, true>), dim3(grid), dim3(kTileThreads), 0, s, g);
    else
      hipLaunchKernelGGL((tile_kernel<MXFP4, true, false>), dim3(grid), dim3(kTileThreads), 0, s, g);
  } else if (g.N % BK)
    hipLaunchKernelGGL((tile_kernel<NF4, true, true>), dim3(grid), dim3(kTileThreads), 0, s, g);
  else
    hipLaunchKernelGGL((tile_kernel<NF4, true, false>), dim3(grid), dim3(kTileThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
