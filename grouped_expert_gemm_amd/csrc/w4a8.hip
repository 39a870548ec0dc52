// W4A8 variant of the MXFP4 grouped GEMM: the released e2m1 weight bytes and
// their e8m0 scales feed gfx950's block-scaled matrix instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4) as they are, against activations
// quantised to MXFP8 (e4m3 elements, one e8m0 scale per 32 k). Prior art: "bw24
// releases, v0.9.0", "Changes since v0.8.0" (a W4A8-FP8 prefill tile: e4m3
// activations times native e2m1 weights in one block-scaled MMA).
//
// Activation quantisation follows the OCP MX v1.0 conversion: per 32-block,
// X = floor(log2 amax) - 8 + 127 clamped to [0, 254] (0 for an all-zero block),
// elements round to nearest e4m3 (ties to even) after the exact division by
// 2^(X - 127), saturating at 448, the sign kept.
//
// Operand layout of the instruction (measured with in-bounds probes on gfx950):
// lane l works on row (A) or column (B) l % 16 and lane group g = l / 16.
//   A (fp8, 8 VGPRs): bytes 0-15 hold k = 16 g + 0..15, bytes 16-31 hold
//     k = 64 + 16 g + 0..15 of the 128-wide step.
//   B (fp4, 4 VGPRs): 32 nibbles, k = 32 g + 0..31, the even k in the low nibble:
//     exactly 16 consecutive bytes of a released MXFP4 row.
//   Scales: lane 16 b + i carries the e8m0 byte of row / column i for k-block b
//     (k = 32 b .. 32 b + 31), in byte 0 of its scale register.
// So every operand loads straight from row-major storage: two 16-byte loads of
// activation codes, one of weight bytes and one byte of each scale per lane and
// 16x16 block. The instruction's dot product keeps about 12 bits below its
// largest product (measured: error up to 3e-4 of max |a w| per instruction,
// unbiased); its results then accumulate in fp32.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int QBM = 256;   // rows per workgroup tile (4 wavefront rows of 64)
constexpr int QBN = 128;   // columns per workgroup tile (2 wavefront columns of 64)
constexpr int QBK = 128;   // k per instruction step
// Offsets stay below 2^31; setting bit 31 moves an access past every buffer
// record (it then reads 0). Arithmetic rather than a select, which the compiler
// would turn into branches around the load.
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) { return off | ((uint32_t)!ok << 31); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t qrsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// fp32 t (|t| < 512, the block's scale already divided out) -> e4m3 byte:
// round to nearest, ties to even, saturating at 448; the sign bit is kept.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  const uint32_t s = (__float_as_uint(t) >> 24) & 0x80u;
  const float a = fabsf(t);
  uint32_t c;
  if (a >= 448.f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {                       // below 2^-6: the 2^-9 grid
    c = (uint32_t)__builtin_rintf(a * 512.f);       // 0..8 (8 is the smallest normal)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;    // floor(log2 a)
    const uint32_t r = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8..16
    c = ((uint32_t)(e + 7) << 3) + (r - 8u);        // r = 16 carries into the exponent
  }
  return c | s;
}

// One thread per 16-byte chunk (8 elements) of a row-major bf16 [M, K]
// (K % 32 == 0): the four lanes of a 32-block (consecutive lanes, the grid
// stride being a multiple of 4) share its largest magnitude through two lane
// exchanges, each converts its 8 elements, and the block's first lane writes
// the scale byte. Scales go to [M, K/32] (row-major), or with STEP_MAJOR to the
// layout the W4A8 kernel stages: for each 128-wide k step st and row m, the 4
// bytes of the step's blocks at (st * M + m) * 4; blocks past K / 32 in the last
// step get 0.
template <bool STEP_MAJOR>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_kernel(const uint16_t* __restrict__ a, int64_t M,
                                                                  int64_t KS, uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales, uint32_t* err) {
  const int64_t nchunks = M * KS * 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx - (threadIdx.x & 3) < nchunks;
       idx += stride) {
    // every lane of a 4-lane group enters together (nchunks is a multiple of 4)
    const u32x4 v = reinterpret_cast<const u32x4*>(a)[idx];
    // largest magnitude: bf16 magnitudes order as their low 15 bits
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
    if (mx >= 0x7F80u && err && (idx & 3) == 0) atomicOr(err, kErrNonFinite);
    // floor(log2 amax) = field - 127 for a normal amax; zero and subnormal blocks
    // land below the clamp, as do their elements on the 2^-9 grid
    const uint32_t field = mx >> 7;
    const int X = field == 0 ? 0 : min(max((int)field - 8, 0), 254);
    const int sh = 127 - X;
    u32x2 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int el = 4 * w + h;   // element of the chunk
        const uint32_t bits = (v[el >> 1] >> (16 * (el & 1))) & 0xFFFFu;
        const float t = __builtin_ldexpf(__uint_as_float(bits << 16), sh);
        word |= e4m3_rne_sat(t) << (8 * h);
      }
      out[w] = word;
    }
    reinterpret_cast<u32x2*>(codes)[idx] = out;
    if ((idx & 3) == 0) {
      const int64_t b = idx >> 2, m = b / KS, kb = b - m * KS;
      scales[STEP_MAJOR ? ((kb >> 2) * M + m) * 4 + (kb & 3) : b] = (uint8_t)X;
    }
  }
  if constexpr (STEP_MAJOR) {
    // zero the scale bytes of the padding blocks of the last step
    const int64_t KS4 = (KS + 3) & ~(int64_t)3, pad = KS4 - KS;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < M * pad; idx += stride) {
      const int64_t m = idx / pad, kb = KS + idx - m * pad;
      scales[((kb >> 2) * M + m) * 4 + (kb & 3)] = 0;
    }
  }
}

struct W4A8Args {
  const uint8_t* aq;      // e4m3 activation codes [M, K]
  const uint8_t* as;      // their e8m0 scales, step-major: [ceil(K/128)][M][4]
  const int32_t* sizes;   // [E]
  const uint8_t* wq;      // e2m1 weight bytes [E, N, K/2]
  const uint8_t* ws;      // e8m0 weight scales [E, N, K/32]
  uint16_t* out;          // bf16 [M, N]
  int64_t M, N, K;
  int32_t E;
  uint32_t* err;
};

constexpr int QThreads = 512;                 // 8 wavefronts: 4 (rows) x 2 (columns)
constexpr int kAStage = QBM * QBK;            // activation bytes per stage (256 rows x 128)
constexpr int kBStage = QBN * (QBK / 2);      // weight bytes per stage (128 columns x 64)
constexpr int kSAOff = kAStage + kBStage;     // activation scales of the stage: [256 rows][4 blocks]
constexpr int kSBOff = kSAOff + QBM * 4;      // weight scales of the stage: [128 columns][4 blocks]
constexpr int kStage = kSBOff + QBN * 4;

// LDS stage layout. Activation row r holds 8 chunks of 16 bytes, chunk c stored
// at c ^ (r % 8); weight column n holds 4 chunks, chunk c stored at
// c ^ ((n / 4) % 4). With those, the fragment reads (16 rows or columns at one
// chunk each, serviced 8 lanes at a time over the 64 banks) touch 8 distinct
// 16-byte bank groups, and the row-wise stores stay conflict-free too.
__device__ __forceinline__ uint32_t a_lds(int r, int c) { return (uint32_t)(r * QBK + ((c ^ (r & 7)) << 4)); }
__device__ __forceinline__ uint32_t b_lds(int n, int c) {
  return (uint32_t)(n * (QBK / 2) + ((c ^ ((n >> 2) & 3)) << 4));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N of this wavefront's loads (those into LDS included) are
// still in flight; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);   // expcnt, lgkmcnt: no wait
}

// End of a pipelined step: this wavefront's LDS reads are done and at most N of
// its loads are in flight, then the workgroup meets. (__syncthreads would also
// wait for every load in flight: its fence orders global memory too.) The
// memory clobber keeps the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0070);   // lgkmcnt(0), vmcnt(N)
  asm volatile("s_barrier" ::: "memory");
}

// Output tiles of 256x128 per workgroup (one workgroup per CU), persistent over
// an XCD-aware order. Each 128-wide k step is staged through LDS by loads that
// write LDS directly: 16 bytes per lane at consecutive slots from a
// wavefront-uniform base, each lane fetching the chunk that belongs in its slot
// under the swizzle. Three stage buffers, two steps of loads in flight while a
// step computes, one barrier per step. The buffers are distinct LDS objects
// and each step names its own at compile time (the step loop is unrolled by 3):
// the compiler then knows a step's LDS reads do not touch the buffers that
// loads are still filling, and adds no wait for those loads.
// Wavefront (wm, wn) computes rows 64 wm .. +63 and columns 64 wn .. +63: 4 x 4
// blocks of the 16x16x128 instruction per step. Scale bytes go straight from
// memory to the lanes that use them.
//
// Work order: class 0 (every full 256-row block, and remainders of more than
// 128 rows) first, expert by expert; class 1 (remainders of at most 128 rows,
// whose idle wavefront rows skip their instructions, so they cost half a tile
// or less) after it, so that the last persistent rounds hold the cheap tiles.
__global__ __launch_bounds__(QThreads, 1) void w4a8_kernel(W4A8Args g) {
  __shared__ int32_t p_off[kMaxExperts + 1];
  __shared__ int32_t p_u0[kMaxExperts + 1];
  __shared__ int32_t p_u1[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kStage];
  const int64_t K = g.K, N = g.N, KS = K >> 5, M = g.M;
  const int n_tiles = (int)((N + QBN - 1) / QBN);
  const int32_t total0 = build_plan2(p_off, p_u0, p_u1, g.sizes, g.E, g.M, g.err, [&](int32_t s, int c) -> int32_t {
    const int32_t full = s / QBM, rem = s % QBM;
    if (c == 0) return (full + (rem > QBM / 2 ? 1 : 0)) * n_tiles;
    return rem > 0 && rem <= QBM / 2 ? n_tiles : 0;
  });
  const int32_t total = total0 + p_u1[g.E];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  const int nst = (int)((K + QBK - 1) / QBK);
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  // Stage copy: wavefront w fills activation rows 8 (w + 8 i) .. +7 (i < 4) and
  // weight columns 16 w .. +15, 1 KB per load instruction; lane l
  // lands in slot l % 8 of row l / 8 (activations) or slot l % 4 of column l / 4
  // (weights) and fetches the chunk the swizzle puts there.
  const int cp_ar = 8 * wave + (lane >> 3), cp_ac = (lane & 7) ^ (cp_ar & 7);   // row, chunk (i = 0)
  const int cp_bn = 16 * wave + (lane >> 2), cp_bc = (lane & 3) ^ ((cp_bn >> 2) & 3);
  // Fragment reads: rows 16 apart share their swizzle, and so do columns 16 apart,
  // so fragment i of the wavefront's rows is read at rd_alo / rd_ahi + 2048 i,
  // fragment j of its columns at rd_b + 1024 j.
  const uint32_t rd_alo = a_lds(64 * wm + r16, grp), rd_ahi = a_lds(64 * wm + r16, 4 + grp);
  const uint32_t rd_b = kAStage + b_lds(64 * wn + r16, grp);
  // scale bytes in LDS: row 64 wm + 16 i + r16, block grp at rd_sa + 64 i; column
  // 64 wn + 16 j + r16 at rd_sb + 64 j
  const uint32_t rd_sa = kSAOff + (uint32_t)((64 * wm + r16) * 4 + grp);
  const uint32_t rd_sb = kSBOff + (uint32_t)((64 * wn + r16) * 4 + grp);
  // weight scale byte this thread stages: column t / 4, block t % 4 of the step
  const int sb_col = t >> 2, sb_blk = t & 3;

  for (int32_t base = 0; base < total; base += G) {
    const int32_t u = base + slot;
    if (u >= total) break;
    int e, mt, nt;
    if (u < total0) {
      e = find_expert(p_u0, g.E, u);
      const int32_t lu = u - p_u0[e];
      mt = lu / n_tiles;
      nt = lu % n_tiles;
    } else {
      const int32_t t1 = u - total0;
      e = find_expert(p_u1, g.E, t1);
      mt = (p_off[e + 1] - p_off[e]) / QBM;   // the remainder block
      nt = t1 - p_u1[e];
    }
    const int64_t row0 = p_off[e] + (int64_t)mt * QBM;
    const int rows = (int)min<int64_t>(QBM, p_off[e + 1] - row0);
    const int64_t n0 = (int64_t)nt * QBN;
    const int ncols = (int)min<int64_t>(QBN, N - n0);
    // rows past the expert's last row and columns past N read as zeros
    const __amdgpu_buffer_rsrc_t RA = qrsrc(g.aq + row0 * K, (int64_t)rows * K);
    // step-major activation scales: the whole array (rows of the next expert read
    // real scale bytes, never 0xFF; their activation chunks read zeros)
    const __amdgpu_buffer_rsrc_t RAS = qrsrc(g.as, (int64_t)nst * M * 4);
    const __amdgpu_buffer_rsrc_t RW = qrsrc(g.wq + ((int64_t)e * N + n0) * (K >> 1), (int64_t)ncols * (K >> 1));
    const __amdgpu_buffer_rsrc_t RWS = qrsrc(g.ws + ((int64_t)e * N + n0) * KS, (int64_t)ncols * KS);

    // Stage st into LDS buffer L: activation and weight chunks, and (wavefront 0)
    // the tile's 256 activation scale dwords of the step, 1 KB. Chunks that start
    // at or past K (the last step when K % 128 != 0, and every chunk of the steps
    // past the last) read zeros. Rows past the tile's rows and columns past N
    // read zeros through the buffer bounds. Five loads per wavefront, six for
    // wavefront 0.
    auto stage = [&](int st, uint8_t* L) {
      const int64_t k0 = (int64_t)st * QBK;
      const bool a_ok = k0 + 16 * cp_ac < K, b_ok = k0 + 32 * cp_bc < K;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)((cp_ar + 64 * i) * K + k0 + 16 * cp_ac);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(RA, (lds_ptr_t)(L + (8 * wave + 64 * i) * QBK), 16,
                                                 oob_unless(a_ok, off), 0, 0, 0);
      }
      const uint32_t boff = (uint32_t)(cp_bn * (K >> 1) + (k0 >> 1) + 16 * cp_bc);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(RW, (lds_ptr_t)(L + kAStage + 16 * wave * (QBK / 2)), 16,
                                               oob_unless(b_ok, boff), 0, 0, 0);
      if (wave == 0) {
        const uint32_t soff = (uint32_t)(((int64_t)st * M + row0) * 4 + 16 * lane);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(RAS, (lds_ptr_t)(L + kSAOff), 16, oob_unless(st < nst, soff), 0, 0, 0);
      }
    };
    // weight scale byte of step st for this thread (column sb_col, block sb_blk);
    // blocks past K read 0 (a scale byte of the next row must not reach the
    // instruction: 0xFF would be NaN)
    auto wscale = [&](int st) -> uint32_t {
      const int64_t kb = (int64_t)st * 4 + sb_blk;
      return __builtin_amdgcn_raw_buffer_load_b8(RWS, oob_unless(kb < KS, (uint32_t)(sb_col * KS + kb)), 0, 0);
    };
    // MFMAs only for the wavefront rows that hold rows of the expert
    const bool live = 64 * wm < rows;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Step st (stage in buffer `cur`, loaded two steps earlier): (1) load this
    // thread's weight scale byte of step st + 2 and start stage st + 2 into
    // `nxt2` (the buffer step st - 1 read; every wavefront left it at the barrier
    // that ended that step), (2) read the step's fragments and scale bytes,
    // (3) run its 16 instructions from registers, (4) wait until stage st + 1 and
    // the scale byte loaded in step st - 1 have landed (the loads of (1) may still
    // be in flight), store that byte into stage st + 1's buffer `nxt1`, and meet at
    // the barrier. `ws1` carries the byte of step st + 1 into this step and
    // returns the one of step st + 2.
    auto step = [&](int st, const uint8_t* cur, uint8_t* nxt1, uint8_t* nxt2, uint32_t& ws1) {
      const uint32_t ws2 = wscale(st + 2);
      stage(st + 2, nxt2);
      if (live) {
        v8i bf[4], af[4];
        uint32_t sa[4], sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(cur + rd_b + 1024 * j);
          bf[j] = v8i{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          sb[j] = cur[rd_sb + 64 * j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(cur + rd_alo + 2048 * i);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(cur + rd_ahi + 2048 * i);
          af[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          sa[i] = cur[rd_sa + 64 * i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 0, 4, 0, (int)sa[i],
                                                                          0, (int)sb[j]);
      }
      __builtin_amdgcn_sched_barrier(0);   // the instructions above overlap the loads
      if (wave == 0)
        wait_vm<7>();
      else
        wait_vm<6>();
      nxt1[kSBOff + t] = (uint8_t)ws1;
      ws1 = ws2;
      step_barrier<7>();   // the byte store is done (lgkmcnt 0); loads: no further wait
    };

    // prologue: stages 0 and 1 and the weight scale bytes of steps 0 and 1; wait
    // for stage 0 and step 0's byte, store it, meet
    uint32_t ws0 = wscale(0);
    stage(0, lds0);
    uint32_t ws1 = wscale(1);
    stage(1, lds1);
    if (wave == 0)
      wait_vm<7>();
    else
      wait_vm<6>();
    lds0[kSBOff + t] = (uint8_t)ws0;
    __syncthreads();
    // whole groups of three steps in one branch-free block (a step's
    // instructions must stay ahead of its wait and barrier; across a branch the
    // compiler would sink them past), then the one or two steps left
    int st = 0;
    for (; st + 3 <= nst; st += 3) {
      step(st, lds0, lds1, lds2, ws1);
      step(st + 1, lds1, lds2, lds0, ws1);
      step(st + 2, lds2, lds0, lds1, ws1);
    }
    if (st < nst) step(st, lds0, lds1, lds2, ws1);
    if (st + 1 < nst) step(st + 1, lds1, lds2, lds0, ws1);
    wait_vm<0>();         // loads past the last step (zeros) land before the buffers are reused
    __syncthreads();

    // Epilogue. acc[i][j][q] is row 16 i + 4 grp + q, column 16 j + r16 of the
    // wavefront's block. Lanes l, l ^ 1 hold neighbouring columns; each trades two
    // values with the other so that the even lane holds rows q = 0, 1 and the odd
    // lane rows q = 2, 3 as bf16 pairs.
    const bool odd = lane & 1;
    if ((N & 7) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 15) == 0) {
      // Through LDS (the stage buffers are idle: every load has landed and every
      // wavefront passed the barrier above): rows 0-127 of the tile in lds0, rows
      // 128-255 in lds1, 272-byte rows; then 16-byte row pieces, 16 threads per
      // 256-byte row.
      constexpr int kEpLd = 2 * QBN + 16;   // bytes per staged row
      uint8_t* half = wm < 2 ? lds0 : lds1;
      const int hr0 = 64 * (wm & 1);        // the wavefront's first row in its half
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = acc[i][j];
          const float x0 = lane_pair_swap(odd ? v[0] : v[2]);
          const float x1 = lane_pair_swap(odd ? v[1] : v[3]);
          const int r = hr0 + 16 * i + 4 * grp + (odd ? 2 : 0);
          const int cb = 2 * (64 * wn + 16 * j + r16 - (odd ? 1 : 0));   // byte of the even column
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float p = odd ? (h ? x1 : x0) : (h ? v[1] : v[0]);
            const float q = odd ? (h ? v[3] : v[2]) : (h ? x1 : x0);
            *reinterpret_cast<uint32_t*>(half + (r + h) * kEpLd + cb) = pack_bf16x2(p, q);
          }
        }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = t + QThreads * k;   // 16-byte piece: row c / 16, piece c % 16
        const int r = c >> 4, pc = c & 15;
        const u32x4 v = *reinterpret_cast<const u32x4*>((r < 128 ? lds0 : lds1) + (r & 127) * kEpLd + 16 * pc);
        const int64_t col = n0 + 8 * pc;
        if (r < rows && col < N) *reinterpret_cast<u32x4*>(g.out + (row0 + r) * N + col) = v;
      }
      __syncthreads();   // the stage buffers are reused by the next tile
      continue;
    }
    const int64_t colp = n0 + 64 * wn + r16 - (odd ? 1 : 0);   // even column of the pair
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = acc[i][j];
        const float x0 = lane_pair_swap(odd ? v[0] : v[2]);
        const float x1 = lane_pair_swap(odd ? v[1] : v[3]);
        const int lr = 64 * wm + 16 * i + 4 * grp + (odd ? 2 : 0);
        const int64_t c = colp + 16 * j;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float p = odd ? (h ? x1 : x0) : (h ? v[1] : v[0]);
          const float q = odd ? (h ? v[3] : v[2]) : (h ? x1 : x0);
          if (lr + h < rows && c < N) {
            uint16_t* dst = g.out + (row0 + lr + h) * N + c;
            if ((N & 1) == 0 && c + 1 < N) {
              *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(p, q);
            } else {
              dst[0] = to_bf16(p);
              if (c + 1 < N) dst[1] = to_bf16(q);
            }
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_mxfp8_quantize(const uint16_t* a, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                 uint32_t* err, int step_major, int cus, hipStream_t s) {
  const int64_t KS = K >> 5;
  const int64_t nchunks = M * KS * 4;
  if (nchunks <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((nchunks + kThreads - 1) / kThreads, (int64_t)cus * 16);
  if (step_major)
    hipLaunchKernelGGL(mxfp8_quantize_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, M, KS, codes,
                       scales, err);
  else
    hipLaunchKernelGGL(mxfp8_quantize_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, M, KS, codes,
                       scales, err);
  return hipGetLastError();
}

hipError_t launch_w4a8(const uint8_t* aq, const uint8_t* as, const int32_t* sizes, const uint8_t* wq,
                       const uint8_t* ws, uint16_t* out, int64_t M, int64_t N, int64_t K, int32_t E, uint32_t* err,
                       int cus, hipStream_t s) {
  W4A8Args g{aq, as, sizes, wq, ws, out, M, N, K, E, err};
  const int64_t n_tiles = (N + QBN - 1) / QBN;
  const int64_t bound = ((M + QBM - 1) / QBM + std::min<int64_t>(E, M)) * n_tiles;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(bound, (int64_t)cus));
  hipLaunchKernelGGL(w4a8_kernel, dim3((unsigned)grid), dim3(QThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
