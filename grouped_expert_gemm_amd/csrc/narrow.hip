// Narrow path of the grouped 4-bit GEMM: experts with a few to a few dozen
// routed rows (a decode batch of many tokens).
//
// The weights are streamed once per 16 or 32 activation rows and decoded once in
// registers, as in the other decode paths; the layout is built around the memory
// side. A workgroup unit is (expert, 16 RB activation rows, 64 CBW weight rows;
// RB = CBW = 1 or 2); each of its four wavefronts owns CBW blocks of 16 weight rows over the
// whole K range, so there is no cross-wavefront reduction. Per 128-wide K step a
// wavefront loads, for each of its 16-row blocks, one 16-byte piece per lane
// (lane l: weight row l % 16, codes k in [32 (l / 16), +32) of the step), i.e.
// 64 contiguous bytes of each of 16 rows per load instruction; it scales its
// private copy of the 16-entry table by the absmax of that piece's 64-block
// (NF4) and decodes the piece into the B operands of four 16x16x32 MFMAs. The
// activations of the step are staged once per workgroup in LDS (fp16 in the NF4
// slot order, or bf16), double-buffered with one barrier per step; global loads
// run NS - 1 steps ahead of use.
//
// MFMA k slots: MFMA j of a step takes codes 8j .. 8j+7 of every lane's piece, so
// its 32 k are {32 g + 8 j + i : g = 0..3, i = 0..7}; the activation operand reads
// the same k. NF4, 16-row units: lane groups g = 0, 1 hold the step's first
// 64-block and g = 2, 3 its second, so each MFMA is issued twice, once per
// block, with the other block's activation lanes reading a zero chunk of LDS; the
// codes go through one unscaled fp16 table shared by all lanes and the fp32
// absmax of each block scales that block's fp32 partial sums (cheaper than a
// per-lane scaled table: the MFMA pipe has room for the extra MFMAs, the vector
// ALUs do not; measured 4-15% faster). NF4, 32-row units: each lane scales its
// own copy of the table by its piece's absmax (one mixed-precision fma per
// entry; with two row blocks the doubled MFMAs and operand reads cost more than
// the table, measured 12%). MXFP4: the
// gfx950 scaled fp4 -> bf16 conversion applies the block scale (a piece is one
// 32-block). Staged activation rows are 256 B with 16-byte chunk c of row r at
// chunk c ^ (r % 16), which keeps the operand reads free of bank conflicts.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int kNStep = 128;                    // K per step

// A stage buffer holds RB blocks of 16 activation rows (256 B each), each block
// followed by a zero chunk: block r starts at r * kRBlk halves.
constexpr int kRBlk = 16 * kNStep + 8;

// Half offset of 16-byte chunk c of staged activation row r.
__device__ __forceinline__ int nswz(int r, int c) {
  return (r >> 4) * kRBlk + (r & 15) * kNStep + ((c ^ (r & 15)) << 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t nrsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Raw data of one K step held in registers: this thread's share of the
// activation stage and the wavefront's weight pieces.
template <int RB, int CBW, int NSC>
struct StepRaw {
  u32x4 a[RB];          // activations: rows 16r + t/16, k chunk t%16 (8 values)
  u32x4 w[CBW];         // codes of weight row n0 + 16 cb + l%16, k in [32 (l/16), +32)
  uint32_t s[CBW][NSC]; // NF4: fp32 absmax bits (of the step's two 64-blocks when
                        // NSC = 2, else of the lane's piece); MXFP4: e8m0 byte
};

template <Fmt F, int RB, int CBW, int NSC, bool SSC>
__device__ __forceinline__ void load_step(StepRaw<RB, CBW, NSC>& d, const __amdgpu_buffer_rsrc_t& A,
                                          const __amdgpu_buffer_rsrc_t& W,
                                          const __amdgpu_buffer_rsrc_t& S, int64_t K, int64_t N,
                                          int64_t n0, int st, int lane) {
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)st * kNStep;
  // activations: thread t loads 16 B of row 16r + t/16 at k0 + 8 (t%16); pieces
  // past K read as zero (offsets pushed past the buffer)
  {
    const int64_t k = k0 + 8 * (t & 15);
    const uint32_t mask = k < K ? 0u : 0xFFFFFFF0u;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int64_t row = 16 * q + (t >> 4);
      d.a[q] = __builtin_amdgcn_raw_buffer_load_b128(A, (uint32_t)((row * K + k) * 2) | mask, 0, 0);
    }
  }
  const int64_t kc = k0 + 32 * (lane >> 4);        // first k of this lane's piece
  const uint32_t mask = kc < K ? 0u : 0xFFFFFFF0u;
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    const int64_t n = n0 + 16 * cb + (lane & 15);  // rows past N read as zero (buffer bounds)
    d.w[cb] = __builtin_amdgcn_raw_buffer_load_b128(W, (uint32_t)(n * (K >> 1) + (kc >> 1)) | mask, 0, 0);
    if constexpr (F == NF4 && NSC == 2) {
      // both 64-blocks of the step for the lane's weight row in one load, unless
      // the unit's scales are staged in LDS. When K % 128 == 64 the second value
      // of the last step is the next row's first scale (or zero past the buffer);
      // it multiplies a partial sum of zero activations.
      if constexpr (!SSC) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(
            S, (uint32_t)((n * (K >> 6) + (k0 >> 6)) * 4) | (k0 < K ? 0u : 0xFFFFFFF0u), 0, 0);
        d.s[cb][0] = v[0];
        d.s[cb][1] = v[1];
      }
    } else if constexpr (F == NF4) {
      d.s[cb][0] = __builtin_amdgcn_raw_buffer_load_b32(S, (uint32_t)((n * (K >> 6) + (kc >> 6)) * 4) | mask, 0, 0);
    } else {
      d.s[cb][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(S, (uint32_t)(n * (K >> 5) + (kc >> 5)) | mask, 0, 0);
    }
  }
}

// SSC: the unit's NF4 absmax values (K <= 2048: at most 32 blocks per row) are
// staged in LDS once per unit instead of being loaded with every step; per-step
// loads of 4-byte values from 16 rows cost as many memory requests as the
// weights themselves.
template <Fmt F, int RB, int CBW, int NS, bool SSC>
__global__ __launch_bounds__(kThreads, 3) void narrow_kernel(GemmArgs g) {
  // step st stages step st+1 from registers loaded two steps earlier
  static_assert(NS >= 3, "the staged step must already be in registers");
  // routing plan in dynamic LDS sized by the expert count: off[E + 1], upre[E + 1]
  extern __shared__ __attribute__((aligned(16))) int32_t nplan[];
  int32_t* const poff = nplan;
  int32_t* const pupre = nplan + g.E + 1;
  // two stage buffers; the zero chunk after each row block is what the
  // activation lanes of the other 64-block read (NF4)
  constexpr int kBuf = RB * kRBlk;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBuf];
  constexpr int RPU = 16 * RB;                     // activation rows per unit
  constexpr int CPU = 4 * 16 * CBW;                // weight rows per unit
  const int32_t n_cols = (int32_t)((g.N + CPU - 1) / CPU);
  const int64_t lo = max<int64_t>(1, (int64_t)g.vec_rows + 1), hi = g.thresh;
  constexpr bool kSplit = F == NF4 && RB == 1;   // per-block MFMA partials, shared table
  // 16-row NF4 units decode through the 32-copy byte table in LDS (two VALU
  // instructions and one conflict-free LDS read per code byte)
  __shared__ __attribute__((aligned(16))) uint32_t blut[kSplit ? nf4_byte_lut_words<32>() : 4];
  const int32_t total = build_plan(
      poff, pupre, g.sizes, g.E, g.M, g.err,
      [&](int32_t s) -> int32_t { return (s >= lo && s <= hi) ? ((s + RPU - 1) / RPU) * n_cols : 0; },
      [&] {
        if constexpr (kSplit) nf4_byte_lut_fill<32>(blut);   // ordered by the plan's barrier
      });
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t K = g.K, N = g.N;
  const int nst = (int)((K + kNStep - 1) / kNStep);
  uint32_t range = 0;
  uint32_t m4, base;
  nf4_selector_consts(m4, base);
  constexpr int kNsc = kSplit ? 2 : 1;
  static_assert(!SSC || kSplit, "staged scales serve the 16-row NF4 units");
  constexpr int kSscLd = 34;                       // floats per staged row (even, bank-spreading)
  __shared__ __attribute__((aligned(16))) float Ssc[SSC ? 64 * CBW * kSscLd : 2];
  const uint32_t lane_off = nf4_byte_lut_lane<32>(lane);
  if (t < 2 * RB)
    *reinterpret_cast<u32x4*>(&As[t / RB][(t % RB) * kRBlk + kRBlk - 8]) = u32x4{0u, 0u, 0u, 0u};
  // A operand offsets within a stage buffer for MFMA j of row block 0 (row
  // l%16, chunk 4 (l/16) + j; block r adds r * kRBlk): NF4 splits them by
  // 64-block, `ab[h]` reading the zero chunk on the lanes of the other block
  const int am = lane & 15, ag = lane >> 4;
  int ab[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int real = nswz(am, 4 * ag + j);
    ab[0][j] = (!kSplit || ag < 2) ? real : kRBlk - 8;
    ab[1][j] = ag >= 2 ? real : kRBlk - 8;
  }

  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(pupre, g.E, u);
    const int32_t lu = u - pupre[e];
    const int64_t row0 = poff[e] + (int64_t)(lu / n_cols) * RPU;
    const int rows = (int)min<int64_t>(RPU, poff[e + 1] - row0);
    const int64_t n0 = (int64_t)(lu % n_cols) * CPU + 16 * CBW * wave;
    const __amdgpu_buffer_rsrc_t A = nrsrc(g.a + row0 * K, (int64_t)rows * K * 2);
    const __amdgpu_buffer_rsrc_t W = nrsrc(g.wq + (int64_t)e * N * (K >> 1), N * (K >> 1));
    const __amdgpu_buffer_rsrc_t S =
        F == NF4 ? nrsrc(reinterpret_cast<const float*>(g.scales) + (int64_t)e * N * (K >> 6), N * (K >> 6) * 4)
                 : nrsrc(reinterpret_cast<const uint8_t*>(g.scales) + (int64_t)e * N * (K >> 5), N * (K >> 5));

    f32x4 acc[RB][CBW];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) acc[r][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // stage the activations of step st (registers -> LDS buffer st % 2)
    auto stage = [&](const StepRaw<RB, CBW, kNsc>& r, int st) {
      uint16_t* Ab = As[st & 1];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        u32x4 v = r.a[q];
        if constexpr (kSplit)
          v = bf16x8_to_f16(v, range);        // natural order, as the byte table decodes
        else if constexpr (F == NF4)
          v = bf16x8_to_f16_slots(v, range);
        *reinterpret_cast<u32x4*>(&Ab[nswz(16 * q + (t >> 4), t & 15)]) = v;
      }
    };
    // staged scales: thread t loads 8 absmax values (blocks 8 (t%4) .. +7) of
    // unit row t/4 (rows past N read as zero; blocks past the row read the next
    // row's values, which only meet zero partial sums)
    constexpr int kSscTpr = 4 / CBW;                 // threads per staged row
    constexpr int kSscQ = 2 * CBW;                   // 16-byte loads per thread
    u32x4 sraw[kSscQ];
    if constexpr (SSC) {
      static_assert(kThreads == 256 && (CBW == 1 || CBW == 2), "256 threads cover 64 CBW rows of 32 blocks");
      const int64_t nrow = (int64_t)(lu % n_cols) * CPU + t / kSscTpr;
      const uint32_t off = (uint32_t)((nrow * (K >> 6) + 8 * CBW * (t % kSscTpr)) * 4);
#pragma unroll
      for (int q = 0; q < kSscQ; ++q) sraw[q] = __builtin_amdgcn_raw_buffer_load_b128(S, off + 16 * q, 0, 0);
    }
    StepRaw<RB, CBW, kNsc> raw[NS];
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) load_step<F, RB, CBW, kNsc, SSC>(raw[i], A, W, S, K, N, n0, i, lane);
    __syncthreads();   // the previous unit is done with both LDS buffers and the scales
    stage(raw[0], 0);
    if constexpr (SSC) {
      float* dst = &Ssc[(t / kSscTpr) * kSscLd + 8 * CBW * (t % kSscTpr)];
#pragma unroll
      for (int q = 0; q < 2 * kSscQ; ++q)
        *reinterpret_cast<u32x2*>(dst + 2 * q) = u32x2{sraw[q >> 1][2 * (q & 1)], sraw[q >> 1][2 * (q & 1) + 1]};
    }
    __syncthreads();

    // Step st: stage st+1, load st+NS-1, compute st from LDS buffer st % 2 and
    // the step's weight registers. raw[] rotates through NS slots (compile-time
    // indices: the loop body covers NS steps). Loads of steps past the last read
    // zeros (their offsets lie past every buffer) and the stage they fill is never
    // read, so every step issues the same loads and the waits for them are
    // counted exactly; full groups of NS steps run without branches, and the last
    // nst % NS steps follow.
    auto step = [&](int jn, int st) {
          // the scheduler would otherwise pull the next steps' decode ahead of
          // this step's, and with it waits for loads that are still in flight
          __builtin_amdgcn_sched_barrier(0);
          StepRaw<RB, CBW, kNsc>& cur = raw[jn];
          stage(raw[(jn + 1) % NS], st + 1);
          load_step<F, RB, CBW, kNsc, SSC>(raw[(jn + NS - 1) % NS], A, W, S, K, N, n0, st + NS - 1, lane);
          const uint16_t* Ab = As[st & 1];
#pragma unroll
          for (int cb = 0; cb < CBW; ++cb) {
            if constexpr (F == NF4 && !kSplit) {
              // 32-row units: a per-lane table scaled by the absmax of the lane's
              // piece (one mixed-precision fma per entry), one MFMA per row block
              Lut16 sl;
              const float sc = __builtin_bit_cast(float, cur.s[cb][0]);
#pragma unroll
              for (int q = 0; q < 4; ++q) nf4_scaled_lut_quarter_mix(sc, q, sl);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4 b = nf4_decode8(sl, cur.w[cb][j]);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                  acc[r][cb] = mfma16<NF4>(*reinterpret_cast<const u32x4*>(&Ab[ab[0][j] + r * kRBlk]), b, acc[r][cb]);
              }
            } else if constexpr (kSplit) {
              // 16-row units: the step's two 64-blocks as separate MFMA partial
              // sums, each scaled by its absmax
              f32x4 part[2][RB];
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < RB; ++r) part[h][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4 b = nf4_byte_lut_decode8<32>(blut, cur.w[cb][j], lane_off);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                  for (int r = 0; r < RB; ++r)
                    part[h][r] = mfma16<NF4>(*reinterpret_cast<const u32x4*>(&Ab[ab[h][j] + r * kRBlk]), b, part[h][r]);
              }
              float s0, s1;
              if constexpr (SSC) {
                const float2 sv = *reinterpret_cast<const float2*>(
                    &Ssc[(16 * (CBW * wave + cb) + (lane & 15)) * kSscLd + 2 * st]);
                s0 = sv.x;
                s1 = sv.y;
              } else {
                s0 = __builtin_bit_cast(float, cur.s[cb][0]);
                s1 = __builtin_bit_cast(float, cur.s[cb][1]);
              }
#pragma unroll
              for (int r = 0; r < RB; ++r) acc[r][cb] += s0 * part[0][r] + s1 * part[1][r];
            } else {
              const float sc = e8m0_to_f32(cur.s[cb][0]);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4 b = mxfp4_decode8(cur.w[cb][j], sc);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                  acc[r][cb] = mfma16<MXFP4>(*reinterpret_cast<const u32x4*>(&Ab[ab[0][j] + r * kRBlk]), b, acc[r][cb]);
              }
            }
          }
          __syncthreads();   // buffer st+1 complete; buffer st free for step st+2
    };
    const int full = nst - nst % NS;
    for (int s0 = 0; s0 < full; s0 += NS) {
#pragma unroll
      for (int jn = 0; jn < NS; ++jn) step(jn, s0 + jn);
    }
#pragma unroll
    for (int jn = 0; jn < NS - 1; ++jn)
      if (full + jn < nst) step(jn, full + jn);
    // acc[r][cb][q]: activation row 16r + 4 (l/16) + q, weight row n0 + 16 cb + l%16
    if (g.glu) {
      // fused expert block: weight rows 2c, 2c+1 (lanes l, l ^ 1) are the gate
      // and up of unit c; the even lane writes out[row, c] of the [M, N/2] output
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) {
        const int64_t n = n0 + 16 * cb + (lane & 15);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float up = lane_pair_swap(acc[r][cb][q]);
            const int lr = 16 * r + 4 * (lane >> 4) + q;
            if (!(lane & 1) && n < N && lr < rows)
              g.out[(row0 + lr) * (N >> 1) + (n >> 1)] = to_bf16(swiglu(acc[r][cb][q], up));
          }
      }
      continue;
    }
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
      const int64_t n = n0 + 16 * cb + (lane & 15);
      if (n < N) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int lr = 16 * r + 4 * (lane >> 4) + q;
            if (lr < rows) g.out[(row0 + lr) * N + n] = to_bf16(acc[r][cb][q]);
          }
      }
    }
  }
  if constexpr (F == NF4) {
    if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
  }
}

template <Fmt F, int RB, int CBW, int NS, bool SSC = false>
hipError_t launch_n(const GemmArgs& g, int cus, hipStream_t s) {
  auto k = narrow_kernel<F, RB, CBW, NS, SSC>;
  const size_t dyn = (size_t)2 * (g.E + 1) * sizeof(int32_t);
  static size_t cached_dyn = 0;
  static int per_cu = 0;
  if (per_cu == 0 || cached_dyn != dyn) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, kThreads, dyn) != hipSuccess || b <= 0) b = 1;
    per_cu = b;
    cached_dyn = dyn;
  }
  constexpr int RPU = 16 * RB, CPU = 64 * CBW;
  const int64_t chunks = (g.M + RPU - 1) / RPU + std::min<int64_t>(g.E, g.M);
  const int64_t units = chunks * ((g.N + CPU - 1) / CPU);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(units, (int64_t)per_cu * cus));
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), dyn, s, g);
  return hipGetLastError();
}

template <Fmt F>
hipError_t launch_narrow_fmt(const GemmArgs& g, int cus, hipStream_t s) {
  // 32-row units (two 16-row blocks per wavefront, 128 weight rows per unit) when
  // the batch's experts are expected to hold more than 16 rows; otherwise 16-row
  // units over 64 weight rows (more, smaller units keep more wavefronts busy).
  if (g.thresh > 16 && g.M > 16 * (int64_t)std::min<int64_t>(g.E, g.M)) return launch_n<F, 2, 2, 3>(g, cus, s);
  if constexpr (F == NF4) {
    if (g.K <= 2048) return launch_n<F, 1, 1, 4, true>(g, cus, s);
  }
  return launch_n<F, 1, 1, 4>(g, cus, s);
}

}  // namespace

hipError_t launch_narrow(int fmt, const GemmArgs& g, int cus, hipStream_t s) {
  return fmt == NF4 ? launch_narrow_fmt<NF4>(g, cus, s) : launch_narrow_fmt<MXFP4>(g, cus, s);
}

}  // namespace geg
