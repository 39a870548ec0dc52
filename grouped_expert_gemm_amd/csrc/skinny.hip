// Skinny (decode-shape) path of the grouped 4-bit GEMM.
//
// For experts with few routed rows (one token broadcast over its top-k slots is
// the decode case: "grouped-nf4-gemm releases", v0.4.0/0.3.1 correction note)
// the work is bound by streaming packed weight bytes. Each weight byte is read
// from HBM exactly once and decoded once in registers; a wavefront's decoded
// weight rows are the B operand of 16x16x32 MFMAs whose A operand is the
// expert's (at most 32, zero-padded) activation rows, staged once per workgroup
// in LDS. The weights are not re-streamed per activation row, which the pages
// list as the limit of their decode GEMV ("grouped-nf4-gemm capability index",
// limitations).
//
// Work unit: (expert, chunk of <= 32 activation rows, 16*CB weight rows, K split
// s). The four wavefronts of a workgroup split the unit's K range (128-k step i
// goes to wavefront i % 4) and add their fp32 partial sums in LDS in fixed order.
// Every workgroup first stages its activations, then issues the loads of all its
// weight bytes (in groups of D steps, the next group in flight while the current
// one is decoded), so one pass over the grid keeps the whole weight stream in
// flight. With S > 1 (split-K across workgroups, listed by the capability index
// under system_manifest.owns) every unit writes fp32 partials of its K range and
// a second launch adds the S partials in order s = 0..S-1, so results never
// depend on which workgroup finished first.
//
// NF4: codes decode through an unscaled fp16 copy of the table; the fp32 absmax
// multiplies the fp32 MFMA partial sum of each 64-wide block (all 32 k of an MFMA
// step lie in one block by construction of the lane layout below). MXFP4: the
// gfx950 scaled fp4 -> bf16 conversion applies 2^(e8m0-127) while decoding.
#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int kWaves = kThreads / 64;
constexpr int kALdsHalves = 34 * 1024;  // 68 KiB of staged activations (two workgroups per CU)
constexpr int kAPad = 8;                // LDS row padding (halves)

// K covered by one staged activation chunk for r8 (rows rounded up to 8) rows.
__device__ __forceinline__ int chunk_k(int r8, int64_t K) {
  const int cap = ((kALdsHalves / r8 - kAPad) / kKStep) * kKStep;
  return (int)min<int64_t>((int64_t)cap, ((K + kKStep - 1) / kKStep) * kKStep);
}

template <Fmt F, int CB, int D>
struct Group {
  // NF4: per step and column block two 8-byte pieces (k in [16kg, 16kg+16) of
  // each 64-block of the step) and two absmax values. MXFP4: 16 bytes (k in
  // [32kg, 32kg+32)) and that 32-block's e8m0 byte (carried in a float slot).
  u32x4 code[D][CB];
  float scale[D][CB][2];
};

// Loads of one group of D steps (steps first_step + 4i, i < nsteps; nsteps is
// uniform across the wavefront). Addresses are clamped into the tensors instead
// of predicating loads; nothing here consumes a loaded value, so the loads of a
// group stay in flight until compute_group uses them. Weight rows n >= N only
// feed output columns that are never stored; a K tail is zeroed through its
// scale at use time (NF4: absmax 0; MXFP4: scale 0).
template <Fmt F, int CB, int D>
__device__ __forceinline__ void load_group(Group<F, CB, D>& r, const GemmArgs& g, int e,
                                           int64_t n0, int kg, int first_step, int nsteps) {
  const int64_t K = g.K;
  const bool pair_scales = (K & 127) == 0 && (reinterpret_cast<uintptr_t>(g.scales) & 7) == 0;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    if (i < nsteps) {
      const int64_t k0 = (int64_t)(first_step + kWaves * i) * kKStep;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t n = n0 + 16 * cb;
        const int64_t rowbase = (int64_t)e * g.N + (n < g.N ? n : g.N - 1);
        const uint8_t* wrow = g.wq + rowbase * (K >> 1);
        if constexpr (F == NF4) {
          // k0 + 64 <= K for every step inside K (K % 64 == 0); the step's second
          // 64-block exists iff k0 + 128 <= K (the same for all lanes).
          const int64_t kb = k0 + 64 < K ? k0 + 64 : k0;
          const float* srow = reinterpret_cast<const float*>(g.scales) + rowbase * (K >> 6);
          const u32x2 pa = *reinterpret_cast<const u32x2*>(wrow + ((k0 + 16 * kg) >> 1));
          const u32x2 pb = *reinterpret_cast<const u32x2*>(wrow + ((kb + 16 * kg) >> 1));
          r.code[i][cb] = u32x4{pa[0], pa[1], pb[0], pb[1]};
          if (pair_scales) {
            // both absmax of the step in one 8-byte load (k0 / 64 is even and the
            // scale rows are 8-byte aligned)
            const u32x2 sv = *reinterpret_cast<const u32x2*>(srow + (k0 >> 6));
            const uint32_t s0 = sv.x, s1 = sv.y;   // scalar copies before the bit casts
            r.scale[i][cb][0] = __builtin_bit_cast(float, s0);
            r.scale[i][cb][1] = __builtin_bit_cast(float, s1);
          } else {
            r.scale[i][cb][0] = srow[k0 >> 6];
            r.scale[i][cb][1] = srow[kb >> 6];
          }
        } else {
          const int64_t ka = k0 + 32 * kg;
          const int64_t kc = ka < K ? ka : K - 32;
          r.code[i][cb] = *reinterpret_cast<const u32x4*>(wrow + (kc >> 1));
          r.scale[i][cb][0] = __builtin_bit_cast(
              float, (uint32_t)reinterpret_cast<const uint8_t*>(g.scales)[rowbase * (K >> 5) + (kc >> 5)]);
          r.scale[i][cb][1] = 0.f;
        }
      }
    }
  }
}

// MFMAs of one group of D steps (steps first_step + 4i, chunk-relative k offset
// kofs0 + 512 i). Activation rows >= r8 read as zero (their LDS address is clamped
// to row 0 and the value discarded).
template <Fmt F, int CB, int D, int G>
__device__ __forceinline__ void compute_group(const Group<F, CB, D>& r, const Lut16& lut,
                                              const uint16_t* As, int ld, int r8, int64_t kabs0,
                                              int64_t K, int kofs0, int nsteps, int kg, int col,
                                              f32x4 (&acc)[G][CB]) {
  bool arow_ok[G];
  int arow_off[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int ar = 16 * gi + col;
    arow_ok[gi] = ar < r8;
    arow_off[gi] = (arow_ok[gi] ? ar : 0) * ld;
  }
  auto load_a = [&](int gi, int kk) -> u32x4 {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&As[arow_off[gi] + kk]);
    return arow_ok[gi] ? v : u32x4{0u, 0u, 0u, 0u};
  };
#pragma unroll
  for (int i = 0; i < D; ++i) {
    if (i < nsteps) {
      const int kstep = kofs0 + kWaves * i * kKStep;
      const bool b_ok = kabs0 + (int64_t)kstep + 64 < K;   // second 64-block inside K
      const bool a_ok = kabs0 + (int64_t)kstep + 32 * kg < K;  // this lane's 32-block inside K
      if constexpr (F == NF4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // 64-wide absmax block h of the step
          f32x4 part[G][CB];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int kk = kstep + 64 * h + 16 * kg + 8 * jj;
            u32x4 a[G];
#pragma unroll
            for (int gi = 0; gi < G; ++gi) a[gi] = load_a(gi, kk);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
              const u32x4 b = nf4_decode8(lut, r.code[i][cb][2 * h + jj]);
#pragma unroll
              for (int gi = 0; gi < G; ++gi)
                part[gi][cb] = mfma16<NF4>(a[gi], b, jj == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[gi][cb]);
            }
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const float s = (h == 0 || b_ok) ? r.scale[i][cb][h] : 0.f;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) acc[gi][cb] += s * part[gi][cb];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kk = kstep + 32 * kg + 8 * j;
          u32x4 a[G];
#pragma unroll
          for (int gi = 0; gi < G; ++gi) a[gi] = load_a(gi, kk);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const uint32_t sbyte = __builtin_bit_cast(uint32_t, r.scale[i][cb][0]);
            const u32x4 b = mxfp4_decode8(r.code[i][cb][j], a_ok ? e8m0_to_f32(sbyte) : 0.f);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) acc[gi][cb] = mfma16<MXFP4>(a[gi], b, acc[gi][cb]);
          }
        }
      }
    }
  }
}

// One unit's K range for G (1 or 2) groups of 16 activation rows: stage the
// activations, stream the weights, return this wavefront's partial sums.
template <Fmt F, int CB, int G>
__device__ __forceinline__ void unit_k_loop(const GemmArgs& g, const Lut16& lut, uint16_t* As,
                                            int e, int64_t row0, int rows, int r8, int kc,
                                            int step_begin, int step_end, int64_t n0, int wave,
                                            int kg, int col, uint32_t& range,
                                            f32x4 (&acc)[G][CB]) {
  constexpr int D = 4 / CB;  // steps per prefetch group
  constexpr int NB = CB == 4 ? 3 : 4;   // groups in flight (as many as the registers hold)
  const int ld = kc + kAPad;
  const int chunk_steps = kc / kKStep;
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[gi][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = step_begin; c0 < step_end; c0 += chunk_steps) {
    const int csteps = min(chunk_steps, step_end - c0);
    // This wavefront's steps of the chunk: c0 + wave + 4i, in groups of D.
    const int my_steps = csteps > wave ? (csteps - wave + kWaves - 1) / kWaves : 0;
    // Activations [r8 rows (rows >= `rows` are zero), k in this chunk], 8 per
    // group, AB loads per thread in flight together.
    constexpr int AB = F == NF4 ? 8 : 4;
    const int64_t kbase = (int64_t)c0 * kKStep;
    const int gpr = csteps * (kKStep / 8);  // 8-element groups per row
    const int ngroups = r8 * gpr;
    u32x4 av[AB];
    auto a_load = [&](int q0) {
#pragma unroll
      for (int b = 0; b < AB; ++b) {
        const int q = q0 + b * kThreads;
        const int rr = q / gpr;
        const int64_t k = kbase + (q % gpr) * 8;
        av[b] = u32x4{0u, 0u, 0u, 0u};
        if (q < ngroups && rr < rows && k < g.K)
          av[b] = *reinterpret_cast<const u32x4*>(g.a + (row0 + rr) * g.K + k);
      }
    };
    auto a_store = [&](int q0) {
#pragma unroll
      for (int b = 0; b < AB; ++b) {
        const int q = q0 + b * kThreads;
        if (q < ngroups) {
          u32x4 v = av[b];
          if constexpr (F == NF4) v = bf16x8_to_f16_slots(v, range);
          *reinterpret_cast<u32x4*>(&As[(q / gpr) * ld + (q % gpr) * 8]) = v;
        }
      }
    };
    // (NF4 issues its first activation loads ahead of the weights; for MXFP4 the
    // extra live registers cost more occupancy than the overlap gains.)
    if constexpr (F == NF4) a_load(threadIdx.x);
    // The first NB groups of weight loads go out before the activations are
    // staged, so that the whole unit's weight stream is requested at once when it
    // fits (the common decode case) and staging overlaps the weights' latency.
    Group<F, CB, D> b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j * D < my_steps)
        load_group<F, CB, D>(b[j], g, e, n0, kg, c0 + wave + kWaves * j * D, min(D, my_steps - j * D));
    __syncthreads();  // LDS reads of the previous chunk are done
    if constexpr (F != NF4) a_load(threadIdx.x);
    a_store(threadIdx.x);
    for (int q0 = threadIdx.x + AB * kThreads; q0 < ngroups; q0 += AB * kThreads) {
      a_load(q0);
      a_store(q0);
    }
    __syncthreads();
    // NB register buffers rotate: a buffer is reloaded with the group NB ahead as
    // soon as it has been decoded.
    for (int s0 = 0; s0 < my_steps; s0 += NB * D) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int s = s0 + j * D;
        if (s < my_steps) {
          compute_group<F, CB, D, G>(b[j], lut, As, ld, r8, (int64_t)c0 * kKStep, g.K,
                                     (wave + kWaves * s) * kKStep, min(D, my_steps - s), kg, col, acc);
          if (s + NB * D < my_steps)
            load_group<F, CB, D>(b[j], g, e, n0, kg, c0 + wave + kWaves * (s + NB * D),
                                 min(D, my_steps - s - NB * D));
        }
      }
    }
  }
}

// Add the four wavefronts' partial sums in fixed order (wave 0 + 1 + 2 + 3) and
// write the unit's rows (bf16 output, or fp32 partials of split ks).
template <int CB, int G>
__device__ __forceinline__ void unit_store(const GemmArgs& g, f32x4 (&acc)[G][CB],
                                           f32x4 (*red)[2 * CB][64], int wave, int lane, int kg,
                                           int64_t row0, int rows, int64_t n0, int ks) {
  __syncthreads();  // every wavefront is done reading activations from As
  if (wave > 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) red[wave - 1][gi * CB + cb][lane] = acc[gi][cb];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[gi][cb] += red[w][gi * CB + cb][lane];
    // acc[gi][cb][q] is row 16*gi + 4*kg + q of the row chunk, column n0 + 16*cb.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int64_t n = n0 + 16 * cb;
      if (n < g.N) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int lr = 16 * gi + 4 * kg + q;
            if (lr < rows) {
              if (g.split == 1)
                g.out[(row0 + lr) * g.N + n] = to_bf16(acc[gi][cb][q]);
              else
                g.partials[((int64_t)ks * g.M + row0 + lr) * g.N + n] = acc[gi][cb][q];
            }
          }
      }
    }
  }
}

template <Fmt F, int CB>
__global__ __launch_bounds__(kThreads, 2) void skinny_kernel(GemmArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) uint16_t As[kALdsHalves];
  // After the K loop the activation buffer holds the cross-wavefront partial sums.
  f32x4 (*red)[2 * CB][64] = reinterpret_cast<f32x4 (*)[2 * CB][64]>(As);
  static_assert((kWaves - 1) * 2 * CB * 64 * sizeof(f32x4) <= sizeof(As), "reduction buffer");

  const int S = g.split;
  const int cols = kSkinnyCols * CB;
  const int n_chunks = (int)((g.N + cols - 1) / cols);
  const int32_t thresh = g.thresh;
  const int64_t lo = max<int64_t>(1, (int64_t)g.vec_rows + 1);   // smaller experts take the vector path
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    if (s < lo || s > thresh) return 0;
    return ((s + kSkinnyRows - 1) / kSkinnyRows) * n_chunks * S;
  });

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int kg = lane >> 4;
  const int col = lane & 15;
  const int KS = (int)((g.K + kKStep - 1) / kKStep);
  const int kps = (KS + S - 1) / S;
  uint32_t range = 0;

  // Unscaled fp16 NF4 table for the lookups (the absmax multiplies partial sums).
  Lut16 lut{};
  if constexpr (F == NF4) lut = nf4_scaled_lut(1.0f);

  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, g.E, u);
    int32_t lu = u - plan.upre[e];
    const int ks = lu % S;
    lu /= S;
    const int chunk = lu % n_chunks;
    const int rcl = lu / n_chunks;
    const int64_t row0 = (int64_t)plan.off[e] + (int64_t)rcl * kSkinnyRows;
    const int rows = min(kSkinnyRows, (int)(plan.off[e + 1] - row0));
    const int r8 = (rows + 7) & ~7;
    const int kc = chunk_k(r8, g.K);
    const int64_t n0 = (int64_t)chunk * cols + col;
    const int step_begin = min(KS, ks * kps);
    const int step_end = min(KS, step_begin + kps);

    if (rows <= 16) {
      f32x4 acc[1][CB];
      unit_k_loop<F, CB, 1>(g, lut, As, e, row0, rows, r8, kc, step_begin, step_end, n0, wave, kg,
                            col, range, acc);
      unit_store<CB, 1>(g, acc, red, wave, lane, kg, row0, rows, n0, ks);
    } else {
      f32x4 acc[2][CB];
      unit_k_loop<F, CB, 2>(g, lut, As, e, row0, rows, r8, kc, step_begin, step_end, n0, wave, kg,
                            col, range, acc);
      unit_store<CB, 2>(g, acc, red, wave, lane, kg, row0, rows, n0, ks);
    }

    __syncthreads();  // red[] is reused by the next unit
  }
  if constexpr (F == NF4) {
    if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
  }
}

// Split-K reduce (S > 1): out[row, n] = bf16(partials[0, row, n] + ... +
// partials[S - 1, row, n]), added in that order, for every row of the experts the
// skinny kernel took. A launch of its own: the kernel boundary orders every
// partial store before these loads on all XCDs, where a reduction by the last
// workgroup to arrive would need a device-scope release, a write-back of its
// XCD's L2, from every unit. One unit = one row and kThreads consecutive
// columns; each thread issues the S loads of its element before adding them.
constexpr int kMaxSplit = 16;
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(GemmArgs g) {
  __shared__ Plan plan;
  const int32_t thresh = g.thresh;
  const int64_t lo = max<int64_t>(1, (int64_t)g.vec_rows + 1);
  const int32_t n_blk = (int32_t)((g.N + kThreads - 1) / kThreads);
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    return (s < lo || s > thresh) ? 0 : s * n_blk;
  });
  const int S = g.split;
  const int64_t slice = g.M * g.N;
  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, g.E, u);
    const int32_t lu = u - plan.upre[e];
    const int64_t row = (int64_t)plan.off[e] + lu / n_blk;
    const int64_t n = (int64_t)(lu % n_blk) * kThreads + threadIdx.x;
    if (n >= g.N) continue;
    const float* p = g.partials + row * g.N + n;
    float v[kMaxSplit];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) v[s] = s < S ? p[s * slice] : 0.f;
    float sum = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSplit; ++s)
      if (s < S) sum += v[s];
    g.out[row * g.N + n] = to_bf16(sum);
  }
}

template <Fmt F>
hipError_t launch_fmt(const GemmArgs& g, int grid, hipStream_t s) {
  switch (g.cb) {
    case 4: hipLaunchKernelGGL((skinny_kernel<F, 4>), dim3(grid), dim3(kThreads), 0, s, g); break;
    case 2: hipLaunchKernelGGL((skinny_kernel<F, 2>), dim3(grid), dim3(kThreads), 0, s, g); break;
    default: hipLaunchKernelGGL((skinny_kernel<F, 1>), dim3(grid), dim3(kThreads), 0, s, g); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  return fmt == NF4 ? launch_fmt<NF4>(g, grid, s) : launch_fmt<MXFP4>(g, grid, s);
}

hipError_t launch_splitk_reduce(const GemmArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
