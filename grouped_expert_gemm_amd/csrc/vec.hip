// Vector (token-decode) path of the grouped 4-bit GEMM: experts with few routed
// rows, taken RV at a time.
//
// One token broadcast over its top-k experts gives each of them a single row
// ("grouped-nf4-gemm releases", v0.4.0/0.3.1 correction note); at that shape the
// work is a matrix-vector product per expert, bound by streaming the packed
// weight bytes. Matrix cores would waste 15 of every 16 rows here, so this path
// uses packed dot products on the vector ALUs and spends its effort on the memory
// side: the weight rows of an expert are one contiguous byte range, and every
// load instruction of a wavefront reads whole rows of it (1 KiB for K = 2048),
// the unit's row loads all in flight at once.
//
// Work unit: one wavefront, one expert, up to RV (4, or 1 for the smallest
// batches) of its activation rows, U (4 or 8) row groups of G = 64 / LPR weight
// rows (LPR lanes per row: 64, or 32 for rows of at most 32 chunks). Lane l of a
// row group owns the 16-byte chunks c = l % LPR + LPR i of its row (32 codes, k in
// [32c, 32c + 32)); it decodes them in registers, takes packed fp32-accumulated
// dot products with the activation rows' slice of that chunk, and the row group's
// lanes add their partial sums with cross-lane shuffles. Wavefronts are
// independent (LDS holds only the routing plan and the NF4 byte table, both
// written before the one barrier).
//
// NF4: code bytes go through the unscaled fp16 byte table in LDS (one 32-bit
// read per two codes, natural k order); the fp32 absmax of the chunk's 64-block
// scales the chunk's fp32 dot product (activations as fp16, range-checked as in
// the other paths). The 64 KiB table leaves room for two workgroups per CU. MXFP4: the gfx950 scaled fp4
// -> bf16 conversion applies 2^(e8m0-127); bf16 activations pair with the decoded
// bf16 values in natural order.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t vrsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c,
                                         false);
}

// Sum over the LPR lanes of a row group (LPR = 64 or 32).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <Fmt F, int LPR, int RV, int U>
__device__ __forceinline__ void vec_unit(const GemmArgs& g, const uint32_t* blut, int e, int64_t n0,
                                         int64_t row0, int rows, int lane, uint32_t& range) {
  constexpr int G = 64 / LPR;
  const int64_t N = g.N, K = g.K;
  const int C = (int)(K >> 5);             // 16-byte chunks per weight row
  const int gl = lane / LPR, li = lane % LPR;
  const __amdgpu_buffer_rsrc_t W = vrsrc(g.wq + (int64_t)e * N * (K >> 1), N * (K >> 1));
  const __amdgpu_buffer_rsrc_t S =
      F == NF4 ? vrsrc(reinterpret_cast<const float*>(g.scales) + (int64_t)e * N * (K >> 6), N * (K >> 6) * 4)
               : vrsrc(reinterpret_cast<const uint8_t*>(g.scales) + (int64_t)e * N * (K >> 5), N * (K >> 5));
  const __amdgpu_buffer_rsrc_t A = vrsrc(g.a + row0 * K, (int64_t)rows * K * 2);
  const uint32_t lane_off = nf4_byte_lut_lane(lane);
  float acc[U][RV];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < RV; ++m) acc[u][m] = 0.f;

  for (int c0 = 0; c0 < C; c0 += LPR) {
    const int c = c0 + li;
    // chunks past the row read as zero: their offsets are pushed past every
    // buffer's end (an OR, so that the loads stay unpredicated)
    const uint32_t off_mask = c < C ? 0u : 0xFFFFFFF0u;
    // activation slice k in [32c, 32c + 32) of rows m < RV (rows >= `rows` and
    // chunks past the row read as zero), then the weight loads row group by row
    // group: loads complete in issue order, so row group u can be decoded while
    // the later ones are still in flight
    u32x4 av[RV][4];
#pragma unroll
    for (int m = 0; m < RV; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t ao = (uint32_t)((m * K + 32 * c) * 2 + 16 * j) | off_mask;
        av[m][j] = __builtin_amdgcn_raw_buffer_load_b128(A, ao, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);   // keep the issue order (waits count in order)
    u32x4 code[U];
    uint32_t sraw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = n0 + G * u + gl;   // rows past N read as zero (buffer bounds)
      const uint32_t wo = (uint32_t)(n * (K >> 1) + 16 * c) | off_mask;
      code[u] = __builtin_amdgcn_raw_buffer_load_b128(W, wo, 0, 0);
      if constexpr (F == NF4) {
        const uint32_t so = (uint32_t)((n * (K >> 6) + (c >> 1)) * 4) | off_mask;
        sraw[u] = __builtin_amdgcn_raw_buffer_load_b32(S, so, 0, 0);
      } else {
        const uint32_t so = (uint32_t)(n * (K >> 5) + c) | off_mask;
        sraw[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(S, so, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (F == NF4) {
#pragma unroll
      for (int m = 0; m < RV; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) av[m][j] = bf16x8_to_f16(av[m][j], range);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (F == NF4) {
        float d[RV];
#pragma unroll
        for (int m = 0; m < RV; ++m) d[m] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 w = nf4_byte_lut_decode8(blut, code[u][j], lane_off);   // k = 8j .. 8j+7
#pragma unroll
          for (int m = 0; m < RV; ++m)
            if (m < rows)
#pragma unroll
              for (int p = 0; p < 4; ++p) d[m] = dot2_f16(w[p], av[m][j][p], d[m]);
        }
        const float s = __builtin_bit_cast(float, sraw[u]);
#pragma unroll
        for (int m = 0; m < RV; ++m) acc[u][m] += s * d[m];
      } else {
        const float s = e8m0_to_f32(sraw[u]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 w = mxfp4_decode8(code[u][j], s);   // codes k = 8j .. 8j+7, natural order
#pragma unroll
          for (int m = 0; m < RV; ++m)
            if (m < rows)
#pragma unroll
              for (int p = 0; p < 4; ++p) acc[u][m] = dot2_bf16(w[p], av[m][j][p], acc[u][m]);
        }
      }
    }
  }
  if (g.glu) {
    // fused expert block: weight rows 2c, 2c+1 are the gate and up of unit c.
    // With one row group per wavefront (G = 1) they are row groups u, u+1 of the
    // same lanes; with two (G = 2) the same u of lane groups 0 and 1.
#pragma unroll
    for (int u = 0; u < U; u += (G == 1 ? 2 : 1)) {
      const int64_t n = n0 + G * u + gl;
#pragma unroll
      for (int m = 0; m < RV; ++m) {
        if (m < rows) {
          const float v = group_sum<LPR>(acc[u][m]);
          const float w = G == 1 ? group_sum<LPR>(acc[u + 1][m]) : __shfl_xor(v, 32, 64);
          if (lane == 0 && n < N) g.out[(row0 + m) * (N >> 1) + (n >> 1)] = to_bf16(swiglu(v, w));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t n = n0 + G * u + gl;
#pragma unroll
    for (int m = 0; m < RV; ++m) {
      if (m < rows) {
        const float v = group_sum<LPR>(acc[u][m]);
        if (li == 0 && n < N) g.out[(row0 + m) * N + n] = to_bf16(v);
      }
    }
  }
}

template <Fmt F, int LPR, int RV, int U>
__global__ __launch_bounds__(kThreads) void vec_kernel(GemmArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) uint32_t blut[F == NF4 ? kNf4ByteLutWords : 4];
  constexpr int RPU = U * (64 / LPR);   // weight rows per unit
  const int32_t n_units = (int32_t)((g.N + RPU - 1) / RPU);
  const int32_t vr = g.vec_rows;
  // an expert with s rows: ceil(s / RV) row chunks x n_units row blocks
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    return (s >= 1 && s <= vr) ? ((s + RV - 1) / RV) * n_units : 0;
  }, [&] {
    if constexpr (F == NF4) nf4_byte_lut_fill(blut);   // ordered by the plan's barrier
  });
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t range = 0;
  const int stride = gridDim.x * (kThreads / 64);
  for (int32_t u = blockIdx.x * (kThreads / 64) + wave; u < total; u += stride) {
    const int e = find_expert(plan, g.E, u);
    const int32_t lu = u - plan.upre[e];
    const int64_t n0 = (int64_t)(lu % n_units) * RPU;
    const int64_t row0 = plan.off[e] + (int64_t)(lu / n_units) * RV;
    const int rows = (int)min<int64_t>(RV, plan.off[e + 1] - row0);
    vec_unit<F, LPR, RV, U>(g, blut, e, n0, row0, rows, lane, range);
  }
  if constexpr (F == NF4) {
    if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
  }
}

// Resident workgroups per CU of a kernel (cached per kernel).
template <typename Kern>
int resident_per_cu(Kern k) {
  static int n = 0;
  if (n == 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, kThreads, 0) != hipSuccess || b <= 0) b = 1;
    n = b;
  }
  return n;
}

template <Fmt F, int LPR, int RV, int U>
hipError_t launch_one(const GemmArgs& g, int64_t units, int cus, hipStream_t s) {
  auto k = vec_kernel<F, LPR, RV, U>;
  const int64_t wgs = std::min<int64_t>((units + 3) / 4, (int64_t)resident_per_cu(k) * cus);
  hipLaunchKernelGGL(k, dim3((unsigned)std::max<int64_t>(1, wgs)), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

// Row groups per unit: 4, or 8 when units of 4 would not all be resident at
// once (a second round of units costs a whole load latency).
template <Fmt F, int LPR, int RV>
hipError_t launch_rv(const GemmArgs& g, int cus, hipStream_t s) {
  constexpr int G = 64 / LPR;
  // bound on row chunks (with one row per chunk, at most M)
  const int64_t chunks = RV == 1 ? g.M : (g.M + RV - 1) / RV + std::min<int64_t>(g.E, g.M);
  const int64_t units4 = chunks * ((g.N + 4 * G - 1) / (4 * G));
  const int64_t resident4 = (int64_t)resident_per_cu(vec_kernel<F, LPR, RV, 4>) * cus * 4;
  if (units4 <= resident4) return launch_one<F, LPR, RV, 4>(g, units4, cus, s);
  return launch_one<F, LPR, RV, 8>(g, chunks * ((g.N + 8 * G - 1) / (8 * G)), cus, s);
}

template <Fmt F, int LPR>
hipError_t launch_lpr(const GemmArgs& g, int cus, hipStream_t s) {
  // one activation row per unit for the smallest batches (a token's experts each
  // get one row): a quarter of the activation registers, more wavefronts resident
  return g.M <= kVecOneRowM ? launch_rv<F, LPR, 1>(g, cus, s) : launch_rv<F, LPR, 4>(g, cus, s);
}

template <Fmt F>
hipError_t launch_vec_fmt(const GemmArgs& g, int cus, hipStream_t s) {
  return (g.K >> 5) <= 32 ? launch_lpr<F, 32>(g, cus, s) : launch_lpr<F, 64>(g, cus, s);
}

}  // namespace

hipError_t launch_vec(int fmt, const GemmArgs& g, int cus, hipStream_t s) {
  return fmt == NF4 ? launch_vec_fmt<NF4>(g, cus, s) : launch_vec_fmt<MXFP4>(g, cus, s);
}

}  // namespace geg
