// Low-rank adapter delta on the grouped expert projection: the trainable B(Ax)
// composed with the frozen 4-bit projection at the pre-activation point, with
// its backward ("grouped-nf4-gemm releases", v0.2.4 section: the differentiable
// grouped GEMM). Per expert e, with A_e [r, K] and B_e [N, r] (fp32 master
// weights) and the layer's scale s:
//   forward   u = x A_e^T (fp32 [M, r], kept for the backward);  y += s u B_e^T
//   backward  g = s dy B_e (fp32 [M, r]);  dx += g A_e;
//             dB_e = s sum_rows dy^T u;  dA_e = sum_rows g^T x   (fp32)
// The contractions with a rank-wide side run on 16x16x32 bf16 MFMAs with every
// fp32 operand split into bf16 parts: x A^T here (bf16 x times A in three
// parts, about 24 significant bits: three instructions), u B^T and g A in the
// tiled kernel's epilogue (both sides in two parts, about 16 bits: three
// instructions, dropping lo x lo), where a plain bf16 operand keeps 8 bits. The delta joins the projection's fp32 accumulators before their one
// bf16 rounding. The contraction dimension is contiguous in both operands; the
// backward gets that from transposed fp32 copies of A and B. The reductions
// over rows for the adapter gradients run on the vector ALUs, one thread per
// column of the wide operand.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lrsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// offsets stay below 2^31; bit 31 moves an access past every record (reads 0)
__device__ __forceinline__ uint32_t l_oob_unless(bool ok, uint32_t off) { return off | ((uint32_t)!ok << 31); }

// Eight consecutive fp32 values of T at elem_off as three bf16 parts each
// (v = hi + mid + lo exactly up to the last bits of lo: about 24 significant
// bits); reads zeros when !ok (bit 31 puts the offset past every record).
struct Split8x3 {
  u32x4 hi, mid, lo;
};
__device__ __forceinline__ Split8x3 load8_split3(const __amdgpu_buffer_rsrc_t& R, uint32_t elem_off, bool ok) {
  const uint32_t b = (elem_off * 4u) | ((uint32_t)!ok << 31);
  const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(R, b, 0, 0);
  const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(R, b + 16u, 0, 0);
  Split8x3 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v0 = __uint_as_float(i < 2 ? p[2 * i] : q[2 * i - 4]);
    const float v1 = __uint_as_float(i < 2 ? p[2 * i + 1] : q[2 * i - 3]);
    const uint32_t h = pack_bf16x2(v0, v1);
    const float r0 = v0 - __uint_as_float(h << 16), r1 = v1 - __uint_as_float(h & 0xFFFF0000u);   // exact
    const uint32_t m = pack_bf16x2(r0, r1);
    t.hi[i] = h;
    t.mid[i] = m;
    t.lo[i] = pack_bf16x2(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xFFFF0000u));
  }
  return t;
}

// U[m, j] = s * sum_c X[m, c] T_e[j, c] for the rows m of each expert: X bf16
// [M, C], T fp32 [E, r, C], U fp32 [M, r]. One workgroup per block of 16 rows
// of one expert, all r columns (NCB = ceil(r / 16) column blocks, the last one
// partial when r % 16 == 8); its four wavefronts take interleaved batches of the
// contraction and are summed through LDS in wave order (deterministic).
// C % 8 == 0; rows past the expert read zeros.
template <int NCB>
__global__ __launch_bounds__(kThreads) void lora_down_kernel(const uint16_t* __restrict__ X, const float* __restrict__ T,
                                                             const int32_t* __restrict__ sizes, int32_t E, int64_t M,
                                                             int64_t C, int32_t r, float s, float* __restrict__ U,
                                                             uint32_t* err) {
  __shared__ Plan plan;
  __shared__ f32x4 red[3][NCB][64];
  const int32_t total = build_plan(plan, sizes, E, M, err, [](int32_t n) -> int32_t { return (n + 15) / 16; });
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, E, u);
    const int64_t row0 = plan.off[e] + (int64_t)(u - plan.upre[e]) * 16;
    const int rows = (int)min<int64_t>(16, plan.off[e + 1] - row0);
    const __amdgpu_buffer_rsrc_t RX = lrsrc(X + row0 * C, (int64_t)rows * C * 2);
    const __amdgpu_buffer_rsrc_t RT = lrsrc(T + (int64_t)e * r * C, (int64_t)r * C * 4);
    f32x4 acc[NCB] = {};
    // kU steps' loads are issued before their MFMAs; steps past C read zeros
    // through bit-31 offsets, so the batch has no branches
    constexpr int kU = NCB <= 2 ? 8 : 4;
    for (int64_t c00 = 32 * kU * wave; c00 < C; c00 += 32 * kU * 4) {
      u32x4 a[kU];
      Split8x3 b[kU][NCB];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int64_t c = c00 + 32 * q + 8 * g;
        const bool ok = c < C;
        a[q] = __builtin_amdgcn_raw_buffer_load_b128(RX, l_oob_unless(ok, (uint32_t)((r16 * C + c) * 2)), 0, 0);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int j = 16 * cb + r16;
          b[q][cb] = load8_split3(RT, (uint32_t)(j * C + c), ok && j < r);
        }
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          acc[cb] = mfma16<MXFP4>(a[q], b[q][cb].hi, acc[cb]);
          acc[cb] = mfma16<MXFP4>(a[q], b[q][cb].mid, acc[cb]);
          acc[cb] = mfma16<MXFP4>(a[q], b[q][cb].lo, acc[cb]);
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) red[wave - 1][cb][lane] = acc[cb];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] += red[w][cb][lane];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int j = 16 * cb + r16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr = 4 * g + q;
          if (lr < rows && j < r) U[(row0 + lr) * r + j] = s * acc[cb][q];
        }
      }
    }
    __syncthreads();   // red is reused by the next unit
  }
}

// G_e = s * sum over the rows m of expert e of Wd[m, c] Nw[m, j]: Wd bf16
// [M, Wc] (the wide operand), Nw fp32 [M, r]; G fp32 [E, Wc, r] (CJ) or
// [E, r, Wc] (JC). One workgroup per (expert, 256 columns), one thread per
// column; the narrow rows go through LDS 64 at a time and each thread issues the
// loads of 32 wide rows before their multiply-adds. Every expert gets its
// workgroups, so experts without rows write zeros.
template <bool JC, int R>
__global__ __launch_bounds__(kThreads) void lora_grad_kernel(const uint16_t* __restrict__ Wd,
                                                             const float* __restrict__ Nw,
                                                             const int32_t* __restrict__ sizes, int32_t E, int64_t M,
                                                             int64_t Wc, float s, float* __restrict__ G,
                                                             uint32_t* err) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) float nrow[64 * R];
  const int32_t nchunks = (int32_t)((Wc + kThreads - 1) / kThreads);
  const int32_t total = build_plan(plan, sizes, E, M, err, [&](int32_t) -> int32_t { return nchunks; });
  const int t = threadIdx.x;
  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, E, u);
    const int64_t c = (int64_t)(u - plan.upre[e]) * kThreads + t;
    const int64_t m0 = plan.off[e], m1 = plan.off[e + 1];
    float acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = 0.f;
    for (int64_t mb = m0; mb < m1; mb += 64) {
      const int nr = (int)min<int64_t>(64, m1 - mb);
      __syncthreads();   // the previous block's rows are consumed
      // rows past the expert's last one read as zeros (no stale or unset LDS)
      for (int i = 4 * t; i < 64 * R; i += 4 * kThreads)   // R % 8 == 0: whole 16-byte pieces
        *reinterpret_cast<float4*>(nrow + i) =
            i < nr * R ? *reinterpret_cast<const float4*>(Nw + mb * R + i) : float4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (c < Wc) {
        // rows past nr get offsets beyond the record and load zeros: no branches,
        // so all 32 loads of a batch are in flight before the multiply-adds
        const __amdgpu_buffer_rsrc_t RW = lrsrc(Wd + mb * Wc, (int64_t)nr * Wc * 2);
        for (int i0 = 0; i0 < nr; i0 += 32) {
          float w[32];
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const uint32_t off = l_oob_unless(i0 + k < nr, (uint32_t)(((int64_t)(i0 + k) * Wc + c) * 2));
            w[k] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(RW, off, 0, 0) << 16);
          }
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const float4* nv = reinterpret_cast<const float4*>(nrow + (i0 + k) * R);   // same address on every lane
#pragma unroll
            for (int j = 0; j < R / 4; ++j) {
              const float4 v = nv[j];
              acc[4 * j] += w[k] * v.x;
              acc[4 * j + 1] += w[k] * v.y;
              acc[4 * j + 2] += w[k] * v.z;
              acc[4 * j + 3] += w[k] * v.w;
            }
          }
        }
      }
    }
    if (c < Wc) {
#pragma unroll
      for (int j = 0; j < R; ++j)
        G[JC ? ((int64_t)e * R + j) * Wc + c : ((int64_t)e * Wc + c) * R + j] = s * acc[j];
    }
    __syncthreads();   // nrow is reused by the next unit
  }
}

// out[e, q, p] = in[e, p, q] for fp32 in [E, P, Qd] (32x32 tiles via LDS).
__global__ __launch_bounds__(kThreads) void lora_transpose_kernel(const float* __restrict__ in, int64_t E, int64_t P,
                                                                  int64_t Qd, float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int64_t tp = (P + 31) / 32, tq = (Qd + 31) / 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int64_t b = blockIdx.x; b < E * tp * tq; b += gridDim.x) {
    const int64_t e = b / (tp * tq), rem = b % (tp * tq), p0 = (rem / tq) * 32, q0 = (rem % tq) * 32;
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
      const int64_t p = p0 + i, q = q0 + tx;
      tile[i][tx] = (p < P && q < Qd) ? in[(e * P + p) * Qd + q] : 0.f;
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
      const int64_t q = q0 + i, p = p0 + tx;
      if (q < Qd && p < P) out[(e * Qd + q) * P + p] = tile[tx][i];
    }
  }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* X, const float* T, const int32_t* sizes, int32_t E, int64_t M, int64_t C,
                            int32_t r, float s, float* U, uint32_t* err, int cus, hipStream_t st) {
  const int64_t units = (M + 15) / 16 + std::min<int64_t>(E, M);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(units, (int64_t)cus * 16));
  switch ((r + 15) / 16) {
    case 1: hipLaunchKernelGGL(lora_down_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, st, X, T, sizes, E, M, C, r, s, U, err); break;
    case 2: hipLaunchKernelGGL(lora_down_kernel<2>, dim3((unsigned)grid), dim3(kThreads), 0, st, X, T, sizes, E, M, C, r, s, U, err); break;
    case 3: hipLaunchKernelGGL(lora_down_kernel<3>, dim3((unsigned)grid), dim3(kThreads), 0, st, X, T, sizes, E, M, C, r, s, U, err); break;
    case 4: hipLaunchKernelGGL(lora_down_kernel<4>, dim3((unsigned)grid), dim3(kThreads), 0, st, X, T, sizes, E, M, C, r, s, U, err); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool JC>
hipError_t launch_grad_r(const uint16_t* Wd, const float* Nw, const int32_t* sizes, int32_t E, int64_t M, int64_t Wc,
                         int32_t r, float s, float* G, uint32_t* err, int64_t grid, hipStream_t st) {
  switch (r) {
#define GEG_LORA_R(RR)                                                                                          \
  case RR:                                                                                                      \
    hipLaunchKernelGGL((lora_grad_kernel<JC, RR>), dim3((unsigned)grid), dim3(kThreads), 0, st, Wd, Nw, sizes, E, M, \
                       Wc, s, G, err);                                                                          \
    break;
    GEG_LORA_R(8) GEG_LORA_R(16) GEG_LORA_R(24) GEG_LORA_R(32) GEG_LORA_R(40) GEG_LORA_R(48) GEG_LORA_R(56)
    GEG_LORA_R(64)
#undef GEG_LORA_R
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lora_grad(const uint16_t* Wd, const float* Nw, const int32_t* sizes, int32_t E, int64_t M,
                            int64_t Wc, int32_t r, float s, float* G, bool jc, uint32_t* err, int cus, hipStream_t st) {
  const int64_t units = (int64_t)E * ((Wc + kThreads - 1) / kThreads);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(units, (int64_t)cus * 4));
  return jc ? launch_grad_r<true>(Wd, Nw, sizes, E, M, Wc, r, s, G, err, grid, st)
            : launch_grad_r<false>(Wd, Nw, sizes, E, M, Wc, r, s, G, err, grid, st);
}

hipError_t launch_lora_transpose(const float* in, int64_t E, int64_t P, int64_t Qd, float* out, int cus,
                                 hipStream_t st) {
  const int64_t tiles = E * ((P + 31) / 32) * ((Qd + 31) / 32);
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(tiles, (int64_t)cus * 8);
  hipLaunchKernelGGL(lora_transpose_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, in, E, P, Qd, out);
  return hipGetLastError();
}

}  // namespace geg
