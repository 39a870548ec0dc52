// Auxiliary kernels: dequantisation exports, the NF4 packer, workspace zeroing.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

// One thread per 8 elements (4 code bytes) of one weight row.
// NF4: fp32 = T[c] * absmax (one fp32 multiply), fp16 through the same scaled
// table and lookup the tiled GEMM path feeds to its MFMA, bf16 = RNE of fp32.
// MXFP4: fp32 = e2m1(c) * 2^(s-127) rounded to fp32; bf16 through the same
// scaled fp4 -> bf16 conversion the GEMMs use; fp16 = RNE of fp32.
template <Fmt F>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ wq,
                                                           const void* __restrict__ scales,
                                                           float* __restrict__ f32,
                                                           uint16_t* __restrict__ bf16,
                                                           uint16_t* __restrict__ f16,
                                                           int64_t rows, int64_t K) {
  const int64_t groups_per_row = K >> 3;
  const int64_t total = rows * groups_per_row;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kThreads) {
    const int64_t row = q / groups_per_row;
    const int64_t k = (q % groups_per_row) << 3;
    const uint32_t x = *reinterpret_cast<const uint32_t*>(wq + row * (K >> 1) + (k >> 1));
    float v[8];
    u32x4 h16 = {0u, 0u, 0u, 0u}, hb = {0u, 0u, 0u, 0u};
    if constexpr (F == NF4) {
      const float s = reinterpret_cast<const float*>(scales)[row * (K >> 6) + (k >> 6)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b = (x >> (8 * i)) & 0xFFu;
        v[2 * i] = nf4_value(b >> 4) * s;
        v[2 * i + 1] = nf4_value(b & 15) * s;
      }
      const u32x4 d = nf4_decode8(nf4_scaled_lut(s), x);  // slot order {0,2},{4,6},{1,3},{5,7}
      h16[0] = perm(d[2], d[0], 0x05040100u);   // k0, k1
      h16[1] = perm(d[2], d[0], 0x07060302u);   // k2, k3
      h16[2] = perm(d[3], d[1], 0x05040100u);   // k4, k5
      h16[3] = perm(d[3], d[1], 0x07060302u);   // k6, k7
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    } else {
      const uint32_t sb = reinterpret_cast<const uint8_t*>(scales)[row * (K >> 5) + (k >> 5)];
      const float s = e8m0_to_f32(sb);
      const double sd = sb == 255 ? __builtin_nan("") : __builtin_ldexp(1.0, (int)sb - 127);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = (x >> (4 * i)) & 15u;  // element 2b in the low nibble of byte b
        const uint32_t ex = (c >> 1) & 3u, m = c & 1u;
        const double mag = ex == 0 ? 0.5 * m : (double)(1u << (ex - 1)) * (1.0 + 0.5 * m);
        const double val = (c & 8u) ? -mag : mag;
        v[i] = (float)(val * sd);
      }
      hb = mxfp4_decode8(x, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x2 h;
        h[0] = (_Float16)v[2 * i];
        h[1] = (_Float16)v[2 * i + 1];
        h16[i] = __builtin_bit_cast(uint32_t, h);
      }
    }
    const int64_t o = row * K + k;
    float4* fo = reinterpret_cast<float4*>(f32 + o);
    fo[0] = make_float4(v[0], v[1], v[2], v[3]);
    fo[1] = make_float4(v[4], v[5], v[6], v[7]);
    if (bf16) *reinterpret_cast<u32x4*>(bf16 + o) = hb;
    if (f16) *reinterpret_cast<u32x4*>(f16 + o) = h16;
  }
}

// NF4 packer: one thread per (row, 64-wide block).
__global__ __launch_bounds__(kThreads) void quantize_nf4_kernel(const float* __restrict__ w,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ absmax,
                                                                int64_t rows, int64_t K) {
  const int64_t blocks_per_row = K >> 6;
  const int64_t total = rows * blocks_per_row;
  // Midpoints between consecutive table values, exact in fp64.
  double mid[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) mid[i] = 0.5 * ((double)nf4_value(i) + (double)nf4_value(i + 1));
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kThreads) {
    const float* src = w + q * 64;  // row-major [rows, K]: block q covers 64 contiguous floats
    float am = 0.f;
    for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(src[i]));
    const double d = (double)am;
    uint32_t packed[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t byte = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 8 * j + 2 * b + h;
          const double x = am > 0.f ? (double)src[i] / d : 0.0;
          uint32_t c = 0;
#pragma unroll
          for (int m = 0; m < 15; ++m) c += x > mid[m] ? 1u : 0u;
          byte |= h == 0 ? (c << 4) : c;  // even k in the high nibble
        }
        word |= byte << (8 * b);
      }
      packed[j] = word;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(codes + q * 32);
    dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    absmax[q] = am;
  }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// Row-scaled fp16 copy of bf16 rows for the NF4 tiled path. The NF4 MFMA takes
// fp16 operands, whose exponent range is far narrower than bf16's: activation
// gradients of 1e-6 and below would fall into fp16's subnormals or flush to
// zero, and values above 65504 would overflow. Each row is therefore multiplied
// by the power of two 2^-rexp[r] that puts its largest magnitude in [2^14, 2^15)
// before the conversion, and the tiled kernel multiplies the row's fp32 results
// by 2^rexp[r] before their bf16 rounding. Both multiplications are exact, so
// a row's result is what unbounded fp16 range would give. Converting once here
// rather than in every output-column tile that reads a row leaves the tiled
// kernel a plain copy of the operand.

// Largest |x| of 8 bf16 values as magnitude bits (ordered like the values;
// 0x7F80 and above are inf and NaN), folded into m.
__device__ __forceinline__ uint32_t absmax8(const u32x4& x, uint32_t m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(x[i] & 0x7FFFu, (x[i] >> 16) & 0x7FFFu));
  return m;
}

// The row exponent floor(log2 max|x|) - 14 from the magnitude bits; a non-finite
// row is converted unscaled and flagged.
__device__ __forceinline__ int row_exponent(uint32_t mx, uint32_t& bad) {
  if (mx >= 0x7F80u) {
    bad = 1;
    return 0;
  }
  if (mx >= 0x80u) return (int)(mx >> 7) - 127 - 14;
  if (mx > 0u) return (31 - __builtin_clz(mx)) - 133 - 14;   // bf16 subnormal: mantissa * 2^-133
  return 0;
}

// 8 bf16 values times 2^-ex as fp16, in the NF4 slot order [0, 2, 4, 6, 1, 3, 5, 7].
__device__ __forceinline__ u32x4 conv8(const u32x4& x, int ex) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, x[i] << 16), -ex);
    f[2 * i + 1] = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, x[i] & 0xFFFF0000u), -ex);
  }
  constexpr int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h;
    h[0] = (_Float16)f[order[2 * i]];
    h[1] = (_Float16)f[order[2 * i + 1]];
    r[i] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// One row per TP = 2^tp_log2 lanes of a wavefront (64 / TP rows per wavefront);
// lane j of a row's group takes the row's 16-byte chunks j, j + TP, ... With
// CPL > 0 each lane holds its (at most CPL) chunks in registers between the
// maximum and the conversion; CPL == 0 reads them again (longer rows).
template <int CPL>
__global__ __launch_bounds__(kThreads) void to_f16_rows_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ a16,
                                                               int32_t* __restrict__ rexp, int64_t M,
                                                               int64_t chunks, int tp_log2,
                                                               uint32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int TP = 1 << tp_log2;
  const int sub = lane & (TP - 1);
  const int rows_per_wave = 64 >> tp_log2;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64) * rows_per_wave;
  uint32_t bad = 0;
  for (int64_t r0 = wave * rows_per_wave; r0 < M; r0 += stride) {
    const int64_t row = r0 + (lane >> tp_log2);
    const bool live = row < M;
    const u32x4* src = a + row * chunks;
    u32x4* dst = a16 + row * chunks;
    uint32_t mx = 0;
    u32x4 v[CPL > 0 ? CPL : 1];
    if constexpr (CPL > 0) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t j = sub + (int64_t)i * TP;
        v[i] = (live && j < chunks) ? src[j] : u32x4{0u, 0u, 0u, 0u};
        mx = absmax8(v[i], mx);
      }
    } else if (live) {
      for (int64_t j = sub; j < chunks; j += TP) mx = absmax8(src[j], mx);
    }
    for (int o = TP >> 1; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    const int ex = row_exponent(mx, bad);
    if (live && sub == 0) rexp[row] = ex;
    if constexpr (CPL > 0) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t j = sub + (int64_t)i * TP;
        if (live && j < chunks) dst[j] = conv8(v[i], ex);
      }
    } else if (live) {
      for (int64_t j = sub; j < chunks; j += TP) dst[j] = conv8(src[j], ex);
    }
  }
  if (bad) atomicOr(err, kErrFp16Range);
}

// Rows of more than 64 x 16 chunks: one row per workgroup, thread t holding
// chunks t, t + 256, ... (at most CPL) in registers; the row maximum goes
// through LDS across the four wavefronts. One read and one write per element.
template <int CPL>
__global__ __launch_bounds__(kThreads) void to_f16_rows_wg_kernel(const u32x4* __restrict__ a,
                                                                  u32x4* __restrict__ a16,
                                                                  int32_t* __restrict__ rexp, int64_t M,
                                                                  int64_t chunks, uint32_t* __restrict__ err) {
  __shared__ uint32_t wmax[2][kThreads / 64];
  const int t = threadIdx.x;
  uint32_t bad = 0;
  int par = 0;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x, par ^= 1) {
    const u32x4* src = a + row * chunks;
    u32x4* dst = a16 + row * chunks;
    uint32_t mx = 0;
    u32x4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t j = t + (int64_t)i * kThreads;
      v[i] = j < chunks ? src[j] : u32x4{0u, 0u, 0u, 0u};
      mx = absmax8(v[i], mx);
    }
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    // alternate the two slots from row to row: one barrier per row suffices
    if ((t & 63) == 0) wmax[par][t >> 6] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) mx = max(mx, wmax[par][w]);
    const int ex = row_exponent(mx, bad);
    if (t == 0) rexp[row] = ex;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t j = t + (int64_t)i * kThreads;
      if (j < chunks) dst[j] = conv8(v[i], ex);
    }
  }
  if (bad) atomicOr(err, kErrFp16Range);
}

int grid_for(int64_t work) {
  int64_t g = (work + kThreads - 1) / kThreads;
  return (int)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* wq, const void* scales, float* f32,
                          uint16_t* bf16, uint16_t* f16, int64_t rows, int64_t K, hipStream_t s) {
  const int grid = grid_for(rows * (K >> 3));
  if (fmt == NF4)
    hipLaunchKernelGGL(dequant_kernel<NF4>, dim3(grid), dim3(kThreads), 0, s, wq, scales, f32,
                       bf16, f16, rows, K);
  else
    hipLaunchKernelGGL(dequant_kernel<MXFP4>, dim3(grid), dim3(kThreads), 0, s, wq, scales, f32,
                       bf16, f16, rows, K);
  return hipGetLastError();
}

hipError_t launch_quantize_nf4(const float* w, uint8_t* codes, float* absmax, int64_t rows,
                               int64_t K, hipStream_t s) {
  hipLaunchKernelGGL(quantize_nf4_kernel, dim3(grid_for(rows * (K >> 6))), dim3(kThreads), 0, s,
                     w, codes, absmax, rows, K);
  return hipGetLastError();
}

hipError_t launch_to_f16_rows(const uint16_t* a, uint16_t* a16, int32_t* rexp, int64_t M, int64_t C,
                              uint32_t* err, int cus, hipStream_t s) {
  const int64_t chunks = C >> 3;
  int tp_log2 = 0;
  while (tp_log2 < 6 && ((int64_t)1 << tp_log2) < chunks) ++tp_log2;
  const int64_t per_lane = (chunks + (1 << tp_log2) - 1) >> tp_log2;
  const int64_t rows_per_block = (kThreads / 64) * (64 >> tp_log2);
  int64_t grid = (M + rows_per_block - 1) / rows_per_block;
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, (int64_t)cus * 16));
  const u32x4* src = reinterpret_cast<const u32x4*>(a);
  u32x4* dst = reinterpret_cast<u32x4*>(a16);
#define GEG_TO_F16(CPL)                                                                                        \
  hipLaunchKernelGGL(to_f16_rows_kernel<CPL>, dim3((int)grid), dim3(kThreads), 0, s, src, dst, rexp, M, chunks, \
                     tp_log2, err)
  const int64_t per_thread_wg = (chunks + kThreads - 1) / kThreads;   // one row per workgroup
  if (per_lane > 16 && per_thread_wg <= 16) {
    const int64_t wgrid = std::max<int64_t>(1, std::min<int64_t>(M, (int64_t)cus * 8));
#define GEG_TO_F16_WG(CPL)                                                                                      \
  hipLaunchKernelGGL(to_f16_rows_wg_kernel<CPL>, dim3((int)wgrid), dim3(kThreads), 0, s, src, dst, rexp, M, chunks, \
                     err)
    if (per_thread_wg <= 8)
      GEG_TO_F16_WG(8);
    else
      GEG_TO_F16_WG(16);
#undef GEG_TO_F16_WG
    return hipGetLastError();
  }
  if (per_lane <= 1)
    GEG_TO_F16(1);
  else if (per_lane <= 2)
    GEG_TO_F16(2);
  else if (per_lane <= 4)
    GEG_TO_F16(4);
  else if (per_lane <= 8)
    GEG_TO_F16(8);
  else if (per_lane <= 16)
    GEG_TO_F16(16);
  else
    GEG_TO_F16(0);
#undef GEG_TO_F16
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)(bytes / 4);
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace geg
