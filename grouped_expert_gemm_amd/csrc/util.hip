// Auxiliary kernels: dequantisation exports, the NF4 packer, workspace zeroing.
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

// bf16 activations -> fp16 in the NF4 slot order, 8 elements (16 bytes) per step.
// The NF4 MFMA consumes fp16 activations; converting them once here, instead of
// in every output-column tile that reads them, leaves the tile kernel a plain
// copy. An element that overflows fp16 sets the range bit of the error word.
__global__ __launch_bounds__(kThreads) void to_f16_kernel(const u32x4* __restrict__ a,
                                                          u32x4* __restrict__ a16, int64_t chunks,
                                                          uint32_t* __restrict__ err) {
  uint32_t range = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * kThreads)
    a16[i] = bf16x8_to_f16_slots(a[i], range);
  if (range_overflowed(range)) atomicOr(err, kErrFp16Range);
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

hipError_t launch_to_f16_slots(const uint16_t* a, uint16_t* a16, int64_t elems, uint32_t* err,
                               hipStream_t s) {
  const int64_t chunks = elems >> 3;
  int64_t g = (chunks + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 2048 ? 2048 : g);
  hipLaunchKernelGGL(to_f16_kernel, dim3((int)g), dim3(kThreads), 0, s,
                     reinterpret_cast<const u32x4*>(a), reinterpret_cast<u32x4*>(a16), chunks, err);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)(bytes / 4);
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace geg
