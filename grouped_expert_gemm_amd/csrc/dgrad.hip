// Input gradient of the grouped NF4 GEMM on the same packed weights:
//   dX[rows of e, :] = dY[rows of e, :] . W_e     (contracts over N)
// ("grouped-nf4-gemm capability index", system_manifest.owns lists the grouped
// packed GEMM together with its dgrad; the consumer page describes the fused
// backward as computing dX on the packed bytes instead of dequantising.)
//
// A workgroup owns a 128-row x 128-k output tile and walks N in chunks of 64.
// The packed rows are contiguous along K while the contraction runs along N, so
// each chunk of 64 weight rows is decoded (table value times its 64-block absmax,
// rounded once to fp16) and written to LDS transposed, [k][n], from where the
// MFMA B operand reads 8 consecutive n per lane. dY is converted bf16 -> fp16
// (range-checked like the forward activations).
#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int kDM = 128;          // output rows per tile
constexpr int kDK = 128;          // output k per tile
constexpr int kDN = 64;           // contraction chunk
constexpr int kLdA = kDN + 8;     // halves
constexpr int kLdB = kDN + 8;

__global__ __launch_bounds__(kThreads) void dgrad_kernel(DgradArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) uint16_t As[kDM][kLdA];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[kDK][kLdB];

  const int k_tiles = (int)((g.K + kDK - 1) / kDK);
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    return s > 0 ? ((s + kDM - 1) / kDM) * k_tiles : 0;
  });

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kg = lane >> 4;
  const int arow = t >> 1, ahalf = t & 1;       // dY staging: row, 32-wide n half
  const int np = t & 31, kq = t >> 5;           // W staging: rows 2np, 2np+1; k in [16kq, 16kq+16)
  const int nchunks = (int)((g.N + kDN - 1) / kDN);
  const int64_t K = g.K, N = g.N;
  uint32_t range = 0;

  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, g.E, u);
    const int32_t lu = u - plan.upre[e];
    const int mt = lu / k_tiles, kt = lu % k_tiles;
    const int64_t row0 = (int64_t)plan.off[e] + (int64_t)mt * kDM;
    const int rows = min(kDM, (int)(plan.off[e + 1] - row0));
    const int64_t k0 = (int64_t)kt * kDK;
    const int64_t kw = k0 + 16 * kq;             // this thread's 16 weight columns
    const bool kw_ok = kw < K;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nchunks; ++c) {
      const int64_t n0 = (int64_t)c * kDN;
      // dY tile -> LDS (fp16, natural order)
      {
        const int64_t nn = n0 + 32 * ahalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (arow < rows && nn + 8 * i < N)
            v = *reinterpret_cast<const u32x4*>(g.dy + (row0 + arow) * N + nn + 8 * i);
          *reinterpret_cast<u32x4*>(&As[arow][32 * ahalf + 8 * i]) = bf16x8_to_f16(v, range);
        }
      }
      // W rows n0+2np, n0+2np+1, k in [kw, kw+16) -> decoded, transposed into Bt[k][n]
      {
        uint32_t v[2][8];  // fp16 values per row, in NF4 slot order per 8
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int64_t n = n0 + 2 * np + rr;
          u32x2 codes = {0x77777777u, 0x77777777u};
          float s = 0.f;
          if (n < N && kw_ok) {
            const int64_t rowbase = (int64_t)e * N + n;
            codes = *reinterpret_cast<const u32x2*>(g.wq + rowbase * (K >> 1) + (kw >> 1));
            s = g.absmax[rowbase * (K >> 6) + (kw >> 6)];
          }
          const Lut16 lut = nf4_scaled_lut(s);
          const u32x4 d0 = nf4_decode8(lut, codes[0]);
          const u32x4 d1 = nf4_decode8(lut, codes[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[rr][i] = d0[i];
            v[rr][4 + i] = d1[i];
          }
        }
        // slot order within 8: dword i holds k = {0,2},{4,6},{1,3},{5,7}
        constexpr int klo[4] = {0, 4, 1, 5};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t r0 = v[0][4 * h + i], r1 = v[1][4 * h + i];
            const int kk = 16 * kq + 8 * h + klo[i];
            // low halves -> k = kk, high halves -> k = kk + 2; pair (row 2np, row 2np+1)
            *reinterpret_cast<uint32_t*>(&Bt[kk][2 * np]) = perm(r1, r0, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&Bt[kk + 2][2 * np]) = perm(r1, r0, 0x07060302u);
          }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = *reinterpret_cast<const u32x4*>(&As[64 * wm + 16 * i + col][32 * s + 8 * kg]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[j] = *reinterpret_cast<const u32x4*>(&Bt[64 * wn + 16 * j + col][32 * s + 8 * kg]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<NF4>(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kc = k0 + 64 * wn + 16 * j + col;
      if (kc < K) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int lr = 64 * wm + 16 * i + 4 * kg + q;
            if (lr < rows) g.dx[(row0 + lr) * K + kc] = to_bf16(acc[i][j][q]);
          }
      }
    }
  }
  if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
}

}  // namespace

hipError_t launch_dgrad(const DgradArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL(dgrad_kernel, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
