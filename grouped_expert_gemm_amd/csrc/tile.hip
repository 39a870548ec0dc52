// Tiled (prefill-shape) path of the grouped 4-bit GEMM.
//
// One persistent launch walks every 128x128 output tile of every expert that has
// more rows than the skinny path takes. Per 64-wide K stage a workgroup stages
// its activation tile (NF4: converted to fp16) and decodes its 128 weight rows
// once into LDS — codes through the 16-value table, times the block scale —
// so the decode is shared by all four wavefronts and all 128 rows of the tile
// ("grouped-nf4-gemm 0.33.1", opening description: table decode in registers,
// blockwise scaling, fp32 accumulation, bf16 epilogue, no dequantised copy of an
// expert in memory). Each wavefront then runs 4x4 16x16x32 MFMAs per 32 k.
#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int kLd = kTileK + 8;  // LDS row stride in halves (144 B: conflict-free 16-B reads)

template <Fmt F>
struct StageRegs {
  u32x4 a[4];      // 32 activations (bf16) of one row
  u32x4 code;      // 32 codes of one weight row
  float scale;     // NF4 absmax of the 64-block / MXFP4 scale as fp32
};

template <Fmt F>
__device__ __forceinline__ void load_stage(StageRegs<F>& r, const GemmArgs& g, int e,
                                           int64_t arow, bool a_ok, int64_t n, int64_t k0,
                                           int half) {
  const int64_t K = g.K;
  const int64_t ka = k0 + 32 * half;
  const bool k_ok = ka < K;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.a[i] = u32x4{0u, 0u, 0u, 0u};
  if (a_ok && k_ok) {
    const u32x4* src = reinterpret_cast<const u32x4*>(g.a + arow * K + ka);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = src[i];
  }
  r.code = u32x4{0u, 0u, 0u, 0u};
  if constexpr (F == NF4) r.code = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
  r.scale = F == NF4 ? 0.f : 1.f;
  if (n < g.N && k_ok) {
    const int64_t rowbase = (int64_t)e * g.N + n;
    r.code = *reinterpret_cast<const u32x4*>(g.wq + rowbase * (K >> 1) + (ka >> 1));
    if constexpr (F == NF4)
      r.scale = reinterpret_cast<const float*>(g.scales)[rowbase * (K >> 6) + (k0 >> 6)];
    else
      r.scale = e8m0_to_f32(reinterpret_cast<const uint8_t*>(g.scales)[rowbase * (K >> 5) + (ka >> 5)]);
  }
}

template <Fmt F>
__global__ __launch_bounds__(kThreads) void tile_kernel(GemmArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) uint16_t As[kTileM][kLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTileN][kLd];

  const int n_tiles = (int)((g.N + kTileN - 1) / kTileN);
  const int32_t thresh = g.thresh;
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    if (s <= thresh) return 0;
    return ((s + kTileM - 1) / kTileM) * n_tiles;
  });

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kg = lane >> 4;
  const int lrow = t >> 1;       // staging row (activation row and weight row)
  const int half = t & 1;        // staging k half (32 of the 64)
  const int nstages = (int)((g.K + kTileK - 1) / kTileK);
  uint32_t range = 0;

  for (int32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = find_expert(plan, g.E, u);
    const int32_t lu = u - plan.upre[e];
    const int mt = lu / n_tiles, nt = lu % n_tiles;
    const int64_t row0 = (int64_t)plan.off[e] + (int64_t)mt * kTileM;
    const int rows = min(kTileM, (int)(plan.off[e + 1] - row0));
    const int64_t n0 = (int64_t)nt * kTileN;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    StageRegs<F> r;
    load_stage<F>(r, g, e, row0 + lrow, lrow < rows, n0 + lrow, 0, half);

    for (int st = 0; st < nstages; ++st) {
      // registers -> LDS (convert activations, decode weights)
      if constexpr (F == NF4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(&As[lrow][32 * half + 8 * i]) = bf16x8_to_f16_slots(r.a[i], range);
        const Lut16 lut = nf4_scaled_lut(r.scale);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(&Bs[lrow][32 * half + 8 * i]) = nf4_decode8(lut, r.code[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<u32x4*>(&As[lrow][32 * half + 8 * i]) = r.a[i];
          *reinterpret_cast<u32x4*>(&Bs[lrow][32 * half + 8 * i]) = mxfp4_decode8(r.code[i], r.scale);
        }
      }
      __syncthreads();
      if (st + 1 < nstages)
        load_stage<F>(r, g, e, row0 + lrow, lrow < rows, n0 + lrow, (int64_t)(st + 1) * kTileK, half);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = *reinterpret_cast<const u32x4*>(&As[64 * wm + 16 * i + col][32 * s + 8 * kg]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[j] = *reinterpret_cast<const u32x4*>(&Bs[64 * wn + 16 * j + col][32 * s + 8 * kg]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<F>(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }

    // Epilogue: acc[i][j][q] is row 64wm+16i+4kg+q, column 64wn+16j+col of the tile.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = n0 + 64 * wn + 16 * j + col;
      if (c < g.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int lr = 64 * wm + 16 * i + 4 * kg + q;
            if (lr < rows) g.out[(row0 + lr) * g.N + c] = to_bf16(acc[i][j][q]);
          }
      }
    }
  }
  if constexpr (F == NF4) {
    if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
  }
}

}  // namespace

hipError_t launch_tile(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == NF4)
    hipLaunchKernelGGL(tile_kernel<NF4>, dim3(grid), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(tile_kernel<MXFP4>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
