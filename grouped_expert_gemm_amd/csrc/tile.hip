// Tiled (prefill-shape) path of the grouped 4-bit GEMM.
//
// One persistent launch walks every 256x256 output tile of every expert that has
// more rows than the skinny path takes. Per 64-wide K stage a workgroup stages
// its activation tile (NF4: converted to fp16) and decodes its 256 weight rows
// once into LDS — codes through the 16-value table, times the block scale — so
// the decode is shared by all four wavefronts and all 256 rows of the tile
// ("grouped-nf4-gemm 0.33.1", opening description: table decode in registers,
// blockwise scaling, fp32 accumulation, bf16 epilogue, no dequantised copy of an
// expert in memory). Eight wavefronts (two per SIMD, so one's decode VALU work
// overlaps the other's MFMAs) each own a 128x64 block of the tile and run 8x4
// 16x16x32 MFMAs per 32 k with their accumulators in AGPRs.
//
// Pipeline: LDS holds two stages. While the MFMAs of stage s read one buffer, the
// raw loads of stage s+1 (already in registers) are converted/decoded into the
// other buffer and the loads of stage s+2 are issued, so one barrier per stage
// separates writers and readers and global latency is hidden behind a stage.
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

union TileLds {
  struct {
    uint16_t a[2][BM * BK];
    uint16_t b[2][BN * BK];
  };
  uint16_t epi[kTileWaves][128 * kEpiLd];  // per-wavefront bf16 result block
};

// Half-element offset of 16-byte chunk `chunk` (0..7) of LDS row `row`. The
// swizzle depends only on the row's low 4 bits, so the 16 rows one MFMA operand
// read touches map to distinct banks, and row blocks 16 apart differ by a fixed
// offset (one address register per operand stream).
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}

// Buffer resource over `bytes` bytes from `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

struct TileSrc {
  __amdgpu_buffer_rsrc_t a;   // activation rows of the tile
  __amdgpu_buffer_rsrc_t w;   // packed codes of the tile's weight rows
  __amdgpu_buffer_rsrc_t s;   // their scales
  uint32_t a_off;             // this lane's activation byte offset (row, chunk) at k = 0
  uint32_t w_off;             // this thread's code byte offset (row t/2, half t%2) at k = 0
  uint32_t s_off;             // this thread's scale-row byte offset at k = 0
};

struct RawStage {
  u32x4 a[4];      // activations: rows 32w + 8i + lane/8, 8 bf16 at chunk lane%8
  u32x4 c;         // 32 codes of weight row t/2, k in [k0 + 32 (t%2), +32)
  float s;         // NF4: absmax of the row's 64-block; MXFP4: e8m0 byte of the 32-block
};

template <Fmt F>
__device__ __forceinline__ TileSrc tile_src(const GemmArgs& g, int e, int64_t row0, int rows,
                                            int64_t n0, int wave, int lane) {
  const int64_t K = g.K;
  TileSrc t;
  // Rows past the expert's last row, and weight rows past N, read as zeros.
  t.a = rsrc(g.a + row0 * K, (int64_t)rows * K * 2);
  const int64_t nrows = min<int64_t>(BN, g.N - n0);
  const int64_t wrow0 = (int64_t)e * g.N + n0;
  t.w = rsrc(g.wq + wrow0 * (K >> 1), nrows * (K >> 1));
  if constexpr (F == NF4)
    t.s = rsrc(reinterpret_cast<const float*>(g.scales) + wrow0 * (K >> 6), nrows * (K >> 6) * 4);
  else
    t.s = rsrc(reinterpret_cast<const uint8_t*>(g.scales) + wrow0 * (K >> 5), nrows * (K >> 5));
  const int tid = threadIdx.x;
  t.a_off = (uint32_t)(((32 * wave + (lane >> 3)) * K + 8 * (lane & 7)) * 2);
  t.w_off = (uint32_t)((tid >> 1) * (K >> 1) + 16 * (tid & 1));
  t.s_off = (uint32_t)(F == NF4 ? (tid >> 1) * (K >> 6) * 4 : (tid >> 1) * (K >> 5) + (tid & 1));
  return t;
}

template <Fmt F>
__device__ __forceinline__ void load_raw(RawStage& r, const TileSrc& t, int64_t K, int64_t k0) {
  // activations, coalesced: 8 lanes cover one row's 128 bytes; rows 8 apart per i
  const uint32_t ka = (uint32_t)(k0 * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(t.a, t.a_off, ka + (uint32_t)(i * 16 * K), 0);
  r.c = __builtin_amdgcn_raw_buffer_load_b128(t.w, t.w_off, (uint32_t)(k0 >> 1), 0);
  if constexpr (F == NF4)
    r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(t.s, t.s_off, (uint32_t)((k0 >> 6) * 4), 0));
  else
    r.s = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(t.s, t.s_off, (uint32_t)(k0 >> 5), 0));
}

// Raw activations -> LDS buffer (NF4: fp16 in the NF4 slot order; k past K is 0).
template <Fmt F>
__device__ __forceinline__ void store_a(const RawStage& r, uint16_t* As, int64_t k0, int64_t K,
                                        int wave, int lane, uint32_t& range) {
  const int chunk = lane & 7;
  const bool k_ok = k0 + 8 * chunk < K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    u32x4 v = k_ok ? r.a[i] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (F == NF4) v = bf16x8_to_f16_slots(v, range);
    *reinterpret_cast<u32x4*>(&As[swz(row, chunk)]) = v;
  }
}

// Raw codes -> decoded weights in LDS (row t/2, chunks 4 (t%2) .. +3). A 32-wide
// piece past K (MXFP4 K tail) decodes with scale 0.
template <Fmt F>
__device__ __forceinline__ void store_b(const RawStage& r, uint16_t* Bs, int64_t k0, int64_t K) {
  const int t = threadIdx.x;
  const int row = t >> 1, c0 = 4 * (t & 1);
  if constexpr (F == NF4) {
    const Lut16 lut = nf4_scaled_lut(r.s);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(&Bs[swz(row, c0 + q)]) = nf4_decode8(lut, r.c[q]);
  } else {
    const bool ok = k0 + 32 * (t & 1) < K;
    const float sc = ok ? e8m0_to_f32(__builtin_bit_cast(uint32_t, r.s)) : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(&Bs[swz(row, c0 + q)]) = mxfp4_decode8(r.c[q], sc);
  }
}

// One 32-k substep of the wavefront's 128x64 block: 8x4 MFMAs (rows past the
// expert and columns past N compute on zeros and are never stored).
// The 64-row halves of the block that hold no row of the expert are skipped
// (`vrows` = rows of the tile at or past this wavefront's first row; the branch
// is uniform across the wavefront).
template <Fmt F>
__device__ __forceinline__ void mma_substep(const uint16_t* As, const uint16_t* Bs, int s, int wm,
                                            int wn, int lane, int vrows, f32x4 (&acc)[8][4]) {
  const int r16 = lane & 15;
  const int chunk = 4 * s + (lane >> 4);
  const uint16_t* ap = As + swz(128 * wm + r16, chunk);   // + 16 rows per i
  const uint16_t* bp = Bs + swz(64 * wn + r16, chunk);
  u32x4 bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bv[j] = *reinterpret_cast<const u32x4*>(bp + 16 * BK * j);
#pragma unroll
  for (int ih = 0; ih < 2; ++ih) {
    if (vrows > 64 * ih) {
      u32x4 av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const u32x4*>(ap + 16 * BK * (4 * ih + i));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * ih + i][j] = mfma16<F>(av[i], bv[j], acc[4 * ih + i][j]);
    }
  }
}

template <Fmt F>
__device__ __forceinline__ void run_tile(TileLds& L, const GemmArgs& g, const TileSrc& src,
                                         int wave, int lane, int rows, uint32_t& range,
                                         f32x4 (&acc)[8][4]) {
  const int wm = wave >> 2, wn = wave & 3;
  const int vrows = __builtin_amdgcn_readfirstlane(rows - 128 * wm);
  const int64_t K = g.K;
  const int nst = (int)((K + BK - 1) / BK);
  RawStage raw;
  load_raw<F>(raw, src, K, 0);
  store_a<F>(raw, L.a[0], 0, K, wave, lane, range);
  store_b<F>(raw, L.b[0], 0, K);
  __syncthreads();
  if (nst > 1) load_raw<F>(raw, src, K, BK);
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < nst;
    const int64_t k1 = (int64_t)(st + 1) * BK;
    if (more) store_a<F>(raw, L.a[cur ^ 1], k1, K, wave, lane, range);
    mma_substep<F>(L.a[cur], L.b[cur], 0, wm, wn, lane, vrows, acc);
    if (more) {
      store_b<F>(raw, L.b[cur ^ 1], k1, K);
      if (st + 2 < nst) load_raw<F>(raw, src, K, (int64_t)(st + 2) * BK);
    }
    mma_substep<F>(L.a[cur], L.b[cur], 1, wm, wn, lane, vrows, acc);
    __syncthreads();
  }
}

template <Fmt F>
__global__ __launch_bounds__(kTileThreads, 1) void tile_kernel(GemmArgs g) {
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) TileLds L;

  const int n_tiles = (int)((g.N + BN - 1) / BN);
  const int32_t thresh = g.thresh;
  const int32_t total = build_plan(plan, g.sizes, g.E, g.M, g.err, [&](int32_t s) -> int32_t {
    if (s <= thresh) return 0;
    return ((s + BM - 1) / BM) * n_tiles;
  });

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  uint32_t range = 0;

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

    const TileSrc src = tile_src<F>(g, e, row0, rows, n0, wave, lane);
    run_tile<F>(L, g, src, wave, lane, rows, range, acc);

    // Epilogue through LDS: each wavefront writes its 128x64 block as bf16
    // (row-major, rows padded to 144 B) over the idle stage buffers, then stores
    // whole 16-byte row pieces. acc[i][j][q] is row 16i + 4(lane/16) + q,
    // column 16j + lane%16 of the block; every write offset is a constant from
    // the lane's base.
    uint16_t* E = L.epi[wave];
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
      const bool vec = (g.N & 7) == 0 && col + 8 <= g.N;
      const uint16_t* src = E + (lane >> 3) * kEpiLd + 8 * chunk;
      for (int rr = 0; rr < 128; rr += 8) {
        const int lr = 128 * wm + rr + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + rr * kEpiLd);
        if (lr < rows) {
          uint16_t* dst = g.out + (row0 + lr) * g.N + col;
          if (vec) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (col + x < g.N) dst[x] = (uint16_t)(v[x >> 1] >> (16 * (x & 1)));
          }
        }
      }
    }
    __syncthreads();  // the stage buffers are reused by the next tile
  }
  if constexpr (F == NF4) {
    if (range_overflowed(range)) atomicOr(g.err, kErrFp16Range);
  }
}

}  // namespace

hipError_t launch_tile(int fmt, const GemmArgs& g, int grid, hipStream_t s) {
  if (fmt == NF4)
    hipLaunchKernelGGL(tile_kernel<NF4>, dim3(grid), dim3(kTileThreads), 0, s, g);
  else
    hipLaunchKernelGGL(tile_kernel<MXFP4>, dim3(grid), dim3(kTileThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace geg
