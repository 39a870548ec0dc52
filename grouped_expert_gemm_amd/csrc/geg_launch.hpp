// Host-side launch interface between the C ABI (geg.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace geg {

enum Fmt : int { NF4 = 0, MXFP4 = 1 };

constexpr int kMaxExperts = 1024;  // experts per call (routing plan kept in LDS)
constexpr int kThreads = 256;      // every kernel runs 4 wave64s per workgroup

// Skinny (decode) path: experts with 1..thresh rows stream their weights once;
// each workgroup covers 16 weight rows, up to kSkinnyRows activation rows and
// one of `split` K ranges (its four wavefronts split that range again).
constexpr int kSkinnyRows = 32;   // activation rows per skinny unit (2 MFMA row groups)
// Experts with up to this many rows take the skinny path (as several row units
// when above kSkinnyRows); larger ones are tiled. In a large batch the tiled
// kernel fills the chip anyway and absorbs mid-size experts at a lower decode
// cost per row, so the skinny path keeps only the smallest ones.
constexpr int kSkinnyMaxRows = 64;
constexpr int kSkinnyMaxRowsLargeM = 16;
constexpr int64_t kLargeM = 2048;   // routed rows above which a batch counts as large
constexpr int64_t kDecodeAvgRows = 32;   // batches with at most this many rows per expert: no tiles
constexpr int kSkinnyCols = 16;   // weight rows (output columns) per skinny unit
constexpr int kKStep = 128;       // K per skinny inner step

// Vector path: experts with few rows (the token-decode case) take packed dot
// products on the vector ALUs, kVecRows activation rows per wavefront unit.
// A batch of at most kVecMaxM routed rows takes it for every expert that is not
// tiled; a larger batch leaves its small experts to the skinny kernel (one
// launch instead of two: the second launch costs more than it saves).
constexpr int kVecRows = 4;
constexpr int64_t kVecMaxM = 64;
constexpr int64_t kVecOneRowM = 8;   // batches up to this many rows: one row per unit

// Tiled (prefill) path: one 256x256 output tile per workgroup at a time.
constexpr int kTileM = 256;
constexpr int kTileN = 256;

struct GemmArgs {
  const uint16_t* a;      // bf16 [M, K]
  const uint16_t* a16;    // NF4 tile path: the activations as fp16 in NF4 slot order, each
                          // row multiplied by 2^-rexp[row] (dgrad: dY [M, N] likewise)
  const int32_t* rexp;    // NF4 tile path: per-row exponents; row results are multiplied by 2^rexp
  const int32_t* sizes;   // [E]
  const uint8_t* wq;      // packed codes [E, N, K/2]
  const void* scales;     // NF4: fp32 [E, N, K/64]; MXFP4: u8 [E, N, K/32]
  uint16_t* out;          // bf16 [M, N]
  int64_t M, N, K;
  int32_t E;
  int32_t thresh;         // skinny path takes experts with 1..thresh rows
  int32_t split;          // skinny K splits
  int32_t cb;             // skinny: 16-row column blocks per wavefront (1, 2 or 4)
  int32_t vec_rows;       // vector path takes experts with 1..vec_rows rows (0: none);
                          // the skinny path takes vec_rows+1..thresh
  uint32_t* err;          // device error word
  float* partials;        // split-K partials [split, M, N]
  // Tiled kernel: the remainder tiles (at most 128 rows) left over for a last,
  // partial persistent round split over the contraction into at most
  // tail_split pieces (1: never); each piece writes fp32 partial sums to
  // tail_part (kTailPieceFloats per piece, at most kMaxTailPieces pieces) and
  // the fixup launch adds them.
  float* tail_part;
  int32_t tail_split;
  int32_t glu;            // 1: columns 2i, 2i+1 are (gate, up) of unit i and out is
                          // [M, N/2] with out[m, i] = bf16(silu(gate) * up)
  // Low-rank adapter delta added to the tiled kernel's accumulators before the
  // bf16 rounding (lora_r == 0: none): acc[m, c] += lora_s * sum_j
  // lora_u[m, j] lora_q[e, c, j], lora_u fp32 [M, lora_r], lora_q fp32
  // [E, output width, lora_r].
  const float* lora_u;
  const float* lora_q;
  int32_t lora_r;
  float lora_s;
};

// Each launcher returns the hipError_t of its launch.
hipError_t launch_skinny(int fmt, const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs& g, int grid, hipStream_t s);   // after a skinny split > 1
hipError_t launch_vec(int fmt, const GemmArgs& g, int cus, hipStream_t s);      // sizes its own grid
hipError_t launch_narrow(int fmt, const GemmArgs& g, int cus, hipStream_t s);   // sizes its own grid
hipError_t launch_tile(int fmt, const GemmArgs& g, int grid, hipStream_t s);
hipError_t launch_tile_dgrad(int fmt, const GemmArgs& g, int grid, hipStream_t s);
// After a tiled launch with tail_split > 1 (same arguments and grid): sums the
// partials of the split remainder tiles into `out` (exits when nothing was split).
hipError_t launch_tile_fixup(const GemmArgs& g, bool dgrad, int tile_grid, hipStream_t s);
constexpr int kMaxTailPieces = 256;
constexpr int kTailPieceFloats = 128 * 256;   // a remainder tile's rows x columns
constexpr int64_t kTailMinContraction = 1024; // contraction length from which tail splits pay
hipError_t launch_dequant(int fmt, const uint8_t* wq, const void* scales, float* f32,
                          uint16_t* bf16, uint16_t* f16, int64_t rows, int64_t K, hipStream_t s);
hipError_t launch_quantize_nf4(const float* w, uint8_t* codes, float* absmax, int64_t rows,
                               int64_t K, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_route_sort(const int32_t* ids, int64_t n, int32_t E, int32_t* counts, int32_t* sizes,
                             int32_t* row_of, int32_t* src_of, uint32_t* err, hipStream_t s);
hipError_t launch_route_gather(const uint16_t* x, int64_t H, int32_t k, const int32_t* src_of, int64_t n,
                               uint16_t* xs, int cus, hipStream_t s);
// W4A8: bf16 [M, K] -> e4m3 codes [M, K] + e8m0 scales (err may be NULL), then
// the grouped GEMM of those with MXFP4 weights. Scales row-major [M, K/32], or
// with step_major as the W4A8 kernel reads them: [ceil(K/128)][M][4], blocks past
// K / 32 zero.
hipError_t launch_mxfp8_quantize(const uint16_t* a, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                 uint32_t* err, int step_major, int cus, hipStream_t s);
hipError_t launch_w4a8(const uint8_t* aq, const uint8_t* as, const int32_t* sizes, const uint8_t* wq,
                       const uint8_t* ws, uint16_t* out, int64_t M, int64_t N, int64_t K, int32_t E, uint32_t* err,
                       int cus, hipStream_t s);
// Low-rank adapter: U = s X T_e^T (T fp32 [E, r, C], U fp32 [M, r]); G_e = s
// sum_rows Wd^T Nw (fp32, [E, Wc, r] or with jc [E, r, Wc]); out[e] = in[e]^T
// for fp32 [E, P, Qd]. The delta U Q^T itself is added in the tiled kernel's
// epilogue (GemmArgs::lora_*).
hipError_t launch_lora_down(const uint16_t* X, const float* T, const int32_t* sizes, int32_t E, int64_t M, int64_t C,
                            int32_t r, float s, float* U, uint32_t* err, int cus, hipStream_t st);
hipError_t launch_lora_grad(const uint16_t* Wd, const float* Nw, const int32_t* sizes, int32_t E, int64_t M,
                            int64_t Wc, int32_t r, float s, float* G, bool jc, uint32_t* err, int cus, hipStream_t st);
hipError_t launch_lora_transpose(const float* in, int64_t E, int64_t P, int64_t Qd, float* out, int cus,
                                 hipStream_t st);
hipError_t launch_route_combine(const uint16_t* y, int64_t N, const int32_t* row_of, const float* w, int64_t T,
                                int32_t k, uint16_t* out, int cus, hipStream_t s);
// Row-scaled fp16 copy of bf16 [M, C] rows (C % 8 == 0) in the NF4 slot order:
// a16[r] = fp16(a[r] * 2^-rexp[r]) with the row's largest magnitude scaled into
// [2^14, 2^15); a non-finite element flags kErrFp16Range.
hipError_t launch_to_f16_rows(const uint16_t* a, uint16_t* a16, int32_t* rexp, int64_t M, int64_t C,
                              uint32_t* err, int cus, hipStream_t s);

// Library-held scratch of gnf4_grouped_gemm_noalloc: the device address of this
// GPU's static array (looked up and its first kNoallocZeroBytes zeroed on `stream`
// at the first call on each device).
constexpr size_t kNoallocScratchBytes = size_t(144) << 20;
constexpr size_t kNoallocZeroBytes = 256;   // the header (error word)
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);

}  // namespace geg
