/*
 * geg.h — grouped 4-bit expert GEMM for MI355X (gfx950), C ABI.
 *
 * One call computes, for every expert of a Mixture-of-Experts layer, the matmul
 * of that expert's routed activation rows with its 4-bit packed weight, in one
 * pass over the packed bytes (no dequantised weight copy is ever written).
 * The operation is the one a per-expert loop computes: rows are grouped by
 * expert, sizes[e] rows belong to expert e, and for each expert
 *     out[rows of e, :] = a[rows of e, :] . W_e^T
 * ("grouped-nf4-gemm releases", v0.2.6 section "The patch point"; the kernel
 * design — table decode, blockwise scaling, fp32 accumulation, bf16 output —
 * is the opening description of "grouped-nf4-gemm 0.33.1").
 *
 * Formats (the same page, opening description):
 *  - NF4: 16-value NormalFloat table (QLoRA, appendix E), one fp32 absmax per 64
 *    consecutive k of a weight row. Packed codes [E, N, K/2] u8: element 2j of a
 *    row is the HIGH nibble of byte j, element 2j+1 the low nibble (bitsandbytes
 *    order). absmax [E, N, K/64] fp32.  W[e,n,k] = T[code] * absmax[e,n,k/64].
 *  - MXFP4: OCP MX v1.0 e2m1 codes, one e8m0 scale per 32 consecutive k. Blocks
 *    [E, N, K/2] u8 (== [E, N, K/32, 16]): element 2j is the LOW nibble of byte j.
 *    Scales [E, N, K/32] u8.  W[e,n,k] = e2m1(code) * 2^(scale - 127); 255 = NaN.
 *
 * Conventions shared by every entry point:
 *  - Pointers: every tensor pointer is a DEVICE pointer (hipMalloc or torch CUDA
 *    memory) of the current device; host memory is refused with
 *    GEG_ERR_NOT_DEVICE_MEMORY (compute on the CPU with the test oracle instead).
 *    All tensors are dense row-major. a/dy/out/dx are bf16 bit patterns.
 *  - Ownership: the caller owns every buffer. The library allocates nothing per
 *    call, keeps no pointer after returning, never writes its inputs (sizes
 *    included), and writes only out/dx and the workspace.
 *  - Asynchrony: every call only enqueues work on `stream` (0 = the null stream)
 *    and never synchronises the host, except geg_read_device_error. No call
 *    reads `sizes` on the host, so calls can be captured in a HIP graph.
 *  - Output coverage: rows r < sum(sizes) are written across all N (or K)
 *    columns; rows >= sum(sizes) are left untouched. Experts with 0 rows cost
 *    no weight reads. M == 0 is a successful no-op.
 *  - Host-side errors: every check that needs no device data runs before any
 *    launch; a non-OK status means nothing was enqueued.
 *  - Device-side errors: sizes live on the device, so the kernels clamp them
 *    (negative -> 0, prefix sums clamped to M; no access outside rows [0, M))
 *    and OR a bit into the workspace's device error word (GEG_DEVERR_*).
 *  - Numerics: fp32 accumulation, bf16 output rounded to nearest even. NF4
 *    multiplies fp16 operands. On the tiled path (prefill and every dgrad) each
 *    activation row (dgrad: each dY row) is first multiplied by a power of two
 *    that puts its largest magnitude in [2^14, 2^15), converted to fp16, and the
 *    row's fp32 results are multiplied back by the inverse power before the bf16
 *    rounding: both steps are exact, so no row under- or overflows fp16 whatever
 *    its scale (elements below 2^-29 of their row's largest lose precision);
 *    a non-finite element sets GEG_DEVERR_FP16_RANGE. The decode paths (vector,
 *    narrow, skinny) convert bf16 -> fp16 directly (exact for 2^-14 <= |x| <=
 *    65504; an activation that overflows fp16 sets GEG_DEVERR_FP16_RANGE).
 *    MXFP4 multiplies bf16 operands (e2m1 * 2^k is exact in bf16 for normal
 *    results). Results are bitwise reproducible run to run.
 *  - Sizes: every kernel addresses one expert's packed weights, and at most 256
 *    rows of an activation, dY or output tensor, through 32-bit buffer windows,
 *    so a call is refused with GEG_ERR_BAD_SHAPE (nothing is clamped) unless
 *    N * K / 2 <= 0x7FFFFFF0 and 512 * max(N, K) <= 0x7FFFFFF0. M itself may
 *    exceed 2^31 / K (the tensors are addressed with 64-bit row offsets); M must
 *    be below 2^31.
 *  - Workspace: `workspace` is a caller-allocated device buffer of at least
 *    geg_workspace_bytes(...) bytes, 256-byte aligned, zeroed once by
 *    geg_workspace_init before its first use. It holds the device error word
 *    (in a 256-byte header), then the call's scratch, all of it written before
 *    it is read by every call, so one workspace can serve every entry point:
 *    split-K partials (fp32 [split, M, N]); for the NF4 tiled path, an fp16
 *    copy of the row-scaled activations (M * K * 2 bytes; dgrad: of dY,
 *    M * N * 2 bytes) and the rows' int32 exponents (M * 4 bytes); and, when
 *    the tiled path's contraction (K, dgrad: N) is at least 1024, 32 MiB for
 *    the fp32 partial sums of remainder tiles split over the contraction. That
 *    last region is optional for the grouped GEMM and dgrad entry points: a
 *    workspace that holds everything before it runs the call without the split
 *    (results equal up to the fp32 summation order of the split tiles).
 *    Calls on one workspace must be ordered (same stream); concurrent calls
 *    must not share one.
 */
#ifndef GEG_H_
#define GEG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEG_VERSION 113 /* 1.1.3 */

typedef enum {
  GEG_OK = 0,
  GEG_ERR_NULL_POINTER = 1,       /* a required pointer is NULL (when M > 0)                     */
  GEG_ERR_BAD_SHAPE = 2,          /* M < 0, N <= 0, K <= 0, E <= 0, K % 64 (NF4) or % 32 (MXFP4),
                                     a buffer window past 0x7FFFFFF0 bytes (see Sizes)            */
  GEG_ERR_MISALIGNED = 3,         /* a, w/blocks, out, dy, dx not 16-byte aligned                */
  GEG_ERR_NOT_DEVICE_MEMORY = 4,  /* a host pointer was passed                                    */
  GEG_ERR_WORKSPACE = 5,          /* workspace NULL, misaligned or too small                      */
  GEG_ERR_UNSUPPORTED_DEVICE = 6, /* the current device is not gfx950                              */
  GEG_ERR_HIP = 7,                /* HIP runtime error; detail in geg_last_error()                 */
  GEG_ERR_BAD_OPTION = 8          /* geg_opts field out of range                                   */
} geg_status;

/* Bits of the device error word (workspace word 0), sticky until geg_workspace_init. */
#define GEG_DEVERR_NEGATIVE_SIZE 0x1u /* some sizes[e] < 0: treated as 0                     */
#define GEG_DEVERR_SIZES_EXCEED_M 0x2u /* sum(sizes) > M: rows past M are not computed        */
#define GEG_DEVERR_FP16_RANGE 0x4u    /* an NF4-path operand overflowed fp16 (|x| > 65504 on a
                                         decode path) or is not finite                         */
#define GEG_DEVERR_BAD_EXPERT_ID 0x8u /* geg_route_sort: a top-k id outside [0, E) (entry dropped) */
#define GEG_DEVERR_NON_FINITE 0x10u  /* W4A8: an activation is inf or NaN (its block's codes are unspecified) */

/* Optional knobs (NULL = automatic). Used by tests to pin a path. */
typedef struct {
  /* 0 auto; 1 every expert on the skinny kernel; 2 every expert tiled; 3 every
   * expert on the vector path (experts with more than 4 rows in chunks of 4);
   * 4 every expert on the narrow kernel (in chunks of 16 or 32 rows) */
  int32_t force_path;
  int32_t split_k;    /* 0 or 1: no split; 2..16 K splits of the skinny kernel (force_path 1),  */
                      /* summed in a fixed order by a second launch                          */
  /* Optional kernel timing: NULL, or 4 events (entries may be NULL) that the call
   * records on `stream` right before and after its tiled kernel (dgrad: the dgrad
   * kernel) and right before and after its decode kernels (vector and skinny, in
   * that order): {tile_start, tile_end, decode_start, decode_end}. Events of
   * kernels the call does not launch are not recorded. The caller creates the
   * events (hipEventCreate) and owns them. */
  hipEvent_t* kernel_events;
  /* 0: size every launch for the device's compute units. n > 0: size every grid
   * as if the device had min(n, its compute units) of them (persistent kernels
   * then walk their work lists in more rounds; the results are the same). For
   * tests of the persistent loops; negative values are refused. */
  int32_t cu_limit;
} geg_opts;

/* Operation ids for geg_workspace_bytes. */
#define GEG_OP_NF4_FWD 0
#define GEG_OP_MXFP4_FWD 1
#define GEG_OP_NF4_DGRAD 2
#define GEG_OP_NF4_BLOCK 3   /* N = H (hidden), K = I (intermediate) */
#define GEG_OP_MXFP4_BLOCK 4 /* N = H (hidden), K = I (intermediate) */
#define GEG_OP_MXFP4_DGRAD 5
#define GEG_OP_MXFP4_W4A8 6   /* gmxfp4_w4a8_grouped_gemm */

/*
 * gnf4_grouped_gemm — out[M, N] = per expert, a_e . W_e^T with W_e in NF4.
 *   a       bf16 [M, K], rows grouped by expert (expert 0 first), 16-B aligned
 *   sizes   int32 [E], rows per local expert 0..E-1 (device memory, not modified)
 *   w       u8 [E, N, K/2] NF4 codes (high nibble = even k), 16-B aligned
 *   absmax  fp32 [E, N, K/64], 4-B aligned
 *   out     bf16 [M, N], 16-B aligned
 *   K % 64 == 0. Paths (automatic choice): in a batch of at most 64 rows every
 *   expert takes the vector path (packed dot products on the vector ALUs,
 *   weight rows read whole, up to 4 activation rows per pass); in a larger batch
 *   of at most 32 rows per expert on average (M <= 32 E) every expert takes the
 *   narrow kernel (weights streamed once per 16 or 32 rows, decoded into MFMA
 *   operands, each wavefront over the whole K range); in a larger batch experts
 *   with up to 64 rows (16 when M > 2048) take the narrow kernel and larger
 *   experts the tiled MFMA path.
 *   The skinny kernel (K split over wavefronts and optionally over workgroups
 *   with a fixed-order reduction) serves the same rows when forced.
 */
geg_status gnf4_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* w,
                             const float* absmax, void* out, int64_t M, int64_t N, int64_t K,
                             int32_t E, void* workspace, size_t workspace_bytes,
                             const geg_opts* opts, hipStream_t stream);

/*
 * gnf4_grouped_gemm_noalloc — gnf4_grouped_gemm for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same operation, arguments and paths, without the
 * workspace. The call allocates nothing. Its scratch (split-K partials, the
 * row-scaled fp16 activations and their row exponents) lives in a library-held
 * static device array of 144 MiB per GPU, created when the library's code is
 * loaded on that GPU and held until the process ends; its 256-byte header is
 * zeroed by a fill kernel on `stream` at the first call on each GPU, and every
 * call writes the rest before reading it.
 *   error_word  device uint32 (4-B aligned) that receives the GEG_DEVERR_* bits of
 *               this call (OR-ed in; the caller clears it), or NULL to drop them
 *   A call whose scratch (geg_workspace_bytes(GEG_OP_NF4_FWD, M, N, K, E, opts),
 *   less the optional 32 MiB of split remainder tiles) exceeds 144 MiB is refused
 *   with GEG_ERR_WORKSPACE before anything is enqueued (for example
 *   M * K * 2 + M * 4 > 140 MiB on the tiled path); when only the split region
 *   does not fit, the call runs without the split.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents: calls ordered on one stream are safe; calls that overlap on one GPU
 *   (unordered streams, several host threads) race on it.
 */
geg_status gnf4_grouped_gemm_noalloc(const void* a, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                     void* out, int64_t M, int64_t N, int64_t K, int32_t E, uint32_t* error_word,
                                     const geg_opts* opts, hipStream_t stream);

/*
 * gmxfp4_grouped_gemm — the same operation on MXFP4 weights exactly as released:
 *   blocks  u8 [E, N, K/2] e2m1 codes (low nibble = even k), 16-B aligned
 *   scales  u8 [E, N, K/32] e8m0
 *   K % 32 == 0. ("grouped-nf4-gemm releases", v0.2.5: experts arrive as
 *   [E, N, K/2] blocks plus [E, N, K/32] scales.)
 */
geg_status gmxfp4_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* blocks,
                               const uint8_t* scales, void* out, int64_t M, int64_t N, int64_t K,
                               int32_t E, void* workspace, size_t workspace_bytes,
                               const geg_opts* opts, hipStream_t stream);

/*
 * gnf4_grouped_dgrad — input gradient of gnf4_grouped_gemm on the same packed
 * weights ("grouped-nf4-gemm capability index", system_manifest.owns):
 *   dx[rows of e, :] = dy[rows of e, :] . W_e      (contracts over N)
 *   dy  bf16 [M, N] (16-B aligned), dx bf16 [M, K] (16-B aligned), K % 64 == 0,
 *   N % 8 == 0.
 */
geg_status gnf4_grouped_dgrad(const void* dy, const int32_t* sizes, const uint8_t* w,
                              const float* absmax, void* dx, int64_t M, int64_t N, int64_t K,
                              int32_t E, void* workspace, size_t workspace_bytes,
                              const geg_opts* opts, hipStream_t stream);

/*
 * gnf4_expert_block — the routed experts' whole SwiGLU MLP in two grouped GEMMs,
 * with the gated unit applied in the first one's epilogue ("grouped-nf4-gemm
 * releases", v0.2.5: a MoE layer forward runs gate, GLU and down straight off
 * the grouped GEMM's packed weights; "grouped-nf4-gemm capability index": the
 * package owns the swiglu glue):
 *   h   = a_e . W13_e^T                       (fp32 accumulation, never stored)
 *   act = bf16( silu(h[:, 2i]) * h[:, 2i+1] )  silu(x) = x / (1 + e^-x)
 *   out = act_e . W2_e^T
 *   a       bf16 [M, H], rows grouped by expert, 16-B aligned
 *   sizes   int32 [E] (device memory, not modified)
 *   w13     u8 [E, 2I, H/2] NF4 codes of the fused gate/up weight; row 2i is the
 *           gate and row 2i+1 the up projection of unit i (interleaved)
 *   absmax13 fp32 [E, 2I, H/64]
 *   w2      u8 [E, H, I/2], absmax2 fp32 [E, H, I/64]
 *   out     bf16 [M, H], 16-B aligned
 *   H % 64 == 0 and I % 64 == 0. The intermediate act [M, I] lives in the
 *   workspace (size it with geg_workspace_bytes(GEG_OP_NF4_BLOCK, M, H, I, E)).
 *   Both projections choose their paths as gnf4_grouped_gemm does; force_path 1
 *   (skinny) is refused with GEG_ERR_BAD_OPTION. kernel_events, when given, are
 *   recorded as {block_start, block_end, NULL, NULL}: around the whole block.
 */
geg_status gnf4_expert_block(const void* a, const int32_t* sizes, const uint8_t* w13,
                             const float* absmax13, const uint8_t* w2, const float* absmax2,
                             void* out, int64_t M, int64_t H, int64_t I, int32_t E,
                             void* workspace, size_t workspace_bytes, const geg_opts* opts,
                             hipStream_t stream);

/*
 * gmxfp4_expert_block — the same block on MXFP4 weights: blocks13 u8 [E, 2I, H/2]
 * with scales13 u8 [E, 2I, H/32], blocks2 u8 [E, H, I/2] with scales2 u8
 * [E, H, I/32]; H % 32 == 0 and I % 32 == 0.
 */
geg_status gmxfp4_expert_block(const void* a, const int32_t* sizes, const uint8_t* blocks13,
                               const uint8_t* scales13, const uint8_t* blocks2,
                               const uint8_t* scales2, void* out, int64_t M, int64_t H, int64_t I,
                               int32_t E, void* workspace, size_t workspace_bytes,
                               const geg_opts* opts, hipStream_t stream);

/*
 * geg_route_sort — the routing step in front of the grouped GEMM, on the device
 * ("grouped-nf4-gemm releases", v0.2.6 "The patch point": the kernel replaces a
 * per-expert loop over rows grouped by expert; capability index, entrypoints:
 * `router_epilogue`). The T*k (token, slot) entries of `topk_ids` are ordered by
 * expert and, within an expert, by flat index t*k + slot (a stable sort):
 *   topk_ids int32 [T, k], ids in [0, E) (device memory, not modified)
 *   sizes    int32 [E] out: entries per expert (the GEMM's `sizes`)
 *   row_of   int32 [T*k] out: sorted row of entry t*k + slot (-1 for an id
 *            outside [0, E), which is dropped and flags GEG_DEVERR_BAD_EXPERT_ID)
 *   src_of   int32 [T*k] out: entry of sorted row r (-1 for rows past sum(sizes))
 *   x        bf16 [T, H] token activations, and x_sorted bf16 [T*k, H] out: the
 *            GEMM's grouped rows, x_sorted[r] = x[src_of[r] / k]. Both NULL to
 *            skip the gather; else H % 8 == 0 and both 16-B aligned. Rows past
 *            sum(sizes) are left untouched.
 *   workspace: at least geg_route_workspace_bytes(T, k, E) bytes, initialised
 *            once with geg_workspace_init (its error word receives the flag).
 * Deterministic: no order depends on atomics.
 */
geg_status geg_route_sort(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, const void* x,
                          int64_t H, int32_t* sizes, int32_t* row_of, int32_t* src_of, void* x_sorted,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of geg_route_sort. */
size_t geg_route_workspace_bytes(int64_t T, int32_t k, int32_t E);

/*
 * geg_route_combine — the top-k weighted combine after the expert GEMMs, back in
 * token order (capability index, entrypoints: `combine_rows`):
 *   out[t, :] = bf16( sum over slots s of weights[t, s] * y[row_of[t*k + s], :] )
 * with fp32 products and sums in slot order; entries with row_of < 0 are skipped.
 *   y        bf16 [T*k, N], rows in the order of geg_route_sort, 16-B aligned
 *   row_of   int32 [T*k] from geg_route_sort (values in [-1, T*k))
 *   weights  fp32 [T, k] router weights, or NULL for all ones
 *   out      bf16 [T, N], 16-B aligned; N % 8 == 0
 */
geg_status geg_route_combine(const void* y, const int32_t* row_of, const float* weights, int64_t T,
                             int32_t k, int64_t N, void* out, hipStream_t stream);

/*
 * gmxfp4_grouped_dgrad — the input gradient of gmxfp4_grouped_gemm on the
 * released MXFP4 bytes: dx[rows of e, :] = dy[rows of e, :] . W_e (contracts over
 * N); blocks u8 [E, N, K/2], scales u8 [E, N, K/32], K % 32 == 0, N % 8 == 0.
 * bf16 MFMA operands (dY as given; the decoded weights are exact in bf16).
 */
geg_status gmxfp4_grouped_dgrad(const void* dy, const int32_t* sizes, const uint8_t* blocks,
                                const uint8_t* scales, void* dx, int64_t M, int64_t N, int64_t K,
                                int32_t E, void* workspace, size_t workspace_bytes,
                                const geg_opts* opts, hipStream_t stream);

/*
 * gmxfp4_w4a8_grouped_gemm — the MXFP4 grouped GEMM with activations quantised to
 * MXFP8 ("bw24 releases, v0.9.0", "Changes since v0.8.0": a W4A8-FP8 tile, e4m3
 * activations times the native e2m1 weights in one block-scaled matrix
 * instruction). Per 32-block of each activation row: e8m0 scale X =
 * floor(log2 amax) - 8 + 127 clamped to [0, 254] (0 for an all-zero block),
 * elements rounded to nearest e4m3 (ties to even) after the exact division by
 * 2^(X - 127), saturating at 448 (the OCP MX v1.0 conversion). Then
 * out[rows of e, :] = dequant(a_e) . W_e^T with fp32 accumulation, rounded to bf16.
 *   a, sizes, blocks, scales, out, M, N, K, E: as gmxfp4_grouped_gemm (K % 32 == 0)
 *   workspace: geg_workspace_bytes(GEG_OP_MXFP4_W4A8, ...) bytes; holds the error
 *            word, the e4m3 codes [M, K] and the activation scales [M, K/32]
 *   opts: force_path and split_k are ignored; kernel_events[0..1] bracket the
 *         GEMM kernel (after the quantisation launch)
 * The block-scaled instruction rounds its 128-wide dot products to about 12 bits
 * below the largest product, so results agree with the exact product of the
 * quantised operands to ~2^-12 of sum |a w| rather than to fp32 rounding.
 * Non-finite activations flag GEG_DEVERR_NON_FINITE.
 */
geg_status gmxfp4_w4a8_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* blocks,
                                    const uint8_t* scales, void* out, int64_t M, int64_t N, int64_t K,
                                    int32_t E, void* workspace, size_t workspace_bytes,
                                    const geg_opts* opts, hipStream_t stream);

/*
 * gmxfp8_quantize — the activation quantisation of gmxfp4_w4a8_grouped_gemm on
 * its own: a bf16 [M, K] (16-B aligned, K % 32 == 0) -> codes u8 [M, K] (e4m3,
 * 16-B aligned) and scales u8 [M, K/32] (e8m0). Codes of a block holding inf or
 * NaN are unspecified (no error word here).
 */
geg_status gmxfp8_quantize(const void* a, uint8_t* codes, uint8_t* scales, int64_t M, int64_t K,
                           hipStream_t stream);

/*
 * Low-rank adapter delta on the grouped projection ("grouped-nf4-gemm releases",
 * v0.2.4 section: the trainable B(Ax) composed with the frozen 4-bit projection
 * at the pre-activation point). Per expert e: lora_a fp32 [E, r, K] (A_e),
 * lora_b fp32 [E, N, r] (B_e), one scale s; r in {8, 16, ..., 64}. The matrix
 * instructions take each fp32 adapter operand as a bf16 high part plus a bf16
 * remainder (about 16 significant bits, fp32 accumulation), and the delta joins
 * the projection's fp32 accumulators before their single bf16 rounding. Every
 * expert runs on the tiled kernel (force_path is ignored).
 *
 * g{nf4,mxfp4}_grouped_gemm_lora: out = x W_e^T + s (x A_e^T) B_e^T; also writes
 *   u = x A_e^T (fp32 [M, r], 16-B aligned) for the backward. Other arguments
 *   and the workspace as g{nf4,mxfp4}_grouped_gemm, sized with
 *   geg_lora_workspace_bytes(GEG_OP_NF4_FWD or GEG_OP_MXFP4_FWD, ...).
 * g{nf4,mxfp4}_grouped_dgrad_lora: with dy bf16 [M, N] (N % 8 == 0), the
 *   forward's x and u: dx = dy W_e + g A_e with g = s dy B_e (bf16 [M, K]);
 *   grad_a = sum over the rows of e of g^T x (fp32 [E, r, K]); grad_b = s sum
 *   over the rows of e of dy^T u (fp32 [E, N, r]); experts without rows (and
 *   M == 0) get zero gradients. Workspace: geg_lora_workspace_bytes(
 *   GEG_OP_NF4_DGRAD or GEG_OP_MXFP4_DGRAD, ...).
 */
size_t geg_lora_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t E, int32_t r);
geg_status gnf4_grouped_gemm_lora(const void* a, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                  const float* lora_a, const float* lora_b, float scale, void* out, void* u, int64_t M,
                                  int64_t N, int64_t K, int32_t E, int32_t r, void* workspace, size_t workspace_bytes,
                                  const geg_opts* opts, hipStream_t stream);
geg_status gmxfp4_grouped_gemm_lora(const void* a, const int32_t* sizes, const uint8_t* blocks, const uint8_t* scales,
                                    const float* lora_a, const float* lora_b, float scale, void* out, void* u,
                                    int64_t M, int64_t N, int64_t K, int32_t E, int32_t r, void* workspace,
                                    size_t workspace_bytes, const geg_opts* opts, hipStream_t stream);
geg_status gnf4_grouped_dgrad_lora(const void* dy, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                   const void* x, const float* lora_a, const float* lora_b, const void* u, float scale,
                                   void* dx, float* grad_a, float* grad_b, int64_t M, int64_t N, int64_t K, int32_t E,
                                   int32_t r, void* workspace, size_t workspace_bytes, const geg_opts* opts,
                                   hipStream_t stream);
geg_status gmxfp4_grouped_dgrad_lora(const void* dy, const int32_t* sizes, const uint8_t* blocks,
                                     const uint8_t* scales, const void* x, const float* lora_a, const float* lora_b,
                                     const void* u, float scale, void* dx, float* grad_a, float* grad_b, int64_t M,
                                     int64_t N, int64_t K, int32_t E, int32_t r, void* workspace,
                                     size_t workspace_bytes, const geg_opts* opts, hipStream_t stream);

/* Workspace bytes needed by one call of operation `op` with these sizes and options. */
size_t geg_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t E,
                           const geg_opts* opts);

/* Zero a workspace's error word on `stream`; call once after allocating it. */
geg_status geg_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Synchronise `stream`, then copy the device error word (GEG_DEVERR_* bits) to *code. */
geg_status geg_read_device_error(const void* workspace, int32_t* code, hipStream_t stream);

/*
 * Dequantisation exports (test and inspection use; the GEMMs never call them).
 * Decode every weight with the same device code the GEMMs use for their
 * blockwise scaling:
 *   out_f32  fp32 [E, N, K] (required): NF4 = fp32 product T[c] * absmax;
 *            MXFP4 = e2m1(c) * 2^(s-127) rounded to fp32 (subnormals kept,
 *            overflow to inf, scale 255 -> NaN)
 *   out_bf16 bf16 [E, N, K] (nullable): bf16 RNE of out_f32
 *   out_f16  fp16 [E, N, K] (nullable): fp16 RNE of out_f32
 */
geg_status gnf4_dequant(const uint8_t* w, const float* absmax, float* out_f32, uint16_t* out_bf16,
                        uint16_t* out_f16, int64_t N, int64_t K, int32_t E, hipStream_t stream);
geg_status gmxfp4_dequant(const uint8_t* blocks, const uint8_t* scales, float* out_f32,
                          uint16_t* out_bf16, uint16_t* out_f16, int64_t N, int64_t K, int32_t E,
                          hipStream_t stream);

/*
 * gnf4_quantize — NF4 packer on the device ("grouped-nf4-gemm 0.33.1", section
 * "Try it on CPU right now", block 1: a weight [N, K] packs to [N, K/2] u8 codes
 * plus [N, K/64] fp32 absmax). Per row and 64-wide block: absmax = max |w|
 * (fp32); x = w / absmax in fp64; code = nearest table value, exact midpoints
 * go to the lower code; an all-zero block gets absmax 0 and code 7.
 *   w fp32 [R, K] (R = E*N rows), codes u8 [R, K/2], absmax fp32 [R, K/64].
 */
geg_status gnf4_quantize(const float* w, uint8_t* codes, float* absmax, int64_t rows, int64_t K,
                         hipStream_t stream);

const char* geg_status_string(geg_status s);
const char* geg_last_error(void); /* thread-local detail of this thread's last failure */
int32_t geg_version(void);
/* Number of kernel launches this process has enqueued through the library. */
uint64_t geg_launch_count(void);

#ifdef __cplusplus
}
#endif
#endif /* GEG_H_ */
