// C ABI of the grouped 4-bit expert GEMM library: argument validation, launch
// planning from (M, N, K, E) only (sizes stay on the device), and kernel launches
// on the caller's stream. See include/geg.h for the contract.
#include "geg.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>

#include "geg_launch.hpp"

namespace {

thread_local std::string g_last_error;
std::atomic<uint64_t> g_launches{0};

geg_status fail(geg_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

geg_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return GEG_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device check that the current device is gfx950, cached.
geg_status check_device() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(GEG_ERR_UNSUPPORTED_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (known[dev] == 2) {
      g_last_error = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950";
    }
  }
  if (known[dev] != 1) return fail(GEG_ERR_UNSUPPORTED_DEVICE, "current device is not gfx950");
  // Launch errors are read with hipGetLastError right after each launch; clear
  // what an unrelated earlier call on this thread may have left there.
  (void)hipGetLastError();
  return GEG_OK;
}

// Device (or managed) memory of the current device; host memory is refused.
geg_status check_device_ptr(const void* p, const char* name) {
  if (p == nullptr) return GEG_OK;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(GEG_ERR_NOT_DEVICE_MEMORY,
                std::string(name) + " is not device memory; this library computes on the GPU "
                "only (the CPU oracle is the reference for host data)");
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(GEG_ERR_NOT_DEVICE_MEMORY,
                std::string(name) + " is host memory; pass device memory (the CPU oracle is the "
                "reference for host data)");
  return GEG_OK;
}

// geg_opts.cu_limit of the entry point running on this thread (0: none).
thread_local int g_cu_limit = 0;

// Sets the launch-sizing limit for the duration of one entry point call.
struct CuScope {
  int prev;
  explicit CuScope(const geg_opts* o) : prev(g_cu_limit) { g_cu_limit = (o && o->cu_limit > 0) ? o->cu_limit : 0; }
  ~CuScope() { g_cu_limit = prev; }
};

// Compute units that launches are sized for: the current device's (256 on
// MI355X when it cannot be queried), or fewer under geg_opts.cu_limit.
int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return g_cu_limit > 0 ? std::min(cus, g_cu_limit) : cus;
}

// Record entry i of the caller's kernel timing events, if any.
hipError_t record_event(const geg_opts* o, int i, hipStream_t stream) {
  if (!o || !o->kernel_events || !o->kernel_events[i]) return hipSuccess;
  return hipEventRecord(o->kernel_events[i], stream);
}

struct Plan {
  int32_t thresh;   // decode paths (vector, skinny) take experts with 1..thresh rows
  int32_t vec_rows; // vector path takes 1..vec_rows, skinny vec_rows+1..thresh
  bool run_vec;
  bool narrow;      // the skinny-range experts go to the narrow kernel instead
  int32_t split;    // skinny K splits
  int32_t cb;       // skinny column blocks of 16 weight rows per wavefront
  bool run_skinny;
  bool run_tile;
  int64_t rc_bound;        // bound on skinny row chunks
  size_t partials_off, partials_bytes;
  size_t a16_off, a16_bytes;   // NF4 tile path: fp16 copy of the row-scaled activations
  size_t rexp_off;             // ... followed by the rows' int32 exponents
  size_t tail_off, tail_bytes; // tiled path, long contractions: partials of split remainder tiles
  size_t total_bytes;
};


constexpr size_t kHeader = 256;   // the device error word, then padding
constexpr int32_t kTailSplitMax = 4;   // contraction pieces per split remainder tile

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Tiled ops with a contraction of at least kTailMinContraction may split their
// remainder tiles over the contraction (see tile.hip); their partial sums take
// a fixed region at the end of the workspace.
void plan_tail(Plan& p, int64_t contraction) {
  if (!p.run_tile || contraction < geg::kTailMinContraction) return;
  p.tail_off = round256(p.total_bytes);
  p.tail_bytes = (size_t)geg::kMaxTailPieces * geg::kTailPieceFloats * 4;
  p.total_bytes = p.tail_off + p.tail_bytes;
}

// The split region is optional: a workspace that holds everything before it
// runs the call with no tile split (the same results up to the fp32 summation
// order of the split tiles).
void fit_tail(Plan& p, size_t ws_bytes) {
  if (p.tail_bytes && ws_bytes < p.total_bytes && ws_bytes >= p.tail_off) {
    p.tail_bytes = 0;
    p.total_bytes = p.tail_off;
  }
}

geg_status make_plan(int op, int64_t M, int64_t N, int64_t K, int32_t E, const geg_opts* o, Plan& p) {
  const int32_t force = o ? o->force_path : 0;
  const int32_t split_req = o ? o->split_k : 0;
  if (force < 0 || force > 4) return fail(GEG_ERR_BAD_OPTION, "force_path must be 0..4");
  if (split_req < 0 || split_req > 16) return fail(GEG_ERR_BAD_OPTION, "split_k must be 0..16");
  if (o && o->cu_limit < 0) return fail(GEG_ERR_BAD_OPTION, "cu_limit must be >= 0");
  std::memset(&p, 0, sizeof(p));
  p.split = 1;
  if (op == GEG_OP_NF4_DGRAD) {
    // row-scaled dY as fp16 for the tiled kernel and the rows' exponents
    p.run_tile = M > 0;
    p.a16_off = kHeader;
    p.a16_bytes = round256((size_t)M * (size_t)N * 2) + round256((size_t)M * 4);
    p.rexp_off = p.a16_off + round256((size_t)M * (size_t)N * 2);
    p.total_bytes = p.a16_off + p.a16_bytes;
    plan_tail(p, N);
    return GEG_OK;
  }
  if (op == GEG_OP_MXFP4_W4A8) {   // e4m3 codes [M, K] and their scales [M, K/32]
    p.a16_off = kHeader;
    // scales step-major, 4 per row and 128-wide k step
    p.a16_bytes = round256((size_t)M * (size_t)K) + round256((size_t)M * (size_t)((K / 32 + 3) & ~3));
    p.total_bytes = p.a16_off + p.a16_bytes;
    return GEG_OK;
  }
  if (op == GEG_OP_MXFP4_DGRAD) {   // bf16 dY feeds the MFMAs as it is
    p.run_tile = M > 0;
    p.total_bytes = kHeader;
    plan_tail(p, N);
    return GEG_OK;
  }
  // A decode-class batch (at most kDecodeAvgRows routed rows per expert on
  // average) keeps every expert off the tiled path: its few tiles would run one
  // per CU over the whole K range, slower than streaming the weights once per
  // 32 rows on every CU, and the call saves the tiled launches.
  const bool decode_class = M <= geg::kDecodeAvgRows * (int64_t)E;
  const int32_t auto_thresh = decode_class ? INT32_MAX
                              : (M > geg::kLargeM ? geg::kSkinnyMaxRowsLargeM : geg::kSkinnyMaxRows);
  p.thresh = (force == 1 || force == 3 || force == 4) ? INT32_MAX : (force == 2 ? 0 : auto_thresh);
  // the narrow kernel serves the skinny range unless the skinny kernel is forced
  p.narrow = force != 1;
  if (force == 0)
    p.vec_rows = M <= geg::kVecMaxM ? p.thresh : 0;
  else
    p.vec_rows = force == 3 ? INT32_MAX : 0;
  p.run_vec = p.vec_rows > 0 && M > 0;
  p.run_skinny = p.thresh > p.vec_rows && M > 0;
  p.run_tile = (force == 0 || force == 2) && M > p.thresh;
  const int64_t ksteps = (K + geg::kKStep - 1) / geg::kKStep;
  if (p.run_skinny && !p.narrow) {
    const int64_t skinny_experts = std::min<int64_t>(E, M);
    // The narrowest column block whose units still fit in one round of resident
    // workgroups (two per CU): smaller units finish sooner, a second round costs
    // a whole unit's latency chain. When none fits, the widest (fewest units).
    p.cb = 4;
    for (int32_t cb = 1; cb <= 4; cb <<= 1) {
      if (skinny_experts * ((N + 16 * cb - 1) / (16 * cb)) <= 2 * (int64_t)cu_count()) {
        p.cb = cb;
        break;
      }
    }
    p.rc_bound = (M + geg::kSkinnyRows - 1) / geg::kSkinnyRows + skinny_experts;
    // K is split across workgroups only on request: on every decode shape
    // measured (T = 1 and 64 of OLMoE, Qwen3 and gpt-oss) each split of 2, 4 or
    // 8 was slower than no split (its reduce launch and the partials' round
    // trip cost more than the shorter per-unit chains save), and the skinny
    // kernel itself is slower there than the vector and narrow kernels.
    int64_t split = split_req == 0 ? 1 : split_req;
    split = std::max<int64_t>(1, std::min<int64_t>(split, ksteps));
    p.split = (int32_t)split;
    if (p.split > 1) {
      p.partials_off = kHeader;
      p.partials_bytes = round256((size_t)p.split * (size_t)M * (size_t)N * 4);
    }
  }
  p.total_bytes = kHeader + p.partials_bytes;
  if (p.run_tile && op == GEG_OP_NF4_FWD) {
    p.a16_off = kHeader + p.partials_bytes;
    p.a16_bytes = round256((size_t)M * (size_t)K * 2) + round256((size_t)M * 4);
    p.rexp_off = p.a16_off + round256((size_t)M * (size_t)K * 2);
    p.total_bytes = p.a16_off + p.a16_bytes;
  }
  plan_tail(p, K);
  return GEG_OK;
}

int persistent_grid(int64_t units_bound, int per_cu) {
  const int64_t cap = (int64_t)cu_count() * per_cu;
  return (int)std::max<int64_t>(1, std::min<int64_t>(units_bound, cap));
}

// Largest byte range one buffer resource of a kernel may cover.
constexpr int64_t kMaxWindow = 0x7FFFFFF0;

geg_status check_shape(int64_t M, int64_t N, int64_t K, int32_t E, int64_t kmult) {
  if (M < 0 || N <= 0 || K <= 0 || E <= 0)
    return fail(GEG_ERR_BAD_SHAPE, "need M >= 0, N > 0, K > 0, E > 0");
  if (E > geg::kMaxExperts) return fail(GEG_ERR_BAD_SHAPE, "E exceeds 1024 experts");
  if (M >= (int64_t)INT32_MAX) return fail(GEG_ERR_BAD_SHAPE, "M must be below 2^31");
  if (K % kmult) return fail(GEG_ERR_BAD_SHAPE, "K must be a multiple of " + std::to_string(kmult));
  // The kernels read one expert's packed weights, and at most 256 rows of an
  // activation / dY / output tensor, through 32-bit buffer windows. Refuse
  // shapes whose windows would not fit instead of clamping them.
  if (512 * std::max(N, K) > kMaxWindow)
    return fail(GEG_ERR_BAD_SHAPE, "256 rows of N or K bf16 values must fit in 0x7FFFFFF0 bytes (N, K <= 4194303)");
  if (N * (K / 2) > kMaxWindow)
    return fail(GEG_ERR_BAD_SHAPE, "an expert's packed weights (N * K / 2 bytes) must not exceed 0x7FFFFFF0 bytes");
  return GEG_OK;
}

// glu = 1: the fused expert block's first projection (out is [M, N/2], see GemmArgs).
// Low-rank adapter delta for the tiled kernel's epilogue (r == 0: none), and a
// step that runs after every check passed and before the GEMM's launches.
struct LoraIn {
  const float* u = nullptr;
  const float* q = nullptr;
  int32_t r = 0;
  float s = 0.f;
  std::function<hipError_t()> pre;
  std::function<hipError_t()> post;
};

// The library-held scratch of gnf4_grouped_gemm_noalloc in place of a caller's
// workspace, and the caller's device error word (NULL: the scratch header's).
struct Scratch {
  bool library = false;
  uint32_t* err_word = nullptr;
};

geg_status gemm_common(int fmt, const void* a, const int32_t* sizes, const uint8_t* wq,
                       const void* scales, void* out, int64_t M, int64_t N, int64_t K, int32_t E,
                       void* ws, size_t ws_bytes, const geg_opts* opts, hipStream_t stream,
                       int32_t glu = 0, const LoraIn& lora = LoraIn{}, const Scratch& scratch = Scratch{}) {
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, fmt == geg::NF4 ? 64 : 32);
  if (st != GEG_OK) return st;
  if (glu && (N % 2)) return fail(GEG_ERR_BAD_SHAPE, "the fused gate/up width must be even");
  if (glu && opts && opts->force_path == 1)
    return fail(GEG_ERR_BAD_OPTION, "the expert block does not run on the skinny kernel (force_path 1)");
  // the adapter delta lives in the tiled kernel's epilogue: every expert is tiled
  geg_opts tiled{};
  if (opts) tiled = *opts;
  tiled.force_path = 2;
  if (lora.r > 0) opts = &tiled;
  Plan p;
  st = make_plan(fmt == geg::NF4 ? GEG_OP_NF4_FWD : GEG_OP_MXFP4_FWD, M, N, K, E, opts, p);
  if (st != GEG_OK) return st;
  if (M == 0) return GEG_OK;
  if (!a || !sizes || !wq || !scales || !out) return fail(GEG_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!ws) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(a, 16) || !aligned(wq, 16) || !aligned(out, 16) || !aligned(sizes, 4) ||
      (fmt == geg::NF4 && !aligned(scales, 4)))
    return fail(GEG_ERR_MISALIGNED, "a, w/blocks and out must be 16-byte aligned");
  if (!aligned(ws, 256)) return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  fit_tail(p, ws_bytes);
  if (ws_bytes < p.total_bytes)
    return fail(GEG_ERR_WORKSPACE, "workspace smaller than geg_workspace_bytes(): need " +
                                       std::to_string(p.total_bytes));
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{a, "a"}, {sizes, "sizes"},
                           {wq, "weights"}, {scales, "scales"}, {out, "out"},
                           {scratch.library ? nullptr : ws, "workspace"}, {scratch.err_word, "error_word"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;

  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  geg::GemmArgs g;
  g.a = reinterpret_cast<const uint16_t*>(a);
  g.sizes = sizes;
  g.wq = wq;
  g.scales = scales;
  g.out = reinterpret_cast<uint16_t*>(out);
  g.M = M;
  g.N = N;
  g.K = K;
  g.E = E;
  g.thresh = p.thresh;
  g.split = p.split;
  g.cb = p.cb;
  g.vec_rows = p.vec_rows;
  g.err = scratch.err_word ? scratch.err_word : reinterpret_cast<uint32_t*>(wsb);
  g.partials = p.split > 1 ? reinterpret_cast<float*>(wsb + p.partials_off) : nullptr;
  g.tail_part = p.tail_bytes ? reinterpret_cast<float*>(wsb + p.tail_off) : nullptr;
  g.tail_split = p.tail_bytes ? kTailSplitMax : 1;
  g.a16 = p.a16_bytes ? reinterpret_cast<const uint16_t*>(wsb + p.a16_off) : nullptr;
  g.rexp = p.a16_bytes ? reinterpret_cast<const int32_t*>(wsb + p.rexp_off) : nullptr;
  g.glu = glu;
  g.lora_u = lora.u;
  g.lora_q = lora.q;
  g.lora_r = lora.r;
  g.lora_s = lora.s;
  if (lora.pre) {
    hipError_t e = lora.pre();
    if (e != hipSuccess) return hip_fail(e, "adapter launch");
  }

  if (p.run_tile) {
    if (fmt == geg::NF4) {
      hipError_t e = geg::launch_to_f16_rows(g.a, const_cast<uint16_t*>(g.a16), const_cast<int32_t*>(g.rexp), M, K,
                                             g.err, cu_count(), stream);
      if (e != hipSuccess) return hip_fail(e, "activation conversion launch");
      ++g_launches;
    }
    const int64_t n_tiles = (N + geg::kTileN - 1) / geg::kTileN;
    const int64_t tile_experts = std::min<int64_t>(E, M / (std::max<int64_t>(p.thresh, 0) + 1));
    const int64_t bound = ((M + geg::kTileM - 1) / geg::kTileM + tile_experts) * n_tiles;
    const int grid = persistent_grid(bound, 1);
    hipError_t e = record_event(opts, 0, stream);
    if (e == hipSuccess) e = geg::launch_tile(fmt, g, grid, stream);
    if (e != hipSuccess) return hip_fail(e, "tile kernel launch");
    ++g_launches;
    if (g.tail_split > 1) {
      e = geg::launch_tile_fixup(g, false, grid, stream);
      if (e != hipSuccess) return hip_fail(e, "tile fixup launch");
      ++g_launches;
    }
    e = record_event(opts, 1, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel event");
  }
  if (p.run_vec) {
    hipError_t e = record_event(opts, 2, stream);
    if (e == hipSuccess) e = geg::launch_vec(fmt, g, cu_count(), stream);
    if (e == hipSuccess && !p.run_skinny) e = record_event(opts, 3, stream);
    if (e != hipSuccess) return hip_fail(e, "vector kernel launch");
    ++g_launches;
  }
  if (p.run_skinny && p.narrow) {
    hipError_t e = p.run_vec ? hipSuccess : record_event(opts, 2, stream);
    if (e == hipSuccess) e = geg::launch_narrow(fmt, g, cu_count(), stream);
    if (e == hipSuccess) e = record_event(opts, 3, stream);
    if (e != hipSuccess) return hip_fail(e, "narrow kernel launch");
    ++g_launches;
  } else if (p.run_skinny) {
    const int64_t n_chunks = (N + 16 * p.cb - 1) / (16 * p.cb);
    const int64_t bound = p.rc_bound * n_chunks * p.split;
    hipError_t e = p.run_vec ? hipSuccess : record_event(opts, 2, stream);
    if (e == hipSuccess) e = geg::launch_skinny(fmt, g, persistent_grid(bound, 2), stream);
    if (e != hipSuccess) return hip_fail(e, "skinny kernel launch");
    ++g_launches;
    if (p.split > 1) {
      // units: (row of a skinny expert, 256 columns); at most M rows
      e = geg::launch_splitk_reduce(g, persistent_grid(M * ((N + geg::kThreads - 1) / geg::kThreads), 8), stream);
      if (e != hipSuccess) return hip_fail(e, "split-K reduce launch");
      ++g_launches;
    }
    e = record_event(opts, 3, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel event");
  }
  return GEG_OK;
}

// Workspace layout of the fused expert block: both projections' own regions
// (they run one after the other and share the error word), then the bf16
// intermediate act [M, I].
geg_status block_layout(int fmt, int64_t M, int64_t H, int64_t I, int32_t E, const geg_opts* o,
                        size_t& act_off, size_t& total) {
  const int op = fmt == geg::NF4 ? GEG_OP_NF4_FWD : GEG_OP_MXFP4_FWD;
  Plan p1, p2;
  geg_status st;
  if ((st = make_plan(op, M, 2 * I, H, E, o, p1)) != GEG_OK) return st;
  if ((st = make_plan(op, M, H, I, E, o, p2)) != GEG_OK) return st;
  // past both GEMMs' scratch
  act_off = round256(std::max(p1.total_bytes, p2.total_bytes));
  total = act_off + round256((size_t)M * (size_t)I * 2);
  return GEG_OK;
}

geg_status block_common(int fmt, const void* a, const int32_t* sizes, const uint8_t* w13,
                        const void* s13, const uint8_t* w2, const void* s2, void* out, int64_t M,
                        int64_t H, int64_t I, int32_t E, void* ws, size_t ws_bytes,
                        const geg_opts* opts, hipStream_t stream) {
  CuScope cu_scope(opts);
  const int64_t kmult = fmt == geg::NF4 ? 64 : 32;
  geg_status st;
  if ((st = check_shape(M, 2 * I, H, E, kmult)) != GEG_OK) return st;
  if (I <= 0 || I % kmult) return fail(GEG_ERR_BAD_SHAPE, "I must be a positive multiple of " + std::to_string(kmult));
  if (opts && opts->force_path == 1)
    return fail(GEG_ERR_BAD_OPTION, "the expert block does not run on the skinny kernel (force_path 1)");
  size_t act_off = 0, total = 0;
  if ((st = block_layout(fmt, M, H, I, E, opts, act_off, total)) != GEG_OK) return st;
  if (M == 0) return GEG_OK;
  if (!w2 || !s2) return fail(GEG_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!ws) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < total)
    return fail(GEG_ERR_WORKSPACE, "workspace smaller than geg_workspace_bytes(): need " + std::to_string(total));
  if (!aligned(w2, 16) || (fmt == geg::NF4 && !aligned(s2, 4)))
    return fail(GEG_ERR_MISALIGNED, "w2/blocks2 must be 16-byte aligned");
  if ((st = check_device_ptr(w2, "w2")) != GEG_OK) return st;
  if ((st = check_device_ptr(s2, "scales2")) != GEG_OK) return st;
  geg_opts inner{};
  if (opts) inner = *opts;
  inner.kernel_events = nullptr;
  hipError_t e = record_event(opts, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  void* act = reinterpret_cast<uint8_t*>(ws) + act_off;
  st = gemm_common(fmt, a, sizes, w13, s13, act, M, 2 * I, H, E, ws, act_off, &inner, stream, 1);
  if (st != GEG_OK) return st;
  st = gemm_common(fmt, act, sizes, w2, s2, out, M, H, I, E, ws, act_off, &inner, stream, 0);
  if (st != GEG_OK) return st;
  e = record_event(opts, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  return GEG_OK;
}

geg_status dgrad_common(int fmt, const void* dy, const int32_t* sizes, const uint8_t* w, const void* absmax,
                        void* dx, int64_t M, int64_t N, int64_t K, int32_t E, void* workspace,
                        size_t workspace_bytes, const geg_opts* opts, hipStream_t stream,
                        const LoraIn& lora = LoraIn{}) {
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, fmt == geg::NF4 ? 64 : 32);
  if (st != GEG_OK) return st;
  if (N % 8) return fail(GEG_ERR_BAD_SHAPE, "dgrad needs N % 8 == 0");
  Plan p;
  if ((st = make_plan(fmt == geg::NF4 ? GEG_OP_NF4_DGRAD : GEG_OP_MXFP4_DGRAD, M, N, K, E, opts, p)) != GEG_OK)
    return st;
  if (M == 0) return GEG_OK;
  if (!dy || !sizes || !w || !absmax || !dx) return fail(GEG_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!workspace) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(dy, 16) || !aligned(w, 16) || !aligned(dx, 16) || (fmt == geg::NF4 && !aligned(absmax, 4)) ||
      !aligned(sizes, 4))
    return fail(GEG_ERR_MISALIGNED, "dy, w and dx must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  fit_tail(p, workspace_bytes);
  if (workspace_bytes < p.total_bytes) return fail(GEG_ERR_WORKSPACE, "workspace too small");
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{dy, "dy"}, {sizes, "sizes"},
                           {w, "w"}, {absmax, "absmax"}, {dx, "dx"}, {workspace, "workspace"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  geg::GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.a = reinterpret_cast<const uint16_t*>(dy);
  g.a16 = p.a16_bytes ? reinterpret_cast<const uint16_t*>(wsb + p.a16_off) : nullptr;
  g.rexp = p.a16_bytes ? reinterpret_cast<const int32_t*>(wsb + p.rexp_off) : nullptr;
  g.sizes = sizes;
  g.wq = w;
  g.scales = absmax;
  g.out = reinterpret_cast<uint16_t*>(dx);
  g.M = M;
  g.N = N;
  g.K = K;
  g.E = E;
  g.thresh = 0;   // every expert with rows goes through the tiled kernel
  g.lora_u = lora.u;
  g.lora_q = lora.q;
  g.lora_r = lora.r;
  g.lora_s = lora.s;
  g.split = 1;
  g.glu = 0;
  g.tail_part = p.tail_bytes ? reinterpret_cast<float*>(wsb + p.tail_off) : nullptr;
  g.tail_split = p.tail_bytes ? kTailSplitMax : 1;
  g.err = reinterpret_cast<uint32_t*>(wsb);
  hipError_t e = hipSuccess;
  if (lora.pre && (e = lora.pre()) != hipSuccess) return hip_fail(e, "adapter launch");
  if (fmt == geg::NF4) {
    e = geg::launch_to_f16_rows(g.a, const_cast<uint16_t*>(g.a16), const_cast<int32_t*>(g.rexp), M, N, g.err,
                                cu_count(), stream);
    if (e != hipSuccess) return hip_fail(e, "dY conversion launch");
    ++g_launches;
  }
  const int64_t k_tiles = (K + geg::kTileN - 1) / geg::kTileN;
  const int64_t bound = ((M + geg::kTileM - 1) / geg::kTileM + std::min<int64_t>(E, M)) * k_tiles;
  const int grid = persistent_grid(bound, 1);
  e = record_event(opts, 0, stream);
  if (e == hipSuccess) e = geg::launch_tile_dgrad(fmt, g, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "dgrad kernel launch");
  ++g_launches;
  if (g.tail_split > 1) {
    e = geg::launch_tile_fixup(g, true, grid, stream);
    if (e != hipSuccess) return hip_fail(e, "dgrad fixup launch");
    ++g_launches;
  }
  e = record_event(opts, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel event");
  if (lora.post && (e = lora.post()) != hipSuccess) return hip_fail(e, "adapter launch");
  return GEG_OK;
}

}  // namespace

extern "C" {

geg_status gnf4_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* w,
                             const float* absmax, void* out, int64_t M, int64_t N, int64_t K,
                             int32_t E, void* workspace, size_t workspace_bytes,
                             const geg_opts* opts, hipStream_t stream) {
  return gemm_common(geg::NF4, a, sizes, w, absmax, out, M, N, K, E, workspace, workspace_bytes,
                     opts, stream);
}

geg_status gnf4_grouped_gemm_noalloc(const void* a, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                     void* out, int64_t M, int64_t N, int64_t K, int32_t E, uint32_t* error_word,
                                     const geg_opts* opts, hipStream_t stream) {
  // Every check that needs no device data first (nothing is enqueued when one
  // fails), then the library-held scratch in place of a workspace.
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, 64);
  if (st != GEG_OK) return st;
  Plan p;
  if ((st = make_plan(GEG_OP_NF4_FWD, M, N, K, E, opts, p)) != GEG_OK) return st;
  if (M == 0) return GEG_OK;
  fit_tail(p, geg::kNoallocScratchBytes);
  if (p.total_bytes > geg::kNoallocScratchBytes)
    return fail(GEG_ERR_WORKSPACE, "this call needs " + std::to_string(p.total_bytes) +
                                       " bytes of scratch; the library-held array holds " +
                                       std::to_string(geg::kNoallocScratchBytes) +
                                       " (144 MiB): call gnf4_grouped_gemm with a workspace");
  if (!a || !sizes || !w || !absmax || !out) return fail(GEG_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(sizes, 4) || !aligned(absmax, 4) ||
      (error_word && !aligned(error_word, 4)))
    return fail(GEG_ERR_MISALIGNED, "a, w and out must be 16-byte aligned, sizes, absmax and error_word 4-byte");
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{a, "a"}, {sizes, "sizes"}, {w, "weights"},
                           {absmax, "absmax"}, {out, "out"}, {error_word, "error_word"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  void* ws = nullptr;
  hipError_t e = geg::noalloc_scratch(&ws, stream);
  if (e != hipSuccess) return hip_fail(e, "library-held scratch");
  Scratch sc;
  sc.library = true;
  sc.err_word = error_word;
  return gemm_common(geg::NF4, a, sizes, w, absmax, out, M, N, K, E, ws, geg::kNoallocScratchBytes, opts, stream, 0,
                     LoraIn{}, sc);
}

geg_status gmxfp4_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* blocks,
                               const uint8_t* scales, void* out, int64_t M, int64_t N, int64_t K,
                               int32_t E, void* workspace, size_t workspace_bytes,
                               const geg_opts* opts, hipStream_t stream) {
  return gemm_common(geg::MXFP4, a, sizes, blocks, scales, out, M, N, K, E, workspace,
                     workspace_bytes, opts, stream);
}

geg_status gnf4_expert_block(const void* a, const int32_t* sizes, const uint8_t* w13,
                             const float* absmax13, const uint8_t* w2, const float* absmax2,
                             void* out, int64_t M, int64_t H, int64_t I, int32_t E,
                             void* workspace, size_t workspace_bytes, const geg_opts* opts,
                             hipStream_t stream) {
  return block_common(geg::NF4, a, sizes, w13, absmax13, w2, absmax2, out, M, H, I, E, workspace,
                      workspace_bytes, opts, stream);
}

geg_status gmxfp4_expert_block(const void* a, const int32_t* sizes, const uint8_t* blocks13,
                               const uint8_t* scales13, const uint8_t* blocks2,
                               const uint8_t* scales2, void* out, int64_t M, int64_t H, int64_t I,
                               int32_t E, void* workspace, size_t workspace_bytes,
                               const geg_opts* opts, hipStream_t stream) {
  return block_common(geg::MXFP4, a, sizes, blocks13, scales13, blocks2, scales2, out, M, H, I, E,
                      workspace, workspace_bytes, opts, stream);
}

geg_status gnf4_grouped_dgrad(const void* dy, const int32_t* sizes, const uint8_t* w,
                              const float* absmax, void* dx, int64_t M, int64_t N, int64_t K,
                              int32_t E, void* workspace, size_t workspace_bytes,
                              const geg_opts* opts, hipStream_t stream) {
  return dgrad_common(geg::NF4, dy, sizes, w, absmax, dx, M, N, K, E, workspace, workspace_bytes, opts, stream);
}

geg_status gmxfp4_grouped_dgrad(const void* dy, const int32_t* sizes, const uint8_t* blocks,
                                const uint8_t* scales, void* dx, int64_t M, int64_t N, int64_t K,
                                int32_t E, void* workspace, size_t workspace_bytes,
                                const geg_opts* opts, hipStream_t stream) {
  return dgrad_common(geg::MXFP4, dy, sizes, blocks, scales, dx, M, N, K, E, workspace, workspace_bytes, opts,
                      stream);
}

geg_status gmxfp4_w4a8_grouped_gemm(const void* a, const int32_t* sizes, const uint8_t* blocks,
                                    const uint8_t* scales, void* out, int64_t M, int64_t N, int64_t K,
                                    int32_t E, void* workspace, size_t workspace_bytes,
                                    const geg_opts* opts, hipStream_t stream) {
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, 32);
  if (st != GEG_OK) return st;
  // 32-bit buffer offsets within a 256-row tile of activation codes
  if (K >= (int64_t)1 << 23) return fail(GEG_ERR_BAD_SHAPE, "K must be below 2^23");
  // the activation scales are read through one window: ceil(K / 128) steps of M rows of 4 bytes
  if ((K + 127) / 128 * M * 4 > kMaxWindow)
    return fail(GEG_ERR_BAD_SHAPE, "the activation scales (ceil(K/128) * M * 4 bytes) must fit in 0x7FFFFFF0 bytes");
  Plan p;
  if ((st = make_plan(GEG_OP_MXFP4_W4A8, M, N, K, E, opts, p)) != GEG_OK) return st;
  if (M == 0) return GEG_OK;
  if (!a || !sizes || !blocks || !scales || !out) return fail(GEG_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!workspace) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(a, 16) || !aligned(blocks, 16) || !aligned(out, 4) || !aligned(sizes, 4))
    return fail(GEG_ERR_MISALIGNED, "a and blocks must be 16-byte aligned, out 4-byte");
  if (!aligned(workspace, 256)) return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.total_bytes)
    return fail(GEG_ERR_WORKSPACE, "workspace smaller than geg_workspace_bytes(): need " +
                                       std::to_string(p.total_bytes));
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{a, "a"}, {sizes, "sizes"}, {blocks, "blocks"},
                           {scales, "scales"}, {out, "out"}, {workspace, "workspace"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  uint32_t* err = reinterpret_cast<uint32_t*>(wsb);
  uint8_t* aq = wsb + p.a16_off;
  uint8_t* as = aq + round256((size_t)M * (size_t)K);
  const int cus = cu_count();
  hipError_t e = geg::launch_mxfp8_quantize(reinterpret_cast<const uint16_t*>(a), M, K, aq, as, err, 1, cus, stream);
  if (e != hipSuccess) return hip_fail(e, "activation quantisation launch");
  ++g_launches;
  e = record_event(opts, 0, stream);
  if (e == hipSuccess)
    e = geg::launch_w4a8(aq, as, sizes, blocks, scales, reinterpret_cast<uint16_t*>(out), M, N, K, E, err, cus,
                         stream);
  if (e == hipSuccess) e = record_event(opts, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "W4A8 kernel launch");
  ++g_launches;
  return GEG_OK;
}

geg_status gmxfp8_quantize(const void* a, uint8_t* codes, uint8_t* scales, int64_t M, int64_t K,
                           hipStream_t stream) {
  if (M < 0 || K <= 0 || K % 32) return fail(GEG_ERR_BAD_SHAPE, "need M >= 0, K > 0, K % 32 == 0");
  if (M == 0) return GEG_OK;
  if (!a || !codes || !scales) return fail(GEG_ERR_NULL_POINTER, "a, codes and scales are required");
  if (!aligned(a, 16) || !aligned(codes, 16)) return fail(GEG_ERR_MISALIGNED, "a and codes must be 16-byte aligned");
  geg_status st;
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{a, "a"}, {codes, "codes"}, {scales, "scales"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  hipError_t e = geg::launch_mxfp8_quantize(reinterpret_cast<const uint16_t*>(a), M, K, codes, scales, nullptr, 0,
                                            cu_count(), stream);
  if (e != hipSuccess) return hip_fail(e, "activation quantisation launch");
  ++g_launches;
  return GEG_OK;
}

size_t geg_lora_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t E, int32_t r) {
  if (M < 0 || N <= 0 || K <= 0 || E <= 0 || r <= 0) return 0;
  Plan p;
  if (op == GEG_OP_NF4_FWD || op == GEG_OP_MXFP4_FWD) {
    geg_opts tiled{};
    tiled.force_path = 2;
    if (make_plan(op, M, N, K, E, &tiled, p) != GEG_OK) return 0;
    return p.total_bytes;
  }
  if (op != GEG_OP_NF4_DGRAD && op != GEG_OP_MXFP4_DGRAD) return 0;
  if (make_plan(op, M, N, K, E, nullptr, p) != GEG_OK) return 0;
  return p.total_bytes + round256((size_t)E * r * N * 4) +
         round256((size_t)E * K * r * 4) + round256((size_t)M * r * 4);
}

}  // extern "C"

namespace {

geg_status lora_args(int32_t r, const float* lora_a, const float* lora_b) {
  if (r < 8 || r > 64 || r % 8) return fail(GEG_ERR_BAD_SHAPE, "the adapter rank r must be 8, 16, ..., 64");
  if (!lora_a || !lora_b) return fail(GEG_ERR_NULL_POINTER, "lora_a and lora_b are required");
  if (!aligned(lora_a, 16) || !aligned(lora_b, 16)) return fail(GEG_ERR_MISALIGNED, "lora_a and lora_b must be 16-byte aligned");
  geg_status st;
  if ((st = check_device_ptr(lora_a, "lora_a")) != GEG_OK) return st;
  return check_device_ptr(lora_b, "lora_b");
}

geg_status gemm_lora(int fmt, const void* a, const int32_t* sizes, const uint8_t* w, const void* scales,
                     const float* lora_a, const float* lora_b, float scale, void* out, void* u, int64_t M, int64_t N,
                     int64_t K, int32_t E, int32_t r, void* workspace, size_t workspace_bytes, const geg_opts* opts,
                     hipStream_t stream) {
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, fmt == geg::NF4 ? 64 : 32);
  if (st != GEG_OK) return st;
  if (M == 0) return GEG_OK;
  if ((st = lora_args(r, lora_a, lora_b)) != GEG_OK) return st;
  if (!u) return fail(GEG_ERR_NULL_POINTER, "u is required");
  if (!aligned(u, 16)) return fail(GEG_ERR_MISALIGNED, "u must be 16-byte aligned");
  if ((st = check_device_ptr(u, "u")) != GEG_OK) return st;
  LoraIn L;
  L.u = reinterpret_cast<const float*>(u);
  L.q = lora_b;
  L.r = r;
  L.s = scale;
  // u = x A_e^T first; the tiled kernel's epilogue then adds s u B_e^T
  L.pre = [=]() -> hipError_t {
    ++g_launches;
    return geg::launch_lora_down(reinterpret_cast<const uint16_t*>(a), lora_a, sizes, E, M, K, r, 1.0f,
                                 reinterpret_cast<float*>(u), reinterpret_cast<uint32_t*>(workspace), cu_count(),
                                 stream);
  };
  return gemm_common(fmt, a, sizes, w, scales, out, M, N, K, E, workspace, workspace_bytes, opts, stream, 0, L);
}

geg_status dgrad_lora(int fmt, const void* dy, const int32_t* sizes, const uint8_t* w, const void* scales,
                      const void* x, const float* lora_a, const float* lora_b, const void* u, float scale, void* dx,
                      float* grad_a, float* grad_b, int64_t M, int64_t N, int64_t K, int32_t E, int32_t r,
                      void* workspace, size_t workspace_bytes, const geg_opts* opts, hipStream_t stream) {
  CuScope cu_scope(opts);
  geg_status st = check_shape(M, N, K, E, fmt == geg::NF4 ? 64 : 32);
  if (st != GEG_OK) return st;
  if (N % 8) return fail(GEG_ERR_BAD_SHAPE, "dgrad needs N % 8 == 0");
  if ((st = lora_args(r, lora_a, lora_b)) != GEG_OK) return st;
  if (!grad_a || !grad_b || !sizes) return fail(GEG_ERR_NULL_POINTER, "grad_a, grad_b and sizes are required");
  if (!aligned(grad_a, 4) || !aligned(grad_b, 4)) return fail(GEG_ERR_MISALIGNED, "grad_a and grad_b must be 4-byte aligned");
  if (M > 0 && (!x || !u)) return fail(GEG_ERR_NULL_POINTER, "x and u are required");
  if (M > 0 && (!aligned(x, 16) || !aligned(u, 16))) return fail(GEG_ERR_MISALIGNED, "x and u must be 16-byte aligned");
  if (!workspace) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = geg_lora_workspace_bytes(fmt == geg::NF4 ? GEG_OP_NF4_DGRAD : GEG_OP_MXFP4_DGRAD, M, N, K, E, r);
  if (workspace_bytes < need)
    return fail(GEG_ERR_WORKSPACE, "workspace smaller than geg_lora_workspace_bytes(): need " + std::to_string(need));
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{grad_a, "grad_a"}, {grad_b, "grad_b"},
                           {sizes, "sizes"}, {workspace, "workspace"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  if (M > 0)
    for (auto [ptr, name] : {std::pair<const void*, const char*>{x, "x"}, {u, "u"}})
      if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  Plan p;
  if ((st = make_plan(fmt == geg::NF4 ? GEG_OP_NF4_DGRAD : GEG_OP_MXFP4_DGRAD, M, N, K, E, nullptr, p)) != GEG_OK)
    return st;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  uint32_t* err = reinterpret_cast<uint32_t*>(wsb);
  // adapter scratch past the dgrad's own
  const size_t lb = p.total_bytes;
  float* Bt = reinterpret_cast<float*>(wsb + lb);                                    // [E, r, N]
  float* At = reinterpret_cast<float*>(wsb + lb + round256((size_t)E * r * N * 4));  // [E, K, r]
  float* g = reinterpret_cast<float*>(wsb + lb + round256((size_t)E * r * N * 4) +
                                      round256((size_t)E * K * r * 4));              // [M, r]
  const int cus = cu_count();
  const uint16_t* dy16 = reinterpret_cast<const uint16_t*>(dy);
  // adapter gradients (zeros for experts without rows, and for M == 0)
  auto grads = [=]() -> hipError_t {
    hipError_t e = geg::launch_lora_grad(dy16, reinterpret_cast<const float*>(u), sizes, E, M, N, r, scale, grad_b,
                                         false, err, cus, stream);
    if (e == hipSuccess)
      e = geg::launch_lora_grad(reinterpret_cast<const uint16_t*>(x), g, sizes, E, M, K, r, 1.0f, grad_a, true, err,
                                cus, stream);
    g_launches += 2;
    return e;
  };
  if (M == 0) {
    hipError_t e = grads();
    return e == hipSuccess ? GEG_OK : hip_fail(e, "adapter launch");
  }
  LoraIn L;
  L.u = g;
  L.q = At;
  L.r = r;
  L.s = 1.0f;
  // g = s dy B_e (from a transposed copy of B) and a transposed copy of A first;
  // the dgrad epilogue adds g A_e; the gradients after
  L.pre = [=]() -> hipError_t {
    hipError_t e = geg::launch_lora_transpose(lora_b, E, N, r, Bt, cus, stream);
    if (e == hipSuccess) e = geg::launch_lora_down(dy16, Bt, sizes, E, M, N, r, scale, g, err, cus, stream);
    if (e == hipSuccess) e = geg::launch_lora_transpose(lora_a, E, r, K, At, cus, stream);
    g_launches += 3;
    return e;
  };
  L.post = grads;
  return dgrad_common(fmt, dy, sizes, w, scales, dx, M, N, K, E, workspace, workspace_bytes, opts, stream, L);
}

}  // namespace

extern "C" {

geg_status gnf4_grouped_gemm_lora(const void* a, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                  const float* lora_a, const float* lora_b, float scale, void* out, void* u, int64_t M,
                                  int64_t N, int64_t K, int32_t E, int32_t r, void* workspace, size_t workspace_bytes,
                                  const geg_opts* opts, hipStream_t stream) {
  return gemm_lora(geg::NF4, a, sizes, w, absmax, lora_a, lora_b, scale, out, u, M, N, K, E, r, workspace,
                   workspace_bytes, opts, stream);
}

geg_status gmxfp4_grouped_gemm_lora(const void* a, const int32_t* sizes, const uint8_t* blocks, const uint8_t* scales,
                                    const float* lora_a, const float* lora_b, float scale, void* out, void* u,
                                    int64_t M, int64_t N, int64_t K, int32_t E, int32_t r, void* workspace,
                                    size_t workspace_bytes, const geg_opts* opts, hipStream_t stream) {
  return gemm_lora(geg::MXFP4, a, sizes, blocks, scales, lora_a, lora_b, scale, out, u, M, N, K, E, r, workspace,
                   workspace_bytes, opts, stream);
}

geg_status gnf4_grouped_dgrad_lora(const void* dy, const int32_t* sizes, const uint8_t* w, const float* absmax,
                                   const void* x, const float* lora_a, const float* lora_b, const void* u, float scale,
                                   void* dx, float* grad_a, float* grad_b, int64_t M, int64_t N, int64_t K, int32_t E,
                                   int32_t r, void* workspace, size_t workspace_bytes, const geg_opts* opts,
                                   hipStream_t stream) {
  return dgrad_lora(geg::NF4, dy, sizes, w, absmax, x, lora_a, lora_b, u, scale, dx, grad_a, grad_b, M, N, K, E, r,
                    workspace, workspace_bytes, opts, stream);
}

geg_status gmxfp4_grouped_dgrad_lora(const void* dy, const int32_t* sizes, const uint8_t* blocks,
                                     const uint8_t* scales, const void* x, const float* lora_a, const float* lora_b,
                                     const void* u, float scale, void* dx, float* grad_a, float* grad_b, int64_t M,
                                     int64_t N, int64_t K, int32_t E, int32_t r, void* workspace,
                                     size_t workspace_bytes, const geg_opts* opts, hipStream_t stream) {
  return dgrad_lora(geg::MXFP4, dy, sizes, blocks, scales, x, lora_a, lora_b, u, scale, dx, grad_a, grad_b, M, N, K,
                    E, r, workspace, workspace_bytes, opts, stream);
}

size_t geg_route_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k <= 0 || E <= 0 || E > geg::kMaxExperts) return 0;
  const int64_t nchunks = (T * k + geg::kThreads - 1) / geg::kThreads;
  // per-chunk expert counts after the header
  return kHeader + round256((size_t)std::max<int64_t>(nchunks, 1) * (size_t)E * 4);
}

geg_status geg_route_sort(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, const void* x,
                          int64_t H, int32_t* sizes, int32_t* row_of, int32_t* src_of, void* x_sorted,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || k <= 0 || E <= 0) return fail(GEG_ERR_BAD_SHAPE, "need T >= 0, k > 0, E > 0");
  if (E > geg::kMaxExperts) return fail(GEG_ERR_BAD_SHAPE, "E exceeds 1024 experts");
  if (T * (int64_t)k >= (int64_t)INT32_MAX) return fail(GEG_ERR_BAD_SHAPE, "T * k must be below 2^31");
  const bool gather = x || x_sorted;
  if (gather && (!x || !x_sorted)) return fail(GEG_ERR_NULL_POINTER, "x and x_sorted go together");
  if (gather && (H <= 0 || H % 8)) return fail(GEG_ERR_BAD_SHAPE, "the gather needs H > 0, H % 8 == 0");
  if (!sizes || !workspace) return fail(GEG_ERR_NULL_POINTER, "sizes and workspace are required");
  if (T > 0 && (!topk_ids || !row_of || !src_of))
    return fail(GEG_ERR_NULL_POINTER, "topk_ids, row_of and src_of are required");
  if ((gather && (!aligned(x, 16) || !aligned(x_sorted, 16))) || !aligned(topk_ids, 4) ||
      !aligned(sizes, 4) || !aligned(row_of, 4) || !aligned(src_of, 4))
    return fail(GEG_ERR_MISALIGNED, "x and x_sorted must be 16-byte aligned, index arrays 4-byte");
  if (!aligned(workspace, 256)) return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < geg_route_workspace_bytes(T, k, E))
    return fail(GEG_ERR_WORKSPACE, "workspace smaller than geg_route_workspace_bytes()");
  geg_status st;
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{topk_ids, "topk_ids"}, {sizes, "sizes"},
                           {row_of, "row_of"}, {src_of, "src_of"}, {x, "x"}, {x_sorted, "x_sorted"},
                           {workspace, "workspace"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  const int64_t n = T * k;
  hipError_t e = geg::launch_route_sort(topk_ids, n, E, reinterpret_cast<int32_t*>(wsb + kHeader), sizes,
                                        row_of, src_of, reinterpret_cast<uint32_t*>(wsb), stream);
  if (e != hipSuccess) return hip_fail(e, "routing sort launch");
  g_launches += n > 0 ? 3 : 1;
  if (gather && n > 0) {
    e = geg::launch_route_gather(reinterpret_cast<const uint16_t*>(x), H, k, src_of, n,
                                 reinterpret_cast<uint16_t*>(x_sorted), cu_count(), stream);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
    ++g_launches;
  }
  return GEG_OK;
}

geg_status geg_route_combine(const void* y, const int32_t* row_of, const float* weights, int64_t T,
                             int32_t k, int64_t N, void* out, hipStream_t stream) {
  if (T < 0 || k <= 0 || N <= 0 || N % 8) return fail(GEG_ERR_BAD_SHAPE, "need T >= 0, k > 0, N > 0, N % 8 == 0");
  if (T * (int64_t)k >= (int64_t)INT32_MAX) return fail(GEG_ERR_BAD_SHAPE, "T * k must be below 2^31");
  if (T == 0) return GEG_OK;
  if (!y || !row_of || !out) return fail(GEG_ERR_NULL_POINTER, "y, row_of and out are required");
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(row_of, 4) || (weights && !aligned(weights, 4)))
    return fail(GEG_ERR_MISALIGNED, "y and out must be 16-byte aligned");
  geg_status st;
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{y, "y"}, {row_of, "row_of"},
                           {weights, "weights"}, {out, "out"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  hipError_t e = geg::launch_route_combine(reinterpret_cast<const uint16_t*>(y), N, row_of, weights, T, k,
                                           reinterpret_cast<uint16_t*>(out), cu_count(), stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  ++g_launches;
  return GEG_OK;
}

size_t geg_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t E,
                           const geg_opts* opts) {
  if (op < 0 || op > 6 || M < 0 || N <= 0 || K <= 0 || E <= 0) return 0;
  if (op == GEG_OP_NF4_BLOCK || op == GEG_OP_MXFP4_BLOCK) {
    size_t act_off = 0, total = 0;
    if (block_layout(op == GEG_OP_NF4_BLOCK ? geg::NF4 : geg::MXFP4, M, N, K, E, opts, act_off, total) != GEG_OK)
      return 0;
    return total;
  }
  Plan p;
  if (make_plan(op, M, N, K, E, opts, p) != GEG_OK) return 0;
  return p.total_bytes;
}

geg_status geg_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return fail(GEG_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256) || workspace_bytes < kHeader)
    return fail(GEG_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= 256 bytes");
  geg_status st;
  if ((st = check_device()) != GEG_OK) return st;
  if ((st = check_device_ptr(workspace, "workspace")) != GEG_OK) return st;
  // Only the error word must start at zero.
  const size_t zero_bytes = kHeader;
  hipError_t e = geg::launch_zero(workspace, zero_bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "workspace zero launch");
  ++g_launches;
  return GEG_OK;
}

geg_status geg_read_device_error(const void* workspace, int32_t* code, hipStream_t stream) {
  if (!workspace || !code) return fail(GEG_ERR_NULL_POINTER, "workspace and code must be non-NULL");
  geg_status st;
  if ((st = check_device_ptr(workspace, "workspace")) != GEG_OK) return st;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t v = 0;
  e = hipMemcpy(&v, workspace, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy of the error word");
  *code = (int32_t)v;
  return GEG_OK;
}

static geg_status dequant_common(int fmt, const uint8_t* wq, const void* scales, float* f32,
                                 uint16_t* bf16, uint16_t* f16, int64_t N, int64_t K, int32_t E,
                                 hipStream_t stream) {
  geg_status st = check_shape(0, N, K, E, fmt == geg::NF4 ? 64 : 32);
  if (st != GEG_OK) return st;
  if (!wq || !scales || !f32) return fail(GEG_ERR_NULL_POINTER, "w, scales and out_f32 are required");
  if (!aligned(wq, 4) || !aligned(f32, 16) || (bf16 && !aligned(bf16, 16)) || (f16 && !aligned(f16, 16)))
    return fail(GEG_ERR_MISALIGNED, "w must be 4-byte and outputs 16-byte aligned");
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{wq, "w"}, {scales, "scales"},
                           {f32, "out_f32"}, {bf16, "out_bf16"}, {f16, "out_f16"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  hipError_t e = geg::launch_dequant(fmt, wq, scales, f32, bf16, f16, (int64_t)E * N, K, stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  ++g_launches;
  return GEG_OK;
}

geg_status gnf4_dequant(const uint8_t* w, const float* absmax, float* out_f32, uint16_t* out_bf16,
                        uint16_t* out_f16, int64_t N, int64_t K, int32_t E, hipStream_t stream) {
  return dequant_common(geg::NF4, w, absmax, out_f32, out_bf16, out_f16, N, K, E, stream);
}

geg_status gmxfp4_dequant(const uint8_t* blocks, const uint8_t* scales, float* out_f32,
                          uint16_t* out_bf16, uint16_t* out_f16, int64_t N, int64_t K, int32_t E,
                          hipStream_t stream) {
  return dequant_common(geg::MXFP4, blocks, scales, out_f32, out_bf16, out_f16, N, K, E, stream);
}

geg_status gnf4_quantize(const float* w, uint8_t* codes, float* absmax, int64_t rows, int64_t K,
                         hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 64) return fail(GEG_ERR_BAD_SHAPE, "need rows >= 0, K > 0, K % 64 == 0");
  if (rows == 0) return GEG_OK;
  if (!w || !codes || !absmax) return fail(GEG_ERR_NULL_POINTER, "w, codes and absmax are required");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
    return fail(GEG_ERR_MISALIGNED, "w and codes must be 16-byte aligned");
  geg_status st;
  if ((st = check_device()) != GEG_OK) return st;
  for (auto [ptr, name] : {std::pair<const void*, const char*>{w, "w"}, {codes, "codes"}, {absmax, "absmax"}})
    if ((st = check_device_ptr(ptr, name)) != GEG_OK) return st;
  hipError_t e = geg::launch_quantize_nf4(w, codes, absmax, rows, K, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  ++g_launches;
  return GEG_OK;
}

const char* geg_status_string(geg_status s) {
  switch (s) {
    case GEG_OK: return "GEG_OK";
    case GEG_ERR_NULL_POINTER: return "GEG_ERR_NULL_POINTER";
    case GEG_ERR_BAD_SHAPE: return "GEG_ERR_BAD_SHAPE";
    case GEG_ERR_MISALIGNED: return "GEG_ERR_MISALIGNED";
    case GEG_ERR_NOT_DEVICE_MEMORY: return "GEG_ERR_NOT_DEVICE_MEMORY";
    case GEG_ERR_WORKSPACE: return "GEG_ERR_WORKSPACE";
    case GEG_ERR_UNSUPPORTED_DEVICE: return "GEG_ERR_UNSUPPORTED_DEVICE";
    case GEG_ERR_HIP: return "GEG_ERR_HIP";
    case GEG_ERR_BAD_OPTION: return "GEG_ERR_BAD_OPTION";
  }
  return "unknown geg_status";
}

const char* geg_last_error(void) { return g_last_error.c_str(); }

int32_t geg_version(void) { return GEG_VERSION; }

uint64_t geg_launch_count(void) { return g_launches.load(); }

}  // extern "C"
