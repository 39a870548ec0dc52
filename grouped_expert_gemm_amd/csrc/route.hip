// Routing around the grouped GEMM, on the device: the sort of a layer's (token,
// slot) pairs by expert that produces the GEMM's grouped rows and `sizes`, and
// the top-k weighted combine of the expert outputs back into token order.
//
// Sort order: by expert, then by flat index t * k + slot (a stable counting
// sort), which is the order in which a per-expert loop meets its rows. Three
// passes over chunks of kRouteChunk entries, each deterministic (no order
// depends on atomics): per-chunk histograms; one workgroup turns them into
// sizes, expert bases and each chunk's first row per expert; each entry's row is
// its chunk's first row for its expert plus the number of earlier entries of the
// chunk with the same expert. The activation gather copies token rows with
// 16-byte accesses; the combine sums k fp32 products per output in slot order.
#include <algorithm>

#include "geg_device.hpp"
#include "geg_launch.hpp"

namespace geg {

namespace {

constexpr int kRouteChunk = kThreads;   // one entry per thread

// Pass 1: histogram of one chunk (invalid ids are counted nowhere and flagged);
// src_of starts at -1 so that rows no valid entry lands on stay marked.
__global__ __launch_bounds__(kThreads) void route_count_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                               int32_t E, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ src_of, uint32_t* err) {
  __shared__ int32_t hist[kMaxExperts];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t f = (int64_t)blockIdx.x * kRouteChunk + t;
  if (f < n) {
    src_of[f] = -1;
    const int32_t x = ids[f];
    if (x < 0 || x >= E)
      atomicOr(err, kErrBadExpertId);
    else
      atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  for (int e = t; e < E; e += kThreads) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Pass 2 (one workgroup): per expert, the running sum over chunks (each
// chunk's first rank), the expert's total (sizes[e]) and, after a prefix sum
// over experts, each chunk's first row per expert.
__global__ __launch_bounds__(kThreads) void route_scan_kernel(int32_t* __restrict__ counts, int64_t nchunks,
                                                              int32_t E, int32_t* __restrict__ sizes) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t base[kMaxExperts + 1];
  const int t = threadIdx.x;
  // chunks 16 at a time: their loads are all in flight before the running sum
  constexpr int B = 16;
  for (int e = t; e < E; e += kThreads) {
    int32_t run = 0;
    for (int64_t c0 = 0; c0 < nchunks; c0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = c0 + j < nchunks ? counts[(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j < nchunks) counts[(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
    tot[e] = run;
    sizes[e] = run;
  }
  __syncthreads();
  if (t < 64) {
    uint32_t carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const uint32_t v = e0 + t < E ? (uint32_t)tot[e0 + t] : 0u;
      const uint32_t incl = wave_scan_sat(v) + carry;
      if (e0 + t < E) base[e0 + t] = (int32_t)(incl - v);
      carry = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    }
  }
  __syncthreads();
  for (int e = t; e < E; e += kThreads) {
    const int32_t b = base[e];
    for (int64_t c0 = 0; c0 < nchunks; c0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = c0 + j < nchunks ? counts[(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j)
        if (c0 + j < nchunks) counts[(c0 + j) * E + e] = v[j] + b;
    }
  }
}

// Pass 3: each entry's row; row_of[f] = row (-1 for an invalid id) and
// src_of[row] = f.
__global__ __launch_bounds__(kThreads) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                 int32_t E, const int32_t* __restrict__ first,
                                                                 int32_t* __restrict__ row_of,
                                                                 int32_t* __restrict__ src_of) {
  __shared__ int32_t cid[kRouteChunk];
  const int t = threadIdx.x;
  const int64_t f = (int64_t)blockIdx.x * kRouteChunk + t;
  int32_t x = -1;
  if (f < n) {
    x = ids[f];
    if (x < 0 || x >= E) x = -1;
  }
  cid[t] = x;
  __syncthreads();
  if (f < n) {
    if (x < 0) {
      row_of[f] = -1;
    } else {
      int32_t rank = 0;
      for (int j = 0; j < t; ++j) rank += cid[j] == x;   // same j on every lane: one broadcast read
      const int32_t row = first[(int64_t)blockIdx.x * E + x] + rank;
      row_of[f] = row;
      src_of[row] = (int32_t)f;
    }
  }
}

// x_sorted[r] = x[src_of[r] / k]; rows with no source are left untouched.
__global__ __launch_bounds__(kThreads) void route_gather_kernel(const uint16_t* __restrict__ x, int64_t H, int32_t k,
                                                                const int32_t* __restrict__ src_of, int64_t n,
                                                                uint16_t* __restrict__ xs) {
  // four rows per pass, their loads all in flight before the stores
  constexpr int R = 4;
  const int64_t chunks = H >> 3;   // 16-byte pieces per row
  for (int64_t r0 = (int64_t)blockIdx.x * R; r0 < n; r0 += (int64_t)gridDim.x * R) {
    int32_t s[R];
#pragma unroll
    for (int u = 0; u < R; ++u) s[u] = r0 + u < n ? src_of[r0 + u] : -1;
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
      u32x4 v[R];
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (s[u] >= 0) v[u] = reinterpret_cast<const u32x4*>(x + (int64_t)(s[u] / k) * H)[c];
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (s[u] >= 0) reinterpret_cast<u32x4*>(xs + (r0 + u) * H)[c] = v[u];
    }
  }
}

// out[t, :] = bf16( sum over slots of w[t, slot] * y[row_of[t k + slot], :] ),
// fp32 products and sums in slot order; slots with no row are skipped.
__global__ __launch_bounds__(kThreads) void route_combine_kernel(const uint16_t* __restrict__ y, int64_t N,
                                                                 const int32_t* __restrict__ row_of,
                                                                 const float* __restrict__ w, int64_t T,
                                                                 int32_t k, uint16_t* __restrict__ out) {
  const int64_t chunks = N >> 3;
  for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x) {
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < k; ++s) {
        const int32_t r = row_of[tok * k + s];
        if (r < 0) continue;
        const float ws = w ? w[tok * k + s] : 1.0f;
        const u32x4 v = reinterpret_cast<const u32x4*>(y + (int64_t)r * N)[c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += ws * __builtin_bit_cast(float, v[i] << 16);
          acc[2 * i + 1] += ws * __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
        }
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      reinterpret_cast<u32x4*>(out + tok * N)[c] = o;
    }
  }
}

}  // namespace

hipError_t launch_route_sort(const int32_t* ids, int64_t n, int32_t E, int32_t* counts, int32_t* sizes,
                             int32_t* row_of, int32_t* src_of, uint32_t* err, hipStream_t s) {
  const int64_t nchunks = (n + kRouteChunk - 1) / kRouteChunk;
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)nchunks), dim3(kThreads), 0, s, ids, n, E, counts,
                       src_of, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kThreads), 0, s, counts, nchunks, E, sizes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)nchunks), dim3(kThreads), 0, s, ids, n, E, counts,
                     row_of, src_of);
  return hipGetLastError();
}

hipError_t launch_route_gather(const uint16_t* x, int64_t H, int32_t k, const int32_t* src_of, int64_t n,
                               uint16_t* xs, int cus, hipStream_t s) {
  const int64_t grid = std::min<int64_t>((n + 3) / 4, (int64_t)cus * 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(route_gather_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, x, H, k, src_of, n, xs);
  return hipGetLastError();
}

hipError_t launch_route_combine(const uint16_t* y, int64_t N, const int32_t* row_of, const float* w, int64_t T,
                                int32_t k, uint16_t* out, int cus, hipStream_t s) {
  const int64_t grid = std::min<int64_t>(T, (int64_t)cus * 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(route_combine_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, y, N, row_of, w, T, k, out);
  return hipGetLastError();
}

}  // namespace geg
