// Device-wide exclusive prefix sum of int32 counts, in place: data[0..n) holds
// counts on entry and their exclusive prefix sums on exit; data[n] receives the
// total.  Three launches: per-tile sums, a one-block scan of the tile sums
// (kept in int64 so an int32 overflow of the total is visible to the host),
// then per-tile scans with the tile offset.  Deterministic.
#include "common.hpp"
#include "nbr.hpp"

namespace tpc {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kTile = kThreads * kItems;

template <typename V>
__device__ V block_exclusive_scan(V v, V* total) {
  __shared__ V warp_sums[kThreads / 64];
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
  V x = v;
  for (int o = 1; o < 64; o <<= 1) {
    V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) warp_sums[w] = x;
  __syncthreads();
  V off = 0, tot = 0;
  for (int k = 0; k < kThreads / 64; ++k) {
    if (k < w) off += warp_sums[k];
    tot += warp_sums[k];
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

__global__ void __launch_bounds__(kThreads) k_tile_sums(const int32_t* __restrict__ d, int64_t n,
                                                        int64_t* __restrict__ part) {
  const int64_t base = blockIdx.x * (int64_t)kTile + threadIdx.x * (int64_t)kItems;
  int64_t s = 0;
  for (int k = 0; k < kItems; ++k)
    if (base + k < n) s += d[base + k];
  int64_t tot;
  block_exclusive_scan<int64_t>(s, &tot);
  if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(kThreads) k_scan_parts(int64_t* __restrict__ part, int64_t nt,
                                                         int32_t* __restrict__ d, int64_t n) {
  // nt <= kTile is guaranteed by the host
  const int64_t base = threadIdx.x * (int64_t)kItems;
  int64_t v[kItems];
  int64_t s = 0;
  for (int k = 0; k < kItems; ++k) {
    v[k] = (base + k < nt) ? part[base + k] : 0;
    s += v[k];
  }
  int64_t tot;
  int64_t off = block_exclusive_scan<int64_t>(s, &tot);
  for (int k = 0; k < kItems; ++k) {
    if (base + k < nt) part[base + k] = off;
    off += v[k];
  }
  if (threadIdx.x == 0) {
    part[nt] = tot;
    d[n] = tot > 2147483647LL ? -1 : (int32_t)tot;
  }
}

__global__ void __launch_bounds__(kThreads) k_tile_scan(int32_t* __restrict__ d, int64_t n,
                                                        const int64_t* __restrict__ part) {
  const int64_t base = blockIdx.x * (int64_t)kTile + threadIdx.x * (int64_t)kItems;
  int32_t v[kItems];
  int64_t s = 0;
  for (int k = 0; k < kItems; ++k) {
    v[k] = (base + k < n) ? d[base + k] : 0;
    s += v[k];
  }
  int64_t tot;
  int64_t off = block_exclusive_scan<int64_t>(s, &tot) + part[blockIdx.x];
  for (int k = 0; k < kItems; ++k) {
    if (base + k < n) d[base + k] = (int32_t)off;
    off += v[k];
  }
}

}  // namespace

int64_t scan_partials_len(int64_t n) { return (n + kTile - 1) / kTile + 1; }

hipError_t launch_scan_exclusive(int32_t* data, int64_t n, int32_t* partials, hipStream_t s) {
  int64_t* part = reinterpret_cast<int64_t*>(partials);
  const int64_t nt = (n + kTile - 1) / kTile;
  if (nt > kTile) return hipErrorInvalidValue;
  if (nt > 0) k_tile_sums<<<(unsigned)nt, kThreads, 0, s>>>(data, n, part);
  k_scan_parts<<<1, kThreads, 0, s>>>(part, nt, data, n);
  if (nt > 0) k_tile_scan<<<(unsigned)nt, kThreads, 0, s>>>(data, n, part);
  return hipGetLastError();
}

}  // namespace tpc
