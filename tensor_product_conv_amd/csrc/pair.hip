// Shared radial rows of an edge and its reverse.
//
// The radial weights depend on the edge length only (FlashCart section 2,
// the distance-dependent weights of each path; FastMACE page "Rewrites and
// precision options", section "Radial network").  The reverse of edge
// (i <- j, S) is (j <- i, -S), whose vector is the exact negation of the
// first in float64, so both have the same length bit for bit and the same
// row of R.  Within one chunk of edges [edge_begin, edge_begin + ne), each
// pair whose two edges both lie in the chunk keeps one row; an edge whose
// reverse lies outside the chunk keeps its own.
//
// The map Rrow [ne + 1] (chunk-relative) is built in three steps:
//   1. Rrow[k] = 1 for an owner (its reverse is outside the chunk, or has a
//      larger index), else 0;
//   2. an exclusive prefix sum in place: an owner's entry becomes its row,
//      Rrow[ne] the number of rows;
//   3. every other edge takes its owner's row, and each owner's basis
//      values are copied to that row of a compacted ef for the radial
//      network.
// Owners keep chunk order, so the rows are deterministic.
#include "common.hpp"
#include "kernels.hpp"
#include "nbr.hpp"

namespace tpc {

namespace {

__global__ void __launch_bounds__(256) k_pair_owner(const int32_t* __restrict__ rev, int64_t edge_begin,
                                                    int64_t ne, int32_t* __restrict__ rrow) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= ne) return;
  const int64_t r = (int64_t)rev[edge_begin + k] - edge_begin;
  rrow[k] = (r < 0 || r >= ne || k < r) ? 1 : 0;
}

template <typename T>
__global__ void __launch_bounds__(256) k_pair_fill(const int32_t* __restrict__ rev, int64_t edge_begin,
                                                   int64_t ne, int32_t* __restrict__ rrow,
                                                   const T* __restrict__ ef, T* __restrict__ ef_rows) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= ne) return;
  const int64_t r = (int64_t)rev[edge_begin + k] - edge_begin;
  if (r < 0 || r >= ne || k < r) {
    // an owner: its entry already holds its row, and no other thread writes it
    if (ef_rows) {
      const int64_t row = rrow[k];
#pragma unroll
      for (int q = 0; q < 8; ++q) ef_rows[row * 8 + q] = ef[k * 8 + q];
    }
  } else {
    // the owner r < k is not written by this kernel
    rrow[k] = rrow[r];
  }
}

}  // namespace

int64_t pair_partials_len(int64_t ne) { return scan_partials_len(ne); }

hipError_t launch_pair_rows(int dtype, const int32_t* rev, int64_t edge_begin, int64_t ne, int32_t* rrow,
                            int32_t* partials, const void* ef, void* ef_rows, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((ne + 255) / 256);
  k_pair_owner<<<blocks, 256, 0, s>>>(rev, edge_begin, ne, rrow);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scan_exclusive(rrow, ne, partials, s);
  if (e != hipSuccess) return e;
  if (dtype == 1)
    k_pair_fill<double><<<blocks, 256, 0, s>>>(rev, edge_begin, ne, rrow, static_cast<const double*>(ef),
                                               static_cast<double*>(ef_rows));
  else
    k_pair_fill<float><<<blocks, 256, 0, s>>>(rev, edge_begin, ne, rrow, static_cast<const float*>(ef),
                                              static_cast<float*>(ef_rows));
  return hipGetLastError();
}

}  // namespace tpc
