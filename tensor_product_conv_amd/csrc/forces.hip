// Force reduction and CSR checks (gfx950).
//
// Forces are the negative position gradient (FlashCart paper, section 2
// "Machine-learned interatomic potentials").  The edge vector r_e runs from
// the receiver to the sender image, so d r_e / d x_src = +I and
// d r_e / d x_recv = -I, and with g_e = dL/dr_e
//     F_k = -dL/dx_k = sum_{e in row k} (g_e - g_{rev(e)})
// because the edges whose sender is k are exactly the reverses of row k.  One
// thread per atom sums its row in CSR order: deterministic, no atomics.
#include "common.hpp"
#include "kernels.hpp"
#include "nbr.hpp"

namespace tpc {

namespace {

template <typename T>
__global__ void __launch_bounds__(256)
k_forces(int64_t n, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ rev,
         const T* __restrict__ g, T* __restrict__ F) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  T fx = T(0), fy = T(0), fz = T(0);
  for (int e = row_ptr[k]; e < row_ptr[k + 1]; ++e) {
    const int r = rev[e];
    fx += g[3 * e] - g[3 * r];
    fy += g[3 * e + 1] - g[3 * r + 1];
    fz += g[3 * e + 2] - g[3 * r + 2];
  }
  F[3 * k] = fx;
  F[3 * k + 1] = fy;
  F[3 * k + 2] = fz;
}

// One thread per row: monotone row pointers, senders in range, rows strictly
// increasing in (src, s1, s2, s3) (or non-decreasing in src when no shifts
// are given), and the chunk's edge range consistent.
__global__ void __launch_bounds__(256)
k_csr_check(int64_t n, int64_t n_edges, const int32_t* __restrict__ row_ptr,
            const int32_t* __restrict__ src, const int32_t* __restrict__ shift, int64_t row_begin,
            int64_t row_end, int64_t edge_begin, int64_t edge_end, int32_t* __restrict__ status) {
  const int64_t i = row_begin + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= row_end) return;
  int flags = 0;
  const int lo = row_ptr[i], hi = row_ptr[i + 1];
  if (hi < lo || lo < 0 || hi > n_edges) flags |= kFlagCsrOrder;
  if (i == row_begin && lo != edge_begin) flags |= kFlagCsrOrder;
  if (i == row_end - 1 && hi != edge_end) flags |= kFlagCsrOrder;
  if (!flags) {
    int64_t prev = -1;
    for (int e = lo; e < hi; ++e) {
      const int j = src[e];
      if (j < 0 || j >= n) {
        flags |= kFlagCsrRange;
        break;
      }
      if (!shift) {  // sender order only
        if (j < prev) {
          flags |= kFlagCsrOrder;
          break;
        }
        prev = j;
        continue;
      }
      const int s1 = shift[3 * e], s2 = shift[3 * e + 1], s3 = shift[3 * e + 2];
      if (s1 < -127 || s1 > 127 || s2 < -127 || s2 > 127 || s3 < -127 || s3 > 127) {
        flags |= kFlagShiftRange;
        break;
      }
      if (j == i && s1 == 0 && s2 == 0 && s3 == 0) {
        flags |= kFlagCsrRange;
        break;
      }
      const int64_t key = ((int64_t)j << 24) | ((int64_t)(s1 + 128) << 16) |
                          ((int64_t)(s2 + 128) << 8) | (int64_t)(s3 + 128);
      if (key <= prev) {
        flags |= kFlagCsrOrder;
        break;
      }
      prev = key;
    }
  }
  if (flags) atomicOr(status, flags);
}

}  // namespace

hipError_t launch_forces(int dtype, int64_t n, const int32_t* row_ptr, const int32_t* rev,
                         const void* g, void* forces, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dtype == 1)
    k_forces<double><<<blocks, 256, 0, s>>>(n, row_ptr, rev, static_cast<const double*>(g),
                                            static_cast<double*>(forces));
  else
    k_forces<float><<<blocks, 256, 0, s>>>(n, row_ptr, rev, static_cast<const float*>(g),
                                           static_cast<float*>(forces));
  return hipGetLastError();
}

hipError_t launch_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const int32_t* shift, int64_t row_begin,
                            int64_t row_end, int64_t edge_begin, int64_t edge_end,
                            int32_t* status, hipStream_t s) {
  const int64_t rows = row_end - row_begin;
  if (rows <= 0) return hipSuccess;
  k_csr_check<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(
      n, n_edges, row_ptr, src, shift, row_begin, row_end, edge_begin, edge_end, status);
  return hipGetLastError();
}

}  // namespace tpc
