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
// are given), and the chunk's edge range consistent.  With a reverse index,
// every edge e = (i <- j) of the row must name an edge r = rev[e] of row j
// whose sender is i and whose reverse is e (and, with shifts, whose shift is
// the negated one): the list is symmetric.
__global__ void __launch_bounds__(256)
k_csr_check(int64_t n, int64_t n_edges, const int32_t* __restrict__ row_ptr,
            const int32_t* __restrict__ src, const int32_t* __restrict__ shift,
            const int32_t* __restrict__ rev, int64_t row_begin, int64_t row_end,
            int64_t edge_begin, int64_t edge_end, int32_t* __restrict__ status) {
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
  if (!flags && rev) {
    for (int e = lo; e < hi; ++e) {
      const int r = rev[e];
      const int j = src[e];
      if (r < 0 || r >= n_edges || r < row_ptr[j] || r >= row_ptr[j + 1] || src[r] != i || rev[r] != e ||
          (shift && (shift[3 * r] != -shift[3 * e] || shift[3 * r + 1] != -shift[3 * e + 1] ||
                     shift[3 * r + 2] != -shift[3 * e + 2]))) {
        flags |= kFlagNoReverse;
        break;
      }
    }
  }
  if (flags) atomicOr(status, flags);
}

// Virial W[a][b] = dL/d(eps_ab) for the strain x -> (I + eps) x of the
// positions and the cell rows (the pet-jax README, "Conventions": the virial
// is the strain derivative of the energy).  With the list fixed every edge
// vector becomes (I + eps) r_e, so W[a][b] = sum_e g_e[a] r_e[b].  r_e is
// formed in float64 exactly as the neighbour build forms it.  One thread per
// row sums its edges in CSR order in float64; each block folds its rows' sums
// with a fixed tree in LDS into one partial; one block then folds the
// partials the same way.  Deterministic, no atomics.
template <typename T>
__global__ void __launch_bounds__(kVirialBlock)
k_virial_rows(int64_t n, GeomArgs a, const T* __restrict__ g, double* __restrict__ part) {
  __shared__ double sm[9][kVirialBlock];
  const int t = threadIdx.x;
  const int64_t i = blockIdx.x * (int64_t)kVirialBlock + t;
  double w[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) w[c] = 0.0;
  if (i < n) {
    for (int e = a.row_ptr[i]; e < a.row_ptr[i + 1]; ++e) {
#pragma clang fp contract(off)
      const int j = a.src[e];
      const double S1 = (double)a.shift[3 * e], S2 = (double)a.shift[3 * e + 1],
                   S3 = (double)a.shift[3 * e + 2];
      double r[3];
#pragma unroll
      for (int k = 0; k < 3; ++k)
        r[k] = (a.pos[3 * j + k] - a.pos[3 * i + k]) +
               ((S1 * a.cell[0][k] + S2 * a.cell[1][k]) + S3 * a.cell[2][k]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const double gp = (double)g[3 * (int64_t)e + p];
#pragma unroll
        for (int q = 0; q < 3; ++q) w[3 * p + q] += gp * r[q];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 9; ++c) sm[c][t] = w[c];
  __syncthreads();
  for (int h = kVirialBlock / 2; h > 0; h >>= 1) {
    if (t < h) {
#pragma unroll
      for (int c = 0; c < 9; ++c) sm[c][t] += sm[c][t + h];
    }
    __syncthreads();
  }
  if (t < 9) part[blockIdx.x * (int64_t)9 + t] = sm[t][0];
}

template <typename T>
__global__ void __launch_bounds__(kVirialBlock)
k_virial_sum(int64_t nblk, const double* __restrict__ part, T* __restrict__ W) {
  __shared__ double sm[9][kVirialBlock];
  const int t = threadIdx.x;
  double w[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) w[c] = 0.0;
  for (int64_t b = t; b < nblk; b += kVirialBlock) {
#pragma unroll
    for (int c = 0; c < 9; ++c) w[c] += part[b * 9 + c];
  }
#pragma unroll
  for (int c = 0; c < 9; ++c) sm[c][t] = w[c];
  __syncthreads();
  for (int h = kVirialBlock / 2; h > 0; h >>= 1) {
    if (t < h) {
#pragma unroll
      for (int c = 0; c < 9; ++c) sm[c][t] += sm[c][t + h];
    }
    __syncthreads();
  }
  if (t < 9) W[t] = (T)sm[t][0];
}

}  // namespace

hipError_t launch_virial(int dtype, int64_t n, const GeomArgs& a, const void* g, double* part,
                         void* W, hipStream_t s) {
  const int64_t nblk = virial_blocks(n);
  if (dtype == 1) {
    if (nblk > 0)
      k_virial_rows<double><<<(unsigned)nblk, kVirialBlock, 0, s>>>(n, a, static_cast<const double*>(g), part);
    k_virial_sum<double><<<1, kVirialBlock, 0, s>>>(nblk, part, static_cast<double*>(W));
  } else {
    if (nblk > 0)
      k_virial_rows<float><<<(unsigned)nblk, kVirialBlock, 0, s>>>(n, a, static_cast<const float*>(g), part);
    k_virial_sum<float><<<1, kVirialBlock, 0, s>>>(nblk, part, static_cast<float*>(W));
  }
  return hipGetLastError();
}

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

template <typename T>
__global__ void __launch_bounds__(256)
k_part_sum(int n_parts, int64_t n, const T* __restrict__ in, T* __restrict__ out) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= n) return;
  T acc = in[t];
  for (int q = 1; q < n_parts; ++q) acc += in[q * n + t];
  out[t] = acc;
}

hipError_t launch_part_sum(int dtype, int n_parts, int64_t ne, int width, const void* in, void* out,
                           hipStream_t s) {
  const int64_t n = ne * width;
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dtype == 1)
    k_part_sum<double><<<blocks, 256, 0, s>>>(n_parts, n, static_cast<const double*>(in), static_cast<double*>(out));
  else
    k_part_sum<float><<<blocks, 256, 0, s>>>(n_parts, n, static_cast<const float*>(in), static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const int32_t* shift, const int32_t* rev,
                            int64_t row_begin, int64_t row_end, int64_t edge_begin,
                            int64_t edge_end, int32_t* status, hipStream_t s) {
  const int64_t rows = row_end - row_begin;
  if (rows <= 0) return hipSuccess;
  k_csr_check<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(
      n, n_edges, row_ptr, src, shift, rev, row_begin, row_end, edge_begin, edge_end, status);
  return hipGetLastError();
}

}  // namespace tpc
