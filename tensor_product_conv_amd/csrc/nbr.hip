// Periodic cell-list neighbour build emitting receiver-sorted CSR (gfx950).
//
// Definition (FlashCart paper, section 2 "Equivariant convolution and
// many-body correlations"): a receiver's neighbourhood is every atom and
// periodic image within r_cut except the receiver itself in the reference
// cell.  Storage (section 4 "Data layout"): edges in receiver order, a row
// pointer array and a sender array.  An edge is keyed by (receiver, sender,
// image shift), the edge identity of the Frost model card.
//
// The edge test is evaluated in float64 with this file compiled without
// floating-point contraction, in the fixed order
//     r = (x_j - x_i) + ((s1*a1 + s2*a2) + s3*a3)
//     d2 = (r_x*r_x + r_y*r_y) + r_z*r_z ;  edge iff d2 < r_cut*r_cut
// so the decision is bitwise reproducible and symmetric: the reverse edge
// (j <- i, -S) evaluates to exactly -r.
//
// Pipeline (all on the caller's stream, one wait for the edge count):
//   bin      fractional coordinates -> bin id, bin counts
//   scan     bin counts -> bin starts;  scatter atoms into bins
//   count    one wave per receiver: stencil bins x bin atoms -> degree
//   scan     degrees -> row_ptr;  read back E
//   fill     one wave per receiver: accepted (src, shift) keys into LDS, each
//            key placed at its rank in the row (rows sorted by key)
//   reverse  one wave per receiver: binary search of (i, -S) in row j
#include "common.hpp"
#include "nbr.hpp"

namespace tpc {

namespace {

constexpr int kWave = 64;
constexpr int kNbrWavesPerBlock = 4;

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_bin(int64_t n, const double* __restrict__ pos, NbrGrid g,
                      const int32_t* __restrict__ species, int n_species,
                      int32_t* __restrict__ bin_of, int32_t* __restrict__ bin_count,
                      int32_t* __restrict__ status) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double x = pos[3 * i], y = pos[3 * i + 1], z = pos[3 * i + 2];
  int flags = 0;
  int c[3];
  for (int k = 0; k < 3; ++k) {
    double f = (x * g.inv[0][k] + y * g.inv[1][k]) + z * g.inv[2][k];
    if (!(f >= -1e-10 && f < 1.0 + 1e-10)) flags |= kFlagUnwrapped;
    f = f < 0.0 ? 0.0 : f;
    int b = (int)floor(f * (double)g.nb[k]);
    b = b < 0 ? 0 : (b >= g.nb[k] ? g.nb[k] - 1 : b);
    c[k] = b;
  }
  if (species) {
    int s = species[i];
    if (s < 0 || s >= n_species) flags |= kFlagSpecies;
  }
  if (flags) atomicOr(status, flags);
  const int flat = (c[0] * g.nb[1] + c[1]) * g.nb[2] + c[2];
  bin_of[i] = flat;
  atomicAdd(&bin_count[flat], 1);
}

// Wrapped positions: every fractional coordinate in [0, 1) (the same test
// and tolerance as the binning above), for the checks of the convolution
// calls.
__global__ void k_wrap_check(int64_t n, const double* __restrict__ pos, NbrGrid g,
                             int32_t* __restrict__ status) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double x = pos[3 * i], y = pos[3 * i + 1], z = pos[3 * i + 2];
  int flags = 0;
  for (int k = 0; k < 3; ++k) {
    const double f = (x * g.inv[0][k] + y * g.inv[1][k]) + z * g.inv[2][k];
    if (!(f >= -1e-10 && f < 1.0 + 1e-10)) flags |= kFlagUnwrapped;
  }
  if (flags) atomicOr(status, flags);
}

__global__ void k_scatter(int64_t n, const int32_t* __restrict__ bin_of,
                          const int32_t* __restrict__ bin_start, int32_t* __restrict__ cursor,
                          int32_t* __restrict__ bin_atoms) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int b = bin_of[i];
  const int slot = atomicAdd(&cursor[b], 1);
  bin_atoms[bin_start[b] + slot] = (int32_t)i;
}

// Visit every candidate (j, S) of receiver i: calls f(j, s1, s2, s3, accepted)
// once per candidate, lanes in parallel over the atoms of each stencil bin.
template <typename F>
__device__ __forceinline__ void for_candidates(int i, const double* __restrict__ pos,
                                               const NbrGrid& g, const int32_t* __restrict__ bin_of,
                                               const int32_t* __restrict__ bin_start,
                                               const int32_t* __restrict__ bin_atoms, F&& f) {
  const int lane = threadIdx.x % kWave;
  const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
  const int bi = bin_of[i];
  const int c2 = bi % g.nb[2];
  const int c1 = (bi / g.nb[2]) % g.nb[1];
  const int c0 = bi / (g.nb[2] * g.nb[1]);
  for (int d0 = -g.K[0]; d0 <= g.K[0]; ++d0) {
    const int t0 = c0 + d0;
    const int s0 = (t0 >= 0 ? t0 / g.nb[0] : -((-t0 + g.nb[0] - 1) / g.nb[0]));
    const int b0 = t0 - s0 * g.nb[0];
    for (int d1 = -g.K[1]; d1 <= g.K[1]; ++d1) {
      const int t1 = c1 + d1;
      const int s1 = (t1 >= 0 ? t1 / g.nb[1] : -((-t1 + g.nb[1] - 1) / g.nb[1]));
      const int b1 = t1 - s1 * g.nb[1];
      for (int d2 = -g.K[2]; d2 <= g.K[2]; ++d2) {
        const int t2 = c2 + d2;
        const int s2 = (t2 >= 0 ? t2 / g.nb[2] : -((-t2 + g.nb[2] - 1) / g.nb[2]));
        const int b2 = t2 - s2 * g.nb[2];
        const int b = (b0 * g.nb[1] + b1) * g.nb[2] + b2;
        const int lo = bin_start[b], hi = bin_start[b + 1];
        const double S1 = (double)s0, S2 = (double)s1, S3 = (double)s2;
        const double ox = (S1 * g.a[0][0] + S2 * g.a[1][0]) + S3 * g.a[2][0];
        const double oy = (S1 * g.a[0][1] + S2 * g.a[1][1]) + S3 * g.a[2][1];
        const double oz = (S1 * g.a[0][2] + S2 * g.a[1][2]) + S3 * g.a[2][2];
        const bool zero_shift = (s0 == 0) && (s1 == 0) && (s2 == 0);
        for (int base = lo; base < hi; base += kWave) {
          const int t = base + lane;
          bool ok = false;
          int j = -1;
          if (t < hi) {
            j = bin_atoms[t];
            const double rx = (pos[3 * j] - xi) + ox;
            const double ry = (pos[3 * j + 1] - yi) + oy;
            const double rz = (pos[3 * j + 2] - zi) + oz;
            const double d2 = (rx * rx + ry * ry) + rz * rz;
            ok = (d2 < g.rc2) && !(zero_shift && j == i);
          }
          f(j, s0, s1, s2, ok, t < hi);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(kWave * kNbrWavesPerBlock)
k_count(int64_t n, const double* __restrict__ pos, NbrGrid g, const int32_t* __restrict__ bin_of,
        const int32_t* __restrict__ bin_start, const int32_t* __restrict__ bin_atoms,
        int32_t* __restrict__ deg, int32_t* __restrict__ status) {
  const int64_t iw = blockIdx.x * (int64_t)kNbrWavesPerBlock + threadIdx.x / kWave;
  if (iw >= n) return;
  const int i = uniform((int)iw);
  int cnt = 0;
  for_candidates(i, pos, g, bin_of, bin_start, bin_atoms,
                 [&](int, int, int, int, bool ok, bool) {
                   cnt += __popcll(__ballot(ok));
                 });
  if (threadIdx.x % kWave == 0) {
    deg[i] = cnt;
    if (cnt > kMaxDegree) atomicOr(status, kFlagDegree);
  }
}

__device__ __forceinline__ uint64_t edge_key(int j, int s1, int s2, int s3) {
  return ((uint64_t)(uint32_t)j << 24) | ((uint64_t)(uint32_t)(s1 + 128) << 16) |
         ((uint64_t)(uint32_t)(s2 + 128) << 8) | (uint64_t)(uint32_t)(s3 + 128);
}

__global__ void __launch_bounds__(kWave * kNbrWavesPerBlock)
k_fill(int64_t n, const double* __restrict__ pos, NbrGrid g, const int32_t* __restrict__ bin_of,
       const int32_t* __restrict__ bin_start, const int32_t* __restrict__ bin_atoms,
       const int32_t* __restrict__ row_ptr, int32_t* __restrict__ src, int32_t* __restrict__ shift) {
  __shared__ uint64_t keys[kNbrWavesPerBlock][kMaxDegree];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t iw = blockIdx.x * (int64_t)kNbrWavesPerBlock + w;
  if (iw >= n) return;
  const int i = uniform((int)iw);
  uint64_t* K = keys[w];
  int cnt = 0;
  for_candidates(i, pos, g, bin_of, bin_start, bin_atoms,
                 [&](int j, int s1, int s2, int s3, bool ok, bool) {
                   const uint64_t m = __ballot(ok);
                   const int before = __popcll(m & ((1ull << lane) - 1ull));
                   if (ok) K[cnt + before] = edge_key(j, s1, s2, s3);
                   cnt += __popcll(m);
                 });
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int base = row_ptr[i];
  for (int t = lane; t < cnt; t += kWave) {
    const uint64_t k = K[t];
    int rank = 0;
    for (int u = 0; u < cnt; ++u) rank += (K[u] < k);
    const int e = base + rank;
    src[e] = (int32_t)(k >> 24);
    shift[3 * e] = (int32_t)((k >> 16) & 0xff) - 128;
    shift[3 * e + 1] = (int32_t)((k >> 8) & 0xff) - 128;
    shift[3 * e + 2] = (int32_t)(k & 0xff) - 128;
  }
}

__global__ void __launch_bounds__(256)
k_reverse(int64_t n, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
          const int32_t* __restrict__ shift, int32_t* __restrict__ rev, int32_t* __restrict__ status) {
  const int64_t iw = blockIdx.x * (int64_t)(256 / kWave) + threadIdx.x / kWave;
  if (iw >= n) return;
  const int i = uniform((int)iw);
  const int lane = threadIdx.x % kWave;
  const int lo = row_ptr[i], hi = row_ptr[i + 1];
  for (int e = lo + lane; e < hi; e += kWave) {
    const int j = src[e];
    const uint64_t want = edge_key(i, -shift[3 * e], -shift[3 * e + 1], -shift[3 * e + 2]);
    int a = row_ptr[j], b = row_ptr[j + 1];   // search [a, b)
    while (a < b) {
      const int mid = (a + b) >> 1;
      const uint64_t km = edge_key(src[mid], shift[3 * mid], shift[3 * mid + 1], shift[3 * mid + 2]);
      if (km < want) a = mid + 1; else b = mid;
    }
    int r = -1;
    if (a < row_ptr[j + 1]) {
      const uint64_t ka = edge_key(src[a], shift[3 * a], shift[3 * a + 1], shift[3 * a + 2]);
      if (ka == want) r = a;
    }
    if (r < 0) atomicOr(status, kFlagNoReverse);
    rev[e] = r;
  }
}

}  // namespace

hipError_t launch_wrap_check(int64_t n, const double* pos, const NbrGrid& g, int32_t* status,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_wrap_check<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, pos, g, status);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill_i32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_nbr_bin(int64_t n, const double* pos, const NbrGrid& g, const int32_t* species,
                          int n_species, int32_t* bin_of, int32_t* bin_count, int32_t* status,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_bin<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, pos, g, species, n_species, bin_of,
                                                   bin_count, status);
  return hipGetLastError();
}

hipError_t launch_nbr_scatter(int64_t n, const int32_t* bin_of, const int32_t* bin_start,
                              int32_t* cursor, int32_t* bin_atoms, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_scatter<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, bin_of, bin_start, cursor, bin_atoms);
  return hipGetLastError();
}

hipError_t launch_nbr_count(int64_t n, const double* pos, const NbrGrid& g, const int32_t* bin_of,
                            const int32_t* bin_start, const int32_t* bin_atoms, int32_t* deg,
                            int32_t* status, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + kNbrWavesPerBlock - 1) / kNbrWavesPerBlock);
  k_count<<<blocks, kWave * kNbrWavesPerBlock, 0, s>>>(n, pos, g, bin_of, bin_start, bin_atoms,
                                                       deg, status);
  return hipGetLastError();
}

hipError_t launch_nbr_fill(int64_t n, const double* pos, const NbrGrid& g, const int32_t* bin_of,
                           const int32_t* bin_start, const int32_t* bin_atoms,
                           const int32_t* row_ptr, int32_t* src, int32_t* shift, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + kNbrWavesPerBlock - 1) / kNbrWavesPerBlock);
  k_fill<<<blocks, kWave * kNbrWavesPerBlock, 0, s>>>(n, pos, g, bin_of, bin_start, bin_atoms,
                                                      row_ptr, src, shift);
  return hipGetLastError();
}

hipError_t launch_nbr_reverse(int64_t n, const int32_t* row_ptr, const int32_t* src,
                              const int32_t* shift, int32_t* rev, int32_t* status, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 3) / 4);
  k_reverse<<<blocks, 256, 0, s>>>(n, row_ptr, src, shift, rev, status);
  return hipGetLastError();
}

}  // namespace tpc
