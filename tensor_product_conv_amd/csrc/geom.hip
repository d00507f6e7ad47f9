// Edge geometry (gfx950): edge vector, length, real harmonics of the
// direction, Bessel basis times polynomial envelope; and the backward that
// turns dL/dY and dL/d(ef) into dL/d(edge vector).
//
// Edge vector (FlashCart paper, section 2 "Equivariant convolution and
// many-body correlations"): r_e points from the receiver to the sender image,
// r = (x_j - x_i) + ((s1*a1 + s2*a2) + s3*a3) in float64, then rounded to T.
// The reverse edge gives exactly -r, so the pair shares R and has harmonics
// differing by (-1)^l.
//
// Harmonics: component-normalised real harmonics (sum_m Y_lm^2 = 2l+1, z polar,
// no Condon-Shortley phase), as Cartesian polynomials of the unit vector.
// Radial basis: b_n(r) = sqrt(2/r_c) sin(n pi r/r_c)/r, n = 1..8, times the
// p = 5 envelope u(x) = 1 - 21 x^5 + 35 x^6 - 15 x^7, x = r/r_c, evaluated as
// (1-x)^3 (1 + 3x + 6x^2 + 10x^3 + 15x^4): the same polynomial, whose triple
// zero at the cutoff this form keeps to full relative accuracy (the expanded
// terms cancel there to a value far below their rounding).
//
// One thread per edge; stores are row-contiguous per edge so the fused
// tensor-product kernels read an edge's harmonics as one scalar block.
#include "common.hpp"
#include "kernels.hpp"

namespace tpc {

namespace {

template <typename T>
__device__ __forceinline__ T sqrt_t(T x);
template <>
__device__ __forceinline__ float sqrt_t<float>(float x) { return sqrtf(x); }
template <>
__device__ __forceinline__ double sqrt_t<double>(double x) { return sqrt(x); }

template <typename T>
__device__ __forceinline__ void sincos_t(T x, T* s, T* c);
template <>
__device__ __forceinline__ void sincos_t<float>(float x, float* s, float* c) { sincosf(x, s, c); }
template <>
__device__ __forceinline__ void sincos_t<double>(double x, double* s, double* c) { sincos(x, s, c); }

// Y_lm(u) for l <= L2, u a unit vector, index l*l + m + l.
template <typename T, int L2>
__device__ __forceinline__ void harmonics(T x, T y, T z, T* Y) {
  Y[0] = T(1);
  if constexpr (L2 >= 1) {
    const T s3 = T(1.7320508075688772935);
    Y[1] = s3 * y;
    Y[2] = s3 * z;
    Y[3] = s3 * x;
  }
  if constexpr (L2 >= 2) {
    const T s15 = T(3.8729833462074168852), s5h = T(1.1180339887498948482);
    Y[4] = s15 * x * y;
    Y[5] = s15 * y * z;
    Y[6] = s5h * (T(3) * z * z - T(1));
    Y[7] = s15 * x * z;
    Y[8] = T(0.5) * s15 * (x * x - y * y);
  }
  if constexpr (L2 >= 3) {
    const T c358 = T(2.0916500663351888), c105 = T(10.246950765959598),
            c218 = T(1.6201851746019651), c7h = T(1.3228756555322953);
    Y[9] = c358 * y * (T(3) * x * x - y * y);
    Y[10] = c105 * x * y * z;
    Y[11] = c218 * y * (T(5) * z * z - T(1));
    Y[12] = c7h * z * (T(5) * z * z - T(3));
    Y[13] = c218 * x * (T(5) * z * z - T(1));
    Y[14] = T(0.5) * c105 * z * (x * x - y * y);
    Y[15] = c358 * x * (x * x - T(3) * y * y);
  }
}

// q = sum_lm w_lm grad P_lm(u), with P_lm the polynomials used in harmonics().
template <typename T, int L2>
__device__ __forceinline__ void harmonics_grad_dot(T x, T y, T z, const T* w, T* q) {
  T gx = T(0), gy = T(0), gz = T(0);
  if constexpr (L2 >= 1) {
    const T s3 = T(1.7320508075688772935);
    gy += s3 * w[1];
    gz += s3 * w[2];
    gx += s3 * w[3];
  }
  if constexpr (L2 >= 2) {
    const T s15 = T(3.8729833462074168852), s5h = T(1.1180339887498948482);
    gx += s15 * y * w[4];
    gy += s15 * x * w[4];
    gy += s15 * z * w[5];
    gz += s15 * y * w[5];
    gz += s5h * T(6) * z * w[6];
    gx += s15 * z * w[7];
    gz += s15 * x * w[7];
    gx += s15 * x * w[8];
    gy -= s15 * y * w[8];
  }
  if constexpr (L2 >= 3) {
    const T c358 = T(2.0916500663351888), c105 = T(10.246950765959598),
            c218 = T(1.6201851746019651), c7h = T(1.3228756555322953);
    gx += c358 * T(6) * x * y * w[9];
    gy += c358 * T(3) * (x * x - y * y) * w[9];
    gx += c105 * y * z * w[10];
    gy += c105 * x * z * w[10];
    gz += c105 * x * y * w[10];
    gy += c218 * (T(5) * z * z - T(1)) * w[11];
    gz += c218 * T(10) * y * z * w[11];
    gz += c7h * (T(15) * z * z - T(3)) * w[12];
    gx += c218 * (T(5) * z * z - T(1)) * w[13];
    gz += c218 * T(10) * x * z * w[13];
    gx += c105 * x * z * w[14];
    gy -= c105 * y * z * w[14];
    gz += T(0.5) * c105 * (x * x - y * y) * w[14];
    gx += c358 * T(3) * (x * x - y * y) * w[15];
    gy -= c358 * T(6) * x * y * w[15];
  }
  q[0] = gx;
  q[1] = gy;
  q[2] = gz;
}

__device__ __forceinline__ int row_of(const int32_t* __restrict__ row_ptr, int lo, int hi, int e) {
  // largest i in [lo, hi) with row_ptr[i] <= e
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_ptr[mid] <= e) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T, int L2>
__global__ void __launch_bounds__(256)
k_geom_fwd(GeomArgs a, T* __restrict__ Y, T* __restrict__ ef, T* __restrict__ rv) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t ne = a.edge_end - a.edge_begin;
  if (t >= ne) return;
  const int e = (int)(a.edge_begin + t);
  const int i = row_of(a.row_ptr, (int)a.row_begin, (int)a.row_end, e);
  const int j = a.src[e];
  const double S1 = (double)a.shift[3 * e], S2 = (double)a.shift[3 * e + 1],
               S3 = (double)a.shift[3 * e + 2];
  double r64[3];
  for (int k = 0; k < 3; ++k)
    r64[k] = (a.pos[3 * j + k] - a.pos[3 * i + k]) +
             ((S1 * a.cell[0][k] + S2 * a.cell[1][k]) + S3 * a.cell[2][k]);
  const T x = (T)r64[0], y = (T)r64[1], z = (T)r64[2];
  const T r = sqrt_t<T>(x * x + y * y + z * z);
  const T ir = T(1) / r;
  constexpr int DSH = (L2 + 1) * (L2 + 1);
  T Yv[DSH];
  harmonics<T, L2>(x * ir, y * ir, z * ir, Yv);
#pragma unroll
  for (int k = 0; k < DSH; ++k) Y[t * DSH + k] = Yv[k];
  const T rc = (T)a.r_cut;
  const T xr = r / rc;
  const T omx = T(1) - xr;
  const T env = omx * omx * omx * (T(1) + xr * (T(3) + xr * (T(6) + xr * (T(10) + T(15) * xr))));
  T s1, c1;
  sincos_t<T>(T(3.14159265358979323846) * xr, &s1, &c1);
  const T pre = sqrt_t<T>(T(2) / rc) * ir * env;
  T sp = T(0), sn = s1;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    ef[t * 8 + n] = pre * sn;
    const T nx = T(2) * c1 * sn - sp;
    sp = sn;
    sn = nx;
  }
  rv[t * 4 + 0] = x;
  rv[t * 4 + 1] = y;
  rv[t * 4 + 2] = z;
  rv[t * 4 + 3] = r;
}

template <typename T, int L2>
__global__ void __launch_bounds__(256)
k_geom_bwd(int64_t ne, int64_t edge_begin, double r_cut, const T* __restrict__ rv,
           const T* __restrict__ dY, int n_parts, const T* __restrict__ d_ef, const T* __restrict__ d_r,
           T* __restrict__ g) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= ne) return;
  constexpr int DSH = (L2 + 1) * (L2 + 1);
  const T x = rv[t * 4], y = rv[t * 4 + 1], z = rv[t * 4 + 2], r = rv[t * 4 + 3];
  const T ir = T(1) / r;
  const T ux = x * ir, uy = y * ir, uz = z * ir;
  T w[DSH];
#pragma unroll
  for (int k = 0; k < DSH; ++k) w[k] = dY[t * DSH + k];
  for (int part = 1; part < n_parts; ++part)
#pragma unroll
    for (int k = 0; k < DSH; ++k) w[k] += dY[(part * ne + t) * DSH + k];
  T q[3];
  harmonics_grad_dot<T, L2>(ux, uy, uz, w, q);
  const T uq = ux * q[0] + uy * q[1] + uz * q[2];
  // radial part: sum_n d_ef_n * d(ef_n)/dr, or dL/dr given directly
  T acc = T(0);
  if (d_r) {
    acc = d_r[t];
  } else {
    const T rc = (T)r_cut;
    const T xr = r / rc;
    const T x2 = xr * xr, x4 = x2 * x2;
    const T omx = T(1) - xr;
    const T env = omx * omx * omx * (T(1) + xr * (T(3) + xr * (T(6) + xr * (T(10) + T(15) * xr))));
    const T denv = T(-105) * x4 * omx * omx / rc;
    T s1, c1;
    sincos_t<T>(T(3.14159265358979323846) * xr, &s1, &c1);
    const T pre = sqrt_t<T>(T(2) / rc);
    const T k1 = T(3.14159265358979323846) / rc;
    T sp = T(0), sn = s1, cp = T(1), cn = c1;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const T b = pre * sn * ir;
      const T db = pre * (k1 * T(n + 1) * cn * ir - sn * ir * ir);
      acc += d_ef[t * 8 + n] * (denv * b + env * db);
      const T ns = T(2) * c1 * sn - sp;
      const T nc = T(2) * c1 * cn - cp;
      sp = sn;
      sn = ns;
      cp = cn;
      cn = nc;
    }
  }
  const int64_t e = edge_begin + t;
  g[3 * e + 0] = (q[0] - uq * ux) * ir + acc * ux;
  g[3 * e + 1] = (q[1] - uq * uy) * ir + acc * uy;
  g[3 * e + 2] = (q[2] - uq * uz) * ir + acc * uz;
}

template <typename T, int L2>
hipError_t geom_fwd_impl(const GeomArgs& a, void* Y, void* ef, void* rv, hipStream_t s) {
  const int64_t ne = a.edge_end - a.edge_begin;
  if (ne <= 0) return hipSuccess;
  k_geom_fwd<T, L2><<<(unsigned)((ne + 255) / 256), 256, 0, s>>>(
      a, static_cast<T*>(Y), static_cast<T*>(ef), static_cast<T*>(rv));
  return hipGetLastError();
}

template <typename T>
hipError_t geom_fwd_t(int L2, const GeomArgs& a, void* Y, void* ef, void* rv, hipStream_t s) {
  switch (L2) {
    case 0: return geom_fwd_impl<T, 0>(a, Y, ef, rv, s);
    case 1: return geom_fwd_impl<T, 1>(a, Y, ef, rv, s);
    case 2: return geom_fwd_impl<T, 2>(a, Y, ef, rv, s);
    case 3: return geom_fwd_impl<T, 3>(a, Y, ef, rv, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int L2>
hipError_t geom_bwd_impl(int64_t ne, int64_t edge_begin, double r_cut, const void* rv,
                         const void* dY, int n_parts, const void* d_ef, const void* d_r, void* g,
                         hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  k_geom_bwd<T, L2><<<(unsigned)((ne + 255) / 256), 256, 0, s>>>(
      ne, edge_begin, r_cut, static_cast<const T*>(rv), static_cast<const T*>(dY), n_parts,
      static_cast<const T*>(d_ef), static_cast<const T*>(d_r), static_cast<T*>(g));
  return hipGetLastError();
}

template <typename T>
hipError_t geom_bwd_t(int L2, int64_t ne, int64_t eb, double rc, const void* rv, const void* dY,
                      int n_parts, const void* d_ef, const void* d_r, void* g, hipStream_t s) {
  switch (L2) {
    case 0: return geom_bwd_impl<T, 0>(ne, eb, rc, rv, dY, n_parts, d_ef, d_r, g, s);
    case 1: return geom_bwd_impl<T, 1>(ne, eb, rc, rv, dY, n_parts, d_ef, d_r, g, s);
    case 2: return geom_bwd_impl<T, 2>(ne, eb, rc, rv, dY, n_parts, d_ef, d_r, g, s);
    case 3: return geom_bwd_impl<T, 3>(ne, eb, rc, rv, dY, n_parts, d_ef, d_r, g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_geom_fwd(int dtype, int L2, const GeomArgs& a, void* Y, void* ef, void* rv,
                           hipStream_t s) {
  return dtype == 1 ? geom_fwd_t<double>(L2, a, Y, ef, rv, s) : geom_fwd_t<float>(L2, a, Y, ef, rv, s);
}

hipError_t launch_geom_bwd(int dtype, int L2, int64_t ne, int64_t edge_begin, double r_cut,
                           const void* rv, const void* dY, int n_parts, const void* d_ef, const void* d_r, void* g,
                           hipStream_t s) {
  return dtype == 1 ? geom_bwd_t<double>(L2, ne, edge_begin, r_cut, rv, dY, n_parts, d_ef, d_r, g, s)
                    : geom_bwd_t<float>(L2, ne, edge_begin, r_cut, rv, dY, n_parts, d_ef, d_r, g, s);
}

}  // namespace tpc
