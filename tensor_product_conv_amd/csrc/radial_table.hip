// Piecewise Chebyshev tables of the radial chain (FastMACE page "Rewrites and
// precision options", section "Radial network", option radial_tables: the
// chain distance -> edge weights is replaced by piecewise Chebyshev tables
// fitted when the plan is built and certified against a float64 evaluation
// of the same weights, for the values and their first derivatives).
//
// The radial weights R(r) [P*C] depend on the edge length only (the radial
// network here takes no species), so one table serves every species pair.
// [0, r_cut] is split into `pieces` equal intervals; on each, every column
// of R is the degree-d interpolant at the d+1 Chebyshev-Gauss points.
//
// Table layout (context dtype), per piece q:
//   rows 0..d        c_k, R(r) = sum_k c_k T_k(x), x = 2 (r - q h) / h - 1
//   rows d+1..2d     e_k, dR/dr = sum_{k<d} e_k T_k(x) (derivative series,
//                    already scaled by 2 / h)
// each row holding P*C columns.
//
// Fit (float64): k_table_nodes evaluates the radial network at the points,
// k_table_coef forms c_k = (2 - [k=0]) / n sum_j f(r_j) cos(pi k (j + 1/2) / n)
// and the derivative series by the recurrence e_{k-1} = e_{k+1} + 2 k c_k.
// Certificate: k_table_cert evaluates the stored table exactly as the
// runtime kernels do, at each piece's start and at points between its
// nodes, and divides its largest error on the piece by the largest float
// rounding scale, on the piece, of the computation it replaces.
// Runtime: k_table_fwd_sorted writes R from the table (Clenshaw), and
// k_table_bwd_sorted forms dL/dr = sum_c dR[c] dR_c/dr for the geometry
// backward, both over edges bucketed by piece (see below).
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "nbr.hpp"

namespace tpc {

namespace {

constexpr double kPi = 3.14159265358979323846;

// float64 basis times envelope (the same definitions as the geometry
// kernel's ef, here with their r-derivatives for the certificate)
__device__ void edge_features_f64(double r, double r_cut, double* ef, double* def) {
  const double x = r / r_cut;
  const double x2 = x * x, x4 = x2 * x2;
  const double omx = 1.0 - x;
  const double env = omx * omx * omx * (1.0 + x * (3.0 + x * (6.0 + x * (10.0 + 15.0 * x))));
  const double denv = -105.0 * x4 * omx * omx / r_cut;
  const double pre = sqrt(2.0 / r_cut);
  for (int n = 1; n <= 8; ++n) {
    const double k = n * kPi / r_cut;
    double b, db;
    if (r > 1e-12) {
      const double s = sin(k * r), c = cos(k * r);
      b = pre * s / r;
      db = pre * (k * c / r - s / (r * r));
    } else {  // limits at r = 0
      b = pre * k;
      db = 0.0;
    }
    ef[n - 1] = env * b;
    def[n - 1] = denv * b + env * db;
  }
}

// One block per point: the network in float64 (activations and their
// r-derivatives in LDS), then every column.  Weights in the context dtype.
template <typename T>
__device__ void network_f64(const RadialWeights<T>& W, int NH, int H, double r, double r_cut, double* a,
                            double* da, double* buf) {
  if (threadIdx.x == 0) edge_features_f64(r, r_cut, a, da);
  __syncthreads();
  int fan_in = 8;
  for (int layer = 0; layer < NH; ++layer) {
    const T* w = W.w[layer];
    double z = 0.0, dz = 0.0;
    const int t = threadIdx.x;
    if (t < H) {
      for (int k = 0; k < fan_in; ++k) {
        const double wk = (double)w[k * H + t];
        z += a[k] * wk;
        dz += da[k] * wk;
      }
    }
    __syncthreads();
    if (t < H) {
      const double sg = 1.0 / (1.0 + exp(-z));
      buf[t] = z * sg;
      buf[64 + t] = sg * (1.0 + z * (1.0 - sg)) * dz;
    }
    __syncthreads();
    if (t < H) {
      a[t] = buf[t];
      da[t] = buf[64 + t];
    }
    __syncthreads();
    fan_in = H;
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
k_table_nodes(RadialWeights<T> W, int NH, int H, int pc, int pieces, int n, double r_cut,
              double* __restrict__ f) {
  __shared__ double a[64], da[64], buf[128];
  const int node = blockIdx.x;
  const int q = node / n, j = node % n;
  const double h = r_cut / pieces;
  const double x = cos(kPi * (j + 0.5) / n);
  const double r = q * h + h * (x + 1.0) / 2.0;
  network_f64<T>(W, NH, H, r, r_cut, a, da, buf);
  const T* wl = W.w[NH];
  for (int c = threadIdx.x; c < pc; c += blockDim.x) {
    double acc = 0.0;
    for (int k = 0; k < H; ++k) acc += a[k] * (double)wl[(int64_t)k * pc + c];
    f[(int64_t)node * pc + c] = acc;
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
k_table_coef(int pc, int pieces, int n, double r_cut, const double* __restrict__ f, T* __restrict__ table) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)pieces * pc) return;
  const int q = (int)(t / pc), c = (int)(t % pc);
  double ck[kTableMaxDegree + 1], ek[kTableMaxDegree + 2];
  for (int k = 0; k < n; ++k) {
    double s = 0.0;
    for (int j = 0; j < n; ++j) s += f[((int64_t)q * n + j) * pc + c] * cos(kPi * k * (j + 0.5) / n);
    ck[k] = (k == 0 ? 1.0 : 2.0) / n * s;
  }
  // derivative series in x, then d/dr = (2 / h) d/dx
  const int d = n - 1;
  ek[d] = 0.0;
  ek[d + 1] = 0.0;
  for (int k = d; k >= 1; --k) ek[k - 1] = ek[k + 1] + 2.0 * k * ck[k];
  ek[0] *= 0.5;
  const double s = 2.0 * pieces / r_cut;
  T* tq = table + (int64_t)q * (2 * n - 1) * pc;
  for (int k = 0; k < n; ++k) tq[(int64_t)k * pc + c] = (T)ck[k];
  for (int k = 0; k < d; ++k) tq[(int64_t)(n + k) * pc + c] = (T)(s * ek[k]);
}

}  // namespace

// Value and r-derivative of column c at r (Clenshaw), in the table's dtype:
// the evaluation the runtime kernels and the certificate share.
template <typename T>
__device__ __forceinline__ void table_eval(const T* __restrict__ table, int pieces, int n, int pc, T r_cut,
                                           T r, int c, T* val, T* der) {
  const T h = r_cut / (T)pieces;
  int q = (int)(r / h);
  q = q < 0 ? 0 : (q >= pieces ? pieces - 1 : q);
  T x = T(2) * (r - (T)q * h) / h - T(1);
  x = x < T(-1) ? T(-1) : (x > T(1) ? T(1) : x);
  const T* tq = table + (int64_t)q * (2 * n - 1) * pc + c;
  T b1 = T(0), b2 = T(0);
  for (int k = n - 1; k >= 1; --k) {
    const T b0 = tq[(int64_t)k * pc] + T(2) * x * b1 - b2;
    b2 = b1;
    b1 = b0;
  }
  *val = tq[0] + x * b1 - b2;
  T d1 = T(0), d2 = T(0);
  for (int k = n - 2; k >= 1; --k) {
    const T b0 = tq[(int64_t)(n + k) * pc] + T(2) * x * d1 - d2;
    d2 = d1;
    d1 = b0;
  }
  *der = n > 1 ? tq[(int64_t)n * pc] + x * d1 - d2 : T(0);
}

namespace {

// One block per piece.  The network (float64) at the piece's check points
// goes to LDS; then, per column, the table's largest error on the piece is
// divided by the largest rounding scale of the replaced computation on the
// piece, and the block writes the largest ratio over its columns.  Taking
// both maxima over the piece keeps the ratio meaningful where the weights
// and their scale vanish together (the derivative at r = 0, the triple zero
// of the envelope at r_cut), where a float table's absolute rounding cannot
// follow the relative accuracy of the network.
template <typename T>
__global__ void __launch_bounds__(256)
k_table_cert(RadialWeights<T> W, int NH, int H, int pc, int pieces, int n, double r_cut,
             const T* __restrict__ table, double* __restrict__ out) {
  constexpr int M = kTableCheckPerPiece;
  __shared__ double a[64], da[64], buf[128];
  __shared__ double act[M][2][64];
  __shared__ double rs[M];
  __shared__ double red[2][256];
  const int q = blockIdx.x;
  const double h = r_cut / pieces;
  for (int m = 0; m < M; ++m) {
    // x = -1 (the piece start) and M - 1 points between the nodes
    const double x = m == 0 ? -1.0 : -1.0 + (2.0 * m - 1.0) / (M - 1);
    const double r = q * h + h * (x + 1.0) / 2.0;
    network_f64<T>(W, NH, H, r, r_cut, a, da, buf);
    if ((int)threadIdx.x < H) {
      act[m][0][threadIdx.x] = a[threadIdx.x];
      act[m][1][threadIdx.x] = da[threadIdx.x];
    }
    if (threadIdx.x == 0) rs[m] = r;
    __syncthreads();
  }
  const double eps = sizeof(T) == 8 ? 1.1102230246251565e-16 : 5.9604644775390625e-08;
  const T* wl = W.w[NH];
  double rv = 0.0, rd = 0.0;
  for (int c = threadIdx.x; c < pc; c += blockDim.x) {
    double ev = 0.0, ed = 0.0, sv = 0.0, sd = 0.0;
    for (int m = 0; m < M; ++m) {
      double R = 0.0, dR = 0.0, S = 0.0, dS = 0.0;
      for (int k = 0; k < H; ++k) {
        const double wk = (double)wl[(int64_t)k * pc + c];
        R += act[m][0][k] * wk;
        dR += act[m][1][k] * wk;
        S += fabs(act[m][0][k] * wk);
        dS += fabs(act[m][1][k] * wk);
      }
      T tv, td;
      table_eval<T>(table, pieces, n, pc, (T)r_cut, (T)rs[m], c, &tv, &td);
      // the rounding scale of the computation replaced: the last layer's dot
      // product and the rounding of the distance it is given
      sv = fmax(sv, H * eps * S + eps * fabs(rs[m] * dR));
      sd = fmax(sd, H * eps * dS + eps * fabs(dR));
      ev = fmax(ev, fabs((double)tv - R));
      ed = fmax(ed, fabs((double)td - dR));
    }
    rv = fmax(rv, ev / (sv + 1e-300));
    rd = fmax(rd, ed / (sd + 1e-300));
  }
  red[0][threadIdx.x] = rv;
  red[1][threadIdx.x] = rd;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      red[0][threadIdx.x] = fmax(red[0][threadIdx.x], red[0][threadIdx.x + s]);
      red[1][threadIdx.x] = fmax(red[1][threadIdx.x], red[1][threadIdx.x + s]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[2 * q] = red[0][0];
    out[2 * q + 1] = red[1][0];
  }
}

// ---------------------------------------------------------------------------
// Runtime evaluation over edges grouped by piece.  Evaluated edge by edge,
// every edge would read (degree + 1) coefficient rows of P*C columns from L2,
// about (degree + 1) times the bytes of the R row it writes.  Instead the
// edges of a chunk are bucketed by piece (a counting sort: k_table_count,
// k_table_offsets, k_table_place), and a block walks a contiguous range of
// the sorted order with its columns' coefficients of the current piece in
// registers, reloading them only when the piece changes.  Each R row (and
// each dL/dr) depends on its own edge only, so the order the atomics give
// the edges within a bucket changes no value.

constexpr int kTabThreads = 512;  // threads per block
constexpr int kTabCols = 6;       // columns per thread: P*C <= 3072
constexpr int kTabChunk = 256;    // sorted positions per block

template <typename T>
__device__ __forceinline__ int table_piece(T r, T r_cut, int pieces) {
  const T h = r_cut / (T)pieces;
  int q = (int)(r / h);
  return q < 0 ? 0 : (q >= pieces ? pieces - 1 : q);
}

template <typename T>
__device__ __forceinline__ T table_x(T r, T r_cut, int pieces, int q) {
  const T h = r_cut / (T)pieces;
  const T x = T(2) * (r - (T)q * h) / h - T(1);
  return x < T(-1) ? T(-1) : (x > T(1) ? T(1) : x);
}

// Clenshaw sum of M coefficients a[0..M-1] at x, in table_eval's order.
template <typename T, int M>
__device__ __forceinline__ T clenshaw(const T (&a)[M], T x) {
  if constexpr (M == 0) {
    return T(0);
  } else {
    T b1 = T(0), b2 = T(0);
#pragma unroll
    for (int k = M - 1; k >= 1; --k) {
      const T b0 = a[k] + T(2) * x * b1 - b2;
      b2 = b1;
      b1 = b0;
    }
    return a[0] + x * b1 - b2;
  }
}

// The counting sort works per block of kSortChunk edges: counts in LDS,
// then one global atomic per piece the block touches (a global atomic per
// edge would serialise on the few piece counters).
constexpr int kSortChunk = 4096;
constexpr int kSortThreads = 256;
constexpr int kMaxPieces = 4096;

template <typename T>
__global__ void __launch_bounds__(kSortThreads)
k_table_count(int64_t ne, int pieces, T r_cut, const T* __restrict__ rv, int* __restrict__ counts) {
  __shared__ int hist[kMaxPieces];
  const int64_t e0 = blockIdx.x * (int64_t)kSortChunk;
  for (int q = threadIdx.x; q < pieces; q += kSortThreads) hist[q] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) {
    const int64_t e = e0 + i;
    if (e < ne) atomicAdd(&hist[table_piece<T>(rv[e * 4 + 3], r_cut, pieces)], 1);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < pieces; q += kSortThreads)
    if (hist[q]) atomicAdd(&counts[q], hist[q]);
}

// counts -> start positions (exclusive scan; the pieces are few)
__global__ void k_table_offsets(int pieces, int* __restrict__ counts) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int run = 0;
  for (int q = 0; q < pieces; ++q) {
    const int n = counts[q];
    counts[q] = run;
    run += n;
  }
}

template <typename T>
__global__ void __launch_bounds__(kSortThreads)
k_table_place(int64_t ne, int pieces, T r_cut, const T* __restrict__ rv, int* __restrict__ cursor,
              int* __restrict__ order) {
  __shared__ int hist[kMaxPieces];
  const int64_t e0 = blockIdx.x * (int64_t)kSortChunk;
  for (int q = threadIdx.x; q < pieces; q += kSortThreads) hist[q] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) {
    const int64_t e = e0 + i;
    if (e < ne) atomicAdd(&hist[table_piece<T>(rv[e * 4 + 3], r_cut, pieces)], 1);
  }
  __syncthreads();
  // reserve the block's range of each piece; hist[q] becomes its next slot
  for (int q = threadIdx.x; q < pieces; q += kSortThreads)
    if (hist[q]) hist[q] = atomicAdd(&cursor[q], hist[q]);
  __syncthreads();
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) {
    const int64_t e = e0 + i;
    if (e < ne) order[atomicAdd(&hist[table_piece<T>(rv[e * 4 + 3], r_cut, pieces)], 1)] = (int)e;
  }
}

// R[e][c] over sorted positions: N = degree + 1 value coefficients per column.
template <typename T, int N>
__global__ void __launch_bounds__(kTabThreads)
k_table_fwd_sorted(int64_t ne, int pc, int pieces, T r_cut, const T* __restrict__ rv,
                   const T* __restrict__ table, const int* __restrict__ order, T* __restrict__ R) {
  __shared__ int se[kTabChunk];
  __shared__ T sr[kTabChunk];
  const int64_t p0 = blockIdx.x * (int64_t)kTabChunk;
  const int np = (int)(p0 + kTabChunk < ne ? kTabChunk : ne - p0);
  const int t = threadIdx.x;
  // the block's edges and lengths first, so the loop below carries no
  // dependent global loads
  if (t < np) {
    const int e = order[p0 + t];
    se[t] = e;
    sr[t] = rv[(int64_t)e * 4 + 3];
  }
  __syncthreads();
  T cf[kTabCols][N];
  int cur = -1;
  for (int i = 0; i < np; ++i) {
    const int e = se[i];
    const T r = sr[i];
    const int q = uniform(table_piece<T>(r, r_cut, pieces));
    if (q != cur) {
      const T* tq = table + (int64_t)q * (2 * N - 1) * pc;
#pragma unroll
      for (int j = 0; j < kTabCols; ++j) {
        const int c = t + kTabThreads * j;
#pragma unroll
        for (int k = 0; k < N; ++k) cf[j][k] = c < pc ? tq[(int64_t)k * pc + c] : T(0);
      }
      cur = q;
    }
    const T x = table_x<T>(r, r_cut, pieces, q);
    T* re = R + (int64_t)e * pc;
#pragma unroll
    for (int j = 0; j < kTabCols; ++j) {
      const int c = t + kTabThreads * j;
      if (c < pc) __builtin_nontemporal_store(clenshaw<T, N>(cf[j], x), re + c);
    }
  }
}

// dL/dr[e] = sum_c dR[e][c] dR_c/dr over sorted positions, GR edges per
// reduction: the group's dR values load first (every load in flight at
// once), then per edge the Clenshaw sums and per-thread partials, a wave sum,
// and the block's waves added in a fixed order.
template <typename T, int N>
__global__ void __launch_bounds__(kTabThreads)
k_table_bwd_sorted(int64_t ne, int pc, int pieces, T r_cut, const T* __restrict__ rv,
                   const T* __restrict__ table, const T* __restrict__ dR, const int* __restrict__ order,
                   T* __restrict__ d_r) {
  constexpr int D = N - 1;  // derivative coefficients per column
  constexpr int W = kTabThreads / 64;
  constexpr int GR = sizeof(T) == 8 ? 4 : 16;  // edges per reduction
  __shared__ T part[W][GR];
  __shared__ int se[kTabChunk];
  __shared__ T sr[kTabChunk];
  const int64_t p0 = blockIdx.x * (int64_t)kTabChunk;
  const int np = (int)(p0 + kTabChunk < ne ? kTabChunk : ne - p0);
  const int t = threadIdx.x, lane = t % 64, wv = t / 64;
  if (t < np) {
    const int e = order[p0 + t];
    se[t] = e;
    sr[t] = rv[(int64_t)e * 4 + 3];
  }
  __syncthreads();
  T cf[kTabCols][D > 0 ? D : 1];
  int cur = -1;
  for (int g0 = 0; g0 < np; g0 += GR) {
    T dv[GR][kTabCols];
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      const int e = se[g0 + i < np ? g0 + i : np - 1];
      const T* de = dR + (int64_t)e * pc;
#pragma unroll
      for (int j = 0; j < kTabCols; ++j) {
        const int c = t + kTabThreads * j;
        dv[i][j] = (c < pc && g0 + i < np) ? __builtin_nontemporal_load(de + c) : T(0);
      }
    }
    T acc[GR];
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      acc[i] = T(0);
      if (g0 + i < np) {
        const T r = sr[g0 + i];
        const int q = uniform(table_piece<T>(r, r_cut, pieces));
        if (q != cur) {
          const T* tq = table + ((int64_t)q * (2 * N - 1) + N) * pc;
#pragma unroll
          for (int j = 0; j < kTabCols; ++j) {
            const int c = t + kTabThreads * j;
#pragma unroll
            for (int k = 0; k < D; ++k) cf[j][k] = c < pc ? tq[(int64_t)k * pc + c] : T(0);
          }
          cur = q;
        }
        const T x = table_x<T>(r, r_cut, pieces, q);
        T sacc = T(0);
#pragma unroll
        for (int j = 0; j < kTabCols; ++j)
          if constexpr (D > 0) sacc += dv[i][j] * clenshaw<T, D>(cf[j], x);
        acc[i] = sacc;
      }
    }
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      T v = acc[i];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) part[wv][i] = v;
    }
    __syncthreads();
    if (t < GR && g0 + t < np) {
      T v = T(0);
#pragma unroll
      for (int w = 0; w < W; ++w) v += part[w][t];
      d_r[se[g0 + t]] = v;
    }
    __syncthreads();
  }
}

}  // namespace

int64_t table_elems(int pieces, int degree, int pc) { return (int64_t)pieces * (2 * degree + 1) * pc; }

hipError_t launch_table_fit(int dtype, int NH, int H, int pc, int pieces, int degree, double r_cut,
                            const void* const* w, double* f64_nodes, void* table, double* cert,
                            hipStream_t s) {
  const int n = degree + 1;
  const int blocks_nodes = pieces * n;
  const int64_t coef_threads = (int64_t)pieces * pc;
  if (dtype == 1) {
    RadialWeights<double> W{};
    for (int k = 0; k <= NH; ++k) W.w[k] = static_cast<const double*>(w[k]);
    k_table_nodes<double><<<blocks_nodes, 256, 0, s>>>(W, NH, H, pc, pieces, n, r_cut, f64_nodes);
    k_table_coef<double><<<(unsigned)((coef_threads + 255) / 256), 256, 0, s>>>(
        pc, pieces, n, r_cut, f64_nodes, static_cast<double*>(table));
    k_table_cert<double><<<pieces, 256, 0, s>>>(W, NH, H, pc, pieces, n, r_cut,
                                                static_cast<const double*>(table), cert);
  } else {
    RadialWeights<float> W{};
    for (int k = 0; k <= NH; ++k) W.w[k] = static_cast<const float*>(w[k]);
    k_table_nodes<float><<<blocks_nodes, 256, 0, s>>>(W, NH, H, pc, pieces, n, r_cut, f64_nodes);
    k_table_coef<float><<<(unsigned)((coef_threads + 255) / 256), 256, 0, s>>>(
        pc, pieces, n, r_cut, f64_nodes, static_cast<float*>(table));
    k_table_cert<float><<<pieces, 256, 0, s>>>(W, NH, H, pc, pieces, n, r_cut,
                                               static_cast<const float*>(table), cert);
  }
  return hipGetLastError();
}

int64_t table_sort_ints(int pieces, int64_t ne) { return (int64_t)pieces + 1 + ne; }

namespace {

template <typename T>
hipError_t table_sort(int64_t ne, int pieces, double r_cut, const T* rv, int* work, hipStream_t s) {
  int* counts = work;
  int* order = work + pieces + 1;
  hipError_t e = launch_fill_i32(counts, pieces + 1, 0, s);
  if (e != hipSuccess) return e;
  if (pieces > kMaxPieces) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((ne + kSortChunk - 1) / kSortChunk);
  k_table_count<T><<<blocks, kSortThreads, 0, s>>>(ne, pieces, (T)r_cut, rv, counts);
  k_table_offsets<<<1, 64, 0, s>>>(pieces, counts);
  k_table_place<T><<<blocks, kSortThreads, 0, s>>>(ne, pieces, (T)r_cut, rv, counts, order);
  return hipGetLastError();
}

#define TPC_TABLE_N(X) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16) X(17)

template <typename T>
hipError_t table_fwd_t(int64_t ne, int pc, int pieces, int n, double r_cut, const T* rv, const T* table,
                       int* work, T* R, hipStream_t s) {
  hipError_t e = table_sort<T>(ne, pieces, r_cut, rv, work, s);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((ne + kTabChunk - 1) / kTabChunk);
  const int* order = work + pieces + 1;
#define TPC_CASE(NN)                                                                                 \
  if (n == NN) {                                                                                     \
    k_table_fwd_sorted<T, NN><<<blocks, kTabThreads, 0, s>>>(ne, pc, pieces, (T)r_cut, rv, table, order, R); \
    return hipGetLastError();                                                                        \
  }
  TPC_TABLE_N(TPC_CASE)
#undef TPC_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t table_bwd_t(int64_t ne, int pc, int pieces, int n, double r_cut, const T* rv, const T* table,
                       const T* dR, int* work, T* d_r, hipStream_t s) {
  hipError_t e = table_sort<T>(ne, pieces, r_cut, rv, work, s);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((ne + kTabChunk - 1) / kTabChunk);
  const int* order = work + pieces + 1;
#define TPC_CASE(NN)                                                                                      \
  if (n == NN) {                                                                                          \
    k_table_bwd_sorted<T, NN><<<blocks, kTabThreads, 0, s>>>(ne, pc, pieces, (T)r_cut, rv, table, dR, order, \
                                                              d_r);                                         \
    return hipGetLastError();                                                                             \
  }
  TPC_TABLE_N(TPC_CASE)
#undef TPC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_table_fwd(int dtype, int64_t ne, int pc, int pieces, int degree, double r_cut,
                            const void* rv, const void* table, void* work, void* R, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  if (pc > kTabThreads * kTabCols) return hipErrorInvalidValue;
  int* w = static_cast<int*>(work);
  if (dtype == 1)
    return table_fwd_t<double>(ne, pc, pieces, degree + 1, r_cut, static_cast<const double*>(rv),
                               static_cast<const double*>(table), w, static_cast<double*>(R), s);
  return table_fwd_t<float>(ne, pc, pieces, degree + 1, r_cut, static_cast<const float*>(rv),
                            static_cast<const float*>(table), w, static_cast<float*>(R), s);
}

hipError_t launch_table_bwd(int dtype, int64_t ne, int pc, int pieces, int degree, double r_cut,
                            const void* rv, const void* table, const void* dR, void* work, void* d_r,
                            hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  if (pc > kTabThreads * kTabCols) return hipErrorInvalidValue;
  int* w = static_cast<int*>(work);
  if (dtype == 1)
    return table_bwd_t<double>(ne, pc, pieces, degree + 1, r_cut, static_cast<const double*>(rv),
                               static_cast<const double*>(table), static_cast<const double*>(dR), w,
                               static_cast<double*>(d_r), s);
  return table_bwd_t<float>(ne, pc, pieces, degree + 1, r_cut, static_cast<const float*>(rv),
                            static_cast<const float*>(table), static_cast<const float*>(dR), w,
                            static_cast<float*>(d_r), s);
}

}  // namespace tpc
