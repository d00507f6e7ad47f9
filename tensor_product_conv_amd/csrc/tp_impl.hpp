// Fused gather + sparse-coupling tensor product + receiver reduction (gfx950).
//
// Forward (FlashCart paper, section 2 "Equivariant convolution and many-body
// correlations"; section 4 receiver-sorted kernel):
//   out[i,(p,m3),u] = s * sum_{e in row i} R[e,p,u] * sum_{m1} M^p_e[m1,m3] h[src_e,(l1,m1),u]
//   M^p_e[m1,m3]   = sum_{m2} C^p[m1,m2,m3] Y[e,(l2,m2)]
// One wave owns one receiver row; lanes own channels (CPL consecutive channels
// per lane).  The edge loop runs in CSR order, so every output is a sum in a
// fixed order, accumulated in registers and stored once: no atomics and no
// per-edge message tensor (the receiver-streaming design of FastMACE's
// "streaming_conv" and FlashCart's receiver-sorted kernel, on a 64-wide wave).
// M^p_e is wave-uniform; its sparsity and the coupling coefficients are
// compile-time constants, so the unrolled code only touches non-zeros.
//
// Backward of L = sum(G * out) (FlashCart section 3 "Symbolic derivatives":
// the weight gradient is the inner product of the incoming gradient with the
// unweighted product; input gradients are the other factors times the weight):
//   edge kernel (wave per receiver i, G[i] loaded once):
//     dR[e,p,u]   = s * sum_m3 G[i,(p,m3),u] * sum_m1 M^p_e[m1,m3] h[j,m1,u]
//     dY[e,l2m2]  = s * sum_p sum_{m1,m3} C^p[m1,m2,m3] sum_u h[j,m1,u] R[e,p,u] G[i,(p,m3),u]
//   node kernel (wave per atom j, over j's own row):
//     dh[j,m1,u]  = s * sum_{e' in row j} sum_p (-1)^{l2} R[e',p,u]
//                       sum_{m3} M^p_{e'}[m1,m3] G[src_e',(p,m3),u]
// The node kernel uses the symmetry of the list: an edge e = (k <- j, S) has
// the reverse e' = (j <- k, -S) in row j with the same length (so the same R)
// and the opposite direction (so Y(e) = (-1)^l2 Y(e')).  Sender gradients are
// therefore gathered per row instead of scattered with atomics (FlashCart's
// VJP uses atomics there) or through a sender permutation.
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "tables.hpp"

namespace tpc {

constexpr int kTPWave = 64;
constexpr int kTPWavesPerBlock = 4;

template <typename T, int N>
struct VecN {
  typedef T type __attribute__((ext_vector_type(N)));
};

template <typename T, int CPL>
__device__ __forceinline__ void load_ch(const T* __restrict__ p, bool on, T (&v)[CPL]) {
  if constexpr (CPL == 1) {
    v[0] = on ? p[0] : T(0);
  } else {
    using V = typename VecN<T, CPL>::type;
    V x = on ? *reinterpret_cast<const V*>(p) : V{};
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = x[c];
  }
}

template <typename T, int CPL>
__device__ __forceinline__ void store_ch(T* __restrict__ p, bool on, const T (&v)[CPL]) {
  if (!on) return;
  if constexpr (CPL == 1) {
    p[0] = v[0];
  } else {
    using V = typename VecN<T, CPL>::type;
    V x;
#pragma unroll
    for (int c = 0; c < CPL; ++c) x[c] = v[c];
    *reinterpret_cast<V*>(p) = x;
  }
}

// M^p[m1][m3] for an edge from its uniform harmonics (compile-time sparsity).
template <typename T, int L1, int L2, int L3, int p, int m1, int m3>
__device__ __forceinline__ T coupling_matrix_entry(const T* y) {
  constexpr Path P = kTable<L1, L2, L3>.path[p];
  T M = T(0);
  static_for<2 * P.l2 + 1>([&](auto m2c) {
    constexpr int m2 = decltype(m2c)::value;
    constexpr double cv = kTable<L1, L2, L3>.cg[p][m1][m2][m3];
    if constexpr (cv != 0.0) M += T(cv) * y[P.l2 * P.l2 + m2];
  });
  return M;
}

// ---------------------------------------------------------------------------
template <typename T, int L1, int L2, int L3, int CPL>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
         int64_t row_end, int64_t edge_begin, int C, T scale, const T* __restrict__ h,
         const T* __restrict__ Y, const T* __restrict__ R, T* __restrict__ out) {
  constexpr int NP = kTable<L1, L2, L3>.np, DIN = kTable<L1, L2, L3>.din, DSH = kTable<L1, L2, L3>.dsh, DOUT = kTable<L1, L2, L3>.dout;
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = blockIdx.x * (int64_t)kTPWavesPerBlock + threadIdx.x / kTPWave;
  if (row_begin + w >= row_end) return;
  const int i = uniform((int)(row_begin + w));
  const int c0 = lane * CPL;
  const bool on = c0 < C;
  const int PC = NP * C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);

  T acc[DOUT][CPL];
#pragma unroll
  for (int o = 0; o < DOUT; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[o][c] = T(0);

  for (int e = e_lo; e < e_hi; ++e) {
    const int j = uniform(src[e]);
    const int64_t el = (int64_t)e - edge_begin;
    T y[DSH];
#pragma unroll
    for (int k = 0; k < DSH; ++k) y[k] = Y[el * DSH + k];
    T hv[DIN][CPL];
#pragma unroll
    for (int m = 0; m < DIN; ++m) load_ch<T, CPL>(h + ((int64_t)j * DIN + m) * C + c0, on, hv[m]);
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr Path P = kTable<L1, L2, L3>.path[p];
      T rp[CPL];
      load_ch<T, CPL>(R + el * PC + p * C + c0, on, rp);
      T hr[2 * P.l1 + 1][CPL];
#pragma unroll
      for (int m1 = 0; m1 < 2 * P.l1 + 1; ++m1)
#pragma unroll
        for (int c = 0; c < CPL; ++c) hr[m1][c] = rp[c] * hv[P.l1 * P.l1 + m1][c];
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        constexpr int row = kTable<L1, L2, L3>.out_row(p, m3);
        static_for<2 * P.l1 + 1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (m13_nonzero(kTable<L1, L2, L3>, p, m1, m3)) {
            const T M = coupling_matrix_entry<T, L1, L2, L3, p, m1, m3>(y);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[row][c] += M * hr[m1][c];
          }
        });
      });
    });
  }
#pragma unroll
  for (int o = 0; o < DOUT; ++o) {
    T v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = scale * acc[o][c];
    store_ch<T, CPL>(out + ((int64_t)i * DOUT + o) * C + c0, on, v);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kTPWave);
  return v;
}

template <typename T, int L1, int L2, int L3, int CPL>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_bwd_edge(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
              int64_t row_begin, int64_t row_end, int64_t edge_begin, int C, T scale,
              const T* __restrict__ h, const T* __restrict__ Y, const T* __restrict__ R,
              const T* __restrict__ G, T* __restrict__ dR, T* __restrict__ dY) {
  constexpr int NP = kTable<L1, L2, L3>.np, DIN = kTable<L1, L2, L3>.din, DSH = kTable<L1, L2, L3>.dsh, DOUT = kTable<L1, L2, L3>.dout;
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = blockIdx.x * (int64_t)kTPWavesPerBlock + threadIdx.x / kTPWave;
  if (row_begin + w >= row_end) return;
  const int i = uniform((int)(row_begin + w));
  const int c0 = lane * CPL;
  const bool on = c0 < C;
  const int PC = NP * C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  if (e_lo == e_hi) return;

  T gi[DOUT][CPL];
#pragma unroll
  for (int o = 0; o < DOUT; ++o) load_ch<T, CPL>(G + ((int64_t)i * DOUT + o) * C + c0, on, gi[o]);

  for (int e = e_lo; e < e_hi; ++e) {
    const int j = uniform(src[e]);
    const int64_t el = (int64_t)e - edge_begin;
    T y[DSH];
#pragma unroll
    for (int k = 0; k < DSH; ++k) y[k] = Y[el * DSH + k];
    T hv[DIN][CPL];
#pragma unroll
    for (int m = 0; m < DIN; ++m) load_ch<T, CPL>(h + ((int64_t)j * DIN + m) * C + c0, on, hv[m]);
    T dy[DSH];
#pragma unroll
    for (int k = 0; k < DSH; ++k) dy[k] = T(0);
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr Path P = kTable<L1, L2, L3>.path[p];
      T rp[CPL];
      load_ch<T, CPL>(R + el * PC + p * C + c0, on, rp);
      T drp[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) drp[c] = T(0);
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        constexpr int row = kTable<L1, L2, L3>.out_row(p, m3);
        T tm[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) tm[c] = T(0);
        T rg[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) rg[c] = rp[c] * gi[row][c];
        static_for<2 * P.l1 + 1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (m13_nonzero(kTable<L1, L2, L3>, p, m1, m3)) {
            const T M = coupling_matrix_entry<T, L1, L2, L3, p, m1, m3>(y);
            T hg = T(0);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              tm[c] += M * hv[P.l1 * P.l1 + m1][c];
              hg += hv[P.l1 * P.l1 + m1][c] * rg[c];
            }
            static_for<2 * P.l2 + 1>([&](auto m2c) {
              constexpr int m2 = decltype(m2c)::value;
              constexpr double cv = kTable<L1, L2, L3>.cg[p][m1][m2][m3];
              if constexpr (cv != 0.0) dy[P.l2 * P.l2 + m2] += T(cv) * hg;
            });
          }
        });
#pragma unroll
        for (int c = 0; c < CPL; ++c) drp[c] += gi[row][c] * tm[c];
      });
#pragma unroll
      for (int c = 0; c < CPL; ++c) drp[c] *= scale;
      store_ch<T, CPL>(dR + el * PC + p * C + c0, on, drp);
    });
#pragma unroll
    for (int k = 0; k < DSH; ++k) {
      const T v = wave_sum(dy[k]);
      if (lane == k) dY[el * DSH + k] = scale * v;
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int L1, int L2, int L3, int CPL>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_bwd_node(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
              int64_t row_begin, int64_t row_end, int64_t edge_begin, int C, T scale,
              const T* __restrict__ Y, const T* __restrict__ R, const T* __restrict__ G,
              T* __restrict__ dh) {
  constexpr int NP = kTable<L1, L2, L3>.np, DIN = kTable<L1, L2, L3>.din, DSH = kTable<L1, L2, L3>.dsh, DOUT = kTable<L1, L2, L3>.dout;
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = blockIdx.x * (int64_t)kTPWavesPerBlock + threadIdx.x / kTPWave;
  if (row_begin + w >= row_end) return;
  const int jn = uniform((int)(row_begin + w));
  const int c0 = lane * CPL;
  const bool on = c0 < C;
  const int PC = NP * C;
  const int e_lo = uniform(row_ptr[jn]), e_hi = uniform(row_ptr[jn + 1]);

  T acc[DIN][CPL];
#pragma unroll
  for (int m = 0; m < DIN; ++m)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[m][c] = T(0);

  for (int e = e_lo; e < e_hi; ++e) {
    const int k = uniform(src[e]);  // the reverse edge (k <- jn) has jn as sender
    const int64_t el = (int64_t)e - edge_begin;
    T y[DSH];
#pragma unroll
    for (int q = 0; q < DSH; ++q) y[q] = Y[el * DSH + q];
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr Path P = kTable<L1, L2, L3>.path[p];
      constexpr T sgn = (P.l2 % 2) ? T(-1) : T(1);
      T rp[CPL];
      load_ch<T, CPL>(R + el * PC + p * C + c0, on, rp);
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        constexpr int row = kTable<L1, L2, L3>.out_row(p, m3);
        T gk[CPL];
        load_ch<T, CPL>(G + ((int64_t)k * DOUT + row) * C + c0, on, gk);
        T rg[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) rg[c] = sgn * rp[c] * gk[c];
        static_for<2 * P.l1 + 1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (m13_nonzero(kTable<L1, L2, L3>, p, m1, m3)) {
            const T M = coupling_matrix_entry<T, L1, L2, L3, p, m1, m3>(y);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[P.l1 * P.l1 + m1][c] += M * rg[c];
          }
        });
      });
    });
  }
#pragma unroll
  for (int m = 0; m < DIN; ++m) {
    T v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = scale * acc[m][c];
    store_ch<T, CPL>(dh + ((int64_t)jn * DIN + m) * C + c0, on, v);
  }
}

// ---------------------------------------------------------------------------
inline unsigned tp_blocks(int64_t rows) {
  return (unsigned)((rows + kTPWavesPerBlock - 1) / kTPWavesPerBlock);
}

}  // namespace tpc

// Instantiated (dtype, node_lmax, sh_lmax, out_lmax, channels-per-lane) sets.
// Channels per lane is 1 for C <= 64 and 2 for C = 128.
#define TPC_TP_CONFIGS(X)                                                          \
  X(float, 1, 2, 1, 1) X(float, 1, 2, 1, 2) X(float, 1, 3, 3, 1) X(float, 1, 3, 3, 2) \
  X(float, 2, 3, 3, 1) X(float, 2, 3, 3, 2) X(float, 3, 3, 3, 1)                   \
  X(double, 1, 2, 1, 1) X(double, 1, 3, 3, 1) X(double, 2, 3, 3, 1) X(double, 3, 3, 3, 1)

inline int tp_cpl(int C) { return C >= 1 && C <= 64 ? 1 : (C == 128 ? 2 : 0); }

namespace tp_detail {
template <typename T>
constexpr int dtype_id() { return std::is_same<T, double>::value ? 1 : 0; }
}  // namespace tp_detail
