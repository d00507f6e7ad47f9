// Radial MLP on the matrix cores (gfx950 MFMA, 16x16x4, float32 or float64).
//
// The radial network maps each edge's basis ef [8] to the per-path,
// per-channel weights R [P*C] of its tensor product (FastMACE page "Rewrites
// and precision options", section "Radial network"; FlashCart section 2 calls
// them the distance-dependent weights).  Bias-free: a_k = SiLU(a_{k-1} W_k) for
// the hidden layers, R = a_{L-1} W_L.  This is the only dense contraction of
// the convolution.
//
// Mapping.  Each MFMA computes D'[n][e] = sum_k W[k][n] * A[e][k] for 16 output
// features n and 16 edges e: the weight matrix is the A operand (lane l gives
// row l%16, k-slot l/16), the activations the B operand (lane l gives k-slot
// l/16, edge l%16).  Lane l then holds D'[row(g, r)][l%16] for r = 0..3 and
// g = l/16, with row(g, r) = 4g + r for the float32 instruction and 4r + g for
// the float64 one (measured lane layouts).  After a layer every lane owns the
// activations of one edge (l%16) at features 16*nb + row(g, r).  Because a
// contraction may visit k in any order, the next layer assigns reduction step
// s = 4*nb + r, k-slot g to feature k = 16*nb + row(g, r): the B operand of
// every step is then a register the lane already holds, so activations never
// leave registers between layers.  A wave owns S strips of 16 edges and
// reuses every weight load S times.
//
// Backward (input gradient only; FastMACE's "fused_folded_backward" idea of
// one kernel for the radial input gradient): the hidden layers are recomputed
// in registers, dA = dR W_L^T runs on MFMA with dR streamed as the B operand,
// then dz = dA * SiLU'(z) and dA_prev = dz W_k^T down to d(ef).
#include "common.hpp"
#include "kernels.hpp"

namespace tpc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  using type = f32x4;
};
template <>
struct Vec4<double> {
  using type = f64x4;
};
template <typename T>
using vec4 = typename Vec4<T>::type;

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mfma(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Row of the 16x16 MFMA result held in register r of a lane in group g.
template <typename T>
__device__ constexpr int drow(int g, int r) {
  return std::is_same<T, double>::value ? 4 * r + g : 4 * g + r;
}

__device__ __forceinline__ float exp_t(float x) { return expf(x); }
__device__ __forceinline__ double exp_t(double x) { return exp(x); }

template <typename T>
__device__ __forceinline__ T silu(T z) {
  return z / (T(1) + exp_t(-z));
}
template <typename T>
__device__ __forceinline__ T silu_dz(T z) {
  const T s = T(1) / (T(1) + exp_t(-z));
  return s * (T(1) + z * (T(1) - s));
}

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// forward
template <typename T, int H, int NH, int S>
__global__ void __launch_bounds__(256)
k_radial_fwd(int64_t ne, int pc, const T* __restrict__ ef, RadialWeights<T> W, T* __restrict__ R) {
  constexpr int NB = H / 16;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  if (e0 >= ne) return;

  T act[S][NB][4];
  // layer 1: K = 8 (two reduction steps, k = 4*s + g)
  {
    T b[S][2];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int64_t e = e0 + st * 16 + el;
#pragma unroll
      for (int s = 0; s < 2; ++s) b[st][s] = e < ne ? ef[e * 8 + 4 * s + g] : T(0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      T a[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) a[s] = W.w[0][(4 * s + g) * H + nb * 16 + el];
#pragma unroll
      for (int st = 0; st < S; ++st) {
        vec4<T> acc = {T(0), T(0), T(0), T(0)};
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mfma(a[s], b[st][s], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<T>(acc[r]);
      }
    }
  }
  // hidden layers 2..NH: K = H, step (nb, r) uses k = 16*nb + row(g, r)
#pragma unroll
  for (int layer = 1; layer < NH; ++layer) {
    const T* __restrict__ Wk = W.w[layer];
    T nxt[S][NB][4];
#pragma unroll
    for (int no = 0; no < NB; ++no) {
      vec4<T> acc[S];
#pragma unroll
      for (int st = 0; st < S; ++st) acc[st] = vec4<T>{T(0), T(0), T(0), T(0)};
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const T a = Wk[(16 * ni + drow<T>(g, r)) * H + no * 16 + el];
#pragma unroll
          for (int st = 0; st < S; ++st) acc[st] = mfma(a, act[st][ni][r], acc[st]);
        }
#pragma unroll
      for (int st = 0; st < S; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) nxt[st][no][r] = silu<T>(acc[st][r]);
    }
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) act[st][nb][r] = nxt[st][nb][r];
  }
  // last layer: R[e][c] for 16 columns per block
  const T* __restrict__ WL = W.w[NH];
  const int nblk = (pc + 15) / 16;
  for (int cb = 0; cb < nblk; ++cb) {
    const int col = cb * 16 + el;
    const bool col_ok = col < pc;
    vec4<T> acc[S];
#pragma unroll
    for (int st = 0; st < S; ++st) acc[st] = vec4<T>{T(0), T(0), T(0), T(0)};
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const T a = col_ok ? WL[(int64_t)(16 * ni + drow<T>(g, r)) * pc + col] : T(0);
#pragma unroll
        for (int st = 0; st < S; ++st) acc[st] = mfma(a, act[st][ni][r], acc[st]);
      }
    // lane holds R[e0 + st*16 + el][cb*16 + row(g, r)]
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int64_t e = e0 + st * 16 + el;
      if (e >= ne) continue;
      T* dst = R + e * (int64_t)pc + cb * 16;
      if (std::is_same<T, float>::value && cb * 16 + 4 * g + 3 < pc && (pc % 4) == 0) {
        *reinterpret_cast<vec4<T>*>(dst + 4 * g) = acc[st];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (cb * 16 + drow<T>(g, r) < pc) dst[drow<T>(g, r)] = acc[st][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward: d(ef) from dR
template <typename T, int H, int NH, int S>
__global__ void __launch_bounds__(256)
k_radial_bwd(int64_t ne, int pc, const T* __restrict__ ef, const T* __restrict__ dR,
             RadialWeights<T> W, T* __restrict__ d_ef) {
  constexpr int NB = H / 16;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  if (e0 >= ne) return;

  // recompute hidden pre-activations z[layer]
  T z[NH][S][NB][4];
  {
    T b[S][2];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int64_t e = e0 + st * 16 + el;
#pragma unroll
      for (int s = 0; s < 2; ++s) b[st][s] = e < ne ? ef[e * 8 + 4 * s + g] : T(0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      T a[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) a[s] = W.w[0][(4 * s + g) * H + nb * 16 + el];
#pragma unroll
      for (int st = 0; st < S; ++st) {
        vec4<T> acc = {T(0), T(0), T(0), T(0)};
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mfma(a[s], b[st][s], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) z[0][st][nb][r] = acc[r];
      }
    }
  }
#pragma unroll
  for (int layer = 1; layer < NH; ++layer) {
    const T* __restrict__ Wk = W.w[layer];
#pragma unroll
    for (int no = 0; no < NB; ++no) {
      vec4<T> acc[S];
#pragma unroll
      for (int st = 0; st < S; ++st) acc[st] = vec4<T>{T(0), T(0), T(0), T(0)};
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const T a = Wk[(16 * ni + drow<T>(g, r)) * H + no * 16 + el];
#pragma unroll
          for (int st = 0; st < S; ++st) acc[st] = mfma(a, silu<T>(z[layer - 1][st][ni][r]), acc[st]);
        }
#pragma unroll
      for (int st = 0; st < S; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[layer][st][no][r] = acc[st][r];
    }
  }

  // dA = dR W_L^T : D[k][e] = sum_n W_L[k][n] dR[e][n]; step (t, r) uses
  // n = 16*t + 4*g + r so each lane reads 4 consecutive columns.
  const T* __restrict__ WL = W.w[NH];
  vec4<T> dA[S][NB];
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) dA[st][kb] = vec4<T>{T(0), T(0), T(0), T(0)};
  const int nt = (pc + 15) / 16;
  for (int t = 0; t < nt; ++t) {
    const int n0 = 16 * t + 4 * g;
    T bv[S][4];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int64_t e = e0 + st * 16 + el;
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[st][r] = (e < ne && n0 + r < pc) ? dR[e * (int64_t)pc + n0 + r] : T(0);
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      T av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        av[r] = (n0 + r < pc) ? WL[(int64_t)(kb * 16 + el) * pc + n0 + r] : T(0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int st = 0; st < S; ++st) dA[st][kb] = mfma(av[r], bv[st][r], dA[st][kb]);
    }
  }
  // back through the hidden layers
#pragma unroll
  for (int layer = NH - 1; layer >= 0; --layer) {
    T dz[S][NB][4];
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dz[st][kb][r] = dA[st][kb][r] * silu_dz<T>(z[layer][st][kb][r]);
    const T* __restrict__ Wk = W.w[layer];
    if (layer > 0) {
      // D[k'][e] = sum_k W_k[k'][k] dz[e][k], k' in H
#pragma unroll
      for (int ko = 0; ko < NB; ++ko) {
#pragma unroll
        for (int st = 0; st < S; ++st) dA[st][ko] = vec4<T>{T(0), T(0), T(0), T(0)};
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const T a = Wk[(ko * 16 + el) * H + 16 * ni + drow<T>(g, r)];
#pragma unroll
            for (int st = 0; st < S; ++st) dA[st][ko] = mfma(a, dz[st][ni][r], dA[st][ko]);
          }
      }
    } else {
      // d(ef)[e][k'] for k' < 8: rows 8..15 of the MFMA tile are zero
      vec4<T> acc[S];
#pragma unroll
      for (int st = 0; st < S; ++st) acc[st] = vec4<T>{T(0), T(0), T(0), T(0)};
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const T a = el < 8 ? Wk[el * H + 16 * ni + drow<T>(g, r)] : T(0);
#pragma unroll
          for (int st = 0; st < S; ++st) acc[st] = mfma(a, dz[st][ni][r], acc[st]);
        }
#pragma unroll
      for (int st = 0; st < S; ++st) {
        const int64_t e = e0 + st * 16 + el;
        if (e >= ne) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (drow<T>(g, r) < 8) d_ef[e * 8 + drow<T>(g, r)] = acc[st][r];
      }
    }
  }
}

template <typename T, int H, int NH>
hipError_t radial_fwd_impl(int64_t ne, int pc, const void* ef, const RadialWeights<T>& W, void* R,
                           hipStream_t s) {
  constexpr int S = 4;
  const int64_t per_block = 4 * 16 * S;
  k_radial_fwd<T, H, NH, S><<<(unsigned)((ne + per_block - 1) / per_block), 256, 0, s>>>(
      ne, pc, static_cast<const T*>(ef), W, static_cast<T*>(R));
  return hipGetLastError();
}

template <typename T, int H, int NH>
hipError_t radial_bwd_impl(int64_t ne, int pc, const void* ef, const void* dR,
                           const RadialWeights<T>& W, void* d_ef, hipStream_t s) {
  constexpr int S = 2;
  const int64_t per_block = 4 * 16 * S;
  k_radial_bwd<T, H, NH, S><<<(unsigned)((ne + per_block - 1) / per_block), 256, 0, s>>>(
      ne, pc, static_cast<const T*>(ef), static_cast<const T*>(dR), W, static_cast<T*>(d_ef));
  return hipGetLastError();
}

template <typename T>
hipError_t radial_dispatch(bool fwd, int H, int NH, int64_t ne, int pc, const void* ef,
                           const void* dR, const void* const* w, void* out, hipStream_t s) {
  RadialWeights<T> W{};
  for (int k = 0; k <= NH; ++k) W.w[k] = static_cast<const T*>(w[k]);
#define TPC_RADIAL_CASE(HH, NN)                                             \
  if (H == HH && NH == NN)                                                  \
    return fwd ? radial_fwd_impl<T, HH, NN>(ne, pc, ef, W, out, s)          \
               : radial_bwd_impl<T, HH, NN>(ne, pc, ef, dR, W, out, s);
  TPC_RADIAL_CASE(16, 1)
  TPC_RADIAL_CASE(16, 2)
  TPC_RADIAL_CASE(16, 3)
  TPC_RADIAL_CASE(32, 1)
  TPC_RADIAL_CASE(32, 2)
  TPC_RADIAL_CASE(32, 3)
  TPC_RADIAL_CASE(64, 1)
  TPC_RADIAL_CASE(64, 2)
  TPC_RADIAL_CASE(64, 3)
#undef TPC_RADIAL_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool radial_supported(int H, int NH) {
  return (H == 16 || H == 32 || H == 64) && NH >= 1 && NH <= 3;
}

hipError_t launch_radial_fwd(int dtype, int H, int NH, int64_t ne, int pc, const void* ef,
                             const void* const* w, void* R, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  return dtype == 1 ? radial_dispatch<double>(true, H, NH, ne, pc, ef, nullptr, w, R, s)
                    : radial_dispatch<float>(true, H, NH, ne, pc, ef, nullptr, w, R, s);
}

hipError_t launch_radial_bwd(int dtype, int H, int NH, int64_t ne, int pc, const void* ef,
                             const void* dR, const void* const* w, void* d_ef, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  return dtype == 1 ? radial_dispatch<double>(false, H, NH, ne, pc, ef, dR, w, d_ef, s)
                    : radial_dispatch<float>(false, H, NH, ne, pc, ef, dR, w, d_ef, s);
}

}  // namespace tpc
