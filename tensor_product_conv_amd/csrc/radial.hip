// Radial MLP on the matrix cores (gfx950 MFMA, 16x16x4, float32 or float64).
//
// The radial network maps each edge's basis ef [8] to the per-path,
// per-channel weights R [P*C] of its tensor product (FastMACE page "Rewrites
// and precision options", section "Radial network"; FlashCart section 2 calls
// them the distance-dependent weights).  Bias-free: a_k = SiLU(a_{k-1} W_k) for
// the hidden layers, R = a_{L-1} W_L.  This is the only dense contraction of
// the convolution, and its last layer (H x P*C) holds nearly all of its flops.
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
// Weights.  k_radial_pack rewrites the caller's weight matrices once per call
// into "operand order": for every 16-wide output block, the values each lane
// feeds to the MFMA steps of that block lie next to each other, so a lane
// fetches a block's weights with 16-byte vector loads and the hot loops carry
// no index arithmetic, bounds tests or scattered loads.  The last layer is
// streamed block by block with the next block's weights in flight while the
// current block's MFMAs run.
//
// Backward (input gradient only; FastMACE's "fused_folded_backward" idea of
// one pass for the radial input gradient): k_radial_bwd_dA forms the big
// product dA = dR W_L^T on MFMA, streaming dR as the B operand and keeping
// only the accumulators live, and writes dA per wave strip in register order;
// k_radial_bwd_mlp recomputes the hidden layers in registers and carries dA
// down through dz = dA * SiLU'(z), dA_prev = dz W_k^T to d(ef).
#include "common.hpp"
#include "kernels.hpp"

namespace tpc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

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

// Four consecutive values from a 16-byte aligned address.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f64x4 ld4(const double* p) {
  const f64x2 a = *reinterpret_cast<const f64x2*>(p);
  const f64x2 b = *reinterpret_cast<const f64x2*>(p + 2);
  return f64x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st4(double* p, f64x4 v) {
  *reinterpret_cast<f64x2*>(p) = f64x2{v[0], v[1]};
  *reinterpret_cast<f64x2*>(p + 2) = f64x2{v[2], v[3]};
}

// Row of the 16x16 MFMA result held in register r of a lane in group g.
template <typename T>
__host__ __device__ constexpr int drow(int g, int r) {
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

template <typename T>
__device__ __forceinline__ vec4<T> zero4() {
  return vec4<T>{T(0), T(0), T(0), T(0)};
}

// ---------------------------------------------------------------------------
// float32 products on the bf16 matrix cores.  Every operand x is split into
// three bf16 parts, x = x1 + x2 + x3 + O(2^-24 |x|) (x1 = bf16(x), x2 =
// bf16(x - x1), x3 = bf16(x - x1 - x2); the differences are exact in
// float32), and a product keeps the six cross terms x_i y_j with i + j <= 4,
// which carry everything above about 2^-24 |xy|, accumulated in float32 from
// the smallest up.  FastMACE's "tf32x3_gemms" precision option splits matrix
// products into reduced-precision tensor-core products the same way; with
// bf16 parts three terms would leave about 2^-17 relative error, six reach
// float32 rounding.  One v_mfma_f32_16x16x32_bf16 covers 32 reduction steps
// in half the cycles of the float32 instruction's 4, so the six terms cost
// 3/8 of the float32 product.
// Lane layout (measured): lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16] for j = 0..7, and receives D[4(l/16)+r][l%16].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split3(float x, __bf16& p1, __bf16& p2, __bf16& p3) {
  p1 = (__bf16)x;
  const float r1 = x - (float)p1;
  p2 = (__bf16)r1;
  const float r2 = r1 - (float)p2;
  p3 = (__bf16)r2;
}

__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// c += A B with A, B given as their three bf16 parts (six terms, small first).
__device__ __forceinline__ f32x4 mfma_x6(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x4 c) {
  c = mfma_bf(a[2], b[0], c);
  c = mfma_bf(a[0], b[2], c);
  c = mfma_bf(a[1], b[1], c);
  c = mfma_bf(a[1], b[0], c);
  c = mfma_bf(a[0], b[1], c);
  c = mfma_bf(a[0], b[0], c);
  return c;
}

// Whether the float32 last layer takes the split-bf16 kernels.
__host__ __device__ constexpr bool x6_shape(int H, int pc) { return H % 32 == 0 && pc % 32 == 0; }

// ---------------------------------------------------------------------------
// weight packing (see RadialPack for the sections)
template <typename T>
__global__ void __launch_bounds__(256) k_radial_pack(RadialPack L, RadialWeights<T> W, T* __restrict__ pk) {
  const int H = L.H, NB = L.H / 16, S4 = 4 * L.H / 16, pc = L.pc;
  const int64_t per_hidden = (int64_t)NB * kWave * S4;
  const T* __restrict__ WL = W.w[L.NH];
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < L.total;
       i += (int64_t)gridDim.x * blockDim.x) {
    T v = T(0);
    if (i < L.fh) {
      const int64_t q = i - L.f0;
      if (q < (int64_t)NB * kWave * 2) {
        const int s = (int)(q % 2), lane = (int)((q / 2) % kWave), nb = (int)(q / (2 * kWave));
        v = W.w[0][(4 * s + lane / 16) * H + nb * 16 + lane % 16];
      }
    } else if (i < L.fl) {
      int64_t q = i - L.fh;
      if (q < (L.NH - 1) * per_hidden) {
        const int k = 1 + (int)(q / per_hidden);
        q %= per_hidden;
        const int j = (int)(q % S4), lane = (int)((q / S4) % kWave), no = (int)(q / (S4 * kWave));
        const int g = lane / 16, el = lane % 16;
        v = W.w[k][(16 * (j / 4) + drow<T>(g, j % 4)) * H + no * 16 + el];
      }
    } else if (i < L.bl) {
      const int64_t q = i - L.fl;
      if (q < (int64_t)L.nblk * kWave * S4) {
        const int j = (int)(q % S4), lane = (int)((q / S4) % kWave);
        const int64_t cb = q / (S4 * kWave);
        const int g = lane / 16, el = lane % 16;
        const int64_t col = cb * 16 + el;
        if (col < pc) v = WL[(int64_t)(16 * (j / 4) + drow<T>(g, j % 4)) * pc + col];
      }
    } else if (i < L.bh) {
      const int64_t q = i - L.bl;
      if (q < (int64_t)L.nblk * kWave * S4) {
        const int j = (int)(q % S4), lane = (int)((q / S4) % kWave);
        const int64_t t = q / (S4 * kWave);
        const int g = lane / 16, el = lane % 16;
        const int64_t col = 16 * t + 4 * g + j % 4;
        if (col < pc) v = WL[(int64_t)((j / 4) * 16 + el) * pc + col];
      }
    } else if (i < L.b0) {
      int64_t q = i - L.bh;
      if (q < (L.NH - 1) * per_hidden) {
        const int k = 1 + (int)(q / per_hidden);
        q %= per_hidden;
        const int j = (int)(q % S4), lane = (int)((q / S4) % kWave), ko = (int)(q / (S4 * kWave));
        const int g = lane / 16, el = lane % 16;
        v = W.w[k][(ko * 16 + el) * H + 16 * (j / 4) + drow<T>(g, j % 4)];
      }
    } else {
      const int64_t q = i - L.b0;
      if (q < (int64_t)kWave * S4) {
        const int j = (int)(q % S4), lane = (int)(q / S4);
        const int g = lane / 16, el = lane % 16;
        if (el < 8) v = W.w[0][el * H + 16 * (j / 4) + drow<T>(g, j % 4)];
      }
    }
    pk[i] = v;
  }
}

// The split-bf16 section fs (float32 weights only): A operand of R = a W_L
// for column block blk, lane (g, el), reduction block kb, part, step j =
// hidden feature 32 kb + 16 (j / 4) + 4 g + j % 4.
__global__ void __launch_bounds__(256) k_radial_pack_x6(RadialPack L, const float* __restrict__ WL,
                                                      __bf16* __restrict__ fs, __bf16* __restrict__ bs) {
  const int KB = L.H / 32, NB = L.H / 16, pc = L.pc;
  const int64_t nfs = (int64_t)L.nblk * kWave * KB * 24;
  const int64_t nbs = (int64_t)(pc / 32) * kWave * NB * 24;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nfs + nbs;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool fwd = i < nfs;
    const int64_t q = fwd ? i : i - nfs;
    const int sub_n = fwd ? KB : NB;
    const int j = (int)(q % 8), part = (int)((q / 8) % 3);
    const int sub = (int)((q / 24) % sub_n);
    const int lane = (int)((q / (24 * sub_n)) % kWave);
    const int64_t blk = q / (24 * (int64_t)sub_n * kWave);
    const int g = lane / 16, el = lane % 16;
    float w;
    if (fwd) {
      // A operand of R = a W_L: column 16 blk + el, reduction step (sub, j)
      const int64_t col = blk * 16 + el;
      const int k = 32 * sub + 16 * (j / 4) + 4 * g + j % 4;
      w = col < pc ? WL[(int64_t)k * pc + col] : 0.f;
    } else {
      // A operand of dA = dR W_L^T: hidden feature 16 sub + el, reduction
      // step (g, j) of block blk = column 32 blk + 8 g + j
      w = WL[(int64_t)(16 * sub + el) * pc + 32 * blk + 8 * g + j];
    }
    __bf16 p[3];
    split3(w, p[0], p[1], p[2]);
    (fwd ? fs : bs)[q] = p[part];
  }
}

// First layer (K = 8, two reduction steps with k = 4*s + g) for S strips;
// pre-activations into z.
template <typename T, int H, int S>
__device__ __forceinline__ void layer0(int64_t e0, int64_t ne, int lane, const T* __restrict__ ef,
                                       const T* __restrict__ w0, T (&z)[S][H / 16][4]) {
  constexpr int NB = H / 16;
  const int g = lane / 16, el = lane % 16;
  T b[S][2];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    int64_t e = e0 + st * 16 + el;
    e = e < ne ? e : ne - 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) b[st][s] = ef[e * 8 + 4 * s + g];
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const T a0 = w0[(nb * kWave + lane) * 2], a1 = w0[(nb * kWave + lane) * 2 + 1];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      vec4<T> acc = mfma(a0, b[st][0], zero4<T>());
      acc = mfma(a1, b[st][1], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) z[st][nb][r] = acc[r];
    }
  }
}

// One H -> H layer: out = act W_k (pre-activation), weights in operand order.
template <typename T, int H, int S>
__device__ __forceinline__ void hidden(int lane, const T* __restrict__ wk, const T (&act)[S][H / 16][4],
                                       T (&out)[S][H / 16][4]) {
  constexpr int NB = H / 16, S4 = 4 * NB;
#pragma unroll
  for (int no = 0; no < NB; ++no) {
    vec4<T> w[NB];
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) w[ni] = ld4(wk + (no * kWave + lane) * S4 + 4 * ni);
    vec4<T> acc[S];
#pragma unroll
    for (int st = 0; st < S; ++st) acc[st] = zero4<T>();
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int st = 0; st < S; ++st) acc[st] = mfma(w[ni][r], act[st][ni][r], acc[st]);
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[st][no][r] = acc[st][r];
  }
}

// Last layer R = act W_L for S strips, one 16-column block at a time, with
// the next block's weights loading while the current block runs (the final
// prefetch of an even block count re-reads the last block, unused).  Lane
// (g, el) holds R[e0 + st*16 + el][cb*16 + row(g, r)].  Used for float64,
// for widths that are not a multiple of 32 and for the last, partial wave.
template <typename T, int H, int S, bool VEC, bool FULL>
__device__ __forceinline__ void radial_last(int64_t e0, int64_t ne, int pc, int lane,
                                            const T* __restrict__ wl, int nblk,
                                            const T (&act)[S][H / 16][4], T* __restrict__ R) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  const int g = lane / 16, el = lane % 16;
  wl += lane * S4;
  T* rowp[S];
#pragma unroll
  for (int st = 0; st < S; ++st) rowp[st] = R + (e0 + st * 16 + el) * (int64_t)pc;
  auto load = [&](int cb, vec4<T>(&w)[NB]) {
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) w[ni] = ld4(wl + (int64_t)cb * kWave * S4 + 4 * ni);
  };
  auto block = [&](int cb, const vec4<T>(&w)[NB]) {
    vec4<T> acc[S];
#pragma unroll
    for (int st = 0; st < S; ++st) acc[st] = zero4<T>();
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int st = 0; st < S; ++st) acc[st] = mfma(w[ni][r], act[st][ni][r], acc[st]);
#pragma unroll
    for (int st = 0; st < S; ++st) {
      if (!FULL && e0 + st * 16 + el >= ne) continue;
      T* dst = rowp[st] + cb * 16;
      if constexpr (VEC) {
        st4(dst + 4 * g, acc[st]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (cb * 16 + drow<T>(g, r) < pc) dst[drow<T>(g, r)] = acc[st][r];
      }
    }
  };
  vec4<T> wa[NB], wb[NB];
  load(0, wa);
  int cb = 0;
  for (; cb + 2 <= nblk; cb += 2) {
    load(cb + 1, wb);
    block(cb, wa);
    load(cb + 2 < nblk ? cb + 2 : nblk - 1, wa);
    block(cb + 1, wb);
  }
  if (cb < nblk) block(cb, wa);
}

// Rotate each 16-lane row of the wave by 8 lanes (DPP row_ror:8).
__device__ __forceinline__ float row_swap8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// Float32 last layer for full waves and widths that are a multiple of 32:
// column blocks go in pairs (one 128-byte line per row).  Before storing, the
// upper half of every 16-lane row of block c trades places with the lower
// half of block c+1, so lanes el < 8 hold the whole line of row el and the
// others the whole line of row el + 8 after the other store: every store
// writes 8 rows x 128 bytes.  R is written once and read much later, so the
// stores are non-temporal.
template <int H, int S>
__device__ __forceinline__ void radial_last_pairs(int64_t e0, int pc, int lane, const float* __restrict__ wl,
                                                  int nblk, const float (&act)[S][H / 16][4],
                                                  float* __restrict__ R) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  const int g = lane / 16, el = lane % 16;
  const bool lo = el < 8;
  wl += lane * S4;
  float* rowp[S];
#pragma unroll
  for (int st = 0; st < S; ++st)
    rowp[st] = R + (e0 + st * 16 + (el & 7)) * (int64_t)pc + (lo ? 0 : 16) + 4 * g;
  auto load = [&](int cb, f32x4(&w)[2][NB]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int ni = 0; ni < NB; ++ni) w[c][ni] = ld4(wl + (int64_t)(cb + c) * kWave * S4 + 4 * ni);
  };
  auto pair = [&](int cb, const f32x4(&w)[2][NB]) {
    f32x4 acc[2][S];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int st = 0; st < S; ++st) acc[c][st] = zero4<float>();
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int st = 0; st < S; ++st) acc[c][st] = mfma(w[c][ni][r], act[st][ni][r], acc[c][st]);
#pragma unroll
    for (int st = 0; st < S; ++st) {
      f32x4 X, Y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = acc[0][st][r], y = acc[1][st][r];
        const float xs = row_swap8(x), ys = row_swap8(y);
        X[r] = lo ? x : ys;
        Y[r] = lo ? xs : y;
      }
      float* dst = rowp[st] + cb * 16;
      __builtin_nontemporal_store(X, reinterpret_cast<f32x4*>(dst));
      __builtin_nontemporal_store(Y, reinterpret_cast<f32x4*>(dst + 8 * (int64_t)pc));
    }
  };
  const int np = nblk / 2;
  f32x4 wa[2][NB], wb[2][NB];
  load(0, wa);
  int q = 0;
  for (; q + 2 <= np; q += 2) {
    load(2 * (q + 1), wb);
    pair(2 * q, wa);
    load(2 * (q + 2 < np ? q + 2 : np - 1), wa);
    pair(2 * (q + 1), wb);
  }
  if (q < np) pair(2 * q, wa);
}

// ---------------------------------------------------------------------------
// forward
// As radial_last_pairs, with the products on the bf16 matrix cores (three-
// part split, six terms).  The activations a lane holds (features 16 nb +
// 4g + r of its edge) are exactly the B-operand values of the two 32-step
// reductions, taking step (kb, j) as feature 16 (2 kb + j / 4) + 4 g + j % 4;
// the packed weights (section fs) follow the same order and are split once
// per wave.
// The four waves of a block share the weights: each pair of column blocks
// (2 * 64 * KB * 24 bf16, contiguous in fs) is copied once into one of two
// LDS buffers while the previous pair is multiplied, with one barrier per
// pair.  The barrier waits for LDS traffic only, so the R stores stay in
// flight across it.  Every wave of the block runs every pair (barrier
// count); FULL = false serves the block holding the last edges (rows at or
// past ne are not stored), so every edge's weights come from the same
// arithmetic wherever the block boundaries fall.
template <int H>
constexpr int kX6Pair = 2 * kWave * (H / 32) * 24;  // bf16 per pair of column blocks
constexpr int kX6PairsPerTile = 2;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int H, int S, bool FULL>
__device__ __forceinline__ void radial_last_pairs_x6(int64_t e0, int64_t ne, int pc, int lane,
                                                     const __bf16* __restrict__ fs, int nblk,
                                                     const float (&act)[S][H / 16][4],
                                                     float* __restrict__ R, __bf16* wt) {
  constexpr int KB = H / 32, PAIR = kX6Pair<H>, TILE = kX6PairsPerTile * PAIR;
  constexpr int NCH = TILE / 8, CPT = (NCH + 255) / 256;  // 16-byte chunks: per tile, per thread
  const int np = nblk / 2;
  const int last_ch = np * (PAIR / 8) - 1;  // last chunk of fs
  const int g = lane / 16, el = lane % 16;
  const bool lo = el < 8;
  bf16x8 bx[S][KB][3];
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 p1, p2, p3;
        split3(act[st][2 * kb + j / 4][j % 4], p1, p2, p3);
        bx[st][kb][0][j] = p1;
        bx[st][kb][1][j] = p2;
        bx[st][kb][2][j] = p3;
      }
  float* rowp[S];
#pragma unroll
  for (int st = 0; st < S; ++st)
    rowp[st] = R + (e0 + st * 16 + (el & 7)) * (int64_t)pc + (lo ? 0 : 16) + 4 * g;
  // chunk indices past the tile or past fs are clamped: the spare threads
  // copy a chunk again (same value, same place), and a tile past the last
  // pair holds values no pair reads
  auto fetch = [&](int t, bf16x8(&pf)[CPT]) __attribute__((always_inline)) {
    const bf16x8* __restrict__ src = reinterpret_cast<const bf16x8*>(fs);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int ch = (int)threadIdx.x + 256 * i;
      ch = t * (TILE / 8) + (ch < NCH ? ch : NCH - 1);
      pf[i] = src[ch < last_ch ? ch : last_ch];
    }
  };
  auto put = [&](int buf, const bf16x8(&pf)[CPT]) __attribute__((always_inline)) {
    bf16x8* dst = reinterpret_cast<bf16x8*>(wt + buf * TILE);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = (int)threadIdx.x + 256 * i;
      dst[ch < NCH ? ch : NCH - 1] = pf[i];
    }
  };
  auto pair = [&](int q, const __bf16* tile) __attribute__((always_inline)) {
    const __bf16* wl = tile + (q % kX6PairsPerTile) * PAIR + lane * KB * 24;
    bf16x8 w[2][KB][3];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int pp = 0; pp < 3; ++pp)
          w[c][kb][pp] = *reinterpret_cast<const bf16x8*>(wl + c * kWave * KB * 24 + kb * 24 + pp * 8);
    f32x4 acc[2][S];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int st = 0; st < S; ++st) acc[c][st] = zero4<float>();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int st = 0; st < S; ++st) acc[c][st] = mfma_x6(w[c][kb], bx[st][kb], acc[c][st]);
#pragma unroll
    for (int st = 0; st < S; ++st) {
      f32x4 X, Y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = acc[0][st][r], y = acc[1][st][r];
        const float xs = row_swap8(x), ys = row_swap8(y);
        X[r] = lo ? x : ys;
        Y[r] = lo ? xs : y;
      }
      float* dst = rowp[st] + q * 32;
      const int64_t row = e0 + st * 16 + (el & 7);
      if (FULL || row < ne) __builtin_nontemporal_store(X, reinterpret_cast<f32x4*>(dst));
      if (FULL || row + 8 < ne) __builtin_nontemporal_store(Y, reinterpret_cast<f32x4*>(dst + 8 * (int64_t)pc));
    }
  };
  const int nt = (np + kX6PairsPerTile - 1) / kX6PairsPerTile;
  bf16x8 pf[CPT];
  fetch(0, pf);
  put(0, pf);
  lds_barrier();
  for (int t = 0; t < nt; ++t) {
    fetch(t + 1 < nt ? t + 1 : t, pf);  // the last round copies its own tile again, unused
    const __bf16* tile = wt + (t & 1) * TILE;
#pragma unroll
    for (int h = 0; h < kX6PairsPerTile; ++h) {
      const int q = t * kX6PairsPerTile + h;
      if (h == 0 || q < np) pair(q, tile);
    }
    put((t + 1) & 1, pf);
    lds_barrier();
  }
}

// VEC: 16-byte stores of whole 16-column blocks (float32, width a multiple
// of 16); PAIRS: width also a multiple of 32, full waves use the paired
// line-wide stores.
// X6: float32 last layer as bf16-split products (off: float32 matrix cores).
// The split kernel at H = 64 asks for three waves per SIMD (at most 168
// registers, from 212; a few spill outside the block loop): the third wave
// overlaps more R stores with the products, 2-3 % faster on both large
// systems measured.
template <typename T, int H, int NH, int S, bool VEC, bool PAIRS, bool X6>
__global__ void __launch_bounds__(256, (sizeof(T) == 4 && X6 && H == 64) ? 3 : 1)
k_radial_fwd(int64_t ne, const int32_t* __restrict__ ne_dev, int pc, const T* __restrict__ ef,
             const T* __restrict__ pk, RadialPack L, T* __restrict__ R) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  const int lane = threadIdx.x % kWave;
  // rows counted on the device (shared rows of edge pairs): the grid covers
  // the largest count, and blocks past the actual one leave at once (every
  // wave of such a block, so no barrier below waits for them)
  if (ne_dev) {
    const int64_t nd = __builtin_amdgcn_readfirstlane(*ne_dev);
    ne = nd < ne ? nd : ne;
    if (blockIdx.x * (int64_t)(blockDim.x / kWave) * (16 * S) >= ne) return;
  }
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  // the shared-weight path keeps waves without edges for its barriers
  constexpr bool kX6 = X6 && PAIRS && x6_shape(H, 32);
  if (!kX6 && e0 >= ne) return;

  T act[S][NB][4];
  layer0<T, H, S>(e0 < ne ? e0 : ne - 1, ne, lane, ef, pk + L.f0, act);
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<T>(act[st][nb][r]);
#pragma unroll
  for (int layer = 1; layer < NH; ++layer) {
    T z[S][NB][4];
    hidden<T, H, S>(lane, pk + L.fh + (int64_t)(layer - 1) * NB * kWave * S4, act, z);
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<T>(z[st][nb][r]);
  }

  // Full waves store without tests, so the wait before each block covers only
  // that block's weight loads and never stores still in flight; the last,
  // partial wave checks each row.
  if constexpr (kX6) {
    __shared__ __attribute__((aligned(16))) __bf16 wt[2 * kX6PairsPerTile * kX6Pair<H>];
    const __bf16* fs = reinterpret_cast<const __bf16*>(pk + L.fs);
    const int64_t b_end = (blockIdx.x + 1) * (int64_t)(blockDim.x / kWave) * (16 * S);
    if (b_end <= ne)
      radial_last_pairs_x6<H, S, true>(e0, ne, pc, lane, fs, L.nblk, act, R, wt);
    else
      radial_last_pairs_x6<H, S, false>(e0, ne, pc, lane, fs, L.nblk, act, R, wt);
  } else if (e0 + 16 * S <= ne) {
    if constexpr (PAIRS)
      radial_last_pairs<H, S>(e0, pc, lane, pk + L.fl, L.nblk, act, R);
    else
      radial_last<T, H, S, VEC, true>(e0, ne, pc, lane, pk + L.fl, L.nblk, act, R);
  } else {
    radial_last<T, H, S, VEC, false>(e0, ne, pc, lane, pk + L.fl, L.nblk, act, R);
  }
}

// The last hidden activations only (float32, H a multiple of 32), for the
// forward that fuses the last layer into the tensor product: each activation
// is split into three bf16 parts and stored in that kernel's A-operand order,
//   act[e][kb][g][part][j] = part `part` of a[e][32 kb + 16 (j / 4) + 4 g + j % 4]
// (the reduction order of the packed last-layer weights, section fs), so a
// lane of that kernel reads its operand as three 16-byte vectors.  The lane
// that computed an edge's activations holds exactly the features of k-slot g.
template <int H, int NH, int S>
__global__ void __launch_bounds__(256)
k_radial_act(int64_t ne, const float* __restrict__ ef, const float* __restrict__ pk, RadialPack L,
             __bf16* __restrict__ act_out) {
  constexpr int NB = H / 16, S4 = 4 * NB, KB = H / 32;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  if (e0 >= ne) return;
  float act[S][NB][4];
  layer0<float, H, S>(e0, ne, lane, ef, pk + L.f0, act);
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<float>(act[st][nb][r]);
#pragma unroll
  for (int layer = 1; layer < NH; ++layer) {
    float z[S][NB][4];
    hidden<float, H, S>(lane, pk + L.fh + (int64_t)(layer - 1) * NB * kWave * S4, act, z);
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<float>(z[st][nb][r]);
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t e = e0 + st * 16 + el;
    if (e >= ne) continue;
    bf16x8* dst = reinterpret_cast<bf16x8*>(act_out + e * (KB * 96)) + g * 3;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8 v[3];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 p1, p2, p3;
        split3(act[st][2 * kb + j / 4][j % 4], p1, p2, p3);
        v[0][j] = p1;
        v[1][j] = p2;
        v[2][j] = p3;
      }
#pragma unroll
      for (int part = 0; part < 3; ++part) dst[kb * 12 + part] = v[part];
    }
  }
}

// ---------------------------------------------------------------------------
// backward, part 1: dA[e][k] = sum_n dR[e][n] W_L[k][n].  Reduction step
// (t, r), k-slot g covers n = 16t + 4g + r, so a lane reads four consecutive
// dR values per strip and step block.  Output in register order per strip:
// dA3[strip][lane][NB*4].
template <typename T, int H, int S, bool VEC>
__global__ void __launch_bounds__(256)
k_radial_bwd_dA(int64_t ne, int pc, const T* __restrict__ dR, const T* __restrict__ pk,
                RadialPack L, T* __restrict__ dA3) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  if (e0 >= ne) return;

  // rows past the end read the last row: their columns of the product are
  // never stored, and every other column is independent of them
  const T* __restrict__ rowp[S];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    int64_t e = e0 + st * 16 + el;
    e = e < ne ? e : ne - 1;
    rowp[st] = dR + e * (int64_t)pc + 4 * g;
  }
  const T* __restrict__ wq = pk + L.bl + lane * S4;
  const int nt = L.nblk;

  vec4<T> dA[S][NB];
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) dA[st][kb] = zero4<T>();

  // CB step blocks per stage: with two, a row's 128-byte line is read by two
  // back-to-back loads
  constexpr int CB = VEC ? 2 : 1;
  auto load = [&](int t, vec4<T>(&bv)[CB][S], vec4<T>(&wv)[CB][NB]) {
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        if constexpr (VEC) {
          bv[c][st] = ld4(rowp[st] + 16 * (t + c));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            bv[c][st][r] = (16 * (t + c) + 4 * g + r < pc) ? rowp[st][16 * (t + c) + r] : T(0);
        }
      }
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) wv[c][kb] = ld4(wq + (int64_t)(t + c) * kWave * S4 + 4 * kb);
  };
  auto step = [&](const vec4<T>(&bv)[CB][S], const vec4<T>(&wv)[CB][NB]) {
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int st = 0; st < S; ++st) dA[st][kb] = mfma(wv[c][kb][r], bv[c][st][r], dA[st][kb]);
  };
  const int nst = nt / CB;
  vec4<T> ba[CB][S], bb[CB][S], wa[CB][NB], wb[CB][NB];
  int q = 0;
  if (nst > 0) {
    load(0, ba, wa);
    for (; q + 2 <= nst; q += 2) {
      load((q + 1) * CB, bb, wb);
      step(ba, wa);
      load((q + 2 < nst ? q + 2 : nst - 1) * CB, ba, wa);
      step(bb, wb);
    }
    if (q < nst) step(ba, wa);
  }
  if constexpr (CB > 1) {
    if (nst * CB < nt) {  // odd block count: the last block alone
      vec4<T> b1[1][S], w1[1][NB];
#pragma unroll
      for (int st = 0; st < S; ++st) b1[0][st] = ld4(rowp[st] + 16 * (nt - 1));
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) w1[0][kb] = ld4(wq + (int64_t)(nt - 1) * kWave * S4 + 4 * kb);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int st = 0; st < S; ++st) dA[st][kb] = mfma(w1[0][kb][r], b1[0][st][r], dA[st][kb]);
    }
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t strip = e0 / 16 + st;
    if (strip * 16 >= ne) continue;
    T* dst = dA3 + (strip * kWave + lane) * S4;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) st4(dst + 4 * kb, dA[st][kb]);
  }
}

// backward, part 1 on the bf16 matrix cores (float32, width and hidden size
// multiples of 32): dA = dR W_L^T with both operands split in three bf16
// parts.  Reduction step (q, g, j) covers column n = 32 q + 8 g + j, so a
// lane reads eight consecutive dR values of its row per step (two 16-byte
// loads; the four lanes of a row cover one 128-byte line) and splits them in
// registers, one step ahead of its products.  The weights (section bs,
// pre-split in the same order, 64 * NB * 24 bf16 per step) are shared by the
// block's four waves through LDS as in the forward: two steps per tile (the
// step count pc / 32 must be even), the next tile copied while the current
// one is used, one barrier per tile.
// Every wave runs every step (barrier count); rows past the end read the last
// row and their strips are not stored.  Output as the float32 kernel.
template <int H, int S>
__global__ void __launch_bounds__(256)
k_radial_bwd_dA_x6(int64_t ne, int pc, const float* __restrict__ dR, const __bf16* __restrict__ bs,
                   float* __restrict__ dA3) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  constexpr int STEP = kWave * NB * 24, TS = 2, TILE = TS * STEP;
  constexpr int NCH = TILE / 8, CPT = (NCH + 255) / 256;  // 16-byte chunks: per tile, per thread
  __shared__ __attribute__((aligned(16))) __bf16 wt[2 * TILE];
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  const float* __restrict__ rowp[S];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    int64_t e = e0 + st * 16 + el;
    e = e < ne ? e : ne - 1;
    rowp[st] = dR + e * (int64_t)pc + 8 * g;
  }
  const int ns = pc / 32, ntile = ns / TS;
  const int last_ch = ns * (STEP / 8) - 1;
  f32x4 dA[S][NB];
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) dA[st][kb] = zero4<float>();
  auto fetch = [&](int t, bf16x8(&pf)[CPT]) __attribute__((always_inline)) {
    const bf16x8* __restrict__ src = reinterpret_cast<const bf16x8*>(bs);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int ch = (int)threadIdx.x + 256 * i;
      ch = t * (TILE / 8) + (ch < NCH ? ch : NCH - 1);
      pf[i] = src[ch < last_ch ? ch : last_ch];
    }
  };
  auto put = [&](int buf, const bf16x8(&pf)[CPT]) __attribute__((always_inline)) {
    bf16x8* dst = reinterpret_cast<bf16x8*>(wt + buf * TILE);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = (int)threadIdx.x + 256 * i;
      dst[ch < NCH ? ch : NCH - 1] = pf[i];
    }
  };
  auto load = [&](int q, f32x4(&bv)[S][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      bv[st][0] = ld4(rowp[st] + 32 * q);
      bv[st][1] = ld4(rowp[st] + 32 * q + 4);
    }
  };
  auto step = [&](const __bf16* w, const f32x4(&bv)[S][2]) __attribute__((always_inline)) {
    bf16x8 wv[NB][3];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) wv[kb][pp] = *reinterpret_cast<const bf16x8*>(w + kb * 24 + pp * 8);
    bf16x8 bx[S][3];
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 p1, p2, p3;
        split3(bv[st][j / 4][j % 4], p1, p2, p3);
        bx[st][0][j] = p1;
        bx[st][1][j] = p2;
        bx[st][2][j] = p3;
      }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int st = 0; st < S; ++st) dA[st][kb] = mfma_x6(wv[kb], bx[st], dA[st][kb]);
  };
  bf16x8 pf[CPT];
  f32x4 ba[S][2], bb[S][2];
  fetch(0, pf);
  put(0, pf);
  load(0, ba);
  lds_barrier();
  for (int t = 0; t < ntile; ++t) {
    fetch(t + 1 < ntile ? t + 1 : t, pf);  // the last round copies its own tile again, unused
    const __bf16* tile = wt + (t & 1) * TILE + lane * NB * 24;
    const int q = TS * t;
    load(q + 1, bb);
    // keep the scheduler from sinking the loads into the products
    __builtin_amdgcn_sched_barrier(0);
    step(tile, ba);
    load(q + 2 < ns ? q + 2 : ns - 1, ba);  // the last step reloads its own row part, unused
    __builtin_amdgcn_sched_barrier(0);
    step(tile + STEP, bb);
    put((t + 1) & 1, pf);
    lds_barrier();
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t strip = e0 / 16 + st;
    if (strip * 16 >= ne) continue;
    float* dst = dA3 + (strip * kWave + lane) * S4;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) st4(dst + 4 * kb, dA[st][kb]);
  }
}

// backward, part 2: recompute the hidden layers, then d(ef) from dA3.
// Float32 asks for two waves per SIMD (at most 256 registers): left free, the
// compiler gave the two-hidden-layer network 260 (accumulator copies) and so
// one wave per SIMD; bounded, it takes 156 with no spills.
template <typename T, int H, int NH, int S>
__global__ void __launch_bounds__(256, sizeof(T) == 4 ? 2 : 1)
k_radial_bwd_mlp(int64_t ne, const T* __restrict__ ef, const T* __restrict__ dA3,
                 const T* __restrict__ pk, RadialPack L, T* __restrict__ d_ef) {
  constexpr int NB = H / 16, S4 = 4 * NB;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, el = lane % 16;
  const int64_t e0 = (blockIdx.x * (int64_t)(blockDim.x / kWave) + threadIdx.x / kWave) * (16 * S);
  if (e0 >= ne) return;

  T z[NH][S][NB][4];
  layer0<T, H, S>(e0, ne, lane, ef, pk + L.f0, z[0]);
#pragma unroll
  for (int layer = 1; layer < NH; ++layer) {
    T act[S][NB][4];
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) act[st][nb][r] = silu<T>(z[layer - 1][st][nb][r]);
    hidden<T, H, S>(lane, pk + L.fh + (int64_t)(layer - 1) * NB * kWave * S4, act, z[layer]);
  }

  vec4<T> dA[S][NB];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int64_t strip = e0 / 16 + st;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
      dA[st][kb] = strip * 16 < ne ? ld4(dA3 + (strip * kWave + lane) * S4 + 4 * kb) : zero4<T>();
  }
#pragma unroll
  for (int layer = NH - 1; layer >= 0; --layer) {
    T dz[S][NB][4];
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dz[st][kb][r] = dA[st][kb][r] * silu_dz<T>(z[layer][st][kb][r]);
    if (layer > 0) {
      // dA_prev[e][k'] = sum_k W_k[k'][k] dz[e][k]
      T nxt[S][NB][4];
      hidden<T, H, S>(lane, pk + L.bh + (int64_t)(layer - 1) * NB * kWave * S4, dz, nxt);
#pragma unroll
      for (int st = 0; st < S; ++st)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) dA[st][kb][r] = nxt[st][kb][r];
    } else {
      // d(ef)[e][k'] for k' < 8 (rows 8..15 of the tile carry zero weights)
      const T* __restrict__ w = pk + L.b0 + lane * S4;
      vec4<T> wv[NB];
#pragma unroll
      for (int ni = 0; ni < NB; ++ni) wv[ni] = ld4(w + 4 * ni);
      vec4<T> acc[S];
#pragma unroll
      for (int st = 0; st < S; ++st) acc[st] = zero4<T>();
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int st = 0; st < S; ++st) acc[st] = mfma(wv[ni][r], dz[st][ni][r], acc[st]);
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

constexpr int kFwdStrips = 3, kMlpStrips = 2;
// the backward product keeps only its accumulators live: 8 strips of 16
// edges in float32 (128 accumulator registers), 2 in float64
template <typename T>
constexpr int kBwdStrips = std::is_same<T, float>::value ? 8 : 2;

template <typename T, int H, int NH>
hipError_t fwd_impl(int64_t ne, const int32_t* ne_dev, int pc, const T* ef, const T* pk, const RadialPack& L,
                    T* R, hipStream_t s) {
  const int64_t per_block = 4 * 16 * kFwdStrips;
  const unsigned blocks = (unsigned)((ne + per_block - 1) / per_block);
  const bool vec = std::is_same<T, float>::value && pc % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(R) % 16 == 0;
  if constexpr (std::is_same<T, float>::value) {
    if (vec && pc % 32 == 0) {
      if (L.x6)
        k_radial_fwd<T, H, NH, kFwdStrips, true, true, true><<<blocks, 256, 0, s>>>(ne, ne_dev, pc, ef, pk, L, R);
      else
        k_radial_fwd<T, H, NH, kFwdStrips, true, true, false><<<blocks, 256, 0, s>>>(ne, ne_dev, pc, ef, pk, L, R);
      return hipGetLastError();
    }
  }
  if (vec)
    k_radial_fwd<T, H, NH, kFwdStrips, true, false, false><<<blocks, 256, 0, s>>>(ne, ne_dev, pc, ef, pk, L, R);
  else
    k_radial_fwd<T, H, NH, kFwdStrips, false, false, false><<<blocks, 256, 0, s>>>(ne, ne_dev, pc, ef, pk, L, R);
  return hipGetLastError();
}

// float32 backward on bf16 matrix cores: strips of 16 edges per wave
constexpr int kBwdStripsX6 = 3;

template <typename T, int H>
hipError_t bwd_dA_impl(int64_t ne, int pc, const T* dR, const T* pk, const RadialPack& L, T* dA3,
                       hipStream_t s) {
  if constexpr (std::is_same<T, float>::value && x6_shape(H, 32)) {
    if (L.x6 && x6_shape(H, pc) && pc % 64 == 0 && reinterpret_cast<uintptr_t>(dR) % 16 == 0) {
      const int64_t per_block = 4 * 16 * kBwdStripsX6;
      const __bf16* bs = reinterpret_cast<const __bf16*>(pk + L.bs);
      k_radial_bwd_dA_x6<H, kBwdStripsX6><<<(unsigned)((ne + per_block - 1) / per_block), 256, 0, s>>>(
          ne, pc, dR, bs, dA3);
      return hipGetLastError();
    }
  }
  const int64_t per_block = 4 * 16 * kBwdStrips<T>;
  const unsigned blocks = (unsigned)((ne + per_block - 1) / per_block);
  // the vector path reads whole 16-column blocks of every row
  const bool vec = pc % 16 == 0 && reinterpret_cast<uintptr_t>(dR) % 16 == 0;
  if (vec)
    k_radial_bwd_dA<T, H, kBwdStrips<T>, true><<<blocks, 256, 0, s>>>(ne, pc, dR, pk, L, dA3);
  else
    k_radial_bwd_dA<T, H, kBwdStrips<T>, false><<<blocks, 256, 0, s>>>(ne, pc, dR, pk, L, dA3);
  return hipGetLastError();
}

template <typename T, int H, int NH>
hipError_t bwd_mlp_impl(int64_t ne, const T* ef, const T* dA3, const T* pk, const RadialPack& L,
                        T* d_ef, hipStream_t s) {
  const int64_t per_block = 4 * 16 * kMlpStrips;
  k_radial_bwd_mlp<T, H, NH, kMlpStrips><<<(unsigned)((ne + per_block - 1) / per_block), 256, 0, s>>>(
      ne, ef, dA3, pk, L, d_ef);
  return hipGetLastError();
}

#define TPC_RADIAL_SHAPES(X) X(16, 1) X(16, 2) X(16, 3) X(32, 1) X(32, 2) X(32, 3) X(64, 1) X(64, 2) X(64, 3)

template <typename T>
hipError_t fwd_dispatch(const RadialPack& L, int64_t ne, const int32_t* ne_dev, const void* ef, const void* pk,
                        void* R, hipStream_t s) {
#define TPC_CASE(HH, NN)                                                                              \
  if (L.H == HH && L.NH == NN)                                                                        \
    return fwd_impl<T, HH, NN>(ne, ne_dev, L.pc, static_cast<const T*>(ef), static_cast<const T*>(pk), L, \
                               static_cast<T*>(R), s);
  TPC_RADIAL_SHAPES(TPC_CASE)
#undef TPC_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t bwd_dA_dispatch(const RadialPack& L, int64_t ne, const void* dR, const void* pk, void* dA3,
                           hipStream_t s) {
  const T* d = static_cast<const T*>(dR);
  const T* p = static_cast<const T*>(pk);
  T* o = static_cast<T*>(dA3);
  if (L.H == 16) return bwd_dA_impl<T, 16>(ne, L.pc, d, p, L, o, s);
  if (L.H == 32) return bwd_dA_impl<T, 32>(ne, L.pc, d, p, L, o, s);
  if (L.H == 64) return bwd_dA_impl<T, 64>(ne, L.pc, d, p, L, o, s);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t bwd_mlp_dispatch(const RadialPack& L, int64_t ne, const void* ef, const void* dA3,
                            const void* pk, void* d_ef, hipStream_t s) {
#define TPC_CASE(HH, NN)                                                                  \
  if (L.H == HH && L.NH == NN)                                                            \
    return bwd_mlp_impl<T, HH, NN>(ne, static_cast<const T*>(ef), static_cast<const T*>(dA3), \
                                   static_cast<const T*>(pk), L, static_cast<T*>(d_ef), s);
  TPC_RADIAL_SHAPES(TPC_CASE)
#undef TPC_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t pack_impl(const RadialPack& L, const void* const* w, void* pk, hipStream_t s) {
  RadialWeights<T> W{};
  for (int k = 0; k <= L.NH; ++k) W.w[k] = static_cast<const T*>(w[k]);
  const int64_t blocks = (L.total + 255) / 256;
  k_radial_pack<T><<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>(L, W, static_cast<T*>(pk));
  if constexpr (std::is_same<T, float>::value) {
    if (L.x6 && x6_shape(L.H, L.pc)) {
      float* base = static_cast<float*>(pk);
      k_radial_pack_x6<<<1024, 256, 0, s>>>(L, W.w[L.NH], reinterpret_cast<__bf16*>(base + L.fs),
                                            reinterpret_cast<__bf16*>(base + L.bs));
    }
  }
  return hipGetLastError();
}

}  // namespace

bool radial_supported(int H, int NH) {
  return (H == 16 || H == 32 || H == 64) && NH >= 1 && NH <= 3;
}

hipError_t launch_radial_pack(int dtype, const RadialPack& L, const void* const* w, void* pk,
                              hipStream_t s) {
  return dtype == 1 ? pack_impl<double>(L, w, pk, s) : pack_impl<float>(L, w, pk, s);
}

hipError_t launch_radial_fwd(int dtype, const RadialPack& L, int64_t ne, const int32_t* ne_dev,
                             const void* ef, const void* pk, void* R, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  return dtype == 1 ? fwd_dispatch<double>(L, ne, ne_dev, ef, pk, R, s)
                    : fwd_dispatch<float>(L, ne, ne_dev, ef, pk, R, s);
}

hipError_t launch_radial_act(const RadialPack& L, int64_t ne, const void* ef, const void* pk, void* act,
                             hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  const int64_t per_block = 4 * 16 * kFwdStrips;
  const unsigned blocks = (unsigned)((ne + per_block - 1) / per_block);
  const float* e = static_cast<const float*>(ef);
  const float* p = static_cast<const float*>(pk);
  __bf16* o = static_cast<__bf16*>(act);
#define TPC_CASE(HH, NN)                                                                   \
  if (L.H == HH && L.NH == NN) {                                                           \
    k_radial_act<HH, NN, kFwdStrips><<<blocks, 256, 0, s>>>(ne, e, p, L, o);                \
    return hipGetLastError();                                                              \
  }
  TPC_CASE(32, 1) TPC_CASE(32, 2) TPC_CASE(32, 3) TPC_CASE(64, 1) TPC_CASE(64, 2) TPC_CASE(64, 3)
#undef TPC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_radial_bwd_dA(int dtype, const RadialPack& L, int64_t ne, const void* dR,
                                const void* pk, void* dA3, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  return dtype == 1 ? bwd_dA_dispatch<double>(L, ne, dR, pk, dA3, s)
                    : bwd_dA_dispatch<float>(L, ne, dR, pk, dA3, s);
}

hipError_t launch_radial_bwd_mlp(int dtype, const RadialPack& L, int64_t ne, const void* ef,
                                 const void* dA3, const void* pk, void* d_ef, hipStream_t s) {
  if (ne <= 0) return hipSuccess;
  return dtype == 1 ? bwd_mlp_dispatch<double>(L, ne, ef, dA3, pk, d_ef, s)
                    : bwd_mlp_dispatch<float>(L, ne, ef, dA3, pk, d_ef, s);
}

}  // namespace tpc
