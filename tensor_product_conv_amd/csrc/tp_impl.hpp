// Fused gather + sparse-coupling tensor product + receiver reduction (gfx950).
//
// Forward (FlashCart paper, section 2 "Equivariant convolution and many-body
// correlations"; section 4 receiver-sorted kernel):
//   out[i,(p,m3),u] = s * sum_{e in row i} R[e,p,u] * sum_{m1} M_e^p[m1,m3] h[src_e,(l1,m1),u]
//   M_e^p[m1,m3]   = sum_{m2} C^p[m1,m2,m3] Y[e,(l2,m2)]
// The coupling coefficients are compile-time constants (tables.hpp), so the
// sparse contraction is straight-line code; an edge's harmonics sit in scalar
// registers and M is formed per edge from them.  A receiver row is owned by
// NG waves, each holding the accumulators of a fixed subset of paths for 64
// lanes x CPL channels.  The edge loop runs in CSR order with the next edge's
// radial weights and sender features loading while the current edge is
// computed, so every output is a fixed-order sum held in registers and stored
// once: no atomics and no per-edge message tensor (the receiver-streaming
// design of FastMACE's "streaming_conv" and FlashCart's receiver-sorted
// kernel, on a 64-wide wave).
//
// Backward of L = sum(G * out) (FlashCart section 3 "Symbolic derivatives":
// the weight gradient is the inner product of the incoming gradient with the
// unweighted product; the input gradients are the other factors times the
// weight).  One wave per receiver row and 64 channels loads G[i] once per row;
// per edge and path it forms K[m1][m2] = sum_m3 C^p[m1,m2,m3] G[i,(p,m3),u] and
// from it
//     W[m1]  = sum_m2 Y[e,(l2,m2)] K[m1][m2]
//     dR[e,p,u] = s * sum_m1 h[src_e,m1,u] W[m1]
//     t[m1]  += R[e,p,u] W[m1]                 (contribution to dh of the sender)
//     Q[m2]  = sum_m1 h[src_e,m1,u] K[m1][m2]
//     dY[e,(l2,m2)] = s * sum_u R[e,p,u] Q[m2]  (channel reduction)
// The channel reduction of dY is a wave reduce-scatter; with several waves per
// row each writes its partial sum and the geometry backward adds them in a
// fixed order.  The sender contribution t is stored at the reverse edge's
// slot: the list is symmetric, and the reverse of e = (i <- j, S) is
// (j <- i, -S) in row j.  k_dh_gather then sums row j in CSR order,
//     dh[j] = s * sum_{e in row j} t_stored[e],
// so sender gradients are gathered per row instead of scattered with atomics
// (FlashCart's VJP uses atomics there) or through a sender permutation.
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "tables.hpp"

namespace tpc {

constexpr int kTPWave = 64;
constexpr int kTPWavesPerBlock = 4;

// NW = waves per row: C = 64 * NW channels, one per lane; NW = 0 stands for
// C < 64 (lanes beyond C masked).  Loads take a wave-uniform base pointer and
// a 32-bit lane offset so they use the scalar-base addressing form.
template <int NW, typename T>
__device__ __forceinline__ T ldc(const T* __restrict__ base, uint32_t off, bool on) {
  if constexpr (NW > 0) {
    return base[off];
  } else {
    return on ? base[off] : T(0);
  }
}

template <int NW, typename T>
__device__ __forceinline__ void stc(T* __restrict__ base, uint32_t off, bool on, T v) {
  if constexpr (NW > 0) {
    base[off] = v;
  } else {
    if (on) base[off] = v;
  }
}

// Streams touched once (R, dR, the per-edge dh contributions) go through
// non-temporal accesses, so they displace less of the sender features that
// the gathers of neighbouring rows reuse from L2.
template <int NW, typename T>
__device__ __forceinline__ T ldc_nt(const T* __restrict__ base, uint32_t off, bool on) {
  if constexpr (NW > 0) {
    return __builtin_nontemporal_load(base + off);
  } else {
    return on ? __builtin_nontemporal_load(base + off) : T(0);
  }
}

template <int NW, typename T>
__device__ __forceinline__ void stc_nt(T* __restrict__ base, uint32_t off, bool on, T v) {
  if constexpr (NW > 0) {
    __builtin_nontemporal_store(v, base + off);
  } else {
    if (on) __builtin_nontemporal_store(v, base + off);
  }
}

// Value held by lane k of v, for every lane (v_readlane; k is uniform).
__device__ __forceinline__ float lane_value(float v, int k) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k));
}
__device__ __forceinline__ double lane_value(double v, int k) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), k);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Rows of at most 64 * kIdxWindows edges keep their sender (and reverse-edge)
// indices in registers: lane k of window q holds a[e_lo + 64 q + k], and an
// edge's index is a v_readlane away instead of a dependent memory load.
// Longer rows take a separate loop that loads each index.
constexpr int kIdxWindows = 2;

template <int NWIN>
struct RowIdx {
  int v[NWIN];
  __device__ __forceinline__ void init(const int32_t* __restrict__ a, int e_lo, int e_hi, int lane) {
#pragma unroll
    for (int q = 0; q < NWIN; ++q) v[q] = a[min(e_lo + 64 * q + lane, e_hi - 1)];
  }
  // entry of edge e_lo + k (k uniform, 0 <= k < 64 * NWIN)
  __device__ __forceinline__ int get(int k) const {
    int r = __builtin_amdgcn_readlane(v[0], k & 63);
#pragma unroll
    for (int q = 1; q < NWIN; ++q) {
      const int t = __builtin_amdgcn_readlane(v[q], k & 63);
      r = (k >> 6) == q ? t : r;
    }
    return r;
  }
};

// compute(e, buf) over the edges [e_lo, e_hi) (non-empty) in order, with the
// next edge's loads in flight in a second buffer.  Every prefetch is
// unconditional (the index is clamped; the final one re-reads the last edge,
// unused) and the loop has a single exit, so the wait before each edge covers
// exactly that edge's loads and never the stores issued since.
template <typename Buf, typename Load, typename Compute>
__device__ __forceinline__ void edge_loop(int e_lo, int e_hi, Load&& load, Compute&& compute) {
  Buf A, B;
  load(e_lo, A);
  int e = e_lo;
  for (; e + 2 <= e_hi; e += 2) {
    load(e + 1, B);
    compute(e, A);
    load(min(e + 2, e_hi - 1), A);
    compute(e + 1, B);
  }
  if (e < e_hi) compute(e, A);
}

template <int NW>
__device__ __forceinline__ int channels(int C) {
  if constexpr (NW > 0) {
    return 64 * NW;
  } else {
    return C;
  }
}

// Coupling-matrix row of one edge from its harmonics (compile-time sparsity).
template <typename T, int L1, int L2, int L3>
__device__ __forceinline__ void coupling_row(const T* y, T* out) {
  static_for<kTable<L1, L2, L3>.np>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr Path P = kTable<L1, L2, L3>.path[p];
    static_for<2 * P.l3 + 1>([&](auto m3c) {
      constexpr int m3 = decltype(m3c)::value;
      static_for<2 * P.l1 + 1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        constexpr int k = kTable<L1, L2, L3>.midx[p][m1][m3];
        if constexpr (k >= 0) {
          T M = T(0);
          static_for<2 * P.l2 + 1>([&](auto m2c) {
            constexpr int m2 = decltype(m2c)::value;
            constexpr double cv = kTable<L1, L2, L3>.cg[p][m1][m2][m3];
            if constexpr (cv != 0.0) M += T(cv) * y[P.l2 * P.l2 + m2];
          });
          out[k] = M;
        }
      });
    });
  });
}

struct RowWave {
  int row;   // receiver (or atom) index
  int c0;    // this lane's channel
  bool on;   // c0 < C
  bool ok;   // the wave has a row to process
};

template <int NW>
__device__ __forceinline__ RowWave row_wave(int64_t row_begin, int64_t row_end, int C) {
  const int lane = threadIdx.x % kTPWave;
  const int wpr = NW > 0 ? NW : 1;  // waves per row
  const int64_t w = xcd_block() * kTPWavesPerBlock + threadIdx.x / kTPWave;
  RowWave r;
  const int64_t row = row_begin + w / wpr;
  r.ok = row < row_end;
  r.row = uniform((int)(r.ok ? row : row_begin));
  r.c0 = (int)(w % wpr) * kTPWave + lane;
  r.on = r.c0 < C;
  return r;
}

// ---------------------------------------------------------------------------
// Forward.  NG * NWC waves share a receiver row: NWC channel slices of
// 64 * CPL channels, and in each slice NG waves that own compile-time subsets
// of the paths (kGroups; the per-edge coupling matrices of a path are
// computed by one wave of the slice, from the edge's harmonics broadcast
// from one vector load).  Lanes own CPL consecutive channels; MASKED kernels
// serve C < 64 with one channel per lane.
template <typename T, int CPL>
__device__ __forceinline__ void ld_vec(const T* __restrict__ base, uint32_t off, bool on, T (&v)[CPL],
                                       bool masked) {
  if constexpr (CPL == 1) {
    v[0] = (!masked || on) ? base[off] : T(0);
  } else {
    using V = T __attribute__((ext_vector_type(CPL)));
    const V x = *reinterpret_cast<const V*>(base + off);
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = x[c];
  }
}

template <typename T, int CPL>
__device__ __forceinline__ void ld_vec_nt(const T* __restrict__ base, uint32_t off, bool on, T (&v)[CPL],
                                          bool masked) {
  if constexpr (CPL == 1) {
    v[0] = (!masked || on) ? __builtin_nontemporal_load(base + off) : T(0);
  } else {
    using V = T __attribute__((ext_vector_type(CPL)));
    const V x = __builtin_nontemporal_load(reinterpret_cast<const V*>(base + off));
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = x[c];
  }
}

template <typename T, int CPL>
__device__ __forceinline__ void st_vec(T* __restrict__ base, uint32_t off, bool on, const T (&v)[CPL],
                                       bool masked) {
  if constexpr (CPL == 1) {
    if (!masked || on) base[off] = v[0];
  } else {
    using V = T __attribute__((ext_vector_type(CPL)));
    V x;
#pragma unroll
    for (int c = 0; c < CPL; ++c) x[c] = v[c];
    *reinterpret_cast<V*>(base + off) = x;
  }
}

// One edge's contribution to the accumulators of the paths in group G (of
// NG): for every such path p and output component m3,
//   acc[(p,m3)] += sum_m1 M^p[m1][m3] * R[p] * h[(l1,m1)],  M^p = C^p . Y,
// with the sparsity of C^p unrolled at compile time.  h and R hold CPL
// channels per lane; ye is the edge's harmonics (uniform across lanes).
template <typename T, int L1, int L2, int L3, bool SUM, int CPL, int NG, int G>
__device__ __forceinline__ void tp_fwd_edge(const T (&hh)[kTable<L1, L2, L3, SUM>.din][CPL],
                                            const T (&rr)[kTable<L1, L2, L3, SUM>.np][CPL], const T (&ye)[16],
                                            T (&acc)[kTable<L1, L2, L3, SUM>.dout][CPL]) {
  constexpr int NP = kTable<L1, L2, L3, SUM>.np;
  static_for<NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    if constexpr (kGroups<L1, L2, L3, SUM, NG, CPL>.group[p] == G) {
      constexpr Path P = kTable<L1, L2, L3, SUM>.path[p];
      T hr[2 * P.l1 + 1][CPL];
#pragma unroll
      for (int m1 = 0; m1 < 2 * P.l1 + 1; ++m1)
#pragma unroll
        for (int c = 0; c < CPL; ++c) hr[m1][c] = rr[p][c] * hh[P.l1 * P.l1 + m1][c];
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        constexpr int row = kTable<L1, L2, L3, SUM>.out_row(p, m3);
        static_for<2 * P.l1 + 1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (kTable<L1, L2, L3, SUM>.midx[p][m1][m3] >= 0) {
            T M = T(0);
            static_for<2 * P.l2 + 1>([&](auto m2c) {
              constexpr int m2 = decltype(m2c)::value;
              constexpr double cv = kTable<L1, L2, L3, SUM>.cg[p][m1][m2][m3];
              if constexpr (cv != 0.0) M += T(cv) * ye[P.l2 * P.l2 + m2];
            });
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[row][c] += M * hr[m1][c];
          }
        });
      });
    }
  });
}

template <typename T, int L1, int L2, int L3, bool SUM, int CPL, int NG, bool MASKED, int G>
__device__ __forceinline__ void tp_fwd_group(const int32_t* __restrict__ src, int e_lo, int e_hi,
                                             int64_t edge_begin, int C, uint32_t c0, bool on,
                                             const T* __restrict__ h, const T* __restrict__ Y,
                                             const T* __restrict__ R, T* __restrict__ oi, T scale) {
  constexpr int NP = kTable<L1, L2, L3, SUM>.np, DIN = kTable<L1, L2, L3, SUM>.din;
  constexpr int DSH = kTable<L1, L2, L3, SUM>.dsh, DOUT = kTable<L1, L2, L3, SUM>.dout;
  const int PC = NP * C;
  T acc[DOUT][CPL];
  static_for<NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    if constexpr (kGroups<L1, L2, L3, SUM, NG, CPL>.group[p] == G) {
      constexpr Path P = kTable<L1, L2, L3, SUM>.path[p];
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int row = kTable<L1, L2, L3, SUM>.out_row(p, decltype(m3c)::value);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[row][c] = T(0);
      });
    }
  });
  // An edge's harmonics travel with its prefetch as one vector load (lane k
  // holds Y[k]) and are broadcast with v_readlane.
  struct Buf {
    T h[DIN][CPL];
    T r[NP][CPL];
    T y;
  };
  const int lane = threadIdx.x % kTPWave;
  const int ylane = (lane & 15) < DSH ? (lane & 15) : DSH - 1;
  auto load_j = [&](int e, int j, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ hj = h + (int64_t)j * DIN * C;
    const T* __restrict__ re = R + ((int64_t)e - edge_begin) * PC;
    // only the rows of the l1 ranks this group's paths read
    static_for<DIN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
      if constexpr (group_uses_l1(kTable<L1, L2, L3, SUM>, kGroups<L1, L2, L3, SUM, NG, CPL>, G, l1))
        ld_vec<T, CPL>(hj, m * C + c0, on, b.h[m], MASKED);
    });
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (kGroups<L1, L2, L3, SUM, NG, CPL>.group[p] == G) ld_vec_nt<T, CPL>(re, p * C + c0, on, b.r[p], MASKED);
    });
    b.y = Y[((int64_t)e - edge_begin) * DSH + ylane];
  };
  auto compute = [&](int, const Buf& b) __attribute__((always_inline)) {
    T ye[16];
#pragma unroll
    for (int k = 0; k < DSH; ++k) ye[k] = lane_value(b.y, k);
    tp_fwd_edge<T, L1, L2, L3, SUM, CPL, NG, G>(b.h, b.r, ye, acc);
  };
  if (e_hi - e_lo > 64 * kIdxWindows) {
    edge_loop<Buf>(e_lo, e_hi, [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, uniform(src[e]), b); }, compute);
  } else if (e_hi > e_lo) {
    RowIdx<kIdxWindows> si;
    si.init(src, e_lo, e_hi, lane);
    edge_loop<Buf>(e_lo, e_hi, [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, si.get(e - e_lo), b); }, compute);
  }
  static_for<NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    if constexpr (kGroups<L1, L2, L3, SUM, NG, CPL>.group[p] == G) {
      constexpr Path P = kTable<L1, L2, L3, SUM>.path[p];
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int row = kTable<L1, L2, L3, SUM>.out_row(p, decltype(m3c)::value);
        T v[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = scale * acc[row][c];
        st_vec<T, CPL>(oi, row * C + c0, on, v, MASKED);
      });
    }
  });
}

template <typename T, int L1, int L2, int L3, bool SUM, int CPL, int NG, bool MASKED, int NWC = 1>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
         int64_t row_end, int64_t edge_begin, int C, T scale, const T* __restrict__ h,
         const T* __restrict__ Y, const T* __restrict__ R, T* __restrict__ out) {
  constexpr int DOUT = kTable<L1, L2, L3, SUM>.dout;
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = xcd_block() * kTPWavesPerBlock + threadIdx.x / kTPWave;
  const int64_t row = row_begin + w / (NG * NWC);
  if (row >= row_end) return;
  const int i = uniform((int)row);
  const int rem = uniform((int)(w % (NG * NWC)));
  const int g = rem % NG, cw = rem / NG;
  const int CC = MASKED ? C : 64 * CPL * NWC;
  const uint32_t c0 = (uint32_t)(cw * 64 * CPL + lane * CPL);
  const bool on = (int)c0 < C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  T* __restrict__ oi = out + (int64_t)i * DOUT * CC;
  static_for<NG>([&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (g == G)
      tp_fwd_group<T, L1, L2, L3, SUM, CPL, NG, MASKED, G>(src, e_lo, e_hi, edge_begin, CC, c0, on, h, Y,
                                                     R, oi, scale);
  });
}

// ---------------------------------------------------------------------------
// Sum of v[0..15] over the 64 lanes of a wave, reduce-scatter style: every
// lane l ends with the total of entry l / 4 (all four lanes of a quad hold
// it).  Each halving step pairs every lane with one in the other half of its
// group, keeps the half of the entries that its own lane bit selects and adds
// the partner's copy of them, so every step moves half the data.  The moves
// stay in the vector ALU (no LDS): v_permlane32_swap across the two 32-lane
// halves, v_permlane16_swap across 16-lane rows, then DPP within rows
// (row_ror:8, row_half_mirror, and quad permutations for the last two steps,
// which leave the total in all four lanes of the quad).
__device__ __forceinline__ uint32_t u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float f32(uint32_t x) { return __builtin_bit_cast(float, x); }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)u32(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// (a, b) -> (a + partner's a, b + partner's b) for lanes keeping a (low half
// of the group) / b (high half), with the two swap instructions.
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(u32(a), u32(b), false, false);
  return f32(r[0]) + f32(r[1]);
}
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(u32(a), u32(b), false, false);
  return f32(r[0]) + f32(r[1]);
}
__device__ __forceinline__ double swap32_add(double a, double b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)ua, (uint32_t)ub, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32), false, false);
  const double x = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]);
  const double y = __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
  return x + y;
}
__device__ __forceinline__ double swap16_add(double a, double b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)ua, (uint32_t)ub, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32), false, false);
  const double x = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]);
  const double y = __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
  return x + y;
}

template <typename T>
__device__ __forceinline__ T wave_reduce_scatter16(const T (&v)[16]) {
  const int lane = threadIdx.x % kTPWave;
  // lanes 0-31 keep entries 0-7, lanes 32-63 entries 8-15: the swap moves
  // the upper half of a[k]'s lanes and the lower half of a[k+8]'s lanes across
  T a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = swap32_add(v[k], v[k + 8]);
  // rows 0 and 2 keep entries (k), rows 1 and 3 entries (k + 4) of the half
  T b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = swap16_add(a[k], a[k + 4]);
  // within a row: lanes 0-7 keep (k), lanes 8-15 keep (k + 2); partner l ^ 8
  T c[2];
  {
    const bool hi = lane & 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const T send = hi ? b[k] : b[k + 2];
      const T keep = hi ? b[k + 2] : b[k];
      c[k] = keep + dpp<0x128>(send);  // row_ror:8
    }
  }
  // within 8 lanes: lanes 0-3 keep (k), lanes 4-7 keep (k + 1); partner 7 - l
  T d;
  {
    const bool hi = lane & 4;
    const T send = hi ? c[0] : c[1];
    const T keep = hi ? c[1] : c[0];
    d = keep + dpp<0x141>(send);  // row_half_mirror
  }
  d += dpp<0x4E>(d);  // quad_perm [2,3,0,1]
  d += dpp<0xB1>(d);  // quad_perm [1,0,3,2]
  return d;
}

// Backward, edge side.  One wave per receiver row and 64 channels (NW waves
// per row, one channel per lane), G[i] held in registers for the whole row.
// Per edge and path, with K[m1][m2] = sum_m3 C^p[m1,m2,m3] G[i,(p,m3)]:
//   W[m1] = sum_m2 Y[m2] K[m1][m2]    Q[m2] = sum_m1 h[j,m1] K[m1][m2]
//   dR    = s * sum_m1 h[j,m1] W[m1]  dY[m2] += R Q[m2]   (channel reduction)
//   t[m1] += R W[m1]                  (the edge's contribution to dh of its
//                                      sender j, stored at the reverse edge's
//                                      slot so dh of j is a contiguous row sum)
template <typename T, int L1, int L2, int L3, bool SUM, int NW>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_bwd_edge(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
              const int32_t* __restrict__ rev, int64_t row_begin, int64_t row_end,
              int64_t edge_begin, int64_t n_chunk_edges, int C, T scale, const T* __restrict__ h,
              const T* __restrict__ Y, const T* __restrict__ R, const T* __restrict__ G,
              T* __restrict__ dR, T* __restrict__ dYp, T* __restrict__ dh_edge) {
  constexpr int NP = kTable<L1, L2, L3, SUM>.np, DIN = kTable<L1, L2, L3, SUM>.din;
  constexpr int DSH = kTable<L1, L2, L3, SUM>.dsh, DOUT = kTable<L1, L2, L3, SUM>.dout;
  static_assert(DSH <= 16, "harmonics beyond l = 3");
  const RowWave rw = row_wave<NW>(row_begin, row_end, C);
  if (!rw.ok) return;
  const int i = rw.row;
  const int CC = channels<NW>(C);
  const int PC = NP * CC;
  const uint32_t c0 = (uint32_t)rw.c0;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  if (e_lo == e_hi) return;
  const int lane = threadIdx.x % kTPWave;
  const int part = rw.c0 / kTPWave;   // which 64-channel slice (partial dY buffer)

  T gi[DOUT];
  {
    const T* __restrict__ gr = G + (int64_t)i * DOUT * CC;
#pragma unroll
    for (int o = 0; o < DOUT; ++o) gi[o] = ldc<NW>(gr, o * CC + c0, rw.on);
  }

  // The edge's harmonics travel with the prefetch as one vector load (lane k
  // holds Y[k]) and are broadcast with v_readlane: held in scalar registers
  // through the whole path loop they would be re-read from memory, each
  // re-read waiting on the scalar cache.
  struct Buf {
    T h[DIN];
    T r[NP];
    T y;
    int er;  // reverse edge
  };
  const int ylane = (lane & 15) < DSH ? (lane & 15) : DSH - 1;
  auto load_j = [&](int e, int j, int er, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ hj = h + (int64_t)j * DIN * CC;
    const T* __restrict__ re = R + ((int64_t)e - edge_begin) * PC;
#pragma unroll
    for (int m = 0; m < DIN; ++m) b.h[m] = ldc<NW>(hj, m * CC + c0, rw.on);
#pragma unroll
    for (int p = 0; p < NP; ++p) b.r[p] = ldc_nt<NW>(re, p * CC + c0, rw.on);
    b.y = Y[((int64_t)e - edge_begin) * DSH + ylane];
    b.er = er;
  };
  auto compute = [&](int e, const Buf& b) __attribute__((always_inline)) {
    const int64_t el = (int64_t)e - edge_begin;
    T ye[16];
#pragma unroll
    for (int k = 0; k < DSH; ++k) ye[k] = lane_value(b.y, k);
    T* __restrict__ dre = dR + el * PC;
    T dy[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) dy[k] = T(0);
    T t[DIN];
#pragma unroll
    for (int m = 0; m < DIN; ++m) t[m] = T(0);
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr Path P = kTable<L1, L2, L3, SUM>.path[p];
      constexpr int n1 = 2 * P.l1 + 1, n2 = 2 * P.l2 + 1;
      T K[n1][n2];
#pragma unroll
      for (int a = 0; a < n1; ++a)
#pragma unroll
        for (int c = 0; c < n2; ++c) K[a][c] = T(0);
      static_for<2 * P.l3 + 1>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        constexpr int row = kTable<L1, L2, L3, SUM>.out_row(p, m3);
        static_for<n1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          static_for<n2>([&](auto m2c) {
            constexpr int m2 = decltype(m2c)::value;
            constexpr double cv = kTable<L1, L2, L3, SUM>.cg[p][m1][m2][m3];
            if constexpr (cv != 0.0) K[m1][m2] += T(cv) * gi[row];
          });
        });
      });
      T dr = T(0);
      static_for<n1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        T w = T(0);
        static_for<n2>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          if constexpr (kTable<L1, L2, L3, SUM>.m12nz(p, m1, m2)) w += ye[P.l2 * P.l2 + m2] * K[m1][m2];
        });
        dr += b.h[P.l1 * P.l1 + m1] * w;
        t[P.l1 * P.l1 + m1] += b.r[p] * w;
      });
      static_for<n2>([&](auto m2c) {
        constexpr int m2 = decltype(m2c)::value;
        T q = T(0);
        static_for<n1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (kTable<L1, L2, L3, SUM>.m12nz(p, m1, m2)) q += b.h[P.l1 * P.l1 + m1] * K[m1][m2];
        });
        dy[P.l2 * P.l2 + m2] += b.r[p] * q;
      });
      stc_nt<NW>(dre, p * CC + c0, rw.on, scale * dr);
    });
    T* __restrict__ te = dh_edge + (int64_t)b.er * DIN * CC;
#pragma unroll
    for (int m = 0; m < DIN; ++m) stc_nt<NW>(te, m * CC + c0, rw.on, t[m]);
    // every lane of a quad holds the same total, so with 16 harmonics all
    // lanes store (identical values per address) and the store needs no
    // branch, which keeps the wait for the next edge's loads exact
    const T tot = wave_reduce_scatter16<T>(dy);
    if (DSH == 16 || (lane >> 2) < DSH)
      dYp[((int64_t)part * n_chunk_edges + el) * DSH + (lane >> 2)] = scale * tot;
  };
  if (e_hi - e_lo > 64 * kIdxWindows) {
    edge_loop<Buf>(e_lo, e_hi, [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, uniform(src[e]), uniform(rev[e]), b); },
                   compute);
  } else {
    RowIdx<kIdxWindows> si, ri;
    si.init(src, e_lo, e_hi, lane);
    ri.init(rev, e_lo, e_hi, lane);
    edge_loop<Buf>(e_lo, e_hi,
                   [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, si.get(e - e_lo), ri.get(e - e_lo), b); }, compute);
  }
}

// ---------------------------------------------------------------------------
// dh[j] = s * sum over the edges e of row j of dh_edge[e]: each slot holds the
// contribution of the reverse edge (whose sender is j), so the sum runs over a
// contiguous range in CSR order (deterministic, no atomics).  One thread per
// (atom, group of V consecutive feature values); every value is summed over
// the row's edges in CSR order, V at a time, with eight edges' loads in
// flight (non-temporal: each value is read once).
template <typename T, int V>
__global__ void __launch_bounds__(256)
k_dh_gather(int64_t n, int din_c, const int32_t* __restrict__ row_ptr, T scale,
            const T* __restrict__ dh_edge, T* __restrict__ dh) {
  typedef T vec __attribute__((ext_vector_type(V)));
  const int groups = din_c / V;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= n * groups) return;
  const int64_t j = t / groups;
  const int q = (int)(t - j * groups) * V;
  vec acc = vec(T(0));
  const int lo = row_ptr[j], hi = row_ptr[j + 1];
  const T* __restrict__ p = dh_edge + q;
  int e = lo;
  for (; e + 8 <= hi; e += 8) {
    vec a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      a[k] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(p + (int64_t)(e + k) * din_c));
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += a[k];
  }
  for (; e < hi; ++e) acc += *reinterpret_cast<const vec*>(p + (int64_t)e * din_c);
  *reinterpret_cast<vec*>(dh + j * din_c + q) = scale * acc;
}

// ---------------------------------------------------------------------------
inline int tp_waves_per_row(int C) { return C <= kTPWave ? 1 : C / kTPWave; }

inline unsigned tp_blocks(int64_t rows, int C) {
  const int64_t waves = rows * tp_waves_per_row(C);
  return (unsigned)((waves + kTPWavesPerBlock - 1) / kTPWavesPerBlock);
}

inline bool tp_channels_ok(int C) { return (C >= 1 && C <= 64) || C == 128; }

// Compile-time waves per row for a channel count (0: fewer than 64 channels).
inline int tp_nw(int C) { return C < 64 ? 0 : C / 64; }

namespace tp_detail {
template <typename T>
constexpr int dtype_id() { return std::is_same<T, double>::value ? 1 : 0; }
}  // namespace tp_detail

}  // namespace tpc

// Built (dtype, node_lmax, sh_lmax, out_lmax) sets.  Channels: 1..64 or 128.
#define TPC_TP_CONFIGS(X)                                                    \
  X(float, 1, 2, 1) X(float, 1, 3, 3) X(float, 2, 3, 3) X(float, 3, 3, 3)   \
  X(double, 1, 2, 1) X(double, 1, 3, 3) X(double, 2, 3, 3) X(double, 3, 3, 3)
