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
// weight): k_tp_bwd below, one pass over the receiver-sorted list that writes
// dR, the channel sums of dY and, by a gather along each receiver's own row
// (the list is symmetric), the sender-feature gradient dh.
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
  // R rows of the row's edges: map[e - edge_begin] (shared rows of edge
  // pairs), or e - edge_begin without a map
  __device__ __forceinline__ void init_rows(const int32_t* __restrict__ map, int64_t edge_begin, int e_lo,
                                            int e_hi, int lane) {
#pragma unroll
    for (int q = 0; q < NWIN; ++q) {
      const int e = min(e_lo + 64 * q + lane, e_hi - 1);
      v[q] = map ? map[e - edge_begin] : (int)(e - edge_begin);
    }
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

// Chunk-relative R row of edge e (a scalar load with a map), for rows too
// long for the index windows.
__device__ __forceinline__ int r_row(const int32_t* __restrict__ map, int64_t edge_begin, int e) {
  return map ? uniform(map[e - edge_begin]) : (int)(e - edge_begin);
}

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

template <typename T, int L1, int L2, int L3, bool SUM, int CPL, int NG, bool MASKED, int G, bool PAIR>
__device__ __forceinline__ void tp_fwd_group(const int32_t* __restrict__ src, int e_lo, int e_hi,
                                             int64_t edge_begin, int C, uint32_t c0, bool on,
                                             const T* __restrict__ h, const T* __restrict__ Y,
                                             const T* __restrict__ R, const int32_t* __restrict__ Rrow,
                                             T* __restrict__ oi, T scale) {
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
  auto load_j = [&](int e, int j, int rr, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ hj = h + (int64_t)j * DIN * C;
    const T* __restrict__ re = PAIR ? R + (int64_t)rr * PC : R + ((int64_t)e - edge_begin) * PC;
    // only the rows of the l1 ranks this group's paths read
    static_for<DIN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
      if constexpr (group_uses_l1(kTable<L1, L2, L3, SUM>, kGroups<L1, L2, L3, SUM, NG, CPL>, G, l1))
        ld_vec<T, CPL>(hj, m * C + c0, on, b.h[m], MASKED);
    });
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      // a shared row is read twice (once per edge of its pair), so it is
      // loaded through the caches, where the partner row may still find it
      if constexpr (kGroups<L1, L2, L3, SUM, NG, CPL>.group[p] == G) {
        if constexpr (PAIR) ld_vec<T, CPL>(re, p * C + c0, on, b.r[p], MASKED);
        else ld_vec_nt<T, CPL>(re, p * C + c0, on, b.r[p], MASKED);
      }
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
    edge_loop<Buf>(e_lo, e_hi,
                   [&](int e, Buf& b) __attribute__((always_inline)) {
                     load_j(e, uniform(src[e]), PAIR ? r_row(Rrow, edge_begin, e) : 0, b);
                   },
                   compute);
  } else if (e_hi > e_lo) {
    RowIdx<kIdxWindows> si;
    si.init(src, e_lo, e_hi, lane);
    if constexpr (PAIR) {
      RowIdx<kIdxWindows> qi;
      qi.init_rows(Rrow, edge_begin, e_lo, e_hi, lane);
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) {
                       load_j(e, si.get(e - e_lo), qi.get(e - e_lo), b);
                     },
                     compute);
    } else {
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, si.get(e - e_lo), 0, b); },
                     compute);
    }
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

template <typename T, int L1, int L2, int L3, bool SUM, int CPL, int NG, bool MASKED, int NWC, bool PAIR>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
         int64_t row_end, int64_t edge_begin, int C, T scale, const T* __restrict__ h,
         const T* __restrict__ Y, const T* __restrict__ R, const int32_t* __restrict__ Rrow,
         T* __restrict__ out) {
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
      tp_fwd_group<T, L1, L2, L3, SUM, CPL, NG, MASKED, G, PAIR>(src, e_lo, e_hi, edge_begin, CC, c0, on, h, Y,
                                                     R, Rrow, oi, scale);
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

// Backward, edge side.  NG * NWC waves share a receiver row: NWC slices of
// 64 channels (one channel per lane; one masked wave for C < 64), and in each
// slice NG waves that own whole l1 classes of the paths (kBwdGroups), so each
// reads only its rows of h, R and G and writes disjoint rows of the dh
// contributions.  G[i] rows of the group's paths stay in registers for the
// whole row.  Per edge and path, with K[m1][m2] = sum_m3 C^p[m1,m2,m3]
// G[i,(p,m3)]:
//   W[m1] = sum_m2 Y[m2] K[m1][m2]    Q[m2] = sum_m1 h[j,m1] K[m1][m2]
//   dR    = s * sum_m1 h[j,m1] W[m1]  dY[m2] += R Q[m2]   (channel reduction,
//                                      one partial slice per wave)
//   t[m1] += R W[m1]                  (the edge's contribution to dh of its
//                                      sender j, stored at the edge's own slot
//                                      of the chunk; k_dh_gather_chunk sums
//                                      them along row j through the reverse
//                                      index)
#define TBL kTable<L1, L2, L3, SUM>
#define BGR kBwdGroups<L1, L2, L3, SUM, NG>
template <typename T, int L1, int L2, int L3, bool SUM, bool MASKED, int NG, int G, bool PAIR>
__device__ __forceinline__ void tp_bwd_edge_group(const int32_t* __restrict__ src, int i, int e_lo, int e_hi,
                                                  int64_t edge_begin, int64_t n_chunk_edges, int CC, uint32_t c0,
                                                  bool on, int part, T scale, const T* __restrict__ h,
                                                  const T* __restrict__ Y, const T* __restrict__ R,
                                                  const int32_t* __restrict__ Rrow,
                                                  const T* __restrict__ Gr, T* __restrict__ dR,
                                                  T* __restrict__ dYp, T* __restrict__ dh_edge) {
  constexpr int NP = TBL.np, DIN = TBL.din, DSH = TBL.dsh, DOUT = TBL.dout;
  static_assert(DSH <= 16, "harmonics beyond l = 3");
  static_assert(BGR.ok, "every wave group owns an l1 class");
  constexpr int NWM = MASKED ? 0 : 1;   // ldc/stc: masked lanes past C
  const int PC = NP * CC;
  const int lane = threadIdx.x % kTPWave;

  T gi[DOUT];
  {
    const T* __restrict__ gr = Gr + (int64_t)i * DOUT * CC;
    static_for<DOUT>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      if constexpr (bwd_group_reads_row(TBL, BGR, G, o)) gi[o] = ldc<NWM>(gr, o * CC + c0, on);
    });
  }

  // The edge's harmonics travel with the prefetch as one vector load (lane k
  // holds Y[k]) and are broadcast with v_readlane: held in scalar registers
  // through the whole path loop they would be re-read from memory, each
  // re-read waiting on the scalar cache.
  struct Buf {
    T h[DIN];
    T r[NP];
    T y;
  };
  const int ylane = (lane & 15) < DSH ? (lane & 15) : DSH - 1;
  auto load_j = [&](int e, int j, int rr, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ hj = h + (int64_t)j * DIN * CC;
    const T* __restrict__ re = PAIR ? R + (int64_t)rr * PC : R + ((int64_t)e - edge_begin) * PC;
    static_for<DIN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
      if constexpr (bwd_group_owns_l1(TBL, BGR, G, l1)) b.h[m] = ldc<NWM>(hj, m * CC + c0, on);
    });
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      // shared rows through the caches (read once per edge of the pair)
      if constexpr (BGR.group[p] == G) b.r[p] = PAIR ? ldc<NWM>(re, p * CC + c0, on) : ldc_nt<NWM>(re, p * CC + c0, on);
    });
    b.y = Y[((int64_t)e - edge_begin) * DSH + ylane];
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
      if constexpr (BGR.group[p] == G) {
        constexpr Path P = TBL.path[p];
        constexpr int n1 = 2 * P.l1 + 1, n2 = 2 * P.l2 + 1;
        T K[n1][n2];
#pragma unroll
        for (int a = 0; a < n1; ++a)
#pragma unroll
          for (int c = 0; c < n2; ++c) K[a][c] = T(0);
        static_for<2 * P.l3 + 1>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          constexpr int row = TBL.out_row(p, m3);
          static_for<n1>([&](auto m1c) {
            constexpr int m1 = decltype(m1c)::value;
            static_for<n2>([&](auto m2c) {
              constexpr int m2 = decltype(m2c)::value;
              constexpr double cv = TBL.cg[p][m1][m2][m3];
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
            if constexpr (TBL.m12nz(p, m1, m2)) w += ye[P.l2 * P.l2 + m2] * K[m1][m2];
          });
          dr += b.h[P.l1 * P.l1 + m1] * w;
          t[P.l1 * P.l1 + m1] += b.r[p] * w;
        });
        static_for<n2>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          T q = T(0);
          static_for<n1>([&](auto m1c) {
            constexpr int m1 = decltype(m1c)::value;
            if constexpr (TBL.m12nz(p, m1, m2)) q += b.h[P.l1 * P.l1 + m1] * K[m1][m2];
          });
          dy[P.l2 * P.l2 + m2] += b.r[p] * q;
        });
        stc_nt<NWM>(dre, p * CC + c0, on, scale * dr);
      }
    });
    T* __restrict__ te = dh_edge + el * DIN * CC;
    static_for<DIN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
      if constexpr (bwd_group_owns_l1(TBL, BGR, G, l1)) stc_nt<NWM>(te, m * CC + c0, on, t[m]);
    });
    // every lane of a quad holds the same total, so with 16 harmonics all
    // lanes store (identical values per address) and the store needs no
    // branch, which keeps the wait for the next edge's loads exact
    const T tot = wave_reduce_scatter16<T>(dy);
    if (DSH == 16 || (lane >> 2) < DSH)
      dYp[((int64_t)part * n_chunk_edges + el) * DSH + (lane >> 2)] = scale * tot;
  };
  if (e_hi - e_lo > 64 * kIdxWindows) {
    edge_loop<Buf>(e_lo, e_hi,
                   [&](int e, Buf& b) __attribute__((always_inline)) {
                     load_j(e, uniform(src[e]), PAIR ? r_row(Rrow, edge_begin, e) : 0, b);
                   },
                   compute);
  } else {
    RowIdx<kIdxWindows> si;
    si.init(src, e_lo, e_hi, lane);
    if constexpr (PAIR) {
      RowIdx<kIdxWindows> qi;
      qi.init_rows(Rrow, edge_begin, e_lo, e_hi, lane);
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) {
                       load_j(e, si.get(e - e_lo), qi.get(e - e_lo), b);
                     },
                     compute);
    } else {
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, si.get(e - e_lo), 0, b); },
                     compute);
    }
  }
}
#undef TBL
#undef BGR

// Wave w of the grid: row w / (NG * NWC), then group and channel slice;
// partial dY slice (channel slice) * NG + group.
template <typename T, int L1, int L2, int L3, bool SUM, bool MASKED, int NG, int NWC, bool PAIR>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_bwd_edge(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
              int64_t row_end, int64_t edge_begin, int64_t n_chunk_edges, int C, T scale, const T* __restrict__ h,
              const T* __restrict__ Y, const T* __restrict__ R, const int32_t* __restrict__ Rrow,
              const T* __restrict__ Gr, T* __restrict__ dR,
              T* __restrict__ dYp, T* __restrict__ dh_edge) {
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = xcd_block() * kTPWavesPerBlock + threadIdx.x / kTPWave;
  const int64_t row = row_begin + w / (NG * NWC);
  if (row >= row_end) return;
  const int i = uniform((int)row);
  const int rem = uniform((int)(w % (NG * NWC)));
  const int g = rem % NG, cw = rem / NG;
  const int CC = MASKED ? C : 64 * NWC;
  const uint32_t c0 = (uint32_t)(cw * 64 + lane);
  const bool on = (int)c0 < C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  if (e_lo == e_hi) return;
  const int part = cw * NG + g;
  static_for<NG>([&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (g == G)
      tp_bwd_edge_group<T, L1, L2, L3, SUM, MASKED, NG, G, PAIR>(src, i, e_lo, e_hi, edge_begin, n_chunk_edges, CC, c0,
                                                           on, part, scale, h, Y, R, Rrow, Gr, dR, dYp, dh_edge);
  });
}

// ---------------------------------------------------------------------------
// dh of every atom j, one receiver chunk at a time.  The backward of the
// chunk's edges leaves each edge's contribution to dh of its sender at the
// edge's own slot of the chunk (t_chunk).  Atom j gathers them along its own
// row through the symmetric list: the entries e' of row j whose sender lies
// in the chunk's rows [row_begin, row_end) have their reverse edges in the
// chunk, at t_chunk[rev(e') - edge_begin].  Row j is sorted by sender, so
// those entries form one contiguous run, and the runs of successive chunks
// follow each other in row order: continuing the running sum chunk after
// chunk adds every term in the same CSR order as a single pass over the
// whole list, so chunked and unchunked results agree bit for bit, and the
// intermediate only spans one chunk's edges.  dh holds the unscaled sum
// between chunks (first: start from zero; last: store s * sum).
//
// One wave per (atom, slab of 64 V feature values), V consecutive values per
// lane, eight terms' loads in flight.  The wave's atom is uniform, so the row
// bounds and reverse indices are scalar loads, and the run is found with one
// coalesced load of up to 64 senders per step and two ballots (the number of
// entries below row_begin and below row_end).  A reverse index outside the
// chunk (a list that is not symmetric or not sender-sorted) contributes
// nothing rather than reading outside t_chunk.  Deterministic, no atomics.
constexpr int kGatherWaves = 4;
template <typename T, int V>
__global__ void __launch_bounds__(64 * kGatherWaves)
k_dh_gather_chunk(int64_t n, int din_c, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
                  const int32_t* __restrict__ rev, int64_t row_begin, int64_t row_end, int64_t edge_begin,
                  int64_t n_chunk_edges, bool first, bool last, T scale, const T* __restrict__ t_chunk,
                  T* __restrict__ dh) {
  typedef T vec __attribute__((ext_vector_type(V)));
  const int lane = threadIdx.x % 64;
  const int slabs = (din_c + 64 * V - 1) / (64 * V);
  const int64_t w = (int64_t)blockIdx.x * kGatherWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if (w >= n * slabs) return;
  const int64_t j = w / slabs;
  const int q = (int)(w - j * slabs) * 64 * V + lane * V;
  const int r0 = row_ptr[j], r1 = row_ptr[j + 1];
  int lo = r0, hi = r1;
  if (n_chunk_edges <= 0) {
    hi = lo;
  } else if (row_begin > 0 || row_end < n) {
    int below_begin = 0, below_end = 0;
    for (int b = r0; b < r1; b += 64) {
      const int e = b + lane;
      const int v = e < r1 ? src[e] : 0x7fffffff;
      below_begin += __popcll(__ballot(v < row_begin));
      below_end += __popcll(__ballot(v < row_end));
    }
    lo = r0 + below_begin;
    hi = r0 + below_end;
  }
  if (q >= din_c) return;
  T* __restrict__ dj = dh + j * din_c + q;
  vec acc = first ? vec(T(0)) : *reinterpret_cast<const vec*>(dj);
  const T* __restrict__ p = t_chunk + q;
  auto term = [&](int e) __attribute__((always_inline)) {
    const int64_t r = (int64_t)rev[e] - edge_begin;
    return (uint64_t)r < (uint64_t)n_chunk_edges ? r : int64_t(-1);
  };
  int e = lo;
  for (; e + 8 <= hi; e += 8) {
    int64_t r[8];
    vec a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = term(e + k);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      a[k] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(p + (r[k] < 0 ? 0 : r[k]) * din_c));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (r[k] >= 0) acc += a[k];
  }
  for (; e < hi; ++e) {
    const int64_t r = term(e);
    if (r >= 0) acc += *reinterpret_cast<const vec*>(p + r * din_c);
  }
  *reinterpret_cast<vec*>(dj) = last ? scale * acc : acc;
}

// ---------------------------------------------------------------------------
// VJP-of-VJP (double backward; FlashCart paper, section 3 "Symbolic
// derivatives": training on forces differentiates through the VJP; section 4
// "Receiver-sorted derivatives": the same receiver-sorted edges, the incoming
// gradient of a receiver loaded once per row).  Given cotangents uh, uY, uR of
// the VJP outputs dh, dY, dR, the scalar <uh,dh> + <uY,dY> + <uR,dR> is
// differentiated with respect to G, h, Y and R.  With T(a, y) the unweighted
// product of path p, i the receiver and j the sender of edge e:
//   g_hat[i,(p,m3)] = s sum_{e in row i} T(h_j, uR Y + R uY) + R T(uh_j, Y)
//   w_hat[e,p]      = s sum_{m1,m2} K[m1][m2] (h_j[m1] uY[m2] + uh_j[m1] Y[m2])
//   y_hat[e,m2]     = s sum_u sum_p sum_m1 K[m1][m2] (uR h_j[m1] + R uh_j[m1])
// with K = C . G[i] per row (as in the VJP), and, gathered along each row
// through the symmetric list (the reverse edge of e has e's R and harmonics
// (-1)^l2 Y[e], and its own cotangents uR[rev e], uY[rev e]):
//   x_hat[i,(l1,m1)] = s sum_{e in row i} sum_p sum_{m2,m3} C^p G[j,(p,m3)]
//                      ((-1)^l2 uR[rev e,p] Y[e,m2] + R[e,p] uY[rev e,m2])
// Two kernels, each over rows with whole l1 classes per wave (kBwdGroups):
// k_tp_dbl_recv (g_hat, w_hat, partial y_hat) and k_tp_dbl_send (x_hat).
// Every sum is a fixed-order register accumulation: deterministic, no atomics.
// Separate (not path-summed) outputs only: each path then owns its rows of
// g_hat, so the waves of a row write disjoint rows.
#define TBL kTable<L1, L2, L3, false>
#define BGR kBwdGroups<L1, L2, L3, false, NG>
template <typename T, int L1, int L2, int L3, int NG, bool MASKED, int G, bool PAIR>
__device__ __forceinline__ void tp_dbl_recv_group(
    const int32_t* __restrict__ src, int i, int e_lo, int e_hi, int64_t edge_begin, int64_t n_chunk_edges,
    int CC, uint32_t c0, bool on, int part, T scale, const T* __restrict__ h, const T* __restrict__ uh,
    const T* __restrict__ Y, const T* __restrict__ uY, const T* __restrict__ R,
    const int32_t* __restrict__ Rrow, const T* __restrict__ uR, const T* __restrict__ Gr, T* __restrict__ g_hat, T* __restrict__ w_hat, T* __restrict__ yhp) {
  constexpr int NP = TBL.np, DIN = TBL.din, DSH = TBL.dsh, DOUT = TBL.dout;
  constexpr int NK = BGR.nk[G] > 0 ? BGR.nk[G] : 1;
  static_assert(BGR.ok, "every wave group owns an l1 class");
  // float32 keeps K = s C . G[i] for the whole row; float64 (twice as wide)
  // keeps the scaled G[i] rows and forms each K entry where it is used
  constexpr bool kHoldK = sizeof(T) == 4;
  const int PC = NP * CC;
  const int lane = threadIdx.x % kTPWave;
  T K[kHoldK ? NK : 1];
  T gi[DOUT];
  {
    const T* __restrict__ gr = Gr + (int64_t)i * DOUT * CC;
    static_for<DOUT>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      if constexpr (bwd_group_reads_row(TBL, BGR, G, o)) gi[o] = scale * ldc<MASKED ? 0 : 1>(gr, o * CC + c0, on);
    });
    if constexpr (kHoldK) static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (BGR.group[p] == G) {
        constexpr Path P = TBL.path[p];
        static_for<2 * P.l1 + 1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          static_for<2 * P.l2 + 1>([&](auto m2c) {
            constexpr int m2 = decltype(m2c)::value;
            constexpr int k = m12_index(TBL, p, m1, m2);
            if constexpr (k >= 0) {
              constexpr int kk = BGR.kofs[p] + k;
              T acc = T(0);
              static_for<2 * P.l3 + 1>([&](auto m3c) {
                constexpr int m3 = decltype(m3c)::value;
                constexpr double cv = TBL.cg[p][m1][m2][m3];
                constexpr int o = TBL.out_row(p, m3);
                if constexpr (cv != 0.0) acc += T(cv) * gi[o];
              });
              K[kk] = acc;
            }
          });
        });
      }
    });
  }
  T ga[DOUT];
#pragma unroll
  for (int o = 0; o < DOUT; ++o) ga[o] = T(0);
  struct Buf {
    T h[DIN];
    T uh[DIN];
    T r[NP];
    T ur[NP];
    T y, uy;
  };
  const int ylane = (lane & 15) < DSH ? (lane & 15) : DSH - 1;
  auto load_j = [&](int e, int j, int rr, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ hj = h + (int64_t)j * DIN * CC;
    const T* __restrict__ uhj = uh + (int64_t)j * DIN * CC;
    const T* __restrict__ re = PAIR ? R + (int64_t)rr * PC : R + ((int64_t)e - edge_begin) * PC;
    const T* __restrict__ ure = uR + (int64_t)e * PC;
    static_for<DIN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
      if constexpr (bwd_group_owns_l1(TBL, BGR, G, l1)) {
        b.h[m] = ldc<MASKED ? 0 : 1>(hj, m * CC + c0, on);
        b.uh[m] = ldc<MASKED ? 0 : 1>(uhj, m * CC + c0, on);
      }
    });
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (BGR.group[p] == G) {
        b.r[p] = ldc_nt<MASKED ? 0 : 1>(re, p * CC + c0, on);
        b.ur[p] = ldc_nt<MASKED ? 0 : 1>(ure, p * CC + c0, on);
      }
    });
    b.y = Y[((int64_t)e - edge_begin) * DSH + ylane];
    b.uy = uY[(int64_t)e * DSH + ylane];
  };
  auto compute = [&](int e, const Buf& b) __attribute__((always_inline)) {
    const int64_t el = (int64_t)e - edge_begin;
    T ye[16], uye[16];
#pragma unroll
    for (int k = 0; k < DSH; ++k) {
      ye[k] = lane_value(b.y, k);
      uye[k] = lane_value(b.uy, k);
    }
    T* __restrict__ we = w_hat + el * PC;
    T dy[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) dy[k] = T(0);
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (BGR.group[p] == G) {
        constexpr Path P = TBL.path[p];
        constexpr int n1 = 2 * P.l1 + 1, n2 = 2 * P.l2 + 1, n3 = 2 * P.l3 + 1;
        // w_hat and the y_hat partial from X1 = h . K and X2 = uh . K
        T w = T(0);
        static_for<n2>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          T x1 = T(0), x2 = T(0);
          static_for<n1>([&](auto m1c) {
            constexpr int m1 = decltype(m1c)::value;
            constexpr int k = m12_index(TBL, p, m1, m2);
            if constexpr (k >= 0) {
              T kv;
              if constexpr (kHoldK) {
                constexpr int kk = BGR.kofs[p] + k;
                kv = K[kk];
              } else {
                kv = T(0);
                static_for<n3>([&](auto m3c) {
                  constexpr int m3 = decltype(m3c)::value;
                  constexpr double cv = TBL.cg[p][m1][m2][m3];
                  constexpr int o = TBL.out_row(p, m3);
                  if constexpr (cv != 0.0) kv += T(cv) * gi[o];
                });
              }
              x1 += b.h[P.l1 * P.l1 + m1] * kv;
              x2 += b.uh[P.l1 * P.l1 + m1] * kv;
            }
          });
          w += uye[P.l2 * P.l2 + m2] * x1 + ye[P.l2 * P.l2 + m2] * x2;
          dy[P.l2 * P.l2 + m2] += b.ur[p] * x1 + b.r[p] * x2;
        });
        stc_nt<MASKED ? 0 : 1>(we, p * CC + c0, on, w);
        // g_hat: T(h, uR Y + R uY) + T(uh, R Y)
        T z[n2], zr[n2];
        static_for<n2>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          z[m2] = b.ur[p] * ye[P.l2 * P.l2 + m2] + b.r[p] * uye[P.l2 * P.l2 + m2];
          zr[m2] = b.r[p] * ye[P.l2 * P.l2 + m2];
        });
        static_for<n3>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          constexpr int o = TBL.out_row(p, m3);
          static_for<n1>([&](auto m1c) {
            constexpr int m1 = decltype(m1c)::value;
            if constexpr (TBL.midx[p][m1][m3] >= 0) {
              T t1 = T(0), t2 = T(0);
              static_for<n2>([&](auto m2c) {
                constexpr int m2 = decltype(m2c)::value;
                constexpr double cv = TBL.cg[p][m1][m2][m3];
                if constexpr (cv != 0.0) {
                  t1 += T(cv) * z[m2];
                  t2 += T(cv) * zr[m2];
                }
              });
              ga[o] += b.h[P.l1 * P.l1 + m1] * t1 + b.uh[P.l1 * P.l1 + m1] * t2;
            }
          });
        });
      }
    });
    const T tot = wave_reduce_scatter16<T>(dy);
    if (DSH == 16 || (lane >> 2) < DSH)
      yhp[((int64_t)part * n_chunk_edges + el) * DSH + (lane >> 2)] = tot;
  };
  if (e_hi - e_lo > 64 * kIdxWindows) {
    edge_loop<Buf>(e_lo, e_hi,
                   [&](int e, Buf& b) __attribute__((always_inline)) {
                     load_j(e, uniform(src[e]), PAIR ? r_row(Rrow, edge_begin, e) : 0, b);
                   },
                   compute);
  } else if (e_hi > e_lo) {
    RowIdx<kIdxWindows> si;
    si.init(src, e_lo, e_hi, lane);
    if constexpr (PAIR) {
      RowIdx<kIdxWindows> qi;
      qi.init_rows(Rrow, edge_begin, e_lo, e_hi, lane);
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) {
                       load_j(e, si.get(e - e_lo), qi.get(e - e_lo), b);
                     },
                     compute);
    } else {
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) { load_j(e, si.get(e - e_lo), 0, b); },
                     compute);
    }
  }
  T* __restrict__ gh = g_hat + (int64_t)i * DOUT * CC;
  static_for<DOUT>([&](auto oc) {
    constexpr int o = decltype(oc)::value;
    if constexpr (bwd_group_reads_row(TBL, BGR, G, o)) stc<MASKED ? 0 : 1>(gh, o * CC + c0, on, scale * ga[o]);
  });
}

template <typename T, int L1, int L2, int L3, int NG, bool MASKED, int G, bool PAIR>
__device__ __forceinline__ void tp_dbl_send_group(
    const int32_t* __restrict__ src, const int32_t* __restrict__ rev, int i, int e_lo, int e_hi,
    int64_t edge_begin, int CC, uint32_t c0, bool on, T scale, const T* __restrict__ Y,
    const T* __restrict__ uY, const T* __restrict__ R, const int32_t* __restrict__ Rrow,
    const T* __restrict__ uR, const T* __restrict__ Gr, T* __restrict__ x_hat) {
  constexpr int NP = TBL.np, DIN = TBL.din, DSH = TBL.dsh, DOUT = TBL.dout;
  static_assert(BGR.ok, "every wave group owns an l1 class");
  const int PC = NP * CC;
  const int lane = threadIdx.x % kTPWave;
  T xa[DIN];
#pragma unroll
  for (int m = 0; m < DIN; ++m) xa[m] = T(0);
  struct Buf {
    T g[DOUT];
    T r[NP];
    T ur[NP];
    T y, uy;
  };
  const int ylane = (lane & 15) < DSH ? (lane & 15) : DSH - 1;
  auto load_j = [&](int e, int j, int er, int rr, Buf& b) __attribute__((always_inline)) {
    const T* __restrict__ gj = Gr + (int64_t)j * DOUT * CC;
    const T* __restrict__ re = PAIR ? R + (int64_t)rr * PC : R + ((int64_t)e - edge_begin) * PC;
    const T* __restrict__ urr = uR + (int64_t)er * PC;
    static_for<DOUT>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      if constexpr (bwd_group_reads_row(TBL, BGR, G, o)) b.g[o] = ldc<MASKED ? 0 : 1>(gj, o * CC + c0, on);
    });
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (BGR.group[p] == G) {
        b.r[p] = ldc_nt<MASKED ? 0 : 1>(re, p * CC + c0, on);
        b.ur[p] = ldc<MASKED ? 0 : 1>(urr, p * CC + c0, on);
      }
    });
    b.y = Y[((int64_t)e - edge_begin) * DSH + ylane];
    b.uy = uY[(int64_t)er * DSH + ylane];
  };
  auto compute = [&](int, const Buf& b) __attribute__((always_inline)) {
    T ye[16], uye[16];
#pragma unroll
    for (int k = 0; k < DSH; ++k) {
      ye[k] = lane_value(b.y, k);
      uye[k] = lane_value(b.uy, k);
    }
    static_for<NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (BGR.group[p] == G) {
        constexpr Path P = TBL.path[p];
        constexpr int n1 = 2 * P.l1 + 1, n2 = 2 * P.l2 + 1, n3 = 2 * P.l3 + 1;
        constexpr T sg = (P.l2 & 1) ? T(-1) : T(1);
        T wv[n2];
        static_for<n2>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          wv[m2] = (sg * b.ur[p]) * ye[P.l2 * P.l2 + m2] + b.r[p] * uye[P.l2 * P.l2 + m2];
        });
        static_for<n1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          static_for<n2>([&](auto m2c) {
            constexpr int m2 = decltype(m2c)::value;
            if constexpr (TBL.m12nz(p, m1, m2)) {
              T kb = T(0);
              static_for<n3>([&](auto m3c) {
                constexpr int m3 = decltype(m3c)::value;
                constexpr double cv = TBL.cg[p][m1][m2][m3];
                constexpr int o = TBL.out_row(p, m3);
                if constexpr (cv != 0.0) kb += T(cv) * b.g[o];
              });
              xa[P.l1 * P.l1 + m1] += wv[m2] * kb;
            }
          });
        });
      }
    });
  };
  if (e_hi - e_lo > 64 * kIdxWindows) {
    edge_loop<Buf>(e_lo, e_hi,
                   [&](int e, Buf& b) __attribute__((always_inline)) {
                     load_j(e, uniform(src[e]), uniform(rev[e]), PAIR ? r_row(Rrow, edge_begin, e) : 0, b);
                   },
                   compute);
  } else if (e_hi > e_lo) {
    RowIdx<kIdxWindows> si, ri;
    si.init(src, e_lo, e_hi, lane);
    ri.init(rev, e_lo, e_hi, lane);
    if constexpr (PAIR) {
      RowIdx<kIdxWindows> qi;
      qi.init_rows(Rrow, edge_begin, e_lo, e_hi, lane);
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) {
                       load_j(e, si.get(e - e_lo), ri.get(e - e_lo), qi.get(e - e_lo), b);
                     },
                     compute);
    } else {
      edge_loop<Buf>(e_lo, e_hi,
                     [&](int e, Buf& b) __attribute__((always_inline)) {
                       load_j(e, si.get(e - e_lo), ri.get(e - e_lo), 0, b);
                     },
                     compute);
    }
  }
  T* __restrict__ xi = x_hat + (int64_t)i * DIN * CC;
  static_for<DIN>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    constexpr int l1 = m >= 9 ? 3 : m >= 4 ? 2 : m >= 1 ? 1 : 0;
    if constexpr (bwd_group_owns_l1(TBL, BGR, G, l1)) stc<MASKED ? 0 : 1>(xi, m * CC + c0, on, scale * xa[m]);
  });
}
#undef TBL
#undef BGR

template <typename T, int L1, int L2, int L3, int NG, bool MASKED, int NWC, bool PAIR>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_dbl_recv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
              int64_t row_end, int64_t edge_begin, int64_t n_chunk_edges, int C, T scale,
              const T* __restrict__ h, const T* __restrict__ uh, const T* __restrict__ Y,
              const T* __restrict__ uY, const T* __restrict__ R, const int32_t* __restrict__ Rrow,
              const T* __restrict__ uR, const T* __restrict__ Gr, T* __restrict__ g_hat, T* __restrict__ w_hat, T* __restrict__ yhp) {
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = xcd_block() * kTPWavesPerBlock + threadIdx.x / kTPWave;
  const int64_t row = row_begin + w / (NG * NWC);
  if (row >= row_end) return;
  const int i = uniform((int)row);
  const int rem = uniform((int)(w % (NG * NWC)));
  const int g = rem % NG, cw = rem / NG;
  const int CC = MASKED ? C : 64 * NWC;
  const uint32_t c0 = (uint32_t)(cw * 64 + lane);
  const bool on = (int)c0 < C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  static_for<NG>([&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (g == G)
      tp_dbl_recv_group<T, L1, L2, L3, NG, MASKED, G, PAIR>(src, i, e_lo, e_hi, edge_begin, n_chunk_edges, CC, c0, on,
                                                      rem, scale, h, uh, Y, uY, R, Rrow, uR, Gr, g_hat, w_hat, yhp);
  });
}

template <typename T, int L1, int L2, int L3, int NG, bool MASKED, int NWC, bool PAIR>
__global__ void __launch_bounds__(kTPWave * kTPWavesPerBlock)
k_tp_dbl_send(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
              const int32_t* __restrict__ rev, int64_t row_begin, int64_t row_end, int64_t edge_begin,
              int C, T scale, const T* __restrict__ Y, const T* __restrict__ uY, const T* __restrict__ R,
              const int32_t* __restrict__ Rrow, const T* __restrict__ uR, const T* __restrict__ Gr,
              T* __restrict__ x_hat) {
  const int lane = threadIdx.x % kTPWave;
  const int64_t w = xcd_block() * kTPWavesPerBlock + threadIdx.x / kTPWave;
  const int64_t row = row_begin + w / (NG * NWC);
  if (row >= row_end) return;
  const int i = uniform((int)row);
  const int rem = uniform((int)(w % (NG * NWC)));
  const int g = rem % NG, cw = rem / NG;
  const int CC = MASKED ? C : 64 * NWC;
  const uint32_t c0 = (uint32_t)(cw * 64 + lane);
  const bool on = (int)c0 < C;
  const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
  static_for<NG>([&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (g == G)
      tp_dbl_send_group<T, L1, L2, L3, NG, MASKED, G, PAIR>(src, rev, i, e_lo, e_hi, edge_begin, CC, c0, on, scale, Y,
                                                      uY, R, Rrow, uR, Gr, x_hat);
  });
}

}  // namespace tpc
