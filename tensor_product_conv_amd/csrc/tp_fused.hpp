// Forward convolution with the radial network's last layer fused into the
// tensor-product kernel (the fused folded forward of FastMACE's "Rewrites and
// precision options", section "Convolution (OEq streaming)": the per-edge
// weights are formed inside the streaming convolution instead of being
// stored and read back).  Float32, bf16-split matrix products (three bf16
// parts per operand, six cross terms: float32 accuracy).
//
// Work split.  A block owns one 16-channel slice of the output and keeps the
// last-layer weights of that slice's columns, for every path, in LDS
// (P x 64 lanes x H/32 x 24 bf16, already in matrix-core operand order),
// followed by each wave's 16 x 16 staging rows for a batch's harmonics; it
// streams a contiguous range of receiver rows through its waves, and the
// blocks of all slices of a row range sit on one XCD so the sender features
// and activations they share stay in that XCD's L2.  A wave takes one row at
// a time in batches of 16 edges.  Per batch and path one 16x16 product
//     D[e][n] = sum_k A[e][k] W_L[k][p*C + 16*slice + n]
// (A: the edge's last hidden activations, stored pre-split by k_radial_act)
// leaves R[e][p][n] in the lane that owns channel n and edges 4g..4g+3 of the
// batch (g = lane / 16): exactly the layout the tensor product wants, so R
// never leaves the registers.  Each lane then accumulates the product of its
// four edges for its channel, and at the end of the row the four lane groups'
// partial sums are added by permlane swaps (a fixed order: every output is a
// deterministic sum) and stored once.
#pragma once

#include "tp_impl.hpp"

namespace tpc {

constexpr int kFuWaves = 8;  // waves per block

typedef __bf16 fu_bf16x8 __attribute__((ext_vector_type(8)));
typedef float fu_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ fu_f32x4 fu_mfma(fu_bf16x8 a, fu_bf16x8 b, fu_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// c += A B from the three bf16 parts of each operand: the six terms whose
// weight is at least 2^-16 of the leading one, smallest first.
__device__ __forceinline__ fu_f32x4 fu_x6(const fu_bf16x8 (&a)[3], const fu_bf16x8 (&b)[3], fu_f32x4 c) {
  c = fu_mfma(a[2], b[0], c);
  c = fu_mfma(a[0], b[2], c);
  c = fu_mfma(a[1], b[1], c);
  c = fu_mfma(a[1], b[0], c);
  c = fu_mfma(a[0], b[1], c);
  c = fu_mfma(a[0], b[0], c);
  return c;
}

// Rows [r0, r1) of row group `grp` of `ngroups` over [row_begin, row_end).
__device__ __forceinline__ void fu_rows(int64_t row_begin, int64_t row_end, int64_t grp, int64_t ngroups,
                                        int64_t* r0, int64_t* r1) {
  const int64_t n = row_end - row_begin;
  *r0 = row_begin + n * grp / ngroups;
  *r1 = row_begin + n * (grp + 1) / ngroups;
}

// Copy the slice's last-layer weights (section fs of the radial pack: column
// block b of 16 columns at b * 64 * KB * 24 bf16, lane-major) into LDS:
// path p's block is p * (C / 16) + slice.
template <int NP, int KB>
__device__ __forceinline__ void fu_load_weights(const __bf16* __restrict__ fs, int ns, int slice, __bf16* wsl) {
  constexpr int WPP = 64 * KB * 24;           // bf16 per path
  constexpr int V = WPP / 8;                  // 16-byte vectors per path
  for (int t = threadIdx.x; t < NP * V; t += blockDim.x) {
    const int p = t / V, v = t % V;
    const int64_t blk = (int64_t)p * ns + slice;
    reinterpret_cast<fu_bf16x8*>(wsl)[t] = reinterpret_cast<const fu_bf16x8*>(fs + blk * WPP)[v];
  }
}

// Sum of acc over the four 16-lane groups of the wave, scattered: afterwards
// lane (g, n) holds in v[k] the total of row k + Q g (Q = ceil(D / 4)).
template <int D>
__device__ __forceinline__ void fu_group_sum(const float (&acc)[D][1], float (&v)[(D + 3) / 4]) {
  constexpr int Q = (D + 3) / 4;
  auto at = [&](int k) __attribute__((always_inline)) { return k < D ? acc[k][0] : 0.f; };
  float a[2 * Q];
#pragma unroll
  for (int k = 0; k < 2 * Q; ++k) a[k] = swap32_add(at(k), at(k + 2 * Q));
#pragma unroll
  for (int k = 0; k < Q; ++k) v[k] = swap16_add(a[k], a[k + Q]);
}

// One path's contribution of one edge for one channel:
//   acc[(p, m3)] += sum_m1 (sum_m2 C^p[m1][m2][m3] Y[(l2, m2)]) R h[(l1, m1)]
// with the sparsity of C^p unrolled at compile time.
template <int L1, int L2, int L3, bool SUM, int p>
__device__ __forceinline__ void fu_path(const float (&hh)[kTable<L1, L2, L3, SUM>.din], float R,
                                        const float (&ye)[16], float (&acc)[kTable<L1, L2, L3, SUM>.dout][1]) {
  constexpr Path P = kTable<L1, L2, L3, SUM>.path[p];
  float hr[2 * P.l1 + 1];
#pragma unroll
  for (int m1 = 0; m1 < 2 * P.l1 + 1; ++m1) hr[m1] = R * hh[P.l1 * P.l1 + m1];
  static_for<2 * P.l3 + 1>([&](auto m3c) {
    constexpr int m3 = decltype(m3c)::value;
    constexpr int row = kTable<L1, L2, L3, SUM>.out_row(p, m3);
    static_for<2 * P.l1 + 1>([&](auto m1c) {
      constexpr int m1 = decltype(m1c)::value;
      if constexpr (kTable<L1, L2, L3, SUM>.midx[p][m1][m3] >= 0) {
        float M = 0.f;
        static_for<2 * P.l2 + 1>([&](auto m2c) {
          constexpr int m2 = decltype(m2c)::value;
          constexpr double cv = kTable<L1, L2, L3, SUM>.cg[p][m1][m2][m3];
          if constexpr (cv != 0.0) M += float(cv) * ye[P.l2 * P.l2 + m2];
        });
        acc[row][0] += M * hr[m1];
      }
    });
  });
}

// STORE_R: also store R for a backward that reads it.  Stores go through a
// buffer descriptor that covers the batch's valid edges only: the hardware
// drops a lane's store past its end, so the batch body has no branches (a
// branch would split it into blocks across which the compiler moves the
// arithmetic away from its loads).
template <int L1, int L2, int L3, bool SUM, int KB, bool STORE_R>
__global__ void __launch_bounds__(64 * kFuWaves)
k_tp_fwd_fused(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src, int64_t row_begin,
               int64_t row_end, int64_t edge_begin, int C, float scale, const float* __restrict__ h,
               const float* __restrict__ Y, const __bf16* __restrict__ act, const __bf16* __restrict__ fs,
               float* __restrict__ R, float* __restrict__ out) {
#define TBL kTable<L1, L2, L3, SUM>
  constexpr int NP = TBL.np, DIN = TBL.din, DSH = TBL.dsh, DOUT = TBL.dout;
  constexpr int Q = (DOUT + 3) / 4;
  constexpr int WPL = KB * 24, WPP = 64 * WPL;
  extern __shared__ __attribute__((aligned(16))) __bf16 wsl[];
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const int g = lane / 16, el = lane % 16;
  const int ns = C / 16;
  const int64_t lb = xcd_block();
  const int slice = (int)(lb % ns);
  const int64_t ngroups = gridDim.x / ns;
  int64_t r0, r1;
  fu_rows(row_begin, row_end, lb / ns, ngroups, &r0, &r1);
  fu_load_weights<NP, KB>(fs, ns, slice, wsl);
  __syncthreads();

  const __bf16* wl = wsl + lane * WPL;
  float* ysh = reinterpret_cast<float*>(wsl + NP * WPP) + wv * 256;  // this wave's 16 x 16 harmonics
  const int c = slice * 16 + el;  // this lane's channel
  const int PC = NP * C;
  for (int64_t row = r0 + wv; row < r1; row += kFuWaves) {
    const int i = uniform((int)row);
    const int e_lo = uniform(row_ptr[i]), e_hi = uniform(row_ptr[i + 1]);
    float acc[DOUT][1];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) acc[k][0] = 0.f;
    for (int eb = e_lo; eb < e_hi; eb += 16) {
      // the lane's edges of the batch and their senders
      int jr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) jr[r] = src[min(eb + 4 * g + r, e_hi - 1)];
      // A operand: activations of edge eb + el (zero past the row's end)
      fu_bf16x8 A[KB][3];
      {
        const bool va = eb + el < e_hi;
        const int64_t ea = (int64_t)min(eb + el, e_hi - 1) - edge_begin;
        const fu_bf16x8* ap = reinterpret_cast<const fu_bf16x8*>(act + ea * (KB * 96)) + g * 3;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int part = 0; part < 3; ++part) {
            const fu_bf16x8 x = ap[kb * 12 + part];
            A[kb][part] = va ? x : fu_bf16x8{};
          }
      }
      // harmonics of the batch's 16 edges into this wave's LDS rows (lane l
      // copies entries 4 (l % 4) .. 4 (l % 4) + 3 of edge l / 4); every lane
      // of a 16-lane group then reads its edges' entries as broadcasts.  The
      // writes complete (s_waitcnt lgkmcnt(0)) before any lane reads; the
      // previous batch's reads were consumed before these writes were issued.
      {
        const int ey = lane / 4, q = lane % 4;
        const int64_t ec = (int64_t)min(eb + ey, e_hi - 1) - edge_begin;
        float* dst = ysh + ey * 16 + 4 * q;
        if constexpr (DSH % 4 == 0) {
          if (4 * q < DSH) *reinterpret_cast<fu_f32x4*>(dst) = reinterpret_cast<const fu_f32x4*>(Y + ec * DSH)[q];
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (4 * q + t < DSH) dst[t] = Y[ec * DSH + 4 * q + t];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
      }
      // sender features of the lane's edges, one edge ahead of its use (zero
      // past the row's end, so those edges add nothing); the first edge's
      // loads fly while the products below run
      auto load_h = [&](int r, float (&hv)[DIN]) __attribute__((always_inline)) {
        const bool ve = eb + 4 * g + r < e_hi;
        const float* hj = h + (int64_t)jr[r] * DIN * C + c;
#pragma unroll
        for (int m = 0; m < DIN; ++m) {
          const float x = hj[m * C];
          hv[m] = ve ? x : 0.f;
        }
      };
      auto load_y = [&](int r, float (&yv)[16]) __attribute__((always_inline)) {
        const float* yr = ysh + (4 * g + r) * 16;
        if constexpr (DSH % 4 == 0) {
#pragma unroll
          for (int q = 0; q < DSH / 4; ++q) {
            const fu_f32x4 v = reinterpret_cast<const fu_f32x4*>(yr)[q];
#pragma unroll
            for (int t = 0; t < 4; ++t) yv[4 * q + t] = v[t];
          }
        } else {
#pragma unroll
          for (int k = 0; k < DSH; ++k) yv[k] = yr[k];
        }
      };
      float hh[2][DIN], ye[2][16];
      load_h(0, hh[0]);
      // R of the batch's valid edges: [min(16, e_hi - eb)][P*C] from edge eb
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          STORE_R ? R + ((int64_t)eb - edge_begin) * PC : R, 0, STORE_R ? min(16, e_hi - eb) * PC * 4 : 0,
          0x00020000);
      uint32_t ro[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ro[r] = STORE_R ? (uint32_t)(((4 * g + r) * PC + c) * 4) : 0u;
      // R of the batch for every path: lane (g, n) receives R[edge 4g + r][p][n]
      // (17 independent product chains at P = 17 keep the matrix unit busy)
      float Rv[NP][4];
      static_for<NP>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        fu_f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          fu_bf16x8 b[3];
#pragma unroll
          for (int part = 0; part < 3; ++part)
            b[part] = *reinterpret_cast<const fu_bf16x8*>(wl + p * WPP + kb * 24 + part * 8);
          d = fu_x6(A[kb], b, d);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Rv[p][r] = d[r];
        if constexpr (STORE_R) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // copy the element out first: a bit cast of a vector-element
            // expression reads element 0 here, whatever the index
            const float x = d[r];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, ro[r] + p * C * 4, 0, 0);
          }
        }
      });
      // then edge by edge (the next edge's features and harmonics loading):
      // every path's contribution
      load_y(0, ye[0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < 3) {
          load_h(r + 1, hh[(r + 1) & 1]);
          load_y(r + 1, ye[(r + 1) & 1]);
        }
        static_for<NP>([&](auto pc) {
          constexpr int p = decltype(pc)::value;
          fu_path<L1, L2, L3, SUM, p>(hh[r & 1], Rv[p][r], ye[r & 1], acc);
        });
      }
    }
    float v[Q];
    fu_group_sum<DOUT>(acc, v);
    // rows k + Q g of this lane: a per-row base plus the uniform offset k C
    // (the per-lane row offsets, hoisted, would each hold a register)
    int og = Q * g * C + c;
    asm volatile("" : "+v"(og));
    float* oi = out + (int64_t)i * DOUT * C + og;
#pragma unroll
    for (int k = 0; k < Q; ++k)
      if (k + Q * g < DOUT) oi[k * C] = scale * v[k];
  }
#undef TBL
}

}  // namespace tpc
