// Built configurations of the fused tensor-product kernels, shared by the
// per-configuration kernel objects and the host dispatch.
//
// Each configuration (dtype, node_lmax, sh_lmax, out_lmax) compiles in its own
// object: the kernel sources tp_fwd.hip and tp_bwd.hip are built once per
// index with -DTPC_CFG=<index>, and tp_dispatch.hip routes a call to the
// matching instantiation.  Channels: 1..64 (lanes past C masked) or 128.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

// Float64 is built for node_lmax <= 1 only: at node_lmax 2 and 3 its
// backward's live state (twice as wide as float32) exceeds the register file
// and spills to scratch memory, so those requests are refused instead.
#define TPC_TP_CONFIGS(X)                                                                 \
  X(0, float, 1, 2, 1) X(1, float, 1, 3, 3) X(2, float, 2, 3, 3) X(3, float, 3, 3, 3)     \
  X(4, double, 1, 2, 1) X(5, double, 1, 3, 3)
#define TPC_TP_N_CONFIGS 6

namespace tpc {

template <int I>
struct TpCfg;
#define TPC_CFG_TRAIT(I, T_, A, B, D)   \
  template <>                           \
  struct TpCfg<I> {                     \
    using T = T_;                       \
    static constexpr int L1 = A, L2 = B, L3 = D; \
  };
TPC_TP_CONFIGS(TPC_CFG_TRAIT)
#undef TPC_CFG_TRAIT

// Waves per row and 64-channel slice in the backward and the double
// backward: whole l1 classes per wave.  Float64 splits further (its
// registers are twice as wide).
constexpr int bwd_groups(bool f64, int L1) {
  if (f64) return L1 + 1;
  return L1 <= 1 ? 1 : L1;
}
// 64-channel slices per row (1 for C <= 64)
constexpr int channel_slices(int C) { return C <= 64 ? 1 : C / 64; }
// Partial dY (backward) and y_hat (double backward) slices: one per wave of
// a row.
constexpr int bwd_parts(bool f64, int L1, int C) { return bwd_groups(f64, L1) * channel_slices(C); }

template <typename T, int L1, int L2, int L3>
hipError_t tp_fwd_cfg(const TPArgs& a, hipStream_t s);
template <typename T, int L1, int L2, int L3>
hipError_t tp_bwd_cfg(const TPArgs& a, hipStream_t s);
template <typename T, int L1, int L2, int L3>
hipError_t tp_dbl_cfg(const TPArgs& a, hipStream_t s);
template <typename T, int L1, int L2, int L3>
hipError_t tp_fused_cfg(const TPArgs& a, hipStream_t s);

// Blocks of the fused forward (one per CU).
constexpr int kFusedBlocks = 256;

}  // namespace tpc
