// Forward tensor product with the fused radial last layer for one built
// configuration (compiled once per configuration index, -DTPC_CFG=<index>;
// float32 configurations only, the float64 ones compile a stub).
#include "tp_config.hpp"
#include "tp_fused.hpp"

#ifndef TPC_CFG
#error "tp_fused.hip is compiled once per configuration with -DTPC_CFG=<index>"
#endif

namespace tpc {

// One block per CU: a block holds 8 waves of up to 256 registers (2 per
// SIMD) and most of the LDS.  Row groups come in multiples of 8 so that every
// XCD holds whole row groups (all their slices).
template <int L1, int L2, int L3, bool SUM, int KB, bool STORE_R>
hipError_t fused_launch(const TPArgs& a, hipStream_t s) {
  constexpr int NP = kTable<L1, L2, L3, SUM>.np;
  const size_t lds = (size_t)NP * 64 * KB * 24 * sizeof(__bf16) + (size_t)kFuWaves * 256 * sizeof(float);
  auto kern = k_tp_fwd_fused<L1, L2, L3, SUM, KB, STORE_R>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int ns = a.C / 16;
  int64_t ngroups = kFusedBlocks / ns;
  ngroups = ngroups < 8 ? 8 : ngroups / 8 * 8;
  const unsigned blocks = (unsigned)(ngroups * ns);
  kern<<<blocks, 64 * kFuWaves, lds, s>>>(a.row_ptr, a.src, a.row_begin, a.row_end, a.edge_begin, a.C,
                                          (float)a.scale, static_cast<const float*>(a.h),
                                          static_cast<const float*>(a.Y), static_cast<const __bf16*>(a.act),
                                          static_cast<const __bf16*>(a.wfs), static_cast<float*>(a.R_out),
                                          static_cast<float*>(a.out));
  return hipGetLastError();
}

template <typename T, int L1, int L2, int L3>
hipError_t tp_fused_cfg(const TPArgs& a, hipStream_t s) {
  if constexpr (!std::is_same<T, float>::value) {
    return hipErrorInvalidValue;
  } else {
    if (a.row_end - a.row_begin <= 0) return hipSuccess;
    if (a.C % 16 != 0 || (a.H != 32 && a.H != 64)) return hipErrorInvalidValue;
#define TPC_GO(SUMP, KB)                                                               \
  return a.R_out ? fused_launch<L1, L2, L3, SUMP, KB, true>(a, s) : fused_launch<L1, L2, L3, SUMP, KB, false>(a, s)
    if (a.sum_paths) {
      if (a.H == 64) TPC_GO(true, 2);
      TPC_GO(true, 1);
    }
    if (a.H == 64) TPC_GO(false, 2);
    TPC_GO(false, 1);
#undef TPC_GO
  }
}

using Cfg = TpCfg<TPC_CFG>;
template hipError_t tp_fused_cfg<Cfg::T, Cfg::L1, Cfg::L2, Cfg::L3>(const TPArgs&, hipStream_t);

}  // namespace tpc
