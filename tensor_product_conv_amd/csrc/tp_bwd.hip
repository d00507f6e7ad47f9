// Receiver-side backward kernel (dR, partial dY and the per-edge dh
// contributions) for one built configuration (compiled once per configuration
// index, -DTPC_CFG=<index>).
#include "tp_config.hpp"
#include "tp_impl.hpp"

#ifndef TPC_CFG
#error "tp_bwd.hip is compiled once per configuration with -DTPC_CFG=<index>"
#endif

namespace tpc {

template <typename T, int L1, int L2, int L3, bool SUM, bool MASKED, int NWC, bool PAIR>
hipError_t bwd_launch(const TPArgs& a, hipStream_t s) {
  constexpr int NG = bwd_groups(sizeof(T) == 8, L1);
  const int64_t waves = (a.row_end - a.row_begin) * NG * NWC;
  k_tp_bwd_edge<T, L1, L2, L3, SUM, MASKED, NG, NWC, PAIR>
      <<<(unsigned)((waves + kTPWavesPerBlock - 1) / kTPWavesPerBlock), kTPWave * kTPWavesPerBlock, 0, s>>>(
          a.row_ptr, a.src, a.row_begin, a.row_end, a.edge_begin, a.n_chunk_edges, a.C, (T)a.scale,
          static_cast<const T*>(a.h), static_cast<const T*>(a.Y), static_cast<const T*>(a.R),
          a.Rrow, static_cast<const T*>(a.G), static_cast<T*>(a.dR), static_cast<T*>(a.dY), static_cast<T*>(a.dh_edge));
  return hipGetLastError();
}

// Per row: one wave per 64-channel slice and l1-class group (one masked
// slice for C < 64).
template <typename T, int L1, int L2, int L3>
hipError_t tp_bwd_cfg(const TPArgs& a, hipStream_t s) {
  if (a.row_end - a.row_begin <= 0) return hipSuccess;
// R rows shared by edge pairs (a.Rrow): unmasked channel counts only.
#define TPC_GO(S)                                                                         \
  if (a.C < 64) return a.Rrow ? hipErrorInvalidValue : bwd_launch<T, L1, L2, L3, S, true, 1, false>(a, s); \
  if (a.C == 64)                                                                          \
    return a.Rrow ? bwd_launch<T, L1, L2, L3, S, false, 1, true>(a, s)                     \
                  : bwd_launch<T, L1, L2, L3, S, false, 1, false>(a, s);                   \
  if (a.C == 128)                                                                         \
    return a.Rrow ? bwd_launch<T, L1, L2, L3, S, false, 2, true>(a, s)                     \
                  : bwd_launch<T, L1, L2, L3, S, false, 2, false>(a, s);                   \
  return hipErrorInvalidValue;
  if (a.sum_paths) {
    TPC_GO(true)
  } else {
    TPC_GO(false)
  }
#undef TPC_GO
}

using Cfg = TpCfg<TPC_CFG>;
template hipError_t tp_bwd_cfg<Cfg::T, Cfg::L1, Cfg::L2, Cfg::L3>(const TPArgs&, hipStream_t);

}  // namespace tpc
