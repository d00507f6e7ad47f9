// Receiver-side backward kernel (dR, partial dY and the per-edge dh
// contributions) for one built configuration (compiled once per configuration
// index, -DTPC_CFG=<index>).
#include "tp_config.hpp"
#include "tp_impl.hpp"

#ifndef TPC_CFG
#error "tp_bwd.hip is compiled once per configuration with -DTPC_CFG=<index>"
#endif

namespace tpc {

template <typename T, int L1, int L2, int L3, bool SUM, int NW>
hipError_t bwd_launch(const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  const int64_t waves = rows * (NW > 0 ? NW : 1);
  k_tp_bwd_edge<T, L1, L2, L3, SUM, NW>
      <<<(unsigned)((waves + kTPWavesPerBlock - 1) / kTPWavesPerBlock), kTPWave * kTPWavesPerBlock, 0, s>>>(
          a.row_ptr, a.src, a.rev, a.row_begin, a.row_end, a.edge_begin, a.n_chunk_edges, a.C, (T)a.scale,
          static_cast<const T*>(a.h), static_cast<const T*>(a.Y), static_cast<const T*>(a.R),
          static_cast<const T*>(a.G), static_cast<T*>(a.dR), static_cast<T*>(a.dY), static_cast<T*>(a.dh_edge));
  return hipGetLastError();
}

// One wave per row and 64 channels (NW = C / 64), or one masked wave for
// C < 64.
template <typename T, int L1, int L2, int L3>
hipError_t tp_bwd_cfg(const TPArgs& a, hipStream_t s) {
  if (a.row_end - a.row_begin <= 0) return hipSuccess;
#define TPC_GO(S)                                                                  \
  if (a.C < 64) return bwd_launch<T, L1, L2, L3, S, 0>(a, s);                      \
  if (a.C == 64) return bwd_launch<T, L1, L2, L3, S, 1>(a, s);                     \
  if (a.C == 128) return bwd_launch<T, L1, L2, L3, S, 2>(a, s);                    \
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
