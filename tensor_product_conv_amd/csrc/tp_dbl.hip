// VJP-of-VJP kernels (g_hat, w_hat, partial y_hat; x_hat) for one built
// configuration (compiled once per configuration index, -DTPC_CFG=<index>).
#include "tp_config.hpp"
#include "tp_impl.hpp"

#ifndef TPC_CFG
#error "tp_dbl.hip is compiled once per configuration with -DTPC_CFG=<index>"
#endif

namespace tpc {

template <typename T, int L1, int L2, int L3>
hipError_t tp_dbl_cfg(const TPArgs& a, hipStream_t s) {
  constexpr int NG = bwd_groups(sizeof(T) == 8, L1);
  const int64_t rows = a.row_end - a.row_begin;
  if (rows <= 0) return hipSuccess;
  if (a.sum_paths) return hipErrorInvalidValue;
  const T sc = (T)a.scale;
#define TPC_GO_P(MASK, NWC, PAIR)                                                                 \
  do {                                                                                            \
    const unsigned blocks = (unsigned)((rows * NG * NWC + kTPWavesPerBlock - 1) / kTPWavesPerBlock); \
    k_tp_dbl_recv<T, L1, L2, L3, NG, MASK, NWC, PAIR><<<blocks, kTPWave * kTPWavesPerBlock, 0, s>>>(    \
        a.row_ptr, a.src, a.row_begin, a.row_end, a.edge_begin, a.n_chunk_edges, a.C, sc,        \
        static_cast<const T*>(a.h), static_cast<const T*>(a.uh), static_cast<const T*>(a.Y),     \
        static_cast<const T*>(a.uY), static_cast<const T*>(a.R), a.Rrow,                         \
        static_cast<const T*>(a.uR), static_cast<const T*>(a.G), static_cast<T*>(a.g_hat), static_cast<T*>(a.w_hat),          \
        static_cast<T*>(a.dY));                                                                   \
    k_tp_dbl_send<T, L1, L2, L3, NG, MASK, NWC, PAIR><<<blocks, kTPWave * kTPWavesPerBlock, 0, s>>>(    \
        a.row_ptr, a.src, a.rev, a.row_begin, a.row_end, a.edge_begin, a.C, sc,                  \
        static_cast<const T*>(a.Y), static_cast<const T*>(a.uY), static_cast<const T*>(a.R),     \
        a.Rrow, static_cast<const T*>(a.uR), static_cast<const T*>(a.G), static_cast<T*>(a.x_hat));      \
  } while (0)
  // R rows shared by edge pairs (a.Rrow): unmasked channel counts only
#define TPC_GO(MASK, NWC)                  \
  do {                                     \
    if (a.Rrow) TPC_GO_P(MASK, NWC, true); \
    else TPC_GO_P(MASK, NWC, false);       \
  } while (0)
  if (a.C < 64) {
    if (a.Rrow) return hipErrorInvalidValue;
    TPC_GO_P(true, 1, false);
  } else if (a.C == 64) {
    TPC_GO(false, 1);
  } else if (a.C == 128) {
    TPC_GO(false, 2);
  } else {
    return hipErrorInvalidValue;
  }
#undef TPC_GO
#undef TPC_GO_P
  return hipGetLastError();
}

using Cfg = TpCfg<TPC_CFG>;
template hipError_t tp_dbl_cfg<Cfg::T, Cfg::L1, Cfg::L2, Cfg::L3>(const TPArgs&, hipStream_t);

}  // namespace tpc
