// Fused forward tensor-product kernel for one built configuration (compiled
// once per configuration index, -DTPC_CFG=<index>).
#include "tp_config.hpp"
#include "tp_impl.hpp"

#ifndef TPC_CFG
#error "tp_fwd.hip is compiled once per configuration with -DTPC_CFG=<index>"
#endif

namespace tpc {

// Waves of a row: C = 128 takes two 64-channel waves, each over every path
// (sender features and radial weights are then read once per edge); C = 64
// splits the paths over two waves when the output block is large, three at
// node l <= 3 (by whole l1 classes where that balances, so each wave reads
// only its rows of h; three waves hold about 130 registers each, four waves
// per SIMD); C < 64 masks the lanes past C.
template <typename T, int L1, int L2, int L3, bool SUM>
hipError_t fwd_launch(const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  constexpr int DOUT = kTable<L1, L2, L3, SUM>.dout;
  const bool masked = a.C < 64;
  const int ng = DOUT >= 96 ? 3 : DOUT >= 64 ? 2 : 1;
  const T sc = (T)a.scale;
  const T* h = static_cast<const T*>(a.h);
  const T* Y = static_cast<const T*>(a.Y);
  const T* R = static_cast<const T*>(a.R);
  T* out = static_cast<T*>(a.out);
#define TPC_GO_P(NG, MASK, NWC, PAIR)                                                            \
  k_tp_fwd<T, L1, L2, L3, SUM, 1, NG, MASK, NWC, PAIR>                                          \
      <<<(unsigned)((rows * NG * NWC + kTPWavesPerBlock - 1) / kTPWavesPerBlock),               \
         kTPWave * kTPWavesPerBlock, 0, s>>>(a.row_ptr, a.src, a.row_begin, a.row_end,           \
                                             a.edge_begin, a.C, sc, h, Y, R, a.Rrow, out)
  // R rows shared by edge pairs (a.Rrow) are built for the unmasked channel
  // counts only
#define TPC_GO(NG, MASK, NWC)                         \
  do {                                                \
    if (a.Rrow) TPC_GO_P(NG, MASK, NWC, true);        \
    else TPC_GO_P(NG, MASK, NWC, false);              \
  } while (0)
  if (masked) {
    if (a.Rrow) return hipErrorInvalidValue;
    TPC_GO_P(1, true, 1, false);
  } else if (a.C == 128) {
    TPC_GO(1, false, 2);
  } else {
    if (ng == 3) TPC_GO(3, false, 1);
    else if (ng == 2) TPC_GO(2, false, 1);
    else TPC_GO(1, false, 1);
  }
#undef TPC_GO
#undef TPC_GO_P
  return hipGetLastError();
}

template <typename T, int L1, int L2, int L3>
hipError_t tp_fwd_cfg(const TPArgs& a, hipStream_t s) {
  if (a.row_end - a.row_begin <= 0) return hipSuccess;
  return a.sum_paths ? fwd_launch<T, L1, L2, L3, true>(a, s) : fwd_launch<T, L1, L2, L3, false>(a, s);
}

using Cfg = TpCfg<TPC_CFG>;
template hipError_t tp_fwd_cfg<Cfg::T, Cfg::L1, Cfg::L2, Cfg::L3>(const TPArgs&, hipStream_t);

}  // namespace tpc
