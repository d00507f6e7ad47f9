// Instantiations of the fused forward tensor-product kernel.
#include "tp_impl.hpp"

namespace tpc {

bool tp_supported(int dtype, int L1, int L2, int L3, int C) {
  if (!tp_channels_ok(C)) return false;
#define TPC_X(T, A, B, D) \
  if (dtype == tp_detail::dtype_id<T>() && L1 == A && L2 == B && L3 == D) return true;
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return false;
}

namespace {

// Waves of a row: C = 128 takes two 64-channel waves, each over every path
// (sender features and radial weights are then read once per edge); C = 64
// splits the paths over two waves when the output block is large (by whole
// l1 classes where that balances, so each wave reads only its rows of h);
// C < 64 masks the lanes past C.
template <typename T, int L1, int L2, int L3, bool SUM>
hipError_t fwd_launch(const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  constexpr int DOUT = kTable<L1, L2, L3, SUM>.dout;
  const bool masked = a.C < 64;
  const int ng = DOUT >= 64 ? 2 : 1;
  const T sc = (T)a.scale;
  const T* h = static_cast<const T*>(a.h);
  const T* Y = static_cast<const T*>(a.Y);
  const T* R = static_cast<const T*>(a.R);
  T* out = static_cast<T*>(a.out);
#define TPC_GO(NG, MASK, NWC)                                                                    \
  k_tp_fwd<T, L1, L2, L3, SUM, 1, NG, MASK, NWC>                                                \
      <<<(unsigned)((rows * NG * NWC + kTPWavesPerBlock - 1) / kTPWavesPerBlock),               \
         kTPWave * kTPWavesPerBlock, 0, s>>>(a.row_ptr, a.src, a.row_begin, a.row_end,           \
                                             a.edge_begin, a.C, sc, h, Y, R, out)
  if (masked) {
    TPC_GO(1, true, 1);
  } else if (a.C == 128) {
    TPC_GO(1, false, 2);
  } else {
    if (ng == 2) TPC_GO(2, false, 1); else TPC_GO(1, false, 1);
  }
#undef TPC_GO
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tp_fwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
  if (a.row_end - a.row_begin <= 0) return hipSuccess;
#define TPC_X(T, A, B, D) \
  if (dtype == tp_detail::dtype_id<T>() && L1 == A && L2 == B && L3 == D)                  \
    return a.sum_paths ? fwd_launch<T, A, B, D, true>(a, s) : fwd_launch<T, A, B, D, false>(a, s);
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return hipErrorInvalidValue;
}

}  // namespace tpc
