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

template <typename T, int L1, int L2, int L3, bool SUM>
hipError_t fwd_launch(const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  constexpr int DOUT = kTable<L1, L2, L3, SUM>.dout;
  const bool masked = a.C < 64;
  const int cpl = a.C == 128 ? 2 : 1;
  const int ng = DOUT * cpl >= 64 ? 2 : 1;
  const unsigned blocks = (unsigned)((rows * ng + kTPWavesPerBlock - 1) / kTPWavesPerBlock);
  const T sc = (T)a.scale;
  const T* h = static_cast<const T*>(a.h);
  const T* Y = static_cast<const T*>(a.Y);
  const T* R = static_cast<const T*>(a.R);
  T* out = static_cast<T*>(a.out);
#define TPC_GO(CPL, NG, MASK)                                                                    \
  k_tp_fwd<T, L1, L2, L3, SUM, CPL, NG, MASK><<<blocks, kTPWave * kTPWavesPerBlock, 0, s>>>(     \
      a.row_ptr, a.src, a.row_begin, a.row_end, a.edge_begin, a.C, sc, h, Y, R, out)
  if (masked) {
    TPC_GO(1, 1, true);
  } else if (cpl == 1) {
    if (ng == 2) TPC_GO(1, 2, false); else TPC_GO(1, 1, false);
  } else {
    if (ng == 2) TPC_GO(2, 2, false); else TPC_GO(2, 1, false);
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
