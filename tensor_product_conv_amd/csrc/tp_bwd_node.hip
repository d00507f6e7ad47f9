// Instantiations of the reverse-row backward kernel (dh without atomics).
#include "tp_impl.hpp"

namespace tpc {

hipError_t launch_tp_bwd_node(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  if (rows <= 0) return hipSuccess;
  const int cpl = tp_cpl(a.C);
#define TPC_X(T, A, B, D, K)                                                                   \
  if (dtype == tp_detail::dtype_id<T>() && L1 == A && L2 == B && L3 == D && cpl == K) {        \
    k_tp_bwd_node<T, A, B, D, K><<<tp_blocks(rows), kTPWave * kTPWavesPerBlock, 0, s>>>(       \
        a.row_ptr, a.src, a.row_begin, a.row_end, a.edge_begin, a.C, (T)a.scale,               \
        static_cast<const T*>(a.Y), static_cast<const T*>(a.R), static_cast<const T*>(a.G),  \
        static_cast<T*>(a.out));                                                              \
    return hipGetLastError();                                                                 \
  }
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return hipErrorInvalidValue;
}

}  // namespace tpc
