// Instantiations of the receiver-side backward kernel (dR, partial dY and
// the per-edge dh contributions).
#include "tp_impl.hpp"

namespace tpc {

hipError_t launch_tp_bwd_edge(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
  const int64_t rows = a.row_end - a.row_begin;
  if (rows <= 0) return hipSuccess;
  const int nw = tp_nw(a.C);
#define TPC_LAUNCH_BE(T, A, B, D, F)                                                             \
  if (a.sum_paths)                                                                               \
    TPC_LAUNCH_BE2(T, A, B, D, true, F)                                                          \
  else                                                                                           \
    TPC_LAUNCH_BE2(T, A, B, D, false, F)
#define TPC_LAUNCH_BE2(T, A, B, D, S, F)                                                         \
  k_tp_bwd_edge<T, A, B, D, S, F><<<tp_blocks(rows, a.C), kTPWave * kTPWavesPerBlock, 0, s>>>(    \
      a.row_ptr, a.src, a.rev, a.row_begin, a.row_end, a.edge_begin, a.n_chunk_edges, a.C,      \
      (T)a.scale, static_cast<const T*>(a.h), static_cast<const T*>(a.Y),                     \
      static_cast<const T*>(a.R), static_cast<const T*>(a.G), static_cast<T*>(a.dR),           \
      static_cast<T*>(a.dY), static_cast<T*>(a.dh_edge));
#define TPC_X(T, A, B, D)                                                                  \
  if (dtype == tp_detail::dtype_id<T>() && L1 == A && L2 == B && L3 == D) {                \
    switch (nw) { case 0: TPC_LAUNCH_BE(T, A, B, D, 0) break; case 1: TPC_LAUNCH_BE(T, A, B, D, 1) break; \
                  case 2: TPC_LAUNCH_BE(T, A, B, D, 2) break; default: return hipErrorInvalidValue; } \
    return hipGetLastError();                                                              \
  }
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
#undef TPC_LAUNCH_BE
#undef TPC_LAUNCH_BE2
  return hipErrorInvalidValue;
}

template <typename T, int V>
hipError_t dh_gather_impl(int64_t n, int din_c, const int32_t* row_ptr, double scale,
                          const void* dh_edge, void* dh, hipStream_t s) {
  const int64_t total = n * (din_c / V);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  k_dh_gather<T, V><<<blocks, 256, 0, s>>>(n, din_c, row_ptr, (T)scale, static_cast<const T*>(dh_edge),
                                           static_cast<T*>(dh));
  return hipGetLastError();
}

hipError_t launch_dh_gather(int dtype, int64_t n, int din_c, const int32_t* row_ptr, double scale,
                            const void* dh_edge, void* dh, hipStream_t s) {
  if (n * din_c <= 0) return hipSuccess;
  // 16-byte vectors when every row of din_c values starts 16-byte aligned
  const size_t tsz = dtype == 1 ? 8 : 4;
  const bool vec = (din_c * tsz) % 16 == 0 && reinterpret_cast<uintptr_t>(dh_edge) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dh) % 16 == 0;
  if (dtype == 1)
    return vec ? dh_gather_impl<double, 2>(n, din_c, row_ptr, scale, dh_edge, dh, s)
               : dh_gather_impl<double, 1>(n, din_c, row_ptr, scale, dh_edge, dh, s);
  return vec ? dh_gather_impl<float, 4>(n, din_c, row_ptr, scale, dh_edge, dh, s)
             : dh_gather_impl<float, 1>(n, din_c, row_ptr, scale, dh_edge, dh, s);
}

}  // namespace tpc
