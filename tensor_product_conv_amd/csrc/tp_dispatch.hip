// Host dispatch of the fused tensor-product kernels to the per-configuration
// objects (tp_config.hpp).
#include "tp_config.hpp"
#include "tp_impl.hpp"

namespace tpc {

namespace {
template <typename T>
constexpr int dtype_id() { return sizeof(T) == 8 ? 1 : 0; }
bool channels_ok(int C) { return (C >= 1 && C <= 64) || C == 128; }
}  // namespace

bool tp_supported(int dtype, int L1, int L2, int L3, int C) {
  if (!channels_ok(C)) return false;
#define TPC_X(I, T, A, B, D) \
  if (dtype == dtype_id<T>() && L1 == A && L2 == B && L3 == D) return true;
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return false;
}

int tp_bwd_parts(int C) { return bwd_parts(C); }
int tp_dbl_parts(int dtype, int L1, int C) { return dbl_parts(dtype == 1, L1, C); }

hipError_t launch_tp_fwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
#define TPC_X(I, T, A, B, D) \
  if (dtype == dtype_id<T>() && L1 == A && L2 == B && L3 == D) return tp_fwd_cfg<T, A, B, D>(a, s);
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return hipErrorInvalidValue;
}

hipError_t launch_tp_fused(int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
#define TPC_X(I, T, A, B, D) \
  if (dtype_id<T>() == 0 && L1 == A && L2 == B && L3 == D) return tp_fused_cfg<T, A, B, D>(a, s);
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return hipErrorInvalidValue;
}

hipError_t launch_tp_bwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
#define TPC_X(I, T, A, B, D) \
  if (dtype == dtype_id<T>() && L1 == A && L2 == B && L3 == D) return tp_bwd_cfg<T, A, B, D>(a, s);
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
  return hipErrorInvalidValue;
}

hipError_t launch_tp_dbl(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s) {
#define TPC_X(I, T, A, B, D) \
  if (dtype == dtype_id<T>() && L1 == A && L2 == B && L3 == D) return tp_dbl_cfg<T, A, B, D>(a, s);
  TPC_TP_CONFIGS(TPC_X)
#undef TPC_X
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
