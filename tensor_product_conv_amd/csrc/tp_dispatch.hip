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

int tp_bwd_parts(int dtype, int L1, int C) { return bwd_parts(dtype == 1, L1, C); }

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
hipError_t dh_gather_impl(const DhGather& g, double scale, hipStream_t s) {
  const int64_t waves = g.n * ((g.din_c + 64 * V - 1) / (64 * V));
  const unsigned blocks = (unsigned)((waves + kGatherWaves - 1) / kGatherWaves);
  k_dh_gather_chunk<T, V><<<blocks, 64 * kGatherWaves, 0, s>>>(
      g.n, g.din_c, g.row_ptr, g.src, g.rev, g.row_begin, g.row_end, g.edge_begin, g.n_chunk_edges, g.first,
      g.last, (T)scale, static_cast<const T*>(g.t_chunk), static_cast<T*>(g.dh));
  return hipGetLastError();
}

hipError_t launch_dh_gather(int dtype, const DhGather& g, double scale, hipStream_t s) {
  if (g.n * g.din_c <= 0) return hipSuccess;
  // 16-byte vectors when every row of din_c values starts 16-byte aligned
  const size_t tsz = dtype == 1 ? 8 : 4;
  const bool vec = (g.din_c * tsz) % 16 == 0 && reinterpret_cast<uintptr_t>(g.t_chunk) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(g.dh) % 16 == 0;
  if (dtype == 1) return vec ? dh_gather_impl<double, 2>(g, scale, s) : dh_gather_impl<double, 1>(g, scale, s);
  return vec ? dh_gather_impl<float, 4>(g, scale, s) : dh_gather_impl<float, 1>(g, scale, s);
}

}  // namespace tpc
