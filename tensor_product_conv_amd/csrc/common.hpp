// Internal helpers shared by the gfx950 kernels and the host library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

namespace tpc {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1.
template <int N, typename F, int... I>
__host__ __device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(static_cast<F&&>(f), std::make_integer_sequence<int, N>{});
}

// Value that is the same in every lane of the wave, kept in a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Block index for row-streaming kernels on the 8 XCDs of the chip.  Blocks
// go to the XCDs round-robin (block b to XCD b % 8), and each XCD has its own
// L2.  This bijection on [0, gridDim.x) gives XCD x one contiguous range of
// logical blocks, so the rows it works on at any moment are neighbours and
// their shared sender data stays in that XCD's L2.
__device__ __forceinline__ int64_t xcd_block() {
  constexpr int64_t kXcds = 8;
  const int64_t nb = gridDim.x, b = blockIdx.x;
  const int64_t q = nb / kXcds, r = nb % kXcds, x = b % kXcds, k = b / kXcds;
  return x * q + (x < r ? x : r) + k;
}

// Launch status from the HIP runtime after a kernel launch.
inline hipError_t launch_status() { return hipGetLastError(); }

// Device-side error flags reported back by the neighbour build and checks.
enum : int {
  kFlagUnwrapped = 1,    // a fractional coordinate outside [0,1)
  kFlagDegree = 2,       // a row longer than the per-row limit
  kFlagNoReverse = 4,    // an edge whose reverse edge is missing
  kFlagCsrOrder = 8,     // row_ptr not monotone / row not sorted
  kFlagCsrRange = 16,    // src outside [0, n_atoms)
  kFlagSpecies = 32,     // species id outside [0, n_species)
  kFlagShiftRange = 64,  // image shift outside [-127, 127]
};

}  // namespace tpc
