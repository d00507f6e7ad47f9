// Neighbour-build launchers and the bin geometry they share with the host.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpc {

constexpr int kMaxDegree = 1024;  // longest row the in-LDS row sort handles

// Bin grid over fractional coordinates.  Bins are at least r_cut*(1+1e-6) wide
// along every lattice direction, so an edge joins bins at most K apart.
struct NbrGrid {
  double a[3][3];    // cell rows a1, a2, a3
  double inv[3][3];  // inverse of the cell matrix: f = x . inv
  int nb[3];         // bins per direction
  int K[3];          // stencil half-width per direction
  double rc2;        // r_cut * r_cut
};

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_scan_exclusive(int32_t* data, int64_t n, int32_t* partials, hipStream_t s);
int64_t scan_partials_len(int64_t n);

hipError_t launch_nbr_bin(int64_t n, const double* pos, const NbrGrid& g, const int32_t* species,
                          int n_species, int32_t* bin_of, int32_t* bin_count, int32_t* status,
                          hipStream_t s);
hipError_t launch_nbr_scatter(int64_t n, const int32_t* bin_of, const int32_t* bin_start,
                              int32_t* cursor, int32_t* bin_atoms, hipStream_t s);
hipError_t launch_nbr_count(int64_t n, const double* pos, const NbrGrid& g, const int32_t* bin_of,
                            const int32_t* bin_start, const int32_t* bin_atoms, int32_t* deg,
                            int32_t* status, hipStream_t s);
hipError_t launch_nbr_fill(int64_t n, const double* pos, const NbrGrid& g, const int32_t* bin_of,
                           const int32_t* bin_start, const int32_t* bin_atoms,
                           const int32_t* row_ptr, int32_t* src, int32_t* shift, hipStream_t s);
hipError_t launch_wrap_check(int64_t n, const double* pos, const NbrGrid& g, int32_t* status,
                             hipStream_t s);
hipError_t launch_nbr_reverse(int64_t n, const int32_t* row_ptr, const int32_t* src,
                              const int32_t* shift, int32_t* rev, int32_t* status, hipStream_t s);

}  // namespace tpc
