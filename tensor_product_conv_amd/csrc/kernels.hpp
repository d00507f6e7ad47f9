// Launch interfaces of the convolution kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpc {

struct GeomArgs {
  const double* pos;
  double cell[3][3];
  const int32_t* row_ptr;
  const int32_t* src;
  const int32_t* shift;
  int64_t row_begin, row_end, edge_begin, edge_end;
  double r_cut;
};

template <typename T>
struct RadialWeights {
  const T* w[8];
};

// Arguments of the fused tensor-product kernels.  Edge-indexed arrays (Y, R,
// dR, dY) are indexed by (edge - edge_begin).
struct TPArgs {
  const int32_t* row_ptr;
  const int32_t* src;
  const int32_t* rev;     // reverse-edge index (backward)
  int64_t row_begin, row_end, edge_begin;
  int64_t n_chunk_edges;  // edges of the chunk (stride of the partial dY slices)
  int C;           // channels
  double scale;    // neighbour normalisation s
  const void* h;   // [N][d_in][C]
  const void* Y;   // [E][d_sh]
  const void* R;   // [E][P*C]
  const void* G;   // [N][d_out][C]  (backward)
  void* out;       // forward: out [N][d_out][C]
  void* dR;        // backward edge kernel: [E][P*C]
  void* dY;        // backward edge kernel: partial dY [C/64 slices][E][d_sh]
  void* dh_edge;   // backward edge kernel: [n_edges][d_in][C], absolute edge index
};

hipError_t launch_geom_fwd(int dtype, int L2, const GeomArgs& a, void* Y, void* ef, void* rv,
                           hipStream_t s);
// dY holds n_parts partial slices [n_parts][ne][d_sh], summed in slice order.
hipError_t launch_geom_bwd(int dtype, int L2, int64_t ne, int64_t edge_begin, double r_cut,
                           const void* rv, const void* dY, int n_parts, const void* d_ef, void* g,
                           hipStream_t s);

bool radial_supported(int H, int NH);
hipError_t launch_radial_fwd(int dtype, int H, int NH, int64_t ne, int pc, const void* ef,
                             const void* const* w, void* R, hipStream_t s);
hipError_t launch_radial_bwd(int dtype, int H, int NH, int64_t ne, int pc, const void* ef,
                             const void* dR, const void* const* w, void* d_ef, hipStream_t s);

// Which (node_lmax, sh_lmax, out_lmax, channels) the fused kernels are built for.
bool tp_supported(int dtype, int L1, int L2, int L3, int C);
hipError_t launch_tp_fwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
hipError_t launch_tp_bwd_edge(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// dh[j] = scale * sum_{e in row j} dh_edge[e] for every atom
hipError_t launch_dh_gather(int dtype, int64_t n, int din_c, const int32_t* row_ptr, double scale,
                            const void* dh_edge, void* dh, hipStream_t s);

hipError_t launch_forces(int dtype, int64_t n, const int32_t* row_ptr, const int32_t* rev,
                         const void* g, void* forces, hipStream_t s);
hipError_t launch_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const int32_t* shift, int64_t row_begin,
                            int64_t row_end, int64_t edge_begin, int64_t edge_end,
                            int32_t* status, hipStream_t s);

}  // namespace tpc
