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
  bool sum_paths;  // path-summed output rows (one block per l3)
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

// The radial MLP's weights rewritten in MFMA operand order (element offsets
// of each section in one buffer; every section starts on a 64-element
// boundary).  NB = H/16 output blocks per hidden layer, S4 = 4*NB reduction
// steps per block, nblk = ceil(pc/16) blocks of the last layer.
//   f0  forward layer 1        [NB][64 lanes][2]
//   fh  forward layers 2..NH   [NH-1][NB][64][S4]
//   fl  forward last layer     [nblk][64][S4]
//   bl  backward last layer    [nblk][64][S4]   (W_L^T as the A operand)
//   bh  backward layers 2..NH  [NH-1][NB][64][S4]
//   b0  backward layer 1       [64][S4]          (rows 8..15 zero)
// and, for the float32 last layer on bf16 matrix cores (three-part split of
// every weight), a bf16 section counted in float slots (two values per slot):
//   fs  forward last layer     [nblk][64][H/32][3 parts][8]
//   bs  backward last layer    [pc/32][64][H/16][3 parts][8]
struct RadialPack {
  int H, NH, pc, nblk;
  int64_t f0, fh, fl, bl, bh, b0, fs, bs, total;
};
inline RadialPack radial_pack_layout(int H, int NH, int pc) {
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };
  RadialPack L{};
  L.H = H;
  L.NH = NH;
  L.pc = pc;
  L.nblk = (pc + 15) / 16;
  const int64_t NB = H / 16, S4 = 4 * NB, hid = (int64_t)(NH - 1) * NB * 64 * S4;
  int64_t off = 0;
  L.f0 = off;
  off += up(NB * 64 * 2);
  L.fh = off;
  off += up(hid);
  L.fl = off;
  off += up((int64_t)L.nblk * 64 * S4);
  L.bl = off;
  off += up((int64_t)L.nblk * 64 * S4);
  L.bh = off;
  off += up(hid);
  L.b0 = off;
  off += up(64 * S4);
  L.fs = off;
  off += up((int64_t)L.nblk * 64 * (H / 32) * 12);
  L.bs = off;
  off += up((int64_t)(pc / 32) * 64 * NB * 12);
  L.total = off;
  return L;
}
// Per-edge buffer of the backward's first stage: dA for every 16-edge strip
// in register order, H values per edge.
inline int64_t radial_dA_elems(int H, int64_t ne) { return (ne + 15) / 16 * 16 * H; }

bool radial_supported(int H, int NH);
hipError_t launch_radial_pack(int dtype, const RadialPack& L, const void* const* w, void* pk,
                              hipStream_t s);
hipError_t launch_radial_fwd(int dtype, const RadialPack& L, int64_t ne, const void* ef,
                             const void* pk, void* R, hipStream_t s);
hipError_t launch_radial_bwd_dA(int dtype, const RadialPack& L, int64_t ne, const void* dR,
                                const void* pk, void* dA3, hipStream_t s);
hipError_t launch_radial_bwd_mlp(int dtype, const RadialPack& L, int64_t ne, const void* ef,
                                 const void* dA3, const void* pk, void* d_ef, hipStream_t s);

// Which (node_lmax, sh_lmax, out_lmax, channels) the fused kernels are built for.
bool tp_supported(int dtype, int L1, int L2, int L3, int C);
hipError_t launch_tp_fwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
hipError_t launch_tp_bwd_edge(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// dh[j] = scale * sum_{e in row j} dh_edge[e] for every atom
hipError_t launch_dh_gather(int dtype, int64_t n, int din_c, const int32_t* row_ptr, double scale,
                            const void* dh_edge, void* dh, hipStream_t s);

hipError_t launch_forces(int dtype, int64_t n, const int32_t* row_ptr, const int32_t* rev,
                         const void* g, void* forces, hipStream_t s);
// Virial: float64 partial sums per block of kVirialBlock rows, then one fold.
constexpr int kVirialBlock = 256;
inline int64_t virial_blocks(int64_t n) { return n > 0 ? (n + kVirialBlock - 1) / kVirialBlock : 0; }
hipError_t launch_virial(int dtype, int64_t n, const GeomArgs& a, const void* g, double* part,
                         void* W, hipStream_t s);
hipError_t launch_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const int32_t* shift, int64_t row_begin,
                            int64_t row_end, int64_t edge_begin, int64_t edge_end,
                            int32_t* status, hipStream_t s);

}  // namespace tpc
