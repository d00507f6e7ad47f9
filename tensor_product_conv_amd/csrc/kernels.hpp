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
  int64_t row_begin, row_end, edge_begin;
  int64_t n_chunk_edges;  // edges of the chunk (stride of the partial dY slices)
  int C;           // channels
  bool sum_paths;  // path-summed output rows (one block per l3)
  double scale;    // neighbour normalisation s
  const void* h;   // [N][d_in][C]
  const void* Y;   // [E][d_sh]
  const void* R;   // [E][P*C], or [rows][P*C] read through Rrow
  const int32_t* Rrow;  // nullable: chunk-relative R row of each edge (shared
                        // rows of edge pairs); null: row (edge - edge_begin)
  const void* G;   // [N][d_out][C]  (backward)
  void* out;       // forward: out [N][d_out][C]
  void* dR;        // backward edge kernel: [E][P*C]
  void* dY;        // backward: partial dY [parts][E][d_sh], parts = tp_bwd_parts
                   // (double backward: partial y_hat, parts = tp_bwd_parts)
  void* dh_edge;   // backward: [E_chunk][d_in][C] per-edge dh contributions
                   // of the chunk's edges, at each edge's own slot
  // double backward: cotangents of the VJP outputs and its results
  const int32_t* rev;  // reverse-edge index [n_edges]
  const void* uh;  // [N][d_in][C]
  const void* uY;  // [n_edges][d_sh], absolute edge index
  const void* uR;  // [n_edges][P*C], absolute edge index
  void* g_hat;     // [N][d_out][C], rows [row_begin, row_end)
  void* x_hat;     // [N][d_in][C], rows [row_begin, row_end)
  void* w_hat;     // [E_chunk][P*C]
  // forward with the fused radial last layer
  const void* act;  // [E_chunk][H / 32][4][3][8] bf16: split last hidden activations
  const void* wfs;  // the packed split last-layer weights (radial pack section fs)
  int H;            // hidden width of the radial network
  void* R_out;      // nullable: R [E_chunk][P*C] stored for a backward that reads it
};

hipError_t launch_geom_fwd(int dtype, int L2, const GeomArgs& a, void* Y, void* ef, void* rv,
                           hipStream_t s);
// dY holds n_parts partial slices [n_parts][ne][d_sh], summed in slice order.
// The radial part comes from d_ef [ne][8] (dL/d(basis)), or, when d_ef is
// null, from d_r [ne] (dL/dr directly, the table path).
hipError_t launch_geom_bwd(int dtype, int L2, int64_t ne, int64_t edge_begin, double r_cut,
                           const void* rv, const void* dY, int n_parts, const void* d_ef, const void* d_r,
                           void* g, hipStream_t s);

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
// x6 off keeps every float32 product on float32 matrix cores.
struct RadialPack {
  int H, NH, pc, nblk;
  bool x6;
  int64_t f0, fh, fl, bl, bh, b0, fs, bs, total;
};
inline RadialPack radial_pack_layout(int H, int NH, int pc, bool x6 = true) {
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };
  RadialPack L{};
  L.x6 = x6;
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
// ne_dev (nullable): the number of rows, read on the device when it is only
// known there (at most ne, which sizes the grid).
hipError_t launch_radial_fwd(int dtype, const RadialPack& L, int64_t ne, const int32_t* ne_dev,
                             const void* ef, const void* pk, void* R, hipStream_t s);
// Shared R rows of the chunk's edge pairs: rrow [ne + 1] (chunk-relative row
// of each edge's R, rrow[ne] = number of rows), partials [pair_partials_len]
// scratch, and each row's basis values copied from ef [ne][8] to
// ef_rows [ne][8] (nullable: the map only).
hipError_t launch_pair_rows(int dtype, const int32_t* rev, int64_t edge_begin, int64_t ne, int32_t* rrow,
                            int32_t* partials, const void* ef, void* ef_rows, hipStream_t s);
int64_t pair_partials_len(int64_t ne);
// Last hidden activations, split for the fused forward (float32, H = 32 or 64):
// act [ne][H / 32][4][3][8] bf16.
hipError_t launch_radial_act(const RadialPack& L, int64_t ne, const void* ef, const void* pk, void* act,
                             hipStream_t s);
hipError_t launch_radial_bwd_dA(int dtype, const RadialPack& L, int64_t ne, const void* dR,
                                const void* pk, void* dA3, hipStream_t s);
hipError_t launch_radial_bwd_mlp(int dtype, const RadialPack& L, int64_t ne, const void* ef,
                                 const void* dA3, const void* pk, void* d_ef, hipStream_t s);

// Which (node_lmax, sh_lmax, out_lmax, channels) the fused kernels are built for.
bool tp_supported(int dtype, int L1, int L2, int L3, int C);
hipError_t launch_tp_fwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// Forward with the radial last layer fused in (float32, C a multiple of 16,
// H = 32 or 64): reads a.act and a.wfs instead of R; writes R too when a.R_out
// is non-null.
hipError_t launch_tp_fused(int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// dR, the partial dY slices and the per-edge dh contributions of rows
// [row_begin, row_end)
hipError_t launch_tp_bwd(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// number of partial dY slices launch_tp_bwd writes, and of partial y_hat
// slices launch_tp_dbl writes (one per wave of a row)
int tp_bwd_parts(int dtype, int L1, int C);
// One receiver chunk's step of dh: for every atom j, the running sum dh[j]
// continues over the entries e of row j whose sender lies in
// [row_begin, row_end), adding t_chunk[rev[e] - edge_begin] (launch_tp_bwd's
// per-edge contributions of the chunk).  first starts the sums from zero,
// last stores scale * sum.
struct DhGather {
  int64_t n = 0;
  int din_c = 0;
  const int32_t* row_ptr = nullptr;
  const int32_t* src = nullptr;
  const int32_t* rev = nullptr;
  int64_t row_begin = 0, row_end = 0, edge_begin = 0, n_chunk_edges = 0;
  bool first = true, last = true;
  const void* t_chunk = nullptr;
  void* dh = nullptr;
};
hipError_t launch_dh_gather(int dtype, const DhGather& g, double scale, hipStream_t s);
// VJP-of-VJP of rows [row_begin, row_end): g_hat, x_hat of the rows, w_hat
// and tp_bwd_parts partial slices of y_hat (in TPArgs::dY) of the chunk's
// edges; separate (not path-summed) outputs only
hipError_t launch_tp_dbl(int dtype, int L1, int L2, int L3, const TPArgs& a, hipStream_t s);
// out[e][k] = sum over the n_parts slices of in[part][e][k], in slice order
hipError_t launch_part_sum(int dtype, int n_parts, int64_t ne, int width, const void* in, void* out,
                           hipStream_t s);

// Piecewise Chebyshev radial tables (radial_table.hip): elements of a table
// of `pieces` pieces and degree d for pc columns; the fit writes float64
// point values, the table and the certificate ratios [pieces][2].
constexpr int kTableMaxDegree = 16;
constexpr int kTableCheckPerPiece = 8;
int64_t table_elems(int pieces, int degree, int pc);
hipError_t launch_table_fit(int dtype, int NH, int H, int pc, int pieces, int degree, double r_cut,
                            const void* const* w, double* f64_nodes, void* table, double* cert,
                            hipStream_t s);
// Work buffer of the runtime table kernels: int32 [pieces + 1 + ne] (piece
// counts, then the chunk's edges sorted by piece).
int64_t table_sort_ints(int pieces, int64_t ne);
hipError_t launch_table_fwd(int dtype, int64_t ne, int pc, int pieces, int degree, double r_cut,
                            const void* rv, const void* table, void* work, void* R, hipStream_t s);
// d_r[e] = dL/dr_e = sum_c dR[e][c] dR_c/dr (the radial part of the edge gradient)
hipError_t launch_table_bwd(int dtype, int64_t ne, int pc, int pieces, int degree, double r_cut,
                            const void* rv, const void* table, const void* dR, void* work, void* d_r,
                            hipStream_t s);

hipError_t launch_forces(int dtype, int64_t n, const int32_t* row_ptr, const int32_t* rev,
                         const void* g, void* forces, hipStream_t s);
// Virial: float64 partial sums per block of kVirialBlock rows, then one fold.
constexpr int kVirialBlock = 256;
inline int64_t virial_blocks(int64_t n) { return n > 0 ? (n + kVirialBlock - 1) / kVirialBlock : 0; }
hipError_t launch_virial(int dtype, int64_t n, const GeomArgs& a, const void* g, double* part,
                         void* W, hipStream_t s);
// rows [row_begin, row_end): order, ranges, and (rev non-null) symmetry
// Fixed device scratch of the entry point that allocates nothing: its size,
// and the device address of the current GPU's copy (looked up on first use
// per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t scratch_for_current_device(void** ptr, size_t* bytes);

hipError_t launch_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const int32_t* shift, const int32_t* rev,
                            int64_t row_begin, int64_t row_end, int64_t edge_begin,
                            int64_t edge_end, int32_t* status, hipStream_t s);

}  // namespace tpc
