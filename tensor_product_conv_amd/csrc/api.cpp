// Host side of the C ABI declared in include/tpconv.h: spec validation, the
// context, workspace planning, argument checks and kernel sequencing.
//
// Every check runs before any device work, so a failing call enqueues nothing,
// and all the failed checks are reported together, as the refusal of an
// unsupported plan does on the FastMACE page "Rewrites and precision options"
// (section "Toggle values").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tpconv.h"
#include "common.hpp"
#include "kernels.hpp"
#include "nbr.hpp"
#include "tables.hpp"

struct tpc_ctx {
  tpc_spec spec;
  tpc::Table tab;
  int hidden;    // hidden width H
  int n_hidden;  // number of hidden layers
  size_t tsize;  // bytes per feature value
  bool table;    // radial weights from a piecewise Chebyshev table
  bool fused;    // the forward forms R inside the tensor-product kernel
  bool pair;     // an edge and its reverse share one row of R
};

namespace {

thread_local std::string g_last_error;

struct Errors {
  std::vector<std::string> msgs;
  tpc_status status = TPC_OK;
  void add(tpc_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    msgs.emplace_back(buf);
    // INVALID outranks UNSUPPORTED, which outranks the rest
    if (status == TPC_OK || s == TPC_ERR_INVALID ||
        (s == TPC_ERR_UNSUPPORTED && status != TPC_ERR_INVALID))
      status = s;
  }
  tpc_status finish() {
    if (status == TPC_OK) {
      g_last_error.clear();
      return TPC_OK;
    }
    std::string all;
    for (auto& m : msgs) {
      if (!all.empty()) all += "; ";
      all += m;
    }
    g_last_error = all;
    return status;
  }
};

tpc_status device_error(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return TPC_ERR_DEVICE;
}

#define TPC_HIP(call, where)                                  \
  do {                                                        \
    hipError_t _e = (call);                                   \
    if (_e != hipSuccess) return device_error(_e, where);     \
  } while (0)

// Optional per-kernel event timing (tpc_timing_enable / tpc_timing_collect).
struct KernelMark {
  const char* name;
  hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<KernelMark> g_marks;
thread_local std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch `call` (a hipError_t expression enqueuing on stream s); time it when
// timing is on.
#define TPC_LAUNCH(name, s, call, where)                                   \
  do {                                                                     \
    hipEvent_t _a = nullptr;                                               \
    if (g_timing && (_a = pooled_event())) hipEventRecord(_a, s);          \
    hipError_t _e = (call);                                                \
    if (_e != hipSuccess) return device_error(_e, where);                  \
    if (_a) {                                                              \
      hipEvent_t _b = pooled_event();                                      \
      if (_b) {                                                            \
        hipEventRecord(_b, s);                                             \
        g_marks.push_back(KernelMark{name, _a, _b});                       \
      } else {                                                             \
        g_event_pool.push_back(_a);                                        \
      }                                                                    \
    }                                                                      \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bin grid for the neighbour build from a host cell.
bool make_grid(const double* cell, double r_cut, tpc::NbrGrid* g, std::string* why) {
  double A[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) A[r][c] = cell[3 * r + c];
  const double det = A[0][0] * (A[1][1] * A[2][2] - A[1][2] * A[2][1]) -
                     A[0][1] * (A[1][0] * A[2][2] - A[1][2] * A[2][0]) +
                     A[0][2] * (A[1][0] * A[2][1] - A[1][1] * A[2][0]);
  if (!std::isfinite(det) || std::fabs(det) < 1e-12) {
    *why = "cell is singular or not finite";
    return false;
  }
  // inverse (adjugate / det); f = x . inv
  double inv[3][3];
  inv[0][0] = (A[1][1] * A[2][2] - A[1][2] * A[2][1]) / det;
  inv[0][1] = (A[0][2] * A[2][1] - A[0][1] * A[2][2]) / det;
  inv[0][2] = (A[0][1] * A[1][2] - A[0][2] * A[1][1]) / det;
  inv[1][0] = (A[1][2] * A[2][0] - A[1][0] * A[2][2]) / det;
  inv[1][1] = (A[0][0] * A[2][2] - A[0][2] * A[2][0]) / det;
  inv[1][2] = (A[0][2] * A[1][0] - A[0][0] * A[1][2]) / det;
  inv[2][0] = (A[1][0] * A[2][1] - A[1][1] * A[2][0]) / det;
  inv[2][1] = (A[0][1] * A[2][0] - A[0][0] * A[2][1]) / det;
  inv[2][2] = (A[0][0] * A[1][1] - A[0][1] * A[1][0]) / det;
  const double vol = std::fabs(det);
  int64_t total = 1;
  for (int k = 0; k < 3; ++k) {
    const double* u = A[(k + 1) % 3];
    const double* v = A[(k + 2) % 3];
    const double cx = u[1] * v[2] - u[2] * v[1], cy = u[2] * v[0] - u[0] * v[2],
                 cz = u[0] * v[1] - u[1] * v[0];
    const double h = vol / std::sqrt(cx * cx + cy * cy + cz * cz);
    const double w = r_cut * (1.0 + 1e-6);
    int nb = (int)std::floor(h / w);
    if (nb < 1) nb = 1;
    if (nb > 1024) nb = 1024;
    const int K = (int)std::ceil(w * nb / h);
    if (K > 16) {
      *why = "cell is too thin for the cutoff (more than 16 images per direction)";
      return false;
    }
    g->nb[k] = nb;
    g->K[k] = K;
    total *= nb;
  }
  if (total > (int64_t)1 << 24) {
    *why = "too many bins";
    return false;
  }
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      g->a[r][c] = A[r][c];
      g->inv[r][c] = inv[r][c];
    }
  g->rc2 = r_cut * r_cut;
  return true;
}

struct NbrWs {
  size_t bin_of, bin_start, cursor, bin_atoms, partials, status, total;
};

NbrWs nbr_layout(int64_t n, int64_t nbin) {
  NbrWs w{};
  size_t off = 0;
  w.bin_of = off;
  off += align_up(sizeof(int32_t) * (size_t)n);
  w.bin_start = off;
  off += align_up(sizeof(int32_t) * (size_t)(nbin + 1));
  w.cursor = off;
  off += align_up(sizeof(int32_t) * (size_t)nbin);
  w.bin_atoms = off;
  off += align_up(sizeof(int32_t) * (size_t)n);
  w.partials = off;
  const int64_t m = n > nbin ? n : nbin;
  off += align_up(sizeof(int64_t) * (size_t)tpc::scan_partials_len(m + 1));
  w.status = off;
  off += align_up(sizeof(int32_t) * 8);
  w.total = off;
  return w;
}

struct BwdWs {
  size_t dR, dY, d_ef, status, pack, dA, tsort, total, total_without_dR;
};

tpc::RadialPack pack_layout(const tpc_ctx* c) {
  return tpc::radial_pack_layout(c->hidden, c->n_hidden, c->tab.np * c->spec.channels,
                                 c->spec.fp32_mfma_only == 0);
}

struct FwdWs {
  size_t status, pack, tsort, pair_part, ef_rows, total;
};

// ne: edges of the chunk (a table context sorts them by piece)
FwdWs fwd_layout(const tpc_ctx* c, int64_t ne) {
  FwdWs w{};
  size_t off = 0;
  w.status = off;
  off += align_up(sizeof(int32_t) * 8);
  w.pack = off;
  if (!c->table) off += align_up(c->tsize * (size_t)pack_layout(c).total);
  w.tsort = off;
  if (c->table) off += align_up(sizeof(int32_t) * (size_t)tpc::table_sort_ints(c->spec.radial_table_pieces, ne));
  // shared R rows: the scan's partial sums and the rows' basis values
  w.pair_part = off;
  if (c->pair) off += align_up(sizeof(int64_t) * (size_t)tpc::pair_partials_len(ne));
  w.ef_rows = off;
  if (c->pair) off += align_up(c->tsize * 8 * (size_t)ne);
  w.total = off;
  return w;
}

// Largest chunk whose shared-row map one scan can number (16 M edges).
constexpr int64_t kPairMaxChunk = (int64_t)4096 * 4096;

struct TableWs {
  size_t nodes, cert, total;
};

TableWs table_layout(const tpc_ctx* c) {
  TableWs w{};
  const int pieces = c->spec.radial_table_pieces, n = c->spec.radial_table_degree + 1;
  size_t off = 0;
  w.nodes = off;
  off += align_up(sizeof(double) * (size_t)pieces * n * c->tab.np * c->spec.channels);
  w.cert = off;
  off += align_up(sizeof(double) * 2 * (size_t)pieces);
  w.total = off;
  return w;
}

size_t table_bytes(const tpc_ctx* c) {
  if (!c->table) return 0;
  return c->tsize * (size_t)tpc::table_elems(c->spec.radial_table_pieces, c->spec.radial_table_degree,
                                             c->tab.np * c->spec.channels);
}

struct VirialWs {
  size_t status, part, total;
};

VirialWs virial_layout(int64_t n) {
  VirialWs w{};
  size_t off = 0;
  w.status = off;
  off += align_up(sizeof(int32_t) * 8);
  w.part = off;
  off += align_up(sizeof(double) * 9 * (size_t)tpc::virial_blocks(n));
  w.total = off;
  return w;
}

int dy_parts(const tpc_ctx* c) { return tpc::tp_bwd_parts(c->spec.dtype, c->spec.node_lmax, c->spec.channels); }
int yh_parts(const tpc_ctx* c) { return dy_parts(c); }

BwdWs bwd_layout(const tpc_ctx* c, int64_t ne) {
  BwdWs w{};
  const size_t T = c->tsize;
  size_t off = 0;
  w.dY = off;  // one partial dY slice per wave of a row
  off += align_up(T * (size_t)ne * c->tab.dsh * dy_parts(c));
  w.d_ef = off;
  off += align_up(T * (size_t)ne * 8);
  w.status = off;
  off += align_up(sizeof(int32_t) * 8);
  w.pack = off;
  if (!c->table) off += align_up(T * (size_t)pack_layout(c).total);
  w.dA = off;
  if (!c->table) off += align_up(T * (size_t)tpc::radial_dA_elems(c->hidden, ne));
  w.tsort = off;
  if (c->table) off += align_up(sizeof(int32_t) * (size_t)tpc::table_sort_ints(c->spec.radial_table_pieces, ne));
  w.total_without_dR = off;
  w.dR = off;
  off += align_up(T * (size_t)ne * c->tab.np * c->spec.channels);
  w.total = off;
  return w;
}

struct DblWs {
  size_t status, yh, total;
};

DblWs dbl_layout(const tpc_ctx* c, int64_t ne) {
  DblWs w{};
  size_t off = 0;
  w.status = off;
  off += align_up(sizeof(int32_t) * 8);
  w.yh = off;  // one partial y_hat slice per wave of a row
  off += align_up(c->tsize * (size_t)ne * c->tab.dsh * yh_parts(c));
  w.total = off;
  return w;
}

void flag_messages(int flags, Errors& E) {
  if (flags & tpc::kFlagUnwrapped)
    E.add(TPC_ERR_PRECONDITION, "positions are not wrapped: a fractional coordinate lies outside [0,1)");
  if (flags & tpc::kFlagSpecies) E.add(TPC_ERR_INVALID, "a species id lies outside [0, n_species)");
  if (flags & tpc::kFlagDegree)
    E.add(TPC_ERR_UNSUPPORTED, "a row has more than %d neighbours", tpc::kMaxDegree);
  if (flags & tpc::kFlagNoReverse) E.add(TPC_ERR_PRECONDITION, "an edge has no reverse edge");
  if (flags & tpc::kFlagCsrOrder)
    E.add(TPC_ERR_PRECONDITION, "CSR is not receiver-sorted (row pointers or row order)");
  if (flags & tpc::kFlagCsrRange) E.add(TPC_ERR_PRECONDITION, "CSR holds an invalid sender");
  if (flags & tpc::kFlagShiftRange) E.add(TPC_ERR_PRECONDITION, "an image shift lies outside [-127,127]");
}

}  // namespace

extern "C" {

const char* tpc_status_string(tpc_status s) {
  switch (s) {
    case TPC_OK: return "ok";
    case TPC_ERR_INVALID: return "invalid argument";
    case TPC_ERR_UNSUPPORTED: return "unsupported";
    case TPC_ERR_CAPACITY: return "edge capacity too small";
    case TPC_ERR_PRECONDITION: return "precondition violated";
    case TPC_ERR_WORKSPACE: return "workspace too small";
    case TPC_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* tpc_last_error(void) { return g_last_error.c_str(); }

tpc_status tpc_timing_enable(int on) {
  g_timing = on != 0;
  return TPC_OK;
}

tpc_status tpc_timing_collect(tpc_kernel_time* out, int max, int* n) {
  Errors E;
  if (!n || (max > 0 && !out)) {
    E.add(TPC_ERR_INVALID, "out and n must be non-null");
    return E.finish();
  }
  std::vector<tpc_kernel_time> agg;
  hipError_t err = hipSuccess;
  for (auto& m : g_marks) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(m.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m.start, m.stop);
    if (e != hipSuccess && err == hipSuccess) err = e;
    size_t k = 0;
    while (k < agg.size() && std::strcmp(agg[k].name, m.name) != 0) ++k;
    if (k == agg.size()) {
      tpc_kernel_time t{};
      std::snprintf(t.name, sizeof(t.name), "%s", m.name);
      agg.push_back(t);
    }
    agg[k].total_ms += ms;
    agg[k].launches += 1;
    g_event_pool.push_back(m.start);
    g_event_pool.push_back(m.stop);
  }
  g_marks.clear();
  if (err != hipSuccess) return device_error(err, "timing");
  const int cnt = (int)agg.size() < max ? (int)agg.size() : max;
  for (int k = 0; k < cnt; ++k) out[k] = agg[k];
  *n = cnt;
  g_last_error.clear();
  return TPC_OK;
}

namespace {

// Whether the forward fuses the radial last layer into the tensor product:
// asked for (spec.fuse_radial), float32 with the bf16-split products, hidden width 32 or 64, 16-channel
// slices, no table, and the slice's weights (P x 64 lanes x H/32 x 24 bf16)
// plus the waves' staging rows within the 160 KiB of LDS.
bool fused_radial_ok(const tpc_spec& s, const tpc::Table& tab, int H) {
  if (!s.fuse_radial || s.dtype != TPC_F32 || s.fp32_mfma_only || s.radial_table_pieces > 0) return false;
  if ((H != 32 && H != 64) || s.channels % 16 != 0 || tab.np <= 0) return false;
  if ((tab.np * s.channels) % 32 != 0) return false;
  const size_t lds = (size_t)tab.np * 64 * (H / 32) * 24 * 2 + 8 * 256 * 4;
  return lds <= 160 * 1024;
}

}  // namespace

tpc_status tpc_ctx_create(const tpc_spec* spec, tpc_ctx** out) {
  Errors E;
  if (!spec || !out) {
    E.add(TPC_ERR_INVALID, "spec and ctx must be non-null");
    return E.finish();
  }
  const tpc_spec& s = *spec;
  if (s.dtype != TPC_F32 && s.dtype != TPC_F64) E.add(TPC_ERR_INVALID, "dtype must be TPC_F32 or TPC_F64");
  if (s.channels < 1) E.add(TPC_ERR_INVALID, "channels must be >= 1");
  bool lok = true;
  if (s.node_lmax < 0 || s.node_lmax > 3) { E.add(TPC_ERR_UNSUPPORTED, "node_lmax must be 0..3"); lok = false; }
  if (s.sh_lmax < 0 || s.sh_lmax > 3) { E.add(TPC_ERR_UNSUPPORTED, "sh_lmax must be 0..3"); lok = false; }
  if (s.out_lmax < 0 || s.out_lmax > 3) { E.add(TPC_ERR_UNSUPPORTED, "out_lmax must be 0..3"); lok = false; }
  if (s.n_bessel != 8) E.add(TPC_ERR_UNSUPPORTED, "n_bessel must be 8");
  if (s.poly_p != 5) E.add(TPC_ERR_UNSUPPORTED, "poly_p must be 5");
  if (s.n_species < 1) E.add(TPC_ERR_INVALID, "n_species must be >= 1");
  if (!(s.r_cut > 0.0) || !std::isfinite(s.r_cut)) E.add(TPC_ERR_INVALID, "r_cut must be finite and > 0");
  tpc::Table tab{};
  if (lok) {
    tab = tpc::make_table(s.node_lmax, s.sh_lmax, s.out_lmax, s.sum_paths != 0);
    if (tab.np == 0) E.add(TPC_ERR_INVALID, "no admissible path for these l ranges");
  }
  int H = 0, NH = 0;
  if (s.n_layers < 2 || s.n_layers > TPC_MAX_LAYERS) {
    E.add(TPC_ERR_INVALID, "n_layers must be 2..%d", TPC_MAX_LAYERS);
  } else {
    if (s.layer_dims[0] != 8) E.add(TPC_ERR_INVALID, "layer_dims[0] must equal n_bessel (8)");
    H = s.layer_dims[1];
    NH = s.n_layers - 1;
    for (int k = 1; k < s.n_layers; ++k)
      if (s.layer_dims[k] != H) E.add(TPC_ERR_UNSUPPORTED, "hidden widths must all be equal");
    if (!tpc::radial_supported(H, NH))
      E.add(TPC_ERR_UNSUPPORTED, "radial MLP needs 1..3 hidden layers of width 16, 32 or 64 (got %d x %d)", NH, H);
    if (lok && tab.np > 0 && s.layer_dims[s.n_layers] != tab.np * s.channels)
      E.add(TPC_ERR_INVALID, "layer_dims[n_layers] must equal paths*channels = %d", tab.np * s.channels);
  }
  if (s.radial_table_pieces < 0 || s.radial_table_pieces > 4096)
    E.add(TPC_ERR_INVALID, "radial_table_pieces must be 0 (radial network) or 1..4096");
  if (s.radial_table_pieces > 0 && (s.radial_table_degree < 1 || s.radial_table_degree > tpc::kTableMaxDegree))
    E.add(TPC_ERR_INVALID, "radial_table_degree must be 1..%d", tpc::kTableMaxDegree);
  if (lok && s.channels >= 1 && (s.dtype == TPC_F32 || s.dtype == TPC_F64) &&
      !tpc::tp_supported(s.dtype, s.node_lmax, s.sh_lmax, s.out_lmax, s.channels))
    E.add(TPC_ERR_UNSUPPORTED,
          "no fused kernel for dtype=%d node_lmax=%d sh_lmax=%d out_lmax=%d channels=%d "
          "(built: (node_lmax, sh_lmax, out_lmax) in (1,2,1),(1,3,3),(2,3,3),(3,3,3) in float32, "
          "(1,2,1),(1,3,3) in float64; channels 1..64 or 128)",
          s.dtype, s.node_lmax, s.sh_lmax, s.out_lmax, s.channels);
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;
  tpc_ctx* c = new tpc_ctx;
  c->spec = s;
  c->tab = tab;
  c->hidden = H;
  c->n_hidden = NH;
  c->tsize = s.dtype == TPC_F64 ? 8 : 4;
  c->table = s.radial_table_pieces > 0;
  c->fused = fused_radial_ok(s, tab, H);
  // shared rows are built for the unmasked tensor-product kernels (64 or 128
  // channels)
  c->pair = s.pair_radial != 0 && !c->fused && !c->table && s.channels >= 64;
  *out = c;
  return TPC_OK;
}

void tpc_ctx_destroy(tpc_ctx* c) { delete c; }

tpc_status tpc_ctx_info(const tpc_ctx* c, tpc_info* info) {
  Errors E;
  if (!c || !info) {
    E.add(TPC_ERR_INVALID, "ctx and info must be non-null");
    return E.finish();
  }
  std::memset(info, 0, sizeof(*info));
  info->n_paths = c->tab.np;
  info->d_in = c->tab.din;
  info->d_sh = c->tab.dsh;
  info->d_out = c->tab.dout;
  info->r_width = c->tab.np * c->spec.channels;
  info->nnz_cg = c->tab.nnz;
  const size_t T = c->tsize;
  info->edge_buffer_bytes = T * (size_t)(c->tab.dsh + 8 + 4 + c->tab.np * c->spec.channels);
  info->dR_bytes = T * (size_t)c->tab.np * c->spec.channels;
  info->fwd_workspace_bytes = fwd_layout(c, 0).total;
  info->bwd_workspace_bytes_per_edge =
      T * (size_t)(c->tab.dsh * dy_parts(c) + 8 + (c->table ? 0 : c->hidden)) +
      T * (size_t)c->tab.np * c->spec.channels + (c->table ? sizeof(int32_t) : 0);
  info->fwd_workspace_bytes_per_edge = c->table ? sizeof(int32_t) : c->pair ? c->tsize * 8 : 0;
  info->bwd_workspace_bytes_fixed = bwd_layout(c, 0).total;
  info->dY_parts = dy_parts(c);
  info->dh_edge_bytes = T * (size_t)c->tab.din * c->spec.channels;
  info->table_bytes = table_bytes(c);
  info->fused_radial = c->fused ? 1 : 0;
  info->act_bytes = c->fused ? (size_t)(c->hidden / 32) * 192 : 0;
  info->pair_radial = c->pair ? 1 : 0;
  for (int p = 0; p < c->tab.np; ++p) {
    info->paths[p][0] = c->tab.path[p].l1;
    info->paths[p][1] = c->tab.path[p].l2;
    info->paths[p][2] = c->tab.path[p].l3;
  }
  return E.finish();
}

tpc_status tpc_cg_table(const tpc_ctx* c, int path, double* out, size_t n) {
  Errors E;
  if (!c || !out) {
    E.add(TPC_ERR_INVALID, "ctx and out must be non-null");
    return E.finish();
  }
  if (path < 0 || path >= c->tab.np) {
    E.add(TPC_ERR_INVALID, "path index out of range");
    return E.finish();
  }
  const tpc::Path& P = c->tab.path[path];
  const size_t need = (size_t)(2 * P.l1 + 1) * (2 * P.l2 + 1) * (2 * P.l3 + 1);
  if (n < need) {
    E.add(TPC_ERR_INVALID, "out holds %zu values, path needs %zu", n, need);
    return E.finish();
  }
  size_t k = 0;
  for (int a = 0; a <= 2 * P.l1; ++a)
    for (int b = 0; b <= 2 * P.l2; ++b)
      for (int d = 0; d <= 2 * P.l3; ++d) out[k++] = c->tab.cg[path][a][b][d];
  return TPC_OK;
}

tpc_status tpc_workspace_query(const tpc_ctx* c, int op, int64_t n_atoms, int64_t n_edges,
                               const double* cell, size_t* bytes) {
  Errors E;
  if (!c || !bytes) {
    E.add(TPC_ERR_INVALID, "ctx and bytes must be non-null");
    return E.finish();
  }
  if (n_atoms < 0 || n_edges < 0) E.add(TPC_ERR_INVALID, "sizes must be >= 0");
  if (op == TPC_OP_NBR) {
    if (!cell) {
      E.add(TPC_ERR_INVALID, "the neighbour build needs the cell");
      return E.finish();
    }
    tpc::NbrGrid g{};
    std::string why;
    if (!make_grid(cell, c->spec.r_cut, &g, &why)) E.add(TPC_ERR_INVALID, "%s", why.c_str());
    if (E.status != TPC_OK) return E.finish();
    *bytes = nbr_layout(n_atoms, (int64_t)g.nb[0] * g.nb[1] * g.nb[2]).total;
  } else if (op == TPC_OP_FWD) {
    *bytes = fwd_layout(c, n_edges).total;
  } else if (op == TPC_OP_BWD) {
    *bytes = bwd_layout(c, n_edges).total;
  } else if (op == TPC_OP_VIRIAL) {
    *bytes = virial_layout(n_atoms).total;
  } else if (op == TPC_OP_DOUBLE_BWD) {
    *bytes = dbl_layout(c, n_edges).total;
  } else if (op == TPC_OP_TABLE_FIT) {
    if (!c->table) E.add(TPC_ERR_INVALID, "the context has no radial table (radial_table_pieces = 0)");
    else *bytes = table_layout(c).total;
  } else {
    E.add(TPC_ERR_INVALID, "unknown op %d", op);
  }
  return E.finish();
}

tpc_status tpc_nbr_build(const tpc_ctx* c, int64_t n, const double* pos, const double* cell,
                         const int32_t* species, int64_t edge_cap, int32_t* row_ptr,
                         int32_t* src, int32_t* shift, int32_t* rev, int64_t* n_edges,
                         void* ws, size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  if (n < 0) E.add(TPC_ERR_INVALID, "n_atoms must be >= 0");
  if (n > (int64_t)1 << 24) E.add(TPC_ERR_UNSUPPORTED, "n_atoms above 2^24");
  if (edge_cap < 0) E.add(TPC_ERR_INVALID, "edge_cap must be >= 0");
  if (!cell) E.add(TPC_ERR_INVALID, "cell (host double[9]) must be non-null");
  if (!row_ptr) E.add(TPC_ERR_INVALID, "row_ptr must be non-null");
  if (!n_edges) E.add(TPC_ERR_INVALID, "n_edges must be non-null");
  if (n > 0 && !pos) E.add(TPC_ERR_INVALID, "pos must be non-null");
  if (pos && !aligned(pos, 8)) E.add(TPC_ERR_INVALID, "pos must be 8-byte aligned");
  if (edge_cap > 0 && (!src || !shift || !rev)) E.add(TPC_ERR_INVALID, "src, shift and rev must be non-null when edge_cap > 0");
  if (!ws && n > 0) E.add(TPC_ERR_INVALID, "workspace must be non-null");
  if (ws && !aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  tpc::NbrGrid g{};
  int64_t nbin = 0;
  if (cell) {
    std::string why;
    for (int k = 0; k < 9; ++k)
      if (!std::isfinite(cell[k])) why = "cell is not finite";
    if (why.empty() && make_grid(cell, c->spec.r_cut, &g, &why))
      nbin = (int64_t)g.nb[0] * g.nb[1] * g.nb[2];
    else
      E.add(TPC_ERR_INVALID, "%s", why.c_str());
  }
  NbrWs L{};
  if (E.status == TPC_OK) {
    L = nbr_layout(n, nbin);
    if (n > 0 && ws_bytes < L.total)
      E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  }
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n == 0) {
    TPC_HIP(tpc::launch_fill_i32(row_ptr, 1, 0, s), "nbr_build");
    *n_edges = 0;
    return TPC_OK;
  }
  char* w = static_cast<char*>(ws);
  int32_t* bin_of = reinterpret_cast<int32_t*>(w + L.bin_of);
  int32_t* bin_start = reinterpret_cast<int32_t*>(w + L.bin_start);
  int32_t* cursor = reinterpret_cast<int32_t*>(w + L.cursor);
  int32_t* bin_atoms = reinterpret_cast<int32_t*>(w + L.bin_atoms);
  int32_t* partials = reinterpret_cast<int32_t*>(w + L.partials);
  int32_t* status = reinterpret_cast<int32_t*>(w + L.status);

  TPC_HIP(tpc::launch_fill_i32(status, 8, 0, s), "nbr_build: clear status");
  TPC_HIP(tpc::launch_fill_i32(bin_start, nbin + 1, 0, s), "nbr_build: clear bins");
  TPC_HIP(tpc::launch_fill_i32(cursor, nbin, 0, s), "nbr_build: clear cursors");
  TPC_LAUNCH("nbr_bin", s, tpc::launch_nbr_bin(n, pos, g, species, c->spec.n_species, bin_of, bin_start, status, s),
             "nbr_build: bin");
  TPC_LAUNCH("nbr_scan", s, tpc::launch_scan_exclusive(bin_start, nbin, partials, s), "nbr_build: bin scan");
  TPC_LAUNCH("nbr_scatter", s, tpc::launch_nbr_scatter(n, bin_of, bin_start, cursor, bin_atoms, s), "nbr_build: scatter");
  TPC_LAUNCH("nbr_count", s, tpc::launch_nbr_count(n, pos, g, bin_of, bin_start, bin_atoms, row_ptr, status, s),
             "nbr_build: count");
  TPC_LAUNCH("nbr_scan", s, tpc::launch_scan_exclusive(row_ptr, n, partials, s), "nbr_build: row scan");
  // one wait: edge total and flags
  int32_t host_status[2] = {0, 0};
  TPC_HIP(hipMemcpyAsync(&host_status[0], status, sizeof(int32_t), hipMemcpyDeviceToHost, s),
          "nbr_build: read status");
  TPC_HIP(hipMemcpyAsync(&host_status[1], row_ptr + n, sizeof(int32_t), hipMemcpyDeviceToHost, s),
          "nbr_build: read edge count");
  TPC_HIP(hipStreamSynchronize(s), "nbr_build: wait");
  if (host_status[0]) {
    flag_messages(host_status[0], E);
    return E.finish();
  }
  if (host_status[1] < 0) {
    E.add(TPC_ERR_UNSUPPORTED, "more than 2^31-1 edges");
    return E.finish();
  }
  const int64_t ne = host_status[1];
  *n_edges = ne;
  if (ne > edge_cap) {
    E.add(TPC_ERR_CAPACITY, "the list needs %lld edges, edge_cap is %lld", (long long)ne,
          (long long)edge_cap);
    return E.finish();
  }
  TPC_LAUNCH("nbr_fill", s, tpc::launch_nbr_fill(n, pos, g, bin_of, bin_start, bin_atoms, row_ptr, src, shift, s),
             "nbr_build: fill");
  TPC_LAUNCH("nbr_reverse", s, tpc::launch_nbr_reverse(n, row_ptr, src, shift, rev, status, s), "nbr_build: reverse");
  // every edge must have found its reverse: the backward relies on symmetry
  TPC_HIP(hipMemcpyAsync(&host_status[0], status, sizeof(int32_t), hipMemcpyDeviceToHost, s),
          "nbr_build: read status");
  TPC_HIP(hipStreamSynchronize(s), "nbr_build: wait");
  if (host_status[0]) {
    flag_messages(host_status[0], E);
    return E.finish();
  }
  g_last_error.clear();
  return TPC_OK;
}

namespace {

void check_chunk(const tpc_ctx* c, int64_t n, int64_t row_begin, int64_t row_end,
                 int64_t edge_begin, int64_t edge_end, Errors& E) {
  if (n < 0) E.add(TPC_ERR_INVALID, "n_atoms must be >= 0");
  if (row_begin < 0 || row_end < row_begin || row_end > n)
    E.add(TPC_ERR_INVALID, "need 0 <= row_begin <= row_end <= n_atoms");
  if (edge_begin < 0 || edge_end < edge_begin) E.add(TPC_ERR_INVALID, "need 0 <= edge_begin <= edge_end");
  if (edge_end > INT32_MAX) E.add(TPC_ERR_UNSUPPORTED, "edge indices above 2^31-1");
  (void)c;
}

// The radial weights: n_layers matrices, or with a table context one
// pointer to the table written by tpc_radial_table_fit.
void check_weights(const tpc_ctx* c, const void* const* weights, Errors& E) {
  if (!weights) {
    E.add(TPC_ERR_INVALID, "weights must be non-null");
    return;
  }
  const int n = c->table ? 1 : c->spec.n_layers;
  for (int k = 0; k < n; ++k)
    if (!weights[k]) E.add(TPC_ERR_INVALID, "weights[%d] must be non-null", k);
}

void need_ptr(const void* p, const char* name, size_t align, Errors& E) {
  if (!p)
    E.add(TPC_ERR_INVALID, "%s must be non-null", name);
  else if (!aligned(p, align))
    E.add(TPC_ERR_INVALID, "%s must be %zu-byte aligned", name, align);
}

// Device checks of the inputs (spec.validate): the CSR rows of the call and,
// when given, the reverse index (symmetry) and the wrapping of the positions
// into the cell.  One wait for the combined status word.
tpc_status run_csr_check(int64_t n, int64_t n_edges, const int32_t* row_ptr, const int32_t* src,
                         const int32_t* shift, const int32_t* rev, int64_t rb, int64_t re,
                         int64_t eb, int64_t ee, int32_t* status, hipStream_t s,
                         const double* pos = nullptr, const tpc::NbrGrid* grid = nullptr) {
  TPC_HIP(tpc::launch_fill_i32(status, 1, 0, s), "csr check");
  TPC_HIP(tpc::launch_csr_check(n, n_edges, row_ptr, src, shift, rev, rb, re, eb, ee, status, s),
          "csr check");
  if (pos && grid) TPC_HIP(tpc::launch_wrap_check(n, pos, *grid, status, s), "position check");
  int32_t h = 0;
  TPC_HIP(hipMemcpyAsync(&h, status, sizeof(int32_t), hipMemcpyDeviceToHost, s), "csr check");
  TPC_HIP(hipStreamSynchronize(s), "csr check");
  if (h) {
    Errors E;
    flag_messages(h, E);
    return E.finish();
  }
  return TPC_OK;
}

}  // namespace

tpc_status tpc_conv_fwd(const tpc_ctx* c, int64_t n, const double* pos, const double* cell,
                        const int32_t* row_ptr, const int32_t* src, const int32_t* shift,
                        const int32_t* rev, int64_t row_begin, int64_t row_end, int64_t edge_begin, int64_t edge_end,
                        const void* h, const void* const* weights, double scale, void* out,
                        const tpc_edge_buffers* eb, void* ws, size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  check_chunk(c, n, row_begin, row_end, edge_begin, edge_end, E);
  if (!cell) E.add(TPC_ERR_INVALID, "cell (host double[9]) must be non-null");
  if (!std::isfinite(scale)) E.add(TPC_ERR_INVALID, "scale must be finite");
  const size_t va = 16;
  need_ptr(row_ptr, "row_ptr", 4, E);
  if (row_end > row_begin) {
    need_ptr(pos, "pos", 8, E);
    need_ptr(h, "h", va, E);
    need_ptr(out, "out", va, E);
  }
  if (edge_end > edge_begin) {
    need_ptr(src, "src", 4, E);
    need_ptr(shift, "shift", 4, E);
  }
  if (!eb) {
    E.add(TPC_ERR_INVALID, "edge buffers must be non-null");
  } else if (edge_end > edge_begin) {
    need_ptr(eb->Y, "eb.Y", va, E);
    need_ptr(eb->ef, "eb.ef", va, E);
    need_ptr(eb->rv, "eb.rv", va, E);
    if (c->fused) {
      need_ptr(eb->A, "eb.A", va, E);
      if (eb->R && !aligned(eb->R, va)) E.add(TPC_ERR_INVALID, "eb.R must be %zu-byte aligned", va);
    } else {
      need_ptr(eb->R, "eb.R", va, E);
    }
    if (c->pair) {
      need_ptr(rev, "rev", 4, E);
      need_ptr(eb->Rrow, "eb.Rrow", 4, E);
      if (edge_end - edge_begin > kPairMaxChunk)
        E.add(TPC_ERR_UNSUPPORTED, "shared R rows (spec.pair_radial) take chunks of at most %lld edges",
              (long long)kPairMaxChunk);
    }
  }
  check_weights(c, weights, E);
  const FwdWs FL = fwd_layout(c, edge_end - edge_begin);
  if (edge_end > edge_begin || c->spec.validate) {
    if (!ws) E.add(TPC_ERR_INVALID, "workspace must be non-null");
    else if (ws_bytes < FL.total)
      E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, FL.total);
  }
  if (ws && !aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->spec.validate) {
    tpc::NbrGrid grid{};
    std::string why;
    if (!make_grid(cell, c->spec.r_cut, &grid, &why)) {
      E.add(TPC_ERR_INVALID, "%s", why.c_str());
      return E.finish();
    }
    st = run_csr_check(n, edge_end, row_ptr, src, shift, nullptr, row_begin, row_end, edge_begin,
                       edge_end, reinterpret_cast<int32_t*>(static_cast<char*>(ws) + FL.status), s,
                       n > 0 ? pos : nullptr, &grid);
    if (st != TPC_OK) return st;
  }
  const int dt = c->spec.dtype;
  tpc::GeomArgs ga{};
  ga.pos = pos;
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) ga.cell[r][k] = cell[3 * r + k];
  ga.row_ptr = row_ptr;
  ga.src = src;
  ga.shift = shift;
  ga.row_begin = row_begin;
  ga.row_end = row_end;
  ga.edge_begin = edge_begin;
  ga.edge_end = edge_end;
  ga.r_cut = c->spec.r_cut;
  const int64_t ne = edge_end - edge_begin;
  if (ne > 0) {
    TPC_LAUNCH("geom_fwd", s, tpc::launch_geom_fwd(dt, c->spec.sh_lmax, ga, eb->Y, eb->ef, eb->rv, s),
               "conv_fwd: geometry");
    if (c->table) {
      TPC_LAUNCH("table_fwd", s,
                 tpc::launch_table_fwd(dt, ne, c->tab.np * c->spec.channels, c->spec.radial_table_pieces,
                                       c->spec.radial_table_degree, c->spec.r_cut, eb->rv, weights[0],
                                       static_cast<char*>(ws) + FL.tsort, eb->R, s),
                 "conv_fwd: radial table");
    } else {
      const tpc::RadialPack PL = pack_layout(c);
      void* pk = static_cast<char*>(ws) + FL.pack;
      TPC_LAUNCH("radial_pack", s, tpc::launch_radial_pack(dt, PL, weights, pk, s),
                 "conv_fwd: radial weight packing");
      if (c->fused)
        TPC_LAUNCH("radial_act", s, tpc::launch_radial_act(PL, ne, eb->ef, pk, eb->A, s),
                   "conv_fwd: radial hidden layers");
      else if (c->pair) {
        // one row of R per edge pair of the chunk: number the rows, gather
        // their basis values, and run the network on the rows only
        void* ef_rows = static_cast<char*>(ws) + FL.ef_rows;
        TPC_LAUNCH("pair_rows", s,
                   tpc::launch_pair_rows(dt, rev, edge_begin, ne, eb->Rrow,
                                         reinterpret_cast<int32_t*>(static_cast<char*>(ws) + FL.pair_part),
                                         eb->ef, ef_rows, s),
                   "conv_fwd: shared R rows");
        TPC_LAUNCH("radial_fwd", s, tpc::launch_radial_fwd(dt, PL, ne, eb->Rrow + ne, ef_rows, pk, eb->R, s),
                   "conv_fwd: radial MLP");
      } else
        TPC_LAUNCH("radial_fwd", s, tpc::launch_radial_fwd(dt, PL, ne, nullptr, eb->ef, pk, eb->R, s),
                   "conv_fwd: radial MLP");
    }
  }
  tpc::TPArgs ta{};
  ta.row_ptr = row_ptr;
  ta.src = src;
  ta.row_begin = row_begin;
  ta.row_end = row_end;
  ta.edge_begin = edge_begin;
  ta.C = c->spec.channels;
  ta.sum_paths = c->spec.sum_paths != 0;
  ta.scale = scale;
  ta.h = h;
  ta.Y = eb ? eb->Y : nullptr;
  ta.R = eb ? eb->R : nullptr;
  ta.Rrow = eb && c->pair ? eb->Rrow : nullptr;
  ta.n_chunk_edges = edge_end - edge_begin;
  ta.out = out;
  // a chunk without edges has no packed weights (the workspace may be null):
  // the unfused kernel writes its rows' zeros without reading any edge data
  if (c->fused && ne > 0) {
    const tpc::RadialPack PL = pack_layout(c);
    ta.act = eb ? eb->A : nullptr;
    ta.wfs = static_cast<const float*>(static_cast<const void*>(static_cast<char*>(ws) + FL.pack)) + PL.fs;
    ta.H = c->hidden;
    ta.R_out = eb ? eb->R : nullptr;
    TPC_LAUNCH("tp_fwd_fused", s,
               tpc::launch_tp_fused(c->spec.node_lmax, c->spec.sh_lmax, c->spec.out_lmax, ta, s),
               "conv_fwd: tensor product with the radial last layer");
  } else {
    TPC_LAUNCH("tp_fwd", s,
               tpc::launch_tp_fwd(dt, c->spec.node_lmax, c->spec.sh_lmax, c->spec.out_lmax, ta, s),
               "conv_fwd: tensor product");
  }
  g_last_error.clear();
  return TPC_OK;
}

tpc_status tpc_conv_fwd_noalloc(const tpc_ctx* c, int64_t n, const double* pos, const double* cell,
                                const int32_t* row_ptr, const int32_t* src, const int32_t* shift,
                                const int32_t* rev, int64_t row_begin, int64_t row_end, int64_t edge_begin, int64_t edge_end,
                                const void* h, const void* const* weights, double scale, void* out,
                                const tpc_edge_buffers* eb, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  void* scratch = nullptr;
  size_t cap = 0;
  const hipError_t e = tpc::scratch_for_current_device(&scratch, &cap);
  if (e != hipSuccess) return device_error(e, "conv_fwd_noalloc: device scratch address");
  const size_t need = fwd_layout(c, edge_end > edge_begin ? edge_end - edge_begin : 0).total;
  if (need > cap) {
    E.add(TPC_ERR_UNSUPPORTED, "this spec's forward needs %zu bytes of scratch; the fixed device scratch holds %zu",
          need, cap);
    return E.finish();
  }
  return tpc_conv_fwd(c, n, pos, cell, row_ptr, src, shift, rev, row_begin, row_end, edge_begin, edge_end, h,
                      weights, scale, out, eb, scratch, cap, stream);
}

tpc_status tpc_conv_bwd(const tpc_ctx* c, int64_t n, int64_t n_edges, const int32_t* row_ptr,
                        const int32_t* src, const int32_t* rev, int64_t row_begin, int64_t row_end,
                        int64_t edge_begin, int64_t edge_end, const void* h,
                        const void* const* weights, double scale, const void* grad_out,
                        const tpc_edge_buffers* eb, void* dR, void* g_edge, void* dh_edge, void* dh,
                        void* forces, void* ws, size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  check_chunk(c, n, row_begin, row_end, edge_begin, edge_end, E);
  if (n_edges < edge_end) E.add(TPC_ERR_INVALID, "n_edges must be >= edge_end");
  if (!std::isfinite(scale)) E.add(TPC_ERR_INVALID, "scale must be finite");
  const size_t va = 16;
  need_ptr(row_ptr, "row_ptr", 4, E);
  if (row_end > row_begin) {
    need_ptr(h, "h", va, E);
    need_ptr(grad_out, "grad_out", va, E);
  }
  if (edge_end > edge_begin) {
    need_ptr(src, "src", 4, E);
    need_ptr(rev, "rev", 4, E);
  }
  if (n_edges > 0) need_ptr(g_edge, "g_edge", 8, E);
  if (edge_end > edge_begin) need_ptr(dh_edge, "dh_edge", va, E);
  if (dh) {
    need_ptr(dh, "dh", va, E);
    if (n_edges > 0) {
      need_ptr(src, "src", 4, E);
      need_ptr(rev, "rev", 4, E);
    }
  }
  if (forces) {
    need_ptr(forces, "forces", 8, E);
    if (n_edges > 0) need_ptr(rev, "rev", 4, E);
  }
  if (dR && !aligned(dR, va)) E.add(TPC_ERR_INVALID, "dR must be 16-byte aligned");
  if (!eb) {
    E.add(TPC_ERR_INVALID, "edge buffers must be non-null");
  } else if (edge_end > edge_begin) {
    need_ptr(eb->Y, "eb.Y", va, E);
    need_ptr(eb->ef, "eb.ef", va, E);
    need_ptr(eb->rv, "eb.rv", va, E);
    need_ptr(eb->R, "eb.R", va, E);
    if (c->pair) need_ptr(eb->Rrow, "eb.Rrow", 4, E);
  }
  check_weights(c, weights, E);
  const int64_t ne = edge_end - edge_begin;
  const BwdWs L = bwd_layout(c, ne > 0 ? ne : 0);
  const size_t need = dR ? L.total_without_dR : L.total;
  if (!ws) E.add(TPC_ERR_INVALID, "workspace must be non-null");
  else if (!aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  if (ws && ws_bytes < need) E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(w + L.status);
  if (c->spec.validate) {
    st = run_csr_check(n, n_edges, row_ptr, src, nullptr, rev, row_begin, row_end, edge_begin, edge_end,
                       status, s);
    if (st != TPC_OK) return st;
  }
  const int dt = c->spec.dtype;
  const int L1 = c->spec.node_lmax, L2 = c->spec.sh_lmax, L3 = c->spec.out_lmax;
  void* dRp = dR ? dR : static_cast<void*>(w + L.dR);
  void* dY = w + L.dY;
  void* d_ef = w + L.d_ef;
  tpc::TPArgs ta{};
  ta.row_ptr = row_ptr;
  ta.src = src;
  ta.row_begin = row_begin;
  ta.row_end = row_end;
  ta.edge_begin = edge_begin;
  ta.C = c->spec.channels;
  ta.sum_paths = c->spec.sum_paths != 0;
  ta.scale = scale;
  ta.h = h;
  ta.Y = eb->Y;
  ta.R = eb->R;
  ta.Rrow = c->pair ? eb->Rrow : nullptr;
  ta.n_chunk_edges = ne;
  ta.G = grad_out;
  ta.rev = rev;
  ta.dR = dRp;
  ta.dY = dY;
  ta.dh_edge = dh_edge;
  if (ne > 0) {
    TPC_LAUNCH("tp_bwd_edge", s, tpc::launch_tp_bwd(dt, L1, L2, L3, ta, s), "conv_bwd: tensor product (edges)");
    if (c->table) {
      // dL/dr from the table's derivative series, into the d_ef region
      TPC_LAUNCH("table_bwd", s,
                 tpc::launch_table_bwd(dt, ne, c->tab.np * c->spec.channels, c->spec.radial_table_pieces,
                                       c->spec.radial_table_degree, c->spec.r_cut, eb->rv, weights[0], dRp,
                                       w + L.tsort, d_ef, s),
                 "conv_bwd: radial table");
      TPC_LAUNCH("geom_bwd", s,
                 tpc::launch_geom_bwd(dt, L2, ne, edge_begin, c->spec.r_cut, eb->rv, dY, dy_parts(c), nullptr,
                                      d_ef, g_edge, s),
                 "conv_bwd: geometry");
    } else {
      const tpc::RadialPack PL = pack_layout(c);
      void* pk = w + L.pack;
      void* dA = w + L.dA;
      TPC_LAUNCH("radial_pack", s, tpc::launch_radial_pack(dt, PL, weights, pk, s),
                 "conv_bwd: radial weight packing");
      TPC_LAUNCH("radial_bwd_dA", s, tpc::launch_radial_bwd_dA(dt, PL, ne, dRp, pk, dA, s),
                 "conv_bwd: radial last layer");
      TPC_LAUNCH("radial_bwd_mlp", s, tpc::launch_radial_bwd_mlp(dt, PL, ne, eb->ef, dA, pk, d_ef, s),
                 "conv_bwd: radial hidden layers");
      TPC_LAUNCH("geom_bwd", s,
                 tpc::launch_geom_bwd(dt, L2, ne, edge_begin, c->spec.r_cut, eb->rv, dY, dy_parts(c), d_ef,
                                      nullptr, g_edge, s),
                 "conv_bwd: geometry");
    }
  }
  if (dh) {
    tpc::DhGather g;
    g.n = n;
    g.din_c = c->tab.din * c->spec.channels;
    g.row_ptr = row_ptr;
    g.src = src;
    g.rev = rev;
    g.row_begin = row_begin;
    g.row_end = row_end;
    g.edge_begin = edge_begin;
    g.n_chunk_edges = ne;
    g.first = row_begin == 0;
    g.last = row_end == n;
    g.t_chunk = dh_edge;
    g.dh = dh;
    TPC_LAUNCH("dh_gather", s, tpc::launch_dh_gather(dt, g, scale, s), "conv_bwd: dh row sums");
  }
  if (forces)
    TPC_LAUNCH("forces", s, tpc::launch_forces(dt, n, row_ptr, rev, g_edge, forces, s), "conv_bwd: forces");
  g_last_error.clear();
  return TPC_OK;
}

tpc_status tpc_conv_double_bwd(const tpc_ctx* c, int64_t n, int64_t n_edges, const int32_t* row_ptr,
                               const int32_t* src, const int32_t* rev, int64_t row_begin, int64_t row_end,
                               int64_t edge_begin, int64_t edge_end, const void* h, double scale,
                               const void* grad_out, const tpc_edge_buffers* eb, const void* u_dh,
                               const void* u_dY, const void* u_dR, void* g_hat, void* h_hat, void* Y_hat,
                               void* R_hat, void* ws, size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  check_chunk(c, n, row_begin, row_end, edge_begin, edge_end, E);
  if (n_edges < edge_end) E.add(TPC_ERR_INVALID, "n_edges must be >= edge_end");
  if (!std::isfinite(scale)) E.add(TPC_ERR_INVALID, "scale must be finite");
  if (c->spec.sum_paths)
    E.add(TPC_ERR_UNSUPPORTED, "the double backward needs separate path outputs (sum_paths = 0)");
  const size_t va = 16;
  need_ptr(row_ptr, "row_ptr", 4, E);
  if (row_end > row_begin) {
    need_ptr(h, "h", va, E);
    need_ptr(grad_out, "grad_out", va, E);
    need_ptr(u_dh, "u_dh", va, E);
    need_ptr(g_hat, "g_hat", va, E);
    need_ptr(h_hat, "h_hat", va, E);
  }
  if (edge_end > edge_begin) {
    need_ptr(src, "src", 4, E);
    need_ptr(rev, "rev", 4, E);
    need_ptr(u_dY, "u_dY", c->tsize, E);
    need_ptr(u_dR, "u_dR", va, E);
    need_ptr(Y_hat, "Y_hat", c->tsize, E);
    need_ptr(R_hat, "R_hat", va, E);
  }
  if (!eb) {
    E.add(TPC_ERR_INVALID, "edge buffers must be non-null");
  } else if (edge_end > edge_begin) {
    need_ptr(eb->Y, "eb.Y", va, E);
    need_ptr(eb->R, "eb.R", va, E);
    if (c->pair) need_ptr(eb->Rrow, "eb.Rrow", 4, E);
  }
  const int64_t ne = edge_end - edge_begin;
  const DblWs L = dbl_layout(c, ne > 0 ? ne : 0);
  if (!ws) E.add(TPC_ERR_INVALID, "workspace must be non-null");
  else if (!aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  if (ws && ws_bytes < L.total) E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (c->spec.validate) {
    st = run_csr_check(n, n_edges, row_ptr, src, nullptr, rev, row_begin, row_end, edge_begin, edge_end,
                       reinterpret_cast<int32_t*>(w + L.status), s);
    if (st != TPC_OK) return st;
  }
  tpc::TPArgs ta{};
  ta.row_ptr = row_ptr;
  ta.src = src;
  ta.rev = rev;
  ta.row_begin = row_begin;
  ta.row_end = row_end;
  ta.edge_begin = edge_begin;
  ta.n_chunk_edges = ne;
  ta.C = c->spec.channels;
  ta.sum_paths = false;
  ta.scale = scale;
  ta.h = h;
  ta.Y = eb->Y;
  ta.R = eb->R;
  ta.Rrow = c->pair ? eb->Rrow : nullptr;
  ta.G = grad_out;
  ta.uh = u_dh;
  ta.uY = u_dY;
  ta.uR = u_dR;
  ta.g_hat = g_hat;
  ta.x_hat = h_hat;
  ta.w_hat = R_hat;
  ta.dY = w + L.yh;
  TPC_LAUNCH("tp_double_bwd", s,
             tpc::launch_tp_dbl(c->spec.dtype, c->spec.node_lmax, c->spec.sh_lmax, c->spec.out_lmax, ta, s),
             "conv_double_bwd: tensor product");
  TPC_LAUNCH("part_sum", s, tpc::launch_part_sum(c->spec.dtype, yh_parts(c), ne, c->tab.dsh, w + L.yh, Y_hat, s),
             "conv_double_bwd: y_hat slices");
  g_last_error.clear();
  return TPC_OK;
}

tpc_status tpc_radial_table_fit(const tpc_ctx* c, const void* const* weights, void* table, size_t table_bytes_,
                                double* certificate, void* ws, size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  if (!c->table) E.add(TPC_ERR_INVALID, "the context has no radial table (radial_table_pieces = 0)");
  if (!weights) {
    E.add(TPC_ERR_INVALID, "weights must be non-null");
  } else {
    for (int k = 0; k < c->spec.n_layers; ++k)
      if (!weights[k]) E.add(TPC_ERR_INVALID, "weights[%d] must be non-null", k);
  }
  if (!certificate) E.add(TPC_ERR_INVALID, "certificate (host double[2]) must be non-null");
  need_ptr(table, "table", 16, E);
  if (E.status == TPC_OK && table_bytes_ < table_bytes(c))
    E.add(TPC_ERR_INVALID, "table holds %zu bytes, needs %zu", table_bytes_, table_bytes(c));
  const TableWs L = c->table ? table_layout(c) : TableWs{};
  if (!ws) E.add(TPC_ERR_INVALID, "workspace must be non-null");
  else if (!aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  if (ws && c->table && ws_bytes < L.total)
    E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  double* cert_dev = reinterpret_cast<double*>(w + L.cert);
  const int pieces = c->spec.radial_table_pieces, deg = c->spec.radial_table_degree;
  TPC_LAUNCH("table_fit", s,
             tpc::launch_table_fit(c->spec.dtype, c->n_hidden, c->hidden, c->tab.np * c->spec.channels, pieces,
                                   deg, c->spec.r_cut, weights, reinterpret_cast<double*>(w + L.nodes), table,
                                   cert_dev, s),
             "radial_table_fit");
  const int npts = pieces;
  std::vector<double> cert(2 * (size_t)npts);
  TPC_HIP(hipMemcpyAsync(cert.data(), cert_dev, sizeof(double) * cert.size(), hipMemcpyDeviceToHost, s),
          "radial_table_fit: read certificate");
  TPC_HIP(hipStreamSynchronize(s), "radial_table_fit: wait");
  double rv = 0.0, rd = 0.0;
  for (int k = 0; k < npts; ++k) {
    rv = cert[2 * k] > rv ? cert[2 * k] : rv;
    rd = cert[2 * k + 1] > rd ? cert[2 * k + 1] : rd;
  }
  certificate[0] = rv;
  certificate[1] = rd;
  if (!(rv <= 1.0) || !(rd <= 1.0)) {
    E.add(TPC_ERR_PRECONDITION,
          "the table is not certified: error / rounding scale %.3g (values), %.3g (derivatives); "
          "more pieces or a higher degree are needed",
          rv, rd);
    return E.finish();
  }
  g_last_error.clear();
  return TPC_OK;
}

tpc_status tpc_virial(const tpc_ctx* c, int64_t n, int64_t n_edges, const double* pos,
                      const double* cell, const int32_t* row_ptr, const int32_t* src,
                      const int32_t* shift, const void* g_edge, void* virial, void* ws,
                      size_t ws_bytes, void* stream) {
  Errors E;
  if (!c) {
    E.add(TPC_ERR_INVALID, "ctx must be non-null");
    return E.finish();
  }
  if (n < 0) E.add(TPC_ERR_INVALID, "n_atoms must be >= 0");
  if (n_edges < 0) E.add(TPC_ERR_INVALID, "n_edges must be >= 0");
  if (n_edges > 0 && n == 0) E.add(TPC_ERR_INVALID, "edges need atoms");
  if (!cell) E.add(TPC_ERR_INVALID, "cell (host double[9]) must be non-null");
  else
    for (int k = 0; k < 9; ++k)
      if (!std::isfinite(cell[k])) {
        E.add(TPC_ERR_INVALID, "cell must be finite");
        break;
      }
  need_ptr(row_ptr, "row_ptr", 4, E);
  if (n_edges > 0) {
    need_ptr(pos, "pos", 8, E);
    need_ptr(src, "src", 4, E);
    need_ptr(shift, "shift", 4, E);
    need_ptr(g_edge, "g_edge", c->tsize, E);
  }
  need_ptr(virial, "virial", c->tsize, E);
  const VirialWs L = virial_layout(n > 0 ? n : 0);
  if (!ws) E.add(TPC_ERR_INVALID, "workspace must be non-null");
  else if (!aligned(ws, 256)) E.add(TPC_ERR_INVALID, "workspace must be 256-byte aligned");
  if (ws && ws_bytes < L.total) E.add(TPC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  tpc_status st = E.finish();
  if (st != TPC_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (c->spec.validate && n > 0) {
    st = run_csr_check(n, n_edges, row_ptr, src, shift, nullptr, 0, n, 0, n_edges,
                       reinterpret_cast<int32_t*>(w + L.status), s);
    if (st != TPC_OK) return st;
  }
  tpc::GeomArgs ga{};
  ga.pos = pos;
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) ga.cell[r][k] = cell[3 * r + k];
  ga.row_ptr = row_ptr;
  ga.src = src;
  ga.shift = shift;
  ga.row_begin = 0;
  ga.row_end = n;
  ga.edge_begin = 0;
  ga.edge_end = n_edges;
  TPC_LAUNCH("virial", s,
             tpc::launch_virial(c->spec.dtype, n, ga, g_edge, reinterpret_cast<double*>(w + L.part),
                                virial, s),
             "virial");
  g_last_error.clear();
  return TPC_OK;
}

}  // extern "C"
