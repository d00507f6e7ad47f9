/*
 * tpconv.h -- C ABI of the MI355X (gfx950) equivariant interaction convolution.
 *
 * The library computes, for a periodic system of atoms, the MACE-style
 * channelwise ("uvu") tensor-product convolution and its backward pass:
 *
 *   out[i,(p,m3),u] = s * sum_{e in row i} R[e,p*C+u] *
 *                     sum_{m1,m2} C^p[m1,m2,m3] h[src_e,(l1,m1),u] Y[e,(l2,m2)]
 *
 * following the equivariant convolution of the FlashCart paper ("FlashCart:
 * Fast Cartesian Tensor Products for Equivariant Interatomic Potentials",
 * section 2, "Equivariant convolution and many-body correlations"): sender
 * features are coupled with the edge's direction tensor along every admissible
 * path (l1,l2)->l3 (section 2, "Irreducible Cartesian tensors"), weighted by a
 * per-path, per-channel radial weight R(|r|) and summed per receiver.  Edges
 * are receiver-sorted CSR (section 4, "Data layout"); the receiver sum is
 * accumulated in registers and stored once, with no atomics.  R comes from a
 * radial MLP (the "Radial network" section of the FastMACE page "Rewrites and
 * precision options") applied to an 8-term Bessel basis times a p=5
 * polynomial envelope.  Forces are the negative position gradient of the
 * surrogate scalar L = sum(G * out) (FlashCart section 2, "Machine-learned
 * interatomic potentials").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Device pointers are HIP device addresses the caller allocated and owns.
 *    Host pointers are marked "host".  The library keeps no pointer after a
 *    call returns and allocates no device memory in any call: scratch comes
 *    from the caller's workspace (size from tpc_workspace_query).
 *  - Positions and the cell are float64 always (positions, momenta and the
 *    integrator stay float64 on the FastMACE page, "PrecisionConfig").
 *    Features, weights and every output use the context dtype (float32 or
 *    float64).  int32 index arrays.
 *  - Cell: host double[9], row-major rows a1, a2, a3 (Angstrom).  An image
 *    shift S = (s1,s2,s3) translates an atom by s1*a1 + s2*a2 + s3*a3.
 *  - Layouts (FlashCart section 4, "Data layout": one contiguous block per
 *    rank, lower ranks first, channels contiguous):
 *      h, dh      [N][d_in][C]   l1 blocks ascending, m1 = -l1..l1
 *      out, G     [N][d_out][C]  l3 blocks ascending; inside an l3 block the
 *                                order is (m3, q, channel), q ranking the
 *                                paths with that l3 in path order (with
 *                                spec.sum_paths: (m3, channel), one block
 *                                per l3)
 *      R, dR      [E][P*C]       column p*C + u, paths in lexicographic
 *                                (l1,l2,l3) order
 *      Y          [E][d_sh]      real harmonics, index l*l + (m+l)
 *  - Streams: every call enqueues on `stream` (a hipStream_t; NULL is the
 *    default stream) and returns without waiting, except tpc_nbr_build which
 *    waits once to learn the edge count.
 *  - Errors: every entry point returns a tpc_status.  On failure nothing is
 *    enqueued (argument checks run before any device work) and
 *    tpc_last_error() lists every failed check.  There is no silent fallback:
 *    a request this library does not implement returns TPC_ERR_UNSUPPORTED.
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs run to run on the same GPU (no floating-point atomics).
 *  - A context is immutable after creation; concurrent calls on different
 *    streams with separate workspaces are allowed.
 */
#ifndef TPCONV_H
#define TPCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tpc_status {
  TPC_OK = 0,
  TPC_ERR_INVALID = 1,      /* bad argument: null/misaligned pointer, size, spec value */
  TPC_ERR_UNSUPPORTED = 2,  /* valid request that this library does not implement */
  TPC_ERR_CAPACITY = 3,     /* edge_cap too small; *n_edges holds the needed count */
  TPC_ERR_PRECONDITION = 4, /* input breaks a documented precondition (unwrapped
                               positions, unsorted or inconsistent CSR) */
  TPC_ERR_WORKSPACE = 5,    /* workspace smaller than tpc_workspace_query reports */
  TPC_ERR_DEVICE = 6        /* the HIP runtime reported an error */
} tpc_status;

enum { TPC_F32 = 0, TPC_F64 = 1 };
enum { TPC_OP_NBR = 0, TPC_OP_FWD = 1, TPC_OP_BWD = 2, TPC_OP_VIRIAL = 3 };

#define TPC_MAX_LAYERS 8
#define TPC_MAX_PATHS 32

typedef struct tpc_ctx tpc_ctx;

/* Immutable description of one convolution.  Node features carry the
 * natural-parity irreps l1 = 0..node_lmax (0e, 1o, 2e, 3o), edges carry real
 * harmonics l2 = 0..sh_lmax, outputs keep l3 = 0..out_lmax; every admissible
 * path is formed (FlashCart section 2, "Irreducible Cartesian tensors"). */
typedef struct tpc_spec {
  int dtype;                 /* TPC_F32 or TPC_F64 */
  int channels;              /* C: 1..64, or 128 */
  int node_lmax;             /* 0..3 */
  int sh_lmax;               /* 0..3 */
  int out_lmax;              /* 0..3 */
  int n_bessel;              /* must be 8 */
  int poly_p;                /* envelope exponent, must be 5 */
  int n_species;             /* species ids must lie in [0, n_species) */
  double r_cut;              /* cutoff radius (Angstrom), > 0 */
  int n_layers;              /* number of weight matrices, 2..TPC_MAX_LAYERS */
  int layer_dims[TPC_MAX_LAYERS + 1]; /* [0] = n_bessel, [n_layers] = P*C; hidden
                                         widths all equal, one of 16, 32, 64 */
  int validate;              /* nonzero: conv_fwd/conv_bwd also check the CSR
                                on the device (sorted rows, src in range) and
                                wait for the result */
  int sum_paths;             /* nonzero: paths with the same output rank add
                                into one block (FlashCart section 3,
                                "Generating Cartesian tensor products"):
                                d_out = sum of (2 l3 + 1) over the ranks that
                                occur, (m3, channel) order inside a block;
                                G follows the same layout */
} tpc_spec;

typedef struct tpc_info {
  int n_paths;               /* P */
  int d_in, d_sh, d_out;     /* feature widths per channel */
  int r_width;               /* P*C */
  int nnz_cg;                /* non-zero coupling coefficients over all paths */
  int paths[TPC_MAX_PATHS][3];  /* (l1, l2, l3) in path order */
} tpc_info;

/* Per-edge buffers.  conv_fwd writes them for the edges of the rows it
 * processes; conv_bwd reads them for the same rows.  Every array is indexed by
 * (edge - edge_begin) of the call, in the context dtype. */
typedef struct tpc_edge_buffers {
  void* Y;    /* [E_chunk][d_sh]    harmonics of the edge direction */
  void* ef;   /* [E_chunk][8]       Bessel basis times envelope */
  void* rv;   /* [E_chunk][4]       edge vector (x, y, z) and its length */
  void* R;    /* [E_chunk][P*C]     radial weights */
} tpc_edge_buffers;

/* Create a context from a spec (host only; no device call).  Checks every
 * field and, on failure, lists every reason (TPC_ERR_INVALID or
 * TPC_ERR_UNSUPPORTED).  *ctx is set on success. */
tpc_status tpc_ctx_create(const tpc_spec* spec, tpc_ctx** ctx);
void tpc_ctx_destroy(tpc_ctx* ctx);
tpc_status tpc_ctx_info(const tpc_ctx* ctx, tpc_info* info);

/* Coupling tensor of path `path` as host double[(2l1+1)(2l2+1)(2l3+1)] in
 * [m1][m2][m3] order: the real Gaunt tensor of the path scaled to unit
 * Frobenius norm (FlashCart section 2: the equivariant couplings of an
 * admissible path form a one-dimensional space). */
tpc_status tpc_cg_table(const tpc_ctx* ctx, int path, double* out, size_t n);

/* Workspace bytes for an operation: TPC_OP_NBR needs n_atoms and the host
 * cell; TPC_OP_FWD and TPC_OP_BWD need the number of edges of the chunk;
 * TPC_OP_VIRIAL needs n_atoms. */
tpc_status tpc_workspace_query(const tpc_ctx* ctx, int op, int64_t n_atoms,
                               int64_t n_edges, const double* cell, size_t* bytes);

/* Neighbour list (FlashCart section 2: every atom and periodic image within
 * r_cut, except the atom itself in the reference cell; section 4: receiver
 * order, row pointers and a sender array).  An edge (i <- j, S) exists iff, in
 * float64 with no fused multiply-add,
 *    r = (x_j - x_i) + ((s1*a1 + s2*a2) + s3*a3),
 *    (r_x*r_x + r_y*r_y) + r_z*r_z < r_cut*r_cut.
 * Rows follow atom order; each row is sorted by (src, s1, s2, s3).
 *   pos       [n_atoms][3] float64, device; fractional coordinates must lie in
 *             [0,1) (a tolerance of 1e-10 is accepted), else
 *             TPC_ERR_PRECONDITION
 *   species   [n_atoms] int32, device, nullable; checked against n_species
 *   edge_cap  capacity of src/shift/rev; if the list needs more edges the call
 *             returns TPC_ERR_CAPACITY with *n_edges = the needed count and
 *             writes only row_ptr (the caller reallocates and calls again, the
 *             overflow protocol of the pet-jax README's two-phase list)
 *   row_ptr   [n_atoms+1] int32, device, out
 *   src       [edge_cap] int32, device, out
 *   shift     [edge_cap][3] int32, device, out
 *   rev       [edge_cap] int32, device, out: index of the reverse edge
 *             (j <- i, -S); the list is symmetric, so it always exists
 *   n_edges   host, out
 * Waits on `stream` once (to read the edge count). */
tpc_status tpc_nbr_build(const tpc_ctx* ctx, int64_t n_atoms, const double* pos,
                         const double* cell, const int32_t* species, int64_t edge_cap,
                         int32_t* row_ptr, int32_t* src, int32_t* shift, int32_t* rev,
                         int64_t* n_edges, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Forward convolution for receivers [row_begin, row_end), whose edges are
 * [edge_begin, edge_end) = [row_ptr[row_begin], row_ptr[row_end]).
 *   pos, cell, row_ptr, src, shift   as produced by tpc_nbr_build (rows must be
 *             receiver-sorted: FastMACE's receiver-streaming kernels give wrong
 *             results on unsorted edges, so with spec.validate the CSR is
 *             checked and TPC_ERR_PRECONDITION returned)
 *   h         [n_atoms][d_in][C], device
 *   weights   host array of n_layers device pointers, W_k [dims[k-1]][dims[k]]
 *             row-major, already scaled; no biases; SiLU after every layer but
 *             the last
 *   scale     s, the neighbour normalisation (1, or 1/avg_num_neighbors)
 *   out       [n_atoms][d_out][C], device; rows [row_begin,row_end) written
 *   eb        per-edge buffers written for the chunk (all four required)
 */
tpc_status tpc_conv_fwd(const tpc_ctx* ctx, int64_t n_atoms, const double* pos,
                        const double* cell, const int32_t* row_ptr, const int32_t* src,
                        const int32_t* shift, int64_t row_begin, int64_t row_end,
                        int64_t edge_begin, int64_t edge_end, const void* h,
                        const void* const* weights, double scale, void* out,
                        const tpc_edge_buffers* eb, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Backward of L = sum(G * out) for receivers [row_begin, row_end).
 *   n_edges   total edges of the list (g_edge, dh_edge and rev span all of them)
 *   rev       [n_edges] int32 from tpc_nbr_build
 *   grad_out  G [n_atoms][d_out][C], device
 *   eb        per-edge buffers of the same chunk, as written by tpc_conv_fwd
 *   dR        [E_chunk][P*C] device, nullable (then kept in the workspace):
 *             dL/dR, the inner product of G with the unweighted product
 *             (FlashCart section 3, "Symbolic derivatives")
 *   g_edge    [n_edges][3] device, out: dL/d(edge vector), absolute edge index
 *   dh_edge   [n_edges][d_in][C] device, out: each edge's contribution to dL/dh
 *             of its sender, stored at the reverse edge's slot (so the
 *             contributions to atom j fill row j of the list)
 *   dh        [n_atoms][d_in][C] device, nullable: dL/dh = s * row sums of
 *             dh_edge, for every atom
 *   forces    [n_atoms][3] device, nullable: F = -dL/dx from g_edge of every
 *             edge
 * dh and forces read the per-edge outputs of every edge, so pass them only on
 * the call that finishes the last chunk (all chunks' per-edge outputs written
 * earlier on this stream); an unchunked call passes everything at once.
 * No atomics: every sum runs in a fixed order.
 */
tpc_status tpc_conv_bwd(const tpc_ctx* ctx, int64_t n_atoms, int64_t n_edges,
                        const int32_t* row_ptr, const int32_t* src, const int32_t* rev,
                        int64_t row_begin, int64_t row_end, int64_t edge_begin,
                        int64_t edge_end, const void* h, const void* const* weights,
                        double scale, const void* grad_out, const tpc_edge_buffers* eb,
                        void* dR, void* g_edge, void* dh_edge, void* dh, void* forces,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Virial of L: W[a][b] = dL/d(eps_ab) for a homogeneous strain
 * x -> (I + eps) x applied to the positions and the cell rows together.  This
 * is the strain derivative the pet-jax README ("Conventions") calls the
 * virial, from one structure's strained cell as in the Stress option of
 * FastMACE's "Rewrites and precision options"; the stress of a structure of
 * volume V is W / V.  With the list fixed every edge vector becomes
 * (I + eps) r_e, so W[a][b] = sum_e g_e[a] r_e[b], with r_e formed in float64
 * exactly as tpc_nbr_build forms it.
 *   pos, cell, row_ptr, src, shift   as for tpc_conv_fwd, all n_atoms rows
 *   g_edge    [n_edges][3] device: dL/dr_e from tpc_conv_bwd (every chunk's
 *             edges written earlier on this stream)
 *   virial    [3][3] device, out: row-major W in the context dtype (zero for
 *             a list without edges)
 * The sums run in float64 in a fixed order (each row in CSR order, then fixed
 * trees over rows and blocks): deterministic, no atomics.  With
 * spec.validate the CSR is checked first (TPC_ERR_PRECONDITION). */
tpc_status tpc_virial(const tpc_ctx* ctx, int64_t n_atoms, int64_t n_edges, const double* pos,
                      const double* cell, const int32_t* row_ptr, const int32_t* src,
                      const int32_t* shift, const void* g_edge, void* virial,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing with HIP events, for benchmarks and profiling.  While
 * enabled on a thread, every kernel the library launches from that thread is
 * bracketed by two hipEventRecord calls on the launch stream.
 * tpc_timing_collect waits for the recorded events, writes one entry per
 * kernel name (total milliseconds and launch count, in first-launch order,
 * at most `max` entries), sets *n and clears the record.  Events come from a
 * per-thread pool created on first use; no device memory is allocated. */
typedef struct tpc_kernel_time {
  char name[32];
  double total_ms;
  int64_t launches;
} tpc_kernel_time;
tpc_status tpc_timing_enable(int on);
tpc_status tpc_timing_collect(tpc_kernel_time* out, int max, int* n);

const char* tpc_status_string(tpc_status status);

/* Messages of the last failed call on this thread ("" if none). */
const char* tpc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPCONV_H */
