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
 *    waits to learn the edge count and the reverse-index status, and calls
 *    with spec.validate, which wait for their input checks.
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
enum { TPC_OP_NBR = 0, TPC_OP_FWD = 1, TPC_OP_BWD = 2, TPC_OP_VIRIAL = 3, TPC_OP_DOUBLE_BWD = 4,
       TPC_OP_TABLE_FIT = 5 };

#define TPC_MAX_LAYERS 8
#define TPC_MAX_PATHS 32

typedef struct tpc_ctx tpc_ctx;

/* Immutable description of one convolution.  Node features carry the
 * natural-parity irreps l1 = 0..node_lmax (0e, 1o, 2e, 3o), edges carry real
 * harmonics l2 = 0..sh_lmax, outputs keep l3 = 0..out_lmax; every admissible
 * path is formed (FlashCart section 2, "Irreducible Cartesian tensors"). */
typedef struct tpc_spec {
  int dtype;                 /* TPC_F32, or TPC_F64 with node_lmax <= 1 */
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
  int validate;              /* nonzero: the calls also check their inputs on
                                the device and wait for the result: sorted rows
                                and senders in range (conv_fwd, conv_bwd,
                                virial), wrapped positions (conv_fwd), a
                                symmetric reverse index (conv_bwd) */
  int sum_paths;             /* nonzero: paths with the same output rank add
                                into one block (FlashCart section 3,
                                "Generating Cartesian tensor products"):
                                d_out = sum of (2 l3 + 1) over the ranks that
                                occur, (m3, channel) order inside a block;
                                G follows the same layout */
  int fp32_mfma_only;        /* float32 only.  0 (default): the radial last
                                layer's float32 products run as six bf16
                                matrix products of three-part operand splits
                                (about float32 accuracy; the split-product
                                option of the FastMACE page "Rewrites and
                                precision options").  Nonzero: every float32
                                product on float32 matrix cores. */
  int radial_table_pieces;   /* 0 (default): radial weights from the radial
                                network.  n > 0: from piecewise Chebyshev
                                tables of n equal pieces on [0, r_cut]
                                (FastMACE "Rewrites and precision options",
                                "Radial network", radial_tables), fitted and
                                certified by tpc_radial_table_fit; the
                                convolution calls then take one weights
                                pointer, the table */
  int radial_table_degree;   /* polynomial degree per piece, 1..16 */
  int fuse_radial;           /* 0 (default): the radial network writes R and
                                the tensor product reads it.  Nonzero, where
                                the shapes allow it (float32, bf16-split
                                products, hidden width 32 or 64, C a multiple
                                of 16, no table): the forward forms R inside
                                the tensor-product kernel from the last hidden
                                activations (the fused folded forward of the
                                FastMACE page "Rewrites and precision
                                options", section "Convolution (OEq
                                streaming)"), so a forward-only call needs no
                                R buffer; tpc_info.fused_radial says whether
                                it does.  It is slower than the two kernels
                                on this GPU (its tensor product runs at two
                                waves per SIMD) and is there for callers
                                short of memory. */
  int pair_radial;           /* 0 (default): one row of R per edge.  Nonzero,
                                with the radial network unfused, no table and
                                64 or 128 channels:
                                an edge and its reverse share one row of R.
                                The radial weights depend on the edge length
                                only (FlashCart section 2, distance-dependent
                                path weights; FastMACE "Rewrites and
                                precision options", "Radial network"), and
                                the reverse of an edge has the negated vector
                                and the same length bit for bit, so the
                                network runs once per pair of the chunk and
                                writes half the rows.  tpc_conv_fwd then
                                needs rev and eb.Rrow; tpc_info.pair_radial
                                says whether the mode is in effect. */
} tpc_spec;

typedef struct tpc_info {
  int n_paths;               /* P */
  int d_in, d_sh, d_out;     /* feature widths per channel */
  int r_width;               /* P*C */
  int nnz_cg;                /* non-zero coupling coefficients over all paths */
  int paths[TPC_MAX_PATHS][3];  /* (l1, l2, l3) in path order */
  /* Sizes of the buffers a caller allocates (bytes). */
  size_t edge_buffer_bytes;  /* per edge: Y, ef, rv and R of tpc_edge_buffers */
  size_t dR_bytes;           /* per edge: one row of dR */
  size_t fwd_workspace_bytes;          /* tpc_conv_fwd workspace: fixed part ... */
  size_t bwd_workspace_bytes_fixed;    /* tpc_conv_bwd workspace: fixed part ... */
  size_t bwd_workspace_bytes_per_edge; /* ... plus this per chunk edge (dR kept in
                                          the workspace when the caller passes
                                          none), up to 16 edges of rounding;
                                          tpc_workspace_query gives the exact
                                          figure */
  int dY_parts;              /* partial dY slices the backward keeps per edge */
  size_t dh_edge_bytes;      /* per chunk edge: one row of the dh_edge
                                buffer of tpc_conv_bwd */
  size_t table_bytes;        /* the radial table (0 without one) */
  size_t fwd_workspace_bytes_per_edge; /* ... plus this per chunk edge (a table
                                          context sorts the chunk's edges by
                                          piece, a pair_radial context keeps
                                          each row's basis values; 0
                                          otherwise), up to 512 bytes of
                                          rounding and, with pair_radial, 8
                                          bytes per 4,096 edges of scan sums;
                                          tpc_workspace_query gives the exact
                                          figure */
  int fused_radial;          /* 1: tpc_conv_fwd forms R inside the tensor-
                                product kernel (see spec.fuse_radial) */
  size_t act_bytes;          /* per edge: one row of tpc_edge_buffers.A (0
                                when fused_radial is 0) */
  int pair_radial;           /* 1: an edge and its reverse share one row of R
                                (see spec.pair_radial); tpc_edge_buffers.Rrow
                                is then required */
} tpc_info;

/* Per-edge buffers.  conv_fwd writes them for the edges of the rows it
 * processes; conv_bwd reads them for the same rows.  Every array is indexed by
 * (edge - edge_begin) of the call, in the context dtype. */
typedef struct tpc_edge_buffers {
  void* Y;    /* [E_chunk][d_sh]    harmonics of the edge direction */
  void* ef;   /* [E_chunk][8]       Bessel basis times envelope */
  void* rv;   /* [E_chunk][4]       edge vector (x, y, z) and its length */
  void* R;    /* [E_chunk][P*C]     radial weights; tpc_conv_bwd and
                                   tpc_conv_double_bwd read them.  With
                                   info.fused_radial the forward writes them
                                   only when R is non-null (a forward-only
                                   caller passes null and no R is stored).
                                   With info.pair_radial, row Rrow[k] holds
                                   the weights of edge edge_begin + k, and
                                   only the first Rrow[E_chunk] rows are
                                   written */
  void* A;    /* [E_chunk][info.act_bytes] bytes: the radial network's last
                 hidden activations in the library's own layout (written by
                 tpc_conv_fwd when info.fused_radial; unused otherwise, may be
                 null) */
  int32_t* Rrow; /* [E_chunk + 1] int32 with info.pair_radial (unused
                    otherwise, may be null): written by tpc_conv_fwd, read by
                    tpc_conv_bwd and tpc_conv_double_bwd.  Rrow[k] is the row
                    of R that edge edge_begin + k reads; Rrow[E_chunk] the
                    number of rows written.  An edge whose reverse lies in the
                    chunk shares the row of the lower-indexed of the two; an
                    edge whose reverse lies outside keeps a row of its own.
                    Rows are numbered in chunk order (deterministic). */
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
 * cell; TPC_OP_FWD, TPC_OP_BWD and TPC_OP_DOUBLE_BWD need the number of edges
 * of the chunk; TPC_OP_VIRIAL needs n_atoms. */
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
 * Waits on `stream` twice: for the edge count, and after the reverse index is
 * built for its status (an edge without a reverse returns
 * TPC_ERR_PRECONDITION). */
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
 *   rev       [n_edges] int32 from tpc_nbr_build, device: read with
 *             info.pair_radial (entries [edge_begin, edge_end)), else unused
 *             and may be null.  The forward trusts it: a reverse index that
 *             is not an involution gives wrong rows of R but no access
 *             outside R (tpc_conv_bwd with spec.validate checks it).  A chunk
 *             holds at most 2^24 edges in this mode (else
 *             TPC_ERR_UNSUPPORTED).
 *   h         [n_atoms][d_in][C], device
 *   weights   host array of n_layers device pointers, W_k [dims[k-1]][dims[k]]
 *             row-major, already scaled; no biases; SiLU after every layer but
 *             the last
 *   scale     s, the neighbour normalisation (1, or 1/avg_num_neighbors)
 *   out       [n_atoms][d_out][C], device; rows [row_begin,row_end) written
 *   eb        per-edge buffers written for the chunk: Y, ef and rv always;
 *             R unless info.fused_radial (then optional); A when
 *             info.fused_radial; Rrow when info.pair_radial
 *   workspace with info.pair_radial it also holds the rows' basis values
 *             (info.fwd_workspace_bytes_per_edge per chunk edge), so the
 *             forward that allocates nothing below refuses pair contexts
 *             whose chunk needs more than its fixed scratch
 */
tpc_status tpc_conv_fwd(const tpc_ctx* ctx, int64_t n_atoms, const double* pos,
                        const double* cell, const int32_t* row_ptr, const int32_t* src,
                        const int32_t* shift, const int32_t* rev, int64_t row_begin, int64_t row_end,
                        int64_t edge_begin, int64_t edge_end, const void* h,
                        const void* const* weights, double scale, void* out,
                        const tpc_edge_buffers* eb, void* workspace, size_t workspace_bytes,
                        void* stream);

/* tpc_conv_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch (the radial weights in
 * matrix-core operand order and a status word) lives in a fixed array of
 * device memory inside the library, 16 MiB per GPU, held from the first call
 * on that GPU until the process ends; the device address of each GPU's copy
 * is looked up once per device.  The call allocates nothing.  Specs whose
 * forward needs more scratch than the array holds (never for the built
 * configurations at up to 128 channels) return TPC_ERR_UNSUPPORTED.  Every
 * call on one GPU uses the same array: calls that overlap on one GPU (on
 * different streams, or from different threads) race on it and must be
 * ordered by the caller.  Arguments, outputs and errors otherwise as for
 * tpc_conv_fwd. */
tpc_status tpc_conv_fwd_noalloc(const tpc_ctx* ctx, int64_t n_atoms, const double* pos,
                                const double* cell, const int32_t* row_ptr, const int32_t* src,
                                const int32_t* shift, const int32_t* rev, int64_t row_begin, int64_t row_end,
                                int64_t edge_begin, int64_t edge_end, const void* h,
                                const void* const* weights, double scale, void* out,
                                const tpc_edge_buffers* eb, void* stream);

/* Backward of L = sum(G * out) for receivers [row_begin, row_end).
 *   n_edges   total edges of the list (g_edge and rev span all of them)
 *   rev       [n_edges] int32 from tpc_nbr_build
 *   grad_out  G [n_atoms][d_out][C], device
 *   eb        per-edge buffers of the same chunk, as written by tpc_conv_fwd
 *             (with info.pair_radial its Rrow map too: each edge's row of R)
 *   dR        [E_chunk][P*C] device, nullable (then kept in the workspace):
 *             dL/dR, the inner product of G with the unweighted product
 *             (FlashCart section 3, "Symbolic derivatives")
 *   g_edge    [n_edges][3] device, out: dL/d(edge vector), absolute edge index
 *   dh_edge   [E_chunk][d_in][C] device, scratch of the call: each chunk
 *             edge's contribution to dL/dh of its sender, at the edge's own
 *             slot (reused by the next chunk's call)
 *   dh        [n_atoms][d_in][C] device, nullable: dL/dh for every atom, the
 *             sum over the entries of row j of the reverse edges'
 *             contributions, times s.  Pass it on every chunk's call (or on
 *             none), chunks in ascending row order covering [0, n_atoms):
 *             each call continues every atom's sum with the entries of its
 *             row whose sender lies in the chunk (the call with row_begin 0
 *             starts the sums; between calls dh holds the unscaled partial
 *             sums; the call with row_end n_atoms stores s * sum).  Each row
 *             must be sorted by sender, as tpc_nbr_build leaves it; the
 *             result then equals the unchunked call's bit for bit.
 *   forces    [n_atoms][3] device, nullable: F = -dL/dx from g_edge of every
 *             edge
 * forces reads g_edge of every edge, so pass it only on the call that
 * finishes the last chunk (all chunks' g_edge written earlier on this
 * stream); an unchunked call passes everything at once.
 * With spec.validate the chunk's rows, sender indices and reverse index are
 * checked first (TPC_ERR_PRECONDITION for an unsorted or non-symmetric list);
 * a reverse index that leaves the chunk adds nothing to dh rather than being
 * read.  No atomics: every sum runs in a fixed order.
 */
tpc_status tpc_conv_bwd(const tpc_ctx* ctx, int64_t n_atoms, int64_t n_edges,
                        const int32_t* row_ptr, const int32_t* src, const int32_t* rev,
                        int64_t row_begin, int64_t row_end, int64_t edge_begin,
                        int64_t edge_end, const void* h, const void* const* weights,
                        double scale, const void* grad_out, const tpc_edge_buffers* eb,
                        void* dR, void* g_edge, void* dh_edge, void* dh, void* forces,
                        void* workspace, size_t workspace_bytes, void* stream);

/* VJP-of-VJP ("double backward") of the tensor product for receivers
 * [row_begin, row_end) (FlashCart section 3, "Symbolic derivatives": training
 * on forces differentiates through the VJP; section 4, "Receiver-sorted
 * derivatives": the same receiver-sorted edges, the incoming gradient of a
 * receiver loaded once per program).  The VJP of tpc_conv_bwd maps
 * (h, Y, R, G) to (dh, dY, dR).  Given cotangents u_dh, u_dY, u_dR of those
 * outputs, this call differentiates
 *     Lam = <u_dh, dh> + <u_dY, dY> + <u_dR, dR>
 * with respect to G, h, Y and R (Y and R taken as independent inputs of the
 * product; chaining into the radial network and the geometry is the
 * caller's).  With T(a, y) the unweighted product of a path:
 *     g_hat[i] = s sum_{e in row i} uR T(h_j, Y) + R T(h_j, uY) + R T(uh_j, Y)
 *     h_hat[j] = s sum_{e: src e = j} sum_p C . (uR Y + R uY) . G[i]
 *     Y_hat[e] = s sum_u sum_p C . (uR h_j + R uh_j) . G[i]
 *     R_hat[e] = s sum_m3 G[i] . (T(h_j, uY) + T(uh_j, Y))
 * h_hat is gathered along each row through the symmetric list (the reverse
 * edge's cotangents are read at rev[e]); every sum has a fixed order, no
 * atomics.
 *   rev       [n_edges] int32 from tpc_nbr_build
 *   h, grad_out, eb (Y and R of the chunk, and Rrow with info.pair_radial)
 *             as for tpc_conv_bwd; R_hat stays per edge (a caller that wants
 *             the gradient of a shared row adds the two edges' rows)
 *   u_dh      [n_atoms][d_in][C] device
 *   u_dY      [n_edges][d_sh] device, every edge (absolute index: the sender
 *             side reads it at reverse edges outside the chunk)
 *   u_dR      [n_edges][P*C] device, every edge (absolute index)
 *   g_hat     [n_atoms][d_out][C] device, out: rows [row_begin, row_end)
 *   h_hat     [n_atoms][d_in][C] device, out: rows [row_begin, row_end)
 *   Y_hat     [E_chunk][d_sh] device, out (chunk index)
 *   R_hat     [E_chunk][P*C] device, out (chunk index)
 *   workspace tpc_workspace_query(TPC_OP_DOUBLE_BWD, n_atoms, E_chunk)
 * Separate path outputs only: with spec.sum_paths the call returns
 * TPC_ERR_UNSUPPORTED.  With spec.validate the rows and the reverse index are
 * checked first. */
tpc_status tpc_conv_double_bwd(const tpc_ctx* ctx, int64_t n_atoms, int64_t n_edges,
                               const int32_t* row_ptr, const int32_t* src, const int32_t* rev,
                               int64_t row_begin, int64_t row_end, int64_t edge_begin,
                               int64_t edge_end, const void* h, double scale, const void* grad_out,
                               const tpc_edge_buffers* eb, const void* u_dh, const void* u_dY,
                               const void* u_dR, void* g_hat, void* h_hat, void* Y_hat, void* R_hat,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Fit and certify the piecewise Chebyshev radial table of a context with
 * spec.radial_table_pieces > 0 (FastMACE page "Rewrites and precision
 * options", section "Radial network", radial_tables: the radial chain is
 * replaced by per-piece Chebyshev tables fitted when the plan is built; the
 * "certified" class of the rewrite classes: the table's error, measured
 * against a float64 evaluation of the same weights, must not exceed the
 * rounding error of the computation it replaces, for values and first
 * derivatives).  The radial weights here depend on the edge length only, so
 * one table serves every species pair.
 *   weights      n_layers device pointers of the radial network (as for
 *                tpc_conv_fwd without a table)
 *   table        device, out: [pieces][2 degree + 1][P*C] in the context
 *                dtype: degree + 1 rows of Chebyshev coefficients of R(r) on
 *                each piece, then degree rows of its r-derivative series
 *   certificate  host double[2], out: over the pieces and columns, the
 *                largest ratio of the table's largest error on a piece
 *                (evaluated as the convolution evaluates it) to the largest
 *                float rounding scale of the replaced computation on that
 *                piece, for values and for r-derivatives; each piece is
 *                checked at 8 points (its start and points between its
 *                interpolation nodes)
 *   workspace    tpc_workspace_query(TPC_OP_TABLE_FIT)
 * The rounding scale at a point is H eps sum_k |a_k W_kc| + eps |r R'| for
 * values and H eps sum_k |a'_k W_kc| + eps |R'| for derivatives (a the last
 * hidden activations, H their count, eps the unit roundoff of the dtype):
 * the last layer's dot product and the rounding of the distance it is given.
 * Both are taken as maxima over the piece (the range the table serves)
 * because the weights and their scale vanish together at points (the
 * derivative at r = 0, the envelope's triple zero at r_cut) where no float
 * table's absolute rounding follows the network's relative accuracy.
 * Waits for the certificate.  Returns TPC_OK when both ratios are at most 1,
 * TPC_ERR_PRECONDITION otherwise (the table is written but must not be used;
 * keep the radial network). */
tpc_status tpc_radial_table_fit(const tpc_ctx* ctx, const void* const* weights, void* table,
                                size_t table_bytes, double* certificate, void* workspace,
                                size_t workspace_bytes, void* stream);

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

/* Messages of the last failed call on this thread ("" if none).  Errors are
 * kept per thread rather than per context: tpc_ctx_create can fail before a
 * context exists, and concurrent calls on one context from several threads
 * each see their own messages. */
const char* tpc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPCONV_H */
