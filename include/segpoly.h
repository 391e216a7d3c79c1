/*
 * segpoly.h -- C ABI of the fused equivariant segmented tensor products on
 * AMD Instinct MI355X (gfx950).
 *
 * Two operations, each one kernel launch:
 *
 *  - the channelwise ("uvu") Clebsch-Gordan tensor-product convolution:
 *    gather node features by source index, couple them with per-edge
 *    spherical harmonics through every (l1, l2, lo) path at once, scale by
 *    per-edge per-path per-channel weights, and sum-scatter into destination
 *    nodes.  Defined by the descriptor [ijk]*a[uv]*b[iu]*c[jv] -> D[kuv]
 *    (e3nn-course "Lesson 12a: Foundations of cuEquivariance", section 21.4)
 *    executed with source/destination indices as in the cuequivariance-torch
 *    skill document, sections "Channelwise product with external per-example
 *    weights" and "SegmentedPolynomial: gather and scatter".
 *
 *  - the symmetric contraction of degrees 1..3 with element-indexed weights
 *    (Lesson 12a, section 21.4.1; skill document, "Other operations and
 *    layers", SymmetricContraction).
 *
 * Conventions common to every function:
 *  - Every function returns SEGPOLY_OK (0) or a negative status; no C++
 *    exception crosses this boundary.  After a failure,
 *    segpoly_last_error() returns a message for the calling thread.
 *  - Device pointers are plain addresses of device memory owned by the
 *    caller; the library never frees them, never keeps them after a call
 *    returns, and never allocates on the compute calls except the one-time
 *    upload of coefficient tables described at tp_conv_fwd / symcon_fwd.
 *  - `stream` is a hipStream_t (NULL: the default stream).  Compute calls
 *    are asynchronous and stream-ordered; they do not synchronise unless the
 *    VALIDATE flag is set.
 *  - Handles hold only host state (descriptor, tables) and may be created,
 *    queried and destroyed on a machine without a GPU.  A handle may be used
 *    from several threads for compute calls; create/destroy are not
 *    concurrent with other uses of the same handle.
 *  - Irreps strings: O(3) irreps "MULxLP + ..." with P = e or o, e.g.
 *    "32x0e + 32x1o" (Lesson 12a, section 21.2).
 *  - Layouts (Lesson 12a, section 21.3): SEGPOLY_MUL_IR stores each block as
 *    [mul][2l+1], SEGPOLY_IR_MUL as [2l+1][mul].  The layout is part of the
 *    handle; passing data in the other layout is not detectable and gives
 *    wrong numbers, as on the pages.
 */
#ifndef SEGPOLY_H
#define SEGPOLY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SEGPOLY_OK 0
#define SEGPOLY_E_INVALID (-1)     /* null pointer, negative size, bad enum, mismatched sizes */
#define SEGPOLY_E_PARSE (-2)       /* malformed irreps string */
#define SEGPOLY_E_UNSUPPORTED (-3) /* outside the supported envelope: fails closed, never falls back */
#define SEGPOLY_E_UNSORTED (-4)    /* VALIDATE: destination indices not sorted ascending */
#define SEGPOLY_E_HIP (-5)         /* a HIP runtime call or kernel launch failed */
#define SEGPOLY_E_OOM (-6)         /* host or device allocation failed */
#define SEGPOLY_E_RANGE (-7)       /* VALIDATE: an index outside its range */

/* layouts, dtypes, index dtypes */
#define SEGPOLY_MUL_IR 0
#define SEGPOLY_IR_MUL 1
#define SEGPOLY_F32 0
#define SEGPOLY_F64 1
#define SEGPOLY_I32 0
#define SEGPOLY_I64 1

/* flags */
#define SEGPOLY_SHARED_WEIGHTS 1u /* weights are one row [1, numel] shared by every edge */
#define SEGPOLY_VALIDATE 2u       /* check index ranges and dst order on the host (synchronises) */
#define SEGPOLY_FORCE_GENERIC 4u  /* use the table-driven kernel even if a specialised one exists */
#define SEGPOLY_REDUCE_MEAN 8u    /* convolution: each output row is the mean over its edges, not the sum
                                     (rows without edges stay zero); the convolution layer's reduce="mean"
                                     of the "cuequivariance-torch" skill document, "Other operations and
                                     layers".  The backward takes the same flag from the handle. */
#define SEGPOLY_MERGE_PATHS 16u   /* tp_create: the paths of one output type sum into a single block of that
                                     type (e3nn-style instructions writing one irrep; a reading, the pages
                                     print no merged example); output blocks in type order, all paths of a
                                     type must have the same multiplicity (E_UNSUPPORTED otherwise); weights
                                     and path order unchanged.  tp_irreps_out reports the merged irreps. */

/* query keys */
#define SEGPOLY_Q_DIM_IN1 0
#define SEGPOLY_Q_DIM_IN2 1
#define SEGPOLY_Q_DIM_OUT 2
#define SEGPOLY_Q_WEIGHT_NUMEL 3
#define SEGPOLY_Q_NUM_PATHS 4
#define SEGPOLY_Q_CG_NNZ 5
#define SEGPOLY_Q_SPECIALIZED 6 /* 1 if a generated kernel serves this handle, 0 for the generic one */
#define SEGPOLY_Q_MUL 7         /* the uniform multiplicity, 0 if multiplicities differ */
#define SEGPOLY_Q_DIM_IN 8      /* symcon: input width */
#define SEGPOLY_Q_NUM_COUPLINGS 9
#define SEGPOLY_Q_NUM_TERMS 10  /* symcon: sorted-monomial terms per channel */
#define SEGPOLY_Q_NUM_ELEMENTS 11
#define SEGPOLY_Q_NUM_MONOMIALS 12 /* symcon: monomial products per channel (pairs and triples) */

typedef struct segpoly_tp* tp_handle;
typedef struct segpoly_symcon* symcon_handle;
typedef struct segpoly_linear* linear_handle;
typedef struct segpoly_fctp* fctp_handle;

/* ------------------------------------------------------------------ TP */

/*
 * tp_create: build the descriptor of a channelwise tensor product.
 *   irreps_in1  features of the source nodes, e.g. "128x0e+128x1o+128x2e".
 *   irreps_in2  per-edge operand (spherical harmonics), every block of
 *               multiplicity 1, e.g. "0e+1o+2e+3o".
 *   irreps_out  the irrep TYPES to keep (multiplicities are ignored): every
 *               path (in1 block, in2 block, lo) with |l1-l2| <= lo <= l1+l2 and
 *               parity p1*p2 whose type is listed gets its own output block
 *               of multiplicity mul(in1 block).  The actual output irreps are
 *               read back with tp_irreps_out (skill document, "Layouts and
 *               weights": the filter selects types, not multiplicities).
 *   layout      SEGPOLY_MUL_IR or SEGPOLY_IR_MUL, for x and out (sh has
 *               multiplicity 1, so both layouts coincide for it).
 *   dtype       SEGPOLY_F32 or SEGPOLY_F64: data and arithmetic type.
 *   flags       SEGPOLY_SHARED_WEIGHTS, SEGPOLY_VALIDATE, SEGPOLY_FORCE_GENERIC.
 * Path order: in1 block, in2 block, lo ascending, then a stable sort by
 * output type (l, natural parity (-1)^l first); the weight row holds one
 * segment of mul channels per path in that order.  Coefficients: real-basis
 * Clebsch-Gordan tensors scaled so that sum_ij C_ijk C_ijk' = delta_kk'.
 * Errors: E_PARSE (string), E_UNSUPPORTED (in2 multiplicity != 1, or a
 * block with l > 6 in any of the three strings, so no path reaches l > 6),
 * E_INVALID (null out, bad enum).  Touches no GPU.
 */
int tp_create(const char* irreps_in1, const char* irreps_in2, const char* irreps_out, int layout,
              int dtype, unsigned flags, tp_handle* out);

/* tp_query: one of the SEGPOLY_Q_* sizes of the descriptor into *value. */
int tp_query(tp_handle h, int key, int64_t* value);

/* tp_irreps_out: the actual output irreps ("32x0e+32x0e+32x1o+...") into
 * buf (NUL-terminated); E_INVALID if cap is too small. */
int tp_irreps_out(tp_handle h, char* buf, size_t cap);

/* tp_path_info: path p (0 <= p < NUM_PATHS) as 10 integers: in1 block,
 * in2 block, l1, l2, lo, parity, mul, output element offset, weight offset,
 * number of non-zero coefficients. */
int tp_path_info(tp_handle h, int p, int64_t* info10);

/* tp_path_cg: the dense coefficient tensor of path p, row-major
 * [2l1+1][2l2+1][2lo+1], as doubles. */
int tp_path_cg(tp_handle h, int p, double* out);

/* tp_kernel_name: name of the kernel that serves this handle. */
int tp_kernel_name(tp_handle h, char* buf, size_t cap);

/*
 * tp_conv_fwd: out[n] = sum over edges e with dst[e] == n of the product
 * of x[src[e]], sh[e] and w[e] through every path; rows with no edge are
 * written as zeros.  `out` is fully overwritten.  The product is the
 * channelwise descriptor of e3nn-course Lesson 12a, section 21.4 (one fused
 * kernel over every path, sections 21.1 and 21.6); the gather by source and
 * the sum into destinations (repeated receivers add, receivers without edges
 * stay zero, the destination count given explicitly) are those of the
 * cuequivariance-torch skill document, "SegmentedPolynomial: gather and
 * scatter".
 *   x       [n_src, DIM_IN1] device, layout of the handle.
 *   sh      [n_edges, DIM_IN2] device.
 *   w       [n_edges, WEIGHT_NUMEL] device, or [1, WEIGHT_NUMEL] with
 *           SEGPOLY_SHARED_WEIGHTS.
 *   src,dst [n_edges] device, int32 or int64 per idx_dtype.  dst must be
 *           sorted ascending (precondition; checked only with VALIDATE).
 *           Sources outside [0, n_src) and destinations outside
 *           [0, n_nodes) contribute nothing (VALIDATE reports them as
 *           E_RANGE).  Both NULL with n_edges > 0 selects batch mode: edge e
 *           feeds row e, and n_edges must equal n_nodes and not exceed
 *           n_src.  With n_edges == 0 every row is zero, whatever the index
 *           pointers.
 *   out     [n_nodes, DIM_OUT] device, layout of the handle.
 * A descriptor served by the generic kernel uploads its coefficient table
 * to the current device once (hipMalloc + hipMemcpy at the first call on
 * that device; freed by tp_destroy).  Sizes: n_nodes < 2^31.
 */
int tp_conv_fwd(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w,
                const void* src, const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes,
                void* out, void* stream);

/*
 * tp_rowptr_build: row pointers of a destination-sorted edge list (the
 * compressed-sparse-row form of the destination ranges; the sorted
 * destinations it is built from are those of tp_conv_fwd, after the
 * cuequivariance-torch skill document, "SegmentedPolynomial: gather and
 * scatter"):
 *   row_ptr[n] = first e with dst[e] >= n, for n = 0 .. n_nodes
 * (row_ptr[n_nodes] = n_edges when every dst is below n_nodes).
 *   dst      [n_edges] device, sorted ascending, int32 or int64 per idx_dtype.
 *   row_ptr  [n_nodes + 1] device, same index dtype, fully overwritten.
 * One launch; build it once per graph and pass it to every
 * tp_conv_fwd_rowptr call on that graph (it replaces the per-destination
 * range search of tp_conv_fwd).  E_UNSUPPORTED for int32 with n_edges or
 * n_nodes at 2^31 or more.
 */
int tp_rowptr_build(const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* row_ptr,
                    void* stream);

/*
 * tp_conv_fwd_rowptr: tp_conv_fwd with the destination ranges given as row
 * pointers instead of dst: destination n sums the edges
 * [row_ptr[n], row_ptr[n + 1]) (values clamped to [0, n_edges], so
 * inconsistent pointers cannot read outside the edge arrays; VALIDATE
 * checks row_ptr[0] = 0, non-decreasing entries and row_ptr[n_nodes] =
 * n_edges, E_RANGE / E_UNSORTED otherwise).  src and row_ptr are required
 * (no batch mode); the result equals tp_conv_fwd's on the dst the pointers
 * were built from, bit for bit.  Other arguments as tp_conv_fwd.
 */
int tp_conv_fwd_rowptr(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w,
                       const void* src, const void* row_ptr, int idx_dtype, int64_t n_edges, int64_t n_nodes,
                       void* out, void* stream);

/*
 * tp_src_rowptr_build: row pointers of the sources in src_perm order (the
 * gathered input's gradient sums over the edges that read it, after the
 * cuequivariance-torch skill document, "SegmentedPolynomial: gather and
 * scatter"; tp_conv_bwd visits each source's edges in this order):
 *   src_row_ptr[s] = first i with src[src_perm[i]] >= s, for s = 0 .. n_src
 * (an entry of src_perm outside [0, n_edges) counts as past every source).
 *   src, src_perm  [n_edges] device, as tp_conv_bwd (src_perm a stable
 *                  argsort of src).
 *   src_row_ptr    [n_src + 1] device, same index dtype, fully overwritten.
 * One launch; build it once per graph for tp_conv_bwd_rowptr.  Errors as
 * tp_rowptr_build (with n_src in the place of n_nodes).
 */
int tp_src_rowptr_build(const void* src, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_src,
                        void* src_row_ptr, void* stream);

/*
 * tp_conv_bwd_workspace: bytes of device workspace tp_conv_bwd needs for
 * n_edges edges, in indexed mode (batch == 0) or batch mode (batch != 0):
 * one source message per edge (n_edges * DIM_IN1 elements of the handle's
 * dtype, indexed mode only), rounded up to 256 bytes, plus, when the
 * multiplicity exceeds 64, ceil(mul / 64) * n_edges * DIM_IN2 elements of
 * per-tile harmonic-gradient partials; in indexed mode then, 256-byte
 * aligned, n_edges int32 (the sources in src_perm order); with
 * SEGPOLY_SHARED_WEIGHTS then, each part 256-byte aligned, n_edges *
 * WEIGHT_NUMEL per-edge weight gradients and ceil(n_edges / 1024) *
 * WEIGHT_NUMEL partial sums of them.  0 means no workspace is needed.
 */
int tp_conv_bwd_workspace(tp_handle h, int64_t n_edges, int batch, size_t* bytes);

/*
 * tp_conv_bwd: vector-Jacobian product of tp_conv_fwd, the gradients of
 * every operand that the pages' examples check ("cuequivariance-torch"
 * skill document, "CPU tensor product and backward" and "SegmentedPolynomial:
 * gather and scatter": gradients of features, vectors and weights; the
 * gradient of a gathered input sums over the edges that read it).  With
 * g = dL/d(out):
 *   grad_w[e]  = g[dst[e]] contracted with the path products of
 *                x[src[e]] and sh[e];
 *   grad_sh[e] = sum over paths and channels of w[e] x[src[e]] g[dst[e]]
 *                contracted with the coupling;
 *   grad_x[s]  = sum over edges e with src[e] == s of w[e] sh[e] g[dst[e]]
 *                contracted with the coupling (zero for a source without
 *                edges).
 * Every element of grad_x, grad_sh and grad_w is overwritten.  Edges whose
 * source or destination lies outside its range get zero gradients and add
 * nothing to grad_x (for an out-of-range source: given finite sh and
 * grad_out, since its x and w enter as zeros).
 *   x, sh, w, src, dst, idx_dtype, n_src, n_edges, n_nodes: as tp_conv_fwd.
 *   src_perm   [n_edges] device, idx_dtype: the edge ids ordered by src
 *              ascending (a stable argsort of src: the order within one
 *              source is the order in which its messages are summed, so a
 *              fixed perm gives bitwise-reproducible grad_x).  A permutation
 *              is a precondition, checked only with VALIDATE (E_RANGE).  NULL
 *              in batch mode.
 *   grad_out   [n_nodes, DIM_OUT] device, layout of the handle.
 *   grad_x     [n_src, DIM_IN1] device.  grad_sh [n_edges, DIM_IN2] device.
 *   grad_w     [n_edges, WEIGHT_NUMEL] device; with SEGPOLY_SHARED_WEIGHTS
 *              [1, WEIGHT_NUMEL], the sum over the edges of their
 *              per-edge gradients (written to the workspace, summed in
 *              fixed chunks of 1024 edges, then the chunks in order).
 *   workspace  device, at least tp_conv_bwd_workspace() bytes, 256-byte
 *              aligned (E_INVALID otherwise); may be NULL when that size
 *              is 0.  Its contents on entry do not matter.
 * Two to four launches on `stream`, no atomics: results are deterministic
 * (bitwise, for fixed inputs and src_perm); two more with shared weights.
 * Fails closed with E_UNSUPPORTED for a descriptor without a specialised
 * kernel.  Sizes: n_nodes, n_src < 2^31.
 */
int tp_conv_bwd(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_nodes,
                const void* grad_out, void* grad_x, void* grad_sh, void* grad_w, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * tp_conv_bwd_rowptr: tp_conv_bwd with both edge ranges given as row
 * pointers: destination n's edges are [row_ptr[n], row_ptr[n + 1])
 * (tp_rowptr_build) and source s's are src_perm[src_row_ptr[s] ..
 * src_row_ptr[s + 1]) (tp_src_rowptr_build), both clamped to
 * [0, n_edges], so inconsistent pointers cannot read outside the edge
 * arrays.  No range search runs and the sorted-source keys are not built
 * (two launches fewer for a reused graph).  src, dst (still read by the
 * table-driven kernels), src_perm and both pointer arrays are required (no
 * batch mode).  With VALIDATE, besides tp_conv_bwd's checks, each pointer
 * array must equal the one its builder gives (E_RANGE otherwise).  The
 * results equal tp_conv_bwd's bit for bit; other arguments, the workspace
 * (same size) and the errors as tp_conv_bwd.
 *   row_ptr      [n_nodes + 1] device, idx_dtype.
 *   src_row_ptr  [n_src + 1] device, idx_dtype.
 */
int tp_conv_bwd_rowptr(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                       const void* dst, const void* src_perm, const void* row_ptr, const void* src_row_ptr,
                       int idx_dtype, int64_t n_edges, int64_t n_nodes, const void* grad_out, void* grad_x,
                       void* grad_sh, void* grad_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_conv_fwd_vec: tp_conv_fwd with the second operand computed in the
 * kernel from the edge vectors, as the harmonics of sh_fwd (the convolution
 * of the pages' message passing takes sh(edge_vectors): "cuequivariance-
 * torch" skill document, "Trainable message passing").  Input 2 of the
 * handle must be 0e + 1o + 2e + ... + L (one copy each, L <= 6) and the
 * descriptor specialised (E_UNSUPPORTED otherwise).
 *   vec        [n_edges, 3] device, the handle's dtype.
 *   normalize  != 0: harmonics of vec / |vec| (a zero vector gives Y_0 = 1,
 *              zeros); 0: the homogeneous polynomials.
 * Other arguments and results as tp_conv_fwd (batch mode included).
 */
int tp_conv_fwd_vec(tp_handle h, const void* x, int64_t n_src, const void* vec, int normalize, const void* w,
                    const void* src, const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out,
                    void* stream);

/* tp_destroy: free the handle (NULL is a no-op). */
int tp_destroy(tp_handle h);

/* ------------------------------------------------------------------ symcon */

/*
 * symcon_create: symmetric contraction of degrees 1..max_degree (1..3):
 * the MACE-style polynomial of e3nn-course Lesson 12a, section 21.4.1 (its
 * degree-1..3 descriptors evaluated in one launch), with the element-indexed
 * weights of the cuequivariance-torch skill document, "Other operations and
 * layers" (SymmetricContraction: uniform multiplicities, one weight row per
 * element).
 *   irreps_in, irreps_out  every block with the same multiplicity.
 *   num_elements           number of species (rows of the weight table).
 * Coupling basis per (degree nu, output block): candidates are the
 * real-coupling tensors of ordered block tuples in lexicographic order (and,
 * for nu = 3, the intermediate l ascending), symmetrised over the nu input
 * slots; a candidate is kept when its Gram-Schmidt residual against those
 * kept before exceeds 1e-8 of its norm; each kept tensor is scaled so that
 * its output components are orthonormal.  Weight segments: degree, then
 * output block, then coupling, each mul channels.
 * Errors: E_PARSE, E_UNSUPPORTED (non-uniform multiplicities, l > 6, degree
 * outside 1..3), E_INVALID.  Touches no GPU.
 */
int symcon_create(const char* irreps_in, const char* irreps_out, int max_degree, int num_elements,
                  int layout, int dtype, unsigned flags, symcon_handle* out);

/* symcon_query: DIM_IN, DIM_OUT, WEIGHT_NUMEL (per element), NUM_COUPLINGS,
 * NUM_TERMS, SPECIALIZED, MUL, NUM_ELEMENTS, NUM_MONOMIALS. */
int symcon_query(symcon_handle h, int key, int64_t* value);

/* symcon_coupling_info: coupling c (weight-segment order) as 4 integers:
 * degree, output block, index k within (degree, block), output l. */
int symcon_coupling_info(symcon_handle h, int c, int64_t* info4);

/* symcon_coupling_dense: coupling c as a dense row-major tensor
 * [n]^degree x [2L+1] (n = input components per channel), doubles. */
int symcon_coupling_dense(symcon_handle h, int c, double* out);

/*
 * symcon_fwd: out[a] = sum over degrees and couplings of
 * w[species[a], segment] * coupling(x[a], ..., x[a]) per channel (Lesson
 * 12a, section 21.4.1; the call sc(x, element_indices) of the skill
 * document, "Other operations and layers").
 *   x        [n_atoms, DIM_IN] device, layout of the handle.
 *   species  [n_atoms] device, int32 or int64 per idx_dtype; an element
 *            outside [0, num_elements) gives a zero row (E_RANGE with
 *            VALIDATE).  Need not be sorted.
 *   w        [num_elements, WEIGHT_NUMEL] device.
 *   out      [n_atoms, DIM_OUT] device, fully overwritten.
 * Generic-kernel tables are uploaded once per device as for tp_conv_fwd.
 */
int symcon_fwd(symcon_handle h, const void* x, const void* species, int idx_dtype, const void* w,
               int64_t n_atoms, void* out, void* stream);

/*
 * symcon_bwd_workspace: bytes of device workspace symcon_bwd needs for
 * n_atoms atoms: a segment table of 2 * (num_elements + 3) int64 values
 * (rounded up to 256 bytes), then per-chunk weight-gradient partials of
 * (ceil(n_atoms / 16) + num_elements + 2) * WEIGHT_NUMEL elements of the
 * handle's dtype.
 */
int symcon_bwd_workspace(symcon_handle h, int64_t n_atoms, size_t* bytes);

/*
 * symcon_bwd: vector-Jacobian product of symcon_fwd (the pages check the
 * gradients of every input: "cuequivariance-torch" skill document, "CPU
 * tensor product and backward"; the polynomial of e3nn-course Lesson 12a,
 * section 21.4.1).  With g = dL/d(out):
 *   grad_x[a] = per channel, the derivative of the degree-1..3 polynomial
 *               of x[a] (product rule) contracted with w[species[a]] and g[a];
 *   grad_w[e] = sum over the atoms a of element e of g[a] contracted with
 *               the polynomial of x[a] (zero for an element without atoms).
 *   x, species, idx_dtype, w, n_atoms: as symcon_fwd.
 *   species_perm [n_atoms] device, idx_dtype: the atom ids ordered by
 *               element ascending (a stable argsort of species); the order
 *               within an element is the order in which grad_w sums them, so
 *               a fixed perm gives bitwise-reproducible grad_w.  Atoms whose
 *               element is out of range get grad_x = 0 and add nothing.
 *               A permutation sorted by element is a precondition, checked
 *               only with VALIDATE (E_RANGE / E_UNSORTED).
 *   grad_out    [n_atoms, DIM_OUT] device, layout of the handle.
 *   grad_x      [n_atoms, DIM_IN] device, fully overwritten.
 *   grad_w      [num_elements, WEIGHT_NUMEL] device, fully overwritten.
 *   workspace   device, at least symcon_bwd_workspace() bytes, 256-byte
 *               aligned (E_INVALID otherwise); its contents on entry do not
 *               matter.
 * Three launches on `stream`, no atomics.  Fails closed with E_UNSUPPORTED
 * for a descriptor without a specialised kernel.  Sizes: n_atoms < 2^31.
 */
int symcon_bwd(symcon_handle h, const void* x, const void* species, const void* species_perm, int idx_dtype,
               const void* w, const void* grad_out, int64_t n_atoms, void* grad_x, void* grad_w, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * symcon_bwd_noalloc: symcon_bwd for callers that cannot allocate device
 * memory on the compute path (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, kernels and
 * results as symcon_bwd, without the workspace: it uses a fixed device array
 * of SEGPOLY_NOALLOC_SCRATCH_BYTES inside this library instead (one copy per
 * device, held from the library's first use on that device until the
 * process ends).  The call itself allocates nothing, device or host.
 *   Errors: E_UNSUPPORTED when symcon_bwd_workspace(h, n_atoms) exceeds
 *   SEGPOLY_NOALLOC_SCRATCH_BYTES (checked before any launch; 128 MiB holds
 *   50,000 atoms of 128 channels with 3,712 weights per element) or when the
 *   handle has SEGPOLY_VALIDATE (its index check copies into host buffers);
 *   otherwise as symcon_bwd.
 * Every call on one device shares that device's array and leaves its own
 * contents there (nothing in it needs to start at zero): calls that overlap
 * on one device (different streams, or threads without ordering) race and
 * must not be issued; calls ordered on one stream are safe.
 */
#define SEGPOLY_NOALLOC_SCRATCH_BYTES (128ull * 1024ull * 1024ull)
int symcon_bwd_noalloc(symcon_handle h, const void* x, const void* species, const void* species_perm, int idx_dtype,
                       const void* w, const void* grad_out, int64_t n_atoms, void* grad_x, void* grad_w,
                       void* stream);

int symcon_destroy(symcon_handle h);

/* ------------------------------------------------------------------ misc */

/* ------------------------------------------------------------------ linear */

/*
 * linear_create: the equivariant linear layer irreps_in -> irreps_out
 * ("cuequivariance-torch" skill document, "Linear: layout conversion and
 * rotations"; "Other operations and layers" for class-indexed weights).
 * Blocks of equal irrep type mix channel by channel with one matrix per
 * (input block, output block) pair, the same for every component m:
 *   out[n, o, m, v] = alpha_t sum over input blocks i of type t of
 *                     sum_u W_io[u, v] x[n, i, m, u],
 * alpha_t = 1 / sqrt(sum of the multiplicities of the input blocks of type
 * t); an output block whose type no input has is zero.  Weight segments:
 * pairs in the order i, then o, each mul_i x mul_o with v fastest
 * (WEIGHT_NUMEL in total).  flags: SEGPOLY_VALIDATE only.  E_UNSUPPORTED
 * beyond 32 blocks on a side or 32 pairs, DIM_IN or DIM_OUT above 65536 or
 * WEIGHT_NUMEL above 2^27.  Touches no GPU.
 */
int linear_create(const char* irreps_in, const char* irreps_out, int layout, int dtype, unsigned flags,
                  linear_handle* out);

/* linear_query: SEGPOLY_Q_DIM_IN, SEGPOLY_Q_DIM_OUT, SEGPOLY_Q_WEIGHT_NUMEL,
 * SEGPOLY_Q_NUM_PATHS (the number of weight segments). */
int linear_query(linear_handle h, int key, int64_t* value);

/*
 * linear_fwd: out = linear(x) for n samples, on the matrix cores.
 *   x        [n, DIM_IN] device, layout of the handle.
 *   w        [1, WEIGHT_NUMEL] device (shared), or with `classes`
 *            [num_classes, WEIGHT_NUMEL]: sample n uses row classes[n].
 *   classes  NULL, or [n] device, int32 or int64 per idx_dtype; a class
 *            outside [0, num_classes) gives a zero row (E_RANGE with
 *            VALIDATE).  Sorted classes run fastest (a tile of rows of one
 *            class costs one pass); any order is correct.
 *   out      [n, DIM_OUT] device, fully overwritten.
 */
int linear_fwd(linear_handle h, const void* x, const void* w, const void* classes, int idx_dtype, int num_classes,
               int64_t n, void* out, void* stream);

/* linear_bwd_workspace: bytes of workspace linear_bwd needs for the weight
 * gradient of n samples: per-chunk partial sums, for each of num_classes
 * weight rows with class-indexed weights (then also two int32 per row
 * chunk: the classes it holds); num_classes = 0 for shared weights. */
int linear_bwd_workspace(linear_handle h, int64_t n, int num_classes, size_t* bytes);

/*
 * linear_bwd: vector-Jacobian product of linear_fwd for g = dL/d(out):
 *   grad_x[n, i, m, u] = alpha_t sum over pairs (i, o) of sum_v W_io[u, v] g[n, o, m, v]
 *   grad_w[W_io][u, v] = alpha_t sum over samples n and components m of x[n, i, m, u] g[n, o, m, v]
 * grad_x [n, DIM_IN] is fully overwritten.  grad_w [1, WEIGHT_NUMEL], or
 * [num_classes, WEIGHT_NUMEL] with `classes` (row c sums over the samples
 * of class c; samples of a class outside [0, num_classes) add nothing),
 * fully overwritten, may be NULL (not computed; x and the workspace are
 * then not used).  The weight gradient sums fixed chunks of 2048 rows and
 * then the chunks in order: deterministic.  With classes each chunk makes
 * one pass per class between its lowest and highest class (sorted classes:
 * one or two passes; at most 65535 classes, E_UNSUPPORTED beyond).  The
 * workspace holds linear_bwd_workspace(n, classes ? num_classes : 0)
 * bytes.  Other arguments as linear_fwd.
 */
int linear_bwd(linear_handle h, const void* x, const void* w, const void* grad_out, const void* classes,
               int idx_dtype, int num_classes, int64_t n, void* grad_x, void* grad_w, void* workspace,
               size_t workspace_bytes, void* stream);

/* linear_destroy: free the handle (NULL is a no-op). */
int linear_destroy(linear_handle h);

/* ------------------------------------------------- fully connected product */

/*
 * fctp_create: the fully connected ("uvw") tensor product
 * irreps_in1 x irreps_in2 -> irreps_out ("cuequivariance-torch" skill
 * document, "CPU tensor product and backward" and "Channelwise product with
 * external per-example weights"; e3nn-course Lesson 12a, exercise 1: the
 * weights carry three channel indices).  Paths: every (input-1 block i,
 * input-2 block j, output block o) with |l1 - l2| <= l3 <= l1 + l2 and
 * p3 = p1 p2, in the order i, then j, then o; the output irreps are taken
 * as given.  Terms without a parity letter ("0 + 1") are SO(3) irreps: no
 * parity rule (all three strings must then be SO(3)).
 *   out[n, o, k, w] = alpha_o sum over paths (i, j, o) of
 *                     sum_(u, v) W_p[u, v, w] sum_(a, b) C[a, b, k] x1[n, i, a, u] x2[n, j, b, v]
 * with the coupling of tp_create (segpoly_real_cg) and
 * alpha_o = 1 / sqrt(sum over the paths into o of mul1 mul2) (0 for an
 * output block no path reaches: its rows are zero).  Weights: one segment
 * per path of mul1 * mul2 * mul3 values, (u, v, w) row-major, shared by all
 * samples ([1, WEIGHT_NUMEL]).  flags: SEGPOLY_VALIDATE (index checks of
 * fctp_conv_fwd), SEGPOLY_REDUCE_MEAN (fctp_conv_fwd averages instead of
 * summing).  E_UNSUPPORTED for l > 6, more than 32 blocks on a side, more
 * than 64 paths, blocks too wide for one workgroup's LDS, or a path whose
 * coupling has more than 16 non-zero entries along one index of any of its
 * three axes (within l <= 6 only couplings with two of l1, l2, l3 at 5 or 6,
 * e.g. 5 x 1 -> 5 with 18).  Touches no GPU.
 */
int fctp_create(const char* irreps_in1, const char* irreps_in2, const char* irreps_out, int layout, int dtype,
                unsigned flags, fctp_handle* out);

/* fctp_query: SEGPOLY_Q_DIM_IN1, SEGPOLY_Q_DIM_IN2, SEGPOLY_Q_DIM_OUT,
 * SEGPOLY_Q_WEIGHT_NUMEL, SEGPOLY_Q_NUM_PATHS. */
int fctp_query(fctp_handle h, int key, int64_t* value);

/* fctp_path_info: path p as {i, j, o, weight offset}. */
int fctp_path_info(fctp_handle h, int p, int64_t* info4);

/*
 * fctp_fwd: out = fctp(x1, x2; w) for n samples, on the matrix cores.
 *   x1 [n, DIM_IN1], x2 [n, DIM_IN2] device, layout of the handle.
 *   w  [1, WEIGHT_NUMEL] device.
 *   out [n, DIM_OUT] device, fully overwritten.  n == 0 does nothing.
 */
int fctp_fwd(fctp_handle h, const void* x1, const void* x2, const void* w, int64_t n, void* out, void* stream);

/* fctp_bwd_workspace: bytes of workspace fctp_bwd needs for n samples:
 * the weight gradient's per-chunk partial sums and two transposed copies of
 * the weights that the input gradients read (0 for n = 0). */
int fctp_bwd_workspace(fctp_handle h, int64_t n, size_t* bytes);

/*
 * fctp_bwd: vector-Jacobian product of fctp_fwd for g = dL/d(out):
 *   grad_x1 [n, DIM_IN1], grad_x2 [n, DIM_IN2], grad_w [1, WEIGHT_NUMEL],
 * each fully overwritten, or NULL (not computed).  Any requested gradient
 * needs `workspace` of fctp_bwd_workspace(n) bytes (overwritten); grad_w
 * sums fixed chunks of 1024 samples and then the chunks in order
 * (deterministic).  Inputs a requested
 * gradient does not read may be NULL (grad_x1 reads x2, g, w; grad_x2 reads
 * x1, g, w; grad_w reads x1, x2, g).
 */
int fctp_bwd(fctp_handle h, const void* x1, const void* x2, const void* w, const void* grad_out, int64_t n,
             void* grad_x1, void* grad_x2, void* grad_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fctp_fwd_per_sample: the product with one weight row per sample (external
 * per-item weights: "cuequivariance-torch" skill document, "Layouts and
 * weights", shared_weights=False with a [batch, weight_numel] operand):
 *   out[s] = fctp(x1[s], x2[s]; w[s]) for s < n.
 *   x1 [n, DIM_IN1], x2 [n, DIM_IN2], w [n, WEIGHT_NUMEL], out [n, DIM_OUT]:
 *   device, row-major, layout and dtype of the handle; out fully overwritten.
 * Each weight row is read once (the product streams the weights).  No
 * workspace.  E_UNSUPPORTED when one sample's staged rows (x1, x2 and 64
 * coupled values per output component) exceed 64 KB of LDS, when a weight
 * row is 2 GiB or more, or n exceeds one launch's grid.
 */
int fctp_fwd_per_sample(fctp_handle h, const void* x1, const void* x2, const void* w, int64_t n, void* out,
                        void* stream);

/*
 * fctp_bwd_per_sample: vector-Jacobian product of fctp_fwd_per_sample for
 * g = dL/d(out) [n, DIM_OUT]:
 *   grad_x1 [n, DIM_IN1], grad_x2 [n, DIM_IN2], grad_w [n, WEIGHT_NUMEL]
 * (one gradient row per sample, no sum over the samples), each fully
 * overwritten, or NULL (not computed).  Every sum is taken in a fixed order
 * (deterministic).  No workspace.  Inputs a requested gradient does not
 * read may be NULL (grad_x1 reads x2, g, w; grad_x2 reads x1, g, w; grad_w
 * reads x1, x2, g).  E_UNSUPPORTED as fctp_fwd_per_sample, the LDS holding
 * also the two input-gradient rows and 64 weight-contracted values per
 * output component.
 */
int fctp_bwd_per_sample(fctp_handle h, const void* x1, const void* x2, const void* w, const void* grad_out,
                        int64_t n, void* grad_x1, void* grad_x2, void* grad_w, void* stream);

/*
 * fctp_conv_fwd: the product as a graph convolution with per-edge weights
 * ("cuequivariance-torch" skill document, "Other operations and layers":
 * FullyConnectedTensorProductConv, whose edge MLP gives one weight row per
 * edge; the MLP itself is the caller's):
 *   out[n] = s_n sum over edges e with dst[e] = n of fctp(x[src[e]], sh[e]; w[e]),
 * s_n = 1, or 1 / (number of edges into n) with SEGPOLY_REDUCE_MEAN; rows
 * without edges are zero.
 *   x    [n_src, DIM_IN1] device, layout of the handle.
 *   sh   [n_edges, DIM_IN2] device: input 2 must have one channel per block
 *        (the edge harmonics; E_UNSUPPORTED otherwise), so its layout is moot.
 *   w    [w_rows, WEIGHT_NUMEL] device, w_rows = n_edges (per edge) or 1
 *        (shared by every edge).
 *   src, dst [n_edges] device, int32 or int64 per idx_dtype; dst sorted
 *        ascending (the precondition of tp_conv_fwd; VALIDATE checks it and
 *        the ranges); an edge whose source is out of range contributes
 *        nothing.
 *   out  [n_nodes, DIM_OUT] device, fully overwritten.
 * Input-1 blocks of more than 64 channels are taken 64 channels at a time;
 * E_UNSUPPORTED when one edge's staged rows (x components times channels,
 * the harmonics, the coupled rows) exceed the 64 KB of LDS of one wave.
 */
int fctp_conv_fwd(fctp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, int64_t w_rows,
                  const void* src, const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out,
                  void* stream);

/* fctp_conv_bwd_workspace: bytes of workspace fctp_conv_bwd needs for
 * n_edges edges and w_rows weight rows (n_edges, or 1 shared): the
 * per-edge source messages [n_edges, DIM_IN1], rounded up to 256 bytes;
 * with a shared row (and n_edges != 1) then the per-edge weight gradients
 * [n_edges, WEIGHT_NUMEL], rounded up to 256 bytes, and
 * ceil(n_edges / 1024) * WEIGHT_NUMEL partial sums.  Elements of the
 * handle's dtype. */
int fctp_conv_bwd_workspace(fctp_handle h, int64_t n_edges, int64_t w_rows, size_t* bytes);

/*
 * fctp_conv_bwd: vector-Jacobian product of fctp_conv_fwd with one weight
 * row per edge (w_rows == n_edges) or one row shared by every edge
 * (w_rows == 1), for grad_out = dL/d(out) [n_nodes, DIM_OUT] device
 * (divided by each row's edge count with SEGPOLY_REDUCE_MEAN, as the
 * forward):
 *   grad_w  [w_rows, WEIGHT_NUMEL]: per edge, dW_e[p][u, w] = sum_k y[p, k, u] G[o, k, w];
 *           a shared row gets the sum over the edges (per-edge rows in the
 *           workspace, summed in chunks of 1024 edges, then in order)
 *   grad_sh [n_edges, DIM_IN2]:      per edge
 *   grad_x  [n_src, DIM_IN1]:        summed over the edges that read each source,
 * all fully overwritten (zero for sources no edge reads and for edges whose
 * destination lies outside [0, n_nodes)).  src_perm [n_edges] (same index
 * dtype) lists the edges ordered by source (a stable argsort of src:
 * structure of the batch, like the sorted dst); VALIDATE checks it and the
 * indices.  The source sums run in src_perm order: deterministic.
 * `workspace` holds fctp_conv_bwd_workspace(n_edges, w_rows) bytes.  Other
 * arguments as fctp_conv_fwd.
 */
int fctp_conv_bwd(fctp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, int64_t w_rows,
                  const void* src, const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges,
                  int64_t n_nodes, const void* grad_out, void* grad_x, void* grad_sh, void* grad_w, void* workspace,
                  size_t workspace_bytes, void* stream);

/* fctp_destroy: free the handle (NULL is a no-op). */
int fctp_destroy(fctp_handle h);

/* ---------------------------------------------------- edge embedding assembly */

/*
 * edge_scalars_fwd: the edge MLP input of the convolution layer with its
 * optional per-node scalars ("cuequivariance-torch" skill document, "Other
 * operations and layers": FullyConnectedTensorProductConv's src_scalars and
 * dst_scalars go with the edge embedding into the edge MLP):
 *   out[e] = [edge_emb[e], src_scalars[src[e]], dst_scalars[dst[e]]]
 *   edge_emb [n_edges, d_emb], src_scalars [n_src, d_src], dst_scalars
 *   [n_dst, d_dst], out [n_edges, d_emb + d_src + d_dst], device, dtype per
 *   `dtype`; d_src = 0 or d_dst = 0 leaves that part out (its pointers may
 *   then be NULL).  src, dst [n_edges] int32/int64.  An index out of range
 *   gives a zero slice.  out is fully overwritten.
 */
int edge_scalars_fwd(int dtype, const void* edge_emb, int64_t d_emb, const void* src_scalars, int64_t d_src,
                     const void* dst_scalars, int64_t d_dst, const void* src, const void* dst, int idx_dtype,
                     int64_t n_edges, int64_t n_src, int64_t n_dst, void* out, void* stream);

/*
 * edge_scalars_bwd: its vector-Jacobian product for grad_out [n_edges,
 * d_emb + d_src + d_dst]: grad_emb [n_edges, d_emb] (the slice), grad_src
 * [n_src, d_src] (sum over the edges reading each source, in src_perm order:
 * a stable argsort of src), grad_dst [n_dst, d_dst] (sum over each
 * destination's edges: dst sorted ascending, the convolution's
 * precondition).  Fully overwritten (zero rows for unread sources and
 * destinations without edges); deterministic.
 */
int edge_scalars_bwd(int dtype, const void* grad_out, int64_t d_emb, int64_t d_src, int64_t d_dst, const void* src,
                     const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_src,
                     int64_t n_dst, void* grad_emb, void* grad_src, void* grad_dst, void* stream);


/* ------------------------------------------------------- spherical harmonics */

/*
 * sh_fwd: real spherical harmonics of n vectors, degrees 0..lmax
 * concatenated (the operand "0e + 1o + 2e + ..." of the convolution),
 * "component" normalisation (sum over m of Y_lm^2 = 2l + 1 on the unit
 * sphere); "cuequivariance-torch" skill document, "Spherical harmonics and a
 * NumPy reference".  normalize != 0 evaluates on v / |v| (a zero vector
 * gives Y_0 = 1 and zeros), normalize == 0 the homogeneous polynomial
 * |v|^l Y_l(v / |v|).  Textbook real basis, index l^2 + l + m, m = -l..l,
 * l = 1 is sqrt(3) (y, z, x).
 *   vec  [n, 3] device, dtype per `dtype`.   out [n, (lmax + 1)^2] device.
 * lmax in [0, 6] (E_UNSUPPORTED otherwise).
 */
int sh_fwd(int lmax, int normalize, int dtype, const void* vec, int64_t n, void* out, void* stream);

/*
 * sh_bwd: vector-Jacobian product of sh_fwd: grad_vec[i] = sum over j of
 * grad_sh[i, j] dY_j(vec[i]) / dvec[i] (zero for a zero vector with
 * normalisation).  grad_sh [n, (lmax + 1)^2], grad_vec [n, 3], device.
 */
int sh_bwd(int lmax, int normalize, int dtype, const void* vec, const void* grad_sh, int64_t n, void* grad_vec,
           void* stream);

/* segpoly_real_cg: the real coupling tensor of l1 x l2 -> l3 (the same
 * coefficients the paths use), row-major [2l1+1][2l2+1][2l3+1]; zeros when
 * the triangle rule fails.  l1, l2, l3 in [0, 6] (E_UNSUPPORTED otherwise). */
int segpoly_real_cg(int l1, int l2, int l3, double* out);

/* Message of the last failure on the calling thread ("" if none). */
const char* segpoly_last_error(void);

/* Library version string. */
const char* segpoly_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGPOLY_H */
