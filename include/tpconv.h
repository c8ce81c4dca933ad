/*
 * tpconv.h -- C ABI of the MI355X (gfx950) E(3)-equivariant tensor-product
 * graph convolution.
 *
 * The operation (the NequIP equivariant convolution of "Accelerating Tensor
 * Products in E(3)-Equivariant Graph Neural Networks", NeurIPS 2026, Abstract;
 * the edge-conditioned product streamed into receivers of "Sobek: Streaming
 * Equivariant Tensor Product Convolutions", Abstract; the full sparse CG
 * product of "FlashTP: Fused, Sparsity-Aware Tensor Product for MLIPs",
 * Abstract).  For every directed edge e = (j -> i):
 *
 *   out[i, k, u, c] += sum_{p : k(p) = k} w[e, p, u]
 *                      * sum_{a, b} C_p[a, b, c] x[j, l1(p), u, a] Y[e, l2(p), b]
 *
 * with p running over every path (l1, l2 -> l3) allowed by the triangle rule,
 * C_p the real-basis Clebsch-Gordan tensor, u the channel ("uvu": channel u
 * of the input feeds channel u of the output) and k(p) the output irrep
 * (l3, parity).  The pages never write this formula; it is the plain reading
 * of their prose.  Conventions (all fixed by this library):
 *   - real components m = -l..l; for l = 1 the order is (y, z, x);
 *   - harmonics are component-normalised: sum_m Y_lm^2 = 2l + 1;
 *   - real CG: Racah closed form, Condon-Shortley phase, orthonormal in the
 *     output index, sign making the first nonzero (a, b, c) positive;
 *   - paths: input irreps in string order, then l2 = 0..lmax_sh, then l3
 *     ascending; output irreps: distinct (l3, parity), l3 ascending, even
 *     before odd; paths on the same output irrep are summed;
 *   - edge vectors point from receiver to sender: r_e = pos[src] - pos[dst].
 *
 * Layouts (row-major, float32 unless stated):
 *   x     [N][xdim]   node rows; irrep blocks in string order, each [U][2l+1]
 *   out   [N][outdim] same, over the output irreps
 *   Y     [E][ysh]    ysh = (lmax_sh+1)^2; l-blocks, m = -l..l
 *   w     [E][P][U]   per-edge, per-path, per-channel weights
 *   Every edge-sized array (Y, w, r_len, grad_Y, grad_w) is in
 *   RECEIVER-SORTED order: position q holds original edge perm[q], where perm
 *   comes from tp_conv_graph_build.  tp_conv_gather_rows applies perm.
 *
 * Ownership: the caller allocates and owns every device buffer, workspace and
 * stream.  A plan owns a small host table and is freed by
 * tp_conv_plan_destroy.  No entry point allocates device memory.
 *
 * Errors: every entry point validates its arguments on the host before any
 * launch and returns a negative tp_status on failure, launching nothing.
 * Launches are asynchronous on the given stream; device faults surface at
 * the caller's next synchronisation.  tp_conv_last_error() describes the
 * last failure on the calling thread.  Outputs are overwritten, never
 * accumulated.  Device pointers must be 4-byte aligned; where an entry point
 * stages rows with 16-byte loads its comment says which pointers must be
 * 16-byte aligned, and a misaligned one is rejected with TP_ERR_ARG.
 *
 * Helper entry points that no page passage defines (plan inspection, buffer
 * sizes, the gather into receiver order, the error text) exist so that a
 * caller can size and lay out its buffers; their comments say so.
 */
#ifndef TPCONV_H
#define TPCONV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tp_status;
#define TP_OK 0
#define TP_ERR_ARG (-1)         /* null pointer, negative or inconsistent size */
#define TP_ERR_IRREPS (-2)      /* irreps string does not parse, mixed
                                   multiplicities, or non-natural parity */
#define TP_ERR_UNSUPPORTED (-3) /* no compiled kernel for this signature */
#define TP_ERR_OVERFLOW (-4)    /* a count does not fit the int32 indices */
#define TP_ERR_WORKSPACE (-5)   /* workspace missing or too small */
#define TP_ERR_HIP (-6)         /* a HIP call failed; text in last_error */
#define TP_ERR_INDEX (-7)       /* checked graph build found src/dst outside [0, N) */

#define TP_MODE_UVU 0   /* channel-wise Clebsch-Gordan product over every path */
#define TP_MODE_GAUNT 1 /* Gaunt (spherical-grid) product: tp_conv_forward_gaunt only */

typedef struct tp_plan_s* tp_plan_t;

/* Receiver- and sender-grouped edge indices, all int32 device pointers owned
 * by the caller, filled by tp_conv_graph_build:
 *   row_ptr[N+1]   receiver offsets into the receiver-sorted edge order
 *   col[E]         sender of each receiver-sorted edge
 *   perm[E]        original edge id of each receiver-sorted position
 *   t_row_ptr[N+1] sender offsets into t_perm
 *   t_perm[E]      receiver-sorted positions grouped by sender (ascending)
 *   t_col[E]       receiver of each sender-grouped edge
 * and, optionally (NULL: node order), filled by tp_conv_graph_launch_order:
 *   order[N]       receivers in the order the receiver-grouped passes launch
 *                  their workgroups
 *   t_order[N]     senders in the order the sender-grouped passes launch theirs
 * Zero-initialise the struct so that unused optional fields are NULL. */
typedef struct {
  int32_t n_nodes;
  int32_t n_edges;
  const int32_t* row_ptr;
  const int32_t* col;
  const int32_t* perm;
  const int32_t* t_row_ptr;
  const int32_t* t_perm;
  const int32_t* t_col;
  const int32_t* order;
  const int32_t* t_order;
} tp_graph;

/* Options of a plan.  Zero-initialised means "none".
 *   radial_basis, radial_hidden, r_cut: edge weights come from a radial
 *     network of the edge length (Bessel basis -> SiLU hidden layer ->
 *     P*U weights), used by the *_radial entry points (compiled for 8 basis
 *     functions and 64 hidden units, with 0e+1o+2e / lmax 2 at multiplicity
 *     16, 32, 64 or 128 and 0e+1o+2e+3o / lmax 3 at 16, 32 or 64; other
 *     plans: TP_ERR_UNSUPPORTED at plan creation);
 *   uvw: a U x U channel mix per output irrep follows the aggregation. */
typedef struct {
  int32_t radial_basis;
  int32_t radial_hidden;
  float r_cut;
  int32_t uvw;
} tp_plan_opts;

/* ---- plan (host only; no HIP calls) ---------------------------------------
 * Builds the path list, output irreps and real CG tables of a channel-wise
 * ("uvu") tensor product of `irreps_in` (e.g. "32x0e+32x1o+32x2e": one shared
 * multiplicity, natural parity) with harmonics up to lmax_sh, keeping output
 * degrees up to lmax_out, and selects the compiled kernel specialisation
 * (compiled: 0e+1o with lmax_sh = lmax_out = 1, 2 or 3; 0e+1o+2e with 2;
 * 0e+1o+2e+3o with 3; multiplicity 8, 16, 32, 64 or 128).
 * Source: path-aggregated sparse CG product ("FlashTP", Abstract).
 * mode TP_MODE_GAUNT builds the plan of the Gaunt product instead (see
 * tp_conv_forward_gaunt: even couplings only, no CG table, nnz = 0).
 * Returns TP_ERR_IRREPS / TP_ERR_UNSUPPORTED / TP_ERR_ARG on failure, in which
 * case *out is set to NULL. */
tp_status tp_conv_plan_create(tp_plan_t* out, const char* irreps_in, int32_t lmax_sh,
                              int32_t lmax_out, int32_t mode, const tp_plan_opts* opts);

/* Sizes of a plan.  Any output pointer may be NULL.  out_irreps receives the
 * output irreps string (NUL-terminated; TP_ERR_ARG if cap is too small).
 * Helper: the sizes a caller needs to allocate its arrays. */
tp_status tp_conv_plan_info(tp_plan_t plan, int32_t* n_paths, int32_t* mul, int32_t* xdim,
                            int32_t* ysh, int32_t* outdim, int32_t* nnz, char* out_irreps,
                            size_t out_irreps_cap);

/* Path list: for path p, l1l2l3k[4p..4p+3] = (l1, l2, l3, output irrep index).
 * Helper for inspection and tests; the path order is the plan's reading of
 * the "all paths" of the path-aggregated product ("FlashTP", Abstract). */
tp_status tp_conv_plan_paths(tp_plan_t plan, int32_t* l1l2l3k);

/* CG nonzeros of the plan, path by path, (a, b, c) lexicographic within a
 * path: pabc[4n..4n+3] = (p, a, b, c), val[n] = coefficient (float64).
 * Helper for inspection and tests: the sparse table the kernels carry as
 * immediates ("FlashTP", Abstract: only the nonzero coefficients are used). */
tp_status tp_conv_plan_cg(tp_plan_t plan, int16_t* pabc, double* val);

/* Frees a plan (NULL is ignored).  Helper: ownership of the plan's table. */
void tp_conv_plan_destroy(tp_plan_t plan);

/* Dense real CG tensor of one path, out[(a*(2l2+1) + b)*(2l3+1) + c], for
 * degrees up to 6 (host only).  TP_ERR_ARG if a degree is out of range; the
 * tensor is all zeros when the triangle rule fails.  Helper: the coupling
 * tensor of the product under the conventions above, for callers and tests. */
tp_status tp_cg_real(int32_t l1, int32_t l2, int32_t l3, double* out);

/* ---- graph (device) --------------------------------------------------------
 * Workspace bytes tp_conv_graph_build needs for (n_nodes, n_edges).  Helper:
 * sizes the caller-owned scratch of the sort. */
tp_status tp_conv_graph_workspace(int32_t n_nodes, int32_t n_edges, size_t* bytes);

#define TP_GRAPH_CHECK 1   /* verify every src/dst is in [0, N); synchronises */

/* Groups the edge list (src[e] -> dst[e], device int32) by receiver and by
 * sender with a stable order (ties keep the original edge order, and the
 * sender grouping keeps receiver-sorted order), filling every array of
 * tp_graph (see above).  Streaming edges grouped by receiver replaces scatter
 * atomics with receiver-side accumulation ("Sobek", Abstract; "The GPU
 * Workload That Rewrites Molecular Physics", section "What Makes MLFF
 * Workloads Structurally Different").  ws must hold
 * tp_conv_graph_workspace bytes.  Without TP_GRAPH_CHECK, indices outside
 * [0, N) give an unspecified grouping: the build never writes out of
 * bounds, and col and t_col are clamped into [0, N), so later calls on the
 * graph never read out of bounds either (their results are meaningless). */
tp_status tp_conv_graph_build(const int32_t* src, const int32_t* dst, int32_t n_edges,
                              int32_t n_nodes, int32_t* row_ptr, int32_t* col, int32_t* perm,
                              int32_t* t_row_ptr, int32_t* t_perm, int32_t* t_col, void* ws,
                              size_t ws_bytes, int32_t flags, hipStream_t stream);

/* tp_conv_graph_build without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The sort's scratch is a static device
 * array of TP_GRAPH_STATIC_SCRATCH_BYTES (24 MiB) inside the library, one per
 * GPU, held until the process ends; no call allocates.  Arguments, results
 * and errors as tp_conv_graph_build (bit-identical arrays), plus
 * TP_ERR_WORKSPACE, before any HIP call, when tp_conv_graph_workspace(n_nodes,
 * n_edges) exceeds TP_GRAPH_STATIC_SCRATCH_BYTES (graphs above about 1.2
 * million edges).  Every call on one GPU uses that GPU's single array: calls
 * that overlap on one GPU (other streams or threads) race, and the caller
 * must serialise them. */
#define TP_GRAPH_STATIC_SCRATCH_BYTES (24u << 20)
tp_status tp_conv_graph_build_static(const int32_t* src, const int32_t* dst, int32_t n_edges,
                                     int32_t n_nodes, int32_t* row_ptr, int32_t* col, int32_t* perm,
                                     int32_t* t_row_ptr, int32_t* t_perm, int32_t* t_col, int32_t flags,
                                     hipStream_t stream);

/* out[q, :] = in[perm[q], :] for q < n_rows, rows of row_words 32-bit words
 * (device pointers).  Puts edge-sized inputs into receiver-sorted order.
 * Helper: the layout every edge-sized argument uses (see above); perm must
 * come from tp_conv_graph_build (its entries index rows of in). */
tp_status tp_conv_gather_rows(const void* in, const int32_t* perm, int64_t n_rows,
                              int64_t row_words, void* out, hipStream_t stream);

/* Real component-normalised harmonics of the directions of r[E][3] (device
 * float32), Y[E][(lmax+1)^2], lmax <= 3.  A zero vector yields the
 * harmonics' polynomials evaluated at the origin (the direction is
 * undefined).  Harmonics of the edge direction are the second operand of the
 * product ("The GPU Workload That Rewrites Molecular Physics", section "What
 * Makes MLFF Workloads Structurally Different"). */
tp_status tp_conv_sph_harm(int32_t lmax, const float* r, int32_t n_edges, float* Y,
                           hipStream_t stream);

/* ---- convolution (device) ---------------------------------------------------
 * Forward: out = conv(x, Y, w) for the edges of `graph` (formula above).
 * One pass streams each receiver's edges, keeps the receiver's outputs in
 * registers and LDS and stores each output row once; no edge-sized
 * intermediate is written ("Sobek", Abstract; "FlashTP", Abstract).
 * x and w must be 16-byte aligned (TP_ERR_ARG). */
tp_status tp_conv_forward(tp_plan_t plan, const tp_graph* graph, const float* x,
                          const float* Y, const float* w, float* out, hipStream_t stream);

/* Backward: gradients of <grad_out, out> with respect to x, Y and w (exact
 * adjoint of the forward; "Sobek", Abstract, backward pass).  grad_x, grad_Y
 * or grad_w may be NULL to skip that output.  grad_x [N][xdim]; grad_Y
 * [E][ysh] and grad_w [E][P][U] in receiver-sorted order.  With grad_x and an
 * edge gradient requested (signatures of at most 256 CG nonzeros: all but
 * 0e+1o+2e+3o / lmax 3) one sender-grouped pass forms
 * all of them, reading w and Y once; otherwise a receiver pass (grad_w,
 * grad_Y) and a sender pass (grad_x).  grad_x needs the graph's sender
 * grouping.  x, w and grad_out must be 16-byte aligned (TP_ERR_ARG).
 * Deterministic: no atomics, fixed summation order. */
tp_status tp_conv_backward(tp_plan_t plan, const tp_graph* graph, const float* x,
                           const float* Y, const float* w, const float* grad_out,
                           float* grad_x, float* grad_Y, float* grad_w, hipStream_t stream);

/* ---- launch order -------------------------------------------------------------
 * Degrees vary from node to node (hub atoms; "The GPU Workload That Rewrites
 * Molecular Physics", section "What Makes MLFF Workloads Structurally
 * Different"), and the forward, the receiver pass, the sender pass and the
 * one-pass backward give each node one workgroup, so a high-degree node whose
 * workgroup starts late leaves the chip idle at the end of the launch.  With
 * graph->order / t_order set, the grid walks the nodes largest degree first
 * (longest first), which shortens that tail; every result is bit for bit the
 * same as in node order.  Helper: a schedule, not an operation of the pages.
 *
 * Workspace bytes tp_conv_graph_launch_order needs for n_nodes. */
tp_status tp_conv_graph_order_workspace(int32_t n_nodes, size_t* bytes);

/* order[k] = the receiver of k-th largest in-degree, t_order[k] = the sender
 * of k-th largest out-degree (ties in ascending node id), from the graph's
 * row_ptr and t_row_ptr; either output may be NULL (not both when N > 0).
 * N int32 each, device, caller-owned; ws must hold
 * tp_conv_graph_order_workspace bytes (TP_ERR_WORKSPACE otherwise).  Store
 * them in the graph's order / t_order fields for the convolution calls;
 * entries are clamped into [0, N), but an array that is not a permutation of
 * the nodes skips some nodes and repeats others. */
tp_status tp_conv_graph_launch_order(const tp_graph* graph, int32_t* order, int32_t* t_order, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* ---- sender-grouped edge layout ---------------------------------------------
 * The same forward and backward with the edge-sized arrays (Y, w, grad_Y,
 * grad_w) stored in the sender grouping: row k belongs to the edge at position
 * k of t_perm, i.e. to receiver-sorted edge t_perm[k].  A caller that forms the
 * per-edge weights and harmonics itself (a radial network and the harmonics of
 * the edge vectors) can form them in this order just as well; then the
 * backward, which walks the edges by sender, reads and writes its edge rows
 * contiguously, and the forward, which walks them by receiver, gathers them
 * (read only) through e_pos.  Streaming edge-local products into bounded node
 * state in whichever grouping keeps the larger edge streams sequential is the
 * schedule of "Sobek", Abstract; the gather-versus-stream trade-off is that of
 * "The GPU Workload That Rewrites Molecular Physics", section "The Compute vs.
 * Memory Bottleneck Shift".  Results equal those of tp_conv_forward /
 * tp_conv_backward on the same edges (summation order unchanged). */

/* e_pos[q] = the sender-grouped position of receiver-sorted edge q (the
 * inverse of graph->t_perm), E int32 on the device, caller-owned.  Helper: the
 * index the forward of this layout reads.  Needs the sender grouping. */
tp_status tp_conv_graph_sender_positions(const tp_graph* graph, int32_t* e_pos, hipStream_t stream);

/* tp_conv_forward with Y [E][ysh] and w [E][P][U] in the sender grouping;
 * e_pos from tp_conv_graph_sender_positions on the same graph.  x and w must
 * be 16-byte aligned (TP_ERR_ARG).  e_pos is not checked: an array that did
 * not come from that call (entries outside [0, E)) makes the forward read
 * outside Y and w.  The sender grouping of any graph from tp_conv_graph_build
 * is a permutation, so the e_pos made from it is always valid. */
tp_status tp_conv_forward_sg(tp_plan_t plan, const tp_graph* graph, const int32_t* e_pos, const float* x,
                             const float* Y, const float* w, float* out, hipStream_t stream);

/* tp_conv_backward with Y, w, grad_Y and grad_w in the sender grouping: one
 * sender-grouped pass for any subset of grad_x, grad_Y, grad_w (each may be
 * NULL), reading and writing the edge rows in order.  Signatures with a
 * one-pass backward only (at most 256 CG nonzeros; 0e+1o+2e+3o / lmax 3 gets
 * TP_ERR_UNSUPPORTED).  x, w and grad_out must be 16-byte aligned.
 * Deterministic. */
tp_status tp_conv_backward_sg(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                              const float* w, const float* grad_out, float* grad_x, float* grad_Y,
                              float* grad_w, hipStream_t stream);

/* ---- edge-vector form: harmonics evaluated on chip -------------------------
 * The layer as a function of the edge vectors r [E][3] (receiver-sorted,
 * r_e = pos[src] - pos[dst]) instead of their harmonics: each edge's
 * Y = Y(r_e / |r_e|) (component-normalised, lmax_sh of the plan; a zero vector
 * gives the polynomials at the origin, as tp_conv_sph_harm) is formed in
 * registers, so no Y array is read or written ("Sobek", Abstract: no
 * edge-sized intermediate; the harmonics of the edge direction are the
 * product's second operand, "The GPU Workload That Rewrites Molecular
 * Physics", section "What Makes MLFF Workloads Structurally Different").
 * tp_conv_forward_r(.., r, ..) equals tp_conv_forward(.., tp_conv_sph_harm(r), ..).
 * x and w must be 16-byte aligned (TP_ERR_ARG). */
tp_status tp_conv_forward_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                            const float* w, float* out, hipStream_t stream);

/* Backward of tp_conv_forward_r: grad_x [N][xdim], grad_w [E][P][U] and
 * grad_r [E][3] = sum_b grad_Y[b] dY_b/dr, the gradient with respect to the
 * edge vectors through the harmonics (the forces of a force field: add
 * -grad_r to each edge's sender and +grad_r to its receiver), formed per edge
 * on chip from the same products as grad_Y without storing grad_Y.  Any
 * output may be NULL.  Same passes, layouts and errors as tp_conv_backward;
 * x, w and grad_out must be 16-byte aligned.  Deterministic. */
tp_status tp_conv_backward_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                             const float* w, const float* grad_out, float* grad_x, float* grad_r,
                             float* grad_w, hipStream_t stream);

/* Second-order backward ("Sobek", Abstract: the streaming schedule extends
 * through forward, backward and double backward), e.g. for training on
 * forces.  Given the inputs of tp_conv_backward and cotangents gg_x [N][xdim],
 * gg_Y [E][ysh], gg_w [E][P][U] of its outputs (any may be NULL: zero), returns
 * the gradients of  L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_w, grad_w>:
 *   d_grad_out = out(gg_x, Y, w) + out(x, gg_Y, w) + out(x, Y, gg_w)   [N][outdim]
 *   d_x = grad_x(gg_Y, w) + grad_x(Y, gg_w)                            [N][xdim]
 *   d_Y = grad_Y(gg_x, w) + grad_Y(x, gg_w)                            [E][ysh]
 *   d_w = grad_w(gg_x, Y) + grad_w(x, gg_Y)                            [E][P][U]
 * (each term a first-order pass with one operand replaced; the layer is
 * linear in each of g, x, Y, w).  Outputs may be NULL to skip them; edge
 * arrays in receiver-sorted order; no atomics, deterministic. */
tp_status tp_conv_double_backward(tp_plan_t plan, const tp_graph* graph, const float* x,
                                  const float* Y, const float* w, const float* grad_out,
                                  const float* gg_x, const float* gg_Y, const float* gg_w,
                                  float* d_x, float* d_Y, float* d_w, float* d_grad_out,
                                  hipStream_t stream);

/* ---- fully connected per-edge weights (second operator family) -------------
 * Per-edge weights that mix channels, W_e[p][u][v] = sum_h R[e][h] Theta[h][p][u][v]
 * (R [E][n_radial] radial features, receiver-sorted; Theta [n_radial][P][U][U]):
 *   out[i, k, v, c] = sum_{e into i} sum_{p->k} sum_u W_e[p,u,v] T_p(x_j[u], Y_e)[c]
 * computed by reassociation ("Sobek", Abstract: radial projection, coupling and
 * aggregation reassociated into bounded receiver-side state; fully connected
 * multiplicity mixing preserved): S_i[h,p,u,c] = sum_e R[e][h] T_p(x_j[u], Y_e)[c]
 * is streamed per receiver into the node-sized workspace (tp_conv_fc_workspace
 * bytes), then out_i = Theta^T S_i per output irrep on the matrix cores.  No
 * per-edge weight or message is formed.  Compiled for 0e+1o+2e / lmax 2 with 16,
 * 32 or 64 channels and 8 radial features (other shapes: TP_ERR_UNSUPPORTED).
 * Errors: TP_ERR_WORKSPACE if ws is smaller than tp_conv_fc_workspace; TP_ERR_ARG
 * if ws is not 16-byte aligned or a needed pointer is NULL.  out is overwritten
 * (isolated receivers get zeros). */
tp_status tp_conv_fc_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_radial, size_t* bytes);
tp_status tp_conv_forward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                             const float* R, int32_t n_radial, const float* Theta, float* out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Adjoint of tp_conv_forward_fc for grad_out = d<., out> [N][outdim] (NULL
 * output: skip): grad_x [N][xdim], grad_Y [E][ysh] and grad_R [E][n_radial]
 * (receiver order), grad_Theta [n_radial][P][U][U].  Reassociated like the
 * forward (Sobek, Abstract: the streaming schedule covers the backward too):
 * the state's gradient gS_i = Theta gout_i is a dense product per receiver; a
 * receiver pass forms grad_R = <gS_i, T_e> and the CG adjoint for grad_Y; a
 * sender pass accumulates the sender-side state Q_j = sum_e R_e (x) G_e
 * (G_e: the CG adjoint terms of gout_i and Y_e), and grad_x = Theta^T Q_j; the
 * forward's state S is needed for grad_Theta = sum S^T gout.  No per-edge
 * weight matrix or message is formed.  ws: tp_conv_fc_backward_workspace
 * bytes; ws and Theta 16-byte aligned; grad_x needs the graph's sender
 * grouping.  flags: 0, or TP_FC_STATE_SAVED when the first
 * tp_conv_fc_workspace bytes of ws still hold the state that
 * tp_conv_forward_fc wrote there for the same plan, graph, x, Y and R (the
 * caller passed this ws to the forward and kept those bytes, as an autograd
 * function keeps what it saved): S is then read, not recomputed.  Without the
 * flag S is recomputed into ws.  Errors as tp_conv_forward_fc, and TP_ERR_ARG
 * for other flags.  Deterministic; both ways give identical results. */
#define TP_FC_STATE_SAVED 1
tp_status tp_conv_fc_backward_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_radial, size_t* bytes);
tp_status tp_conv_backward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                              const float* R, int32_t n_radial, const float* Theta, const float* grad_out,
                              float* grad_x, float* grad_Y, float* grad_R, float* grad_Theta, int32_t flags,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Second-order backward of the fully connected family ("Sobek", Abstract:
 * both operator families through forward, backward and double backward).
 * Given the inputs of tp_conv_backward_fc and cotangents gg_x [N][xdim], gg_Y
 * [E][ysh], gg_R [E][n_radial], gg_Theta [n_radial][P][U][U] of its outputs
 * (any may be NULL: zero), returns the gradients of
 *   L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_R, grad_R> + <gg_Theta, grad_Theta>:
 * the product is linear in each of x, Y, R and Theta, so
 *   d_grad_out = out(gg_x, ..) + out(.., gg_Y, ..) + out(.., gg_R, ..) + out(.., gg_Theta)
 * and d_x, d_Y, d_R, d_Theta are each the sum of the first backward's result
 * with one of the other operands replaced by its cotangent.  Each present
 * cotangent costs one reassociated forward and one backward (no per-edge
 * weight or message is formed); outputs may be NULL to skip them and get
 * zeros when no cotangent reaches them.  ws: tp_conv_fc_double_workspace
 * bytes (the first-order workspace plus one scratch row per output); ws,
 * Theta and gg_Theta 16-byte aligned; d_x needs the graph's sender grouping.
 * Deterministic. */
tp_status tp_conv_fc_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_edges, int32_t n_radial,
                                      size_t* bytes);
tp_status tp_conv_double_backward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                     const float* R, int32_t n_radial, const float* Theta,
                                     const float* grad_out, const float* gg_x, const float* gg_Y,
                                     const float* gg_R, const float* gg_Theta, float* d_x, float* d_Y,
                                     float* d_R, float* d_Theta, float* d_grad_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* ---- Gaunt (spherical-grid) product: a different, cheaper operator ----------
 * The Gaunt tensor product is not the CG product: it lacks the couplings with
 * l1 + l2 + l3 odd (such as the cross product) and so is less expressive, and
 * it can be evaluated on a spherical grid ("The Price of Freedom: Exploring
 * Expressivity and Runtime Tradeoffs in Equivariant Tensor Products",
 * Abstract).  It needs a plan created with mode TP_MODE_GAUNT (whose paths
 * are the even couplings and whose output irreps are l = 0..lmax_out of
 * parity (-1)^l); the CG entry points reject such a plan and the Gaunt ones
 * reject a TP_MODE_UVU plan, so neither replaces the other silently.  Per channel u the sender's row is the signal
 * f(s) = sum_{l,m} x[j,l,u,m] Y_lm(s), the edge the filter
 * g(s) = sum_{l2} w[e][l2][u] sum_m Y[e][l2,m] Y_{l2 m}(s), and
 *   out[i, l3, u, m3] = sum_{e into i} (1/4pi) int f g Y_{l3 m3} dOmega
 *                     = sum_e sum_{l1,l2} w[e][l2][u] sum_{a,b} G[a,b,c] x[j,l1,u,a] Y[e][l2,b],
 * G[a,b,c] = (1/4pi) int Y_a Y_b Y_c (component-normalised real harmonics).
 * Output irreps: 0e, 1o, 2e, ... up to lmax_out, block l3 = [U][2l3+1] at
 * column U*l3^2 (outdim = U (lmax_out+1)^2).  w is [E][lmax_sh+1][U] in
 * receiver order.  Evaluated on a 32-point product grid (4 Gauss-Legendre
 * nodes x 8 azimuths) that is exact for the degrees involved; per edge the
 * two signals on the grid are formed on the matrix cores and multiplied
 * pointwise into the receiver's grid values, which are projected once.
 * Compiled for distinct input degrees <= 2 (natural parity, any order),
 * lmax_sh <= 2, lmax_out <= 2 and U = 16, 32, 64 or 128; otherwise
 * TP_ERR_UNSUPPORTED.  out is overwritten; isolated receivers get zeros.
 * Deterministic (no atomics).  tp_conv_gaunt_dims reports outdim, the weights
 * per edge ((lmax_sh+1) U) and the number of grid points. */
tp_status tp_conv_gaunt_dims(tp_plan_t plan, int32_t* outdim, int32_t* wdim, int32_t* grid_points);
tp_status tp_conv_forward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                const float* w, float* out, hipStream_t stream);

/* Adjoint of tp_conv_forward_gaunt for grad_out = d<., out> [N][outdim]
 * (NULL output: skip):
 *   grad_x[j, l1, u, a] = sum_{e = (j -> i)} sum_{l2} w[e][l2][u] sum_{b,c} G[a,b,c] Y[e][l2,b] grad_out[i, l3, u, c]
 *   grad_w[e][l2][u]    = sum_{l1,l3} sum_{a,b,c} G[a,b,c] x[j, l1, u, a] Y[e][l2,b] grad_out[i, l3, u, c]
 *   grad_Y[e][l2, b]    = sum_u w[e][l2][u] sum_{l1,l3} sum_{a,c} G[a,b,c] x[j, l1, u, a] grad_out[i, l3, u, c]
 * evaluated on the same grid (the adjoint of the projection puts grad_out on
 * the grid): a receiver pass for grad_w and grad_Y (edge arrays in receiver
 * order) and a sender pass for grad_x, which needs the graph's sender grouping
 * (t_row_ptr, t_perm, t_col).  Outputs are overwritten; deterministic.  w must
 * be 16-byte aligned (TP_ERR_ARG); other errors as tp_conv_forward_gaunt. */
tp_status tp_conv_backward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                 const float* w, const float* grad_out, float* grad_x, float* grad_Y,
                                 float* grad_w, hipStream_t stream);

/* Second-order backward of the Gaunt product ("Sobek", Abstract: forward,
 * backward and double backward).  Given the inputs of tp_conv_backward_gaunt
 * and cotangents gg_x [N][xdim], gg_Y [E][ysh], gg_w [E][wdim] of its outputs
 * (any may be NULL: zero), returns the gradients of
 *   L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_w, grad_w>:
 * the product is linear in each of x, Y and w, so
 *   d_grad_out = out(gg_x, Y, w) + out(x, gg_Y, w) + out(x, Y, gg_w)
 * and d_x, d_Y, d_w are each the sum of the first backward's result with one
 * of the other operands replaced by its cotangent (one grid forward and one
 * grid backward per present cotangent).  Outputs may be NULL to skip them
 * and get zeros when no cotangent reaches them; ws:
 * tp_conv_gaunt_double_workspace bytes (one scratch row per output); w and
 * gg_w 16-byte aligned; d_x needs the graph's sender grouping.  Deterministic. */
tp_status tp_conv_gaunt_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_edges, size_t* bytes);
tp_status tp_conv_double_backward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                        const float* w, const float* grad_out, const float* gg_x,
                                        const float* gg_Y, const float* gg_w, float* d_x, float* d_Y, float* d_w,
                                        float* d_grad_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- channel mix ("uvw", dense; fp32 MFMA) ----------------------------------
 * One U x U matrix per output irrep k (Wmix [K][U][U], K = number of output
 * irreps, U = 16, 32, 64 or 128; 1e and 1o never mix):
 *   out[i, k, v, c] = sum_u Wmix[k][u][v] in[i, k, u, c]       (in, out: [N][outdim])
 * The post-aggregation channel mixing of the radial-weight layer ("Sobek",
 * Abstract, on preserving multiplicity mixing).  in and out must not alias
 * and must be 16-byte aligned (whole node blocks move as 16-byte granules;
 * TP_ERR_ARG otherwise). */
tp_status tp_conv_uvw_forward(tp_plan_t plan, int32_t n_nodes, const float* Wmix, const float* in,
                              float* out, hipStream_t stream);

/* Adjoint of tp_conv_uvw_forward for grad_out = d<.,out>:
 *   grad_in[i, k, u, c] = sum_v Wmix[k][u][v] grad_out[i, k, v, c]   (NULL: skip)
 *   grad_Wmix[k][u][v]  = sum_{i,c} in[i, k, u, c] grad_out[i, k, v, c]  (NULL: skip)
 * grad_Wmix is reduced deterministically through ws (tp_conv_uvw_workspace
 * bytes; helper that sizes it).  in, grad_out and grad_in must be 16-byte
 * aligned (TP_ERR_ARG). */
tp_status tp_conv_uvw_backward(tp_plan_t plan, int32_t n_nodes, const float* Wmix, const float* in,
                               const float* grad_out, float* grad_in, float* grad_Wmix, void* ws,
                               size_t ws_bytes, hipStream_t stream);
tp_status tp_conv_uvw_workspace(tp_plan_t plan, size_t* bytes);

/* ---- radial-weight convolution (plan with radial_basis / radial_hidden) ----
 * Edge weights come from a radial network of the edge length r_len[E]
 * (receiver-sorted), computed on chip and never stored ("Sobek", Abstract and
 * AI Summary: radial projection reassociated with coupling and aggregation):
 *   B_n(r) = sqrt(2/r_cut) sin(n pi r / r_cut) / r, n = 1..radial_basis
 *   w[e, p, u] = (SiLU(B(r_e) W1) W2)[p*U + u]
 * W1 [radial_basis][radial_hidden], W2 [radial_hidden][P*U] (device float32).
 * With Wmix (NULL: no mix) the aggregated output is written to out_pre and
 * the mixed output to out (tp_conv_uvw_forward); without it, to out. */
tp_status tp_conv_forward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                 const float* Y, const float* r_len, const float* W1,
                                 const float* W2, const float* Wmix, float* out_pre, float* out,
                                 hipStream_t stream);

/* Backward of tp_conv_forward_radial for the upstream gradient grad_out of its
 * final output ("Sobek", Abstract: the streaming schedule covers the backward
 * pass).  With Wmix, out_pre is the forward's unmixed output and grad_Wmix
 * [K][U][U] is produced; the gradient reaching the aggregation is
 * Wmix-applied grad_out.  Outputs (each may be NULL to skip it):
 *   grad_x [N][xdim], grad_Y [E][ysh] and grad_rlen [E] (receiver-sorted),
 *   grad_W1 and grad_W2 (shapes of W1, W2), grad_Wmix.
 * grad_rlen is the gradient with respect to the edge lengths through the
 * radial basis: sum_n grad_B[e][n] dB_n/dr with grad_B = grad_pre W1^T; with
 * grad_Y it gives the forces on the edge vectors (tp_conv_sph_harm_backward).
 * The per-edge weights, their gradients and the hidden activations are
 * recomputed on chip, never stored.  x, grad_out and W2 must be 16-byte
 * aligned (vector loads of four channels).  Parameter gradients are reduced in a fixed
 * order through ws (tp_conv_radial_workspace bytes for the same sizes), so the
 * results are bitwise reproducible. */
tp_status tp_conv_backward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                  const float* Y, const float* r_len, const float* W1,
                                  const float* W2, const float* Wmix, const float* out_pre,
                                  const float* grad_out, float* grad_x, float* grad_Y,
                                  float* grad_rlen, float* grad_W1, float* grad_W2,
                                  float* grad_Wmix, void* ws, size_t ws_bytes, hipStream_t stream);
/* Workspace bytes of tp_conv_backward_radial for n_nodes nodes (with_mix != 0:
 * a channel mix is differentiated too). */
tp_status tp_conv_radial_workspace(tp_plan_t plan, int32_t n_nodes, int32_t with_mix, size_t* bytes);

/* Edge-vector form of the radial layer: r [E][3] (receiver-sorted) replaces Y
 * and r_len; each edge's harmonics and length |r| are evaluated on chip
 * (tp_conv_forward_r) for the radial network and the product.  The backward
 * returns grad_r [E][3], the gradient with respect to the edge vectors through
 * both the harmonics and the lengths (the forces of the layer), in place of
 * grad_Y and grad_rlen; neither is stored.  Otherwise as
 * tp_conv_forward_radial / tp_conv_backward_radial (same workspace, alignment,
 * outputs that may be NULL, fixed-order parameter sums). */
tp_status tp_conv_forward_radial_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                                   const float* W1, const float* W2, const float* Wmix, float* out_pre,
                                   float* out, hipStream_t stream);
tp_status tp_conv_backward_radial_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                                    const float* W1, const float* W2, const float* Wmix,
                                    const float* out_pre, const float* grad_out, float* grad_x,
                                    float* grad_r, float* grad_W1, float* grad_W2, float* grad_Wmix,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Second-order backward of the radial layer ("Sobek", Abstract: forward,
 * backward and double backward, the radial projection streamed).  Given the
 * inputs of tp_conv_backward_radial and cotangents gg_x [N][xdim], gg_Y
 * [E][ysh] and gg_rlen [E] of its outputs grad_x, grad_Y and grad_rlen (what a
 * loss on forces produces; any may be NULL: zero), returns the gradients of
 *   L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_rlen, grad_rlen>
 * with respect to x (d_x [N][xdim]), Y (d_Y [E][ysh]), r_len (d_rlen [E]),
 * W1, W2 (d_W1, d_W2, their shapes), Wmix (d_Wmix, with a mix) and grad_out
 * (d_grad_out [N][outdim]).  With v = gg_rlen dw/dr the weights' tangent and
 * out_dot = out(gg_x, Y, w) + out(x, gg_Y, w) + out(x, Y, v) (unmixed):
 * d_grad_out = mix(out_dot), d_Wmix = grad_Wmix of <grad_out, mix(out_dot)>,
 * d_x and d_Y are first-order adjoints with one operand replaced, and d_W1,
 * d_W2, d_rlen follow by the chain rule through the network (second
 * derivatives of SiLU and of the basis enter there).  Outputs may be NULL to
 * skip them; d_Wmix needs Wmix.  The weights and their tangent are recomputed
 * on chip, never stored; parameter gradients are fixed-order sums through ws
 * (tp_conv_radial_double_workspace bytes), so results are bitwise
 * reproducible.  x, gg_x, grad_out and W2 must be 16-byte aligned
 * (TP_ERR_ARG); edge arrays receiver-sorted. */
tp_status tp_conv_double_backward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                         const float* Y, const float* r_len, const float* W1,
                                         const float* W2, const float* Wmix, const float* grad_out,
                                         const float* gg_x, const float* gg_Y, const float* gg_rlen,
                                         float* d_x, float* d_Y, float* d_rlen, float* d_W1, float* d_W2,
                                         float* d_Wmix, float* d_grad_out, void* ws, size_t ws_bytes,
                                         hipStream_t stream);
/* Workspace bytes of tp_conv_double_backward_radial for n_nodes nodes
 * (with_mix != 0: a channel mix).  Helper that sizes ws. */
tp_status tp_conv_radial_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t with_mix,
                                          size_t* bytes);

/* Gradient with respect to the edge vectors r[E][3] of a loss that depends on
 * them through Y = tp_conv_sph_harm(lmax, r) (upstream grad_Y[E][(lmax+1)^2])
 * and, optionally, through the edge lengths |r| (upstream grad_rlen[E], NULL:
 * none):  grad_r = sum_b grad_Y[b] dY_b/dr + grad_rlen r/|r|.  The forces on
 * atoms follow by summing -grad_r into the sender and +grad_r into the
 * receiver of each edge (r = pos[src] - pos[dst]).  Forces are what a force
 * field predicts ("The GPU Workload That Rewrites Molecular Physics", opening
 * sections), obtained by differentiating through the layer and the harmonics
 * of the edge direction ("Sobek", Abstract: the schedule extends through the
 * backward pass).  lmax <= 3; all arrays device float32, edge order as given;
 * grad_r is overwritten. */
tp_status tp_conv_sph_harm_backward(int32_t lmax, const float* r, int32_t n_edges,
                                    const float* grad_Y, const float* grad_rlen, float* grad_r,
                                    hipStream_t stream);

/* Thread-local description of the last failure on this thread (helper for
 * error reporting; valid until the next failing call on the thread). */
const char* tp_conv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TPCONV_H */
