// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tpconv.h"

namespace tpc {

// ---- error reporting --------------------------------------------------------
tp_status set_error(tp_status code, const std::string& msg);
tp_status hip_error(hipError_t e, const char* where);

// ---- kernel dispatch --------------------------------------------------------
struct ConvArgs {
  int32_t n_nodes = 0, n_edges = 0;
  const int32_t *row_ptr = nullptr, *col = nullptr;
  const int32_t *t_row_ptr = nullptr, *t_perm = nullptr, *t_col = nullptr;
  // sender_rows: the edge rows (w, Y and their gradients) are stored in the
  // sender grouping (row k = sender-grouped position k); e_pos[q] is then the
  // row of receiver-sorted edge q, which the forward reads
  bool sender_rows = false;
  const int32_t* e_pos = nullptr;
  // launch order of the receiver- and sender-grouped kernels (null: node id)
  const int32_t *r_order = nullptr, *s_order = nullptr;
  const float *x = nullptr, *Y = nullptr, *w = nullptr, *grad_out = nullptr;
  float *out = nullptr, *grad_x = nullptr, *grad_Y = nullptr, *grad_w = nullptr;
  // second-order backward: cotangents of (grad_x, grad_Y, grad_w), outputs
  const float *gg_x = nullptr, *gg_Y = nullptr, *gg_w = nullptr;
  float *d_x = nullptr, *d_Y = nullptr, *d_w = nullptr, *d_g = nullptr;
  // edge-vector form: r [E][3] in place of Y, grad_r [E][3] in place of grad_Y
  const float* r = nullptr;
  float* grad_r = nullptr;
  hipStream_t stream = nullptr;
};

using LaunchFn = hipError_t (*)(const ConvArgs&);

struct KernelSet {
  LaunchFn fwd = nullptr;       // receiver pass: out
  LaunchFn bwd_recv = nullptr;  // receiver pass: grad_w, grad_Y
  LaunchFn bwd_send = nullptr;  // sender pass: grad_x
  LaunchFn dbl_recv = nullptr;  // second order, receiver pass: d_grad_out, d_Y, d_w
  LaunchFn dbl_send = nullptr;  // second order, sender pass: d_x
  LaunchFn bwd_fused = nullptr; // sender-grouped pass: grad_x with grad_w and/or grad_Y
  LaunchFn fwd_r = nullptr;     // forward from edge vectors (harmonics on chip)
  LaunchFn bwd_r = nullptr;     // backward from edge vectors: grad_x, grad_w, grad_r
};

// radial-weight variant (edge weights from a radial network of the length)
struct RadialArgs {
  int32_t n_nodes = 0, n_edges = 0;
  const int32_t *row_ptr = nullptr, *col = nullptr;
  const int32_t *t_row_ptr = nullptr, *t_perm = nullptr, *t_col = nullptr;
  // launch order of the receiver- and sender-grouped passes (null: node id)
  const int32_t *r_order = nullptr, *s_order = nullptr;
  const float *x = nullptr, *Y = nullptr, *r_len = nullptr, *W1 = nullptr, *W2 = nullptr;
  const float* grad_out = nullptr;   // gradient w.r.t. the unmixed output
  float *out = nullptr, *grad_x = nullptr, *grad_Y = nullptr, *grad_W1 = nullptr, *grad_W2 = nullptr;
  float* grad_rlen = nullptr;        // gradient w.r.t. the edge lengths (through the basis)
  float r_cut = 0.f;
  // edge-vector form: Y holds r [E][3] (r_len unused), grad_Y receives grad_r
  // [E][3] (grad_rlen unused)
  bool geom = false;
  // second-order backward: cotangents of (grad_x, grad_Y, grad_rlen) and
  // outputs (out receives d_grad_out before the mix)
  const float *gg_x = nullptr, *gg_Y = nullptr, *gg_rlen = nullptr;
  float *d_x = nullptr, *d_Y = nullptr, *d_rlen = nullptr, *d_W1 = nullptr, *d_W2 = nullptr;
  void* ws = nullptr;
  hipStream_t stream = nullptr;
};
using RadialFn = hipError_t (*)(const RadialArgs&);
struct RadialSet {
  RadialFn fwd = nullptr;
  RadialFn bwd = nullptr;                        // grad_x, grad_Y, grad_rlen, grad_W1, grad_W2
  size_t (*bwd_workspace)(int n_nodes, int n_edges) = nullptr;
  RadialFn dbl = nullptr;                        // d_grad_out (unmixed), d_x, d_Y, d_rlen, d_W1, d_W2
  size_t (*dbl_workspace)(int n_nodes, int n_edges) = nullptr;
};
// fully connected per-edge weights (W_e = sum_h R_e[h] Theta[h]), reassociated
struct FcArgs {
  int32_t n_nodes = 0, n_edges = 0, outdim = 0;
  const int32_t *row_ptr = nullptr, *col = nullptr;
  const int32_t *t_row_ptr = nullptr, *t_perm = nullptr, *t_col = nullptr;
  const int32_t *r_order = nullptr, *s_order = nullptr;   // launch orders (null: node id)
  const float *x = nullptr, *Y = nullptr, *R = nullptr, *Theta = nullptr;
  float* out = nullptr;
  // backward: upstream gradient and outputs (NULL: skip)
  const float* gout = nullptr;
  float *grad_x = nullptr, *grad_Y = nullptr, *grad_R = nullptr, *grad_Theta = nullptr;
  bool state_saved = false;   // backward: ws already holds the forward's state S
  void* ws = nullptr;
  hipStream_t stream = nullptr;
};
// second-order backward: cotangents of (grad_x, grad_Y, grad_R, grad_Theta)
// (NULL: zero) and outputs (NULL: skip); the FcArgs carry the first-order inputs
struct FcDbl {
  const float *gg_x = nullptr, *gg_Y = nullptr, *gg_R = nullptr, *gg_Theta = nullptr;
  float *d_x = nullptr, *d_Y = nullptr, *d_R = nullptr, *d_Theta = nullptr, *d_g = nullptr;
};
struct FcSet {
  hipError_t (*fwd)(const FcArgs&) = nullptr;
  size_t (*workspace)(int n_nodes) = nullptr;
  int n_radial = 0;
  hipError_t (*bwd)(const FcArgs&) = nullptr;
  size_t (*bwd_workspace)(int n_nodes) = nullptr;
  hipError_t (*dbl)(const FcArgs&, const FcDbl&) = nullptr;
  size_t (*dbl_workspace)(int n_nodes, int n_edges) = nullptr;
};
const FcSet* fc_l012_s2(int mul, int n_radial);

// Gaunt (spherical-grid) product: input degrees deg[0..n_in) (distinct, <= 2),
// filter degrees 0..lmax_sh (<= 2), output degrees 0..lmax_out (<= 2)
struct GauntArgs {
  int32_t n_nodes = 0, n_edges = 0, U = 0, n_in = 0, deg[3] = {0, 0, 0};
  int32_t lmax_sh = 0, lmax_out = 0;
  const int32_t *row_ptr = nullptr, *col = nullptr;
  const float *x = nullptr, *Y = nullptr, *w = nullptr;
  float* out = nullptr;
  // backward: the upstream gradient, the sender grouping and the outputs (NULL: skip)
  const float* gout = nullptr;
  const int32_t *t_row_ptr = nullptr, *t_perm = nullptr, *t_col = nullptr;
  float *grad_x = nullptr, *grad_Y = nullptr, *grad_w = nullptr;
  const int32_t *r_order = nullptr, *s_order = nullptr;   // launch orders (null: node id)
  hipStream_t stream = nullptr;
};
hipError_t gaunt_forward(const GauntArgs& a);
hipError_t gaunt_backward(const GauntArgs& a);
// second-order backward: cotangents of (grad_x, grad_Y, grad_w) (NULL: zero),
// outputs (NULL: skip) and scratch of gaunt_double_workspace bytes
struct GauntDbl {
  const float *gg_x = nullptr, *gg_Y = nullptr, *gg_w = nullptr;
  float *d_x = nullptr, *d_Y = nullptr, *d_w = nullptr, *d_g = nullptr;
  void* ws = nullptr;
};
hipError_t gaunt_double_backward(const GauntArgs& a, const GauntDbl& d);
size_t gaunt_double_workspace(const GauntArgs& a);
int gaunt_grid_points();

const RadialSet* find_radial(const std::vector<int>& ls, int lmax_sh, int lmax_out, int mul, int nb,
                             int nh);
const RadialSet* radial_l012_s2(int mul, int nb, int nh);
const RadialSet* radial_l0123_s3(int mul, int nb, int nh);

// Lookup of the compiled specialisation for (input degrees, lmax_sh,
// lmax_out, multiplicity); nullptr if none.
const KernelSet* find_kernels(const std::vector<int>& ls, int lmax_sh, int lmax_out, int mul);

// Per-signature registries (one translation unit each).
const KernelSet* kernels_l01_s1(int mul);
const KernelSet* kernels_l01_s2(int mul);
const KernelSet* kernels_l01_s3(int mul);
const KernelSet* kernels_l012_s2(int mul);
const KernelSet* kernels_l0123_s3(int mul);

// output-irrep description for the channel mix: degree-block sizes (2l+1) and
// per-channel offsets of each output irrep
struct UvwIrreps {
  int n;
  int dim[8];
  int ko[8];
};

// ---- device helpers implemented in graph.hip / sh.hip / uvw.hip --------------
size_t graph_workspace_bytes(int n_nodes, int n_edges);
tp_status graph_build(const int32_t* src, const int32_t* dst, int n_edges, int n_nodes,
                      int32_t* row_ptr, int32_t* col, int32_t* perm, int32_t* t_row_ptr,
                      int32_t* t_perm, int32_t* t_col, void* ws, int32_t flags, hipStream_t st);
tp_status graph_build_static(const int32_t* src, const int32_t* dst, int n_edges, int n_nodes,
                             int32_t* row_ptr, int32_t* col, int32_t* perm, int32_t* t_row_ptr,
                             int32_t* t_perm, int32_t* t_col, int32_t flags, hipStream_t st);
tp_status gather_rows(const void* in, const int32_t* perm, int64_t n_rows, int64_t words, void* out,
                      hipStream_t st);
tp_status sender_positions(const int32_t* t_perm, int n_edges, int32_t* e_pos, hipStream_t st);
size_t order_workspace_bytes(int n_nodes);
tp_status launch_order(const int32_t* row_ptr, const int32_t* t_row_ptr, int n_nodes, int n_edges,
                       int32_t* order, int32_t* t_order, void* ws, hipStream_t st);
tp_status sph_harm(int lmax, const float* r, int n, float* Y, hipStream_t st);
tp_status sph_harm_bwd(int lmax, const float* r, int n, const float* gY, const float* grl, float* gr,
                       hipStream_t st);
size_t uvw_workspace_bytes(int n_irreps, int U);
tp_status uvw_forward(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* W,
                      const float* X, float* Z, bool trans_w, hipStream_t st);
tp_status uvw_grad_w(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* X,
                     const float* G, float* gradW, void* ws, hipStream_t st);

}  // namespace tpc
