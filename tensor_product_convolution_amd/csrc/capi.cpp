// C ABI: plan building (host only), argument validation and kernel dispatch.
// The plan enumerates the paths of a channel-wise product and its output
// irreps (path aggregation over every (l1, l2 -> l3): "FlashTP: Fused,
// Sparsity-Aware Tensor Product for MLIPs", Abstract), computes the real CG
// nonzeros with the same constexpr routines the kernels were specialised
// with, and picks the compiled kernel set for the signature.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cctype>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "cg_table.hpp"
#include "internal.hpp"

struct tp_plan_s {
  int mode = TP_MODE_UVU;
  int mul = 0;
  std::vector<int> ls;                 // input degrees, string order
  int lmax_sh = 0, lmax_out = 0;
  struct Path {
    int in, l1, l2, l3, k;
  };
  std::vector<Path> paths;
  std::vector<std::pair<int, int>> outs;  // (l, parity)
  int xdim = 0, ysh = 0, outdim = 0, nnz = 0;
  std::vector<int16_t> cg_pabc;
  std::vector<double> cg_val;
  std::string out_irreps;
  tp_plan_opts opts{};
  const tpc::KernelSet* ks = nullptr;
  const tpc::RadialSet* rs = nullptr;   // radial-weight kernels (opts.radial_basis > 0)
  tpc::UvwIrreps uvw{};
};

namespace tpc {

namespace {
thread_local std::string g_last_error;
}

tp_status set_error(tp_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

tp_status hip_error(hipError_t e, const char* where) {
  return set_error(TP_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

const RadialSet* find_radial(const std::vector<int>& ls, int lmax_sh, int lmax_out, int mul, int nb,
                             int nh) {
  if (ls == std::vector<int>{0, 1, 2} && lmax_sh == 2 && lmax_out == 2)
    return radial_l012_s2(mul, nb, nh);
  if (ls == std::vector<int>{0, 1, 2, 3} && lmax_sh == 3 && lmax_out == 3)
    return radial_l0123_s3(mul, nb, nh);
  return nullptr;
}

const KernelSet* find_kernels(const std::vector<int>& ls, int lmax_sh, int lmax_out, int mul) {
  if (ls == std::vector<int>{0, 1} && lmax_sh == 1 && lmax_out == 1) return kernels_l01_s1(mul);
  if (ls == std::vector<int>{0, 1} && lmax_sh == 2 && lmax_out == 2) return kernels_l01_s2(mul);
  if (ls == std::vector<int>{0, 1} && lmax_sh == 3 && lmax_out == 3) return kernels_l01_s3(mul);
  if (ls == std::vector<int>{0, 1, 2} && lmax_sh == 2 && lmax_out == 2) return kernels_l012_s2(mul);
  if (ls == std::vector<int>{0, 1, 2, 3} && lmax_sh == 3 && lmax_out == 3)
    return kernels_l0123_s3(mul);
  return nullptr;
}

namespace {

// "MxLp" terms joined by '+'; whitespace around terms is ignored.
bool parse_irreps(const char* s, std::vector<int>* muls, std::vector<int>* ls, std::vector<int>* ps,
                  std::string* err) {
  std::string str(s);
  size_t pos = 0;
  if (str.find_first_not_of(" \t") == std::string::npos) {
    *err = "empty irreps string";
    return false;
  }
  while (true) {
    size_t plus = str.find('+', pos);
    std::string term = str.substr(pos, plus == std::string::npos ? std::string::npos : plus - pos);
    size_t b = term.find_first_not_of(" \t"), e = term.find_last_not_of(" \t");
    term = b == std::string::npos ? std::string() : term.substr(b, e - b + 1);
    size_t x = term.find('x');
    if (term.empty() || x == std::string::npos || x == 0 || x + 2 > term.size()) {
      *err = "bad irreps term '" + term + "'";
      return false;
    }
    std::string m = term.substr(0, x), l = term.substr(x + 1, term.size() - x - 2);
    char p = term.back();
    auto digits = [](const std::string& t) {
      return !t.empty() && t.size() < 7 &&
             std::all_of(t.begin(), t.end(), [](char c) { return std::isdigit((unsigned char)c); });
    };
    if (!digits(m) || !digits(l) || (p != 'e' && p != 'o')) {
      *err = "bad irreps term '" + term + "'";
      return false;
    }
    int mv = std::stoi(m), lv = std::stoi(l);
    if (mv <= 0) {
      *err = "multiplicity must be positive in '" + term + "'";
      return false;
    }
    muls->push_back(mv);
    ls->push_back(lv);
    ps->push_back(p == 'e' ? 1 : -1);
    if (plus == std::string::npos) break;
    pos = plus + 1;
  }
  return true;
}

}  // namespace
}  // namespace tpc

using tpc::set_error;

extern "C" {

const char* tp_conv_last_error(void) { return tpc::g_last_error.c_str(); }

tp_status tp_cg_real(int32_t l1, int32_t l2, int32_t l3, double* out) {
  if (!out) return set_error(TP_ERR_ARG, "tp_cg_real: out is NULL");
  if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > tpc::kMaxL || l2 > tpc::kMaxL || l3 > tpc::kMaxL)
    return set_error(TP_ERR_ARG, "tp_cg_real: degrees must be in 0..6");
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  const bool ok = tpc::triangle(l1, l2, l3);
  const double s = ok ? tpc::real_cg_sign(l1, l2, l3) : 1.0;
  for (int a = 0; a < n1; ++a)
    for (int b = 0; b < n2; ++b)
      for (int c = 0; c < n3; ++c)
        out[(a * n2 + b) * n3 + c] = ok ? tpc::real_cg(l1, l2, l3, a, b, c, s) : 0.0;
  return TP_OK;
}

static tp_status gaunt_supported(tp_plan_t plan, const char* who);

// Gaunt-mode plan: the (l1, l2, l3) couplings with l1 + l2 + l3 even inside
// the triangle (all others vanish), output irreps l = 0..lmax_out of parity
// (-1)^l; no CG table and no CG kernels.
static tp_status gaunt_plan_create(tp_plan_t* out, int mul, const std::vector<int>& ls, int lmax_sh,
                                   int lmax_out, const tp_plan_opts* opts) {
  if (opts && (opts->radial_basis || opts->radial_hidden || opts->uvw))
    return set_error(TP_ERR_UNSUPPORTED, "Gaunt plans take no radial network or mix options");
  auto* p = new tp_plan_s();
  p->mode = TP_MODE_GAUNT;
  p->mul = mul;
  p->ls = ls;
  p->lmax_sh = lmax_sh;
  p->lmax_out = lmax_out;
  tp_status s = gaunt_supported(p, "tp_conv_plan_create");
  if (s != TP_OK) {
    delete p;
    return s;
  }
  for (size_t i = 0; i < ls.size(); ++i)
    for (int l2 = 0; l2 <= lmax_sh; ++l2)
      for (int l3 = std::abs(ls[i] - l2); l3 <= std::min(ls[i] + l2, lmax_out); ++l3)
        if (((ls[i] + l2 + l3) & 1) == 0) p->paths.push_back({(int)i, ls[i], l2, l3, l3});
  if (p->paths.empty()) {
    delete p;
    return set_error(TP_ERR_ARG, "no even coupling satisfies the triangle rule with these lmax");
  }
  for (int l = 0; l <= lmax_out; ++l) p->outs.push_back({l, (l & 1) ? -1 : 1});
  for (int l : ls) p->xdim += mul * (2 * l + 1);
  p->outdim = mul * (lmax_out + 1) * (lmax_out + 1);
  p->ysh = (lmax_sh + 1) * (lmax_sh + 1);
  p->nnz = 0;
  p->uvw.n = (int)p->outs.size();
  for (size_t k = 0; k < p->outs.size(); ++k) {
    if (k) p->out_irreps += "+";
    p->out_irreps += std::to_string(mul) + "x" + std::to_string(p->outs[k].first) +
                     (p->outs[k].second == 1 ? "e" : "o");
    p->uvw.dim[k] = 2 * p->outs[k].first + 1;
    p->uvw.ko[k] = (int)(k * k);
  }
  *out = p;
  return TP_OK;
}

tp_status tp_conv_plan_create(tp_plan_t* out, const char* irreps_in, int32_t lmax_sh,
                              int32_t lmax_out, int32_t mode, const tp_plan_opts* opts) {
  if (!out) return set_error(TP_ERR_ARG, "tp_conv_plan_create: out is NULL");
  *out = nullptr;
  if (!irreps_in) return set_error(TP_ERR_ARG, "tp_conv_plan_create: irreps_in is NULL");
  if (mode != TP_MODE_UVU && mode != TP_MODE_GAUNT)
    return set_error(TP_ERR_UNSUPPORTED, "mode must be TP_MODE_UVU (0) or TP_MODE_GAUNT (1)");
  if (lmax_sh < 0 || lmax_out < 0 || lmax_sh > tpc::kMaxL || lmax_out > tpc::kMaxL)
    return set_error(TP_ERR_ARG, "lmax_sh and lmax_out must be in 0..6");
  std::vector<int> muls, ls, ps;
  std::string err;
  if (!tpc::parse_irreps(irreps_in, &muls, &ls, &ps, &err)) return set_error(TP_ERR_IRREPS, err);
  for (size_t i = 0; i < ls.size(); ++i) {
    if (muls[i] != muls[0])
      return set_error(TP_ERR_IRREPS, "channel-wise product needs one multiplicity for all irreps");
    if (ps[i] != ((ls[i] & 1) ? -1 : 1))
      return set_error(TP_ERR_IRREPS, "input irreps must have natural parity (-1)^l");
    if (ls[i] > tpc::kMaxL) return set_error(TP_ERR_UNSUPPORTED, "input degree above 6");
  }
  if (opts) {
    if (opts->radial_basis < 0 || opts->radial_hidden < 0 || opts->uvw < 0)
      return set_error(TP_ERR_ARG, "negative plan option");
    if ((opts->radial_basis > 0) != (opts->radial_hidden > 0))
      return set_error(TP_ERR_ARG, "radial_basis and radial_hidden must both be set");
    if (opts->radial_basis > 0 && !(opts->r_cut > 0.f))
      return set_error(TP_ERR_ARG, "r_cut must be positive");
  }

  if (mode == TP_MODE_GAUNT) return gaunt_plan_create(out, muls[0], ls, lmax_sh, lmax_out, opts);

  auto* p = new tp_plan_s();
  p->mul = muls[0];
  p->ls = ls;
  p->lmax_sh = lmax_sh;
  p->lmax_out = lmax_out;
  if (opts) p->opts = *opts;
  // paths
  std::vector<std::pair<int, int>> raw_out;
  for (size_t i = 0; i < ls.size(); ++i)
    for (int l2 = 0; l2 <= lmax_sh; ++l2)
      for (int l3 = std::abs(ls[i] - l2); l3 <= std::min(ls[i] + l2, (int)lmax_out); ++l3) {
        p->paths.push_back({(int)i, ls[i], l2, l3, -1});
        raw_out.push_back({l3, ps[i] * ((l2 & 1) ? -1 : 1)});
      }
  if (p->paths.empty()) {
    delete p;
    return set_error(TP_ERR_ARG, "no path satisfies the triangle rule with these lmax");
  }
  for (int l = 0; l <= lmax_out; ++l)
    for (int par : {1, -1})
      if (std::find(raw_out.begin(), raw_out.end(), std::make_pair(l, par)) != raw_out.end())
        p->outs.push_back({l, par});
  for (size_t q = 0; q < p->paths.size(); ++q)
    p->paths[q].k = (int)(std::find(p->outs.begin(), p->outs.end(), raw_out[q]) - p->outs.begin());
  for (int l : ls) p->xdim += p->mul * (2 * l + 1);
  for (auto& o : p->outs) p->outdim += p->mul * (2 * o.first + 1);
  p->ysh = (lmax_sh + 1) * (lmax_sh + 1);
  for (size_t q = 0; q < p->paths.size(); ++q) {
    const auto& pa = p->paths[q];
    const double s = tpc::real_cg_sign(pa.l1, pa.l2, pa.l3);
    for (int a = 0; a <= 2 * pa.l1; ++a)
      for (int b = 0; b <= 2 * pa.l2; ++b)
        for (int c = 0; c <= 2 * pa.l3; ++c) {
          double v = tpc::real_cg(pa.l1, pa.l2, pa.l3, a, b, c, s);
          if (v != 0.0) {
            p->cg_pabc.insert(p->cg_pabc.end(), {(int16_t)q, (int16_t)a, (int16_t)b, (int16_t)c});
            p->cg_val.push_back(v);
          }
        }
  }
  p->nnz = (int)p->cg_val.size();
  for (size_t k = 0; k < p->outs.size(); ++k) {
    if (k) p->out_irreps += "+";
    p->out_irreps += std::to_string(p->mul) + "x" + std::to_string(p->outs[k].first) +
                     (p->outs[k].second == 1 ? "e" : "o");
  }
  p->uvw.n = (int)p->outs.size();
  for (size_t k = 0, ko = 0; k < p->outs.size(); ++k) {
    p->uvw.dim[k] = 2 * p->outs[k].first + 1;
    p->uvw.ko[k] = (int)ko;
    ko += 2 * p->outs[k].first + 1;
  }
  if (opts && opts->uvw) {
    const int m = p->mul;
    if (m > 128 || (m & (m - 1)) || m < 16 || p->outs.size() > 8) {
      delete p;
      return set_error(TP_ERR_UNSUPPORTED, "uvw mix needs a multiplicity of 16, 32, 64 or 128");
    }
  }
  if (opts && opts->radial_basis > 0) {
    p->rs = tpc::find_radial(ls, lmax_sh, lmax_out, p->mul, opts->radial_basis, opts->radial_hidden);
    if (!p->rs) {
      delete p;
      return set_error(TP_ERR_UNSUPPORTED,
                       "no compiled radial-weight kernel for this signature (supported: 0e+1o+2e / "
                       "lmax 2 with multiplicity 16, 32, 64 or 128 and 0e+1o+2e+3o / lmax 3 with 16, "
                       "32 or 64; 8 basis functions, 64 hidden units)");
    }
  }
  p->ks = tpc::find_kernels(ls, lmax_sh, lmax_out, p->mul);
  if (!p->ks) {
    delete p;
    return set_error(TP_ERR_UNSUPPORTED,
                     "no compiled kernel for this signature (supported: 0e+1o / lmax 1, 2 or 3, "
                     "0e+1o+2e / lmax 2, 0e+1o+2e+3o / lmax 3; multiplicity 8, 16, 32, 64 or 128)");
  }
  *out = p;
  return TP_OK;
}

tp_status tp_conv_plan_info(tp_plan_t plan, int32_t* n_paths, int32_t* mul, int32_t* xdim,
                            int32_t* ysh, int32_t* outdim, int32_t* nnz, char* out_irreps,
                            size_t cap) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_plan_info: plan is NULL");
  if (n_paths) *n_paths = (int32_t)plan->paths.size();
  if (mul) *mul = plan->mul;
  if (xdim) *xdim = plan->xdim;
  if (ysh) *ysh = plan->ysh;
  if (outdim) *outdim = plan->outdim;
  if (nnz) *nnz = plan->nnz;
  if (out_irreps) {
    if (cap < plan->out_irreps.size() + 1)
      return set_error(TP_ERR_ARG, "tp_conv_plan_info: out_irreps buffer too small");
    std::memcpy(out_irreps, plan->out_irreps.c_str(), plan->out_irreps.size() + 1);
  }
  return TP_OK;
}

tp_status tp_conv_plan_paths(tp_plan_t plan, int32_t* l1l2l3k) {
  if (!plan || !l1l2l3k) return set_error(TP_ERR_ARG, "tp_conv_plan_paths: NULL argument");
  for (size_t q = 0; q < plan->paths.size(); ++q) {
    l1l2l3k[4 * q] = plan->paths[q].l1;
    l1l2l3k[4 * q + 1] = plan->paths[q].l2;
    l1l2l3k[4 * q + 2] = plan->paths[q].l3;
    l1l2l3k[4 * q + 3] = plan->paths[q].k;
  }
  return TP_OK;
}

tp_status tp_conv_plan_cg(tp_plan_t plan, int16_t* pabc, double* val) {
  if (!plan || !pabc || !val) return set_error(TP_ERR_ARG, "tp_conv_plan_cg: NULL argument");
  std::memcpy(pabc, plan->cg_pabc.data(), plan->cg_pabc.size() * sizeof(int16_t));
  std::memcpy(val, plan->cg_val.data(), plan->cg_val.size() * sizeof(double));
  return TP_OK;
}

void tp_conv_plan_destroy(tp_plan_t plan) { delete plan; }

tp_status tp_conv_graph_workspace(int32_t n_nodes, int32_t n_edges, size_t* bytes) {
  if (!bytes) return set_error(TP_ERR_ARG, "tp_conv_graph_workspace: bytes is NULL");
  if (n_nodes < 0 || n_edges < 0) return set_error(TP_ERR_ARG, "negative size");
  *bytes = tpc::graph_workspace_bytes(n_nodes, n_edges);
  return TP_OK;
}

tp_status tp_conv_graph_build(const int32_t* src, const int32_t* dst, int32_t n_edges,
                              int32_t n_nodes, int32_t* row_ptr, int32_t* col, int32_t* perm,
                              int32_t* t_row_ptr, int32_t* t_perm, int32_t* t_col, void* ws,
                              size_t ws_bytes, int32_t flags, hipStream_t stream) {
  if (n_nodes < 0 || n_edges < 0) return set_error(TP_ERR_ARG, "tp_conv_graph_build: negative size");
  if (n_edges > 0 && n_nodes == 0)
    return set_error(TP_ERR_ARG, "tp_conv_graph_build: edges need at least one node");
  if (!row_ptr || !t_row_ptr) return set_error(TP_ERR_ARG, "tp_conv_graph_build: NULL row pointer");
  if (n_edges > 0 && (!src || !dst || !col || !perm || !t_perm || !t_col))
    return set_error(TP_ERR_ARG, "tp_conv_graph_build: NULL edge array");
  const size_t need = tpc::graph_workspace_bytes(n_nodes, n_edges);
  if (!ws || ws_bytes < need)
    return set_error(TP_ERR_WORKSPACE, "tp_conv_graph_build: workspace needs " +
                                           std::to_string(need) + " bytes");
  return tpc::graph_build(src, dst, n_edges, n_nodes, row_ptr, col, perm, t_row_ptr, t_perm, t_col,
                          ws, flags, stream);
}

tp_status tp_conv_graph_build_static(const int32_t* src, const int32_t* dst, int32_t n_edges,
                                     int32_t n_nodes, int32_t* row_ptr, int32_t* col, int32_t* perm,
                                     int32_t* t_row_ptr, int32_t* t_perm, int32_t* t_col, int32_t flags,
                                     hipStream_t stream) {
  if (n_nodes < 0 || n_edges < 0)
    return set_error(TP_ERR_ARG, "tp_conv_graph_build_static: negative size");
  if (n_edges > 0 && n_nodes == 0)
    return set_error(TP_ERR_ARG, "tp_conv_graph_build_static: edges need at least one node");
  if (!row_ptr || !t_row_ptr) return set_error(TP_ERR_ARG, "tp_conv_graph_build_static: NULL row pointer");
  if (n_edges > 0 && (!src || !dst || !col || !perm || !t_perm || !t_col))
    return set_error(TP_ERR_ARG, "tp_conv_graph_build_static: NULL edge array");
  const size_t need = tpc::graph_workspace_bytes(n_nodes, n_edges);
  if (need > TP_GRAPH_STATIC_SCRATCH_BYTES)
    return set_error(TP_ERR_WORKSPACE,
                     "tp_conv_graph_build_static: " + std::to_string(n_edges) + " edges need " +
                         std::to_string(need) + " bytes of scratch; the static scratch holds " +
                         std::to_string((size_t)TP_GRAPH_STATIC_SCRATCH_BYTES) +
                         " (use tp_conv_graph_build with a workspace)");
  return tpc::graph_build_static(src, dst, n_edges, n_nodes, row_ptr, col, perm, t_row_ptr, t_perm, t_col,
                                 flags, stream);
}

tp_status tp_conv_gather_rows(const void* in, const int32_t* perm, int64_t n_rows,
                              int64_t row_words, void* out, hipStream_t stream) {
  if (n_rows < 0 || row_words < 0) return set_error(TP_ERR_ARG, "tp_conv_gather_rows: negative size");
  if (n_rows > 0 && row_words > 0 && (!in || !perm || !out))
    return set_error(TP_ERR_ARG, "tp_conv_gather_rows: NULL pointer");
  if (n_rows > INT32_MAX) return set_error(TP_ERR_OVERFLOW, "tp_conv_gather_rows: too many rows");
  return tpc::gather_rows(in, perm, n_rows, row_words, out, stream);
}

tp_status tp_conv_sph_harm_backward(int32_t lmax, const float* r, int32_t n_edges, const float* grad_Y,
                                    const float* grad_rlen, float* grad_r, hipStream_t stream) {
  if (n_edges < 0) return set_error(TP_ERR_ARG, "tp_conv_sph_harm_backward: negative size");
  if (n_edges > 0 && (!r || !grad_Y || !grad_r))
    return set_error(TP_ERR_ARG, "tp_conv_sph_harm_backward: NULL pointer");
  return tpc::sph_harm_bwd(lmax, r, n_edges, grad_Y, grad_rlen, grad_r, stream);
}

tp_status tp_conv_sph_harm(int32_t lmax, const float* r, int32_t n_edges, float* Y,
                           hipStream_t stream) {
  if (n_edges < 0) return set_error(TP_ERR_ARG, "tp_conv_sph_harm: negative size");
  if (n_edges > 0 && (!r || !Y)) return set_error(TP_ERR_ARG, "tp_conv_sph_harm: NULL pointer");
  return tpc::sph_harm(lmax, r, n_edges, Y, stream);
}

static tp_status check_graph(const tp_graph* g, bool need_sender) {
  if (!g) return set_error(TP_ERR_ARG, "graph is NULL");
  if (g->n_nodes < 0 || g->n_edges < 0) return set_error(TP_ERR_ARG, "graph has a negative size");
  if (g->n_nodes > 0 && !g->row_ptr) return set_error(TP_ERR_ARG, "graph.row_ptr is NULL");
  if (g->n_edges > 0 && !g->col) return set_error(TP_ERR_ARG, "graph.col is NULL");
  if (need_sender && g->n_nodes > 0 && !g->t_row_ptr)
    return set_error(TP_ERR_ARG, "graph.t_row_ptr is NULL");
  if (need_sender && g->n_edges > 0 && (!g->t_perm || !g->t_col))
    return set_error(TP_ERR_ARG, "graph.t_perm / t_col is NULL");
  return TP_OK;
}

// Rows of x, w and grad_out are staged with 16-byte global->LDS loads (and
// node blocks of the channel mix are moved as 16-byte granules), so these
// pointers must be 16-byte aligned.
static bool misaligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15) return true;
  return false;
}

tp_status tp_conv_forward(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                          const float* w, float* out, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward: plan is NULL");
  tp_status s = check_graph(graph, false);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && (!x || !out)) return set_error(TP_ERR_ARG, "tp_conv_forward: x/out NULL");
  if (graph->n_edges > 0 && (!Y || !w)) return set_error(TP_ERR_ARG, "tp_conv_forward: Y/w NULL");
  if (misaligned16({x, w})) return set_error(TP_ERR_ARG, "tp_conv_forward: x and w must be 16-byte aligned");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.out = out;
  a.stream = stream;
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_forward: not a channel-wise CG plan");
  hipError_t e = plan->ks->fwd(a);
  return e == hipSuccess ? TP_OK : tpc::hip_error(e, "tp_conv_forward launch");
}

tp_status tp_conv_backward(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                           const float* w, const float* grad_out, float* grad_x, float* grad_Y,
                           float* grad_w, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward: plan is NULL");
  tp_status s = check_graph(graph, grad_x != nullptr);
  if (s != TP_OK) return s;
  const bool any_edge_grad = grad_Y || grad_w;
  if (graph->n_nodes > 0 && !grad_out) return set_error(TP_ERR_ARG, "tp_conv_backward: grad_out NULL");
  if (graph->n_edges > 0 && (!Y || !w)) return set_error(TP_ERR_ARG, "tp_conv_backward: Y/w NULL");
  if (graph->n_edges > 0 && any_edge_grad && !x)
    return set_error(TP_ERR_ARG, "tp_conv_backward: x NULL");
  if (misaligned16({x, w, grad_out}))
    return set_error(TP_ERR_ARG, "tp_conv_backward: x, w and grad_out must be 16-byte aligned");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.grad_out = grad_out;
  a.grad_x = grad_x;
  a.grad_Y = grad_Y;
  a.grad_w = grad_w;
  a.stream = stream;
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_backward: not a channel-wise CG plan");
  if (grad_x && any_edge_grad && graph->n_edges > 0 && plan->ks->bwd_fused) {
    // every gradient from one sender-grouped pass: w and Y are read once
    hipError_t e = plan->ks->bwd_fused(a);
    if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward fused pass");
    return TP_OK;
  }
  hipError_t e = plan->ks->bwd_recv(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward receiver pass");
  e = plan->ks->bwd_send(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward sender pass");
  return TP_OK;
}

tp_status tp_conv_graph_order_workspace(int32_t n_nodes, size_t* bytes) {
  if (n_nodes < 0 || !bytes) return set_error(TP_ERR_ARG, "tp_conv_graph_order_workspace: bad argument");
  *bytes = tpc::order_workspace_bytes(n_nodes);
  return TP_OK;
}

tp_status tp_conv_graph_launch_order(const tp_graph* graph, int32_t* order, int32_t* t_order, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  tp_status s = check_graph(graph, t_order != nullptr);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && !order && !t_order)
    return set_error(TP_ERR_ARG, "tp_conv_graph_launch_order: order and t_order both NULL");
  if (graph->n_nodes > 0 && (!ws || ws_bytes < tpc::order_workspace_bytes(graph->n_nodes)))
    return set_error(TP_ERR_WORKSPACE, "tp_conv_graph_launch_order: workspace missing or too small");
  return tpc::launch_order(graph->row_ptr, graph->t_row_ptr, graph->n_nodes, graph->n_edges, order, t_order, ws,
                           stream);
}

tp_status tp_conv_graph_sender_positions(const tp_graph* graph, int32_t* e_pos, hipStream_t stream) {
  tp_status s = check_graph(graph, true);
  if (s != TP_OK) return s;
  if (graph->n_edges > 0 && !e_pos) return set_error(TP_ERR_ARG, "tp_conv_graph_sender_positions: e_pos NULL");
  return tpc::sender_positions(graph->t_perm, graph->n_edges, e_pos, stream);
}

tp_status tp_conv_forward_sg(tp_plan_t plan, const tp_graph* graph, const int32_t* e_pos, const float* x,
                             const float* Y, const float* w, float* out, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward_sg: plan is NULL");
  tp_status s = check_graph(graph, false);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && (!x || !out)) return set_error(TP_ERR_ARG, "tp_conv_forward_sg: x/out NULL");
  if (graph->n_edges > 0 && (!Y || !w || !e_pos))
    return set_error(TP_ERR_ARG, "tp_conv_forward_sg: Y/w/e_pos NULL");
  if (misaligned16({x, w})) return set_error(TP_ERR_ARG, "tp_conv_forward_sg: x and w must be 16-byte aligned");
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_forward_sg: not a channel-wise CG plan");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.sender_rows = true;
  a.e_pos = e_pos;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.out = out;
  a.stream = stream;
  hipError_t e = plan->ks->fwd(a);
  return e == hipSuccess ? TP_OK : tpc::hip_error(e, "tp_conv_forward_sg launch");
}

tp_status tp_conv_backward_sg(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                              const float* w, const float* grad_out, float* grad_x, float* grad_Y,
                              float* grad_w, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward_sg: plan is NULL");
  tp_status s = check_graph(graph, true);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && !grad_out) return set_error(TP_ERR_ARG, "tp_conv_backward_sg: grad_out NULL");
  if (graph->n_edges > 0 && (!Y || !w || !x)) return set_error(TP_ERR_ARG, "tp_conv_backward_sg: x/Y/w NULL");
  if (misaligned16({x, w, grad_out}))
    return set_error(TP_ERR_ARG, "tp_conv_backward_sg: x, w and grad_out must be 16-byte aligned");
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_backward_sg: not a channel-wise CG plan");
  if (!plan->ks->bwd_fused)
    return set_error(TP_ERR_UNSUPPORTED, "tp_conv_backward_sg: this signature has no one-pass backward");
  if (!grad_x && !grad_Y && !grad_w) return TP_OK;
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_col = graph->t_col;
  a.sender_rows = true;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.grad_out = grad_out;
  a.grad_x = grad_x;
  a.grad_Y = grad_Y;
  a.grad_w = grad_w;
  a.stream = stream;
  hipError_t e = plan->ks->bwd_fused(a);
  return e == hipSuccess ? TP_OK : tpc::hip_error(e, "tp_conv_backward_sg launch");
}

tp_status tp_conv_forward_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                            const float* w, float* out, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward_r: plan is NULL");
  tp_status s = check_graph(graph, false);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && (!x || !out)) return set_error(TP_ERR_ARG, "tp_conv_forward_r: x/out NULL");
  if (graph->n_edges > 0 && (!r || !w)) return set_error(TP_ERR_ARG, "tp_conv_forward_r: r/w NULL");
  if (misaligned16({x, w})) return set_error(TP_ERR_ARG, "tp_conv_forward_r: x and w must be 16-byte aligned");
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_forward_r: not a channel-wise CG plan");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.x = x;
  a.r = r;
  a.w = w;
  a.out = out;
  a.stream = stream;
  hipError_t e = plan->ks->fwd_r(a);
  return e == hipSuccess ? TP_OK : tpc::hip_error(e, "tp_conv_forward_r launch");
}

tp_status tp_conv_backward_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                             const float* w, const float* grad_out, float* grad_x, float* grad_r,
                             float* grad_w, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward_r: plan is NULL");
  tp_status s = check_graph(graph, grad_x != nullptr);
  if (s != TP_OK) return s;
  if (graph->n_nodes > 0 && !grad_out) return set_error(TP_ERR_ARG, "tp_conv_backward_r: grad_out NULL");
  if (graph->n_edges > 0 && (!r || !w)) return set_error(TP_ERR_ARG, "tp_conv_backward_r: r/w NULL");
  if (graph->n_edges > 0 && (grad_r || grad_w) && !x)
    return set_error(TP_ERR_ARG, "tp_conv_backward_r: x NULL");
  if (misaligned16({x, w, grad_out}))
    return set_error(TP_ERR_ARG, "tp_conv_backward_r: x, w and grad_out must be 16-byte aligned");
  if (!plan->ks) return set_error(TP_ERR_UNSUPPORTED, "tp_conv_backward_r: not a channel-wise CG plan");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = graph->n_nodes;
  a.n_edges = graph->n_edges;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.r = r;
  a.w = w;
  a.grad_out = grad_out;
  a.grad_x = grad_x;
  a.grad_r = grad_r;
  a.grad_w = grad_w;
  a.stream = stream;
  hipError_t e = plan->ks->bwd_r(a);
  return e == hipSuccess ? TP_OK : tpc::hip_error(e, "tp_conv_backward_r launch");
}

tp_status tp_conv_double_backward(tp_plan_t plan, const tp_graph* graph, const float* x,
                                  const float* Y, const float* w, const float* grad_out,
                                  const float* gg_x, const float* gg_Y, const float* gg_w,
                                  float* d_x, float* d_Y, float* d_w, float* d_grad_out,
                                  hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_double_backward: plan is NULL");
  if (!plan->ks || !plan->ks->dbl_recv) return set_error(TP_ERR_UNSUPPORTED, "no compiled kernels");
  tp_status s = check_graph(graph, d_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && !grad_out && (d_x || d_Y || d_w))
    return set_error(TP_ERR_ARG, "tp_conv_double_backward: grad_out NULL");
  if (E > 0 && (!x || !Y || !w)) return set_error(TP_ERR_ARG, "tp_conv_double_backward: x/Y/w NULL");
  tpc::ConvArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.grad_out = grad_out;
  a.gg_x = gg_x;
  a.gg_Y = gg_Y;
  a.gg_w = gg_w;
  a.d_x = d_x;
  a.d_Y = d_Y;
  a.d_w = d_w;
  a.d_g = d_grad_out;
  a.stream = stream;
  hipError_t e = plan->ks->dbl_recv(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_double_backward receiver pass");
  e = plan->ks->dbl_send(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_double_backward sender pass");
  return TP_OK;
}

static const tpc::FcSet* find_fc(tp_plan_t plan, int n_radial) {
  if (plan->mode == TP_MODE_UVU && plan->ls == std::vector<int>{0, 1, 2} && plan->lmax_sh == 2 && plan->lmax_out == 2)
    return tpc::fc_l012_s2(plan->mul, n_radial);
  return nullptr;
}

tp_status tp_conv_fc_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_radial, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_fc_workspace: NULL argument");
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_fc_workspace: negative size");
  const tpc::FcSet* fs = find_fc(plan, n_radial);
  if (!fs)
    return set_error(TP_ERR_UNSUPPORTED, "no compiled fully connected kernel (supported: 0e+1o+2e / "
                                         "lmax 2 with 16, 32 or 64 channels and 8 radial features)");
  *bytes = fs->workspace(n_nodes);
  return TP_OK;
}

tp_status tp_conv_forward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                             const float* R, int32_t n_radial, const float* Theta, float* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward_fc: plan is NULL");
  size_t need = 0;
  tp_status s = tp_conv_fc_workspace(plan, graph ? graph->n_nodes : 0, n_radial, &need);
  if (s != TP_OK) return s;
  s = check_graph(graph, false);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && (!out || !Theta)) return set_error(TP_ERR_ARG, "tp_conv_forward_fc: out/Theta NULL");
  if (E > 0 && (!x || !Y || !R)) return set_error(TP_ERR_ARG, "tp_conv_forward_fc: x/Y/R NULL");
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, "tp_conv_forward_fc: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 15)
    return set_error(TP_ERR_ARG, "tp_conv_forward_fc: ws must be 16-byte aligned");
  tpc::FcArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.outdim = plan->outdim;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.x = x;
  a.Y = Y;
  a.R = R;
  a.Theta = Theta;
  a.out = out;
  a.ws = ws;
  a.stream = stream;
  hipError_t e = find_fc(plan, n_radial)->fwd(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_forward_fc launch");
  return TP_OK;
}

tp_status tp_conv_fc_backward_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_radial, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_fc_backward_workspace: NULL argument");
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_fc_backward_workspace: negative size");
  const tpc::FcSet* fs = find_fc(plan, n_radial);
  if (!fs || !fs->bwd_workspace)
    return set_error(TP_ERR_UNSUPPORTED, "no compiled fully connected kernel (supported: 0e+1o+2e / "
                                         "lmax 2 with 16, 32 or 64 channels and 8 radial features)");
  *bytes = fs->bwd_workspace(n_nodes);
  return TP_OK;
}

tp_status tp_conv_backward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                              const float* R, int32_t n_radial, const float* Theta, const float* grad_out,
                              float* grad_x, float* grad_Y, float* grad_R, float* grad_Theta, int32_t flags,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward_fc: plan is NULL");
  if (flags & ~TP_FC_STATE_SAVED) return set_error(TP_ERR_ARG, "tp_conv_backward_fc: unknown flags");
  size_t need = 0;
  tp_status s = tp_conv_fc_backward_workspace(plan, graph ? graph->n_nodes : 0, n_radial, &need);
  if (s != TP_OK) return s;
  s = check_graph(graph, grad_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && (!grad_out || !Theta)) return set_error(TP_ERR_ARG, "tp_conv_backward_fc: grad_out/Theta NULL");
  if (E > 0 && (!x || !Y || !R)) return set_error(TP_ERR_ARG, "tp_conv_backward_fc: x/Y/R NULL");
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, "tp_conv_backward_fc: workspace too small");
  if ((reinterpret_cast<uintptr_t>(ws) | reinterpret_cast<uintptr_t>(Theta)) & 15)
    return set_error(TP_ERR_ARG, "tp_conv_backward_fc: ws and Theta must be 16-byte aligned");
  tpc::FcArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.outdim = plan->outdim;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.R = R;
  a.Theta = Theta;
  a.gout = grad_out;
  a.grad_x = grad_x;
  a.grad_Y = grad_Y;
  a.grad_R = grad_R;
  a.grad_Theta = grad_Theta;
  a.state_saved = (flags & TP_FC_STATE_SAVED) != 0;
  a.ws = ws;
  a.stream = stream;
  hipError_t e = find_fc(plan, n_radial)->bwd(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward_fc launch");
  return TP_OK;
}

tp_status tp_conv_fc_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_edges, int32_t n_radial,
                                      size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_fc_double_workspace: NULL argument");
  if (n_nodes < 0 || n_edges < 0) return set_error(TP_ERR_ARG, "tp_conv_fc_double_workspace: negative size");
  const tpc::FcSet* fs = find_fc(plan, n_radial);
  if (!fs || !fs->dbl_workspace)
    return set_error(TP_ERR_UNSUPPORTED, "no compiled fully connected kernel (supported: 0e+1o+2e / "
                                         "lmax 2 with 16, 32 or 64 channels and 8 radial features)");
  *bytes = fs->dbl_workspace(n_nodes, n_edges);
  return TP_OK;
}

tp_status tp_conv_double_backward_fc(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                     const float* R, int32_t n_radial, const float* Theta,
                                     const float* grad_out, const float* gg_x, const float* gg_Y,
                                     const float* gg_R, const float* gg_Theta, float* d_x, float* d_Y,
                                     float* d_R, float* d_Theta, float* d_grad_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  const char* fn = "tp_conv_double_backward_fc";
  if (!plan) return set_error(TP_ERR_ARG, std::string(fn) + ": plan is NULL");
  size_t need = 0;
  tp_status s = tp_conv_fc_double_workspace(plan, graph ? graph->n_nodes : 0, graph ? graph->n_edges : 0,
                                            n_radial, &need);
  if (s != TP_OK) return s;
  s = check_graph(graph, d_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && (!grad_out || !Theta)) return set_error(TP_ERR_ARG, std::string(fn) + ": grad_out/Theta NULL");
  if (E > 0 && (!x || !Y || !R)) return set_error(TP_ERR_ARG, std::string(fn) + ": x/Y/R NULL");
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, std::string(fn) + ": workspace too small");
  if (misaligned16({ws, Theta, gg_Theta}))
    return set_error(TP_ERR_ARG, std::string(fn) + ": ws, Theta and gg_Theta must be 16-byte aligned");
  tpc::FcArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.outdim = plan->outdim;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.R = R;
  a.Theta = Theta;
  a.gout = grad_out;
  a.ws = ws;
  a.stream = stream;
  tpc::FcDbl d;
  d.gg_x = gg_x;
  d.gg_Y = gg_Y;
  d.gg_R = gg_R;
  d.gg_Theta = gg_Theta;
  d.d_x = d_x;
  d.d_Y = d_Y;
  d.d_R = d_R;
  d.d_Theta = d_Theta;
  d.d_g = d_grad_out;
  hipError_t e = find_fc(plan, n_radial)->dbl(a, d);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_double_backward_fc launch");
  return TP_OK;
}

// ---- Gaunt (spherical-grid) product -----------------------------------------
static tp_status gaunt_supported(tp_plan_t plan, const char* who) {
  const int m = plan->mul;
  if (std::string(who) != "tp_conv_plan_create" && plan->mode != TP_MODE_GAUNT)
    return set_error(TP_ERR_UNSUPPORTED, std::string(who) + ": plan was not created with TP_MODE_GAUNT");
  bool ok = (m == 16 || m == 32 || m == 64 || m == 128) && plan->lmax_sh <= 2 && plan->lmax_out <= 2 &&
            !plan->ls.empty() && plan->ls.size() <= 3;
  for (size_t a = 0; ok && a < plan->ls.size(); ++a) {
    if (plan->ls[a] > 2) ok = false;
    for (size_t b = 0; b < a; ++b)
      if (plan->ls[a] == plan->ls[b]) ok = false;
  }
  if (!ok)
    return set_error(TP_ERR_UNSUPPORTED, std::string(who) +
                                             ": the Gaunt product is compiled for distinct input degrees <= 2, "
                                             "lmax_sh and lmax_out <= 2, and 16, 32, 64 or 128 channels");
  return TP_OK;
}

tp_status tp_conv_gaunt_dims(tp_plan_t plan, int32_t* outdim, int32_t* wdim, int32_t* grid_points) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_gaunt_dims: plan is NULL");
  tp_status s = gaunt_supported(plan, "tp_conv_gaunt_dims");
  if (s != TP_OK) return s;
  if (outdim) *outdim = plan->mul * (plan->lmax_out + 1) * (plan->lmax_out + 1);
  if (wdim) *wdim = plan->mul * (plan->lmax_sh + 1);
  if (grid_points) *grid_points = tpc::gaunt_grid_points();
  return TP_OK;
}

tp_status tp_conv_forward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                const float* w, float* out, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward_gaunt: plan is NULL");
  tp_status s = gaunt_supported(plan, "tp_conv_forward_gaunt");
  if (s != TP_OK) return s;
  s = check_graph(graph, false);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && !out) return set_error(TP_ERR_ARG, "tp_conv_forward_gaunt: out NULL");
  if (E > 0 && (!x || !Y || !w)) return set_error(TP_ERR_ARG, "tp_conv_forward_gaunt: x/Y/w NULL");
  tpc::GauntArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.U = plan->mul;
  a.n_in = (int)plan->ls.size();
  for (int b = 0; b < a.n_in; ++b) a.deg[b] = plan->ls[b];
  a.lmax_sh = plan->lmax_sh;
  a.lmax_out = plan->lmax_out;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.out = out;
  a.stream = stream;
  hipError_t e = tpc::gaunt_forward(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_forward_gaunt launch");
  return TP_OK;
}

tp_status tp_conv_backward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                 const float* w, const float* grad_out, float* grad_x, float* grad_Y,
                                 float* grad_w, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward_gaunt: plan is NULL");
  tp_status s = gaunt_supported(plan, "tp_conv_backward_gaunt");
  if (s != TP_OK) return s;
  s = check_graph(graph, grad_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && !grad_out) return set_error(TP_ERR_ARG, "tp_conv_backward_gaunt: grad_out NULL");
  if (E > 0 && (!x || !Y || !w)) return set_error(TP_ERR_ARG, "tp_conv_backward_gaunt: x/Y/w NULL");
  if (reinterpret_cast<uintptr_t>(w) & 15)
    return set_error(TP_ERR_ARG, "tp_conv_backward_gaunt: w must be 16-byte aligned");
  tpc::GauntArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.U = plan->mul;
  a.n_in = (int)plan->ls.size();
  for (int b = 0; b < a.n_in; ++b) a.deg[b] = plan->ls[b];
  a.lmax_sh = plan->lmax_sh;
  a.lmax_out = plan->lmax_out;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.gout = grad_out;
  a.grad_x = grad_x;
  a.grad_Y = grad_Y;
  a.grad_w = grad_w;
  a.stream = stream;
  hipError_t e = tpc::gaunt_backward(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward_gaunt launch");
  return TP_OK;
}

static tpc::GauntArgs gaunt_args(tp_plan_t plan, const tp_graph* graph, int N, int E) {
  tpc::GauntArgs a;
  a.n_nodes = N;
  a.n_edges = E;
  a.U = plan->mul;
  a.n_in = (int)plan->ls.size();
  for (int b = 0; b < a.n_in; ++b) a.deg[b] = plan->ls[b];
  a.lmax_sh = plan->lmax_sh;
  a.lmax_out = plan->lmax_out;
  if (graph) {
    a.r_order = graph->order;
    a.s_order = graph->t_order;
    a.row_ptr = graph->row_ptr;
    a.col = graph->col;
    a.t_row_ptr = graph->t_row_ptr;
    a.t_perm = graph->t_perm;
    a.t_col = graph->t_col;
  }
  return a;
}

tp_status tp_conv_gaunt_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t n_edges, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_gaunt_double_workspace: NULL argument");
  tp_status s = gaunt_supported(plan, "tp_conv_gaunt_double_workspace");
  if (s != TP_OK) return s;
  if (n_nodes < 0 || n_edges < 0) return set_error(TP_ERR_ARG, "tp_conv_gaunt_double_workspace: negative size");
  *bytes = tpc::gaunt_double_workspace(gaunt_args(plan, nullptr, n_nodes, n_edges));
  return TP_OK;
}

tp_status tp_conv_double_backward_gaunt(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                        const float* w, const float* grad_out, const float* gg_x,
                                        const float* gg_Y, const float* gg_w, float* d_x, float* d_Y, float* d_w,
                                        float* d_grad_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "tp_conv_double_backward_gaunt";
  if (!plan) return set_error(TP_ERR_ARG, std::string(fn) + ": plan is NULL");
  tp_status s = gaunt_supported(plan, fn);
  if (s != TP_OK) return s;
  s = check_graph(graph, d_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && !grad_out) return set_error(TP_ERR_ARG, std::string(fn) + ": grad_out NULL");
  if (E > 0 && (!x || !Y || !w)) return set_error(TP_ERR_ARG, std::string(fn) + ": x/Y/w NULL");
  if (misaligned16({w, gg_w})) return set_error(TP_ERR_ARG, std::string(fn) + ": w and gg_w must be 16-byte aligned");
  tpc::GauntArgs a = gaunt_args(plan, graph, N, E);
  const size_t need = tpc::gaunt_double_workspace(a);
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, std::string(fn) + ": workspace too small");
  a.x = x;
  a.Y = Y;
  a.w = w;
  a.gout = grad_out;
  a.stream = stream;
  tpc::GauntDbl d;
  d.gg_x = gg_x;
  d.gg_Y = gg_Y;
  d.gg_w = gg_w;
  d.d_x = d_x;
  d.d_Y = d_Y;
  d.d_w = d_w;
  d.d_g = d_grad_out;
  d.ws = ws;
  hipError_t e = tpc::gaunt_double_backward(a, d);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_double_backward_gaunt launch");
  return TP_OK;
}

static tp_status need_uvw(tp_plan_t plan) {
  const int m = plan->mul;
  if (m > 128 || (m & (m - 1)) || m < 16 || plan->outs.size() > 8)
    return set_error(TP_ERR_UNSUPPORTED, "uvw mix needs a multiplicity of 16, 32, 64 or 128");
  return TP_OK;
}

tp_status tp_conv_uvw_workspace(tp_plan_t plan, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_uvw_workspace: NULL argument");
  tp_status s = need_uvw(plan);
  if (s != TP_OK) return s;
  *bytes = tpc::uvw_workspace_bytes(plan->uvw.n, plan->mul);
  return TP_OK;
}

tp_status tp_conv_uvw_forward(tp_plan_t plan, int32_t n_nodes, const float* Wmix, const float* in,
                              float* out, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_uvw_forward: plan is NULL");
  tp_status s = need_uvw(plan);
  if (s != TP_OK) return s;
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_uvw_forward: negative size");
  if (n_nodes > 0 && (!Wmix || !in || !out))
    return set_error(TP_ERR_ARG, "tp_conv_uvw_forward: NULL pointer");
  if (in == out) return set_error(TP_ERR_ARG, "tp_conv_uvw_forward: in and out must differ");
  if (misaligned16({in, out})) return set_error(TP_ERR_ARG, "tp_conv_uvw_forward: in and out must be 16-byte aligned");
  return tpc::uvw_forward(n_nodes, plan->mul, plan->outdim, plan->uvw, Wmix, in, out, false, stream);
}

tp_status tp_conv_uvw_backward(tp_plan_t plan, int32_t n_nodes, const float* Wmix, const float* in,
                               const float* grad_out, float* grad_in, float* grad_Wmix, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_uvw_backward: plan is NULL");
  tp_status s = need_uvw(plan);
  if (s != TP_OK) return s;
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_uvw_backward: negative size");
  if (n_nodes > 0 && (!Wmix || !grad_out)) return set_error(TP_ERR_ARG, "tp_conv_uvw_backward: NULL pointer");
  if (misaligned16({in, grad_out, grad_in}))
    return set_error(TP_ERR_ARG, "tp_conv_uvw_backward: in, grad_out and grad_in must be 16-byte aligned");
  if (grad_Wmix) {
    if (n_nodes > 0 && !in) return set_error(TP_ERR_ARG, "tp_conv_uvw_backward: in is NULL");
    if (!ws || ws_bytes < tpc::uvw_workspace_bytes(plan->uvw.n, plan->mul))
      return set_error(TP_ERR_WORKSPACE, "tp_conv_uvw_backward: workspace too small");
  }
  if (grad_in) {
    s = tpc::uvw_forward(n_nodes, plan->mul, plan->outdim, plan->uvw, Wmix, grad_out, grad_in, true,
                         stream);
    if (s != TP_OK) return s;
  }
  if (grad_Wmix) return tpc::uvw_grad_w(n_nodes, plan->mul, plan->outdim, plan->uvw, in, grad_out,
                                        grad_Wmix, ws, stream);
  return TP_OK;
}

// geom: Y holds the edge vectors r [E][3] and r_len is unused
static tp_status forward_radial_impl(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                     const float* r_len, const float* W1, const float* W2, const float* Wmix,
                                     float* out_pre, float* out, hipStream_t stream, bool geom) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_forward_radial: plan is NULL");
  if (!plan->rs) return set_error(TP_ERR_UNSUPPORTED, "plan has no radial network");
  tp_status s = check_graph(graph, false);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && (!x || !out)) return set_error(TP_ERR_ARG, "tp_conv_forward_radial: x/out NULL");
  if (E > 0 && (!Y || (!geom && !r_len) || !W1 || !W2))
    return set_error(TP_ERR_ARG, "tp_conv_forward_radial: Y (r) / r_len / W1 / W2 NULL");
  if (Wmix && N > 0 && (!out_pre || out_pre == out))
    return set_error(TP_ERR_ARG, "tp_conv_forward_radial: a mix needs a separate out_pre buffer");
  tpc::RadialArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.x = x;
  a.Y = Y;
  a.r_len = r_len;
  a.W1 = W1;
  a.W2 = W2;
  a.r_cut = plan->opts.r_cut;
  a.out = Wmix ? out_pre : out;
  a.geom = geom;
  a.stream = stream;
  hipError_t e = plan->rs->fwd(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_forward_radial launch");
  if (Wmix) {
    s = need_uvw(plan);
    if (s != TP_OK) return s;
    return tpc::uvw_forward(N, plan->mul, plan->outdim, plan->uvw, Wmix, out_pre, out, false, stream);
  }
  return TP_OK;
}

tp_status tp_conv_forward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                 const float* Y, const float* r_len, const float* W1,
                                 const float* W2, const float* Wmix, float* out_pre, float* out,
                                 hipStream_t stream) {
  return forward_radial_impl(plan, graph, x, Y, r_len, W1, W2, Wmix, out_pre, out, stream, false);
}

tp_status tp_conv_forward_radial_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                                   const float* W1, const float* W2, const float* Wmix, float* out_pre,
                                   float* out, hipStream_t stream) {
  return forward_radial_impl(plan, graph, x, r, nullptr, W1, W2, Wmix, out_pre, out, stream, true);
}

static size_t align_up(size_t b) { return (b + 255) & ~size_t(255); }

tp_status tp_conv_radial_workspace(tp_plan_t plan, int32_t n_nodes, int32_t with_mix, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_radial_workspace: NULL argument");
  if (!plan->rs || !plan->rs->bwd_workspace)
    return set_error(TP_ERR_UNSUPPORTED, "plan has no radial network");
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_radial_workspace: negative size");
  size_t b = plan->rs->bwd_workspace(n_nodes, 0);
  if (with_mix) {
    tp_status s = need_uvw(plan);
    if (s != TP_OK) return s;
    const size_t u = tpc::uvw_workspace_bytes(plan->uvw.n, plan->mul);
    b = align_up((size_t)n_nodes * plan->outdim * sizeof(float)) + (u > b ? u : b);
  }
  *bytes = b;
  return TP_OK;
}

// geom: Y holds the edge vectors r [E][3] (r_len unused) and grad_Y receives
// grad_r [E][3] (grad_rlen unused)
static tp_status backward_radial_impl(tp_plan_t plan, const tp_graph* graph, const float* x, const float* Y,
                                      const float* r_len, const float* W1, const float* W2,
                                      const float* Wmix, const float* out_pre, const float* grad_out,
                                      float* grad_x, float* grad_Y, float* grad_rlen, float* grad_W1,
                                      float* grad_W2, float* grad_Wmix, void* ws, size_t ws_bytes,
                                      hipStream_t stream, bool geom) {
  if (!plan) return set_error(TP_ERR_ARG, "tp_conv_backward_radial: plan is NULL");
  if (!plan->rs || !plan->rs->bwd) return set_error(TP_ERR_UNSUPPORTED, "plan has no radial network");
  tp_status s = check_graph(graph, grad_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && !grad_out) return set_error(TP_ERR_ARG, "tp_conv_backward_radial: grad_out NULL");
  if (!W1 || !W2) return set_error(TP_ERR_ARG, "tp_conv_backward_radial: W1/W2 NULL");
  if (E > 0 && (!x || !Y || (!geom && !r_len)))
    return set_error(TP_ERR_ARG, "tp_conv_backward_radial: x / Y (r) / r_len NULL");
  if (grad_Wmix && !Wmix) return set_error(TP_ERR_ARG, "tp_conv_backward_radial: grad_Wmix without Wmix");
  if (Wmix && grad_Wmix && N > 0 && !out_pre)
    return set_error(TP_ERR_ARG, "tp_conv_backward_radial: grad_Wmix needs out_pre");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(grad_out) |
       reinterpret_cast<uintptr_t>(W2)) & 15)
    return set_error(TP_ERR_ARG, "tp_conv_backward_radial: x, grad_out and W2 must be 16-byte aligned");
  size_t need = 0;
  s = tp_conv_radial_workspace(plan, N, Wmix != nullptr, &need);
  if (s != TP_OK) return s;
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, "tp_conv_backward_radial: workspace too small");
  char* w = static_cast<char*>(ws);
  const float* g = grad_out;
  if (Wmix) {
    float* gmix = reinterpret_cast<float*>(w);
    w += align_up((size_t)N * plan->outdim * sizeof(float));
    if (N > 0) {
      s = tpc::uvw_forward(N, plan->mul, plan->outdim, plan->uvw, Wmix, grad_out, gmix, true, stream);
      if (s != TP_OK) return s;
    }
    if (grad_Wmix) {
      s = tpc::uvw_grad_w(N, plan->mul, plan->outdim, plan->uvw, out_pre, grad_out, grad_Wmix, w, stream);
      if (s != TP_OK) return s;
    }
    g = gmix;
  }
  tpc::RadialArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.r_len = r_len;
  a.W1 = W1;
  a.W2 = W2;
  a.grad_out = g;
  a.grad_x = grad_x;
  a.grad_Y = grad_Y;
  a.grad_rlen = grad_rlen;
  a.grad_W1 = grad_W1;
  a.grad_W2 = grad_W2;
  a.r_cut = plan->opts.r_cut;
  a.geom = geom;
  a.ws = w;
  a.stream = stream;
  hipError_t e = plan->rs->bwd(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_backward_radial launch");
  return TP_OK;
}

tp_status tp_conv_backward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                  const float* Y, const float* r_len, const float* W1,
                                  const float* W2, const float* Wmix, const float* out_pre,
                                  const float* grad_out, float* grad_x, float* grad_Y,
                                  float* grad_rlen, float* grad_W1, float* grad_W2,
                                  float* grad_Wmix, void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_radial_impl(plan, graph, x, Y, r_len, W1, W2, Wmix, out_pre, grad_out, grad_x, grad_Y,
                              grad_rlen, grad_W1, grad_W2, grad_Wmix, ws, ws_bytes, stream, false);
}

tp_status tp_conv_backward_radial_r(tp_plan_t plan, const tp_graph* graph, const float* x, const float* r,
                                    const float* W1, const float* W2, const float* Wmix,
                                    const float* out_pre, const float* grad_out, float* grad_x,
                                    float* grad_r, float* grad_W1, float* grad_W2, float* grad_Wmix,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_radial_impl(plan, graph, x, r, nullptr, W1, W2, Wmix, out_pre, grad_out, grad_x, grad_r,
                              nullptr, grad_W1, grad_W2, grad_Wmix, ws, ws_bytes, stream, true);
}

tp_status tp_conv_radial_double_workspace(tp_plan_t plan, int32_t n_nodes, int32_t with_mix, size_t* bytes) {
  if (!plan || !bytes) return set_error(TP_ERR_ARG, "tp_conv_radial_double_workspace: NULL argument");
  if (!plan->rs) return set_error(TP_ERR_UNSUPPORTED, "plan has no radial network");
  if (!plan->rs->dbl_workspace)
    return set_error(TP_ERR_UNSUPPORTED, "no second-order radial kernels for this signature");
  if (n_nodes < 0) return set_error(TP_ERR_ARG, "tp_conv_radial_double_workspace: negative size");
  size_t b = plan->rs->dbl_workspace(n_nodes, 0);
  if (with_mix) {
    tp_status s = need_uvw(plan);
    if (s != TP_OK) return s;
    // unmixed upstream gradient and out_dot, then the kernels' or the mix's scratch
    const size_t u = tpc::uvw_workspace_bytes(plan->uvw.n, plan->mul);
    b = 2 * align_up((size_t)n_nodes * plan->outdim * sizeof(float)) + (u > b ? u : b);
  }
  *bytes = b;
  return TP_OK;
}

tp_status tp_conv_double_backward_radial(tp_plan_t plan, const tp_graph* graph, const float* x,
                                         const float* Y, const float* r_len, const float* W1,
                                         const float* W2, const float* Wmix, const float* grad_out,
                                         const float* gg_x, const float* gg_Y, const float* gg_rlen,
                                         float* d_x, float* d_Y, float* d_rlen, float* d_W1, float* d_W2,
                                         float* d_Wmix, float* d_grad_out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  const char* fn = "tp_conv_double_backward_radial";
  if (!plan) return set_error(TP_ERR_ARG, std::string(fn) + ": plan is NULL");
  if (!plan->rs) return set_error(TP_ERR_UNSUPPORTED, "plan has no radial network");
  if (!plan->rs->dbl)
    return set_error(TP_ERR_UNSUPPORTED, "no second-order radial kernels for this signature");
  tp_status s = check_graph(graph, d_x != nullptr);
  if (s != TP_OK) return s;
  const int N = graph->n_nodes, E = graph->n_edges;
  if (N > 0 && (!x || !grad_out)) return set_error(TP_ERR_ARG, std::string(fn) + ": x / grad_out NULL");
  if (!W1 || !W2) return set_error(TP_ERR_ARG, std::string(fn) + ": W1/W2 NULL");
  if (E > 0 && (!Y || !r_len)) return set_error(TP_ERR_ARG, std::string(fn) + ": Y / r_len NULL");
  if (d_Wmix && !Wmix) return set_error(TP_ERR_ARG, std::string(fn) + ": d_Wmix without Wmix");
  if (misaligned16({x, gg_x, grad_out, W2}))
    return set_error(TP_ERR_ARG, std::string(fn) + ": x, gg_x, grad_out and W2 must be 16-byte aligned");
  size_t need = 0;
  s = tp_conv_radial_double_workspace(plan, N, Wmix != nullptr, &need);
  if (s != TP_OK) return s;
  if (ws_bytes < need || (need > 0 && !ws))
    return set_error(TP_ERR_WORKSPACE, std::string(fn) + ": workspace too small");
  char* w = static_cast<char*>(ws);
  const float* g = grad_out;
  float* out_dot = d_grad_out;                   // without a mix, out_dot is d_grad_out itself
  if (Wmix) {
    s = need_uvw(plan);
    if (s != TP_OK) return s;
    float* gmix = reinterpret_cast<float*>(w);
    w += align_up((size_t)N * plan->outdim * sizeof(float));
    out_dot = (d_grad_out || d_Wmix) ? reinterpret_cast<float*>(w) : nullptr;
    w += align_up((size_t)N * plan->outdim * sizeof(float));
    if (N > 0) {
      s = tpc::uvw_forward(N, plan->mul, plan->outdim, plan->uvw, Wmix, grad_out, gmix, true, stream);
      if (s != TP_OK) return s;
    }
    g = gmix;
  }
  tpc::RadialArgs a;
  a.r_order = graph->order;
  a.s_order = graph->t_order;
  a.n_nodes = N;
  a.n_edges = E;
  a.row_ptr = graph->row_ptr;
  a.col = graph->col;
  a.t_row_ptr = graph->t_row_ptr;
  a.t_perm = graph->t_perm;
  a.t_col = graph->t_col;
  a.x = x;
  a.Y = Y;
  a.r_len = r_len;
  a.W1 = W1;
  a.W2 = W2;
  a.grad_out = g;
  a.gg_x = gg_x;
  a.gg_Y = gg_Y;
  a.gg_rlen = gg_rlen;
  a.out = out_dot;
  a.d_x = d_x;
  a.d_Y = d_Y;
  a.d_rlen = d_rlen;
  a.d_W1 = d_W1;
  a.d_W2 = d_W2;
  a.r_cut = plan->opts.r_cut;
  a.ws = w;
  a.stream = stream;
  hipError_t e = plan->rs->dbl(a);
  if (e != hipSuccess) return tpc::hip_error(e, "tp_conv_double_backward_radial launch");
  if (Wmix && N > 0) {
    if (d_grad_out) {
      s = tpc::uvw_forward(N, plan->mul, plan->outdim, plan->uvw, Wmix, out_dot, d_grad_out, false, stream);
      if (s != TP_OK) return s;
    }
    if (d_Wmix) {
      // the kernels' partial sums are consumed; their scratch is free again
      s = tpc::uvw_grad_w(N, plan->mul, plan->outdim, plan->uvw, out_dot, grad_out, d_Wmix, w, stream);
      if (s != TP_OK) return s;
    }
  }
  return TP_OK;
}

}  // extern "C"
