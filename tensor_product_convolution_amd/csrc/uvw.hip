// Post-aggregation channel mix ("uvw"): one U x U matrix per output irrep k,
//   out2[i, k, v, c] = sum_u Wmix[k][u][v] out[i, k, u, c]
// and its adjoint.  The mix is a dense contraction, so it runs on fp32 MFMA
// (v_mfma_f32_16x16x4f32): for irrep k of degree l the node rows form a
// [U x N(2l+1)] matrix whose column (i, c) is out[i, k, :, c]; the product with
// Wmix_k^T (forward) or Wmix_k (backward) is tiled into 16-column tiles, one
// per wave, with the whole U x U matrix in LDS (64 KB for U = 128; row m is
// stored with its columns XOR-swizzled by 4*(m mod 16) to spread LDS banks).
//
// MFMA operand layout (16x16x4, wave64): lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and holds D[4(l/16)+i][l%16], i = 0..3.
//
// grad_Wmix[k] = sum over columns of out_col (x) g2_col is a reduction over
// N(2l+1) columns: every workgroup accumulates a partial U x U product for its
// share of columns in registers and writes it to the workspace; a second
// kernel sums the partials in a fixed order (deterministic).
#include "internal.hpp"

namespace tpc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxU = 128;
constexpr int kMaxMT = kMaxU / 16;

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Z_k = A_k X_k for each irrep k (grid.y), 16-column tiles strided over
// waves and workgroups.  TRANS_W: A = Wmix_k (backward), else A = Wmix_k^T.
template <bool TRANS_W>
__global__ void __launch_bounds__(256)
    k_uvw_apply(const float* __restrict__ W, const float* __restrict__ X, float* __restrict__ Z,
                int n_nodes, int U, int outdim, UvwIrreps irr) {
  extern __shared__ float As[];          // [U][U], swizzled
  const int k = blockIdx.y;
  const int d = irr.dim[k], ko = irr.ko[k];
  const float* Wk = W + (size_t)k * U * U;
  auto at = [U](int m, int kk) { return m * U + (kk ^ (((m & 15) << 2) & (U - 1))); };
  for (int t = threadIdx.x; t < U * U; t += blockDim.x) {
    const int r = t / U, c = t % U;      // W[r][c]
    if (TRANS_W) As[at(r, c)] = Wk[t];    // A[u][v] = W[u][v]
    else As[at(c, r)] = Wk[t];            // A[v][u] = W[u][v]
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int MT = U / 16;
  const long long ncols = (long long)n_nodes * d;
  const long long ntiles = (ncols + 15) / 16;
  for (long long tile = (long long)blockIdx.x * 4 + wv; tile < ntiles; tile += (long long)gridDim.x * 4) {
    const long long col = tile * 16 + (lane & 15);
    const bool valid = col < ncols;
    const long long i = valid ? col / d : 0;
    const int c = valid ? (int)(col - i * d) : 0;
    const float* xcol = X + i * outdim + (size_t)U * ko + c;
    f32x4 acc[kMaxMT];
#pragma unroll
    for (int mt = 0; mt < kMaxMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < U / 4; ++kk) {
      const int u = 4 * kk + (lane >> 4);
      const float b = valid ? xcol[(size_t)u * d] : 0.f;
#pragma unroll
      for (int mt = 0; mt < kMaxMT; ++mt)
        if (mt < MT) acc[mt] = mfma16(As[at(16 * mt + (lane & 15), u)], b, acc[mt]);
    }
    if (valid) {
      float* zcol = Z + i * outdim + (size_t)U * ko + c;
#pragma unroll
      for (int mt = 0; mt < kMaxMT; ++mt)
        if (mt < MT)
#pragma unroll
          for (int r = 0; r < 4; ++r) zcol[(size_t)(16 * mt + 4 * (lane >> 4) + r) * d] = acc[mt][r];
    }
  }
}

// Partial grad_Wmix: P_b[k][u][v] = sum over this workgroup's columns of
// X[u][col] G[v][col].  Wave w owns M-tiles w, w+4 (u) and every N-tile (v).
__global__ void __launch_bounds__(256)
    k_uvw_gradw_partial(const float* __restrict__ X, const float* __restrict__ G,
                        float* __restrict__ part, int n_nodes, int U, int outdim, UvwIrreps irr) {
  const int k = blockIdx.y;
  const int d = irr.dim[k], ko = irr.ko[k];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int MT = U / 16;
  const long long ncols = (long long)n_nodes * d;
  // contiguous column range of this workgroup, in steps of 4 columns
  const long long nsteps = (ncols + 3) / 4;
  const long long per = (nsteps + gridDim.x - 1) / gridDim.x;
  const long long s0 = (long long)blockIdx.x * per, s1 = s0 + per < nsteps ? s0 + per : nsteps;
  f32x4 acc[2][kMaxMT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < kMaxMT; ++nt) acc[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (long long s = s0; s < s1; ++s) {
    const long long col = 4 * s + (lane >> 4);
    const bool valid = col < ncols;
    const long long i = valid ? col / d : 0;
    const int c = valid ? (int)(col - i * d) : 0;
    const size_t base = (size_t)i * outdim + (size_t)U * ko + c;
    float a[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int mt = wv + 4 * t;
      a[t] = (valid && mt < MT) ? X[base + (size_t)(16 * mt + (lane & 15)) * d] : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < kMaxMT; ++nt) {
      if (nt < MT) {
        const float b = valid ? G[base + (size_t)(16 * nt + (lane & 15)) * d] : 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (wv + 4 * t < MT) acc[t][nt] = mfma16(a[t], b, acc[t][nt]);
      }
    }
  }
  float* P = part + ((size_t)blockIdx.x * irr.n + k) * U * U;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mt = wv + 4 * t;
    if (mt >= MT) continue;
#pragma unroll
    for (int nt = 0; nt < kMaxMT; ++nt)
      if (nt < MT)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          P[(size_t)(16 * mt + 4 * (lane >> 4) + r) * U + 16 * nt + (lane & 15)] = acc[t][nt][r];
  }
}

// grad_Wmix[k][e] = sum_b part[b][k][e], fixed order over b.
__global__ void __launch_bounds__(256)
    k_sum_partials(const float* __restrict__ part, int nparts, long long n, float* __restrict__ out) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int b = 0; b < nparts; ++b) s += part[(size_t)b * n + e];
  out[e] = s;
}

constexpr int kGradWBlocks = 256;

}  // namespace

size_t uvw_workspace_bytes(int n_irreps, int U) {
  return (size_t)kGradWBlocks * n_irreps * U * U * sizeof(float);
}

tp_status uvw_forward(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* W,
                      const float* X, float* Z, bool trans_w, hipStream_t st) {
  if (n_nodes == 0) return TP_OK;
  const size_t lds = (size_t)U * U * sizeof(float);
  const long long maxcols = (long long)n_nodes * 7;
  long long gx = (maxcols / 16 + 3) / 4;
  if (gx > 512) gx = 512;
  if (gx < 1) gx = 1;
  const dim3 grid((unsigned)gx, irr.n);
  if (trans_w)
    hipLaunchKernelGGL(k_uvw_apply<true>, grid, dim3(256), lds, st, W, X, Z, n_nodes, U, outdim, irr);
  else
    hipLaunchKernelGGL(k_uvw_apply<false>, grid, dim3(256), lds, st, W, X, Z, n_nodes, U, outdim, irr);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "uvw apply launch");
}

tp_status uvw_grad_w(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* X,
                     const float* G, float* gradW, void* ws, hipStream_t st) {
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(k_uvw_gradw_partial, dim3(kGradWBlocks, irr.n), dim3(256), 0, st, X, G, part,
                     n_nodes, U, outdim, irr);
  const long long n = (long long)irr.n * U * U;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     kGradWBlocks, n, gradW);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "uvw grad_W launch");
}

}  // namespace tpc
