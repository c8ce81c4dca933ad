// Post-aggregation channel mix ("uvw"): one U x U matrix per output irrep k,
//   out2[i, k, v, c] = sum_u Wmix[k][u][v] out[i, k, u, c]
// and its adjoint.  The mix is a dense contraction and runs on fp32 MFMA
// (v_mfma_f32_16x16x4f32): for irrep k of degree l the node rows form a
// [U x N(2l+1)] matrix whose column (i, c) is out[i, k, :, c].
//
// A node's block of irrep k ([U][2l+1], U(2l+1) consecutive floats) is the
// unit of memory traffic: a workgroup copies the blocks of a group of nodes
// into LDS with gfx950's direct global->LDS loads (16 bytes per lane, one pad
// quad per node so that column reads spread over the banks), contracts them
// with the mixing matrix, stages the result in the same LDS buffer and writes
// whole node blocks back with 16-byte stores.  Each of the four waves keeps
// the A operands of its two 16-row tiles of the matrix in registers for the
// whole kernel.
//
// MFMA operand layout (16x16x4, wave64): lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and holds D[4(l/16)+i][l%16], i = 0..3.
//
// grad_Wmix[k] = sum over columns of out_col (x) g2_col: each workgroup sums
// its groups of nodes into a U x U partial held in registers (wave w owns
// row tiles w and w+4, all column tiles) and writes it to the workspace; a
// second kernel adds the partials in a fixed order (deterministic).
#include "conv_kernels.hpp"

namespace tpc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxU = 128;
constexpr int kMaxD = 7;              // 2l+1 for l <= 3
constexpr int kGroup = 16;            // nodes per group, mix
constexpr int kGroupG = 8;            // nodes per group, weight gradient (two operands staged)

// workgroups of one launch split over the irreps in proportion to 2l+1 (the
// work per node group): irrep k owns blocks start[k] .. start[k+1]-1
struct UvwSplit {
  int start[9];
};

__device__ __forceinline__ void split_of(const UvwSplit& sp, int nirr, int& k, int& b, int& nb) {
  k = 0;
  while (k + 1 < nirr && (int)blockIdx.x >= sp.start[k + 1]) ++k;
  b = blockIdx.x - sp.start[k];
  nb = sp.start[k + 1] - sp.start[k];
}

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Copy the irrep-k blocks of nodes n0 .. n0+NG-1 (ud floats each, from rows of
// `rowlen` floats starting at base) into LDS at a node stride of ud + 4 floats.
// Nodes past n_nodes are clamped to the last node (their values are not used).
template <int NG>
__device__ __forceinline__ void stage_nodes(float* lds, const float* __restrict__ base, int rowlen,
                                            int n0, int n_nodes, int ud, int wv, int lane) {
  const int qpn = ud / 4 + 1;                  // quads per node in LDS (one pad quad)
  const int total = NG * qpn;
  for (int blk = wv; blk * 64 < total; blk += 4) {
    const int q = blk * 64 + lane;
    if (q < total) {
      const int node = q / qpn, rem = q - node * qpn;
      const int n = n0 + node < n_nodes ? n0 + node : n_nodes - 1;
      const float* src = base + (size_t)n * rowlen + (rem < ud / 4 ? 4 * rem : 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(lds + blk * 256), 16, 0, 0);
    }
  }
}

// Z_k = A_k X_k per irrep k (grid.y); TRANS_W: A = Wmix_k (backward), else
// A = Wmix_k^T.  Workgroups walk groups of kGroup nodes.
template <bool TRANS_W>
__global__ void __launch_bounds__(256)
    k_uvw_apply(const float* __restrict__ W, const float* __restrict__ X, float* __restrict__ Z,
                int n_nodes, int U, int outdim, UvwIrreps irr, UvwSplit sp) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  int k, blk, nblk;
  split_of(sp, irr.n, k, blk, nblk);
  const int d = irr.dim[k], ko = irr.ko[k];
  const int ud = U * d, NS = ud + 4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int MT = U / 16, KS = U / 4;
  const float* Wk = W + (size_t)k * U * U;
  // A[m][kc] of row tiles wv and wv + 4: forward W[kc][m], backward W[m][kc]
  float a[2][kMaxU / 4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = 16 * (wv + 4 * t) + e16;
#pragma unroll
    for (int kk = 0; kk < kMaxU / 4; ++kk) {
      const int kc = 4 * kk + g;
      a[t][kk] = (wv + 4 * t < MT && kk < KS) ? (TRANS_W ? Wk[m * U + kc] : Wk[kc * U + m]) : 0.f;
    }
  }
  const float* base = X + (size_t)U * ko;
  for (int n0 = blk * kGroup; n0 < n_nodes; n0 += nblk * kGroup) {
    __syncthreads();                            // the previous group's LDS reads are done
    stage_nodes<kGroup>(lds, base, outdim, n0, n_nodes, ud, wv, lane);
    wait_vmcnt<0>();
    __syncthreads();
    f32x4 acc[kMaxD][2];
#pragma unroll
    for (int nt = 0; nt < kMaxD; ++nt) {
      acc[nt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt < d) {
        const int col = 16 * nt + e16;          // (node, component) of this lane's column
        const int node = col / d, c = col - node * d;
        const float* bcol = lds + node * NS + c + g * d;
#pragma unroll
        for (int kk = 0; kk < kMaxU / 4; ++kk) {
          if (kk < KS) {
            const float b = bcol[4 * kk * d];
            acc[nt][0] = mfma16(a[0][kk], b, acc[nt][0]);
            if (wv + 4 < MT) acc[nt][1] = mfma16(a[1][kk], b, acc[nt][1]);
          }
        }
      }
    }
    __syncthreads();                            // every wave has read the inputs
#pragma unroll
    for (int nt = 0; nt < kMaxD; ++nt) {
      if (nt < d) {
        const int col = 16 * nt + e16;
        const int node = col / d, c = col - node * d;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (wv + 4 * t < MT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int v = 16 * (wv + 4 * t) + 4 * g + i;
              lds[node * NS + v * d + c] = acc[nt][t][i];
            }
          }
        }
      }
    }
    __syncthreads();
    const int qn = ud / 4;
    for (int q = threadIdx.x; q < kGroup * qn; q += 256) {
      const int node = q / qn, rem = q - node * qn;
      const int n = n0 + node;
      if (n < n_nodes)
        *reinterpret_cast<float4*>(Z + (size_t)n * outdim + (size_t)U * ko + 4 * rem) =
            *reinterpret_cast<const float4*>(lds + node * NS + 4 * rem);
    }
  }
}

// Partial grad_Wmix: P_b[k][u][v] = sum over this workgroup's nodes and
// components of X[u][col] G[v][col].  Wave w owns row tiles w, w+4 (u) and
// every column tile (v).
__global__ void __launch_bounds__(256)
    k_uvw_gradw_partial(const float* __restrict__ X, const float* __restrict__ G,
                        float* __restrict__ part, int n_nodes, int U, int outdim, UvwIrreps irr,
                        UvwSplit sp) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  int k, blk, nblk;
  split_of(sp, irr.n, k, blk, nblk);
  const int d = irr.dim[k], ko = irr.ko[k];
  const int ud = U * d, NS = ud + 4;
  float* ldsX = lds;
  float* ldsG = lds + kGroupG * NS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int MT = U / 16;
  f32x4 acc[2][kMaxU / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nt = 0; nt < kMaxU / 16; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t off = (size_t)U * ko;
  for (int n0 = blk * kGroupG; n0 < n_nodes; n0 += nblk * kGroupG) {
    __syncthreads();
    stage_nodes<kGroupG>(ldsX, X + off, outdim, n0, n_nodes, ud, wv, lane);
    stage_nodes<kGroupG>(ldsG, G + off, outdim, n0, n_nodes, ud, wv, lane);
    wait_vmcnt<0>();
    __syncthreads();
    const int ks_n = 2 * d;                     // kGroupG * d columns, 4 per step
    for (int ks = 0; ks < ks_n; ++ks) {
      const int col = 4 * ks + g;
      const int node = col / d, c = col - node * d;
      const bool valid = n0 + node < n_nodes;
      const float* xc = ldsX + node * NS + c;
      const float* gc = ldsG + node * NS + c;
      float av[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        av[t] = (valid && wv + 4 * t < MT) ? xc[(16 * (wv + 4 * t) + e16) * d] : 0.f;
#pragma unroll
      for (int nt = 0; nt < kMaxU / 16; ++nt) {
        if (nt < MT) {
          const float b = gc[(16 * nt + e16) * d];
          acc[0][nt] = mfma16(av[0], b, acc[0][nt]);
          if (wv + 4 < MT) acc[1][nt] = mfma16(av[1], b, acc[1][nt]);
        }
      }
    }
  }
  float* P = part + (size_t)blockIdx.x * U * U;     // one U x U partial per workgroup
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mt = wv + 4 * t;
    if (mt >= MT) continue;
#pragma unroll
    for (int nt = 0; nt < kMaxU / 16; ++nt)
      if (nt < MT)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P[(size_t)(16 * mt + 4 * g + i) * U + 16 * nt + e16] = acc[t][nt][i];
  }
}

// grad_Wmix[k][e] = sum of the partials of irrep k's workgroups, in order.
__global__ void __launch_bounds__(256)
    k_sum_partials(const float* __restrict__ part, int UU, UvwSplit sp, float* __restrict__ out) {
  const int k = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= UU) return;
  // eight loads in flight at a time, added in block order
  float s = 0.f;
  int b = sp.start[k];
  for (; b + 8 <= sp.start[k + 1]; b += 8) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = part[(size_t)(b + j) * UU + e];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += q[j];
  }
  for (; b < sp.start[k + 1]; ++b) s += part[(size_t)b * UU + e];
  out[(size_t)k * UU + e] = s;
}

constexpr int kApplyBlocks = 1024;    // workgroups per launch (0.91 against 1.01 ms with 512 at 100k nodes)
constexpr int kGradWBlocks = 512;

// blocks per irrep proportional to 2l+1, at least one each and at most the
// number of node groups
UvwSplit make_split(const UvwIrreps& irr, int total, int groups) {
  int dsum = 0;
  for (int k = 0; k < irr.n; ++k) dsum += irr.dim[k];
  UvwSplit sp{};
  sp.start[0] = 0;
  for (int k = 0; k < irr.n; ++k) {
    int nb = (int)((long long)total * irr.dim[k] / dsum);
    nb = nb < 1 ? 1 : nb;
    nb = nb > groups ? (groups > 0 ? groups : 1) : nb;
    sp.start[k + 1] = sp.start[k] + nb;
  }
  return sp;
}

bool misaligned(const void* a, const void* b) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) != 0;
}

int max_dim(const UvwIrreps& irr) {
  int m = 1;
  for (int k = 0; k < irr.n; ++k) m = irr.dim[k] > m ? irr.dim[k] : m;
  return m;
}

}  // namespace

size_t uvw_workspace_bytes(int n_irreps, int U) {
  // make_split gives at most kGradWBlocks + n_irreps blocks (the floor of each share, at least one)
  return (size_t)(kGradWBlocks + n_irreps) * U * U * sizeof(float);
}

tp_status uvw_forward(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* W,
                      const float* X, float* Z, bool trans_w, hipStream_t st) {
  if (n_nodes == 0) return TP_OK;
  if (max_dim(irr) > kMaxD || U > kMaxU || U % 16) return set_error(TP_ERR_UNSUPPORTED, "uvw: shape");
  if (misaligned(X, Z)) return set_error(TP_ERR_ARG, "uvw: node arrays must be 16-byte aligned");
  const size_t lds = (size_t)kGroup * (U * max_dim(irr) + 4) * sizeof(float);
  const UvwSplit sp = make_split(irr, kApplyBlocks, (n_nodes + kGroup - 1) / kGroup);
  const dim3 grid((unsigned)sp.start[irr.n]);
  if (trans_w)
    hipLaunchKernelGGL(k_uvw_apply<true>, grid, dim3(256), lds, st, W, X, Z, n_nodes, U, outdim, irr, sp);
  else
    hipLaunchKernelGGL(k_uvw_apply<false>, grid, dim3(256), lds, st, W, X, Z, n_nodes, U, outdim, irr, sp);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "uvw apply launch");
}

tp_status uvw_grad_w(int n_nodes, int U, int outdim, const UvwIrreps& irr, const float* X,
                     const float* G, float* gradW, void* ws, hipStream_t st) {
  if (max_dim(irr) > kMaxD || U > kMaxU || U % 16) return set_error(TP_ERR_UNSUPPORTED, "uvw: shape");
  if (n_nodes > 0 && misaligned(X, G)) return set_error(TP_ERR_ARG, "uvw: node arrays must be 16-byte aligned");
  float* part = static_cast<float*>(ws);
  const size_t lds = (size_t)2 * kGroupG * (U * max_dim(irr) + 4) * sizeof(float);
  const UvwSplit sp = make_split(irr, kGradWBlocks, (n_nodes + kGroupG - 1) / kGroupG);
  hipLaunchKernelGGL(k_uvw_gradw_partial, dim3((unsigned)sp.start[irr.n]), dim3(256), lds, st, X, G, part,
                     n_nodes, U, outdim, irr, sp);
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((U * U + 255) / 256), irr.n), dim3(256), 0, st, part,
                     U * U, sp, gradW);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "uvw grad_W launch");
}

}  // namespace tpc
