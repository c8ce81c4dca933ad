// Convolution with fully connected per-edge weights, by reassociation
// ("Sobek: Streaming Equivariant Tensor Product Convolutions", Abstract:
// radial projection, harmonic coupling and aggregation are reassociated so
// that edge-local products go straight into bounded receiver-side state;
// fully connected multiplicity mixing is preserved).
//
//   W_e[p, u, v] = sum_h R_e[h] Theta[h, p, u, v]          (never formed)
//   out[i, k, v, c] = sum_{e into i} sum_{p->k} sum_u W_e[p, u, v] T_p(x_j[u], Y_e)[c]
//                   = sum_{h, p->k, u} Theta[h, p, u, v] S_i[h, p, u, c]
//   S_i[h, p, u, c] = sum_{e into i} R_e[h] T_p(x_j[u], Y_e)[c]
//
// Phase 1 (k_fc_state) streams each receiver's edges into S_i: per 16-edge
// tile the lanes form the CG terms T of their edges (VALU, compile-time
// nonzeros) and MFMA accumulates R^T T (M = hidden units, N = 16 channels,
// K = edges).  S is node-sized (no edge-sized array is written) and is laid
// out per output irrep k as rows (i, c) of length K_k = H |P_k| U, ordered
// (h, path of k, u).  Phase 2 (k_fc_contract) is then a dense product per
// irrep, out_k[(i,c)][v] = sum_K S_k[(i,c)][K] Theta_k[K][v], on MFMA.
// MFMA operand layout (16x16x4 f32, wave64): lane l supplies A[l%16][l/16],
// B[l/16][l%16] and holds D[4(l/16)+i][l%16].
#include "radial_kernels.hpp"

namespace tpc {

// per-plan constants of the state layout (host-filled)
struct FcLayout {
  int n_out;                  // output irreps
  long long base[8];          // float offset of S_k
  int d3[8], npk[8], ko[8];   // 2l+1, paths into k, per-channel output offset
  int pg[8][8];               // global path index of the p-th path into k
};

namespace {

// position of path P among the paths into its output irrep
template <class S>
constexpr int path_local(int p) {
  int n = 0;
  for (int q = 0; q < p; ++q)
    if (S::paths.p[q].k == S::paths.p[p].k) ++n;
  return n;
}
template <class S>
constexpr int paths_into(int k) {
  int n = 0;
  for (int q = 0; q < S::NP; ++q)
    if (S::paths.p[q].k == k) ++n;
  return n;
}
// output components of paths [P0, P0 + N)
template <class S>
constexpr int comps(int p0, int n) {
  int t = 0;
  for (int q = p0; q < p0 + n; ++q) t += 2 * S::paths.p[q].l3 + 1;
  return t;
}
template <class S>
constexpr int comp_off(int p0, int p) { return comps<S>(p0, p - p0); }

// contiguous path groups of about equal output-component counts (one group
// per wave of the state kernel)
template <class S, int NG>
struct PathGroups {
  int start[NG + 1];
};
template <class S, int NG>
constexpr PathGroups<S, NG> make_groups() {
  PathGroups<S, NG> g{};
  const int total = comps<S>(0, S::NP);
  int p = 0;
  for (int k = 0; k < NG; ++k) {
    g.start[k] = p;
    const int target = (total * (k + 1) + NG - 1) / NG;
    while (p < S::NP && (k == NG - 1 || comps<S>(0, p + 1) <= target)) ++p;
  }
  g.start[NG] = S::NP;
  return g;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Phase 1.  One workgroup (4 waves) per receiver; wave w owns path group w.
// v_mfma_f32_4x4x1_16b_f32 (16 independent 4 x 4 blocks, K = 1): block b =
// lane / 4 takes A[i] from lane 4b + i, B[j] from lane 4b + j and keeps
// D[i][j] in lane 4b + j, register i.  Lane l = (edge class l / U, channel
// l % U); its block's rows are four of the H = 8 radial features (two
// instructions per term: features 0-3 and 4-7), its columns four channels of
// the same edge.  So each instruction adds R_e[h] T_e[u] for 64 / U edges x
// U channels x 4 features with no idle rows, and the edge classes are summed
// across lanes once at the end.  The receiver's sender indices, Y rows and R
// rows are staged in LDS; x channels are gathered per step, software-
// pipelined (the next step's gathers in flight during this step's arithmetic:
// 9 registers, where gathering two steps before computing them cost more
// occupancy than it hid).
template <class S, int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_state(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
               const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ R,
               float* __restrict__ Sbuf, FcLayout lay, const int32_t* __restrict__ order) {
  constexpr int EPI = 64 / U;                      // edges per instruction (edge classes)
  constexpr int NG = 4;
  constexpr int CH = 128;                          // edges staged in LDS at a time
  static_assert(H == 8 && (U == 16 || U == 32 || U == 64), "fc state tiling");
  constexpr PathGroups<S, NG> PG = make_groups<S, NG>();
  __shared__ int cs[CH];
  __shared__ float ys[CH * S::YC];
  __shared__ float rs[CH * H];
  // node of this workgroup in the launch order (largest degree first), or node order
  const int i = order ? min(max(order[blockIdx.x], 0), n_nodes - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int grp = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ec = lane / U, u = lane % U, p4 = lane % 4;
  static_for<NG>([&](auto G) {
    if (grp != G) return;
    constexpr int P0 = PG.start[G], NPP = PG.start[G + 1] - P0;
    constexpr int NT = comps<S>(P0, NPP);
    v4f acc[NT][2];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k][0] = acc[k][1] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int c0 = beg; c0 < end; c0 += CH) {
      const int cn = end - c0 < CH ? end - c0 : CH;
      __syncthreads();
      for (int k = t; k < cn; k += 256) cs[k] = col[c0 + k];
      for (int k = t; k < cn * S::YC; k += 256) ys[k] = Y[(size_t)c0 * S::YC + k];
      for (int k = t; k < cn * H; k += 256) rs[k] = R[(size_t)c0 * H + k];
      __syncthreads();
      auto xload = [&](int s0, float (&xr)[S::XC]) {
        const int e = s0 * EPI + ec;
        load_x_channel<S, U>(x, cs[e < cn ? e : cn - 1], u, xr);
      };
      auto step = [&](int s0, const float (&xr)[S::XC]) {
        const int e = s0 * EPI + ec;
        const bool ok = e < cn;
        const int ee = ok ? e : cn - 1;
        float yr[S::YC];
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = ys[ee * S::YC + b];
        const float a0 = ok ? rs[ee * H + p4] : 0.f, a1 = ok ? rs[ee * H + 4 + p4] : 0.f;
        float tv[NT];
        static_for<NPP>([&](auto PP) {
          constexpr PathInfo pi = S::paths.p[P0 + PP];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P0 + PP);
          static_for<D3>([&](auto C) { tv[OFF + C] = 0.f; });
          static_for<T::nnz>([&](auto N) {
            constexpr Nz z = T::table.e[N];
            tv[OFF + z.c] = fmaf(z.v, xr[pi.xo + z.a] * yr[pi.yo + z.b], tv[OFF + z.c]);
          });
        });
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          acc[k][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, tv[k], acc[k][0], 0, 0, 0);
          acc[k][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, tv[k], acc[k][1], 0, 0, 0);
        }
      };
      // the next step's gathers are issued before this step's arithmetic
      float xa[S::XC], xb[S::XC];
      xload(0, xa);
      for (int s0 = 0; s0 * EPI < cn; s0 += 2) {
        xload(s0 + 1, xb);
        __builtin_amdgcn_sched_barrier(0);
        step(s0, xa);
        if ((s0 + 1) * EPI >= cn) break;
        xload(s0 + 2, xa);
        __builtin_amdgcn_sched_barrier(0);
        step(s0 + 1, xb);
      }
    }
    // sum the edge classes (lanes u, u + U, ...), then lanes of class 0 store
    // S_k[(i, c)][(h, path of k, u)] for h = 4 half + row
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int off = U; off < 64; off <<= 1) acc[k][hf][r] += __shfl_xor(acc[k][hf][r], off, 64);
    if (ec == 0) {
      static_for<NPP>([&](auto PP) {
        constexpr int P = P0 + PP;
        constexpr PathInfo pi = S::paths.p[P];
        constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P);
        constexpr int NPK = paths_into<S>(pi.k), PL = path_local<S>(P);
        constexpr int KK = H * NPK * U;
        float* Sk = Sbuf + lay.base[pi.k] + (size_t)i * D3 * KK;
        static_for<D3>([&](auto C) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Sk[(size_t)C * KK + (size_t)((4 * hf + r) * NPK + PL) * U + u] = acc[OFF + C][hf][r];
        });
      });
    }
  });
}

// Phase 2.  One workgroup (kCW waves) per kRT tiles of 16 rows (i, c) of one
// output irrep; the waves split the contraction length K_k (wave = radial
// feature h) and meet in LDS.
// Within a wave, lane group l/16 takes four consecutive K per four MFMA steps
// (the order of a sum over K is free), so each lane reads its row with one
// 16-byte load per four steps.  Rows of all irreps are enumerated irrep by
// irrep (blockIdx.x).
// TRANS: the product with Theta transposed in its two channel indices (the
// backward's grad_x, whose state rows carry output channels v and whose
// columns are input channels u).
constexpr int kCW = 8;   // waves per contraction workgroup (each a slice of K)
// 16-row tiles per workgroup, which share every Theta operand load (one tile
// per workgroup spent most of its time loading Theta: 71.9 -> 68.5 us for the
// forward, 87.7 -> 81.7 us for grad_x with two)
constexpr int kRT = 2;
template <int U, int H, bool TRANS>
__global__ void __launch_bounds__(64 * kCW)
    k_fc_contract(int n_nodes, const float* __restrict__ Sbuf, const float* __restrict__ Theta, int P,
                  int outdim, float* __restrict__ out, FcLayout lay) {
  constexpr int NV = U / 16, TR = 16 * kRT;
  __shared__ float red[kCW - 1][kRT][NV][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  int k = 0, first = 0;
  while (k + 1 < lay.n_out && (int)blockIdx.x >= first + (n_nodes * lay.d3[k] + TR - 1) / TR) {
    first += (n_nodes * lay.d3[k] + TR - 1) / TR;
    ++k;
  }
  const int d3 = lay.d3[k], npk = lay.npk[k];
  const int KK = H * npk * U;                       // a multiple of 8 U
  const int rows = n_nodes * d3;
  const int row0 = ((int)blockIdx.x - first) * TR;
  const float* arow[kRT];
  bool va[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int ra = row0 + 16 * rt + e16;             // this lane's A row in tile rt
    va[rt] = ra < rows;
    arow[rt] = Sbuf + lay.base[k] + (size_t)(va[rt] ? ra : rows - 1) * KK;
  }
  const int kq = KK / kCW;                           // this wave's share of K
  const int K0 = wv * kq;
  f32x4 acc[kRT][NV];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  static_assert(H % kCW == 0, "whole (h, path) blocks per wave");
  for (int t = K0 / U; t < (K0 + kq) / U; ++t) {
    const int pl = t % npk, h = t / npk;
    constexpr int RS = TRANS ? 1 : U, CS = TRANS ? U : 1;
    const float* thb = Theta + ((size_t)h * P + lay.pg[k][pl]) * U * U + e16 * CS;
#pragma unroll
    for (int ub = 0; ub < U; ub += 16) {
      float av[kRT][4];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const float4 a4 = *reinterpret_cast<const float4*>(arow[rt] + (size_t)t * U + 4 * g + ub);
        av[rt][0] = va[rt] ? a4.x : 0.f;
        av[rt][1] = va[rt] ? a4.y : 0.f;
        av[rt][2] = va[rt] ? a4.z : 0.f;
        av[rt][3] = va[rt] ? a4.w : 0.f;
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float* th = thb + (size_t)(ub + 4 * g + st) * RS;
        float tv[NV];
#pragma unroll
        for (int n = 0; n < NV; ++n) tv[n] = th[16 * n * CS];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
          for (int n = 0; n < NV; ++n) acc[rt][n] = mfma_16x16x4(av[rt][st], tv[n], acc[rt][n]);
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wv - 1][rt][n][r][lane] = acc[rt][n][r];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = acc[rt][n][r];
#pragma unroll
          for (int w2 = 0; w2 < kCW - 1; ++w2) a += red[w2][rt][n][r][lane];
          acc[rt][n][r] = a;
        }
      // D[row 4g + r][v = 16n + l%16] of tile rt
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * rt + 4 * g + r;
        if (row < rows) {
          const int node = row / d3, c = row - node * d3;
          float* o = out + (size_t)node * outdim + (size_t)U * lay.ko[k] + c;
#pragma unroll
          for (int n = 0; n < NV; ++n) o[(size_t)(16 * n + e16) * d3] = acc[rt][n][r];
        }
      }
    }
  }
}

// ---- backward ----------------------------------------------------------------
// With gS_i[h,p,u,c] = sum_v Theta[h,p,u,v] gout_i[k(p),v,c] (the state's
// gradient) and T_e the forward's CG terms:
//   grad_Theta[h,p,u,v] = sum_{i,c} S_i[h,p,u,c] gout_i[k,v,c]            (k_fc_gradtheta)
//   grad_R[e][h]        = sum_{p,u,c} gS_i[h,p,u,c] T_e[p,u,c]             (k_fc_bwd_recv)
//   grad_Y[e]           = CG adjoint of T with gT_e = sum_h R_e[h] gS_i     (k_fc_bwd_recv)
//   grad_x[j][u][a]     = sum_{h,p,v} Theta[h,p,u,v] Q_j[h,p,v,a],
//   Q_j[h,p,v,a]        = sum_{e = (j -> i)} R_e[h] sum_{b,c} C_p[a,b,c] Y_e[b] gout_i[k,v,c]
// The last is the forward's reassociation mirrored onto the sender side: Q is
// a sender-side state (k_fc_bwd_send, on the same 4x4x1 products) followed by
// the dense contraction with Theta transposed (k_fc_contract<TRANS>).  No
// per-edge weight matrix or message is formed.

// gS_k[(i,c)][(h,pl,u)] = sum_v gout[i][k][v][c] Theta[h,pg,u,v]: one
// workgroup per 16-row tile of one output irrep, its waves taking column
// tiles in turn; A = the tile's gout rows (K = v), B = Theta.
template <int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_expand(int n_nodes, const float* __restrict__ gout, const float* __restrict__ Theta, int P,
                int outdim, float* __restrict__ gS, FcLayout lay) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  int k = 0, first = 0;
  while (k + 1 < lay.n_out && (int)blockIdx.x >= first + (n_nodes * lay.d3[k] + 15) / 16) {
    first += (n_nodes * lay.d3[k] + 15) / 16;
    ++k;
  }
  const int d3 = lay.d3[k], npk = lay.npk[k];
  const int KK = H * npk * U, rows = n_nodes * d3;
  const int row0 = ((int)blockIdx.x - first) * 16;
  const int ra = row0 + e16;
  const bool va = ra < rows;
  const int node = (va ? ra : rows - 1) / d3, c = (va ? ra : rows - 1) % d3;
  // K order (free for a sum): step ks feeds lane group g the channel
  // v = 16 (ks / 4) + 4 g + ks % 4, so each lane reads Theta as 16-byte rows
  // A[row e16][v]
  float av[U / 4];
#pragma unroll
  for (int ks = 0; ks < U / 4; ++ks) {
    const int v = 16 * (ks / 4) + 4 * g + ks % 4;
    av[ks] = va ? gout[(size_t)node * outdim + (size_t)U * lay.ko[k] + v * d3 + c] : 0.f;
  }
  // this wave's column tiles ct = wv + 4 m, four at a time: their Theta
  // operands are all loaded before the products (tiles past the end re-read
  // the last one and are not stored)
  constexpr int CB = 4;
  const int nct = KK / 16;
  for (int c0 = wv; c0 < nct; c0 += 4 * CB) {
    float bv[CB][U / 4];
#pragma unroll
    for (int q = 0; q < CB; ++q) {
      // columns K = 16 ct + e16 = (h npk + pl) U + uu; a 16-block shares (h, pl)
      const int ct = c0 + 4 * q < nct ? c0 + 4 * q : nct - 1;
      const int t = (16 * ct) / U, uu = (16 * ct) % U + e16;
      const int pl = t % npk, h = t / npk;
      const float4* th = reinterpret_cast<const float4*>(Theta + (((size_t)h * P + lay.pg[k][pl]) * U + uu) * U);
#pragma unroll
      for (int b4 = 0; b4 < U / 16; ++b4) {
        const float4 t4 = th[4 * b4 + g];   // v = 16 b4 + 4 g .. + 3
        bv[q][4 * b4] = t4.x;
        bv[q][4 * b4 + 1] = t4.y;
        bv[q][4 * b4 + 2] = t4.z;
        bv[q][4 * b4 + 3] = t4.w;
      }
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) {
      const int ct = c0 + 4 * q;
      if (ct >= nct) break;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < U / 4; ++ks) acc = mfma_16x16x4(av[ks], bv[q][ks], acc);
      // D[row 4g + r][column e16]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 4 * g + r;
        if (row < rows) gS[lay.base[k] + (size_t)row * KK + 16 * ct + e16] = acc[r];
      }
    }
  }
}

// Partial sums of grad_Theta_k[K][v] = sum_rows S_k[row][K] gout_k[row][v]
// over a block of kRowBlock rows: one wave per 16-column K tile (M = K, N = v,
// the sum over rows as K = 4 per product).  part_k[block][K][v].
constexpr int kRowBlock = 256;
template <int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_gradtheta(int n_nodes, const float* __restrict__ Sbuf, const float* __restrict__ gout, int outdim,
                   float* __restrict__ part, FcLayout lay, FcLayout plan_part) {
  constexpr int NV = U / 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  // blocks: irrep by irrep, then (row block, group of four K tiles)
  int k = 0, first = 0;
  auto nblk = [&](int kk) {
    const int rows = n_nodes * lay.d3[kk];
    return ((rows + kRowBlock - 1) / kRowBlock) * ((H * lay.npk[kk] * U / 16 + 3) / 4);
  };
  while (k + 1 < lay.n_out && (int)blockIdx.x >= first + nblk(k)) {
    first += nblk(k);
    ++k;
  }
  const int d3 = lay.d3[k], npk = lay.npk[k];
  const int KK = H * npk * U, rows = n_nodes * d3;
  const int nkq = (KK / 16 + 3) / 4;
  const int b = (int)blockIdx.x - first;
  const int rb = b / nkq, kt = (b % nkq) * 4 + wv;
  if (kt >= KK / 16) return;
  const int K0 = 16 * kt;
  f32x4 acc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r_end = min(rows, (rb + 1) * kRowBlock);
  // this lane's row r = (node, c), advanced by four rows per step without a division
  int r = rb * kRowBlock + g;
  int node = r / d3, c = r - node * d3;
  const int q4 = 4 / d3, m4 = 4 - q4 * d3;
  // kGtBatch steps per batch: every load of the batch is issued (rows past the
  // block's end re-read a valid row and are replaced by zero) before its
  // products, so the wave waits once per batch rather than once per step
  constexpr int kGtBatch = 8;
  const float* Sk = Sbuf + lay.base[k] + K0 + e16;
  const float* gk = gout + (size_t)U * lay.ko[k] + (size_t)e16 * d3;
  for (int r0 = rb * kRowBlock; r0 < r_end; r0 += 4 * kGtBatch) {
    float a[kGtBatch], gv[kGtBatch][NV];
#pragma unroll
    for (int s = 0; s < kGtBatch; ++s) {
      const bool ok = r < r_end;
      const float* gr = gk + (size_t)(ok ? node : 0) * outdim + (ok ? c : 0);
      const float av = Sk[(size_t)(ok ? r : r_end - 1) * KK];
      a[s] = ok ? av : 0.f;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const float gvn = gr[16 * n * d3];
        gv[s][n] = ok ? gvn : 0.f;
      }
      r += 4;
      node += q4;
      c += m4;
      if (c >= d3) {
        c -= d3;
        ++node;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kGtBatch; ++s)
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[n] = mfma_16x16x4(a[s], gv[s][n], acc[n]);
  }
  // D[K = K0 + 4g + r][v = 16 n + e16]
  float* pk = part + plan_part.base[k] + (size_t)rb * KK * U;
#pragma unroll
  for (int n = 0; n < NV; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) pk[(size_t)(K0 + 4 * g + r) * U + 16 * n + e16] = acc[n][r];
}

// output irrep and position among that irrep's paths, per path
struct PathMap {
  int k[16], pl[16];
};

// grad_Theta[h][p][u][v] = sum over row blocks of part_k[block][(h npk + pl) U + u][v]
template <int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_gradtheta_sum(int n_nodes, const float* __restrict__ part, int P, float* __restrict__ gTheta,
                       FcLayout lay, FcLayout plan_part, PathMap pm) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= H * P * U * U) return;
  const int v = idx % U, u = (idx / U) % U, p = (idx / (U * U)) % P, h = idx / (U * U * P);
  const int k = pm.k[p], pl = pm.pl[p];
  const int KK = H * lay.npk[k] * U;
  const int nrb = (n_nodes * lay.d3[k] + kRowBlock - 1) / kRowBlock;
  const float* pk = part + plan_part.base[k] + (size_t)((h * lay.npk[k] + pl) * U + u) * U + v;
  const size_t stride = (size_t)KK * U;
  // eight independent loads in flight per step (partials of blocks rb, rb + 1,
  // ... summed in block order, so the result does not depend on the grouping
  // of the loads)
  float a = 0.f;
  int rb = 0;
  for (; rb + 8 <= nrb; rb += 8) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = pk[(rb + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) a += q[j];
  }
  for (; rb < nrb; ++rb) a += pk[rb * stride];
  gTheta[idx] = a;
}

// Receiver pass: grad_R and grad_Y.  One workgroup per receiver, one wave per
// path group (as the state kernel); the receiver's gS for the group sits in
// registers (8 features x the group's output components per lane).  Per edge
// and lane: the CG terms T, gT = R gS, the partial of grad_R (sum over the
// group's components) and of grad_Y (CG adjoint with gT); both are summed over
// the edge's channel lanes, then over the groups through LDS.
template <class S, int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_bwd_recv(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                  const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ R,
                  const float* __restrict__ gS, float* __restrict__ grad_Y, float* __restrict__ grad_R,
                  FcLayout lay, const int32_t* __restrict__ order) {
  constexpr int EPI = 64 / U, NG = 4, CH = 64, NR = H + S::YC;
  constexpr PathGroups<S, NG> PG = make_groups<S, NG>();
  __shared__ int cs[CH];
  __shared__ float ys[CH * S::YC];
  __shared__ float rs[CH * H];
  __shared__ float red[NG][CH][NR];
  // node of this workgroup in the launch order (largest degree first), or node order
  const int i = order ? min(max(order[blockIdx.x], 0), n_nodes - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int grp = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ec = lane / U, u = lane % U;
  constexpr int NF = ls_final(NR, U);
  const HalvingShare share = halving_share(NR, U, lane);
  static_for<NG>([&](auto G) {
    if (grp != G) return;
    constexpr int P0 = PG.start[G], NPP = PG.start[G + 1] - P0;
    constexpr int NT = comps<S>(P0, NPP);
    float gs[NT][H];
    static_for<NPP>([&](auto PP) {
      constexpr int P = P0 + PP;
      constexpr PathInfo pi = S::paths.p[P];
      constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P);
      constexpr int NPK = paths_into<S>(pi.k), PL = path_local<S>(P);
      constexpr int KK = H * NPK * U;
      const float* gk = gS + lay.base[pi.k] + (size_t)i * D3 * KK;
      static_for<D3>([&](auto C) {
#pragma unroll
        for (int h = 0; h < H; ++h) gs[OFF + C][h] = gk[(size_t)C * KK + (size_t)(h * NPK + PL) * U + u];
      });
    });
    for (int c0 = beg; c0 < end; c0 += CH) {
      const int cn = end - c0 < CH ? end - c0 : CH;
      __syncthreads();
      for (int k = t; k < cn; k += 256) cs[k] = col[c0 + k];
      for (int k = t; k < cn * S::YC; k += 256) ys[k] = Y[(size_t)c0 * S::YC + k];
      for (int k = t; k < cn * H; k += 256) rs[k] = R[(size_t)c0 * H + k];
      __syncthreads();
      auto body = [&](int s0, const float (&xr)[S::XC]) {
        const int e = s0 * EPI + ec;
        const bool ok = e < cn;
        const int ee = ok ? e : cn - 1;
        float yr[S::YC], rr[H];
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = ys[ee * S::YC + b];
#pragma unroll
        for (int h = 0; h < H; ++h) rr[h] = rs[ee * H + h];
        float acc[NR];
#pragma unroll
        for (int q = 0; q < NR; ++q) acc[q] = 0.f;
        static_for<NPP>([&](auto PP) {
          constexpr PathInfo pi = S::paths.p[P0 + PP];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P0 + PP);
          float tv[D3], gt[D3];
          static_for<D3>([&](auto C) {
            tv[C] = 0.f;
            float a = 0.f;
#pragma unroll
            for (int h = 0; h < H; ++h) a = fmaf(rr[h], gs[OFF + C][h], a);
            gt[C] = a;
          });
          static_for<T::nnz>([&](auto N) {
            constexpr Nz z = T::table.e[N];
            tv[z.c] = fmaf(z.v, xr[pi.xo + z.a] * yr[pi.yo + z.b], tv[z.c]);
            acc[H + pi.yo + z.b] = fmaf(z.v, xr[pi.xo + z.a] * gt[z.c], acc[H + pi.yo + z.b]);
          });
          static_for<D3>([&](auto C) {
#pragma unroll
            for (int h = 0; h < H; ++h) acc[h] = fmaf(gs[OFF + C][h], tv[C], acc[h]);
          });
        });
        // sum over the edge's U channel lanes; the lane then holds the totals
        // of values share.first .. share.first + share.len - 1
        lane_sum_halving<NR, U / 2>(acc, lane);
        if (ok) {
#pragma unroll
          for (int j = 0; j < NF; ++j)
            if (j < share.len) red[G][e][share.first + j] = acc[j];
        }
      };
      // the next step's gathers are issued before this step's arithmetic
      auto pload = [&](int s0, float (&xv)[S::XC]) {
        const int e = s0 * EPI + ec;
        load_x_channel<S, U>(x, cs[e < cn ? e : cn - 1], u, xv);
      };
      float xa[S::XC], xb[S::XC];
      pload(0, xa);
      for (int s0 = 0; s0 * EPI < cn; s0 += 2) {
        pload(s0 + 1, xb);
        __builtin_amdgcn_sched_barrier(0);
        body(s0, xa);
        if ((s0 + 1) * EPI >= cn) break;
        pload(s0 + 2, xa);
        __builtin_amdgcn_sched_barrier(0);
        body(s0 + 1, xb);
      }
      __syncthreads();
      for (int k = t; k < cn * NR; k += 256) {
        const int e = k / NR, q = k % NR;
        const float v = (red[0][e][q] + red[1][e][q]) + (red[2][e][q] + red[3][e][q]);
        if (q < H) {
          if (grad_R) grad_R[(size_t)(c0 + e) * H + q] = v;
        } else if (grad_Y) {
          grad_Y[(size_t)(c0 + e) * S::YC + (q - H)] = v;
        }
      }
    }
  });
}

// sender-side path groups: balanced input components (Q's accumulators)
template <class S>
constexpr int comps_in(int p0, int n) {
  int t = 0;
  for (int q = p0; q < p0 + n; ++q) t += 2 * S::paths.p[q].l1 + 1;
  return t;
}
template <class S>
constexpr int paths_from(int b) {
  int n = 0;
  for (int q = 0; q < S::NP; ++q)
    if (S::paths.p[q].in == b) ++n;
  return n;
}
template <class S>
constexpr int path_local_in(int p) {
  int n = 0;
  for (int q = 0; q < p; ++q)
    if (S::paths.p[q].in == S::paths.p[p].in) ++n;
  return n;
}
template <class S, int NG>
constexpr PathGroups<S, NG> make_groups_in() {
  PathGroups<S, NG> g{};
  const int total = comps_in<S>(0, S::NP);
  int p = 0;
  for (int k = 0; k < NG; ++k) {
    g.start[k] = p;
    const int target = (total * (k + 1) + NG - 1) / NG;
    while (p < S::NP && (k == NG - 1 || comps_in<S>(0, p + 1) <= target)) ++p;
  }
  g.start[NG] = S::NP;
  return g;
}

// Sender pass: Q_j[h][p][v][a] = sum_{e out of j} R_e[h] G_e[p][v][a],
// G_e[p][v][a] = sum_{b,c} C_p[a,b,c] Y_e[b] gout_i[k(p)][v][c].  The state
// kernel's layout with the sender grouping: one workgroup per sender, one
// wave per path group, lane = (edge class, output channel v), 4x4x1 products
// of R (rows) and G (columns); Q is written once per sender in the layout of
// the input irreps: Q_b[(j, a)][(h, path of b, v)].
template <class S, int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_bwd_send(int n_nodes, const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                  const int32_t* __restrict__ t_col, const float* __restrict__ Y, const float* __restrict__ R,
                  const float* __restrict__ gout, float* __restrict__ Qbuf, FcLayout lin,
                  const int32_t* __restrict__ order) {
  constexpr int EPI = 64 / U, NG = 4, CH = 128;
  constexpr PathGroups<S, NG> PG = make_groups_in<S, NG>();
  __shared__ int rc[CH];
  __shared__ float ys[CH * S::YC];
  __shared__ float rs[CH * H];
  const int j = order ? min(max(order[blockIdx.x], 0), n_nodes - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  const int grp = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ec = lane / U, v = lane % U, p4 = lane % 4;
  static_for<NG>([&](auto G) {
    if (grp != G) return;
    constexpr int P0 = PG.start[G], NPP = PG.start[G + 1] - P0;
    constexpr int NT = comps_in<S>(P0, NPP);
    v4f acc[NT][2];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k][0] = acc[k][1] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int c0 = beg; c0 < end; c0 += CH) {
      const int cn = end - c0 < CH ? end - c0 : CH;
      __syncthreads();
      for (int k = t; k < cn; k += 256) rc[k] = t_col[c0 + k];
      for (int k = t; k < cn * S::YC; k += 256)
        ys[k] = Y[(size_t)t_perm[c0 + k / S::YC] * S::YC + k % S::YC];
      for (int k = t; k < cn * H; k += 256) rs[k] = R[(size_t)t_perm[c0 + k / H] * H + k % H];
      __syncthreads();
      auto body = [&](int s0, const float (&gr)[S::OC]) {
        const int e = s0 * EPI + ec;
        const bool ok = e < cn;
        const int ee = ok ? e : cn - 1;
        float yr[S::YC];
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = ys[ee * S::YC + b];
        const float a0 = ok ? rs[ee * H + p4] : 0.f, a1 = ok ? rs[ee * H + 4 + p4] : 0.f;
        float gt[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) gt[q] = 0.f;
        static_for<NPP>([&](auto PP) {
          constexpr PathInfo pi = S::paths.p[P0 + PP];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int OFF = comps_in<S>(P0, PP);
          static_for<T::nnz>([&](auto N) {
            constexpr Nz z = T::table.e[N];
            gt[OFF + z.a] = fmaf(z.v, yr[pi.yo + z.b] * gr[pi.ko + z.c], gt[OFF + z.a]);
          });
        });
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          acc[q][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, gt[q], acc[q][0], 0, 0, 0);
          acc[q][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, gt[q], acc[q][1], 0, 0, 0);
        }
      };
      // the next step's gathers are issued before this step's arithmetic
      auto pload = [&](int s0, float (&xv)[S::OC]) {
        const int e = s0 * EPI + ec;
        load_o_channel<S, U>(gout, rc[e < cn ? e : cn - 1], v, xv);
      };
      float xa[S::OC], xb[S::OC];
      pload(0, xa);
      for (int s0 = 0; s0 * EPI < cn; s0 += 2) {
        pload(s0 + 1, xb);
        __builtin_amdgcn_sched_barrier(0);
        body(s0, xa);
        if ((s0 + 1) * EPI >= cn) break;
        pload(s0 + 2, xa);
        __builtin_amdgcn_sched_barrier(0);
        body(s0 + 1, xb);
      }
    }
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int off = U; off < 64; off <<= 1) acc[q][hf][r] += __shfl_xor(acc[q][hf][r], off, 64);
    if (ec == 0) {
      static_for<NPP>([&](auto PP) {
        constexpr int P = P0 + PP;
        constexpr PathInfo pi = S::paths.p[P];
        constexpr int D1 = 2 * pi.l1 + 1, OFF = comps_in<S>(P0, PP);
        constexpr int NPB = paths_from<S>(pi.in), PL = path_local_in<S>(P);
        constexpr int KK = H * NPB * U;
        float* Qb = Qbuf + lin.base[pi.in] + (size_t)j * D1 * KK;
        static_for<D1>([&](auto A) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Qb[(size_t)A * KK + (size_t)((4 * hf + r) * NPB + PL) * U + v] = acc[OFF + A][hf][r];
        });
      });
    }
  });
}

using SigF = Sig<2, 2, 0, 1, 2>;
constexpr int kH = 8;

template <int U>
FcLayout make_layout(int n_nodes) {
  FcLayout L{};
  L.n_out = SigF::NO;
  long long off = 0;
  for (int k = 0; k < SigF::NO; ++k) {
    L.d3[k] = 2 * SigF::outs.o[k].l + 1;
    L.ko[k] = SigF::outs.o[k].ko;
    int n = 0;
    for (int p = 0; p < SigF::NP; ++p)
      if (SigF::paths.p[p].k == k) L.pg[k][n++] = p;
    L.npk[k] = n;
    L.base[k] = off;
    off += (long long)n_nodes * L.d3[k] * kH * n * U;
  }
  return L;
}

template <int U>
size_t fc_ws(int n_nodes) {
  const FcLayout L = make_layout<U>(n_nodes);
  long long tot = 0;
  for (int k = 0; k < L.n_out; ++k) tot += (long long)n_nodes * L.d3[k] * kH * L.npk[k] * U;
  return (size_t)tot * sizeof(float);
}

// the input-irrep layout of the sender-side state Q (and of grad_x)
template <int U>
FcLayout make_layout_in(int n_nodes) {
  FcLayout L{};
  L.n_out = SigF::NIN;
  long long off = 0;
  for (int b = 0; b < SigF::NIN; ++b) {
    L.d3[b] = 2 * SigF::ls.v[b] + 1;
    L.ko[b] = SigF::xoff(b);
    int n = 0;
    for (int p = 0; p < SigF::NP; ++p)
      if (SigF::paths.p[p].in == b) L.pg[b][n++] = p;
    L.npk[b] = n;
    L.base[b] = off;
    off += (long long)n_nodes * L.d3[b] * kH * n * U;
  }
  return L;
}

// offsets of the grad_Theta partial sums per output irrep
template <int U>
FcLayout make_layout_part(int n_nodes) {
  const FcLayout L = make_layout<U>(n_nodes);
  FcLayout P{};
  P.n_out = L.n_out;
  long long off = 0;
  for (int k = 0; k < L.n_out; ++k) {
    P.base[k] = off;
    const long long nrb = ((long long)n_nodes * L.d3[k] + kRowBlock - 1) / kRowBlock;
    off += nrb * kH * L.npk[k] * U * U;
  }
  P.base[L.n_out] = off;   // total (the layout has room for 8 irreps; this signature has 5)
  return P;
}

template <int U>
size_t fc_bwd_ws(int n_nodes) {
  const FcLayout Li = make_layout_in<U>(n_nodes);
  const FcLayout Lp = make_layout_part<U>(n_nodes);
  long long q = 0;
  for (int b = 0; b < Li.n_out; ++b) q += (long long)n_nodes * Li.d3[b] * kH * Li.npk[b] * U;
  return 2 * fc_ws<U>(n_nodes) + (size_t)(q + Lp.base[Lp.n_out]) * sizeof(float);
}

template <int U>
hipError_t launch_fc_fwd(const FcArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  const FcLayout L = make_layout<U>(a.n_nodes);
  float* Sbuf = static_cast<float*>(a.ws);
  hipLaunchKernelGGL((k_fc_state<SigF, U, kH>), dim3(a.n_nodes), dim3(256), 0, a.stream, a.n_nodes, a.row_ptr,
                     a.col, a.x, a.Y, a.R, Sbuf, L, a.r_order);
  int tiles = 0;
  for (int k = 0; k < L.n_out; ++k) tiles += (a.n_nodes * L.d3[k] + 16 * kRT - 1) / (16 * kRT);
  hipLaunchKernelGGL((k_fc_contract<U, kH, false>), dim3(tiles), dim3(64 * kCW), 0, a.stream, a.n_nodes, Sbuf, a.Theta,
                     SigF::NP, a.outdim, a.out, L);
  return hipGetLastError();
}

template <int U>
hipError_t launch_fc_bwd(const FcArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  const FcLayout L = make_layout<U>(a.n_nodes);
  const FcLayout Li = make_layout_in<U>(a.n_nodes);
  const FcLayout Lp = make_layout_part<U>(a.n_nodes);
  float* Sbuf = static_cast<float*>(a.ws);
  float* gS = Sbuf + fc_ws<U>(a.n_nodes) / sizeof(float);
  float* Q = gS + fc_ws<U>(a.n_nodes) / sizeof(float);
  long long qn = 0;
  for (int b = 0; b < Li.n_out; ++b) qn += (long long)a.n_nodes * Li.d3[b] * kH * Li.npk[b] * U;
  float* part = Q + qn;
  int tiles = 0;
  for (int k = 0; k < L.n_out; ++k) tiles += (a.n_nodes * L.d3[k] + 15) / 16;
  if (a.grad_Theta) {
    if (!a.state_saved)   // else the forward's S is still in ws
      hipLaunchKernelGGL((k_fc_state<SigF, U, kH>), dim3(a.n_nodes), dim3(256), 0, a.stream, a.n_nodes,
                         a.row_ptr, a.col, a.x, a.Y, a.R, Sbuf, L, a.r_order);
    int nb = 0;
    for (int k = 0; k < L.n_out; ++k)
      nb += ((a.n_nodes * L.d3[k] + kRowBlock - 1) / kRowBlock) * ((kH * L.npk[k] * U / 16 + 3) / 4);
    hipLaunchKernelGGL((k_fc_gradtheta<U, kH>), dim3(nb), dim3(256), 0, a.stream, a.n_nodes, Sbuf, a.gout,
                       a.outdim, part, L, Lp);
    PathMap pm{};
    for (int p = 0; p < SigF::NP; ++p) {
      pm.k[p] = SigF::paths.p[p].k;
      int n = 0;
      for (int q = 0; q < p; ++q) n += SigF::paths.p[q].k == pm.k[p];
      pm.pl[p] = n;
    }
    const int tot = kH * SigF::NP * U * U;
    hipLaunchKernelGGL((k_fc_gradtheta_sum<U, kH>), dim3((tot + 255) / 256), dim3(256), 0, a.stream, a.n_nodes,
                       part, SigF::NP, a.grad_Theta, L, Lp, pm);
  }
  if ((a.grad_R || a.grad_Y) && a.n_edges > 0) {
    hipLaunchKernelGGL((k_fc_expand<U, kH>), dim3(tiles), dim3(256), 0, a.stream, a.n_nodes, a.gout, a.Theta,
                       SigF::NP, a.outdim, gS, L);
    hipLaunchKernelGGL((k_fc_bwd_recv<SigF, U, kH>), dim3(a.n_nodes), dim3(256), 0, a.stream, a.n_nodes,
                       a.row_ptr, a.col, a.x, a.Y, a.R, gS, a.grad_Y, a.grad_R, L, a.r_order);
  }
  if (a.grad_x) {
    hipLaunchKernelGGL((k_fc_bwd_send<SigF, U, kH>), dim3(a.n_nodes), dim3(256), 0, a.stream, a.n_nodes,
                       a.t_row_ptr, a.t_perm, a.t_col, a.Y, a.R, a.gout, Q, Li, a.s_order);
    int tin = 0;
    for (int b = 0; b < Li.n_out; ++b) tin += (a.n_nodes * Li.d3[b] + 16 * kRT - 1) / (16 * kRT);
    hipLaunchKernelGGL((k_fc_contract<U, kH, true>), dim3(tin), dim3(64 * kCW), 0, a.stream, a.n_nodes, Q, a.Theta,
                       SigF::NP, SigF::XC * U, a.grad_x, Li);
  }
  return hipGetLastError();
}

// ---- second-order backward --------------------------------------------------
// out is linear in each of x, Y, R and Theta, so the gradients of
// L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_R, grad_R> + <gg_Theta, grad_Theta>
// are sums of first-order results with one operand replaced by its cotangent:
// per present cotangent one forward (its term of d_grad_out) and one backward
// (its terms of the other three gradients).  The first term of each output is
// written in place, later ones go through a scratch row and are added.

__global__ void __launch_bounds__(256) k_fc_acc(float* __restrict__ y, const float* __restrict__ x, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) y[i] += x[i];
}
__global__ void __launch_bounds__(256) k_fc_zero(float* __restrict__ y, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) y[i] = 0.f;
}
unsigned fc_elem_grid(long long n) {
  const long long b = (n + 255) / 256;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

size_t fc_align(size_t b) { return (b + 255) & ~size_t(255); }

// scratch rows after the first-order workspace: d_grad_out, d_x, d_Y, d_R, d_Theta
template <int U>
size_t fc_dbl_ws(int n_nodes, int n_edges) {
  return fc_align(fc_bwd_ws<U>(n_nodes)) + fc_align((size_t)n_nodes * SigF::OC * U * 4) +
         fc_align((size_t)n_nodes * SigF::XC * U * 4) + fc_align((size_t)n_edges * SigF::YC * 4) +
         fc_align((size_t)n_edges * kH * 4) + fc_align((size_t)kH * SigF::NP * U * U * 4);
}

struct FcAcc {
  float* out;
  float* tmp;
  long long n;
  bool first;
  float* dest() const { return out ? (first ? out : tmp) : nullptr; }
};

template <int U>
hipError_t launch_fc_dbl(const FcArgs& a, const FcDbl& d) {
  const long long N = a.n_nodes, E = a.n_edges;
  char* w = static_cast<char*>(a.ws) + fc_align(fc_bwd_ws<U>(a.n_nodes));
  auto take = [&](size_t bytes) {
    float* p = reinterpret_cast<float*>(w);
    w += fc_align(bytes);
    return p;
  };
  FcAcc ag{d.d_g, take((size_t)N * SigF::OC * U * 4), N * SigF::OC * U, true};
  FcAcc ax{d.d_x, take((size_t)N * SigF::XC * U * 4), N * SigF::XC * U, true};
  FcAcc aY{d.d_Y, take((size_t)E * SigF::YC * 4), E * SigF::YC, true};
  FcAcc aR{d.d_R, take((size_t)E * kH * 4), E * kH, true};
  FcAcc aT{d.d_Theta, take((size_t)kH * SigF::NP * U * U * 4), (long long)kH * SigF::NP * U * U, true};
  auto done = [&](FcAcc& c) {
    if (!c.out) return;
    if (c.first) {
      c.first = false;
    } else {
      hipLaunchKernelGGL(k_fc_acc, dim3(fc_elem_grid(c.n)), dim3(256), 0, a.stream, c.out, c.tmp, c.n);
    }
  };
  if (N > 0 && E > 0) {
    for (int which = 0; which < 4; ++which) {
      const float* cot = which == 0 ? d.gg_x : which == 1 ? d.gg_Y : which == 2 ? d.gg_R : d.gg_Theta;
      if (!cot) continue;
      FcArgs f = a;
      if (which == 0) f.x = cot;
      if (which == 1) f.Y = cot;
      if (which == 2) f.R = cot;
      if (which == 3) f.Theta = cot;
      if (ag.out) {
        f.out = ag.dest();
        hipError_t e = launch_fc_fwd<U>(f);
        if (e != hipSuccess) return e;
        done(ag);
      }
      FcArgs b = f;
      b.out = nullptr;
      b.state_saved = false;
      b.grad_x = which == 0 ? nullptr : ax.dest();
      b.grad_Y = which == 1 ? nullptr : aY.dest();
      b.grad_R = which == 2 ? nullptr : aR.dest();
      b.grad_Theta = which == 3 ? nullptr : aT.dest();
      if (b.grad_x || b.grad_Y || b.grad_R || b.grad_Theta) {
        hipError_t e = launch_fc_bwd<U>(b);
        if (e != hipSuccess) return e;
        if (which != 0) done(ax);
        if (which != 1) done(aY);
        if (which != 2) done(aR);
        if (which != 3) done(aT);
      }
    }
  }
  // outputs that received no term are zero
  for (FcAcc* c : {&ag, &ax, &aY, &aR, &aT})
    if (c->out && c->first && c->n > 0)
      hipLaunchKernelGGL(k_fc_zero, dim3(fc_elem_grid(c->n)), dim3(256), 0, a.stream, c->out, c->n);
  return hipGetLastError();
}

template <int U>
const FcSet* fc_set() {
  static const FcSet s{&launch_fc_fwd<U>, &fc_ws<U>, kH, &launch_fc_bwd<U>, &fc_bwd_ws<U>,
                       &launch_fc_dbl<U>, &fc_dbl_ws<U>};
  return &s;
}

}  // namespace

const FcSet* fc_l012_s2(int mul, int n_radial) {
  if (n_radial != kH) return nullptr;
  switch (mul) {
    case 16: return fc_set<16>();
    case 32: return fc_set<32>();
    case 64: return fc_set<64>();
    default: return nullptr;
  }
}

}  // namespace tpc
