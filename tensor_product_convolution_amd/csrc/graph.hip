// Edge grouping by receiver and by sender (CSR), on the device.
//
// Receiver-grouped edges let each receiver's state live on chip instead of
// being scatter-added with atomics ("Sobek: Streaming Equivariant Tensor
// Product Convolutions", Abstract; "The GPU Workload That Rewrites Molecular
// Physics", section "What Makes MLFF Workloads Structurally Different", on
// scatter-reduce contention at popular atoms).
//
// The grouping is a stable least-significant-digit radix sort of the
// receiver ids (8-bit digits, as many passes as the node count needs), so
// ties keep the original edge order and the result is unique: the same
// arrays come out on every run, bit for bit.  Each pass:
//   1. tile histogram: a 256-thread workgroup counts the digits of its
//      2048-key tile with LDS atomics (order-free, exact);
//   2. per-digit scan over tiles (one workgroup per digit) and a scan of the
//      256 digit totals give every (digit, tile) its global start;
//   3. ranked scatter: each wave walks its 512 keys in 8 ordered rounds of
//      64; lanes holding the same digit find each other with 8 ballots, so
//      a key's rank among equal digits is the count of equal-digit keys
//      before it -- a stable placement without sorting inside the tile.
// Row pointers come from boundaries of the sorted keys (no atomics).  The
// sender grouping sorts the receiver-sorted sender column the same way, so
// its ties keep receiver-sorted order.
#include <mutex>

#include "internal.hpp"

namespace tpc {
namespace {

constexpr int kWaves = 4;
constexpr int kRounds = 8;
constexpr int kSub = kRounds * 64;        // keys per wave
constexpr int kTile = kWaves * kSub;      // keys per workgroup
constexpr int kDigits = 256;

__global__ void __launch_bounds__(256) k_fill_u32(uint32_t* p, int n, uint32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void __launch_bounds__(256)
    k_check_range(const int32_t* __restrict__ a, const int32_t* __restrict__ b, int n, int lim,
                  uint32_t* __restrict__ flag) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    int va = a[i], vb = b[i];
    if (va < 0 || va >= lim || vb < 0 || vb >= lim) atomicOr(flag, 1u);
  }
}

__global__ void __launch_bounds__(256)
    k_tile_hist(const uint32_t* __restrict__ keys, int n, int shift, int ntiles,
                uint32_t* __restrict__ hist) {
  __shared__ uint32_t cnt[kDigits];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * kTile;
  for (int r = threadIdx.x; r < kTile; r += 256) {
    int idx = base + r;
    if (idx < n) atomicAdd(&cnt[(keys[idx] >> shift) & (kDigits - 1)], 1u);
  }
  __syncthreads();
  hist[threadIdx.x * ntiles + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of one digit's row of tile counts; writes the row total.
__global__ void __launch_bounds__(256)
    k_digit_row_scan(uint32_t* __restrict__ hist, int ntiles, uint32_t* __restrict__ totals) {
  __shared__ uint32_t wsum[4];
  uint32_t* row = hist + (size_t)blockIdx.x * ntiles;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t carry = 0;
  for (int base = 0; base < ntiles; base += 256) {
    int idx = base + threadIdx.x;
    uint32_t v = idx < ntiles ? row[idx] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      uint32_t t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int k = 0; k < wv; ++k) before += wsum[k];
    if (idx < ntiles) row[idx] = before + incl - v;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Exclusive scan of the 256 digit totals (in place).
__global__ void __launch_bounds__(256) k_digit_total_scan(uint32_t* __restrict__ totals) {
  __shared__ uint32_t s[kDigits];
  s[threadIdx.x] = totals[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int d = 0; d < kDigits; ++d) {
      uint32_t t = s[d];
      s[d] = run;
      run += t;
    }
  }
  __syncthreads();
  totals[threadIdx.x] = s[threadIdx.x];
}

__global__ void __launch_bounds__(256)
    k_ranked_scatter(const uint32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, int n,
                     int shift, int ntiles, const uint32_t* __restrict__ hist,
                     const uint32_t* __restrict__ digit_base, uint32_t* __restrict__ keys_out,
                     int32_t* __restrict__ vals_out) {
  __shared__ uint32_t wcnt[kWaves][kDigits];
  __shared__ uint32_t wbase[kWaves][kDigits];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int w = 0; w < kWaves; ++w) wcnt[w][threadIdx.x] = 0;
  __syncthreads();
  const int sub = blockIdx.x * kTile + wv * kSub;
  for (int r = 0; r < kRounds; ++r) {
    int idx = sub + r * 64 + lane;
    if (idx < n) atomicAdd(&wcnt[wv][(keys_in[idx] >> shift) & (kDigits - 1)], 1u);
  }
  __syncthreads();
  {
    const int d = threadIdx.x;
    uint32_t run = digit_base[d] + hist[(size_t)d * ntiles + blockIdx.x];
    for (int w = 0; w < kWaves; ++w) {
      wbase[w][d] = run;
      run += wcnt[w][d];
    }
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < kRounds; ++r) {
    const int idx = sub + r * 64 + lane;
    const bool active = idx < n;
    const uint32_t key = active ? keys_in[idx] : 0u;
    const uint32_t d = (key >> shift) & (kDigits - 1);
    unsigned long long peers = __ballot(active);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool b = (d >> bit) & 1u;
      const unsigned long long m = __ballot(b);
      peers &= b ? m : ~m;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & below);
    const uint32_t cnt = (uint32_t)__popcll(peers);
    const uint32_t base = wbase[wv][d];
    if (active) {
      const uint32_t pos = base + rank;
      keys_out[pos] = key;
      vals_out[pos] = vals_in ? vals_in[idx] : idx;
      if (rank == 0) wbase[wv][d] = base + cnt;
    }
  }
}

// row_ptr[i] = first sorted position whose key is >= i; keys clamped to N.
__global__ void __launch_bounds__(256)
    k_row_ptr(const uint32_t* __restrict__ sorted, int n, int n_nodes, int32_t* __restrict__ row_ptr) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q > n) return;
  long long prev = q == 0 ? -1 : (long long)sorted[q - 1];
  long long cur = q == n ? (long long)n_nodes : (long long)sorted[q];
  if (prev > n_nodes) prev = n_nodes;
  if (cur > n_nodes) cur = n_nodes;
  for (long long i = prev + 1; i <= cur; ++i) row_ptr[i] = q;
}

__global__ void __launch_bounds__(256)
    k_gather_i32(const int32_t* __restrict__ in, const int32_t* __restrict__ idx, int n, int n_nodes,
                 int32_t* __restrict__ out) {
  // node indices are clamped to [0, n_nodes): an unchecked build with bad
  // indices then yields a wrong grouping but never a later out-of-bounds read
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n) out[q] = min(max(in[idx[q]], 0), n_nodes - 1);
}

__global__ void __launch_bounds__(256)
    k_gather2_i32(const int32_t* __restrict__ in, const int32_t* __restrict__ idx1,
                  const int32_t* __restrict__ idx2, int n, int n_nodes, int32_t* __restrict__ out) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n) out[q] = min(max(in[idx1[idx2[q]]], 0), n_nodes - 1);
}

__global__ void __launch_bounds__(256)
    k_gather_rows(const uint32_t* __restrict__ in, const int32_t* __restrict__ perm, int64_t n_rows,
                  int64_t words, uint32_t* __restrict__ out) {
  const int64_t total = n_rows * words;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = t / words;
    const int64_t c = t - q * words;
    out[t] = in[(int64_t)perm[q] * words + c];
  }
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct GraphWs {
  uint32_t *kA, *kB, *sorted, *hist, *totals, *flag;
  int32_t *vA, *vB;
};

size_t ws_layout(int n_nodes, int n_edges, char* base, GraphWs* w) {
  const size_t e4 = align256((size_t)(n_edges > 0 ? n_edges : 1) * 4);
  const int ntiles = cdiv(n_edges > 0 ? n_edges : 1, kTile);
  const size_t h4 = align256((size_t)kDigits * ntiles * 4);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  GraphWs t{};
  t.kA = (uint32_t*)take(e4);
  t.vA = (int32_t*)take(e4);
  t.kB = (uint32_t*)take(e4);
  t.vB = (int32_t*)take(e4);
  t.sorted = (uint32_t*)take(e4);
  t.hist = (uint32_t*)take(h4);
  t.totals = (uint32_t*)take(align256(kDigits * 4));
  t.flag = (uint32_t*)take(256);
  (void)n_nodes;
  if (w) *w = t;
  return off;
}

hipError_t radix_sort(const uint32_t* keys_in, int n, int max_key, uint32_t* keys_out,
                      int32_t* vals_out, const GraphWs& ws, hipStream_t st) {
  int bits = 0;
  while (bits < 32 && (uint32_t)max_key >> bits) ++bits;
  const int passes = bits <= 8 ? 1 : (bits + 7) / 8;
  const int ntiles = cdiv(n, kTile);
  const uint32_t* kin = keys_in;
  const int32_t* vin = nullptr;
  for (int p = 0; p < passes; ++p) {
    const bool last = p == passes - 1;
    uint32_t* kout = last ? keys_out : (p % 2 == 0 ? ws.kA : ws.kB);
    int32_t* vout = last ? vals_out : (p % 2 == 0 ? ws.vA : ws.vB);
    const int shift = 8 * p;
    hipLaunchKernelGGL(k_tile_hist, dim3(ntiles), dim3(256), 0, st, kin, n, shift, ntiles, ws.hist);
    hipLaunchKernelGGL(k_digit_row_scan, dim3(kDigits), dim3(256), 0, st, ws.hist, ntiles, ws.totals);
    hipLaunchKernelGGL(k_digit_total_scan, dim3(1), dim3(256), 0, st, ws.totals);
    hipLaunchKernelGGL(k_ranked_scatter, dim3(ntiles), dim3(256), 0, st, kin, vin, n, shift, ntiles,
                       ws.hist, ws.totals, kout, vout);
    kin = kout;
    vin = vout;
  }
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------

size_t graph_workspace_bytes(int n_nodes, int n_edges) {
  return ws_layout(n_nodes, n_edges, nullptr, nullptr);
}

tp_status graph_build(const int32_t* src, const int32_t* dst, int n_edges, int n_nodes,
                      int32_t* row_ptr, int32_t* col, int32_t* perm, int32_t* t_row_ptr,
                      int32_t* t_perm, int32_t* t_col, void* ws_ptr, int32_t flags,
                      hipStream_t st) {
  GraphWs ws;
  ws_layout(n_nodes, n_edges, static_cast<char*>(ws_ptr), &ws);
  const int eb = cdiv(n_edges > 0 ? n_edges : 1, 256);
  hipError_t e;
  if (flags & TP_GRAPH_CHECK) {
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(256), 0, st, ws.flag, 1, 0u);
    if (n_edges > 0)
      hipLaunchKernelGGL(k_check_range, dim3(eb), dim3(256), 0, st, src, dst, n_edges, n_nodes, ws.flag);
    uint32_t h = 0;
    if ((e = hipMemcpyAsync(&h, ws.flag, 4, hipMemcpyDeviceToHost, st)) != hipSuccess)
      return hip_error(e, "graph check copy");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_error(e, "graph check sync");
    if (h) return set_error(TP_ERR_INDEX, "tp_conv_graph_build: src/dst index outside [0, n_nodes)");
  }
  const int rb = cdiv((int64_t)n_edges + 1, 256);
  if (n_edges > 0) {
    // receiver grouping: sort dst (values = original ids) -> perm, sorted dst
    if ((e = radix_sort(reinterpret_cast<const uint32_t*>(dst), n_edges, n_nodes - 1, ws.sorted,
                        perm, ws, st)) != hipSuccess)
      return hip_error(e, "receiver sort");
  }
  hipLaunchKernelGGL(k_row_ptr, dim3(rb), dim3(256), 0, st, ws.sorted, n_edges, n_nodes, row_ptr);
  if (n_edges > 0) {
    hipLaunchKernelGGL(k_gather_i32, dim3(eb), dim3(256), 0, st, src, perm, n_edges, n_nodes, col);
    // sender grouping of receiver-sorted positions: sort col (values = positions)
    if ((e = radix_sort(reinterpret_cast<const uint32_t*>(col), n_edges, n_nodes - 1, ws.sorted,
                        t_perm, ws, st)) != hipSuccess)
      return hip_error(e, "sender sort");
  }
  hipLaunchKernelGGL(k_row_ptr, dim3(rb), dim3(256), 0, st, ws.sorted, n_edges, n_nodes, t_row_ptr);
  if (n_edges > 0)
    hipLaunchKernelGGL(k_gather2_i32, dim3(eb), dim3(256), 0, st, dst, perm, t_perm, n_edges, n_nodes, t_col);
  if ((e = hipGetLastError()) != hipSuccess) return hip_error(e, "graph build launch");
  return TP_OK;
}

// ---------------------------------------------------------------------------
// Graph build without a workspace argument: the sort's scratch is a device
// array of this translation unit, one per GPU (each GPU that loads the
// library holds its own copy until the process ends).  Its host-side name is
// only a stand-in; the device address comes from hipGetSymbolAddress on the
// first call on each device (with that device current) and is kept per
// device.  Nothing here allocates.  Every scratch word the build reads is
// written by the same build first (tile histograms, scans, sort buffers; the
// range-check flag is cleared by a fill kernel), so the contents a previous
// call left need no clearing.
static __device__ __align__(256) char scratch[TP_GRAPH_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

tp_status graph_build_static(const int32_t* src, const int32_t* dst, int n_edges, int n_nodes,
                             int32_t* row_ptr, int32_t* col, int32_t* perm, int32_t* t_row_ptr,
                             int32_t* t_perm, int32_t* t_col, int32_t flags, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e, "tp_conv_graph_build_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(TP_ERR_ARG, "tp_conv_graph_build_static: device index beyond 64");
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_error(e, "tp_conv_graph_build_static: hipGetSymbolAddress");
      g_scratch_ptr[dev] = p;
    }
    base = g_scratch_ptr[dev];
  }
  return graph_build(src, dst, n_edges, n_nodes, row_ptr, col, perm, t_row_ptr, t_perm, t_col, base,
                     flags, st);
}

tp_status gather_rows(const void* in, const int32_t* perm, int64_t n_rows, int64_t words, void* out,
                      hipStream_t st) {
  if (n_rows == 0 || words == 0) return TP_OK;
  const int64_t total = n_rows * words;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint32_t*>(in), perm, n_rows, words, static_cast<uint32_t*>(out));
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "gather_rows launch");
}

// Launch order of the receiver- or sender-grouped kernels: nodes by
// descending degree, ties in ascending node id, as the stable sort of
// keys[i] = E - deg_i.  Degrees are clamped into [0, E].
__global__ void __launch_bounds__(256)
    k_degree_keys(const int32_t* __restrict__ ptr, int n, int n_edges, uint32_t* __restrict__ keys) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int d = min(max(ptr[i + 1] - ptr[i], 0), n_edges);
    keys[i] = (uint32_t)(n_edges - d);
  }
}

size_t order_workspace_bytes(int n_nodes) {
  return ws_layout(0, n_nodes, nullptr, nullptr) + align256((size_t)(n_nodes > 0 ? n_nodes : 1) * 4);
}

tp_status launch_order(const int32_t* row_ptr, const int32_t* t_row_ptr, int n_nodes, int n_edges,
                       int32_t* order, int32_t* t_order, void* ws_ptr, hipStream_t st) {
  if (n_nodes == 0) return TP_OK;
  GraphWs ws;
  const size_t base = ws_layout(0, n_nodes, static_cast<char*>(ws_ptr), &ws);
  uint32_t* keys = reinterpret_cast<uint32_t*>(static_cast<char*>(ws_ptr) + base);
  const int nb = cdiv(n_nodes, 256);
  const int32_t* ptrs[2] = {row_ptr, t_row_ptr};
  int32_t* outs[2] = {order, t_order};
  for (int s = 0; s < 2; ++s) {
    if (!outs[s]) continue;
    hipLaunchKernelGGL(k_degree_keys, dim3(nb), dim3(256), 0, st, ptrs[s], n_nodes, n_edges, keys);
    hipError_t e = radix_sort(keys, n_nodes, n_edges, ws.sorted, outs[s], ws, st);
    if (e != hipSuccess) return hip_error(e, "launch order sort");
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "launch order launch");
}

// e_pos[t_perm[k]] = k: for each receiver-sorted edge, its sender-grouped
// position (the inverse permutation of t_perm).  Entries outside [0, E) (a
// grouping that did not come from the build) are skipped, never written.
__global__ void __launch_bounds__(256)
    k_invert_perm(const int32_t* __restrict__ t_perm, int n, int32_t* __restrict__ e_pos) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) {
    const int q = t_perm[k];
    if (q >= 0 && q < n) e_pos[q] = k;
  }
}

tp_status sender_positions(const int32_t* t_perm, int n_edges, int32_t* e_pos, hipStream_t st) {
  if (n_edges == 0) return TP_OK;
  hipLaunchKernelGGL(k_invert_perm, dim3((n_edges + 255) / 256), dim3(256), 0, st, t_perm, n_edges, e_pos);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "sender_positions launch");
}

}  // namespace tpc
