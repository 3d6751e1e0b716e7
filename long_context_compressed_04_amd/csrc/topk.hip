// Causal top-k selection over indexer score rows.
//
// "DeepSeek v4" summary page, section "Compressed Sparse Attention": each query
// keeps only the top-k compressed entries chosen by the selector, among the
// preceding (complete) blocks.  Techniques map "DeepSeek-V4-Pro", "Indexer-
// selected sparse attention": index_topk entries, slots past the causal threshold
// marked -1.
//
// One workgroup (1024 threads) per score row.  Scores map to order-preserving
// uint32 keys; rows of up to kLdsKeys keys are held in LDS (one pass over HBM/L2
// with every load in flight), longer rows are re-read from global memory.  A
// min/max pass finds the bits all visible keys share; MSB-first radix passes of up
// to 11 bits (2048-bin LDS histogram, the threshold digit found with one block
// scan) narrow the prefix of the k-th largest key, stopping early once the
// remaining bucket is taken whole.  The final compaction is in index order (two
// block scans): every key above the threshold prefix, then the lowest-index keys
// equal to it -- the exact set "score descending, ties to the lower index", sorted
// by index, -1 padded.
#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "launch_timer.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kBins = 2048;
constexpr int kDigit = 11;
constexpr int kLdsKeys = 32768;

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(IndexArgs A, const float* scores,
                                                                 int32_t* out_idx, float* out_score) {
  extern __shared__ uint32_t keys[];   // IN_LDS: [V]
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[kTopkThreads / 64 + 1];
  __shared__ uint32_t red_min[kTopkThreads / 64], red_max[kTopkThreads / 64];
  __shared__ uint32_t s_prefix, s_need, s_cnt;

  const long row = blockIdx.x;
  const int b = (int)(row / A.n_q);
  const int k = A.topk;
  const int ne = min(A.n_entries[b], A.n_max);
  const int V = visible_entries(A.q_pos[row], ne, A.m);
  const float* src = scores + row * A.n_max;
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;

  if (V <= k) {  // everything visible is selected
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
      oi[i] = i < V ? i : -1;
      if (os) os[i] = i < V ? src[i] : -INFINITY;
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto key_at = [&](int i) -> uint32_t { return IN_LDS ? keys[i] : order_key(src[i]); };

  // ---- load (LDS rows) and the bits every visible key shares
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll 8
  for (int i = threadIdx.x; i < V; i += kTopkThreads) {
    uint32_t key = order_key(src[i]);
    if (IN_LDS) keys[i] = key;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) { red_min[wave] = kmin; red_max[wave] = kmax; }
  __syncthreads();
  kmin = red_min[0]; kmax = red_max[0];
  for (int w = 1; w < kTopkThreads / 64; ++w) { kmin = min(kmin, red_min[w]); kmax = max(kmax, red_max[w]); }

  int hi = (kmin == kmax) ? 0 : 32 - __clz((int)(kmin ^ kmax));   // low bits still undecided
  uint32_t mask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  uint32_t prefix = kmin & mask;
  uint32_t need = (uint32_t)k;

  // ---- MSB-first radix narrowing of the k-th largest key's prefix
  while (hi > 0) {
    const int width = hi < kDigit ? hi : kDigit;
    const int shift = hi - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 8
    for (int i = threadIdx.x; i < V; i += kTopkThreads) {
      uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns bins 2047-2t (upper) and 2046-2t: a scan in thread order counts
    // every key in higher bins
    const int bu = kBins - 1 - 2 * threadIdx.x, bl = bu - 1;
    const uint32_t cu = hist[bu], cl = hist[bl];
    uint32_t total;
    const uint32_t above = block_exclusive_scan<kTopkThreads>(cu + cl, tmp, &total);
    if (above < need && need <= above + cu + cl) {
      if (above + cu >= need) {
        s_prefix = prefix | ((uint32_t)bu << shift);
        s_need = need - above;
        s_cnt = cu;
      } else {
        s_prefix = prefix | ((uint32_t)bl << shift);
        s_need = need - above - cu;
        s_cnt = cl;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= dmask << shift;
    hi = shift;
    const bool whole = s_cnt == need;
    __syncthreads();
    if (whole) break;   // the whole bucket is selected
  }

  // ---- index-ordered compaction: keys whose prefix is above, then the first `need`
  // keys equal to the prefix
  const int seg = (V + kTopkThreads - 1) / kTopkThreads;
  const int lo = threadIdx.x * seg;
  const int hi_i = min(V, lo + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi_i; ++i) {
    uint32_t kp = key_at(i) & mask;
    n_gt += kp > prefix;
    n_eq += kp == prefix;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan<kTopkThreads>(n_eq, tmp, &tot);
  const uint32_t take_eq = eq_before >= need ? 0u : min(n_eq, need - eq_before);
  uint32_t pos = block_exclusive_scan<kTopkThreads>(n_gt + take_eq, tmp, &tot);
  uint32_t eq_seen = eq_before;
  for (int i = lo; i < hi_i; ++i) {
    const uint32_t kp = key_at(i) & mask;
    bool sel = kp > prefix;
    if (kp == prefix) {
      sel = eq_seen < need;
      ++eq_seen;
    }
    if (sel && pos < (uint32_t)k) {
      oi[pos] = i;
      if (os) os[pos] = src[i];
      ++pos;
    }
  }
}

hipError_t launch_topk_rows(const IndexArgs& A, const float* scores, int32_t* out_idx, float* out_score,
                            hipStream_t s) {
  const long rows = (long)A.batch * A.n_q;
  if (rows <= 0) return hipSuccess;
  LaunchTimer timer("topk", s);
  if (A.n_max <= kLdsKeys) {
    const size_t lds = sizeof(uint32_t) * (size_t)A.n_max;
    static hipError_t attr = hipFuncSetAttribute((const void*)topk_rows_kernel<true>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)(sizeof(uint32_t) * kLdsKeys));
    if (attr != hipSuccess) return attr;
    topk_rows_kernel<true><<<dim3((unsigned)rows), kTopkThreads, lds, s>>>(A, scores, out_idx, out_score);
  } else {
    topk_rows_kernel<false><<<dim3((unsigned)rows), kTopkThreads, 0, s>>>(A, scores, out_idx, out_score);
  }
  return hipGetLastError();
}

}  // namespace csa
