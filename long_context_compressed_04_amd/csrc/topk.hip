// Causal top-k selection over indexer score rows.
//
// "DeepSeek v4" summary page, section "Compressed Sparse Attention": each query
// keeps only the top-k compressed entries chosen by the selector, among the
// preceding (complete) blocks.  Techniques map "DeepSeek-V4-Pro", "Indexer-
// selected sparse attention": index_topk entries, slots past the causal threshold
// marked -1.
//
// One workgroup (1024 threads) per score row.  Scores map to order-preserving
// uint32 keys.  A min/max pass finds the bits all visible keys share; MSB-first
// radix passes (<= 8 bits each, LDS histogram) then narrow the prefix of the k-th
// largest key, stopping early once the remaining bucket is taken whole.  The final
// compaction is in index order (two block scans): every key above the threshold
// prefix, then the lowest-index keys equal to it, so the output is the exact set
// "score descending, ties to the lower index", sorted by index, -1 padded.
#include "csa_device.hpp"
#include "csa_kernels.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(IndexArgs A, const float* scores,
                                                                 int32_t* out_idx, float* out_score) {
  const long row = blockIdx.x;
  const int b = (int)(row / A.n_q);
  const int k = A.topk;
  const int ne = min(A.n_entries[b], A.n_max);
  const int V = visible_entries(A.q_pos[row], ne, A.m);
  const float* src = scores + row * A.n_max;
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[kTopkThreads / 64 + 1];
  __shared__ uint32_t red_min[kTopkThreads / 64], red_max[kTopkThreads / 64];
  __shared__ uint32_t s_prefix, s_need, s_cnt;

  if (V <= k) {  // everything visible is selected
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
      oi[i] = i < V ? i : -1;
      if (os) os[i] = i < V ? src[i] : -INFINITY;
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- bits shared by every visible key
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = threadIdx.x; i < V; i += blockDim.x) {
    uint32_t key = order_key(src[i]);
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
    const int width = hi < 8 ? hi : 8;
    const int shift = hi - width;
    const uint32_t dmask = (1u << width) - 1u;
    __syncthreads();
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < V; i += blockDim.x) {
      uint32_t key = order_key(src[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4] = {hist[4 * lane], hist[4 * lane + 1], hist[4 * lane + 2], hist[4 * lane + 3]};
      uint32_t tot = c[0] + c[1] + c[2] + c[3];
      uint32_t suf = tot;  // inclusive suffix sum over lanes (higher lane = higher bins)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = (uint32_t)__shfl_down((int)suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      uint32_t above = suf - tot;
      if (above < need && need <= suf) {
        uint32_t cum = above;
        int d = 3;
        for (; d > 0; --d) {
          if (cum + c[d] >= need) break;
          cum += c[d];
        }
        s_prefix = prefix | ((uint32_t)(4 * lane + d) << shift);
        s_need = need - cum;
        s_cnt = c[d];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= dmask << shift;
    hi = shift;
    if (s_cnt == need) break;   // the whole bucket is selected
  }

  // ---- index-ordered compaction: keys whose prefix is above, then the first `need`
  // keys equal to the prefix
  const int seg = (V + kTopkThreads - 1) / kTopkThreads;
  const int lo = threadIdx.x * seg;
  const int hi_i = min(V, lo + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi_i; ++i) {
    uint32_t kp = order_key(src[i]) & mask;
    n_gt += kp > prefix;
    n_eq += kp == prefix;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan<kTopkThreads>(n_eq, tmp, &tot);
  const uint32_t take_eq = eq_before >= need ? 0u : min(n_eq, need - eq_before);
  uint32_t pos = block_exclusive_scan<kTopkThreads>(n_gt + take_eq, tmp, &tot);
  uint32_t eq_seen = eq_before;
  for (int i = lo; i < hi_i; ++i) {
    const float sv = src[i];
    const uint32_t kp = order_key(sv) & mask;
    bool sel = kp > prefix;
    if (kp == prefix) {
      sel = eq_seen < need;
      ++eq_seen;
    }
    if (sel && pos < (uint32_t)k) {
      oi[pos] = i;
      if (os) os[pos] = sv;
      ++pos;
    }
  }
}

hipError_t launch_topk_rows(const IndexArgs& A, const float* scores, int32_t* out_idx, float* out_score,
                            hipStream_t s) {
  const long rows = (long)A.batch * A.n_q;
  if (rows <= 0) return hipSuccess;
  topk_rows_kernel<<<dim3((unsigned)rows), kTopkThreads, 0, s>>>(A, scores, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace csa
