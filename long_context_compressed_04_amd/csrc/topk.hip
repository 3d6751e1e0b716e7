// Causal top-k selection over indexer score rows.
//
// "DeepSeek v4" summary page, section "Compressed Sparse Attention": each query
// keeps only the top-k compressed entries chosen by the selector, among the
// preceding (complete) blocks.  Techniques map "DeepSeek-V4-Pro", "Indexer-
// selected sparse attention": index_topk entries, slots past the causal threshold
// marked -1.
//
// The selected set is exact: "score descending, ties to the lower index", written
// in ascending index order and -1 padded.  Scores map to order-preserving uint32
// keys.  One 1024-thread workgroup selects one row:
//  - the keys stay in registers (thread t holds the KPT consecutive positions
//    KPT t .. KPT t + KPT - 1, loaded 16 bytes at a time with raw buffer loads that
//    return 0 past the row);
//  - threshold: below the bits every key shares, an 11-bit radix digit is counted
//    in a 2048-bin LDS histogram (padded so that one wave reads it without bank
//    conflicts) and one wave finds the bin of the k-th largest key with two
//    cross-lane scans.  A bin of at most 64 keys is then resolved exactly by one
//    wave, bit by bit with ballots; larger bins take further 11-bit passes;
//  - compaction: each thread counts its keys above the threshold and equal to it;
//    exclusive scans over the threads (which are in position order) give each key
//    its output slot (keys above before it plus the equal keys before it, capped at
//    the number still needed); the selection is assembled in LDS and written out
//    with coalesced stores.
// Rows longer than kRegKeys take two launches.  Many workgroups each derive the same
// threshold from a fixed sample of kSample keys (expected to pass about 3k keys) and
// filter their chunks of the row against it into per-chunk candidate lists (index
// order kept); then one workgroup per row selects among the candidates.  If the
// threshold passes fewer than k keys or more than kCandCap, that row is selected
// straight from its scores in global memory (exact, slower).
#include <type_traits>

#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "launch_timer.hpp"
#include "select_device.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTW = kTopkThreads / 64;
constexpr int kRegKeys = 16384;       // direct path: the whole row in registers (16 keys per thread)
constexpr int kMaxKpt = kRegKeys / kTopkThreads;
constexpr int kCandCap = 16384;       // long rows: candidates kept for the exact selection
constexpr int kSample = 4096;         // long rows: keys in the threshold sample
constexpr int kChunk = 4096;          // long rows: keys per filter workgroup
constexpr int kFilterThreads = 256;
constexpr int kMaxChunks = 2048;
constexpr int kBins = 2048;           // 11-bit radix digit
constexpr int kHistWords = kBins + kBins / 32;
constexpr int kBucketMax = 64;
constexpr int kMaxTopk = 8192;        // largest k: the C ABI's 4096, or a rescoring prefilter's candidates
static_assert(2 * kMaxTopk >= kCandCap, "the output arrays stage a long row's candidates");

struct SelShared {
  uint32_t hist[kHistWords];          // bin b at b + b / 32
  uint32_t red[2 * kTW];
  uint32_t wcnt[2 * kTW];
  alignas(16) uint32_t bkey[kBucketMax];
  union {
    struct {
      int32_t opos[kMaxTopk];         // the selection's positions in output order
      uint32_t okey[kMaxTopk];        // and their keys (when the scores are wanted)
    };
    uint32_t stage[2 * kMaxTopk];     // (long rows: the candidate keys, before the selection)
  };
  uint32_t bcount;
  uint32_t s_prefix, s_need, s_cnt;
};

__device__ __forceinline__ int hslot(int b) { return b + (b >> 5); }

// Minimum and maximum over the 64 lanes (uniform results): within rows by rotations,
// then over the four row results.
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
  auto ror = [](uint32_t v, auto CTRL) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, decltype(CTRL)::value, 0xF, 0xF, false);
  };
  mn = min(mn, ror(mn, std::integral_constant<int, kDppRowRor1>{}));
  mx = max(mx, ror(mx, std::integral_constant<int, kDppRowRor1>{}));
  mn = min(mn, ror(mn, std::integral_constant<int, kDppRowRor2>{}));
  mx = max(mx, ror(mx, std::integral_constant<int, kDppRowRor2>{}));
  mn = min(mn, ror(mn, std::integral_constant<int, kDppRowRor4>{}));
  mx = max(mx, ror(mx, std::integral_constant<int, kDppRowRor4>{}));
  mn = min(mn, ror(mn, std::integral_constant<int, kDppRowRor8>{}));
  mx = max(mx, ror(mx, std::integral_constant<int, kDppRowRor8>{}));
  uint32_t a = mn, c = mx;
  mn = min(min((uint32_t)__builtin_amdgcn_readlane((int)a, 0), (uint32_t)__builtin_amdgcn_readlane((int)a, 16)),
           min((uint32_t)__builtin_amdgcn_readlane((int)a, 32), (uint32_t)__builtin_amdgcn_readlane((int)a, 48)));
  mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)c, 0), (uint32_t)__builtin_amdgcn_readlane((int)c, 16)),
           max((uint32_t)__builtin_amdgcn_readlane((int)c, 32), (uint32_t)__builtin_amdgcn_readlane((int)c, 48)));
}

// Block-wide min and max of one key pair per thread (uniform results; one barrier:
// sh.red is next written only after later barriers).
__device__ __forceinline__ void block_minmax(uint32_t& kmin, uint32_t& kmax, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_minmax(kmin, kmax);
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTW + wave] = kmax;
  }
  __syncthreads();
  kmin = lane < kTW ? sh.red[lane] : 0xffffffffu;
  kmax = lane < kTW ? sh.red[kTW + lane] : 0u;
  wave_minmax(kmin, kmax);
}

// One radix pass's threshold digit.  Wave 0 scans the 2048-bin histogram from the
// top: lane l first sums bins 2047-32l ... 2016-32l; the lane whose range holds the
// need-th largest key is found by a scan over lanes, then its 32 bins are scanned
// across lanes 0..31.  Records the bin's prefix, the count still needed inside it,
// and its size.  Call from every thread after the histogram barrier.
__device__ __forceinline__ void pick_digit(SelShared& sh, uint32_t prefix, int shift, uint32_t need) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    // the 32 bins of lane l sit in consecutive padded slots, 33 words apart per lane
    const uint32_t* hp = sh.hist + hslot(kBins - 32 - 32 * lane);
    uint32_t s = 0;
#pragma unroll 1
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s += hp[8 * g + i];
    }
    const uint32_t inc = wave_inclusive_sum(s);
    const uint64_t hit = __ballot(inc - s < need && need <= inc);
    const int L = hit ? (int)__builtin_ctzll(hit) : 0;
    const uint32_t aboveL = (uint32_t)__builtin_amdgcn_readlane((int)(inc - s), L);   // (L is uniform)
    const int b = kBins - 1 - 32 * L - lane;
    const uint32_t c = lane < 32 ? sh.hist[hslot(b)] : 0u;
    const uint32_t inc2 = aboveL + wave_inclusive_sum(c);
    if (lane < 32 && inc2 - c < need && need <= inc2) {
      sh.s_prefix = prefix | ((uint32_t)b << shift);
      sh.s_need = need - (inc2 - c);
      sh.s_cnt = c;
    }
  }
}

// 11-bit radix passes narrowing (prefix, mask, need) until the remaining bucket is
// taken whole, the bits run out (hi = number of undecided low bits) or max_passes
// passes are done.
// `hist_keys(mask, prefix, shift, dmask)` adds every key matching the prefix to the
// histogram under its digit.  `bucket(prefix, mask, need, cnt)` may resolve a small
// bucket itself and return true.
template <class HistKeys, class Bucket>
__device__ __forceinline__ void radix_passes(HistKeys hist_keys, Bucket bucket, SelShared& sh, int hi,
                                             uint32_t& prefix, uint32_t& mask, uint32_t& need,
                                             int max_passes = 8) {
  for (int pass = 0; hi > 0 && pass < max_passes; ++pass) {
    const int width = hi < 11 ? hi : 11;
    const int shift = hi - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = threadIdx.x; i < kHistWords; i += kTopkThreads) sh.hist[i] = 0u;
    if (threadIdx.x == 0) sh.bcount = 0u;
    __syncthreads();
    hist_keys(mask, prefix, shift, dmask);
    __syncthreads();
    pick_digit(sh, prefix, shift, need);
    __syncthreads();
    prefix = sh.s_prefix;
    need = sh.s_need;
    const uint32_t cnt = sh.s_cnt;
    mask |= dmask << shift;
    hi = shift;
    if (cnt == need || hi == 0 || pass + 1 == max_passes) break;   // uniform across the block
    if (cnt <= (uint32_t)kBucketMax && bucket(prefix, mask, need, cnt)) break;
  }
}

// ---- keys held in registers: key[j] is position KPT t + j; positions >= n are
// never counted
template <int KPT>
__device__ __forceinline__ bool valid_pos(int j, int n) { return KPT * (int)threadIdx.x + j < n; }

// A bucket of cnt <= 64 keys (those with in(j)) holding the need-th largest key of the
// selection: gathered into LDS, then one wave finds that key exactly, bit by bit from
// the highest bit of `undecided` down, with ballots; ties with it are taken in
// position order later.  Leaves the key in sh.s_prefix and the number of keys equal
// to it still to take in sh.s_need.  Contains barriers: call from every thread.
template <int KPT, class In>
__device__ __forceinline__ void resolve_bucket(const uint32_t (&key)[KPT], int n, In in, uint32_t need, uint32_t cnt,
                                               uint32_t undecided, SelShared& sh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool hit = valid_pos<KPT>(j, n) && in(j);
    const uint64_t bm = __ballot(hit);
    if (bm) {   // uniform: one slot reservation per wave and round
      uint32_t base = 0;
      if (lane == (int)__builtin_ctzll(bm)) base = atomicAdd(&sh.bcount, (uint32_t)__popcll(bm));
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, (int)__builtin_ctzll(bm));
      if (hit) sh.bkey[base + lanes_below(bm)] = key[j];
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint32_t kl = (uint32_t)lane < cnt ? sh.bkey[lane] : 0u;
    bool cand = (uint32_t)lane < cnt;
    uint32_t rem = need;
    for (int bit = undecided ? 31 - __clz((int)undecided) : -1; bit >= 0; --bit) {
      const uint64_t ones = __ballot(cand && ((kl >> bit) & 1u));
      const uint32_t c1 = (uint32_t)__popcll(ones);
      const bool take_ones = rem <= c1;
      if (!take_ones) rem -= c1;
      cand = cand && (((kl >> bit) & 1u) == (take_ones ? 1u : 0u));
    }
    const uint64_t left = __ballot(cand);
    if (lane == (int)__builtin_ctzll(left)) {
      sh.s_prefix = kl;
      sh.s_need = rem;
    }
  }
  __syncthreads();
}

// Single-histogram selection for rows held in registers.  kBins equal-width bins span
// the row's smallest to largest score (a monotone map: every key in a higher bin is
// larger).  On scores with a smooth distribution the bin of the k-th largest holds a
// handful of keys; they are gathered, and one wave ranks them exactly.  Returns false
// (with nothing written and the LDS reusable) when that bin holds more than
// kBucketMax keys or the value range cannot be binned; the caller then runs the radix
// passes.  On success: every key > T and the first `need` keys == T (position order)
// are the k largest.  The caller zeroes sh.hist and sh.bcount before its first
// barrier.  Requires 1 <= k <= n.  Contains barriers: call from every thread.
template <int KPT>
__device__ __forceinline__ bool threshold_one_pass(const uint32_t (&key)[KPT], const float (&x)[KPT], int n,
                                                   uint32_t k, SelShared& sh, uint32_t& T, uint32_t& need) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // a wave whose positions all lie below n (every wave but at most one) skips the checks
  const bool wave_full = KPT * (64 * wave + 64) <= n;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (wave_full) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (valid_pos<KPT>(j, n)) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
    }
  }
  wave_minmax(kmin, kmax);
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTW + wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kTW; ++w) {
    kmin = min(kmin, sh.red[w]);
    kmax = max(kmax, sh.red[kTW + w]);
  }
  if (kmin == kmax) {   // every key equal: the first k in position order
    T = kmin;
    need = k;
    return true;
  }
  const float lo = key_to_float(kmin), hi = key_to_float(kmax);
  const float scale = (float)kBins / (hi - lo);
  if (!(scale > 0.f) || !(scale < INFINITY) || !(lo > -INFINITY) || !(hi < INFINITY)) {
    __syncthreads();   // (uniform) every wave has read sh.red before the fallback writes it
    return false;
  }
  // bin = min((x - lo) * scale, 2047) as one fma: still non-decreasing in x
  const float c0 = -lo * scale;
  int bins[KPT];
  if (wave_full) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      bins[j] = (int)fminf(fmaf(x[j], scale, c0), (float)(kBins - 1));
      atomicAdd(&sh.hist[hslot(bins[j])], 1u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      bins[j] = valid_pos<KPT>(j, n) ? (int)fminf(fmaf(x[j], scale, c0), (float)(kBins - 1)) : -1;
      if (bins[j] >= 0) atomicAdd(&sh.hist[hslot(bins[j])], 1u);
    }
  }
  __syncthreads();
  pick_digit(sh, 0u, 0, k);
  __syncthreads();
  const int b = (int)sh.s_prefix;
  const uint32_t nd = sh.s_need, cnt = sh.s_cnt;
  if (cnt > (uint32_t)kBucketMax) return false;   // uniform
  // the bin's keys (a few per thread at most)
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (bins[j] == b) sh.bkey[atomicAdd(&sh.bcount, 1u)] = key[j];
  __syncthreads();
  {   // rank each bucket key among the others, 16 threads per key (4 comparisons each,
      // summed over their DPP row): the nd-th largest is T
    const uint32_t i = threadIdx.x >> 4, part = threadIdx.x & 15;
    const uint32_t mine = i < cnt ? sh.bkey[i] : 0u;
    const uint4 o4 = *(const uint4*)&sh.bkey[4 * part];
    const uint32_t o[4] = {o4.x, o4.y, o4.z, o4.w};
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = 4 * part + r < cnt;
      gt += (in && o[r] > mine) ? 1u : 0u;
      eq += (in && o[r] == mine) ? 1u : 0u;
    }
    gt = row_sum16(gt);
    eq = row_sum16(eq);
    if (part == 0 && i < cnt && gt < nd && nd <= gt + eq) {   // the keys equal to T (same values)
      sh.s_prefix = mine;
      sh.s_need = nd - gt;
    }
  }
  __syncthreads();
  T = sh.s_prefix;
  need = sh.s_need;
  return true;
}

// Finds (prefix, mask, need): the k largest of the n keys are every key with
// (key & mask) > prefix plus the first `need` keys (in position order) with
// (key & mask) == prefix.  Requires 1 <= k <= n.  ONE_PASS: stop after the first
// digit (prefix then has zeros below it: the k-th largest key lies in
// [prefix, prefix + 2^shift) and every key >= prefix is among the k largest or in
// that bin).
template <int KPT, bool ONE_PASS = false>
__device__ __forceinline__ void reg_threshold(const uint32_t (&key)[KPT], int n, uint32_t k, SelShared& sh,
                                              uint32_t& prefix, uint32_t& mask, uint32_t& need) {
  const int lane = threadIdx.x & 63;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (valid_pos<KPT>(j, n)) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  block_minmax(kmin, kmax, sh);
  const int hi = (kmin == kmax) ? 0 : 32 - __clz((int)(kmin ^ kmax));
  mask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  prefix = kmin & mask;
  need = k;
  auto hist = [&](uint32_t msk, uint32_t pre, int shift, uint32_t dmask) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (valid_pos<KPT>(j, n) && (key[j] & msk) == pre) atomicAdd(&sh.hist[hslot((key[j] >> shift) & dmask)], 1u);
    }
  };
  // a bucket of <= 64 keys: resolved exactly by one wave
  bool resolved = false;
  auto bucket = [&](uint32_t pre, uint32_t msk, uint32_t nd, uint32_t cnt) {
    auto in = [&](int j) { return (key[j] & msk) == pre; };
    resolve_bucket<KPT>(key, n, in, nd, cnt, ~msk, sh);
    resolved = true;
    return true;
  };
  radix_passes(hist, bucket, sh, hi, prefix, mask, need, ONE_PASS ? 1 : 8);
  if (resolved) {   // uniform: the exact threshold key and the count of its ties to take
    prefix = sh.s_prefix;
    need = sh.s_need;
    mask = ~0u;
  }
}

// Writes the selection in position order: out_idx[p] = idx_at(pos) for the p-th
// selected position pos, and out_score[p] its score.  Thread t's selected keys (every
// key above the threshold, and the first `need` keys equal to it overall) take
// consecutive output slots from base(t) = (keys above before t) + min(keys equal before
// t, need).  Without scores only their positions are scattered to LDS, by a loop over the
// set bits of the thread's selection mask (about one selected key in sixteen); with
// scores a loop over the KPT keys writes each selected key too.  Exactly k slots are
// then written out in order.
template <int KPT, class IdxAt>
__device__ __forceinline__ void reg_compact(const uint32_t (&key)[KPT], int n, uint32_t prefix, uint32_t mask,
                                            uint32_t need, int k, IdxAt idx_at, int32_t* oi, float* os,
                                            SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(KPT <= 16, "one selection bit per key in 16 bits");
  uint32_t gm = 0, em = 0;   // bit j: key j above / equal to the threshold
  if (KPT * (64 * wave + 64) <= n && mask == 0xffffffffu) {   // (uniform) no range check, no mask
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      gm |= (key[j] > prefix ? 1u : 0u) << j;
      em |= (key[j] == prefix ? 1u : 0u) << j;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool v = valid_pos<KPT>(j, n);
      const uint32_t kp = key[j] & mask;
      gm |= ((v && kp > prefix) ? 1u : 0u) << j;
      em |= ((v && kp == prefix) ? 1u : 0u) << j;
    }
  }
  const uint32_t ng = (uint32_t)__popc(gm), ne = (uint32_t)__popc(em);
  // exclusive scans in position order: within the wave, then over the waves before
  const uint32_t ig = wave_inclusive_sum(ng), ie = wave_inclusive_sum(ne);
  if (lane == 63) {
    sh.wcnt[wave] = ig;
    sh.wcnt[kTW + wave] = ie;
  }
  __syncthreads();
  const uint32_t wg = lane < wave ? sh.wcnt[lane] : 0u;
  const uint32_t we = lane < wave ? sh.wcnt[kTW + lane] : 0u;
  const uint32_t gb = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(wg), 63) + ig - ng;
  const uint32_t eb = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(we), 63) + ie - ne;
  // the equal keys this thread takes: the lowest min(need - eb, ne) set bits of em
  uint32_t et = 0;
  if (eb < need) {
    const uint32_t take = min(need - eb, ne);
    et = em;
    for (uint32_t d = ne; d > take; --d) et &= ~(1u << (31 - __clz((int)et)));   // drop the highest
  }
  uint32_t sel = gm | et;
  uint32_t p = gb + min(eb, need);
  const int pos0 = KPT * (int)threadIdx.x;
  if (os) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if ((sel >> j) & 1u) {
        if (p < (uint32_t)k) {
          sh.opos[p] = pos0 + j;
          sh.okey[p] = key[j];
        }
        ++p;
      }
    }
  } else {
    while (sel) {
      const int j = __builtin_ctz(sel);
      if (p < (uint32_t)k) sh.opos[p] = pos0 + j;
      ++p;
      sel &= sel - 1u;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kTopkThreads) {
    oi[i] = idx_at(sh.opos[i]);
    if (os) os[i] = key_to_float(sh.okey[i]);
  }
}

// ---- keys read from global memory on every pass (long rows whose sampled
// threshold missed): the same selection, slower.
template <class KeyAt>
__device__ __forceinline__ void global_select(KeyAt key_at, int n, int k, int32_t* oi, float* os, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = threadIdx.x; i < n; i += kTopkThreads) {
    const uint32_t key = key_at(i);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
  block_minmax(kmin, kmax, sh);
  const int hi0 = (kmin == kmax) ? 0 : 32 - __clz((int)(kmin ^ kmax));
  uint32_t mask = hi0 >= 32 ? 0u : ~((1u << hi0) - 1u);
  uint32_t prefix = kmin & mask, need = (uint32_t)k;
  auto hist = [&](uint32_t msk, uint32_t pre, int shift, uint32_t dmask) {
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kTopkThreads) {
      const uint32_t key = key_at(i);
      if ((key & msk) == pre) atomicAdd(&sh.hist[hslot((key >> shift) & dmask)], 1u);
    }
  };
  auto no_bucket = [](uint32_t, uint32_t, uint32_t, uint32_t) { return false; };
  radix_passes(hist, no_bucket, sh, hi0, prefix, mask, need);
  // each wave owns a contiguous range of positions; ballots place the selection in order
  const int per = (n + kTopkThreads - 1) / kTopkThreads * 64;
  const int lo = wave * per;
  const int hi = min(n, lo + per);
  uint32_t gt = 0, eq = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool v = i < hi;
    const uint32_t kp = v ? (key_at(i) & mask) : 0u;
    gt += __popcll(__ballot(v && kp > prefix));
    eq += __popcll(__ballot(v && kp == prefix));
  }
  if (lane == 0) {
    sh.wcnt[wave] = gt;
    sh.wcnt[kTW + wave] = eq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += sh.wcnt[w];
    eq_before += sh.wcnt[kTW + w];
  }
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t eq_seen = eq_before;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool v = i < hi;
    const uint32_t key = v ? key_at(i) : 0u;
    const uint32_t kp = key & mask;
    const bool g = v && kp > prefix;
    const bool e = v && kp == prefix;
    const uint64_t be = __ballot(e);
    const bool sel = g || (e && eq_seen + lanes_below(be) < need);
    const uint64_t bs = __ballot(sel);
    const uint32_t p = pos + lanes_below(bs);
    if (sel && p < (uint32_t)k) {
      oi[p] = i;
      if (os) os[p] = key_to_float(key);
    }
    pos += __popcll(bs);
    eq_seen += __popcll(be);
  }
}

__device__ __forceinline__ int row_visible(const IndexArgs& A, long row) {
  const int b = (int)row / A.n_q;   // (rows are an int count: no 64-bit division)
  const int ne = min(A.n_entries[b], A.n_max);
  return visible_entries(A.q_pos[row], ne, A.m);
}

// V <= k: every visible entry in order (through map, when given), then -1.
__device__ __forceinline__ void take_all(const float* src, int V, int k, int32_t* oi, float* os,
                                         const int32_t* map = nullptr) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    oi[i] = i < V ? (map ? map[i] : i) : -1;
    if (os) os[i] = i < V ? src[i] : -INFINITY;
  }
}

// Raw buffer loads over exactly `n_valid` floats: one address register, and
// positions past the end read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t float_rsrc(const float* p, int n_valid) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, n_valid * 4, 0x00020000);
}

// One row of V <= KPT * 1024 scores, held in registers (key[] loaded by load_row),
// 16 bytes per load.  The range covers n rounded up to four positions: score rows
// live in the library's workspace, which keeps 16 bytes of slack after them, and the
// positions past n are never counted.
template <int KPT>
__device__ __forceinline__ void load_row(const float* src, int n, uint32_t (&key)[KPT], float (&x)[KPT]) {
  const __amdgpu_buffer_rsrc_t rs = float_rsrc(src, (n + 3) & ~3);
  static_assert(KPT % 4 == 0, "keys are loaded four at a time");
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, ((int)threadIdx.x * KPT + 4 * q) * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[4 * q + i] = __uint_as_float(v[i]);
      key[4 * q + i] = order_key(x[4 * q + i]);
    }
  }
}

// The caller zeroes sh.hist and sh.bcount before its first barrier (threshold_one_pass).
// x: the keys' scores; map: the row's position map (rescoring: slot p of the row is
// candidate map[p]) or none.
template <int KPT>
__device__ __forceinline__ void select_reg_row(uint32_t (&key)[KPT], const float (&x)[KPT], int V, int k, int32_t* oi,
                                               float* os, SelShared& sh, const int32_t* map) {
  auto idx_at = [map](int pos) { return map ? map[pos] : pos; };
  uint32_t prefix, mask = 0xffffffffu, need;
  if (!threshold_one_pass<KPT>(key, x, V, (uint32_t)k, sh, prefix, need))
    reg_threshold<KPT>(key, V, (uint32_t)k, sh, prefix, mask, need);
  reg_compact<KPT>(key, V, prefix, mask, need, k, idx_at, oi, os, sh);
}

// Zeroes the histogram and the bucket counter (before the caller's first barrier).
__device__ __forceinline__ void clear_select_lds(SelShared& sh) {
  for (int i = threadIdx.x; i < kHistWords; i += kTopkThreads) sh.hist[i] = 0u;
  if (threadIdx.x == 0) sh.bcount = 0u;
}

// ---- rows of up to KPT * 1024 entries: one workgroup per row
// (two workgroups per CU, so that one's loads and barriers overlap the other's work on
// many rows: at most 64 registers per lane)
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_rows_kernel(IndexArgs A, const float* scores, int32_t* out_idx, float* out_score) {
  __shared__ SelShared sh;
  const long row = blockIdx.x;
  const float* src = scores + row * A.n_max;
  // the row's scores are requested before the visible count arrives (positions past
  // it are never counted)
  uint32_t key[KPT];
  float x[KPT];
  load_row<KPT>(src, A.n_max, key, x);
  const int32_t* map = A.map ? A.map + row * A.n_max : nullptr;
  clear_select_lds(sh);
  const int V = row_visible(A, row);
  const int k = A.topk;
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;
  if (V <= k) {
    take_all(src, V, k, oi, os, map);
    return;
  }
  select_reg_row<KPT>(key, x, V, k, oi, os, sh, map);
}

// ---- long rows, launch 1: the threshold from a fixed sample of the row, then the
// keys at or above it, per chunk of kChunk keys, in index order
struct LongWs {
  uint32_t* counts;   // [rows, chunks]
  uint32_t* ckey;     // [rows, n_max]
  int32_t* cidx;      // [rows, n_max]
  int chunks;
};

constexpr int kFilterGroups = kTopkThreads / kFilterThreads;   // chunks per workgroup

// The threshold key: the lower edge of the first-digit bin that holds the key of rank
// r in a fixed sample of the row, r chosen to leave ~3k keys of the row at or above
// it (at most three quarters of the candidate capacity; a larger k keeps a smaller
// margin).  One radix pass: the bin adds a few samples' worth of keys beyond rank r.
// The sample is 64 runs of 64 consecutive keys, evenly spaced over the row's n_max
// slots (n_max > kRegKeys): it does not wait for the visible count, since the
// indexer leaves -inf at and past V (at the bottom of the order, below any rank the
// sample is asked for while V is near n_max).  Any threshold gives the exact
// selection: the candidate kernel falls back to the whole row when it passed fewer
// than k keys or more than kCandCap.
constexpr int kSampleKpt = kSample / kTopkThreads;
// This thread's sample scores (requested before anything else the filter loads: a
// wait for them is then a wait for them alone).
__device__ __forceinline__ void sample_load(const IndexArgs& A, const float* src, float (&x)[kSampleKpt]) {
  constexpr int kRun = 64, kRuns = kSample / kRun;
#pragma unroll
  for (int j = 0; j < kSampleKpt; ++j) {
    const int i = kSampleKpt * (int)threadIdx.x + j;   // sample i: key i % 64 of run i / 64
    x[j] = src[(long)(i / kRun) * (A.n_max / kRuns) + i % kRun];
  }
}
__device__ __forceinline__ uint32_t sample_threshold(const IndexArgs& A, const float (&x)[kSampleKpt], SelShared& sh) {
  constexpr int KPT = kSampleKpt;
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = order_key(x[j]);
  const int want = min(3 * A.topk, kCandCap * 3 / 4);
  int r = (want * kSample + A.n_max - 1) / A.n_max;   // (< 2^31: want <= 12,288)
  r = r < 1 ? 1 : (r > kSample ? kSample : r);
  uint32_t prefix, mask, need;
  reg_threshold<KPT, true>(key, kSample, (uint32_t)r, sh, prefix, mask, need);
  return prefix;
}

// Every workgroup of a row forms the same threshold (the sample and its selection are
// deterministic), then each group of kFilterThreads threads filters one chunk.
__global__ __launch_bounds__(kTopkThreads) void topk_filter_kernel(IndexArgs A, const float* scores, LongWs L) {
  __shared__ SelShared sh;
  __shared__ uint32_t wtot[kTopkThreads / 64];
  const long row = blockIdx.y;
  const float* src = scores + row * A.n_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kGw = kFilterThreads / 64;                  // waves per group
  const int grp = wave / kGw, gw = wave % kGw;
  const int c = blockIdx.x * kFilterGroups + grp;
  const int c0 = c * kChunk;
  constexpr int kIt = kChunk / kFilterThreads;              // 16 keys per lane
  constexpr int kPerWave = kChunk / kGw;
  const int w0 = c0 + gw * kPerWave;
  // the sample, this chunk's scores and the visible count are requested together
  // (slots below n_max lie in the row; those at or past V are never taken)
  float smp[kSampleKpt];
  sample_load(A, src, smp);
  // (raw buffer loads over the row's n_max slots, 0 past them: no branch, so the wait
  // for the sample counts exactly the loads issued after it)
  const __amdgpu_buffer_rsrc_t rs = float_rsrc(src, A.n_max);
  float sc[kIt];
#pragma unroll
  for (int r = 0; r < kIt; ++r)
    sc[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (w0 + r * 64 + lane) * 4, 0, 0));
  const int V = row_visible(A, row);
  const uint32_t tau = sample_threshold(A, smp, sh);
  if (V <= kRegKeys || V <= A.topk) return;   // (uniform, after the threshold's barriers)
  uint32_t key[kIt];
  uint32_t cnt = 0;
#pragma unroll
  for (int r = 0; r < kIt; ++r) {
    const int i = w0 + r * 64 + lane;
    key[r] = i < V ? order_key(sc[r]) : 0u;
    cnt += __popcll(__ballot(i < V && key[r] >= tau));
  }
  if (lane == 0) wtot[wave] = cnt;
  __syncthreads();
  uint32_t pos = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kGw; ++w) {
    pos += w < gw ? wtot[grp * kGw + w] : 0u;
    total += wtot[grp * kGw + w];
  }
  if (c >= L.chunks) return;   // (after the last barrier)
  uint32_t* ck = L.ckey + row * A.n_max + c0;
  int32_t* ci = L.cidx + row * A.n_max + c0;
#pragma unroll
  for (int r = 0; r < kIt; ++r) {
    const int i = w0 + r * 64 + lane;
    const bool sel = i < V && key[r] >= tau;
    const uint64_t bs = __ballot(sel);
    if (sel) {
      const uint32_t p = pos + lanes_below(bs);
      ck[p] = key[r];
      ci[p] = i;
    }
    pos += __popcll(bs);
  }
  if (threadIdx.x == (unsigned)(grp * kFilterThreads)) L.counts[row * L.chunks + c] = total;
}

// Exact selection among the M candidates of a long row (KPT * 1024 >= M <= kCandCap).
// Chunk c's candidates (stored from c * kChunk in the row's lists) are copied, kCopyT
// threads per chunk with coalesced reads, to candidate positions coff[c] .. in LDS
// (keys to the staging area, row positions to cand_idx); thread t then takes
// candidates KPT t .. KPT t + KPT - 1.  The first kSpec per thread of the first
// kTopkThreads / kCopyT chunks were read before the counts were known (spk, spi).
constexpr int kCopyT = 16, kSpec = 8;
template <int KPT>
__device__ __forceinline__ void select_candidates(const uint32_t (&spk)[kSpec], const int32_t (&spi)[kSpec],
                                                  const uint32_t* gk, const int32_t* gi, const uint32_t* coff,
                                                  int nch, int M, int k, int32_t* cand_idx, int32_t* oi,
                                                  float* os, SelShared& sh) {
  const int c_sp = (int)threadIdx.x / kCopyT;
  for (int c = c_sp; c < nch; c += kTopkThreads / kCopyT) {
    const int base = (int)coff[c], n = (int)coff[c + 1] - base;
    const long src = (long)c * kChunk;
    int i = (int)threadIdx.x % kCopyT;
    if (c == c_sp) {
#pragma unroll
      for (int j = 0; j < kSpec; ++j) {
        if (i + kCopyT * j < n) {
          sh.stage[base + i + kCopyT * j] = spk[j];
          cand_idx[base + i + kCopyT * j] = spi[j];
        }
      }
      i += kCopyT * kSpec;
    }
    for (; i < n; i += kCopyT) {
      sh.stage[base + i] = gk[src + i];
      cand_idx[base + i] = gi[src + i];
    }
  }
  __syncthreads();
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int c = KPT * (int)threadIdx.x + j;
    key[j] = c < M ? sh.stage[c] : 0u;
  }
  // (the staging area is next written by the compaction, after the threshold's barriers)
  auto idx_at = [&](int c) { return cand_idx[c]; };
  clear_select_lds(sh);   // (the staging barrier above precedes the next one)
  uint32_t prefix, mask = 0xffffffffu, need;
  float x[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) x[j] = key_to_float(key[j]);
  if (!threshold_one_pass<KPT>(key, x, M, (uint32_t)k, sh, prefix, need))
    reg_threshold<KPT>(key, M, (uint32_t)k, sh, prefix, mask, need);
  reg_compact<KPT>(key, M, prefix, mask, need, k, idx_at, oi, os, sh);
}

// ---- long rows, launch 2: exact selection among the candidates (or the whole row)
__global__ __launch_bounds__(kTopkThreads) void topk_candidates_kernel(IndexArgs A, const float* scores, LongWs L,
                                                                       int32_t* out_idx, float* out_score) {
  __shared__ SelShared sh;
  __shared__ uint32_t coff[kMaxChunks + 1];
  __shared__ int32_t cand_idx[kCandCap];
  const long row = blockIdx.x;
  const int k = A.topk;
  const float* src = scores + row * A.n_max;
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;
  const uint32_t* gk = L.ckey + row * A.n_max;
  const int32_t* gi = L.cidx + row * A.n_max;
  // Requested together with the visible count: the first candidates of the first
  // chunks and the first 64 chunk counts (reads inside the row's lists and counts;
  // what lies past a chunk's count, or in chunks at or past V, is never used)
  uint32_t spk[kSpec];
  int32_t spi[kSpec];
  {
    const int c = (int)threadIdx.x / kCopyT, i = (int)threadIdx.x % kCopyT;
#pragma unroll
    for (int j = 0; j < kSpec; ++j) {
      const long p = (long)c * kChunk + i + kCopyT * j;
      const bool in = c < L.chunks && p < A.n_max;
      spk[j] = in ? gk[p] : 0u;
      spi[j] = in ? gi[p] : -1;
    }
  }
  const int lane = threadIdx.x & 63;
  const uint32_t cnt0 = (threadIdx.x < 64 && lane < L.chunks) ? L.counts[row * L.chunks + lane] : 0u;
  const int V = row_visible(A, row);
  if (V <= k) {
    take_all(src, V, k, oi, os);
    return;
  }
  if (V <= kRegKeys) {
    uint32_t key[kMaxKpt];
    float x[kMaxKpt];
    load_row<kMaxKpt>(src, V, key, x);
    clear_select_lds(sh);
    select_reg_row<kMaxKpt>(key, x, V, k, oi, os, sh, nullptr);
    return;
  }
  const int nch = (V + kChunk - 1) / kChunk;
  // chunk offsets (exclusive scan of the per-chunk counts, one wave)
  if (threadIdx.x < 64) {
    uint32_t run = 0;
    for (int base = 0; base < nch; base += 64) {
      const int c = base + lane;
      const uint32_t v = c < nch ? (base == 0 ? cnt0 : L.counts[row * L.chunks + c]) : 0u;
      const uint32_t inc = wave_inclusive_sum(v);
      if (c < nch) coff[c] = run + inc - v;
      run += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    }
    if (lane == 0) coff[nch] = run;
  }
  __syncthreads();
  const int M = (int)coff[nch];
  if (M < k || M > kCandCap) {   // the sample's threshold missed: select from the row itself
    auto key_at = [&](int i) { return order_key(src[i]); };
    global_select(key_at, V, k, oi, os, sh);
    return;
  }
  // as few registers per thread as the candidate count allows
  if (M <= 4 * kTopkThreads) select_candidates<4>(spk, spi, gk, gi, coff, nch, M, k, cand_idx, oi, os, sh);
  else if (M <= 8 * kTopkThreads) select_candidates<8>(spk, spi, gk, gi, coff, nch, M, k, cand_idx, oi, os, sh);
  else select_candidates<kCandCap / kTopkThreads>(spk, spi, gk, gi, coff, nch, M, k, cand_idx, oi, os, sh);
}

static int long_chunks(const IndexArgs& A) { return (A.n_max + kChunk - 1) / kChunk; }

size_t topk_workspace_bytes(const IndexArgs& A) {
  if (A.n_max <= kRegKeys) return 0;
  const size_t rows = (size_t)A.batch * A.n_q;
  const size_t chunks = (size_t)long_chunks(A);
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return r256(rows * chunks * 4) + 2 * r256(rows * (size_t)A.n_max * 4);
}

hipError_t launch_topk_rows(const IndexArgs& A, const float* scores, int32_t* out_idx, float* out_score, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  const long rows = (long)A.batch * A.n_q;
  if (rows <= 0) return hipSuccess;
  if (A.topk < 1 || A.topk > kMaxTopk) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows), block(kTopkThreads);
  if (A.n_max <= kRegKeys) {
    if (A.n_max <= 4096) return launch("topk", topk_rows_kernel<4>, grid, block, 0, s, A, scores, out_idx, out_score);
    if (A.n_max <= 8192) return launch("topk", topk_rows_kernel<8>, grid, block, 0, s, A, scores, out_idx, out_score);
    return launch("topk", topk_rows_kernel<16>, grid, block, 0, s, A, scores, out_idx, out_score);
  }
  const int chunks = long_chunks(A);
  if (chunks > kMaxChunks || ws_bytes < topk_workspace_bytes(A) || !ws) return hipErrorInvalidValue;
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = (char*)ws;
  LongWs L;
  L.counts = (uint32_t*)p;
  p += r256((size_t)rows * chunks * 4);
  L.ckey = (uint32_t*)p;
  p += r256((size_t)rows * A.n_max * 4);
  L.cidx = (int32_t*)p;
  L.chunks = chunks;
  const unsigned fgroups = (unsigned)((chunks + kFilterGroups - 1) / kFilterGroups);
  hipError_t e = launch("topk", topk_filter_kernel, dim3(fgroups, (unsigned)rows), block, 0, s, A, scores, L);
  if (e != hipSuccess) return e;
  return launch("topk", topk_candidates_kernel, grid, block, 0, s, A, scores, L, out_idx, out_score);
}

}  // namespace csa
