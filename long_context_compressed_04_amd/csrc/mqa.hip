// Core multi-query attention of CSA (sparse: top-k entries + sliding window) and
// HCA (dense: every visible compressed entry + sliding window).
//
// Techniques map "DeepSeek-V4-Pro": "Grouped-query attention" (all query heads
// broadcast from one KV head; the entry is key and value), "Sliding-window
// attention" (window 128, w-1 past tokens plus the current one), "QK
// normalization".  Anthology record ARXIV-2606.19348, Key takeaways: an RMSNorm on
// each query head and on the single compressed-KV head just before the core
// attention.  "DeepSeek v4" summary page, "Compressed Sparse Attention": the
// selected compressed entries plus a small set of sliding-window entries; hybrid
// CSA/HCA section: HCA keeps attention dense.
//
// Attended items of a query (sparse): its `topk` index slots (-1 masked), then the
// window tokens max(0, t-w+1) .. t.  Dense: entries 0 .. V(t)-1, then the window.
//
// bf16 kernel (head_dim 512): a workgroup = NW waves x 16 heads, one (query, split)
// unit.  Item tiles of 32 rows are staged in LDS (row-major, padded); each row's
// 1/rms comes from the same load.  Per wave and tile:
//   S^T[32 items x 16 heads] = K . q^T   (v_mfma_f32_16x16x32_bf16; A = K rows from
//                                         LDS, B = normalised q^T held in registers)
//   online softmax per head column (exp2, fp32)
//   O^T[512 x 16] += V^T . P^T           (A = V^T via ds_read_b64_tr_b16 from the same
//                                         row-major tile, B = P^T straight from the
//                                         S^T registers: the MFMA's k order is chosen
//                                         to match the rows each lane already holds)
// RMSNorm is folded: q is normalised (times g^2) before the product, 1/rms of each
// row scales its logit and its softmax weight, and g multiplies the output.
// Splits write fp32 partials (unnormalised O, running max, sum) that a second
// kernel combines in fixed split order (deterministic).
#include "csa_device.hpp"
#include "csa_kernels.hpp"

namespace csa {

// Item i of a query -> source row pointer (nullptr = masked).
struct ItemSource {
  const uint8_t* kv;      // sequence base of kv
  const uint8_t* raw;     // sequence base of kv_raw
  const int32_t* idx;     // query's index slots (sparse) or nullptr (dense)
  int n_first;            // topk (sparse) or V (dense)
  int kv_rows;            // rows of kv that may be read
  int win_lo;             // first window token
  int raw_base, raw_cap;
  int row_bytes;
  int idx_off;            // idx[i - idx_off] holds slot i
  __device__ __forceinline__ const uint8_t* row(int i) const {
    if (i < n_first) {
      int e = idx ? idx[i - idx_off] : i;
      if (e < 0 || e >= kv_rows) return nullptr;
      return kv + (long)e * row_bytes;
    }
    int r = win_lo + (i - n_first) - raw_base;
    if (r < 0 || r >= raw_cap) return nullptr;
    return raw + (long)r * row_bytes;
  }
};

__device__ __forceinline__ void query_items(const MqaArgs& A, int b, long row, int elem_bytes, ItemSource& src,
                                            int& total) {
  const int t = A.q_pos[row];
  const int win_lo = max(0, t - A.window + 1);
  const int n_win = A.window > 0 ? max(0, t - win_lo + 1) : 0;
  src.row_bytes = A.dim * elem_bytes;
  src.kv = (const uint8_t*)A.kv + (long)b * A.kv_cap * src.row_bytes;
  src.raw = (const uint8_t*)A.kv_raw + (long)b * A.raw_cap * src.row_bytes;
  src.win_lo = win_lo;
  src.raw_base = A.raw_base[b];
  src.raw_cap = A.raw_cap;
  src.idx_off = 0;
  if (A.dense) {
    const int ne = min(min(A.n_entries[b], A.n_max), A.kv_cap);
    src.idx = nullptr;
    src.n_first = visible_entries(t, ne, A.m);
    src.kv_rows = ne;
  } else {
    src.idx = A.idx + row * A.topk;
    src.n_first = A.topk;
    src.kv_rows = A.kv_cap;
  }
  total = src.n_first + n_win;
}

// ---------------------------------------------------------------- fp32 (VALU)
// One workgroup (4 waves) per (sequence, query, head).  Each wave walks every 4th
// item with the head dimension spread over its lanes; online softmax per wave, then
// a 4-way merge.  For the fp32 workloads (head_dim <= 512).
constexpr int kF32Waves = 4;

__global__ __launch_bounds__(kF32Waves * 64) void mqa_f32_kernel(MqaArgs A) {
  const int h = blockIdx.x, qi = blockIdx.y, b = blockIdx.z;
  const long row = (long)b * A.n_q + qi;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = A.dim;
  constexpr int PER = 8;  // dims per lane (D <= 512)
  __shared__ float sm[kF32Waves], sl[kF32Waves];
  __shared__ float so[kF32Waves][512];

  ItemSource src;
  int total;
  query_items(A, b, row, 4, src, total);

  const float* qrow = (const float*)A.q + (row * A.heads + h) * D;
  float qv[PER], g[PER];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int d = lane + 64 * j;
    qv[j] = d < D ? qrow[d] : 0.f;
    g[j] = (d < D) ? (A.gamma ? A.gamma[d] : 1.f) : 0.f;
    ss = fmaf(qv[j], qv[j], ss);
  }
  ss = wave_sum(ss);
  const float qinv = 1.f / sqrtf(ss / D + A.eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) qv[j] = qv[j] * qinv * g[j] * g[j];  // q_hat * g (g of k_hat folded)

  float m_run = -INFINITY, l_run = 0.f, acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;

  for (int i = wave; i < total; i += kF32Waves) {
    const float* kr = (const float*)src.row(i);
    if (!kr) continue;
    float kv[PER], s2 = 0.f, dot = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int d = lane + 64 * j;
      kv[j] = d < D ? kr[d] : 0.f;
      s2 = fmaf(kv[j], kv[j], s2);
      dot = fmaf(qv[j], kv[j], dot);
    }
    s2 = wave_sum(s2);
    dot = wave_sum(dot);
    const float kinv = 1.f / sqrtf(s2 / D + A.eps);
    const float logit = A.scale * dot * kinv;
    const float m_new = fmaxf(m_run, logit);
    const float corr = expf(m_run - m_new);
    const float p = expf(logit - m_new);
    l_run = l_run * corr + p;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = acc[j] * corr + p * kinv * kv[j];
    m_run = m_new;
  }
  if (lane == 0) { sm[wave] = m_run; sl[wave] = l_run; }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int d = lane + 64 * j;
    if (d < D) so[wave][d] = acc[j];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < kF32Waves; ++w) M = fmaxf(M, sm[w]);
  float L = 0.f, fw[kF32Waves];
  for (int w = 0; w < kF32Waves; ++w) {
    fw[w] = (sm[w] == -INFINITY) ? 0.f : expf(sm[w] - M);
    L += sl[w] * fw[w];
  }
  float* orow = (float*)A.out + (row * A.heads + h) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.f;
    for (int w = 0; w < kF32Waves; ++w) o += so[w][d] * fw[w];
    orow[d] = (L > 0.f) ? o / L * (A.gamma ? A.gamma[d] : 1.f) : 0.f;
  }
  if (A.lse && threadIdx.x == 0) A.lse[row * A.heads + h] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

// ---------------------------------------------------------------- bf16 (MFMA)
constexpr int kD = 512;
constexpr int kTile = 32;
constexpr int kRowB = kD * 2 + 16;      // LDS row stride in bytes (padded)

struct MqaLaunch {
  int nsplit, ips, n_hg, units, nw;   // nw: waves per workgroup (16 heads each)
  int slots;                          // index slots of a split copied to LDS
};

__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void mqa_bf16_kernel(MqaArgs A, MqaLaunch L, float* part_o, float* part_ml) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const tiles = lds;                                    // [2][kTile][kRowB]
  float* const inv_rms = (float*)(lds + 2 * kTile * kRowB);      // [2][kTile]
  int32_t* const slot_idx = (int32_t*)(inv_rms + 2 * kTile);     // [L.ips] (sparse)

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  // ---- XCD-aware unit mapping: every head group of a unit runs on the same XCD
  const int f = blockIdx.x;
  const int xcd = f & 7, r8 = f >> 3;
  const int hg = r8 % L.n_hg, ug = r8 / L.n_hg;
  const int unit = ug * 8 + xcd;
  if (unit >= L.units) return;
  const long row = unit / L.nsplit;
  const int split = unit % L.nsplit;
  const int b = (int)(row / A.n_q);
  const int head = hg * (NW * 16) + wave * 16 + c16;   // this lane's head (column)

  ItemSource src;
  int total;
  query_items(A, b, row, 2, src, total);
  const int it0 = split * L.ips;
  const int it1 = min(total, it0 + L.ips);
  // index slots of this split, copied once so that row addresses need no global load
  if (src.idx && L.slots) {
    for (int i = threadIdx.x; i < L.ips; i += NW * 64) {
      const int it = it0 + i;
      slot_idx[i] = (it < min(it1, src.n_first)) ? src.idx[it] : -1;
    }
    src.idx = slot_idx;           // item i < n_first reads slot_idx[i - it0]
    src.idx_off = it0;
  }
  __syncthreads();

  // ---- normalised q (times g^2) as B operands: dims 32*ks + 8*g + [0, 8)
  bf16x8_t qf[16];
  {
    const uint16_t* qrow = (const uint16_t*)A.q + (row * A.heads + head) * kD;
    uint4 raw[16];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      raw[ks] = *(const uint4*)(qrow + 32 * ks + 8 * g);
      uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xffff0000u);
        ss = fmaf(lo, lo, fmaf(hi, hi, ss));
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float qinv = 1.f / sqrtf(ss * (1.f / kD) + A.eps);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
      uint32_t o4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = 32 * ks + 8 * g + 2 * k;
        float g0 = A.gamma ? A.gamma[d0] : 1.f, g1 = A.gamma ? A.gamma[d0 + 1] : 1.f;
        float lo = __uint_as_float(w4[k] << 16) * qinv * g0 * g0;
        float hi = __uint_as_float(w4[k] & 0xffff0000u) * qinv * g1 * g1;
        o4[k] = pack_bf16x2(lo, hi);
      }
      qf[ks] = as_bf16x8(make_uint4(o4[0], o4[1], o4[2], o4[3]));
    }
  }

  const float sl2 = A.scale * kLog2e;  // logits in log2 units
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Tile pipeline: rows of tile i+1 are fetched into registers while tile i is
  // computed from LDS; two LDS buffers, one barrier per tile.
  constexpr int RPW = kTile / NW;   // rows each wave fetches per tile
  uint4 stage[RPW];
  bool stage_ok[RPW];
  auto fetch = [&](int tb) {
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int item = tb + wave + NW * rr;
      const uint8_t* p = (item < it1) ? src.row(item) : nullptr;
      stage_ok[rr] = p != nullptr;
      stage[rr] = p ? *(const uint4*)(p + 16 * lane) : make_uint4(0, 0, 0, 0);
    }
  };
  if (it0 < it1) fetch(it0);
  int buf = 0;
  for (int tb = it0; tb < it1; tb += kTile, buf ^= 1) {
    uint8_t* const tile = tiles + buf * (kTile * kRowB);
    float* const irms = inv_rms + buf * kTile;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = wave + NW * rr;
      const uint4 v = stage[rr];
      *(uint4*)(tile + r * kRowB + 16 * lane) = v;
      uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xffff0000u);
        ss = fmaf(lo, lo, fmaf(hi, hi, ss));
      }
      ss = wave_sum(ss);
      if (lane == 0) irms[r] = stage_ok[rr] ? 1.f / sqrtf(ss * (1.f / kD) + A.eps) : 0.f;
    }
    __syncthreads();
    if (tb + kTile < it1) fetch(tb + kTile);

    // ---- S^T = K . q^T for items [0,16) and [16,32)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int cb = (32 * ks + 8 * g) * 2;
      bf16x8_t a0 = as_bf16x8(*(const uint4*)(tile + c16 * kRowB + cb));
      bf16x8_t a1 = as_bf16x8(*(const uint4*)(tile + (16 + c16) * kRowB + cb));
      s0 = mfma16x16x32(a0, qf[ks], s0);
      s1 = mfma16x16x32(a1, qf[ks], s1);
    }
    // ---- online softmax for this lane's head over its 8 items (16*bb + 4*g + r)
    float lg[8], ir[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i0 = 4 * g + r, i1 = 16 + 4 * g + r;
      ir[r] = irms[i0];
      ir[4 + r] = irms[i1];
      lg[r] = (ir[r] > 0.f) ? s0[r] * sl2 * ir[r] : -INFINITY;
      lg[4 + r] = (ir[4 + r] > 0.f) ? s1[r] * sl2 * ir[4 + r] : -INFINITY;
    }
    float tmax = lg[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, lg[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // Every head sees the same masked items, so m_new == -inf (nothing valid yet)
    // is uniform across the wave; written branch-free all the same, because the
    // MFMAs and transpose reads below are cross-lane.
    const float m_new = fmaxf(m_run, tmax);
    const bool none = m_new == -INFINITY;
    const float corr = none ? 1.f : exp2f(m_run - m_new);   // m_run = -inf -> 0
    float pw[8], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float p = none ? 0.f : exp2f(lg[r] - m_new);          // masked: exp2(-inf) = 0
      psum += p;
      pw[r] = p * ir[r];                                    // weight on the raw row (1/rms folded)
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    uint4 pk = make_uint4(pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]), pack_bf16x2(pw[4], pw[5]),
                          pack_bf16x2(pw[6], pw[7]));
    const bf16x8_t pb = as_bf16x8(pk);
    // ---- O^T += V^T . P^T
    const uint8_t* base1 = tile + (4 * g + (c16 >> 2)) * kRowB + 8 * (c16 & 3);
    const uint8_t* base2 = base1 + 16 * kRowB;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      i16x4_t v0 = lds_read_tr16(base1 + 32 * db);
      i16x4_t v1 = lds_read_tr16(base2 + 32 * db);
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      i16x8_t vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[db] = o[db] * corr;
      o[db] = mfma16x16x32(__builtin_bit_cast(bf16x8_t, vv), pb, o[db]);
    }
  }

  // ---- finish: total sum per head across the 4 lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (L.nsplit == 1) {
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* orow = (uint16_t*)A.out + (row * A.heads + head) * kD;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const int d0 = 16 * db + 4 * g;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[db][r] * inv_l * (A.gamma ? A.gamma[d0 + r] : 1.f);
      *(uint2*)(orow + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    if (A.lse && g == 0) A.lse[row * A.heads + head] = l_run > 0.f ? m_run * kLn2 + logf(l_run) : -INFINITY;
  } else {
    float* po = part_o + (((long)row * L.nsplit + split) * A.heads + head) * kD;
#pragma unroll
    for (int db = 0; db < 32; ++db) *(f32x4_t*)(po + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      float* pm = part_ml + (((long)row * L.nsplit + split) * A.heads + head) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// Fixed-order merge of split partials: out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
constexpr int kMaxSplit = 128;

__global__ __launch_bounds__(128) void mqa_combine_kernel(MqaArgs A, MqaLaunch L, const float* part_o,
                                                          const float* part_ml) {
  const int head = blockIdx.x;
  const long row = blockIdx.y;
  const int S = L.nsplit;
  __shared__ float ms[kMaxSplit], ls[kMaxSplit], wts[kMaxSplit];
  __shared__ float s_M, s_L;
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const float* pm = part_ml + ((row * S + s) * A.heads + head) * 2;
    ms[s] = pm[0];
    ls[s] = pm[1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ms[s]);
    float Ls = 0.f;
    for (int s = 0; s < S; ++s) {
      const float w = (ms[s] == -INFINITY) ? 0.f : exp2f(ms[s] - M);
      wts[s] = w;
      Ls += ls[s] * w;
    }
    s_M = M;
    s_L = Ls;
  }
  __syncthreads();
  const float Lsum = s_L;
  const float inv_l = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int d0 = threadIdx.x * 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = part_o + ((row * S) * A.heads + head) * kD + d0;
  const long sstride = (long)A.heads * kD;
#pragma unroll 8
  for (int s = 0; s < S; ++s) acc += *(const f32x4_t*)(po + s * sstride) * wts[s];
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = acc[r] * inv_l * (A.gamma ? A.gamma[d0 + r] : 1.f);
  uint16_t* orow = (uint16_t*)A.out + (row * A.heads + head) * kD;
  *(uint2*)(orow + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  if (A.lse && threadIdx.x == 0) A.lse[row * A.heads + head] = Lsum > 0.f ? s_M * kLn2 + logf(Lsum) : -INFINITY;
}

static MqaLaunch plan_mqa(const MqaArgs& A) {
  MqaLaunch L;
  L.nw = (A.heads % 64 == 0) ? 4 : ((A.heads % 32 == 0) ? 2 : 1);
  L.n_hg = A.heads / (L.nw * 16);
  const long rows = (long)A.batch * A.n_q;
  const int total_max = (A.dense ? A.n_max : A.topk) + A.window;
  const int tiles_max = (total_max + kTile - 1) / kTile;
  // One workgroup per CU fits (about 370 registers per lane): aim at one round of
  // at most 256 workgroups, splitting each query's items when there are few queries.
  long want = 256 / (rows * L.n_hg);
  if (want < 1) want = 1;
  int tps = (int)((tiles_max + want - 1) / want);      // tiles per split
  if (tps < 1) tps = 1;
  int nsplit = (tiles_max + tps - 1) / tps;
  if (nsplit > kMaxSplit) {
    tps = (tiles_max + kMaxSplit - 1) / kMaxSplit;
    nsplit = (tiles_max + tps - 1) / tps;
  }
  L.ips = tps * kTile;
  L.nsplit = nsplit < 1 ? 1 : nsplit;
  L.units = (int)(rows * L.nsplit);
  L.slots = (!A.dense && L.ips <= 16384) ? 1 : 0;
  return L;
}

static size_t mqa_lds_bytes(const MqaLaunch& L) {
  return (size_t)2 * kTile * kRowB + 2 * kTile * sizeof(float) + (L.slots ? (size_t)L.ips * sizeof(int32_t) : 0);
}

size_t mqa_workspace_bytes(const MqaArgs& A) {
  if (!A.bf16) return 0;
  MqaLaunch L = plan_mqa(A);
  if (L.nsplit == 1) return 0;
  const size_t parts = (size_t)A.batch * A.n_q * L.nsplit * A.heads;
  return parts * kD * sizeof(float) + parts * 2 * sizeof(float);
}

hipError_t launch_mqa(const MqaArgs& A, void* ws, size_t ws_bytes, hipStream_t s) {
  if (A.batch <= 0 || A.n_q <= 0) return hipSuccess;
  if (!A.bf16) {
    dim3 grid(A.heads, A.n_q, A.batch);
    mqa_f32_kernel<<<grid, kF32Waves * 64, 0, s>>>(A);
    return hipGetLastError();
  }
  MqaLaunch L = plan_mqa(A);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (L.nsplit > 1) {
    const size_t parts = (size_t)A.batch * A.n_q * L.nsplit * A.heads;
    if (ws_bytes < parts * (kD + 2) * sizeof(float) || !ws) return hipErrorInvalidValue;
    part_o = (float*)ws;
    part_ml = part_o + parts * kD;
  }
  const size_t lds = mqa_lds_bytes(L);
  static hipError_t attr = [] {
    hipError_t e = hipSuccess;
    const void* fns[3] = {(const void*)mqa_bf16_kernel<1>, (const void*)mqa_bf16_kernel<2>,
                          (const void*)mqa_bf16_kernel<4>};
    for (const void* fn : fns) {
      hipError_t r = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (r != hipSuccess) e = r;
    }
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const long groups = ((long)L.units + 7) / 8;
  dim3 grid((unsigned)(groups * 8 * L.n_hg));
  if (L.nw == 4) mqa_bf16_kernel<4><<<grid, 4 * 64, lds, s>>>(A, L, part_o, part_ml);
  else if (L.nw == 2) mqa_bf16_kernel<2><<<grid, 2 * 64, lds, s>>>(A, L, part_o, part_ml);
  else mqa_bf16_kernel<1><<<grid, 64, lds, s>>>(A, L, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.nsplit == 1) return e;
  dim3 cgrid(A.heads, (unsigned)((long)A.batch * A.n_q));
  mqa_combine_kernel<<<cgrid, kD / 4, 0, s>>>(A, L, part_o, part_ml);
  return hipGetLastError();
}

}  // namespace csa
