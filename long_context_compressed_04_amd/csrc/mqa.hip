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
// bf16 kernels (head_dim 512), chosen by the host:
//  - mqa_w8_kernel (unit RMSNorm weight): 8 waves = the 128 heads of a (query,
//    split) unit, two waves per SIMD; prefill, dense HCA decode;
//  - mqa_sd_kernel (few queries, unit weight): 16 waves = one group of 32 heads of a
//    (query, split) unit, split into logit, value and gather roles on a software
//    pipeline; sparse and dense decode;
//  - mqa_bf16_kernel (any RMSNorm weight): NW waves x 16 heads with an online
//    (running maximum) softmax.
// All stage 32-row item tiles in LDS (row-major, padded) and form S^T = K . u^T and
// O^T += V^T . P^T on MFMA.  RMSNorm is folded: q is normalised (times g^2) before
// the product, 1/rms of each row scales its logit and its softmax weight, and g
// multiplies the output.  Splits write partials (their own softmax average in fp16,
// maximum and sum in fp32) that a second kernel combines in fixed split order
// (deterministic).
//
// Options on every path: per-head sink logits in the softmax denominator (techniques
// map, "Learnable attention sink"), and the rope-conjugate rotation of the output's
// trailing 64 dims with the query's cos and sin ("Gated attention output", "Partial
// RoPE"), both applied where the output is finished.  The split-role kernel also reads
// FP8 E4M3 caches ("FP8 KV-cache quantization"), converting each row to bf16 on its way
// into LDS; with many queries the 8-wave kernel's pre-pass converts them into its
// normalised bf16 copy.
#include <cmath>
#include <type_traits>

#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "launch_timer.hpp"

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

// The end of a softmax: a head's weights were formed as 2^(l2_j - m2) (log2 units;
// m2 = 0 on the paths without a running maximum) and sum to l.  Returns the factor
// that turns the weighted sum of rows into the output, and the natural-log
// denominator.  A sink logit s joins the denominator only: with s2 = s log2(e) and
// M = max(m2, s2) the denominator is l 2^(m2 - M) + 2^(s2 - M) (in units of 2^M).
struct SoftmaxEnd {
  float mul, lse;
};
// 1 / x by the hardware reciprocal (v_rcp_f32, within 1 ulp) instead of the IEEE
// division's dozen instructions: the denominators here are softmax sums, normal
// floats, and the quotient is rounded to bf16 or fp16 afterwards.
__device__ __forceinline__ float rcp_f32(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ SoftmaxEnd softmax_end(float m2, float l, const float* sink, int head) {
  const bool none = !(l > 0.f);
  if (!sink) return {none ? 0.f : rcp_f32(l), none ? -INFINITY : m2 * kLn2 + logf(l)};
  const float s2 = sink[head] * kLog2e;
  const float M = none ? s2 : fmaxf(m2, s2);
  const float scale = none ? 0.f : exp2f(m2 - M);
  const float den = l * scale + exp2f(s2 - M);
  return {scale * rcp_f32(den), M * kLn2 + logf(den)};
}

// Rope-conjugate rotation of dim i (0..63) of a head's rotated slice (the trailing 64
// dims), from its value x and the value xp of its partner dim i ^ 1 (V4's rotary turns
// interleaved pairs): x cos_i - rotate_half(x)_i sin_i, with rotate_half(x)_i =
// -x_{i+1} (i even) or x_{i-1} (i odd).  cs = cos[64] then sin[64] of the query.
__device__ __forceinline__ float rope_conj(float x, float xp, int i, const float* cs) {
  return fmaf(x, cs[i], ((i & 1) ? -xp : xp) * cs[64 + i]);
}

// Split partials.  A split stores its own softmax average O_s / l_s (fp16, 4 dims per
// call; 0 for a split with nothing to attend) beside (m_s, l_s) in fp32; the merge
// weights split s by l_s 2^(m_s - M).  The average is a convex combination of
// RMS-normalised rows (|value| <= sqrt(512)), so fp16 holds it with a relative error
// of 2^-11, below the bf16 rounding of the output (2^-9).
__device__ __forceinline__ uint2 partial4(f32x4_t v, float il) {
  auto h = [](float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); };
  return make_uint2(h(v[0] * il) | (h(v[1] * il) << 16), h(v[2] * il) | (h(v[3] * il) << 16));
}
__device__ __forceinline__ f32x4_t partial4_value(uint2 u) {
  auto f = [](uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); };
  return f32x4_t{f(u.x & 0xffffu), f(u.x >> 16), f(u.y & 0xffffu), f(u.y >> 16)};
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
  const SoftmaxEnd fin = softmax_end(M * kLog2e, L, A.sink, h);   // (M is in natural-log units)
  float* orow = (float*)A.out + (row * A.heads + h) * D;
  auto val = [&](int d) {
    float o = 0.f;
    for (int w = 0; w < kF32Waves; ++w) o += so[w][d] * fw[w];
    return o * fin.mul * (A.gamma ? A.gamma[d] : 1.f);
  };
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const int i = d - (D - 64);   // position in the rotated slice
    if (A.rope && i >= 0)
      orow[d] = rope_conj(val(d), val(d ^ 1), i, A.rope + row * 128);
    else
      orow[d] = val(d);
  }
  if (A.lse && threadIdx.x == 0) A.lse[row * A.heads + h] = fin.lse;
}

// ---------------------------------------------------------------- bf16 (MFMA)
constexpr int kD = 512;
constexpr int kTile = 32;
constexpr int kRowB = kD * 2 + 16;      // LDS row stride in bytes (padded)

struct MqaLaunch {
  int nsplit, ips, n_hg, units, nw;   // nw: waves per workgroup
  int slots;                          // index slots of a split copied to LDS
  int kind;   // 0: 16-head waves, 3: 128-head 8-wave workgroups, 4: split-role 32-head
              // workgroups
  int pre;    // kind 3: row 1/rms from the per-cache pre-pass
};

// Masked items are loaded from this all-zero row, so that no lane ever reads
// outside the caller's buffers and masked rows hold no NaN/Inf.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kD * 2];

__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
}

// 1/sqrt(x) for a row's mean square (plus eps) in the per-tile paths: the hardware
// reciprocal square root (one instruction, ~1 ulp) instead of a rounded square root and
// a division (a dozen instructions on the step's critical path).
__device__ __forceinline__ float inv_rms(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ void load_row_to_lds(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// Row sums of squares for the RPW rows a wave staged: part[rr] holds this lane's
// share of row rr.  A row-splitting butterfly: each exchange step halves the rows a
// lane keeps; the lane then holds the total of row row_of_lane(lane).
__device__ __forceinline__ float rows_total8(const float (&p)[8], int lane) {
  // a permlane swap of two registers hands each half of the lanes the other half's copy
  // of the registers it keeps: lanes 0..31 keep rows 0..3, lanes 32..63 rows 4..7
  float a[4], c[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[j]), __float_as_uint(p[4 + j]), false, false);
    a[j] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {   // even 16-lane rows keep a[j], odd ones a[2 + j]
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[j]), __float_as_uint(a[2 + j]), false, false);
    c[j] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
  const bool up = (lane & 8) != 0;   // lanes 8..15 of a row keep c[1]; lane ^ 8 is 15 - lane's mirror pair
  // (mirror pairs lane i with 15 - i: the other 8-lane half, as lane ^ 8 would)
  float v = (up ? c[1] : c[0]) + dpp_f32<kDppMirror>(up ? c[0] : c[1]);
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  return v + dpp_f32<kDppHalfMirror>(v);
}

template <int RPW>
__device__ __forceinline__ void row_totals(const float (&part)[RPW], int lane, float* irms, int wave, int nw,
                                           uint32_t okmask, float eps) {
  if constexpr (RPW == 8) {
    const float s = rows_total8(part, lane);
    const int rr = 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
    if ((lane & 7) == 0) irms[wave + nw * rr] = ((okmask >> rr) & 1u) ? inv_rms(s * (1.f / 512) + eps) : 0.f;
  } else {
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const float s = wave_sum(part[rr]);
      if (lane == 0) irms[wave + nw * rr] = ((okmask >> rr) & 1u) ? inv_rms(s * (1.f / 512) + eps) : 0.f;
    }
  }
}

// Per-workgroup state of the bf16 MQA kernel that the tile loop needs.
struct TileCtx {
  uint8_t* tiles;      // [2][kTile][kRowB] LDS
  float* inv_rms;      // [2][kTile] LDS
  ItemSource src;
  int it0, it1, wave, lane, g, c16;
  float sl2, eps;
};

// The tile loop.  ONLINE = false: every head of the workgroup has a fixed softmax
// maximum (no rescaling, the accumulators are only touched by MFMAs); ONLINE = true:
// running maximum with rescaling for heads whose bound is too large.
template <int NW, bool ONLINE>
__device__ __forceinline__ void mqa_tiles(const TileCtx& C, const bf16x8_t (&qf)[16], bool fixed, float& m_run,
                                          float& l_run, f32x4_t (&o)[32]) {
  constexpr int RPW = kTile / NW;   // rows each wave loads per tile
  const int lane = C.lane, wave = C.wave, g = C.g, c16 = C.c16;
  uint32_t okmask = 0;              // validity of this wave's rows in the tile being loaded
  auto issue = [&](int tb, int buf) {
    uint32_t ok = 0;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = wave + NW * rr;
      const int item = tb + r;
      const uint8_t* p = (item < C.it1) ? C.src.row(item) : nullptr;
      ok |= (p != nullptr ? 1u : 0u) << rr;
      load_row_to_lds((p ? p : g_zero_row) + 16 * lane, C.tiles + buf * (kTile * kRowB) + r * kRowB);
    }
    okmask = ok;
  };
  if (C.it0 < C.it1) issue(C.it0, 0);
  int buf = 0;
  for (int tb = C.it0; tb < C.it1; tb += kTile, buf ^= 1) {
    uint8_t* const tile = C.tiles + buf * (kTile * kRowB);
    float* const irms = C.inv_rms + buf * kTile;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's rows of tile `buf` have landed
    {
      float part[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const uint4 v = *(const uint4*)(tile + (wave + NW * rr) * kRowB + 16 * lane);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xffff0000u);
          ss = fmaf(lo, lo, fmaf(hi, hi, ss));
        }
        part[rr] = ss;
      }
      row_totals<RPW>(part, lane, irms, wave, NW, okmask, C.eps);
    }
    __syncthreads();
    if (tb + kTile < C.it1) issue(tb + kTile, buf ^ 1);

    // ---- S^T = K . u^T for items [0,16) and [16,32)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* ka = tile + c16 * kRowB + 16 * g;
      constexpr int PF = 3;   // A fragments in flight ahead of the MFMAs
      uint4 a0[PF], a1[PF];
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        a0[j] = *(const uint4*)(ka + 64 * j);
        a1[j] = *(const uint4*)(ka + 16 * kRowB + 64 * j);
      }
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 c0 = a0[ks % PF], c1 = a1[ks % PF];
        if (ks + PF < 16) {
          a0[ks % PF] = *(const uint4*)(ka + 64 * (ks + PF));
          a1[ks % PF] = *(const uint4*)(ka + 16 * kRowB + 64 * (ks + PF));
        }
        s0 = mfma16x16x32(as_bf16x8(c0), qf[ks], s0);
        s1 = mfma16x16x32(as_bf16x8(c1), qf[ks], s1);
      }
    }
    // ---- softmax weights for this lane's head over its 8 items (16*bb + 4*g + r)
    float lg[8], ir[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ir[r] = irms[4 * g + r];
      ir[4 + r] = irms[16 + 4 * g + r];
      lg[r] = (ir[r] > 0.f) ? s0[r] * C.sl2 * ir[r] : -INFINITY;
      lg[4 + r] = (ir[4 + r] > 0.f) ? s1[r] * C.sl2 * ir[4 + r] : -INFINITY;
    }
    float pw[8], psum = 0.f;
    if constexpr (ONLINE) {
      float tmax = lg[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, lg[r]);
      tmax = max_xor32(max_xor16(tmax));
      const float m_new = fixed ? m_run : fmaxf(m_run, tmax);
      const bool none = m_new == -INFINITY;   // nothing valid yet for this head
      const float corr = none ? 1.f : exp2f(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float p = none ? 0.f : exp2f(lg[r] - m_new);
        psum += p;
        pw[r] = p * ir[r];
      }
      l_run = l_run * corr + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 32; ++db) o[db] = o[db] * corr;
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float p = __builtin_amdgcn_exp2f(lg[r] - m_run);   // masked: exp2(-inf) = 0
        psum += p;
        pw[r] = p * ir[r];                        // weight on the raw row (1/rms folded)
      }
      l_run += psum;
    }
    const bf16x8_t pb = as_bf16x8(make_uint4(pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                             pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7])));
    // ---- O^T += V^T . P^T  (V^T fragments by transposing LDS reads of the same tile)
    const uint8_t* base1 = tile + (4 * g + (c16 >> 2)) * kRowB + 8 * (c16 & 3);
    const uint8_t* base2 = base1 + 16 * kRowB;
    {
      constexpr int PF = 4;   // V^T fragments in flight ahead of the MFMAs
      i16x4_t v0[PF], v1[PF];
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        v0[j] = lds_read_tr16(base1 + 32 * j);
        v1[j] = lds_read_tr16(base2 + 32 * j);
      }
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const i16x4_t c0 = v0[db % PF], c1 = v1[db % PF];
        if (db + PF < 32) {
          v0[db % PF] = lds_read_tr16(base1 + 32 * (db + PF));
          v1[db % PF] = lds_read_tr16(base2 + 32 * (db + PF));
        }
        typedef short i16x8_t __attribute__((ext_vector_type(8)));
        const i16x8_t vv = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        o[db] = mfma16x16x32(__builtin_bit_cast(bf16x8_t, vv), pb, o[db]);
      }
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void mqa_bf16_kernel(MqaArgs A, MqaLaunch L, uint16_t* part_o, float* part_ml) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* const gam = (float*)(lds + 2 * kTile * kRowB + 2 * kTile * sizeof(float));   // [kD]
  int32_t* const slot_idx = (int32_t*)(gam + kD);                                   // [L.ips] (sparse)

  TileCtx C;
  C.tiles = lds;
  C.inv_rms = (float*)(lds + 2 * kTile * kRowB);
  C.lane = threadIdx.x & 63;
  C.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  C.g = C.lane >> 4;
  C.c16 = C.lane & 15;
  const int g = C.g;

  // ---- XCD-aware unit mapping: every head group of a unit runs on the same XCD
  const int f = blockIdx.x;
  const int xcd = f & 7, r8 = f >> 3;
  const int hg = r8 % L.n_hg, ug = r8 / L.n_hg;
  const int unit = ug * 8 + xcd;
  if (unit >= L.units) return;
  // (32-bit quotients: a 64-bit division is a hundred scalar instructions on the way to
  // the first loads; units and rows are int counts)
  const int row32 = unit / L.nsplit;
  const long row = row32;
  const int split = unit - row32 * L.nsplit;
  const int b = row32 / A.n_q;
  const int head = hg * (NW * 16) + C.wave * 16 + C.c16;   // this lane's head (column)

  int total;
  query_items(A, b, row, 2, C.src, total);
  C.it0 = split * L.ips;
  C.it1 = min(total, C.it0 + L.ips);
  if (C.src.idx && L.slots) {  // index slots of this split, copied once
    for (int i = threadIdx.x; i < L.ips; i += NW * 64) {
      const int it = C.it0 + i;
      slot_idx[i] = (it < min(C.it1, C.src.n_first)) ? C.src.idx[it] : -1;
    }
    C.src.idx = slot_idx;
    C.src.idx_off = C.it0;
  }
  for (int i = threadIdx.x; i < kD; i += NW * 64) gam[i] = A.gamma ? A.gamma[i] : 1.f;
  __syncthreads();

  // ---- u = q * g^2 / rms(q) as bf16 B operands (dims 32*ks + 8*g + [0, 8)); the
  // softmax bound M = scale * sqrt(d) * |u| >= |logit| for every row (each row's
  // 1/rms makes |k| * inv_rms <= sqrt(d)).
  bf16x8_t qf[16];
  float m_fix;
  {
    const uint16_t* qrow = (const uint16_t*)A.q + (row * A.heads + head) * kD;
    uint4 raw[16];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      raw[ks] = *(const uint4*)(qrow + 32 * ks + 8 * g);
      const uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xffff0000u);
        ss = fmaf(lo, lo, fmaf(hi, hi, ss));
      }
    }
    ss = add_xor32(add_xor16(ss));
    const float qinv = 1.f / sqrtf(ss * (1.f / kD) + A.eps);
    float uu = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
      uint32_t o4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = 32 * ks + 8 * g + 2 * k;
        const float g0 = gam[d0], g1 = gam[d0 + 1];
        o4[k] = pack_bf16x2(__uint_as_float(w4[k] << 16) * qinv * g0 * g0,
                            __uint_as_float(w4[k] & 0xffff0000u) * qinv * g1 * g1);
        const float r0 = __uint_as_float(o4[k] << 16), r1 = __uint_as_float(o4[k] & 0xffff0000u);
        uu = fmaf(r0, r0, fmaf(r1, r1, uu));
      }
      qf[ks] = as_bf16x8(make_uint4(o4[0], o4[1], o4[2], o4[3]));
    }
    uu = add_xor32(add_xor16(uu));
    m_fix = A.scale * kLog2e * sqrtf((float)kD * uu) * 1.0001f + 1e-6f;   // log2 units
  }
  // A fixed maximum needs no rescaling: exp2(l - M) >= 2^(-2M) stays a normal
  // float when M <= 60.  Larger bounds (large g or scale) use the running maximum.
  const bool fixed = m_fix <= 60.f;
  const bool block_fixed = __syncthreads_and(fixed ? 1 : 0) != 0;
  C.sl2 = A.scale * kLog2e;
  C.eps = A.eps;
  float m_run = fixed ? m_fix : -INFINITY, l_run = 0.f;
  f32x4_t o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (block_fixed) mqa_tiles<NW, false>(C, qf, fixed, m_run, l_run, o);
  else mqa_tiles<NW, true>(C, qf, fixed, m_run, l_run, o);

  // ---- finish: total sum per head across the 4 lane groups
  l_run = add_xor32(add_xor16(l_run));
  if (L.nsplit == 1) {
    const SoftmaxEnd fin = softmax_end(m_run, l_run, A.sink, head);
    const float inv_l = fin.mul;
    uint16_t* orow = (uint16_t*)A.out + (row * A.heads + head) * kD;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const int d0 = 16 * db + 4 * g;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[db][r] * inv_l * gam[d0 + r];
      if (db >= 28 && A.rope) {   // dims 448 ..: the partner of dim d0 + r is d0 + (r ^ 1), in this lane
        const float x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = rope_conj(x[r], x[r ^ 1], d0 + r - (kD - 64), A.rope + row * 128);
      }
      *(uint2*)(orow + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    if (A.lse && g == 0) A.lse[row * A.heads + head] = fin.lse;
  } else {
    uint16_t* po = part_o + (((long)row * L.nsplit + split) * A.heads + head) * kD;
    const float il = l_run > 0.f ? rcp_f32(l_run) : 0.f;
#pragma unroll
    for (int db = 0; db < 32; ++db) *(uint2*)(po + 16 * db + 4 * g) = partial4(o[db], il);
    if (g == 0) {
      float* pm = part_ml + (((long)row * L.nsplit + split) * A.heads + head) * 2;
      pm[0] = l_run > 0.f ? m_run : -INFINITY;
      pm[1] = l_run;
    }
  }
}

// ------------------------------------------------ bf16, 32 heads per wave (MFMA 32x32x16)
// Per wave and 32-row tile, with the heads as the N side of v_mfma_f32_32x32x16_bf16:
//   S^T[32 rows x 32 heads] = K . u^T        (A = K rows from LDS, B = normalised q)
//   O^T[dims x 32 heads]   += V^T . P^T      (A = V^T by ds_read_b64_tr_b16 from the
//                                             same row-major tile, B = P^T straight
//                                             from the S^T registers)
// Softmax without a running maximum: with unit RMSNorm weight every logit obeys
// |l| <= scale * d (|u|, |k_hat| <= sqrt(d)), so for scale * d * log2(e) <= 100
// exp2(l * log2 e) stays a normal float with no overflow (host-checked); weights are
// exp2 of the logit itself, sums need no rescaling and splits merge by addition.
//
// Gathered rows land in LDS by direct-to-LDS loads, two tiles ahead.  The three tile
// buffers are separate static LDS objects and each tile loop is unrolled by three, so
// the compiler can see that reads of one buffer never alias the loads still landing
// in another (one shared array would force a wait for every load before any LDS
// read); the barriers are plain s_barrier with explicit LDS waits for the same reason.
constexpr int kRowB2 = kD * 2 + 48;   // LDS row stride: conflict-free b128 and tr16 reads
constexpr int kNB = 3;                // LDS tile buffers
constexpr int kXS = 16;             // logits per lane exchanged between waves
constexpr int kStageRow = 128 + 4;  // fp32 words per head row of the output staging (padded)
constexpr int kSlotsLds = 2048;     // index slots of a split held in LDS

// Barrier without a memory fence: waits only for this wave's LDS operations, so
// direct-to-LDS loads of later tiles stay in flight across it (a workgroup fence
// would wait for them).  The signal fences keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum of squares of 8 bf16 values added to acc (exact fp32 widening, full-rate FMAs).
__device__ __forceinline__ float sumsq_bf16x8(uint4 v, float acc) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xffff0000u);
    acc = fmaf(lo, lo, fmaf(hi, hi, acc));
  }
  return acc;
}

// Gathers RPW rows (items item0 + STRIDE * rr) of one wave into LDS rows
// dst + STRIDE * rr * kRowB2, 16 bytes per lane.  Lane rr resolves row rr (all
// lookups at once); the loop reads the addresses back as scalars.  A masked row is
// loaded from the zero row.  Returns the mask of rows that exist.
template <int RPW, int STRIDE, class Resolve>
__device__ __forceinline__ uint32_t issue_rows(Resolve resolve, int item0, int lane, uint8_t* dst) {
  const uint8_t* pl = resolve(item0 + STRIDE * (lane % RPW));
  const uint64_t pv = (uint64_t)(pl ? pl : g_zero_row);
  const uint32_t lo = (uint32_t)pv, hi = (uint32_t)(pv >> 32);
  const uint32_t ok = (uint32_t)__ballot(pl != nullptr) & ((1u << RPW) - 1u);
  // a rolled loop: few distinct direct-to-LDS instructions for the compiler to track
#pragma unroll 1
  for (int rr = 0; rr < RPW; ++rr) {
    const uint64_t p = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, rr) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)lo, rr);
    load_row_to_lds((const uint8_t*)p + 16 * lane, dst + STRIDE * rr * kRowB2);
  }
  return ok;
}

// acc + (both bf16 halves of w) squared, by the bf16 dot-product instruction
__device__ __forceinline__ float dot2_bf16(uint32_t w, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

struct RowSrc {
  const uint8_t* kv;
  const uint8_t* raw;
  const int32_t* gidx;   // global index slots (sparse, when not copied to LDS)
  int it0, it1, n_first, kv_rows, win_lo, raw_base, raw_cap, use_slots, dense;
};

// ---------------------------------------------------------------------------------
// Split-role decode kernel: one workgroup = one group of 32 heads of a (query,
// split) unit, sixteen waves in three roles on a software pipeline over 32-row tiles
// (step s: tile s weighed while tile s-1 is accumulated and tile s+2 is gathered):
//  - logit waves 0..3: wave w takes rows 16 (w >> 1) .. + 15 of tile s against heads
//    16 (w & 1) .. + 15 over all 512 dims, S on v_mfma_f32_16x16x32_bf16 (A =
//    normalised q held in registers, B = K rows), so that a lane's four logits all
//    belong to one row; the rows' sums of squares come from the same K fragments by
//    bf16 dot products (four independent sums, reduced across the lanes of the row by
//    permlane swaps), then the softmax weights go into LDS: no partial logits cross
//    waves and no per-row value crosses lanes of different rows;
//  - value waves 4..7: O^T for dims 128 (w - 4) .. of tile s-1 on
//    v_mfma_f32_32x32x16_bf16 (A = V^T by transposing LDS reads, B = the weights of
//    the previous step);
//  - gather waves 8..15: the rows of tile s+2, four each, by direct-to-LDS loads.
//    A wave issues a row only every hundred-odd cycles, so the gather rate of a CU
//    grows with the number of waves issuing; these waves read no tile buffer, so
//    waiting for all but their last four loads needs no help from the compiler.
// One barrier per step; four tile buffers: two tiles in flight, one being weighed,
// one being accumulated.  The weights are stored row-major (tile row, head), and the
// value waves read them with the same transposing reads as the rows, so both
// operands of the 32x32x16 product take their k index in the same order.
constexpr int kSdQk = 4, kSdPv = 4, kSdGa = 8;
constexpr int kSdWaves = kSdQk + kSdPv + kSdGa;
constexpr int kSdRpw = kTile / kSdGa;   // rows each gather wave loads per tile
constexpr int kWRow = 2 * 32 + 8;       // bytes per tile row of a weight buffer (32 heads, padded)

// 16 FP8 E4M3 values -> bf16, stored as 32 bytes (exact: E4M3 has 3 mantissa bits and
// a narrower exponent range than bf16).  gfx950's scaled conversion turns two codes
// into a bf16 pair in one instruction (a scale of 1 leaves the values as they are).
__device__ __forceinline__ void fp8x16_to_bf16(uint4 v, uint8_t* dst) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.f, false));   // bytes 0, 1
    o[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.f, true));   // 2, 3
  }
  *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
  *(uint4*)(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
}

// F8: the cache (kv and the window rows) holds FP8 E4M3 rows of 512 bytes.  The gather
// waves load them into registers instead, 1 KB (two rows) per instruction and wave,
// three tiles ahead (tile s+3 requested at step s), and at step s write tile s+1 to
// its tile buffer as bf16; the logit and value waves are the same as without F8.
template <bool F8>
__global__ __launch_bounds__(kSdWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mqa_sd_kernel(MqaArgs A, MqaLaunch L, uint16_t* part_o, float* part_ml) {
  constexpr int kRowG = F8 ? kD : 2 * kD;   // bytes per cache row
  __shared__ __attribute__((aligned(16))) uint8_t tb0[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t tb2[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t tb3[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t wts[2][kTile * kWRow];
  __shared__ int32_t slot[kSlotsLds];
  __shared__ __attribute__((aligned(16))) float lsum[2][32];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f = blockIdx.x;
  const int xcd = f & 7, r8 = f >> 3;
  const int hg = r8 % L.n_hg, ug = r8 / L.n_hg;
  const int unit = ug * 8 + xcd;
  if (unit >= L.units) return;
  // (32-bit quotients: a 64-bit division is a hundred scalar instructions on the way to
  // the first loads; units and rows are int counts)
  const int row32 = unit / L.nsplit;
  const long row = row32;
  const int split = unit - row32 * L.nsplit;
  const int b = row32 / A.n_q;

  // raw q rows of the heads this wave normalises (heads wave + 16 j), 16 bytes a lane;
  // loaded before the slots, so waiting for the slots has waited for them too
  constexpr int kQn = 32 / kSdWaves;
  uint4 qraw[kQn];
#pragma unroll
  for (int j = 0; j < kQn; ++j)
    qraw[j] = *(const uint4*)((const uint16_t*)A.q + (row * A.heads + hg * 32 + wave + kSdWaves * j) * kD + 8 * lane);
  // ---- the items of this (query, split): index slots to LDS
  RowSrc R;
  {
    ItemSource src;
    int total;
    query_items(A, b, row, F8 ? 1 : 2, src, total);   // bytes per element of the cache
    R.kv = src.kv; R.raw = src.raw; R.n_first = src.n_first; R.kv_rows = src.kv_rows; R.win_lo = src.win_lo;
    R.raw_base = src.raw_base; R.raw_cap = src.raw_cap; R.dense = A.dense;
    R.it0 = split * L.ips;
    R.it1 = min(total, R.it0 + L.ips);
    R.gidx = src.idx;
    R.use_slots = !A.dense;
    if (R.use_slots)
      for (int i = threadIdx.x; i < L.ips; i += kSdWaves * 64) {
        const int it = R.it0 + i;
        slot[i] = (it < min(R.it1, R.n_first)) ? src.idx[it] : -1;
      }
  }
  wait_vmcnt<0>();   // q has arrived: nothing later waits for it behind the gathers
  lds_barrier();     // the slots are in LDS

  auto resolve = [&](int item) -> const uint8_t* {
    if (item >= R.it1) return nullptr;
    if (item < R.n_first) {
      const int e = R.dense ? item : slot[item - R.it0];
      return (e >= 0 && e < R.kv_rows) ? R.kv + (long)e * kRowG : nullptr;
    }
    const int r = R.win_lo + (item - R.n_first) - R.raw_base;
    return (r >= 0 && r < R.raw_cap) ? R.raw + (long)r * kRowG : nullptr;
  };
  const int n_tiles = (R.it1 - R.it0 + kTile - 1) / kTile;
  const int gw = wave - kSdQk - kSdPv;   // gather-wave index (>= 0 for gather waves)
  auto issue = [&](int t, uint8_t* dst) {
    issue_rows<kSdRpw, kSdGa>(resolve, R.it0 + t * kTile + gw, lane, dst + gw * kRowB2);
  };
  // F8: gather wave gw takes rows 2 gw, 2 gw + 1 (registers r[0]) and 16 + 2 gw,
  // 17 + 2 gw (r[1]) of a tile, lanes 32 .. 63 the second row of each pair.  Tiles past
  // the last are read from the zero row, so every step makes the same requests.
  auto load8 = [&](int t, uint4 (&r)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* p = resolve(R.it0 + t * kTile + 2 * gw + 16 * j + (lane >> 5));
      r[j] = *(const uint4*)((p ? p : g_zero_row) + 16 * (lane & 31));
    }
  };
  auto store8 = [&](const uint4 (&r)[2], uint8_t* tile) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fp8x16_to_bf16(r[j], tile + (2 * gw + 16 * j + (lane >> 5)) * kRowB2 + 32 * (lane & 31));
  };
  // ---- u = q / rms(q), staged in tile buffer 3 (free until tile 3 is gathered)
  auto stage_q = [&]() {
#pragma unroll
    for (int j = 0; j < kQn; ++j) {
      const int hq = wave + kSdWaves * j;
      const uint4 v = qraw[j];
      const float ss = wave_sum(sumsq_bf16x8(v, 0.f));
      const float qinv = inv_rms(ss * (1.f / kD) + A.eps);   // (u is rounded to bf16 next)
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      uint32_t o4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o4[k] = pack_bf16x2(__uint_as_float(w4[k] << 16) * qinv, __uint_as_float(w4[k] & 0xffff0000u) * qinv);
      *(uint4*)(tb3 + hq * kRowB2 + 16 * lane) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
  };
  if constexpr (F8) {
    if (gw >= 0) {
      // ============================================================ FP8 gather waves
      // (their whole path, so that the registers in flight never meet another
      // role's code)
      uint4 rf8[3][2];   // tiles in flight, tile t in rf8[t % 3]
      load8(0, rf8[0]);
      load8(1, rf8[1]);
      load8(2, rf8[2]);
      stage_q();
      store8(rf8[0], tb0);
      lds_barrier();   // q staged, tile 0 in its buffer
      // step s: request tile s+3, write tile s+1 to buffer (s+1) % 4 (tile s-3 was
      // accumulated at step s-2)
      auto gstep = [&](auto KC, int s) {
        constexpr int K = decltype(KC)::value;   // s % 3
        load8(s + 3, rf8[K]);
        const int bi = (s + 1) & 3;
        store8(rf8[(K + 1) % 3], bi == 0 ? tb0 : (bi == 1 ? tb1 : (bi == 2 ? tb2 : tb3)));
        lds_barrier();
      };
      // steps 0 .. n_tiles: whole groups of three in the loop (the registers in flight are
      // the same at every entry), the remainder after it.  (A loop left from inside a
      // group made the compiler wait for every load in flight at the loop head.)
      int s = 0;
      for (; s + 2 <= n_tiles; s += 3) {
        gstep(std::integral_constant<int, 0>{}, s);
        gstep(std::integral_constant<int, 1>{}, s + 1);
        gstep(std::integral_constant<int, 2>{}, s + 2);
      }
      if (s <= n_tiles) gstep(std::integral_constant<int, 0>{}, s);
      if (s + 1 <= n_tiles) gstep(std::integral_constant<int, 1>{}, s + 1);
      lds_barrier();   // the head sums are in LDS
      return;
    }
  } else if (gw >= 0) {
    if (n_tiles > 0) issue(0, tb0);
    if (n_tiles > 1) issue(1, tb1);
  }
  stage_q();
  if (!F8 && gw >= 0) {
    if (n_tiles > 1) wait_vmcnt<kSdRpw>();
    else wait_vmcnt<0>();
  }
  lds_barrier();   // q staged, tile 0 landed

  const float sl2 = A.scale * kLog2e;
  const float eps = A.eps;
  if (wave < kSdQk) {
    // ================================================================ logit waves
    const int hb = wave & 1, rb = wave >> 1;
    const int g = lane >> 4, c16 = lane & 15;
    bf16x8_t qf[16];   // A fragments: head 16 hb + c16, dims 32 ks + 8 g ..
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qf[ks] = as_bf16x8(*(const uint4*)(tb3 + (16 * hb + c16) * kRowB2 + 64 * ks + 16 * g));
    float lh[4] = {0.f, 0.f, 0.f, 0.f};   // heads 16 hb + 4 g + r, over this lane's rows
    auto step = [&](auto BUFC, int s) {
      constexpr int BUF = decltype(BUFC)::value;
      if (s < n_tiles) {
        const uint8_t* tile = BUF == 0 ? tb0 : (BUF == 1 ? tb1 : (BUF == 2 ? tb2 : tb3));
        const uint8_t* ka = tile + (16 * rb + c16) * kRowB2 + 16 * g;
        // row 16 rb + c16 of the tile: masked or not (its slot is read before the product)
        const bool ok = resolve(R.it0 + s * kTile + 16 * rb + c16) != nullptr;
        f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        float ss4[4] = {0.f, 0.f, 0.f, 0.f};
        constexpr int PF = 4;
        uint4 a[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) a[j] = *(const uint4*)(ka + 64 * j);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const uint4 c = a[ks % PF];
          if (ks + PF < 16) a[ks % PF] = *(const uint4*)(ka + 64 * (ks + PF));
          sacc[ks & 1] = mfma16x16x32(qf[ks], as_bf16x8(c), sacc[ks & 1]);
          ss4[0] = dot2_bf16(c.x, ss4[0]);
          ss4[1] = dot2_bf16(c.y, ss4[1]);
          ss4[2] = dot2_bf16(c.z, ss4[2]);
          ss4[3] = dot2_bf16(c.w, ss4[3]);
        }
        // sv[r]: head 16 hb + 4 g + r against row 16 rb + c16
        const f32x4_t sv = sacc[0] + sacc[1];
        const float ss = add_xor32(add_xor16((ss4[0] + ss4[1]) + (ss4[2] + ss4[3])));   // row c16's sum of squares
        const float irow = ok ? inv_rms(ss * (1.f / kD) + eps) : 0.f;
        const float li = sl2 * irow;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(sv[r] * li);
          const float w = ok ? e : 0.f;
          lh[r] += w;
          p[r] = w * irow;
        }
        *(uint2*)(wts[s & 1] + (16 * rb + c16) * kWRow + 2 * (16 * hb + 4 * g)) =
            make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      }
      lds_barrier();
    };
    for (int s = 0; s <= n_tiles; s += 4) {
      step(std::integral_constant<int, 0>{}, s);
      if (s + 1 <= n_tiles) step(std::integral_constant<int, 1>{}, s + 1);
      if (s + 2 <= n_tiles) step(std::integral_constant<int, 2>{}, s + 2);
      if (s + 3 <= n_tiles) step(std::integral_constant<int, 3>{}, s + 3);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) lh[r] = row_sum16f(lh[r]);   // over the wave's 16 rows
    if (c16 == 0) *(f32x4_t*)&lsum[rb][16 * hb + 4 * g] = f32x4_t{lh[0], lh[1], lh[2], lh[3]};
    lds_barrier();   // the head sums are in LDS
    if (wave == 0 && lane < 32) {
      const float l = lsum[0][lane] + lsum[1][lane];
      const int head = hg * 32 + lane;
      if (L.nsplit == 1) {
        if (A.lse) A.lse[row * A.heads + head] = softmax_end(0.f, l, A.sink, head).lse;
      } else {
        float* pm = part_ml + (((long)row * L.nsplit + split) * A.heads + head) * 2;
        pm[0] = l > 0.f ? 0.f : -INFINITY;
        pm[1] = l;
      }
    }
    return;
  }
  if (gw >= 0) {
    // ================================================================= gather waves
    for (int s = 0; s <= n_tiles; ++s) {
      const int t = s + 2;
      if (t < n_tiles) {
        const int bi = t & 3;
        issue(t, bi == 0 ? tb0 : (bi == 1 ? tb1 : (bi == 2 ? tb2 : tb3)));
        wait_vmcnt<kSdRpw>();   // tile s+1 has landed; tile s+2 may still be in flight
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
    }
    lds_barrier();   // the head sums are in LDS
    return;
  }
  // ================================================================== value waves
  const int pw = wave - kSdQk;
  const int h = lane >> 5, c32 = lane & 31;
  const int G = lane >> 4, sl = lane & 15;
  const int vb_off = (4 * h + (sl >> 2)) * kRowB2 + 256 * pw + (16 * (G & 1) + 4 * (sl & 3)) * 2;
  const int pb_off = (4 * h + (sl >> 2)) * kWRow + (16 * (G & 1) + 4 * (sl & 3)) * 2;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};
  auto step = [&](auto BUFC, int s) {
    constexpr int BV = (decltype(BUFC)::value + 3) % 4;   // tile s-1's buffer
    const uint8_t* const tv = BV == 0 ? tb0 : (BV == 1 ? tb1 : (BV == 2 ? tb2 : tb3));
    if (s >= 1) {
      // P^T fragments by the same transposing reads as V^T: k = rows 4 h .. and 8 + 4 h ..
      // of each 16-row step, n = head c32
      const uint8_t* P = wts[(s - 1) & 1] + pb_off;
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      i16x4_t pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[j] = lds_read_tr16(P + 8 * j * kWRow);
      const bf16x8_t pb0 = __builtin_bit_cast(bf16x8_t, i16x8_t{pr[0][0], pr[0][1], pr[0][2], pr[0][3],
                                                                 pr[1][0], pr[1][1], pr[1][2], pr[1][3]});
      const bf16x8_t pb1 = __builtin_bit_cast(bf16x8_t, i16x8_t{pr[2][0], pr[2][1], pr[2][2], pr[2][3],
                                                                 pr[3][0], pr[3][1], pr[3][2], pr[3][3]});
      const uint8_t* vb = tv + vb_off;
      i16x4_t v0[8], v1[8];
      auto vaddr = [&](int k) { return vb + (16 * (k & 1)) * kRowB2 + 64 * (k >> 1); };   // k = 2 db + step
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v0[k] = lds_read_tr16(vaddr(k));
        v1[k] = lds_read_tr16(vaddr(k) + 8 * kRowB2);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        typedef short i16x8_t __attribute__((ext_vector_type(8)));
        const i16x8_t vv = {v0[k][0], v0[k][1], v0[k][2], v0[k][3], v1[k][0], v1[k][1], v1[k][2], v1[k][3]};
        o[k >> 1] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, vv), (k & 1) ? pb1 : pb0, o[k >> 1]);
      }
    }
    lds_barrier();
  };
  for (int s = 0; s <= n_tiles; s += 4) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 <= n_tiles) step(std::integral_constant<int, 1>{}, s + 1);
    if (s + 2 <= n_tiles) step(std::integral_constant<int, 2>{}, s + 2);
    if (s + 3 <= n_tiles) step(std::integral_constant<int, 3>{}, s + 3);
  }
  lds_barrier();   // the head sums are in LDS
  // o[db][r] holds dim 128 pw + 32 db + 8 (r/4) + 4 h + r%4 of head c32.  The
  // 32 x 128 block goes through LDS (every tile buffer is free after the last step)
  // so that each store instruction writes two whole head rows.
  float* stage = (float*)(pw == 0 ? tb0 : (pw == 1 ? tb1 : (pw == 2 ? tb2 : tb3)));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4_t*)(stage + c32 * kStageRow + 32 * db + 8 * j + 4 * h) =
          f32x4_t{o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
  __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes are done (wave-private region)
  const int hl = lane >> 5, d4 = lane & 31;
  const bool rot = A.rope && pw == 3 && d4 >= 16;   // this lane's dims are in the rotated slice
  if (L.nsplit == 1) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int hh = 2 * k + hl;
      const float il = softmax_end(0.f, lsum[0][hh] + lsum[1][hh], A.sink, hg * 32 + hh).mul;
      f32x4_t v = *(const f32x4_t*)(stage + hh * kStageRow + 4 * d4);
      if (rot) {   // dims 448 ..: the partner of dim d is d ^ 1, in the same four
        const f32x4_t x = v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = rope_conj(x[r], x[r ^ 1], 4 * (d4 - 16) + r, A.rope + row * 128);
      }
      uint16_t* orow = (uint16_t*)A.out + (row * A.heads + hg * 32 + hh) * kD + 128 * pw + 4 * d4;
      *(uint2*)orow = make_uint2(pack_bf16x2(v[0] * il, v[1] * il), pack_bf16x2(v[2] * il, v[3] * il));
    }
  } else {
    uint16_t* po = part_o + (((long)row * L.nsplit + split) * A.heads + hg * 32) * kD + 128 * pw + 4 * d4;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int hh = 2 * k + hl;
      const float l = lsum[0][hh] + lsum[1][hh];
      *(uint2*)(po + (long)hh * kD) = partial4(*(const f32x4_t*)(stage + hh * kStageRow + 4 * d4), l > 0.f ? rcp_f32(l) : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------------
// Row 1/rms pre-pass for many queries (prefill): a compressed entry is normalised
// once, not once per query that selects it.

// One wave per row: every row of kv (all kv_cap rows of every sequence) and kv_raw,
// RMS-normalised (unit weight) and rounded to bf16, into kvn [batch, kv_cap, 512] and
// rawn [batch, raw_cap, 512]: the keys and values the attention itself reads.  F8: the
// rows are FP8 E4M3 codes (512 bytes), taken at their exact values.
template <bool F8>
__global__ __launch_bounds__(256) void row_normalize_kernel(MqaArgs A, uint16_t* kvn, uint16_t* rawn) {
  constexpr int kRowG = F8 ? kD : 2 * kD;   // bytes per cache row
  const long gw = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long n_kv = (long)A.batch * A.kv_cap, n_raw = (long)A.batch * A.raw_cap;
  if (gw >= n_kv + n_raw) return;
  const uint8_t* rowp = gw < n_kv ? (const uint8_t*)A.kv + gw * kRowG : (const uint8_t*)A.kv_raw + (gw - n_kv) * kRowG;
  uint16_t* dst = gw < n_kv ? kvn + gw * kD : rawn + (gw - n_kv) * kD;
  uint32_t w4[4];   // this lane's 8 values (dims 8 lane ..) as bf16 pairs
  if (F8) {
    const uint2 c = *(const uint2*)(rowp + 8 * lane);
    w4[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, false));
    w4[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, true));
    w4[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, false));
    w4[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, true));
  } else {
    const uint4 v = *(const uint4*)(rowp + 16 * lane);
    w4[0] = v.x; w4[1] = v.y; w4[2] = v.z; w4[3] = v.w;
  }
  const float ss = wave_sum(sumsq_bf16x8(make_uint4(w4[0], w4[1], w4[2], w4[3]), 0.f));
  const float r = 1.f / sqrtf(ss * (1.f / kD) + A.eps);
  uint32_t o4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o4[k] = pack_bf16x2(__uint_as_float(w4[k] << 16) * r, __uint_as_float(w4[k] & 0xffff0000u) * r);
  *(uint4*)(dst + 8 * lane) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
}

// ---------------------------------------------------------------------------------
// Eight-wave kernel: a workgroup = one (query, split) unit x 128 heads, two waves per
// SIMD so that one wave's MFMAs run while the other waits on LDS (on MI355X a wave
// alone on its SIMD keeps an LDS-fed MFMA stream roughly half busy; two reach about
// four fifths).  Per 32-row tile:
//   QK: wave w = (head block hb = w & 3, dim half dh = w >> 2) forms the partial
//       S^T[32 rows x 32 heads] over its 256 dims.  The pair (hb, 0), (hb, 1) swaps
//       halves through LDS and each finishes 16 rows: their softmax weights, packed
//       to bf16, are exactly the B operand of k-step dh of the P V product.
//   PV: wave w = (head pair hp = w & 1, dim quarter dq = w >> 1) accumulates
//       O^T[128 dims x 64 heads]; each V^T fragment (ds_read_b64_tr_b16, the slow
//       LDS read) feeds two MFMAs.
// Row RMSNorm: PRE (many queries) reads a normalised bf16 copy of the cache made by a
// pre-pass (each row normalised once; the tile's per-row factor is then 1, or 0 for a
// masked row); otherwise each wave sums the squares of the 4 rows it loaded (few
// queries: a pre-pass would read the whole cache for a few hundred rows).
constexpr int kW8Waves = 8;
constexpr int kW8Rpw = kTile / kW8Waves;   // rows each wave gathers per tile
constexpr int kW8Stage = 64 + 4;           // fp32 words per head row of the output staging

// Row sums of squares of the 4 rows a wave loaded (part[rr]: this lane's share of
// row rr): a row-splitting butterfly; the lane ends with the total of row
// 2 * bit5(lane) + bit4(lane).
__device__ __forceinline__ float rows_total4(const float (&p)[4], int lane) {
  float a[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {   // lanes 0..31 keep rows 0, 1; lanes 32..63 rows 2, 3
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[j]), __float_as_uint(p[2 + j]), false, false);
    a[j] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
  // even 16-lane rows keep a[0], odd ones a[1]
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[0]), __float_as_uint(a[1]), false, false);
  return row_sum16f(__uint_as_float(t[0]) + __uint_as_float(t[1]));
}

template <bool PRE>
__global__ __launch_bounds__(kW8Waves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mqa_w8_kernel(MqaArgs A, MqaLaunch L, uint16_t* part_o, float* part_ml, const uint16_t* kvn,
                   const uint16_t* rawn) {
  __shared__ __attribute__((aligned(16))) uint8_t tb0[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) uint8_t tb2[kTile * kRowB2];
  __shared__ __attribute__((aligned(16))) float irms[kNB][kTile];
  __shared__ __attribute__((aligned(16))) f32x4_t xs[kW8Waves][2][64];   // partial S^T halves
  __shared__ __attribute__((aligned(16))) uint4 pbuf[4][2][64];          // P^T B operands
  __shared__ float red[kW8Waves][64];                                    // q norms, then l
  __shared__ int32_t slot[kSlotsLds];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, c32 = lane & 31;
  const int hb = wave & 3, dh = wave >> 2;   // QK role
  const int hp = wave & 1, dq = wave >> 1;   // PV role

  // The units of one XCD are consecutive, so neighbouring queries (which share their
  // window rows and many selected entries) meet in one L2.
  const int total_units = L.units * L.n_hg;
  const int upx = (total_units + 7) / 8;
  const int unit = (blockIdx.x & 7) * upx + (blockIdx.x >> 3);
  if (unit >= total_units) return;
  const int hg = unit % L.n_hg;
  const int rs = unit / L.n_hg;   // (32-bit quotients, as in the split-role kernel)
  const int row32 = rs / L.nsplit;
  const long row = row32;
  const int split = rs - row32 * L.nsplit;
  const int b = row32 / A.n_q;

  RowSrc R;
  {
    ItemSource src;
    int total;
    query_items(A, b, row, 2, src, total);
    R.kv = src.kv; R.raw = src.raw; R.n_first = src.n_first; R.kv_rows = src.kv_rows; R.win_lo = src.win_lo;
    R.raw_base = src.raw_base; R.raw_cap = src.raw_cap; R.dense = A.dense;
    R.it0 = split * L.ips;
    R.it1 = min(total, R.it0 + L.ips);
    R.gidx = src.idx;
    R.use_slots = !A.dense;
    if (R.use_slots)
      for (int i = threadIdx.x; i < L.ips; i += kW8Waves * 64) {
        const int it = R.it0 + i;
        slot[i] = (it < min(R.it1, R.n_first)) ? src.idx[it] : -1;
      }
  }
  if (PRE) {   // rows from the normalised copy (same layout as kv and kv_raw)
    R.kv = (const uint8_t*)(kvn + (long)b * A.kv_cap * kD);
    R.raw = (const uint8_t*)(rawn + (long)b * A.raw_cap * kD);
  }
  // this lane's query head (QK role) and its dims 256 dh + 16 ks + 8 h + [0, 8)
  const uint16_t* qrow = (const uint16_t*)A.q + (row * A.heads + hg * 128 + 32 * hb + c32) * kD + 256 * dh + 8 * h;
  uint4 qraw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qraw[ks] = *(const uint4*)(qrow + 16 * ks);
  lds_barrier();   // the slots are in LDS

  const int n_tiles = (R.it1 - R.it0 + kTile - 1) / kTile;
  // Gathering a tile takes the index slots of its rows, read from LDS one step ahead
  // (slots_of, at the start of a step, where the read's latency hides behind the
  // products), then turns them into row addresses without branches (resolve).
  struct Slots {
    int row;   // slot of this lane's row wave + 8 (lane % 4)
  };
  auto slot_at = [&](int item) -> int {   // (an in-bounds read; ignored where no slot applies)
    return R.use_slots ? slot[min(max(item - R.it0, 0), kSlotsLds - 1)] : 0;
  };
  auto slots_of = [&](int ti) -> Slots {
    const int item0 = R.it0 + ti * kTile;
    Slots sv;
    sv.row = slot_at(item0 + wave + kW8Waves * (lane & (kW8Rpw - 1)));
    return sv;
  };
  // tile row item (its slot sv) -> source row (nullptr: masked)
  auto resolve = [&](int item, int sv) -> const uint8_t* {
    const bool first = item < R.n_first;
    const int e = first ? (R.dense ? item : sv) : R.win_lo + (item - R.n_first) - R.raw_base;
    const bool ok = item < R.it1 && e >= 0 && e < (first ? R.kv_rows : R.raw_cap);
    return ok ? (first ? R.kv : R.raw) + (long)e * (kD * 2) : nullptr;
  };
  // Gathering tile ti: lane rr of every wave resolves the wave's row wave + 8 rr (a
  // masked row reads the zero row).
  struct Gather {
    uint32_t lo, hi;   // row address of lane rr
    uint32_t ok;       // rows that exist
  };
  auto resolve_tile = [&](int ti, const Slots& sv) -> Gather {
    Gather g;
    const int item0 = R.it0 + ti * kTile;
    const uint8_t* pl = resolve(item0 + wave + kW8Waves * (lane & (kW8Rpw - 1)), sv.row);
    g.ok = (uint32_t)__ballot(pl != nullptr) & ((1u << kW8Rpw) - 1u);
    const uint64_t pv = (uint64_t)(pl ? pl : g_zero_row);
    g.lo = (uint32_t)pv;
    g.hi = (uint32_t)(pv >> 32);
    return g;
  };
  // PRE: the tile's per-row factors (1 for a row that exists, 0 for a masked one), the
  // wave's four rows from lanes 0..3
  auto row_mask = [&](uint32_t ok, float* irms_dst) {
    if (PRE && lane < kW8Rpw) irms_dst[wave + kW8Waves * lane] = ((ok >> lane) & 1u) ? 1.f : 0.f;
  };
  auto load_row = [&](const Gather& g, int rr, uint8_t* dst) {
    const uint64_t p = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)g.hi, rr) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)g.lo, rr);
    load_row_to_lds((const uint8_t*)p + 16 * lane, dst + (wave + kW8Waves * rr) * kRowB2);
  };
  auto issue = [&](int ti, const Slots& sv, uint8_t* dst, float* irms_dst) -> uint32_t {
    const Gather g = resolve_tile(ti, sv);
    row_mask(g.ok, irms_dst);
#pragma unroll 1
    for (int rr = 0; rr < kW8Rpw; ++rr) load_row(g, rr, dst);
    return g.ok;
  };
  auto buf_ptr = [&](int bi) -> uint8_t* { return bi == 0 ? tb0 : (bi == 1 ? tb1 : tb2); };
  uint32_t okm[kNB] = {0, 0, 0};
  if (n_tiles > 0) okm[0] = issue(0, slots_of(0), tb0, irms[0]);
  if (n_tiles > 1) okm[1] = issue(1, slots_of(1), tb1, irms[1]);

  // ---- u = q / rms(q): the pair (hb, 0), (hb, 1) holds the two dim halves of a head
  bf16x8_t qf[16];
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) ss = sumsq_bf16x8(qraw[ks], ss);
    ss = add_xor32(ss);
    red[wave][lane] = ss;
    lds_barrier();
    const float qinv = 1.f / sqrtf((ss + red[wave ^ 4][lane]) * (1.f / kD) + A.eps);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t w4[4] = {qraw[ks].x, qraw[ks].y, qraw[ks].z, qraw[ks].w};
      uint32_t o4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o4[k] = pack_bf16x2(__uint_as_float(w4[k] << 16) * qinv, __uint_as_float(w4[k] & 0xffff0000u) * qinv);
      qf[ks] = as_bf16x8(make_uint4(o4[0], o4[1], o4[2], o4[3]));
    }
  }
  const float sl2 = A.scale * kLog2e;
  float l_run = 0.f;
  f32x16_t o[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[j][db] = f32x16_t{};

  const int G = lane >> 4, sl = lane & 15;
  const int ka_base = c32 * kRowB2 + 16 * h;   // K: row c32, dims 256 dh + 16 ks + 8 h
  const int vb_base = (4 * h + (sl >> 2)) * kRowB2 + (16 * (G & 1) + 4 * (sl & 3)) * 2 + 256 * dq;
  // V^T fragment f = 2 db + t: dims 128 dq + 32 db + [0, 32), rows of k-step t
  auto vb_off = [](int f) { return (16 * (f & 1)) * kRowB2 + 64 * (f >> 1); };

  // DH: this wave's dim half as a compile-time constant (register indices must be static)
  auto step = [&](auto BUFC, auto DHC, int ti) {
    constexpr int BUF = decltype(BUFC)::value;
    constexpr int DH = decltype(DHC)::value;
    uint8_t* const tile = BUF == 0 ? tb0 : (BUF == 1 ? tb1 : tb2);
    // the slots of tile ti + 2, for its gather after the first barrier
    const Slots sv2 = slots_of(ti + 2);
    // tile ti is in LDS (waited before the previous barrier)
    if (!PRE) {
      // 1/rms of the 4 rows this wave loaded (read before the barrier: they are its own)
      float part[kW8Rpw];
#pragma unroll
      for (int rr = 0; rr < kW8Rpw; ++rr) {   // one row at a time: few live registers
        part[rr] = sumsq_bf16x8(*(const uint4*)(tile + (wave + kW8Waves * rr) * kRowB2 + 16 * lane), 0.f);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float s = rows_total4(part, lane);
      const int rr = 2 * ((lane >> 5) & 1) + ((lane >> 4) & 1);
      if ((lane & 15) == 0)
        irms[BUF][wave + kW8Waves * rr] = ((okm[BUF] >> rr) & 1u) ? inv_rms(s * (1.f / kD) + A.eps) : 0.f;
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- partial S^T over this wave's 256 dims: 16 k-steps.  Behind the first product,
    // tile ti + 2's row addresses are resolved (wave-uniform: scalar registers until the
    // P V phase issues the loads) and, with PRE, its row mask written: that work needs
    // only the slots read above, and its irms slot (tile ti - 1's) was last read before
    // the previous step's second barrier, so the scalar and vector units do it while
    // the matrix unit runs instead of after the exchange barrier.
    const bool gi = ti + 2 < n_tiles;
    uint64_t growp[kW8Rpw] = {};
    f32x16_t s = f32x16_t{};
    {
      const uint8_t* ka = tile + ka_base + 512 * DH;
      constexpr int PF = 2;
      uint4 a[PF];
#pragma unroll
      for (int j = 0; j < PF; ++j) a[j] = *(const uint4*)(ka + 32 * j);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 c = a[ks % PF];
        if (ks + PF < 16) a[ks % PF] = *(const uint4*)(ka + 32 * (ks + PF));
        s = mfma32x32x16(as_bf16x8(c), qf[ks], s);
        if (ks == 0 && gi) {
          const Gather gn = resolve_tile(ti + 2, sv2);
          row_mask(gn.ok, irms[(BUF + 2) % kNB]);
          okm[(BUF + 2) % kNB] = gn.ok;
#pragma unroll
          for (int rr = 0; rr < kW8Rpw; ++rr)
            growp[rr] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)gn.hi, rr) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)gn.lo, rr);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- the partner finishes the rows of k-step 1 - dh: hand it those 8 partials
    {
      constexpr int g = 8 * (1 - DH);
      xs[wave][0][lane] = f32x4_t{s[g], s[g + 1], s[g + 2], s[g + 3]};
      xs[wave][1][lane] = f32x4_t{s[g + 4], s[g + 5], s[g + 6], s[g + 7]};
    }
    lds_barrier();
    // rows of k-step dh: s[8 dh + k] is row 16 dh + 8 (k / 4) + 4 h + k % 4
    {
      const f32x4_t x0 = xs[wave ^ 4][0][lane], x1 = xs[wave ^ 4][1][lane];
      const f32x4_t ir0 = *(const f32x4_t*)&irms[BUF][16 * DH + 4 * h];
      const f32x4_t ir1 = *(const f32x4_t*)&irms[BUF][16 * DH + 8 + 4 * h];
      float sf[8], ir[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sf[k] = s[8 * DH + k] + x0[k];
        sf[4 + k] = s[8 * DH + 4 + k] + x1[k];
        ir[k] = ir0[k];
        ir[4 + k] = ir1[k];
      }
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        float p2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float e = __builtin_amdgcn_exp2f(sf[k + u] * sl2 * ir[k + u]);
          const float p = ir[k + u] > 0.f ? e : 0.f;
          psum += p;
          p2[u] = p * ir[k + u];
        }
        pk[k / 2] = pack_bf16x2(p2[0], p2[1]);
      }
      l_run += psum;
      pbuf[hb][DH][lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    // this wave's loads of tile ti + 1 (the only ones in flight) are done; after the
    // barrier every wave's are, and every wave's P of tile ti is in LDS
    wait_vmcnt<0>();
    lds_barrier();
    // ---- O^T[128 dq .. + 128 dims x 64 heads] += V^T . P^T, with the gather of tile
    // ti + 2 into the buffer of tile ti - 1 (every wave is past it since the first
    // barrier): one row after every second pair of products, so that a load that waits for room in the memory pipeline
    // holds up this wave while the products already issued, and the other wave of the
    // SIMD, keep the matrix unit busy
    {
      uint8_t* const gdst = buf_ptr((BUF + 2) % kNB);
      const bf16x8_t p00 = as_bf16x8(pbuf[2 * hp][0][lane]), p01 = as_bf16x8(pbuf[2 * hp][1][lane]);
      const bf16x8_t p10 = as_bf16x8(pbuf[2 * hp + 1][0][lane]), p11 = as_bf16x8(pbuf[2 * hp + 1][1][lane]);
      const uint8_t* vb = tile + vb_base;
      constexpr int PV = 2;
      i16x4_t v0[PV], v1[PV];
#pragma unroll
      for (int j = 0; j < PV; ++j) {
        v0[j] = lds_read_tr16(vb + vb_off(j));
        v1[j] = lds_read_tr16(vb + vb_off(j) + 8 * kRowB2);
      }
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const i16x4_t c0 = v0[f % PV], c1 = v1[f % PV];
        if (f + PV < 8) {
          v0[f % PV] = lds_read_tr16(vb + vb_off(f + PV));
          v1[f % PV] = lds_read_tr16(vb + vb_off(f + PV) + 8 * kRowB2);
        }
        typedef short i16x8_t __attribute__((ext_vector_type(8)));
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, i16x8_t{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]});
        o[0][f >> 1] = mfma32x32x16(va, (f & 1) ? p01 : p00, o[0][f >> 1]);
        o[1][f >> 1] = mfma32x32x16(va, (f & 1) ? p11 : p10, o[1][f >> 1]);
        if (gi && (f & 1))
          load_row_to_lds((const uint8_t*)growp[f >> 1] + 16 * lane, gdst + (wave + kW8Waves * (f >> 1)) * kRowB2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  static_assert(kW8Rpw == 4, "one gathered row per two of the eight P V k-steps");
  // tile 0 in LDS (tile 1's kW8Rpw row loads, the last this wave issued, may be in flight)
  if (n_tiles > 1) wait_vmcnt<kW8Rpw>();
  else wait_vmcnt<0>();
  lds_barrier();
  auto run = [&](auto DHC) {
    for (int ti = 0; ti < n_tiles; ti += kNB) {
      step(std::integral_constant<int, 0>{}, DHC, ti);
      if (ti + 1 < n_tiles) step(std::integral_constant<int, 1>{}, DHC, ti + 1);
      if (ti + 2 < n_tiles) step(std::integral_constant<int, 2>{}, DHC, ti + 2);
    }
  };
  if (dh) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  // ---- softmax denominators: head 32 hb + c32 summed over the two lane halves here,
  // then over the pair (hb, 0), (hb, 1) through LDS
  l_run = add_xor32(l_run);
  lds_barrier();   // every wave is past its last tile: the tile buffers and red are free
  red[wave][lane] = l_run;
  lds_barrier();
  float inv_l[2], l_tot[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hbj = 2 * hp + j;
    l_tot[j] = red[hbj][c32] + red[hbj + 4][c32];
    inv_l[j] = L.nsplit == 1 ? softmax_end(0.f, l_tot[j], A.sink, hg * 128 + 64 * hp + 32 * j + c32).mul
                             : (l_tot[j] > 0.f ? rcp_f32(l_tot[j]) : 0.f);   // a split's own average
  }
  // ---- O^T -> rows of 64 dims through a wave-private LDS region, four chunks
  // (head block j of the pair, dim half of the quarter)
  float* stage = (float*)(buf_ptr(wave / 3) + (wave % 3) * (32 * kW8Stage * 4));
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int dbl = 0; dbl < 2; ++dbl)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16_t& od = o[j][2 * half + dbl];
          *(f32x4_t*)(stage + c32 * kW8Stage + 32 * dbl + 8 * q + 4 * h) =
              f32x4_t{od[4 * q], od[4 * q + 1], od[4 * q + 2], od[4 * q + 3]};
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int dim0 = 128 * dq + 64 * half + 4 * (lane & 15);
      const int head0 = hg * 128 + 64 * hp + 32 * j;
      const bool rot = A.rope && dq == 3 && half == 1;
      if (L.nsplit == 1) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int hh = 4 * k + (lane >> 4);
          const float il = __shfl(inv_l[j], hh, 64);
          f32x4_t v = *(const f32x4_t*)(stage + hh * kW8Stage + 4 * (lane & 15));
          if (rot) {   // the chunk is the rotated slice; the partner of dim d is d ^ 1, in the same four
            const f32x4_t x = v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = rope_conj(x[r], x[r ^ 1], 4 * (lane & 15) + r, A.rope + row * 128);
          }
          uint16_t* orow = (uint16_t*)A.out + (row * A.heads + head0 + hh) * kD + dim0;
          *(uint2*)orow = make_uint2(pack_bf16x2(v[0] * il, v[1] * il), pack_bf16x2(v[2] * il, v[3] * il));
        }
      } else {
        uint16_t* po = part_o + (((long)row * L.nsplit + split) * A.heads + head0) * kD + dim0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int hh = 4 * k + (lane >> 4);
          const float il = __shfl(inv_l[j], hh, 64);
          *(uint2*)(po + (long)hh * kD) = partial4(*(const f32x4_t*)(stage + hh * kW8Stage + 4 * (lane & 15)), il);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next chunk overwrites
    }
  if (dq == 0 && h == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int head = hg * 128 + 64 * hp + 32 * j + c32;
      if (L.nsplit == 1) {
        if (A.lse) A.lse[row * A.heads + head] = softmax_end(0.f, l_tot[j], A.sink, head).lse;
      } else {
        float* pm = part_ml + (((long)row * L.nsplit + split) * A.heads + head) * 2;
        pm[0] = l_tot[j] > 0.f ? 0.f : -INFINITY;
        pm[1] = l_tot[j];
      }
    }
  }
}

// Fixed-order merge of split partials (each the split's average A_s = O_s / l_s):
// out = sum_s A_s l_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
constexpr int kMaxSplit = 128;

__global__ __launch_bounds__(128) void mqa_combine_kernel(MqaArgs A, MqaLaunch L, const uint16_t* part_o,
                                                          const float* part_ml) {
  constexpr int kPre = 16;   // splits whose partials are requested before the weights exist
  const int head = blockIdx.x;
  const long row = blockIdx.y;
  const int S = L.nsplit;
  const int d0 = threadIdx.x * 4;
  const uint16_t* po = part_o + ((row * S) * A.heads + head) * kD + d0;
  const long sstride = (long)A.heads * kD;
  // the first splits' partials are in flight while the weights are formed (kept as
  // loaded: converting them here would wait for each load in turn)
  uint2 pre[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) pre[s] = *(const uint2*)(po + min(s, S - 1) * sstride);   // (no branch)
  // (m_s, l_s) are the same for every thread of the workgroup: each thread forms the
  // weights w_s = l_s 2^(m_s - M) and their sum itself, from uniform loads, with no
  // cross-lane step or barrier on the way to the first multiply
  const float* pm = part_ml + ((row * S) * A.heads + head) * 2;
  const long mstride = (long)A.heads * 2;
  float2 ml[kPre];   // requested together (no branch), so their latencies overlap
#pragma unroll
  for (int s = 0; s < kPre; ++s) ml[s] = *(const float2*)(pm + min(s, S - 1) * mstride);
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kPre; ++s) M = fmaxf(M, ml[s].x);   // (repeats of the last split change nothing)
  for (int s = kPre; s < S; ++s) M = fmaxf(M, pm[s * mstride]);
  auto weight = [&](float m, float l) { return m == -INFINITY ? 0.f : l * exp2f(m - M); };
  float Lsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < S) {
      const float w = weight(ml[s].x, ml[s].y);
      Lsum += w;
      acc += partial4_value(pre[s]) * w;
    }
  for (int s = kPre; s < S; ++s) {
    const float w = weight(pm[s * mstride], pm[s * mstride + 1]);
    Lsum += w;
    acc += partial4_value(*(const uint2*)(po + s * sstride)) * w;
  }
  const SoftmaxEnd fin = softmax_end(M, Lsum, A.sink, head);
  const float inv_l = fin.mul;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = acc[r] * inv_l * (A.gamma ? A.gamma[d0 + r] : 1.f);
  if (A.rope && d0 >= kD - 64) {   // dims 448 ..: the partner of dim d0 + r is d0 + (r ^ 1)
    const float x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = rope_conj(x[r], x[r ^ 1], d0 + r - (kD - 64), A.rope + row * 128);
  }
  uint16_t* orow = (uint16_t*)A.out + (row * A.heads + head) * kD;
  *(uint2*)(orow + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  if (A.lse && threadIdx.x == 0) A.lse[row * A.heads + head] = fin.lse;
}

static MqaLaunch plan_mqa(const MqaArgs& A) {
  MqaLaunch L;
  L.pre = 0;
  const long rows = (long)A.batch * A.n_q;
  const int total_max = (A.dense ? A.n_max : A.topk) + A.window;
  const int tiles_max = (total_max + kTile - 1) / kTile;
  // The 32- and 128-head MFMA paths need the unit RMSNorm weight and a scale that
  // keeps every exp2(logit) normal without a running maximum.
  const bool fixed = A.gamma == nullptr && A.scale * kLog2e * kD * 1.01f <= 100.f;
  if (A.split_items > 0) {
    // Batch-invariant: the kernel and the split boundaries (multiples of split_items
    // from a query's first item) follow from the configuration alone, never from the
    // batch, and the merge runs in split order; a query's arithmetic is then the
    // same in any batch.
    if (A.kv_f8 || (fixed && A.heads % 32 == 0)) {   // (an FP8 cache implies both)
      L.kind = 4;
      L.n_hg = A.heads / 32;
      L.nw = kSdWaves;
    } else {
      L.kind = 0;
      L.nw = (A.heads % 64 == 0) ? 4 : ((A.heads % 32 == 0) ? 2 : 1);
      L.n_hg = A.heads / (L.nw * 16);
    }
    L.ips = A.split_items;
    L.nsplit = (total_max + L.ips - 1) / L.ips;
    if (L.nsplit < 1) L.nsplit = 1;
    L.units = (int)(rows * L.nsplit);
    L.slots = (!A.dense && L.ips <= 8192) ? 1 : 0;
    return L;
  }
  L.kind = 0;
  if (fixed) {
    // Kernel and split count from a cost model fitted to MI355X timings (microseconds):
    // rounds of <= 256 workgroups (one per CU), each a fixed start-up cost plus its
    // 32-row tiles; with splits, the fp16 partials are written and read back once
    // (about 4 MB per microsecond each way) and the merge is one more launch.
    double best = 1e30;
    for (int variant = 0; variant < 3; ++variant) {
      // 0: split-role 32-head workgroups (32 query rows at most); 1, 2: 8-wave
      // 128-head workgroups with row norms from the gathered tiles / from the pre-pass
      const bool hg = variant == 0;
      const bool pre = variant == 2;
      // (an FP8 cache is read by the split-role kernel, and by the 8-wave kernel through
      // the pre-pass's normalised bf16 copy)
      if (hg && (A.heads % 32 != 0 || (rows > 32 && !A.kv_f8))) continue;
      if (!hg && (A.heads % 128 != 0 || (A.kv_f8 && !pre))) continue;
      const int wg_heads = hg ? 32 : 128;
      const int n_hg = A.heads / wg_heads;
      // (the 8-wave kernel gathers only ~1.5 tiles ahead: on rows scattered over HBM,
      // as in sparse decode, it waits on memory)
      // (the split-role kernel is bound by the gather rate when every CU gathers:
      // about 0.9 us a tile; its start-up waits on the index slots, then on the
      // first two tiles, and its partial leaves at the end)
      const double t_tile = hg ? 0.9 : (pre ? 2.4 : (A.dense ? 3.0 : 5.0));
      // the pre-pass reads every cached row once and writes its normalised copy (~5 TB/s)
      const double t_norms = pre ? 3.0 + (A.kv_f8 ? 1.5 : 2.0) * (double)A.batch * ((double)A.kv_cap + A.raw_cap) *
                                             (kD * 2) / 5.0e6
                                 : 0.0;
      for (int sp = 1; sp <= kMaxSplit && sp <= tiles_max; ++sp) {
        const int tps = (tiles_max + sp - 1) / sp;
        const int s_eff = (tiles_max + tps - 1) / tps;
        if (!A.dense && tps * kTile > kSlotsLds) continue;   // index slots must fit in LDS
        const double wgs = (double)rows * n_hg * s_eff;
        const double rounds = std::ceil(wgs / 256.0);
        const double part_mb = s_eff > 1 ? wgs * wg_heads * kD * 2.0 / 1.0e6 : 0.0;
        // start-up: first gathers, and the workgroup's partial (128 KB for 128 heads)
        // leaving through one CU
        const double t_start = hg ? 13.0 : (s_eff > 1 ? 13.0 : 4.0);
        const double cost = t_norms + rounds * (t_start + tps * t_tile) + (s_eff > 1 ? 4.0 + part_mb / 2.0 : 0.0);
        if (cost < best - 1e-9) {
          best = cost;
          L.kind = hg ? 4 : 3;
          L.pre = pre ? 1 : 0;
          L.n_hg = n_hg;
          L.nw = hg ? kSdWaves : kW8Waves;
          L.ips = tps * kTile;
          L.nsplit = s_eff;
        }
      }
    }
  }
  if (L.kind == 0) {
    L.nw = (A.heads % 64 == 0) ? 4 : ((A.heads % 32 == 0) ? 2 : 1);
    L.n_hg = A.heads / (L.nw * 16);
    // One workgroup per CU fits (about 380 registers per lane): aim at one round of
    // at most 256 workgroups, splitting each query's items when there are few queries.
    long want = 256 / (rows * L.n_hg);
    if (want < 1) want = 1;
    int tps = (int)((tiles_max + want - 1) / want);
    if (tps < 1) tps = 1;
    int nsplit = (tiles_max + tps - 1) / tps;
    if (nsplit > kMaxSplit) {
      tps = (tiles_max + kMaxSplit - 1) / kMaxSplit;
      nsplit = (tiles_max + tps - 1) / tps;
    }
    L.ips = tps * kTile;
    L.nsplit = nsplit;
  }
  if (L.nsplit < 1) L.nsplit = 1;
  L.units = (int)(rows * L.nsplit);
  L.slots = (!A.dense && L.ips <= 8192) ? 1 : 0;
  return L;
}

// Dynamic LDS ceiling: 160 KiB per CU less room for the kernel's static LDS.
constexpr int kMaxDynLds = 152 * 1024;

static size_t mqa_lds_bytes(const MqaLaunch& L) {
  const size_t slots = L.slots ? (size_t)L.ips * sizeof(int32_t) : 0;
  if (L.kind != 0) return 0;   // static LDS only
  return (size_t)2 * kTile * kRowB + 2 * kTile * sizeof(float) + kD * sizeof(float) + slots;
}

static size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t partial_bytes(const MqaArgs& A, const MqaLaunch& L) {
  if (L.nsplit == 1) return 0;
  const size_t parts = (size_t)A.batch * A.n_q * L.nsplit * A.heads;
  return r256(parts * kD * sizeof(uint16_t) + parts * 2 * sizeof(float));   // fp16 averages, fp32 (m, l)
}

// The normalised copy of the full-dim kernel's rows: [batch, kv_cap, 512] then
// [batch, raw_cap, 512] bf16.
static size_t norm_bytes(const MqaArgs& A, const MqaLaunch& L) {
  if (!(L.kind == 3 && L.pre)) return 0;
  return r256((size_t)A.batch * A.kv_cap * kD * 2) + r256((size_t)A.batch * A.raw_cap * kD * 2);
}

// The plan depends on whether a norm weight is given, which the size query does not
// know: size for both.
size_t mqa_workspace_bytes(const MqaArgs& A) {
  if (!A.bf16) return 0;
  MqaArgs B = A;
  B.gamma = nullptr;
  const MqaLaunch La = plan_mqa(B);
  const size_t a = partial_bytes(B, La) + norm_bytes(B, La);
  static const float one = 1.f;
  B.gamma = &one;
  const MqaLaunch Lb = plan_mqa(B);
  const size_t b = partial_bytes(B, Lb) + norm_bytes(B, Lb);
  return a > b ? a : b;
}

hipError_t launch_mqa(const MqaArgs& A, void* ws, size_t ws_bytes, hipStream_t s) {
  if (A.batch <= 0 || A.n_q <= 0) return hipSuccess;
  if (!A.bf16) {
    dim3 grid(A.heads, A.n_q, A.batch);
    return launch("mqa_f32", mqa_f32_kernel, grid, dim3(kF32Waves * 64), 0, s, A);
  }
  MqaLaunch L = plan_mqa(A);
  uint16_t* part_o = nullptr;
  float* part_ml = nullptr;
  const size_t pb = partial_bytes(A, L), nb = norm_bytes(A, L);
  if (pb + nb > 0 && (ws_bytes < pb + nb || !ws)) return hipErrorInvalidValue;
  if (L.nsplit > 1) {
    const size_t parts = (size_t)A.batch * A.n_q * L.nsplit * A.heads;
    part_o = (uint16_t*)ws;
    part_ml = (float*)(part_o + parts * kD);
  }
  uint16_t* kvn = nullptr;
  uint16_t* rawn = nullptr;
  if (nb > 0) {
    kvn = (uint16_t*)((char*)ws + pb);
    rawn = (uint16_t*)((char*)ws + pb + r256((size_t)A.batch * A.kv_cap * kD * 2));
    const long n_rows = (long)A.batch * ((long)A.kv_cap + A.raw_cap);
    hipError_t e = A.kv_f8 ? launch("mqa_row_norms", row_normalize_kernel<true>, dim3((unsigned)((n_rows + 3) / 4)),
                                    dim3(256), 0, s, A, kvn, rawn)
                           : launch("mqa_row_norms", row_normalize_kernel<false>, dim3((unsigned)((n_rows + 3) / 4)),
                                    dim3(256), 0, s, A, kvn, rawn);
    if (e != hipSuccess) return e;
  }
  const size_t lds = mqa_lds_bytes(L);
  static hipError_t attr = [] {
    hipError_t e = hipSuccess;
    const void* fns[3] = {(const void*)mqa_bf16_kernel<1>, (const void*)mqa_bf16_kernel<2>,
                          (const void*)mqa_bf16_kernel<4>};
    for (const void* fn : fns) {
      hipError_t r = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
      if (r != hipSuccess) e = r;
    }
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (lds > (size_t)kMaxDynLds) return hipErrorInvalidValue;
  // FP8 rows are read by the split-role kernel, or normalised into bf16 by the pre-pass
  if (A.kv_f8 && !(L.kind == 4 || (L.kind == 3 && L.pre))) return hipErrorInvalidValue;
  const long groups = ((long)L.units + 7) / 8;
  dim3 grid((unsigned)(groups * 8 * L.n_hg));
  if (L.kind == 3) grid = dim3((unsigned)((((long)L.units * L.n_hg + 7) / 8) * 8));
  hipError_t e;
  if (L.kind == 3 && L.pre)
    e = launch("mqa_bf16_w8", mqa_w8_kernel<true>, grid, dim3(kW8Waves * 64), lds, s, A, L, part_o, part_ml,
               (const uint16_t*)kvn, (const uint16_t*)rawn);
  else if (L.kind == 3)
    e = launch("mqa_bf16_w8", mqa_w8_kernel<false>, grid, dim3(kW8Waves * 64), lds, s, A, L, part_o, part_ml,
               (const uint16_t*)nullptr, (const uint16_t*)nullptr);
  else if (L.kind == 4 && A.kv_f8)
    e = launch("mqa_f8_sd", mqa_sd_kernel<true>, grid, dim3(kSdWaves * 64), lds, s, A, L, part_o, part_ml);
  else if (L.kind == 4)
    e = launch("mqa_bf16_sd", mqa_sd_kernel<false>, grid, dim3(kSdWaves * 64), lds, s, A, L, part_o, part_ml);
  else if (L.nw == 4)
    e = launch("mqa_bf16_h16", mqa_bf16_kernel<4>, grid, dim3(4 * 64), lds, s, A, L, part_o, part_ml);
  else if (L.nw == 2)
    e = launch("mqa_bf16_h16", mqa_bf16_kernel<2>, grid, dim3(2 * 64), lds, s, A, L, part_o, part_ml);
  else
    e = launch("mqa_bf16_h16", mqa_bf16_kernel<1>, grid, dim3(64), lds, s, A, L, part_o, part_ml);
  if (e != hipSuccess || L.nsplit == 1) return e;
  dim3 cgrid(A.heads, (unsigned)((long)A.batch * A.n_q));
  return launch("mqa_combine", mqa_combine_kernel, cgrid, dim3(kD / 4), 0, s, A, L, (const uint16_t*)part_o,
                (const float*)part_ml);
}

}  // namespace csa
