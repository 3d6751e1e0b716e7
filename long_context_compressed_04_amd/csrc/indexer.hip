// Lightning-indexer scores.
//
// "DeepSeek v4" summary page, section "Compressed Sparse Attention", lightning
// indexer: several indexer query heads per query token; the score of each
// preceding compressed block s is the sum over heads of a per-head weight times
// ReLU(q_h . K_s).  Techniques map "DeepSeek-V4-Pro", "Indexer-selected sparse
// attention": 64 indexer heads x 128 dims, entries at or past the causal threshold
// are invalid.  FP4 activations on this QK path: forum post on the DeepSeek V4
// paper; techniques map, "FP4 precision for the attention indexer".
//
// Kernels
//  * index_scores_f32: VALU, one thread per entry (fp32 workloads, any shape).
//  * index_scores_mfma<HB, FP4>: heads on the MFMA M axis (HB blocks of 32 heads),
//    entries on N (32 per tile).  Each wave keeps TPW key tiles in registers
//    (B operands loaded straight from HBM, 16 B per lane), then loops over the
//    workgroup's queries with q staged through LDS, so keys are read once per
//    query tile.  bf16 uses v_mfma_f32_32x32x16_bf16; MXFP4 uses the block-scaled
//    v_mfma_scale_f32_32x32x64_f8f6f4 (e2m1 operands, e8m0 scale per 32 k-values).
//    Epilogue: ReLU, per-head weight, reduction over the 32 rows of each block
//    (16 in-lane, then the partner lane l^32), one fp32 score per entry.
#include <type_traits>

#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "launch_timer.hpp"

namespace csa {

// ------------------------------------------------------------------ fp32 (VALU)
constexpr int kIdxF32Threads = 256;

__global__ __launch_bounds__(kIdxF32Threads) void index_scores_f32(IndexArgs A, float* scores) {
  extern __shared__ float smem[];
  const int b = blockIdx.z, qi = blockIdx.y;
  const int H = A.heads, D = A.dim;
  float* qs = smem;            // [H * D]
  float* ws = smem + H * D;    // [H]
  const long row = (long)b * A.n_q + qi;
  const float* q = (const float*)A.q + row * H * D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qs[i] = q[i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) ws[i] = A.w[row * H + i];
  __syncthreads();
  const int ne = min(A.n_entries[b], A.n_max);
  const int V = visible_entries(A.q_pos[row], ne, A.m);
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= A.n_max) return;
  float total = -INFINITY;
  if (s < V) {
    const float* k = (const float*)A.k + ((long)b * A.k_cap + s) * D;
    total = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      for (int i = 0; i < D; ++i) dot = fmaf(qs[h * D + i], k[i], dot);
      total = fmaf(ws[h], fmaxf(dot, 0.f), total);
    }
  }
  scores[row * A.n_max + s] = total;
}

// ------------------------------------------------------------ MFMA (bf16 / MXFP4)
constexpr int kIdxWaves = 4;
constexpr int kIdxDim = 128;                 // indexer head dim on the MFMA paths
constexpr int kQRowBf16 = kIdxDim * 2 + 16;  // LDS row stride (bytes), padded
constexpr int kQRowFp4 = kIdxDim / 2 + 16;

template <int HB, bool FP4, int TPW, bool QQ>
__global__ __launch_bounds__(kIdxWaves * 64) void index_scores_mfma(IndexArgs A, float* scores, int q_tile) {
  constexpr int H = HB * 32;
  constexpr int KS = FP4 ? 2 : 8;           // k-steps over the 128 dims
  constexpr int QROW = FP4 ? kQRowFp4 : kQRowBf16;
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[H * QROW];
  __shared__ uint32_t qs_lds[H];            // FP4: 4 scale bytes per head
  __shared__ float w_lds[H];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int b = blockIdx.z;
  const int chunk0 = blockIdx.x * (kIdxWaves * TPW * 32);
  const int wave0 = chunk0 + wave * TPW * 32;

  const int q_begin = blockIdx.y * q_tile;
  const int q_end = min(A.n_q, q_begin + q_tile);
  const long row0 = (long)b * A.n_q + q_begin;
  const int ne_raw = A.n_entries[b];
  // QQ (fp32 queries quantised here): the first query's q block of this thread (block i:
  // head i / 4, dims 32 (i % 4) ..), its head weight and its position are requested
  // before the keys.  Loads return in order: requested after the keys, waiting for them
  // waited for every key, and the tiles' products all started after the last key landed.
  static_assert(!QQ || FP4, "in-call quantisation belongs to the MXFP4 path");
  float qv0[QQ ? 32 : 1];
  float w0 = 0.f;
  int qpos0 = 0;
  if constexpr (QQ) {
    const int i = min((int)threadIdx.x, H * 4 - 1);
    const float* qg = (const float*)A.q + (row0 * H + (i >> 2)) * kIdxDim + 32 * (i & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 f = *(const float4*)(qg + 4 * j);
      qv0[4 * j] = f.x; qv0[4 * j + 1] = f.y; qv0[4 * j + 2] = f.z; qv0[4 * j + 3] = f.w;
    }
    w0 = A.w[row0 * H + min((int)threadIdx.x, H - 1)];
    qpos0 = A.q_pos[row0];
    __builtin_amdgcn_sched_barrier(0);   // (the scheduler would hoist the key loads above)
  }

  // ---- keys for this wave's TPW tiles (registers, B operands).  Rows up to n_max lie
  // inside the cache (n_max <= k_cap): they are loaded without waiting for the entry
  // count, and the scores past the visible count are masked below.
  uint4 kb[TPW][KS];
  uint32_t ksc[TPW];
  // FP4: raw buffer loads over the sequence's n_max rows (codes and scales read as 0 past
  // them; such entries are never stored), with no branch, so each tile's products wait
  // for that tile's loads alone
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)A.k + (long)b * A.k_cap * (kIdxDim / 2)), (short)0, A.n_max * (kIdxDim / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A.k_scale + (long)b * A.k_cap * (kIdxDim / 32)), (short)0, A.n_max * (kIdxDim / 32), 0x00020000);
  if (FP4) {   // the scale words first, then the codes tile by tile
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      ksc[t] = __builtin_amdgcn_raw_buffer_load_b32(srs, (wave0 + t * 32 + col) * (kIdxDim / 32), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int e = wave0 + t * 32 + col;
    const bool ok = e < A.n_max;
    if (FP4) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(krs, e * (kIdxDim / 2) + 32 * ks + 16 * half, 0, 0);
        kb[t][ks] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    } else {
      const uint16_t* kr = (const uint16_t*)A.k + ((long)b * A.k_cap + (ok ? e : 0)) * kIdxDim;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[t][ks] = ok ? *(const uint4*)(kr + 16 * ks + 8 * half) : make_uint4(0, 0, 0, 0);
    }
  }

  const int ne = min(ne_raw, A.n_max);
  // one query: FIRST (a compile-time flag) marks the first query of a QQ workgroup,
  // whose inputs were requested before the keys
  auto process = [&](const int qi, auto FIRSTC) {
    constexpr bool FIRST = decltype(FIRSTC)::value;
    const long row = (long)b * A.n_q + qi;
    // ---- stage q (and its scales) and w for this query in LDS
    __syncthreads();
    if (FP4 && A.q_quantize) {
      // fp32 q, quantised here block by block (as the standalone quantiser): block i
      // is head i / 4, dims 32 (i % 4) ..; its codes land where the staged codes would
      const float* qg = (const float*)A.q + row * H * kIdxDim;
      constexpr int kThreads = kIdxWaves * 64;
      auto stage_block = [&](int i, const float (&v)[32]) {
        uint8_t sc;
        *(uint4*)(q_lds + (i >> 2) * QROW + 16 * (i & 3)) = mxfp4_block(v, sc);
        ((uint8_t*)qs_lds)[i] = sc;   // (byte 4 h + p of the scale words: i itself)
      };
      auto load_block = [&](int i, float (&v)[32]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float4 f = *(const float4*)(qg + (i >> 2) * kIdxDim + 32 * (i & 3) + 4 * j);
          v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
        }
      };
      // (the first query's first block per thread was requested before the keys; the
      // branch is uniform, so the wait before its use counts those loads alone)
      int i0 = threadIdx.x;
      if (FIRST) {
        if (i0 < H * 4) {
          float v[32];
#pragma unroll
          for (int j = 0; j < 32; ++j) v[j] = qv0[QQ ? j : 0];
          stage_block(i0, v);
        }
        i0 += kThreads;
      }
      for (int i = i0; i < H * 4; i += kThreads) {
        float v[32];
        load_block(i, v);
        stage_block(i, v);
      }
    } else if (FP4) {
      const uint8_t* qg = (const uint8_t*)A.q + row * H * (kIdxDim / 2);
      for (int i = threadIdx.x; i < H * 4; i += blockDim.x) {   // 16 B pieces: 4 per head
        int h = i >> 2, p = i & 3;
        *(uint4*)(q_lds + h * QROW + 16 * p) = *(const uint4*)(qg + h * 64 + 16 * p);
      }
      for (int h = threadIdx.x; h < H; h += blockDim.x)
        qs_lds[h] = *(const uint32_t*)(A.q_scale + (row * H + h) * 4);
    } else {
      const uint16_t* qg = (const uint16_t*)A.q + row * H * kIdxDim;
      for (int i = threadIdx.x; i < H * 16; i += blockDim.x) {  // 16 B pieces: 16 per head
        int h = i >> 4, p = i & 15;
        *(uint4*)(q_lds + h * QROW + 16 * p) = *(const uint4*)(qg + h * kIdxDim + 8 * p);
      }
    }
    static_assert(H <= kIdxWaves * 64, "one head weight per thread");
    if (FIRST) {
      if ((int)threadIdx.x < H) w_lds[threadIdx.x] = w0;
    } else if ((int)threadIdx.x < H) {
      w_lds[threadIdx.x] = A.w[row * H + threadIdx.x];
    }
    __syncthreads();

    const int V = visible_entries((FIRST) ? qpos0 : A.q_pos[row], ne, A.m);
    // weights of the 16 heads this lane's accumulator rows hold, per head block
    float wl[HB][16];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) wl[hb][r] = w_lds[hb * 32 + 8 * (r / 4) + 4 * half + (r % 4)];

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tile0 = wave0 + t * 32;
      if (tile0 >= V) break;                 // whole tile masked (uniform per wave)
      float part = 0.f;
      // (an empty asm on the tile's scale word keeps its byte extraction in the loop: the
      // compiler would hoist it above the query loop and wait there for every key)
      uint32_t kst = ksc[t];
      if (FP4) asm volatile("" : "+v"(kst));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int head = hb * 32 + col;      // A-operand row of this lane
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (FP4) {
            uint4 a4 = *(const uint4*)(q_lds + head * QROW + 32 * ks + 16 * half);
            i32x8_t av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
            i32x8_t bv = {(int)kb[t][ks].x, (int)kb[t][ks].y, (int)kb[t][ks].z, (int)kb[t][ks].w, 0, 0, 0, 0};
            const int sa = (int)((qs_lds[head] >> (8 * (2 * ks + half))) & 0xff);
            const int sb = (int)((kst >> (8 * (2 * ks + half))) & 0xff);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, sa, 0, sb);
          } else {
            uint4 a4 = *(const uint4*)(q_lds + head * QROW + (16 * ks + 8 * half) * 2);
            acc = mfma32x32x16(as_bf16x8(a4), as_bf16x8(kb[t][ks]), acc);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) part = fmaf(wl[hb][r], relu_f32(acc[r]), part);
      }
      part = add_xor32(part);
      const int e = tile0 + col;
      if (half == 0 && e < A.n_max) scores[row * A.n_max + e] = (e < V) ? part : -INFINITY;
    }
    // tiles skipped above still need their masked scores
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int e = wave0 + t * 32 + col;
      if (wave0 + t * 32 >= V && half == 0 && e < A.n_max) scores[row * A.n_max + e] = -INFINITY;
    }
  };
  if constexpr (QQ) {
    process(q_begin, std::true_type{});   // (QQ workgroups hold one query)
  } else {
    for (int qi = q_begin; qi < q_end; ++qi) process(qi, std::false_type{});
  }
}

// ------------------------------------------- bf16, few queries: keys staged in LDS
// For decode-sized query counts the scores are a stream over the index keys.  A
// workgroup owns 256 consecutive entries: its waves bring the 64 KB of keys (and the
// query's 64 x 128 q) into LDS with direct-to-LDS loads, each instruction 1 KB of
// contiguous rows, so HBM sees whole lines in order.  Inside a 256-byte row the 16-byte
// chunk c lands in slot c ^ (row % 16): the MFMA operand reads (32 rows, one chunk
// each) then hit 16 distinct bank groups.  80 KB of LDS: two workgroups per CU.
constexpr int kIdxLdsEntries = 256;

__device__ __attribute__((aligned(16))) uint8_t g_zero_key[kIdxDim * 2];

__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// SEL: slot e of a row scores key row A.sel[row * n_max + e] (-1: masked) instead of e.
// Each wave owns two 32-entry tiles.  Without SEL the key loads do not wait for
// the entry count: rows up to n_max lie inside the cache (n_max <= k_cap), and the
// scores past the visible count are replaced by -inf whatever the rows hold.
template <int HB, bool SEL>
__global__ __launch_bounds__(kIdxWaves * 64) void index_scores_lds(IndexArgs A, float* scores) {
  constexpr int H = HB * 32;
  constexpr int RB = kIdxDim * 2;                                   // 256-byte rows
  constexpr int TPW = kIdxLdsEntries / (32 * kIdxWaves);            // tiles per wave
  static_assert(TPW == 2, "two key tiles per wave");
  constexpr bool QREG = HB <= 2;   // q fragments held in registers (32 HB of them)
  // tile t of wave w: rows 32 w .. 32 w + 31 of kt[t], entries e0 + 32 (2 w + t) ..
  __shared__ __attribute__((aligned(16))) uint8_t kt0[32 * kIdxWaves * RB];
  __shared__ __attribute__((aligned(16))) uint8_t kt1[32 * kIdxWaves * RB];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[H * RB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int b = blockIdx.z;
  const int qi = blockIdx.y;
  const long row = (long)b * A.n_q + qi;
  const int e0 = blockIdx.x * kIdxLdsEntries;
  const int32_t* sel = SEL ? A.sel + row * A.n_max : nullptr;
  // slot e -> key row to load: -1 = the zero row
  auto key_row = [&](int e) -> int {
    if (e >= A.n_max) return -1;
    if (SEL) return sel[e];
    return e;
  };

  // ---- loads: the visible count, head weights, q, the keys
  const int ne = min(A.n_entries[b], A.n_max);
  const int V = visible_entries(A.q_pos[row], ne, A.m);
  // head weights of this lane's accumulator rows: head 32 hb + 8 (r / 4) + 4 half + r % 4
  f32x4_t wl[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int g = 0; g < 4; ++g) wl[hb][g] = *(const f32x4_t*)(A.w + row * H + 32 * hb + 8 * g + 4 * half);
  // lane l of a 1 KB instruction fills row 4 j + l / 16, slot l % 16 (chunk slot ^ (row % 16))
  const int r_in = lane >> 4, slot = lane & 15;
  const uint8_t* qg = (const uint8_t*)A.q + row * H * RB;
#pragma unroll
  for (int j = 0; j < H / 16; ++j) {   // H / 4 instructions over the 4 waves
    const int hd = (H / 4) * wave + 4 * j + r_in;
    dma16(qg + (long)hd * RB + 16 * (slot ^ (hd & 15)), q_lds + ((H / 4) * wave + 4 * j) * RB);
  }
  int krow[TPW][8];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) krow[t][j] = key_row(e0 + 32 * (TPW * wave + t) + 4 * j + r_in);
  const uint8_t* kb = (const uint8_t*)A.k + (long)b * A.k_cap * RB;
  auto issue_tile = [&](uint8_t* kt, int t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + r_in;   // row within the tile (row % 16 as in the array)
      const int kr = krow[t][j];
      const uint8_t* src = kr >= 0 ? kb + (long)kr * RB + 16 * (slot ^ (r & 15)) : g_zero_key;
      dma16(src, kt + (32 * wave + 4 * j) * RB);
    }
  };
  issue_tile(kt0, 0);
  issue_tile(kt1, 1);
  // (one wait for every load: the compiler cannot tell the LDS arrays the direct loads
  // fill apart, and waits for all of them before the first LDS read anyway)
  wait_vmcnt<0>();
  __syncthreads();   // every wave's share of q

  // q fragments (A operands): head 32 hb + col, 16-byte chunk 2 ks + half
  auto q_frag = [&](int hb, int ks) {
    const int hd = 32 * hb + col, c = 2 * ks + half;
    return *(const uint4*)(q_lds + hd * RB + 16 * (c ^ (hd & 15)));
  };
  uint4 qf[QREG ? HB : 1][8];
  if (QREG) {
#pragma unroll
    for (int hb = 0; hb < (QREG ? HB : 1); ++hb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[hb][ks] = q_frag(hb, ks);
  }
  auto tile = [&](const uint8_t* kt, int t) {
    const int r = 32 * wave + col;               // this lane's entry row (B column) in the array
    const int e = e0 + 32 * (TPW * wave + t) + col;
    f32x16_t acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = 2 * ks + half;
      const uint4 b4 = *(const uint4*)(kt + r * RB + 16 * (c ^ (r & 15)));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        acc[hb] = mfma32x32x16(as_bf16x8(QREG ? qf[QREG ? hb : 0][ks] : q_frag(hb, ks)), as_bf16x8(b4), acc[hb]);
    }
    float part = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int k = 0; k < 4; ++k) part = fmaf(wl[hb][g][k], relu_f32(acc[hb][4 * g + k]), part);
    part = add_xor32(part);
    const bool valid = SEL ? key_row(e) >= 0 : e < V;
    if (half == 0 && e < A.n_max) scores[row * A.n_max + e] = valid ? part : -INFINITY;
  };
  tile(kt0, 0);
  tile(kt1, 1);
}

// ------------------------------------------ bf16, many queries (prefill)
// A workgroup owns 256 consecutive entries (keys in registers, B operands, loaded
// once) and kIdxPfQueries consecutive queries, taken kIdxPfPair at a time.  The next
// pair's q (64 x 128 each, rows swizzled as above) and head weights are loaded into
// the other half of a double buffer by direct-to-LDS loads while this pair's scores
// are formed: one barrier per pair.  Each q fragment read from LDS feeds the MFMAs of
// both key tiles.
constexpr int kIdxPfQueries = 64;
constexpr int kIdxPfPair = 2;

__device__ __forceinline__ void dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

template <int HB>
__global__ __launch_bounds__(kIdxWaves * 64) void index_scores_pf(IndexArgs A, float* scores) {
  constexpr int H = HB * 32;
  constexpr int RB = kIdxDim * 2;
  constexpr int TPW = 2;
  constexpr int P = kIdxPfPair;
  constexpr int QI = H / 16;   // q loads per wave per query (1 KB = 4 heads each)
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[2][P][H * RB];
  __shared__ __attribute__((aligned(16))) float w_lds[2][P][H];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int b = blockIdx.z;
  const int wave0 = blockIdx.x * (kIdxWaves * TPW * 32) + wave * TPW * 32;
  const int ne = min(A.n_entries[b], A.n_max);
  const int q_begin = blockIdx.y * kIdxPfQueries;
  const int q_end = min(A.n_q, q_begin + kIdxPfQueries);
  const int r_in = lane >> 4, slot = lane & 15;
  // the positions of the workgroup's queries, one per lane, read once (a query's V(t) is
  // then a lane broadcast, not a load the causal skip would wait for)
  static_assert(kIdxPfQueries <= 64, "one query position per lane");
  const int qp_lane = q_begin + lane < q_end ? A.q_pos[(long)b * A.n_q + q_begin + lane] : 0;

  // q of the queries q0 .. q0 + P - 1 that exist (and, from wave 0, their head
  // weights) into buffer bi
  auto load_q = [&](int q0, int bi) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (q0 + u >= q_end) break;
      const long row = (long)b * A.n_q + q0 + u;
      const uint8_t* qg = (const uint8_t*)A.q + row * H * RB;
#pragma unroll
      for (int j = 0; j < QI; ++j) {
        const int hd = (H / 4) * wave + 4 * j + r_in;
        dma16(qg + (long)hd * RB + 16 * (slot ^ (hd & 15)), q_lds[bi][u] + ((H / 4) * wave + 4 * j) * RB);
      }
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < H; j += 64)
          if (j + lane < H) dma4(A.w + row * H + j + lane, w_lds[bi][u] + j);
      }
    }
  };
  if (q_begin < q_end) load_q(q_begin, 0);

  // ---- keys for this wave's TPW tiles (registers, B operands); rows up to n_max lie
  // inside the cache, so the loads do not wait for the entry count
  uint4 kb[TPW][8];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int e = wave0 + t * 32 + col;
    const bool ok = e < A.n_max;
    const uint16_t* kr = (const uint16_t*)A.k + ((long)b * A.k_cap + (ok ? e : 0)) * kIdxDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kb[t][ks] = ok ? *(const uint4*)(kr + 16 * ks + 8 * half) : make_uint4(0, 0, 0, 0);
  }

  // A pair's scores are stored one step later, after the next q loads are issued, so
  // that the wait for those loads (which counts stores too) finds the stores done.
  float held[P][TPW];
  long held_row[P];
  int held_V[P];
  int n_held = 0;
  auto store_held = [&]() {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (u >= n_held) break;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int e = wave0 + t * 32 + col;
        if (half == 0 && e < A.n_max) scores[held_row[u] * A.n_max + e] = (e < held_V[u]) ? held[u][t] : -INFINITY;
      }
    }
  };
  for (int q0 = q_begin; q0 < q_end; q0 += P) {
    const int bi = ((q0 - q_begin) / P) & 1;
    // this wave's loads of the pair have landed (the keys, issued later, may not have:
    // the wait covers them too on the first pair)
    wait_vmcnt<0>();
    __syncthreads();   // every wave's, and every wave is past the previous pair
    if (q0 + P < q_end) load_q(q0 + P, bi ^ 1);
    store_held();
    n_held = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (q0 + u >= q_end) break;
      const long row = (long)b * A.n_q + q0 + u;
      const int V = visible_entries(__builtin_amdgcn_readlane(qp_lane, q0 + u - q_begin), ne, A.m);
      const uint8_t* qb = q_lds[bi][u];
      float part[TPW] = {};
      // causal skip: every entry of this wave's tiles at or past V(t) (uniform per wave;
      // the store writes -inf for them)
      if (wave0 < V) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const int hd = 32 * hb + col;
          f32x16_t acc[TPW];
#pragma unroll
          for (int t = 0; t < TPW; ++t) acc[t] = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const int c = 2 * ks + half;
            const uint4 a4 = *(const uint4*)(qb + hd * RB + 16 * (c ^ (hd & 15)));
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t] = mfma32x32x16(as_bf16x8(a4), as_bf16x8(kb[t][ks]), acc[t]);
          }
          // head 32 hb + 8 (r / 4) + 4 half + r % 4 of accumulator row r
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4_t wv = *(const f32x4_t*)&w_lds[bi][u][32 * hb + 8 * g + 4 * half];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
              for (int k = 0; k < 4; ++k) part[t] = fmaf(wv[k], relu_f32(acc[t][4 * g + k]), part[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) held[u][t] = add_xor32(part[t]);
      held_row[u] = row;
      held_V[u] = V;
      n_held = u + 1;
    }
  }
  store_held();
}

template <int HB, bool FP4>
static hipError_t launch_mfma_hb(const IndexArgs& A, float* scores, hipStream_t s) {
  const dim3 block(kIdxWaves * 64);
  if (!FP4 && (A.n_q < 64 || A.sel)) {   // few queries or rescoring: keys through LDS
    dim3 grid((A.n_max + kIdxLdsEntries - 1) / kIdxLdsEntries, A.n_q, A.batch);
    if (A.sel) return launch("index_rescore_bf16", index_scores_lds<HB, true>, grid, block, 0, s, A, scores);
    return launch("index_scores_bf16", index_scores_lds<HB, false>, grid, block, 0, s, A, scores);
  }
  if (!FP4) {   // many queries: keys in registers, q double-buffered in LDS
    dim3 grid((A.n_max + kIdxLdsEntries - 1) / kIdxLdsEntries, (A.n_q + kIdxPfQueries - 1) / kIdxPfQueries,
              A.batch);
    return launch("index_scores_bf16", index_scores_pf<HB>, grid, block, 0, s, A, scores);
  }
  const int q_tile = A.n_q >= 64 ? 16 : 1;
  if (A.q_quantize) {
    // every workgroup reads and quantises all of q (32 KB of fp32 for 64 heads): more
    // entries per workgroup, fewer copies of q read
    constexpr int TPW = 8;
    const int chunk = kIdxWaves * TPW * 32;
    dim3 grid((A.n_max + chunk - 1) / chunk, (A.n_q + q_tile - 1) / q_tile, A.batch);
    // one query per workgroup (decode): its q, head weights and position are requested
    // ahead of the keys (QQ)
    if (q_tile == 1)
      return launch("index_scores_mxfp4", index_scores_mfma<HB, FP4, TPW, FP4>, grid, block, 0, s, A, scores, q_tile);
    return launch("index_scores_mxfp4", index_scores_mfma<HB, FP4, TPW, false>, grid, block, 0, s, A, scores, q_tile);
  }
  constexpr int TPW = 2;
  const int chunk = kIdxWaves * TPW * 32;
  dim3 grid((A.n_max + chunk - 1) / chunk, (A.n_q + q_tile - 1) / q_tile, A.batch);
  return launch("index_scores_mxfp4", index_scores_mfma<HB, FP4, TPW, false>, grid, block, 0, s, A, scores, q_tile);
}

hipError_t launch_index_scores(const IndexArgs& A, float* scores, hipStream_t s) {
  if (A.batch <= 0 || A.n_q <= 0 || A.n_max <= 0) return hipSuccess;
  if (A.dtype == 0) {
    dim3 grid((A.n_max + kIdxF32Threads - 1) / kIdxF32Threads, A.n_q, A.batch);
    size_t lds = sizeof(float) * ((size_t)A.heads * A.dim + A.heads);
    return launch("index_scores_f32", index_scores_f32, grid, dim3(kIdxF32Threads), lds, s, A, scores);
  }
  const bool fp4 = A.dtype == 2;
  switch (A.heads / 32) {
    case 1: return fp4 ? launch_mfma_hb<1, true>(A, scores, s) : launch_mfma_hb<1, false>(A, scores, s);
    case 2: return fp4 ? launch_mfma_hb<2, true>(A, scores, s) : launch_mfma_hb<2, false>(A, scores, s);
    case 3: return fp4 ? launch_mfma_hb<3, true>(A, scores, s) : launch_mfma_hb<3, false>(A, scores, s);
    case 4: return fp4 ? launch_mfma_hb<4, true>(A, scores, s) : launch_mfma_hb<4, false>(A, scores, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
