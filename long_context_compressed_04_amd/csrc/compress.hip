// Compression of token rows into compressed KV entries and indexer keys.
//
// "DeepSeek v4" summary page, section "Compressed Sparse Attention", compressed KV
// entries: two token-level series (streams A and B) with compression weights and
// learnable positional biases; every compressed entry is a row-wise softmax over
// 2m elements; for the first block the previous block's weights are -inf and its
// rows 0.  Anthology record ARXIV-2606.19348, Key takeaways: each entry pools an
// overlapping window of 2m tokens drawn from the two streams.
//
// Entry j: A rows [m*j, m*j+m), B rows [m*(j-1), m*j).  Memory bound: one
// workgroup per (entry, sequence); the 2m softmax weights are computed once into
// LDS (shared logits) or per channel (per-channel logits), then every thread
// streams channels with coalesced row reads.  fp32 arithmetic throughout.
// Optionally the pooled entry is RMS-normalised before it is stored (DeepSeek-V4's
// compressors normalise each pooled entry, index keys included): the fp32 entry is
// kept in LDS until the block has its sum of squares.
#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "launch_timer.hpp"

namespace csa {

constexpr int kCompressThreads = 256;
constexpr int kMaxM = 256;

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs A) {
  const int j = A.entry_begin + blockIdx.x;
  const int b = blockIdx.y;
  const int m = A.m, c = A.channels, zc = A.zc;
  __shared__ float wts[2 * kMaxM];
  __shared__ float red[kCompressThreads / 64];
  __shared__ float pooled[kCompressNormMaxChannels];   // (A.norm only)

  const long a0 = (long)m * j - A.tok_base;      // first A row (relative)
  const long b0 = (long)m * (j - 1) - A.tok_base; // first B row (relative)
  const bool has_b = j > 0;
  const long rows_off = (long)b * A.n_rows;

  auto in_val = [&](const void* base, long row, int ch) -> float {
    long e = (rows_off + row) * c + ch;
    if (IN_BF16) return bf16_to_f32(((const uint16_t*)base)[e]);
    return ((const float*)base)[e];
  };
  auto store = [&](int ch, float v) {
    long o = ((long)b * A.out_cap + j) * c + ch;
    if (OUT_BF16) ((uint16_t*)A.out)[o] = f32_to_bf16(v);
    else ((float*)A.out)[o] = v;
  };
  // the pooled value of channel ch: stored, or kept for the normalisation
  auto emit = [&](int ch, float v) {
    if (A.norm) pooled[ch] = v;
    else store(ch, v);
  };

  if (zc == 1) {
    // Shared logits: softmax over 2m slots computed once.
    float mx = -INFINITY;
    for (int r = threadIdx.x; r < 2 * m; r += blockDim.x) {
      float l;
      if (r < m) {
        l = A.za[rows_off + a0 + r] + (A.bias_a ? A.bias_a[r] : 0.f);
      } else {
        l = has_b ? A.zb[rows_off + b0 + (r - m)] + (A.bias_b ? A.bias_b[r - m] : 0.f) : -INFINITY;
      }
      wts[r] = l;
      mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int i = 1; i < kCompressThreads / 64; ++i) mx = fmaxf(mx, red[i]);
    __syncthreads();
    float part = 0.f;
    for (int r = threadIdx.x; r < 2 * m; r += blockDim.x) {
      float l = wts[r];
      float e = (l == -INFINITY) ? 0.f : expf(l - mx);
      wts[r] = e;
      part += e;
    }
    part = wave_sum(part);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    float den = 0.f;
    for (int i = 0; i < kCompressThreads / 64; ++i) den += red[i];
    const float inv = 1.f / den;
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) {
      float acc = 0.f;
      for (int r = 0; r < m; ++r) acc += (wts[r] * inv) * in_val(A.a, a0 + r, ch);
      if (has_b)
        for (int r = 0; r < m; ++r) acc += (wts[m + r] * inv) * in_val(A.b, b0 + r, ch);
      emit(ch, acc);
    }
  } else {
    // Per-channel logits: each thread owns channels and runs its own softmax.
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) {
      float mx = -INFINITY;
      for (int r = 0; r < m; ++r)
        mx = fmaxf(mx, A.za[(rows_off + a0 + r) * zc + ch] + (A.bias_a ? A.bias_a[r * zc + ch] : 0.f));
      if (has_b)
        for (int r = 0; r < m; ++r)
          mx = fmaxf(mx, A.zb[(rows_off + b0 + r) * zc + ch] + (A.bias_b ? A.bias_b[r * zc + ch] : 0.f));
      float den = 0.f, acc = 0.f;
      for (int r = 0; r < m; ++r) {
        float e = expf(A.za[(rows_off + a0 + r) * zc + ch] + (A.bias_a ? A.bias_a[r * zc + ch] : 0.f) - mx);
        den += e;
        acc += e * in_val(A.a, a0 + r, ch);
      }
      if (has_b)
        for (int r = 0; r < m; ++r) {
          float e = expf(A.zb[(rows_off + b0 + r) * zc + ch] + (A.bias_b ? A.bias_b[r * zc + ch] : 0.f) - mx);
          den += e;
          acc += e * in_val(A.b, b0 + r, ch);
        }
      emit(ch, acc / den);
    }
  }
  if (A.norm) {   // uniform: x * g / sqrt(mean(x^2) + eps) over the entry's channels
    __syncthreads();
    float ss = 0.f;
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) ss = fmaf(pooled[ch], pooled[ch], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < kCompressThreads / 64; ++i) tot += red[i];
    const float inv = 1.f / sqrtf(tot / c + A.norm_eps);
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x)
      store(ch, pooled[ch] * inv * (A.norm_weight ? A.norm_weight[ch] : 1.f));
  }
}

hipError_t launch_compress(const CompressArgs& A, hipStream_t s) {
  int n = A.entry_end - A.entry_begin;
  if (n <= 0 || A.batch <= 0) return hipSuccess;
  dim3 grid(n, A.batch), block(kCompressThreads);
  if (A.in_bf16 && A.out_bf16) return launch("compress", compress_kernel<true, true>, grid, block, 0, s, A);
  if (A.in_bf16) return launch("compress", compress_kernel<true, false>, grid, block, 0, s, A);
  if (A.out_bf16) return launch("compress", compress_kernel<false, true>, grid, block, 0, s, A);
  return launch("compress", compress_kernel<false, false>, grid, block, 0, s, A);
}

// ---------------------------------------------------------------------------------
// MXFP4 (OCP MX v1.0) quantisation: one thread per block of 32 values.
// E = floor(log2 amax) - 2 (clamped to [-127, 127]; -127 for an all-zero block);
// codes = nearest e2m1 value of x * 2^-E with ties to the even code, saturating.

template <bool IN_BF16>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const void* x, int64_t n_blocks, uint8_t* codes,
                                                             uint8_t* scales) {
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  float v[32];
  if (IN_BF16) {
    const uint4* p = (const uint4*)((const uint16_t*)x + blk * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 q = p[i];
      uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[i * 8 + 2 * k] = __uint_as_float(w4[k] << 16);
        v[i * 8 + 2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = (const float4*)((const float*)x + blk * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 q = p[i];
      v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
  }
  uint8_t scale;
  *(uint4*)(codes + blk * 16) = mxfp4_block(v, scale);
  scales[blk] = scale;
}

// FP8 E4M3 quantisation: one thread per 8 values.  gfx950's conversion rounds to the
// nearest E4M3 value (ties to even) but turns values beyond the range into NaN, so
// they are clamped to +-448 first.
template <bool IN_BF16>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void* x, int64_t n8, uint8_t* codes) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n8) return;
  float v[8];
  if (IN_BF16) {
    const uint4 q = *((const uint4*)x + g);
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w4[k] << 16);
      v[2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
    }
  } else {
    const float4 a = *((const float4*)x + 2 * g), b = *((const float4*)x + 2 * g + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = fminf(fmaxf(v[4 * h + k], -448.f), 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], r, true);
    w[h] = (uint32_t)r;
  }
  *((uint2*)codes + g) = make_uint2(w[0], w[1]);
}

hipError_t launch_fp8_quantize(int in_bf16, const void* x, int64_t n, uint8_t* codes, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  if (in_bf16) return launch("fp8_quantize", fp8_quantize_kernel<true>, grid, block, 0, s, x, n8, codes);
  return launch("fp8_quantize", fp8_quantize_kernel<false>, grid, block, 0, s, x, n8, codes);
}

hipError_t launch_mxfp4_quantize(int in_bf16, const void* x, int64_t n_blocks, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)((n_blocks + 255) / 256)), block(256);
  if (in_bf16) return launch("mxfp4_quantize", mxfp4_quantize_kernel<true>, grid, block, 0, s, x, n_blocks, codes, scales);
  return launch("mxfp4_quantize", mxfp4_quantize_kernel<false>, grid, block, 0, s, x, n_blocks, codes, scales);
}

}  // namespace csa
