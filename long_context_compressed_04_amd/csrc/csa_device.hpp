// Device-side helpers shared by the CSA / HCA kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

// max(x, 0) as one integer max on the bits: a float with the sign bit set is a
// negative int32.  (fmaxf costs a second instruction, which quiets a signalling NaN
// first; here a NaN with a clear sign bit passes through unchanged.)
__device__ __forceinline__ float relu_f32(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Order-preserving map fp32 -> uint32 (larger float <=> larger key).
// (u ^ mask, mask = all ones for a negative float and only the sign bit otherwise:
// three VALU operations, where the select form takes four)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// s_waitcnt for "at most N vector-memory operations of this wave still outstanding"
// (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left unwaited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---- cross-lane steps on the VALU (no trip through LDS, unlike a shuffle)
// v of lane l ^ 1, l ^ 2 (DPP quad permutations), 7 - l within 8 lanes (half mirror),
// 15 - l within 16 (mirror): every lane has a source, and summing over these pairs
// gives every lane of a group the same bits.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// the value of lane ^ 16 (^ 32) beside the lane's own: a permlane swap of v with
// itself exchanges odd and even 16-lane rows (the two 32-lane halves); the pair it
// returns holds both values, in an order that depends on the lane
__device__ __forceinline__ float add_xor16(float v) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
// sum (max) over each 16-lane row; every lane of the row gets the same value
__device__ __forceinline__ float row_sum16f(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  return v + dpp_f32<kDppMirror>(v);
}
__device__ __forceinline__ float row_max16f(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f32<kDppMirror>(v));
}
__device__ __forceinline__ float wave_sum(float v) { return add_xor32(add_xor16(row_sum16f(v))); }
__device__ __forceinline__ float wave_max(float v) { return max_xor32(max_xor16(row_max16f(v))); }

// Number of compressed entries visible to the query at absolute position t:
// only complete blocks, V(t) = min(N, floor((t+1)/m)).
__device__ __forceinline__ int visible_entries(int t, int n_entries, int m) {
  int v = (t + 1) / m;
  v = v < n_entries ? v : n_entries;
  return v < 0 ? 0 : v;
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Block-wide exclusive scan of one uint32 per thread (NT threads, NT % 64 == 0).
// `tmp` must hold NT/64 + 1 words of LDS.  Returns the exclusive prefix; *total
// receives the sum.  Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      uint32_t t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[NT / 64] = run;
  }
  __syncthreads();
  uint32_t res = tmp[wave] + inc - v;
  *total = tmp[NT / 64];
  __syncthreads();
  return res;
}


// ---- MXFP4 (OCP MX v1.0): one block of 32 values -> 16 code bytes (element 2i in
// the low nibble of byte i) and its e8m0 scale byte.  Shared exponent
// E = floor(log2(max|x|)) - 2 clamped to [-127, 127] (-127 for an all-zero block);
// element code = nearest e2m1 value of |x| / 2^E (ties to the even code, saturating
// at 6) with the sign of x.
__device__ __forceinline__ int floor_log2_f32(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xff);
  if (e != 0) return e - 127;
  uint32_t mant = u & 0x7fffffu;                 // subnormal: position of leading one
  return -149 + (31 - __clz((int)mant));
}

// The division and rounding are gfx950's scaled FP4 conversion (two values per
// instruction, byte `sel` of the word): it divides by the scale and reads only the
// scale's exponent field, so 2^E is built from E + 127 directly (all zero bits for
// E = -127).
__device__ __forceinline__ uint4 mxfp4_block(const float (&v)[32], uint8_t& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int E = (amax == 0.f) ? -127 : floor_log2_f32(amax) - 2;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    w[p] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[p], v[8 * p], v[8 * p + 1], sc, 0);
    w[p] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[p], v[8 * p + 2], v[8 * p + 3], sc, 1);
    w[p] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[p], v[8 * p + 4], v[8 * p + 5], sc, 2);
    w[p] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[p], v[8 * p + 6], v[8 * p + 7], sc, 3);
  }
  scale = (uint8_t)(E + 127);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace csa
