// Device helpers for top-k selection: order keys and cross-lane scans.
#pragma once
#include "csa_device.hpp"

namespace csa {

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Cross-lane steps on DPP (data-parallel primitives: a VALU operand read from another
// lane of the same 16-lane row, a few cycles) rather than LDS permutes.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowRor1 = 0x121, kDppRowRor2 = 0x122, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// v of lane src(CTRL) for lanes in ROW_MASK rows, 0 elsewhere and for lanes with no source
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes: within rows by shifts 1, 2, 4, 8, then row
// totals carried across rows (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp0<kDppRowShr1>(v);
  v += dpp0<kDppRowShr2>(v);
  v += dpp0<kDppRowShr4>(v);
  v += dpp0<kDppRowShr8>(v);
  v += dpp0<kDppRowBcast15, 0xA>(v);
  v += dpp0<kDppRowBcast31, 0xC>(v);
  return v;
}

// Sum over the 16 lanes of each row (every lane of the row gets it): rotations 1, 2, 4, 8.
__device__ __forceinline__ uint32_t row_sum16(uint32_t v) {
  v += dpp0<kDppRowRor1>(v);
  v += dpp0<kDppRowRor2>(v);
  v += dpp0<kDppRowRor4>(v);
  v += dpp0<kDppRowRor8>(v);
  return v;
}

}  // namespace csa
