// Internal launcher interface between the C ABI (csa_api.cpp) and the HIP kernels.
// All sizes were validated by the caller; launchers only enqueue work.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa_limits.hpp"

namespace csa {

struct CompressArgs {
  int batch, channels, m, zc, n_rows, tok_base, entry_begin, entry_end, out_cap;
  int in_bf16, out_bf16;
  const void* a; const void* b; const float* za; const float* zb;
  const float* bias_a; const float* bias_b; void* out;
  int norm = 0;                       // RMSNorm of each produced entry
  float norm_eps = 0.f;
  const float* norm_weight = nullptr; // [channels] or ones
};
hipError_t launch_compress(const CompressArgs& A, hipStream_t s);

hipError_t launch_mxfp4_quantize(int in_bf16, const void* x, int64_t n_blocks, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_fp8_quantize(int in_bf16, const void* x, int64_t n, uint8_t* codes, hipStream_t s);

// dtype: 0 = fp32, 1 = bf16, 2 = mxfp4
struct IndexArgs {
  int batch, n_q, heads, dim, m, topk, n_max, k_cap, dtype;
  const void* q; const uint8_t* q_scale; const float* w;
  const void* k; const uint8_t* k_scale;
  const int32_t* n_entries; const int32_t* q_pos;
  // Rescoring (bf16, few-query kernel): score slot e of row r is key row
  // sel[r * n_max + e] (-1: masked) instead of key row e.
  const int32_t* sel = nullptr;
  // Top-k: the selected slot p of row r is written as map[r * n_max + p].
  const int32_t* map = nullptr;
  // MXFP4: q holds fp32 values, quantised in the indexer as the standalone quantiser does
  int q_quantize = 0;
};
// Score rows [batch*n_q, n_max] (-inf past the visible count).
hipError_t launch_index_scores(const IndexArgs& A, float* scores, hipStream_t s);
// Top-k per score row.
// Rows longer than the LDS-resident limit use `ws` (topk_workspace_bytes).
size_t topk_workspace_bytes(const IndexArgs& A);
hipError_t launch_topk_rows(const IndexArgs& A, const float* scores, int32_t* out_idx,
                            float* out_score, void* ws, size_t ws_bytes, hipStream_t s);

struct MqaArgs {
  int batch, n_q, heads, dim, topk, m, n_max, window, kv_cap, raw_cap, dense, bf16;
  float scale, eps;
  const void* q; const void* kv; const int32_t* idx; const int32_t* n_entries;
  const void* kv_raw; const int32_t* raw_base; const int32_t* q_pos; const float* gamma;
  void* out; float* lse;
  int split_items = 0;   // > 0: batch-invariant split boundaries (multiples of it)
  int kv_f8 = 0;         // kv and kv_raw hold FP8 E4M3 rows (bf16 path, 32-head groups)
  const float* sink = nullptr;   // [heads] sink logits (natural log), or none
  const float* rope = nullptr;   // [rows, 128] cos[64], sin[64] of each query: rope-conjugate output
};
// Workspace bytes the MQA path needs for these sizes (split partials).
size_t mqa_workspace_bytes(const MqaArgs& A);
hipError_t launch_mqa(const MqaArgs& A, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace csa
