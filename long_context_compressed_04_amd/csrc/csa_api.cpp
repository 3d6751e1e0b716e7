// C ABI of libcsa.so: dispatch (declarations and the contract of every entry point
// are in include/csa.h).  Every argument is checked first by the HIP-free
// validation in validate.cpp, so a rejected request enqueues nothing and touches no
// device.
#include "csa.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "csa_kernels.hpp"
#include "validate.hpp"

namespace {

using csa::aligned16;
using csa::check_compress;
using csa::check_index;
using csa::check_mqa;
using csa::fail;

csa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

csa::IndexArgs index_args(const csa_index_desc* d, const void* q, const uint8_t* qs, const float* w, const void* k,
                          const uint8_t* ks, const int32_t* ne, const int32_t* qpos) {
  csa::IndexArgs A;
  A.batch = d->batch; A.n_q = d->n_q; A.heads = d->idx_heads; A.dim = d->idx_dim; A.m = d->m; A.topk = d->topk;
  A.n_max = d->n_max; A.k_cap = d->k_cap; A.dtype = d->dtype;
  A.q = q; A.q_scale = qs; A.w = w; A.k = k; A.k_scale = ks; A.n_entries = ne; A.q_pos = qpos;
  A.q_quantize = d->dtype == CSA_MXFP4 ? d->q_quantize : 0;
  return A;
}

// Score rows, with 16 bytes of slack: the top-k kernels read rows 16 bytes at a time.
size_t scores_ws(const csa_index_desc* d) {
  return round256(sizeof(float) * (size_t)d->batch * d->n_q * (size_t)d->n_max + 16);
}
size_t index_ws(const csa_index_desc* d) {
  csa::IndexArgs A{};
  A.batch = d->batch; A.n_q = d->n_q; A.n_max = d->n_max; A.topk = d->topk;
  return scores_ws(d) + round256(csa::topk_workspace_bytes(A));
}

// --------------------------------------------------------------------- MQA
csa::MqaArgs mqa_args(const csa_mqa_desc* d, int dense) {
  csa::MqaArgs A{};
  A.batch = d->batch; A.n_q = d->n_q; A.heads = d->heads; A.dim = d->head_dim; A.topk = dense ? 0 : d->topk;
  A.m = d->m; A.n_max = d->n_max; A.window = d->window; A.kv_cap = d->kv_cap; A.raw_cap = d->raw_cap;
  A.dense = dense; A.bf16 = d->dtype == CSA_BF16;
  A.scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->head_dim);
  A.eps = d->eps;
  A.split_items = d->split_items;
  A.kv_f8 = d->kv_dtype == CSA_FP8;
  return A;
}

}  // namespace


extern "C" {


csa_status csa_compress(const csa_compress_desc* d, const void* a, const void* b, const float* za, const float* zb,
                        const float* bias_a, const float* bias_b, const float* norm_weight, void* out, void* stream) {
  csa_status st = check_compress(d, a, b, za, zb, out);
  if (st != CSA_OK) return st;
  csa::CompressArgs A;
  A.batch = d->batch; A.channels = d->channels; A.m = d->m; A.zc = d->zc; A.n_rows = d->n_rows;
  A.tok_base = d->tok_base; A.entry_begin = d->entry_begin; A.entry_end = d->entry_end; A.out_cap = d->out_cap;
  A.in_bf16 = d->in_dtype == CSA_BF16; A.out_bf16 = d->out_dtype == CSA_BF16;
  A.a = a; A.b = b; A.za = za; A.zb = zb; A.bias_a = bias_a; A.bias_b = bias_b; A.out = out;
  A.norm = d->norm; A.norm_eps = d->norm_eps; A.norm_weight = norm_weight;
  return hip_status(csa::launch_compress(A, (hipStream_t)stream), "csa_compress");
}

csa_status csa_fp8_quantize(int32_t dtype, const void* x, int64_t n, uint8_t* codes, void* stream) {
  if (!x || !codes) return fail(CSA_ERR_NULL, "csa_fp8_quantize: x and codes are required");
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "csa_fp8_quantize: dtype must be CSA_F32 or CSA_BF16");
  if (n < 0 || n % 8 != 0) return fail(CSA_ERR_SHAPE, "csa_fp8_quantize: n must be a non-negative multiple of 8");
  if (!aligned16(x) || ((uintptr_t)codes & 7u))
    return fail(CSA_ERR_ALIGN, "csa_fp8_quantize: x must be 16-byte and codes 8-byte aligned");
  return hip_status(csa::launch_fp8_quantize(dtype == CSA_BF16, x, n, codes, (hipStream_t)stream),
                    "csa_fp8_quantize");
}

csa_status csa_mxfp4_quantize(int32_t dtype, const void* x, int64_t n_blocks, uint8_t* codes, uint8_t* scales,
                              void* stream) {
  if (!x || !codes || !scales) return fail(CSA_ERR_NULL, "csa_mxfp4_quantize: x, codes and scales are required");
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "csa_mxfp4_quantize: dtype must be CSA_F32 or CSA_BF16");
  if (n_blocks < 0) return fail(CSA_ERR_SHAPE, "csa_mxfp4_quantize: n_blocks < 0");
  if (!aligned16(x) || !aligned16(codes)) return fail(CSA_ERR_ALIGN, "csa_mxfp4_quantize: x and codes must be 16-byte aligned");
  return hip_status(csa::launch_mxfp4_quantize(dtype == CSA_BF16, x, n_blocks, codes, scales, (hipStream_t)stream),
                    "csa_mxfp4_quantize");
}

size_t csa_index_workspace_size(const csa_index_desc* d) { return d ? index_ws(d) : 0; }

csa_status csa_index_scores(const csa_index_desc* d, const void* q, const uint8_t* qs, const float* w, const void* k,
                            const uint8_t* ks, const int32_t* ne, const int32_t* qpos, float* scores, void* stream) {
  csa_status st = check_index("csa_index_scores", d, q, qs, w, k, ks, ne, qpos);
  if (st != CSA_OK) return st;
  if (!scores) return fail(CSA_ERR_NULL, "csa_index_scores: scores is required");
  csa::IndexArgs A = index_args(d, q, qs, w, k, ks, ne, qpos);
  return hip_status(csa::launch_index_scores(A, scores, (hipStream_t)stream), "csa_index_scores");
}

csa_status csa_index_topk(const csa_index_desc* d, const void* q, const uint8_t* qs, const float* w, const void* k,
                          const uint8_t* ks, const int32_t* ne, const int32_t* qpos, int32_t* out_idx, float* out_score,
                          void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_index("csa_index_topk", d, q, qs, w, k, ks, ne, qpos);
  if (st != CSA_OK) return st;
  if (!out_idx) return fail(CSA_ERR_NULL, "csa_index_topk: out_idx is required");
  const size_t need = index_ws(d);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_index_topk: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  csa::IndexArgs A = index_args(d, q, qs, w, k, ks, ne, qpos);
  hipStream_t s = (hipStream_t)stream;
  float* scores = (float*)ws;
  st = hip_status(csa::launch_index_scores(A, scores, s), "csa_index_topk (scores)");
  if (st != CSA_OK) return st;
  const size_t sws = scores_ws(d);
  return hip_status(csa::launch_topk_rows(A, scores, out_idx, out_score, (char*)ws + sws, ws_bytes - sws, s),
                    "csa_index_topk (select)");
}

// --------------------------------------------------------- MXFP4 + rescoring
static size_t rescore_ws(const csa_index_desc* d, int32_t cand) {
  csa_index_desc dc = *d;
  dc.topk = cand;
  const size_t rows = (size_t)d->batch * d->n_q;
  return index_ws(&dc) + round256(rows * (size_t)cand * sizeof(int32_t)) +
         round256(rows * (size_t)cand * sizeof(float) + 16);   // (rescored rows: 16 bytes of slack)
}

size_t csa_index_rescored_workspace_size(const csa_index_desc* d, int32_t cand) {
  return (d && cand >= 1) ? rescore_ws(d, cand) : 0;
}

csa_status csa_index_topk_rescored(const csa_index_desc* d, int32_t cand, const void* q, const uint8_t* qs,
                                   const void* q16, const float* w, const void* k, const uint8_t* ks,
                                   const void* k16, const int32_t* ne, const int32_t* qpos, int32_t* out_idx,
                                   float* out_score, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_index_topk_rescored";
  csa_status st = check_index(fn, d, q, qs, w, k, ks, ne, qpos);
  if (st != CSA_OK) return st;
  if (d->dtype != CSA_MXFP4) return fail(CSA_ERR_DTYPE, "%s: the prefilter must be CSA_MXFP4", fn);
  if (cand < d->topk || cand > 8192) return fail(CSA_ERR_SHAPE, "%s: need topk <= cand <= 8192", fn);
  if (!out_idx || !q16 || !k16) return fail(CSA_ERR_NULL, "%s: out_idx, q_bf16 and k_bf16 are required", fn);
  if (!aligned16(q16) || !aligned16(k16)) return fail(CSA_ERR_ALIGN, "%s: q_bf16 and k_bf16 must be 16-byte aligned", fn);
  const size_t need = rescore_ws(d, cand);
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  csa_index_desc dc = *d;
  dc.topk = cand;
  const size_t rows = (size_t)d->batch * d->n_q;
  const size_t iws = index_ws(&dc), sws = scores_ws(&dc);
  int32_t* cands = (int32_t*)((char*)ws + iws);
  float* rescored = (float*)((char*)ws + iws + round256(rows * (size_t)cand * sizeof(int32_t)));
  hipStream_t s = (hipStream_t)stream;
  // 1. MXFP4 scores, the cand best (ascending, -1 padded)
  csa::IndexArgs A = index_args(&dc, q, qs, w, k, ks, ne, qpos);
  float* scores = (float*)ws;
  st = hip_status(csa::launch_index_scores(A, scores, s), "csa_index_topk_rescored (prefilter scores)");
  if (st != CSA_OK) return st;
  st = hip_status(csa::launch_topk_rows(A, scores, cands, nullptr, (char*)ws + sws, iws - sws, s),
                  "csa_index_topk_rescored (prefilter select)");
  if (st != CSA_OK) return st;
  // 2. bf16 scores of the candidates: slot e of a row is key cands[e]
  csa::IndexArgs B = A;
  B.dtype = CSA_BF16;
  B.q = q16;
  B.q_scale = nullptr;
  B.k = k16;
  B.k_scale = nullptr;
  B.q_quantize = 0;
  B.n_max = cand;
  B.sel = cands;
  st = hip_status(csa::launch_index_scores(B, rescored, s), "csa_index_topk_rescored (rescore)");
  if (st != CSA_OK) return st;
  // 3. the topk best candidates; a row holds min(cand, V) valid candidates, which is
  //    the visible count with n_max = cand
  csa::IndexArgs C = B;
  C.topk = d->topk;
  C.sel = nullptr;
  C.map = cands;
  return hip_status(csa::launch_topk_rows(C, rescored, out_idx, out_score, nullptr, 0, s),
                    "csa_index_topk_rescored (select)");
}

size_t csa_mqa_workspace_size(const csa_mqa_desc* d, int32_t dense) {
  if (!d) return 0;
  csa::MqaArgs A = mqa_args(d, dense);
  return round256(csa::mqa_workspace_bytes(A));
}

static csa_status run_mqa(const char* fn, const csa_mqa_desc* d, int dense, const void* q, const void* kv,
                          const int32_t* idx, const int32_t* ne, const void* kv_raw, const int32_t* raw_base,
                          const int32_t* qpos, const float* g, const float* sink, const float* rope, void* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t s) {
  csa::MqaArgs A = mqa_args(d, dense);
  const size_t need = round256(csa::mqa_workspace_bytes(A));
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  A.q = q; A.kv = kv; A.idx = idx; A.n_entries = ne; A.kv_raw = kv_raw; A.raw_base = raw_base; A.q_pos = qpos;
  A.gamma = g; A.sink = sink; A.rope = rope; A.out = out; A.lse = lse;
  if (rope && d->head_dim < 64) return fail(CSA_ERR_SHAPE, "%s: rope needs head_dim >= 64", fn);
  if (A.kv_f8 && g) return fail(CSA_ERR_UNSUPPORTED, "%s: an FP8 cache needs rms_weight NULL", fn);
  return hip_status(csa::launch_mqa(A, ws, ws_bytes, s), fn);
}

csa_status csa_sparse_mqa(const csa_mqa_desc* d, const void* q, const void* kv, const int32_t* idx, const void* kv_raw,
                          const int32_t* raw_base, const int32_t* qpos, const float* g, const float* sink,
                          const float* rope, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_mqa("csa_sparse_mqa", d, 0, q, kv, idx, kv_raw, raw_base, qpos, out);
  if (st != CSA_OK) return st;
  return run_mqa("csa_sparse_mqa", d, 0, q, kv, idx, nullptr, kv_raw, raw_base, qpos, g, sink, rope, out, lse, ws,
                 ws_bytes, (hipStream_t)stream);
}

csa_status hca_dense_mqa(const csa_mqa_desc* d, const void* q, const void* kv, const int32_t* ne, const void* kv_raw,
                         const int32_t* raw_base, const int32_t* qpos, const float* g, const float* sink,
                         const float* rope, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_mqa("hca_dense_mqa", d, 1, q, kv, ne, kv_raw, raw_base, qpos, out);
  if (st != CSA_OK) return st;
  return run_mqa("hca_dense_mqa", d, 1, q, kv, nullptr, ne, kv_raw, raw_base, qpos, g, sink, rope, out, lse, ws,
                 ws_bytes, (hipStream_t)stream);
}

size_t csa_decode_workspace_size(const csa_decode_args* a) {
  if (!a) return 0;
  csa::MqaArgs M = mqa_args(&a->attn, 0);
  return index_ws(&a->index) + round256(csa::mqa_workspace_bytes(M));
}

csa_status csa_decode(const csa_decode_args* a, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = csa::check_decode(a);
  if (st != CSA_OK) return st;
  const size_t iws = index_ws(&a->index);
  const size_t need = csa_decode_workspace_size(a);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_decode: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  hipStream_t s = (hipStream_t)stream;
  const csa_compress_job* jobs[2] = {a->kv_job, a->key_job};
  for (const csa_compress_job* j : jobs) {
    if (!j) continue;
    st = csa_compress(&j->desc, j->a, j->b, j->za, j->zb, j->bias_a, j->bias_b, j->norm_weight, j->out, stream);
    if (st != CSA_OK) return st;
  }
  st = csa_index_topk(&a->index, a->q_idx, a->q_idx_scale, a->w, a->k_idx, a->k_idx_scale, a->n_entries, a->q_pos,
                      a->out_idx, a->out_score, ws, iws, stream);
  if (st != CSA_OK) return st;
  return run_mqa("csa_decode", &a->attn, 0, a->q, a->kv, a->out_idx, nullptr, a->kv_raw, a->raw_base, a->q_pos,
                 a->rms_weight, a->sink, a->rope, a->out, a->lse, (uint8_t*)ws + iws, ws_bytes - iws, s);
}

}  // extern "C"
