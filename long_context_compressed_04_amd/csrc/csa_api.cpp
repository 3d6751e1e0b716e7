// C ABI of libcsa.so: host-side validation and dispatch (declarations and the
// contract of every entry point are in include/csa.h).
//
// Validation runs entirely on the host and makes no HIP call, so a rejected
// request enqueues nothing and touches no device.
#include "csa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "csa_kernels.hpp"

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// ----------------------------------------------------------------- compress
csa_status check_compress(const csa_compress_desc* d, const void* a, const void* b, const float* za,
                          const float* zb, const void* out) {
  if (!d) return fail(CSA_ERR_NULL, "csa_compress: desc is NULL");
  if (!a || !b || !za || !zb || !out) return fail(CSA_ERR_NULL, "csa_compress: a, b, za, zb and out are required");
  if ((d->in_dtype != CSA_F32 && d->in_dtype != CSA_BF16) || (d->out_dtype != CSA_F32 && d->out_dtype != CSA_BF16))
    return fail(CSA_ERR_DTYPE, "csa_compress: in_dtype/out_dtype must be CSA_F32 or CSA_BF16");
  if (d->batch < 0 || d->channels < 1 || d->m < 1 || d->m > 256 || d->n_rows < 0 || d->out_cap < 0)
    return fail(CSA_ERR_SHAPE, "csa_compress: need batch >= 0, channels >= 1, 1 <= m <= 256");
  if (d->norm != 0 && d->norm != 1) return fail(CSA_ERR_SHAPE, "csa_compress: norm must be 0 or 1");
  if (d->norm && (d->channels > csa::kCompressNormMaxChannels || !(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps)))
    return fail(CSA_ERR_SHAPE, "csa_compress: norm needs channels <= %d and a finite norm_eps >= 0",
                csa::kCompressNormMaxChannels);
  if (!(d->zc == 1 || d->zc == d->channels)) return fail(CSA_ERR_SHAPE, "csa_compress: zc must be 1 or channels");
  if (d->entry_begin < 0 || d->entry_end < d->entry_begin || d->entry_end > d->out_cap)
    return fail(CSA_ERR_SHAPE, "csa_compress: need 0 <= entry_begin <= entry_end <= out_cap");
  if (d->entry_end > d->entry_begin) {
    long first = (long)d->m * d->entry_begin - (d->entry_begin > 0 ? d->m : 0);
    long last = (long)d->m * d->entry_end;
    if (first < d->tok_base || last > (long)d->tok_base + d->n_rows)
      return fail(CSA_ERR_SHAPE, "csa_compress: token rows [%d, %d) do not cover tokens [%ld, %ld)", d->tok_base,
                  d->tok_base + d->n_rows, first, last);
  }
  return CSA_OK;
}

// ------------------------------------------------------------------- index
csa_status check_index(const char* fn, const csa_index_desc* d, const void* q, const uint8_t* qs, const float* w,
                       const void* k, const uint8_t* kscale, const int32_t* ne, const int32_t* qpos) {
  if (!d) return fail(CSA_ERR_NULL, "%s: desc is NULL", fn);
  if (!q || !w || !k || !ne || !qpos) return fail(CSA_ERR_NULL, "%s: q_idx, w, k_idx, n_entries, q_pos are required", fn);
  if (d->batch < 0 || d->n_q < 0 || d->n_max < 0 || d->k_cap < d->n_max || d->m < 1 || d->topk < 1 || d->topk > 4096)
    return fail(CSA_ERR_SHAPE, "%s: need batch, n_q >= 0, 0 <= n_max <= k_cap, m >= 1, 1 <= topk <= 4096", fn);
  if (d->dtype == CSA_F32) {
    if (d->idx_heads < 1 || d->idx_heads > 128 || d->idx_dim < 1 || d->idx_dim > 256)
      return fail(CSA_ERR_SHAPE, "%s: fp32 indexer needs 1 <= idx_heads <= 128, 1 <= idx_dim <= 256", fn);
    if ((long)d->idx_heads * d->idx_dim > 16384) return fail(CSA_ERR_SHAPE, "%s: idx_heads * idx_dim > 16384", fn);
  } else if (d->dtype == CSA_BF16 || d->dtype == CSA_MXFP4) {
    if (d->idx_dim != 128 || d->idx_heads % 32 != 0 || d->idx_heads < 32 || d->idx_heads > 128)
      return fail(CSA_ERR_UNSUPPORTED, "%s: bf16/MXFP4 indexer needs idx_dim == 128 and idx_heads in {32,64,96,128}", fn);
    if (!aligned16(q) || !aligned16(k)) return fail(CSA_ERR_ALIGN, "%s: q_idx and k_idx must be 16-byte aligned", fn);
    if (d->dtype == CSA_MXFP4) {
      if (d->q_quantize != 0 && d->q_quantize != 1) return fail(CSA_ERR_SHAPE, "%s: q_quantize must be 0 or 1", fn);
      if ((!qs && !d->q_quantize) || !kscale) return fail(CSA_ERR_NULL, "%s: MXFP4 needs q_scale and k_scale", fn);
      if ((qs && !d->q_quantize && ((uintptr_t)qs & 3u)) || ((uintptr_t)kscale & 3u))
        return fail(CSA_ERR_ALIGN, "%s: q_scale and k_scale must be 4-byte aligned", fn);
    } else if (d->q_quantize) {
      return fail(CSA_ERR_DTYPE, "%s: q_quantize applies to CSA_MXFP4 only", fn);
    }
  } else {
    return fail(CSA_ERR_DTYPE, "%s: dtype must be CSA_F32, CSA_BF16 or CSA_MXFP4", fn);
  }
  return CSA_OK;
}

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
csa_status check_mqa(const char* fn, const csa_mqa_desc* d, int dense, const void* q, const void* kv,
                     const void* sel, const void* kv_raw, const int32_t* raw_base, const int32_t* qpos,
                     const void* out) {
  if (!d) return fail(CSA_ERR_NULL, "%s: desc is NULL", fn);
  if (!q || !kv || !sel || !kv_raw || !raw_base || !qpos || !out)
    return fail(CSA_ERR_NULL, "%s: q, kv, %s, kv_raw, raw_base, q_pos and out are required", fn,
                dense ? "n_entries" : "idx");
  if (d->batch < 0 || d->n_q < 0 || d->heads < 1 || d->window < 0 || d->kv_cap < 0 || d->raw_cap < 1)
    return fail(CSA_ERR_SHAPE, "%s: need batch, n_q >= 0, heads >= 1, window >= 0, raw_cap >= 1", fn);
  if (dense) {
    if (d->m < 1 || d->n_max < 0 || d->n_max > d->kv_cap) return fail(CSA_ERR_SHAPE, "%s: need m >= 1, 0 <= n_max <= kv_cap", fn);
  } else if (d->topk < 0 || d->topk > 65536) {
    return fail(CSA_ERR_SHAPE, "%s: need 0 <= topk <= 65536", fn);
  }
  if (!(d->eps >= 0.f) || !std::isfinite(d->scale)) return fail(CSA_ERR_SHAPE, "%s: eps must be >= 0, scale finite", fn);
  if (d->split_items != 0) {
    const long total = (long)(dense ? d->n_max : d->topk) + d->window;
    if (d->split_items < 0 || d->split_items % 32 != 0 || d->split_items > 2048 ||
        (total + d->split_items - 1) / d->split_items > 128)
      return fail(CSA_ERR_SHAPE, "%s: split_items must be 0, or a multiple of 32 <= 2048 giving at most 128 splits",
                  fn);
  }
  if (d->dtype == CSA_F32) {
    if (d->head_dim < 1 || d->head_dim > 512) return fail(CSA_ERR_SHAPE, "%s: fp32 path needs 1 <= head_dim <= 512", fn);
  } else if (d->dtype == CSA_BF16) {
    if (d->head_dim != 512 || d->heads % 16 != 0)
      return fail(CSA_ERR_UNSUPPORTED, "%s: bf16 path needs head_dim == 512 and heads a multiple of 16", fn);
    if (!aligned16(q) || !aligned16(kv) || !aligned16(kv_raw) || !aligned16(out))
      return fail(CSA_ERR_ALIGN, "%s: q, kv, kv_raw and out must be 16-byte aligned", fn);
  } else {
    return fail(CSA_ERR_DTYPE, "%s: dtype must be CSA_F32 or CSA_BF16", fn);
  }
  if (d->kv_dtype != 0) {
    if (d->kv_dtype != CSA_FP8) return fail(CSA_ERR_DTYPE, "%s: kv_dtype must be 0 or CSA_FP8", fn);
    const float sc = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->head_dim);
    if (d->dtype != CSA_BF16 || d->heads % 32 != 0 || sc * 512.f > 68.f)
      return fail(CSA_ERR_UNSUPPORTED, "%s: an FP8 cache needs dtype CSA_BF16, heads a multiple of 32 and scale <= 68/512",
                  fn);
  }
  return CSA_OK;
}

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

namespace csa {

int api_fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

}  // namespace csa

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(int s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "required pointer is NULL";
    case CSA_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case CSA_ERR_DTYPE: return "unsupported dtype";
    case CSA_ERR_ALIGN: return "misaligned pointer";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

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

static csa_status check_decode(const csa_decode_args* a) {
  if (!a) return fail(CSA_ERR_NULL, "csa_decode: args is NULL");
  if (!a->out_idx) return fail(CSA_ERR_NULL, "csa_decode: out_idx is required");
  if (a->index.batch != a->attn.batch || a->index.n_q != a->attn.n_q || a->index.topk != a->attn.topk)
    return fail(CSA_ERR_SHAPE, "csa_decode: index and attn must agree on batch, n_q and topk");
  csa_status st = check_index("csa_decode", &a->index, a->q_idx, a->q_idx_scale, a->w, a->k_idx, a->k_idx_scale,
                              a->n_entries, a->q_pos);
  if (st != CSA_OK) return st;
  st = check_mqa("csa_decode", &a->attn, 0, a->q, a->kv, a->out_idx, a->kv_raw, a->raw_base, a->q_pos, a->out);
  if (st != CSA_OK) return st;
  if (a->attn.kv_dtype != 0 && a->kv_job)
    return fail(CSA_ERR_UNSUPPORTED, "csa_decode: no kv_job with an FP8 cache (compress, then csa_fp8_quantize)");
  const csa_compress_job* jobs[2] = {a->kv_job, a->key_job};
  for (const csa_compress_job* j : jobs) {
    if (!j) continue;
    st = check_compress(&j->desc, j->a, j->b, j->za, j->zb, j->out);
    if (st != CSA_OK) return st;
  }
  return CSA_OK;
}

size_t csa_decode_workspace_size(const csa_decode_args* a) {
  if (!a) return 0;
  csa::MqaArgs M = mqa_args(&a->attn, 0);
  return index_ws(&a->index) + round256(csa::mqa_workspace_bytes(M));
}

csa_status csa_decode(const csa_decode_args* a, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_decode(a);
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
