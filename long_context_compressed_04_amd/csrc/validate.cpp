// Host-side validation of the C ABI's arguments (declarations in validate.hpp).
// No HIP: a rejected request enqueues nothing and touches no device.
#include "validate.hpp"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "csa_limits.hpp"

namespace csa {
namespace {

thread_local std::string g_last_error;

}  // namespace

const char* last_error() { return g_last_error.c_str(); }

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

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
  if (d->norm && (d->channels > kCompressNormMaxChannels || !(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps)))
    return fail(CSA_ERR_SHAPE, "csa_compress: norm needs channels <= %d and a finite norm_eps >= 0",
                kCompressNormMaxChannels);
  if (!(d->zc == 1 || d->zc == d->channels)) return fail(CSA_ERR_SHAPE, "csa_compress: zc must be 1 or channels");
  if (d->entry_begin < 0 || d->entry_end < d->entry_begin || d->entry_end > d->out_cap)
    return fail(CSA_ERR_SHAPE, "csa_compress: need 0 <= entry_begin <= entry_end <= out_cap");
  if (d->entry_end > d->entry_begin) {
    long first = (long)d->m * d->entry_begin - (d->entry_begin > 0 ? d->m : 0);
    long last = (long)d->m * d->entry_end;
    if (last > INT_MAX) return fail(CSA_ERR_SHAPE, "csa_compress: token positions past 2^31 - 1");
    if (first < d->tok_base || last > (long)d->tok_base + d->n_rows)
      return fail(CSA_ERR_SHAPE, "csa_compress: token rows [%d, %ld) do not cover tokens [%ld, %ld)", d->tok_base,
                  (long)d->tok_base + d->n_rows, first, last);
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
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
      return fail(CSA_ERR_ALIGN, "%s: q_idx, k_idx and w must be 16-byte aligned", fn);
    if (d->dtype == CSA_MXFP4) {
      if (d->q_quantize != 0 && d->q_quantize != 1) return fail(CSA_ERR_SHAPE, "%s: q_quantize must be 0 or 1", fn);
      // (the kernel reads a sequence's keys through a buffer descriptor of n_max * 64 bytes)
      if (d->n_max > (1 << 24)) return fail(CSA_ERR_SHAPE, "%s: MXFP4 needs n_max <= 16777216", fn);
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

csa_status check_decode(const csa_decode_args* a) {
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

const char* csa_last_error(void) { return csa::last_error(); }

}  // extern "C"
