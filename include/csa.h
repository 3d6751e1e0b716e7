/*
 * csa.h -- C ABI of libcsa.so: Compressed Sparse Attention (CSA) and Heavily
 * Compressed Attention (HCA) of DeepSeek-V4 on AMD Instinct MI355X (gfx950).
 *
 * The method, as the public pages describe it:
 *  - "DeepSeek v4" (Korean summary page), section "Compressed Sparse Attention":
 *    compressed KV entries (two token-level series C_a, C_b with weights Z_a, Z_b
 *    and positional biases, a row-wise softmax over 2m elements, the first block
 *    padded), the lightning indexer (score = sum over indexer heads of a per-head
 *    weight times ReLU(q . K) for each preceding compressed block), the top-k
 *    selector, and the sliding-window entries appended to the selected ones;
 *    section on the hybrid CSA/HCA attention (HCA compresses m' >> m tokens per
 *    entry and stays dense).
 *  - "DeepSeek-AI (2026) - ARXIV-2606.19348" anthology record, Key takeaways: two
 *    latent KV streams pooled over overlapping 2m-token windows; an RMSNorm on each
 *    query head and on the single compressed-KV head before the core attention.
 *  - "DeepSeek-V4-Pro" techniques map: one KV head shared by all query heads
 *    (multi-query attention), sliding window of 128 (the window keeps w-1 past
 *    tokens plus the current one), index_topk with invalid slots set to -1, QK
 *    normalisation, FP4 precision for the attention indexer.
 *
 * Conventions common to every call
 *  - Tensor pointers are DEVICE pointers (HIP device memory, e.g. from torch).
 *    Descriptors and scalar arguments live in host memory and are read before the
 *    call returns.  The caller owns every buffer, including the workspace.
 *  - Layouts are row-major with the innermost dimension contiguous.  Per-sequence
 *    caches are [batch, capacity, width]: sequence b's row r starts at element
 *    (b * capacity + r) * width.  Token positions are absolute int32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    the call returns without synchronising.  The library allocates no device
 *    memory and keeps no state between calls (launch timing, at the end of this
 *    file, aside).
 *  - Errors: every argument is validated on the host before anything is launched;
 *    on failure nothing is enqueued, a csa_status code is returned and
 *    csa_last_error() describes it.  A failed launch returns CSA_ERR_HIP.  Values
 *    that live in device memory (positions, counts, indices) cannot be checked on
 *    the host: kernels never access memory outside the described buffers, and an
 *    index or window row outside its buffer is skipped (contributes nothing).
 *  - Workspaces: sized by the matching *_workspace_size call.  A workspace must be
 *    zero-filled before its first use; any counters the library keeps in it are back
 *    at zero when the enqueued work completes.  Two calls in flight at once must not
 *    share one workspace.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL */
  CSA_ERR_SHAPE = 2,       /* sizes inconsistent or outside the supported range */
  CSA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination */
  CSA_ERR_ALIGN = 4,       /* a pointer is not aligned as the kernel requires */
  CSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than *_workspace_size */
  CSA_ERR_UNSUPPORTED = 6, /* valid request the library does not implement */
  CSA_ERR_HIP = 7          /* the HIP runtime reported an error */
} csa_status;

typedef enum {
  CSA_F32 = 0,   /* IEEE binary32 */
  CSA_BF16 = 1,  /* bfloat16 stored as uint16 bit patterns */
  CSA_MXFP4 = 2, /* OCP MX v1.0 MXFP4: 4-bit e2m1 codes, two per byte (even element in
                    the low nibble), plus one e8m0 scale byte per 32 elements */
  CSA_FP8 = 3    /* OCP FP8 E4M3 ("E4M3FN"): one byte per element, bias 7, max 448, no
                    scale (the KV cache variant: csa_mqa_desc.kv_dtype) */
} csa_dtype;

/* Returns CSA_ABI_VERSION. */
int csa_abi_version(void);
/* Static description of a status code. */
const char* csa_status_string(int status);
/* Detail of the last failure on the calling thread (thread-local storage; valid until
   the next call on that thread). */
const char* csa_last_error(void);

/* ------------------------------------------------------------------------------
 * csa_compress -- overlapping two-stream softmax pooling of token rows into
 * compressed entries ("DeepSeek v4" summary, "Compressed Sparse Attention",
 * compressed KV entries; anthology record, Key takeaways).  Also builds the
 * indexer keys, which use the same operation on their own streams.
 *
 * Entry j pools the A stream over tokens [m*j, m*j+m) and the B stream over the
 * previous block [m*(j-1), m*j): logits l = z + positional bias over those 2m
 * slots, weights = softmax(l) (per channel when zc == channels, shared when
 * zc == 1), entry = sum of weight * row.  Entry 0 has no B half (logits -inf,
 * rows 0).  Arithmetic in fp32.
 *
 *   a, b     [batch, n_rows, channels]  in_dtype; row r = absolute token tok_base + r
 *   za, zb   [batch, n_rows, zc]        fp32 pooling logits of the A and B streams
 *   bias_a, bias_b  [m, zc] fp32 positional biases, or NULL for zero
 *   out      [batch, out_cap, channels] out_dtype; entry j is written to row j
 * Entries [entry_begin, entry_end) are produced.  Requires the rows they need to be
 * present: m*entry_begin - (entry_begin > 0 ? m : 0) >= tok_base and
 * m*entry_end <= tok_base + n_rows; entry_end <= out_cap; 1 <= m <= 256.
 * A bias_b of -inf everywhere masks the lagging stream: every entry then pools the
 * m tokens of its own block only (non-overlapping, single-stream pooling).
 * norm = 1: each entry is RMS-normalised in fp32 before it is stored,
 * entry * g / sqrt(mean(entry^2) + norm_eps) with g = norm_weight [channels] fp32
 * (NULL = ones); channels <= 4096.  (DeepSeek-V4's compressors normalise every
 * pooled entry, the indexer's keys included; the attention calls of this library
 * normalise the KV rows they read themselves, so the KV cache needs no norm here.)
 * ---------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t channels;
  int32_t m;
  int32_t zc;            /* 1 or channels */
  int32_t n_rows;
  int32_t tok_base;
  int32_t entry_begin;
  int32_t entry_end;
  int32_t out_cap;
  int32_t in_dtype;      /* CSA_F32 or CSA_BF16 */
  int32_t out_dtype;     /* CSA_F32 or CSA_BF16 */
  int32_t norm;          /* 0: entries as pooled; 1: RMS-normalised (see above) */
  float norm_eps;        /* norm = 1: epsilon, >= 0 */
} csa_compress_desc;

csa_status csa_compress(const csa_compress_desc* desc, const void* a, const void* b,
                        const float* za, const float* zb, const float* bias_a,
                        const float* bias_b, const float* norm_weight, void* out, void* stream);

/* ------------------------------------------------------------------------------
 * csa_mxfp4_quantize -- OCP MX v1.0 MXFP4 encoding of n_blocks blocks of 32
 * consecutive values (the pages' FP4 indexer QK path: forum post on the DeepSeek
 * V4 paper; techniques map, "FP4 precision for the attention indexer").
 * Shared exponent E = floor(log2(max|x|)) - 2 clamped to [-127, 127] (E = -127 for
 * an all-zero block), scale byte = E + 127; element code = x / 2^E rounded to the
 * nearest e2m1 value (ties to the even code), saturating at 6, sign bit = sign of x.
 *   x       [n_blocks * 32]  dtype CSA_F32 or CSA_BF16
 *   codes   [n_blocks * 16]  bytes
 *   scales  [n_blocks]       bytes
 * ---------------------------------------------------------------------------- */
csa_status csa_mxfp4_quantize(int32_t dtype, const void* x, int64_t n_blocks, uint8_t* codes,
                              uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------------
 * csa_fp8_quantize -- FP8 E4M3 encoding of n values ("DeepSeek-V4-Pro" techniques
 * map, inference quantization: FP8 KV-cache quantization), for a compressed KV
 * cache and window rows kept in FP8 (csa_mqa_desc.kv_dtype = CSA_FP8).  Per
 * element, no scale: x is clamped to [-448, 448] and rounded to the nearest E4M3
 * value, ties to the even code; the sign bit copies the sign of x.
 *   x      [n]  dtype CSA_F32 or CSA_BF16, 16-byte aligned
 *   codes  [n]  bytes, 8-byte aligned;   n a multiple of 8
 * ---------------------------------------------------------------------------- */
csa_status csa_fp8_quantize(int32_t dtype, const void* x, int64_t n, uint8_t* codes, void* stream);

/* ------------------------------------------------------------------------------
 * Lightning indexer and top-k ("DeepSeek v4" summary, "Compressed Sparse
 * Attention", lightning indexer; techniques map, "Indexer-selected sparse
 * attention").  For each query (sequence b, query i at absolute position
 * t = q_pos[b*n_q+i]) only complete, preceding blocks are visible:
 * V = min(n_entries[b], floor((t+1)/m)).  For s < V:
 *     score[s] = sum_h w[h] * max(0, q_idx[h] . k_idx[s])        (no scale)
 * csa_index_topk keeps the `topk` largest scores (ties by lower index) and writes
 * their entry indices in ascending index order, then -1 for the remaining slots
 * when V < topk.  The indexer does not normalise q or k.
 *
 *   q_idx  [batch, n_q, idx_heads, idx_dim]  dtype (MXFP4: codes [.., idx_dim/2] bytes)
 *   q_scale  MXFP4 only: [batch, n_q, idx_heads, idx_dim/32] bytes, else NULL
 *   w      [batch, n_q, idx_heads] fp32 head weights
 *   k_idx  [batch, k_cap, idx_dim] dtype (MXFP4: codes [batch, k_cap, idx_dim/2])
 *   k_scale  MXFP4 only: [batch, k_cap, idx_dim/32] bytes, else NULL
 *   n_entries [batch] int32 (<= n_max);  q_pos [batch, n_q] int32
 *   out_idx   [batch, n_q, topk] int32
 *   out_score [batch, n_q, topk] fp32 score of each selected entry (-inf for -1), or NULL
 * Supported: CSA_F32 any idx_dim <= 256 and idx_heads <= 128; CSA_BF16 and CSA_MXFP4
 * with idx_dim == 128 and idx_heads in {32, 64, 96, 128}.  1 <= topk <= 4096,
 * n_max <= k_cap; CSA_MXFP4 also n_max <= 16,777,216 (else CSA_ERR_SHAPE).
 * ---------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t n_q;
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t m;
  int32_t topk;
  int32_t n_max;      /* upper bound of n_entries[b] over the batch */
  int32_t k_cap;      /* rows per sequence in k_idx */
  int32_t dtype;      /* CSA_F32, CSA_BF16 or CSA_MXFP4 (q_idx and k_idx) */
  int32_t q_quantize; /* CSA_MXFP4 only: 0 = q_idx / q_scale hold MXFP4 codes and scales;
                         1 = q_idx holds fp32 values [.., idx_dim], quantised inside the
                         call exactly as csa_mxfp4_quantize would (q_scale unused) */
} csa_index_desc;

size_t csa_index_workspace_size(const csa_index_desc* desc);

/* Scores only: writes score rows [batch, n_q, n_max] fp32 (-inf at s >= V). */
csa_status csa_index_scores(const csa_index_desc* desc, const void* q_idx, const uint8_t* q_scale,
                            const float* w, const void* k_idx, const uint8_t* k_scale,
                            const int32_t* n_entries, const int32_t* q_pos, float* scores,
                            void* stream);

csa_status csa_index_topk(const csa_index_desc* desc, const void* q_idx, const uint8_t* q_scale,
                          const float* w, const void* k_idx, const uint8_t* k_scale,
                          const int32_t* n_entries, const int32_t* q_pos, int32_t* out_idx,
                          float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * csa_index_topk_rescored -- the MXFP4 selector as a prefilter, then an exact
 * rescoring (the pages' FP4 QK selector: forum post on the DeepSeek V4 paper;
 * techniques map, "FP4 precision for the attention indexer"; the pages give no
 * rescoring step: this is a labelled variant that trades one small gather for
 * selection recall).  Per query:
 *   1. the `cand` best visible entries by the MXFP4 score (as csa_index_topk with
 *      topk = cand; q_idx / k_idx and their scales as there);
 *   2. each candidate's score recomputed with the bf16 indexer from q_bf16 and
 *      k_bf16, bf16 copies of the same queries and keys (same formula, fp32
 *      accumulation);
 *   3. the desc->topk best rescored candidates (ties to the lower entry index),
 *      written in ascending index order, -1 padded when fewer than topk are
 *      visible; out_score (nullable) receives their rescored scores.
 *   desc     dtype CSA_MXFP4, idx_dim 128, idx_heads in {32, 64, 96, 128}
 *   cand     desc->topk <= cand <= 8192
 *   q_bf16   [batch, n_q, idx_heads, 128] bf16, 16-byte aligned
 *   k_bf16   [batch, k_cap, 128] bf16, 16-byte aligned
 * The workspace (csa_index_rescored_workspace_size) holds the MXFP4 score rows, the
 * candidate lists and their rescored scores.
 * ---------------------------------------------------------------------------- */
size_t csa_index_rescored_workspace_size(const csa_index_desc* desc, int32_t cand);
csa_status csa_index_topk_rescored(const csa_index_desc* desc, int32_t cand, const void* q_idx,
                                   const uint8_t* q_scale, const void* q_bf16, const float* w,
                                   const void* k_idx, const uint8_t* k_scale, const void* k_bf16,
                                   const int32_t* n_entries, const int32_t* q_pos, int32_t* out_idx,
                                   float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Core multi-query attention ("DeepSeek-V4-Pro" techniques map, "Grouped-query
 * attention", "Sliding-window attention", "QK normalization"; anthology record,
 * Key takeaways: RMSNorm on every query head and on the compressed KV head).
 * All `heads` query heads share one KV head; each KV row is both key and value.
 * Every query head and every attended row is RMS-normalised:
 *     x_hat = x * g / sqrt(mean(x^2) + eps),  g = rms_weight (NULL = ones).
 * The attended set of the query at position t is its compressed entries (sparse:
 * idx, -1 skipped; dense: every s < V(t)) plus the raw tokens
 * u in [max(0, t-window+1), t], read from kv_raw row u - raw_base[b].  One softmax
 * over the whole set with logits scale * q_hat . k_hat (scale <= 0 selects
 * 1/sqrt(head_dim)); out = sum softmax * k_hat.  An empty set gives out = 0 and
 * lse = -inf.
 * Attention sink ("DeepSeek-V4-Pro" techniques map, "Learnable attention sink": one
 * learnable logit per head joins the softmax denominator): sink [heads] fp32, or
 * NULL for none.  With a sink s_h the softmax runs over the set plus one extra logit
 * s_h whose value vector is zero, so out = sum exp(l_j) k_hat_j / (sum exp(l_j) +
 * exp(s_h)) and lse includes exp(s_h).  |s_h| <= 80.
 * Rope-conjugate output ("DeepSeek-V4-Pro" techniques map, "Gated attention output" and
 * "Partial RoPE": the output is rotated back before the output projection; RoPE
 * covers the trailing 64 dims of a head, x*cos + rotate_half(x)*sin).  V4's rotary
 * turns interleaved pairs: within the rotated slice, rotate_half(x)_{2j} = -x_{2j+1}
 * and rotate_half(x)_{2j+1} = x_{2j}.  rope [batch, n_q, 128] fp32 = the query's
 * cos[64] then sin[64], one value per rotated dim (V4's per-pair angle repeated on
 * both dims of its pair), or NULL for none.  With rope, dims head_dim-64 ..
 * head_dim-1 of every output head become x*cos - rotate_half(x)*sin (head_dim >= 64);
 * lse is unchanged.
 *
 *   q      [batch, n_q, heads, head_dim] dtype
 *   kv     [batch, kv_cap, head_dim]     dtype, or E4M3 bytes with kv_dtype = CSA_FP8
 *                                        (compressed entries)
 *   idx    [batch, n_q, topk] int32 (sparse only)
 *   n_entries [batch] int32 (dense only, <= n_max)
 *   kv_raw [batch, raw_cap, head_dim] as kv;  raw_base [batch] int32
 *   q_pos  [batch, n_q] int32
 *   out    [batch, n_q, heads, head_dim] dtype
 *   lse    [batch, n_q, heads] fp32 natural-log softmax denominator, or NULL
 * Supported: CSA_F32 with head_dim <= 512; CSA_BF16 with head_dim == 512 and heads a
 * multiple of 16.  q, kv, kv_raw, out 16-byte aligned.
 * ---------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t n_q;
  int32_t heads;
  int32_t head_dim;
  int32_t topk;       /* sparse: idx slots per query */
  int32_t m;          /* dense: compression ratio for V(t) */
  int32_t n_max;      /* dense: upper bound of n_entries[b] */
  int32_t window;     /* >= 0 */
  int32_t kv_cap;
  int32_t raw_cap;
  float scale;
  float eps;
  int32_t dtype;      /* CSA_F32 or CSA_BF16 */
  int32_t split_items; /* 0: the library picks the kernel and where a query's items
                          are split for speed, which may change with the batch;
                          > 0 (a multiple of 32, <= 2048, at most 128 splits of the
                          largest set): batch-invariant decoding, the set is split at
                          multiples of split_items and the splits are merged in a
                          fixed order by a fixed kernel, so each query's output is the
                          same, bit for bit, whatever batch it is computed in
                          ("DeepSeek-V4-Pro" techniques map, inference kernels:
                          batch-invariant attention decoding, separate split-K outputs
                          with a deterministic reduction) */
  int32_t kv_dtype;   /* 0: kv and kv_raw hold `dtype` rows.  CSA_FP8: they hold FP8
                         E4M3 rows of head_dim bytes (csa_fp8_quantize; no scale),
                         read as their exact bf16 values ("DeepSeek-V4-Pro"
                         techniques map, FP8 KV cache).  Requires dtype CSA_BF16,
                         head_dim 512, heads a multiple of 32, rms_weight NULL and
                         a scale <= 68/512 (0 selects 1/sqrt(512)); kv and kv_raw
                         16-byte aligned.  Otherwise CSA_ERR_UNSUPPORTED */
} csa_mqa_desc;

/* Workspace of csa_sparse_mqa / hca_dense_mqa (dense = 1) for desc: the split partials
 * (per query, split and head: the split's softmax average in fp16, its maximum and sum
 * in fp32) and, for the 128-head kernel with many queries, an RMS-normalised bf16 copy
 * of every kv and kv_raw row (1 KiB per cached row), written by the call itself.
 * 0 when the call needs none. */
size_t csa_mqa_workspace_size(const csa_mqa_desc* desc, int32_t dense);

csa_status csa_sparse_mqa(const csa_mqa_desc* desc, const void* q, const void* kv,
                          const int32_t* idx, const void* kv_raw, const int32_t* raw_base,
                          const int32_t* q_pos, const float* rms_weight, const float* sink,
                          const float* rope, void* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

csa_status hca_dense_mqa(const csa_mqa_desc* desc, const void* q, const void* kv,
                         const int32_t* n_entries, const void* kv_raw, const int32_t* raw_base,
                         const int32_t* q_pos, const float* rms_weight, const float* sink,
                         const float* rope, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------------
 * csa_decode -- one fused CSA step for n_q queries per sequence, stream-ordered:
 * optional compression of newly completed blocks (kv_job / key_job, as
 * csa_compress), then the indexer and top-k (as csa_index_topk, writing out_idx),
 * then sparse MQA over the selected entries plus the window (as csa_sparse_mqa).
 * index.batch/n_q must equal attn.batch/n_q and index.topk == attn.topk.
 * A job writes its entries [entry_begin, entry_end) before the indexer reads the
 * keys, so n_entries[b] must already count them (entry_end when the step's block
 * has just completed: t + 1 = m * entry_end).  The jobs' out pointers are normally
 * the kv and k_idx caches of this call; one entry range serves the whole batch.
 * ---------------------------------------------------------------------------- */
typedef struct {
  csa_compress_desc desc;
  const void* a;
  const void* b;
  const float* za;
  const float* zb;
  const float* bias_a;
  const float* bias_b;
  const float* norm_weight;
  void* out;
} csa_compress_job;

typedef struct {
  csa_index_desc index;
  csa_mqa_desc attn;
  const csa_compress_job* kv_job;   /* NULL = none */
  const csa_compress_job* key_job;  /* NULL = none */
  const void* q;
  const void* kv;
  const void* kv_raw;
  const int32_t* raw_base;
  const int32_t* q_pos;
  const float* rms_weight;
  const float* sink;                /* nullable: per-head sink logits (as csa_sparse_mqa) */
  const float* rope;                /* nullable: cos/sin of the query positions (as csa_sparse_mqa) */
  const void* q_idx;
  const uint8_t* q_idx_scale;
  const float* w;
  const void* k_idx;
  const uint8_t* k_idx_scale;
  const int32_t* n_entries;
  int32_t* out_idx;                 /* required: the selected entries */
  float* out_score;                 /* nullable */
  void* out;
  float* lse;                       /* nullable */
} csa_decode_args;

size_t csa_decode_workspace_size(const csa_decode_args* args);
csa_status csa_decode(const csa_decode_args* args, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * csa_decode_noalloc -- csa_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is the library's own device-resident scratch array of
 * CSA_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU, held from the first call on that
 * GPU until the process ends; nothing is allocated or freed by the call.  Arguments
 * and outputs as csa_decode (the caller still passes every input and output).
 * Returns CSA_ERR_WORKSPACE, enqueueing nothing, when csa_decode_workspace_size(args)
 * exceeds the scratch size (csa_decode with a workspace of the caller's serves
 * larger steps).  Every call on one GPU uses that GPU's one array, which keeps the
 * previous call's contents (harmless: the step writes every workspace byte it reads
 * before reading it, and keeps no counters there): calls that overlap in time on one
 * GPU (other streams or threads) race and give undefined results; serialise them.
 * ---------------------------------------------------------------------------- */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa_status csa_decode_noalloc(const csa_decode_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * Launch timing (diagnostics; not part of the method).  csa_timing_enable(1)
 * makes the library bracket every later kernel launch with a pair of HIP events
 * recorded on the launch stream (launches on a stream that is being captured into
 * a graph are not timed); csa_timing_enable(0) stops it.  This is the one piece of
 * state the library keeps across calls: the events, created on first use and
 * reused.  csa_timing_collect waits for every recorded launch to finish, writes
 * up to `cap` per-kernel aggregates (in order of first launch; kernels beyond `cap`
 * are dropped) to `out` and forgets the records; it returns the number of entries
 * written.  With out == NULL it only returns the number of distinct kernels
 * launched so far: it neither waits nor forgets anything.  Thread-safe.
 * ---------------------------------------------------------------------------- */
typedef struct {
  char name[40];      /* kernel name, NUL-terminated */
  int32_t launches;
  double total_us;
  double min_us;
  double max_us;
} csa_kernel_time;

csa_status csa_timing_enable(int32_t on);
int32_t csa_timing_collect(csa_kernel_time* out, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
