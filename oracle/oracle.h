/*
 * Prototypes of the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.
 * The arithmetic, its citations and the readings it takes are documented beside
 * each function in oracle.c.  Used by oracle.c itself (so that the definitions
 * match) and by the sanitizer driver of the test suite.
 */
#ifndef ORACLE_H_
#define ORACLE_H_
#include <stdint.h>

int oracle_compress(const double* A, const double* Bv, const double* za, const double* zb, const double* bias_a,
                    const double* bias_b, long tok_base, long n_rows, int c, int m, int zc, long entry_begin,
                    long entry_end, double* out);
void oracle_rmsnorm(const double* x, long rows, int d, const double* gamma, double eps, double* out);
long oracle_visible(long t, long n_entries, int m);
void oracle_index_scores(const double* q, const double* w, const double* K, int H_I, int d_I, long n,
                         double* scores);
void oracle_topk(const double* scores, long n_visible, int k, int32_t* out);
int oracle_sparse_mqa(const double* q, const double* kv, long n_entries, const int32_t* idx, int k,
                      const double* kv_raw, long n_raw, long raw_base, long t, int window, int H, int d,
                      double scale, double eps, const double* gamma, const double* sink, double* out,
                      double* lse);
int oracle_dense_mqa(const double* q, const double* kv, long n_entries, int m, const double* kv_raw, long n_raw,
                     long raw_base, long t, int window, int H, int d, double scale, double eps,
                     const double* gamma, const double* sink, double* out, double* lse);
void oracle_mxfp4_quantize(const double* x, long n_blocks, uint8_t* codes, uint8_t* scales);
void oracle_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, long n_blocks, double* x);
void oracle_fp8_quantize(const double* x, long n, uint8_t* codes);
void oracle_fp8_dequantize(const uint8_t* codes, long n, double* x);
void oracle_rope_conjugate(double* out, int H, int d, const double* cs);

#endif /* ORACLE_H_ */
