// Host-side validation of the C ABI's arguments.  Plain C++ with no HIP types or
// calls, so that it can be built and exercised on any host (the sanitizer build of
// the test suite compiles validate.cpp with g++ alone).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Records a printf-style message as the calling thread's last error; returns s.
csa_status fail(csa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
const char* last_error();
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

csa_status check_compress(const csa_compress_desc* d, const void* a, const void* b, const float* za,
                          const float* zb, const void* out);
csa_status check_index(const char* fn, const csa_index_desc* d, const void* q, const uint8_t* qs, const float* w,
                       const void* k, const uint8_t* kscale, const int32_t* ne, const int32_t* qpos);
csa_status check_mqa(const char* fn, const csa_mqa_desc* d, int dense, const void* q, const void* kv,
                     const void* sel, const void* kv_raw, const int32_t* raw_base, const int32_t* qpos,
                     const void* out);
csa_status check_decode(const csa_decode_args* a);

}  // namespace csa
