// Host-only stand-ins for the library's kernel launchers (launch.h), so that
// the C ABI layer (abi.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and exercised on a machine without a GPU.
//
// Each launcher records its name and arguments and returns hipSuccess, or the
// error set by _fp8bsq_stub_fail_next (to check the ELAUNCH mapping).  The
// accessors start with an underscore so the export check of the ABI tests
// leaves them out.  Test infrastructure only: nothing here is linked into
// libfp8bsq.so.
#include <stdint.h>
#include <string.h>

#include "launch.h"

namespace {

struct Record {
  char name[64];
  int64_t ints[16];
  const void *ptrs[12];
  int nints, nptrs;
};

Record g_last;
int g_calls = 0;
hipError_t g_fail = hipSuccess;

struct Rec {
  explicit Rec(const char *name) {
    memset(&g_last, 0, sizeof(g_last));
    strncpy(g_last.name, name, sizeof(g_last.name) - 1);
    ++g_calls;
  }
  Rec &i(int64_t v) {
    g_last.ints[g_last.nints++] = v;
    return *this;
  }
  Rec &p(const void *v) {
    g_last.ptrs[g_last.nptrs++] = v;
    return *this;
  }
};

hipError_t result() {
  const hipError_t e = g_fail;
  g_fail = hipSuccess;
  return e;
}

}  // namespace

namespace fp8bsq {

hipError_t launch_act_quant(const void *x, bool x_bf16, int64_t nblocks, bool ue8m0, uint8_t *y,
                            float *s, hipStream_t stream) {
  Rec("act_quant").p(x).i(x_bf16).i(nblocks).i(ue8m0).p(y).p(s).p(stream);
  return result();
}

hipError_t launch_weight_dequant(const uint8_t *x, const float *s, int64_t m, int64_t n, void *y,
                                 bool y_bf16, hipStream_t stream) {
  Rec("weight_dequant").p(x).p(s).i(m).i(n).p(y).i(y_bf16).p(stream);
  return result();
}

hipError_t launch_weight_quant(const void *x, bool x_bf16, int64_t m, int64_t n, bool ue8m0,
                               uint8_t *y, float *s, hipStream_t stream) {
  Rec("weight_quant").p(x).i(x_bf16).i(m).i(n).i(ue8m0).p(y).p(s).p(stream);
  return result();
}

hipError_t launch_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream, const void *bias, bool a_s_pow2) {
  Rec("block_gemm").p(a).p(a_s).p(b).p(b_s).p(c).i(c_bf16).i(m).i(n).i(k).p(stream).p(bias).i(a_s_pow2);
  return result();
}

hipError_t launch_block_gemm_reference(const uint8_t *a, const float *a_s, const uint8_t *b,
                                       const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                       int64_t k, hipStream_t stream, const void *bias) {
  Rec("block_gemm_reference").p(a).p(a_s).p(b).p(b_s).p(c).i(c_bf16).i(m).i(n).i(k).p(stream).p(bias);
  return result();
}

size_t block_gemm_split_bytes(int64_t m, int64_t n, int64_t k) {
  return (size_t)(m * 1000000 + n * 1000 + k);   // a value the test can recognize
}

hipError_t launch_block_gemm_split(const uint8_t *a, const float *a_s, const uint8_t *b,
                                   const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                   int64_t k, hipStream_t stream, bool a_s_pow2, void *workspace,
                                   size_t workspace_bytes) {
  Rec("block_gemm_split").p(a).p(a_s).p(b).p(b_s).p(c).i(c_bf16).i(m).i(n).i(k).p(stream).i(a_s_pow2)
      .p(workspace).i((int64_t)workspace_bytes);
  return result();
}

// the stand-in's scratch is "too small" for m == 777
hipError_t launch_block_gemm_split_noalloc(const uint8_t *a, const float *a_s, const uint8_t *b,
                                           const float *b_s, void *c, bool c_bf16, int64_t m,
                                           int64_t n, int64_t k, hipStream_t stream, bool a_s_pow2,
                                           bool *too_big) {
  *too_big = m == 777;
  if (*too_big) return hipSuccess;
  Rec("block_gemm_split_noalloc").p(a).p(a_s).p(b).p(b_s).p(c).i(c_bf16).i(m).i(n).i(k).p(stream).i(a_s_pow2);
  return result();
}

hipError_t launch_act_quant_gemm_fused(const void *x, bool ue8m0, const uint8_t *b,
                                      const float *b_s, const void *bias, void *c, bool c_bf16,
                                      int64_t m, int64_t n, int64_t k, uint8_t *a_q, float *a_s,
                                      hipStream_t stream) {
  Rec("act_quant_gemm_fused").p(x).i(ue8m0).p(b).p(b_s).p(bias).p(c).i(c_bf16).i(m).i(n).i(k).p(a_q)
      .p(a_s).p(stream);
  return result();
}

// the stand-in fuses bf16 activations of up to 16 rows and 96 K codes
bool act_quant_gemm_fusable(bool x_bf16, int64_t m, int64_t k) {
  return x_bf16 && m <= 16 && k > 0 && k <= 20480 && m * k <= 98304;
}

}  // namespace fp8bsq

extern "C" {

// Name, integer and pointer arguments of the last launcher call; returns the
// number of launcher calls so far.
__attribute__((visibility("default"))) int _fp8bsq_stub_last(char *name, int name_len, int64_t *ints,
                                                             const void **ptrs) {
  strncpy(name, g_last.name, (size_t)name_len - 1);
  name[name_len - 1] = 0;
  memcpy(ints, g_last.ints, sizeof(g_last.ints));
  memcpy(ptrs, g_last.ptrs, sizeof(g_last.ptrs));
  return g_calls;
}

// The next launcher call returns hipErrorLaunchFailure.
__attribute__((visibility("default"))) void _fp8bsq_stub_fail_next(void) { g_fail = hipErrorLaunchFailure; }

}  // extern "C"
