// CPU build of the packer's exact integer arithmetic (quant_exact.h), exported
// for tests that run without a GPU. The GPU kernels compile the same header.
#include <cstdint>

#include "quant_exact.h"

#define HC_API extern "C" __attribute__((visibility("default")))

HC_API int64_t mqh_fp16_units(uint32_t h) { return mq::fp16_units(h); }
HC_API uint32_t mqh_fp16_div7(uint64_t A, uint64_t* S) { return mq::fp16_div7(A, S); }
HC_API uint32_t mqh_fp16_round_units(uint64_t V, uint64_t* R) { return mq::fp16_round_units(V, R); }
HC_API uint32_t mqh_fp32_div7(uint64_t Mx, uint64_t* m, int* Q) { return mq::fp32_div7(Mx, m, Q); }
HC_API int mqh_quant7(int64_t a, uint64_t S) { return mq::quant7(a, S); }
HC_API int mqh_quant7_scaled(int64_t e, uint64_t m, int Q) { return mq::quant7_scaled(e, m, Q); }
HC_API uint64_t mqh_err_key(uint64_t abs_e) { return mq::err_key(abs_e); }
HC_API uint32_t mqh_fp16_div7_h(uint32_t h) { return mq::fp16_div7_h(h); }
HC_API int mqh_quant7_f(float x, float s) { return mq::quant7_f(x, s); }
