// gdn_kernels.hpp -- launch parameters and host launchers shared between the
// kernel translation units and the C-ABI front end.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct DecodeParams {
    int B, Hk, Hv, G;
    float scale, eps_l2, eps_rms;
    const float* conv_w;
    const float* A_log;
    const float* dt_bias;
    const float* norm_w;
    const void *q, *k, *v, *z, *a, *b;
    int64_t qs, ks, vs, zs, as, bs;     // token strides, elements
    const float* state_in;
    float* state_out;
    const void* conv_in;
    void* conv_out;
    void* out;
    int out_bf16;
    float* core_out;
};

struct PrefillParams {
    int N, Hk, Hv, G;
    int64_t T;
    int max_chunks;                      // grid bound on sum_n ceil(L_n / C)
    float scale, eps_l2, eps_rms;
    const int32_t* cu;
    const float* conv_w;
    const float* A_log;
    const float* dt_bias;
    const float* norm_w;
    const void *q, *k, *v, *z, *a, *b;
    int64_t qs, ks, vs, zs, as, bs;
    const float* state_in;
    float* state_out;
    const void* conv_in;
    void* conv_out;
    void* out;
    int out_bf16;
    float* core;                          // o before the gated norm (user or workspace)
    // workspace views
    int32_t* chunk_off;                   // [N+1] first chunk of each sequence
    float* decay;                         // [max_chunks][Hv] exp(gamma_last)
    uint8_t* vch;                         // [max_chunks][Hv] per-chunk operand blocks
};

// Bytes of the per-(chunk, value head) operand block for a compiled shape.
__host__ __device__ constexpr int ck_pad(int C) { return C < 32 ? 32 : C; }
__host__ __device__ constexpr int64_t vch_bytes(int DK, int DV, int C) {
    return 4ll * C * DK        // -W   (A fragments, hi+lo bf16)
         + 4ll * C * DK        // Q_G  (A fragments)
         + 4ll * DK * ck_pad(C)  // K_d^T (A fragments)
         + 4ll * C * ck_pad(C)   // P    (A fragments)
         + 4ll * C * DV;       // U~   (fp32 accumulator fragments)
}

hipError_t launch_decode(int DK, int DV, bool bf16, const DecodeParams& p, hipStream_t s,
                         bool* supported);
// events: NULL, or 5 events recorded before each of the 4 kernels and after the last
hipError_t launch_prefill(int DK, int DV, int C, bool bf16, const PrefillParams& p,
                          hipStream_t s, bool* supported, hipEvent_t const* events);
bool prefill_shape_supported(int DK, int DV, int C);
bool decode_shape_supported(int DK, int DV);
hipError_t launch_selftest_mfma(const float* A, const float* B, float* C, hipStream_t s);

}  // namespace gdn
