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
    int Ts;                              // 0: one token (decode); else tokens per sequence (rows b*Ts ..)
    float* snap;                         // [B][Ts][Hv][dk][dv] state after each token, or NULL
    const int32_t* slots;                // [B] pool entry of each sequence's states, or NULL (entry b)
    int num_slots;                       // pool entries (with slots)
    int32_t* status;                     // optional: a sequence with an out-of-range entry is skipped and reported
    // one-token step with one work-group per value head (Ts = 0 only):
    // arrival counters [B][Hk], zero on entry and left zero.  NULL: one
    // work-group per key head.
    uint32_t* arrive;
};


constexpr int kMaxVerifyTokens = 16;     // tokens per sequence of one multi-token decode

// Pool entry holding sequence n's recurrent and conv state.
__device__ __forceinline__ int state_slot(const int32_t* slots, int n) { return slots ? slots[n] : n; }

// Status bit of a device-side index out of its documented range
// (cu_seqlens not starting at 0, decreasing or not ending at T_total; a
// state pool entry outside [0, num_slots)); equal to GDN_STATUS_BAD_INDEX.
constexpr int32_t kStatusBadIndex = 2;

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
    int core_f16;                         // 1: `core` holds o as fp16 (the workspace copy), 0: fp32 (core_out)
    const int32_t* slots;                 // [N] pool entry of each sequence's states, or NULL (entry n)
    int num_slots;                        // pool entries (with slots)
    int32_t* status;                      // optional: cleared by the first kernel, then status bits ORed in
    // workspace views
    int32_t* chunk_off;                   // [N+1] first chunk of each sequence (written by the first prep);
                                          // chunk_off[N] < 0: the call's indices were rejected
    float* decay;                         // [max_chunks][Hv] exp(gamma_last)
    float* sink;                          // [64] target of stores to rows past a sequence end
    float* carry;                         // [2][Hv][dk][dv] state across a window boundary
    uint8_t* vch;                         // [win_slots][Hv] per-chunk operand blocks of a window
    // chunk-slot window [win_lo, win_hi) of one prep + scan pass (window
    // win_idx of ceil(max_chunks / win_slots)); the operand blocks of a
    // window are reused by the next one
    int win_slots, win_lo, win_hi, win_idx;
};

// Bytes of the per-(chunk, value head) operand block for a compiled shape:
// the scan's matrix-core operands as fp16 fragments (the output products'
// Q_G and P as hi + lo pairs), U~ as fp32 fragments.
__host__ __device__ constexpr int ck_pad(int C) { return C < 32 ? 32 : C; }
__host__ __device__ constexpr int64_t vch_bytes(int DK, int DV, int C) {
    return 2ll * C * DK          // -W    (A fragments)
         + 4ll * C * DK          // Q_G   (A fragments, hi and lo)
         + 2ll * DK * ck_pad(C)  // K_d^T (A fragments)
         + 4ll * C * ck_pad(C)   // P     (A fragments, hi and lo)
         + 4ll * C * DV;         // U~    (fp32 accumulator fragments)
}

// Target size of one window's operand blocks.  One sequence: as large as
// still stays in the 256 MiB Infinity Cache between the kernel that writes
// them and the one that reads them (the other traffic of a step passes it
// by: inputs are read and outputs written non-temporally); at 128/128/64 and
// 32 value heads that is 64 chunk slots, 230 MB, four rounds of prep
// work-groups.  A batch of several sequences uses the same size: the
// sequences whose chunks share a window run concurrently, and keeping the
// blocks cached outweighs the serialisation at window boundaries.
constexpr int64_t kPrefillWindowBytes = 240ll << 20;

// Chunk slots per window for a layer: as many as the target size allows.
// When that takes several windows and holds at least one round of prep
// work-groups over the compute units (one per value-head pair, or per value
// head when a key head has an odd number of them, per chunk slot), the
// window is cut to whole rounds: a window of 2.5 rounds costs as much prep
// time as one of 3.  Otherwise the slots are evened out over the windows.
inline int64_t prefill_window_slots(int DK, int DV, int C, int Hk, int Hv, int N, int64_t max_chunks,
                                    int compute_units) {
    const int64_t slot = static_cast<int64_t>(Hv) * vch_bytes(DK, DV, C);
    int64_t w = kPrefillWindowBytes / slot;
    const int64_t cap = max_chunks > 1 ? max_chunks : 1;
    w = w < 1 ? 1 : (w > cap ? cap : w);
    const int G = Hk > 0 ? Hv / Hk : 1;
    const int64_t per_slot = G % 2 == 0 ? Hv / 2 : Hv;             // prep work-groups per slot
    const int64_t round = compute_units / (per_slot > 0 ? per_slot : 1);
    if (w < cap && round >= 1 && w >= round) return w / round * round;
    const int64_t nwin = (cap + w - 1) / w;
    return (cap + nwin - 1) / nwin;
}

// Compute units of the current device (256 where there is none).
int compute_units();

// Kernel launches of one prefill: (prep, scan) per window, epi.
inline int64_t prefill_launches(int64_t max_chunks, int64_t win_slots) {
    const int64_t nwin = max_chunks > win_slots ? (max_chunks + win_slots - 1) / win_slots : 1;
    return 1 + 2 * nwin;
}

hipError_t launch_decode(int DK, int DV, bool bf16, const DecodeParams& p, hipStream_t s,
                         bool* supported);
// events: NULL, or prefill_launches() + 1 events: one before the first
// kernel and one after each
hipError_t launch_prefill(int DK, int DV, int C, bool bf16, const PrefillParams& p,
                          hipStream_t s, bool* supported, hipEvent_t const* events);
bool prefill_shape_supported(int DK, int DV, int C);
bool decode_shape_supported(int DK, int DV);
hipError_t launch_selftest_mfma(const float* A, const float* B, float* C, hipStream_t s);
// Which GEMM kernel family computes a product.  Each family sums every
// output element in an order that depends on K (and, for the few-row one,
// on N) but never on M, so a row's bits are independent of the other rows
// as long as the family is fixed:
//   kGemmAuto        up to 64 rows kGemmLibraryFew, else kGemmLibrary
//   kGemmTiled       always this library's tiled kernel
//   kGemmSkinny      always this library's few-row kernel, over 64-row
//                    blocks
//   kGemmLibrary     hipBLASLt with one algorithm per shape, chosen at 4096
//                    rows and used at every M (the layer's prefill
//                    projections), N past a multiple of 256 as two
//                    products (the full 256-column blocks, the rest); the
//                    tiled kernel where the library declines (no handle,
//                    no algorithm for the shape)
//   kGemmLibraryFew  the same with the algorithm chosen at 64 rows (the
//                    layer's decode projections, at any batch size); the
//                    few-row kernel where the library declines
// The values are those of GDN_GEMM_* in gdn.h.
enum GemmPath { kGemmAuto = 0, kGemmTiled = 1, kGemmSkinny = 2, kGemmLibrary = 3, kGemmLibraryFew = 4 };

// The library path (gdn_blaslt.hip) with its algorithm chosen at pin_rows
// rows: true when the product was enqueued (*err the launch status), false
// when the library declines it.
bool gemm_library(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                  bool out_bf16, int64_t M, int64_t N, int64_t K, int64_t pin_rows, hipStream_t s,
                  hipError_t* err);

// C[M][N] = A[M][K] B[N][K]^T, bf16 in, fp32 accumulation, bf16 or fp32 out
hipError_t launch_gemm_bf16_nt(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                               int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K,
                               hipStream_t s, GemmPath path = kGemmAuto);

}  // namespace gdn
