// gdn_device.hpp -- device helpers shared by the gfx950 Gated DeltaNet kernels.
//
// Matrix-core fragments (one wave of 64 lanes):
//   v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x32_f16
//     A operand, 16 rows x 32 k:  lane l holds row (l % 16), k = 8*(l/16) + e,
//                                 e = 0..7 (eight 16-bit values, 16 bytes)
//     B operand, 32 k x 16 cols:  lane l holds col (l % 16), k = 8*(l/16) + e
//   v_mfma_f32_16x16x16_bf16: the same with k = 4*(l/16) + e, e = 0..3
//     (four bf16, 8 bytes), so its B operand is laid out like C/D below
//   C/D,        16 x 16 fp32:     lane l holds col (l % 16), rows 4*(l/16) + i,
//                                 i = 0..3
// gdn_selftest_mfma checks these layouts on the device.
//
// Two product precisions, both with fp32 accumulation:
//  * split bf16 (inside a chunk): x = hi + lo with hi = bf16(x) and
//    lo = bf16(x - hi), and a*b ~= a_hi*b_hi + a_hi*b_lo + a_lo*b_hi (Henry,
//    Tang, Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype
//    For Higher-Precision Computations", ARITH 2019).  The dropped a_lo*b_lo
//    term and the rounding of lo leave ~2^-16 relative error per product,
//    against 2^-8 for a single bf16 rounding.
//  * single fp16 (between chunks, in the scan): both operands rounded once to
//    fp16 (2^-11 relative), one product.  The rounding does not compound
//    along the sequence: the state itself stays in fp32 accumulators and
//    only its operand copy is rounded, afresh at every chunk.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- scalar conversions ---------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 <-> fp16 bits, round to nearest even (v_cvt_f16_f32)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Split x into hi + lo, both bf16 bit patterns: hi = bf16(x), lo = bf16(x - hi)
// (x - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The same for a pair (a in the low half-words, b in the high ones): one
// packed conversion per word, six instructions per pair.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const f32x2 v = {a, b};
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 h = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - h, bf16x2));
}

// Two floats to packed fp16, round to nearest even (v_cvt_pk_f16_f32); a in
// the low half-word.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ uint2 pack4_f16(f32x4 x) {
    return uint2{pack_f16(x[0], x[1]), pack_f16(x[2], x[3])};
}

// Four floats as fp16 hi = fp16(x) and lo = fp16(x - hi) (x - hi is exact
// in fp32 for |x| in the fp16 normal range).
__device__ __forceinline__ void split4_f16(f32x4 x, uint2& hi, uint2& lo) {
    hi = pack4_f16(x);
    const f16x2 h0 = __builtin_bit_cast(f16x2, hi.x), h1 = __builtin_bit_cast(f16x2, hi.y);
    const f32x4 r = {x[0] - static_cast<float>(h0[0]), x[1] - static_cast<float>(h0[1]),
                     x[2] - static_cast<float>(h1[0]), x[3] - static_cast<float>(h1[1])};
    lo = pack4_f16(r);
}

__device__ __forceinline__ u32x4 pack8_f16(const float* x) {
    return u32x4{pack_f16(x[0], x[1]), pack_f16(x[2], x[3]), pack_f16(x[4], x[5]),
                 pack_f16(x[6], x[7])};
}

// e^x for x <= 0 through the hardware 2^x (v_exp_f32); relative error about
// |x| * 2^-24 + 2 ulp, used for in-chunk decay factors only.
__device__ __forceinline__ float exp_neg(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

template <bool BF16>
struct Act;
template <>
struct Act<true> {
    using T = uint16_t;
    __device__ __forceinline__ static float load(const T* p) { return bf16_bits_to_f32(*p); }
    __device__ __forceinline__ static T from_f32(float x) { return f32_to_bf16_bits(x); }
};
template <>
struct Act<false> {
    using T = float;
    __device__ __forceinline__ static float load(const T* p) { return *p; }
    __device__ __forceinline__ static T from_f32(float x) { return x; }
};

// ---- elementwise math (ROCm device libm) ------------------------------------

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

__device__ __forceinline__ float softplus(float x) {
    return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// SiLU on the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32, each about
// 1 ulp): a few ulp of relative error, used on the prefill path where it is
// evaluated for every conv output.  x -> -inf gives -0.
__device__ __forceinline__ float silu_fast(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// ---- matrix-core product ---------------------------------------------------

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// acc += a * b on fp16 fragments (eight fp16 per 16-byte register).
__device__ __forceinline__ f32x4 mfma_h(u32x4 a, u32x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

// The same on fp16 hi + lo fragments (16x16x32 f16).
__device__ __forceinline__ f32x4 mfma_h3(u32x4 ahi, u32x4 alo, u32x4 bhi, u32x4 blo, f32x4 acc) {
    acc = mfma_h(alo, bhi, acc);
    acc = mfma_h(ahi, blo, acc);
    return mfma_h(ahi, bhi, acc);
}

// acc += (a_hi + a_lo) * (b_hi + b_lo) without the lo*lo term.
__device__ __forceinline__ f32x4 mfma3(u32x4 ahi, u32x4 alo, u32x4 bhi, u32x4 blo,
                                        f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo), as_bf16x8(bhi), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi), as_bf16x8(blo), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi), as_bf16x8(bhi), acc, 0, 0, 0);
    return acc;
}

// acc += (a_hi + a_lo) * (b_hi + b_lo) without the lo*lo term, on the
// 16x16x16 shape (a, b: two dwords = four bf16 each).
__device__ __forceinline__ f32x4 mfma3_k16(uint2 ahi, uint2 alo, uint2 bhi, uint2 blo, f32x4 acc) {
    const s16x4 ah = __builtin_bit_cast(s16x4, ahi), al = __builtin_bit_cast(s16x4, alo);
    const s16x4 bh = __builtin_bit_cast(s16x4, bhi), bl = __builtin_bit_cast(s16x4, blo);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    return acc;
}

// Split four floats into packed bf16 hi and lo words (element e in bits
// 16*(e%2) of word e/2).
__device__ __forceinline__ void split4(f32x4 x, uint2& hi, uint2& lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
}

// Pack 8 bf16 bit patterns (e = 0..7) into one 16-byte fragment register.
__device__ __forceinline__ u32x4 pack8(const uint16_t* h) {
    u32x4 r;
    r[0] = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
    r[1] = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
    r[2] = static_cast<uint32_t>(h[4]) | (static_cast<uint32_t>(h[5]) << 16);
    r[3] = static_cast<uint32_t>(h[6]) | (static_cast<uint32_t>(h[7]) << 16);
    return r;
}

// Lane swap of a float inside a row of 16 lanes by a DPP control word.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N = 4, 8 or 16 lanes on DPP lane swaps inside a
// row of 16 (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror): one VALU op per step instead of an LDS permute.  Every lane
// of a group ends with the same bits: at each step the two partners add the
// same two values, and fp32 addition is commutative.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    x += dpp_f32<0xB1>(x);                           // quad_perm [1,0,3,2]
    x += dpp_f32<0x4E>(x);                           // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_f32<0x141>(x);    // row_half_mirror
    if constexpr (N >= 16) x += dpp_f32<0x140>(x);   // row_mirror
    return x;
}

// A value every lane of the wave holds with the same bits, moved to a
// scalar register
__device__ __forceinline__ float uniform_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// A pointer every lane of the wave holds, as a wave-uniform integer
template <typename P>
__device__ __forceinline__ uintptr_t uniform_ptr(const P* ptr) {
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sets bit 0 of *status when any lane of the wave passes `bad` (one atomic
// per wave, from its lowest such lane)
__device__ __forceinline__ void flag_nonfinite(int32_t* status, bool bad) {
    const uint64_t m = __ballot(bad);
    if (status && m && (__lane_id() == static_cast<unsigned>(__builtin_ctzll(m))))
        __hip_atomic_fetch_or(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0): every vector memory access this wave has issued,
// loads and stores alike, has completed (gfx9 encoding: expcnt and lgkmcnt
// left at their maxima)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Deterministic wave-wide sum: rows of 16 on DPP swaps, then the four rows
// through two xor permutes; every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float x) {
    x = group_sum<16>(x);
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

}  // namespace gdn
