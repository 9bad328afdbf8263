// gdn_prep.hpp -- chunk-parallel operand kernel of the chunked prefill.
//
// One work-group (512 threads, 8 waves) per (chunk slot, value head h).  For
// the chunk's C tokens it computes, entirely on chip:
//   q^, k^  conv1d(K=4) + SiLU + L2 norm of key head h/G (row items of 8
//           channels: 16-byte loads, norms reduced across the lanes of a row)
//   v^      conv1d + SiLU of value head h
//   g, beta the gates; gamma = in-chunk inclusive cumsum of g
//   G_kk = K^K^T, G_qk = Q^K^T         split-bf16 MFMA, lower tiles only
//   A  = strict_tril(beta_r e^{gamma_r - gamma_s} G_kk)
//   Tm = (I + A)^{-1}                   16x16 diagonal blocks by substitution,
//                                       off-diagonal blocks by the block
//                                       recursion T_ij = -T_ii sum_k A_ik T_kj
//   [W | U~] = Tm diag(beta) [diag(e^gamma) K^ | V^]     split-bf16 MFMA
// and writes the scan's operands in MFMA fragment order: -W, Q_G =
// diag(e^gamma) Q^, K_d^T = (diag(e^{gamma_last - gamma}) K^)^T,
// P = tril_incl(G_qk (.) e^{gamma_r - gamma_s}) and U~, plus e^{gamma_last}.
// (Chunk form of Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025,
// on the UT transform of Yang et al., NeurIPS 2024.)
#pragma once
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

template <int DK, int DV, int C>
struct PrepSmem {
    static constexpr int CK = ck_pad(C);
    static constexpr int SQ = DK + 8;    // bf16 row stride of Q^, K^, W staging [C][SQ]
    static constexpr int ST = CK + 8;    // bf16 row stride of K^T, V^T [*][ST] and Tp [C][ST]
    static constexpr int SG = C + 4;     // fp32 row stride of G_kk, G_qk, Tm [C][SG]
    static constexpr int qk_bytes = C * SQ * 4;     // hi + lo
    static constexpr int kt_bytes = DK * ST * 4;
    static constexpr int vt_bytes = DV * ST * 4;
    static constexpr int g_bytes = 2 * C * SG * 4;
    static constexpr int tp_bytes = C * ST * 4;
    static constexpr int tm_bytes = C * SG * 4;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int oQ = 0;                              // Q^ -> K^T (Gamma-scaled)
    static constexpr int oK = oQ + cmax(qk_bytes, kt_bytes);  // K^ -> W staging
    static constexpr int oV = oK + qk_bytes;                  // V^T
    static constexpr int oG = oV + vt_bytes;                  // G_kk (-> A), G_qk -> Tp
    static constexpr int oT = oG + cmax(g_bytes, tp_bytes);   // Tm
    static constexpr int oS = oT + tm_bytes;                  // per-token gate vectors
    static constexpr int total = oS + 5 * C * 4;
};

// Eight consecutive activation elements starting at element `off` of `base`
// (16-byte aligned for bf16, 32-byte aligned for fp32 rows of 8).
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* x) {
    if constexpr (BF16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(v[e] << 16);
            x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
    }
}

// Raw input rows of one conv item: 8 channels [c0, c0+8) for the 7 token
// positions r0-3 .. r0+3 of a chunk (chunk rows at or past `valid` and
// history before the first conv-state row read as zeros).
template <bool BF16>
struct RawRows {
    u32x4 r[7][BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void load_rows(const PrefillParams& p, int n, int64_t start, int64_t t0,
                                          int r0, int valid, const void* src, int64_t rs, int col,
                                          int c0, int Cc, RawRows<BF16>& raw) {
    constexpr int W = BF16 ? 1 : 2;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const int rr = r0 - 3 + j;
        const int64_t pp = t0 + rr;
        const void* base = nullptr;
        int64_t off = 0;
        if (rr < valid && pp >= start) {
            base = src;
            off = pp * rs + col;
        } else if (rr < valid && p.conv_in && pp - start >= -3) {
            base = p.conv_in;
            off = (static_cast<int64_t>(n) * 3 + 3 + (pp - start)) * Cc + c0;
        }
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (base) {
                const u32x4* q = BF16 ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off)
                                      : reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + off);
                raw.r[j][w] = q[w];
            } else {
                raw.r[j][w] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void row8(const RawRows<BF16>& raw, int j, float* x) {
    if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(raw.r[j][0][e] << 16);
            x[2 * e + 1] = __uint_as_float(raw.r[j][0][e] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(raw.r[j][0][e]);
            x[4 + e] = __uint_as_float(raw.r[j][1][e]);
        }
    }
}

// conv1d(K=4) + SiLU of the item's 8 channels at its 4 tokens; tokens at or
// past `valid` give zeros.
template <bool BF16>
__device__ __forceinline__ void conv_rows(const RawRows<BF16>& raw, const f32x4* w, int r0,
                                          int valid, float (*y)[8]) {
    float x[7][8];
#pragma unroll
    for (int j = 0; j < 7; ++j) row8<BF16>(raw, j, x[j]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = w[e][0] * x[t][e];
            acc = fmaf(w[e][1], x[t + 1][e], acc);
            acc = fmaf(w[e][2], x[t + 2][e], acc);
            acc = fmaf(w[e][3], x[t + 3][e], acc);
            y[t][e] = (r0 + t < valid) ? silu_fast(acc) : 0.f;
        }
    }
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void unpack8(u32x4 hi, u32x4 lo, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(hi[e] << 16) + __uint_as_float(lo[e] << 16);
        x[2 * e + 1] = __uint_as_float(hi[e] & 0xFFFF0000u) + __uint_as_float(lo[e] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16(x[e], h[e], l[e]);
    hi = pack8(h);
    lo = pack8(l);
}

__device__ __forceinline__ void store_frag(uint8_t* tile, int lane, u32x4 hi, u32x4 lo) {
    *reinterpret_cast<u32x4*>(tile + lane * 16) = hi;
    *reinterpret_cast<u32x4*>(tile + 1024 + lane * 16) = lo;
}

// bf16 element of a split pair back to fp32
__device__ __forceinline__ float hl(const uint16_t* h, const uint16_t* l, int i) {
    return bf16_bits_to_f32(h[i]) + bf16_bits_to_f32(l[i]);
}

constexpr int kPrepThreads = 512;     // 8 waves: two per SIMD share the 160 KiB LDS

template <int DK, int DV, int C, bool BF16>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrefillParams p) {
    using S = PrepSmem<DK, DV, C>;
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = S::CK, SQ = S::SQ, ST = S::ST, SG = S::SG;
    constexpr int NB = C / 16;           // 16-token blocks in a chunk
    constexpr int NT = kPrepThreads;
    constexpr int NW = NT / kWave;
    static_assert(C % 16 == 0 && DK % 32 == 0 && DV % 16 == 0 && DK <= 128, "shape");
    static_assert(S::total <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint8_t smem[S::total];
    uint16_t* sQh = reinterpret_cast<uint16_t*>(smem + S::oQ);
    uint16_t* sQl = sQh + C * SQ;
    uint16_t* sKTh = reinterpret_cast<uint16_t*>(smem + S::oQ);
    uint16_t* sKTl = sKTh + DK * ST;
    uint16_t* sKh = reinterpret_cast<uint16_t*>(smem + S::oK);
    uint16_t* sKl = sKh + C * SQ;
    uint16_t* sVTh = reinterpret_cast<uint16_t*>(smem + S::oV);
    uint16_t* sVTl = sVTh + DV * ST;
    float* sGkk = reinterpret_cast<float*>(smem + S::oG);
    float* sGqk = sGkk + C * SG;
    uint16_t* sTph = reinterpret_cast<uint16_t*>(smem + S::oG);
    uint16_t* sTpl = sTph + C * ST;
    float* sTm = reinterpret_cast<float*>(smem + S::oT);
    float* sg = reinterpret_cast<float*>(smem + S::oS);
    float* sbeta = sg + C;
    float* sgam = sbeta + C;
    float* sE = sgam + C;       // e^{gamma_r}
    float* sD = sE + C;         // e^{gamma_last - gamma_r}

    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    const int hk = h / p.G;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int total = p.chunk_off[p.N];
    if (slot >= total) return;
    const int n = seq_of_chunk(p.chunk_off, p.N, slot);
    const int64_t start = p.cu[n], end = p.cu[n + 1];
    const int64_t t0 = start + static_cast<int64_t>(slot - p.chunk_off[n]) * C;
    const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
    const int qk = p.Hk * DK;
    const int Cc = 2 * qk + p.Hv * DV;
    uint8_t* blk = p.vch + (static_cast<int64_t>(slot) * p.Hv + h) * L::bytes;

    // ---- 1. conv inputs, then conv + SiLU (+ L2 norm for q, k) ----
    // An item is 4 tokens x 8 channels.  Each thread owns at most one q/k
    // item and one v item and issues all of its loads (both items' 7 input
    // rows, their conv weights, the gate inputs) before any arithmetic, so
    // the chunk's inputs cost one memory round trip.
    static_assert(C % 4 == 0, "row groups");
    {
        constexpr int GPRK = DK / 8, GPRV = DV / 8;        // lanes per token row
        constexpr int IQK = 2 * (C / 4) * GPRK, IV = (C / 4) * GPRV;
        static_assert(IQK <= NT && IV <= NT && kWave % GPRK == 0, "one item of a kind per thread");
        const bool has_qk = tid < IQK, has_v = tid < IV;
        const int qtensor = tid / ((C / 4) * GPRK);
        const int qrem = tid % ((C / 4) * GPRK);
        const int qgrp = qrem % GPRK, qr0 = (qrem / GPRK) * 4;
        const int vgrp = tid % GPRV, vr0 = (tid / GPRV) * 4;
        const int qc0 = qtensor * qk + hk * DK + qgrp * 8;
        const int vc0 = 2 * qk + h * DV + vgrp * 8;
        RawRows<BF16> rq, rv;
        f32x4 wq[8], wv[8];
        float av = 0.f, bv = 0.f;
        if (has_qk)
            load_rows<BF16>(p, n, start, t0, qr0, Lc, qtensor ? p.k : p.q, qtensor ? p.ks : p.qs,
                            hk * DK + qgrp * 8, qc0, Cc, rq);
        if (has_v)
            load_rows<BF16>(p, n, start, t0, vr0, Lc, p.v, p.vs, h * DV + vgrp * 8, vc0, Cc, rv);
        if (tid < Lc) {
            using A = Act<BF16>;
            using T = typename A::T;
            av = A::load(static_cast<const T*>(p.a) + (t0 + tid) * p.as + h);
            bv = A::load(static_cast<const T*>(p.b) + (t0 + tid) * p.bs + h);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (has_qk) wq[e] = *reinterpret_cast<const f32x4*>(p.conv_w + (qc0 + e) * 4);
            if (has_v) wv[e] = *reinterpret_cast<const f32x4*>(p.conv_w + (vc0 + e) * 4);
        }
        if (has_qk) {
            float y[4][8];
            conv_rows<BF16>(rq, wq, qr0, Lc, y);
            uint16_t* dh = qtensor ? sKh : sQh;
            uint16_t* dl = qtensor ? sKl : sQl;
            const float sc = qtensor ? 1.0f : p.scale;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[t][e], y[t][e], ss);
#pragma unroll
                for (int off = GPRK / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
                const float f = sc / sqrtf(ss + p.eps_l2);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[t][e] *= f;
                u32x4 hi, lo;
                split8(y[t], hi, lo);
                *reinterpret_cast<u32x4*>(dh + (qr0 + t) * SQ + qgrp * 8) = hi;
                *reinterpret_cast<u32x4*>(dl + (qr0 + t) * SQ + qgrp * 8) = lo;
            }
        }
        if (has_v) {
            float y[4][8];
            conv_rows<BF16>(rv, wv, vr0, Lc, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) split_bf16(y[t][e], hi[t], lo[t]);
                const int off = (vgrp * 8 + e) * ST + vr0;
                *reinterpret_cast<uint2*>(sVTh + off) =
                    make_uint2(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16));
                *reinterpret_cast<uint2*>(sVTl + off) =
                    make_uint2(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16));
            }
        }
        if constexpr (CK > C) {
            for (int i = tid; i < DV * (CK - C); i += NT) {
                const int j = i / (CK - C), s = C + i % (CK - C);
                sVTh[j * ST + s] = 0;
                sVTl[j * ST + s] = 0;
            }
        }
        // ---- gates ----
        if (tid < C) {
            float g = 0.f, beta = 0.f;
            if (tid < Lc) {
                g = -expf(p.A_log[h]) * softplus(av + p.dt_bias[h]);
                beta = sigmoid(bv);
            }
            sg[tid] = g;
            sbeta[tid] = beta;
        }
    }
    __syncthreads();
    if (wave == 0) {
        // inclusive prefix sum over the chunk (Hillis-Steele, fixed order)
        float v = lane < C ? sg[lane] : 0.f;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float u = __shfl_up(v, off, kWave);
            if (lane >= off) v += u;
        }
        const float glast = __shfl(v, C - 1, kWave);
        if (lane < C) {
            sgam[lane] = v;
            sE[lane] = exp_neg(v);
            sD[lane] = exp_neg(glast - v);
        }
        if (lane == 0) p.decay[static_cast<int64_t>(slot) * p.Hv + h] = expf(glast);
    }

    // ---- 2. Gram matrices on the matrix cores (lower tiles) ----
    {
        constexpr int NTI = NB * (NB + 1) / 2;
        for (int job = wave; job < 2 * NTI; job += NW) {
            const int which = job / NTI;          // 0: K K^T, 1: Q K^T
            int idx = job % NTI, mt = 0;
            while (idx > mt) { idx -= mt + 1; ++mt; }
            const int nt = idx;
            const uint16_t* ah = which ? sQh : sKh;
            const uint16_t* al = which ? sQl : sKl;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < DK / 32; ++kt) {
                const int ao = (mt * 16 + l16) * SQ + kt * 32 + lq * 8;
                const int bo = (nt * 16 + l16) * SQ + kt * 32 + lq * 8;
                acc = mfma3(lds16(ah + ao), lds16(al + ao), lds16(sKh + bo), lds16(sKl + bo), acc);
            }
            float* G = which ? sGqk : sGkk;
#pragma unroll
            for (int i = 0; i < 4; ++i) G[(mt * 16 + lq * 4 + i) * SG + nt * 16 + l16] = acc[i];
        }
    }
    __syncthreads();

    // ---- 3. Q_G, K_d^T, P fragments; A in place of G_kk ----
    for (int sl = tid; sl < C * DK / 8; sl += NT) {           // Q_G [C][DK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (DK / 32), kt = tile % (DK / 32);
        const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
        float x[8];
        unpack8(lds16(sQh + r * SQ + c0), lds16(sQl + r * SQ + c0), x);
        const float e = sE[r];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= e;
        u32x4 hi, lo;
        split8(x, hi, lo);
        store_frag(blk + L::QG + tile * 2048, ln, hi, lo);
    }
    for (int sl = tid; sl < DK * CK / 8; sl += NT) {          // K_d^T [DK][CK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int i = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = s < C ? sD[s] * hl(sKh, sKl, s * SQ + i) : 0.f;
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        store_frag(blk + L::KdT + tile * 2048, ln, hi, lo);
    }
    for (int sl = tid; sl < C * CK / 8; sl += NT) {           // P [C][CK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int r = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = (s <= r && s < C) ? sGqk[r * SG + s] * exp_neg(sgam[r] - sgam[s]) : 0.f;
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        store_frag(blk + L::P + tile * 2048, ln, hi, lo);
    }
    for (int idx = tid; idx < C * C; idx += NT) {             // A, strict lower
        const int r = idx / C, s = idx % C;
        sGkk[r * SG + s] = (s < r) ? sbeta[r] * exp_neg(sgam[r] - sgam[s]) * sGkk[r * SG + s] : 0.f;
    }
    __syncthreads();

    // ---- 4. K^T scaled by e^gamma (over Q^), Tm diagonal blocks ----
    for (int idx = tid; idx < DK * (CK / 8); idx += NT) {
        const int i = idx / (CK / 8), s0 = (idx % (CK / 8)) * 8;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = s < C ? sE[s] * hl(sKh, sKl, s * SQ + i) : 0.f;
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<u32x4*>(sKTh + i * ST + s0) = hi;
        *reinterpret_cast<u32x4*>(sKTl + i * ST + s0) = lo;
    }
    if (wave == 0 && lq < NB) {
        // lane (block lq, column l16): x_r = delta_rc - sum_{s<r} A_rs x_s;
        // row r+1 of the block is read while row r is computed
        const int b0 = lq * 16;
        float x[16];
        f32x4 arow[4], anext[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) arow[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (r + 1 < 16) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    anext[q] = *reinterpret_cast<const f32x4*>(sGkk + (b0 + r + 1) * SG + b0 + 4 * q);
            }
            float acc = (r == l16) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc = fmaf(-arow[s / 4][s % 4], x[s], acc);
            x[r] = acc;
#pragma unroll
            for (int q = 0; q < 4; ++q) arow[q] = anext[q];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sTm[(b0 + r) * SG + b0 + l16] = x[r];
    }
    __syncthreads();
    // ---- 5. Tm off-diagonal blocks, by distance d from the diagonal ----
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        // M_ij = sum_{k=j}^{i-1} A_ik T_kj, parked in the unused upper block (j, i)
        for (int e = tid; e < (NB - d) * 256; e += NT) {
            const int j = e / 256, i = j + d, rr = (e % 256) / 16, cc = e % 16;
            float acc = 0.f;
            for (int k = j; k < i; ++k)
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc = fmaf(sGkk[(16 * i + rr) * SG + 16 * k + s], sTm[(16 * k + s) * SG + 16 * j + cc], acc);
            sTm[(16 * j + rr) * SG + 16 * i + cc] = acc;
        }
        __syncthreads();
        // T_ij = -T_ii M_ij
        for (int e = tid; e < (NB - d) * 256; e += NT) {
            const int j = e / 256, i = j + d, rr = (e % 256) / 16, cc = e % 16;
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s)
                acc = fmaf(sTm[(16 * i + rr) * SG + 16 * i + s], sTm[(16 * j + s) * SG + 16 * i + cc], acc);
            sTm[(16 * i + rr) * SG + 16 * j + cc] = -acc;
        }
        __syncthreads();
    }
    // ---- 6. Tp = Tm diag(beta) (lower, zero padded), split, over G ----
    for (int idx = tid; idx < C * (CK / 8); idx += NT) {
        const int r = idx / (CK / 8), s0 = (idx % (CK / 8)) * 8;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = (s <= r && s < C) ? sTm[r * SG + s] * sbeta[s] : 0.f;
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<u32x4*>(sTph + r * ST + s0) = hi;
        *reinterpret_cast<u32x4*>(sTpl + r * ST + s0) = lo;
    }
    __syncthreads();

    // ---- 7. [W | U~] = Tp [e^gamma K^ | V^] on the matrix cores ----
    constexpr int NTW = DK / 16, NTU = DV / 16, NTT = NTW + NTU;
    constexpr int JOBS = NB * NTT;
    constexpr int JPW = (JOBS + NW - 1) / NW;
    f32x4 wres[JPW];
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
        const int job = wave + NW * q;
        if (job >= JOBS) continue;
        const int mt = job / NTT, nt = job % NTT;
        const bool isw = nt < NTW;
        const uint16_t* bh = isw ? sKTh + (nt * 16 + l16) * ST : sVTh + ((nt - NTW) * 16 + l16) * ST;
        const uint16_t* bl = isw ? sKTl + (nt * 16 + l16) * ST : sVTl + ((nt - NTW) * 16 + l16) * ST;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < CK / 32; ++kt) {
            const int ao = (mt * 16 + l16) * ST + kt * 32 + lq * 8;
            acc = mfma3(lds16(sTph + ao), lds16(sTpl + ao), lds16(bh + kt * 32 + lq * 8),
                        lds16(bl + kt * 32 + lq * 8), acc);
        }
        if (isw) {
            wres[q] = acc;
        } else {
            const int tile = mt * NTU + (nt - NTW);
            *reinterpret_cast<f32x4*>(blk + L::Ut + tile * 1024 + lane * 16) = acc;
        }
    }
    __syncthreads();
    // ---- 8. stage -W (split) over K^, then copy out as A fragments ----
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
        const int job = wave + NW * q;
        if (job >= JOBS) continue;
        const int mt = job / NTT, nt = job % NTT;
        if (nt >= NTW) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t hi, lo;
            split_bf16(-wres[q][i], hi, lo);
            const int off = (mt * 16 + lq * 4 + i) * SQ + nt * 16 + l16;
            sKh[off] = hi;
            sKl[off] = lo;
        }
    }
    __syncthreads();
    for (int sl = tid; sl < C * DK / 8; sl += NT) {
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (DK / 32), kt = tile % (DK / 32);
        const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
        store_frag(blk + L::negW + tile * 2048, ln, lds16(sKh + r * SQ + c0), lds16(sKl + r * SQ + c0));
    }
}

}  // namespace gdn
