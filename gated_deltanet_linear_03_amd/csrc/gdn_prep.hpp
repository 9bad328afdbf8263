// gdn_prep.hpp -- chunk-parallel operand kernel of the chunked prefill.
//
// One work-group (1024 threads, 16 waves) per (chunk slot, value head h) of
// a window of chunk slots.
// For the chunk's C tokens it computes, entirely on chip:
//   q^, k^  conv1d(K=4) + SiLU + L2 norm of key head h/G (items of 4 tokens x
//           8 channels: 16-byte loads, norms reduced across a row's lanes)
//   v^      conv1d + SiLU of value head h
//   g, beta the gates; gamma = in-chunk inclusive cumsum of g
//   A  = strict_tril(beta_r e^{gamma_r - gamma_s} K^K^T)   split-bf16 MFMA
//   P  = tril_incl(e^{gamma_r - gamma_s} Q^K^T)            (lower tiles only)
//   T_bb = 16x16 diagonal blocks of Tm = (I + A)^{-1}, by substitution
//   [W | U~] = Tm [diag(beta e^gamma) K^ | diag(beta) V^] by block forward
//           substitution X_i = T_ii (B_i - sum_{j<i} A_ij X_j) over the
//           16-token blocks, split-bf16 MFMA
// and writes the scan's operands in MFMA fragment order: -W, Q_G =
// diag(e^gamma) Q^, K_d^T = (diag(e^{gamma_last - gamma}) K^)^T and P as
// fp16, U~ as fp32, plus e^{gamma_last}.  (Chunk form of Yang, Kautz, Hatamizadeh, "Gated Delta
// Networks", ICLR 2025, on the UT transform of Yang et al., NeurIPS 2024.)
#pragma once
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

template <int DK, int DV, int C>
struct PrepSmem {
    static constexpr int CK = ck_pad(C);
    static constexpr int NB = C / 16;
    static constexpr int SQ = DK + 8;    // bf16 row stride of Q^, K^ and the W staging [C][SQ]
    static constexpr int SV = DV + 8;    // fp32 row stride of V^ [C][SV]
    static constexpr int SG = C + 4;     // fp32 row stride of P [C][SG]
    static constexpr int SA = C + 8;     // bf16 row stride of -A below the diagonal blocks [C][SA]
    static constexpr int SD = 20;        // fp32 row stride of A's diagonal blocks [NB][16][SD]
    static constexpr int STT = 24;       // bf16 row stride of the blocks T_bb [NB][16][STT]
    static constexpr int qk_bytes = C * SQ * 4;     // hi + lo
    static constexpr int v_bytes = C * SV * 4;
    static constexpr int ad_bytes = NB * 16 * SD * 4;
    static constexpr int a_bytes = C * SA * 4;
    static constexpr int p_bytes = C * SG * 4;
    static constexpr int w_bytes = (2 * DK + DV) * 16;
    static constexpr int tt_bytes = NB * 16 * STT * 4;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int oQ = 0;                                   // Q^ -> -W staging
    static constexpr int oK = oQ + qk_bytes;                       // K^
    static constexpr int oV = oK + qk_bytes;                       // V^
    static constexpr int oG = oV + v_bytes;                        // conv weights -> A blocks, -A, P
    static constexpr int oT = oG + cmax(ad_bytes + a_bytes + p_bytes, w_bytes);   // T_bb
    static constexpr int oS = oT + tt_bytes;                       // per-token gate vectors
    static constexpr int total = oS + 4 * C * 4;
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
// history before the first conv-state row read as zeros); history before the
// sequence start comes from conv-state entry `slot`.
template <bool BF16>
struct RawRows {
    u32x4 r[7][BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void load_rows(const PrefillParams& p, int slot, int64_t start, int64_t t0,
                                          int r0, int valid, const void* src, int64_t rs, int col,
                                          int c0, int Cc, RawRows<BF16>& raw) {
    using T = typename Act<BF16>::T;
    constexpr int W = BF16 ? 1 : 2;
    const T* row = static_cast<const T*>(src) + (t0 + r0 - 3) * rs + col;   // row j at row + j rs
    const int hist = static_cast<int>(min(t0 - start, static_cast<int64_t>(3)));  // sequence rows before the chunk, up to 3
    if (r0 - 3 + hist >= 0 && r0 + 3 < valid) {
        // the common case: all seven rows inside the chunk's sequence rows
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            const u32x4* q = reinterpret_cast<const u32x4*>(row + j * rs);
#pragma unroll
            for (int w = 0; w < W; ++w) raw.r[j][w] = q[w];
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const int rr = r0 - 3 + j;
        const u32x4* q = nullptr;
        if (rr < valid && rr + hist >= 0) {
            q = reinterpret_cast<const u32x4*>(row + j * rs);
        } else if (rr < valid && p.conv_in && rr + hist >= -3) {
            q = reinterpret_cast<const u32x4*>(static_cast<const T*>(p.conv_in) +
                                               (static_cast<int64_t>(slot) * 3 + 3 + rr + hist) * Cc + c0);
        }
#pragma unroll
        for (int w = 0; w < W; ++w) raw.r[j][w] = q ? q[w] : u32x4{0u, 0u, 0u, 0u};
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
            y[t][e] = silu_fast(acc);
        }
    }
    if (r0 + 4 > valid) {       // only the group that straddles the chunk's end
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (r0 + t >= valid) y[t][e] = 0.f;
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t h, l;
        split2(x[2 * e], x[2 * e + 1], h, l);
        hi[e] = h;
        lo[e] = l;
    }
}

// bf16 element of a split pair back to fp32
__device__ __forceinline__ float hl(const uint16_t* h, const uint16_t* l, int i) {
    return bf16_bits_to_f32(h[i]) + bf16_bits_to_f32(l[i]);
}

constexpr int kPrepThreads = 1024;    // 16 waves: four per SIMD share the 160 KiB LDS

template <int DK, int DV, int C, bool BF16>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrefillParams p) {
    using S = PrepSmem<DK, DV, C>;
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = S::CK, SQ = S::SQ, SV = S::SV, SG = S::SG, SA = S::SA, SD = S::SD, STT = S::STT;
    constexpr int NB = C / 16;           // 16-token blocks in a chunk
    constexpr int NT = kPrepThreads;
    constexpr int NW = NT / kWave;
    static_assert(C % 16 == 0 && C <= kWave && DK % 32 == 0 && DV % 16 == 0 && DK <= 128, "shape");
    static_assert(S::total <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint8_t smem[S::total];
    uint16_t* sQh = reinterpret_cast<uint16_t*>(smem + S::oQ);
    uint16_t* sQl = sQh + C * SQ;
    uint16_t* sW = sQh;                  // -W staging (fp16) over Q^
    uint16_t* sKh = reinterpret_cast<uint16_t*>(smem + S::oK);
    uint16_t* sKl = sKh + C * SQ;
    float* sV = reinterpret_cast<float*>(smem + S::oV);     // V^ (fp32: only a B-operand source)
    f32x4* sCw = reinterpret_cast<f32x4*>(smem + S::oG);
    float* sAd = reinterpret_cast<float*>(smem + S::oG);
    uint16_t* sAh = reinterpret_cast<uint16_t*>(smem + S::oG + S::ad_bytes);
    uint16_t* sAl = sAh + C * SA;
    float* sP = reinterpret_cast<float*>(smem + S::oG + S::ad_bytes + S::a_bytes);
    uint16_t* sTh = reinterpret_cast<uint16_t*>(smem + S::oT);
    uint16_t* sTl = sTh + NB * 16 * STT;
    float* sbeta = reinterpret_cast<float*>(smem + S::oS);
    float* sgam = sbeta + C;
    float* sE = sgam + C;       // e^{gamma_r}
    float* sD = sE + C;         // e^{gamma_last - gamma_r}

    const int slot = p.win_lo + blockIdx.x;
    const int h = blockIdx.y;
    const int hk = h / p.G;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int total = min(p.chunk_off[p.N], p.win_hi);
    if (slot >= total) return;
    const int n = seq_of_chunk(p.chunk_off, p.N, slot);
    const int64_t start = p.cu[n], end = p.cu[n + 1];
    const int64_t t0 = start + static_cast<int64_t>(slot - p.chunk_off[n]) * C;
    const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
    const int qk = p.Hk * DK;
    const int Cc = 2 * qk + p.Hv * DV;
    uint8_t* blk = p.vch + (static_cast<int64_t>(slot - p.win_lo) * p.Hv + h) * L::bytes;

    // ---- 1. conv inputs, then conv + SiLU (+ L2 norm for q, k), gates ----
    // The first NSW waves (dispatched first) stage the head's conv weights in
    // LDS (each weight is read by every token group) and wave 0 loads the
    // gate inputs; the waves after them own one item each, 4 tokens x 8
    // channels of q, k or v (q items, then k items, then v items), and issue
    // its 7 input-row loads before anything else, so the chunk's inputs cost
    // one memory round trip.  Wave 0 then computes the gates and the
    // in-chunk cumulative decay while the others run the conv.
    static_assert(C % 4 == 0, "row groups");
    constexpr int GPRK = DK / 8, GPRV = DV / 8;        // lanes per token row
    constexpr int IQ = (C / 4) * GPRK, IV = (C / 4) * GPRV;
    constexpr int NSW = 4;                              // staging waves
    // (a row's GPRK lanes are always of one kind: the norm reduces over them)
    static_assert(2 * IQ + IV <= NT - NSW * kWave && kWave % GPRK == 0, "one item per thread");
    constexpr int NCW = 2 * DK + DV;                    // staged weight rows (q | k | v)
    {
        const int ti = tid - NSW * kWave;
        const int kind = ti < 0 ? 3 : (ti < IQ ? 0 : (ti < 2 * IQ ? 1 : (ti < 2 * IQ + IV ? 2 : 3)));
        const int it = ti - (kind == 0 ? 0 : (kind == 1 ? IQ : 2 * IQ));
        const int gpr = kind == 2 ? GPRV : GPRK;
        const int grp = it % gpr, r0 = (it / gpr) * 4;
        const int col = (kind == 2 ? h * DV : hk * DK) + grp * 8;
        const int c0 = (kind == 2 ? 2 * qk : kind * qk) + col;
        const void* src = kind == 0 ? p.q : (kind == 1 ? p.k : p.v);
        const int64_t rs = kind == 0 ? p.qs : (kind == 1 ? p.ks : p.vs);
        RawRows<BF16> raw;
        float av = 0.f, bv = 0.f;
        if (wave < NSW) {
            if (wave == 0 && lane < Lc) {
                using A = Act<BF16>;
                using T = typename A::T;
                av = A::load(static_cast<const T*>(p.a) + (t0 + lane) * p.as + h);
                bv = A::load(static_cast<const T*>(p.b) + (t0 + lane) * p.bs + h);
            }
            constexpr int WPT = (NCW + NSW * kWave - 1) / (NSW * kWave);
            f32x4 wst[WPT];
#pragma unroll
            for (int u = 0; u < WPT; ++u) {         // all loads first: one round trip
                const int i = tid + u * NSW * kWave;
                const int ch = i < DK ? hk * DK + i
                             : (i < 2 * DK ? qk + hk * DK + (i - DK) : 2 * qk + h * DV + (i - 2 * DK));
                if (i < NCW) wst[u] = *reinterpret_cast<const f32x4*>(p.conv_w + ch * 4);
            }
#pragma unroll
            for (int u = 0; u < WPT; ++u) {
                const int i = tid + u * NSW * kWave;
                if (i < NCW) sCw[i] = wst[u];
            }
        } else if (kind < 3) {
            load_rows<BF16>(p, state_slot(p.slots, n), start, t0, r0, Lc, src, rs, col, c0, Cc, raw);
        }
        __syncthreads();
        if (kind < 3) {
            f32x4 w[8];
            const int wb = (kind == 0 ? 0 : (kind == 1 ? DK : 2 * DK)) + grp * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = sCw[wb + e];
            float y[4][8];
            conv_rows<BF16>(raw, w, r0, Lc, y);
            uint16_t* dh = kind == 0 ? sQh : sKh;
            uint16_t* dl = kind == 0 ? sQl : sKl;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (kind == 2) {
                    float* dv = sV + (r0 + t) * SV + grp * 8;
                    *reinterpret_cast<f32x4*>(dv) = f32x4{y[t][0], y[t][1], y[t][2], y[t][3]};
                    *reinterpret_cast<f32x4*>(dv + 4) = f32x4{y[t][4], y[t][5], y[t][6], y[t][7]};
                    continue;
                }
                if (kind < 2) {
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss = fmaf(y[t][e], y[t][e], ss);
                    ss = group_sum<GPRK>(ss);
                    const float f = (kind ? 1.0f : p.scale) * __builtin_amdgcn_rsqf(ss + p.eps_l2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[t][e] *= f;
                }
                u32x4 hi, lo;
                split8(y[t], hi, lo);
                *reinterpret_cast<u32x4*>(dh + (r0 + t) * SQ + grp * 8) = hi;
                *reinterpret_cast<u32x4*>(dl + (r0 + t) * SQ + grp * 8) = lo;
            }
        }
        if (wave == 0) {
            // gates, then the inclusive prefix sum over the chunk (Hillis-Steele,
            // fixed order); tokens past the chunk's end have g = beta = 0
            float g = 0.f, beta = 0.f;
            if (lane < Lc) {
                g = -expf(p.A_log[h]) * softplus(av + p.dt_bias[h]);
                beta = sigmoid(bv);
            }
            float v = g;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float u = __shfl_up(v, off, kWave);
                if (lane >= off) v += u;
            }
            const float glast = __shfl(v, C - 1, kWave);
            if (lane < C) {
                sbeta[lane] = beta;
                sgam[lane] = v;
                sE[lane] = exp_neg(v);
                sD[lane] = exp_neg(glast - v);
            }
            if (lane == 0) p.decay[static_cast<int64_t>(slot) * p.Hv + h] = expf(glast);
        }
    }
    __syncthreads();

    // ---- 2. Gram matrices on the matrix cores (lower tiles), scaled on the
    //         way out: A = strict_tril(beta_r e^{gamma_r - gamma_s} K^K^T) and
    //         P = tril_incl(e^{gamma_r - gamma_s} Q^K^T).  Wave b < NB takes
    //         diagonal tile b of K^K^T and goes straight on to the 16x16
    //         diagonal block T_bb of Tm = (I + A)^{-1} (its own LDS writes are
    //         visible to it in program order); the other waves take the
    //         remaining tiles, then the Q_G fragments. ----
    static_assert(NB < NW, "a wave per diagonal block and some to spare");
    if (wave < NB) {
        __builtin_amdgcn_s_setprio(2);
        const int b0 = wave * 16;
        {   // diagonal tile of K K^T (its A and B fragments coincide)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < DK / 32; ++kt) {
                const int o = (b0 + l16) * SQ + kt * 32 + lq * 8;
                const u32x4 ah = lds16(sKh + o), al = lds16(sKl + o);
                acc = mfma3(ah, al, ah, al, acc);
            }
            const int s = b0 + l16;
            const float gs = sgam[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = b0 + lq * 4 + i;
                sAd[r * SD + l16] = (s < r) ? sbeta[r] * exp_neg(sgam[r] - gs) * acc[i] : 0.f;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lq == 0) {
            // lane l16 (column): x_r = delta_rc - sum_{s<r} A_rs x_s; row r+1
            // of the block is read while row r is computed
            float x[16];
            f32x4 arow[4], anext[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) arow[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r + 1 < 16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        anext[q] = *reinterpret_cast<const f32x4*>(sAd + (b0 + r + 1) * SD + 4 * q);
                }
                float acc = (r == l16) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc = fmaf(-arow[s / 4][s % 4], x[s], acc);
                x[r] = acc;
#pragma unroll
                for (int q = 0; q < 4; ++q) arow[q] = anext[q];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint16_t hi, lo;
                split_bf16(x[r], hi, lo);
                sTh[(b0 + r) * STT + l16] = hi;
                sTl[(b0 + r) * STT + l16] = lo;
            }
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        constexpr int NOFF = NB * (NB - 1) / 2;            // K K^T tiles below the diagonal
        constexpr int NTI = NB * (NB + 1) / 2;             // Q K^T lower tiles
        for (int job = wave - NB; job < NOFF + NTI; job += NW - NB) {
            const bool isq = job >= NOFF;
            int idx = isq ? job - NOFF : job, mt, nt;
            if (isq) {
                mt = 0;
                while (idx > mt) { idx -= mt + 1; ++mt; }
            } else {
                mt = 1;
                while (idx >= mt) { idx -= mt; ++mt; }
            }
            nt = idx;
            const uint16_t* ah = isq ? sQh : sKh;
            const uint16_t* al = isq ? sQl : sKl;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < DK / 32; ++kt) {
                const int ao = (mt * 16 + l16) * SQ + kt * 32 + lq * 8;
                const int bo = (nt * 16 + l16) * SQ + kt * 32 + lq * 8;
                acc = mfma3(lds16(ah + ao), lds16(al + ao), lds16(sKh + bo), lds16(sKl + bo), acc);
            }
            const int s = nt * 16 + l16;
            const float gs = sgam[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mt * 16 + lq * 4 + i;
                const float d = exp_neg(sgam[r] - gs);
                if (isq) {
                    sP[r * SG + s] = (s <= r) ? acc[i] * d : 0.f;
                } else {                                 // -A split, a matrix-core operand
                    uint16_t hi, lo;
                    split_bf16(-(sbeta[r] * d * acc[i]), hi, lo);
                    sAh[r * SA + s] = hi;
                    sAl[r * SA + s] = lo;
                }
            }
        }
        const int t1 = tid - NB * kWave;
        constexpr int NT1 = NT - NB * kWave;
        for (int sl = t1; sl < C * DK / 8; sl += NT1) {           // Q_G [C][DK]
            const int tile = sl / 64, ln = sl % 64;
            const int mt = tile / (DK / 32), kt = tile % (DK / 32);
            const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
            float x[8];
            unpack8(lds16(sQh + r * SQ + c0), lds16(sQl + r * SQ + c0), x);
            const float e = sE[r];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= e;
            *reinterpret_cast<u32x4*>(blk + L::QG + tile * 1024 + ln * 16) = pack8_f16(x);
        }
    }
    __syncthreads();

    // ---- 3. [W | U~] = Tm [diag(beta e^gamma) K^ | diag(beta) V^] by block
    //         forward substitution over the 16-token blocks,
    //             X_i = T_ii (B_i - sum_{j<i} A_ij X_j),
    //         one 16-column tile per wave on split-bf16 k = 16 matrix-core
    //         products: their accumulator layout is their B-operand layout,
    //         so X_j stays in registers and the waves never wait for each
    //         other.  U~ goes out directly, -W is staged (fp16) over Q^
    //         (dead).
    //         Then the P and K_d^T fragments. ----
    constexpr int NTW = DK / 16, NTU = DV / 16, NTT = NTW + NTU;
    static_assert(NTT <= NW, "one column tile per wave");
    if (wave < NTT) {
        const bool isw = wave < NTW;
        const int ch = (isw ? wave : wave - NTW) * 16 + l16;
        f32x4 X[NB];
        uint2 xh[NB], xl[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int s0 = 16 * i + 4 * lq;
            const f32x4 be = *reinterpret_cast<const f32x4*>(sbeta + s0);
            const f32x4 ee = *reinterpret_cast<const f32x4*>(sE + s0);
            f32x4 acc;
            if (isw) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = hl(sKh + ch, sKl + ch, (s0 + e) * SQ) * (be[e] * ee[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = sV[(s0 + e) * SV + ch] * be[e];
            }
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const int ao = (16 * i + l16) * SA + 16 * j + 4 * lq;
                acc = mfma3_k16(*reinterpret_cast<const uint2*>(sAh + ao), *reinterpret_cast<const uint2*>(sAl + ao),
                                xh[j], xl[j], acc);
            }
            const int to = (16 * i + l16) * STT + 4 * lq;
            uint2 yh, yl;
            split4(acc, yh, yl);
            X[i] = mfma3_k16(*reinterpret_cast<const uint2*>(sTh + to), *reinterpret_cast<const uint2*>(sTl + to),
                             yh, yl, f32x4{0.f, 0.f, 0.f, 0.f});
            if (i + 1 < NB) split4(X[i], xh[i], xl[i]);
        }
        if (isw) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sW[(16 * i + 4 * lq + r) * SQ + wave * 16 + l16] =
                        __builtin_bit_cast(uint16_t, static_cast<_Float16>(-X[i][r]));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int tile = i * NTU + (wave - NTW);
                *reinterpret_cast<f32x4*>(blk + L::Ut + tile * 1024 + lane * 16) = X[i];
            }
        }
    }
    for (int sl = tid; sl < C * CK / 8; sl += NT) {               // P [C][CK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int r = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = (s / 16 <= r / 16 && s < C) ? sP[r * SG + s] : 0.f;
        }
        *reinterpret_cast<u32x4*>(blk + L::P + tile * 1024 + ln * 16) = pack8_f16(x);
    }
    for (int sl = tid; sl < DK * CK / 8; sl += NT) {              // K_d^T [DK][CK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int i = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            x[e] = s < C ? sD[s] * hl(sKh, sKl, s * SQ + i) : 0.f;
        }
        *reinterpret_cast<u32x4*>(blk + L::KdT + tile * 1024 + ln * 16) = pack8_f16(x);
    }
    __syncthreads();

    // ---- 4. -W out as A fragments ----
    for (int sl = tid; sl < C * DK / 8; sl += NT) {
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (DK / 32), kt = tile % (DK / 32);
        const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
        *reinterpret_cast<u32x4*>(blk + L::negW + tile * 1024 + ln * 16) = lds16(sW + r * SQ + c0);
    }
}

}  // namespace gdn
