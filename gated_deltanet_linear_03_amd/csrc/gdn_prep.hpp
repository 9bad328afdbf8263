// gdn_prep.hpp -- chunk-parallel operand kernel of the chunked prefill.
//
// One work-group (1024 threads, 16 waves) per (chunk slot, group of GH value
// heads that share one key head) of a window of chunk slots; GH = 2 when the
// value heads per key head come in pairs, else 1.  The key head's q^ and k^
// and their Gram matrices serve every value head of the group, so they are
// computed once per group.  For the chunk's C tokens it computes, on chip:
//   q^, k^  conv1d(K=4) + SiLU + L2 norm of the key head (items of 4 tokens x
//           8 channels: 16-byte loads, norms reduced across a row's lanes)
//   v^      conv1d + SiLU of each value head of the group
//   g, beta the gates of each value head; gamma = in-chunk inclusive cumsum
//   K^K^T, Q^K^T  lower tiles, split-bf16 MFMA, once for the group; scaled
//           per value head into
//           A = strict_tril(beta_r e^{gamma_r - gamma_s} K^K^T) and
//           P = tril_incl(e^{gamma_r - gamma_s} Q^K^T)
//   T_bb = 16x16 diagonal blocks of Tm = (I + A)^{-1}, by substitution
//   [W | U~] = Tm [diag(beta e^gamma) K^ | diag(beta) V^] by block forward
//           substitution X_i = T_ii (B_i - sum_{j<i} A_ij X_j) over the
//           16-token blocks, split-bf16 MFMA; a wave runs one W and one U~
//           column tile of a head, which share the A and T fragments
// and writes, per value head, the scan's operands in MFMA fragment order:
// -W and K_d^T = (diag(e^{gamma_last - gamma}) K^)^T as fp16, Q_G =
// diag(e^gamma) Q^ and P as fp16 hi + lo pairs (the output products run
// split), U~ as fp32, plus e^{gamma_last}.  (Chunk form of Yang,
// Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025, on the UT
// transform of Yang et al., NeurIPS 2024.)  Every value head's operands are
// the same bits whichever GH produced them.
#pragma once
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

template <int DK, int DV, int C, int GH>
struct PrepSmem {
    static constexpr int CK = ck_pad(C);
    static constexpr int NB = C / 16;
    static constexpr int SQ = DK + 8;    // bf16 row stride of Q^, K^ [C][SQ]; fp16 stride of the -W staging
    static constexpr int SV = DV + 8;    // fp32 row stride of V^ [C][SV]
    static constexpr int SP = C + 8;     // fp16 row stride of P (hi, lo) [C][SP]
    static constexpr int NBLK = NB * (NB - 1) / 2;   // 16x16 blocks of A below the diagonal blocks
    static constexpr int SAB = 24;       // bf16 row stride inside a block of -A (hi, lo) [NBLK][16][SAB]
    static constexpr int SD = 20;        // fp32 row stride of A's diagonal blocks [NB][16][SD]
    static constexpr int STT = 24;       // bf16 row stride of the blocks T_bb [NB][16][STT]
    static constexpr int qk_bytes = C * SQ * 4;     // hi + lo
    static constexpr int w_bytes = (2 * DK + GH * DV) * 16;
    static constexpr int v_bytes = C * SV * 4;
    // per value head, after the conv: A's diagonal blocks, -A (hi, lo), P (hi, lo), T_bb (hi, lo)
    static constexpr int ad_bytes = NB * 16 * SD * 4;
    static constexpr int a_bytes = NBLK * 16 * SAB * 4;
    static constexpr int p_bytes = C * SP * 4;
    static constexpr int tt_bytes = NB * 16 * STT * 4;
    static constexpr int oA = ad_bytes, oP = oA + a_bytes, oT = oP + p_bytes;
    static constexpr int head_bytes = oT + tt_bytes;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int oQ = 0;                                   // Q^ -> -W staging of the GH heads
    static constexpr int oK = oQ + qk_bytes;                       // K^
    static constexpr int oR = oK + qk_bytes;                       // conv weights + V^ -> per-head blocks
    static constexpr int oS = oR + cmax(w_bytes + GH * v_bytes, GH * head_bytes);   // gate vectors
    static constexpr int total = oS + GH * 4 * C * 4;
};

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
        // the common case: all seven rows inside the chunk's sequence rows,
        // read non-temporally (used once: they should not push the window's
        // operand blocks or the pre-norm output out of the caches)
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            const u32x4* q = reinterpret_cast<const u32x4*>(row + j * rs);
#pragma unroll
            for (int w = 0; w < W; ++w) raw.r[j][w] = __builtin_nontemporal_load(q + w);
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

template <int DK, int DV, int C, int GH, bool BF16>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrefillParams p) {
    using S = PrepSmem<DK, DV, C, GH>;
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = S::CK, SQ = S::SQ, SV = S::SV, SP = S::SP, SAB = S::SAB, SD = S::SD, STT = S::STT;
    constexpr int NBLK = S::NBLK;
    constexpr int NB = C / 16;           // 16-token blocks in a chunk
    constexpr int NT = kPrepThreads;
    constexpr int NW = NT / kWave;
    static_assert(C % 16 == 0 && C <= kWave && DK % 32 == 0 && DV % 16 == 0 && DK <= 128, "shape");
    static_assert(GH == 1 || GH == 2, "one or two value heads per work-group");
    static_assert(S::total <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint8_t smem[S::total];
    uint16_t* sQh = reinterpret_cast<uint16_t*>(smem + S::oQ);
    uint16_t* sQl = sQh + C * SQ;
    uint16_t* sKh = reinterpret_cast<uint16_t*>(smem + S::oK);
    uint16_t* sKl = sKh + C * SQ;
    f32x4* sCw = reinterpret_cast<f32x4*>(smem + S::oR);
    // per value head g of the group
    auto sV = [&](int g) { return reinterpret_cast<float*>(smem + S::oR + S::w_bytes + g * S::v_bytes); };
    auto hb = [&](int g) { return smem + S::oR + g * S::head_bytes; };
    auto sAd = [&](int g) { return reinterpret_cast<float*>(hb(g)); };
    auto sAh = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oA); };
    auto sAl = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oA) + NBLK * 16 * SAB; };
    auto sP = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oP); };
    auto sPl = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oP) + C * SP; };
    // block (i, j), j < i, of -A: NBLK blocks of 16 x 16 in row-major block order
    auto ablk = [&](int i, int j) { return (i * (i - 1) / 2 + j) * 16 * SAB; };
    auto sTh = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oT); };
    auto sTl = [&](int g) { return reinterpret_cast<uint16_t*>(hb(g) + S::oT) + NB * 16 * STT; };
    auto sW = [&](int g) { return sQh + g * C * SQ; };      // -W staging (fp16) over Q^
    auto sbeta = [&](int g) { return reinterpret_cast<float*>(smem + S::oS) + g * 4 * C; };
    auto sgam = [&](int g) { return sbeta(g) + C; };
    auto sE = [&](int g) { return sbeta(g) + 2 * C; };     // e^{gamma_r}
    auto sD = [&](int g) { return sbeta(g) + 3 * C; };     // e^{gamma_last - gamma_r}

    const int slot = p.win_lo + blockIdx.x;
    const int h0 = blockIdx.y * GH;
    const int hk = h0 / p.G;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    // the chunk table: built here in the first window (work-group (0, 0)
    // stores it), read from the workspace after that
    int total, n = 0, first = 0;
    if (p.win_idx == 0) {
        // the call's first kernel: clear the caller's status word
        const bool lead = blockIdx.x == 0 && blockIdx.y == 0;
        if (p.status && lead && threadIdx.x == 0) *p.status = 0;
        const ChunkPos cp = chunk_table<kPrepThreads>(p, C, slot, reinterpret_cast<int32_t*>(smem + S::oS),
                                                      lead ? p.chunk_off : nullptr);
        if (cp.bad) {
            // The device-side indices broke their contract (cu_seqlens not
            // starting at 0, decreasing or not ending at T_total; a pool
            // entry outside [0, num_slots)).  Nothing is computed: the chunk
            // table's total becomes -1, which every later kernel of the call
            // takes as "return at once", and the status word gets
            // kStatusBadIndex.
            if (lead && tid == 0) {
                p.chunk_off[p.N] = -1;
                if (p.status)
                    __hip_atomic_fetch_or(p.status, kStatusBadIndex, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return;
        }
        total = cp.total;
        n = cp.n;
        first = cp.first;
    } else {
        total = p.chunk_off[p.N];
    }
    total = min(total, p.win_hi);
    if (slot >= total) return;
    if (p.win_idx != 0) {
        n = seq_of_chunk(p.chunk_off, p.N, slot);
        first = p.chunk_off[n];
    }
    const int64_t start = p.cu[n], end = p.cu[n + 1];
    const int64_t t0 = start + static_cast<int64_t>(slot - first) * C;
    const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
    const int qk = p.Hk * DK;
    const int Cc = 2 * qk + p.Hv * DV;
    auto blk = [&](int g) {
        return p.vch + (static_cast<int64_t>(slot - p.win_lo) * p.Hv + h0 + g) * L::bytes;
    };

    // ---- 1. conv inputs, then conv + SiLU (+ L2 norm for q, k), gates ----
    // Each thread owns one item, 4 tokens x 8 channels of q, k or one value
    // head's v (q items, then k items, then v items head by head), and issues
    // its 7 input-row loads, one conv-weight row for the LDS copy and, in
    // waves g < GH, the gate inputs of head g before anything else, so the
    // chunk's inputs cost one memory round trip.  Waves g < GH then compute
    // head g's gates and in-chunk cumulative decay after their conv.
    static_assert(C % 4 == 0, "row groups");
    constexpr int GPRK = DK / 8, GPRV = DV / 8;        // lanes per token row
    constexpr int IQ = (C / 4) * GPRK, IV = (C / 4) * GPRV;
    // (a row's GPRK lanes are always of one kind: the norm reduces over them)
    static_assert(2 * IQ + GH * IV <= NT && kWave % GPRK == 0, "one item per thread");
    constexpr int NCW = 2 * DK + GH * DV;               // staged weight rows (q | k | v of each head)
    static_assert(NCW <= NT && GH <= NW, "one weight row per thread");
    {
        const int kind = tid < IQ ? 0 : (tid < 2 * IQ ? 1 : (tid < 2 * IQ + GH * IV ? 2 : 3));
        const int it = kind == 0 ? tid : (kind == 1 ? tid - IQ : (tid - 2 * IQ) % IV);
        const int vg = kind == 2 ? (tid - 2 * IQ) / IV : 0;     // value head of a v item
        const int gpr = kind == 2 ? GPRV : GPRK;
        const int grp = it % gpr, r0 = (it / gpr) * 4;
        const int col = (kind == 2 ? (h0 + vg) * DV : hk * DK) + grp * 8;
        const int c0 = (kind == 2 ? 2 * qk : kind * qk) + col;
        const void* src = kind == 0 ? p.q : (kind == 1 ? p.k : p.v);
        const int64_t rs = kind == 0 ? p.qs : (kind == 1 ? p.ks : p.vs);
        RawRows<BF16> raw;
        if (kind < 3)
            load_rows<BF16>(p, state_slot(p.slots, n), start, t0, r0, Lc, src, rs, col, c0, Cc, raw);
        f32x4 wrow;
        if (tid < NCW) {
            const int ch = tid < DK ? hk * DK + tid
                         : (tid < 2 * DK ? qk + hk * DK + (tid - DK) : 2 * qk + h0 * DV + (tid - 2 * DK));
            wrow = *reinterpret_cast<const f32x4*>(p.conv_w + ch * 4);
        }
        float av = 0.f, bv = 0.f;
        if (wave < GH && lane < Lc) {
            using A = Act<BF16>;
            using T = typename A::T;
            av = A::load(static_cast<const T*>(p.a) + (t0 + lane) * p.as + h0 + wave);
            bv = A::load(static_cast<const T*>(p.b) + (t0 + lane) * p.bs + h0 + wave);
        }
        if (tid < NCW) sCw[tid] = wrow;
        __syncthreads();
        if (kind < 3) {
            f32x4 w[8];
            const int wb = (kind == 0 ? 0 : (kind == 1 ? DK : 2 * DK + vg * DV)) + grp * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = sCw[wb + e];
            float y[4][8];
            conv_rows<BF16>(raw, w, r0, Lc, y);
            uint16_t* dh = kind == 0 ? sQh : sKh;
            uint16_t* dl = kind == 0 ? sQl : sKl;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (kind == 2) {
                    float* dv = sV(vg) + (r0 + t) * SV + grp * 8;
                    *reinterpret_cast<f32x4*>(dv) = f32x4{y[t][0], y[t][1], y[t][2], y[t][3]};
                    *reinterpret_cast<f32x4*>(dv + 4) = f32x4{y[t][4], y[t][5], y[t][6], y[t][7]};
                    continue;
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[t][e], y[t][e], ss);
                ss = group_sum<GPRK>(ss);
                const float f = (kind ? 1.0f : p.scale) * __builtin_amdgcn_rsqf(ss + p.eps_l2);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[t][e] *= f;
                u32x4 hi, lo;
                split8(y[t], hi, lo);
                *reinterpret_cast<u32x4*>(dh + (r0 + t) * SQ + grp * 8) = hi;
                *reinterpret_cast<u32x4*>(dl + (r0 + t) * SQ + grp * 8) = lo;
            }
        }
        if (wave < GH) {
            // gates of head h0 + wave, then the inclusive prefix sum over the
            // chunk (Hillis-Steele, fixed order); tokens past the chunk's end
            // have g = beta = 0
            const int h = h0 + wave;
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
                sbeta(wave)[lane] = beta;
                sgam(wave)[lane] = v;
                sE(wave)[lane] = exp_neg(v);
                sD(wave)[lane] = exp_neg(glast - v);
            }
            if (lane == 0) p.decay[static_cast<int64_t>(slot) * p.Hv + h] = expf(glast);
        }
    }
    __syncthreads();

    // ---- the substitution's waves take their V^ columns (times beta) into
    //      registers now: the per-head blocks below overwrite V^.  Wave
    //      g * WPH + j runs W column tile j and U~ column tile j of head g. ----
    constexpr int NTW = DK / 16, NTU = DV / 16;
    constexpr int WPH = NTW > NTU ? NTW : NTU;
    static_assert(GH * WPH <= NW, "a W and a U~ column tile per wave");
    const bool sub = wave < GH * WPH;
    const int g3 = sub ? wave / WPH : 0, j3 = wave % WPH;
    const bool has_w = sub && j3 < NTW, has_u = sub && j3 < NTU;
    f32x4 Vb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) Vb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (has_u) {
        const float* v = sV(g3);
        const float* be = sbeta(g3);
        const int ch = j3 * 16 + l16;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * i + 4 * lq + e;
                Vb[i][e] = v[s * SV + ch] * be[s];
            }
    }
    __syncthreads();

    // ---- 2. Gram matrices on the matrix cores (lower tiles, once for the
    //         group), scaled per value head on the way out:
    //         A = strict_tril(beta_r e^{gamma_r - gamma_s} K^K^T) and
    //         P = tril_incl(e^{gamma_r - gamma_s} Q^K^T).  Wave b < NB takes
    //         diagonal tile b of K^K^T and goes straight on to the 16x16
    //         diagonal blocks T_bb of Tm = (I + A)^{-1}, lanes 16 g .. 16 g + 15
    //         solving head g's (its own LDS writes are visible to it in
    //         program order); the other waves take the remaining tiles, then
    //         the Q_G fragments.  Each lane's four gate values are read as
    //         one vector per head before any arithmetic. ----
    static_assert(NB < NW && GH * 16 <= kWave, "a wave per diagonal block and some to spare");
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
            const int s = b0 + l16, r0 = b0 + lq * 4;
            f32x4 gr[GH], br[GH];
            float gs[GH];
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                gr[g] = *reinterpret_cast<const f32x4*>(sgam(g) + r0);
                br[g] = *reinterpret_cast<const f32x4*>(sbeta(g) + r0);
                gs[g] = sgam(g)[s];
            }
#pragma unroll
            for (int g = 0; g < GH; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sAd(g)[(r0 + i) * SD + l16] = (s < r0 + i) ? br[g][i] * exp_neg(gr[g][i] - gs[g]) * acc[i] : 0.f;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lq < GH) {
            // lane l16 of row group g = lq (column l16 of head g's block):
            // x_r = delta_rc - sum_{s<r} A_rs x_s; row r+1 of the block is
            // read while row r is computed
            const float* ad = sAd(lq);
            float x[16];
            f32x4 arow[4], anext[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) arow[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r + 1 < 16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        anext[q] = *reinterpret_cast<const f32x4*>(ad + (b0 + r + 1) * SD + 4 * q);
                }
                float acc = (r == l16) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc = fmaf(-arow[s / 4][s % 4], x[s], acc);
                x[r] = acc;
#pragma unroll
                for (int q = 0; q < 4; ++q) arow[q] = anext[q];
            }
            uint16_t* th = sTh(lq);
            uint16_t* tl = sTl(lq);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint16_t hi, lo;
                split_bf16(x[r], hi, lo);
                th[(b0 + r) * STT + l16] = hi;
                tl[(b0 + r) * STT + l16] = lo;
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
            const int s = nt * 16 + l16, r0 = mt * 16 + lq * 4;
            f32x4 gr[GH], br[GH];
            float gs[GH];
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                gr[g] = *reinterpret_cast<const f32x4*>(sgam(g) + r0);
                br[g] = *reinterpret_cast<const f32x4*>(sbeta(g) + r0);
                gs[g] = sgam(g)[s];
            }
            if (isq) {                                       // P as fp16 hi + lo
#pragma unroll
                for (int g = 0; g < GH; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float d = exp_neg(gr[g][i] - gs[g]);
                        const float v = (s <= r0 + i) ? acc[i] * d : 0.f;
                        const _Float16 hi = static_cast<_Float16>(v);
                        sP(g)[(r0 + i) * SP + s] = __builtin_bit_cast(uint16_t, hi);
                        sPl(g)[(r0 + i) * SP + s] =
                            __builtin_bit_cast(uint16_t, static_cast<_Float16>(v - static_cast<float>(hi)));
                    }
            } else {                                         // -A split, a matrix-core operand
                const int bo = ablk(mt, nt) + (lq * 4) * SAB + l16;
#pragma unroll
                for (int g = 0; g < GH; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float d = exp_neg(gr[g][i] - gs[g]);
                        uint16_t hi, lo;
                        split_bf16(-(br[g][i] * d * acc[i]), hi, lo);
                        sAh(g)[bo + i * SAB] = hi;
                        sAl(g)[bo + i * SAB] = lo;
                    }
            }
        }
        // Q_G slots, the last threads first: the first waves of this group
        // may have taken one tile more
        constexpr int NT1 = NT - NB * kWave;
        const int t1 = NT1 - 1 - (tid - NB * kWave);
        for (int sl = t1; sl < C * DK / 8; sl += NT1) {           // Q_G [C][DK]
            const int tile = sl / 64, ln = sl % 64;
            const int mt = tile / (DK / 32), kt = tile % (DK / 32);
            const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
            float x[8];
            unpack8(lds16(sQh + r * SQ + c0), lds16(sQl + r * SQ + c0), x);
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const float e = sE(g)[r];
                float y[8], yl[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    y[i] = x[i] * e;
                    yl[i] = y[i] - static_cast<float>(static_cast<_Float16>(y[i]));
                }
                *reinterpret_cast<u32x4*>(blk(g) + L::QG + tile * 1024 + ln * 16) = pack8_f16(y);
                *reinterpret_cast<u32x4*>(blk(g) + L::QGl + tile * 1024 + ln * 16) = pack8_f16(yl);
            }
        }
    }
    __syncthreads();

    // ---- the P and K_d^T fragments go out first: they read only LDS the
    //      substitution leaves alone (P, K^ and the decays), so their stores
    //      drain while it computes ----
    constexpr int NPS = C * CK / 8;                                // P slots per head
    for (int sl = tid; sl < GH * NPS; sl += NT) {                  // P [C][CK]
        const int g = sl / NPS, tile = (sl % NPS) / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int r = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        if (kt * 32 > mt * 16 + 15) continue;       // a zero tile: never read
        // eight columns of one 16-column tile: tiles above the diagonal and
        // columns past C are zero
        const bool nz = s0 / 16 <= r / 16 && s0 < C;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(blk(g) + L::P + tile * 1024 + ln * 16) = nz ? lds16(sP(g) + r * SP + s0) : zero;
        *reinterpret_cast<u32x4*>(blk(g) + L::Pl + tile * 1024 + ln * 16) = nz ? lds16(sPl(g) + r * SP + s0) : zero;
    }
    for (int sl = tid; sl < DK * CK / 8; sl += NT) {              // K_d^T [DK][CK]
        const int tile = sl / 64, ln = sl % 64;
        const int mt = tile / (CK / 32), kt = tile % (CK / 32);
        const int i = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
        float kv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = s0 + e < C ? hl(sKh, sKl, (s0 + e) * SQ + i) : 0.f;
#pragma unroll
        for (int g = 0; g < GH; ++g) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = s0 + e < C ? sD(g)[s0 + e] * kv[e] : 0.f;
            *reinterpret_cast<u32x4*>(blk(g) + L::KdT + tile * 1024 + ln * 16) = pack8_f16(x);
        }
    }

    // ---- 3. [W | U~] = Tm [diag(beta e^gamma) K^ | diag(beta) V^] by block
    //         forward substitution over the 16-token blocks,
    //             X_i = T_ii (B_i - sum_{j<i} A_ij X_j),
    //         on split-bf16 k = 16 matrix-core products: their accumulator
    //         layout is their B-operand layout, so X_j stays in registers and
    //         the waves never wait for each other.  A wave's W and U~ tiles
    //         are two independent chains on the same A and T fragments.  U~
    //         goes out block by block, -W once the wave's chain is done. ----
    if (sub) {
        const float* be = sbeta(g3);
        const float* ee = sE(g3);
        const uint16_t* ahp = sAh(g3);
        const uint16_t* alp = sAl(g3);
        const uint16_t* thp = sTh(g3);
        const uint16_t* tlp = sTl(g3);
        const int ch = j3 * 16 + l16;
        f32x4 XW[NB], XU[NB];
        uint2 wh[NB], wl[NB], uh[NB], ul[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int s0 = 16 * i + 4 * lq;
            f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = Vb[i];
            if (has_w) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(be + s0);
                const f32x4 e4 = *reinterpret_cast<const f32x4*>(ee + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) aw[e] = hl(sKh + ch, sKl + ch, (s0 + e) * SQ) * (b4[e] * e4[e]);
            }
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const int ao = ablk(i, j) + l16 * SAB + 4 * lq;
                const uint2 a_h = *reinterpret_cast<const uint2*>(ahp + ao);
                const uint2 a_l = *reinterpret_cast<const uint2*>(alp + ao);
                if (has_w) aw = mfma3_k16(a_h, a_l, wh[j], wl[j], aw);
                if (has_u) au = mfma3_k16(a_h, a_l, uh[j], ul[j], au);
            }
            const int to = (16 * i + l16) * STT + 4 * lq;
            const uint2 t_h = *reinterpret_cast<const uint2*>(thp + to);
            const uint2 t_l = *reinterpret_cast<const uint2*>(tlp + to);
            if (has_w) {
                uint2 yh, yl;
                split4(aw, yh, yl);
                XW[i] = mfma3_k16(t_h, t_l, yh, yl, f32x4{0.f, 0.f, 0.f, 0.f});
                if (i + 1 < NB) split4(XW[i], wh[i], wl[i]);
            }
            if (has_u) {
                uint2 yh, yl;
                split4(au, yh, yl);
                XU[i] = mfma3_k16(t_h, t_l, yh, yl, f32x4{0.f, 0.f, 0.f, 0.f});
                if (i + 1 < NB) split4(XU[i], uh[i], ul[i]);
                // block i of U~ is final: out now, while the later blocks compute
                *reinterpret_cast<f32x4*>(blk(g3) + L::Ut + (i * NTU + j3) * 1024 + lane * 16) = XU[i];
            }
        }
        if (has_w) {
            // ---- 4. -W out as A fragments, by each wave for its own 16
            //      columns: they go through LDS (fp16, over Q^, dead) to
            //      change lanes, and the wave stores its half of each 16 x 32
            //      fragment tile (lanes 16 h' .. 16 h' + 15 with h' = 2 (j3 % 2)
            //      + h) as soon as its substitution is done, with no wait on
            //      the other waves ----
            uint16_t* sw = sW(g3);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sw[(16 * i + 4 * lq + r) * SQ + ch] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-XW[i][r]));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint8_t* b = blk(g3) + L::negW;
            for (int idx = lane; idx < NB * 32; idx += kWave) {
                const int mt = idx / 32, h = (idx / 16) % 2, row = idx % 16;
                const int slot = (2 * (j3 % 2) + h) * 16 + row;          // lane slot in the tile
                const int tile = mt * (DK / 32) + j3 / 2;
                *reinterpret_cast<u32x4*>(b + tile * 1024 + slot * 16) =
                    lds16(sw + (16 * mt + row) * SQ + 16 * j3 + 8 * h);
            }
        }
    }
}

}  // namespace gdn
