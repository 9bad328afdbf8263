// gdn_prefill.hip -- chunked Gated DeltaNet prefill over packed sequences.
//
// Chunk form (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025,
// chunkwise algorithm built on the WY/UT representation of Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", NeurIPS 2024).  For a chunk of C tokens with in-chunk cumulative
// decay gamma_r = sum_{s<=r} g_s and entering state H = S^T [dk][dv]:
//     A_rs = beta_r e^{gamma_r - gamma_s} (k_r . k_s),  s < r
//     Tm   = (I + A)^{-1}
//     W    = Tm diag(beta e^gamma) K,        U~ = Tm diag(beta) V
//     U    = U~ - W H
//     O    = diag(e^gamma) Q H + tril_incl(Q K^T (.) D) U,  D_rs = e^{gamma_r-gamma_s}
//     H'   = e^{gamma_last} H + (diag(e^{gamma_last - gamma}) K)^T U
// Only exponentials of non-positive differences are formed, so decays that
// underflow inside a chunk go to zero as they should.
//
// Kernels, in stream order:
//   plan_kernel   first chunk index of every sequence (chunks restart at each
//                 sequence start, so results do not depend on the packing)
//   prep_kernel   chunk-parallel over (chunk, key head): conv1d+SiLU, L2 norms,
//                 gates, Gram matrices, triangular solve, and the per-chunk
//                 operands -W, Q_G = diag(e^gamma) Q, K_d^T, P, U~ written in
//                 matrix-core fragment order (split bf16 hi/lo)
//   scan_kernel   sequential over the chunks of one (sequence, value head,
//                 dv slice): U, O and H' on split-bf16 matrix-core products,
//                 H kept in fp32 accumulators for the whole sequence; also
//                 writes the final state and the conv state tail
//   epi_kernel    token-parallel SiLU(z)-gated RMSNorm of o.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// plan: chunk_off[n] = sum_{m<n} ceil(L_m / C), chunk_off[N] = total chunks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* cu, int N, int C,
                                                   int32_t* chunk_off) {
    __shared__ int32_t part[256];
    const int tid = threadIdx.x;
    const int per = (N + 255) / 256;
    const int n0 = min(N, tid * per), n1 = min(N, n0 + per);
    int32_t s = 0;
    for (int n = n0; n < n1; ++n) s += (cu[n + 1] - cu[n] + C - 1) / C;
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int i = 0; i < 256; ++i) {
            const int32_t v = part[i];
            part[i] = acc;
            acc += v;
        }
        chunk_off[N] = acc;
    }
    __syncthreads();
    int32_t acc = part[tid];
    for (int n = n0; n < n1; ++n) {
        chunk_off[n] = acc;
        acc += (cu[n + 1] - cu[n] + C - 1) / C;
    }
}

// Sequence owning chunk slot c: the last n with chunk_off[n] <= c.
__device__ __forceinline__ int seq_of_chunk(const int32_t* chunk_off, int N, int c) {
    int lo = 0, hi = N;   // invariant: chunk_off[lo] <= c < chunk_off[hi+1] region
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Byte offsets of the operand arrays inside one (chunk, value head) block.
template <int DK, int DV, int C>
struct VchLayout {
    static constexpr int CK = ck_pad(C);
    static constexpr int64_t negW = 0;
    static constexpr int64_t QG = negW + 4ll * C * DK;
    static constexpr int64_t KdT = QG + 4ll * C * DK;
    static constexpr int64_t P = KdT + 4ll * DK * CK;
    static constexpr int64_t Ut = P + 4ll * C * CK;
    static constexpr int64_t bytes = Ut + 4ll * C * DV;
    static_assert(bytes == vch_bytes(DK, DV, C), "layout");
};

// Raw input of channel c at token position pos of the sequence starting at
// `start`; earlier positions read the conv state row (K-1) + (pos - start).
template <bool BF16>
__device__ __forceinline__ float raw_in(const PrefillParams& p, int n, int64_t start,
                                        int64_t pos, int c, int Cc, int qk) {
    using A = Act<BF16>;
    using T = typename A::T;
    if (pos < start) {
        const int64_t r = 3 + (pos - start);
        if (r < 0 || !p.conv_in) return 0.f;
        return A::load(static_cast<const T*>(p.conv_in) + (static_cast<int64_t>(n) * 3 + r) * Cc + c);
    }
    if (c < qk) return A::load(static_cast<const T*>(p.q) + pos * p.qs + c);
    if (c < 2 * qk) return A::load(static_cast<const T*>(p.k) + pos * p.ks + (c - qk));
    return A::load(static_cast<const T*>(p.v) + pos * p.vs + (c - 2 * qk));
}

template <bool BF16>
__device__ __forceinline__ float conv_silu_at(const PrefillParams& p, int n, int64_t start,
                                              int64_t pos, int c, int Cc, int qk) {
    const float* w = p.conv_w + static_cast<size_t>(c) * 4;
    float acc = w[0] * raw_in<BF16>(p, n, start, pos - 3, c, Cc, qk);
    acc = fmaf(w[1], raw_in<BF16>(p, n, start, pos - 2, c, Cc, qk), acc);
    acc = fmaf(w[2], raw_in<BF16>(p, n, start, pos - 1, c, Cc, qk), acc);
    acc = fmaf(w[3], raw_in<BF16>(p, n, start, pos, c, Cc, qk), acc);
    return silu(acc);
}

// Store 8 fp32 values as one A-fragment slot (hi and lo bf16 halves).
__device__ __forceinline__ void store_afrag(uint8_t* tile, int lane, const float* x8) {
    uint16_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16(x8[e], hi[e], lo[e]);
    *reinterpret_cast<u32x4*>(tile + lane * 16) = pack8(hi);
    *reinterpret_cast<u32x4*>(tile + 1024 + lane * 16) = pack8(lo);
}

// ---------------------------------------------------------------------------
// prep: one work-group per (chunk slot, key head).
// ---------------------------------------------------------------------------
template <int DK, int DV, int C, bool BF16>
__global__ __launch_bounds__(256) void prep_kernel(PrefillParams p) {
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = L::CK;
    constexpr int NT = 256;
    constexpr int SD = DK + 4, SV = DV + 4, SC = C + 1;
    __shared__ float sQ[C * SD], sK[C * SD], sV[C * SV];
    __shared__ float sGkk[C * SC], sGqk[C * SC], sT[C * SC];
    __shared__ float sg[C], sbeta[C], sgam[C], cW[C], cU[C], eG[C], eD[C], sacc[C];

    const int slot = blockIdx.x;
    const int hk = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int total = p.chunk_off[p.N];
    if (slot >= total) return;
    const int n = seq_of_chunk(p.chunk_off, p.N, slot);
    const int64_t start = p.cu[n], end = p.cu[n + 1];
    const int64_t t0 = start + static_cast<int64_t>(slot - p.chunk_off[n]) * C;
    const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
    const int qk = p.Hk * DK;
    const int Cc = 2 * qk + p.Hv * DV;

    // 1. conv + SiLU of q and k; padding rows are zero.
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        float yq = 0.f, yk = 0.f;
        if (r < Lc) {
            yq = conv_silu_at<BF16>(p, n, start, t0 + r, hk * DK + i, Cc, qk);
            yk = conv_silu_at<BF16>(p, n, start, t0 + r, qk + hk * DK + i, Cc, qk);
        }
        sQ[r * SD + i] = yq;
        sK[r * SD + i] = yk;
    }
    __syncthreads();
    // 2. L2 norms per token (one wave per token).
    for (int r = wave; r < C; r += NT / kWave) {
        float sq = 0.f, sk = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            sq = fmaf(sQ[r * SD + i], sQ[r * SD + i], sq);
            sk = fmaf(sK[r * SD + i], sK[r * SD + i], sk);
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float rq = p.scale / sqrtf(sq + p.eps_l2);
        const float rk = 1.0f / sqrtf(sk + p.eps_l2);
        for (int i = lane; i < DK; i += kWave) {
            sQ[r * SD + i] *= rq;
            sK[r * SD + i] *= rk;
        }
    }
    __syncthreads();
    // 3. Gram matrices K K^T (strict lower) and Q K^T (lower incl. diagonal).
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, s = idx % C;
        float gkk = 0.f, gqk = 0.f;
        if (s <= r) {
            for (int i = 0; i < DK; ++i) {
                gkk = fmaf(sK[r * SD + i], sK[s * SD + i], gkk);
                gqk = fmaf(sQ[r * SD + i], sK[s * SD + i], gqk);
            }
        }
        sGkk[r * SC + s] = gkk;
        sGqk[r * SC + s] = gqk;
    }
    __syncthreads();

    for (int gi = 0; gi < p.G; ++gi) {
        const int h = hk * p.G + gi;
        uint8_t* blk = p.vch + (static_cast<int64_t>(slot) * p.Hv + h) * L::bytes;
        // 4. v conv, gates.
        for (int idx = tid; idx < C * DV; idx += NT) {
            const int r = idx / DV, j = idx % DV;
            float y = 0.f;
            if (r < Lc) y = conv_silu_at<BF16>(p, n, start, t0 + r, 2 * qk + h * DV + j, Cc, qk);
            sV[r * SV + j] = y;
        }
        if (tid < C) {
            float g = 0.f, beta = 0.f;
            if (tid < Lc) {
                using A = Act<BF16>;
                using T = typename A::T;
                const float av = A::load(static_cast<const T*>(p.a) + (t0 + tid) * p.as + h);
                const float bv = A::load(static_cast<const T*>(p.b) + (t0 + tid) * p.bs + h);
                g = -expf(p.A_log[h]) * softplus(av + p.dt_bias[h]);
                beta = sigmoid(bv);
            }
            sg[tid] = g;
            sbeta[tid] = beta;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += sg[r];
                sgam[r] = acc;
            }
        }
        __syncthreads();
        const float glast = sgam[C - 1];
        if (tid < C) {
            const float gm = sgam[tid];
            cW[tid] = sbeta[tid] * expf(gm);
            cU[tid] = sbeta[tid];
            eG[tid] = expf(gm);
            eD[tid] = expf(glast - gm);
        }
        // A (strict lower) into sT; forward substitution in place, row by row.
        for (int idx = tid; idx < C * C; idx += NT) {
            const int r = idx / C, s = idx % C;
            sT[r * SC + s] = (s < r) ? sbeta[r] * expf(sgam[r] - sgam[s]) * sGkk[r * SC + s] : 0.f;
        }
        __syncthreads();
        // Row r of Tm: Tm[r][c] = delta_rc - sum_{c<=s<r} A[r][s] Tm[s][c].
        // Rows < r of sT already hold Tm; row r still holds A.
        for (int r = 0; r < C; ++r) {
            float acc = 0.f;
            if (tid < C) {
                const int c = tid;
                if (c < r) {
                    for (int s = c; s < r; ++s) acc = fmaf(sT[r * SC + s], sT[s * SC + c], acc);
                    acc = -acc;
                } else {
                    acc = (c == r) ? 1.f : 0.f;
                }
                sacc[c] = acc;
            }
            __syncthreads();
            if (tid < C) sT[r * SC + tid] = sacc[tid];
            __syncthreads();
        }
        // 5. operands in fragment order.
        // -W [C][DK]: A tiles (mt, kt), 8 consecutive k per lane slot.
        for (int slotf = tid; slotf < C * DK / 8; slotf += NT) {
            const int tile = slotf / 64, ln = slotf % 64;
            const int mt = tile / (DK / 32), kt = tile % (DK / 32);
            const int r = mt * 16 + ln % 16, c0 = kt * 32 + 8 * (ln / 16);
            float w8[8], q8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { w8[e] = 0.f; }
            for (int s = 0; s <= r; ++s) {
                const float coef = sT[r * SC + s] * cW[s];
#pragma unroll
                for (int e = 0; e < 8; ++e) w8[e] = fmaf(coef, sK[s * SD + c0 + e], w8[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                w8[e] = -w8[e];
                q8[e] = eG[r] * sQ[r * SD + c0 + e];
            }
            store_afrag(blk + L::negW + tile * 2048, ln, w8);
            store_afrag(blk + L::QG + tile * 2048, ln, q8);
        }
        // K_d^T [DK][CK]: row i, col s = e^{glast - gamma_s} k_s[i] (0 for s >= C).
        for (int slotf = tid; slotf < DK * CK / 8; slotf += NT) {
            const int tile = slotf / 64, ln = slotf % 64;
            const int mt = tile / (CK / 32), kt = tile % (CK / 32);
            const int i = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
            float x8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                x8[e] = (s < C) ? eD[s] * sK[s * SD + i] : 0.f;
            }
            store_afrag(blk + L::KdT + tile * 2048, ln, x8);
        }
        // P [C][CK]: row r, col s = (s <= r) Gqk[r][s] e^{gamma_r - gamma_s}.
        for (int slotf = tid; slotf < C * CK / 8; slotf += NT) {
            const int tile = slotf / 64, ln = slotf % 64;
            const int mt = tile / (CK / 32), kt = tile % (CK / 32);
            const int r = mt * 16 + ln % 16, s0 = kt * 32 + 8 * (ln / 16);
            float x8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                x8[e] = (s <= r && s < C) ? sGqk[r * SC + s] * expf(sgam[r] - sgam[s]) : 0.f;
            }
            store_afrag(blk + L::P + tile * 2048, ln, x8);
        }
        // U~ [C][DV] in accumulator order: tile (mt, nt), lane: rows 4*(l/16)+i, col l%16.
        for (int slotf = tid; slotf < C * DV / 4; slotf += NT) {
            const int tile = slotf / 64, ln = slotf % 64;
            const int mt = tile / (DV / 16), nt = tile % (DV / 16);
            const int j = nt * 16 + ln % 16, r0 = mt * 16 + 4 * (ln / 16);
            f32x4 u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i;
                float acc = 0.f;
                for (int s = 0; s <= r; ++s) acc = fmaf(sT[r * SC + s] * cU[s], sV[s * SV + j], acc);
                u[i] = acc;
            }
            *reinterpret_cast<f32x4*>(blk + L::Ut + tile * 1024 + ln * 16) = u;
        }
        if (tid == 0) p.decay[static_cast<int64_t>(slot) * p.Hv + h] = expf(glast);
        __syncthreads();   // sV, sT, gates reused by the next value head
    }
}

// ---------------------------------------------------------------------------
// scan: one work-group per (sequence, value head, dv slice of DVS columns).
// ---------------------------------------------------------------------------
template <int DK, int DV, int C, int DVS, bool BF16>
__global__ __launch_bounds__(256) void scan_kernel(PrefillParams p) {
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = L::CK;
    constexpr int NW = 4;
    constexpr int NS = DV / DVS;          // slices per head
    constexpr int NTL = DVS / 16;         // n tiles per slice
    constexpr int MT = C / 16;            // U/O m tiles
    constexpr int MTH = DK / 16;          // H m tiles
    constexpr int KTH = DK / 32;          // k steps over dk
    constexpr int KTC = CK / 32;          // k steps over the chunk
    constexpr int QU = (MT + NW - 1) / NW;
    constexpr int QH = (MTH + NW - 1) / NW;
    constexpr int HS = DK + 8;            // LDS row stride (bf16) of H^T
    constexpr int US = CK + 8;            // LDS row stride (bf16) of U^T
    static_assert(DV % DVS == 0 && DVS % 16 == 0 && DK % 32 == 0 && C % 16 == 0, "shape");

    __shared__ __align__(16) uint16_t HThi[DVS * HS], HTlo[DVS * HS];
    __shared__ __align__(16) uint16_t UThi[DVS * US], UTlo[DVS * US];

    // XCD-aware order: the NS slices of one head land on the same XCD
    // (consecutive work-groups are dealt round-robin over the 8 XCDs), so the
    // per-chunk operands they all read are shared in that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid % 8, j = bid / 8;
    const int sl = j % NS;
    const int pair = (j / NS) * 8 + xcd;
    if (pair >= p.N * p.Hv) return;
    const int n = pair / p.Hv, h = pair % p.Hv;

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int col0 = sl * DVS;

    // zero U^T (including the padded chunk rows C..CK-1, never written later)
    for (int i = tid; i < DVS * US; i += 256) { UThi[i] = 0; UTlo[i] = 0; }

    // H slice in accumulator fragments: tile (mth = wave + NW*qh, nt).
    f32x4 hacc[QH][NTL];
    const size_t sbase = (static_cast<size_t>(n) * p.Hv + h) * DK * DV;
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) {
        const int mth = wave + NW * qh;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (mth < MTH && p.state_in) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mth * 16 + lq * 4 + i;
                    v[i] = p.state_in[sbase + static_cast<size_t>(row) * DV + col0 + nt * 16 + l16];
                }
            }
            hacc[qh][nt] = v;
        }
    }
    auto store_H_lds = [&]() {
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) {
            const int mth = wave + NW * qh;
            if (mth >= MTH) continue;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) split_bf16(hacc[qh][nt][i], hi[i], lo[i]);
                const int off = (nt * 16 + l16) * HS + mth * 16 + lq * 4;
                *reinterpret_cast<uint2*>(&HThi[off]) =
                    make_uint2(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16));
                *reinterpret_cast<uint2*>(&HTlo[off]) =
                    make_uint2(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16));
            }
        }
    };
    store_H_lds();
    __syncthreads();

    const int c_begin = p.chunk_off[n], c_end = p.chunk_off[n + 1];
    const int64_t start = p.cu[n], end = p.cu[n + 1];
    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = start + static_cast<int64_t>(c - c_begin) * C;
        const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
        const uint8_t* blk = p.vch + (static_cast<int64_t>(c) * p.Hv + h) * L::bytes;

        f32x4 accu[QU][NTL], acco[QU][NTL];
        // (1) U = U~ - W H and O = Q_G H for this wave's chunk rows.
#pragma unroll
        for (int qu = 0; qu < QU; ++qu) {
            const int mt = wave + NW * qu;
            if (mt >= MT) continue;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const int tile = mt * (DV / 16) + sl * NTL + nt;
                accu[qu][nt] = *reinterpret_cast<const f32x4*>(blk + L::Ut + tile * 1024 + lane * 16);
                acco[qu][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) {
                const uint8_t* tw = blk + L::negW + (mt * KTH + kt) * 2048;
                const uint8_t* tq = blk + L::QG + (mt * KTH + kt) * 2048;
                const u32x4 awh = *reinterpret_cast<const u32x4*>(tw + lane * 16);
                const u32x4 awl = *reinterpret_cast<const u32x4*>(tw + 1024 + lane * 16);
                const u32x4 aqh = *reinterpret_cast<const u32x4*>(tq + lane * 16);
                const u32x4 aql = *reinterpret_cast<const u32x4*>(tq + 1024 + lane * 16);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const int off = (nt * 16 + l16) * HS + kt * 32 + lq * 8;
                    const u32x4 bh = *reinterpret_cast<const u32x4*>(&HThi[off]);
                    const u32x4 bl = *reinterpret_cast<const u32x4*>(&HTlo[off]);
                    accu[qu][nt] = mfma3(awh, awl, bh, bl, accu[qu][nt]);
                    acco[qu][nt] = mfma3(aqh, aql, bh, bl, acco[qu][nt]);
                }
            }
            // (2) U^T into LDS (split).
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) split_bf16(accu[qu][nt][i], hi[i], lo[i]);
                const int off = (nt * 16 + l16) * US + mt * 16 + lq * 4;
                *reinterpret_cast<uint2*>(&UThi[off]) =
                    make_uint2(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16));
                *reinterpret_cast<uint2*>(&UTlo[off]) =
                    make_uint2(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16));
            }
        }
        __syncthreads();
        // (3) O += P U, store valid rows.
#pragma unroll
        for (int qu = 0; qu < QU; ++qu) {
            const int mt = wave + NW * qu;
            if (mt >= MT) continue;
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                const uint8_t* tp = blk + L::P + (mt * KTC + kt) * 2048;
                const u32x4 aph = *reinterpret_cast<const u32x4*>(tp + lane * 16);
                const u32x4 apl = *reinterpret_cast<const u32x4*>(tp + 1024 + lane * 16);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const int off = (nt * 16 + l16) * US + kt * 32 + lq * 8;
                    const u32x4 bh = *reinterpret_cast<const u32x4*>(&UThi[off]);
                    const u32x4 bl = *reinterpret_cast<const u32x4*>(&UTlo[off]);
                    acco[qu][nt] = mfma3(aph, apl, bh, bl, acco[qu][nt]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = mt * 16 + lq * 4 + i;
                    if (r < Lc)
                        p.core[((t0 + r) * p.Hv + h) * DV + col0 + nt * 16 + l16] = acco[qu][nt][i];
                }
            }
        }
        // (4) H' = e^{gamma_last} H + K_d^T U.
        const float dec = p.decay[static_cast<int64_t>(c) * p.Hv + h];
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) {
            const int mth = wave + NW * qh;
            if (mth >= MTH) continue;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) hacc[qh][nt][i] *= dec;
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                const uint8_t* tk = blk + L::KdT + (mth * KTC + kt) * 2048;
                const u32x4 akh = *reinterpret_cast<const u32x4*>(tk + lane * 16);
                const u32x4 akl = *reinterpret_cast<const u32x4*>(tk + 1024 + lane * 16);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const int off = (nt * 16 + l16) * US + kt * 32 + lq * 8;
                    const u32x4 bh = *reinterpret_cast<const u32x4*>(&UThi[off]);
                    const u32x4 bl = *reinterpret_cast<const u32x4*>(&UTlo[off]);
                    hacc[qh][nt] = mfma3(akh, akl, bh, bl, hacc[qh][nt]);
                }
            }
        }
        // (5) H into LDS for the next chunk (all waves finished reading H in (1)).
        store_H_lds();
        __syncthreads();
    }

    // final state
    if (p.state_out) {
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) {
            const int mth = wave + NW * qh;
            if (mth >= MTH) continue;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mth * 16 + lq * 4 + i;
                    p.state_out[sbase + static_cast<size_t>(row) * DV + col0 + nt * 16 + l16] =
                        hacc[qh][nt][i];
                }
        }
    }
    // conv state tail: the last K-1 raw rows of (old conv state ++ inputs).
    // Slice 0 of each value head owns its v channels, and head h % G == 0
    // also owns its key head's q and k channels; one thread per channel reads
    // all taps before writing, so conv_state_out may alias conv_state_in.
    if (sl == 0 && p.conv_out) {
        using A = Act<BF16>;
        using T = typename A::T;
        const int qk = p.Hk * DK;
        const int Cc = 2 * qk + p.Hv * DV;
        const int hk = h / p.G;
        const int nch = DV + ((h % p.G == 0) ? 2 * DK : 0);
        T* cout = static_cast<T*>(p.conv_out);
        const T* cin = static_cast<const T*>(p.conv_in);
        for (int e = tid; e < nch; e += 256) {
            int cch, src_kind, src_off;   // 0 q, 1 k, 2 v
            if (e < DV) { cch = 2 * qk + h * DV + e; src_kind = 2; src_off = h * DV + e; }
            else if (e < DV + DK) { cch = hk * DK + (e - DV); src_kind = 0; src_off = hk * DK + (e - DV); }
            else { cch = qk + hk * DK + (e - DV - DK); src_kind = 1; src_off = hk * DK + (e - DV - DK); }
            T vals[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int64_t pos = end - 3 + r;
                T v = T(0);
                if (pos >= start) {
                    const T* base = src_kind == 0 ? static_cast<const T*>(p.q) + pos * p.qs
                                  : src_kind == 1 ? static_cast<const T*>(p.k) + pos * p.ks
                                                  : static_cast<const T*>(p.v) + pos * p.vs;
                    v = base[src_off];
                } else if (cin) {
                    const int64_t rr = 3 + (pos - start);
                    v = cin[(static_cast<int64_t>(n) * 3 + rr) * Cc + cch];
                }
                vals[r] = v;
            }
#pragma unroll
            for (int r = 0; r < 3; ++r) cout[(static_cast<int64_t>(n) * 3 + r) * Cc + cch] = vals[r];
        }
    }
}

// ---------------------------------------------------------------------------
// epilogue: out = norm_w (.) o / sqrt(mean(o^2) + eps) (.) SiLU(z); one wave
// per (token, value head) row, fixed-order reduction.
// ---------------------------------------------------------------------------
template <int DV, bool BF16>
__global__ __launch_bounds__(256) void epi_kernel(PrefillParams p) {
    using A = Act<BF16>;
    using T = typename A::T;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= p.T * p.Hv) return;
    const int64_t t = row / p.Hv;
    const int h = static_cast<int>(row % p.Hv);
    constexpr int PER = (DV + kWave - 1) / kWave;
    float o[PER];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int j = lane + kWave * m;
        o[m] = (j < DV) ? p.core[row * DV + j] : 0.f;
        ss = fmaf(o[m], o[m], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / DV + p.eps_rms);
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int j = lane + kWave * m;
        if (j >= DV) continue;
        const float zz = A::load(static_cast<const T*>(p.z) + t * p.zs + h * DV + j);
        const float y = p.norm_w[j] * (o[m] * r) * silu(zz);
        if (p.out_bf16) static_cast<uint16_t*>(p.out)[row * DV + j] = f32_to_bf16_bits(y);
        else static_cast<float*>(p.out)[row * DV + j] = y;
    }
}

// ---------------------------------------------------------------------------
template <int DK, int DV, int C, int DVS, bool BF16>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s,
                                   hipEvent_t const* ev) {
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (ev && e == hipSuccess) e = hipEventRecord(ev[i], s);
    };
    mark(0);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p.cu, p.N, C, p.chunk_off);
    mark(1);
    if (p.max_chunks > 0) {
        hipLaunchKernelGGL((prep_kernel<DK, DV, C, BF16>), dim3(p.max_chunks, p.Hk), dim3(256),
                           0, s, p);
    }
    mark(2);
    const int pairs = p.N * p.Hv;
    if (pairs > 0) {
        const int groups = (pairs + 7) / 8;
        hipLaunchKernelGGL((scan_kernel<DK, DV, C, DVS, BF16>), dim3(groups * 8 * (DV / DVS)),
                           dim3(256), 0, s, p);
    }
    mark(3);
    if (p.T > 0) {
        const int64_t rows = p.T * p.Hv;
        hipLaunchKernelGGL((epi_kernel<DV, BF16>), dim3(static_cast<unsigned>((rows + 3) / 4)),
                           dim3(256), 0, s, p);
    }
    mark(4);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

bool prefill_shape_supported(int DK, int DV, int C) {
    return (DK == 128 && DV == 128 && C == 64) || (DK == 32 && DV == 32 && C == 16) ||
           (DK == 32 && DV == 64 && C == 16);
}

hipError_t launch_prefill(int DK, int DV, int C, bool bf16, const PrefillParams& p,
                          hipStream_t s, bool* supported, hipEvent_t const* events) {
    *supported = true;
#define GDN_PF(dk, dv, c, dvs)                                                            \
    if (DK == dk && DV == dv && C == c)                                                   \
        return bf16 ? launch_prefill_t<dk, dv, c, dvs, true>(p, s, events)                \
                    : launch_prefill_t<dk, dv, c, dvs, false>(p, s, events);
    GDN_PF(128, 128, 64, 32)
    GDN_PF(32, 32, 16, 32)
    GDN_PF(32, 64, 16, 32)
#undef GDN_PF
    *supported = false;
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// self-test of the fragment layout: C = A B, A [16][32], B [32][16] row-major.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void selftest_mfma_kernel(const float* A, const float* B,
                                                           float* Cm) {
    const int l = threadIdx.x;
    uint16_t ah[8], al[8], bh[8], bl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = 8 * (l / 16) + e;
        split_bf16(A[(l % 16) * 32 + k], ah[e], al[e]);
        split_bf16(B[k * 16 + (l % 16)], bh[e], bl[e]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma3(pack8(ah), pack8(al), pack8(bh), pack8(bl), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) Cm[(4 * (l / 16) + i) * 16 + (l % 16)] = acc[i];
}

hipError_t launch_selftest_mfma(const float* A, const float* B, float* Cm, hipStream_t s) {
    hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, s, A, B, Cm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);
}

}  // namespace gdn
