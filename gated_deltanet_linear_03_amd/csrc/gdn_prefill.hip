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
//   prep_kernel   chunk-parallel over (chunk, one or two value heads of a
//                 key head); its first window also builds the chunk table
//                 (first chunk of every sequence): conv1d+SiLU, L2 norms, gates, Gram matrices, the
//                 diagonal blocks of (I + A)^{-1} and a block forward
//                 substitution for W and U~; writes the per-chunk operands
//                 -W, Q_G = diag(e^gamma) Q, K_d^T, P (fp16) and U~ (fp32) in
//                 matrix-core fragment order; see gdn_prep.hpp
//   scan_kernel   sequential over the chunks of one (sequence, value head,
//                 dv slice of 16 or 32 columns): U, O and H' on fp16
//                 matrix-core products, H kept in fp32 accumulators for the
//                 whole sequence; also writes the final state and the conv
//                 state tail
//   epi_kernel    token-parallel SiLU(z)-gated RMSNorm of o.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// Chunk table: chunk_off[n] = sum_{m<n} ceil(L_m / C), chunk_off[N] = total
// chunks (chunks restart at each sequence start, so results do not depend on
// the packing).  Each work-group of the first prep window derives the total
// and its own slot's sequence from cu_seqlens with a block-wide scan,
// checking on the way that cu_seqlens starts at 0, never decreases and ends
// at T_total and that pool entries lie in [0, num_slots) (every work-group
// reads the same values, so all reach the same verdict); the one given `out`
// also stores the table for the kernels after it.  `scratch`: NT / 64 + 2
// ints of LDS.
// ---------------------------------------------------------------------------
struct ChunkPos {
    int total;   // chunks of the batch
    int n;       // sequence owning the slot (when slot < total)
    int first;   // its first chunk
    bool bad;    // the indices broke their contract: nothing else is set
};

template <int NT>
__device__ ChunkPos chunk_table(const PrefillParams& p, int C, int slot, int32_t* scratch, int32_t* out) {
    constexpr int NW = NT / kWave;
    const int N = p.N;
    const int32_t* cu = p.cu;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int per = (N + NT - 1) / NT;
    const int n0 = min(N, tid * per), n1 = min(N, n0 + per);
    bool bad = tid == 0 && (cu[0] != 0 || static_cast<int64_t>(cu[N]) != p.T);
    int s = 0;
    for (int m = n0; m < n1; ++m) {
        const int32_t a = cu[m], b = cu[m + 1];
        bad |= b < a;
        if (p.slots) bad |= static_cast<unsigned>(p.slots[m]) >= static_cast<unsigned>(p.num_slots);
        s += (b - a + C - 1) / C;
    }
    int incl = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += u;
    }
    if (lane == kWave - 1) scratch[wave] = incl;
    ChunkPos r;
    r.bad = __syncthreads_or(bad);
    if (r.bad) return r;
    int acc = incl - s, total = 0;
    for (int w = 0; w < NW; ++w) {
        const int v = scratch[w];
        acc += w < wave ? v : 0;
        total += v;
    }
    for (int m = n0; m < n1; ++m) {
        const int c = (cu[m + 1] - cu[m] + C - 1) / C;
        if (out) out[m] = acc;
        if (acc <= slot && slot < acc + c) {
            scratch[NW] = m;
            scratch[NW + 1] = acc;
        }
        acc += c;
    }
    if (out && tid == 0) out[N] = total;
    __syncthreads();
    r.total = total;
    r.n = scratch[NW];
    r.first = scratch[NW + 1];
    return r;
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
// -W, Q_G, K_d^T and P are fp16 A fragments, 1 KiB per 16 x 32 tile (tile
// (m, k) at (m * ktiles + k) KiB); U~ is fp32 C/D fragments, 1 KiB per 16 x 16
// tile.
template <int DK, int DV, int C>
struct VchLayout {
    static constexpr int CK = ck_pad(C);
    static constexpr int64_t negW = 0;
    static constexpr int64_t QG = negW + 2ll * C * DK;
    static constexpr int64_t QGl = QG + 2ll * C * DK;       // lo parts, same tile order
    static constexpr int64_t KdT = QGl + 2ll * C * DK;
    static constexpr int64_t P = KdT + 2ll * DK * CK;
    static constexpr int64_t Pl = P + 2ll * C * CK;
    static constexpr int64_t Ut = Pl + 2ll * C * CK;
    static constexpr int64_t bytes = Ut + 4ll * C * DV;
    static_assert(bytes == vch_bytes(DK, DV, C), "layout");
};

}  // namespace gdn

#include "gdn_prep.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// scan: one work-group per (sequence, value head, dv slice of DVS columns),
// eight waves in two roles around the slice's state, shared through LDS:
//   state waves 0..3   U = U~ - W H for chunk-row tile `wave`, then
//                      H' = e^{gamma_last} H + K_d^T U for the H row tiles
//                      wave, wave + 4, ...  (registers, fp32)
//   output waves 4..7  O = Q_G H + P U for chunk-row tile `wave - 4`
// Per chunk:  [state: U -> LDS | output: Q_G H, all but its last k step]  barrier
//             [state: H' -> the other H^T buffer | output: last k step of
//              Q_G H, + P U, store O]  barrier.
// Only the state waves are on the chunk-to-chunk chain; the output products,
// their stores and their operand loads run beside it on the other wave of
// each SIMD.  H^T is double-buffered by chunk parity, so the output waves
// can read chunk c's copy in both halves of the step while the state waves
// write chunk c+1's.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 512;

// O16: the output waves store o as fp16 (the workspace copy the epilogue
// reads), else as fp32 (the caller's core_out).
template <int DK, int DV, int C, int DVS, bool BF16, bool O16>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(PrefillParams p) {
    using L = VchLayout<DK, DV, C>;
    constexpr int CK = L::CK;
    constexpr int NW = 4;                 // waves per role
    constexpr int NS = DV / DVS;          // slices per head
    constexpr int NTL = DVS / 16;         // n tiles per slice
    constexpr int MT = C / 16;            // U/O row tiles
    constexpr int MTH = DK / 16;          // H row tiles
    constexpr int KTH = DK / 32;          // k steps over dk
    constexpr int KTC = CK / 32;          // k steps over the chunk
    constexpr int QH = (MTH + NW - 1) / NW;
    constexpr int HS = DK + 8;            // LDS row stride (fp16) of H^T
    constexpr int US = CK + 8;            // LDS row stride (fp16) of U^T
    constexpr bool ALL_H = (MTH % NW) == 0;   // every state wave owns QH H row tiles
    static_assert(DV % DVS == 0 && DVS % 16 == 0 && DK % 32 == 0 && C % 16 == 0, "shape");
    static_assert(MT <= NW, "one chunk-row tile per wave");

    // the matrix-core copies of H^T and U^T as fp16 hi and lo parts (the
    // state itself stays in fp32 accumulators); the state chain uses the hi
    // parts, the output products both
    // H^T double-buffered by chunk parity: the state waves write chunk c+1's
    // copy while the output waves still read chunk c's
    __shared__ __align__(16) uint16_t HTb[2 * DVS * HS];
    __shared__ __align__(16) uint16_t HTlb[2 * DVS * HS];
    auto HT = [&](int c) { return HTb + (c & 1) * (DVS * HS); };
    auto HTl = [&](int c) { return HTlb + (c & 1) * (DVS * HS); };
    __shared__ __align__(16) uint16_t UT[DVS * US];
    __shared__ __align__(16) uint16_t UTl[DVS * US];

    // XCD-aware order: the NS slices of one head land on the same XCD
    // (consecutive work-groups are dealt round-robin over the 8 XCDs), so the
    // per-chunk operands they all read are shared in that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid % 8, j = bid / 8;
    const int sl = j % NS;
    const int pair = (j / NS) * 8 + xcd;
    if (pair >= p.N * p.Hv) return;
    if (p.chunk_off[p.N] < 0) return;      // the call's indices were rejected
    const int n = pair / p.Hv, h = pair % p.Hv;
    // this window's chunks of sequence n; a sequence without chunks passes
    // its states through in window 0
    const int cb = p.chunk_off[n], ce = p.chunk_off[n + 1];
    const bool no_chunks = cb == ce;
    const int c_begin = max(cb, p.win_lo), c_end = min(ce, p.win_hi);
    if (no_chunks ? p.win_idx != 0 : c_begin >= c_end) return;
    const bool seq_first = no_chunks || c_begin == cb;   // the sequence starts in this window
    const bool seq_last = no_chunks || c_end == ce;      // ... and ends in it

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int col0 = sl * DVS;
    const bool out_role = wave >= NW;
    const int mt = wave % NW;                 // chunk-row tile (U or O), if < MT
    const bool has_row = (MT >= NW) || mt < MT;

    // zero U^T (including the padded chunk rows C..CK-1, never written later)
    for (int i = tid; i < DVS * US; i += kScanThreads) {
        UT[i] = 0;
        UTl[i] = 0;
    }

    // entering state: the caller's initial state where the sequence starts,
    // else what the previous window left in the carry slot of its parity
    const int sn = state_slot(p.slots, n);                 // pool entry of the states
    const size_t sbase = (static_cast<size_t>(sn) * p.Hv + h) * DK * DV;
    const size_t cbase = static_cast<size_t>(h) * DK * DV;
    const size_t cslot = static_cast<size_t>(p.Hv) * DK * DV;
    const float* hin = seq_first ? (p.state_in ? p.state_in + sbase : nullptr)
                                 : p.carry + ((p.win_idx - 1) & 1) * cslot + cbase;
    float* hout = seq_last ? (p.state_out ? p.state_out + sbase : nullptr)
                           : p.carry + (p.win_idx & 1) * cslot + cbase;

    // H slice in accumulator fragments of the state waves: tile
    // (mth = wave + NW*qh, nt)
    f32x4 hacc[QH][NTL];
    auto store_H_lds = [&](int c) {      // H entering chunk c
        uint16_t* ht = HT(c);
        uint16_t* htl = HTl(c);
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) {
            const int mth = wave + NW * qh;
            if (!ALL_H && mth >= MTH) continue;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const int off = (nt * 16 + l16) * HS + mth * 16 + lq * 4;
                uint2 hi, lo;
                split4_f16(hacc[qh][nt], hi, lo);
                *reinterpret_cast<uint2*>(&ht[off]) = hi;
                *reinterpret_cast<uint2*>(&htl[off]) = lo;
            }
        }
    };
    if (!out_role) {
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) {
            const int mth = wave + NW * qh;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (mth < MTH && hin) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = mth * 16 + lq * 4 + i;
                        v[i] = hin[static_cast<size_t>(row) * DV + col0 + nt * 16 + l16];
                    }
                }
                hacc[qh][nt] = v;
            }
        }
        store_H_lds(c_begin);
    }
    __syncthreads();

    const int64_t start = p.cu[n], end = p.cu[n + 1];
    auto block_of = [&](int c) {
        return p.vch + (static_cast<int64_t>(c - p.win_lo) * p.Hv + h) * L::bytes;
    };
    // B fragments of H^T (k over dk) and of U^T (k over the chunk) from LDS
    auto read_H = [&](const uint16_t* ht, int kt, u32x4* b) {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
            b[nt] = *reinterpret_cast<const u32x4*>(&ht[(nt * 16 + l16) * HS + kt * 32 + lq * 8]);
    };
    auto read_U = [&](const uint16_t* ut, u32x4 (*ub)[NTL]) {
#pragma unroll
        for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                ub[kt][nt] = *reinterpret_cast<const u32x4*>(&ut[(nt * 16 + l16) * US + kt * 32 + lq * 8]);
    };
    // one lane's 16 bytes of a 1 KiB fp16 fragment tile
    auto frag = [&](const uint8_t* tile) { return *reinterpret_cast<const u32x4*>(tile + lane * 16); };

    if (!out_role) {
        // ---------------- state waves ----------------
        // they are the chain: raised issue priority lets their dependent
        // instructions win the SIMD over the output wave sharing it
        __builtin_amdgcn_s_setprio(3);
        // Three operand sets in registers, rotated: chunk c+2's fragments
        // load while chunk c computes (W's per k step between the products,
        // K_d^T's after the state update), two chunk steps ahead of use.
        struct Ops {
            u32x4 w[KTH];
            f32x4 ut[NTL];
            u32x4 k[QH][KTC];
            float dec;
        };
        auto load_w = [&](Ops& o, int c, int kt) {
            const uint8_t* blk = block_of(c);
            if (kt == 0) {
                o.dec = p.decay[static_cast<int64_t>(c) * p.Hv + h];
                if (has_row) {
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) {
                        const int tile = mt * (DV / 16) + sl * NTL + nt;
                        o.ut[nt] = *reinterpret_cast<const f32x4*>(blk + L::Ut + tile * 1024 + lane * 16);
                    }
                }
            }
            if (has_row) o.w[kt] = frag(blk + L::negW + (mt * KTH + kt) * 1024);
        };
        auto load_k = [&](Ops& o, int c) {
            const uint8_t* blk = block_of(c);
#pragma unroll
            for (int qh = 0; qh < QH; ++qh) {
                const int mth = wave + NW * qh;
                if (!ALL_H && mth >= MTH) continue;
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt)
                    o.k[qh][kt] = frag(blk + L::KdT + (mth * KTC + kt) * 1024);
            }
        };
        auto step = [&](Ops& cur, Ops& nxt, int c, int cn) {
            // (1) U = U~ - W H for this wave's chunk rows; even and odd k
            // steps accumulate separately (two independent chains)
            f32x4 a0[NTL], a1[NTL];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                a0[nt] = cur.ut[nt];
                a1[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) {
                load_w(nxt, cn, kt);
                if (!has_row) continue;
                u32x4 b[NTL];
                read_H(HT(c), kt, b);
                f32x4* a = (kt & 1) ? a1 : a0;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) a[nt] = mfma_h(cur.w[kt], b[nt], a[nt]);
            }
            if (has_row) {
                // (2) U^T into LDS
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    f32x4 u;
#pragma unroll
                    for (int i = 0; i < 4; ++i) u[i] = a0[nt][i] + a1[nt][i];
                    uint2 hi, lo;
                    split4_f16(u, hi, lo);
                    *reinterpret_cast<uint2*>(&UT[(nt * 16 + l16) * US + mt * 16 + lq * 4]) = hi;
                    *reinterpret_cast<uint2*>(&UTl[(nt * 16 + l16) * US + mt * 16 + lq * 4]) = lo;
                }
            }
            __syncthreads();
            // (3) H' = e^{gamma_last} H + K_d^T U
            u32x4 ub[KTC][NTL];
            read_U(UT, ub);
#pragma unroll
            for (int qh = 0; qh < QH; ++qh) {
                if (!ALL_H && wave + NW * qh >= MTH) continue;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) hacc[qh][nt][i] *= cur.dec;
            }
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
#pragma unroll
                for (int qh = 0; qh < QH; ++qh) {
                    if (!ALL_H && wave + NW * qh >= MTH) continue;
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) hacc[qh][nt] = mfma_h(cur.k[qh][kt], ub[kt][nt], hacc[qh][nt]);
                }
            }
            // (4) H' into LDS for the next chunk, in the other buffer (the
            // output waves read this chunk's until the step's last barrier)
            store_H_lds(c + 1);
            load_k(nxt, cn);
            __syncthreads();
        };

        Ops opA, opB, opC;
        if (c_begin < c_end) {
            const int c1 = min(c_begin + 1, c_end - 1);
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) load_w(opA, c_begin, kt);
            load_k(opA, c_begin);
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) load_w(opB, c1, kt);
            load_k(opB, c1);
        }
        // drain the memory counter once before the loop, so the loop's waits
        // are set by its own steady-state load/store order
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // at the top of each round opA holds chunk c and opB chunk c + 1;
        // loads past the window's last chunk repeat that chunk (unused)
        int c = c_begin;
        for (; c + 2 < c_end; c += 3) {
            step(opA, opC, c, c + 2);
            step(opB, opA, c + 1, min(c + 3, c_end - 1));
            step(opC, opB, c + 2, min(c + 4, c_end - 1));
        }
        if (c < c_end) step(opA, opC, c, c_end - 1);
        if (c + 1 < c_end) step(opB, opA, c + 1, c_end - 1);

        // leaving state
        if (hout) {
            bool bad = false;
#pragma unroll
            for (int qh = 0; qh < QH; ++qh) {
                const int mth = wave + NW * qh;
                if (mth >= MTH) continue;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = mth * 16 + lq * 4 + i;
                        hout[static_cast<size_t>(row) * DV + col0 + nt * 16 + l16] = hacc[qh][nt][i];
                        bad |= !isfinite(hacc[qh][nt][i]);
                    }
            }
            // a non-finite final state is reported too
            if (seq_last) flag_nonfinite(p.status, bad);
        }
    } else {
        // ---------------- output waves ----------------
        struct Ops {
            u32x4 q[KTH], ql[KTH];
            u32x4 p[KTC], pl[KTC];
        };
        auto load_q = [&](Ops& o, int c, int kt) {
            if (!has_row) return;
            const uint8_t* blk = block_of(c);
            o.q[kt] = frag(blk + L::QG + (mt * KTH + kt) * 1024);
            o.ql[kt] = frag(blk + L::QGl + (mt * KTH + kt) * 1024);
        };
        // P tiles wholly above the diagonal (first column past the tile's
        // last row) are zero: prep does not write them and they are neither
        // loaded nor multiplied
        auto p_tile = [&](int kt) { return kt * 32 <= mt * 16 + 15; };
        auto load_p = [&](Ops& o, int c) {
            if (!has_row) return;
            const uint8_t* blk = block_of(c);
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                if (!p_tile(kt)) continue;
                o.p[kt] = frag(blk + L::P + (mt * KTC + kt) * 1024);
                o.pl[kt] = frag(blk + L::Pl + (mt * KTC + kt) * 1024);
            }
        };
        // o rows of this lane: element offset of (row mt*16 + 4 lq, column l16)
        // from a chunk's first row, and the stride between token rows
        const int64_t rstride = static_cast<int64_t>(p.Hv) * DV;
        const int64_t lane_off = (mt * 16 + lq * 4) * rstride + l16;
        auto step = [&](Ops& cur, Ops& nxt, int c, int cn) {
            const int64_t t0 = start + static_cast<int64_t>(c - cb) * C;
            const int Lc = static_cast<int>(min(static_cast<int64_t>(C), end - t0));
            // (1) O = Q_G H (even / odd k steps apart, as for U)
            f32x4 a0[NTL], a1[NTL];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                a0[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                a1[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // the last k step of Q_G H waits for the step's second half, so
            // that each half carries about the same matrix-core work
            auto qh_step = [&](int kt) {
                load_q(nxt, cn, kt);
                if (!has_row) return;
                u32x4 b[NTL], bl[NTL];
                read_H(HT(c), kt, b);
                read_H(HTl(c), kt, bl);
                f32x4* a = (kt & 1) ? a1 : a0;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) a[nt] = mfma_h3(cur.q[kt], cur.ql[kt], b[nt], bl[nt], a[nt]);
            };
#pragma unroll
            for (int kt = 0; kt < KTH - 1; ++kt) qh_step(kt);
            __syncthreads();
            qh_step(KTH - 1);
            f32x4 acco[NTL];
            if (has_row) {
                // (2) O += P U; the valid rows are stored after the barrier
                u32x4 ub[KTC][NTL], ubl[KTC][NTL];
                read_U(UT, ub);
                read_U(UTl, ubl);
                load_p(nxt, cn);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acco[nt][i] = a0[nt][i] + a1[nt][i];
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) {
                    if (!p_tile(kt)) continue;
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt)
                        acco[nt] = mfma_h3(cur.p[kt], cur.pl[kt], ub[kt][nt], ubl[kt][nt], acco[nt]);
                }
            }
            // the step's last barrier first: the state waves need not wait
            // for the conversions and stores below, which then overlap the
            // next step's first half
            __syncthreads();
            if (has_row) {
                // a full chunk stores at a per-chunk base plus this lane's
                // offset; in a partial one, rows past the sequence end go to
                // a sink, so that every lane issues the same stores (the
                // memory counter the next chunk's operand waits rely on then
                // counts them exactly).  The workspace copy for the epilogue
                // is fp16 (half the bytes out and back); a caller's core_out
                // gets fp32.  Non-temporal: o is read again only by the
                // epilogue after the last window, and should not evict the
                // operand blocks the next steps read.
                const int64_t cofs = (t0 * p.Hv + h) * DV + col0;
                auto store_o = [&](auto* cbase, auto* sink, auto cvt) {
                    if (Lc == C) {
#pragma unroll
                        for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(cvt(acco[nt][i]), cbase + lane_off + i * rstride + nt * 16);
                    } else {
#pragma unroll
                        for (int nt = 0; nt < NTL; ++nt) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = mt * 16 + lq * 4 + i;
                                auto* dst = r < Lc ? cbase + lane_off + i * rstride + nt * 16 : sink;
                                __builtin_nontemporal_store(cvt(acco[nt][i]), dst);
                            }
                        }
                    }
                };
                if constexpr (O16)
                    store_o(reinterpret_cast<uint16_t*>(p.core) + cofs, reinterpret_cast<uint16_t*>(p.sink) + lane,
                            [](float x) { return f32_to_f16_bits(x); });
                else
                    store_o(p.core + cofs, p.sink + lane, [](float x) { return x; });
            }
        };

        Ops opA, opB, opC;
        if (c_begin < c_end) {
            const int c1 = min(c_begin + 1, c_end - 1);
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) load_q(opA, c_begin, kt);
            load_p(opA, c_begin);
#pragma unroll
            for (int kt = 0; kt < KTH; ++kt) load_q(opB, c1, kt);
            load_p(opB, c1);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        int c = c_begin;
        for (; c + 2 < c_end; c += 3) {
            step(opA, opC, c, c + 2);
            step(opB, opA, c + 1, min(c + 3, c_end - 1));
            step(opC, opB, c + 2, min(c + 4, c_end - 1));
        }
        if (c < c_end) step(opA, opC, c, c_end - 1);
        if (c + 1 < c_end) step(opB, opA, c + 1, c_end - 1);
    }

    // conv state tail: the last K-1 raw rows of (old conv state ++ inputs).
    // Slice 0 of each value head owns its v channels, and head h % G == 0
    // also owns its key head's q and k channels; one thread per channel reads
    // all taps before writing, so conv_state_out may alias conv_state_in.
    if (seq_last && sl == 0 && p.conv_out) {
        using A = Act<BF16>;
        using T = typename A::T;
        const int qk = p.Hk * DK;
        const int Cc = 2 * qk + p.Hv * DV;
        const int hk = h / p.G;
        const int nch = DV + ((h % p.G == 0) ? 2 * DK : 0);
        T* cout = static_cast<T*>(p.conv_out);
        const T* cin = static_cast<const T*>(p.conv_in);
        for (int e = tid; e < nch; e += kScanThreads) {
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
                    v = cin[(static_cast<int64_t>(sn) * 3 + rr) * Cc + cch];
                }
                vals[r] = v;
            }
#pragma unroll
            for (int r = 0; r < 3; ++r) cout[(static_cast<int64_t>(sn) * 3 + r) * Cc + cch] = vals[r];
        }
    }
}

// ---------------------------------------------------------------------------
// epilogue: out = norm_w (.) o / sqrt(mean(o^2) + eps) (.) SiLU(z); one wave
// per (token, value head) row, fixed-order reduction.
// ---------------------------------------------------------------------------
// DV/4 lanes per (token, head) row, 16-byte accesses, fixed-order reduction
// over the row's lanes.
template <int DV>
struct EpiGeom {
    static constexpr int LPR = DV / 4;                 // lanes per row
    static constexpr int RPB = 256 / LPR;              // rows per 256-thread block
    static_assert(DV % 4 == 0 && LPR <= kWave && kWave % LPR == 0, "row geometry");
};

// O16: o comes as fp16 (the scan's workspace copy), else as the caller's
// fp32 core_out, rounded to fp16 here the same way so that `out` has the
// same bits either way (a template argument, not a branch: the o and z
// loads must both be in flight before the first wait).
template <int DV, bool BF16, bool O16>
__global__ __launch_bounds__(256) void epi_kernel(PrefillParams p) {
    using G = EpiGeom<DV>;
    const int lr = threadIdx.x % G::LPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * G::RPB + threadIdx.x / G::LPR;
    const bool valid = row < p.T * p.Hv;
    const int64_t rr = valid ? row : 0;
    const int64_t t = rr / p.Hv;
    const int h = static_cast<int>(rr % p.Hv);
    float o[4];
    if constexpr (O16) {
        const uint2 oo = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.core) + rr * DV + 4 * lr);
        o[0] = f16_bits_to_f32(static_cast<uint16_t>(oo.x));
        o[1] = f16_bits_to_f32(static_cast<uint16_t>(oo.x >> 16));
        o[2] = f16_bits_to_f32(static_cast<uint16_t>(oo.y));
        o[3] = f16_bits_to_f32(static_cast<uint16_t>(oo.y >> 16));
    } else {
        const f32x4 oo = *reinterpret_cast<const f32x4*>(p.core + rr * DV + 4 * lr);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f16_bits_to_f32(f32_to_f16_bits(oo[e]));
    }
    float z[4];
    if constexpr (BF16) {
        const uint2 zz = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.z) + t * p.zs + h * DV + 4 * lr);
        z[0] = __uint_as_float(zz.x << 16);
        z[1] = __uint_as_float(zz.x & 0xFFFF0000u);
        z[2] = __uint_as_float(zz.y << 16);
        z[3] = __uint_as_float(zz.y & 0xFFFF0000u);
    } else {
        const f32x4 zz = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.z) + t * p.zs + h * DV + 4 * lr);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = zz[e];
    }
    const f32x4 w = *reinterpret_cast<const f32x4*>(p.norm_w + 4 * lr);
    float ss = o[0] * o[0];
    ss = fmaf(o[1], o[1], ss);
    ss = fmaf(o[2], o[2], ss);
    ss = fmaf(o[3], o[3], ss);
    if constexpr (G::LPR <= 16) {
        ss = group_sum<G::LPR>(ss);
    } else {
        ss = group_sum<16>(ss);
#pragma unroll
        for (int off = 16; off < G::LPR; off <<= 1) ss += __shfl_xor(ss, off, kWave);
    }
    const float r = 1.0f / sqrtf(ss / DV + p.eps_rms);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = w[e] * (o[e] * r) * silu(z[e]);
    // nothing is written when the call's indices were rejected (o was not
    // computed); the flag is read here, after the loads were issued, so that
    // they do not wait for it
    const bool ok = p.chunk_off[p.N] >= 0;
    // a non-finite output (with finite inputs: the scan's fp16 operand range
    // exceeded upstream) is reported, never passed on silently
    flag_nonfinite(p.status, ok && valid && !(isfinite(y[0]) && isfinite(y[1]) && isfinite(y[2]) && isfinite(y[3])));
    if (!valid || !ok) return;
    if (p.out_bf16) {
        uint2 v;
        v.x = f32_to_bf16_bits(y[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(y[1])) << 16);
        v.y = f32_to_bf16_bits(y[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(y[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + row * DV + 4 * lr) = v;
    } else {
        // out is not read again here: streamed past the caches
        __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]},
                                    reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + row * DV + 4 * lr));
    }
}

// ---------------------------------------------------------------------------
// Compute units of the current device (cached per device).
int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();          // no device here: plan for 256
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// The scan runs one work-group per compute unit (its registers admit one),
// so it uses the narrow slice DVS when the (sequence, head, slice) groups
// fit in one round over the compute units, else the wide one DVSW (less
// operand traffic per column).  Each output column's arithmetic does not
// depend on the slicing, so results are the same bits either way.
template <int DK, int DV, int C, int DVS, int DVSW, bool BF16>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s,
                                   hipEvent_t const* ev) {
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (ev && e == hipSuccess) e = hipEventRecord(ev[i], s);
    };
    int ev_i = 0;
    mark(ev_i++);
    // windows of chunk slots: prep writes a window's operand blocks, scan
    // consumes them while they are still cache-resident, then the next
    // window reuses the blocks
    const int W = p.win_slots;
    const int nwin = static_cast<int>(prefill_launches(p.max_chunks, W) - 1) / 2;
    const int pairs = p.N * p.Hv;
    for (int w = 0; w < nwin; ++w) {
        PrefillParams q = p;
        q.win_idx = w;
        q.win_lo = w * W;
        q.win_hi = min(p.max_chunks, (w + 1) * W);
        // the first window runs even without chunks: it writes the chunk table
        const int gx = max(q.win_hi - q.win_lo, w == 0 ? 1 : 0);
        if (gx > 0) {
            // value heads in pairs when each key head has an even number of them
            if (p.G % 2 == 0)
                hipLaunchKernelGGL((prep_kernel<DK, DV, C, 2, BF16>), dim3(gx, p.Hv / 2),
                                   dim3(kPrepThreads), 0, s, q);
            else
                hipLaunchKernelGGL((prep_kernel<DK, DV, C, 1, BF16>), dim3(gx, p.Hv),
                                   dim3(kPrepThreads), 0, s, q);
        }
        mark(ev_i++);
        if (pairs > 0) {
            const int groups = (pairs + 7) / 8;
            const bool narrow = static_cast<int64_t>(groups) * 8 * (DV / DVS) <= compute_units();
            const dim3 grid(groups * 8 * (DV / (narrow ? DVS : DVSW)));
            if (narrow && p.core_f16)
                hipLaunchKernelGGL((scan_kernel<DK, DV, C, DVS, BF16, true>), grid, dim3(kScanThreads), 0, s, q);
            else if (narrow)
                hipLaunchKernelGGL((scan_kernel<DK, DV, C, DVS, BF16, false>), grid, dim3(kScanThreads), 0, s, q);
            else if (p.core_f16)
                hipLaunchKernelGGL((scan_kernel<DK, DV, C, DVSW, BF16, true>), grid, dim3(kScanThreads), 0, s, q);
            else
                hipLaunchKernelGGL((scan_kernel<DK, DV, C, DVSW, BF16, false>), grid, dim3(kScanThreads), 0, s, q);
        }
        mark(ev_i++);
    }
    if (p.T > 0) {
        const int64_t rows = p.T * p.Hv;
        constexpr int RPB = EpiGeom<DV>::RPB;
        const dim3 grid(static_cast<unsigned>((rows + RPB - 1) / RPB));
        if (p.core_f16)
            hipLaunchKernelGGL((epi_kernel<DV, BF16, true>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((epi_kernel<DV, BF16, false>), grid, dim3(256), 0, s, p);
    }
    mark(ev_i++);
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
#define GDN_PF(dk, dv, c, dvs, dvsw)                                                      \
    if (DK == dk && DV == dv && C == c)                                                   \
        return bf16 ? launch_prefill_t<dk, dv, c, dvs, dvsw, true>(p, s, events)          \
                    : launch_prefill_t<dk, dv, c, dvs, dvsw, false>(p, s, events);
    GDN_PF(128, 128, 64, 16, 32)
    GDN_PF(32, 32, 16, 16, 32)
    GDN_PF(32, 64, 16, 16, 32)
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
    // the same product as two k = 16 halves on v_mfma_f32_16x16x16_bf16
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 16 * half + 4 * (l / 16) + e;
            a[e] = A[(l % 16) * 32 + k];
            b[e] = B[k * 16 + (l % 16)];
        }
        uint2 a_h, a_l, b_h, b_l;
        split4(a, a_h, a_l);
        split4(b, b_h, b_l);
        acc2 = mfma3_k16(a_h, a_l, b_h, b_l, acc2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Cm[256 + (4 * (l / 16) + i) * 16 + (l % 16)] = acc2[i];
    // A and B rounded once to fp16, one v_mfma_f32_16x16x32_f16
    float a8[8], b8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = 8 * (l / 16) + e;
        a8[e] = A[(l % 16) * 32 + k];
        b8[e] = B[k * 16 + (l % 16)];
    }
    const f32x4 acc3 = mfma_h(pack8_f16(a8), pack8_f16(b8), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int i = 0; i < 4; ++i) Cm[512 + (4 * (l / 16) + i) * 16 + (l % 16)] = acc3[i];
}

hipError_t launch_selftest_mfma(const float* A, const float* B, float* Cm, hipStream_t s) {
    hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, s, A, B, Cm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);
}

}  // namespace gdn
