// gdn_decode.hip -- one-token Gated DeltaNet step against carried state.
//
// One work-group per (sequence b, key head hk) handles the key head's conv,
// its L2 norms, and every value head h = hk*G + g of its group.  Grouping by
// key head lets each conv channel be owned by exactly one thread of the grid,
// so the conv state may be updated in place; each state element is likewise
// read and rewritten by one thread, so the recurrent state may be updated in
// place too.
//
// The state of one value head is H = S^T [dk][dv] fp32 (dv fastest).  With
// u = beta (v - e^g S k) and S_t = e^g S + u k^T (the gated delta rule of
// Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025, rewritten by
// distributivity), one token needs
//     r_k = H^T k^,  r_q = H^T q^          (one streaming read of H)
//     u   = beta (v~ - e^g r_k),  o = e^g r_q + (k^.q^) u
//     H' = e^g H + k^ u^T                  (one streaming write)
// so the step is a pure HBM stream of 2 x dk x dv x 4 bytes per head; the
// fixed state size per sequence is the one the llmxabe README's model
// section gives (~60 MiB over 30 layers, i.e. 2 MiB per layer).
//
// The work-group has 512 threads: each half streams one value head of the
// group, so the two heads' state loads, arithmetic and stores overlap.
//
// The same kernel applies up to kMaxVerifyTokens tokens per sequence in one
// launch (multi-token verify of speculative decoding): the state is read
// once, updated token by token in registers with the one-token arithmetic,
// optionally written after every token (snapshots for rollback) and written
// once at the end.
// Thread layout over H: DV/4 column groups (one float4 each) x RG row groups;
// thread (rg, cg) holds a block of DK/RG consecutive rows.  Loads of one
// instruction cover whole 512-byte rows, so the stream is fully coalesced.  Column sums over the row
// groups are combined through LDS in a fixed order, so the result does not
// depend on the batch: a sequence is bit-identical batched or alone (llmxabe
// README, "Status").
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

constexpr int kDecodeHalf = 256;                 // threads per value head
constexpr int kDecodeThreads = 2 * kDecodeHalf;  // two value heads stream at once

// z-gated RMSNorm of one value head's o over dv, shared by the one-token and
// the multi-token kernels so that both give the same bits: lane t < DV/4 of one wave holds
// columns 4t..4t+3 of o and of z; the sum of squares is the lane's four
// terms in a fixed order, then the wave sum.  Stores y to out (bf16 or fp32)
// and, when core is given, o to core.
template <int DV>
__device__ __forceinline__ void gated_rmsnorm_store(int t, const f32x4& o, const float* z,
                                                    const float* norm_w, float eps, void* out,
                                                    int out_bf16, float* core, size_t obase) {
    constexpr int CG = DV / 4;
    float ps = 0.f;
    if (t < CG) ps = fmaf(o[3], o[3], fmaf(o[2], o[2], fmaf(o[1], o[1], o[0] * o[0])));
    ps = wave_sum(ps);
    if (t >= CG) return;
    const float r = 1.0f / sqrtf(ps / DV + eps);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = norm_w[4 * t + e] * (o[e] * r) * silu(z[e]);
    if (out_bf16) {
        uint16_t* op = static_cast<uint16_t*>(out) + obase;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = f32_to_bf16_bits(y[e]);
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + obase) = f32x4{y[0], y[1], y[2], y[3]};
    }
    if (core) *reinterpret_cast<f32x4*>(core + obase) = o;
}

// conv1d (K = 4) + SiLU of one channel: oldest tap first, the token last
__device__ __forceinline__ float conv4_silu(const f32x4& w, float t0, float t1, float t2, float x) {
    float acc = w[0] * t0;
    acc = fmaf(w[1], t1, acc);
    acc = fmaf(w[2], t2, acc);
    acc = fmaf(w[3], x, acc);
    return silu(acc);
}

// 1 / sqrt(sum of squares + eps) times num, over DK values in LDS: lane l
// sums entries l, l + 64, ... in order, then the wave sum (every lane of the
// wave takes part)
template <int DK>
__device__ __forceinline__ float l2_sumsq(const float* src, int lane) {
    float ss = 0.f;
    for (int i = lane; i < DK; i += kWave) ss = fmaf(src[i], src[i], ss);
    return ss;
}
__device__ __forceinline__ float l2_finish(float ss, float num, float eps) { return num / sqrtf(ss + eps); }
template <int DK>
__device__ __forceinline__ float l2_scale(const float* src, int lane, float num, float eps) {
    return l2_finish(wave_sum(l2_sumsq<DK>(src, lane)), num, eps);
}

// k^ . q^ over DK values in LDS, in the same lane order
template <int DK>
__device__ __forceinline__ float dot_wave(const float* a, const float* b, int lane) {
    float d = 0.f;
    for (int i = lane; i < DK; i += kWave) d = fmaf(a[i], b[i], d);
    return wave_sum(d);
}

// One-token step.  A work-group holds HPW value heads of one key head (256
// threads per value head):
//   HPW = 2  one work-group per (sequence, key head); the key head's value
//            heads two at a time.  It alone reads and rewrites the key head's
//            q/k conv channels.
//   HPW = 1  one work-group per (sequence, value head), so a small batch
//            spreads its state stream over twice as many compute units.  The
//            G work-groups of a key head all read its q/k conv history; the
//            last of them to count itself in on a per-(sequence, key head)
//            arrival counter (decode workspace) writes the new history and
//            puts the counter back to zero.  Nothing waits on another
//            work-group, and no result passes between them.
// Both compute each value head with the same operations in the same order,
// so they give the same bits.  With HPW = 1 the conv and gate inputs are
// loaded before the state stream (loads complete in issue order), so the
// conv, the gates and the L2 norms run while the state arrives; with HPW = 2
// the conv runs before the stream is issued.
template <int DK, int DV, bool BF16, int HPW>
__global__ __launch_bounds__(HPW * kDecodeHalf, 4) void decode_kernel(DecodeParams p) {
    using A = Act<BF16>;
    using T = typename A::T;
    constexpr int NT = kDecodeHalf;
    constexpr int NTH = HPW * NT;
    constexpr int CG = DV / 4;          // float4 column groups
    constexpr int RG = NT / CG;         // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    static_assert(CG <= 64 && NT % CG == 0 && DK % RG == 0 && RPT >= 1, "shape");
    static_assert(HPW == 1 || HPW == 2, "one or two value heads per work-group");

    __shared__ float sq[DK], sk[DK], sv[HPW][DV], sz[HPW][DV];
    __shared__ f32x4 red_k[HPW][RG][CG], red_q[HPW][RG][CG];
    __shared__ float s_eg[HPW], s_beta[HPW];
    __shared__ T s_tap[HPW == 1 ? 3 : 1][HPW == 1 ? 2 * DK : 1];   // new q/k history (HPW = 1)

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    int b, hk, gfirst, gend;
    if constexpr (HPW == 1) {
        b = blockIdx.x / p.Hv;
        const int h = blockIdx.x % p.Hv;
        hk = h / p.G;
        gfirst = h % p.G;
        gend = gfirst + 1;
    } else {
        b = blockIdx.x / p.Hk;
        hk = blockIdx.x % p.Hk;
        gfirst = 0;
        gend = p.G;
    }
    // value head slot (uniform per wave, so the state base lives in SGPRs)
    const int half = HPW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / NT);
    const int t = tid % NT;
    const int Cc = 2 * p.Hk * DK + p.Hv * DV;
    const T* cin = static_cast<const T*>(p.conv_in);
    T* cout = static_cast<T*>(p.conv_out);
    const int sb = state_slot(p.slots, b);                // pool entry of the states
    if (p.slots && static_cast<unsigned>(sb) >= static_cast<unsigned>(p.num_slots)) {
        // an entry outside the pool: the sequence is skipped (nothing read
        // or written for it, no arrival counted) and reported
        if (tid == 0 && p.status)
            __hip_atomic_fetch_or(p.status, kStatusBadIndex, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const size_t crow = static_cast<size_t>(sb) * 3 * Cc;

    // ---- conv and gate inputs ----
    // Each thread takes at most one q/k channel (threads [0, 2 DK)) and one
    // v channel (threads [VOFF, VOFF + HPW DV)).  The loads are issued
    // unconditionally from clamped indices and the raw values kept until
    // the conv, so that issuing them never waits on memory; with no conv
    // history the tap loads read channel 0 of q instead and are zeroed at use.
    constexpr int VOFF = NTH >= 2 * DK + HPW * DV ? 2 * DK : 0;
    static_assert(VOFF + HPW * DV <= NTH && 2 * DK <= NTH, "one q/k and one v channel per thread");
    const bool has_qk = tid < 2 * DK;
    const int qc = has_qk ? tid : 0;
    // whether the channel is a k channel: wave-uniform when DK is a multiple
    // of the wave, so the choice of source is a scalar select
    const bool isk = DK % kWave == 0 ? __builtin_amdgcn_readfirstlane(qc >= DK) != 0 : qc >= DK;
    const int qi = qc - (isk ? DK : 0);
    const int c_qk = (isk ? p.Hk * DK : 0) + hk * DK + qi;
    const T* const hist = cin ? cin : static_cast<const T*>(p.q);
    // all-ones with a conv history, else zero: tap indices collapse to 0
    const size_t hmask = cin ? ~size_t(0) : size_t(0);
    T xqk, tqk0, tqk1, tqk2, xv, tv0, tv1, tv2, zv, av, bv;
    f32x4 wqk, wv;
    float alog, dtb;
    auto conv_loads = [&](int g0, bool with_qk) {
        if (with_qk) {
            const T* src = isk ? static_cast<const T*>(p.k) + b * p.ks : static_cast<const T*>(p.q) + b * p.qs;
            xqk = src[hk * DK + qi];
            tqk0 = hist[(crow + c_qk) & hmask];
            tqk1 = hist[(crow + Cc + c_qk) & hmask];
            tqk2 = hist[(crow + 2 * Cc + c_qk) & hmask];
            wqk = *reinterpret_cast<const f32x4*>(p.conv_w + static_cast<size_t>(c_qk) * 4);
        }
        const int vc = min(max(tid - VOFF, 0), HPW * DV - 1);
        const int vh = vc / DV, j = vc % DV;
        const int h = hk * p.G + (g0 + vh < gend ? g0 + vh : g0);
        const int c = 2 * p.Hk * DK + h * DV + j;
        xv = static_cast<const T*>(p.v)[b * p.vs + h * DV + j];
        tv0 = hist[(crow + c) & hmask];
        tv1 = hist[(crow + Cc + c) & hmask];
        tv2 = hist[(crow + 2 * Cc + c) & hmask];
        wv = *reinterpret_cast<const f32x4*>(p.conv_w + static_cast<size_t>(c) * 4);
        zv = static_cast<const T*>(p.z)[b * p.zs + h * DV + j];
        av = static_cast<const T*>(p.a)[b * p.as + h];
        bv = static_cast<const T*>(p.b)[b * p.bs + h];
        alog = p.A_log[h];
        dtb = p.dt_bias[h];
    };
    // conv + SiLU into LDS, the gates, and the new conv history (q/k
    // channels: with HPW = 2 here, by their single owner; with HPW = 1 into
    // LDS, for the last of the key head's work-groups)
    auto conv_compute = [&](int g0, bool with_qk) {
        auto ld = [&](const T& x) { return cin ? A::load(&x) : 0.f; };
        if (with_qk && has_qk) {
            const float y = conv4_silu(wqk, ld(tqk0), ld(tqk1), ld(tqk2), A::load(&xqk));
            (isk ? sk : sq)[qi] = y;
            const T n0 = cin ? tqk1 : T(0), n1 = cin ? tqk2 : T(0);
            if constexpr (HPW == 1) {
                s_tap[0][tid] = n0;
                s_tap[1][tid] = n1;
                s_tap[2][tid] = xqk;
            } else {
                cout[crow + c_qk] = n0;
                cout[crow + Cc + c_qk] = n1;
                cout[crow + 2 * Cc + c_qk] = xqk;
            }
        }
        const int vc = tid - VOFF;
        const int vh = vc / DV, j = vc % DV;
        if (vc >= 0 && vc < HPW * DV && g0 + vh < gend) {
            const int h = hk * p.G + g0 + vh;
            const int c = 2 * p.Hk * DK + h * DV + j;
            sv[vh][j] = conv4_silu(wv, ld(tv0), ld(tv1), ld(tv2), A::load(&xv));
            sz[vh][j] = A::load(&zv);
            if (j == 0) {
                const float gg = -expf(alog) * softplus(A::load(&av) + dtb);
                s_eg[vh] = expf(gg);
                s_beta[vh] = sigmoid(A::load(&bv));
            }
            cout[crow + c] = cin ? tv1 : T(0);
            cout[crow + Cc + c] = cin ? tv2 : T(0);
            cout[crow + 2 * Cc + c] = xv;
        }
    };

    // thread (rg, cg) owns rows rg*RPT .. rg*RPT+RPT-1 of columns 4cg..4cg+3;
    // one load instruction covers whole 512-byte rows
    const int cg = t % CG, rg = t / CG;
    const uint32_t toff = static_cast<uint32_t>(rg * RPT * DV + 4 * cg);
    f32x4 H[RPT];
    // Unconditional loads (a branch around them would make every later wait
    // for the conv inputs also wait for the stream): a slot past the last
    // head reads the pair's first head, and with no initial state the loads
    // read state_out (same shape; the values are replaced by zeros at use).
    auto load_state = [&](int g0) {
        const int g = g0 + half < gend ? g0 + half : g0;
        const float* src = (p.state_in ? p.state_in : p.state_out) +
                           (static_cast<size_t>(sb) * p.Hv + hk * p.G + g) * DK * DV;
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            H[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + toff + m * DV));
    };

    if constexpr (HPW == 1) {
        conv_loads(gfirst, true);
        __builtin_amdgcn_sched_barrier(0);      // keep the conv inputs ahead of the stream
        load_state(gfirst);
        conv_compute(gfirst, true);
    } else {
        // two heads' state leaves no registers to hold the conv inputs
        // across the stream: the conv first, then the stream (with many
        // work-groups per compute unit, others keep the stream busy)
        conv_loads(gfirst, true);
        conv_compute(gfirst, true);
        __builtin_amdgcn_sched_barrier(0);
        load_state(gfirst);
    }
    __syncthreads();
    uint32_t* counter = nullptr;
    uint32_t prev;      // lane 0 of wave 0 only (no default: a merge would force a wait on the atomic)
    if constexpr (HPW == 1) {
        // every q/k history load of this work-group has been consumed: count
        // it in with a wrapping increment (old >= G - 1 stores 0), so the
        // last arrival also puts the counter back to zero.  Wave 0 uses the
        // answer only at its end, so waiting for it (loads complete in order)
        // costs nothing then.
        counter = p.arrive + static_cast<size_t>(b) * p.Hk + hk;
        if (tid == 0)
            prev = __builtin_amdgcn_atomic_inc32(counter, static_cast<uint32_t>(p.G - 1), __ATOMIC_RELAXED, "agent");
    }
    // the key head's norms, computed by every wave from the conv outputs:
    // q^ = s q~ / |q~|, k^ = k~ / |k~| (scaled as they are read) and k^ . q^
    // (every lane of a wave holds the same bits: kept as wave-uniform
    // values); the two sums of squares are reduced side by side
    float ssq = l2_sumsq<DK>(sq, lane), ssk = l2_sumsq<DK>(sk, lane);
    ssq = wave_sum(ssq);
    ssk = wave_sum(ssk);
    const float rq = uniform_f32(l2_finish(ssq, p.scale, p.eps_l2));
    const float rk = uniform_f32(l2_finish(ssk, 1.0f, p.eps_l2));
    float kq;
    {
        float d = 0.f;
        for (int i = lane; i < DK; i += kWave) d = fmaf(sk[i] * rk, sq[i] * rq, d);
        kq = uniform_f32(wave_sum(d));
    }

    for (int g0 = gfirst; g0 < gend; g0 += HPW) {
        const int g = g0 + half;
        const bool active = g < gend;
        const int h = hk * p.G + g;
        const size_t hbase = (static_cast<size_t>(sb) * p.Hv + h) * DK * DV;
        if (g0 != gfirst) {
            // the next pair of heads (HPW = 2, G > 2): their v channels and
            // gates, then their state
            conv_loads(g0, false);
            conv_compute(g0, false);
            __builtin_amdgcn_sched_barrier(0);
            load_state(g0);
            __syncthreads();
        }
        if (!p.state_in) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) H[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 rkv = {0.f, 0.f, 0.f, 0.f}, rqv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg * RPT + m;
            const float kk = sk[i] * rk, qq = sq[i] * rq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rkv[e] = fmaf(H[m][e], kk, rkv[e]);
                rqv[e] = fmaf(H[m][e], qq, rqv[e]);
            }
        }
        red_k[half][rg][cg] = rkv;
        red_q[half][rg][cg] = rqv;
        __syncthreads();
        if (active) {
            f32x4 RK = red_k[half][0][cg], RQ = red_q[half][0][cg];
#pragma unroll
            for (int r = 1; r < RG; ++r) {
                f32x4 a = red_k[half][r][cg], c = red_q[half][r][cg];
#pragma unroll
                for (int e = 0; e < 4; ++e) { RK[e] += a[e]; RQ[e] += c[e]; }
            }
            const float eg = s_eg[half], beta = s_beta[half];
            f32x4 u, o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[e] = beta * (sv[half][4 * cg + e] - eg * RK[e]);
                o[e] = fmaf(eg, RQ[e], kq * u[e]);
            }
            float* so = p.state_out + hbase;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float kk = sk[rg * RPT + m] * rk;
                f32x4 hn;
#pragma unroll
                for (int e = 0; e < 4; ++e) hn[e] = fmaf(eg, H[m][e], kk * u[e]);
                __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(so + toff + m * DV));
            }
            // z-gated RMSNorm over dv: row group 0 = lanes 0..CG-1 of the
            // half's first wave.
            if (t < kWave)
                gated_rmsnorm_store<DV>(t, o, &sz[half][4 * cg], p.norm_w, p.eps_rms, p.out, p.out_bf16,
                                        p.core_out, (static_cast<size_t>(b) * p.Hv + h) * DV + 4 * cg);
        }
        if constexpr (HPW == 1) {
            // the last of the key head's work-groups (wave 0 of it) writes
            // the key head's q/k history
            if (wave == 0 && __shfl(prev, 0, kWave) + 1 == static_cast<uint32_t>(p.G)) {
                for (int ch = lane; ch < 2 * DK; ch += kWave) {
                    const int c = (ch >= DK ? p.Hk * DK - DK : 0) + hk * DK + ch;
                    cout[crow + c] = s_tap[0][ch];
                    cout[crow + Cc + c] = s_tap[1][ch];
                    cout[crow + 2 * Cc + c] = s_tap[2][ch];
                }
            }
        }
        if (g0 + HPW < gend) __syncthreads();   // LDS (sv, sz, red_*) reused by the next pair of heads
    }
}

// ---------------------------------------------------------------------------
// Multi-token verify: p.Ts <= TSM tokens per sequence.  The same work-group
// layout and the same per-token arithmetic as the one-token kernel above, in
// the same order, with the state held in registers between tokens, so the
// result equals p.Ts single decode steps bit for bit.  The state is written
// after every token to p.snap when given, and after the last one to
// state_out.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool BF16, int TSM = kMaxVerifyTokens>
__global__ __launch_bounds__(kDecodeThreads, 2) void verify_kernel(DecodeParams p) {
    using A = Act<BF16>;
    using T = typename A::T;
    constexpr int NT = kDecodeHalf;
    constexpr int CG = DV / 4;          // float4 column groups
    constexpr int RG = NT / CG;         // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    static_assert(CG <= 64 && NT % CG == 0 && DK % RG == 0 && RPT >= 1, "shape");
    static_assert(2 * DK <= kDecodeThreads, "one thread per q/k channel");

    __shared__ float sq[TSM][DK], sk[TSM][DK], sv[2][TSM][DV], sz[2][TSM][DV];
    __shared__ f32x4 red_k[2][RG][CG], red_q[2][RG][CG];
    __shared__ float s_r[2][TSM], s_kq[TSM], s_eg[2][TSM], s_beta[2][TSM];

    const int Ts = p.Ts;
    const int b = blockIdx.x / p.Hk;
    const int hk = blockIdx.x % p.Hk;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    // value head slot (uniform per wave, so the state base lives in SGPRs)
    const int half = __builtin_amdgcn_readfirstlane(tid / NT);
    const int t = tid % NT;
    const int Cc = 2 * p.Hk * DK + p.Hv * DV;
    const T* cin = static_cast<const T*>(p.conv_in);
    T* cout = static_cast<T*>(p.conv_out);
    const int sb = state_slot(p.slots, b);                // pool entry of the states
    if (p.slots && static_cast<unsigned>(sb) >= static_cast<unsigned>(p.num_slots)) {
        // an entry outside the pool: the sequence is skipped and reported
        if (tid == 0 && p.status)
            __hip_atomic_fetch_or(p.status, kStatusBadIndex, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const size_t crow = static_cast<size_t>(sb) * 3 * Cc;
    const int64_t row0 = static_cast<int64_t>(b) * Ts;   // the sequence's first token row

    // thread (rg, cg) owns rows rg*RPT .. rg*RPT+RPT-1 of columns 4cg..4cg+3;
    // one load instruction still covers whole 512-byte rows.  The first pair
    // of heads' state stream is issued before anything else so its latency
    // overlaps the conv and the norms.
    const int cg = t % CG, rg = t / CG;
    const uint32_t toff = static_cast<uint32_t>(rg * RPT * DV + 4 * cg);
    f32x4 H[RPT];
    auto load_state = [&](int g0) {
        const int g = g0 + half;
        if (g < p.G && p.state_in) {
            const float* src = p.state_in + (static_cast<size_t>(sb) * p.Hv + hk * p.G + g) * DK * DV;
#pragma unroll
            for (int m = 0; m < RPT; ++m)
                H[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + toff + m * DV));
        } else {
#pragma unroll
            for (int m = 0; m < RPT; ++m) H[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    load_state(0);

    // conv1d(K=4) + SiLU of channel c over the sequence's tokens: the window
    // (w0, w1, w2) holds the three previous raw inputs (the conv state for the
    // first token) and slides by one per token; the last window is the new
    // conv state.  All of the channel's loads are issued before arithmetic.
    auto conv_channel = [&](int c, const T* src, int64_t rs, float* y, int ystride) {
        T xs[TSM];
#pragma unroll
        for (int s = 0; s < TSM; ++s)
            if (s < Ts) xs[s] = src[(row0 + s) * rs];
        T w0 = cin ? cin[crow + c] : T(0);
        T w1 = cin ? cin[crow + Cc + c] : T(0);
        T w2 = cin ? cin[crow + 2 * Cc + c] : T(0);
        const f32x4 w = *reinterpret_cast<const f32x4*>(p.conv_w + static_cast<size_t>(c) * 4);
#pragma unroll
        for (int s = 0; s < TSM; ++s) {
            if (s < Ts) {
                y[s * ystride] = conv4_silu(w, A::load(&w0), A::load(&w1), A::load(&w2), A::load(&xs[s]));
                w0 = w1;
                w1 = w2;
                w2 = xs[s];
            }
        }
        cout[crow + c] = w0;
        cout[crow + Cc + c] = w1;
        cout[crow + 2 * Cc + c] = w2;
    };
    // z and the gates of value head h (slot `slot`) for every token
    auto head_inputs = [&](int h, int slot, int j, bool gate) {
#pragma unroll
        for (int s = 0; s < TSM; ++s)
            if (s < Ts) sz[slot][s][j] = A::load(static_cast<const T*>(p.z) + (row0 + s) * p.zs + h * DV + j);
        if (gate) {
            float av[TSM], bv[TSM];
#pragma unroll
            for (int s = 0; s < TSM; ++s) {
                if (s < Ts) {
                    av[s] = A::load(static_cast<const T*>(p.a) + (row0 + s) * p.as + h);
                    bv[s] = A::load(static_cast<const T*>(p.b) + (row0 + s) * p.bs + h);
                }
            }
#pragma unroll
            for (int s = 0; s < TSM; ++s) {
                if (s < Ts) {
                    const float gg = -expf(p.A_log[h]) * softplus(av[s] + p.dt_bias[h]);
                    s_eg[slot][s] = expf(gg);
                    s_beta[slot][s] = sigmoid(bv[s]);
                }
            }
        }
    };

    // q and k: one conv channel per thread, threads [0, 2 DK)
    if (tid < 2 * DK) {
        const int isk = tid >= DK;
        const int i = tid - isk * DK;
        conv_channel(isk * p.Hk * DK + hk * DK + i,
                     (isk ? static_cast<const T*>(p.k) : static_cast<const T*>(p.q)) + hk * DK + i,
                     isk ? p.ks : p.qs, (isk ? &sk[0][0] : &sq[0][0]) + i, DK);
    }
    __syncthreads();
    if (wave < 2) {
        for (int s = 0; s < Ts; ++s) {
            const float r = l2_scale<DK>(wave == 0 ? sq[s] : sk[s], lane, wave == 0 ? p.scale : 1.0f,
                                         p.eps_l2);
            if (lane == 0) s_r[wave][s] = r;
        }
    }
    __syncthreads();
    if (tid < 2 * DK) {
        for (int s = 0; s < Ts; ++s) {
            if (tid < DK) sq[s][tid] *= s_r[0][s];
            else sk[s][tid - DK] *= s_r[1][s];
        }
    }
    __syncthreads();
    if (wave == 0) {
        for (int s = 0; s < Ts; ++s) {
            const float d = dot_wave<DK>(sk[s], sq[s], lane);
            if (lane == 0) s_kq[s] = d;
        }
    }

    for (int g0 = 0; g0 < p.G; g0 += 2) {
        const int g = g0 + half;
        const bool active = g < p.G;
        const int h = hk * p.G + g;
        const size_t hbase = (static_cast<size_t>(sb) * p.Hv + h) * DK * DV;
        if (g0 > 0) load_state(g0);
        // conv + SiLU of this head's v channels, z and gates
        if (active) {
            for (int j = t; j < DV; j += NT) {
                conv_channel(2 * p.Hk * DK + h * DV + j, static_cast<const T*>(p.v) + h * DV + j, p.vs,
                             &sv[half][0][j], DV);
                head_inputs(h, half, j, j == 0);
            }
        }
        for (int s = 0; s < Ts; ++s) {
            f32x4 rk = {0.f, 0.f, 0.f, 0.f}, rq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int i = rg * RPT + m;
                const float kk = sk[s][i], qq = sq[s][i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rk[e] = fmaf(H[m][e], kk, rk[e]);
                    rq[e] = fmaf(H[m][e], qq, rq[e]);
                }
            }
            red_k[half][rg][cg] = rk;
            red_q[half][rg][cg] = rq;
            __syncthreads();
            if (active) {
                f32x4 RK = red_k[half][0][cg], RQ = red_q[half][0][cg];
#pragma unroll
                for (int r = 1; r < RG; ++r) {
                    f32x4 a = red_k[half][r][cg], c = red_q[half][r][cg];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { RK[e] += a[e]; RQ[e] += c[e]; }
                }
                const float eg = s_eg[half][s], beta = s_beta[half][s], kq = s_kq[s];
                f32x4 u, o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u[e] = beta * (sv[half][s][4 * cg + e] - eg * RK[e]);
                    o[e] = fmaf(eg, RQ[e], kq * u[e]);
                }
                // H' = e^g H + k u^T: the last token's goes to state_out, each
                // token's to its snapshot when asked for
                float* so = (s == Ts - 1) ? p.state_out + hbase : nullptr;
                float* sn = p.snap ? p.snap + ((row0 + s) * p.Hv + h) * DK * DV : nullptr;
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const float kk = sk[s][rg * RPT + m];
                    f32x4 hn;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hn[e] = fmaf(eg, H[m][e], kk * u[e]);
                    if (s + 1 < Ts) H[m] = hn;       // (dead after the last token)
                    if (so) __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(so + toff + m * DV));
                    if (sn) __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(sn + toff + m * DV));
                }
                // z-gated RMSNorm over dv: row group 0 = lanes 0..CG-1 of the
                // half's first wave.
                if (t < kWave)
                    gated_rmsnorm_store<DV>(t, o, &sz[half][s][4 * cg], p.norm_w, p.eps_rms, p.out,
                                            p.out_bf16, p.core_out,
                                            (static_cast<size_t>(row0 + s) * p.Hv + h) * DV + 4 * cg);
            }
            __syncthreads();   // red_* reused by the next token, sv/sz by the next pair
        }
    }
}

template <int DK, int DV, bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
    const unsigned B = static_cast<unsigned>(p.B);
    if (p.Ts != 0)
        hipLaunchKernelGGL((verify_kernel<DK, DV, BF16>), dim3(B * static_cast<unsigned>(p.Hk)),
                           dim3(kDecodeThreads), 0, s, p);
    else if (p.arrive)
        hipLaunchKernelGGL((decode_kernel<DK, DV, BF16, 1>), dim3(B * static_cast<unsigned>(p.Hv)),
                           dim3(kDecodeHalf), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, BF16, 2>), dim3(B * static_cast<unsigned>(p.Hk)),
                           dim3(kDecodeThreads), 0, s, p);
    return hipGetLastError();
}

bool decode_shape_supported(int DK, int DV) {
    return (DK == 128 && DV == 128) || (DK == 32 && DV == 32) || (DK == 32 && DV == 64) ||
           (DK == 64 && DV == 64);
}

hipError_t launch_decode(int DK, int DV, bool bf16, const DecodeParams& p, hipStream_t s,
                         bool* supported) {
    *supported = true;
#define GDN_DEC(dk, dv)                                                              \
    if (DK == dk && DV == dv)                                                        \
        return bf16 ? launch_decode_t<dk, dv, true>(p, s) : launch_decode_t<dk, dv, false>(p, s);
    GDN_DEC(128, 128)
    GDN_DEC(32, 32)
    GDN_DEC(32, 64)
    GDN_DEC(64, 64)
#undef GDN_DEC
    *supported = false;
    return hipSuccess;
}

}  // namespace gdn
