// gdn_gemm.hip -- the layer's projections as bf16 matrix-core GEMMs.
//
// C[M][N] = A[M][K] * B[N][K]^T, bf16 operands with fp32 accumulation, bf16
// or fp32 output: A is the activations (row-major, k contiguous) and B a
// weight matrix in the [out][in] layout, so both operands load as 16-byte
// runs along k, which is the k-contiguous fragment order of
// v_mfma_f32_16x16x32_bf16 (lane l holds row / column l % 16, k = 8*(l/16)+e).
//
// A work-group computes a 256 x 256 tile (256 x 128 when that leaves compute
// units idle) with 8 waves, two per SIMD; at 256 x 256 each wave owns 128 x
// 64 (8 x 4 matrix-core tiles of 16 x 16: 12 fragment reads from LDS per 32
// products).  The k loop runs over BK = 64 slices with two LDS stages: while
// the waves multiply slice k, slice k+1 comes from global memory into
// registers and then into the other stage, one barrier per slice.  Rows past
// M or N and k past K read as zeros; only in-range outputs are stored.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

namespace {

constexpr int kBK = 64;
constexpr int kGemmThreads = 512;             // 8 waves, two per SIMD
constexpr int kLS = kBK + 8;                  // LDS row stride (bf16) of both tiles

// BM x BN work-group tile; the 8 waves are WGM x WGN, each owning a
// (BM/WGM) x (BN/WGN) block of 16 x 16 matrix-core tiles.
template <int BM, int BN>
struct GemmGeom {
    static constexpr int WGM = BN == 256 ? 2 : 4, WGN = 8 / WGM;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int AC = BM * kBK / 8 / kGemmThreads;    // 16-byte loads per thread (A)
    static constexpr int BC = BN * kBK / 8 / kGemmThreads;    // (B)
    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0 && AC >= 1 && BC >= 1, "tile");
};

template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_nt_kernel(
        const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
        void* __restrict__ Cv, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    using G = GemmGeom<BM, BN>;
    // two LDS stages: slice k is multiplied from one while slice k+1 is
    // written into the other
    __shared__ __align__(16) uint16_t As[2][BM * kLS];
    __shared__ __align__(16) uint16_t Bs[2][BN * kLS];

    // tile order: consecutive work-groups walk down M inside one N column of
    // tiles, so a B (weight) slice is shared in L2 by the work-groups near it
    const int64_t mtiles = (M + BM - 1) / BM;
    const int64_t m0 = (blockIdx.x % mtiles) * BM, n0 = (blockIdx.x / mtiles) * BN;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int wm = wave / G::WGN, wn = wave % G::WGN;

    // global -> register staging: chunk c of a tile is row c / 8, k 8*(c % 8)
    u32x4 ra[G::AC], rb[G::BC];
    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int u = 0; u < G::AC; ++u) {
            const int c = tid + u * kGemmThreads;
            const int64_t r = m0 + c / 8, k = k0 + 8 * (c % 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < M && k < K) v = *reinterpret_cast<const u32x4*>(A + r * lda + k);
            ra[u] = v;
        }
#pragma unroll
        for (int u = 0; u < G::BC; ++u) {
            const int c = tid + u * kGemmThreads;
            const int64_t r = n0 + c / 8, k = k0 + 8 * (c % 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < N && k < K) v = *reinterpret_cast<const u32x4*>(B + r * ldb + k);
            rb[u] = v;
        }
    };
    auto store_tiles = [&](int st) {
#pragma unroll
        for (int u = 0; u < G::AC; ++u) {
            const int c = tid + u * kGemmThreads;
            *reinterpret_cast<u32x4*>(&As[st][(c / 8) * kLS + 8 * (c % 8)]) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < G::BC; ++u) {
            const int c = tid + u * kGemmThreads;
            *reinterpret_cast<u32x4*>(&Bs[st][(c / 8) * kLS + 8 * (c % 8)]) = rb[u];
        }
    };

    f32x4 acc[G::TM][G::TN];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    int st = 0;
    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        const bool more = k0 + kBK < K;
        if (more) load_tiles(k0 + kBK);            // next slice in flight during the products
        const uint16_t* as = As[st];
        const uint16_t* bs = Bs[st];
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            u32x4 fb[G::TN];
#pragma unroll
            for (int j = 0; j < G::TN; ++j)
                fb[j] = *reinterpret_cast<const u32x4*>(&bs[(wn * G::WN + j * 16 + l16) * kLS + ks * 32 + lq * 8]);
#pragma unroll
            for (int i = 0; i < G::TM; ++i) {
                const u32x4 fa = *reinterpret_cast<const u32x4*>(&as[(wm * G::WM + i * 16 + l16) * kLS + ks * 32 + lq * 8]);
#pragma unroll
                for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma(fa, fb[j], acc[i][j]);
            }
        }
        if (more) store_tiles(st ^ 1);             // the other stage: nobody reads it now
        __syncthreads();
        st ^= 1;
    }

    // C/D fragment: lane holds column l16 and rows 4*lq + e of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
            const int64_t col = n0 + wn * G::WN + j * 16 + l16;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * G::WM + i * 16 + lq * 4 + e;
                if (row >= M) continue;
                if constexpr (OUT_BF16)
                    static_cast<uint16_t*>(Cv)[row * ldc + col] = f32_to_bf16_bits(acc[i][j][e]);
                else
                    static_cast<float*>(Cv)[row * ldc + col] = acc[i][j][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K % 32 == 0: the k loop streams 32-wide slices straight from global memory
// into four LDS stages (global_load_lds_dwordx4: each lane's 16 bytes land at
// the wave's LDS block + 16 * lane, no registers in between), so a slice is
// requested three slices before it is multiplied.  A stage holds rows of 32
// bf16 (64 bytes) with the 16-byte chunks of row r permuted by
// chunk ^ ((r >> 2) & 3), which keeps a 16-lane fragment read on 16 distinct
// groups of four banks.
// ---------------------------------------------------------------------------
constexpr int kSK = 32;                       // k per stage
constexpr int kStages = 4;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_nt_dma_kernel(
        const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
        void* __restrict__ Cv, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    using G = GemmGeom<BM, BN>;
    constexpr int AW = BM * kSK * 2 / 1024, BW = BN * kSK * 2 / 1024;   // 1 KiB wave loads per stage
    constexpr int NW = kGemmThreads / kWave;
    static_assert(AW % NW == 0 && BW % NW == 0, "loads per wave");
    __shared__ __align__(1024) uint16_t As0[BM * kSK], As1[BM * kSK], As2[BM * kSK], As3[BM * kSK];
    __shared__ __align__(1024) uint16_t Bs0[BN * kSK], Bs1[BN * kSK], Bs2[BN * kSK], Bs3[BN * kSK];

    const int64_t mtiles = (M + BM - 1) / BM;
    const int64_t m0 = (blockIdx.x % mtiles) * BM, n0 = (blockIdx.x / mtiles) * BN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int wm = wave / G::WGN, wn = wave % G::WGN;

    // wave load j of a stage covers rows 16 j .. 16 j + 15; lane l fills
    // physical chunk l % 4 of row 16 j + l / 4, i.e. logical chunk
    // swz(row, l % 4) of that row; rows past M / N read row 0 (their outputs
    // are never stored).  Stages are separate LDS objects addressed with
    // compile-time indices, so the compiler can tell that a slice's reads do
    // not depend on the loads still in flight into the other stages.
    const int lrow = lane / 4, lpc = lane % 4;
    auto issue = [&](uint16_t* as, uint16_t* bs, int64_t k0) {
#pragma unroll
        for (int u = 0; u < AW / NW; ++u) {
            const int j = wave + u * NW;
            const int row = 16 * j + lrow;
            const int64_t gr = m0 + row < M ? m0 + row : 0;
            const uint16_t* src = A + gr * lda + k0 + 8 * swz(row, lpc);
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(as + j * 512), 16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < BW / NW; ++u) {
            const int j = wave + u * NW;
            const int row = 16 * j + lrow;
            const int64_t gr = n0 + row < N ? n0 + row : 0;
            const uint16_t* src = B + gr * ldb + k0 + 8 * swz(row, lpc);
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(bs + j * 512), 16, 0, 0);
        }
    };

    f32x4 acc[G::TM][G::TN];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto multiply = [&](const uint16_t* as, const uint16_t* bs) {
        u32x4 fb[G::TN];
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
            const int row = wn * G::WN + j * 16 + l16;
            fb[j] = *reinterpret_cast<const u32x4*>(bs + row * kSK + 8 * swz(row, lq));
        }
#pragma unroll
        for (int i = 0; i < G::TM; ++i) {
            const int row = wm * G::WM + i * 16 + l16;
            const u32x4 fa = *reinterpret_cast<const u32x4*>(as + row * kSK + 8 * swz(row, lq));
#pragma unroll
            for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma(fa, fb[j], acc[i][j]);
        }
    };

    const int64_t nk = K / kSK;
    constexpr int per = (AW + BW) / NW;      // loads per wave per slice
    // slice k from stage (as, bs); slice k + 3 into stage (an, bn), the one
    // slice k - 1 used
    auto step = [&](int64_t k, const uint16_t* as, const uint16_t* bs, uint16_t* an, uint16_t* bn) {
        // this wave's loads of slice k have landed once at most the loads of
        // the (up to two) later slices are outstanding
        if (k + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * per));
        else if (k + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | per);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        // every wave's slice k is in and slice k-1's stage is free.  A plain
        // s_barrier: the waits above already cover the loads that matter,
        // and __syncthreads' release fence would also wait for the slices
        // still in flight
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k + 3 < nk) issue(an, bn, (k + 3) * kSK);
        multiply(as, bs);
    };
    if (nk > 0) issue(As0, Bs0, 0);
    if (nk > 1) issue(As1, Bs1, kSK);
    if (nk > 2) issue(As2, Bs2, 2 * kSK);
    int64_t k = 0;
    for (; k + 3 < nk; k += 4) {
        step(k, As0, Bs0, As3, Bs3);
        step(k + 1, As1, Bs1, As0, Bs0);
        step(k + 2, As2, Bs2, As1, Bs1);
        step(k + 3, As3, Bs3, As2, Bs2);
    }
    if (k < nk) step(k, As0, Bs0, As3, Bs3);
    if (k + 1 < nk) step(k + 1, As1, Bs1, As0, Bs0);
    if (k + 2 < nk) step(k + 2, As2, Bs2, As1, Bs1);

#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
            const int64_t col = n0 + wn * G::WN + j * 16 + l16;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * G::WM + i * 16 + lq * 4 + e;
                if (row >= M) continue;
                if constexpr (OUT_BF16)
                    static_cast<uint16_t*>(Cv)[row * ldc + col] = f32_to_bf16_bits(acc[i][j][e]);
                else
                    static_cast<float*>(Cv)[row * ldc + col] = acc[i][j][e];
            }
        }
    }
}

template <int BM, int BN>
hipError_t launch_gemm_t(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, void* C,
                         int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(static_cast<unsigned>(tiles)), block(kGemmThreads);
    const bool dma = K % kSK == 0 && lda % 8 == 0 && ldb % 8 == 0;
    if (dma && out_bf16)
        hipLaunchKernelGGL((gemm_bf16_nt_dma_kernel<BM, BN, true>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    else if (dma)
        hipLaunchKernelGGL((gemm_bf16_nt_dma_kernel<BM, BN, false>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    else if (out_bf16)
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, true>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    else
        hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, false>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    return hipGetLastError();
}

// ---- skinny products: M <= kSkinnyMax rows (decode batches) ----
// With few rows of A the product is a stream over the weight matrix B, which
// a tiled kernel reads at a fraction of the memory bandwidth.  Here a
// work-group owns NTW matrix-core n tiles (16 NTW rows of B) and splits K
// over its NWV waves.  Per 128-wide k step, lane (l16, q) reads 64 contiguous
// bytes of B row n0 + l16 (of each n tile), k in [32 q, 32 q + 32), as four
// 8-wide fragments, and the same k set of every A row (the products only
// need both operands to use one k mapping), so each B row is read as
// 256-byte runs.  Every pair of the MT 16-row tiles of A and the NTW B tiles
// is multiplied; the waves' partial tiles are summed in LDS in wave order.
// Each output depends on its A row, B row, K and NWV only, never on M or on
// the other rows.  More than 64 rows run as 64-row blocks over the grid's
// second dimension.
constexpr int kSkinnyMax = 64;
constexpr int kSkinnyStep = 128;

template <int MT, int NTW, int NWV, bool OUT_BF16>
__global__ __launch_bounds__(NWV * kWave) void gemm_skinny_kernel(
        const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
        void* __restrict__ Cv, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    __shared__ f32x4 part[NWV][MT * NTW][kWave];
    // this work-group's block of (at most kSkinnyMax) rows
    A += static_cast<int64_t>(blockIdx.y) * kSkinnyMax * lda;
    M -= static_cast<int64_t>(blockIdx.y) * kSkinnyMax;
    if (M > kSkinnyMax) M = kSkinnyMax;
    if constexpr (OUT_BF16)
        Cv = static_cast<uint16_t*>(Cv) + static_cast<int64_t>(blockIdx.y) * kSkinnyMax * ldc;
    else
        Cv = static_cast<float*>(Cv) + static_cast<int64_t>(blockIdx.y) * kSkinnyMax * ldc;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16 * NTW;
    const int64_t steps = (K + kSkinnyStep - 1) / kSkinnyStep;
    const int64_t s0 = steps * wave / NWV, s1 = steps * (wave + 1) / NWV;
    const uint16_t* brow[NTW];
    bool nok[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const int64_t n = n0 + t * 16 + l16;
        nok[t] = n < N;
        brow[t] = B + (nok[t] ? n : 0) * ldb;
    }
    const uint16_t* arow[MT];
    bool mok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mt * 16 + l16;
        mok[mt] = m < M;
        arow[mt] = A + (mok[mt] ? m : 0) * lda;
    }
    f32x4 acc[MT][NTW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll 2
    for (int64_t st = s0; st < s1; ++st) {
        const int64_t kb = st * kSkinnyStep + lq * 32;
        u32x4 bf[NTW][4];
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t k = kb + 8 * j;
                bf[t][j] = (nok[t] && k < K) ? *reinterpret_cast<const u32x4*>(brow[t] + k) : zero;
            }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            u32x4 af[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t k = kb + 8 * j;
                af[j] = (mok[mt] && k < K) ? *reinterpret_cast<const u32x4*>(arow[mt] + k) : zero;
            }
#pragma unroll
            for (int t = 0; t < NTW; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[mt][t] = mfma(af[j], bf[t][j], acc[mt][t]);
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) part[wave][mt * NTW + t][lane] = acc[mt][t];
    __syncthreads();
    // wave i sums output tile i (m tile i / NTW, n tile i % NTW) over the
    // waves in order and stores it
    for (int i = wave; i < MT * NTW; i += NWV) {
        const int mt = i / NTW, t = i % NTW;
        f32x4 s = part[0][i][lane];
        for (int w = 1; w < NWV; ++w) {
            const f32x4 v = part[w][i][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += v[e];
        }
        const int64_t n = n0 + t * 16 + l16;
        if (n >= N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = mt * 16 + lq * 4 + e;
            if (m >= M) continue;
            if constexpr (OUT_BF16)
                static_cast<uint16_t*>(Cv)[m * ldc + n] = f32_to_bf16_bits(s[e]);
            else
                static_cast<float*>(Cv)[m * ldc + n] = s[e];
        }
    }
}

template <int MT, int NTW, int NWV>
hipError_t launch_skinny_t(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, void* C,
                           int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((N + 16 * NTW - 1) / (16 * NTW)),
                    static_cast<unsigned>((M + kSkinnyMax - 1) / kSkinnyMax)),
        block(NWV * kWave);
    if (out_bf16)
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, NTW, NWV, true>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, NTW, NWV, false>), grid, block, 0, s, a, lda, b, ldb, C, ldc, M, N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_nt(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                               int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K,
                               hipStream_t s, GemmPath path) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const auto a = static_cast<const uint16_t*>(A);
    const auto b = static_cast<const uint16_t*>(B);
    // 256 x 256 tiles when they still give every compute unit work, else
    // 256 x 128
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const bool few = path == kGemmSkinny || path == kGemmLibraryFew || (path == kGemmAuto && M <= kSkinnyMax);
    if (path == kGemmLibraryFew || (path == kGemmAuto && M <= kSkinnyMax)) {
        hipError_t e = hipSuccess;
        if (gemm_library(A, lda, B, ldb, C, ldc, out_bf16, M, N, K, kSkinnyMax, s, &e)) return e;
    }
    if (few) {
        // few rows (A rows and lda are 16-byte aligned, K a multiple of 8)
        // With n tiles to spare (at least two per compute unit) K is split
        // over 4 waves and, past 16 rows, a work-group takes 4 n tiles so
        // that each A fragment serves 4 B tiles; otherwise K is split over 16
        // waves, one n tile each.  The split depends on N only, so a row's
        // bits do not depend on M.
        const bool many = (N + 15) / 16 >= 2ll * cus;
        const int mt = static_cast<int>(((M < kSkinnyMax ? M : kSkinnyMax) + 15) / 16);
#define GDN_SKINNY(MT_, NTW_, NWV_) \
    return launch_skinny_t<MT_, NTW_, NWV_>(a, lda, b, ldb, C, ldc, out_bf16, M, N, K, s)
        if (many) {
            switch (mt) {
                case 1: GDN_SKINNY(1, 1, 4);
                case 2: GDN_SKINNY(2, 4, 4);
                case 3: GDN_SKINNY(3, 4, 4);
                default: GDN_SKINNY(4, 4, 4);
            }
        }
        switch (mt) {
            case 1: GDN_SKINNY(1, 1, 16);
            case 2: GDN_SKINNY(2, 1, 16);
            case 3: GDN_SKINNY(3, 1, 16);
            default: GDN_SKINNY(4, 1, 16);
        }
#undef GDN_SKINNY
    }
    if (path == kGemmAuto || path == kGemmLibrary) {
        // N past a multiple of 256 (in_proj's 12352 = 48 x 256 + 64 for the
        // a and b gates) leaves the library's tile grid a last column of
        // nearly empty tiles, and at 4096 rows a nearly empty last round of
        // them over the compute units: the full 256-column blocks run as one
        // product and the rest as another (each with its own algorithm;
        // columns are independent, so each column's bits are still fixed by
        // its range alone)
        hipError_t e = hipSuccess;
        const int64_t rest = N % 256;
        const int64_t main_n = N > 256 ? N - rest : N;
        if (gemm_library(A, lda, B, ldb, C, ldc, out_bf16, M, main_n, K, 4096, s, &e)) {
            if (e != hipSuccess || main_n == N) return e;
            return launch_gemm_bf16_nt(A, lda, b + main_n * ldb, ldb,
                                       static_cast<uint8_t*>(C) + main_n * (out_bf16 ? 2 : 4), ldc, out_bf16, M,
                                       rest, K, s, kGemmLibrary);
        }
    }
    const int64_t wide = ((M + 255) / 256) * ((N + 255) / 256);
    if (wide >= cus) return launch_gemm_t<256, 256>(a, lda, b, ldb, C, ldc, out_bf16, M, N, K, s);
    return launch_gemm_t<256, 128>(a, lda, b, ldb, C, ldc, out_bf16, M, N, K, s);
}

}  // namespace gdn
