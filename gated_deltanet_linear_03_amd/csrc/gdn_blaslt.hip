// gdn_blaslt.hip -- the projections' large GEMMs through hipBLASLt.
//
// C[M][N] = A[M][K] B[N][K]^T (row-major, bf16 in, fp32 accumulation, bf16 or
// fp32 out) is, in the library's column-major terms, C^T (N x M) = op_T(B)
// op_N(A) with B stored as a K x N and A as a K x M column-major matrix.
//
// One algorithm per (device, N, K, leading dimensions, output type, pinning
// size): the first of the library's ranked choices for that shape at the
// pinning size in rows (4096 for the prefill projections, 64 for the decode
// ones) that needs no workspace (so no split of K over work-groups; some library
// versions rank such a split first even when asked for no workspace).  It is
// then used at every M, so an output element is summed in the same order
// whatever the number of rows (a row's bits do not depend on the batch), and
// the choice does not depend on timing, so it is the same in every process on
// the same library and device.  The algorithm's fitness (and its need of no
// workspace) is only established up to the size it was chosen at, and the
// library does not check a caller's algorithm against a larger problem, so a
// product with more rows runs in blocks of at most that many rows; rows are
// independent, so blocking changes no bit.  Only the library's C interface is
// used.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gdn_kernels.hpp"

namespace gdn {

namespace {

constexpr int kRanked = 16;          // ranked choices looked through

struct PlanKey {
    int dev;
    int64_t n, k, lda, ldb, ldc, pin;
    bool bf16;
    bool operator<(const PlanKey& o) const {
        return std::tie(dev, n, k, lda, ldb, ldc, pin, bf16) <
               std::tie(o.dev, o.n, o.k, o.lda, o.ldb, o.ldc, o.pin, o.bf16);
    }
};

struct Plan {
    bool ok = false;
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;     // per device, for the life of the process
std::map<PlanKey, Plan> g_plans;

// The three layouts of one product with M rows; false if the library
// refuses them (nothing to destroy then).
bool make_layouts(int64_t M, const PlanKey& k, hipblasLtMatrixLayout_t* l) {
    l[0] = l[1] = l[2] = nullptr;
    bool ok = hipblasLtMatrixLayoutCreate(&l[0], HIP_R_16BF, k.k, k.n, k.ldb) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&l[1], HIP_R_16BF, k.k, M, k.lda) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&l[2], k.bf16 ? HIP_R_16BF : HIP_R_32F, k.n, M, k.ldc) ==
                  HIPBLAS_STATUS_SUCCESS;
    if (!ok) {
        for (int i = 0; i < 3; ++i)
            if (l[i]) hipblasLtMatrixLayoutDestroy(l[i]);
    }
    return ok;
}

void drop_layouts(hipblasLtMatrixLayout_t* l) {
    for (int i = 0; i < 3; ++i) hipblasLtMatrixLayoutDestroy(l[i]);
}

Plan make_plan(hipblasLtHandle_t h, const PlanKey& key) {
    Plan p;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return Plan{};
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    hipblasLtMatrixLayout_t l[3];
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t no_ws = 0;
    hipblasLtMatmulHeuristicResult_t res[kRanked] = {};
    int got = 0;
    const bool ok =
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
            HIPBLAS_STATUS_SUCCESS &&
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
            HIPBLAS_STATUS_SUCCESS &&
        make_layouts(key.pin, key, l);
    if (!ok) {
        hipblasLtMatmulDescDestroy(p.desc);
        return Plan{};
    }
    const bool queried =
        hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                              sizeof(no_ws)) == HIPBLAS_STATUS_SUCCESS &&
        hipblasLtMatmulAlgoGetHeuristic(h, p.desc, l[0], l[1], l[2], l[2], pref, kRanked, res, &got) ==
            HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    drop_layouts(l);
    int pick = -1;
    for (int i = 0; queried && i < got && pick < 0; ++i)
        if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize == 0) pick = i;
    if (pick < 0) {
        hipblasLtMatmulDescDestroy(p.desc);
        return Plan{};
    }
    p.algo = res[pick].algo;
    p.ok = true;
    return p;
}

}  // namespace

bool gemm_library(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                  bool out_bf16, int64_t M, int64_t N, int64_t K, int64_t pin_rows, hipStream_t s,
                  hipError_t* err) {
    *err = hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(g_mu);
    auto hit = g_handles.find(dev);
    if (hit == g_handles.end()) {
        hipblasLtHandle_t h = nullptr;
        if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) h = nullptr;
        hit = g_handles.emplace(dev, h).first;          // a failed handle is not retried
    }
    hipblasLtHandle_t h = hit->second;
    if (!h) return false;
    const PlanKey key{dev, N, K, lda, ldb, ldc, pin_rows, out_bf16};
    auto pit = g_plans.find(key);
    if (pit == g_plans.end()) pit = g_plans.emplace(key, make_plan(h, key)).first;
    Plan& plan = pit->second;
    if (!plan.ok) return false;
    const float alpha = 1.f, beta = 0.f;
    const size_t c_elem = out_bf16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < M; m0 += pin_rows) {
        const int64_t mb = M - m0 < pin_rows ? M - m0 : pin_rows;
        hipblasLtMatrixLayout_t l[3];
        if (!make_layouts(mb, key, l)) return m0 == 0 ? false : (*err = hipErrorUnknown, true);
        const void* a = static_cast<const uint16_t*>(A) + m0 * lda;
        void* c = static_cast<uint8_t*>(C) + static_cast<size_t>(m0 * ldc) * c_elem;
        const hipblasStatus_t st =
            hipblasLtMatmul(h, plan.desc, &alpha, B, l[0], a, l[1], &beta, c, l[2], c, l[2], &plan.algo, nullptr, 0, s);
        drop_layouts(l);
        // the library declining the first block leaves room for another
        // family; a later refusal leaves rows already written, so it is an error
        if (st != HIPBLAS_STATUS_SUCCESS) return m0 == 0 ? false : (*err = hipErrorUnknown, true);
    }
    return true;
}

}  // namespace gdn
