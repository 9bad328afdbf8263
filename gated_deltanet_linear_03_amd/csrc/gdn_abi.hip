// gdn_abi.hip -- C-ABI front end: argument validation, workspace carving and
// dispatch to the compiled kernel instantiations.  No allocation, no host
// synchronisation (except the self-test and the snapshot calls), no exceptions
// across the ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_kernels.hpp"

// Device scratch of gdn_prefill_noalloc, one copy per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t act_size(int32_t dt) { return dt == GDN_DTYPE_BF16 ? 2 : 4; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// [lo, hi) byte ranges overlap partially (identical ranges are allowed).
bool bad_alias(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    if (a0 == b0 && na == nb) return false;
    return a0 < b0 + nb && b0 < a0 + na;
}

// [lo, hi) byte ranges share any byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// An output buffer (out, core_out) that shares bytes with a recurrent or
// conv state would be overwritten, or overwrite it, while the kernels run.
bool output_hits_state(const void* o, size_t no, const void* s_in, const void* s_out, size_t ns,
                       const void* c_in, const void* c_out, size_t nc) {
    return overlaps(o, no, s_in, ns) || overlaps(o, no, s_out, ns) || overlaps(o, no, c_in, nc) ||
           overlaps(o, no, c_out, nc);
}

gdn_status check_layer(const gdn_layer* L, bool prefill) {
    if (!L) return fail(GDN_ERR_INVALID_ARGUMENT, "layer is NULL");
    if (L->Hk <= 0 || L->Hv <= 0 || L->dk <= 0 || L->dv <= 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "head counts and dims must be positive (Hk=%d Hv=%d dk=%d dv=%d)",
                    L->Hk, L->Hv, L->dk, L->dv);
    if (L->Hv % L->Hk != 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "Hv (%d) must be a multiple of Hk (%d)", L->Hv, L->Hk);
    if (L->conv_K != 4) return fail(GDN_ERR_UNSUPPORTED, "conv_K=%d not compiled (only 4)", L->conv_K);
    if (L->act_dtype != GDN_DTYPE_FP32 && L->act_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_INVALID_ARGUMENT, "act_dtype %d unknown", L->act_dtype);
    if (L->out_dtype != GDN_DTYPE_FP32 && L->out_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_INVALID_ARGUMENT, "out_dtype %d unknown", L->out_dtype);
    if (!(L->eps_l2 >= 0.f) || !(L->eps_rms >= 0.f))
        return fail(GDN_ERR_INVALID_ARGUMENT, "epsilons must be >= 0");
    if (!L->conv_w || !L->A_log || !L->dt_bias || !L->norm_w)
        return fail(GDN_ERR_INVALID_ARGUMENT, "layer parameter pointer is NULL");
    if (!aligned(L->conv_w, 16) || !aligned(L->A_log, 4) || !aligned(L->dt_bias, 4) ||
        !aligned(L->norm_w, 4))
        return fail(GDN_ERR_INVALID_ARGUMENT, "conv_w must be 16-byte aligned, other parameters 4-byte");
    if (prefill) {
        if (L->chunk <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "chunk must be positive");
        if (!gdn::prefill_shape_supported(L->dk, L->dv, L->chunk))
            return fail(GDN_ERR_UNSUPPORTED, "prefill shape dk=%d dv=%d chunk=%d not compiled",
                        L->dk, L->dv, L->chunk);
    } else if (!gdn::decode_shape_supported(L->dk, L->dv)) {
        return fail(GDN_ERR_UNSUPPORTED, "decode shape dk=%d dv=%d not compiled", L->dk, L->dv);
    }
    return GDN_OK;
}

struct WsLayout {
    int64_t max_chunks = 0, win_slots = 0;
    int64_t off_chunk = 0, off_sink = 0, off_decay = 0, off_core = 0, off_carry = 0, off_vch = 0;
    int64_t slot_bytes = 0, total = 0;
};

// Workspace: chunk table, store sink, per-chunk decays, the fp32 pre-norm
// output when the caller gives no core_out, two state carry slots, and the
// operand blocks of one window of win_slots chunk slots (win_slots = 0:
// the default window).
WsLayout ws_layout(const gdn_layer* L, int32_t N, int64_t T, bool need_core, int64_t win_slots) {
    WsLayout w;
    // sum_n ceil(L_n / C) <= (T + N (C - 1)) / C for every split of T into N lengths
    w.max_chunks = L->chunk > 0 ? (T + static_cast<int64_t>(N) * (L->chunk - 1)) / L->chunk : N;
    w.win_slots = win_slots > 0 ? win_slots
                                : gdn::prefill_window_slots(L->dk, L->dv, L->chunk, L->Hk, L->Hv, N,
                                                            w.max_chunks, gdn::compute_units());
    w.slot_bytes = static_cast<int64_t>(L->Hv) * gdn::vch_bytes(L->dk, L->dv, L->chunk);
    int64_t o = 0;
    w.off_chunk = o;
    o = round_up(o + 4 * (static_cast<int64_t>(N) + 1), 256);
    w.off_sink = o;                       // 64 floats that absorb masked-off stores
    o += 256;
    w.off_decay = o;
    o = round_up(o + 4 * w.max_chunks * L->Hv, 256);
    w.off_core = o;
    if (need_core) o = round_up(o + 2 * T * L->Hv * L->dv, 256);   // o as fp16
    w.off_carry = o;
    o = round_up(o + 2ll * 4 * L->Hv * L->dk * L->dv, 256);
    w.off_vch = o;
    o += w.win_slots * w.slot_bytes;
    w.total = round_up(o, 256);
    return w;
}

int64_t stride_or(int64_t s, int64_t dense) { return s == 0 ? dense : s; }

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }
static_assert(gdn::kStatusBadIndex == GDN_STATUS_BAD_INDEX, "status bits of the kernels and the header");
static_assert(gdn::kGemmAuto == GDN_GEMM_AUTO && gdn::kGemmTiled == GDN_GEMM_TILED &&
                  gdn::kGemmSkinny == GDN_GEMM_FEW_ROWS && gdn::kGemmLibrary == GDN_GEMM_LIBRARY &&
                  gdn::kGemmLibraryFew == GDN_GEMM_LIBRARY_FEW_ROWS,
              "GEMM paths of the kernels and the header");

const char* gdn_status_string(gdn_status st) {
    switch (st) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* gdn_last_error(void) { return g_err; }

size_t gdn_prefill_workspace_bytes(const gdn_layer* L, int32_t N, int64_t T) {
    g_err[0] = 0;
    if (check_layer(L, true) != GDN_OK) return 0;
    if (N < 0 || T < 0) {
        fail(GDN_ERR_INVALID_ARGUMENT, "N and T_total must be >= 0");
        return 0;
    }
    // sized for the case without a caller core_out (the larger one)
    return static_cast<size_t>(ws_layout(L, N, T, true, 0).total);
}

// Window for the workspace the caller gave: the default one, or a smaller
// one when the workspace holds fewer operand blocks (at least one slot).
static gdn_status fit_workspace(const gdn_layer* L, int32_t N, int64_t T, bool need_core, const void* ws,
                                size_t ws_bytes, WsLayout* out) {
    WsLayout w = ws_layout(L, N, T, need_core, 0);
    if (w.max_chunks > (int64_t(1) << 30)) return fail(GDN_ERR_INVALID_ARGUMENT, "too many chunks");
    if (!ws) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (need %lld bytes)", static_cast<long long>(w.total));
    if (!aligned(ws, 256)) return fail(GDN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < static_cast<size_t>(w.total)) {
        const int64_t fits = (static_cast<int64_t>(ws_bytes) - w.off_vch) / w.slot_bytes;
        if (fits < 1)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, need %lld (at least %lld)", ws_bytes,
                        static_cast<long long>(w.total), static_cast<long long>(w.off_vch + w.slot_bytes));
        w = ws_layout(L, N, T, need_core, fits);
    }
    *out = w;
    return GDN_OK;
}

static gdn_status prefill_impl(const gdn_layer* L, const gdn_prefill_io* io, void* ws,
                               size_t ws_bytes, void* stream, hipEvent_t const* events,
                               bool launch = true) {
    g_err[0] = 0;
    gdn_status st = check_layer(L, true);
    if (st != GDN_OK) return st;
    if (!io) return fail(GDN_ERR_INVALID_ARGUMENT, "io is NULL");
    const int32_t N = io->N;
    const int64_t T = io->T_total;
    if (N < 0 || T < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "N (%d) and T_total (%lld) must be >= 0",
                                    N, static_cast<long long>(T));
    if (T > 0 && N == 0) return fail(GDN_ERR_INVALID_ARGUMENT, "T_total > 0 with N == 0");
    if (T >= (int64_t(1) << 31)) return fail(GDN_ERR_INVALID_ARGUMENT, "T_total must be < 2^31");
    if (N > 0 && !io->cu_seqlens) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    const size_t es = act_size(L->act_dtype);
    const int Hk = L->Hk, Hv = L->Hv, dk = L->dk, dv = L->dv;
    if (T > 0) {
        if (!io->q || !io->k || !io->v || !io->z || !io->a || !io->b)
            return fail(GDN_ERR_INVALID_ARGUMENT, "a token input pointer is NULL");
        if (!io->out) return fail(GDN_ERR_INVALID_ARGUMENT, "out is NULL");
        if (!aligned(io->q, 16) || !aligned(io->k, 16) || !aligned(io->v, 16) || !aligned(io->z, 16) ||
            !aligned(io->out, 16) || (io->core_out && !aligned(io->core_out, 16)))
            return fail(GDN_ERR_INVALID_ARGUMENT, "q/k/v/z/out/core_out must be 16-byte aligned");
        if (!aligned(io->a, es) || !aligned(io->b, es))
            return fail(GDN_ERR_INVALID_ARGUMENT, "a/b must be element aligned");
    }
    const int64_t qs = stride_or(io->q_stride, int64_t(Hk) * dk), ks = stride_or(io->k_stride, int64_t(Hk) * dk);
    const int64_t vs = stride_or(io->v_stride, int64_t(Hv) * dv), zs = stride_or(io->z_stride, int64_t(Hv) * dv);
    const int64_t as = stride_or(io->a_stride, Hv), bs = stride_or(io->b_stride, Hv);
    if (qs < int64_t(Hk) * dk || ks < int64_t(Hk) * dk || vs < int64_t(Hv) * dv || zs < int64_t(Hv) * dv ||
        as < Hv || bs < Hv)
        return fail(GDN_ERR_INVALID_ARGUMENT, "a token stride is smaller than one token's row");
    if (qs % 8 || ks % 8 || vs % 8 || zs % 8)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q/k/v/z strides must be multiples of 8 elements");
    if (io->state_slots && io->num_slots < N)
        return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots (%d) < N (%d) with state_slots", io->num_slots, N);
    const int64_t entries = io->state_slots ? io->num_slots : N;    // state pool size
    const size_t state_bytes = size_t(entries) * Hv * dk * dv * 4;
    const int64_t Cc = 2ll * Hk * dk + int64_t(Hv) * dv;
    const size_t conv_bytes = size_t(entries) * 3 * Cc * es;
    if ((io->initial_state && !aligned(io->initial_state, 16)) || (io->final_state && !aligned(io->final_state, 16)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "states must be 16-byte aligned");
    if ((io->conv_state_in && !aligned(io->conv_state_in, 16)) ||
        (io->conv_state_out && !aligned(io->conv_state_out, 16)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "conv states must be 16-byte aligned");
    if (bad_alias(io->initial_state, state_bytes, io->final_state, state_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "final_state partially overlaps initial_state");
    if (bad_alias(io->conv_state_in, conv_bytes, io->conv_state_out, conv_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "conv_state_out partially overlaps conv_state_in");
    const size_t out_bytes = size_t(T) * Hv * dv * (L->out_dtype == GDN_DTYPE_BF16 ? 2 : 4);
    if (io->core_out && bad_alias(io->out, out_bytes, io->core_out, size_t(T) * Hv * dv * 4) &&
        static_cast<const void*>(io->out) != static_cast<const void*>(io->core_out))
        return fail(GDN_ERR_INVALID_ARGUMENT, "out overlaps core_out");
    if (io->core_out && static_cast<const void*>(io->out) == static_cast<const void*>(io->core_out) && T > 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "out and core_out must be different buffers");
    if (output_hits_state(io->out, out_bytes, io->initial_state, io->final_state, state_bytes,
                          io->conv_state_in, io->conv_state_out, conv_bytes) ||
        output_hits_state(io->core_out, size_t(T) * Hv * dv * 4, io->initial_state, io->final_state,
                          state_bytes, io->conv_state_in, io->conv_state_out, conv_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "out or core_out overlaps a state");
    if (io->status) {
        if (!aligned(io->status, 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "status must be 4-byte aligned");
        if (overlaps(io->status, 4, io->out, out_bytes) ||
            overlaps(io->status, 4, io->core_out, size_t(T) * Hv * dv * 4) ||
            output_hits_state(io->status, 4, io->initial_state, io->final_state, state_bytes, io->conv_state_in,
                              io->conv_state_out, conv_bytes) ||
            overlaps(io->status, 4, ws, ws_bytes))
            return fail(GDN_ERR_INVALID_ARGUMENT, "status overlaps an output, a state or the workspace");
    }

    WsLayout w;
    st = fit_workspace(L, N, T, io->core_out == nullptr, ws, ws_bytes, &w);
    if (st != GDN_OK) return st;

    gdn::PrefillParams p{};
    p.N = N; p.Hk = Hk; p.Hv = Hv; p.G = Hv / Hk; p.T = T;
    p.max_chunks = static_cast<int>(w.max_chunks);
    p.scale = L->scale; p.eps_l2 = L->eps_l2; p.eps_rms = L->eps_rms;
    p.cu = io->cu_seqlens;
    p.conv_w = L->conv_w; p.A_log = L->A_log; p.dt_bias = L->dt_bias; p.norm_w = L->norm_w;
    p.q = io->q; p.k = io->k; p.v = io->v; p.z = io->z; p.a = io->a; p.b = io->b;
    p.qs = qs; p.ks = ks; p.vs = vs; p.zs = zs; p.as = as; p.bs = bs;
    p.state_in = io->initial_state; p.state_out = io->final_state;
    p.conv_in = io->conv_state_in; p.conv_out = io->conv_state_out;
    p.out = io->out; p.out_bf16 = L->out_dtype == GDN_DTYPE_BF16;
    uint8_t* base = static_cast<uint8_t*>(ws);
    p.core = io->core_out ? io->core_out : reinterpret_cast<float*>(base + w.off_core);
    p.core_f16 = io->core_out ? 0 : 1;
    p.slots = io->state_slots;
    p.num_slots = static_cast<int>(entries);
    p.status = io->status;
    p.chunk_off = reinterpret_cast<int32_t*>(base + w.off_chunk);
    p.decay = reinterpret_cast<float*>(base + w.off_decay);
    p.sink = reinterpret_cast<float*>(base + w.off_sink);
    p.carry = reinterpret_cast<float*>(base + w.off_carry);
    p.vch = base + w.off_vch;
    p.win_slots = static_cast<int>(w.win_slots);
    if (!launch) return GDN_OK;

    bool supported = false;
    hipError_t e = gdn::launch_prefill(dk, dv, L->chunk, L->act_dtype == GDN_DTYPE_BF16, p,
                                       static_cast<hipStream_t>(stream), &supported, events);
    if (!supported) return fail(GDN_ERR_UNSUPPORTED, "prefill shape not compiled");
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_prefill(const gdn_layer* L, const gdn_prefill_io* io, void* ws, size_t ws_bytes,
                       void* stream) {
    return prefill_impl(L, io, ws, ws_bytes, stream, nullptr);
}

// Device address of `scratch` on the stream's device, looked up with that
// device current on the first call there and kept per device.
static gdn_status noalloc_scratch(void* stream, void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
        if (static_cast<int>(sd) != cur)
            return fail(GDN_ERR_INVALID_ARGUMENT, "the stream belongs to device %d, device %d is current: "
                        "make the stream's device current", static_cast<int>(sd), cur);
    }
    if (cur < 0 || cur >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device index %d >= %d", cur, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[cur]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        addr[cur] = ptr;
    }
    *out = addr[cur];
    return GDN_OK;
}

gdn_status gdn_prefill_noalloc(const gdn_layer* L, const gdn_prefill_io* io, void* stream) {
    g_err[0] = 0;
    void* ws = nullptr;
    gdn_status st = noalloc_scratch(stream, &ws);
    if (st != GDN_OK) return st;
    st = prefill_impl(L, io, ws, GDN_NOALLOC_SCRATCH_BYTES, stream, nullptr);
    if (st == GDN_ERR_WORKSPACE) {
        char detail[sizeof g_err];
        memcpy(detail, g_err, sizeof detail);
        return fail(GDN_ERR_WORKSPACE, "gdn_prefill_noalloc: its %llu-byte scratch is too small for these "
                    "sizes (%s)", static_cast<unsigned long long>(GDN_NOALLOC_SCRATCH_BYTES), detail);
    }
    return st;
}

// The layout gdn_prefill fits into a workspace of ws_bytes (which depends
// only on its size, not on where it is), or -1.
static int64_t planned_layout(const gdn_layer* L, int32_t N, int64_t T, size_t ws_bytes, int32_t with_core,
                              WsLayout* w) {
    g_err[0] = 0;
    if (check_layer(L, true) != GDN_OK) return -1;
    if (N < 0 || T < 0) {
        fail(GDN_ERR_INVALID_ARGUMENT, "N and T_total must be >= 0");
        return -1;
    }
    static const uint8_t probe[256] __attribute__((aligned(256))) = {0};
    if (fit_workspace(L, N, T, with_core == 0, probe, ws_bytes, w) != GDN_OK) return -1;
    return 0;
}

int64_t gdn_prefill_launches(const gdn_layer* L, int32_t N, int64_t T, size_t ws_bytes, int32_t with_core) {
    WsLayout w;
    if (planned_layout(L, N, T, ws_bytes, with_core, &w) < 0) return -1;
    return gdn::prefill_launches(w.max_chunks, w.win_slots);
}

int64_t gdn_prefill_window_slots(const gdn_layer* L, int32_t N, int64_t T, size_t ws_bytes, int32_t with_core) {
    WsLayout w;
    if (planned_layout(L, N, T, ws_bytes, with_core, &w) < 0) return -1;
    return w.win_slots;
}

gdn_status gdn_prefill_timed(const gdn_layer* L, const gdn_prefill_io* io, void* ws,
                             size_t ws_bytes, void* stream, void* const* events, int n_events) {
    g_err[0] = 0;
    gdn_status st = check_layer(L, true);
    if (st != GDN_OK) return st;
    if (!io) return fail(GDN_ERR_INVALID_ARGUMENT, "io is NULL");
    WsLayout w;
    st = fit_workspace(L, io->N, io->T_total, io->core_out == nullptr, ws, ws_bytes, &w);
    if (st != GDN_OK) return st;
    const int64_t need = gdn::prefill_launches(w.max_chunks, w.win_slots) + 1;
    if (!events || n_events != need)
        return fail(GDN_ERR_INVALID_ARGUMENT, "need %lld timing events", static_cast<long long>(need));
    for (int i = 0; i < n_events; ++i)
        if (!events[i]) return fail(GDN_ERR_INVALID_ARGUMENT, "timing event %d is NULL", i);
    return prefill_impl(L, io, ws, ws_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
}


// The decode workspace: the arrival counters [B][Hk] uint32 of the
// one-work-group-per-value-head kernel, rounded up to 256 bytes.  Counter
// (b, hk) sits at the same place for every B, so a workspace sized for B
// serves every smaller batch.
static size_t decode_ws_bytes(const gdn_layer* L, int32_t B) {
    return (size_t(B) * L->Hk * 4 + 255) / 256 * 256;
}


size_t gdn_decode_workspace_bytes(const gdn_layer* L, int32_t B) {
    g_err[0] = 0;
    if (check_layer(L, false) != GDN_OK) return 0;
    if (B < 0) {
        fail(GDN_ERR_INVALID_ARGUMENT, "B (%d) must be >= 0", B);
        return 0;
    }
    return B == 0 ? 256 : decode_ws_bytes(L, B);
}

// Ts = 0: one token per sequence (gdn_decode); Ts >= 1: the multi-token kernel.
static gdn_status decode_impl(const gdn_layer* L, const gdn_decode_io* io, int32_t Ts, float* snap,
                              void* stream, bool launch = true) {
    gdn_status st = check_layer(L, false);
    if (st != GDN_OK) return st;
    if (!io) return fail(GDN_ERR_INVALID_ARGUMENT, "io is NULL");
    const int32_t B = io->B;
    if (B < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "B (%d) must be >= 0", B);
    if (B == 0) return GDN_OK;
    const int Hk = L->Hk, Hv = L->Hv, dk = L->dk, dv = L->dv;
    const size_t es = act_size(L->act_dtype);
    if (!io->q || !io->k || !io->v || !io->z || !io->a || !io->b)
        return fail(GDN_ERR_INVALID_ARGUMENT, "a token input pointer is NULL");
    if (!io->out || !io->state_out || !io->conv_state_out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "out, state_out and conv_state_out are required");
    if (!aligned(io->out, 16) || !aligned(io->state_out, 16) || !aligned(io->conv_state_out, 16) ||
        (io->state_in && !aligned(io->state_in, 16)) || (io->conv_state_in && !aligned(io->conv_state_in, 16)) ||
        (io->core_out && !aligned(io->core_out, 16)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "out/core_out/states must be 16-byte aligned");
    if (!aligned(io->q, es) || !aligned(io->k, es) || !aligned(io->v, es) || !aligned(io->z, es) ||
        !aligned(io->a, es) || !aligned(io->b, es))
        return fail(GDN_ERR_INVALID_ARGUMENT, "token inputs must be element aligned");
    const int64_t qs = stride_or(io->q_stride, int64_t(Hk) * dk), ks = stride_or(io->k_stride, int64_t(Hk) * dk);
    const int64_t vs = stride_or(io->v_stride, int64_t(Hv) * dv), zs = stride_or(io->z_stride, int64_t(Hv) * dv);
    const int64_t as = stride_or(io->a_stride, Hv), bs = stride_or(io->b_stride, Hv);
    if (qs < int64_t(Hk) * dk || ks < int64_t(Hk) * dk || vs < int64_t(Hv) * dv || zs < int64_t(Hv) * dv ||
        as < Hv || bs < Hv)
        return fail(GDN_ERR_INVALID_ARGUMENT, "a token stride is smaller than one token's row");
    if (io->state_slots && io->num_slots < B)
        return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots (%d) < B (%d) with state_slots", io->num_slots, B);
    const int64_t entries = io->state_slots ? io->num_slots : B;    // state pool size
    const size_t state_bytes = size_t(entries) * Hv * dk * dv * 4;
    const int64_t Cc = 2ll * Hk * dk + int64_t(Hv) * dv;
    const size_t conv_bytes = size_t(entries) * 3 * Cc * es;
    if (bad_alias(io->state_in, state_bytes, io->state_out, state_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "state_out partially overlaps state_in");
    if (bad_alias(io->conv_state_in, conv_bytes, io->conv_state_out, conv_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "conv_state_out partially overlaps conv_state_in");
    if (static_cast<int64_t>(B) * Hk >= (int64_t(1) << 31) || static_cast<int64_t>(B) * Ts >= (int64_t(1) << 31))
        return fail(GDN_ERR_INVALID_ARGUMENT, "B * Hk or B * tokens too large");
    {
        const size_t rows = size_t(B) * (Ts > 0 ? Ts : 1);
        const size_t ob = rows * Hv * dv * (L->out_dtype == GDN_DTYPE_BF16 ? 2 : 4);
        if (output_hits_state(io->out, ob, io->state_in, io->state_out, state_bytes, io->conv_state_in,
                              io->conv_state_out, conv_bytes) ||
            output_hits_state(io->core_out, rows * Hv * dv * 4, io->state_in, io->state_out, state_bytes,
                              io->conv_state_in, io->conv_state_out, conv_bytes))
            return fail(GDN_ERR_INVALID_ARGUMENT, "out or core_out overlaps a state");
    }
    const size_t dws_need = decode_ws_bytes(L, B);
    // with a workspace, one work-group per value head (measured as fast or
    // faster at every batch size; the same bits either way)
    const bool head_wg = Ts == 0 && io->workspace != nullptr;
    if (Ts == 0 && io->workspace) {
        if (!aligned(io->workspace, 256))
            return fail(GDN_ERR_WORKSPACE, "decode workspace must be 256-byte aligned");
        if (io->workspace_bytes < dws_need)
            return fail(GDN_ERR_WORKSPACE, "decode workspace of %zu bytes, B = %d needs %zu", io->workspace_bytes,
                        B, dws_need);
        const size_t ob = size_t(B) * Hv * dv * (L->out_dtype == GDN_DTYPE_BF16 ? 2 : 4);
        if (overlaps(io->workspace, io->workspace_bytes, io->state_in, state_bytes) ||
            overlaps(io->workspace, io->workspace_bytes, io->state_out, state_bytes) ||
            overlaps(io->workspace, io->workspace_bytes, io->conv_state_in, conv_bytes) ||
            overlaps(io->workspace, io->workspace_bytes, io->conv_state_out, conv_bytes) ||
            overlaps(io->workspace, io->workspace_bytes, io->out, ob) ||
            overlaps(io->workspace, io->workspace_bytes, io->core_out, size_t(B) * Hv * dv * 4))
            return fail(GDN_ERR_INVALID_ARGUMENT, "decode workspace overlaps a state or an output");
    }
    if (io->status) {
        const size_t rows = size_t(B) * (Ts > 0 ? Ts : 1);
        const size_t ob = rows * Hv * dv * (L->out_dtype == GDN_DTYPE_BF16 ? 2 : 4);
        if (!aligned(io->status, 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "status must be 4-byte aligned");
        if (overlaps(io->status, 4, io->out, ob) || overlaps(io->status, 4, io->core_out, rows * Hv * dv * 4) ||
            output_hits_state(io->status, 4, io->state_in, io->state_out, state_bytes, io->conv_state_in,
                              io->conv_state_out, conv_bytes) ||
            (head_wg && overlaps(io->status, 4, io->workspace, io->workspace_bytes)))
            return fail(GDN_ERR_INVALID_ARGUMENT, "status overlaps an output, a state or the workspace");
    }
    if (snap) {
        const size_t snap_bytes = size_t(B) * Ts * Hv * dk * dv * 4;
        if (!aligned(snap, 16)) return fail(GDN_ERR_INVALID_ARGUMENT, "state_snapshots must be 16-byte aligned");
        if (overlaps(snap, snap_bytes, io->state_in, state_bytes) ||
            overlaps(snap, snap_bytes, io->state_out, state_bytes))
            return fail(GDN_ERR_INVALID_ARGUMENT, "state_snapshots overlaps a state");
    }

    gdn::DecodeParams p{};
    p.B = B; p.Hk = Hk; p.Hv = Hv; p.G = Hv / Hk;
    p.scale = L->scale; p.eps_l2 = L->eps_l2; p.eps_rms = L->eps_rms;
    p.conv_w = L->conv_w; p.A_log = L->A_log; p.dt_bias = L->dt_bias; p.norm_w = L->norm_w;
    p.q = io->q; p.k = io->k; p.v = io->v; p.z = io->z; p.a = io->a; p.b = io->b;
    p.qs = qs; p.ks = ks; p.vs = vs; p.zs = zs; p.as = as; p.bs = bs;
    p.state_in = io->state_in; p.state_out = io->state_out;
    p.conv_in = io->conv_state_in; p.conv_out = io->conv_state_out;
    p.out = io->out; p.out_bf16 = L->out_dtype == GDN_DTYPE_BF16; p.core_out = io->core_out;
    p.Ts = Ts; p.snap = snap;     // Ts = 0: the one-token kernel
    p.slots = io->state_slots;
    p.num_slots = static_cast<int>(entries);
    p.status = io->status;
    if (head_wg) p.arrive = static_cast<uint32_t*>(io->workspace);
    if (!launch) return GDN_OK;
    bool supported = false;
    hipError_t e = gdn::launch_decode(dk, dv, L->act_dtype == GDN_DTYPE_BF16, p,
                                      static_cast<hipStream_t>(stream), &supported);
    if (!supported) return fail(GDN_ERR_UNSUPPORTED, "decode shape not compiled");
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_decode(const gdn_layer* L, const gdn_decode_io* io, void* stream) {
    g_err[0] = 0;
    return decode_impl(L, io, 0, nullptr, stream);
}

gdn_status gdn_step(const gdn_layer* L, const gdn_prefill_io* prefill, const gdn_decode_io* decode,
                    void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const bool has_d = decode && decode->B > 0;
    const bool has_p = prefill && (prefill->N > 0 || prefill->T_total > 0);
    gdn_status st = GDN_OK;
    if (has_d && (st = decode_impl(L, decode, 0, nullptr, stream, false)) != GDN_OK) return st;
    if (has_p && (st = prefill_impl(L, prefill, ws, ws_bytes, stream, nullptr, false)) != GDN_OK) return st;
    if (has_d && has_p && decode->workspace && overlaps(decode->workspace, decode->workspace_bytes, ws, ws_bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "the decode and prefill workspaces overlap");
    if (has_d && (st = decode_impl(L, decode, 0, nullptr, stream)) != GDN_OK) return st;
    if (has_p && (st = prefill_impl(L, prefill, ws, ws_bytes, stream, nullptr)) != GDN_OK) return st;
    return GDN_OK;
}

gdn_status gdn_decode_multi(const gdn_layer* L, const gdn_decode_io* io, int32_t tokens,
                            float* state_snapshots, void* stream) {
    g_err[0] = 0;
    if (tokens < 1 || tokens > gdn::kMaxVerifyTokens)
        return fail(GDN_ERR_INVALID_ARGUMENT, "tokens (%d) must be in [1, %d]", tokens, gdn::kMaxVerifyTokens);
    return decode_impl(L, io, tokens, state_snapshots, stream);
}

// ---- projections and the whole layer ---------------------------------------

gdn_status gdn_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                         int32_t c_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    return gdn_gemm_bf16_path(A, lda, B, ldb, C, ldc, c_dtype, M, N, K, GDN_GEMM_AUTO, stream);
}

gdn_status gdn_gemm_bf16_path(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                              int32_t c_dtype, int64_t M, int64_t N, int64_t K, int32_t path, void* stream) {
    g_err[0] = 0;
    if (path < GDN_GEMM_AUTO || path > GDN_GEMM_LIBRARY_FEW_ROWS) return fail(GDN_ERR_INVALID_ARGUMENT, "path %d unknown", path);
    if (M < 0 || N < 0 || K < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "M, N, K must be >= 0");
    if (c_dtype != GDN_DTYPE_BF16 && c_dtype != GDN_DTYPE_FP32)
        return fail(GDN_ERR_INVALID_ARGUMENT, "c_dtype %d unknown", c_dtype);
    if (M == 0 || N == 0) return GDN_OK;
    if (!A || !B || !C) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL operand");
    if (K % 8 || lda % 8 || ldb % 8 || !aligned(A, 16) || !aligned(B, 16))
        return fail(GDN_ERR_INVALID_ARGUMENT, "K, lda and ldb must be multiples of 8 and A, B 16-byte aligned");
    if (lda < K || ldb < K || ldc < N) return fail(GDN_ERR_INVALID_ARGUMENT, "leading dimension below the row length");
    if (!aligned(C, c_dtype == GDN_DTYPE_BF16 ? 2 : 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "C misaligned");
    hipError_t e = gdn::launch_gemm_bf16_nt(A, lda, B, ldb, C, ldc, c_dtype == GDN_DTYPE_BF16, M, N, K,
                                            static_cast<hipStream_t>(stream), static_cast<gdn::GemmPath>(path));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "gemm launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

namespace {

struct LayerWs {
    int64_t P = 0, off_proj = 0, off_gated = 0, off_pf = 0, total = 0;
};

// Decode only: arrival counters of the one-work-group-per-value-head
// decode kernel at the start of the workspace, at a place and size that do
// not depend on B (up to this many (sequence, key head) pairs; beyond, the
// step runs one work-group per key head and needs none)
constexpr int64_t kLayerDecodeCounterBytes = 64 << 10;

// (decode: the counters,) the projection [rows][P] and the gated output
// [rows][Hv*dv], bf16
gdn_status proj_ws(const gdn_layer* L, const gdn_proj* pr, int64_t rows, bool prefill, LayerWs* w) {
    gdn_status st = check_layer(L, prefill);
    if (st != GDN_OK) return st;
    if (!pr) return fail(GDN_ERR_INVALID_ARGUMENT, "proj is NULL");
    if (pr->hidden <= 0 || pr->hidden % 8)
        return fail(GDN_ERR_INVALID_ARGUMENT, "hidden (%d) must be a positive multiple of 8", pr->hidden);
    if (L->act_dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_INVALID_ARGUMENT, "the layer path needs act_dtype bf16");
    if (rows < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "row count must be >= 0");
    w->P = 2ll * L->Hk * L->dk + 2ll * L->Hv * L->dv + 2ll * L->Hv;
    if ((2ll * L->Hk * L->dk) % 8 || (static_cast<int64_t>(L->Hv) * L->dv) % 8 || w->P % 8)
        return fail(GDN_ERR_INVALID_ARGUMENT, "projection widths must be multiples of 8");
    int64_t o = prefill ? 0 : kLayerDecodeCounterBytes;
    w->off_proj = o;
    o = round_up(o + 2 * rows * w->P, 256);
    w->off_gated = o;
    o = round_up(o + 2 * rows * static_cast<int64_t>(L->Hv) * L->dv, 256);
    w->off_pf = o;
    w->total = o;
    return GDN_OK;
}


gdn_status layer_ws(const gdn_layer* L, const gdn_proj* pr, int32_t N, int64_t T, LayerWs* w) {
    if (N < 0 || T < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "N and T_total must be >= 0");
    gdn_status st = proj_ws(L, pr, T, true, w);
    if (st != GDN_OK) return st;
    w->total = w->off_pf + ws_layout(L, N, T, true, 0).total;
    return GDN_OK;
}

}  // namespace

size_t gdn_layer_prefill_workspace_bytes(const gdn_layer* L, const gdn_proj* pr, int32_t N, int64_t T) {
    g_err[0] = 0;
    LayerWs w;
    if (layer_ws(L, pr, N, T, &w) != GDN_OK) return 0;
    return static_cast<size_t>(w.total);
}

gdn_status gdn_layer_prefill(const gdn_layer* L, const gdn_proj* pr, const gdn_layer_io* io, void* ws,
                             size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!io) return fail(GDN_ERR_INVALID_ARGUMENT, "io is NULL");
    LayerWs w;
    gdn_status st = layer_ws(L, pr, io->N, io->T_total, &w);
    if (st != GDN_OK) return st;
    const int64_t T = io->T_total;
    const int64_t HD = static_cast<int64_t>(L->Hv) * L->dv;
    if (T > 0 && (!io->x || !io->y || !pr->w_in || !pr->w_out))
        return fail(GDN_ERR_INVALID_ARGUMENT, "x, y, w_in and w_out are required");
    if (io->y_dtype != GDN_DTYPE_BF16 && io->y_dtype != GDN_DTYPE_FP32)
        return fail(GDN_ERR_INVALID_ARGUMENT, "y_dtype %d unknown", io->y_dtype);
    if (T > 0 && (!aligned(io->x, 16) || !aligned(pr->w_in, 16) || !aligned(pr->w_out, 16) || !aligned(io->y, 16)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "x, y, w_in and w_out must be 16-byte aligned");
    if (!ws || !aligned(ws, 256)) return fail(GDN_ERR_WORKSPACE, "workspace missing or not 256-byte aligned");
    if (static_cast<int64_t>(ws_bytes) < w.off_pf)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, the layer needs %lld", ws_bytes,
                    static_cast<long long>(w.total));
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* proj = reinterpret_cast<uint16_t*>(base + w.off_proj);
    uint16_t* gated = reinterpret_cast<uint16_t*>(base + w.off_gated);
    const int64_t qk = static_cast<int64_t>(L->Hk) * L->dk;

    gdn_layer Lg = *L;                  // the gated output feeds out_proj as bf16
    Lg.out_dtype = GDN_DTYPE_BF16;
    gdn_prefill_io pio{};
    pio.N = io->N;
    pio.T_total = T;
    pio.cu_seqlens = io->cu_seqlens;
    pio.q = proj;
    pio.k = proj + qk;
    pio.v = proj + 2 * qk;
    pio.z = proj + 2 * qk + HD;
    pio.a = proj + 2 * qk + 2 * HD;
    pio.b = proj + 2 * qk + 2 * HD + L->Hv;
    pio.q_stride = pio.k_stride = pio.v_stride = pio.z_stride = pio.a_stride = pio.b_stride = w.P;
    pio.initial_state = io->initial_state;
    pio.final_state = io->final_state;
    pio.conv_state_in = io->conv_state_in;
    pio.conv_state_out = io->conv_state_out;
    pio.out = gated;
    pio.core_out = nullptr;
    pio.state_slots = io->state_slots;
    pio.num_slots = io->num_slots;
    pio.status = io->status;
    // The prefill inside the layer runs windows of half the default size:
    // in_proj's output, just written, shares the Infinity Cache with the
    // operand blocks here (measured at 4096 tokens: 0.463 ms per layer step
    // with 32-slot windows, 0.492 with 64).  Only the window changes, not
    // the bits.
    const WsLayout pw = ws_layout(&Lg, io->N, T, true, 0);
    const size_t pf_cap = static_cast<size_t>(pw.off_vch + std::max<int64_t>(1, pw.win_slots / 2) * pw.slot_bytes);
    const size_t pf_bytes = std::min(ws_bytes - w.off_pf, pf_cap);
    // validate the prefill part before enqueueing anything
    st = prefill_impl(&Lg, &pio, base + w.off_pf, pf_bytes, stream, nullptr, false);
    if (st != GDN_OK) return st;
    if (T == 0) return prefill_impl(&Lg, &pio, base + w.off_pf, pf_bytes, stream, nullptr);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // one kernel family at every T (the library's pinned algorithm): a
    // sequence's bits do not depend on how many tokens share the call
    hipError_t e = gdn::launch_gemm_bf16_nt(io->x, pr->hidden, pr->w_in, pr->hidden, proj, w.P, true, T, w.P,
                                            pr->hidden, s, gdn::kGemmLibrary);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "in_proj launch failed: %s", hipGetErrorString(e));
    st = prefill_impl(&Lg, &pio, base + w.off_pf, pf_bytes, stream, nullptr);
    if (st != GDN_OK) return st;
    e = gdn::launch_gemm_bf16_nt(gated, HD, pr->w_out, HD, io->y, pr->hidden, io->y_dtype == GDN_DTYPE_BF16, T,
                                 pr->hidden, HD, s, gdn::kGemmLibrary);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "out_proj launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}


size_t gdn_layer_decode_workspace_bytes(const gdn_layer* L, const gdn_proj* pr, int32_t B) {
    g_err[0] = 0;
    LayerWs w;
    if (proj_ws(L, pr, B, false, &w) != GDN_OK) return 0;
    return static_cast<size_t>(w.total > 0 ? w.total : 256);
}

gdn_status gdn_layer_decode(const gdn_layer* L, const gdn_proj* pr, const gdn_layer_decode_io* io, void* ws,
                            size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!io) return fail(GDN_ERR_INVALID_ARGUMENT, "io is NULL");
    LayerWs w;
    gdn_status st = proj_ws(L, pr, io->B, false, &w);
    if (st != GDN_OK) return st;
    const int64_t B = io->B;
    if (B == 0) return GDN_OK;
    const int64_t HD = static_cast<int64_t>(L->Hv) * L->dv;
    if (!io->x || !io->y || !pr->w_in || !pr->w_out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "x, y, w_in and w_out are required");
    if (io->y_dtype != GDN_DTYPE_BF16 && io->y_dtype != GDN_DTYPE_FP32)
        return fail(GDN_ERR_INVALID_ARGUMENT, "y_dtype %d unknown", io->y_dtype);
    if (!aligned(io->x, 16) || !aligned(pr->w_in, 16) || !aligned(pr->w_out, 16) || !aligned(io->y, 16))
        return fail(GDN_ERR_INVALID_ARGUMENT, "x, y, w_in and w_out must be 16-byte aligned");
    if (!ws || !aligned(ws, 256)) return fail(GDN_ERR_WORKSPACE, "workspace missing or not 256-byte aligned");
    if (static_cast<int64_t>(ws_bytes) < w.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, the layer needs %lld", ws_bytes,
                    static_cast<long long>(w.total));
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* proj = reinterpret_cast<uint16_t*>(base + w.off_proj);
    uint16_t* gated = reinterpret_cast<uint16_t*>(base + w.off_gated);
    const int64_t qk = static_cast<int64_t>(L->Hk) * L->dk;
    gdn_layer Lg = *L;
    Lg.out_dtype = GDN_DTYPE_BF16;
    gdn_decode_io dio{};
    dio.B = io->B;
    dio.q = proj;
    dio.k = proj + qk;
    dio.v = proj + 2 * qk;
    dio.z = proj + 2 * qk + HD;
    dio.a = proj + 2 * qk + 2 * HD;
    dio.b = proj + 2 * qk + 2 * HD + L->Hv;
    dio.q_stride = dio.k_stride = dio.v_stride = dio.z_stride = dio.a_stride = dio.b_stride = w.P;
    dio.state_in = io->state_in;
    dio.state_out = io->state_out;
    dio.conv_state_in = io->conv_state_in;
    dio.conv_state_out = io->conv_state_out;
    dio.out = gated;
    dio.core_out = nullptr;
    dio.state_slots = io->state_slots;
    dio.num_slots = io->num_slots;
    dio.status = io->status;
    if (B * L->Hk * 4 <= kLayerDecodeCounterBytes) {
        dio.workspace = base;
        dio.workspace_bytes = static_cast<size_t>(kLayerDecodeCounterBytes);
    }
    st = decode_impl(&Lg, &dio, 0, nullptr, stream, false);
    if (st != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // one kernel family at every B (the library's algorithm pinned at 64
    // rows): a sequence's bits do not depend on the batch size
    hipError_t e = gdn::launch_gemm_bf16_nt(io->x, pr->hidden, pr->w_in, pr->hidden, proj, w.P, true, B, w.P,
                                            pr->hidden, s, gdn::kGemmLibraryFew);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "in_proj launch failed: %s", hipGetErrorString(e));
    st = decode_impl(&Lg, &dio, 0, nullptr, stream);
    if (st != GDN_OK) return st;
    e = gdn::launch_gemm_bf16_nt(gated, HD, pr->w_out, HD, io->y, pr->hidden, io->y_dtype == GDN_DTYPE_BF16, B,
                                 pr->hidden, HD, s, gdn::kGemmLibraryFew);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "out_proj launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

// ---- session snapshots ------------------------------------------------------

static_assert(sizeof(gdn_snapshot_header) == 64, "snapshot header is 64 bytes");

static uint64_t fnv1a64(const uint8_t* p, size_t n) {
    uint64_t h = 14695981039346656037ull;    // FNV-1a 64 offset basis
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;                   // FNV 64 prime
    }
    return h;
}

static void snapshot_sizes(const gdn_layer* L, uint64_t* sb, uint64_t* cb) {
    const int64_t Cc = 2ll * L->Hk * L->dk + static_cast<int64_t>(L->Hv) * L->dv;
    *sb = static_cast<uint64_t>(L->Hv) * L->dk * L->dv * 4;
    *cb = static_cast<uint64_t>(L->conv_K - 1) * Cc * act_size(L->act_dtype);
}

static gdn_status snapshot_args(const gdn_layer* L, const void* state, const void* conv, int32_t slot,
                                int32_t num_slots, const void* host, size_t host_bytes) {
    gdn_status st = check_layer(L, false);
    if (st != GDN_OK) return st;
    if (!state || !conv || !host) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL state, conv state or host buffer");
    if (num_slots <= 0 || slot < 0 || slot >= num_slots)
        return fail(GDN_ERR_INVALID_ARGUMENT, "slot %d outside [0, num_slots=%d)", slot, num_slots);
    uint64_t sb, cb;
    snapshot_sizes(L, &sb, &cb);
    if (host_bytes < sizeof(gdn_snapshot_header) + sb + cb)
        return fail(GDN_ERR_INVALID_ARGUMENT, "host buffer of %zu bytes, a snapshot needs %llu", host_bytes,
                    static_cast<unsigned long long>(sizeof(gdn_snapshot_header) + sb + cb));
    return GDN_OK;
}

size_t gdn_snapshot_bytes(const gdn_layer* L) {
    g_err[0] = 0;
    if (check_layer(L, false) != GDN_OK) return 0;
    uint64_t sb, cb;
    snapshot_sizes(L, &sb, &cb);
    return sizeof(gdn_snapshot_header) + sb + cb;
}

gdn_status gdn_snapshot_save(const gdn_layer* L, const float* state, const void* conv, int32_t slot,
                             int32_t num_slots, void* host, size_t host_bytes, void* stream) {
    g_err[0] = 0;
    gdn_status st = snapshot_args(L, state, conv, slot, num_slots, host, host_bytes);
    if (st != GDN_OK) return st;
    uint64_t sb, cb;
    snapshot_sizes(L, &sb, &cb);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* payload = static_cast<uint8_t*>(host) + sizeof(gdn_snapshot_header);
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(payload, reinterpret_cast<const uint8_t*>(state) + sb * slot, sb,
                           hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(payload + sb, static_cast<const uint8_t*>(conv) + cb * slot, cb,
                           hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "snapshot copy failed: %s", hipGetErrorString(e));
    gdn_snapshot_header hd{};
    hd.magic = GDN_SNAPSHOT_MAGIC;
    hd.version = GDN_SNAPSHOT_VERSION;
    hd.Hk = L->Hk; hd.Hv = L->Hv; hd.dk = L->dk; hd.dv = L->dv;
    hd.conv_K = L->conv_K;
    hd.act_dtype = L->act_dtype;
    hd.state_bytes = sb;
    hd.conv_bytes = cb;
    hd.checksum = fnv1a64(payload, sb + cb);
    hd.reserved = 0;
    memcpy(host, &hd, sizeof hd);
    return GDN_OK;
}

gdn_status gdn_snapshot_inspect(const void* host, size_t host_bytes, gdn_snapshot_header* out) {
    g_err[0] = 0;
    if (!host) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL snapshot buffer");
    if (host_bytes < sizeof(gdn_snapshot_header))
        return fail(GDN_ERR_INVALID_ARGUMENT, "buffer of %zu bytes is shorter than a snapshot header", host_bytes);
    gdn_snapshot_header hd;
    memcpy(&hd, host, sizeof hd);
    if (hd.magic != GDN_SNAPSHOT_MAGIC) return fail(GDN_ERR_INVALID_ARGUMENT, "not a snapshot (bad magic)");
    if (hd.version != GDN_SNAPSHOT_VERSION)
        return fail(GDN_ERR_INVALID_ARGUMENT, "snapshot version %u, this library reads %u", hd.version,
                    static_cast<unsigned>(GDN_SNAPSHOT_VERSION));
    // each dimension below 2^16 and K below 2^8: the size products and their
    // sum below stay far from wrapping around 64 bits, so a header cannot
    // pass the size checks with wrapped values
    constexpr int32_t kDimMax = 1 << 16;
    if (hd.Hk <= 0 || hd.Hv <= 0 || hd.dk <= 0 || hd.dv <= 0 || hd.conv_K < 1 || hd.Hk > kDimMax ||
        hd.Hv > kDimMax || hd.dk > kDimMax || hd.dv > kDimMax || hd.conv_K > 256 ||
        (hd.act_dtype != GDN_DTYPE_FP32 && hd.act_dtype != GDN_DTYPE_BF16))
        return fail(GDN_ERR_INVALID_ARGUMENT, "snapshot header has an invalid geometry or dtype");
    const uint64_t Cc = 2ull * hd.Hk * hd.dk + static_cast<uint64_t>(hd.Hv) * hd.dv;
    if (hd.state_bytes != static_cast<uint64_t>(hd.Hv) * hd.dk * hd.dv * 4 ||
        hd.conv_bytes != static_cast<uint64_t>(hd.conv_K - 1) * Cc * act_size(hd.act_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, "snapshot payload sizes do not match its geometry");
    if (host_bytes - sizeof hd < hd.state_bytes + hd.conv_bytes)
        return fail(GDN_ERR_INVALID_ARGUMENT, "snapshot truncated: %zu payload bytes, header says %llu",
                    host_bytes - sizeof hd, static_cast<unsigned long long>(hd.state_bytes + hd.conv_bytes));
    const uint8_t* payload = static_cast<const uint8_t*>(host) + sizeof hd;
    if (fnv1a64(payload, hd.state_bytes + hd.conv_bytes) != hd.checksum)
        return fail(GDN_ERR_INVALID_ARGUMENT, "snapshot checksum mismatch (corrupted payload)");
    if (out) *out = hd;
    return GDN_OK;
}

gdn_status gdn_snapshot_restore(const gdn_layer* L, const void* host, size_t host_bytes, float* state,
                                void* conv, int32_t slot, int32_t num_slots, void* stream) {
    g_err[0] = 0;
    gdn_snapshot_header hd;
    gdn_status st = gdn_snapshot_inspect(host, host_bytes, &hd);
    if (st != GDN_OK) return st;
    if ((st = check_layer(L, false)) != GDN_OK) return st;
    if (hd.Hk != L->Hk || hd.Hv != L->Hv || hd.dk != L->dk || hd.dv != L->dv || hd.conv_K != L->conv_K ||
        hd.act_dtype != L->act_dtype)
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "snapshot of a layer with Hk=%d Hv=%d dk=%d dv=%d K=%d act_dtype=%d does not fit this "
                    "layer (Hk=%d Hv=%d dk=%d dv=%d K=%d act_dtype=%d)", hd.Hk, hd.Hv, hd.dk, hd.dv,
                    hd.conv_K, hd.act_dtype, L->Hk, L->Hv, L->dk, L->dv, L->conv_K, L->act_dtype);
    if ((st = snapshot_args(L, state, conv, slot, num_slots, host, host_bytes)) != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* payload = static_cast<const uint8_t*>(host) + sizeof hd;
    hipError_t e = hipMemcpyAsync(reinterpret_cast<uint8_t*>(state) + hd.state_bytes * slot, payload,
                                  hd.state_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(static_cast<uint8_t*>(conv) + hd.conv_bytes * slot, payload + hd.state_bytes,
                           hd.conv_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "snapshot restore failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_selftest_mfma(const float* A, const float* B, float* C, void* stream) {
    g_err[0] = 0;
    if (!A || !B || !C) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL pointer");
    hipError_t e = gdn::launch_selftest_mfma(A, B, C, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "self-test failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // extern "C"
