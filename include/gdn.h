/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet layer library.
 *
 * The layer is the recurrent block of the hybrid Qwen3.x models described on
 * the llmxabe README ("Status" and the model section: three of every four
 * layers are Gated DeltaNet, each carrying a fixed-size recurrent state of
 * about 2 MiB per sequence, ~60 MiB over 30 layers) and on skindeep.ai "Our
 * own inference runtime" ("What it is": 36 of 48 layers are gated delta net).
 * It computes, per sequence and value head, token by token:
 *
 *   conv:   x~ = SiLU(causal depthwise conv1d_K(x)) over the q|k|v channels
 *   norm:   q^ = scale * q~ / sqrt(|q~|^2 + eps_l2),  k^ = k~ / sqrt(|k~|^2 + eps_l2)
 *   gates:  g = -exp(A_log) * softplus(a + dt_bias),  beta = sigmoid(b)
 *   rule:   S_t = exp(g_t) S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v~_t k^_t^T,
 *           o_t = S_t q^_t                      (Yang, Kautz, Hatamizadeh,
 *           "Gated Delta Networks", ICLR 2025, gated delta rule)
 *   gate:   out = norm_w (.) o / sqrt(mean(o^2) + eps_rms) (.) SiLU(z)
 *
 * Two entry points: gdn_prefill (many tokens per sequence, packed varlen,
 * chunked WY/UT form, optional carried state in and out) and gdn_decode (one
 * token per sequence against carried conv and recurrent state).  Batched
 * results are bit-identical to the same sequence run alone -- the serving
 * contract on the llmxabe README, "Status": a sequence decodes identically
 * whether batched with others or alone.
 *
 * Conventions common to every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   allocates nothing, keeps no state besides its code objects, and never
 *   synchronises the host (except gdn_selftest_mfma and the gdn_snapshot_*
 *   calls); all work is enqueued on `stream` (a hipStream_t; NULL = the
 *   default stream).  Device-side faults surface at the caller's
 *   next synchronisation.
 * - Layouts are row-major, innermost dimension contiguous:
 *     q, k           [tokens][Hk][dk]    (token stride q_stride/k_stride)
 *     v, z           [tokens][Hv][dv]    (token stride v_stride/z_stride)
 *     a, b           [tokens][Hv]        (token stride a_stride/b_stride)
 *     out, core_out  [tokens][Hv][dv]    dense
 *     state          [seq][Hv][dk][dv]   fp32, holding S^T:
 *                                        state[n][h][i][j] = S_{n,h}[j][i]
 *     conv state     [seq][K-1][Cc]      act dtype, oldest tap first,
 *                                        Cc = 2*Hk*dk + Hv*dv, channels
 *                                        q (head-major), then k, then v
 *     conv_w         [Cc][K] fp32, conv_w[c][K-1] multiplies the current token
 *   Token strides are in elements; 0 means dense.  Value head h reads key
 *   head h / (Hv/Hk).
 * - Alignment: q, k, v, z, out, core_out, states, conv states and conv_w
 *   16 bytes; strides of q/k/v/z multiples of 8 elements; a, b element
 *   aligned; A_log, dt_bias, norm_w 4 bytes.
 * - Errors: the return value is GDN_OK after a successful enqueue, otherwise
 *   a status code with detail text in gdn_last_error() (thread-local).  No
 *   work is enqueued when a call returns an error.  Device contents
 *   (cu_seqlens values, NaNs) are not validated.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 13

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad sizes, bad aliasing */
    GDN_ERR_UNSUPPORTED = 2,      /* shape or dtype combination not compiled */
    GDN_ERR_WORKSPACE = 3,        /* workspace missing or too small */
    GDN_ERR_HIP = 4               /* a HIP runtime call failed */
} gdn_status;

typedef enum { GDN_DTYPE_FP32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;

/* Static description of one layer.  Compiled shapes: prefill (dk, dv,
 * chunk) = (128, 128, 64), (32, 32, 16), (32, 64, 16); decode (dk, dv) =
 * (128, 128), (64, 64), (32, 32), (32, 64); conv_K = 4; act_dtype fp32 or
 * bf16; out_dtype fp32 or bf16.  Other shapes return GDN_ERR_UNSUPPORTED. */
typedef struct {
    int32_t Hk, Hv;          /* key/query heads, value heads; Hv % Hk == 0 */
    int32_t dk, dv;          /* key and value head dims */
    int32_t conv_K;          /* conv taps (4) */
    int32_t chunk;           /* prefill chunk length C */
    int32_t act_dtype;       /* gdn_dtype of q, k, v, z, a, b and conv states */
    int32_t out_dtype;       /* gdn_dtype of out */
    float scale;             /* q scale (1/sqrt(dk) for the Qwen3.x layers) */
    float eps_l2;            /* L2-norm epsilon */
    float eps_rms;           /* RMSNorm epsilon */
    const float* conv_w;     /* [Cc][K] */
    const float* A_log;      /* [Hv] */
    const float* dt_bias;    /* [Hv] */
    const float* norm_w;     /* [dv], shared by all heads */
} gdn_layer;

/* Chunked prefill over N packed sequences.  Sequence n owns tokens
 * [cu_seqlens[n], cu_seqlens[n+1]); lengths may be 0 (states pass through).
 * initial_state NULL means zeros; final_state may equal initial_state
 * (in-place update) but must not partially overlap it; NULL = not written.
 * conv_state_in NULL means zero history; conv_state_out may equal
 * conv_state_in; NULL = not written.  core_out (optional) receives o_t
 * before the gated RMSNorm, in fp32.  The gated RMSNorm normalises o_t
 * rounded to fp16 (to nearest even), with or without core_out, so `out`
 * has the same bits either way. */
typedef struct {
    int32_t N;
    int64_t T_total;               /* == cu_seqlens[N] */
    const int32_t* cu_seqlens;     /* device int32 [N+1], non-decreasing, [0] = 0
                                    * (checked on the device: see status) */
    const void *q, *k, *v, *z, *a, *b;
    int64_t q_stride, k_stride, v_stride, z_stride, a_stride, b_stride;
    const float* initial_state;
    float* final_state;
    const void* conv_state_in;
    void* conv_state_out;
    void* out;                     /* out_dtype */
    float* core_out;               /* optional */
    /* optional state pool (a serving engine's bank of per-sequence states,
     * batched across whichever sequences are ready: llmxabe README,
     * "Status", batched prefill and decode across parallel sequences):
     * device int32 [N], distinct entries in
     * [0, num_slots); sequence n's recurrent and conv states are then entry
     * state_slots[n] of initial_state / final_state ([num_slots][Hv][dk][dv])
     * and of conv_state_in / conv_state_out ([num_slots][K-1][Cc]).  NULL:
     * entry n, as without a pool (num_slots ignored). */
    const int32_t* state_slots;
    int32_t num_slots;
    /* optional device int32: the call's first kernel stores 0 there, then
     * ORs in status bits:
     *   GDN_STATUS_NONFINITE when a value of out or of final_state is not
     *     finite.  With finite inputs that happens only when a value on the
     *     scan's fp16 operand path left the fp16 range (|x| >= 65520 rounds
     *     to inf): the state S, or u = beta (v - e^g S k), of magnitude
     *     beyond ~6.5e4 -- activations far beyond a layer's normal scale.
     *   GDN_STATUS_BAD_INDEX when the device-side indices break their
     *     contract: cu_seqlens[0] != 0, a decreasing step, cu_seqlens[N] !=
     *     T_total, or a state_slots entry outside [0, num_slots).  The call
     *     then computes and writes nothing (out, core_out, final_state and
     *     conv_state_out keep their contents), with or without a status
     *     word; no memory is touched through the bad index.  (Duplicate
     *     state_slots entries are not detected.)
     * Read it once the stream has passed the call; NULL: no report. */
    int32_t* status;
} gdn_prefill_io;

#define GDN_STATUS_NONFINITE 1
#define GDN_STATUS_BAD_INDEX 2

/* One token for each of B sequences.  state_out may equal state_in and
 * conv_state_out may equal conv_state_in (in-place); partial overlap is an
 * error.  state_in NULL means zeros; conv_state_in NULL means zero history.
 *
 * workspace (optional, gdn_decode and gdn_step only; gdn_decode_multi
 * ignores it): device memory of at least gdn_decode_workspace_bytes(layer,
 * B) bytes, 256-byte aligned, that must hold zeros before its first use.
 * With it, the step runs one work-group per (sequence, value head), which
 * spreads a small batch's state stream over twice as many compute units;
 * the work-groups of a key head share its q/k conv history, and the last of
 * them to count itself in on a per-(sequence, key head) arrival counter in
 * the workspace writes the new history and puts the counter back to zero.
 * So every call leaves the workspace at zero (no fill between calls or
 * graph replays), results are bit-identical to the call without a
 * workspace, and a workspace serves one call at a time (calls that may run
 * concurrently need their own).  NULL: one work-group per (sequence, key
 * head). */
typedef struct {
    int32_t B;
    const void *q, *k, *v, *z, *a, *b;   /* one token per sequence */
    int64_t q_stride, k_stride, v_stride, z_stride, a_stride, b_stride;
    const float* state_in;
    float* state_out;                    /* required */
    const void* conv_state_in;
    void* conv_state_out;                /* required */
    void* out;                           /* [B][Hv][dv], out_dtype */
    float* core_out;                     /* optional [B][Hv][dv] fp32 */
    const int32_t* state_slots;          /* optional pool entries, as in gdn_prefill_io */
    int32_t num_slots;
    void* workspace;                     /* optional, see above */
    size_t workspace_bytes;
    /* optional device int32, never cleared by the call:
     * GDN_STATUS_BAD_INDEX is ORed in when a state_slots entry lies outside
     * [0, num_slots).  That sequence is skipped: nothing is read or written
     * for it (its out and core_out rows and its pool entries keep their
     * contents), the others are computed as usual.  NULL: no report (the
     * sequence is skipped all the same). */
    int32_t* status;
} gdn_decode_io;

/* Bytes of a gdn_decode workspace for up to B sequences: arrival counters
 * [B][Hk] uint32, rounded up to 256 bytes; 0 on error.  A workspace sized
 * for B serves any smaller batch. */
size_t gdn_decode_workspace_bytes(const gdn_layer* layer, int32_t B);

/* Version of this header's structs and layouts. */
int gdn_abi_version(void);

/* Bytes of device workspace gdn_prefill needs for N sequences holding
 * T_total tokens in all (an upper bound over every length split).  It holds
 * the chunk table, the pre-norm output as fp16 (when no core_out is given),
 * two recurrent-state carry slots and the per-chunk operand blocks of one
 * window of chunks.  The prefill runs window by window: the window is at
 * most about 240 MiB of operand blocks (sized for the Infinity Cache; cut to
 * whole rounds of the first kernel's work-groups over the device's compute
 * units when the batch takes several windows), so the size grows with
 * T_total only through the pre-norm output.  Returns 0 and sets
 * gdn_last_error() if the layer is invalid or unsupported. */
size_t gdn_prefill_workspace_bytes(const gdn_layer* layer, int32_t N,
                                   int64_t T_total);

/* Enqueue the chunked prefill.  workspace: device memory, 256-byte aligned,
 * not shared with a concurrently running call, of
 * gdn_prefill_workspace_bytes(layer, N, T_total) bytes; a smaller workspace
 * is accepted down to the fixed parts plus one chunk slot of operand blocks
 * and runs with correspondingly smaller windows (same results, more kernel
 * launches).  GDN_ERR_WORKSPACE below that. */
gdn_status gdn_prefill(const gdn_layer* layer, const gdn_prefill_io* io,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array behind gdn_prefill_noalloc. */
#define GDN_NOALLOC_SCRATCH_BYTES (128ull << 20)

/* gdn_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller passes the inputs and outputs as for gdn_prefill but no
 * workspace: the library uses a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES instead, one per device, allocated when the
 * library's device code is loaded and held until the process ends (its
 * address is looked up on the first call on each device).  It calls no
 * allocating routine.  Same kernels and bit-identical results as
 * gdn_prefill with a workspace of that size.  Sizes whose workspace does not
 * fit that array (the fixed parts plus one chunk slot of operand blocks,
 * plus T_total*Hv*dv*2 bytes of fp16 pre-norm output when core_out is NULL) are
 * refused with GDN_ERR_WORKSPACE before anything is enqueued.  The stream's
 * device must be the current device (else GDN_ERR_INVALID_ARGUMENT).  All
 * calls on one device share its array: calls that overlap in time on one
 * device (other streams, other threads) race and must not be made; calls
 * in one stream's order are safe (nothing in the array needs to start at
 * zero: every byte a kernel reads was written earlier in the same call). */
gdn_status gdn_prefill_noalloc(const gdn_layer* layer, const gdn_prefill_io* io,
                               void* stream);

/* Number of kernels gdn_prefill enqueues for these sizes and this
 * workspace size, in order: per window prep (chunk-parallel operands; the
 * first one also builds the chunk table) and scan (sequential state
 * passing), then epi (gated RMSNorm): 1 + 2 * windows.  with_core_out:
 * nonzero if the call passes core_out (the workspace then holds no pre-norm
 * output, so more chunk slots fit in a given size).  -1 on an invalid
 * layer, sizes or a too small workspace (detail in gdn_last_error()). */
int64_t gdn_prefill_launches(const gdn_layer* layer, int32_t N,
                             int64_t T_total, size_t workspace_bytes,
                             int32_t with_core_out);

/* Chunk slots per window gdn_prefill runs with for these sizes, this
 * workspace size and with or without core_out (operand blocks of that many
 * chunks of every value head fit the workspace at once); -1 as for
 * gdn_prefill_launches. */
int64_t gdn_prefill_window_slots(const gdn_layer* layer, int32_t N,
                                 int64_t T_total, size_t workspace_bytes,
                                 int32_t with_core_out);

/* gdn_prefill that also records caller-created timing events (hipEvent_t
 * handles) on `stream`: events[0] before the first kernel and events[i]
 * after kernel i-1 (numbering as in gdn_prefill_launches), so consecutive
 * events bracket each kernel.  n_events must be gdn_prefill_launches() + 1
 * (with with_core_out set as io->core_out is given).
 * Same results as gdn_prefill; meant for per-kernel timing. */
gdn_status gdn_prefill_timed(const gdn_layer* layer, const gdn_prefill_io* io,
                             void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events, int n_events);

/* Enqueue one decode step (no workspace needed). */
gdn_status gdn_decode(const gdn_layer* layer, const gdn_decode_io* io,
                      void* stream);

/* One serving step of a layer over a state pool (the llmxabe README,
 * "Status": prefill and decode batched across parallel sequences in one
 * engine step): the decode batch (one
 * token per sequence; NULL or B = 0 for none) and the prefill batch (NULL or
 * N = 0 for none), each as its own call describes, enqueued on `stream`
 * decode first.  The two batches' sequences must use distinct pool entries
 * (state_slots) when they share pools.  Both are validated before anything
 * is enqueued.  workspace as for gdn_prefill (may be NULL without a prefill
 * batch). */
gdn_status gdn_step(const gdn_layer* layer, const gdn_prefill_io* prefill,
                    const gdn_decode_io* decode, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Most tokens per sequence gdn_decode_multi takes. */
#define GDN_MAX_VERIFY_TOKENS 16

/* Several tokens per sequence against carried state, in order -- the
 * multi-token verify step of speculative decoding (the block drafters of
 * the xwen README's speculative-decoding section propose up to 15 tokens).
 * io is read as for gdn_decode except that the token tensors q, k, v, z,
 * a, b and out / core_out hold B * tokens rows, sequence b's tokens at rows
 * b * tokens .. b * tokens + tokens - 1 (token strides as in gdn_decode);
 * the conv state advances by all the tokens.  The state is read once and
 * updated token by token with the arithmetic of gdn_decode, so every output
 * and state is bit-identical to `tokens` successive gdn_decode calls.
 * state_snapshots: NULL, or device fp32 [B][tokens][Hv][dk][dv] receiving
 * the state after each token (the last equals state_out), for rolling back
 * to any accepted prefix; it must not overlap state_in or state_out.  (The
 * conv state after an accepted prefix of k tokens is the last K-1 raw
 * inputs of the old conv state followed by those k tokens, which the caller
 * already holds.)  tokens in [1, GDN_MAX_VERIFY_TOKENS], else
 * GDN_ERR_INVALID_ARGUMENT. */
gdn_status gdn_decode_multi(const gdn_layer* layer, const gdn_decode_io* io,
                            int32_t tokens, float* state_snapshots, void* stream);

/* ---- the projections either side of the layer --------------------------
 * in_proj maps the model's hidden state to q, k, v, z, a, b and out_proj
 * maps the gated output back (llmxabe README, model section: the hybrid
 * stack around these layers; its LM-head figure, 540 MB per token for an
 * untied 248,320-row head, fits a width of 2048 at 8.5 bits per weight).
 * Both are bf16 GEMMs on the matrix cores with fp32 accumulation. */

/* C[M][N] = A[M][K] * B[N][K]^T: A, B bf16 (k contiguous, leading dims lda,
 * ldb in elements), C in c_dtype (GDN_DTYPE_BF16 or GDN_DTYPE_FP32, leading
 * dim ldc), fp32 accumulation.  K, lda, ldb multiples of 8 and A, B 16-byte
 * aligned; M, N, K >= 0.  Enqueued on `stream`.  Up to 64 rows run on the
 * library path pinned at 64 rows, more on the one pinned at 4096 (below);
 * each sums an output in an order that depends on K and N only, but the
 * orders may differ, so a row's bits may change when M crosses 64.  gdn_layer_prefill
 * and gdn_layer_decode each keep to one kernel family at every size, so
 * their results do not depend on the batch. */
gdn_status gdn_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                         void* C, int64_t ldc, int32_t c_dtype, int64_t M,
                         int64_t N, int64_t K, void* stream);

/* gdn_gemm_bf16 on a chosen kernel family:
 *   GDN_GEMM_AUTO       as gdn_gemm_bf16
 *   GDN_GEMM_TILED      this library's tiled kernel (256-row tiles)
 *   GDN_GEMM_FEW_ROWS   this library's weight-streaming few-row kernel,
 *                       over 64-row blocks at any M
 *   GDN_GEMM_LIBRARY    hipBLASLt (the vendor's GEMM library; plain GEMMs
 *                       are its job) with one algorithm per (device, N, K,
 *                       leading dimensions, C type): the first of its
 *                       ranked choices at 4096 rows that needs no
 *                       workspace, kept for the life of the process and
 *                       used at every M (a larger M in blocks of 4096
 *                       rows: an algorithm is only known to fit the size
 *                       it was ranked at), so a row's bits do not depend
 *                       on M and, on the same library and device, not on
 *                       the process either (gdn_layer_prefill's
 *                       projections).  An N past a multiple of 256 runs as
 *                       two products, the full 256-column blocks and the
 *                       rest, each with its own algorithm (a nearly empty
 *                       last column of tiles would cost a whole round of
 *                       them).
 *                       Where the library declines a shape the tiled
 *                       kernel runs.
 *   GDN_GEMM_LIBRARY_FEW_ROWS  the same with the algorithm chosen at 64
 *                       rows and run in blocks of 64 rows
 *                       (gdn_layer_decode's projections, at any batch
 *                       size); the few-row kernel where the library
 *                       declines.
 * The library path keeps a hipBLASLt handle per device for the life of the
 * process; its first call on a device and shape must not be under graph
 * capture (it loads the algorithm's code).  An unknown path:
 * GDN_ERR_INVALID_ARGUMENT. */
#define GDN_GEMM_AUTO 0
#define GDN_GEMM_TILED 1
#define GDN_GEMM_FEW_ROWS 2
#define GDN_GEMM_LIBRARY 3
#define GDN_GEMM_LIBRARY_FEW_ROWS 4
gdn_status gdn_gemm_bf16_path(const void* A, int64_t lda, const void* B, int64_t ldb,
                              void* C, int64_t ldc, int32_t c_dtype, int64_t M,
                              int64_t N, int64_t K, int32_t path, void* stream);

typedef struct {
    int32_t hidden;         /* model width; a multiple of 8 */
    const void* w_in;       /* [P][hidden] bf16, P = 2*Hk*dk + 2*Hv*dv + 2*Hv
                             * output rows ordered q (head-major) | k | v | z |
                             * a | b, so the conv channels q|k|v come first */
    const void* w_out;      /* [hidden][Hv*dv] bf16 */
} gdn_proj;

/* One sequence batch through the whole layer: x [T][hidden] bf16 in, y
 * [T][hidden] in y_dtype out; states and cu_seqlens as in gdn_prefill_io. */
typedef struct {
    int32_t N;
    int64_t T_total;
    const int32_t* cu_seqlens;
    const void* x;
    void* y;
    int32_t y_dtype;               /* GDN_DTYPE_BF16 or GDN_DTYPE_FP32 */
    const float* initial_state;    /* optional, as in gdn_prefill_io */
    float* final_state;
    const void* conv_state_in;
    void* conv_state_out;
    const int32_t* state_slots;    /* optional pool entries */
    int32_t num_slots;
    int32_t* status;               /* optional, as in gdn_prefill_io; on
                                    * GDN_STATUS_BAD_INDEX the states keep
                                    * their contents and y is unspecified
                                    * (out_proj still runs) */
} gdn_layer_io;

/* Workspace of gdn_layer_prefill: the projection [T][P] bf16, the gated
 * output [T][Hv*dv] bf16 and gdn_prefill's own workspace. */
size_t gdn_layer_prefill_workspace_bytes(const gdn_layer* layer,
                                         const gdn_proj* proj, int32_t N,
                                         int64_t T_total);

/* in_proj GEMM -> gdn_prefill on views into the projection (token stride
 * P) -> out_proj GEMM, on `stream`.  The layer's act_dtype must be bf16 (the
 * projection's dtype); the gated output between the GDN and out_proj is
 * bf16 whatever the layer's out_dtype.  Same validation and error
 * behaviour as gdn_prefill, plus the projection's shapes. */
gdn_status gdn_layer_prefill(const gdn_layer* layer, const gdn_proj* proj,
                             const gdn_layer_io* io, void* workspace,
                             size_t workspace_bytes, void* stream);

/* One token per sequence through the whole layer: x [B][hidden] bf16 in, y
 * [B][hidden] in y_dtype out, states as in gdn_decode_io (state pools
 * included).  The workspace holds the projection [B][P] and the gated
 * output [B][Hv*dv] (bf16). */
typedef struct {
    int32_t B;
    const void* x;
    void* y;
    int32_t y_dtype;
    const float* state_in;
    float* state_out;
    const void* conv_state_in;
    void* conv_state_out;
    const int32_t* state_slots;
    int32_t num_slots;
    int32_t* status;               /* optional, as in gdn_decode_io; a
                                    * skipped sequence's row of y is
                                    * unspecified (out_proj still runs) */
} gdn_layer_decode_io;

size_t gdn_layer_decode_workspace_bytes(const gdn_layer* layer,
                                        const gdn_proj* proj, int32_t B);

/* in_proj GEMM -> gdn_decode on views into the projection -> out_proj GEMM,
 * on `stream`; validation as for gdn_decode plus the projection's shapes.
 * The workspace's first 64 KiB serve as the decode step's arrival counters
 * (see gdn_decode_io): they must hold zeros before the first use, every call
 * leaves them so, and a workspace serves one call at a time. */
gdn_status gdn_layer_decode(const gdn_layer* layer, const gdn_proj* proj,
                            const gdn_layer_decode_io* io, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---- session snapshots ------------------------------------------------
 * Park one sequence's layer state (recurrent + conv) in host memory and
 * resume it later, in this process or another -- the session swap of
 * skindeep.ai "Our own inference runtime" ("Session swap": save, inspect,
 * restore and delete with compatibility checks; a restart-and-continue must
 * reproduce the output exactly).  A snapshot is a gdn_snapshot_header
 * followed by the state [Hv][dk][dv] fp32 and the conv state [K-1][Cc] in
 * the act dtype, byte for byte as they are in device memory, so a restore
 * continues bit-identically.  Deleting a snapshot is freeing its buffer.
 * These calls synchronise `stream` (parking is not on the per-token path). */
#define GDN_SNAPSHOT_MAGIC 0x50534E47u   /* "GNSP" little-endian */
#define GDN_SNAPSHOT_VERSION 1

typedef struct {
    uint32_t magic;            /* GDN_SNAPSHOT_MAGIC */
    uint32_t version;          /* GDN_SNAPSHOT_VERSION */
    int32_t Hk, Hv, dk, dv;    /* layer geometry the state belongs to */
    int32_t conv_K;
    int32_t act_dtype;         /* dtype of the conv state */
    uint64_t state_bytes;      /* Hv*dk*dv*4 */
    uint64_t conv_bytes;       /* (K-1)*Cc*act size */
    uint64_t checksum;         /* FNV-1a 64 over the payload bytes */
    uint64_t reserved;         /* 0 */
} gdn_snapshot_header;         /* 64 bytes; the payload follows it */

/* Bytes of one snapshot for this layer (header + payload), 0 on error. */
size_t gdn_snapshot_bytes(const gdn_layer* layer);

/* Copy pool entry `slot` of state [num_slots][Hv][dk][dv] and conv_state
 * [num_slots][K-1][Cc] (device) into `host_buf` (host memory, at least
 * gdn_snapshot_bytes(layer) bytes) and seal it with the header.  Waits for
 * the stream first, so the state saved is the one after all work enqueued
 * before this call.  slot outside [0, num_slots) or a short buffer:
 * GDN_ERR_INVALID_ARGUMENT; nothing is written then. */
gdn_status gdn_snapshot_save(const gdn_layer* layer, const float* state,
                             const void* conv_state, int32_t slot,
                             int32_t num_slots, void* host_buf,
                             size_t host_bytes, void* stream);

/* Validate a snapshot in host memory (magic, version, geometry with every
 * dimension in [1, 65536] and conv_K in [1, 256], sizes, checksum) and
 * return its header; touches no device and reads at most host_bytes.
 * GDN_ERR_INVALID_ARGUMENT with the reason in gdn_last_error() when it is not
 * a whole, intact snapshot. */
gdn_status gdn_snapshot_inspect(const void* host_buf, size_t host_bytes,
                                gdn_snapshot_header* header);

/* Validate the snapshot as gdn_snapshot_inspect does, check that it belongs
 * to this layer's geometry and conv dtype (else GDN_ERR_INVALID_ARGUMENT,
 * nothing written), then copy it into pool entry `slot` of state and
 * conv_state (device) and wait for the copy to finish. */
gdn_status gdn_snapshot_restore(const gdn_layer* layer, const void* host_buf,
                                size_t host_bytes, float* state,
                                void* conv_state, int32_t slot,
                                int32_t num_slots, void* stream);

/* Static text for a status code. */
const char* gdn_status_string(gdn_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gdn_last_error(void);

/* Library self-test of the matrix-core fragment layouts the kernels rely on:
 * computes C = A[16][32] * B[32][16] through bf16 hi/lo split products into
 * C[0][16][16] on v_mfma_f32_16x16x32_bf16 and into C[1][16][16] on
 * v_mfma_f32_16x16x16_bf16 (two k halves), and with A and B rounded to fp16
 * into C[2][16][16] on v_mfma_f32_16x16x32_f16; row-major fp32 in/out,
 * device pointers (C holds 768 floats).  Synchronises the stream.
 * Returns GDN_OK or GDN_ERR_HIP. */
gdn_status gdn_selftest_mfma(const float* A, const float* B, float* C,
                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H_ */
