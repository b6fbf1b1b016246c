/*
 * moe_expert.h -- C ABI of the MoE expert operation of a speculative-decoding
 * verification pass, for AMD Instinct MI355X (gfx950).
 *
 * Source of every definition below: Y. Lan, "Speculative Decoding for
 * Mixture-of-Experts Models: Expert Bytes, Kernel Bandwidth and the Best Draft
 * Length", arXiv:2610.34440 ("the paper").
 *
 * The expert operation (paper, Section 1): for a pass of n tokens, each routed to
 * m of the layer's N experts, compute for every token t
 *     y_t = sum_{j<m} w_tj * W_down[e_tj] ( silu(W_gate[e_tj] x_t) * (W_up[e_tj] x_t) )
 * with silu(z) = z / (1 + exp(-z)).  A slot is one of a token's m selections, so a
 * pass has n*m slots, numbered s = t*m + j.  Two kernels compute this same
 * function:
 *   - per-slot:       one read of the selected expert's weights per slot;
 *   - deduplicating:  groups the pass's slots by expert and reads each distinct
 *                     expert once, against all of that expert's tokens.
 *
 * Conventions shared by every device entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library keeps no pointer after the call returns and allocates nothing.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  A return value other than MOE_OK means nothing was
 *     enqueued (except MOE_E_HIP, returned when a launch itself failed).
 *   - Host-side validation happens before any launch.  No C++ exception crosses
 *     this interface; no entry point aborts.
 *   - Weights and x are bf16 (bit patterns, round-to-nearest-even) or fp32;
 *     all accumulation is fp32; y is fp32.
 *   - Weight layouts, row-major and contiguous:
 *         W_gate, W_up : [N][d_ff][d_model]      W_down : [N][d_model][d_ff]
 *     (or W_down packed by moe_pack_w_down, flagged MOE_FLAG_WDOWN_PACKED, or all
 *     three tiled by moe_pack_tiled, flagged MOE_FLAG_TILED);
 *     x : [n][d_model];  ids : [n][m] int32;  w : [n][m] fp32;  y : [n][d_model].
 *   - Workspaces (`ws`) are caller-owned device memory that must be zero-filled
 *     once before first use (e.g. hipMemset); every call that runs to completion
 *     leaves the workspace's synchronisation words zero again.  Calls that share
 *     a workspace must not overlap in time.
 */
#ifndef MOE_EXPERT_H
#define MOE_EXPERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_E_INVAL = -1,     /* null pointer, size out of range, misaligned pointer */
    MOE_E_DTYPE = -2,     /* unknown dtype, or d_model / d_ff not a multiple of 8 */
    MOE_E_WORKSPACE = -3, /* workspace smaller than moe_workspace_bytes() */
    MOE_E_HIP = -4,       /* a HIP launch failed, or (in info) an internal wait expired */
    MOE_E_IDS = -5        /* an expert id out of [0, N), or repeated within a token */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

enum { MOE_KIND_SLOT = 0, MOE_KIND_DEDUP = 1 };

#define MOE_MAX_SLOTS 256     /* n * m */
#define MOE_MAX_TOKENS 64     /* n */
#define MOE_MAX_EXPERTS 1024  /* N */
#define MOE_MAX_SHARED 16     /* n_shared */
#define MOE_FLAG_ACCUMULATE 1u /* y += result (else y = result) */
/* w_down is in the packed layout of moe_pack_w_down (else [N][d_model][d_ff]) */
#define MOE_FLAG_WDOWN_PACKED 2u
/* w_gate, w_up and w_down (routed and shared) are all in the tiled layout of
 * moe_pack_tiled; excludes MOE_FLAG_WDOWN_PACKED */
#define MOE_FLAG_TILED 4u
/* matrices of moe_pack_tiled */
#define MOE_MAT_GATE_UP 0 /* W_gate or W_up [N][d_ff][d_model]: rows d_ff, contraction d_model */
#define MOE_MAT_DOWN 1    /* W_down [N][d_model][d_ff]: rows d_model, contraction d_ff */

/* One MoE layer.  1 <= m <= N (m == N is allowed, so that always-on experts can
 * also run as a layer of their own whose every token selects all of them). */
typedef struct {
    int32_t N;        /* routed experts in the layer */
    int32_t m;        /* experts selected per token */
    int32_t d_model;  /* d: token width; multiple of 8 */
    int32_t d_ff;     /* expert hidden width; multiple of 8 */
    int32_t dtype;    /* moe_dtype of the weights and of x */
    uint32_t flags;   /* MOE_FLAG_* */
    int32_t n_shared; /* always-on (shared) experts computed in the same call,
                         0 .. MOE_MAX_SHARED; 0 = none.  Same d_model, d_ff, dtype
                         and weight layout (plain, W_down packed, or all three
                         tiled, as flags say) as the routed experts. */
} moe_layer_desc;

/* Device pointers, caller-owned, 16-byte aligned, layouts as above.  The shared
 * experts' tensors hold n_shared experts ([n_shared][d_ff][d_model] and so on) and
 * are read only when desc->n_shared > 0 (else they may be NULL). */
typedef struct {
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const void* w_gate_shared;
    const void* w_up_shared;
    const void* w_down_shared;
} moe_layer_weights;

/*
 * moe_route_group -- group the slots of a pass by expert (the deduplicating
 * kernel "groups the pass's tokens by expert", paper Section 1; the union
 * X(n) = |S_t u ... u S_{t+n-1}| is its number of groups, Section 1 "Routing,
 * union and reuse").  One workgroup; bit-exact, deterministic.
 *   ids            device [n*m]  expert id of slot s = t*m + j
 *   count          device [N]    slots per expert (in-range slots only)
 *   offset         device [N+1]  exclusive prefix sum of count; offset[N] = in-range slots
 *   slot_by_expert device [n*m]  slots of expert e at [offset[e], offset[e+1]), in
 *                                increasing s; entries from offset[N] on are -1
 *   distinct       device [N]    experts with count > 0 in increasing id, then -1
 *   u_and_err      device [2]    [0] = U (number of distinct experts),
 *                                [1] = MOE_OK or MOE_E_IDS (an id outside [0, N), which
 *                                      takes no part in the grouping, or an id repeated
 *                                      within a token, which does)
 * Limits: 1 <= n, 1 <= m <= N, n*m <= MOE_MAX_SLOTS, N <= MOE_MAX_EXPERTS.
 */
int moe_route_group(const int32_t* ids, int32_t n, int32_t m, int32_t N, int32_t* count,
                    int32_t* offset, int32_t* slot_by_expert, int32_t* distinct,
                    int32_t* u_and_err, void* hip_stream);

/* Workspace bytes that moe_expert_perslot (kind MOE_KIND_SLOT) or
 * moe_expert_dedup (MOE_KIND_DEDUP) needs for passes of up to n tokens; 0 on
 * invalid arguments.  For a pass of k tokens with S = k*m + n_shared*k slots (the
 * routed slots, then one per token and shared expert) the workspace holds 224 KB
 * of synchronisation counters (one per 128-byte line), the slots' hidden
 * activations (S*d_ff*4 bytes), their expert outputs (S*P*d_model*4 bytes, P = 1..4
 * parts of the d_ff contraction; P > 1 only for passes that may stream their
 * down-projection work with fewer than 4 items per compute unit) and, when the
 * pass's gate/up work may be cut between work groups (per-slot: fewer than 512
 * row tiles, or, for bf16 passes of at most 16 tokens without shared experts,
 * d_model >= 4096 and d_ff > 1536 (both multiples of 32), the tiles beyond whole
 * rounds of 256; deduplicating: any pass, since it plans for the experts it finds),
 * the partial sums of tiles that work groups share (3*S*d_ff*8 bytes), each piece
 * aligned to 256 bytes.  The
 * size returned is the largest over k = 1..n, so a workspace sized for n serves
 * every smaller n of the same layer.  d_model is limited to 16384. */
size_t moe_workspace_bytes(const moe_layer_desc* desc, int32_t n, int32_t kind);

/*
 * moe_expert_perslot -- the expert operation by the per-slot kernel: every slot
 * reads its expert's W_gate, W_up and W_down rows once (n*m expert reads per
 * pass, paper Section 1 "Bytes": E_slot(n) = n m w).  One kernel launch.
 * With desc->n_shared > 0 the same launch also computes the always-on experts,
 * each read once per pass against all n tokens with weight 1 (the D(n) bytes of
 * paper Eq. 5, outside E_p, in both kernels), and adds them to each token's y
 * after its routed slots, in increasing shared-expert index.
 * Limits: n*m + n_shared <= MOE_MAX_SLOTS.
 *   x    device [n][d_model]  (dtype of desc)
 *   ids  device [n][m]        ids outside [0, N) are skipped (their slot adds 0)
 *   w    device [n][m] fp32   routing weights
 *   y    device [n][d_model] fp32, overwritten (or accumulated with MOE_FLAG_ACCUMULATE)
 *   info device [3] int32 or NULL: [0] = U, the number of distinct in-range experts
 *        of the pass; [1] = MOE_OK or MOE_E_IDS (an id outside [0, N) or repeated
 *        within a token); [2] = MOE_OK, or MOE_E_HIP when an internal bounded wait
 *        expired (only with a workspace that was not zero-filled); y is then invalid
 *        and the workspace must be zero-filled again
 *   ws   device workspace, ws_bytes >= moe_workspace_bytes(desc, n, MOE_KIND_SLOT),
 *        256-byte aligned, zero-filled before first use (see above).
 * Per token, slot contributions are added in increasing j.  The result is
 * deterministic (bitwise equal over repeated calls) and equal to
 * moe_expert_dedup's up to fp32 summation order.
 */
int moe_expert_perslot(const moe_layer_desc* desc, const moe_layer_weights* weights,
                       const void* x, const int32_t* ids, const float* w, int32_t n, float* y,
                       int32_t* info, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * moe_expert_dedup -- the expert operation by the deduplicating kernel: the
 * pass's slots are grouped by expert (the grouping of moe_route_group, computed
 * inside the same launch) and each distinct expert is read once, against all of
 * its tokens (paper Section 1; E_dedup = X(n) w).  Arguments as for
 * moe_expert_perslot, workspace kind MOE_KIND_DEDUP.  With MOE_E_IDS in info[1],
 * a token's repeated id counts as often as it appears; out-of-range slots add 0.
 */
int moe_expert_dedup(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                     const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info,
                     void* ws, size_t ws_bytes, void* hip_stream);

/*
 * moe_expert_auto -- the crossover-driven switch between the two kernels (paper
 * Section 2 "Bytes against bandwidth" and Section 4: the deduplicating kernel should
 * run from the pass size at which its saving S(n) stays positive): passes of
 * n >= crossover tokens run moe_expert_dedup, smaller ones moe_expert_perslot;
 * crossover = 0 (no crossover) always runs the per-slot kernel.  The crossover comes
 * from measured times (step_time_model's crossover, or the measured S(n)).
 * Arguments as for moe_expert_perslot; ws must serve the kernel that runs (a
 * workspace of the larger of the two moe_workspace_bytes serves both).  kind_out
 * (host, may be NULL) receives MOE_KIND_SLOT or MOE_KIND_DEDUP.  Returns what the
 * chosen call returns, or MOE_E_INVAL for crossover < 0.
 */
int moe_expert_auto(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                    const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info,
                    void* ws, size_t ws_bytes, int32_t crossover, int32_t* kind_out,
                    void* hip_stream);

/*
 * moe_expert_auto_noalloc -- moe_expert_auto with no workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The kernels' workspace (counters, h, O,
 * partial sums) is a file-scope device array of MOE_SCRATCH_BYTES in the library,
 * one per GPU, held until the process ends.  Nothing is allocated: no hipMalloc,
 * hipFree or allocating library routine is called.
 *   Arguments as for moe_expert_auto, minus ws and ws_bytes.  The current device must
 *   be the device of hip_stream (the array used is the current device's).
 *   Each call first clears the array's counter words with a small kernel on
 *   hip_stream (a kernel, not a memset, so a graph capture records a kernel node),
 *   then runs the kernel moe_expert_auto would run: two launches per call.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (on different streams, or from different threads without ordering) race and
 *   their results are undefined.  Calls on one stream are ordered and safe.
 * Returns what moe_expert_auto returns; MOE_E_WORKSPACE (nothing enqueued) when the
 * pass needs more than MOE_SCRATCH_BYTES (moe_workspace_bytes of the kernel that
 * would run); MOE_E_INVAL when the stream's device is not the current device;
 * MOE_E_HIP when the array's address cannot be obtained.
 */
#define MOE_SCRATCH_BYTES (16u << 20)
int moe_expert_auto_noalloc(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                            const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info,
                            int32_t crossover, int32_t* kind_out, void* hip_stream);

/*
 * moe_pack_w_down -- copy W_down [N][d_model][d_ff] into the packed layout
 * [N][d_ff/8][d_model][8]: element (e, i, f) goes to
 *     ((e*(d_ff/8) + f/8)*d_model + i)*8 + f%8,
 * so that every run of 8 hidden columns of all output rows is contiguous (a
 * block of d_ff rows then reads its down-projection columns in whole cache lines
 * instead of 16- to 64-byte pieces of every output row).  Same byte size as the
 * source.  Expert calls read W_down in this layout when desc->flags has
 * MOE_FLAG_WDOWN_PACKED, in the same kernels and with the same result as the plain
 * layout (the down items' loads become whole-line reads).  A weight-load-time step,
 * not part of the expert operation.
 *   w_down, w_down_packed  device, 16-byte aligned, not overlapping; desc->flags ignored.
 * Asynchronous on hip_stream.  Returns MOE_OK, MOE_E_INVAL / MOE_E_DTYPE for bad
 * arguments (nothing enqueued), or MOE_E_HIP. */
int moe_pack_w_down(const moe_layer_desc* desc, const void* w_down, void* w_down_packed,
                    void* hip_stream);

/*
 * moe_pack_tiled -- copy one weight tensor of desc->N experts into the tiled
 * layout that expert calls read when desc->flags has MOE_FLAG_TILED (then W_gate,
 * W_up and W_down, routed and shared, must all be tiled).  The tensor is
 * [N][R][K]: rows R and contraction K are (d_ff, d_model) for MOE_MAT_GATE_UP and
 * (d_model, d_ff) for MOE_MAT_DOWN.  With step = 64 bytes / element size (32 bf16 or
 * 16 fp32 elements), both d_model and d_ff must be multiples of the step.  The
 * copy is made of 1024-byte blocks, 16 rows x one step each, in (expert, row
 * block, step) order; in block (e, r, s), lane l = 0..63 holds 16 bytes at 16*l:
 * row 16*r + l%16, the 16/size elements from column step*s + (l/16)*(16/size).  Same
 * byte size as the source.  The row-block-and-step blocks are the operands of one
 * 16-row MFMA step (weights of the matrix operand in the lane order the
 * instruction takes), so one load instruction of a wave reads one whole block,
 * and the four waves of a work group, which take every fourth step, read
 * adjacent blocks.  Same result as the plain layout up to the fp32 summation
 * order.  A weight-load-time step, not part of the expert operation (Lan,
 * Section 1: the per-expert feed-forward W_down (silu(W_gate x) * W_up x); the
 * layout is this library's).  Shared experts are packed with desc->N = n_shared.
 *   w, w_tiled  device, 16-byte aligned, not overlapping; desc->flags and
 *               desc->n_shared are ignored.
 * Asynchronous on hip_stream.  Returns MOE_OK, MOE_E_INVAL for a bad matrix code,
 * pointers or sizes that are not whole steps, MOE_E_DTYPE for a bad dtype (nothing
 * enqueued), or MOE_E_HIP. */
int moe_pack_tiled(const moe_layer_desc* desc, const void* w, void* w_tiled, int32_t mat,
                   void* hip_stream);

/*
 * moe_router_topk -- the router ahead of the expert operation: it sends each token
 * to m of the N experts (paper Section 1).  For every token t of the pass:
 *   logits[t][e] = W_r[e] . x_t                  (fp32 accumulation, e < N)
 *   ids[t][0..m)  the m largest logits, in descending order; equal logits: lower id first
 *   w[t][j]       = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the m selected logits
 *                 (the same weights as a softmax over all N renormalised to the m)
 * The ids and weights are in the layout the expert calls take.
 *   desc      N, m, d_model, dtype (d_ff, flags and n_shared are not used);
 *             m <= MOE_MAX_SLOTS
 *   w_router  device [N][d_model], dtype of desc, 16-byte aligned
 *   x         device [n][d_model], 16-byte aligned; 1 <= n <= MOE_MAX_TOKENS
 *   logits    device [n][N] fp32 (written)
 *   ids, w    device [n][m] int32 / fp32 (written)
 *   ws        device workspace of ws_bytes >= moe_router_workspace_bytes(desc, n),
 *             4-byte aligned: partial logits of up to 16 parts of the d contraction,
 *             added in a fixed order (no zero-fill needed)
 * Logits should be finite: NaN logits are never selected, and a slot left without
 * a candidate gets id -1 (which the expert calls skip).  Two kernel launches on
 * hip_stream, deterministic.
 * Returns MOE_OK, MOE_E_INVAL / MOE_E_DTYPE / MOE_E_WORKSPACE for bad arguments
 * (nothing enqueued), or MOE_E_HIP.
 */
int moe_router_topk(const moe_layer_desc* desc, const void* w_router, const void* x, int32_t n,
                    float* logits, int32_t* ids, float* w, void* ws, size_t ws_bytes,
                    void* hip_stream);

/* Workspace bytes of moe_router_topk for passes of up to n tokens (the largest over
 * 1..n), or 0 for invalid arguments. */
size_t moe_router_workspace_bytes(const moe_layer_desc* desc, int32_t n);

/* Number of kernel launches moe_expert_perslot / moe_expert_dedup enqueue per
 * call (moe_route_group is a separate, optional launch), or a negative status for
 * a bad kind. */
int moe_kernels_per_call(int32_t kind);

/* As moe_expert_perslot / moe_expert_dedup, and also records hip events:
 * events[0] before the first launch and events[i] after launch i, so
 * n_events must be moe_kernels_per_call(kind) + 1.  `events` are hipEvent_t
 * handles created by the caller.  For per-kernel timing. */
int moe_expert_perslot_ev(const moe_layer_desc* desc, const moe_layer_weights* weights,
                          const void* x, const int32_t* ids, const float* w, int32_t n, float* y,
                          int32_t* info, void* ws, size_t ws_bytes, void* hip_stream,
                          void* const* events, int32_t n_events);
int moe_expert_dedup_ev(const moe_layer_desc* desc, const moe_layer_weights* weights,
                        const void* x, const int32_t* ids, const float* w, int32_t n, float* y,
                        int32_t* info, void* ws, size_t ws_bytes, void* hip_stream,
                        void* const* events, int32_t n_events);

/*
 * bytes_requested -- expert bytes the kernel `kind` requests for the pass whose
 * ids (host [n][m]) are given (paper Section 1 "Bytes" and Section 3.1): with
 * w = 3 d_model d_ff sizeof(W),
 *     MOE_KIND_SLOT:  n m w           MOE_KIND_DEDUP:  X(n) w   (byte factor f = 1)
 * x, y, ids and routing-weight bytes are not counted, nor are the always-on experts
 * of desc->n_shared (the D(n) term of Eq. 5).  Host only, synchronous.
 * Returns the byte count, or -MOE_E_* (negative) for invalid arguments or ids.
 */
int64_t bytes_requested(int32_t kind, const moe_layer_desc* desc, const int32_t* ids_host,
                        int32_t n);

/* ---------------------------------------------------------------------------
 * step_time_model -- host-only evaluation of the paper's step-time model and
 * best draft length (Sections 1, 3.1-3.4; Appendix B), in double.
 *
 *   tau_p(n) = t0 + D(n)/beta_D + E_p(n)/beta_p(n) + phi_p(n),  D(n) = D + kv(n-1)   (Eq. 5)
 *   S(n)     = tau_slot(n) - tau_dedup(n)                                            (Eq. 6)
 *   crossover = smallest n in [2, n_max] with S(n') > 0 for all n' in [n, n_max]; 0 = none
 *   V_p(k)   = tau_p(k+1) + h(k);  V_p(0) = tau_slot(1) + h(0) for both kernels
 *              (a one-token pass runs the same kernel either way, Section 3.1)
 *   G_a(k)   = 1 + a + ... + a^k;  T_a(k) = G_a(k)/V(k);  k*(a) = smallest maximizer
 *   a0_p     = V_p(1)/V_p(0) - 1                                                     (B.4)
 *   speedup  = T_a(k*)/T_a(0)                                                        (Eq. 9)
 *   step point a_j = max_{i<j} min_{k>=j} alpha_{k,i},
 *              alpha_{k,i} = inf{a in [0,1) : T_a(k) > T_a(i)} (1 if empty)          (B.31)
 *   a1_convex = min(c_1/V(0), 1), valid when 0 <= c_1 <= ... (convex = 1)            (B.36)
 *   rho*_k(a) (Eq. 14, deduplicating engine):
 *       1 - (B_k/(m W k)) [(G_a(k)-1) tau(1) - (kv(k)-kv(0))/beta_D - dphi_k] - (B_k/beta(1) - 1)/k
 *       B_k = beta_dedup(k+1), beta(1) = beta_slot(1), tau(1) = tau_slot(1),
 *       dphi_k = phi_dedup(k+1) - phi_slot(1)
 *   rho*_k bytes (Eq. 16): 1 - [(G_a(k)-1)(D + m W + kv(0)) - (kv(k)-kv(0))]/(m W k)
 * Indexing: arrays over n use index n-1; arrays over k use index k.
 * Returns MOE_OK, or MOE_E_INVAL for sizes out of range or non-positive
 * bandwidths / m W.  Pure function, thread-safe.
 * ------------------------------------------------------------------------- */
#define MOE_STEP_NMAX 16
#define MOE_STEP_AMAX 64

typedef struct {
    int32_t n_max;                  /* pass sizes 1..n_max, 2 <= n_max <= MOE_STEP_NMAX */
    int32_t n_a;                    /* acceptance grid points, 1..MOE_STEP_AMAX */
    double a[MOE_STEP_AMAX];        /* acceptance values in [0, 1] */
    double m_W;                     /* m W: expert bytes of one token over the layers, > 0 */
    double t0;                      /* time outside memory reads */
    double D;                       /* bytes read once per pass */
    double kv[MOE_STEP_NMAX];       /* kv(k), k = 0..n_max-1 */
    double beta_D;                  /* bandwidth of the D(n) bytes, > 0 */
    double E[2][MOE_STEP_NMAX];     /* E_p(n), p = MOE_KIND_SLOT / MOE_KIND_DEDUP */
    double beta[2][MOE_STEP_NMAX];  /* beta_p(n), > 0 */
    double phi[2][MOE_STEP_NMAX];   /* phi_p(n) */
    double h[MOE_STEP_NMAX];        /* h(k), k = 0..n_max-1 */
} moe_step_in;

typedef struct {
    double tau[2][MOE_STEP_NMAX];
    double S[MOE_STEP_NMAX];
    int32_t crossover;
    double V[2][MOE_STEP_NMAX];
    double a0[2];
    int32_t kstar[2][MOE_STEP_AMAX];
    double speedup[2][MOE_STEP_AMAX];
    double step_point[2][MOE_STEP_NMAX]; /* a_j at index j, j = 1..n_max-1 */
    int32_t convex[2];
    double a1_convex[2];
    double rho_star[MOE_STEP_AMAX][MOE_STEP_NMAX];       /* [a index][k], k = 1..n_max-1 */
    double rho_star_bytes[MOE_STEP_AMAX][MOE_STEP_NMAX]; /* [a index][k] */
} moe_step_out;

int step_time_model(const moe_step_in* in, moe_step_out* out);

/*
 * moe_fit_times -- least-squares fit of one kernel's measured times over passes
 * with chosen ids (paper Section 2; a pass of n tokens whose n*m slots name U
 * distinct experts), host only, double:
 *   MOE_KIND_SLOT  (Eq. 4):   t = t_op + c_u U b + c_re (n m - U) b   coef = (t_op, c_u, c_re)
 *   MOE_KIND_DEDUP (Eq. E.1): t = t_op + c_g U b + c_t n             coef = (t_op, c_g, c_t)
 * b = bytes of one expert of the timed layer.  c_re / c_u is the re-read cost: 1
 * when a repeated slot is read again from memory, near 0 when a cache serves it.
 *   n, U, t  host [count]; 1 <= U[i] <= n[i] m; t in any fixed time unit
 *   coef     host [3], written on success
 * Householder QR on the column-scaled system.  Returns MOE_OK, or MOE_E_INVAL for
 * bad arguments, count < 3, or passes that do not determine all three constants.
 */
int moe_fit_times(int32_t kind, int32_t count, const int32_t* n, const int32_t* U, int32_t m,
                  const double* t, double b, double* coef);

/*
 * moe_error_bounds -- the factors of the bounds of paper Table 2 (Section 3.5,
 * Appendix C) for a relative bandwidth error |e| <= eps, 0 <= eps < 1/2, host only:
 *   out[0] = eps/(1-eps): (17) |tau^_p(n) - tau_p(n)| <= out[0] M_p(n) <= out[0] tau_p(n);
 *            (18) |S^(n) - S(n)| <= out[0] (M^e_slot(n) + M^e_dedup(n))
 *   out[1] = ln((1+eps)/(1-eps)): (19) the predicted faster kernel is the true one
 *            when |ln r(n) - ln u(n)| > out[1]
 *   out[2] = delta = eps/(1-eps), the relative step-time error from bandwidth errors
 *   out[3] = (1-delta)/(1+delta): (20) T_a(k^*) >= out[3] T_a(k*), and k^* = k* when
 *            T_a(i) < out[3] T_a(k*) for every i != k*
 *   out[4] = (1+delta)/(1-delta) = 1/(1-2 eps): (21) the predicted best speedup is
 *            within [1/out[4], out[4]] times the true one
 * Returns MOE_OK or MOE_E_INVAL.
 */
int moe_error_bounds(double eps, double* out);

/* ---------------------------------------------------------------------------
 * moe_tree_select -- the verification subtree of a draft tree chosen by reward over
 * predicted cycle time (SpecFit, arXiv:2610.15417, Sections 3.1-3.3, Algorithm 1),
 * host only.  Node 0 is the root s (the current token), nodes 1..V the draft pool,
 * parent[v] < v (parents before descendants; parent[v] = 0 for children of the root).
 *   legal family: S ancestor-closed (v in S => parent[v] in S or is the root), |S| <= K
 *   R(S) = 1 + sum_{v in S} p[v]
 *   F(S) = sum over layers l of |E_l(root) u U_{v in S} E_l(v)|   (expert bitmaps, popcount)
 *   T(S) = b[|S|] + beta F(S)
 * The selection maximises R/T; equal ratios prefer the larger R, the smaller F, fewer
 * nodes, then the lexicographically smaller list of node ids.  The search is the
 * depth-first enumeration that adds nodes in increasing id order, each only when its
 * parent is present, carrying the per-layer unions as bitmaps; ratios are compared by
 * cross-multiplication.  With max_level > 0 only nodes with level[v] <= max_level take
 * part (the selection after drafting max_level levels, Appendix A.2).
 * Used here with T calibrated from the deduplicating kernel's measured cost per union
 * expert and per pass (beta = c_g w, b_k from t_op + c_t (k+1)), in place of SpecFit's
 * host-to-device transfer cost.
 * Returns MOE_OK, or MOE_E_INVAL for sizes out of range, a bad parent, b or beta not
 * positive, or p negative.
 */
#define MOE_TREE_MAXV 63   /* draft nodes */
#define MOE_TREE_MAXK 16   /* largest subtree */
#define MOE_TREE_MAXW 16   /* 64-bit words of one layer's expert bitmap (N <= 1024) */
typedef struct {
    int32_t V;               /* draft nodes 1..V */
    int32_t L;               /* layers */
    int32_t words;           /* 64-bit words per layer bitmap, 1..MOE_TREE_MAXW */
    int32_t K;               /* largest subtree, 0..MOE_TREE_MAXK */
    const int32_t* parent;   /* [V+1]; parent[0] ignored */
    const double* p;         /* [V+1]; commit probability of node v; p[0] ignored */
    const uint64_t* bitmap;  /* [(V+1)][L][words]: bit e of layer l of node v = expert e */
    const double* b;         /* [K+1] intercepts, > 0 */
    double beta;             /* cost per union expert, > 0 */
    int32_t max_level;       /* <= 0: every node */
    const int32_t* level;    /* [V+1] depth of each node (root 0), read when max_level > 0 */
} moe_tree_in;
typedef struct {
    uint64_t selected;       /* bit v-1 set for each selected node v */
    int32_t count;           /* |S| */
    int32_t F;               /* union feature of S */
    double R, T;             /* reward and predicted cycle time of S */
    int64_t visited;         /* legal subtrees enumerated (the root-only one included) */
} moe_tree_out;
int moe_tree_select(const moe_tree_in* in, moe_tree_out* out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_H */
