/*
 * dp.h -- C ABI of the MI355X (gfx950) DeltaProduct forward library, libdp.so.
 *
 * What is computed (by page title; section / equation on that page):
 *
 *  "DeltaProduct: Improving State-Tracking in Linear RNNs via Householder
 *   Products" (study notes of arXiv 2502.10297v7)
 *   - sec. 2.2, Eq.(3): each token i applies n_h ordered generalized
 *     Householder updates to a per-head dk x dv matrix memory,
 *       H_{i,j} = (I - b_{ij} k_{ij} k_{ij}^T) H_{i,j-1} + b_{ij} k_{ij} v_{ij}^T,
 *     with H_{i,0} = H_{i-1} and unit keys k_{ij} (L2-normalised here);
 *   - sec. 2.6: an optional per-token gate g_i scales the state once,
 *     before the token's first sub-step (H_{i,0} = g_i H_{i-1}); the
 *     readout is o_i = H_i^T q_i;
 *   - sec. 4.1 (Sec.5.1): the computation runs as a chunkwise delta-rule scan
 *     over the expanded sequence of L*n_h interleaved sub-steps with gate
 *     (g_1, 1, .., 1, g_2, 1, ..), keeping only each token's last sub-step.
 *  "OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
 *   Attention" (study notes of arXiv 2605.13473v1)
 *   - sec. 2.2, Eqs.(2)/(5): asymmetric write key; the residual uses the
 *     read key k, the write uses kt: H += b kt (v - H^T k)^T;
 *   - sec. 2.5 (App.A.2): chunkwise form T = (I + tril(B K Kt^T, -1))^-1,
 *     W = T B K, U = T B V, state S += (U - W S^T)^T Kt, scores Q Kt^T;
 *   - sec. 2.4 (Alg.1): phase-1 preconditioner scan producing kt = d_t * k_t.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them.  Layouts are dense,
 *     row-major, in the order given.  q, k, kt, v and dout must be 16-byte
 *     aligned.
 *   - "T" is the path element type: IEEE float for *_f32 entry points,
 *     bfloat16 (raw uint16 bits) for *_bf16.  beta, g, h0, final_state and
 *     the phase-1 vector d are always float32.
 *   - Validation happens on the host, before any HIP call; on failure the
 *     call returns a negative dp_status and enqueues nothing.  On success the
 *     work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns DP_OK without waiting for it.
 *   - Inputs are read-only and must not overlap out, final_state or the
 *     workspace.  When L == 0 the per-token tensors are empty and may be NULL.  h0 and final_state MAY be the same buffer (in-place resume).
 *   - The library keeps no global state, with one stated exception (the
 *     fixed scratch array of dp_fwd_varlen_noalloc_bf16): calls on different
 *     streams may run concurrently as long as their buffers are disjoint.
 *   - NaN and Inf in the inputs propagate; nothing is silently repaired.
 *   - Precision: the state and every accumulation are fp32.  On the bf16
 *     path the computed MFMA operands (normalised keys, queries, write keys,
 *     a rounded copy of the state, T diag(beta), pseudo-values, scores) are
 *     fp16, so q, kt, v and the state must stay within fp16 range
 *     (|x| < 65504): past it the operand is +-Inf, the results that depend
 *     on it are not finite (a query: its token's output row; a pseudo-value:
 *     its head from that chunk on) and other heads are unaffected.  The fp32
 *     path uses fp32 throughout.
 *   - Supported shapes: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64}
 *     (counted in sub-steps of the expanded sequence); 1 <= n_h <= 64.
 *     B, H >= 1, L >= 0.  L*n_h need not be a multiple of chunk: the tail is
 *     padded internally with beta = 0 sub-steps, which are exact identities.
 */
#ifndef DP_H
#define DP_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DP_OK = 0,
    DP_EINVAL = -1,     /* null required pointer, bad size, misaligned pointer */
    DP_ENOTSUP = -2,    /* dk/dv/chunk/n_h outside the supported set */
    DP_EWORKSPACE = -3, /* workspace missing or smaller than dp_fwd_workspace_size */
    DP_EHIP = -4,       /* a HIP launch or runtime call failed */
    DP_ESCRATCH = -5    /* beyond the fixed scratch of dp_fwd_varlen_noalloc_bf16 */
} dp_status;

typedef void* dp_stream; /* hipStream_t */

/* Stage bits for dp_fwd_ex_*.  DP_STAGE_ALL is what dp_fwd_* run. */
#define DP_STAGE_UT 1   /* per-chunk prep + UT transform -> workspace          */
#define DP_STAGE_SCAN 2 /* inter-chunk state scan + readout + final state       */
#define DP_STAGE_ALL 3

/* Static string for a status code (never NULL). */
const char* dp_status_str(int status);

/*
 * Workspace bytes needed by dp_fwd_* / dp_fwd_wk_* for these sizes.
 * elem_bytes: 4 for the f32 path, 2 for the bf16 path.  Writes *bytes and
 * returns DP_OK, or a negative status (sizes validated as for dp_fwd_*).
 * The workspace holds, per chunk of every head: on the fp32 path and the
 * bf16 write-key path, the matrix T*diag(beta) (chunk x chunk) and two floats
 * per sub-step (1/|k| and the chunk-local cumulative log-gate); on the bf16
 * symmetric path, one operand block (T*diag(beta), the unit keys, the readout
 * queries and their masked scores in fp16, then the per-sub-step decay
 * factors and the readout rows' output offsets), plus one float per lane of
 * the chunk-scan launch.
 */
int dp_fwd_workspace_size(int n_h, int B, int H, int L, int dk, int dv, int chunk,
                          int elem_bytes, size_t* bytes);

/*
 * Launch plan the forward would use for these sizes (for measurement and
 * tuning; nothing is launched).  asym: 0 symmetric, 1 write-key variant.
 * info[0] = BV, the value columns per scan workgroup (16, 32 or 64)
 * info[1] = scan (or fused) workgroups (B*H*dv/BV), info[2] = UT workgroups
 * (chunks; 0 when the default call runs the fused kernel),
 * info[3] = scan LDS bytes, info[4] = prep / UT LDS bytes, info[5] = readout rows
 * per chunk (padded to 16).  Returns DP_OK or a validation status.
 */
int dp_fwd_launch_info(int n_h, int B, int H, int L, int dk, int dv, int chunk, int elem_bytes,
                       int asym, int* info);

/*
 * Symmetric DeltaProduct forward (DeltaProduct notes sec. 2.2 Eq.(3),
 * sec. 2.6, sec. 4.1).
 *   q     [B, L, H, dk]         T   readout queries, used as given
 *   k     [B, L, H, n_h, dk]    T   raw keys; each is divided by
 *                                   max(|k|_2, 1e-6) inside
 *   v     [B, L, H, n_h, dv]    T
 *   beta  [B, L, H, n_h]      f32   clamped to [0, 2] inside
 *   g     [B, L, H]           f32   per-token gate in [0, 1]; NULL = no gate.
 *                                   g = 0 is handled as log(FLT_MIN).
 *   out   [B, L, H, dv]         T   written: H_t^T q_t after token t's last
 *                                   sub-step (rounded to nearest even for bf16)
 *   final_state [B, H, dk, dv] f32  written with H_L; NULL = not returned
 *   h0    [B, H, dk, dv]      f32   initial state H_0; NULL = zero
 *   workspace / workspace_bytes     device scratch of at least
 *                                   dp_fwd_workspace_size() bytes, 256-byte
 *                                   aligned; its contents on entry are ignored
 * Errors: DP_EINVAL, DP_ENOTSUP, DP_EWORKSPACE (before any HIP call),
 * DP_EHIP (launch failure).
 */
int dp_fwd_f32(const float* q, const float* k, const float* v, const float* beta,
               const float* g, int n_h, int B, int H, int L, int dk, int dv, int chunk,
               float* out, float* final_state, const float* h0, void* workspace,
               size_t workspace_bytes, dp_stream stream);
int dp_fwd_bf16(const void* q, const void* k, const void* v, const float* beta,
                const float* g, int n_h, int B, int H, int L, int dk, int dv, int chunk,
                void* out, float* final_state, const float* h0, void* workspace,
                size_t workspace_bytes, dp_stream stream);

/*
 * Asymmetric write-key forward (OSDN notes sec. 2.2 Eqs.(2)/(5), sec. 2.5):
 * the residual and the transform's left factor use the normalised read key k,
 * the write and the readout scores use kt exactly as given (not normalised).
 *   kt    [B, L, H, n_h, dk]    T   write keys (e.g. from dp_osdn_precond_*)
 * Every other argument is as for dp_fwd_*.
 */
int dp_fwd_wk_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, int n_h, int B, int H, int L, int dk,
                  int dv, int chunk, float* out, float* final_state, const float* h0,
                  void* workspace, size_t workspace_bytes, dp_stream stream);
int dp_fwd_wk_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, int n_h, int B, int H, int L, int dk,
                   int dv, int chunk, void* out, float* final_state, const float* h0,
                   void* workspace, size_t workspace_bytes, dp_stream stream);

/*
 * General form of the forward: kt may be NULL (symmetric, as dp_fwd_*) or a
 * write-key tensor (as dp_fwd_wk_*); ga may be NULL or the per-key-channel
 * gate of the KDA host (OSDN notes sec. 2.7):
 *   ga    [B, L, H, dk]         f32   alpha_t in (0, 1]: before token t's
 *                                     sub-steps, state row (key channel) c is
 *                                     multiplied by ga[t][c] (then by g[t])
 * With ga the forward runs the UT and scan kernels for either input type
 * (fp32 arithmetic on the fp32 path, fp16 operands on the bf16 path, as
 * elsewhere): each decay factor is formed for its own pair of sub-steps and is
 * at most 1, so no channel's decay can overflow an operand.  A gate of 0 is
 * taken as FLT_MIN.  `flags` is an OR of
 *   DP_STAGE_UT    run the per-chunk prep + UT launch (fills the workspace)
 *   DP_STAGE_SCAN  run the chunk-scan launch (reads the workspace; writes out
 *                  and final_state)
 *   DP_OUT_F32     write `out` as float32 [B, L, H, dv] instead of T (bf16
 *                  path only; the fp32 path always writes float32).  With bf16
 *                  out the output carries the bf16 rounding of every element
 *                  (relative 2^-9) on top of the fp32 accumulation: at long
 *                  sequences with large state norms (L = 16384, H = 8) that
 *                  rounding reaches ~2.5e-2 of max|out|, so callers that need
 *                  the tighter figure ask for fp32 out
 *   DP_FWD_SPLIT   symmetric bf16 keys: run the two-kernel path (a prep kernel
 *                  writes each chunk's operand blocks to the workspace, a chain
 *                  kernel reads them)
 *   DP_FWD_FUSED   symmetric bf16 keys, no ga, dk and chunk multiples of 32, both
 *                  stages: run the single fused kernel (each workgroup builds
 *                  its chunk's operands in LDS; no workspace is read or written,
 *                  and `workspace` may be NULL with workspace_bytes 0).
 *                  DP_ENOTSUP where those conditions do not hold
 * At least one stage bit must be set; DP_FWD_SPLIT with DP_FWD_FUSED is
 * DP_EINVAL.  Without either, symmetric bf16 keys take the fused kernel where
 * one workgroup holds all dv columns of a head (dv <= 32, dk and chunk
 * multiples of 32, both stages) and the two-kernel path elsewhere; the
 * workspace from dp_fwd_workspace_size covers both.  Both paths compute the
 * same forward to within their rounding.  DP_STAGE_UT then DP_STAGE_SCAN with
 * the same arguments is exactly one DP_STAGE_ALL call on the two-kernel path;
 * DP_STAGE_SCAN alone requires a workspace filled by DP_STAGE_UT for the same
 * k, kt, beta, g and sizes.  The stages exist for measurement and inspection.
 */
#define DP_OUT_F32 4
#define DP_FWD_SPLIT 8
#define DP_FWD_FUSED 16

int dp_fwd_ex_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, const float* ga, int n_h, int B, int H, int L,
                  int dk, int dv, int chunk, float* out, float* final_state, const float* h0,
                  void* workspace, size_t workspace_bytes, int flags, dp_stream stream);
int dp_fwd_ex_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, const float* ga, int n_h, int B, int H, int L,
                   int dk, int dv, int chunk, void* out, float* final_state, const float* h0,
                   void* workspace, size_t workspace_bytes, int flags, dp_stream stream);

/*
 * OSDN phase 1 (OSDN notes sec. 2.3-2.4, Alg.1), one sequential scan per head:
 *   k_t  <- k_t / max(|k_t|_2, 1e-6),  s = k_t * k_t,  b = clamp(beta_t, 0, 2)
 *   kt_t  = d_t * k_t                          (emitted before the update)
 *   d_{t+1} = clamp(d_t + eta * b * (1 - b <d_t, s>) / max(sum(s), eps) * s,
 *                   dmin, dmax)                (elementwise projection)
 *   k       [B, L, H, dk]   T    raw keys (the n_h = 1 key layout)
 *   beta    [B, L, H]     f32
 *   d_state [B, H, dk]    f32    in: d_1 (the notes use all ones); out: d_{L+1}
 *   kt      [B, L, H, dk]   T    written
 * eta, dmin, dmax, eps: the notes' final setting is 3e-3, 0.5, 2, 1e-6;
 * requires 0 < dmin <= dmax and eps > 0.  dk in {16, 32, 64, 128}.
 */
int dp_osdn_precond_f32(const float* k, const float* beta, int B, int H, int L, int dk,
                        float eta, float dmin, float dmax, float eps, float* d_state,
                        float* kt, dp_stream stream);
int dp_osdn_precond_bf16(const void* k, const float* beta, int B, int H, int L, int dk,
                         float eta, float dmin, float dmax, float eps, float* d_state,
                         void* kt, dp_stream stream);

/*
 * Phase-1 variants (OSDN notes sec. 2.6 and sec. 2.7), same scan and layouts:
 *   r      [B, L, H] f32  APF retention gate of d (sec. 2.6, Sec.4.4), or NULL
 *                         (= 1, exactly dp_osdn_precond_*):
 *                           d_{t+1} = P[ r_t d_t + step(d_t) ]
 *                         the step is computed from d_t before the retention;
 *   flags  0, or DP_PRECOND_BETA_FREE: the beta-free step of the 1.3B
 *          configuration (sec. 2.7, App.B/C), eta (1 - <d_t, s>) / max(|k|^2, eps) s,
 *          i.e. the step above with b = 1 (the forward's write still uses beta);
 *   P      the box [dmin, dmax]; here dmin may be <= 0 and the bounds may be
 *          -inf / +inf (no projection), as long as dmin <= dmax.
 * Errors: as dp_osdn_precond_*, plus DP_EINVAL for an unknown flag.
 */
#define DP_PRECOND_BETA_FREE 1

int dp_osdn_precond_ex_f32(const float* k, const float* beta, const float* r, int flags, int B,
                           int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                           float* d_state, float* kt, dp_stream stream);
int dp_osdn_precond_ex_bf16(const void* k, const float* beta, const float* r, int flags, int B,
                            int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                            float* d_state, void* kt, dp_stream stream);

/*
 * Pipeline handle for dp_osdn_fwd_bf16: a second stream on one device (non-
 * blocking, default priority) and the events that order it against the
 * caller's stream.  dp_pipeline_create makes one on the current device and
 * returns DP_OK, DP_EINVAL for a NULL `out`, or DP_EHIP (nothing is then
 * left allocated).  The caller owns it: dp_pipeline_destroy waits for the
 * work enqueued on its stream, then releases it (NULL is a no-op).  Calls
 * that use one handle are serialised on its stream and may come from several
 * host threads (each call holds the handle for its enqueue sequence); calls
 * that should overlap in time use handles of their own.
 */
typedef struct dp_pipeline_s* dp_pipeline;
int dp_pipeline_create(dp_pipeline* out);
int dp_pipeline_destroy(dp_pipeline pipe);

/* OSDN phase 1 and the write-key forward in one call, pipelined over token
 * segments (OSDN notes sec. 2.4 Alg. 1 for phase 1, sec. 2.5 for phase 2; the
 * DeltaProduct notes sec. 2.2 and 2.6 for the recurrence, with n_h = 1).
 * Computes what dp_osdn_precond_bf16 followed by dp_fwd_wk_bf16 with the
 * emitted write keys computes, but the sequence is cut into `segments` runs
 * of whole chunks: while the forward of one run proceeds on the second stream
 * of `pipe`, phase 1 already runs on the next run on `stream`, and `stream`
 * waits for both at the end.  With pipe == NULL the runs go one after another
 * on `stream` (no overlap; the same results bit for bit).
 * Phase 1 here: for dk < 64 the sequential scan of dp_osdn_precond_bf16 (the
 * same results bit for bit); for dk >= 64 its chunked form: each run's
 * 64-token chunks solve their linear system in parallel, d passes from chunk
 * to chunk, and a head whose step comes within 1e-5 (relative, at least
 * 1e-5 absolute) of a finite bound of the box, or is NaN, runs the
 * sequential scan again from the start of that chunk.  The result is the
 * sequential definition's to fp32 rounding (not bit for bit: the sums are
 * ordered differently).
 *   q [B,L,H,dk], k [B,L,H,dk] (raw read keys), v [B,L,H,dv]  bf16
 *   beta [B,L,H] f32;  h0 [B,H,dk,dv] f32 or NULL (zero)
 *   eta, dmin, dmax, eps: the phase-1 constants (3e-3, 0.5, 2, 1e-6)
 *   d_state [B,H,dk] f32 in/out: d_1 on entry, d_{L+1} on exit
 *   kt [B,L,H,dk] bf16 written: the write keys d_t o kh_t
 *   out [B,L,H,dv] bf16 written;  final_state [B,H,dk,dv] f32 written (the
 *   state passes through it between runs: it must not be NULL when the call
 *   makes more than one run, and may alias h0)
 *   workspace: dp_osdn_fwd_workspace_size() bytes (one run's forward, then for
 *              dk >= 64 one run's chunked phase 1), 256-byte aligned
 *   segments: 1 .. 16 (runs of ceil(ceil(L / segments) / chunk) chunks)
 *   pipe: a handle from dp_pipeline_create on the current device, or NULL
 * Every argument of every run is checked before the first run is enqueued:
 * on failure nothing is enqueued and d_state, kt, out and final_state are
 * untouched.  Errors: those of the two calls it replaces; DP_EINVAL for
 * segments outside 1 .. 16, a NULL final_state with several runs, or a
 * handle made on another device; DP_EHIP when a HIP call fails (runs already
 * enqueued then stay enqueued). */
int dp_osdn_fwd_workspace_size(int B, int H, int L, int dk, int dv, int chunk, int segments,
                               size_t* bytes);
int dp_osdn_fwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* h0,
                     int B, int H, int L, int dk, int dv, int chunk, float eta, float dmin, float dmax,
                     float eps, float* d_state, void* kt, void* out, float* final_state, void* workspace,
                     size_t workspace_bytes, int segments, dp_pipeline pipe, dp_stream stream);

/*
 * Packed variable-length sequences, bf16 with symmetric keys (DeltaProduct
 * notes sec. 2.2, 2.6, 4.1): nseq independent sequences packed along one
 * token axis, sequence d being tokens cu_seqlens[d] .. cu_seqlens[d+1]-1.  Each
 * sequence starts from its own initial state and is chunked on its own (no
 * chunk straddles two sequences), so every result equals dp_fwd_bf16 run on
 * that sequence alone.
 *   q [T, H, dk], k [T, H, n_h, dk], v [T, H, n_h, dv]   bf16
 *   beta [T, H, n_h], g [T, H] or NULL                   f32
 *   cu_seqlens [nseq + 1] int32, DEVICE memory: 0 = cu[0] <= cu[1] <= ..
 *              <= cu[nseq] = T.  Offsets that break this are not read as
 *              sequences: every sequence is then treated as empty (out is not
 *              written, final_state receives h0).
 *   out [T, H, dv] bf16 (float32 with DP_OUT_F32)
 *   h0, final_state [nseq, H, dk, dv] f32, each nullable (as in dp_fwd_*)
 *   workspace: dp_fwd_varlen_workspace_size() bytes, 256-byte aligned
 *   flags: stage bits as for dp_fwd_ex_* (DP_STAGE_SCAN alone needs a
 *          workspace filled by DP_STAGE_UT for the same inputs) | DP_OUT_F32
 * Errors: as dp_fwd_ex_bf16; nseq < 1 or T < 0 is DP_EINVAL.
 */
int dp_fwd_varlen_workspace_size(int n_h, int nseq, int H, int T, int dk, int dv, int chunk,
                                 size_t* bytes);
int dp_fwd_varlen_bf16(const void* q, const void* k, const void* v, const float* beta,
                       const float* g, const int* cu_seqlens, int nseq, int n_h, int H, int T,
                       int dk, int dv, int chunk, void* out, float* final_state, const float* h0,
                       void* workspace, size_t workspace_bytes, int flags, dp_stream stream);

/*
 * The packed forward on fp32 inputs (q, k, kt, v and out all float32; the
 * UT / scan kernels), symmetric keys or write keys; otherwise as
 * dp_fwd_varlen_bf16 and dp_fwd_varlen_wk_bf16, with the same workspace size.
 * Each result equals dp_fwd_f32 / dp_fwd_wk_f32 run on that sequence alone.
 * Errors: as dp_fwd_ex_f32; kt NULL with T > 0 (write keys) is DP_EINVAL.
 */
int dp_fwd_varlen_f32(const float* q, const float* k, const float* v, const float* beta,
                      const float* g, const int* cu_seqlens, int nseq, int n_h, int H, int T,
                      int dk, int dv, int chunk, float* out, float* final_state, const float* h0,
                      void* workspace, size_t workspace_bytes, int flags, dp_stream stream);
int dp_fwd_varlen_wk_f32(const float* q, const float* k, const float* kt, const float* v,
                         const float* beta, const float* g, const int* cu_seqlens, int nseq,
                         int n_h, int H, int T, int dk, int dv, int chunk, float* out,
                         float* final_state, const float* h0, void* workspace,
                         size_t workspace_bytes, int flags, dp_stream stream);

/*
 * Packed variable-length write-key forward (OSDN notes sec. 2.5 phase 2, on
 * the packed batches of sec. 3.4: documents packed along one token axis, the
 * state restarting at each document): dp_fwd_varlen_bf16 with the write keys
 * kt [T, H, n_h, dk] bf16 (e.g. from dp_osdn_precond_varlen_bf16) in the
 * state update and the readout scores, as dp_fwd_wk_bf16 does for one batch.
 * Each result equals dp_fwd_wk_bf16 run on that sequence alone.  Runs on the
 * prep / chain pair: dk and chunk multiples of 32, else DP_ENOTSUP.
 * workspace: dp_fwd_varlen_workspace_size() bytes (one size serves both
 * packed forms).  Errors: as dp_fwd_varlen_bf16; kt NULL with T > 0 or not
 * 16-byte aligned is DP_EINVAL; DP_FWD_FUSED is DP_ENOTSUP.
 */
int dp_fwd_varlen_wk_bf16(const void* q, const void* k, const void* kt, const void* v,
                          const float* beta, const float* g, const int* cu_seqlens, int nseq,
                          int n_h, int H, int T, int dk, int dv, int chunk, void* out,
                          float* final_state, const float* h0, void* workspace,
                          size_t workspace_bytes, int flags, dp_stream stream);

/*
 * Packed variable-length OSDN phase 1 (OSDN notes sec. 2.4 and the packed
 * batches of sec. 3.4): phase 1 of dp_osdn_precond_ex_* run on each of nseq
 * sequences packed along one token axis, every sequence from its own d.
 *   k [T, H, dk] T, beta [T, H] f32, r [T, H] f32 or NULL, kt [T, H, dk] T
 *   cu_seqlens [nseq + 1] int32, DEVICE memory; sequence d is tokens
 *              cu_seqlens[d] .. cu_seqlens[d+1]-1.
 *   d_state [nseq, H, dk] f32   in: each sequence's d_1; out: its d after its
 *              last token.
 *   flags, eta, dmin, dmax, eps: as dp_osdn_precond_ex_* (the box may be open).
 *   workspace: NULL, or dp_osdn_precond_varlen_workspace_size() bytes, 256-byte
 *              aligned.  Without one, the exact sequential scan per sequence:
 *              each sequence's kt and d equal dp_osdn_precond_ex_* on it alone,
 *              bit for bit.  With one and dk >= 64, the 64-token chunked form
 *              of dp_osdn_fwd_bf16 (chunks from each sequence's start; a head
 *              that comes within a margin of the box, or meets a NaN, runs the
 *              exact scan from that chunk): the same values up to rounding.
 * Offsets: in the exact scan a sequence is read only if 0 = cu[0], cu[d] <=
 * cu[d+1] and cu[nseq] = T; in the chunked form every sequence is empty
 * unless 0 = cu[0] <= cu[1] <= .. <= cu[nseq] = T.  An empty sequence writes
 * no kt row and keeps its d.  Offsets that decrease make sequences overlap in
 * the exact scan, and the kt rows they share are then undefined.
 * Errors: as dp_osdn_precond_ex_*; cu_seqlens NULL, nseq < 1 or T < 0 is
 * DP_EINVAL; a workspace too small or misaligned is DP_EWORKSPACE.
 */
int dp_osdn_precond_varlen_workspace_size(int nseq, int H, int T, int dk, size_t* bytes);
int dp_osdn_precond_varlen_f32(const float* k, const float* beta, const float* r, int flags,
                               const int* cu_seqlens, int nseq, int H, int T, int dk, float eta,
                               float dmin, float dmax, float eps, float* d_state, float* kt,
                               void* workspace, size_t workspace_bytes, dp_stream stream);
int dp_osdn_precond_varlen_bf16(const void* k, const float* beta, const float* r, int flags,
                                const int* cu_seqlens, int nseq, int H, int T, int dk, float eta,
                                float dmin, float dmax, float eps, float* d_state, void* kt,
                                void* workspace, size_t workspace_bytes, dp_stream stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dp_fwd_varlen_bf16 with DP_FWD_FUSED, without a workspace.  The fused
 * kernel's only scratch, the per-sequence chunk-offset table (nseq + 1 ints),
 * lives in a fixed array inside the library: (DP_NOALLOC_MAX_SEQS + 1) ints =
 * 256 KiB on every device the library runs on, held until the process ends.
 * The call allocates nothing.  Arguments as for dp_fwd_varlen_bf16, with
 *   flags: 0 or DP_OUT_F32 (both stages always run)
 * Results equal dp_fwd_varlen_bf16 with DP_FWD_FUSED bit for bit.  Nothing in
 * the array needs clearing: each call writes all nseq + 1 entries before its
 * forward reads them.  Calls on one device share the array: two calls that
 * overlap in time there (other streams, other threads) race, and their
 * results are undefined; the caller serialises them.
 * Errors: as dp_fwd_varlen_bf16; DP_ESCRATCH when nseq > DP_NOALLOC_MAX_SEQS;
 * DP_ENOTSUP when dk or chunk is not a multiple of 32 (no fused kernel).
 */
#define DP_NOALLOC_MAX_SEQS 65535
int dp_fwd_varlen_noalloc_bf16(const void* q, const void* k, const void* v, const float* beta,
                               const float* g, const int* cu_seqlens, int nseq, int n_h, int H,
                               int T, int dk, int dv, int chunk, void* out, float* final_state,
                               const float* h0, int flags, dp_stream stream);

/*
 * One recurrent decode step (DeltaProduct notes sec. 2.2 Eq.(3) and the
 * per-token pseudocode of sec. 2.6; OSDN notes sec. 2.2 Eqs.(2)/(5) for kt,
 * sec. 2.7 for the KDA host's per-key-channel gate): every head applies ONE
 * token's n_h sub-steps to its resident state and reads it out, exactly as
 * one token of dp_fwd_* / dp_fwd_wk_* (with ga == NULL):
 *   H <- g H;  H <- Diag(ga) H  (each when given);
 *   for j < n_h: H <- H + clamp(b_j,0,2) w_j (v_j - H^T kn_j)^T;
 *   out = H^T q,
 * kn_j = k_j / max(|k_j|_2, 1e-6), w_j = kn_j (kt == NULL) or kt_j as given.
 * The per-token tensors are the forward's with L = 1:
 *   q    [B, H, dk]          T
 *   k    [B, H, n_h, dk]     T   raw keys
 *   kt   [B, H, n_h, dk]     T   write keys, or NULL (symmetric)
 *   v    [B, H, n_h, dv]     T
 *   beta [B, H, n_h]       f32
 *   g    [B, H]            f32   or NULL (no gate); the state is multiplied
 *                                by g as given
 *   ga   [B, H, dk]        f32   or NULL: per-key-channel gate alpha (KDA
 *                                host), state row r multiplied by ga[r]
 *   out  [B, H, dv]          T   written (float32 with DP_OUT_F32; the _f32
 *                                entry point always writes float32)
 *   state [B, H, dk, dv]   f32   in/out: H_{t-1} on entry, H_t on exit (the
 *                                final_state of a dp_fwd_* prefill continues
 *                                here unchanged)
 * flags: 0 or DP_OUT_F32.  The state is updated in place: it must not overlap
 * any other argument.  The whole step is fp32 arithmetic on the fp32 state.
 * Errors: DP_EINVAL (null required pointer, size <= 0, unknown flag),
 * DP_ENOTSUP (dk or dv outside {16, 32, 64, 128}, n_h > 64), DP_EHIP.
 */
int dp_decode_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, const float* ga, int n_h, int B, int H,
                  int dk, int dv, float* out, float* state, int flags, dp_stream stream);
int dp_decode_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, const float* ga, int n_h, int B, int H,
                   int dk, int dv, void* out, float* state, int flags, dp_stream stream);

/*
 * Gradient of the symmetric forward (dp_fwd_f32 / dp_fwd_bf16 without write
 * keys) w.r.t. all of its inputs: the reverse-mode derivative of the
 * recurrence of DeltaProduct notes sec. 2.2 Eq.(3) with the gate and readout
 * of sec. 2.6 over the expanded sequence of sec. 4.1, computed in the
 * chunkwise form of the OSDN notes sec. 2.5 / App.A.2.  For a loss with
 * gradient dout on out and dfinal on final_state it returns
 *   dq    [B, L, H, dk]        f32   written
 *   dk_out [B, L, H, n_h, dk]  f32   written: w.r.t. the RAW keys (through
 *                                    k / max(|k|_2, 1e-6))
 *   dv_out [B, L, H, n_h, dv]  f32   written
 *   dbeta [B, L, H, n_h]       f32   written: w.r.t. the raw beta; zero where
 *                                    beta lies outside [0, 2] (the clamp)
 *   dg    [B, L, H]            f32   written when g is given, else untouched;
 *                                    may be NULL.  Zero where g < FLT_MIN (the
 *                                    forward uses log(max(g, FLT_MIN)))
 *   dh0   [B, H, dk, dv]       f32   written, or NULL (not returned); the
 *                                    gradient w.r.t. h0 (zero h0 when NULL)
 * The inputs are the forward's (q, k, v, beta, g, h0 with the same layouts
 * and types; T = float or bf16 by suffix), plus
 *   dout   [B, L, H, dv]   T     gradient on out
 *   dfinal [B, H, dk, dv]  f32   gradient on final_state, or NULL (zero)
 * The backward recomputes the forward's chunk states itself: nothing from a
 * forward call is needed.  workspace: dp_bwd_workspace_size() bytes,
 * 256-byte aligned, caller-owned (T and the key scalars per 32-sub-step
 * chunk, the chunk-start states and their gradients, all fp32: about
 * 2 dk dv 4 B per 32 sub-steps per head).  The state, its gradient and
 * every accumulation are fp32; the MFMA operands are fp32 on the fp32 path
 * and fp16 on the bf16 path (as the forward's, with the same range).
 * Errors: DP_EINVAL (null required pointer, sizes <= 0), DP_ENOTSUP (dk or
 * dv outside {16, 32, 64, 128}, n_h > 64, sizes past the 32-bit index
 * limits), DP_EWORKSPACE, DP_EHIP.
 */
int dp_bwd_workspace_size(int n_h, int B, int H, int L, int dk, int dv, size_t* bytes);
int dp_bwd_f32(const float* q, const float* k, const float* v, const float* beta, const float* g,
               const float* h0, const float* dout, const float* dfinal, int n_h, int B, int H,
               int L, int dk, int dv, float* dq, float* dk_out, float* dv_out, float* dbeta,
               float* dg, float* dh0, void* workspace, size_t workspace_bytes, dp_stream stream);
int dp_bwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* g,
                const float* h0, const void* dout, const float* dfinal, int n_h, int B, int H,
                int L, int dk, int dv, float* dq, float* dk_out, float* dv_out, float* dbeta,
                float* dg, float* dh0, void* workspace, size_t workspace_bytes, dp_stream stream);

/*
 * Gradient of the write-key forward (dp_fwd_wk_*; OSDN notes sec. 2.5 phase 2,
 * App.A.2: M = strict_tril(diag(beta)(K W^T)), the state update and the
 * readout scores with the write keys W, the state read and X with the unit
 * read keys K).  Arguments as dp_bwd_*, plus
 *   kt   [B, L, H, n_h, dk]  T    the write keys, as the forward used them
 *   dkt  [B, L, H, n_h, dk]  f32  written: the gradient w.r.t. kt (kt is used
 *                                 as given, so no normalisation is undone)
 * and dk_out is then the gradient w.r.t. the raw read keys only.  Workspace:
 * dp_bwd_workspace_size() bytes.  Errors as dp_bwd_*, and DP_EINVAL for a
 * NULL kt or dkt when L > 0.
 */
int dp_bwd_wk_f32(const float* q, const float* k, const float* kt, const float* v, const float* beta,
                  const float* g, const float* h0, const float* dout, const float* dfinal, int n_h, int B,
                  int H, int L, int dk, int dv, float* dq, float* dk_out, float* dkt, float* dv_out,
                  float* dbeta, float* dg, float* dh0, void* workspace, size_t workspace_bytes,
                  dp_stream stream);
int dp_bwd_wk_bf16(const void* q, const void* k, const void* kt, const void* v, const float* beta,
                   const float* g, const float* h0, const void* dout, const float* dfinal, int n_h, int B,
                   int H, int L, int dk, int dv, float* dq, float* dk_out, float* dkt, float* dv_out,
                   float* dbeta, float* dg, float* dh0, void* workspace, size_t workspace_bytes,
                   dp_stream stream);

/*
 * Gradient of OSDN phase 1 (OSDN notes sec. 2.5, closing paragraph: the write
 * key kt_t = d_t o kh_t passes its gradient into d_t and k_t, and the
 * gradient of d runs back through the recursion of sec. 2.4; with the
 * retention of sec. 2.6 and the beta-free step of sec. 2.7).  The derivative
 * of the projection onto the box is taken as 1 on [dmin, dmax] (end points
 * included) and 0 outside, per coordinate, as for the beta clamp.  Phase 1 is
 * run again first from d0, keeping every d_t in the workspace.
 *   k, beta, r, flags, eta, dmin, dmax, eps: as dp_osdn_precond_ex_* (n_h = 1
 *                layout; r may be NULL)
 *   d0       [B, H, dk]    f32  d_1, or NULL (all ones)
 *   dkt      [B, L, H, dk] f32  gradient on the emitted write keys
 *   dd_final [B, H, dk]    f32  gradient on the final d, or NULL (zero)
 *   dk_out   [B, L, H, dk] f32  ACCUMULATED into: += the raw-key gradient
 *   dbeta    [B, L, H]     f32  ACCUMULATED into: += the beta gradient (none
 *                               with DP_PRECOND_BETA_FREE or outside [0, 2])
 *   dret     [B, L, H]     f32  written (zero without r), or NULL
 *   dd0      [B, H, dk]    f32  written: the gradient on d_1, or NULL
 * dk_out and dbeta accumulate so that they can already hold the write-key
 * forward's gradients on the same keys and beta (dp_bwd_wk_*, n_h = 1); clear
 * them first for phase 1 alone.  workspace: dp_osdn_precond_bwd_workspace_size()
 * bytes, 256-byte aligned.  Errors: those of dp_osdn_precond_ex_*, DP_EINVAL
 * for a NULL dkt, dk_out or dbeta when L > 0, DP_EWORKSPACE, DP_EHIP.
 */
int dp_osdn_precond_bwd_workspace_size(int B, int H, int L, int dk, size_t* bytes);
int dp_osdn_precond_bwd_f32(const float* k, const float* beta, const float* r, const float* d0,
                            const float* dkt, const float* dd_final, int flags, int B, int H, int L,
                            int dk, float eta, float dmin, float dmax, float eps, float* dk_out,
                            float* dbeta, float* dret, float* dd0, void* workspace,
                            size_t workspace_bytes, dp_stream stream);
int dp_osdn_precond_bwd_bf16(const void* k, const float* beta, const float* r, const float* d0,
                             const float* dkt, const float* dd_final, int flags, int B, int H, int L,
                             int dk, float eta, float dmin, float dmax, float eps, float* dk_out,
                             float* dbeta, float* dret, float* dd0, void* workspace,
                             size_t workspace_bytes, dp_stream stream);

/*
 * Gradient of the whole OSDN layer (n_h = 1; OSDN notes sec. 2.5): phase 1
 * over (k, beta) emits the write keys, the write-key forward reads q, the raw
 * keys k, v, beta, g and h0 with them.  One call runs phase 1 again (keeping
 * d_t), the write-key backward, then phase 1's reverse scan; the two routes
 * into k and beta are summed.
 *   q [B,L,H,dk], k [B,L,H,dk], v [B,L,H,dv], dout [B,L,H,dv]   T
 *   beta, r [B,L,H] f32; g [B,L,H] f32 or NULL; h0, dfinal [B,H,dk,dv] f32 or
 *   NULL; d0, dd_final [B,H,dk] f32 or NULL; flags, eta, dmin, dmax, eps as
 *   dp_osdn_precond_ex_*.
 * Outputs (f32, written): dq, dk_out [B,L,H,dk], dv_out [B,L,H,dv], dbeta
 * [B,L,H], dg (when g; may be NULL), dh0, dret, dd0 (each may be NULL).
 * workspace: dp_osdn_bwd_workspace_size() bytes, 256-byte aligned (phase 1's
 * trajectory and write keys, the write-key gradient, the backward's own).
 * Every check runs before anything is enqueued.  Errors: those of dp_bwd_*
 * and dp_osdn_precond_ex_*.
 */
int dp_osdn_bwd_workspace_size(int B, int H, int L, int dk, int dv, size_t* bytes);
int dp_osdn_bwd_f32(const float* q, const float* k, const float* v, const float* beta, const float* g,
                    const float* h0, const float* r, const float* d0, const float* dout,
                    const float* dfinal, const float* dd_final, int flags, int B, int H, int L, int dk,
                    int dv, float eta, float dmin, float dmax, float eps, float* dq, float* dk_out,
                    float* dv_out, float* dbeta, float* dg, float* dh0, float* dret, float* dd0,
                    void* workspace, size_t workspace_bytes, dp_stream stream);
int dp_osdn_bwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* g,
                     const float* h0, const float* r, const float* d0, const void* dout,
                     const float* dfinal, const float* dd_final, int flags, int B, int H, int L, int dk,
                     int dv, float eta, float dmin, float dmax, float eps, float* dq, float* dk_out,
                     float* dv_out, float* dbeta, float* dg, float* dh0, float* dret, float* dd0,
                     void* workspace, size_t workspace_bytes, dp_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* DP_H */
