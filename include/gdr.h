/*
 * gdr.h -- C ABI of the gated delta-rule linear-attention forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  Per batch row b and head h, a fast-weight state
 * S in R^{dk x dv} (rows = key channels, columns = value channels; "Kaczmarz
 * Linear Attention", Implementation section, which keeps the state shape
 * S in R^{d_k x d_v}) is carried along the sequence.  Token t first decays the
 * state, S~ = D_t S_{t-1}, then reads it along an erase key a_t and writes the
 * residual along k_t, and the output reads the updated state:
 *
 *     S_t = (I - k_t a_t^T) D_t S_{t-1} + k_t u_t^T,       o_t = S_t^T q_t.
 *
 * Equivalently delta_t = u_t - S~^T a_t and S_t = S~ + k_t delta_t^T, which is
 * the KLA update of "Kaczmarz Linear Attention" (KLA update rule: residual
 * e_t = v_t - S~_{t-1}^T k_t, step S_t = S~_{t-1} + beta_t k_t e_t^T).
 * The variants differ only in D_t, a_t and u_t:
 *
 *   GDR_DELTANET        D = I            a = beta k     u = beta v
 *   GDR_GATED_DELTANET  D = alpha I      a = beta k     u = beta v
 *   GDR_KDA             D = Diag(alpha)  a = beta k     u = beta v
 *   GDR_GDN2            D = Diag(alpha)  a = b (.) k    u = w (.) v
 *   GDR_KLA             D = alpha I      a = beta k     u = beta v,
 *                       beta = eta / (||k||^2 + eps)
 *
 * ("Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
 * Routing": DeltaNet writes the difference, Gated DeltaNet adds a scalar forget
 * gate, Kimi Delta Attention makes the forget gate channel-wise, Gated
 * DeltaNet-2 separates erase and write; "Gated DeltaNet-2: Decoupling Erase and
 * Write in Linear Attention", novelty section: a channel-wise erase gate b_t on
 * the key side and a channel-wise write gate w_t on the value side, reducing to
 * KDA when both collapse to one scalar; "Kaczmarz Linear Attention", KLA update
 * rule: the key-norm-normalised step size.)  Channel-wise decay acts on the key
 * rows of S.
 *
 * Two entry points compute it (a third, gdr_backward_chunked below, computes
 * its gradient): a chunkwise-parallel prefill over a whole
 * sequence ("Kaczmarz Linear Attention", Implementation section: the
 * chunk-wise parallel algorithm is kept and only the per-chunk diagonal
 * coefficient matrix Diag(beta_1..beta_C) changes; "Gated DeltaNet-2", technical
 * core: a chunkwise WY algorithm with the decay folded into the erase factor)
 * and a single-token recurrent decode step ("Gated DeltaNet-2", introduction:
 * a fixed-size recurrent state gives linear-time mixing and constant decode
 * memory).
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is device memory owned by the caller.  The library
 *     never allocates device memory, frees or synchronises; work is enqueued on
 *     the HIP stream passed as `hip_stream` (a hipStream_t; NULL = the null
 *     stream), and only there: a long bf16 prefill (512 chunks or more; 256
 *     for KDA and GDN-2, and for the others when B * H * dv / 16 is above a
 *     quarter and at most half of the device's compute units) is pipelined
 *     in blocks of 64 chunks by launches that each run one block's scan
 *     beside the next block's prep, in order on `hip_stream`.  A bf16 prefill
 *     of 64 chunks or more whose B * H * dv / 16 column slices are at most a
 *     quarter of the compute units runs as 2 to 16 segments whose chains run
 *     side by side (each segment's transition and local end state, a serial
 *     combine, then each segment's outputs), the state map of a chunk being
 *     affine ("Kaczmarz Linear Attention", Implementation: the chunk-wise
 *     parallel algorithm), when its workspace fits in 1 GiB; the gradient's
 *     forward pass and its reverse pass (whose map is affine too) then run in
 *     the same segments.  Every call can be captured into a HIP graph.
 *   - Layouts are dense row-major:
 *       q, k     [B, T, H, dk]        v, o      [B, T, H, dv]
 *       alpha    GATED_DELTANET, KLA: [B, T, H];  KDA, GDN2: [B, T, H, dk];
 *                DELTANET: must be NULL.  Linear decay in (0, 1].  A scalar
 *                decay is applied exactly everywhere.  A channel-wise decay
 *                (KDA, GDN2) below e^-10 (about 4.5e-5; with
 *                GDR_FLAG_RAW_GATES, decay_scale * softplus(x) above 10) is
 *                applied as e^-10 by the chunked forward and its gradient: the
 *                chunk form splits the decay between two matrix-core operands,
 *                and this floor keeps both factors inside the float range.  At
 *                most 4.5e-5 of that channel's state then passes the token
 *                where less should; decays at or above e^-10 are exact.  The
 *                decode step applies every decay as given.
 *       beta     DELTANET, GATED_DELTANET, KDA: beta [B, T, H];
 *                KLA: eta [B, T, H];  GDN2: must be NULL.
 *       erase_b  GDN2: [B, T, H, dk], else NULL.
 *       write_w  GDN2: [B, T, H, dv], else NULL.
 *       state_in, state_out  [B, H, dk, dv] float32.
 *     q, k, v and o share one element type (`dtype`); gates and state are
 *     float32.  Every pointer must be 16-byte aligned.
 *   - Arguments are validated before any HIP call; a rejected call enqueues
 *     nothing.  Gate values are device data and are not checked: NaN or Inf
 *     propagate.  Launch failures return GDR_ERR_HIP; faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - The functions may be called from several host threads at once.  Calls
 *     keep no data of their own between them; the library keeps, per device,
 *     its compute-unit count and the resident-workgroup counts of its kernels
 *     (queried once; the workspace size of a call depends on the current
 *     device's unit count), never released.  A thread-local message explains
 *     the last failure.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARGUMENT = 1, /* null/extra pointer, bad size, misalignment */
    GDR_ERR_UNSUPPORTED = 2,      /* valid request this build does not implement */
    GDR_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    GDR_ERR_HIP = 4               /* a HIP launch or query failed */
} gdr_status;

typedef enum {
    GDR_DELTANET = 0,
    GDR_GATED_DELTANET = 1,
    GDR_KDA = 2,
    GDR_GDN2 = 3,
    GDR_KLA = 4
} gdr_variant;

typedef enum {
    GDR_F32 = 0, /* q, k, v, o in float32 */
    GDR_BF16 = 1 /* q, k, v, o in bfloat16; products on bf16 matrix cores, fp32 accumulation */
} gdr_dtype;

/* Input transforms the kernels apply as they load the inputs (gdr_args.flags),
 * so that a caller holding raw projections needs no separate pass over them.
 * The recurrence then runs on the transformed values exactly as on stored ones;
 * stored bf16 inputs are transformed in fp32 from their stored values.  ("Kaczmarz
 * Linear Attention", ablations: key normalisation and the gating are what keep
 * the delta rule stable; the transforms below are the usual parameterisation of
 * the gates and keys of this family.) */
typedef enum {
    /* q <- q / sqrt(sum_i q_i^2 + 1e-6) and the same for k, over the dk
     * channels of each (b, t, h). */
    GDR_FLAG_QK_L2NORM = 1,
    /* alpha <- exp(-decay_scale * softplus(alpha)), softplus(x) = log(1 + e^x),
     * elementwise (scalar or per channel); beta (eta for KLA), erase_b and
     * write_w <- sigmoid(x) = 1 / (1 + e^-x). */
    GDR_FLAG_RAW_GATES = 2
} gdr_flag;

typedef struct gdr_args {
    int32_t variant;   /* gdr_variant */
    int32_t dtype;     /* gdr_dtype */
    int64_t B, T, H;   /* batch rows, tokens, heads; all >= 1; B, H <= 65535, B * H <= 2^24
                          and T <= 2^31, else GDR_ERR_UNSUPPORTED */
    int64_t dk, dv;    /* key and value head sizes: 64 or 128 each */
    int32_t chunk;     /* chunk length of the prefill; 0 = default (64); decode ignores it */
    int32_t flags;     /* bitwise OR of gdr_flag; 0 = inputs used as stored */
    const void *q, *k, *v;
    const float *alpha;
    const float *beta;
    const float *erase_b;
    const float *write_w;
    float eps;         /* KLA stabiliser added to ||k||^2; ignored otherwise */
    float decay_scale; /* with GDR_FLAG_RAW_GATES and a decaying variant: the scale s
                          of exp(-s * softplus(alpha)), finite and > 0; else 0 */
    const float *state_in; /* NULL = zero initial state */
    float *state_out;      /* NULL = final state not written; may equal state_in */
    void *o;               /* required */
    /* Cross-layer routing ("Linear Attention Architectures: Mechanisms,
     * Trade-offs, and Cross-Layer Routing", the cross-layer routing section: a
     * lower layer hands a higher layer either its value target, CLVR, or its
     * error, CLER). */
    const void *v_route;   /* optional [B, T, H, dv] in `dtype`: a value routed in
                              from another layer; the kernels use v + v_route as
                              the value as they load it.  NULL = none */
    void *delta_out;       /* optional output [B, T, H, dv] in `dtype`: the residual
                              delta_t each token writes, S_t = S~_t + k_t delta_t^T
                              (beta_t (v_t - S~_t^T k_t) for the beta variants).
                              NULL = not written */
} gdr_args;

/* Validate `a` for gdr_forward_chunked (for_decode = 0) or gdr_decode_step
 * (for_decode = 1) without touching the GPU.  Returns GDR_OK or the error the
 * entry point would return (GDR_ERR_WORKSPACE is never returned here). */
gdr_status gdr_check_args(const gdr_args *a, int for_decode);

/* Bytes of device workspace gdr_forward_chunked needs for `a` (0 if `a` is
 * invalid).  The workspace holds per-chunk intermediate factors; its content
 * is undefined before and after a call. */
size_t gdr_forward_workspace_size(const gdr_args *a);

/* Chunkwise-parallel forward over T tokens for every (b, h): writes o and,
 * if state_out != NULL, the final state.  state_out may alias state_in; no
 * other output may overlap an input.  `workspace` must be 256-byte aligned and
 * at least gdr_forward_workspace_size(a) bytes.  It holds the per-chunk
 * factors: of every chunk for sequences shorter than 512 chunks of 64 tokens
 * (256 in the cases above; at most 1 GiB; 72.5 KB per chunk and head at
 * dk = dv = 128 in bf16), and for a segmented prefill, with each segment
 * boundary's transition, local end state and start state (fp32, dk x dk and
 * twice dk x dv per head);
 * else of two blocks of 64 chunks plus a state carrier and a work counter, so
 * it stops growing with T.  Calls that share a workspace must be ordered on
 * one stream. */
gdr_status gdr_forward_chunked(const gdr_args *a, void *workspace, size_t ws_bytes,
                               void *hip_stream);

/* gdr_forward_chunked for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with the
 * workspace taken from a static device array of GDR_NOALLOC_WORKSPACE_MAX bytes
 * that the library holds on every device it runs on until the process ends.
 * The call allocates and frees nothing; its first call with a device current
 * looks up that device's array.  Like gdr_forward_chunked it enqueues its
 * kernels on `hip_stream` only and creates no stream or event.
 * A segmented prefill (see above) whose workspace would exceed
 * GDR_NOALLOC_WORKSPACE_MAX runs here pipelined or in one pass instead, so
 * its results then agree with gdr_forward_chunked's to the forward's
 * tolerance rather than bit for bit.
 * Returns GDR_ERR_WORKSPACE, enqueuing nothing, when the plan it takes needs
 * more than GDR_NOALLOC_WORKSPACE_MAX (for a prefill that gdr_forward_chunked
 * does not segment: when gdr_forward_workspace_size(a) exceeds it).  All calls
 * on one device share its array: calls that may overlap on a device (other
 * streams, other threads) race and must be ordered by the caller. */
#define GDR_NOALLOC_WORKSPACE_MAX ((size_t)256 << 20)
gdr_status gdr_forward_chunked_noalloc(const gdr_args *a, void *hip_stream);

/* One recurrent decode step (requires T == 1) for every (b, h): reads
 * state_in (required), writes o and state_out (required; may equal state_in
 * for an in-place update). */
gdr_status gdr_decode_step(const gdr_args *a, void *hip_stream);

/* ---- gradient of the chunked forward ----------------------------------------
 *
 * Given upstream gradients dO = dL/do and dS_T = dL/dS_T of a loss L, the
 * gradient of L with respect to every input of gdr_forward_chunked.  It is the
 * chain rule through the chunk form the prefill computes (the WY / UT
 * representation of "Gated DeltaNet-2", technical core, and the chunk-wise
 * algorithm of "Kaczmarz Linear Attention", Implementation section): a reverse
 * pass over the chunks carries dL/dS backwards, and every chunk then
 * back-propagates through its triangular solve and Gram products
 * independently.  The forward's per-chunk factors and states are recomputed;
 * nothing from an earlier forward call is needed.
 */
typedef struct gdr_grads {
    const void *d_o;          /* [B, T, H, dv] in the args' dtype; NULL = zero */
    const float *d_state_out; /* [B, H, dk, dv]; NULL = zero */
    /* Outputs, float32, dense row-major, shaped like the inputs they belong
     * to.  Each is required exactly when the variant takes that input. */
    float *d_q, *d_k;         /* [B, T, H, dk] */
    float *d_v;               /* [B, T, H, dv] */
    float *d_alpha;           /* shaped like alpha: gradient w.r.t. the linear decay,
                                 formed as (dL/d log alpha) / alpha, so its
                                 absolute error grows like 1/alpha for small
                                 decays; for a channel-wise decay below e^-10
                                 it is taken at e^-10 (see alpha above) */
    float *d_beta;            /* shaped like beta (w.r.t. eta for KLA) */
    float *d_erase_b;         /* GDN2 [B, T, H, dk] */
    float *d_write_w;         /* GDN2 [B, T, H, dv] */
    float *d_state_in;        /* [B, H, dk, dv]; NULL = not written.  Written also
                                 when state_in is NULL (zero initial state). */
} gdr_grads;

/* Bytes of device workspace gdr_backward_chunked needs for `a` (0 if `a` is
 * not valid for it).  It grows linearly with B * H * T: the per-chunk factors,
 * the fp32 state entering every chunk and its gradient, plus a fixed scratch
 * area for the per-chunk gradient workers. */
size_t gdr_backward_workspace_size(const gdr_args *a);

/* Gradient of gdr_forward_chunked's outputs o and state_out with respect to
 * q, k, v, the gates and state_in.  `a` describes the forward call (o and
 * state_out are ignored and may be NULL); a->flags must be 0 (input transforms
 * are not differentiated: GDR_ERR_UNSUPPORTED).  Outputs must not overlap the
 * inputs or each other.  `workspace` must be 256-byte aligned and hold at
 * least gdr_backward_workspace_size(a) bytes. */
gdr_status gdr_backward_chunked(const gdr_args *a, const gdr_grads *g, void *workspace,
                                size_t ws_bytes, void *hip_stream);

/* The forward of a training step that keeps what its gradient needs.  It
 * writes o and state_out exactly as gdr_forward_chunked does (over all
 * chunks in one pass, or in the same segments as gdr_forward_chunked where
 * that call runs in segments), and leaves in
 * `workspace` (256-byte aligned, at least
 * gdr_backward_workspace_size(a) bytes, owned by the caller) every chunk's
 * factors of the chunk form and the state and residual entering each chunk:
 * the first pass gdr_backward_chunked would otherwise recompute.  Besides the
 * forward's checks, `a` must be valid for the gradient (flags 0, v_route
 * NULL: GDR_ERR_UNSUPPORTED), and delta_out must be NULL
 * (GDR_ERR_UNSUPPORTED). */
gdr_status gdr_forward_chunked_save(const gdr_args *a, void *workspace, size_t ws_bytes,
                                    void *hip_stream);

/* gdr_backward_chunked without its first pass: it reads the records that
 * gdr_forward_chunked_save left in `workspace`.  The caller passes the same
 * `a` (the same inputs, unchanged since) and the same workspace, untouched in
 * between and ordered after that call (same stream, or synchronised); the
 * library cannot check this, and results are undefined otherwise.  Results
 * equal gdr_backward_chunked's, bit for bit except where that call sums per
 * token with atomic additions of varying order (d_alpha, d_beta, and d_k for
 * KLA), which differ in their last bits from one call to the next either way.
 * Same arguments and errors as gdr_backward_chunked; the workspace is
 * overwritten past the kept records. */
gdr_status gdr_backward_chunked_saved(const gdr_args *a, const gdr_grads *g, void *workspace,
                                      size_t ws_bytes, void *hip_stream);

/* Static description of a status code. */
const char *gdr_status_string(int status);

/* Thread-local detail of the last non-OK status returned on this thread
 * (empty string if none). */
const char *gdr_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
