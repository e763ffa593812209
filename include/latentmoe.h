/*
 * latentmoe.h -- C ABI of the MI355X (gfx950) LatentMoE layer forward.
 *
 * The operation (the pages' three steps, with the readings this library
 * takes where the pages are silent):
 *   z      = W_down x                     x of width d -> latent width l
 *            (qingkeai.online LatentMoE article, section "LatentMoE 具体怎么做",
 *            first bullet; zhichai.net "LatentMoE: How MoE Made a Key Paradigm
 *            Leap in 2026", section 2, step 1)
 *   logit  = W_router x (+ bias)          router at the full width d: the gate
 *            stays at d (same qingkeai.online section, last paragraph;
 *            zhichai.net section 2, last paragraph)
 *   S, g   = top-K of softmax(logit), ties to the lower expert index, kept
 *            probabilities renormalised to sum 1 (gate function: a reading)
 *   s      = sum_k g_k W2[S_k] relu(W1[S_k] z)^2   experts in the latent space,
 *            their weights l x m instead of d x m (qingkeai.online, same
 *            section, second bullet); outputs aggregated in l before the
 *            projection back (10100.com article, section 2.2, Figure 3b)
 *   out    = x + W_up s                   back to width d (third bullet),
 *            plus the residual (a reading)
 * Standard mode (W_down == W_up == NULL, l == d): z = x and out = x + s, the
 * plain MoE of 10100.com Figure 3a, run through the same kernels.
 * Optional shared expert (latentmoe_forward_shared, dims.m_shared > 0): a
 * dense FFN at the full width d beside the routed experts, its output added:
 *   out   += W_shared2 relu(W_shared1 x)^2
 * (the shared expert stays at d: qingkeai.online article, same section, last
 * paragraph; its output is summed with the routed one: 10100.com article,
 * section 3.3).  Its width and activation are readings.
 *
 * Layout: every array is dense and row-major, with the reduction index
 * fastest (the PyTorch nn.Linear [out, in] convention), so both operands of
 * every matrix product are contiguous along the reduction:
 *   x        [T, d]            out      [T, d]
 *   W_down   [l, d]            W_router [N, d]
 *   W1       [N, m, l]  (expert e at W1 + e*m*l)
 *   W2       [N, l, m]  (expert e at W2 + e*l*m)
 *   W_up     [d, l]
 *   W_shared1 [m_shared, d]    W_shared2 [d, m_shared]
 *   router_bias [N] float32, topk_ids [T, K] int32, topk_gates [T, K] float32
 * One element type covers x, the weights and out: float32 or bfloat16.
 * Accumulation is float32; router logits and gates are float32 throughout.
 * Optional FP8 expert weights (bfloat16 layers, dims.expert_format =
 * LMOE_EXPERTS_FP8_E4M3, through latentmoe_forward_ex): W1 and W2 hold one
 * OCP FP8 E4M3 code per element in the same layout, with float32 row scales
 * W1_scale [N, m] (W1[e][j][:] = code * W1_scale[e][j]) and W2_scale [N, l].
 * The pages name low-precision expert weights (NVFP4 / MXFP4) without a
 * format; this per-row FP8 format is a reading.
 * Optional MXFP4 expert weights (bfloat16 layers, dims.expert_format =
 * LMOE_EXPERTS_MXFP4, through latentmoe_forward_ex), the OCP microscaling
 * format the pages name (zhichai.net section 4 and 10100.com section 2):
 * W1 [N, m, l/2] and W2 [N, l, m/2] bytes hold two E2M1 codes each (sign,
 * 2 exponent bits with bias 1, 1 mantissa bit), the even element in the low
 * nibble; W1_scale [N, m, l/32] and W2_scale [N, l, m/32] bytes hold one
 * E8M0 scale (2^(b-127)) per 32 consecutive elements along the reduction
 * index: weight = e2m1(code) * 2^(b-127).  Scale bytes 1 .. 254 are decoded
 * exactly; byte 0 (2^-127) decodes to 0, which changes a product term by at
 * most 6 * 2^-127 (below every nonzero float32 sum it joins); byte 255 (NaN
 * in the format) is not supported and gives undefined results.  The nibble
 * order, the blocks' direction and the scale range are readings.
 * Optional zero-computation experts (through latentmoe_forward_ex; after
 * MoE++, 10100.com article, section 3.2): dims.n_zero zero experts,
 * dims.n_copy copy experts and dims.n_const constant experts take the
 * routed ids N, N+1, ... in that order (Nr = N + n_zero + n_copy + n_const
 * ids in all).  The router scores all Nr ids (W_router [Nr, d], router_bias
 * [Nr]) and softmax, top-K and renormalisation run over all of them.  A
 * selected zero expert adds nothing to s, a copy expert adds g * z (its
 * input), constant expert q adds g * zc_const[q] (zc_const [n_const, l] in
 * the layer's element type).  That they sit among the latent experts (input
 * z, output in l) is a reading: the pages describe them for a plain MoE.
 * topk_ids then range over [0, Nr).
 *
 * Memory: all tensor pointers are DEVICE pointers owned by the caller.  The
 * library allocates nothing in latentmoe_forward, keeps no pointer after it
 * returns, and writes only `out`, `topk_ids`, `topk_gates` and `workspace`.
 * The call enqueues work on `stream` (a hipStream_t; NULL = the default
 * stream) and returns without synchronising: buffers must stay alive until
 * the stream has finished.  It never synchronises the host and so can be
 * captured into a HIP graph.
 *
 * Errors: arguments are checked before anything is enqueued; on a check
 * failure nothing is written and a negative lmoe_status is returned.
 * latentmoe_last_error() gives a thread-local text for the last failure.
 */
#ifndef LATENTMOE_H
#define LATENTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LMOE_OK = 0,
    LMOE_EINVAL = -1,        /* a NULL pointer, a bad size or a bad combination */
    LMOE_EUNSUPPORTED = -2,  /* legal arguments outside what the kernels cover */
    LMOE_EWORKSPACE = -3,    /* workspace NULL or smaller than latentmoe_workspace_bytes */
    LMOE_EHIP = -4           /* a HIP launch failed; see latentmoe_last_error() */
} lmoe_status;

typedef enum { LMOE_F32 = 0, LMOE_BF16 = 1 } lmoe_dtype;

/* Which kernel family runs the expert FFN (bf16 only; float32 always uses
 * the float32 kernels).  AUTO picks STREAM when the mean number of rows per
 * expert, T*K/N, is at most 16, else TILED.  STREAM streams each active
 * expert's weights once per 16 routed rows (decode shapes); TILED runs
 * LDS-tiled grouped GEMMs (prefill shapes).  Both give results within the
 * same tolerance of the exact layer. */
typedef enum { LMOE_PATH_AUTO = 0, LMOE_PATH_STREAM = 1, LMOE_PATH_TILED = 2 } lmoe_path;

/* Storage of the routed experts' W1 / W2. */
typedef enum { LMOE_EXPERTS_DENSE = 0, LMOE_EXPERTS_FP8_E4M3 = 1, LMOE_EXPERTS_MXFP4 = 2 } lmoe_expert_format;

typedef struct {
    int32_t T;      /* tokens, >= 1 */
    int32_t d;      /* model width, multiple of 64 */
    int32_t l;      /* latent width, multiple of 64; == d in standard mode */
    int32_t N;      /* FFN experts, 1 .. 2048 */
    int32_t m;      /* expert hidden width, multiple of 64 */
    int32_t dtype;  /* lmoe_dtype */
    int32_t path;   /* lmoe_path */
    int32_t m_shared; /* shared expert width: 0 (none) or a multiple of 64 */
    int32_t expert_format; /* lmoe_expert_format */
    int32_t n_zero;  /* zero-computation experts: zero, copy, constant (>= 0, */
    int32_t n_copy;  /* N + n_zero + n_copy + n_const <= 2048); all 0 except */
    int32_t n_const; /* through latentmoe_forward_ex */
} lmoe_dims;

/* Bytes of device workspace latentmoe_forward needs for these dims and K
 * (0 when the arguments are invalid).  The size depends on the resolved path. */
size_t latentmoe_workspace_bytes(const lmoe_dims* dims, int32_t K);

/*
 * The layer forward.  K: experts per token, 1 <= K <= min(N, 64).
 * router_bias: NULL or [N] float32 added to the logits before the softmax
 * (it changes both the selection and the gates).
 * topk_ids / topk_gates: NULL, or caller buffers that receive the selected
 * experts in rank order (largest logit first) and their gates.
 * The buffers the call writes -- out, topk_ids, topk_gates and the
 * workspace -- must not overlap one another or any array it reads (x, the
 * weights, their scales, zc_const, router_bias): LMOE_EINVAL otherwise, from
 * the byte ranges the dims give.  dims->m_shared must be 0 (the shared
 * expert goes through latentmoe_forward_shared) and dims->expert_format
 * LMOE_EXPERTS_DENSE (FP8 experts go through latentmoe_forward_ex).
 */
int latentmoe_forward(const void* x, const void* W_down, const void* W_router,
                      const void* W1, const void* W2, const void* W_up, int32_t K,
                      void* out, const lmoe_dims* dims, const float* router_bias,
                      int32_t* topk_ids, float* topk_gates,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The layer forward with a shared expert: latentmoe_forward plus
 * out += W_shared2 relu(W_shared1 x)^2, W_shared1 [m_shared, d] and
 * W_shared2 [d, m_shared] in the element type of x, dims->m_shared > 0 (a
 * multiple of 64).  The shared expert's output is added to the layer's before
 * the single rounding of out.  Same memory, stream and error rules.
 */
int latentmoe_forward_shared(const void* x, const void* W_down, const void* W_router,
                             const void* W1, const void* W2, const void* W_up,
                             const void* W_shared1, const void* W_shared2, int32_t K,
                             void* out, const lmoe_dims* dims, const float* router_bias,
                             int32_t* topk_ids, float* topk_gates,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * latentmoe_forward_shared with stage timing, for benchmarks and profilers
 * (W_shared1 = W_shared2 = NULL and dims->m_shared = 0: latentmoe_forward).
 * events: an array of LMOE_N_STAGE_EVENTS hipEvent_t handles created by
 * the caller; NULL entries are skipped.  Event i is recorded on `stream` at
 * the start of stage i, the last one after the final stage.  Stages:
 * 0 projection + router logits (and the shared expert's two products),
 * 1 top-K gates, 2 dispatch, 3 expert FFN first kernel (the whole FFN on the
 * streaming path), 4 expert FFN second kernel (empty on the streaming path),
 * 5 combine, 6 projection back to d (empty in standard mode).  On the
 * streaming path, when events 3 and 4 are both given and the stream is not
 * being captured, they are the FFN kernel's own start and end (recorded
 * with its launch by hipExtLaunchKernel) instead of event packets around
 * it.  The computation is the same as the untimed call's.
 */
#define LMOE_N_STAGE_EVENTS 8
int latentmoe_forward_timed(const void* x, const void* W_down, const void* W_router,
                            const void* W1, const void* W2, const void* W_up,
                            const void* W_shared1, const void* W_shared2, int32_t K,
                            void* out, const lmoe_dims* dims, const float* router_bias,
                            int32_t* topk_ids, float* topk_gates,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events);

/*
 * The general entry point: every option of the layer in one argument block.
 * Pointers as in latentmoe_forward; W_shared1 / W_shared2 with
 * dims->m_shared > 0 (else NULL); W1_scale / W2_scale with FP8 or MXFP4
 * experts (else NULL; FP8 float32 scales 16-byte aligned, MXFP4 scale
 * bytes 8-byte aligned); zc_const [n_const, l] with dims->n_const > 0 (else
 * NULL; 16-byte aligned); events NULL or as in latentmoe_forward_timed.  The other
 * forward entry points are this call with the options they do not name
 * turned off.
 */
typedef struct {
    const void* x;
    const void* W_down;
    const void* W_router;
    const void* W1;
    const void* W2;
    const void* W_up;
    const void* W_shared1;
    const void* W_shared2;
    const void* W1_scale;   /* FP8: float32 row scales; MXFP4: E8M0 block scale bytes */
    const void* W2_scale;
    const void* zc_const;
    const float* router_bias;
    void* out;
    int32_t* topk_ids;
    float* topk_gates;
    void* workspace;
    size_t workspace_bytes;
    void* stream;
    void* const* events;
} lmoe_args;

int latentmoe_forward_ex(const lmoe_args* args, int32_t K, const lmoe_dims* dims);

/*
 * latentmoe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a static
 * device array of the library, LMOE_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * device, created when the library's code is loaded on a device and held
 * until the process ends; the call allocates nothing.  Dims whose
 * latentmoe_workspace_bytes() exceeds that size are rejected with
 * LMOE_EUNSUPPORTED (at d = 4096, l = 1024, 512 experts, top-22 that is
 * T > 600).  Every call on one device uses the same array and leaves the
 * last call's routing data in it: calls that may overlap on one device --
 * on two streams, or from two threads -- race and must be serialised by
 * the caller.  Arguments, results, errors and the stream rules are those of
 * latentmoe_forward; the first call on a device also looks up the array's
 * address (hipGetSymbolAddress), whose failure returns LMOE_EHIP.
 */
#define LMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int latentmoe_forward_noalloc(const void* x, const void* W_down, const void* W_router,
                              const void* W1, const void* W2, const void* W_up, int32_t K,
                              void* out, const lmoe_dims* dims, const float* router_bias,
                              int32_t* topk_ids, float* topk_gates, void* stream);

/* Static text for a status code. */
const char* latentmoe_status_string(int status);

/* Thread-local detail of the last failure in this thread ("" if none). */
const char* latentmoe_last_error(void);

/* The path latentmoe_forward resolves for these dims and K
 * (LMOE_PATH_STREAM or LMOE_PATH_TILED), or a negative status. */
int latentmoe_resolved_path(const lmoe_dims* dims, int32_t K);

/*
 * Where the dispatch arrays live inside the workspace after a forward (byte
 * offsets from the workspace base), so that callers and tests can inspect the
 * token -> expert permutation.  `written` is 1 when a forward with these dims
 * writes them, 0 when it does not: the streaming path with T <= 256 has no
 * dispatch (each expert's workgroups find its rows from the top-K ids), and
 * the arrays then hold whatever was there before.  The arrays:
 *   counts   [Nr]     int32  rows routed to each id (Nr = N without
 *                            zero-computation experts)
 *   offsets  [Nr + 1] int32  exclusive prefix sum of counts
 *   perm     [T*K]    int32  slot -> flat pair index t*K + k; the slots of one
 *                            expert are contiguous and in increasing pair order
 *   slot_of  [T*K]    int32  flat pair index -> slot (the inverse of perm)
 *   n_active [1]      int32  FFN experts (ids < N) with at least one row
 */
typedef struct {
    size_t counts, offsets, perm, slot_of, n_active;
    size_t written;
} lmoe_ws_layout;

int latentmoe_workspace_layout(const lmoe_dims* dims, int32_t K, lmoe_ws_layout* layout);

#ifdef __cplusplus
}
#endif

#endif /* LATENTMOE_H */
