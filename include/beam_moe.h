/*
 * beam_moe.h -- C ABI of a single-GPU Beam mixture-of-experts layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (Glonce, "Reflection releases Beam, a 501B open MoE model with 1M
 * context", architecture paragraphs; transformers v5.20.1 model doc "Beam",
 * Overview, bullet "Sparse MoE"):
 *   - router: logits l = u W_r^T, sigmoid scores s = sigmoid(l), biased scores
 *     s' = s + b (the per-expert bias only selects), experts split into n_group
 *     contiguous groups, a group scores the sum of its two largest s', the best
 *     topk_group groups are kept and the top_k largest s' inside them chosen;
 *     weights w = routed_scaling * s / sum(s) over the chosen;
 *   - experts: SwiGLU MLPs  z = W_d (silu(W_g u) * (W_u u)), no shared expert;
 *   - output y = sum_j w_j z_j.
 * Routing, the SwiGLU activation and RMSNorm scaling are computed in FP32
 * (same model doc, Overview, numerics paragraph).  Optional sublayer wrapping
 * (Glonce, residual paragraph; model doc, "Sandwich norms with depth-scaled
 * residuals"): u = RMSNorm_pre(x); out = sqrt((k-1)/k) x + RMSNorm_post(y)/sqrt(k).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are caller-owned DEVICE memory, row-major, contiguous,
 *     16-byte aligned.  The library allocates nothing and keeps no state between
 *     calls; scratch memory comes in through `ws` (size from
 *     beam_moe_workspace_size).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work and return; they never synchronise the device.  Results are valid when
 *     the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and outputs are untouched.
 *   - Results are deterministic: a call with the same inputs gives bitwise the
 *     same outputs.
 *   - Concurrent calls must not share a workspace.
 *   - T = 0 is a valid no-op (no workspace needed; beam_moe_permute then only
 *     zeroes `offsets`).
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BEAM_MOE_ABI_VERSION 1

typedef enum beam_status {
    BEAM_OK = 0,
    BEAM_ERR_INVALID_ARG = 1, /* NULL required pointer, inconsistent or out-of-range shape */
    BEAM_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype, alignment of H/I) */
    BEAM_ERR_WORKSPACE = 3,   /* ws NULL or smaller than beam_moe_workspace_size */
    BEAM_ERR_HIP = 4          /* a HIP launch failed (hipGetLastError) */
} beam_status;

/* element type of activations (x, u, out, moe_y) and expert weights */
typedef enum beam_dtype { BEAM_F32 = 0, BEAM_BF16 = 1 } beam_dtype;

/*
 * Layer shape.  Limits: T >= 0, T * top_k < 2^31; 1 <= E <= 1024;
 * E % n_group == 0; E / n_group <= 1024; 1 <= n_group <= 64;
 * 1 <= topk_group <= n_group; 1 <= top_k <= min(32, topk_group * E / n_group);
 * H, I >= 1.  With BEAM_BF16, beam_moe_forward needs H % 256 == 0 and
 * I % 128 == 0, and beam_moe_route needs H % 128 == 0 (else BEAM_ERR_UNSUPPORTED).
 * Beam: H = 5120, E = 256, I = 2560, n_group = 8, topk_group = 4, top_k = 8,
 * routed_scaling = 2.5.
 */
typedef struct beam_moe_shape {
    int64_t T;            /* tokens */
    int32_t H;            /* hidden size */
    int32_t E;            /* routed experts */
    int32_t I;            /* expert intermediate size */
    int32_t n_group;      /* expert groups (contiguous index ranges of E / n_group) */
    int32_t topk_group;   /* groups kept per token */
    int32_t top_k;        /* experts chosen per token */
    float routed_scaling; /* multiplies the normalised routing weights */
    int32_t dtype;        /* beam_dtype of activations and expert weights */
} beam_moe_shape;

/*
 * Sandwich norm + depth-scaled residual around the MoE block (bf16 only).
 * pre_gain, post_gain: [H] fp32 device arrays.  eps > 0.  residual_k >= 1 is the
 * index of this addition when the embedding counts as contribution 1.
 */
typedef struct beam_sublayer {
    const float* pre_gain;
    const float* post_gain;
    float eps;
    float residual_k;
} beam_sublayer;

/* what a workspace is for */
typedef enum beam_op {
    BEAM_OP_ROUTE = 0,            /* beam_moe_route */
    BEAM_OP_PERMUTE = 1,          /* beam_moe_permute */
    BEAM_OP_FORWARD = 2,          /* beam_moe_forward without sublayer */
    BEAM_OP_FORWARD_SUBLAYER = 3  /* beam_moe_forward with sublayer */
} beam_op;

/* stage boundaries recorded by beam_moe_forward when stage events are given */
#define BEAM_STAGE_PRENORM 0
#define BEAM_STAGE_ROUTER_LOGITS 1
#define BEAM_STAGE_ROUTER_SELECT 2
#define BEAM_STAGE_PERMUTE 3
#define BEAM_STAGE_GATE_UP 4
#define BEAM_STAGE_DOWN 5
#define BEAM_STAGE_COMBINE 6
#define BEAM_NUM_STAGES 7

/*
 * Bytes of workspace `op` needs for `shape` (written to *bytes).
 * Errors: BEAM_ERR_INVALID_ARG for a NULL pointer, an invalid shape or op.
 * At the Beam shape the forward workspace is about P*(2I + 2H) + T*E*4 bytes
 * (P = T*top_k), e.g. ~1.1 GB at T = 8192 and ~4.4 GB at T = 32768 with sublayer.
 */
beam_status beam_moe_workspace_size(const beam_moe_shape* shape, int32_t op, size_t* bytes);

/*
 * Pre-RMSNorm (the "norm before" of the sandwich; model doc "Sandwich norms with
 * depth-scaled residuals"; FP32 RMSNorm scaling, Overview numerics paragraph):
 *   r_t = fp32(1 / sqrt(mean_h x[t,h]^2 + eps))   (mean square accumulated in fp64,
 *                                                   r rounded once to fp32)
 *   u[t,h] = bf16_rne(fp32(fp32(x[t,h] * r_t) * gain[h]))
 * x, u: [T,H] bf16, 16-byte aligned (u may not alias x); gain [H] fp32.
 * shape->dtype must be BEAM_BF16 and H % 8 == 0 (else BEAM_ERR_UNSUPPORTED); only T
 * and H are read.  Bitwise reproducible given x, gain, eps.
 */
beam_status beam_moe_rmsnorm(const beam_moe_shape* shape, const void* x, const float* gain, float eps, void* u,
                             void* stream);

/*
 * Router (Glonce architecture paragraph; model doc "Sparse MoE"; FP32 routing).
 *   x        [T,H] activations (shape->dtype)
 *   w_router [E,H] fp32;  bias [E] fp32 (selection only)
 *   topk_idx [T,top_k] int32 out: chosen experts, descending s', ties -> lower id
 *   topk_w   [T,top_k] fp32 out: routed_scaling * s / sum(s) of the chosen
 *   logits_out [T,E] fp32 out, optional (the router logits before the sigmoid)
 *   ws       scratch of beam_moe_workspace_size(BEAM_OP_ROUTE) bytes (fp64 partial
 *            logits; several H ranges are reduced by different work-groups when T
 *            is small)
 * Logits are accumulated from exact bf16 x bf16 partial products: each 32-term
 * block is summed on the matrix cores in fp32, the blocks and H ranges are summed in
 * fp64 in a fixed order, and the logit is rounded once to fp32; s, s', group scores
 * and all comparisons are fp32.
 */
beam_status beam_moe_route(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                           int32_t* topk_idx, float* topk_w, float* logits_out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Token permutation: a stable counting sort of the P = T*top_k (token, choice)
 * pairs by expert.  Pair p = t*top_k + j has expert topk_idx[p].
 *   offsets      [E+1] int32 out: offsets[e] = number of pairs with expert < e
 *   sorted_pairs [P] int32 out: pair ids in expert order, ascending p within an expert
 *   pair_pos     [P] int32 out: pair_pos[p] = position of p in sorted_pairs
 *   ws           scratch of beam_moe_workspace_size(BEAM_OP_PERMUTE) bytes
 * Entries of topk_idx outside [0,E) are skipped: they get no row, their pair_pos
 * entry is not written and offsets[E] counts only the valid pairs (the router never
 * writes such entries).
 */
beam_status beam_moe_permute(const beam_moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                             int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream);

/*
 * Whole layer: [pre-norm] -> router -> permutation -> grouped gate/up GEMM with the
 * SwiGLU epilogue -> grouped down GEMM -> weighted combine [-> post-norm + residual].
 *   x        [T,H] (shape->dtype);  w_router [E,H] fp32;  bias [E] fp32
 *   w_gate, w_up [E,I,H] and w_down [E,H,I] (shape->dtype): row = output feature
 *   sub      optional sublayer (bf16 only); NULL: out = y
 *   out      [T,H] (shape->dtype) out
 *   topk_idx, topk_w  optional [T,top_k] outputs of the routing (as beam_moe_route)
 *   moe_y    optional [T,H] (shape->dtype) out: y before the post-norm (sublayer only)
 *   ws       scratch of beam_moe_workspace_size(BEAM_OP_FORWARD[_SUBLAYER]) bytes
 *   stage_events optional array of BEAM_NUM_STAGES + 1 hipEvent_t created by the
 *            caller; event i is recorded on `stream` where stage i starts and event
 *            BEAM_NUM_STAGES at the end (skipped stages are empty intervals).
 * Precision (bf16): gate/up and down products accumulate in fp32 (MFMA); the SwiGLU
 * activation is fp32; the intermediate h and the per-pair expert outputs are rounded
 * to bf16; the combine, post-norm and residual run in fp32.
 */
beam_status beam_moe_forward(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                             const void* w_gate, const void* w_up, const void* w_down, const beam_sublayer* sub,
                             void* out, int32_t* topk_idx, float* topk_w, void* moe_y, void* ws, size_t ws_bytes,
                             void* const* stage_events, void* stream);

/*
 * beam_moe_forward with 8-bit expert weights (bf16 activations; shape->dtype must be
 * BEAM_BF16, else BEAM_ERR_UNSUPPORTED).  Each weight is stored as an OCP FP8 E4M3 code
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; S.1111.111 is NaN; largest finite 448) and every 32 consecutive
 * elements of a row along the reduction dimension share one E8M0 scale byte s, meaning
 * 2^(s - 127); the weight is e4m3(code) * 2^(s - 127).
 *   w_gate, w_up [E,I,H] and w_down [E,H,I]: E4M3 codes, one byte each, the layout of the
 *            bf16 weights of beam_moe_forward (16-byte aligned)
 *   s_gate, s_up [E,I,H/32] and s_down [E,H,I/32]: E8M0 scale bytes (16-byte aligned):
 *            2^(s - 127) for s = 0 .. 254 (s = 0 is 2^-127) and NaN for s = 255, as the
 *            E8M0 format defines them
 * Every other argument, the workspace and the results are as for beam_moe_forward.  A
 * weight whose decoded value is a normal bf16 number (or zero) is decoded exactly (an E4M3
 * value times a power of two is then a bf16 value) and the layer computes exactly what
 * beam_moe_forward computes on the decoded weights; only the weight bytes read from memory
 * halve.  Decoded values beyond that range are rounded to bf16 (to nearest, ties to even:
 * below 2^-126 to a subnormal or zero, above the largest bf16 to infinity); a NaN code or a
 * NaN scale makes the outputs of the tokens routed to that expert NaN.  This storage format is
 * not on the Beam pages (they quote FP8 checkpoints without a scale scheme); it is the
 * block-scaled layout of the OCP microscaling formats with 32-element blocks.
 */
beam_status beam_moe_forward_fp8(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                                 const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                                 const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down,
                                 const beam_sublayer* sub, void* out, int32_t* topk_idx, float* topk_w, void* moe_y,
                                 void* ws, size_t ws_bytes, void* const* stage_events, void* stream);

/*
 * beam_moe_forward with 4-bit expert weights (MXFP4; bf16 activations; shape->dtype must
 * be BEAM_BF16, else BEAM_ERR_UNSUPPORTED).  Each weight is stored as an OCP FP4 E2M1 code
 * (sign bit 3, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinities or NaN), two codes per byte: element 2i in bits 0..3 and element
 * 2i+1 in bits 4..7.  Every 32 consecutive elements of a row along the reduction dimension
 * share one E8M0 scale byte s, meaning 2^(s - 127); the weight is e2m1(code) * 2^(s - 127).
 *   w_gate, w_up [E,I,H/2] and w_down [E,H,I/2]: packed E2M1 codes, the rows of the bf16
 *            weights of beam_moe_forward at half a byte per element (16-byte aligned)
 *   s_gate, s_up [E,I,H/32] and s_down [E,H,I/32]: E8M0 scale bytes (16-byte aligned):
 *            2^(s - 127) for s = 0 .. 254 and NaN for s = 255, as for beam_moe_forward_fp8
 * Every other argument, the workspace and the results are as for beam_moe_forward.  A
 * weight whose decoded value is a normal bf16 number (or zero) is decoded exactly and the
 * layer computes exactly what beam_moe_forward computes on the decoded weights; the weight
 * bytes read from memory are a quarter (plus 1/32 byte of scale per weight).  Decoded
 * values beyond that range are rounded to bf16 as for beam_moe_forward_fp8; a NaN scale
 * makes the outputs of the tokens routed to that expert NaN.  The pages quote a ~4.5-bit checkpoint
 * format for another GPU family without its layout; this is the OCP microscaling MXFP4
 * format, the 4-bit format of this GPU's matrix cores.
 */
beam_status beam_moe_forward_mxfp4(const beam_moe_shape* shape, const void* x, const float* w_router,
                                   const float* bias, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                   const uint8_t* s_down, const beam_sublayer* sub, void* out, int32_t* topk_idx,
                                   float* topk_w, void* moe_y, void* ws, size_t ws_bytes, void* const* stage_events,
                                   void* stream);

/*
 * beam_moe_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a static device array of BEAM_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (no allocation per call; the
 * array's address is looked up once per device, on the first call there).
 *   Arguments and results: as beam_moe_forward, minus ws / ws_bytes.  stream must belong to
 *   the current device (else BEAM_ERR_INVALID_ARG).
 *   Limit: shapes whose beam_moe_workspace_size (BEAM_OP_FORWARD, or
 *   BEAM_OP_FORWARD_SUBLAYER with sub) exceeds BEAM_NOALLOC_SCRATCH_BYTES are rejected with
 *   BEAM_ERR_WORKSPACE before any launch (T <= 768 tokens at the Beam layer's shape,
 *   H = 5120, I = 2560, E = 256, top-8; use beam_moe_forward beyond).
 *   Calls on one GPU share its array: calls that overlap on one GPU (different streams, or
 *   different host threads) race and give wrong results; serialize them.
 * Its results are those of beam_moe_forward on the same arguments (same kernels).
 */
#define BEAM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
beam_status beam_moe_forward_noalloc(const beam_moe_shape* shape, const void* x, const float* w_router,
                                     const float* bias, const void* w_gate, const void* w_up, const void* w_down,
                                     const beam_sublayer* sub, void* out, int32_t* topk_idx, float* topk_w,
                                     void* moe_y, void* const* stage_events, void* stream);

/* Static description of a status code. */
const char* beam_status_string(beam_status status);

/* BEAM_MOE_ABI_VERSION of the built library. */
int32_t beam_moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
