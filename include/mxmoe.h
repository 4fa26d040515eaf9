/*
 * mxmoe.h -- C ABI of the gfx950 (AMD Instinct MI355X) routed-expert forward of an MXFP4 Stable
 * LatentMoE layer, as used by Kimi K3 / K3.1.
 *
 * What the layer computes (pages: "Kimi K3.1 Pro on AMD Instinct GPUs", section "Kimi K3.1 Pro
 * at a glance"; "Day 0 Kimi-K3 Inference Deployment with ATOM on AMD Instinct MI355X GPUs",
 * sections "Model Architecture" and "HBM Usage Under TP8"):
 *   z   = bf16(x . W_down^T)                          latent down-projection (BF16 weights)
 *   l   = fp32(x . W_router^T) + bias                  router logits (BF16 router)
 *   ids = top-K experts by (l descending, index ascending)
 *   w   = sigmoid(l[ids]) / sum(sigmoid(l[ids]))        gate weights over the selected K
 *   y_p = bf16(bf16(silu(z.Wg_e^T) * (z.Wu_e^T)) . Wd_e^T) for every pair p = (token, slot),
 *         Wg/Wu/Wd in MXFP4: E2M1 codes with one E8M0 scale per 32 values along the input axis
 *   zc  = bf16(sum over slots, in slot order, of w * y)
 *   out = bf16(zc . W_up^T + sum_s h_s . Wd_s^T),  h_s = bf16(silu(x.Wg_s^T) * (x.Wu_s^T))
 * Without latent projections (has_latent_proj = 0) x is the latent itself, the router reads it,
 * there are no shared experts and out = zc.
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument except the handle, the config and the structs themselves is DEVICE
 *    memory owned by the caller. The library never allocates device memory (no hipMalloc).
 *  - BF16 tensors are passed as 16-bit bit patterns, row-major, innermost dimension contiguous.
 *  - `stream` is a hipStream_t (NULL = the null stream). All device work is enqueued on it and the
 *    call returns without synchronising. Argument errors are reported synchronously before
 *    anything is enqueued; launch failures return MOE_ERR_HIP; device faults surface at the
 *    caller's next synchronisation. No C++ exception crosses this boundary.
 *  - Results are deterministic: identical inputs give bitwise-identical outputs (no
 *    floating-point atomics; every sum has a fixed order).
 *  - One handle may serve concurrent calls on different streams only with distinct workspaces,
 *    routing buffers and outputs.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,      /* bad config, shape, pointer or size                      */
    MOE_ERR_UNSUPPORTED = -2,      /* valid request outside what this build implements         */
    MOE_ERR_BUFFER_TOO_SMALL = -3, /* packed buffer or workspace smaller than moe_query says    */
    MOE_ERR_HIP = -4               /* a HIP launch or runtime call failed                      */
} moe_status;

/* Expert activation. The pages name the activation "SiTU-GLU" without defining it; the one
 * implemented reads it as the SiLU-gated GLU h = silu(g) * u, silu(g) = g * sigmoid(g). */
typedef enum { MOE_ACT_SILU_GLU = 0 } moe_act;

/* Arithmetic of the routed experts' second stage (the down product y = h . Wd_e^T).
 * MOE_STAGE2_BF16: h is the BF16 GLU output (the layer as defined above).
 * MOE_STAGE2_FP8:  h is first quantised to MX FP8 and the down product reads the quantised
 *   values, as the reference engine's FP8 second stage does (page "Kimi K3.1 Pro on AMD Instinct
 *   GPUs", section "What we optimized" and its appendix of environment variables). The pages fix
 *   neither the FP8 format nor the scale granularity; this build takes the OCP MX FP8 reading:
 *   per pair row, blocks of 32 consecutive h values along I share one E8M0 scale 2^X with
 *   X = floor(log2(max |h| in the block)) - 8 (clamped to [-127, 127]; -127 for an all-zero
 *   block), and each element h / 2^X is rounded to nearest even to an E4M3 code (4 significant
 *   bits, subnormal quantum 2^-9, no infinities) that saturates at +-448 and keeps the sign of h.
 *   The packed buffer then also holds the down weights in the layout of gfx950's scaled MX
 *   matrix-core instruction. */
typedef enum { MOE_STAGE2_BF16 = 0, MOE_STAGE2_FP8 = 1 } moe_stage2;

/* Arithmetic of the routed experts' first stage (the gate|up product with the GLU).
 * MOE_STAGE1_BF16:  the product reads z in BF16 (the layer as defined above).
 * MOE_STAGE1_MXFP4: z is first quantised to MX FP4 and the product reads the quantised values, as
 *   the reference engine's A4W4 mode does (page "Kimi K3.1 Pro on AMD Instinct GPUs", section "What
 *   we optimized" and its appendix of environment variables). The pages fix neither the scale rule
 *   nor the rounding; this build takes the OCP MX reading: per token row, blocks of 32 consecutive
 *   z values along Lt share one E8M0 scale 2^X with X = floor(log2(max |z| in the block)) - 2
 *   (clamped to [-127, 127]; -127 for an all-zero block), and each element z / 2^X is rounded to
 *   nearest even to an E2M1 code (2 significant bits, subnormal quantum 1/2) that saturates at +-6
 *   and keeps the sign of z; codes are packed two per byte, the even element in the low nibble.
 *   h = bf16(silu(g) * u) from those values; everything after h is unchanged. The packed buffer then
 *   also holds the gate|up weights in the layout of gfx950's scaled MX matrix-core instruction. */
typedef enum { MOE_STAGE1_BF16 = 0, MOE_STAGE1_MXFP4 = 1 } moe_stage1;

/* Where the shared experts' gate/up product (h_s = bf16(silu(x Wg_s^T) (x Wu_s^T))) runs. The
 * reference engine runs the shared experts on a second stream, concurrently with the routed
 * experts (page "Kimi K3.1 Pro on AMD Instinct GPUs", section "Serving with ATOM", "What we
 * optimized", paragraph on the MXFP4 latent MoE).
 * MOE_SHARED_FUSED:  its columns are part of the x-side product over x (one weight stream, one launch).
 * MOE_SHARED_STREAM: it is a product of its own on a second stream that the handle owns (created by
 *   moe_create at the default priority, destroyed by moe_destroy). Each call forks that stream off
 *   the caller's stream at its start (an event recorded on the caller's stream) and joins it back
 *   before the output product (the caller's stream waits on an event recorded on the second
 *   stream), so every call stays ordered on the caller's stream and can be captured into a HIP
 *   graph. The outputs are bit-identical to MOE_SHARED_FUSED. The packed buffer holds the shared
 *   gate/up rows apart from the x-side rows. Without shared experts the field has no effect. Calls
 *   on one handle with this mode must come from one host thread at a time: they share the second
 *   stream and its two events. */
typedef enum { MOE_SHARED_FUSED = 0, MOE_SHARED_STREAM = 1 } moe_shared_stream;

typedef struct {
    int32_t hidden;          /* H: width of x and out (multiple of 128); unused without latent  */
    int32_t latent;          /* Lt: latent width (multiple of 128)                               */
    int32_t n_experts;       /* E: routed experts, 1..1024                                       */
    int32_t top_k;           /* K: experts per token, 1..min(32, E)                              */
    int32_t inter;           /* I: routed-expert intermediate (multiple of 128)                  */
    int32_t n_shared;        /* S: shared experts, 0..8 (must be 0 without latent projections)   */
    int32_t shared_inter;    /* Is: shared-expert intermediate (multiple of 32 when S > 0)       */
    int32_t has_latent_proj; /* 1: x is the hidden state (down/up projections, shared experts)   */
    int32_t act;             /* moe_act                                                          */
    int32_t stage2;          /* moe_stage2                                                       */
    int32_t stage1;          /* moe_stage1                                                       */
    int32_t shared_stream;   /* moe_shared_stream                                                */
} moe_config;

/* Canonical weights (device, caller-owned; only read by moe_create's packing kernels, so they
 * may be freed once `stream` has passed moe_create). Hin = hidden if has_latent_proj else latent.
 * MXFP4 matrices: codes u8 [rows, cols/2], element 2i in the low nibble of byte i (bit 3 sign,
 * bits 2..1 exponent, bit 0 mantissa); scales u8 [rows, cols/32], one E8M0 byte (2^(e-127))
 * per 32 consecutive values of a row. Scale bytes 0 and 255 are outside the supported range. */
typedef struct {
    const void *w_router;     /* bf16 [E, Hin]                                        */
    const void *w_down;       /* bf16 [Lt, H]    (latent projections only)            */
    const void *w_up;         /* bf16 [H, Lt]    (latent projections only)            */
    const void *gate_codes;   /* u8 [E, I, Lt/2]                                      */
    const void *gate_scales;  /* u8 [E, I, Lt/32]                                     */
    const void *up_codes;     /* u8 [E, I, Lt/2]                                      */
    const void *up_scales;    /* u8 [E, I, Lt/32]                                     */
    const void *down_codes;   /* u8 [E, Lt, I/2]                                      */
    const void *down_scales;  /* u8 [E, Lt, I/32]                                     */
    const void *sh_gate;      /* bf16 [S, Is, H] (S > 0 only)                         */
    const void *sh_up;        /* bf16 [S, Is, H] (S > 0 only)                         */
    const void *sh_down;      /* bf16 [S, H, Is] (S > 0 only)                         */
} moe_weights;

/* Routing produced by moe_route and consumed by moe_forward (device, caller-allocated).
 * Pair p = t*K + j is token t's slot j; slots are in rank order. */
typedef struct {
    int32_t *topk_ids;        /* [T, K] expert of each slot                                   */
    float *topk_w;            /* [T, K] gate weight of each slot                              */
    int32_t *counts;          /* [E]    pairs routed to each expert                           */
    int32_t *offsets;         /* [E+1]  exclusive prefix sum of counts; offsets[E] = T*K      */
    int32_t *sorted_pairs;    /* [T*K]  pair ids grouped by expert, ascending within an expert */
    int32_t *inv;             /* [T*K]  inv[p] = position of pair p in sorted_pairs           */
} moe_routing;

typedef struct moe_handle moe_handle;

/* Sizes for a config: the packed-weight buffer moe_create needs and the workspace moe_route /
 * moe_forward need for up to T_max tokens (one workspace serves both calls). Either output
 * pointer may be NULL. Host-only; enqueues nothing. */
moe_status moe_query(const moe_config *cfg, int32_t T_max, size_t *packed_bytes,
                     size_t *workspace_bytes);

/* Test hook: byte offsets inside the workspace for T tokens, in this order: FP32 logits [T,E],
 * per-block expert histogram, the expert tile list, z [T,Lt], [zc | h_s] [T, Lt + S Is],
 * h [T K, I] and y [T K, Lt] (expert-sorted rows, BF16), the MX FP8 h of MOE_STAGE2_FP8 (E4M3
 * codes [T K, I], then from byte offset T K I the E8M0 scales [T K, I/32]; empty otherwise),
 * the MX FP4 z of MOE_STAGE1_MXFP4 (E2M1 codes [T, Lt/2], then from byte offset T Lt/2 the E8M0
 * scales [T, Lt/32]; empty otherwise), FP32 split-K partials, then the total size. `offsets` is a
 * host array of 11 entries.
 * Host-only. */
moe_status moe_query_workspace_layout(const moe_config *cfg, int32_t T, size_t *offsets);

/* Validate the config and weights, then enqueue the packing of every weight into `packed`
 * (device, >= packed_bytes from moe_query, 256-byte aligned): dense BF16 weights are tiled in
 * matrix-core fragment order, MXFP4 experts are tiled per 16 rows x 128 inputs with their scales
 * alongside, gate and up rows interleaved per 16 so one tile holds both halves of the GLU.
 * On success *out is a host-side handle (host memory only); `packed` must stay alive and
 * unmodified until moe_destroy. */
moe_status moe_create(const moe_config *cfg, const moe_weights *w, void *packed,
                      size_t packed_bytes, void *stream, moe_handle **out);

/* Routing for T tokens (0 <= T; T = 0 enqueues nothing and leaves `r` untouched).
 * x: bf16 [T, Hin], 16-byte aligned. logit_bias: fp32 [E] added to the router product, or NULL.
 * logits_in: fp32 [T, E] final logits to select on instead of computing them (then x and
 * logit_bias must be NULL). logits_out: fp32 [T, E] receives the computed logits, or NULL.
 * Writes every array of `r`. workspace: >= moe_query(cfg, T).workspace_bytes. */
moe_status moe_route(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                     const float *logits_in, float *logits_out, const moe_routing *r,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Forward for the same T tokens, given the routing moe_route produced for them.
 * x: bf16 [T, Hin]; out: bf16 [T, H] (or [T, Lt] without latent projections), must not alias
 * x; both 16-byte aligned (MOE_ERR_INVALID_ARG otherwise). workspace: 256-byte aligned, >=
 * moe_query(cfg, T).workspace_bytes (may be the one given to moe_route). */
moe_status moe_forward(moe_handle *h, const void *x, int32_t T, const moe_routing *r, void *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* moe_route (with logits_in = NULL) followed by moe_forward, in one call, with results identical
 * bit for bit to the two calls. With latent projections the router and the x-side products
 * (latent down-projection, shared gate/up), which both read only x, run as one product over a
 * combined copy of their weights kept in the packed buffer, so x is read once and one launch
 * streams both weight matrices. All work runs on `stream`, in order.
 * Arguments as for the two calls; logits_out may be NULL and must not alias x or out. */
moe_status moe_route_forward(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                             float *logits_out, const moe_routing *r, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Size of the device scratch array that moe_route_forward_static works in: 40 MiB, enough for the
 * workspace of up to ~280 tokens at one GPU's TP8 share of the Kimi K3 layer (64 decode tokens
 * need 29.5 MiB) and of every call whose moe_query workspace_bytes is at most this size. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)40 << 20)

/* moe_route_forward without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The workspace is a file-scope device array of MOE_STATIC_SCRATCH_BYTES inside the library, one
 * per GPU, allocated when the library's code is loaded on that GPU and held until the process
 * ends; the call itself allocates nothing (no hipMalloc / hipFree). Results are identical bit for
 * bit to moe_route_forward's with a caller workspace. Arguments and errors as for
 * moe_route_forward, plus MOE_ERR_BUFFER_TOO_SMALL when this call's workspace (moe_query with
 * T_max = T) exceeds MOE_STATIC_SCRATCH_BYTES, returned before anything is enqueued.
 * Every call on one GPU uses that GPU's single array, which keeps the previous call's contents:
 * calls that overlap on one GPU (concurrent streams, or several handles) race on it and must be
 * serialised by the caller (e.g. one stream per GPU). */
moe_status moe_route_forward_static(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                                    float *logits_out, const moe_routing *r, void *out, void *stream);

/* The whole few-token step as one HIP graph (the fused decode step: route, grouping, expert
 * products, combine and shared experts replayed as a unit; page "Kimi K3.1 Pro on AMD Instinct
 * GPUs", sections "Serving with ATOM / What we optimized", paragraph "Mono decode", and "Serving
 * with vLLM / What we optimized", paragraph on fused low-latency decode).
 * moe_graph_create captures moe_route_forward's launches for these exact arguments into an
 * executable graph: the graph keeps the pointers (x, logit_bias, logits_out, every array of r,
 * out, workspace), so the caller writes each step's tokens into the same x buffer and keeps every
 * buffer alive and unmoved until moe_graph_destroy. Capture runs on a stream of the library's own
 * and enqueues no work; it returns MOE_ERR_INVALID_ARG for T = 0, for arguments moe_route_forward
 * would reject, and while the profiling hook is active on h. The graph holds no memset node.
 * moe_graph_launch enqueues one replay on `stream` (allocating nothing): results are identical
 * bit for bit to moe_route_forward on the buffers' contents at that point of the stream. Replays
 * that overlap (several streams) race on the workspace like overlapping calls. */
typedef struct moe_graph moe_graph;
moe_status moe_graph_create(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                            float *logits_out, const moe_routing *r, void *out, void *workspace,
                            size_t workspace_bytes, moe_graph **g);
moe_status moe_graph_launch(moe_graph *g, void *stream);
/* Free the graph (its host and driver objects; no buffer it refers to). NULL is a no-op. */
void moe_graph_destroy(moe_graph *g);

/* Test hook: dequantise expert e's packed matrix `which` (0 gate [I, Lt], 1 up [I, Lt],
 * 2 down [Lt, I]) back to canonical row-major BF16 in `out` through the same in-register
 * E2M1/E8M0 conversion the expert GEMMs use. */
moe_status moe_unpack_expert(moe_handle *h, int32_t e, int32_t which, void *out, void *stream);

/* Kernels of the path, as reported by the profiling hook. */
typedef enum {
    MOE_KERNEL_ROUTER = 0,   /* router product -> FP32 logits                       */
    MOE_KERNEL_TOPK = 1,     /* top-K selection and gate weights                    */
    MOE_KERNEL_PERMUTE = 2,  /* histogram, scan and stable scatter (three launches) */
    MOE_KERNEL_XSIDE = 3,    /* latent down-projection + shared gate/up GLU         */
    MOE_KERNEL_TILEMAP = 4,  /* tile lists of the expert products                   */
    MOE_KERNEL_GATEUP = 5,   /* routed gate/up product with the GLU                 */
    MOE_KERNEL_DOWN = 6,     /* routed down product                                 */
    MOE_KERNEL_COMBINE = 7,  /* gate-weighted combine                               */
    MOE_KERNEL_OUT = 8,      /* up-projection + shared down-projection              */
    MOE_KERNEL_XSIDE_EPI = 9,/* few-token x-side partial sums, GLU and tile lists   */
    MOE_KERNEL_OUT_EPI = 10, /* few-token output partial sums                       */
    MOE_KERNEL_ROUTER_XSIDE = 11,/* router + x-side product as one (moe_route_forward) */
    MOE_KERNEL_H_QUANT = 12, /* MX FP8 quantisation of h (MOE_STAGE2_FP8)           */
    MOE_KERNEL_Z_QUANT = 13, /* MX FP4 quantisation of z (MOE_STAGE1_MXFP4)         */
    MOE_KERNEL_SHARED = 14   /* shared gate/up product and its GLU (MOE_SHARED_STREAM, second stream) */
} moe_kernel;

/* Profiling hook (benchmarks, tests): after moe_profile_begin, every kernel launch of moe_route
 * and moe_forward on this handle is bracketed by two HIP events recorded on the call's stream,
 * for at most max_launches launches (events are host-created objects, no device allocation).
 * moe_profile_end waits for the recorded events, writes up to *n entries (kernel id, elapsed ms)
 * into the host arrays, sets *n to the number written and stops profiling. */
moe_status moe_profile_begin(moe_handle *h, int32_t max_launches);
moe_status moe_profile_end(moe_handle *h, int32_t *kernel_ids, float *ms, int32_t *n);

/* Free the host handle (not the packed buffer, which the caller owns). NULL is a no-op. */
void moe_destroy(moe_handle *h);

/* Static description of a status code. */
const char *moe_strerror(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
