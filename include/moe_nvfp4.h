/*
 * moe_nvfp4.h -- C ABI of the routed NVFP4 mixture-of-experts FFN for one AMD MI355X (gfx950).
 *
 * The layer (the routed MoE FFN that the memra-engine probes moe_sk_repro.rs,
 * moe_sel_census.rs and moe_union_probe.rs time, and whose rank-local E256 shape the Rocket
 * post "Rank-local E256 MoE misses the Qwen K1 and K4 step budgets" measures):
 *
 *   for every token t and slot j < k with local expert e = topk_ids[t*k+j] - expert_base:
 *     g = Wg[e] x_t,  u = Wu[e] x_t,  h = silu(g) * u,  d = Wd[e] h
 *   y_t = sum over local slots j, in ascending j, of topk_w[t*k+j] * d     (fp32, no atomics)
 *
 * Two calls make one layer: moe_route_bucket (expert-first CSR of the routed pairs) and then
 * moe_ffn_nvfp4 (the FFN over that CSR). moe_router_topk can produce the routed pairs and their
 * weights from router logits first.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are GPU device addresses; the library never allocates, frees,
 *    copies to the host or synchronizes. All work is enqueued on `stream` in order.
 *  - The caller owns every buffer. Workspaces are caller-allocated device memory of at least the
 *    size the matching *_ws() function returns; their content need not be initialized and is
 *    overwritten.
 *  - Return value: MOE_OK, or an error code for conditions the host can check (arguments,
 *    sizes, launch limits) -- nothing is enqueued then. A device fault surfaces at the caller's
 *    next synchronization. Inputs holding NaN or Inf give undefined outputs.
 *  - Calls that share no workspace or output may run concurrently on different streams.
 *
 * NVFP4 weight format (moe_sel_census.rs, its block constants; moe_union_probe.rs, its
 * per-expert byte arithmetic): 64 weights per 36-byte block; bytes 0..3 hold the UE4M3 scales of
 * weights 16j..16j+15 (j = 0..3), bytes 4..35 hold E2M1 codes, weight 2i in the low nibble and
 * weight 2i+1 in the high nibble of byte 4+i. E2M1 is the OCP MX FP4 element type; UE4M3 is the
 * OCP FP8 E4M3 type with its sign bit 0 (bytes 0x00..0x7E; others are undefined). A weight is
 * code value * scale. A row holds in_f weights (in_f/64 blocks) for one output feature and is
 * contiguous along the input features (moe_sk_repro.rs, its bank construction: row_bytes =
 * in_f/64*36 and per-expert stride out_f*row_bytes).
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *moe_stream_t; /* a hipStream_t; NULL is the default stream */

/* Status codes. */
enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,  /* null pointer, negative T, k<1, E<1, k>4096, H or F not a positive
                        multiple of 64, bank base or stride not a multiple of 16 bytes */
    MOE_EWS = 2,     /* workspace smaller than the matching *_ws() size */
    MOE_ESHAPE = 3,  /* a size beyond what this build can launch (see MOE_MAX_*) */
    MOE_ELAUNCH = 4  /* the HIP runtime reported an error when the work was enqueued */
};

/* Path selection for moe_ffn_nvfp4. */
enum {
    MOE_PATH_AUTO = 0,          /* the path moe_auto_path() names for the sizes */
    MOE_PATH_DECODE = 1,        /* force the bandwidth-bound decode path */
    MOE_PATH_PREFILL = 2        /* force the grouped-GEMM path (f16 MFMA) */
};

#define MOE_MAX_EXPERTS 2048       /* E limit of the bucketing kernel */
#define MOE_MAX_PAIRS (1 << 24)    /* T*k limit */
#define MOE_MAX_HIDDEN 16384       /* H limit */
#define MOE_MAX_FF 8192            /* F limit */
#define MOE_MAX_ROUTER_K 64        /* k limit of moe_router_topk (one slot per wavefront lane) */
#define MOE_AUTO_PAIRS_PER_EXPERT 16   /* MOE_PATH_AUTO's decode limit: routed pairs per expert */

/*
 * One weight bank: expert e's rows start at base + e*expert_stride (bytes, device).
 * scale2 (device, fp32 [E], or NULL): the optional second level of two-level NVFP4 (the
 * ModelOpt form of the Rocket post's banks; moe_union_probe.rs names its "modelopt" kernels):
 * every weight of expert e in this bank is code value * UE4M3 group scale * scale2[e]. The
 * factor multiplies the bank's fp32 sums once, before SiLU for gate and up, at the output for
 * down. NULL means 1 for every expert. Must be 4-byte aligned.
 * experts (device, [E] device pointers, or NULL): the per-expert table form (moe_sk_repro.rs
 * builds a table of per-expert weight pointers for its grouped calls): when not NULL, expert e's
 * rows start at experts[e] and base / expert_stride are not used (base may be NULL). Every
 * experts[e] of an expert that is routed to must be 16-byte aligned (not checkable on the host:
 * a misaligned entry gives undefined results); the table itself must be 8-byte aligned.
 * kpack (device, or NULL): an optional second copy of the same weights in the K-step-packed
 * layout that moe_kpack() writes (see there). When not NULL, the grouped-GEMM (prefill) path
 * reads the weights from it instead of base / experts; the decode path always reads base /
 * experts. Must be 16-byte aligned, and must hold this bank's rows exactly (the row count and
 * in-width of the call, the E experts of the call): it is not checked against base.
 */
typedef struct {
    const uint8_t *base;
    int64_t expert_stride;
    const float *scale2;
    const uint8_t *const *experts;
    const uint8_t *kpack;
} moe_bank;

/*
 * The K-step-packed copy of a bank for the grouped-GEMM path (a weight layout prepared once, like
 * the weight shuffling that grouped GEMMs apply before they run; the pages' kernels for other
 * hardware read the row-major banks). Rows are taken in groups of MOE_KPACK_ROWS; within a
 * group, the 36-byte NVFP4 blocks of one 64-wide K step of all its rows form one run of
 * MOE_KPACK_ROWS * 36 bytes, dst[e][g][b][0 .. MOE_KPACK_ROWS*36 - 1] (e < E, g <
 * ceil(out_f / MOE_KPACK_ROWS), b < in_f / 64), for rows g*MOE_KPACK_ROWS + r of expert e and
 * their block b (bytes 0..3 the four UE4M3 scales, 4..35 the 32 bytes of E2M1 codes, as in the
 * row-major bank); rows at or past out_f are zero bytes. A run is 8 slices of 32 rows, 1152
 * bytes each; slice s holds rows 32 s + 16 t + n (tile t < 2, n < 16) as
 *     bytes 512 t + 8 l + j (lane l = n + 16 p < 64, j < 8): code byte 4 + 8 p + j of row n of
 *                                                           tile t,
 *     bytes 1024 + 2 l + t:                                 scale byte p of row n of tile t,
 * i.e. the order in which a 64-lane wave takes them as 16 x 32 matrix-core operands. So the copy
 * holds the same 36 bytes per 64 weights plus the padding of the last group. A GEMM K step then
 * stages one contiguous run per weight tile instead of a 36-byte piece of each of its rows, and
 * reads its operands from LDS without bank conflicts (both grouped GEMMs measured 7%, then a
 * further 2% faster).
 *
 * moe_kpack_bytes: the bytes of the copy (0 for invalid sizes).
 * moe_kpack: writes the copy of bank src (its base / expert_stride or experts table; scale2 and
 * kpack are ignored) for E experts of out_f rows of in_f weights into dst (device, 16-byte
 * aligned, moe_kpack_bytes(E, out_f, in_f) bytes), enqueued on stream; it allocates nothing.
 * Returns MOE_EINVAL for a null or misaligned dst, E, out_f or in_f not positive, in_f not a
 * multiple of 64, or a bank that fails the checks of moe_ffn_nvfp4; MOE_ESHAPE for out_f or
 * in_f above MOE_MAX_HIDDEN or E above MOE_MAX_EXPERTS; MOE_ELAUNCH if the launch fails.
 */
#define MOE_KPACK_ROWS 256
size_t moe_kpack_bytes(int32_t E, int32_t out_f, int32_t in_f);
int moe_kpack(moe_bank src, int32_t E, int32_t out_f, int32_t in_f, uint8_t *dst,
              moe_stream_t stream);

/*
 * Workspace bytes moe_route_bucket needs for T tokens, k slots and E local experts.
 */
size_t moe_route_bucket_ws(int32_t T, int32_t k, int32_t E);

/*
 * Expert-first bucketing of the routed (token, expert) pairs (moe_sk_repro.rs: the host
 * bucketing that builds ex_ids / ex_off / ex_pairs before the grouped calls, and the gather
 * index csr_tok = pair / top_k).
 *
 *   topk_ids  (device) int32 [T*k], pair p = t*k + j names expert topk_ids[p].
 *   expert_base        local expert of p is topk_ids[p] - expert_base; pairs whose local id is
 *                      outside [0, E) belong to another expert-parallel rank and are not routed.
 *   offsets   (device, out) int32 [E+1]: offsets[e] = number of local pairs with local expert
 *                      < e; offsets[E] = number of local pairs.
 *   pair_ids  (device, out) int32 [T*k]: positions [offsets[e], offsets[e+1]) list the pairs of
 *                      expert e in ascending p (stable); positions [offsets[E], T*k) list the
 *                      non-local pairs in ascending p.
 *   active    (device, out) int32 [E]: the first n_active entries are the non-empty local
 *                      experts in ascending order; the rest are unspecified.
 *   counts    (device, out) int32 [2]: n_active, n_nonlocal.
 *   ws, ws_bytes (device) scratch of at least moe_route_bucket_ws(T, k, E) bytes.
 *
 * Bit-exact: outputs depend only on topk_ids. T = 0 is valid (offsets all 0, counts 0).
 * Errors: MOE_EINVAL (null pointer, T<0, k<1, E<1), MOE_ESHAPE (E > MOE_MAX_EXPERTS or
 * T*k > MOE_MAX_PAIRS), MOE_EWS, MOE_ELAUNCH.
 */
int moe_route_bucket(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t expert_base,
                     int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts,
                     void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * The path MOE_PATH_AUTO takes in moe_ffn_nvfp4 and moe_layer_nvfp4 for these sizes, decided on
 * the host alone (no device work): MOE_PATH_DECODE for T <= 128 or T*k <= MOE_AUTO_PAIRS_PER_EXPERT
 * * E where the decode kernels can launch for (T, k, E, H, F), else MOE_PATH_PREFILL. The pages
 * split the work the same way, a bandwidth-bound path for a few tokens per expert and grouped GEMMs
 * for prefill (moe_sk_repro.rs, its decode and prefill regimes); the pairs-per-expert limit is near
 * where the two paths measured equal on one MI355X, the GEMMs reading K-step-packed copies (about
 * 12 and 16 pairs per expert on the skewed hidden-4096 routings at ff 1280 and 640, 18 on the
 * uniform E256 one; the decode kernels stream an expert's weights once per run of 16 pairs).
 * Returns the path, or minus an MOE_E* code for sizes moe_ffn_nvfp4 would refuse (-MOE_EINVAL,
 * -MOE_ESHAPE).
 */
int32_t moe_auto_path(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);

/*
 * Workspace bytes moe_ffn_nvfp4 needs (for any path).
 */
size_t moe_ffn_nvfp4_ws(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);

/*
 * The routed FFN over the CSR that moe_route_bucket wrote (moe_union_probe.rs: the fused
 * gate/up + SiLU and down kernels it prices, reading each distinct expert's weights once per
 * call; moe_sk_repro.rs: the gate, up and down grouped calls of a prefill layer).
 *
 *   x         (device) bf16 bit patterns [T, H], row-major.
 *   topk_w    (device) fp32 [T*k] router weights, used as given.
 *   offsets, pair_ids, active, counts  (device) exactly as moe_route_bucket wrote them for the
 *                      same topk_ids, T, k, E.
 *   gate, up  rows of H weights: expert e's gate row o (o < F) starts at
 *                      gate.base + e*gate.expert_stride + o*(H/64*36) (gate.experts[e] +
 *                      o*(H/64*36) for a bank given as a pointer table); likewise up. A fused
 *                      gate_up bank [E, 2F, H] with gate rows first is gate = {B, 2F*rb},
 *                      up = {B + F*rb, 2F*rb}, rb = H/64*36.
 *   down      rows of F weights: expert e's down row r (r < H) starts at
 *                      down.base + e*down.expert_stride + r*(F/64*36) (or down.experts[e] + ...).
 *             Each bank may also carry a K-step-packed copy (kpack: moe_kpack of that bank with
 *             out_f F for gate and up, H for down); gate and up carry one both or neither
 *             (MOE_EINVAL otherwise). The GEMM path then reads the packed copies; y is the same
 *             bit for bit.
 *   y         (device, out) fp32 [T, H], fully overwritten; a token with no local slot gets 0.
 *   path      MOE_PATH_AUTO / MOE_PATH_DECODE / MOE_PATH_PREFILL.
 *   ws, ws_bytes (device) scratch of at least moe_ffn_nvfp4_ws(T, k, E, H, F) bytes.
 *
 * Deterministic: the same inputs give bit-identical y on every call (the combine sums each
 * token's slots in ascending j in fp32, with no atomics).
 * Errors: MOE_EINVAL, MOE_ESHAPE (H > MOE_MAX_HIDDEN, F > MOE_MAX_FF, E > MOE_MAX_EXPERTS,
 * T*k > MOE_MAX_PAIRS), MOE_EWS, MOE_ELAUNCH. T = 0 is a valid no-op.
 */
int moe_ffn_nvfp4(const uint16_t *x, const float *topk_w, const int32_t *offsets,
                  const int32_t *pair_ids, const int32_t *active, const int32_t *counts,
                  moe_bank gate, moe_bank up, moe_bank down, int32_t T, int32_t k, int32_t E,
                  int32_t H, int32_t F, float *y, int32_t path, void *ws, size_t ws_bytes,
                  moe_stream_t stream);

/*
 * Workspace bytes moe_layer_nvfp4 needs (for any path).
 */
size_t moe_layer_nvfp4_ws(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);

/*
 * The whole routed layer in one call: moe_route_bucket followed by moe_ffn_nvfp4, from the routed
 * expert ids to y (moe_sk_repro.rs, its host bucketing and the three grouped calls;
 * moe_union_probe.rs, the fused gate/up + SiLU and down kernels it prices), without the CSR as
 * an output. On the decode path with at most 2048 routed pairs and at most 1024 experts, the
 * decode kernels bucket the pairs themselves (each workgroup in its LDS, into the same stable
 * expert-first CSR) and no bucketing launch is made; otherwise the bucketing kernel runs first,
 * into the workspace.
 *   topk_ids, expert_base  as for moe_route_bucket (ids outside [expert_base, expert_base + E)
 *                      are not routed).
 *   x, topk_w, gate, up, down, T, k, E, H, F, y, path  as for moe_ffn_nvfp4.
 *   ws, ws_bytes (device) scratch of at least moe_layer_nvfp4_ws(T, k, E, H, F) bytes, 256-byte
 *                      aligned.
 * y equals, bit for bit, what moe_route_bucket + moe_ffn_nvfp4 give on the same path (both
 * paths are deterministic). Errors: as for moe_ffn_nvfp4 (MOE_EINVAL also for a null topk_ids).
 */
int moe_layer_nvfp4(const int32_t *topk_ids, int32_t expert_base, const uint16_t *x,
                    const float *topk_w, moe_bank gate, moe_bank up, moe_bank down, int32_t T,
                    int32_t k, int32_t E, int32_t H, int32_t F, float *y, int32_t path, void *ws,
                    size_t ws_bytes, moe_stream_t stream);

/*
 * moe_ffn_nvfp4 without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The workspace is a library-owned device array of MOE_STATIC_WS_BYTES per GPU (held from the
 * library's first use on that GPU until the process ends); the call allocates nothing.
 * Arguments, outputs and errors are those of moe_ffn_nvfp4, plus MOE_EWS when
 * moe_ffn_nvfp4_ws(T, k, E, H, F) exceeds MOE_STATIC_WS_BYTES (checked on the host before
 * anything is enqueued), and MOE_ELAUNCH if the array's device address cannot be found.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or from several threads without ordering) race and give undefined results.
 * The array's content is not carried from one call to the next.
 */
#define MOE_STATIC_WS_BYTES (128u << 20)
int moe_ffn_nvfp4_static(const uint16_t *x, const float *topk_w, const int32_t *offsets,
                         const int32_t *pair_ids, const int32_t *active, const int32_t *counts,
                         moe_bank gate, moe_bank up, moe_bank down, int32_t T, int32_t k,
                         int32_t E, int32_t H, int32_t F, float *y, int32_t path,
                         moe_stream_t stream);

/*
 * Router step (the step before moe_route_bucket; the pages route each token to k distinct experts
 * with softmax router weights -- the Rocket post's E512 top-10, the moe_sk_repro.rs top-8 -- but
 * leave the router itself unspecified; the reading implemented here is the plain one):
 *   for each token t, slot j < k holds the expert with the j-th largest logit of row t, equal
 *   logits taken in ascending expert id, no expert twice (a total order: the result is unique);
 *   topk_w[t*k+j] = exp(l_j - l_0) / sum over the k selected of exp(l_i - l_0), in fp32.
 * The outputs are the topk_ids / topk_w arrays moe_route_bucket and moe_ffn_nvfp4 take.
 *   logits    (device) fp32 [T, E], row-major.
 *   topk_ids  (device) int32 [T, k]; topk_w (device) fp32 [T, k].
 * No workspace. T = 0 is a valid no-op. Logits must be finite (NaN or Inf: undefined outputs).
 * Errors: MOE_EINVAL (null pointer with T > 0, T<0, E<1, k<1, k>E), MOE_ESHAPE (E >
 * MOE_MAX_EXPERTS, k > MOE_MAX_ROUTER_K or T*k > MOE_MAX_PAIRS), MOE_ELAUNCH.
 */
int moe_router_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                    float *topk_w, moe_stream_t stream);

/*
 * Diagnostics: timing of one kernel of the layer with caller-created HIP events.
 * After this call, the next n_events launches of kernel `kernel_id` (a MOE_KERNEL_* value) are
 * bracketed by hipEventRecord(start_events[i]) / hipEventRecord(stop_events[i]) on the launch
 * stream. kernel_id = MOE_KERNEL_NONE (or n_events = 0) switches this off. The event arrays
 * (host arrays of hipEvent_t) must stay valid while it is on. Process-wide state, not thread
 * safe; meant for benchmarks. Returns MOE_OK, or MOE_EINVAL for a bad id or null arrays.
 */
enum {
    MOE_KERNEL_NONE = 0,
    MOE_KERNEL_BUCKET = 1,       /* moe_route_bucket's kernel */
    MOE_KERNEL_GU_DECODE = 2,    /* decode gate/up + SiLU */
    MOE_KERNEL_DN_DECODE = 3,    /* decode down projection */
    MOE_KERNEL_COMBINE = 4,      /* ordered router-weighted combine */
    MOE_KERNEL_SCHEDULE = 5,     /* prefill tile schedule */
    MOE_KERNEL_GU_PREFILL = 6,   /* prefill gate/up grouped GEMM */
    MOE_KERNEL_DN_PREFILL = 7,   /* prefill down grouped GEMM */
    MOE_KERNEL_ROUTER = 8        /* moe_router_topk's kernel */
};
int moe_profile_kernel(int32_t kernel_id, void *const *start_events, void *const *stop_events,
                       int32_t n_events);
/* Number of launches recorded since the last moe_profile_kernel call. */
int32_t moe_profile_count(void);

/* Name of a status code ("MOE_OK", ...); never NULL. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
