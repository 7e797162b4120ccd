/*
 * dlm.h -- C ABI of the MI355X (gfx950) hot path of token-level pre-gated
 * dynamic LoRA adapters (AdaFuse: "Accelerating Dynamic Adapter Inference via
 * Token-Level Pre-Gating and Fused Kernel Optimization").
 *
 * Three operations:
 *   dlm_pregate  one top-2 routing decision per token, made once and reused by
 *                every adapted layer (AdaFuse digest, section 2-ga "token-level
 *                pre-gating"; English abstract, "decide-once, apply-everywhere").
 *   dlm_switch   one launch that removes the previous token's gated adapters
 *                from every adapted weight of every layer and merges the current
 *                token's, in place (digest section 2-na "fused adapter
 *                switching": concatenated adapters, parallel GEMM in one
 *                kernel, in-place update, prefetch).
 *   dlm_sgmm     the unmerged batched form for rows with different expert sets,
 *                y += sum_k g_k (x A_k^T) B_k^T, segmenting rows by their set
 *                (digest section 2-na names the SGMM, "segmented gather matrix
 *                multiplication", kernel).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer and every stream; `stream` is a hipStream_t passed as void*
 *     (NULL = the legacy default stream).  Calls only enqueue work on `stream`
 *     and return; device-side failures are reported through the status calls.
 *   - Layouts are row-major.  Adapted weight W is [d_out][d_in]; expert bank A
 *     is [E][r][d_in] (A_e = the LoRA "down" matrix), B is [E][d_out][r] (B_e =
 *     the LoRA "up" matrix); the delta of expert e is B_e A_e.
 *   - An expert set is two slots (idx[2] int32, g[2] fp32).  idx = -1 is an
 *     empty slot; a NULL set pointer is the empty set.  Slot order does not
 *     change results of dlm_switch (the kernel orders the slots itself).
 *   - dtype: DLM_F32 or DLM_BF16 for every floating tensor of a call (x, Wr,
 *     W, A, B, y); gates g are always fp32, indices int32.
 *   - bf16 arithmetic: bf16 operands, fp32 accumulation; results are rounded
 *     to bf16 once, to nearest even.
 *   - Every call validates its arguments on the host before touching the GPU;
 *     on a negative status nothing was enqueued and no memory was changed.
 *     dlm_last_error() gives a text for the last failure of the calling thread.
 *   - Thread safety: calls on distinct handles / workspaces may run
 *     concurrently; one handle or workspace must not be used by two calls in
 *     flight at once (the caller orders its streams).
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DLM_OK = 0,
    DLM_EINVAL = -1,     /* null pointer, bad count, bad value */
    DLM_ESHAPE = -2,     /* a size out of the supported range, or sizes whose
                            launch grid would exceed 2^32 - 1 work-items (refused
                            before anything is launched) */
    DLM_EDTYPE = -3,     /* unknown or unsupported dtype */
    DLM_EALIGN = -4,     /* a pointer or row pitch not 16-byte aligned (bf16 fast path) */
    DLM_EWORKSPACE = -5, /* workspace missing or too small */
    DLM_EHIP = -6,       /* a HIP runtime call failed */
    DLM_EDEVICE = -7,    /* the device rejected an expert set (index out of range,
                            non-finite gate); reported by the status calls */
    DLM_ENOMEM = -8      /* a host or device allocation failed */
} dlm_status;

typedef enum { DLM_F32 = 0, DLM_BF16 = 1 } dlm_dtype;

/* Compile-time limits of the library. */
#define DLM_MAX_EXPERTS 32
#define DLM_MAX_RANK 128
#define DLM_MAX_CENTROIDS 1024   /* per adapter, dlm_pregate_centroid */

/* Text of the calling thread's last non-OK status (static storage). */
const char* dlm_last_error(void);

/* Library version string. */
const char* dlm_version(void);

/* ------------------------------------------------------------------ router */

/*
 * Top-2 pre-gate for T tokens (digest section 2-ga: a lightweight top-2 router
 * at the first layer selects each token's expert set; the set is then reused by
 * every layer).
 *   x  [T][d]  token activations at the first layer (dtype)
 *   Wr [d][E]  router weight (dtype)
 *   idx [T][2] out, int32: slot 0 = expert with the largest logit l = x.Wr,
 *              slot 1 = largest of the rest; equal logits -> lower index.
 *   g   [T][2] out, fp32: softmax over all E renormalised over the kept two,
 *              i.e. g0 = 1/(1+exp(l1-l0)), g1 = 1 - g0 (computed in binary64,
 *              rounded once to fp32).
 * Logits accumulate in binary64 (the products of fp32/bf16 inputs are exact),
 * so the decision is exact up to the summation order.  idx is always in
 * [0, E) and idx[t][0] != idx[t][1], also for non-finite inputs.
 * Requires 2 <= E <= DLM_MAX_EXPERTS, d >= 1, 0 <= T < 2^31 (T = 0 enqueues
 * nothing).
 */
int dlm_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int32_t E,
                int32_t dtype, int32_t* idx, float* g, void* stream);

/*
 * Training-free nearest-centroid pre-gate (the ARIADNE page: each adapter is
 * represented by centroids of its training data's embeddings; the input's
 * embedding is compared with them and the closest adapter is chosen), with the
 * same output format as dlm_pregate so it feeds dlm_switch / dlm_sgmm as is:
 *   x [T][d], C [E][J][d] (row-major, dtype; C adapter-major: J centroids of
 *   adapter 0, then adapter 1, ...).  Adapter distance = min over its J
 *   centroids of sum_k (x_k - c_k)^2, accumulated in binary64 with a fixed
 *   reduction order.  idx[t] = {nearest adapter (ties -> lower index), -1},
 *   g[t] = {1, 0}.
 * Requires 1 <= E <= DLM_MAX_EXPERTS, 1 <= J <= DLM_MAX_CENTROIDS, d >= 1,
 * 0 <= T < 2^31.  One launch on `stream`, no allocation.
 */
int dlm_pregate_centroid(const void* x, const void* C, int64_t T, int64_t d, int32_t E,
                         int32_t J, int32_t dtype, int32_t* idx, float* g, void* stream);

/* ------------------------------------------------------------ fused switch */

/* One adapted weight and its expert bank. */
typedef struct {
    void* W;        /* [d_out][d_in], updated in place by dlm_switch */
    const void* A;  /* [E][r][d_in] */
    const void* B;  /* [E][d_out][r] */
    int64_t d_out;
    int64_t d_in;
} dlm_proj;

typedef struct dlm_layers dlm_layers;

/*
 * Build the table of every adapted weight of every layer (L*P entries) that
 * one dlm_switch call updates.  Copies the host descriptors to a small device
 * table plus a device error word.  The buffers themselves stay owned by the
 * caller and must outlive the handle.
 *   projs (host) [n]; E in [1, DLM_MAX_EXPERTS]; r in [1, DLM_MAX_RANK];
 *   scale = the LoRA scale s multiplying every delta.
 * bf16: every W/A/B pointer 16-byte aligned and every d_in a multiple of 8.
 * bf16 with r in 17..64: the handle also allocates and fills a packed copy of
 * every A bank (E * ceil(d_in/64) * 64 * 16*ceil(r/16) bf16 per weight, about
 * the size of A) that the switch stages into LDS with direct copies; the
 * device is synchronised before returning.  The copy is taken here: after
 * changing an A bank in place call dlm_layers_repack.  Otherwise does not
 * synchronise.  All of it is freed by destroy.  *out (host) receives the handle.
 */
int dlm_layers_create(const dlm_proj* projs, int32_t n, int32_t E, int32_t r,
                      float scale, int32_t dtype, dlm_layers** out);

/* Free the handle's device memory (synchronises the device first). */
int dlm_layers_destroy(dlm_layers* h);

/*
 * Refresh the handle's packed A copies from the caller's A banks: one launch
 * per weight on `stream`, no allocation (no-op when the handle keeps none).
 */
int dlm_layers_repack(dlm_layers* h, void* stream);

/*
 * One fused switch over every weight of the handle, one kernel launch:
 *   W <- round( W - s*sum_{k in old} g_k B_k A_k + s*sum_{k in new} g_k B_k A_k )
 * (digest section 2-na: remove the previous token's adapters and merge the
 * current token's, on concatenated adapter matrices, in place).  The sets are
 * read from DEVICE memory (idx[2] int32, g[2] fp32; NULL = empty set), so a
 * router output can feed the switch with no host synchronisation.  Each
 * slot's product is accumulated separately in fp32 and scaled by s*g_k in
 * fp32; the old and new halves use the same expression, so a switch to the
 * same set leaves W bitwise unchanged.
 * A set with an index outside [-1, E) or a non-finite gate on a used slot is
 * rejected on the device: no weight is written and the handle's error word is
 * set (read it with dlm_layers_status).
 * No allocation; one launch on `stream`.  Reads the packed A copy where the
 * handle keeps one, so A banks changed after create need dlm_layers_repack.
 */
int dlm_switch(dlm_layers* h, const int32_t* old_idx, const float* old_g,
               const int32_t* new_idx, const float* new_g, void* stream);

/* Number of kernel launches one dlm_switch call makes (always 1). */
int dlm_switch_launches(const dlm_layers* h);

/* -------------------------------------------- merged-weight products */

/*
 * The decode step after a switch: each adapted projection is the product of
 * its merged weight with the layer input, y_i = W_i x_i (Chinese digest,
 * "technical framework": the fused kernel merges the selected adapters into
 * the backbone and carries out the computation in a single kernel).
 *
 * Bind one input and one output vector to every weight of the handle:
 *   x (host) [n] device pointers, x_i [d_in_i] in the handle's dtype (bf16:
 *   16-byte aligned); y (host) [n] device pointers, y_i [d_out_i] fp32, not
 *   overlapping x_i or W_i.  The device is synchronised first (launches in
 *   flight on any stream finish with the previous binding), then the pointers
 *   are copied into the device table; the buffers stay owned by the caller.  bf16 handles with
 *   r <= 16 also get a partial-product buffer (sum of ceil(d_in_i/256) *
 *   d_out_i floats), and every handle a buffer for dlm_gemv_unmerged's rank
 *   vectors (sum of ceil(d_in_i/2048) * 2 r floats), freed by destroy.
 *   Binding again replaces the vectors.
 */
int dlm_layers_bind_vectors(dlm_layers* h, const void* const* x, float* const* y);

/*
 * y_i = W_i x_i for every weight (fp32 accumulation, one rounding to fp32 per
 * lane sum, then a fixed-order reduction: bitwise reproducible).  One launch,
 * no allocation.  DLM_EINVAL if no vectors are bound.
 */
int dlm_gemv(dlm_layers* h, void* stream);

/*
 * dlm_switch followed by y_i = W'_i x_i with the new (rounded) weights.  bf16
 * with r <= 16: one fused kernel reads each W once, writes W' and forms
 * per-256-column partial products, and a second launch adds each row's
 * partials in column order.  Otherwise the switch and dlm_gemv's kernel run
 * back to back.  Two launches either way, no allocation.  A set the switch
 * rejects leaves W and y unchanged (the error word is set as for dlm_switch).
 */
int dlm_switch_gemv(dlm_layers* h, const int32_t* old_idx, const float* old_g,
                    const int32_t* new_idx, const float* new_g, void* stream);

/* Number of kernel launches one dlm_switch_gemv call makes (always 2). */
int dlm_switch_gemv_launches(const dlm_layers* h);

/*
 * The decode product with one set's adapters left unmerged: for every weight
 * with its bound vectors,
 *   y_i = W_i x_i + s * sum_k g_k * B_{e_k,i} (A_{e_k,i} x_i)          (fp32 y)
 * W is not modified.  The set is made once per token and applied by every
 * adapted layer (AdaFuse, KR digest section 2-ga, token-level pre-gating); the
 * adapters are the per-row gated LoRA product of the SGMM formula, applied
 * to the token's input here instead of merged into W.
 *   idx [2] int32, g [2] fp32 (device): the set, in dlm_switch's format.
 * Two launches, no allocation: the rank vectors' partials A_e x per (weight,
 * 2048-wide K slice, group of 8 rank vectors) into the handle's buffer
 * (dlm_layers_bind_vectors), then the product, each output row adding its adapters' B row times the slices'
 * sum (slices added in order; every result bitwise reproducible, and the
 * same for the set's two slots in either order).  A set dlm_switch would
 * reject leaves y unchanged and sets the error word (dlm_layers_status).
 * DLM_EINVAL if no vectors are bound or idx / g is null.
 */
int dlm_gemv_unmerged(dlm_layers* h, const int32_t* idx, const float* g, void* stream);

/* Number of kernel launches one dlm_gemv_unmerged call makes (always 2). */
int dlm_gemv_unmerged_launches(const dlm_layers* h);

/*
 * Synchronise `stream`, then read and clear the handle's device error word:
 * *code (host) = DLM_OK or DLM_EDEVICE.
 */
int dlm_layers_status(dlm_layers* h, int32_t* code, void* stream);

/* ------------------------------------------------------------------- SGMM */

/*
 * Workspace bytes dlm_sgmm / dlm_sgmm_group_run need for T rows, problems with
 * d_in up to d_in_max, E experts, rank r and n_problems problems sharing one
 * set of rows: row segmentation, the shrink's per-K-slice partial results
 * (fp32, [n_problems][ceil(d_in_max / 2048)][T][2][r]) and the device status
 * word.  *bytes is host memory.
 */
int dlm_sgmm_workspace_size(int64_t T, int64_t d_in_max, int32_t E, int32_t r,
                            int32_t n_problems, size_t* bytes);

/*
 * Batched unmerged adapters for rows with different expert sets:
 *   y[t] <- round( y[t] + sum_k s*g[t][k] * B_{idx[t][k]} (A_{idx[t][k]} x[t]) )
 *   x [T][d_in], y [T][d_out] (in place, must not overlap x),
 *   idx [T][2] int32 (-1 = empty slot), g [T][2] fp32,
 *   A [E][r][d_in], B [E][d_out][r].
 * Launches: segment (rows sorted by their unordered expert pair, 32-row
 * tiles, the experts each tile uses; a per-1024-row count launch first when
 * T > 8192), shrink (v = x A^T on the tile's experts
 * over 2048-wide K slices staged through LDS 512 columns at a time, bf16
 * MFMA, fp32 partial results kept in the workspace), a K-slice sum in a fixed
 * order (only when d_in > 2048 and r > 64) and
 * expand (y += (s g v) B^T, MFMA with v*s*g split into two bf16 terms, fp32
 * accumulate, one bf16 rounding of y; up to rank 64 it adds the K slices'
 * partials of its tile itself, in the same fixed order).  A bf16 call with at most 4 rows (a
 * decode step) skips the segmentation: with one problem a single launch, in
 * which each 1024-column group computes the rows' rank vectors (fp32 dot
 * products over all of K) and adds s*g*v*B^T to its columns with one rounding;
 * with several, one launch for the rank vectors per 2048-wide K slice and one
 * for the columns.  A bf16 call with 5 to 64 rows and no K-slice sum launch
 * has no segmentation launch either: every shrink and expand workgroup orders
 * the rows itself, in the same order (one wave, one row per lane), so the
 * results are those of the segmented launches bit for bit.  Results are
 * bitwise reproducible run to run.
 * Rows whose two slots are empty are not touched.
 * A row with an index outside [-1, E) or a non-finite gate on a used slot makes
 * the whole call a no-op on y and sets the workspace status word (read it with
 * dlm_sgmm_status).
 * bf16: x, y, A, B 16-byte aligned; d_in and d_out multiples of 8.
 * workspace: >= dlm_sgmm_workspace_size(T, d_in, E, r, 1) bytes, 256-byte aligned.
 * T = 0 enqueues nothing and looks at no buffer (they may be null).
 */
int dlm_sgmm(const void* x, const int32_t* idx, const float* g, const void* A,
             const void* B, void* y, int64_t T, int64_t d_in, int64_t d_out, int32_t E,
             int32_t r, float scale, int32_t dtype, void* workspace, size_t ws_bytes,
             void* stream);

/*
 * dlm_sgmm for callers that cannot allocate device memory at all (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches and results as dlm_sgmm, with the workspace in
 * the library's own scratch array instead of a caller buffer.  The array is a
 * static device array of DLM_SGMM_NOALLOC_SCRATCH_BYTES, held by every device
 * that loads the library until the process ends; its device address is looked
 * up on the first call on a device (which is when the runtime places the array
 * in that device's memory).  The call itself allocates nothing.
 *   status (device, may be NULL): receives 0 when every row's set was valid,
 *     nonzero when the device rejected one (then y is left unchanged) -- the
 *     workspace status word of dlm_sgmm, written where the caller can read it.
 * Every other argument as for dlm_sgmm.  `stream` must belong to the current
 * device (DLM_EINVAL otherwise).  A call whose workspace
 * (dlm_sgmm_workspace_size(T, d_in, E, r, 1)) exceeds the array returns
 * DLM_EWORKSPACE before anything is enqueued.
 * All calls on one device share that device's array and each call overwrites
 * it: calls that can overlap on one device (different streams, or several host
 * threads) race and give wrong results; order them on one stream.
 */
#define DLM_SGMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dlm_sgmm_noalloc(const void* x, const int32_t* idx, const float* g, const void* A,
                     const void* B, void* y, int64_t T, int64_t d_in, int64_t d_out, int32_t E,
                     int32_t r, float scale, int32_t dtype, int32_t* status, void* stream);

/* One problem of a grouped SGMM: every problem shares the rows' sets. */
typedef struct {
    const void* x;  /* [T][d_in] */
    const void* A;  /* [E][r][d_in] */
    const void* B;  /* [E][d_out][r] */
    void* y;        /* [T][d_out], in place */
    int64_t d_in;
    int64_t d_out;
} dlm_sgmm_problem;

typedef struct dlm_sgmm_group dlm_sgmm_group;

/*
 * Register n problems (e.g. every adapted projection of every layer) that are
 * run together on the same rows' expert sets: the decide-once routing means
 * one segmentation serves all of them.  Copies the descriptors (host) to a
 * small device table; x, B and y stay owned by the caller and are used in place.
 * bf16: the handle also keeps a packed copy of every distinct A bank
 * (Ap[e][k/8][rho][8] = A[e][rho][k..k+8), the same size as A, allocated and
 * filled here; the device is synchronised before returning), so that the shrink
 * reads A in contiguous runs.  The copy is taken at create time: after
 * changing an A bank in place call dlm_sgmm_group_repack.
 */
int dlm_sgmm_group_create(const dlm_sgmm_problem* probs, int32_t n, int32_t E, int32_t r,
                          float scale, int32_t dtype, dlm_sgmm_group** out);
int dlm_sgmm_group_destroy(dlm_sgmm_group* h);

/*
 * Refresh the handle's packed A copies from the caller's A banks: one launch
 * per distinct bank on `stream`, no allocation (no-op for fp32 groups).
 */
int dlm_sgmm_group_repack(dlm_sgmm_group* h, void* stream);

/*
 * Run every problem of the group for T rows: one segment launch shared by all
 * problems (none up to 64 rows without a K-slice sum, as for dlm_sgmm), then
 * one shrink, one K-slice sum (only when some d_in > 2048 and r > 64) and one
 * expand launch covering all problems.
 * workspace: >= dlm_sgmm_workspace_size(T, max d_in, E, r, n_problems) bytes.
 */
int dlm_sgmm_group_run(dlm_sgmm_group* h, const int32_t* idx, const float* g, int64_t T,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * Synchronise `stream`, then read and clear the workspace status word:
 * *code (host) = DLM_OK or DLM_EDEVICE.  Besides a rejected expert set, the
 * one-launch shrink + expand sets it if an expand work item waited about a
 * second for its shrink items (status 2) or found they ran on another XCD
 * (status 3); y is then not to be trusted.  Neither happens when the device
 * starts workgroups in order and round-robin over its XCDs.
 */
int dlm_sgmm_status(void* workspace, int32_t* code, void* stream);

/*
 * Number of kernel launches one dlm_sgmm, dlm_sgmm_noalloc or
 * dlm_sgmm_group_run call makes for T rows and n_problems problems of rank r
 * with d_in up to d_in_max: 0 for T = 0; for bf16 with T <= 4, 1 (one problem)
 * or 2; for bf16 up to rank 64 with n_problems x ceil(T / 32) >= 256 (and
 * d_in_max up to 4095 x 2048), the segmentation (2 launches when T > 8192,
 * else 1) and one launch running the shrink and the expand; otherwise for bf16
 * with T <= 64 and no K-slice sum, 2 (shrink and expand); else the
 * segmentation, the shrink, the K-slice sum (bf16 with d_in_max > 2048 and
 * r > 64 only) and the expand.  Returns -1 (with the last
 * error set) for a negative T, d_in_max < 1, r outside [1, DLM_MAX_RANK],
 * n_problems < 1 or an unknown dtype.
 */
int dlm_sgmm_launches(int64_t T, int64_t d_in_max, int32_t r, int32_t n_problems, int32_t dtype);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H */
