/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN forward.
 *
 * The forward of one MoE FFN layer on one GPU, in five steps:
 *   route      per token, softmax over E router logits, top-k, renormalise;
 *   permute    stable counting sort of the T*k (token, slot) pairs by expert and
 *              a row gather into expert-contiguous order;
 *   GEMM1      per expert, [gate | up] = x W1^T, h = silu(gate) * up (SwiGLU);
 *   GEMM2      per expert, y = h W2^T;
 *   combine    per token, out = sum over its k slots of w_j * y_j.
 * The steps follow the fused MoE kernels described on the FlashInfer pull request
 * "[SM90] Add W4A8 MegaMoE support" (dispatch, two expert GEMMs, clamped SwiGLU,
 * top-k reduction), the GEMM + SwiGLU fused MLP of Megatron-LM "Support GEMM +
 * Swiglu fused MLP", and the permute / unpermute fused into dispatch / combine of
 * Megatron-LM "add permute fusion into hybrid ep".
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless a parameter says otherwise; the problem
 *    and weight descriptors themselves are host structs.
 *  - `stream` is a hipStream_t (NULL = the null stream); the header declares the
 *    handle type itself (an opaque pointer, the same typedef as HIP's), so a caller
 *    needs no HIP header.  Every call enqueues its kernels on that stream and
 *    returns; none synchronises, allocates device memory, or keeps a pointer after
 *    it returns.  Buffers must stay alive until the stream has executed the work.
 *    Weights are borrowed, never copied (the FlashInfer Usage section: buffers are
 *    allocated by the caller before graph capture).
 *  - All arrays are row-major with the last index contiguous.  bf16 is passed as
 *    raw 16-bit patterns, fp8 as OCP E4M3FN bytes, fp4 as OCP E2M1 nibbles.
 *  - Argument checks run on the host before anything is enqueued and read no
 *    device memory; a failed check enqueues nothing.  T == 0 is valid and
 *    enqueues nothing.  Device-side preconditions (not checked): logits finite;
 *    tables consistent with one another; every array holds at least the bytes its
 *    description gives for the problem's precision and weight layout (the library
 *    sees pointers only: a bf16 problem over fp8 / fp4 buffers reads past them).
 *    Expert ids outside [0, E) are treated as -1 (dropped) by every kernel that
 *    reads them.
 *  - Return value: a moe_status; MOE_ERR_HIP means a launch failed, and
 *    moe_last_hip_error() gives its hipError_t code.
 *  - The library is stateless; calls on different streams may run concurrently
 *    when they use disjoint buffers and workspaces.
 */
#ifndef TPG_MOE_H
#define TPG_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (hip_runtime_api.h declares the same typedef). */
typedef struct ihipStream_t *hipStream_t;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a size is out of range (see moe_problem) */
    MOE_ERR_UNSUPPORTED = 3, /* an option value this library does not implement */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = 5,         /* a kernel launch failed */
    MOE_ERR_SCRATCH = 6      /* moe_forward_noalloc: the problem needs more than MOE_NOALLOC_SCRATCH_BYTES */
} moe_status;

/* Arithmetic of the expert GEMMs. */
enum {
    /* x bf16 [T][H]; W1 bf16 [E][2I][H]; W2 bf16 [E][H][I]; fp32 accumulation;
     * h and y rounded to bf16 (round to nearest even); out bf16 [T][H]. */
    MOE_PREC_BF16 = 0,
    /* FlashInfer "[SM90] Add W4A8 MegaMoE support", Usage section: FP8 E4M3
     * activations with one fp32 scale per 128 channels; NVFP4 weights = E2M1 codes
     * packed two per byte (low nibble = even K index, follow-up #6517 point 4), one
     * E4M3 scale per 16 values along K, and one fp32 global scale per expert and
     * matrix.  Each weight is dequantised in-kernel to FP8 (e2m1 * scale rounded to
     * E4M3) and multiplied on FP8 matrix cores; h is re-quantised to FP8 per
     * (row, 128 columns) with s = amax/448 (the split family's note that the
     * second GEMM's activation scales are per 128 like the first's).  out bf16. */
    MOE_PREC_W4A8 = 1,
    /* The same with MXFP4 weights (the Usage section's "E8M0 per 32 values"): E2M1
     * codes packed as above, one E8M0 scale (2^(code - 127)) per 32 values along K,
     * and one fp32 global scale per expert and matrix.  The codes and their scales
     * go to the FP4 matrix cores as they are: each product e2m1 * 2^s * fp8 is exact
     * (no FP8 rounding of the weight, so no scale-range limit). */
    MOE_PREC_W4A8_MX = 2
};

/* Selects which call moe_call_workspace_bytes() sizes the workspace for. */
enum { MOE_WS_PERMUTE = 0, MOE_WS_GROUPED_FFN = 1, MOE_WS_FORWARD = 2 };

typedef struct moe_problem {
    int32_t T;              /* tokens, >= 0 */
    int32_t H;              /* hidden size, multiple of 128 (W4A8, W4A8_MX: of 256), 128..65536 */
    int32_t I;              /* per-expert intermediate size, multiple of 128 (W4A8, W4A8_MX: of 256);
                               one expert matrix (2*I*H bf16) must be below 2 GB */
    int32_t E;              /* experts, 1..256 */
    int32_t k;              /* experts per token, 1..E; T*k < 2^31 */
    int32_t prec;           /* MOE_PREC_BF16, MOE_PREC_W4A8 or MOE_PREC_W4A8_MX */
    /* Megatron-LM "Support GEMM + Swiglu fused MLP", option
     * moe_mlp_glu_interleave_size: 0 = W1 rows are [gate (I rows) | up (I rows)]
     * (the fused fc1 layout in Megatron-LM PR #5984's log); 32 = stored row
     * 64q + r is gate row 32q + r for r < 32 and up row 32q + r - 32 otherwise. */
    int32_t glu_interleave;
    /* 0 = plain SwiGLU; c > 0 = clamp both gate and up to [-c, c] before the
     * activation ("ClampedSwiGLU" in Megatron-LM PR #5984's log; the clamped
     * SwiGLU of the FlashInfer fused kernel). */
    float swiglu_clamp;
    /* 0, MOE_FLAG_SINGLE_LAUNCH or MOE_FLAG_SCATTER_Y (moe_forward only; one at a time). */
    int32_t flags;
} moe_problem;

/* moe_forward runs the whole W4A8 forward (routing, tables, both GEMMs with the SwiGLU and
 * the re-quantisation, the combine) in one persistent launch, as the FlashInfer fused kernel
 * does through 256 tokens per rank (its opening description and Usage section).  Needs
 * MOE_PREC_W4A8 or MOE_PREC_W4A8_MX, T <= 256, T*k <= 2048, H and I multiples of 1024, and
 * every weight array below 2 GB (else MOE_ERR_UNSUPPORTED).  Bitwise the same output as the
 * default multi-launch forward.  Workgroups hand work to each other through counters in the
 * workspace, which the kernel resets itself (graph replay works); every wait is bounded.  On
 * this library's kernels it is slower than the default path, which stays the default. */
#define MOE_FLAG_SINGLE_LAUNCH 1

/* moe_forward stores GEMM2's output rows in slot order instead of expert order: row r of the
 * expert-major order goes to row row_src[r] = t*k + j of the workspace's y buffer (dropped
 * slots' rows stay unwritten), and the combine reads a token's k rows as one contiguous run.
 * This is the second kernel of the FlashInfer split family ("[SM90] Add W4A8 MegaMoE support",
 * the commit that adds the BN128 split family: the second GEMM with a contiguous scatter), and
 * the unpermute folded into the producer as Megatron-LM "add permute fusion into hybrid ep"
 * folds it.  Any precision; not with MOE_FLAG_SINGLE_LAUNCH (MOE_ERR_UNSUPPORTED).  Bitwise the
 * same output as the default forward (the same rows, summed in the same order).  On MI355X the
 * combine gains 2-5 % from it and GEMM2's scattered row stores lose about as much (whole
 * forward within noise on the bf16 and W4A8 layers), so the default stays the expert order. */
#define MOE_FLAG_SCATTER_Y 2

/* Expert weights (device pointers, borrowed).  bf16: only w1 and w2 are used.
 * w4a8: w1 uint8 [E][2I][H/2], w1_bscale uint8 [E][2I][H/16], w1_gscale fp32 [E];
 *       w2 uint8 [E][H][I/2],  w2_bscale uint8 [E][H][I/16],  w2_gscale fp32 [E].
 * w4a8_mx: the same with w1_bscale uint8 [E][2I][H/32], w2_bscale uint8 [E][H][I/32].
 * w4_layout (W4A8 and W4A8_MX only) says how the codes and block scales of each
 * matrix are stored: MOE_W4_LAYOUT_ROWS, the row-major arrays above, or
 * MOE_W4_LAYOUT_TILED, the same bytes regrouped by moe_w4a8_tile_weights so that
 * the GEMMs stream every 32-row, 256-wide piece as one contiguous run already in their
 * matrix instructions' operand order (the FlashInfer Usage section likewise prepares
 * weights once with a transform function), NVFP4 codes also reordered within each 4-byte
 * group so that the in-kernel dequant yields K order directly.  Both give bitwise the same
 * results. */
enum { MOE_W4_LAYOUT_ROWS = 0, MOE_W4_LAYOUT_TILED = 1 };
typedef struct moe_weights {
    const void *w1;
    const void *w1_bscale;
    const float *w1_gscale;
    const void *w2;
    const void *w2_bscale;
    const float *w2_gscale;
    int32_t w4_layout;
} moe_weights;

/* Host only.  Bytes of device workspace that serve every entry point for this
 * problem (the largest plan: moe_forward's); 0 if the problem is invalid.  The
 * size depends only on the problem, never on the routing, so one allocation made
 * before graph capture serves every call of that shape (the FlashInfer pull request
 * "[SM90] Add W4A8 MegaMoE support" sizes its workspace for the largest plan, and
 * its Usage section has the caller allocate it before capture).  Workspace
 * contents need not be initialised and are not preserved between calls. */
size_t moe_workspace_bytes(const moe_problem *p);

/* Host only.  The smaller workspace one step entry point needs (MOE_WS_PERMUTE for
 * moe_permute, MOE_WS_GROUPED_FFN for moe_grouped_ffn, MOE_WS_FORWARD as
 * moe_workspace_bytes); 0 if the problem or `which` is invalid. */
size_t moe_call_workspace_bytes(const moe_problem *p, int which);

/* Host only.  Static English text for a moe_status value. */
const char *moe_status_str(int status);

/* Host only.  The hipError_t code behind the calling thread's most recent
 * MOE_ERR_HIP (0 if there was none). */
int moe_last_hip_error(void);

/* Route.  logits fp32 [T][E]; slot_drop uint8 [T][k] or NULL (nonzero = the
 * slot is routed to no local expert, as the FlashInfer Usage section's "-1 masks
 * a route").  Writes topk_idx int32 [T][k] (expert ids by descending logit, ties
 * to the lower id; -1 where dropped) and topk_w fp32 [T][k] (softmax over all E,
 * restricted to the k chosen and renormalised to sum to 1; a dropped slot keeps
 * its weight and is skipped by the combine). */
int moe_route_topk(const float *logits, const uint8_t *slot_drop, const moe_problem *p, int32_t *topk_idx,
                   float *topk_w, hipStream_t stream);

/* Permute.  From topk_idx int32 [T][k] builds the tables
 *   offsets int32 [E+1]  exclusive prefix of the expert counts (offsets[E] = R,
 *                        the number of non-dropped slots);
 *   row_src int32 [T*k]  row r < R holds slot s = t*k + j; rows are grouped by
 *                        expert and ascending in s within an expert; -1 for r >= R;
 *   slot_row int32 [T*k] inverse: row of slot s, or -1 if the slot is dropped;
 * and gathers x_perm[r] = x[row_src[r] / k] for r < R (bf16 [T*k][H], or for
 * W4A8 fp8 [T*k][H] plus x_perm_scale fp32 [T*k][H/128] from x_scale
 * [T][H/128]).  Rows r >= R of x_perm are not written.  The tables are a pure
 * function of topk_idx (bit-exact, deterministic). */
int moe_permute(const void *x, const float *x_scale, const int32_t *topk_idx, const moe_problem *p,
                int32_t *offsets, int32_t *row_src, int32_t *slot_row, void *x_perm, float *x_perm_scale, void *ws,
                size_t ws_bytes, hipStream_t stream);

/* moe_permute with timing marks: identical work, plus hipEventRecord of
 * stage_events[i] (MOE_N_PERMUTE_EVENTS hipEvent_t handles, created by the
 * caller) on `stream`: [0] tables [1] row gather [2].  For measurement of the
 * gather kernel on its own (moe_forward folds the gather into the first GEMM, see
 * moe_forward). */
#define MOE_N_PERMUTE_EVENTS 3
int moe_permute_timed(const void *x, const float *x_scale, const int32_t *topk_idx, const moe_problem *p,
                      int32_t *offsets, int32_t *row_src, int32_t *slot_row, void *x_perm, float *x_perm_scale,
                      void *ws, size_t ws_bytes, hipStream_t stream, void *const *stage_events);

/* Grouped expert FFN: the two expert GEMMs with the SwiGLU between them (the
 * FlashInfer fused kernel's two FFN GEMMs and clamped SwiGLU; the GEMM + SwiGLU
 * fused MLP of Megatron-LM "Support GEMM + Swiglu fused MLP", whose
 * moe_mlp_glu_interleave_size option glu_interleave follows).
 * For every expert e and row r in [offsets[e], offsets[e+1]):
 * y_perm[r] = (silu(g) * u) W2_e^T with [g | u] = x_perm[r] W1_e^T (clamped if
 * swiglu_clamp > 0).  x_perm as produced by moe_permute; y_perm bf16 [T*k][H];
 * rows >= offsets[E] are not written.  Needs ws of at least
 * moe_call_workspace_bytes(p, MOE_WS_GROUPED_FFN) bytes (holds h and the tile list). */
int moe_grouped_ffn(const void *x_perm, const float *x_perm_scale, const int32_t *offsets, const moe_weights *w,
                    const moe_problem *p, void *y_perm, void *ws, size_t ws_bytes, hipStream_t stream);

/* Unpermute and combine: the top-k reduction that ends the FlashInfer fused MoE
 * (-1 routes skipped), with the unpermute folded in as Megatron-LM "add permute
 * fusion into hybrid ep" folds it into the combine:
 * out[t] = bf16( sum_{j=0..k-1, slot_row[t*k+j] >= 0}
 * topk_w[t][j] * y_perm[slot_row[t*k+j]] ), accumulated in fp32 in ascending j
 * with no atomics (deterministic).  A token whose slots are all dropped gets 0. */
int moe_unpermute_combine(const void *y_perm, const int32_t *slot_row, const float *topk_w, const moe_problem *p,
                          void *out, hipStream_t stream);

/* The whole forward: route, permute, grouped FFN, combine, on one stream, with
 * every intermediate in ws (at least moe_workspace_bytes(p)).
 * Whenever the byte offsets into x fit 31 bits (T*H*2 < 2^31 for bf16, T*H < 2^31
 * for W4A8) the row gather is folded into GEMM1, which reads row r of the
 * expert-major order (and, for W4A8, its activation scales) straight from
 * x[row_src[r] / k] (the permute fused into the expert kernel, as Megatron-LM "add
 * permute fusion into hybrid ep" fuses it into dispatch); no x_perm is written and
 * the workspace holds none.  The result is bitwise the same as moe_permute +
 * moe_grouped_ffn + moe_unpermute_combine. */
int moe_forward(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                const moe_weights *w, const moe_problem *p, void *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward with timing marks: identical work, plus hipEventRecord of
 * stage_events[i] (MOE_N_STAGE_EVENTS hipEvent_t handles, created by the caller)
 * on `stream` at each stage boundary:
 *   [0] route [1] permutation tables [2] row gather [3] GEMM tile list [4]
 *   GEMM1 + SwiGLU [5] GEMM2 [6] combine [7]
 * (for W4A8 the two GEMMs run between marks 4 and 5 and mark 6 follows at once;
 * where the gather is folded into GEMM1, mark 3 follows mark 2 at once; the tile
 * list is written by the tables' launches, so mark 4 follows mark 3 at once; for
 * at most 1024 slots and 256 tokens one launch routes and builds the tables and the
 * tile list, between marks 0 and 1).
 * For measurement; the marks add no work to the kernels. */
#define MOE_N_STAGE_EVENTS 8
int moe_forward_timed(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                      const moe_weights *w, const moe_problem *p, void *out, void *ws, size_t ws_bytes, hipStream_t stream,
                      void *const *stage_events);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The intermediates live in a scratch array the library holds
 * in device memory, MOE_NOALLOC_SCRATCH_BYTES on each GPU it runs on (allocated
 * with the library's code on that GPU, kept until the process ends; its address is
 * looked up on the first call for a device, which should therefore not be made
 * under graph capture).  The call allocates nothing.  Returns MOE_ERR_SCRATCH when
 * moe_workspace_bytes(p) exceeds the scratch (it covers, e.g., the W4A8 layer with
 * H = 7168, I = 2048, E = 32, top-8 up to 256 tokens).  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap in time on one GPU (different streams
 * without ordering between them) race and give undefined results.  Otherwise the
 * same work and bitwise the same output as moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                        const moe_weights *w, const moe_problem *p, void *out, hipStream_t stream);

/* Diagnostic: the W4A8 dequant of every (e2m1 code, e4m3 block scale s) pair at
 * every nibble position, through the same device routine as the W4A8 GEMMs
 * (FlashInfer #6343: NVFP4 -> FP8 dequant; e2m1 value times scale, rounded to
 * nearest even, saturating at +-448).  out8 is uint8 [8][16][256] (device):
 * a dword holding code (c + p) mod 16 at nibble position p = 0..7 (low nibble
 * first) is dequantised with scale s, and out8[p][c][s] receives result byte p,
 * so out8[p][c][s] is the e4m3 code of code (c + p) mod 16 times scale s.  A NaN
 * block scale, outside the defined domain, gives the NaN code with the product's
 * sign. */
int moe_w4a8_dequant_table(uint8_t *out8, hipStream_t stream);

/* W4A8 weight preparation: one matrix stack of E experts with N rows and K columns
 * (N a multiple of 32, K of 256), row-major codes uint8 [E][N][K/2] and block scales
 * uint8 [E][N][K/bs] (bs = 16 for MOE_PREC_W4A8, 32 for MOE_PREC_W4A8_MX), rewritten
 * into MOE_W4_LAYOUT_TILED: every expert e's 32-row block b and 256-wide K piece c is one
 * contiguous run (4096 code bytes at codes_tiled + ((e N/32 + b) K/256 + c) 4096, and
 * 32 x 256/bs scale bytes at the same piece index times that size in bscale_tiled), stored in
 * the order in which the GEMMs' matrix instructions take it: with row r < 32, the 16-byte
 * granule g < 8 of the row's 128 code bytes of the piece, q = g / 4, h = (g / 2) % 2,
 * t = g % 2, sits at byte 1024 (2 q + t) + 16 (32 h + r) of the piece's codes; scale byte j of
 * the row's piece sits, for MOE_PREC_W4A8 (16 per row; j = 8 q + 4 h + u, u < 4), at byte
 * 8 (32 h + r) + 4 q + u, and for MOE_PREC_W4A8_MX (8 per row; j = 4 q + 2 h + u, u < 2) at
 * byte 4 (32 h + r) + 2 q + u (the same array sizes).  For MOE_PREC_W4A8 each 4-byte group
 * of codes, which holds the codes of 8 consecutive K positions k0..k0+7, also stores k0 + i in
 * the low nibble and k0 + 4 + i in the high nibble of its byte i (the row-major bytes hold
 * k0 + 2i and k0 + 2i + 1).  MXFP4 codes keep the row-major packing.  Device pointers; the outputs must not overlap the inputs;
 * enqueued on `stream`.  Call it once per matrix (W1: N = 2I, K = H; W2: N = H, K =
 * I) when the weights are loaded. */
int moe_w4a8_tile_weights(const void *codes, const void *bscale, void *codes_tiled, void *bscale_tiled,
                          int32_t E, int32_t N, int32_t K, int32_t prec, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TPG_MOE_H */
