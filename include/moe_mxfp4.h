/*
 * moe_mxfp4.h - C ABI of the fused MXFP4 Mixture-of-Experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * One call runs the whole layer on one GPU stream:
 *   1. top-k routing from router logits (softmax over the selected experts),
 *      or caller-given top-k ids and weights;
 *   2. the shared-expert append: S extra columns per token with weight
 *      sigmoid(bf16 logit) * shared_scale ("SGLang MoE shared-expert
 *      optimisation", the fused append kernel);
 *   3. the map of global ids to the local range [expert_offset,
 *      expert_offset + E) with -1 for other ids, and a deterministic sort of
 *      the token slots into per-expert rows and B-row chunks ("Generalizing
 *      the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape template",
 *      sections 1 and 5; "SGLang CUTLASS MoE", section 1);
 *   4. a device-side choice between the split and the dense GEMM2 path
 *      ("Device-side gating of the MoE GEMM2 path", sections 1-2);
 *   5. the gathered grouped GEMM1 against MXFP4 W13 with SwiGLU (optional
 *      clamp) fused ("SGLang CUTLASS MoE", section 4; Shape-template page,
 *      section 4);
 *   6. the grouped GEMM2 against MXFP4 W2;
 *   7. the routing-weighted sum back to token order ("SGLang CUTLASS MoE",
 *      section 5).
 *
 * Conventions for every function:
 *   - Pointers named *_dev are device pointers; the caller owns all memory.
 *     The library never allocates, frees, synchronises or reads device
 *     memory from the host, so a forward call can be captured in a graph.
 *   - Shapes are passed by host pointer and read during the call only.
 *   - Every function returns MOE_OK (0) or one of the MOE_ERR_* codes below;
 *     validation errors are returned before anything is enqueued.
 *   - Nibble-packed operands hold two E2M1 codes per byte, the low nibble
 *     being the element with the even K index. Scales are E8M0 bytes
 *     (value 2^(e-127)), one per 32 consecutive K elements.
 *   - Activations, router inputs, scales and outputs are row-major. The
 *     weight codes w13 and w2 are read in the packed layout that
 *     moe_mxfp4_prepack writes from the row-major one; the shape's
 *     weight_layout field states it (MOE_WEIGHTS_PACKED), and a forward call
 *     tagged otherwise is rejected before any launch.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID 1     /* null or inconsistent arguments */
#define MOE_ERR_UNSUPPORTED 2 /* shape outside the supported range */
#define MOE_ERR_WORKSPACE 3   /* workspace too small or not 256-byte aligned */
#define MOE_ERR_HIP 4         /* a kernel launch failed */
#define MOE_ERR_SCRATCH 5     /* workspace beyond what moe_mxfp4_forward_noalloc holds */

/* Activation kinds. */
#define MOE_ACT_SWIGLU 0 /* act = silu(g) * u on the gate half g, up half u */
#define MOE_ACT_SITU 1   /* act = beta tanh(g/beta) sigmoid(g) * lb tanh(u/lb): the
                            SiTU activation of the Kimi-K3.1 decode page, section 4
                            (printed there for beta = 4, lb = 25) */

/* Activation (A operand) formats. */
#define MOE_ADTYPE_BF16 0  /* W4A16: bf16 activations, bf16 MFMA */
#define MOE_ADTYPE_MXFP8 1 /* W4A8: activations quantised to MXFP8 (E4M3 elements,
                              one E8M0 per 32 K), scaled f8f6f4 MFMA */
#define MOE_ADTYPE_MXFP4 2 /* W4A4: activations quantised to MXFP4 (E2M1 elements,
                              one E8M0 per 32 K), scaled f8f6f4 MFMA with both
                              operands E2M1 ("SGLang CUTLASS MoE", section 6: FP4
                              activations; here in the weights' MX block format) */

/* Layout of the weight codes w13_dev / w2_dev (moe_mxfp4_shape.weight_layout).
 * MOE_WEIGHTS_ROW_MAJOR: [E', rows, K/2] row-major, as drawn or stored; the
 * forward calls do not read it (MOE_ERR_UNSUPPORTED): pass it through
 * moe_mxfp4_prepack once, when the weights are loaded.
 * MOE_WEIGHTS_PACKED: the output of moe_mxfp4_prepack (1 KB blocks of 16 rows
 * x 64 bytes), the only layout the forward calls read. The repack is the kind
 * the Marlin MoE kernel page (section 2) applies to its MXFP4 weights so that
 * its loads match the MMA fragments. */
#define MOE_WEIGHTS_ROW_MAJOR 0
#define MOE_WEIGHTS_PACKED 1

/* GEMM2 path forcing (tests): -1 lets the device gate decide. */
#define MOE_GEMM2_AUTO (-1)
#define MOE_GEMM2_SPLIT 0
#define MOE_GEMM2_DENSE 1

/*
 * Layer shape. The Shape template of the Kimi-K3.1 decode page (section 1)
 * fixes (experts, top-k, hidden, inter, BlockN) at compile time; here they
 * are run-time fields, checked by moe_mxfp4_query.
 *
 *   T               tokens (0 allowed: the call does nothing)
 *   E               local routed experts
 *   E_global        global routed experts: width of the router logits and
 *                   range of routed ids
 *   topk            routed experts per token, 1..32
 *   S               shared experts appended per token, 0..8; their weights
 *                   sit after the E routed experts in w13/s13/w2/s2
 *   H, I            hidden and intermediate sizes; H % 512 == 0, I % 128 == 0,
 *                   both at most 8192
 *   block_n         B: rows per chunk ("virtual expert"). 16 or 32 select the
 *                   decode GEMM1 (tokens on the MFMA N side); 64, 128 or 256
 *                   the prefill GEMM1 (tokens on the M side)
 *   expert_offset   global id of local expert 0
 *   activation      MOE_ACT_SWIGLU or MOE_ACT_SITU
 *   a_dtype         MOE_ADTYPE_BF16, MOE_ADTYPE_MXFP8 (W4A8) or
 *                   MOE_ADTYPE_MXFP4 (W4A4); the MX formats need I <= 512.
 *                   They quantise x (per 32 along H) and the activation
 *                   output act (per 32 along I, before GEMM2) to MXFP8 or
 *                   MXFP4 (shared exponent floor(log2 amax) - 8 or - 2,
 *                   round to nearest even, saturating); the GEMMs run on
 *                   scaled f8f6f4 MFMA with the E2M1 weights fed as they are
 *   force_gemm2_path  MOE_GEMM2_AUTO, _SPLIT or _DENSE
 *   swiglu_limit    > 0: gate = min(gate, L), up = clamp(up, -L, L)
 *                   before silu(gate) * up; <= 0: no clamp
 *   shared_scale    multiplier of the shared-expert sigmoid (1/ep_size on
 *                   the page; 1.0 on one GPU)
 *   act_beta        SiTU gate cap beta (> 0, finite; the K3.1 value is 4)
 *   act_linear_beta SiTU up cap (> 0, finite; the K3.1 value is 25). Both
 *                   are read only for MOE_ACT_SITU, which ignores swiglu_limit
 *   weight_layout   MOE_WEIGHTS_PACKED (required by the forward calls) or
 *                   MOE_WEIGHTS_ROW_MAJOR (accepted by query and
 *                   workspace_layout, which do not read weights); other
 *                   values are MOE_ERR_INVALID
 */
typedef struct moe_mxfp4_shape {
  int32_t T;
  int32_t E;
  int32_t E_global;
  int32_t topk;
  int32_t S;
  int32_t H;
  int32_t I;
  int32_t block_n;
  int32_t expert_offset;
  int32_t activation;
  int32_t a_dtype;
  int32_t force_gemm2_path;
  float swiglu_limit;
  float shared_scale;
  float act_beta;
  float act_linear_beta;
  int32_t weight_layout;
} moe_mxfp4_shape;

/*
 * Byte offsets of the arrays inside the caller's workspace (all 256-byte
 * aligned), as carved by one layout function (the Shape-template page,
 * section 3: one byte tensor holds counters, chunk table, activations).
 * With K' = topk + S, E' = E + S and R_max = T * K':
 *
 *   counters      int32[64]       [0] number of chunks num_v, [1] number of
 *                                 16-row units, [4..7] gate word
 *                                 {path (0 split, 1 dense), touched experts U,
 *                                 rows R, dense tiles}
 *   route_ids     int32[T*topk]   selected global ids (logits mode)
 *   slot_expert   int32[T*K']     local expert of slot t*K'+k, or -1
 *   slot_w        float[T*K']     routing weight of the slot
 *   range_counts  int32[n_ranges*E'] per-slot-range expert counts, then
 *                 each range's first row within the expert (large sorts only)
 *   counts        int32[E']       rows per expert
 *   offsets       int32[E'+1]     first row of each expert; offsets[E'] = R
 *   sorted_slot   int32[R_max]    row -> slot
 *   expanded_idx  int32[T*K']     slot -> row, or -1
 *   vinfo         int32[kmax_v*4] chunk table (expert, first_row, rows, chunk)
 *   dense_tiles   int32[max_dense_tiles*4] dense-path tiles (same fields)
 *   units16       int32[max_units16*4] the rows again in units of at most 16
 *                 (same fields; counters[1] holds their number): the work list
 *                 of the decode GEMMs
 *   act           [rows_pad, I]   bf16 (W4A16) or E4M3 bytes (W4A8), or
 *                 uint8[rows_pad, I/2] E2M1 pairs (W4A4, low nibble first)
 *   act_scales    uint8[rows_pad, I/32] E8M0 (W4A8, W4A4)
 *   y             bf16[rows_pad, H] GEMM2 output in row order
 *   xq, xs        uint8[T, H] (W4A8) or [T, H/2] (W4A4), uint8[T, H/32]:
 *                 MX-quantised x (W4A8, W4A4 only)
 */
typedef struct moe_mxfp4_ws_layout {
  uint64_t total_bytes;
  uint64_t counters;
  uint64_t route_ids;
  uint64_t slot_expert;
  uint64_t slot_w;
  uint64_t range_counts;
  uint64_t counts;
  uint64_t offsets;
  uint64_t sorted_slot;
  uint64_t expanded_idx;
  uint64_t vinfo;
  uint64_t dense_tiles;
  uint64_t units16;
  uint64_t act;
  uint64_t act_scales;
  uint64_t y;
  uint64_t xq;
  uint64_t xs;
  int32_t kmax_v;          /* E' + (T*K') / B: bound on chunks */
  int32_t max_dense_tiles; /* E' + (T*K') / 128 */
  int32_t max_units16;     /* E' + (T*K') / 16 */
  int32_t n_ranges;        /* slot ranges of the large sort */
  int32_t rows_pad;        /* R_max plus padding rows */
} moe_mxfp4_ws_layout;

/*
 * Check a shape and return the workspace size it needs.
 * Host only; touches no device. Returns MOE_OK, MOE_ERR_INVALID (null
 * pointer, negative sizes, offset range outside E_global, unknown
 * weight_layout) or
 * MOE_ERR_UNSUPPORTED (H % 512, I % 128, H or I > 8192, block_n, topk, S, E + S > 2048,
 * T * K' > 2^23, unknown activation or a_dtype, MXFP8 or MXFP4 with I > 512).
 */
int moe_mxfp4_query(const moe_mxfp4_shape* shape, uint64_t* workspace_bytes);

/* The workspace carve for a shape (same checks as moe_mxfp4_query). */
int moe_mxfp4_workspace_layout(const moe_mxfp4_shape* shape, moe_mxfp4_ws_layout* layout);

/*
 * Run the layer on `stream` (a hipStream_t; NULL = the default stream).
 *
 * Inputs (device, read only):
 *   x_dev              bf16 [T, H]
 *   router_logits_dev  float [T, E_global], or NULL when ids are given
 *   topk_ids_dev       int32 [T, topk] global ids (-1 = masked), or NULL
 *   topk_w_dev         float [T, topk], or NULL (given together with ids)
 *   shared_logits_dev  bf16 [T, S] (needed when S > 0, else ignored)
 *   w13_dev            uint8 [E', 2I, H/2]: rows [0, I) gate, [I, 2I) up,
 *                      in the packed layout of moe_mxfp4_prepack (the shape's
 *                      weight_layout must say MOE_WEIGHTS_PACKED)
 *   s13_dev            uint8 [E', 2I, H/32] (row-major, not packed)
 *   w2_dev             uint8 [E', H, I/2], packed like w13_dev
 *   s2_dev             uint8 [E', H, I/32] (row-major, not packed)
 * Output (device): out_dev bf16 [T, H]. Tokens with no local expert get 0.
 * Workspace: workspace_dev, 256-byte aligned, >= moe_mxfp4_query's size;
 * the call overwrites it and its contents after the call are the maps
 * listed in moe_mxfp4_ws_layout.
 *
 * Alignment: x_dev, out_dev, w13_dev, s13_dev, w2_dev and s2_dev 16 bytes;
 * router_logits_dev, topk_ids_dev and topk_w_dev 4 bytes; shared_logits_dev
 * 2 bytes (MOE_ERR_INVALID otherwise). Each input is read only within the
 * sizes listed above.
 *
 * Exactly one of router_logits_dev and (topk_ids_dev, topk_w_dev) must be
 * non-NULL. Errors: MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED (also for
 * weight_layout MOE_WEIGHTS_ROW_MAJOR), MOE_ERR_WORKSPACE before any launch; MOE_ERR_HIP if a launch fails (earlier kernels of the
 * chain may have run). Calls on different streams need different
 * workspaces. Duplicate routed ids within a token (possible only in ids
 * mode) each get their own row.
 */
int moe_mxfp4_forward(const void* x_dev, const float* router_logits_dev,
                      const int32_t* topk_ids_dev, const float* topk_w_dev,
                      const void* shared_logits_dev, const uint8_t* w13_dev,
                      const uint8_t* s13_dev, const uint8_t* w2_dev, const uint8_t* s2_dev,
                      const moe_mxfp4_shape* shape, void* out_dev, void* workspace_dev,
                      uint64_t workspace_bytes, void* stream);

/*
 * Stages of the launch chain, in order: routing (+ shared append), sort
 * (count, scan, scatter) + GEMM2 gate, GEMM1 (+ SwiGLU), GEMM2 (split and
 * dense kernels), finalize.
 */
#define MOE_NUM_STAGES 5

/*
 * moe_mxfp4_forward, with per-stage timing for measurement tools: before
 * each of the MOE_NUM_STAGES stages and after the last one it records
 * stage_events[i] (MOE_NUM_STAGES + 1 hipEvent_t created by the caller) on
 * `stream`; elapsed time between events i and i+1 is stage i. Same work,
 * kernels and results as moe_mxfp4_forward; not meant for graph capture.
 * MOE_ERR_INVALID if stage_events or any of its entries is NULL.
 */
int moe_mxfp4_forward_timed(const void* x_dev, const float* router_logits_dev,
                            const int32_t* topk_ids_dev, const float* topk_w_dev,
                            const void* shared_logits_dev, const uint8_t* w13_dev,
                            const uint8_t* s13_dev, const uint8_t* w2_dev, const uint8_t* s2_dev,
                            const moe_mxfp4_shape* shape, void* out_dev, void* workspace_dev,
                            uint64_t workspace_bytes, void* stream, void* const* stage_events);

/*
 * Reorder a row-major nibble-packed weight matrix (rows x row_bytes bytes,
 * e.g. w13 as [E' * 2I, H/2] or w2 as [E' * H, I/2]) into the packed layout
 * the forward calls read: blocks of 16 rows x 64 bytes (16 rows x 128 K
 * elements, 1 KB each); the blocks of one 16-row group follow each other in
 * K order, and the groups follow each other in row order. Byte b of row r
 * moves to ((r / 16) * (row_bytes / 64) + b / 64) * 1024 + (r % 16) * 64 + b % 64.
 * The same bytes, only moved: a one-time step when weights are loaded,
 * like the repack the Marlin MoE kernel page describes for its weights, so
 * that every 16-lane weight load of the GEMMs reads 1 KB of contiguous
 * memory instead of 64 bytes from each of 16 rows.
 *
 * w_dev and w_packed_dev: device buffers of rows * row_bytes bytes, 16-byte
 * aligned, not overlapping; the caller owns both. Enqueued on `stream`.
 * Errors: MOE_ERR_INVALID (null or overlapping pointers, misalignment,
 * rows or row_bytes not positive), MOE_ERR_UNSUPPORTED (rows % 16 != 0 or
 * row_bytes % 64 != 0), MOE_ERR_HIP (launch failure).
 */
int moe_mxfp4_prepack(const uint8_t* w_dev, uint8_t* w_packed_dev, int64_t rows,
                      int64_t row_bytes, void* stream);

/*
 * moe_mxfp4_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under graph capture, tight serving loops,
 * harnesses that forbid allocation. The call allocates nothing and runs the
 * same launch chain and kernels as moe_mxfp4_forward, with the workspace in
 * a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES (128 MiB): one
 * copy per GPU the library runs on, held until the process ends. Arguments
 * as for moe_mxfp4_forward; the stream must belong to the current device,
 * whose copy is used.
 *
 * Limits and behaviour:
 *   - shapes whose moe_mxfp4_query size exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     fail with MOE_ERR_SCRATCH before any launch (the T = 64 and T = 256
 *     decode shapes of the K3.1 layer and the T = 512, H = 7168 shared-expert
 *     shape fit; a 32k-token prefill does not);
 *   - every call on one GPU shares that GPU's array and leaves its maps in
 *     it: calls that overlap on one GPU (other streams, other threads) race
 *     and give undefined results; serialise them;
 *   - the first call on a device looks the array's address up
 *     (hipGetSymbolAddress, which may load the code object): make it outside
 *     graph capture. MOE_ERR_HIP if that lookup fails.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (128ull << 20)
int moe_mxfp4_forward_noalloc(const void* x_dev, const float* router_logits_dev,
                              const int32_t* topk_ids_dev, const float* topk_w_dev,
                              const void* shared_logits_dev, const uint8_t* w13_dev,
                              const uint8_t* s13_dev, const uint8_t* w2_dev,
                              const uint8_t* s2_dev, const moe_mxfp4_shape* shape,
                              void* out_dev, void* stream);

/* Static text for a return code. */
const char* moe_mxfp4_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
