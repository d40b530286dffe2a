/*
 * dwdp.h -- C ABI of the one-rank DWDP MoE block for AMD Instinct MI355X (gfx950).
 *
 * DWDP (Distributed Weight Data Parallelism; paper summary "DWDP: Distributed
 * Weight Data Parallelism for High-Performance LLM Inference on NVL72") keeps
 * every rank data-parallel, leaves each rank a resident share of every MoE
 * layer's experts, and pulls the missing experts of layer l+1 into the other
 * half of a double buffer while layer l runs (§2 Methodology Overview).  The
 * expert GEMM reads the resident and the prefetched buffers directly instead of
 * merging them first (§4.2), and the pulls are cut into fixed-size slices
 * issued round-robin (§4.3.2).  This library is that rank's hot path:
 *
 *   dwdp_route_topk       router GEMM, top-k selection, renormalised softmax weights
 *   dwdp_permute          expert histogram, prefix scan, stable scatter, row gather
 *                         (with per-token fp8 quantisation when asked)
 *   dwdp_moe_grouped_ffn  grouped SwiGLU expert FFN over a per-expert pointer table
 *   dwdp_combine          weighted unpermute + shared expert
 *   dwdp_prefetch_chunks  chunked round-robin copy of the next layer's experts
 *
 * Conventions shared by every entry point
 *   - Device pointers are plain device addresses; the caller allocates and owns
 *     every buffer, stream and event.  The library allocates no device memory
 *     and keeps no pointer after a call returns.
 *   - `stream` arguments are hipStream_t values (NULL = the legacy default
 *     stream); `event` arguments are hipEvent_t values.
 *   - Calls are asynchronous and stream ordered; the caller keeps every buffer
 *     alive until the enqueued work has finished.
 *   - Arguments are validated before anything is enqueued; on error nothing is
 *     launched, a DWDP_ERR_* code is returned and dwdp_last_error() describes it.
 *   - T == 0 (no tokens) is a valid no-op.
 *   - Results are bitwise deterministic for identical inputs and do not depend
 *     on which buffer or slot an expert's weights sit in.
 *   - Device-side index values outside their range are not diagnosed (that would
 *     need a host synchronisation); kernels stay in bounds and the results stay
 *     defined.  A topk_idx entry outside [0, E) is dropped: see dwdp_permute.
 *   - One kernel launch holds fewer than 2^32 work-items.  Per-row and per-token
 *     kernels walk any count with a bounded grid.  The tiled GEMMs reject, with
 *     DWDP_ERR_INVALID_ARG ("too large"), a call whose tile grid would not fit:
 *     the router above ceil(T/64) * ceil(E/64) ~ 2^24 tiles (about 2^26 tokens at
 *     E = 1024), the grouped FFN above (rows/BM + n_groups) * max(2I, H)/256 ~ 2^23
 *     tiles (BM the tile height, 256 at prefill: about 75M rows at H = 7168).
 *
 * Layouts (row-major, C order)
 *   x          [T, H]            tokens, bf16 (f32 for the f32 path)
 *   w_router   [E, H]            router weight, same dtype as x
 *   expert e   W13 [2I, H]       gate rows 0..I-1, then up rows (Wg stacked on Wu)
 *              W2  [H, I]        down projection
 *              (f32: row-major; bf16 / fp8: fragment-major, see dwdp_pack_weights)
 *              fp8 only: S13 [2I/128, H/128] and S2 [H/128, I/128] fp32 block
 *              scales, one per 128x128 block of W13 / W2 ([out, in] blocks)
 *   x_perm     [rows, H]         rows = T*k + shared*T: routed rows ordered by
 *                                expert and, inside an expert, by t*k+j; then
 *                                the T shared-expert rows in token order
 *   offsets    [E+shared+1]      group g owns x_perm rows [offsets[g], offsets[g+1])
 *   y_perm     [rows, H]         expert outputs in x_perm's row order
 */
#ifndef DWDP_H_
#define DWDP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DWDP_OK = 0,
    DWDP_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad dtype combination */
    DWDP_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement */
    DWDP_ERR_WORKSPACE = 3,     /* workspace smaller than dwdp_workspace_bytes() */
    DWDP_ERR_HIP = 4            /* a HIP runtime call failed (message in dwdp_last_error) */
} dwdp_status;

typedef enum {
    DWDP_F32 = 0,               /* IEEE binary32 */
    DWDP_BF16 = 1,              /* bfloat16 */
    DWDP_FP8_E4M3 = 2           /* OCP FP8 E4M3 ("FN": no infinities, 448 max), fp32 scales */
} dwdp_dtype;

typedef enum {
    DWDP_OP_PERMUTE = 0,
    DWDP_OP_GROUPED_FFN = 1
} dwdp_op;

typedef enum {
    DWDP_COPY_HIPMEMCPY = 0,    /* one hipMemcpyAsync per slice, slices issued round-robin */
    DWDP_COPY_KERNEL = 1,       /* one launch of the library's slice-copy kernel walking the same plan */
    DWDP_COPY_SDMA = 2          /* one hipMemcpyAsync per slice of kind hipMemcpyDeviceToDeviceNoCU: the
                                   DMA engines move the bytes and no compute unit takes part, like the
                                   copy engines of the pages' design */
} dwdp_copy_engine;

/* One entry of the per-expert pointer table (the split-weight "TensorList",
 * paper summary §4.2): where group g's weights live.  s13/s2 are NULL unless
 * the weights are fp8.  Any entry may point into any buffer; two entries may
 * point at the same weights (redundant placement, §2). */
typedef struct {
    const void* w13;
    const void* w2;
    const float* s13;
    const float* s2;
} dwdp_expert_ptrs;

/* One prefetch source: `bytes` bytes at device address `src` go to dst + dst_offset. */
typedef struct {
    const void* src;
    size_t dst_offset;
    size_t bytes;
} dwdp_copy_src;

/* One slice of a prefetch plan, in issue order. */
typedef struct {
    int32_t source;
    int32_t pad_;
    size_t src_offset;
    size_t dst_offset;
    size_t bytes;
} dwdp_chunk;

/* Router: logits = x * w_router^T + bias (fp32 accumulation; bf16 inputs are
 * multiplied exactly), then per token the k largest logits (equal logits: the
 * lower expert index first; slots ordered by logit descending) and their
 * weights softmax(logits of the chosen k).  The pages give no gate formula;
 * this softmax top-k gate with renormalisation over the chosen k is the
 * reading taken.
 *   x [T,H], w_router [E,H]: DWDP_F32 or DWDP_BF16 (in_dtype), 16-byte aligned.
 *   bias [E] fp32 or NULL.   1 <= k <= E <= 1024, k <= 32; H % 64 == 0 (bf16) or
 *   H % 16 == 0 (f32).
 *   logits_out [T,E] fp32, topk_idx [T,k] int32, topk_w [T,k] fp32. */
int dwdp_route_topk(const void* x, const void* w_router, int in_dtype, const float* bias,
                    int64_t T, int H, int E, int k,
                    float* logits_out, int32_t* topk_idx, float* topk_w, void* stream);

/* Permutation by expert (counting sort, stable in t*k+j) and row gather.
 * The pages give no permutation (DWDP paper summary §2 only says that each rank
 * runs its own MoE block on its own batch); the reading taken is the textbook
 * one: experts in ascending order, inside an expert the assignments in
 * ascending flattened index t*k+j, then the shared expert's T rows in token
 * order.  The library builds it without atomics, so it is bitwise reproducible.
 *   topk_idx [T,k] int32.  shared in {0,1}.
 *   x [T,H] of x_dtype (F32 or BF16).  act_dtype == x_dtype copies rows bitwise;
 *   act_dtype == DWDP_FP8_E4M3 (x_dtype BF16, H % 128 == 0) quantises each row
 *   per 128-column group: scale = amax/448 (1 when amax is 0), code =
 *   E4M3(value/scale) rounded to nearest even, saturating; x_perm then holds
 *   codes (uint8) and x_perm_scale [rows, H/128] the scales.
 *   Outputs: x_perm [rows,H], offsets [E+shared+1], perm_src [rows] (source token
 *   of each row), inv_perm [T,k] (row of each (t,j)).
 *   Dropped entries: a topk_idx entry outside [0, E) is counted in no expert and
 *   gets inv_perm = -1 (dwdp_combine skips it).  offsets[E] is T*k in every case,
 *   so with D dropped entries the last D rows of the routed region, [T*k-D, T*k),
 *   close the last routed group (expert E-1's range holds D more rows than its
 *   count); their perm_src is 0, the grouped FFN computes them from token 0 and
 *   nothing reads their output.  With valid indices (dwdp_route_topk's) D = 0.
 *   x_perm == NULL computes only offsets, perm_src and inv_perm (x, x_perm_scale
 *   are then not read): the caller feeds the tokens to
 *   dwdp_moe_grouped_ffn_tokens, which gathers the rows itself.
 *   ws: dwdp_workspace_bytes(DWDP_OP_PERMUTE, ...) bytes of device scratch. */
int dwdp_permute(const int32_t* topk_idx, int64_t T, int k, int E, int shared,
                 const void* x, int x_dtype, int act_dtype, int H,
                 void* x_perm, float* x_perm_scale,
                 int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                 void* ws, size_t ws_bytes, void* stream);

/* Per-token fp8 quantisation, exactly as dwdp_permute quantises a row:
 *   x [T,H] bf16 (16-byte aligned), H % 128 == 0.  q [T,H] E4M3 codes, q_scale
 *   [T,H/128] fp32: per 128-column group scale = amax/448 (1 when amax is 0),
 *   code = E4M3(value/scale), nearest even, saturating.  T == 0 is a no-op. */
int dwdp_quantize_tokens_fp8(const void* x, int64_t T, int H, void* q, float* q_scale, void* stream);

/* Grouped SwiGLU FFN, reading each group's weights through `table` (device
 * array of n_groups entries) -- no merge of the split buffers (paper summary §4.2).
 *   For group g and its rows X = x_perm[offsets[g]:offsets[g+1]]:
 *     A = silu(X W13[0:I]^T) * (X W13[I:2I]^T),   y_perm rows = A W2^T
 *   w_dtype F32: x_perm, weights and y_perm fp32, fp32 math.
 *   w_dtype BF16: x_perm and weights bf16, fp32 accumulation, A rounded to bf16,
 *     y_perm bf16.
 *   w_dtype FP8_E4M3: x_perm codes + x_perm_scale (see dwdp_permute; 16-byte
 *     aligned), weights
 *     codes + 128x128 block scales; products accumulated in fp32 per 128-wide K
 *     block and scaled by (row scale * block scale); A quantised per row and
 *     128-column group like x; y_perm bf16.
 *   rows must equal offsets[n_groups] (not checked on the device).  H % 256 == 0,
 *   I % 128 == 0 (BF16/FP8; FP8 also H, I <= 8192); H % 64 == 0, I % 32 == 0
 *   (F32).  Other shapes return DWDP_ERR_INVALID_ARG.  offsets is read on the
 *   device only; no host synchronisation happens.
 *   ws: dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, ...) bytes.  After GEMM1 it
 *     begins with A [rows, I] row-major in the activation type (fp32, bf16, or
 *     E4M3 codes), followed for FP8 at the next 256-byte boundary by A's scales
 *     [rows, I/128] fp32; the tile schedule sits after them. */
int dwdp_moe_grouped_ffn(const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets,
                         const void* x_perm, const float* x_perm_scale, int64_t rows, int H, int I,
                         int w_dtype, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* The grouped FFN in two halves, for callers that enqueue or time them apart:
 * stage 1 builds the tile schedule and runs GEMM1 + SwiGLU, leaving A in ws;
 * stage 2 runs GEMM2 from the A left in ws by a stage-1 call with the same
 * arguments (and nothing else writing ws in between); stage 0 runs both and is
 * dwdp_moe_grouped_ffn.  y_perm may be NULL for stage 1. */
int dwdp_moe_grouped_ffn_stage(int stage, const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets,
                               const void* x_perm, const float* x_perm_scale, int64_t rows, int H, int I,
                               int w_dtype, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* The grouped FFN reading token rows instead of permuted rows: GEMM1's row r is
 * x[perm_src[r]] (out-of-range indices clamp to [0, T)), which spares the row
 * gather of dwdp_permute and its x_perm round trip through HBM.  x [T,H] holds the
 * tokens (F32 / BF16 as w_dtype; for FP8 the codes of dwdp_quantize_tokens_fp8
 * with x_scale [T,H/128]).  Everything else -- stage, table, offsets, rows,
 * workspace, outputs -- is as in dwdp_moe_grouped_ffn_stage, and the results
 * are bitwise those of the x_perm path. */
int dwdp_moe_grouped_ffn_tokens(int stage, const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets,
                                const int32_t* perm_src, const void* x, const float* x_scale, int64_t T,
                                int64_t rows, int H, int I, int w_dtype, void* y_perm, void* ws, size_t ws_bytes,
                                void* stream);

/* dwdp_moe_grouped_ffn_tokens without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is a fixed array inside the library, dwdp_static_scratch_bytes() = 64 MiB on each GPU the
 * library runs on, held until the process ends.  The call allocates nothing.  It computes exactly what
 * dwdp_moe_grouped_ffn_tokens computes with the same arguments (bitwise), and rejects with
 * DWDP_ERR_WORKSPACE, before anything is enqueued, a shape whose workspace
 * (dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, ...)) exceeds that size -- with bf16 weights and I = 2048
 * about 16K permuted rows, e.g. a decode batch of up to ~1800 tokens at top-8 plus a shared expert.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents: a stage-2 call
 * reads the A left by the last stage-1 call on that GPU, and calls whose executions overlap on one GPU
 * (other streams, other threads) race on the array and give undefined results. */
int dwdp_moe_grouped_ffn_tokens_static(int stage, const dwdp_expert_ptrs* table, int n_groups,
                                       const int32_t* offsets, const int32_t* perm_src, const void* x,
                                       const float* x_scale, int64_t T, int64_t rows, int H, int I, int w_dtype,
                                       void* y_perm, void* stream);

/* Bytes of the fixed workspace array dwdp_moe_grouped_ffn_tokens_static uses (64 MiB). */
size_t dwdp_static_scratch_bytes(void);

/* Combine: y[t] = sum_{j<k} topk_w[t,j] * y_perm[inv_perm[t,j]] (+ y_perm[T*k + t]
 * when shared), summed in fp32 in slot order then the shared row, rounded once
 * to out_dtype.  y_perm is fp32 for out_dtype F32, bf16 otherwise.  The pages
 * give no combine formula (DWDP paper summary §2: the rank runs an ordinary MoE
 * block); this weighted sum with the shared expert added at weight 1 is the
 * reading taken, with the summation order fixed so that the result is bitwise
 * reproducible.  Slots with inv_perm < 0 or >= T*k + shared*T contribute nothing.
 *   T >= 0, 1 <= k <= 64, H % 8 == 0; y_perm and y 16-byte aligned; y [T,H]. */
int dwdp_combine(const void* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T, int k,
                 int shared, int H, int out_dtype, void* y, void* stream);

/* Layer-ahead prefetch (paper summary §2 and §4.3.2): copy every source into
 * dst + dst_offset, cut into chunk_bytes slices issued round-robin over the
 * sources (slice c of every source before slice c+1 of any; the last slice of
 * a source may be short).  Destination ranges must not overlap.
 *   srcs: host array of n_src entries (1 <= n_src <= 64).
 *   engine: DWDP_COPY_HIPMEMCPY, DWDP_COPY_KERNEL or DWDP_COPY_SDMA; max_workgroups
 *   bounds the kernel engine's grid (0 = 48) and is ignored by the other engines.
 *   wait_event (nullable): copy_stream waits on it first (the last reader of the
 *   destination slots).  done_event (nullable): recorded on copy_stream after
 *   the last slice. */
int dwdp_prefetch_chunks(void* dst, const dwdp_copy_src* srcs, int n_src, size_t chunk_bytes,
                         int engine, int max_workgroups,
                         void* copy_stream, void* wait_event, void* done_event);

/* Host only: the slice plan dwdp_prefetch_chunks issues, in issue order.  Writes
 * at most max_chunks entries to out (out may be NULL to count) and the total
 * number of slices to *n_chunks. */
int dwdp_prefetch_plan(const dwdp_copy_src* srcs, int n_src, size_t chunk_bytes,
                       dwdp_chunk* out, size_t max_chunks, size_t* n_chunks);

/* Host only: fill a host pointer table from a placement.  Group g's record
 * starts at buffers[buf_of[g]] + slot_of[g] * record_bytes, laid out as
 * [W13 | W2 | S13 | S2] with every part 256-byte aligned (S13/S2 for fp8 only).
 * The caller uploads `out` (n_groups entries) to device memory. */
int dwdp_fill_expert_table(void* const* buffers, int n_buffers, const int32_t* buf_of,
                           const int32_t* slot_of, int n_groups, int H, int I, int w_dtype,
                           dwdp_expert_ptrs* out);

/* Host only: bytes of one expert record in the layout above. */
size_t dwdp_expert_record_bytes(int H, int I, int w_dtype);

/* Byte offsets of W2, S13 and S2 inside an expert record. */
int dwdp_expert_record_offsets(int H, int I, int w_dtype, size_t* off_w2, size_t* off_s13,
                               size_t* off_s2);

/* Re-lay a weight matrix w [N, K] (bf16, or fp8 E4M3 codes) into the fragment-major layout the
 * grouped FFN reads (out: N*K elements, same size, must not alias w).  bf16 (K % 64 == 0): the
 * 32 x 16 block (nb, kb) of W is 1 KB at byte (nb*K/16 + kb)*1024, lane l holding row 32nb + l%32,
 * columns 16kb + 8(l/32) .. +7.  fp8 (K % 128 == 0): the 32 x 64 block (nb, kb) is 2 KB at byte
 * (nb*K/64 + kb)*2048; lane l holds row 32nb + l%32, columns 64kb + 32(l/32) .. +31, split in two
 * 16-byte halves at +h*1024 + 16l.  N % 32 == 0.  This is the layout of one MFMA operand per
 * 1-2 KB, so every weight load of the GEMM is a contiguous lane-ordered 1 KB read. */
int dwdp_pack_weights(const void* w, int64_t N, int64_t K, int dtype, void* out, void* stream);

/* Block-quantise a weight matrix w [rows, cols] (fp32) to E4M3 codes q [rows, cols]
 * and fp32 scales s [rows/128, cols/128]: per 128x128 block, scale = amax/448
 * (1 when amax is 0) and code = E4M3(w/scale).  rows, cols multiples of 128. */
int dwdp_quantize_weight_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                             void* stream);

/* Device scratch the given operation needs (0 when none). */
size_t dwdp_workspace_bytes(int op, int64_t T, int k, int E, int H, int I, int dtype, int shared);

/* Description of the last error on the calling thread ("" if none).  Valid
 * until the next dwdp_* call on the same thread. */
const char* dwdp_last_error(void);

/* Library version string. */
const char* dwdp_version(void);

/* ---------------------------------------------------------------- diagnostics
 * Measurements of the machine and of the expert GEMM's schedule.  They are not
 * steps of the MoE block, and nothing on its path calls them. */

/* Operand-stream probe: the rate at which workgroups move bytes from device memory into LDS
 * with global_load_lds, the path every operand of the expert GEMM takes.  `grid` workgroups of
 * 512 threads (one per compute unit at grid <= 256); workgroup b reads the `span` bytes at
 * src + b*stride, `iters` times, in 32 KB steps (8 waves x 4 KB) into a ring of five 32 KB LDS
 * slots, keeping `in_flight` steps (1..5) outstanding.  cpol 0 is the default cache policy, 2
 * non-temporal.  stride 0 makes every workgroup read the same bytes (L2 hits once warm).
 * The caller guarantees that src holds (grid-1)*stride + span bytes (the library cannot see
 * the allocation).  span: a positive multiple of 32768; 1 <= grid <= 65536; iters >= 1.
 * Reads only; time it with events on `stream`. */
int dwdp_diag_operand_stream(const void* src, size_t span, size_t stride, int iters, int grid,
                             int in_flight, int cpol, void* stream);

/* LDS read probe: `grid` workgroups of `waves` waves (4, 8 or 16) each read a 128 KB LDS array with
 * ds_read_b128 (lane-consecutive 16-byte slots, so no bank conflicts; 16 reads in flight per wave)
 * `iters` times 16 KB per wave.  Thread 0 of workgroup b stores the shader-clock (s_memtime) and
 * real-time (100 MHz) counter deltas over the read loop to clocks[2b] and clocks[2b+1] (device,
 * 2*grid values, 16-byte aligned); bytes per clock per CU = iters * 16384 * waves / clocks[2b].
 * sink: device, grid words, written only in the unlikely case that the data's checksum hits a
 * constant (it keeps the reads from being optimised away).  1 <= grid <= 65536. */
int dwdp_diag_lds_read(int grid, int waves, int iters, uint32_t* sink, unsigned long long* clocks,
                       void* stream);

/* Tile trace of the expert GEMM (bf16 and fp8 paths).  A library built with
 * -DDWDP_TILE_TRACE=1 has every workgroup of an expert-GEMM launch write one record into a fixed
 * device array of 131072 records, at the workgroup's index: its tile, the XCD it ran on and the
 * GPU's real-time counter (100 MHz) when it started and when its last wave finished.  Clear the
 * array, run ONE grouped-FFN stage, synchronise, read.  Slots of workgroups that ran no tile (or
 * beyond the array) keep t_end == 0.  Other builds return DWDP_ERR_UNSUPPORTED. */
typedef struct {
    uint64_t t_start;           /* real-time counter when the workgroup took its tile */
    uint64_t t_end;             /* ... and after its last wave finished the tile */
    int32_t order;              /* the tile's position in the schedule */
    int32_t group;              /* expert group */
    int32_t first_row;          /* first permuted row of the tile */
    int32_t rows;               /* rows of the tile */
    int32_t n_tile;             /* 256-column output tile (GEMM1: 128 gate + 128 up columns) */
    int32_t group_m_tiles;      /* m-tiles of the group */
    int32_t xcd;                /* XCD the workgroup ran on */
    int32_t hw_id;              /* its compute unit inside the XCD: bits 15:8 of the HW_ID hardware
                                   register (CU, shader array and shader engine numbers) */
} dwdp_tile_record;

/* Zero the trace array on the current device (stream ordered). */
int dwdp_diag_tile_trace_clear(void* stream);
/* Copy the first min(max_records, 131072) records of the current device's array to host memory
 * `out` (synchronous: waits for the device) and store that count in *n_records. */
int dwdp_diag_tile_trace_read(dwdp_tile_record* out, size_t max_records, size_t* n_records);

#ifdef __cplusplus
}
#endif

#endif /* DWDP_H_ */
