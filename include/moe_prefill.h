/*
 * moe_prefill.h -- C ABI of the MI355X (gfx950) prefill routed-expert product.
 *
 * One MoE layer's routed experts over a prompt chunk of T tokens, in the
 * steps the "Strata" pages describe (PR #3752 "GP100 weight-stationary
 * experts": commit list and Approach; PR #2145 "fused int8 prompt experts on
 * Turing": description):
 *
 *   moe_weights_pack   (once per layer, at load) weights -> the kernels' tiled layout
 *   moe_prefill_plan   routing ids -> expert-sorted rows, offsets, chunk table
 *   moe_prefill_plan_device   the same plan built on the GPU from device ids
 *   quantize_scatter   X (fp32) -> q8_1 rows, one copy per (token, expert)
 *   expert_gate_up     q8_1 rows x Q2_0 (or NL4) gate/up weights -> GU (fp32)
 *   swiglu_q8          GU -> q8_1 of silu(gate) * up, H never stored as floats
 *   expert_gate_up_swiglu_q8   the two above in one launch, GU never stored
 *   expert_down        q8_1 H rows x down weights -> one fp32 row per (token, expert)
 *   moe_combine        routing-weighted sum of each token's expert rows -> [tokens x hidden]
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory.  `stream` is a hipStream_t (NULL
 *     is the null stream).  Work is enqueued asynchronously on `stream`.
 *   - The caller owns every device buffer (inputs, outputs, weights, the plan
 *     workspace).  The library never allocates device memory.  The moe_plan
 *     object is a host object owned by the library until moe_plan_destroy.
 *   - Every call validates its arguments on the host before it enqueues
 *     anything; on error it returns a negative moe_status and launches
 *     nothing.  A step over a plan with no rows (tokens == 0) does nothing
 *     and accepts NULL buffers.  Launch failures reported by HIP return MOE_EHIP.  No call
 *     throws across the ABI.
 *   - Results are deterministic: no floating-point atomics, every output
 *     element is written by exactly one thread with a fixed operation order.
 *
 * Data formats (the byte layouts are this project's own; the pages name the
 * formats but do not print their bits):
 *   q8_1 row of C values (C % 32 == 0), moe_q8_1_bytes(1, C) = 1.25*C bytes:
 *       int8 q[C] | fp32 d[C/32] | int32 s[C/32]
 *     block b holds values 32b..32b+31 with d = max|x|/127 (fp32 divide),
 *     q = x/d rounded half away from zero and clamped to [-127, 127],
 *     s = sum of the block's q; a block with d == 0 is all zeros.
 *   Q2_0 matrix [rows x cols] (cols % 64 == 0), rows*cols/64*18 bytes
 *   (scales must satisfy |2d| <= 65504, so that d*(code-2) is a binary16):
 *       codes plane: rows*cols/64 blocks of 16 bytes, row-major (row, block);
 *         value 16*j+b of a block is bits 2j..2j+1 of byte b; weight = d*(code-2)
 *       scales plane: rows*cols/64 binary16 d, same order, right after the codes.
 *   NL4 matrix [rows x cols] (cols % 32 == 0), rows*cols/32*18 bytes:
 *       codes plane: 16-byte blocks of 32 values, value b in the low nibble of
 *         byte b, value 16+b in the high nibble; weight = d*codebook[code]
 *       scales plane: binary16 d per 32-value block.
 *   Tiled layout (MOE_W_TILED, what the product kernels read; written by
 *   moe_weights_pack): the same two planes with the same sizes, each in
 *   (row tile, block, row in tile) order for 32-row tiles -- block b of row
 *   32*i + r sits at slot (i * blocks_per_row + b) * 32 + r of its plane, so
 *   the 32 rows of one block are 512 contiguous code bytes and 64 scale bytes.
 *   Within a Q2_0 block the codes are also reordered: the code of value
 *   v = 32*h + 16*g + 8*kq + p (h, g, kq < 2, p < 8) sits at bits
 *   2*g + 4*(p%2) .. +1 of byte 8*kq + 4*h + p/2.  NL4 blocks are unchanged.
 *   Expert outputs are fp32.  The per-32-value epilogue is, for each output,
 *       acc = 0; for each 32-value block b in K order:
 *         acc = fmaf(dx_b, dw_b * (float)dot_b, acc)
 *     where dot_b is the exact int32 dot of the block's q with the weight's
 *     integer codes (Q2_0: code-2; NL4: codebook entry) and dw_b the block's
 *     weight scale (a Q2_0 block's two 32-value halves share it).
 */
#ifndef MOE_PREFILL_H
#define MOE_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,   /* null pointer, non-positive or inconsistent size, id out of range */
    MOE_EALIGN = -2,   /* a pointer or offset is not 16-byte aligned */
    MOE_EFORMAT = -3,  /* unknown weight type, or dims not a multiple of the block */
    MOE_ESIZE = -4,    /* a caller buffer is smaller than the size query demands */
    MOE_EHIP = -5,     /* HIP reported an error while enqueueing */
    MOE_ESTATE = -6,   /* the plan was built without a device workspace */
    MOE_ENOMEM = -7    /* host memory ran out (plans, their queries, the pack's checks);
                          nothing was launched and no plan was returned */
} moe_status;

typedef enum {
    MOE_W_Q2_0 = 1,
    MOE_W_NL4 = 2,
    MOE_W_TILED = 0x100,           /* the kernels' layout, written by moe_weights_pack */
    MOE_W_GU_INTERLEAVED = 0x200   /* gate/up rows alternate: row 2j gate j, 2j+1 up j */
} moe_wtype;

/* The weights of one product (gate/up or down) for all experts of a layer,
 * read in place: expert e's matrix starts at base + offset[e] ("Strata"
 * PR #3752, commit list: a per-layer offset table from the expert cache's
 * base, uploaded with the group bounds).
 *   type      MOE_W_Q2_0 or MOE_W_NL4 (each product its own); the plan takes
 *             weights in the tiled layout, type | MOE_W_TILED
 *   rows      output features (gate/up: 2*n_ff; down: hidden), % 64 == 0
 *   cols      contraction length (gate/up: hidden; down: n_ff), % 64 (Q2_0)
 *             or % 32 (NL4) == 0; one expert's matrix (rows * cols / block
 *             * 18 bytes) below 2^31 bytes (MOE_EINVAL beyond: the kernels
 *             address inside an expert with 32-bit offsets)
 *   n_expert  number of experts
 *   base      device pointer, 16-byte aligned
 *   base_bytes size of the buffer at base (every expert must lie inside it)
 *   offset    host pointer [n_expert]: byte offsets, each 16-byte aligned
 *   codebook  host pointer [16] int8, NL4 only (NULL for Q2_0)
 * The descriptor is copied by moe_prefill_plan; the weight bytes themselves
 * must stay valid and unchanged while the plan is used. */
typedef struct {
    int type;
    int rows;
    int cols;
    int n_expert;
    const void *base;
    size_t base_bytes;
    const uint64_t *offset;
    const int8_t *codebook;
} moe_weights;

typedef struct moe_plan moe_plan;  /* opaque host object */

/* Bytes of `rows` q8_1 rows of `cols` values: rows * 1.25 * cols.
 * Returns 0 if cols % 32 != 0 or a size is negative. */
size_t moe_q8_1_bytes(int rows, int cols);

/* Bytes of one expert's matrix in the given format, either layout (0 on a
 * bad format/dim). */
size_t moe_weight_bytes(int type, int rows, int cols);

/* Write the tiled layout of every expert of `w` (row-major planes, type
 * MOE_W_Q2_0 or MOE_W_NL4 without MOE_W_TILED) into dst: expert e's tiled
 * matrix at dst + w->offset[e], the same offsets and sizes as the source, so
 * the descriptor {type | MOE_W_TILED, ..., base = dst, base_bytes =
 * dst_bytes, same offsets} then describes the packed weights.  A pure byte
 * permutation inside each plane, done once when a layer is loaded (one launch
 * when the experts sit at a constant stride, else one per expert).
 * Gate/up weights stored with alternating rows (type | MOE_W_GU_INTERLEAVED,
 * the other row order the pages' swiglu_quant test covers) are packed into
 * split order, gate rows first; the packed descriptor does not carry the flag
 * (the plan refuses it).
 *   dst        device buffer, 16-byte aligned, every expert inside dst_bytes,
 *              not overlapping w->base's buffer; owned by the caller.
 * Experts must share a matrix (equal offsets) or not overlap.  Asynchronous
 * on `stream`; the source must stay valid until the copy has run. */
int moe_weights_pack(const moe_weights *w, void *dst, size_t dst_bytes, void *stream);

/* Device workspace the plan needs for T tokens, top-k, n_expert experts and
 * chunks of at most chunk_rows rows (sorted-row maps, expert offsets, the
 * chunk table, the per-product work lists and both weight offset tables).
 * Returns 0 on invalid sizes. */
size_t moe_plan_device_bytes(int tokens, int topk, int n_expert, int chunk_rows);

/* Build a layer's plan ("Strata" PR #3752: quantize_scatter sorts each
 * expert's rows together; the CTAs take row chunks of the experts, largest
 * expert first; every expert at its own row count, no padding).
 *   ids_host   host int32 [tokens*topk], ids_host[t*topk+k] = k-th expert of
 *              token t, each in [0, n_expert).  A token may name an expert
 *              twice; that gives two rows.
 *   chunk_rows 1..128: rows per chunk (the pages take 64-row chunks; one
 *              workgroup processes one chunk against 256 weight rows).
 *   w_gu       gate/up weights: Q2_0 or NL4, rows = 2*n_ff, cols = hidden.
 *   w_down     down weights: Q2_0 or NL4, rows = hidden, cols = n_ff.
 *              Both in the tiled layout (type | MOE_W_TILED), else MOE_EFORMAT.
 *   plan_dev   device workspace of moe_plan_device_bytes(...) bytes, 16-byte
 *              aligned, owned by the caller, not touched by anything else
 *              while the plan lives; NULL builds a host-only plan (for
 *              inspection: the kernels refuse it with MOE_ESTATE).
 *   stream     the plan is uploaded with one asynchronous host-to-device
 *              copy on this stream; later launches on the same stream see it.
 * Sorted rows: expert e owns rows [off[e], off[e+1]); inside an expert the
 * rows keep ascending t*topk+k order.  Chunks are (expert, first row, rows),
 * experts by descending row count, ties by ascending expert id.
 * MOE_EINVAL if a product launch over the plan would exceed one HIP grid
 * (2^32 - 1 threads: 8 workgroups of 256 threads per item of the longest XCD
 * list, an item being one chunk against 256 weight rows, or 128 j's of the
 * fused gate/up).
 * On success *out receives the plan; on error *out is left NULL. */
int moe_prefill_plan(const int32_t *ids_host, int tokens, int topk, int n_expert,
                     int chunk_rows, const moe_weights *w_gu, const moe_weights *w_down,
                     void *plan_dev, size_t plan_dev_bytes, void *stream, moe_plan **out);

/* The same plan built on the device from routing ids that live there (the
 * pages build the bounds and the chunk table on the host and upload them,
 * PR #3752 commit list; a router on the GPU leaves its ids in device memory).
 * Arguments as moe_prefill_plan, except:
 *   ids_dev    device int32 [tokens*topk], 16-byte aligned, read by kernels
 *              enqueued on `stream` (it must stay valid until they ran).
 *   plan_dev   required.  Every section the kernels read holds the same bytes
 *              as a host-built plan of the same ids.
 *   n_expert   at most 2048, and tokens*topk below 2^29 (MOE_EINVAL beyond;
 *              also when the launches' grid bound below exceeds one HIP grid,
 *              as for moe_prefill_plan -- e.g. chunk_rows 1 with 32K tokens
 *              at top-10).
 * Nothing is read back: the call enqueues a host-to-device copy of the two
 * weight offset tables and four small integer launches (per tile of ids, its
 * rows per expert, which also clears the chunk table; per expert, a prefix
 * over the tiles; one launch whose first workgroup takes the offsets, ranks
 * the experts and deals them to the XCDs while the others place each tile's
 * rows, stable in t*topk+k order; the chunk lists), then returns.  An id outside [0, n_expert)
 * cannot be refused at the call: its rows join no product (their outputs are
 * left unwritten) and moe_plan_query on the plan returns MOE_EINVAL.  Because
 * the per-XCD chunk counts stay on the device, the product launches over such
 * a plan size their grids for the largest possible list (tokens*topk /
 * chunk_rows + n_expert + 1 chunks per XCD); the surplus workgroups exit at
 * once. */
int moe_prefill_plan_device(const int32_t *ids_dev, int tokens, int topk, int n_expert,
                            int chunk_rows, const moe_weights *w_gu, const moe_weights *w_down,
                            void *plan_dev, size_t plan_dev_bytes, void *stream, moe_plan **out);

/* moe_prefill_plan_device for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the plan is built in the library's own
 * workspace, a 4 MiB array of device memory that each GPU the library runs on
 * holds until the process ends.  The call allocates nothing (no hipMalloc,
 * hipHostMalloc, event or host heap memory) and copies nothing from the host:
 * the weight offset tables are written on the device, so every expert of
 * w_gu and of w_down must sit at a constant stride from the first
 * (offset[e] = offset[0] + e * stride; stride 0 shares one matrix), else
 * MOE_EINVAL.
 * Arguments and checks as moe_prefill_plan_device, without plan_dev; the
 * plan's moe_plan_device_bytes(tokens, topk, n_expert, chunk_rows) must be at
 * most 4 MiB (MOE_ESIZE beyond: about 180,000 rows at 512 experts).
 * Every plan built this way on a device shares that device's workspace and
 * one host object: *out stays valid until the next call of this function on
 * the same device, which overwrites it (finish the steps over one plan before
 * building the next; calls that overlap on one device race).  moe_plan_destroy
 * on it does nothing.  moe_plan_query waits for `stream`. */
int moe_prefill_plan_device_noalloc(const int32_t *ids_dev, int tokens, int topk, int n_expert,
                                    int chunk_rows, const moe_weights *w_gu,
                                    const moe_weights *w_down, void *stream, moe_plan **out);

/* Host view of a plan, for inspection and tests: any pointer may be NULL.
 * For a device-built plan it waits for the plan's kernels and reads the plan
 * back (MOE_EINVAL if a routing id was out of range).
 * counts [n_expert], offsets [n_expert+1], perm [tokens*topk] (sorted row ->
 * t*topk+k), chunks [4*n_chunks] (expert, first row, rows, 0). */
int moe_plan_query(const moe_plan *plan, int *rows, int *n_chunks,
                   int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *chunks);

/* Release the plan (waits for its upload to finish; does not free plan_dev).
 * The pinned host buffer its upload was staged in is kept by the library for
 * later plans (until the process ends), so destroying a plan never waits for
 * the rest of the device. */
void moe_plan_destroy(moe_plan *plan);

/* Step 1 ("Strata" PR #3752, commit list: quantize_scatter).  Quantize each
 * token's row of x to q8_1 and write it to each of its topk expert-sorted
 * rows.  x: device fp32 [tokens x hidden] row-major, 16-byte aligned.
 * xq: device, moe_q8_1_bytes(tokens*topk, hidden) bytes, 16-byte aligned. */
int quantize_scatter(const moe_plan *plan, const float *x, void *xq, void *stream);

/* Step 2 ("Strata" PR #3752: gate/up as one launch over all experts;
 * PR #2145: exact int32 block sums, per-32-value fp32 epilogue).
 * gu[r][n] for every sorted row r and n < 2*n_ff: the epilogue above over the
 * q8_1 row r of xq and row n of its expert's gate/up matrix.  Gate is
 * n < n_ff, up is n >= n_ff.
 * xq: device q8_1 rows [tokens*topk x hidden]; gu: device fp32
 * [tokens*topk x 2*n_ff] in sorted-row order, 16-byte aligned. */
int expert_gate_up(const moe_plan *plan, const void *xq, float *gu, void *stream);

/* Step 3 ("Strata" PR #3752, swiglu_quant commit: swiglu and the q8_1 rows
 * the down product reads, in one pass, H never stored).  For each sorted row
 * and j < n_ff: h_j = silu(g_j) * u_j with g_j = gu[r][j], u_j = gu[r][n_ff+j]
 * and silu(g) = g / (1 + E) in fp32, E = e^-g rounded to the nearest binary32
 * (through a binary64 exponential); hq row r = q8_1 of h.
 * gu: device fp32 [tokens*topk x 2*n_ff]; hq: device
 * moe_q8_1_bytes(tokens*topk, n_ff) bytes; both 16-byte aligned. */
int swiglu_q8(const moe_plan *plan, const float *gu, void *hq, void *stream);

/* Steps 2 and 3 in one launch: the gate/up product of step 2 with the
 * swiglu and q8_1 of step 3 applied to its fp32 results in registers, so GU
 * never reaches memory (the same fusion PR #3752 makes for swiglu_quant, one
 * step earlier).  hq is byte for byte what expert_gate_up followed by
 * swiglu_q8 writes.  xq: device q8_1 rows [tokens*topk x hidden]; hq: device
 * moe_q8_1_bytes(tokens*topk, n_ff) bytes; both 16-byte aligned. */
int expert_gate_up_swiglu_q8(const moe_plan *plan, const void *xq, void *hq, void *stream);

/* Step 4 ("Strata" PR #3752: the down product as one launch into one row per
 * (token, expert), the K loop stopping at n_ff).
 * dm[t*topk+k][n] for n < hidden: the epilogue over sorted row r (whose
 * perm[r] = t*topk+k) of hq and row n of the expert's down matrix.
 * hq: device q8_1 rows [tokens*topk x n_ff]; dm: device fp32
 * [tokens*topk x hidden], 16-byte aligned. */
int expert_down(const moe_plan *plan, const void *hq, float *dm, void *stream);

/* The MoE combine, the step after step 4 (the pages name it among the
 * prompt-path fusions PR #3752 leaves out and print no formula; this is the
 * plain routing-weighted sum):
 *   out[t][n] = sum over k of w[t*topk+k] * dm[t*topk+k][n],
 * evaluated in fp32 as one fmaf per term, k ascending, starting from 0.
 * dm: device fp32 [tokens*topk x hidden] as expert_down writes it; w: device
 * fp32 [tokens x topk] routing weights; out: device fp32 [tokens x hidden];
 * all 16-byte aligned.  One thread per four outputs: MOE_EINVAL if
 * tokens * hidden / 4 exceeds 2^32 - 1 (the launch's thread count). */
int moe_combine(const moe_plan *plan, const float *dm, const float *w, float *out, void *stream);

/* Test export: the exact int32 dots of every (sorted row, output, 32-value
 * block) of one product, computed by the product kernels' templates in a dots
 * mode (for Q2_0 the matrix-core kernel decodes every scale as 1, so its
 * matrix unit returns the dot itself; the small-chunk kernel returns its
 * int8 dot products), each dot stored as it leaves the matrix or dot unit.
 * product 0 = gate/up (act = xq), 1 = down (act = hq).  Rows
 * [row_begin, row_begin+n_rows) of the sorted order; dots: device int32
 * [n_rows x out_rows x cols/32], 16-byte aligned. */
int moe_debug_block_dots(const moe_plan *plan, int product, const void *act,
                         int row_begin, int n_rows, int32_t *dots, void *stream);

/* Text of a status code (static storage). */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PREFILL_H */
