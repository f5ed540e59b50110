/*
 * fp8bs.h -- C ABI of the FP8 (E4M3) 128x128 block-scaled decode GEMM for
 * AMD MI355X (gfx950).
 *
 * The operation, as the pages state it:
 *   - weights are converted once to FP8 E4M3 with one fp32 scale per
 *     128 x 128 block ("The profiler said the kernel ran zero times",
 *     section "The output layer, which did run"; "A 23% faster GPU kernel,
 *     and a model that did not move", section "Why this shape is hard");
 *   - the multiply's inputs are cast to FP8 on every call ("The profiler said
 *     the kernel ran zero times", section "What the trace showed"); the
 *     activation scale granularity is not given on the pages and is taken
 *     here as one scale per row per 128 columns, aligned with the weight's
 *     K blocks;
 *   - the long K dimension is split across compute units and the partial
 *     results are reduced in a fixed order ("A 23% faster GPU kernel...",
 *     section "Why this shape is hard");
 *   - the shapes are decode shapes: a handful of activation rows (about
 *     eight), where the multiply is bound by reading the weights ("A 23%
 *     faster GPU kernel...", section "Why this shape is hard";
 *     "Kernel-Level Optimisations for LLM Inference and Training", section
 *     "Start with the bound: memory or compute").
 *
 * FP8 format: E4M3 with largest finite value 448 (exponent bias 7,
 * subnormals, no infinities, NaN only at 0x7F / 0xFF) -- "Kernel-Level
 * Optimisations...", section "Quantisation kernels".
 *
 * Quantization rule (weights and activations alike): for each block,
 *   amax  = max |x| over the block,
 *   scale = fl32(amax / 448)                      (IEEE fp32 division),
 *   code  = RNE_e4m3(fl32(x / scale))             (ties to even mantissa,
 *           saturating at +-448, sign of zero kept);
 * an all-zero block has scale 0 and codes 0x00 / 0x80 (sign of each zero).
 * Dequantized value = decode(code) * scale.
 *
 * GEMM: Y[m][n] = sum over K blocks kb of
 *         (sum_{k in kb} dec(xq[m][k]) * dec(wq[n][k])) * xs[m][kb] * ws[n/128][kb]
 * accumulated in fp32 and rounded once to bf16 (round to nearest even).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *     The library never allocates, frees or synchronizes.
 *   - `stream` is a hipStream_t (NULL = the null stream); calls are
 *     asynchronous on it.
 *   - Arguments are checked before anything is launched. On any non-OK
 *     status nothing has been launched and no memory has been touched.
 *     Checks, in order: shapes (a call whose output is empty returns
 *     FP8BS_OK right after them, whatever its pointers), NULL pointers,
 *     alignment, explicit kernel configuration, workspace size, device
 *     (must be gfx950). The first failing check decides the status. A failed
 *     launch returns FP8BS_ERR_LAUNCH; faults inside a kernel surface at the
 *     caller's next synchronization.
 *   - There is no fallback: an unsupported shape is an error, never a
 *     silently slower path.
 *   - Determinism: the same inputs, shape, device and library build give
 *     bit-identical outputs. The GEMM uses no floating-point atomics.
 *   - Shapes: n and k must be multiples of 128 (whole blocks); m may be any
 *     value >= 0 for the quantizers and 0..2^20 for the GEMM (decode kernels
 *     up to 32 rows, the prefill kernel above). The GEMM also needs
 *     n < 2^31 (n/128 < 2^24) and k/128 <= 2^20. A zero extent is a no-op
 *     (k == 0 in the GEMM writes zeros: the empty sum).
 *   - Alignment: bf16 and code pointers 16-byte aligned; scale pointers
 *     4-byte aligned; workspace 16-byte aligned.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL = 1,      /* a required pointer is NULL */
  FP8BS_ERR_SHAPE = 2,     /* n or k not a multiple of 128, m out of range, negative extent */
  FP8BS_ERR_ALIGN = 3,     /* a pointer is not aligned as documented above */
  FP8BS_ERR_WORKSPACE = 4, /* workspace smaller than fp8bs_gemm_workspace_bytes(...) */
  FP8BS_ERR_DEVICE = 5,    /* no current HIP device, or it is not gfx950 */
  FP8BS_ERR_LAUNCH = 6,    /* the kernel launch itself failed */
  FP8BS_ERR_CONFIG = 7     /* an explicit kernel configuration is invalid for this shape */
} fp8bs_status;

/* Weight quantization, one scale per 128x128 block (done once per weight).
 *   w_bf16  [n][k] bf16, in
 *   w_fp8   [n][k] E4M3 codes, out
 *   w_scale [n/128][k/128] fp32, out                                        */
fp8bs_status fp8bs_quantize_weight(const void* w_bf16, int64_t n, int64_t k,
                                   uint8_t* w_fp8, float* w_scale, void* stream);

/* Activation quantization, one scale per row per 128 columns: the same rule
 * the GEMM applies internally on every call (fp8bs_gemm fuses it).
 *   x_bf16  [m][k] bf16, in
 *   x_fp8   [m][k] E4M3 codes, out
 *   x_scale [m][k/128] fp32, out                                            */
fp8bs_status fp8bs_quantize_act(const void* x_bf16, int64_t m, int64_t k,
                                uint8_t* x_fp8, float* x_scale, void* stream);

/* Y = X . W^T with the activation cast fused in; 0 <= m <= 2^20.
 * m <= 32 (decode) runs the bandwidth-bound kernels with the cast inside the
 * GEMM. m > 32 (prefill, "Kernel-Level Optimisations for LLM Inference and
 * Training", section "Start with the bound: memory or compute") runs the
 * tiled matrix-core kernel: the activations are first cast into the
 * workspace (m*k code bytes, padded to 256, then m*k/128 fp32 scales), with
 * the same rule as fp8bs_quantize_act. That kernel forms 32-bit offsets
 * within a 256-row slab of W, so m > 32 needs k < 2^24 (else
 * FP8BS_ERR_SHAPE).
 *   x_bf16  [m][k] bf16; w_fp8 [n][k] codes; w_scale [n/128][k/128] fp32;
 *   y_bf16  [m][n] bf16, out.
 *   workspace: device scratch of at least fp8bs_gemm_workspace_bytes(m,n,k)
 *   bytes (may be NULL when that is 0). Its contents need no initialization
 *   and are garbage afterwards. Calls that share a workspace must be ordered
 *   on one stream.                                                          */
fp8bs_status fp8bs_gemm(const void* x_bf16, int64_t m,
                        const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                        void* y_bf16, void* workspace, size_t workspace_bytes,
                        void* stream);

/* fp8bs_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). It allocates nothing and calls no
 * allocating routine: split-K partials, arrival counters and the prefill
 * path's cast activations go to a fixed scratch array in the library, one
 * copy per GPU, held from library load until the process ends, of
 * fp8bs_gemm_noalloc_max_scratch() bytes (8 MiB). A shape whose selected
 * configuration needs more scratch than that (large prefill m) returns
 * FP8BS_ERR_WORKSPACE before any launch. Same configuration as fp8bs_gemm,
 * hence the same bits. Nothing in the scratch must start at zero: partials
 * are written before they are read and counters carry a per-launch epoch.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (different streams without ordering between them) race; calls
 * ordered on one stream do not.                                            */
fp8bs_status fp8bs_gemm_noalloc(const void* x_bf16, int64_t m,
                                const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                                void* y_bf16, void* stream);
size_t fp8bs_gemm_noalloc_max_scratch(void);

/* Same product from already-quantized activations (codes [m][k] and scales
 * [m][k/128] as produced by fp8bs_quantize_act). With the same shape it runs
 * the same kernel configuration as fp8bs_gemm, so
 * fp8bs_gemm(x) == fp8bs_gemm_q(fp8bs_quantize_act(x)) bit for bit. It needs
 * no workspace on the prefill path.                                         */
fp8bs_status fp8bs_gemm_q(const uint8_t* x_fp8, const float* x_scale, int64_t m,
                          const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                          void* y_bf16, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes the automatically selected configuration needs (0 when
 * the K dimension is not split across workgroups), enough for both weight
 * layouts (fp8bs_gemm* and fp8bs_gemm*_tiles). Returns 0 for shapes
 * fp8bs_gemm would reject.                                                  */
size_t fp8bs_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* ---- explicit kernel configuration (tuning and tests) ------------------- */

enum {
  FP8BS_PATH_AUTO = 0,
  FP8BS_PATH_MFMA = 1,
  FP8BS_PATH_DOT = 2,
  FP8BS_PATH_MFMA_ROWS = 3,
  FP8BS_PATH_MFMA_STREAM = 4,
  FP8BS_PATH_PREFILL = 5,
  FP8BS_PATH_MFMA_ROWS_REG = 6,
  FP8BS_PATH_MFMA_STREAMK = 7,
  FP8BS_PATH_MFMA_ROWS_DMA = 8
};
enum { FP8BS_REDUCE_KERNEL = 0, FP8BS_REDUCE_LAST_ARRIVER = 1 };
enum { FP8BS_EPILOGUE_SEPARATE = 0, FP8BS_EPILOGUE_IN_GEMM = 1 };
enum { FP8BS_LAYOUT_ROWS = 0, FP8BS_LAYOUT_TILES = 1 };

/* How one GEMM is laid out on the GPU.
 *   path      MFMA (16x16x128 FP8 matrix instructions, a grid of row
 *             groups x K splits), DOT (per-lane fp32 dot products, for the
 *             smallest m), or MFMA_ROWS (one workgroup per compute unit, each
 *             owning a contiguous range of output columns over the whole K
 *             range; waves_k and depth apply, tiles_n gives how many of
 *             the depth tiles are requested before the activation cast,
 *             waves_n and split_k must be 1), or MFMA_STREAM (the work split
 *             of MFMA_ROWS without a staging phase: each wave casts the
 *             activation blocks it uses as the first tile reaches them;
 *             tiles_n, waves_n and split_k must be 1; needs m*k*2 < 2^31), or
 *             PREFILL (any m; reduce must be FP8BS_REDUCE_KERNEL): with
 *             tiles_n 1 or 2, waves_k 2 and waves_n 2 or 4, workgroups of
 *             2 waves_n waves own (64 waves_n) x 128 output tiles and step
 *             through K in 128-deep blocks: depth 1 = through registers one
 *             block ahead, depth 2..4 = a ring of LDS stages filled by
 *             direct loads, refilled when the next block starts (tiles_n
 *             1) or once every wave holds a block's operands (tiles_n 2);
 *             with tiles_n 3 or 4, waves_n 2, waves_k 4 or 3 and depth 2,
 *             the wide kernel: 8 waves own (64 waves_k) x 256 output tiles
 *             (16 waves_k x 128 each), on a grid of tiles with K split over
 *             split_k workgroups (tiles_n 3), or on the 1-D schedule
 *             (tiles_n 4, split_k 1): whole tiles in complete rounds of 256
 *             workgroups, the tiles left over as 128-column halves; with
 *             tiles_n 5 (split_k 1, n a multiple of 160) the same kernel on
 *             narrow (64 waves_k) x 160 tiles, one workgroup per tile; or
 *             MFMA_ROWS_REG (the work split of MFMA_ROWS with each wave's
 *             activation operands held in registers instead of LDS, so m up
 *             to 32 runs unsplit at any K the registers hold: depth is the
 *             number of K blocks per wave and k / 128 must not exceed
 *             waves_k * depth; tiles_n gives how many weight blocks are
 *             requested before the cast; waves_n and split_k must be 1).
 *             MFMA_STREAMK (stream-K: 256 workgroups, one per compute unit
 *             of a full MI355X, each streaming an equal share of the
 *             (16-row tile, K block) units in one launch; K is cut into
 *             split_k chunks (split_k divides k/128; with split_k > 1 every
 *             workgroup must get whole cells of one chunk); tiles that the
 *             share cuts into pieces are summed in a fixed order by the
 *             workgroup completing them, found with one 64-bit arrival
 *             counter per tile in the workspace; waves_k streaming waves
 *             plus one output wave per workgroup, depth tiles in flight per
 *             wave, tiles_n of them requested before the activation cast;
 *             waves_n selects the partition: 1 = equal runs of units, tiles
 *             cut where needed; 2 = whole tiles only (split_k must be 1),
 *             the workgroups' tile counts differing by at most one, no
 *             workspace; needs n*k < 2^31 and m <= 32).
 *             MFMA_ROWS_DMA (tile-layout weights, m <= 16: the work split
 *             of MFMA_ROWS with 8 waves along K,
 *             the weight tiles streamed into a ring of `depth` LDS stages of
 *             16 KB (3 or 6) by four more waves that only issue direct
 *             loads; waves_k must be 8, tiles_n, waves_n and split_k 1; the
 *             staged activations and the ring must fit in the LDS).
 *             Paths 1-4 and 6-8 take m <= 32.
 *   tiles_n   MFMA: 16-row tiles per wave (1, 2, 4); DOT: 8-row groups per wave (1, 2, 4)
 *   waves_n   waves side by side along N in one workgroup (1, 2, 4)
 *   waves_k   waves splitting a workgroup's K range (1, 2, 4, 8); their
 *             partials are summed in wave order inside the workgroup
 *   depth     K blocks of weights each wave keeps in flight (1..8)
 *   split_k   workgroups splitting K (1..64); their fp32 partials are summed
 *             in split order, never with atomics on data
 *   reduce    how split partials are combined when split_k > 1:
 *             FP8BS_REDUCE_KERNEL = a second kernel sums them;
 *             FP8BS_REDUCE_LAST_ARRIVER = in the same launch, the last
 *             workgroup of each output tile to finish sums them in split
 *             order. It is found with one 64-bit integer arrival counter per
 *             tile, kept in the workspace and tagged with a per-launch epoch,
 *             so the workspace still needs no initialization. The integer
 *             counter is the only atomic; the partials are plain loads and
 *             stores summed in a fixed order.
 *   epilogue  where the SwiGLU epilogue of fp8bs_gemm_swiglu* runs (ignored
 *             by the plain GEMM calls; set it to 0 there):
 *             FP8BS_EPILOGUE_SEPARATE = with split_k > 1 in the kernel that
 *             sums the split partials, otherwise in a second small kernel;
 *             FP8BS_EPILOGUE_IN_GEMM = (split_k == 1, MFMA grid or row-range
 *             paths) inside the GEMM launch: the workgroup that completes
 *             the outputs of a 128-column block of h, found with one 64-bit
 *             arrival counter per block in the workspace, applies it.
 *   weight_layout  how w_fp8 is stored: FP8BS_LAYOUT_ROWS (row-major
 *             [n][k], every path) or FP8BS_LAYOUT_TILES (the tile layout of
 *             fp8bs_pack_weight; MFMA, MFMA_ROWS, MFMA_STREAM and
 *             MFMA_ROWS_REG paths, for the kernel shapes the tile-layout
 *             table selects, and PREFILL with the direct-load kernel of 2
 *             stages and the wide kernel; not with DOT, nor with the
 *             SwiGLU epilogue inside the GEMM).                            */
typedef struct {
  int32_t path;
  int32_t tiles_n;
  int32_t waves_n;
  int32_t waves_k;
  int32_t depth;
  int32_t split_k;
  int32_t reduce;
  int32_t epilogue;
  int32_t weight_layout;
} fp8bs_gemm_config;

/* The configuration fp8bs_gemm uses for this shape (a fixed table: the same
 * shape always gets the same configuration, hence the same bits).          */
fp8bs_status fp8bs_gemm_select_config(int64_t m, int64_t n, int64_t k,
                                      fp8bs_gemm_config* out);

/* Workspace bytes a given configuration needs.                              */
size_t fp8bs_gemm_config_workspace_bytes(const fp8bs_gemm_config* cfg,
                                         int64_t m, int64_t n, int64_t k);

/* Self-check of the stream-K work partition (path MFMA_STREAMK) for an
 * n x k weight cut into `split` K chunks over `workgroups` workgroups
 * (whole = 1: the whole-tile partition, waves_n = 2 in a configuration), run
 * on the host with the partition code the kernel runs: 0 when every (16-row
 * tile, K block) unit is computed exactly once, each workgroup stays in one
 * K chunk, and every tile's pieces are listed in K order in distinct
 * workspace slots; 1 when the partition is not one the kernel supports;
 * another value names the first inconsistency found. No GPU is involved.  */
int32_t fp8bs_streamk_plan_check(int64_t n, int64_t k, int32_t split, int32_t workgroups,
                                 int32_t whole);

/* fp8bs_gemm / fp8bs_gemm_q with an explicit configuration (cfg != NULL).
 * x_bf16 != NULL selects the fused cast; otherwise x_fp8 and x_scale are
 * used.                                                                     */
fp8bs_status fp8bs_gemm_ex(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale,
                           int64_t m,
                           const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                           void* y_bf16, void* workspace, size_t workspace_bytes,
                           const fp8bs_gemm_config* cfg, void* stream);

/* ---- tile layout of the weight codes -------------------------------------
 * The same E4M3 codes and scales as above, stored so that the decode GEMM
 * streams them with contiguous loads: the codes of 16 rows x 128 columns
 * (one K block of one 16-row matrix-core tile) are 2 KB of consecutive
 * bytes, tile (r/16, kb) at byte ((r/16) * (k/128) + kb) * 2048. Inside a
 * tile, bytes 0..1023 hold columns 32g + 0..15 and bytes 1024..2047 columns
 * 32g + 16..31 of each 32-column quarter g; within each KB the 16 bytes of
 * row r%16, quarter g sit at (16g + r%16) * 16. The layout is a property of
 * the storage only: the GEMM computes the product defined at the top of this
 * header on the same codes, and with the same kernel configuration the
 * result is bit-identical to the row-major call. Weights are rearranged
 * once, like the quantization itself. The weight scales keep their layout.
 * Every m the row-major calls take is served: the decode kernels (m <= 32)
 * and the prefill kernel (m > 32) both have tile-layout builds.             */

/* Rearrange row-major codes w_fp8 [n][k] into the tile layout (n*k bytes at
 * w_tiles, which must not overlap w_fp8). Both pointers 16-byte aligned;
 * n*k up to 2^43 bytes (else FP8BS_ERR_SHAPE).                              */
fp8bs_status fp8bs_pack_weight(const uint8_t* w_fp8, int64_t n, int64_t k, uint8_t* w_tiles,
                               void* stream);

/* fp8bs_gemm on tile-layout weights (activation cast fused), 0 <= m <= 2^20.
 * Workspace as for fp8bs_gemm (fp8bs_gemm_workspace_bytes covers both
 * layouts).                                                                 */
fp8bs_status fp8bs_gemm_tiles(const void* x_bf16, int64_t m, const uint8_t* w_tiles,
                              const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                              void* workspace, size_t workspace_bytes, void* stream);

/* fp8bs_gemm_q on tile-layout weights; the same configuration as
 * fp8bs_gemm_tiles, so fp8bs_gemm_tiles(x) == fp8bs_gemm_q_tiles(
 * fp8bs_quantize_act(x)) bit for bit.                                       */
fp8bs_status fp8bs_gemm_q_tiles(const uint8_t* x_fp8, const float* x_scale, int64_t m,
                                const uint8_t* w_tiles, const float* w_scale, int64_t n,
                                int64_t k, void* y_bf16, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The configuration fp8bs_gemm_tiles uses for this shape (weight_layout =
 * FP8BS_LAYOUT_TILES): a fixed table of the same shape and m classes as
 * fp8bs_gemm_select_config's, measured on tile-layout weights (the MFMA
 * grid kernels gain most from the layout, so it takes them more often).    */
fp8bs_status fp8bs_gemm_tiles_select_config(int64_t m, int64_t n, int64_t k,
                                            fp8bs_gemm_config* out);

/* ---- MLP epilogue: SwiGLU and the FP8 cast of its output ------------------
 * Fusing the element-wise steps between the matmuls of a transformer layer
 * into the matmul ("Kernel-Level Optimisations for LLM Inference and
 * Training", section "Scheduling decides the shapes your kernels see", on
 * fused SwiGLU) and casting the down projection's input to FP8 ("The
 * profiler said the kernel ran zero times", section "What the trace
 * showed"). SwiGLU is the published gated unit (Shazeer, "GLU Variants
 * Improve Transformer"): h = silu(gate) * up, silu(g) = g / (1 + e^-g).
 *
 * Layout: the up/gate projection's output y [m][2*inter] bf16 holds the gate
 * in columns 0 .. inter-1 and the up projection in inter .. 2*inter-1 (its
 * weight stacks the gate rows above the up rows). h is evaluated in fp32 on
 * the bf16 gate and up values, rounded to bf16, then cast per row per 128
 * columns with the activation rule of fp8bs_quantize_act: codes h_fp8
 * [m][inter], scales h_scale [m][inter/128] fp32, ready for fp8bs_gemm_q of
 * the down projection. inter must be a multiple of 128. Every way of running
 * it (standalone, after a split sum, inside the GEMM) gives the same bits.
 * Alignment: y_bf16 and h_fp8 16 bytes, h_scale 4 bytes.                    */

/* Standalone epilogue: y [m][2*inter] bf16 -> h codes and scales.           */
fp8bs_status fp8bs_swiglu_quant(const void* y_bf16, int64_t m, int64_t inter, uint8_t* h_fp8,
                                float* h_scale, void* stream);

/* The up/gate projection with the epilogue fused in, in one call: y = X . W^T
 * exactly as fp8bs_gemm computes it (written to y_bf16, [m][n]; with the
 * same kernel configuration the bits are identical), and h_fp8 / h_scale as
 * fp8bs_swiglu_quant(y) gives them, bit for bit. n = 2*inter must be a
 * multiple of 256; 0 <= m <= 65535. The automatic choice is fp8bs_gemm's
 * configuration with FP8BS_EPILOGUE_SEPARATE (the faster way at decode sizes
 * on MI355X: the epilogue rides on the split-sum kernel when K is split, and
 * takes a second small kernel otherwise). The workspace holds the split
 * partials or, for FP8BS_EPILOGUE_IN_GEMM, one 64-bit arrival counter per
 * 128-column block of h (tagged with a per-launch epoch: no initialization
 * needed); size from fp8bs_gemm_swiglu_workspace_bytes. Calls that share a
 * workspace must be ordered on one stream.                                  */
fp8bs_status fp8bs_gemm_swiglu(const void* x_bf16, int64_t m, const uint8_t* w_fp8,
                               const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                               uint8_t* h_fp8, float* h_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/* fp8bs_gemm_swiglu on tile-layout weights (fp8bs_pack_weight), 0 <= m <= 65535:
 * y bit-identical to fp8bs_gemm_tiles on the same inputs, h as
 * fp8bs_swiglu_quant(y). The epilogue runs after the split sum or in a
 * second kernel (FP8BS_EPILOGUE_SEPARATE); workspace as for
 * fp8bs_gemm_tiles (fp8bs_gemm_workspace_bytes covers it).                  */
fp8bs_status fp8bs_gemm_swiglu_tiles(const void* x_bf16, int64_t m, const uint8_t* w_tiles,
                                     const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                                     uint8_t* h_fp8, float* h_scale, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Same with an explicit configuration (cfg != NULL; x_bf16 != NULL selects
 * the fused cast, otherwise x_fp8 / x_scale). Accepted with
 * FP8BS_EPILOGUE_SEPARATE: every configuration fp8bs_gemm_ex accepts except
 * the last-arriver reduce. With FP8BS_EPILOGUE_IN_GEMM: split_k == 1 on the
 * MFMA path, or on the MFMA_ROWS / MFMA_STREAM / MFMA_ROWS_REG paths for
 * the compiled shapes (waves_k 8 with depth 3, 4 or 6; MFMA_STREAM, depth 4
 * or 6; MFMA_ROWS_REG, depth 5 with tiles_n 1).
 * Anything else is FP8BS_ERR_CONFIG.                                        */
fp8bs_status fp8bs_gemm_swiglu_ex(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale,
                                  int64_t m, const uint8_t* w_fp8, const float* w_scale,
                                  int64_t n, int64_t k, void* y_bf16, uint8_t* h_fp8,
                                  float* h_scale, void* workspace, size_t workspace_bytes,
                                  const fp8bs_gemm_config* cfg, void* stream);

/* The configuration fp8bs_gemm_swiglu uses (fp8bs_gemm's, epilogue
 * FP8BS_EPILOGUE_SEPARATE).                                                 */
fp8bs_status fp8bs_gemm_swiglu_select_config(int64_t m, int64_t n, int64_t k,
                                             fp8bs_gemm_config* out);

/* Workspace bytes of the fused call for cfg (NULL = the automatic choice);
 * 0 for shapes it rejects or that need none.                                */
size_t fp8bs_gemm_swiglu_workspace_bytes(const fp8bs_gemm_config* cfg, int64_t m, int64_t n,
                                         int64_t k);

/* ---- utilities ----------------------------------------------------------- */

/* Encode fp32 values to E4M3 codes with the quantizers' rounding rule
 * (nearest, ties to even mantissa, saturate at +-448, sign kept).
 * mode 0 = the encoder the quantizers use; 1 = the hardware conversion
 * instruction; 2 = the integer software encoder. in/out 4-byte aligned.     */
fp8bs_status fp8bs_encode_e4m3(const float* in, int64_t count, uint8_t* out,
                               int32_t mode, void* stream);

/* Human-readable name of a status.                                          */
const char* fp8bs_status_string(fp8bs_status s);

/* Host-side count of launches of each kernel family since load: 0 = weight
 * quantizer, 1 = activation quantizer, 2 = MFMA GEMM, 3 = DOT GEMM,
 * 4 = split reduce (plain or with the SwiGLU epilogue), 5 = encoder utility,
 * 6 = read/copy diagnostics, 7 = standalone SwiGLU epilogue,
 * 8 = weight rearrangement into the tile layout.
 * Lets a caller check that the kernels it benchmarks actually ran.          */
uint64_t fp8bs_launch_count(int32_t which);

/* Build identification string (compiler, target, flags).                    */
const char* fp8bs_build_info(void);

/* ---- diagnostics (bandwidth reference kernels) --------------------------- */

/* Streaming read of `bytes` bytes (multiple of 16, 16-byte aligned); sink
 * is a 16-byte device buffer written only on an impossible checksum, so the
 * reads cannot be elided. blocks = workgroups of 256 threads (0 = about
 * four 16-byte loads per lane, at most 16 per CU).                          */
fp8bs_status fp8bs_diag_read(const void* src, size_t bytes, void* sink, int32_t blocks,
                             void* stream);

/* Streaming-read ceiling over `bytes` bytes (multiple of 16, 16-byte
 * aligned): `blocks` workgroups of 512 threads each read one contiguous
 * range of about bytes/blocks with non-temporal 16-byte loads, 2 * depth
 * loads per lane in flight (depth 4, 8 or 16); or (depth 0) workgroups of
 * 4 waves request the range's 1 KB pieces straight into LDS, unpaced
 * (non-temporal direct-to-LDS loads, one workgroup per compute unit). The
 * plain read a weight stream could reach at best at this size; sink as for
 * fp8bs_diag_read (unused with depth 0). bytes/blocks must stay below about
 * 2^31.                                                                     */
fp8bs_status fp8bs_diag_stream(const void* src, size_t bytes, void* sink, int32_t blocks,
                               int32_t depth, void* stream);

/* Writes the GPU's constant-rate wall-clock counter to out[0] (8-byte
 * aligned device pointer) when the launch runs on `stream`: two of them
 * around a run of kernels in a captured graph time exactly that run.
 * fp8bs_diag_timestamp_hz gives the counter's rate for the current device
 * (0 if it cannot be read).                                                */
fp8bs_status fp8bs_diag_timestamp(uint64_t* out, void* stream);
uint64_t fp8bs_diag_timestamp_hz(void);

/* Plain copy of `bytes` bytes (multiple of 16, both 16-byte aligned).       */
fp8bs_status fp8bs_diag_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
