/* fp8gemm.h -- block-scaled FP8 GEMM library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes is defined on "DeepSeek open-source week, day 3:
 * DeepGEMM" (explinks.com): an FP8 E4M3 GEMM in NT layout (LHS m x k not
 * transposed, RHS n x k "transposed", both K-contiguous) with fine-grained
 * scaling -- one FP32 scale per row and 128-wide K group on the LHS, one FP32
 * scale per 128 x 128 block on the RHS -- and a BF16 output ("Basic usage"
 * example); partial products are promoted into an FP32 accumulator once per
 * 128-wide K group, final += (scale_a * scale_b) * partial ("Core features",
 * two-level accumulation; "Source walk-through" part 3).  The same core runs
 * as a dense GEMM, as a contiguous-layout grouped GEMM (MoE prefill: experts'
 * rows concatenated along M) and as a masked-layout grouped GEMM (MoE decode:
 * a fixed slot per group plus a device tensor of valid row counts, so the
 * host never learns them) -- the page's three GEMM kinds.  Per-token-group
 * activation quantisation (scale = amax / 448, q = fp8(x / scale)) follows
 * the kwkr.cn DeepGEMM usage article, section 3.1 and its section 4.2 code.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to dense row-major storage.  FP8
 *     tensors hold OCP E4M3FN codes (uint8); BF16 tensors hold bit patterns
 *     (uint16); scales are FP32.  Every pointer must be 16-byte aligned.
 *   - KG = ceil(k / 128) and NB = ceil(n / 128).
 *   - LHS scales are stored MN-major: element (row r, K group g) lives at
 *     lhs_scales[g * lhs_scales_ld + r], with rows <= lhs_scales_ld <
 *     2^31 and lhs_scales_ld % 4 == 0.  RHS scales are row-major [NB][KG].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream, never synchronises and never reads device
 *     data on the host, so calls may be captured into a HIP graph.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     retains caller memory.
 *   - Errors that the host can check are reported before anything is
 *     launched: FP8G_EINVAL for null pointers, negative sizes or misaligned
 *     pointers; FP8G_EUNSUPPORTED for shapes outside this version's limits
 *     (k % 128 != 0, k > 65536, n % 8 != 0, contiguous m_total % 128 != 0,
 *     a bad scales ld); FP8G_ELAUNCH if the launch itself fails.  No C++ exception
 *     crosses this interface.
 *   - Zero-sized problems (m = 0, n = 0, num_groups = 0) succeed and launch
 *     nothing.
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP8G_OK = 0,
  FP8G_EINVAL = -1,
  FP8G_EUNSUPPORTED = -2,
  FP8G_ELAUNCH = -3,
  FP8G_ESCRATCH = -4  /* fp8_gemm_nt_noalloc: the problem needs more than its static scratch */
};

/* Element type of the cast helper's input. */
enum { FP8G_F32 = 0, FP8G_BF16 = 1 };

/* FP8 formats ("DeepGEMM: FP8 GEMM kernel optimisation practice on Hopper
 * Tensor Cores", sections 1.3 and 3.1: A and B in E4M3 or E5M2).  OCP E4M3FN
 * (max 448, no infinities) and OCP E5M2 (max 57344).  The entry points
 * without a format argument use E4M3. */
enum { FP8G_E4M3 = 0, FP8G_E5M2 = 1 };

/* Dense NT GEMM: out[m][n] = bf16( sum_k dec(lhs[i][t]) * sa(i, t/128)
 *                                        * dec(rhs[j][t]) * sb(j/128, t/128) ),
 * evaluated with one FP32 promotion per 128-wide K group.
 *   lhs        [m][k] E4M3 codes;   lhs_scales [KG][lhs_scales_ld] FP32
 *   rhs        [n][k] E4M3 codes;   rhs_scales [NB][KG] FP32
 *   out        [m][n] BF16 (written in full)
 *   workspace  optional device scratch (16-byte aligned) for split-K: per
 *              output tile an arrival counter, then the FP32 partial sums.
 *              Pass at least fp8_gemm_workspace_bytes() bytes to allow
 *              split-K; a smaller (or NULL) workspace selects a configuration
 *              without split-K, which is never an error.  The workspace needs
 *              no initialisation (each counter carries a tag; a word without
 *              the library's current tag is restarted) and is left in a
 *              state the next call accepts, also under HIP graph replay;
 *              two calls that may run concurrently must not share a
 *              workspace.  A split call that fails with FP8G_ELAUNCH may
 *              leave counts part-way: the library then moves to a new tag,
 *              but a graph captured before the failure that uses the same
 *              workspace must be captured again.  The last workgroup to
 *              finish a tile adds the partials in split order, so a given
 *              configuration always produces bit-identical output; results
 *              with and without split-K differ only by FP32 rounding
 *              order. */
int fp8_gemm_nt(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                const uint8_t* rhs, const float* rhs_scales,
                uint16_t* out, int m, int n, int k,
                void* workspace, size_t workspace_bytes, void* stream);

/* fp8_gemm_nt for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes
 * no workspace and allocates nothing; the split-K arrival counters and
 * partial sums live in a static device array of 32 MiB inside the library
 * (one per device, allocated when the library's code is loaded there and
 * held until the process ends).  Same arguments, checks and configuration
 * as fp8_gemm_nt with a large enough workspace, so the same bits.  A
 * problem whose configuration needs more than 32 MiB of split-K scratch is
 * refused with FP8G_ESCRATCH before anything is launched (on a 256-CU
 * device the library's own configurations need at most about 16 MiB).
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: the arrival counters
 * carry a tag, as with fp8_gemm_nt's workspace): calls that may overlap on
 * one device -- other streams, other threads, other graphs in flight --
 * race on it and must be serialised (one stream) by the caller.  The first call on a device looks
 * up the array's device address (no allocation and no stream operation);
 * make one call before capturing the entry point in a HIP graph. */
int fp8_gemm_nt_noalloc(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                        const uint8_t* rhs, const float* rhs_scales,
                        uint16_t* out, int m, int n, int k, void* stream);

/* Host only, launches nothing: writes a one-line description of the dense
 * configuration fp8_gemm_nt picks for (m, n, k) when the split-K workspace
 * is large enough ("tile=BMxBN waves=W stages=S ku=U splits=P grid=G", or
 * "empty"), NUL-terminated and truncated to len bytes.  The counterpart of
 * the JIT debug output in "DeepSeek open-source week, day 3: DeepGEMM"
 * (environment variables).  FP8G_EINVAL for a null buffer or negative m;
 * FP8G_EUNSUPPORTED for n, k fp8_gemm_nt rejects. */
int fp8_gemm_describe(int m, int n, int k, char* buf, size_t len);

/* Host only, launches nothing: the tile scheduler's decision for every
 * workgroup of a GEMM call, for checking the scheduler without a device.
 * "DeepSeek open-source week, day 3: DeepGEMM" lets the grouped kinds skip
 * what has no work (the contiguous kind's per-row group index, the masked
 * kind's device-side counts); this reports which work unit each workgroup
 * takes, decoded by the same functions the kernels run, across the
 * consecutive launches a CU limit (fp8_set_num_cus) makes.
 *   mode        FP8G_JIT_DENSE (the configuration fp8_gemm_nt picks with a
 *               large enough workspace), FP8G_JIT_CONTIGUOUS or
 *               FP8G_JIT_MASKED (the ahead-of-time grouped kernels)
 *   m           dense: m; contiguous: m_total; masked: max_m
 *   group_data  HOST int32 array: contiguous m_indices [m]; masked
 *               masked_m [num_groups]; dense: unused (may be NULL)
 *   units       HOST int32 [capacity][6], one record per workgroup in launch
 *               order: {taken (1 = has a unit, 0 = exits), group, first row,
 *               rows, column tile, split}; records past capacity are not
 *               written
 * Returns the number of workgroups of the call (>= 0), or a negative status
 * (FP8G_EINVAL for bad arguments, FP8G_EUNSUPPORTED for shapes the GEMM
 * entry points reject). */
int fp8_gemm_schedule(int mode, int m, int n, int k, int num_groups, const int32_t* group_data,
                      int32_t* units, int capacity);

/* fp8_gemm_nt with each operand's format given: lhs_format / rhs_format are
 * FP8G_E4M3 or FP8G_E5M2, in any combination (FP8G_EINVAL otherwise).  The
 * arithmetic is the same; only the decoding of the codes changes. */
int fp8_gemm_nt_fmt(const uint8_t* lhs, int lhs_format, const float* lhs_scales, int64_t lhs_scales_ld,
                    const uint8_t* rhs, int rhs_format, const float* rhs_scales,
                    uint16_t* out, int m, int n, int k,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Contiguous-layout grouped GEMM (MoE prefill / training forward).
 *   lhs        [m_total][k];  lhs_scales [KG][lhs_scales_ld >= m_total]
 *   rhs        [num_groups][n][k];  rhs_scales [num_groups][NB][KG]
 *   m_indices  [m_total] int32 on the device: the group of each row.  Rows
 *              are consumed in aligned blocks of 128; every row of a block
 *              must carry the same index (each expert's row count is a
 *              multiple of 128).  A negative index marks a block whose
 *              output rows are left untouched.  An index >= num_groups is
 *              undefined behaviour.
 *   out        [m_total][n] BF16
 *   m_total % 128 must be 0.  The workspace is not used (may be NULL). */
int fp8_grouped_gemm_contiguous(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                const uint8_t* rhs, const float* rhs_scales,
                                uint16_t* out, const int32_t* m_indices,
                                int m_total, int n, int k, int num_groups,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Masked-layout grouped GEMM (MoE decode).
 *   lhs        [num_groups][max_m][k];
 *   lhs_scales [num_groups][KG][lhs_scales_ld >= max_m]
 *   rhs        [num_groups][n][k];  rhs_scales [num_groups][NB][KG]
 *   masked_m   [num_groups] int32 on the device: valid rows per group,
 *              clamped to [0, max_m].  Only rows r < masked_m[g] of group g
 *              are computed and written; every other row of `out` is left
 *              untouched, and whatever the LHS rows or scales past the count
 *              hold (NaN codes included) cannot reach a written element.
 *   out        [num_groups][max_m][n] BF16
 *   The workspace is not used (may be NULL). */
int fp8_grouped_gemm_masked(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                            const uint8_t* rhs, const float* rhs_scales,
                            uint16_t* out, const int32_t* masked_m,
                            int num_groups, int max_m, int n, int k,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Per-token-group cast (kwkr.cn usage article, section 3.1 and 4.2 code):
 * for each row and each 128-wide K group, amax = max |x|, scale =
 * fl32(amax / 448) (1.0 when amax == 0), q = E4M3(fl32(x / scale)) rounded to
 * nearest-even (saturating at +-448), with IEEE correctly rounded fp32
 * division.  Inputs must be finite.
 *   x       [m][k] FP32 (x_dtype FP8G_F32) or BF16 bits (FP8G_BF16)
 *   q       [m][k] E4M3 codes
 *   scales  [KG][scales_ld >= m] FP32 (the MN-major layout the GEMMs read) */
int fp8_cast_per_token_group(const void* x, int x_dtype, int m, int k,
                             uint8_t* q, float* scales, int64_t scales_ld, void* stream);

/* ---- Runtime shape specialisation -------------------------------------------
 * ("DeepSeek open-source week, day 3: DeepGEMM", "Core features": kernels
 * compiled at run time per shape; its environment-variable list: a cache
 * directory and JIT debug output; the kwkr.cn usage article, sections 2.3
 * and 3.3: per-shape compilation, a warm-up, a cache kept across restarts.)
 *
 * The fp8_jit_* GEMMs take the same arguments as the entry points above plus
 * a tile configuration (NULL: the one the ahead-of-time path would use).
 * The kernel for (configuration, operand formats, target, and n and k when
 * `specialize` is set) is compiled on first use by the ROCm compiler run as
 * a child process, with the device code-generation options of the library
 * build, kept on disk in the
 * cache directory (default $FP8G_CACHE_DIR, else $HOME/.cache/fp8gemm) and
 * loaded once per device per process.  A cache file that does not match its
 * key, size or checksum is ignored, counted and replaced.  A build that
 * would need scratch memory (register spills) is refused with
 * FP8G_EUNSUPPORTED, and the refusal is recorded in the cache, so later
 * processes refuse it without compiling.  The first call
 * for a configuration therefore compiles (about a second) or reads the
 * disk; later calls only launch.  FP8G_JIT_DEBUG=1 reports compilations and
 * cache use on stderr; FP8G_JIT_COMPILER names the compiler (default
 * $ROCM_PATH/llvm/bin/clang++); without a device, FP8G_JIT_TARGET names the
 * target to build for (default gfx950), so a cache can be filled ahead of
 * time for another machine.  Calls are thread-safe; a first call of a
 * configuration compiles or loads a module, which is not a stream operation:
 * warm a configuration up (fp8_jit_warmup or one call) before capturing its
 * calls in a HIP graph.  Results equal the ahead-of-time kernels' for the
 * same configuration. */
enum { FP8G_JIT_DENSE = 0, FP8G_JIT_CONTIGUOUS = 1, FP8G_JIT_MASKED = 2 };

typedef struct fp8_gemm_config {
  int block_m;      /* tile rows (tokens), <= 256, a multiple of 8 * waves */
  int block_n;      /* tile columns (outputs), <= 256, a multiple of 8 * waves */
  int waves_m;      /* wave grid over the tile: waves_m * waves_n * waves_k is 4 or 8; */
  int waves_n;      /*   each wave's share is a multiple of 16 by 16, at most 32 MFMA */
  int waves_k;      /*   tiles, and its n range divides 128 */
  int stages;       /* LDS ring stages, 1..8; 1 is the single-buffer debug form
                       ("DeepGEMM: FP8 GEMM kernel optimisation practice on
                       Hopper Tensor Cores", section 6.2): no copy overlaps
                       the products.  FP8G_PIPELINE_DEPTH=d sets every
                       configuration's stages to d. */
  int k_per_stage;  /* 128-wide K groups per stage, 1..4, a multiple of waves_k */
  int splits;       /* split-K workgroups per tile, 1..8 (dense only; grouped: 1) */
  int specialize;   /* nonzero: n and k are compiled in */
} fp8_gemm_config;

/* The configuration the ahead-of-time path uses for `mode` (FP8G_JIT_*) and
 * this shape. */
int fp8_jit_default_config(int mode, int m, int n, int k, fp8_gemm_config* config);
/* FP8G_OK if `config` can be built for `mode`, FP8G_EUNSUPPORTED if not
 * (limits listed in fp8_gemm_config; LDS use <= 160 KB). */
int fp8_jit_config_supported(int mode, const fp8_gemm_config* config);
/* Compiles (or finds in the cache) and loads the kernel for a shape without
 * launching it: the warm-up before timing.  Without a device it only fills
 * the disk cache. */
int fp8_jit_warmup(int mode, int n, int k, int lhs_format, int rhs_format, const fp8_gemm_config* config);
/* Split-K workspace of fp8_jit_gemm_nt for this configuration (0 if none);
 * fp8_jit_gemm_nt uses it as fp8_gemm_nt uses its workspace (same layout,
 * same counter tag, no initialisation needed). */
size_t fp8_jit_gemm_workspace_bytes(int m, int n, int k, const fp8_gemm_config* config);
int fp8_jit_gemm_nt(const uint8_t* lhs, int lhs_format, const float* lhs_scales, int64_t lhs_scales_ld,
                    const uint8_t* rhs, int rhs_format, const float* rhs_scales,
                    uint16_t* out, int m, int n, int k, const fp8_gemm_config* config,
                    void* workspace, size_t workspace_bytes, void* stream);
/* config->block_m must be 256 (tiles are one or two 128-row blocks). */
int fp8_jit_grouped_gemm_contiguous(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                    const uint8_t* rhs, const float* rhs_scales,
                                    uint16_t* out, const int32_t* m_indices,
                                    int m_total, int n, int k, int num_groups,
                                    const fp8_gemm_config* config, void* stream);
int fp8_jit_grouped_gemm_masked(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                const uint8_t* rhs, const float* rhs_scales,
                                uint16_t* out, const int32_t* masked_m,
                                int num_groups, int max_m, int n, int k,
                                const fp8_gemm_config* config, void* stream);
/* Cache directory for later compilations (NULL or "": the default). */
int fp8_jit_set_cache_dir(const char* dir);
int fp8_jit_get_cache_dir(char* buf, size_t len);
/* Up to 5 counters since the library was loaded: kernels found loaded in
 * memory, read from the disk cache, compiled, cache files rejected,
 * compilations that failed. */
int fp8_jit_stats(long long* counts, int n);

/* The per-token-group cast to either format: q_format FP8G_E4M3 (scale =
 * amax / 448) or FP8G_E5M2 (scale = amax / 57344, q = E5M2(x / scale),
 * round-to-nearest-even, saturating at +-57344). */
int fp8_cast_per_token_group_fmt(const void* x, int x_dtype, int q_format, int m, int k,
                                 uint8_t* q, float* scales, int64_t scales_ld, void* stream);

/* 128 x 128 block cast for weights (the RHS scale granularity of the
 * "Basic usage" example): one scale per block, computed as above over the
 * block's real elements (edge blocks may be partial).
 *   w       [n][k] FP32;  q [n][k] E4M3 codes;  scales [NB][KG] FP32 */
int fp8_cast_per_block(const float* w, int n, int k,
                       uint8_t* q, float* scales, void* stream);
/* The same to either format (q_format as for fp8_cast_per_token_group_fmt). */
int fp8_cast_per_block_fmt(const float* w, int q_format, int n, int k,
                           uint8_t* q, float* scales, void* stream);

/* ---- MoE layout steps around the grouped GEMMs -----------------------------
 * The flow of the kwkr.cn DeepGEMM usage article (section 3.2; section 4.3:
 * order the tokens by expert index, count each expert's tokens, run the
 * grouped GEMM, put the outputs back in token order), producing the two
 * grouped layouts of "DeepSeek open-source week, day 3: DeepGEMM".  Token t
 * is routed to expert expert_idx[t]; an index outside [0, num_groups) routes
 * it nowhere.  rank[t] = number of earlier tokens routed to the same expert
 * (a stable order, so every output below is unique).  num_groups <= 1024.
 * All arrays are int32 device arrays (4-byte aligned).  The layout calls
 * need a caller workspace of fp8_moe_layout_workspace_bytes() bytes; it
 * needs no initialisation and is not shared by concurrent calls. */

/* Rows that always suffice for the contiguous layout of num_tokens tokens
 * over num_groups experts (each expert pads to a multiple of 128); -1 on bad
 * arguments.  Host-only. */
int fp8_moe_contiguous_rows(int num_tokens, int num_groups);
size_t fp8_moe_layout_workspace_bytes(int num_tokens, int num_groups);

/* Contiguous layout (MoE prefill):
 *   counts[G]        tokens per expert
 *   offsets[G + 1]   offsets[g + 1] = offsets[g] + ceil(counts[g] / 128) * 128
 *   dst_row[T]       offsets[e] + rank[t], or -1 for an unrouted token
 *   m_indices[m_rows] expert of each laid-out row (its padding rows too),
 *                    -1 from offsets[G] on: the input of
 *                    fp8_grouped_gemm_contiguous (m_total = m_rows).
 * m_rows must be at least fp8_moe_contiguous_rows(T, G) (FP8G_EINVAL
 * otherwise).  Padding rows receive no token: fill them (e.g. with zero
 * codes) before the GEMM if their outputs are to be defined. */
int fp8_moe_layout_contiguous(const int32_t* expert_idx, int num_tokens, int num_groups,
                              int32_t* counts, int32_t* offsets, int32_t* dst_row,
                              int32_t* m_indices, int m_rows,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Masked layout (MoE decode): a slot of max_m rows per expert.
 *   counts[G]    tokens per expert
 *   dst_row[T]   e * max_m + rank[t] when rank[t] < max_m, else -1 (the
 *                token does not fit its expert's slot and is dropped)
 *   masked_m[G]  min(counts[g], max_m): the input of fp8_grouped_gemm_masked */
int fp8_moe_layout_masked(const int32_t* expert_idx, int num_tokens, int num_groups, int max_m,
                          int32_t* counts, int32_t* dst_row, int32_t* masked_m,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Moves each token's E4M3 row and its scales to its laid-out row d =
 * dst_row[t] (tokens with d < 0 or d >= out_rows stay put):
 *   q [T][k] codes, scales MN-major [KG][scales_ld >= T] (the cast's output);
 *   q_out [out_rows][k]; scales_out: row d sits in group d / rows_per_group,
 *   at row d % rows_per_group of that group's MN-major
 *   [KG][scales_out_ld >= rows_per_group] block.  Contiguous layout:
 *   rows_per_group = out_rows (one block); masked layout: rows_per_group =
 *   max_m, out_rows = G * max_m.  k % 16 == 0; q and q_out 16-byte aligned.
 * Rows no token lands on are not written. */
int fp8_moe_scatter_rows(const uint8_t* q, const float* scales, int64_t scales_ld,
                         int num_tokens, int k, const int32_t* dst_row,
                         int rows_per_group, int out_rows,
                         uint8_t* q_out, float* scales_out, int64_t scales_out_ld, void* stream);

/* Puts the GEMM's BF16 rows back in token order: out[t] = y[dst_row[t]]
 * (out [T][n], y [y_rows][n]); a row of zeros where dst_row[t] < 0 or
 * >= y_rows.  n % 8 == 0; y and out 16-byte aligned. */
int fp8_moe_gather_rows(const uint16_t* y, int n, int y_rows, const int32_t* dst_row,
                        int num_tokens, uint16_t* out, void* stream);

/* Workspace bytes that let fp8_gemm_nt choose split-K for this shape
 * (0 = never needed).  An upper bound; depends on the CU limit in force. */
size_t fp8_gemm_workspace_bytes(int m, int n, int k, int num_groups);

/* Limit the number of compute units the GEMMs use (the page's "SM resource
 * control"), process-wide.  Tile choices are made for that many CUs, and a
 * GEMM with more workgroups than that runs as consecutive launches of at
 * most that many workgroups on its stream, so at most that many CUs run it
 * at any time and the rest stay free for concurrent work.  Results do not
 * depend on the slicing.  0 restores "all"; values above the device's count
 * are clamped.  Returns the previous value. */
int fp8_set_num_cus(int num_cus);
int fp8_get_num_cus(void);

/* Human-readable name of a status code (static storage). */
const char* fp8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H */
