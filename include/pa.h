/*
 * pa.h — C ABI of libpa: unified paged attention for AMD Instinct MI355X (gfx950).
 *
 * One call computes attention for a whole varlen batch in which every sequence
 * may have a different query length: decode steps (one query), chunks of a
 * chunked prefill and whole prefills are served by the same launch.  The call
 * follows the flash_attn_varlen_func statement of the problem that the unified
 * kernel adopts (page "[Kernel] Unified Triton kernel that doesn't distinguish
 * between prefill + decode", PR description), reads keys and values from a
 * paged cache in the FlashAttention layout (same passage), and needs no
 * metadata beyond what a serving engine already has for chunked prefill plus
 * decode in one batch (page "[Kernel] [V1] Improved performance for V1 Triton
 * (ROCm) backend", section "How is this performance improvement achieved?").
 *
 * For query i (0-based) of sequence s, with q_s = cu_seqlens_q[s+1] -
 * cu_seqlens_q[s] queries and L_s = seqused_k[s] context tokens (the new tokens
 * included, already written to the cache), and q-head h reading kv-head
 * h / (Hq / Hkv):
 *
 *     out[cu_seqlens_q[s] + i, h, :] = sum_j softmax_j(scale * q . k_j) v_j
 *
 * over the admissible keys j: all j < L_s when causal == 0, and
 * j <= L_s - q_s + i when causal != 0 (the causal mask is aligned to the end
 * of each sequence's context, so a decode query sees its whole context and a
 * prefill chunk sees its cached prefix).  Key j of sequence s is slot
 * j % block_size of physical block block_table[s, j / block_size].  A row
 * with no admissible key (L_s == 0, or causal with q_s > L_s for the first
 * q_s - L_s queries) is written as exactly 0.
 *
 * No HIP header is needed to include this file.  Every data pointer in a
 * pa_tensor is a DEVICE pointer on the current HIP device; all shapes, strides
 * and scalars are passed by value on the host.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_VERSION 6   /* 6: pa_plan_info.unit_xcd, wide tiles at head sizes 96
                          and 256; 5: pa_plan_info.partial_rows; 4:
                          pa_workspace_bytes; 3: fp16 (PA_F16), block sizes
                          32 and 64, head sizes 96 and 256 */

/* Return codes.  Every failure is reported before anything is launched, with
 * one exception: PA_ERR_HIP, which may also come from the launch itself. */
typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  PA_ERR_DTYPE = -2,       /* wrong dtype code for an argument                 */
  PA_ERR_SHAPE = -3,       /* ndim or extents inconsistent between arguments   */
  PA_ERR_UNSUPPORTED = -4, /* valid but not built: head_dim, block_size, G ... */
  PA_ERR_ALIGN = -5,       /* pointer or stride breaks the 16-byte rule        */
  PA_ERR_ALIAS = -6,       /* out overlaps q, k_cache or v_cache               */
  PA_ERR_WORKSPACE = -7,   /* caller workspace missing or too small            */
  PA_ERR_CONTENT = -8,     /* metadata contents invalid (only when checked)    */
  PA_ERR_HIP = -9          /* the HIP runtime reported an error                */
} pa_status;

/* PA_FP8_E4M3: OCP 8-bit float E4M3 ("fn": finite, S.1111.111 is NaN), one
 * byte per element, for k_cache / v_cache only (page "[Kernel] [V1] Improved
 * performance for V1 Triton (ROCm) backend", review discussion of the
 * fp8_e4m3fn KV cache).  Element (b, t, h, i) of a cache then stands for
 * decode(code) * k_scale (keys) or * v_scale (values); see pa_options. */
/* PA_F16: IEEE binary16.  q, out and 16-bit caches are all bf16 or all fp16
 * (the element type is the caller's; the kernels compute in fp32 either way). */
typedef enum { PA_BF16 = 1, PA_INT32 = 2, PA_FP32 = 3, PA_FP8_E4M3 = 4, PA_F16 = 5 } pa_dtype;

/* A strided view of device memory.  shape/stride entries beyond ndim are
 * ignored; strides are in ELEMENTS. */
typedef struct {
  void* data;
  int32_t dtype;     /* pa_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} pa_tensor;

/* Test and tuning switches for pa_unified_attention_ex.  Zero-initialise
 * for defaults. */
typedef struct {
  int32_t force_num_splits; /* >0: split every row's keys into this many
                               key ranges merged by log-sum-exp (clamped so each
                               range holds at least one 64-key stage)          */
  int32_t force_tile;       /* 0: heuristic; 1: one query tile per sequence of
                               at most 16/G tokens (requires max_seqlen_q*G <=
                               16), persistent decode kernel; 2: wide query
                               tiles (128 rows, 32 per wave), and the wide
                               code path even for tiles of <= 16 rows; 3: as 1
                               but one work-group per item on the unified
                               kernel; 4: wide tiles of 256 rows on the
                               eight-wave kernel (two wave groups in opposite
                               phases; head_dim 64/128, 16-bit caches)        */
  int32_t check_contents;   /* !=0: copy the metadata to the host (synchronous)
                               and return PA_ERR_CONTENT if it breaks the
                               preconditions listed below                      */
  int32_t decode_grid;      /* >0: work-groups of the persistent decode kernel
                               (rounded down to a multiple of 8; default: the
                               resident work-groups of the device, or one per
                               CU when an even split streams 16-bit caches)   */
  float k_scale;            /* fp8 caches: dequantisation scale of k_cache
                               (0 reads as 1; ignored for bf16 caches)        */
  float v_scale;            /* fp8 caches: dequantisation scale of v_cache
                               (0 reads as 1; ignored for bf16 caches)        */
} pa_options;

/* Launch shape chosen for a batch (pa_plan_describe). */
typedef struct {
  int32_t tile_tokens;   /* query tokens per work-group tile                  */
  int32_t tile_rows;     /* packed (token, q-head) rows per tile              */
  int32_t num_slots;     /* query-tile slots in the grid                      */
  int32_t slots_direct;  /* 1: slot == sequence index (one tile per sequence) */
  int32_t num_splits;    /* key ranges per row (1: no merge kernel)           */
  int32_t split_keys;    /* keys per range (multiple of 64)                   */
  int64_t num_workgroups;/* main-kernel grid size                             */
  int64_t workspace_bytes;
  int32_t persistent;    /* 1: persistent decode kernel; items (sequence, key
                            split, kv-head) are enumerated on the device, and
                            num_splits bounds a row's split count            */
  int32_t balanced;      /* 1 (persistent only): even split.  The device lays
                            the rows (sequence, kv-head) end to end as one
                            stream of cache blocks and cuts it into equal
                            chunks, one or more per wave, so every wave
                            streams the same bytes however ragged the
                            lengths; a chunk has at least split_keys / 16
                            blocks and a row's parts are the chunks it
                            touches (at most num_splits)                     */
  int32_t longest_first; /* 1 (grid plans with wide tiles, at most 2048
                            sequences): work-group b takes the (b / Hkv)-th
                            (sequence, query tile, key split) in order of
                            decreasing key count, kv-head b % Hkv            */
  int32_t unit_xcd;      /* 1 (longest_first plans whose every sequence is
                            one tile): work-group b takes rank
                            8 (b / 8 / Hkv) + b % 8 and kv-head b / 8 % Hkv,
                            so the kv-heads of a unit run together on one
                            XCD (b % 8)                                       */
  int64_t partial_rows;  /* (token, q-head) rows of split partial outputs the
                            workspace holds (0: no split).  Fixed parts:
                            num_splits copies of the batch's rows.  Even
                            split: slots of tile_tokens tokens, one per
                            (sequence, chunk it touches)                     */
} pa_plan_info;

/*
 * pa_unified_attention — the whole varlen batch in one call.
 *
 *  q            bf16 [T, Hq, d]; stride[2] == 1; stride[0], stride[1] multiples
 *               of 8; 16-byte aligned.  T = total query tokens.
 *  k_cache      bf16 or fp8 E4M3 [NB, B, Hkv, d]; stride[1..3] contiguous
 *               (B*Hkv*d is not required for stride[0], which must be a
 *               multiple of 16 bytes and at least B*Hkv*d); 16-byte aligned.
 *               With fp8 caches, scores use k_scale * decode(code) and outputs
 *               v_scale * decode(code); this entry point uses scales of 1
 *               (pa_unified_attention_ex takes them in pa_options).
 *  v_cache      same dtype, shape and strides as k_cache.
 *  out          bf16 [T, Hq, d]; same rules as q; fully overwritten; must not
 *               overlap q, k_cache or v_cache.
 *  cu_seqlens_q int32 [S+1], contiguous: query offsets of the S sequences.
 *  seqused_k    int32 [S], contiguous: context length L_s of each sequence.
 *  block_table  int32 [S, MB]; stride[1] == 1; entries j < ceil(L_s / B) of
 *               row s are physical block ids in [0, NB).  Ids may repeat within
 *               and across rows (shared prefixes); entries past ceil(L_s/B)
 *               are never read.
 *  max_seqlen_q upper bound on q_s (used only for launch sizing).
 *  max_seqlen_k upper bound on L_s; must not exceed MB * B.
 *  softmax_scale multiplies q . k before the softmax.
 *  causal       0: every key of the context is admissible; else end-aligned
 *               causal mask (see above).
 *  stream       hipStream_t to launch on (NULL = the null stream).
 *
 * Supported: d in {64, 96, 128, 256}; B in {16, 32, 64}; Hq % Hkv == 0 with G = Hq/Hkv in
 * {1, 2, 4, 8, 16}.  Unsupported values return PA_ERR_UNSUPPORTED.
 *
 * Preconditions on device contents (unchecked unless check_contents is set;
 * breaking them is undefined behaviour): cu_seqlens_q[0] == 0, non-decreasing,
 * cu_seqlens_q[S] == T; q_s <= max_seqlen_q; 0 <= L_s <= max_seqlen_k; block
 * ids in range.  The kernels read every context length as
 * min(max(seqused_k[s], 0), max_seqlen_k), so an overstated seqused_k gives
 * wrong values for that sequence but never reads the block table past
 * max_seqlen_k / B entries or writes past the workspace.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer after
 * return.  This entry point uses a library-owned split workspace (device
 * memory, one per (device, stream), grown on demand with hipMalloc after
 * synchronising the device, kept until process exit); use
 * pa_unified_attention_ex with a caller workspace under stream capture.
 *
 * Asynchronous: returns after enqueueing on `stream`.  Deterministic: the
 * same inputs and launch plan give bit-identical output, and the output does
 * not depend on the physical placement of blocks.  Thread-safe.
 */
int pa_unified_attention(const pa_tensor* q, const pa_tensor* k_cache,
                         const pa_tensor* v_cache, pa_tensor* out,
                         const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                         const pa_tensor* block_table, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                         void* stream);

/*
 * pa_unified_attention_ex — as above with options and a caller workspace.
 * workspace may be NULL iff pa_workspace_bytes(...) returns 0 for the same
 * arguments and options; it must be 256-byte aligned, device memory, at least
 * that many bytes, and not used by anything else until the work enqueued here
 * has finished.  opt may be NULL (defaults).
 */
int pa_unified_attention_ex(const pa_tensor* q, const pa_tensor* k_cache,
                            const pa_tensor* v_cache, pa_tensor* out,
                            const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                            const pa_tensor* block_table, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                            const pa_options* opt, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind pa_unified_attention_noalloc
 * (one copy per GPU, held until the process ends). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pa_unified_attention_noalloc — pa_unified_attention_ex without any device
 * allocation, for callers that cannot allocate: code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The split workspace
 * (partial outputs, per-row part counts, the longest-first unit order) lives in
 * a static device array of PA_NOALLOC_SCRATCH_BYTES per GPU instead of a
 * caller or library buffer; the launches, kernels and results are those of
 * pa_unified_attention_ex with the same options.
 *
 *  Arguments as for pa_unified_attention_ex (opt may be NULL); there is no
 *  workspace argument.
 *  Errors: a batch whose plan needs more workspace than
 *  PA_NOALLOC_SCRATCH_BYTES (pa_workspace_bytes tells) returns
 *  PA_ERR_WORKSPACE and launches nothing; opt->check_contents (which copies
 *  to the host and synchronises) returns PA_ERR_UNSUPPORTED.
 *  Calls no hipMalloc / hipFree.  The first call on a device looks up that
 *  device's copy of the array.
 *  Concurrency: every call on one GPU uses the same array, which keeps the last
 *  call's contents; calls whose work overlaps on one GPU (other streams or
 *  threads) race and must be ordered by the caller.
 */
int pa_unified_attention_noalloc(const pa_tensor* q, const pa_tensor* k_cache,
                                 const pa_tensor* v_cache, pa_tensor* out,
                                 const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                                 const pa_tensor* block_table, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                                 const pa_options* opt, void* stream);

/*
 * pa_unified_attention_lse — as pa_unified_attention_ex, and also writes each
 * row's log-sum-exp: lse[t, h] = ln sum_j exp(softmax_scale * k_scale * q . k_j)
 * over the row's admissible keys (-inf for a row with none).  With the outputs
 * of two calls over disjoint key sets of the same queries, pa_merge_attention
 * gives the result over their union (the log-sum-exp export that cascade /
 * shared-prefix attention composes, page "[Kernel] Unified Triton kernel that
 * doesn't distinguish between prefill + decode", review discussion of the
 * non-causal mode for cascade attention).
 *  lse          fp32 [T, Hq]; stride[1] == 1; 4-byte aligned; must not overlap
 *               q, out or the caches.  Fully overwritten.
 *  workspace    as for pa_unified_attention_ex, except that NULL selects the
 *               library workspace.
 */
int pa_unified_attention_lse(const pa_tensor* q, const pa_tensor* k_cache,
                             const pa_tensor* v_cache, pa_tensor* out, pa_tensor* lse,
                             const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                             const pa_tensor* block_table, int32_t max_seqlen_q,
                             int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                             const pa_options* opt, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * pa_merge_attention — combine two attention results of the same rows over
 * disjoint key sets: with natural-log lse a, b, out = (e^a out_a + e^b out_b) /
 * (e^a + e^b) and lse_out = ln(e^a + e^b); a side with lse = -inf has no keys
 * and drops out (a row with no keys on either side gives 0 and -inf).
 *  out_a, out_b, out  bf16, or all three fp16, [T, Hq, d], d in {64, 96, 128,
 *               256}; stride[2] == 1;
 *               stride[0], stride[1] multiples of 4; 8-byte aligned.
 *  lse_a, lse_b fp32 [T, Hq]; stride[1] == 1.
 *  lse_out      fp32 [T, Hq] or NULL.  Outputs must not overlap the inputs.
 */
int pa_merge_attention(const pa_tensor* out_a, const pa_tensor* lse_a, const pa_tensor* out_b,
                       const pa_tensor* lse_b, pa_tensor* out, pa_tensor* lse_out, void* stream);

/*
 * pa_workspace_bytes — bytes of workspace pa_unified_attention_ex needs for
 * these arguments and options (0 when the batch needs no key split).  Host
 * only: reads descriptors, never device memory.  Returns (size_t)-1 and sets
 * pa_last_error when the arguments are invalid.
 */
size_t pa_workspace_bytes(const pa_tensor* q, const pa_tensor* k_cache,
                          const pa_tensor* v_cache, const pa_tensor* out,
                          const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                          const pa_tensor* block_table, int32_t max_seqlen_q,
                          int32_t max_seqlen_k, const pa_options* opt);

/* pa_workspace_size — the same function under its earlier name. */
size_t pa_workspace_size(const pa_tensor* q, const pa_tensor* k_cache,
                         const pa_tensor* v_cache, const pa_tensor* out,
                         const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                         const pa_tensor* block_table, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, const pa_options* opt);

/*
 * pa_plan_describe — the launch plan the library would use, without
 * launching (host only).  num_cus: compute units to plan for (0 = the
 * current device's count, or 256 when no device is visible).
 */
int pa_plan_describe(const pa_tensor* q, const pa_tensor* k_cache,
                     const pa_tensor* v_cache, const pa_tensor* out,
                     const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                     const pa_tensor* block_table, int32_t max_seqlen_q,
                     int32_t max_seqlen_k, const pa_options* opt, int32_t num_cus,
                     pa_plan_info* info);

/*
 * pa_cache_write — write new tokens' keys and values into the paged caches,
 * the step before attention reads them (same cache layout as above).
 *
 *  key, value   bf16 [N, Hkv, d]; stride[2] == 1; stride[0], stride[1]
 *               multiples of 8; 16-byte aligned.
 *  k_cache      bf16 or fp8 E4M3 [NB, B, Hkv, d], B in {16, 32, 64}, as for
 *               pa_unified_attention;
 *  v_cache      same dtype, shape and strides.  Written in place.
 *  slot_mapping int32 [N], contiguous: token i goes to slot slot_mapping[i] =
 *               physical block * B + position in the block; a negative slot,
 *               or one at or past NB * B (outside the cache), skips the token
 *               (checked on the device).  Slots should be distinct (unchecked;
 *               a repeated slot receives one of its tokens).
 *  k_scale, v_scale  fp8 caches: the stored code is x / scale (IEEE fp32
 *               division) rounded to the nearest E4M3 value, ties to even,
 *               saturated at +-448 (the format has no infinity), NaN kept;
 *               0 reads as 1.  Ignored for bf16 caches (values copied).
 *  stream       hipStream_t (NULL = the null stream).
 *
 * Errors as for pa_unified_attention (validation on the host, nothing
 * launched on failure).  Requires NB * 16 < 2^31.  Asynchronous; the caches
 * must not be read by other work until the write has completed on `stream`.
 */
int pa_cache_write(const pa_tensor* key, const pa_tensor* value, pa_tensor* k_cache,
                   pa_tensor* v_cache, const pa_tensor* slot_mapping, float k_scale,
                   float v_scale, void* stream);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Detail text of the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/* PA_VERSION of the built library. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
