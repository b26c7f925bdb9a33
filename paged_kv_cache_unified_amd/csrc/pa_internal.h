// Internal interface between the host library (pa_api.cpp) and the gfx950
// kernels (pa_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;    // keys of a sub-block, the unit the kernels address (cache blocks
                                  // of 32 or 64 keys are read as 2 or 4 sub-blocks)
constexpr int kStageKeys = 64;    // keys staged in LDS per pipeline step
constexpr int kThreads = 256;     // 4 wave64s per work-group
constexpr int kTileRows = 128;    // packed rows of a wide query tile (32 per wave)
constexpr int kTileRows8 = 256;   // packed rows of an eight-wave wide tile (32 per wave)
constexpr int kNarrowRows = 16;   // rows of a narrow (decode) tile
constexpr int kMaxSplitKeys = 4096;  // keys per split: at most 64 blocks per wave (narrow)
constexpr int kMaxDecodeSeqs = 2048; // sequences the persistent decode kernel can enumerate
constexpr int kEvenMinBlocks = 16;   // even split: smallest chunk (cache blocks per wave)
constexpr int kEvenMinContext = 1024; // decode batches with shorter rows keep one part per row
constexpr int kEvenMaxParts = 256;   // even split: chunks grow so a row has at most ~this many parts
constexpr int kDecodeRing = 2;        // cache blocks in flight per wave (persistent decode; 3 measured no faster)
constexpr int kLptMaxSeqs = 2048;   // longest-first order: LDS tables of 3 ints per sequence
constexpr int kCompactRow = 1 << 30; // row part count flag: the parts sit in compact slots (ws_rbase)

// Everything the forward kernel needs, by value.  Strides in elements.
struct FwdParams {
  const uint16_t* q;       // bf16 or fp16 [T, Hq, d]
  uint16_t* out;           // q's type [T, Hq, d]
  const unsigned char* k;  // [NB, B, Hkv, d] cache elements: q's type, or fp8 E4M3 codes
  const unsigned char* v;
  const int32_t* cu_q;     // [S+1]
  const int32_t* seq_k;    // [S]
  const int32_t* bt;       // [S, bt_stride]
  float* ws_o;             // fp32 [n_split, T, Hq, d]   (n_split > 1 only)
  float* ws_lse;           // fp32 [n_split, T, Hq]      log2-domain lse
  int64_t q_st, q_sh;      // q strides (token, head)
  int64_t o_st, o_sh;      // out strides
  int64_t kv_sb;           // cache stride between physical blocks
  int64_t sub_sb;          // cache stride between 16-key sub-blocks of a block (16 * Hkv * d)
  int32_t bshift;          // block size = 16 << bshift (16, 32 or 64 keys)
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t total_q;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_k;           // max_seqlen_k: every context length is read as min(seq_k[s], max_k)
                           // (the plan sizes splits and the workspace from it)
  int32_t tile_tokens;     // tokens per query tile
  int32_t num_slots;       // query-tile slots
  int32_t slots_direct;    // 1: slot index is the sequence index
  int32_t n_split;
  int32_t split_keys;      // multiple of kStageKeys
  int32_t balanced;        // persistent decode, even split: the batch's (sequence, kv-head,
                           // block) stream is cut into equal chunks of at least
                           // split_keys / 16 blocks, one or more per wave
  int32_t* ws_rparts;      // n_split > 1: parts of each row (token, q-head) [T * Hq],
                           // written by the row's first part (| kCompactRow: see ws_rbase)
  int32_t* ws_rbase;       // even split: partial row of each row's part 0 [T * Hq]; part sg
                           // is at + sg * dq_tokens * Hq (slots of dq_tokens tokens)
  int32_t dq_tokens;       // even split: query tokens per partial slot (max_seqlen_q)
  int32_t num_items;       // num_slots * num_kv_heads * n_split
  int32_t items_per_xcd;   // ceil(num_items / 8): contiguous item range per XCD
  int32_t kv_major;        // item order: 1 = (kv-head, slot, split), 0 = (slot, kv-head, split)
  int32_t causal;
  int32_t narrow_rows;     // tiles with at most this many packed rows take the narrow path
  int32_t lpt;             // grid plans: units in longest-first order (block b -> rank b / Hkv)
  int32_t unit_xcd;        // lpt: the kv-heads of a unit run together on one XCD
                           // (block b -> rank 8 (b / 8 / Hkv) + b % 8, kv-head b / 8 % Hkv)
  int32_t lpt_units;       // entries of lpt_order (the grid's unit capacity)
  int4* lpt_order;         // [lpt_units] (s, tile, split, -) of each rank, from pa_rank_kernel
  float scale_log2;        // softmax_scale * k_scale * log2(e)
  float out_scale;         // v_scale (1 for 16-bit caches): multiplies every output row
  float* lse_out;          // optional fp32 [T, Hq] (row stride lse_st): natural-log lse
  int64_t lse_st;
};

struct MergeParams {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* row_parts;  // [T * Hq]: parts of each row; rows with one part were
                             // written by the forward kernel and are skipped
  const int32_t* row_base;   // [T * Hq]: part-0 partial row of rows flagged kCompactRow
  int64_t part_stride_c;     // partial rows between consecutive parts of such a row
  uint16_t* out;
  int64_t o_st, o_sh;
  int32_t total_q;
  int32_t num_q_heads;
  int32_t n_split;           // upper bound on parts per row
  int32_t even;              // the bound is loose (even decode split): most rows have 1-2
  float* lse_out;            // optional: merged natural-log lse [T, Hq] (row stride lse_st)
  int64_t lse_st;
};

// Two partial results over disjoint key sets -> one (cascade composition).
struct Merge2Params {
  const uint16_t* oa;      // bf16 or fp16 [T, Hq, d]
  const uint16_t* ob;
  const float* la;         // fp32 [T, Hq], natural-log lse (-inf: no key)
  const float* lb;
  uint16_t* out;           // oa's type [T, Hq, d]
  float* lse;              // optional fp32 [T, Hq]
  int64_t oa_st, oa_sh, ob_st, ob_sh, o_st, o_sh, la_st, lb_st, l_st;
  int32_t total_q, num_q_heads;
};

// New tokens' keys and values -> paged cache slots (pa_cache_kernels.hip).
struct CacheWriteParams {
  const uint16_t* key;      // bf16 or fp16 [N, Hkv, d]
  const uint16_t* value;
  unsigned char* k_cache;   // [NB, B, Hkv, d] of the key's 16-bit type, or fp8 E4M3 codes
  unsigned char* v_cache;
  const int32_t* slot_mapping;   // [N]; < 0: skip
  int64_t k_st, k_sh, v_st, v_sh;   // source strides (elements)
  int64_t cache_sb;         // cache stride between physical blocks (elements)
  int32_t block_size;       // slots per block (16, 32 or 64)
  int32_t num_slots;        // NB * block_size: slots at or past it are skipped like negative ones
  int32_t num_tokens;
  int32_t slot_elems;       // Hkv * d
  int32_t chunks_per_token; // Hkv * d / 8
  int32_t chunks_per_head;  // d / 8
  float k_scale, v_scale;   // fp8: codes of x / scale
};

hipError_t launch_cache_write(const CacheWriteParams& p, bool kv8, bool f16, hipStream_t stream);

// Device address of the static scratch (PA_NOALLOC_SCRATCH_BYTES) on the
// current device; looked up once per device (pa_noalloc.hip).
hipError_t noalloc_scratch(void** out);

// Launchers (pa_kernels.hip, one object per head size d).  Return the
// hipError_t of the launch.
// wide = 0 launches the narrow-only specialization (every tile <= 16 rows), 1
// the wide one, 2 the wide one with streaming K/V loads (no tile's K/V is read
// by another tile: every sequence one tile; 16-bit caches, else as 1).
// kv8: the caches hold fp8 E4M3 codes (else 16-bit elements); f16: q, out and
// 16-bit caches are fp16 (else bf16).
#define PA_DECLARE_HEAD_DIM(DV)                                                                  \
  hipError_t launch_fwd_d##DV(const FwdParams& p, int group, int wide, bool kv8, bool f16,      \
                              int64_t num_workgroups, hipStream_t stream);                     \
  hipError_t launch_decode_d##DV(const FwdParams& p, int group, bool kv8, bool f16,             \
                                 int64_t num_workgroups, hipStream_t stream);                  \
  hipError_t launch_fwd8_d##DV(const FwdParams& p, int group, bool f16, int64_t num_workgroups, \
                               hipStream_t stream);                                            \
  int decode_blocks_per_cu_d##DV(int group, bool kv8, bool f16);                                \
  hipError_t launch_merge_d##DV(const MergeParams& p, bool f16, hipStream_t stream);            \
  hipError_t launch_merge2_d##DV(const Merge2Params& p, bool f16, hipStream_t stream);
PA_DECLARE_HEAD_DIM(64)
PA_DECLARE_HEAD_DIM(96)
PA_DECLARE_HEAD_DIM(128)
PA_DECLARE_HEAD_DIM(256)
#undef PA_DECLARE_HEAD_DIM

#define PA_BY_HEAD_DIM(D_, FN, ...)                     \
  switch (D_) {                                         \
    case 64: return FN##_d64(__VA_ARGS__);              \
    case 96: return FN##_d96(__VA_ARGS__);              \
    case 128: return FN##_d128(__VA_ARGS__);            \
    case 256: return FN##_d256(__VA_ARGS__);            \
    default: break;                                     \
  }

inline hipError_t launch_fwd(const FwdParams& p, int head_dim, int group, int wide, bool kv8,
                             bool f16, int64_t num_workgroups, hipStream_t stream) {
  PA_BY_HEAD_DIM(head_dim, launch_fwd, p, group, wide, kv8, f16, num_workgroups, stream)
  return hipErrorInvalidValue;
}
// Eight-wave grid kernel (wide tiles of 256 rows; d = 64 and 128, 16-bit caches).
inline hipError_t launch_fwd8(const FwdParams& p, int head_dim, int group, bool f16,
                              int64_t num_workgroups, hipStream_t stream) {
  PA_BY_HEAD_DIM(head_dim, launch_fwd8, p, group, f16, num_workgroups, stream)
  return hipErrorInvalidValue;
}
inline hipError_t launch_merge(const MergeParams& p, int head_dim, bool f16, hipStream_t stream) {
  PA_BY_HEAD_DIM(head_dim, launch_merge, p, f16, stream)
  return hipErrorInvalidValue;
}
// f16: the outputs are fp16 (else bf16)
inline hipError_t launch_merge2(const Merge2Params& p, int head_dim, bool f16, hipStream_t stream) {
  PA_BY_HEAD_DIM(head_dim, launch_merge2, p, f16, stream)
  return hipErrorInvalidValue;
}
// Longest-first unit order of a grid plan into p.lpt_order (one work-group).
hipError_t launch_rank(const FwdParams& p, hipStream_t stream);
// Persistent decode kernel (every tile narrow, num_seqs <= kMaxDecodeSeqs).
inline hipError_t launch_decode(const FwdParams& p, int head_dim, int group, bool kv8, bool f16,
                                int64_t num_workgroups, hipStream_t stream) {
  PA_BY_HEAD_DIM(head_dim, launch_decode, p, group, kv8, f16, num_workgroups, stream)
  return hipErrorInvalidValue;
}
// Resident work-groups per CU of the decode kernel (0 if unknown).
inline int decode_blocks_per_cu(int head_dim, int group, bool kv8, bool f16) {
  PA_BY_HEAD_DIM(head_dim, decode_blocks_per_cu, group, kv8, f16)
  return 0;
}
inline bool fwd_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 96 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}
#undef PA_BY_HEAD_DIM

}  // namespace pa
