// gfx950 (CDNA4) kernels of libpa: the unified paged-attention forward kernel
// and the log-sum-exp merge of key-split partial results.
//
// Operation: softmax(scale * q k^T + mask) v for a varlen batch whose sequences
// have arbitrary query lengths (decode, chunked prefill, prefill in one grid),
// keys and values read from a paged cache [num_blocks, B, Hkv, d] (B = 16, 32
// or 64, read as 16-key sub-blocks) through a block table (page "[Kernel] Unified Triton kernel that doesn't distinguish
// between prefill + decode", PR description; the causal mask is end-aligned so
// decode queries and prefill chunks share one kernel, page "[Kernel] [V1]
// Improved performance for V1 Triton (ROCm) backend", section "How is this
// performance improvement achieved?").
//
// Kernels.
//  * pa_fwd_kernel: the unified grid kernel.  One work-group (4 wave64s) owns
//    one unit (sequence, query tile, key split) for one kv-head; decode rows,
//    chunks and prefills share the launch.  The q-heads of one kv-head (the
//    GQA group, G of them) are packed with the tile's tokens into the rows of
//    the MFMA tiles (row r <-> token r / G, head r % G), so one K/V read
//    serves G heads (the packing of a kv-head's query heads into the query
//    dimension that the unified-kernel page adopts).  Tiles of at most 16
//    packed rows take the narrow path (four waves split the keys), larger ones
//    the wide path (each wave owns 32 rows, 32x32x16 MFMA; every head size).
//    Wide plans run their units longest-first, in the order pa_rank_kernel
//    sorts them into.
//  * pa_decode_kernel: persistent decode for batches whose every sequence is
//    one narrow tile; each wave streams items of fixed-size key parts, or of
//    the even split of the batch's block stream.
//  * pa_merge_*: log-sum-exp merge of key-split partial results.
//
// Element types: bf16 or fp16 q / out / caches, or fp8 E4M3 caches; head
// sizes 64, 96, 128 and 256.
//
// Scores are computed transposed, S^T = K Q^T, so each lane holds one packed
// row's scores and softmax row reductions stay within a lane plus cross-lane
// steps; P^T (16-bit) feeds O^T += V^T P^T straight from the score accumulators,
// with V^T operands from the gfx950 LDS transpose read (ds_read_b64_tr_b16) of
// row-major V.  Softmax runs online in fp32 in the log2 domain.
//
// Key splits: a sequence of L keys has ceil(L / split) parts (or the parts of
// the even split in the persistent decode kernel); a part writes its
// normalised fp32 output and log2-domain lse to the workspace and pa_merge
// combines them.  Split boundaries depend on lengths only, so results are
// deterministic.
//
// Address math for the cache is 64-bit (physical block * block stride), since
// one cache tensor can exceed 2^31 elements (the int64 cast discussed in the
// review of page "[ROCM][KERNEL] Paged attention for V1").

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PA_LDS __attribute__((address_space(3)))

// The 16-bit element type of q, out and unquantised caches: bf16 (F16 =
// false) or IEEE fp16 (F16 = true).  Operands travel as raw 16-bit lanes (u32x4
// = 8 elements, u32x2 = 4) and meet their type only in these wrappers: the
// MFMAs of that type, round-to-nearest-even packing of fp32 pairs, and the
// exact fp8 E4M3 -> element conversion (every E4M3 value is exact in both).
template <bool F16>
struct Elem;
template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // v_cvt_scalef32_pk_bf16_fp8 with scale 1: codes (byte 2*SEL, 2*SEL+1) of w
  template <bool SEL>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL));
  }
  // the element in the low 16 bits of u, as fp32 (exact)
  static __device__ __forceinline__ float unpack(uint32_t u) {
    return __builtin_bit_cast(float, u << 16);
  }
};
template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  template <bool SEL>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL));
  }
  static __device__ __forceinline__ float unpack(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
  }
};

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform value as a scalar (lets the compiler keep branches scalar).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void* uniform_ptr(const void* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}
// Cache policy of K/V loads that nothing else in the call reads again: the
// non-temporal (nt) bit of the cache-policy operand, which marks the data as
// streaming.  Used by the persistent decode kernel and by the wide tiles of
// plans whose sequences are one tile each.  Measured on this GPU against
// ordinary loads: the 256 x 1k-key decode batch 178 against 199 us, the 16 x
// 32k-128k decode batch 796 against 886 us.  K/V that other query tiles of a
// sequence read again keep ordinary loads, and so does the grid's narrow path
// (streaming made the narrow-only grids slower).
constexpr int kStreamLoad = 2;

// 16-byte global -> LDS DMA: lane i's 16 bytes (at voffset of the buffer
// resource) land at LDS byte address lds + 16 i.  Callers wait with
// wait_dma() before the barrier that publishes the data.  AUX: cache policy.
template <int AUX = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (PA_LDS void*)(uintptr_t)lds, 16, voff, 0, 0, AUX);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Work-group barrier that orders LDS accesses only (this wave's LDS reads and
// writes have completed; outstanding global loads, LDS DMA included, keep
// running, unlike __syncthreads, whose fence waits for every memory access)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// x *= s in place (tied operands keep a conditionally rescaled accumulator in
// its own registers instead of a copy per branch)
__device__ __forceinline__ void scale_inplace(float& x, float s) {
  asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(s));
}

// Cache element formats: the 16-bit element type, or fp8 E4M3 codes (OCP
// 8-bit float, the "fn" variant: no infinities, S.1111.111 is NaN) converted
// to the element type right after the load.  Every E4M3 value is exact in
// bf16 and fp16, so the MFMA paths see the operands a 16-bit cache of the
// decoded codes would give; the per-tensor scales are folded into the
// softmax scale (K) and the output (V).
template <bool KV8>
struct Kv {
  static constexpr int ESZ = KV8 ? 1 : 2;                                 // bytes per element
  using raw8 = typename std::conditional<KV8, u32x2, u32x4>::type;        // 8 elements as loaded
};
// 8 loaded cache elements as 8 elements of the 16-bit type
template <bool F16>
__device__ __forceinline__ u32x4 to_elem8(u32x4 v) { return v; }
template <bool F16>
__device__ __forceinline__ u32x4 to_elem8(u32x2 v) {
  using E = Elem<F16>;
  return u32x4{E::template fp8x2<false>(v[0]), E::template fp8x2<true>(v[0]),
               E::template fp8x2<false>(v[1]), E::template fp8x2<true>(v[1])};
}
// 8 consecutive cache elements at a byte address / a buffer byte offset
template <bool KV8>
__device__ __forceinline__ typename Kv<KV8>::raw8 gload8(const unsigned char* ptr) {
  return *reinterpret_cast<const typename Kv<KV8>::raw8*>(ptr);
}
template <bool KV8, int AUX = 0>     // AUX: cache policy
__device__ __forceinline__ typename Kv<KV8>::raw8 bload8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  if constexpr (KV8)
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, AUX));
  else
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX);
}

// Natural-log lse of a row from its log2-domain value (kept in the library's
// kernels: scores in log2 units of softmax_scale * k_scale * q.k).
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ void store_lse(float* lse_out, int64_t lse_st, int64_t tok, int head,
                                          float lse2) {
  if (lse_out) lse_out[tok * lse_st + head] = lse2 == -__builtin_huge_valf() ? lse2 : lse2 * kLn2;
}

// Cache blocks of B = 16 * 2^bshift keys are read as 2^bshift sub-blocks of 16
// keys.  Sub-block j of a sequence is part j % 2^bshift of block-table entry
// j >> bshift; its id packs (physical block, part) into one int.
__device__ __forceinline__ int sub_block_id(const int32_t* row, int j, int bshift) {
  return (row[j >> bshift] << bshift) | (j & ((1 << bshift) - 1));
}
// element offset of a sub-block in the cache
__device__ __forceinline__ int64_t sub_block_base(const FwdParams& p, int id) {
  return (int64_t)(id >> p.bshift) * p.kv_sb + (int64_t)(id & ((1 << p.bshift) - 1)) * p.sub_sb;
}

// Context length of sequence s, clamped to [0, max_seqlen_k]: the plan sized
// the key splits, the workspace and the block-table reads from max_seqlen_k, so
// a larger seqused_k (a broken precondition) cannot take a kernel past them.
__device__ __forceinline__ int context_len(const FwdParams& p, int s) {
  return min(max(p.seq_k[s], 0), p.max_k);
}

__device__ __forceinline__ float max_across_groups(float x) {
  // lanes l, l^16, l^32, l^48 hold the same packed row
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float sum_across_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Online softmax of one 16-key block on the 16-column tiles (narrow path and
// decode kernel).  x holds this lane's 4 scores of the block in log2 units
// (masked keys at -inf); m, l and acc are its row's running state, shared by
// the 4 lanes of the row.  The reference max m moves, and O and l are
// rescaled, only when a score of the wave exceeds its row's reference by more
// than 2^8 (or a row sees its first key).  O and l share the reference, so
// this is exact, and every weight stays at most 256.  The common path has no
// cross-lane step and no rescale: the test is one ballot of the lanes' own
// scores, and only the rare move takes the row max over the lane groups.
template <int DT>
__device__ __forceinline__ void block_weights(const float (&x)[4], float& m, float& l,
                                              f32x4 (&acc)[DT], float (&pr)[4]) {
  constexpr float kThr = 8.f;
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__builtin_amdgcn_ballot_w64(mx > m + kThr)) {        // wave-uniform
    const float m_new = fmaxf(m, max_across_groups(mx));
    const float alpha = m_new == m ? 1.f : exp2_fast(m - m_new);   // m = -inf: 0
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  }
  const float m_use = m == kNegInf ? 0.f : m;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = exp2_fast(x[r] - m_use);
    rs += pr[r];
  }
  l += rs;
}

// LDS layouts of one (block, kv-head) tile of 16 keys x D, in 16-byte chunks.
//  K: chunk (key, dc) at index dc*16 + (key ^ dc): an A-operand read (16 keys
//     at one d-chunk per lane group) is 256 contiguous bytes, and the
//     row-contiguous store of a key row touches 16 distinct bank groups.
//  V: chunk (key, c) at index key*CPR + (c ^ f(key)); f keeps the two chunks a
//     transpose read takes from each row adjacent while spreading the rows of
//     one read over distinct bank windows.
template <int D>
struct Layout {
  static constexpr int CPR = D / 8;                  // chunks per key row
  static constexpr int BLK_BYTES = kBlockSize * D * 2;
  // XOR swizzle of a V row's chunks; d = 96 (12 chunks, not closed under
  // XOR) keeps the plain order
  static __device__ __forceinline__ int v_swz(int key) {
    if constexpr (D == 96) return 0;
    return D >= 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
  }
  static __device__ __forceinline__ int v_chunk(int key, int c) { return key * CPR + (c ^ v_swz(key)); }
};

// One work item: (query tile, kv-head, key split) and the key range it covers.
struct Item {
  int s, kvh, sigma;
  int parts;          // key splits of this sequence (1: rows are written to out)
  int q0, q_len, tok0, n_tok, rows;
  int L, diag;        // context length; causal: token t sees keys < diag + t + 1
  int kbeg, kend;     // keys [kbeg, kend) of this split that some row may need
  int kmin;           // smallest per-row key limit within the tile
};

// Fills the item for (sequence s, query tile, split sigma, kv-head); false if
// the tile or split does not exist for this sequence.
template <int G>
__device__ __forceinline__ bool fill_item(const FwdParams& p, int s, int tile, int sigma, int kvh,
                                          Item& it) {
  it.s = s;
  it.kvh = kvh;
  it.sigma = sigma;
  it.q0 = p.cu_q[s];
  it.q_len = p.cu_q[s + 1] - it.q0;
  it.tok0 = tile * p.tile_tokens;
  if (it.tok0 >= it.q_len) return false;            // empty slot (whole work-group)
  it.n_tok = min(p.tile_tokens, it.q_len - it.tok0);
  it.rows = it.n_tok * G;
  it.L = context_len(p, s);
  // a sequence has ceil(L / split) parts (at least one): items past them idle
  it.parts = min(max((it.L + p.split_keys - 1) / p.split_keys, 1), p.n_split);
  if (it.sigma >= it.parts) return false;
  it.diag = it.L - it.q_len;
  const int k_need = p.causal ? min(it.L, it.diag + it.tok0 + it.n_tok) : it.L;
  it.kbeg = it.sigma * p.split_keys;
  it.kend = min(k_need, it.kbeg + p.split_keys);
  it.kmin = p.causal ? min(it.kend, it.diag + it.tok0 + 1) : it.kend;
  return true;
}

// Inclusive prefix sum over the 64 lanes of a wave in six DPP moves: row
// shifts by 1, 2, 4 and 8 lanes (zero from outside the 16-lane row) scan each
// row, then lane 15 is broadcast into row 1 and 3 and lane 31 into rows 2 and
// 3.  All vector ALU work, no LDS round trip per step.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over the work-group (256 threads); *total receives the
// sum.  scratch: 8 ints of LDS.  Contains barriers: call from every thread.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();                                   // scratch may be reused
  *total = all;
  return before + x - v;
}

// Stages (64 keys) of unit (s, tile, sigma), from the per-sequence lengths.
__device__ __forceinline__ int unit_stages(const FwdParams& p, int q_len, int L, int tile,
                                           int sigma) {
  const int tok0 = tile * p.tile_tokens;
  const int n_tok = min(p.tile_tokens, q_len - tok0);
  const int k_need = p.causal ? min(L, L - q_len + tok0 + n_tok) : L;
  const int kbeg = sigma * p.split_keys;
  const int kend = min(k_need, kbeg + p.split_keys);
  return kend > kbeg ? (kend - kbeg + kStageKeys - 1) / kStageKeys : 0;
}

// Longest-first order of the batch's units (sequence, query tile, key split),
// so the work-group scheduler starts the most expensive tiles first and the
// grid drains with short ones (list scheduling, longest processing time
// first).  One work-group computes the order once per call from the lengths
// and writes order[r] = (s, tile, split) for rank r, ranks running over the
// 64-key stage counts descending; ranks past the last unit get s = -1.
// Sequence s owns unit indices [P[s], P[s] + tiles_s * parts_s), index j
// within it being (tile j % tiles_s, split j / tiles_s).  Units of equal stage
// count take their ranks in any order (LDS atomics): the order decides only
// which work-group computes a unit, never its result.
#if PA_TU_HEAD_DIM == 64
__global__ __launch_bounds__(kThreads) void pa_rank_kernel(FwdParams p) {
  extern __shared__ int tab[];     // 3 S + 1 + 65 + 65 + 8 ints
  const int S = p.num_seqs;
  int* qlen = tab;                 // [S]
  int* klen = tab + S;             // [S]
  int* pre = tab + 2 * S;          // [S + 1] first unit index of each sequence
  int* hist = tab + 3 * S + 1;     // [65] units per stage count (0..64)
  int* next = hist + 65;           // [65] next free rank of each stage count
  int* scr = next + 65;            // [8] scan scratch
  const int tid = threadIdx.x;
  const int Tq = p.tile_tokens;
  // per-sequence tables; threads own contiguous runs of sequences
  const int per = (S + kThreads - 1) / kThreads;
  const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
  int mine = 0;
  for (int s = s0; s < s1; ++s) {
    const int q = p.cu_q[s + 1] - p.cu_q[s];
    const int L = context_len(p, s);
    qlen[s] = q;
    klen[s] = L;
    const int parts = min(max((L + p.split_keys - 1) / p.split_keys, 1), p.n_split);
    mine += ((q + Tq - 1) / Tq) * parts;
  }
  if (tid < 65) hist[tid] = 0;
  int U;
  int run = block_exclusive_scan(mine, scr, &U);
  for (int s = s0; s < s1; ++s) {
    pre[s] = run;
    const int q = qlen[s], L = klen[s];
    const int parts = min(max((L + p.split_keys - 1) / p.split_keys, 1), p.n_split);
    run += ((q + Tq - 1) / Tq) * parts;
  }
  if (tid == 0) pre[S] = U;
  __syncthreads();
  // each thread walks a contiguous run of unit indices
  const int cu = (U + kThreads - 1) / kThreads;
  const int u0 = min(U, tid * cu), u1 = min(U, u0 + cu);
  int s_first = 0;
  if (u0 < u1) {
    int lo = 0, hi = S - 1;                          // last s with pre[s] <= u0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= u0) lo = mid; else hi = mid - 1;
    }
    s_first = lo;
  }
  auto walk = [&](auto&& visit) {
    int s = s_first;
    for (int u = u0; u < u1; ++u) {
      while (u >= pre[s + 1]) ++s;                   // skips sequences without units
      const int q = qlen[s];
      const int nt = (q + Tq - 1) / Tq;
      const int j = u - pre[s];
      const int tile = j % nt, sg = j / nt;
      visit(s, tile, sg, unit_stages(p, q, klen[s], tile, sg));
    }
  };
  walk([&](int, int, int, int w) { atomicAdd(&hist[w], 1); });
  __syncthreads();
  {
    // first rank of each stage count: an exclusive scan of the counts taken
    // from the longest (64 stages) down, thread t holding stage count 64 - t
    const int c = tid <= 64 ? hist[64 - tid] : 0;
    int all;
    const int first = block_exclusive_scan(c, scr, &all);
    if (tid <= 64) next[64 - tid] = first;
  }
  __syncthreads();
  walk([&](int s, int tile, int sg, int w) {
    const int r = atomicAdd(&next[w], 1);
    p.lpt_order[r] = int4{s, tile, sg, 0};
  });
  for (int r = U + tid; r < p.lpt_units; r += kThreads) p.lpt_order[r] = int4{-1, 0, 0, 0};
}
#endif

template <int G>
__device__ __forceinline__ bool decode_item(const FwdParams& p, Item& it) {
  if (p.lpt) {
    // block b -> unit rank b / Hkv, kv-head b % Hkv: with 8 kv-heads every
    // XCD (b % 8) serves one kv-head, so K/V of its sequences stay in its L2.
    // Units that share no K/V (every sequence one tile) instead put a unit's
    // kv-heads on consecutive blocks of one XCD: rank 8 (b / 8 / Hkv) + b % 8,
    // kv-head b / 8 % Hkv, so they read each cache block at about one time.
    const int j = (int)blockIdx.x >> 3;
    const int r = p.unit_xcd ? (j / p.num_kv_heads) * 8 + ((int)blockIdx.x & 7)
                             : (int)blockIdx.x / p.num_kv_heads;
    const int kvh = p.unit_xcd ? j % p.num_kv_heads : (int)blockIdx.x % p.num_kv_heads;
    if (r >= p.lpt_units) return false;              // the grid is rounded up to 8 blocks
    const int4 u = p.lpt_order[r];                   // written by pa_rank_kernel
    if (u.x < 0) return false;
    return fill_item<G>(p, u.x, u.y, u.z, kvh, it);
  }
  // Work-groups are dispatched round-robin over the 8 XCDs (XCD = id % 8);
  // give each XCD a contiguous range of items so items that share data
  // (the q-tiles of one kv-head's context, or the kv-heads of one sequence's
  // blocks) run close in time on the same L2.
  const int item = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);
  if (item >= p.num_items) return false;
  const int sigma = item % p.n_split;
  const int rest = item / p.n_split;
  int slot, kvh;
  if (p.kv_major) {
    slot = rest % p.num_slots;
    kvh = rest / p.num_slots;
  } else {
    kvh = rest % p.num_kv_heads;
    slot = rest / p.num_kv_heads;
  }
  int s, tile;
  if (p.slots_direct) {
    s = slot;
    tile = 0;
  } else {
    // sequence s owns slots [cu[s]/Tq + s, cu[s+1]/Tq + s + 1)
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_q[mid] / p.tile_tokens + mid <= slot) lo = mid; else hi = mid - 1;
    }
    s = lo;
    tile = slot - (p.cu_q[lo] / p.tile_tokens + lo);
  }
  return fill_item<G>(p, s, tile, sigma, kvh, it);
}

// Q^T operand (B of S^T = K Q^T) for packed row `row` of the tile: lane group
// h4 holds d = 32 ks + 8 h4 .. +7 for each contraction step ks.
template <int D, int G>
__device__ __forceinline__ void load_q(const FwdParams& p, const Item& it, int row, int h4,
                                       u32x4 (&qB)[D / 32]) {
  const bool ok = row < it.rows;
  const int t_in = row / G;
  const int head = it.kvh * G + row % G;
  const uint16_t* qp = p.q + (int64_t)(it.q0 + it.tok0 + (ok ? t_in : 0)) * p.q_st +
                       (int64_t)head * p.q_sh + 8 * h4;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
    qB[ks] = v;
  }
}

// Shared-memory budgets (NW: waves of the work-group).
template <int D, int NW = 4>
struct NarrowCfg {
  static constexpr int BLK_BYTES = kBlockSize * D * 2;
  static constexpr int VBUF_BYTES = NW * 2 * BLK_BYTES;           // 2 V buffers per wave
  static constexpr int RED_STRIDE = D + 4;                        // floats per merged row
  static constexpr int RED_BYTES = (2 * 16 * NW + NW * 16 * RED_STRIDE) * 4;
  static constexpr int SMEM = VBUF_BYTES > RED_BYTES ? VBUF_BYTES : RED_BYTES;
};

// ---------------------------------------------------------------------------
// Narrow tiles (<= 16 packed rows: decode steps, short chunks).
//
// All 16 columns of one MFMA tile hold the tile's rows in every wave; wave w
// of the NW waves owns the item's cache blocks w, w+NW, ... and streams them on its own,
// with no work-group barrier until the final merge.  Each wave keeps a ring of
// P blocks in flight in registers: K lands directly in the A-operand layout of
// S^T = K Q^T (lane: key l16, d-chunk h4 + 4 ks), V in natural row order and
// goes through a wave-private LDS buffer for the transpose read.  The block
// ids of the wave's (at most 64) blocks are fetched once into one VGPR and
// read per block with readlane, so no KV load waits on a block-table load.
// ---------------------------------------------------------------------------
template <int D, int G, int P, bool KV8, bool F16, int NW = 4>
__device__ __forceinline__ void attend_narrow(const FwdParams& p, const Item& it,
                                              unsigned char* smem) {
  using E = Elem<F16>;
  constexpr int ESZ = Kv<KV8>::ESZ;
  using raw8 = typename Kv<KV8>::raw8;
  using Lay = Layout<D>;
  using Cfg = NarrowCfg<D, NW>;
  constexpr int CPR = Lay::CPR;
  constexpr int BLK_BYTES = Lay::BLK_BYTES;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int VPL = kBlockSize * CPR / 64;      // V chunks per lane per block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int h4 = lane >> 4;
  const int l16 = lane & 15;

  u32x4 qB[KS];
  load_q<D, G>(p, it, l16, h4, qB);
  const int t_in = l16 / G;
  const int klim = p.causal ? min(it.kend, it.diag + it.tok0 + t_in + 1) : it.kend;

  const int blk0 = it.kbeg / kBlockSize;
  const int nblk = it.kend > it.kbeg ? (it.kend + kBlockSize - 1) / kBlockSize - blk0 : 0;
  const int nb = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;   // <= 64: split_keys <= 4096
  const int32_t* btrow = p.bt + (int64_t)it.s * p.bt_stride;
  int ids = 0;
  if (lane < nb) ids = sub_block_id(btrow, blk0 + wave + NW * lane, p.bshift);

  const int slot_stride = p.num_kv_heads * D;
  const unsigned char* kbase = p.k + (int64_t)it.kvh * D * ESZ;
  const unsigned char* vbase = p.v + (int64_t)it.kvh * D * ESZ;
  const int koff = l16 * slot_stride + 8 * h4;
  int voff[VPL], vlds[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const int c = lane + 64 * u;
    const int key = c / CPR, dc = c % CPR;
    voff[u] = key * slot_stride + dc * 8;
    vlds[u] = Lay::v_chunk(key, dc) * 16;
  }

  raw8 kst[P][KS];
  raw8 vst[P][VPL];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    if (j < nb) {
      const int64_t boff = sub_block_base(p, __builtin_amdgcn_readlane(ids, j));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kst[j][ks] = gload8<KV8>(kbase + (boff + koff + 32 * ks) * ESZ);
#pragma unroll
      for (int u = 0; u < VPL; ++u) vst[j][u] = gload8<KV8>(vbase + (boff + voff[u]) * ESZ);
    }
  }

  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;
  unsigned char* vbuf0 = smem + wave * 2 * BLK_BYTES;
  const int tr_key = 4 * h4 + (l16 >> 2);
  const int tr_c_lo = (l16 & 3) >> 1;
  const int tr_half = (l16 & 1) * 8;

  for (int i0 = 0; i0 < nb; i0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = i0 + j;
      if (i < nb) {
        const int kb = (blk0 + wave + NW * i) * kBlockSize;
        unsigned char* vbuf = vbuf0 + (i & 1) * BLK_BYTES;
#pragma unroll
        for (int u = 0; u < VPL; ++u)
          *reinterpret_cast<u32x4*>(vbuf + vlds[u]) = to_elem8<F16>(vst[j][u]);
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc = E::mma16(to_elem8<F16>(kst[j][ks]), qB[ks], sc);
        // refill this ring slot with block i + P
        if (i + P < nb) {
          const int64_t boff = sub_block_base(p, __builtin_amdgcn_readlane(ids, i + P));
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kst[j][ks] = gload8<KV8>(kbase + (boff + koff + 32 * ks) * ESZ);
#pragma unroll
          for (int u = 0; u < VPL; ++u) vst[j][u] = gload8<KV8>(vbase + (boff + voff[u]) * ESZ);
        }
        const bool need_mask = kb + kBlockSize > it.kmin;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = sc[r] * p.scale_log2;
          if (need_mask && kb + 4 * h4 + r >= klim) x[r] = kNegInf;
        }
        float pr[4];
        block_weights<DT>(x, m, l, acc, pr);
        const u32x2 pB = {E::pack2(pr[0], pr[1]), E::pack2(pr[2], pr[3])};
        const bool vmask = kb + kBlockSize > it.kend;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const unsigned char* a =
              vbuf + Lay::v_chunk(tr_key, 2 * dt + tr_c_lo) * 16 + tr_half;
          i16x4 va = __builtin_bit_cast(
              i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PA_LDS bf16x4*)(a)));
          if (vmask) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb + 4 * h4 + e >= it.kend) va[e] = 0;
          }
          acc[dt] = E::mma16k16(__builtin_bit_cast(u32x2, va), pB, acc[dt]);
        }
      }
    }
  }

  // merge the NW waves' states of the same 16 rows
  l = sum_across_groups(l);
  __syncthreads();                        // every wave is done with its V buffers
  float* red_m = reinterpret_cast<float*>(smem);
  float* red_l = red_m + 16 * NW;
  float* red_o = red_m + 32 * NW;         // [wave][row][RED_STRIDE]
  constexpr int RS = Cfg::RED_STRIDE;
  if (h4 == 0) {
    red_m[wave * 16 + l16] = m;
    red_l[wave * 16 + l16] = l;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(red_o + (wave * 16 + l16) * RS + 16 * dt + 4 * h4) = acc[dt];
  __syncthreads();

  constexpr int DPER = D / 16;            // d values per thread (16 threads per row)
  const int n = tid >> 4;
  const int d0 = (tid & 15) * DPER;
  if (n >= it.rows) return;
  float mw[NW], M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = red_m[w * 16 + n];
    M = fmaxf(M, mw[w]);
  }
  const float M_use = M == kNegInf ? 0.f : M;
  float wt[NW], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = exp2_fast(mw[w] - M_use);
    Ls += wt[w] * red_l[w * 16 + n];
  }
  const float inv = Ls > 0.f ? p.out_scale / Ls : 0.f;
  // DPER = 4, 6, 8 or 16 values per thread: pairs (8-byte aligned: d0 is even)
  float o[DPER];
#pragma unroll
  for (int e = 0; e < DPER; e += 2) {
    f32x2 a = {0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w)
      a += wt[w] * *reinterpret_cast<const f32x2*>(red_o + (w * 16 + n) * RS + d0 + e);
    o[e] = a[0] * inv;
    o[e + 1] = a[1] * inv;
  }
  const int64_t tok = it.q0 + it.tok0 + n / G;
  const int hn = it.kvh * G + n % G;
  if (p.ws_rparts && it.sigma == 0 && (tid & 15) == 0)
    p.ws_rparts[tok * p.num_q_heads + hn] = it.parts;     // the row's part count, for pa_merge
  if (it.parts == 1) {
    if ((tid & 15) == 0)
      store_lse(p.lse_out, p.lse_st, tok, hn, Ls > 0.f ? M + __log2f(Ls) : kNegInf);
    uint16_t* op = p.out + tok * p.o_st + (int64_t)hn * p.o_sh + d0;
    if constexpr (DPER % 8 == 0) {               // 16-byte stores
#pragma unroll
      for (int e = 0; e < DPER; e += 8)
        *reinterpret_cast<u32x4*>(op + e) = u32x4{E::pack2(o[e], o[e + 1]), E::pack2(o[e + 2], o[e + 3]),
                                                  E::pack2(o[e + 4], o[e + 5]), E::pack2(o[e + 6], o[e + 7])};
    } else if constexpr (DPER % 4 == 0) {        // 8-byte stores
#pragma unroll
      for (int e = 0; e < DPER; e += 4)
        *reinterpret_cast<u32x2*>(op + e) = u32x2{E::pack2(o[e], o[e + 1]), E::pack2(o[e + 2], o[e + 3])};
    } else {                                     // d = 96: 4-byte stores (d0 = 6 j)
#pragma unroll
      for (int e = 0; e < DPER; e += 2)
        *reinterpret_cast<uint32_t*>(op + e) = E::pack2(o[e], o[e + 1]);
    }
  } else {
    const int64_t r = ((int64_t)it.sigma * p.total_q + tok) * p.num_q_heads + hn;
    float* wp = p.ws_o + r * D + d0;
#pragma unroll
    for (int e = 0; e < DPER; e += 2) *reinterpret_cast<f32x2*>(wp + e) = f32x2{o[e], o[e + 1]};
    if ((tid & 15) == 0) p.ws_lse[r] = Ls > 0.f ? M + __log2f(Ls) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Wide tiles (17..128 packed rows: prefill and longer chunks).
//
// Each wave owns 32 packed rows of the tile and all four waves sweep the same
// 64-key stages, so both contractions run on v_mfma_f32_32x32x16_bf16 (a
// 32-row B operand halves the LDS bytes read per flop compared with 16-row
// tiles).  Lane l holds row l % 32; lanes l and l ^ 32 split that row's keys
// (S^T = K Q^T puts key 8(r/4) + 4(l/32) + r%4 of a 32-key block in
// accumulator r), so a row maximum is a lane-local reduction plus one
// exchange between lanes l and l ^ 32.  P^T feeds O^T += V^T P^T straight from the score
// registers: the contraction index of a 16-key slice is permuted to the
// order the score accumulators hold, and the V^T operand is read in that
// same order with two LDS transpose reads.
//
// Online softmax (fp32, log2 domain).  The running reference max m is kept in
// raw score units and p = exp2(s c - m c) with c = |scale| log2(e) (Q is
// negated on load for a negative scale), one FMA and one exp per score.  The
// reference is moved, and O and l rescaled, only when some row's max exceeds
// it by more than 2^8 (or a row sees its first key): exact in real
// arithmetic, since O and l share the reference, and P <= 256 stays well
// inside bf16 and fp32 range.  Masks (causal diagonal, context end) are applied
// only in the stages that reach them.
//
// K and V of stage st+1 are copied by 16-byte DMA (buffer loads into LDS; a
// block past the context end has zero records, so it reads as zeros without
// touching memory) into the other of two LDS buffers while stage st is
// computed: one barrier per stage, no staging registers.
// ---------------------------------------------------------------------------
// Head size of the wide path's LDS layout: d = 96 uses the d = 128 one.
constexpr int wide_layout_dim(int d) { return d == 96 ? 128 : d; }
// A buffer offset past the records of any cache block (reads as zeros).
constexpr int kPadOffset = 1 << 30;

template <int D>
struct WideCfg {
  static_assert(D == 64 || D == 128 || D == 256, "wide-tile LDS layouts: d = 64, 128, 256");
  static constexpr int CPR = D / 8;                        // 16-byte chunks per key row
  static constexpr int TENSOR_BYTES = kStageKeys * D * 2;  // K (or V) of one stage
  static constexpr int STAGE_BYTES = 2 * TENSOR_BYTES;
  static constexpr int OFFS_OFFSET = 2 * STAGE_BYTES;
  // byte offsets of the unit's sub-blocks, with 4 entries of padding (the
  // loads of the stage past the end read them, and touch no memory)
  static constexpr int OFFS_ENTRIES = kMaxSplitKeys / kBlockSize + 4;
  static constexpr int SMEM_RAW = OFFS_OFFSET + OFFS_ENTRIES * 8;
  static constexpr int SMEM = SMEM_RAW > NarrowCfg<D>::SMEM ? SMEM_RAW : NarrowCfg<D>::SMEM;
  static constexpr int RPI = 64 / CPR;                     // key rows per wave-wide 1 KB load
  static constexpr int CPT = kStageKeys / (4 * RPI);       // loads per thread per tensor
  // LDS chunk of (key row r, chunk c): r * CPR + (c ^ f(r)).  fk spreads the
  // 16 keys one K-operand read takes at a fixed chunk over 16 bank windows;
  // fv does the same for the 4 rows x 4 chunks of each half-wave of a V
  // transpose read.  Both depend on r % 16 only.
  static __device__ __forceinline__ int fk(int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int fv(int r) {
    return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  }
};

// Lanes l and l ^ 32 hold halves of one row.  v_permlane32_swap exchanges
// the upper half-wave of its first operand with the lower half-wave of its
// second: with both holding x, the results are x of lanes 0..31 and x of
// lanes 32..63 in every lane, so one max / add combines a row's halves.
// Written as asm: the compiler's builtin folds the two results into one.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float swap_halves_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

// Transpose read through a restrict pointer.  Inlined, the access carries
// alias metadata, so the compiler orders it against LDS DMA by the explicit
// waits and barriers of the caller (as it does the plain LDS reads) instead
// of waiting for every DMA in flight.
__device__ __forceinline__ i16x4 lds_read_tr(const PA_LDS bf16x4* __restrict__ a) {
  return __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PA_LDS bf16x4*)a));
}

// Epilogue of a 32-row wave on the 32x32 layouts: lanes l and l ^ 32
// together hold row l % 32.  One-part rows go to out (and the lse export),
// rows of split sequences to the workspace as normalised fp32 partials with
// their log2-domain lse.
template <int D, int G, bool F16>
__device__ __forceinline__ void wide_epilogue(const FwdParams& p, const Item& it,
                                              f32x16 (&acc)[D / 32], float m, float l, float c,
                                              bool row_ok, int t_in, int head, int h) {
  using E = Elem<F16>;
  constexpr int DT = D / 32;
  const float lt = swap_halves_sum(l);
  if (!row_ok) return;
  const float inv = lt > 0.f ? p.out_scale / lt : 0.f;
  const int64_t tok = it.q0 + it.tok0 + t_in;
  if (p.ws_rparts && it.sigma == 0 && h == 0)
    p.ws_rparts[tok * p.num_q_heads + head] = it.parts;   // the row's part count, for pa_merge
  if (it.parts == 1) {
    if (h == 0) store_lse(p.lse_out, p.lse_st, tok, head, lt > 0.f ? m * c + __log2f(lt) : kNegInf);
    uint16_t* op = p.out + tok * p.o_st + (int64_t)head * p.o_sh + 4 * h;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 w = {E::pack2(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv),
                         E::pack2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * j) = w;
      }
  } else {
    const int64_t r = ((int64_t)it.sigma * p.total_q + tok) * p.num_q_heads + head;
    float* wp = p.ws_o + r * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv,
                         acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(wp + 32 * dt + 8 * j) = v;
      }
    if (h == 0) p.ws_lse[r] = lt > 0.f ? m * c + __log2f(lt) : kNegInf;
  }
}

// STREAM: the tile's K/V stages are read by no other tile (16-bit caches:
// streaming DMA loads).
template <int D, int G, bool KV8, bool F16, bool STREAM>
__device__ __forceinline__ void attend_wide(const FwdParams& p, const Item& it,
                                            unsigned char* smem) {
  using E = Elem<F16>;
  // LDS layout of the stages: d = 96 rides in the d = 128 layout, its key
  // rows padded with zeros to 16 chunks (the padding chunks load as zeros and
  // no MFMA reads them), so the swizzles and DMA shapes of d = 128 serve it
  constexpr int DL = wide_layout_dim(D);
  using Cfg = WideCfg<DL>;
  constexpr int ESZ = Kv<KV8>::ESZ;
  using raw8 = typename Kv<KV8>::raw8;
  constexpr int CPR = Cfg::CPR;
  constexpr int KS = D / 16;             // contraction steps of S^T = K Q^T
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int CPT = Cfg::CPT;
  constexpr int RPI = Cfg::RPI;
  constexpr int TB = Cfg::TENSOR_BYTES;
  constexpr int SB = Cfg::STAGE_BYTES;
  constexpr float kThr = 8.f;            // log2 headroom before the reference max moves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- rows of this lane
  // A tile of at most 64 rows splits every stage's keys instead: waves w and
  // w + 2 own the same 32 rows, wave w the first 32 keys of each stage and
  // wave w + 2 the last 32; the two halves' (m, l, O) merge after the loop.
  const bool ksplit = it.rows <= 64;
  const int rw = ksplit ? (wave & 1) : wave;          // 32-row block of this wave
  const int kh = ksplit ? (wave >> 1) : 0;            // key half (ksplit)
  const int row = rw * 32 + l32;
  const bool row_ok = row < it.rows;
  const int t_in = row / G;
  const int head = it.kvh * G + row % G;
  const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4 qB[KS];                           // B operand of S^T: d = 16 ks + 8 h + e
  {
    const uint16_t* qp = p.q + (int64_t)(it.q0 + it.tok0 + (row_ok ? t_in : 0)) * p.q_st +
                         (int64_t)head * p.q_sh + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      v ^= qflip;
      qB[ks] = v;
    }
  }
  const int kbeg = it.kbeg, kend = it.kend;
  const int klim = p.causal ? min(kend, it.diag + it.tok0 + t_in + 1) : kend;
  // keys below w_kmin are admissible for every row of this wave (no mask)
  const int w_kmin = p.causal ? min(kend, it.diag + it.tok0 + (rw * 32) / G + 1) : kend;

  const int blk0 = kbeg / kBlockSize;
  const int nblk = kend > kbeg ? (kend + kBlockSize - 1) / kBlockSize - blk0 : 0;
  const int n_stage = kend > kbeg ? (kend - kbeg + kStageKeys - 1) / kStageKeys : 0;
  const int32_t* btrow = p.bt + (int64_t)it.s * p.bt_stride;
  const int64_t head_off = (int64_t)it.kvh * D;
  // byte offset of each sub-block's (kv-head) tile; entries past nblk are
  // padding (loads past the end have zero records and read nothing)
  int64_t* offs = reinterpret_cast<int64_t*>(smem + Cfg::OFFS_OFFSET);
  for (int i = tid; i < 4 * n_stage + 4; i += kThreads)
    offs[i] = i < nblk ? (sub_block_base(p, sub_block_id(btrow, blk0 + i, p.bshift)) + head_off) * ESZ
                       : 0;
  __syncthreads();

  // ---- one stage of K and V.  bf16: global -> LDS by 16-byte DMA; lane i of
  // a wave's load lands at LDS base + 16 i, so each lane fetches the chunk
  // the swizzled layout keeps at its slot (key row r, slot s holds chunk
  // s ^ f(r)).  fp8: each lane loads its row chunk's 8 codes into registers
  // and, after the stage's compute, writes them as bf16 to the swizzled slot.
  const int slot_elems = p.num_kv_heads * D;
  // Load u of a wave covers stage rows u * 4 RPI + wave * RPI + [0, RPI);
  // this lane takes row ld_r of them (+ u * 4 RPI) and slot / chunk ld_p.
  // The swizzle depends on the row mod 16, which is ld_r's except at d = 256
  // (8 rows per load: odd loads are rows 8 .. 15 of their block), hence NV
  // address sets, load u using set u % NV.
  constexpr int NV = DL == 256 ? 2 : 1;
  const int ld_r = wave * RPI + lane / CPR;
  const int ld_p = lane % CPR;                       // slot (bf16) or chunk (fp8) in the row
  int ld_gk[NV], ld_gv[NV], ld_sk[NV], ld_sv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int r = ld_r + v * 4 * RPI;                // stage row mod 16 of loads u = v (mod NV)
    // (a padding chunk, d = 96: an offset past every block's records, so the
    // load returns zeros without a memory access)
    const int ck = KV8 ? ld_p : (ld_p ^ Cfg::fk(r));
    const int cv = KV8 ? ld_p : (ld_p ^ Cfg::fv(r));
    ld_gk[v] = ck < D / 8 ? ((r % kBlockSize) * slot_elems + ck * 8) * ESZ : kPadOffset;
    ld_gv[v] = cv < D / 8 ? ((r % kBlockSize) * slot_elems + cv * 8) * ESZ : kPadOffset;
    ld_sk[v] = (ld_r * CPR + (ld_p ^ Cfg::fk(r))) * 16;   // fp8: LDS slot of the chunk
    ld_sv[v] = (ld_r * CPR + (ld_p ^ Cfg::fv(r))) * 16;
  }
  const uint32_t lds0 = uniform((int)(uint32_t)(uintptr_t)smem) + wave * RPI * CPR * 16;
  raw8 kraw[KV8 ? CPT : 1], vraw[KV8 ? CPT : 1];
  // wave-uniform copies: the per-block address and bound arithmetic is scalar
  const int kend_u = uniform(kend), blk0_u = uniform(blk0);
  auto load_stage = [&](int st, int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      // block within the stage of this wave's rows: 2u + wave/2 (d = 64), u
      // (d = 128) or u/2 (d = 256)
      const int bi = (u * 4 * RPI + wave * RPI) / kBlockSize;
      const int jl = st * (kStageKeys / kBlockSize) + bi;
      const int64_t boff = uniform64(offs[jl]);
      // keys of the block inside the item (0 past its end: no memory access,
      // the DMA writes zeros)
      const int valid = min(max(kend_u - (blk0_u + jl) * kBlockSize, 0), kBlockSize);
      const int nrec = uniform(valid * p.num_kv_heads * D * ESZ);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.k + boff), (short)0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.v + boff), (short)0, nrec, 0x00020000);
      if constexpr (KV8) {
        kraw[u] = bload8<true>(rk, ld_gk[u % NV]);
        vraw[u] = bload8<true>(rv, ld_gv[u % NV]);
      } else {
        const uint32_t dst = lds0 + buf * SB + u * 4 * RPI * CPR * 16;
        dma16<STREAM ? kStreamLoad : 0>(rk, ld_gk[u % NV], dst);
        dma16<STREAM ? kStreamLoad : 0>(rv, ld_gv[u % NV], dst + TB);
      }
    }
  };
  // fp8: the registers of the last load_stage, as bf16, into LDS buffer buf
  auto store_stage = [&](int buf) {
    if constexpr (KV8) {
      unsigned char* base = smem + buf * SB;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        *reinterpret_cast<u32x4*>(base + u * 4 * RPI * CPR * 16 + ld_sk[u % NV]) = to_elem8<F16>(kraw[u]);
        *reinterpret_cast<u32x4*>(base + TB + u * 4 * RPI * CPR * 16 + ld_sv[u % NV]) =
            to_elem8<F16>(vraw[u]);
      }
    }
  };

  // ---- per-lane LDS read offsets
  int koff[KS];                          // K operand: key row l32 (+32 kb), chunk 2 ks + h
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (l32 * CPR + ((2 * ks + h) ^ Cfg::fk(l32))) * 16;
  const int j16 = lane & 15;
  const int tr_row = 4 * h + (j16 >> 2);               // + 16 slice + 8 half
  int voff[DT];                          // V^T operand: transpose read of 4 rows x 16 d
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int chunk = 4 * dt + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    voff[dt] = (tr_row * CPR + (chunk ^ Cfg::fv(tr_row))) * 16 + 8 * (j16 & 1);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = kNegInf;                     // reference max (raw score units)
  float l = 0.f;                         // this lane's half of the row sum
  const float thr = kThr / c;

  // One stage (HALF: only key half kh of it).  S^T for the stage's keys, mask
  // (only where a row limit falls inside the stage), then per 32-key half:
  // row max, (rare) rescale, exp, O^T += V^T P^T.  The half-0 softmax
  // overlaps the half-1 score MFMAs and the half-0 P V MFMAs overlap the
  // half-1 softmax.  No branch touches the accumulators except the in-place
  // rescale.
  auto compute = [&](const unsigned char* Kb, int kst, auto halfc) {
    constexpr bool HALF = decltype(halfc)::value;
    constexpr int NKB = HALF ? 1 : 2;                // 32-key halves computed
    const int kb0 = HALF ? kh : 0;
    const unsigned char* Vb = Kb + TB;
    f32x16 s[NKB];
#pragma unroll
    for (int i = 0; i < NKB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.f;
#pragma unroll
    for (int i = 0; i < NKB; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(Kb + (kb0 + i) * 32 * CPR * 16 + koff[ks]);
        s[i] = E::mma32(a, qB[ks], s[i]);
      }
    // operand reads run 4 ahead of the MFMAs: latency hidden, 16 registers
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NKB * KS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (kst + kStageKeys > w_kmin) {
      // element (i, r) is key 32 (kb0 + i) + 8(r/4) + r%4 + 4h of the stage
      const int rel = klim - kst - 4 * h - 32 * kb0;
#pragma unroll
      for (int i = 0; i < NKB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * i + 8 * (r >> 2) + (r & 3) >= rel) s[i][r] = kNegInf;
    }
#pragma unroll
    for (int i = 0; i < NKB; ++i) {
      const int kb = kb0 + i;
      float mx = s[i][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[i][r]);
      mx = swap_halves_max(mx);
      const float mnew = fmaxf(m, mx);
      if (__builtin_amdgcn_ballot_w64(mnew > m + thr)) {
        const float alpha = m == kNegInf ? 0.f : exp2_fast((m - mnew) * c);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = acc[dt][r];
            scale_inplace(x, alpha);
            acc[dt][r] = x;
          }
      }
      const float mc = m == kNegInf ? 0.f : m * c;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = exp2_fast(__builtin_fmaf(s[i][r], c, -mc));
        l += pr[r];
      }
      u32x4 pb[2];                               // P^T operand of slice 2 kb + hs
#pragma unroll
      for (int r = 0; r < 16; r += 2) pb[r >> 3][(r & 7) >> 1] = E::pack2(pr[r], pr[r + 1]);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int sl = 2 * kb + hs;                // 16-key slice of the stage
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const unsigned char* a = Vb + sl * 16 * CPR * 16 + voff[dt];
          const i16x4 a0 = lds_read_tr((PA_LDS bf16x4*)(a));
          const i16x4 a1 = lds_read_tr((PA_LDS bf16x4*)(a + 8 * CPR * 16));
          const u32x4 packed = {__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                                __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]};
          acc[dt] = E::mma32(packed, pb[hs], acc[dt]);
        }
      }
    }
  };

  // One pipeline step; `buf` is a constant so LDS offsets fold into the reads.
  // The other buffer was released by the previous step's barrier; its DMA
  // completes (vmcnt) before this step's barrier.  The loads of the step after
  // the last one have zero records (no memory access) and are never read.  A
  // wave whose 32 rows all lie past the tile's rows (a short tile) only loads
  // and synchronises: its scores and weights would go nowhere.
  const bool wave_rows = uniform(rw * 32 < it.rows ? 1 : 0) != 0;
  auto run = [&](auto halfc) {
    auto step = [&](int st, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      load_stage(st + 1, buf ^ 1);
      if (wave_rows) compute(smem + buf * SB, kbeg + st * kStageKeys, halfc);
      store_stage(buf ^ 1);
      wait_dma();
      __syncthreads();
    };
    for (int st = 0; st < n_stage; st += 2) {
      step(st, std::integral_constant<int, 0>());
      if (st + 1 < n_stage) step(st + 1, std::integral_constant<int, 1>());
    }
  };

  if (n_stage > 0) {
    load_stage(0, 0);
    store_stage(0);
  }
  wait_dma();
  __syncthreads();
  if (ksplit) run(std::true_type());
  else run(std::false_type());

  // ---- key halves: wave w + 2 hands its (m, l, O) to wave w (same rows and
  // lane layout) through the now idle stage buffers
  if (ksplit) {
    constexpr int RS = 16 * DT + 4;                   // floats per lane (16-byte aligned)
    float* red = reinterpret_cast<float*>(smem) + (wave & 1) * 64 * RS;
    float* mine = red + lane * RS;
    if (kh == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *reinterpret_cast<f32x4*>(mine + 16 * dt + r) =
              f32x4{acc[dt][r], acc[dt][r + 1], acc[dt][r + 2], acc[dt][r + 3]};
      mine[16 * DT] = m;
      mine[16 * DT + 1] = l;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = mine[16 * DT], l1 = mine[16 * DT + 1];
    const float mm = fmaxf(m, m1);
    const float a0 = m == kNegInf ? 0.f : exp2_fast((m - mm) * c);
    const float a1 = m1 == kNegInf ? 0.f : exp2_fast((m1 - mm) * c);
    l = a0 * l + a1 * l1;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(mine + 16 * dt + r);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][r + e] = a0 * acc[dt][r + e] + a1 * o[e];
      }
    m = mm;
  }

  wide_epilogue<D, G, F16>(p, it, acc, m, l, c, row_ok, t_in, head, h);
}

// ---------------------------------------------------------------------------
// Eight-wave wide tiles (up to 256 packed rows; d = 64 and 128; 16-bit caches).
//
// Waves 0-3 (group A) and 4-7 (group B) each own 32 rows, and waves w and w + 4
// share SIMD w.  The two groups run in opposite phases, half a stage apart,
// with a work-group barrier at every half-step: while one group issues its
// MFMA block (P V of the previous stage and S^T = K Q^T of the current one)
// the other computes the softmax of its last scores, so every SIMD has a
// matrix-core stream and a vector-ALU stream from two different waves.
//
//   half-step 2t    : A  P V(t-1), S(t)     B  softmax(t-1)
//   half-step 2t+1  : A  softmax(t)         B  P V(t-1), S(t)
//
// Stage t's K is read at half-steps 2t and 2t+1, its V at 2t+2 and 2t+3.  K
// and V stages go global -> LDS by 16-byte DMA into a ring of four stage
// buffers, issued two stages (four half-steps) ahead, at even half-steps into
// the buffer stage t - 2 released; each wave waits for its own part of the
// stage needed next (vmcnt) before the barrier that publishes it.  The
// softmax of a stage takes the max over all 64 keys first, then moves the
// reference (rescaling O and l) at most once, so both halves' weights share
// one reference.  Row and key layouts are those of the four-wave path.
// ---------------------------------------------------------------------------
// cache blocks in flight per wave on the narrow path (d = 256: one, for registers)
template <int D>
constexpr int narrow_ring() { return D == 256 ? 1 : 2; }

constexpr int kWide8Threads = 512;

template <int D>
struct Wide8Cfg {
  static constexpr int NW = 8;
  static constexpr int NBUF = 4;                            // stage buffers in the ring
  static constexpr int AHEAD = 2;                           // stages loaded ahead of use
  static constexpr int CPR = D / 8;
  static constexpr int TENSOR_BYTES = kStageKeys * D * 2;
  static constexpr int STAGE_BYTES = 2 * TENSOR_BYTES;     // K, then V
  static constexpr int OFFS_OFFSET = NBUF * STAGE_BYTES;
  // sub-block byte offsets of the unit; the loads of the stages past the end
  // read padding entries (and touch no memory)
  static constexpr int OFFS_ENTRIES = kMaxSplitKeys / kBlockSize + 4 * (AHEAD + 1);
  static constexpr int SMEM_RAW = OFFS_OFFSET + OFFS_ENTRIES * 8;
  static constexpr int SMEM = SMEM_RAW > NarrowCfg<D, 8>::SMEM ? SMEM_RAW : NarrowCfg<D, 8>::SMEM;
  static constexpr int RPI = 64 / CPR;                      // key rows per wave-wide 1 KB DMA
  static constexpr int DPW = kStageKeys / (NW * RPI);       // DMAs per wave per tensor per stage
};

template <int D, int G, bool F16>
__device__ __forceinline__ void attend_wide8(const FwdParams& p, const Item& it,
                                             unsigned char* smem) {
  using E = Elem<F16>;
  using Cfg = Wide8Cfg<D>;
  using WC = WideCfg<D>;                 // LDS chunk swizzles
  constexpr int CPR = Cfg::CPR;
  constexpr int KS = D / 16;             // contraction steps of S^T = K Q^T
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int TB = Cfg::TENSOR_BYTES;
  constexpr int SB = Cfg::STAGE_BYTES;
  constexpr int RPI = Cfg::RPI;
  constexpr int DPW = Cfg::DPW;
  constexpr int NBUF = Cfg::NBUF;
  constexpr int NW = Cfg::NW;
  constexpr float kThr = 8.f;            // log2 headroom before the reference max moves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2;             // 0: group A, 1: group B
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int row = wave * 32 + l32;
  const bool row_ok = row < it.rows;
  const int t_in = row / G;
  const int head = it.kvh * G + row % G;
  const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4 qB[KS];                          // B operand of S^T: d = 16 ks + 8 h + e
  {
    const uint16_t* qp = p.q + (int64_t)(it.q0 + it.tok0 + (row_ok ? t_in : 0)) * p.q_st +
                         (int64_t)head * p.q_sh + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      v ^= qflip;
      qB[ks] = v;
    }
  }
  const int kbeg = it.kbeg, kend = it.kend;
  const int klim = p.causal ? min(kend, it.diag + it.tok0 + t_in + 1) : kend;
  // keys below w_kmin are admissible for every row of this wave (no mask);
  // keys at or past w_kend are admissible for none of them
  const bool wave_rows = wave * 32 < it.rows;
  const int w_kmin = p.causal ? min(kend, it.diag + it.tok0 + (wave * 32) / G + 1) : kend;
  const int w_last = min(wave * 32 + 31, it.rows - 1);
  const int w_kend = !wave_rows ? kbeg : (p.causal ? min(kend, it.diag + it.tok0 + w_last / G + 1) : kend);
  const int n_stage = kend > kbeg ? (kend - kbeg + kStageKeys - 1) / kStageKeys : 0;
  const int w_nst = uniform(w_kend > kbeg ? (w_kend - kbeg + kStageKeys - 1) / kStageKeys : 0);

  const int blk0 = kbeg / kBlockSize;
  const int nblk = kend > kbeg ? (kend + kBlockSize - 1) / kBlockSize - blk0 : 0;
  const int32_t* btrow = p.bt + (int64_t)it.s * p.bt_stride;
  const int64_t head_off = (int64_t)it.kvh * D;
  int64_t* offs = reinterpret_cast<int64_t*>(smem + Cfg::OFFS_OFFSET);
  for (int i = tid; i < 4 * (n_stage + Cfg::AHEAD + 1); i += kWide8Threads)
    offs[i] = i < nblk ? (sub_block_base(p, sub_block_id(btrow, blk0 + i, p.bshift)) + head_off) * 2
                       : 0;
  __syncthreads();

  // ---- DMA of one stage: DPW 1 KB loads per tensor per wave.  Load u of wave
  // w covers key rows r0 = (u NW + w) RPI .. + RPI; lane i fetches the chunk
  // the swizzled layout keeps at LDS slot i % CPR of row r0 + i / CPR.
  const int slot_elems = p.num_kv_heads * D;
  int ld_gk[DPW], ld_gv[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int r = (u * NW + wave) * RPI + lane / CPR;
    const int sl = lane % CPR;
    ld_gk[u] = ((r % kBlockSize) * slot_elems + (sl ^ WC::fk(r)) * 8) * 2;
    ld_gv[u] = ((r % kBlockSize) * slot_elems + (sl ^ WC::fv(r)) * 8) * 2;
  }
  const uint32_t lds0 = uniform((int)(uint32_t)(uintptr_t)smem);
  const int kend_u = uniform(kend), blk0_u = uniform(blk0);
  // stage st into ring buffer BUF (st % NBUF, a constant at every call site)
  auto issue_stage = [&](int st, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int r0 = (u * NW + wave) * RPI;
      const int jl = st * (kStageKeys / kBlockSize) + r0 / kBlockSize;
      const int64_t boff = uniform64(offs[jl]);
      const int valid = min(max(kend_u - (blk0_u + jl) * kBlockSize, 0), kBlockSize);
      const int nrec = uniform(valid * slot_elems * 2);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.k + boff), (short)0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.v + boff), (short)0, nrec, 0x00020000);
      const uint32_t dst = lds0 + buf * SB + r0 * CPR * 16;
      dma16(rk, ld_gk[u], dst);
      dma16(rv, ld_gv[u], dst + TB);
    }
  };

  // ---- per-lane LDS read offsets (within a stage buffer)
  int koff[KS];                          // K operand: key row l32 (+32 kb), chunk 2 ks + h
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (l32 * CPR + ((2 * ks + h) ^ WC::fk(l32))) * 16;
  const int j16 = lane & 15;
  const int tr_row = 4 * h + (j16 >> 2);
  int voff[DT];                          // V^T operand: transpose read of 4 rows x 16 d
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int chunk = 4 * dt + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    voff[dt] = TB + (tr_row * CPR + (chunk ^ WC::fv(tr_row))) * 16 + 8 * (j16 & 1);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = kNegInf;                     // reference max (raw score units)
  float l = 0.f;                         // this lane's half of the row sum
  const float thr = kThr / c;
  f32x16 sc[2];                          // S^T of the stage, from the MFMA block to the softmax
  u32x4 pb[4];                           // P^T operands of the stage's four 16-key slices
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[i][r] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = u32x4{0u, 0u, 0u, 0u};

  // MFMA block: O^T += V^T P^T of the previous stage (if pv), then S^T = K Q^T
  // of this stage (if s).  Consecutive MFMAs of a product alternate between
  // independent accumulators (the d tiles of O^T, the two score halves); the
  // products run one after the other, so the scores and the P^T operands are
  // never live at the same time.
  constexpr int NSTEP = 4 * DT;          // == 2 KS: MFMAs of each product per stage
  auto pv_operand = [&](const unsigned char* Vb, int j) -> u32x4 {
    const int sl = j / DT, dt = j % DT;
    const unsigned char* a = Vb + sl * 16 * CPR * 16 + voff[dt];
    const i16x4 a0 = lds_read_tr((PA_LDS bf16x4*)(a));
    const i16x4 a1 = lds_read_tr((PA_LDS bf16x4*)(a + 8 * CPR * 16));
    return u32x4{__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                 __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]};
  };
  auto k_operand = [&](const unsigned char* Kb, int j) -> u32x4 {
    const int i = j & 1, ks = j >> 1;    // score half i, contraction step ks
    return *reinterpret_cast<const u32x4*>(Kb + i * 32 * CPR * 16 + koff[ks]);
  };
  auto zero_scores = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[i][r] = 0.f;
  };
  // KBUF: ring buffer of stage t (its K); stage t - 1 (its V) is the one before
  auto mfma_block = [&](auto kbufc, bool do_s, bool do_pv) {
    constexpr int KBUF = decltype(kbufc)::value;
    const unsigned char* Kb = smem + KBUF * SB;
    const unsigned char* Vb = smem + ((KBUF + NBUF - 1) % NBUF) * SB;
    // each product's operand reads run LA steps ahead of its MFMAs (source
    // order is issue order)
    constexpr int LA = 4;
    if (do_pv) {
      u32x4 win[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) win[j] = pv_operand(Vb, j);
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        const u32x4 cur = win[j % LA];
        if (j + LA < NSTEP) win[j % LA] = pv_operand(Vb, j + LA);
        acc[j % DT] = E::mma32(cur, pb[j / DT], acc[j % DT]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);     // LA steps of reads
#pragma unroll
      for (int j = 0; j < NSTEP - LA; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // an MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // the reads LA steps ahead
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    }
    if (do_s) {
      zero_scores();
      u32x4 win[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) win[j] = k_operand(Kb, j);
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        const u32x4 cur = win[j % LA];
        if (j + LA < NSTEP) win[j % LA] = k_operand(Kb, j + LA);
        sc[j & 1] = E::mma32(cur, qB[j >> 1], sc[j & 1]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int j = 0; j < NSTEP - LA; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    }
  };

  // softmax of stage st (its scores in sc): mask where a row limit falls in
  // the stage, stage max over all 64 keys, (rare) move of the reference with
  // O and l rescaled, weights into the P^T operands.
  auto softmax = [&](int st) {
    const int kst = kbeg + st * kStageKeys;
    if (kst + kStageKeys > w_kmin) {
      // element (i, r) is key 32 i + 8(r/4) + r%4 + 4h of the stage
      const int rel = klim - kst - 4 * h;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * i + 8 * (r >> 2) + (r & 3) >= rel) sc[i][r] = kNegInf;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    mx = swap_halves_max(mx);
    const float mnew = fmaxf(m, mx);
    if (__builtin_amdgcn_ballot_w64(mnew > m + thr)) {
      const float alpha = m == kNegInf ? 0.f : exp2_fast((m - mnew) * c);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = acc[dt][r];
          scale_inplace(x, alpha);
          acc[dt][r] = x;
        }
    }
    const float mc = m == kNegInf ? 0.f : m * c;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = exp2_fast(__builtin_fmaf(sc[i][r], c, -mc));
        l += pr[r];
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) pb[2 * i + (r >> 3)][(r & 7) >> 1] = E::pack2(pr[r], pr[r + 1]);
    }
  };

  // ---- the half-step loop: n_stage + 1 steps of two half-steps; both groups
  // meet the same barriers (one per half-step but the last).  The barriers
  // order LDS only: the DMA stages are ordered by each wave's vmcnt waits.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  issue_stage(0, B0());
  issue_stage(1, B1());
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DPW) : "memory");   // stage 0 landed
  lds_barrier();
  // One step t (two half-steps) of group A or B; stage t lives in buffer KB,
  // stage t + 2 goes to buffer KB + 2.  Returns false after the last step.
  // Each group has its own loop, unrolled over the ring so every LDS address
  // is a per-lane register plus an immediate.
  auto step_a = [&](int t, auto kbc) -> bool {
    constexpr int KB = decltype(kbc)::value;
    issue_stage(t + Cfg::AHEAD, std::integral_constant<int, (KB + Cfg::AHEAD) % NBUF>());
    mfma_block(kbc, t < w_nst, t >= 1 && t - 1 < w_nst);
    lds_barrier();
    if (t < w_nst) softmax(t);
    if (t == n_stage) return false;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DPW) : "memory");
    lds_barrier();
    return true;
  };
  auto step_b = [&](int t, auto kbc) -> bool {
    constexpr int KB = decltype(kbc)::value;
    issue_stage(t + Cfg::AHEAD, std::integral_constant<int, (KB + Cfg::AHEAD) % NBUF>());
    if (t >= 1 && t - 1 < w_nst) softmax(t - 1);
    lds_barrier();
    mfma_block(kbc, t < w_nst, t >= 1 && t - 1 < w_nst);
    if (t == n_stage) return false;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DPW) : "memory");
    lds_barrier();
    return true;
  };
  if (grp == 0) {
    for (int t = 0;; t += NBUF)
      if (!step_a(t, B0()) || !step_a(t + 1, B1()) || !step_a(t + 2, B2()) || !step_a(t + 3, B3()))
        break;
  } else {
    for (int t = 0;; t += NBUF)
      if (!step_b(t, B0()) || !step_b(t + 1, B1()) || !step_b(t + 2, B2()) || !step_b(t + 3, B3()))
        break;
  }

  wide_epilogue<D, G, F16>(p, it, acc, m, l, c, row_ok, t_in, head, h);
}

// The eight-wave unified grid kernel: wide tiles of up to 256 rows on the
// ping-pong path, narrow tiles on the narrow path with eight waves.
template <int D, int G, bool F16>
__global__ __launch_bounds__(kWide8Threads) __attribute__((amdgpu_waves_per_eu(2)))
void pa_fwd8_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[Wide8Cfg<D>::SMEM];
  Item it;
  if (!decode_item<G>(p, it)) return;
  if (it.rows <= p.narrow_rows) attend_narrow<D, G, narrow_ring<D>(), false, F16, 8>(p, it, smem);
  else attend_wide8<D, G, F16>(p, it, smem);
}

// WIDE = 0: every tile of the batch is narrow (the plan guarantees it); 1:
// wide tiles (16-bit caches at d = 64 and 128: those of one-tile sequences
// stream their K/V; at d = 96 and 256 the second copy of the wide path in the
// kernel measured 1.5% and 4% slower on prefill, so they do not); 2:
// wide tiles whose K/V no other tile reads (every sequence one tile; 16-bit
// caches), loaded as streaming data.  KV8: the caches hold fp8
// E4M3 codes.  F16: q, out (and 16-bit caches) are fp16, else bf16.  Two
// work-groups per CU, except wide tiles at d = 256, whose registers
// (accumulators in AGPRs) allow one wave per SIMD.
template <int D, int G, int WIDE, bool KV8, bool F16>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(WIDE != 0 && D == 256 ? 1 : 2)))
void pa_fwd_kernel(FwdParams p) {
  constexpr bool HAS_WIDE = WIDE != 0;
  constexpr int WSMEM = WideCfg<wide_layout_dim(HAS_WIDE ? D : 128)>::SMEM;
  constexpr int SMEM = HAS_WIDE && WSMEM > NarrowCfg<D>::SMEM ? WSMEM : NarrowCfg<D>::SMEM;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  Item it;
  if (!decode_item<G>(p, it)) return;
  if (it.rows <= p.narrow_rows) {
    attend_narrow<D, G, narrow_ring<D>(), KV8, F16>(p, it, smem);
  } else {
    if constexpr (HAS_WIDE) {
      // a sequence of one tile: no other tile reads its K/V (decode rows and
      // short chunks next to prefill tiles), so they stream
      if constexpr (WIDE == 1 && !KV8 && (D == 64 || D == 128)) {
        if (it.q_len <= p.tile_tokens) attend_wide<D, G, KV8, F16, true>(p, it, smem);
        else attend_wide<D, G, KV8, F16, false>(p, it, smem);
      } else {
        attend_wide<D, G, KV8, F16, WIDE == 2>(p, it, smem);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent decode kernel (batches whose every sequence is one narrow tile).
//
// Work list, two modes.  Fixed parts: sequence s contributes n_s key parts of
// split_keys keys (one if L_s = 0, none if it has no query) and every (s,
// part, kv-head) is one item; items are dealt to XCDs in contiguous ranges
// and the waves of one XCD stride through its range, so the kv-heads of a
// sequence (which share its cache blocks) stream together.  Even split (for
// ragged batches): the sequences, each ceil(L_s / 16) blocks long (at least
// one), are laid end to end as one stream of blocks, cut into equal chunks;
// every (chunk, kv-head) pair is one wave's work (one or more pairs per wave),
// an item is the piece of one sequence inside a chunk for that kv-head, and a
// row's parts are the chunks its sequence touches.  Every wave then streams
// the same number of blocks however skewed the lengths (stream-K), and the
// waves of a work-group read the same blocks for different kv-heads.
// Either way one item is streamed by ONE wave from start to end: no
// cross-wave merge and no work-group barrier after the set-up.  Each
// work-group builds the prefix sums of the per-sequence units in LDS once and
// stages the per-sequence metadata there.
//
// A wave's block stream continues across items: the last refills of an item
// already fetch the next item's first blocks (its block ids and Q were loaded
// one item ahead), so HBM keeps streaming while the wave writes its rows.  A
// sequence with one part writes its rows directly; rows of sequences with
// several parts go to the workspace for pa_merge.
// ---------------------------------------------------------------------------
constexpr int kMaxItemBlocks = kMaxSplitKeys / kBlockSize;   // 256 blocks per item

template <int D>
struct DecodeCfg {
  // cache blocks in flight per wave (d = 256: one, for registers and LDS)
  static constexpr int RING = D == 256 ? 1 : kDecodeRing;
  static constexpr int BLK_BYTES = kBlockSize * D * 2;
  static constexpr int VBUF_BYTES = 4 * RING * BLK_BYTES;         // a V buffer per ring slot
  static constexpr int IDS_OFFSET = VBUF_BYTES;                   // int [4 waves][2][256]
  static constexpr int PREF_OFFSET = IDS_OFFSET + 4 * 2 * kMaxItemBlocks * 4;  // int [S + 1]
  static constexpr int Q0_OFFSET = PREF_OFFSET + (kMaxDecodeSeqs + 1) * 4;   // int [S + 1]
  static constexpr int LEN_OFFSET = Q0_OFFSET + (kMaxDecodeSeqs + 1) * 4;   // int [S]
  static constexpr int SLOT_OFFSET = LEN_OFFSET + kMaxDecodeSeqs * 4;        // int [S + 1]
  static constexpr int SCAN_OFFSET = (SLOT_OFFSET + (kMaxDecodeSeqs + 1) * 4 + 7) / 8 * 8;  // 4 x i64
  static constexpr int SMEM = SCAN_OFFSET + 32;
};


// Key parts of a sequence with `ql` queries and context L (fixed-size parts
// of `target` keys, at most n_split).
__device__ __forceinline__ int seq_parts(const FwdParams& p, int ql, int L, int target) {
  if (ql <= 0) return 0;
  return min(max((L + target - 1) / target, 1), p.n_split);
}

struct DItem {
  int valid;
  int s, kvh, sigma, units;
  int slot;              // even split: partial slot of the item (the sequence's first slot + sigma)
  int q0, q_len, rows, L, diag;
  int kbeg, kend, kmin;
  int blk0, nb;          // first block and number of blocks of the item
  int c, next;           // even split: (chunk, kv-head) pair and stream position after the item;
                         // fixed parts: the wave's next item ordinal
};

// Largest s in [0, S) with pref[s] <= key, for a non-decreasing table with
// pref[0] = 0 <= key (key wave-uniform, S <= 2048, the table holding 2049
// entries): two 64-lane ballots, over every 32nd entry and then over the 32
// entries of the group found, instead of a chain of dependent LDS reads.
__device__ __forceinline__ int seq_of(const int* pref, int S, int key) {
  const int lane = threadIdx.x & 63;
  const int i1 = lane * 32;                          // <= 2016
  const bool le1 = i1 < S && pref[i1] <= key;
  const int g = uniform(__popcll(__ballot(le1)) - 1);
  const int i2 = g * 32 + (lane & 31);               // <= 2047
  const bool le2 = lane < 32 && i2 < S && pref[i2] <= key;
  return uniform(g * 32 + __popcll(__ballot(le2)) - 1);
}

// Item -> (sequence, part, kv-head) from the LDS tables only.
template <int G>
__device__ __forceinline__ DItem describe_item(const FwdParams& p, const int* pref,
                                               const int* q0t, const int* lent, int n_items,
                                               int item, int target) {
  DItem d = {};            // an invalid item is all zeros: kv-head 0, no blocks
  d.valid = item < n_items;
  if (!d.valid) return d;
  const int unit = item / p.num_kv_heads;
  d.kvh = item - unit * p.num_kv_heads;
  const int lo = seq_of(pref, p.num_seqs, unit);   // largest s with pref[s] <= unit
  d.s = lo;
  d.sigma = unit - uniform(pref[lo]);
  d.units = uniform(pref[lo + 1]) - uniform(pref[lo]);
  d.q0 = uniform(q0t[lo]);
  d.q_len = uniform(q0t[lo + 1]) - d.q0;
  d.rows = d.q_len * G;
  d.L = uniform(lent[lo]);
  d.diag = d.L - d.q_len;
  d.kbeg = d.sigma * target;
  d.kend = max(0, min(d.L, d.kbeg + target));
  d.kmin = p.causal ? min(d.kend, d.diag + 1) : d.kend;
  d.blk0 = d.kbeg / kBlockSize;
  d.nb = d.kend > d.kbeg ? (d.kend + kBlockSize - 1) / kBlockSize - d.blk0 : 0;
  return d;
}

template <int D, int G, bool KV8, bool F16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void pa_decode_kernel(FwdParams p) {
  using E = Elem<F16>;
  constexpr int ESZ = Kv<KV8>::ESZ;
  using raw8 = typename Kv<KV8>::raw8;
  using Lay = Layout<D>;
  using Cfg = DecodeCfg<D>;
  constexpr int CPR = Lay::CPR;
  constexpr int BLK_BYTES = Lay::BLK_BYTES;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int VPL = kBlockSize * CPR / 64;
  constexpr int IDL = kMaxItemBlocks / 64;          // block ids per lane per item
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int h4 = lane >> 4;
  const int l16 = lane & 15;
  int* pref = reinterpret_cast<int*>(smem + Cfg::PREF_OFFSET);
  int* q0t = reinterpret_cast<int*>(smem + Cfg::Q0_OFFSET);
  int* lent = reinterpret_cast<int*>(smem + Cfg::LEN_OFFSET);
  int* slots = reinterpret_cast<int*>(smem + Cfg::SLOT_OFFSET);
  int* wsum = reinterpret_cast<int*>(smem + Cfg::SCAN_OFFSET);
  int* idsw = reinterpret_cast<int*>(smem + Cfg::IDS_OFFSET) + wave * 2 * kMaxItemBlocks;

  // ---- per-sequence metadata and prefix sums of per-sequence units ----
  // Thread t owns sequences s0 .. s1 - 1 and keeps their query lengths,
  // contexts, units and first positions in registers, so the scans read no
  // LDS but the per-wave totals; the tables go to LDS for the item lookups.
  const int S = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  constexpr int CM = (kMaxDecodeSeqs + kThreads - 1) / kThreads;   // sequences per thread, at most
  const int C = (S + kThreads - 1) / kThreads;
  const int s0 = min(S, tid * C), s1 = min(S, s0 + C);
  const int workers = (int)gridDim.x * 4;
  const int target = p.split_keys;                   // fixed parts: keys per part
  int ur[CM], xr[CM];                                // units and first position of s0 + c
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    ur[c] = 0;
    if (c >= C) continue;                            // (uniform: batches of <= 256 take one)
    const int s = s0 + c;
    const int sc = min(s, S - 1);                    // a valid index (S >= 1: the host launches
                                                     // nothing for an empty batch), so the
                                                     // loads need no branch
    const int q0 = p.cu_q[sc];
    const int ql = p.cu_q[sc + 1] - q0;
    const int L = context_len(p, sc);
    const bool own = c < C && s < s1;
    if (own) {
      q0t[s] = q0;
      lent[s] = L;
    }
    // units of a sequence per kv-head: its parts (fixed), or its blocks in
    // the stream (even split; a row with no key still takes one position, so
    // its zero output gets written)
    const int u = p.balanced ? (ql > 0 ? max((L + kBlockSize - 1) / kBlockSize, 1) : 0)
                             : seq_parts(p, ql, L, target);
    if (own) ur[c] = u;
  }
  if (tid == 0) q0t[S] = p.cu_q[S];
  // exclusive prefix over the sequences of v[] (this thread's run) into
  // out[0..S], per-wave totals in wsum[slot0 .. slot0 + 3]; one barrier.
  // Returns the total; first[c] receives the prefix of sequence s0 + c.
  auto scan_seqs = [&](const int (&v)[CM], int (&first)[CM], int* out, int slot0) -> int {
    int local = 0;
#pragma unroll
    for (int c = 0; c < CM; ++c) local += v[c];
    const int incl = wave_incl_scan(local);
    if (lane == 63) wsum[slot0 + wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = wsum[slot0 + w];
      base += w < wave ? t : 0;
      total += t;
    }
    int run = base + incl - local;
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      first[c] = run;
      if (c < C && s0 + c < s1) out[s0 + c] = run;
      run += v[c];
    }
    if (tid == 0) out[S] = total;
    return uniform(total);
  };
  const int n_seq_units = scan_seqs(ur, xr, pref, 0);
  // fixed parts: items, kv-heads included; even split: the blocks of the
  // per-sequence stream (one kv-head's worth)
  const int n_units = n_seq_units * (p.balanced ? 1 : Hkv);
  // Even split: the stream is cut into n_chunks chunks of `chunk` blocks, and
  // every (chunk, kv-head) pair is one wave's work: kpw pairs per wave, each at
  // most kMaxItemBlocks blocks (one item's block-id table) and at least
  // split_keys / 16.
  int chunk = 1, n_pairs = 0;
  if (p.balanced) {
    const int all = n_units * Hkv;                     // blocks over all kv-heads
    const int cap = workers * kMaxItemBlocks;
    const int kpw = max(1, (all + cap - 1) / cap);
    chunk = max((all + workers * kpw - 1) / (workers * kpw), target / kBlockSize);
    n_pairs = (n_units + chunk - 1) / chunk * Hkv;
    // partial slots: a sequence gets one per chunk it touches (its parts), so
    // the batch needs at most (chunks + sequences) slots, whatever its token
    // count; slot(s, part) = slots[s] + part
    int vr[CM], unused[CM];
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      const int x0 = xr[c], x1 = xr[c] + ur[c];
      vr[c] = x1 > x0 ? (x1 - 1) / chunk - x0 / chunk + 1 : 0;
    }
    scan_seqs(vr, unused, slots, 4);
  }
  __syncthreads();                                   // the tables, for every wave's lookups
  // Fixed parts: items are dealt to XCDs in contiguous ranges (work-group w
  // runs on XCD w % 8); the waves of one XCD stride through its range, and
  // consecutive items (the kv-heads of one sequence, which read the same cache
  // blocks) go to the waves of one work-group, i.e. one CU.  Even split: wave
  // gw (numbered XCD-major) takes pairs gw, gw + workers, ...; pair q is chunk
  // q / Hkv for kv-head q % Hkv, so the waves of a work-group read the same
  // blocks for different kv-heads.
  const int xcd = blockIdx.x & 7;
  const int wpx = (int)(gridDim.x >> 3) * 4;           // waves per XCD (grid % 8 == 0)
  const int n_items = p.balanced ? 0 : n_units;
  const int per_xcd = (n_items + 7) >> 3;
  const int range_end = min(n_items, (xcd + 1) * per_xcd);
  const int item0 = xcd * per_xcd + (int)(blockIdx.x >> 3) * 4 + wave;
  const int gw = xcd * wpx + (int)(blockIdx.x >> 3) * 4 + wave;
  auto item_at = [&](int m) -> int {                   // m-th item of this wave
    const int it = item0 + m * wpx;
    return it < range_end ? it : n_items;              // n_items marks "none"
  };
  if (p.balanced ? gw >= n_pairs : item_at(0) >= n_items) return;   // whole wave idle

  // Fixed parts: pos is the wave's item ordinal.  Even split: the item is the
  // piece of pair q's chunk from stream position pos to the end of its
  // sequence or of the chunk, for the pair's kv-head.
  auto describe = [&](int q, int pos) -> DItem {
    if (!p.balanced) {
      DItem d = describe_item<G>(p, pref, q0t, lent, n_items, item_at(pos), target);
      d.next = pos + 1;
      return d;
    }
    DItem d = {};
    d.valid = q < n_pairs;
    if (!d.valid) return d;
    const int c = q / Hkv;
    const int xe = min((c + 1) * chunk, n_units);
    const int lo = seq_of(pref, S, pos);               // largest s with its first block <= pos
    const int L = uniform(lent[lo]);
    const int nbe = max((L + kBlockSize - 1) / kBlockSize, 1);
    const int x0 = uniform(pref[lo]);                  // the sequence's first position
    const int b0 = pos - x0;
    const int b1 = min(nbe, b0 + (xe - pos));
    d.s = lo;
    d.kvh = q - c * Hkv;
    d.sigma = c - x0 / chunk;
    d.units = (x0 + nbe - 1) / chunk - x0 / chunk + 1;
    d.q0 = uniform(q0t[lo]);
    d.q_len = uniform(q0t[lo + 1]) - d.q0;
    d.rows = d.q_len * G;
    d.L = L;
    d.diag = L - d.q_len;
    d.kbeg = b0 * kBlockSize;
    d.kend = max(0, min(L, b1 * kBlockSize));
    d.kmin = p.causal ? min(d.kend, d.diag + 1) : d.kend;
    d.blk0 = b0;
    d.nb = d.kend > d.kbeg ? (d.kend + kBlockSize - 1) / kBlockSize - b0 : 0;
    d.slot = uniform(slots[lo]) + d.sigma;
    d.c = q;
    d.next = pos + (b1 - b0);
    return d;
  };
  auto after = [&](const DItem& d) -> DItem {
    if (!d.valid) return d;
    if (!p.balanced) return describe(0, d.next);
    int q = d.c, pos = d.next;
    if (pos >= min((q / Hkv + 1) * chunk, n_units)) {
      q += workers;
      if (q >= n_pairs) return describe(q, 0);         // invalid: no pair left
      pos = q / Hkv * chunk;
    }
    return describe(q, pos);
  };

  const int slot_stride = p.num_kv_heads * D;
  const int koff = l16 * slot_stride + 8 * h4;
  int voff[VPL], vlds[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const int c = lane + 64 * u;
    const int key = c / CPR, dc = c % CPR;
    voff[u] = key * slot_stride + dc * 8;
    vlds[u] = Lay::v_chunk(key, dc) * 16;
  }
  const int tr_key = 4 * h4 + (l16 >> 2);
  const int tr_c_lo = (l16 & 3) >> 1;
  const int tr_half = (l16 & 1) * 8;
  unsigned char* vbuf0 = smem + wave * Cfg::RING * BLK_BYTES;

  // Block ids of item d: lane l holds those of blocks l, l + 64, ... .  The
  // table row is read through a buffer resource that ends at the item's last
  // entry, and no lane branches around its load, so the loads of every item
  // in flight go out together (one round trip, not one per load).  Lanes past
  // the item's blocks hold ids that are never read (every use checks the
  // block index against nb); their loads past the resource read 0 without a
  // memory access.
  auto load_ids = [&](const DItem& d, int (&v)[IDL]) {
    const int bsh = p.bshift;
    const int entries = d.valid && d.nb > 0 ? ((d.blk0 + d.nb - 1) >> bsh) + 1 : 0;
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(p.bt + (int64_t)(d.valid ? d.s : 0) * p.bt_stride), (short)0,
        uniform(entries * 4), 0x00020000);
#pragma unroll
    for (int k = 0; k < IDL; ++k) {
      const int j = d.blk0 + lane + 64 * k;
      const int e = __builtin_amdgcn_raw_buffer_load_b32(rt, (j >> bsh) * 4, 0, 0);
      v[k] = (e << bsh) | (j & ((1 << bsh) - 1));
    }
  };
  auto store_ids = [&](int buf, const int (&v)[IDL]) {
#pragma unroll
    for (int k = 0; k < IDL; ++k) idsw[buf * kMaxItemBlocks + lane + 64 * k] = v[k];
  };
  auto load_qb = [&](const DItem& d, u32x4 (&qB)[KS]) {
    const bool ok = d.valid && l16 < d.rows;
    const uint16_t* qp = p.q + (int64_t)(d.q0 + (ok ? l16 / G : 0)) * p.q_st +
                         (int64_t)(d.kvh * G + l16 % G) * p.q_sh + 8 * h4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      qB[ks] = v;
    }
  };

  // Ring of kDecodeRing cache blocks per wave.  Every refill issues the same
  // buffer loads through a per-block resource; a slot with nothing left to
  // fetch gets a resource of zero records, so its loads return zeros without
  // touching memory while the wait counts stay the same on every path.
  constexpr int RING = Cfg::RING;
  // Every cache byte is read once per call: streaming loads (measured: the
  // 256 x 1k-key batch 178 against 199 us).  fp8 K is the exception: a wave
  // reads each 128-byte key row with four 8-byte-per-lane loads, and with
  // streaming loads the fp8 batch took 129 against 105 us; with only V
  // streaming it takes 90.
  constexpr int KAUX = KV8 ? 0 : kStreamLoad;
  raw8 kst[RING][KS];
  raw8 vst[RING][VPL];
  const int blk_extent = kBlockSize * slot_stride * ESZ;    // bytes of one block, all heads
  auto issue = [&](int kvh, int phys, bool live, int j) {
    const int64_t boff = (sub_block_base(p, phys) + (int64_t)kvh * D) * ESZ;
    const int nrec = live ? blk_extent : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + boff), (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + boff), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kst[j][ks] = bload8<KV8, KAUX>(rk, (koff + 32 * ks) * ESZ);
#pragma unroll
    for (int u = 0; u < VPL; ++u) vst[j][u] = bload8<KV8, kStreamLoad>(rv, voff[u] * ESZ);
  };

  // items m (cur), m+1 (nxt), m+2 (nx2): ids of cur and nxt live in LDS, ids of
  // nx2 in VGPRs until cur finishes; Q of nxt is prefetched.
  // Set-up: the block ids and Q of the current item, then its first ring
  // loads, whose block ids come straight from registers; the next two items
  // are described and their block ids (and the next Q) loaded after that.
  DItem cur = p.balanced ? describe(gw, gw / Hkv * chunk) : describe(0, 0);
  int ids_v0[IDL], ids_v1[IDL], ids_v2[IDL];
  load_ids(cur, ids_v0);
  // Q of the next item is loaded one item ahead (d = 256: at the switch, for
  // registers)
  constexpr bool QPRE = D <= 128;
  u32x4 qB[KS], qB_n[KS];
  load_qb(cur, qB);
  int cb = 0;
  // the first RING blocks of the first item (idle slots load nothing)
#pragma unroll
  for (int j = 0; j < RING; ++j)
    issue(cur.kvh, cur.nb > j ? __builtin_amdgcn_readlane(ids_v0[0], j) : 0, cur.nb > j, j);
  // the next two items are described while those blocks are in flight
  DItem nxt = after(cur);
  load_ids(nxt, ids_v1);
  DItem nx2 = after(nxt);
  load_ids(nx2, ids_v2);
  if constexpr (QPRE) load_qb(nxt, qB_n);
  store_ids(0, ids_v0);
  store_ids(1, ids_v1);

  while (true) {
    const int* ids_c = idsw + cb * kMaxItemBlocks;
    const int* ids_n = idsw + (cb ^ 1) * kMaxItemBlocks;
    const int klim = p.causal ? min(cur.kend, cur.diag + l16 / G + 1) : cur.kend;
    f32x4 acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;
    // stream positions of this item, padded to whole ring turns so the next
    // item's block k sits in slot k
    const int nbp = max(RING, (cur.nb + RING - 1) / RING * RING);
    for (int i = 0; i < nbp; i += RING) {
#pragma unroll
      for (int j = 0; j < RING; ++j) {
        const int b = i + j;
        // what refills slot j once it is consumed: stream position b + RING
        // of this item, else of the next item, else nothing (a zero-record load)
        const int t = b + RING;
        const bool in_cur = t < cur.nb;
        const bool in_nxt = !in_cur && t >= nbp && t - nbp < nxt.nb;
        const int r_phys = in_cur ? uniform(ids_c[t]) : (in_nxt ? uniform(ids_n[t - nbp]) : 0);
        const int r_kvh = in_cur ? cur.kvh : (in_nxt ? nxt.kvh : 0);
        const bool r_live = in_cur || in_nxt;
        // (1) consume slot j: V rows to LDS, scores S^T = K Q^T
        const bool live = b < cur.nb;
        const int kb = (cur.blk0 + b) * kBlockSize;
        unsigned char* vbuf = vbuf0 + j * BLK_BYTES;         // the slot's V buffer
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        if (live) {
#pragma unroll
          for (int u = 0; u < VPL; ++u)
            *reinterpret_cast<u32x4*>(vbuf + vlds[u]) = to_elem8<F16>(vst[j][u]);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sc = E::mma16(to_elem8<F16>(kst[j][ks]), qB[ks], sc);
        }
        // (2) refill slot j (one call site, so the ring registers never move)
        issue(r_kvh, r_phys, r_live, j);
        // (3) online softmax and O^T += V^T P^T
        if (live) {
          const bool need_mask = kb + kBlockSize > cur.kmin;
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[r] = sc[r] * p.scale_log2;
            if (need_mask && kb + 4 * h4 + r >= klim) x[r] = kNegInf;
          }
          float pr[4];
          block_weights<DT>(x, m, l, acc, pr);
          const u32x2 pB = {E::pack2(pr[0], pr[1]), E::pack2(pr[2], pr[3])};
          const bool vmask = kb + kBlockSize > cur.kend;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const unsigned char* a =
                vbuf + Lay::v_chunk(tr_key, 2 * dt + tr_c_lo) * 16 + tr_half;
            i16x4 va = __builtin_bit_cast(
                i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PA_LDS bf16x4*)(a)));
            if (vmask) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (kb + 4 * h4 + e >= cur.kend) va[e] = 0;
            }
            acc[dt] = E::mma16k16(__builtin_bit_cast(u32x2, va), pB, acc[dt]);
          }
        }
      }
    }

    // ---- this wave's rows of the item ----
    l = sum_across_groups(l);
    // (a token past max_seqlen_q, a broken precondition, has no partial slot)
    if (l16 < cur.rows && l16 / G < p.dq_tokens) {
      const float inv = l > 0.f ? p.out_scale / l : 0.f;
      const int64_t tok = cur.q0 + l16 / G;
      const int hn = cur.kvh * G + l16 % G;
      // partial row of part sigma: even split, compact slots of dq_tokens
      // tokens each; fixed parts, part-major over the batch's tokens
      const int64_t prow = p.balanced
          ? ((int64_t)cur.slot * p.dq_tokens + l16 / G) * p.num_q_heads + hn
          : ((int64_t)cur.sigma * p.total_q + tok) * p.num_q_heads + hn;
      if (p.ws_rparts && cur.sigma == 0 && h4 == 0) {
        // the row's part count (and, compact, its part-0 row), for pa_merge
        p.ws_rparts[tok * p.num_q_heads + hn] = cur.units | (p.balanced ? kCompactRow : 0);
        if (p.balanced) p.ws_rbase[tok * p.num_q_heads + hn] = (int32_t)prow;
      }
      if (cur.units == 1) {
        if (h4 == 0) store_lse(p.lse_out, p.lse_st, tok, hn, l > 0.f ? m + __log2f(l) : kNegInf);
        uint16_t* op = p.out + tok * p.o_st + (int64_t)hn * p.o_sh + 4 * h4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          u32x2 w = {E::pack2(acc[dt][0] * inv, acc[dt][1] * inv),
                     E::pack2(acc[dt][2] * inv, acc[dt][3] * inv)};
          *reinterpret_cast<u32x2*>(op + 16 * dt) = w;
        }
      } else {
        float* wp = p.ws_o + prow * D + 4 * h4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(wp + 16 * dt) = acc[dt] * inv;
        if (h4 == 0) p.ws_lse[prow] = l > 0.f ? m + __log2f(l) : kNegInf;
      }
    }
    if (!nxt.valid) break;
    // advance: nxt becomes current; nx2's ids move to LDS; fetch the one after
    cur = nxt;
    nxt = nx2;
    cb ^= 1;
    store_ids(cb ^ 1, ids_v2);
    nx2 = after(nxt);
    load_ids(nx2, ids_v2);
    if constexpr (QPRE) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qB[ks] = qB_n[ks];
      load_qb(nxt, qB_n);
    } else {
      load_qb(cur, qB);
    }
  }
}

// Log-sum-exp merge of key-split partials (all lse in the log2 domain):
// w_sigma = 2^(lse_sigma - max lse), out = sum w O_sigma / sum w.  Parts with no
// key carry lse = -inf and are skipped (their O is never read).
// Parts of a row and where they are, from the forward kernel's first part (1
// part: the row was written straight to out and is skipped).  Part sg of the
// row is partial row base + sg * stride: part-major over the batch's rows, or
// (compact even split) consecutive slots from the row's recorded base.
struct MergeRow {
  int parts;
  int64_t base, stride;
};
__device__ __forceinline__ MergeRow merge_row(const MergeParams& p, int64_t row, int64_t nrows) {
  // both words in one round trip: the base is loaded whether or not the row
  // turns out compact (the array exists whenever a plan has compact rows)
  const int raw = p.row_parts[row];
  const int cbase = p.row_base ? p.row_base[row] : 0;
  MergeRow r;
  r.parts = raw & ~kCompactRow;
  r.base = row;
  r.stride = nrows;
  if (raw & kCompactRow) {
    r.base = cbase;
    r.stride = p.part_stride_c;
  }
  return r;
}

template <bool F16>
__device__ __forceinline__ void merge_store(const MergeParams& p, int64_t row, int d0, f32x4 o,
                                            float wsum, float M) {
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t tok = row / p.num_q_heads;
  const int hd = (int)(row % p.num_q_heads);
  if (d0 == 0) store_lse(p.lse_out, p.lse_st, tok, hd, wsum > 0.f ? M + __log2f(wsum) : kNegInf);
  uint16_t* op = p.out + tok * p.o_st + (int64_t)hd * p.o_sh + d0;
  u32x2 w = {Elem<F16>::pack2(o[0] * inv, o[1] * inv), Elem<F16>::pack2(o[2] * inv, o[3] * inv)};
  *reinterpret_cast<u32x2*>(op) = w;
}

// One part into running sums kept against the largest lse seen so far (M):
// a larger lse moves M and rescales the sums first.  A part with no key
// (lse = -inf) adds nothing, whatever its O slot holds (a branch, not a
// multiply by 0).
__device__ __forceinline__ void merge_add(float ls, f32x4 o, float& M, f32x4& a, float& ws) {
  if (ls == kNegInf) return;
  if (ls > M) {
    const float s = M == kNegInf ? 0.f : exp2_fast(M - ls);
    ws *= s;
    a *= s;
    M = ls;
  }
  const float w = exp2_fast(ls - M);
  ws += w;
  a += w * o;
}

// Parts sg0, sg0 + step, ... of a row into (M, a, ws), four at a time: the
// lse and O loads of the four are issued before any of them is combined (a
// part's slot exists for every sg < parts).
template <int D>
__device__ __forceinline__ void merge_parts(const MergeParams& p, const MergeRow& mr, int d0,
                                            int sg0, int step, float& M, f32x4& a, float& ws) {
  for (int sg = sg0; sg < mr.parts; sg += 4 * step) {
    float ls[4];
    f32x4 o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = sg + k * step;
      const int64_t r = mr.base + (int64_t)min(q, mr.parts - 1) * mr.stride;
      ls[k] = q < mr.parts ? p.ws_lse[r] : kNegInf;
      o[k] = *reinterpret_cast<const f32x4*>(p.ws_o + r * D + d0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) merge_add(ls[k], o[k], M, a, ws);
  }
}

// Few parts per row: D/4 threads per row, each loops over the parts.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pa_merge_rows_kernel(MergeParams p) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;                     // d = 96: 10 rows, 16 threads idle
  if ((int)threadIdx.x >= RPB * TPR) return;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int64_t nrows = (int64_t)p.total_q * p.num_q_heads;
  if (row >= nrows) return;
  const MergeRow mr = merge_row(p, row, nrows);
  const int n_part = mr.parts;
  if (n_part <= 1) return;
  const int d0 = (threadIdx.x % TPR) * 4;
  float M = kNegInf;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
  merge_parts<D>(p, mr, d0, 0, 1, M, a, ws);
  merge_store<F16>(p, row, d0, a, ws, M);
}

// Many parts per row: one work-group per row; its threads form NG groups that
// take every NG-th part (several loads in flight each), then reduce in LDS.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pa_merge_wide_kernel(MergeParams p) {
  constexpr int TPG = D / 4;                 // threads per group (4 outputs each)
  constexpr int NG = 256 / TPG;              // groups (d = 96: 10, 16 threads in none)
  __shared__ float red[NG][D + 4];
  __shared__ float wred[NG];
  __shared__ float mred[NG];
  const int64_t row = blockIdx.x;
  const int64_t nrows = (int64_t)p.total_q * p.num_q_heads;
  const MergeRow mr = merge_row(p, row, nrows);
  if (mr.parts <= 1) return;   // uniform over the work-group
  const int t = threadIdx.x;
  const int g = t / TPG;
  const int d0 = (t % TPG) * 4;
  float M = kNegInf;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
  if (g < NG) {
    merge_parts<D>(p, mr, d0, g, NG, M, a, ws);
    *reinterpret_cast<f32x4*>(&red[g][d0]) = a;
    if (t % TPG == 0) {
      wred[g] = ws;
      mred[g] = M;
    }
  }
  __syncthreads();
  if (g != 0) return;
  // the groups' sums, each against its own largest lse
  float Mt = kNegInf;
#pragma unroll
  for (int k = 0; k < NG; ++k) Mt = fmaxf(Mt, mred[k]);
  float wt = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (Mt != kNegInf) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float mk = mred[k];
      if (mk == kNegInf) continue;
      const float s = exp2_fast(mk - Mt);
      wt += s * wred[k];
      o += s * *reinterpret_cast<const f32x4*>(&red[k][d0]);
    }
  }
  merge_store<F16>(p, row, d0, o, wt, Mt);
}

// Two partial results over disjoint key sets (natural-log lse):
// out = (e^la oa + e^lb ob) / (e^la + e^lb), lse = ln(e^la + e^lb); a side
// with lse = -inf (no key) drops out.  D/4 threads per row, 4 outputs each.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pa_merge2_kernel(Merge2Params p) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;                     // d = 96: 10 rows, 16 threads idle
  if ((int)threadIdx.x >= RPB * TPR) return;
  constexpr float kLog2e = 1.4426950408889634f;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= (int64_t)p.total_q * p.num_q_heads) return;
  const int64_t tok = row / p.num_q_heads;
  const int hd = (int)(row % p.num_q_heads);
  const int d0 = (threadIdx.x % TPR) * 4;
  const float la = p.la[tok * p.la_st + hd], lb = p.lb[tok * p.lb_st + hd];
  const float M = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f;
  if (M != kNegInf) {
    wa = la == kNegInf ? 0.f : exp2_fast((la - M) * kLog2e);
    wb = lb == kNegInf ? 0.f : exp2_fast((lb - M) * kLog2e);
  }
  const float ws = wa + wb;
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
  const u32x2 xa = *reinterpret_cast<const u32x2*>(p.oa + tok * p.oa_st + (int64_t)hd * p.oa_sh + d0);
  const u32x2 xb = *reinterpret_cast<const u32x2*>(p.ob + tok * p.ob_st + (int64_t)hd * p.ob_sh + d0);
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float fa = Elem<F16>::unpack(xa[e >> 1] >> (16 * (e & 1)));
    const float fb = Elem<F16>::unpack(xb[e >> 1] >> (16 * (e & 1)));
    // a side with no weight is not read into the sum (its value may be anything)
    o[e] = ((wa > 0.f ? wa * fa : 0.f) + (wb > 0.f ? wb * fb : 0.f)) * inv;
  }
  const u32x2 w = {Elem<F16>::pack2(o[0], o[1]), Elem<F16>::pack2(o[2], o[3])};
  *reinterpret_cast<u32x2*>(p.out + tok * p.o_st + (int64_t)hd * p.o_sh + d0) = w;
  if (p.lse && d0 == 0) p.lse[tok * p.l_st + hd] = ws > 0.f ? M + __logf(ws) : kNegInf;
}

template <int D, int G, bool KV8, bool F16>
hipError_t launch_fwd_t(const FwdParams& p, int wide, int64_t nwg, hipStream_t stream) {
  if constexpr (!KV8) {
    if (wide == 2) {
      hipLaunchKernelGGL((pa_fwd_kernel<D, G, 2, KV8, F16>), dim3((unsigned)nwg),
                         dim3(kThreads), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (wide) {
    hipLaunchKernelGGL((pa_fwd_kernel<D, G, 1, KV8, F16>), dim3((unsigned)nwg), dim3(kThreads),
                       0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((pa_fwd_kernel<D, G, 0, KV8, F16>), dim3((unsigned)nwg), dim3(kThreads),
                       0, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool F16>
hipError_t launch_fwd8_t(const FwdParams& p, int64_t nwg, hipStream_t stream) {
  if constexpr (D == 64 || D == 128) {
    hipLaunchKernelGGL((pa_fwd8_kernel<D, G, F16>), dim3((unsigned)nwg), dim3(kWide8Threads), 0,
                       stream, p);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;                       // no eight-wave tiles for this head size
}

template <int D, int G, bool KV8, bool F16>
hipError_t launch_decode_t(const FwdParams& p, int64_t nwg, hipStream_t stream) {
  hipLaunchKernelGGL((pa_decode_kernel<D, G, KV8, F16>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, int G, bool KV8, bool F16>
int decode_blocks_per_cu_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pa_decode_kernel<D, G, KV8, F16>, kThreads,
                                                   0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int D, bool F16>
hipError_t launch_merge_t(const MergeParams& p, bool wide, int64_t rows, hipStream_t stream) {
  if (wide)
    hipLaunchKernelGGL((pa_merge_wide_kernel<D, F16>), dim3((unsigned)rows), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((pa_merge_rows_kernel<D, F16>), dim3((unsigned)((rows + 1024 / D - 1) / (1024 / D))),
                       dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_merge2_t(const Merge2Params& p, int64_t rows, hipStream_t stream) {
  hipLaunchKernelGGL((pa_merge2_kernel<D, F16>), dim3((unsigned)((rows + 1024 / D - 1) / (1024 / D))),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// This file is compiled once per head size (-DPA_TU_HEAD_DIM=64, 96, 128 or
// 256, in parallel); each object defines the launchers of its head size, and
// the D = 64 object also the head-size independent kernels.
#ifndef PA_TU_HEAD_DIM
#error "compile with -DPA_TU_HEAD_DIM=64, 96, 128 or 256"
#endif
#define PA_CAT2(a, b) a##b
#define PA_CAT(a, b) PA_CAT2(a, b)
#define PA_SFX(name) PA_CAT(name, PA_TU_HEAD_DIM)

#define PA_DISPATCH_G(G_, CALL)                                        \
  switch (G_) {                                                        \
    case 1: { constexpr int GG = 1; CALL; }                            \
    case 2: { constexpr int GG = 2; CALL; }                            \
    case 4: { constexpr int GG = 4; CALL; }                            \
    case 8: { constexpr int GG = 8; CALL; }                            \
    case 16: { constexpr int GG = 16; CALL; }                          \
    default: break;                                                    \
  }

// cache format x element type x group -> one specialization of this head size
#define PA_DISPATCH(G_, K8_, F16_, CALL)                                              \
  do {                                                                                \
    constexpr int DD = PA_TU_HEAD_DIM;                                                \
    if (K8_) {                                                                        \
      [[maybe_unused]] constexpr bool KK = true;                                      \
      if (F16_) { constexpr bool FF = true; PA_DISPATCH_G(G_, CALL); }                \
      else { constexpr bool FF = false; PA_DISPATCH_G(G_, CALL); }                    \
    } else {                                                                          \
      [[maybe_unused]] constexpr bool KK = false;                                     \
      if (F16_) { constexpr bool FF = true; PA_DISPATCH_G(G_, CALL); }                \
      else { constexpr bool FF = false; PA_DISPATCH_G(G_, CALL); }                    \
    }                                                                                 \
  } while (0)

hipError_t PA_SFX(launch_decode_d)(const FwdParams& p, int group, bool kv8, bool f16, int64_t nwg,
                                  hipStream_t stream) {
  PA_DISPATCH(group, kv8, f16, return (launch_decode_t<DD, GG, KK, FF>(p, nwg, stream)));
  return hipErrorInvalidValue;
}

hipError_t PA_SFX(launch_fwd8_d)(const FwdParams& p, int group, bool f16, int64_t nwg,
                                hipStream_t stream) {
  PA_DISPATCH(group, false, f16, return (launch_fwd8_t<DD, GG, FF>(p, nwg, stream)));
  return hipErrorInvalidValue;
}

int PA_SFX(decode_blocks_per_cu_d)(int group, bool kv8, bool f16) {
  PA_DISPATCH(group, kv8, f16, return (decode_blocks_per_cu_t<DD, GG, KK, FF>()));
  return 0;
}

hipError_t PA_SFX(launch_fwd_d)(const FwdParams& p, int group, int wide, bool kv8, bool f16,
                               int64_t nwg, hipStream_t stream) {
  PA_DISPATCH(group, kv8, f16, return (launch_fwd_t<DD, GG, KK, FF>(p, wide, nwg, stream)));
  return hipErrorInvalidValue;
}

hipError_t PA_SFX(launch_merge2_d)(const Merge2Params& p, bool f16, hipStream_t stream) {
  const int64_t rows = (int64_t)p.total_q * p.num_q_heads;
  if (rows <= 0) return hipSuccess;
  return f16 ? launch_merge2_t<PA_TU_HEAD_DIM, true>(p, rows, stream)
             : launch_merge2_t<PA_TU_HEAD_DIM, false>(p, rows, stream);
}

hipError_t PA_SFX(launch_merge_d)(const MergeParams& p, bool f16, hipStream_t stream) {
  const int64_t rows = (int64_t)p.total_q * p.num_q_heads;
  if (rows <= 0) return hipSuccess;
  // many parts per row: a work-group per row; otherwise D/4 threads per row,
  // looping over the row's parts.  An even decode split bounds a row's parts
  // loosely (most rows have one or two): there many rows take the loop form.
  const bool wide = p.n_split > 4 && (!p.even || rows <= 4096);
  return f16 ? launch_merge_t<PA_TU_HEAD_DIM, true>(p, wide, rows, stream)
             : launch_merge_t<PA_TU_HEAD_DIM, false>(p, wide, rows, stream);
}

#if PA_TU_HEAD_DIM == 64
hipError_t launch_rank(const FwdParams& p, hipStream_t stream) {
  const size_t lds = (size_t)(3 * p.num_seqs + 1 + 65 + 65 + 8) * sizeof(int);
  hipLaunchKernelGGL(pa_rank_kernel, dim3(1), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}
#endif

}  // namespace pa
