// gfx950 (CDNA4) kernels of libpa: the unified paged-attention forward kernel
// and the log-sum-exp merge of key-split partial results.
//
// Operation: softmax(scale * q k^T + mask) v for a varlen batch whose sequences
// have arbitrary query lengths (decode, chunked prefill, prefill in one grid),
// keys and values read from a paged cache [num_blocks, 16, Hkv, d] through a
// block table (page "[Kernel] Unified Triton kernel that doesn't distinguish
// between prefill + decode", PR description; the causal mask is end-aligned so
// decode queries and prefill chunks share one kernel, page "[Kernel] [V1]
// Improved performance for V1 Triton (ROCm) backend", section "How is this
// performance improvement achieved?").
//
// Work decomposition.  One work-group (4 wave64s) owns one item
// (query tile, kv-head, key split).  The q-heads of one kv-head (the GQA group,
// G of them) are packed with the tile's tokens into the rows of the MFMA tiles
// (row r <-> token r / G, head r % G), so one K/V read serves G heads (the
// "GQA packing along the query dimension" of the unified-kernel page).
//
//  * Narrow tiles (at most 16 packed rows: decode, short chunks) keep all rows
//    in one 16-column MFMA tile in every wave; the four waves take different
//    16-key blocks of each 64-key stage and merge their softmax states through
//    LDS at the end.  This keeps four waves streaming one item's cache blocks.
//  * Wide tiles (17..64 rows) give each wave its own 16 rows; all four waves
//    sweep the same 64-key stages.
//
// Per stage, the 16-byte chunks of 4 cache blocks of K and V are loaded
// row-contiguously from HBM (a wave reads whole 256-byte key rows), held in
// registers while the previous stage is computed, and written to the other of
// two LDS buffers.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16 so each lane holds one row's scores and the softmax
// row reductions stay within a lane plus two cross-lane steps.  P^T (bf16)
// feeds O^T += V^T P^T directly from the score accumulators; V^T operands come
// from the gfx950 LDS transpose read (ds_read_b64_tr_b16) of row-major V.
// Softmax runs online in fp32 in the log2 domain (scale folded into log2 e).
//
// Key splits: with n_split > 1 each item covers keys [sigma*split, (sigma+1)
// *split) and writes its normalised fp32 output and log2-domain lse to the
// workspace; pa_merge combines them.  Split boundaries depend on lengths only,
// so results are deterministic.
//
// Address math for the cache is 64-bit (physical block * block stride), since
// one cache tensor can exceed 2^31 elements (the int64 cast discussed in the
// review of page "[ROCM][KERNEL] Paged attention for V1").

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PA_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 pair, packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
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
  static __device__ __forceinline__ int k_chunk(int key, int dc) { return dc * 16 + (key ^ dc); }
  static __device__ __forceinline__ int v_swz(int key) {
    return D == 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
  }
  static __device__ __forceinline__ int v_chunk(int key, int c) { return key * CPR + (c ^ v_swz(key)); }
};

// One work item: (query tile, kv-head, key split) and the key range it covers.
struct Item {
  int s, kvh, sigma;
  int q0, q_len, tok0, n_tok, rows;
  int L, diag;        // context length; causal: token t sees keys < diag + t + 1
  int kbeg, kend;     // keys [kbeg, kend) of this split that some row may need
  int kmin;           // smallest per-row key limit within the tile
};

template <int G>
__device__ __forceinline__ bool decode_item(const FwdParams& p, Item& it) {
  // Work-groups are dispatched round-robin over the 8 XCDs (XCD = id % 8);
  // give each XCD a contiguous range of items so items that share data
  // (the q-tiles of one kv-head's context, or the kv-heads of one sequence's
  // blocks) run close in time on the same L2.
  const int item = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);
  if (item >= p.num_items) return false;
  it.sigma = item % p.n_split;
  const int rest = item / p.n_split;
  int slot;
  if (p.kv_major) {
    slot = rest % p.num_slots;
    it.kvh = rest / p.num_slots;
  } else {
    it.kvh = rest % p.num_kv_heads;
    slot = rest / p.num_kv_heads;
  }
  int tile;
  if (p.slots_direct) {
    it.s = slot;
    tile = 0;
  } else {
    // sequence s owns slots [cu[s]/Tq + s, cu[s+1]/Tq + s + 1)
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_q[mid] / p.tile_tokens + mid <= slot) lo = mid; else hi = mid - 1;
    }
    it.s = lo;
    tile = slot - (p.cu_q[lo] / p.tile_tokens + lo);
  }
  it.q0 = p.cu_q[it.s];
  it.q_len = p.cu_q[it.s + 1] - it.q0;
  it.tok0 = tile * p.tile_tokens;
  if (it.tok0 >= it.q_len) return false;            // empty slot (whole work-group)
  it.n_tok = min(p.tile_tokens, it.q_len - it.tok0);
  it.rows = it.n_tok * G;
  it.L = p.seq_k[it.s];
  it.diag = it.L - it.q_len;
  const int k_need = p.causal ? min(it.L, it.diag + it.tok0 + it.n_tok) : it.L;
  it.kbeg = it.sigma * p.split_keys;
  it.kend = min(k_need, it.kbeg + p.split_keys);
  it.kmin = p.causal ? min(it.kend, it.diag + it.tok0 + 1) : it.kend;
  return true;
}

// Q^T operand (B of S^T = K Q^T) for packed row `row` of the tile: lane group
// h4 holds d = 32 ks + 8 h4 .. +7 for each contraction step ks.
template <int D, int G>
__device__ __forceinline__ void load_q(const FwdParams& p, const Item& it, int row, int h4,
                                       bf16x8 (&qB)[D / 32]) {
  const bool ok = row < it.rows;
  const int t_in = row / G;
  const int head = it.kvh * G + row % G;
  const uint16_t* qp = p.q + (int64_t)(it.q0 + it.tok0 + (ok ? t_in : 0)) * p.q_st +
                       (int64_t)head * p.q_sh + 8 * h4;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
    qB[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Shared-memory budgets.
template <int D>
struct NarrowCfg {
  static constexpr int BLK_BYTES = kBlockSize * D * 2;
  static constexpr int VBUF_BYTES = 4 * 2 * BLK_BYTES;            // 2 V buffers per wave
  static constexpr int RED_STRIDE = D + 4;                        // floats per merged row
  static constexpr int RED_BYTES = (2 * 64 + 4 * 16 * RED_STRIDE) * 4;
  static constexpr int SMEM = VBUF_BYTES > RED_BYTES ? VBUF_BYTES : RED_BYTES;
};
template <int D>
struct WideCfg {
  static constexpr int BLK_BYTES = kBlockSize * D * 2;
  static constexpr int NBS = kStageKeys / kBlockSize;
  static constexpr int HALF_BYTES = NBS * BLK_BYTES;
  static constexpr int STAGE_BYTES = 2 * HALF_BYTES;
  static constexpr int IDS_OFFSET = 2 * STAGE_BYTES;
  static constexpr int SMEM_RAW = IDS_OFFSET + (kMaxSplitKeys / kBlockSize) * 4;
  static constexpr int SMEM = SMEM_RAW > NarrowCfg<D>::SMEM ? SMEM_RAW : NarrowCfg<D>::SMEM;
};

// ---------------------------------------------------------------------------
// Narrow tiles (<= 16 packed rows: decode steps, short chunks).
//
// All 16 columns of one MFMA tile hold the tile's rows in every wave; wave w
// owns the item's cache blocks w, w+4, w+8, ... and streams them on its own,
// with no work-group barrier until the final merge.  Each wave keeps a ring of
// P blocks in flight in registers: K lands directly in the A-operand layout of
// S^T = K Q^T (lane: key l16, d-chunk h4 + 4 ks), V in natural row order and
// goes through a wave-private LDS buffer for the transpose read.  The block
// ids of the wave's (at most 64) blocks are fetched once into one VGPR and
// read per block with readlane, so no KV load waits on a block-table load.
// ---------------------------------------------------------------------------
template <int D, int G, int P>
__device__ __forceinline__ void attend_narrow(const FwdParams& p, const Item& it,
                                              unsigned char* smem) {
  using Lay = Layout<D>;
  using Cfg = NarrowCfg<D>;
  constexpr int CPR = Lay::CPR;
  constexpr int BLK_BYTES = Lay::BLK_BYTES;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int VPL = kBlockSize * CPR / 64;      // V chunks per lane per block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h4 = lane >> 4;
  const int l16 = lane & 15;

  bf16x8 qB[KS];
  load_q<D, G>(p, it, l16, h4, qB);
  const int t_in = l16 / G;
  const int klim = p.causal ? min(it.kend, it.diag + it.tok0 + t_in + 1) : it.kend;

  const int blk0 = it.kbeg / kBlockSize;
  const int nblk = it.kend > it.kbeg ? (it.kend + kBlockSize - 1) / kBlockSize - blk0 : 0;
  const int nb = nblk > wave ? (nblk - wave + 3) / 4 : 0;     // <= 64: split_keys <= 4096
  const int32_t* btrow = p.bt + (int64_t)it.s * p.bt_stride;
  int ids = 0;
  if (lane < nb) ids = btrow[blk0 + wave + 4 * lane];

  const int slot_stride = p.num_kv_heads * D;
  const uint16_t* kbase = p.k + it.kvh * D;
  const uint16_t* vbase = p.v + it.kvh * D;
  const int koff = l16 * slot_stride + 8 * h4;
  int voff[VPL], vlds[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const int c = lane + 64 * u;
    const int key = c / CPR, dc = c % CPR;
    voff[u] = key * slot_stride + dc * 8;
    vlds[u] = Lay::v_chunk(key, dc) * 16;
  }

  u32x4 kst[P][KS];
  u32x4 vst[P][VPL];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    if (j < nb) {
      const int64_t boff = (int64_t)__builtin_amdgcn_readlane(ids, j) * p.kv_sb;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kst[j][ks] = *reinterpret_cast<const u32x4*>(kbase + boff + koff + 32 * ks);
#pragma unroll
      for (int u = 0; u < VPL; ++u)
        vst[j][u] = *reinterpret_cast<const u32x4*>(vbase + boff + voff[u]);
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
        const int kb = (blk0 + wave + 4 * i) * kBlockSize;
        unsigned char* vbuf = vbuf0 + (i & 1) * BLK_BYTES;
#pragma unroll
        for (int u = 0; u < VPL; ++u) *reinterpret_cast<u32x4*>(vbuf + vlds[u]) = vst[j][u];
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kst[j][ks]),
                                                       qB[ks], sc, 0, 0, 0);
        // refill this ring slot with block i + P
        if (i + P < nb) {
          const int64_t boff = (int64_t)__builtin_amdgcn_readlane(ids, i + P) * p.kv_sb;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kst[j][ks] = *reinterpret_cast<const u32x4*>(kbase + boff + koff + 32 * ks);
#pragma unroll
          for (int u = 0; u < VPL; ++u)
            vst[j][u] = *reinterpret_cast<const u32x4*>(vbase + boff + voff[u]);
        }
        const bool need_mask = kb + kBlockSize > it.kmin;
        float x[4];
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = sc[r] * p.scale_log2;
          if (need_mask && kb + 4 * h4 + r >= klim) x[r] = kNegInf;
          mx = fmaxf(mx, x[r]);
        }
        mx = max_across_groups(mx);
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2_fast(m - m_use);
        float pr[4], rs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = exp2_fast(x[r] - m_use);
          rs += pr[r];
        }
        l = l * alpha + rs;
        m = m_new;
        u32x2 pk = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
        const i16x4 pB = __builtin_bit_cast(i16x4, pk);
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
          acc[dt] *= alpha;
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pB, acc[dt], 0, 0, 0);
        }
      }
    }
  }

  // merge the four waves' states of the same 16 rows
  l = sum_across_groups(l);
  __syncthreads();                        // every wave is done with its V buffers
  float* red_m = reinterpret_cast<float*>(smem);
  float* red_l = red_m + 64;
  float* red_o = red_m + 128;             // [wave][row][RED_STRIDE]
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
  float mw[4], M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = red_m[w * 16 + n];
    M = fmaxf(M, mw[w]);
  }
  const float M_use = M == kNegInf ? 0.f : M;
  float wt[4], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = exp2_fast(mw[w] - M_use);
    Ls += wt[w] * red_l[w * 16 + n];
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  float o[DPER];
#pragma unroll
  for (int e = 0; e < DPER; e += 4) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w)
      a += wt[w] * *reinterpret_cast<const f32x4*>(red_o + (w * 16 + n) * RS + d0 + e);
#pragma unroll
    for (int k = 0; k < 4; ++k) o[e + k] = a[k] * inv;
  }
  const int64_t tok = it.q0 + it.tok0 + n / G;
  const int hn = it.kvh * G + n % G;
  if (p.n_split == 1) {
    uint16_t* op = p.out + tok * p.o_st + (int64_t)hn * p.o_sh + d0;
    if constexpr (DPER == 8) {
      u32x4 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                 pack_bf16x2(o[6], o[7])};
      *reinterpret_cast<u32x4*>(op) = w;
    } else {
      u32x2 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(op) = w;
    }
  } else {
    const int64_t r = ((int64_t)it.sigma * p.total_q + tok) * p.num_q_heads + hn;
    float* wp = p.ws_o + r * D + d0;
#pragma unroll
    for (int e = 0; e < DPER; e += 4)
      *reinterpret_cast<f32x4*>(wp + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
    if ((tid & 15) == 0) p.ws_lse[r] = Ls > 0.f ? M + __log2f(Ls) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Wide tiles (17..64 packed rows: prefill and longer chunks).
//
// Each wave owns 16 rows; the four waves sweep the same 64-key stages.  A
// stage's 4 cache blocks of K and V are loaded row-contiguously into
// registers while the previous stage is computed, then written into the other
// of two LDS buffers (one barrier per stage).
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ __forceinline__ void attend_wide(const FwdParams& p, const Item& it,
                                            unsigned char* smem) {
  using Lay = Layout<D>;
  using Cfg = WideCfg<D>;
  constexpr int CPR = Lay::CPR;
  constexpr int BLK_BYTES = Lay::BLK_BYTES;
  constexpr int NBS = Cfg::NBS;
  constexpr int HALF_BYTES = Cfg::HALF_BYTES;
  constexpr int STAGE_BYTES = Cfg::STAGE_BYTES;
  constexpr int CPT = NBS * kBlockSize * CPR / kThreads; // chunks per thread per tensor
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  static_assert(CPT * kThreads == NBS * kBlockSize * CPR, "stage must split evenly");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h4 = lane >> 4;
  const int l16 = lane & 15;

  const int row = wave * 16 + l16;
  bf16x8 qB[KS];
  load_q<D, G>(p, it, row, h4, qB);
  const int t_in = row / G;
  const int head = it.kvh * G + row % G;
  const bool row_ok = row < it.rows;
  const int klim = p.causal ? min(it.kend, it.diag + it.tok0 + t_in + 1) : it.kend;
  const int kbeg = it.kbeg, kend = it.kend, kmin = it.kmin;

  const int nblk = (kend + kBlockSize - 1) / kBlockSize;
  const int blk0 = kbeg / kBlockSize;
  const int n_stage = kend > kbeg ? (kend - kbeg + kStageKeys - 1) / kStageKeys : 0;
  const int32_t* btrow = p.bt + (int64_t)it.s * p.bt_stride;
  const int64_t slot_stride = (int64_t)p.num_kv_heads * D;
  const uint16_t* kbase = p.k + (int64_t)it.kvh * D;
  const uint16_t* vbase = p.v + (int64_t)it.kvh * D;

  // the item's block ids (at most kMaxSplitKeys / 16) staged once in LDS
  int32_t* ids = reinterpret_cast<int32_t*>(smem + Cfg::IDS_OFFSET);
  if (tid < nblk - blk0) ids[tid] = btrow[blk0 + tid];
  __syncthreads();

  u32x4 kreg[CPT], vreg[CPT];
  auto load_stage = [&](int st) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + kThreads * u;
      const int blk = c / (kBlockSize * CPR);
      const int r = c % (kBlockSize * CPR);
      const int key = r / CPR, dc = r % CPR;
      const int jb = blk0 + st * NBS + blk;
      if (jb < nblk) {
        const int64_t off = (int64_t)ids[jb - blk0] * p.kv_sb + key * slot_stride + dc * 8;
        kreg[u] = *reinterpret_cast<const u32x4*>(kbase + off);
        vreg[u] = *reinterpret_cast<const u32x4*>(vbase + off);
      }
    }
  };
  auto store_stage = [&](int st, int buf) {
    unsigned char* kb = smem + buf * STAGE_BYTES;
    unsigned char* vb = kb + HALF_BYTES;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + kThreads * u;
      const int blk = c / (kBlockSize * CPR);
      const int r = c % (kBlockSize * CPR);
      const int key = r / CPR, dc = r % CPR;
      const int jb = blk0 + st * NBS + blk;
      if (jb < nblk) {
        *reinterpret_cast<u32x4*>(kb + blk * BLK_BYTES + Lay::k_chunk(key, dc) * 16) = kreg[u];
        *reinterpret_cast<u32x4*>(vb + blk * BLK_BYTES + Lay::v_chunk(key, dc) * 16) = vreg[u];
      }
    }
  };

  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;
  float l = 0.f;
  const int tr_key = 4 * h4 + (l16 >> 2);
  const int tr_c_lo = (l16 & 3) >> 1;
  const int tr_half = (l16 & 1) * 8;
  auto vt_read = [&](const unsigned char* vblk, int dt) -> i16x4 {
    const unsigned char* a = vblk + Lay::v_chunk(tr_key, 2 * dt + tr_c_lo) * 16 + tr_half;
    return __builtin_bit_cast(i16x4,
                              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PA_LDS bf16x4*)(a)));
  };
  auto vt_mask = [&](i16x4 v, int key_first) -> i16x4 {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key_first + e >= kend) v[e] = 0;
    return v;
  };

  if (n_stage > 0) {
    load_stage(0);
    store_stage(0, 0);
  }
  __syncthreads();

  for (int st = 0; st < n_stage; ++st) {
    const int buf = st & 1;
    if (st + 1 < n_stage) load_stage(st + 1);
    const unsigned char* Kb = smem + buf * STAGE_BYTES;
    const unsigned char* Vb = Kb + HALF_BYTES;
    const int kst = kbeg + st * kStageKeys;
    if (wave * 16 < it.rows) {
      f32x4 sc[NBS];
#pragma unroll
      for (int b = 0; b < NBS; ++b) {
        sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* kblk = Kb + b * BLK_BYTES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kblk + Lay::k_chunk(l16, 4 * ks + h4) * 16);
          sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[ks], sc[b], 0, 0, 0);
        }
      }
      const bool need_mask = kst + kStageKeys > kmin;
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < NBS; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sc[b][r] * p.scale_log2;
          if (need_mask && kst + 16 * b + 4 * h4 + r >= klim) x = kNegInf;
          sc[b][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_across_groups(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int b = 0; b < NBS; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = exp2_fast(sc[b][r] - m_use);
          sc[b][r] = pr;
          rs += pr;
        }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      const bool vmask = kst + kStageKeys > kend;
#pragma unroll
      for (int half = 0; half < NBS / 2; ++half) {
        const int b0 = 2 * half;
        u32x4 pk = {pack_bf16x2(sc[b0][0], sc[b0][1]), pack_bf16x2(sc[b0][2], sc[b0][3]),
                    pack_bf16x2(sc[b0 + 1][0], sc[b0 + 1][1]),
                    pack_bf16x2(sc[b0 + 1][2], sc[b0 + 1][3])};
        const bf16x8 pB = __builtin_bit_cast(bf16x8, pk);
        const unsigned char* vlo = Vb + b0 * BLK_BYTES;
        const unsigned char* vhi = vlo + BLK_BYTES;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          i16x4 a0 = vt_read(vlo, dt);
          i16x4 a1 = vt_read(vhi, dt);
          if (vmask) {
            a0 = vt_mask(a0, kst + 16 * b0 + 4 * h4);
            a1 = vt_mask(a1, kst + 16 * (b0 + 1) + 4 * h4);
          }
          u32x4 packed = {__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                          __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]};
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, packed), pB,
                                                           acc[dt], 0, 0, 0);
        }
      }
    }
    if (st + 1 < n_stage) store_stage(st + 1, buf ^ 1);
    __syncthreads();
  }

  l = sum_across_groups(l);
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t tok = it.q0 + it.tok0 + t_in;
  if (p.n_split == 1) {
    uint16_t* op = p.out + tok * p.o_st + (int64_t)head * p.o_sh + 4 * h4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 w = {pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                 pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(op + 16 * dt) = w;
    }
  } else {
    const int64_t r = ((int64_t)it.sigma * p.total_q + tok) * p.num_q_heads + head;
    float* wp = p.ws_o + r * D + 4 * h4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(wp + 16 * dt) = acc[dt] * inv;
    if (h4 == 0) p.ws_lse[r] = l > 0.f ? m + __log2f(l) : kNegInf;
  }
}

constexpr int kRing = 2;   // cache blocks in flight per wave on the narrow path

// WIDE = false: every tile of the batch is narrow (the plan guarantees it).
template <int D, int G, bool WIDE>
__global__ __launch_bounds__(kThreads) void pa_fwd_kernel(FwdParams p) {
  constexpr int SMEM = WIDE ? WideCfg<D>::SMEM : NarrowCfg<D>::SMEM;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  Item it;
  if (!decode_item<G>(p, it)) return;
  if (it.rows <= p.narrow_rows) {
    attend_narrow<D, G, kRing>(p, it, smem);
  } else {
    if constexpr (WIDE) attend_wide<D, G>(p, it, smem);
  }
}

// Log-sum-exp merge of key-split partials (all lse in the log2 domain):
// w_sigma = 2^(lse_sigma - max lse), out = sum w O_sigma / sum w.  Parts with no
// key carry lse = -inf and are skipped (their O is never read).
template <int D>
__global__ __launch_bounds__(256) void pa_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;                 // threads per (token, head) row
  constexpr int RPB = 256 / TPR;             // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int64_t nrows = (int64_t)p.total_q * p.num_q_heads;
  if (row >= nrows) return;
  const int d0 = (threadIdx.x % TPR) * 4;
  float M = kNegInf;
  for (int sg = 0; sg < p.n_split; ++sg) M = fmaxf(M, p.ws_lse[sg * nrows + row]);
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
  if (M != kNegInf) {
    for (int sg = 0; sg < p.n_split; ++sg) {
      const float ls = p.ws_lse[sg * nrows + row];
      if (ls == kNegInf) continue;
      const float w = exp2_fast(ls - M);
      ws += w;
      a += w * *reinterpret_cast<const f32x4*>(p.ws_o + (sg * nrows + row) * D + d0);
    }
  }
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
  const int64_t tok = row / p.num_q_heads;
  const int hd = (int)(row % p.num_q_heads);
  uint16_t* op = p.out + tok * p.o_st + (int64_t)hd * p.o_sh + d0;
  u32x2 w = {pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
  *reinterpret_cast<u32x2*>(op) = w;
}

template <int D, int G>
hipError_t launch_fwd_t(const FwdParams& p, bool wide, int64_t nwg, hipStream_t stream) {
  if (wide)
    hipLaunchKernelGGL((pa_fwd_kernel<D, G, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((pa_fwd_kernel<D, G, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, int group, bool wide, int64_t nwg, hipStream_t stream) {
  switch (group) {
    case 1: return launch_fwd_t<D, 1>(p, wide, nwg, stream);
    case 2: return launch_fwd_t<D, 2>(p, wide, nwg, stream);
    case 4: return launch_fwd_t<D, 4>(p, wide, nwg, stream);
    case 8: return launch_fwd_t<D, 8>(p, wide, nwg, stream);
    case 16: return launch_fwd_t<D, 16>(p, wide, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fwd_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

hipError_t launch_fwd(const FwdParams& p, int head_dim, int group, bool wide, int64_t nwg,
                      hipStream_t stream) {
  if (head_dim == 128) return launch_fwd_d<128>(p, group, wide, nwg, stream);
  if (head_dim == 64) return launch_fwd_d<64>(p, group, wide, nwg, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.total_q * p.num_q_heads;
  if (head_dim == 128) {
    const int64_t nb = (rows + 7) / 8;
    hipLaunchKernelGGL(pa_merge_kernel<128>, dim3((unsigned)nb), dim3(256), 0, stream, p);
  } else if (head_dim == 64) {
    const int64_t nb = (rows + 15) / 16;
    hipLaunchKernelGGL(pa_merge_kernel<64>, dim3((unsigned)nb), dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
