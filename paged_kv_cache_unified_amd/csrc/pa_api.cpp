// Host side of libpa: descriptor validation, the launch-shape heuristic,
// workspace management and kernel launches.  The C ABI is declared in
// include/pa.h.  Validation and planning read descriptors only (never device
// memory) so they run, and are tested, on machines without a GPU.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

struct Shapes {
  int64_t T, Hq, D, NB, B, Hkv, S, MB, G;
  int64_t q_st, q_sh, o_st, o_sh, kv_sb, bt_stride;
  bool kv8;          // caches hold fp8 E4M3 codes (else 16-bit elements)
  bool f16;          // q, out and 16-bit caches are fp16 (else bf16)
};

struct Plan {
  int32_t tile_tokens, tile_rows, num_slots, slots_direct, n_split, split_keys;
  bool wide;        // launch the specialization with the wide-tile path
  bool eight;       // wide plan on the eight-wave kernel (256-row tiles)
  bool lpt;         // grid plan with longest-first unit order
  bool unit_xcd;    // lpt: a unit's kv-heads on one XCD (units share no K/V)
  bool persistent;  // persistent decode kernel with per-sequence split counts
  bool balanced;    // persistent: even split of the block stream, chunks sized on the device
  int64_t num_items;
  int64_t nwg;
  size_t ws_bytes;
  size_t ws_lse_offset;
  size_t ws_parts_offset;   // row part counts [T * Hq] int32
  size_t ws_base_offset;    // even split: part-0 partial row of each row [T * Hq] int32
  int64_t partial_rows;     // rows of the partial-output region (0: no split)
  size_t ws_lpt_offset;     // longest-first unit order [lpt_units] int4
  int64_t lpt_units;
};

constexpr int64_t kMaxInt32 = 0x7fffffff;

int64_t extent_elems(const pa_tensor* t) {
  int64_t e = 1;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] == 0) return 0;
    e += (t->shape[i] - 1) * t->stride[i];
  }
  return e;
}

bool overlaps(const pa_tensor* a, int64_t a_elem_bytes, const pa_tensor* b, int64_t b_elem_bytes) {
  const int64_t ea = extent_elems(a), eb = extent_elems(b);
  if (ea == 0 || eb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a->data);
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b->data);
  const uintptr_t a1 = a0 + static_cast<uintptr_t>(ea * a_elem_bytes);
  const uintptr_t b1 = b0 + static_cast<uintptr_t>(eb * b_elem_bytes);
  return a0 < b1 && b0 < a1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* out,
             const pa_tensor* cu, const pa_tensor* sk, const pa_tensor* bt, int32_t max_q,
             int32_t max_k, Shapes* sh) {
  if (!q || !k || !v || !out || !cu || !sk || !bt)
    return fail(PA_ERR_NULL, "a tensor descriptor pointer is NULL");
  struct {
    const pa_tensor* t;
    const char* name;
    int dtype;
    int ndim;
  } spec[] = {{q, "q", PA_BF16, 3},          {k, "k_cache", PA_BF16, 4},
              {v, "v_cache", PA_BF16, 4},    {out, "out", PA_BF16, 3},
              {cu, "cu_seqlens_q", PA_INT32, 1}, {sk, "seqused_k", PA_INT32, 1},
              {bt, "block_table", PA_INT32, 2}};
  // q and out: bf16 or fp16; caches: the same 16-bit type, or fp8 E4M3 codes
  // (both caches the same)
  const bool f16 = q->dtype == PA_F16;
  if (f16) spec[0].dtype = spec[1].dtype = spec[2].dtype = spec[3].dtype = PA_F16;
  const bool kv8 = k->dtype == PA_FP8_E4M3;
  if (kv8) spec[1].dtype = spec[2].dtype = PA_FP8_E4M3;
  for (auto& e : spec) {
    if (e.t->dtype != e.dtype)
      return fail(PA_ERR_DTYPE, "%s: dtype code %d, expected %d", e.name, e.t->dtype, e.dtype);
    if (e.t->ndim != e.ndim)
      return fail(PA_ERR_SHAPE, "%s: ndim %d, expected %d", e.name, e.t->ndim, e.ndim);
    for (int i = 0; i < e.ndim; ++i)
      if (e.t->shape[i] < 0 || e.t->stride[i] < 0)
        return fail(PA_ERR_SHAPE, "%s: negative extent or stride in dim %d", e.name, i);
  }
  Shapes s{};
  s.kv8 = kv8;
  s.f16 = f16;
  const int64_t kv_esz = kv8 ? 1 : 2;
  s.T = q->shape[0];
  s.Hq = q->shape[1];
  s.D = q->shape[2];
  s.NB = k->shape[0];
  s.B = k->shape[1];
  s.Hkv = k->shape[2];
  s.S = sk->shape[0];
  s.MB = bt->shape[1];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i])
      return fail(PA_ERR_SHAPE, "out shape differs from q in dim %d", i);
  for (int i = 0; i < 4; ++i)
    if (v->shape[i] != k->shape[i] || v->stride[i] != k->stride[i])
      return fail(PA_ERR_SHAPE, "v_cache shape/strides differ from k_cache in dim %d", i);
  if (k->shape[3] != s.D) return fail(PA_ERR_SHAPE, "cache head_dim %lld != q head_dim %lld",
                                      (long long)k->shape[3], (long long)s.D);
  if (cu->shape[0] != s.S + 1)
    return fail(PA_ERR_SHAPE, "cu_seqlens_q has %lld entries, expected num_seqs+1 = %lld",
                (long long)cu->shape[0], (long long)(s.S + 1));
  if (bt->shape[0] != s.S)
    return fail(PA_ERR_SHAPE, "block_table has %lld rows, expected %lld",
                (long long)bt->shape[0], (long long)s.S);
  if (s.Hq == 0 || s.Hkv == 0 || s.Hq % s.Hkv)
    return fail(PA_ERR_SHAPE, "num_q_heads %lld must be a positive multiple of num_kv_heads %lld",
                (long long)s.Hq, (long long)s.Hkv);
  if (s.S == 0 && s.T != 0) return fail(PA_ERR_SHAPE, "total_q > 0 with no sequences");
  if (max_q < 0 || max_k < 0) return fail(PA_ERR_SHAPE, "negative max_seqlen");
  s.G = s.Hq / s.Hkv;
  if (s.D != 64 && s.D != 96 && s.D != 128 && s.D != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %lld (supported: 64, 96, 128, 256)", (long long)s.D);
  if (s.B != 16 && s.B != 32 && s.B != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %lld (supported: 16, 32, 64)", (long long)s.B);
  // the kernels address 16-key sub-blocks: physical block * (B / 16) + part
  if (s.NB * (s.B / pa::kBlockSize) > kMaxInt32)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size / 16 beyond the 32-bit range");
  if (!pa::fwd_supported((int)s.D, (int)s.G))
    return fail(PA_ERR_UNSUPPORTED, "GQA group %lld (supported: 1, 2, 4, 8, 16)", (long long)s.G);
  if (s.S > 0 && (int64_t)max_k > s.MB * s.B)
    return fail(PA_ERR_SHAPE, "max_seqlen_k %d exceeds block_table capacity %lld", max_k,
                (long long)(s.MB * s.B));
  if (s.T > kMaxInt32 / 2 || s.S > kMaxInt32 / 2 || s.NB > kMaxInt32 || s.Hq > 4096)
    return fail(PA_ERR_UNSUPPORTED, "sizes beyond the 32-bit index range");
  // strides
  if (q->stride[2] != 1 || out->stride[2] != 1)
    return fail(PA_ERR_UNSUPPORTED, "q/out need a unit stride along head_dim");
  if (k->stride[3] != 1 || k->stride[2] != s.D || k->stride[1] != s.Hkv * s.D)
    return fail(PA_ERR_UNSUPPORTED, "caches need contiguous [block_size, num_kv_heads, head_dim]");
  if (s.NB > 1 && k->stride[0] < s.B * s.Hkv * s.D)
    return fail(PA_ERR_SHAPE, "cache block stride smaller than one block");
  if ((q->stride[0] | q->stride[1] | out->stride[0] | out->stride[1]) % 8)
    return fail(PA_ERR_ALIGN, "q/out strides must be multiples of 8 elements");
  if ((k->stride[0] * kv_esz) % 16)
    return fail(PA_ERR_ALIGN, "cache block stride must be a multiple of 16 bytes");
  if (s.B * s.Hkv * s.D * kv_esz > kMaxInt32)
    return fail(PA_ERR_UNSUPPORTED, "one cache block exceeds 2^31 bytes");
  if (cu->stride[0] != 1 && cu->shape[0] > 1) return fail(PA_ERR_UNSUPPORTED, "cu_seqlens_q not contiguous");
  if (sk->stride[0] != 1 && s.S > 1) return fail(PA_ERR_UNSUPPORTED, "seqused_k not contiguous");
  if (bt->stride[1] != 1 && s.MB > 1) return fail(PA_ERR_UNSUPPORTED, "block_table rows not contiguous");
  if (s.S > 1 && bt->stride[0] < s.MB) return fail(PA_ERR_SHAPE, "block_table row stride < width");
  if (bt->stride[0] > kMaxInt32) return fail(PA_ERR_UNSUPPORTED, "block_table row stride too large");
  // pointers
  if (s.T > 0 && (!q->data || !out->data)) return fail(PA_ERR_NULL, "q/out data is NULL");
  if (!cu->data) return fail(PA_ERR_NULL, "cu_seqlens_q data is NULL");
  if (s.S > 0 && (!sk->data || !bt->data)) return fail(PA_ERR_NULL, "seqused_k/block_table data is NULL");
  if (s.S > 0 && s.NB > 0 && (!k->data || !v->data)) return fail(PA_ERR_NULL, "cache data is NULL");
  if (!aligned(q->data, 16) || !aligned(out->data, 16) || !aligned(k->data, 16) ||
      !aligned(v->data, 16))
    return fail(PA_ERR_ALIGN, "q/out/cache data must be 16-byte aligned");
  if (!aligned(cu->data, 4) || !aligned(sk->data, 4) || !aligned(bt->data, 4))
    return fail(PA_ERR_ALIGN, "int32 metadata must be 4-byte aligned");
  if (overlaps(out, 2, q, 2) || overlaps(out, 2, k, kv_esz) || overlaps(out, 2, v, kv_esz))
    return fail(PA_ERR_ALIAS, "out overlaps q, k_cache or v_cache");
  s.q_st = q->stride[0];
  s.q_sh = q->stride[1];
  s.o_st = out->stride[0];
  s.o_sh = out->stride[1];
  s.kv_sb = k->stride[0];
  s.bt_stride = s.MB > 0 ? bt->stride[0] : 0;
  *sh = s;
  return PA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Launch shape from shapes only (no device reads, no autotuning):
//  * a batch whose every sequence fits one narrow tile (max_seqlen_q * G <= 16:
//    pure decode, or short chunks) gets one tile per sequence;
//  * otherwise query tiles of 128 packed rows (128/G tokens); sequences are
//    mapped to tile slots by the bound floor(cu[s]/Tq) + s, so the grid is
//    known without reading cu_seqlens_q; tiles of <= 16 rows inside such a
//    batch (its decode sequences) still run the narrow code path;
//  * keys are split only when the items cannot fill the GPU: enough splits to
//    reach ~4 work-groups per CU, each split at least 512 keys and at most
//    kMaxSplitKeys.  A sequence has ceil(L_s / split) parts, so rows of short
//    sequences are never split.  Split sizes depend on max_seqlen_k and the
//    grid only, so results are deterministic.
int make_plan(const Shapes& s, int32_t max_q, int32_t max_k, const pa_options* opt, int num_cus,
              int decode_blocks_per_cu, Plan* out) {
  Plan p{};
  const int force_tile = opt ? opt->force_tile : 0;
  const int force_split = opt ? opt->force_num_splits : 0;
  const int64_t G = s.G;
  const int64_t mq = std::max<int64_t>(max_q, 1);
  const int64_t mk = std::max<int64_t>(max_k, 1);
  const bool narrow_fits = mq * G <= pa::kNarrowRows;
  if ((force_tile == 1 || force_tile == 3) && !narrow_fits)
    return fail(PA_ERR_UNSUPPORTED, "force_tile=%d needs max_seqlen_q * G <= 16", force_tile);
  if (force_tile < 0 || force_tile > 4)
    return fail(PA_ERR_UNSUPPORTED, "force_tile must be 0, 1, 2, 3 or 4");
  // eight-wave tiles exist for d = 64 and 128 over 16-bit caches
  if (force_tile == 4 && !(s.D == 64 || s.D == 128))
    return fail(PA_ERR_UNSUPPORTED, "force_tile=4 (eight-wave tiles) needs head_dim 64 or 128");
  if (force_tile == 4 && s.kv8)
    return fail(PA_ERR_UNSUPPORTED, "force_tile=4 (eight-wave tiles) needs 16-bit caches");
  const bool narrow = force_tile == 1 || force_tile == 3 || (force_tile == 0 && narrow_fits);
  // (the decode kernel's idle ring slots re-read pool block 0, so the pool
  // must hold at least one block)
  if (narrow && force_tile != 3 && s.S <= pa::kMaxDecodeSeqs && s.NB > 0) {
    // Persistent decode kernel: one narrow tile per sequence; items are the
    // (sequence, key split, kv-head) triples enumerated on the device.
    p.persistent = true;
    p.wide = false;
    p.tile_tokens = (int32_t)mq;
    p.tile_rows = (int32_t)(mq * G);
    p.slots_direct = 1;
    p.num_slots = (int32_t)s.S;
    // resident work-groups, a multiple of 8 (the kernel deals items per XCD)
    int64_t resident = (int64_t)std::max(num_cus, 1) * std::max(decode_blocks_per_cu, 1);
    if (opt && opt->decode_grid > 0) resident = opt->decode_grid;
    const int64_t grid = std::max<int64_t>(8, resident / 8 * 8);
    int64_t split_keys;
    p.balanced = false;
    if (force_split > 0 || (mk <= pa::kMaxSplitKeys && s.S * s.Hkv >= 4 * grid) ||
        mk <= pa::kEvenMinContext) {
      // fixed-size parts; without a forced count a whole (sequence, kv-head)
      // for every wave: the batch fills every wave, or its rows are so short
      // that a merge pass would cost more than the imbalance
      split_keys = force_split > 0 ? (mk + force_split - 1) / force_split : mk;
      split_keys = (split_keys + pa::kStageKeys - 1) / pa::kStageKeys * pa::kStageKeys;
      split_keys = std::min<int64_t>(split_keys, pa::kMaxSplitKeys);
      p.n_split = (int32_t)((mk + split_keys - 1) / split_keys);
    } else {
      // even split: the device cuts the stream of (sequence, kv-head, block)
      // into equal chunks, so every wave streams the same bytes however ragged
      // the batch.  A chunk has at least cmin blocks, cmin chosen so a row has
      // at most ~kEvenMaxParts parts; a row's parts are the chunks it touches.
      p.balanced = true;
      const int64_t mkb = (mk + pa::kBlockSize - 1) / pa::kBlockSize;
      const int64_t cmin = std::min<int64_t>(
          std::max<int64_t>(pa::kEvenMinBlocks, (mkb + pa::kEvenMaxParts - 1) / pa::kEvenMaxParts),
          pa::kMaxSplitKeys / pa::kBlockSize);
      split_keys = cmin * pa::kBlockSize;
      p.n_split = (int32_t)((mkb + cmin - 1) / cmin + 1);
      // stream positions stay in int32 on the device
      if ((int64_t)s.S * (mkb + 1) * s.Hkv * 2 > kMaxInt32)
        return fail(PA_ERR_UNSUPPORTED, "decode batch too large for the even split");
    }
    p.split_keys = (int32_t)split_keys;
    p.num_items = 0;                         // known on the device only
    p.nwg = grid;
    // Even split over 16-bit caches: one work-group per CU.  Each wave then
    // streams a chunk twice as long (fewer parts per row, less ramp-up and
    // drain per wave) and the waves still keep enough bytes in flight to
    // saturate HBM (the ragged decode batches measured 2-4% faster).  fp8
    // caches, half the bytes per block, keep every resident work-group.
    if (p.balanced && !s.kv8 && !(opt && opt->decode_grid > 0))
      p.nwg = std::max<int64_t>(8, (int64_t)std::max(num_cus, 1) / 8 * 8);
    if (p.n_split > 1) {
      // fixed parts: n_split part-major copies of the batch's rows.  Even
      // split: compact slots of max_seqlen_q tokens, one per (sequence, chunk
      // it touches), at most chunks + sequences of them; the chunk count is
      // bounded from the grid and the largest possible stream
      size_t rows = (size_t)s.T * (size_t)s.Hq * (size_t)p.n_split;
      if (p.balanced) {
        const int64_t workers = p.nwg * 4;
        const int64_t mkb = std::max<int64_t>((mk + pa::kBlockSize - 1) / pa::kBlockSize, 1);
        const int64_t all_max = s.S * mkb * s.Hkv;
        const int64_t kpw_max = std::max<int64_t>(
            1, (all_max + workers * pa::kMaxSplitKeys / pa::kBlockSize - 1) /
                   (workers * pa::kMaxSplitKeys / pa::kBlockSize));
        const int64_t cmin = p.split_keys / pa::kBlockSize;
        const int64_t chunks = std::min<int64_t>(workers * kpw_max / s.Hkv + 1,
                                                 (s.S * mkb + cmin - 1) / cmin);
        rows = (size_t)(chunks + s.S) * (size_t)mq * (size_t)s.Hq;
      }
      p.partial_rows = (int64_t)rows;
      p.ws_lse_offset = align256(rows * (size_t)s.D * sizeof(float));
      p.ws_parts_offset = p.ws_lse_offset + align256(rows * sizeof(float));
      p.ws_base_offset = p.ws_parts_offset + align256((size_t)s.T * (size_t)s.Hq * sizeof(int32_t));
      p.ws_bytes = p.ws_base_offset + (p.balanced ? align256((size_t)s.T * (size_t)s.Hq * sizeof(int32_t)) : 0);
    }
    *out = p;
    return PA_OK;
  }
  if (narrow) {
    p.tile_tokens = (int32_t)mq;
    p.slots_direct = 1;
    p.num_slots = (int32_t)s.S;
    p.wide = false;
  } else {
    p.wide = true;
    p.eight = force_tile == 4;
    p.tile_tokens = (int32_t)((p.eight ? pa::kTileRows8 : pa::kTileRows) / G);
    if (mq <= p.tile_tokens) {
      p.slots_direct = 1;
      p.num_slots = (int32_t)s.S;
    } else {
      p.slots_direct = 0;
      p.num_slots = (int32_t)(s.T / p.tile_tokens + s.S);
    }
  }
  p.tile_rows = (int32_t)(p.tile_tokens * G);
  const int64_t items = (int64_t)p.num_slots * s.Hkv;
  int64_t n_split = 1;
  if (force_split > 0) {
    n_split = force_split;
  } else if (items > 0) {
    // about two rounds of the 2 resident work-groups per CU; a split costs a
    // workspace round trip of every row it touches, so fuller grids do not split
    const int64_t target = 4LL * std::max(num_cus, 1);
    if (items < target) {
      const int64_t by_len = (mk + 511) / 512;
      n_split = std::min((target + items - 1) / items, by_len);
    }
  }
  n_split = std::max<int64_t>(n_split, 1);
  int64_t split_keys = (mk + n_split - 1) / n_split;
  split_keys = (split_keys + pa::kStageKeys - 1) / pa::kStageKeys * pa::kStageKeys;
  split_keys = std::min<int64_t>(split_keys, pa::kMaxSplitKeys);
  n_split = (mk + split_keys - 1) / split_keys;
  p.n_split = (int32_t)n_split;
  p.split_keys = (int32_t)split_keys;
  p.num_items = items * n_split;
  p.nwg = (p.num_items + 7) / 8 * 8;
  // wide plans rank their units longest-first on the device (one work-group
  // sorts the units by stage count into the workspace before the grid runs);
  // larger batches keep the index order
  p.lpt = p.wide && s.S <= pa::kLptMaxSeqs;
  if (p.num_items > kMaxInt32) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  size_t off = 0;
  if (n_split > 1) {
    const size_t rows = (size_t)s.T * (size_t)s.Hq * (size_t)n_split;
    p.partial_rows = (int64_t)rows;
    p.ws_lse_offset = align256(rows * (size_t)s.D * sizeof(float));
    p.ws_parts_offset = p.ws_lse_offset + align256(rows * sizeof(float));
    off = p.ws_parts_offset + align256((size_t)s.T * (size_t)s.Hq * sizeof(int32_t));
  }
  if (p.lpt) {
    p.lpt_units = (int64_t)p.num_slots * n_split;     // units the grid can hold
    // Every sequence in one tile: no two units read the same K/V (their key
    // ranges are disjoint), so nothing is gained by keeping a kv-head's
    // units on one XCD's L2.  The kv-heads of one unit, which read the same
    // cache blocks (each block holds every kv-head), then run side by side
    // on one XCD instead, as the decode kernel's waves do.
    p.unit_xcd = p.slots_direct != 0;
    if (p.unit_xcd) p.nwg = (p.lpt_units + 7) / 8 * 8 * s.Hkv;
    p.ws_lpt_offset = off;
    off += align256((size_t)p.lpt_units * 4 * sizeof(int32_t));
  }
  p.ws_bytes = off;
  *out = p;
  return PA_OK;
}

int device_cu_count(bool* ok) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    *ok = false;
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      *ok = false;
      return 256;
    }
    cache[dev] = n;
  }
  *ok = true;
  return cache[dev];
}

int decode_blocks_per_cu_cached(int head_dim, int group, bool kv8, bool f16) {
  static std::mutex mu;
  static int cache[4][2][2][17] = {};
  const int di = head_dim == 64 ? 0 : (head_dim == 96 ? 1 : (head_dim == 128 ? 2 : 3));
  const int ki = kv8 ? 1 : 0;
  const int fi = f16 ? 1 : 0;
  std::lock_guard<std::mutex> lock(mu);
  int& c = cache[di][ki][fi][group];
  if (c == 0) {
    const int n = pa::decode_blocks_per_cu(head_dim, group, kv8, f16);
    c = n > 0 ? n : -1;
  }
  return c > 0 ? c : 2;
}

int check_contents(const Shapes& s, const pa_tensor* cu, const pa_tensor* sk, const pa_tensor* bt,
                   int32_t max_q, int32_t max_k, hipStream_t stream) {
  std::vector<int32_t> hcu(s.S + 1), hsk(s.S), hbt((size_t)s.S * (size_t)s.bt_stride);
  hipError_t e = hipMemcpyAsync(hcu.data(), cu->data, hcu.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && s.S > 0)
    e = hipMemcpyAsync(hsk.data(), sk->data, hsk.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && s.S > 0 && s.MB > 0)
    e = hipMemcpyAsync(hbt.data(), bt->data, ((size_t)(s.S - 1) * s.bt_stride + s.MB) * 4,
                       hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "metadata copy: %s", hipGetErrorString(e));
  if (hcu[0] != 0) return fail(PA_ERR_CONTENT, "cu_seqlens_q[0] = %d", hcu[0]);
  for (int64_t i = 0; i < s.S; ++i) {
    const int32_t ql = hcu[i + 1] - hcu[i];
    if (ql < 0) return fail(PA_ERR_CONTENT, "cu_seqlens_q decreases at %lld", (long long)i);
    if (ql > max_q) return fail(PA_ERR_CONTENT, "sequence %lld: q_len %d > max_seqlen_q %d", (long long)i, ql, max_q);
    if (hsk[i] < 0 || hsk[i] > max_k)
      return fail(PA_ERR_CONTENT, "sequence %lld: seqused_k %d outside [0, %d]", (long long)i, hsk[i], max_k);
    const int64_t nb = (hsk[i] + s.B - 1) / s.B;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = hbt[(size_t)i * s.bt_stride + j];
      if (id < 0 || id >= s.NB)
        return fail(PA_ERR_CONTENT, "block_table[%lld, %lld] = %d outside [0, %lld)", (long long)i,
                    (long long)j, id, (long long)s.NB);
    }
  }
  if (hcu[s.S] != s.T) return fail(PA_ERR_CONTENT, "cu_seqlens_q[S] = %d != total_q %lld", hcu[s.S], (long long)s.T);
  return PA_OK;
}

// One workspace per (device, stream): calls on different streams never share
// split partials; calls on one stream are ordered by the stream.  Each entry
// has its own lock, which a call holds from the lookup until its kernels are
// enqueued: a second thread on the same stream that needs a larger buffer
// waits, and then frees the old one only after the stream has drained, so no
// enqueued kernel can see its workspace freed.
struct DeviceWorkspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t bytes = 0;
};

DeviceWorkspace* workspace_entry(hipStream_t stream, int* rc) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, std::unique_ptr<DeviceWorkspace>> pool;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  std::unique_ptr<DeviceWorkspace>& w = pool[std::make_pair(dev, stream)];
  if (!w) w.reset(new DeviceWorkspace());
  *rc = PA_OK;
  return w.get();
}

// Grows the entry to `need` bytes; the caller holds w->mu.
int grow_workspace(DeviceWorkspace* w, size_t need, hipStream_t stream) {
  if (w->bytes >= need) return PA_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(PA_ERR_WORKSPACE,
                "library workspace must grow to %zu bytes during stream capture; use "
                "pa_unified_attention_ex with a caller workspace", need);
  hipError_t e;
  if (w->ptr) {
    // every kernel that used the old buffer was enqueued on this stream
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipFree(w->ptr);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
    w->ptr = nullptr;
    w->bytes = 0;
  }
  const size_t grow = std::max(need, w->bytes + w->bytes / 2);
  e = hipMalloc(&w->ptr, grow);
  if (e != hipSuccess) {
    w->ptr = nullptr;
    return fail(PA_ERR_HIP, "workspace hipMalloc(%zu): %s", grow, hipGetErrorString(e));
  }
  w->bytes = grow;
  return PA_OK;
}

// lse: optional fp32 [T, Hq] receiving each row's natural-log log-sum-exp.
int validate_lse(const pa_tensor* lse, const Shapes& s, const pa_tensor* q, const pa_tensor* k,
                 const pa_tensor* v, const pa_tensor* out) {
  if (lse->dtype != PA_FP32) return fail(PA_ERR_DTYPE, "lse: dtype code %d, expected %d", lse->dtype, PA_FP32);
  if (lse->ndim != 2 || lse->shape[0] != s.T || lse->shape[1] != s.Hq)
    return fail(PA_ERR_SHAPE, "lse must be fp32 [total_q, num_q_heads]");
  if (lse->stride[1] != 1 && s.Hq > 1) return fail(PA_ERR_UNSUPPORTED, "lse needs a unit head stride");
  if (lse->stride[0] < 0) return fail(PA_ERR_SHAPE, "lse: negative stride");
  if (s.T > 0 && !lse->data) return fail(PA_ERR_NULL, "lse data is NULL");
  if (!aligned(lse->data, 4)) return fail(PA_ERR_ALIGN, "lse must be 4-byte aligned");
  const int64_t kv_esz = s.kv8 ? 1 : 2;
  if (overlaps(lse, 4, out, 2) || overlaps(lse, 4, q, 2) || overlaps(lse, 4, k, kv_esz) ||
      overlaps(lse, 4, v, kv_esz))
    return fail(PA_ERR_ALIAS, "lse overlaps q, out or a cache");
  return PA_OK;
}

// Where a call's split workspace comes from.
enum class WsMode { kLibrary, kCaller, kStatic };

int run(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, pa_tensor* out,
        const pa_tensor* lse, const pa_tensor* cu, const pa_tensor* sk, const pa_tensor* bt,
        int32_t max_q, int32_t max_k, float scale, int32_t causal, const pa_options* opt,
        WsMode ws_mode, void* ws, size_t ws_bytes, void* stream_v) {
  g_last_error.clear();
  Shapes s;
  int rc = validate(q, k, v, out, cu, sk, bt, max_q, max_k, &s);
  if (rc != PA_OK) return rc;
  if (lse) {
    rc = validate_lse(lse, s, q, k, v, out);
    if (rc != PA_OK) return rc;
  }
  // the options are checked for every batch, an empty one included
  bool have_dev = false;
  const int ncu = device_cu_count(&have_dev);
  const int dbpc = have_dev ? decode_blocks_per_cu_cached((int)s.D, (int)s.G, s.kv8, s.f16) : 2;
  Plan plan;
  rc = make_plan(s, max_q, max_k, opt, ncu, dbpc, &plan);
  if (rc != PA_OK) return rc;
  if (s.T == 0 || s.S == 0) return PA_OK;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
  std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
  if (ws_mode == WsMode::kLibrary) {
    if (plan.ws_bytes) {
      DeviceWorkspace* w = workspace_entry(stream, &rc);
      if (rc != PA_OK) return rc;
      ws_lock = std::unique_lock<std::mutex>(w->mu);
      rc = grow_workspace(w, plan.ws_bytes, stream);
      if (rc != PA_OK) return rc;
      ws = w->ptr;
    }
  } else if (ws_mode == WsMode::kStatic) {
    if (opt && opt->check_contents)
      return fail(PA_ERR_UNSUPPORTED, "check_contents synchronises and copies to the host; "
                                      "not available without allocation");
    if (plan.ws_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES)
      return fail(PA_ERR_WORKSPACE,
                  "this batch needs %zu bytes of split workspace; the static scratch holds %zu "
                  "(use pa_unified_attention_ex with a caller workspace)",
                  plan.ws_bytes, (size_t)PA_NOALLOC_SCRATCH_BYTES);
    if (plan.ws_bytes) {
      const hipError_t e = pa::noalloc_scratch(&ws);
      if (e != hipSuccess) return fail(PA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
    }
  } else if (plan.ws_bytes) {
    if (!ws) return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required", plan.ws_bytes);
    if (ws_bytes < plan.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, plan.ws_bytes);
    if (!aligned(ws, 256)) return fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  if (opt && opt->check_contents) {
    rc = check_contents(s, cu, sk, bt, max_q, max_k, stream);
    if (rc != PA_OK) return rc;
  }
  pa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q->data);
  p.out = static_cast<uint16_t*>(out->data);
  p.k = static_cast<const unsigned char*>(k->data);
  p.v = static_cast<const unsigned char*>(v->data);
  p.cu_q = static_cast<const int32_t*>(cu->data);
  p.seq_k = static_cast<const int32_t*>(sk->data);
  p.bt = static_cast<const int32_t*>(bt->data);
  p.ws_o = plan.n_split > 1 ? static_cast<float*>(ws) : nullptr;
  p.ws_lse = plan.n_split > 1
                 ? reinterpret_cast<float*>(static_cast<char*>(ws) + plan.ws_lse_offset)
                 : nullptr;
  p.q_st = s.q_st;
  p.q_sh = s.q_sh;
  p.o_st = s.o_st;
  p.o_sh = s.o_sh;
  p.kv_sb = s.kv_sb;
  p.bt_stride = (int32_t)s.bt_stride;
  p.num_seqs = (int32_t)s.S;
  p.total_q = (int32_t)s.T;
  p.num_q_heads = (int32_t)s.Hq;
  p.num_kv_heads = (int32_t)s.Hkv;
  p.max_k = max_k;
  p.tile_tokens = plan.tile_tokens;
  p.num_slots = plan.num_slots;
  p.slots_direct = plan.slots_direct;
  p.n_split = plan.n_split;
  p.split_keys = plan.split_keys;
  p.balanced = plan.balanced ? 1 : 0;
  p.ws_rparts = plan.n_split > 1
                   ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan.ws_parts_offset)
                   : nullptr;
  p.ws_rbase = plan.n_split > 1 && plan.balanced
                   ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan.ws_base_offset)
                   : nullptr;
  p.dq_tokens = plan.tile_tokens;
  p.num_items = (int32_t)plan.num_items;
  p.items_per_xcd = (int32_t)(plan.nwg / 8);
  p.kv_major = plan.wide ? 1 : 0;
  p.sub_sb = (int64_t)pa::kBlockSize * s.Hkv * s.D;
  p.bshift = s.B == 64 ? 2 : (s.B == 32 ? 1 : 0);
  p.lpt = plan.lpt ? 1 : 0;
  p.unit_xcd = plan.unit_xcd ? 1 : 0;
  p.lpt_units = (int32_t)plan.lpt_units;
  p.lpt_order = plan.lpt ? reinterpret_cast<int4*>(static_cast<char*>(ws) + plan.ws_lpt_offset)
                         : nullptr;
  p.causal = causal ? 1 : 0;
  // Rows of at most 16 take the narrow path, except in longest-first wide
  // plans over 16-bit caches at d = 64 and 128: there a decode row or short chunk
  // takes a wide tile too, whose K/V stream (its sequence is one tile).  On the
  // 248-decode-row + 8-chunk batch that measured 188.8-188.9 us back to back
  // against 196.9-200.4 with narrow decode rows (same box).
  const bool rows_wide =
      plan.wide && !plan.eight && plan.lpt && !s.kv8 && (s.D == 64 || s.D == 128);
  p.narrow_rows = ((opt && opt->force_tile == 2) || rows_wide) ? 0 : pa::kNarrowRows;
  // fp8 caches: k_scale folds into the score scale, v_scale into the output
  const double k_scale = s.kv8 && opt && opt->k_scale != 0.f ? opt->k_scale : 1.0;
  const double v_scale = s.kv8 && opt && opt->v_scale != 0.f ? opt->v_scale : 1.0;
  p.scale_log2 = (float)((double)scale * k_scale * 1.4426950408889634);
  p.out_scale = (float)v_scale;
  p.lse_out = lse ? static_cast<float*>(lse->data) : nullptr;
  p.lse_st = lse ? lse->stride[0] : 0;
  if (plan.nwg > 0 && plan.lpt) {
    const hipError_t e = pa::launch_rank(p, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "rank launch: %s", hipGetErrorString(e));
  }
  if (plan.nwg > 0) {
    // wide tiles of a plan whose every sequence is one tile read K/V that no
    // other tile reads: the kernel variant with streaming loads
    const int wide = plan.wide ? (plan.slots_direct ? 2 : 1) : 0;
    hipError_t e =
        plan.persistent ? pa::launch_decode(p, (int)s.D, (int)s.G, s.kv8, s.f16, plan.nwg, stream)
        : plan.eight    ? pa::launch_fwd8(p, (int)s.D, (int)s.G, s.f16, plan.nwg, stream)
                        : pa::launch_fwd(p, (int)s.D, (int)s.G, wide, s.kv8, s.f16, plan.nwg,
                                         stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  }
  if (plan.n_split > 1) {
    pa::MergeParams mp{};
    mp.ws_o = p.ws_o;
    mp.ws_lse = p.ws_lse;
    mp.out = p.out;
    mp.o_st = s.o_st;
    mp.o_sh = s.o_sh;
    mp.total_q = (int32_t)s.T;
    mp.num_q_heads = (int32_t)s.Hq;
    mp.n_split = plan.n_split;
    mp.row_parts = p.ws_rparts;
    mp.row_base = p.ws_rbase;
    mp.part_stride_c = (int64_t)plan.tile_tokens * s.Hq;
    mp.even = plan.balanced ? 1 : 0;
    mp.lse_out = p.lse_out;
    mp.lse_st = p.lse_st;
    hipError_t e = pa::launch_merge(mp, (int)s.D, s.f16, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_unified_attention(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         pa_tensor* out, const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                         const pa_tensor* block_table, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         float softmax_scale, int32_t causal, void* stream) {
  return run(q, k_cache, v_cache, out, nullptr, cu_seqlens_q, seqused_k, block_table,
             max_seqlen_q, max_seqlen_k, softmax_scale, causal, nullptr, WsMode::kLibrary, nullptr,
             0, stream);
}

int pa_unified_attention_ex(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                            pa_tensor* out, const pa_tensor* cu_seqlens_q,
                            const pa_tensor* seqused_k, const pa_tensor* block_table,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                            int32_t causal, const pa_options* opt, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return run(q, k_cache, v_cache, out, nullptr, cu_seqlens_q, seqused_k, block_table,
             max_seqlen_q, max_seqlen_k, softmax_scale, causal, opt, WsMode::kCaller, workspace,
             workspace_bytes, stream);
}

int pa_unified_attention_noalloc(const pa_tensor* q, const pa_tensor* k_cache,
                                 const pa_tensor* v_cache, pa_tensor* out,
                                 const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                                 const pa_tensor* block_table, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                                 const pa_options* opt, void* stream) {
  return run(q, k_cache, v_cache, out, nullptr, cu_seqlens_q, seqused_k, block_table,
             max_seqlen_q, max_seqlen_k, softmax_scale, causal, opt, WsMode::kStatic, nullptr, 0,
             stream);
}

int pa_unified_attention_lse(const pa_tensor* q, const pa_tensor* k_cache,
                             const pa_tensor* v_cache, pa_tensor* out, pa_tensor* lse,
                             const pa_tensor* cu_seqlens_q, const pa_tensor* seqused_k,
                             const pa_tensor* block_table, int32_t max_seqlen_q,
                             int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                             const pa_options* opt, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!lse) {
    g_last_error.clear();
    return fail(PA_ERR_NULL, "lse descriptor is NULL");
  }
  return run(q, k_cache, v_cache, out, lse, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
             max_seqlen_k, softmax_scale, causal, opt,
             workspace == nullptr ? WsMode::kLibrary : WsMode::kCaller, workspace,
             workspace_bytes, stream);
}

int pa_merge_attention(const pa_tensor* out_a, const pa_tensor* lse_a, const pa_tensor* out_b,
                       const pa_tensor* lse_b, pa_tensor* out, pa_tensor* lse_out, void* stream) {
  g_last_error.clear();
  if (!out_a || !lse_a || !out_b || !lse_b || !out)
    return fail(PA_ERR_NULL, "a tensor descriptor pointer is NULL");
  const pa_tensor* outs[] = {out_a, out_b, out};
  const pa_tensor* lses[] = {lse_a, lse_b, lse_out};
  const bool f16 = out->dtype == PA_F16;
  for (const pa_tensor* t : outs) {
    if (t->dtype != (f16 ? PA_F16 : PA_BF16))
      return fail(PA_ERR_DTYPE, "outputs must all be bf16 or all fp16");
    if (t->ndim != 3) return fail(PA_ERR_SHAPE, "outputs must be [total_q, num_q_heads, head_dim]");
    for (int i = 0; i < 3; ++i)
      if (t->shape[i] != out->shape[i]) return fail(PA_ERR_SHAPE, "output shapes differ");
    if (t->stride[2] != 1) return fail(PA_ERR_UNSUPPORTED, "outputs need a unit head_dim stride");
    if ((t->stride[0] | t->stride[1]) % 4) return fail(PA_ERR_ALIGN, "output strides must be multiples of 4");
    if (!aligned(t->data, 8)) return fail(PA_ERR_ALIGN, "outputs must be 8-byte aligned");
  }
  const int64_t T = out->shape[0], Hq = out->shape[1], D = out->shape[2];
  for (const pa_tensor* t : lses) {
    if (!t) continue;
    if (t->dtype != PA_FP32) return fail(PA_ERR_DTYPE, "lse tensors must be fp32");
    if (t->ndim != 2 || t->shape[0] != T || t->shape[1] != Hq)
      return fail(PA_ERR_SHAPE, "lse tensors must be [total_q, num_q_heads]");
    if (t->stride[1] != 1 && Hq > 1) return fail(PA_ERR_UNSUPPORTED, "lse needs a unit head stride");
    if (!aligned(t->data, 4)) return fail(PA_ERR_ALIGN, "lse must be 4-byte aligned");
  }
  if (D != 64 && D != 96 && D != 128 && D != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %lld (supported: 64, 96, 128, 256)", (long long)D);
  if (T * Hq > kMaxInt32) return fail(PA_ERR_UNSUPPORTED, "too many rows");
  if (overlaps(out, 2, out_a, 2) || overlaps(out, 2, out_b, 2) ||
      (lse_out && (overlaps(lse_out, 4, lse_a, 4) || overlaps(lse_out, 4, lse_b, 4) ||
                   overlaps(lse_out, 4, out, 2))))
    return fail(PA_ERR_ALIAS, "merge outputs overlap its inputs");
  if (T == 0 || Hq == 0) return PA_OK;
  pa::Merge2Params mp{};
  mp.oa = static_cast<const uint16_t*>(out_a->data);
  mp.ob = static_cast<const uint16_t*>(out_b->data);
  mp.la = static_cast<const float*>(lse_a->data);
  mp.lb = static_cast<const float*>(lse_b->data);
  mp.out = static_cast<uint16_t*>(out->data);
  mp.lse = lse_out ? static_cast<float*>(lse_out->data) : nullptr;
  mp.oa_st = out_a->stride[0];
  mp.oa_sh = out_a->stride[1];
  mp.ob_st = out_b->stride[0];
  mp.ob_sh = out_b->stride[1];
  mp.o_st = out->stride[0];
  mp.o_sh = out->stride[1];
  mp.la_st = lse_a->stride[0];
  mp.lb_st = lse_b->stride[0];
  mp.l_st = lse_out ? lse_out->stride[0] : 0;
  mp.total_q = (int32_t)T;
  mp.num_q_heads = (int32_t)Hq;
  const hipError_t e = pa::launch_merge2(mp, (int)D, f16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return PA_OK;
}

size_t pa_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         const pa_tensor* out, const pa_tensor* cu_seqlens_q,
                         const pa_tensor* seqused_k, const pa_tensor* block_table,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, const pa_options* opt) {
  g_last_error.clear();
  Shapes s;
  if (validate(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
               max_seqlen_k, &s) != PA_OK)
    return (size_t)-1;
  bool have_dev = false;
  const int ncu = device_cu_count(&have_dev);
  const int dbpc = have_dev ? decode_blocks_per_cu_cached((int)s.D, (int)s.G, s.kv8, s.f16) : 2;
  Plan plan;
  if (make_plan(s, max_seqlen_q, max_seqlen_k, opt, ncu, dbpc, &plan) != PA_OK) return (size_t)-1;
  if (s.T == 0 || s.S == 0) return 0;           // (options checked above)
  return plan.ws_bytes;
}

size_t pa_workspace_bytes(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                          const pa_tensor* out, const pa_tensor* cu_seqlens_q,
                          const pa_tensor* seqused_k, const pa_tensor* block_table,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, const pa_options* opt) {
  return pa_workspace_size(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table,
                           max_seqlen_q, max_seqlen_k, opt);
}

int pa_plan_describe(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                     const pa_tensor* out, const pa_tensor* cu_seqlens_q,
                     const pa_tensor* seqused_k, const pa_tensor* block_table,
                     int32_t max_seqlen_q, int32_t max_seqlen_k, const pa_options* opt,
                     int32_t num_cus, pa_plan_info* info) {
  g_last_error.clear();
  if (!info) return fail(PA_ERR_NULL, "info is NULL");
  Shapes s;
  int rc = validate(q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table, max_seqlen_q,
                    max_seqlen_k, &s);
  if (rc != PA_OK) return rc;
  bool have_dev = false;
  const int ncu = num_cus > 0 ? num_cus : device_cu_count(&have_dev);
  if (num_cus > 0) (void)device_cu_count(&have_dev);
  const int dbpc = have_dev ? decode_blocks_per_cu_cached((int)s.D, (int)s.G, s.kv8, s.f16) : 2;
  Plan plan;
  rc = make_plan(s, max_seqlen_q, max_seqlen_k, opt, ncu, dbpc, &plan);
  if (rc != PA_OK) return rc;
  if (s.T == 0 || s.S == 0) {
    plan.nwg = 0;
    plan.ws_bytes = 0;
  }
  info->tile_tokens = plan.tile_tokens;
  info->longest_first = plan.lpt ? 1 : 0;
  info->unit_xcd = plan.unit_xcd ? 1 : 0;
  info->tile_rows = plan.tile_rows;
  info->num_slots = plan.num_slots;
  info->slots_direct = plan.slots_direct;
  info->num_splits = plan.n_split;
  info->split_keys = plan.split_keys;
  info->num_workgroups = plan.nwg;
  info->workspace_bytes = (int64_t)plan.ws_bytes;
  info->persistent = plan.persistent ? 1 : 0;
  info->balanced = plan.balanced ? 1 : 0;
  info->partial_rows = (s.T == 0 || s.S == 0) ? 0 : plan.partial_rows;
  return PA_OK;
}

int pa_cache_write(const pa_tensor* key, const pa_tensor* value, pa_tensor* k_cache,
                   pa_tensor* v_cache, const pa_tensor* slot_mapping, float k_scale,
                   float v_scale, void* stream) {
  g_last_error.clear();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "a tensor descriptor pointer is NULL");
  const bool kv8 = k_cache->dtype == PA_FP8_E4M3;
  const bool f16 = key->dtype == PA_F16;
  const int sdt = f16 ? PA_F16 : PA_BF16;
  const int cdt = kv8 ? PA_FP8_E4M3 : sdt;
  const int64_t esz = kv8 ? 1 : 2;
  struct {
    const pa_tensor* t;
    const char* name;
    int dtype;
    int ndim;
  } spec[] = {{key, "key", sdt, 3},           {value, "value", sdt, 3},
              {k_cache, "k_cache", cdt, 4},   {v_cache, "v_cache", cdt, 4},
              {slot_mapping, "slot_mapping", PA_INT32, 1}};
  for (auto& e : spec) {
    if (e.t->dtype != e.dtype)
      return fail(PA_ERR_DTYPE, "%s: dtype code %d, expected %d", e.name, e.t->dtype, e.dtype);
    if (e.t->ndim != e.ndim)
      return fail(PA_ERR_SHAPE, "%s: ndim %d, expected %d", e.name, e.t->ndim, e.ndim);
    for (int i = 0; i < e.ndim; ++i)
      if (e.t->shape[i] < 0 || e.t->stride[i] < 0)
        return fail(PA_ERR_SHAPE, "%s: negative extent or stride in dim %d", e.name, i);
  }
  const int64_t N = key->shape[0], Hkv = k_cache->shape[2], D = k_cache->shape[3];
  const int64_t NB = k_cache->shape[0], B = k_cache->shape[1];
  for (int i = 0; i < 3; ++i)
    if (value->shape[i] != key->shape[i]) return fail(PA_ERR_SHAPE, "value shape differs from key");
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i] || v_cache->stride[i] != k_cache->stride[i])
      return fail(PA_ERR_SHAPE, "v_cache shape/strides differ from k_cache in dim %d", i);
  if (key->shape[1] != Hkv || key->shape[2] != D)
    return fail(PA_ERR_SHAPE, "key [N, %lld, %lld] does not match the cache heads / head_dim",
                (long long)key->shape[1], (long long)key->shape[2]);
  if (slot_mapping->shape[0] != N)
    return fail(PA_ERR_SHAPE, "slot_mapping has %lld entries, expected %lld",
                (long long)slot_mapping->shape[0], (long long)N);
  if (B != 16 && B != 32 && B != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %lld (supported: 16, 32, 64)", (long long)B);
  if (D % 8 || D <= 0) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a positive multiple of 8");
  if (N > kMaxInt32 || NB * B > kMaxInt32 || Hkv * D > kMaxInt32 / 8)
    return fail(PA_ERR_UNSUPPORTED, "sizes beyond the 32-bit slot range");
  if (key->stride[2] != 1 || value->stride[2] != 1)
    return fail(PA_ERR_UNSUPPORTED, "key/value need a unit stride along head_dim");
  if ((key->stride[0] | key->stride[1] | value->stride[0] | value->stride[1]) % 8)
    return fail(PA_ERR_ALIGN, "key/value strides must be multiples of 8 elements");
  if (k_cache->stride[3] != 1 || k_cache->stride[2] != D || k_cache->stride[1] != Hkv * D)
    return fail(PA_ERR_UNSUPPORTED, "caches need contiguous [block_size, num_kv_heads, head_dim]");
  if (NB > 1 && k_cache->stride[0] < B * Hkv * D)
    return fail(PA_ERR_SHAPE, "cache block stride smaller than one block");
  if ((k_cache->stride[0] * esz) % 16)
    return fail(PA_ERR_ALIGN, "cache block stride must be a multiple of 16 bytes");
  if (slot_mapping->stride[0] != 1 && N > 1) return fail(PA_ERR_UNSUPPORTED, "slot_mapping not contiguous");
  if (N == 0) return PA_OK;
  if (!key->data || !value->data || !k_cache->data || !v_cache->data || !slot_mapping->data)
    return fail(PA_ERR_NULL, "data pointer is NULL");
  if (!aligned(key->data, 16) || !aligned(value->data, 16) || !aligned(k_cache->data, 16) ||
      !aligned(v_cache->data, 16))
    return fail(PA_ERR_ALIGN, "key/value/cache data must be 16-byte aligned");
  if (!aligned(slot_mapping->data, 4)) return fail(PA_ERR_ALIGN, "slot_mapping must be 4-byte aligned");
  if (overlaps(k_cache, esz, key, 2) || overlaps(k_cache, esz, value, 2) ||
      overlaps(v_cache, esz, key, 2) || overlaps(v_cache, esz, value, 2) ||
      overlaps(k_cache, esz, v_cache, esz))
    return fail(PA_ERR_ALIAS, "caches overlap each other or the new keys / values");
  pa::CacheWriteParams p{};
  p.key = static_cast<const uint16_t*>(key->data);
  p.value = static_cast<const uint16_t*>(value->data);
  p.k_cache = static_cast<unsigned char*>(k_cache->data);
  p.v_cache = static_cast<unsigned char*>(v_cache->data);
  p.slot_mapping = static_cast<const int32_t*>(slot_mapping->data);
  p.k_st = key->stride[0];
  p.k_sh = key->stride[1];
  p.v_st = value->stride[0];
  p.v_sh = value->stride[1];
  p.cache_sb = k_cache->stride[0];
  p.block_size = (int32_t)B;
  p.num_slots = (int32_t)(NB * B);
  p.num_tokens = (int32_t)N;
  p.slot_elems = (int32_t)(Hkv * D);
  p.chunks_per_token = (int32_t)(Hkv * D / 8);
  p.chunks_per_head = (int32_t)(D / 8);
  p.k_scale = k_scale != 0.f ? k_scale : 1.f;
  p.v_scale = v_scale != 0.f ? v_scale : 1.f;
  const hipError_t e = pa::launch_cache_write(p, kv8, f16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch: %s", hipGetErrorString(e));
  return PA_OK;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_DTYPE: return "wrong dtype";
    case PA_ERR_SHAPE: return "inconsistent shape";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_ALIGN: return "misaligned pointer or stride";
    case PA_ERR_ALIAS: return "output aliases an input";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_CONTENT: return "invalid metadata contents";
    case PA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return PA_VERSION; }

}  // extern "C"
