// Driver for a sanitizer build of libpa's host code: pa_api.cpp compiled with
// AddressSanitizer and UndefinedBehaviorSanitizer against stub launchers
// (launch_stubs.cpp).  Seeded random and edge-case descriptors go through the
// validation and planning of every entry point: pa_plan_describe and
// pa_workspace_bytes over thousands of batch shapes (valid ones and ones with
// a broken field), the attention, merge and cache-write calls with invalid
// arguments (they must fail before anything runs), and pa_last_error after
// each failure.  No device memory is touched: descriptor addresses are never
// dereferenced by the host code.  Prints "ok <calls>" when every check holds.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "pa.h"

namespace {

std::mt19937_64 rng(20261203);

int64_t pick(std::initializer_list<int64_t> v) {
  return *(v.begin() + (int64_t)(rng() % v.size()));
}
int64_t uniform(int64_t lo, int64_t hi) {  // [lo, hi]
  return hi <= lo ? lo : lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
}

// A contiguous descriptor at a fake, 256-byte aligned address.
pa_tensor desc(uint64_t addr, int dtype, std::vector<int64_t> shape) {
  pa_tensor t;
  std::memset(&t, 0, sizeof(t));
  t.data = reinterpret_cast<void*>(addr);
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int64_t st = 1;
  for (int i = (int)shape.size() - 1; i >= 0; --i) {
    t.shape[i] = shape[i];
    t.stride[i] = st;
    st *= shape[i] > 0 ? shape[i] : 1;
  }
  return t;
}

int failures = 0;
void check(bool cond, const char* what, long it) {
  if (!cond) {
    std::printf("FAIL %s (iteration %ld): %s\n", what, it, pa_last_error());
    ++failures;
  }
}

}  // namespace

int main() {
  long calls = 0, planned = 0;
  const int iters = 4000;
  for (long it = 0; it < iters; ++it) {
    const int64_t D = pick({64, 96, 128, 256, 64, 128, 32, 512});
    const int64_t Hkv = pick({1, 2, 4, 8});
    const int64_t G = pick({1, 2, 4, 8, 16, 3, 32});
    const int64_t Hq = Hkv * G;
    const int64_t B = pick({16, 32, 64, 16, 8, 128});
    const int64_t S = pick({0, 1, 3, 17, 256, 2048, 2049, 5000});
    const int64_t max_q = pick({0, 1, 1, 5, 16, 33, 512, 4000});
    const int64_t max_k = pick({0, 1, 64, 1000, 4096, 131072, 1 << 22});
    const int64_t T = S == 0 ? 0 : std::min<int64_t>(S * uniform(0, max_q), 1 << 20);
    const int64_t MB = (max_k + B - 1) / B + uniform(0, 2);
    const int64_t NB = std::max<int64_t>(1, uniform(0, S * MB + 1));
    const int qdt = pick({PA_BF16, PA_F16});
    const int kvdt = uniform(0, 3) == 0 ? PA_FP8_E4M3 : qdt;
    std::vector<pa_tensor> d = {
        desc(1ull << 40, qdt, {T, Hq, D}),
        desc(2ull << 40, kvdt, {NB, B, Hkv, D}),
        desc(3ull << 40, kvdt, {NB, B, Hkv, D}),
        desc(4ull << 40, qdt, {T, Hq, D}),
        desc(5ull << 40, PA_INT32, {S + 1}),
        desc(6ull << 40, PA_INT32, {S}),
        desc(7ull << 40, PA_INT32, {S, MB}),
    };
    // one field in four iterations is broken
    switch (uniform(0, 15)) {
      case 0: d[uniform(0, 6)].data = nullptr; break;
      case 1: d[uniform(0, 6)].dtype = (int32_t)uniform(-1, 7); break;
      case 2: d[uniform(0, 6)].ndim = (int32_t)uniform(0, 5); break;
      case 3: d[uniform(0, 6)].shape[uniform(0, 3)] = uniform(-3, 3); break;
      default: break;
    }
    if (uniform(0, 9) == 0) d[0].stride[0] = uniform(-8, 1 << 20);
    if (uniform(0, 9) == 0) d[1].data = reinterpret_cast<void*>((2ull << 40) + 8);  // misaligned
    pa_options opt;
    std::memset(&opt, 0, sizeof(opt));
    opt.force_num_splits = (int32_t)pick({0, 0, 0, 1, 2, 3, 7, 1000, -1});
    opt.force_tile = (int32_t)pick({0, 0, 0, 1, 2, 3, 4, 5, -1});
    opt.decode_grid = (int32_t)pick({0, 0, 8, 100, 1 << 20});
    opt.k_scale = (float)pick({0, 1, 2}) / 64.f;
    const int32_t num_cus = (int32_t)pick({0, 1, 80, 256, 304, -5});
    const pa_options* po = uniform(0, 3) == 0 ? nullptr : &opt;
    pa_plan_info info;
    std::memset(&info, 0, sizeof(info));
    const int rc = pa_plan_describe(&d[0], &d[1], &d[2], &d[3], &d[4], &d[5], &d[6],
                                    (int32_t)max_q, (int32_t)max_k, po, num_cus, &info);
    const size_t ws = pa_workspace_bytes(&d[0], &d[1], &d[2], &d[3], &d[4], &d[5], &d[6],
                                         (int32_t)max_q, (int32_t)max_k, po);
    calls += 2;
    if (rc == PA_OK) {
      ++planned;
      check(info.num_workgroups >= 0, "grid size is not negative", it);
      check(info.num_splits >= 1, "at least one split", it);
      check(info.tile_rows >= 1 && info.tile_rows <= 256, "tile rows in range", it);
      check(info.partial_rows >= 0, "partial rows not negative", it);
      check(ws != (size_t)-1, "workspace size of a valid plan", it);
      // (pa_workspace_bytes plans for the device's CU count: 256 without a device)
      if (num_cus <= 0 || num_cus == 256)
        check(ws == (size_t)info.workspace_bytes, "workspace size agrees with the plan", it);
    } else {
      check(ws == (size_t)-1, "invalid arguments give no workspace size", it);
      check(std::strlen(pa_last_error()) > 0, "an error message after a failure", it);
    }
  }
  // entry points that launch: invalid arguments fail before any launch
  pa_tensor q = desc(1ull << 40, PA_BF16, {4, 8, 128});
  pa_tensor kc = desc(2ull << 40, PA_BF16, {8, 16, 2, 128});
  pa_tensor cu = desc(5ull << 40, PA_INT32, {3});
  pa_tensor sk = desc(6ull << 40, PA_INT32, {2});
  pa_tensor bt = desc(7ull << 40, PA_INT32, {2, 4});
  pa_tensor bad = q;
  bad.ndim = 2;
  check(pa_unified_attention(nullptr, &kc, &kc, &q, &cu, &sk, &bt, 2, 64, 0.1f, 1, nullptr) ==
            PA_ERR_NULL, "attention: NULL q", -1);
  check(pa_unified_attention(&bad, &kc, &kc, &q, &cu, &sk, &bt, 2, 64, 0.1f, 1, nullptr) ==
            PA_ERR_SHAPE, "attention: q of rank 2", -1);
  check(pa_unified_attention_ex(&q, &kc, &kc, &q, &cu, &sk, &bt, 2, 64, 0.1f, 1, nullptr,
                                nullptr, 0, nullptr) != PA_OK, "attention_ex: out aliases q", -1);
  check(pa_unified_attention_noalloc(&bad, &kc, &kc, &q, &cu, &sk, &bt, 2, 64, 0.1f, 1, nullptr,
                                     nullptr) == PA_ERR_SHAPE, "noalloc: q of rank 2", -1);
  pa_tensor lse = desc(8ull << 40, PA_FP32, {4, 8});
  check(pa_merge_attention(&bad, &lse, &q, &lse, &q, nullptr, nullptr) != PA_OK,
        "merge: out_a of rank 2", -1);
  pa_tensor key = desc(9ull << 40, PA_BF16, {3, 2, 128});
  pa_tensor slots = desc(10ull << 40, PA_INT32, {2});
  check(pa_cache_write(&key, &key, &kc, &kc, &slots, 1.f, 1.f, nullptr) != PA_OK,
        "cache write: slot count differs from tokens", -1);
  calls += 6;
  std::printf("planned %ld of %d\n", planned, iters);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok %ld\n", calls);
  return 0;
}
