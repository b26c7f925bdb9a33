// gfx950 kernel of libpa: writing new tokens' keys and values into the paged
// KV cache [num_blocks, block_size, Hkv, d] (the cache layout of the unified kernel,
// page "[Kernel] Unified Triton kernel that doesn't distinguish between
// prefill + decode", PR description).  Token i goes to cache slot
// slot_mapping[i] = physical block * block_size + position in the block; a negative
// slot is skipped.  16-bit caches receive the bf16 / fp16 values unchanged; fp8 caches
// (OCP E4M3 "fn", the KV-cache format discussed in the review of page
// "[Kernel] [V1] Improved performance for V1 Triton (ROCm) backend") receive
// the code of x / scale rounded to nearest, ties to even, saturated at +-448
// (the format has no infinity); NaN stays NaN.
//
// HBM-bound copy: each thread iteration moves one 16-byte chunk of bf16 (8
// elements) of one token's [Hkv, d] row; the row is contiguous in the
// destination slot, so a wave writes whole slot rows.

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E4M3 ("fn") code of x: round to nearest even on the format's grid, values
// at or beyond the rounding limit of 448 saturate to +-448.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if (__builtin_isnan(x)) return sign | 0x7Fu;
  const float a = __builtin_fabsf(x);
  if (a >= 464.f) return sign | 0x7Eu;              // 464 = midpoint of 448 and 480
  if (a < 0.015625f) {                              // below 2^-6: quantum 2^-9
    // a * 2^9 < 8 is exact; rint rounds half to even; 8 is the code of 2^-6
    return sign | (uint32_t)__builtin_rintf(a * 512.f);
  }
  int e = (int)((bits >> 23) & 0xFFu) - 127;        // a is a normal float: 2^e <= a
  int m = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // a / 2^(e-3) in [8, 16]
  if (m == 16) {
    m = 8;
    e += 1;
  }
  return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)(m - 8);
}

// the two 16-bit source elements of w (low, high) as fp32, exactly
template <bool F16>
__device__ __forceinline__ float src_lo(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  return __builtin_bit_cast(float, w << 16);
}
template <bool F16>
__device__ __forceinline__ float src_hi(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// KV8: fp8 caches (else the source's 16-bit type, copied); F16: fp16 sources
// (else bf16)
template <bool KV8, bool F16>
__global__ __launch_bounds__(256) void pa_cache_write_kernel(CacheWriteParams p) {
  const int64_t per_tensor = (int64_t)p.num_tokens * p.chunks_per_token;
  const int64_t total = 2 * per_tensor;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = c >= per_tensor;
    const int64_t r = is_v ? c - per_tensor : c;
    const int tok = (int)(r / p.chunks_per_token);
    const int ch = (int)(r - (int64_t)tok * p.chunks_per_token);
    const int slot = p.slot_mapping[tok];
    if (slot < 0 || slot >= p.num_slots) continue;   // padding token, or a slot outside the cache
    const int head = ch / p.chunks_per_head;
    const int dc = ch - head * p.chunks_per_head;
    const uint16_t* src = (is_v ? p.value : p.key) + (int64_t)tok * (is_v ? p.v_st : p.k_st) +
                          (int64_t)head * (is_v ? p.v_sh : p.k_sh) + dc * 8;
    const u32x4 w = *reinterpret_cast<const u32x4*>(src);
    // element offset of the chunk in the cache
    const int64_t dst = (int64_t)(slot / p.block_size) * p.cache_sb +
                        (int64_t)(slot % p.block_size) * p.slot_elems + (int64_t)ch * 8;
    unsigned char* cache = is_v ? p.v_cache : p.k_cache;
    if constexpr (!KV8) {
      *reinterpret_cast<u32x4*>(cache + dst * 2) = w;
    } else {
      const float s = is_v ? p.v_scale : p.k_scale;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = e4m3_code(__fdiv_rn(src_lo<F16>(w[e]), s));
        const uint32_t b = e4m3_code(__fdiv_rn(src_hi<F16>(w[e]), s));
        const uint32_t pair = a | (b << 8);
        if (e < 2) lo |= pair << (16 * e);
        else hi |= pair << (16 * (e - 2));
      }
      *reinterpret_cast<u32x2*>(cache + dst) = u32x2{lo, hi};
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, bool kv8, bool f16, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)p.num_tokens * p.chunks_per_token;
  if (total <= 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (kv8 && f16)
    hipLaunchKernelGGL((pa_cache_write_kernel<true, true>), dim3(grid), dim3(256), 0, stream, p);
  else if (kv8)
    hipLaunchKernelGGL((pa_cache_write_kernel<true, false>), dim3(grid), dim3(256), 0, stream, p);
  else
    // a 16-bit copy does not depend on the element type
    hipLaunchKernelGGL((pa_cache_write_kernel<false, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
