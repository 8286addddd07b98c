// common.h -- internal helpers shared by the gfx950 kernels of libdynconv.
// Not part of the public interface (that is include/dynconv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dynconv.h"

namespace dynconv {

typedef __bf16 bf16;

// 16-byte vector of the I/O dtype: 8 bf16 or 4 fp32 channels.
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Load one 16-byte vector and widen it to fp32.
template <typename T>
__device__ __forceinline__ void load_vec(const T *p, float (&out)[Vec<T>::N]) {
  const uint4 raw = *reinterpret_cast<const uint4 *>(p);
  if constexpr (sizeof(T) == 4) {
    out[0] = __uint_as_float(raw.x);
    out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z);
    out[3] = __uint_as_float(raw.w);
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Narrow 16 bytes' worth of fp32 values to T and store them.
template <typename T>
__device__ __forceinline__ void store_vec(T *p, const float (&v)[Vec<T>::N]) {
  uint4 raw;
  if constexpr (sizeof(T) == 4) {
    raw.x = __float_as_uint(v[0]);
    raw.y = __float_as_uint(v[1]);
    raw.z = __float_as_uint(v[2]);
    raw.w = __float_as_uint(v[3]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 lo = (bf16)v[2 * i], hi = (bf16)v[2 * i + 1];
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    raw = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *reinterpret_cast<uint4 *>(p) = raw;
}

// Everything a kernel needs to know about the problem (passed by value).
struct Shape {
  int64_t B, T, BT, d, D;
  int k, kind, n_heads, rank;
  int N;   // generator outputs per token: n_heads*k or rank
  int hd;  // channels per head (head-wise)
  // packed documents: per token, its position in its document (low byte)
  // and the tokens after it in that document (high byte), both clamped to
  // 255 (more than any tap reaches); NULL when every row is one sequence
  const uint16_t *seqpos;
  bool packed;  // the problem has packed documents (seqpos is set before any conv kernel)
  // static filter only (no generator): head-wise in form, one head of D
  // channels, N = 0 generator values (the kernels read zeros for u)
  bool stat;
};

// Position of token row r in its sequence, and the tokens after it there
// (clamped to 255), for kernels that look them up per token.
__device__ __forceinline__ int seq_pos(const Shape &s, int64_t r) {
  return s.seqpos ? (int)(s.seqpos[r] & 255u) : (int)(r % s.T);
}
__device__ __forceinline__ int seq_rem(const Shape &s, int64_t r) {
  return s.seqpos ? (int)(s.seqpos[r] >> 8) : (int)(s.T - 1 - r % s.T);
}

// Launch helpers (defined in api.hip, used by the kernel files).
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dynconv
