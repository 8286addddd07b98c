// conv_fwd_headwise.hip -- forward of the head-wise dynamic short convolution.
//
//   y[row, c] = x[row, c] + sum_{j<k, j<=pos} (u[row, head(c)*k + j] + w0[c, j]) * x[row-j, c]
//
// (gist.science Technical Summary of "Dynamic Short Convolutions Improve
// Transformers", Methodology -> Dynamic Short Convolutions: Mechanism; the
// head-wise tying of the Parameterization item; the residual of Placement.)
// u = h W comes from the generator projection kernel; the filter itself is
// formed in registers and never written to memory.
//
// Layout on the chip: a thread owns one 16-byte vector of channels (8 bf16 or
// 4 fp32) and walks a chunk of consecutive tokens, keeping the last k-1 rows
// of x in registers, so x is read once (plus a k-1 row halo per chunk) and y
// is written once, both as 16-byte loads/stores that are contiguous across
// the 64 lanes of a wave (1 KiB per wave instruction).  A block is 64 vectors
// x 4 token chunks; the grid covers (D / vector / 64) x (tokens / (4 * TC)).
// The HBM roofline bounds it: per token it moves 2*D*eb bytes of x and y plus
// the n_heads*k*4 bytes of u (a broadcast read, cached).
#include "kernels.h"

namespace dynconv {
namespace {

constexpr int kFwdChunk = 32;  // tokens per thread

template <typename T, int KP>
__global__ void __launch_bounds__(256)
k_fwd_headwise(Shape s, const float *__restrict__ u, const T *__restrict__ w0,
               const T *__restrict__ x, T *__restrict__ y) {
  constexpr int V = Vec<T>::N;
  const int nvec = (int)(s.D / V);
  const int v = blockIdx.x * 64 + threadIdx.x;
  if (v >= nvec) return;
  const int64_t row0 = ((int64_t)blockIdx.y * 4 + threadIdx.y) * kFwdChunk;
  if (row0 >= s.BT) return;
  const int64_t row1 = row0 + kFwdChunk < s.BT ? row0 + kFwdChunk : s.BT;
  const int c0 = v * V;
  const int k = s.k;

  // heads of this vector's channels: the first (ea) and, when the vector
  // straddles a head boundary, the next one; `second` flags channels of the
  // later head.  When heads are narrower than a vector, fall back to a
  // per-channel lookup.
  const int ea = c0 / s.hd;
  const bool two_heads_max = s.hd >= V;
  int second = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) second |= ((c0 + i) / s.hd != ea) << i;

  float b[V][KP];
#pragma unroll
  for (int i = 0; i < V; ++i)
#pragma unroll
    for (int j = 0; j < KP; ++j) b[i][j] = (w0 && j < k) ? to_f32(w0[(int64_t)(c0 + i) * k + j]) : 0.f;

  // window: xw[j] = x[row - j]; rows before the sequence start are zero
  float xw[KP][V];
  int64_t pos = row0 % s.T;
#pragma unroll
  for (int j = 1; j < KP; ++j) {
    if (j < k && pos - j >= 0) {
      load_vec(x + (row0 - j) * s.D + c0, xw[j]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) xw[j][i] = 0.f;
    }
  }

  for (int64_t row = row0; row < row1; ++row, ++pos) {
    if (pos == s.T) {  // a new sequence starts: clear the history
      pos = 0;
#pragma unroll
      for (int j = 1; j < KP; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) xw[j][i] = 0.f;
    }
    load_vec(x + row * s.D + c0, xw[0]);
    const float *ur = u + row * s.N;
    float ua[KP], ub[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      ua[j] = j < k ? ur[ea * k + j] : 0.f;
      ub[j] = (j < k && second) ? ur[(ea + 1) * k + j] : 0.f;
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float a = xw[0][i];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        float uj;
        if (two_heads_max) {
          uj = ((second >> i) & 1) ? ub[j] : ua[j];
        } else {
          uj = j < k ? ur[((c0 + i) / s.hd) * k + j] : 0.f;
        }
        a = fmaf(uj + b[i][j], xw[j][i], a);
      }
      acc[i] = a;
    }
    store_vec(y + row * s.D + c0, acc);
#pragma unroll
    for (int j = KP - 1; j > 0; --j)
#pragma unroll
      for (int i = 0; i < V; ++i) xw[j][i] = xw[j - 1][i];
  }
}

template <typename T, int KP>
void launch(const Shape &s, const float *u, const void *w0, const void *x, void *y, hipStream_t st) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  dim3 grid((unsigned)ceil_div(nvec, 64), (unsigned)ceil_div(s.BT, 4 * kFwdChunk));
  hipLaunchKernelGGL((k_fwd_headwise<T, KP>), grid, dim3(64, 4), 0, st, s, u, (const T *)w0,
                     (const T *)x, (T *)y);
}

}  // namespace

template <typename T>
int fwd_headwise(const Shape &s, const float *u, const void *w0, const void *x, void *y,
                 hipStream_t st) {
  const bool tr = trace_begin(DYNCONV_K_FWD_CONV, st);
  if (s.k <= 4)
    launch<T, 4>(s, u, w0, x, y, st);
  else
    launch<T, 8>(s, u, w0, x, y, st);
  trace_end(tr, st);
  return 0;
}

template int fwd_headwise<float>(const Shape &, const float *, const void *, const void *, void *,
                                 hipStream_t);
template int fwd_headwise<bf16>(const Shape &, const float *, const void *, const void *, void *,
                                hipStream_t);

}  // namespace dynconv
