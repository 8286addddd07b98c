// simple_kernels.hip -- plain VALU kernels of the dynamic short convolution.
//
// One thread per output element (or per 16-byte output vector when rows are
// whole vectors), fp32
// accumulation in the order of each defining sum, no atomics.  They are the
// fp32 path of the library (where bf16 MFMA would not meet fp32 accuracy)
// and the general fallback for shapes the tuned bf16 kernels do not cover.
//
// The formulas are those of "Dynamic Short Convolutions Improve
// Transformers" (gist.science Technical Summary, Methodology -> Dynamic
// Short Convolutions: Mechanism, Parameterization, Placement), restated in
// include/dynconv.h together with the backward.
#include "kernels.h"

namespace dynconv {

// ---------------------------------------------------------------------------
// out[t, n] = sum_i a[t, i] * m[i, n]      (u = h W, or z = h A)
// A tiled product: a block of 16 x 16 threads computes 64 rows x 64
// columns, each thread 4 x 4 of them, with a and m staged in LDS 16 values
// of i at a time; every output sums over i in increasing order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_gen_proj(const T *__restrict__ a, const T *__restrict__ m, float *__restrict__ out, int64_t rows,
           int K, int N) {
  __shared__ float as[16][64 + 4];  // [i][row]
  __shared__ float ms[16][64 + 4];  // [i][column]
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int n0 = (int)blockIdx.y * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = ty + 16 * u;
      const int64_t t = t0 + r;
      as[tx][r] = (t < rows && k0 + tx < K) ? to_f32(a[t * K + k0 + tx]) : 0.f;
      // m: 16 rows of i, 64 columns; thread (ty, tx) loads columns tx + 16 u of row k0 + ty
      const int n = n0 + tx + 16 * u;
      ms[ty][tx + 16 * u] = (k0 + ty < K && n < N) ? to_f32(m[(int64_t)(k0 + ty) * N + n]) : 0.f;
    }
    __syncthreads();
    const int kn = min(16, K - k0);
    for (int kk = 0; kk < kn; ++kk) {
      float x[4], y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = as[kk][4 * ty + q], y[q] = ms[kk][4 * tx + q];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(x[q], y[r], acc[q][r]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * ty + q;
    if (t >= rows) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * tx + r;
      if (n < N) out[t * N + n] = acc[q][r];
    }
  }
}

// the producing projection: x[t, c] = sum_i h[t, i] * Wp[i, c], written in T
template <typename T>
__global__ void __launch_bounds__(256)
k_proj_simple(const T *__restrict__ h, const T *__restrict__ Wp, T *__restrict__ x, int64_t rows, int64_t K,
              int64_t D) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * D) return;
  const int64_t t = g / D, c = g - t * D;
  float acc = 0.f;
  for (int64_t i = 0; i < K; ++i) acc = fmaf(to_f32(h[t * K + i]), to_f32(Wp[i * D + c]), acc);
  x[g] = from_f32<T>(acc);
}

// Filter tap j of channel c at token row `row`:
// head-wise u[row, head(c)*k + j] + w0, low-rank sum_q z[row,q] U[q, c*k+j] + w0.
template <typename T>
__device__ __forceinline__ float filter_tap(const Shape &s, const float *__restrict__ gen,
                                            const T *__restrict__ U, const T *__restrict__ w0,
                                            int64_t row, int64_t c, int j) {
  float w;
  if (s.kind == DYNCONV_HEADWISE) {
    w = gen[row * s.N + (c / s.hd) * s.k + j];
  } else {
    w = 0.f;
    const float *zr = gen + row * s.N;
    for (int q = 0; q < s.N; ++q)
      w = fmaf(zr[q], to_f32(U[(int64_t)q * s.D * s.k + c * s.k + j]), w);
  }
  if (w0) w += to_f32(w0[c * s.k + j]);
  return w;
}

// ---------------------------------------------------------------------------
// forward conv: y[row, c] = x[row, c] + sum_j [t-j>=0] w[row,c,j] x[row-j, c]
// One thread per 16-byte vector of channels.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_conv_fwd_simple(Shape s, const float *__restrict__ gen, const T *__restrict__ U,
                  const T *__restrict__ w0, const T *__restrict__ x, T *__restrict__ y) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * nvec) return;
  const int64_t row = g / nvec;
  const int64_t c0 = (g - row * nvec) * V;
  const int pos = seq_pos(s, row);
  float acc[V];
  load_vec(x + row * s.D + c0, acc);
  for (int j = 0; j < s.k && j <= pos; ++j) {
    float xv[V];
    load_vec(x + (row - j) * s.D + c0, xv);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(filter_tap(s, gen, U, w0, row, c0 + i, j), xv[i], acc[i]);
  }
  store_vec(y + row * s.D + c0, acc);
}

// The low-rank forward with the filter of the thread's V channels formed
// for all K taps at once: per rank q, one z value and the V*K contiguous
// values of U row q (K 16-byte loads), each tap summing over q in increasing
// order and then adding the bias, as filter_tap does.
template <typename T, int K>
__global__ void __launch_bounds__(256)
k_conv_fwd_lr(Shape s, const float *__restrict__ gen, const T *__restrict__ U, const T *__restrict__ w0,
              const T *__restrict__ x, T *__restrict__ y) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * nvec) return;
  const int64_t row = g / nvec;
  const int64_t c0 = (g - row * nvec) * V;
  float w[V * K];
#pragma unroll
  for (int e = 0; e < V * K; ++e) w[e] = 0.f;
  const float *zr = gen + row * s.N;
  const T *ub = U + c0 * K;
  for (int q = 0; q < s.N; ++q) {
    const float zq = zr[q];
    const T *uq = ub + (int64_t)q * s.D * K;
#pragma unroll
    for (int m = 0; m < K; ++m) {  // values V m .. V m + V - 1 of the segment
      float uv[V];
      load_vec(uq + V * m, uv);
#pragma unroll
      for (int i = 0; i < V; ++i) w[V * m + i] = fmaf(zq, uv[i], w[V * m + i]);
    }
  }
  if (w0) {
#pragma unroll
    for (int m = 0; m < K; ++m) {
      float bv[V];
      load_vec(w0 + c0 * K + V * m, bv);
#pragma unroll
      for (int i = 0; i < V; ++i) w[V * m + i] += bv[i];
    }
  }
  // segment value e is channel c0 + e / K, tap e % K
  const int pos = seq_pos(s, row);
  float acc[V];
  load_vec(x + row * s.D + c0, acc);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (j > pos) break;
    float xv[V];
    load_vec(x + (row - j) * s.D + c0, xv);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i * K + j], xv[i], acc[i]);
  }
  store_vec(y + row * s.D + c0, acc);
}

// ---------------------------------------------------------------------------
// dx[row, c] = dy[row, c] + sum_j [t+j<=T-1] w[row+j, c, j] dy[row+j, c]
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_conv_dx_simple(Shape s, const float *__restrict__ gen, const T *__restrict__ U,
                 const T *__restrict__ w0, const T *__restrict__ dy, T *__restrict__ dx) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * nvec) return;
  const int64_t row = g / nvec;
  const int64_t c0 = (g - row * nvec) * V;
  const int rem = seq_rem(s, row);
  float acc[V];
  load_vec(dy + row * s.D + c0, acc);
  for (int j = 0; j < s.k && j <= rem; ++j) {
    float gv[V];
    load_vec(dy + (row + j) * s.D + c0, gv);
#pragma unroll
    for (int i = 0; i < V; ++i)
      acc[i] = fmaf(filter_tap(s, gen, U, w0, row + j, c0 + i, j), gv[i], acc[i]);
  }
  store_vec(dx + row * s.D + c0, acc);
}

// The low-rank dx with the filters of all K taps formed together: tap j uses
// the z row of token row + j, so per rank q the thread reads K z values and
// the V*K contiguous values of U row q once (K 16-byte loads); each filter
// value sums over q in increasing order and then adds the bias, as
// filter_tap does.  Rows past the sequence end are never read (rem).
template <typename T, int K>
__global__ void __launch_bounds__(256)
k_conv_dx_lr(Shape s, const float *__restrict__ gen, const T *__restrict__ U, const T *__restrict__ w0,
             const T *__restrict__ dy, T *__restrict__ dx) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * nvec) return;
  const int64_t row = g / nvec;
  const int64_t c0 = (g - row * nvec) * V;
  const int rem = seq_rem(s, row);
  float w[V * K];  // value e: channel c0 + e / K, tap e % K
#pragma unroll
  for (int e = 0; e < V * K; ++e) w[e] = 0.f;
  const T *ub = U + c0 * K;
  for (int q = 0; q < s.N; ++q) {
    float zq[K];
#pragma unroll
    for (int j = 0; j < K; ++j) zq[j] = j <= rem ? gen[(row + j) * s.N + q] : 0.f;
    const T *uq = ub + (int64_t)q * s.D * K;
#pragma unroll
    for (int m = 0; m < K; ++m) {
      float uv[V];
      load_vec(uq + V * m, uv);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = V * m + i;
        w[e] = fmaf(zq[e % K], uv[i], w[e]);
      }
    }
  }
  if (w0) {
#pragma unroll
    for (int m = 0; m < K; ++m) {
      float bv[V];
      load_vec(w0 + c0 * K + V * m, bv);
#pragma unroll
      for (int i = 0; i < V; ++i) w[V * m + i] += bv[i];
    }
  }
  float acc[V];
  load_vec(dy + row * s.D + c0, acc);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (j > rem) break;
    float gv[V];
    load_vec(dy + (row + j) * s.D + c0, gv);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i * K + j], gv[i], acc[i]);
  }
  store_vec(dx + row * s.D + c0, acc);
}

// The same two convolutions for any D, one thread per element (rows that are
// not whole 16-byte vectors cannot be read as such).
template <typename T>
__global__ void __launch_bounds__(256)
k_conv_fwd_scalar(Shape s, const float *__restrict__ gen, const T *__restrict__ U,
                  const T *__restrict__ w0, const T *__restrict__ x, T *__restrict__ y) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * s.D) return;
  const int64_t row = g / s.D;
  const int64_t c = g - row * s.D;
  const int pos = seq_pos(s, row);
  float acc = to_f32(x[g]);
  for (int j = 0; j < s.k && j <= pos; ++j)
    acc = fmaf(filter_tap(s, gen, U, w0, row, c, j), to_f32(x[g - j * s.D]), acc);
  y[g] = from_f32<T>(acc);
}

template <typename T>
__global__ void __launch_bounds__(256)
k_conv_dx_scalar(Shape s, const float *__restrict__ gen, const T *__restrict__ U,
                 const T *__restrict__ w0, const T *__restrict__ dy, T *__restrict__ dx) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= s.BT * s.D) return;
  const int64_t row = g / s.D;
  const int64_t c = g - row * s.D;
  const int rem = seq_rem(s, row);
  float acc = to_f32(dy[g]);
  for (int j = 0; j < s.k && j <= rem; ++j)
    acc = fmaf(filter_tap(s, gen, U, w0, row + j, c, j), to_f32(dy[g + j * s.D]), acc);
  dx[g] = from_f32<T>(acc);
}

// G[row, c, j] = [row-j in row's sequence] dy[row, c] x[row-j, c]
template <typename T>
__device__ __forceinline__ float gtap(const Shape &s, const T *__restrict__ x,
                                      const T *__restrict__ dy, int64_t row, int64_t c, int j) {
  if (j > seq_pos(s, row)) return 0.f;
  return to_f32(dy[row * s.D + c]) * to_f32(x[(row - j) * s.D + c]);
}

// head-wise: g[row, e*k+j] = du = sum_{c in head e} G[row, c, j]
template <typename T>
__global__ void __launch_bounds__(256)
k_du_simple(Shape s, const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.BT * s.N) return;
  const int64_t row = idx / s.N;
  const int n = (int)(idx - row * s.N);
  const int e = n / s.k, j = n - e * s.k;
  float acc = 0.f;
  for (int64_t c = (int64_t)e * s.hd; c < (int64_t)(e + 1) * s.hd; ++c) acc += gtap(s, x, dy, row, c, j);
  g[idx] = acc;
}

// The same du for heads of whole 16-byte vectors: 16-byte loads of dy and of
// x at lag j, the products added in the same channel order.
template <typename T>
__global__ void __launch_bounds__(256)
k_du_vec(Shape s, const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ g) {
  constexpr int V = Vec<T>::N;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.BT * s.N) return;
  const int64_t row = idx / s.N;
  const int n = (int)(idx - row * s.N);
  const int e = n / s.k, j = n - e * s.k;
  float acc = 0.f;
  if (j <= seq_pos(s, row)) {
    const T *dr = dy + row * s.D, *xr = x + (row - j) * s.D;
    for (int64_t c0 = (int64_t)e * s.hd; c0 < (int64_t)(e + 1) * s.hd; c0 += V) {
      float dv[V], xv[V];
      load_vec(dr + c0, dv);
      load_vec(xr + c0, xv);
#pragma unroll
      for (int i = 0; i < V; ++i) acc += dv[i] * xv[i];
    }
  }
  g[idx] = acc;
}

// low-rank: g[row, q] = dz = sum_{c,j} G[row, c, j] U[q, c*k+j]
template <typename T>
__global__ void __launch_bounds__(256)
k_dz_simple(Shape s, const T *__restrict__ x, const T *__restrict__ dy, const T *__restrict__ U,
            float *__restrict__ g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.BT * s.N) return;
  const int64_t row = idx / s.N;
  const int q = (int)(idx - row * s.N);
  const T *Uq = U + (int64_t)q * s.D * s.k;
  float acc = 0.f;
  for (int64_t c = 0; c < s.D; ++c)
    for (int j = 0; j < s.k; ++j) acc = fmaf(gtap(s, x, dy, row, c, j), to_f32(Uq[c * s.k + j]), acc);
  g[idx] = acc;
}

// The same dz for rows of whole 16-byte vectors and K taps: per V channels
// one load of dy, one per tap of x and K 16-byte loads of U row q; the
// products are added in the same order (channel, then tap) as above.
template <typename T, int K>
__global__ void __launch_bounds__(256)
k_dz_vec(Shape s, const T *__restrict__ x, const T *__restrict__ dy, const T *__restrict__ U,
         float *__restrict__ g) {
  constexpr int V = Vec<T>::N;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.BT * s.N) return;
  const int64_t row = idx / s.N;
  const int q = (int)(idx - row * s.N);
  const int pos = seq_pos(s, row);
  const T *Uq = U + (int64_t)q * s.D * K;
  float acc = 0.f;
  for (int64_t c0 = 0; c0 < s.D; c0 += V) {
    float dv[V], xv[K][V], uv[K * V];
    load_vec(dy + row * s.D + c0, dv);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (j <= pos) {
        load_vec(x + (row - j) * s.D + c0, xv[j]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) xv[j][i] = 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < K; ++m) {
      float t[V];
      load_vec(Uq + c0 * K + V * m, t);
#pragma unroll
      for (int i = 0; i < V; ++i) uv[V * m + i] = t[i];
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) acc = fmaf(dv[i] * xv[j][i], uv[i * K + j], acc);
  }
  g[idx] = acc;
}


// Sums over rows for 16 outputs per block: thread (tx, ty) of a 16 x 16
// block adds term(o, row) for output o = 16 blockIdx.x + tx over rows ty,
// ty + 16, ... in ascending order; the 16 row groups are then added in order
// (deterministic).  Consecutive outputs read neighbouring channels of a row.
template <typename F>
__device__ __forceinline__ void rows_reduce(int64_t n_out, int64_t rows, F term, float *__restrict__ out) {
  __shared__ float part[16][17];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int64_t o = (int64_t)blockIdx.x * 16 + tx;
  float acc = 0.f;
  if (o < n_out)
    for (int64_t row = ty; row < rows; row += 16) acc += term(o, row);
  part[ty][tx] = acc;
  __syncthreads();
  if (ty == 0 && o < n_out) {
    float t = 0.f;
    for (int r = 0; r < 16; ++r) t += part[r][tx];
    out[o] = t;
  }
}

// low-rank: dU[q, c*k+j] = sum_rows z[row, q] G[row, c, j], with each
// G[row, c, j] formed once for 16 ranks: block (16,
// 16) takes 16 consecutive (c, j) columns (tx) and ranks q0 .. q0 + 15 (grid
// y); thread row group ty adds rows ty, ty + 16, ... in ascending order, and
// the 16 row groups are added in order at the end, as rows_reduce does.
template <typename T>
__global__ void __launch_bounds__(256)
k_dU_rows(Shape s, const float *__restrict__ z, const T *__restrict__ x, const T *__restrict__ dy,
          float *__restrict__ dU) {
  __shared__ float part[16][16][17];  // [row group][rank][column]
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int64_t Dk = s.D * s.k;
  const int64_t m = (int64_t)blockIdx.x * 16 + tx;
  const int q0 = (int)blockIdx.y * 16;
  const int nq = min(16, s.N - q0);
  float acc[16];
#pragma unroll
  for (int qq = 0; qq < 16; ++qq) acc[qq] = 0.f;
  if (m < Dk) {
    const int64_t c = m / s.k;
    const int j = (int)(m - c * s.k);
    for (int64_t row = ty; row < s.BT; row += 16) {
      const float G = gtap(s, x, dy, row, c, j);
      const float *zr = z + row * s.N + q0;
#pragma unroll
      for (int qq = 0; qq < 16; ++qq)
        if (qq < nq) acc[qq] += zr[qq] * G;
    }
  }
#pragma unroll
  for (int qq = 0; qq < 16; ++qq) part[ty][qq][tx] = acc[qq];
  __syncthreads();
  // thread (tx, ty) finishes rank q0 + ty of column m
  if (m < Dk && ty < nq) {
    float t = 0.f;
    for (int r = 0; r < 16; ++r) t += part[r][ty][tx];
    dU[(int64_t)(q0 + ty) * Dk + m] = t;
  }
}

// dw0[c, j] = sum_rows G[row, c, j]
template <typename T>
__global__ void __launch_bounds__(256)
k_dw0_simple(Shape s, const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ dw0) {
  rows_reduce(s.D * s.k, s.BT, [&](int64_t idx, int64_t row) {
    const int64_t c = idx / s.k;
    const int j = (int)(idx - c * s.k);
    return gtap(s, x, dy, row, c, j);
  }, dw0);
}

// dM[i, n] = sum_rows h[row, i] g[row, n]      (dW or dA)
template <typename T>
__global__ void __launch_bounds__(256)
k_dgen_simple(Shape s, const T *__restrict__ h, const float *__restrict__ g, float *__restrict__ dM) {
  rows_reduce(s.d * s.N, s.BT, [&](int64_t idx, int64_t row) {
    const int64_t i = idx / s.N;
    const int n = (int)(idx - i * s.N);
    return to_f32(h[row * s.d + i]) * g[row * s.N + n];
  }, dM);
}

// dh[t, i] = sum_n g[t, n] M[i, n] (M = W or A) as a tiled product: a block of 16 x 16
// threads computes 64 tokens x 64 columns of d, each thread 4 x 4 of them,
// with g and M staged in LDS 16 generator columns at a time; every output
// sums over n in increasing order.
template <typename T>
__global__ void __launch_bounds__(256)
k_dh_tiled(Shape s, const float *__restrict__ g, const T *__restrict__ M, T *__restrict__ dh) {
  __shared__ float gs[16][64 + 4];  // [n][token]
  __shared__ float ms[16][64 + 4];  // [n][i]
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int64_t i0 = (int64_t)blockIdx.y * 64;
  const int N = s.N;
  float acc[4][4] = {};
  for (int n0 = 0; n0 < N; n0 += 16) {
    // each thread stages 4 values of each tile: row r = threadIdx / 16 + 16 u, column n0 + tx
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = ty + 16 * u;
      const int n = n0 + tx;
      const int64_t t = t0 + r, i = i0 + r;
      gs[tx][r] = (t < s.BT && n < N) ? g[t * N + n] : 0.f;
      ms[tx][r] = (i < s.d && n < N) ? to_f32(M[i * N + n]) : 0.f;
    }
    __syncthreads();
    const int kn = min(16, N - n0);
    for (int kk = 0; kk < kn; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = gs[kk][4 * ty + q], b[q] = ms[kk][4 * tx + q];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(a[q], b[r], acc[q][r]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * ty + q;
    if (t >= s.BT) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t i = i0 + 4 * tx + r;
      if (i < s.d) dh[t * s.d + i] = from_f32<T>(acc[q][r]);
    }
  }
}

// Packed documents: per token t, its position in its document and the tokens
// after it there, each clamped to [0, 255], from the document offsets cu
// (n + 1 entries, 0 = cu[0] <= ... <= cu[n] = BT).  The document of t is the
// last i < n with cu[i] <= t (a binary search); offsets that break the rule
// still give values in range.
__global__ void __launch_bounds__(256)
k_seqpos(const int32_t *__restrict__ cu, int64_t n, int64_t BT, uint16_t *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= BT) return;
  int64_t lo = 0, hi = n - 1;  // invariant: the document is in [lo, hi]
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  int64_t start = cu[lo], end = cu[lo + 1];
  start = start < 0 ? 0 : (start > t ? t : start);
  end = end > BT ? BT : (end <= t ? t + 1 : end);
  const int64_t pos = t - start, rem = end - 1 - t;
  out[t] = (uint16_t)((pos < 255 ? pos : 255) | ((rem < 255 ? rem : 255) << 8));
}

void seqpos_fill(const int32_t *cu, int64_t n_seqs, int64_t BT, uint16_t *out, hipStream_t st) {
  if (BT > 0) hipLaunchKernelGGL(k_seqpos, dim3((unsigned)ceil_div(BT, 256)), dim3(256), 0, st, cu, n_seqs, BT, out);
}

__global__ void __launch_bounds__(256) k_zero(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

__global__ void __launch_bounds__(256) k_zero16(uint16_t *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static inline dim3 grid1(int64_t n) { return dim3((unsigned)ceil_div(n, 256)); }
static inline dim3 grid16(int64_t n) { return dim3((unsigned)ceil_div(n, 16)); }  // rows_reduce: 16 outputs per block
// k_dh_tiled: 64 tokens (grid x) by 64 columns of d (grid y) per block
static inline dim3 dh_grid(const Shape &s) {
  return dim3((unsigned)ceil_div(s.BT, 64), (unsigned)ceil_div(s.d, 64));
}

void zero_fill(float *p, int64_t n, hipStream_t st) {
  if (p && n > 0) hipLaunchKernelGGL(k_zero, grid1(n), dim3(256), 0, st, p, n);
}

void zero_fill_bytes(void *p, size_t nbytes, hipStream_t st) {
  const int64_t n = (int64_t)(nbytes / 2);
  if (p && n > 0) hipLaunchKernelGGL(k_zero16, grid1(n), dim3(256), 0, st, (uint16_t *)p, n);
}

template <typename T>
int simple_gen_proj(const Shape &s, const void *h, const void *M, float *out, hipStream_t st) {
  if (s.BT * s.N == 0) return 0;
  hipLaunchKernelGGL(k_gen_proj<T>, dim3((unsigned)ceil_div(s.BT, 64), (unsigned)ceil_div(s.N, 64)), dim3(256), 0, st,
                     (const T *)h, (const T *)M,
                     out, s.BT, (int)s.d, s.N);
  return 0;
}

template <typename T>
int simple_fwd_conv(const Shape &s, const float *gen, const void *U, const void *w0, const void *x,
                    void *y, hipStream_t st) {
  if (s.D % Vec<T>::N == 0 && s.kind == DYNCONV_LOWRANK) {
    const int64_t n = s.BT * (s.D / Vec<T>::N);
    switch (s.k) {
#define LRK(K_)                                                                                             \
  case K_:                                                                                                  \
    hipLaunchKernelGGL((k_conv_fwd_lr<T, K_>), grid1(n), dim3(256), 0, st, s, gen, (const T *)U, (const T *)w0, \
                       (const T *)x, (T *)y);                                                               \
    break;
      LRK(1) LRK(2) LRK(3) LRK(4) LRK(5) LRK(6) LRK(7) LRK(8)
#undef LRK
      default: return DYNCONV_E_LIMIT;
    }
  } else if (s.D % Vec<T>::N == 0) {
    const int64_t n = s.BT * (s.D / Vec<T>::N);
    hipLaunchKernelGGL(k_conv_fwd_simple<T>, grid1(n), dim3(256), 0, st, s, gen, (const T *)U,
                       (const T *)w0, (const T *)x, (T *)y);
  } else {
    hipLaunchKernelGGL(k_conv_fwd_scalar<T>, grid1(s.BT * s.D), dim3(256), 0, st, s, gen, (const T *)U,
                       (const T *)w0, (const T *)x, (T *)y);
  }
  return 0;
}

template <typename T>
int simple_bwd(const Shape &s, const float *gen, const void *W, const void *A, const void *U,
               const void *w0, const void *h, const void *x, const void *dy, void *dx, void *dh,
               const dynconv_gen_grad &gg, float *g, hipStream_t st) {
  if (s.D % Vec<T>::N == 0 && s.kind == DYNCONV_LOWRANK) {
    const int64_t nv = s.BT * (s.D / Vec<T>::N);
    switch (s.k) {
#define LRK(K_)                                                                                             \
  case K_:                                                                                                  \
    hipLaunchKernelGGL((k_conv_dx_lr<T, K_>), grid1(nv), dim3(256), 0, st, s, gen, (const T *)U, (const T *)w0, \
                       (const T *)dy, (T *)dx);                                                             \
    break;
      LRK(1) LRK(2) LRK(3) LRK(4) LRK(5) LRK(6) LRK(7) LRK(8)
#undef LRK
      default: return DYNCONV_E_LIMIT;
    }
  } else if (s.D % Vec<T>::N == 0) {
    const int64_t nv = s.BT * (s.D / Vec<T>::N);
    hipLaunchKernelGGL(k_conv_dx_simple<T>, grid1(nv), dim3(256), 0, st, s, gen, (const T *)U,
                       (const T *)w0, (const T *)dy, (T *)dx);
  } else {
    hipLaunchKernelGGL(k_conv_dx_scalar<T>, grid1(s.BT * s.D), dim3(256), 0, st, s, gen, (const T *)U,
                       (const T *)w0, (const T *)dy, (T *)dx);
  }
  if (gg.dw0)
    hipLaunchKernelGGL(k_dw0_simple<T>, grid16(s.D * s.k), dim3(16, 16), 0, st, s, (const T *)x,
                       (const T *)dy, gg.dw0);
  if (s.stat) return 0;  // no generator (the caller has cleared dh)
  if (s.kind == DYNCONV_HEADWISE) {
    if (s.hd % Vec<T>::N == 0)
      hipLaunchKernelGGL(k_du_vec<T>, grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x, (const T *)dy, g);
    else
      hipLaunchKernelGGL(k_du_simple<T>, grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x,
                         (const T *)dy, g);
    hipLaunchKernelGGL(k_dgen_simple<T>, grid16(s.d * s.N), dim3(16, 16), 0, st, s, (const T *)h, g, gg.dW);
    if (dh)
      hipLaunchKernelGGL(k_dh_tiled<T>, dh_grid(s), dim3(256), 0, st, s, g, (const T *)W,
                         (T *)dh);
  } else {
    if (s.D % Vec<T>::N == 0) {
      switch (s.k) {
#define DZK(K_)                                                                                             \
  case K_:                                                                                                  \
    hipLaunchKernelGGL((k_dz_vec<T, K_>), grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x, (const T *)dy, \
                       (const T *)U, g);                                                                    \
    break;
        DZK(1) DZK(2) DZK(3) DZK(4) DZK(5) DZK(6) DZK(7) DZK(8)
#undef DZK
        default: return DYNCONV_E_LIMIT;
      }
    } else {
      hipLaunchKernelGGL(k_dz_simple<T>, grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x,
                         (const T *)dy, (const T *)U, g);
    }
    hipLaunchKernelGGL(k_dU_rows<T>, dim3((unsigned)ceil_div((int64_t)s.D * s.k, 16), (unsigned)ceil_div(s.N, 16)),
                       dim3(16, 16), 0, st, s, gen, (const T *)x, (const T *)dy, gg.dU);
    hipLaunchKernelGGL(k_dgen_simple<T>, grid16(s.d * s.N), dim3(16, 16), 0, st, s, (const T *)h, g, gg.dA);
    if (dh)
      hipLaunchKernelGGL(k_dh_tiled<T>, dh_grid(s), dim3(256), 0, st, s, g, (const T *)A,
                         (T *)dh);
  }
  return 0;
}

template <typename T>
int simple_proj(const Shape &s, const void *h, const void *Wp, void *x, hipStream_t st) {
  if (s.BT * s.D == 0) return 0;
  hipLaunchKernelGGL(k_proj_simple<T>, grid1(s.BT * s.D), dim3(256), 0, st, (const T *)h, (const T *)Wp, (T *)x,
                     s.BT, s.d, s.D);
  return 0;
}

#define INST(T)                                                                                  \
  template int simple_gen_proj<T>(const Shape &, const void *, const void *, float *, hipStream_t); \
  template int simple_proj<T>(const Shape &, const void *, const void *, void *, hipStream_t);       \
  template int simple_fwd_conv<T>(const Shape &, const float *, const void *, const void *,        \
                                  const void *, void *, hipStream_t);                             \
  template int simple_bwd<T>(const Shape &, const float *, const void *, const void *,            \
                             const void *, const void *, const void *, const void *,              \
                             const void *, void *, void *, const dynconv_gen_grad &, float *,     \
                             hipStream_t);
INST(float)
INST(bf16)
#undef INST

}  // namespace dynconv
