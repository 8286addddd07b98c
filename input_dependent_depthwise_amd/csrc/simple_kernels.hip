// simple_kernels.hip -- plain VALU kernels of the dynamic short convolution.
//
// One thread per output element (or per 16-byte output vector), fp32
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
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_gen_proj(const T *__restrict__ a, const T *__restrict__ m, float *__restrict__ out, int64_t rows,
           int K, int N) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * N) return;
  const int64_t t = g / N;
  const int n = (int)(g - t * N);
  const T *at = a + t * K;
  float acc = 0.f;
  for (int i = 0; i < K; ++i) acc = fmaf(to_f32(at[i]), to_f32(m[(int64_t)i * N + n]), acc);
  out[g] = acc;
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
  const int64_t t = row % s.T;
  float acc[V];
  load_vec(x + row * s.D + c0, acc);
  for (int j = 0; j < s.k && j <= t; ++j) {
    float xv[V];
    load_vec(x + (row - j) * s.D + c0, xv);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(filter_tap(s, gen, U, w0, row, c0 + i, j), xv[i], acc[i]);
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
  const int64_t t = row % s.T;
  float acc[V];
  load_vec(dy + row * s.D + c0, acc);
  for (int j = 0; j < s.k && t + j <= s.T - 1; ++j) {
    float gv[V];
    load_vec(dy + (row + j) * s.D + c0, gv);
#pragma unroll
    for (int i = 0; i < V; ++i)
      acc[i] = fmaf(filter_tap(s, gen, U, w0, row + j, c0 + i, j), gv[i], acc[i]);
  }
  store_vec(dx + row * s.D + c0, acc);
}

// G[row, c, j] = [t-j>=0] dy[row, c] x[row-j, c]
template <typename T>
__device__ __forceinline__ float gtap(const Shape &s, const T *__restrict__ x,
                                      const T *__restrict__ dy, int64_t row, int64_t c, int j) {
  const int64_t t = row % s.T;
  if (t - j < 0) return 0.f;
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

// low-rank: dU[q, c*k+j] = sum_rows z[row, q] G[row, c, j]
template <typename T>
__global__ void __launch_bounds__(256)
k_dU_simple(Shape s, const float *__restrict__ z, const T *__restrict__ x, const T *__restrict__ dy,
            float *__restrict__ dU) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t Dk = s.D * s.k;
  if (idx >= (int64_t)s.N * Dk) return;
  const int q = (int)(idx / Dk);
  const int64_t m = idx - (int64_t)q * Dk;
  const int64_t c = m / s.k;
  const int j = (int)(m - c * s.k);
  float acc = 0.f;
  for (int64_t row = 0; row < s.BT; ++row) acc = fmaf(z[row * s.N + q], gtap(s, x, dy, row, c, j), acc);
  dU[idx] = acc;
}

// dw0[c, j] = sum_rows G[row, c, j]
template <typename T>
__global__ void __launch_bounds__(256)
k_dw0_simple(Shape s, const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ dw0) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.D * s.k) return;
  const int64_t c = idx / s.k;
  const int j = (int)(idx - c * s.k);
  float acc = 0.f;
  for (int64_t row = 0; row < s.BT; ++row) acc += gtap(s, x, dy, row, c, j);
  dw0[idx] = acc;
}

// dM[i, n] = sum_rows h[row, i] g[row, n]      (dW or dA)
template <typename T>
__global__ void __launch_bounds__(256)
k_dgen_simple(Shape s, const T *__restrict__ h, const float *__restrict__ g, float *__restrict__ dM) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.d * s.N) return;
  const int64_t i = idx / s.N;
  const int n = (int)(idx - i * s.N);
  float acc = 0.f;
  for (int64_t row = 0; row < s.BT; ++row) acc = fmaf(to_f32(h[row * s.d + i]), g[row * s.N + n], acc);
  dM[idx] = acc;
}

// dh[row, i] = sum_n g[row, n] M[i, n]      (M = W or A)
template <typename T>
__global__ void __launch_bounds__(256)
k_dh_simple(Shape s, const float *__restrict__ g, const T *__restrict__ M, T *__restrict__ dh) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= s.BT * s.d) return;
  const int64_t row = idx / s.d;
  const int64_t i = idx - row * s.d;
  float acc = 0.f;
  for (int n = 0; n < s.N; ++n) acc = fmaf(g[row * s.N + n], to_f32(M[i * s.N + n]), acc);
  dh[idx] = from_f32<T>(acc);
}

__global__ void __launch_bounds__(256) k_zero(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static inline dim3 grid1(int64_t n) { return dim3((unsigned)ceil_div(n, 256)); }

void zero_fill(float *p, int64_t n, hipStream_t st) {
  if (p && n > 0) hipLaunchKernelGGL(k_zero, grid1(n), dim3(256), 0, st, p, n);
}

template <typename T>
int simple_gen_proj(const Shape &s, const void *h, const void *M, float *out, hipStream_t st) {
  if (s.BT * s.N == 0) return 0;
  hipLaunchKernelGGL(k_gen_proj<T>, grid1(s.BT * s.N), dim3(256), 0, st, (const T *)h, (const T *)M,
                     out, s.BT, (int)s.d, s.N);
  return 0;
}

template <typename T>
int simple_fwd_conv(const Shape &s, const float *gen, const void *U, const void *w0, const void *x,
                    void *y, hipStream_t st) {
  const int64_t n = s.BT * (s.D / Vec<T>::N);
  hipLaunchKernelGGL(k_conv_fwd_simple<T>, grid1(n), dim3(256), 0, st, s, gen, (const T *)U,
                     (const T *)w0, (const T *)x, (T *)y);
  return 0;
}

template <typename T>
int simple_bwd(const Shape &s, const float *gen, const void *W, const void *A, const void *U,
               const void *w0, const void *h, const void *x, const void *dy, void *dx, void *dh,
               const dynconv_gen_grad &gg, float *g, hipStream_t st) {
  const int64_t nv = s.BT * (s.D / Vec<T>::N);
  hipLaunchKernelGGL(k_conv_dx_simple<T>, grid1(nv), dim3(256), 0, st, s, gen, (const T *)U,
                     (const T *)w0, (const T *)dy, (T *)dx);
  if (gg.dw0)
    hipLaunchKernelGGL(k_dw0_simple<T>, grid1(s.D * s.k), dim3(256), 0, st, s, (const T *)x,
                       (const T *)dy, gg.dw0);
  if (s.kind == DYNCONV_HEADWISE) {
    hipLaunchKernelGGL(k_du_simple<T>, grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x,
                       (const T *)dy, g);
    hipLaunchKernelGGL(k_dgen_simple<T>, grid1(s.d * s.N), dim3(256), 0, st, s, (const T *)h, g, gg.dW);
    if (dh)
      hipLaunchKernelGGL(k_dh_simple<T>, grid1(s.BT * s.d), dim3(256), 0, st, s, g, (const T *)W,
                         (T *)dh);
  } else {
    hipLaunchKernelGGL(k_dz_simple<T>, grid1(s.BT * s.N), dim3(256), 0, st, s, (const T *)x,
                       (const T *)dy, (const T *)U, g);
    hipLaunchKernelGGL(k_dU_simple<T>, grid1((int64_t)s.N * s.D * s.k), dim3(256), 0, st, s, gen,
                       (const T *)x, (const T *)dy, gg.dU);
    hipLaunchKernelGGL(k_dgen_simple<T>, grid1(s.d * s.N), dim3(256), 0, st, s, (const T *)h, g, gg.dA);
    if (dh)
      hipLaunchKernelGGL(k_dh_simple<T>, grid1(s.BT * s.d), dim3(256), 0, st, s, g, (const T *)A,
                         (T *)dh);
  }
  return 0;
}

#define INST(T)                                                                                  \
  template int simple_gen_proj<T>(const Shape &, const void *, const void *, float *, hipStream_t); \
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
