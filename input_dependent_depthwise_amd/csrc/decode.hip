// decode.hip -- one decoding step of the dynamic short convolution: a new
// token for each of B sequences, with the last k-1 rows of x of every
// sequence kept by the caller between steps.
//
// The layer (gist.science Technical Summary of "Dynamic Short Convolutions
// Improve Transformers", Methodology -> Dynamic Short Convolutions:
// Mechanism, Parameterization) at the newest position t of a sequence:
//   y[c] = x_t[c] + sum_{j<k} w_t[c,j] x_{t-j}[c],  w_t from h_t as in the forward,
// where x_{t-j} for j >= 1 comes from the history (zero before the start of
// the sequence: a new sequence starts from a zeroed history).  The pages
// note that inference is left unoptimised (atlas.scime.ai, Limitations);
// this step is what a decoder runs per token.
//
// Block: one or four sequences (four once there are enough blocks without
// it) and 256 channels, one channel per thread.  The block
// first computes the generator values its channels use -- z = h A (all rank
// values) or u = h W for the heads its channels fall in -- each a dot product
// over d_model: a wave takes every fourth value, its lanes stride d_model,
// and a fixed xor butterfly adds the lanes (deterministic).  Each thread then
// forms its channel's k taps in fp32 for the block's sequences (every weight
// value it reads serves all of them), convolves, writes y and shifts the
// history of its channel in place (it reads all of its rows before writing).
// The step is latency-bound for decoding batch sizes: it reads the generator
// weights once per block (from L2 after the first blocks) and B rows of h, x
// and the history.
#include "kernels.h"

namespace dynconv {
namespace dec {

constexpr int kThreads = 256;
constexpr int kMaxG = 256;  // generator values per sequence a block computes at most (n_heads*k, rank <= 256)

// One sequence per block (small batches: enough blocks without grouping).
template <typename T>
__global__ void __launch_bounds__(kThreads)
k_decode_one(Shape s, const T *__restrict__ h, const T *__restrict__ W, const T *__restrict__ A,
             const T *__restrict__ U, const T *__restrict__ w0, const T *__restrict__ x, T *__restrict__ state,
             T *__restrict__ y) {
  __shared__ float gv[kMaxG];
  const int b = blockIdx.y;
  const int c0 = blockIdx.x * kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = (int)s.d, D = (int)s.D, K = s.k;
  const bool lowrank = s.kind == DYNCONV_LOWRANK;
  const T *hb = h + (int64_t)b * d;
  int e0 = 0, nv = s.rank;
  if (!lowrank) {
    e0 = c0 / s.hd;
    const int e1 = (min(c0 + kThreads, D) - 1) / s.hd;
    nv = s.stat ? 0 : (e1 - e0 + 1) * K;  // static filter: no generator values
  }
  const T *M = lowrank ? A : W;
  const int ldm = s.N;
  const int col0 = lowrank ? 0 : e0 * K;
  for (int v = wave; v < nv; v += 4) {
    const T *mc = M + col0 + v;
    float acc = 0.f;
    int i = lane;
    for (; i + 192 < d; i += 256) {  // four independent loads per pass
      const float a0 = to_f32(hb[i]) * to_f32(mc[(int64_t)i * ldm]);
      const float a1 = to_f32(hb[i + 64]) * to_f32(mc[(int64_t)(i + 64) * ldm]);
      const float a2 = to_f32(hb[i + 128]) * to_f32(mc[(int64_t)(i + 128) * ldm]);
      const float a3 = to_f32(hb[i + 192]) * to_f32(mc[(int64_t)(i + 192) * ldm]);
      acc += a0;
      acc += a1;
      acc += a2;
      acc += a3;
    }
    for (; i < d; i += 64) acc = fmaf(to_f32(hb[i]), to_f32(mc[(int64_t)i * ldm]), acc);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) gv[v] = acc;
  }
  __syncthreads();
  const int c = c0 + tid;
  if (c >= D) return;
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= K) break;
    float v;
    if (lowrank) {
      v = 0.f;
      for (int q = 0; q < s.rank; ++q) v = fmaf(gv[q], to_f32(U[(int64_t)q * D * K + (int64_t)c * K + j]), v);
    } else {
      v = s.stat ? 0.f : gv[(c / s.hd - e0) * K + j];
    }
    w[j] = w0 ? v + to_f32(w0[(int64_t)c * K + j]) : v;
  }
  T *st = K > 1 ? state + (int64_t)b * (K - 1) * D + c : nullptr;
  T hist[7];
#pragma unroll
  for (int m = 0; m < 7; ++m)
    if (m < K - 1) hist[m] = st[(int64_t)m * D];
  const T xr = x[(int64_t)b * D + c];
  const float xc = to_f32(xr);
  float out = fmaf(w[0], xc, xc);
#pragma unroll
  for (int j = 1; j < 8; ++j)
    if (j < K) out = fmaf(w[j], to_f32(hist[K - 1 - j]), out);
  y[(int64_t)b * D + c] = from_f32<T>(out);
#pragma unroll
  for (int m = 0; m < 6; ++m)
    if (m < K - 2) st[(int64_t)m * D] = hist[m + 1];
  if (K > 1) st[(int64_t)(K - 2) * D] = xr;
}

// kBG sequences per block: each generator weight value a block reads serves all of them
template <typename T, int kBG>
__global__ void __launch_bounds__(kThreads)
k_decode(Shape s, const T *__restrict__ h, const T *__restrict__ W, const T *__restrict__ A,
         const T *__restrict__ U, const T *__restrict__ w0, const T *__restrict__ x, T *__restrict__ state,
         T *__restrict__ y) {
  __shared__ float gv[kBG][kMaxG];
  const int b0 = blockIdx.y * kBG;
  const int nb = min(kBG, (int)s.B - b0);  // sequences of this block
  const int c0 = blockIdx.x * kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = (int)s.d, D = (int)s.D, K = s.k;
  const bool lowrank = s.kind == DYNCONV_LOWRANK;

  // generator values of each sequence: low-rank z[q] (q < rank); head-wise
  // u[e*k+j] of the heads e0 .. e1 that channels c0 .. c0+255 fall in,
  // stored from e0 on.  A wave takes every fourth value; its lanes stride
  // d_model, read the weight once for all the block's sequences, and a fixed
  // xor butterfly adds them.
  int e0 = 0, nv = s.rank;
  if (!lowrank) {
    e0 = c0 / s.hd;
    const int e1 = (min(c0 + kThreads, D) - 1) / s.hd;
    nv = s.stat ? 0 : (e1 - e0 + 1) * K;  // static filter: no generator values
  }
  const T *M = lowrank ? A : W;
  const int ldm = s.N;                    // row length of A (rank) or W (n_heads*k)
  const int col0 = lowrank ? 0 : e0 * K;  // first column used
  for (int v = wave; v < nv; v += 4) {
    const T *mc = M + col0 + v;
    float acc[kBG];
#pragma unroll
    for (int r = 0; r < kBG; ++r) acc[r] = 0.f;
    int i = lane;
    for (; i + 192 < d; i += 256) {  // four rows of the weight per pass, loads issued together
      float m[4], hv[kBG][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) m[u] = to_f32(mc[(int64_t)(i + 64 * u) * ldm]);
#pragma unroll
      for (int r = 0; r < kBG; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) hv[r][u] = r < nb ? to_f32(h[(int64_t)(b0 + r) * d + i + 64 * u]) : 0.f;
#pragma unroll
      for (int r = 0; r < kBG; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[r] = fmaf(hv[r][u], m[u], acc[r]);
    }
    for (; i < d; i += 64) {
      const float m = to_f32(mc[(int64_t)i * ldm]);
#pragma unroll
      for (int r = 0; r < kBG; ++r)
        if (r < nb) acc[r] = fmaf(to_f32(h[(int64_t)(b0 + r) * d + i]), m, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kBG; ++r) {
      float a = acc[r];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m);
      if (lane == 0) gv[r][v] = a;
    }
  }
  __syncthreads();

  const int c = c0 + tid;
  if (c >= D) return;
  // taps of channel c for each sequence: generated part (each U value read
  // once for the block's sequences), then the bias
  float w[kBG][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= K) break;
#pragma unroll
    for (int r = 0; r < kBG; ++r) w[r][j] = 0.f;
    if (lowrank) {
      for (int q = 0; q < s.rank; ++q) {
        const float u = to_f32(U[(int64_t)q * D * K + (int64_t)c * K + j]);
#pragma unroll
        for (int r = 0; r < kBG; ++r) w[r][j] = fmaf(gv[r][q], u, w[r][j]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < kBG; ++r) w[r][j] = s.stat ? 0.f : gv[r][(c / s.hd - e0) * K + j];
    }
    if (w0) {
      const float bias = to_f32(w0[(int64_t)c * K + j]);
#pragma unroll
      for (int r = 0; r < kBG; ++r) w[r][j] += bias;
    }
  }
#pragma unroll
  for (int r = 0; r < kBG; ++r) {
    if (r >= nb) break;
    const int b = b0 + r;
    // history rows m = 0 .. k-2 of channel c: row k-1-j is the token j back
    T *st = K > 1 ? state + (int64_t)b * (K - 1) * D + c : nullptr;
    T hist[7];
#pragma unroll
    for (int m = 0; m < 7; ++m)
      if (m < K - 1) hist[m] = st[(int64_t)m * D];
    const T xr = x[(int64_t)b * D + c];
    const float xc = to_f32(xr);
    float out = fmaf(w[r][0], xc, xc);
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j < K) out = fmaf(w[r][j], to_f32(hist[K - 1 - j]), out);
    y[(int64_t)b * D + c] = from_f32<T>(out);
    // drop the oldest row, append x
#pragma unroll
    for (int m = 0; m < 6; ++m)
      if (m < K - 2) st[(int64_t)m * D] = hist[m + 1];
    if (K > 1) st[(int64_t)(K - 2) * D] = xr;
  }
}

}  // namespace dec

template <typename T>
int decode_step(const Shape &s, const void *h, const void *W, const void *A, const void *U, const void *w0,
                const void *x, void *state, void *y, hipStream_t st) {
  // one sequence per block while that fills the chip, else four (fewer reads of the weights)
  const int64_t slices = ceil_div(s.D, dec::kThreads);
  if (slices * s.B <= 1024) {
    hipLaunchKernelGGL((dec::k_decode_one<T>), dim3((unsigned)slices, (unsigned)s.B), dim3(dec::kThreads), 0, st, s,
                       (const T *)h, (const T *)W, (const T *)A, (const T *)U, (const T *)w0, (const T *)x,
                       (T *)state, (T *)y);
  } else {
    hipLaunchKernelGGL((dec::k_decode<T, 4>), dim3((unsigned)slices, (unsigned)ceil_div(s.B, 4)),
                       dim3(dec::kThreads), 0, st, s, (const T *)h, (const T *)W, (const T *)A, (const T *)U,
                       (const T *)w0, (const T *)x, (T *)state, (T *)y);
  }
  return 0;
}

template int decode_step<float>(const Shape &, const void *, const void *, const void *, const void *,
                                const void *, const void *, void *, void *, hipStream_t);
template int decode_step<bf16>(const Shape &, const void *, const void *, const void *, const void *,
                               const void *, const void *, void *, void *, hipStream_t);

}  // namespace dynconv
