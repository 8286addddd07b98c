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
// values) or u = h W for the heads its channels fall in -- as dot products
// over d_model.  k_decode_rows reads the weight by rows in 16-byte chunks
// (below); k_decode_one / k_decode, for weights whose rows are not whole
// chunks, give each wave every fourth value, its lanes striding d_model, and a
// fixed xor butterfly adds the lanes (deterministic).  Each thread then
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

// Generator values by weight rows: the block's generator columns are read as
// whole 16-byte chunks of the weight's rows (coalesced: consecutive threads
// take consecutive chunks of one row), every thread walking rows with a
// fixed stride and keeping CE column sums per sequence; the partial sums of
// the threads that share a chunk are added by a fixed xor butterfly within
// each wave, then the four waves' sums in order (deterministic).  The
// per-channel operands (x, the history, the bias) are loaded before the
// generator pass, so their latency overlaps it.  Needs weight rows of whole
// 16-byte chunks and at most 64 chunks of generator columns per block.
template <typename T, int kBG>
__global__ void __launch_bounds__(kThreads)
k_decode_rows(Shape s, const T *__restrict__ h, const T *__restrict__ W, const T *__restrict__ A,
              const T *__restrict__ U, const T *__restrict__ w0, const T *__restrict__ x, T *__restrict__ state,
              T *__restrict__ y) {
  constexpr int CE = 16 / sizeof(T);  // columns per chunk
  constexpr int RB = kBG == 1 ? 16 : 8;  // rows a thread loads at once
  __shared__ float wsum[4][kBG][64 * CE];  // per wave: sums per (chunk, column); at most 64 chunks
  __shared__ float gv[kBG > 1 ? kBG : 1][kBG > 1 ? kMaxG : 1];
  const int b0 = blockIdx.y * kBG;
  const int nb = min(kBG, (int)s.B - b0);  // sequences of this block
  const int c0 = blockIdx.x * kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = (int)s.d, D = (int)s.D, K = s.k;
  const bool lowrank = s.kind == DYNCONV_LOWRANK;
  const int c = c0 + tid;
  const bool cact = c < D;

  // per-channel operands first: x, the k-1 history rows, the bias
  T xr[kBG], hist[kBG][7];
  float bias[8];
#pragma unroll
  for (int r = 0; r < kBG; ++r) {
    const bool ok = cact && r < nb;
    xr[r] = ok ? x[(int64_t)(b0 + r) * D + c] : T(0.f);
#pragma unroll
    for (int m = 0; m < 7; ++m)
      hist[r][m] = ok && m < K - 1 ? state[((int64_t)(b0 + r) * (K - 1) + m) * D + c] : T(0.f);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) bias[j] = w0 && cact && j < K ? to_f32(w0[(int64_t)c * K + j]) : 0.f;
  // generator columns [col0, col0 + nv): all of z (low-rank), or u of the
  // heads e0 .. e1 that channels c0 .. c0+255 fall in (head-wise)
  int e0 = 0, nv = s.rank;
  if (!lowrank) {
    e0 = c0 / s.hd;
    const int e1 = (min(c0 + kThreads, D) - 1) / s.hd;
    nv = s.stat ? 0 : (e1 - e0 + 1) * K;  // static filter: no generator values
  }
  const T *M = lowrank ? A : W;
  const int ldm = s.N;
  const int col0 = lowrank ? 0 : e0 * K;
  if (nv > 0) {
    const int k0 = col0 / CE, cpr = (col0 + nv + CE - 1) / CE - k0;  // chunks per row
    int cp2 = 1;
    while (cp2 < cpr) cp2 *= 2;                                      // <= 64 (nv <= 256)
    const int R = kThreads / cp2;                                    // rows per pass
    const int kc = tid & (cp2 - 1), rg = tid / cp2;
    const bool kact = kc < cpr;
    float acc[kBG][CE];
#pragma unroll
    for (int r = 0; r < kBG; ++r)
#pragma unroll
      for (int e = 0; e < CE; ++e) acc[r][e] = 0.f;
    const T *mrow = M + (int64_t)(k0 + kc) * CE;
    for (int i0 = rg; i0 < d; i0 += RB * R) {
      uint4 mv[RB];
      float hv[kBG][RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int i = i0 + u * R;
        mv[u] = kact && i < d ? *reinterpret_cast<const uint4 *>(mrow + (int64_t)i * ldm) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < kBG; ++r) hv[r][u] = r < nb && i < d ? to_f32(h[(int64_t)(b0 + r) * d + i]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        float mf[CE];
        if constexpr (sizeof(T) == 2) {
          const uint32_t wv[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            mf[2 * q] = __uint_as_float(wv[q] << 16);
            mf[2 * q + 1] = __uint_as_float(wv[q] & 0xffff0000u);
          }
        } else {
          mf[0] = __uint_as_float(mv[u].x);
          mf[1] = __uint_as_float(mv[u].y);
          mf[2] = __uint_as_float(mv[u].z);
          mf[3] = __uint_as_float(mv[u].w);
        }
#pragma unroll
        for (int r = 0; r < kBG; ++r)
#pragma unroll
          for (int e = 0; e < CE; ++e) acc[r][e] = fmaf(hv[r][u], mf[e], acc[r][e]);
      }
    }
    // the lanes of a wave with the same chunk differ in the lane bits >= log2(cp2)
#pragma unroll
    for (int r = 0; r < kBG; ++r)
#pragma unroll
      for (int e = 0; e < CE; ++e)
        for (int m = 32; m >= cp2; m >>= 1) acc[r][e] += __shfl_xor(acc[r][e], m);
    if (lane < cp2 && kact) {
#pragma unroll
      for (int r = 0; r < kBG; ++r)
#pragma unroll
        for (int e = 0; e < CE; ++e) wsum[wave][r][lane * CE + e] = acc[r][e];
    }
    __syncthreads();
    if constexpr (kBG > 1) {  // several sequences: add the waves' sums once, into gv
      for (int o = tid; o < kBG * nv; o += kThreads) {
        const int r = o / nv, v = o - r * nv;
        const int ci = col0 + v - k0 * CE;  // chunk-relative column
        gv[r][v] = ((wsum[0][r][ci] + wsum[1][r][ci]) + wsum[2][r][ci]) + wsum[3][r][ci];
      }
      __syncthreads();
    }
  }
  // generator value v (column col0 + v) of sequence r: the four waves' sums,
  // in order (one sequence: read where they are used, no further barrier)
  const int cof = col0 - (col0 / CE) * CE;  // chunk-relative column of value 0
  auto gval = [&](int r, int v) {
    if constexpr (kBG > 1) return gv[r][v];
    const int ci = cof + v;
    return ((wsum[0][r][ci] + wsum[1][r][ci]) + wsum[2][r][ci]) + wsum[3][r][ci];
  };
  if (!cact) return;

  // taps of channel c for each sequence: the bias, then the generated part
  // (each U value read once for the block's sequences)
  float w[kBG][8];
#pragma unroll
  for (int r = 0; r < kBG; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) w[r][j] = bias[j];
  if (lowrank) {
    for (int j = 0; j < 8; ++j) {
      if (j >= K) break;
      for (int q = 0; q < s.rank; ++q) {
        const float u = to_f32(U[(int64_t)q * D * K + (int64_t)c * K + j]);
#pragma unroll
        for (int r = 0; r < kBG; ++r) w[r][j] = fmaf(gval(r, q), u, w[r][j]);
      }
    }
  } else if (!s.stat) {
    const int hb = (c / s.hd - e0) * K;
#pragma unroll
    for (int r = 0; r < kBG; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < K) w[r][j] += gval(r, hb + j);
  }
#pragma unroll
  for (int r = 0; r < kBG; ++r) {
    if (r >= nb) break;
    const int b = b0 + r;
    const float xc = to_f32(xr[r]);
    float out = fmaf(w[r][0], xc, xc);
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j < K) out = fmaf(w[r][j], to_f32(hist[r][K - 1 - j]), out);
    y[(int64_t)b * D + c] = from_f32<T>(out);
    // drop the oldest row, append x
    if (K > 1) {
      T *st = state + (int64_t)b * (K - 1) * D + c;
#pragma unroll
      for (int m = 0; m < 6; ++m)
        if (m < K - 2) st[(int64_t)m * D] = hist[r][m + 1];
      st[(int64_t)(K - 2) * D] = xr[r];
    }
  }
}

}  // namespace dec

template <typename T>
int decode_step(const Shape &s, const void *h, const void *W, const void *A, const void *U, const void *w0,
                const void *x, void *state, void *y, hipStream_t st) {
  // one sequence per block while that fills the chip, else four (fewer reads of the weights)
  const int64_t slices = ceil_div(s.D, dec::kThreads);
  // weight rows of whole 16-byte chunks, and at most 64 of them per block
  // (bf16: N <= 256 always; fp32: N <= 128): the generator pass by rows
  if (s.stat || (((int64_t)s.N * (int64_t)sizeof(T)) % 16 == 0 && (sizeof(T) == 2 || s.N <= 128))) {
    if (slices * s.B <= 1024)
      hipLaunchKernelGGL((dec::k_decode_rows<T, 1>), dim3((unsigned)slices, (unsigned)s.B), dim3(dec::kThreads), 0,
                         st, s, (const T *)h, (const T *)W, (const T *)A, (const T *)U, (const T *)w0, (const T *)x,
                         (T *)state, (T *)y);
    else
      hipLaunchKernelGGL((dec::k_decode_rows<T, 4>), dim3((unsigned)slices, (unsigned)ceil_div(s.B, 4)),
                         dim3(dec::kThreads), 0, st, s, (const T *)h, (const T *)W, (const T *)A, (const T *)U,
                         (const T *)w0, (const T *)x, (T *)state, (T *)y);
    return 0;
  }
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
