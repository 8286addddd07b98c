// gen_mfma.hip -- the generator projection on bf16 matrix cores.
//
//   out[t, n] = sum_i h[t, i] * M[i, n]     (u = h W head-wise, z = h A low-rank)
//
// The filter is a learned linear map of the current hidden state (gist.science
// Technical Summary of "Dynamic Short Convolutions Improve Transformers",
// Methodology -> Dynamic Short Convolutions, Parameterization); this is that
// map's first (dense) factor, a tall-skinny GEMM: rows = tokens (16k-33k),
// K = d_model (768-2048), N = n_heads*k or rank (16-256).
//
// One wave computes 32 rows x Np columns (Np = N rounded up to 16) with
// v_mfma_f32_16x16x32_bf16: A fragments are 16-byte loads straight from h
// (rows are K-contiguous), B fragments are 16-byte loads from a transposed,
// zero-padded copy Mt[Np][Kp] of the weight that a prep kernel writes into
// the workspace (Kp = K rounded up to 32), so no bounds checks are needed on
// B and the weight stays L2-resident.  When N is small the 4 waves of a block
// split K and reduce through LDS in a fixed order (bitwise deterministic), so
// that the grid still has several blocks per CU.  h is read once: the kernel
// is bound by HBM for N <= 64 and near the MFMA/HBM ridge at N = 256.
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace {

// Mt[n][k] = M[k][n] (zero outside N x K), bf16, n < Np, k < Kp.
__global__ void __launch_bounds__(256)
k_transpose_pad(const bf16 *__restrict__ M, bf16 *__restrict__ Mt, int K, int N, int Kp, int Np) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Np * Kp) return;
  const int n = (int)(idx / Kp), k = (int)(idx - (int64_t)n * Kp);
  Mt[idx] = (n < N && k < K) ? M[(int64_t)k * N + n] : (bf16)0.f;
}

template <int NT, int KS>
__global__ void __launch_bounds__(256)
k_gen_proj_mfma(const bf16 *__restrict__ h, const bf16 *__restrict__ Mt, float *__restrict__ out,
                int64_t M, int K, int Kp, int N) {
  constexpr int RG = 4 / KS;  // row groups of 32 per block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave % RG;   // row group of this wave
  const int ks = wave / RG;   // K slice of this wave
  const int64_t rbase = ((int64_t)blockIdx.x * RG + rg) * 32;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  // rows this lane feeds as A (clamped: rows >= M are computed but never stored)
  const int64_t ra = rbase + lr < M ? rbase + lr : M - 1;
  const int64_t rb = rbase + 16 + lr < M ? rbase + 16 + lr : M - 1;
  const bf16 *ha = h + ra * K;
  const bf16 *hb = h + rb * K;

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = Kp / 32;
  const int per = (steps + KS - 1) / KS;
  const int s0 = ks * per, s1 = min(steps, s0 + per);
  for (int s = s0; s < s1; ++s) {
    const int k = s * 32 + lk;
    bf16x8 a0 = zero_bf16x8(), a1 = zero_bf16x8();
    if (k < K) {  // K is a multiple of 8, so a fragment is all-in or all-out
      a0 = as_bf16x8(*reinterpret_cast<const uint4 *>(ha + k));
      a1 = as_bf16x8(*reinterpret_cast<const uint4 *>(hb + k));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(Mt + (int64_t)(n * 16 + lr) * Kp + k));
      acc[0][n] = mfma16(a0, b, acc[0][n]);
      acc[1][n] = mfma16(a1, b, acc[1][n]);
    }
  }

  if constexpr (KS > 1) {
    // fixed-order reduction of the K slices through LDS
    __shared__ f32x4 red[KS - 1][RG][2][NT][64];
    if (ks > 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[ks - 1][rg][r][n][lane] = acc[r][n];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int q = 0; q < KS - 1; ++q)
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[r][n] += red[q][rg][r][n][lane];
  }

  // D fragment: lane holds D[4*(lane/16) + i][lane%16]
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int col = n * 16 + lr;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = rbase + r * 16 + (lane >> 4) * 4 + i;
        if (row < M) out[row * N + col] = acc[r][n][i];
      }
    }
}

template <int NT>
void launch_nt(const bf16 *h, const bf16 *Mt, float *out, int64_t M, int K, int Kp, int N,
               hipStream_t st) {
  // split K across the block's waves when the row count alone gives too few blocks
  if constexpr (NT <= 4) {
    if (M / 128 < 1024) {
      hipLaunchKernelGGL((k_gen_proj_mfma<NT, 4>), dim3((unsigned)ceil_div(M, 32)), dim3(256), 0, st,
                         h, Mt, out, M, K, Kp, N);
      return;
    }
  }
  {
    hipLaunchKernelGGL((k_gen_proj_mfma<NT, 1>), dim3((unsigned)ceil_div(M, 128)), dim3(256), 0, st, h,
                       Mt, out, M, K, Kp, N);
  }
}

}  // namespace

size_t gen_proj_mfma_ws_bytes(const Shape &s) {
  const int Np = (int)ceil_div(s.N, 16) * 16;
  const int Kp = (int)ceil_div(s.d, 32) * 32;
  return (size_t)Np * Kp * sizeof(bf16);
}

int gen_proj_mfma(const Shape &s, const void *h, const void *M, float *out, void *ws, hipStream_t st) {
  const int N = s.N, K = (int)s.d;
  const int Np = (int)ceil_div(N, 16) * 16;
  const int Kp = (int)ceil_div(K, 32) * 32;
  bf16 *Mt = (bf16 *)ws;
  hipLaunchKernelGGL(k_transpose_pad, dim3((unsigned)ceil_div((int64_t)Np * Kp, 256)), dim3(256), 0, st,
                     (const bf16 *)M, Mt, K, N, Kp, Np);
  const bf16 *hh = (const bf16 *)h;
  const bool tr = trace_begin(DYNCONV_K_GEN_PROJ, st);
  switch (Np / 16) {
#define CASE(nt) \
  case nt: launch_nt<nt>(hh, Mt, out, s.BT, K, Kp, N, st); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: trace_end(tr, st); return DYNCONV_E_LIMIT;
  }
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
