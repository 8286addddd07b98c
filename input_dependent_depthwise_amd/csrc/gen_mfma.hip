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
// A block of 4 waves computes 64 (or 128) rows x Np columns (Np = N rounded
// up to 16) with v_mfma_f32_16x16x32_bf16: A fragments are 16-byte loads
// straight from h (rows are K-contiguous); B comes from a transposed,
// zero-padded copy Mt[Np][Kp] of the weight that a prep kernel writes into
// the workspace (Kp = K rounded up to 32), staged one K-slice at a time in
// LDS and shared by the block's waves, so the weight is read from L2 once
// per block.  Narrow weights (N <= 32) use a K-split variant instead, which
// stages the weight itself in LDS when it fits (no prep kernel).  h is read
// once: the kernel is bound by HBM for N <= 64 and near the MFMA/HBM ridge at
// N = 256.
#include "kernels.h"
#include "bufio.h"
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

// Block: 4 waves = (4 / KS) row groups x KS slices of K; a row group covers
// 16 * RW rows of h, all Np columns.  Per K-step of 32 the block stages the
// KS [Np][32] slices of Mt it needs in LDS (double-buffered, one barrier per
// step); each wave reads its h rows straight from global memory (16-byte A
// fragments) and multiplies them against every column tile of its slice.
// Both operands of the next step are loaded while the current one is used;
// loads are buffer accesses on every path (masked: outside the buffer).  With
// KS = 2 the two K halves meet in LDS at the end in a fixed order.
template <int NT, int RW, int KS>
__global__ void __launch_bounds__(256)
k_gen_proj_mfma(const bf16 *__restrict__ h, const bf16 *__restrict__ Mt, float *__restrict__ out,
                int64_t M, int K, int Kp, int N) {
  constexpr int NP = NT * 16;
  constexpr int BROW = 40;                       // LDS row of the B slice: 32 k + pad (bf16)
  constexpr int SCH = NP * 4;                    // 16-byte chunks of one [NP][32] slice
  constexpr int CPT = (KS * SCH + 255) / 256;    // chunks per thread
  constexpr int RG = 4 / KS;                     // row groups
  constexpr int ROWS = RG * 16 * RW;             // rows per block
  __shared__ __attribute__((aligned(16))) bf16 bs[2][KS][NP * BROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RG, ks = wave / RG;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int64_t rblk = (int64_t)blockIdx.x * ROWS;
  const int nrows = (int)min<int64_t>(ROWS, M - rblk);
  const auto rh = make_rsrc(h + rblk * K, (uint32_t)((int64_t)nrows * K * 2));
  const auto rb = make_rsrc(Mt, (uint32_t)((int64_t)NP * Kp * 2));

  f32x4 acc[RW][NT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = Kp / 32;
  const int S = (steps + KS - 1) / KS;  // K-steps per slice (the last slice may run past K: zeros)
  uint4 bpre[CPT];
  bf16x8 apre[RW];
  auto load = [&](int st) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = tid + c * 256;
      const int sl = e / SCH, e2 = e - sl * SCH;
      const int n = e2 >> 2, kc = (e2 & 3) * 8;
      const int kst = sl * S + st;
      const uint32_t off = ((KS * SCH) % 256 == 0 || e < KS * SCH) && kst < steps
                               ? (uint32_t)(((int64_t)n * Kp + kst * 32 + kc) * 2)
                               : kOutside;
      bpre[c] = buf_load16(rb, off);
    }
    const int k = (ks * S + st) * 32 + lk;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int row = (rg * RW + r) * 16 + lr;  // rows past the matrix read zeros and are never stored
      apre[r] = as_bf16x8(buf_load16(rh, k < K ? (uint32_t)((row * K + k) * 2) : kOutside));
    }
  };
  load(0);
  for (int st = 0; st < S; ++st) {
    const int buf = st & 1;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = tid + c * 256;
      if ((KS * SCH) % 256 == 0 || e < KS * SCH) {
        const int sl = e / SCH, e2 = e - sl * SCH;
        *reinterpret_cast<uint4 *>(&bs[buf][sl][(e2 >> 2) * BROW + (e2 & 3) * 8]) = bpre[c];
      }
    }
    bf16x8 a[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) a[r] = apre[r];
    __syncthreads();
    load(st + 1);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(&bs[buf][ks][(n * 16 + lr) * BROW + lk]));
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[r][n] = mfma16(a[r], b, acc[r][n]);
    }
  }

  if constexpr (KS == 2) {
    // the second K half hands its sums to the first through LDS
    f32x4 *red = reinterpret_cast<f32x4 *>(&bs[0][0][0]);
    static_assert(sizeof(bs) >= RG * RW * NT * 64 * sizeof(f32x4), "reduction buffer");
    __syncthreads();
    if (ks == 1) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[((rg * RW + r) * NT + n) * 64 + lane] = acc[r][n];
    }
    __syncthreads();
    if (ks == 1) return;
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[r][n] += red[((rg * RW + r) * NT + n) * 64 + lane];
  }

  // D fragment: lane holds D[4*(lane/16) + i][lane%16]
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int col = n * 16 + lr;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = rblk + (rg * RW + r) * 16 + (lane >> 4) * 4 + i;
        if (row < M) out[row * N + col] = acc[r][n][i];
      }
    }
}

// Narrow weights (N <= 32): the B slice is too small to be worth staging,
// and one row tile per wave would leave the chip mostly idle.  A block is 4
// waves over the same 32 rows, each summing a quarter of K; B fragments are
// read straight from the (L2-resident) padded weight.  Four K-steps of loads
// are issued before their MFMAs so that enough of h is in flight.  The K
// quarters are reduced through LDS in a fixed order (bitwise deterministic).
template <int NT>
__global__ void __launch_bounds__(256)
k_gen_proj_ksplit(const bf16 *__restrict__ h, const bf16 *__restrict__ Mt, float *__restrict__ out,
                  int64_t M, int K, int Kp, int N) {
  constexpr int KS = 4, U = 4;
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int64_t rbase = (int64_t)blockIdx.x * 32;
  const int64_t ra = rbase + lr < M ? rbase + lr : M - 1;  // rows >= M are never stored
  const int64_t rb = rbase + 16 + lr < M ? rbase + 16 + lr : M - 1;
  const bf16 *ha = h + ra * K + lk;
  const bf16 *hb = h + rb * K + lk;
  const bf16 *mb = Mt + (int64_t)lr * Kp + lk;

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = Kp / 32, full = K / 32;
  const int per = (steps + KS - 1) / KS;
  const int s0 = ks * per, s1 = min(steps, s0 + per);
  const int s1f = min(s1, full);  // steps whose 32 k all lie below K
  int s = s0;
  for (; s + U <= s1f; s += U) {
    bf16x8 a0[U], a1[U], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32;
      a0[u] = as_bf16x8(*reinterpret_cast<const uint4 *>(ha + k));
      a1[u] = as_bf16x8(*reinterpret_cast<const uint4 *>(hb + k));
#pragma unroll
      for (int n = 0; n < NT; ++n)
        b[u][n] = as_bf16x8(*reinterpret_cast<const uint4 *>(mb + (int64_t)n * 16 * Kp + k));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[0][n] = mfma16(a0[u], b[u][n], acc[0][n]);
        acc[1][n] = mfma16(a1[u], b[u][n], acc[1][n]);
      }
  }
  for (; s < s1; ++s) {
    const int k = s * 32;
    bf16x8 a0 = zero_bf16x8(), a1 = zero_bf16x8();
    if (k + lk < K) {  // K is a multiple of 8: a fragment is all-in or all-out
      a0 = as_bf16x8(*reinterpret_cast<const uint4 *>(ha + k));
      a1 = as_bf16x8(*reinterpret_cast<const uint4 *>(hb + k));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(mb + (int64_t)n * 16 * Kp + k));
      acc[0][n] = mfma16(a0, b, acc[0][n]);
      acc[1][n] = mfma16(a1, b, acc[1][n]);
    }
  }

  __shared__ f32x4 red[KS - 1][2][NT][64];
  if (ks > 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) red[ks - 1][r][n][lane] = acc[r][n];
  }
  __syncthreads();
  if (ks > 0) return;
#pragma unroll
  for (int q = 0; q < KS - 1; ++q)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[r][n] += red[q][r][n][lane];
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

// Narrow weights with N a multiple of 8 whose whole (row-padded) copy fits
// in 64 KB of LDS: as k_gen_proj_ksplit, but each block first stages the
// weight itself in LDS, rows k as given (Np columns, zeros past N), and every
// B fragment is two transposed LDS reads (read_tr16: four k of one column
// per read), so no transposed copy and no prep kernel are needed.  Bank
// spread: with 16 columns, the 128-byte blocks of four rows are stored at
// position b ^ ((b >> 1) & 1); with 32, the two 32-byte halves of row k at
// half h ^ ((k >> 3) & 1).  Either way the two token groups of a 32-lane
// pass (8 rows apart) read disjoint banks.
constexpr size_t kNarrowLds = 48 * 1024;  // staged weight (the K-quarter sums take 12 KB more)
template <int NT>
__device__ __forceinline__ int wrow_off(int k, int half) {
  if constexpr (NT == 1) {
    const int b = k >> 2;
    return ((b ^ ((b >> 1) & 1)) << 7) + ((k & 3) << 5) + half * 16;
  } else {
    return (k << 6) + (((half >> 1) ^ ((k >> 3) & 1)) << 5) + (half & 1) * 16;
  }
}

template <int NT>
__global__ void __launch_bounds__(256)
k_gen_proj_narrow(const bf16 *__restrict__ h, const bf16 *__restrict__ Mw, float *__restrict__ out,
                  int64_t M, int K, int Kp, int N) {
  constexpr int KS = 4, U = 4;
  constexpr int CPR = NT * 2;  // 16-byte chunks per staged row
  extern __shared__ __attribute__((aligned(16))) unsigned char wl[];  // Kp rows x 32*NT bytes
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int64_t rbase = (int64_t)blockIdx.x * 32;

  const int64_t ra = rbase + lr < M ? rbase + lr : M - 1;  // rows >= M are never stored
  const int64_t rb = rbase + 16 + lr < M ? rbase + 16 + lr : M - 1;
  const bf16 *ha = h + ra * K + lk;
  const bf16 *hb = h + rb * K + lk;
  const int steps = Kp / 32, full = K / 32;
  const int per = (steps + KS - 1) / KS;
  const int s0 = ks * per, s1 = min(steps, s0 + per);
  const int s1f = min(s1, full);  // steps whose 32 k all lie below K
  bf16x8 a0[U], a1[U];
  auto load_a = [&](int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (st + u) * 32;
      a0[u] = as_bf16x8(*reinterpret_cast<const uint4 *>(ha + k));
      a1[u] = as_bf16x8(*reinterpret_cast<const uint4 *>(hb + k));
    }
  };
  // the first h fragments, and those of the tail (the fewer than U steps
  // after the full groups, the last one possibly partial), are in flight
  // while the weight is staged
  int s = s0;
  if (s + U <= s1f) load_a(s);
  const int sg = s0 + max(0, s1f - s0) / U * U;  // first tail step
  bf16x8 t0[U], t1[U];
#pragma unroll
  for (int q = 0; q < U; ++q) {
    const int k = (sg + q) * 32;
    t0[q] = t1[q] = zero_bf16x8();
    if (sg + q < s1 && k + lk < K) {  // K is a multiple of 8: a fragment is all-in or all-out
      t0[q] = as_bf16x8(*reinterpret_cast<const uint4 *>(ha + k));
      t1[q] = as_bf16x8(*reinterpret_cast<const uint4 *>(hb + k));
    }
  }

  // stage the weight: chunk e -> row k = e / CPR, 8 columns 8c .. 8c+7
  // (rows past K and columns past N read zeros from outside the buffer)
  {
    const auto rw = make_rsrc(Mw, (uint32_t)((int64_t)K * N * 2));
    const int nch = Kp * CPR;
    for (int e = threadIdx.x; e < nch; e += 256) {
      const int k = e / CPR, c = e - k * CPR;
      const uint32_t off = 8 * c < N ? (uint32_t)(k * N + 8 * c) * 2u : kOutside;
      *reinterpret_cast<uint4 *>(wl + wrow_off<NT>(k, c)) = buf_load16(rw, off);
    }
  }
  __syncthreads();

  // B fragment (K-step at k, column tile n): lane lr of token group g reads
  // row k + 8g + 4q + lr/4 (q = 0, 1), columns 16n + 4(lr%4) .. +3, i.e.
  // chunk 2n + (lr%4)/2 of the row, byte 8(lr%2) of it; it receives
  // B[k + 8g + i][16n + lr], i = 4q .. 4q+3
  auto bfrag = [&](int k, int n) -> bf16x8 {
    const int r0 = k + lk + (lr >> 2), c = 2 * n + ((lr & 3) >> 1), b8 = (lr & 1) * 8;
    const uint2 lo = read_tr16(wl + wrow_off<NT>(r0, c) + b8);
    const uint2 hi = read_tr16(wl + wrow_off<NT>(r0 + 4, c) + b8);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // groups of U K-steps; the next group's h loads are issued behind the
  // current group's MFMAs
  for (; s + U <= s1f; s += U) {
    bf16x8 b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n) b[u][n] = bfrag((s + u) * 32, n);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[0][n] = mfma16(a0[u], b[u][n], acc[0][n]);
        acc[1][n] = mfma16(a1[u], b[u][n], acc[1][n]);
      }
    if (s + 2 * U <= s1f) load_a(s + U);
  }
#pragma unroll
  for (int q = 0; q < U; ++q) {
    if (sg + q >= s1) break;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = bfrag((sg + q) * 32, n);
      acc[0][n] = mfma16(t0[q], b, acc[0][n]);
      acc[1][n] = mfma16(t1[q], b, acc[1][n]);
    }
  }

  __shared__ f32x4 red[KS - 1][2][NT][64];
  if (ks > 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) red[ks - 1][r][n][lane] = acc[r][n];
  }
  __syncthreads();
  if (ks > 0) return;
#pragma unroll
  for (int q = 0; q < KS - 1; ++q)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[r][n] += red[q][r][n][lane];
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
  if constexpr (NT <= 2) {
    hipLaunchKernelGGL((k_gen_proj_ksplit<NT>), dim3((unsigned)ceil_div(M, 32)), dim3(256), 0, st, h, Mt,
                       out, M, K, Kp, N);
  } else {
    // about two blocks per CU: 64-row blocks when the rows give 512 of them,
    // else 32-row blocks with K split in two
    if (M >= 512 * 64) {
      hipLaunchKernelGGL((k_gen_proj_mfma<NT, 1, 1>), dim3((unsigned)ceil_div(M, 64)), dim3(256), 0, st, h, Mt,
                         out, M, K, Kp, N);
    } else {
      hipLaunchKernelGGL((k_gen_proj_mfma<NT, 1, 2>), dim3((unsigned)ceil_div(M, 32)), dim3(256), 0, st, h, Mt,
                         out, M, K, Kp, N);
    }
  }
}

}  // namespace

size_t gen_proj_mfma_ws_bytes(const Shape &s) {
  if (gen_proj_wide_ok(s)) return 0;
  const int Np = (int)ceil_div(s.N, 16) * 16;
  const int Kp = (int)ceil_div(s.d, 32) * 32;
  return (size_t)Np * Kp * sizeof(bf16);
}

int gen_proj_mfma(const Shape &s, const void *h, const void *M, float *out, void *ws, hipStream_t st) {
  const int N = s.N, K = (int)s.d;
  const int Np = (int)ceil_div(N, 16) * 16;
  const int Kp = (int)ceil_div(K, 32) * 32;
  const bf16 *hh = (const bf16 *)h;
  // narrow weights that fit in LDS: staged from the weight itself, no prep kernel
  if (Np <= 32 && N % 8 == 0 && (size_t)Kp * Np * 2 <= kNarrowLds) {
    const bool tr = trace_begin(DYNCONV_K_GEN_PROJ, st);
    const dim3 grid((unsigned)ceil_div(s.BT, 32)), block(256);
    const size_t lds = (size_t)Kp * Np * 2;
    if (Np == 16)
      hipLaunchKernelGGL((k_gen_proj_narrow<1>), grid, block, lds, st, hh, (const bf16 *)M, out, s.BT, K, Kp, N);
    else
      hipLaunchKernelGGL((k_gen_proj_narrow<2>), grid, block, lds, st, hh, (const bf16 *)M, out, s.BT, K, Kp, N);
    trace_end(tr, st);
    return 0;
  }
  if (gen_proj_wide_ok(s)) return gen_proj_wide(s, h, M, out, st);
  bf16 *Mt = (bf16 *)ws;
  hipLaunchKernelGGL(k_transpose_pad, dim3((unsigned)ceil_div((int64_t)Np * Kp, 256)), dim3(256), 0, st,
                     (const bf16 *)M, Mt, K, N, Kp, Np);
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
