// gen_bwd.hip -- gradients into the generator, bf16 path.
//
// The generator's first factor is a linear map of the hidden state (u = h W
// head-wise, z = h A low-rank; gist.science Technical Summary of "Dynamic
// Short Convolutions Improve Transformers", Methodology -> Dynamic Short
// Convolutions, Parameterization).  Given g = du (or dz) from the fused conv
// backward:
//   dh[t, i]  = sum_n g[t, n] M[i, n]          (M = W or A)
//   dM[i, n]  = sum_t h[t, i] g[t, n]
// Kernels:
//   k_combine  g = fixed-order sum of the conv kernel's per-slice partials,
//              written once as bf16 [BT, Np] (the MFMA operand precision);
//   k_dh       dh^T tiles = M . g^T on v_mfma_f32_32x32x16_bf16, blocks of one
//              32-token tile x 128 rows of d, mapped so that all row blocks of
//              a token tile run on the same XCD (its g tile stays in that L2);
//   k_dM       per (64-row chunk of d, token range) partials of h^T g on
//              v_mfma_f32_16x16x32_bf16, both operands staged transposed in
//              LDS (token-contiguous);
//   k_finalize fixed-order sums of all weight-gradient partials (dU, dw0, dM).
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace gbwd {

// g[t, n] for n < N (zero-padded to Np), bf16; four columns per thread.  The
// slice partials are loaded 6 at a time ahead of the adds, which stay in
// slice order (fixed-order sums).
__global__ void __launch_bounds__(256)
k_combine(Shape s, const float *__restrict__ gpart, int n_slices, int R, int Dt, int Np,
          bf16 *__restrict__ g) {
  const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (idx >= s.BT * Np) return;
  const int64_t t = idx / Np;
  const int n0 = (int)(idx - t * Np);  // Np is a multiple of 16: the four columns share a row
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (s.kind == DYNCONV_LOWRANK) {
    if (n0 + 4 <= s.N && R % 4 == 0) {
      const float *src = gpart + t * R + n0;
      const int64_t stride = s.BT * R;
      int d = 0;
      for (; d + 6 <= n_slices; d += 6) {
        float4 a[6];
#pragma unroll
        for (int u = 0; u < 6; ++u) a[u] = *reinterpret_cast<const float4 *>(src + (d + u) * stride);
#pragma unroll
        for (int u = 0; u < 6; ++u) v[0] += a[u].x, v[1] += a[u].y, v[2] += a[u].z, v[3] += a[u].w;
      }
      for (; d < n_slices; ++d) {
        const float4 a = *reinterpret_cast<const float4 *>(src + d * stride);
        v[0] += a.x, v[1] += a.y, v[2] += a.z, v[3] += a.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n0 + c < s.N)
          for (int d = 0; d < n_slices; ++d) v[c] += gpart[((int64_t)d * s.BT + t) * R + n0 + c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int n = n0 + c;
      if (n >= s.N) continue;
      const int e = n / s.k, j = n - e * s.k;
      const int d0 = (int)((int64_t)e * s.hd / Dt), d1 = (int)(((int64_t)(e + 1) * s.hd - 1) / Dt);
      for (int d = d0; d <= d1; ++d) {
        const int slot = e - (int)((int64_t)d * Dt / s.hd);
        v[c] += gpart[((int64_t)d * s.BT + t) * R + slot * s.k + j];
      }
    }
  }
  uint2 o;
  o.x = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[1]) << 16);
  o.y = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[3]) << 16);
  *reinterpret_cast<uint2 *>(g + idx) = o;
}

// Mp[i, n] = M[i, n] zero-padded to Np columns (bf16).
__global__ void __launch_bounds__(256)
k_pad_cols(const bf16 *__restrict__ M, bf16 *__restrict__ Mp, int64_t rows, int N, int Np) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * Np) return;
  const int64_t i = idx / Np;
  const int n = (int)(idx - i * Np);
  Mp[idx] = n < N ? M[i * N + n] : (bf16)0.f;
}

// dh^T[i, t] = sum_n Mp[i, n] g[t, n].  Block: 4 waves x 32 rows of d, one
// 32-token tile.  Lane l holds rows 8b + 4(l/32) + r, token l%32.
template <int KS>
__global__ void __launch_bounds__(256)
k_dh(const bf16 *__restrict__ g, const bf16 *__restrict__ Mp, bf16 *__restrict__ dh, int64_t BT,
     int d, int Np, int n_ib, int Mcols) {
  // XCD-aware mapping: blocks go round-robin over 8 XCDs; keep a token tile's
  // row blocks on one XCD.
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int tile = (slot / n_ib) * 8 + xcd, ib = slot % n_ib;
  const int64_t t0 = (int64_t)tile * 32;
  if (t0 >= BT) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int i0 = ib * 128 + wave * 32;
  if (i0 >= d) return;
  const int64_t t = t0 + tl;
  const int ia = min(i0 + tl, d - 1);
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int n = ks * 16 + hh * 8;
    // Mp has Mcols columns: Np (a padded copy) or N itself when N % 8 == 0, so
    // that each 8-column chunk is all in or all out
    const bf16x8 a = n < Mcols ? as_bf16x8(*reinterpret_cast<const uint4 *>(Mp + (int64_t)ia * Mcols + n))
                               : zero_bf16x8();
    const bf16x8 bb = t < BT ? as_bf16x8(*reinterpret_cast<const uint4 *>(g + t * Np + n)) : zero_bf16x8();
    acc = mfma32(a, bb, acc);
  }
  if (t >= BT) return;
#pragma unroll
  for (int bq = 0; bq < 4; ++bq) {
    const int i = i0 + 8 * bq + 4 * hh;
    if (i >= d) continue;  // d is a multiple of 8, so i..i+3 are all in or all out
    const bf16 v0 = (bf16)acc[4 * bq], v1 = (bf16)acc[4 * bq + 1], v2 = (bf16)acc[4 * bq + 2],
               v3 = (bf16)acc[4 * bq + 3];
    uint2 raw;
    raw.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
    raw.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
    *reinterpret_cast<uint2 *>(dh + t * d + i) = raw;
  }
}

constexpr int kRowB = 80;  // 32 tokens of bf16, padded

// dMp[range][i, n] = sum over the range's tokens of h[t, i] g[t, n].
// Block: 64 rows of d (wave w: rows 16w..16w+15) x all Np columns.
template <int NB>
__global__ void __launch_bounds__(256)
k_dM(const bf16 *__restrict__ h, const bf16 *__restrict__ g, float *__restrict__ dMp, int64_t BT,
     int d, int N, int Np, int tpb, int n_tiles) {
  __shared__ __attribute__((aligned(16))) unsigned char ht[64 * kRowB];
  __shared__ __attribute__((aligned(16))) unsigned char gtt[NB * 16 * kRowB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = blockIdx.x * 64;
  const int tile_lo = blockIdx.y * tpb, tile_hi = min(n_tiles, tile_lo + tpb);
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    const int64_t t0 = (int64_t)tile * 32;
    __syncthreads();
    // h tile transposed: thread -> (token tt, 8 consecutive rows i)
    {
      const int tt = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;
      const int64_t row = t0 + tt;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (row < BT && i0 + c8 < d) raw = *reinterpret_cast<const uint4 *>(h + row * d + i0 + c8);
      const uint16_t *hv = reinterpret_cast<const uint16_t *>(&raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<uint16_t *>(ht + (c8 + e) * kRowB + tt * 2) = hv[e];
    }
    // g tile transposed: thread -> (token, 8 consecutive columns)
    for (int e = threadIdx.x; e < 32 * (Np / 8); e += 256) {
      const int tt = e / (Np / 8), n8 = (e - tt * (Np / 8)) * 8;
      const int64_t row = t0 + tt;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (row < BT) raw = *reinterpret_cast<const uint4 *>(g + row * Np + n8);
      const uint16_t *gv = reinterpret_cast<const uint16_t *>(&raw);
#pragma unroll
      for (int q = 0; q < 8; ++q) *reinterpret_cast<uint16_t *>(gtt + (n8 + q) * kRowB + tt * 2) = gv[q];
    }
    __syncthreads();
    const bf16x8 a = as_bf16x8(
        *reinterpret_cast<const uint4 *>(ht + (wave * 16 + (lane & 15)) * kRowB + (lane >> 4) * 16));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 b = as_bf16x8(
          *reinterpret_cast<const uint4 *>(gtt + (nb * 16 + (lane & 15)) * kRowB + (lane >> 4) * 16));
      acc[nb] = mfma16(a, b, acc[nb]);
    }
  }
  // D fragment: lane holds D[4(l/16) + r][l%16] of each 16x16 block
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wave * 16 + (lane >> 4) * 4 + r;
      const int n = nb * 16 + (lane & 15);
      if (i < d && n < N) dMp[((int64_t)blockIdx.y * d + i) * N + n] = acc[nb][r];
    }
}

// out[e] = sum_p part[p][e] for e < n, p < np (fixed order), for up to three
// independent reductions packed into one launch.
struct Red {
  const float *part;
  float *out;
  int64_t n;
  int np;
};

// Four consecutive outputs per thread; the partial rows are loaded 8 at a
// time ahead of the adds, which stay in partial order (fixed-order sums).
__global__ void __launch_bounds__(256) k_finalize(Red r0, Red r1, Red r2) {
  int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t q0 = (r0.n + 3) / 4 * 4, q1 = (r1.n + 3) / 4 * 4, q2 = (r2.n + 3) / 4 * 4;
  const Red *r;
  if (idx < q0) {
    r = &r0;
  } else if ((idx -= q0) < q1) {
    r = &r1;
  } else if ((idx -= q1) < q2) {
    r = &r2;
  } else {
    return;
  }
  if (!r->out || idx >= r->n) return;
  const int64_t n = r->n;
  if (idx + 4 <= n && n % 4 == 0) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    const float *src = r->part + idx;
    int p = 0;
    for (; p + 8 <= r->np; p += 8) {
      float4 a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = *reinterpret_cast<const float4 *>(src + (int64_t)(p + u) * n);
#pragma unroll
      for (int u = 0; u < 8; ++u) v.x += a[u].x, v.y += a[u].y, v.z += a[u].z, v.w += a[u].w;
    }
    for (; p < r->np; ++p) {
      const float4 a = *reinterpret_cast<const float4 *>(src + (int64_t)p * n);
      v.x += a.x, v.y += a.y, v.z += a.z, v.w += a.w;
    }
    *reinterpret_cast<float4 *>(r->out + idx) = v;
  } else {
    for (int64_t e = idx; e < idx + 4 && e < n; ++e) {
      float v = 0.f;
      for (int p = 0; p < r->np; ++p) v += r->part[(int64_t)p * n + e];
      r->out[e] = v;
    }
  }
}

}  // namespace gbwd

GenBwdLayout gen_bwd_layout(const Shape &s) {
  GenBwdLayout L;
  L.Np = (int)ceil_div(s.N, 16) * 16;
  L.n_tiles = (int)ceil_div(s.BT, 32);
  L.n_chunks = (int)ceil_div(s.d, 64);
  int tpb = 1;
  while ((int64_t)L.n_chunks * ceil_div(L.n_tiles, tpb) > 512) ++tpb;
  L.tpb = tpb;
  L.n_ranges = (int)ceil_div(L.n_tiles, tpb);
  return L;
}

size_t gen_bwd_g_bytes(const Shape &s) { return (size_t)s.BT * gen_bwd_layout(s).Np * sizeof(bf16); }
size_t gen_bwd_mp_bytes(const Shape &s) { return (size_t)s.d * gen_bwd_layout(s).Np * sizeof(bf16); }
size_t gen_bwd_part_bytes(const Shape &s) {
  return (size_t)gen_bwd_layout(s).n_ranges * s.d * s.N * sizeof(float);
}

int gen_bwd(const Shape &s, const float *gpart, int n_slices, int R, int Dt, const void *h,
            const void *M, bf16 *g, bf16 *Mp, void *dh, float *dMp, hipStream_t st) {
  const GenBwdLayout L = gen_bwd_layout(s);
  hipLaunchKernelGGL(gbwd::k_combine, dim3((unsigned)ceil_div(s.BT * L.Np / 4, 256)), dim3(256), 0, st, s,
                     gpart, n_slices, R, Dt, L.Np, g);
  const bool tr = trace_begin(DYNCONV_K_GEN_BWD, st);
  if (dh) {
    // the weight is read in place when its rows are whole 8-column chunks
    const bool direct = s.N % 8 == 0;
    if (!direct)
      hipLaunchKernelGGL(gbwd::k_pad_cols, dim3((unsigned)ceil_div(s.d * L.Np, 256)), dim3(256), 0, st,
                         (const bf16 *)M, Mp, s.d, s.N, L.Np);
    const bf16 *Ma = direct ? (const bf16 *)M : Mp;
    const int Mcols = direct ? s.N : L.Np;
    const int n_ib = (int)ceil_div(s.d, 128);
    const int tiles8 = (int)ceil_div(L.n_tiles, 8) * 8;
    const unsigned nblk = (unsigned)(tiles8 * n_ib);
    switch (L.Np / 16) {
#define CASE(ks)                                                                                      \
  case ks:                                                                                            \
    hipLaunchKernelGGL(gbwd::k_dh<ks>, dim3(nblk), dim3(256), 0, st, g, Ma, (bf16 *)dh, s.BT, (int)s.d, \
                       L.Np, n_ib, Mcols);                                                            \
    break;
      CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
      CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
      default: trace_end(tr, st); return DYNCONV_E_LIMIT;
    }
  }
  dim3 grid((unsigned)L.n_chunks, (unsigned)L.n_ranges);
  switch (L.Np / 16) {
#define CASE(nb)                                                                                  \
  case nb:                                                                                        \
    hipLaunchKernelGGL(gbwd::k_dM<nb>, grid, dim3(256), 0, st, (const bf16 *)h, g, dMp, s.BT,     \
                       (int)s.d, s.N, L.Np, L.tpb, L.n_tiles);                                    \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: trace_end(tr, st); return DYNCONV_E_LIMIT;
  }
  trace_end(tr, st);
  return 0;
}

int finalize(const float *p0, float *o0, int64_t n0, int np0, const float *p1, float *o1, int64_t n1,
             int np1, const float *p2, float *o2, int64_t n2, int np2, hipStream_t st) {
  gbwd::Red r0{p0, o0, o0 ? n0 : 0, np0}, r1{p1, o1, o1 ? n1 : 0, np1}, r2{p2, o2, o2 ? n2 : 0, np2};
  const int64_t quads = ceil_div(r0.n, 4) + ceil_div(r1.n, 4) + ceil_div(r2.n, 4);
  if (quads == 0) return 0;
  const bool tr = trace_begin(DYNCONV_K_FINALIZE, st);
  hipLaunchKernelGGL(gbwd::k_finalize, dim3((unsigned)ceil_div(quads, 256)), dim3(256), 0, st, r0, r1, r2);
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
