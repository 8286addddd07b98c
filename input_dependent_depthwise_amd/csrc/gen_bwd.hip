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
//              written as bf16 (the MFMA operand precision) twice: g [BT, Np]
//              for dh and g^T [Np, BTp] (token-contiguous) for dM
//              (k_combine_lr: the same for rank 16 on finer blocks);
//   k_dh       dh^T tiles = M . g^T on v_mfma_f32_32x32x16_bf16; a block holds
//              256 rows of M in registers and walks a token range with the g
//              tiles staged in LDS, writing dh rows through LDS;
//   k_dM       per (128-row chunk of d, token range) partials of h^T g on
//              v_mfma_f32_16x16x32_bf16, h staged in LDS, g^T tiles as loaded;
//              the row chunks of one token range share an XCD (and its L2);
//   k_dh_dM    both in one launch for weights up to 128 columns;
//   k_finalize fixed-order sums of all weight-gradient partials (dU, dw0, dM).
#include "kernels.h"
#include "bufio.h"
#include "mfma.h"

namespace dynconv {
namespace gbwd {

constexpr int kMaxSpan = 16;  // most slices one head's du may be split over

// Block: TT = 2048 / CW tokens x CW columns (CW = 16, 32 or 64; column group
// blockIdx.y), two quads of four columns per thread.  g = fixed-order sum of
// the conv kernel's slice partials (low-rank: [slice][BT][R] rows of dz, all
// slices; head-wise: a head's du lies in the one or few slices its channels
// fall in, at a slot given by the head's place in the slice; that column ->
// (slice, slot) table is built once per block in LDS).  The slice loop is
// outermost so that both quads' loads are in flight together.  g [BT][Np] is
// written straight from registers (row-major, for dh); the bf16 tile also
// goes through LDS to write g^T [Np][BTp] (token-contiguous, zero for tokens
// past BT), the operand layout of the dM kernel.  The LDS row pitch CW + 2
// puts the eight tokens a column gather reads in distinct banks.
template <int CW>
__global__ void __launch_bounds__(256)
k_combine(Shape s, const float *__restrict__ gpart, int n_slices, int R, int Dt, int Np, int64_t BTp, int span,
          bf16 *__restrict__ g, bf16 *__restrict__ gT) {
  constexpr int TT = 2048 / CW, Q = CW / 4, P = CW + 2;
  __shared__ __attribute__((aligned(16))) uint16_t ct[TT * P];
  __shared__ int64_t tab[CW][kMaxSpan];  // head-wise: element offset of (slice, slot) in gpart, or -1
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int c0 = blockIdx.y * CW;
  const bool lowrank = s.kind == DYNCONV_LOWRANK;
  if (!lowrank) {
    for (int e = tid; e < CW * span; e += 256) {
      const int nl = e / span, p = e - nl * span, n = c0 + nl;
      int64_t off = -1;
      if (n < s.N) {
        const int eh = n / s.k, j = n - eh * s.k;  // head, tap
        const int d0 = eh * s.hd / Dt, d1 = ((eh + 1) * s.hd - 1) / Dt, d = d0 + p;
        if (d <= d1) off = (int64_t)d * s.BT * R + (eh - d * Dt / s.hd) * s.k + j;
      }
      tab[nl][p] = off;
    }
    __syncthreads();
  }
  float v[2][4];
  int64_t tq[2];
  int nq[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int e = tid + 256 * qi;
    tq[qi] = t0 + e / Q;
    nq[qi] = (e % Q) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[qi][c] = 0.f;
  }
  if (lowrank) {
    const int64_t stride = s.BT * R;
    bool vec[2];
    const float *src[2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      const int n0 = c0 + nq[qi];
      vec[qi] = tq[qi] < s.BT && n0 + 4 <= s.N && R % 4 == 0;
      src[qi] = gpart + (tq[qi] < s.BT ? tq[qi] : 0) * R + n0;
    }
    if (vec[0] && vec[1]) {
      int d = 0;
      for (; d + 4 <= n_slices; d += 4) {
        float4 a[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int qi = 0; qi < 2; ++qi) a[u][qi] = *reinterpret_cast<const float4 *>(src[qi] + (d + u) * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int qi = 0; qi < 2; ++qi)
            v[qi][0] += a[u][qi].x, v[qi][1] += a[u][qi].y, v[qi][2] += a[u][qi].z, v[qi][3] += a[u][qi].w;
      }
      for (; d < n_slices; ++d)
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          const float4 a = *reinterpret_cast<const float4 *>(src[qi] + d * stride);
          v[qi][0] += a.x, v[qi][1] += a.y, v[qi][2] += a.z, v[qi][3] += a.w;
        }
    } else {
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (tq[qi] < s.BT && c0 + nq[qi] + c < s.N)
            for (int d = 0; d < n_slices; ++d) v[qi][c] += src[qi][d * stride + c];
    }
  } else if (s.k == 4) {
    // a quad is one head's four taps: contiguous (and 16-byte aligned, R being
    // a multiple of 4) in each slice's partial row
    for (int p = 0; p < span; ++p) {
      float4 a[2];
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        const int64_t off = tab[nq[qi]][p];
        a[qi] = (off >= 0 && tq[qi] < s.BT) ? *reinterpret_cast<const float4 *>(gpart + off + tq[qi] * R)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
        v[qi][0] += a[qi].x, v[qi][1] += a[qi].y, v[qi][2] += a[qi].z, v[qi][3] += a[qi].w;
    }
  } else {
    for (int p = 0; p < span; ++p) {
      float a[2][4];
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t off = tab[nq[qi] + c][p];
          a[qi][c] = (off >= 0 && tq[qi] < s.BT) ? gpart[off + tq[qi] * R] : 0.f;
        }
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[qi][c] += a[qi][c];
    }
  }
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[qi][0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[qi][1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[qi][2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[qi][3]) << 16);
    const int n0 = c0 + nq[qi];
    if (tq[qi] < s.BT && n0 < Np) *reinterpret_cast<uint2 *>(g + tq[qi] * Np + n0) = make_uint2(lo, hi);
    uint32_t *w = reinterpret_cast<uint32_t *>(ct + (tq[qi] - t0) * P + nq[qi]);  // 4-byte aligned
    w[0] = lo;
    w[1] = hi;
  }
  if (!gT) return;  // g^T not wanted (the wide dM kernel reads g)
  __syncthreads();
  {  // one 8-token piece of one column per thread
    const int nl = tid / (TT / 8), tc = (tid % (TT / 8)) * 8;
    const int n = c0 + nl;
    if (n < Np && t0 + tc < BTp) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        w[p] = (uint32_t)ct[(tc + 2 * p) * P + nl] | ((uint32_t)ct[(tc + 2 * p + 1) * P + nl] << 16);
      *reinterpret_cast<uint4 *>(gT + (int64_t)n * BTp + t0 + tc) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Low-rank g for rank 16 (Np = R): the same fixed-order sums over more,
// smaller blocks (rank 32, with 8-token blocks, was slower than k_combine).
// Block: 64 / (R/4) tokens; lane = token x
// column quad, so each wave's load of one slice is one contiguous 1 KB run of
// dz rows; wave w sums its quarter of the slices (ascending), and wave 0
// adds the four quarters in order.  g and g^T (zeros past BT) are written
// straight from registers.
__global__ void __launch_bounds__(256)
k_combine_lr(const float *__restrict__ gpart, int64_t BT, int R, int n_slices, int64_t BTp,
             bf16 *__restrict__ g, bf16 *__restrict__ gT) {
  __shared__ float4 part[3][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Q = R / 4, tpw = 64 / Q;  // column quads per token, tokens per block
  const int64_t t = (int64_t)blockIdx.x * tpw + lane / Q;
  const int n0 = (lane % Q) * 4;
  const bool live = t < BT;
  const int d0 = w * n_slices / 4, d1 = (w + 1) * n_slices / 4;
  const int64_t stride = BT * R;
  const float *src = gpart + (live ? t : 0) * R + n0;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    int d = d0;
    for (; d + 4 <= d1; d += 4) {
      float4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = *reinterpret_cast<const float4 *>(src + (d + u) * stride);
#pragma unroll
      for (int u = 0; u < 4; ++u) v.x += a[u].x, v.y += a[u].y, v.z += a[u].z, v.w += a[u].w;
    }
    for (; d < d1; ++d) {
      const float4 a = *reinterpret_cast<const float4 *>(src + d * stride);
      v.x += a.x, v.y += a.y, v.z += a.z, v.w += a.w;
    }
  }
  if (w > 0) part[w - 1][lane] = v;
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const float4 a = part[q][lane];
    v.x += a.x, v.y += a.y, v.z += a.z, v.w += a.w;
  }
  const bf16 o[4] = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
  if (live) {
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, o[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, o[1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, o[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, o[3]) << 16);
    *reinterpret_cast<uint2 *>(g + t * R + n0) = make_uint2(lo, hi);
  }
  if (t < BTp) {
#pragma unroll
    for (int c = 0; c < 4; ++c) gT[(int64_t)(n0 + c) * BTp + t] = o[c];
  }
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

// Blocks of a grid of n_work items run round-robin over the 8 XCDs; item q =
// xcd * slots + slot makes neighbouring items (the row blocks of one token
// range) share an XCD and so its L2.
__device__ __forceinline__ int xcd_item(int slots) {
  return (int)(blockIdx.x & 7) * slots + (int)(blockIdx.x >> 3);
}

constexpr int kOP = 36;  // dh staging tile row (one token): 32 rows of d + pad, bf16

// dh[t, i] = sum_n g[t, n] Mp[i, n], as dh^T tiles on v_mfma_f32_32x32x16_bf16
// (A = 32 rows of Mp, B = 32 tokens of g).  Block: 8 waves x 32 rows of d
// (256 rows) over a range of 32-token tiles.  A wave keeps its rows' weight
// fragments in registers for the whole range.  The block stages each g tile
// [32 tokens][Np] in LDS (double-buffered, one barrier per tile; loaded two
// tiles ahead in two register sets), and a wave writes its dh tile through a
// private LDS tile so that every store is a whole 64-byte row segment.
// LDS of one dh block (bf16 elements): two g tiles, eight per-wave output tiles
template <int KS>
constexpr int dh_lds_elems() { return 2 * 32 * (KS * 16 + 8) + 8 * 32 * kOP; }

template <int KS>
__device__ __forceinline__ void dh_body(const bf16 *__restrict__ g, const bf16 *__restrict__ Mp,
                                        bf16 *__restrict__ dh, int64_t BT, int d, int Mcols, int n_rb, int n_tr,
                                        int tpr, int n_tiles, const int q, bf16 *lds) {
  constexpr int NP = KS * 16;
  constexpr int GP = NP + 8;            // LDS row of the g tile (one token), bf16
  constexpr int CH = 4 * NP;            // 16-byte pieces of a g tile
  constexpr int CPT = (CH + 511) / 512;  // per thread
  bf16 (*gs)[32 * GP] = reinterpret_cast<bf16 (*)[32 * GP]>(lds);
  bf16 (*ot)[32 * kOP] = reinterpret_cast<bf16 (*)[32 * kOP]>(lds + 2 * 32 * GP);
  if (q >= n_rb * n_tr) return;
  const int tr = q / n_rb, rb = q - tr * n_rb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int i0 = rb * 256 + wave * 32;
  const bool active = i0 < d;  // idle waves still load g tiles and meet the barriers, store nothing
  const int tile_lo = tr * tpr, ntl = min(n_tiles, tile_lo + tpr) - tile_lo;
  const int64_t tok_lo = (int64_t)tile_lo * 32;
  const int64_t tok_n = min(BT, tok_lo + (int64_t)ntl * 32) - tok_lo;

  bf16x8 mf[KS];
  {
    const int ia = min(i0 + l32, d - 1);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(Mp, (uint32_t)((int64_t)d * Mcols * 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int n = ks * 16 + hh * 8;  // Mcols is Np or a multiple of 8: chunks are all in or all out
      mf[ks] = as_bf16x8(buf_load16(rm, n < Mcols ? (uint32_t)((ia * Mcols + n) * 2) : kOutside));
    }
  }
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + tok_lo * NP, (uint32_t)(tok_n * NP * 2));
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dh + tok_lo * d, (uint32_t)(tok_n * d * 2));
  auto goff = [&](int tile, int c) -> uint32_t {
    const int e = tid + 512 * c;
    return (tile < ntl && (CH % 512 == 0 || e < CH))
               ? (uint32_t)(((tile * 32 + e / (NP / 8)) * NP + (e % (NP / 8)) * 8) * 2)
               : kOutside;
  };
  uint4 gr[2][CPT];
  auto load = [&](int set, int tile) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) gr[set][c] = buf_load16(rg, goff(tile, c));
  };
  bf16 *my = ot[wave];
  const int tok_r = lane >> 2, c8 = (lane & 3) * 8;
  const uint32_t col_ok = active && i0 + c8 < d;  // d is a multiple of 8
  auto step = [&](int set, int tile) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {  // pieces past CH (loaded as zeros) are not stored
      const int e = tid + 512 * c;
      if (CH % 512 == 0 || e < CH)
        *reinterpret_cast<uint4 *>(gs[set] + (e / (NP / 8)) * GP + (e % (NP / 8)) * 8) = gr[set][c];
    }
    __syncthreads();
    load(set, tile + 2);
    // computed on every path (an idle wave or a tile past the range stores
    // nothing): the memory instruction count stays the same on all paths
    f32x16 acc = {};
    const bf16 *gb = gs[set] + l32 * GP + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma32(mf[ks], as_bf16x8(*reinterpret_cast<const uint4 *>(gb + ks * 16)), acc);
    // lane holds dh^T[8b + 4hh + r][l32], b, r = 0..3: four consecutive rows of one token
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)acc[4 * b]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)acc[4 * b + 1]) << 16);
      const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)acc[4 * b + 2]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)acc[4 * b + 3]) << 16);
      *reinterpret_cast<uint2 *>(my + l32 * kOP + 8 * b + 4 * hh) = make_uint2(lo, hi);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tok = tok_r + 16 * p;
      const uint2 a = *reinterpret_cast<const uint2 *>(my + tok * kOP + c8);
      const uint2 bq = *reinterpret_cast<const uint2 *>(my + tok * kOP + c8 + 4);
      const uint32_t off =
          col_ok && tile < ntl ? (uint32_t)((((int64_t)tile * 32 + tok) * d + i0 + c8) * 2) : kOutside;
      buf_store16(rd, off, make_uint4(a.x, a.y, bq.x, bq.y));
    }
  };
  // The loop issues, per tile, the loads two tiles ahead and then two stores.
  // The prologue keeps that order (with stores that fall outside dh and are
  // dropped), so the compiler's wait counts at the loop head are the steady
  // state ones and the second prefetch set stays in flight.
  // (distinct offsets, so that none of these stores is folded away)
  __builtin_amdgcn_sched_barrier(0);
  load(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  buf_store16(rd, kOutside, make_uint4(0, 0, 0, 0));
  buf_store16(rd, kOutside + 16, make_uint4(0, 0, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  load(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  buf_store16(rd, kOutside + 32, make_uint4(0, 0, 0, 0));
  buf_store16(rd, kOutside + 48, make_uint4(0, 0, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  for (int tile = 0; tile < ntl; tile += 2) {
    step(0, tile);
    step(1, tile + 1);
  }
}

template <int KS>
__global__ void __launch_bounds__(512)
k_dh(const bf16 *__restrict__ g, const bf16 *__restrict__ Mp, bf16 *__restrict__ dh, int64_t BT, int d,
     int Mcols, int n_rb, int n_tr, int tpr, int n_tiles, int slots) {
  __shared__ __attribute__((aligned(16))) bf16 lds[dh_lds_elems<KS>()];
  dh_body<KS>(g, Mp, dh, BT, d, Mcols, n_rb, n_tr, tpr, n_tiles, xcd_item(slots), lds);
}

constexpr int kHP = 132;  // dM h tile row (one token): 128 rows of d + pad, bf16
constexpr int kGP = 40;   // dM g^T tile row (one column): 32 tokens + pad, bf16

// dMp[range][i, n] = sum over the range's tokens of h[t, i] g[t, n], on
// v_mfma_f32_16x16x32_bf16 with A = h^T (rows of d x tokens) and B = g (tokens
// x columns).  Block: 128 rows of d (wave w: rows 32w..32w+31) x all Np
// columns over a range of 32-token tiles.  Per tile the block stages h
// row-major in LDS (the A fragments are then gathered 16 bits at a time; the
// 264-byte row pitch spreads the four token groups of a gather over distinct
// banks) and the g^T tile (16-byte B fragments), double-buffered with one
// barrier per tile.  h is loaded two tiles ahead in two register sets, g^T one tile
// ahead; loads are issued g^T first so that waiting for a tile's g^T leaves
// the later h tile in flight.  Tiles past the range read as zeros.
template <int NT>
constexpr int dM_lds_elems() { return 2 * 32 * kHP + 2 * NT * 16 * kGP; }

// tiles of item q (q = range * n_chunks + chunk), 0 past the last item
__device__ __forceinline__ int dM_tiles(int q, int n_chunks, int n_ranges, int tpb, int n_tiles) {
  if (q >= n_chunks * n_ranges) return 0;
  const int lo = q / n_chunks * tpb;
  return min(n_tiles, lo + tpb) - lo;
}

// One item on 256 threads (tid); the loop takes n_loop tiles (at least the
// item's own; more when it shares a block's barriers with another item, the
// extra tiles loading zeros).  An item past the last (q >= n_chunks *
// n_ranges) loads nothing and stores nothing but meets the barriers.
template <int NT>
__device__ __forceinline__ void dM_body(const bf16 *__restrict__ h, const bf16 *__restrict__ gT,
                                        float *__restrict__ dMp, int64_t BT, int64_t BTp, int d, int N,
                                        int n_chunks, int n_ranges, int tpb, int n_tiles, const int q, const int tid,
                                        const int n_loop, bf16 *lds) {
  constexpr int CH = NT * 64;            // 16-byte chunks of a g^T tile
  constexpr int CPT = (CH + 255) / 256;  // per thread
  bf16 (*hs)[32 * kHP] = reinterpret_cast<bf16 (*)[32 * kHP]>(lds);
  bf16 (*gs)[NT * 16 * kGP] = reinterpret_cast<bf16 (*)[NT * 16 * kGP]>(lds + 2 * 32 * kHP);
  const bool valid = q < n_chunks * n_ranges;
  const int qv = valid ? q : 0;
  const int range = qv / n_chunks, chunk = qv - range * n_chunks;
  const int lane = tid & 63, wave = tid >> 6;
  const int i0 = chunk * 128;
  const int tile_lo = range * tpb, ntl = dM_tiles(q, n_chunks, n_ranges, tpb, n_tiles);
  const int64_t tok_lo = (int64_t)tile_lo * 32;
  const int64_t tok_n = min(BT, tok_lo + (int64_t)ntl * 32) - tok_lo;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(h + tok_lo * d, (uint32_t)(tok_n * d * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gT + tok_lo, (uint32_t)(((int64_t)NT * 16 * BTp - tok_lo) * 2));

  // this thread's pieces: h chunk c -> token tid/16 + 16c, rows i0 + 8(tid%16)
  const int h_tok = tid >> 4, h_col = (tid & 15) * 8;
  const bool h_in = i0 + h_col < d;  // d is a multiple of 8
  auto hoff = [&](int tile, int c) -> uint32_t {
    return (tile < ntl && h_in) ? (uint32_t)(((tile * 32 + h_tok + 16 * c) * d + i0 + h_col) * 2) : kOutside;
  };
  auto goff = [&](int tile, int c) -> uint32_t {
    const int e = tid + 256 * c;
    return (tile < ntl && (CH % 256 == 0 || e < CH)) ? (uint32_t)((((int64_t)(e >> 2)) * BTp + tile * 32 + (e & 3) * 8) * 2)
                                  : kOutside;
  };

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 hr[2][2], gr[CPT];
  auto load_g = [&](int tile) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) gr[c] = buf_load16(rg, goff(tile, c));
  };
  auto load_h = [&](int set, int tile) {
#pragma unroll
    for (int c = 0; c < 2; ++c) hr[set][c] = buf_load16(rh, hoff(tile, c));
  };
  const uint16_t *hsu = reinterpret_cast<const uint16_t *>(&hs[0][0]);
  auto step = [&](int set, int tile) {
    bf16 *hb = hs[set];
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // rows of 264 bytes: two 8-byte writes per piece
      uint2 *dst = reinterpret_cast<uint2 *>(hb + (h_tok + 16 * c) * kHP + h_col);
      dst[0] = make_uint2(hr[set][c].x, hr[set][c].y);
      dst[1] = make_uint2(hr[set][c].z, hr[set][c].w);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {  // pieces past CH (loaded as zeros) are not stored
      const int e = tid + 256 * c;
      if (CH % 256 == 0 || e < CH) *reinterpret_cast<uint4 *>(gs[set] + (e >> 2) * kGP + (e & 3) * 8) = gr[c];
    }
    __syncthreads();
    load_g(tile + 1);
    load_h(set, tile + 2);
    // A fragment r: rows 32w + 16r + lane%16, tokens 8(lane/16) .. +7
    const uint16_t *ha = hsu + set * 32 * kHP + 8 * (lane >> 4) * kHP + 32 * wave + (lane & 15);
    bf16x8 a[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        w[p] = (uint32_t)ha[2 * p * kHP + 16 * r] | ((uint32_t)ha[(2 * p + 1) * kHP + 16 * r] << 16);
      a[r] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
    const bf16 *gb = gs[set] + (lane & 15) * kGP + 8 * (lane >> 4);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(gb + n * 16 * kGP));
      acc[0][n] = mfma16(a[0], b, acc[0][n]);
      acc[1][n] = mfma16(a[1], b, acc[1][n]);
    }
  };
  load_g(0);
  load_h(0, 0);
  load_h(1, 1);
  for (int tile = 0; tile < n_loop; tile += 2) {
    step(0, tile);
    step(1, tile + 1);
  }
  if (!valid) return;
  // D fragment: lane holds D[4(lane/16) + r][lane%16] of each 16x16 block
  float *out = dMp + (int64_t)range * d * N;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = i0 + 32 * wave + 16 * r + 4 * (lane >> 4) + k;
        const int col = n * 16 + (lane & 15);
        if (i < d && col < N) out[(int64_t)i * N + col] = acc[r][n][k];
      }
}

template <int NT>
__global__ void __launch_bounds__(256, 2)
k_dM(const bf16 *__restrict__ h, const bf16 *__restrict__ gT, float *__restrict__ dMp, int64_t BT, int64_t BTp,
     int d, int N, int n_chunks, int n_ranges, int tpb, int n_tiles, int slots) {
  __shared__ __attribute__((aligned(16))) bf16 lds[dM_lds_elems<NT>()];
  const int q = xcd_item(slots);
  if (q >= n_chunks * n_ranges) return;
  dM_body<NT>(h, gT, dMp, BT, BTp, d, N, n_chunks, n_ranges, tpb, n_tiles, q, threadIdx.x,
              dM_tiles(q, n_chunks, n_ranges, tpb, n_tiles), lds);
}

// dMp[range][i, n] for weights of 129..256 columns, on v_mfma_f32_32x32x16_bf16
// with A = h^T (rows of d x tokens) and B = g (tokens x columns), both read
// from row-major LDS tiles with ds_read_b64_tr_b16 (g^T is not needed).
// Block: 8 waves (two per SIMD) over 128 rows of d x 256 columns; wave w
// takes rows 64 (w & 1) .. +63 and columns 64 (w >> 1) .. +63 (2 x 2
// fragments of 32 x 32).  Per 32-token tile the block stages h [32][128] and
// g [32][256] in LDS (double-buffered, one barrier per tile); every thread
// loads three 16-byte pieces per tile into a ring of four register sets, so
// four tiles are in flight while one is computed.  Row pitches of 288 and 544
// bytes put the four rows of each 16-lane transposed read in distinct banks.
// Tiles past the range, rows past d and columns past Np read as zeros.
constexpr int kWH = 144;  // LDS row of the h tile (one token): 128 rows of d + pad, bf16
constexpr int kWG = 272;  // LDS row of the g tile (one token): 256 columns + pad, bf16
constexpr int kWRing = 8; // register sets in flight (tiles loaded ahead)

__global__ void __launch_bounds__(512, 1)
k_dM_wide(const bf16 *__restrict__ h, const bf16 *__restrict__ g, float *__restrict__ dMp, int64_t BT, int d,
          int N, int Np, int n_chunks, int n_ranges, int tpb, int n_tiles, int slots) {
  __shared__ __attribute__((aligned(16))) bf16 hs[2][32 * kWH];
  __shared__ __attribute__((aligned(16))) bf16 gs[2][32 * kWG];
  const int q = xcd_item(slots);
  if (q >= n_chunks * n_ranges) return;
  const int range = q / n_chunks, chunk = q - range * n_chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave & 1, wn = wave >> 1;
  const int i0 = chunk * 128;
  const int tile_lo = range * tpb, ntl = min(n_tiles, tile_lo + tpb) - tile_lo;
  const int n_loop = (ntl + kWRing - 1) / kWRing * kWRing;
  const int64_t tok_lo = (int64_t)tile_lo * 32;
  const int64_t tok_n = min(BT, tok_lo + (int64_t)ntl * 32) - tok_lo;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(h + tok_lo * d, (uint32_t)(tok_n * d * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + tok_lo * Np, (uint32_t)(tok_n * Np * 2));

  // pieces: 0 -> h (token tid/16, rows i0 + 8 (tid%16)); 1, 2 -> g (token
  // e/32, columns 8 (e%32), e = tid + 512 (c - 1))
  const int h_tok = tid >> 4, h_col = (tid & 15) * 8;
  const uint32_t h_base = i0 + h_col < d ? (uint32_t)((h_tok * d + i0 + h_col) * 2) : kOutside;
  uint32_t g_base[2];
  int g_tok[2], g_col[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int e = tid + 512 * c;
    g_tok[c] = e >> 5;
    g_col[c] = (e & 31) * 8;
    g_base[c] = g_col[c] < Np ? (uint32_t)((g_tok[c] * Np + g_col[c]) * 2) : kOutside;
  }
  const uint32_t h_step = (uint32_t)(32 * d * 2), g_step = (uint32_t)(32 * Np * 2);
  auto off = [&](uint32_t base, uint32_t step, int tile) -> uint32_t {
    return (base == kOutside || tile >= ntl) ? kOutside : base + (uint32_t)tile * step;
  };
  uint4 rr[kWRing][3];
  auto load = [&](int set, int tile) {
    rr[set][0] = buf_load16(rh, off(h_base, h_step, tile));
    rr[set][1] = buf_load16(rg, off(g_base[0], g_step, tile));
    rr[set][2] = buf_load16(rg, off(g_base[1], g_step, tile));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // transposed-read addresses (bytes): group G = lane/16 takes columns
  // 16 (G & 1) .. +15 and tokens 8 (G >> 1) .. +7; lane L = lane%16 reads
  // token + L/4 at column 4 (L%4)
  const int G = lane >> 4, L = lane & 15;
  const int tr_tok = 8 * (G >> 1) + (L >> 2), tr_col = 16 * (G & 1) + 4 * (L & 3);
  const unsigned char *hs_b = reinterpret_cast<const unsigned char *>(&hs[0][0]);
  const unsigned char *gs_b = reinterpret_cast<const unsigned char *>(&gs[0][0]);
  const int ha = (tr_tok * kWH + 64 * wi + tr_col) * 2;
  const int ga = (tr_tok * kWG + 64 * wn + tr_col) * 2;

  auto step = [&](int set, int tile) {
    const int buf = set & 1;
    *reinterpret_cast<uint4 *>(&hs[buf][h_tok * kWH + h_col]) = rr[set][0];
#pragma unroll
    for (int c = 0; c < 2; ++c) *reinterpret_cast<uint4 *>(&gs[buf][g_tok[c] * kWG + g_col[c]]) = rr[set][1 + c];
    __syncthreads();
    load(set, tile + kWRing);
    const unsigned char *hb = hs_b + buf * (32 * kWH * 2) + ha;
    const unsigned char *gb = gs_b + buf * (32 * kWG * 2) + ga;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const unsigned char *pa = hb + (16 * kh * kWH + 32 * x) * 2;
        const uint2 a0 = read_tr16(pa), a1 = read_tr16(pa + 4 * kWH * 2);
        af[x] = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
        const unsigned char *pb = gb + (16 * kh * kWG + 32 * x) * 2;
        const uint2 b0 = read_tr16(pb), b1 = read_tr16(pb + 4 * kWG * 2);
        bfr[x] = as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
    }
  };
  // The prologue issues its loads in the loop's order (h, then the two g
  // pieces, set by set), so that the compiler's wait count at the loop head
  // is the steady-state one and three sets stay in flight.
#pragma unroll
  for (int s = 0; s < kWRing; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    rr[s][0] = buf_load16(rh, off(h_base, h_step, s));
    __builtin_amdgcn_sched_barrier(0);
    rr[s][1] = buf_load16(rg, off(g_base[0], g_step, s));
    __builtin_amdgcn_sched_barrier(0);
    rr[s][2] = buf_load16(rg, off(g_base[1], g_step, s));
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int tile = 0; tile < n_loop; tile += kWRing) {
#pragma unroll
    for (int s = 0; s < kWRing; ++s) step(s, tile + s);
  }
  // D fragment: lane holds D[8b + 4 (lane/32) + r][lane%32] in element 4b + r
  float *out = dMp + (int64_t)range * d * N;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = 64 * wn + 32 * b + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = i0 + 64 * wi + 32 * a + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (i < d && col < N) out[(int64_t)i * N + col] = acc[a][b][e];
      }
    }
}

// dh and dM in one launch: dh writes as much as dM reads, and each alone
// leaves the chip mostly waiting on memory.  Blocks below 8 * dh_slots are
// dh blocks (512 threads); the others each run two dM items, one per half,
// which meet the same barriers (both loop over the longer item's tiles).
// The LDS of the two kinds overlaps.
template <int KS>
__global__ void __launch_bounds__(512)
k_dh_dM(const bf16 *__restrict__ g, const bf16 *__restrict__ Mp, bf16 *__restrict__ dh, const bf16 *__restrict__ h,
        const bf16 *__restrict__ gT, float *__restrict__ dMp, int64_t BT, int64_t BTp, int d, int Mcols, int N,
        int n_rb, int n_tr, int tpr, int n_chunks, int n_ranges, int tpb, int n_tiles, int dh_slots, int dm_slots) {
  constexpr int DH = dh_lds_elems<KS>(), DM = dM_lds_elems<KS>();
  __shared__ __attribute__((aligned(16))) bf16 lds[DH > 2 * DM ? DH : 2 * DM];
  const int b = blockIdx.x;
  if (b < 8 * dh_slots) {
    dh_body<KS>(g, Mp, dh, BT, d, Mcols, n_rb, n_tr, tpr, n_tiles, (b & 7) * dh_slots + (b >> 3), lds);
    return;
  }
  const int bm = b - 8 * dh_slots;
  const int pair = (bm & 7) * dm_slots + (bm >> 3);
  if (2 * pair >= n_chunks * n_ranges) return;  // the whole block
  const int n_loop = max(dM_tiles(2 * pair, n_chunks, n_ranges, tpb, n_tiles),
                         dM_tiles(2 * pair + 1, n_chunks, n_ranges, tpb, n_tiles));
  const int half = threadIdx.x >> 8;
  dM_body<KS>(h, gT, dMp, BT, BTp, d, N, n_chunks, n_ranges, tpb, n_tiles, 2 * pair + half, threadIdx.x & 255,
              n_loop, lds + half * DM);
}

// out[e] = sum_p part[p][e] for e < n, p < np, for up to three independent
// reductions packed into one launch.
struct Red {
  const float *part;
  float *out;
  int64_t n;
  int np;
  int lp;         // lanes per output quad (1, 2, 4 or 8): each sums every lp-th partial
  int64_t lanes;  // threads of this reduction, a whole number of waves
  int acc;        // 1: add the sum to what out holds (a later chunk of sequences), 0: overwrite
};

// Four consecutive outputs per group of lp adjacent lanes.  Lane `sub` of a
// group sums partials sub, sub + lp, ... in ascending order (loads issued 8
// at a time ahead of the adds); the group then adds its lanes' sums with an
// xor butterfly, which gives every lane the same bits (each step adds the
// same two values), so the result is fixed-order and deterministic.
__global__ void __launch_bounds__(256) k_finalize(Red r0, Red r1, Red r2) {
  int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const Red *r;
  if (th < r0.lanes) {
    r = &r0;
  } else if ((th -= r0.lanes) < r1.lanes) {
    r = &r1;
  } else if ((th -= r1.lanes) < r2.lanes) {
    r = &r2;
  } else {
    return;  // whole waves: a reduction's lanes never share a wave with another's
  }
  const int lp = r->lp, np = r->np;
  const int sub = (int)(th & (lp - 1));
  const int64_t idx = (th / lp) * 4;
  const int64_t n = r->n;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  const bool vec = n % 4 == 0;
  if (idx < n && vec) {
    const float *src = r->part + idx;
    // eight partials per batch, all loads issued before the adds (the last
    // batch masked, so a partial count that is not a multiple of 8 lp does
    // not end in a chain of one-at-a-time loads)
    for (int p = sub; p < np; p += 8 * lp) {
      float4 a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        a[u] = p + u * lp < np ? *reinterpret_cast<const float4 *>(src + (int64_t)(p + u * lp) * n)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p + u * lp < np) v.x += a[u].x, v.y += a[u].y, v.z += a[u].z, v.w += a[u].w;
    }
  } else if (idx < n) {
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < 4; ++c)
      if (idx + c < n)
        for (int p = sub; p < np; p += lp) w[c] += r->part[(int64_t)p * n + idx + c];
    v = make_float4(w[0], w[1], w[2], w[3]);
  }
  for (int m = 1; m < lp; m <<= 1) {
    v.x += __shfl_xor(v.x, m);
    v.y += __shfl_xor(v.y, m);
    v.z += __shfl_xor(v.z, m);
    v.w += __shfl_xor(v.w, m);
  }
  if (sub != 0 || idx >= n || !r->out) return;
  if (vec) {
    if (r->acc) {
      const float4 o = *reinterpret_cast<const float4 *>(r->out + idx);
      v.x = o.x + v.x, v.y = o.y + v.y, v.z = o.z + v.z, v.w = o.w + v.w;
    }
    *reinterpret_cast<float4 *>(r->out + idx) = v;
  } else {
    const float w[4] = {v.x, v.y, v.z, v.w};
    for (int c = 0; c < 4 && idx + c < n; ++c) r->out[idx + c] = r->acc ? r->out[idx + c] + w[c] : w[c];
  }
}

}  // namespace gbwd

// Head-wise: the most conv-kernel slices (Dt channels each) one head's
// channels fall in.
static int combine_span(const Shape &s, int Dt) {
  int span = 1;
  for (int e = 0; e < s.n_heads; ++e) {
    const int64_t d0 = (int64_t)e * s.hd / Dt, d1 = ((int64_t)(e + 1) * s.hd - 1) / Dt;
    span = std::max<int>(span, (int)(d1 - d0 + 1));
  }
  return span;
}

GenBwdLayout gen_bwd_layout(const Shape &s) {
  GenBwdLayout L;
  L.Np = (int)ceil_div(s.N, 16) * 16;
  L.n_tiles = (int)ceil_div(s.BT, 32);
  L.BTp = (int64_t)L.n_tiles * 32;
  L.n_chunks = (int)ceil_div(s.d, 128);
  // about two blocks per CU; an even tile count per range (the dM loop takes
  // tiles in pairs); a range's slice of h stays below 1 GiB (32-bit offsets)
  // (at least one pair of tiles per range, also for an empty batch)
  int tpb = std::max(2, (int)ceil_div(L.n_tiles, std::max<int64_t>(1, 512 / L.n_chunks)));
  tpb += tpb & 1;
  while ((int64_t)tpb * 32 * s.d * 2 >= ((int64_t)1 << 30) && tpb > 2) tpb -= 2;
  L.wide = L.Np > 128;
  if (L.wide) {
    // one block of 8 waves per CU: about 256 (chunk, range) items; whole
    // rings of four tiles per range
    tpb = (int)ceil_div(L.n_tiles, std::max<int64_t>(1, 256 / L.n_chunks));
    tpb = std::max(1, (int)ceil_div(tpb, gbwd::kWRing)) * gbwd::kWRing;
    while ((int64_t)tpb * 32 * std::max<int64_t>(s.d, L.Np) * 2 >= ((int64_t)1 << 30) && tpb > gbwd::kWRing)
      tpb -= gbwd::kWRing;
  }
  L.tpb = tpb;
  L.n_ranges = (int)ceil_div(L.n_tiles, tpb);
  L.n_rb = (int)ceil_div(s.d, 256);
  int tpr = std::max(2, (int)ceil_div(L.n_tiles, std::max<int64_t>(1, 512 / L.n_rb)));
  tpr += tpr & 1;
  while ((int64_t)tpr * 32 * std::max<int64_t>(s.d, L.Np) * 2 >= ((int64_t)1 << 30) && tpr > 2) tpr -= 2;
  L.tpr = tpr;
  L.n_tr = (int)ceil_div(L.n_tiles, tpr);
  return L;
}

bool gen_bwd_supported(const Shape &s) {
  // g and g^T are addressed with 32-bit byte offsets; head-wise column ->
  // slice tables hold at most kMaxSpan slices per head
  const GenBwdLayout L = gen_bwd_layout(s);
  if (s.kind == DYNCONV_HEADWISE && combine_span(s, bwd_layout(s).Dt) > gbwd::kMaxSpan) return false;
  return L.Np <= 256 && (int64_t)L.Np * L.BTp * 2 < ((int64_t)1 << 31) - 64;
}

// g [BT, Np] then g^T [Np, BTp], the latter on a 256-byte boundary
static size_t g_rows_bytes(const Shape &s, const GenBwdLayout &L) {
  return ((size_t)s.BT * L.Np * sizeof(bf16) + 255) / 256 * 256;
}

size_t gen_bwd_g_bytes(const Shape &s) {
  const GenBwdLayout L = gen_bwd_layout(s);
  return g_rows_bytes(s, L) + (L.wide ? 0 : (size_t)L.Np * L.BTp * sizeof(bf16));
}
size_t gen_bwd_mp_bytes(const Shape &s) { return (size_t)s.d * gen_bwd_layout(s).Np * sizeof(bf16); }
size_t gen_bwd_part_bytes(const Shape &s) {
  return (size_t)gen_bwd_layout(s).n_ranges * s.d * s.N * sizeof(float);
}

int gen_bwd(const Shape &s, const float *gpart, int n_slices, int R, int Dt, const void *h,
            const void *M, bf16 *g, bf16 *Mp, void *dh, float *dMp, hipStream_t st) {
  const GenBwdLayout L = gen_bwd_layout(s);
  // the wide dM kernel reads g itself; the others read g^T
  bf16 *gT = L.wide ? nullptr : (bf16 *)((char *)g + g_rows_bytes(s, L));
  const int span = s.kind == DYNCONV_HEADWISE ? combine_span(s, Dt) : 0;
  if (span > gbwd::kMaxSpan) return DYNCONV_E_LIMIT;
  if (s.kind == DYNCONV_LOWRANK && R == 16 && L.Np == R) {
    hipLaunchKernelGGL(gbwd::k_combine_lr, dim3((unsigned)(L.BTp / (256 / R))), dim3(256), 0, st, gpart, s.BT,
                       R, n_slices, L.BTp, g, gT);
  } else if (L.Np <= 32) {
    const int cw = L.Np;  // 16 or 32
    const dim3 grid((unsigned)ceil_div(L.BTp, 2048 / cw));
    if (cw == 16)
      hipLaunchKernelGGL(gbwd::k_combine<16>, grid, dim3(256), 0, st, s, gpart, n_slices, R, Dt, L.Np, L.BTp,
                         span, g, gT);
    else
      hipLaunchKernelGGL(gbwd::k_combine<32>, grid, dim3(256), 0, st, s, gpart, n_slices, R, Dt, L.Np, L.BTp,
                         span, g, gT);
  } else {
    const dim3 grid((unsigned)ceil_div(L.BTp, 32), (unsigned)ceil_div(L.Np, 64));
    hipLaunchKernelGGL(gbwd::k_combine<64>, grid, dim3(256), 0, st, s, gpart, n_slices, R, Dt, L.Np, L.BTp, span,
                       g, gT);
  }
  const bool tr = trace_begin(DYNCONV_K_GEN_BWD, st);
  const int dm_items = L.n_chunks * L.n_ranges;
  if (dh) {
    // the weight is read in place when its rows are whole 8-column chunks
    const bool direct = s.N % 8 == 0;
    if (!direct)
      hipLaunchKernelGGL(gbwd::k_pad_cols, dim3((unsigned)ceil_div(s.d * L.Np, 256)), dim3(256), 0, st,
                         (const bf16 *)M, Mp, s.d, s.N, L.Np);
    const bf16 *Ma = direct ? (const bf16 *)M : Mp;
    const int Mcols = direct ? s.N : L.Np;
    const int dh_slots = (int)ceil_div((int64_t)L.n_rb * L.n_tr, 8);
    if (L.Np <= 128) {
      // dh and dM in one launch (for wider weights, where both are long, it
      // was no faster than two)
      const int dm_slots = (int)ceil_div(ceil_div(dm_items, 2), 8);
      const dim3 grid((unsigned)(8 * (dh_slots + dm_slots)));
      switch (L.Np / 16) {
#define CASE(ks)                                                                                              \
  case ks:                                                                                                    \
    hipLaunchKernelGGL(gbwd::k_dh_dM<ks>, grid, dim3(512), 0, st, g, Ma, (bf16 *)dh, (const bf16 *)h, gT, dMp, \
                       s.BT, L.BTp, (int)s.d, Mcols, s.N, L.n_rb, L.n_tr, L.tpr, L.n_chunks, L.n_ranges, L.tpb,    \
                       L.n_tiles, dh_slots, dm_slots);                                                        \
    break;
        CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
        default: trace_end(tr, st); return DYNCONV_E_LIMIT;
      }
      trace_end(tr, st);
      return 0;
    }
    switch (L.Np / 16) {
#define CASE(ks)                                                                                          \
  case ks:                                                                                                \
    hipLaunchKernelGGL(gbwd::k_dh<ks>, dim3((unsigned)(8 * dh_slots)), dim3(512), 0, st, g, Ma, (bf16 *)dh, \
                       s.BT, (int)s.d, Mcols, L.n_rb, L.n_tr, L.tpr, L.n_tiles, dh_slots);                \
    break;
      CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
      default: trace_end(tr, st); return DYNCONV_E_LIMIT;
    }
  }
  const int slots = (int)ceil_div((int64_t)dm_items, 8);
  if (L.wide) {
    hipLaunchKernelGGL(gbwd::k_dM_wide, dim3((unsigned)(8 * slots)), dim3(512), 0, st, (const bf16 *)h, g, dMp,
                       s.BT, (int)s.d, s.N, L.Np, L.n_chunks, L.n_ranges, L.tpb, L.n_tiles, slots);
    trace_end(tr, st);
    return 0;
  }
  switch (L.Np / 16) {
#define CASE(nb)                                                                                      \
  case nb:                                                                                            \
    hipLaunchKernelGGL(gbwd::k_dM<nb>, dim3((unsigned)(8 * slots)), dim3(256), 0, st, (const bf16 *)h, \
                       gT, dMp, s.BT, L.BTp, (int)s.d, s.N, L.n_chunks, L.n_ranges, L.tpb, L.n_tiles, \
                       slots);                                                                        \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: trace_end(tr, st); return DYNCONV_E_LIMIT;
  }
  trace_end(tr, st);
  return 0;
}

// lanes per output quad: enough that each lane sums at most 8 partials
static gbwd::Red make_red(const float *p, float *o, int64_t n, int np, bool acc) {
  gbwd::Red r{p, o, o ? n : 0, np, 1, 0, acc ? 1 : 0};
  while (r.lp < 8 && r.lp * 8 < np) r.lp *= 2;
  r.lanes = ceil_div(ceil_div(r.n, 4) * r.lp, 64) * 64;
  return r;
}

int finalize(const float *p0, float *o0, int64_t n0, int np0, const float *p1, float *o1, int64_t n1,
             int np1, const float *p2, float *o2, int64_t n2, int np2, bool acc, hipStream_t st) {
  const gbwd::Red r0 = make_red(p0, o0, n0, np0, acc), r1 = make_red(p1, o1, n1, np1, acc),
                  r2 = make_red(p2, o2, n2, np2, acc);
  const int64_t lanes = r0.lanes + r1.lanes + r2.lanes;
  if (lanes == 0) return 0;
  const bool tr = trace_begin(DYNCONV_K_FINALIZE, st);
  hipLaunchKernelGGL(gbwd::k_finalize, dim3((unsigned)ceil_div(lanes, 256)), dim3(256), 0, st, r0, r1, r2);
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
