// conv_bwd.hip -- fused backward of the dynamic short convolution (bf16 I/O).
//
// For L = sum(dy * y) with y = x + sum_j w[t,c,j] x[t-j,c] (gist.science
// Technical Summary of "Dynamic Short Convolutions Improve Transformers",
// Methodology -> Dynamic Short Convolutions: Mechanism, Parameterization,
// Placement), one pass over x and dy produces
//   dx[s,c]  = dy[s,c] + sum_j [s+j <= T-1] w[s+j,c,j] dy[s+j,c]
//   G[t,c,j] = [t-j >= 0] dy[t,c] x[t-j,c]                  (never written out)
//   head-wise: du[t,e,j] = sum_{c in e} G[t,c,j]             -> partial per 128-channel slice
//   low-rank : dz[t,q]  = sum_{c,j} G[t,c,j] U[q,c*k+j]      -> partial per slice
//              dU[q,c*k+j] = sum_t z[t,q] G[t,c,j]           -> partial per token range
//   dw0[c,j] = sum_t G[t,c,j]                                -> partial per token range
// and the filter w is recomputed on chip, as in the forward.
//
// Work split.  A block owns a 128-channel slice and a range of 32-token
// tiles, walked from the last tile down so that the right halo that dx
// needs (w and dy of the next k-1 tokens) comes from the tile processed
// just before.  Each of its 4 waves owns two 16-channel groups; lane l owns
// token l%32 and channels 8*(l/32)..+7 of a group:
//   * filter: low-rank -- two v_mfma_f32_32x32x16_bf16 chains (z U + w0),
//     exactly as in the forward; head-wise -- u[t, head(c)] + w0 gathered;
//   * dx: the products w[t,c,j] dy[t,c] move to token t-j by lane shuffles
//     (ds_bpermute), the k-1 that cross into the next tile through LDS;
//   * dz / du: G stays in the lane and is the B operand of 32x32x16 MFMAs
//     whose A operand is U rearranged (low-rank) or the 0/1 head-membership
//     matrix (head-wise); the 4 waves' partial sums meet in LDS and the block
//     writes one fp32 partial per (slice, token);
//   * dU and dw0: G goes to LDS transposed (token-contiguous, bf16) and feeds
//     v_mfma_f32_16x16x32_bf16 with z as the other operand; dw0 is the row
//     sum of the same fragments.  Each block writes one partial per token
//     range; a finalize kernel sums them in a fixed order (no float atomics).
// x for the tile (plus k-1 rows of history) is staged in LDS with coalesced
// 16-byte loads, double-buffered: the next tile's x, dy and z / u are loaded
// while the current tile is computed.
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace bwd {

constexpr int kCPW = 2;             // 16-channel groups per wave
constexpr int kDt = 4 * kCPW * 16;  // channels per block
constexpr int kRowB = kDt * 2 + 16; // LDS row stride of the x tile (bytes)
constexpr int kGtRowB = 80;         // LDS row stride of the transposed G tile (32 tokens, padded)

struct Params {
  Shape s;
  const bf16 *x, *dy;
  bf16 *dx;
  const float *gen;   // z [BT, r] (low-rank) or u [BT, n_heads*k] (head-wise)
  const bf16 *Uf;     // low-rank: filter-MFMA A fragments (prep_lowrank_frags)
  const bf16 *Udz;    // low-rank: dz-MFMA A fragments (prep_dz_frags)
  const bf16 *w0;     // head-wise bias (may be NULL); low-rank bias is inside Uf
  float *gpart;       // [n_slices][BT][R]: dz (R = r) or du slots (R = SL*k)
  float *dUp;         // low-rank: [n_ranges][r][D*k]
  float *dw0p;        // [n_ranges][D*k]
  int tpb;            // tiles per block (token range length / 32)
  int n_tiles;        // ceil(BT / 32)
  int SL;             // head-wise: head slots per slice
  int R;              // columns of gpart
};

__device__ __forceinline__ void unpack8(const uint4 &raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int KIND, int KP, int KQ, int NCB>
__global__ void __launch_bounds__(256)
k_bwd(Params P) {
  constexpr int KH = KP - 1;
  constexpr int THP = KP / 4;
  constexpr int GROWS = 16 * KP;  // (channel, tap) rows of one 16-channel group
  const Shape &s = P.s;
  const int k = s.k;

  __shared__ __attribute__((aligned(16))) unsigned char xs[2][(32 + KH) * kRowB];
  __shared__ __attribute__((aligned(16))) unsigned char gt[4][kCPW][GROWS * kGtRowB];
  __shared__ __attribute__((aligned(16))) unsigned char zt[2][KIND == DYNCONV_LOWRANK ? 32 * kGtRowB : 16];
  __shared__ __attribute__((aligned(16))) float red[4][64][16];
  __shared__ __attribute__((aligned(16))) float pc[4][kCPW][KH][KH][2][8];
  __shared__ float w0s[KIND == DYNCONV_HEADWISE ? kDt * KP : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int64_t cblk = (int64_t)blockIdx.x * kDt;
  const int nch = (int)min<int64_t>(kDt, s.D - cblk);
  const int tile_lo = blockIdx.y * P.tpb;
  const int tile_hi = min(P.n_tiles, tile_lo + P.tpb);  // exclusive
  const int e_base = KIND == DYNCONV_HEADWISE ? (int)(cblk / s.hd) : 0;

  if constexpr (KIND == DYNCONV_HEADWISE) {
    for (int e = threadIdx.x; e < kDt * KP; e += 256) {
      const int c = e / KP, j = e - c * KP;
      w0s[e] = (P.w0 && c < nch && j < k) ? (float)P.w0[(cblk + c) * k + j] : 0.f;
    }
  }

  // ---- per-lane constants -------------------------------------------------
  // channels of this lane in group g: cblk + 16*(wave*kCPW + g) + 8*hh + i
  bool glive[kCPW];
#pragma unroll
  for (int g = 0; g < kCPW; ++g) glive[g] = (wave * kCPW + g) * 16 < nch;

  // low-rank: filter-MFMA A fragments [g][p][th][kq]
  bf16x8 af[KIND == DYNCONV_LOWRANK ? kCPW : 1][2][THP][KQ];
  if constexpr (KIND == DYNCONV_LOWRANK) {
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      const int64_t gg = (cblk >> 4) + wave * kCPW + g;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int th = 0; th < THP; ++th)
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) {
            const int64_t rowf = ((gg * 2 + p) * THP + th) * 32 + tl;
            af[g][p][th][kq] = glive[g] ? as_bf16x8(*reinterpret_cast<const uint4 *>(
                                              P.Uf + rowf * (KQ * 16) + kq * 16 + hh * 8))
                                        : zero_bf16x8();
          }
    }
  }

  // accumulators that live across tiles
  f32x4 dUacc[KIND == DYNCONV_LOWRANK ? kCPW : 1][KP][NCB];
  float dw0acc[kCPW][KP];
#pragma unroll
  for (int g = 0; g < kCPW; ++g)
#pragma unroll
    for (int rb = 0; rb < KP; ++rb) {
      dw0acc[g][rb] = 0.f;
      if constexpr (KIND == DYNCONV_LOWRANK)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) dUacc[g][rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // ---- prefetch state (next tile) -----------------------------------------
  const int chunks = nch / 8;                       // 16-byte chunks per x row
  constexpr int kXLoads = ((32 + KH) * (kDt / 8) + 255) / 256;
  uint4 xpre[kXLoads];
  uint4 dypre[kCPW];
  float genpre[KIND == DYNCONV_LOWRANK ? KQ * 8 : kCPW * 2 * KP];

  auto prefetch = [&](int tile) {
    const int64_t t0 = (int64_t)tile * 32;
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      const int e = threadIdx.x + q * 256;
      const int r = e / chunks, c16 = e - r * chunks;
      const int64_t row = t0 - KH + r;
      xpre[q] = make_uint4(0, 0, 0, 0);
      if (r < 32 + KH && row >= 0 && row < s.BT)
        xpre[q] = *reinterpret_cast<const uint4 *>(P.x + row * s.D + cblk + c16 * 8);
    }
    const int64_t t = t0 + tl;
    const bool tv = t < s.BT;
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      const int64_t c = cblk + (wave * kCPW + g) * 16 + hh * 8;
      dypre[g] = (tv && glive[g]) ? *reinterpret_cast<const uint4 *>(P.dy + t * s.D + c)
                                  : make_uint4(0, 0, 0, 0);
    }
    if constexpr (KIND == DYNCONV_LOWRANK) {
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int q = kq * 16 + hh * 8 + i;
          genpre[kq * 8 + i] = (tv && q < s.rank) ? P.gen[t * s.rank + q] : (q == s.rank ? 1.f : 0.f);
        }
    } else {
#pragma unroll
      for (int g = 0; g < kCPW; ++g) {
        const int c = (int)cblk + (wave * kCPW + g) * 16 + hh * 8;
        const int ea = c / s.hd;
        const bool two = (c + 7) / s.hd != ea;
#pragma unroll
        for (int j = 0; j < KP; ++j) {
          genpre[(g * 2 + 0) * KP + j] = (tv && glive[g] && j < k) ? P.gen[t * s.N + ea * k + j] : 0.f;
          genpre[(g * 2 + 1) * KP + j] =
              (tv && glive[g] && j < k && two) ? P.gen[t * s.N + (ea + 1) * k + j] : 0.f;
        }
      }
    }
  };

  // filter of this lane's 8 channels of group g at its token: wv[i][j],
  // from the generator values gv (z of the token, or the u of its heads)
  auto filter = [&](int g, const float *gv, float (&wv)[8][KP]) {
    if constexpr (KIND == DYNCONV_LOWRANK) {
      bf16x8 bz[KQ];
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gv[kq * 8 + i];
        bz[kq] = pack_bf16x8(v);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int th = 0; th < THP; ++th) {
          f32x16 acc = {};
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) acc = mfma32(af[g][p][th][kq], bz[kq], acc);
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[4 * p + b][4 * th + r] = acc[4 * b + r];
        }
    } else {
      const int cl = (wave * kCPW + g) * 16 + hh * 8;  // block-local channel
      const int ea = (int)(cblk + cl) / s.hd;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool second = (int)(cblk + cl + i) / s.hd != ea;
#pragma unroll
        for (int j = 0; j < KP; ++j)
          wv[i][j] = (j < k ? gv[(g * 2 + (second ? 1 : 0)) * KP + j] : 0.f) + w0s[(cl + i) * KP + j];
      }
    }
  };

  __syncthreads();  // w0s ready

  // ---- right halo: products of the tile after this block's range ----------
  if (tile_hi < P.n_tiles) {
    prefetch(tile_hi);
    const int64_t t = (int64_t)tile_hi * 32 + tl;
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      float wv[8][KP];
      filter(g, genpre, wv);
      float dyv[8];
      unpack8(dypre[g], dyv);
      if (tl < KH)
#pragma unroll
        for (int j = 1; j < KP; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pc[wave][g][j - 1][tl][hh][i] = (t < s.BT && j < k) ? wv[i][j] * dyv[i] : 0.f;
    }
  } else if (tl < KH) {
#pragma unroll
    for (int g = 0; g < kCPW; ++g)
#pragma unroll
      for (int j = 1; j < KP; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) pc[wave][g][j - 1][tl][hh][i] = 0.f;
  }

  if (tile_hi > tile_lo) prefetch(tile_hi - 1);

  int buf = 0;
  for (int tile = tile_hi - 1; tile >= tile_lo; --tile, buf ^= 1) {
    const int64_t t0 = (int64_t)tile * 32;
    const int64_t t = t0 + tl;
    const bool tv = t < s.BT;
    const int pos = tv ? (int)(t % s.T) : 0;

    // ---- stage x (and z^T) of this tile from the prefetch registers ----
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      const int e = threadIdx.x + q * 256;
      const int r = e / chunks, c16 = e - r * chunks;
      if (r < 32 + KH) *reinterpret_cast<uint4 *>(xs[buf] + r * kRowB + c16 * 16) = xpre[q];
    }
    uint4 dycur[kCPW];
#pragma unroll
    for (int g = 0; g < kCPW; ++g) dycur[g] = dypre[g];
    float gencur[KIND == DYNCONV_LOWRANK ? KQ * 8 : kCPW * 2 * KP];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(gencur) / sizeof(float)); ++i) gencur[i] = genpre[i];
    if constexpr (KIND == DYNCONV_LOWRANK) {
      // z^T tile: zt[q][token], bf16, rows of 80 bytes (tokens 0..31)
      for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int q = e >> 5, tt = e & 31;
        const int64_t row = t0 + tt;
        const float zv = (row < s.BT && q < s.rank) ? P.gen[row * s.rank + q] : 0.f;
        *reinterpret_cast<bf16 *>(zt[buf] + q * kGtRowB + tt * 2) = (bf16)zv;
      }
    }
    __syncthreads();
    if (tile - 1 >= tile_lo) prefetch(tile - 1);

    f32x16 dzacc = {};
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      if (!glive[g]) continue;
      const int cl = (wave * kCPW + g) * 16 + hh * 8;
      float xv[KP][8];
#pragma unroll
      for (int j = 0; j < KP; ++j)
        unpack8(*reinterpret_cast<const uint4 *>(xs[buf] + (tl + KH - j) * kRowB + cl * 2), xv[j]);
      float dyv[8];
      unpack8(dycur[g], dyv);
      float wv[8][KP];
      filter(g, gencur, wv);

      // G and the products for dx
      float G[8][KP];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < KP; ++j) G[i][j] = (tv && j <= pos && j < k) ? dyv[i] * xv[j][i] : 0.f;

      float dxv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) dxv[i] = dyv[i] + (tv ? wv[i][0] * dyv[i] : 0.f);
#pragma unroll
      for (int j = 1; j < KP; ++j) {
        const bool ok = tv && j < k && pos + j <= s.T - 1 && t + j < s.BT;
        const bool from_next = tl + j >= 32;
        const int src = lane + j;  // same half when !from_next
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float mine = tv ? wv[i][j] * dyv[i] : 0.f;
          float v = __shfl(mine, src & 63);
          if (from_next) v = pc[wave][g][j - 1][tl + j - 32][hh][i];
          if (ok) dxv[i] += v;
        }
      }
      // carry this tile's first k-1 tokens' products to the tile below
      if (tl < KH)
#pragma unroll
        for (int j = 1; j < KP; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) pc[wave][g][j - 1][tl][hh][i] = (tv && j < k) ? wv[i][j] * dyv[i] : 0.f;
      if (tv) store_vec(P.dx + t * s.D + cblk + cl, dxv);

      // dz / du: B operand = G of this lane, 8 (channel, tap) values per step
#pragma unroll
      for (int st = 0; st < KP; ++st) {
        float bv[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int e = 8 * st + e8;
          bv[e8] = G[e / KP][e % KP];
        }
        const bf16x8 b = pack_bf16x8(bv);
        bf16x8 a;
        if constexpr (KIND == DYNCONV_LOWRANK) {
          const int64_t gg = (cblk >> 4) + wave * kCPW + g;
          a = as_bf16x8(*reinterpret_cast<const uint4 *>(
              P.Udz + (((gg * KP + st) * 32 + tl) * 2 + hh) * 8));
        } else {
          // 0/1 head membership: row tl = slot*KP + j', column (channel, tap)
          const int slot = tl / KP, jr = tl % KP;
          float av[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) {
            const int e = 8 * st + e8;
            const int c = (int)cblk + (wave * kCPW + g) * 16 + hh * 8 + e / KP;
            av[e8] = (e % KP == jr && jr < k && c / s.hd - e_base == slot) ? 1.f : 0.f;
          }
          a = pack_bf16x8(av);
        }
        dzacc = mfma32(a, b, dzacc);
      }

      // transposed G for dU / dw0: row (channel-in-group, tap), column token
      unsigned char *gtw = gt[wave][g];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < KP; ++j)
          *reinterpret_cast<bf16 *>(gtw + ((hh * 8 + i) * KP + j) * kGtRowB + tl * 2) = (bf16)G[i][j];
    }

    // ---- cross-wave dz / du sum, dU and dw0 accumulation ----
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][lane][e] = dzacc[e];
    __syncthreads();
    {
      const int rg = threadIdx.x >> 5, tt = threadIdx.x & 31;  // rows 4rg..4rg+3, token tt
      const int src = 32 * (rg & 1) + tt, el = 4 * (rg >> 1);
      float sum[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] = red[0][src][el + r];
#pragma unroll
      for (int w = 1; w < 4; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[r] += red[w][src][el + r];
      const int64_t row = t0 + tt;
      if (row < s.BT) {
        float *dst = P.gpart + ((int64_t)blockIdx.x * s.BT + row) * P.R;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * rg + r;
          if constexpr (KIND == DYNCONV_LOWRANK) {
            if (m < s.rank) dst[m] = sum[r];
          } else {
            const int slot = m / KP, jr = m % KP;
            if (slot < P.SL && jr < k) dst[slot * k + jr] = sum[r];
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      if (!glive[g]) continue;
      const unsigned char *gtr = gt[wave][g];
#pragma unroll
      for (int rb = 0; rb < KP; ++rb) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(gtr + (rb * 16 + (lane & 15)) * kGtRowB +
                                                           (lane >> 4) * 16);
        float gv[8];
        unpack8(raw, gv);
        float sacc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sacc += gv[i];
        dw0acc[g][rb] += sacc;
        if constexpr (KIND == DYNCONV_LOWRANK) {
          const bf16x8 a = as_bf16x8(raw);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(
                zt[buf] + (cb * 16 + (lane & 15)) * kGtRowB + (lane >> 4) * 16));
            dUacc[g][rb][cb] = mfma16(a, b, dUacc[g][rb][cb]);
          }
        }
      }
    }
  }

  // ---- block epilogue: dU and dw0 partials of this token range ----
  const int64_t Dk = s.D * k;
#pragma unroll
  for (int g = 0; g < kCPW; ++g) {
#pragma unroll
    for (int rb = 0; rb < KP; ++rb) {
      // dw0: lanes with the same lane%16 hold the same row; add the 4 token chunks
      float v = dw0acc[g][rb];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      const int row = rb * 16 + (lane & 15);  // (channel-in-group, tap) row
      const int cg = row / KP, j = row % KP;
      const int64_t c = cblk + (wave * kCPW + g) * 16 + cg;
      if (glive[g] && lane < 16 && j < k) P.dw0p[(int64_t)blockIdx.y * Dk + c * k + j] = v;
      if constexpr (KIND == DYNCONV_LOWRANK) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = rb * 16 + (lane >> 4) * 4 + i;  // D row of the 16x16 fragment
            const int q = cb * 16 + (lane & 15);
            const int cg2 = rr / KP, j2 = rr % KP;
            const int64_t c2 = cblk + (wave * kCPW + g) * 16 + cg2;
            if (glive[g] && q < s.rank && j2 < k)
              P.dUp[((int64_t)blockIdx.y * s.rank + q) * Dk + c2 * k + j2] = dUacc[g][rb][cb][i];
          }
      }
    }
  }
}

// dz-MFMA A fragments: Udz[((g*KP + st)*32 + q)*2 + hh][e8] = U[q, c*k + j] with
// e = 8*st + e8, c = 16g + 8hh + e/KP, j = e%KP (0 if q >= r or j >= k).
__global__ void __launch_bounds__(256)
k_prep_dz(Shape s, const bf16 *__restrict__ U, bf16 *__restrict__ Udz, int KP) {
  const int64_t total = (s.D / 16) * KP * 32 * 2 * 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int e8 = (int)(idx % 8);
  int64_t rest = idx / 8;
  const int hh = (int)(rest % 2);
  rest /= 2;
  const int q = (int)(rest % 32);
  rest /= 32;
  const int st = (int)(rest % KP);
  const int64_t g = rest / KP;
  const int e = 8 * st + e8;
  const int64_t c = 16 * g + 8 * hh + e / KP;
  const int j = e % KP;
  float v = 0.f;
  if (q < s.rank && j < s.k) v = (float)U[(int64_t)q * s.D * s.k + c * s.k + j];
  Udz[idx] = (bf16)v;
}

}  // namespace bwd

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
BwdLayout bwd_layout(const Shape &s) {
  BwdLayout L;
  L.KP = s.k <= 4 ? 4 : 8;
  L.n_slices = (int)ceil_div(s.D, bwd::kDt);
  L.n_tiles = (int)ceil_div(s.BT, 32);
  // token ranges: as few as keep ~512 blocks in one round
  const int target = 512;
  int tpb = 1;
  while ((int64_t)L.n_slices * ceil_div(L.n_tiles, tpb) > target) ++tpb;
  L.tpb = tpb;
  L.n_ranges = (int)ceil_div(L.n_tiles, tpb);
  if (s.kind == DYNCONV_LOWRANK) {
    L.SL = 0;
    L.R = s.rank;
  } else {
    int sl = 0;
    for (int d = 0; d < L.n_slices; ++d) {
      const int64_t c0 = (int64_t)d * bwd::kDt;
      const int64_t c1 = (s.D < c0 + bwd::kDt ? s.D : c0 + bwd::kDt) - 1;
      const int n = (int)(c1 / s.hd - c0 / s.hd + 1);
      if (n > sl) sl = n;
    }
    L.SL = sl;
    L.R = sl * s.k;
  }
  return L;
}

bool bwd_fused_supported(const Shape &s) {
  if (s.D % 16 != 0) return false;
  const int KP = s.k <= 4 ? 4 : 8;
  if (s.kind == DYNCONV_LOWRANK) return s.rank <= 32 && fwd_lowrank_supported(s);
  if (s.hd < 8) return false;
  return bwd_layout(s).SL * KP <= 32;
}

size_t bwd_prep_dz_bytes(const Shape &s) {
  const int KP = s.k <= 4 ? 4 : 8;
  return s.kind == DYNCONV_LOWRANK ? (size_t)(s.D / 16) * KP * 32 * 2 * 8 * sizeof(bf16) : 0;
}

int prep_dz_frags(const Shape &s, const void *U, void *Udz, hipStream_t st) {
  const int KP = s.k <= 4 ? 4 : 8;
  const int64_t total = (s.D / 16) * KP * 32 * 2 * 8;
  hipLaunchKernelGGL(bwd::k_prep_dz, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, st, s,
                     (const bf16 *)U, (bf16 *)Udz, KP);
  return 0;
}

int bwd_conv(const Shape &s, const BwdLayout &L, const float *gen, const void *Uf, const void *Udz,
             const void *w0, const void *x, const void *dy, void *dx, float *gpart, float *dUp,
             float *dw0p, hipStream_t st) {
  bwd::Params P;
  P.s = s;
  P.x = (const bf16 *)x;
  P.dy = (const bf16 *)dy;
  P.dx = (bf16 *)dx;
  P.gen = gen;
  P.Uf = (const bf16 *)Uf;
  P.Udz = (const bf16 *)Udz;
  P.w0 = (const bf16 *)w0;
  P.gpart = gpart;
  P.dUp = dUp;
  P.dw0p = dw0p;
  P.tpb = L.tpb;
  P.n_tiles = L.n_tiles;
  P.SL = L.SL;
  P.R = L.R;
  dim3 grid((unsigned)L.n_slices, (unsigned)L.n_ranges);
  const bool tr = trace_begin(DYNCONV_K_BWD_CONV, st);
  int rc = 0;
  if (s.kind == DYNCONV_LOWRANK) {
    const int KQ = (int)ceil_div(s.rank + 1, 16);
    const int NCB = (int)ceil_div(s.rank, 16);
#define L_LR(KP_, KQ_, NCB_) \
  hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_LOWRANK, KP_, KQ_, NCB_>), grid, dim3(256), 0, st, P)
    if (L.KP == 4) {
      if (KQ == 1 && NCB == 1) L_LR(4, 1, 1);
      else if (KQ == 2 && NCB == 1) L_LR(4, 2, 1);
      else if (KQ == 2 && NCB == 2) L_LR(4, 2, 2);
      else if (KQ == 3 && NCB == 2) L_LR(4, 3, 2);
      else rc = DYNCONV_E_LIMIT;
    } else {
      if (KQ == 1 && NCB == 1) L_LR(8, 1, 1);
      else if (KQ == 2 && NCB == 1) L_LR(8, 2, 1);
      else if (KQ == 2 && NCB == 2) L_LR(8, 2, 2);
      else if (KQ == 3 && NCB == 2) L_LR(8, 3, 2);
      else rc = DYNCONV_E_LIMIT;
    }
#undef L_LR
  } else {
    if (L.KP == 4)
      hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 4, 1, 1>), grid, dim3(256), 0, st, P);
    else
      hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 8, 1, 1>), grid, dim3(256), 0, st, P);
  }
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
