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

constexpr int kW = 8;               // waves per block
constexpr int kCPW = 1;             // 16-channel groups per wave
constexpr int kDt = kW * kCPW * 16; // channels per block
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const uint4 &raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int KIND, int K, int KQ, int NCB>
__global__ void __launch_bounds__(kW * 64, 2)
k_bwd(Params P) {
  constexpr int KP = 4;             // taps padded to 4 in the fragment layouts
  constexpr int KH = K - 1;         // history rows of x (left halo)
  constexpr int KHA = KH > 0 ? KH : 1;
  constexpr int GROWS = 16 * KP;    // (channel, tap) rows of one 16-channel group
  constexpr bool LR = KIND == DYNCONV_LOWRANK;
  constexpr int ZW = KQ * 16;       // low-rank: z columns used (rank, bias row, zero padding)
  constexpr int ZWP = ZW + 8;       // padded row of the z tile (bf16)
  constexpr int UWP = 8 * KP + 4;   // head-wise: padded row of the u tile (8 head slots, fp32)
  constexpr int RB = LR ? 2 * NCB : 4;  // 8-row blocks of the 32x32 dz result that are used
  constexpr int RS = RB * 4 + 4;    // padded lane stride of the reduction buffer (floats)
  constexpr int NT = kW * 64;
  const Shape &s = P.s;

  __shared__ __attribute__((aligned(16))) unsigned char xs[2][(32 + KH) * kRowB];
  __shared__ __attribute__((aligned(16))) unsigned char dys[2][32 * kRowB];
  __shared__ __attribute__((aligned(16))) unsigned char gt[kW][GROWS * kGtRowB];
  __shared__ __attribute__((aligned(16))) bf16 zs[2][LR ? 32 * ZWP : 8];
  __shared__ __attribute__((aligned(16))) unsigned char zt[2][LR ? 32 * kGtRowB : 16];
  __shared__ __attribute__((aligned(16))) float us[2][LR ? 4 : 32 * UWP];
  __shared__ __attribute__((aligned(16))) float red[kW][64 * RS];
  __shared__ __attribute__((aligned(16))) float pc[kW][2][KHA][KHA][2][4];
  __shared__ __attribute__((aligned(16))) float w0s[LR ? 4 : kDt * KP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int64_t cblk = (int64_t)blockIdx.x * kDt;
  const int nch = (int)min<int64_t>(kDt, s.D - cblk);
  const int tile_lo = blockIdx.y * P.tpb;
  const int tile_hi = min(P.n_tiles, tile_lo + P.tpb);  // exclusive
  const int e_base = LR ? 0 : (int)(cblk / s.hd);
  const bool glive = wave * 16 < nch;     // this wave's 16-channel group exists
  const int cl = wave * 16 + hh * 8;      // block-local first channel of the lane's 8

  // ---- block-constant LDS ----
  if constexpr (!LR) {
    for (int e = threadIdx.x; e < kDt * KP; e += NT) {
      const int c = e / KP, j = e - c * KP;
      w0s[e] = (P.w0 && c < nch && j < K) ? (float)P.w0[(cblk + c) * K + j] : 0.f;
    }
  } else {
    for (int e = threadIdx.x; e < 2 * 32 * ZWP; e += NT) {
      const int q = e % ZWP;
      if (q >= s.rank) (&zs[0][0])[e] = (bf16)(q == s.rank ? 1.f : 0.f);
    }
    for (int e = threadIdx.x; e < 2 * 32 * 32; e += NT) {
      const int b = e >> 10, q = (e >> 5) & 31, tt = e & 31;
      if (q >= s.rank) *reinterpret_cast<bf16 *>(zt[b] + q * kGtRowB + tt * 2) = (bf16)0.f;
    }
  }

  // ---- per-lane constants ----
  bf16x8 af[LR ? 2 : 1][KQ];  // filter-MFMA A fragments, quads p = 0, 1 (low-rank)
  bf16x8 adz[LR ? KP : 1];    // dz-MFMA A fragments (low-rank)
  int sa = 0, nxt = 0;        // head-wise: slot of the lane's first head; next-head mask
  {
    const int64_t gg = (cblk >> 4) + wave;
    if constexpr (LR) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
          af[p][kq] = glive ? as_bf16x8(*reinterpret_cast<const uint4 *>(
                                  P.Uf + ((gg * 2 + p) * 32 + tl) * (KQ * 16) + kq * 16 + hh * 8))
                            : zero_bf16x8();
#pragma unroll
      for (int st = 0; st < KP; ++st)
        adz[st] = glive ? as_bf16x8(*reinterpret_cast<const uint4 *>(
                              P.Udz + (((gg * KP + st) * 32 + tl) * 2 + hh) * 8))
                        : zero_bf16x8();
    } else {
      const int c0 = (int)cblk + cl;
      const int ea = c0 / s.hd;
      sa = ea - e_base;
#pragma unroll
      for (int i = 0; i < 8; ++i) nxt |= ((c0 + i) / s.hd != ea) << i;
    }
  }

  f32x4 dUacc[LR ? KP : 1][NCB];
  float dw0acc[KP];
#pragma unroll
  for (int rb = 0; rb < KP; ++rb) {
    dw0acc[rb] = 0.f;
    if constexpr (LR)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) dUacc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- prefetch: x rows (with history) and dy rows as 16-byte chunks; z or u ----
  constexpr int CH = kDt / 8;  // 16-byte chunks per full row
  const int ex = (32 + KH) * CH;
  constexpr int kVLoads = ((32 + KH + 32) * CH + NT - 1) / NT;
  constexpr int kSLoads = LR ? (32 * ZW + NT - 1) / NT : (32 * 8 * KP + NT - 1) / NT;
  uint4 vpre[kVLoads];
  float spre[kSLoads];

  auto prefetch = [&](int tile) {
    const int64_t t0 = (int64_t)tile * 32;
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) {
      const int e = threadIdx.x + q * NT;
      vpre[q] = make_uint4(0, 0, 0, 0);
      const bool isx = e < ex;
      const int e2 = isx ? e : e - ex;
      const int r = e2 / CH, c16 = e2 % CH;
      const int64_t row = isx ? t0 - KH + r : t0 + r;
      if (r < (isx ? 32 + KH : 32) && c16 * 8 < nch && row >= 0 && row < s.BT)
        vpre[q] = *reinterpret_cast<const uint4 *>((isx ? P.x : P.dy) + row * s.D + cblk + c16 * 8);
    }
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) {
      const int e = threadIdx.x + q * NT;
      spre[q] = 0.f;
      if constexpr (LR) {
        const int tt = e / ZW, qq = e % ZW;
        const int64_t row = t0 + tt;
        if (tt < 32 && qq < s.rank && row < s.BT) spre[q] = P.gen[row * s.rank + qq];
      } else {
        const int tt = e / (8 * KP), rem = e % (8 * KP);
        const int slot = rem / KP, j = rem % KP;
        const int64_t row = t0 + tt;
        if (tt < 32 && j < K && slot < P.SL && e_base + slot < s.n_heads && row < s.BT)
          spre[q] = P.gen[row * s.N + (e_base + slot) * K + j];
      }
    }
  };
  auto stage = [&](int b) {
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) {
      const int e = threadIdx.x + q * NT;
      const bool isx = e < ex;
      const int e2 = isx ? e : e - ex;
      const int r = e2 / CH, c16 = e2 % CH;
      if (r < (isx ? 32 + KH : 32))
        *reinterpret_cast<uint4 *>((isx ? xs[b] : dys[b]) + r * kRowB + c16 * 16) = vpre[q];
    }
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) {
      const int e = threadIdx.x + q * NT;
      if constexpr (LR) {
        const int tt = e / ZW, qq = e % ZW;
        if (tt < 32 && qq < s.rank) {
          const bf16 v = (bf16)spre[q];
          zs[b][tt * ZWP + qq] = v;
          *reinterpret_cast<bf16 *>(zt[b] + qq * kGtRowB + tt * 2) = v;
        }
      } else {
        const int tt = e / (8 * KP), rem = e % (8 * KP);
        if (tt < 32) us[b][tt * UWP + rem] = spre[q];
      }
    }
  };

  // filter taps of channels 4p..4p+3 of the lane's 8, at tile row tt of buffer b: w[b4][j]
  auto filter_quad = [&](int b, int p, int tt, float (&w)[4][KP]) {
    if constexpr (LR) {
      f32x16 acc = {};
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        acc = mfma32(af[p][kq],
                     as_bf16x8(*reinterpret_cast<const uint4 *>(&zs[b][tt * ZWP + kq * 16 + hh * 8])), acc);
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
        for (int r = 0; r < 4; ++r) w[b4][r] = acc[4 * b4 + r];
    } else {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int i = 4 * p + b4;
        const int slot = sa + ((nxt >> i) & 1);
        const float4 uv = *reinterpret_cast<const float4 *>(&us[b][tt * UWP + slot * KP]);
        const float4 b0 = *reinterpret_cast<const float4 *>(&w0s[(cl + i) * KP]);
        w[b4][0] = uv.x + b0.x;
        w[b4][1] = uv.y + b0.y;
        w[b4][2] = uv.z + b0.z;
        w[b4][3] = uv.w + b0.w;
      }
    }
  };

  // ---- right halo: the products of the tile after this block's range ----
  if (tile_hi < P.n_tiles) {
    prefetch(tile_hi);
    stage(1);
  }
  __syncthreads();
  if (KH > 0 && tl < KH) {
    const bool have = tile_hi < P.n_tiles;
    float dyv[8];
    unpack8(*reinterpret_cast<const uint4 *>(dys[1] + tl * kRowB + cl * 2), dyv);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float w[4][KP];
      filter_quad(1, p, tl, w);
#pragma unroll
      for (int j = 1; j <= KH; ++j)
        *reinterpret_cast<float4 *>(&pc[wave][p][j - 1][tl][hh][0]) =
            have ? make_float4(w[0][j] * dyv[4 * p], w[1][j] * dyv[4 * p + 1], w[2][j] * dyv[4 * p + 2],
                               w[3][j] * dyv[4 * p + 3])
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  if (tile_hi > tile_lo) prefetch(tile_hi - 1);

  int buf = 0;
  for (int tile = tile_hi - 1; tile >= tile_lo; --tile, buf ^= 1) {
    const int64_t t0 = (int64_t)tile * 32;
    const int64_t t = t0 + tl;
    const bool tv = t < s.BT;
    const int pos = (int)(t % s.T);

    stage(buf);
    __syncthreads();
    if (tile - 1 >= tile_lo) prefetch(tile - 1);

    f32x16 dzacc = {};
    if (glive) {
      // x history rows, masked where they precede this token's sequence
      uint4 xr[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        xr[j] = *reinterpret_cast<const uint4 *>(xs[buf] + (tl + KH - j) * kRowB + cl * 2);
        if (j > pos) xr[j] = make_uint4(0, 0, 0, 0);
      }
      const uint4 dyraw = *reinterpret_cast<const uint4 *>(dys[buf] + tl * kRowB + cl * 2);
      float dyv[8];
      unpack8(dyraw, dyv);
      // dy as bf16 pairs with one half cleared: G = x * dy by a bf16 dot product
      uint32_t dylo[4], dyhi[4];
      {
        const uint32_t d4[4] = {dyraw.x, dyraw.y, dyraw.z, dyraw.w};
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          dylo[w2] = d4[w2] & 0x0000ffffu;
          dyhi[w2] = d4[w2] & 0xffff0000u;
        }
      }
      bool ok[KHA];
#pragma unroll
      for (int j = 1; j <= KH; ++j) ok[j - 1] = tv && pos + j <= s.T - 1 && t + j < s.BT;
      float dxv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) dxv[i] = dyv[i];
      unsigned char *gtw = gt[wave];

#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float w[4][KP];
        filter_quad(buf, p, tl, w);
        float G[4][KP];
        float pj[4][KP];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int i = 4 * p + b4;
#pragma unroll
          for (int j = 0; j < KP; ++j) {
            if (j < K) {
              const uint32_t xw = (&xr[j].x)[i >> 1];
              const uint32_t dw = (i & 1) ? dyhi[i >> 1] : dylo[i >> 1];
              G[b4][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw),
                                                         __builtin_bit_cast(bf16x2_t, dw), 0.f, false);
              pj[b4][j] = w[b4][j] * dyv[i];
            } else {
              G[b4][j] = 0.f;
              pj[b4][j] = 0.f;
            }
          }
          dxv[i] += pj[b4][0];
        }
        // products of the next j tokens, by lane shuffles; the last j lanes take
        // the values carried from the tile above
#pragma unroll
        for (int j = 1; j <= KH; ++j) {
          float4 prev = make_float4(0.f, 0.f, 0.f, 0.f);
          if (tl < j) prev = *reinterpret_cast<const float4 *>(&pc[wave][p][j - 1][tl][hh][0]);
          const int src = hh * 32 + ((tl + j) & 31);
          const float v0 = __shfl(tl < j ? prev.x : pj[0][j], src);
          const float v1 = __shfl(tl < j ? prev.y : pj[1][j], src);
          const float v2 = __shfl(tl < j ? prev.z : pj[2][j], src);
          const float v3 = __shfl(tl < j ? prev.w : pj[3][j], src);
          if (ok[j - 1]) {
            dxv[4 * p + 0] += v0;
            dxv[4 * p + 1] += v1;
            dxv[4 * p + 2] += v2;
            dxv[4 * p + 3] += v3;
          }
        }
        if (tl < KH)
#pragma unroll
          for (int j = 1; j <= KH; ++j)
            *reinterpret_cast<float4 *>(&pc[wave][p][j - 1][tl][hh][0]) =
                make_float4(pj[0][j], pj[1][j], pj[2][j], pj[3][j]);

        // dz / du: G of this quad is the B operand of steps 2p, 2p+1
#pragma unroll
        for (int sq = 0; sq < 2; ++sq) {
          const int st = 2 * p + sq;
          float bv[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) bv[e8] = G[2 * sq + e8 / KP][e8 % KP];
          bf16x8 a;
          if constexpr (LR) {
            a = adz[st];
          } else {
            // 0/1 head membership: row tl = slot*KP + jr, column (channel, tap)
            const int slot = tl / KP, jr = tl % KP;
            float av[8];
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) {
              const int i = 2 * st + e8 / KP, j = e8 % KP;
              av[e8] = (j == jr && jr < K && sa + ((nxt >> i) & 1) == slot) ? 1.f : 0.f;
            }
            a = pack_bf16x8(av);
          }
          const bf16x8 bb = pack_bf16x8(bv);
          dzacc = mfma32(a, bb, dzacc);
          // transposed G for dU / dw0: row ((channel*KP + tap)*2 + half), column token
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) {
            const int i = 2 * st + e8 / KP, j = e8 % KP;
            *reinterpret_cast<bf16 *>(gtw + ((i * KP + j) * 2 + hh) * kGtRowB + tl * 2) = bb[e8];
          }
        }
      }
      if (tv) store_vec(P.dx + t * s.D + cblk + cl, dxv);

      // dU and dw0 from this group's G^T (written by this wave; LDS is in order per wave)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int rb = 0; rb < KP; ++rb) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(gtw + (rb * 16 + (lane & 15)) * kGtRowB +
                                                           (lane >> 4) * 16);
        const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
        float sacc = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          sacc += __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, r4[w2]),
                                                  __builtin_bit_cast(bf16x2_t, 0x3f803f80u), 0.f, false);
        dw0acc[rb] += sacc;
        if constexpr (LR) {
          const bf16x8 a = as_bf16x8(raw);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const bf16x8 bz = as_bf16x8(*reinterpret_cast<const uint4 *>(
                zt[buf] + (cb * 16 + (lane & 15)) * kGtRowB + (lane >> 4) * 16));
            dUacc[rb][cb] = mfma16(a, bz, dUacc[rb][cb]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- cross-wave dz / du sum -> per-slice partial ----
    // lane holds rows 8b + 4hh + r of the 32x32 result in element 4b + r
#pragma unroll
    for (int e4 = 0; e4 < RB; ++e4)
      *reinterpret_cast<float4 *>(&red[wave][lane * RS + 4 * e4]) =
          make_float4(dzacc[4 * e4], dzacc[4 * e4 + 1], dzacc[4 * e4 + 2], dzacc[4 * e4 + 3]);
    __syncthreads();
    if (threadIdx.x < 64 * RB) {
      const int rg = threadIdx.x >> 5, tt = threadIdx.x & 31;  // rows 4rg..4rg+3, token tt
      const int src = 32 * (rg & 1) + tt, el = 4 * (rg >> 1);
      float4 sum = *reinterpret_cast<const float4 *>(&red[0][src * RS + el]);
#pragma unroll
      for (int w = 1; w < kW; ++w) {
        const float4 v = *reinterpret_cast<const float4 *>(&red[w][src * RS + el]);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
      }
      const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
      const int64_t row = t0 + tt;
      if (row < s.BT) {
        float *dst = P.gpart + ((int64_t)blockIdx.x * s.BT + row) * P.R;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * rg + r;
          if constexpr (LR) {
            if (m < s.rank) dst[m] = sv[r];
          } else {
            const int slot = m / KP, jr = m % KP;
            if (slot < P.SL && jr < K) dst[slot * K + jr] = sv[r];
          }
        }
      }
    }
  }

  // ---- block epilogue: dU and dw0 partials of this token range ----
  const int64_t Dk = s.D * K;
#pragma unroll
  for (int rb = 0; rb < KP; ++rb) {
    // dw0: lanes with the same lane%16 hold the same row; add the 4 token chunks
    float v = dw0acc[rb];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    {
      const int row = rb * 16 + (lane & 15);  // ((channel*KP + tap)*2 + half)
      const int half = row & 1, ci = (row >> 1) / KP, j = (row >> 1) % KP;
      const int64_t c = cblk + wave * 16 + half * 8 + ci;
      if (glive && lane < 16 && j < K) P.dw0p[(int64_t)blockIdx.y * Dk + c * K + j] = v;
    }
    if constexpr (LR) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = rb * 16 + (lane >> 4) * 4 + i;  // D row of the 16x16 fragment
          const int q = cb * 16 + (lane & 15);
          const int half = rr & 1, ci = (rr >> 1) / KP, j2 = (rr >> 1) % KP;
          const int64_t c2 = cblk + wave * 16 + half * 8 + ci;
          if (glive && q < s.rank && j2 < K)
            P.dUp[((int64_t)blockIdx.y * s.rank + q) * Dk + c2 * K + j2] = dUacc[rb][cb][i];
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
  // token ranges: as few as keep every block resident in one round (one
  // 512-thread block per CU: its LDS and 2 waves per SIMD)
  const int target = 256;
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
  if (s.D % 16 != 0 || s.k > 4) return false;
  const int KP = 4;
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
  const dim3 block(bwd::kW * 64);
  if (s.kind == DYNCONV_LOWRANK) {
    const int KQ = (int)ceil_div(s.rank + 1, 16);
    const int NCB = (int)ceil_div(s.rank, 16);
#define L_LR(K_, KQ_, NCB_) \
  hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_LOWRANK, K_, KQ_, NCB_>), grid, block, 0, st, P)
#define L_K(K_)                                   \
  if (KQ == 1 && NCB == 1) L_LR(K_, 1, 1);        \
  else if (KQ == 2 && NCB == 1) L_LR(K_, 2, 1);   \
  else if (KQ == 2 && NCB == 2) L_LR(K_, 2, 2);   \
  else if (KQ == 3 && NCB == 2) L_LR(K_, 3, 2);   \
  else rc = DYNCONV_E_LIMIT;
    switch (s.k) {
      case 1: L_K(1) break;
      case 2: L_K(2) break;
      case 3: L_K(3) break;
      case 4: L_K(4) break;
      default: rc = DYNCONV_E_LIMIT;
    }
#undef L_K
#undef L_LR
  } else {
    switch (s.k) {
      case 1: hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 1, 1, 1>), grid, block, 0, st, P); break;
      case 2: hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 2, 1, 1>), grid, block, 0, st, P); break;
      case 3: hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 3, 1, 1>), grid, block, 0, st, P); break;
      case 4: hipLaunchKernelGGL((bwd::k_bwd<DYNCONV_HEADWISE, 4, 1, 1>), grid, block, 0, st, P); break;
      default: rc = DYNCONV_E_LIMIT;
    }
  }
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
