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
  constexpr int KH = K - 1;         // history rows of x (left halo) = lookahead rows of dy, z, u
  constexpr int GROWS = 16 * KP;    // (channel, tap) rows of one 16-channel group
  constexpr bool LR = KIND == DYNCONV_LOWRANK;
  constexpr int ZW = KQ * 16;       // low-rank: z columns used (rank, bias row, zero padding)
  constexpr int ZWP = ZW + 8;       // padded row of the z tile (bf16)
  constexpr int UWP = 8 * KP + 4;   // head-wise: padded row of the u tile (8 head slots, fp32)
  constexpr int RB = LR ? 2 * NCB : 4;  // 8-row blocks of the 32x32 dz result that are used
  constexpr int RS = RB * 4 + 4;    // padded lane stride of the reduction buffer (floats)
  constexpr int NT = kW * 64;
  constexpr int TR = 32 + KH;       // rows of each staged tile
  const Shape &s = P.s;

  __shared__ __attribute__((aligned(16))) unsigned char xs[2][TR * kRowB];   // x rows t0-KH .. t0+31
  __shared__ __attribute__((aligned(16))) unsigned char dys[2][TR * kRowB];  // dy rows t0 .. t0+31+KH
  __shared__ __attribute__((aligned(16))) unsigned char gt[kW][GROWS * kGtRowB];
  __shared__ __attribute__((aligned(16))) bf16 zs[2][LR ? TR * ZWP : 8];     // z rows t0 .. t0+31+KH
  __shared__ __attribute__((aligned(16))) unsigned char zt[2][LR ? 32 * kGtRowB : 16];
  __shared__ __attribute__((aligned(16))) float us[2][LR ? 4 : TR * UWP];    // u rows t0 .. t0+31+KH
  __shared__ __attribute__((aligned(16))) float red[kW][64 * RS];
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
    for (int e = threadIdx.x; e < 2 * TR * ZWP; e += NT) {
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

  // ---- per-thread load slots, fixed for the block ----
  constexpr int CH = kDt / 8;  // 16-byte chunks per full row
  constexpr int kVLoads = (2 * TR * CH + NT - 1) / NT;
  constexpr int SW = LR ? ZW : 8 * KP;  // scalar columns staged per row
  constexpr int kSLoads = (TR * SW + NT - 1) / NT;
  // per-thread load slots (constant divisors: cheap to recompute each time)
  auto vslot = [&](int q, bool &isx, bool &ok, int &row, int &goff, int &loff) {
    const int e = threadIdx.x + q * NT;
    isx = e < TR * CH;
    const int e2 = isx ? e : e - TR * CH;
    const int r = e2 / CH, c16 = e2 % CH;
    ok = r < TR && c16 * 8 < nch;
    row = isx ? r - KH : r;
    goff = c16 * 8;
    loff = r * kRowB + c16 * 16;
  };
  auto sslot = [&](int q, bool &ok, int &tt, int &col, int &loff) {
    const int e = threadIdx.x + q * NT;
    tt = e / SW;
    const int rem = e % SW;
    if constexpr (LR) {
      ok = tt < TR && rem < s.rank;
      col = rem;
    } else {
      const int slot = rem / KP, j = rem % KP;
      ok = tt < TR && j < K && slot < P.SL && e_base + slot < s.n_heads;
      col = (e_base + slot) * K + j;
    }
    loff = rem;
  };
  const int scol_stride = LR ? s.rank : s.N;
  uint4 vpre[kVLoads];
  float spre[kSLoads];

  auto prefetch = [&](int tile) {
    const int64_t t0 = (int64_t)tile * 32;
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) {
      bool isx, ok;
      int rr, goff, loff;
      vslot(q, isx, ok, rr, goff, loff);
      const int64_t row = t0 + rr;
      vpre[q] = make_uint4(0, 0, 0, 0);
      if (ok && row >= 0 && row < s.BT)
        vpre[q] = *reinterpret_cast<const uint4 *>((isx ? P.x : P.dy) + row * s.D + cblk + goff);
    }
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) {
      bool ok;
      int tt, col, loff;
      sslot(q, ok, tt, col, loff);
      const int64_t row = t0 + tt;
      spre[q] = (ok && row < s.BT) ? P.gen[row * scol_stride + col] : 0.f;
    }
  };
  auto stage = [&](int b) {
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) {
      bool isx, ok;
      int rr, goff, loff;
      vslot(q, isx, ok, rr, goff, loff);
      if (ok) *reinterpret_cast<uint4 *>((isx ? xs[b] : dys[b]) + loff) = vpre[q];
    }
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) {
      bool ok;
      int tt, col, loff;
      sslot(q, ok, tt, col, loff);
      if constexpr (LR) {
        if (ok) {
          const bf16 v = (bf16)spre[q];
          zs[b][tt * ZWP + loff] = v;
          if (tt < 32) *reinterpret_cast<bf16 *>(zt[b] + loff * kGtRowB + tt * 2) = v;
        }
      } else {
        if (tt < TR) us[b][tt * UWP + loff] = spre[q];
      }
    }
  };

  // The backward needs the filter only along its diagonal: tap j at token t+j,
  // wd[b4][j] = w[t+j][channel 4p+b4][j] (dx is the transposed shift).
  // Low-rank: one MFMA chain whose K block j multiplies z of token t+j by the
  // rows of tap j (the lane's A fragment is zeroed unless its row's tap is j),
  // so accumulator element 4*b4 + j is exactly that diagonal value.
  auto filter_diag = [&](int b, int p, float (&wd)[4][KP]) {
    if constexpr (LR) {
      f32x16 acc = {};
      const int rtap = tl & 3;  // tap of the MFMA row this lane feeds
#pragma unroll
      for (int j = 0; j <= KH; ++j) {
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
          const bf16x8 a = rtap == j ? af[p][kq] : zero_bf16x8();
          acc = mfma32(a, as_bf16x8(*reinterpret_cast<const uint4 *>(&zs[b][(tl + j) * ZWP + kq * 16 + hh * 8])),
                       acc);
        }
        // let ALU and MFMA work move across, but keep each block's LDS reads
        // next to their MFMAs (hoisting them all costs registers)
        __builtin_amdgcn_sched_barrier(0x000E);
      }
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
        for (int r = 0; r < 4; ++r) wd[b4][r] = acc[4 * b4 + r];
    } else {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int i = 4 * p + b4;
        const int slot = sa + ((nxt >> i) & 1);
        const float4 b0 = *reinterpret_cast<const float4 *>(&w0s[(cl + i) * KP]);
        const float bj[4] = {b0.x, b0.y, b0.z, b0.w};
#pragma unroll
        for (int j = 0; j < KP; ++j)
          wd[b4][j] = j <= KH ? us[b][(tl + j) * UWP + slot * KP + j] + bj[j] : 0.f;
      }
    }
  };

  if (tile_hi > tile_lo) prefetch(tile_lo);
  int buf = 0;
  for (int tile = tile_lo; tile < tile_hi; ++tile, buf ^= 1) {
    const int64_t t0 = (int64_t)tile * 32;
    const int64_t t = t0 + tl;
    const bool tv = t < s.BT;
    const int pos = (int)((uint32_t)t % (uint32_t)s.T);  // B*T < 2^31
    // only waves that touch a sequence start / end need the masks
    const bool edge_lo = __any(KH > 0 && pos < KH);
    const bool edge_hi = __any(KH > 0 && pos + KH > s.T - 1);

    stage(buf);
    __syncthreads();
    if (tile + 1 < tile_hi) prefetch(tile + 1);

    f32x16 dzacc = {};
    if (glive) {
      float dxv[8];
      unsigned char *gtw = gt[wave];

#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // this quad's 4 channels: x history rows (masked before the sequence start),
        // dy of this token
        uint2 xr[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          xr[j] = *reinterpret_cast<const uint2 *>(xs[buf] + (tl + KH - j) * kRowB + (cl + 4 * p) * 2);
          if (edge_lo && j > pos) xr[j] = make_uint2(0, 0);
        }
        const uint2 dy2 = *reinterpret_cast<const uint2 *>(dys[buf] + tl * kRowB + (cl + 4 * p) * 2);
        const float dyq[4] = {__uint_as_float(dy2.x << 16), __uint_as_float(dy2.x & 0xffff0000u),
                              __uint_as_float(dy2.y << 16), __uint_as_float(dy2.y & 0xffff0000u)};
        float wd[4][KP];
        filter_diag(buf, p, wd);
        float G[4][KP];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const uint32_t dword = b4 < 2 ? dy2.x : dy2.y;
          // dy as a bf16 pair with the other half cleared: G = x * dy by a bf16 dot product
          const uint32_t dw = (b4 & 1) ? (dword & 0xffff0000u) : (dword & 0x0000ffffu);
#pragma unroll
          for (int j = 0; j < KP; ++j) {
            if (j < K) {
              const uint32_t xw = b4 < 2 ? xr[j].x : xr[j].y;
              G[b4][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw),
                                                         __builtin_bit_cast(bf16x2_t, dw), 0.f, false);
            } else {
              G[b4][j] = 0.f;
            }
          }
          dxv[4 * p + b4] = fmaf(wd[b4][0], dyq[b4], dyq[b4]);
        }
        // dx: tap j of the filter at token t+j times dy there (the transposed shift)
#pragma unroll
        for (int j = 1; j <= KH; ++j) {
          uint2 dyj2 = *reinterpret_cast<const uint2 *>(dys[buf] + (tl + j) * kRowB + (cl + 4 * p) * 2);
          if (edge_hi && pos + j > s.T - 1) dyj2 = make_uint2(0, 0);  // next sequence
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const uint32_t word = b4 < 2 ? dyj2.x : dyj2.y;
            const float dyj = __uint_as_float((b4 & 1) ? (word & 0xffff0000u) : (word << 16));
            dxv[4 * p + b4] = fmaf(wd[b4][j], dyj, dxv[4 * p + b4]);
          }
        }

        // dz / du: G of this quad is the B operand of steps 2p, 2p+1
#pragma unroll
        for (int sq = 0; sq < 2; ++sq) {
          const int st = 2 * p + sq;
          float bv[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) bv[e8] = G[2 * sq + e8 / KP][e8 % KP];
          bf16x8 a;
          if constexpr (LR) {
            // dz-MFMA A fragment (U in fragment order; small, cache-resident)
            a = as_bf16x8(*reinterpret_cast<const uint4 *>(
                P.Udz + ((((cblk >> 4) + wave) * KP + st) * 32 + tl) * 16 + hh * 8));
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
  if (s.kind == DYNCONV_HEADWISE) return bwd_headwise_layout(s);
  BwdLayout L;
  L.KP = s.k <= 4 ? 4 : 8;
  L.Dt = bwd::kDt;
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
  if (s.kind == DYNCONV_HEADWISE) return bwd_headwise_supported(s);
  if (s.D % 16 != 0 || s.k > 4) return false;
  return s.rank <= 32 && fwd_lowrank_supported(s);
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
  if (s.kind == DYNCONV_HEADWISE) return bwd_headwise(s, L, gen, w0, x, dy, dx, gpart, dw0p, st);
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
    rc = DYNCONV_E_LIMIT;  // head-wise goes to bwd_headwise
  }
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
