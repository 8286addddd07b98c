// conv_fwd_lowrank.hip -- fused forward of the low-rank dynamic short convolution.
//
//   w[t, c, j] = sum_q z[t, q] U[q, c*k+j] + w0[c, j]       (z = h A, from the projection kernel)
//   y[t, c]    = x[t, c] + sum_{j<k, j<=pos(t)} w[t, c, j] x[t-j, c]
//
// The pages' Fused Low-Rank Kernel (gist.science Technical Summary of
// "Dynamic Short Convolutions Improve Transformers", Efficient Training
// Implementation) reads z and U, forms zU on chip and convolves at once,
// never writing the filter to HBM.  This kernel does the same on gfx950: the
// product zU (plus the bias) is one v_mfma_f32_32x32x16_bf16 chain per 32
// tokens x 16 channels, and its fp32 result feeds the conv from registers.
//
// Fragment mapping.  MFMA rows are (channel, tap) pairs, columns are the 32
// tokens of a tile, K is the rank.  Lane l owns token l%32 and the 8
// channels 8*(l/32)..+7 of a 16-channel group; two MFMAs ("quads" p = 0, 1)
// give it taps 0..3 of channels 8*(l/32)+4p+b (b = 0..3) in accumulator
// elements 4b+r.  For k > 4 two more MFMAs give taps 4..7.  The bias w0
// enters the same MFMA chain as one extra K row: the B operand (z) carries a
// constant 1 at q = r and the A operand carries w0 there, so the filter
// leaves the matrix core complete.  The A operand (U, w0 rearranged into
// fragment order, bf16) is written once per call into the workspace by a
// prep kernel and held in VGPRs while a block walks its tokens.
//
// x rows t-k+1 .. t are read from an LDS tile (16-byte reads, rows padded
// to spread banks) that the block fills with coalesced 16-byte loads; y is
// written as 16-byte stores.  HBM roofline: per token 2*D*2 bytes of x and y
// plus 4*r bytes of z.
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace lowrank {

// ---------------------------------------------------------------------------
// prep: A-operand fragments.  For 16-channel group g, quad p, tap half th,
// MFMA row m, K index q (0 .. KQ*16-1):
//   channel c = 16g + 8*((m/4)%2) + 4p + m/8,  tap j = 4*th + m%4
//   value   = U[q, c*k+j] for q < r,  w0[c, j] for q == r,  0 otherwise (and 0 if j >= k)
// stored as Uf[((g*2 + p)*THP + th)*32 + m][q], bf16, q contiguous.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_prep_frag(Shape s, const bf16 *__restrict__ U, const bf16 *__restrict__ w0, bf16 *__restrict__ Uf,
            int THP, int KQ) {
  const int QP = KQ * 16;
  const int64_t total = (s.D / 16) * 2 * THP * 32 * (int64_t)QP;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int q = (int)(idx % QP);
  int64_t rest = idx / QP;
  const int m = (int)(rest % 32);
  rest /= 32;
  const int th = (int)(rest % THP);
  rest /= THP;
  const int p = (int)(rest % 2);
  const int64_t g = rest / 2;
  const int64_t c = 16 * g + 8 * ((m / 4) % 2) + 4 * p + m / 8;
  const int j = 4 * th + m % 4;
  float v = 0.f;
  if (j < s.k) {
    if (q < s.rank)
      v = (float)U[(int64_t)q * s.D * s.k + c * s.k + j];
    else if (q == s.rank && w0)
      v = (float)w0[c * s.k + j];
  }
  Uf[idx] = (bf16)v;
}

constexpr int kCPW = 2;               // 16-channel groups per wave
constexpr int kDt = 4 * kCPW * 16;    // channels per block (4 waves)
constexpr int kTilesPerBlock = 4;     // 32-token tiles a block walks
constexpr int kRowPad = 16;           // LDS row padding (bytes)

template <int KP, int KQ>
__global__ void __launch_bounds__(256)
k_fwd_lowrank(Shape s, const float *__restrict__ z, const bf16 *__restrict__ Uf,
              const bf16 *__restrict__ x, bf16 *__restrict__ y) {
  constexpr int THP = KP / 4;
  constexpr int KH = KP - 1;                         // halo rows
  constexpr int ROWB = kDt * 2 + kRowPad;            // LDS row stride (bytes)
  __shared__ __attribute__((aligned(16))) unsigned char xs[(32 + KH) * ROWB];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int64_t cblk = (int64_t)blockIdx.x * kDt;    // first channel of the block
  const int nch = (int)min<int64_t>(kDt, s.D - cblk);  // channels present (multiple of 16)

  // A fragments for this wave's groups: [cg][p][th][kq]
  bf16x8 af[kCPW][2][THP][KQ];
#pragma unroll
  for (int cg = 0; cg < kCPW; ++cg) {
    const int64_t g = (cblk >> 4) + wave * kCPW + cg;
    const bool live = (wave * kCPW + cg) * 16 < nch;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int th = 0; th < THP; ++th)
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
          const int64_t rowf = ((g * 2 + p) * THP + th) * 32 + tl;
          af[cg][p][th][kq] = live ? as_bf16x8(*reinterpret_cast<const uint4 *>(
                                         Uf + rowf * (KQ * 16) + kq * 16 + hh * 8))
                                   : zero_bf16x8();
        }
  }

  const int64_t tile0 = (int64_t)blockIdx.y * kTilesPerBlock;
  for (int it = 0; it < kTilesPerBlock; ++it) {
    const int64_t t0 = (tile0 + it) * 32;
    if (t0 >= s.BT) break;

    // ---- stage x rows [t0-KH, t0+32) x [cblk, cblk+nch) in LDS ----
    __syncthreads();
    {
      const int chunks = nch / 8;  // 16-byte chunks per row
      for (int e = threadIdx.x; e < (32 + KH) * chunks; e += 256) {
        const int r = e / chunks, q = e - r * chunks;
        const int64_t row = t0 - KH + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row >= 0 && row < s.BT)
          v = *reinterpret_cast<const uint4 *>(x + row * s.D + cblk + q * 8);
        *reinterpret_cast<uint4 *>(xs + r * ROWB + q * 16) = v;
      }
    }

    // ---- B operand: z for this tile's tokens, plus the constant-1 bias row ----
    const int64_t t = t0 + tl;
    const bool trow = t < s.BT;
    bf16x8 bz[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = kq * 16 + hh * 8 + i;
        v[i] = (trow && q < s.rank) ? z[t * s.rank + q] : (q == s.rank ? 1.f : 0.f);
      }
      bz[kq] = pack_bf16x8(v);
    }
    const int pos = trow ? (int)(t % s.T) : 0;
    __syncthreads();

#pragma unroll
    for (int cg = 0; cg < kCPW; ++cg) {
      const int cl = (wave * kCPW + cg) * 16 + hh * 8;  // first of this lane's 8 channels (block-local)
      if ((wave * kCPW + cg) * 16 >= nch) break;
      // x[t-j][8 channels] for j = 0..KP-1
      float xv[KP][8];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(xs + (tl + KH - j) * ROWB + cl * 2);
        const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[j][2 * i] = __uint_as_float(wds[i] << 16);
          xv[j][2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
        }
      }
      float out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = xv[0][i];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int th = 0; th < THP; ++th) {
          f32x16 acc = {};
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) acc = mfma32(af[cg][p][th][kq], bz[kq], acc);
          // acc[4b + r] = w[t][channel 4p+b of this half][tap 4th + r]
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 4 * th + r;
              if (j < KP && j <= pos && j < s.k) out[4 * p + b] = fmaf(acc[4 * b + r], xv[j][4 * p + b], out[4 * p + b]);
            }
        }
      if (trow) store_vec(y + t * s.D + cblk + cl, out);
    }
  }
}

}  // namespace lowrank

size_t fwd_lowrank_ws_bytes(const Shape &s) {
  const int THP = s.k <= 4 ? 1 : 2;
  const int KQ = (int)ceil_div(s.rank + 1, 16);
  return (size_t)(s.D / 16) * 2 * THP * 32 * KQ * 16 * sizeof(bf16);
}

bool fwd_lowrank_supported(const Shape &s) { return s.D % 16 == 0 && s.rank + 1 <= 64; }

int prep_lowrank_frags(const Shape &s, const void *U, const void *w0, void *Uf, hipStream_t st) {
  const int THP = s.k <= 4 ? 1 : 2;
  const int KQ = (int)ceil_div(s.rank + 1, 16);
  const int64_t total = (s.D / 16) * 2 * THP * 32 * (int64_t)KQ * 16;
  hipLaunchKernelGGL(lowrank::k_prep_frag, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, st, s,
                     (const bf16 *)U, (const bf16 *)w0, (bf16 *)Uf, THP, KQ);
  return 0;
}

int fwd_lowrank(const Shape &s, const float *z, const void *Uf, const void *x, void *y, hipStream_t st) {
  using namespace lowrank;
  const int KQ = (int)ceil_div(s.rank + 1, 16);
  dim3 grid((unsigned)ceil_div(s.D, kDt), (unsigned)ceil_div(ceil_div(s.BT, 32), kTilesPerBlock));
  const bool tr = trace_begin(DYNCONV_K_FWD_CONV, st);
#define LAUNCH(KP_, KQ_)                                                                          \
  hipLaunchKernelGGL((k_fwd_lowrank<KP_, KQ_>), grid, dim3(256), 0, st, s, z, (const bf16 *)Uf, \
                     (const bf16 *)x, (bf16 *)y)
  if (s.k <= 4) {
    switch (KQ) {
      case 1: LAUNCH(4, 1); break;
      case 2: LAUNCH(4, 2); break;
      case 3: LAUNCH(4, 3); break;
      case 4: LAUNCH(4, 4); break;
      default: trace_end(tr, st); return DYNCONV_E_LIMIT;
    }
  } else {
    switch (KQ) {
      case 1: LAUNCH(8, 1); break;
      case 2: LAUNCH(8, 2); break;
      case 3: LAUNCH(8, 3); break;
      case 4: LAUNCH(8, 4); break;
      default: trace_end(tr, st); return DYNCONV_E_LIMIT;
    }
  }
#undef LAUNCH
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
