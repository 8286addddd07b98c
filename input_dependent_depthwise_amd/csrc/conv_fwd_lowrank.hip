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
// leaves the matrix core complete.  Each lane gathers its A-operand values
// (U and w0 in fragment order, bf16) from global memory when the block
// starts and holds them in VGPRs while the block walks its tokens.
//
// x rows t-k+1 .. t are read from an LDS tile (16-byte reads, rows padded
// to spread banks) that the block fills with coalesced 16-byte loads; y is
// written as 16-byte stores.  HBM roofline: per token 2*D*2 bytes of x and y
// plus 4*r bytes of z.
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace lowrank {

constexpr int kCPW = 2;               // 16-channel groups per wave
constexpr int kDt = 4 * kCPW * 16;    // channels per block (4 waves)
constexpr int kRowB = kDt * 2 + 16;   // LDS row stride of the x tile (bytes, padded)

template <int K, int KQ>
__global__ void __launch_bounds__(256)
k_fwd_lowrank(Shape s, const float *__restrict__ z, const bf16 *__restrict__ U, const bf16 *__restrict__ w0,
              const bf16 *__restrict__ x, bf16 *__restrict__ y, int tpb, int n_tiles) {
  constexpr int KP = 4;
  constexpr int KH = K - 1;             // history rows
  constexpr int ZW = KQ * 16, ZWP = ZW + 8;
  constexpr int CH = kDt / 8;           // 16-byte chunks per row
  constexpr int kVLoads = ((32 + KH) * CH + 255) / 256;
  constexpr int kSLoads = (32 * ZW + 255) / 256;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][(32 + KH) * kRowB];
  __shared__ __attribute__((aligned(16))) bf16 zs[2][32 * ZWP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int64_t cblk = (int64_t)blockIdx.x * kDt;
  const int nch = (int)min<int64_t>(kDt, s.D - cblk);
  const int tile_lo = blockIdx.y * tpb, tile_hi = min(n_tiles, tile_lo + tpb);

  // bias / padding columns of the z tile (constant): 1 at q = r, 0 beyond
  for (int e = threadIdx.x; e < 2 * 32 * ZWP; e += 256) {
    const int q = e % ZWP;
    if (q >= s.rank) (&zs[0][0])[e] = (bf16)(q == s.rank ? 1.f : 0.f);
  }

  // A fragments for this wave's groups [g][p][kq], gathered by each lane from
  // U and w0: row m = tl is (channel 16gg + 8((m/4)%2) + 4p + m/8, tap m%4),
  // K index q = 16kq + 8hh + i is U's row for q < r, the bias w0 for q = r,
  // zero beyond (and for taps >= k)
  bf16x8 af[kCPW][2][KQ];
  bool glive[kCPW];
#pragma unroll
  for (int g = 0; g < kCPW; ++g) {
    const int64_t gg = (cblk >> 4) + wave * kCPW + g;
    glive[g] = (wave * kCPW + g) * 16 < nch;
    const int j = tl % 4;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t c = 16 * gg + 8 * ((tl / 4) % 2) + 4 * p + tl / 8;
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int q = 16 * kq + 8 * hh + i;
          float u = 0.f;
          if (glive[g] && j < K) {
            if (q < s.rank) u = (float)U[(int64_t)q * s.D * K + c * K + j];
            else if (q == s.rank && w0) u = (float)w0[c * K + j];
          }
          v[i] = u;
        }
        af[g][p][kq] = pack_bf16x8(v);
      }
    }
  }

  // per-thread load slots
  int v_row[kVLoads], v_col[kVLoads], v_loff[kVLoads];
  bool v_ok[kVLoads];
#pragma unroll
  for (int q = 0; q < kVLoads; ++q) {
    const int e = threadIdx.x + q * 256;
    const int r = e / CH, c16 = e % CH;
    v_ok[q] = r < 32 + KH && c16 * 8 < nch;
    v_row[q] = r - KH;
    v_col[q] = c16 * 8;
    v_loff[q] = r * kRowB + c16 * 16;
  }
  int s_tt[kSLoads], s_q[kSLoads];
  bool s_ok[kSLoads];
#pragma unroll
  for (int q = 0; q < kSLoads; ++q) {
    const int e = threadIdx.x + q * 256;
    s_tt[q] = e / ZW;
    s_q[q] = e % ZW;
    s_ok[q] = s_tt[q] < 32 && s_q[q] < s.rank;
  }
  uint4 vpre[kVLoads];
  float spre[kSLoads];
  auto prefetch = [&](int tile) {
    const int64_t t0 = (int64_t)tile * 32;
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) {
      const int64_t row = t0 + v_row[q];
      vpre[q] = make_uint4(0, 0, 0, 0);
      if (v_ok[q] && row >= 0 && row < s.BT)
        vpre[q] = *reinterpret_cast<const uint4 *>(x + row * s.D + cblk + v_col[q]);
    }
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) {
      const int64_t row = t0 + s_tt[q];
      spre[q] = (s_ok[q] && row < s.BT) ? z[row * s.rank + s_q[q]] : 0.f;
    }
  };

  if (tile_hi > tile_lo) prefetch(tile_lo);
  int buf = 0;
  for (int tile = tile_lo; tile < tile_hi; ++tile, buf ^= 1) {
    // ---- stage this tile, then start loading the next ----
#pragma unroll
    for (int q = 0; q < kVLoads; ++q)
      if (v_ok[q]) *reinterpret_cast<uint4 *>(xs[buf] + v_loff[q]) = vpre[q];
#pragma unroll
    for (int q = 0; q < kSLoads; ++q)
      if (s_ok[q]) zs[buf][s_tt[q] * ZWP + s_q[q]] = (bf16)spre[q];
    __syncthreads();
    if (tile + 1 < tile_hi) prefetch(tile + 1);

    const int64_t t = (int64_t)tile * 32 + tl;
    const bool tv = t < s.BT;
    const int pos = (int)((uint32_t)t % (uint32_t)s.T);
    const bool edge = __any(KH > 0 && pos < KH);
    bf16x8 bz[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      bz[kq] = as_bf16x8(*reinterpret_cast<const uint4 *>(&zs[buf][tl * ZWP + kq * 16 + hh * 8]));

#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      if (!glive[g]) continue;
      const int cl = (wave * kCPW + g) * 16 + hh * 8;  // block-local first channel of the lane's 8
      float xv[K][8];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        uint4 raw = *reinterpret_cast<const uint4 *>(xs[buf] + (tl + KH - j) * kRowB + cl * 2);
        if (edge && j > pos) raw = make_uint4(0, 0, 0, 0);
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
      for (int p = 0; p < 2; ++p) {
        f32x16 acc = {};
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) acc = mfma32(af[g][p][kq], bz[kq], acc);
        // acc[4b + r] = w[t][channel 4p+b of this half][tap r]
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
          for (int j = 0; j < K; ++j) out[4 * p + b4] = fmaf(acc[4 * b4 + j], xv[j][4 * p + b4], out[4 * p + b4]);
      }
      if (tv) store_vec(y + t * s.D + cblk + cl, out);
    }
  }
  (void)KP;
}

}  // namespace lowrank

bool fwd_lowrank_supported(const Shape &s) { return s.D % 16 == 0 && s.rank + 1 <= 64 && s.k <= 4; }

int fwd_lowrank(const Shape &s, const float *z, const void *U, const void *w0, const void *x, void *y,
                hipStream_t st) {
  using namespace lowrank;
  const int KQ = (int)ceil_div(s.rank + 1, 16);
  const int n_slices = (int)ceil_div(s.D, kDt);
  const int n_tiles = (int)ceil_div(s.BT, 32);
  // enough blocks for ~4 per CU, each walking a run of tiles
  int tpb = 1;
  while ((int64_t)n_slices * ceil_div(n_tiles, tpb) > 1024) ++tpb;
  dim3 grid((unsigned)n_slices, (unsigned)ceil_div(n_tiles, tpb));
  const bool tr = trace_begin(DYNCONV_K_FWD_CONV, st);
  int rc = 0;
#define LAUNCH(K_, KQ_)                                                                             \
  hipLaunchKernelGGL((k_fwd_lowrank<K_, KQ_>), grid, dim3(256), 0, st, s, z, (const bf16 *)U,     \
                     (const bf16 *)w0, (const bf16 *)x, (bf16 *)y, tpb, n_tiles)
#define LAUNCH_K(K_)                          \
  switch (KQ) {                               \
    case 1: LAUNCH(K_, 1); break;             \
    case 2: LAUNCH(K_, 2); break;             \
    case 3: LAUNCH(K_, 3); break;             \
    case 4: LAUNCH(K_, 4); break;             \
    default: rc = DYNCONV_E_LIMIT;            \
  }
  switch (s.k) {
    case 1: LAUNCH_K(1) break;
    case 2: LAUNCH_K(2) break;
    case 3: LAUNCH_K(3) break;
    default: LAUNCH_K(4) break;
  }
#undef LAUNCH_K
#undef LAUNCH
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
