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
// elements 4b+r; filters of 5..8 taps take a second pair of MFMAs per group
// for taps 4..7 ("tap halves").  The bias w0
// enters the same MFMA chain as one extra K row: the B operand (z) carries a
// constant 1 at q = r and the A operand carries w0 there, so the filter
// leaves the matrix core complete.  Each lane gathers its A-operand values
// (U and w0 in fragment order, bf16) from global memory when the block
// starts and holds them in VGPRs while the block walks its tokens.
//
// x rows t-k+1 .. t are read from an LDS tile (16-byte reads, rows padded
// to spread banks) that the block fills with coalesced 16-byte loads.  y goes
// through an LDS tile too (double-buffered): the lanes, which own tokens,
// write it there, and after the next tile's barrier the block stores it
// row-contiguous, four rows of 256 bytes per wave instruction (a store
// straight from the token-owning lanes would cover 32 rows x 32 bytes).  HBM roofline: per token 2*D*2 bytes of x and y
// plus 4*r bytes of z.
#include "kernels.h"
#include "bufio.h"
#include "mfma.h"

namespace dynconv {
namespace lowrank {

constexpr int kCPW = 2;               // 16-channel groups per wave
constexpr int kDt = 4 * kCPW * 16;    // channels per block (4 waves)
constexpr int kRowB = kDt * 2 + 16;   // LDS row stride of the x tile (bytes, padded)

// Loads and stores are raw buffer accesses issued on every path (a masked
// slot gets an offset outside the buffer: zeros in, nothing out), so the
// compiler's wait counts stay exact: tile i+2 is in flight while tile i is
// computed (two register sets, tiles taken in pairs).
// VAR: packed documents; each lane's token position comes from the per-token
// table, loaded with the tile's other operands two tiles ahead.
template <int K, int KQ, bool VAR>
__global__ void __launch_bounds__(256)
k_fwd_lowrank(Shape s, const float *__restrict__ z, const bf16 *__restrict__ U, const bf16 *__restrict__ w0,
              const bf16 *__restrict__ x, bf16 *__restrict__ y, int tpb, int n_tiles) {
  constexpr int TH = K > 4 ? 2 : 1;     // tap halves (taps 0..3, 4..7)
  constexpr int KH = K - 1;             // history rows
  constexpr int ZW = KQ * 16, ZWP = ZW + 8;
  constexpr int CH = kDt / 8;           // 16-byte chunks per row
  constexpr int kVLoads = ((32 + KH) * CH + 255) / 256;
  constexpr int kXRows = kVLoads * 256 / CH;  // x tile rows incl. spare ones for unused load slots
  constexpr int kSLoads = (32 * ZW + 255) / 256;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][kXRows * kRowB];
  __shared__ __attribute__((aligned(16))) bf16 zs[2][32 * ZWP + 8];  // + a spare slot for unused z loads
  __shared__ __attribute__((aligned(16))) unsigned char ys[2][32 * kRowB];  // y of a tile, same row layout as x

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, tl = lane & 31;
  const int cblk = blockIdx.x * kDt;
  const int D = (int)s.D, BT = (int)s.BT, rank = s.rank;  // BT*D and BT*rank*2 < 2^30 (host-checked)
  const int nch = min(kDt, D - cblk);
  const int tile_lo = blockIdx.y * tpb, tile_hi = min(n_tiles, tile_lo + tpb);

  // bias / padding columns of the z tile (constant): 1 at q = r, 0 beyond
  for (int e = tid; e < 2 * (32 * ZWP + 8); e += 256) {
    const int q = (e % (32 * ZWP + 8)) % ZWP;
    if (q >= rank) (&zs[0][0])[e] = (bf16)(q == rank ? 1.f : 0.f);
  }

  // A fragments for this wave's groups [g][p][th][kq], gathered by each lane
  // from U and w0: row m = tl is (channel 16gg + 8((m/4)%2) + 4p + m/8, tap
  // 4th + m%4), K index q = 16kq + 8hh + i is U's row for q < r, the bias w0
  // for q = r, zero beyond (and for taps >= k)
  bf16x8 af[kCPW][2][TH][KQ];
  bool glive[kCPW];
  {
    const auto ru = make_rsrc(U, (uint32_t)((int64_t)rank * D * K * 2));
    const auto rw = make_rsrc(w0, w0 ? (uint32_t)(D * K * 2) : 0u);  // no bias: every load reads 0
    const int kqb = rank / 16, ib = rank % 8, hb = (rank / 8) % 2;  // where q = rank sits
#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      const int gl = wave * kCPW + g;
      glive[g] = gl * 16 < nch;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = cblk + 16 * gl + 8 * ((tl / 4) % 2) + 4 * p + tl / 8;
#pragma unroll
        for (int th = 0; th < TH; ++th) {
          const int j = 4 * th + tl % 4;
          const bool ok = glive[g] && j < K;
          const float bias = bf16_bits_to_float(
              __builtin_amdgcn_raw_buffer_load_b16(rw, ok && hh == hb ? (uint32_t)((c * K + j) * 2) : kOutside, 0, 0));
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int q = 16 * kq + 8 * hh + i;
              const uint32_t off = ok && q < rank ? (uint32_t)((q * D * K + c * K + j) * 2) : kOutside;
              v[i] = bf16_bits_to_float(__builtin_amdgcn_raw_buffer_load_b16(ru, off, 0, 0)) +
                     (kq == kqb && i == ib ? bias : 0.f);
            }
            af[g][p][th][kq] = pack_bf16x8(v);
          }
        }
      }
    }
  }

  // per-thread load slots (fixed for the block): byte offset at tile 0 and
  // LDS destination.  Per tile the offset advances by the tile's rows; the
  // buffer's range check returns zeros for rows past BT and masked slots
  // (kOutside + advance), and rows before 0 (tile 0's history rows) wrap to
  // the top of the 32-bit range, clamped below 2^32 - 256 so that offset +
  // access size never wraps.  Tiles past the block's range (the second of a
  // pair, the loads two ahead) load whatever their offsets reach: their
  // results are never stored.
  uint32_t v_gbase[kVLoads];
  int v_loff[kVLoads];
#pragma unroll
  for (int q = 0; q < kVLoads; ++q) {
    const int e = tid + q * 256;
    const int r = e / CH, c16 = e % CH;
    const bool ok = r < 32 + KH && c16 * 8 < nch;
    v_gbase[q] = ok ? (uint32_t)((r - KH) * D + cblk + c16 * 8) * 2u : kOutside;
    v_loff[q] = r * kRowB + c16 * 16;
  }
  // y store slots (from the LDS tile): chunk e = tid + 256 q is row e / CH,
  // 16-byte chunk e % CH; offset at tile 0, kOutside past the slice's channels
  constexpr int kYS = 32 * CH / 256;  // stores per thread and tile
  uint32_t y_base[kYS];
  int y_loff[kYS];
#pragma unroll
  for (int q = 0; q < kYS; ++q) {
    const int e = tid + q * 256;
    const int r = e / CH, c16 = e % CH;
    y_base[q] = c16 * 8 < nch ? (uint32_t)(r * D + cblk + c16 * 8) * 2u : kOutside;
    y_loff[q] = r * kRowB + c16 * 16;
  }
  uint32_t s_gbase[kSLoads];
  int s_loff[kSLoads];
#pragma unroll
  for (int q = 0; q < kSLoads; ++q) {
    const int e = tid + q * 256;
    const int tt = e / ZW, sq = e % ZW;
    const bool ok = tt < 32 && sq < rank;
    s_gbase[q] = ok ? (uint32_t)(tt * rank + sq) * 4u : kOutside;
    s_loff[q] = ok ? tt * ZWP + sq : 32 * ZWP;  // unused slots write the spare element
  }
  const auto rx = make_rsrc(x, (uint32_t)(BT * D * 2));
  const auto rz = make_rsrc(z, (uint32_t)(BT * rank * 4));
  const auto ry = make_rsrc(y, (uint32_t)(BT * D * 2));
  uint4 vpre[2][kVLoads];
  float spre[2][kSLoads];
  uint32_t ppre[2] = {0u, 0u};  // VAR: table entry of the lane's token (zero past BT)
  const auto rp = make_rsrc(s.seqpos, VAR ? (uint32_t)(BT * 2) : 0u);
  auto prefetch = [&](int set, int tile) {
    const bool tin = tile < tile_hi;
    const uint32_t vstep = tin ? (uint32_t)(tile * 32 * D) * 2u : kOutside;
    const uint32_t zstep = tin ? (uint32_t)(tile * 32 * rank) * 4u : kOutside;
    constexpr uint32_t kTop = 0xffffff00u;
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) vpre[set][q] = buf_load16(rx, min(v_gbase[q] + vstep, kTop));
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) spre[set][q] = buf_load_f32(rz, min(s_gbase[q] + zstep, kTop));
    if constexpr (VAR)
      ppre[set] = __builtin_amdgcn_raw_buffer_load_b16(rp, tin ? (uint32_t)(tile * 32 + tl) * 2u : kOutside, 0, 0);
  };

  // y of a tile from its LDS tile (rows past BT fall outside ry; tiles past
  // the block's range store nothing)
  auto store_y = [&](const int set, const int tile) {
    const bool tin = tile >= tile_lo && tile < tile_hi;
    const uint32_t ystep = (uint32_t)(tile * 32 * D) * 2u;
#pragma unroll
    for (int q = 0; q < kYS; ++q)
      buf_store16(ry, tin ? y_base[q] + ystep : kOutside, *reinterpret_cast<const uint4 *>(ys[set] + y_loff[q]));
  };

  auto step = [&](const int set, const int tile) {
    // ---- stage this tile, then start loading the one two ahead ----
#pragma unroll
    for (int q = 0; q < kVLoads; ++q) *reinterpret_cast<uint4 *>(xs[set] + v_loff[q]) = vpre[set][q];
#pragma unroll
    for (int q = 0; q < kSLoads; ++q) zs[set][s_loff[q]] = (bf16)spre[set][q];
    const int t = tile * 32 + tl;
    // (read before the prefetch below refills the set)
    const int pos = VAR ? (int)(ppre[set] & 255u) : (int)((uint32_t)t % (uint32_t)s.T);
    __syncthreads();
    // the previous tile's y is complete in the other LDS tile (its writes
    // precede this barrier); this tile's y tile was last read before it
    store_y(set ^ 1, tile - 1);
    prefetch(set, tile + 2);
    bf16x8 bz[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      bz[kq] = as_bf16x8(*reinterpret_cast<const uint4 *>(&zs[set][tl * ZWP + kq * 16 + hh * 8]));

#pragma unroll
    for (int g = 0; g < kCPW; ++g) {
      const int cl = (wave * kCPW + g) * 16 + hh * 8;  // block-local first channel of the lane's 8
      float xv[K][8];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        uint4 raw = *reinterpret_cast<const uint4 *>(xs[set] + (tl + KH - j) * kRowB + cl * 2);
        if (j > pos) raw = make_uint4(0, 0, 0, 0);  // x[t-j] belongs to the previous sequence
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
        for (int th = 0; th < TH; ++th) {
          f32x16 acc = {};
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) acc = mfma32(af[g][p][th][kq], bz[kq], acc);
          // acc[4b + r] = w[t][channel 4p+b of this half][tap 4th + r]
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 4 * th + r;
              if (j < K) out[4 * p + b4] = fmaf(acc[4 * b4 + r], xv[j][4 * p + b4], out[4 * p + b4]);
            }
        }
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)out[2 * i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)out[2 * i + 1]) << 16);
      *reinterpret_cast<uint4 *>(ys[set] + tl * kRowB + cl * 2) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  prefetch(0, tile_lo);
  prefetch(1, tile_lo + 1);
  int tile = tile_lo;
  for (; tile < tile_hi; tile += 2) {
    step(0, tile);
    step(1, tile + 1);
  }
  // the last pair's second tile (set 1) is still in LDS
  __syncthreads();
  store_y(1, tile - 1);
}

}  // namespace lowrank

bool fwd_lowrank_supported(const Shape &s) {
  // 32-bit element and byte offsets into x, y and z
  const int64_t lim = ((int64_t)1 << 31) - 64;
  return s.D % 8 == 0 && s.rank <= 64 && s.k <= 8 && s.BT * s.D * 2 < lim && s.BT * s.rank * 4 < lim &&
         (int64_t)s.rank * s.D * s.k * 2 < lim;
}

int fwd_lowrank(const Shape &s, const float *z, const void *U, const void *w0, const void *x, void *y,
                hipStream_t st) {
  using namespace lowrank;
  const int KQ = (int)ceil_div(s.rank + 1, 16);
  const int n_slices = (int)ceil_div(s.D, kDt);
  const int n_tiles = (int)ceil_div(s.BT, 32);
  // about two blocks per CU, each walking an even run of tiles
  int tpb = 2;
  while ((int64_t)n_slices * ceil_div(n_tiles, tpb) > 512) tpb += 2;
  dim3 grid((unsigned)n_slices, (unsigned)ceil_div(n_tiles, tpb));
  const bool tr = trace_begin(DYNCONV_K_FWD_CONV, st);
  int rc = 0;
#define LAUNCH(K_, KQ_)                                                                                \
  do {                                                                                                 \
    if (s.seqpos)                                                                                      \
      hipLaunchKernelGGL((k_fwd_lowrank<K_, KQ_, true>), grid, dim3(256), 0, st, s, z, (const bf16 *)U,  \
                         (const bf16 *)w0, (const bf16 *)x, (bf16 *)y, tpb, n_tiles);                 \
    else                                                                                               \
      hipLaunchKernelGGL((k_fwd_lowrank<K_, KQ_, false>), grid, dim3(256), 0, st, s, z, (const bf16 *)U, \
                         (const bf16 *)w0, (const bf16 *)x, (bf16 *)y, tpb, n_tiles);                 \
  } while (0)
#define LAUNCH_K(K_)                          \
  switch (KQ) {                               \
    case 1: LAUNCH(K_, 1); break;             \
    case 2: LAUNCH(K_, 2); break;             \
    case 3: LAUNCH(K_, 3); break;             \
    case 4: LAUNCH(K_, 4); break;             \
    case 5: LAUNCH(K_, 5); break;             \
    default: rc = DYNCONV_E_LIMIT;            \
  }
  switch (s.k) {
    case 1: LAUNCH_K(1) break;
    case 2: LAUNCH_K(2) break;
    case 3: LAUNCH_K(3) break;
    case 4: LAUNCH_K(4) break;
    case 5: LAUNCH_K(5) break;
    case 6: LAUNCH_K(6) break;
    case 7: LAUNCH_K(7) break;
    default: LAUNCH_K(8) break;
  }
#undef LAUNCH_K
#undef LAUNCH
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
