// conv_bwd_lowrank.hip -- fused backward of the low-rank dynamic short
// convolution (bf16 I/O) on matrix cores.
//
// Layer (gist.science Technical Summary of "Dynamic Short Convolutions Improve
// Transformers", Methodology -> Dynamic Short Convolutions: Mechanism,
// Parameterization): y[t,c] = x[t,c] + sum_j w[t,c,j] x[t-j,c] with the
// low-rank filter w[t,c,j] = sum_q z[t,q] U[q,c*k+j] + w0[c,j], z = h A.
// For L = sum(dy * y), one pass over x and dy gives
//   dx[s,c]   = dy[s,c] + sum_j [s, s+j in one sequence] w[s+j,c,j] dy[s+j,c]
//   G[t,c,j]  = [t-j in t's sequence] dy[t,c] x[t-j,c]         (never stored)
//   dz[t,q]   = sum_{c,j} G[t,c,j] U[q,c*k+j]    -> one fp32 partial per 64/128-channel slice
//   dU[q,c*k+j] = sum_t z[t,q] G[t,c,j]          -> one fp32 partial per token range
//   dw0[c,j]  = sum_t G[t,c,j]                   -> one fp32 partial per token range
//
// Work split.  A block (4 waves for rank <= 16, for ranks 33..64 and for
// 5..8 taps, else 8) owns 64 or 128 channels and a range of 32-token tiles; wave w owns 16 of the channels.  Per tile the block stages x (rows
// t0-k+1 .. t0+31), dy and z (rows t0 .. t0+31+k-1) in LDS.  Every product is
// a v_mfma_f32_16x16x32_bf16; a lane (n = lane%16, g = lane/16) holds tokens
// n and 16+n of the tile and channels 4g .. 4g+3 of the wave's 16:
//   * filter, per tap j and 16-token block: D[channel][token] = U^T z with the
//     z rows shifted by j, so the lane of token s gets w[s+j, c, j] directly
//     (the diagonal the transposed conv needs); the bias w0 rides as an extra
//     K row against a constant 1 column of z (K = 32 covers rank <= 31);
//   * dx accumulates w[s+j,c,j] dy[s+j,c] in registers;
//   * G for tap j comes from bf16 dot products (v_dot2) of x[s-j] with dy[s]
//     (one half of each pair cleared); rounded to bf16 once, two taps at a time
//     are the B operand of D[q][token] = U G (dz, summed over taps and
//     channels in the accumulator);
//   * G goes to LDS token-major (8-byte writes) and comes back transposed
//     (ds_read_b64_tr_b16, four tokens of one channel per lane) as the A
//     operand of D[channel][q] = G^T z over the tile's 32 tokens (dU);
//   * dw0 sums the fp32 G products (before their rounding to bf16) per lane
//     in its own LDS slots (no registers held across the walk),
//     then over the lanes at the end.
// The block's waves' dz meet in LDS; the block writes one partial per (slice,
// token).  The global loads of the next tile (or, where registers allow, of
// the one after) are in flight while a tile is computed.  Matrix-core fragments of U are built by each lane from global
// memory at start (no separate preparation pass).
#include "bufio.h"
#include "kernels.h"
#include "mfma.h"

namespace dynconv {
namespace bwdlr {

constexpr int kCW = 16;          // channels per wave
// Waves per block: 4 (64 channels) when rank <= 16, else 8 (128 channels),
// except ranks 33..64 and 5..8 taps (below).
// Two 4-wave blocks share a CU, so one block's barriers overlap the other's
// work; with a larger rank the per-slice dz partials (rank floats per token
// and slice) grow too much for the narrower slices.  Filters of 5..8 taps
// and ranks 33..64 take 4-wave blocks of one wave per SIMD: their U
// fragments and dU accumulators need more registers than two waves per SIMD
// leave.
inline int waves_for(const Shape &s) { return (s.rank <= 16 || s.rank > 32 || s.k > 4) ? 4 : 8; }
constexpr int kGRow = 40;        // LDS row of the token-contiguous z^T tile: 32 tokens + pad (bf16)
// G of one tap in LDS: 32 token rows of 16 channels (32 bytes), 128 bytes of
// pad after every 8 rows and the row's four 8-byte channel quads swapped in
// pairs on rows 8..15 and 24..31, so that both the writes (16 rows x 2 quads
// per 32 lanes) and the transposed reads (4 rows x 4 quads per 16 lanes) use
// 64 distinct banks
constexpr int kGTap = 32 * 32 + 4 * 128;
__device__ __forceinline__ int g_off(int t, int quad) {
  return 32 * t + 128 * (t >> 3) + 8 * (quad ^ (2 * ((t >> 3) & 1)));
}

struct Params {
  Shape s;
  const bf16 *x, *dy;
  bf16 *dx;
  const float *z;   // [BT, r]
  const bf16 *U;    // [r, D*k]
  const bf16 *w0;   // [D, k] or NULL
  float *gpart;     // [n_slices][BT][r]
  float *dUp;       // [n_ranges][r][D*k]
  float *dw0p;      // [n_ranges][D*k]
  int tpb;          // tiles per block
  int n_tiles;      // ceil(BT / 32)
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
// a.lo*b.lo + a.hi*b.hi (written with the builtin: hand-issued VALU code
// would bypass the compiler's hazard tracking)
__device__ __forceinline__ float dot2z(uint32_t a, uint32_t b) { return dot2(a, b, 0.f); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2_t p = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// K: taps; KQ: 32-row K-steps over rank + bias; NQ: 16-row blocks of rank.
// VAR: packed documents (each token's position and the tokens after it in
// its document come from the per-token table, loaded with the tile's other
// operands; every tile takes the masked path).
template <int K, int KQ, int NQ, int kW, bool VAR>
__global__ void __launch_bounds__(kW * 64, K <= 4 && NQ <= 2 ? 2 : 1)
k_bwd_lr(Params P) {
  constexpr int kDt = kW * kCW;    // channels per block
  // LDS row of the x / dy tiles (bf16 elements): 36 or 68 dwords, so that the
  // 8-byte reads of 16 consecutive token rows x 2 channel quads cover all 64
  // banks once
  constexpr int kRow = kDt + 8;
  constexpr int KH = K - 1;
  constexpr int KP = (K + 1) / 2;             // tap pairs
  constexpr int TR = 32 + KH;                 // rows of a staged tile
  constexpr int ZW = 32 * KQ + 8;             // z row in LDS (bf16): rank, bias column, zeros, pad
  constexpr int NT = kW * 64;
  constexpr int CH = kDt / 8;                 // 16-byte chunks per x / dy row
  constexpr int CHX = TR * CH;                 // 16-byte chunks of one staged tensor (x or dy)
  constexpr int CHXP = (CHX + 63) / 64 * 64;  // padded to whole waves: a load slot's tensor is wave-uniform
  constexpr int kVL = (2 * CHXP + NT - 1) / NT;
  constexpr int ZC = 16 * NQ;                 // z columns staged (rank padded)
  constexpr int kZL = (TR * ZC + NT - 1) / NT;
  constexpr int RV = 8 * NQ;                  // dz values per lane and tile
  constexpr int RVP = RV + 4;                 // lane stride of the dz reduction buffer (bank spread)
  constexpr int NSET = KQ * NQ * K <= 4 ? 2 : 1;  // register sets of prefetched tiles (as registers allow)
  const Shape &s = P.s;
  const int rank = s.rank;

  // (each with a spare row or element that unused load slots write to)
  __shared__ __attribute__((aligned(16))) bf16 xs[(TR + 1) * kRow];    // x rows t0-KH .. t0+31
  __shared__ __attribute__((aligned(16))) bf16 dys[(TR + 1) * kRow];   // dy rows t0 .. t0+31+KH
  __shared__ __attribute__((aligned(16))) bf16 zs[TR * ZW + 8];        // z rows t0 .. t0+31+KH, bf16
  __shared__ __attribute__((aligned(16))) bf16 zt[ZC * kGRow + 8];     // z^T: rows q, tokens t0 .. t0+31
  __shared__ __attribute__((aligned(16))) unsigned char gt[kW][2 * kGTap];  // per wave: G of a tap pair
  __shared__ __attribute__((aligned(16))) float red[kW][64 * RVP];     // per wave: dz partial of a tile
  __shared__ float dwl[kW][4 * K * 64];  // per lane: dw0 of its 4 channels x K taps, [tap*4 + r][lane]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t cblk = (int64_t)blockIdx.x * kDt;
  const int64_t cw = cblk + wave * kCW;  // the wave's first channel
  const int64_t Dk = s.D * K;

  // ---- block constants in LDS: z's bias and zero columns, zero z^T rows ----
  for (int e = tid; e < TR * ZW; e += NT) {
    const int q = e % ZW;
    if (q >= rank) zs[e] = (bf16)(q == rank ? 1.f : 0.f);
  }
  for (int e = tid; e < ZC * kGRow; e += NT) zt[e] = (bf16)0.f;

  // ---- matrix-core fragments of U ----
  // filter A (tap j, K-step kq): A[m = channel cw + n][k = q = 32kq + 8g + i]; bias row q = rank
  bf16x8 fa[K][KQ];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 32 * kq + 8 * g + i;
        const int64_t c = cw + n;
        float u = 0.f;
        if (c < s.D) {
          if (q < rank) u = (float)P.U[(int64_t)q * Dk + c * K + j];
          else if (q == rank && P.w0) u = (float)P.w0[c * K + j];
        }
        v[i] = u;
      }
      fa[j][kq] = pack_bf16x8(v);
    }
  // dz A (tap pair jp, q block mq): A[m = q = 16mq + n][k = 8g + i],
  //   k <-> (channel cw + 4g + i%4, tap 2jp + i/4)
  bf16x8 za[KP][NQ];
#pragma unroll
  for (int jp = 0; jp < KP; ++jp)
#pragma unroll
    for (int mq = 0; mq < NQ; ++mq) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 16 * mq + n, j = 2 * jp + (i >> 2);
        const int64_t c = cw + 4 * g + (i & 3);
        v[i] = (q < rank && j < K && c < s.D) ? (float)P.U[(int64_t)q * Dk + c * K + j] : 0.f;
      }
      za[jp][mq] = pack_bf16x8(v);
    }

  f32x4 dUacc[K][NQ];
#pragma unroll
  for (int j = 0; j < K; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dwl[wave][(4 * j + r) * 64 + lane] = 0.f;  // (only this lane touches its slots)
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) dUacc[j][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- global -> register prefetch of one tile ----
  // Each thread's load slots are fixed for the block: precompute their byte
  // offset at tile 0 and their LDS destination once.  Per tile the offset only
  // advances; the buffer's range check returns zeros for every slot whose
  // offset falls outside the tensor: rows before 0 (the offset wraps to the
  // top of the 32-bit range; clamped to kTop so that the offset plus the
  // access size never wraps past 2^32), rows past BT, and masked slots
  // (offset kOutside + tile advance, still above the tensor, which is under
  // 2 GiB).
  const int tile_lo = blockIdx.y * P.tpb;
  const int tile_hi = min(P.n_tiles, tile_lo + P.tpb);
  const int D = (int)s.D;  // B*T*D < 2^31 (host-checked)
  // slot q of a thread: chunk e of the virtual list [x chunks, padded][dy
  // chunks, padded]; whether it is x or dy is the same for the whole wave (a
  // scalar choice of buffer resource, not a per-lane one)
  const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);
  uint32_t v_gbase[kVL];
  int v_loff[kVL];
  bool v_isx[kVL];
#pragma unroll
  for (int q = 0; q < kVL; ++q) {
    const bool isx = q * NT + wave_base < CHXP;
    const int e = tid + q * NT;
    const int e2 = isx ? e : e - CHXP;
    const int r = e2 / CH, c16 = e2 % CH;
    const bool in = e2 < CHX;                        // the slot has a place in the tile
    const bool ok = in && cblk + c16 * 8 < s.D;      // ... and its channels exist (else zeros)
    v_isx[q] = isx;
    v_gbase[q] = ok ? (uint32_t)((isx ? r - KH : r) * D + (int)cblk + c16 * 8) * 2u : kOutside;
    v_loff[q] = in ? r * kRow + c16 * 8 : TR * kRow;
  }
  uint32_t z_gbase[kZL];
  int zs_off[kZL], zt_off[kZL];
#pragma unroll
  for (int q = 0; q < kZL; ++q) {
    const int e = tid + q * NT;
    const int zr = e / ZC, zc = e % ZC;
    const bool ok = e < TR * ZC && zc < rank;
    z_gbase[q] = ok ? (uint32_t)(zr * rank + zc) * 4u : kOutside;
    zs_off[q] = ok ? zr * ZW + zc : TR * ZW;
    zt_off[q] = ok && zr < 32 ? zc * kGRow + zr : ZC * kGRow;
  }
  // NSET register sets: tile i+NSET is loaded while tile i is computed
  uint4 vpre[NSET][kVL];
  float zpre[NSET][kZL];
  // loads are issued unconditionally (masked slots read zeros from outside the buffer)
  const auto rx = make_rsrc(P.x, (uint32_t)(s.BT * s.D * 2)), rdy = make_rsrc(P.dy, (uint32_t)(s.BT * s.D * 2));
  const auto rz = make_rsrc(P.z, (uint32_t)(s.BT * rank * 4));
  uint32_t ppre[NSET][2] = {};  // VAR: table entries of the lane's tokens n, 16 + n (zero past BT)
  const auto rp = make_rsrc(s.seqpos, VAR ? (uint32_t)(s.BT * 2) : 0u);
  auto prefetch = [&](int set, int tile) {
    const uint32_t vstep = (uint32_t)(tile * 32 * D) * 2u, zstep = (uint32_t)(tile * 32 * rank) * 4u;
    constexpr uint32_t kTop = 0xffffff00u;
#pragma unroll
    for (int q = 0; q < kVL; ++q) vpre[set][q] = buf_load16(v_isx[q] ? rx : rdy, min(v_gbase[q] + vstep, kTop));
#pragma unroll
    for (int q = 0; q < kZL; ++q) zpre[set][q] = buf_load_f32(rz, z_gbase[q] + zstep);
    if constexpr (VAR) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        ppre[set][tb] = __builtin_amdgcn_raw_buffer_load_b16(rp, (uint32_t)(tile * 32 + 16 * tb + n) * 2u, 0, 0);
    }
  };
  auto stage = [&](int set) {
#pragma unroll
    for (int q = 0; q < kVL; ++q) *reinterpret_cast<uint4 *>((v_isx[q] ? xs : dys) + v_loff[q]) = vpre[set][q];
#pragma unroll
    for (int q = 0; q < kZL; ++q) {
      const bf16 v = (bf16)zpre[set][q];
      zs[zs_off[q]] = v;
      zt[zt_off[q]] = v;
    }
  };

  if (tile_hi > tile_lo) prefetch(0, tile_lo);
  if (NSET > 1 && tile_hi > tile_lo + 1) prefetch(NSET - 1, tile_lo + 1);
  const auto rdx = make_rsrc(P.dx, (uint32_t)(s.BT * s.D * 2));
  const auto rg = make_rsrc(P.gpart + (int64_t)blockIdx.x * s.BT * rank, (uint32_t)(s.BT * rank * 4));
  // store offsets at tile 0 (the range checks of rdx / rg drop rows past BT
  // and masked slots): dx of the lane's token n, channels cw+4g .. +3; the dz
  // partial of thread -> (q, token), token fastest (consecutive threads read
  // consecutive lanes' rows of the exchange buffer)
  const uint32_t dx_base = cw + 4 * g + 4 <= s.D ? (uint32_t)(n * D + (int)cw + 4 * g) * 2u : kOutside;
  constexpr int NIT = (32 * ZC + NT - 1) / NT;
  uint32_t dz_base[NIT];
  int dz_src[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int o = tid + it * NT;
    const int sr = o % 32, q = o / 32;
    const bool ok = o < 32 * ZC && q < rank;
    const int tb = sr >> 4, nn = sr & 15, mq = q >> 4, gg = (q >> 2) & 3, r = q & 3;
    dz_src[it] = ok ? (16 * gg + nn) * RVP + (tb * NQ + mq) * 4 + r : 0;
    dz_base[it] = ok ? (uint32_t)(sr * rank + q) * 4u : kOutside;
  }
  const int wc = wave * kCW + 4 * g;     // the lane's first channel within the tile rows
  unsigned char *gtw = gt[wave];
  // G writes: token row 16tb + n, channel quad g; transposed reads for the
  // dU A operand: lane (channel n, token group g) supplies row 8g + 4h + n/4,
  // quad n%4 and receives tokens 8g+4h .. +3 of channel n
  const int gw_off[2] = {g_off(n, g), g_off(16 + n, g)};
  const int gr_off[2] = {g_off(8 * g + n / 4, n % 4), g_off(8 * g + 4 + n / 4, n % 4)};

  // position in its sequence of the current tile's first token (wave-uniform,
  // advanced by one tile per step)
  const int T = s.T;
  int p0 = (int)((uint32_t)(tile_lo * 32) % (uint32_t)T);
  auto tile_step = [&](const int set, const int tile) {
    const int64_t t0 = (int64_t)tile * 32;
    // only tiles that hold a token with pos < KH (x before its sequence start)
    // or rem < KH (dy past its sequence end: rem tokens follow it there) need
    // the per-token masks
    bool edge_lo, edge_hi;
    int pos[2] = {0, 0}, rem[2] = {0, 0};
    if constexpr (VAR) {
      edge_lo = edge_hi = KH > 0;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) pos[tb] = (int)(ppre[set][tb] & 255u), rem[tb] = (int)(ppre[set][tb] >> 8);
    } else {
      edge_lo = KH > 0 && (p0 < KH || T - p0 <= 31);
      edge_hi = KH > 0 && T - KH - p0 <= 31;
      if (edge_lo || edge_hi) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          pos[tb] = (int)((uint32_t)(p0 + 16 * tb + n) % (uint32_t)T);
          rem[tb] = T - 1 - pos[tb];
        }
      }
      p0 = T >= 32 ? (p0 + 32 >= T ? p0 + 32 - T : p0 + 32) : (p0 + 32) % T;
    }

    __syncthreads();  // the previous tile's LDS reads are done
    stage(set);
    __syncthreads();
    if (tile + NSET < tile_hi) prefetch(set, tile + NSET);

    // dy of the lane's two tokens: fp32 (dx starts as dy) and bf16 pairs with one half cleared
    float dxacc[2][4];
    uint32_t dlo[2][2], dhi[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint2 d = *reinterpret_cast<const uint2 *>(&dys[(16 * tb + n) * kRow + wc]);
      const uint32_t w[2] = {d.x, d.y};
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        dhi[tb][p] = w[p] & 0xffff0000u;
        dlo[tb][p] = w[p] & 0x0000ffffu;
        dxacc[tb][2 * p] = __uint_as_float(w[p] << 16);
        dxacc[tb][2 * p + 1] = __uint_as_float(dhi[tb][p]);
      }
    }
    // z^T fragments for dU: B[k = token 8g + i][n = q - 16nq]
    bf16x8 zb[NQ];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq)
      zb[nq] = as_bf16x8(*reinterpret_cast<const uint4 *>(&zt[(16 * nq + n) * kGRow + 8 * g]));

    f32x4 dzacc[2][NQ];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int mq = 0; mq < NQ; ++mq) dzacc[tb][mq] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t gev[2][2];  // G of the even tap of the current pair: bf16 pairs of channels 4g.. 4g+3

#pragma unroll
    for (int j = 0; j < K; ++j) {
      float gv[2][4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        // filter diagonal: element r = w[t0 + 16tb + n + j, channel wc + r, j]
        f32x4 wd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
          wd = mfma16(fa[j][kq],
                      as_bf16x8(*reinterpret_cast<const uint4 *>(&zs[(16 * tb + n + j) * ZW + 32 * kq + 8 * g])), wd);
        // dx += w[s+j] dy[s+j] (dy past the sequence end is zero)
        uint32_t w[2];
        if (j == 0) {
          w[0] = dlo[tb][0] | dhi[tb][0], w[1] = dlo[tb][1] | dhi[tb][1];
        } else {
          const uint2 d = *reinterpret_cast<const uint2 *>(&dys[(16 * tb + n + j) * kRow + wc]);
          w[0] = d.x, w[1] = d.y;
          if (__builtin_expect(edge_hi, 0) && j > rem[tb]) w[0] = 0u, w[1] = 0u;
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          dxacc[tb][2 * p] = fmaf(wd[2 * p], __uint_as_float(w[p] << 16), dxacc[tb][2 * p]);
          dxacc[tb][2 * p + 1] = fmaf(wd[2 * p + 1], __uint_as_float(w[p] & 0xffff0000u), dxacc[tb][2 * p + 1]);
        }
        // G[s, c, j] = dy[s, c] x[s-j, c] (x before the sequence start is zero)
        const uint2 xv = *reinterpret_cast<const uint2 *>(&xs[(16 * tb + n + KH - j) * kRow + wc]);
        uint32_t xw[2] = {xv.x, xv.y};
        if (__builtin_expect(edge_lo, 0) && j > pos[tb]) xw[0] = 0u, xw[1] = 0u;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          gv[tb][2 * p] = dot2z(xw[p], dlo[tb][p]);
          gv[tb][2 * p + 1] = dot2z(xw[p], dhi[tb][p]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) dwl[wave][(4 * j + r) * 64 + lane] += gv[0][r] + gv[1][r];
      // G of tap j rounded to bf16 once, channel pairs; token-major copy in LDS
      const bool odd = j & 1;
      uint32_t gq[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) gq[tb][h] = pack2(gv[tb][2 * h], gv[tb][2 * h + 1]);
        *reinterpret_cast<uint2 *>(gtw + (odd ? kGTap : 0) + gw_off[tb]) = make_uint2(gq[tb][0], gq[tb][1]);
      }
      if (!odd && j < K - 1) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int h = 0; h < 2; ++h) gev[tb][h] = gq[tb][h];
        continue;
      }
      // a tap pair (2jp, 2jp+1) is complete (the odd tap is zero past k):
      // the dz MFMA, then dU from the transposed copy
      const int jp = j >> 1;
      // dz: B[k = 8g + i][token n], k <-> (channel 4g + i%4, tap 2jp + i/4)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 bb = odd ? as_bf16x8(make_uint4(gev[tb][0], gev[tb][1], gq[tb][0], gq[tb][1]))
                              : as_bf16x8(make_uint4(gq[tb][0], gq[tb][1], 0u, 0u));
#pragma unroll
        for (int mq = 0; mq < NQ; ++mq) dzacc[tb][mq] = mfma16(za[jp][mq], bb, dzacc[tb][mq]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // dU: A[m = channel n][k = token 8g + i] = G of the tap; B = z^T
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jt = 2 * jp + jj;
        if (jt < K) {
          const uint2 lo = read_tr16(gtw + jj * kGTap + gr_off[0]);
          const uint2 hi = read_tr16(gtw + jj * kGTap + gr_off[1]);
          const uint4 raw = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int nq = 0; nq < NQ; ++nq) dUacc[jt][nq] = mfma16(as_bf16x8(raw), zb[nq], dUacc[jt][nq]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // dx of the lane's two tokens (stores issued unconditionally; masked
    // lanes write outside the buffer, which drops them)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint32_t off = dx_base + (uint32_t)(((int)t0 + 16 * tb) * D) * 2u;
      buf_store8(rdx, off, make_uint2(pack2(dxacc[tb][0], dxacc[tb][1]), pack2(dxacc[tb][2], dxacc[tb][3])));
    }
    // dz partial of the wave: element (tb*NQ + mq)*4 + r = dz[t0 + 16tb + n][16mq + 4g + r]
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int mq = 0; mq < NQ; ++mq)
        *reinterpret_cast<float4 *>(&red[wave][lane * RVP + (tb * NQ + mq) * 4]) =
            make_float4(dzacc[tb][mq][0], dzacc[tb][mq][1], dzacc[tb][mq][2], dzacc[tb][mq][3]);
    __syncthreads();
    // the waves' sum, one partial per (slice, token): thread -> (q, token),
    // token fastest (consecutive threads read consecutive lanes' rows)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float v = red[0][dz_src[it]];
#pragma unroll
      for (int w = 1; w < kW; ++w) v += red[w][dz_src[it]];
      buf_store_f32(rg, dz_base[it] + (uint32_t)((int)t0 * rank) * 4u, v);
    }
  };
  // unrolled by two so that each register set has fixed registers
  for (int tile = tile_lo; tile < tile_hi; tile += 2) {
    tile_step(0, tile);
    if (tile + 1 < tile_hi) tile_step(NSET - 1, tile + 1);
  }

  // ---- block epilogue: dU and dw0 partials of this token range ----
#pragma unroll
  for (int j = 0; j < K; ++j) {
    // dw0: the 16 lanes of one g hold the same channels, different tokens
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = dwl[wave][(4 * j + r) * 64 + lane];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      const int64_t c = cw + 4 * g + r;
      if (n == 0 && c < s.D) P.dw0p[(int64_t)blockIdx.y * Dk + c * K + j] = v;
    }
    // dU: lane holds D[m = 4g + r][q - 16nq = n] = dU[q][(cw + 4g + r) * k + j]
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = 16 * nq + n;
        const int64_t c2 = cw + 4 * g + r;
        if (q < rank && c2 < s.D) P.dUp[((int64_t)blockIdx.y * rank + q) * Dk + c2 * K + j] = dUacc[j][nq][r];
      }
  }
}

}  // namespace bwdlr

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool bwd_fused_supported(const Shape &s) {
  return s.kind == DYNCONV_HEADWISE ? bwd_headwise_supported(s) : bwd_lowrank_supported(s);
}

BwdLayout bwd_layout(const Shape &s) {
  return s.kind == DYNCONV_HEADWISE ? bwd_headwise_layout(s) : bwd_lowrank_layout(s);
}

bool bwd_lowrank_supported(const Shape &s) {
  // 32-bit element and byte offsets: x, dy, dx below 2 GiB
  return s.kind == DYNCONV_LOWRANK && s.D % 8 == 0 && s.k <= 8 && s.rank >= 1 && s.rank <= 64 &&
         s.BT * s.D * 2 < ((int64_t)1 << 31) - 64;
}

BwdLayout bwd_lowrank_layout(const Shape &s) {
  BwdLayout L = {};
  L.Dt = bwdlr::waves_for(s) * bwdlr::kCW;
  L.n_slices = (int)ceil_div(s.D, L.Dt);
  L.n_tiles = (int)ceil_div(s.BT, 32);
  // token ranges: 512 blocks (one round of two resident 4-wave blocks per CU,
  // or two rounds of one 8-wave block)
  const int target = 512;
  int tpb = 1;
  while ((int64_t)L.n_slices * ceil_div(L.n_tiles, tpb) > target) ++tpb;
  L.tpb = tpb;
  L.n_ranges = (int)ceil_div(L.n_tiles, tpb);
  L.SL = 0;
  L.R = s.rank;
  return L;
}

int bwd_lowrank(const Shape &s, const BwdLayout &L, const float *z, const void *U, const void *w0, const void *x,
                const void *dy, void *dx, float *gpart, float *dUp, float *dw0p, hipStream_t st) {
  bwdlr::Params P;
  P.s = s;
  P.x = (const bf16 *)x;
  P.dy = (const bf16 *)dy;
  P.dx = (bf16 *)dx;
  P.z = z;
  P.U = (const bf16 *)U;
  P.w0 = (const bf16 *)w0;
  P.gpart = gpart;
  P.dUp = dUp;
  P.dw0p = dw0p;
  P.tpb = L.tpb;
  P.n_tiles = L.n_tiles;
  const int kw = bwdlr::waves_for(s);
  const dim3 grid((unsigned)L.n_slices, (unsigned)L.n_ranges), block(kw * 64);
  const int KQ = (int)ceil_div(s.rank + 1, 32), NQ = (int)ceil_div(s.rank, 16);
  const bool tr = trace_begin(DYNCONV_K_BWD_CONV, st);
  int rc = 0;
  // one 16-row block of rank (NQ = 1) <=> rank <= 16 <=> 4 waves per block
#define LR(K_, KQ_, NQ_, W_)                                                                  \
  do {                                                                                        \
    if (s.seqpos)                                                                             \
      hipLaunchKernelGGL((bwdlr::k_bwd_lr<K_, KQ_, NQ_, W_, true>), grid, block, 0, st, P);  \
    else                                                                                      \
      hipLaunchKernelGGL((bwdlr::k_bwd_lr<K_, KQ_, NQ_, W_, false>), grid, block, 0, st, P); \
  } while (0)
// ranks 33..64 (three or four 16-row blocks): 4-wave blocks, one wave per
// SIMD (their U fragments and dU accumulators take most of the registers)
#define LR_WIDE(K_)                                         \
  else if (KQ == 2 && NQ == 3) LR(K_, 2, 3, 4);             \
  else if (KQ == 2 && NQ == 4) LR(K_, 2, 4, 4);             \
  else if (KQ == 3 && NQ == 4) LR(K_, 3, 4, 4);
#define LR_K(K_)                                            \
  if (KQ == 1 && NQ == 1 && kw == 4) LR(K_, 1, 1, 4);       \
  else if (KQ == 1 && NQ == 2 && kw == 8) LR(K_, 1, 2, 8);  \
  else if (KQ == 2 && NQ == 2 && kw == 8) LR(K_, 2, 2, 8);  \
  LR_WIDE(K_)                                               \
  else rc = DYNCONV_E_LIMIT;
#define LR_K8(K_)                                           \
  if (KQ == 1 && NQ == 1) LR(K_, 1, 1, 4);                  \
  else if (KQ == 1 && NQ == 2) LR(K_, 1, 2, 4);             \
  else if (KQ == 2 && NQ == 2) LR(K_, 2, 2, 4);             \
  LR_WIDE(K_)                                               \
  else rc = DYNCONV_E_LIMIT;
  switch (s.k) {
    case 1: LR_K(1) break;
    case 2: LR_K(2) break;
    case 3: LR_K(3) break;
    case 4: LR_K(4) break;
    case 5: LR_K8(5) break;
    case 6: LR_K8(6) break;
    case 7: LR_K8(7) break;
    case 8: LR_K8(8) break;
    default: rc = DYNCONV_E_LIMIT;
  }
#undef LR_K8
#undef LR_K
#undef LR_WIDE
#undef LR
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
