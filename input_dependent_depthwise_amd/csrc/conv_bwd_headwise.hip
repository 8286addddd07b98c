// conv_bwd_headwise.hip -- fused backward of the head-wise dynamic short
// convolution (bf16 I/O), one lane per run of channels walking along time.
//
// Layer (gist.science Technical Summary of "Dynamic Short Convolutions Improve
// Transformers", Methodology -> Dynamic Short Convolutions: Mechanism,
// Parameterization): y[t,c] = x[t,c] + sum_j w[t,c,j] x[t-j,c] with the
// head-wise filter w[t,c,j] = u[t,head(c),j] + w0[c,j].  For L = sum(dy * y):
//   dx[s,c]   = dy[s,c] + sum_j [s, s+j in one sequence] w[s+j,c,j] dy[s+j,c]
//   du[t,e,j] = sum_{c in head e} dy[t,c] x[t-j,c]      (x before the sequence start is 0)
//   dw0[c,j]  = sum_t dy[t,c] x[t-j,c]
//
// Mapping.  A lane owns CPL = 8 (or 4) consecutive channels of one head; a
// wave covers 64*CPL channels (a "span") and walks a contiguous run of tokens.
// All lanes of a wave sit on the same token at every step, so sequence
// boundaries are wave-uniform scalar tests, and the k-tap history of x and the
// k-1 dx accumulators still open stay in registers:
//   * dx is formed in scatter order: token t adds w[t,c,j] dy[t,c] to the
//     accumulator of token t-j, which is complete (and stored) k-1 steps later;
//   * du partials per lane are bf16 dot products over the lane's channel pairs
//     (v_dot2), then summed over the lanes of a head either with DPP
//     transpose-reductions (heads of 1..16 lanes, aligned) or as differences
//     of a wave-wide prefix sum (any other head width), and written as one
//     fp32 partial per span.  Head widths of 4 mod 8 (e.g. 68) keep 8
//     channels per lane: a lane's two quads of 4 channels may then lie in two
//     heads, each quad with its own u and its own du sum;
//   * dw0 accumulates in registers over the wave's tokens; the block's 4 waves
//     (same span, consecutive token runs) add theirs in LDS and write one
//     fp32 partial per block, summed later in a fixed order.
// Loads run 4 tokens ahead, into 8-slot rings (for x the ring doubles as the
// k-tap history).
#include "kernels.h"
#include "bufio.h"

namespace dynconv {
namespace bwdhw {

struct Params {
  Shape s;
  const bf16 *x, *dy;
  bf16 *dx;
  const float *u;     // [BT, n_heads*k]
  const bf16 *w0;     // [D, k] or NULL
  float *gpart;       // [n_spans][BT][R]: du partial per head slot of the span
  float *dw0p;        // [n_groups][D*k]
  int L;              // tokens per wave
  int SL, R;          // head slots per span, R = SL*k
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// within each row of 16 lanes (lanes whose source lies before their row add
// 0), then rows 1 and 3 add the last lane of the row before them (row_bcast:15)
// and rows 2 and 3 the last lane of row 1 (row_bcast:31).
__device__ __forceinline__ float wave_prefix(float v) {
  v += dpp<0x111>(v);
  v += dpp<0x112>(v);
  v += dpp<0x114>(v);
  v += dpp<0x118>(v);
  v += dpp_rows<0x142, 0xa>(v);
  v += dpp_rows<0x143, 0xc>(v);
  return v;
}

// DPP partner patterns, by the highest lane-index bit they flip: xor 15
// (row_mirror), xor 7 (row_half_mirror), xor 2, xor 1 (quad_perm).
template <int B>
constexpr int kXorCtrl = B == 3 ? 0x140 : B == 2 ? 0x141 : B == 1 ? 0x4E : 0xB1;

// One halving step of a transpose-reduction over lane pairs that differ in
// bit B of the lane index: the lane with bit B clear keeps the low half of its
// NV values, the other the high half, each adding the partner's copy of the
// half it keeps.
template <int NV, int B, int N>
__device__ __forceinline__ void tr_step(float (&v)[N], int lane) {
  const bool up = (lane >> B) & 1;
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const float keep = up ? v[NV / 2 + i] : v[i];
    const float send = up ? v[i] : v[NV / 2 + i];
    v[i] = keep + dpp<kXorCtrl<B>>(send);
  }
}

// Sum the 4 tap values over aligned groups of S lanes (S = 1, 2, 4, 8, 16).
// Afterwards lane p of a group holds the sums of taps p*NV .. p*NV+NV-1 in
// v[0 .. NV-1] with NV = 4/S (S <= 4); for S > 4 it holds tap p/(S/4) in v[0].
template <int S>
__device__ __forceinline__ void group_reduce4(float (&v)[4], int lane) {
  if constexpr (S == 16) {
    tr_step<4, 3>(v, lane);
    tr_step<2, 2>(v, lane);
    v[0] += dpp<kXorCtrl<1>>(v[0]);
    v[0] += dpp<kXorCtrl<0>>(v[0]);
  } else if constexpr (S == 8) {
    tr_step<4, 2>(v, lane);
    tr_step<2, 1>(v, lane);
    v[0] += dpp<kXorCtrl<0>>(v[0]);
  } else if constexpr (S == 4) {
    tr_step<4, 1>(v, lane);
    tr_step<2, 0>(v, lane);
  } else if constexpr (S == 2) {
    tr_step<4, 0>(v, lane);
  }
}

// Raw buffer accesses: 32-bit byte offsets from a per-tensor resource (base
// address in SGPRs), so per-token addressing is one scalar add.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

template <int CPL>
__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t (&w)[CPL / 2]) {
  if constexpr (CPL == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = v[0], w[1] = v[1];
  }
}

template <int K, int KU>
__device__ __forceinline__ void bload_u(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float (&u)[KU]) {
  if constexpr (K > 4) {  // taps 0..3, then the rest
    float lo[4], hi[4];
    bload_u<4, 4>(r, voff, soff, lo);
    bload_u<K - 4, 4>(r, voff + 16u, soff, hi);
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = lo[j], u[4 + j] = hi[j];
  } else if constexpr (K == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    u[0] = __uint_as_float(v[0]), u[1] = __uint_as_float(v[1]), u[2] = __uint_as_float(v[2]),
    u[3] = __uint_as_float(v[3]);
  } else if constexpr (K == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    u[0] = __uint_as_float(v[0]), u[1] = __uint_as_float(v[1]), u[2] = __uint_as_float(v[2]), u[3] = 0.f;
  } else if constexpr (K == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    u[0] = __uint_as_float(v[0]), u[1] = __uint_as_float(v[1]), u[2] = 0.f, u[3] = 0.f;
  } else {
    u[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0)), u[1] = 0.f, u[2] = 0.f,
    u[3] = 0.f;
  }
}

template <int CPL>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const uint32_t (&w)[CPL / 2]) {
  if constexpr (CPL == 8) {
    __builtin_amdgcn_raw_buffer_store_b128((__attribute__((ext_vector_type(4))) unsigned){w[0], w[1], w[2], w[3]},
                                           r, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64((__attribute__((ext_vector_type(2))) unsigned){w[0], w[1]}, r, voff, soff, 0);
  }
}

// S: lanes per head when heads are 1..16 lanes wide and aligned to spans; 0:
// any head width that is a multiple of CPL (prefix sums); -1 (CPL = 8): head
// widths of 4 mod 8, at least 12 (prefix sums over channel quads); -2: static
// filter, no generator (no du at all).  VAR: packed documents (positions from
// the per-token table).
template <int K, int CPL, int S, bool VAR>
__global__ void __launch_bounds__(256, 2)
k_bwd_hw(Params P) {
  constexpr bool QUAD = S == -1;
  constexpr bool NODU = S == -2;
  static_assert(!QUAD || CPL == 8, "quad heads: 8 channels per lane");
  static_assert(K <= 4 || (CPL == 4 && S <= 0 && S != -1), "5..8 taps: 4 channels per lane, prefix sums");
  constexpr int NP = CPL / 2;        // bf16 pairs per lane
  constexpr int SPAN = 64 * CPL;
  // Tokens loaded ahead.  Eight (with rings twice as deep) measured no
  // faster: the compiler's wait counts across the per-token branches then
  // stop short of the deeper rings.
  constexpr int PD = 4;
  constexpr int KU = K <= 4 ? 4 : 8;             // tap slots (u, bias, du sums)
  constexpr int AR = KU;                         // dx accumulators: tokens still open (slot = (s - t_a) mod AR)
  constexpr int XS = K <= 4 ? 2 * PD : 4 * PD;   // x ring slots: the k-1 history plus the loads in flight
  constexpr int YS = PD;                         // dy and u ring slots
  constexpr int BLK = XS;                        // tokens per unrolled block
  static_assert(XS >= K + PD, "x ring");
  const Shape &s = P.s;

  __shared__ __attribute__((aligned(16))) float dwred[4][64 * CPL * K];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int span = blockIdx.x;
  const int Dc = (int)s.D;
  const int span_c0 = span * SPAN;
  const int c0 = span_c0 + lane * CPL;
  const bool act = c0 < Dc;
  const bool all_act = span_c0 + SPAN <= Dc;
  const int cc = act ? c0 : Dc - CPL;  // clamped: inactive lanes read valid memory, use dy = 0
  const int e = (int)(cc / s.hd);
  const int e2 = QUAD ? (int)((cc + 4) / s.hd) : e;  // head of the lane's second quad
  const int e_lo = (int)(span_c0 / s.hd);
  const int BT = (int)s.BT;  // the host keeps every tensor below 2 GiB (32-bit byte offsets)
  const int T = s.T;

  // per-lane bias: CPL*K contiguous bf16 at w0[cc*K], read as dwords with
  // unconditional buffer loads (no bias: an empty buffer, every load reads 0)
  float w0r[CPL][KU];
  {
    const auto rw = rsrc(P.w0, P.w0 ? (uint32_t)(Dc * K * 2) : 0u);
    constexpr int NW = CPL * K / 2;
    uint32_t wv[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q) wv[q] = __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(cc * K * 2 + 4 * q), 0, 0);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < KU; ++j) {
        const int el = i * K + j;
        w0r[i][j] = j < K ? __uint_as_float((el & 1) ? (wv[el >> 1] & 0xffff0000u) : (wv[el >> 1] << 16)) : 0.f;
      }
  }

  float dwacc[CPL][K];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int j = 0; j < K; ++j) dwacc[i][j] = 0.f;

  const int t_a = ((int)blockIdx.y * 4 + wave) * P.L;
  const int t_b = t_a + P.L < BT ? t_a + P.L : BT;
  // dx needs k-1 steps past the run (their dy and u, where they exist) before
  // the run's last accumulators are complete
  const int t_end = t_b + K - 1;

  const uint32_t row_x = (uint32_t)s.D * 2u, row_u = (uint32_t)s.N * 4u;
  const auto rx = rsrc(P.x, (uint32_t)(BT * row_x)), rdy = rsrc(P.dy, (uint32_t)(BT * row_x));
  const auto rdx = rsrc(P.dx, (uint32_t)(BT * row_x)), ru = rsrc(P.u, (uint32_t)(BT * row_u));
  const uint32_t voff_x = (uint32_t)cc * 2u, voff_u = (uint32_t)e * K * 4u, voff_u2 = (uint32_t)e2 * K * 4u;
  // du partials of this span: [BT][R] fp32
  const uint32_t row_g = (uint32_t)P.R * 4u;
  const auto rg = rsrc(P.gpart + (size_t)span * BT * P.R, (uint32_t)BT * row_g);
  const uint32_t voff_g = (uint32_t)(e - e_lo) * K * 4u;
  // any head width (S = 0): this lane's head covers lanes [hla, lb) of the
  // span (heads are whole lanes: hd is a multiple of CPL); its last lane
  // writes the head's sums
  int hla = 0;
  bool hlast = false;
  if constexpr (S == 0) {
    const int nact = all_act ? 64 : (Dc - span_c0) / CPL;
    hla = max(0, (e * s.hd - span_c0) / CPL);
    const int lb = min(nact, ((e + 1) * s.hd - span_c0) / CPL);
    hlast = act && lane == lb - 1;
  }
  // quad heads: at most one head starts in a lane, at its first quad (qA) or
  // its second (qB); sb = the wave's prefix sum up to that start.  The lane
  // holding the start of head h+1 writes head h's sum (its sb minus the sb of
  // the lane where h starts, or minus 0 when h starts at or before the span);
  // the last active lane also writes the head of its second quad (its
  // inclusive prefix minus that head's start).  q_src: the lane whose sb this
  // lane needs (h's start for the first write, else the last quad's head's).
  bool qA = false, qB = false, q_prev = false, q_last = false, q_zero = true;
  int q_src = 0;
  if constexpr (QUAD) {
    const int hd = (int)s.hd;
    const int nact = all_act ? 64 : (Dc - span_c0) / CPL;
    qA = act && cc % hd == 0;
    qB = act && (cc + 4) % hd == 0;
    q_prev = (qA && lane > 0) || qB;
    q_last = act && lane == nact - 1;
    const int st = (q_prev ? e2 - 1 : e2) * hd - span_c0;  // that head's first channel, from the span start
    q_zero = st <= 0;
    q_src = q_zero ? 0 : st / CPL;
  }

  if (t_a < BT) {
    // token rings: x in XS slots (slot = (t - t_a) mod XS) holding tokens
    // t-3 .. t+PD (the k-tap history plus the loads in flight), dy and u in YS
    // (slot = (t - t_a) mod YS) holding tokens t .. t+PD
    uint32_t xr[XS][NP], dyr[YS][NP];
    float ur[YS][KU], ur2[YS][KU];  // u of the lane's head (quad heads: of each quad's head)
    float acc[AR][CPL];             // dx accumulators
#pragma unroll
    for (int a = 0; a < AR; ++a)
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[a][i] = 0.f;

    int pos = VAR ? 0 : (int)(t_a % T);  // position in its sequence of the next token to process
    // VAR (packed documents): positions from the per-token table, the eight of
    // a block in two scalar loads issued a block ahead (t_a and the run length
    // are multiples of 4; the table is padded past its last token)
    const uint64_t *sp4 = reinterpret_cast<const uint64_t *>(s.seqpos);
    uint64_t pn[BLK / 4];
#pragma unroll
    for (int q = 0; q < BLK / 4; ++q) pn[q] = VAR ? sp4[(t_a >> 2) + q] : 0;
    // Loads are unconditional: row offsets are clamped to the batch, and what
    // they bring past the run is never consumed (tokens past t_end are not
    // processed, x past t_b feeds no product, and every token past the batch
    // end starts a new "sequence" for the position tests).
    auto row = [&](int t) { return (uint32_t)(t < BT ? (t > 0 ? t : 0) : BT - 1); };
    // x history before t_a (the taps that reach before the sequence start are
    // skipped by the position tests, not zeroed)
#pragma unroll
    for (int j = KU - 1; j >= 1; --j) {
      if (j < K) bload<CPL>(rx, voff_x, row(t_a - j) * row_x, xr[XS - j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // token t into x slot xs, dy and u slot xs mod 4
    auto load_tok = [&](int t, int xs) {
      const uint32_t r = row(t);
      bload<CPL>(rx, voff_x, r * row_x, xr[xs]);
      bload<CPL>(rdy, voff_x, r * row_x, dyr[xs & (YS - 1)]);
      bload_u<K, KU>(ru, voff_u, r * row_u, ur[xs & (YS - 1)]);
      if constexpr (QUAD) bload_u<K, KU>(ru, voff_u2, r * row_u, ur2[xs & (YS - 1)]);
    };
    // (issued in the loop's own order, so that the wait counts the compiler
    // derives at the loop head hold for the first pass too)
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      load_tok(t_a + i, i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Registers of the last stores stay reserved until the next token's loads
    // are issued: on this target a register read by a pending store can only be
    // rewritten after a vmcnt wait, which would also drain the loads in flight.
    constexpr int NH = NP + (QUAD ? 8 : KU);
    uint32_t held[NH];  // dx of this token, du of the previous one
#pragma unroll
    for (int p = 0; p < NH; ++p) held[p] = 0u;

    // one block of BLK tokens from tg.  The tests on t and pos are wave-uniform
    // (scalar branches); keeping them in every block rather than compiling a
    // second, test-free copy keeps the register allocation of the rings simple.
    auto block = [&](int tg) {
      uint64_t pc[BLK / 4];
#pragma unroll
      for (int q = 0; q < BLK / 4; ++q) {
        pc[q] = pn[q];
        if constexpr (VAR) pn[q] = sp4[(tg >> 2) + BLK / 4 + q];
      }
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        const int t = tg + i;
        float vals[KU], valsb[KU];  // (quad heads: valsb = the second quad's sums)
#pragma unroll
        for (int j = 0; j < KU; ++j) vals[j] = 0.f, valsb[j] = 0.f;
        // a token past the batch end starts a new "sequence" (its loads were clamped)
        if constexpr (VAR) pos = t < BT ? (int)((pc[i >> 2] >> (16 * (i & 3))) & 255u) : 0;
        if (t < t_end) {
          const bool main = t < t_b;
          // (lanes past D in a partial last span compute on the clamped
          // channels; nothing of theirs is stored or summed)
          uint32_t dw[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) dw[p] = dyr[i & (YS - 1)][p];
          // dy as fp32 and as bf16 pairs with one half cleared
          float dyf[CPL];
          uint32_t dlo[NP], dhi[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            dhi[p] = dw[p] & 0xffff0000u;
            dlo[p] = dw[p] & 0x0000ffffu;
            dyf[2 * p] = __uint_as_float(dw[p] << 16);
            dyf[2 * p + 1] = __uint_as_float(dhi[p]);
          }
          // taps j reaching before the sequence start (pos < j) contribute nothing
#pragma unroll
          for (int j = 0; j < K; ++j) {
            if (j == 0 || pos >= j) {
              const int xs = (i - j) & (XS - 1);
              if constexpr (!NODU) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                  if (QUAD && p >= 2)
                    valsb[j] = dot2(xr[xs][p], dw[p], valsb[j]);
                  else
                    vals[j] = dot2(xr[xs][p], dw[p], vals[j]);
                }
              }
              if (main) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                  dwacc[2 * p][j] = dot2(xr[xs][p], dlo[p], dwacc[2 * p][j]);
                  dwacc[2 * p + 1][j] = dot2(xr[xs][p], dhi[p], dwacc[2 * p + 1][j]);
                }
              }
            }
          }
          if (main) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const float u0 = (QUAD && c >= 4) ? ur2[i & (YS - 1)][0] : ur[i & (YS - 1)][0];
              acc[i & (AR - 1)][c] = fmaf(u0 + w0r[c][0], dyf[c], dyf[c]);
            }
          }
#pragma unroll
          for (int j = 1; j < K; ++j) {
            if (pos >= j) {
#pragma unroll
              for (int c = 0; c < CPL; ++c) {
                const float uj = (QUAD && c >= 4) ? ur2[i & (YS - 1)][j] : ur[i & (YS - 1)][j];
                acc[(i - j) & (AR - 1)][c] = fmaf(uj + w0r[c][j], dyf[c], acc[(i - j) & (AR - 1)][c]);
              }
            }
          }
          // token t-k+1 has all its terms
          const int so = t - (K - 1);
          if (so >= t_a && so < t_b) {
            const float *a = acc[(i - (K - 1)) & (AR - 1)];
            uint32_t o[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const bf16x2_t pr = {(bf16)a[2 * p], (bf16)a[2 * p + 1]};
              o[p] = __builtin_bit_cast(uint32_t, pr);
            }
            if (all_act)
              bstore<CPL>(rdx, voff_x, (uint32_t)so * row_x, o);
            else if (act)
              bstore<CPL>(rdx, voff_x, (uint32_t)so * row_x, o);
#pragma unroll
            for (int p = 0; p < NP; ++p) held[p] = o[p];
          }
          if constexpr (!VAR) {
            if (++pos == T) pos = 0;
          }
        }
        // refill: token t+PD into the slot just released
        load_tok(t + PD, (i + PD) & (XS - 1));
        // the previous token's stores have been followed by these loads; their
        // registers may be reused from here on
#pragma unroll
        for (int p = 0; p < NH; ++p) asm volatile("" ::"v"(held[p]));
        // du of this token: sum over the lanes of each head
        if constexpr (NODU) {
        } else if constexpr (S > 0) {
          if (t < t_b) {
            group_reduce4<S>(vals, lane);
            const int p = lane % S;
            const uint32_t so_g = (uint32_t)t * row_g;
            if constexpr (S <= 4) {
              constexpr int NV = 4 / S;
#pragma unroll
              for (int r = 0; r < NV; ++r) {
                if ((all_act || act) && p * NV + r < K)
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vals[r]), rg,
                                                        voff_g + (uint32_t)(p * NV + r) * 4u, so_g, 0);
                held[NP + r] = __float_as_uint(vals[r]);
              }
            } else {
              const int j = p / (S / 4);
              if ((all_act || act) && p % (S / 4) == 0 && j < K)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vals[0]), rg, voff_g + (uint32_t)j * 4u, so_g,
                                                      0);
              held[NP] = __float_as_uint(vals[0]);
            }
          }
        } else if constexpr (QUAD) {
          if (t < t_b) {
            float hp[4], hl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float pre = wave_prefix(vals[j] + valsb[j]);
              const float sb = pre - valsb[j] - (qA ? vals[j] : 0.f);
              const float got =
                  __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * q_src, __builtin_bit_cast(int, sb)));
              const float start = q_zero ? 0.f : got;
              hp[j] = sb - start;
              hl[j] = pre - ((qA || qB) ? sb : start);
            }
            const uint32_t og = (uint32_t)t * row_g;
            const uint32_t op = og + (uint32_t)(e2 - 1 - e_lo) * K * 4u, ol = og + (uint32_t)(e2 - e_lo) * K * 4u;
            if constexpr (K == 4) {
              buf_store16(rg, q_prev ? op : kOutside,
                          make_uint4(__float_as_uint(hp[0]), __float_as_uint(hp[1]), __float_as_uint(hp[2]),
                                     __float_as_uint(hp[3])));
              buf_store16(rg, q_last ? ol : kOutside,
                          make_uint4(__float_as_uint(hl[0]), __float_as_uint(hl[1]), __float_as_uint(hl[2]),
                                     __float_as_uint(hl[3])));
            } else {
#pragma unroll
              for (int j = 0; j < K; ++j) {
                buf_store_f32(rg, q_prev ? op + (uint32_t)j * 4u : kOutside, hp[j]);
                buf_store_f32(rg, q_last ? ol + (uint32_t)j * 4u : kOutside, hl[j]);
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              held[NP + j] = __float_as_uint(hp[j]);
              held[NP + 4 + j] = __float_as_uint(hl[j]);
            }
          }
        } else {
          // any head width: head sums as differences of the wave's prefix sums
          if (t < t_b) {
            float hs[KU];
#pragma unroll
            for (int j = 0; j < KU; ++j) {
              if (j >= K) {
                hs[j] = 0.f;
                continue;
              }
              const float pre = wave_prefix(vals[j]);
              const float before = __builtin_bit_cast(
                  float, __builtin_amdgcn_ds_bpermute(4 * (hla > 0 ? hla - 1 : 0), __builtin_bit_cast(int, pre)));
              hs[j] = hla > 0 ? pre - before : pre;
            }
            // (the partials stay below 2 GiB, so kOutside lies past them)
            const uint32_t og = (uint32_t)t * row_g + voff_g;
            if constexpr (K == 4) {
              buf_store16(rg, hlast ? og : kOutside,
                          make_uint4(__float_as_uint(hs[0]), __float_as_uint(hs[1]), __float_as_uint(hs[2]),
                                     __float_as_uint(hs[3])));
            } else {
#pragma unroll
              for (int j = 0; j < K; ++j) buf_store_f32(rg, hlast ? og + (uint32_t)j * 4u : kOutside, hs[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) held[NP + j] = __float_as_uint(hs[j]);
          }
        }
        // keep each token's work in its own scheduling region: interleaving
        // tokens only raises register pressure (the loads are already ahead)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int tg = t_a; tg < t_end; tg += BLK) block(tg);
  }

  // dw0: add the block's 4 waves (same channels), one partial per block
  {
    float *dst = &dwred[wave][lane * CPL * K];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) dst[i * K + j] = dwacc[i][j];
  }
  __syncthreads();
  const int nvals = (Dc - span_c0 < SPAN ? Dc - span_c0 : SPAN) * K;
  float *out = P.dw0p + (size_t)blockIdx.y * Dc * K + (size_t)span_c0 * K;
  for (int idx = threadIdx.x; idx < nvals; idx += 256)
    out[idx] = ((dwred[0][idx] + dwred[1][idx]) + dwred[2][idx]) + dwred[3][idx];
}

}  // namespace bwdhw

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// channels per lane: 8 when heads are a multiple of 8 wide, or 4 mod 8 and
// at least 12 (quad heads); 4 for heads of 4 channels, and for 5..8 taps
// (whose rings take twice the registers) with any head width that is a
// multiple of 4
static bool hw_quad(const Shape &s) { return s.k <= 4 && s.hd % 8 == 4 && s.hd >= 12; }
static int hw_cpl(const Shape &s) {
  if (s.k > 4) return s.hd % 4 == 0 ? 4 : 0;
  return (s.hd % 8 == 0 || hw_quad(s)) ? 8 : (s.hd % 4 == 0 ? 4 : 0);
}

BwdLayout bwd_headwise_layout(const Shape &s) {
  BwdLayout L = {};
  const int cpl = hw_cpl(s);
  const int span = 64 * cpl;
  L.Dt = span;
  L.n_slices = (int)ceil_div(s.D, span);
  // Blocks (4 waves, one per SIMD) resident per CU, from each variant's
  // register count (512 per SIMD lane): the grid is sized to one round of
  // them over the 256 CUs, never more, so no block waits for a second round.
  static const int kBlocksPerCU[3][8] = {{8, 6, 5, 4, 3, 2, 2, 2},  // 4 channels per lane, k = 1..8
                                         {6, 3, 3, 2, 0, 0, 0, 0},      // 8 channels per lane
                                         {5, 3, 2, 2, 0, 0, 0, 0}};     // quad heads
  const int64_t slots = 256 * kBlocksPerCU[hw_quad(s) ? 2 : (cpl == 8)][s.k - 1];
  const int64_t ranges = slots / L.n_slices > 1 ? slots / L.n_slices : 1;
  int64_t l = ceil_div(s.BT, 4 * ranges);  // tokens per wave
  l = (l + 3) / 4 * 4;
  if (l < 4) l = 4;
  L.tpb = (int)l;
  L.n_tiles = 0;
  L.n_ranges = (int)ceil_div(s.BT, 4 * l);
  int sl = 0;
  for (int d = 0; d < L.n_slices; ++d) {
    const int64_t c0 = (int64_t)d * span;
    const int64_t c1 = (s.D < c0 + span ? s.D : c0 + span) - 1;
    const int n = (int)(c1 / s.hd - c0 / s.hd + 1);
    if (n > sl) sl = n;
  }
  L.SL = s.stat ? 0 : sl;  // static filter: no du partials
  L.R = L.SL * s.k;
  return L;
}

bool bwd_headwise_supported(const Shape &s) {
  if (s.kind != DYNCONV_HEADWISE || s.k > 8 || hw_cpl(s) == 0) return false;
  // 32-bit byte offsets into x, dy, dx, u and the du partials, each tensor
  // below 2 GiB like those of the other tuned kernels
  const int64_t lim = ((int64_t)1 << 31) - 64;
  if (s.BT * s.D * 2 >= lim || s.BT * s.N * 4 >= lim) return false;
  const BwdLayout L = bwd_headwise_layout(s);
  return s.BT * L.R * 4 < ((int64_t)1 << 31) - 64;
}

int bwd_headwise(const Shape &s, const BwdLayout &L, const float *u, const void *w0, const void *x,
                 const void *dy, void *dx, float *gpart, float *dw0p, hipStream_t st) {
  bwdhw::Params P;
  P.s = s;
  P.x = (const bf16 *)x;
  P.dy = (const bf16 *)dy;
  P.dx = (bf16 *)dx;
  P.u = u;
  P.w0 = (const bf16 *)w0;
  P.gpart = gpart;
  P.dw0p = dw0p;
  P.L = L.tpb;
  P.SL = L.SL;
  P.R = L.R;
  const int cpl = hw_cpl(s);
  const int lanes_per_head = s.hd / cpl;
  int S = 0;
  if (s.stat)
    S = -2;
  else if (s.k > 4)
    S = 0;  // prefix sums for any head width
  else if (hw_quad(s))
    S = -1;
  else if (lanes_per_head == 1 || lanes_per_head == 2 || lanes_per_head == 4 || lanes_per_head == 8 ||
      lanes_per_head == 16)
    S = lanes_per_head;
  const dim3 grid((unsigned)L.n_slices, (unsigned)L.n_ranges), block(256);
  const bool tr = trace_begin(DYNCONV_K_BWD_CONV, st);
  int rc = 0;
#define HW(K_, C_, S_)                                                                \
  do {                                                                                \
    if (s.seqpos)                                                                     \
      hipLaunchKernelGGL((bwdhw::k_bwd_hw<K_, C_, S_, true>), grid, block, 0, st, P);  \
    else                                                                              \
      hipLaunchKernelGGL((bwdhw::k_bwd_hw<K_, C_, S_, false>), grid, block, 0, st, P); \
  } while (0)
#define HW_S8(K_)                      \
  switch (S) {                         \
    case 1: HW(K_, 8, 1); break;       \
    case 2: HW(K_, 8, 2); break;       \
    case 4: HW(K_, 8, 4); break;       \
    case 8: HW(K_, 8, 8); break;       \
    case 16: HW(K_, 8, 16); break;     \
    case -1: HW(K_, 8, -1); break;     \
    case -2: HW(K_, 8, -2); break;     \
    default: HW(K_, 8, 0); break;      \
  }
#define HW_K(K_)                         \
  if (cpl == 8) {                        \
    HW_S8(K_)                            \
  } else {                               \
    HW(K_, 4, 1); /* heads of 4 */       \
  }
#define HW_K8(K_)          \
  if (S == -2) {           \
    HW(K_, 4, -2);         \
  } else {                 \
    HW(K_, 4, 0);          \
  }
  switch (s.k) {
    case 1: HW_K(1) break;
    case 2: HW_K(2) break;
    case 3: HW_K(3) break;
    case 4: HW_K(4) break;
    case 5: HW_K8(5) break;
    case 6: HW_K8(6) break;
    case 7: HW_K8(7) break;
    case 8: HW_K8(8) break;
    default: rc = DYNCONV_E_LIMIT;
  }
#undef HW_K8
#undef HW_K
#undef HW_S8
#undef HW
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
