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
//     transpose-reductions (heads of 1..16 lanes, aligned) or through LDS
//     (any other head width), and written as one fp32 partial per span;
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

template <int K>
__device__ __forceinline__ void bload_u(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float (&u)[4]) {
  if constexpr (K == 4) {
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
// any head width (LDS reduction).  VAR: packed documents (positions from the
// per-token table).
template <int K, int CPL, int S, bool VAR>
__global__ void __launch_bounds__(256, 2)
k_bwd_hw(Params P) {
  constexpr int NP = CPL / 2;        // bf16 pairs per lane
  constexpr int SPAN = 64 * CPL;
  constexpr int PD = 4;              // tokens loaded ahead
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
  const int e_lo = (int)(span_c0 / s.hd);
  const int BT = (int)s.BT;  // the host keeps every tensor below 2 GiB (32-bit byte offsets)
  const int T = s.T;

  // per-lane bias: CPL*K contiguous bf16 at w0[cc*K], read as dwords with
  // unconditional buffer loads (no bias: an empty buffer, every load reads 0)
  float w0r[CPL][4];
  {
    const auto rw = rsrc(P.w0, P.w0 ? (uint32_t)(Dc * K * 2) : 0u);
    constexpr int NW = CPL * K / 2;
    uint32_t wv[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q) wv[q] = __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(cc * K * 2 + 4 * q), 0, 0);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
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
  const uint32_t voff_x = (uint32_t)cc * 2u, voff_u = (uint32_t)e * K * 4u;
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

  if (t_a < BT) {
    // token rings: x in 8 slots (slot = (t - t_a) mod 8) holding tokens
    // t-3 .. t+PD (the k-tap history plus the loads in flight), dy and u in 4
    // (slot = (t - t_a) mod 4) holding tokens t .. t+PD
    uint32_t xr[8][NP], dyr[4][NP];
    float ur[4][4];
    float acc[4][CPL];  // dx accumulators (slot = (s - t_a) mod 4)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[a][i] = 0.f;

    int pos = VAR ? 0 : (int)(t_a % T);  // position in its sequence of the next token to process
    // VAR (packed documents): positions from the per-token table, the eight of
    // a block in two scalar loads issued a block ahead (t_a and the run length
    // are multiples of 4; the table is padded past its last token)
    const uint64_t *sp4 = reinterpret_cast<const uint64_t *>(s.seqpos);
    uint64_t pn[2] = {0, 0};
    if constexpr (VAR) pn[0] = sp4[t_a >> 2], pn[1] = sp4[(t_a >> 2) + 1];
    // Loads are unconditional: row offsets are clamped to the batch, and what
    // they bring past the run is never consumed (tokens past t_end are not
    // processed, x past t_b feeds no product, and every token past the batch
    // end starts a new "sequence" for the position tests).
    auto row = [&](int t) { return (uint32_t)(t < BT ? (t > 0 ? t : 0) : BT - 1); };
    // x history before t_a (the taps that reach before the sequence start are
    // skipped by the position tests, not zeroed)
#pragma unroll
    for (int j = 3; j >= 1; --j) {
      if (j < K) bload<CPL>(rx, voff_x, row(t_a - j) * row_x, xr[8 - j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // token t into x slot xs, dy and u slot xs mod 4
    auto load_tok = [&](int t, int xs) {
      const uint32_t r = row(t);
      bload<CPL>(rx, voff_x, r * row_x, xr[xs]);
      bload<CPL>(rdy, voff_x, r * row_x, dyr[xs & 3]);
      bload_u<K>(ru, voff_u, r * row_u, ur[xs & 3]);
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
    uint32_t held[NP + 4];  // dx of this token, du of the previous one
#pragma unroll
    for (int p = 0; p < NP + 4; ++p) held[p] = 0u;

    // one block of 8 tokens from tg.  The tests on t and pos are wave-uniform
    // (scalar branches); keeping them in every block rather than compiling a
    // second, test-free copy keeps the register allocation of the rings simple.
    auto block = [&](int tg) {
      const uint64_t pc[2] = {pn[0], pn[1]};
      if constexpr (VAR) pn[0] = sp4[(tg >> 2) + 2], pn[1] = sp4[(tg >> 2) + 3];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = tg + i;
        float vals[4] = {0.f, 0.f, 0.f, 0.f};
        // a token past the batch end starts a new "sequence" (its loads were clamped)
        if constexpr (VAR) pos = t < BT ? (int)((pc[i >> 2] >> (16 * (i & 3))) & 255u) : 0;
        if (t < t_end) {
          const bool main = t < t_b;
          // (lanes past D in a partial last span compute on the clamped
          // channels; nothing of theirs is stored or summed)
          uint32_t dw[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) dw[p] = dyr[i & 3][p];
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
              const int xs = (i - j) & 7;
#pragma unroll
              for (int p = 0; p < NP; ++p) vals[j] = dot2(xr[xs][p], dw[p], vals[j]);
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
            for (int c = 0; c < CPL; ++c) acc[i & 3][c] = fmaf(ur[i & 3][0] + w0r[c][0], dyf[c], dyf[c]);
          }
#pragma unroll
          for (int j = 1; j < K; ++j) {
            if (pos >= j) {
#pragma unroll
              for (int c = 0; c < CPL; ++c)
                acc[(i - j) & 3][c] = fmaf(ur[i & 3][j] + w0r[c][j], dyf[c], acc[(i - j) & 3][c]);
            }
          }
          // token t-k+1 has all its terms
          const int so = t - (K - 1);
          if (so >= t_a && so < t_b) {
            const float *a = acc[(i - (K - 1)) & 3];
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
        load_tok(t + PD, (i + PD) & 7);
        // the previous token's stores have been followed by these loads; their
        // registers may be reused from here on
#pragma unroll
        for (int p = 0; p < NP + 4; ++p) asm volatile("" ::"v"(held[p]));
        // du of this token: sum over the lanes of each head
        if constexpr (S > 0) {
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
        } else {
          // any head width: head sums as differences of the wave's prefix sums
          if (t < t_b) {
            float hs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
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
            for (int j = 0; j < 4; ++j) held[NP + j] = __float_as_uint(hs[j]);
          }
        }
        // keep each token's work in its own scheduling region: interleaving
        // tokens only raises register pressure (the loads are already ahead)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int tg = t_a; tg < t_end; tg += 8) block(tg);
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
static int hw_cpl(const Shape &s) { return (s.hd % 8 == 0) ? 8 : (s.hd % 4 == 0 ? 4 : 0); }

BwdLayout bwd_headwise_layout(const Shape &s) {
  BwdLayout L = {};
  const int cpl = hw_cpl(s);
  const int span = 64 * cpl;
  L.Dt = span;
  L.n_slices = (int)ceil_div(s.D, span);
  // tokens per wave: about one round of resident waves over 256 CUs (the
  // 8-channel variants with k >= 3 hold 2 waves per SIMD, the others 4)
  const int waves_per_cu = (cpl == 8 && s.k >= 3) ? 8 : 16;
  int64_t l = ceil_div(s.BT * L.n_slices, 256 * waves_per_cu);
  l = (l + 3) / 4 * 4;
  if (l < 4) l = 4;
  L.tpb = (int)l;  // tokens per wave
  L.n_tiles = 0;
  L.n_ranges = (int)ceil_div(s.BT, 4 * l);
  int sl = 0;
  for (int d = 0; d < L.n_slices; ++d) {
    const int64_t c0 = (int64_t)d * span;
    const int64_t c1 = (s.D < c0 + span ? s.D : c0 + span) - 1;
    const int n = (int)(c1 / s.hd - c0 / s.hd + 1);
    if (n > sl) sl = n;
  }
  L.SL = sl;
  L.R = sl * s.k;
  return L;
}

bool bwd_headwise_supported(const Shape &s) {
  if (s.kind != DYNCONV_HEADWISE || s.k > 4 || hw_cpl(s) == 0) return false;
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
  if (lanes_per_head == 1 || lanes_per_head == 2 || lanes_per_head == 4 || lanes_per_head == 8 ||
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
    default: HW(K_, 8, 0); break;      \
  }
#define HW_K(K_)                         \
  if (cpl == 8) {                        \
    HW_S8(K_)                            \
  } else if (S == 1) {                   \
    HW(K_, 4, 1);                        \
  } else {                               \
    HW(K_, 4, 0);                        \
  }
  switch (s.k) {
    case 1: HW_K(1) break;
    case 2: HW_K(2) break;
    case 3: HW_K(3) break;
    case 4: HW_K(4) break;
    default: rc = DYNCONV_E_LIMIT;
  }
#undef HW_K
#undef HW_S8
#undef HW
  trace_end(tr, st);
  return rc;
}

}  // namespace dynconv
