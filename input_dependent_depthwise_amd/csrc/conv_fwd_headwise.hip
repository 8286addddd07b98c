// conv_fwd_headwise.hip -- forward of the head-wise dynamic short convolution.
//
//   y[row, c] = x[row, c] + sum_{j<k, j<=pos} (u[row, head(c)*k + j] + w0[c, j]) * x[row-j, c]
//
// (gist.science Technical Summary of "Dynamic Short Convolutions Improve
// Transformers", Methodology -> Dynamic Short Convolutions: Mechanism; the
// head-wise tying of the Parameterization item; the residual of Placement.)
// u = h W comes from the generator projection kernel; the filter itself is
// formed in registers and never written to memory.
//
// Layout on the chip: a thread owns one 16-byte vector of channels (8 bf16 or
// 4 fp32) and walks a chunk of consecutive tokens, keeping the last k-1 rows
// of x in registers, so x is read once (plus a k-1 row halo per chunk) and y
// is written once, both as 16-byte loads/stores that are contiguous across
// the 64 lanes of a wave (1 KiB per wave instruction).  A block is 64 vectors
// x 4 token chunks; the grid covers (D / vector / 64) x (tokens / (4 * TC)).
// The HBM roofline bounds it: per token it moves 2*D*eb bytes of x and y plus
// the n_heads*k*4 bytes of u (a broadcast read, cached).
#include "kernels.h"
#include "bufio.h"

namespace dynconv {
namespace {

// bf16 path.  A lane owns 8 channels (16 bytes), a wave 512 consecutive
// channels, and walks a run of tokens.  x rows and the lane's u values are
// loaded PD = 4 tokens ahead into register rings; the k-1 previous rows are
// kept converted to fp32.  Every load and store is a raw buffer access issued
// on every path (masked ones fall outside the buffer), so the compiler's wait
// counts keep the ring in flight; a sequence start clears the history in a
// uniform branch that holds no memory access.  S2: a vector may straddle two
// heads (head width not a multiple of 8, at least 8).  VAR: packed documents,
// the positions come from the per-token table, four tokens per scalar load
// issued a step ahead (the table is padded, so reads just past the last
// token stay inside it; their values are never used).
//
// Folding (n_fold > 0): the last channel group holds at most 256 channels
// and the batch an even number of sequences.  Its waves then fold the batch:
// lanes 0..31 walk the first half of the rows, lanes 32..63 the same channels
// at the same positions of the second half (rows + BT/2, whole sequences
// further on), so no wave walks with half its lanes idle.  Runs 0 ..
// n_fold-1 have a wave for every group (the folded one last), the later runs
// one for each full group.
template <int K, bool S2, bool VAR>
__global__ void __launch_bounds__(256)
k_fwd_hw_ring(Shape s, const float *__restrict__ u, const bf16 *__restrict__ w0, const bf16 *__restrict__ x,
              bf16 *__restrict__ y, int n_vg, int n_runs, int tpw, int n_fold) {
  constexpr int PD = 4;
  constexpr int HS = K <= 4 ? 4 : 8;  // x history slots (and tokens per unrolled block)
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) run bounds and sequence position
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nv = n_fold > 0 ? n_vg - 1 : n_vg;  // waves of a run past the folded ones
  if (gw >= n_fold * n_vg + (n_runs - n_fold) * nv) return;  // whole waves only; no block-wide synchronisation
  int run, vg;
  if (gw < n_fold * n_vg) {
    run = gw / n_vg;
    vg = gw - run * n_vg;
  } else {
    const int g2 = gw - n_fold * n_vg;
    run = n_fold + g2 / nv;
    vg = g2 - (run - n_fold) * nv;
  }
  const int D = (int)s.D, BT = (int)s.BT, N = s.N, T = (int)s.T;  // BT*D, BT*N*2 < 2^30 (host-checked)
  const bool fold = n_fold > 0 && vg == n_vg - 1;
  const int cl = fold ? lane & 31 : lane;                  // the lane's place in its half
  const int hoff = fold ? (lane >> 5) * (BT >> 1) : 0;     // row offset of the lane's half
  const int BTw = fold ? BT >> 1 : BT;                     // rows of the walk
  const int c0 = vg * 512 + cl * 8;
  const bool act = c0 < D;
  const int t_lo = run * tpw, t_hi = min(BTw, t_lo + tpw);
  const int ea = act ? c0 / s.hd : 0;
  const int eb = S2 ? min(ea + 1, s.n_heads - 1) : ea;
  int second = 0;  // channels of the later head
  if (S2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) second |= ((c0 + i) / s.hd != ea) << i;
  }
  const auto rx = make_rsrc(x, (uint32_t)(BT * D * 2));
  const auto ry = make_rsrc(y, (uint32_t)(BT * D * 2));
  const auto ru = make_rsrc(u, (uint32_t)(BT * N * 4));

  float b[8][K];  // bias of the lane's channels: w0[c0 + i][j], contiguous 16 * K bytes
  {
    const auto rw = make_rsrc(w0, w0 ? (uint32_t)(D * K * 2) : 0u);  // no bias: zeros
    uint32_t wv[4 * K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const uint4 r = buf_load16(rw, act ? (uint32_t)(c0 * K * 2 + 16 * q) : kOutside);
      wv[4 * q] = r.x, wv[4 * q + 1] = r.y, wv[4 * q + 2] = r.z, wv[4 * q + 3] = r.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int e = i * K + j;
        b[i][j] = __uint_as_float((e & 1) ? (wv[e >> 1] & 0xffff0000u) : (wv[e >> 1] << 16));
      }
  }

  auto xoff = [&](int t) -> uint32_t {
    return (act && t >= 0 && t < t_hi) ? (uint32_t)((t + hoff) * D + c0) * 2u : kOutside;
  };
  auto uoff = [&](int t, int e, int j) -> uint32_t {
    return (act && t < t_hi) ? (uint32_t)((t + hoff) * N + e * K + j) * 4u : kOutside;
  };
  uint4 xr[PD];
  float ua[PD][K], ub[PD][K];
  auto load_tok = [&](int slot, int t) {
    xr[slot] = buf_load16(rx, xoff(t));
    if constexpr (K > 4) {  // taps 0..3 (and 4..7 for 8 taps) as 16-byte loads, the rest one by one
#pragma unroll
      for (int q = 0; q < K / 4; ++q) {
        const uint4 a = buf_load16(ru, uoff(t, ea, 4 * q));
        ua[slot][4 * q] = __uint_as_float(a.x), ua[slot][4 * q + 1] = __uint_as_float(a.y);
        ua[slot][4 * q + 2] = __uint_as_float(a.z), ua[slot][4 * q + 3] = __uint_as_float(a.w);
        if constexpr (S2) {
          const uint4 c = buf_load16(ru, uoff(t, eb, 4 * q));
          ub[slot][4 * q] = __uint_as_float(c.x), ub[slot][4 * q + 1] = __uint_as_float(c.y);
          ub[slot][4 * q + 2] = __uint_as_float(c.z), ub[slot][4 * q + 3] = __uint_as_float(c.w);
        }
      }
#pragma unroll
      for (int j = K / 4 * 4; j < K; ++j) {
        ua[slot][j] = buf_load_f32(ru, uoff(t, ea, j));
        if constexpr (S2) ub[slot][j] = buf_load_f32(ru, uoff(t, eb, j));
      }
    } else if constexpr (K == 4) {
      const uint4 a = buf_load16(ru, uoff(t, ea, 0));
      ua[slot][0] = __uint_as_float(a.x), ua[slot][1] = __uint_as_float(a.y);
      ua[slot][2] = __uint_as_float(a.z), ua[slot][3] = __uint_as_float(a.w);
      if constexpr (S2) {
        const uint4 c = buf_load16(ru, uoff(t, eb, 0));
        ub[slot][0] = __uint_as_float(c.x), ub[slot][1] = __uint_as_float(c.y);
        ub[slot][2] = __uint_as_float(c.z), ub[slot][3] = __uint_as_float(c.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        ua[slot][j] = buf_load_f32(ru, uoff(t, ea, j));
        if constexpr (S2) ub[slot][j] = buf_load_f32(ru, uoff(t, eb, j));
      }
    }
  };
  auto cvt = [&](const uint4 r, float (&f)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  };

  // history: xf[(i - j) mod HS] holds x[t - j] (fp32) at step i; rows of the
  // previous sequence read as zero
  float xf[HS][8];
  int pos = 0;
  uint64_t pq = 0;  // VAR: table entries of the next four tokens (t_lo and tpw are multiples of 4)
  const uint64_t *sp4 = reinterpret_cast<const uint64_t *>(s.seqpos);
  if constexpr (VAR) {
    pq = sp4[t_lo >> 2];
    pos = (int)(pq & 255u);
  } else {
    pos = t_lo % T;
  }
#pragma unroll
  for (int j = 1; j < HS; ++j) {
    const uint4 r = buf_load16(rx, (j < K && pos - j >= 0) ? xoff(t_lo - j) : kOutside);
    cvt(r, xf[(HS - j) & (HS - 1)]);
  }
  // the loop issues, per token, a store and then the loads PD tokens ahead;
  // the prologue keeps that order (its stores fall outside y and are
  // dropped) so the wait counts at the loop head are the steady-state ones
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    buf_store16(ry, kOutside + 16 * q, make_uint4(0, 0, 0, 0));  // distinct, so none is folded away
    load_tok(q, t_lo + q);
  }
  __builtin_amdgcn_sched_barrier(0);

  // (blocks of HS tokens; tokens past t_hi load nothing and store nothing)
  const int n_iter = (t_hi - t_lo + HS - 1) / HS * HS;
  for (int it = 0; it < n_iter; it += HS) {
    uint64_t pc[HS / 4];
#pragma unroll
    for (int q = 0; q < HS / 4; ++q) {
      if constexpr (VAR) {
        pc[q] = q == 0 ? pq : sp4[((t_lo + it) >> 2) + q];
      } else {
        pc[q] = 0;
      }
    }
    if constexpr (VAR) pq = sp4[(t_lo + it + HS) >> 2];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      const int t = t_lo + it + i;
      cvt(xr[i & (PD - 1)], xf[i]);
      if constexpr (VAR) pos = (int)((pc[i >> 2] >> (16 * (i & 3))) & 255u);
      if (pos == 0) {  // a new sequence starts: no history
#pragma unroll
        for (int j = 1; j < HS; ++j)
#pragma unroll
          for (int c = 0; c < 8; ++c) xf[(i + HS - j) & (HS - 1)][c] = 0.f;
      }
      float out[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float a = xf[i][c];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const int sl = i & (PD - 1);
          const float uj = S2 ? (((second >> c) & 1) ? ub[sl][j] : ua[sl][j]) : ua[sl][j];
          a = fmaf(uj + b[c][j], xf[(i + HS - j) & (HS - 1)][c], a);
        }
        out[c] = a;
      }
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)out[2 * q]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)out[2 * q + 1]) << 16);
      buf_store16(ry, xoff(t), make_uint4(w[0], w[1], w[2], w[3]));
      load_tok(i & (PD - 1), t + PD);
      if constexpr (!VAR) pos = pos + 1 == T ? 0 : pos + 1;
    }
  }
}

// tokens per thread (chunk): 32, or as few as 4 when that is what it takes
// to give the chip about 64K threads (short inputs are a latency chain per
// thread otherwise)
constexpr int kFwdChunk = 32;

template <typename T, int KP>
__global__ void __launch_bounds__(256)
k_fwd_headwise(Shape s, const float *__restrict__ u, const T *__restrict__ w0,
               const T *__restrict__ x, T *__restrict__ y, int chunk) {
  constexpr int V = Vec<T>::N;
  const int nvec = (int)(s.D / V);
  const int v = blockIdx.x * 64 + threadIdx.x;
  if (v >= nvec) return;
  const int64_t row0 = ((int64_t)blockIdx.y * 4 + threadIdx.y) * chunk;
  if (row0 >= s.BT) return;
  const int64_t row1 = row0 + chunk < s.BT ? row0 + chunk : s.BT;
  const int c0 = v * V;
  const int k = s.k;

  // heads of this vector's channels: the first (ea) and, when the vector
  // straddles a head boundary, the next one; `second` flags channels of the
  // later head.  When heads are narrower than a vector, fall back to a
  // per-channel lookup.
  const int ea = c0 / s.hd;
  const bool two_heads_max = s.hd >= V;
  int second = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) second |= ((c0 + i) / s.hd != ea) << i;

  float b[V][KP];
#pragma unroll
  for (int i = 0; i < V; ++i)
#pragma unroll
    for (int j = 0; j < KP; ++j) b[i][j] = (w0 && j < k) ? to_f32(w0[(int64_t)(c0 + i) * k + j]) : 0.f;

  // window: xw[j] = x[row - j]; rows before the sequence start are zero
  float xw[KP][V];
  int64_t pos = seq_pos(s, row0);
#pragma unroll
  for (int j = 1; j < KP; ++j) {
    if (j < k && pos - j >= 0) {
      load_vec(x + (row0 - j) * s.D + c0, xw[j]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) xw[j][i] = 0.f;
    }
  }

  for (int64_t row = row0; row < row1; ++row, ++pos) {
    if (s.seqpos) pos = seq_pos(s, row);  // packed documents: from the table
    if (s.seqpos ? (pos == 0 && row > row0) : pos == s.T) {  // a new sequence starts: clear the history
      pos = 0;
#pragma unroll
      for (int j = 1; j < KP; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) xw[j][i] = 0.f;
    }
    load_vec(x + row * s.D + c0, xw[0]);
    const float *ur = u + row * s.N;
    float ua[KP], ub[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      ua[j] = j < k ? ur[ea * k + j] : 0.f;
      ub[j] = (j < k && second) ? ur[(ea + 1) * k + j] : 0.f;
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float a = xw[0][i];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        float uj;
        if (two_heads_max) {
          uj = ((second >> i) & 1) ? ub[j] : ua[j];
        } else {
          uj = j < k ? ur[((c0 + i) / s.hd) * k + j] : 0.f;
        }
        a = fmaf(uj + b[i][j], xw[j][i], a);
      }
      acc[i] = a;
    }
    store_vec(y + row * s.D + c0, acc);
#pragma unroll
    for (int j = KP - 1; j > 0; --j)
#pragma unroll
      for (int i = 0; i < V; ++i) xw[j][i] = xw[j - 1][i];
  }
}

template <typename T, int KP>
void launch(const Shape &s, const float *u, const void *w0, const void *x, void *y, hipStream_t st) {
  constexpr int V = Vec<T>::N;
  const int64_t nvec = s.D / V;
  int chunk = (int)std::min<int64_t>(kFwdChunk, ceil_div(s.BT * nvec, (int64_t)1 << 16));
  chunk = std::max(4, chunk);
  dim3 grid((unsigned)ceil_div(nvec, 64), (unsigned)ceil_div(s.BT, 4 * chunk));
  hipLaunchKernelGGL((k_fwd_headwise<T, KP>), grid, dim3(64, 4), 0, st, s, u, (const T *)w0,
                     (const T *)x, (T *)y, chunk);
}

}  // namespace

// the ring kernel: bf16, k <= 4, at most two heads per 8-channel vector,
// 32-bit offsets
static bool ring_ok(const Shape &s) {
  const int64_t lim = ((int64_t)1 << 30);
  return s.hd >= 8 && s.D % 8 == 0 && s.BT * s.D < lim && s.BT * s.N * 2 < lim;
}

template <int K, bool S2>
static void launch_ring(const Shape &s, const float *u, const void *w0, const void *x, void *y, hipStream_t st) {
  const int n_vg = (int)ceil_div(s.D, 512);
  // the last group folds the batch when it holds at most 256 channels and
  // the rows split into two halves of whole sequences
  const bool fold = !s.packed && s.B % 2 == 0 && s.D - (int64_t)(n_vg - 1) * 512 <= 256;
  // about three waves per SIMD (two for 5..8 taps, which hold that many),
  // runs of a multiple of 4 tokens
  int tpw = (int)ceil_div(s.BT * (2 * n_vg - (fold ? 1 : 0)), 2 * (K <= 4 ? 3 : 2) * 4 * 256);
  tpw = std::max(16, (tpw + 3) & ~3);
  const int n_runs = (int)ceil_div(s.BT, tpw);
  const int n_fold = fold ? (int)ceil_div(s.BT / 2, tpw) : 0;
  const int waves = n_fold * n_vg + (n_runs - n_fold) * (fold ? n_vg - 1 : n_vg);
  const dim3 grid((unsigned)ceil_div(waves, 4)), block(256);
  if (s.seqpos)
    hipLaunchKernelGGL((k_fwd_hw_ring<K, S2, true>), grid, block, 0, st, s, u, (const bf16 *)w0, (const bf16 *)x,
                       (bf16 *)y, n_vg, n_runs, tpw, n_fold);
  else
    hipLaunchKernelGGL((k_fwd_hw_ring<K, S2, false>), grid, block, 0, st, s, u, (const bf16 *)w0, (const bf16 *)x,
                       (bf16 *)y, n_vg, n_runs, tpw, n_fold);
}

template <typename T>
int fwd_headwise(const Shape &s, const float *u, const void *w0, const void *x, void *y,
                 hipStream_t st) {
  const bool tr = trace_begin(DYNCONV_K_FWD_CONV, st);
  if (std::is_same<T, bf16>::value && ring_ok(s)) {
    const bool s2 = s.hd % 8 != 0;
    switch (s.k * 2 + (s2 ? 1 : 0)) {
      case 2: launch_ring<1, false>(s, u, w0, x, y, st); break;
      case 3: launch_ring<1, true>(s, u, w0, x, y, st); break;
      case 4: launch_ring<2, false>(s, u, w0, x, y, st); break;
      case 5: launch_ring<2, true>(s, u, w0, x, y, st); break;
      case 6: launch_ring<3, false>(s, u, w0, x, y, st); break;
      case 7: launch_ring<3, true>(s, u, w0, x, y, st); break;
      case 8: launch_ring<4, false>(s, u, w0, x, y, st); break;
      case 9: launch_ring<4, true>(s, u, w0, x, y, st); break;
      case 10: launch_ring<5, false>(s, u, w0, x, y, st); break;
      case 11: launch_ring<5, true>(s, u, w0, x, y, st); break;
      case 12: launch_ring<6, false>(s, u, w0, x, y, st); break;
      case 13: launch_ring<6, true>(s, u, w0, x, y, st); break;
      case 14: launch_ring<7, false>(s, u, w0, x, y, st); break;
      case 15: launch_ring<7, true>(s, u, w0, x, y, st); break;
      case 16: launch_ring<8, false>(s, u, w0, x, y, st); break;
      default: launch_ring<8, true>(s, u, w0, x, y, st); break;
    }
  } else if (s.k <= 4)
    launch<T, 4>(s, u, w0, x, y, st);
  else
    launch<T, 8>(s, u, w0, x, y, st);
  trace_end(tr, st);
  return 0;
}

bool fwd_headwise_ring_ok(const Shape &s) { return ring_ok(s); }

template int fwd_headwise<float>(const Shape &, const float *, const void *, const void *, void *,
                                 hipStream_t);
template int fwd_headwise<bf16>(const Shape &, const float *, const void *, const void *, void *,
                                hipStream_t);

}  // namespace dynconv
