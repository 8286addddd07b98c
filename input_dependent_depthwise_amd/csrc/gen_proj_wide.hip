// gen_proj_wide.hip -- bf16 matrix-core projections of the hidden state with
// the weights read in place:
//
//   the generator projection for wide generator weights
//     out[t, n] = sum_i h[t, i] * M[i, n]     (u = h W head-wise, z = h A low-rank)
//   and the producing projection fused with it
//     [x | gen][t, :] = h[t, :] . [Wp | M]    x bf16 [BT, D], gen fp32 [BT, N]
//
// The filter is a learned linear map of the current hidden state
// (gist.science Technical Summary of "Dynamic Short Convolutions Improve
// Transformers", Methodology -> Dynamic Short Convolutions, Parameterization);
// the generator projection is its first, dense factor (rows = tokens, K =
// d_model, N = n_heads*k or rank: 64 to 256 columns here, e.g. 96 and 256 for
// the 2B-QKV and Mamba-2 shapes).  The layer itself sits after a projection
// of that same hidden state (Placement: on the query, key and value
// projections, or after any linear layer), so the fused form reads h once
// for both the layer's input x and the filter generator.
//
// Block: 4 waves (one per SIMD) = RG row groups of 32 rows x KS parts of K,
// over one slab of 32 NT columns (the grid walks row blocks x slabs, slabs
// fastest, so the slabs of a row block share its rows of h in L2); 256-column
// slabs take two such groups of 4 waves, each on half the columns.  Per step
// of 64 k:
//   * each wave multiplies its 32 rows by every 32-column tile (of its group) of the staged
//     weight slice on v_mfma_f32_32x32x16_bf16, accumulators resident.  A
//     fragments are four 16-byte loads per lane straight from h (the 128-byte
//     run of each row), issued three steps ahead into a ring of three
//     register sets, so the loads of the next two steps stay in flight across
//     the barriers;
//   * the weight slice (64 rows of the slab's columns, contiguous in memory)
//     is staged row-major in LDS, double-buffered, one barrier per step; its
//     loads are issued a step ahead, before that step's A loads, so waiting
//     for them never waits for A.  A B fragment is two ds_read_b64_tr_b16
//     (four k of one column each); the reads of the next k-substep are issued
//     before the current substep's MFMAs.  Rows are padded by 64 bytes so that
//     the four rows a 32-lane pass reads fall on disjoint quarters of the banks.
// The K parts meet in LDS at the end in a fixed order.
#include "kernels.h"
#include "bufio.h"
#include "mfma.h"

namespace dynconv {
namespace {

constexpr int kKT = 64;  // k per step

template <int NT, int RG, int KS, int CG>
struct WideCfg {
  static constexpr int NTH = 64 * RG * KS * CG;  // threads per block
  static constexpr int NTW = NT / CG;            // column tiles per wave
  static constexpr int BM = RG * 32;             // rows per block
  static constexpr int NP = NT * 32;             // columns per slab (zeros past the weights)
  static constexpr int LDW = NP + 32;            // LDS row stride (bf16)
  static constexpr int SLICE = kKT * LDW;        // bf16 per staged slice
  static constexpr int STAGE = KS * SLICE;       // bf16 per stage (KS slices)
  static constexpr int CPR = NP / 8;             // 16-byte chunks per staged row
  static constexpr int CH = KS * kKT * CPR;      // chunks per stage
  static constexpr int CPT = (CH + NTH - 1) / NTH;  // chunks per thread
  static constexpr size_t LDS = (size_t)2 * STAGE * 2;
  static_assert(RG * KS == 4, "4 waves per column group");
  static_assert(NT % CG == 0, "whole column tiles per wave");
  // the K parts' sums pass through the (then free) stages at the end
  static_assert(KS == 1 || LDS >= (size_t)(KS - 1) * RG * NT * 16 * 64 * 4, "reduction buffer");
};

// The weight columns: [0, N0) from W0 (row stride N0), [N0, N0 + N1) from W1
// (row stride N1); the outputs: columns below N0 to xb (bf16, row stride N0)
// when it is given, every other column to out (fp32, row stride N - split).
struct Cols {
  const bf16 *W0, *W1;
  int N0, N1;     // N0 and N1 are multiples of 8 (a 16-byte chunk is one source's)
  bf16 *xb;       // fused: the producing projection's output x; else NULL
  float *out;     // the generator values
};

template <int NT, int RG, int KS, int CG, bool FUSED>
__global__ void __launch_bounds__(64 * RG * KS * CG, 1)
k_gen_proj_wide(const bf16 *__restrict__ h, Cols cols, int64_t M, int K, int n_slabs) {
  using C = WideCfg<NT, RG, KS, CG>;
  constexpr int NTW = C::NTW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  bf16 *bs = reinterpret_cast<bf16 *>(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RG, ks = (wave / RG) % KS, cg = wave / (RG * KS);
  const int slab = (int)(blockIdx.x % n_slabs);
  const int64_t row0 = (int64_t)(blockIdx.x / n_slabs) * C::BM;
  const int col0 = slab * C::NP;
  const int N = cols.N0 + cols.N1;
  const int nrows = (int)min<int64_t>(C::BM, M - row0);
  const auto rh = make_rsrc(h + row0 * K, (uint32_t)((int64_t)nrows * K * 2));
  const auto rw0 = make_rsrc(cols.W0, (uint32_t)((int64_t)K * cols.N0 * 2));
  const auto rw1 = make_rsrc(cols.W1, FUSED ? (uint32_t)((int64_t)K * cols.N1 * 2) : 0u);
  const int S = (K + kKT - 1) / kKT;  // steps over all of K
  const int SH = (S + KS - 1) / KS;   // steps per K part (the last part may run past K: zeros)

  uint4 breg[C::CPT];
  auto load_b = [&](int st) {
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int e = tid + c * C::NTH;
      const int sl = e / (kKT * C::CPR), e2 = e - sl * (kKT * C::CPR);
      const int r = e2 / C::CPR, gc = col0 + (e2 - r * C::CPR) * 8;
      const int k = (sl * SH + st) * kKT + r;
      const bool live = (C::CH % C::NTH == 0 || e < C::CH) && k < K;
      // a chunk lies wholly in one source, or past both (zeros); the other
      // source's load falls outside its buffer and reads zeros, so no lane
      // chooses between resources
      breg[c] = buf_load16(rw0, live && gc < cols.N0 ? (uint32_t)(k * cols.N0 + gc) * 2u : kOutside);
      if constexpr (FUSED) {
        const uint4 b1 = buf_load16(
            rw1, live && gc >= cols.N0 && gc < N ? (uint32_t)(k * cols.N1 + gc - cols.N0) * 2u : kOutside);
        breg[c] = make_uint4(breg[c].x | b1.x, breg[c].y | b1.y, breg[c].z | b1.z, breg[c].w | b1.w);
      }
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int e = tid + c * C::NTH;
      if (C::CH % C::NTH == 0 || e < C::CH) {
        const int sl = e / (kKT * C::CPR), e2 = e - sl * (kKT * C::CPR);
        const int r = e2 / C::CPR, cc = (e2 - r * C::CPR) * 8;
        *reinterpret_cast<uint4 *>(&bs[buf * C::STAGE + sl * C::SLICE + r * C::LDW + cc]) = breg[c];
      }
    }
  };
  // A fragment q of a step: row (lane % 32) of the wave's rows, k = 16 q + 8 (lane / 32) .. +7
  const int arow = rg * 32 + (lane & 31);
  auto load_a = [&](bf16x8(&a)[4], int st) {
    const int kb = (ks * SH + st) * kKT + 8 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = kb + 16 * q;  // K is a multiple of 8: a fragment is wholly inside or outside
      a[q] = as_bf16x8(buf_load16(rh, k < K ? (uint32_t)(arow * K + k) * 2u : kOutside));
    }
  };
  // B fragment of k-substep q, column tile n: the lanes of 16-group gi read
  // rows 8 (gi / 2) + 4 p + (lr / 4) (p = 0, 1), columns 32 n + 16 (gi % 2) +
  // 4 (lr % 4) .. +3; lane l then holds B[8 (l / 32) + i][32 n + l % 32]
  const int lr = lane & 15, gi = lane >> 4;
  const int boff = (8 * (gi >> 1) + (lr >> 2)) * C::LDW + 16 * (gi & 1) + 4 * (lr & 3) + 32 * NTW * cg;
  auto bfrags = [&](bf16x8(&b)[NTW], int buf, int q) {
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const unsigned char *p = reinterpret_cast<const unsigned char *>(
          &bs[buf * C::STAGE + ks * C::SLICE + 16 * q * C::LDW + 32 * n + boff]);
      const uint2 lo = read_tr16(p);
      const uint2 hi = read_tr16(p + 4 * C::LDW * 2);
      b[n] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  };

  f32x16 acc[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;

  // issue order: A0 B0 A1 | B1 A2 | B2 A3 | ...: the B loads of a step are
  // older than the A loads of the step after it
  bf16x8 a0[4], a1[4], a2[4];
  load_a(a0, 0);
  load_b(0);
  load_a(a1, 1);
  store_b(0);
  load_b(1);
  load_a(a2, 2);
  __syncthreads();
  // Step st: multiply (A of st, stage st % 2), stage B of st + 1, issue the
  // B loads of st + 2 and the A loads of st + 3 (into the set just used),
  // meet at the barrier.
  auto step = [&](int st, bf16x8(&a)[4], int buf) {
    bf16x8 bc[NTW], bn[NTW];
    bfrags(bc, buf, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) bfrags(bn, buf, q + 1);
#pragma unroll
      for (int n = 0; n < NTW; ++n) acc[n] = mfma32(a[q], bc[n], acc[n]);
      if (q < 3) {
#pragma unroll
        for (int n = 0; n < NTW; ++n) bc[n] = bn[n];
      }
    }
    // the other stage was last read in the previous step, before its barrier
    store_b(buf ^ 1);
    load_b(st + 2);
    load_a(a, st + 3);
    __syncthreads();
  };
  int st = 0;
  for (; st + 6 <= SH; st += 6) {
    step(st, a0, 0);
    step(st + 1, a1, 1);
    step(st + 2, a2, 0);
    step(st + 3, a0, 1);
    step(st + 4, a1, 0);
    step(st + 5, a2, 1);
  }
  // the tail (fewer than six steps), same ring order
  if (st < SH) step(st, a0, 0);
  if (st + 1 < SH) step(st + 1, a1, 1);
  if (st + 2 < SH) step(st + 2, a2, 0);
  if (st + 3 < SH) step(st + 3, a0, 1);
  if (st + 4 < SH) step(st + 4, a1, 0);

  if constexpr (KS > 1) {
    static_assert(CG == 1, "K parts with one column group");
    // K parts 1 .. KS-1 hand their sums to part 0, added in part order
    float *red = reinterpret_cast<float *>(lds_raw);
    auto slot = [&](int part, int n, int i) { return ((((part - 1) * RG + rg) * NT + n) * 16 + i) * 64 + lane; };
    if (ks > 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[slot(ks, n, i)] = acc[n][i];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int p = 1; p < KS; ++p)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[n][i] += red[slot(p, n, i)];
  }

  // D: lane holds D[8 b + 4 (lane / 32) + r][lane % 32] in element 4 b + r
  const int split = FUSED ? cols.N0 : 0;
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    const int col = col0 + 32 * (NTW * cg + n) + (lane & 31);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rg * 32 + 8 * b + 4 * (lane >> 5) + r;
        if (col >= N || row >= nrows) continue;
        const float v = acc[n][4 * b + r];
        if (FUSED && col < split)
          cols.xb[(row0 + row) * cols.N0 + col] = (bf16)v;  // round to nearest even
        else
          cols.out[(row0 + row) * (N - split) + col - split] = v;
      }
  }
}

template <int NT, int RG, int KS, int CG, bool FUSED>
void launch(const bf16 *h, const Cols &cols, int64_t M, int K, hipStream_t st) {
  using C = WideCfg<NT, RG, KS, CG>;
  const size_t lds = C::LDS;
  const int n_slabs = (int)ceil_div(cols.N0 + cols.N1, C::NP);
  hipLaunchKernelGGL((k_gen_proj_wide<NT, RG, KS, CG, FUSED>), dim3((unsigned)(ceil_div(M, C::BM) * n_slabs)),
                     dim3(C::NTH), lds, st, h, cols, M, K, n_slabs);
}

// One block of 4 waves per CU: 128-row blocks when the blocks number at least
// 256, else 64-row blocks with K in two parts.  The fused form always takes
// 128-row blocks: its slabs are many (the producing projection's D columns),
// and its two-part variant would spill registers.
template <int NT, bool FUSED>
void launch_nt(const bf16 *h, const Cols &cols, int64_t M, int K, hipStream_t st) {
  const int64_t slabs = ceil_div(cols.N0 + cols.N1, NT * 32);
  // 256-column slabs: two column groups of 4 waves, two waves per SIMD (the
  // second hides the first's A loads; 12 % faster for the fused form, 5 % for
  // 256 generator columns, than one group)
  constexpr int CG = NT == 8 ? 2 : 1;
  if constexpr (FUSED) {
    launch<NT, 4, 1, CG, true>(h, cols, M, K, st);
  } else {
    if (ceil_div(M, 128) * slabs >= 256)
      launch<NT, 4, 1, CG, false>(h, cols, M, K, st);
    else
      launch<NT, 2, 2, 1, false>(h, cols, M, K, st);
  }
}

}  // namespace

bool gen_proj_wide_ok(const Shape &s) {
  // 32-bit byte offsets into h (per block) and the weight
  return s.N % 8 == 0 && s.N >= 64 && s.N <= 256 && s.d % 8 == 0 && s.d * s.N * 2 < ((int64_t)1 << 31);
}

int gen_proj_wide(const Shape &s, const void *h, const void *M, float *out, hipStream_t st) {
  const bool tr = trace_begin(DYNCONV_K_GEN_PROJ, st);
  const bf16 *hh = (const bf16 *)h;
  const Cols cols{(const bf16 *)M, nullptr, s.N, 0, nullptr, out};
  const int K = (int)s.d;
  switch (ceil_div(s.N, 32)) {
    case 2: launch_nt<2, false>(hh, cols, s.BT, K, st); break;
    case 3: launch_nt<3, false>(hh, cols, s.BT, K, st); break;
    case 4: launch_nt<4, false>(hh, cols, s.BT, K, st); break;
    case 5: launch_nt<5, false>(hh, cols, s.BT, K, st); break;
    case 6: launch_nt<6, false>(hh, cols, s.BT, K, st); break;
    case 7: launch_nt<7, false>(hh, cols, s.BT, K, st); break;
    default: launch_nt<8, false>(hh, cols, s.BT, K, st); break;
  }
  trace_end(tr, st);
  return 0;
}

bool proj_fused_ok(const Shape &s) {
  // chunk-aligned sources; 32-bit byte offsets into h, both weights and x
  const int64_t lim = ((int64_t)1 << 31) - 64;
  return s.D % 8 == 0 && s.N % 8 == 0 && s.d % 8 == 0 && s.d * s.D * 2 < lim && s.d * s.N * 2 < lim &&
         s.BT * s.D * 2 < lim && s.BT * s.d * 2 < lim;
}

int proj_fused(const Shape &s, const void *h, const void *Wp, const void *M, void *x, float *gen, hipStream_t st) {
  const bool tr = trace_begin(DYNCONV_K_GEN_PROJ, st);
  const Cols cols{(const bf16 *)Wp, (const bf16 *)M, (int)s.D, s.N, (bf16 *)x, gen};
  launch_nt<8, true>((const bf16 *)h, cols, s.BT, (int)s.d, st);
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
