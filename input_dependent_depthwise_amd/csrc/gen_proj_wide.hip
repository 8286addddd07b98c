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
// Two kernels:
//   * k_gen_proj_wide, for 64..192 columns.  Block: 4 waves (one per SIMD) =
//     RG row groups of 32 rows x KS parts of K, over one slab of 32 NT columns.
//     Per step of 64 k each wave multiplies its 32 rows by every 32-column tile
//     of the staged weight slice on v_mfma_f32_32x32x16_bf16, accumulators
//     resident.  A fragments are four 16-byte loads per lane straight from h
//     (the 128-byte run of each row), issued three steps ahead into a ring of
//     three register sets; the weight slice (64 rows of the slab's columns) is
//     staged row-major in LDS, double-buffered, one barrier per step, its loads
//     issued a step ahead, before that step's A loads.  A B fragment is two
//     ds_read_b64_tr_b16 (four k of one column each); the reads of the next
//     k-substep are issued before the current substep's MFMAs.  Rows are padded
//     by 64 bytes so that the four rows a 32-lane pass reads fall on disjoint
//     quarters of the banks.
//   * k_proj_tile, for 193..256 columns and for the fused form (below).
// (k_gen_proj_wide: the K parts meet in LDS at the end in a fixed order.)
#include "kernels.h"
#include "bufio.h"
#include "mfma.h"

namespace dynconv {
namespace {

constexpr int kKT = 64;  // k per step

template <int NT, int RG, int KS>
struct WideCfg {
  static constexpr int NTH = 64 * RG * KS;       // threads per block
  static constexpr int NTW = NT;                 // column tiles per wave
  static constexpr int BM = RG * 32;             // rows per block
  static constexpr int NP = NT * 32;             // columns per slab (zeros past the weights)
  static constexpr int LDW = NP + 32;            // LDS row stride (bf16)
  static constexpr int SLICE = kKT * LDW;        // bf16 per staged slice
  static constexpr int STAGE = KS * SLICE;       // bf16 per stage (KS slices)
  static constexpr int CPR = NP / 8;             // 16-byte chunks per staged row
  static constexpr int CH = KS * kKT * CPR;      // chunks per stage
  static constexpr int CPT = (CH + NTH - 1) / NTH;  // chunks per thread
  static constexpr size_t LDS = (size_t)2 * STAGE * 2;
  static_assert(RG * KS == 4, "4 waves per block");
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

template <int NT, int RG, int KS>
__global__ void __launch_bounds__(64 * RG * KS, 1)
k_gen_proj_wide(const bf16 *__restrict__ h, Cols cols, int64_t M, int K, int n_slabs) {
  using C = WideCfg<NT, RG, KS>;
  constexpr int NTW = C::NTW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  bf16 *bs = reinterpret_cast<bf16 *>(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RG, ks = wave / RG;
  const int slab = (int)(blockIdx.x % n_slabs);
  const int64_t row0 = (int64_t)(blockIdx.x / n_slabs) * C::BM;
  const int col0 = slab * C::NP;
  const int N = cols.N0 + cols.N1;
  const int nrows = (int)min<int64_t>(C::BM, M - row0);
  const auto rh = make_rsrc(h + row0 * K, (uint32_t)((int64_t)nrows * K * 2));
  const auto rw0 = make_rsrc(cols.W0, (uint32_t)((int64_t)K * cols.N0 * 2));
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
      breg[c] = buf_load16(rw0, live && gc < cols.N0 ? (uint32_t)(k * cols.N0 + gc) * 2u : kOutside);
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
  const int boff = (8 * (gi >> 1) + (lr >> 2)) * C::LDW + 16 * (gi & 1) + 4 * (lr & 3);
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
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    const int col = col0 + 32 * n + (lane & 31);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rg * 32 + 8 * b + 4 * (lane >> 5) + r;
        if (col >= N || row >= nrows) continue;
        cols.out[(row0 + row) * N + col] = acc[n][4 * b + r];
      }
  }
}

template <int NT, int RG, int KS>
void launch(const bf16 *h, const Cols &cols, int64_t M, int K, hipStream_t st) {
  using C = WideCfg<NT, RG, KS>;
  const size_t lds = C::LDS;
  const int n_slabs = (int)ceil_div(cols.N0, C::NP);
  hipLaunchKernelGGL((k_gen_proj_wide<NT, RG, KS>), dim3((unsigned)(ceil_div(M, C::BM) * n_slabs)),
                     dim3(C::NTH), lds, st, h, cols, M, K, n_slabs);
}

// One block of 4 waves per CU: 128-row blocks when the blocks number at least
// 256, else 64-row blocks with K in two parts.
template <int NT>
void launch_nt(const bf16 *h, const Cols &cols, int64_t M, int K, hipStream_t st) {
  if (ceil_div(M, 128) >= 256)
    launch<NT, 4, 1>(h, cols, M, K, st);
  else
    launch<NT, 2, 2>(h, cols, M, K, st);
}

// Tile kernel for 193..256 generator columns and for the fused form: 8 waves
// (two per SIMD) over 128 rows x one 256-column slab, wave w on rows 64 (w & 1)
// .. +63 and columns 64 (w >> 1) .. +63 (2 x 2 fragments of 32 x 32, so every
// fragment read from LDS serves two MFMAs).  Per step of KT k (64 for slabs
// from one source, 32 for the two-source slab) the block stages the h tile
// [128][KT] and the weight tile [KT][256] in LDS (double-buffered, one
// barrier per step); every thread loads 3 KT/32 16-byte pieces per step into
// a ring of register sets (four, or eight of the smaller steps), so that many
// steps are in flight.  A fragments are 16-byte reads of h rows (row pitch 80
// or 144 bytes: the eight rows of a read pass fall on distinct banks); B
// fragments are two ds_read_b64_tr_b16 (row pitch 544 bytes).  Blocks run
// over the XCDs so that the slabs of one row block share an XCD (and its L2
// copy of those rows of h).
constexpr int kPB = 272;  // LDS row of the weight tile (one k): 256 columns + pad, bf16
// TWO: the launch's columns may come from both sources (each piece is loaded
// from both, one of the two loads falling outside its buffer); else every
// column of the launch lies in W0.  The launch covers the columns from c_lo
// on; columns below cols.N0 go to xb when it is given.  R register sets.
// KT: k per step (32, or 64: twice the pieces per thread and the MFMAs
// between two barriers; h row pitch 144 bytes, again eight distinct bank
// groups per read pass).
template <bool TWO, int R, int KT>
__global__ void __launch_bounds__(512, 1)
k_proj_tile(const bf16 *__restrict__ h, Cols cols, int64_t M, int K, int c_lo, int n_slabs, int n_items,
            int slots) {
  constexpr int kPA = KT + 8;       // LDS row of the h tile: KT k + pad, bf16
  constexpr int NA = KT / 32;       // h pieces per thread and step
  constexpr int NB = KT / 16;       // weight pieces per thread and step
  __shared__ __attribute__((aligned(16))) bf16 as_[2][128 * kPA];
  __shared__ __attribute__((aligned(16))) bf16 bs_[2][KT * kPB];
  const int item = (int)(blockIdx.x & 7) * slots + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave & 1, wc = wave >> 1;
  const int slab = item % n_slabs;
  const int64_t row0 = (int64_t)(item / n_slabs) * 128;
  const int col0 = c_lo + slab * 256;
  const int N = cols.N0 + cols.N1;
  const int nrows = (int)min<int64_t>(128, M - row0);
  const auto rh = make_rsrc(h + row0 * K, (uint32_t)((int64_t)nrows * K * 2));
  const auto rw0 = make_rsrc(cols.W0, (uint32_t)((int64_t)K * cols.N0 * 2));
  const auto rw1 = make_rsrc(cols.W1, TWO ? (uint32_t)((int64_t)K * cols.N1 * 2) : 0u);
  const int S = (K + KT - 1) / KT;
  const int n_loop = (S + R - 1) / R * R;

  // pieces: 0 .. NA-1 -> h (row e/(KT/8), k 8 (e%(KT/8)), e = tid + 512 a);
  // NA .. -> weight (k e/32, column 8 (e%32) of the slab, e = tid + 512 b); a
  // weight chunk lies wholly in one source or past both (zeros)
  int a_row[NA], a_k[NA];
  uint32_t a_base[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int e = tid + 512 * a;
    a_row[a] = e / (KT / 8);
    a_k[a] = (e % (KT / 8)) * 8;
    a_base[a] = (uint32_t)((a_row[a] * K + a_k[a]) * 2);
  }
  int b_r[NB], b_c[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int e = tid + 512 * c;
    b_r[c] = e >> 5;
    b_c[c] = (e & 31) * 8;
  }
  uint4 rr[R][NA + NB];
  auto load = [&](int set, int st) {
    const int k0 = st * KT;
#pragma unroll
    for (int a = 0; a < NA; ++a)
      rr[set][a] = buf_load16(rh, k0 + a_k[a] < K ? a_base[a] + (uint32_t)(k0 * 2) : kOutside);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int k = k0 + b_r[c], gc = col0 + b_c[c];
      const bool live = k < K;
      rr[set][NA + c] = buf_load16(rw0, live && gc < cols.N0 ? (uint32_t)(k * cols.N0 + gc) * 2u : kOutside);
      if constexpr (TWO) {
        const uint4 b1 =
            buf_load16(rw1, live && gc >= cols.N0 && gc < N ? (uint32_t)(k * cols.N1 + gc - cols.N0) * 2u : kOutside);
        rr[set][NA + c] = make_uint4(rr[set][NA + c].x | b1.x, rr[set][NA + c].y | b1.y, rr[set][NA + c].z | b1.z,
                                     rr[set][NA + c].w | b1.w);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // A fragment (a, kh): row 64 wr + 32 a + lane%32, k 16 kh + 8 (lane/32) .. +7
  const int a_rd = ((64 * wr + (lane & 31)) * kPA + 8 * (lane >> 5)) * 2;
  // B fragment (kh, b): group G = lane/16 takes columns 16 (G & 1) .. +15 and k
  // 8 (G >> 1) .. +7; lane L = lane%16 reads k + L/4 at column 4 (L%4)
  const int G = lane >> 4, L = lane & 15;
  const int b_rd = ((8 * (G >> 1) + (L >> 2)) * kPB + 64 * wc + 16 * (G & 1) + 4 * (L & 3)) * 2;
  const unsigned char *as_b = reinterpret_cast<const unsigned char *>(&as_[0][0]);
  const unsigned char *bs_b = reinterpret_cast<const unsigned char *>(&bs_[0][0]);

  auto step = [&](int set, int st) {
    const int buf = set & 1;
#pragma unroll
    for (int a = 0; a < NA; ++a) *reinterpret_cast<uint4 *>(&as_[buf][a_row[a] * kPA + a_k[a]]) = rr[set][a];
#pragma unroll
    for (int c = 0; c < NB; ++c) *reinterpret_cast<uint4 *>(&bs_[buf][b_r[c] * kPB + b_c[c]]) = rr[set][NA + c];
    __syncthreads();
    load(set, st + R);
    const unsigned char *ab = as_b + buf * (128 * kPA * 2) + a_rd;
    const unsigned char *bb = bs_b + buf * (KT * kPB * 2) + b_rd;
#pragma unroll
    for (int kh = 0; kh < KT / 16; ++kh) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        af[x] = as_bf16x8(*reinterpret_cast<const uint4 *>(ab + (32 * x * kPA + 16 * kh) * 2));
        const unsigned char *pb = bb + (16 * kh * kPB + 32 * x) * 2;
        const uint2 b0 = read_tr16(pb), b1 = read_tr16(pb + 4 * kPB * 2);
        bfr[x] = as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
    }
  };
  // the prologue issues its loads in the loop's order, set by set, so that the
  // compiler's wait count at the loop head is the steady-state one
#pragma unroll
  for (int s = 0; s < R; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    load(s, s);
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int st = 0; st < n_loop; st += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) step(s, st + s);
  }

  // D: lane holds D[8 b + 4 (lane / 32) + r][lane % 32] in element 4 b + r
  const int split = cols.xb ? cols.N0 : 0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = col0 + 64 * wc + 32 * b + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 64 * wr + 32 * a + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (col >= N || row >= nrows) continue;
        const float v = acc[a][b][e];
        if (col < split)
          cols.xb[(row0 + row) * cols.N0 + col] = (bf16)v;  // round to nearest even
        else
          cols.out[(row0 + row) * (N - split) + col - split] = v;
      }
    }
}

// columns [c_lo, c_hi) in slabs of 256
template <bool TWO, int R, int KT = 32>
void launch_tile(const bf16 *h, const Cols &cols, int64_t M, int K, int c_lo, int c_hi, hipStream_t st) {
  const int n_slabs = (int)ceil_div(c_hi - c_lo, 256);
  const int n_items = (int)(ceil_div(M, 128) * n_slabs);
  const int slots = (int)ceil_div(n_items, 8);
  if (n_items == 0) return;
  hipLaunchKernelGGL((k_proj_tile<TWO, R, KT>), dim3((unsigned)(8 * slots)), dim3(512), 0, st, h, cols, M, K, c_lo,
                     n_slabs, n_items, slots);
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
  if (s.N > 192) {
    launch_tile<false, 4, 64>(hh, cols, s.BT, K, 0, s.N, st);
    trace_end(tr, st);
    return 0;
  }
  switch (ceil_div(s.N, 32)) {
    case 2: launch_nt<2>(hh, cols, s.BT, K, st); break;
    case 3: launch_nt<3>(hh, cols, s.BT, K, st); break;
    case 4: launch_nt<4>(hh, cols, s.BT, K, st); break;
    case 5: launch_nt<5>(hh, cols, s.BT, K, st); break;
    default: launch_nt<6>(hh, cols, s.BT, K, st); break;
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
  // the producing projection's whole slabs read Wp alone; the rest (a slab
  // holding both weights' columns, then the generator's) read both sources
  const int whole = (int)(s.D / 256 * 256);
  launch_tile<false, 4, 64>((const bf16 *)h, cols, s.BT, (int)s.d, 0, whole, st);
  launch_tile<true, 4>((const bf16 *)h, cols, s.BT, (int)s.d, whole, (int)s.D + s.N, st);
  trace_end(tr, st);
  return 0;
}

}  // namespace dynconv
