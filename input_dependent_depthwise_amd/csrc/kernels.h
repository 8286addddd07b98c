// kernels.h -- host-side launchers of libdynconv's kernels (internal).
#pragma once

#include "common.h"

namespace dynconv {

// Profiling hook (dynconv_trace_next): a launcher calls trace_begin right
// before the traced kernel's launch and trace_end right after it.
bool trace_begin(int kernel, hipStream_t st);
void trace_end(bool armed, hipStream_t st);

// Writes n zeros at p (no-op when p is NULL or n is 0).
void zero_fill(float *p, int64_t n, hipStream_t st);
// Writes nbytes (a multiple of 2) of zeros at p.
void zero_fill_bytes(void *p, size_t nbytes, hipStream_t st);

// Packed documents: the per-token position table of Shape::seqpos from the
// document offsets cu[0 .. n_seqs] (simple_kernels.hip).
void seqpos_fill(const int32_t *cu, int64_t n_seqs, int64_t BT, uint16_t *out, hipStream_t st);

// --- plain VALU kernels (simple_kernels.hip); T = float or bf16 ---
template <typename T>
int simple_gen_proj(const Shape &s, const void *h, const void *M, float *out, hipStream_t st);
template <typename T>
int simple_fwd_conv(const Shape &s, const float *gen, const void *U, const void *w0, const void *x,
                    void *y, hipStream_t st);
template <typename T>
int simple_bwd(const Shape &s, const float *gen, const void *W, const void *A, const void *U,
               const void *w0, const void *h, const void *x, const void *dy, void *dx, void *dh,
               const dynconv_gen_grad &gg, float *g, hipStream_t st);

// --- one decoding step, T = float or bf16 (decode.hip) ---
template <typename T>
int decode_step(const Shape &s, const void *h, const void *W, const void *A, const void *U, const void *w0,
                const void *x, void *state, void *y, hipStream_t st);

// --- bf16 matrix-core generator projection (gen_mfma.hip) ---
size_t gen_proj_mfma_ws_bytes(const Shape &s);
int gen_proj_mfma(const Shape &s, const void *h, const void *M, float *out, void *ws, hipStream_t st);
// wide weights (N a multiple of 8, 64..256 columns), read in place (gen_proj_wide.hip)
bool gen_proj_wide_ok(const Shape &s);
int gen_proj_wide(const Shape &s, const void *h, const void *M, float *out, hipStream_t st);
// the producing projection x = h Wp fused with it: one pass over h writes x
// (bf16 [BT, D]) and the generator values (fp32 [BT, N]) (gen_proj_wide.hip)
bool proj_fused_ok(const Shape &s);
int proj_fused(const Shape &s, const void *h, const void *Wp, const void *M, void *x, float *gen, hipStream_t st);
// the producing projection alone, plain kernel: x[t, c] = sum_i h[t, i] Wp[i, c] in T
template <typename T>
int simple_proj(const Shape &s, const void *h, const void *Wp, void *x, hipStream_t st);

// --- head-wise forward conv, coalesced per-vector walk (conv_fwd_headwise.hip) ---
template <typename T>
int fwd_headwise(const Shape &s, const float *u, const void *w0, const void *x, void *y,
                 hipStream_t st);

// --- fused low-rank forward on matrix cores (conv_fwd_lowrank.hip), bf16 ---
bool fwd_lowrank_supported(const Shape &s);
// the head-wise forward's ring kernel takes the shape (bf16)
bool fwd_headwise_ring_ok(const Shape &s);
int fwd_lowrank(const Shape &s, const float *z, const void *U, const void *w0, const void *x, void *y,
                hipStream_t st);

// --- fused backward conv, bf16 ---
// Layout of one backward pass over the channels (slices of Dt channels, grid
// x) and the tokens (n_ranges blocks, grid y), and of its partial sums.
struct BwdLayout {
  int Dt;        // channels per slice
  int n_slices;  // slices (grid x)
  int n_tiles;   // low-rank: 32-token tiles
  int tpb;       // low-rank: tiles per block; head-wise: tokens per wave
  int n_ranges;  // blocks along the tokens (grid y): rows of the dU / dw0 partials
  int SL;        // head-wise: head slots per slice
  int R;         // columns of the per-slice partial (rank, or SL*k)
};
// whether the fused path covers the shape, and its layout (dispatches on kind)
bool bwd_fused_supported(const Shape &s);
BwdLayout bwd_layout(const Shape &s);
// head-wise: one lane per 8 (or 4) channels walking along time (conv_bwd_headwise.hip)
bool bwd_headwise_supported(const Shape &s);
BwdLayout bwd_headwise_layout(const Shape &s);
int bwd_headwise(const Shape &s, const BwdLayout &L, const float *u, const void *w0, const void *x,
                 const void *dy, void *dx, float *gpart, float *dw0p, hipStream_t st);
// low-rank: filter, dz and dU on matrix cores, 8 waves x 16 channels per block
// (conv_bwd_lowrank.hip); R = rank
bool bwd_lowrank_supported(const Shape &s);
BwdLayout bwd_lowrank_layout(const Shape &s);
int bwd_lowrank(const Shape &s, const BwdLayout &L, const float *z, const void *U, const void *w0, const void *x,
                const void *dy, void *dx, float *gpart, float *dUp, float *dw0p, hipStream_t st);

// --- generator gradients (gen_bwd.hip), bf16 ---
struct GenBwdLayout {
  int Np;        // N padded to 16
  int n_tiles;   // 32-token tiles
  int64_t BTp;   // tokens padded to whole tiles (row length of g^T)
  int n_chunks;  // 128-row chunks of d_model (dM)
  int tpb;       // tiles per block of the dM kernel (even)
  int n_ranges;  // token ranges of the dM kernel (partials)
  int n_rb;      // 256-row blocks of d_model (dh)
  int tpr;       // tiles per token range of the dh kernel (even)
  int n_tr;      // token ranges of the dh kernel
  bool wide;     // Np > 128: the dM kernel for wide weights (reads g, no g^T)
};
GenBwdLayout gen_bwd_layout(const Shape &s);
bool gen_bwd_supported(const Shape &s);
size_t gen_bwd_g_bytes(const Shape &s);
size_t gen_bwd_mp_bytes(const Shape &s);
size_t gen_bwd_part_bytes(const Shape &s);
int gen_bwd(const Shape &s, const float *gpart, int n_slices, int R, int Dt, const void *h,
            const void *M, bf16 *g, bf16 *Mp, void *dh, float *dMp, hipStream_t st);
// out_i[e] = sum_p part_i[p][e] (acc: out_i[e] += that sum); an output may be
// NULL to skip it.
int finalize(const float *p0, float *o0, int64_t n0, int np0, const float *p1, float *o1, int64_t n1,
             int np1, const float *p2, float *o2, int64_t n2, int np2, bool acc, hipStream_t st);

}  // namespace dynconv
