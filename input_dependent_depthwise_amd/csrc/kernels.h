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

// --- bf16 matrix-core generator projection (gen_mfma.hip) ---
size_t gen_proj_mfma_ws_bytes(const Shape &s);
int gen_proj_mfma(const Shape &s, const void *h, const void *M, float *out, void *ws, hipStream_t st);

// --- head-wise forward conv, coalesced per-vector walk (conv_fwd_headwise.hip) ---
template <typename T>
int fwd_headwise(const Shape &s, const float *u, const void *w0, const void *x, void *y,
                 hipStream_t st);

// --- fused low-rank forward on matrix cores (conv_fwd_lowrank.hip), bf16 ---
bool fwd_lowrank_supported(const Shape &s);
size_t fwd_lowrank_ws_bytes(const Shape &s);
int prep_lowrank_frags(const Shape &s, const void *U, const void *w0, void *Uf, hipStream_t st);
int fwd_lowrank(const Shape &s, const float *z, const void *Uf, const void *x, void *y, hipStream_t st);

}  // namespace dynconv
