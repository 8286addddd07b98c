// kernels.h -- host-side launchers of libdynconv's kernels (internal).
#pragma once

#include "common.h"

namespace dynconv {

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

}  // namespace dynconv
