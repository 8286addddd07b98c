/*
 * dynconv.h -- C ABI of the MI355X (gfx950) dynamic short convolution
 * library, libdynconv.so.
 *
 * The layer ("Dynamic Short Convolutions Improve Transformers", gist.science
 * Technical Summary, Methodology -> Dynamic Short Convolutions):
 *   - Mechanism: the output at position t is a causal depthwise convolution
 *     of width k whose taps w_t are specific to position t and channel c;
 *     tap j multiplies the input j positions back.
 *   - Parameterization: w_t is a learned linear map of the current hidden
 *     state h_t, either low-rank (w_t = z_t U with z_t = h_t A) or head-wise
 *     (one k-tap filter per head, shared by that head's consecutive
 *     channels).  A static per-channel bias w0[D,k] is added to the
 *     generated filter, so the layer contains the static short convolution
 *     as the special case of a zero generator.
 *   - Placement: the result is added back residually.
 * Together, for every batch row b, token t and channel c:
 *
 *   y[b,t,c] = x[b,t,c] + sum_{j=0}^{k-1} [t-j >= 0] w[b,t,c,j] * x[b,t-j,c]
 *   w[b,t,c,j] = u[b,t,head(c),j] + w0[c,j]        head-wise, head(c) = c / (D/n_heads)
 *   w[b,t,c,j] = sum_q z[b,t,q] U[q, c*k+j] + w0[c,j],  z = h A   low-rank
 *   u[b,t,e,j] = sum_i h[b,t,i] W[i, e*k+j]
 *
 * Tokens before the start of each sequence count as zero and nothing
 * crosses batch rows, nor, in a packed row, document boundaries (see
 * dynconv_problem).  The filter w is never written to memory (the
 * Efficient Training Implementation section's Fused Low-Rank Kernel item
 * describes the same: the product zU is formed on chip).
 *
 * The backward (dynconv_bwd) is the exact gradient of L = sum(dy * y):
 *   dx[s,c] = dy[s,c] + sum_j [s+j <= T-1] w[s+j,c,j] dy[s+j,c]
 *   G[t,c,j] = [t-j >= 0] dy[t,c] x[t-j,c],  dw0 = sum_{b,t} G
 *   head-wise: du[t,e,j] = sum_{c in e} G[t,c,j], dW = sum_t h_t^T du_t, dh = du W^T
 *   low-rank : dz[t,q] = sum_{c,j} G[t,c,j] U[q,c*k+j], dU = sum_t z_t^T G_t,
 *              dA = sum_t h_t^T dz_t, dh = dz A^T
 *
 * Layout: every tensor is row-major and contiguous.
 *   h[B,T,d_model], x, y, dy, dx [B,T,D], W[d_model, n_heads*k] (column e*k+j),
 *   A[d_model, rank], U[rank, D*k] (column c*k+j), w0[D,k].
 *   gen_cache: fp32 [B*T, n_heads*k] (u) or [B*T, rank] (z).
 * Precision: activations, generator weights and w0 are in the I/O dtype
 *   (fp32 or bf16); every sum accumulates in fp32; dx and dh are written in
 *   the I/O dtype with round-to-nearest-even; weight gradients are fp32.
 *
 * Ownership and execution: the caller owns every buffer; all pointers are
 * device pointers except the three structs, which are read on the host
 * during the call only.  The library never allocates or frees device
 * memory, never copies between host and device and never synchronises: a
 * call validates its arguments on the host and then only enqueues kernels
 * on `stream`, so it returns before the work is done.  Inputs are read-only.
 * Outputs must not overlap any input or each other.  The workspace must
 * not be used by anything else until the enqueued work has finished.
 * Results are bitwise deterministic for fixed inputs and shapes (no float
 * atomics; every reduction runs in a fixed order).  A batch whose tensors
 * are too large for the tuned kernels' 32-bit offsets (a 2 GiB tensor)
 * runs as consecutive chunks of whole sequences, each the largest the
 * tuned kernels take; the per-sequence outputs are those of a call on that
 * chunk alone, the weight gradients the chunks' sums added in chunk order,
 * and the workspace that of the largest chunk.  Packed rows run whole.
 * The library is
 * thread-safe.  Its global state is the one-shot event pair that
 * dynconv_trace_next arms, kept per host thread, and the static scratch of
 * dynconv_fwd_noalloc (one array per GPU, with a mutex-guarded table of its
 * per-GPU addresses).
 *
 * Errors: every call returns DYNCONV_OK (0) or a negative status.  Argument
 * errors are detected on the host before anything is enqueued, and the
 * outputs are then untouched.  DYNCONV_E_HIP reports a failed launch; a
 * fault during kernel execution surfaces at the caller's next
 * synchronisation.  With B*T == 0 the forward enqueues nothing and the
 * backward only writes the (empty-sum) zero weight gradients; both return
 * DYNCONV_OK.  No C++ exception crosses this interface and nothing is
 * printed.
 *
 * Sizes: any D and d_model are accepted.  The tuned kernels take rows made
 * of whole 16-byte vectors (D and d_model multiples of 8 for bf16, of 4 for
 * fp32); other widths run on plain per-element kernels with the same
 * results up to summation order.
 */
#ifndef DYNCONV_H
#define DYNCONV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DYNCONV_ABI_VERSION 3

#ifndef DYNCONV_API
#define DYNCONV_API __attribute__((visibility("default")))
#endif

/* I/O dtype.  Accumulation is fp32 for both. */
typedef enum { DYNCONV_FP32 = 0, DYNCONV_BF16 = 1 } dynconv_dtype;

/* Filter-generator parameterisation.  DYNCONV_STATIC: no generator, the
 * filter is the static bias alone, w[t,c,j] = w0[c,j]: the fixed depthwise
 * short convolution the pages take as the baseline primitive (gist.science
 * Technical Summary, Problem; the dynamic layer with a zero generator).  With
 * it, h and d_model are not used (h may be NULL, d_model 0) except by
 * dynconv_fwd_proj, n_heads, rank, W, A, U and the generator cache are
 * ignored (the cache holds 0 bytes), w0 is required, and the backward writes
 * dx and dw0 and fills dh, when given, with zeros (y does not depend on h). */
typedef enum { DYNCONV_HEADWISE = 0, DYNCONV_LOWRANK = 1, DYNCONV_STATIC = 2 } dynconv_kind;

enum {
  DYNCONV_OK = 0,
  DYNCONV_E_NULL = -1,      /* a required pointer is NULL                        */
  DYNCONV_E_SHAPE = -2,     /* a size <= 0 (B, T may be 0), D % n_heads != 0,    */
                            /* rank <= 0, or packed documents with B != 1 or     */
                            /* n_seqs < 1 (or given to the decode step)           */
  DYNCONV_E_K = -3,         /* k outside [1, 8]                                   */
  DYNCONV_E_DTYPE = -4,     /* dtype or kind not one of the enums                 */
  DYNCONV_E_ALIGN = -5,     /* a tensor pointer not 16-byte aligned (cu_seqlens:  */
                            /* not 4-byte aligned)                                */
  DYNCONV_E_ALIAS = -6,     /* an output overlaps an input or another output      */
  DYNCONV_E_WORKSPACE = -7, /* workspace NULL or smaller than required            */
  DYNCONV_E_HIP = -8,       /* a kernel launch failed                             */
  DYNCONV_E_LIMIT = -9,     /* a size exceeds what the kernels index (see below)  */
  DYNCONV_E_SCRATCH = -10   /* dynconv_fwd_noalloc: the call needs more workspace */
                            /* than its static scratch holds                      */
};

/* Problem sizes.  B*T tokens, hidden width d_model, D convolved channels,
 * filter width k (1..8).  Limits: B*T*max(D, d_model) < 2^31 elements per
 * tensor; n_heads*k and rank <= 256 (rank <= 64 on the bf16 path).
 *
 * Packed documents (cu_seqlens != NULL): the single row (B must be 1) holds
 * n_seqs documents back to back, document i being tokens cu_seqlens[i] ..
 * cu_seqlens[i+1]-1.  The causal window stops at every document start as it
 * stops at a row start: a tap that would reach a token of the previous
 * document contributes nothing, in the forward and in every gradient.  So
 * the packed row gives each document's results exactly as if it were run as
 * its own sequence (the pages are silent on packing; this is the plain
 * reading of the Mechanism item, whose window only looks back within a
 * sequence).  cu_seqlens is a device array of n_seqs + 1 int32, 4-byte
 * aligned, with 0 = cu_seqlens[0] <= cu_seqlens[1] <= ... <= cu_seqlens[n_seqs]
 * = T (empty documents allowed).  It is read on the device only, so the host
 * cannot check those values: offsets that break the rule give unspecified
 * results (never an access outside the tensors).  The decode step takes no
 * packing (cu_seqlens must be NULL there). */
typedef struct {
  int64_t B, T, d_model, D;
  int32_t k;
  int32_t dtype; /* dynconv_dtype */
  const int32_t *cu_seqlens; /* NULL, or document offsets (device, n_seqs + 1 entries) */
  int64_t n_seqs;            /* documents in the packed row (used with cu_seqlens only) */
} dynconv_problem;

/* Generator weights (device pointers, I/O dtype). */
typedef struct {
  int32_t kind;    /* dynconv_kind                                  */
  int32_t n_heads; /* head-wise: number of heads, D % n_heads == 0  */
  int32_t rank;    /* low-rank: rank r                              */
  int32_t reserved;
  const void *W;  /* head-wise [d_model, n_heads*k]; unused otherwise */
  const void *A;  /* low-rank [d_model, rank]; unused otherwise       */
  const void *U;  /* low-rank [rank, D*k]; unused otherwise           */
  const void *w0; /* static bias [D, k], or NULL for none (required    */
                  /* with DYNCONV_STATIC)                              */
} dynconv_gen;

/* Weight gradients, fp32 device pointers, overwritten (not accumulated).
 * Head-wise needs dW; low-rank needs dA and dU.  dw0 may be NULL to skip. */
typedef struct {
  float *dW;  /* [d_model, n_heads*k] */
  float *dA;  /* [d_model, rank]      */
  float *dU;  /* [rank, D*k]          */
  float *dw0; /* [D, k]               */
} dynconv_gen_grad;

/*
 * Forward: y = x + dynconv(x) (see the header comment).
 *   h, x      inputs, I/O dtype, [B,T,d_model] and [B,T,D]
 *   y         output, I/O dtype, [B,T,D]
 *   gen_cache NULL, or an fp32 buffer of dynconv_gen_cache_bytes() that
 *             receives u = h W (head-wise) or z = h A (low-rank) for reuse
 *             by dynconv_bwd with the same inputs and weights
 *   workspace device scratch of at least dynconv_workspace_bytes(p, g, 0),
 *             or (p, g, DYNCONV_WS_CACHED) when gen_cache is given
 */
DYNCONV_API int dynconv_fwd(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x,
                void *y, void *gen_cache, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * Forward with the producing projection fused in.  The layer sits after a
 * linear projection of the same hidden state that generates its filters
 * (gist.science Technical Summary, Methodology -> Dynamic Short
 * Convolutions, Placement: on the query, key and value projections, or after
 * any linear layer), so its input is x = h Wp.  This call computes that x and
 * the generator values (u = h W or z = h A) in one pass over h (on the bf16
 * path, one matrix-core GEMM against [Wp | W] or [Wp | A] with the weights
 * read in place), then the layer on x as dynconv_fwd does:
 *   x[t, c] = sum_i h[t, i] Wp[i, c]      (written to x, I/O dtype, rounded to nearest even)
 *   y = x + dynconv(x)
 *   Wp        [d_model, D], I/O dtype, row-major (the projection's weight)
 *   x         output [B,T,D], I/O dtype
 * Everything else as for dynconv_fwd (same workspace size).  x must not
 * overlap any input or other output.  The projection's own backward (dh +=
 * dx Wp^T, dWp = h^T dx) is the caller's: dynconv_bwd returns dx.
 */
DYNCONV_API int dynconv_fwd_proj(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *Wp,
                                 void *x, void *y, void *gen_cache, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * dynconv_fwd with the same arguments except the workspace, which is a
 * static device array of DYNCONV_NOALLOC_SCRATCH_BYTES inside the library.
 * The call itself allocates nothing (no hipMalloc or hipFree, no allocating
 * library routine).  Each GPU the library runs on holds one such array from
 * its first use until the process ends; the call runs on the current device
 * (`stream` must belong to it).  All calls on one GPU share that GPU's
 * array, so calls that overlap in time on one GPU race and must be
 * serialised by the caller (one stream, or events).  Nothing in the array
 * needs to start at zero: the forward writes every byte it later reads.
 * Returns DYNCONV_E_SCRATCH, enqueuing nothing, when the forward needs more
 * workspace than the array holds (dynconv_workspace_bytes with pass 0, or
 * DYNCONV_WS_CACHED with a caller cache, tells how much it needs); all
 * other errors as for dynconv_fwd.  The results equal dynconv_fwd's bitwise.
 */
#define DYNCONV_NOALLOC_SCRATCH_BYTES (16u << 20)
DYNCONV_API int dynconv_fwd_noalloc(const dynconv_problem *p, const dynconv_gen *g, const void *h,
                                    const void *x, void *y, void *gen_cache, hipStream_t stream);

/*
 * Backward of L = sum(dy * y) for the forward above.
 *   h, x, dy  inputs (I/O dtype); dy is [B,T,D]
 *   gen_cache the cache a dynconv_fwd with the same inputs filled, or NULL
 *             to recompute it
 *   dx        output [B,T,D], I/O dtype
 *   dh        output [B,T,d_model], I/O dtype, or NULL to skip
 *   gg        weight gradients (fp32), overwritten
 *   workspace device scratch of at least dynconv_workspace_bytes(p, g, 1),
 *             or (p, g, 1 | DYNCONV_WS_CACHED) when gen_cache is given
 */
DYNCONV_API int dynconv_bwd(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x,
                const void *dy, const void *gen_cache, void *dx, void *dh,
                const dynconv_gen_grad *gg, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * Decode step (inference): one new token for each of B sequences.  The taps
 * of the causal convolution (Mechanism) reach the k-1 previous rows of x, so
 * a decoder keeps those rows per sequence; the filter of the new token comes
 * from its hidden state as in the forward (Parameterization).  The pages
 * leave inference unoptimised (atlas.scime.ai, "Dynamic Convolutions Improve
 * Transformers", Limitations).  For every sequence b and channel c:
 *
 *   y[b,c] = x[b,c] + w[b,c,0] x[b,c] + sum_{j=1}^{k-1} w[b,c,j] state[b,k-1-j,c]
 *
 * with w[b,c,j] formed from h[b] exactly as in dynconv_fwd, then the history
 * shifts by one row: state[b,m] = state[b,m+1] for m < k-2, state[b,k-2] =
 * x[b].  Starting from a zeroed state, the t-th call on a sequence returns
 * row t of dynconv_fwd on that sequence (up to summation order).
 *   p      sizes with T == 1 (one token per sequence); B may be 0 (no-op)
 *   h, x   inputs [B, d_model] and [B, D], I/O dtype
 *   state  [B, k-1, D], I/O dtype, read and updated in place (the oldest row
 *          first); may be NULL when k == 1
 *   y      output [B, D], I/O dtype
 * No workspace.  Errors as for dynconv_fwd; DYNCONV_E_SHAPE if T != 1,
 * DYNCONV_E_LIMIT if B > 65535.  y and state must not overlap each other or
 * any input.
 */
DYNCONV_API int dynconv_decode(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x,
                   void *state, void *y, hipStream_t stream);

/* Workspace bytes a pass needs: pass 0 = forward, 1 = backward, each
 * optionally or-ed with DYNCONV_WS_CACHED when the caller passes gen_cache
 * to that call (the library then needs no slot of its own for the
 * generator cache, B*T * (n_heads*k or rank) * 4 bytes less).  Without the
 * flag the size covers both cases.  0 on invalid arguments.  Depends only
 * on the sizes and the flag, never on pointers. */
#define DYNCONV_WS_CACHED 2
DYNCONV_API size_t dynconv_workspace_bytes(const dynconv_problem *p, const dynconv_gen *g, int pass);

/* Bytes of the fp32 generator cache (B*T * (n_heads*k or rank) * 4). */
DYNCONV_API size_t dynconv_gen_cache_bytes(const dynconv_problem *p, const dynconv_gen *g);

/* Static description of a status code; never NULL. */
DYNCONV_API const char *dynconv_status_str(int status);

/* DYNCONV_ABI_VERSION of the built library. */
DYNCONV_API int dynconv_abi_version(void);

/* Kernels of the path, as named by dynconv_trace_next. */
typedef enum {
  DYNCONV_K_GEN_PROJ = 1, /* u = h W or z = h A                              */
  DYNCONV_K_FWD_CONV = 2, /* filter formation + causal conv + residual (fwd)  */
  DYNCONV_K_BWD_CONV = 3, /* dx, filter gradient, du / dz, dU and dw0 parts   */
  DYNCONV_K_GEN_BWD = 4,  /* dh and the dW / dA parts                         */
  DYNCONV_K_FINALIZE = 5  /* fixed-order sums of the weight-gradient parts    */
} dynconv_kernel;

/*
 * Profiling aid for callers that time one kernel with their own HIP events
 * (not part of the layer's computation).  Arms a one-shot pair for the
 * calling host thread: the next dynconv_fwd / dynconv_bwd on this thread
 * that launches `kernel` records `start` on its stream right before that
 * launch and `stop` right after it, then disarms.  Passing NULL events
 * disarms.  Returns DYNCONV_OK, or DYNCONV_E_DTYPE for an unknown kernel.
 * The events belong to the caller.
 */
DYNCONV_API int dynconv_trace_next(int kernel, hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif /* DYNCONV_H */
