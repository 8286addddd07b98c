// api.hip -- the C ABI of libdynconv (declared in include/dynconv.h):
// argument validation on the host, workspace planning, kernel dispatch.
//
// Nothing here allocates, frees, copies or synchronises.  Every entry point
// validates everything before it enqueues anything, so a rejected call
// leaves all outputs untouched.
#include <new>

#include "kernels.h"

namespace dynconv {
namespace {

constexpr size_t kAlign = 256;  // sub-buffers of the workspace start on 256-byte boundaries

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const void *p;
  size_t bytes;
};

inline bool overlap(const Range &a, const Range &b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Structural validation shared by every entry point.  Fills `s`.
int check_problem(const dynconv_problem *p, const dynconv_gen *g, Shape &s) {
  if (!p || !g) return DYNCONV_E_NULL;
  if (p->dtype != DYNCONV_FP32 && p->dtype != DYNCONV_BF16) return DYNCONV_E_DTYPE;
  if (g->kind != DYNCONV_HEADWISE && g->kind != DYNCONV_LOWRANK) return DYNCONV_E_DTYPE;
  if (p->k < 1 || p->k > 8) return DYNCONV_E_K;
  if (p->B < 0 || p->T < 0 || p->d_model <= 0 || p->D <= 0) return DYNCONV_E_SHAPE;
  const int64_t vec = p->dtype == DYNCONV_BF16 ? 8 : 4;
  if (p->D % vec != 0 || p->d_model % vec != 0) return DYNCONV_E_SHAPE;
  int N;
  if (g->kind == DYNCONV_HEADWISE) {
    if (g->n_heads <= 0 || p->D % g->n_heads != 0) return DYNCONV_E_SHAPE;
    if ((int64_t)g->n_heads * p->k > 256) return DYNCONV_E_LIMIT;
    N = g->n_heads * p->k;
  } else {
    if (g->rank <= 0) return DYNCONV_E_SHAPE;
    if (g->rank > (p->dtype == DYNCONV_BF16 ? 64 : 256)) return DYNCONV_E_LIMIT;
    N = g->rank;
  }
  // every tensor must be indexable with 31-bit element offsets
  const int64_t lim = (int64_t)1 << 31;
  if (p->B > lim || p->T > lim) return DYNCONV_E_LIMIT;
  const int64_t BT = p->B * p->T;
  if (BT > 0 && (BT > lim / p->D || BT > lim / p->d_model || BT > lim / N)) return DYNCONV_E_LIMIT;
  if (p->D * p->k > lim / 256 || p->d_model * N > lim) return DYNCONV_E_LIMIT;
  s.B = p->B;
  s.T = p->T;
  s.BT = BT;
  s.d = p->d_model;
  s.D = p->D;
  s.k = p->k;
  s.kind = g->kind;
  s.n_heads = g->kind == DYNCONV_HEADWISE ? g->n_heads : 0;
  s.rank = g->kind == DYNCONV_LOWRANK ? g->rank : 0;
  s.N = N;
  s.hd = g->kind == DYNCONV_HEADWISE ? (int)(p->D / g->n_heads) : 0;
  return DYNCONV_OK;
}

// Workspace layout of one pass.  Regions start on 256-byte boundaries.
struct Plan {
  size_t cache = 0;  // generator cache slot, fp32 [BT, N] (used when the caller gives none)
  size_t g = 0;      // simple path: du or dz, fp32 [BT, N]; fused path: g, bf16 [BT, Np]
  size_t mt = 0;     // transposed, padded generator weight for the MFMA projection (bf16)
  size_t gpart = 0;  // per-slice du / dz partials, fp32
  size_t dup = 0;    // per-range dU partials, fp32
  size_t dw0p = 0;   // per-range dw0 partials, fp32
  size_t mp = 0;     // generator weight padded to Np columns (bf16)
  size_t dmp = 0;    // per-range dW / dA partials, fp32
  size_t total = 0;
};

inline bool fast_lowrank(const Shape &s, int dtype) {
  return dtype == DYNCONV_BF16 && s.kind == DYNCONV_LOWRANK && fwd_lowrank_supported(s);
}
inline bool fast_bwd(const Shape &s, int dtype) {
  return dtype == DYNCONV_BF16 && bwd_fused_supported(s) && gen_bwd_supported(s);
}

Plan plan(const Shape &s, int dtype, int pass) {
  Plan pl;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes);
    return at;
  };
  pl.cache = take((size_t)s.BT * s.N * sizeof(float));
  if (dtype == DYNCONV_BF16) pl.mt = take(gen_proj_mfma_ws_bytes(s));
  if (pass == 1) {
    if (fast_bwd(s, dtype)) {
      const BwdLayout L = bwd_layout(s);
      pl.gpart = take((size_t)L.n_slices * s.BT * L.R * sizeof(float));
      if (s.kind == DYNCONV_LOWRANK) pl.dup = take((size_t)L.n_ranges * s.N * s.D * s.k * sizeof(float));
      pl.dw0p = take((size_t)L.n_ranges * s.D * s.k * sizeof(float));
      pl.g = take(gen_bwd_g_bytes(s));
      pl.mp = take(gen_bwd_mp_bytes(s));
      pl.dmp = take(gen_bwd_part_bytes(s));
    } else {
      pl.g = take((size_t)s.BT * s.N * sizeof(float));
    }
  }
  pl.total = off;
  return pl;
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? DYNCONV_OK : DYNCONV_E_HIP;
}

// Byte sizes of the problem's tensors.
struct Sizes {
  size_t h, x, W, A, U, w0, cache, dW, dA, dU, dw0;
};

Sizes sizes(const Shape &s, int eb) {
  Sizes z;
  z.h = (size_t)s.BT * s.d * eb;
  z.x = (size_t)s.BT * s.D * eb;
  z.W = s.kind == DYNCONV_HEADWISE ? (size_t)s.d * s.N * eb : 0;
  z.A = s.kind == DYNCONV_LOWRANK ? (size_t)s.d * s.N * eb : 0;
  z.U = s.kind == DYNCONV_LOWRANK ? (size_t)s.N * s.D * s.k * eb : 0;
  z.w0 = (size_t)s.D * s.k * eb;
  z.cache = (size_t)s.BT * s.N * sizeof(float);
  z.dW = s.kind == DYNCONV_HEADWISE ? (size_t)s.d * s.N * sizeof(float) : 0;
  z.dA = s.kind == DYNCONV_LOWRANK ? (size_t)s.d * s.N * sizeof(float) : 0;
  z.dU = s.kind == DYNCONV_LOWRANK ? (size_t)s.N * s.D * s.k * sizeof(float) : 0;
  z.dw0 = (size_t)s.D * s.k * sizeof(float);
  return z;
}

int check_weights(const Shape &s, const dynconv_gen *g) {
  if (s.kind == DYNCONV_HEADWISE && !g->W) return DYNCONV_E_NULL;
  if (s.kind == DYNCONV_LOWRANK && (!g->A || !g->U)) return DYNCONV_E_NULL;
  const void *ws[] = {g->W, g->A, g->U, g->w0};
  for (const void *w : ws)
    if (w && !aligned16(w)) return DYNCONV_E_ALIGN;
  return DYNCONV_OK;
}

// Generator projection (u = h W or z = h A) into `cache`.
int gen_proj(const Shape &s, int dtype, const dynconv_gen *g, const void *h, float *cache,
             void *ws, const Plan &pl, hipStream_t st) {
  const void *M = s.kind == DYNCONV_HEADWISE ? g->W : g->A;
  if (dtype == DYNCONV_BF16) return gen_proj_mfma(s, h, M, cache, (char *)ws + pl.mt, st);
  return simple_gen_proj<float>(s, h, M, cache, st);
}

}  // namespace

// One-shot event pair armed by dynconv_trace_next (per host thread).
namespace {
struct Trace {
  int kernel = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local Trace g_trace;
}  // namespace

bool trace_begin(int kernel, hipStream_t st) {
  if (g_trace.kernel == 0 || g_trace.kernel != kernel) return false;
  (void)hipEventRecord(g_trace.start, st);
  return true;
}

void trace_end(bool armed, hipStream_t st) {
  if (!armed) return;
  (void)hipEventRecord(g_trace.stop, st);
  g_trace = Trace();
}

}  // namespace dynconv

using namespace dynconv;

extern "C" {

int dynconv_abi_version(void) { return DYNCONV_ABI_VERSION; }

int dynconv_trace_next(int kernel, hipEvent_t start, hipEvent_t stop) {
  if (!start || !stop) {
    g_trace = Trace();
    return DYNCONV_OK;
  }
  if (kernel < DYNCONV_K_GEN_PROJ || kernel > DYNCONV_K_FINALIZE) return DYNCONV_E_DTYPE;
  g_trace.kernel = kernel;
  g_trace.start = start;
  g_trace.stop = stop;
  return DYNCONV_OK;
}

const char *dynconv_status_str(int status) {
  switch (status) {
    case DYNCONV_OK: return "ok";
    case DYNCONV_E_NULL: return "a required pointer is NULL";
    case DYNCONV_E_SHAPE: return "invalid shape (size <= 0, D % n_heads != 0, rank <= 0, or D/d_model not a multiple of 16 bytes)";
    case DYNCONV_E_K: return "filter width k outside [1, 8]";
    case DYNCONV_E_DTYPE: return "unknown dtype or generator kind";
    case DYNCONV_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case DYNCONV_E_ALIAS: return "an output overlaps an input or another output";
    case DYNCONV_E_WORKSPACE: return "workspace missing or too small";
    case DYNCONV_E_HIP: return "kernel launch failed";
    case DYNCONV_E_LIMIT: return "a size exceeds the library's limits";
    default: return "unknown status";
  }
}

size_t dynconv_gen_cache_bytes(const dynconv_problem *p, const dynconv_gen *g) {
  Shape s;
  if (check_problem(p, g, s) != DYNCONV_OK) return 0;
  return (size_t)s.BT * s.N * sizeof(float);
}

size_t dynconv_workspace_bytes(const dynconv_problem *p, const dynconv_gen *g, int pass) {
  Shape s;
  if ((pass != 0 && pass != 1) || check_problem(p, g, s) != DYNCONV_OK) return 0;
  return plan(s, p->dtype, pass).total;
}

int dynconv_fwd(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x,
                void *y, void *gen_cache, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
  Shape s;
  int rc = check_problem(p, g, s);
  if (rc) return rc;
  if (s.BT == 0) return DYNCONV_OK;
  if (!h || !x || !y) return DYNCONV_E_NULL;
  if ((rc = check_weights(s, g))) return rc;
  const void *ptrs[] = {h, x, y, gen_cache, workspace};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return DYNCONV_E_ALIGN;
  const Plan pl = plan(s, p->dtype, 0);
  if (workspace_bytes < pl.total || (pl.total > 0 && !workspace)) return DYNCONV_E_WORKSPACE;
  const int eb = p->dtype == DYNCONV_BF16 ? 2 : 4;
  const Sizes z = sizes(s, eb);
  const Range ins[] = {{h, z.h}, {x, z.x}, {g->W, z.W}, {g->A, z.A}, {g->U, z.U},
                       {g->w0, g->w0 ? z.w0 : 0}};
  const Range outs[] = {{y, z.x}, {gen_cache, gen_cache ? z.cache : 0}, {workspace, pl.total}};
  for (const Range &o : outs) {
    for (const Range &i : ins)
      if (overlap(o, i)) return DYNCONV_E_ALIAS;
  }
  for (int a = 0; a < 3; ++a)
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], outs[b])) return DYNCONV_E_ALIAS;

  float *cache = gen_cache ? (float *)gen_cache : (float *)((char *)workspace + pl.cache);
  if ((rc = gen_proj(s, p->dtype, g, h, cache, workspace, pl, stream))) return rc;
  if (s.kind == DYNCONV_HEADWISE) {
    rc = p->dtype == DYNCONV_BF16 ? fwd_headwise<bf16>(s, cache, g->w0, x, y, stream)
                                  : fwd_headwise<float>(s, cache, g->w0, x, y, stream);
  } else if (fast_lowrank(s, p->dtype)) {
    rc = fwd_lowrank(s, cache, g->U, g->w0, x, y, stream);
  } else if (p->dtype == DYNCONV_BF16) {
    rc = simple_fwd_conv<bf16>(s, cache, g->U, g->w0, x, y, stream);
  } else {
    rc = simple_fwd_conv<float>(s, cache, g->U, g->w0, x, y, stream);
  }
  if (rc) return rc;
  return launch_status();
}

int dynconv_decode(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x, void *state,
                   void *y, hipStream_t stream) {
  Shape s;
  int rc = check_problem(p, g, s);
  if (rc) return rc;
  if (p->T != 1) return DYNCONV_E_SHAPE;
  if (s.B == 0) return DYNCONV_OK;
  if (!h || !x || !y || (s.k > 1 && !state)) return DYNCONV_E_NULL;
  if ((rc = check_weights(s, g))) return rc;
  if (s.B > 65535) return DYNCONV_E_LIMIT;  // grid rows of four sequences stay far below the limit
  const void *ptrs[] = {h, x, y, state};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return DYNCONV_E_ALIGN;
  const int eb = p->dtype == DYNCONV_BF16 ? 2 : 4;
  const Sizes z = sizes(s, eb);
  const size_t st_bytes = s.k > 1 ? (size_t)s.B * (s.k - 1) * s.D * eb : 0;
  const Range ins[] = {{h, z.h}, {x, z.x}, {g->W, z.W}, {g->A, z.A}, {g->U, z.U}, {g->w0, g->w0 ? z.w0 : 0}};
  const Range outs[] = {{y, z.x}, {state, st_bytes}};
  for (const Range &o : outs)
    for (const Range &i : ins)
      if (overlap(o, i)) return DYNCONV_E_ALIAS;
  if (overlap(outs[0], outs[1])) return DYNCONV_E_ALIAS;
  rc = p->dtype == DYNCONV_BF16 ? decode_step<bf16>(s, h, g->W, g->A, g->U, g->w0, x, state, y, stream)
                                : decode_step<float>(s, h, g->W, g->A, g->U, g->w0, x, state, y, stream);
  if (rc) return rc;
  return launch_status();
}

int dynconv_bwd(const dynconv_problem *p, const dynconv_gen *g, const void *h, const void *x,
                const void *dy, const void *gen_cache, void *dx, void *dh,
                const dynconv_gen_grad *gg, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
  Shape s;
  int rc = check_problem(p, g, s);
  if (rc) return rc;
  if (!gg) return DYNCONV_E_NULL;
  if (s.kind == DYNCONV_HEADWISE && !gg->dW) return DYNCONV_E_NULL;
  if (s.kind == DYNCONV_LOWRANK && (!gg->dA || !gg->dU)) return DYNCONV_E_NULL;
  if ((rc = check_weights(s, g))) return rc;
  if (s.BT == 0) {
    // No tokens: the weight gradients are empty sums.  Written by a fill
    // kernel, not a memset, so that the call can sit inside a captured graph.
    const Sizes z0 = sizes(s, p->dtype == DYNCONV_BF16 ? 2 : 4);
    const void *gp[] = {gg->dW, gg->dA, gg->dU, gg->dw0};
    for (const void *q : gp)
      if (q && !aligned16(q)) return DYNCONV_E_ALIGN;
    zero_fill(gg->dW, z0.dW / sizeof(float), stream);
    zero_fill(gg->dA, z0.dA / sizeof(float), stream);
    zero_fill(gg->dU, z0.dU / sizeof(float), stream);
    zero_fill(gg->dw0, z0.dw0 / sizeof(float), stream);
    return launch_status();
  }
  if (!h || !x || !dy || !dx) return DYNCONV_E_NULL;
  const void *ptrs[] = {h, x, dy, gen_cache, dx, dh, workspace, gg->dW, gg->dA, gg->dU, gg->dw0};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return DYNCONV_E_ALIGN;
  const Plan pl = plan(s, p->dtype, 1);
  if (workspace_bytes < pl.total || (pl.total > 0 && !workspace)) return DYNCONV_E_WORKSPACE;
  const int eb = p->dtype == DYNCONV_BF16 ? 2 : 4;
  const Sizes z = sizes(s, eb);
  const Range ins[] = {{h, z.h},       {x, z.x},   {dy, z.x},  {gen_cache, gen_cache ? z.cache : 0},
                       {g->W, z.W},    {g->A, z.A}, {g->U, z.U}, {g->w0, g->w0 ? z.w0 : 0}};
  const Range outs[] = {{dx, z.x},          {dh, dh ? z.h : 0},     {gg->dW, gg->dW ? z.dW : 0},
                        {gg->dA, gg->dA ? z.dA : 0}, {gg->dU, gg->dU ? z.dU : 0},
                        {gg->dw0, gg->dw0 ? z.dw0 : 0}, {workspace, pl.total}};
  constexpr int n_out = sizeof(outs) / sizeof(outs[0]);
  for (const Range &o : outs)
    for (const Range &i : ins)
      if (overlap(o, i)) return DYNCONV_E_ALIAS;
  for (int a = 0; a < n_out; ++a)
    for (int b = a + 1; b < n_out; ++b)
      if (overlap(outs[a], outs[b])) return DYNCONV_E_ALIAS;
  const float *cache = (const float *)gen_cache;
  if (!cache) {
    float *c = (float *)((char *)workspace + pl.cache);
    if ((rc = gen_proj(s, p->dtype, g, h, c, workspace, pl, stream))) return rc;
    cache = c;
  }
  char *ws = (char *)workspace;
  if (fast_bwd(s, p->dtype)) {
    const BwdLayout L = bwd_layout(s);
    const GenBwdLayout G = gen_bwd_layout(s);
    float *gpart = (float *)(ws + pl.gpart), *dUp = (float *)(ws + pl.dup), *dw0p = (float *)(ws + pl.dw0p);
    rc = s.kind == DYNCONV_HEADWISE
             ? bwd_headwise(s, L, cache, g->w0, x, dy, dx, gpart, dw0p, stream)
             : bwd_lowrank(s, L, cache, g->U, g->w0, x, dy, dx, gpart, dUp, dw0p, stream);
    if (rc) return rc;
    const void *M = s.kind == DYNCONV_HEADWISE ? g->W : g->A;
    float *dMp = (float *)(ws + pl.dmp);
    if ((rc = gen_bwd(s, gpart, L.n_slices, L.R, L.Dt, h, M, (bf16 *)(ws + pl.g), (bf16 *)(ws + pl.mp), dh,
                      dMp, stream)))
      return rc;
    const int64_t Dk = s.D * s.k, dN = s.d * s.N;
    float *dM = s.kind == DYNCONV_HEADWISE ? gg->dW : gg->dA;
    if ((rc = finalize(dUp, s.kind == DYNCONV_LOWRANK ? gg->dU : nullptr, (int64_t)s.N * Dk, L.n_ranges,
                       dw0p, gg->dw0, Dk, L.n_ranges, dMp, dM, dN, G.n_ranges, stream)))
      return rc;
    return launch_status();
  }
  float *gbuf = (float *)(ws + pl.g);
  if (p->dtype == DYNCONV_BF16)
    rc = simple_bwd<bf16>(s, cache, g->W, g->A, g->U, g->w0, h, x, dy, dx, dh, *gg, gbuf, stream);
  else
    rc = simple_bwd<float>(s, cache, g->W, g->A, g->U, g->w0, h, x, dy, dx, dh, *gg, gbuf, stream);
  if (rc) return rc;
  return launch_status();
}

}  // extern "C"
