// C ABI of libdion3.so: argument checks, workspace layout and the launch
// schedule of the Dion3 step on one stream.  The contract of every entry
// point is stated in include/dion3.h.
#include <math.h>
#include <string.h>

#include "../../include/dion3.h"
#include "dion3_internal.h"

#include <utility>

using namespace dion3;

namespace {

thread_local int g_last_hip_error = 0;

dion3_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return DION3_ERR_HIP;
}

#define HIP_TRY(expr)                              \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e);     \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shapes of one group of B same-shape matrices (n x m, k selected rows).
// The selected rows X live in zero-padded fp16 blocks per matrix, both in
// rows layout [kp][mp] and transposed [mp][kp], so that every product reads
// K-contiguous operands; the Gram side s = min(k, m) pads to sp and the
// other side L = max(k, m) to Lp.  Zero padding is exact for Gram
// Newton-Schulz: the padded block stays decoupled from the real one and its
// output rows and columns are zero.
struct Shape {
  int B;
  long long n, m, k;
  bool tr;                 // k > m: the Gram is X^T X (s = m)
  long long kp, mp, sp, Lp;
};

Shape make_shape(int B, long long n, long long m, long long k) {
  Shape P;
  P.B = B; P.n = n; P.m = m; P.k = k;
  P.tr = k > m;
  P.kp = pad_to(k, kTile);
  P.mp = pad_to(m, kTile);
  P.sp = P.tr ? P.mp : P.kp;
  P.Lp = P.tr ? P.kp : P.mp;
  return P;
}

// Workspace regions of one group: fp64 l1 and sum of squares per row, the
// selected indices, the per-matrix scale and two X pairs (ping-pong for the
// restart).
struct GroupLayout {
  Shape P;
  size_t o_l1, o_sq, o_idx, o_scale, o_Xa, o_XaT, o_Xb, o_XbT;
  int side;              // its Gram-side set, or -1 (the fused path needs none)
  long long side_off;    // its first matrix inside that set
};

// Gram-side buffers R, Z, T, Q, Q' ([batch][sp][sp] fp16 each) of the groups
// whose Gram sides are equal (same s, hence same sp): their s x s products,
// the polynomial and the symmetric products of the level-2 paragraph, run
// as one launch over the matrices of all of them.
struct SideLayout {
  long long sp, s;
  int batch;
  size_t o_R, o_Z, o_T, o_Q0, o_Q1;
};

struct CallLayout {
  int ng, nside;
  GroupLayout g[DION3_MAX_GROUPS];
  SideLayout sd[DION3_MAX_GROUPS];
  size_t total;
};

long long side_of(const Shape& P) { return P.tr ? P.m : P.k; }

// Relative time of one s x s product launch over `batch` matrices of padded
// side sp, in rounds of 256-wide tiles over the 256 CUs: the launch takes the
// 256 tile from 512 such tiles on, else the 128 tile two per CU, whose round
// of 512 tiles (half the work of a 256 round) measured two thirds as long
// (symmetric products at side 1024: 29 us per small-tile round, 43.6 us per
// large-tile round).  Merging two groups' launches pays off only when it
// adds no more than that: the 1B and 14B sets share (-0.2 ms per step), and
// so does the 7B set at f = 1/4 (attention and down-projection groups, 1280
// + 320 tiles: 7 rounds merged against 5 plus a small-tile launch of 3
// small rounds apart, measured 0.2 ms per step faster merged).
double side_cost(long long sp, long long batch) {
  const long long t = (sp + 255) / 256, u = sp / 128;
  const long long big = t * (t + 1) / 2 * batch;
  if (big >= 512) return (double)((big + 255) / 256);
  const long long small = u * (u + 1) / 2 * batch;
  return 2.0 * (double)((small + 511) / 512) / 3.0;
}

// Regions in order: every group's rows and X pairs, then the side sets.  A
// group with no_side[g] set gets no side set; the others join a set of their
// Gram side when side_cost says the shared launches are no slower, else
// start a set of their own.
void make_layout(CallLayout& L, int ng, const Shape* shapes, const bool* no_side) {
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.ng = ng;
  L.nside = 0;
  for (int i = 0; i < ng; ++i) {
    GroupLayout& G = L.g[i];
    const Shape& P = shapes[i];
    G.P = P;
    G.o_l1 = take((size_t)P.B * P.n * 8);
    G.o_sq = take((size_t)P.B * P.n * 8);
    G.o_idx = take((size_t)P.B * P.k * 4);
    G.o_scale = take((size_t)P.B * 8);
    const size_t xb = (size_t)P.B * P.kp * P.mp * 2;
    G.o_Xa = take(xb);
    G.o_XaT = take(xb);
    G.o_Xb = take(xb);
    G.o_XbT = take(xb);
    G.side = -1;
    G.side_off = 0;
    if (no_side[i]) continue;
    int j = 0;
    while (j < L.nside &&
           !(L.sd[j].sp == P.sp && L.sd[j].s == side_of(P) &&
             side_cost(P.sp, L.sd[j].batch + P.B) <=
                 side_cost(P.sp, L.sd[j].batch) + side_cost(P.sp, P.B) + 1e-9))
      ++j;
    if (j == L.nside) {
      L.sd[j].sp = P.sp;
      L.sd[j].s = side_of(P);
      L.sd[j].batch = 0;
      ++L.nside;
    }
    G.side = j;
    G.side_off = L.sd[j].batch;
    L.sd[j].batch += P.B;
  }
  for (int j = 0; j < L.nside; ++j) {
    SideLayout& S = L.sd[j];
    const size_t sb = (size_t)S.batch * S.sp * S.sp * 2;
    S.o_R = take(sb);
    S.o_Z = take(sb);
    S.o_T = take(sb);
    S.o_Q0 = take(sb);
    S.o_Q1 = take(sb);
  }
  L.total = off;
}

// The layout of a one-group call: always with a side set, so that its size
// does not depend on the schedule (dion3_workspace_size takes no cfg).
void make_single_layout(CallLayout& L, int B, long long n, long long m, long long k) {
  const Shape P = make_shape(B, n, m, k);
  const bool no_side = false;
  make_layout(L, 1, &P, &no_side);
}

// Size checks of the step's entry points, in the order the header states:
// a size below 1 or k outside [1, n] is an argument error; only sizes that
// are valid but above DION3_MAX_DIM are unsupported.
dion3_status check_dims(long long n, long long m, long long k) {
  if (n < 1 || m < 1 || k < 1 || k > n) return DION3_ERR_ARG;
  if (n > DION3_MAX_DIM || m > DION3_MAX_DIM) return DION3_ERR_UNSUPPORTED;
  return DION3_OK;
}

// The products address each matrix through a buffer resource with 32-bit
// byte offsets, so every padded per-matrix operand must stay below 2^31 bytes.
constexpr long long kMaxOperandBytes = 1LL << 31;
// The grid of every product (128-wide tiles at most, times the batch) must
// also fit a launch, checked here so that no kernel runs before a refusal.
constexpr long long kMaxGrid = 0x7fffffffLL;
bool shape_fits(const Shape& P) {
  const long long ts = P.sp / kTile, tl = P.Lp / kTile;
  const long long tiles = ts * (ts + 1) / 2 > ts * tl ? ts * (ts + 1) / 2 : ts * tl;
  return P.kp * P.mp * 2 < kMaxOperandBytes && P.sp * P.sp * 2 < kMaxOperandBytes &&
         tiles * P.B <= kMaxGrid;
}
bool layout_fits(const CallLayout& L) {
  for (int i = 0; i < L.ng; ++i)
    if (!shape_fits(L.g[i].P)) return false;
  for (int j = 0; j < L.nside; ++j) {
    const long long ts = L.sd[j].sp / kTile;
    if (ts * (ts + 1) / 2 * L.sd[j].batch > kMaxGrid) return false;
  }
  return true;
}

dion3_status check_cfg(const dion3_ns_cfg* c) {
  if (c->iters < 1 || c->iters > DION3_MAX_ITERS) return DION3_ERR_ARG;
  if (c->n_restart < 0 || c->n_restart > DION3_MAX_RESTARTS) return DION3_ERR_ARG;
  int prev = 1;
  for (int i = 0; i < c->n_restart; ++i) {
    const int r = c->restart_at[i];
    if (r < 2 || r > c->iters || r <= prev) return DION3_ERR_ARG;
    prev = r;
  }
  if (!(c->eps >= 0.0f) || !isfinite(c->eps)) return DION3_ERR_ARG;
  if (c->method != DION3_NS_GRAM && c->method != DION3_NS_STANDARD) return DION3_ERR_ARG;
  if (c->path != DION3_PATH_AUTO && c->path != DION3_PATH_TILED && c->path != DION3_PATH_FUSED)
    return DION3_ERR_ARG;
  for (int t = 0; t < c->iters; ++t)
    for (int j = 0; j < 3; ++j)
      if (!isfinite(c->abc[t][j])) return DION3_ERR_ARG;
  return DION3_OK;
}

dion3_status check_norm(const dion3_norm_cfg* norm) {
  if (!(norm->beta2 >= 0.0f && norm->beta2 < 1.0f) || !(norm->eps >= 0.0f) || !isfinite(norm->eps))
    return DION3_ERR_ARG;
  return DION3_OK;
}

dion3_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ((uintptr_t)ws & 255) != 0) return DION3_ERR_WORKSPACE;
  if (ws_bytes < need) return DION3_ERR_WORKSPACE;
  return DION3_OK;
}

bool restart_at(const dion3_ns_cfg& c, int t) {
  for (int i = 0; i < c.n_restart; ++i)
    if (c.restart_at[i] == t) return true;
  return false;
}

// --------------------------------------------------------------- Gram NS

// A selected-row block's two layout slots, X [kp][mp] and XT [mp][kp] (the
// tiled Gram path fills only the one its products read; null when unused).
struct XPair {
  f16 *X, *XT;
};

double dbl(long long v) { return (double)v; }

// Unpadded Gram-side sizes: s = min(k, m), L = max(k, m).
double s_of(const Shape& P) { return dbl(P.tr ? P.m : P.k); }
double L_of(const Shape& P) { return dbl(P.tr ? P.k : P.m); }

// The Gram side works on X_math (sp x Lp): the selected rows when k <= m,
// their transpose when k > m.  Its row-form copy has row stride Lp and its
// transpose (Lp x sp) row stride sp.
// Inner dimension of a product over an unpadded extent: the padded
// operands are zero past it (the Gram-side cross terms between the real and
// the padded block are zero too), so only K steps that touch it are run.
int k_loop(double extent) { return (int)pad_to((long long)extent, kKStep); }

const f16* xmath(const Shape& P, const XPair& x) { return P.tr ? x.XT : x.X; }
const f16* xmathT(const Shape& P, const XPair& x) { return P.tr ? x.X : x.XT; }

// R = X_math X_math^T.
GemmDesc gram_desc(const Shape& P, const XPair& x, f16* R) {
  const double sv = s_of(P), L = L_of(P);
  GemmDesc d = {};
  d.trace_flops = P.B * sv * sv * L;
  d.trace_bytes = 2.0 * P.B * sv * (L + sv);          // read X, write R
  d.role = kRoleGram;
  d.A = d.B = xmath(P, x); d.sA = d.sB = P.kp * P.mp; d.lda = d.ldb = (int)P.Lp;
  d.C = R; d.sC = P.sp * P.sp; d.ldc = (int)P.sp;
  d.M = d.N = (int)P.sp; d.K = k_loop(L); d.batch = P.B;
  d.zrows = d.zcols = (int)sv;   // X_math's padding rows
  d.lower = true; d.epilogue = false;
  d.alpha = 1.0f;
  return d;
}

hipError_t gram(const Shape& P, const XPair& x, f16* R, hipStream_t s) {
  const GemmDesc d = gram_desc(P, x, R);
  return launch_gemm(d, s);
}

// Lower-triangle products of one kind for several groups or side sets, as
// few launches as kGemmMaxSeg allows; each launch takes the products with
// the longest tiles (largest inner dimension) first.
hipError_t launch_lower(GemmDesc* d, int n, hipStream_t s) {
  for (int i = 1; i < n; ++i)   // insertion sort, stable, by K descending
    for (int j = i; j > 0 && d[j].K > d[j - 1].K; --j) {
      const GemmDesc t = d[j];
      d[j] = d[j - 1];
      d[j - 1] = t;
    }
  for (int i = 0; i < n; i += kGemmMaxSeg) {
    const hipError_t e = launch_gemm_multi(d + i, n - i < kGemmMaxSeg ? n - i : kGemmMaxSeg, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// C = alpha A B + beta D + gamma I for symmetric commuting s x s matrices,
// over every matrix of a side set.
GemmDesc symm_desc(const SideLayout& S, const f16* A, const f16* B, const f16* D, f16* C,
                   float alpha, float beta, float gamma, bool epi) {
  const double sv = dbl(S.s);
  GemmDesc d = {};
  d.trace_flops = S.batch * sv * sv * sv;
  d.trace_bytes = (epi ? 4.0 : 6.0) * S.batch * sv * sv;   // read A (= B = D) or A and B, write C
  d.role = epi ? kRolePoly : kRoleSymm;
  const long long ss = S.sp * S.sp;
  d.A = A; d.sA = ss; d.lda = (int)S.sp;
  d.B = B; d.sB = ss; d.ldb = (int)S.sp;
  d.C = C; d.sC = ss; d.ldc = (int)S.sp;
  d.D = D; d.sD = ss; d.ldd = (int)S.sp;
  d.M = d.N = (int)S.sp; d.K = k_loop(sv); d.batch = S.batch;
  d.lower = true; d.epilogue = epi;
  d.alpha = alpha; d.beta = beta; d.gamma = gamma;
  d.gdiag = (int)sv;   // the identity of the unpadded Gram side only
  d.zrows = d.zcols = (int)sv;   // the padding block stays zero
  return d;
}

hipError_t symm(const SideLayout& S, const f16* A, const f16* B, const f16* D, f16* C, float alpha,
                float beta, float gamma, bool epi, hipStream_t s) {
  const GemmDesc d = symm_desc(S, A, B, D, C, alpha, beta, gamma, epi);
  return launch_gemm(d, s);
}

// Row-sparse update fused into the final product: W[idx[r]] -= lr * O[r]
// and, when requested, O_out = O (rows layout, unpadded).
struct UpdateSink {
  BatchPtr<float> W;
  long long ldw;
  const int* idx;
  float lr;
  f16* Oout;
  long long sO;   // elements between consecutive matrices' O blocks (>= k * m)
  // the rows' 128-column block sums of squares of O (per-neuron
  // normalization), written by the final product when its output rows are
  // the C pass (k <= m); ignored otherwise
  float* part;
};

void set_sink(GemmDesc& d, const Shape& P, const UpdateSink& sink) {
  // rows layout is the math layout when k <= m (the C pass) and its
  // transpose when k > m (the CT pass)
  d.sink = P.tr ? 2 : 1;
  d.C = nullptr;
  d.CT = nullptr;
  d.W = sink.W; d.ldw = sink.ldw; d.idx = sink.idx; d.lr = sink.lr; d.Oout = sink.Oout;
  d.sO = sink.sO;
  d.kval = (int)P.k; d.mval = (int)P.m; d.nrows = (int)P.n;
  if (!P.tr && sink.part) {
    d.part = sink.part;
    d.nblk = (int)((P.m + 127) / 128);
  }
}

// Y_math = Q X_math.  X_math (sp x Lp, the layout the Gram reads) is the
// product's second operand as it is, K x N with N contiguous, read through
// transposing LDS reads, so no kernel has to keep a transposed copy of X.
// The restart's Y_math is stored in the same layout for the next Gram.  The
// final product (sink set) stores nothing: its rows-layout output (the math
// layout when k <= m, its transpose when k > m) goes straight into the
// update of W (and O_out).
hipError_t rect(const Shape& P, const f16* Q, const XPair& x, const XPair& y, hipStream_t s,
                const UpdateSink* sink = nullptr) {
  const double sv = s_of(P), L = L_of(P);
  GemmDesc d = {};
  d.trace_flops = 2.0 * P.B * sv * sv * L;
  d.role = sink ? kRoleBack : kRoleRect;
  d.A = Q; d.sA = P.sp * P.sp; d.lda = (int)P.sp;
  d.B = xmath(P, x); d.sB = P.kp * P.mp; d.ldb = (int)P.Lp; d.b_kn = true;
  d.C = (f16*)xmath(P, y); d.sC = P.kp * P.mp; d.ldc = (int)P.Lp;
  if (sink) {
    set_sink(d, P, *sink);
    // read Q and X, read and write the selected rows of W (fp32), and write
    // O when asked
    const bool w = sink->W.ptrs || sink->W.base;
    d.trace_bytes = P.B * (2.0 * sv * sv + (2.0 + (w ? 8.0 : 0.0) + (sink->Oout ? 2.0 : 0.0)) * sv * L);
  } else {
    d.trace_bytes = P.B * (2.0 * sv * sv + 4.0 * sv * L);   // read Q and X, write Y
  }
  d.M = (int)P.sp; d.N = (int)P.Lp; d.K = k_loop(sv); d.batch = P.B;
  d.zrows = (int)sv; d.zcols = (int)L;   // Q's padding rows, X_math's padding columns
  d.lower = false; d.epilogue = false;
  d.alpha = 1.0f;
  return launch_gemm(d, s);
}

// Algorithmic flops of the whole Gram iteration on unpadded sizes, with the
// symmetric products counted at half (lower triangle), as the tiled
// launches record them.
double gram_ns_flops(const Shape& P, const dion3_ns_cfg& cfg) {
  const double sv = s_of(P), L = L_of(P), B = P.B;
  double f = B * sv * sv * L;               // first Gram
  bool q_identity = true;
  for (int t = 1; t <= cfg.iters; ++t) {
    if (restart_at(cfg, t)) {
      if (!q_identity) f += 2.0 * B * sv * sv * L;
      f += B * sv * sv * L;
      q_identity = true;
    }
    f += B * sv * sv * sv;                  // Z
    if (!q_identity) f += B * sv * sv * sv; // Q <- Z Q
    q_identity = false;
    if (t < cfg.iters && !restart_at(cfg, t + 1)) f += 2.0 * B * sv * sv * sv;
  }
  return f + 2.0 * B * sv * sv * L;         // O = Q X
}

// The fused one-launch path covers Gram sides that pad to one 128 tile.  It
// runs one workgroup per matrix, so its time grows with the row length L
// while the tiled launches spread long rows over many CUs.  Sides up to 64
// take the one-wave kernel, which gains most.  Measured on MI355X, one
// dion3_gram_ns call (us, fused / tiled): side 32: 32 / 136 at 1 x 32 x 512,
// 100 / 194 at 1 x 32 x 4096, 194 / 297 at 16 x 32 x 8192, 226 / 438 at 64 x
// 32 x 8192; side 64: 191 / 195 at 1 x 64 x 4096, 200 / 212 at 16 x 64 x
// 4096, 364 / 301 at 16 x 64 x 8192, 404 / 460 at 64 x 64 x 8192, 69 / 477 at
// 512 x 64 x 256; side 128: 113 / 152 at 1 x 128 x 1024, 171 / 168 at 1 x 128
// x 2048, 184 / 191 at 32 x 128 x 2048, 300 / 224 at 16 x 128 x 4096, 117 /
// 247 at 256 x 128 x 512.
bool use_fused(const Shape& P, const dion3_ns_cfg& cfg) {
  if (cfg.method != DION3_NS_GRAM) return false;
  if (cfg.path == DION3_PATH_TILED || P.sp != kTile) return false;
  if (cfg.path == DION3_PATH_FUSED) return true;
  const long long side = P.tr ? P.m : P.k;
  if (side <= 32) return P.Lp <= 8192;
  if (side <= 64) return P.Lp <= 4096 || (P.Lp <= 8192 && P.B >= 64);
  return P.Lp <= 1024 || (P.Lp <= 2048 && P.B >= 32);
}

// The fused path was asked for explicitly but the Gram side exceeds 128.
bool path_ok(const Shape& P, const dion3_ns_cfg& cfg) {
  return !(cfg.method == DION3_NS_GRAM && cfg.path == DION3_PATH_FUSED && P.sp != kTile);
}

// One group inside the orthogonalization: its layout, its current and free
// X pairs and where its result goes.
struct GroupRun {
  const GroupLayout* G;
  XPair x, xalt;
  UpdateSink sink;
};

void swap_pairs(GroupRun* r, int nr) {
  for (int i = 0; i < nr; ++i) {
    XPair t = r[i].x;
    r[i].x = r[i].xalt;
    r[i].xalt = t;
  }
}

// The Gram-side matrices of one group inside its set's buffer.
f16* slice(f16* base, const SideLayout& S, const GroupLayout& G) {
  return base + G.side_off * S.sp * S.sp;
}

// Gram Newton-Schulz on the normalized, padded X of every group of every
// side set ("Dion3: Full-Stack Orthogonal Updates", agihunt.info, level-1
// paragraph).  Every matrix here is a polynomial in the first Gram, so all
// products commute, are symmetric, and only their lower triangles are
// computed.  The sets run the same schedule in step: each s x s product is
// one launch over every set, and each Gram one launch over every group (the
// tails of several small launches become one).  The restart's X <- Q X and
// the final multiply-back run per group; the final product hands O to each
// group's sink.
struct SetRun {
  const SideLayout* S;
  GroupRun* r;
  int nr;
  f16 *R, *Z, *Tm, *Q, *Qn;
};

dion3_status gram_ns_sets(const dion3_ns_cfg& cfg, SetRun* set, int ns, hipStream_t s) {
  GemmDesc d[2 * DION3_MAX_GROUPS];   // up to two products per set in one launch
  auto grams = [&]() -> hipError_t {
    int n = 0;
    for (int j = 0; j < ns; ++j)
      for (int i = 0; i < set[j].nr; ++i) {
        const GroupRun& r = set[j].r[i];
        d[n++] = gram_desc(r.G->P, r.x, slice(set[j].R, *set[j].S, *r.G));
      }
    return launch_lower(d, n, s);
  };
  // one s x s product per set, C_j = alpha A_j B_j + beta D_j + gamma I,
  // appended to d[n..]
  auto add = [&](int& n, f16* SetRun::*A, f16* SetRun::*B, f16* SetRun::*D, f16* SetRun::*C,
                 float alpha, float beta, float gamma, bool epi) {
    for (int j = 0; j < ns; ++j)
      d[n++] = symm_desc(*set[j].S, set[j].*A, set[j].*B, D ? set[j].*D : nullptr, set[j].*C,
                         alpha, beta, gamma, epi);
  };
  auto sides = [&](f16* SetRun::*A, f16* SetRun::*B, f16* SetRun::*D, f16* SetRun::*C, float alpha,
                   float beta, float gamma, bool epi) -> hipError_t {
    int n = 0;
    add(n, A, B, D, C, alpha, beta, gamma, epi);
    return launch_lower(d, n, s);
  };
  HIP_TRY(grams());
  bool q_identity = true;
  const int T = cfg.iters;
  for (int t = 1; t <= T; ++t) {
    if (restart_at(cfg, t)) {      // X <- Q X, R <- X X^T, Q <- I
      if (!q_identity)
        for (int j = 0; j < ns; ++j) {
          for (int i = 0; i < set[j].nr; ++i) {
            GroupRun& r = set[j].r[i];
            HIP_TRY(rect(r.G->P, slice(set[j].Q, *set[j].S, *r.G), r.x, r.xalt, s));
          }
          swap_pairs(set[j].r, set[j].nr);
        }
      HIP_TRY(grams());
      q_identity = true;
    }
    const float a = cfg.abc[t - 1][0], b = cfg.abc[t - 1][1], c = cfg.abc[t - 1][2];
    // Z = a I + b R + c R^2  (the "A^2 + B" product)
    HIP_TRY(sides(&SetRun::R, &SetRun::R, &SetRun::R, &SetRun::Z, c, b, a, true));
    const bool next_r = t < T && !restart_at(cfg, t + 1);   // R <- Z R Z follows
    f16* SetRun::*Zv;
    if (q_identity) {           // Q <- Z Q with Q = I: just adopt Z
      for (int j = 0; j < ns; ++j) std::swap(set[j].Q, set[j].Z);
      Zv = &SetRun::Q;
      q_identity = false;
      if (next_r) HIP_TRY(sides(Zv, &SetRun::R, nullptr, &SetRun::Tm, 1.0f, 0.0f, 0.0f, false));
    } else {
      // Q' = Z Q, and T = Z R when R is updated too: independent products
      // that both read Z, one launch
      int n = 0;
      add(n, &SetRun::Z, &SetRun::Q, nullptr, &SetRun::Qn, 1.0f, 0.0f, 0.0f, false);
      if (next_r) add(n, &SetRun::Z, &SetRun::R, nullptr, &SetRun::Tm, 1.0f, 0.0f, 0.0f, false);
      HIP_TRY(launch_lower(d, n, s));
      for (int j = 0; j < ns; ++j) std::swap(set[j].Q, set[j].Qn);
      Zv = &SetRun::Z;
    }
    if (next_r) HIP_TRY(sides(&SetRun::Tm, Zv, nullptr, &SetRun::R, 1.0f, 0.0f, 0.0f, false));
  }
  for (int j = 0; j < ns; ++j)
    for (int i = 0; i < set[j].nr; ++i) {
      GroupRun& r = set[j].r[i];
      HIP_TRY(rect(r.G->P, slice(set[j].Q, *set[j].S, *r.G), r.x, r.xalt, s, &r.sink));
    }
  return DION3_OK;
}

// Standard quintic Newton-Schulz on X itself (the iteration the Gram form
// replaces, level-1 paragraph): A = X X^T, B = b A + c A^2, X <- a X + B X.
// The last update goes to `sink`.
hipError_t ns_update(const Shape& P, const f16* B, const XPair& x, const XPair& y, float a,
                     bool both, hipStream_t s, const UpdateSink* sink) {
  const double sv = s_of(P), L = L_of(P);
  GemmDesc d = {};
  d.trace_flops = 2.0 * P.B * sv * sv * L;
  d.trace_bytes = P.B * (2.0 * sv * sv + 4.0 * sv * L);
  d.role = kRoleNsX;
  d.A = B; d.sA = P.sp * P.sp; d.lda = (int)P.sp;
  d.B = xmathT(P, x); d.sB = P.kp * P.mp; d.ldb = (int)P.sp;
  d.D = xmathT(P, x); d.sD = P.kp * P.mp; d.ldd = (int)P.sp;   // a X, read transposed
  d.epilogue = true; d.alpha = 1.0f; d.beta = a; d.gamma = 0.0f;
  const bool want_math = both || !P.tr, want_mathT = both || P.tr;
  d.C = want_math ? (f16*)xmath(P, y) : nullptr; d.sC = P.kp * P.mp; d.ldc = (int)P.Lp;
  d.CT = want_mathT ? (f16*)xmathT(P, y) : nullptr; d.sCT = P.kp * P.mp; d.ldct = (int)P.sp;
  if (sink) set_sink(d, P, *sink);
  d.M = (int)P.sp; d.N = (int)P.Lp; d.K = (int)P.sp; d.batch = P.B;
  return launch_gemm(d, s);
}

dion3_status standard_ns_set(const dion3_ns_cfg& cfg, const SideLayout& S, char* w, GroupRun* r,
                             int nr, hipStream_t s) {
  f16 *R = (f16*)(w + S.o_R), *Z = (f16*)(w + S.o_Z);
  for (int t = 1; t <= cfg.iters; ++t) {
    const float a = cfg.abc[t - 1][0], b = cfg.abc[t - 1][1], c = cfg.abc[t - 1][2];
    for (int i = 0; i < nr; ++i) HIP_TRY(gram(r[i].G->P, r[i].x, slice(R, S, *r[i].G), s));  // A = X X^T
    HIP_TRY(symm(S, R, R, R, Z, c, b, 0.0f, true, s));                                        // B = b A + c A^2
    const bool last = t == cfg.iters;
    for (int i = 0; i < nr; ++i)
      HIP_TRY(ns_update(r[i].G->P, slice(Z, S, *r[i].G), r[i].x, r[i].xalt, a, !last, s,
                        last ? &r[i].sink : nullptr));
    if (!last) swap_pairs(r, nr);
  }
  return DION3_OK;
}

// The orthogonalization of every group of a call: groups on the fused
// path one launch each, then each side set with its member groups.
dion3_status orthogonalize(const CallLayout& L, const dion3_ns_cfg& cfg, char* w, GroupRun* runs,
                           hipStream_t s) {
  for (int i = 0; i < L.ng; ++i) {
    const Shape& P = L.g[i].P;
    if (!use_fused(P, cfg)) continue;
    const GroupRun& r = runs[i];
    HIP_TRY(launch_gram_ns_small((f16*)xmath(P, r.x), (f16*)xmathT(P, r.x), (f16*)xmath(P, r.xalt),
                                 (f16*)xmathT(P, r.xalt), P.kp * P.mp, P.B, (int)P.Lp, P.tr, cfg,
                                 r.sink.W, r.sink.ldw, r.sink.idx, r.sink.lr, r.sink.Oout,
                                 r.sink.sO, (int)P.k, (int)P.m, (int)P.n, gram_ns_flops(P, cfg),
                                 s));
  }
  GroupRun members[DION3_MAX_GROUPS];
  SetRun sets[DION3_MAX_GROUPS];
  int nm = 0, ns = 0;
  for (int j = 0; j < L.nside; ++j) {
    GroupRun* first = members + nm;
    for (int i = 0; i < L.ng; ++i)
      if (L.g[i].side == j && !use_fused(L.g[i].P, cfg)) members[nm++] = runs[i];
    const int nr = (int)(members + nm - first);
    if (nr == 0) continue;
    if (cfg.method == DION3_NS_STANDARD) {
      const dion3_status st = standard_ns_set(cfg, L.sd[j], w, first, nr, s);
      if (st != DION3_OK) return st;
      continue;
    }
    const SideLayout& S = L.sd[j];
    sets[ns++] = {&S, first, nr, (f16*)(w + S.o_R), (f16*)(w + S.o_Z), (f16*)(w + S.o_T),
                  (f16*)(w + S.o_Q0), (f16*)(w + S.o_Q1)};
  }
  return ns ? gram_ns_sets(cfg, sets, ns, s) : DION3_OK;
}

// The X pair that the orthogonalization no longer reads once it has started
// its last product: every restart (Gram) or every iteration but the last
// (standard) swaps the two pairs, starting from the first.
bool free_pair_is_b(const dion3_ns_cfg& cfg) {
  const int swaps = cfg.method == DION3_NS_STANDARD ? cfg.iters - 1 : cfg.n_restart;
  return swaps % 2 == 0;
}

XPair pair_a(const GroupLayout& G, char* w) { return {(f16*)(w + G.o_Xa), (f16*)(w + G.o_XaT)}; }

// The layouts of the selected rows that the orthogonalization reads: the
// tiled Gram iteration and the one-wave fused kernel (Gram sides up to 64)
// read only X_math (rows when k <= m, their transpose when k > m); the
// 128-padded fused kernel and the standard iteration read both.  The gather
// writes only those (a null pointer skips a layout).
XPair gather_layouts(const Shape& P, const dion3_ns_cfg& cfg, const XPair& x) {
  const long long side = P.tr ? P.m : P.k;
  if (cfg.method == DION3_NS_STANDARD || (use_fused(P, cfg) && side > 64)) return x;
  return P.tr ? XPair{nullptr, x.XT} : XPair{x.X, nullptr};
}
XPair pair_b(const GroupLayout& G, char* w) { return {(f16*)(w + G.o_Xb), (f16*)(w + G.o_XbT)}; }

// One group's arguments in a step call.
struct GroupArgs {
  BatchPtr<float> W, M;
  BatchPtr<const float> G;   // gradients accumulated first, or none
  BatchPtr<float> V;         // per-neuron normalization state, or none
  long long ld;
  float lr;
  int32_t* idx_out;
  uint16_t* O_out;
};

// The whole step for every group of a call: rows (score, select, gather
// with decay) group by group, the orthogonalization, then the per-neuron
// normalization (when `norm` is set) and the index copies.  Every check has
// been made before this runs.
dion3_status run_step(const CallLayout& L, const GroupArgs* A, float mu, const dion3_ns_cfg& cfg,
                      const dion3_norm_cfg* norm, char* w, hipStream_t s) {
  TraceChain chain(s);
  GroupRun runs[DION3_MAX_GROUPS];
  for (int i = 0; i < L.ng; ++i) {
    const GroupLayout& G = L.g[i];
    const Shape& P = G.P;
    const GroupArgs& a = A[i];
    double* l1 = (double*)(w + G.o_l1);
    double* sq = (double*)(w + G.o_sq);
    int* idx = (int*)(w + G.o_idx);
    double* scale = (double*)(w + G.o_scale);
    const bool all = (P.k == P.n);
    const double Bd = P.B, nm = dbl(P.n) * dbl(P.m), km = dbl(P.k) * dbl(P.m);
    const int n = (int)P.n, m = (int)P.m, k = (int)P.k;
    BatchPtr<const float> Mc = {a.M.base, a.M.stride, (const float* const*)a.M.ptrs};
    if (a.G.base || a.G.ptrs) {   // accumulate the gradient into the buffer while scoring
      TraceScope ts("accum_score", 0.0, Bd * nm * 12.0, s);
      HIP_TRY(launch_accum_score_f32(a.M, a.G, P.B, n, m, a.ld, all ? nullptr : l1, sq, s));
    } else {
      TraceScope ts("row_score", 0.0, Bd * nm * 4.0, s);
      HIP_TRY(launch_row_score_f32(Mc, P.B, n, m, a.ld, all ? nullptr : l1, sq, s));
    }
    {
      TraceScope ts("topk", 0.0, Bd * dbl(P.n) * 16.0, s);
      HIP_TRY(launch_topk(l1, sq, P.B, n, k, idx, scale, (double)cfg.eps, s));
    }
    const XPair xa = pair_a(G, w), xb = pair_b(G, w);
    {
      const XPair out = gather_layouts(P, cfg, xa);
      // the rows-only gather is a kernel of its own (k_gather_rows)
      TraceScope ts(out.XT ? "gather" : "gather_rows", 0.0, Bd * km * 10.0, s);
      HIP_TRY(launch_gather_f32(a.M, P.B, n, m, a.ld, idx, k, scale, mu, true, out.X, out.XT,
                                P.kp * P.mp, (int)P.kp, (int)P.mp, s));
    }
    GroupRun& r = runs[i];
    r.G = &G;
    r.x = xa;
    r.xalt = xb;
    if (!norm) {
      r.sink = {a.W, a.ld, idx, a.lr, (f16*)a.O_out, P.k * P.m, nullptr};
    } else {
      // O into the free X buffer, each matrix's rows [k][m] inside that
      // matrix's own padded block (so that in the fused one-launch path no
      // workgroup writes where another matrix may still be read), and the
      // rows' block sums of squares into the free pair's other buffer, which
      // no product of this call reads
      const XPair& fp = free_pair_is_b(cfg) ? xb : xa;
      r.sink = {{nullptr, 0, nullptr}, 0, idx, a.lr, fp.X, P.kp * P.mp, (float*)fp.XT};
    }
  }
  dion3_status st = orthogonalize(L, cfg, w, runs, s);
  if (st != DION3_OK) return st;
  for (int i = 0; i < L.ng; ++i) {
    const GroupLayout& G = L.g[i];
    const Shape& P = G.P;
    const GroupArgs& a = A[i];
    int* idx = (int*)(w + G.o_idx);
    if (norm) {
      // the row statistics reuse the score region and the per-matrix scale
      // the norm region
      const f16* Obuf = runs[i].sink.Oout;
      const long long sO = runs[i].sink.sO;
      // the tiled final product wrote the block sums already when its
      // output rows are O's rows (k <= m); the fused kernel does not
      const bool part_ready = !P.tr && !use_fused(P, cfg);
      HIP_TRY(launch_normalize(Obuf, sO, P.B, (int)P.k, (int)P.m, idx, a.V, norm->beta2, norm->eps,
                               a.W, a.ld, a.lr, runs[i].sink.part, part_ready,
                               (float2*)(w + G.o_l1), s));
      if (a.O_out) {
        trace_break();   // an untimed copy between timed kernels
        HIP_TRY(hipMemcpy2DAsync(a.O_out, (size_t)P.k * P.m * sizeof(uint16_t), Obuf,
                                 (size_t)sO * sizeof(uint16_t), (size_t)P.k * P.m * sizeof(uint16_t),
                                 (size_t)P.B, hipMemcpyDeviceToDevice, s));
      }
    }
    if (a.idx_out) {
      trace_break();
      HIP_TRY(hipMemcpyAsync(a.idx_out, idx, (size_t)P.B * P.k * sizeof(int32_t),
                             hipMemcpyDeviceToDevice, s));
    }
  }
  return DION3_OK;
}

// The checks shared by every one-group step entry point, then the step.
dion3_status step_one(const GroupArgs& a, int batch, long long n, long long m, long long k,
                      float mu, const dion3_ns_cfg* cfg_in, const dion3_norm_cfg* norm, void* ws,
                      size_t ws_bytes, void* stream) {
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  if (norm && (!(a.V.base || a.V.ptrs) || check_norm(norm) != DION3_OK)) return DION3_ERR_ARG;
  dion3_status st = check_dims(n, m, k);
  if (st != DION3_OK) return st;
  if (a.ld < m) return DION3_ERR_ARG;
  if (!isfinite(a.lr) || !isfinite(mu)) return DION3_ERR_ARG;
  dion3_ns_cfg cfg;
  if (cfg_in) cfg = *cfg_in; else dion3_ns_cfg_default(&cfg);
  st = check_cfg(&cfg);
  if (st != DION3_OK) return st;
  CallLayout L;
  make_single_layout(L, batch, n, m, k);
  if (!layout_fits(L) || !path_ok(L.g[0].P, cfg)) return DION3_ERR_UNSUPPORTED;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != DION3_OK) return st;
  return run_step(L, &a, mu, cfg, norm, (char*)ws, (hipStream_t)stream);
}

// Layout of a grouped call.  Groups that take the fused path get no side set;
// the others share one per Gram side where side_cost says so.
dion3_status group_layout(CallLayout& L, const dion3_group* groups, int32_t ngroups,
                          const dion3_ns_cfg& cfg) {
  if (!groups || ngroups < 1 || ngroups > DION3_MAX_GROUPS) return DION3_ERR_ARG;
  Shape shapes[DION3_MAX_GROUPS];
  bool no_side[DION3_MAX_GROUPS];
  dion3_status worst = DION3_OK;
  for (int i = 0; i < ngroups; ++i) {
    const dion3_group& g = groups[i];
    if (g.batch < 1 || g.batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
    const dion3_status st = check_dims(g.n, g.m, g.k);
    if (st == DION3_ERR_ARG) return st;
    if (st != DION3_OK) worst = st;
    if (g.ld < g.m) return DION3_ERR_ARG;
  }
  if (worst != DION3_OK) return worst;
  for (int i = 0; i < ngroups; ++i) {
    shapes[i] = make_shape(groups[i].batch, groups[i].n, groups[i].m, groups[i].k);
    if (!path_ok(shapes[i], cfg)) return DION3_ERR_UNSUPPORTED;
    no_side[i] = use_fused(shapes[i], cfg);
  }
  make_layout(L, ngroups, shapes, no_side);
  return layout_fits(L) ? DION3_OK : DION3_ERR_UNSUPPORTED;
}

// Best rational approximation p/q of x = mant / 2^e with q <= qmax
// (continued-fraction convergents and the last semiconvergent).
void best_rational(unsigned long long mant, int e, unsigned long long qmax,
                   unsigned long long* pp, unsigned long long* qq) {
  typedef unsigned __int128 u128;
  const u128 num0 = mant, den0 = (u128)1 << e;
  if (den0 <= qmax) {
    u128 g = num0, h = den0;
    while (h) { u128 t = g % h; g = h; h = t; }
    *pp = (unsigned long long)(num0 / g);
    *qq = (unsigned long long)(den0 / g);
    return;
  }
  u128 p0 = 0, q0 = 1, p1 = 1, q1 = 0, nn = num0, dd = den0;
  for (;;) {
    const u128 a = nn / dd;
    const u128 q2 = q0 + a * q1;
    if (q2 > qmax) break;
    const u128 p2 = p0 + a * p1;
    p0 = p1; q0 = q1; p1 = p2; q1 = q2;
    const u128 r = nn - a * dd;
    nn = dd; dd = r;
    if (dd == 0) break;
  }
  const u128 j = (qmax - q0) / q1;
  const u128 pb = p0 + j * p1, qb = q0 + j * q1;
  // |p/q - x| = |p 2^e - mant q| / (q 2^e); compare the two candidates.
  auto dist = [&](u128 p, u128 q) {
    const u128 lhs = p * den0, rhs = num0 * q;
    return lhs > rhs ? lhs - rhs : rhs - lhs;
  };
  const u128 d1 = dist(p1, q1), db = dist(pb, qb);
  if (d1 * qb <= db * q1) { *pp = (unsigned long long)p1; *qq = (unsigned long long)q1; }
  else { *pp = (unsigned long long)pb; *qq = (unsigned long long)qb; }
}

}  // namespace

namespace dion3 {
dion3_status note_hip_error(hipError_t e) { return hip_fail(e); }
}  // namespace dion3

extern "C" {

int dion3_version(void) { return 1; }

size_t dion3_ns_cfg_size(void) { return sizeof(dion3_ns_cfg); }

void dion3_ns_cfg_default(dion3_ns_cfg* cfg) {
  if (!cfg) return;
  memset(cfg, 0, sizeof(*cfg));
  cfg->iters = 5;
  cfg->n_restart = 1;
  cfg->restart_at[0] = 3;
  for (int t = 0; t < DION3_MAX_ITERS; ++t) {
    cfg->abc[t][0] = 3.4445f;
    cfg->abc[t][1] = -4.7750f;
    cfg->abc[t][2] = 2.0315f;
  }
  cfg->eps = 1e-7f;
}

int64_t dion3_k_from_fraction(double f, int64_t n) {
  if (n < 1 || !(f > 0.0) || !isfinite(f)) return -1;
  if (f >= 1.0) return n;
  const unsigned long long qmax = 1ull << 20;
  unsigned long long p, q;
  if (f < ldexp(1.0, -21)) {          // nearer to 0/1 than to 1/2^20
    p = 0; q = 1;
  } else {
    int ex;
    const double fr = frexp(f, &ex);  // f = fr * 2^ex, fr in [0.5, 1)
    unsigned long long mant = (unsigned long long)ldexp(fr, 53);
    int e = 53 - ex;                  // f = mant / 2^e, e <= 74
    while (e > 0 && (mant & 1ull) == 0) { mant >>= 1; --e; }
    best_rational(mant, e, qmax, &p, &q);
  }
  const unsigned __int128 num = (unsigned __int128)p * (unsigned long long)n;
  unsigned __int128 k = (num + q - 1) / q;
  if (k < 1) k = 1;
  if (k > (unsigned __int128)n) k = n;
  return (int64_t)k;
}

dion3_status dion3_workspace_size(int32_t batch, int64_t n, int64_t m, int64_t k, size_t* bytes) {
  if (!bytes) return DION3_ERR_ARG;
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  const dion3_status st = check_dims(n, m, k);
  if (st != DION3_OK) return st;
  CallLayout L;
  make_single_layout(L, batch, n, m, k);
  if (!layout_fits(L)) return DION3_ERR_UNSUPPORTED;
  *bytes = L.total;
  return DION3_OK;
}

dion3_status dion3_row_select(const float* M, int32_t batch, int64_t n, int64_t m, int64_t ld,
                              int64_t k, int32_t* idx, double* scores, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!M || !idx) return DION3_ERR_ARG;
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  dion3_status st = check_dims(n, m, k);
  if (st != DION3_OK) return st;
  if (ld < m) return DION3_ERR_ARG;
  CallLayout L;
  make_single_layout(L, batch, n, m, k);
  const GroupLayout& G = L.g[0];
  st = check_ws(ws, ws_bytes, G.o_Xa);   // the row regions only
  if (st != DION3_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  double* l1 = (double*)(w + G.o_l1);
  double* sq = (double*)(w + G.o_sq);
  double* scale = (double*)(w + G.o_scale);
  BatchPtr<const float> Mb = {M, n * ld, nullptr};
  HIP_TRY(launch_row_score_f32(Mb, batch, (int)n, (int)m, ld, l1, sq, s));
  HIP_TRY(launch_topk(l1, sq, batch, (int)n, (int)k, idx, scale, 0.0, s));
  if (scores)
    HIP_TRY(hipMemcpyAsync(scores, l1, (size_t)batch * n * sizeof(double), hipMemcpyDeviceToDevice,
                           s));
  return DION3_OK;
}

dion3_status dion3_gram_ns(const uint16_t* X, uint16_t* O, int32_t batch, int64_t k, int64_t m,
                           const dion3_ns_cfg* cfg_in, void* ws, size_t ws_bytes, void* stream) {
  if (!X || !O) return DION3_ERR_ARG;
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  dion3_status st = check_dims(k, m, k);
  if (st != DION3_OK) return st;
  dion3_ns_cfg cfg;
  if (cfg_in) cfg = *cfg_in; else dion3_ns_cfg_default(&cfg);
  st = check_cfg(&cfg);
  if (st != DION3_OK) return st;
  CallLayout L;
  make_single_layout(L, batch, k, m, k);
  const GroupLayout& G = L.g[0];
  if (!layout_fits(L) || !path_ok(G.P, cfg)) return DION3_ERR_UNSUPPORTED;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != DION3_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  double* sq = (double*)(w + G.o_sq);
  int* idx = (int*)(w + G.o_idx);
  double* scale = (double*)(w + G.o_scale);
  const XPair xa = pair_a(G, w), xb = pair_b(G, w);
  BatchPtr<const f16> Xb = {(const f16*)X, k * m, nullptr};
  HIP_TRY(launch_row_score_f16(Xb, batch, (int)k, (int)m, m, sq, s));
  HIP_TRY(launch_topk(nullptr, sq, batch, (int)k, (int)k, idx, scale, (double)cfg.eps, s));
  const XPair out = gather_layouts(G.P, cfg, xa);
  HIP_TRY(launch_gather_f16(Xb, batch, (int)m, m, (int)k, scale, out.X, out.XT, G.P.kp * G.P.mp,
                            (int)G.P.kp, (int)G.P.mp, s));
  GroupRun r;
  r.G = &G;
  r.x = xa;
  r.xalt = xb;
  r.sink = {{nullptr, 0, nullptr}, 0, idx, 0.0f, (f16*)O, k * m, nullptr};
  TraceChain chain(s);   // (the untimed kernels above are all enqueued)
  return orthogonalize(L, cfg, w, &r, s);
}

dion3_status dion3_step(float* W, float* M, int64_t n, int64_t m, int64_t ld, int64_t k, float lr,
                        float mu, const dion3_ns_cfg* cfg, int32_t* idx_out, uint16_t* O_out,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!W || !M) return DION3_ERR_ARG;
  const GroupArgs a = {{W, 0, nullptr}, {M, 0, nullptr}, {nullptr, 0, nullptr},
                       {nullptr, 0, nullptr}, ld, lr, idx_out, O_out};
  return step_one(a, 1, n, m, k, mu, cfg, nullptr, ws, ws_bytes, stream);
}

dion3_status dion3_step_accum(float* W, float* M, const float* G, int64_t n, int64_t m, int64_t ld,
                              int64_t k, float lr, float mu, const dion3_ns_cfg* cfg,
                              int32_t* idx_out, uint16_t* O_out, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!W || !M || !G) return DION3_ERR_ARG;
  const GroupArgs a = {{W, 0, nullptr}, {M, 0, nullptr}, {G, 0, nullptr},
                       {nullptr, 0, nullptr}, ld, lr, idx_out, O_out};
  return step_one(a, 1, n, m, k, mu, cfg, nullptr, ws, ws_bytes, stream);
}

dion3_status dion3_step_megabatch(float* const* W, float* const* M, int32_t batch, int64_t n,
                                  int64_t m, int64_t ld, int64_t k, float lr, float mu,
                                  const dion3_ns_cfg* cfg, int32_t* idx_out, uint16_t* O_out,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (!W || !M) return DION3_ERR_ARG;
  const GroupArgs a = {{nullptr, 0, W}, {nullptr, 0, M}, {nullptr, 0, nullptr},
                       {nullptr, 0, nullptr}, ld, lr, idx_out, O_out};
  return step_one(a, batch, n, m, k, mu, cfg, nullptr, ws, ws_bytes, stream);
}

dion3_status dion3_step_megabatch_accum(float* const* W, float* const* M, const float* const* G,
                                        int32_t batch, int64_t n, int64_t m, int64_t ld, int64_t k,
                                        float lr, float mu, const dion3_ns_cfg* cfg,
                                        int32_t* idx_out, uint16_t* O_out, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (!W || !M || !G) return DION3_ERR_ARG;
  const GroupArgs a = {{nullptr, 0, W}, {nullptr, 0, M}, {nullptr, 0, G},
                       {nullptr, 0, nullptr}, ld, lr, idx_out, O_out};
  return step_one(a, batch, n, m, k, mu, cfg, nullptr, ws, ws_bytes, stream);
}

dion3_status dion3_step_megabatch_norm(float* const* W, float* const* M, const float* const* G,
                                       float* const* V, int32_t batch, int64_t n, int64_t m,
                                       int64_t ld, int64_t k, float lr, float mu,
                                       const dion3_ns_cfg* cfg, const dion3_norm_cfg* norm,
                                       int32_t* idx_out, uint16_t* O_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!W || !M || !V || !norm) return DION3_ERR_ARG;
  const GroupArgs a = {{nullptr, 0, W}, {nullptr, 0, M}, {nullptr, 0, G},
                       {nullptr, 0, V}, ld, lr, idx_out, O_out};
  return step_one(a, batch, n, m, k, mu, cfg, norm, ws, ws_bytes, stream);
}

size_t dion3_group_size(void) { return sizeof(dion3_group); }

dion3_status dion3_workspace_size_groups(const dion3_group* groups, int32_t ngroups,
                                         const dion3_ns_cfg* cfg_in, size_t* bytes) {
  if (!bytes) return DION3_ERR_ARG;
  dion3_ns_cfg cfg;
  if (cfg_in) cfg = *cfg_in; else dion3_ns_cfg_default(&cfg);
  dion3_status st = check_cfg(&cfg);
  if (st != DION3_OK) return st;
  CallLayout L;
  st = group_layout(L, groups, ngroups, cfg);
  if (st != DION3_OK) return st;
  *bytes = L.total;
  return DION3_OK;
}

dion3_status dion3_step_groups(const dion3_group* groups, int32_t ngroups, float mu,
                               const dion3_ns_cfg* cfg_in, const dion3_norm_cfg* norm, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!groups || ngroups < 1 || ngroups > DION3_MAX_GROUPS) return DION3_ERR_ARG;
  if (!isfinite(mu)) return DION3_ERR_ARG;
  if (norm && check_norm(norm) != DION3_OK) return DION3_ERR_ARG;
  GroupArgs A[DION3_MAX_GROUPS];
  for (int i = 0; i < ngroups; ++i) {
    const dion3_group& g = groups[i];
    if (!g.W || !g.M || !isfinite(g.lr) || (norm && !g.V)) return DION3_ERR_ARG;
    A[i] = {{nullptr, 0, g.W}, {nullptr, 0, g.M}, {nullptr, 0, g.G}, {nullptr, 0, g.V},
            g.ld, g.lr, g.idx_out, g.O_out};
  }
  dion3_ns_cfg cfg;
  if (cfg_in) cfg = *cfg_in; else dion3_ns_cfg_default(&cfg);
  dion3_status st = check_cfg(&cfg);
  if (st != DION3_OK) return st;
  CallLayout L;
  st = group_layout(L, groups, ngroups, cfg);
  if (st != DION3_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != DION3_OK) return st;
  return run_step(L, A, mu, cfg, norm, (char*)ws, (hipStream_t)stream);
}

dion3_status dion3_syrk_f16(const uint16_t* A, uint16_t* R, int32_t batch, int64_t rows,
                            int64_t cols, int64_t lda, int64_t ldr, void* stream) {
  if (!A || !R) return DION3_ERR_ARG;
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  if (rows < 1 || cols < 1) return DION3_ERR_ARG;
  if (rows > DION3_MAX_DIM || cols > DION3_MAX_DIM) return DION3_ERR_UNSUPPORTED;
  if (rows % kTile || cols % kTile || lda < cols || ldr < rows || lda % 8 || ldr % 8)
    return DION3_ERR_ARG;
  if (rows * lda * 2 >= kMaxOperandBytes || rows * ldr * 2 >= kMaxOperandBytes)
    return DION3_ERR_UNSUPPORTED;
  if (((uintptr_t)A | (uintptr_t)R) & 15) return DION3_ERR_ARG;
  GemmDesc d = {};
  d.role = kRoleGram;
  d.trace_flops = (double)batch * rows * rows * cols;
  d.A = (const f16*)A; d.sA = rows * lda; d.lda = (int)lda;
  d.B = (const f16*)A; d.sB = rows * lda; d.ldb = (int)lda;
  d.C = (f16*)R; d.sC = rows * ldr; d.ldc = (int)ldr;
  d.M = d.N = (int)rows; d.K = (int)cols; d.batch = batch;
  d.lower = true; d.alpha = 1.0f;
  HIP_TRY(launch_gemm(d, (hipStream_t)stream));
  return DION3_OK;
}

dion3_status dion3_symm_f16(const uint16_t* A, const uint16_t* B, const uint16_t* D, uint16_t* C,
                            int32_t batch, int64_t s, int64_t ld, float alpha, float beta,
                            float gamma, void* stream) {
  if (!A || !B || !C || (beta != 0.0f && !D)) return DION3_ERR_ARG;
  if (batch < 1 || batch > DION3_MAX_BATCH) return DION3_ERR_ARG;
  if (s < 1) return DION3_ERR_ARG;
  if (s > DION3_MAX_DIM) return DION3_ERR_UNSUPPORTED;
  if (s % kTile || ld < s || ld % 8) return DION3_ERR_ARG;
  if (s * ld * 2 >= kMaxOperandBytes) return DION3_ERR_UNSUPPORTED;
  if (!isfinite(alpha) || !isfinite(beta) || !isfinite(gamma)) return DION3_ERR_ARG;
  if (C == A || C == B || (D && C == D)) return DION3_ERR_ARG;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C | (uintptr_t)D) & 15) return DION3_ERR_ARG;
  GemmDesc d = {};
  d.role = kRolePoly;
  d.trace_flops = (double)batch * s * s * s;
  const long long ss = s * ld;
  d.A = (const f16*)A; d.sA = ss; d.lda = (int)ld;
  d.B = (const f16*)B; d.sB = ss; d.ldb = (int)ld;
  d.C = (f16*)C; d.sC = ss; d.ldc = (int)ld;
  d.D = beta != 0.0f ? (const f16*)D : nullptr; d.sD = ss; d.ldd = (int)ld;
  d.M = d.N = d.K = (int)s; d.batch = batch;
  d.lower = true; d.epilogue = true;
  d.alpha = alpha; d.beta = beta; d.gamma = gamma;
  HIP_TRY(launch_gemm(d, (hipStream_t)stream));
  return DION3_OK;
}

const char* dion3_status_string(dion3_status st) {
  switch (st) {
    case DION3_OK: return "ok";
    case DION3_ERR_ARG: return "invalid argument";
    case DION3_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DION3_ERR_UNSUPPORTED: return "shape beyond the library's limits";
    case DION3_ERR_HIP: return "HIP call or kernel launch failed";
  }
  return "unknown status";
}

int dion3_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
