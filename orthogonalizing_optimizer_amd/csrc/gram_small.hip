// Whole Gram Newton-Schulz in one workgroup per matrix, for Gram sides of at
// most 128 ("Dion3: Full-Stack Orthogonal Updates", agihunt.info, level-1
// paragraph): k_gram_ns_small (described here) pads the side to 128;
// k_gram_ns_tiny (further down) takes sides up to 64 with one wave running
// the s x s products.  Small matrices would otherwise pay one launch per product
// (about 20 per step, each a few microseconds of fixed cost); here R, Z, Q
// and T stay in LDS (4 x 34 KB), 64-wide K slices of X stream through an
// 18 KB staging buffer with a register prefetch of several slices, and the final
// product feeds the row-sparse update directly (its output blocks staged in
// the LDS matrices that are free by then).
//
// 4 waves in a 2 x 2 grid over the 128 x 128 output, each wave 64 x 64 as
// 2 x 2 v_mfma_f32_32x32x16_f16.  Every element accumulates its k-slices in
// increasing order and goes through the same fp32 epilogue as the tiled
// kernels, and each symmetric result takes at (i, j) and (j, i) the value
// the tiled kernels compute for the lower triangle, so the result equals
// the tiled path bit for bit.  Symmetric outputs are written without a
// mirror pass: the lower-left wave stores its block transposed (one 8-byte
// run per 4 accumulators) into the upper-right quadrant, the upper-right
// wave computes the lower-left block with its operands exchanged (exact
// fp16 products commute) and stores it transposed into the lower-left
// quadrant, and the two diagonal waves store their lower triangles both
// ways.
#include "../../include/dion3.h"
#include "dion3_internal.h"

namespace dion3 {
namespace {

constexpr int S = 128;           // padded Gram side
constexpr int SL = S + 8;        // LDS row stride of the s x s matrices (halves)
constexpr int BK = 64;           // K slice of X
constexpr int XL = BK + 8;       // LDS row stride of the staging buffer
constexpr int NT = 256;
constexpr int kLdsHalves = 4 * S * SL + S * XL;   // 154 KB
// Register prefetch depth (K slices held in registers) of the two streamed
// products: four for the Gram; two for the multiply-back, whose epilogue
// leaves no room for more without spills.
constexpr int kGramDepth = 4;
constexpr int kRectDepth = 2;

typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef f16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct SmallArgs {
  // X_math (128 x Lp, row stride Lp) and its transpose (Lp x 128), then the
  // second pair the restart writes into; per-matrix stride sX halves
  f16 *X, *XT, *Y, *YT;
  long long sX;
  int Lp;
  int tr;                        // X_math is the transpose of the selected rows (k > m)
  dion3_ns_cfg cfg;
  BatchPtr<float> W;
  long long ldw;
  const int* idx;
  float lr;
  f16* Oout;
  long long sO;                  // elements between consecutive matrices' O blocks
  int kval, mval, nrows;
};

// A wave of the 2 x 2 grid: quadrant (wm, wn) of the output.
struct Wave {
  int lane, tid, wm, wn;
  __device__ bool diag() const { return wm == wn; }
};

__device__ __forceinline__ void zero_acc(floatx16 (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

// acc[i][j] += P[pr + 32 i + ..][k] * Q[qr + 32 j + ..][k] over k < KN, both
// operands K-contiguous in LDS with row strides LP, LQ.
template <int LP, int LQ, int KN>
__device__ __forceinline__ void mma(const f16* P, int pr, const f16* Q, int qr, int lane,
                                    floatx16 (&acc)[2][2]) {
  const f16* p_s = P + (pr + (lane & 31)) * LP + (lane >> 5) * 8;
  const f16* q_s = Q + (qr + (lane & 31)) * LQ + (lane >> 5) * 8;
  // fragments double-buffered: those of slice kk + 16 are requested before
  // the MFMAs of slice kk, so the LDS latency hides behind them
  half8 pf[2][2], qf[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) pf[0][i] = *(const half8*)(p_s + i * 32 * LP);
#pragma unroll
  for (int j = 0; j < 2; ++j) qf[0][j] = *(const half8*)(q_s + j * 32 * LQ);
#pragma unroll
  for (int kk = 0; kk < KN; kk += 16) {
    const int cb = (kk >> 4) & 1;
    if (kk + 16 < KN) {
#pragma unroll
      for (int i = 0; i < 2; ++i) pf[cb ^ 1][i] = *(const half8*)(p_s + i * 32 * LP + kk + 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) qf[cb ^ 1][j] = *(const half8*)(q_s + j * 32 * LQ + kk + 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[cb][i], qf[cb][j], acc[i][j], 0, 0, 0);
  }
}

// The symmetric product's operands for this wave (see the file comment).
template <int LA, int KN>
__device__ __forceinline__ void mma_sym(const f16* A, const f16* B, const Wave& w,
                                        floatx16 (&acc)[2][2]) {
  if (w.wm == 0 && w.wn == 1)
    mma<LA, LA, KN>(B, 0, A, 64, w.lane, acc);
  else
    mma<LA, LA, KN>(A, w.wm * 64, B, w.wn * 64, w.lane, acc);
}

// Epilogue of a symmetric product into `out` (LDS, stride SL):
// value = alpha acc + beta D + gamma I (POLY) or acc, rounded to fp32 and
// then fp16, stored at both (r, c) and (c, r) as the lower element's value.
// Accumulator (i, j, v) of lane l is element (p + v % 4, q) with
// p = 32 i + 8 (v / 4) + 4 (l / 32) and q = 32 j + l % 32 (plus the wave's
// row and column bases).  Every block is stored transposed (one 8-byte run
// per 4 accumulators), which puts the lower values into the upper triangle;
// the lower triangle of the off-diagonal quadrant comes from the swapped
// wave, that of the strictly lower blocks of the diagonal quadrants from
// direct stores, and that of the four diagonal 32 x 32 blocks from a short
// copy of their upper halves after a barrier.  The caller's barrier follows.
template <bool POLY>
__device__ __forceinline__ void epi_sym(f16* out, const floatx16 (&acc)[2][2], float alpha,
                                        const f16* D, float beta, float gamma, const Wave& w,
                                        int gd) {
  const bool swap = (w.wm == 0 && w.wn == 1);
  const int pr = swap ? 0 : w.wm * 64, qr = swap ? 64 : w.wn * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (w.diag() && i < j) continue;          // upper block of a diagonal quadrant
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int p = pr + i * 32 + 8 * v4 + 4 * (w.lane >> 5);
        const int q = qr + j * 32 + (w.lane & 31);
        float val[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[i][j][4 * v4 + e];
        if (POLY) {
          const half4 d = *(const half4*)(D + q * SL + p);   // D[p + e][q] (D symmetric)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            val[e] = __builtin_fmaf(val[e], alpha, beta * (float)d[e]);
            if (p + e == q && q < gd) val[e] += gamma;   // identity of the real block only
            asm("" : "+v"(val[e]));   // fp32 rounding, then fp16, as in the tiled kernels
          }
        }
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (f16)val[e];
        *(half4*)(out + q * SL + p) = h;
        if (w.diag() && i > j)
#pragma unroll
          for (int e = 0; e < 4; ++e) out[(p + e) * SL + q] = h[e];
      }
    }
  __syncthreads();
  if (w.diag()) {
    // lower triangle of the diagonal blocks (b, b), b = 2 wm, 2 wm + 1: the
    // element (x, y), x > y, takes (y, x); the others rewrite their own value
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int base = w.wm * 64 + blk * 32;
      f16 v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int id = w.lane + 64 * e, x = id >> 5, y = id & 31;
        const int sx = x > y ? y : x, sy = x > y ? x : y;
        v[e] = out[(base + sx) * SL + base + sy];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int id = w.lane + 64 * e, x = id >> 5, y = id & 31;
        out[(base + x) * SL + base + y] = v[e];
      }
    }
  }
}

// out = alpha A B + beta D + gamma I (POLY) or A B, all symmetric s x s in
// LDS.  out may be A or B: the product is finished before anything is
// written.  The inner dimension runs to kn, the Gram side rounded up to 32:
// past it every operand of the real block is zero padding, so the real
// block's sums are the same bits (its accumulators start at +0, and adding
// exact zeros changes no value and no sign), and the padding block, which
// no real output ever reads, stays zero.
template <bool POLY>
__device__ __forceinline__ void symm_lds(f16* out, const f16* A, const f16* B, const f16* D,
                                         float alpha, float beta, float gamma, const Wave& w,
                                         int kn, int sreal) {
  floatx16 acc[2][2];
  zero_acc(acc);
  if (kn <= 32)
    mma_sym<SL, 32>(A, B, w, acc);
  else if (kn <= 64)
    mma_sym<SL, 64>(A, B, w, acc);
  else
    mma_sym<SL, S>(A, B, w, acc);
  __syncthreads();
  epi_sym<POLY>(out, acc, alpha, D, beta, gamma, w, sreal);
  __syncthreads();
}

// Streams 128-row x 64-half slices of a K-contiguous global matrix through
// the LDS staging buffer.  Slice t covers rows row0(t).. and columns
// col0(t)..; each thread moves 4 chunks of 8 halves.
struct Slices {
  const f16* src;
  int ld;
  __device__ __forceinline__ void load(half8 (&r)[4], int row0, int col0, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i;
      r[i] = *(const half8*)(src + (long long)(row0 + (c >> 3)) * ld + col0 + (c & 7) * 8);
    }
  }
};

__device__ __forceinline__ void lds_store(f16* xs, const half8 (&r)[4], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NT * i;
    *(half8*)(xs + (c >> 3) * XL + (c & 7) * 8) = r[i];
  }
}

// Runs consume(t) for t = 0 .. n-1 with K slice t in the staging buffer,
// the slices arriving through a ring of D register sets (D - 1 slices in
// flight while one is multiplied).  coord(t, row0, col0) places slice t.
template <int D, class Coord, class Consume>
__device__ __forceinline__ void stream_slices(const Slices& sl, int n, f16* xs, int tid,
                                              Coord coord, Consume consume) {
  half8 r[D][4];
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < n) {
      int r0, c0;
      coord(u, r0, c0);
      sl.load(r[u], r0, c0, tid);
    }
  for (int t = 0; t < n; t += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (t + u < n) {
        __syncthreads();                     // the previous slice is consumed
        lds_store(xs, r[u], tid);
        if (t + u + D < n) {
          int r0, c0;
          coord(t + u + D, r0, c0);
          sl.load(r[u], r0, c0, tid);
        }
        __syncthreads();
        consume(t + u);
      }
    }
  }
}

// R = X X^T (K = Lp), X from global (rows layout, row stride Lp).
__device__ __forceinline__ void gram_small(f16* R, f16* xs, const f16* X, int Lp, const Wave& w) {
  const Slices sl = {X, Lp};
  floatx16 acc[2][2];
  zero_acc(acc);
  stream_slices<kGramDepth>(
      sl, Lp / BK, xs, w.tid, [](int t, int& r0, int& c0) { r0 = 0; c0 = t * BK; },
      [&](int) { mma_sym<XL, BK>(xs, xs, w, acc); });
  __syncthreads();
  epi_sym<false>(R, acc, 1.0f, nullptr, 0.0f, 0.0f, w, S);
  __syncthreads();
}

// One 8-wide chunk of O in rows layout (row orow, columns ocol..ocol+7)
// goes to the row-sparse update: W[idx[orow]][ocol..] -= lr * O and
// optionally O_out = O; the same arithmetic as the tiled kernels' update.
__device__ __forceinline__ void sink8(const SmallArgs& p, int b, int orow, int ocol,
                                      const half8& v) {
  if (orow >= p.kval || ocol >= p.mval) return;
  const bool full = ocol + 8 <= p.mval;
  if (p.Oout) {
    f16* o = p.Oout + (long long)b * p.sO + (long long)orow * p.mval + ocol;
    if (full && ((uintptr_t)o & 15) == 0) {
      *(half8*)o = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ocol + e < p.mval) o[e] = v[e];
    }
  }
  if (p.W.ptrs || p.W.base) {
    const int row = p.idx[(long long)b * p.kval + orow];
    if (row < 0 || row >= p.nrows) return;
    float* wp = p.W.get(b) + (long long)row * p.ldw + ocol;
    if (full && ((uintptr_t)wp & 15) == 0) {
      float4 w0 = ((float4*)wp)[0], w1 = ((float4*)wp)[1];
      w0.x = __builtin_fmaf(-p.lr, (float)v[0], w0.x);
      w0.y = __builtin_fmaf(-p.lr, (float)v[1], w0.y);
      w0.z = __builtin_fmaf(-p.lr, (float)v[2], w0.z);
      w0.w = __builtin_fmaf(-p.lr, (float)v[3], w0.w);
      w1.x = __builtin_fmaf(-p.lr, (float)v[4], w1.x);
      w1.y = __builtin_fmaf(-p.lr, (float)v[5], w1.y);
      w1.z = __builtin_fmaf(-p.lr, (float)v[6], w1.z);
      w1.w = __builtin_fmaf(-p.lr, (float)v[7], w1.w);
      ((float4*)wp)[0] = w0;
      ((float4*)wp)[1] = w1;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ocol + e < p.mval) wp[e] = __builtin_fmaf(-p.lr, (float)v[e], wp[e]);
    }
  }
}

// Y = Q X_math over the L side in 128-wide column blocks (two K slices of
// X^T each).  Each 128 x 128 block is staged in two free s x s buffers (SA
// in the math layout, SB transposed) and leaves in 16-byte runs: to Y and
// YT (restart) or, in rows layout, into the update (final).
__device__ __forceinline__ void rect_small(const f16* Q, f16* xs, f16* SA, f16* SB, const f16* XT,
                                           int Lp, f16* Y, f16* YT, const SmallArgs& p, int b,
                                           bool final_pass, const Wave& w, int kn) {
  const Slices sl = {XT, S};
  const bool rows = !final_pass || !p.tr, cols = !final_pass || p.tr;
  floatx16 acc[2][2];
  auto coord = [](int t, int& r0, int& c0) { r0 = (t >> 1) * S; c0 = (t & 1) * BK; };
  auto consume = [&](int t) {
    if ((t & 1) == 0) {
      zero_acc(acc);
      mma<SL, XL, BK>(Q, w.wm * 64, xs, w.wn * 64, w.lane, acc);
      return;
    }
    // Q's columns from 64 on are zero padding when the Gram side is at
    // most 64 (see symm_lds)
    if (kn > BK) mma<SL, XL, BK>(Q + BK, w.wm * 64, xs, w.wn * 64, w.lane, acc);
    const int j0 = (t >> 1) * S;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int r = w.wm * 64 + i * 32 + 8 * v4 + 4 * (w.lane >> 5);   // rows r..r+3
          const int c = w.wn * 64 + jj * 32 + (w.lane & 31);               // block column
          half4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (f16)acc[i][jj][4 * v4 + e];
          if (rows)
#pragma unroll
            for (int e = 0; e < 4; ++e) SA[(r + e) * SL + c] = h[e];
          if (cols) *(half4*)(SB + c * SL + r) = h;
        }
    __syncthreads();
    // 128 rows x 16 chunks of 8 halves per layout, 8 chunks per thread
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = w.tid + NT * i, row = e >> 4, ch = (e & 15) * 8;
      if (!final_pass) {
        *(half8*)(Y + (long long)row * Lp + j0 + ch) = *(const half8*)(SA + row * SL + ch);
        *(half8*)(YT + (long long)(j0 + row) * S + ch) = *(const half8*)(SB + row * SL + ch);
      } else if (!p.tr) {   // rows layout = math layout: O[row][j0 + ch..]
        sink8(p, b, row, j0 + ch, *(const half8*)(SA + row * SL + ch));
      } else {              // rows layout = transposed: O[j0 + row][ch..]
        sink8(p, b, j0 + row, ch, *(const half8*)(SB + row * SL + ch));
      }
    }
  };
  stream_slices<kRectDepth>(sl, 2 * (Lp / S), xs, w.tid, coord, consume);
  __syncthreads();
}

__device__ __forceinline__ bool is_restart(const dion3_ns_cfg& c, int t) {
  for (int i = 0; i < c.n_restart; ++i)
    if (c.restart_at[i] == t) return true;
  return false;
}

__global__ __launch_bounds__(NT, 1) void k_gram_ns_small(SmallArgs p) {
  __shared__ __attribute__((aligned(16))) f16 lds[kLdsHalves];
  f16* xs = lds + 4 * S * SL;
  const int b = blockIdx.x;
  Wave w;
  w.tid = threadIdx.x;
  w.lane = w.tid & 63;
  w.wm = (w.tid >> 6) >> 1;
  w.wn = (w.tid >> 6) & 1;
  f16* X = p.X + (long long)b * p.sX;
  f16* XT = p.XT + (long long)b * p.sX;
  f16* Y = p.Y + (long long)b * p.sX;
  f16* YT = p.YT + (long long)b * p.sX;

  f16 *R = lds, *Z = lds + S * SL, *Q = lds + 2 * S * SL, *T = lds + 3 * S * SL;
  // the unpadded Gram side, and the inner extent of the s x s products: that
  // side rounded up to 32
  const int sreal = p.tr ? p.mval : p.kval;
  const int kn = (sreal + 31) / 32 * 32;
  gram_small(R, xs, X, p.Lp, w);
  bool q_identity = true;
  const int iters = p.cfg.iters;
  for (int t = 1; t <= iters; ++t) {
    if (is_restart(p.cfg, t)) {      // X <- Q X, R <- X X^T, Q <- I
      if (!q_identity) {
        rect_small(Q, xs, R, T, XT, p.Lp, Y, YT, p, b, false, w, kn);
        f16* tx = X; X = Y; Y = tx;
        f16* tt = XT; XT = YT; YT = tt;
      }
      gram_small(R, xs, X, p.Lp, w);
      q_identity = true;
    }
    const float a = p.cfg.abc[t - 1][0], bb = p.cfg.abc[t - 1][1], c = p.cfg.abc[t - 1][2];
    symm_lds<true>(Z, R, R, R, c, bb, a, w, kn, sreal);            // Z = a I + b R + c R^2
    f16* Zv;
    if (q_identity) {                                    // Q = I: adopt Z
      f16* tmp = Q; Q = Z; Z = tmp;
      Zv = Q;
      q_identity = false;
    } else {
      symm_lds<false>(Q, Z, Q, nullptr, 1.0f, 0.0f, 0.0f, w, kn, sreal);   // Q <- Z Q
      Zv = Z;
    }
    if (t < iters && !is_restart(p.cfg, t + 1)) {      // R <- Z R Z
      symm_lds<false>(T, Zv, R, nullptr, 1.0f, 0.0f, 0.0f, w, kn, sreal);
      symm_lds<false>(R, T, Zv, nullptr, 1.0f, 0.0f, 0.0f, w, kn, sreal);
    }
  }
  rect_small(Q, xs, R, T, XT, p.Lp, Y, YT, p, b, true, w, kn);
}


// ---------------------------------------------------------------------------
// Gram sides of at most 64: the s x s matrices are one or two 32 x 32 blocks
// per side (NB), so each symmetric product of the iteration is a handful of
// MFMAs.  One wave runs all of them back to back, with R, Z, Q and T in LDS
// and no workgroup barrier between products (a wave's LDS accesses execute
// in order); the Gram (X staged through LDS by all four waves, one lower
// 32 x 32 block per wave) and the multiply-backs (32 x 32 output blocks
// dealt to the four waves) stream X.  Every element is computed as
// in the tiled kernels: its k-groups of 16 in increasing order into one fp32
// accumulator that starts at +0, the same epilogue, and symmetric results
// taken from the lower triangle (so the bits equal the tiled path's).
constexpr int TS = 64;           // padded side
constexpr int TL = TS + 8;       // LDS row stride of R, Z, Q, T (halves)
constexpr int TB = 32 + 8;       // row stride of a wave's 32 x 32 output staging

// Orders this wave's LDS accesses around the call (writes before, reads
// after) without a workgroup barrier.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Accumulator (v) of lane l in a 32 x 32 MFMA block: row 8 (v / 4) + 4 (l / 32)
// + v % 4, column l % 32.
__device__ __forceinline__ int acc_row(int v4, int lane) { return 8 * v4 + 4 * (lane >> 5); }

// Stores the fp16 value h (4 consecutive rows p..p+3 of column q) of a
// symmetric result: the lower elements (row >= column) at both (row, col)
// and (col, row); the upper ones come from their mirror.  An upper element of
// a diagonal block is written to the row's padding columns TS .. TS + 7,
// which nothing reads, instead of being skipped: the stores need no branch
// (a branch per element took about 40 % of a 32 x 32 product's time).
// OPAQUE hides p and q from the optimizer, which otherwise keeps every
// store address of every product in registers (256 VGPRs and one wave per
// SIMD for the 64-side kernel).
template <bool OPAQUE>
__device__ __forceinline__ void store_sym4(f16* out, int p, int q, bool diag, const half4& h) {
  if (OPAQUE) asm volatile("" : "+v"(p), "+v"(q));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool keep = !diag || p + e >= q;
    out[(p + e) * TL + (keep ? q : TS + e)] = h[e];
    out[q * TL + (keep ? p + e : TS + 4 + e)] = h[e];
  }
}

// out = alpha A B + beta D + gamma I (POLY) or A B for symmetric NB x NB-block
// matrices in LDS, by one wave.  out may be A or B: every operand read comes
// before the first store.
template <int NB, bool POLY>
__device__ __forceinline__ void tiny_symm(f16* out, const f16* A, const f16* B, const f16* D,
                                          float alpha, float beta, float gamma, int lane, int gd) {
  constexpr int NL = NB * (NB + 1) / 2;
  floatx16 acc[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[l][v] = 0.0f;
  const int fr = (lane & 31) * TL + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < 2 * NB; ++s) {
    half8 af[NB], bf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      af[i] = *(const half8*)(A + i * 32 * TL + fr + 16 * s);
      bf[i] = *(const half8*)(B + i * 32 * TL + fr + 16 * s);
    }
    int l = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j <= i; ++j, ++l)
        acc[l] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[l], 0, 0, 0);
  }
  int l = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j, ++l)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int p = i * 32 + acc_row(v4, lane), q = j * 32 + (lane & 31);
        float val[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[l][4 * v4 + e];
        if (POLY) {
          const half4 d = *(const half4*)(D + q * TL + p);   // D[p + e][q] (D symmetric)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            val[e] = __builtin_fmaf(val[e], alpha, beta * (float)d[e]);
            if (p + e == q && q < gd) val[e] += gamma;
            asm("" : "+v"(val[e]));   // fp32 rounding, then fp16, as in the tiled kernels
          }
        }
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (f16)val[e];
        store_sym4<(NB > 1)>(out, p, q, i == j, h);
      }
  wave_lds_fence();
}

// R = X X^T with X streamed through LDS by all four waves: chunks of CW
// columns (32 NB rows x CW, 32 KB) are staged in `buf` (the s x s matrices'
// space, all dead during a Gram) while the next chunk is already on its way
// into registers; the lower 32 x 32 blocks accumulate on waves 0 .. NL - 1,
// each from +0 over its k-groups in increasing order (the tiled Gram's order).
// One wave reading X from global memory itself waited for every batch of
// loads; here each chunk's loads have a whole chunk of MFMAs to arrive.
template <int NB>
__device__ __forceinline__ void tiny_gram_lds(f16* R, f16* buf, const f16* X, int Lp, int tid,
                                              int wave, int lane) {
  constexpr int NL = NB * (NB + 1) / 2, ROWS = 32 * NB, CW = 512 / NB, LS = CW + 8;
  constexpr int CPR = CW / 8, NCH = ROWS * CPR / NT;   // 16-byte runs per row, per thread
  static_assert(NCH * NT == ROWS * CPR && ROWS * LS <= 4 * TS * TL, "chunk fits");
  const int nc = (Lp + CW - 1) / CW;
  half8 pre[NCH];
  auto gl = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int e = tid + NT * i, r = e / CPR, cc = (e % CPR) * 8;
      if (c0 + cc < Lp) pre[i] = *(const half8*)(X + (long long)r * Lp + c0 + cc);
    }
  };
  auto st = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int e = tid + NT * i, r = e / CPR, cc = (e % CPR) * 8;
      if (c0 + cc < Lp) *(half8*)(buf + r * LS + cc) = pre[i];
    }
  };
  const int bi = (NB == 2 && wave >= 1) ? 1 : 0, bj = (NB == 2 && wave == 2) ? 1 : 0;
  const bool dg = bi == bj;
  const f16* ra = buf + (bi * 32 + (lane & 31)) * LS + 8 * (lane >> 5);
  const f16* rb = buf + (bj * 32 + (lane & 31)) * LS + 8 * (lane >> 5);
  floatx16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  gl(0);
  for (int c = 0; c < nc; ++c) {
    const int c0 = c * CW;
    st(c0);
    __syncthreads();
    if (c + 1 < nc) gl(c0 + CW);
    if (wave < NL) {
      const int nkg = min(CW, Lp - c0) / 16;   // a multiple of 8
      for (int kg = 0; kg < nkg; kg += 8) {
        half8 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a[u] = *(const half8*)(ra + 16 * (kg + u));
          b[u] = dg ? a[u] : *(const half8*)(rb + 16 * (kg + u));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[u], b[u], acc, 0, 0, 0);
      }
    }
    __syncthreads();   // the chunk's reads end before the next chunk (or R) overwrites buf
  }
  if (wave < NL) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int p = bi * 32 + acc_row(v4, lane), q = bj * 32 + (lane & 31);
      half4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (f16)acc[4 * v4 + e];
      store_sym4<(NB > 1)>(R, p, q, dg, h);
    }
  }
}

// Y = Q X_math over the L side in 32 x 32 output blocks (NB row blocks x
// Lp / 32 column blocks, dealt to the waves in turn).  The block's operand,
// X_math rows 0 .. 32 NB - 1 by 32 columns, is loaded one block ahead with
// 16-byte runs, staged in this wave's LDS block (row stride TX) and read as
// MFMA fragments (8 consecutive K of one column) with two transposing reads
// each, so only the rows layout of X is ever read.  The output block goes
// through the same LDS block (column-major: St[c][r]) and leaves in 16-byte
// runs: to Y (restart) or into the update (final; a W update in rows layout
// takes tiny_final below instead).
constexpr int TX = 32 + 8;       // row stride of the staged X_math block (halves)
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;

template <int NB>
__device__ __forceinline__ void tiny_rect(const f16* Q, const f16* Xm, int Lp, f16* Y, f16* St,
                                          const SmallArgs& p, int b, bool final_pass, int wave,
                                          int lane) {
  typedef f16 half4v __attribute__((ext_vector_type(4)));
  const int ncb = Lp / 32, nblk = NB * ncb;
  const int fr = (lane & 31) * TL + 8 * (lane >> 5);
  // this lane's two 16-byte runs of the X block: run c = lane + 64 u is row
  // c / 4, columns 8 (c % 4) ..
  auto load = [&](int blk, half8 (&f)[2 * NB]) {
    const int j0 = (blk % ncb) * 32;
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {
      const int c = lane + 64 * u;
      f[u] = *(const half8*)(Xm + (long long)(c >> 2) * Lp + j0 + (c & 3) * 8);
    }
  };
  // transposing-read address: row 8 (lane / 32) + (lane % 16) / 4, column
  // 16 ((lane / 16) % 2) + 4 (lane % 4) of the staged block
  const int toff = (8 * (lane >> 5) + ((lane & 15) >> 2)) * TX + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  half8 xn[2 * NB];
  if (wave < nblk) load(wave, xn);
  for (int blk = wave; blk < nblk; blk += 4) {
    const int bi = blk / ncb, j0 = (blk - bi * ncb) * 32;
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {
      const int c = lane + 64 * u;
      *(half8*)(St + (c >> 2) * TX + (c & 3) * 8) = xn[u];
    }
    wave_lds_fence();
    if (blk + 4 < nblk) load(blk + 4, xn);
    half8 xf[2 * NB];
#pragma unroll
    for (int s = 0; s < 2 * NB; ++s) {
      const f16* q = St + toff + 16 * s * TX;
      const half4v lo =
          __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)q));
      const half4v hi = __builtin_bit_cast(
          half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(q + 4 * TX)));
      xf[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int s = 0; s < 2 * NB; ++s) {
      const half8 qf = *(const half8*)(Q + bi * 32 * TL + fr + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf, xf[s], acc, 0, 0, 0);
    }
    // the fragments are in registers: the block's LDS now stages the output
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int r = acc_row(v4, lane), c = lane & 31;
      half4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (f16)acc[4 * v4 + e];
      *(half4*)(St + c * TB + r) = h;
    }
    wave_lds_fence();
    // 32 x 32 block = 128 runs of 8, two per lane
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = lane + 64 * u, a = e >> 2, c8 = (e & 3) * 8;
      const int row0 = bi * 32;
      if (final_pass && p.tr) {
        // rows layout = transposed: O[j0 + a][row0 + c8 ..], a column run
        sink8(p, b, j0 + a, row0 + c8, *(const half8*)(St + a * TB + c8));
      } else {
        // row a, columns c8..c8+7, gathered from St's columns
        half8 rowrun;
#pragma unroll
        for (int q = 0; q < 8; ++q) rowrun[q] = St[(c8 + q) * TB + a];
        if (!final_pass)
          *(half8*)(Y + (long long)(row0 + a) * Lp + j0 + c8) = rowrun;
        else
          sink8(p, b, row0 + a, j0 + c8, rowrun);
      }
    }
    wave_lds_fence();   // the next block's staging overwrites St
  }
}

// The final pass when the output rows are the selected rows of W (rows
// layout, O = Q X_math) and W is updated: as tiny_rect's final pass, but the
// selected-row indices of this lane's two output runs per row block are read
// once up front, and each block's W runs are requested one block ahead
// together with its X block, so they are in flight during the previous
// block's products instead of starting after the block's own (megabatches
// of 128 x 4096 matrices at f = 1/4: 191 -> 163 us per step; the same
// arithmetic, so the same bits).  Every pass issues the same loads (see
// wload and the next-block index), so the waits before a block's staging
// and update count only the loads that block needs.
template <int NB>
__device__ __forceinline__ void tiny_final(const f16* Q, const f16* Xm, int Lp, f16* St,
                                           const SmallArgs& p, int b, int wave, int lane) {
  typedef f16 half4v __attribute__((ext_vector_type(4)));
  const int ncb = Lp / 32, nblk = NB * ncb;
  const int fr = (lane & 31) * TL + 8 * (lane >> 5);
  float* Wb = (p.W.ptrs || p.W.base) ? p.W.get(b) : nullptr;
  const bool vec = Wb && ((uintptr_t)Wb & 15) == 0 && (p.ldw & 3) == 0;
  // selected W row of run u (output row 32 bi + (lane + 64 u) / 4), or -1
  int rows0[2], rows1[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int a = (lane + 64 * u) >> 2;
    int r0 = -1, r1 = -1;
    if (Wb && a < p.kval) r0 = p.idx[(long long)b * p.kval + a];
    if (NB == 2 && Wb && 32 + a < p.kval) r1 = p.idx[(long long)b * p.kval + 32 + a];
    rows0[u] = (r0 >= 0 && r0 < p.nrows) ? r0 : -1;
    rows1[u] = (r1 >= 0 && r1 < p.nrows) ? r1 : -1;
  }
  auto load = [&](int blk, half8 (&f)[2 * NB]) {
    const int j0 = (blk % ncb) * 32;
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {
      const int c = lane + 64 * u;
      f[u] = *(const half8*)(Xm + (long long)(c >> 2) * Lp + j0 + (c & 3) * 8);
    }
  };
  // W runs of a block, read by every lane (a lane whose run does not take
  // this path reads W's first 8 elements instead)
  const bool pre = vec && p.mval >= 8;
  auto wload = [&](int blk, float4 (&w)[2][2]) {
    const int bi = blk / ncb, j0 = (blk - bi * ncb) * 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = (NB == 2 && bi) ? rows1[u] : rows0[u];
      const int c = j0 + ((lane + 64 * u) & 3) * 8;
      const bool real = row >= 0 && c + 8 <= p.mval;
      const float4* q = (const float4*)(real ? Wb + (long long)row * p.ldw + c : Wb);
      w[u][0] = q[0];
      w[u][1] = q[1];
    }
  };
  const int toff = (8 * (lane >> 5) + ((lane & 15) >> 2)) * TX + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  half8 xn[2 * NB];
  float4 wn[2][2];
  if (wave < nblk) {
    load(wave, xn);
    if (pre) wload(wave, wn);
  }
  for (int blk = wave; blk < nblk; blk += 4) {
    const int bi = blk / ncb, j0 = (blk - bi * ncb) * 32;
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {
      const int c = lane + 64 * u;
      *(half8*)(St + (c >> 2) * TX + (c & 3) * 8) = xn[u];
    }
    float4 wc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      wc[u][0] = wn[u][0];
      wc[u][1] = wn[u][1];
    }
    wave_lds_fence();
    // the next block's operands (the last block requests its own again)
    const int nx = blk + 4 < nblk ? blk + 4 : blk;
    load(nx, xn);
    if (pre) wload(nx, wn);
    half8 xf[2 * NB];
#pragma unroll
    for (int s = 0; s < 2 * NB; ++s) {
      const f16* q = St + toff + 16 * s * TX;
      const half4v lo =
          __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)q));
      const half4v hi = __builtin_bit_cast(
          half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(q + 4 * TX)));
      xf[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int s = 0; s < 2 * NB; ++s) {
      const half8 qf = *(const half8*)(Q + bi * 32 * TL + fr + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf, xf[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int r = acc_row(v4, lane), c = lane & 31;
      half4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (f16)acc[4 * v4 + e];
      *(half4*)(St + c * TB + r) = h;
    }
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = lane + 64 * u, a = e >> 2, c8 = (e & 3) * 8;
      half8 v;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = St[(c8 + q) * TB + a];
      const int orow = bi * 32 + a, ocol = j0 + c8;
      if (orow >= p.kval || ocol >= p.mval) continue;
      const bool full = ocol + 8 <= p.mval;
      if (p.Oout) {
        f16* o = p.Oout + (long long)b * p.sO + (long long)orow * p.mval + ocol;
        if (full && ((uintptr_t)o & 15) == 0) {
          *(half8*)o = v;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (ocol + q < p.mval) o[q] = v[q];
        }
      }
      const int row = (NB == 2 && bi) ? rows1[u] : rows0[u];
      if (row < 0) continue;
      float* wp = Wb + (long long)row * p.ldw + ocol;
      if (pre && full) {
        float4 w0 = wc[u][0], w1 = wc[u][1];
        w0.x = __builtin_fmaf(-p.lr, (float)v[0], w0.x);
        w0.y = __builtin_fmaf(-p.lr, (float)v[1], w0.y);
        w0.z = __builtin_fmaf(-p.lr, (float)v[2], w0.z);
        w0.w = __builtin_fmaf(-p.lr, (float)v[3], w0.w);
        w1.x = __builtin_fmaf(-p.lr, (float)v[4], w1.x);
        w1.y = __builtin_fmaf(-p.lr, (float)v[5], w1.y);
        w1.z = __builtin_fmaf(-p.lr, (float)v[6], w1.z);
        w1.w = __builtin_fmaf(-p.lr, (float)v[7], w1.w);
        ((float4*)wp)[0] = w0;
        ((float4*)wp)[1] = w1;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (ocol + q < p.mval) wp[q] = __builtin_fmaf(-p.lr, (float)v[q], wp[q]);
      }
    }
    wave_lds_fence();   // the next block's staging overwrites St
  }
}

template <int NB>
__global__ __launch_bounds__(NT) void k_gram_ns_tiny(SmallArgs p) {
  __shared__ __attribute__((aligned(16))) f16 mats[4 * TS * TL];
  // per wave: the staged X_math block (32 NB x TX) and then the output block
  // (32 x TB) in the same place
  constexpr int SW = 32 * NB * TX > 32 * TB ? 32 * NB * TX : 32 * TB;
  __shared__ __attribute__((aligned(16))) f16 stage[4 * SW];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // only the rows layout of X_math (and of the restart's output) is used
  f16* X = p.X + (long long)b * p.sX;
  f16* Y = p.Y + (long long)b * p.sX;
  f16 *R = mats, *Z = mats + TS * TL, *Q = mats + 2 * TS * TL, *T = mats + 3 * TS * TL;
  f16* St = stage + wave * SW;
  const int sreal = p.tr ? p.mval : p.kval;
  tiny_gram_lds<NB>(R, mats, X, p.Lp, tid, wave, lane);
  __syncthreads();
  bool q_identity = true;
  const int iters = p.cfg.iters;
  for (int t = 1; t <= iters; ++t) {
    if (is_restart(p.cfg, t)) {      // X <- Q X, R <- X X^T, Q <- I
      if (!q_identity) {
        __syncthreads();             // Q complete
        tiny_rect<NB>(Q, X, p.Lp, Y, St, p, b, false, wave, lane);
        f16* tx = X; X = Y; Y = tx;
        __syncthreads();             // the new X in memory, Q read
      }
      tiny_gram_lds<NB>(R, mats, X, p.Lp, tid, wave, lane);
      __syncthreads();
      q_identity = true;
    }
    const float a = p.cfg.abc[t - 1][0], bb = p.cfg.abc[t - 1][1], c = p.cfg.abc[t - 1][2];
    const bool next_r = t < iters && !is_restart(p.cfg, t + 1);
    // the products of this iteration, all on wave 0 (uniform pointer swaps on every wave)
    f16* Zv;
    if (wave == 0) tiny_symm<NB, true>(Z, R, R, R, c, bb, a, lane, sreal);   // Z = a I + b R + c R^2
    if (q_identity) {
      f16* tmp = Q; Q = Z; Z = tmp;
      Zv = Q;
      q_identity = false;
    } else {
      if (wave == 0) tiny_symm<NB, false>(Q, Z, Q, nullptr, 1.0f, 0.0f, 0.0f, lane, sreal);
      Zv = Z;
    }
    if (next_r && wave == 0) {       // R <- Z R Z
      tiny_symm<NB, false>(T, Zv, R, nullptr, 1.0f, 0.0f, 0.0f, lane, sreal);
      tiny_symm<NB, false>(R, T, Zv, nullptr, 1.0f, 0.0f, 0.0f, lane, sreal);
    }
  }
  __syncthreads();                   // Q complete
  if (p.tr || !(p.W.ptrs || p.W.base)) tiny_rect<NB>(Q, X, p.Lp, Y, St, p, b, true, wave, lane);
  else tiny_final<NB>(Q, X, p.Lp, St, p, b, wave, lane);
}
}  // namespace

hipError_t launch_gram_ns_small(f16* X, f16* XT, f16* Y, f16* YT, long long sX, int batch, int Lp,
                                bool tr, const dion3_ns_cfg& cfg, BatchPtr<float> W, long long ldw,
                                const int* idx, float lr, f16* Oout, long long sO, int kval,
                                int mval, int nrows, double trace_flops, hipStream_t s) {
  if (Lp < S || Lp % S != 0 || batch < 1) return hipErrorInvalidValue;
  SmallArgs p;
  p.X = X; p.XT = XT; p.Y = Y; p.YT = YT; p.sX = sX;
  p.Lp = Lp; p.tr = tr ? 1 : 0;
  p.cfg = cfg;
  p.W = W; p.ldw = ldw; p.idx = idx; p.lr = lr; p.Oout = Oout; p.sO = sO;
  p.kval = kval; p.mval = mval; p.nrows = nrows;
  // algorithmic bytes: X read once, the selected rows of W read and written
  const double sL = (double)kval * mval;
  const double bytes =
      (double)batch * sL * (2.0 + (W.ptrs || W.base ? 8.0 : 0.0) + (Oout ? 2.0 : 0.0));
  // Gram sides up to 64: the one-wave s x s path
  const int sreal = tr ? mval : kval;
  if (sreal <= 32) {
    TraceScope trace("gram_ns_fused_32", trace_flops, bytes, s);
    hipLaunchKernelGGL(k_gram_ns_tiny<1>, dim3(batch), dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  if (sreal <= TS) {
    TraceScope trace("gram_ns_fused_64", trace_flops, bytes, s);
    hipLaunchKernelGGL(k_gram_ns_tiny<2>, dim3(batch), dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  TraceScope trace("gram_ns_fused_128", trace_flops, bytes, s);
  hipLaunchKernelGGL(k_gram_ns_small, dim3(batch), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace dion3
