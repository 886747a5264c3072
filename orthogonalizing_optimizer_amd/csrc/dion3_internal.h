// Internal interfaces between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dion3.h"

namespace dion3 {

typedef _Float16 f16;

// A batch of same-shape matrices: either `ptrs[b]` (a device array of
// pointers, the megabatch form) or `base + b * stride`.
template <typename T>
struct BatchPtr {
  T* base;
  long long stride;
  T* const* ptrs;
  __device__ __forceinline__ T* get(int b) const { return ptrs ? ptrs[b] : base + (long long)b * stride; }
};

// Tile edge of every GEMM output tile; workspace dimensions are padded to it.
constexpr int kTile = 128;

inline long long pad_to(long long x, long long p) { return (x + p - 1) / p * p; }

// K advances through every GEMM 64 at a time.  A product whose inner
// dimension is padded past the next multiple of 64 only reads the padding's
// zero cross terms there, so its K loop stops at that multiple.
constexpr int kKStep = 64;

// C = alpha * A * B^T (+ beta * D + gamma * I when `epilogue`), batched.
//  A is M x K stored A[m * lda + k]; B is N x K stored B[n * ldb + k].
//  Rows outside M (or N) read as zero; outputs outside M x N are not written.
//  lower: M == N, only tiles on or below the diagonal are computed and each
//  element (r >= c) is written to both C[r][c] and C[c][r].
//  Otherwise C[m][n] is written when C is set and CT[n][m] when CT is set.
// M, N must be multiples of 128, K a multiple of 64, ld* multiples of 8.
// kRoleNsX: the standard-iteration update X' = B X + beta X (rectangular,
// epilogue reading D = X^T as contiguous runs).  kRoleBack: the final
// rectangular product, whose output goes to the fused row-sparse update
// (sink) instead of memory; kRoleRect: the restart's rectangular product.
enum GemmRole { kRoleGram = 0, kRolePoly = 1, kRoleSymm = 2, kRoleRect = 3, kRoleNsX = 4,
                kRoleBack = 5 };

struct GemmDesc {
  int role;
  const f16* A; long long sA; int lda;
  const f16* B; long long sB; int ldb;
  // b_kn (rectangular roles): B is given as its transpose, K x N stored
  // B[k * ldb + n] (N contiguous), and read through transposing LDS reads;
  // rows k >= K are never read
  bool b_kn;
  f16* C; long long sC; int ldc;
  f16* CT; long long sCT; int ldct;
  const f16* D; long long sD; int ldd;
  int M, N, K, batch;
  bool lower, epilogue;
  float alpha, beta, gamma;
  // gamma is added on the diagonal elements (i, i) with i < gdiag only (0:
  // all of them).  The Gram-side products pass the unpadded side, so the
  // zero padding block stays exactly zero instead of growing as a power of
  // the polynomial's constant term (which overflows fp16 after about nine
  // iterations without a restart and then turns the cross terms into NaN).
  int gdiag;
  // Operand rows known to be zero: A's rows >= zrows and B's rows (its
  // columns with b_kn) >= zcols, the zero padding of the Gram-side
  // matrices and of X.  Output blocks wholly past them accumulate exactly
  // +0, which the kernel then keeps without running their MFMAs.  0: none
  // known (M, N).
  int zrows, zcols;
  double trace_flops;   // algorithmic flops of this launch, for the timing trace
  double trace_bytes;   // algorithmic HBM bytes of this launch (operands once, outputs once)
  // Fused row-sparse update (rectangular products only): the output in rows
  // layout (the C pass when sink == 1, the CT pass when sink == 2) is not
  // stored; instead, for output row r < kval and column c < mval,
  //   W[b][idx[b][r]][c] = fma(-lr, O[r][c], W[...])   (when W has pointers)
  //   Oout[b * sO + r * mval + c] = O[r][c]           (when Oout is set;
  //                                                    sO >= kval * mval).
  int sink;
  BatchPtr<float> W;
  long long ldw;
  const int* idx;
  float lr;
  f16* Oout;
  long long sO;            // elements between the Oout blocks of consecutive matrices
  int kval, mval, nrows;   // nrows: rows of W (row indices outside are skipped)
  // rows layout from the C pass (sink == 1) only: when set, the 128-column
  // block sums of squares of every output row in the order normalize.hip
  // fixes, part[(b * kval + r) * nblk + column / 128]
  float* part;
  int nblk;
};
// Records e as the calling thread's last HIP error (dion3_last_hip_error)
// and returns DION3_ERR_HIP.
dion3_status note_hip_error(hipError_t e);

// Launches the product; records it in the timing trace (when enabled) under
// "<role>_<tile edge>", e.g. "gemm_symm_256".
hipError_t launch_gemm(const GemmDesc& d, hipStream_t s);
// Up to kGemmMaxSeg lower-triangle products of one role and epilogue
// (alpha, beta, gamma, addend or none) in one launch: each XCD takes a
// contiguous share of every product's tiles, the products in the given
// order (longest tiles first keeps the tail short).  The large tile is used
// when all of them together have 512 large tiles.
constexpr int kGemmMaxSeg = 4;
hipError_t launch_gemm_multi(const GemmDesc* d, int n, hipStream_t s);

// Optional kernel timing trace (benchmarks): while enabled, each launch is
// timed by HIP events on its stream and its algorithmic work noted.  Inside
// one library call (a TraceChain on the call's stream) the kernels follow
// one another with nothing in between, so a kernel's start is the previous
// kernel's end event and only one event is recorded per kernel; anything
// else enqueued in between must call trace_break() first.
struct TraceScope {
  TraceScope(const char* name, double flops, double bytes, hipStream_t s);
  ~TraceScope();
  int slot;
  hipStream_t stream;
};
struct TraceChain {
  explicit TraceChain(hipStream_t s);
  ~TraceChain();
};
void trace_break();

// Per-row l1 (optional) and sum of squares in fp64, one wave per row.
hipError_t launch_row_score_f32(BatchPtr<const float> M, int batch, int n, int m, long long ld,
                                double* l1, double* sq, hipStream_t s);
// M <- M + G (fp32) fused with the scoring of the updated rows.
hipError_t launch_accum_score_f32(BatchPtr<float> M, BatchPtr<const float> G, int batch, int n, int m,
                                  long long ld, double* l1, double* sq, hipStream_t s);
hipError_t launch_row_score_f16(BatchPtr<const f16> X, int batch, int n, int m, long long ld,
                                double* sq, hipStream_t s);

// Top-k on l1 (ties to lowest index), ascending idx[b][k]; scale[b] =
// 1 / (sqrt(sum_{i in S} sq[i]) + eps).  k == n selects every row.
hipError_t launch_topk(const double* l1, const double* sq, int batch, int n, int k, int* idx,
                       double* scale, double eps, hipStream_t s);

// Gather of the selected rows into X[b][r][j] and/or XT[b][j][r] =
// fp16(M[b][idx[r]][j] * scale[b]) for r < k, j < m, zero in the padding up
// to kp x mp (X) and mp x kp (XT); a null X or XT is not written.  With decay,
// M[b][idx[r]][j] *= mu (one fp32 multiply).  idx == nullptr: identity.
hipError_t launch_gather_f32(BatchPtr<float> M, int batch, int n, int m, long long ld,
                             const int* idx, int k, const double* scale, float mu, bool decay,
                             f16* X, f16* XT, long long sX, int kp, int mp, hipStream_t s);
hipError_t launch_gather_f16(BatchPtr<const f16> Xin, int batch, int m, long long ld, int k,
                             const double* scale, f16* X, f16* XT, long long sX, int kp, int mp,
                             hipStream_t s);

// The whole Gram Newton-Schulz (the schedule in cfg) for matrices whose Gram
// side pads to 128, one workgroup per matrix: X_math [128][Lp] and its
// transpose XT [Lp][128] per matrix at stride sX (halves), Y/YT the second
// pair written by a restart.  The result goes to the fused update (W, idx,
// lr; rows layout = X_math, or its transpose when tr) and/or Oout ([k][m]
// per matrix, matrices sO elements apart).
hipError_t launch_gram_ns_small(f16* X, f16* XT, f16* Y, f16* YT, long long sX, int batch, int Lp,
                                bool tr, const dion3_ns_cfg& cfg, BatchPtr<float> W, long long ldw,
                                const int* idx, float lr, f16* Oout, long long sO, int kval,
                                int mval, int nrows,
                                double trace_flops, hipStream_t s);

// Per-neuron normalization of O ([k][m] fp16 rows per matrix, matrices sO
// elements apart) and the update W[idx[i]] -= lr * U_i; V holds one fp32
// state per row of each matrix.  part ([batch][k][ceil(m / 128)] fp32) holds
// the rows' 128-column block sums of squares in the fixed order of
// normalize.hip: already written by the product that wrote O when
// part_ready, else computed here from O; the region must also hold, after
// those sums (16-byte aligned), 16 bytes per matrix per 256 rows of scratch.
// stats ([batch][k]) is scratch.
hipError_t launch_normalize(const f16* O, long long sO, int batch, int k, int m, const int* idx,
                            BatchPtr<float> V, float beta2, float eps, BatchPtr<float> W,
                            long long ldw, float lr, float* part, bool part_ready, float2* stats,
                            hipStream_t s);

}  // namespace dion3
