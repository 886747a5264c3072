// Per-neuron normalization of the orthogonalized update.  The pages say that
// Dion3 inherits NorMuon's per-neuron normalization ("Dion3 Cuts Muon
// Optimizer Time by Up to 6x", quasa.io, section "Dion3's fastest path is a
// combined systems stack") and that it runs in float32 ("Dion3: Full-Stack
// Orthogonal Updates", agihunt.info, limitations paragraph); they give no
// formula.  The reading implemented here, for the k selected rows of one
// matrix with orthogonalized rows O (k x m, fp16) and a float32 state V (one
// entry per row of the matrix):
//   q_i = mean_j O_ij^2,  V[S_i] <- beta2 V[S_i] + (1 - beta2) q_i,
//   U_i = O_i / (sqrt(V[S_i]) + eps)  (0 for a zero row with zero state),
//   U  <- U ||O||_F / ||U||_F,  W[S] <- W[S] - lr U.
// Passes, each reduction in a fixed order (results do not depend on the
// launch or on which kernel summed the squares):
//   row block sums: the epilogue of the product that writes O, or
//     k_norm_rows (one wave per selected row) reading O back;
//   k_norm_stats  one thread per row: s_i, the state, r_i = 1/(sqrt(v_i) + eps),
//     and per workgroup the sums behind g = ||O|| / ||U||;
//   k_norm_update g from those sums (in workgroup order), then
//     W[S_i][j] = fma(-lr g r_i, O_ij, W[S_i][j])
#include "dion3_internal.h"

namespace dion3 {
namespace {

typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef f16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per-row sums of squares of O in one fixed order, whatever computes them
// (this kernel from O in memory, or the epilogue of the product that writes O,
// gemm_f16.hip): the row is cut into 128-column blocks; in a block, each of
// the 16 eight-column chunks sums its squares in column order (fp32 fma from
// +0), and the 16 chunk sums combine by the butterfly xor 1, 2, 4, 8 (a
// balanced tree in chunk order).  part[b][i][blk] holds block blk's sum; the
// row's total adds the blocks in increasing order (k_norm_stats).  One wave
// per row, its four 16-lane quarters on four consecutive blocks.
__device__ __forceinline__ float chunk_sumsq(const f16* __restrict__ row, int c, int m, bool vec) {
  float acc = 0.0f;
  if (vec && c + 8 <= m) {
    const half8 h = *(const half8*)(row + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)h[e], (float)h[e], acc);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = c + e < m ? (float)row[c + e] : 0.0f;
      acc = __builtin_fmaf(x, x, acc);
    }
  }
  return acc;
}

__global__ __launch_bounds__(256) void k_norm_rows(const f16* __restrict__ O, long long sO, int k,
                                                   int m, int nblk, float* __restrict__ part) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= k) return;                       // whole waves leave together
  const f16* __restrict__ row = O + (long long)b * sO + (long long)i * m;
  const bool vec = ((uintptr_t)row & 15) == 0;
  const int quarter = lane >> 4, ch = lane & 15;
  for (int b0 = 0; b0 < nblk; b0 += 4) {
    const int blk = b0 + quarter;
    float v = blk < nblk ? chunk_sumsq(row, blk * 128 + ch * 8, m, vec) : 0.0f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
    if (ch == 0 && blk < nblk) part[((long long)b * k + i) * nblk + blk] = v;
  }
}

// One thread per selected row (256 rows per workgroup): the row's sum of
// squares s_i (its block sums in block order), the state update and
// r_i = 1 / (sqrt(v_i) + eps); each workgroup also leaves the fp64 sums of s_i
// and s_i r_i^2 over its rows (a fixed tree) for the scale g.  The
// workgroup's block sums (contiguous in memory) pass through LDS 32 blocks
// of every row at a time, read with consecutive threads on consecutive
// floats.
constexpr int kStatsCols = 32;
__global__ __launch_bounds__(256) void k_norm_stats(const float* __restrict__ part, int k, int m,
                                                    int nblk, const int* __restrict__ idx,
                                                    BatchPtr<float> V, float beta2, float eps,
                                                    float2* __restrict__ stats,
                                                    double2* __restrict__ wsum) {
  __shared__ double sh0[256], sh1[256];
  __shared__ float blk[256][kStatsCols + 1];
  const int b = blockIdx.y, t = threadIdx.x, i0 = blockIdx.x * 256, i = i0 + t;
  const int rows = min(256, k - i0);
  const float* __restrict__ pw = part + ((long long)b * k + i0) * nblk;   // this workgroup's rows
  float s = 0.0f;
  for (int c0 = 0; c0 < nblk; c0 += kStatsCols) {
    const int cols = min(kStatsCols, nblk - c0);
    for (int e = t; e < rows * cols; e += 256) {
      const int r = e / cols, c = e - r * cols;
      blk[r][c] = pw[(long long)r * nblk + c0 + c];
    }
    __syncthreads();
    if (i < k)
      for (int c = 0; c < cols; ++c) s += blk[t][c];
    __syncthreads();
  }
  double a0 = 0.0, a1 = 0.0;
  if (i < k) {
    float* v = V.get(b) + idx[(long long)b * k + i];
    const float q = s / (float)m;
    const float nv = __builtin_fmaf(beta2, *v, (1.0f - beta2) * q);
    *v = nv;
    const float d = sqrtf(nv) + eps;
    const float r = d > 0.0f ? 1.0f / d : 0.0f;
    stats[(long long)b * k + i] = make_float2(s, r);
    a0 = (double)s;
    a1 = (double)s * (double)r * (double)r;
  }
  sh0[t] = a0;
  sh1[t] = a1;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (t < o) {
      sh0[t] += sh0[t + o];
      sh1[t] += sh1[t + o];
    }
    __syncthreads();
  }
  if (t == 0) wsum[(long long)b * gridDim.x + blockIdx.x] = make_double2(sh0[0], sh1[0]);
}

// W[idx[i]][j] = fma(-lr g r_i, O_ij, W[idx[i]][j]): one workgroup per 4 rows
// x 256 columns of O, one wave per row, one 16-byte W run and one 8-byte O
// run per lane (short workgroups with a single load per thread stream faster
// than one wave walking a whole row: measured on the 7B shapes).  Grid:
// x = (row groups of 4) x (256-column blocks), y = matrices.
// The scale g = sqrt(sum_i s_i / sum_i s_i r_i^2) comes from k_norm_stats'
// per-workgroup sums, added in workgroup order (every thread of a matrix gets
// the same bits).
__global__ __launch_bounds__(256) void k_norm_update(const f16* __restrict__ O, long long sO, int k,
                                                     int m, const int* __restrict__ idx,
                                                     BatchPtr<float> W, long long ldw, float lr,
                                                     const float2* __restrict__ stats,
                                                     const double2* __restrict__ wsum, int nwg) {
  // workgroup x: column block fastest, so consecutive workgroups take
  // consecutive pieces of the same four rows
  const int b = blockIdx.y;
  const int ncb = (m + 255) / 256;
  const int rg = blockIdx.x / ncb, cb = blockIdx.x - rg * ncb;
  const int i = rg * 4 + (threadIdx.x >> 6);
  const int j = cb * 256 + 4 * (threadIdx.x & 63);
  if (i >= k || j >= m) return;
  double a0 = 0.0, a1 = 0.0;
  for (int q = 0; q < nwg; ++q) {
    const double2 w2 = wsum[(long long)b * nwg + q];
    a0 += w2.x;
    a1 += w2.y;
  }
  const double g = a1 > 0.0 ? sqrt(a0 / a1) : 0.0;
  const float c = -lr * (float)g * stats[(long long)b * k + i].y;
  const f16* __restrict__ src = O + (long long)b * sO + (long long)i * m;
  float* __restrict__ w = W.get(b) + (long long)idx[(long long)b * k + i] * ldw;
  // both runs are used once, so they stream with the nontemporal hint
  if (j + 3 < m && ((uintptr_t)(w + j) & 15) == 0 && ((uintptr_t)(src + j) & 7) == 0) {
    f32x4 x = __builtin_nontemporal_load((const f32x4*)(w + j));
    const half4 o = __builtin_nontemporal_load((const half4*)(src + j));
    x[0] = __builtin_fmaf(c, (float)o[0], x[0]);
    x[1] = __builtin_fmaf(c, (float)o[1], x[1]);
    x[2] = __builtin_fmaf(c, (float)o[2], x[2]);
    x[3] = __builtin_fmaf(c, (float)o[3], x[3]);
    __builtin_nontemporal_store(x, (f32x4*)(w + j));
  } else {
    for (int e = 0; e < 4 && j + e < m; ++e)
      w[j + e] = __builtin_fmaf(c, (float)src[j + e], w[j + e]);
  }
}

}  // namespace

hipError_t launch_normalize(const f16* O, long long sO, int batch, int k, int m, const int* idx,
                            BatchPtr<float> V, float beta2, float eps, BatchPtr<float> W,
                            long long ldw, float lr, float* part, bool part_ready, float2* stats,
                            hipStream_t s) {
  const dim3 grid((k + 3) / 4, batch);
  const double km = (double)batch * k * m;
  const int nblk = (m + 127) / 128;
  const int nwg = (k + 255) / 256;
  // the per-workgroup sums sit right after the block sums, 16-byte aligned
  double2* wsum = (double2*)(part + (((long long)batch * k * nblk + 3) & ~3LL));
  if (!part_ready) {
    TraceScope ts("norm_rows", 0.0, km * 2.0, s);
    hipLaunchKernelGGL(k_norm_rows, grid, dim3(256), 0, s, O, sO, k, m, nblk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TraceScope ts("norm_stats", 0.0, (double)batch * k * (4.0 * nblk + 8.0), s);
    hipLaunchKernelGGL(k_norm_stats, dim3(nwg, batch), dim3(256), 0, s, part, k, m, nblk, idx, V,
                       beta2, eps, stats, wsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope ts("norm_update", 0.0, km * 10.0, s);
  hipLaunchKernelGGL(k_norm_update, dim3(((k + 3) / 4) * ((m + 255) / 256), batch), dim3(256), 0,
                     s, O, sO, k, m, idx, W, ldw, lr, stats, wsum, nwg);
  return hipGetLastError();
}

}  // namespace dion3
