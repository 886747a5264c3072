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
// Three passes, each reduction in a fixed order (results do not depend on
// the launch):
//   k_norm_rows   one wave per selected row: q, the state, r_i = 1/(sqrt+eps)
//   k_norm_scale  one workgroup per matrix: g = ||O|| / ||U|| from the rows
//   k_norm_update W[S_i][j] = fma(-lr g r_i, O_ij, W[S_i][j])
#include "dion3_internal.h"

namespace dion3 {
namespace {

typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef f16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly over the 64 lanes: every lane ends with the same sum
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Row stats of O (rows [k][m] per matrix, matrices sO apart): s_i = sum of
// squares (fp32 lanes, fixed butterfly), the state update and r_i.
__global__ __launch_bounds__(256) void k_norm_rows(const f16* __restrict__ O, long long sO, int k,
                                                   int m, const int* __restrict__ idx,
                                                   BatchPtr<float> V,
                                                   float beta2, float eps,
                                                   float2* __restrict__ stats) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= k) return;                       // whole waves leave together
  const f16* __restrict__ row = O + (long long)b * sO + (long long)i * m;
  float acc = 0.0f;
  const bool vec = ((uintptr_t)row & 15) == 0;
  int j = 0;
  if (vec) {
    for (; j + 8 * 64 <= m; j += 8 * 64) {
      const half8 h = *(const half8*)(row + j + 8 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)h[e], (float)h[e], acc);
    }
  }
  for (int c = j + lane; c < m; c += 64) {
    const float x = (float)row[c];
    acc = __builtin_fmaf(x, x, acc);
  }
  const float s = wave_sum(acc);
  if (lane == 0) {
    const int r = idx[(long long)b * k + i];
    float* v = V.get(b) + r;
    const float q = s / (float)m;
    const float nv = __builtin_fmaf(beta2, *v, (1.0f - beta2) * q);
    *v = nv;
    const float d = sqrtf(nv) + eps;
    stats[(long long)b * k + i] = make_float2(s, d > 0.0f ? 1.0f / d : 0.0f);
  }
}

// g = sqrt(sum_i s_i / sum_i s_i r_i^2) per matrix (fp64, fixed order).
__global__ __launch_bounds__(256) void k_norm_scale(const float2* __restrict__ stats, int k,
                                                    double* __restrict__ g) {
  __shared__ double sh0[256], sh1[256];
  const int b = blockIdx.x, t = threadIdx.x;
  double a0 = 0.0, a1 = 0.0;
  for (int i = t; i < k; i += 256) {
    const float2 st = stats[(long long)b * k + i];
    a0 += (double)st.x;
    a1 += (double)st.x * (double)st.y * (double)st.y;
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
  if (t == 0) g[b] = sh1[0] > 0.0 ? sqrt(sh0[0] / sh1[0]) : 0.0;
}

// W[idx[i]][j] = fma(-lr g r_i, O_ij, W[idx[i]][j]): one workgroup per 4 rows
// of O, 64 lanes along a row, 4 columns per lane per pass.
__global__ __launch_bounds__(256) void k_norm_update(const f16* __restrict__ O, long long sO, int k,
                                                     int m, const int* __restrict__ idx,
                                                     BatchPtr<float> W, long long ldw, float lr,
                                                     const float2* __restrict__ stats,
                                                     const double* __restrict__ g) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= k) return;
  const float c = -lr * (float)g[b] * stats[(long long)b * k + i].y;
  const f16* __restrict__ src = O + (long long)b * sO + (long long)i * m;
  float* __restrict__ w = W.get(b) + (long long)idx[(long long)b * k + i] * ldw;
  for (int j = 4 * lane; j < m; j += 4 * 64) {
    // one 16-byte W run and one 8-byte O run per lane; both are used once,
    // so they stream with the nontemporal hint (measured 5 % faster)
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
}

}  // namespace

hipError_t launch_normalize(const f16* O, long long sO, int batch, int k, int m, const int* idx,
                            BatchPtr<float> V, float beta2, float eps, BatchPtr<float> W,
                            long long ldw, float lr, float2* stats, double* g, hipStream_t s) {
  const dim3 grid((k + 3) / 4, batch);
  const double km = (double)batch * k * m;
  {
    TraceScope ts("norm_rows", 0.0, km * 2.0, s);
    hipLaunchKernelGGL(k_norm_rows, grid, dim3(256), 0, s, O, sO, k, m, idx, V, beta2, eps,
                       stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TraceScope ts("norm_scale", 0.0, (double)batch * k * 8.0, s);
    hipLaunchKernelGGL(k_norm_scale, dim3(batch), dim3(256), 0, s, stats, k, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope ts("norm_update", 0.0, km * 10.0, s);
  hipLaunchKernelGGL(k_norm_update, grid, dim3(256), 0, s, O, sO, k, m, idx, W, ldw, lr, stats,
                     g);
  return hipGetLastError();
}

}  // namespace dion3
