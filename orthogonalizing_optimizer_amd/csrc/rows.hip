// Row kernels of the Dion3 step on gfx950: l1 scoring, top-k selection and
// gather + normalize + momentum decay (the row-sparse weight update is fused
// into the epilogue of the final multiply-back product)
// ("Dion3: Full-Stack Orthogonal Updates", agihunt.info, level-3 paragraph:
// k = ceil(f n) rows picked by l1 norm, only those weight rows updated, only
// those momentum rows decayed by mu, the rest left untouched).
//
// Scoring and gather stream HBM: scoring runs one 64-lane wave per row, 16-byte
// loads when the row is 16-byte aligned.  Every reduction runs in a fixed
// order in fp64, so results are deterministic run to run.
#include "dion3_internal.h"

namespace dion3 {
namespace {

typedef f16 half4 __attribute__((ext_vector_type(4)));
typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------- scoring

__global__ __launch_bounds__(256) void k_row_score_f32(BatchPtr<const float> M, int n, int m,
                                                       long long ld, double* __restrict__ l1,
                                                       double* __restrict__ sq) {
  const int b = blockIdx.y;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float* __restrict__ src = M.get(b) + (long long)row * ld;
  double a0 = 0.0, a1 = 0.0, q0 = 0.0, q1 = 0.0;
  if (((uintptr_t)src & 15) == 0 && (m & 3) == 0) {
    const float4* s4 = (const float4*)src;
    const int m4 = m >> 2;
    int j = lane;
    // single-use stream: nontemporal loads (measured 6-9 % faster on the 7B set)
    const f32x4* v4 = (const f32x4*)s4;
    for (; j + 64 < m4; j += 128) {
      const f32x4 xv = __builtin_nontemporal_load(v4 + j), yv = __builtin_nontemporal_load(v4 + j + 64);
      const float4 x = make_float4(xv[0], xv[1], xv[2], xv[3]);
      const float4 y = make_float4(yv[0], yv[1], yv[2], yv[3]);
      a0 += (double)fabsf(x.x) + (double)fabsf(x.y) + (double)fabsf(x.z) + (double)fabsf(x.w);
      a1 += (double)fabsf(y.x) + (double)fabsf(y.y) + (double)fabsf(y.z) + (double)fabsf(y.w);
      q0 += (double)x.x * x.x + (double)x.y * x.y + (double)x.z * x.z + (double)x.w * x.w;
      q1 += (double)y.x * y.x + (double)y.y * y.y + (double)y.z * y.z + (double)y.w * y.w;
    }
    if (j < m4) {
      const float4 x = s4[j];
      a0 += (double)fabsf(x.x) + (double)fabsf(x.y) + (double)fabsf(x.z) + (double)fabsf(x.w);
      q0 += (double)x.x * x.x + (double)x.y * x.y + (double)x.z * x.z + (double)x.w * x.w;
    }
  } else {
    for (int j = lane; j < m; j += 64) {
      const double x = (double)src[j];
      a0 += fabs(x);
      q0 += x * x;
    }
  }
  const double a = wave_sum(a0 + a1), q = wave_sum(q0 + q1);
  if (lane == 0) {
    if (l1) l1[(long long)b * n + row] = a;
    sq[(long long)b * n + row] = q;
  }
}

// Gradient accumulation fused into scoring: M <- M + G (one fp32 add per
// element, written back) and the l1 / sum of squares of the updated row.
__global__ __launch_bounds__(256) void k_accum_score_f32(BatchPtr<float> M, BatchPtr<const float> G,
                                                         int n, int m, long long ld,
                                                         double* __restrict__ l1,
                                                         double* __restrict__ sq) {
  const int b = blockIdx.y;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  float* __restrict__ dst = M.get(b) + (long long)row * ld;
  const float* __restrict__ g = G.get(b) + (long long)row * ld;
  double a = 0.0, q = 0.0;
  if (((uintptr_t)dst & 15) == 0 && ((uintptr_t)g & 15) == 0 && (m & 3) == 0) {
    float4* d4 = (float4*)dst;
    const float4* g4 = (const float4*)g;
    // single-use streams: nontemporal loads and store (measured 6 % faster)
    for (int j = lane; j < (m >> 2); j += 64) {
      const f32x4 xv = __builtin_nontemporal_load((const f32x4*)(d4 + j));
      const f32x4 yv = __builtin_nontemporal_load((const f32x4*)(g4 + j));
      const float4 z = make_float4(xv[0] + yv[0], xv[1] + yv[1], xv[2] + yv[2], xv[3] + yv[3]);
      __builtin_nontemporal_store(f32x4{z.x, z.y, z.z, z.w}, (f32x4*)(d4 + j));
      a += (double)fabsf(z.x) + (double)fabsf(z.y) + (double)fabsf(z.z) + (double)fabsf(z.w);
      q += (double)z.x * z.x + (double)z.y * z.y + (double)z.z * z.z + (double)z.w * z.w;
    }
  } else {
    for (int j = lane; j < m; j += 64) {
      const float z = dst[j] + g[j];
      dst[j] = z;
      a += fabs((double)z);
      q += (double)z * z;
    }
  }
  a = wave_sum(a);
  q = wave_sum(q);
  if (lane == 0) {
    if (l1) l1[(long long)b * n + row] = a;
    sq[(long long)b * n + row] = q;
  }
}

__global__ __launch_bounds__(256) void k_row_score_f16(BatchPtr<const f16> X, int n, int m,
                                                       long long ld, double* __restrict__ sq) {
  const int b = blockIdx.y;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const f16* __restrict__ src = X.get(b) + (long long)row * ld;
  double q = 0.0;
  if (((uintptr_t)src & 15) == 0 && (m & 7) == 0) {
    const half8* s8 = (const half8*)src;
    for (int j = lane; j < (m >> 3); j += 64) {
      const half8 x = s8[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) q += (double)x[e] * (double)x[e];
    }
  } else {
    for (int j = lane; j < m; j += 64) {
      const double x = (double)src[j];
      q += x * x;
    }
  }
  q = wave_sum(q);
  if (lane == 0) sq[(long long)b * n + row] = q;
}

// ------------------------------------------------------------- top-k

constexpr int TK_THREADS = 1024;

// Exclusive prefix sum over the block (one value per thread); returns the
// block total through `total`.
__device__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < TK_THREADS; off <<= 1) {
    const int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  total = sh[TK_THREADS - 1];
  __syncthreads();
  return incl - v;
}

// One workgroup per matrix.  Scores are non-negative doubles, so their bit
// patterns order like the values; an MSB-first 8-bit radix select narrows
// the k-th largest key down to a prefix P of its top bytes (mask): rows with
// masked key > P are taken, and of the rows with masked key == P the
// lowest-index need_eq ones, compacted in index order.  The select stops as
// soon as every remaining candidate is taken (for distinct scores after two
// or three bytes); the set is the same as with the full 64-bit threshold.
__global__ __launch_bounds__(TK_THREADS) void k_topk(const double* __restrict__ l1,
                                                     const double* __restrict__ sq, int n, int k,
                                                     int* __restrict__ idx,
                                                     double* __restrict__ scale, double eps) {
  __shared__ unsigned hist[256];
  __shared__ unsigned wsum_sh[4];
  __shared__ int scan_sh[TK_THREADS];
  __shared__ double red_sh[TK_THREADS];
  __shared__ unsigned long long prefix_sh;
  __shared__ int rem_sh, done_sh;

  const int b = blockIdx.x, tid = threadIdx.x;
  const double* __restrict__ sc = l1 + (long long)b * n;
  const double* __restrict__ q = sq + (long long)b * n;
  int* __restrict__ out = idx + (long long)b * k;

  unsigned long long T = 0, mask = 0;
  int need_eq = 0;
  const bool all = (k >= n);
  if (!all) {
    unsigned long long prefix = 0;
    int rem = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += TK_THREADS) {
        const unsigned long long key = (unsigned long long)__double_as_longlong(sc[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // The digit: the largest d whose count of candidates with digit >= d
      // reaches rem.  Thread t < 256 holds digit 255 - t; an inclusive scan
      // over t (in-wave shuffles, then the wave totals) gives those counts.
      const int d = 255 - tid;
      unsigned h = 0, incl = 0;
      if (tid < 256) {
        h = hist[d];
        incl = h;
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned t = __shfl_up(incl, o, 64);
          if ((tid & 63) >= o) incl += t;
        }
        if ((tid & 63) == 63) wsum_sh[tid >> 6] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < (tid >> 6); ++w) incl += wsum_sh[w];
        const unsigned excl = incl - h;       // candidates with a larger digit
        if (excl < (unsigned)rem && incl >= (unsigned)rem) {   // exactly one thread
          prefix_sh = prefix | ((unsigned long long)d << shift);
          rem_sh = rem - (int)excl;
          done_sh = (h == (unsigned)(rem - (int)excl));
        }
      }
      __syncthreads();
      prefix = prefix_sh;
      rem = rem_sh;
      mask |= 255ull << shift;
      const bool done = done_sh != 0;
      __syncthreads();
      if (done) break;
    }
    T = prefix;
    need_eq = rem;
  }

  // Contiguous chunk per thread, so prefix sums follow index order.
  const int per = (n + TK_THREADS - 1) / TK_THREADS;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  int n_eq = 0;
  if (!all)
    for (int i = c0; i < c1; ++i)
      n_eq += (((unsigned long long)__double_as_longlong(sc[i]) & mask) == T);
  int tot;
  const int eq_start = all ? 0 : block_exclusive_scan(n_eq, scan_sh, tot);
  int n_sel = 0;
  int eqb = eq_start;
  for (int i = c0; i < c1; ++i) {
    bool take = all;
    if (!all) {
      const unsigned long long key = (unsigned long long)__double_as_longlong(sc[i]) & mask;
      take = key > T || (key == T && eqb < need_eq);
      eqb += (key == T);
    }
    n_sel += take;
  }
  int pos = block_exclusive_scan(n_sel, scan_sh, tot);
  // Second pass over the chunk: write the taken indices in index order and
  // sum their squares (fixed order, then a fixed tree over the block).
  double part = 0.0;
  eqb = eq_start;
  for (int i = c0; i < c1; ++i) {
    bool take = all;
    if (!all) {
      const unsigned long long key = (unsigned long long)__double_as_longlong(sc[i]) & mask;
      take = key > T || (key == T && eqb < need_eq);
      eqb += (key == T);
    }
    if (take && pos < k) {
      out[pos++] = i;
      part += q[i];
    }
  }
  red_sh[tid] = part;
  __syncthreads();
  for (int off = TK_THREADS / 2; off >= 1; off >>= 1) {
    if (tid < off) red_sh[tid] += red_sh[tid + off];
    __syncthreads();
  }
  if (tid == 0) scale[b] = 1.0 / (sqrt(red_sh[0]) + eps);
}

// Top-k for matrices of at most 256 rows, one thread per row: a row's rank
// is the number of rows ahead of it (a larger score, or an equal one at a
// lower index, scores compared as the same fp64 bit patterns as k_topk), the
// rows of rank < k are taken and written in index order through wave
// ballots, and ||X||_F^2 goes through k_topk's fixed tree (whose levels above
// 256 only add zeros when n <= 256), so idx and scale are k_topk's bit for
// bit with a handful of barriers instead of about seventy.
constexpr int TKS_THREADS = 256;

__global__ __launch_bounds__(TKS_THREADS) void k_topk_small(const double* __restrict__ l1,
                                                          const double* __restrict__ sq, int n,
                                                          int k, int* __restrict__ idx,
                                                          double* __restrict__ scale, double eps) {
  __shared__ unsigned long long key_sh[TKS_THREADS];
  __shared__ int wcnt_sh[TKS_THREADS / 64];
  __shared__ double red_sh[TKS_THREADS];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool all = k >= n, valid = tid < n;
  unsigned long long key = 0;
  if (!all && valid) key = (unsigned long long)__double_as_longlong(l1[(long long)b * n + tid]);
  key_sh[tid] = key;
  __syncthreads();
  bool take = valid;
  if (!all && valid) {
    int ahead = 0;
    for (int j = 0; j < n; ++j) {
      const unsigned long long kj = key_sh[j];
      ahead += (kj > key) || (kj == key && j < tid);
    }
    take = ahead < k;
  }
  const unsigned long long bal = __ballot(take);
  if (lane == 0) wcnt_sh[w] = __popcll(bal);
  __syncthreads();
  int pos = __popcll(bal & ((1ull << lane) - 1ull));
  for (int v = 0; v < w; ++v) pos += wcnt_sh[v];
  if (take) idx[(long long)b * k + pos] = tid;
  red_sh[tid] = take ? sq[(long long)b * n + tid] : 0.0;
  __syncthreads();
  for (int off = TKS_THREADS / 2; off >= 1; off >>= 1) {
    if (tid < off) red_sh[tid] += red_sh[tid + off];
    __syncthreads();
  }
  if (tid == 0) scale[b] = 1.0 / (sqrt(red_sh[0]) + eps);
}

// ------------------------------------------------------------- gather

// One block per 64 selected rows x 256 columns: reads 1 KB of each selected
// row of M, writes X in rows layout directly and/or, through an LDS tile, its
// transpose XT (eight lanes per 128-byte run of an XT row), whichever of the
// two is not null: the layout the products of the Gram iteration read, or
// both for the paths that read both; with DECAY it also writes the rows of M
// back times mu.  (When only the rows layout is wanted, k_gather_rows below
// does the same with one 16-byte load per thread.)  The rows of M are read and
// written once, and X and XT (read again only by the next products) are far
// larger than the caches, so the fp32 loads and all stores carry the
// nontemporal hint (measured on the 7B set: 10-15 % less kernel time than
// plain accesses with one thread per XT run, bitwise the same outputs).
constexpr int GR = 64, GC = 256, GPAD = 8;

template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ src, int c, int m, float (&v)[4]) {
  if (sizeof(T) == 4 && c + 3 < m && ((uintptr_t)src & 15) == 0) {
    const f32x4 x = __builtin_nontemporal_load((const f32x4*)src);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else if (sizeof(T) == 2 && c + 3 < m && ((uintptr_t)src & 7) == 0) {
    const half4 x = *(const half4*)src;
    v[0] = (float)x[0]; v[1] = (float)x[1]; v[2] = (float)x[2]; v[3] = (float)x[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = c + e < m ? (float)src[e] : 0.0f;
  }
}

__device__ __forceinline__ void decay4(float* __restrict__ src, int c, int m, float mu,
                                       const float (&v)[4]) {
  if (c + 3 < m && ((uintptr_t)src & 15) == 0) {
    const f32x4 d = {mu * v[0], mu * v[1], mu * v[2], mu * v[3]};
    __builtin_nontemporal_store(d, (f32x4*)src);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < m) src[e] = mu * v[e];
  }
}

template <typename T, bool DECAY>
__global__ __launch_bounds__(256) void k_gather(BatchPtr<T> M, int n, int m, long long ld,
                                                const int* __restrict__ idx, int k,
                                                const double* __restrict__ scale, float mu,
                                                f16* __restrict__ X, f16* __restrict__ XT,
                                                long long sX, int kp, int mp) {
  __shared__ __attribute__((aligned(16))) f16 tile[GR][GC + GPAD];
  const int b = blockIdx.z;
  const int c0 = blockIdx.x * GC, r0 = blockIdx.y * GR;
  const int tid = threadIdx.x;
  const int cl = 4 * (tid & 63);          // 4 columns per thread
  const int rq = tid >> 6;                // rows rq, rq + 4, ..., rq + 60
  const float sc = (float)scale[b];
  // (no arithmetic on a null layout pointer: the tests below must stay)
  f16* __restrict__ Xb = X ? X + (long long)b * sX : nullptr;
  f16* __restrict__ XTb = XT ? XT + (long long)b * sX : nullptr;
  T* base = M.get(b);
  const int c = c0 + cl;
  if (c < mp) {
    // the rows' indices stay in registers for the decay: reading them again
    // after the loads (dependent global reads before the first store) cost
    // about a quarter of the kernel's time
    float v[16][4];
    int rows[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = r0 + rq + 4 * i;
      int row = -1;
      if (r < k) {
        row = idx ? idx[(long long)b * k + r] : r;
        if (row >= n) row = -1;
      }
      rows[i] = row;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = 0.0f;
      if (row >= 0 && c < m) load4<T>(base + (long long)row * ld + c, c, m, v[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = rq + 4 * i, r = r0 + rl;
      if constexpr (DECAY) {
        if (rows[i] >= 0 && c < m)
          decay4((float*)(base + (long long)rows[i] * ld + c), c, m, mu, v[i]);
      }
      half4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // X = fp16(fl32(M * scale)): round the product to fp32 first.  Left
        // alone, the compiler fuses some of these multiplies with the
        // conversion into a mixed-precision fma that rounds once, so equal
        // inputs could round differently from element to element.
        float t = v[i][e] * sc;
        asm("" : "+v"(t));
        h[e] = (f16)t;
      }
      if (XTb) *(half4*)&tile[rl][cl] = h;
      if (Xb) __builtin_nontemporal_store(h, (half4*)(Xb + (long long)r * mp + c));
    }
  }
  if (!XTb) return;   // uniform: from the kernel argument
  __syncthreads();
  // transposed: XT[c0 + col][r0 .. r0 + 63], 128 bytes per XT row, eight
  // lanes per row, so that each store instruction writes eight whole
  // 128-byte runs
#pragma unroll
  for (int j = 0; j < GC / 32; ++j) {
    const int col = (tid >> 3) + 32 * j, r8 = tid & 7;
    if (c0 + col < mp) {
      half8 v;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = tile[r8 * 8 + q][col];
      __builtin_nontemporal_store(v, (half8*)(XTb + (long long)(c0 + col) * kp + r0 + r8 * 8));
    }
  }
}

// The gather when only the rows layout X is wanted: one block per 4 selected
// rows x 256 columns, each thread one 16-byte run of one row (load, decayed
// store, fp16 store), with no LDS tile.  The same arithmetic as k_gather,
// element by element.  Short blocks with a single load per thread stream
// faster than k_gather's 16 loads per thread (measured on the 7B shapes:
// 5.6-6.2 against 5.3-5.6 TB/s in isolation).  Grid: x = (kp / 4 row
// blocks) x (column blocks), y = matrices.
template <typename T, bool DECAY>
__global__ __launch_bounds__(256) void k_gather_rows(BatchPtr<T> M, int n, int m, long long ld,
                                                     const int* __restrict__ idx, int k,
                                                     const double* __restrict__ scale, float mu,
                                                     f16* __restrict__ X, long long sX, int mp) {
  // workgroup x: column block fastest, so consecutive workgroups take
  // consecutive 1 KB pieces of the same four rows
  const int b = blockIdx.y;
  const int ncb = (mp + GC - 1) / GC;
  const int rg = blockIdx.x / ncb, cb = blockIdx.x - rg * ncb;
  const int r = rg * 4 + (threadIdx.x >> 6);
  const int c = cb * GC + 4 * (threadIdx.x & 63);
  if (c >= mp) return;
  int row = -1;
  if (r < k) {
    row = idx ? idx[(long long)b * k + r] : r;
    if (row >= n) row = -1;
  }
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  T* base = M.get(b);
  if (row >= 0 && c < m) {
    load4<T>(base + (long long)row * ld + c, c, m, v);
    if constexpr (DECAY) decay4((float*)(base + (long long)row * ld + c), c, m, mu, v);
  }
  const float sc = (float)scale[b];
  half4 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float t = v[e] * sc;   // rounded to fp32 before the conversion, as in k_gather
    asm("" : "+v"(t));
    h[e] = (f16)t;
  }
  __builtin_nontemporal_store(h, (half4*)(X + (long long)b * sX + (long long)r * mp + c));
}

inline unsigned blocks_for(long long rows) { return (unsigned)((rows + 3) / 4); }

}  // namespace

hipError_t launch_row_score_f32(BatchPtr<const float> M, int batch, int n, int m, long long ld,
                                double* l1, double* sq, hipStream_t s) {
  hipLaunchKernelGGL(k_row_score_f32, dim3(blocks_for(n), batch), dim3(256), 0, s, M, n, m, ld, l1,
                     sq);
  return hipGetLastError();
}

hipError_t launch_accum_score_f32(BatchPtr<float> M, BatchPtr<const float> G, int batch, int n, int m,
                                  long long ld, double* l1, double* sq, hipStream_t s) {
  hipLaunchKernelGGL(k_accum_score_f32, dim3(blocks_for(n), batch), dim3(256), 0, s, M, G, n, m, ld,
                     l1, sq);
  return hipGetLastError();
}

hipError_t launch_row_score_f16(BatchPtr<const f16> X, int batch, int n, int m, long long ld,
                                double* sq, hipStream_t s) {
  hipLaunchKernelGGL(k_row_score_f16, dim3(blocks_for(n), batch), dim3(256), 0, s, X, n, m, ld, sq);
  return hipGetLastError();
}

hipError_t launch_topk(const double* l1, const double* sq, int batch, int n, int k, int* idx,
                       double* scale, double eps, hipStream_t s) {
  if (n <= TKS_THREADS)
    hipLaunchKernelGGL(k_topk_small, dim3(batch), dim3(TKS_THREADS), 0, s, l1, sq, n, k, idx,
                       scale, eps);
  else
    hipLaunchKernelGGL(k_topk, dim3(batch), dim3(TK_THREADS), 0, s, l1, sq, n, k, idx, scale, eps);
  return hipGetLastError();
}

hipError_t launch_gather_f32(BatchPtr<float> M, int batch, int n, int m, long long ld,
                             const int* idx, int k, const double* scale, float mu, bool decay,
                             f16* X, f16* XT, long long sX, int kp, int mp, hipStream_t s) {
  if (X && !XT) {
    const dim3 grid((kp / 4) * ((mp + GC - 1) / GC), batch);
    if (decay)
      hipLaunchKernelGGL((k_gather_rows<float, true>), grid, dim3(256), 0, s, M, n, m, ld, idx, k,
                         scale, mu, X, sX, mp);
    else
      hipLaunchKernelGGL((k_gather_rows<float, false>), grid, dim3(256), 0, s, M, n, m, ld, idx, k,
                         scale, mu, X, sX, mp);
    return hipGetLastError();
  }
  const dim3 grid((mp + GC - 1) / GC, kp / GR, batch);
  if (decay)
    hipLaunchKernelGGL((k_gather<float, true>), grid, dim3(256), 0, s, M, n, m, ld, idx, k, scale,
                       mu, X, XT, sX, kp, mp);
  else
    hipLaunchKernelGGL((k_gather<float, false>), grid, dim3(256), 0, s, M, n, m, ld, idx, k, scale,
                       mu, X, XT, sX, kp, mp);
  return hipGetLastError();
}

hipError_t launch_gather_f16(BatchPtr<const f16> Xin, int batch, int m, long long ld, int k,
                             const double* scale, f16* X, f16* XT, long long sX, int kp, int mp,
                             hipStream_t s) {
  if (X && !XT) {
    const dim3 grid((kp / 4) * ((mp + GC - 1) / GC), batch);
    hipLaunchKernelGGL((k_gather_rows<const f16, false>), grid, dim3(256), 0, s, Xin, k, m, ld,
                       nullptr, k, scale, 1.0f, X, sX, mp);
    return hipGetLastError();
  }
  const dim3 grid((mp + GC - 1) / GC, kp / GR, batch);
  hipLaunchKernelGGL((k_gather<const f16, false>), grid, dim3(256), 0, s, Xin, k, m, ld, nullptr, k,
                     scale, 1.0f, X, XT, sX, kp, mp);
  return hipGetLastError();
}


}  // namespace dion3
