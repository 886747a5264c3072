// fp16 MFMA GEMM for gfx950 with fp32 accumulation: the Gram products,
// the symmetric "A^2 + B" products and the rectangular multiply-back of
// Gram Newton-Schulz ("Dion3: Full-Stack Orthogonal Updates", agihunt.info,
// level-1 and level-2 paragraphs: symmetric products need only the lower
// triangle, which is then copied to the upper one).
//
// Block tile 128 x 128, K step 64, 256 threads = 4 waves in a 2 x 2 grid,
// each wave owning a 64 x 64 sub-tile as 2 x 2 v_mfma_f32_32x32x16_f16.
// Operand tiles are staged through LDS in K-contiguous rows (padded by 8
// halves) with a register prefetch of the next K step and two LDS buffers,
// so one barrier per K step.  Operands stored with M/N contiguous ("col"
// form) are transposed while being written to LDS.
#include "dion3_internal.h"

namespace dion3 {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK + 8;   // halves per LDS row (144 bytes: 16-byte aligned, bank-skewed)

typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const f16* A; const f16* B; f16* C; const f16* D;
  long long sA, sB, sC, sD;
  int lda, ldb, ldc, ldd;
  int K;
  int tilesN, tilesPerMat, total;
  float alpha, beta, gamma;
};

__device__ __forceinline__ void tri_index(int t, int& bi, int& bj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  bi = i;
  bj = t - i * (i + 1) / 2;
}

template <bool COL>
__device__ __forceinline__ void load_tile(const f16* __restrict__ g, int ld, int r0, int k0, int tid,
                                          half8 (&reg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + 256 * i;
    if (!COL) {
      int row = c >> 3, kc = c & 7;
      reg[i] = *(const half8*)(g + (long long)(r0 + row) * ld + k0 + kc * 8);
    } else {
      int kr = c >> 4, rc = c & 15;
      reg[i] = *(const half8*)(g + (long long)(k0 + kr) * ld + r0 + rc * 8);
    }
  }
}

template <bool COL>
__device__ __forceinline__ void store_tile(f16* __restrict__ s, int tid, const half8 (&reg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + 256 * i;
    if (!COL) {
      int row = c >> 3, kc = c & 7;
      *(half8*)(s + row * LDSK + kc * 8) = reg[i];
    } else {
      int kr = c >> 4, rc = c & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) s[(rc * 8 + e) * LDSK + kr] = reg[i][e];
    }
  }
}

// ROLE only names the instance (0 Gram, 1 polynomial, 2 symmetric product,
// 3 rectangular) so that profilers report each role as its own kernel.
template <int ROLE, bool A_COL, bool B_COL, bool C_T, bool LOWER, bool EPI>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) f16 sA[2][BM * LDSK];
  __shared__ __attribute__((aligned(16))) f16 sB[2][BN * LDSK];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // that each XCD works on a contiguous run of tiles (mostly the same
  // matrices), which keeps their operand panels in that XCD's L2.
  const int w = blockIdx.x, G = p.total;
  const int q = G >> 3, rem = G & 7, xcd = w & 7, slot = w >> 3;
  const int lid = xcd * q + min(xcd, rem) + slot;
  const int b = lid / p.tilesPerMat;
  const int t = lid - b * p.tilesPerMat;
  int bi, bj;
  if (LOWER) {
    tri_index(t, bi, bj);
  } else {
    bi = t / p.tilesN;
    bj = t - bi * p.tilesN;
  }
  const int m0 = bi * BM, n0 = bj * BN;

  const f16* __restrict__ Ab = p.A + (long long)b * p.sA;
  const f16* __restrict__ Bb = p.B + (long long)b * p.sB;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  half8 ra[4], rb[4];
  const int nk = p.K / BK;
  load_tile<A_COL>(Ab, p.lda, m0, 0, tid, ra);
  load_tile<B_COL>(Bb, p.ldb, n0, 0, tid, rb);
  store_tile<A_COL>(sA[0], tid, ra);
  store_tile<B_COL>(sB[0], tid, rb);
  __syncthreads();

  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_tile<A_COL>(Ab, p.lda, m0, (kt + 1) * BK, tid, ra);
      load_tile<B_COL>(Bb, p.ldb, n0, (kt + 1) * BK, tid, rb);
    }
    const f16* a_s = sA[cur] + (wm * 64 + frag_row) * LDSK + frag_k;
    const f16* b_s = sB[cur] + (wn * 64 + frag_row) * LDSK + frag_k;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const half8*)(a_s + i * 32 * LDSK + kk * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *(const half8*)(b_s + j * 32 * LDSK + kk * 16);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_tile<A_COL>(sA[cur ^ 1], tid, ra);
      store_tile<B_COL>(sB[cur ^ 1], tid, rb);
    }
    __syncthreads();
  }

  // Epilogue.  Accumulator layout of the 32x32 MFMA: lane l, value v holds
  // row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the 32x32 block.
  f16* __restrict__ Cb = p.C + (long long)b * p.sC;
  const f16* __restrict__ Db = EPI && p.D ? p.D + (long long)b * p.sD : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int cc = n0 + wn * 64 + j * 32 + (lane & 31);
        float val = acc[i][j][v];
        if (EPI) {
          val *= p.alpha;
          if (Db) val += p.beta * (float)Db[(long long)rr * p.ldd + cc];
          if (rr == cc) val += p.gamma;
        }
        const f16 h = (f16)val;
        if (LOWER) {
          if (rr >= cc) {
            Cb[(long long)rr * p.ldc + cc] = h;
            Cb[(long long)cc * p.ldc + rr] = h;
          }
        } else if (C_T) {
          Cb[(long long)cc * p.ldc + rr] = h;
        } else {
          Cb[(long long)rr * p.ldc + cc] = h;
        }
      }
}

template <int ROLE, bool A_COL, bool B_COL, bool C_T, bool LOWER, bool EPI>
hipError_t launch(const GemmDesc& d, hipStream_t s) {
  GemmArgs p;
  p.A = d.A; p.B = d.B; p.C = d.C; p.D = d.D;
  p.sA = d.sA; p.sB = d.sB; p.sC = d.sC; p.sD = d.sD;
  p.lda = d.lda; p.ldb = d.ldb; p.ldc = d.ldc; p.ldd = d.ldd;
  p.K = d.K;
  const int tm = d.M / BM, tn = d.N / BN;
  p.tilesN = tn;
  p.tilesPerMat = LOWER ? tm * (tm + 1) / 2 : tm * tn;
  const long long total = (long long)p.tilesPerMat * d.batch;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  p.total = (int)total;
  p.alpha = d.alpha; p.beta = d.beta; p.gamma = d.gamma;
  hipLaunchKernelGGL((k_gemm<ROLE, A_COL, B_COL, C_T, LOWER, EPI>), dim3(p.total), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M % BM || d.N % BN || d.K % BK || d.K <= 0 || d.batch <= 0) return hipErrorInvalidValue;
  if (d.lower && d.M != d.N) return hipErrorInvalidValue;
  switch (d.role) {
    case kRoleGram:
      if (!d.lower || d.c_t || d.epilogue || d.a_col != d.b_col) break;
      return d.a_col ? launch<kRoleGram, true, true, false, true, false>(d, s)
                     : launch<kRoleGram, false, false, false, true, false>(d, s);
    case kRolePoly:
      if (!d.lower || d.c_t || !d.epilogue || d.a_col || d.b_col) break;
      return launch<kRolePoly, false, false, false, true, true>(d, s);
    case kRoleSymm:
      if (!d.lower || d.c_t || d.epilogue || d.a_col || d.b_col) break;
      return launch<kRoleSymm, false, false, false, true, false>(d, s);
    case kRoleRect:
      if (d.lower || d.epilogue || d.a_col) break;
      if (d.b_col && !d.c_t) return launch<kRoleRect, false, true, false, false, false>(d, s);
      if (!d.b_col && d.c_t) return launch<kRoleRect, false, false, true, false, false>(d, s);
      if (!d.b_col && !d.c_t) return launch<kRoleRect, false, false, false, false, false>(d, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace dion3
