// fp16 MFMA GEMM for gfx950 with fp32 accumulation: the Gram products,
// the symmetric "A^2 + B" products and the rectangular multiply-back of
// Gram Newton-Schulz ("Dion3: Full-Stack Orthogonal Updates", agihunt.info,
// level-1 and level-2 paragraphs: symmetric products need only the lower
// triangle, which is then copied to the upper one).
//
// C = alpha * A * B^T (+ beta * D + gamma * I).  A is stored K-contiguous;
// B either K-contiguous too ([N][K]) or N-contiguous ([K][N], the X of the
// multiply-backs, read through transposing LDS reads).  Two tile
// configurations:
//   * 256 x 256 block, 8 waves in 2 x 4, each wave 128 x 64 = 4 x 2
//     v_mfma_f32_32x32x16_f16 tiles (one block per CU, 147 KB of LDS);
//   * 128 x 128 block, 4 waves in 2 x 2, each wave 64 x 64 (two blocks per CU),
//     for grids too small to fill 256 CUs with the large tile.
// K advances 64 at a time through two LDS buffers (rows padded by 8 halves:
// conflict-free 16-byte fragment reads).  Operands arrive through raw buffer
// loads (rows past the matrix read as zero) into a register prefetch of one
// K step (the large tile's 128 accumulators leave no room for more at two
// waves per SIMD; a second set in the small tile spilled once the fragments
// were carried across steps); the next tile's LDS stores and global loads
// are issued at the start of each step's MFMAs.  The instruction order of
// each k-slice is fixed by hand (see mma_step) and the next step's first
// fragments are read under the current step's last MFMAs.  In the large
// tile each wave runs the K loop for only the 32 x 32 blocks whose values
// are needed and not known to be zero (see k_gemm).  The epilogue stages
// the fp16 tile in LDS and writes it with 16-byte stores as rows, and for
// the mirrored (symmetric) or transposed outputs as columns.  One launch
// may hold several lower-triangle products (segments; see locate()).
#include "dion3_internal.h"

namespace dion3 {
namespace {

constexpr int BK = 64;
constexpr int LDSK = BK + 8;   // halves per LDS operand row

typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// One product of a launch (a segment): its operands, sizes and tile counts.
struct Seg {
  const f16* A; const f16* B; f16* C; const f16* D;
  long long sA, sB, sC, sD;
  int lda, ldb, ldc, ldd;
  int M, N, K;
  int tilesM, tilesN, tilesPerMat, ntiles;
  int gdiag;   // gamma only on diagonal elements below this index
  int zrows, zcols;   // A's rows and B's rows (columns with a [K][N] B) past these are zero
};

struct GemmArgs {
  int nseg;
  Seg seg[kGemmMaxSeg];
  f16* CT;            // (one-segment launches only)
  long long sCT;
  int ldct;
  int total;
  float alpha, beta, gamma;
  int sink;
  BatchPtr<float> W;
  long long ldw;
  const int* idx;
  float lr;
  f16* Oout;
  long long sO;
  int kval, mval, nrows;
  float* part;
  int nblk;
};

// One 8-wide chunk of the output in rows layout (row r, columns c..c+7)
// goes to the fused update instead of memory: W[idx[r]][c..] -= lr * O and
// optionally O_out[r][c..] = O (matrix b's rows start sO elements after
// matrix b-1's).
__device__ __forceinline__ void sink_chunk(const GemmArgs& p, int b, int r, int c, const half8& v) {
  if (r >= p.kval || c >= p.mval) return;
  const bool full = c + 8 <= p.mval;
  if (p.Oout) {
    f16* o = p.Oout + (long long)b * p.sO + (long long)r * p.mval + c;
    if (full && ((uintptr_t)o & 15) == 0) {
      *(half8*)o = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < p.mval) o[e] = v[e];
    }
  }
  if (p.W.ptrs || p.W.base) {
    const int row = p.idx[(long long)b * p.kval + r];
    if (row < 0 || row >= p.nrows) return;
    float* w = p.W.get(b) + (long long)row * p.ldw + c;
    if (full && ((uintptr_t)w & 15) == 0) {
      float4 w0 = ((float4*)w)[0], w1 = ((float4*)w)[1];
      w0.x = __builtin_fmaf(-p.lr, (float)v[0], w0.x);
      w0.y = __builtin_fmaf(-p.lr, (float)v[1], w0.y);
      w0.z = __builtin_fmaf(-p.lr, (float)v[2], w0.z);
      w0.w = __builtin_fmaf(-p.lr, (float)v[3], w0.w);
      w1.x = __builtin_fmaf(-p.lr, (float)v[4], w1.x);
      w1.y = __builtin_fmaf(-p.lr, (float)v[5], w1.y);
      w1.z = __builtin_fmaf(-p.lr, (float)v[6], w1.z);
      w1.w = __builtin_fmaf(-p.lr, (float)v[7], w1.w);
      ((float4*)w)[0] = w0;
      ((float4*)w)[1] = w1;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < p.mval) w[e] = __builtin_fmaf(-p.lr, (float)v[e], w[e]);
    }
  }
}

template <int BM_, int WAVES_M, int WAVES_N, int PF_>
struct Cfg {
  static constexpr int BM = BM_, BN = BM_;
  static constexpr int PF = PF_;                         // K steps of register prefetch
  static_assert(PF == 1, "the K loop carries one register set");
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int CH = BM * (BK / 8) / NT;          // 16-byte chunks per thread per operand
  // B given as [K][N] (N contiguous) takes BK rows of RSB halves in a stage
  // (the 32-half pad puts the four rows of a transposing read in four
  // different 64-byte bank windows); [N][K] takes BN rows of LDSK
  static constexpr int RSB = BN + 32;
  static constexpr int BPART = (BN * LDSK > BK * RSB) ? BN * LDSK : BK * RSB;
  static constexpr int STAGE = BM * LDSK + BPART;        // halves per LDS stage
  static constexpr int EP = BN + 8;                      // epilogue staging row stride
  static constexpr int LDS = (2 * STAGE > BM * EP) ? 2 * STAGE : BM * EP;
  static_assert(CH * NT == BM * (BK / 8), "chunk split");
};

typedef Cfg<256, 2, 4, 1> CfgL;   // large tile, 8 waves of 128 x 64 (2 waves per SIMD)
typedef Cfg<128, 2, 2, 1> CfgS;   // small tile

// The fused update for one staged tile (S: the fp16 tile in LDS, row stride
// C::EP).  SINK 1: output rows are the tile's rows (O row m0 + r); SINK 2:
// they are its columns (O row n0 + c).  Each thread owns NCH 8-wide chunks
// at fixed positions; it loads the selected-row indices of all of them
// first, then the W rows of BATCH chunks at a time, and only then does the
// fma and the stores, so the global round trips overlap instead of running
// one after another per chunk.  Chunks at a ragged column end, or W rows
// that are not 16-byte aligned, take sink_chunk's element path.
template <class C, int SINK>
__device__ __forceinline__ void sink_tile(const GemmArgs& p, int b, int m0, int n0,
                                          const f16* __restrict__ S, int tid) {
  constexpr int NCH = C::BM * C::BN / 8 / C::NT;
  constexpr int BATCH = 8;
  static_assert(NCH % BATCH == 0, "chunk batches");
  constexpr int CPR = C::BN / 8;   // SINK 1: chunks per staged row
  static_assert(C::NT % CPR == 0 && C::NT % C::BN == 0, "fixed chunk columns per thread");
  float* __restrict__ Wb = (p.W.ptrs || p.W.base) ? p.W.get(b) : nullptr;
  const bool vec = Wb && ((uintptr_t)Wb & 15) == 0 && (p.ldw & 3) == 0;
  const int* __restrict__ ib = p.idx + (long long)b * p.kval;
  // output row and first column of chunk q, and its place in S
  auto where = [&](int q, int& gr, int& gc, int& sr, int& sc) {
    if (SINK == 1) {
      sr = tid / CPR + q * (C::NT / CPR);
      sc = (tid % CPR) * 8;
      gr = m0 + sr;
      gc = n0 + sc;
    } else {
      sc = tid % C::BN;
      sr = (tid / C::BN + q * (C::NT / C::BN)) * 8;
      gr = n0 + sc;
      gc = m0 + sr;
    }
  };
  auto staged = [&](int sr, int sc) {
    half8 v;
    if (SINK == 1) {
      v = *(const half8*)(S + sr * C::EP + sc);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = S[(sr + k) * C::EP + sc];
    }
    return v;
  };
  // SINK 1 with p.part: each chunk's sum of squares (column order, fp32 fma
  // from +0; zero for chunks outside the output), combined below into the
  // rows' 128-column block sums in the order normalize.hip fixes
  float cs[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q) cs[q] = 0.0f;
  int row[NCH];
  if (SINK == 1) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      int gr, gc, sr, sc;
      where(q, gr, gc, sr, sc);
      row[q] = gr < p.kval ? ib[gr] : -1;
    }
  } else {
    int gr, gc, sr, sc;
    where(0, gr, gc, sr, sc);
    const int r = gr < p.kval ? ib[gr] : -1;
#pragma unroll
    for (int q = 0; q < NCH; ++q) row[q] = r;
  }
#pragma unroll
  for (int q0 = 0; q0 < NCH; q0 += BATCH) {
    float4 w0[BATCH], w1[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      int gr, gc, sr, sc;
      where(q0 + u, gr, gc, sr, sc);
      const int r = row[q0 + u];
      if (vec && r >= 0 && r < p.nrows && gc + 8 <= p.mval) {
        const float4* w = (const float4*)(Wb + (long long)r * p.ldw + gc);
        w0[u] = w[0];
        w1[u] = w[1];
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      int gr, gc, sr, sc;
      where(q0 + u, gr, gc, sr, sc);
      if (gr >= p.kval || gc >= p.mval) continue;
      const half8 v = staged(sr, sc);
      if (SINK == 1 && p.part) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = gc + e < p.mval ? (float)v[e] : 0.0f;
          a = __builtin_fmaf(x, x, a);
        }
        cs[q0 + u] = a;
      }
      const int r = row[q0 + u];
      if (!(vec && r >= 0 && r < p.nrows && gc + 8 <= p.mval)) {
        sink_chunk(p, b, gr, gc, v);
        continue;
      }
      if (p.Oout) {
        f16* o = p.Oout + (long long)b * p.sO + (long long)gr * p.mval + gc;
        if (((uintptr_t)o & 15) == 0) {
          *(half8*)o = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = v[e];
        }
      }
      float4 a = w0[u], c = w1[u];
      a.x = __builtin_fmaf(-p.lr, (float)v[0], a.x);
      a.y = __builtin_fmaf(-p.lr, (float)v[1], a.y);
      a.z = __builtin_fmaf(-p.lr, (float)v[2], a.z);
      a.w = __builtin_fmaf(-p.lr, (float)v[3], a.w);
      c.x = __builtin_fmaf(-p.lr, (float)v[4], c.x);
      c.y = __builtin_fmaf(-p.lr, (float)v[5], c.y);
      c.z = __builtin_fmaf(-p.lr, (float)v[6], c.z);
      c.w = __builtin_fmaf(-p.lr, (float)v[7], c.w);
      float4* w = (float4*)(Wb + (long long)r * p.ldw + gc);
      w[0] = a;
      w[1] = c;
    }
  }
  if (SINK == 1 && p.part) {
    // the 16 lanes tid & ~15 .. hold the 16 chunks of one row's 128-column
    // block (columns n0 + 8 (tid % CPR) ..; n0 is a multiple of 128): the
    // butterfly xor 1, 2, 4, 8, with every lane taking part
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      float v = cs[q];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      int gr, gc, sr, sc;
      where(q, gr, gc, sr, sc);
      if ((tid & 15) == 0 && gr < p.kval && gc < p.mval)
        p.part[((long long)b * p.kval + gr) * p.nblk + gc / 128] = v;
    }
  }
}

__device__ __forceinline__ void tri_index(int t, int& bi, int& bj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  bi = i;
  bj = t - i * (i + 1) / 2;
}

typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer resource over one operand matrix: `rows` rows of `ld` halves.  Raw
// buffer loads past num_records return zero, which zero-fills the rows of a
// tile that lie beyond the matrix without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const f16* base, int rows, int ld) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * ld * 2, 0x00020000);
}

template <class C>
__device__ __forceinline__ void gload(__amdgpu_buffer_rsrc_t rs, int ld, int r0, int k0, int tid,
                                      half8 (&reg)[C::CH]) {
  const int row = tid >> 3, kc = tid & 7;
  const int voff = ((r0 + row) * ld + kc * 8) * 2;
  constexpr int ROWS_PER = C::NT / 8;
#pragma unroll
  for (int i = 0; i < C::CH; ++i) {
    const int4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + i * ROWS_PER * ld * 2, k0 * 2, 0);
    reg[i] = __builtin_bit_cast(half8, v);
  }
}

// The B tile of a [K][N] operand: BK rows (K) of BN halves (N), row k0 + r,
// columns n0 .. n0 + BN - 1; thread chunk e = tid + NT i covers row e / (BN / 8),
// columns 8 (e % (BN / 8)) ..
template <class C>
__device__ __forceinline__ void gload_kn(__amdgpu_buffer_rsrc_t rs, int ld, int n0, int k0, int tid,
                                         half8 (&reg)[C::CH]) {
  constexpr int CPR = C::BN / 8;
#pragma unroll
  for (int i = 0; i < C::CH; ++i) {
    const int e = tid + C::NT * i, r = e / CPR, c = e % CPR;
    const int4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, (r * ld + n0 + c * 8) * 2, k0 * ld * 2, 0);
    reg[i] = __builtin_bit_cast(half8, v);
  }
}

template <class C>
__device__ __forceinline__ void lstore_kn(f16* __restrict__ s, int tid, const half8 (&reg)[C::CH]) {
  constexpr int CPR = C::BN / 8;
#pragma unroll
  for (int i = 0; i < C::CH; ++i) {
    const int e = tid + C::NT * i;
    *(half8*)(s + (e / CPR) * C::RSB + (e % CPR) * 8) = reg[i];
  }
}

typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;

// One MFMA B fragment (8 consecutive K of column n = lane % 32, from
// K = 8 (lane / 32)) out of a [K][N] LDS tile, as two transposing reads: in
// each 16-lane group, lane 4e + u points at row e, columns 4u .. 4u + 3 of a
// 4 x 16 block and receives that block's column (lane % 16), i.e. 4
// consecutive K of one column.  `p` is this lane's address for the first
// four K (see boff_kn); the second four are 4 rows further.
template <class C>
__device__ __forceinline__ half8 bfrag_kn(const f16* p) {
  typedef f16 half4v __attribute__((ext_vector_type(4)));
  const half4v lo = __builtin_bit_cast(
      half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p));
  const half4v hi = __builtin_bit_cast(
      half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(p + 4 * C::RSB)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <class C>
__device__ __forceinline__ void lstore(f16* __restrict__ s, int tid, const half8 (&reg)[C::CH]) {
#pragma unroll
  for (int i = 0; i < C::CH; ++i) {
    const int c = tid + C::NT * i;
    *(half8*)(s + (c >> 3) * LDSK + (c & 7) * 8) = reg[i];
  }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// Which 32 x 32 blocks of its wave tile a wave computes: bit FN i + j of MSK
// for block (i, j).  Blocks whose values are never stored or are known to be
// +0 (see k_gemm) are skipped with their fragment reads.
template <class C, int MSK>
struct Blocks {
  static constexpr bool on(int i, int j) { return ((MSK >> (i * C::FN + j)) & 1) != 0; }
  static constexpr bool arow(int i) {
    for (int j = 0; j < C::FN; ++j)
      if (on(i, j)) return true;
    return false;
  }
  static constexpr bool bcol(int j) {
    for (int i = 0; i < C::FM; ++i)
      if (on(i, j)) return true;
    return false;
  }
  static constexpr int count() {
    int n = 0;
    for (int i = 0; i < C::FM; ++i)
      for (int j = 0; j < C::FN; ++j) n += on(i, j) ? 1 : 0;
    return n;
  }
  static constexpr int arows() {
    int n = 0;
    for (int i = 0; i < C::FM; ++i) n += arow(i) ? 1 : 0;
    return n;
  }
  static constexpr int bcols() {
    int n = 0;
    for (int j = 0; j < C::FN; ++j) n += bcol(j) ? 1 : 0;
    return n;
  }
};

template <class C, int MSK>
__device__ __forceinline__ void mfma_slice(const half8 (&af)[C::FM], const half8 (&bf)[C::FN],
                                           floatx16 (&acc)[C::FM][C::FN]) {
  typedef Blocks<C, MSK> K;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      if (K::on(i, j))
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// One K step (four 16-wide k-slices) of MFMAs on LDS stage `st`, with the
// fragments of its first slice already in fa0/fb0.  Every slice issues the
// LDS reads of the next slice before its own MFMAs, so LDS latency hides
// behind them.  Slice 0 also writes the next tile (held in registers) into
// stage `nxt` (STORE) and refills the registers with the tile after that
// (LOAD).  The step's one barrier sits before the last slice's MFMAs, and
// right after it the first-slice fragments of `nxt` are read into fa0/fb0
// (NEXT).  Those reads overlap the last MFMAs instead of waiting at the top
// of the next step.
// The order inside each slice is fixed with scheduling barriers, which the
// compiler would otherwise reorder to save registers:
//   slice 0:     the next slice's reads, then MFMA / LDS write / global
//                load, one of each in turn;
//   slices 1, 2: LDS read / MFMA in turn;
//   slice 3:     barrier, next stage's reads, MFMAs.
// On the 7B shapes this is 14-25 % faster than the same step left to the
// compiler's scheduler, with bitwise identical results (the MFMA order per
// accumulator is unchanged).
// B fragment j of k-slice kk from a stage: [N][K] rows (boff: this lane's
// row and K offset) or, with BKN, a [K][N] tile read transposed (boff: this
// lane's offset for bfrag_kn).
template <class C, bool BKN>
__device__ __forceinline__ half8 bfrag(const f16* __restrict__ st, int boff, int j, int kk) {
  if constexpr (BKN) return bfrag_kn<C>(st + C::BM * LDSK + boff + j * 32 + kk * 16 * C::RSB);
  return *(const half8*)(st + boff + j * 32 * LDSK + kk * 16);
}

// Slice 0's order: MFMA q, then its share of the NW LDS writes and of the NW
// global loads, the shares spread as evenly as they go over the NM MFMAs.
template <int NM, int NW, int Q>
__device__ __forceinline__ void slice0_order() {
  if constexpr (Q < NM) {
    constexpr int w = ((Q + 1) * NW + NM - 1) / NM - (Q * NW + NM - 1) / NM;
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if constexpr (w > 0) {
      __builtin_amdgcn_sched_group_barrier(kSgDsWrite, w, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVmemRead, w, 0);
    }
    slice0_order<NM, NW, Q + 1>();
  }
}

template <class C, bool STORE, bool LOAD, bool NEXT, bool BKN, int MSK>
__device__ __forceinline__ void mma_step(const f16* __restrict__ st, f16* __restrict__ nxt,
                                         __amdgpu_buffer_rsrc_t Ab, __amdgpu_buffer_rsrc_t Bb,
                                         int lda, int ldb, int m0, int n0, int k0_next, int tid,
                                         half8 (&ra)[C::CH], half8 (&rb)[C::CH], int aoff,
                                         int boff, half8 (&fa0)[C::FM], half8 (&fb0)[C::FN],
                                         floatx16 (&acc)[C::FM][C::FN]) {
  typedef Blocks<C, MSK> K;
  constexpr int NS = BK / 16;
  constexpr int NR = K::arows() + (BKN ? 2 : 1) * K::bcols(), NM = K::count();
  constexpr int NW = 2 * C::CH;   // LDS writes (and global loads) of slice 0
  static_assert(MSK != (1 << (C::FM * C::FN)) - 1 || NW % NM == 0, "slice schedules assume these counts");
  constexpr int NP = NM < NR ? NM : NR;   // read / MFMA pairs of slices 1 and 2
  const f16* a_s = st + aoff;
  half8 af[2][C::FM], bf[2][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) af[0][i] = fa0[i];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) bf[0][j] = fb0[j];
#pragma unroll
  for (int kk = 0; kk < NS; ++kk) {
    const int cb = kk & 1;
    if (kk + 1 < NS) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        if (K::arow(i)) af[cb ^ 1][i] = *(const half8*)(a_s + i * 32 * LDSK + (kk + 1) * 16);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        if (K::bcol(j)) bf[cb ^ 1][j] = bfrag<C, BKN>(st, boff, j, kk + 1);
    }
    if (kk == NS - 1) {
      __syncthreads();
      if (NEXT) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          if (K::arow(i)) fa0[i] = *(const half8*)(nxt + aoff + i * 32 * LDSK);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          if (K::bcol(j)) fb0[j] = bfrag<C, BKN>(nxt, boff, j, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_slice<C, MSK>(af[cb], bf[cb], acc);
      __builtin_amdgcn_sched_barrier(0);
      continue;
    }
    if (kk == 0 && STORE) {
      lstore<C>(nxt, tid, ra);
      if constexpr (BKN) lstore_kn<C>(nxt + C::BM * LDSK, tid, rb);
      else lstore<C>(nxt + C::BM * LDSK, tid, rb);
    }
    if (kk == 0 && LOAD) {
      gload<C>(Ab, lda, m0, k0_next, tid, ra);
      if constexpr (BKN) gload_kn<C>(Bb, ldb, n0, k0_next, tid, rb);
      else gload<C>(Bb, ldb, n0, k0_next, tid, rb);
    }
    mfma_slice<C, MSK>(af[cb], bf[cb], acc);
    if (kk == 0) {
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, NR, 0);
      if constexpr (NM == 0) {
        __builtin_amdgcn_sched_group_barrier(kSgDsWrite, NW, 0);
        __builtin_amdgcn_sched_group_barrier(kSgVmemRead, NW, 0);
      } else {
        slice0_order<NM, NW, 0>();
      }
    } else {
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      }
      if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(kSgMfma, NM - NP, 0);
      if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(kSgDsRead, NR - NP, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The K loop of one tile, blocks MSK of the wave tile (wm, wn).  One register
// set: step t multiplies stage t%2; at its start tile t+1 goes from the
// registers into the other stage (free since the barrier that ended step t-1)
// and tile t+2 is requested into the registers.  Every instance passes the
// same barriers, so the waves of one workgroup may run different instances.
template <class C, bool BKN, int MSK>
__device__ __forceinline__ void k_loop(f16* lds, __amdgpu_buffer_rsrc_t Ab,
                                       __amdgpu_buffer_rsrc_t Bb, const Seg& p, int m0,
                                       int n0, int tid, int wm, int wn,
                                       floatx16 (&acc)[C::FM][C::FN]) {
  typedef Blocks<C, MSK> K;
  const int lane = tid & 63;
  const int nk = p.K / BK;
  half8 ra[C::CH], rb[C::CH];
  gload<C>(Ab, p.lda, m0, 0, tid, ra);
  if constexpr (BKN) gload_kn<C>(Bb, p.ldb, n0, 0, tid, rb);
  else gload<C>(Bb, p.ldb, n0, 0, tid, rb);
  lstore<C>(lds, tid, ra);
  if constexpr (BKN) lstore_kn<C>(lds + C::BM * LDSK, tid, rb);
  else lstore<C>(lds + C::BM * LDSK, tid, rb);
  if (nk > 1) {
    gload<C>(Ab, p.lda, m0, BK, tid, ra);
    if constexpr (BKN) gload_kn<C>(Bb, p.ldb, n0, BK, tid, rb);
    else gload<C>(Bb, p.ldb, n0, BK, tid, rb);
  }
  __syncthreads();
  // the first slice's fragments of stage 0; each step then reads those of
  // the stage after it
  const int aoff = (wm * C::WTM + (lane & 31)) * LDSK + (lane >> 5) * 8;
  // B, [N][K]: this lane's row and K offset; [K][N]: its transposing-read
  // address inside the 4 x 16 blocks (row 8 (lane / 32) + (lane % 16) / 4,
  // column 16 ((lane / 16) % 2) + 4 (lane % 4) of the wave's columns)
  const int boff = BKN ? ((lane >> 5) * 8 + ((lane & 15) >> 2)) * C::RSB + wn * C::WTN +
                             ((lane >> 4) & 1) * 16 + (lane & 3) * 4
                       : (C::BM + wn * C::WTN + (lane & 31)) * LDSK + (lane >> 5) * 8;
  half8 fa0[C::FM], fb0[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    if (K::arow(i)) fa0[i] = *(const half8*)(lds + aoff + i * 32 * LDSK);
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    if (K::bcol(j)) fb0[j] = bfrag<C, BKN>(lds, boff, j, 0);
  // all steps but the last two store the next tile and load the one after
  int kt = 0;
  for (; kt + 2 < nk; ++kt)
    mma_step<C, true, true, true, BKN, MSK>(lds + (kt & 1) * C::STAGE, lds + ((kt + 1) & 1) * C::STAGE,
                                            Ab, Bb, p.lda, p.ldb, m0, n0, (kt + 2) * BK, tid, ra,
                                            rb, aoff, boff, fa0, fb0, acc);
  if (kt + 1 < nk) {   // next to last: store only
    mma_step<C, true, false, true, BKN, MSK>(lds + (kt & 1) * C::STAGE, lds + ((kt + 1) & 1) * C::STAGE,
                                             Ab, Bb, p.lda, p.ldb, m0, n0, 0, tid, ra, rb, aoff,
                                             boff, fa0, fb0, acc);
    ++kt;
  }
  // last step: its barrier also frees the LDS for the epilogue
  mma_step<C, false, false, false, BKN, MSK>(lds + (kt & 1) * C::STAGE, lds + ((kt + 1) & 1) * C::STAGE,
                                             Ab, Bb, p.lda, p.ldb, m0, n0, 0, tid, ra, rb, aoff,
                                             boff, fa0, fb0, acc);
}

// The K loop of the first block set in MSKS that covers `need` (the last
// one must be every block).
template <class C, bool BKN, int MSK, int... REST>
__device__ __forceinline__ void k_loop_cover(int need, f16* lds, __amdgpu_buffer_rsrc_t Ab,
                                             __amdgpu_buffer_rsrc_t Bb, const Seg& p, int m0,
                                             int n0, int tid, int wm, int wn,
                                             floatx16 (&acc)[C::FM][C::FN]) {
  if constexpr (sizeof...(REST) == 0) {
    static_assert(MSK == (1 << (C::FM * C::FN)) - 1, "the last set holds every block");
    k_loop<C, BKN, MSK>(lds, Ab, Bb, p, m0, n0, tid, wm, wn, acc);
  } else {
    if ((need & ~MSK) == 0)
      k_loop<C, BKN, MSK>(lds, Ab, Bb, p, m0, n0, tid, wm, wn, acc);
    else
      k_loop_cover<C, BKN, REST...>(need, lds, Ab, Bb, p, m0, n0, tid, wm, wn, acc);
  }
}

// Workgroup w's segment and its tile there.  Each XCD (the workgroups with
// one value of w % 8) takes a contiguous share of every segment's tiles, the
// segments in order, so each XCD gets the same mix; a segment's ntiles % 8
// leftover tiles go one each to consecutive XCDs, continuing where the
// previous segment's left off, so every XCD gets exactly the workgroups the
// hardware sends it.  With one segment this is XCD x taking tiles
// x q + min(x, r) ...
__device__ __forceinline__ void locate(const GemmArgs& p, int w, int& si, int& lid) {
  const int xcd = w & 7;
  int slot = w >> 3, off = 0;
  for (int s = 0;; ++s) {
    const int n = p.seg[s].ntiles, q = n >> 3, r = n & 7;
    int before = 0;   // leftover tiles of this segment on XCDs below this one
    for (int y = 0; y < xcd; ++y) before += ((y - off) & 7) < r ? 1 : 0;
    const int cnt = q + (((xcd - off) & 7) < r ? 1 : 0);
    if (slot < cnt || s == p.nseg - 1) {
      si = s;
      lid = xcd * q + before + slot;
      return;
    }
    slot -= cnt;
    off = (off + r) & 7;
  }
}

// ROLE only names the instance (0 Gram, 1 polynomial, 2 symmetric product,
// 3 rectangular, 4 standard-iteration update, 5 final rectangular product
// with the fused update) so that profilers report each role as its own
// kernel.
template <class C, int ROLE, bool LOWER, bool EPI, bool BKN>
__global__ __launch_bounds__(C::NT, (C::BM == 256 ? 1 : 2)) void k_gemm(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) f16 lds[C::LDS];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // that each XCD works on a contiguous run of tiles (mostly of the same
  // matrices), which keeps their operand panels in that XCD's L2.
  // (Only lower-triangle products share launches; the others have one
  // segment and take the plain mapping, which keeps their registers free.)
  int si = 0, lid;
  if constexpr (LOWER) {
    locate(p, blockIdx.x, si, lid);
  } else {
    const int w = blockIdx.x, q = p.total >> 3, rem = p.total & 7, xcd = w & 7;
    lid = xcd * q + min(xcd, rem) + (w >> 3);
  }
  const Seg& g = p.seg[si];
  const int b = lid / g.tilesPerMat;
  const int t = lid - b * g.tilesPerMat;
  int bi, bj;
  if (LOWER) {
    tri_index(t, bi, bj);
  } else {
    // groups of 8 tile rows, column-major inside a group: consecutive tiles
    // share the B panel and cycle through 8 A panels
    const int GR = 8;
    const int per_group = GR * g.tilesN;
    const int g0 = (t / per_group) * GR;
    const int gsz = min(g.tilesM - g0, GR);
    const int r = t - (t / per_group) * per_group;
    bi = g0 + r % gsz;
    bj = r / gsz;
  }
  const int m0 = bi * C::BM, n0 = bj * C::BN;

  const __amdgpu_buffer_rsrc_t Ab = operand_rsrc(g.A + (long long)b * g.sA, g.M, g.lda);
  // B: N rows of K, or with BKN the [K][N] form, K rows of N
  const __amdgpu_buffer_rsrc_t Bb = operand_rsrc(g.B + (long long)b * g.sB, BKN ? g.K : g.N, g.ldb);

  // the wave index, in a scalar register: the wave's branches below are
  // uniform
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  int wm = wid / (C::BN / C::WTN), wn = wid % (C::BN / C::WTN);

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // A diagonal tile of a symmetric output: its stored values are the lower
  // triangle (the upper one is their mirror), so 32 x 32 blocks wholly above
  // the diagonal need no MFMAs.  In the large tile that leaves, by wave tile
  // (wm, wn), 8 blocks for (1, 0) and (1, 1), 7 for (0, 0) and (1, 2) (all
  // but block (0, 1)), 3 for (0, 1) and (1, 3) (blocks (2, 0), (3, 0),
  // (3, 1)) and none for (0, 2) and (0, 3).  Waves w and w + 4 of a
  // workgroup share a SIMD, so there the wave tiles are dealt out to pair 8
  // with 0 and 7 with 3: at most 10 blocks of MFMAs per SIMD instead of 15.
  if (LOWER && C::BM == 256 && C::FM == 4 && C::FN == 2 && bi == bj) {
    // waves 0..7 take (wm, wn) = (1,0) (1,1) (0,0) (1,2) (0,2) (0,3) (0,1) (1,3)
    constexpr int kWm = 0x8B;      // bit w: wm of wave w
    constexpr int kWn = 0xDE84;    // bits 2w, 2w + 1: wn of wave w
    wm = (kWm >> wid) & 1;
    wn = (kWn >> (2 * wid)) & 3;
  }
  // The blocks this wave computes: not wholly above the diagonal of a
  // diagonal tile, and not wholly in the rows or columns past zrows / zcols,
  // whose accumulators stay exactly +0 (an MFMA over zero rows adds signed
  // zeros to +0, which gives +0).  The wave runs the K loop of the smallest
  // compiled block set that covers them; every computed block keeps its
  // MFMA order, so the results are the same bits as with every block.
  // (Large tile only: in the small tile skipping blocks measured 1-3 %
  // slower.)
  if constexpr (C::FM == 4 && C::FN == 2) {
    int need = 0;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = wm * C::WTM + i * 32, c = wn * C::WTN + j * 32;   // block corner
        bool on = m0 + r < g.zrows && n0 + c < g.zcols;
        if (LOWER && bi == bj) on = on && c <= r;
        need |= on ? 1 << (i * C::FN + j) : 0;
      }
    // none; row 0; the diagonal tile's 3-block set; rows 0-1; column 0;
    // rows 0-2; all but block (0, 1); all
    k_loop_cover<C, BKN, 0x00, 0x03, 0xD0, 0x0F, 0x55, 0x3F, 0xFD, 0xFF>(need, lds, Ab, Bb, g, m0,
                                                                        n0, tid, wm, wn, acc);
  } else {
    k_loop<C, BKN, (1 << (C::FM * C::FN)) - 1>(lds, Ab, Bb, g, m0, n0, tid, wm, wn, acc);
  }

  // Epilogue: final fp32 value (alpha, D, gamma I) -> fp16, kept in registers.
  // Accumulator layout of the 32x32 MFMA: lane l, value v holds row
  // 8*(v/4) + 4*(l/32) + v%4, column l%32 of its 32x32 block, so each lane
  // owns runs of 4 consecutive rows of one column.  The 4 values
  // D[r..r+3][c] are read as the contiguous run Dt[c][r..r+3] of the
  // transposed addend: D itself when it is symmetric (the polynomial), the
  // transposed copy of X for the standard-iteration update.
  typedef f16 half4 __attribute__((ext_vector_type(4)));
  // The addend D is read as the block D[n0 + c][m0 + r]: each lane needs,
  // for its run of rows r..r+3 of column c, the 4 contiguous halves
  // D[n0 + c][m0 + r .. + 3].  The block is staged in LDS (row stride DST)
  // with coalesced 16-byte loads, 32 lanes per D row, through a buffer
  // resource bounded by D's N rows (rows n0 + c >= N read as zero; columns
  // past M belong to outputs that are never stored), then each run is one
  // 8-byte LDS read.  The LDS is free here: the last K step's barrier came
  // after every operand read.
  half4 dvs[C::FM][C::FN][4];
  if (EPI) {
    constexpr int DST = C::BM + 8;
    static_assert(C::BN * DST <= C::LDS, "addend block fits");
    if (g.D) {
      const __amdgpu_buffer_rsrc_t Dr = operand_rsrc(g.D + (long long)b * g.sD, g.N, g.ldd);
      constexpr int NCHD = C::BN * (C::BM / 8) / C::NT;   // 16-byte chunks per thread
      int4v dchunk[NCHD];
#pragma unroll
      for (int q = 0; q < NCHD; ++q) {
        const int e = tid + q * C::NT, c = e / (C::BM / 8), r8 = e % (C::BM / 8);
        const unsigned off = (unsigned)(min(n0 + c, g.N) * g.ldd + m0 + 8 * r8) * 2u;
        dchunk[q] = __builtin_amdgcn_raw_buffer_load_b128(Dr, off, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < NCHD; ++q) {
        const int e = tid + q * C::NT, c = e / (C::BM / 8), r8 = e % (C::BM / 8);
        *(int4v*)(lds + c * DST + 8 * r8) = dchunk[q];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int r = wm * C::WTM + i * 32 + 8 * v4 + 4 * (lane >> 5);
            const int c = wn * C::WTN + j * 32 + (lane & 31);
            dvs[i][j][v4] = *(const half4*)(lds + c * DST + r);
          }
      __syncthreads();   // the staging below reuses the LDS
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) dvs[i][j][v4] = half4{};
    }
  }
  half4 hv[C::FM][C::FN][4];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int r = wm * C::WTM + i * 32 + 8 * v4 + 4 * (lane >> 5);
        const int c = wn * C::WTN + j * 32 + (lane & 31);
        float val[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[i][j][4 * v4 + e];
        if (EPI) {
          const int gr = m0 + r, gc = n0 + c;
          const half4 dv = dvs[i][j][v4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            val[e] = __builtin_fmaf(val[e], p.alpha, p.beta * (float)dv[e]);
            if (gr + e == gc && gc < g.gdiag) val[e] += p.gamma;
            // Keep the fp32 result as written (round to fp32, then to fp16):
            // otherwise the compiler may fuse the fma with the conversion
            // into one mixed-precision fma that rounds once, in some
            // elements only, and the fused small-matrix kernel would no
            // longer match bit for bit.
            asm("" : "+v"(val[e]));
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[i][j][v4][e] = (f16)val[e];
      }

  // Outputs: rows (C[m0 + r][n0 + c], or the fused update) and columns (the
  // mirror of an off-diagonal lower tile into C, or the transposed output
  // CT[n0 + c][m0 + r]).
  f16* __restrict__ Cb = g.C ? g.C + (long long)b * g.sC : nullptr;
  f16* __restrict__ Tb = nullptr;
  int ldt = 0;
  if (LOWER) {
    if (bi != bj) { Tb = Cb; ldt = g.ldc; }
  } else if (p.CT) {
    Tb = p.CT + (long long)b * p.sCT;
    ldt = p.ldct;
  }
  // Column outputs (Tb) always go through a column-major restaging of the
  // tile.  (Reading them from the row-major staging, 8 strided halves per
  // chunk, had been kept for symmetric products with K < 2048; since the
  // diagonal mirror moved into the staging pass the restaging is as fast or
  // faster there too: 1B step -2.5 %, 14B symmetric products +5 %.)
  const bool tcols = Tb != nullptr;
  f16* S = lds;
  if (Cb || (!LOWER && p.sink)) {
    // the tile row-major in LDS, row stride C::EP.  A diagonal tile of a
    // symmetric product keeps its lower triangle (diagonal included) and
    // fills the upper one with the mirror of the lower values in the same
    // pass: a lane's run of 4 rows r..r+3 of column c lies below the
    // diagonal where r + e > c, and then goes to row c, columns r + e (one
    // 8-byte write when the whole run is below).  The two sets of positions
    // are disjoint, so one barrier covers both.
    // (The two cases are separate loops: a per-element test in the common
    // one slowed every tile's staging.)
    if (LOWER && bi == bj) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int r = wm * C::WTM + i * 32 + 8 * v4 + 4 * (lane >> 5);
            const int c = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (r + e >= c) S[(r + e) * C::EP + c] = hv[i][j][v4][e];
            if (r > c) {
              *(half4*)(S + c * C::EP + r) = hv[i][j][v4];
            } else if (r + 3 > c) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (r + e > c) S[c * C::EP + r + e] = hv[i][j][v4][e];
            }
          }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int r = wm * C::WTM + i * 32 + 8 * v4 + 4 * (lane >> 5);
            const int c = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[(r + e) * C::EP + c] = hv[i][j][v4][e];
          }
    }
    __syncthreads();
    if constexpr (!LOWER) {
      if (p.sink == 1) {
        sink_tile<C, 1>(p, b, m0, n0, S, tid);
        return;
      }
      if (p.sink == 2) {
        sink_tile<C, 2>(p, b, m0, n0, S, tid);
        return;
      }
    }
    if (Cb) {
      for (int e = tid; e < C::BM * (C::BN / 8); e += C::NT) {
        const int r = e / (C::BN / 8), c8 = e - r * (C::BN / 8);
        const int gr = m0 + r, gc = n0 + c8 * 8;
        if (gr < g.M && gc < g.N)
          *(half8*)(Cb + (long long)gr * g.ldc + gc) = *(const half8*)(S + r * C::EP + c8 * 8);
      }
    }
  }
  if (tcols) {
    // the tile again, column-major (St[c][r], row stride EPT: each lane's
    // run of 4 rows of one column is one 8-byte write), then written with
    // consecutive lanes on consecutive 8-wide chunks of one output row
    constexpr int EPT = C::BM + 8;
    static_assert(C::BN * EPT <= C::LDS, "column-major staging fits");
    if (Cb) __syncthreads();
    f16* St = lds;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int r = wm * C::WTM + i * 32 + 8 * v4 + 4 * (lane >> 5);
          const int c = wn * C::WTN + j * 32 + (lane & 31);
          *(half4*)(St + c * EPT + r) = hv[i][j][v4];
        }
    __syncthreads();
    for (int e = tid; e < C::BN * (C::BM / 8); e += C::NT) {
      const int c = e / (C::BM / 8), r8 = e - c * (C::BM / 8);
      const int gr = n0 + c, gc = m0 + r8 * 8;
      if (gr < g.N && gc < g.M)
        *(half8*)(Tb + (long long)gr * ldt + gc) = *(const half8*)(St + c * EPT + r8 * 8);
    }
  }
}

template <class C, int ROLE, bool LOWER, bool EPI, bool BKN>
hipError_t launch(const GemmDesc* d, int n, hipStream_t s) {
  GemmArgs p = {};
  p.nseg = n;
  long long total = 0;
  for (int i = 0; i < n; ++i) {
    const GemmDesc& e = d[i];
    Seg& g = p.seg[i];
    g.A = e.A; g.B = e.B; g.C = e.C; g.D = e.D;
    g.sA = e.sA; g.sB = e.sB; g.sC = e.sC; g.sD = e.sD;
    g.lda = e.lda; g.ldb = e.ldb; g.ldc = e.ldc; g.ldd = e.ldd;
    g.M = e.M; g.N = e.N; g.K = e.K;
    g.tilesM = (e.M + C::BM - 1) / C::BM;
    g.tilesN = (e.N + C::BN - 1) / C::BN;
    g.tilesPerMat = LOWER ? g.tilesM * (g.tilesM + 1) / 2 : g.tilesM * g.tilesN;
    const long long tiles = (long long)g.tilesPerMat * e.batch;
    if (tiles <= 0 || tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    g.ntiles = (int)tiles;
    total += tiles;
    g.gdiag = e.gdiag > 0 ? e.gdiag : e.M;
    g.zrows = e.zrows > 0 ? e.zrows : e.M;
    g.zcols = e.zcols > 0 ? e.zcols : e.N;
  }
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  p.total = (int)total;
  p.CT = d[0].CT; p.sCT = d[0].sCT; p.ldct = d[0].ldct;
  p.alpha = d[0].alpha; p.beta = d[0].beta; p.gamma = d[0].gamma;
  p.sink = d[0].sink; p.W = d[0].W; p.ldw = d[0].ldw; p.idx = d[0].idx; p.lr = d[0].lr;
  p.Oout = d[0].Oout; p.sO = d[0].sO;
  p.kval = d[0].kval; p.mval = d[0].mval; p.nrows = d[0].nrows;
  p.part = d[0].part; p.nblk = d[0].nblk;
  hipLaunchKernelGGL((k_gemm<C, ROLE, LOWER, EPI, BKN>), dim3(p.total), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// The large tile needs about two full waves of blocks over the 256 CUs to
// beat the small one (two blocks per CU), or half a wave when every K loop
// is long enough (K >= 2048) for its faster K step to outweigh its larger
// fixed cost per tile (a 16 x 1024 x 4096 Gram: 588 -> 697 TFLOP/s; at
// K = 512-1024 the small tile stays ahead).  A launch of several products
// counts all of their tiles.
bool use_large(const GemmDesc* d, int n) {
  long long tiles = 0;
  int kmin = d[0].K;
  for (int i = 0; i < n; ++i) {
    const long long tm = (d[i].M + 255) / 256, tn = (d[i].N + 255) / 256;
    tiles += (d[i].lower ? tm * (tm + 1) / 2 : tm * tn) * d[i].batch;
    kmin = min(kmin, d[i].K);
  }
  return tiles >= 512 || (tiles >= 128 && kmin >= 2048);
}

const char* trace_name(int role, bool large) {
  static const char* names[6][2] = {{"gemm_gram_128", "gemm_gram_256"},
                                    {"gemm_poly_128", "gemm_poly_256"},
                                    {"gemm_symm_128", "gemm_symm_256"},
                                    {"gemm_rect_128", "gemm_rect_256"},
                                    {"gemm_nsx_128", "gemm_nsx_256"},
                                    {"gemm_back_128", "gemm_back_256"}};
  return names[role][large ? 1 : 0];
}

template <int ROLE, bool LOWER, bool EPI, bool BKN = false>
hipError_t launch_cfg(const GemmDesc* d, int n, hipStream_t s) {
  const bool large = use_large(d, n);
  double flops = 0.0, bytes = 0.0;
  for (int i = 0; i < n; ++i) {
    flops += d[i].trace_flops;
    bytes += d[i].trace_bytes;
  }
  TraceScope ts(trace_name(ROLE, large), flops, bytes, s);
  return large ? launch<CfgL, ROLE, LOWER, EPI, BKN>(d, n, s)
               : launch<CfgS, ROLE, LOWER, EPI, BKN>(d, n, s);
}

bool desc_ok(const GemmDesc& d) {
  if (d.M % 128 || d.N % 128 || d.K % BK || d.K <= 0 || d.batch <= 0) return false;
  if (d.lower && (d.M != d.N || d.CT || !d.C)) return false;
  if (d.b_kn && (d.lower || d.epilogue || d.ldb % 8)) return false;
  if (!d.lower && !d.C && !d.CT && !d.sink) return false;
  if (d.sink && (d.lower || d.C || d.CT || (d.sink != 1 && d.sink != 2))) return false;
  if (d.part && (d.sink != 1 || d.nblk != (d.mval + 127) / 128)) return false;
  return true;
}

// Products that may share a launch: the same kernel and epilogue constants;
// only lower-triangle products, which have no transposed output or sink.
bool same_launch(const GemmDesc& a, const GemmDesc& b) {
  return a.lower && b.lower && a.role == b.role && a.epilogue == b.epilogue &&
         a.alpha == b.alpha && a.beta == b.beta && a.gamma == b.gamma && !a.D == !b.D;
}

}  // namespace

hipError_t launch_gemm_multi(const GemmDesc* d, int n, hipStream_t s) {
  if (!d || n < 1 || n > kGemmMaxSeg) return hipErrorInvalidValue;
  for (int i = 0; i < n; ++i) {
    if (!desc_ok(d[i])) return hipErrorInvalidValue;
    if (i > 0 && !same_launch(d[0], d[i])) return hipErrorInvalidValue;
  }
  const GemmDesc& e = d[0];
  switch (e.role) {
    case kRoleGram:
      if (!e.lower || e.epilogue) break;
      return launch_cfg<kRoleGram, true, false>(d, n, s);
    case kRolePoly:
      if (!e.lower || !e.epilogue) break;
      return launch_cfg<kRolePoly, true, true>(d, n, s);
    case kRoleSymm:
      if (!e.lower || e.epilogue) break;
      return launch_cfg<kRoleSymm, true, false>(d, n, s);
    case kRoleRect:
      if (e.lower || e.epilogue || e.sink) break;
      return e.b_kn ? launch_cfg<kRoleRect, false, false, true>(d, n, s)
                    : launch_cfg<kRoleRect, false, false>(d, n, s);
    case kRoleBack:
      if (e.lower || e.epilogue || !e.sink) break;
      return e.b_kn ? launch_cfg<kRoleBack, false, false, true>(d, n, s)
                    : launch_cfg<kRoleBack, false, false>(d, n, s);
    case kRoleNsX:
      if (e.lower || !e.epilogue || !e.D) break;
      return launch_cfg<kRoleNsX, false, true>(d, n, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s) { return launch_gemm_multi(&d, 1, s); }

}  // namespace dion3
