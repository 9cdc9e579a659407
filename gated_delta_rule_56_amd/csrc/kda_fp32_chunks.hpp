// fp32 chunk-plane machinery shared by the backward pass and the general
// DPLR forward pass: sequence geometry over global chunk indices, the chunk
// table, a batched fp32 product, LDS staging and the fp32 MFMA step.  Each
// translation unit that includes it gets its own copies (anonymous namespace).
#pragma once

#include "kda_device.hpp"

namespace kda {
namespace {

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

// Sequence geometry of a pass over the local chunks [c0, c0 + L) of every
// sequence (a segment; c0 = 0 and L past every sequence's length for a whole
// pass).  The pass's planes hold those chunks in order: sequence n's chunk
// ci sits at plane slot base(n) + ci - c0, with base(n) = off[n] (varlen:
// cu on the device, off from chunk_table_kernel) or n * slot_cnt (fixed
// length: num_seqs sequences of seq_len tokens).
struct Geo {
  const int32_t* cu;
  const int32_t* off;  // varlen only
  int num_seqs, seq_len, total_tokens, H, nchunks;
  int c0, L, slot_cnt;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Placement of the serial passes' workgroups, one per (sequence, head) and
// block of NVB value columns.  Consecutive block ids rotate over the chip's
// eight XCDs, so the NVB column blocks of one (sequence, head) take ids on
// the same XCD and share its L2 for the chunk operands that all of them
// read.  Launch serial_blocks(pairs, NVB) workgroups; serial_slot gives a
// workgroup its pair nh and column block vb, false for the padding ids.
inline int serial_blocks(int pairs, int nvb) { return (pairs + 7) / 8 * 8 * nvb; }
template <int NVB>
__device__ __forceinline__ bool serial_slot(int pairs, int& nh, int& vb) {
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  nh = (slot / NVB) * 8 + xcd;
  vb = slot % NVB;
  return nh < pairs;
}

template <int C>
__device__ __forceinline__ void seq_of(const Geo& g, int n, int& bos, int& eos, int& base) {
  if (g.cu) {
    bos = clampi(g.cu[n], 0, g.total_tokens);
    eos = clampi(g.cu[n + 1], bos, g.total_tokens);
    base = g.off[n];
  } else {
    bos = n * g.seq_len;
    eos = bos + g.seq_len;
    base = n * g.slot_cnt;
  }
}

// The pass's chunks [lo, hi) of the sequence [bos, eos).
template <int C>
__device__ __forceinline__ void seg_range(const Geo& g, int bos, int eos, int& lo, int& hi) {
  const int nch = (eos - bos + C - 1) / C;
  lo = min(g.c0, nch);
  hi = min(g.c0 + g.L, nch);
}

// Plane slot -> (sequence, first token, length).
template <int C>
__device__ __forceinline__ void chunk_of(const Geo& g, int gch, int& n, int& t0, int& len) {
  if (g.cu) {
    int lo = 0, hi = g.num_seqs - 1;  // last n with off[n] <= gch
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.off[mid] <= gch)
        lo = mid;
      else
        hi = mid - 1;
    }
    n = lo;
  } else {
    n = clampi(gch / max(g.slot_cnt, 1), 0, g.num_seqs - 1);
  }
  int bos, eos, base;
  seq_of<C>(g, n, bos, eos, base);
  t0 = clampi(bos + (g.c0 + gch - base) * C, bos, eos);
  len = clampi(eos - t0, 0, C);
}

// off[n] = the pass's chunk counts of the sequences before n (block scan):
// sequence n contributes its local chunks in [c0, c0 + L).
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* __restrict__ cu,
                                                         int32_t* __restrict__ off, int num_seqs,
                                                         int total_tokens, int C, int c0, int L) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (num_seqs + 1023) / 1024;
  const int n0 = t * per, n1 = min(n0 + per, num_seqs);
  auto nch = [&](int n) {
    const int b = clampi(cu[n], 0, total_tokens), e = clampi(cu[n + 1], b, total_tokens);
    return clampi((e - b + C - 1) / C - c0, 0, L);
  };
  int s = 0;
  for (int n = n0; n < n1; ++n) s += nch(n);
  part[t] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
    const int x = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  for (int n = n0; n < n1; ++n) {
    off[n] = run;
    run += nch(n);
  }
  if (t == 1023) off[num_seqs] = part[1023];
}

// The serial passes run their products on v_mfma_f32_16x16x4f32 (fp32
// operands): lane l supplies A[m = l & 15][k = l >> 4] and B[k = l >> 4][n =
// l & 15] and receives D rows 4 (l >> 4) + i of column l & 15.  Operands are
// staged in LDS; a matrix read as A[m][k] = X[m][k] has row stride +4 floats,
// one read transposed (A[m][k] = X[k][m]) +16, so the 64 lanes of a read hit
// 64 different banks; 16-column blocks have stride 16.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}


// Batched C = alpha op(A) op(B) (+ C when acc) with op(A) [M x K] stored as
// A[m][k] (TA = false) or A[k][m] (TA = true), op(B) [K x N] stored as B[k][n]
// (TB = false) or B[n][k] (TB = true), leading dimensions lda, ldb, ldc, and
// an optional mask on C (1: keep n <= m, 2: keep n < m).  One 64 x 64 tile of
// C per workgroup of 256 threads; each wave computes a 32 x 32 quarter as
// four 16 x 16 tiles on v_mfma_f32_16x16x4f32 (fp32 operands, fp32
// accumulation); K a multiple of 16, M and N of 4.  K runs in stages of 64:
// a stage of op(A)'s and op(B)'s tiles is loaded with 16-byte loads along each
// matrix's contiguous dimension (all of a thread's loads issued together),
// written to LDS as As[m][k] and Bs[n][k], and the next stage's loads are
// issued before this stage's products, so they overlap.  Within each block of
// 16 k the lanes of group g (lanes 16 g .. 16 g + 15) take k = 4 g .. 4 g + 3
// in four successive MFMAs, so one 16-byte LDS read per operand and tile feeds
// four products; with 68-float rows the reads of eight lanes cover the 32
// banks once.
constexpr int kGemmKStage = 64, kGemmLd = 64 + 4;
constexpr size_t kGemmLds = (size_t)2 * kGemmKStage * kGemmLd * sizeof(float);

// A second product in the same launch (X modes of fp32_gemm_kernel):
// kGemmDual: C2 = alpha2 op(A2) op(B), same B, shapes and strides as the
// first, mask2 on C2 (two outputs, B read once); kGemmCat: C = alpha (op(A)
// op(B) + op(A2) op(B2)) with A2, B2 laid out like A, B and K2 more k (one
// output, written once).
constexpr int kGemmOne = 0, kGemmDual = 1, kGemmCat = 2;
struct GemmX {
  const float* A2 = nullptr;
  const float* B2 = nullptr;
  float* C2 = nullptr;
  int K2 = 0;
  float alpha2 = 1.f;
  int mask2 = 0;
};

template <bool TA, bool TB, int X, bool SPLIT>
__global__ __launch_bounds__(256) void fp32_gemm_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ Cm, int M, int N, int K,
                                                       int lda, int ldb, int ldc, size_t sa,
                                                       size_t sb, size_t sc, float alpha, int acc_c,
                                                       int mask, size_t nb, GemmX x2) {
  constexpr bool DUAL = X == kGemmDual;
  __shared__ __attribute__((aligned(16))) float As[(DUAL ? 2 : 1) * 64 * kGemmLd];  // As[m][k] (then A2's)
  __shared__ __attribute__((aligned(16))) float Bs[64 * kGemmLd];                   // Bs[n][k]
  constexpr int LD = kGemmLd, NV = kGemmKStage * 16 / 256;  // vectors per thread and matrix
  // Items in groups of eight, the tiles of a group's items interleaved: item
  // j of a group and tile t take block 8 t + j of the group, so an item's
  // tiles (which share an operand) run close together on one XCD, since
  // consecutive block ids go to the chip's eight XCDs in turn.
  const int ntn = (N + 63) / 64, ntiles = ntn * ((M + 63) / 64);
  const int grp = blockIdx.x / (8 * ntiles), rem = blockIdx.x % (8 * ntiles);
  const int bt = 8 * grp + rem % 8, tile = rem / 8;
  if ((size_t)bt >= nb) return;
  const int m0 = (tile / ntn) * 64, n0 = (tile % ntn) * 64;
  // Stages of up to kGemmKStage k: the first product's, then (kGemmCat) the
  // second's, so no stage mixes the two.
  const int ns1 = (K + kGemmKStage - 1) / kGemmKStage;
  const int nst = ns1 + (X == kGemmCat ? (x2.K2 + kGemmKStage - 1) / kGemmKStage : 0);
  auto stage_at = [&](int si, bool& second, int& kk, int& ks) {
    second = X == kGemmCat && si >= ns1;
    kk = kGemmKStage * (second ? si - ns1 : si);
    const int kend = second ? x2.K2 : K;
    ks = kend - kk < kGemmKStage ? kend - kk : kGemmKStage;
  };
  const int tid = threadIdx.x;
  f32x4 xa[NV], xb[NV], xc[DUAL ? NV : 1];
  // Vector v = tid + 256 x of stage k0 (x < ks / 16, ks = its k extent): for
  // a matrix stored with k as its row (TA for A, !TB for B) row k0 + 16 x +
  // tid % 16, columns 4 (tid / 16) ..; otherwise row v / (ks / 4) of the 64,
  // columns k0 + 4 (v % (ks / 4)) ...  (In the first case sixteen consecutive
  // threads take sixteen rows, so their transposing LDS writes hit distinct
  // banks.)  Rows and columns past M or N are loaded from the last ones and
  // zeroed when written to LDS, so the loads take no branch.
  auto fetch = [&](int si) {
    bool second;
    int kk, ks;
    stage_at(si, second, kk, ks);
    const float* sa_ = (second ? x2.A2 : A) + (size_t)bt * sa;
    const float* sb_ = (second ? x2.B2 : B) + (size_t)bt * sb;
    const float* sc_ = X == kGemmDual ? x2.A2 + (size_t)bt * sa : nullptr;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      if (x >= ks / 16) break;
      const int v = tid + 256 * x, kr = 16 * x + tid % 16, c4 = 4 * (tid / 16);
      const int q = ks / 4, rv = v / q, cv = kk + 4 * (v % q);
      size_t oa;
      if (TA) oa = (size_t)(kk + kr) * lda + min(m0 + c4, M - 4);
      else oa = (size_t)min(m0 + rv, M - 1) * lda + cv;
      xa[x] = *reinterpret_cast<const f32x4*>(sa_ + oa);
      if constexpr (DUAL) xc[x] = *reinterpret_cast<const f32x4*>(sc_ + oa);
      size_t ob;
      if (!TB) ob = (size_t)(kk + kr) * ldb + min(n0 + c4, N - 4);
      else ob = (size_t)min(n0 + rv, N - 1) * ldb + cv;
      xb[x] = *reinterpret_cast<const f32x4*>(sb_ + ob);
    }
  };
  auto stA = [&](float* dst, const f32x4& val, int v, int kr, int c4, int ks) {
    if (TA) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(c4 + e) * LD + kr] = val[e];
    } else {
      *reinterpret_cast<f32x4*>(dst + (v / (ks / 4)) * LD + 4 * (v % (ks / 4))) = val;
    }
  };
  auto stage = [&](int ks) {
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      if (x >= ks / 16) break;
      const int v = tid + 256 * x, kr = 16 * x + tid % 16, c4 = 4 * (tid / 16), rv = v / (ks / 4);
      const bool ina = (TA ? m0 + c4 : m0 + rv) < M, inb = (TB ? n0 + rv : n0 + c4) < N;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      stA(As, ina ? xa[x] : z, v, kr, c4, ks);
      if constexpr (DUAL) stA(As + 64 * LD, ina ? xc[x] : z, v, kr, c4, ks);
      const f32x4 b = inb ? xb[x] : z;
      if (!TB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[(c4 + e) * LD + kr] = b[e];
      } else {
        *reinterpret_cast<f32x4*>(Bs + rv * LD + 4 * (v % (ks / 4))) = b;
      }
    }
  };
  // MFMA operands: lane l = 16 g + i holds row i of the A tile and column i
  // of the B tile at the k this step gives group g; output register r is row
  // 4 g + r, column i of the tile.
  const int l = tid & 63, lm = l & 15, lg = l >> 4;
  const int wm = (tid >> 7) * 32, wn = ((tid >> 6) & 1) * 32;  // this wave's quarter
  f32x4 acc[2][2], acc2[DUAL ? 2 : 1][DUAL ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (DUAL) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  fetch(0);
  for (int si = 0; si < nst; ++si) {
    bool second;
    int kk, ks;
    stage_at(si, second, kk, ks);
    (void)second;
    (void)kk;
    if (si > 0) __syncthreads();  // the previous stage's reads are done
    stage(ks);
    __syncthreads();
    if (si + 1 < nst) fetch(si + 1);
    auto kblock = [&](int kb) {  // k = 16 kb .. 16 kb + 15 of the stage
      const int ko = 16 * kb + 4 * lg;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(As + (wm + lm) * LD + ko);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(As + (wm + 16 + lm) * LD + ko);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(Bs + (wn + lm) * LD + ko);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(Bs + (wn + 16 + lm) * LD + ko);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[0][0] = mfma4(a0[s], b0[s], acc[0][0]);
        acc[0][1] = mfma4(a0[s], b1[s], acc[0][1]);
        acc[1][0] = mfma4(a1[s], b0[s], acc[1][0]);
        acc[1][1] = mfma4(a1[s], b1[s], acc[1][1]);
      }
      if constexpr (DUAL) {
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(As + (64 + wm + lm) * LD + ko);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(As + (64 + wm + 16 + lm) * LD + ko);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc2[0][0] = mfma4(c0[s], b0[s], acc2[0][0]);
          acc2[0][1] = mfma4(c0[s], b1[s], acc2[0][1]);
          acc2[1][0] = mfma4(c1[s], b0[s], acc2[1][0]);
          acc2[1][1] = mfma4(c1[s], b1[s], acc2[1][1]);
        }
      }
    };
    // SPLIT: each 32 k on v_mfma_f32_16x16x32_bf16 with split-bf16 operands
    // (x = hi + lo, products hi hi + hi lo + lo hi, fp32 accumulation),
    // formed from the same fp32 LDS tiles: lane group g takes the k of its
    // 16-byte reads in two consecutive 16-blocks as its eight k, for A and B
    // alike, so the 32 k of the pair are each summed once.
    auto split8 = [&](const float* row, int ko, ModeBF16::PFrag& f) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(row + ko);
      const f32x4 q = *reinterpret_cast<const f32x4*>(row + ko + 16);
      const float v[8] = {p[0], p[1], p[2], p[3], q[0], q[1], q[2], q[3]};
      f = make_pfrag(ModeBF16{}, v);
    };
    auto kpair = [&](int kb) {  // k = 16 kb .. 16 kb + 31 of the stage
      const int ko = 16 * kb + 4 * lg;
      ModeBF16::PFrag b0, b1, a;
      split8(Bs + (wn + lm) * LD, ko, b0);
      split8(Bs + (wn + 16 + lm) * LD, ko, b1);
      // one A row tile at a time: three fragments live, not six
#pragma unroll
      for (int t = 0; t < (DUAL ? 4 : 2); ++t) {
        split8(As + ((t >> 1) * 64 + wm + 16 * (t & 1) + lm) * LD, ko, a);
        f32x4* ac = t < 2 ? acc[t & 1] : acc2[DUAL ? (t & 1) : 0];
        ac[0] = mma_pp(a, b0, ac[0]);
        ac[1] = mma_pp(a, b1, ac[1]);
      }
    };
    if (ks == kGemmKStage) {
      if constexpr (SPLIT) {
#pragma unroll
        for (int kb = 0; kb < kGemmKStage / 16; kb += 2) kpair(kb);
      } else {
#pragma unroll
        for (int kb = 0; kb < kGemmKStage / 16; ++kb) kblock(kb);
      }
    } else {
      int kb = 0;
      if constexpr (SPLIT)
        for (; kb + 1 < ks / 16; kb += 2) kpair(kb);
      for (; kb < ks / 16; ++kb) kblock(kb);
    }
  }
  auto put = [&](float* cm, const f32x4 (&ac)[2][2], float al, int mk) {
    float* c = cm + bt * sc;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm + 16 * ti + 4 * lg + i, nn = n0 + wn + 16 * tj + lm;
          if (m < M && nn < N) {
            const bool keep = mk == 0 || (mk == 1 ? nn <= m : nn < m);
            const float v = keep ? al * ac[ti][tj][i] : 0.f;
            c[(size_t)m * ldc + nn] = acc_c ? c[(size_t)m * ldc + nn] + v : v;
          }
        }
  };
  put(Cm, acc, alpha, mask);
  if constexpr (DUAL) put(x2.C2, acc2, x2.alpha2, x2.mask2);
}

// Operand orientations of fp32_gemm_kernel, as tags for launch_fp32_gemm.
struct GemmNN { static constexpr bool TA = false, TB = false; };
struct GemmNT { static constexpr bool TA = false, TB = true; };
struct GemmTN { static constexpr bool TA = true, TB = false; };

// Launch of fp32_gemm_kernel over NB batch items (x2: the second product of
// kGemmDual or kGemmCat).
template <bool TA, bool TB, int X = kGemmOne, bool SPLIT = false>
inline hipError_t launch_fp32_gemm(const float* A, const float* B, float* Cm, int M, int N, int K,
                                   int lda, int ldb, int ldc, size_t sa, size_t sb, size_t sc,
                                   float alpha, int acc_c, int mask, size_t NB, hipStream_t stream,
                                   GemmX x2 = GemmX{}) {
  if (K % 16 || M % 4 || N % 4) return hipErrorInvalidValue;
  if (X == kGemmCat && (x2.K2 % 16 || !x2.A2 || !x2.B2)) return hipErrorInvalidValue;
  if (X == kGemmDual && (!x2.A2 || !x2.C2)) return hipErrorInvalidValue;
  const size_t blocks = (NB + 7) / 8 * 8 * (size_t)((N + 63) / 64) * ((M + 63) / 64);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fp32_gemm_kernel<TA, TB, X, SPLIT>), dim3((unsigned)blocks), dim3(256), 0, stream, A, B, Cm, M,
                     N, K, lda, ldb, ldc, sa, sb, sc, alpha, acc_c, mask, NB, x2);
  return hipGetLastError();
}

// Register-staged copy of a ROWS x COLS fp32 block (row-major in global
// memory with row stride SLD, COLS by default) spread over NT threads:
// load() issues every load of the thread, store<LD>() writes the block into
// LDS with row stride LD (a multiple of 4, so each write is one 16-byte LDS
// store).  Loading the next chunk's operands while the current chunk
// computes hides their latency.
template <int ROWS, int COLS, int NT, int SLD = COLS>
struct Prefetch {
  static constexpr int C4 = COLS / 4, N = (ROWS * C4 + NT - 1) / NT;
  static_assert(COLS % 4 == 0 && SLD % 4 == 0, "float4 rows");
  f32x4 v[N];
  __device__ __forceinline__ void load(const float* __restrict__ src) {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int idx = threadIdx.x + NT * x;
      if (idx < ROWS * C4)
        v[x] = *reinterpret_cast<const f32x4*>(src + (size_t)(idx / C4) * SLD + 4 * (idx % C4));
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(float* dst) const {
    static_assert(LD % 4 == 0, "16-byte LDS rows");
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int idx = threadIdx.x + NT * x;
      if (idx < ROWS * C4) *reinterpret_cast<f32x4*>(dst + (idx / C4) * LD + 4 * (idx % C4)) = v[x];
    }
  }
};

// M = (I + Diag(rs) A)^{-1} for a strictly lower-triangular C x C block A
// per item (rs: a row scale, or nullptr for none), and optionally
// T = M Diag(rs).  Blocked: the 16 x 16 diagonal blocks by forward
// substitution (one thread per column), then the off-diagonal blocks level by
// level, M_ij = -M_ii sum_{j <= k < i} A_ik M_kj, as 16 x 16 x 16 products
// spread over 256 threads.
template <int C>
__global__ __launch_bounds__(256) void unit_lower_inverse_kernel(const float* __restrict__ A,
                                                                 const float* __restrict__ rs,
                                                                 float* __restrict__ M,
                                                                 float* __restrict__ Tm) {
  constexpr int NB = C / 16;
  __shared__ float As[C][C + 1];
  __shared__ float Xs[C][C + 1];
  __shared__ float Ys[NB][16][17];
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t pcc = (size_t)b * C * C;
  const float* r = rs ? rs + (size_t)b * C : nullptr;
  // Every load of the staging first (a loop that waited for each element's
  // load before its LDS write took most of the kernel's time).
  constexpr int NS = C * C / 256;
  static_assert(NS * 256 == C * C, "whole elements per thread");
  float av[NS], rv[NS];
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    const int idx = tid + 256 * x;
    av[x] = A[pcc + idx];
    rv[x] = r ? r[idx / C] : 1.f;
  }
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    const int idx = tid + 256 * x, i = idx / C, j = idx % C;
    As[i][j] = j < i ? rv[x] * av[x] : 0.f;
    Xs[i][j] = 0.f;
  }
  __syncthreads();
  if (tid < 16 * NB) {  // diagonal blocks
    const int base = 16 * (tid / 16), j = tid % 16;
    for (int i = j; i < 16; ++i) {
      float s = i == j ? 1.f : 0.f;
      for (int l = j; l < i; ++l) s -= As[base + i][base + l] * Xs[base + l][base + j];
      Xs[base + i][base + j] = s;
    }
  }
  __syncthreads();
  for (int d = 1; d < NB; ++d) {
    // Y_i = sum_{k = j .. i-1} A_ik X_kj for the block pairs (i, j = i - d)
    for (int e = tid; e < (NB - d) * 256; e += 256) {
      const int bi = d + e / 256, bj = bi - d, rr = (e % 256) / 16, cc = e % 16;
      float s = 0.f;
      for (int k = 16 * bj; k < 16 * bi; ++k) s += As[16 * bi + rr][k] * Xs[k][16 * bj + cc];
      Ys[bi][rr][cc] = s;
    }
    __syncthreads();
    for (int e = tid; e < (NB - d) * 256; e += 256) {  // X_ij = -X_ii Y_i
      const int bi = d + e / 256, bj = bi - d, rr = (e % 256) / 16, cc = e % 16;
      float s = 0.f;
      for (int k = 0; k <= rr; ++k) s -= Xs[16 * bi + rr][16 * bi + k] * Ys[bi][k][cc];
      Xs[16 * bi + rr][16 * bj + cc] = s;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx / C, j = idx % C;
    M[pcc + idx] = Xs[i][j];
    if (Tm) Tm[pcc + idx] = Xs[i][j] * (r ? r[j] : 1.f);
  }
}

}  // namespace
}  // namespace kda
