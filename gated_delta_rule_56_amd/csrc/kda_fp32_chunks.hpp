// fp32 chunk-plane machinery shared by the backward pass and the general
// DPLR forward pass: sequence geometry over global chunk indices, the chunk
// table, a batched fp32 product, LDS staging and the fp32 MFMA step.  Each
// translation unit that includes it gets its own copies (anonymous namespace).
#pragma once

#include "kda_device.hpp"

namespace kda {
namespace {

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

// Sequence geometry.  Fixed length: num_seqs sequences of seq_len tokens;
// varlen: cu (device) and off[n] = first global chunk of sequence n.
struct Geo {
  const int32_t* cu;
  const int32_t* off;  // varlen only
  int num_seqs, seq_len, total_tokens, H, nchunks;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <int C>
__device__ __forceinline__ void seq_of(const Geo& g, int n, int& bos, int& eos, int& base) {
  if (g.cu) {
    bos = clampi(g.cu[n], 0, g.total_tokens);
    eos = clampi(g.cu[n + 1], bos, g.total_tokens);
    base = g.off[n];
  } else {
    bos = n * g.seq_len;
    eos = bos + g.seq_len;
    base = n * ((g.seq_len + C - 1) / C);
  }
}

// Global chunk -> (sequence, first token, length).
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
    n = clampi(gch / ((g.seq_len + C - 1) / C), 0, g.num_seqs - 1);
  }
  int bos, eos, base;
  seq_of<C>(g, n, bos, eos, base);
  t0 = clampi(bos + (gch - base) * C, bos, eos);
  len = clampi(eos - t0, 0, C);
}

// off[n] = sum of the chunk counts of the sequences before n (block scan).
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* __restrict__ cu,
                                                         int32_t* __restrict__ off, int num_seqs,
                                                         int total_tokens, int C) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (num_seqs + 1023) / 1024;
  const int n0 = t * per, n1 = min(n0 + per, num_seqs);
  auto nch = [&](int n) {
    const int b = clampi(cu[n], 0, total_tokens), e = clampi(cu[n + 1], b, total_tokens);
    return (e - b + C - 1) / C;
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

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void fp32_gemm_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ Cm, int M, int N, int K,
                                                       int lda, int ldb, int ldc, size_t sa,
                                                       size_t sb, size_t sc, float alpha, int acc_c,
                                                       int mask) {
  __shared__ __attribute__((aligned(16))) float As[64 * kGemmLd];  // As[m][k]
  __shared__ __attribute__((aligned(16))) float Bs[64 * kGemmLd];  // Bs[n][k]
  constexpr int LD = kGemmLd, NV = kGemmKStage * 16 / 256;  // vectors per thread and matrix
  const int bt = blockIdx.x;  // batch on x: up to 2^31 - 1 blocks
  const int m0 = blockIdx.z * 64, n0 = blockIdx.y * 64;
  const float* a = A + bt * sa;
  const float* bb = B + bt * sb;
  const int tid = threadIdx.x;
  f32x4 xa[NV], xb[NV];
  // Vector v = tid + 256 x of stage k0 (ks = its k extent): for a matrix
  // stored with k as its row (TA for A, !TB for B) row k0 + 16 x + tid % 16,
  // columns 4 (tid / 16) ..; otherwise row v / (ks / 4) of the 64, columns
  // k0 + 4 (v % (ks / 4)) ...  (In the first case sixteen consecutive threads
  // take sixteen rows, so their transposing LDS writes hit distinct banks.)
  auto fetch = [&](int k0, int ks) {
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int v = tid + 256 * x, kr = 16 * x + tid % 16, c4 = 4 * (tid / 16);
      xa[x] = f32x4{0, 0, 0, 0};
      xb[x] = f32x4{0, 0, 0, 0};
      if (v < ks * 16) {
        if (TA) {
          if (m0 + c4 < M) xa[x] = *reinterpret_cast<const f32x4*>(a + (size_t)(k0 + kr) * lda + m0 + c4);
        } else {
          const int mm = v / (ks / 4);
          if (m0 + mm < M)
            xa[x] = *reinterpret_cast<const f32x4*>(a + (size_t)(m0 + mm) * lda + k0 + 4 * (v % (ks / 4)));
        }
        if (!TB) {
          if (n0 + c4 < N) xb[x] = *reinterpret_cast<const f32x4*>(bb + (size_t)(k0 + kr) * ldb + n0 + c4);
        } else {
          const int nn = v / (ks / 4);
          if (n0 + nn < N)
            xb[x] = *reinterpret_cast<const f32x4*>(bb + (size_t)(n0 + nn) * ldb + k0 + 4 * (v % (ks / 4)));
        }
      }
    }
  };
  auto stage = [&](int ks) {
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int v = tid + 256 * x, kr = 16 * x + tid % 16, c4 = 4 * (tid / 16);
      if (v < ks * 16) {
        if (TA) {
#pragma unroll
          for (int e = 0; e < 4; ++e) As[(c4 + e) * LD + kr] = xa[x][e];
        } else {
          *reinterpret_cast<f32x4*>(As + (v / (ks / 4)) * LD + 4 * (v % (ks / 4))) = xa[x];
        }
        if (!TB) {
#pragma unroll
          for (int e = 0; e < 4; ++e) Bs[(c4 + e) * LD + kr] = xb[x][e];
        } else {
          *reinterpret_cast<f32x4*>(Bs + (v / (ks / 4)) * LD + 4 * (v % (ks / 4))) = xb[x];
        }
      }
    }
  };
  // MFMA operands: lane l = 16 g + i holds row i of the A tile and column i
  // of the B tile at the k this step gives group g; output register r is row
  // 4 g + r, column i of the tile.
  const int l = tid & 63, lm = l & 15, lg = l >> 4;
  const int wm = (tid >> 7) * 32, wn = ((tid >> 6) & 1) * 32;  // this wave's quarter
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0, K < kGemmKStage ? K : kGemmKStage);
  for (int k0 = 0; k0 < K; k0 += kGemmKStage) {
    const int ks = K - k0 < kGemmKStage ? K - k0 : kGemmKStage;
    if (k0 > 0) __syncthreads();  // the previous stage's reads are done
    stage(ks);
    __syncthreads();
    if (k0 + kGemmKStage < K) {
      const int k1 = k0 + kGemmKStage;
      fetch(k1, K - k1 < kGemmKStage ? K - k1 : kGemmKStage);
    }
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
    };
    if (ks == kGemmKStage) {
#pragma unroll
      for (int kb = 0; kb < kGemmKStage / 16; ++kb) kblock(kb);
    } else {
      for (int kb = 0; kb < ks / 16; ++kb) kblock(kb);
    }
  }
  float* c = Cm + bt * sc;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm + 16 * ti + 4 * lg + i, nn = n0 + wn + 16 * tj + lm;
        if (m < M && nn < N) {
          const bool keep = mask == 0 || (mask == 1 ? nn <= m : nn < m);
          const float v = keep ? alpha * acc[ti][tj][i] : 0.f;
          c[(size_t)m * ldc + nn] = acc_c ? c[(size_t)m * ldc + nn] + v : v;
        }
      }
}

// Operand orientations of fp32_gemm_kernel, as tags for launch_fp32_gemm.
struct GemmNN { static constexpr bool TA = false, TB = false; };
struct GemmNT { static constexpr bool TA = false, TB = true; };
struct GemmTN { static constexpr bool TA = true, TB = false; };

// Launch of fp32_gemm_kernel over NB batch items.
template <bool TA, bool TB>
inline hipError_t launch_fp32_gemm(const float* A, const float* B, float* Cm, int M, int N, int K,
                                   int lda, int ldb, int ldc, size_t sa, size_t sb, size_t sc,
                                   float alpha, int acc_c, int mask, size_t NB, hipStream_t stream) {
  if (K % 16 || M % 4 || N % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)NB, (N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL((fp32_gemm_kernel<TA, TB>), grid, dim3(256), 0, stream, A, B, Cm, M, N, K, lda,
                     ldb, ldc, sa, sb, sc, alpha, acc_c, mask);
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
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx / C, j = idx % C;
    As[i][j] = j < i ? (r ? r[i] : 1.f) * A[pcc + idx] : 0.f;
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
