// KDA chunked forward pass (prompt processing), gfx950.
//
// The chunkwise algorithm follows the Kimi Linear report as summarised on the
// greeksharifa.github.io page (section 3.1 "Hardware-Efficient Chunkwise
// Algorithm", section 3.2 "Efficiency Analysis", Appendix B/C notes): within a
// chunk the rank-1 updates are gathered into a WY representation whose
// auxiliary matrix comes from a UT transform (a unit lower-triangular inverse
// by forward substitution); the output is the incoming-state term plus a
// causally masked intra-chunk term; the state is carried between chunks.
// Written out for a chunk of n <= C rows entering with state S (d_k x d_v):
//
//   Gamma_r = sum_{s<=r} g_s         (per key channel), gam_r = exp(Gamma_r)
//   A[r,i]  = beta_r sum_c k_rc k_ic exp(Gamma_rc - Gamma_ic)     (i < r)
//   P[r,i]  =        sum_c q_rc k_ic exp(Gamma_rc - Gamma_ic)     (i <= r)
//   T       = (I + A)^{-1} Diag(beta)
//   W       = T (K * gam),   U0 = T V
//   U       = U0 - W S
//   O       = (Q * gam) S + P U
//   S'      = Diag(gam_n) S + (K * exp(Gamma_n - Gamma))^T U
//
// Two kernels split the work the way the method does ("parallel within each
// chunk, recurrent between chunks"):
//
//  intra_chunk_kernel  one workgroup per (chunk, head), all in parallel:
//                      decay cumsum, decayed operands, the two Grams A and P,
//                      the UT-transform solve, W.  It writes Q*gam, W,
//                      (K*exp(Gamma_n-Gamma))^T, P, T and gam_n to the
//                      workspace, already in MFMA fragment order.
//  inter_chunk_kernel  one workgroup per (sequence, head, 16 value columns):
//                      the serial loop over the sequence's chunks, with the
//                      state block held in MFMA accumulator registers.
//
// Decay factorisation.  The Grams need exp(Gamma_r - Gamma_i).  When the
// total decay inside a chunk is moderate (max over channels of -Gamma_n <=
// kSpanLimit), the kernel factors it as exp(Gamma_r) * exp(-Gamma_i) and runs
// both Grams on MFMA; every factor then stays well inside the fp32/bf16
// exponent range.  Otherwise the Grams are evaluated pair by pair with the
// exact exponent of the difference (slow, but only strong decay reaches it).
#include "kda_device.hpp"
#include "kda_launch.hpp"

#include <stdlib.h>

namespace kda {

constexpr float kSpanLimit = 40.f;
constexpr int kIntraThreads = 512;

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
template <class M, int D, int C>
struct Layout {
  static constexpr int NRT = C / 16;             // token row tiles per chunk
  static constexpr int KC = C < 32 ? 32 : C;     // token contraction extent (padded)
  static constexpr int NKC = KC / 32;            // fragments along tokens
  static constexpr int NKD = D / 32;             // fragments along channels
  static constexpr int NDT = D / 16;             // channel row tiles
  static constexpr int PF = M::kPFragBytes;
  static constexpr int FF = M::kFragBytes;
  static constexpr size_t kQt = 0;                                   // precise [C x D]
  static constexpr size_t kW = kQt + (size_t)NRT * NKD * PF;         // precise [C x D]
  static constexpr size_t kKb = kW + (size_t)NRT * NKD * PF;         // precise [D x KC]
  static constexpr size_t kP = kKb + (size_t)NDT * NKC * PF;         // precise [C x KC]
  static constexpr size_t kT = kP + (size_t)NRT * NKC * PF;          // precise [C x KC]
  static constexpr size_t kV = kT + (size_t)NRT * NKC * PF;          // plain   [D x KC] (V^T)
  static constexpr size_t kGam = kV + (size_t)NDT * NKC * FF;        // fp32 [D]
  static constexpr size_t kBytes = ((kGam + D * 4) + 255) / 256 * 256;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <class M>
static size_t chunk_bytes_m(int D, int C) {
  if (D == 64) {
    if (C == 16) return Layout<M, 64, 16>::kBytes;
    if (C == 32) return Layout<M, 64, 32>::kBytes;
    return Layout<M, 64, 64>::kBytes;
  }
  if (C == 16) return Layout<M, 128, 16>::kBytes;
  if (C == 32) return Layout<M, 128, 32>::kBytes;
  return Layout<M, 128, 64>::kBytes;
}

size_t prefill_chunk_bytes(int D, int chunk, bool in_bf16) {
  return in_bf16 ? chunk_bytes_m<ModeBF16>(D, chunk) : chunk_bytes_m<ModeF32>(D, chunk);
}

static size_t table_bytes(int num_seqs, int total_chunks) {
  return align256(sizeof(int32_t) * (size_t)(num_seqs + 1)) +
         align256(sizeof(int32_t) * (size_t)total_chunks);
}

size_t prefill_workspace_bytes(int num_seqs, int total_chunks, int H, int D, int chunk,
                               bool in_bf16) {
  return table_bytes(num_seqs, total_chunks) +
         (size_t)total_chunks * H * prefill_chunk_bytes(D, chunk, in_bf16);
}

// ---------------------------------------------------------------------------
// Sequence geometry shared by both kernels
// ---------------------------------------------------------------------------
struct SeqInfo {
  const int32_t* cu;        // device cu_seqlens or nullptr
  const int32_t* chunk_off; // [num_seqs + 1] chunk offsets (varlen only)
  const int32_t* chunk_seq; // [total_chunks] sequence of each chunk (varlen only)
  int num_seqs, seq_len, total_tokens, total_chunks;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ void seq_bounds(const SeqInfo& s, int n, int& bos, int& eos) {
  if (s.cu) {
    bos = clampi(s.cu[n], 0, s.total_tokens);
    eos = clampi(s.cu[n + 1], bos, s.total_tokens);
  } else {
    bos = n * s.seq_len;
    eos = bos + s.seq_len;
  }
}

template <int C>
__device__ __forceinline__ int chunks_of(int len) { return (len + C - 1) / C; }

// Varlen chunk table: block n writes chunk_off[n] (and chunk_off[N] for the
// last block) and chunk_seq[chunk_off[n] .. chunk_off[n+1]) = n.
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu,
                                                          int32_t* __restrict__ chunk_off,
                                                          int32_t* __restrict__ chunk_seq,
                                                          int num_seqs, int total_tokens,
                                                          int total_chunks, int C) {
  const int n = blockIdx.x;
  __shared__ int part[256];
  int acc = 0;
  for (int m = threadIdx.x; m < n; m += 256) {
    const int b = clampi(cu[m], 0, total_tokens), e = clampi(cu[m + 1], b, total_tokens);
    acc += (e - b + C - 1) / C;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  const int off = part[0];
  const int b = clampi(cu[n], 0, total_tokens), e = clampi(cu[n + 1], b, total_tokens);
  const int nc = (e - b + C - 1) / C;
  if (threadIdx.x == 0) {
    chunk_off[n] = off;
    if (n == num_seqs - 1) chunk_off[num_seqs] = off + nc;
  }
  for (int c = threadIdx.x; c < nc; c += 256)
    if (off + c < total_chunks) chunk_seq[off + c] = n;
}

// ---------------------------------------------------------------------------
// Precise 16x16x16 product from fp32 LDS matrices (used by the block solve).
// acc += A[ra.., ca..] (16x16) * B[rb.., cb..] (16x16); row-major, strides sa/sb.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 prod16(ModeBF16, f32x4 acc, const float* A, int sa, int ra, int ca,
                                        const float* B, int sb, int rb, int cb) {
  const int l = lane_id();
  const int g = l >> 4, r = l & 15;
  // MFMA 1: [A_hi | A_lo] x [B_hi ; B_hi]; MFMA 2: [A_hi | 0] x [B_lo ; 0].
  const int kbase = 8 * (g & 1);
  bf16x8 a1, b1, a2, b2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float av = A[(ra + r) * sa + ca + kbase + e];
    const float bv = B[(rb + kbase + e) * sb + cb + r];
    const bf16 ah = f2bf(av), bh = f2bf(bv);
    const bf16 al = f2bf(av - bf2f(ah)), bl = f2bf(bv - bf2f(bh));
    a1[e] = g < 2 ? ah : al;
    b1[e] = bh;
    a2[e] = g < 2 ? ah : f2bf(0.f);
    b2[e] = g < 2 ? bl : f2bf(0.f);
  }
  acc = mfma_bf16(a2, b2, acc);
  return mfma_bf16(a1, b1, acc);
}
__device__ __forceinline__ f32x4 prod16(ModeF32, f32x4 acc, const float* A, int sa, int ra, int ca,
                                        const float* B, int sb, int rb, int cb) {
  const int l = lane_id();
  const int g = l >> 4, r = l & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kk = 4 * s + g;
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(ra + r) * sa + ca + kk],
                                               B[(rb + kk) * sb + cb + r], acc, 0, 0, 0);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// LDS plan of the intra-chunk kernel.  One region is reused by the phases:
//   A  (fast path, per half of the channels): Qt', Kt', Kh' precise [C x 64]
//   S  (strong-decay path): Gamma fp32 [C x (D+1)]
//   B  (after the Grams): X, Y scratch, A, P (fp32)
//   C  (W product): X, KtT precise [D x KC]
// plus the persistent scan totals, beta and a flag.
// ---------------------------------------------------------------------------
template <class M, int D, int C>
struct IntraLds {
  typedef typename M::in_t plain_t;  // element of one half of a precise matrix
  static constexpr int KC = Layout<M, D, C>::KC;
  static constexpr int NCG = D / 8;
  static constexpr int RPT = (C * NCG / kIntraThreads) > 1 ? (C * NCG / kIntraThreads) : 1;
  static constexpr int NRG = C / RPT;
  static constexpr int DH = 64;                      // channels per Gram pass
  static constexpr int NHALF = D / DH;
  static constexpr int SH = DH + kPad;               // row stride of [C x DH] operands
  static constexpr int SK = KC + kPad;               // row stride of [D x KC] operands
  static constexpr int SF = KC + 1;                  // row stride of fp32 [C x KC] matrices
  static constexpr int SG = D + 1;                   // row stride of the fp32 Gamma array
  static constexpr size_t kHalfPlain = (size_t)C * SH * sizeof(plain_t);
  static constexpr size_t kHalfPrecise = M::kSplit ? 2 * kHalfPlain : kHalfPlain;
  static constexpr size_t kPhaseA = 3 * kHalfPrecise;
  static constexpr size_t kPhaseS = (size_t)C * SG * 4;
  static constexpr size_t kFMat = ((size_t)C * SF * 4 + 15) / 16 * 16;
  static constexpr size_t kYsc = 4 * 16 * 17 * 4;
  static constexpr size_t kPhaseB = 3 * kFMat + kYsc;
  static constexpr size_t kKtTplain = ((size_t)D * SK * sizeof(plain_t) + 15) / 16 * 16;
  static constexpr size_t kKtT = M::kSplit ? 2 * kKtTplain : kKtTplain;
  static constexpr size_t kPhaseC = kFMat + kKtT;
  // Phase K (before A): K-bar^T (precise) and V^T (plain) staged [D x KC]
  // for the fragment copy-out.
  static constexpr size_t kPhaseK = kKtT + kKtTplain;
  static constexpr size_t m0 = kPhaseA > kPhaseK ? kPhaseA : kPhaseK;
  static constexpr size_t m1 = m0 > kPhaseS ? m0 : kPhaseS;
  static constexpr size_t m2 = kPhaseB > kPhaseC ? kPhaseB : kPhaseC;
  static constexpr size_t kUnion = ((m1 > m2 ? m1 : m2) + 15) / 16 * 16;
  static constexpr size_t kScan = (size_t)NRG * D * 4;
  static constexpr size_t kBeta = (size_t)KC * 4;
  static constexpr size_t kTotal = kUnion + kScan + kBeta + 16;
  // offsets
  static constexpr size_t oQt = 0, oKt = kHalfPrecise, oKh = 2 * kHalfPrecise;  // phase A
  static constexpr size_t oG = 0;                                              // phase S
  static constexpr size_t oX = 0, oY = kFMat, oA = kFMat + kYsc, oP = 2 * kFMat + kYsc;  // B
  static constexpr size_t oKtT = kFMat;                                        // phase C
  static constexpr size_t oKbS = 0, oVS = kKtT;                                // phase K
  static constexpr size_t oScan = kUnion, oBeta = oScan + kScan, oFlag = oBeta + kBeta;
};

template <class M>
struct LdsPrecise;  // pointers to a precise LDS matrix
template <>
struct LdsPrecise<ModeBF16> {
  bf16* hi;
  bf16* lo;
  __device__ LdsPrecise(char* base, size_t plain_bytes)
      : hi(reinterpret_cast<bf16*>(base)), lo(reinterpret_cast<bf16*>(base + plain_bytes)) {}
  __device__ void store(int idx, float x) {
    const bf16 h = f2bf(x);
    hi[idx] = h;
    lo[idx] = f2bf(x - bf2f(h));
  }
  // N consecutive elements starting at idx (idx a multiple of N).
  template <int N>
  __device__ void storeN(int idx, const float* x) {
    typedef __bf16 vec_t __attribute__((ext_vector_type(N)));
    vec_t h, l;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      h[e] = f2bf(x[e]);
      l[e] = f2bf(x[e] - bf2f(h[e]));
    }
    *reinterpret_cast<vec_t*>(hi + idx) = h;
    *reinterpret_cast<vec_t*>(lo + idx) = l;
  }
  __device__ ModeBF16::PFrag pfrag(int stride, int row0, int k0) const {
    return lds_pfrag(ModeBF16{}, hi, lo, stride, row0, k0);
  }
};
template <>
struct LdsPrecise<ModeF32> {
  float* v;
  __device__ LdsPrecise(char* base, size_t) : v(reinterpret_cast<float*>(base)) {}
  __device__ void store(int idx, float x) { v[idx] = x; }
  template <int N>
  __device__ void storeN(int idx, const float* x) {
    typedef float vec_t __attribute__((ext_vector_type(N)));
    vec_t t;
#pragma unroll
    for (int e = 0; e < N; ++e) t[e] = x[e];
    *reinterpret_cast<vec_t*>(v + idx) = t;
  }
  __device__ ModeF32::PFrag pfrag(int stride, int row0, int k0) const {
    return lds_pfrag(ModeF32{}, v, nullptr, stride, row0, k0);
  }
};

// Write eight consecutive-k fp32 values of one lane into a global fragment.
// `lane` is the lane that owns (row, k-group) in the fragment.
__device__ __forceinline__ void gst_pfrag8(ModeBF16, char* frag, int lane, const float* x) {
  bf16x8 h, lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f2bf(x[e]);
    lo[e] = f2bf(x[e] - bf2f(h[e]));
  }
  *reinterpret_cast<bf16x8*>(frag + lane * 16) = h;
  *reinterpret_cast<bf16x8*>(frag + 1024 + lane * 16) = lo;
}
__device__ __forceinline__ void gst_pfrag8(ModeF32, char* frag, int lane, const float* x) {
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[e];
  *reinterpret_cast<f32x8*>(frag + lane * 32) = v;
}
// Store a run of N (1, 2 or 4) consecutive k values starting at element e0
// (a multiple of N) of a lane's slot in a precise fragment, as one store per
// half.
template <int N>
__device__ __forceinline__ void gst_pfrag_run(ModeBF16, char* frag, int lane, int e0, const float* x) {
  typedef __bf16 vec_t __attribute__((ext_vector_type(N)));
  vec_t h, lo;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    h[e] = f2bf(x[e]);
    lo[e] = f2bf(x[e] - bf2f(h[e]));
  }
  *reinterpret_cast<vec_t*>(frag + lane * 16 + e0 * 2) = h;
  *reinterpret_cast<vec_t*>(frag + 1024 + lane * 16 + e0 * 2) = lo;
}
// The same for a plain fragment (one bf16 or fp32 value per element).
template <int N>
__device__ __forceinline__ void gst_frag_run(ModeBF16, char* frag, int lane, int e0, const bf16* x) {
  typedef __bf16 vec_t __attribute__((ext_vector_type(N)));
  vec_t h;
#pragma unroll
  for (int e = 0; e < N; ++e) h[e] = x[e];
  *reinterpret_cast<vec_t*>(frag + lane * 16 + e0 * 2) = h;
}
template <int N>
__device__ __forceinline__ void gst_frag_run(ModeF32, char* frag, int lane, int e0, const float* x) {
  typedef float vec_t __attribute__((ext_vector_type(N)));
  vec_t v;
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = x[e];
  *reinterpret_cast<vec_t*>(frag + lane * 32 + e0 * 4) = v;
}
template <int N>
__device__ __forceinline__ void gst_pfrag_run(ModeF32, char* frag, int lane, int e0, const float* x) {
  typedef float vec_t __attribute__((ext_vector_type(N)));
  vec_t v;
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = x[e];
  *reinterpret_cast<vec_t*>(frag + lane * 32 + e0 * 4) = v;
}

struct KernelPtrs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* o;
  const float* s0;
  float* s1;
  char* ops;       // per-(chunk, head) operand blocks
  int H;
};

// Lower-triangular 16x16 tile t (row-major order over b <= a) -> (a, b).
__device__ __forceinline__ void tile_ab(int t, int& a, int& b) {
  a = 0;
  while ((a + 1) * (a + 2) / 2 <= t) ++a;
  b = t - a * (a + 1) / 2;
}

// ---------------------------------------------------------------------------
// Intra-chunk kernel: grid (total_chunks, H), 512 threads (8 waves), two
// workgroups per CU, so four waves share each SIMD to cover each other's
// latency.
// ---------------------------------------------------------------------------
template <class M, int D, int C>
__global__ __launch_bounds__(kIntraThreads, 4) void intra_chunk_kernel(KernelPtrs kp, SeqInfo si) {
  typedef typename M::in_t in_t;
  typedef Layout<M, D, C> LY;
  typedef IntraLds<M, D, C> L;
  constexpr int NRT = LY::NRT, KC = LY::KC, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int NCG = L::NCG, RPT = L::RPT, NRG = L::NRG, SH = L::SH, SK = L::SK, SF = L::SF;
  constexpr int NTILE = NRT * (NRT + 1) / 2;
  constexpr int NW = kIntraThreads / 64;
  constexpr int TPW = (NTILE + NW - 1) / NW;  // Gram tiles per wave
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int cid = blockIdx.x;
  const int h = blockIdx.y;
  const int H = kp.H;
  const int tid = threadIdx.x;
  const int w = wave_id(), l = lane_id();

  // ---- which sequence and token range ----
  int n, ci;
  if (si.cu) {
    n = clampi(si.chunk_seq[cid], 0, si.num_seqs - 1);
    ci = cid - si.chunk_off[n];
  } else {
    const int per = chunks_of<C>(si.seq_len);
    n = cid / per;
    ci = cid % per;
  }
  int bos, eos;
  seq_bounds(si, n, bos, eos);
  // A device table that disagrees with the host one can only shorten chunks,
  // never move them outside [bos, eos].
  const long long t0l = (long long)bos + (long long)(ci < 0 ? 0 : ci) * C;
  const int t0 = (int)(t0l < eos ? t0l : eos);
  const int len = clampi(eos - t0, 0, C);
  char* blk = kp.ops + ((size_t)cid * H + h) * LY::kBytes;

  const in_t* qg = reinterpret_cast<const in_t*>(kp.q);
  const in_t* kg = reinterpret_cast<const in_t*>(kp.k);
  const in_t* vg = reinterpret_cast<const in_t*>(kp.v);
  float* scan = reinterpret_cast<float*>(smem + L::oScan);
  float* beta_s = reinterpret_cast<float*>(smem + L::oBeta);
  int* flag = reinterpret_cast<int*>(smem + L::oFlag);
  typedef typename L::plain_t plain_t;
  LdsPrecise<M> KbS(smem + L::oKbS, L::kKtTplain);
  plain_t* VS = reinterpret_cast<plain_t*>(smem + L::oVS);

  // ---- step 1: loads (all issued up front), cumulative decay ----
  const bool active = tid < NCG * NRG;
  const int cg = tid % NCG, rg = tid / NCG;
  float gam[RPT][8], qv[RPT][8], kv[RPT][8];
  in_t vv[8][RPT];  // V^T run: value column 8cg+e, tokens rg*RPT .. +RPT-1
  if (active) {
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
      const int r = rg * RPT + p;
      if (r < len) {
        const size_t base = ((size_t)(t0 + r) * H + h) * D + 8 * cg;
        load8(kp.g + base, gam[p]);
        load8(qg + base, qv[p]);
        load8(kg + base, kv[p]);
        float vtmp[8];
        load8(vg + base, vtmp);
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e][p] = (in_t)vtmp[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { gam[p][e] = 0.f; qv[p][e] = 0.f; kv[p][e] = 0.f; vv[e][p] = (in_t)0.f; }
      }
    }
  }
  for (int i = tid; i < KC; i += kIntraThreads) beta_s[i] = (i < len) ? kp.beta[(size_t)(t0 + i) * H + h] : 0.f;
  if (tid == 0) *flag = 0;
  if (active) {
#pragma unroll
    for (int p = 1; p < RPT; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[p][e] += gam[p - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) scan[rg * D + 8 * cg + e] = gam[RPT - 1][e];
  }
  __syncthreads();
  float last[8];
  if (active) {
    float off[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { off[e] = 0.f; last[e] = 0.f; }
    // Partial unrolling only: a fully unrolled loop would hoist every
    // load of the scan table into registers.
#pragma unroll 2
    for (int j = 0; j < NRG; ++j) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(scan + j * D + 8 * cg);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(scan + j * D + 8 * cg + 4);
      const float m = j < rg ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        off[e] += m * s0[e];
        off[4 + e] += m * s1[e];
        last[e] += s0[e];
        last[4 + e] += s1[e];
      }
    }
    bool big = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) big |= (last[e] < -kSpanLimit);
    if (big) atomicOr(flag, 1);
#pragma unroll
    for (int p = 0; p < RPT; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[p][e] += off[e];
  }
  __syncthreads();
  const bool fast = (*flag == 0);

  // ---- decayed operands.  Q*gam and K*exp(Gamma_n - Gamma) go straight to
  // their global fragments; K*gam and K/gam stay in registers.
  float kt[RPT][8], kh[RPT][8];
  if (active) {
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) reinterpret_cast<float*>(blk + LY::kGam)[8 * cg + e] = __expf(last[e]);
    }
    float kb[8][RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
      const int r = rg * RPT + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ep = __expf(gam[p][e]);
        qv[p][e] *= ep;                                   // now Q * gam
        kt[p][e] = kv[p][e] * ep;
        kh[p][e] = fast ? kv[p][e] * __expf(-gam[p][e]) : 0.f;
        kb[e][p] = kv[p][e] * __expf(last[e] - gam[p][e]);
      }
      // Q*gam fragment: row r, k = 8cg..8cg+7 -> fragment (r/16, cg/4), lane (r%16)+16(cg%4).
      gst_pfrag8(M{}, blk + LY::kQt + ((size_t)(r / 16) * NKD + cg / 4) * LY::PF,
                 (r % 16) + 16 * (cg % 4), qv[p]);
    }
    // K-bar^T and V^T go to LDS transposed (row = channel c = 8cg+e, k =
    // tokens rg*RPT .. +RPT-1), then out as whole fragments below: storing
    // these short transposed runs straight to memory costs far more.
    const int r0 = rg * RPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * cg + e;
      KbS.template storeN<RPT>(c * SK + r0, kb[e]);
#pragma unroll
      for (int p = 0; p < RPT; ++p) VS[c * SK + r0 + p] = vv[e][p];
    }
  }
  if (KC > C) {  // zero the padded tokens
    for (int idx = tid; idx < D * (KC - C); idx += kIntraThreads) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      KbS.store(c * SK + i, 0.f);
      VS[c * SK + i] = (plain_t)0.f;
    }
  }
  __syncthreads();
  // Fragment (channel tile rt, token block kb): lane l reads row 16rt + (l&15),
  // tokens 32kb + 8(l>>4) .. +7, and stores them as one contiguous slot.
  for (int f = w; f < NDT * NKC; f += NW) {
    const int rt = f / NKC, kb = f % NKC;
    st_pfrag(M{}, blk + LY::kKb + (size_t)f * LY::PF, KbS.pfrag(SK, 16 * rt, 32 * kb));
    st_frag(M{}, blk + LY::kV + (size_t)f * LY::FF, lds_frag(M{}, VS, SK, 16 * rt, 32 * kb));
  }
  __syncthreads();  // the Gram operands reuse this region

  // ---- step 2: Grams A and P ----
  f32x4 accA[TPW], accP[TPW];
#pragma unroll
  for (int s = 0; s < TPW; ++s) { accA[s] = f32x4{0, 0, 0, 0}; accP[s] = accA[s]; }
  if (fast) {
    LdsPrecise<M> Qh(smem + L::oQt, L::kHalfPlain);
    LdsPrecise<M> Kth(smem + L::oKt, L::kHalfPlain);
    LdsPrecise<M> Khh(smem + L::oKh, L::kHalfPlain);
#pragma unroll
    for (int half = 0; half < L::NHALF; ++half) {
      if (active && (cg * 8) / L::DH == half) {
        const int c0 = 8 * cg - half * L::DH;
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
          const int r = rg * RPT + p;
          Qh.template storeN<8>(r * SH + c0, qv[p]);
          Kth.template storeN<8>(r * SH + c0, kt[p]);
          Khh.template storeN<8>(r * SH + c0, kh[p]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < TPW; ++s) {
        const int t = w + NW * s;
        if (t < NTILE) {
          int a, b;
          tile_ab(t, a, b);
#pragma unroll
          for (int kb = 0; kb < L::DH / 32; ++kb) {
            const auto khf = Khh.pfrag(SH, 16 * b, 32 * kb);
            accP[s] = mma_pp(Qh.pfrag(SH, 16 * a, 32 * kb), khf, accP[s]);
            accA[s] = mma_pp(Kth.pfrag(SH, 16 * a, 32 * kb), khf, accA[s]);
          }
        }
      }
      __syncthreads();  // the next half (or phase B) overwrites the operands
    }
  } else {
    // Strong decay: exact pairwise evaluation.  Gamma goes to LDS; thread tid
    // owns row r = tid / 8 and columns i = tid % 8, +8, ... <= r.
    float* Gs = reinterpret_cast<float*>(smem + L::oG);
    if (active) {
#pragma unroll
      for (int p = 0; p < RPT; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) Gs[(rg * RPT + p) * L::SG + 8 * cg + e] = gam[p][e];
    }
    __syncthreads();
  }
  float* As = reinterpret_cast<float*>(smem + L::oA);
  float* Ps = reinterpret_cast<float*>(smem + L::oP);
  float* Xs = reinterpret_cast<float*>(smem + L::oX);
  float* Ysc = reinterpret_cast<float*>(smem + L::oY);
  constexpr int NPAIR = (C + 7) / 8;  // columns per thread in the pairwise path
  float pa[NPAIR], pp[NPAIR];
  if (!fast) {
    const float* Gs = reinterpret_cast<const float*>(smem + L::oG);
    const int r = tid >> 3;
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) { pa[m] = 0.f; pp[m] = 0.f; }
    if (r < len) {
#pragma unroll
      for (int m = 0; m < NPAIR; ++m) {
        const int i = (tid & 7) + 8 * m;
        if (i <= r) {
          float sa = 0.f, sp = 0.f;
          for (int c = 0; c < D; ++c) {
            const float kr = (float)kg[((size_t)(t0 + r) * H + h) * D + c];
            const float ki = (float)kg[((size_t)(t0 + i) * H + h) * D + c];
            const float qr = (float)qg[((size_t)(t0 + r) * H + h) * D + c];
            const float ex = __expf(Gs[r * L::SG + c] - Gs[i * L::SG + c]);
            sa += kr * ki * ex;
            sp += qr * ki * ex;
          }
          pa[m] = sa;
          pp[m] = sp;
        }
      }
    }
    __syncthreads();  // Gamma reads done before A/P overwrite it
  }
  // ---- A (strictly lower, times beta_r), P (lower), X cleared ----
  for (int idx = tid; idx < C * KC; idx += kIntraThreads) {
    const int r = idx / KC, i = idx % KC;
    As[r * SF + i] = 0.f;
    Ps[r * SF + i] = 0.f;
    Xs[r * SF + i] = 0.f;
  }
  __syncthreads();
  if (fast) {
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      const int t = w + NW * s;
      if (t < NTILE) {
        int a, b;
        tile_ab(t, a, b);
        const int i = 16 * b + (l & 15);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 16 * a + 4 * (l >> 4) + x;
          if (i < r) As[r * SF + i] = beta_s[r] * accA[s][x];
          if (i <= r) Ps[r * SF + i] = accP[s][x];
        }
      }
    }
  } else {
    const int r = tid >> 3;
    if (r < C) {
#pragma unroll
      for (int m = 0; m < NPAIR; ++m) {
        const int i = (tid & 7) + 8 * m;
        if (i <= r && r < len) {
          if (i < r) As[r * SF + i] = beta_s[r] * pa[m];
          Ps[r * SF + i] = pp[m];
        }
      }
    }
  }
  __syncthreads();

  // ---- step 3: X = (I + A)^{-1} by blocked forward substitution ----
  if (w == 0) {
    // diagonal 16x16 blocks: lane = 16*block + column
    const int bk = l >> 4, j = l & 15;
    if (bk < NRT) {
      float x[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) x[s] = (s == j) ? 1.f : 0.f;
      const float* Ab = As + (16 * bk) * SF + 16 * bk;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int s = r + 1; s < 16; ++s) x[s] -= Ab[s * SF + r] * x[r];
        // Keep each elimination step's LDS reads next to their use; hoisting
        // all 120 of them would cost as many registers.
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) Xs[(16 * bk + s) * SF + 16 * bk + j] = x[s];
    }
  }
  __syncthreads();
  // off-diagonal blocks, one level (a - b) at a time:
  //   X_ab = -X_aa * sum_{m=b}^{a-1} A_am X_mb
#pragma unroll
  for (int lev = 1; lev < NRT; ++lev) {
    const int a = lev + w, b = w;
    const bool mine = (w < NRT - lev);
    if (mine) {
      f32x4 y = {0, 0, 0, 0};
      for (int m = b; m < a; ++m) y = prod16(M{}, y, As, SF, 16 * a, 16 * m, Xs, SF, 16 * m, 16 * b);
      float* Yw = Ysc + w * 16 * 17;
#pragma unroll
      for (int x = 0; x < 4; ++x) Yw[(4 * (l >> 4) + x) * 17 + (l & 15)] = y[x];
    }
    __syncthreads();
    if (mine) {
      f32x4 xab = {0, 0, 0, 0};
      xab = prod16(M{}, xab, Xs, SF, 16 * a, 16 * a, Ysc + w * 16 * 17, 17, 0, 0);
#pragma unroll
      for (int x = 0; x < 4; ++x) Xs[(16 * a + 4 * (l >> 4) + x) * SF + 16 * b + (l & 15)] = -xab[x];
    }
    __syncthreads();
  }

  // ---- step 4: T = X Diag(beta) and P fragments (fragment (rt, kb)) ----
  for (int f = w; f < NRT * NKC; f += NW) {
    const int r = 16 * (f / NKC) + (l & 15), i0 = 32 * (f % NKC) + 8 * (l >> 4);
    float tv[8], pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tv[e] = Xs[r * SF + i0 + e] * beta_s[i0 + e];
      pv[e] = Ps[r * SF + i0 + e];
    }
    gst_pfrag8(M{}, blk + LY::kT + (size_t)f * LY::PF, l, tv);
    gst_pfrag8(M{}, blk + LY::kP + (size_t)f * LY::PF, l, pv);
  }
  __syncthreads();  // A and P are dead; K*gam^T may overwrite them
  LdsPrecise<M> KtT(smem + L::oKtT, L::kKtTplain);
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float run[RPT];
#pragma unroll
      for (int p = 0; p < RPT; ++p) run[p] = kt[p][e];
      KtT.template storeN<RPT>((8 * cg + e) * SK + rg * RPT, run);
    }
  }
  if (KC > C) {
    for (int idx = tid; idx < D * (KC - C); idx += kIntraThreads) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      KtT.store(c * SK + i, 0.f);
    }
  }
  __syncthreads();
  // ---- W^T = (K*gam)^T T^T, tile (channel tile ct, token tile rt).  The
  // accumulator lane l holds W[16rt + (l&15)][16ct + 4(l>>4) + x], which is
  // four consecutive k values of one lane slot of the W fragment (rt, ct/2).
  for (int t = w; t < NRT * NDT; t += NW) {
    const int rt = t / NDT, ct = t % NDT;
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      if (32 * kb > 16 * rt + 15) break;
      const int r = 16 * rt + (l & 15), i0 = 32 * kb + 8 * (l >> 4);
      float tv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = Xs[r * SF + i0 + e] * beta_s[i0 + e];
      acc = mma_pp(KtT.pfrag(SK, 16 * ct, 32 * kb), make_pfrag(M{}, tv), acc);
    }
    const int q4 = l >> 4;
    const int lane_w = (l & 15) + 16 * (2 * (ct & 1) + (q4 >> 1));
    float wv[4] = {acc[0], acc[1], acc[2], acc[3]};
    gst_pfrag_run<4>(M{}, blk + LY::kW + ((size_t)rt * NKD + ct / 2) * LY::PF, lane_w,
                     4 * (q4 & 1), wv);
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel: one workgroup per (sequence, head, block of value columns).
// ---------------------------------------------------------------------------
// Operands of one chunk, as held by one wave.  The phase-1 group (W, Q*gam,
// T, V^T) feeds U = T V - W S and Q*gam S; the phase-2 group (P, K-bar^T,
// gam_n) feeds the output and the state update.
template <class M, int D, int C, int NCT>
struct ChunkFrags {
  typedef Layout<M, D, C> LY;
  static constexpr int NST = LY::NDT / 4 > 0 ? LY::NDT / 4 : 1;  // state tiles per wave
  typename M::PFrag W[LY::NKD];
  typename M::PFrag Qt[LY::NKD];
  typename M::PFrag Tm[LY::NKC];
  typename M::Frag V[NCT][LY::NKC];
  typename M::PFrag P[LY::NKC];
  typename M::PFrag Kb[NST][LY::NKC];
  float gam[NST][4];
};

template <class M, int D, int C, int NCT>
__device__ __forceinline__ void load_frags_phase1(ChunkFrags<M, D, C, NCT>& f, const char* blk, int w,
                                                  int vt0) {
  typedef Layout<M, D, C> LY;
  // Every wave issues the same loads.  With fewer than four row tiles the
  // waves past the last one re-read it (their products are skipped): a load
  // that only some waves issue leaves the compiler's count of outstanding
  // loads wrong for the others, and a wait can then pass before the data
  // it guards has arrived.
  const int rt = LY::NRT == 4 ? w : min(w, LY::NRT - 1);
#pragma unroll
  for (int kb = 0; kb < LY::NKD; ++kb) {
    f.W[kb] = ld_pfrag(M{}, blk + LY::kW + (size_t)(rt * LY::NKD + kb) * LY::PF);
    f.Qt[kb] = ld_pfrag(M{}, blk + LY::kQt + (size_t)(rt * LY::NKD + kb) * LY::PF);
  }
#pragma unroll
  for (int kb = 0; kb < LY::NKC; ++kb) {
    f.Tm[kb] = ld_pfrag(M{}, blk + LY::kT + (size_t)(rt * LY::NKC + kb) * LY::PF);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      f.V[ct][kb] = ld_frag(M{}, blk + LY::kV + (size_t)((vt0 + ct) * LY::NKC + kb) * LY::FF);
  }
}

template <class M, int D, int C, int NCT>
__device__ __forceinline__ void load_frags_phase2(ChunkFrags<M, D, C, NCT>& f, const char* blk, int w) {
  typedef Layout<M, D, C> LY;
  constexpr int NST = ChunkFrags<M, D, C, NCT>::NST;
  const int l = lane_id();
  // Unconditional for every wave, as in load_frags_phase1.
  const int rt = LY::NRT == 4 ? w : min(w, LY::NRT - 1);
#pragma unroll
  for (int kb = 0; kb < LY::NKC; ++kb)
    f.P[kb] = ld_pfrag(M{}, blk + LY::kP + (size_t)(rt * LY::NKC + kb) * LY::PF);
  static_assert(LY::NDT == 4 * NST, "every wave owns NST state tiles");
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int st = w * NST + s;
#pragma unroll
    for (int kb = 0; kb < LY::NKC; ++kb)
      f.Kb[s][kb] = ld_pfrag(M{}, blk + LY::kKb + (size_t)(st * LY::NKC + kb) * LY::PF);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(blk + LY::kGam) + 16 * st + 4 * (l >> 4));
#pragma unroll
    for (int x = 0; x < 4; ++x) f.gam[s][x] = gv[x];
  }
}

template <class M, int D, int C, int NCT>
struct InterLds {
  typedef typename M::in_t plain_t;
  static constexpr int KC = Layout<M, D, C>::KC;
  static constexpr int SD = D + kPad;
  static constexpr int SK = KC + kPad;
  static constexpr int DVB = 16 * NCT;  // value columns per workgroup
  static constexpr size_t kSTplain = (size_t)DVB * SD * sizeof(plain_t);
  static constexpr size_t kUTplain = (size_t)DVB * SK * sizeof(plain_t);
  static constexpr size_t oST = 0;
  static constexpr size_t oUT = oST + (M::kSplit ? 2 : 1) * kSTplain;
  static constexpr size_t kTotal = oUT + (M::kSplit ? 2 : 1) * kUTplain;
};

// NCT = number of 16-column value tiles per workgroup (16, 32 or 64 columns).
// Every wave applies each operand fragment it loads to all NCT tiles, so a
// wider block divides the per-chunk operand traffic among fewer workgroups.
//
// Pipeline: two operand sets alternate between even and odd chunks.  After
// phase 1 of chunk c its set receives the phase-1 group of chunk c+2, and
// after phase 2 the other set receives the phase-2 group of chunk c+1.  That
// keeps about 55 loads per wave in flight, inside the 63-entry vmcnt range.
template <class M, int D, int C, int NCT, bool OUT_BF16>
__global__ __launch_bounds__(256) void inter_chunk_kernel(KernelPtrs kp, SeqInfo si, int num_pairs) {
  typedef Layout<M, D, C> LY;
  typedef InterLds<M, D, C, NCT> L;
  typedef ChunkFrags<M, D, C, NCT> CF;
  constexpr int NRT = LY::NRT, KC = LY::KC, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int NST = CF::NST;
  constexpr int DVB = L::DVB;
  constexpr int NVB = D / DVB;
  constexpr int SD = L::SD, SK = L::SK;
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  // XCD-aware mapping: consecutive block ids rotate over the 8 XCDs, so the
  // NVB column blocks of one (sequence, head) are given ids that land on the
  // same XCD and share its L2 for the per-chunk operands.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int pair = (slot / NVB) * 8 + xcd;
  const int vb = slot % NVB;
  if (pair >= num_pairs) return;
  const int H = kp.H;
  const int n = pair / H, h = pair % H;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int col0 = DVB * vb;  // first value column of this block

  int bos, eos;
  seq_bounds(si, n, bos, eos);
  const int cid0 = si.cu ? clampi(si.chunk_off[n], 0, si.total_chunks)
                         : n * chunks_of<C>(si.seq_len);
  // Never walk past the chunks the workspace was sized for.
  const int nch = min(chunks_of<C>(eos - bos), si.total_chunks - cid0);

  LdsPrecise<M> ST(smem + L::oST, L::kSTplain);
  LdsPrecise<M> UT(smem + L::oUT, L::kUTplain);

  // ---- state block in accumulator layout: tile (st, ct) holds rows
  // 16st.., columns col0 + 16ct.. ----
  f32x4 S[NST][NCT];
  const size_t sbase = ((size_t)n * H + h) * D * D;
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int st = w * NST + s;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = 16 * st + 4 * (l >> 4) + x;
        S[s][ct][x] = (kp.s0 && st < NDT)
                          ? kp.s0[sbase + (size_t)c * D + col0 + 16 * ct + (l & 15)] : 0.f;
      }
  }
  auto write_state_lds = [&]() {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (NDT == 4 * NST || st < NDT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float v4[4] = {S[s][ct][0], S[s][ct][1], S[s][ct][2], S[s][ct][3]};
          ST.template storeN<4>((16 * ct + (l & 15)) * SD + 16 * st + 4 * (l >> 4), v4);
        }
      }
    }
  };
  write_state_lds();
  // Zero the padded token columns of UT once (KC > C); nothing writes them.
  if (KC > C) {
    for (int idx = tid; idx < DVB * (KC - C); idx += 256) UT.store((idx / (KC - C)) * SK + C + idx % (KC - C), 0.f);
  }

  auto blk_of = [&](int ci) { return kp.ops + ((size_t)(cid0 + ci) * H + h) * LY::kBytes; };
  const int vt0 = col0 / 16;  // first V^T fragment row tile of this block

  // One chunk.  `f` holds chunk ci; `g` is the other set.  Fetches past the
  // end re-read the last chunk: they stay unconditional, since a fetch under a
  // branch makes the compiler drain every outstanding load where the paths
  // join.
  auto process = [&](CF& f, CF& g, int ci) {
    const int t0 = bos + ci * C;
    const int len = eos - t0 < C ? eos - t0 : C;
    __syncthreads();  // ST ready
    f32x4 qs[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) qs[ct] = f32x4{0, 0, 0, 0};
    if (NRT == 4 || w < NRT) {
      // All B-operand fragments of this phase are read from LDS first, so
      // their latency is paid once rather than in front of every product.
      typename M::PFrag sf[NKD][NCT];
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) sf[kb][ct] = ST.pfrag(SD, 16 * ct, 32 * kb);
      f32x4 ws[NCT], u[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) { ws[ct] = f32x4{0, 0, 0, 0}; u[ct] = ws[ct]; }
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) u[ct] = mma_pf(f.Tm[kb], f.V[ct][kb], u[ct]);
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          ws[ct] = mma_pp(f.W[kb], sf[kb][ct], ws[ct]);
          qs[ct] = mma_pp(f.Qt[kb], sf[kb][ct], qs[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float v4[4] = {u[ct][0] - ws[ct][0], u[ct][1] - ws[ct][1], u[ct][2] - ws[ct][2],
                       u[ct][3] - ws[ct][3]};
        UT.template storeN<4>((16 * ct + (l & 15)) * SK + 16 * w + 4 * (l >> 4), v4);
      }
    }
    load_frags_phase1<M, D, C, NCT>(f, blk_of(min(ci + 2, nch - 1)), w, vt0);
    __syncthreads();  // UT ready; ST reads done
    typename M::PFrag uf[NKC][NCT];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) uf[kb][ct] = UT.pfrag(SK, 16 * ct, 32 * kb);
    if (NRT == 4 || w < NRT) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 o = qs[ct];
        // P is lower triangular: token blocks past this row tile are zero.
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb)
          if (32 * kb <= 16 * w + 15) o = mma_pp(f.P[kb], uf[kb][ct], o);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 16 * w + 4 * (l >> 4) + x;
          if (r < len) {
            const size_t oi = ((size_t)(t0 + r) * H + h) * D + col0 + 16 * ct + (l & 15);
            if constexpr (OUT_BF16)
              reinterpret_cast<bf16*>(kp.o)[oi] = f2bf(o[x]);
            else
              reinterpret_cast<float*>(kp.o)[oi] = o[x];
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (NDT == 4 * NST || st < NDT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int x = 0; x < 4; ++x) S[s][ct][x] *= f.gam[s][x];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) S[s][ct] = mma_pp(f.Kb[s][kb], uf[kb][ct], S[s][ct]);
      }
    }
    load_frags_phase2<M, D, C, NCT>(g, blk_of(min(ci + 1, nch - 1)), w);
    // ST is read again only after the next chunk's first barrier, and every
    // read of this chunk's ST happened before the second barrier.
    write_state_lds();
  };

  CF fa, fb;
  if (nch > 0) {
    load_frags_phase1<M, D, C, NCT>(fa, blk_of(0), w, vt0);
    load_frags_phase2<M, D, C, NCT>(fa, blk_of(0), w);
    load_frags_phase1<M, D, C, NCT>(fb, blk_of(min(1, nch - 1)), w, vt0);
  }
  for (int ci = 0; ci < nch; ci += 2) {
    process(fa, fb, ci);
    if (ci + 1 >= nch) break;
    process(fb, fa, ci + 1);
  }
  if (kp.s1) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (st < NDT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int c = 16 * st + 4 * (l >> 4) + x;
            kp.s1[sbase + (size_t)c * D + col0 + 16 * ct + (l & 15)] = S[s][ct][x];
          }
      }
    }
  }
}

// Value-column block width of the inter-chunk pass: wide blocks cut the
// per-chunk operand traffic (each block re-reads the chunk's operands), narrow
// ones give more workgroups.  Heuristic: keep at least ~2 workgroups per CU
// of work available when there are many (sequence, head) pairs.
// KDA_PREFILL_DVB (16, 32 or 64) overrides it, for tuning.
static int choose_nct(int pairs, int D) {
  static int env = -1;
  if (env < 0) {
    const char* e = getenv("KDA_PREFILL_DVB");
    const int v = e ? atoi(e) : 0;
    env = (v == 16 || v == 32 || v == 64) ? v / 16 : 0;
  }
  int nct = env;
  if (nct == 0) {
    const long long units16 = (long long)pairs * (D / 16);
    nct = units16 >= 4096 ? 4 : (units16 >= 1024 ? 2 : 1);
  }
  while (nct > 1 && D / (16 * nct) < 1) nct >>= 1;
  return nct;
}

template <class M, int D, int C, int NCT>
static void launch_inter(const PrefillArgs& a, const KernelPtrs& kp, const SeqInfo& si) {
  const int pairs = a.num_seqs * a.H;
  const int nvb = D / (16 * NCT);
  const int blocks = ((pairs + 7) / 8) * 8 * nvb;
  if (a.out_bf16)
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, NCT, true>), dim3(blocks), dim3(256), 0, a.stream,
                       kp, si, pairs);
  else
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, NCT, false>), dim3(blocks), dim3(256), 0, a.stream,
                       kp, si, pairs);
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
template <class M, int D, int C>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  typedef Layout<M, D, C> LY;
  char* ws = reinterpret_cast<char*>(a.workspace);
  SeqInfo si;
  si.cu = a.cu_seqlens;
  si.num_seqs = a.num_seqs;
  si.seq_len = a.seq_len;
  si.total_tokens = a.total_tokens;
  si.total_chunks = a.total_chunks;
  si.chunk_off = reinterpret_cast<const int32_t*>(ws);
  si.chunk_seq = reinterpret_cast<const int32_t*>(ws + align256(sizeof(int32_t) * (a.num_seqs + 1)));
  KernelPtrs kp;
  kp.q = a.q;
  kp.k = a.k;
  kp.v = a.v;
  kp.g = a.g;
  kp.beta = a.beta;
  kp.o = a.o;
  kp.s0 = a.initial_state;
  kp.s1 = a.final_state;
  kp.ops = ws + table_bytes(a.num_seqs, a.total_chunks);
  kp.H = a.H;

  if (a.cu_seqlens) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(a.num_seqs), dim3(256), 0, a.stream, a.cu_seqlens,
                       const_cast<int32_t*>(si.chunk_off), const_cast<int32_t*>(si.chunk_seq),
                       a.num_seqs, a.total_tokens, a.total_chunks, C);
  }
  if (a.total_chunks > 0) {
    constexpr size_t lds = IntraLds<M, D, C>::kTotal;
    static_assert(lds <= 160 * 1024, "intra-chunk LDS");
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&intra_chunk_kernel<M, D, C>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((intra_chunk_kernel<M, D, C>), dim3(a.total_chunks, a.H), dim3(kIntraThreads), lds,
                       a.stream, kp, si);
  }
  const int nct = choose_nct(a.num_seqs * a.H, D);
  if (nct == 4)
    launch_inter<M, D, C, 4>(a, kp, si);
  else if (nct == 2)
    launch_inter<M, D, C, 2>(a, kp, si);
  else
    launch_inter<M, D, C, 1>(a, kp, si);
  return hipGetLastError();
}

template <class M>
static hipError_t launch_prefill_m(const PrefillArgs& a) {
  if (a.D == 64) {
    if (a.chunk == 16) return launch_prefill_t<M, 64, 16>(a);
    if (a.chunk == 32) return launch_prefill_t<M, 64, 32>(a);
    return launch_prefill_t<M, 64, 64>(a);
  }
  if (a.chunk == 16) return launch_prefill_t<M, 128, 16>(a);
  if (a.chunk == 32) return launch_prefill_t<M, 128, 32>(a);
  return launch_prefill_t<M, 128, 64>(a);
}

hipError_t launch_prefill(const PrefillArgs& a) {
  return a.in_bf16 ? launch_prefill_m<ModeBF16>(a) : launch_prefill_m<ModeF32>(a);
}

}  // namespace kda
