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

namespace kda {

constexpr float kSpanLimit = 40.f;

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
  static constexpr size_t kGam = kT + (size_t)NRT * NKC * PF;        // fp32 [D]
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
// LDS plan of the intra-chunk kernel
// ---------------------------------------------------------------------------
template <class M, int D, int C>
struct IntraLds {
  typedef typename M::in_t plain_t;  // element of a plain LDS operand (bf16 or fp32)
  static constexpr int KC = Layout<M, D, C>::KC;
  static constexpr int NCG = D / 8;
  static constexpr int RPT = (C * NCG / 256) > 1 ? (C * NCG / 256) : 1;
  static constexpr int NRG = C / RPT;
  static constexpr int SD = D + kPad;    // row stride of [C x D] operands
  static constexpr int SK = KC + kPad;   // row stride of [D x KC] operands
  static constexpr int SF = KC + 1;      // row stride of fp32 [C x KC] matrices
  static constexpr int SG = D + 1;       // row stride of the fp32 Gamma array (slow path)
  static constexpr size_t kPlainMat = (size_t)C * SD * sizeof(plain_t);
  static constexpr size_t kPreciseMat = M::kSplit ? 2 * kPlainMat : kPlainMat;
  // Phase A, fast path (cumsum .. Grams): Qt, Kt, Kh (all precise).
  static constexpr size_t kPhaseA = 3 * kPreciseMat;
  // Phase B (after Grams): A, P, X (fp32 [C x SF]), Y scratch, W staging (fp32).
  static constexpr size_t kFMat = (size_t)C * SF * 4;
  static constexpr size_t kYsc = 4 * 16 * 17 * 4;
  static constexpr size_t kWst = (size_t)C * SD * 4;
  static constexpr size_t kPhaseB = 3 * kFMat + kYsc + kWst;
  // Strong-decay path: the fp32 Gamma array sits after A and P (it is dead by
  // the time X is formed there).
  static constexpr size_t kGammaBytes = (size_t)C * SG * 4;
  static constexpr size_t kPhaseS = 2 * kFMat + kGammaBytes;
  static constexpr size_t kMax1 = kPhaseA > kPhaseB ? kPhaseA : kPhaseB;
  static constexpr size_t kUnion = ((kMax1 > kPhaseS ? kMax1 : kPhaseS) + 15) / 16 * 16;
  // Persistent: KtT (precise [D x SK]), scan totals, beta, flag.
  static constexpr size_t kKtTplain = ((size_t)D * SK * sizeof(plain_t) + 15) / 16 * 16;
  static constexpr size_t kKtT = M::kSplit ? 2 * kKtTplain : kKtTplain;
  static constexpr size_t kScan = (size_t)NRG * D * 4;
  static constexpr size_t kBeta = (size_t)KC * 4;
  static constexpr size_t kTotal = kUnion + kKtT + kScan + kBeta + 16;
  // offsets
  static constexpr size_t oQt = 0, oKt = kPreciseMat, oKh = 2 * kPreciseMat;
  static constexpr size_t oA = 0, oP = kFMat, oX = 2 * kFMat, oY = 3 * kFMat, oWs = 3 * kFMat + kYsc;
  static constexpr size_t oG = 2 * kFMat;
  static constexpr size_t oKtT = kUnion, oScan = kUnion + kKtT, oBeta = oScan + kScan,
                          oFlag = oBeta + kBeta;
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
  __device__ ModeBF16::PFrag pfrag(int stride, int row0, int k0) const {
    return lds_pfrag(ModeBF16{}, hi, lo, stride, row0, k0);
  }
  __device__ ModeBF16::Frag hifrag(int stride, int row0, int k0) const {
    return lds_frag(ModeBF16{}, hi, stride, row0, k0);
  }
};
template <>
struct LdsPrecise<ModeF32> {
  float* v;
  __device__ LdsPrecise(char* base, size_t) : v(reinterpret_cast<float*>(base)) {}
  __device__ void store(int idx, float x) { v[idx] = x; }
  __device__ ModeF32::PFrag pfrag(int stride, int row0, int k0) const {
    return lds_pfrag(ModeF32{}, v, nullptr, stride, row0, k0);
  }
  __device__ ModeF32::Frag hifrag(int stride, int row0, int k0) const {
    return lds_frag(ModeF32{}, v, stride, row0, k0);
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
__device__ __forceinline__ void gst_frag8(ModeBF16, char* frag, int lane, const float* x) {
  bf16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = f2bf(x[e]);
  *reinterpret_cast<bf16x8*>(frag + lane * 16) = h;
}
__device__ __forceinline__ void gst_frag8(ModeF32, char* frag, int lane, const float* x) {
  gst_pfrag8(ModeF32{}, frag, lane, x);
}
// Store a run of `n` (<= 8) consecutive k values starting at element e0 of a
// lane's slot in a precise fragment.
template <int N>
__device__ __forceinline__ void gst_pfrag_run(ModeBF16, char* frag, int lane, int e0, const float* x) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const bf16 h = f2bf(x[e]);
    reinterpret_cast<bf16*>(frag + lane * 16)[e0 + e] = h;
    reinterpret_cast<bf16*>(frag + 1024 + lane * 16)[e0 + e] = f2bf(x[e] - bf2f(h));
  }
}
template <int N>
__device__ __forceinline__ void gst_pfrag_run(ModeF32, char* frag, int lane, int e0, const float* x) {
#pragma unroll
  for (int e = 0; e < N; ++e) reinterpret_cast<float*>(frag + lane * 32)[e0 + e] = x[e];
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

// ---------------------------------------------------------------------------
// Intra-chunk kernel: grid (total_chunks, H), 256 threads.
// ---------------------------------------------------------------------------
template <class M, int D, int C>
__global__ __launch_bounds__(256) void intra_chunk_kernel(KernelPtrs kp, SeqInfo si) {
  typedef typename M::in_t in_t;
  typedef Layout<M, D, C> LY;
  typedef IntraLds<M, D, C> L;
  constexpr int NRT = LY::NRT, KC = LY::KC, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int NCG = L::NCG, RPT = L::RPT, NRG = L::NRG, SD = L::SD, SK = L::SK, SF = L::SF;
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

  float* scan = reinterpret_cast<float*>(smem + L::oScan);
  float* beta_s = reinterpret_cast<float*>(smem + L::oBeta);
  int* flag = reinterpret_cast<int*>(smem + L::oFlag);
  LdsPrecise<M> Qt(smem + L::oQt, L::kPlainMat);
  LdsPrecise<M> Kt(smem + L::oKt, L::kPlainMat);
  LdsPrecise<M> Kh(smem + L::oKh, L::kPlainMat);
  LdsPrecise<M> KtT(smem + L::oKtT, L::kKtTplain);

  // ---- step 1: cumulative decay and decayed operands ----
  for (int i = tid; i < KC; i += 256) beta_s[i] = (i < len) ? kp.beta[(size_t)(t0 + i) * H + h] : 0.f;
  if (tid == 0) *flag = 0;
  // Zero the padded token columns of KtT (only when KC > C).
  if (KC > C) {
    for (int idx = tid; idx < D * (KC - C); idx += 256) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      KtT.store(c * SK + i, 0.f);
    }
  }
  const bool active = tid < NCG * NRG;
  const int cg = tid % NCG, rg = tid / NCG;
  float gam[RPT][8];
  if (active) {
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
      const int r = rg * RPT + p;
      float gv[8];
      if (r < len) {
        load8(kp.g + ((size_t)(t0 + r) * H + h) * D + 8 * cg, gv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[p][e] = (p ? gam[p - 1][e] : 0.f) + gv[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) scan[rg * D + 8 * cg + e] = gam[RPT - 1][e];
  }
  __syncthreads();
  float last[8];
  if (active) {
    float off[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { off[e] = 0.f; last[e] = 0.f; }
    for (int j = 0; j < NRG; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = scan[j * D + 8 * cg + e];
        if (j < rg) off[e] += s;
        last[e] += s;
      }
    }
#pragma unroll
    for (int p = 0; p < RPT; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[p][e] += off[e];
    bool big = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) big |= (last[e] < -kSpanLimit);
    if (big) atomicOr(flag, 1);
  }
  __syncthreads();
  const bool fast = (*flag == 0);

  if (active) {
    // gam_n (chunk decay) for the state update
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) reinterpret_cast<float*>(blk + LY::kGam)[8 * cg + e] = __expf(last[e]);
    }
    float* Gs = reinterpret_cast<float*>(smem + L::oG);  // strong-decay path only
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
      const int r = rg * RPT + p;
      float qv[8], kv[8];
      if (r < len) {
        load8(qg + ((size_t)(t0 + r) * H + h) * D + 8 * cg, qv);
        load8(kg + ((size_t)(t0 + r) * H + h) * D + 8 * cg, kv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { qv[e] = 0.f; kv[e] = 0.f; }
      }
      float qt[8], kt[8], kb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ep = __expf(gam[p][e]);
        qt[e] = qv[e] * ep;
        kt[e] = kv[e] * ep;
        kb[e] = kv[e] * __expf(last[e] - gam[p][e]);
      }
      // LDS operands
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * cg + e;
        KtT.store(c * SK + r, kt[e]);
        if (fast) {
          Qt.store(r * SD + c, qt[e]);
          Kt.store(r * SD + c, kt[e]);
          Kh.store(r * SD + c, kv[e] * __expf(-gam[p][e]));
        } else {
          Gs[r * L::SG + c] = gam[p][e];
        }
      }
      // Global Qt fragment: row r, k = 8cg..8cg+7 -> fragment (r/16, cg/4), lane (r%16)+16(cg%4).
      gst_pfrag8(M{}, blk + LY::kQt + ((size_t)(r / 16) * NKD + cg / 4) * LY::PF,
                 (r % 16) + 16 * (cg % 4), qt);
      // Global KbT fragments: row c = 8cg+e, k = token r.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * cg + e;
        char* fr = blk + LY::kKb + ((size_t)(c / 16) * NKC + r / 32) * LY::PF;
        gst_pfrag_run<1>(M{}, fr, (c % 16) + 16 * ((r % 32) / 8), r % 8, &kb[e]);
      }
    }
  }
  // Zero the padded token range of the KbT fragments (KC > C): lanes of
  // k-groups C/8 .. 3 in each fragment.
  if (KC > C) {
    for (int idx = tid; idx < NDT * 64; idx += 256) {
      const int rt = idx / 64, ln = idx % 64;
      if ((ln >> 4) >= C / 8) {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        gst_pfrag8(M{}, blk + LY::kKb + (size_t)rt * NKC * LY::PF, ln, z);
      }
    }
  }
  __syncthreads();

  // ---- step 2: Grams A and P ----
  float* As = reinterpret_cast<float*>(smem + L::oA);
  float* Ps = reinterpret_cast<float*>(smem + L::oP);
  constexpr int NTILE = NRT * (NRT + 1) / 2;
  f32x4 accA[(NTILE + 3) / 4], accP[(NTILE + 3) / 4];
  if (fast) {
#pragma unroll
    for (int s = 0; s < (NTILE + 3) / 4; ++s) {
      const int t = w + 4 * s;
      accA[s] = f32x4{0, 0, 0, 0};
      accP[s] = f32x4{0, 0, 0, 0};
      if (t < NTILE) {
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= t) ++a;
        const int b = t - a * (a + 1) / 2;
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
          const auto kh = Kh.pfrag(SD, 16 * b, 32 * kb);
          accP[s] = mma_pp(Qt.pfrag(SD, 16 * a, 32 * kb), kh, accP[s]);
          accA[s] = mma_pp(Kt.pfrag(SD, 16 * a, 32 * kb), kh, accA[s]);
        }
      }
    }
  } else {
    // Exact pairwise evaluation for strong decay.  Thread tid handles rows
    // r = tid / 4 and columns i = tid % 4, +4, ... <= r.
    const float* Gs = reinterpret_cast<const float*>(smem + L::oG);
#pragma unroll
    for (int s = 0; s < (NTILE + 3) / 4; ++s) { accA[s] = f32x4{0, 0, 0, 0}; accP[s] = accA[s]; }
    for (int idx = tid; idx < C * KC; idx += 256) {
      As[(idx / KC) * SF + idx % KC] = 0.f;
      Ps[(idx / KC) * SF + idx % KC] = 0.f;
    }
    __syncthreads();
    for (int r = tid / 4; r < C; r += 64) {
      if (r >= len) continue;
      for (int i = tid % 4; i <= r; i += 4) {
        float sa = 0.f, sp = 0.f;
        for (int c = 0; c < D; ++c) {
          const float kr = (float)kg[((size_t)(t0 + r) * H + h) * D + c];
          const float ki = (float)kg[((size_t)(t0 + i) * H + h) * D + c];
          const float qr = (float)qg[((size_t)(t0 + r) * H + h) * D + c];
          const float ex = __expf(Gs[r * L::SG + c] - Gs[i * L::SG + c]);
          sa += kr * ki * ex;
          sp += qr * ki * ex;
        }
        if (i < r) As[r * SF + i] = beta_s[r] * sa;
        Ps[r * SF + i] = sp;
      }
    }
  }
  __syncthreads();  // Grams done reading Qt/Kt/Kh; As/Ps may overwrite them
  if (fast) {
    // zero everything, then scatter the lower tiles
    for (int idx = tid; idx < C * KC; idx += 256) {
      As[(idx / KC) * SF + idx % KC] = 0.f;
      Ps[(idx / KC) * SF + idx % KC] = 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < (NTILE + 3) / 4; ++s) {
      const int t = w + 4 * s;
      if (t < NTILE) {
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= t) ++a;
        const int b = t - a * (a + 1) / 2;
        const int i = 16 * b + (l & 15);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 16 * a + 4 * (l >> 4) + x;
          if (i < r) As[r * SF + i] = beta_s[r] * accA[s][x];
          if (i <= r) Ps[r * SF + i] = accP[s][x];
        }
      }
    }
  }
  __syncthreads();

  // ---- step 3: X = (I + A)^{-1} by blocked forward substitution ----
  float* Xs = reinterpret_cast<float*>(smem + L::oX);
  float* Ysc = reinterpret_cast<float*>(smem + L::oY);
  for (int idx = tid; idx < C * KC; idx += 256) Xs[(idx / KC) * SF + idx % KC] = 0.f;
  __syncthreads();
  if (w == 0) {
    // diagonal 16x16 blocks: lane = 16*blk + column
    const int bk = l >> 4, j = l & 15;
    if (bk < NRT) {
      float x[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) x[s] = (s == j) ? 1.f : 0.f;
      const float* Ab = As + (16 * bk) * SF + 16 * bk;
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int s = r + 1; s < 16; ++s) x[s] -= Ab[s * SF + r] * x[r];
#pragma unroll
      for (int s = 0; s < 16; ++s) Xs[(16 * bk + s) * SF + 16 * bk + j] = x[s];
    }
  }
  __syncthreads();
  // off-diagonal blocks, one level (a - b) at a time
#pragma unroll
  for (int lev = 1; lev < NRT; ++lev) {
    const int a = lev + w, b = w;
    const bool mine = (w < NRT - lev);
    if (mine) {
      f32x4 y = {0, 0, 0, 0};
      for (int m = b; m < a; ++m)
        y = prod16(M{}, y, As, SF, 16 * a, 16 * m, Xs, SF, 16 * m, 16 * b);
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

  // ---- step 4: W = T (K * gam), T = X Diag(beta); write P, T, W ----
  // T and P fragments: (row tile rt, token block kb), lane (row, k-group).
  for (int f = w; f < NRT * NKC; f += 4) {
    const int rt = f / NKC, kb = f % NKC;
    const int r = 16 * rt + (l & 15), i0 = 32 * kb + 8 * (l >> 4);
    float tv[8], pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tv[e] = Xs[r * SF + i0 + e] * beta_s[i0 + e];
      pv[e] = Ps[r * SF + i0 + e];
    }
    gst_pfrag8(M{}, blk + LY::kT + (size_t)f * LY::PF, l, tv);
    gst_pfrag8(M{}, blk + LY::kP + (size_t)f * LY::PF, l, pv);
  }
  float* Ws = reinterpret_cast<float*>(smem + L::oWs);
  for (int t = w; t < NRT * NDT; t += 4) {
    const int rt = t / NDT, ct = t % NDT;
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      if (32 * kb > 16 * rt + 15) break;
      const int r = 16 * rt + (l & 15), i0 = 32 * kb + 8 * (l >> 4);
      float tv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = Xs[r * SF + i0 + e] * beta_s[i0 + e];
      acc = mma_pp(make_pfrag(M{}, tv), KtT.pfrag(SK, 16 * ct, 32 * kb), acc);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) Ws[(16 * rt + 4 * (l >> 4) + x) * SD + 16 * ct + (l & 15)] = acc[x];
  }
  __syncthreads();
  for (int f = w; f < NRT * NKD; f += 4) {
    const int rt = f / NKD, kb = f % NKD;
    const float* src = Ws + (16 * rt + (l & 15)) * SD + 32 * kb + 8 * (l >> 4);
    gst_pfrag8(M{}, blk + LY::kW + (size_t)f * LY::PF, l, src);
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel: one workgroup per (sequence, head, 16 value columns).
// ---------------------------------------------------------------------------
template <class M, int D, int C>
struct ChunkFrags {
  typedef Layout<M, D, C> LY;
  static constexpr int NST = LY::NDT / 4 > 0 ? LY::NDT / 4 : 1;  // state tiles per wave
  typename M::PFrag W[LY::NKD];
  typename M::PFrag Tm[LY::NKC];
  typename M::PFrag Qt[LY::NKD];
  typename M::PFrag P[LY::NKC];
  typename M::PFrag Kb[NST][LY::NKC];
  float gam[NST][4];
};

template <class M, int D, int C>
__device__ __forceinline__ void load_chunk_frags(ChunkFrags<M, D, C>& f, const char* blk, int w) {
  typedef Layout<M, D, C> LY;
  constexpr int NST = ChunkFrags<M, D, C>::NST;
  const int l = lane_id();
  if (w < LY::NRT) {
    const int rt = w;
#pragma unroll
    for (int kb = 0; kb < LY::NKD; ++kb) {
      f.W[kb] = ld_pfrag(M{}, blk + LY::kW + (size_t)(rt * LY::NKD + kb) * LY::PF);
      f.Qt[kb] = ld_pfrag(M{}, blk + LY::kQt + (size_t)(rt * LY::NKD + kb) * LY::PF);
    }
#pragma unroll
    for (int kb = 0; kb < LY::NKC; ++kb) {
      f.Tm[kb] = ld_pfrag(M{}, blk + LY::kT + (size_t)(rt * LY::NKC + kb) * LY::PF);
      f.P[kb] = ld_pfrag(M{}, blk + LY::kP + (size_t)(rt * LY::NKC + kb) * LY::PF);
    }
  }
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int st = w * NST + s;
    if (st < LY::NDT) {
#pragma unroll
      for (int kb = 0; kb < LY::NKC; ++kb)
        f.Kb[s][kb] = ld_pfrag(M{}, blk + LY::kKb + (size_t)(st * LY::NKC + kb) * LY::PF);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(
          reinterpret_cast<const float*>(blk + LY::kGam) + 16 * st + 4 * (l >> 4));
#pragma unroll
      for (int x = 0; x < 4; ++x) f.gam[s][x] = gv[x];
    }
  }
}

template <class M, int D, int C>
struct InterLds {
  typedef typename M::in_t plain_t;
  static constexpr int KC = Layout<M, D, C>::KC;
  static constexpr int SD = D + kPad;
  static constexpr int SK = KC + kPad;
  static constexpr size_t kSTplain = (size_t)16 * SD * sizeof(plain_t);
  static constexpr size_t kUTplain = (size_t)16 * SK * sizeof(plain_t);
  static constexpr size_t oST = 0;
  static constexpr size_t oUT = oST + (M::kSplit ? 2 : 1) * kSTplain;
  static constexpr size_t oVT = oUT + (M::kSplit ? 2 : 1) * kUTplain;
  static constexpr size_t kTotal = oVT + kUTplain;
};

template <class M, int D, int C, bool OUT_BF16>
__global__ __launch_bounds__(256) void inter_chunk_kernel(KernelPtrs kp, SeqInfo si, int num_pairs) {
  typedef typename M::in_t in_t;
  typedef Layout<M, D, C> LY;
  typedef InterLds<M, D, C> L;
  typedef typename L::plain_t plain_t;
  constexpr int NRT = LY::NRT, KC = LY::KC, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int NST = ChunkFrags<M, D, C>::NST;
  constexpr int NVB = D / 16;
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

  int bos, eos;
  seq_bounds(si, n, bos, eos);
  const int cid0 = si.cu ? clampi(si.chunk_off[n], 0, si.total_chunks)
                         : n * chunks_of<C>(si.seq_len);
  // Never walk past the chunks the workspace was sized for.
  const int nch = min(chunks_of<C>(eos - bos), si.total_chunks - cid0);

  LdsPrecise<M> ST(smem + L::oST, L::kSTplain);
  LdsPrecise<M> UT(smem + L::oUT, L::kUTplain);
  plain_t* VT = reinterpret_cast<plain_t*>(smem + L::oVT);

  // ---- state block in accumulator layout: tile st rows 16st.., cols 16vb.. ----
  f32x4 S[NST];
  const size_t sbase = ((size_t)n * H + h) * D * D;
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int st = w * NST + s;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int c = 16 * st + 4 * (l >> 4) + x;
      S[s][x] = (kp.s0 && st < NDT) ? kp.s0[sbase + (size_t)c * D + 16 * vb + (l & 15)] : 0.f;
    }
  }
  auto write_state_lds = [&]() {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (st < NDT) {
#pragma unroll
        for (int x = 0; x < 4; ++x) ST.store((l & 15) * SD + 16 * st + 4 * (l >> 4) + x, S[s][x]);
      }
    }
  };
  write_state_lds();

  // V tile loader: thread -> (token i, 4 columns)
  const in_t* vg = reinterpret_cast<const in_t*>(kp.v);
  const int vi = tid >> 2, vj = 4 * (tid & 3);
  float vreg[4];
  auto load_v = [&](int ci) {
    const int t0 = bos + ci * C;
    const int len = eos - t0;
#pragma unroll
    for (int e = 0; e < 4; ++e) vreg[e] = 0.f;
    if (vi < C && vi < len) {
      const in_t* p = vg + ((size_t)(t0 + vi) * H + h) * D + 16 * vb + vj;
#pragma unroll
      for (int e = 0; e < 4; ++e) vreg[e] = (float)p[e];
    }
  };
  auto store_v = [&]() {
    if (vi < KC) {
#pragma unroll
      for (int e = 0; e < 4; ++e) VT[(vj + e) * SK + vi] = (plain_t)vreg[e];
    }
  };
  // Zero the padded token columns of VT and UT once (KC > C).
  if (KC > C) {
    for (int idx = tid; idx < 16 * (KC - C); idx += 256) {
      const int j = idx / (KC - C), i = C + idx % (KC - C);
      VT[j * SK + i] = (plain_t)0.f;
      UT.store(j * SK + i, 0.f);
    }
  }

  ChunkFrags<M, D, C> cur, nxt;
  if (nch > 0) {
    load_chunk_frags<M, D, C>(cur, kp.ops + ((size_t)cid0 * H + h) * LY::kBytes, w);
    load_v(0);
  }
  for (int ci = 0; ci < nch; ++ci) {
    const int t0 = bos + ci * C;
    const int len = eos - t0 < C ? eos - t0 : C;
    store_v();
    __syncthreads();  // VT and ST ready
    if (ci + 1 < nch) {
      load_chunk_frags<M, D, C>(nxt, kp.ops + ((size_t)(cid0 + ci + 1) * H + h) * LY::kBytes, w);
      load_v(ci + 1);
    }
    f32x4 qs = {0, 0, 0, 0};
    if (w < NRT) {
      f32x4 ws = {0, 0, 0, 0}, u = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        const auto sf = ST.pfrag(SD, 0, 32 * kb);
        ws = mma_pp(cur.W[kb], sf, ws);
        qs = mma_pp(cur.Qt[kb], sf, qs);
      }
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) u = mma_pf(cur.Tm[kb], lds_frag(M{}, VT, SK, 0, 32 * kb), u);
#pragma unroll
      for (int x = 0; x < 4; ++x) UT.store((l & 15) * SK + 16 * w + 4 * (l >> 4) + x, u[x] - ws[x]);
    }
    __syncthreads();  // UT ready; ST/VT reads done
    if (w < NRT) {
      f32x4 o = qs;
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        if (32 * kb > 16 * w + 15) break;
        o = mma_pp(cur.P[kb], UT.pfrag(SK, 0, 32 * kb), o);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 16 * w + 4 * (l >> 4) + x;
        if (r < len) {
          const size_t oi = ((size_t)(t0 + r) * H + h) * D + 16 * vb + (l & 15);
          if constexpr (OUT_BF16)
            reinterpret_cast<bf16*>(kp.o)[oi] = f2bf(o[x]);
          else
            reinterpret_cast<float*>(kp.o)[oi] = o[x];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (st < NDT) {
#pragma unroll
        for (int x = 0; x < 4; ++x) S[s][x] *= cur.gam[s][x];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) S[s] = mma_pp(cur.Kb[s][kb], UT.pfrag(SK, 0, 32 * kb), S[s]);
      }
    }
    // ST is read again only after the next iteration's first barrier, and
    // every read of this chunk's ST/VT happened before the second barrier.
    write_state_lds();
    if (ci + 1 < nch) cur = nxt;
  }
  if (kp.s1) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
      if (st < NDT) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = 16 * st + 4 * (l >> 4) + x;
          kp.s1[sbase + (size_t)c * D + 16 * vb + (l & 15)] = S[s][x];
        }
      }
    }
  }
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
    hipLaunchKernelGGL((intra_chunk_kernel<M, D, C>), dim3(a.total_chunks, a.H), dim3(256), lds,
                       a.stream, kp, si);
  }
  const int pairs = a.num_seqs * a.H;
  const int nvb = D / 16;
  const int blocks = ((pairs + 7) / 8) * 8 * nvb;
  if (a.out_bf16)
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, true>), dim3(blocks), dim3(256), 0, a.stream, kp,
                       si, pairs);
  else
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, false>), dim3(blocks), dim3(256), 0, a.stream, kp,
                       si, pairs);
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
