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
//                      the UT-transform solve, W and U0.  It writes Q*gam, W,
//                      (K*exp(Gamma_n-Gamma))^T, P, U0 and gam_n to the
//                      workspace, already in the layouts the MFMA products
//                      of the inter-chunk pass consume.
//  inter_chunk_kernel  one workgroup per (sequence, head, 16 value columns):
//                      the serial loop over the sequence's chunks, with the
//                      state block held in MFMA accumulator registers.
//
// Decay factorisation (secondary chunking; greeksharifa.github.io summary,
// section 3.2 "Efficiency Analysis").  The Grams need exp(Gamma_r -
// Gamma_i) for i <= r.  The chunk is cut into 16-row tiles; for rows r of
// tile a and columns i of tile b <= a the factor is split as
//   exp(Gamma_r - Gamma_s) * exp(Gamma_s - Gamma_e) * exp(Gamma_e - Gamma_i)
// with s the row before tile a and e the last row of tile b: the row operand
// (tile-local decay of row r), a per-channel factor of the block, and the
// column operand (decay from row i to the end of its tile).  Off the
// diagonal (b < a, so s >= e) all three are <= 1: a factor that underflows
// belongs to a term below exp(-87).  On the diagonal the middle factor is
// exp(span of tile a) >= 1; a tile whose span on some channel exceeds
// kTileSpanLimit has its diagonal block evaluated pair by pair with the
// exact exponent of each difference instead.  Every block runs on MFMA.
//
// Most chunks need none of this: while no channel decays by more than
// exp(-kChunkSpanLimit) over the whole chunk, one factorisation per chunk
// (rows exp(Gamma_r) <= 1, columns exp(-Gamma_i) <= exp(kChunkSpanLimit)) is
// exact to rounding and needs no per-block factors.  So the intra pass runs
// twice per segment: the chunk-wide pass (TILE = false) handles those
// chunks and only flags the others in their block; the tile pass (TILE =
// true) exits at once for unflagged blocks.  The two code paths live in two
// kernels so that the common one keeps its registers (as one kernel, the
// tile path's values spilled in both).
#include "kda_device.hpp"
#include "kda_launch.hpp"

#include <stdint.h>

namespace kda {

constexpr float kTileSpanLimit = 64.f;  // largest tile span on the diagonal's product path
constexpr float kChunkSpanLimit = 40.f;  // largest chunk span of the chunk-wide factoring
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
  // U0 = T V, fp32 [C x D] as 16x16 accumulator tiles (row tile, column
  // tile): lane l holds rows 4(l>>4)..+3 of column l&15, 16 B per lane.
  static constexpr size_t kU0 = kP + (size_t)NRT * NKC * PF;
  static constexpr size_t kGam = kU0 + (size_t)NRT * NDT * 1024;      // fp32 [D]
  // int: 1 when the chunk's decay needs tile-local factors (set by the
  // chunk-wide intra pass, which then leaves the block to the tile pass)
  static constexpr size_t kFlag = kGam + (size_t)D * 4;
  static constexpr size_t kBytes = ((kFlag + 4) + 255) / 256 * 256;
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

// The prefill runs in segments: segment s covers the local chunks
// [s L, (s + 1) L) of every sequence (chunk 0 starts at the sequence's first
// token), so all sequences advance together.  A segment is the intra-chunk
// pass over its chunks, then the inter-chunk pass, which carries each
// sequence's state into the next segment.  The workspace holds one segment's
// operands, so it stays bounded for long inputs, and a segment's operands are
// read back soon after they are written, while the 256 MB Infinity Cache
// still holds them.  That pays when the inter-chunk pass is latency-bound,
// with at most 512 workgroups (two per CU): then the budget is 160 MiB.  With
// more (sequence, head) pairs the pass is throughput-bound, extra segments
// only add start-up and tail time, and the budget is 8 GiB, which only bounds
// the workspace.  L is the largest length (at least 16 chunks, to amortise
// the passes' start-up) whose operands fit the budget, then evened out over
// the segments.  The caller's tuning may fix the budget or L instead; with a
// workspace cap, L is the largest length (any, down to one chunk) whose whole
// workspace fits the cap.
static size_t segment_budget_bytes(long long inter_workgroups, const PrefillTuning& t) {
  if (t.segment_bytes >= 1) return t.segment_bytes;
  return inter_workgroups <= 512 ? (size_t)160 << 20 : (size_t)8 << 30;
}

namespace {
struct SeqCounts {  // chunk counts of the sequences, on the host
  int num_seqs;
  const int32_t* cu;  // host cu_seqlens or nullptr
  int seq_len, C;
  int nch(int n) const {
    const long long len = cu ? (long long)cu[n + 1] - cu[n] : seq_len;
    return (int)((len + C - 1) / C);
  }
  // chunk slots of the segment that starts at local chunk c0
  long long slots(int c0, int L) const {
    long long t = 0;
    for (int n = 0; n < num_seqs; ++n) {
      const int c = nch(n) - c0;
      t += c <= 0 ? 0 : (c < L ? c : L);
    }
    return t;
  }
};
}  // namespace

// The slot table exists for varlen input only.
static size_t table_bytes(int num_seqs, bool varlen) {
  return varlen ? align256(sizeof(int32_t) * (size_t)(num_seqs + 1)) : 0;
}

static size_t carry_bytes(const SegmentPlan& p, int num_seqs, int H, int D) {
  return p.nseg > 1 ? align256((size_t)num_seqs * H * D * D * sizeof(float)) : 0;
}

// Raw o of one segment for the layer epilogue: fp32 [slot][H][C][D].
static size_t raw_o_bytes(const SegmentPlan& p, int H, int D, int chunk, bool epilogue) {
  return epilogue ? align256((size_t)p.max_slots * H * chunk * D * sizeof(float)) : 0;
}

// With the layer epilogue and several segments, segment s's epilogue runs in
// segment s + 1's chunk-wide launch, after the slot table of s + 1 is made:
// the varlen slot tables of consecutive segments then alternate between two
// copies.
static int table_copies(const SegmentPlan& p, bool epilogue) { return epilogue && p.nseg > 1 ? 2 : 1; }

static size_t plan_bytes(const SegmentPlan& p, int num_seqs, bool varlen, int H, int D, int chunk,
                         bool in_bf16, bool epilogue) {
  return table_copies(p, epilogue) * table_bytes(num_seqs, varlen) + carry_bytes(p, num_seqs, H, D) +
         (size_t)p.max_slots * H * prefill_chunk_bytes(D, chunk, in_bf16) +
         raw_o_bytes(p, H, D, chunk, epilogue);
}

SegmentPlan plan_segments(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D,
                          int chunk, bool in_bf16, bool epilogue, const PrefillTuning& tuning) {
  const SeqCounts sc{num_seqs, cu_host, seq_len, chunk};
  int max_nch = 0;
  for (int n = 0; n < num_seqs; ++n) max_nch = max_nch > sc.nch(n) ? max_nch : sc.nch(n);
  SegmentPlan p;
  if (max_nch == 0) {  // one pass of the inter kernel settles the states
    if (tuning.workspace_cap &&
        plan_bytes(p, num_seqs, cu_host != nullptr, H, D, chunk, in_bf16, epilogue) >
            tuning.workspace_cap)
      p.nseg = 0;
    return p;
  }
  auto make = [&](int L) {
    SegmentPlan q;
    q.nseg = (max_nch + L - 1) / L;
    q.L = (max_nch + q.nseg - 1) / q.nseg;
    q.max_slots = (int)sc.slots(0, q.L);
    return q;
  };
  const size_t per = (size_t)H * prefill_chunk_bytes(D, chunk, in_bf16);
  int lo;
  if (tuning.segment_chunks >= 1) {
    lo = tuning.segment_chunks < max_nch ? tuning.segment_chunks : max_nch;
  } else {
    // inter-chunk workgroups at 16 value columns each
    const size_t budget = segment_budget_bytes((long long)num_seqs * H * (D / 16), tuning);
    lo = max_nch < 16 ? max_nch : 16;
    int hi = max_nch;
    if ((size_t)sc.slots(0, lo) * per <= budget) {
      while (lo < hi) {  // largest L that fits (slots grow with L)
        const int mid = lo + (hi - lo + 1) / 2;
        if ((size_t)sc.slots(0, mid) * per <= budget)
          lo = mid;
        else
          hi = mid - 1;
      }
    }
  }
  p = make(lo);
  if (tuning.workspace_cap) {
    auto fits = [&](int L) {
      return plan_bytes(make(L), num_seqs, cu_host != nullptr, H, D, chunk, in_bf16, epilogue) <=
             tuning.workspace_cap;
    };
    if (!fits(lo)) {
      // The whole workspace of L = 1..lo grows with L (more slots, and the
      // carry buffer once there are two segments): take the largest that fits.
      int a = 1, b = lo;
      if (!fits(1)) {
        p.L = 0;
        p.nseg = 0;
        p.max_slots = 0;
        return p;
      }
      while (a < b) {
        const int mid = a + (b - a + 1) / 2;
        if (fits(mid))
          a = mid;
        else
          b = mid - 1;
      }
      p = make(a);
    }
  }
  return p;
}

size_t prefill_workspace_bytes(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D,
                               int chunk, bool in_bf16, bool epilogue,
                               const PrefillTuning& tuning) {
  const SegmentPlan p =
      plan_segments(num_seqs, cu_host, seq_len, H, D, chunk, in_bf16, epilogue, tuning);
  if (p.nseg == 0) return SIZE_MAX;
  return plan_bytes(p, num_seqs, cu_host != nullptr, H, D, chunk, in_bf16, epilogue);
}

// ---------------------------------------------------------------------------
// Sequence geometry shared by both kernels
// ---------------------------------------------------------------------------
struct SeqInfo {
  const int32_t* cu;        // device cu_seqlens or nullptr
  const int32_t* slot_off;  // varlen: [num_seqs + 1] first workspace slot of each sequence
  int num_seqs, seq_len, total_tokens;
  int c0, L;                // this segment: local chunks [c0, c0 + L) of every sequence
  int slot_cnt;             // fixed length: slots of each sequence in this segment
  int max_slots;            // workspace capacity, in (chunk, all heads) slots
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

// Varlen segment table: slot_off[n] = sum over m < n of the number of local
// chunks of sequence m in [c0, c0 + L); slot_off[N] is the segment's total.
// One workgroup; thread t handles a contiguous run of sequences.
__global__ __launch_bounds__(1024) void segment_table_kernel(const int32_t* __restrict__ cu,
                                                             int32_t* __restrict__ slot_off,
                                                             int num_seqs, int total_tokens, int C,
                                                             int c0, int L) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (num_seqs + 1023) / 1024;
  const int n0 = t * per, n1 = min(num_seqs, n0 + per);
  auto count = [&](int n) {
    const int b = clampi(cu[n], 0, total_tokens), e = clampi(cu[n + 1], b, total_tokens);
    return clampi((e - b + C - 1) / C - c0, 0, L);
  };
  int acc = 0;
  for (int n = n0; n < n1; ++n) acc += count(n);
  part[t] = acc;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int off = part[t] - acc;
  for (int n = n0; n < n1; ++n) {
    slot_off[n] = off;
    off += count(n);
  }
  if (t == 1023) slot_off[num_seqs] = part[1023];
}

// ---------------------------------------------------------------------------
// Block forward substitution on 16x16 tiles.  A chain operand is a 16x16
// block in the A-operand layout of the 16x16x16 products: lane l holds
// A[l & 15][4 (l >> 4) + e], e = 0..3, kept in LDS as 16 B per lane (split
// hi + lo for bf16, fp32 otherwise).  The right operand is an accumulator
// tile itself (lane l holds Y[4 (l >> 4) + i][l & 15]), which is exactly the
// B-operand layout of those products, so a chain of them never moves data
// between lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void cfrag_store(ModeBF16, char* p, const float* x) {
  bf16x4 h, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f2bf(x[e]);
    lo[e] = f2bf(x[e] - bf2f(h[e]));
  }
  bf16x4* q = reinterpret_cast<bf16x4*>(p + 16 * lane_id());
  q[0] = h;
  q[1] = lo;
}
__device__ __forceinline__ void cfrag_store(ModeF32, char* p, const float* x) {
  *reinterpret_cast<f32x4*>(p + 16 * lane_id()) = f32x4{x[0], x[1], x[2], x[3]};
}
// acc += A Y for a chain operand A at p and an accumulator-layout tile Y.
__device__ __forceinline__ f32x4 chain_mma(ModeBF16, const char* p, f32x4 y, f32x4 acc) {
  const bf16x4* q = reinterpret_cast<const bf16x4*>(p + 16 * lane_id());
  const bf16x4 ah = q[0], al = q[1];
  bf16x4 yh, yl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    yh[e] = f2bf(y[e]);
    yl[e] = f2bf(y[e] - bf2f(yh[e]));
  }
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, yh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, yl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, yh, acc, 0, 0, 0);
}
// fp32: four 16x16x4 products; the s-th takes k = 4 (l >> 4) + s, which is
// element s of both the lane's chain operand and its accumulator.
__device__ __forceinline__ f32x4 chain_mma(ModeF32, const char* p, f32x4 y, f32x4 acc) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 16 * lane_id());
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], y[s], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------------------
// LDS plan of the intra-chunk kernel: two regions that the phases reuse,
//   R0: K-bar^T staging (precise [D x KC])  ->  the Gram column operands
//       (precise, in fragment order)
//       ->  the solve's operands: inverses of the diagonal blocks of I + A
//       (fp32 [NRT][16][17]) and the chain operands (the blocks A_am below
//       the diagonal, then the inverses)
//   R1: A and P (fp32 [C x (KC+1)])  ->  (K*gam)^T staging (precise
//       [D x KC]), overwritten in place by W^T  ->  V^T staging
// plus the per-tile totals of the decay scan, beta, and the layer prologue's
// norm partials and per-token factors.
// ---------------------------------------------------------------------------
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

constexpr int kMaxConv = 4;  // widest short convolution

template <class M, int D, int C>
struct IntraLds {
  typedef typename M::in_t plain_t;  // element of one half of a precise matrix
  static constexpr int KC = Layout<M, D, C>::KC;
  static constexpr int NRT = C / 16;
  static constexpr int NOFF = NRT * (NRT - 1) / 2;  // blocks below the diagonal
  static constexpr int SK = KC + kPad;  // row stride of [D x KC] staging
  static constexpr int SF = KC + 1;     // row stride of fp32 [C x KC] matrices
  static constexpr size_t kStPlain = ((size_t)D * SK * sizeof(plain_t) + 15) / 16 * 16;
  static constexpr size_t kStPrecise = M::kSplit ? 2 * kStPlain : kStPlain;
  static constexpr size_t kKhFrags = (size_t)NRT * (D / 32) * M::kPFragBytes;
  static constexpr size_t kFMat = ((size_t)C * SF * 4 + 15) / 16 * 16;
  static constexpr size_t kXD = ((size_t)NRT * 16 * 17 * 4 + 15) / 16 * 16;
  static constexpr size_t kSolve = kXD + (size_t)(NOFF + NRT) * 1024;
  static constexpr size_t kR0 = cmax(cmax(kStPrecise, kKhFrags), kSolve);
  static constexpr size_t kR1 = cmax(2 * kFMat, kStPrecise);
  static constexpr size_t oR0 = 0, oR1 = kR0;
  static constexpr size_t oTot = kR0 + kR1;              // fp32 [NRT][D]
  static constexpr size_t oBeta = oTot + (size_t)NRT * D * 4;
  static constexpr size_t oNrm = oBeta + (size_t)KC * 4;      // fp32 [8 waves][16][2]
  static constexpr size_t kTotal = oNrm + 8 * 16 * 2 * 4;
  // With the convolution: v's weights, [D][kMaxConv] fp32, taps from the
  // current row back (q's and k's sit in R0 while the prologue runs).
  static constexpr size_t oCWv = kTotal;
  static constexpr size_t kTotalConv = oCWv + (size_t)D * kMaxConv * 4;
  // offsets inside the regions
  static constexpr size_t oKbS = oR0;                    // staging
  static constexpr size_t oKh = oR0;                      // Gram column operands
  static constexpr size_t oA = oR1, oP = oR1 + kFMat;    // Grams
  static constexpr size_t oXD = oR0, oCF = oR0 + kXD;    // solve
  static constexpr size_t oKtT = oR1;                    // W
  static constexpr size_t oVT = oR1;                     // U0 (after W)
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
  // element e of a lane's precise fragment, already split
  __device__ void put(int idx, const ModeBF16::PFrag& f, int e) {
    hi[idx] = f.hi[e];
    lo[idx] = f.lo[e];
  }
  __device__ float get(int idx) const { return bf2f(hi[idx]) + bf2f(lo[idx]); }
  // four consecutive elements starting at idx (a multiple of 4)
  __device__ void get4(int idx, float* x) const {
    const bf16x4 h = *reinterpret_cast<const bf16x4*>(hi + idx);
    const bf16x4 l = *reinterpret_cast<const bf16x4*>(lo + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = bf2f(h[e]) + bf2f(l[e]);
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
  __device__ void put(int idx, const ModeF32::PFrag& f, int e) { v[idx] = f.v[e]; }
  __device__ float get(int idx) const { return v[idx]; }
  __device__ void get4(int idx, float* x) const {
    const f32x4 t = *reinterpret_cast<const f32x4*>(v + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = t[e];
  }
};

// The eight values of a lane's precise fragment.
__device__ __forceinline__ void pfrag_values(const ModeBF16::PFrag& f, float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = bf2f(f.hi[e]) + bf2f(f.lo[e]);
}
__device__ __forceinline__ void pfrag_values(const ModeF32::PFrag& f, float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = f.v[e];
}

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
  float* carry;    // [num_seqs, H, D, D] state between segments, or nullptr
  char* ops;       // per-(chunk, head) operand blocks of the current segment
  float* o_slots;  // with the layer epilogue: raw o, fp32 [slot][H][C][D]; else nullptr
  const void* gate;          // layer epilogue: sigmoid gate [tokens, H, D] (in dtype)
  const float* norm_weight;  // layer epilogue: RMSNorm weight [D]
  float norm_eps;
  const float* cw[3];  // short convolution of q, k, v: weights [H][D][conv_w]
  const void* cs[3];   // their carried inputs [num_seqs][H][conv_w - 1][D] (in dtype), or nullptr
  int conv_w;          // convolution width (1..4) when the prologue convolves
  int H;
};

// Layer prologue pieces (the "Kimi Linear" notes, docsaid.org, section
// "Other Components"): Swish of the projected q, k, v; sigmoid of beta.
// The reciprocal is the hardware's (about 1 ulp), not a correctly rounded
// division: both stay within a few fp32 ulp, and large |x| give the limits
// (x or 0, 1 or 0) since 1 / inf is 0.
__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float swishf(float x) { return x * sigmoidf(x); }
constexpr float kL2Floor = 1e-12f;  // L2 norms below this count as this

// Eight input elements of one row held as loaded (bf16 or fp32).
template <class T>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 v;
  __device__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ void zero() { v = bf16x8{}; }
  __device__ float get(int e) const { return bf2f(v[e]); }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ void zero() { a = b = f32x4{0, 0, 0, 0}; }
  __device__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Precise fragment in LDS, stored as in global memory (hi: lane*16 B, lo:
// 1024 + lane*16 B for bf16; lane*32 B for fp32).
__device__ __forceinline__ void lds_st_pfrag(ModeBF16 m, char* p, const ModeBF16::PFrag& f) { st_pfrag(m, p, f); }
__device__ __forceinline__ void lds_st_pfrag(ModeF32 m, char* p, const ModeF32::PFrag& f) { st_pfrag(m, p, f); }

// One (slot, head) item of a segment: its token range and operand block.
// item = slot * H + head; slot indexes the segment's (sequence, local chunk)
// pairs (varlen: through the segment table).
struct Item {
  int h, t0, len;
  int n, bos;  // sequence and its first token
  char* blk;
};

template <int C>
__device__ __forceinline__ Item intra_item(const SeqInfo& si, const KernelPtrs& kp, int item,
                                           size_t block_bytes) {
  const int H = kp.H;
  const int slot = item / H;
  Item x;
  x.h = item - slot * H;
  int n, ci;
  if (si.cu) {
    int lo = 0, hi = si.num_seqs - 1;  // last n with slot_off[n] <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (si.slot_off[mid] <= slot)
        lo = mid;
      else
        hi = mid - 1;
    }
    n = lo;
    ci = si.c0 + (slot - si.slot_off[n]);
  } else {
    n = clampi(slot / si.slot_cnt, 0, si.num_seqs - 1);
    ci = si.c0 + slot % si.slot_cnt;
  }
  int bos, eos;
  seq_bounds(si, n, bos, eos);
  x.n = n;
  x.bos = bos;
  // A device table that disagrees with the host one can only shorten chunks,
  // never move them outside [bos, eos].
  const long long t0l = (long long)bos + (long long)(ci < 0 ? 0 : ci) * C;
  x.t0 = (int)(t0l < eos ? t0l : eos);
  x.len = clampi(eos - x.t0, 0, C);
  x.blk = kp.ops + ((size_t)slot * H + x.h) * block_bytes;
  return x;
}

// ---------------------------------------------------------------------------
// Short convolution of the layer prologue (the "Kimi Linear" notes,
// docsaid.org, section "Other Components": q, k and v pass through a short
// convolution before Swish).  Causal and depthwise: for token t of a sequence
// starting at bos, y_c = sum_{i<W} w[c][i] x_c(t - (W-1) + i), where inputs
// before bos come from the carried state (row (W-1) + (s - bos)), or are zero.
// ---------------------------------------------------------------------------

// The inputs one lane needs besides its own token row r = 16 rt + lr: lanes
// lr >= 16 - (kMaxConv - 1) load the rows 16 rt - 3 .. 16 rt - 1 of the chunk
// (earlier tokens of the sequence, or state rows before its start).
template <class T, int D>
__device__ __forceinline__ void load_halo(Raw8<T>& ext, const KernelPtrs& kp, int x, const Item& it,
                                          int rt, int lr, int c0, int total_tokens) {
  ext.zero();
  if (lr < 16 - (kMaxConv - 1)) return;
  const int W = kp.conv_w, H = kp.H;
  const int te = it.t0 + 16 * rt + lr - 16;
  const T* src = x == 0 ? (const T*)kp.q : x == 1 ? (const T*)kp.k : (const T*)kp.v;
  if (te >= it.bos) {
    ext.load(src + ((size_t)clampi(te, 0, total_tokens - 1) * H + it.h) * D + c0);
  } else {
    const int j = (W - 1) + (te - it.bos);
    if (j >= 0 && kp.cs[x])
      ext.load(reinterpret_cast<const T*>(kp.cs[x]) + (((size_t)it.n * H + it.h) * (W - 1) + j) * D + c0);
  }
}

// Rotate a value right by N lanes within each 16-lane row (DPP row_ror):
// lane lr receives the value of lane (lr - N) mod 16 of its row.
// Every lane has a source, so no old value is needed.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF,
                                                            true));
}

// Shift a value right by N lanes within each 16-lane row (DPP row_shr): lane
// lr receives the value of lane lr - N, lanes lr < N receive 0.  Every lane
// of the wave must execute it.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x110 + N, 0xF, 0xF, false));
}

// Exchange with the lane whose index differs in bit 0 (X = 1) or bit 1
// (X = 2), by a DPP quad permutation.  Every lane of the wave must execute it.
template <int X>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl,
                                                               0xF, 0xF, false));
}

// 4x4 transpose within each quad of lanes: if lane j of the quad holds
// a[i] = M[i][j], lane r ends with M[r][0..3].  Two butterfly rounds: the
// off-diagonal 2x2 blocks swap between lanes r and r^2, then the elements
// of each 2x2 block between lanes r and r^1.  Every lane must execute it.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 a) {
  const int r = lane_id() & 3;
  const bool h2 = (r & 2) != 0, h1 = (r & 1) != 0;
  float w0 = quad_xor<2>(h2 ? a[0] : a[2]), w1 = quad_xor<2>(h2 ? a[1] : a[3]);
  if (h2) { a[0] = w0; a[1] = w1; } else { a[2] = w0; a[3] = w1; }
  w0 = quad_xor<1>(h1 ? a[0] : a[1]);
  w1 = quad_xor<1>(h1 ? a[2] : a[3]);
  if (h1) { a[0] = w0; a[2] = w1; } else { a[1] = w0; a[3] = w1; }
  return a;
}

// Inclusive prefix sum over the 16 lanes of each row.
__device__ __forceinline__ float row_scan16(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}

// Convolved values of one lane's 8 channels (c0 .. c0 + 7) of row 16 rt + lr,
// from the lane's own row and the halo rows of lanes 13..15 of its 16-lane
// group.  w4 holds the channels' weights in LDS, [8][kMaxConv], w4[4e + j]
// the weight of row lr - j.  Tap j needs lane lr - j's own value, or for
// lr < j the halo value of lane lr - j + 16: each source lane s first picks
// its halo value when s >= 16 - j, and one row rotation by j delivers it.
// Full width (the usual case) runs every tap with no test; a narrower width
// skips the taps at or past W, whose rows must not be read (a non-finite
// input there would leak through a zero weight).
template <class T>
__device__ __forceinline__ void conv8(const Raw8<T>& own, const Raw8<T>& ext, const float* w4,
                                      int W, int lr, float out[8]) {
  static_assert(kMaxConv == 4, "three taps before the current row");
  if (W == kMaxConv) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xo = own.get(e), xe = ext.get(e);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w4 + 4 * e);
      float acc = wv[0] * xo;
      acc += wv[1] * row_ror<1>(lr >= 15 ? xe : xo);
      acc += wv[2] * row_ror<2>(lr >= 14 ? xe : xo);
      acc += wv[3] * row_ror<3>(lr >= 13 ? xe : xo);
      out[e] = acc;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xo = own.get(e), xe = ext.get(e);
      float acc = w4[4 * e] * xo;
      if (W > 1) acc += w4[4 * e + 1] * row_ror<1>(lr >= 15 ? xe : xo);
      if (W > 2) acc += w4[4 * e + 2] * row_ror<2>(lr >= 14 ? xe : xo);
      out[e] = acc;
    }
  }
}


// ---------------------------------------------------------------------------
// Intra-chunk kernel: grid (slots of the segment, H), 512 threads (8 waves),
// two workgroups per CU.
//
// Thread layout follows the MFMA fragments: the chunk's [C x D] token-by-
// channel matrices are cut into 16-token x 32-channel fragments; wave w holds
// fragments w, w + 8, ... (row tile f % NRT, channel block f / NRT), lane l
// the eight channels 32 kb + 8 (l >> 4) .. + 7 of token 16 rt + (l & 15).  So
// the decayed Q and K are Gram A-operands in registers, Q*gam goes out as
// whole fragments, and the decay cumsum runs across the 16 lanes of a tile.
// ---------------------------------------------------------------------------
// SDEC: scalar decay (Gated DeltaNet), one log-decay per token and head, g
// [tokens, H]; otherwise one per key channel, g [tokens, H, D].
// SDEC: scalar decay (one g per token and head).  PRO: the layer prologue
// is applied to the inputs as they are read: 1 = Swish + L2 norm of q and k,
// Swish of v, sigmoid of beta; 2 = the same after the short convolution of
// q, k and v.
// The work of one (chunk slot, head) item; smem is the workgroup's dynamic
// LDS.  Every wave of the workgroup calls it for the same item.
template <class M, int D, int C, bool SDEC, int PRO, bool TILE>
__device__ __forceinline__ void intra_item_body(const KernelPtrs& kp, const SeqInfo& si, int item, char* smem) {
  typedef typename M::in_t in_t;
  typedef typename M::PFrag PFrag;
  typedef Layout<M, D, C> LY;
  typedef IntraLds<M, D, C> L;
  typedef typename L::plain_t plain_t;
  constexpr int NRT = LY::NRT, KC = LY::KC, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int SK = L::SK, SF = L::SF;
  constexpr int NW = kIntraThreads / 64;
  constexpr int NFRAG = NRT * NKD;            // fragments of a [C x D] matrix
  constexpr int FPW = (NFRAG + NW - 1) / NW;  // fragments per wave
  static_assert(NW % NRT == 0, "a wave's fragments share one row tile");
  static_assert(NDT <= NW, "one wave per column tile in the solve");

  const int H = kp.H;
  const Item it = intra_item<C>(si, kp, item, LY::kBytes);
  const int h = it.h, t0 = it.t0, len = it.len;
  char* blk = it.blk;
  if constexpr (TILE) {  // only the blocks the chunk-wide pass left
    if (*reinterpret_cast<const int*>(blk + LY::kFlag) == 0) return;
  }
  const int tid = threadIdx.x;
  const int w = wave_id(), l = lane_id();
  const int lr = l & 15, lg = l >> 4;

  float* tot = reinterpret_cast<float*>(smem + L::oTot);
  float* beta_s = reinterpret_cast<float*>(smem + L::oBeta);

  // ---- this wave's fragments (surplus waves repeat the last one, without
  // storing anything: their loads stay unconditional) ----
  bool fv[FPW];
  int fkb[FPW];
  const int rt = (w % NRT);  // row tile shared by every fragment of this wave
  const int r = 16 * rt + lr;
  const bool rv = r < len;
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const int f = w + NW * j;
    fv[j] = f < NFRAG;
    fkb[j] = (f < NFRAG ? f : NFRAG - NRT + rt) / NRT;
  }
  const bool any_frag = fv[0];

  // ---- step 1: loads, all issued up front (rows past the chunk re-read a
  // valid row and are zeroed at use).  With the convolution its weights come
  // first: a wait for them then covers no other load ----
  const int tok = clampi(t0 + (r < len ? r : len - 1), 0, si.total_tokens - 1);
  constexpr int NWT = PRO == 2 ? (3 * D * kMaxConv + kIntraThreads - 1) / kIntraThreads : 1;
  float cwv[NWT];
  if constexpr (PRO == 2) {
    const int W = kp.conv_w;
#pragma unroll
    for (int x = 0; x < NWT; ++x) {
      const int idx = tid + kIntraThreads * x;
      const int t = idx / (D * kMaxConv), c = (idx / kMaxConv) % D, j = idx % kMaxConv;
      // selected, not indexed: a per-lane index into the argument block
      // would load the pointer from memory and wait for it first
      const float* wt = t == 0 ? kp.cw[0] : t == 1 ? kp.cw[1] : kp.cw[2];
      cwv[x] = idx < 3 * D * kMaxConv && j < W ? wt[((size_t)h * D + c) * W + (W - 1 - j)] : 0.f;
    }
  }
  Raw8<float> graw[FPW];
  Raw8<in_t> qraw[FPW], kraw[FPW];
  float gscalar = 0.f;
  if constexpr (SDEC) gscalar = kp.g[(size_t)tok * H + h];
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const size_t base = ((size_t)tok * H + h) * D + 32 * fkb[j] + 8 * lg;
    if constexpr (!SDEC) graw[j].load(kp.g + base);
    qraw[j].load(reinterpret_cast<const in_t*>(kp.q) + base);
    kraw[j].load(reinterpret_cast<const in_t*>(kp.k) + base);
  }
  // beta (the sigmoid of its logit with the prologue) into LDS.  Its store
  // waits for the load, so with the convolution it comes after the halo
  // loads below: issued first, it would hold them back by a round trip.
  auto stage_beta = [&]() {
    if (tid < KC) {
      const int tb = clampi(t0 + (tid < len ? tid : 0), 0, si.total_tokens - 1);
      const float bv = kp.beta[(size_t)tb * H + h];
      beta_s[tid] = tid < len ? (PRO ? sigmoidf(bv) : bv) : 0.f;
    }
  };
  if constexpr (PRO != 2) stage_beta();
  // Layer prologue: Swish of q and k, after their short convolution when
  // PRO == 2.  Where the Gram region (unused until step 4) holds 32 B per
  // lane and fragment, the convolved, activated k waits there instead of in
  // registers.
  constexpr bool kPark = PRO == 2 && (size_t)kIntraThreads * FPW * 32 <= L::kR1;
  float qc[PRO == 2 ? FPW : 1][8], kc_reg[PRO == 2 && !kPark ? FPW : 1][8];
  f32x4* kpark = reinterpret_cast<f32x4*>(smem + L::oR1) + 2 * (64 * (FPW * w) + l);
  if constexpr (PRO == 2) {
    // The head's weights into LDS first (q's and k's in R0, unused until
    // step 3; v's in their own region, used in step 8).
    float* cwq = reinterpret_cast<float*>(smem + L::oR0);
    float* cwk = cwq + D * kMaxConv;
    const int W = kp.conv_w;
    Raw8<in_t> qe[FPW], ke[FPW];
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      load_halo<in_t, D>(qe[j], kp, 0, it, rt, lr, 32 * fkb[j] + 8 * lg, si.total_tokens);
      load_halo<in_t, D>(ke[j], kp, 1, it, rt, lr, 32 * fkb[j] + 8 * lg, si.total_tokens);
    }
    stage_beta();
#pragma unroll
    for (int x = 0; x < NWT; ++x) {
      const int idx = tid + kIntraThreads * x;
      if (idx < 3 * D * kMaxConv) {
        const int t = idx / (D * kMaxConv);
        (t == 0 ? cwq : t == 1 ? cwk : reinterpret_cast<float*>(smem + L::oCWv))[idx % (D * kMaxConv)] = cwv[x];
      }
    }
    __syncthreads();  // weights staged
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      const int c0 = 32 * fkb[j] + 8 * lg;
      float kc[8];
      conv8(qraw[j], qe[j], cwq + c0 * kMaxConv, W, lr, qc[j]);
      conv8(kraw[j], ke[j], cwk + c0 * kMaxConv, W, lr, kc);
#pragma unroll
      for (int e = 0; e < 8; ++e) qc[j][e] = swishf(qc[j][e]);
      if constexpr (kPark) {
        kpark[128 * j] = f32x4{swishf(kc[0]), swishf(kc[1]), swishf(kc[2]), swishf(kc[3])};
        kpark[128 * j + 1] = f32x4{swishf(kc[4]), swishf(kc[5]), swishf(kc[6]), swishf(kc[7])};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kc_reg[j][e] = swishf(kc[e]);
      }
    }
  }
  // activated (Swish, before the L2 norm) inputs of the prologue
  auto qact = [&](int j, int e) {
    if constexpr (PRO == 2) return qc[j][e]; else return swishf(qraw[j].get(e));
  };
  auto kact = [&](int j, int e) {
    if constexpr (kPark) return kpark[128 * j + (e >> 2)][e & 3];
    else if constexpr (PRO == 2) return kc_reg[j][e];
    else return swishf(kraw[j].get(e));
  };

  // ---- step 2: cumulative decay.  Inclusive scan over the 16 tokens of the
  // tile (lanes lr of one lane group), then the totals of earlier tiles ----
  float G[FPW][8];
  if constexpr (SDEC) {
    const float x = row_scan16(rv ? gscalar : 0.f);  // one scan serves every channel
#pragma unroll
    for (int j = 0; j < FPW; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[j][e] = x;
  } else {
#pragma unroll
    for (int j = 0; j < FPW; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[j][e] = row_scan16(rv ? graw[j].get(e) : 0.f);
  }
  if (lr == 15) {
#pragma unroll
    for (int j = 0; j < FPW; ++j)
      if (fv[j]) {
        f32x4 a = {G[j][0], G[j][1], G[j][2], G[j][3]}, b = {G[j][4], G[j][5], G[j][6], G[j][7]};
        *reinterpret_cast<f32x4*>(tot + rt * D + 32 * fkb[j] + 8 * lg) = a;
        *reinterpret_cast<f32x4*>(tot + rt * D + 32 * fkb[j] + 8 * lg + 4) = b;
      }
  }
  // Layer prologue: this wave's part of |swish(q)|^2 and |swish(k)|^2 for
  // its token, summed over its lane groups; the waves sharing the row tile
  // hold the other channels.
  constexpr int NCW = (NFRAG < NW ? NFRAG : NW) / NRT;  // waves per row tile
  float* nrm = reinterpret_cast<float*>(smem + L::oNrm);
  if (PRO) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < FPW; ++j)
      if (fv[j]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = qact(j, e), b = kact(j, e);
          sq += a * a;
          sk += b * b;
        }
      }
    sq += __shfl_xor(sq, 16);
    sk += __shfl_xor(sk, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 32);
    if (lg == 0) {
      nrm[(w * 16 + lr) * 2] = sq;
      nrm[(w * 16 + lr) * 2 + 1] = sk;
    }
  }
  __syncthreads();  // B1: tile totals, beta, prologue norms
  float iq = 1.f, ik = 1.f;
  if (PRO) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      sq += nrm[((rt + c * NRT) * 16 + lr) * 2];
      sk += nrm[((rt + c * NRT) * 16 + lr) * 2 + 1];
    }
    iq = 1.f / fmaxf(sqrtf(sq), kL2Floor);
    ik = 1.f / fmaxf(sqrtf(sk), kL2Floor);
  }
  // G stays the decay accumulated within the row tile (from the row before
  // it).  The full cumulative decay adds the totals of the earlier tiles,
  // read per fragment from `tot` where they are used.
  // Per-channel sums of tile totals for the lane's eight channels of
  // fragment j: tiles [t0, t1).
  auto tot_sum = [&](int j, int t0, int t1, float* out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = 0.f;
    for (int t = t0; t < t1; ++t) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(tot + t * D + 32 * fkb[j] + 8 * lg);
      const f32x4 b = *reinterpret_cast<const f32x4*>(tot + t * D + 32 * fkb[j] + 8 * lg + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[e] += a[e];
        out[4 + e] += b[e];
      }
    }
  };
  // Span checks over all channels: this wave's row tile, and the chunk (the
  // same verdict in every wave).
  bool big = false, wide = false;
  for (int c = l; c < D; c += 64) {
    big |= tot[rt * D + c] < -kTileSpanLimit;
    float span = 0.f;
#pragma unroll
    for (int t = 0; t < NRT; ++t) span += tot[t * D + c];
    wide |= span < -kChunkSpanLimit;
  }
  const bool bad_tile = __any(big);
  constexpr bool tile_mode = TILE;
  if constexpr (!TILE) {
    // every wave reaches the same verdict; the tile pass takes the block
    const bool leave = __any(wide);
    if (tid == 0) *reinterpret_cast<int*>(blk + LY::kFlag) = leave ? 1 : 0;
    if (leave) return;
  }
  // inputs after the prologue
  auto kin = [&](int j, int e) { return rv ? (PRO ? kact(j, e) * ik : kraw[j].get(e)) : 0.f; };
  auto qin = [&](int j, int e) { return rv ? (PRO ? qact(j, e) * iq : qraw[j].get(e)) : 0.f; };

  // The diagonal block of a tile whose span is too large for the product
  // path, pair by pair with the exact exponent, in the accumulator layout of
  // the products (lane (lr, lg), element x: row R = 4 lg + x, column I =
  // lr).  A lane of lane group g holds row lr's values on channel set g, so
  // for every target lane group t it forms the partial sum of pair
  // (R = 4 t + x, I = lr) over set g, fetching row R from lane R + 16 g; the
  // four sets' partials for each target are then summed across the lane
  // groups, and the lane of group t keeps its own.  The result merges with
  // the other waves' channel parts as the products do.
  f32x4 accAd = {0, 0, 0, 0}, accPd = {0, 0, 0, 0};
  if (TILE && bad_tile) {
    float kvv[FPW][8], qvv[FPW][8];
#pragma unroll
    for (int j = 0; j < FPW; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kvv[j][e] = fv[j] ? kin(j, e) : 0.f;
        qvv[j][e] = fv[j] ? qin(j, e) : 0.f;
      }
#pragma unroll 1
    for (int x = 0; x < 4; ++x) {
      float pa[4], pp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int R = 4 * t + x;
        const int src = R + 16 * lg;
        float sa = 0.f, sp = 0.f;
#pragma unroll
        for (int j = 0; j < FPW; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kR = __shfl(kvv[j][e], src), qR = __shfl(qvv[j][e], src);
            const float gR = __shfl(G[j][e], src);
            const float ex = lr <= R ? __expf(gR - G[j][e]) : 0.f;  // exp(Gamma_R - Gamma_I), I <= R
            sa += kR * kvv[j][e] * ex;
            sp += qR * kvv[j][e] * ex;
          }
        sa += __shfl_xor(sa, 16);
        sp += __shfl_xor(sp, 16);
        sa += __shfl_xor(sa, 32);
        sp += __shfl_xor(sp, 32);
        pa[t] = sa;
        pp[t] = sp;
      }
      const float va = lg == 0 ? pa[0] : lg == 1 ? pa[1] : lg == 2 ? pa[2] : pa[3];
      const float vp = lg == 0 ? pp[0] : lg == 1 ? pp[1] : lg == 2 ? pp[2] : pp[3];
      if (x == 0) { accAd[0] = va; accPd[0] = vp; }
      else if (x == 1) { accAd[1] = va; accPd[1] = vp; }
      else if (x == 2) { accAd[2] = va; accPd[2] = vp; }
      else { accAd[3] = va; accPd[3] = vp; }
    }
  }

  // ---- step 3: decayed operands.  Q*gam leaves as whole fragments;
  // K-bar^T is staged transposed; the Gram operands stay in registers: rows
  // q and k times their tile-local decay exp(G), and the column operand
  // k exp(tot_rt - G), the decay from the row to the end of its tile ----
  PFrag qrf[FPW], krf[FPW], khf[FPW];
  LdsPrecise<M> KbS(smem + L::oKbS, L::kStPlain);
  {
    // references: per tile (rows x exp(G), columns k exp(tot_rt - G)), or
    // for the whole chunk (rows x exp(Gamma), columns k exp(-Gamma))
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      float qt[8], qr[8], kr[8], kh[8], gsa[8], trt[8], gn[8];
      tot_sum(j, 0, rt, gsa);
      tot_sum(j, rt, rt + 1, trt);
      tot_sum(j, 0, NRT, gn);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = kin(j, e), qv = qin(j, e);
        const float gf = G[j][e] + gsa[e];  // cumulative decay of the row
        const float ew = __expf(tile_mode ? G[j][e] : gf);
        qt[e] = qv * __expf(gf);
        qr[e] = qv * ew;
        kr[e] = kv * ew;
        kh[e] = kv * __expf(tile_mode ? trt[e] - G[j][e] : -gf);
        if (fv[j]) KbS.store((32 * fkb[j] + 8 * lg + e) * SK + r, kv * __expf(gn[e] - gf));
      }
      qrf[j] = make_pfrag(M{}, qr);
      krf[j] = make_pfrag(M{}, kr);
      khf[j] = make_pfrag(M{}, kh);
      if (fv[j]) st_pfrag(M{}, blk + LY::kQt + (size_t)(rt * NKD + fkb[j]) * LY::PF, make_pfrag(M{}, qt));
    }
  }
  if (any_frag && rt == 0 && lr == 0) {
    // gam_n: channels 32 kb + 8 lg .. + 7 of each fragment of row tile 0
#pragma unroll
    for (int j = 0; j < FPW; ++j)
      if (fv[j]) {
        float gn[8];
        tot_sum(j, 0, NRT, gn);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          reinterpret_cast<float*>(blk + LY::kGam)[32 * fkb[j] + 8 * lg + e] = __expf(gn[e]);
      }
  }
  if (KC > C) {  // zero the padded tokens
    for (int idx = tid; idx < D * (KC - C); idx += kIntraThreads) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      KbS.store(c * SK + i, 0.f);
    }
  }
  __syncthreads();  // B2: staging complete
  // Fragment (channel tile ct, token block kb): lane l reads row 16ct + (l&15),
  // tokens 32kb + 8(l>>4) .. +7, and stores them as one contiguous slot.
  for (int f = w; f < NDT * NKC; f += NW) {
    const int ct = f / NKC, kb = f % NKC;
    st_pfrag(M{}, blk + LY::kKb + (size_t)f * LY::PF, KbS.pfrag(SK, 16 * ct, 32 * kb));
  }
  __syncthreads();  // B3: staging regions free

  // ---- step 4: Grams A and P ----
  float* As = reinterpret_cast<float*>(smem + L::oA);
  float* Ps = reinterpret_cast<float*>(smem + L::oP);
  for (int idx = 4 * tid; idx < 2 * (int)(L::kFMat / 4); idx += 4 * kIntraThreads)
    *reinterpret_cast<f32x4*>(As + idx) = f32x4{0, 0, 0, 0};  // A and P are adjacent
#pragma unroll
  for (int j = 0; j < FPW; ++j)
    if (fv[j]) lds_st_pfrag(M{}, smem + L::oKh + (size_t)(rt * NKD + fkb[j]) * LY::PF, khf[j]);
  __syncthreads();  // B4: column operands staged, zeroed A and P
  // Partial Grams over this wave's channel blocks for every tile b <= rt.
  // Column tile b's operand is multiplied, per channel, by the block's
  // factor exp(Gamma_s - Gamma_e): 1 for b = rt - 1, exp(sum of the totals of
  // tiles b+1 .. rt-1) (<= 1) below that, exp(-tot_rt) on the diagonal.
  // The NC waves that share a row tile add their parts into A and P in turn,
  // one barrier apart (LDS float atomics are far slower).
  constexpr int NC = (NFRAG < NW ? NFRAG : NW) / NRT;
  f32x4 accA[NRT], accP[NRT];
#pragma unroll
  for (int b = 0; b < NRT; ++b) { accA[b] = f32x4{0, 0, 0, 0}; accP[b] = accA[b]; }
  if (any_frag) {
#pragma unroll
    for (int b = 0; b < NRT; ++b) {
      if (b > rt) break;
      if (TILE && b == rt && bad_tile) {
        accA[b] = accAd;
        accP[b] = accPd;
        continue;
      }
#pragma unroll
      for (int j = 0; j < FPW; ++j) {
        if (!fv[j]) continue;
        PFrag kbf = ld_pfrag(M{}, smem + L::oKh + (size_t)(b * NKD + fkb[j]) * LY::PF);
        if (tile_mode && b != rt - 1) {
          float ex[8];
          if (b == rt) {
            tot_sum(j, rt, rt + 1, ex);
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = -ex[e];
          } else {
            tot_sum(j, b + 1, rt, ex);
          }
          float x[8];
          pfrag_values(kbf, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= __expf(ex[e]);
          kbf = make_pfrag(M{}, x);
        }
        accP[b] = mma_pp(qrf[j], kbf, accP[b]);
        accA[b] = mma_pp(krf[j], kbf, accA[b]);
      }
    }
  }
  float brow[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) brow[x] = beta_s[16 * rt + 4 * lg + x];
  const int cix = w / NRT;  // this wave's turn among those sharing the row tile
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (any_frag && cix == c) {
      // all reads of earlier contributions first, then the writes
      float po[NRT][4], ao[NRT][4];
#pragma unroll
      for (int b = 0; b < NRT; ++b)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int rr = 16 * rt + 4 * lg + x, i = 16 * b + lr;
          po[b][x] = (c > 0 && b <= rt) ? Ps[rr * SF + i] : 0.f;
          ao[b][x] = (c > 0 && b <= rt) ? As[rr * SF + i] : 0.f;
        }
#pragma unroll
      for (int b = 0; b < NRT; ++b) {
        if (b > rt) break;
        const int i = 16 * b + lr;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int rr = 16 * rt + 4 * lg + x;
          if (i <= rr) Ps[rr * SF + i] = accP[b][x] + po[b][x];
          if (i < rr) As[rr * SF + i] = brow[x] * accA[b][x] + ao[b][x];
        }
      }
    }
    if (c + 1 < NC) __syncthreads();
  }
  __syncthreads();  // B5: A and P complete; R0 free

  // ---- step 5: P fragments out, and the operands of the solve.  T =
  // (I + A)^{-1} Diag(beta) is never formed: W = T (K*gam) and U0 = T V come
  // from block forward substitution on the right-hand sides beta (K*gam)
  // and beta V, one row block a at a time,
  //   Y_a = X_a (R_a - sum_{m<a} A_am Y_m),  X_a = (I + A_aa)^{-1},
  // with each wave carrying one 16-column tile of Y in accumulators ----
  // P fragments above the diagonal are zero: they are neither written nor
  // read.
  for (int f = w; f < NRT * NKC; f += NW) {
    if (32 * (f % NKC) > 16 * (f / NKC) + 15) continue;
    const int rr = 16 * (f / NKC) + lr, i0 = 32 * (f % NKC) + 8 * lg;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = Ps[rr * SF + i0 + e];
    gst_pfrag8(M{}, blk + LY::kP + (size_t)f * LY::PF, l, pv);
  }
  constexpr int NOFF = L::NOFF;
  float* XD = reinterpret_cast<float*>(smem + L::oXD);  // X_a, fp32 [NRT][16][17]
  char* CF = smem + L::oCF;  // chain operands: A_am (a > m) in order, then X_a
  if (w == 0) {
    // diagonal 16x16 blocks: lane = 16*block + column
    const int bk = lg, jc = lr;
    if (bk < NRT) {
      float x[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) x[s] = (s == jc) ? 1.f : 0.f;
      const float* Ab = As + (16 * bk) * SF + 16 * bk;
      // Column q of the block is read one elimination step ahead of its use;
      // hoisting all 120 reads would cost as many registers.
      float cur[16], nxt[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) { cur[s] = s > 0 ? Ab[s * SF] : 0.f; nxt[s] = 0.f; }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
#pragma unroll
        for (int s = q + 2; s < 16; ++s) nxt[s] = Ab[s * SF + q + 1];
#pragma unroll
        for (int s = q + 1; s < 16; ++s) x[s] -= cur[s] * x[q];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 16; ++s) cur[s] = nxt[s];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) XD[(16 * bk + s) * 17 + jc] = x[s];
    }
  } else {
    // block p = a (a - 1) / 2 + m below the diagonal
    for (int p = w - 1; p < NOFF; p += NW - 1) {
      int a = 1;
      while ((a + 1) * a / 2 <= p) ++a;
      const int m = p - a * (a - 1) / 2;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = As[(16 * a + lr) * SF + 16 * m + 4 * lg + e];
      cfrag_store(M{}, CF + (size_t)p * 1024, x);
    }
  }
  __syncthreads();  // B6: A consumed; X_a in fp32

  // ---- step 6: X_a as chain operands; (K*gam)^T staged over A and P.  V
  // is fetched here for step 8 ----
  Raw8<in_t> vraw[FPW], vext[PRO == 2 ? FPW : 1];
  {
    // The row addresses are formed again from opaque copies of the item's
    // fields: kept from step 1 they would be spilled to scratch and read
    // back at memory latency.
    Item iv = it;
    int rr = r;
    asm volatile("" : "+v"(iv.t0), "+v"(iv.len), "+v"(iv.bos), "+v"(iv.n), "+v"(iv.h), "+v"(rr));
    const int tk = clampi(iv.t0 + (rr < iv.len ? rr : iv.len - 1), 0, si.total_tokens - 1);
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      vraw[j].load(reinterpret_cast<const in_t*>(kp.v) + ((size_t)tk * H + iv.h) * D + 32 * fkb[j] + 8 * lg);
      if constexpr (PRO == 2) load_halo<in_t, D>(vext[j], kp, 2, iv, rt, lr, 32 * fkb[j] + 8 * lg, si.total_tokens);
    }
  }
  if (w < NRT) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = XD[(16 * w + lr) * 17 + 4 * lg + e];
    cfrag_store(M{}, CF + (size_t)(NOFF + w) * 1024, x);
  }
  // K*gam: the Gram row operand k exp(Gamma) itself with chunk-wide
  // factoring; per tile, (k exp(G)) exp(Gsa), the row operand times the decay
  // of the earlier tiles (both factors <= 1, so an underflow is a true zero).
  LdsPrecise<M> KtT(smem + L::oKtT, L::kStPlain);
  if constexpr (!TILE) {
#pragma unroll
    for (int j = 0; j < FPW; ++j)
      if (fv[j]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) KtT.put((32 * fkb[j] + 8 * lg + e) * SK + r, krf[j], e);
      }
  } else {
#pragma unroll
    for (int j = 0; j < FPW; ++j)
      if (fv[j]) {
        float x[8], gs[8];
        pfrag_values(krf[j], x);
        tot_sum(j, 0, rt, gs);
#pragma unroll
        for (int e = 0; e < 8; ++e) KtT.store((32 * fkb[j] + 8 * lg + e) * SK + r, x[e] * __expf(gs[e]));
      }
  }
  if (KC > C) {
    for (int idx = tid; idx < D * (KC - C); idx += kIntraThreads) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      KtT.store(c * SK + i, 0.f);
    }
  }
  __syncthreads();  // B7: chain operands ready, (K*gam)^T staged

  // The substitution for column tile ct of a right-hand side staged
  // transposed in Rs ([columns x KC]): lane (lg, lr) reads tokens 16a +
  // 4lg .. +3 of column 16ct + lr, the B-operand slot of its tile.
  auto substitute = [&](const LdsPrecise<M>& Rs, int ct, f32x4 (&Y)[NRT]) {
#pragma unroll
    for (int a = 0; a < NRT; ++a) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < a; ++m) acc = chain_mma(M{}, CF + (size_t)(a * (a - 1) / 2 + m) * 1024, Y[m], acc);
      float rh[4];
      Rs.get4((16 * ct + lr) * SK + 16 * a + 4 * lg, rh);
      f32x4 rhs;
#pragma unroll
      for (int e = 0; e < 4; ++e) rhs[e] = beta_s[16 * a + 4 * lg + e] * rh[e] - acc[e];
      Y[a] = chain_mma(M{}, CF + (size_t)(NOFF + a) * 1024, rhs, f32x4{0, 0, 0, 0});
    }
  };

  // ---- step 7: W.  Each wave solves one channel tile and writes it back
  // over the columns of (K*gam)^T it alone read; W fragments then leave in
  // the layout of the inter-chunk pass (lane slot: one token, eight
  // consecutive channels) ----
  if (w < NDT) {
    f32x4 Y[NRT];
    substitute(KtT, w, Y);
#pragma unroll
    for (int a = 0; a < NRT; ++a) {
      const float y4[4] = {Y[a][0], Y[a][1], Y[a][2], Y[a][3]};
      KtT.template storeN<4>((16 * w + lr) * SK + 16 * a + 4 * lg, y4);
    }
  }
  __syncthreads();  // B8: W^T staged
  for (int f = w; f < NRT * NKD; f += NW) {
    const int wt = f / NKD, cb = f % NKD;
    float wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = KtT.get((32 * cb + 8 * lg + e) * SK + 16 * wt + lr);
    gst_pfrag8(M{}, blk + LY::kW + (size_t)f * LY::PF, l, wv);
  }
  __syncthreads();  // B9: W^T reads done

  // ---- step 8: U0 = T V, tile (token tile a, value tile ct), stored in the
  // accumulator layout the inter-chunk pass adds to.  V^T is staged (split
  // into hi + lo, so V need not be bf16-exact) over W^T ----
  LdsPrecise<M> VT(smem + L::oVT, L::kStPlain);
#pragma unroll
  for (int j = 0; j < FPW; ++j)
    if (fv[j]) {
      float vx[8];
      if constexpr (PRO == 2) {
        const int c0 = 32 * fkb[j] + 8 * lg;
        conv8(vraw[j], vext[j], reinterpret_cast<const float*>(smem + L::oCWv) + c0 * kMaxConv, kp.conv_w, lr, vx);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vx[e] = vraw[j].get(e);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        VT.store((32 * fkb[j] + 8 * lg + e) * SK + r, rv ? (PRO ? swishf(vx[e]) : vx[e]) : 0.f);
    }
  if (KC > C) {
    for (int idx = tid; idx < D * (KC - C); idx += kIntraThreads) {
      const int c = idx / (KC - C), i = C + idx % (KC - C);
      VT.store(c * SK + i, 0.f);
    }
  }
  __syncthreads();  // B10: V^T staged
  if (w < NDT) {
    f32x4 Y[NRT];
    substitute(VT, w, Y);
#pragma unroll
    for (int a = 0; a < NRT; ++a)
      *reinterpret_cast<f32x4*>(blk + LY::kU0 + (size_t)(a * NDT + w) * 1024 + l * 16) = Y[a];
  }
}

// ---------------------------------------------------------------------------
// Layer epilogue (the "Kimi Linear" notes, docsaid.org, section "Other
// Components"; greeksharifa.github.io summary, section 4): per token and
// head, y = o / sqrt(mean_c o_c^2 + eps) * weight * sigmoid(gate).  The norm
// spans all D value columns, which the inter-chunk pass splits over
// workgroups, so it runs after that pass, per segment, on the raw o it left
// in the workspace.  Four waves per (slot, head), C / 4 rows per wave.
// D / 4 consecutive lanes hold one row, four columns each, so a wave's
// 16-byte loads cover whole rows (two for d = 128); every row's loads are
// issued before the first use, and the mean square is summed over the row's
// lanes.  No barrier: a wave may leave early.  With the convolution, every
// segment's epilogue but the last runs in the next segment's chunk-wide intra
// launch, as workgroups after its items (two items each): the raw o is
// untouched until that segment's carry pass, and this HBM-bound work fills
// compute units beside the VALU-bound intra items.  The last segment's runs as
// a launch of its own.
// ---------------------------------------------------------------------------
template <class M, int D, int C, bool OUT_BF16>
__device__ __forceinline__ void layer_epilogue_item(const KernelPtrs& kp, const SeqInfo& si, int item,
                                                    int wave) {
  typedef typename M::in_t in_t;
  constexpr int LPR = D / 4;       // lanes per row
  constexpr int RPI = 64 / LPR;    // rows per wave and pass
  constexpr int NI = C / 4 / RPI;  // passes per wave
  static_assert(NI >= 1 && C % (4 * RPI) == 0, "whole passes per wave");
  const Item it = intra_item<C>(si, kp, item, 0);
  if (it.len <= 0) return;
  const int slot = item / kp.H;
  const int l = lane_id();
  const int c0 = 4 * (l % LPR);
  const int rb = (C / 4) * wave + l / LPR;
  const in_t* gate = reinterpret_cast<const in_t*>(kp.gate);
  const f32x4 wt = *reinterpret_cast<const f32x4*>(kp.norm_weight + c0);
  f32x4 x[NI], gv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = rb + RPI * i;
    const int rr = row < it.len ? row : 0;  // rows past the chunk read row 0 and store nothing
    x[i] = *reinterpret_cast<const f32x4*>(kp.o_slots + (((size_t)slot * kp.H + it.h) * C + rr) * D + c0);
    const size_t ti = ((size_t)(it.t0 + rr) * kp.H + it.h) * D + c0;
    if constexpr (sizeof(in_t) == 2) {
      const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(gate + ti);
      gv[i] = f32x4{(float)g4[0], (float)g4[1], (float)g4[2], (float)g4[3]};
    } else {
      gv[i] = *reinterpret_cast<const f32x4*>(gate + ti);
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = rb + RPI * i;
    float ss = x[i][0] * x[i][0] + x[i][1] * x[i][1] + x[i][2] * x[i][2] + x[i][3] * x[i][3];
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.f / sqrtf(ss / D + kp.norm_eps);
    if (row < it.len) {
      const size_t ti = ((size_t)(it.t0 + row) * kp.H + it.h) * D + c0;
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = x[i][e] * inv * wt[e] * sigmoidf(gv[i][e]);
      if constexpr (OUT_BF16) {
        bf16x4 yb;
#pragma unroll
        for (int e = 0; e < 4; ++e) yb[e] = f2bf(y[e]);
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(kp.o) + ti) = yb;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(kp.o) + ti) = y;
      }
    }
  }
}

// The previous segment's layer epilogue, carried by a chunk-wide launch.
struct EpiJob {
  SeqInfo si;    // the previous segment
  int items;     // its (slot, head) items; 0: none
  int out_bf16;  // y in bf16 (else fp32)
};

// The chunk-wide pass: one workgroup per item (item = slot * H + head), then
// with the layer prologue and its convolution the workgroups of the previous
// segment's epilogue.  (Without the convolution the branch would cost the
// item path a spill; there every segment's epilogue has a launch of its own.)
template <class M, int D, int C, bool SDEC, int PRO>
__global__ __launch_bounds__(kIntraThreads, 4) void intra_chunk_kernel(KernelPtrs kp, SeqInfo si, int items,
                                                                       EpiJob ej) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int b = blockIdx.x;
  if constexpr (PRO == 2) {
    if (b >= items) {
      const int e = 2 * (b - items) + (wave_id() >> 2);
      if (e < ej.items) {
        if (ej.out_bf16)
          layer_epilogue_item<M, D, C, true>(kp, ej.si, e, wave_id() & 3);
        else
          layer_epilogue_item<M, D, C, false>(kp, ej.si, e, wave_id() & 3);
      }
      return;
    }
  }
  intra_item_body<M, D, C, SDEC, PRO, false>(kp, si, b, smem);
}

// The tile pass: each workgroup looks at two items and works on the ones the
// chunk-wide pass flagged, so a segment without any costs one launch of half
// the size (at T = 4096, H = 32, one round of two workgroups per CU).  Two
// written-out calls, not a loop: in a loop the compiler keeps per-lane
// values live across the body and spills hundreds of bytes.
template <class M, int D, int C, bool SDEC, int PRO>
__global__ __launch_bounds__(kIntraThreads, 4) void intra_tile_kernel(KernelPtrs kp, SeqInfo si, int items) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  intra_item_body<M, D, C, SDEC, PRO, true>(kp, si, 2 * blockIdx.x, smem);
  __syncthreads();  // the first item's last LDS reads before the second's writes
  if (2 * (int)blockIdx.x + 1 < items)
    intra_item_body<M, D, C, SDEC, PRO, true>(kp, si, 2 * blockIdx.x + 1, smem);
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel: one workgroup per (sequence, head, block of value
// columns), 512 threads in two roles that share the chunk loop:
//
//   U-waves (0..3) carry the state.  Wave w owns row tile w of U and the
//     NST state row tiles NST*w ..; per chunk it forms U = U0 - W S,
//     publishes U^T in LDS, then updates its state tiles
//     S <- Diag(gam_n) S + K-bar^T U and publishes S^T in LDS.
//   O-waves (4..7) produce the output.  Wave 4 + r forms Q*gam S for row
//     tile r from the published state, then O = Q*gam S + P U from the
//     published U, and stores it.
//
// Each SIMD runs one wave of each role, so one wave's operand loads overlap
// the other's matrix products; the two roles split the per-chunk operands
// (U-waves: W, U0, K-bar^T, gam_n; O-waves: Q*gam, P).
// ---------------------------------------------------------------------------
constexpr int kInterThreads = 512;

template <class M, int D, int C, int NCT>
struct UFrags {
  typedef Layout<M, D, C> LY;
  static constexpr int NST = LY::NDT / 4;  // state tiles per U-wave
  typename M::PFrag W[LY::NKD];
  f32x4 U0[NCT];                           // T V tiles of this row tile
  typename M::PFrag Kb[NST][LY::NKC];
  float gam[NST][4];
};

template <class M, int D, int C>
struct OFrags {
  typedef Layout<M, D, C> LY;
  typename M::PFrag Qt[LY::NKD];
  typename M::PFrag P[LY::NKC];
};

// Every wave of a role issues the same loads.  With fewer than four row
// tiles the surplus waves re-read the last one (and skip its products): a
// load that only some paths issue leaves the compiler's count of outstanding
// loads wrong, and a later wait can pass before its data has arrived.
template <class M, int D, int C, int NCT>
__device__ __forceinline__ void load_u1(UFrags<M, D, C, NCT>& f, const char* blk, int rt, int vt0) {
  typedef Layout<M, D, C> LY;
#pragma unroll
  for (int kb = 0; kb < LY::NKD; ++kb)
    f.W[kb] = ld_pfrag(M{}, blk + LY::kW + (size_t)(rt * LY::NKD + kb) * LY::PF);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
    f.U0[ct] = *reinterpret_cast<const f32x4*>(blk + LY::kU0 + (size_t)(rt * LY::NDT + vt0 + ct) * 1024 +
                                               lane_id() * 16);
}
template <class M, int D, int C, int NCT>
__device__ __forceinline__ void load_u2(UFrags<M, D, C, NCT>& f, const char* blk, int w) {
  typedef Layout<M, D, C> LY;
  constexpr int NST = UFrags<M, D, C, NCT>::NST;
  const int l = lane_id();
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
template <class M, int D, int C>
__device__ __forceinline__ void load_o1(OFrags<M, D, C>& f, const char* blk, int rt) {
  typedef Layout<M, D, C> LY;
#pragma unroll
  for (int kb = 0; kb < LY::NKD; ++kb)
    f.Qt[kb] = ld_pfrag(M{}, blk + LY::kQt + (size_t)(rt * LY::NKD + kb) * LY::PF);
}
// The first NP token blocks of P (the rest of the row tile is zero).
template <class M, int D, int C, int NP>
__device__ __forceinline__ void load_o2(OFrags<M, D, C>& f, const char* blk, int rt) {
  typedef Layout<M, D, C> LY;
#pragma unroll
  for (int kb = 0; kb < NP; ++kb)
    f.P[kb] = ld_pfrag(M{}, blk + LY::kP + (size_t)(rt * LY::NKC + kb) * LY::PF);
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

// Geometry of one inter-chunk workgroup.  This launch runs the sequence's
// chunks [ci_lo, ci_hi); chunk ci's operand block is number cbase + ci of
// the segment.  The state enters from s_in (nullptr = zeros) and leaves to
// s_out (nullptr = not written).
struct InterGeom {
  int n, h, H, bos, eos, nch, col0, vb;
  int ci_lo, ci_hi, cbase;
  const float* s_in;
  float* s_out;
};

// Pipeline (both roles): two operand sets alternate between even and odd
// chunks.  After phase 1 of chunk c its set receives the phase-1 group of
// chunk c+2; after phase 2 the other set receives the phase-2 group of chunk
// c+1.  Loads past the last chunk re-read it: they stay unconditional.
template <class M, int D, int C, int NCT>
__device__ __forceinline__ void inter_u_role(const KernelPtrs& kp, const InterGeom& gm, char* smem,
                                             int w) {
  typedef Layout<M, D, C> LY;
  typedef InterLds<M, D, C, NCT> L;
  typedef UFrags<M, D, C, NCT> UF;
  constexpr int NRT = LY::NRT, NKC = LY::NKC, NKD = LY::NKD, NDT = LY::NDT;
  constexpr int NST = UF::NST;
  constexpr int SD = L::SD, SK = L::SK;
  static_assert(NDT == 4 * NST, "every U-wave owns NST state tiles");
  const int l = lane_id();
  LdsPrecise<M> ST(smem + L::oST, L::kSTplain);
  LdsPrecise<M> UT(smem + L::oUT, L::kUTplain);
  const int rt = NRT == 4 ? w : min(w, NRT - 1);
  const bool act = NRT == 4 || w < NRT;
  const int vt0 = gm.col0 / 16;

  f32x4 S[NST][NCT];
  const size_t sbase = ((size_t)gm.n * gm.H + gm.h) * D * D;
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int st = w * NST + s;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = 16 * st + 4 * (l >> 4) + x;
        S[s][ct][x] = gm.s_in ? gm.s_in[sbase + (size_t)c * D + gm.col0 + 16 * ct + (l & 15)] : 0.f;
      }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float v4[4] = {S[s][ct][0], S[s][ct][1], S[s][ct][2], S[s][ct][3]};
        ST.template storeN<4>((16 * ct + (l & 15)) * SD + 16 * st + 4 * (l >> 4), v4);
      }
    }
  };
  publish_state();

  auto blk_of = [&](int ci) { return kp.ops + ((size_t)(gm.cbase + ci) * gm.H + gm.h) * LY::kBytes; };
  const int last = gm.ci_hi - 1;
  // The chain's products keep two partial sums (even and odd k blocks) so
  // that consecutive MFMAs do not wait on each other's accumulator.
  // The loads of later chunks are spread over the products: a fragment of
  // this chunk is replaced by the one two chunks ahead right after its last
  // use (W, U0), and the next chunk's K-bar and gam go into the other set
  // between the K-bar^T U products, so the load path stays busy through the
  // step instead of taking bursts that stall the issuing wave.
  auto step = [&](UF& f, UF& g, int ci) {
    const char* b2 = blk_of(min(ci + 2, last));
    const char* b1 = blk_of(min(ci + 1, last));
    __syncthreads();  // S^T published; last chunk's U^T reads done
    f32x4 ws0[NCT], ws1[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) { ws0[ct] = f32x4{0, 0, 0, 0}; ws1[ct] = ws0[ct]; }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      if (act) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const auto sf = ST.pfrag(SD, 16 * ct, 32 * kb);
          if (kb & 1)
            ws1[ct] = mma_pp(f.W[kb], sf, ws1[ct]);
          else
            ws0[ct] = mma_pp(f.W[kb], sf, ws0[ct]);
        }
      }
      f.W[kb] = ld_pfrag(M{}, b2 + LY::kW + (size_t)(rt * NKD + kb) * LY::PF);
    }
    if (act) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float v4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) v4[x] = f.U0[ct][x] - (ws0[ct][x] + ws1[ct][x]);
        UT.template storeN<4>((16 * ct + (l & 15)) * SK + 16 * rt + 4 * (l >> 4), v4);
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      f.U0[ct] = *reinterpret_cast<const f32x4*>(b2 + LY::kU0 + (size_t)(rt * NDT + vt0 + ct) * 1024 +
                                                 l * 16);
    __syncthreads();  // U^T published; S^T reads done
    f32x4 S1[NST][NCT];
#pragma unroll
    for (int s = 0; s < NST; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        S1[s][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int x = 0; x < 4; ++x) S[s][ct][x] *= f.gam[s][x];
      }
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(
          reinterpret_cast<const float*>(b1 + LY::kGam) + 16 * (w * NST + s) + 4 * (l >> 4));
#pragma unroll
      for (int x = 0; x < 4; ++x) g.gam[s][x] = gv[x];
    }
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const auto uf = UT.pfrag(SK, 16 * ct, 32 * kb);
#pragma unroll
        for (int s = 0; s < NST; ++s) {
          if (kb & 1)
            S1[s][ct] = mma_pp(f.Kb[s][kb], uf, S1[s][ct]);
          else
            S[s][ct] = mma_pp(f.Kb[s][kb], uf, S[s][ct]);
        }
      }
#pragma unroll
      for (int s = 0; s < NST; ++s)
        g.Kb[s][kb] = ld_pfrag(M{}, b1 + LY::kKb + (size_t)((w * NST + s) * NKC + kb) * LY::PF);
    }
#pragma unroll
    for (int s = 0; s < NST; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S[s][ct] += S1[s][ct];
    publish_state();
  };

  UF fa, fb;
  if (gm.ci_lo < gm.ci_hi) {
    load_u1<M, D, C, NCT>(fa, blk_of(gm.ci_lo), rt, vt0);
    load_u2<M, D, C, NCT>(fa, blk_of(gm.ci_lo), w);
    load_u1<M, D, C, NCT>(fb, blk_of(min(gm.ci_lo + 1, last)), rt, vt0);
  }
  for (int ci = gm.ci_lo; ci < gm.ci_hi; ci += 2) {
    step(fa, fb, ci);
    if (ci + 1 >= gm.ci_hi) break;
    step(fb, fa, ci + 1);
  }
  if (gm.s_out) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int st = w * NST + s;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = 16 * st + 4 * (l >> 4) + x;
          gm.s_out[sbase + (size_t)c * D + gm.col0 + 16 * ct + (l & 15)] = S[s][ct][x];
        }
    }
  }
}

// NP: token blocks of P that are not zero for this wave's row tile.
template <class M, int D, int C, int NCT, bool OUT_BF16, int NP>
__device__ __forceinline__ void inter_o_role(const KernelPtrs& kp, const InterGeom& gm, char* smem,
                                             int r) {
  typedef Layout<M, D, C> LY;
  typedef InterLds<M, D, C, NCT> L;
  typedef OFrags<M, D, C> OF;
  constexpr int NRT = LY::NRT, NKC = LY::NKC, NKD = LY::NKD;
  constexpr int SD = L::SD, SK = L::SK;
  const int l = lane_id();
  LdsPrecise<M> ST(smem + L::oST, L::kSTplain);
  LdsPrecise<M> UT(smem + L::oUT, L::kUTplain);
  const int rt = NRT == 4 ? r : min(r, NRT - 1);
  const bool act = NRT == 4 || r < NRT;
  const int H = gm.H;

  auto blk_of = [&](int ci) { return kp.ops + ((size_t)(gm.cbase + ci) * H + gm.h) * LY::kBytes; };
  const int last = gm.ci_hi - 1;

  // Loads spread over the products as in the U-waves: Q*gam fragments two
  // chunks ahead replace this chunk's right after use; the next chunk's P
  // fragments go into the other set between the P U products.
  auto step = [&](OF& f, OF& g, int ci) {
    const int t0 = gm.bos + ci * C;
    const int len = gm.eos - t0 < C ? gm.eos - t0 : C;
    const char* b2 = blk_of(min(ci + 2, last));
    const char* b1 = blk_of(min(ci + 1, last));
    __syncthreads();  // S^T published
    f32x4 qs[NCT], qs1[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) { qs[ct] = f32x4{0, 0, 0, 0}; qs1[ct] = qs[ct]; }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      if (act) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const auto sf = ST.pfrag(SD, 16 * ct, 32 * kb);
          if (kb & 1)
            qs1[ct] = mma_pp(f.Qt[kb], sf, qs1[ct]);
          else
            qs[ct] = mma_pp(f.Qt[kb], sf, qs[ct]);
        }
      }
      f.Qt[kb] = ld_pfrag(M{}, b2 + LY::kQt + (size_t)(rt * NKD + kb) * LY::PF);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) qs[ct] += qs1[ct];
    __syncthreads();  // U^T published
#pragma unroll
    for (int kb = 0; kb < NP; ++kb) {
      if (act) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) qs[ct] = mma_pp(f.P[kb], UT.pfrag(SK, 16 * ct, 32 * kb), qs[ct]);
      }
      g.P[kb] = ld_pfrag(M{}, b1 + LY::kP + (size_t)(rt * NKC + kb) * LY::PF);
    }
    if (act) {
      // After a transpose inside each lane quad, lane l holds four
      // consecutive columns 4((l & 15) >> 2) .. of row 4(l >> 4) + (l & 3):
      // one vector store per lane and tile.
      const int row = 16 * rt + 4 * (l >> 4) + (l & 3);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const f32x4 o = quad_transpose(qs[ct]);
        const int col = gm.col0 + 16 * ct + 4 * ((l & 15) >> 2);
        if (row < len) {
          if (kp.o_slots) {  // raw o for the layer epilogue
            *reinterpret_cast<f32x4*>(kp.o_slots + (((size_t)(gm.cbase + ci) * H + gm.h) * C + row) * D +
                                      col) = o;
          } else {
            const size_t oi = ((size_t)(t0 + row) * H + gm.h) * D + col;
            if constexpr (OUT_BF16) {
              bf16x4 ob;
#pragma unroll
              for (int x = 0; x < 4; ++x) ob[x] = f2bf(o[x]);
              *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(kp.o) + oi) = ob;
            } else {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(kp.o) + oi) = o;
            }
          }
        }
      }
    }
  };

  OF fa, fb;
  if (gm.ci_lo < gm.ci_hi) {
    load_o1<M, D, C>(fa, blk_of(gm.ci_lo), rt);
    load_o2<M, D, C, NP>(fa, blk_of(gm.ci_lo), rt);
    load_o1<M, D, C>(fb, blk_of(min(gm.ci_lo + 1, last)), rt);
  }
  for (int ci = gm.ci_lo; ci < gm.ci_hi; ci += 2) {
    step(fa, fb, ci);
    if (ci + 1 >= gm.ci_hi) break;
    step(fb, fa, ci + 1);
  }
}

template <class M, int D, int C, bool OUT_BF16>
__global__ __launch_bounds__(256) void layer_epilogue_kernel(KernelPtrs kp, SeqInfo si) {
  layer_epilogue_item<M, D, C, OUT_BF16>(kp, si, blockIdx.x, wave_id());
}

// NCT = number of 16-column value tiles per workgroup (16 or 32 columns).
template <class M, int D, int C, int NCT, bool OUT_BF16>
__global__ __launch_bounds__(kInterThreads, 2) void inter_chunk_kernel(KernelPtrs kp, SeqInfo si,
                                                                       int num_pairs) {
  typedef Layout<M, D, C> LY;
  typedef InterLds<M, D, C, NCT> L;
  constexpr int KC = LY::KC;
  constexpr int DVB = L::DVB;
  constexpr int NVB = D / DVB;
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  // XCD-aware mapping: consecutive block ids rotate over the 8 XCDs, so the
  // NVB column blocks of one (sequence, head) are given ids that land on the
  // same XCD and share its L2 for the per-chunk operands.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int pair = (slot / NVB) * 8 + xcd;
  InterGeom gm;
  gm.vb = slot % NVB;
  if (pair >= num_pairs) return;
  gm.H = kp.H;
  gm.n = pair / gm.H;
  gm.h = pair % gm.H;
  gm.col0 = DVB * gm.vb;
  seq_bounds(si, gm.n, gm.bos, gm.eos);
  gm.nch = chunks_of<C>(gm.eos - gm.bos);
  // This launch covers the sequence's local chunks [c0, c0 + L), held in the
  // workspace slots base .. base + count - 1.  A sequence without chunks is
  // settled (final = initial state) by the first segment.
  const int base = si.cu ? clampi(si.slot_off[gm.n], 0, si.max_slots) : gm.n * si.slot_cnt;
  gm.ci_lo = si.c0;
  // Never walk past the slots the workspace was sized for.
  gm.ci_hi = min(min(si.c0 + si.L, gm.nch), si.c0 + (si.max_slots - base));
  if (gm.nch > 0 ? gm.ci_lo >= gm.ci_hi : si.c0 != 0) return;
  if (gm.nch == 0) gm.ci_hi = gm.ci_lo;
  gm.cbase = base - si.c0;
  gm.s_in = gm.ci_lo == 0 ? kp.s0 : kp.carry;
  gm.s_out = gm.ci_hi == gm.nch ? kp.s1 : kp.carry;

  // Zero the padded token columns of U^T once (KC > C); nothing writes them.
  if (KC > C) {
    LdsPrecise<M> UT(smem + L::oUT, L::kUTplain);
    for (int idx = threadIdx.x; idx < DVB * (KC - C); idx += kInterThreads)
      UT.store((idx / (KC - C)) * L::SK + C + idx % (KC - C), 0.f);
  }
  const int w = wave_id();
  constexpr int NRT = LY::NRT, NKC = LY::NKC;
  static_assert(NKC <= 2, "P spans at most two token blocks");
  if (w < 4) {
    inter_u_role<M, D, C, NCT>(kp, gm, smem, w);
  } else {
    // P is lower triangular: row tiles 0 and 1 use only its first 32 tokens.
    const int rt = NRT == 4 ? w - 4 : min(w - 4, NRT - 1);
    if (NKC == 2 && 16 * rt + 15 >= 32)
      inter_o_role<M, D, C, NCT, OUT_BF16, NKC>(kp, gm, smem, w - 4);
    else
      inter_o_role<M, D, C, NCT, OUT_BF16, 1>(kp, gm, smem, w - 4);
  }
}

// The carried inputs of the short convolution after the call: the last W-1
// inputs of each sequence (of its state rows where it is shorter).  One
// workgroup per (sequence, head) and tensor, one thread per channel; each
// thread reads state row len + j before it writes row j, so the output may
// overwrite the input state in place.
struct ConvStateArgs {
  const void* x[3];
  const void* in[3];
  void* out[3];
  int W, H;
};

template <class T, int D>
__device__ __forceinline__ void conv_state_item(const ConvStateArgs& ca, const SeqInfo& si, int n, int h,
                                                int x, int c) {
  int bos, eos;
  seq_bounds(si, n, bos, eos);
  const int W1 = ca.W - 1, len = eos - bos;
  const T* src = reinterpret_cast<const T*>(ca.x[x]);
  const T* in = reinterpret_cast<const T*>(ca.in[x]);
  T* out = reinterpret_cast<T*>(ca.out[x]);
  const size_t sb = ((size_t)n * ca.H + h) * W1 * D + c;
  for (int j = 0; j < W1; ++j) {
    const int te = eos - W1 + j;
    T v;
    if (te >= bos)
      v = src[((size_t)te * ca.H + h) * D + c];
    else
      v = in ? in[sb + (size_t)(len + j) * D] : T(0.f);
    out[sb + (size_t)j * D] = v;
  }
}

template <class T, int D>
__global__ __launch_bounds__(D) void conv_state_kernel(ConvStateArgs ca, SeqInfo si) {
  const int x = blockIdx.y;
  if (!ca.out[x]) return;
  conv_state_item<T, D>(ca, si, blockIdx.x / ca.H, blockIdx.x % ca.H, x, threadIdx.x);
}

// The last segment's layer epilogue (items workgroups) and then the carried
// convolution inputs (one workgroup per (sequence, head), the three tensors
// over its threads) in one launch: it follows every pass that reads the old
// carried inputs.
template <class M, int D, int C, bool OUT_BF16>
__global__ __launch_bounds__(256) void layer_epilogue_conv_kernel(KernelPtrs kp, SeqInfo si,
                                                                  ConvStateArgs ca, int items) {
  const int b = blockIdx.x;
  if (b < items) {
    layer_epilogue_item<M, D, C, OUT_BF16>(kp, si, b, wave_id());
    return;
  }
  static_assert(256 % D == 0, "whole tensors per pass");
  const int pair = b - items, c = threadIdx.x % D;
  for (int x = threadIdx.x / D; x < 3; x += 256 / D)
    if (ca.out[x]) conv_state_item<typename M::in_t, D>(ca, si, pair / ca.H, pair % ca.H, x, c);
}

// Value-column block width of the inter-chunk pass: wide blocks cut the
// per-chunk operand traffic (each block re-reads the chunk's operands),
// narrow ones give more workgroups.  32 columns once there are enough
// (sequence, head) pairs to fill the chip twice over with them, unless the
// caller's tuning fixes the width.
static int choose_nct(int pairs, int D, const PrefillTuning& t) {
  if (t.value_block == 16 || t.value_block == 32) return t.value_block / 16;
  return (long long)pairs * (D / 32) >= 512 ? 2 : 1;
}

template <class M, int D, int C, int NCT>
static void launch_inter(const PrefillArgs& a, const KernelPtrs& kp, const SeqInfo& si) {
  const int pairs = a.num_seqs * a.H;
  const int nvb = D / (16 * NCT);
  const int blocks = ((pairs + 7) / 8) * 8 * nvb;
  if (a.out_bf16)
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, NCT, true>), dim3(blocks), dim3(kInterThreads), 0,
                       a.stream, kp, si, pairs);
  else
    hipLaunchKernelGGL((inter_chunk_kernel<M, D, C, NCT, false>), dim3(blocks), dim3(kInterThreads), 0,
                       a.stream, kp, si, pairs);
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
template <class M, int D, int C, bool SDEC>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  typedef Layout<M, D, C> LY;
  char* ws = reinterpret_cast<char*>(a.workspace);
  const bool epi = a.layer.gate != nullptr;
  const SegmentPlan plan = plan_segments(a.num_seqs, a.cu_seqlens_host, a.seq_len, a.H, D, C,
                                         a.in_bf16, epi, a.tuning);
  if (plan.nseg == 0) return hipErrorInvalidValue;  // checked before, on the host
  const SeqCounts sc{a.num_seqs, a.cu_seqlens_host, a.seq_len, C};
  SeqInfo si;
  si.cu = a.cu_seqlens;
  si.num_seqs = a.num_seqs;
  si.seq_len = a.seq_len;
  si.total_tokens = a.total_tokens;
  const size_t tbytes = table_bytes(a.num_seqs, a.cu_seqlens != nullptr);
  const int ntab = table_copies(plan, epi);
  const int32_t* tables[2] = {reinterpret_cast<const int32_t*>(ws),
                              reinterpret_cast<const int32_t*>(ws + (ntab - 1) * tbytes)};
  si.slot_off = tables[0];
  si.max_slots = plan.max_slots;
  si.L = plan.L;
  KernelPtrs kp;
  kp.q = a.q;
  kp.k = a.k;
  kp.v = a.v;
  kp.g = a.g;
  kp.beta = a.beta;
  kp.o = a.o;
  kp.s0 = a.initial_state;
  kp.s1 = a.final_state;
  char* after_table = ws + ntab * tbytes;
  const size_t carry = carry_bytes(plan, a.num_seqs, a.H, D);
  kp.carry = carry ? reinterpret_cast<float*>(after_table) : nullptr;
  kp.ops = after_table + carry;
  kp.H = a.H;
  kp.o_slots = epi ? reinterpret_cast<float*>(kp.ops + (size_t)plan.max_slots * a.H * LY::kBytes)
                   : nullptr;
  kp.gate = a.layer.gate;
  kp.norm_weight = a.layer.norm_weight;
  kp.norm_eps = a.layer.norm_eps;
  kp.conv_w = a.layer.conv_w;
  for (int x = 0; x < 3; ++x) {
    kp.cw[x] = a.layer.conv_weight[x];
    kp.cs[x] = a.layer.conv_state_in[x];
  }

  constexpr size_t lds0 = IntraLds<M, D, C>::kTotal, lds_conv = IntraLds<M, D, C>::kTotalConv;
  static_assert(lds_conv <= 80 * 1024, "two intra-chunk workgroups per compute unit");
  // The prologue is built for the per-channel decay only.
  constexpr int P1 = SDEC ? 0 : 1, P2 = SDEC ? 0 : 2;
  if (SDEC && a.layer.prologue) return hipErrorInvalidValue;
  const int pro = !a.layer.prologue ? 0 : a.layer.conv_w > 0 ? 2 : 1;
  const size_t lds = pro == 2 ? lds_conv : lds0;
  const void* intra_fn[2] = {
      pro == 2   ? reinterpret_cast<const void*>(&intra_chunk_kernel<M, D, C, SDEC, P2>)
      : pro == 1 ? reinterpret_cast<const void*>(&intra_chunk_kernel<M, D, C, SDEC, P1>)
                 : reinterpret_cast<const void*>(&intra_chunk_kernel<M, D, C, SDEC, 0>),
      pro == 2   ? reinterpret_cast<const void*>(&intra_tile_kernel<M, D, C, SDEC, P2>)
      : pro == 1 ? reinterpret_cast<const void*>(&intra_tile_kernel<M, D, C, SDEC, P1>)
                 : reinterpret_cast<const void*>(&intra_tile_kernel<M, D, C, SDEC, 0>)};
  if (plan.max_slots > 0) {
    for (const void* fn : intra_fn) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
  }
  const int nct = choose_nct(a.num_seqs * a.H, D, a.tuning);
  auto launch_epilogue = [&](const SeqInfo& sq, int items) {
    if (a.out_bf16)
      hipLaunchKernelGGL((layer_epilogue_kernel<M, D, C, true>), dim3(items), dim3(256), 0, a.stream, kp, sq);
    else
      hipLaunchKernelGGL((layer_epilogue_kernel<M, D, C, false>), dim3(items), dim3(256), 0, a.stream, kp,
                         sq);
  };
  EpiJob ej;  // the epilogue still to run: the previous segment's
  ej.si = si;
  ej.items = 0;
  ej.out_bf16 = a.out_bf16 ? 1 : 0;
  for (int s = 0; s < plan.nseg; ++s) {
    si.c0 = s * plan.L;
    si.slot_off = tables[s & 1];
    const long long slots = sc.slots(si.c0, plan.L);
    if (a.cu_seqlens) {
      hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens,
                         const_cast<int32_t*>(si.slot_off), a.num_seqs, a.total_tokens, C, si.c0,
                         plan.L);
      si.slot_cnt = 0;
    } else {
      const int c = sc.nch(0) - si.c0;
      si.slot_cnt = c <= 0 ? 0 : (c < plan.L ? c : plan.L);
    }
    // the chunk-wide intra pass (with the previous segment's epilogue), then
    // the tile pass for the blocks it left
    if (slots > 0) {
      int items = (int)(slots * a.H);
      const dim3 igrid((unsigned)(items + (ej.items + 1) / 2));
      void* args[] = {&kp, &si, &items, &ej};
      hipError_t e = hipLaunchKernel(intra_fn[0], igrid, dim3(kIntraThreads), args, lds, a.stream);
      if (e != hipSuccess) return e;
      ej.items = 0;
      void* targs[] = {&kp, &si, &items};
      e = hipLaunchKernel(intra_fn[1], dim3((unsigned)((items + 1) / 2)), dim3(kIntraThreads), targs, lds,
                          a.stream);
      if (e != hipSuccess) return e;
    }
    // with no intra launch to carry it, the previous epilogue before the
    // carry pass overwrites the raw o
    if (ej.items > 0) launch_epilogue(ej.si, ej.items);
    if (nct == 2)
      launch_inter<M, D, C, 2>(a, kp, si);
    else
      launch_inter<M, D, C, 1>(a, kp, si);
    if (epi && pro == 2) {  // carried by the next chunk-wide launch
      ej.si = si;
      ej.items = (int)(slots * a.H);
    } else if (epi && slots > 0) {
      launch_epilogue(si, (int)(slots * a.H));
    }
  }
  // The carried convolution inputs, after every pass that reads the old ones
  // (they may share memory); with the epilogue, in its last launch.
  const bool conv_out = a.layer.conv_state_out[0] || a.layer.conv_state_out[1] ||
                        a.layer.conv_state_out[2];
  const bool conv_state = pro == 2 && a.layer.conv_w > 1 && conv_out && a.num_seqs > 0;
  ConvStateArgs ca;
  ca.W = a.layer.conv_w;
  ca.H = a.H;
  for (int x = 0; x < 3; ++x) {
    ca.x[x] = x == 0 ? a.q : x == 1 ? a.k : a.v;
    ca.in[x] = a.layer.conv_state_in[x];
    ca.out[x] = a.layer.conv_state_out[x];
  }
  if (ej.items > 0 && conv_state) {  // the last segment's epilogue and the carried inputs
    const dim3 grid((unsigned)(ej.items + a.num_seqs * a.H));
    if (a.out_bf16)
      hipLaunchKernelGGL((layer_epilogue_conv_kernel<M, D, C, true>), grid, dim3(256), 0, a.stream, kp, ej.si,
                         ca, ej.items);
    else
      hipLaunchKernelGGL((layer_epilogue_conv_kernel<M, D, C, false>), grid, dim3(256), 0, a.stream, kp,
                         ej.si, ca, ej.items);
  } else {
    if (ej.items > 0) launch_epilogue(ej.si, ej.items);  // the last segment's
    if (conv_state)
      hipLaunchKernelGGL((conv_state_kernel<typename M::in_t, D>), dim3(a.num_seqs * a.H, 3), dim3(D), 0,
                         a.stream, ca, si);
  }
  return hipGetLastError();
}

template <class M, bool SG>
static hipError_t launch_prefill_m(const PrefillArgs& a) {
  if (a.D == 64) {
    if (a.chunk == 16) return launch_prefill_t<M, 64, 16, SG>(a);
    if (a.chunk == 32) return launch_prefill_t<M, 64, 32, SG>(a);
    return launch_prefill_t<M, 64, 64, SG>(a);
  }
  if (a.chunk == 16) return launch_prefill_t<M, 128, 16, SG>(a);
  if (a.chunk == 32) return launch_prefill_t<M, 128, 32, SG>(a);
  return launch_prefill_t<M, 128, 64, SG>(a);
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.scalar_g)
    return a.in_bf16 ? launch_prefill_m<ModeBF16, true>(a) : launch_prefill_m<ModeF32, true>(a);
  return a.in_bf16 ? launch_prefill_m<ModeBF16, false>(a) : launch_prefill_m<ModeF32, false>(a);
}

}  // namespace kda
