// KDA backward pass (gradients of q, k, v, g, beta and the initial state),
// gfx950, fp32 arithmetic.
//
// The pages say the chunkwise algorithm also serves training (greeksharifa
// summary, section 3.1 "Hardware-Efficient Chunkwise Algorithm" and section
// 6.3; zeroshot.it.com deep-dive, section 4) but derive no gradients; the
// steps below are the chain rule applied to the chunk form of the forward
// pass.  For a chunk of C rows (padded with zero inputs: g = 0 keeps the last
// row's cumulative decay equal to the last real token's) entering with state
// S and leaving with S', and Gamma = cumsum(g), gam = exp(Gamma), gam_n =
// exp(Gamma_{C-1}):
//
//   Qt = Q*gam, Kt = K*gam, Kb = K*exp(Gamma_n - Gamma)
//   Bm[r,i] = sum_c k_rc k_ic exp(Gamma_rc - Gamma_ic)   (i < r, exact pairs)
//   P[r,i]  = sum_c q_rc k_ic exp(Gamma_rc - Gamma_ic)   (i <= r)
//   M = (I + Diag(beta) Bm)^{-1},  T = M Diag(beta)
//   R = V - Kt S,  U = T R,  O = Qt S + P U,  S' = Diag(gam_n) S + Kb^T U
//
// and, given dO and dS' (the gradient of the state after the chunk):
//
//   dU = P^T dO + Kb dS',   dR = T^T dU  (= dV),
//   dS = Diag(gam_n) dS' + Qt^T dO - Kt^T dR          (carried backwards)
//   dQt = dO S^T,  dKb = U dS'^T,  dKt = -dR S^T,  dT = dU R^T,
//   dP = tril(dO U^T),  dgam_n = rowsum(dS' * S)
//   dM = dT Diag(beta),  dbeta += colsum(M * dT),
//   dA = strict_tril(-M^T dM M^T),  dbeta += rowsum(dA * Bm),  dBm = Diag(beta) dA
//   then the exact pairwise terms of Bm and P, the decays, and dg as the
//   reverse cumulative sum of dGamma over the chunk.
//
// Decay factorisation.  When the chunk's total decay is moderate (max over
// channels of -Gamma_{C-1} <= 40), exp(Gamma_r - Gamma_i) = gam_r / gam_i
// holds to rounding in fp32, and every pairwise sum is a product with
// Kh = K*exp(-Gamma): Bm = strict_tril(Kt Kh^T), P = tril(Qt Kh^T), and the
// pairwise gradient terms come from Y1 = dBm Kh, Y2 = dP Kh and
// Y3 = dBm^T Kt + dP^T Qt.  Other chunks evaluate every pair with the exact
// exponent of its difference.
//
// Kernels (one launch each, in order):
//   chunk_table_kernel    first global chunk of each packed sequence
//   bwd_prep_kernel       per (chunk, head): padded fp32 copies, Gamma, Qt, Kt,
//                         Kb, Kh and the span verdict
//   fp32_gemm_kernel      batched fp32 products (Grams, contractions over value
//                         columns, pairwise gradient terms)
//   bwd_gram_kernel       per strong-decay (chunk, head): Bm and P pair by pair
//   unit_lower_inverse_kernel per (chunk, head): M = (I + Diag(beta) Bm)^-1, T
//   bwd_fwd_states_kernel per (sequence, head, 16 value columns), serial over
//                         chunks: the entering state S of every chunk, R, U
//   bwd_bwd_states_kernel the same, reverse: dS' of every chunk, dU, dR, dS0
//   bwd_cc_kernel         per (chunk, head): the C x C algebra of M and A
//   bwd_final_fast_kernel per moderate-decay (chunk, head): decays, reverse
//                         cumsum, scatter to the token-major outputs
//   bwd_final_kernel      the same for strong-decay chunks, with the pairwise
//                         gradient terms evaluated pair by pair
#include "kda_device.hpp"
#include "kda_fp32_chunks.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kCols = 16;  // value columns per serial workgroup
constexpr float kSpan = 40.f;  // decay span up to which exp(-Gamma) is factored out

// fp32 planes, each [NB][size] with NB = chunks x heads.
// R, U and dU are dead once the value-column contractions are done and then
// hold Y1, Y2 and Y3.
struct Planes {
  float *Q, *K, *V, *dO, *Gam, *Qt, *Kt, *Kb, *Kh, *R, *U, *dU, *dR, *dQt, *dKb, *dKt;  // [C][D]
  float *P, *Bm, *M, *T, *dP, *dT, *dBm;                                          // [C][C]
  float *S, *dSn;                                                                 // [D][D]
  float *beta, *db;                                                               // [C]
  float *gn;                                                                      // [D]
  int32_t* fast;                                                                  // [1] per (chunk, head)
};

size_t plane_bytes(size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4), dd = a256(NB * D * D * 4);
  return 16 * cd + 7 * cc + 2 * dd + 2 * a256(NB * C * 4) + a256(NB * D * 4) + a256(NB * 4);
}

Planes carve(char* p, size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4), dd = a256(NB * D * D * 4);
  Planes x;
  float** cdp[] = {&x.Q, &x.K, &x.V, &x.dO, &x.Gam, &x.Qt, &x.Kt, &x.Kb, &x.Kh,
                   &x.R, &x.U, &x.dU, &x.dR, &x.dQt, &x.dKb, &x.dKt};
  for (float** f : cdp) { *f = reinterpret_cast<float*>(p); p += cd; }
  float** ccp[] = {&x.P, &x.Bm, &x.M, &x.T, &x.dP, &x.dT, &x.dBm};
  for (float** f : ccp) { *f = reinterpret_cast<float*>(p); p += cc; }
  x.S = reinterpret_cast<float*>(p); p += dd;
  x.dSn = reinterpret_cast<float*>(p); p += dd;
  x.beta = reinterpret_cast<float*>(p); p += a256(NB * C * 4);
  x.db = reinterpret_cast<float*>(p); p += a256(NB * C * 4);
  x.gn = reinterpret_cast<float*>(p);
  p += a256(NB * D * 4);
  x.fast = reinterpret_cast<int32_t*>(p);
  return x;
}

struct BwdIn {
  const void *q, *k, *v;
  const float *g, *beta, *dout;
};

// Padded fp32 copies of the chunk's inputs, Gamma = cumsum(g), Qt, Kt, Kb.
// Four consecutive input elements as fp32.
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Four consecutive channels per thread and item: 16-byte stores of every
// plane; q and k stay in registers between the two passes.
template <class in_t, int D, int C>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdIn in, Planes p, Geo geo) {
  constexpr int SG = D + 4, NV = C * D / 4 / 256;
  static_assert(NV * 256 * 4 == C * D, "whole vectors per thread");
  __shared__ __attribute__((aligned(16))) float G[C][SG];
  const int b = blockIdx.x, H = geo.H;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D;
  const in_t* q = reinterpret_cast<const in_t*>(in.q);
  const in_t* k = reinterpret_cast<const in_t*>(in.k);
  const in_t* v = reinterpret_cast<const in_t*>(in.v);
  f32x4 qv[NV], kv[NV];
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    const int idx = 4 * ((int)threadIdx.x + 256 * x);
    const int r = idx / D, c = idx % D;
    const bool ok = r < len;
    const size_t ti = ((size_t)(t0 + (ok ? r : 0)) * H + h) * D + c;
    const f32x4 z = {0, 0, 0, 0};
    qv[x] = ok ? load4(q + ti) : z;
    kv[x] = ok ? load4(k + ti) : z;
    const f32x4 vv = ok ? load4(v + ti) : z, dv = ok ? load4(in.dout + ti) : z;
    const f32x4 gv = ok ? load4(in.g + ti) : z;
    *reinterpret_cast<f32x4*>(p.Q + pcd + idx) = qv[x];
    *reinterpret_cast<f32x4*>(p.K + pcd + idx) = kv[x];
    *reinterpret_cast<f32x4*>(p.V + pcd + idx) = vv;
    *reinterpret_cast<f32x4*>(p.dO + pcd + idx) = dv;
    *reinterpret_cast<f32x4*>(&G[r][c]) = gv;
  }
  if (threadIdx.x < C) {
    const int r = threadIdx.x;
    p.beta[(size_t)b * C + r] = r < len ? in.beta[(size_t)(t0 + r) * H + h] : 0.f;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float s = 0.f;
    for (int r = 0; r < C; ++r) {
      s += G[r][c];
      G[r][c] = s;
    }
    p.gn[(size_t)b * D + c] = __expf(s);
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // span verdict over all channels (one wave)
    bool big = false;
    for (int c = threadIdx.x; c < D; c += 64) big |= G[C - 1][c] < -kSpan;
    big = __any(big);
    if (threadIdx.x == 0) p.fast[b] = big ? 0 : 1;
  }
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    const int idx = 4 * ((int)threadIdx.x + 256 * x);
    const int r = idx / D, c = idx % D;
    const f32x4 gm = *reinterpret_cast<const f32x4*>(&G[r][c]);
    const f32x4 gl = *reinterpret_cast<const f32x4*>(&G[C - 1][c]);
    f32x4 qt, kt, kb, kh;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ga = __expf(gm[e]);
      qt[e] = qv[x][e] * ga;
      kt[e] = kv[x][e] * ga;
      kb[e] = kv[x][e] * __expf(gl[e] - gm[e]);
      kh[e] = kv[x][e] * __expf(-gm[e]);  // finite where the chunk is factored
    }
    *reinterpret_cast<f32x4*>(p.Gam + pcd + idx) = gm;
    *reinterpret_cast<f32x4*>(p.Qt + pcd + idx) = qt;
    *reinterpret_cast<f32x4*>(p.Kt + pcd + idx) = kt;
    *reinterpret_cast<f32x4*>(p.Kb + pcd + idx) = kb;
    *reinterpret_cast<f32x4*>(p.Kh + pcd + idx) = kh;
  }
}

// Bm (strictly lower) and P (lower) with the exact exponent of every pair,
// for strong-decay chunks.
// Lane = row r; the four waves step through the columns i.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_gram_kernel(Planes p, int NB) {
  extern __shared__ float sm[];
  float* Ks = sm;                  // [C][D + 1]
  float* Qs = Ks + C * (D + 1);
  float* Gs = Qs + C * (D + 1);
  const int b = blockIdx.x;
  if (p.fast[b]) return;  // formed as a product
  const size_t pcd = (size_t)b * C * D;
  for (int idx = threadIdx.x; idx < C * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    Ks[r * (D + 1) + c] = p.K[pcd + idx];
    Qs[r * (D + 1) + c] = p.Q[pcd + idx];
    Gs[r * (D + 1) + c] = p.Gam[pcd + idx];
  }
  __syncthreads();
  const int r = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (r >= C) return;
  const size_t pcc = (size_t)b * C * C;
  for (int i = w; i < C; i += 4) {
    float sb = 0.f, sp = 0.f;
    if (i <= r) {
      for (int c = 0; c < D; ++c) {
        const float e = __expf(Gs[r * (D + 1) + c] - Gs[i * (D + 1) + c]);
        const float ki = Ks[i * (D + 1) + c] * e;
        sb += Ks[r * (D + 1) + c] * ki;
        sp += Qs[r * (D + 1) + c] * ki;
      }
    }
    p.Bm[pcc + r * C + i] = i < r ? sb : 0.f;
    p.P[pcc + r * C + i] = i <= r ? sp : 0.f;
  }
}


template <int D, int C>
struct FwdLds {
  float Kt[C][D + 4];
  float Kb[C][D + 16];
  float T[C][C + 4];
  float S[D][kCols];
  float R[C][kCols];
  float U[C][kCols];
  float V[C][kCols];
  float gn[D];
};

constexpr int kSerThreads = 512;

// Serial forward over a sequence's chunks for 16 value columns: the state
// entering every chunk, R = V - Kt S and U = T R.  Eight waves; the next
// chunk's Kt, Kb, T are loaded into registers while this chunk computes.
template <int D, int C>
__global__ __launch_bounds__(kSerThreads) void bwd_fwd_states_kernel(Planes p, Geo geo,
                                                                     const float* __restrict__ s0) {
  extern __shared__ float sm[];
  FwdLds<D, C>& L = *reinterpret_cast<FwdLds<D, C>*>(sm);
  constexpr int NVB = D / kCols, NT = kSerThreads, NW = NT / 64;
  const int H = geo.H;
  const int vb = blockIdx.x % NVB, nh = blockIdx.x / NVB;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  int bos, eos, base;
  seq_of<C>(geo, n, bos, eos, base);
  const int nch = (eos - bos + C - 1) / C;
  for (int idx = tid; idx < D * kCols; idx += NT) {
    const int i = idx / kCols, j = idx % kCols;
    L.S[i][j] = s0 ? s0[(((size_t)n * H + h) * D + i) * D + col0 + j] : 0.f;
  }
  Prefetch<C, D, NT> pKt, pKb;
  Prefetch<C, C, NT> pT;
  Prefetch<C, kCols, NT, D> pV;  // this workgroup's value columns
  Prefetch<1, D, NT> pG;         // gam_n
  auto blk = [&](int ci) { return (size_t)(base + ci) * H + h; };
  auto fetch = [&](size_t b) {
    pKt.load(p.Kt + b * C * D);
    pKb.load(p.Kb + b * C * D);
    pT.load(p.T + b * C * C);
    pV.load(p.V + b * C * D + col0);
    pG.load(p.gn + b * D);
  };
  if (nch > 0) fetch(blk(0));
  for (int ci = 0; ci < nch; ++ci) {
    const size_t b = blk(ci);
    const size_t pcd = b * C * D;
    __syncthreads();
    pKt.template store<D + 4>(&L.Kt[0][0]);
    pKb.template store<D + 16>(&L.Kb[0][0]);
    pT.template store<C + 4>(&L.T[0][0]);
    pV.template store<kCols>(&L.V[0][0]);
    pG.template store<D>(&L.gn[0]);
    for (int idx = tid; idx < D * kCols; idx += NT) {
      const int i = idx / kCols, j = idx % kCols;
      p.S[(b * D + i) * D + col0 + j] = L.S[i][j];
    }
    __syncthreads();
    if (ci + 1 < nch) fetch(blk(ci + 1));
    for (int rt = w; rt < C / 16; rt += NW) {  // R = V - Kt S
      f32x4 acc = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 8) {
        acc = mfma4(L.Kt[16 * rt + m][k0 + g], L.S[k0 + g][m], acc);
        acc1 = mfma4(L.Kt[16 * rt + m][k0 + 4 + g], L.S[k0 + 4 + g][m], acc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float x = L.V[r][m] - acc[i] - acc1[i];
        L.R[r][m] = x;
        p.R[pcd + r * D + col0 + m] = x;
      }
    }
    __syncthreads();
    for (int rt = w; rt < C / 16; rt += NW) {  // U = T R (T lower triangular)
      f32x4 acc = {0, 0, 0, 0};
      for (int k0 = 0; k0 < 16 * (rt + 1); k0 += 4) acc = mfma4(L.T[16 * rt + m][k0 + g], L.R[k0 + g][m], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        L.U[r][m] = acc[i];
        p.U[pcd + r * D + col0 + m] = acc[i];
      }
    }
    __syncthreads();
    for (int t = w; t < D / 16; t += NW) {  // S = gam_n S + Kb^T U, one tile per wave
      f32x4 acc, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * t + 4 * g + i;
        acc[i] = L.gn[c] * L.S[c][m];
      }
#pragma unroll 8
      for (int k0 = 0; k0 < C; k0 += 8) {
        acc = mfma4(L.Kb[k0 + g][16 * t + m], L.U[k0 + g][m], acc);
        acc1 = mfma4(L.Kb[k0 + 4 + g][16 * t + m], L.U[k0 + 4 + g][m], acc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) L.S[16 * t + 4 * g + i][m] = acc[i] + acc1[i];
    }
  }
}

template <int D, int C>
struct BwdLds {
  union {
    struct {
      float P[C][C + 16];   // read transposed
      float T[C][C + 16];   // read transposed
      float Kb[C][D + 4];
    } a;
    struct {
      float Qt[C][D + 16];  // read transposed
      float Kt[C][D + 16];  // read transposed
    } b;
  } u;
  float X[D][kCols];     // dS'
  float dO[C][kCols];
  float dU[C][kCols];
  float ndR[C][kCols];   // -dR
  float gn[D];
};

// Serial backward over a sequence's chunks for 16 value columns: dS' of
// every chunk, dU = P^T dO + Kb dS', dR = T^T dU, and the carried
// dS = gam_n dS' + Qt^T dO - Kt^T dR; the last one is dS0.  Eight waves; the
// next chunk's P, T, Kb and this chunk's Qt, Kt load while earlier work runs.
template <int D, int C>
__global__ __launch_bounds__(kSerThreads) void bwd_bwd_states_kernel(Planes p, Geo geo,
                                                                     const float* __restrict__ dfin,
                                                                     float* __restrict__ ds0) {
  extern __shared__ float sm[];
  BwdLds<D, C>& L = *reinterpret_cast<BwdLds<D, C>*>(sm);
  constexpr int NVB = D / kCols, NT = kSerThreads, NW = NT / 64;
  const int H = geo.H;
  const int vb = blockIdx.x % NVB, nh = blockIdx.x / NVB;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  int bos, eos, base;
  seq_of<C>(geo, n, bos, eos, base);
  const int nch = (eos - bos + C - 1) / C;
  for (int idx = tid; idx < D * kCols; idx += NT) {
    const int i = idx / kCols, j = idx % kCols;
    L.X[i][j] = dfin ? dfin[(((size_t)n * H + h) * D + i) * D + col0 + j] : 0.f;
  }
  Prefetch<C, C, NT> pP, pT;
  Prefetch<C, D, NT> pKb, pQt, pKt;
  Prefetch<C, kCols, NT, D> pdO;  // this workgroup's value columns
  Prefetch<1, D, NT> pG;          // gam_n
  auto blk = [&](int ci) { return (size_t)(base + ci) * H + h; };
  // P, T, K-bar, dO and gam_n of a chunk load a step ahead, Q*gam and K*gam
  // half a step ahead (after the previous chunk's copies are stored).
  auto fetch_a = [&](size_t b) {
    pP.load(p.P + b * C * C);
    pT.load(p.T + b * C * C);
    pKb.load(p.Kb + b * C * D);
    pdO.load(p.dO + b * C * D + col0);
    pG.load(p.gn + b * D);
  };
  auto fetch_b = [&](size_t b) {
    pQt.load(p.Qt + b * C * D);
    pKt.load(p.Kt + b * C * D);
  };
  if (nch > 0) {
    fetch_a(blk(nch - 1));
    fetch_b(blk(nch - 1));
  }
  for (int ci = nch - 1; ci >= 0; --ci) {
    const size_t b = blk(ci);
    const size_t pcd = b * C * D;
    __syncthreads();
    pP.template store<C + 16>(&L.u.a.P[0][0]);
    pT.template store<C + 16>(&L.u.a.T[0][0]);
    pKb.template store<D + 4>(&L.u.a.Kb[0][0]);
    pdO.template store<kCols>(&L.dO[0][0]);
    pG.template store<D>(&L.gn[0]);
    for (int idx = tid; idx < D * kCols; idx += NT) {
      const int i = idx / kCols, j = idx % kCols;
      p.dSn[(b * D + i) * D + col0 + j] = L.X[i][j];
    }
    __syncthreads();
    if (ci > 0) fetch_a(blk(ci - 1));
    for (int rt = w; rt < C / 16; rt += NW) {  // dU = P^T dO + Kb dS'
      f32x4 acc = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
      for (int k0 = 16 * rt; k0 < C; k0 += 4) acc = mfma4(L.u.a.P[k0 + g][16 * rt + m], L.dO[k0 + g][m], acc);
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 8) {
        acc1 = mfma4(L.u.a.Kb[16 * rt + m][k0 + g], L.X[k0 + g][m], acc1);
        acc = mfma4(L.u.a.Kb[16 * rt + m][k0 + 4 + g], L.X[k0 + 4 + g][m], acc);
      }
      acc += acc1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        L.dU[r][m] = acc[i];
        p.dU[pcd + r * D + col0 + m] = acc[i];
      }
    }
    __syncthreads();
    for (int rt = w; rt < C / 16; rt += NW) {  // dR = T^T dU
      f32x4 acc = {0, 0, 0, 0};
      for (int k0 = 16 * rt; k0 < C; k0 += 4) acc = mfma4(L.u.a.T[k0 + g][16 * rt + m], L.dU[k0 + g][m], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        L.ndR[r][m] = -acc[i];
        p.dR[pcd + r * D + col0 + m] = acc[i];
      }
    }
    __syncthreads();
    pQt.template store<D + 16>(&L.u.b.Qt[0][0]);
    pKt.template store<D + 16>(&L.u.b.Kt[0][0]);
    if (ci > 0) fetch_b(blk(ci - 1));
    __syncthreads();
    for (int t = w; t < D / 16; t += NW) {  // dS = gam_n dS' + Qt^T dO - Kt^T dR
      f32x4 acc, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * t + 4 * g + i;
        acc[i] = L.gn[c] * L.X[c][m];
      }
#pragma unroll 8
      for (int k0 = 0; k0 < C; k0 += 4) {
        acc = mfma4(L.u.b.Qt[k0 + g][16 * t + m], L.dO[k0 + g][m], acc);
        acc1 = mfma4(L.u.b.Kt[k0 + g][16 * t + m], L.ndR[k0 + g][m], acc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) L.X[16 * t + 4 * g + i][m] = acc[i] + acc1[i];
    }
  }
  __syncthreads();
  if (ds0) {
    for (int idx = tid; idx < D * kCols; idx += NT) {
      const int i = idx / kCols, j = idx % kCols;
      ds0[(((size_t)n * H + h) * D + i) * D + col0 + j] = L.X[i][j];
    }
  }
}

// dM = dT Diag(beta); dbeta = colsum(M * dT) + rowsum(dA * Bm) with
// dA = strict_tril(-M^T dM M^T); dBm = Diag(beta) dA.
template <int C>
__global__ __launch_bounds__(256) void bwd_cc_kernel(Planes p) {
  // Both products on v_mfma_f32_16x16x4f32, one 16 x 16 tile per
  // accumulator: wave w owns tiles w, w + 4, ... of the NT x NT grid.  Rows of
  // 68 floats let a lane read four consecutive k in one 16-byte LDS read (lane
  // group g takes k = 4 g .. 4 g + 3 of each block of 16) with the eight lanes
  // served together on distinct banks.
  constexpr int LDC = C + 4, NT = C / 16, TPW = (NT * NT + 3) / 4;
  __shared__ __attribute__((aligned(16))) float Ms[C][LDC];   // M
  __shared__ __attribute__((aligned(16))) float MTs[C][LDC];  // M^T
  __shared__ __attribute__((aligned(16))) float dMs[C][LDC];  // dM = dT Diag(beta), later dA * Bm
  __shared__ __attribute__((aligned(16))) float Xs[C][LDC];   // X = dM M^T
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t pcc = (size_t)b * C * C;
  const float* beta = p.beta + (size_t)b * C;
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    const float m = p.M[pcc + idx];
    Ms[r][i] = m;
    MTs[i][r] = m;
    dMs[r][i] = p.dT[pcc + idx] * beta[i];
  }
  __syncthreads();
  const int w = tid >> 6, l = tid & 63, lm = l & 15, lg = l >> 4;
  f32x4 acc[TPW];
  // X = dM M^T: A[r][l] = dM[r][l], B[l][i] = M[i][l]
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < C; k += 16) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = w + 4 * j;
      if (t < NT * NT) {
        const int r0 = 16 * (t / NT), c0 = 16 * (t % NT);
        const f32x4 a = *reinterpret_cast<const f32x4*>(&dMs[r0 + lm][k + 4 * lg]);
        const f32x4 bq = *reinterpret_cast<const f32x4*>(&Ms[c0 + lm][k + 4 * lg]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j] = mfma4(a[q], bq[q], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = w + 4 * j;
    if (t < NT * NT) {
      const int r0 = 16 * (t / NT), c0 = 16 * (t % NT);
#pragma unroll
      for (int v = 0; v < 4; ++v) Xs[r0 + 4 * lg + v][c0 + lm] = acc[j][v];
    }
  }
  __syncthreads();
  // dA = -M^T X, strictly lower: A[r][l] = M^T[r][l], B[l][i] = X[l][i]
  // (tiles wholly above the diagonal are zero and skip the products)
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < C; k += 16) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = w + 4 * j;
      const int r0 = 16 * (t / NT), c0 = 16 * (t % NT);
      if (t < NT * NT && c0 <= r0) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&MTs[r0 + lm][k + 4 * lg]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j] = mfma4(a[q], Xs[k + 4 * lg + q][c0 + lm], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = w + 4 * j;
    if (t < NT * NT) {
      const int r0 = 16 * (t / NT), c0 = 16 * (t % NT);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = r0 + 4 * lg + v, i = c0 + lm;
        const float sv = i < r ? -acc[j][v] : 0.f;
        p.dBm[pcc + r * C + i] = beta[r] * sv;
        dMs[r][i] = sv * p.Bm[pcc + r * C + i];  // dA * Bm, for the row sums
      }
    }
  }
  __syncthreads();
  if (tid < C) {
    const int j = tid;
    float s = 0.f;
    for (int r = 0; r < C; ++r) s += Ms[r][j] * p.dT[pcc + r * C + j] + dMs[j][r];
    p.db[(size_t)b * C + j] = s;
  }
}

struct BwdOut {
  float *dq, *dk, *dv, *dg, *dbeta;
};

// The pairwise terms of Bm and P, the decays, the reverse cumulative sum of
// dGamma, and the scatter to token-major outputs.  2 D threads: thread c < D
// walks the pairs (r, i <= r) row by row and keeps the row-r terms of channel
// c in registers; thread D + c walks them column by column and keeps the
// row-i terms, which it hands over through LDS (the row-i term of dGamma is
// minus that of dk times k_i).  Each exponent is evaluated by both.
template <int D, int C>
__global__ __launch_bounds__(2 * D) void bwd_final_kernel(Planes p, Geo geo, BwdOut out) {
  extern __shared__ float sm[];
  float* Ks = sm;               // [C][D]
  float* Gs = Ks + C * D;       // [C][D]
  float* Qs = Gs + C * D;       // [C][D]
  float* xK = Qs + C * D;       // [C][D] row-i terms of dk
  float* dBm = xK + C * D;      // [C][C]
  float* dP = dBm + C * C;      // [C][C]
  const int b = blockIdx.x, H = geo.H;
  if (p.fast[b]) return;  // bwd_final_fast_kernel
  const int c = threadIdx.x % D, half = threadIdx.x / D;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D, pcc = (size_t)b * C * C;
  for (int idx = threadIdx.x; idx < C * D; idx += 2 * D) {
    Ks[idx] = p.K[pcd + idx];
    Gs[idx] = p.Gam[pcd + idx];
    Qs[idx] = p.Q[pcd + idx];
  }
  for (int idx = threadIdx.x; idx < C * C; idx += 2 * D) {
    dBm[idx] = p.dBm[pcc + idx];
    dP[idx] = p.dP[pcc + idx];
  }
  __syncthreads();
  if (half == 1) {
    // column i: dk_i += sum_{r >= i} (dBm[r,i] k_r + dP[r,i] q_r) e_ri,
    // dGamma_i -= sum_{r >= i} (dBm[r,i] k_r + dP[r,i] q_r) k_i e_ri
    for (int i = 0; i < C; ++i) {
      const float gi = Gs[i * D + c];
      float ak0 = 0.f, ak1 = 0.f;
      int r = i;
      for (; r + 1 < C; r += 2) {
        ak0 += (dBm[r * C + i] * Ks[r * D + c] + dP[r * C + i] * Qs[r * D + c]) *
               __expf(Gs[r * D + c] - gi);
        ak1 += (dBm[(r + 1) * C + i] * Ks[(r + 1) * D + c] + dP[(r + 1) * C + i] * Qs[(r + 1) * D + c]) *
               __expf(Gs[(r + 1) * D + c] - gi);
      }
      if (r < C) ak0 += (dBm[r * C + i] * Ks[r * D + c] + dP[r * C + i] * Qs[r * D + c]) * __expf(Gs[r * D + c] - gi);
      xK[i * D + c] = ak0 + ak1;
    }
  }
  // Row-r terms go to dk and dg of the token (padded rows carry none), and
  // are completed after the barrier by the same thread.
  float kbsum = 0.f, dgn = 0.f;
  if (half == 0) {
    {
      const float* S = p.S + ((size_t)b * D + c) * D;
      const float* dS = p.dSn + ((size_t)b * D + c) * D;
      for (int j = 0; j < D; ++j) dgn += S[j] * dS[j];
    }
    for (int r = 0; r < C; ++r) {
      const float kr = Ks[r * D + c], qr = Qs[r * D + c], gr = Gs[r * D + c];
      float dkr = 0.f, dqr = 0.f, dgr = 0.f;
      for (int i = 0; i <= r; ++i) {
        const float e = __expf(gr - Gs[i * D + c]);
        const float ki = Ks[i * D + c];
        const float wb = dBm[r * C + i] * e, wp = dP[r * C + i] * e;
        dkr += wb * ki;
        dqr += wp * ki;
        dgr += (wb * kr + wp * qr) * ki;
      }
      const float ga = __expf(gr);
      const size_t e0 = pcd + r * D + c;
      const float dqt = p.dQt[e0], dkt = p.dKt[e0], dkb = p.dKb[e0];
      const float kb = p.Kb[e0];
      kbsum += dkb * kb;
      if (r < len) {
        const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
        out.dq[ti] = dqt * ga + dqr;
        out.dk[ti] = dkr + dkt * ga + dkb * __expf(Gs[(C - 1) * D + c] - gr);
        out.dg[ti] = dgr + dqt * p.Qt[e0] + dkt * p.Kt[e0] - dkb * kb;
      }
    }
  }
  __syncthreads();
  if (half == 0) {
    const float gn = p.gn[(size_t)b * D + c];
    float run = kbsum + dgn * gn;  // dGamma_n lands on the last row
    for (int r = C - 1; r >= 0; --r) {
      run -= xK[r * D + c] * Ks[r * D + c];
      if (r < len) {
        const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
        run += out.dg[ti];
        out.dg[ti] = run;
        out.dk[ti] += xK[r * D + c];
        out.dv[ti] = p.dR[pcd + r * D + c];
      }
    }
    if (c < len) out.dbeta[(size_t)(t0 + c) * H + h] = p.db[(size_t)b * C + c];
  }
}

// Moderate-decay chunks: the pairwise gradient terms are the products
// Y1 = dBm Kh, Y2 = dP Kh, Y3 = dBm^T Kt + dP^T Qt (in the R, U, dU planes):
// dq += gam Y2, dk += gam Y1 + exp(-Gamma) Y3, dGamma += Kt Y1 + Qt Y2 - Kh Y3.
// One thread per channel.
template <int D, int C>
__global__ __launch_bounds__(D) void bwd_final_fast_kernel(Planes p, Geo geo, BwdOut out) {
  const int b = blockIdx.x, c = threadIdx.x, H = geo.H;
  if (!p.fast[b]) return;  // bwd_final_kernel
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D;
  const float* Y1 = p.R + pcd;
  const float* Y2 = p.U + pcd;
  const float* Y3 = p.dU + pcd;
  // dgam_n[c] = rowsum(dS' * S)[c]: each wave reduces whole rows, its lanes
  // reading them contiguously, and parks the sums in LDS.
  __shared__ float rowsum[D];
  {
    constexpr int NWV = D / 64, PL = D / 64;  // waves; elements per lane and row
    const int w = c >> 6, l = c & 63;
    const float* S = p.S + (size_t)b * D * D;
    const float* dS = p.dSn + (size_t)b * D * D;
    for (int i = w; i < D; i += NWV) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < PL; ++e) t += S[(size_t)i * D + 64 * e + l] * dS[(size_t)i * D + 64 * e + l];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
      if (l == 0) rowsum[i] = t;
    }
  }
  float kbsum = 0.f;
#pragma unroll 8
  for (int r = 0; r < C; ++r) kbsum += p.dKb[pcd + r * D + c] * p.Kb[pcd + r * D + c];
  __syncthreads();
  const float dgn = rowsum[c];
  const float gl = p.Gam[pcd + (C - 1) * D + c];
  float run = kbsum + dgn * p.gn[(size_t)b * D + c];  // dGamma_n lands on the last row
#pragma unroll 4
  for (int r = C - 1; r >= 0; --r) {
    const size_t e0 = pcd + r * D + c;
    const float gr = p.Gam[e0], ga = __expf(gr);
    const float dqt = p.dQt[e0], dkt = p.dKt[e0], dkb = p.dKb[e0];
    const float y1 = Y1[r * D + c], y2 = Y2[r * D + c], y3 = Y3[r * D + c];
    run += dqt * p.Qt[e0] + dkt * p.Kt[e0] - dkb * p.Kb[e0] + p.Kt[e0] * y1 + p.Qt[e0] * y2 -
           p.Kh[e0] * y3;
    if (r < len) {
      const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
      out.dq[ti] = (dqt + y2) * ga;
      out.dk[ti] = (dkt + y1) * ga + dkb * __expf(gl - gr) + __expf(-gr) * y3;
      out.dg[ti] = run;
      out.dv[ti] = p.dR[e0];
    }
  }
  if (c < len) out.dbeta[(size_t)(t0 + c) * H + h] = p.db[(size_t)b * C + c];
}

template <int D, int C>
size_t final_lds() { return ((size_t)4 * C * D + 2 * C * C) * sizeof(float); }

template <class in_t, int D, int C>
hipError_t launch_backward_t(const BackwardArgs& a) {
  const size_t NB = (size_t)a.total_chunks * a.H;
  char* ws = reinterpret_cast<char*>(a.workspace);
  Geo geo;
  geo.cu = a.cu_seqlens;
  geo.off = reinterpret_cast<const int32_t*>(ws);
  geo.num_seqs = a.num_seqs;
  geo.seq_len = a.seq_len;
  geo.total_tokens = a.total_tokens;
  geo.H = a.H;
  geo.nchunks = a.total_chunks;
  Planes p = carve(ws + a256(sizeof(int32_t) * (a.num_seqs + 1)), NB, C, D);
  if (a.cu_seqlens)
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens,
                       const_cast<int32_t*>(geo.off), a.num_seqs, a.total_tokens, C);
  const int serial = a.num_seqs * a.H * (D / kCols);
  const size_t flds_s = sizeof(FwdLds<D, C>), blds_s = sizeof(BwdLds<D, C>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_fwd_states_kernel<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)flds_s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_bwd_states_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)blds_s);
  if (e != hipSuccess) return e;
  if (NB == 0) {
    // No tokens: dS0 = dS_N.
    if (a.d_initial_state && serial > 0)
      hipLaunchKernelGGL((bwd_bwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), blds_s, a.stream,
                         p, geo, a.d_final_state, a.d_initial_state);
    return hipGetLastError();
  }
  BwdIn in{a.q, a.k, a.v, a.g, a.beta, a.d_o};
  BwdOut out{a.dq, a.dk, a.dv, a.dg, a.dbeta};
  hipLaunchKernelGGL((bwd_prep_kernel<in_t, D, C>), dim3(NB), dim3(256), 0, a.stream, in, p, geo);
  const size_t glds = (size_t)3 * C * (D + 1) * sizeof(float);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_gram_kernel<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)glds);
  if (e != hipSuccess) return e;
  hipError_t gerr = hipSuccess;
  auto gemm = [&](auto op, const float* A, const float* B, float* Cm, int M, int N, int K,
                  int lda, int ldb, size_t sa, size_t sb, float alpha, int acc_c, int mask) {
    typedef decltype(op) O;
    const hipError_t e = launch_fp32_gemm<O::TA, O::TB>(A, B, Cm, M, N, K, lda, ldb, N, sa, sb,
                                                         (size_t)M * N, alpha, acc_c, mask, NB,
                                                         a.stream);
    if (gerr == hipSuccess) gerr = e;
  };
  const size_t scd = (size_t)C * D, scc = (size_t)C * C, sdd = (size_t)D * D;
  const GemmNT NT;
  const GemmNN NN;
  const GemmTN TN;
  // Grams of the moderate-decay chunks, then the others pair by pair.
  gemm(NT, p.Kt, p.Kh, p.Bm, C, C, D, D, D, scd, scd, 1.f, 0, 2);  // strict_tril(Kt Kh^T)
  gemm(NT, p.Qt, p.Kh, p.P, C, C, D, D, D, scd, scd, 1.f, 0, 1);   // tril(Qt Kh^T)
  hipLaunchKernelGGL((bwd_gram_kernel<D, C>), dim3(NB), dim3(256), glds, a.stream, p, (int)NB);
  hipLaunchKernelGGL((unit_lower_inverse_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p.Bm, p.beta,
                     p.M, p.T);
  hipLaunchKernelGGL((bwd_fwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), flds_s, a.stream, p,
                     geo, a.initial_state);
  hipLaunchKernelGGL((bwd_bwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), blds_s, a.stream, p,
                     geo, a.d_final_state, a.d_initial_state);
  // p.S and p.dSn are [D][D] per chunk and head: the B operand "rows" are the
  // key channels, contracted over the value columns.
  gemm(NT, p.dO, p.S, p.dQt, C, D, D, D, D, scd, sdd, 1.f, 0, 0);   // dQt = dO S^T
  gemm(NT, p.U, p.dSn, p.dKb, C, D, D, D, D, scd, sdd, 1.f, 0, 0);  // dKb = U dS'^T
  gemm(NT, p.dR, p.S, p.dKt, C, D, D, D, D, scd, sdd, -1.f, 0, 0);  // dKt = -dR S^T
  gemm(NT, p.dU, p.R, p.dT, C, C, D, D, D, scd, scd, 1.f, 0, 0);    // dT = dU R^T
  gemm(NT, p.dO, p.U, p.dP, C, C, D, D, D, scd, scd, 1.f, 0, 1);    // dP = tril(dO U^T)
  hipLaunchKernelGGL((bwd_cc_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p);
  // Pairwise gradient terms of the moderate-decay chunks (R, U, dU are free).
  gemm(NN, p.dBm, p.Kh, p.R, C, D, C, C, D, scc, scd, 1.f, 0, 0);   // Y1 = dBm Kh
  gemm(NN, p.dP, p.Kh, p.U, C, D, C, C, D, scc, scd, 1.f, 0, 0);    // Y2 = dP Kh
  gemm(TN, p.dBm, p.Kt, p.dU, C, D, C, C, D, scc, scd, 1.f, 0, 0);  // Y3 = dBm^T Kt
  gemm(TN, p.dP, p.Qt, p.dU, C, D, C, C, D, scc, scd, 1.f, 1, 0);   //    + dP^T Qt
  if (gerr != hipSuccess) return gerr;
  hipLaunchKernelGGL((bwd_final_fast_kernel<D, C>), dim3(NB), dim3(D), 0, a.stream, p, geo, out);
  const size_t flds = final_lds<D, C>();
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_final_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)flds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_final_kernel<D, C>), dim3(NB), dim3(2 * D), flds, a.stream, p, geo, out);
  return hipGetLastError();
}

template <class in_t>
hipError_t launch_backward_i(const BackwardArgs& a) {
  if (a.D == 64) {
    if (a.chunk == 16) return launch_backward_t<in_t, 64, 16>(a);
    if (a.chunk == 32) return launch_backward_t<in_t, 64, 32>(a);
    return launch_backward_t<in_t, 64, 64>(a);
  }
  if (a.chunk == 16) return launch_backward_t<in_t, 128, 16>(a);
  if (a.chunk == 32) return launch_backward_t<in_t, 128, 32>(a);
  return launch_backward_t<in_t, 128, 64>(a);
}

}  // namespace

size_t backward_workspace_bytes(long long total_chunks, int num_seqs, int H, int D, int chunk) {
  return a256(sizeof(int32_t) * (size_t)(num_seqs + 1)) +
         plane_bytes((size_t)total_chunks * H, chunk, D);
}

hipError_t launch_backward(const BackwardArgs& a) {
  return a.in_bf16 ? launch_backward_i<bf16>(a) : launch_backward_i<float>(a);
}

}  // namespace kda
