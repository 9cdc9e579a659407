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
// Kernels (one launch each, in order):
//   bwd_table_kernel      first global chunk of each packed sequence
//   bwd_prep_kernel       per (chunk, head): padded fp32 copies, Gamma, Qt, Kt, Kb
//   bwd_gram_kernel       per (chunk, head): Bm and P pair by pair (exact exps)
//   bwd_solve_kernel      per (chunk, head): M by forward substitution, T
//   bwd_fwd_states_kernel per (sequence, head, 16 value columns), serial over
//                         chunks: the entering state S of every chunk, R, U
//   bwd_bwd_states_kernel the same, reverse: dS' of every chunk, dU, dR, dS0
//   bwd_nt_gemm_kernel    batched fp32 products over value columns
//   bwd_cc_kernel         per (chunk, head): the C x C algebra of M and A
//   bwd_final_kernel      per (chunk, head): pairwise gradients, decays,
//                         reverse cumsum, scatter to the token-major outputs
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kCols = 16;  // value columns per serial workgroup

// fp32 planes, each [NB][size] with NB = chunks x heads.
struct Planes {
  float *Q, *K, *V, *dO, *Gam, *Qt, *Kt, *Kb, *R, *U, *dU, *dR, *dQt, *dKb, *dKt;  // [C][D]
  float *P, *Bm, *M, *T, *dP, *dT, *dBm;                                          // [C][C]
  float *S, *dSn;                                                                 // [D][D]
  float *beta, *db;                                                               // [C]
  float *gn;                                                                      // [D]
};

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

size_t plane_bytes(size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4), dd = a256(NB * D * D * 4);
  return 15 * cd + 7 * cc + 2 * dd + 2 * a256(NB * C * 4) + a256(NB * D * 4);
}

Planes carve(char* p, size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4), dd = a256(NB * D * D * 4);
  Planes x;
  float** cdp[] = {&x.Q, &x.K, &x.V, &x.dO, &x.Gam, &x.Qt, &x.Kt, &x.Kb,
                   &x.R, &x.U, &x.dU, &x.dR, &x.dQt, &x.dKb, &x.dKt};
  for (float** f : cdp) { *f = reinterpret_cast<float*>(p); p += cd; }
  float** ccp[] = {&x.P, &x.Bm, &x.M, &x.T, &x.dP, &x.dT, &x.dBm};
  for (float** f : ccp) { *f = reinterpret_cast<float*>(p); p += cc; }
  x.S = reinterpret_cast<float*>(p); p += dd;
  x.dSn = reinterpret_cast<float*>(p); p += dd;
  x.beta = reinterpret_cast<float*>(p); p += a256(NB * C * 4);
  x.db = reinterpret_cast<float*>(p); p += a256(NB * C * 4);
  x.gn = reinterpret_cast<float*>(p);
  return x;
}

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
__global__ __launch_bounds__(1024) void bwd_table_kernel(const int32_t* __restrict__ cu,
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

struct BwdIn {
  const void *q, *k, *v;
  const float *g, *beta, *dout;
};

// Padded fp32 copies of the chunk's inputs, Gamma = cumsum(g), Qt, Kt, Kb.
template <class in_t, int D, int C>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdIn in, Planes p, Geo geo) {
  __shared__ float G[C][D + 1];
  const int b = blockIdx.x, H = geo.H;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D;
  const in_t* q = reinterpret_cast<const in_t*>(in.q);
  const in_t* k = reinterpret_cast<const in_t*>(in.k);
  const in_t* v = reinterpret_cast<const in_t*>(in.v);
  for (int idx = threadIdx.x; idx < C * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    const bool ok = r < len;
    const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
    p.Q[pcd + idx] = ok ? (float)q[ti] : 0.f;
    p.K[pcd + idx] = ok ? (float)k[ti] : 0.f;
    p.V[pcd + idx] = ok ? (float)v[ti] : 0.f;
    p.dO[pcd + idx] = ok ? in.dout[ti] : 0.f;
    G[r][c] = ok ? in.g[ti] : 0.f;
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
  for (int idx = threadIdx.x; idx < C * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    const float gm = G[r][c], ga = __expf(gm);
    const float kv = p.K[pcd + idx];
    p.Gam[pcd + idx] = gm;
    p.Qt[pcd + idx] = p.Q[pcd + idx] * ga;
    p.Kt[pcd + idx] = kv * ga;
    p.Kb[pcd + idx] = kv * __expf(G[C - 1][c] - gm);
  }
}

// Bm (strictly lower) and P (lower) with the exact exponent of every pair.
// Lane = row r; the four waves step through the columns i.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_gram_kernel(Planes p, int NB) {
  extern __shared__ float sm[];
  float* Ks = sm;                  // [C][D + 1]
  float* Qs = Ks + C * (D + 1);
  float* Gs = Qs + C * (D + 1);
  const int b = blockIdx.x;
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

// M = (I + Diag(beta) Bm)^{-1} by forward substitution, one column per
// thread; T = M Diag(beta).
template <int C>
__global__ __launch_bounds__(64) void bwd_solve_kernel(Planes p) {
  __shared__ float A[C][C + 1];
  __shared__ float X[C][C + 1];
  const int b = blockIdx.x, j = threadIdx.x;
  const size_t pcc = (size_t)b * C * C;
  const float* beta = p.beta + (size_t)b * C;
  for (int idx = j; idx < C * C; idx += 64) {
    const int r = idx / C, i = idx % C;
    A[r][i] = beta[r] * p.Bm[pcc + idx];
  }
  __syncthreads();
  if (j < C) {
    for (int i = 0; i < C; ++i) {
      float s = i == j ? 1.f : 0.f;
      for (int l = j; l < i; ++l) s -= A[i][l] * X[l][j];
      X[i][j] = i < j ? 0.f : s;
    }
  }
  __syncthreads();
  for (int idx = j; idx < C * C; idx += 64) {
    const int r = idx / C, i = idx % C;
    p.M[pcc + idx] = X[r][i];
    p.T[pcc + idx] = X[r][i] * beta[i];
  }
}

// Serial forward over a sequence's chunks for 16 value columns: the state
// entering every chunk, R = V - Kt S and U = T R.
template <int D, int C>
struct FwdLds {
  float Ks[C][D + 1];  // Kt, then Kb
  float Ts[C][C + 1];
  float Ss[D][kCols + 1];
  float Rs[C][kCols + 1];
  float Us[C][kCols + 1];
};

template <int D, int C>
__global__ __launch_bounds__(256) void bwd_fwd_states_kernel(Planes p, Geo geo,
                                                             const float* __restrict__ s0) {
  extern __shared__ float sm[];
  FwdLds<D, C>& L = *reinterpret_cast<FwdLds<D, C>*>(sm);
  auto& Ks = L.Ks;
  auto& Ts = L.Ts;
  auto& Ss = L.Ss;
  auto& Rs = L.Rs;
  auto& Us = L.Us;
  constexpr int NVB = D / kCols;
  const int H = geo.H;
  const int blk = blockIdx.x;
  const int vb = blk % NVB, nh = blk / NVB;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x;
  int bos, eos, base;
  seq_of<C>(geo, n, bos, eos, base);
  const int nch = (eos - bos + C - 1) / C;
  for (int idx = tid; idx < D * kCols; idx += 256) {
    const int i = idx / kCols, j = idx % kCols;
    Ss[i][j] = s0 ? s0[(((size_t)n * H + h) * D + i) * D + col0 + j] : 0.f;
  }
  for (int ci = 0; ci < nch; ++ci) {
    const size_t b = (size_t)(base + ci) * H + h;
    const size_t pcd = b * C * D, pcc = b * C * C;
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += 256) Ks[idx / D][idx % D] = p.Kt[pcd + idx];
    for (int idx = tid; idx < C * C; idx += 256) Ts[idx / C][idx % C] = p.T[pcc + idx];
    for (int idx = tid; idx < D * kCols; idx += 256) {
      const int i = idx / kCols, j = idx % kCols;
      p.S[(b * D + i) * D + col0 + j] = Ss[i][j];
    }
    __syncthreads();
    for (int idx = tid; idx < C * kCols; idx += 256) {  // R = V - Kt S
      const int r = idx / kCols, j = idx % kCols;
      float s = p.V[pcd + r * D + col0 + j];
      for (int c = 0; c < D; ++c) s -= Ks[r][c] * Ss[c][j];
      Rs[r][j] = s;
      p.R[pcd + r * D + col0 + j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * kCols; idx += 256) {  // U = T R
      const int r = idx / kCols, j = idx % kCols;
      float s = 0.f;
      for (int i = 0; i <= r; ++i) s += Ts[r][i] * Rs[i][j];
      Us[r][j] = s;
      p.U[pcd + r * D + col0 + j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += 256) Ks[idx / D][idx % D] = p.Kb[pcd + idx];
    __syncthreads();
    for (int idx = tid; idx < D * kCols; idx += 256) {  // S = gam_n S + Kb^T U
      const int c = idx / kCols, j = idx % kCols;
      float s = p.gn[b * D + c] * Ss[c][j];
      for (int r = 0; r < C; ++r) s += Ks[r][c] * Us[r][j];
      Ss[c][j] = s;  // each (c, j) read and written by this thread only
    }
  }
}

// Serial backward over a sequence's chunks for 16 value columns: dS' of
// every chunk, dU = P^T dO + Kb dS', dR = T^T dU, and the carried
// dS = gam_n dS' + Qt^T dO - Kt^T dR; the last one is dS0.
template <int D, int C>
struct BwdLds {
  float Xs[C][D + 1];  // Kb, then Qt
  float Ys[C][D + 1];  // Kt
  float Ps[C][C + 1];
  float Ts[C][C + 1];
  float Ds[D][kCols + 1];
  float Os[C][kCols + 1];
  float dUs[C][kCols + 1];
  float dRs[C][kCols + 1];
};

template <int D, int C>
__global__ __launch_bounds__(256) void bwd_bwd_states_kernel(Planes p, Geo geo,
                                                             const float* __restrict__ dfin,
                                                             float* __restrict__ ds0) {
  extern __shared__ float sm[];
  BwdLds<D, C>& L = *reinterpret_cast<BwdLds<D, C>*>(sm);
  auto& Xs = L.Xs;
  auto& Ys = L.Ys;
  auto& Ps = L.Ps;
  auto& Ts = L.Ts;
  auto& Ds = L.Ds;
  auto& Os = L.Os;
  auto& dUs = L.dUs;
  auto& dRs = L.dRs;
  constexpr int NVB = D / kCols;
  const int H = geo.H;
  const int blk = blockIdx.x;
  const int vb = blk % NVB, nh = blk / NVB;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x;
  int bos, eos, base;
  seq_of<C>(geo, n, bos, eos, base);
  const int nch = (eos - bos + C - 1) / C;
  for (int idx = tid; idx < D * kCols; idx += 256) {
    const int i = idx / kCols, j = idx % kCols;
    Ds[i][j] = dfin ? dfin[(((size_t)n * H + h) * D + i) * D + col0 + j] : 0.f;
  }
  for (int ci = nch - 1; ci >= 0; --ci) {
    const size_t b = (size_t)(base + ci) * H + h;
    const size_t pcd = b * C * D, pcc = b * C * C;
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += 256) Xs[idx / D][idx % D] = p.Kb[pcd + idx];
    for (int idx = tid; idx < C * C; idx += 256) {
      Ps[idx / C][idx % C] = p.P[pcc + idx];
      Ts[idx / C][idx % C] = p.T[pcc + idx];
    }
    for (int idx = tid; idx < C * kCols; idx += 256) {
      const int r = idx / kCols, j = idx % kCols;
      Os[r][j] = p.dO[pcd + r * D + col0 + j];
    }
    for (int idx = tid; idx < D * kCols; idx += 256) {
      const int i = idx / kCols, j = idx % kCols;
      p.dSn[(b * D + i) * D + col0 + j] = Ds[i][j];
    }
    __syncthreads();
    for (int idx = tid; idx < C * kCols; idx += 256) {  // dU = P^T dO + Kb dS'
      const int r = idx / kCols, j = idx % kCols;
      float s = 0.f;
      for (int i = r; i < C; ++i) s += Ps[i][r] * Os[i][j];
      for (int c = 0; c < D; ++c) s += Xs[r][c] * Ds[c][j];
      dUs[r][j] = s;
      p.dU[pcd + r * D + col0 + j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * kCols; idx += 256) {  // dR = T^T dU
      const int r = idx / kCols, j = idx % kCols;
      float s = 0.f;
      for (int i = r; i < C; ++i) s += Ts[i][r] * dUs[i][j];
      dRs[r][j] = s;
      p.dR[pcd + r * D + col0 + j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += 256) {
      Xs[idx / D][idx % D] = p.Qt[pcd + idx];
      Ys[idx / D][idx % D] = p.Kt[pcd + idx];
    }
    __syncthreads();
    for (int idx = tid; idx < D * kCols; idx += 256) {  // dS = gam_n dS' + Qt^T dO - Kt^T dR
      const int c = idx / kCols, j = idx % kCols;
      float s = p.gn[b * D + c] * Ds[c][j];
      for (int r = 0; r < C; ++r) s += Xs[r][c] * Os[r][j] - Ys[r][c] * dRs[r][j];
      Ds[c][j] = s;
    }
  }
  __syncthreads();
  if (ds0) {
    for (int idx = tid; idx < D * kCols; idx += 256) {
      const int i = idx / kCols, j = idx % kCols;
      ds0[(((size_t)n * H + h) * D + i) * D + col0 + j] = Ds[i][j];
    }
  }
}

// Batched C = alpha * A B^T (row-major A [M][K], B [N][K], C [M][N]) with an
// optional lower-triangular mask on C.  64 x 64 tile, 256 threads, 4 x 4
// outputs each; M, N, K multiples of 16.
__global__ __launch_bounds__(256) void bwd_nt_gemm_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ B,
                                                          float* __restrict__ Cm, int M, int N,
                                                          int K, size_t sa, size_t sb, size_t sc,
                                                          float alpha, int lower) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int bt = blockIdx.x;  // batch on x: up to 2^31 - 1 blocks
  const int m0 = blockIdx.z * 64, n0 = blockIdx.y * 64;
  const float* a = A + bt * sa;
  const float* bb = B + bt * sb;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
      const int rr = idx / 16, kk = idx % 16;
      As[kk][rr] = m0 + rr < M ? a[(size_t)(m0 + rr) * K + k0 + kk] : 0.f;
      Bs[kk][rr] = n0 + rr < N ? bb[(size_t)(n0 + rr) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        av[x] = As[kk][ty * 4 + x];
        bv[x] = Bs[kk][tx * 4 + x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += av[x] * bv[y];
    }
    __syncthreads();
  }
  float* c = Cm + bt * sc;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int m = m0 + ty * 4 + x, nn = n0 + tx * 4 + y;
      if (m < M && nn < N) c[(size_t)m * N + nn] = (lower && nn > m) ? 0.f : alpha * acc[x][y];
    }
}

// dM = dT Diag(beta); dbeta = colsum(M * dT) + rowsum(dA * Bm) with
// dA = strict_tril(-M^T dM M^T); dBm = Diag(beta) dA.
template <int C>
__global__ __launch_bounds__(256) void bwd_cc_kernel(Planes p) {
  __shared__ float Ms[C][C + 1];
  __shared__ float dMs[C][C + 1];
  __shared__ float Xs[C][C + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t pcc = (size_t)b * C * C;
  const float* beta = p.beta + (size_t)b * C;
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    Ms[r][i] = p.M[pcc + idx];
    dMs[r][i] = p.dT[pcc + idx] * beta[i];
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += 256) {  // X = dM M^T
    const int r = idx / C, i = idx % C;
    float s = 0.f;
    for (int l = 0; l < C; ++l) s += dMs[r][l] * Ms[i][l];
    Xs[r][i] = s;
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += 256) {  // dA = -M^T X, strictly lower
    const int r = idx / C, i = idx % C;
    float s = 0.f;
    if (i < r)
      for (int l = 0; l < C; ++l) s -= Ms[l][r] * Xs[l][i];
    p.dBm[pcc + idx] = beta[r] * s;
    dMs[r][i] = s * p.Bm[pcc + idx];  // dA * Bm, for the row sums
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

// One thread per channel c: the pairwise terms of Bm and P (row-i parts
// accumulated in this thread's own LDS column), the decays, the reverse
// cumulative sum of dGamma, and the scatter to token-major outputs.
template <int D, int C>
__global__ __launch_bounds__(D) void bwd_final_kernel(Planes p, Geo geo, BwdOut out) {
  extern __shared__ float sm[];
  float* Ks = sm;               // [C][D]
  float* Gs = Ks + C * D;       // [C][D]
  float* aK = Gs + C * D;       // [C][D] row-i terms of dk
  float* aG = aK + C * D;       // [C][D] row-i terms of dGamma
  const int b = blockIdx.x, c = threadIdx.x, H = geo.H;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D, pcc = (size_t)b * C * C;
  for (int r = 0; r < C; ++r) {
    Ks[r * D + c] = p.K[pcd + r * D + c];
    Gs[r * D + c] = p.Gam[pcd + r * D + c];
    aK[r * D + c] = 0.f;
    aG[r * D + c] = 0.f;
  }
  const float* dBm = p.dBm + pcc;
  const float* dP = p.dP + pcc;
  const float gn = p.gn[(size_t)b * D + c];
  float dgn = 0.f;  // rowsum(dS' * S) for channel c
  {
    const float* S = p.S + ((size_t)b * D + c) * D;
    const float* dS = p.dSn + ((size_t)b * D + c) * D;
    for (int j = 0; j < D; ++j) dgn += S[j] * dS[j];
  }
  float kbsum = 0.f;  // sum_r dKb * Kb
  for (int r = 0; r < C; ++r) {
    const float kr = Ks[r * D + c], qr = p.Q[pcd + r * D + c], gr = Gs[r * D + c];
    float dkr = 0.f, dqr = 0.f, dgr = 0.f;
    for (int i = 0; i <= r; ++i) {
      const float e = __expf(gr - Gs[i * D + c]);
      const float ki = Ks[i * D + c];
      const float wb = dBm[r * C + i] * e, wp = dP[r * C + i] * e;
      dkr += wb * ki;
      dqr += wp * ki;
      const float t = wb * kr + wp * qr;
      aK[i * D + c] += t;
      const float z = t * ki;
      dgr += z;
      aG[i * D + c] -= z;
    }
    const float ga = __expf(gr);
    const size_t e0 = pcd + r * D + c;
    const float dqt = p.dQt[e0], dkt = p.dKt[e0], dkb = p.dKb[e0];
    const float kb = p.Kb[e0];
    kbsum += dkb * kb;
    aK[r * D + c] += dkr + dkt * ga + dkb * __expf(Gs[(C - 1) * D + c] - gr);
    aG[r * D + c] += dgr + dqt * p.Qt[e0] + dkt * p.Kt[e0] - dkb * kb;
    if (r < len) out.dq[((size_t)(t0 + r) * H + h) * D + c] = dqt * ga + dqr;
  }
  aG[(C - 1) * D + c] += kbsum + dgn * gn;
  float run = 0.f;
  for (int r = C - 1; r >= 0; --r) {
    run += aG[r * D + c];
    if (r < len) {
      const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
      out.dg[ti] = run;
      out.dk[ti] = aK[r * D + c];
      out.dv[ti] = p.dR[pcd + r * D + c];
    }
  }
  if (c < len) out.dbeta[(size_t)(t0 + c) * H + h] = p.db[(size_t)b * C + c];
}

template <int D, int C>
size_t final_lds() { return (size_t)4 * C * D * sizeof(float); }

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
    hipLaunchKernelGGL(bwd_table_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens,
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
      hipLaunchKernelGGL((bwd_bwd_states_kernel<D, C>), dim3(serial), dim3(256), blds_s, a.stream,
                         p, geo, a.d_final_state, a.d_initial_state);
    return hipGetLastError();
  }
  BwdIn in{a.q, a.k, a.v, a.g, a.beta, a.d_o};
  hipLaunchKernelGGL((bwd_prep_kernel<in_t, D, C>), dim3(NB), dim3(256), 0, a.stream, in, p, geo);
  const size_t glds = (size_t)3 * C * (D + 1) * sizeof(float);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_gram_kernel<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)glds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_gram_kernel<D, C>), dim3(NB), dim3(256), glds, a.stream, p, (int)NB);
  hipLaunchKernelGGL((bwd_solve_kernel<C>), dim3(NB), dim3(64), 0, a.stream, p);
  hipLaunchKernelGGL((bwd_fwd_states_kernel<D, C>), dim3(serial), dim3(256), flds_s, a.stream, p,
                     geo, a.initial_state);
  hipLaunchKernelGGL((bwd_bwd_states_kernel<D, C>), dim3(serial), dim3(256), blds_s, a.stream, p,
                     geo, a.d_final_state, a.d_initial_state);
  auto gemm = [&](const float* A, const float* B, float* Cm, int M, int N, float alpha,
                  int lower) {
    const dim3 grid((unsigned)NB, (N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(bwd_nt_gemm_kernel, grid, dim3(256), 0, a.stream, A, B, Cm, M, N, D,
                       (size_t)M * D, (size_t)N * D, (size_t)M * N, alpha, lower);
  };
  // p.S and p.dSn are [D][D] per chunk and head: the B operand "rows" are the
  // key channels, contracted over the value columns.
  gemm(p.dO, p.S, p.dQt, C, D, 1.f, 0);    // dQt = dO S^T
  gemm(p.U, p.dSn, p.dKb, C, D, 1.f, 0);   // dKb = U dS'^T
  gemm(p.dR, p.S, p.dKt, C, D, -1.f, 0);   // dKt = -dR S^T
  gemm(p.dU, p.R, p.dT, C, C, 1.f, 0);     // dT = dU R^T
  gemm(p.dO, p.U, p.dP, C, C, 1.f, 1);     // dP = tril(dO U^T)
  hipLaunchKernelGGL((bwd_cc_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p);
  const size_t flds = final_lds<D, C>();
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_final_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)flds);
  if (e != hipSuccess) return e;
  BwdOut out{a.dq, a.dk, a.dv, a.dg, a.dbeta};
  hipLaunchKernelGGL((bwd_final_kernel<D, C>), dim3(NB), dim3(D), flds, a.stream, p, geo, out);
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
