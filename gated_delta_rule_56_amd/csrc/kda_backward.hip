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
// Y3 = dBm^T Kt + dP^T Qt.  Other chunks are factored per 16-row tile, with
// one per-channel factor bridging each pair of tiles (see
// bwd_gram_tile_kernel), still on the matrix units.
//
// Kernels (one launch each, in order):
//   chunk_table_kernel    first global chunk of each packed sequence
//   bwd_prep_kernel       per (chunk, head): padded fp32 copies, Gamma, Qt, Kt,
//                         Kb, Kh and the span verdict
//   fp32_gemm_kernel      batched fp32 products (Grams, contractions over value
//                         columns)
//   bwd_gram_tile_kernel  per strong-decay (chunk, head): Bm and P, tile-factored
//   unit_lower_inverse_kernel per (chunk, head): M = (I + Diag(beta) Bm)^-1, T
//   bwd_fwd_states_kernel per (sequence, head, 16 value columns), serial over
//                         chunks: the entering state S of every chunk, R, U
//   bwd_bwd_states_kernel the same, reverse: dS' of every chunk, dU, dR, dS0
//   bwd_cc_kernel         per (chunk, head): the C x C algebra of M and A
//   bwd_pairs_tile_kernel per strong-decay (chunk, head): the pairwise
//                         gradient terms, tile-factored
//   bwd_final_prod_kernel per (chunk, head, 64 channels): the pairwise
//                         gradient terms of the factored chunks, decays,
//                         reverse cumsum, scatter to the token-major outputs
#include <type_traits>

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
  float *dgp;  // [D/16][D]: rowsum(dS' * S) over each serial workgroup's 16 value columns
  int32_t* fast;                                                                  // [1] per (chunk, head)
};

size_t plane_bytes(size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4), dd = a256(NB * D * D * 4);
  return 16 * cd + 7 * cc + 2 * dd + 2 * a256(NB * C * 4) + a256(NB * D * 4) + a256(NB * (D / 16) * D * 4) +
         a256(NB * 4);
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
  x.dgp = reinterpret_cast<float*>(p);
  p += a256(NB * (D / 16) * D * 4);
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
  // Inputs are loaded unconditionally (rows past the chunk re-read its first
  // row) and zeroed after, and each vector's loads are issued before the
  // previous vector's stores: a load under the row test made every one wait
  // for the last, and the compiler may not move a load above a store that
  // could alias it.
  f32x4 qv[NV], kv[NV], vr[2], dr[2], gr[2];
  auto fetch = [&](int x) {
    const int idx = 4 * ((int)threadIdx.x + 256 * x), r = idx / D, c = idx % D;
    const size_t ti = ((size_t)(t0 + (r < len ? r : 0)) * H + h) * D + c;
    qv[x] = load4(q + ti);
    kv[x] = load4(k + ti);
    vr[x & 1] = load4(v + ti);
    dr[x & 1] = load4(in.dout + ti);
    gr[x & 1] = load4(in.g + ti);
  };
  fetch(0);
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    if (x + 1 < NV) fetch(x + 1);
    const int idx = 4 * ((int)threadIdx.x + 256 * x);
    const int r = idx / D, c = idx % D;
    const bool ok = r < len;
    const f32x4 z = {0, 0, 0, 0};
    qv[x] = ok ? qv[x] : z;
    kv[x] = ok ? kv[x] : z;
    const f32x4 vv = ok ? vr[x & 1] : z, dv = ok ? dr[x & 1] : z;
    const f32x4 gv = ok ? gr[x & 1] : z;
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

// Strong-decay chunks (span > kSpan) are factored per 16-row tile, as the
// forward prefill does.  With Gamma_s(a) the cumulative decay before tile a
// and Gamma_e(b) at the end of tile b, for rows r of tile a and columns i of
// tile b <= a,
//   exp(Gamma_r - Gamma_i) = exp(Gamma_r - Gamma_s(a)) f_ab exp(Gamma_e(b) - Gamma_i),
//   f_ab = exp(Gamma_s(a) - Gamma_e(b)),
// all three factors <= 1 off the diagonal; on the diagonal f_aa =
// exp(-(span of tile a)) >= 1, which stays in range up to a tile span of
// kTileSpan; a diagonal block beyond that is summed pair by pair with the
// exact exponent.  The tile operands, in LDS:
//   Kr, Qr  rows scaled by exp(Gamma_r - Gamma_s(a))   [C][D + 4]
//   Kc      K scaled by exp(Gamma_e(b) - Gamma_i)      [C][D + 4]
constexpr float kTileSpan = 64.f;

template <int D, int C>
struct TileLds {
  static constexpr int NT = C / 16, SD = D + 4, SC = C + 4;
  float Kr[C][SD], Qr[C][SD], Kc[C][SD];
  float Gs[NT][D], Ge[NT][D];  // Gamma before tile t and at its end
  float dBm[C][SC], dP[C][SC];  // the final stage only
};

// The tile operands of item b, and whether each diagonal tile spans more
// than kTileSpan on some channel (bad[t], wave-uniform after the barrier).
template <int D, int C, bool PAIRS = false>
__device__ __forceinline__ void tile_operands(const Planes& p, size_t b, TileLds<D, C>& L, bool* bad) {
  constexpr int NT = C / 16, NI = C * D / 256, NG = (NT * D + 255) / 256, NCC = PAIRS ? C * C / 256 : 0;
  static_assert(NI * 256 == C * D && (!PAIRS || NCC * 256 == C * C), "whole elements per thread");
  const size_t pcd = b * C * D, pcc = b * C * C;
  const int tid = threadIdx.x;
  // Every global load first (a loop that waited for each element's loads
  // before its LDS writes took most of these kernels' time): Gamma, K, Q of
  // the thread's elements, Gamma before and at the end of each tile, and
  // (PAIRS) dBm and dP.
  float gv[NI], kv[NI], qv[NI], gsv[NG], gev[NG], bmv[NCC > 0 ? NCC : 1], dpv[NCC > 0 ? NCC : 1];
#pragma unroll
  for (int x = 0; x < NI; ++x) {
    const size_t e = pcd + tid + 256 * x;
    gv[x] = p.Gam[e];
    kv[x] = p.K[e];
    qv[x] = p.Q[e];
  }
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    const int idx = min(tid + 256 * x, NT * D - 1), t = idx / D, c = idx % D;
    gsv[x] = p.Gam[pcd + (size_t)(t == 0 ? 0 : 16 * t - 1) * D + c];
    gev[x] = p.Gam[pcd + (size_t)(16 * t + 15) * D + c];
  }
#pragma unroll
  for (int x = 0; x < NCC; ++x) {
    bmv[x] = p.dBm[pcc + tid + 256 * x];
    dpv[x] = p.dP[pcc + tid + 256 * x];
  }
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    const int idx = tid + 256 * x, t = idx / D, c = idx % D;
    if (NT * D % 256 == 0 || idx < NT * D) {
      L.Gs[t][c] = t == 0 ? 0.f : gsv[x];
      L.Ge[t][c] = gev[x];
    }
  }
  if constexpr (PAIRS) {
#pragma unroll
    for (int x = 0; x < NCC; ++x) {
      const int idx = tid + 256 * x, r = idx / C, i = idx % C;
      L.dBm[r][i] = bmv[x];
      L.dP[r][i] = dpv[x];
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NI; ++x) {
    const int idx = tid + 256 * x, r = idx / D, c = idx % D, t = r / 16;
    const float g = gv[x], k = kv[x], q = qv[x];
    const float er = __expf(g - L.Gs[t][c]);
    L.Kr[r][c] = k * er;
    L.Qr[r][c] = q * er;
    L.Kc[r][c] = k * __expf(L.Ge[t][c] - g);
  }
  // Every thread reads the tile spans itself (same verdict in every wave).
  for (int t = 0; t < NT; ++t) {
    bool big = false;
    for (int c = lane_id(); c < D; c += 64) big |= L.Ge[t][c] - L.Gs[t][c] < -kTileSpan;
    bad[t] = __any(big);
  }
  __syncthreads();
}

// Bm (strictly lower) and P (lower) of the strong-decay chunks, block by
// block on v_mfma_f32_16x16x4f32: the column operand of block (a, b) is Kc
// of tile b times f_ab per channel.  Four waves share the blocks.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_gram_tile_kernel(Planes p) {
  extern __shared__ float sm[];
  TileLds<D, C>& L = *reinterpret_cast<TileLds<D, C>*>(sm);
  constexpr int NT = C / 16, NBLK = NT * (NT + 1) / 2;
  const size_t b = blockIdx.x;
  if (p.fast[b]) return;  // formed as a product
  bool bad[NT];
  tile_operands<D, C>(p, b, L, bad);
  const int w = wave_id(), l = lane_id(), m = l & 15, g = l >> 4;
  const size_t pcc = b * C * C;
  for (int blk = w; blk < NBLK; blk += 4) {
    int ta = 0;
    while ((ta + 1) * (ta + 2) / 2 <= blk) ++ta;
    const int tb = blk - ta * (ta + 1) / 2;  // tb <= ta
    f32x4 accB = {0, 0, 0, 0}, accP = {0, 0, 0, 0};
    if (tb < ta || !bad[ta]) {
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const int c = k0 + g;
        const float kc = L.Kc[16 * tb + m][c] * __expf(L.Gs[ta][c] - L.Ge[tb][c]);
        accB = mfma4(L.Kr[16 * ta + m][c], kc, accB);
        accP = mfma4(L.Qr[16 * ta + m][c], kc, accP);
      }
    } else {
      // tile span beyond kTileSpan: each pair with its exact exponent
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const size_t rr = 16 * ta + 4 * g + x, ii = 16 * tb + m;
        float sb = 0.f, sp = 0.f;
        if (ii <= rr) {
          for (int c = 0; c < D; ++c) {
            const float e = __expf(p.Gam[(b * C + rr) * D + c] - p.Gam[(b * C + ii) * D + c]);
            const float ki = p.K[(b * C + ii) * D + c] * e;
            sb += p.K[(b * C + rr) * D + c] * ki;
            sp += p.Q[(b * C + rr) * D + c] * ki;
          }
        }
        accB[x] = sb;
        accP[x] = sp;
      }
    }
    // lane (m, g) holds rows 4 g + x of column m of the block
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = 16 * ta + 4 * g + x, i = 16 * tb + m;
      p.Bm[pcc + r * C + i] = i < r ? accB[x] : 0.f;
      p.P[pcc + r * C + i] = i <= r ? accP[x] : 0.f;
    }
  }
  // blocks above the diagonal
  for (int idx = threadIdx.x; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    if (i / 16 > r / 16) {
      p.Bm[pcc + idx] = 0.f;
      p.P[pcc + idx] = 0.f;
    }
  }
}

// The pairwise gradient terms of the strong-decay chunks, as the exact sums
//   Z1[r,c] = sum_{i<r} dBm[r,i] k_ic e_ric,  Z2[r,c] = sum_{i<=r} dP[r,i] k_ic e_ric,
//   Z3[i,c] = sum_{r>=i} (dBm[r,i] k_rc + dP[r,i] q_rc) e_ric,  e_ric = exp(Gamma_rc - Gamma_ic),
// into the planes that hold Y1, Y2, Y3 for the factored chunks (R, U, dU).
// Per output tile: the block products of the tile operands, each block's
// result scaled column by column by f_ab, then the row factor of the
// output's own tile.  Four waves share the output tiles.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_pairs_tile_kernel(Planes p) {
  extern __shared__ float sm[];
  TileLds<D, C>& L = *reinterpret_cast<TileLds<D, C>*>(sm);
  constexpr int NT = C / 16, NCT = D / 16;
  const size_t b = blockIdx.x;
  if (p.fast[b]) return;  // the products Y1, Y2, Y3
  const size_t pcd = b * C * D;
  bool bad[NT];
  tile_operands<D, C, true>(p, b, L, bad);  // with dBm and dP
  const int w = wave_id(), l = lane_id(), m = l & 15, g = l >> 4;
  for (int ot = w; ot < NT * NCT; ot += 4) {
    const int ta = ot / NCT, ct = ot % NCT;
    const int c = 16 * ct + m;  // this lane's output channel
    // Z1, Z2 for rows of tile ta: blocks tb <= ta
    // z: factored sums (times the row factor at the end); zd: a diagonal
    // tile summed with exact exponents
    f32x4 z1 = {0, 0, 0, 0}, z2 = {0, 0, 0, 0}, z1d = {0, 0, 0, 0}, z2d = {0, 0, 0, 0};
    for (int tb = 0; tb <= ta; ++tb) {
      if (tb < ta || !bad[ta]) {
        const float f = __expf(L.Gs[ta][c] - L.Ge[tb][c]);
        f32x4 y1 = {0, 0, 0, 0}, y2 = {0, 0, 0, 0};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float kc = L.Kc[16 * tb + k0 + g][c];
          y1 = mfma4(L.dBm[16 * ta + m][16 * tb + k0 + g], kc, y1);
          y2 = mfma4(L.dP[16 * ta + m][16 * tb + k0 + g], kc, y2);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          z1[x] += f * y1[x];
          z2[x] += f * y2[x];
        }
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 16 * ta + 4 * g + x;
          const float gr = p.Gam[pcd + (size_t)r * D + c];
          for (int i = 16 * tb; i <= r; ++i) {
            const float ki = p.K[pcd + (size_t)i * D + c] * __expf(gr - p.Gam[pcd + (size_t)i * D + c]);
            z1d[x] += L.dBm[r][i] * ki;
            z2d[x] += L.dP[r][i] * ki;
          }
        }
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = 16 * ta + 4 * g + x;
      const float rf = __expf(p.Gam[pcd + (size_t)r * D + c] - L.Gs[ta][c]);
      p.R[pcd + (size_t)r * D + c] = z1[x] * rf + z1d[x];
      p.U[pcd + (size_t)r * D + c] = z2[x] * rf + z2d[x];
    }
    // Z3 for columns (tokens) of tile ta: blocks tr >= ta (rows r of tile tr)
    f32x4 z3 = {0, 0, 0, 0}, z3d = {0, 0, 0, 0};
    for (int tr = ta; tr < NT; ++tr) {
      if (tr > ta || !bad[ta]) {
        const float f = __expf(L.Gs[tr][c] - L.Ge[ta][c]);
        f32x4 y = {0, 0, 0, 0};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int r = 16 * tr + k0 + g;
          y = mfma4(L.dBm[r][16 * ta + m], L.Kr[r][c], y);
          y = mfma4(L.dP[r][16 * ta + m], L.Qr[r][c], y);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) z3[x] += f * y[x];
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 16 * ta + 4 * g + x;
          const float gi = p.Gam[pcd + (size_t)i * D + c];
          for (int r = i; r < 16 * tr + 16; ++r) {
            const float e = __expf(p.Gam[pcd + (size_t)r * D + c] - gi);
            z3d[x] += (L.dBm[r][i] * p.K[pcd + (size_t)r * D + c] + L.dP[r][i] * p.Q[pcd + (size_t)r * D + c]) * e;
          }
        }
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int i = 16 * ta + 4 * g + x;
      p.dU[pcd + (size_t)i * D + c] = z3[x] * __expf(L.Ge[ta][c] - p.Gam[pcd + (size_t)i * D + c]) + z3d[x];
    }
  }
}

constexpr int kSerThreads = 512;

// Serial passes over a sequence's chunks, one workgroup per (sequence, head,
// 16 value columns), eight waves.  The carried 16-column block (S forward,
// dS' backward) stays in the MFMA accumulators of waves 0 .. D/16 - 1, one
// 16 x 16 tile each.  Every product is cut into 16 x 16 tiles on
// v_mfma_f32_16x16x4f32, whose lane l supplies A[l & 15][k] and B[k][l & 15]
// for k = l >> 4 and ends with rows 4 (l >> 4) .. + 3 of column l & 15.  A
// tile's contraction is spread over several waves where the tiles are fewer
// than the waves, each wave's share ending as a partial tile in LDS that the
// next stage sums while reading it.  Within a share, lane group g takes a
// contiguous run of the contraction index, so a lane's A values are
// consecutive in memory where the plane's rows run along that index.  Every
// operand a stage takes from global memory is loaded into registers one chunk
// ahead, right after its last use.
template <int D, int C>
struct SerGeom {
  static constexpr int NW = kSerThreads / 64;
  static constexpr int NRT = C / 16;   // 16-row tiles of a chunk
  static constexpr int NST = D / 16;   // 16-row tiles of the carried block
  static constexpr int KS = NW / NRT;  // waves sharing a row tile's D-long contraction
  static constexpr int DK = D / KS;    // channels per share
  static constexpr int RJ = DK / 4;    // products per share
  static constexpr int SJ = C / 4;     // products of a C-long contraction
  static constexpr int TJ = C / 8;     // most products of a half of a triangular one
  static constexpr int FIN = (C * 16 + kSerThreads - 1) / kSerThreads;  // C x 16 elements per thread
  static_assert(NW % NRT == 0 && D % (4 * KS) == 0 && NST <= NW, "work split");
};

// Sum over the 16 lanes of each row of the wave (DPP row rotations; every
// lane ends with its row's sum).
__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xF, 0xF, true));
  return x;
}

// N consecutive floats (16-byte aligned when N % 4 == 0, 8-byte when even).
template <int N>
__device__ __forceinline__ void ld_run(float (&d)[N], const float* src) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N / 4; ++x) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * x);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * x + e] = v[e];
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N / 2; ++x) {
      const float2 v = *reinterpret_cast<const float2*>(src + 2 * x);
      d[2 * x] = v.x;
      d[2 * x + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) d[x] = src[x];
  }
}

// A 16-column slab of a chunk plane (rows r0 .. r0 + nr - 1 of [C][ld], columns
// c0 .. c0 + 15) moved through one wave: fetch() loads it with 16-byte loads
// (C / 16 per lane; rows past nr re-read the last one), put() writes it
// transposed into the wave's own LDS tile [16][C + 4], so that lane (m, g)
// then reads a contiguous run of rows of column m.  The tile belongs to one
// wave, so no barrier separates put() from the reads that follow it.
template <int C>
struct Slab {
  static constexpr int NU = C / 16;
  f32x4 v[NU];
  __device__ __forceinline__ void fetch(const float* plane, int ld, int r0, int nr, int c0, int l) {
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int u = l + 64 * x, r = (u >> 2) < nr ? (u >> 2) : nr - 1;
      v[x] = *reinterpret_cast<const f32x4*>(plane + (size_t)(r0 + r) * ld + c0 + 4 * (u & 3));
    }
  }
  __device__ __forceinline__ void put(float* tile, int nr, int l) const {
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int u = l + 64 * x, r = (u >> 2) < nr ? (u >> 2) : nr - 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[(4 * (u & 3) + e) * (C + 4) + r] = v[x][e];
    }
  }
};

// Requests every 128-byte line of one chunk's operand blocks ahead of their
// loads, so those loads find them in L2 rather than in HBM: each of the NVB
// workgroups of a (sequence, head), which share an L2, takes every NVB-th
// line, one per lane of each wave (lanes past the lines touch the first one
// again).  Returns the 4-byte value read; the caller keeps it until the next
// step and then marks it used (touch_done), so nothing waits for it sooner.
template <int NS>
__device__ __forceinline__ float l2_touch(const float* const (&base)[NS], const int (&lines)[NS], int vb,
                                          int nvb, int w, int nw, int l) {
  int line = vb + nvb * (64 * w + l);
  const float* ptr = base[0];
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    if (line >= 0 && line < lines[x]) ptr = base[x] + 32 * line;
    line -= lines[x];
  }
  (void)nw;
  return *ptr;
}
// Marks a touch value as used without any instruction (its load must have
// completed here).
__device__ __forceinline__ void touch_done(float x) { asm volatile("" ::"v"(x)); }

template <int D, int C>
struct FwdLds {
  float St[16][D + 4];                          // S^T: [value column][channel]
  float Rp[SerGeom<D, C>::KS][16][C + 4];       // shares of Kt S - V, transposed
  float Up[2][16][C + 4];                       // halves of T R, transposed
  float Kw[SerGeom<D, C>::NW][16][C + 4];       // each wave's Kb slab, transposed
};

// Serial forward over a sequence's chunks for 16 value columns: the state
// entering every chunk, R = V - Kt S and U = T R, and S' = gam_n S + Kb^T U.
// R stage: wave w takes row tile w % NRT and channel share w / NRT.  U stage:
// waves w < 2 NRT take row tile w % NRT and half w / NRT of its k < 16 (rt+1).
// S stage: wave t < D/16 updates its state tile.
template <int D, int C>
__global__ __launch_bounds__(kSerThreads) void bwd_fwd_states_kernel(Planes p, Geo geo,
                                                                     const float* __restrict__ s0,
                                                                     float* __restrict__ s_out) {
  typedef SerGeom<D, C> G;
  constexpr int NVB = D / kCols, NRT = G::NRT, NST = G::NST, DK = G::DK, RJ = G::RJ, SJ = G::SJ;
  constexpr int UJM = 2 * NRT;  // most U-stage products per lane
  constexpr int kFin = G::FIN;
  extern __shared__ float sm[];
  FwdLds<D, C>& L = *reinterpret_cast<FwdLds<D, C>*>(sm);
  const int H = geo.H;
  int nh, vb;
  if (!serial_slot<NVB>(geo.num_seqs * H, nh, vb)) return;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int m = l & 15, g = l >> 4;
  int bos, eos, base, lo, hi;
  seq_of<C>(geo, n, bos, eos, base);
  seg_range<C>(geo, bos, eos, lo, hi);
  const int rrt = w % NRT, rks = w / NRT;                       // R stage
  const int urt = w % NRT, uhs = (w / NRT) & 1;                 // U stage (w < 2 NRT)
  const int ulh = 8 * (urt + 1), uj = ulh / 4;                  // its half's length, products
  const int st = w < NST ? w : NST - 1;                         // S stage tile
  auto blk = [&](int ci) { return (size_t)(base + ci - geo.c0) * H + h; };

  float ra[RJ], rv[4], ta[UJM], sreg[4];
  Slab<C> kb;
  f32x4 gam;
  auto load_r = [&](size_t b) {
    ld_run<RJ>(ra, p.Kt + (b * C + 16 * rrt + m) * D + rks * DK + g * RJ);
#pragma unroll
    for (int i = 0; i < 4; ++i) rv[i] = p.V[(b * C + 16 * rrt + 4 * g + i) * D + col0 + m];
  };
  auto load_u = [&](size_t b) {  // uj is even, and so is the run's offset
    const float* src = p.T + (b * C + 16 * urt + m) * C + uhs * ulh + g * uj;
#pragma unroll
    for (int j = 0; j < UJM; j += 2) {
      const float2 x = *reinterpret_cast<const float2*>(src + (j < uj ? j : 0));
      ta[j] = x.x;
      ta[j + 1] = x.y;
    }
  };
  auto load_s = [&](size_t b) {
    kb.fetch(p.Kb + b * C * D, D, 0, C, 16 * st, l);
    gam = *reinterpret_cast<const f32x4*>(p.gn + b * D + 16 * st + 4 * g);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sreg[i] = s0 ? s0[(((size_t)n * H + h) * D + 16 * st + 4 * g + i) * D + col0 + m] : 0.f;
  // The initial state in full before any prefetch: left pending, it would
  // make the compiler's waits in the loop count every later load.
  __builtin_amdgcn_s_waitcnt(0);
  float tch = 0.f;  // the last L2 request's value
  if (lo < hi) {
    load_r(blk(lo));
    load_u(blk(lo));
    load_s(blk(lo));
  }
  // R and U of a chunk go out at the top of the next step (and of the last
  // chunk after the loop), so every step issues the same memory operations
  // in the same order, the first one included (its store goes to the first
  // chunk's rows, which the second step then overwrites); the compiler's
  // waits for the operands loaded a step earlier then cover nothing newer.
  auto put_ru = [&](size_t b) {
    const size_t pcd = b * C * D;
#pragma unroll
    for (int xf = 0; xf < kFin; ++xf) {
      const int e = tid + kSerThreads * xf, nn = e & 15, r = e >> 4;
      if (C * 16 % kSerThreads != 0 && e >= C * 16) break;
      float x = 0.f;
#pragma unroll
      for (int k = 0; k < G::KS; ++k) x += L.Rp[k][nn][r];
      p.R[pcd + r * D + col0 + nn] = -x;  // R = -(sum of the shares)
      p.U[pcd + r * D + col0 + nn] = L.Up[0][nn][r] + L.Up[1][nn][r];
    }
  };
  for (int ci = lo; ci < hi; ++ci) {
    const size_t b = blk(ci), bn = blk(ci + 1 < hi ? ci + 1 : ci);
    put_ru(blk(ci > lo ? ci - 1 : ci));
    if (NST == G::NW || w < NST) {  // publish the entering state (every wave at d = 128)
      *reinterpret_cast<f32x4*>(&L.St[m][16 * w + 4 * g]) = f32x4{sreg[0], sreg[1], sreg[2], sreg[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) p.S[(b * D + 16 * w + 4 * g + i) * D + col0 + m] = sreg[i];
    }
    __syncthreads();
    {  // chunk ci + 2's operands into L2
      static_assert(NVB * kSerThreads >= (3 * C * D + C * C) / 32 + D / 32, "one line per lane covers them");
      const size_t b2 = blk(ci + 2 < hi ? ci + 2 : hi - 1);
      const float* const bp[5] = {p.Kt + b2 * C * D, p.Kb + b2 * C * D, p.V + b2 * C * D, p.T + b2 * C * C,
                                  p.gn + b2 * D};
      const int ln[5] = {C * D / 32, C * D / 32, C * D / 32, C * C / 32, D / 32};
      touch_done(tch);
      tch = l2_touch<5>(bp, ln, vb, NVB, w, G::NW, l);
    }
    {  // share rks of Kt S (minus V in share 0) for row tile rrt
      f32x4 acc = rks == 0 ? f32x4{-rv[0], -rv[1], -rv[2], -rv[3]} : f32x4{0, 0, 0, 0};
      float sb[RJ];
      ld_run<RJ>(sb, &L.St[m][rks * DK + g * RJ]);
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc = mfma4(ra[j], sb[j], acc);
      *reinterpret_cast<f32x4*>(&L.Rp[rks][m][16 * rrt + 4 * g]) = acc;
    }
    load_r(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
    __syncthreads();
    if (2 * NRT == G::NW || w < 2 * NRT) {  // half uhs of T R for row tile urt
      f32x4 acc = {0, 0, 0, 0};
      const int k0 = uhs * ulh + g * uj;
      // R^T in pairs (8-byte reads: one lane's run is contiguous in the
      // transposed shares; single floats put lanes 16 apart on one bank)
      float2 rx[UJM / 2];
#pragma unroll
      for (int j = 0; j < UJM; j += 2) {
        const int jj = j < uj ? j : 0;
        rx[j / 2] = float2{0.f, 0.f};
#pragma unroll
        for (int k = 0; k < G::KS; ++k) {
          const float2 v = *reinterpret_cast<const float2*>(&L.Rp[k][m][k0 + jj]);
          rx[j / 2].x += v.x;
          rx[j / 2].y += v.y;
        }
      }
#pragma unroll
      for (int j = 0; j < UJM; j += 2)
        if (j < uj) {
          acc = mfma4(ta[j], -rx[j / 2].x, acc);
          acc = mfma4(ta[j + 1], -rx[j / 2].y, acc);
        }
      *reinterpret_cast<f32x4*>(&L.Up[uhs][m][16 * urt + 4 * g]) = acc;
    }
    load_u(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
    __syncthreads();
    if (NST == G::NW || w < NST) {  // S' = gam_n S + Kb^T U for state tile w
      float* kw = &L.Kw[w][0][0];
      kb.put(kw, C, l);
      f32x4 acc = {gam[0] * sreg[0], gam[1] * sreg[1], gam[2] * sreg[2], gam[3] * sreg[3]};
      float a[SJ], u0[SJ], u1[SJ];
      ld_run<SJ>(a, kw + m * (C + 4) + g * SJ);
      ld_run<SJ>(u0, &L.Up[0][m][g * SJ]);
      ld_run<SJ>(u1, &L.Up[1][m][g * SJ]);
#pragma unroll
      for (int j = 0; j < SJ; ++j) acc = mfma4(a[j], u0[j] + u1[j], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sreg[i] = acc[i];
    }
    load_s(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
  }
  if (lo < hi) put_ru(blk(hi - 1));
  if (s_out && w < NST) {  // the state after the pass's last chunk
#pragma unroll
    for (int i = 0; i < 4; ++i) s_out[(((size_t)n * H + h) * D + 16 * w + 4 * g + i) * D + col0 + m] = sreg[i];
  }
}

template <int D, int C>
struct BwdLds {
  float Xt[16][D + 4];                          // dS'^T: [value column][channel]
  float Up[SerGeom<D, C>::KS][16][C + 4];       // shares of dU, transposed
  float Rp[2][16][C + 4];                       // halves of dR, transposed
  float dOt[2][16][C + 4];                      // dO slice, transposed; by chunk parity
  float Wt[SerGeom<D, C>::NW][2][16][C + 4];    // each wave's slabs, transposed
};

// Serial backward over a sequence's chunks for 16 value columns: dS' of
// every chunk, dU = P^T dO + Kb dS', dR = T^T dU, and the carried
// dS = gam_n dS' + Qt^T dO - Kt^T dR; the last one is dS0.  dU stage: wave w
// takes row tile w % NRT and channel share w / NRT of Kb dS' (share 0 adds
// P^T dO, over k >= 16 rt).  dR stage: waves w < 2 NRT take row tile w % NRT
// and half w / NRT of its k >= 16 rt.  dS stage: wave t < D/16 updates its
// tile of the carried gradient.
template <int D, int C>
__global__ __launch_bounds__(kSerThreads) void bwd_bwd_states_kernel(Planes p, Geo geo,
                                                                     const float* __restrict__ dfin,
                                                                     float* __restrict__ ds0) {
  typedef SerGeom<D, C> G;
  constexpr int NVB = D / kCols, NRT = G::NRT, NST = G::NST, DK = G::DK, RJ = G::RJ, SJ = G::SJ,
                TJ = G::TJ, kFin = G::FIN;
  extern __shared__ float sm[];
  BwdLds<D, C>& L = *reinterpret_cast<BwdLds<D, C>*>(sm);
  const int H = geo.H;
  int nh, vb;
  if (!serial_slot<NVB>(geo.num_seqs * H, nh, vb)) return;
  const int n = nh / H, h = nh % H, col0 = vb * kCols;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int m = l & 15, g = l >> 4;
  int bos, eos, base, lo, hi;
  seq_of<C>(geo, n, bos, eos, base);
  seg_range<C>(geo, bos, eos, lo, hi);
  const int urt = w % NRT, uks = w / NRT;                 // dU stage
  const int pn = C - 16 * urt, pj = pn / 4;               // its P^T part (share 0): k >= 16 urt
  const int rrt = w % NRT, rhs = (w / NRT) & 1;           // dR stage (w < 2 NRT)
  const int rn = C - 16 * rrt, rj = rn / 8;               // k >= 16 rrt, in two halves
  const int st = w < NST ? w : NST - 1;                   // dS stage tile
  auto blk = [&](int ci) { return (size_t)(base + ci - geo.c0) * H + h; };
  float* w0 = &L.Wt[w][0][0][0];
  float* w1 = &L.Wt[w][1][0][0];

  float ua[RJ], xreg[4];
  Slab<C> ps, ts, qs, ks;
  f32x4 dov, gam;
  float sv[4];  // S entering the chunk: rows 16 st + 4 g .. + 3, this lane's value column
  const int du = tid < 4 * C ? tid : 4 * C - 1;  // this thread's 16 bytes of the dO slice
  // The dO slice and the S slice are requested first: both are used at the top
  // of the next step, so a late request would hold that step back by a
  // memory round trip.
  auto load_u = [&](size_t b) {
    dov = *reinterpret_cast<const f32x4*>(p.dO + (b * C + (du >> 2)) * D + col0 + 4 * (du & 3));
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = p.S[(b * D + 16 * st + 4 * g + i) * D + col0 + m];
    ld_run<RJ>(ua, p.Kb + (b * C + 16 * urt + m) * D + uks * DK + g * RJ);
    ps.fetch(p.P + b * C * C, C, 16 * urt, pn, 16 * urt, l);
  };
  auto load_r = [&](size_t b) { ts.fetch(p.T + b * C * C, C, 16 * rrt, rn, 16 * rrt, l); };
  auto load_s = [&](size_t b) {
    qs.fetch(p.Qt + b * C * D, D, 0, C, 16 * st, l);
    ks.fetch(p.Kt + b * C * D, D, 0, C, 16 * st, l);
    gam = *reinterpret_cast<const f32x4*>(p.gn + b * D + 16 * st + 4 * g);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xreg[i] = dfin ? dfin[(((size_t)n * H + h) * D + 16 * st + 4 * g + i) * D + col0 + m] : 0.f;
  __builtin_amdgcn_s_waitcnt(0);  // as in the forward pass
  float tch = 0.f;  // the last L2 request's value
  if (lo < hi) {
    load_u(blk(hi - 1));
    load_r(blk(hi - 1));
    load_s(blk(hi - 1));
  }
  // dU and dR of a chunk go out at the top of the next step (and of the last
  // one after the loop), as in the forward pass.
  auto put_ur = [&](size_t b) {
    const size_t pcd = b * C * D;
#pragma unroll
    for (int xf = 0; xf < kFin; ++xf) {
      const int e = tid + kSerThreads * xf, nn = e & 15, r = e >> 4;
      if (C * 16 % kSerThreads != 0 && e >= C * 16) break;
      float x = 0.f;
#pragma unroll
      for (int k = 0; k < G::KS; ++k) x += L.Up[k][nn][r];
      p.dU[pcd + r * D + col0 + nn] = x;
      p.dR[pcd + r * D + col0 + nn] = L.Rp[0][nn][r] + L.Rp[1][nn][r];
    }
  };
  for (int ci = hi - 1; ci >= lo; --ci) {
    const size_t b = blk(ci), bn = blk(ci > lo ? ci - 1 : ci);
    put_ur(blk(ci < hi - 1 ? ci + 1 : ci));
    float* dot = &L.dOt[ci & 1][0][0];
    if (tid < 4 * C) {  // this chunk's dO slice, transposed
#pragma unroll
      for (int e = 0; e < 4; ++e) dot[(4 * (du & 3) + e) * (C + 4) + (du >> 2)] = dov[e];
    }
    if (NST == G::NW || w < NST) {  // publish dS'; this block's share of rowsum(dS' * S)
      *reinterpret_cast<f32x4*>(&L.Xt[m][16 * w + 4 * g]) = f32x4{xreg[0], xreg[1], xreg[2], xreg[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) p.dSn[(b * D + 16 * w + 4 * g + i) * D + col0 + m] = xreg[i];
      float t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = row_sum16(xreg[i] * sv[i]);  // over the 16 columns
      // every lane stores (lanes m and m + 4k store the same value)
      const int i4 = m & 3;
      p.dgp[(b * NVB + vb) * D + 16 * w + 4 * g + i4] = i4 == 0 ? t[0] : i4 == 1 ? t[1] : i4 == 2 ? t[2] : t[3];
    }
    __syncthreads();
    {  // chunk ci - 2's operands into L2
      static_assert(NVB * kSerThreads >= (4 * C * D + 2 * C * C + D * D) / 32 + D / 32,
                    "one line per lane covers them");
      const size_t b2 = blk(ci - 2 >= lo ? ci - 2 : lo);
      const float* const bp[8] = {p.Kb + b2 * C * D, p.Qt + b2 * C * D, p.Kt + b2 * C * D, p.dO + b2 * C * D,
                                  p.P + b2 * C * C, p.T + b2 * C * C, p.S + b2 * D * D, p.gn + b2 * D};
      const int ln[8] = {C * D / 32, C * D / 32, C * D / 32, C * D / 32, C * C / 32, C * C / 32, D * D / 32, D / 32};
      touch_done(tch);
      tch = l2_touch<8>(bp, ln, vb, NVB, w, G::NW, l);
    }
    {  // share uks of Kb dS' (plus P^T dO in share 0) for row tile urt
      f32x4 acc = {0, 0, 0, 0};
      float xb[RJ];
      ld_run<RJ>(xb, &L.Xt[m][uks * DK + g * RJ]);
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc = mfma4(ua[j], xb[j], acc);
      if (uks == 0) {
        ps.put(w0, pn, l);
        float a[SJ], d[SJ];
        ld_run<SJ>(a, w0 + m * (C + 4) + g * pj);       // P[16 urt + g pj + j][16 urt + m]
        ld_run<SJ>(d, dot + m * (C + 4) + 16 * urt + g * pj);  // dO[16 urt + g pj + j][m]
#pragma unroll
        for (int j = 0; j < SJ; ++j)
          if (j < pj) acc = mfma4(a[j], d[j], acc);
      }
      *reinterpret_cast<f32x4*>(&L.Up[uks][m][16 * urt + 4 * g]) = acc;
    }
    load_u(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
    __syncthreads();
    if (2 * NRT == G::NW || w < 2 * NRT) {  // half rhs of T^T dU for row tile rrt
      ts.put(w0, rn, l);
      const int k0 = rhs * (rn / 2) + g * rj;  // relative to row 16 rrt
      f32x4 acc = {0, 0, 0, 0};
      // both operands in pairs (rj and k0 are even), as in the forward U stage
      float2 tx[TJ / 2], ux[TJ / 2];
#pragma unroll
      for (int j = 0; j < TJ; j += 2) {
        const int jj = j < rj ? j : 0;
        tx[j / 2] = *reinterpret_cast<const float2*>(w0 + m * (C + 4) + k0 + jj);
        ux[j / 2] = float2{0.f, 0.f};
#pragma unroll
        for (int k = 0; k < G::KS; ++k) {
          const float2 v = *reinterpret_cast<const float2*>(&L.Up[k][m][16 * rrt + k0 + jj]);
          ux[j / 2].x += v.x;
          ux[j / 2].y += v.y;
        }
      }
#pragma unroll
      for (int j = 0; j < TJ; j += 2)
        if (j < rj) {
          acc = mfma4(tx[j / 2].x, ux[j / 2].x, acc);
          acc = mfma4(tx[j / 2].y, ux[j / 2].y, acc);
        }
      *reinterpret_cast<f32x4*>(&L.Rp[rhs][m][16 * rrt + 4 * g]) = acc;
    }
    load_r(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
    __syncthreads();
    if (NST == G::NW || w < NST) {  // dS = gam_n dS' + Qt^T dO - Kt^T dR for tile w
      qs.put(w0, C, l);
      ks.put(w1, C, l);
      f32x4 acc = {gam[0] * xreg[0], gam[1] * xreg[1], gam[2] * xreg[2], gam[3] * xreg[3]};
      float qa[SJ], ka[SJ], d[SJ], r0[SJ], r1[SJ];
      ld_run<SJ>(qa, w0 + m * (C + 4) + g * SJ);
      ld_run<SJ>(ka, w1 + m * (C + 4) + g * SJ);
      ld_run<SJ>(d, dot + m * (C + 4) + g * SJ);
      ld_run<SJ>(r0, &L.Rp[0][m][g * SJ]);
      ld_run<SJ>(r1, &L.Rp[1][m][g * SJ]);
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        acc = mfma4(qa[j], d[j], acc);
        acc = mfma4(ka[j], -(r0[j] + r1[j]), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xreg[i] = acc[i];
    }
    load_s(bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are
  }
  if (lo < hi) put_ur(blk(lo));
  if (ds0 && w < NST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ds0[(((size_t)n * H + h) * D + 16 * w + 4 * g + i) * D + col0 + m] = xreg[i];
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
  constexpr int NS = C * C / 256, CP = 256 / C;  // elements per thread; threads per column
  static_assert(NS * 256 == C * C, "whole elements per thread");
  __shared__ float colp[CP][C];  // partial column sums of M * dT
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t pcc = (size_t)b * C * C;
  const float* beta = p.beta + (size_t)b * C;
  const int w = tid >> 6, l = tid & 63, lm = l & 15, lg = l >> 4;
  // Every global load is issued here, before the first wait: M and dT (this
  // thread's column i = tid % C, rows tid / C + CP x), beta_i, and the Bm
  // values and beta rows of this lane's accumulator positions for the last
  // stage (whose stores the compiler may not move those loads past).
  float mv[NS], tv[NS], bmv[TPW][4], brv[TPW][4];
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    mv[x] = p.M[pcc + tid + 256 * x];
    tv[x] = p.dT[pcc + tid + 256 * x];
  }
  const float bi = beta[tid % C];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = min(w + 4 * j, NT * NT - 1);
    const int r0 = 16 * (t / NT), c0 = 16 * (t % NT);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      bmv[j][v] = p.Bm[pcc + (size_t)(r0 + 4 * lg + v) * C + c0 + lm];
      brv[j][v] = beta[r0 + 4 * lg + v];
    }
  }
  float cs = 0.f;
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    const int idx = tid + 256 * x, r = idx / C, i = idx % C;
    Ms[r][i] = mv[x];
    MTs[i][r] = mv[x];
    dMs[r][i] = tv[x] * bi;
    cs += mv[x] * tv[x];
  }
  colp[tid / C][tid % C] = cs;
  __syncthreads();
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
        p.dBm[pcc + r * C + i] = brv[j][v] * sv;
        dMs[r][i] = sv * bmv[j][v];  // dA * Bm, for the row sums
      }
    }
  }
  __syncthreads();
  if (tid < C) {
    const int j = tid;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < CP; ++x) s += colp[x][j];  // colsum(M * dT)
    for (int r = 0; r < C; ++r) s += dMs[j][r];     // rowsum(dA * Bm)
    p.db[(size_t)b * C + j] = s;
  }
}

struct BwdOut {
  float *dq, *dk, *dv, *dg, *dbeta;
};

// The final pass: the pairwise gradient terms, the decays, the reverse
// cumulative sum of dGamma and the scatter to the token-major outputs, for
// one (chunk, head) and 64 channels.  For factored chunks the pairwise terms
// are the products Y1 = dBm Kh, Y2 = dP Kh, Y3 = dBm^T Kt + dP^T Qt, formed
// here on v_mfma_f32_16x16x4f32 (each wave 16 channels and every row tile of
// the chunk), with dq += gam Y2, dk += gam Y1 + exp(-Gamma) Y3, dGamma +=
// Kt Y1 + Qt Y2 - Kh Y3 taken straight from the accumulators; for
// strong-decay chunks they are the sums Z1, Z2, Z3 that bwd_pairs_tile_kernel
// left in the R, U, dU planes, with dq += Z2, dk += Z1 + Z3, dGamma +=
// k (Z1 - Z3) + q Z2.  The contraction index of every product is
// k = 16 q + 4 g + s for lane group g, so the B-operand registers (column c
// of Kh, Kt, Qt at those rows) are also the values the combine needs at rows
// 16 a + 4 g + i of the accumulators.  dBm and dP (zero above, resp. on and
// above, the diagonal) are staged in LDS; blocks of them that are zero skip
// their products.  Items in groups of eight with the tiles of a group's
// items interleaved, so both tiles of an item run on one XCD.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_final_prod_kernel(Planes p, Geo geo, BwdOut out, int nb) {
  constexpr int NRT = C / 16, NQ = C / 16, NCT = D / 64, LDX = C + 4, LDT = 64 + 4;
  __shared__ __attribute__((aligned(16))) float Xb[C][LDX];   // dBm
  __shared__ __attribute__((aligned(16))) float Xp[C][LDX];   // dP
  __shared__ __attribute__((aligned(16))) float term[C][LDT];  // dGamma terms of the tile
  __shared__ float kbp[4][64];                                  // partial sums of dKb Kb per lane group
  const int grp = blockIdx.x / (8 * NCT), rem = blockIdx.x % (8 * NCT);
  const int b = 8 * grp + rem % 8, ct = rem / 8;
  if (b >= nb) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4, H = geo.H;
  const int cl = 16 * w + m, c = 64 * ct + cl;  // this lane's channel (local, global)
  const bool fast = p.fast[b] != 0;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D, pcc = (size_t)b * C * C;
  // (the item's plane base is uniform, the in-plane offset 32-bit)
  auto at = [&](const float* x, int r) { return (x + pcd)[r * D + c]; };
  // Every load of the product phase is issued first and unconditionally
  // (all addresses are valid; a strong-decay chunk ignores what it does not
  // use): dBm and dP for the LDS staging, then column c of Kh, Kt, Qt at rows
  // 16 q + 4 g + s.
  constexpr int NSTG = (C * C / 4 + 255) / 256;  // 16-byte pieces of dBm (and dP) per thread
  f32x4 sb[NSTG], sp[NSTG];
#pragma unroll
  for (int x = 0; x < NSTG; ++x) {
    const int idx = min(tid + 256 * x, C * C / 4 - 1), r = idx / (C / 4), k4 = 4 * (idx % (C / 4));
    sb[x] = *reinterpret_cast<const f32x4*>(p.dBm + pcc + (size_t)r * C + k4);
    sp[x] = *reinterpret_cast<const f32x4*>(p.dP + pcc + (size_t)r * C + k4);
  }
  float bt[4 * NQ], bq[4 * NQ], bh[4 * NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int r = 16 * q + 4 * g + s2;
      bt[4 * q + s2] = at(p.Kt, r);
      bq[4 * q + s2] = at(p.Qt, r);
      bh[4 * q + s2] = at(p.Kh, r);
    }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the staging writes
  f32x4 y1[NRT], y2[NRT], y3[NRT];
#pragma unroll
  for (int a = 0; a < NRT; ++a) {
    y1[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    y2[a] = y1[a];
    y3[a] = y1[a];
  }
  if (fast) {
#pragma unroll
    for (int x = 0; x < NSTG; ++x) {
      const int idx = tid + 256 * x, r = idx / (C / 4), k4 = 4 * (idx % (C / 4));
      if (C * C / 4 % 256 == 0 || idx < C * C / 4) {
        *reinterpret_cast<f32x4*>(&Xb[r][k4]) = sb[x];
        *reinterpret_cast<f32x4*>(&Xp[r][k4]) = sp[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < NRT; ++a) {
      // Y1, Y2 (rows 16 a + .., k <= 16 a + 15)
#pragma unroll
      for (int q = 0; q <= a; ++q) {
        const f32x4 xb = *reinterpret_cast<const f32x4*>(&Xb[16 * a + m][16 * q + 4 * g]);
        const f32x4 xp = *reinterpret_cast<const f32x4*>(&Xp[16 * a + m][16 * q + 4 * g]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          y1[a] = mfma4(xb[s2], bh[4 * q + s2], y1[a]);
          y2[a] = mfma4(xp[s2], bh[4 * q + s2], y2[a]);
        }
      }
      // Y3 (columns 16 a + .. of dBm, dP; k >= 16 a)
#pragma unroll
      for (int q = a; q < NQ; ++q)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const int k = 16 * q + 4 * g + s2;
          y3[a] = mfma4(Xb[k][16 * a + m], bt[4 * q + s2], y3[a]);
          y3[a] = mfma4(Xp[k][16 * a + m], bq[4 * q + s2], y3[a]);
        }
    }
  }
  // Combine: lane (m, g) holds rows 16 a + 4 g + i of column c.  A row
  // tile's plane values are loaded before the previous tile's outputs are
  // stored (the compiler may not move a load above a store that could alias
  // it), so one memory round trip per tile overlaps the previous tile's work.
  // Two copies, for the factored and the strong-decay chunks, so that no load
  // sits under a branch.
  const float gl = at(p.Gam, C - 1);
  float kbsum = 0.f;
  auto combine = [&](auto fc) {
    constexpr bool F = decltype(fc)::value;
    constexpr int NV = F ? 6 : 11;  // planes read per row
    auto load_tile = [&](int a, float (&t)[NV][4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * g + i;
        t[0][i] = at(p.Gam, r);
        t[1][i] = at(p.dQt, r);
        t[2][i] = at(p.dKt, r);
        t[3][i] = at(p.dKb, r);
        t[4][i] = at(p.Kb, r);
        t[5][i] = at(p.dR, r);
        if constexpr (!F) {
          t[6][i] = at(p.R, r);
          t[7][i] = at(p.U, r);
          t[8][i] = at(p.dU, r);
          t[9][i] = at(p.K, r);
          t[10][i] = at(p.Q, r);
        }
      }
    };
    float tv[2][NV][4];
    load_tile(0, tv[0]);
#pragma unroll
    for (int a = 0; a < NRT; ++a) {
      if (a + 1 < NRT) load_tile(a + 1, tv[(a + 1) & 1]);
      const float(&t)[NV][4] = tv[a & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * g + i;
        const float gr = t[0][i], dqt = t[1][i], dkt = t[2][i], dkb = t[3][i], kbv = t[4][i];
        const float qt = bq[4 * a + i], kt = bt[4 * a + i];
        const float ga = __expf(gr), gb = dkb * __expf(gl - gr);
        float dq, dk, tm;
        if constexpr (F) {
          const float v1 = y1[a][i], v2 = y2[a][i], v3 = y3[a][i];
          tm = dqt * qt + dkt * kt - dkb * kbv + kt * v1 + qt * v2 - bh[4 * a + i] * v3;
          dq = (dqt + v2) * ga;
          dk = (dkt + v1) * ga + gb + __expf(-gr) * v3;
        } else {
          const float v1 = t[6][i], v2 = t[7][i], v3 = t[8][i], x1 = t[9][i], x2 = t[10][i];
          tm = dqt * qt + dkt * kt - dkb * kbv + x1 * v1 + x2 * v2 - x1 * v3;
          dq = dqt * ga + v2;
          dk = dkt * ga + v1 + gb + v3;
        }
        term[r][cl] = tm;
        kbsum += dkb * kbv;
        touch_done(t[5][i]);  // dR is stored only for rows < len: keep its load out of that branch
        if (r < len) {
          const size_t ti = ((size_t)(t0 + r) * H + h) * D + c;
          out.dq[ti] = dq;
          out.dk[ti] = dk;
          out.dv[ti] = t[5][i];
        }
      }
    }
  };
  if (fast)
    combine(std::true_type{});
  else
    combine(std::false_type{});
  kbp[g][cl] = kbsum;
  __syncthreads();
  if (tid < 64) {  // dg = reverse cumulative sum of dGamma; dGamma_n lands on the last row
    const int cc = 64 * ct + tid;
    float dgn = 0.f;  // rowsum(dS' * S)[cc], from the serial pass's per-block shares
#pragma unroll
    for (int v = 0; v < D / 16; ++v) dgn += p.dgp[((size_t)b * (D / 16) + v) * D + cc];
    float run = dgn * p.gn[(size_t)b * D + cc] + kbp[0][tid] + kbp[1][tid] + kbp[2][tid] + kbp[3][tid];
#pragma unroll 8
    for (int r = C - 1; r >= 0; --r) {
      run += term[r][tid];
      if (r < len) out.dg[((size_t)(t0 + r) * H + h) * D + cc] = run;
    }
  }
  if (ct == 0 && tid < len) out.dbeta[(size_t)(t0 + tid) * H + h] = p.db[(size_t)b * C + tid];
}

// Chunk counts of the sequences, on the host.
struct BwdCounts {
  int num_seqs;
  const int32_t* cu;  // host cu_seqlens or nullptr
  int seq_len, C;
  int nch(int n) const {
    const long long len = cu ? (long long)cu[n + 1] - cu[n] : seq_len;
    return (int)((len + C - 1) / C);
  }
  long long slots(int c0, int L) const {  // plane slots of the segment at c0
    long long t = 0;
    for (int n = 0; n < num_seqs; ++n) {
      const int c = nch(n) - c0;
      t += c <= 0 ? 0 : (c < L ? c : L);
    }
    return t;
  }
  int max_nch() const {
    int m = 0;
    for (int n = 0; n < num_seqs; ++n) m = nch(n) > m ? nch(n) : m;
    return m;
  }
};

// The backward runs in segments of L local chunks of every sequence, like the
// forward prefill: a forward sweep over the segments keeps only the state
// entering each one, and the backward sweep, last segment first, recomputes a
// segment's forward planes from that state before its gradients.  The planes
// of one segment fit the budget (4 GiB unless the caller's tuning says
// otherwise), so the workspace is bounded for any length; an input that fits
// in one segment runs exactly as one pass.
struct BwdPlan {
  int L = 0, nseg = 0;
  long long max_slots = 0;
};

BwdPlan plan_backward(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D, int C,
                      const PrefillTuning& t) {
  const BwdCounts sc{num_seqs, cu_host, seq_len, C};
  const int maxc = sc.max_nch();
  BwdPlan p;
  auto finish = [&](int L) {
    p.L = L < 1 ? 1 : L;
    p.nseg = maxc == 0 ? 1 : (maxc + p.L - 1) / p.L;
    p.max_slots = 0;
    for (int s = 0; s < p.nseg; ++s) {
      const long long x = sc.slots(s * p.L, p.L);
      p.max_slots = x > p.max_slots ? x : p.max_slots;
    }
  };
  if (t.segment_chunks >= 1) {
    finish(t.segment_chunks);
    return p;
  }
  const size_t budget = t.segment_bytes >= 1 ? t.segment_bytes : (size_t)4 << 30;
  // the largest L whose planes fit, at least one chunk; then even out
  int lo = 1, hi = maxc > 0 ? maxc : 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (plane_bytes((size_t)sc.slots(0, mid) * H, C, D) <= budget)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int nseg = maxc == 0 ? 1 : (maxc + lo - 1) / lo;
  finish(maxc == 0 ? 1 : (maxc + nseg - 1) / nseg);
  return p;
}

size_t bwd_bytes(const BwdPlan& p, int num_seqs, bool varlen, int H, int D, int C) {
  const size_t nhdd = (size_t)num_seqs * H * D * D * sizeof(float);
  return (varlen ? a256(sizeof(int32_t) * (size_t)(num_seqs + 1)) : 0) +
         (p.nseg > 1 ? a256((size_t)p.nseg * nhdd) : 0) + plane_bytes((size_t)p.max_slots * H, C, D);
}

template <class in_t, int D, int C>
hipError_t launch_backward_t(const BackwardArgs& a) {
  const BwdPlan plan = plan_backward(a.num_seqs, a.cu_seqlens_host, a.seq_len, a.H, D, C, a.tuning);
  const BwdCounts sc{a.num_seqs, a.cu_seqlens_host, a.seq_len, C};
  const size_t nhdd = (size_t)a.num_seqs * a.H * D * D;
  char* ws = reinterpret_cast<char*>(a.workspace);
  Geo geo;
  geo.cu = a.cu_seqlens;
  geo.off = reinterpret_cast<const int32_t*>(ws);
  geo.num_seqs = a.num_seqs;
  geo.seq_len = a.seq_len;
  geo.total_tokens = a.total_tokens;
  geo.H = a.H;
  geo.L = plan.L;
  char* after_table = ws + (a.cu_seqlens ? a256(sizeof(int32_t) * (a.num_seqs + 1)) : 0);
  // States entering segments 1 .. nseg-1, then the carried dS, then planes.
  float* ckpt = reinterpret_cast<float*>(after_table);
  float* dcarry = ckpt + (plan.nseg > 1 ? (size_t)(plan.nseg - 1) * nhdd : 0);
  char* planes = after_table + (plan.nseg > 1 ? a256((size_t)plan.nseg * nhdd * sizeof(float)) : 0);
  const size_t NBmax = (size_t)plan.max_slots * a.H;
  Planes p = carve(planes, NBmax, C, D);
  auto state_in = [&](int s) { return s == 0 ? a.initial_state : ckpt + (size_t)(s - 1) * nhdd; };

  const int serial = serial_blocks(a.num_seqs * a.H, D / kCols);
  const size_t flds_s = sizeof(FwdLds<D, C>), blds_s = sizeof(BwdLds<D, C>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_fwd_states_kernel<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)flds_s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_bwd_states_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)blds_s);
  if (e != hipSuccess) return e;
  const size_t tlds = sizeof(TileLds<D, C>);
  static_assert(sizeof(TileLds<D, C>) <= 160 * 1024, "tile operands fit LDS");
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_gram_tile_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)tlds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_pairs_tile_kernel<D, C>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)tlds);
  if (e != hipSuccess) return e;

  // With bf16 inputs the batched products run on split-bf16 operands (about
  // 16 significant bits, as the forward pass's products); fp32 inputs keep
  // fp32 products for their tighter bound.
  constexpr bool kSplitGemm = sizeof(in_t) == 2;
  BwdIn in{a.q, a.k, a.v, a.g, a.beta, a.d_o};
  BwdOut out{a.dq, a.dk, a.dv, a.dg, a.dbeta};
  hipError_t gerr = hipSuccess;
  size_t NB = 0;
  auto gemm = [&](auto op, const float* A, const float* B, float* Cm, int M, int N, int K,
                  int lda, int ldb, size_t sa, size_t sb, float alpha, int acc_c, int mask) {
    typedef decltype(op) O;
    const hipError_t e = launch_fp32_gemm<O::TA, O::TB, kGemmOne, kSplitGemm>(A, B, Cm, M, N, K, lda, ldb, N, sa, sb,
                                                         (size_t)M * N, alpha, acc_c, mask, NB,
                                                         a.stream);
    if (gerr == hipSuccess) gerr = e;
  };
  // Two products in one launch: kGemmDual (second A and C, same B) or
  // kGemmCat (second A and B, summed into C).
  auto gemm2 = [&](auto op, auto mode, const float* A, const float* B, float* Cm, int M, int N, int K,
                   int lda, int ldb, size_t sa, size_t sb, float alpha, int mask, GemmX x2) {
    typedef decltype(op) O;
    const hipError_t e = launch_fp32_gemm<O::TA, O::TB, decltype(mode)::value, kSplitGemm>(
        A, B, Cm, M, N, K, lda, ldb, N, sa, sb, (size_t)M * N, alpha, 0, mask, NB, a.stream, x2);
    if (gerr == hipSuccess) gerr = e;
  };
  const std::integral_constant<int, kGemmDual> dual;
  const size_t scd = (size_t)C * D, sdd = (size_t)D * D;
  const GemmNT NT;
  // Segment s: its geometry, then prep, the Grams, the inverse (through the
  // forward operands of the serial pass); `grams_p` adds P.
  auto segment_setup = [&](int s, bool grams_p) {
    geo.c0 = s * plan.L;
    const long long slots = sc.slots(geo.c0, plan.L);
    NB = (size_t)slots * a.H;
    geo.nchunks = (int)slots;
    if (a.cu_seqlens) {
      hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens,
                         const_cast<int32_t*>(geo.off), a.num_seqs, a.total_tokens, C, geo.c0, plan.L);
      geo.slot_cnt = 0;
    } else {
      const int c = sc.nch(0) - geo.c0;
      geo.slot_cnt = c <= 0 ? 0 : (c < plan.L ? c : plan.L);
    }
    if (NB == 0) return;
    hipLaunchKernelGGL((bwd_prep_kernel<in_t, D, C>), dim3(NB), dim3(256), 0, a.stream, in, p, geo);
    // Grams of the moderate-decay chunks, then the others pair by pair.
    if (grams_p) {  // strict_tril(Kt Kh^T) and tril(Qt Kh^T), Kh read once
      GemmX x2;
      x2.A2 = p.Qt;
      x2.C2 = p.P;
      x2.mask2 = 1;
      gemm2(NT, dual, p.Kt, p.Kh, p.Bm, C, C, D, D, D, scd, scd, 1.f, 2, x2);
    } else {
      gemm(NT, p.Kt, p.Kh, p.Bm, C, C, D, D, D, scd, scd, 1.f, 0, 2);  // strict_tril(Kt Kh^T)
    }
    hipLaunchKernelGGL((bwd_gram_tile_kernel<D, C>), dim3(NB), dim3(256), tlds, a.stream, p);
    hipLaunchKernelGGL((unit_lower_inverse_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p.Bm, p.beta,
                       p.M, p.T);
  };
  // Forward sweep: the state entering every segment after the first (only
  // the serial forward pass of each segment is needed for it).
  for (int s = 0; s + 1 < plan.nseg; ++s) {
    segment_setup(s, false);
    if (serial > 0)
      hipLaunchKernelGGL((bwd_fwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), flds_s, a.stream,
                         p, geo, state_in(s), ckpt + (size_t)s * nhdd);
  }
  // Backward sweep, last segment first; dS crosses segments in dcarry.
  for (int s = plan.nseg - 1; s >= 0; --s) {
    segment_setup(s, true);
    const float* ds_in = s == plan.nseg - 1 ? a.d_final_state : dcarry;
    float* ds_out = s == 0 ? a.d_initial_state : dcarry;
    if (serial > 0) {
      if (NB > 0)
        hipLaunchKernelGGL((bwd_fwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), flds_s, a.stream,
                           p, geo, state_in(s), static_cast<float*>(nullptr));
      // (with no chunk in the segment this only hands dS through)
      hipLaunchKernelGGL((bwd_bwd_states_kernel<D, C>), dim3(serial), dim3(kSerThreads), blds_s, a.stream,
                         p, geo, ds_in, ds_out);
    }
    if (NB == 0) continue;
    // p.S and p.dSn are [D][D] per chunk and head: the B operand "rows" are
    // the key channels, contracted over the value columns.
    {  // dQt = dO S^T and dKt = -dR S^T, S read once
      GemmX x2;
      x2.A2 = p.dR;
      x2.C2 = p.dKt;
      x2.alpha2 = -1.f;
      gemm2(NT, dual, p.dO, p.S, p.dQt, C, D, D, D, D, scd, sdd, 1.f, 0, x2);
    }
    gemm(NT, p.U, p.dSn, p.dKb, C, D, D, D, D, scd, sdd, 1.f, 0, 0);  // dKb = U dS'^T
    gemm(NT, p.dU, p.R, p.dT, C, C, D, D, D, scd, scd, 1.f, 0, 0);    // dT = dU R^T
    gemm(NT, p.dO, p.U, p.dP, C, C, D, D, D, scd, scd, 1.f, 0, 1);    // dP = tril(dO U^T)
    hipLaunchKernelGGL((bwd_cc_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p);
    if (gerr != hipSuccess) return gerr;
    // Pairwise gradient terms: Z1..Z3 of the strong-decay chunks into the R,
    // U, dU planes (free by now), then the final pass, which forms those of
    // the other chunks itself.
    hipLaunchKernelGGL((bwd_pairs_tile_kernel<D, C>), dim3(NB), dim3(256), tlds, a.stream, p);
    hipLaunchKernelGGL((bwd_final_prod_kernel<D, C>), dim3((NB + 7) / 8 * 8 * (D / 64)), dim3(256), 0, a.stream,
                       p, geo, out, (int)NB);
  }
  if (gerr != hipSuccess) return gerr;
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

size_t backward_workspace_bytes(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D, int chunk,
                                const PrefillTuning& tuning) {
  const BwdPlan plan = plan_backward(num_seqs, cu_host, seq_len, H, D, chunk, tuning);
  if (plan.nseg == 0) return SIZE_MAX;
  return bwd_bytes(plan, num_seqs, cu_host != nullptr, H, D, chunk);
}

hipError_t launch_backward(const BackwardArgs& a) {
  return a.in_bf16 ? launch_backward_i<bf16>(a) : launch_backward_i<float>(a);
}

}  // namespace kda
