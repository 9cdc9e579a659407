// General diagonal-plus-low-rank (DPLR) chunked forward pass, gfx950, fp32.
//
//   S_t = (Diag(exp g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
//
// (zeroshot.it.com deep-dive, section 3.2 "DPLR Structure"; greeksharifa
// summary, section 6.2 "Relation to DPLR": KDA is the case a = beta k,
// b = k * alpha with the write beta k v^T, and needs two of the general
// form's four intra-chunk matrices).  For a chunk of C rows (zero-padded; g = 0
// on padded rows) entering with state S, Gamma = cumsum(g), Gamma' = Gamma - g
// (decay up to the previous row), gam_n = exp(Gamma_{C-1}):
//
//   Qt = q e^Gamma,  Bt = b e^Gamma',  Ah = a e^-Gamma,  Kh = k e^-Gamma,
//   Ab = a e^(Gamma_n - Gamma),  Kb = k e^(Gamma_n - Gamma)
//   Aba = strict_tril(Bt Ah^T), Abk = strict_tril(Bt Kh^T),
//   Aqa = tril(Qt Ah^T),        Aqk = tril(Qt Kh^T)
//   M = (I + Aba)^{-1}
//   U = -M (Bt S + Abk V)        (U row r = -b_r^T S_{r-1})
//   O = Qt S + Aqa U + Aqk V,    S' = Diag(gam_n) S + Ab^T U + Kb^T V
//
// With the tied (KDA) structure a = k_w = beta k, b = alpha k, so Aba = Abk,
// Aqa = Aqk and Ab = Kb; then U~ = U + V = M (V - Bt S) and O = Qt S + Aqa U~,
// S' = Diag(gam_n) S + Ab^T U~: two Grams and two products fewer.  The tied
// mode runs KDA through this same pipeline, the like-for-like baseline for the
// general form's extra work.
//
// Grams of chunks whose decay span (max -Gamma_{C-1}) is at most 40 are
// products of the factored operands; others are factored per 16-row tile
// (dplr_gram_tile_kernel), still on the matrix units.
//
// Kernels: chunk_table_kernel (varlen), dplr_prep_kernel, fp32_gemm_kernel
// (Grams, then Wb = M Bt, the V terms), dplr_gram_tile_kernel (strong decay),
// unit_lower_inverse_kernel (M), dplr_states_kernel (serial over chunks per
// (sequence, head, 16 value columns), fp32 MFMA, writes o and the final state).
#include "kda_device.hpp"
#include "kda_fp32_chunks.hpp"
#include "kda_launch.hpp"

#include <type_traits>

namespace kda {
namespace {

constexpr int kColsD = 16;
constexpr float kSpanD = 40.f;

struct DPlanes {
  float *Q, *K, *V, *A, *B, *Gam, *G;   // padded inputs (A, B: the low-rank factors), Gamma, g
  float *Qt, *Bt, *Ah, *Kh, *Ab, *Kb;   // decayed operands
  float *Wb, *Y, *OV, *X;               // Wb = M Bt; Y = M V (tied) or -M Abk V; OV = Aqk V
  float *Aba, *Abk, *Aqa, *Aqk, *M;     // [C][C]
  float* gn;                            // [D]
  int32_t* fast;
};

size_t dplr_plane_bytes(size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4);
  return 17 * cd + 5 * cc + a256(NB * D * 4) + a256(NB * 4);
}

DPlanes dcarve(char* p, size_t NB, int C, int D) {
  const size_t cd = a256(NB * C * D * 4), cc = a256(NB * C * C * 4);
  DPlanes x;
  float** cdp[] = {&x.Q, &x.K, &x.V, &x.A, &x.B, &x.Gam, &x.G, &x.Qt, &x.Bt,
                   &x.Ah, &x.Kh, &x.Ab, &x.Kb, &x.Wb, &x.Y, &x.OV, &x.X};
  for (float** f : cdp) { *f = reinterpret_cast<float*>(p); p += cd; }
  float** ccp[] = {&x.Aba, &x.Abk, &x.Aqa, &x.Aqk, &x.M};
  for (float** f : ccp) { *f = reinterpret_cast<float*>(p); p += cc; }
  x.gn = reinterpret_cast<float*>(p);
  p += a256(NB * D * 4);
  x.fast = reinterpret_cast<int32_t*>(p);
  return x;
}

struct DIn {
  const void *q, *k, *v, *a, *b;  // a, b unused when tied
  const float *g, *beta;          // beta used when tied
};

// Padded fp32 inputs, Gamma, the decayed operands and the span verdict.
template <class in_t, int D, int C, bool TIED>
__global__ __launch_bounds__(256) void dplr_prep_kernel(DIn in, DPlanes p, Geo geo) {
  // Four consecutive channels per thread: 16-byte loads and stores.
  constexpr int SG = D + 4;
  __shared__ __attribute__((aligned(16))) float Gs[C][SG];
  const int b = blockIdx.x, H = geo.H;
  const int gch = b / H, h = b % H;
  int n, t0, len;
  chunk_of<C>(geo, gch, n, t0, len);
  const size_t pcd = (size_t)b * C * D;
  auto ld4 = [&](const void* ptr, size_t ti) -> f32x4 {
    if constexpr (std::is_same<in_t, float>::value) {
      return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(ptr) + ti);
    } else {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const in_t*>(ptr) + ti);
      return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
  };
  auto st4 = [&](float* plane, int idx, f32x4 x) { *reinterpret_cast<f32x4*>(plane + pcd + idx) = x; };
  auto ld4p = [&](const float* plane, int idx) { return *reinterpret_cast<const f32x4*>(plane + pcd + idx); };
  // Inputs are loaded unconditionally (rows past the chunk re-read its first
  // row) and zeroed after, and each vector's loads are issued before the
  // previous vector's stores: a load under the row test made every one wait
  // for the last, and the compiler may not move a load above a store that
  // could alias it.
  constexpr int NV = C * D / 4 / 256;
  static_assert(NV * 256 * 4 == C * D, "whole vectors per thread");
  f32x4 kl[2], gl4[2], ql[2], vl[2], al[2], bl[2];
  float bel[2];
  auto fetch = [&](int x) {
    const int idx = 4 * ((int)threadIdx.x + 256 * x), r = idx / D, c = idx % D;
    const int rr = r < len ? r : 0, s2 = x & 1;
    const size_t ti = ((size_t)(t0 + rr) * H + h) * D + c;
    kl[s2] = ld4(in.k, ti);
    gl4[s2] = *reinterpret_cast<const f32x4*>(in.g + ti);
    ql[s2] = ld4(in.q, ti);
    vl[s2] = ld4(in.v, ti);
    if (TIED) {
      bel[s2] = in.beta[(size_t)(t0 + rr) * H + h];
    } else {
      al[s2] = ld4(in.a, ti);
      bl[s2] = ld4(in.b, ti);
    }
  };
  fetch(0);
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    if (x + 1 < NV) fetch(x + 1);
    const int idx = 4 * ((int)threadIdx.x + 256 * x), r = idx / D, c = idx % D, s2 = x & 1;
    const bool ok = r < len;
    const f32x4 z = {0, 0, 0, 0};
    const f32x4 kv = ok ? kl[s2] : z, gv = ok ? gl4[s2] : z;
    f32x4 av, bv;
    if (TIED) {
      const float be = ok ? bel[s2] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = be * kv[e];               // a = write key = beta k
        bv[e] = __expf(gv[e]) * kv[e];    // b = alpha k
      }
    } else {
      av = ok ? al[s2] : z;
      bv = ok ? bl[s2] : z;
    }
    st4(p.Q, idx, ok ? ql[s2] : z);
    st4(p.K, idx, TIED ? av : kv);  // the key that writes v
    st4(p.V, idx, ok ? vl[s2] : z);
    st4(p.A, idx, av);
    st4(p.B, idx, bv);
    st4(p.G, idx, gv);
    *reinterpret_cast<f32x4*>(&Gs[r][c]) = gv;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float s = 0.f;
    for (int r = 0; r < C; ++r) {
      s += Gs[r][c];
      Gs[r][c] = s;
    }
    p.gn[(size_t)b * D + c] = __expf(s);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    bool big = false;
    for (int c = threadIdx.x; c < D; c += 64) big |= Gs[C - 1][c] < -kSpanD;
    big = __any(big);
    if (threadIdx.x == 0) p.fast[b] = big ? 0 : 1;
  }
  // The planes written above are read back (from L2) a vector ahead of the
  // stores that could alias them, as in the first loop.
  f32x4 rav[2], rkv[2], rqv[2], rbv[2], rgv[2];
  auto refetch = [&](int x) {
    const int idx = 4 * ((int)threadIdx.x + 256 * x), s2 = x & 1;
    rav[s2] = ld4p(p.A, idx);
    rkv[s2] = ld4p(p.K, idx);
    rqv[s2] = ld4p(p.Q, idx);
    rbv[s2] = ld4p(p.B, idx);
    rgv[s2] = ld4p(p.G, idx);
  };
  refetch(0);
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    if (x + 1 < NV) refetch(x + 1);
    const int idx = 4 * ((int)threadIdx.x + 256 * x), r = idx / D, c = idx % D, s2 = x & 1;
    const f32x4 gm = *reinterpret_cast<const f32x4*>(&Gs[r][c]);
    const f32x4 gl = *reinterpret_cast<const f32x4*>(&Gs[C - 1][c]);
    const f32x4 av = rav[s2], kv = rkv[s2], qv = rqv[s2], bv = rbv[s2], gv = rgv[s2];
    f32x4 qt, bt, ah, kh, ab, kb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ea = __expf(gm[e]), eh = __expf(-gm[e]), eb = __expf(gl[e] - gm[e]);
      qt[e] = qv[e] * ea;
      bt[e] = bv[e] * __expf(gm[e] - gv[e]);
      ah[e] = av[e] * eh;  // finite where the chunk is factored
      kh[e] = kv[e] * eh;
      ab[e] = av[e] * eb;
      kb[e] = kv[e] * eb;
    }
    st4(p.Gam, idx, gm);
    st4(p.Qt, idx, qt);
    st4(p.Bt, idx, bt);
    st4(p.Ah, idx, ah);
    st4(p.Kh, idx, kh);
    st4(p.Ab, idx, ab);
    st4(p.Kb, idx, kb);
  }
}

// Strong-decay chunks: the four (tied: two) Grams pair by pair with the
// exact exponent of each difference.  Lane = row r; waves step through i.
// Strong-decay chunks (span > kSpanD), factored per 16-row tile: with
// Gamma_s(a) the cumulative decay before tile a and Gamma_e(b) at the end of
// tile b, for rows r of tile a and columns i of tile b <= a
//   exp(X_r - Gamma_i) = exp(X_r - Gamma_s(a)) f_ab exp(Gamma_e(b) - Gamma_i),
//   f_ab = exp(Gamma_s(a) - Gamma_e(b)),
// where X_r is Gamma_r (rows of Q) or Gamma'_r = Gamma_r - g_r (rows of B):
// every factor <= 1 off the diagonal; on the diagonal f_aa = exp(span of
// tile a), in range up to a span of kTileSpanD, beyond which the diagonal
// block is summed pair by pair.  Blocks run on v_mfma_f32_16x16x4f32 with the
// bridge factor on the column operand, channel by channel.
constexpr float kTileSpanD = 64.f;

template <int D, int C>
struct DTileLds {
  static constexpr int NT = C / 16, SD = D + 4;
  float Br[C][SD], Qr[C][SD], Ac[C][SD], Kc[C][SD];
  float Gs[NT][D], Ge[NT][D];
};

template <int D, int C, bool TIED>
__global__ __launch_bounds__(256) void dplr_gram_tile_kernel(DPlanes p) {
  extern __shared__ float sm[];
  DTileLds<D, C>& L = *reinterpret_cast<DTileLds<D, C>*>(sm);
  constexpr int NT = C / 16, NBLK = NT * (NT + 1) / 2;
  const size_t b = blockIdx.x;
  if (p.fast[b]) return;  // formed as products
  const size_t pcd = b * C * D, pcc = b * C * C;
  // Every staging load before the first LDS write (a loop that waited for
  // each element's loads took most of the kernel's time).
  constexpr int NI = C * D / 256, NG = (NT * D + 255) / 256;
  static_assert(NI * 256 == C * D, "whole elements per thread");
  const int tid = threadIdx.x;
  float gmv[NI], qv[NI], bv[NI], gv[NI], av[NI], kv[NI], gsv[NG], gev[NG];
#pragma unroll
  for (int x = 0; x < NI; ++x) {
    const size_t e = pcd + tid + 256 * x;
    gmv[x] = p.Gam[e];
    qv[x] = p.Q[e];
    bv[x] = p.B[e];
    gv[x] = p.G[e];
    av[x] = p.A[e];
    kv[x] = TIED ? 0.f : p.K[e];
  }
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    const int idx = min(tid + 256 * x, NT * D - 1), t = idx / D, c = idx % D;
    gsv[x] = p.Gam[pcd + (size_t)(t == 0 ? 0 : 16 * t - 1) * D + c];
    gev[x] = p.Gam[pcd + (size_t)(16 * t + 15) * D + c];
  }
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    const int idx = tid + 256 * x, t = idx / D, c = idx % D;
    if (NT * D % 256 == 0 || idx < NT * D) {
      L.Gs[t][c] = t == 0 ? 0.f : gsv[x];
      L.Ge[t][c] = gev[x];
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NI; ++x) {
    const int idx = tid + 256 * x, r = idx / D, c = idx % D, t = r / 16;
    const float gm = gmv[x], gs = L.Gs[t][c], ce = __expf(L.Ge[t][c] - gm);
    L.Qr[r][c] = qv[x] * __expf(gm - gs);
    L.Br[r][c] = bv[x] * __expf(gm - gv[x] - gs);
    L.Ac[r][c] = av[x] * ce;
    if (!TIED) L.Kc[r][c] = kv[x] * ce;
  }
  bool bad[NT];
  for (int t = 0; t < NT; ++t) {
    bool big = false;
    for (int c = lane_id(); c < D; c += 64) big |= L.Ge[t][c] - L.Gs[t][c] < -kTileSpanD;
    bad[t] = __any(big);
  }
  __syncthreads();
  const int w = wave_id(), l = lane_id(), m = l & 15, g = l >> 4;
  for (int blk = w; blk < NBLK; blk += 4) {
    int ta = 0;
    while ((ta + 1) * (ta + 2) / 2 <= blk) ++ta;
    const int tb = blk - ta * (ta + 1) / 2;
    f32x4 ba = {0, 0, 0, 0}, qa = ba, bk = ba, qk = ba;
    if (tb < ta || !bad[ta]) {
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const int c = k0 + g;
        const float f = __expf(L.Gs[ta][c] - L.Ge[tb][c]);
        const float ac = L.Ac[16 * tb + m][c] * f;
        ba = mfma4(L.Br[16 * ta + m][c], ac, ba);
        qa = mfma4(L.Qr[16 * ta + m][c], ac, qa);
        if (!TIED) {
          const float kc = L.Kc[16 * tb + m][c] * f;
          bk = mfma4(L.Br[16 * ta + m][c], kc, bk);
          qk = mfma4(L.Qr[16 * ta + m][c], kc, qk);
        }
      }
    } else {
      // tile span beyond kTileSpanD: each pair with its exact exponents
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const size_t rr = 16 * ta + 4 * g + x, ii = 16 * tb + m;
        if (ii > rr) continue;
        for (int c = 0; c < D; ++c) {
          const float gi = p.Gam[pcd + ii * D + c], gr = p.Gam[pcd + rr * D + c];
          const float eq = __expf(gr - gi), eb = __expf(gr - p.G[pcd + rr * D + c] - gi);
          const float ai = p.A[pcd + ii * D + c];
          ba[x] += p.B[pcd + rr * D + c] * ai * eb;
          qa[x] += p.Q[pcd + rr * D + c] * ai * eq;
          if (!TIED) {
            const float ki = p.K[pcd + ii * D + c];
            bk[x] += p.B[pcd + rr * D + c] * ki * eb;
            qk[x] += p.Q[pcd + rr * D + c] * ki * eq;
          }
        }
      }
    }
    // lane (m, g) holds rows 4 g + x of column m of the block
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = 16 * ta + 4 * g + x, i = 16 * tb + m;
      p.Aba[pcc + r * C + i] = i < r ? ba[x] : 0.f;
      p.Aqa[pcc + r * C + i] = i <= r ? qa[x] : 0.f;
      if (!TIED) {
        p.Abk[pcc + r * C + i] = i < r ? bk[x] : 0.f;
        p.Aqk[pcc + r * C + i] = i <= r ? qk[x] : 0.f;
      }
    }
  }
  for (int idx = threadIdx.x; idx < C * C; idx += 256) {  // blocks above the diagonal
    const int r = idx / C, i = idx % C;
    if (i / 16 > r / 16) {
      p.Aba[pcc + idx] = 0.f;
      p.Aqa[pcc + idx] = 0.f;
      if (!TIED) {
        p.Abk[pcc + idx] = 0.f;
        p.Aqk[pcc + idx] = 0.f;
      }
    }
  }
}

template <int D, int C>
struct StLds {
  union {
    struct {
      float Wb[C][D + 4];
      float Qt[C][D + 4];
      float Aqa[C][C + 4];
    } a;
    struct {
      float Ab[C][D + 16];   // read transposed
      float Kb[C][D + 16];   // read transposed
    } b;
  } u;
  float S[D][kColsD];
  float U[C][kColsD];
  float Yb[C][kColsD];
  float Vb[C][kColsD];
  float OV[C][kColsD];
  float gn[D];
};

constexpr int kStThreads = 512;

// Serial pass over a sequence's chunks for 16 value columns:
//   U~ = Y - Wb S;  O = Qt S + Aqa U~ (+ Aqk V);  S' = gam_n S + Ab^T U~ (+ Kb^T V)
// (general form: U~ = U, Y = -M Abk V; tied: U~ = U + V, Y = M V).  Eight
// waves; the next chunk's Wb, Qt, Aqa are loaded into registers while this
// chunk computes, and this chunk's Ab, Kb while its first half computes.
template <int D, int C, bool TIED>
__global__ __launch_bounds__(kStThreads) void dplr_states_kernel(DPlanes p, Geo geo,
                                                                 const float* __restrict__ s0,
                                                                 float* __restrict__ s1,
                                                                 float* __restrict__ o) {
  extern __shared__ float sm[];
  StLds<D, C>& L = *reinterpret_cast<StLds<D, C>*>(sm);
  constexpr int NVB = D / kColsD, NT = kStThreads, NW = NT / 64;
  const int H = geo.H;
  int nh, vb;
  if (!serial_slot<NVB>(geo.num_seqs * H, nh, vb)) return;
  const int n = nh / H, h = nh % H, col0 = vb * kColsD;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  int bos, eos, base;
  seq_of<C>(geo, n, bos, eos, base);
  const int nch = (eos - bos + C - 1) / C;
  for (int idx = tid; idx < D * kColsD; idx += NT) {
    const int i = idx / kColsD, j = idx % kColsD;
    L.S[i][j] = s0 ? s0[(((size_t)n * H + h) * D + i) * D + col0 + j] : 0.f;
  }
  Prefetch<C, D, NT> pW, pQ, pA, pK;
  Prefetch<C, C, NT> pP;
  Prefetch<C, kColsD, NT, D> pY, pV, pOV;  // this workgroup's value columns
  Prefetch<1, D, NT> pG;                   // gam_n
  auto blk = [&](int ci) { return (size_t)(base + ci) * H + h; };
  // The first-half operands of a chunk (and its value-column slices and
  // gam_n) load a step ahead; Ab and Kb at the start of their chunk.
  auto fetch = [&](size_t b) {
    pW.load(p.Wb + b * C * D);
    pQ.load(p.Qt + b * C * D);
    pP.load(p.Aqa + b * C * C);
    pY.load(p.Y + b * C * D + col0);
    if (!TIED) {
      pV.load(p.V + b * C * D + col0);
      pOV.load(p.OV + b * C * D + col0);
    }
    pG.load(p.gn + b * D);
  };
  if (nch > 0) fetch(blk(0));
  for (int ci = 0; ci < nch; ++ci) {
    const size_t b = blk(ci);
    const size_t pcd = b * C * D;
    const int t0 = bos + ci * C, len = min(C, eos - t0);
    __syncthreads();  // the previous chunk's reads of the union are done
    pW.template store<D + 4>(&L.u.a.Wb[0][0]);
    pQ.template store<D + 4>(&L.u.a.Qt[0][0]);
    pP.template store<C + 4>(&L.u.a.Aqa[0][0]);
    pY.template store<kColsD>(&L.Yb[0][0]);
    if (!TIED) {
      pV.template store<kColsD>(&L.Vb[0][0]);
      pOV.template store<kColsD>(&L.OV[0][0]);
    }
    pG.template store<D>(&L.gn[0]);
    pA.load(p.Ab + pcd);
    if (!TIED) pK.load(p.Kb + pcd);
    __syncthreads();
    if (ci + 1 < nch) fetch(blk(ci + 1));
    for (int rt = w; rt < C / 16; rt += NW) {  // U~ = Y - Wb S
      f32x4 acc = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 8) {
        acc = mfma4(L.u.a.Wb[16 * rt + m][k0 + g], L.S[k0 + g][m], acc);
        acc1 = mfma4(L.u.a.Wb[16 * rt + m][k0 + 4 + g], L.S[k0 + 4 + g][m], acc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        L.U[r][m] = L.Yb[r][m] - acc[i] - acc1[i];
      }
    }
    __syncthreads();
    for (int rt = w; rt < C / 16; rt += NW) {  // O = Qt S + Aqa U~ (+ OV)
      f32x4 acc = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 4) acc = mfma4(L.u.a.Qt[16 * rt + m][k0 + g], L.S[k0 + g][m], acc);
      for (int k0 = 0; k0 < 16 * (rt + 1); k0 += 4) acc1 = mfma4(L.u.a.Aqa[16 * rt + m][k0 + g], L.U[k0 + g][m], acc1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        float x = acc[i] + acc1[i];
        if (!TIED) x += L.OV[r][m];
        if (r < len) o[((size_t)(t0 + r) * H + h) * D + col0 + m] = x;
      }
    }
    __syncthreads();
    pA.template store<D + 16>(&L.u.b.Ab[0][0]);
    if (!TIED) pK.template store<D + 16>(&L.u.b.Kb[0][0]);
    __syncthreads();
    for (int t = w; t < D / 16; t += NW) {  // S = gam_n S + Ab^T U~ (+ Kb^T V)
      f32x4 acc, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * t + 4 * g + i;
        acc[i] = L.gn[c] * L.S[c][m];
      }
#pragma unroll 8
      for (int k0 = 0; k0 < C; k0 += 4) {
        acc = mfma4(L.u.b.Ab[k0 + g][16 * t + m], L.U[k0 + g][m], acc);
        if (!TIED) acc1 = mfma4(L.u.b.Kb[k0 + g][16 * t + m], L.Vb[k0 + g][m], acc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) L.S[16 * t + 4 * g + i][m] = acc[i] + acc1[i];
    }
  }
  __syncthreads();
  if (s1) {
    for (int idx = tid; idx < D * kColsD; idx += NT) {
      const int i = idx / kColsD, j = idx % kColsD;
      s1[(((size_t)n * H + h) * D + i) * D + col0 + j] = L.S[i][j];
    }
  }
}

template <class in_t, int D, int C, bool TIED>
hipError_t launch_dplr_t(const DplrArgs& a) {
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
  geo.c0 = 0;  // one pass over every chunk
  geo.L = INT32_MAX / 2;
  geo.slot_cnt = a.cu_seqlens ? 0 : (a.seq_len + C - 1) / C;
  DPlanes p = dcarve(ws + a256(sizeof(int32_t) * (a.num_seqs + 1)), NB, C, D);
  if (a.cu_seqlens)
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens,
                       const_cast<int32_t*>(geo.off), a.num_seqs, a.total_tokens, C, 0, INT32_MAX / 2);
  const int serial = serial_blocks(a.num_seqs * a.H, D / kColsD);
  const size_t slds = sizeof(StLds<D, C>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dplr_states_kernel<D, C, TIED>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)slds);
  if (e != hipSuccess) return e;
  static_assert(sizeof(DTileLds<D, C>) <= 160 * 1024, "tile operands fit LDS");
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dplr_gram_tile_kernel<D, C, TIED>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(DTileLds<D, C>));
  if (e != hipSuccess) return e;
  // bf16 inputs: batched products on split-bf16 operands; fp32 inputs: fp32.
  constexpr bool kSplitGemm = sizeof(in_t) == 2;
  if (NB > 0) {
    DIn in{a.q, a.k, a.v, a.a, a.b, a.g, a.beta};
    hipLaunchKernelGGL((dplr_prep_kernel<in_t, D, C, TIED>), dim3(NB), dim3(256), 0, a.stream, in,
                       p, geo);
    hipError_t gerr = hipSuccess;
    auto gemm = [&](auto op, const float* A, const float* B, float* Cm, int M, int N, int K,
                    int lda, int ldb, size_t sa, size_t sb, float alpha, int mask) {
      typedef decltype(op) O;
      const hipError_t e = launch_fp32_gemm<O::TA, O::TB, kGemmOne, kSplitGemm>(
          A, B, Cm, M, N, K, lda, ldb, N, sa, sb, (size_t)M * N, alpha, 0, mask, NB, a.stream);
      if (gerr == hipSuccess) gerr = e;
    };
    // Two products sharing B (and its load) in one launch.
    auto gemm_dual = [&](auto op, const float* A, const float* B, float* Cm, int M, int N, int K, int lda,
                         int ldb, size_t sa, size_t sb, int mask, const float* A2, float* C2, int mask2) {
      typedef decltype(op) O;
      GemmX x2;
      x2.A2 = A2;
      x2.C2 = C2;
      x2.mask2 = mask2;
      const hipError_t e = launch_fp32_gemm<O::TA, O::TB, kGemmDual, kSplitGemm>(
          A, B, Cm, M, N, K, lda, ldb, N, sa, sb, (size_t)M * N, 1.f, 0, mask, NB, a.stream, x2);
      if (gerr == hipSuccess) gerr = e;
    };
    const size_t scd = (size_t)C * D, scc = (size_t)C * C;
    const GemmNT NT;
    const GemmNN NN;
    // strict_tril(Bt Ah^T) and tril(Qt Ah^T)
    gemm_dual(NT, p.Bt, p.Ah, p.Aba, C, C, D, D, D, scd, scd, 2, p.Qt, p.Aqa, 1);
    if (!TIED)  // strict_tril(Bt Kh^T) and tril(Qt Kh^T)
      gemm_dual(NT, p.Bt, p.Kh, p.Abk, C, C, D, D, D, scd, scd, 2, p.Qt, p.Aqk, 1);
    hipLaunchKernelGGL((dplr_gram_tile_kernel<D, C, TIED>), dim3(NB), dim3(256), sizeof(DTileLds<D, C>),
                       a.stream, p);
    hipLaunchKernelGGL((unit_lower_inverse_kernel<C>), dim3(NB), dim3(256), 0, a.stream, p.Aba,
                       (const float*)nullptr, p.M, (float*)nullptr);
    gemm(NN, p.M, p.Bt, p.Wb, C, D, C, C, D, scc, scd, 1.f, 0);      // Wb = M Bt
    if (TIED) {
      gemm(NN, p.M, p.V, p.Y, C, D, C, C, D, scc, scd, 1.f, 0);      // Y = M V
    } else {
      gemm_dual(NN, p.Abk, p.V, p.X, C, D, C, C, D, scc, scd, 0, p.Aqk, p.OV, 0);  // X = Abk V, OV = Aqk V
      gemm(NN, p.M, p.X, p.Y, C, D, C, C, D, scc, scd, -1.f, 0);     // Y = -M X
    }
    if (gerr != hipSuccess) return gerr;
  }
  if (serial > 0)
    hipLaunchKernelGGL((dplr_states_kernel<D, C, TIED>), dim3(serial), dim3(kStThreads), slds, a.stream,
                       p, geo, a.initial_state, a.final_state, a.o);
  return hipGetLastError();
}

template <class in_t, bool TIED>
hipError_t launch_dplr_i(const DplrArgs& a) {
  if (a.D == 64) {
    if (a.chunk == 16) return launch_dplr_t<in_t, 64, 16, TIED>(a);
    if (a.chunk == 32) return launch_dplr_t<in_t, 64, 32, TIED>(a);
    return launch_dplr_t<in_t, 64, 64, TIED>(a);
  }
  if (a.chunk == 16) return launch_dplr_t<in_t, 128, 16, TIED>(a);
  if (a.chunk == 32) return launch_dplr_t<in_t, 128, 32, TIED>(a);
  return launch_dplr_t<in_t, 128, 64, TIED>(a);
}

}  // namespace

size_t dplr_workspace_bytes(long long total_chunks, int num_seqs, int H, int D, int chunk) {
  return a256(sizeof(int32_t) * (size_t)(num_seqs + 1)) +
         dplr_plane_bytes((size_t)total_chunks * H, chunk, D);
}

hipError_t launch_dplr(const DplrArgs& a) {
  if (a.tied)
    return a.in_bf16 ? launch_dplr_i<bf16, true>(a) : launch_dplr_i<float, true>(a);
  return a.in_bf16 ? launch_dplr_i<bf16, false>(a) : launch_dplr_i<float, false>(a);
}

}  // namespace kda
