// KDA single-token recurrent step (generation), gfx950.
//
// For each (sequence n, head h) one workgroup streams the Dk x Dv fp32 state
// through registers exactly once:
//   S' = Diag(exp g) S               (decay first)
//   r  = S'^T k,  p = S'^T q,  kq = k . q
//   u  = beta (v - r)
//   S  = S' + k u^T                  (delta correction + write)
//   o  = S^T q = p + kq * u          (read from the updated state)
// Source: greeksharifa.github.io summary of the Kimi Linear report, section 3
// (recurrence, decay before correction) and section 6.3 (generation runs the
// recurrent update).
//
// Work split: 256 threads.  TPR = Dv/4 threads cover one state row with one
// float4 each (a row is one contiguous 512 B / 256 B segment), and the
// 256/TPR row groups stride over the Dk rows.  Each thread keeps its rows in
// registers between the read and the write, so HBM sees 2 * Dk * Dv * 4
// bytes per (n, h) plus the small per-token vectors.  The column reductions
// over rows run in registers, then across the lanes of a wave with xor
// shuffles, then across the four waves through LDS.
//
// LAYER adds the layer's elementwise work (the "Kimi Linear" notes,
// docsaid.org, section "Other Components"): the short causal convolution of
// q, k and v (weight W-1 on the new token, the others on the carried inputs),
// Swish and L2 normalisation of q and k, Swish of v and the sigmoid of beta on
// the way in, and with a gate the head-wise RMSNorm times sigmoid(gate) on the
// way out.  The norms of q and k are scalars per (n, h), so the reductions run
// on the un-normalised values and are rescaled once the norms are known.  One
// thread per (tensor, channel) convolves and shifts that channel's carried
// inputs; the results reach the other threads through LDS.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

struct LayerPtrs {
  int prologue;
  const void* gate;  // nullptr: no epilogue
  const float* norm_weight;
  float norm_eps;
  // short convolution of q, k, v before Swish: width (0 = none), weights
  // [H][D][conv_w], carried inputs [N][H][conv_w - 1][D] read from cs_in
  // and shifted into cs_out (either may be nullptr; they may be equal)
  int conv_w, H;
  const float* cw[3];
  const void* cs_in[3];
  void* cs_out[3];
};

// Hardware reciprocal (about 1 ulp) instead of a correctly rounded
// division; 1 / inf is 0, so large |x| give the limits.
__device__ __forceinline__ float sigmoid_d(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float swish_d(float x) { return x * sigmoid_d(x); }

// An input element kept as loaded, widened to 32 bits (a bf16 in the low
// half): 16-bit values held this way are not packed in pairs, which would make
// the compiler wait for the loads where they are issued.
__device__ __forceinline__ unsigned raw32(const bf16* p) {
  return *reinterpret_cast<const unsigned short*>(p);
}
__device__ __forceinline__ unsigned raw32(const float* p) { return __builtin_bit_cast(unsigned, *p); }
template <typename T>
__device__ __forceinline__ float raw_to_f(unsigned u) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(float, u << 16);  // bf16 is the high half of an fp32
  else
    return __builtin_bit_cast(float, u);
}
template <typename T>
__device__ __forceinline__ T raw_to_t(unsigned u) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(T, (unsigned short)u);
  else
    return __builtin_bit_cast(T, u);
}

// SG: scalar gate (Gated DeltaNet): g holds one log-decay per (n, h).
template <typename in_t, int DK, int DV, bool OUT_BF16, bool SG, bool LAYER>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const in_t* __restrict__ q, const in_t* __restrict__ k, const in_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, int NH, LayerPtrs lp) {
  constexpr int TPR = DV / 4;          // threads per state row
  constexpr int RG = 256 / TPR;        // row groups
  constexpr int RPT = DK / RG;         // rows per thread
  static_assert(RPT * RG == DK, "row split");

  const int nh = blockIdx.x;
  if (nh >= NH) return;
  const int t = threadIdx.x;
  const int cg = t % TPR;
  const int rg = t / TPR;

  const size_t tok = (size_t)nh;
  const in_t* qp = q + tok * DK;
  const in_t* kp = k + tok * DK;
  const float* gp = g + tok * (SG ? 1 : DK);
  const float ag = SG ? __expf(gp[0]) : 0.f;
  float* sp = state + tok * (size_t)DK * DV;

  float kk[RPT], qq[RPT], ga[RPT];
  f32x4 s[RPT];
  const int W1 = LAYER ? lp.conv_w - 1 : -1;
  const bool conv = LAYER && W1 >= 0;
  auto load_state = [&]() {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = rg + RG * m;
      s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)i * DV + 4 * cg));
    }
  };
  // Every per-token input is requested with the state and before any wait:
  // a small load issued after a wait (the compiler had put v after the state
  // had arrived and beta after the cross-wave barrier) is a memory round trip
  // of its own between the reduction and the write-back, 3 % of the step.
  // Without the layer's convolution the inputs go first, so each state row is
  // decayed and reduced as soon as it arrives.  Values are kept as loaded
  // (raw32), addresses are clamped instead of branched on, and the scheduling
  // barrier keeps the compiler from sinking the loads to their first uses.
  if constexpr (LAYER) load_state();
  const float b_in = beta[tok];
  unsigned kraw[RPT], qraw[RPT], vraw[4];
#pragma unroll
  for (int m = 0; m < RPT; ++m) ga[m] = SG ? 0.f : gp[rg + RG * m];
  {  // unused after the convolution, but unconditional (see below)
    const in_t* vp0 = v + tok * DV + 4 * cg;
#pragma unroll
    for (int c = 0; c < 4; ++c) vraw[c] = raw32(vp0 + c);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      kraw[m] = raw32(kp + rg + RG * m);
      qraw[m] = raw32(qp + rg + RG * m);
    }
  }
  // Short convolution: each (tensor, channel) of this (n, h) is convolved by
  // one thread, which also shifts that channel's carried inputs (it alone
  // reads them), and published through LDS.  Its inputs: the new value, the
  // W weights and the W-1 carried inputs of each of the thread's items.
  // The layer's loads are unconditional, from a valid stand-in address where
  // an input is absent: a load under a branch leaves the other path waiting
  // for it, and for every load issued before it, wherever that path reuses
  // its register.
  constexpr int NIT = LAYER ? (3 * DK + 255) / 256 : 1;
  unsigned xr[NIT], ol[NIT][3], gt_in[4];
  float wv[NIT][4], nw_in[4];
  if constexpr (LAYER) {
    const int hh = nh % lp.H, w1c = W1 > 0 ? W1 : 0;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      // clamped: an item past the end repeats the last one and is not used
      const int item = min(t + 256 * it, 3 * DK - 1);
      const int x = item / DK, i = item % DK;
      xr[it] = raw32((x == 0 ? q : x == 1 ? k : v) + tok * DK + i);
      const float* wr = conv ? (x == 0 ? lp.cw[0] : x == 1 ? lp.cw[1] : lp.cw[2]) +
                                   ((size_t)hh * DK + i) * (W1 + 1)
                             : gp;
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[it][j] = wr[j <= W1 ? j : w1c];
      // carried inputs j < W1 (nullptr: zeros)
      const in_t* in = reinterpret_cast<const in_t*>(x == 0 ? lp.cs_in[0] : x == 1 ? lp.cs_in[1] : lp.cs_in[2]);
      const bool has_in = conv && in != nullptr && W1 > 0;
      const in_t* ib = has_in ? in + (size_t)nh * W1 * DK + i : q + tok * DK;
#pragma unroll
      for (int j = 0; j < 3; ++j) ol[it][j] = raw32(ib + (has_in && j < W1 ? (size_t)j * DK : 0));
    }
    // the epilogue's gate and RMSNorm weight (used by the threads of row group 0)
    const in_t* gt = lp.gate ? reinterpret_cast<const in_t*>(lp.gate) + tok * DV + 4 * cg : q + tok * DK;
    const float* nw = lp.gate ? lp.norm_weight + 4 * cg : gp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gt_in[c] = raw32(gt + (lp.gate ? c : 0));
      nw_in[c] = nw[lp.gate ? c : 0];
    }
  }
  if constexpr (!LAYER) load_state();
  __builtin_amdgcn_sched_barrier(0);
  float r[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0}, kq = 0.f, nq = 0.f, nk = 0.f;
  __shared__ float cv[LAYER ? 3 : 1][LAYER ? DK : 1];
  if (conv) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int item = t + 256 * it;
      if (item < 3 * DK) {
        const int x = item / DK, i = item % DK;
        float wl = 0.f;  // the weight on the new value, W - 1
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == W1) wl = wv[it][j];
        const in_t* in = reinterpret_cast<const in_t*>(x == 0 ? lp.cs_in[0] : x == 1 ? lp.cs_in[1] : lp.cs_in[2]);
        float acc = wl * raw_to_f<in_t>(xr[it]);
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < W1) acc += wv[it][j] * (in ? raw_to_f<in_t>(ol[it][j]) : 0.f);
        cv[LAYER ? x : 0][LAYER ? i : 0] = acc;
        in_t* out = reinterpret_cast<in_t*>(x == 0 ? lp.cs_out[0] : x == 1 ? lp.cs_out[1] : lp.cs_out[2]);
        if (out && W1 > 0) {
          const size_t b0 = (size_t)nh * W1 * DK + i;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (j + 1 < W1) out[b0 + (size_t)j * DK] = in ? raw_to_t<in_t>(ol[it][j + 1]) : in_t(0.f);
          out[b0 + (size_t)(W1 - 1) * DK] = raw_to_t<in_t>(xr[it]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    kk[m] = conv ? cv[LAYER ? 1 : 0][LAYER ? i : 0] : raw_to_f<in_t>(kraw[m]);
    qq[m] = conv ? cv[0][LAYER ? i : 0] : raw_to_f<in_t>(qraw[m]);
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    if (LAYER && lp.prologue) {
      kk[m] = swish_d(kk[m]);
      qq[m] = swish_d(qq[m]);
      nk += kk[m] * kk[m];
      nq += qq[m] * qq[m];
    }
    const float a = SG ? ag : __expf(ga[m]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s[m][c] *= a;
      r[c] += kk[m] * s[m][c];
      p[c] += qq[m] * s[m][c];
    }
    kq += kk[m] * qq[m];
  }
  // Reduce over the row groups held by this wave (lanes differ in the bits
  // above log2(TPR)).
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] += __shfl_xor(r[c], off);
      p[c] += __shfl_xor(p[c], off);
    }
    kq += __shfl_xor(kq, off);
    if (LAYER) {
      nq += __shfl_xor(nq, off);
      nk += __shfl_xor(nk, off);
    }
  }
  constexpr int NRED = LAYER ? 11 : 9;
  __shared__ float red[4][TPR][NRED];
  float vv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vv[c] = conv ? cv[LAYER ? 2 : 0][LAYER ? 4 * cg + c : 0] : raw_to_f<in_t>(vraw[c]);
  const int w = t >> 6;
  if ((t & 63) < TPR) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      red[w][cg][c] = r[c];
      red[w][cg][4 + c] = p[c];
    }
    red[w][cg][8] = kq;
    if (LAYER) {
      red[w][cg][9] = nq;
      red[w][cg][10] = nk;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r[c] = red[0][cg][c] + red[1][cg][c] + red[2][cg][c] + red[3][cg][c];
    p[c] = red[0][cg][4 + c] + red[1][cg][4 + c] + red[2][cg][4 + c] + red[3][cg][4 + c];
  }
  kq = red[0][cg][8] + red[1][cg][8] + red[2][cg][8] + red[3][cg][8];

  float b = b_in;
  if (LAYER && lp.prologue) {
    // L2 normalisation: scale the reductions by 1/|q|, 1/|k| (floored).
    nq = red[0][cg][9] + red[1][cg][9] + red[2][cg][9] + red[3][cg][9];
    nk = red[0][cg][10] + red[1][cg][10] + red[2][cg][10] + red[3][cg][10];
    const float iq = 1.f / fmaxf(sqrtf(nq), 1e-12f), ik = 1.f / fmaxf(sqrtf(nk), 1e-12f);
#pragma unroll
    for (int m = 0; m < RPT; ++m) kk[m] *= ik;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] *= ik;
      p[c] *= iq;
      vv[c] = swish_d(vv[c]);
    }
    kq *= ik * iq;
    b = sigmoid_d(b);
  }
  float u[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = b * (vv[c] - r[c]);

#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
#pragma unroll
    for (int c = 0; c < 4; ++c) s[m][c] += kk[m] * u[c];
    __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(sp + (size_t)i * DV + 4 * cg));
  }
  if (rg == 0) {
    float y[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = p[c] + kq * u[c];
    if (LAYER && lp.gate) {
      // RMSNorm over the Dv outputs of this (n, h): lanes 0 .. TPR-1 of wave 0.
      float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
      const float inv = 1.f / sqrtf(ss / DV + lp.norm_eps);
#pragma unroll
      for (int c = 0; c < 4; ++c) y[c] = y[c] * inv * nw_in[c] * sigmoid_d(raw_to_f<in_t>(gt_in[c]));
    }
    if constexpr (OUT_BF16) {
      bf16x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = f2bf(y[c]);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(o) + tok * DV + 4 * cg) = ov;
    } else {
      f32x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = y[c];
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + tok * DV + 4 * cg) = ov;
    }
  }
}

// The plain step at d = 128 streams the state fastest with two workgroups per
// compute unit: 176 us per step at two against 193 at three, 198 at four (its
// 123 registers allow four) and 186-196 at one, for 256 sequences x 32 heads.
// An unused dynamic LDS allocation of more than a third of the unit's 160 KB
// caps it at two.  The layer step (152 registers, three per unit) and other
// widths keep the occupancy their registers give.
constexpr unsigned kDecodeLdsPad = 56 * 1024;

template <typename in_t, int D, bool OUT_BF16, bool LAYER>
static void launch_decode_l(const DecodeArgs& a) {
  const int NH = a.N * a.H;
  dim3 grid(NH), block(256);
  const unsigned pad = !LAYER && D == 128 ? kDecodeLdsPad : 0;
  LayerPtrs lp{a.layer.prologue ? 1 : 0, a.layer.gate, a.layer.norm_weight, a.layer.norm_eps,
               a.layer.prologue ? a.layer.conv_w : 0, a.H};
  for (int x = 0; x < 3; ++x) {
    lp.cw[x] = a.layer.conv_weight[x];
    lp.cs_in[x] = a.layer.conv_state_in[x];
    lp.cs_out[x] = a.layer.conv_state_out[x];
  }
  if (a.scalar_g)
    hipLaunchKernelGGL((decode_step_kernel<in_t, D, D, OUT_BF16, true, LAYER>), grid, block, pad,
                       a.stream, (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, a.g, a.beta,
                       a.state, a.o, NH, lp);
  else
    hipLaunchKernelGGL((decode_step_kernel<in_t, D, D, OUT_BF16, false, LAYER>), grid, block, pad,
                       a.stream, (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, a.g, a.beta,
                       a.state, a.o, NH, lp);
}

template <typename in_t, int D, bool OUT_BF16>
static void launch_decode_o(const DecodeArgs& a) {
  if (a.layer.prologue || a.layer.gate)
    launch_decode_l<in_t, D, OUT_BF16, true>(a);
  else
    launch_decode_l<in_t, D, OUT_BF16, false>(a);
}

template <typename in_t, int D>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  if (a.out_bf16)
    launch_decode_o<in_t, D, true>(a);
  else
    launch_decode_o<in_t, D, false>(a);
  return hipGetLastError();
}

// General DPLR single-token step (zeroshot.it.com deep-dive, section 3.2
// "DPLR Structure"): S' = Diag(alpha) S - a (b^T S) + k v^T, o = S'^T q,
// alpha = exp(g).  One pass over the state as in decode_step_kernel: the row
// reductions r = S^T b and p = (Diag(alpha) S)^T q, with a.q and k.q, give
// o = p - (a.q) r + (k.q) v before the state is rewritten.
template <typename in_t, int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void dplr_decode_step_kernel(
    const in_t* __restrict__ q, const in_t* __restrict__ k, const in_t* __restrict__ v,
    const in_t* __restrict__ av, const in_t* __restrict__ bv, const float* __restrict__ g,
    float* __restrict__ state, void* __restrict__ o, int NH) {
  constexpr int TPR = D / 4, RG = 256 / TPR, RPT = D / RG;
  const int nh = blockIdx.x;
  if (nh >= NH) return;
  const int t = threadIdx.x, cg = t % TPR, rg = t / TPR;
  const size_t tok = (size_t)nh;
  float* sp = state + tok * (size_t)D * D;
  f32x4 s[RPT];
  float al[RPT], aa[RPT], kk[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)(rg + RG * m) * D + 4 * cg));
  float r[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0}, aq = 0.f, kq = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    const float qi = (float)q[tok * D + i], bi = (float)bv[tok * D + i];
    al[m] = __expf(g[tok * D + i]);
    aa[m] = (float)av[tok * D + i];
    kk[m] = (float)k[tok * D + i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] += bi * s[m][c];
      p[c] += qi * al[m] * s[m][c];
    }
    aq += aa[m] * qi;
    kq += kk[m] * qi;
  }
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] += __shfl_xor(r[c], off);
      p[c] += __shfl_xor(p[c], off);
    }
    aq += __shfl_xor(aq, off);
    kq += __shfl_xor(kq, off);
  }
  __shared__ float red[4][TPR][10];
  const int w = t >> 6;
  if ((t & 63) < TPR) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      red[w][cg][c] = r[c];
      red[w][cg][4 + c] = p[c];
    }
    red[w][cg][8] = aq;
    red[w][cg][9] = kq;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r[c] = red[0][cg][c] + red[1][cg][c] + red[2][cg][c] + red[3][cg][c];
    p[c] = red[0][cg][4 + c] + red[1][cg][4 + c] + red[2][cg][4 + c] + red[3][cg][4 + c];
  }
  aq = red[0][cg][8] + red[1][cg][8] + red[2][cg][8] + red[3][cg][8];
  kq = red[0][cg][9] + red[1][cg][9] + red[2][cg][9] + red[3][cg][9];
  float vv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vv[c] = (float)v[tok * D + 4 * cg + c];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
#pragma unroll
    for (int c = 0; c < 4; ++c) s[m][c] = al[m] * s[m][c] - aa[m] * r[c] + kk[m] * vv[c];
    __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(sp + (size_t)(rg + RG * m) * D + 4 * cg));
  }
  if (rg == 0) {
    float y[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = p[c] - aq * r[c] + kq * vv[c];
    if constexpr (OUT_BF16) {
      bf16x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = f2bf(y[c]);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(o) + tok * D + 4 * cg) = ov;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + tok * D + 4 * cg) = f32x4{y[0], y[1], y[2], y[3]};
    }
  }
}

template <typename in_t, int D>
static void launch_dplr_decode_t(const DplrDecodeArgs& a) {
  const int NH = a.N * a.H;
  const dim3 grid(NH), block(256);
  if (a.out_bf16)
    hipLaunchKernelGGL((dplr_decode_step_kernel<in_t, D, true>), grid, block, 0, a.stream,
                       (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, (const in_t*)a.a,
                       (const in_t*)a.b, a.g, a.state, a.o, NH);
  else
    hipLaunchKernelGGL((dplr_decode_step_kernel<in_t, D, false>), grid, block, 0, a.stream,
                       (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, (const in_t*)a.a,
                       (const in_t*)a.b, a.g, a.state, a.o, NH);
}

hipError_t launch_dplr_decode(const DplrDecodeArgs& a) {
  if (a.N * a.H == 0) return hipSuccess;
  if (a.in_bf16)
    a.D == 128 ? launch_dplr_decode_t<bf16, 128>(a) : launch_dplr_decode_t<bf16, 64>(a);
  else
    a.D == 128 ? launch_dplr_decode_t<float, 128>(a) : launch_dplr_decode_t<float, 64>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.N * a.H == 0) return hipSuccess;
  if (a.in_bf16) {
    return a.D == 128 ? launch_decode_t<bf16, 128>(a) : launch_decode_t<bf16, 64>(a);
  }
  return a.D == 128 ? launch_decode_t<float, 128>(a) : launch_decode_t<float, 64>(a);
}

}  // namespace kda
