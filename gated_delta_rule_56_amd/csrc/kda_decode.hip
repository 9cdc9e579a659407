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
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// SG: scalar gate (Gated DeltaNet): g holds one log-decay per (n, h).
template <typename in_t, int DK, int DV, bool OUT_BF16, bool SG>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const in_t* __restrict__ q, const in_t* __restrict__ k, const in_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, int NH) {
  constexpr int TPR = DV / 4;          // threads per state row
  constexpr int RG = 256 / TPR;        // row groups
  constexpr int RPT = DK / RG;         // rows per thread
  constexpr int RG_PER_WAVE = 64 / TPR;
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

  float kk[RPT], qq[RPT];
  f32x4 s[RPT];
  // Issue the state loads first: they are the long pole.
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)i * DV + 4 * cg));
  }
  float r[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0}, kq = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    kk[m] = (float)kp[i];
    qq[m] = (float)qp[i];
    const float a = SG ? ag : __expf(gp[i]);
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
  }
  __shared__ float red[4][TPR][9];
  const int w = t >> 6;
  if ((t & 63) < TPR) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      red[w][cg][c] = r[c];
      red[w][cg][4 + c] = p[c];
    }
    red[w][cg][8] = kq;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r[c] = red[0][cg][c] + red[1][cg][c] + red[2][cg][c] + red[3][cg][c];
    p[c] = red[0][cg][4 + c] + red[1][cg][4 + c] + red[2][cg][4 + c] + red[3][cg][4 + c];
  }
  kq = red[0][cg][8] + red[1][cg][8] + red[2][cg][8] + red[3][cg][8];

  const float b = beta[tok];
  const in_t* vp = v + tok * DV + 4 * cg;
  float u[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = b * ((float)vp[c] - r[c]);

#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
#pragma unroll
    for (int c = 0; c < 4; ++c) s[m][c] += kk[m] * u[c];
    __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(sp + (size_t)i * DV + 4 * cg));
  }
  if (rg == 0) {
    if constexpr (OUT_BF16) {
      bf16x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = f2bf(p[c] + kq * u[c]);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(o) + tok * DV + 4 * cg) = ov;
    } else {
      f32x4 ov;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = p[c] + kq * u[c];
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + tok * DV + 4 * cg) = ov;
    }
  }
}

template <typename in_t, int D, bool OUT_BF16>
static void launch_decode_o(const DecodeArgs& a) {
  const int NH = a.N * a.H;
  dim3 grid(NH), block(256);
  if (a.scalar_g)
    hipLaunchKernelGGL((decode_step_kernel<in_t, D, D, OUT_BF16, true>), grid, block, 0, a.stream,
                       (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, a.g, a.beta,
                       a.state, a.o, NH);
  else
    hipLaunchKernelGGL((decode_step_kernel<in_t, D, D, OUT_BF16, false>), grid, block, 0, a.stream,
                       (const in_t*)a.q, (const in_t*)a.k, (const in_t*)a.v, a.g, a.beta,
                       a.state, a.o, NH);
}

template <typename in_t, int D>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  if (a.out_bf16)
    launch_decode_o<in_t, D, true>(a);
  else
    launch_decode_o<in_t, D, false>(a);
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
