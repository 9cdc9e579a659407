// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Matrix products run on 16x16 MFMA tiles.  Two operand precisions exist:
//
//   * ModeBF16: inputs arrive as bfloat16.  A "plain" operand is one bf16
//     value; a "precise" operand is an unevaluated sum hi + lo of two bf16
//     values (about 16 significant bits).  A precise x precise product is
//     three v_mfma_f32_16x16x32_bf16 (hi*hi + hi*lo + lo*hi); precise x plain
//     is two.  Accumulation is always fp32.
//   * ModeF32: inputs arrive as float32 and every product uses
//     v_mfma_f32_16x16x4_f32 on fp32 operands (plain and precise coincide).
//
// Fragment convention (both modes).  A fragment covers a 16-row x 32-k slab
// of a matrix whose k index is the contraction index.  Lane l holds row
// (l & 15) and the eight k values 8*(l >> 4) + e, e = 0..7.  The A operand
// of a product uses rows of A; the B operand uses columns of B, i.e. rows of
// B^T, with the same layout.  The 16x16 fp32 result tile in lane l holds
// rows 4*(l >> 4) + i (i = 0..3) of column (l & 15).
//
// In ModeF32 one fragment feeds eight 16x16x4 MFMAs: step e contracts the
// four k values {8g + e : g = 0..3}, one per lane group, which visits all 32
// k values of the slab exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Operand modes
// ---------------------------------------------------------------------------
struct ModeBF16 {
  typedef bf16 in_t;
  static constexpr bool kSplit = true;
  struct PFrag { bf16x8 hi, lo; };   // precise fragment
  struct Frag { bf16x8 v; };         // plain fragment
  // Bytes of one fragment (64 lanes) in global storage.
  static constexpr int kPFragBytes = 2048;
  static constexpr int kFragBytes = 1024;
};

struct ModeF32 {
  typedef float in_t;
  static constexpr bool kSplit = false;
  struct PFrag { f32x8 v; };
  struct Frag { f32x8 v; };
  static constexpr int kPFragBytes = 2048;
  static constexpr int kFragBytes = 2048;
};

// ----- building fragments from eight fp32 values (in the lane's k order) ---
__device__ __forceinline__ ModeBF16::PFrag make_pfrag(ModeBF16, const float* x) {
  ModeBF16::PFrag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h = f2bf(x[e]);
    f.hi[e] = h;
    f.lo[e] = f2bf(x[e] - bf2f(h));
  }
  return f;
}
__device__ __forceinline__ ModeF32::PFrag make_pfrag(ModeF32, const float* x) {
  ModeF32::PFrag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}
__device__ __forceinline__ ModeBF16::Frag make_frag(ModeBF16, const float* x) {
  ModeBF16::Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = f2bf(x[e]);
  return f;
}
__device__ __forceinline__ ModeF32::Frag make_frag(ModeF32, const float* x) {
  ModeF32::Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}

// ----- products on one 16x16 tile ------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32x8(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// precise x precise
__device__ __forceinline__ f32x4 mma_pp(const ModeBF16::PFrag& a, const ModeBF16::PFrag& b, f32x4 c) {
  c = mfma_bf16(a.lo, b.hi, c);
  c = mfma_bf16(a.hi, b.lo, c);
  return mfma_bf16(a.hi, b.hi, c);
}
__device__ __forceinline__ f32x4 mma_pp(const ModeF32::PFrag& a, const ModeF32::PFrag& b, f32x4 c) {
  return mfma_f32x8(a.v, b.v, c);
}
// precise x plain
__device__ __forceinline__ f32x4 mma_pf(const ModeBF16::PFrag& a, const ModeBF16::Frag& b, f32x4 c) {
  c = mfma_bf16(a.lo, b.v, c);
  return mfma_bf16(a.hi, b.v, c);
}
__device__ __forceinline__ f32x4 mma_pf(const ModeF32::PFrag& a, const ModeF32::Frag& b, f32x4 c) {
  return mfma_f32x8(a.v, b.v, c);
}
// plain x plain
__device__ __forceinline__ f32x4 mma_ff(const ModeBF16::Frag& a, const ModeBF16::Frag& b, f32x4 c) {
  return mfma_bf16(a.v, b.v, c);
}
__device__ __forceinline__ f32x4 mma_ff(const ModeF32::Frag& a, const ModeF32::Frag& b, f32x4 c) {
  return mfma_f32x8(a.v, b.v, c);
}

// ---------------------------------------------------------------------------
// LDS operand arrays.  A matrix that feeds fragments lives row-major in LDS
// with a padded row stride (elements).  ModeBF16 keeps a precise matrix as two
// bf16 arrays (hi, lo) of the same shape; ModeF32 keeps one float array.
// ---------------------------------------------------------------------------
// Row stride padding: 8 elements shifts consecutive rows by 16 B (bf16) or
// 32 B (fp32), which spreads the 16 rows of a fragment read over the banks.
constexpr int kPad = 8;

// Read a fragment at (row0, k0) from row-major LDS arrays.
__device__ __forceinline__ ModeBF16::PFrag lds_pfrag(ModeBF16, const bf16* hi, const bf16* lo,
                                                     int stride, int row0, int k0) {
  const int l = lane_id();
  const int off = (row0 + (l & 15)) * stride + k0 + 8 * (l >> 4);
  ModeBF16::PFrag f;
  f.hi = *reinterpret_cast<const bf16x8*>(hi + off);
  f.lo = *reinterpret_cast<const bf16x8*>(lo + off);
  return f;
}
__device__ __forceinline__ ModeF32::PFrag lds_pfrag(ModeF32, const float* v, const float*,
                                                    int stride, int row0, int k0) {
  const int l = lane_id();
  const int off = (row0 + (l & 15)) * stride + k0 + 8 * (l >> 4);
  ModeF32::PFrag f;
  f.v = *reinterpret_cast<const f32x8*>(v + off);
  return f;
}
__device__ __forceinline__ ModeBF16::Frag lds_frag(ModeBF16, const bf16* v, int stride, int row0, int k0) {
  const int l = lane_id();
  ModeBF16::Frag f;
  f.v = *reinterpret_cast<const bf16x8*>(v + (row0 + (l & 15)) * stride + k0 + 8 * (l >> 4));
  return f;
}
__device__ __forceinline__ ModeF32::Frag lds_frag(ModeF32, const float* v, int stride, int row0, int k0) {
  const int l = lane_id();
  ModeF32::Frag f;
  f.v = *reinterpret_cast<const f32x8*>(v + (row0 + (l & 15)) * stride + k0 + 8 * (l >> 4));
  return f;
}

// ----- global fragment storage ----------------------------------------------
// A precise fragment occupies 2 KB: ModeBF16 stores [hi: lane*16 B][lo:
// 1024 + lane*16 B]; ModeF32 stores lane*32 B.  A plain fragment is 1 KB
// (bf16, lane*16 B) or 2 KB (fp32, lane*32 B).
__device__ __forceinline__ void st_pfrag(ModeBF16, char* base, const ModeBF16::PFrag& f) {
  const int l = lane_id();
  *reinterpret_cast<bf16x8*>(base + l * 16) = f.hi;
  *reinterpret_cast<bf16x8*>(base + 1024 + l * 16) = f.lo;
}
__device__ __forceinline__ void st_pfrag(ModeF32, char* base, const ModeF32::PFrag& f) {
  *reinterpret_cast<f32x8*>(base + lane_id() * 32) = f.v;
}
__device__ __forceinline__ ModeBF16::PFrag ld_pfrag(ModeBF16, const char* base) {
  const int l = lane_id();
  ModeBF16::PFrag f;
  f.hi = *reinterpret_cast<const bf16x8*>(base + l * 16);
  f.lo = *reinterpret_cast<const bf16x8*>(base + 1024 + l * 16);
  return f;
}
__device__ __forceinline__ ModeF32::PFrag ld_pfrag(ModeF32, const char* base) {
  ModeF32::PFrag f;
  f.v = *reinterpret_cast<const f32x8*>(base + lane_id() * 32);
  return f;
}
__device__ __forceinline__ void st_frag(ModeBF16, char* base, const ModeBF16::Frag& f) {
  *reinterpret_cast<bf16x8*>(base + lane_id() * 16) = f.v;
}
__device__ __forceinline__ void st_frag(ModeF32, char* base, const ModeF32::Frag& f) {
  *reinterpret_cast<f32x8*>(base + lane_id() * 32) = f.v;
}
__device__ __forceinline__ ModeBF16::Frag ld_frag(ModeBF16, const char* base) {
  ModeBF16::Frag f;
  f.v = *reinterpret_cast<const bf16x8*>(base + lane_id() * 16);
  return f;
}
__device__ __forceinline__ ModeF32::Frag ld_frag(ModeF32, const char* base) {
  ModeF32::Frag f;
  f.v = *reinterpret_cast<const f32x8*>(base + lane_id() * 32);
  return f;
}

// ----- loading eight consecutive input elements as fp32 ---------------------
__device__ __forceinline__ void load8(const bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = bf2f(v[e]);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
}

}  // namespace kda
