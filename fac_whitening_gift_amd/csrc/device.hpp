// Device-side helpers shared by the gfx950 kernels: the OCP E4M3 codec,
// wave/workgroup reductions and the grouped-launch descriptors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gift.h"

namespace gift {

constexpr int kRank = GIFT_RANK;          // columns of one rank block
constexpr int kMaxRank = GIFT_MAX_RANK;   // largest factor rank (two rank blocks)

// storage columns of a rank-r factor: one rank block up to rank 32, else two
__host__ __device__ __forceinline__ int factor_cols(int rank) { return rank > kRank ? 2 * kRank : kRank; }
constexpr int kBlock = GIFT_BLOCK;
constexpr int kMaxGroup = 16;          // layers per grouped launch (descriptors inline)
// Above this many amax partials in a layer they are first reduced by one
// workgroup (k_amax_final) instead of by every quantize workgroup.
constexpr int kPartialLimit = 2048;
constexpr int kXcd = 8;                // XCDs of the MI355X; workgroups go to them in turn
constexpr float kE4M3Max = 448.0f;     // largest finite OCP E4M3 magnitude

// ---------------------------------------------------------------------------
// E4M3 codec.  The hardware conversion rounds to nearest even on the OCP E4M3
// grid; the explicit median-of-three clamp makes every finite input (and
// +-inf) saturate to +-448 instead of overflowing, and NaN inputs are mapped
// to 0x7F explicitly so the code does not depend on the NaN the converter
// emits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_nan_fix(uint32_t packed, float a, float b,
                                                 float c, float d) {
  uint32_t m = (a != a ? 0x000000ffu : 0u) | (b != b ? 0x0000ff00u : 0u) |
               (c != c ? 0x00ff0000u : 0u) | (d != d ? 0xff000000u : 0u);
  return (packed & ~m) | (0x7f7f7f7fu & m);
}

// Encode four already-scaled values that are not NaN (true whenever the
// amax they were scaled by is finite); byte i of the result = element i.
__device__ __forceinline__ uint32_t e4m3_encode4_num(float a, float b, float c, float d) {
  float ca = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  float cb = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  float cc = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  float cd = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, w, true);
  return (uint32_t)w;
}

// Encode four already-scaled fp32 values, any of them possibly NaN.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  return e4m3_nan_fix(e4m3_encode4_num(a, b, c, d), a, b, c, d);
}

// Encode with the scale of an amax: values scaled by the scale of a finite
// amax are never NaN, so the NaN mapping is only needed for a non-finite one.
__device__ __forceinline__ uint32_t e4m3_encode4_scaled(const float4& v, float scale,
                                                        bool nonfinite) {
  const float a = v.x * scale, b = v.y * scale, c = v.z * scale, d = v.w * scale;
  return nonfinite ? e4m3_encode4(a, b, c, d) : e4m3_encode4_num(a, b, c, d);
}

__device__ __forceinline__ uint8_t e4m3_encode1(float a) {
  return (uint8_t)(e4m3_encode4(a, 0.f, 0.f, 0.f) & 0xffu);
}

// Decode byte `sel` (0..3) of a packed word.
__device__ __forceinline__ float e4m3_decode(uint32_t packed, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)packed, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)packed, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)packed, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)packed, 3);
  }
}

// |x| as an unsigned bit pattern: ordering these is ordering |x|, with NaN
// above +inf above every finite value.
__device__ __forceinline__ uint32_t abs_bits(float x) {
  return __float_as_uint(x) & 0x7fffffffu;
}

// ---------------------------------------------------------------------------
// Accesses of the bulk tensors.  G and the codes are read with plain loads:
// the whiten's second read of a slab row block finds part of G still in the
// caches (with nontemporal G loads the whiten of eight hidden-4096 blocks
// took 5.5 ms instead of 4.8), and nontemporal code loads made the
// dequantize side of a hidden-1024 block about 15% slower.  The codes and G^
// are written once per pass and go out with the nontemporal (`nt`) bit, so
// the stores do not evict the operands that are reused (packs, row
// coefficients).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) unsigned nt_u4;
typedef __attribute__((ext_vector_type(4))) float nt_f4;

__device__ __forceinline__ float4 ld_g(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ uint4 ld_q16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld_q4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void st_f4(float* p, const float4& v) {
  __builtin_nontemporal_store(nt_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f4*>(p));
}
__device__ __forceinline__ void st_q16(uint8_t* p, const uint4& v) {
  __builtin_nontemporal_store(nt_u4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u4*>(p));
}
__device__ __forceinline__ void st_q4(uint8_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<unsigned*>(p));
}

// scale / inv / flags from an amax given as |x| bits (IEEE division).  A
// finite amax below 448 / FLT_MAX makes the quotient overflow; such a tensor
// gets the largest finite scale, so its zeros stay zeros (0 * inf would be
// NaN) and no finite value becomes a NaN code.
struct Scale {
  float scale, inv;
  uint32_t flags;
};
__device__ __forceinline__ Scale scale_from_amax_bits(uint32_t bits) {
  Scale s;
  float a = __uint_as_float(bits);
  s.flags = bits >= 0x7f800000u ? GIFT_FLAG_NONFINITE : 0u;
  if (bits == 0u) {
    s.scale = 1.0f;
    s.inv = 1.0f;
    s.flags |= GIFT_FLAG_ZERO_AMAX;
  } else {
    s.scale = kE4M3Max / a;
    s.inv = a / kE4M3Max;
    // only a finite amax can give +inf here (NaN and inf amax give NaN and 0)
    if (s.scale > __FLT_MAX__) s.scale = __FLT_MAX__;
  }
  return s;
}

// ---------------------------------------------------------------------------
// OCP MX FP4 (MXFP4): E2M1 elements, one E8M0 scale 2^(code - 127) per 32
// consecutive elements of a row, code = floor(log2 amax) - 2 + 127 clamped
// to [0, 254]; 0xFF is the NaN scale.  The gfx950 FP4 conversions take the
// scale as an fp32 operand of which they use only the exponent field, round
// to nearest even, saturate to +-6 (+-inf included), keep the sign of zero,
// and put the first value of a pair in the low nibble.  NaN inputs are
// mapped to +0 here; they occur only in blocks whose amax is NaN, which
// decode to NaN through their scale.
// ---------------------------------------------------------------------------
constexpr int kMxBlock = 32;
constexpr uint32_t kMxScaleNaN = 0xFFu;

// E8M0 code of a block whose amax is given as |x| bits; flags as for E4M3
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t bits, uint32_t& flags) {
  if (bits >= 0x7f800000u) {
    flags |= GIFT_FLAG_NONFINITE;
    return kMxScaleNaN;
  }
  if (bits == 0u) {
    flags |= GIFT_FLAG_ZERO_AMAX;
    return 127u;
  }
  const int field = (int)(bits >> 23);
  const int floor_log2 = field ? field - 127 : (31 - __clz((int)bits)) - 149;
  int e = floor_log2 - 2;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return (uint32_t)(e + 127);
}

// scale operand of the conversions (the NaN scale encodes with 2^0)
__device__ __forceinline__ float mx_scale_operand(uint32_t code) {
  return __uint_as_float((code == kMxScaleNaN ? 127u : code) << 23);
}

// four values -> four E2M1 codes in 16 bits, value 0 in the low nibble
__device__ __forceinline__ uint32_t mx_encode4(float4 v, float s, bool nonfinite) {
  if (nonfinite) {
    v.x = v.x != v.x ? 0.f : v.x;
    v.y = v.y != v.y ? 0.f : v.y;
    v.z = v.z != v.z ? 0.f : v.z;
    v.w = v.w != v.w ? 0.f : v.w;
  }
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v.x, v.y, s, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v.z, v.w, s, 1);
  return r & 0xffffu;
}

// four E2M1 codes (16 bits) -> code value * 2^(scale code - 127), exact
__device__ __forceinline__ float4 mx_decode4(uint32_t c16, uint32_t code) {
  const float s = mx_scale_operand(code);
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c16, s, 0);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c16, s, 1);
  float4 v = make_float4(lo[0], lo[1], hi[0], hi[1]);
  if (code == kMxScaleNaN) v = make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                           __builtin_nanf(""), __builtin_nanf(""));
  return v;
}

// ---------------------------------------------------------------------------
// fp32-accurate products on the bf16 matrix cores: every fp32 operand is split
// into three bf16 parts, x = x1 + x2 + x3 exactly, and the six partial
// products of weight >= 2^-16 are accumulated in fp32.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// x = s[0] + s[1] + s[2] exactly (RNE at each level; the remainders are exact)
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8 (&s)[3]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 a = (__bf16)x[i];
    const float r = x[i] - (float)a;
    const __bf16 b = (__bf16)r;
    const float r2 = r - (float)b;
    s[0][i] = a;
    s[1][i] = b;
    s[2][i] = (__bf16)r2;
  }
}

// acc += (a0 + a1 + a2)(b0 + b1 + b2), products of weight >= 2^-16
__device__ __forceinline__ f32x4 mfma3x3(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x4 acc) {
  acc = mfma(a[2], b[0], acc);
  acc = mfma(a[1], b[1], acc);
  acc = mfma(a[0], b[2], acc);
  acc = mfma(a[1], b[0], acc);
  acc = mfma(a[0], b[1], acc);
  return mfma(a[0], b[0], acc);
}

// The six products of mfma3x3, issued round-robin over N independent
// accumulators (acc[i] += a[ia[i]] * b[ib[i]]) so the matrix pipe never waits
// on one accumulator's previous product.
template <int N>
__device__ __forceinline__ void mfma3x3_n(const bf16x8 (*const (&a)[N])[3],
                                          const bf16x8 (*const (&b)[N])[3], f32x4 (&acc)[N]) {
  constexpr int ia[6] = {2, 1, 0, 1, 0, 0};
  constexpr int ib[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
  for (int p = 0; p < 6; ++p)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = mfma((*a[i])[ia[p]], (*b[i])[ib[p]], acc[i]);
}

// acc += (a0 + a1 + a2) b  (b exact in bf16)
__device__ __forceinline__ f32x4 mfma3x1(const bf16x8 (&a)[3], const bf16x8& b, f32x4 acc) {
  acc = mfma(a[2], b, acc);
  acc = mfma(a[1], b, acc);
  return mfma(a[0], b, acc);
}

// ---------------------------------------------------------------------------
// reductions (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ uint32_t half_wave_max_u32(uint32_t v) {  // within 32 lanes
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroup max of one value per thread; every thread gets the result.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds /*kThreads/64*/) {
  constexpr int kWaves = kThreads / 64;
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = r > lds[i] ? r : lds[i];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// grouped-launch descriptors (passed by value as kernel arguments)
// ---------------------------------------------------------------------------
struct LayerDev {
  const float* G;
  uint8_t* q;
  float* inv;
  float* Ghat;
  float* Wout;
  const float* U;       // d_in x 32 (NULL: Euclidean layer)
  const float* coef;    // GIFT_COEF_COUNT
  const uint4* P;       // the factor's split MFMA operand packs
  float* cbuf;          // workspace: column-group partials of the row coefficients
  float* cfin;          // workspace: c' of every row (fp32, in the lanes' fragment order)
  uint32_t* part;       // workspace: one partial amax per tile
  uint32_t* amax;       // workspace: the layer's amax as |x| bits
  double* part2;        // workspace: two fp64 partial sums per tile
  int64_t d_out, d_in;
  int64_t n_rb;         // row blocks of the tile kernels
  int ngrp;             // column groups of the tile kernels
  int tile_begin, n_tiles;
  int n_part;           // amax partials of the layer (tiles, or row blocks of a slab layer)
  int rb_begin;         // first row block of the layer in the group
};

struct GroupDev {
  int n;
  int total_tiles;
  int total_rb;         // row blocks over the group (tile kernels)
  uint32_t* flags;      // may be NULL
  double* out;          // roundtrip_error output, may be NULL
  // NULL: the n <= kMaxGroup layers are L[0 .. n).  Else the descriptors of
  // all n layers in device memory; only k_slab_whiten is launched so (it
  // looks its layer up with find_layer_rb and layer_at).
  const LayerDev* Lx;
  LayerDev L[kMaxGroup];
};

// One factor to pack: U (d_in x 32 fp32) -> P (bf16x3 operand packs).
// One rank block (32 columns) of a factor to pack: U points at the block's
// first column of a d_in x ucols matrix (ucols 32 or 64).
struct PackDev {
  const float* U;
  uint4* P;
  int d_in;
  int ucols;
};
struct PackGroup {
  int n;
  PackDev f[kMaxGroup];
};

// Layer of a workgroup: all tile_begin values are read at once (one round
// trip to the kernel arguments, not one per layer).
__device__ __forceinline__ int find_layer(const GroupDev& g, int tile) {
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < g.n && tile >= g.L[i].tile_begin) l = i;
  return l;
}

__device__ __forceinline__ int find_layer_rb(const GroupDev& g, int rb) {
  if (g.Lx) {  // the last layer whose first row block is <= rb
    int lo = 0, hi = g.n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rb >= g.Lx[mid].rb_begin) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  }
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < g.n && rb >= g.L[i].rb_begin) l = i;
  return l;
}

__device__ __forceinline__ LayerDev layer_at(const GroupDev& g, int i) {
  return g.Lx ? g.Lx[i] : g.L[i];
}

}  // namespace gift
