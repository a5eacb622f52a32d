// GIFT FP8 round trip on gfx950: whiten + quantize, dequantize + un-whiten,
// the Euclidean baseline and the error reduction.
//
// The operation (GIFT review, "What carries the argument"): the gradient G is
// right-multiplied by A_r^-1/2 = alpha I + U diag(D_w) U^T before FP8 and by
// A_r^1/2 = beta I + U diag(D_u) U^T after it.  Per row g of G:
//     c = g U (32 numbers), w = alpha g + (c * D_w) U^T.
// Both rank-32 products are dense contractions and run on the matrix cores
// (v_mfma_f32_16x16x32_bf16) with every fp32 operand split into three bf16
// parts, x = x1 + x2 + x3 exactly; the six partial products with combined
// weight down to 2^-16 are kept, which leaves an fp32-level product.  E4M3
// codes are exact in bf16, so in dequantize the first product needs only
// the three parts of U.
//
// Layout ("transposed" products): a 16x16 MFMA result tile holds, in lane l,
// four consecutive columns (d_in indices 4(l/16)..+3) of gradient row l%16,
// so gradient loads/stores are float4 per lane.  The first product
// C^T = U^T G^T runs over 32-column chunks; its K order inside a chunk is
// permuted so lane l's eight K slots are exactly the 2 x 4 columns it holds
// in the two 16-column result tiles of that chunk, and its result (lane l:
// ranks 4g..4g+3 and 16+4g..+3 of row l%16) is used unchanged as the K=32
// operand of the second product W^T = U C'^T with the rank order permuted the
// same way.  U's two operand forms are split and packed once per call
// (k_pack_u).
//
// A workgroup takes kRT*16 rows over the full row length; its 8 waves split
// the 32-column chunks, reduce c across waves through LDS, and then apply the
// correction to their own chunks (re-reading G, most recent chunk first).
// Per-tensor scaling takes two launches (pass 1: c' and a partial amax per
// workgroup; pass 2: the amax of the layer from the partials, W again and the
// codes); 1x128 block scaling needs only the row and is one launch.
#include "device.hpp"

namespace gift {

constexpr int kThreads = 256;       // flat kernels
constexpr int kFlatTile = 4096;     // elements per workgroup (flat kernels)
constexpr int kWaves = 8;           // waves per workgroup (row kernels)
constexpr int kRowThreads = 64 * kWaves;
constexpr int kRT = 2;              // 16-row tiles per row workgroup
constexpr int kRows = 16 * kRT;
constexpr int kChunk = 32;          // columns per MFMA K chunk

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

// acc += (a0 + a1 + a2) b  (b exact in bf16)
__device__ __forceinline__ f32x4 mfma3x1(const bf16x8 (&a)[3], const bf16x8& b, f32x4 acc) {
  acc = mfma(a[2], b, acc);
  acc = mfma(a[1], b, acc);
  return mfma(a[0], b, acc);
}

// ---------------------------------------------------------------------------
// operand packs.  For a factor with nch = d_in/32 chunks, P holds two arrays
// of nch*2*3*64 uint4 (8 bf16 each), indexed ((c*2 + h)*3 + split)*64 + lane:
//   first  (U^T operand of c = g U):  element i of lane l (r16 = l%16,
//          g = l/16) = U[32c + perm(i)][16h + r16]
//   second (U operand of w = c' U^T): element i = U[32c + 16h + r16][perm(i)]
// with perm(i) = 16*(i/4) + 4g + i%4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm8(int i, int g) { return 16 * (i >> 2) + 4 * g + (i & 3); }

__global__ __launch_bounds__(kThreads) void k_pack_u(PackGroup pg) {
  const PackDev& F = pg.f[blockIdx.y];
  const int nch = F.d_in / kChunk;
  const int per = nch * 2 * 64;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= 2 * per) return;
  const int which = e / per, r = e % per;
  const int lane = r & 63, ch = r >> 6;  // ch = c*2 + h
  const int c = ch >> 1, h = ch & 1;
  const int r16 = lane & 15, g = lane >> 4;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = perm8(i, g);
    v[i] = which == 0 ? F.U[(int64_t)(kChunk * c + p) * kRank + 16 * h + r16]
                      : F.U[(int64_t)(kChunk * c + 16 * h + r16) * kRank + p];
  }
  bf16x8 s[3];
  split3(v, s);
  uint4* out = F.P + (size_t)which * nch * 2 * 3 * 64;
#pragma unroll
  for (int k = 0; k < 3; ++k)
    out[(size_t)(ch * 3 + k) * 64 + lane] = __builtin_bit_cast(uint4, s[k]);
}

// ---------------------------------------------------------------------------
// row-workgroup geometry
// ---------------------------------------------------------------------------
struct RowCtx {
  int64_t row[kRT];   // clamped row of each 16-row tile for this lane
  bool ok[kRT];       // row < d_out
  int c0, c1;         // this wave's chunk range
  int lane, wave, r16, g;
};

__device__ __forceinline__ RowCtx row_ctx(const LayerDev& L, int tile, int unit) {
  RowCtx x;
  x.lane = threadIdx.x & 63;
  x.wave = threadIdx.x >> 6;
  x.r16 = x.lane & 15;
  x.g = x.lane >> 4;
  const int64_t row0 = (int64_t)tile * kRows;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int64_t r = row0 + 16 * rt + x.r16;
    x.ok[rt] = r < L.d_out;
    x.row[rt] = x.ok[rt] ? r : L.d_out - 1;
  }
  const int nunits = (int)(L.d_in / kChunk) / unit;
  x.c0 = (x.wave * nunits / kWaves) * unit;
  x.c1 = ((x.wave + 1) * nunits / kWaves) * unit;
  return x;
}

// Sum the per-wave partial products (16 values per lane) over the 8 waves in
// a fixed order; every lane gets the totals for its own positions.
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[2][kRT], float (*red)[kRT * 8][64],
                                             const RowCtx& x, float (&tot)[kRT][8]) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[x.wave][rt * 8 + h * 4 + i][x.lane] = acc[h][rt][i];
  __syncthreads();
  for (int p = threadIdx.x; p < kRT * 8 * 64; p += kRowThreads) {
    const int q = p >> 6, ln = p & 63;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w][q][ln];
    red[0][q][ln] = s;
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int j = 0; j < 8; ++j) tot[rt][j] = red[0][rt * 8 + j][x.lane];
}

// First product c^T = U^T G^T over the wave's chunks (G fp32, split 3 ways).
__device__ __forceinline__ void gemm1_g(const LayerDev& L, const RowCtx& x, f32x4 (&acc)[2][kRT]) {
  const uint4* P1 = L.P;
  const int64_t d_in = L.d_in;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = x.c0; c < x.c1; ++c) {
    bf16x8 a[2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 3; ++s) a[h][s] = as_bf16x8(P1[(size_t)((c * 2 + h) * 3 + s) * 64 + x.lane]);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const float* gp = L.G + x.row[rt] * d_in + kChunk * c + 4 * x.g;
      const float4 u = *reinterpret_cast<const float4*>(gp);
      const float4 v = *reinterpret_cast<const float4*>(gp + 16);
      const float gv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
      bf16x8 b[3];
      split3(gv, b);
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h][rt] = mfma3x3(a[h], b, acc[h][rt]);
    }
  }
}

// c' (lane's 8 ranks of each row tile) -> split second-product operands
__device__ __forceinline__ void cprime_operands(const float (&cp)[kRT][8], bf16x8 (&b)[kRT][3]) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) split3(cp[rt], b[rt]);
}

// Correction tile (16 cols x 16 rows) for chunk c, half t, row tile rt.
__device__ __forceinline__ void load_p2(const LayerDev& L, int c, int lane, bf16x8 (&a)[2][3]) {
  const int nch = (int)(L.d_in / kChunk);
  const uint4* P2 = L.P + (size_t)nch * 2 * 3 * 64;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 3; ++s) a[t][s] = as_bf16x8(P2[(size_t)((c * 2 + t) * 3 + s) * 64 + lane]);
}

// rank index of element j (0..7) of a lane's c' vector
__device__ __forceinline__ int rank_of(int j, int g) { return 16 * (j >> 2) + 4 * g + (j & 3); }

__device__ __forceinline__ float4 f4(const f32x4& v) { return make_float4(v[0], v[1], v[2], v[3]); }

// ---------------------------------------------------------------------------
// whiten, pass 1 of per-tensor scaling: c' -> cbuf, partial amax per workgroup
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads) void k_whiten_p1(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, 1);
  __shared__ float red[kWaves][kRT * 8][64];
  __shared__ uint32_t mx[kWaves];
  f32x4 acc[2][kRT];
  gemm1_g(L, x, acc);
  float cp[kRT][8];
  reduce_waves(acc, red, x, cp);
  const float* dw = L.coef + GIFT_COEF_DW;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = dw[rank_of(j, x.g)];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) cp[rt][j] *= d;
  }
  if (x.wave == 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      if (x.ok[rt]) {
        float* cb = L.cbuf + x.row[rt] * kRank + 4 * x.g;
        *reinterpret_cast<float4*>(cb) = make_float4(cp[rt][0], cp[rt][1], cp[rt][2], cp[rt][3]);
        *reinterpret_cast<float4*>(cb + 16) = make_float4(cp[rt][4], cp[rt][5], cp[rt][6], cp[rt][7]);
      }
  }
  bf16x8 b[kRT][3];
  cprime_operands(cp, b);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  uint32_t m = 0u;
  for (int c = x.c1 - 1; c >= x.c0; --c) {
    bf16x8 a[2][3];
    load_p2(L, c, x.lane, a);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const f32x4 corr = mfma3x3(a[t], b[rt], f32x4{0.f, 0.f, 0.f, 0.f});
        if (!x.ok[rt]) continue;
        const float4 gv = *reinterpret_cast<const float4*>(L.G + x.row[rt] * L.d_in + kChunk * c +
                                                           16 * t + 4 * x.g);
        m = max(m, abs_bits(fmaf(alpha, gv.x, corr[0])));
        m = max(m, abs_bits(fmaf(alpha, gv.y, corr[1])));
        m = max(m, abs_bits(fmaf(alpha, gv.z, corr[2])));
        m = max(m, abs_bits(fmaf(alpha, gv.w, corr[3])));
      }
  }
  m = block_max_u32<kRowThreads>(m, mx);
  if (threadIdx.x == 0) L.part[tile] = m;
}

// ---------------------------------------------------------------------------
// whiten, pass 2 of per-tensor scaling: layer amax from the partials, W
// again from G and c' (cbuf), E4M3 codes.
// ---------------------------------------------------------------------------
template <bool kWriteW>
__global__ __launch_bounds__(kRowThreads) void k_whiten_p2(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, 1);
  __shared__ uint32_t mx[kWaves];
  uint32_t m = 0u;
  for (int i = threadIdx.x; i < L.n_tiles; i += kRowThreads) m = max(m, L.part[i]);
  m = block_max_u32<kRowThreads>(m, mx);
  const Scale sc = scale_from_amax_bits(m);
  if (tile == 0 && threadIdx.x == 0) {
    L.inv[0] = sc.inv;
    if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
  }
  float cp[kRT][8];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const float* cb = L.cbuf + x.row[rt] * kRank + 4 * x.g;
    const float4 u = *reinterpret_cast<const float4*>(cb);
    const float4 v = *reinterpret_cast<const float4*>(cb + 16);
    cp[rt][0] = u.x; cp[rt][1] = u.y; cp[rt][2] = u.z; cp[rt][3] = u.w;
    cp[rt][4] = v.x; cp[rt][5] = v.y; cp[rt][6] = v.z; cp[rt][7] = v.w;
  }
  bf16x8 b[kRT][3];
  cprime_operands(cp, b);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  for (int c = x.c0; c < x.c1; ++c) {
    bf16x8 a[2][3];
    load_p2(L, c, x.lane, a);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const f32x4 corr = mfma3x3(a[t], b[rt], f32x4{0.f, 0.f, 0.f, 0.f});
        if (!x.ok[rt]) continue;
        const int64_t o = x.row[rt] * L.d_in + kChunk * c + 16 * t + 4 * x.g;
        const float4 gv = *reinterpret_cast<const float4*>(L.G + o);
        const float w0 = fmaf(alpha, gv.x, corr[0]), w1 = fmaf(alpha, gv.y, corr[1]);
        const float w2 = fmaf(alpha, gv.z, corr[2]), w3 = fmaf(alpha, gv.w, corr[3]);
        *reinterpret_cast<uint32_t*>(L.q + o) =
            e4m3_encode4(w0 * sc.scale, w1 * sc.scale, w2 * sc.scale, w3 * sc.scale);
        if (kWriteW) *reinterpret_cast<float4*>(L.Wout + o) = make_float4(w0, w1, w2, w3);
      }
  }
}

// ---------------------------------------------------------------------------
// whiten + quantize with 1x128 block scaling (one launch).  Waves own whole
// 128-column segments; a segment's amax is the max over the lane's 32 values
// and the four lanes holding the same row.
// ---------------------------------------------------------------------------
template <bool kWriteW>
__global__ __launch_bounds__(kRowThreads) void k_whiten_b128(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kBlock / kChunk);
  __shared__ float red[kWaves][kRT * 8][64];
  f32x4 acc[2][kRT];
  gemm1_g(L, x, acc);
  float cp[kRT][8];
  reduce_waves(acc, red, x, cp);
  const float* dw = L.coef + GIFT_COEF_DW;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = dw[rank_of(j, x.g)];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) cp[rt][j] *= d;
  }
  bf16x8 b[kRT][3];
  cprime_operands(cp, b);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  const int64_t nseg = L.d_in / kBlock;
  for (int s0 = x.c0; s0 < x.c1; s0 += kBlock / kChunk) {
    float w[kRT][kBlock / kChunk][2][4];
#pragma unroll
    for (int k = 0; k < kBlock / kChunk; ++k) {
      const int c = s0 + k;
      bf16x8 a[2][3];
      load_p2(L, c, x.lane, a);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const f32x4 corr = mfma3x3(a[t], b[rt], f32x4{0.f, 0.f, 0.f, 0.f});
          const float4 gv = *reinterpret_cast<const float4*>(L.G + x.row[rt] * L.d_in +
                                                             kChunk * c + 16 * t + 4 * x.g);
          w[rt][k][t][0] = fmaf(alpha, gv.x, corr[0]);
          w[rt][k][t][1] = fmaf(alpha, gv.y, corr[1]);
          w[rt][k][t][2] = fmaf(alpha, gv.z, corr[2]);
          w[rt][k][t][3] = fmaf(alpha, gv.w, corr[3]);
        }
    }
    const int seg = s0 / (kBlock / kChunk);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < kBlock / kChunk; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = max(m, abs_bits(w[rt][k][t][i]));
      uint32_t o = __shfl_xor(m, 16, 64);
      m = max(m, o);
      o = __shfl_xor(m, 32, 64);
      m = max(m, o);
      const Scale sc = scale_from_amax_bits(m);
      if (!x.ok[rt]) continue;
      if (x.g == 0) {
        L.inv[x.row[rt] * nseg + seg] = sc.inv;
        if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
      }
#pragma unroll
      for (int k = 0; k < kBlock / kChunk; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int64_t o2 = x.row[rt] * L.d_in + kChunk * (s0 + k) + 16 * t + 4 * x.g;
          const float* v = w[rt][k][t];
          *reinterpret_cast<uint32_t*>(L.q + o2) =
              e4m3_encode4(v[0] * sc.scale, v[1] * sc.scale, v[2] * sc.scale, v[3] * sc.scale);
          if (kWriteW) *reinterpret_cast<float4*>(L.Wout + o2) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dequantize + un-whiten: W^ = decode(q) * inv; G^ = beta W^ + (W^ U * D_u) U^T.
// The first product runs on the exact codes and is scaled by inv afterwards
// (per tensor, or per 128-column segment).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void decode8(uint32_t lo, uint32_t hi, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode(lo, i);
    v[4 + i] = e4m3_decode(hi, i);
  }
}

template <bool kBlockScale>
__global__ __launch_bounds__(kRowThreads) void k_dequant_unwhiten(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kBlockScale ? kBlock / kChunk : 1);
  __shared__ float red[kWaves][kRT * 8][64];
  const int64_t d_in = L.d_in, nseg = d_in / kBlock;
  const float inv0 = kBlockScale ? 1.f : L.inv[0];
  const uint4* P1 = L.P;
  f32x4 acc[2][kRT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 sacc[2][kRT];
  for (int c = x.c0; c < x.c1; ++c) {
    if (kBlockScale && (c & 3) == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) sacc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 a[2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 3; ++s) a[h][s] = as_bf16x8(P1[(size_t)((c * 2 + h) * 3 + s) * 64 + x.lane]);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const uint8_t* qp = L.q + x.row[rt] * d_in + kChunk * c + 4 * x.g;
      float v[8];
      decode8(*reinterpret_cast<const uint32_t*>(qp), *reinterpret_cast<const uint32_t*>(qp + 16), v);
      bf16x8 bq;
#pragma unroll
      for (int i = 0; i < 8; ++i) bq[i] = (__bf16)v[i];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (kBlockScale) sacc[h][rt] = mfma3x1(a[h], bq, sacc[h][rt]);
        else acc[h][rt] = mfma3x1(a[h], bq, acc[h][rt]);
      }
    }
    if (kBlockScale && (c & 3) == 3) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const float s = L.inv[x.row[rt] * nseg + (c >> 2)];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][rt][i] = fmaf(sacc[h][rt][i], s, acc[h][rt][i]);
      }
    }
  }
  float cp[kRT][8];
  reduce_waves(acc, red, x, cp);
  const float* du = L.coef + GIFT_COEF_DU;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = du[rank_of(j, x.g)] * inv0;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) cp[rt][j] *= d;
  }
  bf16x8 b[kRT][3];
  cprime_operands(cp, b);
  const float beta = L.coef[GIFT_COEF_BETA];
  for (int c = x.c1 - 1; c >= x.c0; --c) {
    bf16x8 a[2][3];
    load_p2(L, c, x.lane, a);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const f32x4 corr = mfma3x3(a[t], b[rt], f32x4{0.f, 0.f, 0.f, 0.f});
        if (!x.ok[rt]) continue;
        const int64_t o = x.row[rt] * d_in + kChunk * c + 16 * t + 4 * x.g;
        const float s = kBlockScale ? L.inv[x.row[rt] * nseg + (c >> 2)] : inv0;
        const uint32_t qv = *reinterpret_cast<const uint32_t*>(L.q + o);
        float4 out;
        out.x = fmaf(beta, e4m3_decode(qv, 0) * s, corr[0]);
        out.y = fmaf(beta, e4m3_decode(qv, 1) * s, corr[1]);
        out.z = fmaf(beta, e4m3_decode(qv, 2) * s, corr[2]);
        out.w = fmaf(beta, e4m3_decode(qv, 3) * s, corr[3]);
        *reinterpret_cast<float4*>(L.Ghat + o) = out;
      }
  }
}

// ---------------------------------------------------------------------------
// flat kernels: Euclidean quantization, plain dequantization, error sums
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_flat_amax(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  __shared__ uint32_t mx[kThreads / 64];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    if (e < n) {
      const float4 v = *reinterpret_cast<const float4*>(L.G + e);
      m = max(max(m, abs_bits(v.x)), max(abs_bits(v.y), max(abs_bits(v.z), abs_bits(v.w))));
    }
  }
  m = block_max_u32<kThreads>(m, mx);
  if (threadIdx.x == 0) L.part[tile] = m;
}

// Euclidean quantize (pass 2 of per-tensor, or the single pass of 1x128),
// optionally dequantizing in the same pass (the round trip).
template <bool kBlockScale, bool kDeq, bool kWriteW>
__global__ __launch_bounds__(kThreads) void k_flat_quant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  __shared__ uint32_t mx[kThreads / 64];
  Scale sc{1.f, 1.f, 0u};
  if (!kBlockScale) {
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) m = max(m, L.part[i]);
    m = block_max_u32<kThreads>(m, mx);
    sc = scale_from_amax_bits(m);
    if (tile == 0 && threadIdx.x == 0) {
      L.inv[0] = sc.inv;
      if (g.flags && sc.flags) atomicOr(g.flags, sc.flags);
    }
  }
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    const bool act = e < n;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) v = *reinterpret_cast<const float4*>(L.G + e);
    if (kBlockScale) {
      // 32 consecutive lanes hold one 128-element segment (d_in % 128 == 0)
      uint32_t m = max(max(abs_bits(v.x), abs_bits(v.y)), max(abs_bits(v.z), abs_bits(v.w)));
      m = half_wave_max_u32(m);
      sc = scale_from_amax_bits(m);
      if (act && (threadIdx.x & 31) == 0) {
        L.inv[e / kBlock] = sc.inv;
        if (g.flags && sc.flags) atomicOr(g.flags, sc.flags);
      }
    }
    if (!act) continue;
    const uint32_t c = e4m3_encode4(v.x * sc.scale, v.y * sc.scale, v.z * sc.scale, v.w * sc.scale);
    *reinterpret_cast<uint32_t*>(L.q + e) = c;
    if (kWriteW) *reinterpret_cast<float4*>(L.Wout + e) = v;
    if (kDeq) {
      float4 o;
      o.x = e4m3_decode(c, 0) * sc.inv;
      o.y = e4m3_decode(c, 1) * sc.inv;
      o.z = e4m3_decode(c, 2) * sc.inv;
      o.w = e4m3_decode(c, 3) * sc.inv;
      *reinterpret_cast<float4*>(L.Ghat + e) = o;
    }
  }
}

// plain dequantize of Euclidean layers: G^ = decode(q) * inv
template <bool kBlockScale>
__global__ __launch_bounds__(kThreads) void k_flat_dequant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  const float inv0 = kBlockScale ? 1.f : L.inv[0];
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    if (e >= n) continue;
    const float s = kBlockScale ? L.inv[e / kBlock] : inv0;
    const uint32_t c = *reinterpret_cast<const uint32_t*>(L.q + e);
    float4 o;
    o.x = e4m3_decode(c, 0) * s;
    o.y = e4m3_decode(c, 1) * s;
    o.z = e4m3_decode(c, 2) * s;
    o.w = e4m3_decode(c, 3) * s;
    *reinterpret_cast<float4*>(L.Ghat + e) = o;
  }
}

__global__ __launch_bounds__(kThreads) void k_err_partial(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  __shared__ double sh[2][kThreads / 64];
  double se = 0.0, sg = 0.0;
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    if (e < n) {
      const float4 a = *reinterpret_cast<const float4*>(L.G + e);
      const float4 b = *reinterpret_cast<const float4*>(L.Ghat + e);
      const double d0 = (double)b.x - (double)a.x, d1 = (double)b.y - (double)a.y;
      const double d2 = (double)b.z - (double)a.z, d3 = (double)b.w - (double)a.w;
      se += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
      sg += (double)a.x * a.x + (double)a.y * a.y + (double)a.z * a.z + (double)a.w * a.w;
    }
  }
  se = wave_sum_f64(se);
  sg = wave_sum_f64(sg);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sh[0][wave] = se; sh[1][wave] = sg; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) { a += sh[0][w]; b += sh[1][w]; }
    L.part2[2 * tile] = a;
    L.part2[2 * tile + 1] = b;
  }
}

// one workgroup per layer: fixed-order sum of the tile partials
__global__ __launch_bounds__(kThreads) void k_err_final(GroupDev g, int out_base) {
  const LayerDev& L = g.L[blockIdx.x];
  __shared__ double sh[2][kThreads / 64];
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) {
    a += L.part2[2 * i];
    b += L.part2[2 * i + 1];
  }
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sh[0][wave] = a; sh[1][wave] = b; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double x = 0.0, y = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) { x += sh[0][w]; y += sh[1][w]; }
    g.out[2 * (out_base + blockIdx.x)] = x;
    g.out[2 * (out_base + blockIdx.x) + 1] = y;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int row_tiles(int64_t d_out) { return (int)((d_out + kRows - 1) / kRows); }
int flat_tiles(int64_t n) { return (int)((n + kFlatTile - 1) / kFlatTile); }
size_t pack_bytes(int64_t d_in) { return (size_t)(d_in / kChunk) * 2 * 2 * 3 * 64 * 16; }

hipError_t launch_pack(const PackGroup& pg, hipStream_t s) {
  int maxd = 0;
  for (int i = 0; i < pg.n; ++i) maxd = pg.f[i].d_in > maxd ? pg.f[i].d_in : maxd;
  const int per = 2 * (maxd / kChunk) * 2 * 64;
  k_pack_u<<<dim3((per + kThreads - 1) / kThreads, pg.n), dim3(kThreads), 0, s>>>(pg);
  return hipGetLastError();
}

hipError_t launch_whiten_quantize(const GroupDev& g, bool block, bool write_w, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kRowThreads);
  if (block) {
    if (write_w) k_whiten_b128<true><<<grid, blk, 0, s>>>(g);
    else k_whiten_b128<false><<<grid, blk, 0, s>>>(g);
  } else {
    k_whiten_p1<<<grid, blk, 0, s>>>(g);
    if (write_w) k_whiten_p2<true><<<grid, blk, 0, s>>>(g);
    else k_whiten_p2<false><<<grid, blk, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_flat_quantize(const GroupDev& g, bool block, bool deq, bool write_w,
                                hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kThreads);
  if (!block) k_flat_amax<<<grid, blk, 0, s>>>(g);
#define GIFT_FQ(B, D, W) k_flat_quant<B, D, W><<<grid, blk, 0, s>>>(g)
  if (block) {
    if (deq) { if (write_w) GIFT_FQ(true, true, true); else GIFT_FQ(true, true, false); }
    else     { if (write_w) GIFT_FQ(true, false, true); else GIFT_FQ(true, false, false); }
  } else {
    if (deq) { if (write_w) GIFT_FQ(false, true, true); else GIFT_FQ(false, true, false); }
    else     { if (write_w) GIFT_FQ(false, false, true); else GIFT_FQ(false, false, false); }
  }
#undef GIFT_FQ
  return hipGetLastError();
}

hipError_t launch_dequant(const GroupDev& g, bool block, bool white, hipStream_t s) {
  if (white) {
    const dim3 grid(g.total_tiles), blk(kRowThreads);
    if (block) k_dequant_unwhiten<true><<<grid, blk, 0, s>>>(g);
    else k_dequant_unwhiten<false><<<grid, blk, 0, s>>>(g);
  } else {
    const dim3 grid(g.total_tiles), blk(kThreads);
    if (block) k_flat_dequant<true><<<grid, blk, 0, s>>>(g);
    else k_flat_dequant<false><<<grid, blk, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_error(const GroupDev& g, int out_base, hipStream_t s) {
  k_err_partial<<<dim3(g.total_tiles), dim3(kThreads), 0, s>>>(g);
  k_err_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g, out_base);
  return hipGetLastError();
}

}  // namespace gift
