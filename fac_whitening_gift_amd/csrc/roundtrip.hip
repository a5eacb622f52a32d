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
// row-workgroup geometry.  A layer's row kernels use tiles of kRows rows x
// one column group; a column group is kWaves units of `unit` chunks, one unit
// per wave (unit = 2 chunks for per-tensor scaling, 4 = one 128-column
// segment for block scaling).  tile = row_block * ngrp + group.
// ---------------------------------------------------------------------------
struct RowCtx {
  int64_t row[kRT];   // clamped row of each 16-row tile for this lane
  bool ok[kRT];       // row < d_out
  int grp;            // column group of the workgroup
  int c0, c1;         // this wave's chunk range (may be empty)
  int lane, wave, r16, g;
};

__device__ __forceinline__ RowCtx row_ctx(const LayerDev& L, int tile, int unit) {
  RowCtx x;
  x.lane = threadIdx.x & 63;
  x.wave = threadIdx.x >> 6;
  x.r16 = x.lane & 15;
  x.g = x.lane >> 4;
  x.grp = tile % L.ngrp;
  const int64_t row0 = (int64_t)(tile / L.ngrp) * kRows;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int64_t r = row0 + 16 * rt + x.r16;
    x.ok[rt] = r < L.d_out;
    x.row[rt] = x.ok[rt] ? r : L.d_out - 1;
  }
  const int nch = (int)(L.d_in / kChunk);
  const int u = x.grp * kWaves + x.wave;
  x.c0 = min(nch, u * unit);
  x.c1 = min(nch, x.c0 + unit);
  return x;
}

// Two-stage software pipeline over n iterations: the loads of iteration i+1
// are issued before the compute of iteration i.
// pipeline2 with the first iteration's buffer already loaded (its loads were
// issued before other independent loads of the caller)
template <class Buf, class Map, class Load, class Comp>
__device__ __forceinline__ void pipeline2_from(int n, Buf& a, Map map, Load load, Comp comp) {
  Buf b;
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) load(map(i + 1), b);
    comp(map(i), a);
    if (i + 1 >= n) break;
    if (i + 2 < n) load(map(i + 2), a);
    comp(map(i + 1), b);
  }
}

template <class Buf, class Map, class Load, class Comp>
__device__ __forceinline__ void pipeline2(int n, Map map, Load load, Comp comp) {
  Buf a, b;
  if (n > 0) load(map(0), a);
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) load(map(i + 1), b);
    comp(map(i), a);
    if (i + 1 >= n) break;
    if (i + 2 < n) load(map(i + 2), a);
    comp(map(i + 1), b);
  }
}

__device__ __forceinline__ void load_a(const uint4* P, int c, int lane, uint4 (&a)[2][3]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int s = 0; s < 3; ++s) a[h][s] = P[(size_t)((c * 2 + h) * 3 + s) * 64 + lane];
}

__device__ __forceinline__ void as_ops(const uint4 (&u)[2][3], bf16x8 (&a)[2][3]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int s = 0; s < 3; ++s) a[h][s] = as_bf16x8(u[h][s]);
}

__device__ __forceinline__ const uint4* p2_of(const LayerDev& L) {
  return L.P + (size_t)(L.d_in / kChunk) * 2 * 3 * 64;
}

// rank index of element j (0..7) of a lane's c vector
__device__ __forceinline__ int rank_of(int j, int g) { return 16 * (j >> 2) + 4 * g + (j & 3); }

// Sum the 8 waves' partial c (16 values per lane) in a fixed order and store
// the workgroup's partial for its column group: cpart[grp][row][rank].
__device__ __forceinline__ void store_cpart(const LayerDev& L, const RowCtx& x, int tile,
                                            f32x4 (&acc)[2][kRT], float (*red)[kRT * 8][64]) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[x.wave][rt * 8 + h * 4 + i][x.lane] = acc[h][rt][i];
  __syncthreads();
  const int64_t row0 = (int64_t)(tile / L.ngrp) * kRows;
  for (int p = threadIdx.x; p < kRT * 8 * 64; p += kRowThreads) {
    const int q = p >> 6, ln = p & 63;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w][q][ln];
    const int rt = q >> 3, j = q & 7;
    const int64_t row = row0 + 16 * rt + (ln & 15);
    if (row < L.d_out) L.cbuf[((int64_t)x.grp * L.d_out + row) * kRank + rank_of(j, ln >> 4)] = s;
  }
}

// c of the workgroup's rows = fixed-order sum of the column-group partials.
// The 32 rows x 8 rank quads are spread over the workgroup (one float4 per
// group per thread, all loads in flight together) and summed into LDS; then
// each lane takes its 8 ranks of each row tile, times dk[rank] * extra, split
// into the second product's bf16 operands.  Contains a workgroup barrier.
struct CSum {
  float v[kRows][kRank + 4];
};

__device__ __forceinline__ void load_c_operands(const LayerDev& L, const RowCtx& x, int tile,
                                                const float* dk, float extra, CSum& cs,
                                                bf16x8 (&b)[kRT][3]) {
  constexpr int kItems = kRows * kRank / 4;  // float4 items per workgroup
  constexpr int kBatch = 8;
  const int64_t row0 = (int64_t)(tile / L.ngrp) * kRows;
  for (int e = threadIdx.x; e < kItems; e += kRowThreads) {
    const int r = e >> 3, q4 = e & 7;
    const int64_t row = min(row0 + r, L.d_out - 1);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g0 = 0; g0 < L.ngrp; g0 += kBatch) {
      float4 u[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int gi = g0 + k < L.ngrp ? g0 + k : L.ngrp - 1;
        u[k] = *reinterpret_cast<const float4*>(L.cbuf + ((int64_t)gi * L.d_out + row) * kRank +
                                                4 * q4);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (g0 + k < L.ngrp) {
          sum.x += u[k].x; sum.y += u[k].y; sum.z += u[k].z; sum.w += u[k].w;
        }
      }
    }
    *reinterpret_cast<float4*>(&cs.v[r][4 * q4]) = sum;
  }
  __syncthreads();
  float d8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) d8[j] = dk[rank_of(j, x.g)] * extra;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float cp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cp[j] = cs.v[16 * rt + x.r16][rank_of(j, x.g)] * d8[j];
    split3(cp, b[rt]);
  }
}

// ---------------------------------------------------------------------------
// first product, partial over a column group: c^T = U^T G^T (G fp32 split
// three ways), or U^T decode(q)^T on the exact codes (dequantize; with block
// scaling each 128-column segment's product is scaled by its inv).
// ---------------------------------------------------------------------------
struct G1Buf {
  uint4 a[2][3];
  float4 g[kRT][2];
};

template <int kUnit>
__global__ __launch_bounds__(kRowThreads) void k_cpart_g(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kUnit);
  // the per-tensor amax slot starts at 0; the next launch max-combines into it
  if (L.amax && tile == 0 && threadIdx.x == 0) *L.amax = 0u;
  __shared__ float red[kWaves][kRT * 8][64];
  const uint4* P1 = L.P;
  const int64_t d_in = L.d_in;
  f32x4 acc[2][kRT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  pipeline2<G1Buf>(
      x.c1 - x.c0, [&](int i) { return x.c0 + i; },
      [&](int c, G1Buf& b) {
        load_a(P1, c, x.lane, b.a);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const float* gp = L.G + x.row[rt] * d_in + kChunk * c + 4 * x.g;
          b.g[rt][0] = *reinterpret_cast<const float4*>(gp);
          b.g[rt][1] = *reinterpret_cast<const float4*>(gp + 16);
        }
      },
      [&](int, const G1Buf& b) {
        bf16x8 a[2][3];
        as_ops(b.a, a);
        bf16x8 sp[kRT][3];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const float4 u = b.g[rt][0], v = b.g[rt][1];
          const float gv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
          split3(gv, sp[rt]);
        }
        f32x4 t4[2 * kRT];
        const bf16x8(*pa[2 * kRT])[3];
        const bf16x8(*pb[2 * kRT])[3];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            t4[h * kRT + rt] = acc[h][rt];
            pa[h * kRT + rt] = &a[h];
            pb[h * kRT + rt] = &sp[rt];
          }
        mfma3x3_n<2 * kRT>(pa, pb, t4);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) acc[h][rt] = t4[h * kRT + rt];
      });
  store_cpart(L, x, tile, acc, red);
}

__device__ __forceinline__ void decode8(uint32_t lo, uint32_t hi, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode(lo, i);
    v[4 + i] = e4m3_decode(hi, i);
  }
}

struct Q1Buf {
  uint4 a[2][3];
  uint32_t q[kRT][2];
};

template <bool kBlockScale>
__global__ __launch_bounds__(kRowThreads) void k_cpart_q(GroupDev gd) {
  constexpr int kUnit = kBlockScale ? kBlock / kChunk : 2;
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kUnit);
  __shared__ float red[kWaves][kRT * 8][64];
  const uint4* P1 = L.P;
  const int64_t d_in = L.d_in;
  f32x4 acc[2][kRT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[h][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  pipeline2<Q1Buf>(
      x.c1 - x.c0, [&](int i) { return x.c0 + i; },
      [&](int c, Q1Buf& b) {
        load_a(P1, c, x.lane, b.a);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const uint8_t* qp = L.q + x.row[rt] * d_in + kChunk * c + 4 * x.g;
          b.q[rt][0] = *reinterpret_cast<const uint32_t*>(qp);
          b.q[rt][1] = *reinterpret_cast<const uint32_t*>(qp + 16);
        }
      },
      [&](int, const Q1Buf& b) {
        bf16x8 a[2][3];
        as_ops(b.a, a);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          float v[8];
          decode8(b.q[rt][0], b.q[rt][1], v);
          bf16x8 bq;
#pragma unroll
          for (int i = 0; i < 8; ++i) bq[i] = (__bf16)v[i];
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[h][rt] = mfma3x1(a[h], bq, acc[h][rt]);
        }
      });
  if (kBlockScale && x.c0 < x.c1) {
    // the wave's unit is exactly one 128-column segment
    const int64_t nseg = d_in / kBlock;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const float s = L.inv[x.row[rt] * nseg + (x.c0 >> 2)];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][rt][i] *= s;
    }
  }
  store_cpart(L, x, tile, acc, red);
}

// ---------------------------------------------------------------------------
// whitened tensor for one chunk: w = alpha g + correction
// ---------------------------------------------------------------------------
struct G3Buf {
  uint4 a[2][3];
  float4 g[2][kRT];
};

__device__ __forceinline__ void load_g3(const LayerDev& L, const RowCtx& x, int c, G3Buf& b) {
  load_a(p2_of(L), c, x.lane, b.a);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      b.g[t][rt] = *reinterpret_cast<const float4*>(L.G + x.row[rt] * L.d_in + kChunk * c +
                                                    16 * t + 4 * x.g);
}

__device__ __forceinline__ void whiten_chunk(const G3Buf& b, const bf16x8 (&cb)[kRT][3],
                                             float alpha, float4 (&w)[2][kRT]) {
  bf16x8 a[2][3];
  as_ops(b.a, a);
  f32x4 corr[2 * kRT];
  const bf16x8(*pa[2 * kRT])[3];
  const bf16x8(*pb[2 * kRT])[3];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      corr[t * kRT + rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pa[t * kRT + rt] = &a[t];
      pb[t * kRT + rt] = &cb[rt];
    }
  mfma3x3_n<2 * kRT>(pa, pb, corr);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const f32x4 c = corr[t * kRT + rt];
      const float4 gv = b.g[t][rt];
      w[t][rt] = make_float4(fmaf(alpha, gv.x, c[0]), fmaf(alpha, gv.y, c[1]),
                             fmaf(alpha, gv.z, c[2]), fmaf(alpha, gv.w, c[3]));
    }
}

__device__ __forceinline__ uint32_t amax4(uint32_t m, const float4& v) {
  m = max(m, abs_bits(v.x));
  m = max(m, abs_bits(v.y));
  m = max(m, abs_bits(v.z));
  return max(m, abs_bits(v.w));
}

// ---------------------------------------------------------------------------
// per-tensor scaling, pass 1: partial amax of W per workgroup
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads) void k_whiten_amax(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, 2);
  __shared__ uint32_t mx[kWaves];
  __shared__ CSum cs;
  G3Buf first;
  if (x.c0 < x.c1) load_g3(L, x, x.c0, first);
  bf16x8 b[kRT][3];
  load_c_operands(L, x, tile, L.coef + GIFT_COEF_DW, 1.f, cs, b);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  uint32_t m = 0u;
  pipeline2_from<G3Buf>(
      x.c1 - x.c0, first, [&](int i) { return x.c0 + i; },
      [&](int c, G3Buf& buf) { load_g3(L, x, c, buf); },
      [&](int, const G3Buf& buf) {
        float4 w[2][kRT];
        whiten_chunk(buf, b, alpha, w);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            if (x.ok[rt]) m = amax4(m, w[t][rt]);
      });
  m = block_max_u32<kRowThreads>(m, mx);
  // unsigned max is order-independent: the result does not depend on timing
  if (threadIdx.x == 0) atomicMax(L.amax, m);
}

// per-tensor scaling, pass 2: layer amax from the partials, W again, codes
template <bool kWriteW>
__global__ __launch_bounds__(kRowThreads) void k_whiten_quant(GroupDev gd) {
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, 2);
  G3Buf first;
  if (x.c0 < x.c1) load_g3(L, x, x.c0, first);
  const Scale sc = scale_from_amax_bits(*L.amax);
  if (tile == 0 && threadIdx.x == 0) {
    L.inv[0] = sc.inv;
    if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
  }
  __shared__ CSum cs;
  bf16x8 b[kRT][3];
  load_c_operands(L, x, tile, L.coef + GIFT_COEF_DW, 1.f, cs, b);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  pipeline2_from<G3Buf>(
      x.c1 - x.c0, first, [&](int i) { return x.c0 + i; },
      [&](int c, G3Buf& buf) { load_g3(L, x, c, buf); },
      [&](int c, const G3Buf& buf) {
        float4 w[2][kRT];
        whiten_chunk(buf, b, alpha, w);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            if (!x.ok[rt]) continue;
            const int64_t o = x.row[rt] * L.d_in + kChunk * c + 16 * t + 4 * x.g;
            const float4 v = w[t][rt];
            *reinterpret_cast<uint32_t*>(L.q + o) =
                e4m3_encode4(v.x * sc.scale, v.y * sc.scale, v.z * sc.scale, v.w * sc.scale);
            if (kWriteW) *reinterpret_cast<float4*>(L.Wout + o) = v;
          }
      });
}

// ---------------------------------------------------------------------------
// 1x128 block scaling: each wave owns one 128-column segment of 32 rows; a
// segment's amax is the max over the lane's 32 values and the four lanes that
// hold the same row.
// ---------------------------------------------------------------------------
template <bool kWriteW>
__global__ __launch_bounds__(kRowThreads) void k_whiten_b128(GroupDev gd) {
  constexpr int kPer = kBlock / kChunk;
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kPer);
  __shared__ CSum cs;
  const bool busy = x.c0 < x.c1;
  G3Buf buf[2];
  if (busy) load_g3(L, x, x.c0, buf[0]);
  bf16x8 b[kRT][3];
  load_c_operands(L, x, tile, L.coef + GIFT_COEF_DW, 1.f, cs, b);
  if (!busy) return;  // no barrier below
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  const int64_t nseg = L.d_in / kBlock;
  float4 w[kPer][2][kRT];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k + 1 < kPer) load_g3(L, x, x.c0 + k + 1, buf[(k + 1) & 1]);
    whiten_chunk(buf[k & 1], b, alpha, w[k]);
  }
  const int seg = x.c0 / kPer;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
#pragma unroll
      for (int t = 0; t < 2; ++t) m = amax4(m, w[k][t][rt]);
    m = max(m, (uint32_t)__shfl_xor(m, 16, 64));
    m = max(m, (uint32_t)__shfl_xor(m, 32, 64));
    const Scale sc = scale_from_amax_bits(m);
    if (!x.ok[rt]) continue;
    if (x.g == 0) {
      L.inv[x.row[rt] * nseg + seg] = sc.inv;
      if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t o2 = x.row[rt] * L.d_in + kChunk * (x.c0 + k) + 16 * t + 4 * x.g;
        const float4 v = w[k][t][rt];
        *reinterpret_cast<uint32_t*>(L.q + o2) =
            e4m3_encode4(v.x * sc.scale, v.y * sc.scale, v.z * sc.scale, v.w * sc.scale);
        if (kWriteW) *reinterpret_cast<float4*>(L.Wout + o2) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// dequantize + un-whiten: G^ = beta W^ + (W^ U * D_u) U^T, W^ = decode(q) * inv
// ---------------------------------------------------------------------------
struct Q3Buf {
  uint4 a[2][3];
  uint32_t q[2][kRT];
  float s[kRT];
};

template <bool kBlockScale>
__global__ __launch_bounds__(kRowThreads) void k_unwhiten(GroupDev gd) {
  constexpr int kUnit = kBlockScale ? kBlock / kChunk : 2;
  const int l = find_layer(gd, blockIdx.x);
  const LayerDev& L = gd.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const RowCtx x = row_ctx(L, tile, kUnit);
  __shared__ CSum cs;
  const bool busy = x.c0 < x.c1;
  const int64_t d_in = L.d_in, nseg = d_in / kBlock;
  const float inv0 = kBlockScale ? 1.f : L.inv[0];
  const uint4* P2 = p2_of(L);
  auto load = [&](int c, Q3Buf& bf) {
    load_a(P2, c, x.lane, bf.a);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        bf.q[t][rt] = *reinterpret_cast<const uint32_t*>(L.q + x.row[rt] * d_in + kChunk * c +
                                                         16 * t + 4 * x.g);
      bf.s[rt] = kBlockScale ? L.inv[x.row[rt] * nseg + (c >> 2)] : inv0;
    }
  };
  Q3Buf first;
  if (busy) load(x.c0, first);
  bf16x8 b[kRT][3];
  load_c_operands(L, x, tile, L.coef + GIFT_COEF_DU, inv0, cs, b);
  if (!busy) return;  // no barrier below
  const float beta = L.coef[GIFT_COEF_BETA];
  pipeline2_from<Q3Buf>(
      x.c1 - x.c0, first, [&](int i) { return x.c0 + i; }, load,
      [&](int c, const Q3Buf& bf) {
        bf16x8 a[2][3];
        as_ops(bf.a, a);
        f32x4 cr[2 * kRT];
        const bf16x8(*pa[2 * kRT])[3];
        const bf16x8(*pb[2 * kRT])[3];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            cr[t * kRT + rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            pa[t * kRT + rt] = &a[t];
            pb[t * kRT + rt] = &b[rt];
          }
        mfma3x3_n<2 * kRT>(pa, pb, cr);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            const f32x4 corr = cr[t * kRT + rt];
            if (!x.ok[rt]) continue;
            const int64_t o = x.row[rt] * d_in + kChunk * c + 16 * t + 4 * x.g;
            const float s = bf.s[rt];
            const uint32_t qv = bf.q[t][rt];
            float4 out;
            out.x = fmaf(beta, e4m3_decode(qv, 0) * s, corr[0]);
            out.y = fmaf(beta, e4m3_decode(qv, 1) * s, corr[1]);
            out.z = fmaf(beta, e4m3_decode(qv, 2) * s, corr[2]);
            out.w = fmaf(beta, e4m3_decode(qv, 3) * s, corr[3]);
            *reinterpret_cast<float4*>(L.Ghat + o) = out;
          }
      });
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

// one workgroup per layer: the layer's amax from the tile partials
__global__ __launch_bounds__(kThreads) void k_amax_final(GroupDev g) {
  const LayerDev& L = g.L[blockIdx.x];
  __shared__ uint32_t mx[kThreads / 64];
  uint32_t m = 0u;
  for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) m = max(m, L.part[i]);
  m = block_max_u32<kThreads>(m, mx);
  if (threadIdx.x == 0) *L.amax = m;
}

// Euclidean quantize (pass 2 of per-tensor, or the single pass of 1x128),
// optionally dequantizing in the same pass (the round trip).
template <bool kBlockScale, bool kDeq, bool kWriteW>
__global__ __launch_bounds__(kThreads) void k_flat_quant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  Scale sc{1.f, 1.f, 0u};
  if (!kBlockScale) {
    sc = scale_from_amax_bits(*L.amax);
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
int row_blocks(int64_t d_out) { return (int)((d_out + kRows - 1) / kRows); }
// column groups of a whitened layer: kWaves units of 2 chunks (per-tensor
// scaling) or of one 128-column segment (block scaling)
int col_groups(int64_t d_in, bool block) {
  const int64_t unit = block ? kBlock / kChunk : 2;
  const int64_t units = (d_in / kChunk + unit - 1) / unit;
  return (int)((units + kWaves - 1) / kWaves);
}
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
    k_cpart_g<kBlock / kChunk><<<grid, blk, 0, s>>>(g);
    if (write_w) k_whiten_b128<true><<<grid, blk, 0, s>>>(g);
    else k_whiten_b128<false><<<grid, blk, 0, s>>>(g);
  } else {
    k_cpart_g<2><<<grid, blk, 0, s>>>(g);
    k_whiten_amax<<<grid, blk, 0, s>>>(g);
    if (write_w) k_whiten_quant<true><<<grid, blk, 0, s>>>(g);
    else k_whiten_quant<false><<<grid, blk, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_flat_quantize(const GroupDev& g, bool block, bool deq, bool write_w,
                                hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kThreads);
  if (!block) {
    k_flat_amax<<<grid, blk, 0, s>>>(g);
    k_amax_final<<<dim3(g.n), blk, 0, s>>>(g);
  }
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
    if (block) {
      k_cpart_q<true><<<grid, blk, 0, s>>>(g);
      k_unwhiten<true><<<grid, blk, 0, s>>>(g);
    } else {
      k_cpart_q<false><<<grid, blk, 0, s>>>(g);
      k_unwhiten<false><<<grid, blk, 0, s>>>(g);
    }
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
