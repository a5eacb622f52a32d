// GIFT FP8 round trip on gfx950: whiten + quantize, dequantize + un-whiten,
// the Euclidean baseline and the error reduction.
//
// The operation (GIFT review, "What carries the argument"): the gradient G is
// right-multiplied by A_r^-1/2 = alpha I + U diag(D_w) U^T before FP8 and by
// A_r^1/2 = beta I + U diag(D_u) U^T after it.  Per row g of G:
//     c = g U (32 numbers), w = alpha g + (c * D_w) U^T,
// so every output element needs the full-row reduction c first.  These
// kernels give each workgroup a block of kRows rows over the full row
// length: phase A reduces c for the block (rank index on the lane, columns
// striped over waves, a fixed-order LDS reduction), phase B streams the
// columns again and applies the rank-32 correction with U's row in
// registers.  Per-tensor scaling needs the amax of the whole whitened
// tensor before any code can be written, so it takes two launches: pass 1
// writes one partial amax per row block, pass 2 reduces the partials of its
// layer and quantizes.  1x128 block scaling needs only the row and is one
// launch.
#include "device.hpp"

namespace gift {

constexpr int kThreads = 256;
constexpr int kRows = 8;            // rows of G per workgroup (row kernels)
constexpr int kFlatTile = 4096;     // elements per workgroup (flat kernels)

// ---------------------------------------------------------------------------
// shared building blocks of the row kernels
// ---------------------------------------------------------------------------

// cs[r][k] = dk[k] * sum_j x(r, j) U[j][k] for the kRows rows of the block.
// Lane k of each half-wave owns rank index k; the 8 half-waves stripe the
// columns; the 8 partial sums are added in a fixed order.
template <class Load>
__device__ __forceinline__ void rank_coeffs(Load load, int64_t d_in,
                                            const float* __restrict__ U,
                                            const float* __restrict__ dk,
                                            float (*red)[kRows][kRank],
                                            float (*cs)[kRank]) {
  const int k = threadIdx.x & (kRank - 1);
  const int jg = threadIdx.x >> 5;
  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
#pragma unroll 2
  for (int64_t j = jg; j < d_in; j += kThreads / kRank) {
    const float u = U[j * kRank + k];
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = fmaf(load(r, j), u, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) red[jg][r][k] = acc[r];
  __syncthreads();
  {
    const int r = threadIdx.x >> 5;  // kRows * kRank == kThreads
    float s = 0.f;
#pragma unroll
    for (int gI = 0; gI < kThreads / kRank; ++gI) s += red[gI][r][k];
    cs[r][k] = s * dk[k];
  }
  __syncthreads();
}

// U[j][0..31] -> registers
__device__ __forceinline__ void load_urow(const float* __restrict__ U, int64_t j,
                                          float (&u)[kRank]) {
  const float4* p = reinterpret_cast<const float4*>(U + j * kRank);
#pragma unroll
  for (int i = 0; i < kRank / 4; ++i) {
    float4 v = p[i];
    u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
  }
}

// x0 * xv + sum_k cs[k] u[k]  (explicit fma chain: the same bits in every pass)
__device__ __forceinline__ float apply_row(const float* __restrict__ csr,
                                           const float (&u)[kRank], float x0, float xv) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kRank; ++k) s = fmaf(csr[k], u[k], s);
  return fmaf(x0, xv, s);
}

// ---------------------------------------------------------------------------
// whiten, pass 1 (per-tensor scaling): c' = (G U) * D_w -> cbuf, partial amax
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_whiten_amax(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t row0 = (int64_t)tile * kRows, d_in = L.d_in;
  const int nrows = (int)min<int64_t>(kRows, L.d_out - row0);
  __shared__ float red[kThreads / kRank][kRows][kRank];
  __shared__ float cs[kRows][kRank];
  __shared__ uint32_t mx[kThreads / 64];
  const float* __restrict__ G = L.G;
  auto loadG = [&](int r, int64_t j) { return G[(row0 + min(r, nrows - 1)) * d_in + j]; };
  rank_coeffs(loadG, d_in, L.U, L.coef + GIFT_COEF_DW, red, cs);
  {
    const int r = threadIdx.x >> 5, k = threadIdx.x & 31;
    if (r < nrows) L.cbuf[(row0 + r) * kRank + k] = cs[r][k];
  }
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  uint32_t m = 0u;
  for (int64_t j = threadIdx.x; j < d_in; j += kThreads) {
    float u[kRank];
    load_urow(L.U, j, u);
    for (int r = 0; r < nrows; ++r) {
      const float w = apply_row(cs[r], u, alpha, G[(row0 + r) * d_in + j]);
      m = max(m, abs_bits(w));
    }
  }
  m = block_max_u32<kThreads>(m, mx);
  if (threadIdx.x == 0) L.part[tile] = m;
}

// ---------------------------------------------------------------------------
// whiten, quantize: pass 2 of per-tensor scaling (c' from cbuf, amax from the
// partials) or the single pass of 1x128 scaling (c' computed here).
// ---------------------------------------------------------------------------
template <bool kBlockScale, bool kWriteW>
__global__ __launch_bounds__(kThreads) void k_whiten_quant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t row0 = (int64_t)tile * kRows, d_in = L.d_in;
  const int nrows = (int)min<int64_t>(kRows, L.d_out - row0);
  __shared__ float red[kThreads / kRank][kRows][kRank];
  __shared__ float cs[kRows][kRank];
  __shared__ uint32_t mx[kThreads / 64];
  __shared__ uint32_t seg[kRows][kThreads / 64];
  const float* __restrict__ G = L.G;
  auto loadG = [&](int r, int64_t j) { return G[(row0 + min(r, nrows - 1)) * d_in + j]; };
  Scale sc{1.f, 1.f, 0u};
  if (kBlockScale) {
    rank_coeffs(loadG, d_in, L.U, L.coef + GIFT_COEF_DW, red, cs);
  } else {
    const int r = threadIdx.x >> 5, k = threadIdx.x & 31;
    cs[r][k] = L.cbuf[(row0 + min(r, nrows - 1)) * kRank + k];
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < L.n_tiles; i += kThreads) m = max(m, L.part[i]);
    m = block_max_u32<kThreads>(m, mx);  // also orders the cs stores
    sc = scale_from_amax_bits(m);
    if (tile == 0 && threadIdx.x == 0) {
      L.inv[0] = sc.inv;
      if (g.flags && sc.flags) atomicOr(g.flags, sc.flags);
    }
  }
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  const int wave = threadIdx.x >> 6, half = threadIdx.x >> 7;
  for (int64_t j0 = 0; j0 < d_in; j0 += kThreads) {
    const int64_t j = j0 + threadIdx.x;
    const bool act = j < d_in;
    float u[kRank];
    if (act) {
      load_urow(L.U, j, u);
    } else {
#pragma unroll
      for (int k = 0; k < kRank; ++k) u[k] = 0.f;
    }
    float w[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      w[r] = (act && r < nrows) ? apply_row(cs[r], u, alpha, G[(row0 + r) * d_in + j]) : 0.f;
      if (kBlockScale) {
        const uint32_t m = wave_max_u32(abs_bits(w[r]));
        if ((threadIdx.x & 63) == 0) seg[r][wave] = m;
      }
    }
    if (kBlockScale) __syncthreads();
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (!(act && r < nrows)) continue;
      if (kBlockScale) {
        const uint32_t a = seg[r][2 * half], b = seg[r][2 * half + 1];
        sc = scale_from_amax_bits(a > b ? a : b);
        if ((threadIdx.x & 127) == 0) {
          L.inv[(row0 + r) * (d_in / kBlock) + j / kBlock] = sc.inv;
          if (g.flags && sc.flags) atomicOr(g.flags, sc.flags);
        }
      }
      const int64_t o = (row0 + r) * d_in + j;
      L.q[o] = e4m3_encode1(w[r] * sc.scale);
      if (kWriteW) L.Wout[o] = w[r];
    }
    if (kBlockScale) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dequantize (+ un-whiten): W^ = decode(q) * inv; G^ = beta W^ + (W^ U * D_u) U^T
// ---------------------------------------------------------------------------
template <bool kBlockScale, bool kWhite>
__global__ __launch_bounds__(kThreads) void k_dequant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t row0 = (int64_t)tile * kRows, d_in = L.d_in;
  const int nrows = (int)min<int64_t>(kRows, L.d_out - row0);
  __shared__ float red[kThreads / kRank][kRows][kRank];
  __shared__ float cs[kRows][kRank];
  const uint8_t* __restrict__ q = L.q;
  const float* __restrict__ inv = L.inv;
  const float inv0 = kBlockScale ? 0.f : inv[0];
  auto loadW = [&](int r, int64_t j) {
    const int64_t row = row0 + min(r, nrows - 1);
    const float s = kBlockScale ? inv[row * (d_in / kBlock) + j / kBlock] : inv0;
    return e4m3_decode(q[row * d_in + j], 0) * s;
  };
  float beta = 1.f;
  if (kWhite) {
    rank_coeffs(loadW, d_in, L.U, L.coef + GIFT_COEF_DU, red, cs);
    beta = L.coef[GIFT_COEF_BETA];
  }
  for (int64_t j = threadIdx.x; j < d_in; j += kThreads) {
    float u[kRank];
    if (kWhite) load_urow(L.U, j, u);
    for (int r = 0; r < nrows; ++r) {
      const float wh = loadW(r, j);
      L.Ghat[(row0 + r) * d_in + j] = kWhite ? apply_row(cs[r], u, beta, wh) : wh;
    }
  }
}

// ---------------------------------------------------------------------------
// flat kernels: Euclidean quantization and the error sums
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

hipError_t launch_whiten_quantize(const GroupDev& g, bool block, bool write_w, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kThreads);
  if (block) {
    if (write_w) k_whiten_quant<true, true><<<grid, blk, 0, s>>>(g);
    else k_whiten_quant<true, false><<<grid, blk, 0, s>>>(g);
  } else {
    k_whiten_amax<<<grid, blk, 0, s>>>(g);
    if (write_w) k_whiten_quant<false, true><<<grid, blk, 0, s>>>(g);
    else k_whiten_quant<false, false><<<grid, blk, 0, s>>>(g);
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
  const dim3 grid(g.total_tiles), blk(kThreads);
  if (block) {
    if (white) k_dequant<true, true><<<grid, blk, 0, s>>>(g);
    else k_dequant<true, false><<<grid, blk, 0, s>>>(g);
  } else {
    if (white) k_dequant<false, true><<<grid, blk, 0, s>>>(g);
    else k_dequant<false, false><<<grid, blk, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_error(const GroupDev& g, int out_base, hipStream_t s) {
  k_err_partial<<<dim3(g.total_tiles), dim3(kThreads), 0, s>>>(g);
  k_err_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g, out_base);
  return hipGetLastError();
}

}  // namespace gift
