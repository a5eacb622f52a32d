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
// same way.  U's two operand forms are split and packed when the factor is
// refreshed (or once per call, k_pack_u).
//
// Work is split into tiles of 64 (or 32) rows by 256 columns (one workgroup
// each).  A row's c = g U needs every column, so it is formed in two
// launches: each tile writes its partial c, then one workgroup per row block
// sums the column groups' partials in a fixed order (k_tile_cpart,
// k_tile_reduce).
// Per-tensor scaling then takes two more passes over G (k_tile_whiten: the
// tiles' amax; k_tile_quant: the layer amax, W again and the codes); 1x128
// block scaling and MXFP4 take one (k_tile_whiten with codes and scales).
// The dequantize side is k_tile_cpart on the codes, k_tile_reduce and
// k_tile_unwhiten.
#include <type_traits>

#include "device.hpp"

// No implicit contraction of a*b + c into fma: the two whitening passes of
// per-tensor scaling must compute bit-identical W (pass 1 takes its amax,
// pass 2 encodes it), and pass 1 multiplies c by D_w in registers where pass
// 2 reads the rounded product back.  Every fma below is written out.
#pragma clang fp contract(off)

// Tile height of the tile kernels, in 16-row MFMA tiles: this file is built
// twice, with 64-row tiles (namespace rt4) and, from roundtrip_rt2.hip, with
// 32-row tiles (namespace rt2) for groups too small to fill the machine with
// 64-row tiles.
#ifndef GIFT_TILE_RT
#define GIFT_TILE_RT 4
#define GIFT_TILE_NS rt4
#endif

namespace gift {
namespace GIFT_TILE_NS {

constexpr int kThreads = 256;       // flat kernels
constexpr int kFlatTile = 4096;     // elements per workgroup (flat kernels)
constexpr int kChunk = 32;          // columns per MFMA K chunk

// ---------------------------------------------------------------------------
// operand packs.  For a factor with nch = d_in/32 chunks, P holds two arrays
// of nch*2*3*64 uint4 (8 bf16 each), indexed ((c*2 + h)*3 + split)*64 + lane:
//   first  (U^T operand of c = g U):  element i of lane l (r16 = l%16,
//          g = l/16) = U[32c + perm(i)][16h + r16]
//   second (U operand of w = c' U^T): element i = U[32c + 16h + r16][perm(i)]
// with perm(i) = 16*(i/4) + 4g + i%4.
// A factor of rank above 32 stores U with 64 columns as two rank blocks of
// 32; its packs are the two blocks' packs one after the other (block b at
// uint4 offset b * nch * 2 * 2 * 3 * 64), and the kernels below take the
// number of rank blocks kRB as a template argument: one set of partial and
// final row coefficients per block, the second product summed over blocks.
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
    v[i] = which == 0 ? F.U[(int64_t)(kChunk * c + p) * F.ucols + 16 * h + r16]
                      : F.U[(int64_t)(kChunk * c + 16 * h + r16) * F.ucols + p];
  }
  bf16x8 s[3];
  split3(v, s);
  uint4* out = F.P + (size_t)which * nch * 2 * 3 * 64;
#pragma unroll
  for (int k = 0; k < 3; ++k)
    out[(size_t)(ch * 3 + k) * 64 + lane] = __builtin_bit_cast(uint4, s[k]);
}

// ---------------------------------------------------------------------------
// tile geometry.  A workgroup owns a tile of kTR x 16 gradient rows (64 or
// 32) by one column group of kTW * kCPW 32-column chunks; each wave takes
// kCPW chunks of the group for all the tile's rows, so every operand-pack
// load feeds kTR 16-row MFMA tiles.  A row's c = g U is split over the column groups: each
// tile stores its partial (summed over its waves through LDS), and the next
// pass sums the partials of a row block in column-group order.
//
// Memory-wait discipline: a wave issues all loads of its chunks together
// (unconditionally inside a wave-uniform branch), and stores come last, so
// the compiler waits for exactly the operands in use; with a store in flight
// every wait for a load would become a wait for all memory operations.
//
// Partial and final row coefficients are kept in "fragment" order:
// [row block][rt * 8 + k][lane] holds, for the lane's row 16 rt + lane % 16,
// rank rank_of(k, lane / 16) -- exactly the eight values a lane feeds to the
// second product, so they are read and written coalesced.
// ---------------------------------------------------------------------------
constexpr int kTW = 8;                    // waves per tile workgroup
constexpr int kTileThreads = 64 * kTW;
constexpr int kTR = GIFT_TILE_RT;         // 16-row MFMA tiles per workgroup
constexpr int kTileRows = 16 * kTR;
constexpr int kFrag = kTR * 8 * 64;       // floats of one row block's coefficients
constexpr int kReduceThreads = kTR * 64;  // one thread per lane of each 16-row tile
// the waves' partial c are summed through LDS in kHalves passes of kPerHalf
// 16-row tiles (kRedRows floats per lane and wave)
constexpr int kHalves = kTR >= 2 ? 2 : 1;
constexpr int kPerHalf = kTR / kHalves;
constexpr int kRedRows = kPerHalf * 8;

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// f(integral_constant<int, n>) for the wave-uniform n, 1 <= n <= kMax;
// nothing for n < 1
template <int kMax, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (kMax > 0) {
    if (n >= kMax) f(std::integral_constant<int, kMax>{});
    else with_count<kMax - 1>(n, f);
  }
}

struct Tile {
  int row[kTR];      // this lane's gradient row in each 16-row tile (clamped)
  bool ok[kTR];      // row < d_out
  int64_t rb;        // row block
  int cg;            // column group
  int c0;            // first chunk of this wave
  int nmine;         // chunks of this wave (0..kCPW, wave-uniform)
  int lane, wave, r16, g;
};

template <int kCPW>
__device__ __forceinline__ Tile tile_ctx(const LayerDev& L, int tile) {
  Tile x;
  x.lane = threadIdx.x & 63;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  x.r16 = x.lane & 15;
  x.g = x.lane >> 4;
  // Workgroups are handed to the kXcd XCDs in turn.  The tiles of one row
  // block are numbered kXcd apart (within groups of kXcd row blocks), so they
  // all run on one XCD, close together in time, and read the row block's
  // shared data (c' in operand form) through one L2.  The last, shorter
  // group of a layer spaces its tiles by its own row-block count.
  const int span = kXcd * L.ngrp;
  const int sg = tile / span, w = tile - sg * span;
  const int rb_left = (int)L.n_rb - sg * kXcd;
  const int nr = rb_left < kXcd ? rb_left : kXcd;
  x.rb = (int64_t)sg * kXcd + w % nr;
  x.cg = w / nr;
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt) {
    const int64_t r = x.rb * kTileRows + 16 * rt + x.r16;
    x.ok[rt] = r < L.d_out;
    x.row[rt] = (int)(x.ok[rt] ? r : L.d_out - 1);
  }
  const int nch = (int)(L.d_in / kChunk);
  x.c0 = (x.cg * kTW + x.wave) * kCPW;
  const int left = nch - x.c0;
  x.nmine = left <= 0 ? 0 : (left < kCPW ? left : kCPW);
  return x;
}

// E4M3 codes of a whole tile are staged in LDS and stored as 16-byte pieces
// of whole row segments (up to 256 or 512 bytes per row): a wave's own stores
// would write 32 bytes per row and instruction, a quarter of a cache line.
// One 32-bit word holds four codes; the row stride (8 words per chunk plus 4)
// puts the 64 lanes of a write on distinct banks.
template <int kCPW>
struct CodeTile {
  static constexpr int kStride = kTW * kCPW * 8 + 4;
  uint32_t w[kTileRows][kStride];
};

// the four codes of chunk j, 16-row tile rt, half t of this lane
template <int kCPW>
__device__ __forceinline__ void put_codes(CodeTile<kCPW>& ct, const Tile& x, int j, int rt, int t,
                                          uint32_t c) {
  ct.w[16 * rt + x.r16][8 * (x.wave * kCPW + j) + 4 * t + x.g] = c;
}

// after a workgroup barrier: every row of the tile inside the layer, every
// chunk inside d_in
template <int kCPW>
__device__ __forceinline__ void store_code_tile(const LayerDev& L, const Tile& x,
                                                const CodeTile<kCPW>& ct) {
  constexpr int kQ = kTW * kCPW * 2;  // 16-byte pieces per row
  constexpr int kN = kTileRows * kQ;  // pieces per tile
  const int nch = (int)(L.d_in / kChunk), cfirst = x.cg * kTW * kCPW;
  const int nvalid = nch - cfirst < kTW * kCPW ? nch - cfirst : kTW * kCPW;
#pragma unroll
  for (int h = 0; h < (kN + kTileThreads - 1) / kTileThreads; ++h) {
    const int e = threadIdx.x + h * kTileThreads, r = e / kQ, qd = e % kQ;
    const int64_t row = x.rb * kTileRows + r;
    if (e < kN && row < L.d_out && (qd >> 1) < nvalid)
      st_q16(L.q + row * L.d_in + kChunk * cfirst + 16 * qd,
             *reinterpret_cast<const uint4*>(&ct.w[r][4 * qd]));
  }
}

// The reverse for the dequantize side: the tile's codes are loaded as 16-byte
// pieces of whole row segments (zero outside the layer), put in LDS in the
// same layout, and each lane then takes its words.
template <int kCPW>
struct CodePieces {
  static constexpr int kQ = kTW * kCPW * 2;                 // 16-byte pieces per row
  static constexpr int kPieces = kTileRows * kQ;             // per tile
  static constexpr int kN = (kPieces + kTileThreads - 1) / kTileThreads;  // per thread
  uint4 v[kN];
};

template <int kCPW>
__device__ __forceinline__ void load_code_pieces(const LayerDev& L, const Tile& x,
                                                 CodePieces<kCPW>& pc) {
  constexpr int kQ = CodePieces<kCPW>::kQ;
  const int nch = (int)(L.d_in / kChunk), cfirst = x.cg * kTW * kCPW;
  const int nvalid = nch - cfirst < kTW * kCPW ? nch - cfirst : kTW * kCPW;
#pragma unroll
  for (int h = 0; h < CodePieces<kCPW>::kN; ++h) {
    const int e = threadIdx.x + h * kTileThreads, r = e / kQ, qd = e % kQ;
    const int64_t row = x.rb * kTileRows + r;
    const bool in = e < CodePieces<kCPW>::kPieces && row < L.d_out && (qd >> 1) < nvalid;
    pc.v[h] = in ? ld_q16(L.q + row * L.d_in + kChunk * cfirst + 16 * qd)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int kCPW>
__device__ __forceinline__ void put_code_pieces(CodeTile<kCPW>& ct, const CodePieces<kCPW>& pc) {
  constexpr int kQ = CodePieces<kCPW>::kQ;
#pragma unroll
  for (int h = 0; h < CodePieces<kCPW>::kN; ++h) {
    const int e = threadIdx.x + h * kTileThreads;
    if (e < CodePieces<kCPW>::kPieces)
      *reinterpret_cast<uint4*>(&ct.w[e / kQ][4 * (e % kQ)]) = pc.v[h];
  }
}

template <int kCPW>
__device__ __forceinline__ uint32_t get_codes(const CodeTile<kCPW>& ct, const Tile& x, int j,
                                              int rt, int t) {
  return ct.w[16 * rt + x.r16][8 * (x.wave * kCPW + j) + 4 * t + x.g];
}

// The same for MXFP4: per row and chunk 16 bytes of E2M1 codes (16 bits per
// lane and half) and one E8M0 scale byte.
template <int kCPW>
struct MxTile {
  static constexpr int kChunks = kTW * kCPW;
  static constexpr int kStride = kChunks * 8 + 8;  // 16-bit units per row of codes
  uint16_t c[kTileRows][kStride];
  uint8_t s[kTileRows][kChunks + 8];
};

template <int kCPW>
__device__ __forceinline__ int mx_valid(const LayerDev& L, const Tile& x) {
  const int nch = (int)(L.d_in / kChunk), cfirst = x.cg * kTW * kCPW;
  return nch - cfirst < kTW * kCPW ? nch - cfirst : kTW * kCPW;
}

template <int kCPW>
__device__ __forceinline__ void store_mx_tile(const LayerDev& L, const Tile& x,
                                              const MxTile<kCPW>& mt) {
  constexpr int kQ = MxTile<kCPW>::kChunks;  // 16-byte pieces (one chunk each) per row
  const int cfirst = x.cg * kTW * kCPW, nvalid = mx_valid<kCPW>(L, x);
  const int64_t nblk = L.d_in / kMxBlock;
  for (int e = threadIdx.x; e < kTileRows * kQ; e += kTileThreads) {
    const int r = e / kQ, qd = e % kQ;
    const int64_t row = x.rb * kTileRows + r;
    if (row < L.d_out && qd < nvalid) {
      st_q16(L.q + row * (L.d_in / 2) + 16 * (cfirst + qd),
             *reinterpret_cast<const uint4*>(&mt.c[r][8 * qd]));
      reinterpret_cast<uint8_t*>(L.inv)[row * nblk + cfirst + qd] = mt.s[r][qd];
    }
  }
}

template <int kCPW>
__device__ __forceinline__ void load_mx_tile(const LayerDev& L, const Tile& x, MxTile<kCPW>& mt) {
  constexpr int kQ = MxTile<kCPW>::kChunks;
  constexpr int kN = (kTileRows * kQ + kTileThreads - 1) / kTileThreads;
  const int cfirst = x.cg * kTW * kCPW, nvalid = mx_valid<kCPW>(L, x);
  const int64_t nblk = L.d_in / kMxBlock;
  uint4 v[kN];
  uint32_t sc[kN];
#pragma unroll
  for (int h = 0; h < kN; ++h) {
    const int e = threadIdx.x + h * kTileThreads, r = e / kQ, qd = e % kQ;
    const int64_t row = x.rb * kTileRows + r;
    const bool in = e < kTileRows * kQ && row < L.d_out && qd < nvalid;
    v[h] = in ? ld_q16(L.q + row * (L.d_in / 2) + 16 * (cfirst + qd))
              : make_uint4(0u, 0u, 0u, 0u);
    sc[h] = in ? reinterpret_cast<const uint8_t*>(L.inv)[row * nblk + cfirst + qd] : 127u;
  }
#pragma unroll
  for (int h = 0; h < kN; ++h) {
    const int e = threadIdx.x + h * kTileThreads;
    if (e < kTileRows * kQ) {
      *reinterpret_cast<uint4*>(&mt.c[e / kQ][8 * (e % kQ)]) = v[h];
      mt.s[e / kQ][e % kQ] = (uint8_t)sc[h];
    }
  }
}

template <int kCPW>
__device__ __forceinline__ void get_mx(const MxTile<kCPW>& mt, const Tile& x, int j, int rt,
                                       uint32_t (&v)[2], uint32_t& code) {
  const int r = 16 * rt + x.r16, k = x.wave * kCPW + j;
  v[0] = mt.c[r][8 * k + x.g];
  v[1] = mt.c[r][8 * k + 4 + x.g];
  code = mt.s[r][k];
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

// first-form packs of rank block b, and (p2_of) its second-form packs
__device__ __forceinline__ const uint4* p1_of(const LayerDev& L, int b = 0) {
  return L.P + (size_t)b * (L.d_in / kChunk) * 2 * 2 * 3 * 64;
}
__device__ __forceinline__ const uint4* p2_of(const LayerDev& L, int b = 0) {
  return p1_of(L, b) + (size_t)(L.d_in / kChunk) * 2 * 3 * 64;
}

// rank index of element k (0..7) of a lane's c vector
__device__ __forceinline__ int rank_of(int k, int g) { return 16 * (k >> 2) + 4 * g + (k & 3); }

// gradient values of one chunk for this lane and 16-row tile: columns
// 32c + 4g .. +3 (t = 0) and 32c + 16 + 4g .. +3 (t = 1) of its row
__device__ __forceinline__ void load_gc(const LayerDev& L, int64_t row, int g, int c,
                                        float4 (&v)[2]) {
  const float* p = L.G + row * L.d_in + kChunk * c + 4 * g;
  v[0] = ld_g(p);
  v[1] = ld_g(p + 16);
}

__device__ __forceinline__ void load_qc(const LayerDev& L, int64_t row, int g, int c,
                                        uint32_t (&v)[2]) {
  const uint8_t* p = L.q + row * L.d_in + kChunk * c + 4 * g;
  v[0] = ld_q4(p);
  v[1] = ld_q4(p + 16);
}

// first product on MXFP4 values (code value * 2^e is exact in bf16)
__device__ __forceinline__ void cpart_mx(const bf16x8 (&a)[2][3], const uint32_t (&qv)[2],
                                         uint32_t code, f32x4 (&acc)[2]) {
  const float4 lo = mx_decode4(qv[0], code), hi = mx_decode4(qv[1], code);
  const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  bf16x8 bq;
#pragma unroll
  for (int i = 0; i < 8; ++i) bq[i] = (__bf16)v[i];
#pragma unroll
  for (int h = 0; h < 2; ++h) acc[h] = mfma3x1(a[h], bq, acc[h]);
}

__device__ __forceinline__ void decode8(uint32_t lo, uint32_t hi, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode(lo, i);
    v[4 + i] = e4m3_decode(hi, i);
  }
}

__device__ __forceinline__ uint32_t amax4(uint32_t m, const float4& v) {
  m = max(m, abs_bits(v.x));
  m = max(m, abs_bits(v.y));
  m = max(m, abs_bits(v.z));
  return max(m, abs_bits(v.w));
}

// first product, one chunk and 16-row tile: acc[h] += (U^T)_h (g split three ways)
__device__ __forceinline__ void cpart_g(const bf16x8 (&a)[2][3], const float4 (&gv)[2],
                                        f32x4 (&acc)[2]) {
  const float v[8] = {gv[0].x, gv[0].y, gv[0].z, gv[0].w, gv[1].x, gv[1].y, gv[1].z, gv[1].w};
  bf16x8 sp[3];
  split3(v, sp);
  const bf16x8(*pa2[2])[3] = {&a[0], &a[1]};
  const bf16x8(*pb2[2])[3] = {&sp, &sp};
  mfma3x3_n<2>(pa2, pb2, acc);
}

// first product on codes (exact in bf16): acc[h] += (U^T)_h decode(q)
__device__ __forceinline__ void cpart_q(const bf16x8 (&a)[2][3], const uint32_t (&qv)[2],
                                        f32x4 (&acc)[2]) {
  float v[8];
  decode8(qv[0], qv[1], v);
  bf16x8 bq;
#pragma unroll
  for (int i = 0; i < 8; ++i) bq[i] = (__bf16)v[i];
#pragma unroll
  for (int h = 0; h < 2; ++h) acc[h] = mfma3x1(a[h], bq, acc[h]);
}

// second product, one chunk and 16-row tile: corr[t] = (c' U^T) for the
// lane's 2 x 4 columns
__device__ __forceinline__ void correction(const bf16x8 (&a)[2][3], const bf16x8 (&cb)[3],
                                           f32x4 (&corr)[2]) {
  corr[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  corr[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8(*pa2[2])[3] = {&a[0], &a[1]};
  const bf16x8(*pb2[2])[3] = {&cb, &cb};
  mfma3x3_n<2>(pa2, pb2, corr);
}

// Sum the waves' partial c (acc of every wave) in wave order through LDS and
// store the tile's partial for its column group in fragment order, in
// kHalves passes of kPerHalf row tiles.  Contains workgroup barriers.
template <int kRB>
__device__ __forceinline__ void store_partial(const LayerDev& L, const Tile& x,
                                              const f32x4 (&acc)[kTR][2],
                                              float (*red)[kRedRows][64], int b) {
  constexpr int kN = kFrag / kHalves;  // floats per pass
  float* out = L.cbuf + (((int64_t)x.cg * L.n_rb + x.rb) * kRB + b) * kFrag;
#pragma unroll
  for (int half = 0; half < kHalves; ++half) {
    if (half) __syncthreads();  // the first half has been read
#pragma unroll
    for (int r = 0; r < kPerHalf; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[x.wave][r * 8 + 4 * h + i][x.lane] = acc[half * kPerHalf + r][h][i];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < (kN + kTileThreads - 1) / kTileThreads; ++e) {
      const int p = e * kTileThreads + threadIdx.x;
      if (p < kN) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kTW; ++w) s += red[w][p >> 6][p & 63];
        out[half * kN + p] = s;
      }
    }
  }
}

// The row block's c' operand of the second product in LDS, split three
// ways: [rt][split][lane] 16-byte groups of 8 bf16 (kCOp uint4 per row block
// and rank block).  In the workspace c' is kept in fp32, [rt][half][lane]
// float4s (kCF per row block and rank block, rank block b of row block rb at
// (rb * kRB + b) * kCF): two thirds of the bytes of the split form, which
// every tile of the row block reads.  stage_c splits it as it fills LDS (the
// same split3 as where c' is formed, so the operand is the same bits).
// Contains a workgroup barrier.
constexpr int kCOp = kTR * 3 * 64;
constexpr int kCF = kTR * 2 * 64;

// c' of one (rank block, 16-row tile, lane) into the workspace
__device__ __forceinline__ void put_cfin(const LayerDev& L, int64_t rbb, int rt, int lane,
                                         const float (&cp)[8]) {
  float4* out = reinterpret_cast<float4*>(L.cfin) + rbb * kCF + (rt * 2) * 64 + lane;
  out[0] = make_float4(cp[0], cp[1], cp[2], cp[3]);
  out[64] = make_float4(cp[4], cp[5], cp[6], cp[7]);
}

template <int kRB = 1>
__device__ __forceinline__ void stage_c(const LayerDev& L, const Tile& x, uint4* lds) {
  const float4* src = reinterpret_cast<const float4*>(L.cfin) + x.rb * kCF * kRB;
  for (int e = threadIdx.x; e < kTR * 64 * kRB; e += kTileThreads) {
    const int b = e / (kTR * 64), rt = (e / 64) % kTR, lane = e % 64;
    const float4 lo = src[b * kCF + (rt * 2) * 64 + lane];
    const float4 hi = src[b * kCF + (rt * 2 + 1) * 64 + lane];
    const float cp[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    bf16x8 cb[3];
    split3(cp, cb);
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) lds[b * kCOp + (rt * 3 + sp) * 64 + lane] = __builtin_bit_cast(uint4, cb[sp]);
  }
  __syncthreads();
}

// the lane's operand of the second product for 16-row tile rt
__device__ __forceinline__ void c_operand(const uint4* lds, int rt, int lane, bf16x8 (&cb)[3]) {
#pragma unroll
  for (int s = 0; s < 3; ++s) cb[s] = as_bf16x8(lds[(rt * 3 + s) * 64 + lane]);
}

// second product over the kRB rank blocks, one chunk and 16-row tile:
// corr[t] = sum over blocks b in order of (c'_b U_b^T) for the lane's 2 x 4
// columns (c' of block b in lds at b * kCOp)
template <int kRB>
__device__ __forceinline__ void correction_rb(const bf16x8 (&a)[kRB][2][3], const uint4* lds,
                                              int rt, int lane, f32x4 (&corr)[2]) {
  corr[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  corr[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    bf16x8 cb[3];
    c_operand(lds + b * kCOp, rt, lane, cb);
    const bf16x8(*pa2[2])[3] = {&a[b][0], &a[b][1]};
    const bf16x8(*pb2[2])[3] = {&cb, &cb};
    mfma3x3_n<2>(pa2, pb2, corr);
  }
}

template <int kRB>
__device__ __forceinline__ void load_a_rb(const LayerDev& L, bool second, int c, int lane,
                                          uint4 (&a)[kRB][2][3]) {
#pragma unroll
  for (int b = 0; b < kRB; ++b) load_a(second ? p2_of(L, b) : p1_of(L, b), c, lane, a[b]);
}

template <int kRB>
__device__ __forceinline__ void as_ops_rb(const uint4 (&u)[kRB][2][3], bf16x8 (&a)[kRB][2][3]) {
#pragma unroll
  for (int b = 0; b < kRB; ++b) as_ops(u[b], a[b]);
}

// ---------------------------------------------------------------------------
// first product of a tile: partial c over the column group (whiten: of G;
// dequantize: of the codes, each chunk scaled by its inverse scale).
// ---------------------------------------------------------------------------
template <int kCPW, bool kCodes, int kFmt, int kRB>
__global__ __launch_bounds__(kTileThreads) void k_tile_cpart(GroupDev gd) {
  constexpr bool kB128 = kFmt == GIFT_SCALE_BLOCK128, kMX = kFmt == GIFT_SCALE_MXFP4;
  // a local copy: the descriptor's fields stay in scalar registers
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kCPW>(L, tile);
  __shared__ float red[kTW][kRedRows][64];
  f32x4 acc[kRB][kTR][2];
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt) acc[b][rt][0] = acc[b][rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t nseg = L.d_in / kBlock;
  constexpr bool kStaged = kCodes && !kMX;  // E4M3 codes come through LDS
  __shared__ __align__(16) uint32_t ctw[kStaged ? sizeof(CodeTile<kCPW>) / 4
                          : kMX ? (sizeof(MxTile<kCPW>) + 3) / 4 : 1];
  CodeTile<kCPW>& ct = *reinterpret_cast<CodeTile<kCPW>*>(ctw);
  MxTile<kCPW>& mt = *reinterpret_cast<MxTile<kCPW>*>(ctw);
  if constexpr (kStaged) {
    CodePieces<kCPW> pcs;
    load_code_pieces(L, x, pcs);
    put_code_pieces(ct, pcs);
    __syncthreads();
  } else if constexpr (kMX) {
    load_mx_tile(L, x, mt);
    __syncthreads();
  }
  with_count<kCPW>(x.nmine, [&](auto N) {
    constexpr int n = decltype(N)::value;
    uint4 pa[n][kRB][2][3];
    float4 gv[kCodes ? 1 : n][kTR][2];
    uint32_t qv[kCodes ? n : 1][kTR][2];
    float sc[kB128 ? n : 1][kTR];
    uint32_t mc[kMX ? n : 1][kTR];
    static_for<n>([&](auto J) {
      constexpr int j = decltype(J)::value;
      load_a_rb<kRB>(L, false, x.c0 + j, x.lane, pa[j]);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        if constexpr (kMX) get_mx(mt, x, j, rt, qv[j][rt], mc[j][rt]);
        else if constexpr (kCodes)
#pragma unroll
          for (int t = 0; t < 2; ++t) qv[j][rt][t] = get_codes(ct, x, j, rt, t);
        else load_gc(L, x.row[rt], x.g, x.c0 + j, gv[j][rt]);
        if constexpr (kB128) sc[j][rt] = L.inv[x.row[rt] * nseg + ((x.c0 + j) >> 2)];
      }
    });
    static_for<n>([&](auto J) {
      constexpr int j = decltype(J)::value;
#pragma unroll
      for (int b = 0; b < kRB; ++b) {
        bf16x8 a[2][3];
        as_ops(pa[j][b], a);
#pragma unroll
        for (int rt = 0; rt < kTR; ++rt) {
          if constexpr (kMX) {
            cpart_mx(a, qv[j][rt], mc[j][rt], acc[b][rt]);
          } else if constexpr (kCodes) {
            if constexpr (kB128) {
              f32x4 t[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
              cpart_q(a, qv[j][rt], t);
#pragma unroll
              for (int h = 0; h < 2; ++h) acc[b][rt][h] += t[h] * sc[j][rt];
            } else {
              cpart_q(a, qv[j][rt], acc[b][rt]);
            }
          } else {
            cpart_g(a, gv[j][rt], acc[b][rt]);
          }
        }
      }
    });
  });
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    if (b) __syncthreads();  // the previous block's partial has been read from LDS
    store_partial<kRB>(L, x, acc[b], red, b);
  }
}

// ---------------------------------------------------------------------------
// c' of every row block: the column-group partials summed in group order,
// times the lane's rank coefficient (whiten: D_w; dequantize: D_u, and the
// tensor's inverse scale for per-tensor scaling).  One workgroup per row block.
// ---------------------------------------------------------------------------
template <bool kDequant, bool kBlockScale, int kRB>
__device__ __forceinline__ void reduce_row_block(const LayerDev& L, int64_t rb, int tid, int b) {
  const int rt = tid >> 6, lane = tid & 63;  // one lane of one 16-row tile
  // D_w at 8, D_u after the factor's 32 kRB D_w entries; block b's ranks 32 b ..
  const float* dk = L.coef + 8 + (kDequant ? kRank * kRB : 0) + kRank * b;
  const float extra = (kDequant && !kBlockScale) ? L.inv[0] : 1.f;
  float d8[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) d8[k] = dk[rank_of(k, lane >> 4)] * extra;
  // partials in group order; eight groups' loads in flight at a time
  constexpr int kB = 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* base = L.cbuf + (rb * kRB + b) * kFrag + rt * 8 * 64 + lane;
  const int64_t stride = L.n_rb * kRB * kFrag;
  for (int c0 = 0; c0 < L.ngrp; c0 += kB) {
    float v[kB][8];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int cg = c0 + b < L.ngrp ? c0 + b : L.ngrp - 1;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[b][k] = base[cg * stride + k * 64];
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (c0 + b < L.ngrp)
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] += v[b][k];
  }
  float cp[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) cp[k] = s[k] * d8[k];
  put_cfin(L, rb * kRB + b, rt, lane, cp);
}

template <bool kDequant, bool kBlockScale, int kRB>
__global__ __launch_bounds__(kReduceThreads) void k_tile_reduce(GroupDev gd) {
  const LayerDev L = gd.L[find_layer_rb(gd, blockIdx.x)];
#pragma unroll
  for (int b = 0; b < kRB; ++b)
    reduce_row_block<kDequant, kBlockScale, kRB>(L, blockIdx.x - L.rb_begin, threadIdx.x, b);
}

// ---------------------------------------------------------------------------
// whiten pass 2, by scaling mode kFmt:
//   GIFT_SCALE_TENSOR: W of the tile, its amax to the layer's partials.
//   GIFT_SCALE_BLOCK128 (the last pass): W, the segment amax (the 4 chunks
//     of a segment are held by 4 / kCPW waves), codes and inverse scales.
//   GIFT_SCALE_MXFP4 (the last pass): W, the 32-element block amax (one
//     chunk of one row: four lanes of one wave), E8M0 scales, E2M1 codes.
//   The last two optionally write W.
// ---------------------------------------------------------------------------
// scaling-mode value of k_tile_whiten for un-whitening an fp32 tensor:
// G^ = beta S + c'(D_u) U^T, written to G_hat
constexpr int kFmtUnwhiten = 3;

template <int kCPW, int kFmt, bool kWriteW, int kRB>
__global__ __launch_bounds__(kTileThreads) void k_tile_whiten(GroupDev gd) {
  constexpr bool kBlock128 = kFmt == GIFT_SCALE_BLOCK128;
  constexpr int kWPS = 4 / kCPW;  // waves per segment (block scaling)
  static_assert(!kBlock128 || kCPW <= 4, "a segment spans whole waves");
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kCPW>(L, tile);
  __shared__ uint4 cs[kCOp * kRB];
  __shared__ uint32_t mx[kBlock128 ? kTW * kTR * 64 : kTW];
  __shared__ __align__(16) uint32_t ctw[kBlock128 ? sizeof(CodeTile<kCPW>) / 4
                          : kFmt == GIFT_SCALE_MXFP4 ? (sizeof(MxTile<kCPW>) + 3) / 4 : 1];
  CodeTile<kCPW>* ct = reinterpret_cast<CodeTile<kCPW>*>(ctw);
  const float alpha = L.coef[kFmt == kFmtUnwhiten ? GIFT_COEF_BETA : GIFT_COEF_ALPHA];
  // this wave's operands and gradient in flight while c' is staged
  uint4 pa[kCPW][kRB][2][3];
  float4 gv[kCPW][kTR][2];
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
      load_a_rb<kRB>(L, true, x.c0 + j, x.lane, pa[j]);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) load_gc(L, x.row[rt], x.g, x.c0 + j, gv[j][rt]);
    });
  });
  stage_c<kRB>(L, x, cs);
  float4 w[kCPW][kTR][2];
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
      bf16x8 a[kRB][2][3];
      as_ops_rb<kRB>(pa[j], a);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        f32x4 corr[2];
        correction_rb<kRB>(a, cs, rt, x.lane, corr);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float4 gg = gv[j][rt][t];
          w[j][rt][t] = make_float4(fmaf(alpha, gg.x, corr[t][0]), fmaf(alpha, gg.y, corr[t][1]),
                                    fmaf(alpha, gg.z, corr[t][2]), fmaf(alpha, gg.w, corr[t][3]));
        }
      }
    });
  });
  if constexpr (kFmt == GIFT_SCALE_TENSOR) {
    uint32_t m = 0u;
    with_count<kCPW>(x.nmine, [&](auto N) {
      static_for<decltype(N)::value>([&](auto J) {
#pragma unroll
        for (int rt = 0; rt < kTR; ++rt)
          if (x.ok[rt]) m = amax4(amax4(m, w[J.value][rt][0]), w[J.value][rt][1]);
      });
    });
    m = block_max_u32<kTileThreads>(m, mx);
    if (threadIdx.x == 0) L.part[tile] = m;
  } else if constexpr (kFmt == kFmtUnwhiten) {
    if (x.nmine == 0) return;
    with_count<kCPW>(x.nmine, [&](auto N) {
      static_for<decltype(N)::value>([&](auto J) {
        constexpr int j = decltype(J)::value;
#pragma unroll
        for (int rt = 0; rt < kTR; ++rt) {
          if (!x.ok[rt]) continue;
#pragma unroll
          for (int t = 0; t < 2; ++t)
            st_f4(L.Ghat + x.row[rt] * L.d_in + kChunk * (x.c0 + j) + 16 * t + 4 * x.g,
                  w[j][rt][t]);
        }
      });
    });
  } else if constexpr (kFmt == GIFT_SCALE_MXFP4) {
    MxTile<kCPW>& mt = *reinterpret_cast<MxTile<kCPW>*>(ctw);
    with_count<kCPW>(x.nmine, [&](auto N) {
      static_for<decltype(N)::value>([&](auto J) {
        constexpr int j = decltype(J)::value;
#pragma unroll
        for (int rt = 0; rt < kTR; ++rt) {
          uint32_t m = amax4(amax4(0u, w[j][rt][0]), w[j][rt][1]);
          m = max(m, (uint32_t)__shfl_xor(m, 16, 64));
          m = max(m, (uint32_t)__shfl_xor(m, 32, 64));
          uint32_t fl = 0u;
          const uint32_t code = mx_scale_code(m, fl);
          const float s = mx_scale_operand(code);
          const bool nonfinite = code == kMxScaleNaN;
          const int r = 16 * rt + x.r16, k = x.wave * kCPW + j;
          mt.c[r][8 * k + x.g] = (uint16_t)mx_encode4(w[j][rt][0], s, nonfinite);
          mt.c[r][8 * k + 4 + x.g] = (uint16_t)mx_encode4(w[j][rt][1], s, nonfinite);
          if (x.g == 0) mt.s[r][k] = (uint8_t)code;
          if (!x.ok[rt]) continue;
          if (x.g == 0 && gd.flags && fl) atomicOr(gd.flags, fl);
          if (kWriteW && L.Wout) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
              *reinterpret_cast<float4*>(L.Wout + x.row[rt] * L.d_in + kChunk * (x.c0 + j) +
                                         16 * t + 4 * x.g) = w[j][rt][t];
          }
        }
      });
    });
    __syncthreads();
    store_mx_tile(L, x, mt);
  } else {
    // per-segment amax: lane max over its chunks of the segment, then over
    // the lanes of the same row (xor 16, 32), then over the segment's waves
    uint32_t (*sm)[kTR][64] = reinterpret_cast<uint32_t (*)[kTR][64]>(mx);
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt) {
      uint32_t m = 0u;
      with_count<kCPW>(x.nmine, [&](auto N) {
        static_for<decltype(N)::value>([&](auto J) {
          m = amax4(amax4(m, w[J.value][rt][0]), w[J.value][rt][1]);
        });
      });
      m = max(m, (uint32_t)__shfl_xor(m, 16, 64));
      m = max(m, (uint32_t)__shfl_xor(m, 32, 64));
      sm[x.wave][rt][x.lane] = m;
    }
    __syncthreads();
    const int w0 = x.wave - x.wave % kWPS;
    const int seg = x.c0 / 4;
    const int64_t nseg = L.d_in / kBlock;
    if (x.nmine) {  // wave-uniform
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        uint32_t m = 0u;
#pragma unroll
        for (int v = 0; v < kWPS; ++v) m = max(m, sm[w0 + v][rt][x.lane]);
        const Scale sc = scale_from_amax_bits(m);
        if (x.ok[rt] && x.g == 0 && x.wave == w0) {
          L.inv[x.row[rt] * nseg + seg] = sc.inv;
          if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
        }
        with_count<kCPW>(x.nmine, [&](auto N) {
          static_for<decltype(N)::value>([&](auto J) {
            constexpr int j = decltype(J)::value;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const float4 v = w[j][rt][t];
              put_codes(*ct, x, j, rt, t,
                        e4m3_encode4_scaled(v, sc.scale, sc.flags & GIFT_FLAG_NONFINITE));
              if (kWriteW && L.Wout && x.ok[rt])
                *reinterpret_cast<float4*>(L.Wout + x.row[rt] * L.d_in + kChunk * (x.c0 + j) +
                                           16 * t + 4 * x.g) = v;
            }
          });
        });
      }
    }
    __syncthreads();
    store_code_tile(L, x, *ct);
  }
}

// ---------------------------------------------------------------------------
// per-tensor whiten pass 3: layer amax from the tile partials (or from
// k_amax_final for very tall layers), W again from the row block's c', codes.
// ---------------------------------------------------------------------------
template <int kCPW, bool kWriteW, int kRB>
__global__ __launch_bounds__(kTileThreads) void k_tile_quant(GroupDev gd) {
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kCPW>(L, tile);
  __shared__ uint4 cs[kCOp * kRB];
  __shared__ uint32_t mx[kTW];
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  uint4 pa[kCPW][kRB][2][3];
  float4 gv[kCPW][kTR][2];
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
      load_a_rb<kRB>(L, true, x.c0 + j, x.lane, pa[j]);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) load_gc(L, x.row[rt], x.g, x.c0 + j, gv[j][rt]);
    });
  });
  uint32_t m = 0u;
  if (L.n_part > kPartialLimit) {
    m = *L.amax;
  } else {
    for (int i = threadIdx.x; i < L.n_part; i += kTileThreads) m = max(m, L.part[i]);
    m = block_max_u32<kTileThreads>(m, mx);
  }
  const Scale sc = scale_from_amax_bits(m);
  if (tile == 0 && threadIdx.x == 0) {
    L.inv[0] = sc.inv;
    if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
  }
  stage_c<kRB>(L, x, cs);
  __shared__ __align__(16) CodeTile<kCPW> ct;
  const bool nonfinite = (sc.flags & GIFT_FLAG_NONFINITE) != 0;
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
      bf16x8 a[kRB][2][3];
      as_ops_rb<kRB>(pa[j], a);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        f32x4 corr[2];
        correction_rb<kRB>(a, cs, rt, x.lane, corr);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float4 gg = gv[j][rt][t];
          const float4 v = make_float4(fmaf(alpha, gg.x, corr[t][0]), fmaf(alpha, gg.y, corr[t][1]),
                                       fmaf(alpha, gg.z, corr[t][2]), fmaf(alpha, gg.w, corr[t][3]));
          put_codes(ct, x, j, rt, t, e4m3_encode4_scaled(v, sc.scale, nonfinite));
          if (kWriteW && L.Wout && x.ok[rt])
            *reinterpret_cast<float4*>(L.Wout + x.row[rt] * L.d_in + kChunk * (x.c0 + j) + 16 * t +
                                       4 * x.g) = v;
        }
      }
    });
  });
  __syncthreads();
  store_code_tile(L, x, ct);
}

// ---------------------------------------------------------------------------
// block-diagonal factor (block-A-b, b = 32 or 64): W[:, block i] =
// G[:, block i] S_i and G^[:, block i] = W^[:, block i] S_i^-1 on MFMA with
// the bf16x3 split.  A wave owns one block (b/32 chunks) of the tile's 64
// rows, so the tile kernels' geometry holds with b/32 chunks per wave.  The
// G values a lane loads (load_gc: K-permuted) are the B operand as they
// are; the operand packs hold, for M = S (m = 0) or S^-1 (m = 1), output
// chunk oc and K chunk kc of block i, element e of lane l (r16 = l % 16,
// g = l / 16) = M_i[32 kc + perm(e)][32 oc + 16 h + r16] at uint4 index
// (((((m nblk + i) kb + oc) kb + kc) 2 + h) 3 + split) 64 + l, kb = b / 32.
// U of a block factor is d_in x 2b: row b i + a = [row a of S_i, row a of S_i^-1].
// ---------------------------------------------------------------------------
size_t blk_pack_bytes(int64_t d_in, int b) {
  const int64_t kb = b / kChunk;
  return (size_t)(2 * (d_in / b) * kb * kb * 2 * 3 * 64) * sizeof(uint4);
}

__global__ __launch_bounds__(kThreads) void k_pack_blk(PackGroup pg, int b) {
  const PackDev& F = pg.f[blockIdx.y];
  const int kb = b / kChunk;
  const int64_t nblk = F.d_in / b;
  const int64_t lanes = 2 * nblk * kb * kb * 2 * 64;
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= lanes) return;
  const int lane = (int)(e & 63);
  const int64_t q = e >> 6;  // (((m nblk + i) kb + oc) kb + kc) 2 + h
  int64_t r = q;
  const int h = (int)(r & 1);
  r >>= 1;
  const int kc = (int)(r % kb);
  r /= kb;
  const int oc = (int)(r % kb);
  r /= kb;
  const int64_t i = r % nblk;
  const int m = (int)(r / nblk);
  const int r16 = lane & 15, g = lane >> 4;
  float v[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t row = b * i + kChunk * kc + perm8(t, g);
    v[t] = F.U[row * 2 * b + m * b + kChunk * oc + 16 * h + r16];
  }
  bf16x8 sp[3];
  split3(v, sp);
#pragma unroll
  for (int t = 0; t < 3; ++t) F.P[(size_t)(q * 3 + t) * 64 + lane] = __builtin_bit_cast(uint4, sp[t]);
}

template <int kb>
__device__ __forceinline__ void load_blk_packs(const uint4* P, int64_t nblk, int m, int64_t blk,
                                               int oc, int lane, uint4 (&a)[kb][2][3]) {
#pragma unroll
  for (int kc = 0; kc < kb; ++kc)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 3; ++t)
        a[kc][h][t] = P[(size_t)((((((m * nblk + blk) * kb + oc) * kb + kc) * 2 + h) * 3 + t) * 64) + lane];
}

// one output chunk of one 16-row tile: sum over the block's K chunks of
// (M packs) x (G chunk split three ways)
template <int kb>
__device__ __forceinline__ void blk_product(const uint4 (&pa)[kb][2][3], const float4 (*gv)[2],
                                            f32x4 (&out)[2]) {
  out[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  out[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < kb; ++kc) {
    bf16x8 a[2][3];
    as_ops(pa[kc], a);
    const float v[8] = {gv[kc][0].x, gv[kc][0].y, gv[kc][0].z, gv[kc][0].w,
                        gv[kc][1].x, gv[kc][1].y, gv[kc][1].z, gv[kc][1].w};
    bf16x8 sp[3];
    split3(v, sp);
    const bf16x8(*pa2[2])[3] = {&a[0], &a[1]};
    const bf16x8(*pb2[2])[3] = {&sp, &sp};
    mfma3x3_n<2>(pa2, pb2, out);
  }
}

// kMode 0: per-tensor amax pass (tile partial to L.part); 1: per-tensor
// quantize pass; 2: 1x128 block scaling (codes and segment scales)
template <int kB, int kMode, bool kWriteW>
__global__ __launch_bounds__(kTileThreads) void k_blk_whiten(GroupDev gd) {
  constexpr int kb = kB / kChunk;
  constexpr int kWPS = 4 / kb;  // waves per 128-column segment
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kb>(L, tile);
  __shared__ uint32_t mx[kMode == 2 ? kTW * kTR * 64 : kTW];
  __shared__ __align__(16) uint32_t ctw[kMode != 0 ? sizeof(CodeTile<kb>) / 4 : 1];
  CodeTile<kb>& ct = *reinterpret_cast<CodeTile<kb>*>(ctw);
  const int64_t nblk = L.d_in / kB, blk = x.c0 / kb;
  float4 w[kb][kTR][2];
  if (x.nmine) {  // wave-uniform: a wave has a whole block or nothing
    float4 gv[kTR][kb][2];
    uint4 pa[kb][2][3];
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt)
#pragma unroll
      for (int kc = 0; kc < kb; ++kc) load_gc(L, x.row[rt], x.g, x.c0 + kc, gv[rt][kc]);
    load_blk_packs<kb>(L.P, nblk, 0, blk, 0, x.lane, pa);
#pragma unroll
    for (int oc = 0; oc < kb; ++oc) {
      if (oc) load_blk_packs<kb>(L.P, nblk, 0, blk, oc, x.lane, pa);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        f32x4 out[2];
        blk_product<kb>(pa, gv[rt], out);
#pragma unroll
        for (int t = 0; t < 2; ++t) w[oc][rt][t] = make_float4(out[t][0], out[t][1], out[t][2], out[t][3]);
      }
    }
  }
  if constexpr (kMode == 0) {
    uint32_t m = 0u;
    if (x.nmine)
#pragma unroll
      for (int oc = 0; oc < kb; ++oc)
#pragma unroll
        for (int rt = 0; rt < kTR; ++rt)
          if (x.ok[rt]) m = amax4(amax4(m, w[oc][rt][0]), w[oc][rt][1]);
    m = block_max_u32<kTileThreads>(m, mx);
    if (threadIdx.x == 0) L.part[tile] = m;
  } else if constexpr (kMode == 1) {
    uint32_t m = 0u;
    if (L.n_part > kPartialLimit) {
      m = *L.amax;
    } else {
      for (int i = threadIdx.x; i < L.n_part; i += kTileThreads) m = max(m, L.part[i]);
      m = block_max_u32<kTileThreads>(m, mx);
    }
    const Scale sc = scale_from_amax_bits(m);
    if (tile == 0 && threadIdx.x == 0) {
      L.inv[0] = sc.inv;
      if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
    }
    const bool nonfinite = (sc.flags & GIFT_FLAG_NONFINITE) != 0;
    if (x.nmine)  // wave-uniform
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt)
#pragma unroll
        for (int oc = 0; oc < kb; ++oc)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            put_codes(ct, x, oc, rt, t, e4m3_encode4_scaled(w[oc][rt][t], sc.scale, nonfinite));
            if (kWriteW && L.Wout && x.ok[rt])
              *reinterpret_cast<float4*>(L.Wout + (int64_t)x.row[rt] * L.d_in +
                                         kChunk * (x.c0 + oc) + 16 * t + 4 * x.g) = w[oc][rt][t];
          }
    __syncthreads();
    store_code_tile(L, x, ct);
  } else {
    // per-segment amax: lane max over its chunks, then over the lanes of the
    // same row (xor 16, 32), then over the segment's waves through LDS
    uint32_t (*sm)[kTR][64] = reinterpret_cast<uint32_t (*)[kTR][64]>(mx);
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt) {
      uint32_t m = 0u;
      if (x.nmine)
#pragma unroll
        for (int oc = 0; oc < kb; ++oc) m = amax4(amax4(m, w[oc][rt][0]), w[oc][rt][1]);
      m = max(m, (uint32_t)__shfl_xor(m, 16, 64));
      m = max(m, (uint32_t)__shfl_xor(m, 32, 64));
      sm[x.wave][rt][x.lane] = m;
    }
    __syncthreads();
    const int w0 = x.wave - x.wave % kWPS;
    const int seg = x.c0 / 4;
    const int64_t nseg = L.d_in / kBlock;
    if (x.nmine)  // wave-uniform
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        uint32_t m = 0u;
#pragma unroll
        for (int v = 0; v < kWPS; ++v) m = max(m, sm[w0 + v][rt][x.lane]);
        const Scale sc = scale_from_amax_bits(m);
        if (x.ok[rt] && x.g == 0 && x.wave == w0) {
          L.inv[x.row[rt] * nseg + seg] = sc.inv;
          if (gd.flags && sc.flags) atomicOr(gd.flags, sc.flags);
        }
#pragma unroll
        for (int oc = 0; oc < kb; ++oc)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            put_codes(ct, x, oc, rt, t,
                      e4m3_encode4_scaled(w[oc][rt][t], sc.scale, sc.flags & GIFT_FLAG_NONFINITE));
            if (kWriteW && L.Wout && x.ok[rt])
              *reinterpret_cast<float4*>(L.Wout + (int64_t)x.row[rt] * L.d_in +
                                         kChunk * (x.c0 + oc) + 16 * t + 4 * x.g) = w[oc][rt][t];
          }
      }
    __syncthreads();
    store_code_tile(L, x, ct);
  }
}

// G^[:, block] = inv * (decode(q)[:, block] S^-1): codes are exact in bf16,
// so the product takes the three splits of S^-1 only; the scale (per tensor,
// or the 128-column segment's, which holds the whole block) comes after.
// The codes come through LDS as in k_tile_unwhiten.
template <int kB, bool kB128>
__global__ __launch_bounds__(kTileThreads) void k_blk_dequant(GroupDev gd) {
  constexpr int kb = kB / kChunk;
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kb>(L, tile);
  const int64_t nblk = L.d_in / kB, blk = x.c0 / kb;
  uint32_t qv[kTR][kb][2];
  uint4 pa[kb][2][3];
  float inv[kTR];
  __shared__ __align__(16) CodeTile<kb> ct;
  if (x.nmine) {  // wave-uniform
    load_blk_packs<kb>(L.P, nblk, 1, blk, 0, x.lane, pa);
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt)
      inv[rt] = kB128 ? L.inv[(int64_t)x.row[rt] * (L.d_in / kBlock) + x.c0 / 4] : L.inv[0];
  }
  CodePieces<kb> pcs;
  load_code_pieces(L, x, pcs);
  put_code_pieces(ct, pcs);
  __syncthreads();
  if (x.nmine == 0) return;  // wave-uniform; no barrier below
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt)
#pragma unroll
    for (int kc = 0; kc < kb; ++kc)
#pragma unroll
      for (int t = 0; t < 2; ++t) qv[rt][kc][t] = get_codes(ct, x, kc, rt, t);
  float4 gh[kb][kTR][2];
#pragma unroll
  for (int oc = 0; oc < kb; ++oc) {
    if (oc) load_blk_packs<kb>(L.P, nblk, 1, blk, oc, x.lane, pa);
#pragma unroll
    for (int rt = 0; rt < kTR; ++rt) {
      f32x4 out[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kc = 0; kc < kb; ++kc) {
        bf16x8 a[2][3];
        as_ops(pa[kc], a);
        float v[8];
        decode8(qv[rt][kc][0], qv[rt][kc][1], v);
        bf16x8 bq;
#pragma unroll
        for (int t = 0; t < 8; ++t) bq[t] = (__bf16)v[t];
#pragma unroll
        for (int h = 0; h < 2; ++h) out[h] = mfma3x1(a[h], bq, out[h]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
        gh[oc][rt][t] = make_float4(inv[rt] * out[t][0], inv[rt] * out[t][1], inv[rt] * out[t][2],
                                    inv[rt] * out[t][3]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt) {
    if (!x.ok[rt]) continue;
#pragma unroll
    for (int oc = 0; oc < kb; ++oc)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        st_f4(L.Ghat + (int64_t)x.row[rt] * L.d_in + kChunk * (x.c0 + oc) + 16 * t + 4 * x.g,
              gh[oc][rt][t]);
  }
}

// ---------------------------------------------------------------------------
// dequantize + un-whiten, pass 2: G^ = beta W^ + c'^ U^T with
// W^ = decode(q) * inv and c'^ the row block's (W^ U) * D_u.
// ---------------------------------------------------------------------------
template <int kCPW, int kFmt, int kRB>
__global__ __launch_bounds__(kTileThreads) void k_tile_unwhiten(GroupDev gd) {
  constexpr bool kB128 = kFmt == GIFT_SCALE_BLOCK128, kMX = kFmt == GIFT_SCALE_MXFP4;
  const LayerDev L = gd.L[find_layer(gd, blockIdx.x)];
  const int tile = blockIdx.x - L.tile_begin;
  const Tile x = tile_ctx<kCPW>(L, tile);
  __shared__ uint4 cs[kCOp * kRB];
  const int64_t nseg = L.d_in / kBlock;
  const float inv0 = kFmt == GIFT_SCALE_TENSOR ? L.inv[0] : 1.f;
  const float beta = L.coef[GIFT_COEF_BETA];
  uint4 pa[kCPW][kRB][2][3];
  uint32_t qv[kCPW][kTR][2];
  float sc[kCPW][kTR];
  uint32_t mc[kMX ? kCPW : 1][kTR];
  __shared__ __align__(16) uint32_t ctw[kMX ? (sizeof(MxTile<kCPW>) + 3) / 4 : sizeof(CodeTile<kCPW>) / 4];
  CodeTile<kCPW>& ct = *reinterpret_cast<CodeTile<kCPW>*>(ctw);
  MxTile<kCPW>& mt = *reinterpret_cast<MxTile<kCPW>*>(ctw);
  CodePieces<kCPW> pcs;
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
      load_a_rb<kRB>(L, true, x.c0 + j, x.lane, pa[j]);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        if constexpr (!kMX) sc[j][rt] = kB128 ? L.inv[x.row[rt] * nseg + ((x.c0 + j) >> 2)] : inv0;
      }
    });
  });
  if constexpr (kMX) {
    load_mx_tile(L, x, mt);
  } else {
    load_code_pieces(L, x, pcs);
    put_code_pieces(ct, pcs);
  }
  stage_c<kRB>(L, x, cs);  // its barrier also publishes the codes
  if (x.nmine == 0) return;  // wave-uniform; no barrier below
  with_count<kCPW>(x.nmine, [&](auto N) {
    static_for<decltype(N)::value>([&](auto J) {
      constexpr int j = decltype(J)::value;
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        if constexpr (kMX) {
          get_mx(mt, x, j, rt, qv[j][rt], mc[j][rt]);
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) qv[j][rt][t] = get_codes(ct, x, j, rt, t);
        }
      }
    });
  });
  float4 out[kCPW][kTR][2];
  with_count<kCPW>(x.nmine, [&](auto N) {
    constexpr int n = decltype(N)::value;
    static_for<n>([&](auto J) {
      constexpr int j = decltype(J)::value;
      bf16x8 a[kRB][2][3];
      as_ops_rb<kRB>(pa[j], a);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        f32x4 corr[2];
        correction_rb<kRB>(a, cs, rt, x.lane, corr);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t qq = qv[j][rt][t];
          float4 wv;
          if constexpr (kMX) {
            wv = mx_decode4(qq, mc[j][rt]);
          } else {
            const float s = sc[j][rt];
            wv = make_float4(e4m3_decode(qq, 0) * s, e4m3_decode(qq, 1) * s,
                             e4m3_decode(qq, 2) * s, e4m3_decode(qq, 3) * s);
          }
          out[j][rt][t] = make_float4(fmaf(beta, wv.x, corr[t][0]), fmaf(beta, wv.y, corr[t][1]),
                                      fmaf(beta, wv.z, corr[t][2]), fmaf(beta, wv.w, corr[t][3]));
        }
      }
    });
    static_for<n>([&](auto J) {
      constexpr int j = decltype(J)::value;
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        if (!x.ok[rt]) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          st_f4(L.Ghat + x.row[rt] * L.d_in + kChunk * (x.c0 + j) + 16 * t + 4 * x.g,
                out[j][rt][t]);
      }
    });
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
      const float4 v = ld_g(L.G + e);
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
  for (int i = threadIdx.x; i < L.n_part; i += kThreads) m = max(m, L.part[i]);
  m = block_max_u32<kThreads>(m, mx);
  if (threadIdx.x == 0) *L.amax = m;
}

// Euclidean quantize (pass 2 of per-tensor, or the single pass of 1x128 and
// MXFP4), optionally dequantizing in the same pass (the round trip).
template <int kFmt, bool kDeq, bool kWriteW>
__global__ __launch_bounds__(kThreads) void k_flat_quant(GroupDev g) {
  constexpr bool kB128 = kFmt == GIFT_SCALE_BLOCK128, kMX = kFmt == GIFT_SCALE_MXFP4;
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  Scale sc{1.f, 1.f, 0u};
  if (kFmt == GIFT_SCALE_TENSOR) {
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
    if (act) v = ld_g(L.G + e);
    uint32_t m = max(max(abs_bits(v.x), abs_bits(v.y)), max(abs_bits(v.z), abs_bits(v.w)));
    if constexpr (kB128) {
      // 32 consecutive lanes hold one 128-element segment (d_in % 128 == 0)
      m = half_wave_max_u32(m);
      sc = scale_from_amax_bits(m);
      if (act && (threadIdx.x & 31) == 0) {
        L.inv[e / kBlock] = sc.inv;
        if (g.flags && sc.flags) atomicOr(g.flags, sc.flags);
      }
    }
    if constexpr (kMX) {
      // 8 consecutive lanes hold one 32-element block (d_in % 32 == 0)
#pragma unroll
      for (int o = 4; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor(m, o, 64));
      uint32_t fl = 0u;
      const uint32_t code = mx_scale_code(m, fl);
      const uint32_t q = mx_encode4(v, mx_scale_operand(code), code == kMxScaleNaN);
      if (!act) continue;
      *reinterpret_cast<uint16_t*>(L.q + e / 2) = (uint16_t)q;
      if ((threadIdx.x & 7) == 0) {
        reinterpret_cast<uint8_t*>(L.inv)[e / kMxBlock] = (uint8_t)code;
        if (g.flags && fl) atomicOr(g.flags, fl);
      }
      if (kWriteW && L.Wout) *reinterpret_cast<float4*>(L.Wout + e) = v;
      if (kDeq) st_f4(L.Ghat + e, mx_decode4(q, code));
      continue;
    }
    if (!act) continue;
    const uint32_t c = e4m3_encode4_scaled(v, sc.scale, sc.flags & GIFT_FLAG_NONFINITE);
    st_q4(L.q + e, c);
    if (kWriteW && L.Wout) *reinterpret_cast<float4*>(L.Wout + e) = v;
    if (kDeq) {
      float4 o;
      o.x = e4m3_decode(c, 0) * sc.inv;
      o.y = e4m3_decode(c, 1) * sc.inv;
      o.z = e4m3_decode(c, 2) * sc.inv;
      o.w = e4m3_decode(c, 3) * sc.inv;
      st_f4(L.Ghat + e, o);
    }
  }
}

// plain dequantize of Euclidean layers: G^ = decode(q) * inv
template <int kFmt>
__global__ __launch_bounds__(kThreads) void k_flat_dequant(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  const float inv0 = kFmt == GIFT_SCALE_TENSOR ? L.inv[0] : 1.f;
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    if (e >= n) continue;
    if constexpr (kFmt == GIFT_SCALE_MXFP4) {
      const uint32_t q = *reinterpret_cast<const uint16_t*>(L.q + e / 2);
      const uint32_t code = reinterpret_cast<const uint8_t*>(L.inv)[e / kMxBlock];
      st_f4(L.Ghat + e, mx_decode4(q, code));
      continue;
    }
    const float s = kFmt == GIFT_SCALE_BLOCK128 ? L.inv[e / kBlock] : inv0;
    const uint32_t c = ld_q4(L.q + e);
    float4 o;
    o.x = e4m3_decode(c, 0) * s;
    o.y = e4m3_decode(c, 1) * s;
    o.z = e4m3_decode(c, 2) * s;
    o.w = e4m3_decode(c, 3) * s;
    st_f4(L.Ghat + e, o);
  }
}

// dequantize and accumulate: G_hat = decode(q) * inv (kFirst) or
// fl32(G_hat + decode(q) * inv), element by element
template <int kFmt, bool kFirst>
__global__ __launch_bounds__(kThreads) void k_flat_accumulate(GroupDev g) {
  const int l = find_layer(g, blockIdx.x);
  const LayerDev& L = g.L[l];
  const int tile = blockIdx.x - L.tile_begin;
  const int64_t n = L.d_out * L.d_in, base = (int64_t)tile * kFlatTile;
  const float inv0 = kFmt == GIFT_SCALE_TENSOR ? L.inv[0] : 1.f;
#pragma unroll
  for (int i = 0; i < kFlatTile / (4 * kThreads); ++i) {
    const int64_t e = base + 4 * ((int64_t)i * kThreads + threadIdx.x);
    if (e >= n) continue;
    float4 o;
    if constexpr (kFmt == GIFT_SCALE_MXFP4) {
      const uint32_t q = *reinterpret_cast<const uint16_t*>(L.q + e / 2);
      o = mx_decode4(q, reinterpret_cast<const uint8_t*>(L.inv)[e / kMxBlock]);
    } else {
      const float s = kFmt == GIFT_SCALE_BLOCK128 ? L.inv[e / kBlock] : inv0;
      const uint32_t c = ld_q4(L.q + e);
      o = make_float4(e4m3_decode(c, 0) * s, e4m3_decode(c, 1) * s, e4m3_decode(c, 2) * s,
                      e4m3_decode(c, 3) * s);
    }
    float4* dst = reinterpret_cast<float4*>(L.Ghat + e);
    if constexpr (!kFirst) {
      const float4 a = *dst;
      o = make_float4(a.x + o.x, a.y + o.y, a.z + o.z, a.w + o.w);
    }
    *dst = o;
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
      const float4 a = ld_g(L.G + e);
      const float4 b = ld_g(L.Ghat + e);
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

#if GIFT_TILE_RT == 4
// ---------------------------------------------------------------------------
// slab kernels.  A workgroup of kSW waves owns one row block -- kTileRows
// rows of one layer and every column -- so a row's c = g U is complete
// inside it: no partial buffer and no reduction launch.  Wave w takes the
// 32-column chunks w, w + kSW, w + 2 kSW, ... (the waves of one step cover
// adjacent columns).  Phase 1 forms the wave's partial c over its chunks on
// MFMA with the next chunk's operands in flight while the current one is
// multiplied; the waves' partials are summed in wave order through LDS, c'
// is formed and split into the second product's operand form; phase 2 walks
// the chunks again, last first (the most recently read data is the likeliest
// to be still in a cache), for the second product.  The gradient is read
// twice, both times by the same workgroup.  Chunk loads are issued
// unconditionally (past the wave's last chunk it loads its current chunk
// again, a cache hit), so every wait is for the chunk in use.  Only the
// whiten side runs this way: a dequantize slab (codes read twice, G^
// written once, no partials) measured slower than the three tile kernels.
// ---------------------------------------------------------------------------
constexpr int kSW = 8;                    // waves per slab workgroup
constexpr int kSlabThreads = 64 * kSW;

struct Slab {
  int row[kTR];   // this lane's gradient row in each 16-row tile (clamped)
  bool ok[kTR];   // row < d_out
  int nch;        // 32-column chunks of the layer
  int nmine;      // chunks of this wave: wave, wave + kSW, ...
  int lane, wave, r16, g;
};

__device__ __forceinline__ Slab slab_ctx(const LayerDev& L, int64_t rb) {
  Slab x;
  x.lane = threadIdx.x & 63;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  x.r16 = x.lane & 15;
  x.g = x.lane >> 4;
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt) {
    const int64_t r = rb * kTileRows + 16 * rt + x.r16;
    x.ok[rt] = r < L.d_out;
    x.row[rt] = (int)(x.ok[rt] ? r : L.d_out - 1);
  }
  x.nch = (int)(L.d_in / kChunk);
  x.nmine = x.wave < x.nch ? (x.nch - x.wave + kSW - 1) / kSW : 0;
  return x;
}

// the operands of the wave's k-th chunk (k clamped to its last chunk)
template <bool kCodes>
struct SlabOps {
  uint4 pa[2][3];
  float4 gv[kCodes ? 1 : kTR][2];
  uint32_t qv[kCodes ? kTR : 1][2];
};

template <bool kCodes>
__device__ __forceinline__ void slab_load(const LayerDev& L, const Slab& x, const uint4* P, int k,
                                          SlabOps<kCodes>& o) {
  const int c = x.wave + kSW * (k < x.nmine ? k : x.nmine - 1);
  load_a(P, c, x.lane, o.pa);
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt) {
    if constexpr (kCodes) load_qc(L, x.row[rt], x.g, c, o.qv[rt]);
    else load_gc(L, x.row[rt], x.g, c, o.gv[rt]);
  }
}

// Phase 1 and the reduction: c' of the slab's rows (times D_w; on codes,
// times D_u and the tensor's inverse scale) in operand form in cs, and, when
// cfin is not NULL, also in global memory for a later pass.  Contains
// workgroup barriers.
template <bool kCodes>
__device__ __forceinline__ void slab_cprime(const LayerDev& L, const Slab& x, int64_t rb,
                                            float (*red)[kTR * 8][64], uint4* cs) {
  f32x4 acc[kTR][2];
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (x.nmine > 0) {  // wave-uniform
    SlabOps<kCodes> o[2];
    slab_load<kCodes>(L, x, L.P, 0, o[0]);
    auto mult = [&](const SlabOps<kCodes>& op) {
      bf16x8 a[2][3];
      as_ops(op.pa, a);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        if constexpr (kCodes) cpart_q(a, op.qv[rt], acc[rt]);
        else cpart_g(a, op.gv[rt], acc[rt]);
      }
    };
    for (int k = 0; k < x.nmine; k += 2) {
      slab_load<kCodes>(L, x, L.P, k + 1, o[1]);
      mult(o[0]);
      if (k + 1 >= x.nmine) break;
      slab_load<kCodes>(L, x, L.P, k + 2, o[0]);
      mult(o[1]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < kTR; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[x.wave][rt * 8 + 4 * h + i][x.lane] = acc[rt][h][i];
  __syncthreads();
  for (int e = threadIdx.x; e < kTR * 64; e += kSlabThreads) {
    const int rt = e >> 6, lane = e & 63;
    const float* dk = L.coef + (kCodes ? GIFT_COEF_DU : GIFT_COEF_DW);
    const float extra = kCodes ? L.inv[0] : 1.f;
    float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSW; ++w)
#pragma unroll
      for (int k = 0; k < 8; ++k) s8[k] += red[w][rt * 8 + k][lane];
    float cp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cp[k] = s8[k] * (dk[rank_of(k, lane >> 4)] * extra);
    bf16x8 cb[3];
    split3(cp, cb);
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) cs[(rt * 3 + sp) * 64 + lane] = __builtin_bit_cast(uint4, cb[sp]);
    if (L.cfin) put_cfin(L, rb, rt, lane, cp);
  }
  __syncthreads();
}

// whiten, first pass of per-tensor scaling: c' (to the workspace, for the
// quantize pass) and the slab's amax of |W| (to the layer's partials).
// grid: one workgroup per row block of the group.
__global__ __launch_bounds__(kSlabThreads) void k_slab_whiten(GroupDev gd) {
  const LayerDev L = layer_at(gd, find_layer_rb(gd, blockIdx.x));
  const int64_t rb = blockIdx.x - L.rb_begin;
  const Slab x = slab_ctx(L, rb);
  __shared__ float red[kSW][kTR * 8][64];
  __shared__ uint4 cs[kCOp];
  __shared__ uint32_t mx[kSW];
  slab_cprime<false>(L, x, rb, red, cs);
  const uint4* P2 = p2_of(L);
  const float alpha = L.coef[GIFT_COEF_ALPHA];
  uint32_t m = 0u;
  if (x.nmine > 0) {  // wave-uniform
    SlabOps<false> o[2];
    const int last = x.nmine - 1;
    slab_load<false>(L, x, P2, last, o[0]);
    auto amax_of = [&](const SlabOps<false>& op) {
      bf16x8 a[2][3];
      as_ops(op.pa, a);
#pragma unroll
      for (int rt = 0; rt < kTR; ++rt) {
        bf16x8 cb[3];
        c_operand(cs, rt, x.lane, cb);
        f32x4 corr[2];
        correction(a, cb, corr);
        if (!x.ok[rt]) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float4 gg = op.gv[rt][t];
          const float4 w = make_float4(fmaf(alpha, gg.x, corr[t][0]), fmaf(alpha, gg.y, corr[t][1]),
                                       fmaf(alpha, gg.z, corr[t][2]), fmaf(alpha, gg.w, corr[t][3]));
          m = amax4(m, w);
        }
      }
    };
    for (int k = last; k >= 0; k -= 2) {
      slab_load<false>(L, x, P2, k > 0 ? k - 1 : 0, o[1]);
      amax_of(o[0]);
      if (k == 0) break;
      slab_load<false>(L, x, P2, k > 1 ? k - 2 : 0, o[0]);
      amax_of(o[1]);
    }
  }
  m = block_max_u32<kSlabThreads>(m, mx);
  if (threadIdx.x == 0) L.part[rb] = m;
}

#endif  // GIFT_TILE_RT == 4

// descriptors of a large group into device memory, kPutLayers per launch
// (the kernel argument holds them)
constexpr int kPutLayers = 24;
struct LayerBatch {
  int n;
  LayerDev L[kPutLayers];
};
__global__ __launch_bounds__(64) void k_put_layers(LayerBatch b, LayerDev* dst) {
  if ((int)threadIdx.x < b.n) dst[threadIdx.x] = b.L[threadIdx.x];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_put_layers(const LayerDev* host, int n, LayerDev* dst, hipStream_t s) {
  for (int i0 = 0; i0 < n; i0 += kPutLayers) {
    LayerBatch b{};
    b.n = n - i0 < kPutLayers ? n - i0 : kPutLayers;
    for (int i = 0; i < b.n; ++i) b.L[i] = host[i0 + i];
    k_put_layers<<<dim3(1), dim3(64), 0, s>>>(b, dst + i0);
  }
  return hipGetLastError();
}

constexpr int kCPW = 1;  // chunks per wave of the tile kernels

int64_t row_blocks(int64_t d_out) { return (d_out + kTileRows - 1) / kTileRows; }
int col_groups(int64_t d_in) {
  const int64_t nch = d_in / kChunk, per = (int64_t)kTW * kCPW;
  return (int)((nch + per - 1) / per);
}
int frag_floats() { return kFrag; }
int cop_bytes() { return kCF * 16; }
int flat_tiles(int64_t n) { return (int)((n + kFlatTile - 1) / kFlatTile); }
size_t pack_bytes(int64_t d_in) { return (size_t)(d_in / kChunk) * 2 * 2 * 3 * 64 * 16; }

hipError_t launch_pack(const PackGroup& pg, hipStream_t s) {
  int maxd = 0;
  for (int i = 0; i < pg.n; ++i) maxd = pg.f[i].d_in > maxd ? pg.f[i].d_in : maxd;
  const int per = 2 * (maxd / kChunk) * 2 * 64;
  k_pack_u<<<dim3((per + kThreads - 1) / kThreads, pg.n), dim3(kThreads), 0, s>>>(pg);
  return hipGetLastError();
}

// scaling: GIFT_SCALE_TENSOR, GIFT_SCALE_BLOCK128 or GIFT_SCALE_MXFP4
template <int kRB>
hipError_t whiten_quantize_rb(const GroupDev& g, int scaling, bool write_w, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kTileThreads);
  k_tile_cpart<kCPW, false, GIFT_SCALE_TENSOR, kRB><<<grid, blk, 0, s>>>(g);
  k_tile_reduce<false, false, kRB><<<dim3(g.total_rb), dim3(kReduceThreads), 0, s>>>(g);
#define GIFT_TW(F, W) k_tile_whiten<kCPW, F, W, kRB><<<grid, blk, 0, s>>>(g)
  if (scaling == GIFT_SCALE_BLOCK128) {
    if (write_w) GIFT_TW(GIFT_SCALE_BLOCK128, true); else GIFT_TW(GIFT_SCALE_BLOCK128, false);
    return hipGetLastError();
  }
  if (scaling == GIFT_SCALE_MXFP4) {
    if (write_w) GIFT_TW(GIFT_SCALE_MXFP4, true); else GIFT_TW(GIFT_SCALE_MXFP4, false);
    return hipGetLastError();
  }
  GIFT_TW(GIFT_SCALE_TENSOR, false);
#undef GIFT_TW
  bool tall = false;
  for (int i = 0; i < g.n; ++i) tall |= g.L[i].n_part > kPartialLimit;
  if (tall) k_amax_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g);
  if (write_w) k_tile_quant<kCPW, true, kRB><<<grid, blk, 0, s>>>(g);
  else k_tile_quant<kCPW, false, kRB><<<grid, blk, 0, s>>>(g);
  return hipGetLastError();
}

// rb: rank blocks of the group's factors (1: rank <= 32, 2: rank <= 64)
hipError_t launch_whiten_quantize(const GroupDev& g, int scaling, bool write_w, hipStream_t s,
                                  int rb) {
  return rb == 2 ? whiten_quantize_rb<2>(g, scaling, write_w, s)
                 : whiten_quantize_rb<1>(g, scaling, write_w, s);
}

hipError_t launch_flat_quantize(const GroupDev& g, int scaling, bool deq, bool write_w,
                                hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kThreads);
  if (scaling == GIFT_SCALE_TENSOR) {
    k_flat_amax<<<grid, blk, 0, s>>>(g);
    k_amax_final<<<dim3(g.n), blk, 0, s>>>(g);
  }
#define GIFT_FQ(F, D, W) k_flat_quant<F, D, W><<<grid, blk, 0, s>>>(g)
#define GIFT_FQ_ALL(F)                                                        \
  if (deq) { if (write_w) GIFT_FQ(F, true, true); else GIFT_FQ(F, true, false); } \
  else     { if (write_w) GIFT_FQ(F, false, true); else GIFT_FQ(F, false, false); }
  if (scaling == GIFT_SCALE_BLOCK128) {
    GIFT_FQ_ALL(GIFT_SCALE_BLOCK128)
  } else if (scaling == GIFT_SCALE_MXFP4) {
    GIFT_FQ_ALL(GIFT_SCALE_MXFP4)
  } else {
    GIFT_FQ_ALL(GIFT_SCALE_TENSOR)
  }
#undef GIFT_FQ_ALL
#undef GIFT_FQ
  return hipGetLastError();
}

#if GIFT_TILE_RT == 4
// per-tensor whiten + quantize of layers whose row blocks run as slabs:
// k_slab_whiten (c' and one amax partial per row block) runs once over all
// of them -- its workgroups are long, so a launch per 16 layers would leave
// the machine part idle at each launch's end -- then, per group of inline
// descriptors, the layer amax (k_amax_final for layers of more than
// kPartialLimit row blocks) and the 64-row tile quantize pass on the slabs'
// c'.  The quantize workgroups are short: looking their layer up in device
// memory would cost them more than the launch ends cost.
hipError_t launch_slab_whiten(const GroupDev& all, hipStream_t s) {
  k_slab_whiten<<<dim3(all.total_rb), dim3(kSlabThreads), 0, s>>>(all);
  return hipGetLastError();
}

hipError_t launch_slab_quantize(const GroupDev& g, bool write_w, hipStream_t s) {
  bool tall = false;
  for (int i = 0; i < g.n; ++i) tall |= g.L[i].n_part > kPartialLimit;
  if (tall) k_amax_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g);
  const dim3 grid(g.total_tiles), blk(kTileThreads);
  if (write_w) k_tile_quant<kCPW, true, 1><<<grid, blk, 0, s>>>(g);
  else k_tile_quant<kCPW, false, 1><<<grid, blk, 0, s>>>(g);
  return hipGetLastError();
}

#endif

// chunks per wave of the dequantize side's first product: column groups of
// 256 kDeqCPW columns, so half the partial coefficients are written and
// summed (the un-whiten pass keeps kCPW: with two chunks per wave it spills)
constexpr int kDeqCPW = 2;

// g with the column groups of kDeqCPW chunks per wave (the tiles of the
// first product and the partials the reduction sums)
GroupDev deq_groups(const GroupDev& g) {
  GroupDev w = g;
  int tiles = 0;
  for (int i = 0; i < g.n; ++i) {
    LayerDev& L = w.L[i];
    const int nch = (int)(L.d_in / kChunk), per = kTW * kDeqCPW;
    L.ngrp = (nch + per - 1) / per;
    L.n_tiles = (int)L.n_rb * L.ngrp;
    L.tile_begin = tiles;
    tiles += L.n_tiles;
  }
  w.total_tiles = tiles;
  return w;
}

template <int kRB>
void dequant_white_rb(const GroupDev& g, int scaling, hipStream_t s) {
  const GroupDev gw = kDeqCPW == kCPW ? g : deq_groups(g);
  const dim3 grid(g.total_tiles), wgrid(gw.total_tiles), blk(kTileThreads);
  const dim3 rgrid(g.total_rb), rblk(kReduceThreads);
  if (scaling == GIFT_SCALE_BLOCK128) {
    k_tile_cpart<kDeqCPW, true, GIFT_SCALE_BLOCK128, kRB><<<wgrid, blk, 0, s>>>(gw);
    k_tile_reduce<true, true, kRB><<<rgrid, rblk, 0, s>>>(gw);
    k_tile_unwhiten<kCPW, GIFT_SCALE_BLOCK128, kRB><<<grid, blk, 0, s>>>(g);
  } else if (scaling == GIFT_SCALE_MXFP4) {
    k_tile_cpart<kDeqCPW, true, GIFT_SCALE_MXFP4, kRB><<<wgrid, blk, 0, s>>>(gw);
    k_tile_reduce<true, true, kRB><<<rgrid, rblk, 0, s>>>(gw);
    k_tile_unwhiten<kCPW, GIFT_SCALE_MXFP4, kRB><<<grid, blk, 0, s>>>(g);
  } else {
    k_tile_cpart<kDeqCPW, true, GIFT_SCALE_TENSOR, kRB><<<wgrid, blk, 0, s>>>(gw);
    k_tile_reduce<true, false, kRB><<<rgrid, rblk, 0, s>>>(gw);
    k_tile_unwhiten<kCPW, GIFT_SCALE_TENSOR, kRB><<<grid, blk, 0, s>>>(g);
  }
}

hipError_t launch_dequant(const GroupDev& g, int scaling, bool white, hipStream_t s, int rb) {
  if (white) {
    if (rb == 2) dequant_white_rb<2>(g, scaling, s);
    else dequant_white_rb<1>(g, scaling, s);
  } else {
    const dim3 grid(g.total_tiles), blk(kThreads);
    if (scaling == GIFT_SCALE_BLOCK128) k_flat_dequant<GIFT_SCALE_BLOCK128><<<grid, blk, 0, s>>>(g);
    else if (scaling == GIFT_SCALE_MXFP4) k_flat_dequant<GIFT_SCALE_MXFP4><<<grid, blk, 0, s>>>(g);
    else k_flat_dequant<GIFT_SCALE_TENSOR><<<grid, blk, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_blk_pack(const PackGroup& pg, int b, hipStream_t s) {
  int64_t maxl = 0;
  for (int i = 0; i < pg.n; ++i) {
    const int64_t kb = b / kChunk, l = 2 * (pg.f[i].d_in / b) * kb * kb * 2 * 64;
    maxl = l > maxl ? l : maxl;
  }
  k_pack_blk<<<dim3((unsigned)((maxl + kThreads - 1) / kThreads), pg.n), dim3(kThreads), 0, s>>>(pg, b);
  return hipGetLastError();
}

int blk_col_groups(int64_t d_in, int b) {
  const int64_t per = (int64_t)kTW * (b / kChunk);  // chunks per workgroup
  return (int)((d_in / kChunk + per - 1) / per);
}

// block-diagonal factors of block size b (32 or 64); scaling: per tensor or 1x128
hipError_t launch_blk_whiten(const GroupDev& g, int b, int scaling, bool write_w, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kTileThreads);
#define GIFT_BW(B, M, W) k_blk_whiten<B, M, W><<<grid, blk, 0, s>>>(g)
  if (scaling == GIFT_SCALE_BLOCK128) {
    if (b == 32) { if (write_w) GIFT_BW(32, 2, true); else GIFT_BW(32, 2, false); }
    else { if (write_w) GIFT_BW(64, 2, true); else GIFT_BW(64, 2, false); }
    return hipGetLastError();
  }
  if (b == 32) GIFT_BW(32, 0, false); else GIFT_BW(64, 0, false);
  bool tall = false;
  for (int i = 0; i < g.n; ++i) tall |= g.L[i].n_part > kPartialLimit;
  if (tall) k_amax_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g);
  if (b == 32) { if (write_w) GIFT_BW(32, 1, true); else GIFT_BW(32, 1, false); }
  else { if (write_w) GIFT_BW(64, 1, true); else GIFT_BW(64, 1, false); }
#undef GIFT_BW
  return hipGetLastError();
}

hipError_t launch_blk_dequant(const GroupDev& g, int b, int scaling, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kTileThreads);
  const bool b128 = scaling == GIFT_SCALE_BLOCK128;
  if (b == 32) { if (b128) k_blk_dequant<32, true><<<grid, blk, 0, s>>>(g); else k_blk_dequant<32, false><<<grid, blk, 0, s>>>(g); }
  else { if (b128) k_blk_dequant<64, true><<<grid, blk, 0, s>>>(g); else k_blk_dequant<64, false><<<grid, blk, 0, s>>>(g); }
  return hipGetLastError();
}

hipError_t launch_accumulate(const GroupDev& g, int scaling, bool first, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kThreads);
#define GIFT_ACC(F)                                                     \
  if (first) k_flat_accumulate<F, true><<<grid, blk, 0, s>>>(g);         \
  else k_flat_accumulate<F, false><<<grid, blk, 0, s>>>(g);
  if (scaling == GIFT_SCALE_BLOCK128) {
    GIFT_ACC(GIFT_SCALE_BLOCK128)
  } else if (scaling == GIFT_SCALE_MXFP4) {
    GIFT_ACC(GIFT_SCALE_MXFP4)
  } else {
    GIFT_ACC(GIFT_SCALE_TENSOR)
  }
#undef GIFT_ACC
  return hipGetLastError();
}

// G_hat = G_hat A_r^1/2 in place (the descriptors' G points at G_hat)
template <int kRB>
void unwhiten_f32_rb(const GroupDev& g, hipStream_t s) {
  const dim3 grid(g.total_tiles), blk(kTileThreads);
  k_tile_cpart<kCPW, false, GIFT_SCALE_TENSOR, kRB><<<grid, blk, 0, s>>>(g);
  k_tile_reduce<true, true, kRB><<<dim3(g.total_rb), dim3(kReduceThreads), 0, s>>>(g);
  k_tile_whiten<kCPW, kFmtUnwhiten, false, kRB><<<grid, blk, 0, s>>>(g);
}

hipError_t launch_unwhiten_f32(const GroupDev& g, hipStream_t s, int rb) {
  if (rb == 2) unwhiten_f32_rb<2>(g, s);
  else unwhiten_f32_rb<1>(g, s);
  return hipGetLastError();
}

hipError_t launch_error(const GroupDev& g, int out_base, hipStream_t s) {
  k_err_partial<<<dim3(g.total_tiles), dim3(kThreads), 0, s>>>(g);
  k_err_final<<<dim3(g.n), dim3(kThreads), 0, s>>>(g, out_base);
  return hipGetLastError();
}

}  // namespace GIFT_TILE_NS
}  // namespace gift
