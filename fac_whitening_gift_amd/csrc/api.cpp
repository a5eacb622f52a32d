// Host side of the C ABI declared in include/gift.h: argument validation,
// workspace carving and grouping of layers into launches.  Every call only
// enqueues kernels on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "device.hpp"

namespace gift {
// roundtrip.hip, built with 64-row tiles (rt4) and 32-row tiles (rt2)
#define GIFT_TILE_DECLS                                                                          \
  hipError_t launch_whiten_quantize(const GroupDev& g, int scaling, bool write_w, hipStream_t s,  \
                                    int rb);                                                     \
  hipError_t launch_flat_quantize(const GroupDev& g, int scaling, bool deq, bool write_w,         \
                                  hipStream_t s);                                                \
  hipError_t launch_dequant(const GroupDev& g, int scaling, bool white, hipStream_t s, int rb);   \
  hipError_t launch_error(const GroupDev& g, int out_base, hipStream_t s);                       \
  hipError_t launch_accumulate(const GroupDev& g, int scaling, bool first, hipStream_t s);        \
  hipError_t launch_unwhiten_f32(const GroupDev& g, hipStream_t s, int rb);                      \
  hipError_t launch_pack(const PackGroup& pg, hipStream_t s);                                    \
  hipError_t launch_blk_pack(const PackGroup& pg, int b, hipStream_t s);                         \
  hipError_t launch_blk_whiten(const GroupDev& g, int b, int scaling, bool write_w,              \
                               hipStream_t s);                                                   \
  hipError_t launch_blk_dequant(const GroupDev& g, int b, int scaling, hipStream_t s);            \
  int blk_col_groups(int64_t d_in, int b);                                                       \
  size_t blk_pack_bytes(int64_t d_in, int b);                                                    \
  int64_t row_blocks(int64_t d_out);                                                             \
  int col_groups(int64_t d_in);                                                                  \
  int frag_floats();                                                                             \
  int cop_bytes();                                                                               \
  int flat_tiles(int64_t n);                                                                     \
  size_t pack_bytes(int64_t d_in);
namespace rt4 {
GIFT_TILE_DECLS
hipError_t launch_slab_whiten(const GroupDev& all, hipStream_t s);
hipError_t launch_slab_quantize(const GroupDev& g, bool write_w, hipStream_t s);
hipError_t launch_put_layers(const LayerDev* host, int n, LayerDev* dst, hipStream_t s);
}
namespace rt2 {
GIFT_TILE_DECLS
}
#undef GIFT_TILE_DECLS
// what does not depend on the tile height comes from rt4
using rt4::blk_col_groups;
using rt4::blk_pack_bytes;
using rt4::col_groups;
using rt4::flat_tiles;
using rt4::launch_accumulate;
using rt4::launch_blk_pack;
using rt4::launch_error;
using rt4::launch_flat_quantize;
using rt4::launch_pack;
using rt4::pack_bytes;

// The tile-height dependent part: rows per tile and the launchers.
struct TileOps {
  int64_t (*row_blocks)(int64_t d_out);
  int (*frag_floats)();
  int (*cop_bytes)();
  hipError_t (*whiten_quantize)(const GroupDev& g, int scaling, bool write_w, hipStream_t s,
                                int rb);
  hipError_t (*dequant)(const GroupDev& g, int scaling, bool white, hipStream_t s, int rb);
  hipError_t (*unwhiten_f32)(const GroupDev& g, hipStream_t s, int rb);
  hipError_t (*blk_whiten)(const GroupDev& g, int b, int scaling, bool write_w, hipStream_t s);
  hipError_t (*blk_dequant)(const GroupDev& g, int b, int scaling, hipStream_t s);
};
const TileOps kTiles64 = {rt4::row_blocks,           rt4::frag_floats,      rt4::cop_bytes,
                          rt4::launch_whiten_quantize, rt4::launch_dequant,
                          rt4::launch_unwhiten_f32,    rt4::launch_blk_whiten,
                          rt4::launch_blk_dequant};
const TileOps kTiles32 = {rt2::row_blocks,           rt2::frag_floats,      rt2::cop_bytes,
                          rt2::launch_whiten_quantize, rt2::launch_dequant,
                          rt2::launch_unwhiten_f32,    rt2::launch_blk_whiten,
                          rt2::launch_blk_dequant};

// refresh.hip
size_t refresh_workspace_bytes(int64_t d_in, int64_t n_tokens, int x_dtype, int width);
gift_status refresh_factor(const void* X, int x_dtype, int64_t n_tokens, const gift_factor* f,
                           float damp_eps, int damping_mode, int width, int power_steps,
                           uint64_t seed, const float* sketch, float* A_out, uint32_t* flags,
                           void* ws, size_t ws_bytes, hipStream_t s, std::string* err);
gift_status draw_sketch(float* out, int64_t d, int width, uint64_t seed, hipStream_t s,
                        std::string* err);
size_t refresh_group_workspace_bytes(const gift_refresh_input* in, int n, int width);
gift_status refresh_factors(const gift_refresh_input* in, int n, float damp_eps, int damping_mode,
                            int width, int power_steps, uint32_t* flags, void* ws, size_t ws_bytes,
                            hipStream_t st, std::string* err);
}  // namespace gift

using namespace gift;

namespace {

thread_local std::string t_err;

gift_status fail(gift_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_err = buf;
  return s;
}

gift_status hip_fail(hipError_t e, const char* where) {
  return fail(GIFT_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 36;

enum class Op { Whiten, Dequant, Euclid, Error, Accumulate, UnwhitenF32 };

bool whitened(const gift_layer& L, Op op) {
  return L.factor != nullptr && (op == Op::Whiten || op == Op::Dequant || op == Op::UnwhitenF32);
}

// block size of a layer's factor: 0 for the rank-r factor (or no factor)
int fblock(const gift_layer& L) { return L.factor ? L.factor->block : 0; }

// rank blocks (32 columns each) of a layer's rank-r factor: 1 or 2
int frb(const gift_layer& L) {
  return L.factor && !L.factor->block ? factor_cols(L.factor->rank) / kRank : 1;
}

// Per-layer workspace needs of one grouped op.
struct LayerWs {
  size_t cbuf = 0, cfin = 0, part = 0, part2 = 0, amax = 0;
  size_t total() const {
    return align_up(cbuf) + align_up(cfin) + align_up(part) + align_up(part2) + align_up(amax);
  }
};

// workgroups of a whitened layer's tile kernels: row blocks x column groups
int row_tiles(const gift_layer& L, const TileOps& t) {
  const int b = fblock(L);
  return (int)(t.row_blocks(L.d_out) * (b ? blk_col_groups(L.d_in, b) : col_groups(L.d_in)));
}

int row_tiles_max(const gift_layer& L) {
  const int a = row_tiles(L, kTiles64), b = row_tiles(L, kTiles32);
  return a > b ? a : b;
}

LayerWs layer_ws(const gift_layer& L, Op op, bool block) {
  LayerWs w;
  const int64_t n = L.d_out * L.d_in;
  // either tile height (the larger of the two layouts)
  size_t frag = 0, cop = 0;
  for (const TileOps* t : {&kTiles64, &kTiles32}) {
    const size_t f = (size_t)t->row_blocks(L.d_out) * t->frag_floats() * sizeof(float);
    const size_t c = (size_t)t->row_blocks(L.d_out) * t->cop_bytes();
    frag = f > frag ? f : frag;
    cop = c > cop ? c : cop;
  }
  switch (op) {
    case Op::Whiten:
      if (L.factor && L.factor->block) {
        if (!block) {  // one amax per tile, the layer amax
          w.part = (size_t)row_tiles_max(L) * sizeof(uint32_t);
          w.amax = sizeof(uint32_t);
        }
      } else if (L.factor) {
        w.cbuf = (size_t)col_groups(L.d_in) * frag * frb(L);  // partial c per column group
        w.cfin = cop * frb(L);                                 // c' of every row (fp32)
        if (!block) {  // one amax per tile, the layer amax
          w.part = (size_t)row_tiles_max(L) * sizeof(uint32_t);
          w.amax = sizeof(uint32_t);
        }
      } else if (!block) {
        w.part = (size_t)flat_tiles(n) * sizeof(uint32_t);
        w.amax = sizeof(uint32_t);
      }
      break;
    case Op::Euclid:
      if (!block) {
        w.part = (size_t)flat_tiles(n) * sizeof(uint32_t);
        w.amax = sizeof(uint32_t);
      }
      break;
    case Op::Dequant:
    case Op::UnwhitenF32:
      if (L.factor && !L.factor->block) {
        w.cbuf = (size_t)col_groups(L.d_in) * frag * frb(L);
        w.cfin = cop * frb(L);
      }
      break;
    case Op::Error:
      w.part2 = (size_t)flat_tiles(n) * 2 * sizeof(double);
      break;
    case Op::Accumulate:
      break;
  }
  return w;
}

// Operand packs: one region per distinct factor (identified by its U
// pointer) among the whitened layers of the call, at the start of ws.
struct Packs {
  std::vector<const float*> U;
  std::vector<int> d_in;
  std::vector<int> cols;   // storage columns of U (32 or 64)
  std::vector<size_t> off;
  size_t bytes = 0;
  size_t find(const float* u) const {
    for (size_t i = 0; i < U.size(); ++i)
      if (U[i] == u) return off[i];
    return 0;
  }
};

Packs plan_packs(const gift_layer* layers, int n, Op op) {
  Packs p;
  for (int i = 0; i < n; ++i) {
    if (!whitened(layers[i], op) || layers[i].factor->packs || layers[i].factor->block) continue;
    const float* u = layers[i].factor->U;
    bool seen = false;
    for (const float* v : p.U) seen |= v == u;
    if (seen) continue;
    const int cols = factor_cols(layers[i].factor->rank);
    p.U.push_back(u);
    p.d_in.push_back((int)layers[i].d_in);
    p.cols.push_back(cols);
    p.off.push_back(p.bytes);
    p.bytes += align_up(pack_bytes(layers[i].d_in) * (cols / kRank));
  }
  return p;
}

bool slab_layer(const gift_layer& L, int scaling);

// Descriptors of the slab layers of a whiten call in device memory, after
// the per-layer slices, when there are more than fit inline in a launch.
size_t slab_desc_bytes(const gift_layer* layers, int n, Op op, bool block) {
  if (op != Op::Whiten || block) return 0;
  int k = 0;
  for (int i = 0; i < n; ++i) k += slab_layer(layers[i], GIFT_SCALE_TENSOR);
  return k > kMaxGroup ? align_up((size_t)k * sizeof(LayerDev)) : 0;
}

size_t group_ws(const gift_layer* layers, int n, Op op, bool block) {
  size_t t = plan_packs(layers, n, op).bytes;
  for (int i = 0; i < n; ++i) t += layer_ws(layers[i], op, block).total();
  return t + slab_desc_bytes(layers, n, op, block);
}

// One pack launch entry per rank block: U's block b starts at column 32 b,
// its packs at b * pack_bytes(d_in).
gift_status launch_factor_packs(const std::vector<PackDev>& blocks, hipStream_t st) {
  PackGroup pg{};
  for (size_t i = 0; i < blocks.size(); ++i) {
    pg.f[pg.n++] = blocks[i];
    if (pg.n == kMaxGroup || i + 1 == blocks.size()) {
      hipError_t e = launch_pack(pg, st);
      if (e != hipSuccess) return hip_fail(e, "pack launch");
      pg.n = 0;
    }
  }
  return GIFT_OK;
}

void add_pack_blocks(std::vector<PackDev>& out, const float* U, uint4* P, int d_in, int cols) {
  for (int b = 0; b < cols / kRank; ++b) {
    PackDev d{};
    d.U = U + kRank * b;
    d.P = P + b * pack_bytes(d_in) / sizeof(uint4);
    d.d_in = d_in;
    d.ucols = cols;
    out.push_back(d);
  }
}

gift_status run_packs(const Packs& p, void* ws, hipStream_t st) {
  std::vector<PackDev> blocks;
  for (size_t i = 0; i < p.U.size(); ++i)
    add_pack_blocks(blocks, p.U[i], reinterpret_cast<uint4*>((char*)ws + p.off[i]), p.d_in[i],
                    p.cols[i]);
  return launch_factor_packs(blocks, st);
}

gift_status check_layers(const gift_layer* layers, int n, Op op, int scaling) {
  if (n < 0) return fail(GIFT_ERR_INVALID_ARG, "n_layers < 0");
  if (n > 0 && !layers) return fail(GIFT_ERR_INVALID_ARG, "layers is NULL");
  if (scaling != GIFT_SCALE_TENSOR && scaling != GIFT_SCALE_BLOCK128 &&
      scaling != GIFT_SCALE_MXFP4)
    return fail(GIFT_ERR_INVALID_ARG, "unknown scaling %d", scaling);
  for (int i = 0; i < n; ++i) {
    const gift_layer& L = layers[i];
    if (L.d_out < 1 || L.d_in < 1 || L.d_out > kMaxDim || L.d_in > kMaxDim ||
        L.d_out * L.d_in > kMaxElems)
      return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: d_out=%lld d_in=%lld out of range", i,
                  (long long)L.d_out, (long long)L.d_in);
    if (L.d_in % 4)
      return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: d_in %% 4 != 0", i);
    if (scaling == GIFT_SCALE_BLOCK128 && L.d_in % kBlock)
      return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: block scaling needs d_in %% 128 == 0", i);
    if (scaling == GIFT_SCALE_MXFP4 && L.d_in % kMxBlock)
      return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: MXFP4 needs d_in %% 32 == 0", i);
    const bool need_g = op == Op::Whiten || op == Op::Euclid || op == Op::Error;
    const bool need_q = op != Op::Error && op != Op::UnwhitenF32;
    const bool need_ghat = op != Op::Whiten;
    if ((need_g && !L.G) || (need_q && (!L.q || !L.inv_scale)) || (need_ghat && !L.G_hat))
      return fail(GIFT_ERR_INVALID_ARG, "layer %d: a required tensor pointer is NULL", i);
    if (!aligned16(L.G) || !aligned16(L.q) || !aligned16(L.inv_scale) || !aligned16(L.G_hat) ||
        !aligned16(L.W_out))
      return fail(GIFT_ERR_INVALID_ARG, "layer %d: device pointers must be 16-byte aligned", i);
    if (L.factor && L.factor->block) {
      const gift_factor& f = *L.factor;
      if (op == Op::UnwhitenF32)
        return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: block factors are not taken here", i);
      if (whitened(L, op)) {
        if (f.block != 32 && f.block != 64)
          return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: factor block %d not 32 or 64", i, f.block);
        if (scaling == GIFT_SCALE_MXFP4)
          return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: block factors take no MXFP4", i);
        if (f.d_in != L.d_in)
          return fail(GIFT_ERR_INVALID_ARG, "layer %d: factor d_in %d != layer d_in %lld", i,
                      f.d_in, (long long)L.d_in);
        if (L.d_in % f.block)
          return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: d_in %% block != 0", i);
        if (!f.packs || !aligned16(f.packs))
          return fail(GIFT_ERR_INVALID_ARG, "layer %d: block factor packs NULL or misaligned", i);
      }
    } else if (whitened(L, op)) {
      const gift_factor& f = *L.factor;
      if (f.rank < 1 || f.rank > kMaxRank)
        return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: factor rank %d not in [1, %d]", i, f.rank,
                    kMaxRank);
      if (f.d_in != L.d_in)
        return fail(GIFT_ERR_INVALID_ARG, "layer %d: factor d_in %d != layer d_in %lld", i,
                    f.d_in, (long long)L.d_in);
      if (L.d_in < 64 || L.d_in % 32)
        return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "layer %d: whitening needs d_in >= 64, %% 32 == 0",
                    i);
      if (!f.U || !f.coef || !aligned16(f.U) || !aligned16(f.coef) || !aligned16(f.packs))
        return fail(GIFT_ERR_INVALID_ARG, "layer %d: factor U/coef NULL or misaligned", i);
    }
  }
  return GIFT_OK;
}

// Groups below this many whitened gradient elements (about 2048 tiles of 64
// rows) run the 32-row tile kernels: with twice the workgroups, the last
// round of workgroups on the machine is shorter.
constexpr int64_t kSmallGroupElems = int64_t(1) << 25;

// Rank-r whitened layers of at least this many elements, with per-tensor
// scaling, whiten as slabs (one workgroup per 64-row block: no partial
// buffer, no reduction launch), then quantize on the 64-row tile kernels.
// The choice depends on the layer alone, so a layer's results do not depend
// on the group it is called with.
constexpr int64_t kSlabMinElems = int64_t(1) << 22;

bool slab_layer(const gift_layer& L, int scaling) {
  return L.factor && !L.factor->block && L.factor->rank <= kRank && scaling == GIFT_SCALE_TENSOR &&
         L.d_out * L.d_in >= kSlabMinElems;
}

const TileOps& tile_ops(const gift_layer* layers, int n, Op op) {
  int64_t e = 0;
  for (int i = 0; i < n; ++i)
    if (whitened(layers[i], op)) e += layers[i].d_out * layers[i].d_in;
  return e < kSmallGroupElems ? kTiles32 : kTiles64;
}

// Walk the layers selected by `pick` in chunks of kMaxGroup, filling the
// descriptors (workspace slices in layer order) and calling `launch` per
// chunk.  slab: the layers whiten as slabs; k_slab_whiten first runs once
// over all of them (descriptors past kMaxGroup in device memory, after the
// per-layer slices), then `launch` quantizes chunk by chunk.
template <class Pick, class Tiles, class Launch>
gift_status run_grouped(const gift_layer* layers, int n, Op op, bool block, void* ws,
                        uint32_t* flags, double* out, Pick pick, Tiles tiles, Launch launch,
                        const TileOps& geo = kTiles64, bool slab = false,
                        hipStream_t st = nullptr) {
  // workspace: operand packs first, then per-layer slices in layer order
  // (independent of the chunking)
  const Packs packs = plan_packs(layers, n, op);
  std::vector<size_t> off(n + 1, packs.bytes);
  for (int i = 0; i < n; ++i) off[i + 1] = off[i] + layer_ws(layers[i], op, block).total();
  std::vector<LayerDev> all;
  std::vector<int> index;  // call position of each picked layer
  int64_t tiles_all = 0, rb_all = 0;
  for (int i = 0; i < n; ++i) {
    const gift_layer& L = layers[i];
    if (!pick(L)) continue;
    LayerWs lw = layer_ws(L, op, block);
    char* base = (char*)ws + off[i];
    LayerDev d{};
    d.G = op == Op::UnwhitenF32 ? L.G_hat : L.G;
    d.q = L.q;
    d.inv = L.inv_scale;
    d.Ghat = L.G_hat;
    d.Wout = L.W_out;
    if (whitened(L, op)) {
      d.U = L.factor->U;
      d.coef = L.factor->coef;
      d.P = L.factor->packs ? static_cast<const uint4*>(L.factor->packs)
                            : reinterpret_cast<const uint4*>((char*)ws + packs.find(L.factor->U));
    }
    d.cbuf = lw.cbuf ? (float*)base : nullptr;
    base += align_up(lw.cbuf);
    d.cfin = lw.cfin ? (float*)base : nullptr;
    base += align_up(lw.cfin);
    d.part = lw.part ? (uint32_t*)base : nullptr;
    base += align_up(lw.part);
    d.part2 = lw.part2 ? (double*)base : nullptr;
    base += align_up(lw.part2);
    d.amax = lw.amax ? (uint32_t*)base : nullptr;
    d.d_out = L.d_out;
    d.d_in = L.d_in;
    d.n_rb = geo.row_blocks(L.d_out);
    d.ngrp = !whitened(L, op) ? 1 : fblock(L) ? blk_col_groups(L.d_in, fblock(L)) : col_groups(L.d_in);
    d.n_tiles = tiles(L);
    d.n_part = slab ? (int)d.n_rb : d.n_tiles;  // one amax partial per row block or per tile
    d.tile_begin = (int)tiles_all;
    tiles_all += d.n_tiles;
    d.rb_begin = (int)rb_all;
    if (whitened(L, op)) rb_all += d.n_rb;
    all.push_back(d);
    index.push_back(i);
  }
  if (all.empty()) return GIFT_OK;
  GroupDev g{};
  g.flags = flags;
  g.out = out;
  if (slab) {  // the slab pass over all layers at once
    if (rb_all > INT32_MAX) return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "too many row blocks in one call");
    GroupDev ga = g;
    ga.n = (int)all.size();
    ga.total_rb = (int)rb_all;
    if (ga.n <= kMaxGroup) {
      for (int k = 0; k < ga.n; ++k) ga.L[k] = all[k];
    } else {
      LayerDev* dst = reinterpret_cast<LayerDev*>((char*)ws + off[n]);
      hipError_t e = rt4::launch_put_layers(all.data(), ga.n, dst, st);
      if (e != hipSuccess) return hip_fail(e, "kernel launch");
      ga.Lx = dst;
    }
    hipError_t e = rt4::launch_slab_whiten(ga, st);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
  }
  // chunks of kMaxGroup layers with inline descriptors, tiles and row blocks
  // counted from each chunk's start
  for (size_t c0 = 0; c0 < all.size(); c0 += kMaxGroup) {
    const size_t c1 = all.size() - c0 < (size_t)kMaxGroup ? all.size() : c0 + kMaxGroup;
    g.n = 0;
    g.total_tiles = 0;
    g.total_rb = 0;
    for (size_t k = c0; k < c1; ++k) {
      LayerDev& d = g.L[g.n++];
      d = all[k];
      d.tile_begin = g.total_tiles;
      g.total_tiles += d.n_tiles;
      d.rb_begin = g.total_rb;
      if (whitened(layers[index[k]], op)) g.total_rb += (int)d.n_rb;
    }
    hipError_t e = launch(g, index[c0]);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
  }
  return GIFT_OK;
}

int tiles_flat(const gift_layer& L) { return flat_tiles(L.d_out * L.d_in); }

gift_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(GIFT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need && !ws) return fail(GIFT_ERR_INVALID_ARG, "workspace is NULL");
  if (ws && ((uintptr_t)ws % kAlign))
    return fail(GIFT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return GIFT_OK;
}

// Scratch of gift_whiten_quantize_static: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address: each device's copy is found once with
// hipGetSymbolAddress (with that device current) and kept in
// g_scratch_ptr.  The whiten kernels need nothing in it zeroed: every word
// they read there was written earlier in the same call.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

gift_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "device %d: the static scratch serves devices 0..%d",
                dev, kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p % kAlign))
      return fail(GIFT_ERR_HIP, "static scratch of device %d is not 256-byte aligned", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GIFT_OK;
}

}  // namespace

extern "C" {

int gift_abi_version(void) { return GIFT_ABI_VERSION; }

#ifndef GIFT_BUILD_HASH
#define GIFT_BUILD_HASH "unknown"
#endif
const char* gift_build_hash(void) { return GIFT_BUILD_HASH; }

const char* gift_last_error(void) { return t_err.c_str(); }

const char* gift_status_string(int s) {
  switch (s) {
    case GIFT_OK: return "GIFT_OK";
    case GIFT_ERR_INVALID_ARG: return "GIFT_ERR_INVALID_ARG";
    case GIFT_ERR_UNSUPPORTED_SHAPE: return "GIFT_ERR_UNSUPPORTED_SHAPE";
    case GIFT_ERR_WORKSPACE_TOO_SMALL: return "GIFT_ERR_WORKSPACE_TOO_SMALL";
    case GIFT_ERR_HIP: return "GIFT_ERR_HIP";
    default: return "GIFT_ERR_UNKNOWN";
  }
}

size_t gift_group_workspace_bytes(int op, const gift_layer* layers, int n_layers, int scaling) {
  if (n_layers <= 0 || !layers) return 0;
  const bool block = scaling != GIFT_SCALE_TENSOR;  // no per-tensor amax
  switch (op) {
    case GIFT_OP_WHITEN_QUANTIZE: return group_ws(layers, n_layers, Op::Whiten, block);
    case GIFT_OP_DEQUANT_UNWHITEN: return group_ws(layers, n_layers, Op::Dequant, block);
    case GIFT_OP_EUCLID_ROUNDTRIP: return group_ws(layers, n_layers, Op::Euclid, block);
    case GIFT_OP_ROUNDTRIP_ERROR: return group_ws(layers, n_layers, Op::Error, false);
    case GIFT_OP_UNWHITEN_F32: return group_ws(layers, n_layers, Op::UnwhitenF32, true);
    default: return 0;
  }
}

gift_status gift_whiten_quantize(const gift_layer* layers, int n_layers, int scaling,
                                 uint32_t* dev_flags, void* ws, size_t ws_bytes, void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Whiten, scaling);
  if (s != GIFT_OK) return s;
  const bool block = scaling != GIFT_SCALE_TENSOR;  // no per-tensor amax
  s = check_ws(ws, ws_bytes, group_ws(layers, n_layers, Op::Whiten, block));
  if (s != GIFT_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  s = run_packs(plan_packs(layers, n_layers, Op::Whiten), ws, st);
  if (s != GIFT_OK) return s;
  const TileOps& geo = tile_ops(layers, n_layers, Op::Whiten);
  // groups: rank-r factors of one rank block on tiles, Euclidean layers,
  // block factors of 32, of 64, rank-r factors as slabs, rank-r factors of
  // two rank blocks on tiles
  for (int wgrp = 0; wgrp < 6; ++wgrp) {
    auto pick = [&](const gift_layer& L) {
      const bool rankr = L.factor != nullptr && !L.factor->block;
      return wgrp == 0 ? rankr && frb(L) == 1 && !slab_layer(L, scaling)
           : wgrp == 1 ? L.factor == nullptr
           : wgrp == 4 ? slab_layer(L, scaling)
           : wgrp == 5 ? rankr && frb(L) == 2
                       : fblock(L) == (wgrp == 2 ? 32 : 64);
    };
    bool any_w = false;
    for (int i = 0; i < n_layers; ++i)
      if (pick(layers[i]) && layers[i].W_out) any_w = true;
    auto tiles_rows = [&](const gift_layer& L) { return row_tiles(L, geo); };
    if (wgrp == 0 || wgrp == 5)
      s = run_grouped(layers, n_layers, Op::Whiten, block, ws, dev_flags, nullptr, pick,
                      tiles_rows, [&](const GroupDev& g, int) {
                        return geo.whiten_quantize(g, scaling, any_w, st, wgrp == 5 ? 2 : 1);
                      }, geo);
    else if (wgrp == 1)
      s = run_grouped(layers, n_layers, Op::Whiten, block, ws, dev_flags, nullptr, pick,
                      tiles_flat, [&](const GroupDev& g, int) {
                        return launch_flat_quantize(g, scaling, false, any_w, st);
                      });
    else if (wgrp == 4)
      s = run_grouped(layers, n_layers, Op::Whiten, block, ws, dev_flags, nullptr, pick,
                      [&](const gift_layer& L) { return row_tiles(L, kTiles64); },
                      [&](const GroupDev& g, int) {
                        return rt4::launch_slab_quantize(g, any_w, st);
                      }, kTiles64, true, st);
    else
      s = run_grouped(layers, n_layers, Op::Whiten, block, ws, dev_flags, nullptr, pick,
                      tiles_rows, [&](const GroupDev& g, int) {
                        return geo.blk_whiten(g, wgrp == 2 ? 32 : 64, scaling, any_w, st);
                      }, geo);
    if (s != GIFT_OK) return s;
  }
  return GIFT_OK;
}

size_t gift_static_scratch_bytes(void) { return kScratchBytes; }

gift_status gift_whiten_quantize_static(const gift_layer* layers, int n_layers, int scaling,
                                        uint32_t* dev_flags, void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Whiten, scaling);
  if (s != GIFT_OK) return s;
  const size_t need = group_ws(layers, n_layers, Op::Whiten, scaling != GIFT_SCALE_TENSOR);
  if (need > kScratchBytes)
    return fail(GIFT_ERR_WORKSPACE_TOO_SMALL,
                "gift_whiten_quantize_static: the call needs %zu bytes of scratch, more than the "
                "%zu of the static array; split the group or call gift_whiten_quantize",
                need, kScratchBytes);
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != GIFT_OK) return s;
  return gift_whiten_quantize(layers, n_layers, scaling, dev_flags, ws, kScratchBytes, stream);
}

gift_status gift_dequant_unwhiten(const gift_layer* layers, int n_layers, int scaling, void* ws,
                                  size_t ws_bytes, void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Dequant, scaling);
  if (s != GIFT_OK) return s;
  const bool block = scaling != GIFT_SCALE_TENSOR;
  s = check_ws(ws, ws_bytes, group_ws(layers, n_layers, Op::Dequant, block));
  if (s != GIFT_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  s = run_packs(plan_packs(layers, n_layers, Op::Dequant), ws, st);
  if (s != GIFT_OK) return s;
  const TileOps& geo = tile_ops(layers, n_layers, Op::Dequant);
  // groups: rank-r factors of one rank block, Euclidean layers, block
  // factors of 32, of 64, rank-r factors of two rank blocks
  for (int wgrp = 0; wgrp < 5; ++wgrp) {
    auto pick = [&](const gift_layer& L) {
      const bool rankr = L.factor != nullptr && !L.factor->block;
      return wgrp == 0 ? rankr && frb(L) == 1
           : wgrp == 1 ? L.factor == nullptr
           : wgrp == 4 ? rankr && frb(L) == 2
                       : fblock(L) == (wgrp == 2 ? 32 : 64);
    };
    auto tiles = [&](const gift_layer& L) { return wgrp == 1 ? tiles_flat(L) : row_tiles(L, geo); };
    s = run_grouped(layers, n_layers, Op::Dequant, block, ws, nullptr, nullptr, pick, tiles,
                    [&](const GroupDev& g, int) {
                      if (wgrp == 2 || wgrp == 3)
                        return geo.blk_dequant(g, wgrp == 2 ? 32 : 64, scaling, st);
                      return geo.dequant(g, scaling, wgrp != 1, st, wgrp == 4 ? 2 : 1);
                    }, geo);
    if (s != GIFT_OK) return s;
  }
  return GIFT_OK;
}

gift_status gift_euclid_fp8_roundtrip(const gift_layer* layers, int n_layers, int scaling,
                                      uint32_t* dev_flags, void* ws, size_t ws_bytes,
                                      void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Euclid, scaling);
  if (s != GIFT_OK) return s;
  const bool block = scaling != GIFT_SCALE_TENSOR;
  s = check_ws(ws, ws_bytes, group_ws(layers, n_layers, Op::Euclid, block));
  if (s != GIFT_OK) return s;
  bool any_w = false;
  for (int i = 0; i < n_layers; ++i) any_w |= layers[i].W_out != nullptr;
  hipStream_t st = (hipStream_t)stream;
  return run_grouped(layers, n_layers, Op::Euclid, block, ws, dev_flags, nullptr,
                     [](const gift_layer&) { return true; }, tiles_flat,
                     [&](const GroupDev& g, int) {
                       return launch_flat_quantize(g, scaling, true, any_w, st);
                     });
}

gift_status gift_roundtrip_error(const gift_layer* layers, int n_layers, double* dev_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Error, GIFT_SCALE_TENSOR);
  if (s != GIFT_OK) return s;
  if (n_layers > 0 && (!dev_out || ((uintptr_t)dev_out & 7u)))
    return fail(GIFT_ERR_INVALID_ARG, "dev_out NULL or not 8-byte aligned");
  s = check_ws(ws, ws_bytes, group_ws(layers, n_layers, Op::Error, false));
  if (s != GIFT_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  return run_grouped(layers, n_layers, Op::Error, false, ws, nullptr, dev_out,
                     [](const gift_layer&) { return true; }, tiles_flat,
                     [&](const GroupDev& g, int first) { return launch_error(g, first, st); });
}

gift_status gift_dequant_accumulate(const gift_layer* layers, int n_layers, int scaling,
                                    int first, void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::Accumulate, scaling);
  if (s != GIFT_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  return run_grouped(layers, n_layers, Op::Accumulate, true, nullptr, nullptr, nullptr,
                     [](const gift_layer&) { return true; }, tiles_flat,
                     [&](const GroupDev& g, int) {
                       return launch_accumulate(g, scaling, first != 0, st);
                     });
}

gift_status gift_unwhiten_f32(const gift_layer* layers, int n_layers, void* ws, size_t ws_bytes,
                              void* stream) {
  gift_status s = check_layers(layers, n_layers, Op::UnwhitenF32, GIFT_SCALE_TENSOR);
  if (s != GIFT_OK) return s;
  s = check_ws(ws, ws_bytes, group_ws(layers, n_layers, Op::UnwhitenF32, true));
  if (s != GIFT_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  s = run_packs(plan_packs(layers, n_layers, Op::UnwhitenF32), ws, st);
  if (s != GIFT_OK) return s;
  const TileOps& geo = tile_ops(layers, n_layers, Op::UnwhitenF32);
  auto tiles = [&](const gift_layer& L) { return row_tiles(L, geo); };
  for (int rb = 1; rb <= 2; ++rb) {
    auto pick = [&](const gift_layer& L) { return L.factor != nullptr && frb(L) == rb; };
    s = run_grouped(layers, n_layers, Op::UnwhitenF32, true, ws, nullptr, nullptr, pick, tiles,
                    [&](const GroupDev& g, int) { return geo.unwhiten_f32(g, st, rb); }, geo);
    if (s != GIFT_OK) return s;
  }
  return GIFT_OK;
}

size_t gift_refresh_workspace_bytes(int64_t d_in, int64_t n_tokens, int x_dtype,
                                    int sketch_width) {
  return refresh_workspace_bytes(d_in, n_tokens, x_dtype, sketch_width);
}

gift_status gift_refresh_factor(const void* X, int x_dtype, int64_t n_tokens,
                                const gift_factor* f, float damp_eps, int damping_mode,
                                int sketch_width, int power_steps, uint64_t seed,
                                const float* sketch, float* A_out, uint32_t* dev_flags, void* ws,
                                size_t ws_bytes, void* stream) {
  return refresh_factor(X, x_dtype, n_tokens, f, damp_eps, damping_mode, sketch_width,
                        power_steps, seed, sketch, A_out, dev_flags, ws, ws_bytes,
                        (hipStream_t)stream, &t_err);
}

size_t gift_factor_pack_bytes(int64_t d_in) { return d_in > 0 ? pack_bytes(d_in) : 0; }

size_t gift_factor_pack_bytes_rank(int64_t d_in, int rank) {
  if (d_in <= 0 || rank < 1 || rank > kMaxRank) return 0;
  return pack_bytes(d_in) * (factor_cols(rank) / kRank);
}

size_t gift_block_factor_pack_bytes(int64_t d_in, int block) {
  if ((block != 32 && block != 64) || d_in < block || d_in % block) return 0;
  return blk_pack_bytes(d_in, block);
}

gift_status gift_prepare_factor(const gift_factor* f, void* stream) {
  if (!f || !f->U || !f->packs) return fail(GIFT_ERR_INVALID_ARG, "factor, U or packs is NULL");
  if (!aligned16(f->U) || !aligned16(f->packs))
    return fail(GIFT_ERR_INVALID_ARG, "U / packs must be 16-byte aligned");
  if (f->block) {
    if ((f->block != 32 && f->block != 64) || f->d_in < f->block || f->d_in % f->block ||
        f->d_in > kMaxDim)
      return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "block must be 32 or 64 and divide d_in");
    PackGroup pg{};
    pg.n = 1;
    pg.f[0].U = f->U;
    pg.f[0].P = static_cast<uint4*>(f->packs);
    pg.f[0].d_in = f->d_in;
    hipError_t e = launch_blk_pack(pg, f->block, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    return GIFT_OK;
  }
  if (f->rank < 1 || f->rank > kMaxRank)
    return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "rank must be in [1, 64]");
  if (f->d_in < 64 || f->d_in % 32 || f->d_in > kMaxDim)
    return fail(GIFT_ERR_UNSUPPORTED_SHAPE, "d_in must be >= 64 and a multiple of 32");
  std::vector<PackDev> blocks;
  add_pack_blocks(blocks, f->U, static_cast<uint4*>(f->packs), f->d_in, factor_cols(f->rank));
  return launch_factor_packs(blocks, (hipStream_t)stream);
}

gift_status gift_refresh_factors(const gift_refresh_input* inputs, int n, float damp_eps,
                                 int damping_mode, int sketch_width, int power_steps,
                                 uint32_t* dev_flags, void* ws, size_t ws_bytes, void* stream) {
  return refresh_factors(inputs, n, damp_eps, damping_mode, sketch_width, power_steps, dev_flags,
                         ws, ws_bytes, (hipStream_t)stream, &t_err);
}

size_t gift_refresh_group_workspace_bytes(const gift_refresh_input* inputs, int n,
                                          int sketch_width) {
  if (!inputs || n <= 0) return 0;
  return refresh_group_workspace_bytes(inputs, n, sketch_width);
}

gift_status gift_draw_sketch(float* out, int64_t d_in, int width, uint64_t seed, void* stream) {
  return draw_sketch(out, d_in, width, seed, (hipStream_t)stream, &t_err);
}

}  // extern "C"
