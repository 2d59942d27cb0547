// Per-workgroup problem resolution shared by the attention kernels:
// sequence extents (batch or group mode), tensor base pointers, the dropout
// key, and small wave-level helpers for the fp32 path.
#pragma once
#include "sdpa_device.h"
#include "sdpa_params.h"

namespace sdpa {

struct SeqPos {
  int64_t qtok, ktok;  // first token of this sequence (0 in batch mode)
  int32_t sq, skv;     // this sequence's lengths
  int64_t bsel;        // batch index to multiply batch strides by (0 in group mode)
};

__device__ __forceinline__ SeqPos resolve_seq(const SeqInfo& s, int b) {
  SeqPos p;
  if (s.cu_q) {
    p.qtok = s.cu_q[b];
    p.sq = s.cu_q[b + 1] - (int32_t)p.qtok;
    p.ktok = s.cu_kv[b];
    p.skv = s.cu_kv[b + 1] - (int32_t)p.ktok;
    p.bsel = 0;
  } else {
    p.qtok = 0; p.ktok = 0;
    p.sq = s.s_q; p.skv = s.s_kv;
    p.bsel = b;
  }
  return p;
}

template <typename T>
__device__ __forceinline__ const T* base_ptr(const void* p, const Str& s, const SeqPos& sp,
                                             int h, bool is_q) {
  return (const T*)p + sp.bsel * s.b + (int64_t)h * s.h + (is_q ? sp.qtok : sp.ktok) * s.s;
}
template <typename T>
__device__ __forceinline__ T* base_ptr_mut(void* p, const Str& s, const SeqPos& sp, int h,
                                           bool is_q) {
  return (T*)p + sp.bsel * s.b + (int64_t)h * s.h + (is_q ? sp.qtok : sp.ktok) * s.s;
}

// Group mode: rows per head of the caller's LSE [h, rows] (the packed query
// length, or cu_q[B] when the caller gave none).  0 in batch mode.
__device__ __forceinline__ int64_t lse_group_rows(const SeqInfo& s, int B) {
  if (!s.cu_q) return 0;
  return s.t_q > 0 ? s.t_q : (int64_t)s.cu_q[B];
}

// Index of row 0 of (b, h) in a dense per-row fp32 array:
//   batch mode [B,H,S_q]; group mode [H, T] with T = `group_rows`.
__device__ __forceinline__ int64_t row_stat_base(const SeqInfo& s, const SeqPos& sp, int b,
                                                 int h, int H, int64_t group_rows) {
  if (s.cu_q) return (int64_t)h * group_rows + sp.qtok;
  return ((int64_t)b * H + h) * s.s_q;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2, and each XCD starts its workgroups in increasing id order.  The tile
// kernels use a 1-D grid in which XCD x = id mod 8 owns a contiguous range
// of (batch, head) pairs, so every tile of a head - which all read the same
// K/V (or Q/dO) - runs behind one L2.  Within an XCD the heads go in groups
// of G, and within a group the tiles are ordered rank-major: rank r of every
// head of the group before rank r + 1.  The kernels number ranks heaviest
// first under a causal mask, so this is largest-first list scheduling over
// the XCD's compute units (head-major order starts the last heads' heaviest
// tiles last and leaves the machine idle at the end), while G bounds how
// many heads' tiles share the L2 at a time.  Any bijection is correct; this
// one only changes placement and order.
//
// In group mode the sequences differ in length, and causal work grows with
// the square of the length, so (batch, head) ranges that hold all heads of a
// few sequences load the XCDs unevenly (1.7x the mean on the busiest XCD for
// 16 lengths drawn from U[64, 4096]).  There the pairs are enumerated
// head-major (`hmajor`): every XCD gets the same heads of every sequence,
// which carry equal work.
struct WorkItem {
  int b, h, tile;
  bool valid;
};
// the item of position `id` of that grid (id = blockIdx.x, or a position a
// persistent workgroup takes on)
__device__ __forceinline__ WorkItem xcd_work_at(int id, int ntiles, int H, int B, int G, bool hmajor) {
  const int BH = B * H;
  const int x = id & 7, pos = id >> 3;
  const int h_lo = (int)((int64_t)x * BH / 8);
  const int nh = (int)((int64_t)(x + 1) * BH / 8) - h_lo;  // heads owned by XCD x
  WorkItem wi;
  wi.valid = nh > 0 && pos < nh * ntiles;
  const int gi = pos / (G * ntiles);           // head group
  const int off = pos - gi * G * ntiles;
  const int gsz = max(1, min(G, nh - gi * G));  // the last group may be smaller
  const int r = off / gsz;
  const int hb = h_lo + gi * G + (off - r * gsz);
  wi.tile = r;
  if (hmajor) {
    wi.h = hb / B;
    wi.b = hb - wi.h * B;
  } else {
    wi.b = hb / H;
    wi.h = hb - wi.b * H;
  }
  return wi;
}
__device__ __forceinline__ WorkItem xcd_work(int ntiles, int H, int B, int G, bool hmajor = false) {
  return xcd_work_at((int)blockIdx.x, ntiles, H, B, G, hmajor);
}
inline dim3 xcd_grid(int ntiles, int H, int B) {
  const long BH = (long)B * H;
  return dim3((unsigned)(8 * ((BH + 7) / 8) * ntiles), 1, 1);
}

// The band of a sequence: key j is visible from row i iff
// lo <= j - i <= hi (the mask's lo/hi shifted by the bottom-right offset
// s_kv - s_q when br is set), clamped to +-kBandInf.
struct Band {
  int32_t lo, hi;
};
__device__ __forceinline__ Band seq_band(int32_t br, int32_t lo, int32_t hi, int sq, int skv) {
  const int64_t off = br ? (int64_t)skv - sq : 0;
  const int64_t l = off + lo, h = off + hi;
  Band b;
  b.lo = (int32_t)(l < -kBandInf ? -kBandInf : (l > kBandInf ? kBandInf : l));
  b.hi = (int32_t)(h < -kBandInf ? -kBandInf : (h > kBandInf ? kBandInf : h));
  return b;
}

// A lane's visible range within a tile, for masks applied to elements at
// compile-time offsets o (0 <= o < 2^20) from a per-lane base index: the
// element at base + o is visible iff first <= base + o <= last (absolute,
// inclusive), tested as one unsigned compare instead of a chain of
// short-circuit branches.  An empty range never matches.
struct TileWindow {
  int32_t first;  // first visible offset, clamped to [0, 2^20]
  uint32_t span;  // last - first, last clamped to 2^20
  __device__ __forceinline__ bool has(int o) const { return (uint32_t)(o - first) <= span; }
};
__device__ __forceinline__ TileWindow tile_window(int64_t first_abs, int64_t last_abs, int64_t base) {
  constexpr int64_t kOffMax = 1 << 20;
  int64_t f = first_abs - base, l = last_abs - base;
  f = f < 0 ? 0 : f;
  l = l > kOffMax ? kOffMax : l;
  TileWindow w;
  if (l < f) {  // empty (or wholly outside [0, 2^20])
    w.first = (int32_t)(2 * kOffMax);
    w.span = 0;
  } else {
    w.first = (int32_t)f;
    w.span = (uint32_t)(l - f);
  }
  return w;
}
// Keys visible from row `row` (band mask and sequence end): [first, last].
// (The row is made opaque so that the window is formed where it is used,
// not hoisted out of the tile loop into registers held across it.)
__device__ __forceinline__ TileWindow keys_of_row(int row, const Band& bd, bool band, int skv,
                                                  int64_t base) {
  __asm__ volatile("" : "+v"(row));
  const int64_t first = band ? (int64_t)row + bd.lo : 0;
  const int64_t last = band ? min((int64_t)skv - 1, (int64_t)row + bd.hi) : (int64_t)skv - 1;
  return tile_window(first, last, base);
}
// Rows that see key `kv` (band mask and sequence end): [kv - hi, kv - lo].
__device__ __forceinline__ TileWindow rows_of_key(int kv, const Band& bd, bool band, int sq,
                                                  int64_t base) {
  __asm__ volatile("" : "+v"(kv));
  const int64_t first = band ? (int64_t)kv - bd.hi : 0;
  const int64_t last = band ? min((int64_t)sq - 1, (int64_t)kv - bd.lo) : (int64_t)sq - 1;
  return tile_window(first, last, base);
}

// ALiBi of one (sequence, head): the term is slope * |j - i - off|
// (slope already negated), zero slope when there is none.
struct AlibiTerm {
  float slope;
  int32_t off;
};
__device__ __forceinline__ AlibiTerm alibi_term(const float* alibi, int64_t sb, int32_t br, int b,
                                                int h, int sq, int skv) {
  AlibiTerm t;
  t.slope = alibi ? -alibi[(int64_t)b * sb + h] : 0.f;
  t.off = br ? skv - sq : 0;
  return t;
}
__device__ __forceinline__ float alibi_at(const AlibiTerm& t, int kv, int row) {
  return t.slope * fabsf((float)(kv - row - t.off));
}

struct DropKey {
  uint32_t k0, k1, off, thr;
};
__device__ __forceinline__ DropKey drop_key(const DropoutArgs& d) {
  uint64_t seed = d.seed, off = d.offset;
  if (d.seed_offset_dev) {
    seed = d.seed_offset_dev[0];
    off = d.seed_offset_dev[1];
  }
  DropKey k;
  k.k0 = (uint32_t)seed;
  k.k1 = (uint32_t)(seed >> 32);
  k.off = (uint32_t)off;
  k.thr = d.threshold;
  return k;
}

// Keep bit of one element from one Philox call (fp32 path, no sharing).
__device__ __forceinline__ bool keep_one(const DropKey& k, uint32_t bh, int i, int j) {
  uint32_t r[4];
  Philox::block((uint32_t)j >> 2, (uint32_t)i >> 2, bh, k.off, k.k0, k.k1, r);
  uint32_t w = r[i & 3];
  return ((w >> (8 * (j & 3))) & 0xffu) >= k.thr;
}

// Wave-wide sum with every lane receiving lane 0's value (bitwise uniform).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return __shfl(x, 0, 64);
}

template <typename T> __device__ __forceinline__ float ld_elem(const T* p);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_elem<__bf16>(const __bf16* p) {
  return to_f32<__bf16>(*(const uint16_t*)p);
}
template <> __device__ __forceinline__ float ld_elem<_Float16>(const _Float16* p) {
  return to_f32<_Float16>(*(const uint16_t*)p);
}
template <typename T> __device__ __forceinline__ void st_elem(T* p, float v);
template <> __device__ __forceinline__ void st_elem<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_elem<__bf16>(__bf16* p, float v) {
  *(uint16_t*)p = (uint16_t)(pack2<__bf16>(v, 0.f) & 0xffffu);
}
template <> __device__ __forceinline__ void st_elem<_Float16>(_Float16* p, float v) {
  *(uint16_t*)p = (uint16_t)(pack2<_Float16>(v, 0.f) & 0xffffu);
}

}  // namespace sdpa
