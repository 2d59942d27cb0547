// Thin-query forward (decode): few query rows per sequence, long key/value
// sequences, no bias and no dropout.
//
// The same O = softmax(scale * Q K^T, masked) V and natural-log LSE as the
// main forward, organised for the shape where it is bound by streaming K and
// V from HBM rather than by the matrix cores:
//   - the query rows of every query head that shares one key/value head are
//     packed into the same 32-row MFMA tile (oneDNN "SDPA primitive"
//     execute_forward batches a single-query problem over the key/value
//     heads so that several query heads share one workgroup), so K and V are
//     read once per key/value head instead of once per query head;
//   - the key range is split over workgroups (split-KV), so that a handful
//     of (batch, key/value head) pairs still fills the chip; each split
//     writes a normalised partial O and its LSE, and a second kernel merges
//     them with weights exp(LSE_split - LSE);
//   - inside a workgroup the four waves stream disjoint 32-key tiles into
//     their own double-buffered LDS tiles (no workgroup barrier in the
//     loop) and merge their running (max, sum, O) once at the end.  A wave
//     copies its current tile's operands into registers first and at once
//     reuses the buffer for the tile after next, so two tiles per wave are
//     in flight while it computes (the chip needs several MB in flight to
//     cover HBM latency, and LDS only holds two buffers per wave).
// Per 32-key tile a wave computes S^T = K Q^T and O^T += V^T P^T exactly as
// the main forward does (sig-permuted K rows, transposing LDS reads of V),
// with the same base-2 online softmax and lazy rescale.
//
// Q8: K and V arrive as int8 codes with one fp32 scale (and optionally one
// int8 zero point) per token and group of head-dim elements - the grouped
// key / value quantization of the oneDNN micro SDPA host driver.  The
// codes stream into double-buffered int8 staging tiles (half the bytes),
// each lane dequantizes 16-byte chunks, x = (code - zp) * scale, into one
// 16-bit tile per operand, and the tile step above runs unchanged on it.
#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "sdpa_kcommon.h"

namespace sdpa {

// Dequantize one 32-row int8 tile (rows of D bytes, staged with the Lds<D/2>
// layout of 16-bit elements) into a 16-bit tile (Lds<D> layout).  Lane l
// converts 16-byte chunk l & (D/16 - 1) of rows (l / (D/16)) + (64 / (D/16)) u;
// sc[u] / zp[u] are that chunk's scale and zero point.
template <typename T, int D>
__device__ __forceinline__ void dequant_tile(const uint16_t* src, T* dst, const float (&sc)[4],
                                             const int (&zp)[4], int lane) {
  constexpr int CPR = D / 16;  // 16-byte int8 chunks per row
  constexpr int RPU = 64 / CPR;
  static_assert(32 * CPR == 64 * 4, "four chunks per lane");
  const int cc = lane & (CPR - 1);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = lane / CPR + RPU * u;
    const u32x4 raw = lds_load16(lds_addr(src + Lds<D / 2>::off(row, 8 * cc)));
    const float s = sc[u], o = -(float)zp[u] * sc[u];
    uint32_t outw[8];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const uint32_t x = raw[wd];
      float f[4];
#pragma unroll
      for (int by = 0; by < 4; ++by) f[by] = __builtin_fmaf((float)(int8_t)(x >> (8 * by)), s, o);
      outw[2 * wd] = pack2<T>(f[0], f[1]);
      outw[2 * wd + 1] = pack2<T>(f[2], f[3]);
    }
    *(u32x4*)(dst + Lds<D>::off(row, 16 * cc)) = u32x4{outw[0], outw[1], outw[2], outw[3]};
    *(u32x4*)(dst + Lds<D>::off(row, 16 * cc + 8)) = u32x4{outw[4], outw[5], outw[6], outw[7]};
  }
}

// A 32-row tile of 4-bit codes (rows of D/2 bytes, two codes per byte, low
// nibble first), staged row-major without swizzle, dequantized into a
// 16-bit tile (Lds<D> layout).  Lane l converts 16-byte chunk l % (D/32)
// (32 codes) of rows l / (D/32) + (64 / (D/32)) u, u = 0, 1; sc[u] / zp[u]
// are that chunk's scale and zero point (one group per chunk: g >= 32).
template <typename T, int D, bool SIGNED>
__device__ __forceinline__ void dequant_tile4(const uint8_t* src, T* dst, const float (&sc)[4],
                                              const int (&zp)[4], int lane) {
  constexpr int LPR = D / 32;  // lanes (16-byte chunks) per row
  constexpr int RSTEP = 64 / LPR;
  const int cc = lane % LPR;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = lane / LPR + RSTEP * u;
    const u32x4 raw = lds_load16(lds_addr(src + (D / 2) * row + 16 * cc));
    const float s = sc[u], o = -(float)zp[u] * sc[u];
    uint32_t outw[16];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const uint32_t x = raw[wd];
      float f[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int code = SIGNED ? ((int)(x << (28 - 4 * k)) >> 28) : (int)((x >> (4 * k)) & 15u);
        f[k] = __builtin_fmaf((float)code, s, o);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) outw[4 * wd + k] = pack2<T>(f[2 * k], f[2 * k + 1]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(u32x4*)(dst + Lds<D>::off(row, 32 * cc + 8 * q)) =
          u32x4{outw[4 * q], outw[4 * q + 1], outw[4 * q + 2], outw[4 * q + 3]};
  }
}

// Direct-to-LDS loads of a 32-row tile of 4-bit codes (rows of D/2 bytes)
// into a row-major, unswizzled staging tile: 16-byte chunk c of the tile is
// row c / (D/32), column chunk c % (D/32), at LDS byte 16 c; with one wave,
// lane l loads chunks l + 64 j.  Rows past row_limit are clamped (masked by
// the caller), as in TileLoader.
template <int D> struct Int4TileLoader {
  static constexpr int CPR = D / 32;  // 16-byte chunks per row
  static constexpr int PER_WAVE = 32 * CPR / 64;
  static_assert(32 * CPR % 64 == 0, "whole wave loads");
  const char* g;
  int64_t stride_b;
  uint32_t voff[PER_WAVE];
  __device__ __forceinline__ void init(const void* g_, int64_t row_stride_bytes, int, int lane) {
    g = (const char*)g_;
    stride_b = row_stride_bytes;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int c = 64 * j + lane;
      voff[j] = (uint32_t)((c / CPR) * stride_b + 16 * (c % CPR));
    }
  }
  __device__ __forceinline__ void load(void* tile, int row0, int row_limit, int, int lane) const {
    if (row0 + 32 <= row_limit) {
      const char* base = g + row0 * stride_b;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(base + voff[j]),
                                         (lds_void*)((char*)tile + 1024 * j), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int c = 64 * j + lane;
        const int gr = min(row0 + c / CPR, row_limit - 1);
        __builtin_amdgcn_global_load_lds((const void*)(g + gr * stride_b + 16 * (c % CPR)),
                                         (lds_void*)((char*)tile + 1024 * j), 16, 0, 0);
      }
    }
  }
};

// QM: 0 = 16-bit K/V; quantized K/V with scales: 1 = int8, 3 = signed
// 4-bit, 5 = unsigned 4-bit; 2, 4, 6: the same with zero points
template <typename T, int DQK, int DV, bool BAND, int QM>
__global__ void __launch_bounds__(256, 1) fwd_decode(const FwdArgs a, const DecodeArgs d) {
  constexpr bool Q8 = QM != 0;     // quantized K/V (8- or 4-bit codes)
  constexpr bool Q4 = QM >= 3;     // 4-bit codes
  constexpr bool QZP = QM == 2 || QM == 4 || QM == 6;
  constexpr int BC = 32;        // keys per wave tile
  constexpr int KT = DQK / 16;  // 16-wide k-steps over d_qk
  constexpr int DB = DV / 32;   // 32-wide blocks of d_v
  constexpr float TAU = 8.f;
  // Per-wave LDS tiles, each buffer its own object: the compiler orders a
  // transposing LDS read after every pending direct-to-LDS load into the
  // same object, which would wait for the next tile's load.  16-bit io:
  // K and V tiles double-buffered (sK0/sK1, sV0/sV1).  Q8: one dequantized
  // K and V tile (sK0, sV0) and double-buffered int8 staging tiles.  After
  // the loop, the wave's partial O (32 x DV fp32) is rows 0-15 in sK0 and
  // rows 16-31 in sV0, its row max / sum in sK1 (sKq0 for Q8).
  static_assert(!Q8 || (DQK == 128 && DV == 128), "quantized K/V: head dim 128");
  static_assert(16 * DV * 4 <= BC * DV * 2, "half an O partial fits a V tile");
  __shared__ __attribute__((aligned(1024))) T sK0[4][BC * DQK];
  __shared__ __attribute__((aligned(1024))) T sK1[4][Q8 ? 1 : BC * DQK];
  __shared__ __attribute__((aligned(1024))) T sV0[4][BC * DV];
  __shared__ __attribute__((aligned(1024))) T sV1[4][Q8 ? 1 : BC * DV];
  __shared__ __attribute__((aligned(1024))) uint16_t sKq0[4][Q8 ? BC * DQK / 2 : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t sKq1[4][Q8 ? BC * DQK / 2 : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t sVq0[4][Q8 ? BC * DV / 2 : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t sVq1[4][Q8 ? BC * DV / 2 : 1];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = wave_id();
  const int Hkv = a.H / a.G;
  // XCD x = id mod 8 owns a contiguous range of the (batch, kv head, split,
  // row group) units, row groups innermost (they read the same K/V)
  const int64_t n_units = (int64_t)a.B * Hkv * d.ns * d.rg;
  const int64_t per_xcd = (n_units + 7) / 8;
  const int64_t pos = blockIdx.x >> 3;
  const int64_t u = (int64_t)(blockIdx.x & 7) * per_xcd + pos;
  if (pos >= per_xcd || u >= n_units) return;
  const int rg = (int)(u % d.rg);
  const int split = (int)((u / d.rg) % d.ns);
  const int hk = (int)((u / ((int64_t)d.rg * d.ns)) % Hkv);
  const int b = (int)(u / ((int64_t)d.rg * d.ns * Hkv));
  const SeqPos sp = resolve_seq(a.seq, b);
  const int sq = sp.sq, skv = sp.skv;
  const int nrows = a.G * sq;  // (query head of the group, position) pairs
  const int r0 = 32 * rg;
  if (r0 >= nrows) return;

  // this lane's row: query head hk*G + gi, position s
  const int r = r0 + l32;
  const bool row_ok = r < nrows;
  const int gi = row_ok ? r / sq : 0;
  const int s_pos = row_ok ? r - gi * sq : 0;
  const int h = hk * a.G + gi;

  // positions covered by the workgroup's rows, and the keys they can see
  const int r1 = min(r0 + 32, nrows) - 1;
  const bool one_head = r0 / sq == r1 / sq;
  const int s_lo = one_head ? r0 % sq : 0, s_hi = one_head ? r1 % sq : sq - 1;
  const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sq, skv);
  const int k_begin = BAND ? (int)max((int64_t)0, (int64_t)s_lo + bd.lo) : 0;
  const int k_end = BAND ? (int)min((int64_t)skv, (int64_t)s_hi + bd.hi + 1) : skv;
  // this split's keys, in 32-key tiles; wave w takes tiles tb + w + 4j
  const int ks = max(k_begin, (int)min((int64_t)split * d.chunk, (int64_t)skv));
  const int ke = min(k_end, (int)min((int64_t)(split + 1) * d.chunk, (int64_t)skv));
  const int tb = ks / BC;
  const int te = ke > ks ? (ke + BC - 1) / BC : tb;
  const int ntw = te - tb > w ? (te - tb - w + 3) / 4 : 0;

  // Q first: loads complete in issue order, so waiting for Q does not wait
  // for the K/V tiles behind it
  const T* qrow = base_ptr<T>(a.q, a.sq_, sp, h, true) + (int64_t)s_pos * a.sq_.s;
  u32x4 qreg[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
    qreg[t] = row_ok ? *(const u32x4*)(qrow + 16 * t + 8 * g) : u32x4{0, 0, 0, 0};

  // tiles: LT is the 16-bit element type the loaders move (int8 rows are
  // moved as rows of D/2 16-bit elements)
  using LT = std::conditional_t<Q8, uint16_t, T>;
  constexpr int LDQK = Q8 ? DQK / 2 : DQK, LDV = Q8 ? DV / 2 : DV;
  using KLoader = std::conditional_t<Q4, Int4TileLoader<DQK>, TileLoader<LDQK, BC, LT, 1>>;
  using VLoader = std::conditional_t<Q4, Int4TileLoader<DV>, TileLoader<LDV, BC, LT, 1>>;
  T* const kd = sK0[w];  // Q8: dequantized K tile
  T* const vd = sV0[w];  // Q8: dequantized V tile
  // the tiles the loads fill (buf a compile-time constant)
  auto ktile = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if constexpr (Q8) return buf ? sKq1[w] : sKq0[w];
    else return buf ? sK1[w] : sK0[w];
  };
  auto vtile = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if constexpr (Q8) return buf ? sVq1[w] : sVq0[w];
    else return buf ? sV1[w] : sV0[w];
  };
  KLoader ldK;
  VLoader ldV;
  if constexpr (Q4) {
    // strides count bytes
    const int8_t* kq = (const int8_t*)a.k + sp.bsel * a.sk_.b + (int64_t)hk * a.sk_.h + sp.ktok * a.sk_.s;
    const int8_t* vq = (const int8_t*)a.v + sp.bsel * a.sv_.b + (int64_t)hk * a.sv_.h + sp.ktok * a.sv_.s;
    ldK.init(kq, a.sk_.s, 0, lane);
    ldV.init(vq, a.sv_.s, 0, lane);
  } else if constexpr (Q8) {
    const int8_t* kq = (const int8_t*)a.k + sp.bsel * a.sk_.b + (int64_t)hk * a.sk_.h + sp.ktok * a.sk_.s;
    const int8_t* vq = (const int8_t*)a.v + sp.bsel * a.sv_.b + (int64_t)hk * a.sv_.h + sp.ktok * a.sv_.s;
    ldK.init((const LT*)kq, a.sk_.s / 2, 0, lane);
    ldV.init((const LT*)vq, a.sv_.s / 2, 0, lane);
  } else {
    ldK.init(base_ptr<LT>(a.k, a.sk_, sp, hk, false), a.sk_.s, 0, lane);
    ldV.init(base_ptr<LT>(a.v, a.sv_, sp, hk, false), a.sv_.s, 0, lane);
  }
  // Quantized K/V: a lane dequantizes chunks of CPC codes, LPR lanes per
  // row, at rows lane / LPR + RSTEP u (u < NSC).  This lane's scale / zero
  // point column (its chunk's group) and the per-token scale rows of this
  // sequence and key/value head:
  constexpr int CPC = Q4 ? 32 : 16, LPR = DQK / CPC, RSTEP = 64 / LPR, NSC = Q4 ? 2 : 4;
  const int qcol = Q8 ? (CPC * (lane % LPR)) / d.qgs : 0;
  const int64_t sc_base = sp.bsel * d.ss.b + (int64_t)hk * d.ss.h + sp.ktok * d.ss.s + qcol;
  // this lane's scale (zero point) entries for tile row lane / LPR; the
  // lane's u-th row then only adds the uniform (n0 + RSTEP u) rows
  const int64_t sc_lane = sc_base + (int64_t)(lane / LPR) * d.ss.s;
  float ksc[2][4], vsc[2][4];
  int kzp[2][4], vzp[2][4];
  // (buf is a compile-time constant: the scale registers are indexed by it)
  auto load_tile = [&](auto bufc, int n0) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    ldK.load(ktile(bufc), n0, skv, 0, lane);
    ldV.load(vtile(bufc), n0, skv, 0, lane);
    if constexpr (Q8) {
      if (n0 + BC <= skv) {
        // whole tile in range: per-lane offset plus a uniform row offset
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
          const int64_t o = sc_lane + (int64_t)(n0 + RSTEP * u) * d.ss.s;
          ksc[buf][u] = d.k_sc[o];
          vsc[buf][u] = d.v_sc[o];
        }
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
          const int64_t o = sc_lane + (int64_t)(n0 + RSTEP * u) * d.ss.s;
          kzp[buf][u] = QZP ? d.k_zp[o] : 0;
          vzp[buf][u] = QZP ? d.v_zp[o] : 0;
        }
      } else {
        // the last tile: rows clamped to the sequence (those keys are masked)
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
          const int row = min(n0 + lane / LPR + RSTEP * u, skv - 1);
          ksc[buf][u] = d.k_sc[sc_base + (int64_t)row * d.ss.s];
          vsc[buf][u] = d.v_sc[sc_base + (int64_t)row * d.ss.s];
        }
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
          const int row = min(n0 + lane / LPR + RSTEP * u, skv - 1);
          kzp[buf][u] = QZP ? d.k_zp[sc_base + (int64_t)row * d.ss.s] : 0;
          vzp[buf][u] = QZP ? d.v_zp[sc_base + (int64_t)row * d.ss.s] : 0;
        }
      }
    }
  };
  if (ntw > 0) load_tile(std::integral_constant<int, 0>{}, (tb + w) * BC);
  if (ntw > 1) load_tile(std::integral_constant<int, 1>{}, (tb + w + 4) * BC);
  // vector memory operations of one tile (K and V direct-to-LDS loads, and
  // the scales and zero points of quantized K/V)
  constexpr int TILE_LOADS =
      KLoader::PER_WAVE + VLoader::PER_WAVE + (Q8 ? 2 * NSC * (QZP ? 2 : 1) : 0);

  const float c = a.scale_log2;
  // a zero scale cannot hide a score with an infinity through the FMA: such
  // tiles use raw scores 0 (visible) / -inf (hidden) and an effective scale 1
  const bool zs = c == 0.f;
  const float ce = zs ? 1.f : c;
  const bool pos_scale = ce >= 0.f;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;  // m_run in scaled log2 units

  RowReader<DQK, T> rdK;
  TrReader<DV, T> rdV;
  rdK.init(lane);
  rdV.init(lane);

  // Tile j sits in buffer j % 2 == buf; tile j + 1, if any, is in flight
  // into the other buffer.
  auto tile = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int n0 = (tb + w + 4 * j) * BC;
    // tile j has landed (tile j + 1 may still be loading)
    if (j + 1 < ntw) wait_vm<TILE_LOADS>();
    else wait_vm<0>();
    const T* cK;
    const T* cV;
    if constexpr (Q4) {
      constexpr bool SG = QM <= 4;  // signed codes
      dequant_tile4<T, DQK, SG>((const uint8_t*)ktile(bufc), kd, ksc[buf], kzp[buf], lane);
      dequant_tile4<T, DV, SG>((const uint8_t*)vtile(bufc), vd, vsc[buf], vzp[buf], lane);
    } else if constexpr (Q8) {
      dequant_tile<T, DQK>(ktile(bufc), kd, ksc[buf], kzp[buf], lane);
      dequant_tile<T, DV>(vtile(bufc), vd, vsc[buf], vzp[buf], lane);
    }
    if constexpr (Q8) {
      wait_lds();  // the 16-bit tiles are written, the staging tiles read
      if (j + 2 < ntw) load_tile(bufc, n0 + 8 * BC);
      cK = kd;
      cV = vd;
    } else {
      cK = (const T*)ktile(bufc);
      cV = (const T*)vtile(bufc);
    }
    u32x4 kop[KT], vop[2 * DB];
    static_for<KT>([&](auto t) __attribute__((always_inline)) { kop[t] = rdK.template read<t>(cK, 0); });
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      static_for<DB>([&](auto db) __attribute__((always_inline)) {
        vop[tt * DB + db] = rdV.template read<32 * db>(cV, 16 * tt);
      });
    if (!Q8 && j + 2 < ntw) {
      wait_lds();  // the operands are in registers: the buffers are free
      load_tile(bufc, n0 + 8 * BC);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) s = mfma32<T>(kop[t], qreg[t], s);

    // masked unless every key of the tile is visible from every position
    const bool need_mask =
        (n0 + BC > skv) || (BAND && !(n0 - s_hi >= bd.lo && n0 + BC - 1 - s_lo <= bd.hi));
    auto visible = [&](int rr) {
      const int kv = n0 + 16 * (rr >> 3) + 8 * g + (rr & 7);
      return kv < skv && (!BAND || (kv - s_pos >= bd.lo && kv - s_pos <= bd.hi));
    };
    const float hide = pos_scale ? -INFINITY : INFINITY;
    if (need_mask || zs) {
      keep_branch();
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s[rr] = visible(rr) ? (zs ? 0.f : s[rr]) : hide;
    }
    float mrow;
    if (pos_scale) {
      float mx = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
      mx = max_pair32(mx);
      mrow = mx == -INFINITY ? -INFINITY : mx * ce;
    } else {
      float mn = INFINITY;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mn = fminf(mn, s[rr]);
      mn = -max_pair32(-mn);
      mrow = mn == INFINITY ? -INFINITY : mn * ce;
    }

    const float m_new = fmaxf(m_run, mrow);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + TAU) != 0) {
      keep_branch();
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tt + 2 * e], ce, -m_run));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tt + 2 * e + 1], ce, -m_run));
        psum += x0 + x1;
        pb[e] = pack2<T>(x0, x1);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = mfma32<T>(vop[tt * DB + db], pb, oacc[db]);
    }
    l_run += psum;
  };

  for (int j = 0; j < ntw; j += 2) {
    tile(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntw) tile(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the four waves' (max, sum, O) through LDS -----------------
  wait_all();
  // rows of DV floats with 16-byte chunks XOR-swizzled by row
  // (conflict-free column writes); rows 0-15 in sK0, 16-31 in sV0
  auto orow_ptr = [&](int wv, int rl) __attribute__((always_inline)) {
    return (float*)(rl < 16 ? (void*)sK0[wv] : (void*)sV0[wv]) + (rl & 15) * DV;
  };
  auto ml_ptr = [&](int wv) __attribute__((always_inline)) {
    if constexpr (Q8) return (float*)sKq0[wv];
    else return (float*)sK1[wv];
  };
  float* sMLw = ml_ptr(w);  // [32] max, then [32] sum
  const float l_row = sum_pair32(l_run);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int dd = 32 * db + 8 * rr + 4 * g;
      *(f32x4*)(orow_ptr(w, l32) + ((((dd >> 2) ^ l32) & (DV / 4 - 1)) << 2)) =
          f32x4{oacc[db][4 * rr], oacc[db][4 * rr + 1], oacc[db][4 * rr + 2], oacc[db][4 * rr + 3]};
    }
  if (g == 0) {
    sMLw[l32] = m_run;
    sMLw[32 + l32] = l_row;
  }
  __syncthreads();

  const int64_t st_group_rows = lse_group_rows(a.seq, a.B);
  for (int e = tid; e < 32 * DV; e += 256) {
    const int rl = e / DV, dd = e - rl * DV;
    const int rr_ = r0 + rl;
    if (rr_ >= nrows) break;  // rows are contiguous: the rest are past the end too
    float M = -1e30f;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, ml_ptr(v)[rl]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float* ml = ml_ptr(v);
      const float f = __builtin_amdgcn_exp2f(ml[rl] - M);
      L += f * ml[32 + rl];
      O += f * orow_ptr(v, rl)[((((dd >> 2) ^ rl) & (DV / 4 - 1)) << 2) + (dd & 3)];
    }
    const float o = L > 0.f ? O / L : 0.f;
    const float lse = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    const int gr = rr_ / sq, sr = rr_ - gr * sq, hr = hk * a.G + gr;
    const int64_t st = row_stat_base(a.seq, sp, b, hr, a.H, st_group_rows) + sr;
    if (d.ns == 1) {
      T* orow = base_ptr_mut<T>(a.o, a.so_, sp, hr, true) + (int64_t)sr * a.so_.s;
      st_elem<T>(orow + dd, o);
      if (a.lse && dd == 0) a.lse[st] = lse;
    } else {
      d.part_o[((int64_t)split * d.nr + st) * DV + dd] = o;
      if (dd == 0) d.part_lse[(int64_t)split * d.nr + st] = lse;
    }
  }
}

// Merge the splits of one row per wave: LSE = log sum_i exp(LSE_i), O = sum_i
// exp(LSE_i - LSE) O_i, in ascending split order.
template <typename T, int DV>
__global__ void __launch_bounds__(256) fwd_decode_combine(const FwdArgs a, const DecodeArgs d) {
  const int lane = threadIdx.x & 63;
  const int64_t st = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  // the row's output address: batch rows are ((b H + h) s_q + s), group rows
  // (h T + token)
  T* orow;
  if (a.seq.cu_q) {
    const int64_t T_ = lse_group_rows(a.seq, a.B);
    if (st >= (int64_t)a.H * T_) return;
    const int64_t h = st / T_, tok = st - h * T_;
    if (tok >= a.seq.cu_q[a.B]) return;  // packed rows past the last sequence
    orow = (T*)a.o + h * a.so_.h + tok * a.so_.s;
  } else {
    if (st >= d.nr) return;
    const int64_t bh = st / a.seq.s_q, s = st - bh * a.seq.s_q;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    orow = (T*)a.o + b * a.so_.b + h * a.so_.h + s * a.so_.s;
  }
  float M = -INFINITY;
  for (int i = 0; i < d.ns; ++i) M = fmaxf(M, d.part_lse[(int64_t)i * d.nr + st]);
  constexpr int PER = (DV + 63) / 64;
  float acc[PER], L = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < d.ns; ++i) {
      const float f = __builtin_amdgcn_exp2f((d.part_lse[(int64_t)i * d.nr + st] - M) * kLog2e);
      L += f;
      const float* po = d.part_o + ((int64_t)i * d.nr + st) * DV;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (lane + 64 * k < DV) acc[k] += f * po[lane + 64 * k];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (lane + 64 * k < DV) st_elem<T>(orow + lane + 64 * k, acc[k] * inv);
  if (a.lse && lane == 0) a.lse[st] = L > 0.f ? M + logf(L) : -INFINITY;
}

// ---------------------------------------------------------------------------
DecodePlan plan_decode(int64_t B, int64_t H, int32_t G, int64_t s_q, int64_t s_kv,
                       int64_t target_wgs) {
  DecodePlan pl;
  pl.rg = (int32_t)((G * s_q + 31) / 32);
  const int64_t units = B * (H / G) * pl.rg;
  // enough splits to give about target_wgs workgroups, but at least 256
  // keys (two tiles per wave) per split
  int64_t ns = units > 0 ? (target_wgs + units - 1) / units : 1;
  ns = std::max<int64_t>(1, std::min(ns, (s_kv + 255) / 256));
  int64_t chunk = (s_kv + ns - 1) / ns;
  chunk = (chunk + 127) / 128 * 128;
  pl.chunk = (int32_t)chunk;
  pl.ns = (int32_t)((s_kv + chunk - 1) / chunk);
  return pl;
}

template <typename T, int DQK, int DV>
static hipError_t decode_dims(bool band, const FwdArgs& a, const DecodeArgs& d, hipStream_t st) {
  const int64_t units = (int64_t)a.B * (a.H / a.G) * d.ns * d.rg;
  dim3 grid((unsigned)(8 * ((units + 7) / 8))), block(256);
  // kernel code format: 0 16-bit; 1 int8, 3 signed 4-bit, 5 unsigned 4-bit;
  // one more with zero points
  const int qm = d.k_sc == nullptr ? 0 : (2 * d.qfmt - 1 + (d.k_zp != nullptr ? 1 : 0));
  if constexpr (DQK == 128 && DV == 128) {
#define SDPA_DEC_Q(QMV)                                                                            \
    if (qm == QMV && band) hipLaunchKernelGGL((fwd_decode<T, DQK, DV, true, QMV>), grid, block, 0, st, a, d); \
    if (qm == QMV && !band) hipLaunchKernelGGL((fwd_decode<T, DQK, DV, false, QMV>), grid, block, 0, st, a, d);
    SDPA_DEC_Q(1) SDPA_DEC_Q(2) SDPA_DEC_Q(3) SDPA_DEC_Q(4) SDPA_DEC_Q(5) SDPA_DEC_Q(6)
#undef SDPA_DEC_Q
  } else if (qm != 0) {
    return hipErrorInvalidValue;
  }
  if (qm == 0 && band) hipLaunchKernelGGL((fwd_decode<T, DQK, DV, true, 0>), grid, block, 0, st, a, d);
  if (qm == 0 && !band) hipLaunchKernelGGL((fwd_decode<T, DQK, DV, false, 0>), grid, block, 0, st, a, d);
  if (log_enabled()) {
    char tile[128];
    std::snprintf(tile, sizeof(tile), "%d row groups of 32 x %d splits of %d keys, K/V codes %d",
                  d.rg, d.ns, d.chunk, qm);
    log_launch("fwd_decode", std::is_same<T, __bf16>::value ? IoType::BF16 : IoType::F16, DQK, DV,
               band, false, false, tile, grid, block);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || d.ns == 1) return e;
  dim3 cgrid((unsigned)((d.nr + 3) / 4));
  hipLaunchKernelGGL((fwd_decode_combine<T, DV>), cgrid, block, 0, st, a, d);
  log_launch("fwd_decode_combine", std::is_same<T, __bf16>::value ? IoType::BF16 : IoType::F16, DQK,
             DV, band, false, false, "one wave per row", cgrid, block);
  return hipGetLastError();
}

template <typename T>
static hipError_t decode_type(int dqk, int dv, bool band, const FwdArgs& a, const DecodeArgs& d,
                              hipStream_t st) {
  if (dqk == 64 && dv == 64) return decode_dims<T, 64, 64>(band, a, d, st);
  if (dqk == 128 && dv == 128) return decode_dims<T, 128, 128>(band, a, d, st);
  if (dqk == 192 && dv == 128) return decode_dims<T, 192, 128>(band, a, d, st);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_decode(IoType t, int dqk, int dv, bool band, const FwdArgs& a,
                             const DecodeArgs& d, hipStream_t st) {
  if (t == IoType::BF16) return decode_type<__bf16>(dqk, dv, band, a, d, st);
  if (t == IoType::F16) return decode_type<_Float16>(dqk, dv, band, a, d, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
