// Backward attention kernels for gfx950.
//
// What is computed (Composable Kernel "fmha_bwd_kernel.hpp Source File",
// formula comment dV, dP, D, dS'', dBias, dK, dQ):
//   D = rowsum(dO o O);  P = exp(S'' - LSE) recomputed from the saved stats;
//   dV = (P o Z)^T dO;  dP = (dO V^T) o Z;  dS = P o (dP - D);  dBias = dS;
//   dK = scale dS^T Q;  dQ = scale dS K.
//
// Three kernels, all deterministic (no atomics, every output element owned
// and written by exactly one workgroup, every sum in a fixed order):
//   bwd_pre   D = rowsum(dO o O) in fp32 - the separate preprocess of CK
//             (FmhaBwdOGradDotOKernel) and of oneDNN's execute_backward.
//   dkdv_*    key-stationary: one workgroup per 128 keys of a (batch, head)
//             (the grid of CK's GridSize and of oneDNN's backward main
//             kernel) keeps K and V in registers and accumulates dK, dV over
//             all query tiles; it also writes dBias.
//   dq_*      query-stationary: one workgroup per 128 query rows recomputes
//             S and dP for its rows and accumulates dQ in registers over all
//             key tiles, in ascending key order.
// Splitting dQ off trades two recomputed products (S and dP) for a dQ
// reduction with no workspace, no atomics and no inter-workgroup waiting;
// CK instead writes one fp32 dQ slice per key tile and sums the slices in
// FmhaBwdConvertQGradKernel, and oneDNN adds fp32 dQ atomically.
#include <type_traits>

#include "sdpa_kcommon.h"

// heads whose tiles are interleaved rank-major on one XCD (see xcd_work)
#ifndef SDPA_DKDV_BIAS_LDS_MAXD
#define SDPA_DKDV_BIAS_LDS_MAXD 192
#endif

// Role A of a dK/dV trip of two query blocks: 0 runs the blocks one after
// the other; 1 interleaves one block's exponentials with the other's matrix
// products in source order; 2 (default) also pins that order with empty
// scheduling barriers (the compiler otherwise groups the products together).
#ifndef SDPA_DKDV_PIPE
#define SDPA_DKDV_PIPE 2
#endif


// dK/dV trips of two query blocks under dropout too
#ifndef SDPA_DKDV_DROP2
#define SDPA_DKDV_DROP2 1
#endif

// a streaming dK/dV wave does not wait for its stationary operands at the
// first barrier of a unit
#ifndef SDPA_DKDV_ENTER_NOWAIT
#define SDPA_DKDV_ENTER_NOWAIT 1
#endif

namespace sdpa {

// ---------------------------------------------------------------------------
// D = rowsum(dO o O): 16 lanes per row, 16-byte loads, fp32 accumulation.
// The same pass also stores LSE * log2(e) beside D, so that the main kernels
// form P = exp2(scale*log2e * S - LSE*log2e) with one FMA per element.
template <typename T>
__global__ void __launch_bounds__(256) bwd_pre(const BwdArgs a, int dv) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  const int b = blockIdx.z, h = blockIdx.y;
  const SeqPos sp = resolve_seq(a.seq, b);
  const int sub = threadIdx.x & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool ok = row < sp.sq;
  float acc = 0.f;
  if (ok) {
    const T* o = base_ptr<T>(a.o, a.so_, sp, h, true) + (int64_t)row * a.so_.s;
    const T* d = base_ptr<T>(a.dout, a.sdo_, sp, h, true) + (int64_t)row * a.sdo_.s;
    for (int c = sub; c * EPC < dv; c += 16) {
      u32x4 x = *(const u32x4*)(o + c * EPC);
      u32x4 y = *(const u32x4*)(d + c * EPC);
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += __uint_as_float(x[e]) * __uint_as_float(y[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += to_f32<T>((uint16_t)(x[e] & 0xffffu)) * to_f32<T>((uint16_t)(y[e] & 0xffffu));
          acc += to_f32<T>((uint16_t)(x[e] >> 16)) * to_f32<T>((uint16_t)(y[e] >> 16));
        }
      }
    }
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (ok && sub == 0) {
    const int64_t base = row_stat_base(a.seq, sp, b, h, a.H, (int64_t)a.B * a.seq.s_q);
    a.dvec[base + row] = acc;
    if (a.lse2) {
      const int64_t lb = row_stat_base(a.seq, sp, b, h, a.H, lse_group_rows(a.seq, a.B));
      a.lse2[base + row] = a.lse[lb + row] * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV (and dBias).  Workgroup = 128 keys, 8 waves in two roles; wave
// kb = w & 3 owns keys kv0 + 32 kb + l32 (one key per lane) in both roles.
// Query tiles of 32 rows stream through LDS; per tile, with the queries
// fetched in sig order:
//   role A (w < 4):  S = Q K^T (B = K^T in registers), P = exp2(c S - LSE'),
//                    dV^T += dO^T (P o Z)   (A = dO^T by transposing read)
//                    and P is handed to role B through LDS;
//   role B (w >= 4), one tile behind:
//                    dP = dO V^T (B = V^T in registers),
//                    dS = P o (dP o Z - D), dBias = dS,
//                    dK^T += Q^T dS          (A = Q^T by transposing read).
// The two waves of a key block share a SIMD, so one's exponentials and
// element-wise work overlap the other's matrix products, and each role keeps
// only half of the stationary state (K and dV, or V and dK) in registers.
template <typename T, int DQK, int DV, bool BAND, bool BIAS, bool DROP>
__global__ void __launch_bounds__(512, 1) dkdv_mfma(const BwdArgs a) {
  // QBLK 32-row query blocks per trip (two where the LDS holds them), so
  // that each barrier and P hand-over covers QBLK blocks' products
  constexpr int QBLK = (!BIAS && (!DROP || SDPA_DKDV_DROP2) && DQK <= 128 && DV <= 128) ? 2 : 1;
  constexpr int BC = 128, BQ = 32 * QBLK, NSET = 3;
  // STREAM: a workgroup may take several units (the launch caps the grid at
  // the compute units), and role A's waves load every query-side tile.  The
  // bias and dropout instances, whose role A has the longer element-wise
  // work, run one unit per workgroup with all eight waves sharing the loads
  // (measured faster for them).
  constexpr bool STREAM = !BIAS && !DROP;
  constexpr int KT = DQK / 16, VT = DV / 16, QB = DQK / 32, VB = DV / 32;
  constexpr bool BIAS_LDS = BIAS && DQK <= SDPA_DKDV_BIAS_LDS_MAXD;
  // Query-side tiles are triple-buffered: role A reads set i % 3, role B
  // set (i - 1) % 3 and set (i + 1) % 3 is loading.
  __shared__ __attribute__((aligned(1024))) T sQ[NSET][BQ * DQK];
  __shared__ __attribute__((aligned(1024))) T sO[NSET][BQ * DV];
  __shared__ __attribute__((aligned(1024))) T sB[BIAS_LDS ? NSET : 1][BIAS_LDS ? BQ * BC : 64];
  __shared__ __attribute__((aligned(256))) float sL[NSET][BQ], sD[NSET][BQ];
  // P from role A to role B in the io type: [slot][key block][query block]
  // [2 groups of 8 elements][lane]
  __shared__ __attribute__((aligned(1024))) u32x4 sP[2][4][QBLK][2][64];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = wave_id();
  const int kb = w & 3;
  const bool roleA = w < 4;
  const int G = a.G;
  const bool want_dbias = BIAS && a.dbias != nullptr;
  const bool alibi = BIAS && a.alibi != nullptr;  // computed in place of the bias tensor
  DropKey dk{};
  if (DROP) dk = drop_key(a.drop);
  const float rescale = DROP ? a.drop.rescale : 1.f;
  const float c = a.scale_log2;
  // per query head: its bias / dBias rows
  auto bias_head = [&](int b, int h) __attribute__((always_inline)) {
    return (const uint16_t*)a.bias + (int64_t)b * a.sb_.b + (int64_t)h * a.sb_.h;
  };
  auto dbias_head = [&](int b, int h) __attribute__((always_inline)) {
    return (uint16_t*)a.dbias + (int64_t)b * a.sdb_.b + (int64_t)h * a.sdb_.h;
  };

  // ---- work units ----------------------------------------------------------
  // A unit is one (batch, key/value head, 128-key tile): it accumulates dK
  // and dV over the query tiles of every query head of the head's group.
  // With fewer workgroups than units, workgroup p = 8 r + x takes the units
  // of XCD x at positions r, 2R-1-r, 2R+r, 4R-1-r, ... (R workgroups per
  // XCD; every other round reversed, which evens out the heaviest-first
  // order) and streams their query tiles back to back: the trip pipeline
  // runs across unit boundaries, and each role loads the next unit's
  // stationary operands while the other role finishes the previous one.
  const int ntiles = (a.seq.s_kv + BC - 1) / BC;
  const int HG = a.H / G;
  const int R = (int)(gridDim.x >> 3), xg = (int)(blockIdx.x & 7), rg = (int)(blockIdx.x >> 3);
  const int npos = (int)(((int64_t)a.B * HG + 7) / 8) * ntiles;
  // (only the scalars the trip loop needs: the sequence's token offsets are
  // looked up again where pointers are formed)
  struct Unit {
    Band bd;
    int b, hk, kv0, sq, skv, q_begin, nq;
    int n;  // items: G nq query tiles (one empty item when nq = 0); 0 past the keys
  };
  auto get_unit = [&](int k, Unit& u) __attribute__((always_inline)) -> bool {
    const int pos = k * R + ((k & 1) ? R - 1 - rg : rg);
    if (pos >= npos) return false;
    const WorkItem wi = xcd_work_at(8 * pos + xg, ntiles, HG, a.B, a.dkdv_head_group, a.seq.cu_q != nullptr);
    if (!wi.valid) return false;
    u.b = wi.b;
    u.hk = wi.h;
    u.kv0 = wi.tile * BC;
    const SeqPos sp = resolve_seq(a.seq, u.b);
    u.sq = sp.sq;
    u.skv = sp.skv;
    u.bd = seq_band(a.band_br, a.band_lo, a.band_hi, u.sq, u.skv);
    // banded: only rows [kv0 - hi, kv_last - lo] see any of these keys; the
    // query tiles run over them from a tile boundary
    int q_begin = 0, q_end = u.sq;
    if (BAND) {
      const int64_t kv_last = min(u.kv0 + BC, u.skv) - 1;
      const int64_t r_lo = max((int64_t)0, (int64_t)u.kv0 - u.bd.hi);
      const int64_t r_hi = min((int64_t)u.sq, kv_last - u.bd.lo + 1);
      q_begin = r_lo < r_hi ? (int)(r_lo / BQ) * BQ : 0;
      q_end = r_lo < r_hi ? (int)r_hi : 0;
    }
    u.q_begin = q_begin;
    u.nq = q_end > q_begin ? (q_end - q_begin + BQ - 1) / BQ : 0;
    u.n = u.kv0 < u.skv ? max(G * u.nq, 1) : 0;
    return true;
  };
  // the first unit at index >= k that has keys here (its index, or -1)
  auto find_unit = [&](int k, Unit& u) __attribute__((always_inline)) -> int {
    for (;; ++k) {
      if (!get_unit(k, u)) return -1;
      if (u.n > 0) return k;
    }
  };
  // an item: query tile q0 of query head h; item j of a unit is query tile
  // j % nq of head hk G + j / nq
  struct Item {
    int h, q0;
  };
  auto next_item = [&](const Unit& u, Item it) __attribute__((always_inline)) {
    it.q0 += BQ;
    if (it.q0 >= u.q_begin + u.nq * BQ) {
      it.q0 = u.q_begin;
      ++it.h;
    }
    return it;
  };

  // bias tiles come through LDS when the whole 32 x 128 tile is in range and
  // its rows are 16-byte aligned; otherwise each lane reads its elements.
  auto bias_lds_of = [&](const Unit& u) __attribute__((always_inline)) {
    return BIAS_LDS && a.bias_vec && u.kv0 + BC <= u.skv;
  };
  // waves sharing each tile's loads, and the two that load LSE and D
  constexpr int NWQ = STREAM ? 4 : ((BQ * DQK / 8) % 512 == 0 ? 8 : 4);
  constexpr int NWO = STREAM ? 4 : ((BQ * DV / 8) % 512 == 0 ? 8 : 4);
  constexpr int NWB = STREAM ? 4 : 8;
  constexpr int WL = STREAM ? 2 : 6, WD = WL + 1;
  TileLoader<DQK, BQ, T, NWQ> ldQ;
  TileLoader<DV, BQ, T, NWO> ldO;
  TileLoader<BC, BQ, T, NWB> ldB;
  // the loaders' per-lane offsets depend only on the row strides; each item
  // moves their base
  if (w < NWQ) ldQ.init((const T*)a.q, a.sq_.s, w, lane);
  if (w < NWO) ldO.init((const T*)a.dout, a.sdo_.s, w, lane);
  if (BIAS_LDS && w < NWB) ldB.init((const T*)a.bias, a.sb_.s, w, lane);
  // (sp: the unit's sequence, resolve_seq(a.seq, u.b))
  auto issue = [&](int set, const Unit& u, const SeqPos& sp, Item it) __attribute__((always_inline)) {
    if (u.nq == 0) return;  // the empty item of a unit no query row sees
    const int q0 = it.q0, h = it.h, sq = u.sq;
    if (w < NWQ) {
      ldQ.g = (const char*)base_ptr<T>(a.q, a.sq_, sp, h, true);
      ldQ.load(sQ[set], q0, sq, w, lane);
    }
    if (w < NWO) {
      ldO.g = (const char*)base_ptr<T>(a.dout, a.sdo_, sp, h, true);
      ldO.load(sO[set], q0, sq, w, lane);
    }
    if (BIAS_LDS && w < NWB && bias_lds_of(u)) {
      ldB.g = (const char*)(bias_head(u.b, h) + u.kv0);
      ldB.load(sB[set], q0, sq, w, lane);
    }
    // the BQ LSE*log2(e) (wave WL) and D (wave WD) values, one row per lane,
    // rows clamped to the sequence
    if ((w == WL || w == WD) && lane < BQ) {
      int r = q0 + lane;
      r = r < sq ? r : sq - 1;
      const int64_t st_base = row_stat_base(a.seq, sp, u.b, h, a.H, (int64_t)a.B * a.seq.s_q);
      const float* src = (w == WL ? a.lse2 : a.dvec) + st_base + r;
      float* dst = w == WL ? sL[set] : sD[set];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst, 4, 0, 0);
    }
  };
  // key - row over this wave's 32 keys and the item's rows spans
  // [wk0 - (q0 + BQ - 1), wk0 + 31 - q0]
  auto tile_active = [&](const Unit& u, Item it) __attribute__((always_inline)) {
    const int wk0 = u.kv0 + 32 * kb;
    return u.nq > 0 && wk0 < u.skv &&
           (!BAND || (wk0 + 31 - it.q0 >= u.bd.lo && wk0 - (it.q0 + BQ - 1) <= u.bd.hi));
  };

  RowReader<DQK, T> rdQ;
  TrReader<DV, T> rdOt;
  RowReader<DV, T> rdO;
  TrReader<DQK, T> rdQt;
  rdQ.init(lane);
  rdOt.init(lane);
  rdO.init(lane);
  rdQt.init(lane);
  // this lane's P slot: per query block 2 x 16 bytes at stride 1 KiB
  const uint32_t p_lane = lds_addr(&sP[0][kb][0][0][0]) + 16 * lane;
  constexpr uint32_t P_SLOT = 4 * QBLK * 2 * 64 * 16;

  // ---- role A: S, P, dV for tile i -----------------------------------------
  auto stepA = [&](int i, int set, const Unit& u, Item it, const u32x4* reg, f32x16* acc)
      __attribute__((always_inline)) {
    const int b = u.b, sq = u.sq, skv = u.skv;
    const Band bd = u.bd;
    const int wk0 = u.kv0 + 32 * kb, kvr = wk0 + l32;
    const bool kv_ok = kvr < skv;
    // the same for one 32-row block starting at row q0
    auto block_active = [&](int q0) __attribute__((always_inline)) {
      return !BAND || (wk0 + 31 - q0 >= bd.lo && wk0 - (q0 + 31) <= bd.hi);
    };
    // (bitwise, so that evaluating it needs no branches)
    auto block_needs_mask = [&](int q0) __attribute__((always_inline)) {
      return (q0 + 32 > sq) | (wk0 + 31 >= skv) |
             (BAND & !((wk0 - (q0 + 31) >= bd.lo) & (wk0 + 31 - q0 <= bd.hi)));
    };
    const bool bias_lds = bias_lds_of(u);
    const int h = it.h;
    const uint32_t bh = (uint32_t)(b * a.H + h);
    const uint16_t* bg = BIAS ? bias_head(b, h) : nullptr;
    const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sq, skv);
    const auto vQ = rdQ.view(sQ[set]);
    const auto vOt = rdOt.view(sO[set]);
    // Operand reads issue in source order (their address XORs are volatile),
    // so each phase's operands are all requested before its products, and
    // the dV operands before the element-wise work.
    // (in two halves when there are more than 8 operands, to bound registers)
    constexpr int KH = KT > 8 ? KT / 2 : KT;
    // dV operands: requested before the element-wise work, unless the
    // element-wise work itself needs the registers (bias, wide Q/K rows)
    constexpr bool EARLY_O = !BIAS && DQK <= 128;
    // S = Q K^T of query block QB2
    // (hook(n) runs after the n-th product)
    auto scores = [&](auto qbc, auto&& hook) __attribute__((always_inline)) {
      constexpr int QB2 = decltype(qbc)::value;
      u32x4 qop[KH];
      f32x16 s = f32x16{};
      static_for<KT / KH>([&](auto hf) __attribute__((always_inline)) {
        static_for<KH>([&](auto j) __attribute__((always_inline)) {
          qop[j] = vQ.template read<hf * KH + j>(32 * QB2);
        });
        static_for<KH>([&](auto j) __attribute__((always_inline)) {
          s = mfma32<T>(qop[j], reg[hf * KH + j], s);
          hook(std::integral_constant<int, hf * KH + j>{});
        });
      });
      return s;
    };
    auto read_oop = [&](auto qbc, u32x4 (&oop)[2 * VB]) __attribute__((always_inline)) {
      constexpr int QB2 = decltype(qbc)::value;
      static_for<VB>([&](auto vb) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) oop[tt * VB + vb] = vOt.template read<32 * vb>(16 * tt + 32 * QB2);
      });
    };
    // P = exp2(c S + log2e bias - LSE log2e) of block QB2 (unmasked)
    auto exps = [&](auto qbc, const f32x16& s, float (&pv)[16]) __attribute__((always_inline)) {
      constexpr int QB2 = decltype(qbc)::value;
      const int q0 = it.q0 + 32 * QB2;
      const float* cL = sL[set] + 32 * QB2;
      const T* cB = sB[BIAS_LDS ? set : 0];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int lb = 16 * hh + 8 * g;  // first of my 8 consecutive rows
        const f32x4 L0 = *(const f32x4*)(cL + lb), L1 = *(const f32x4*)(cL + lb + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hh + e;
          float x = -(e < 4 ? L0[e] : L1[e - 4]);  // exponent = c s + log2e bias - LSE log2e
          if (BIAS) {
            const int ql = 32 * QB2 + lb + e, qr = q0 + lb + e;
            float bval = 0.f;
            if (alibi)
              bval = alibi_at(at, kvr, qr);
            else if (bias_lds)
              bval = to_f32<T>(*(const uint16_t*)(cB + Lds<BC>::off(ql, 32 * kb + l32)));
            else if (kv_ok && qr < sq)
              bval = to_f32<T>(bg[(int64_t)qr * a.sb_.s + kvr]);
            x = __builtin_fmaf(bval, kLog2e, x);
          }
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, x));
        }
      }
    };
    // without bias: the exponent's offsets -LSE log2e of block QB2's rows,
    // and element r's probability
    auto neg_lse = [&](auto qbc, float (&nl)[16]) __attribute__((always_inline)) {
      constexpr int QB2 = decltype(qbc)::value;
      const float* cL = sL[set] + 32 * QB2;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 L0 = *(const f32x4*)(cL + 16 * hh + 8 * g), L1 = *(const f32x4*)(cL + 16 * hh + 8 * g + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nl[8 * hh + e] = -L0[e];
          nl[8 * hh + 4 + e] = -L1[e];
        }
      }
    };
    auto exp_at = [&](const f32x16& s, const float (&nl)[16], int r) __attribute__((always_inline)) {
      return __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, nl[r]));
    };
    // masks P of block QB2, hands it to role B and returns P o Z packed as
    // the dV product's B operand
    // (dropout) the keep bytes of block QB2: 4x4 patches along this lane's
    // queries (the first 4 of the 8 used)
    auto keep_words = [&](auto qbc, uint32_t (&kw)[8]) __attribute__((always_inline)) {
      if (DROP) {
        const int q0 = it.q0 + 32 * decltype(qbc)::value;
        uint32_t var4[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) var4[k] = (uint32_t)((q0 + 16 * (k >> 1) + 8 * g) >> 2) + (k & 1);
        quad_keep_words<false>(var4, (uint32_t)kvr >> 2, bh, dk.off, dk.k0, dk.k1, lane, kw);
      }
    };
    auto finish = [&](auto qbc, float (&pv)[16], const uint32_t (&kw)[8], u32x4 (&pb)[2]) __attribute__((always_inline)) {
      constexpr int QB2 = decltype(qbc)::value;
      const int q0 = it.q0 + 32 * QB2;
      if (block_needs_mask(q0)) {
        keep_branch();
        // row q0 + 8 g + 16 (r >> 3) + (r & 7) against this lane's key
        const TileWindow win = kv_ok ? rows_of_key(kvr, bd, BAND, sq, q0 + 8 * g) : tile_window(1, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = win.has(16 * (r >> 3) + (r & 7)) ? pv[r] : 0.f;
      }
      // hand P to role B in the io type (P >= 0, so under dropout the sign
      // bit of each element marks it dropped)
      u32x4 ph[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * tt + 2 * e;
          const uint32_t wd = pack2<T>(pv[r], pv[r + 1]);
          if (DROP) {
            uint32_t keep[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int k = 2 * ((r + u) >> 3) + (((r + u) & 7) >> 2);
              keep[u] = ((kw[k] >> (8 * ((r + u) & 3))) & 0xffu) >= dk.thr;
            }
            ph[tt][e] = wd | (keep[0] ? 0u : 0x8000u) | (keep[1] ? 0u : 0x80000000u);
            pb[tt][e] = wd & ((keep[0] ? 0xffffu : 0u) | (keep[1] ? 0xffff0000u : 0u));
          } else {
            ph[tt][e] = wd;
            pb[tt][e] = wd;
          }
        }
      const uint32_t pa = p_lane + (uint32_t)(i & 1) * P_SLOT + 2048 * QB2;
#pragma unroll
      for (int j = 0; j < 2; ++j) *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(pa + 1024 * j) = ph[j];
    };
    // dV^T += dO^T (P o Z)
    auto dv = [&](const u32x4 (&oop)[2 * VB], const u32x4 (&pb)[2], auto&& hook) __attribute__((always_inline)) {
      static_for<2 * VB>([&](auto n) __attribute__((always_inline)) {
        constexpr int tt = n / VB, vb = n % VB;
        acc[vb] = mfma32<T>(oop[tt * VB + vb], pb[tt], acc[vb]);
        hook(n);
      });
    };
    auto none = [](auto) {};
    // one block, phase after phase
    auto block = [&](auto qbc) __attribute__((always_inline)) {
      const f32x16 s = scores(qbc, none);
      u32x4 oop[2 * VB], pb[2];
      if constexpr (EARLY_O) read_oop(qbc, oop);
      uint32_t kw[8];
      keep_words(qbc, kw);
      float pv[16];
      exps(qbc, s, pv);
      finish(qbc, pv, kw, pb);
      if constexpr (!EARLY_O) read_oop(qbc, oop);
      dv(oop, pb, none);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, QBLK - 1>;
    if constexpr (QBLK == 1) {
      block(B0{});
    } else {
      static_assert(QBLK == 2 && !BIAS, "two-block trips are for attention without bias");
      if (SDPA_DKDV_PIPE) {
        // The first block's exponentials are interleaved with the second
        // block's score products, and the second block's exponentials with
        // the first block's dV products, so that one wave's matrix products
        // and vector work overlap (the empty scheduling barriers keep the
        // compiler from regrouping them).  A block none of the wave's keys
        // see (at most one of the two, on the band's edge) goes through the
        // same steps: its mask leaves P = 0, which adds nothing to dV, and
        // role B skips it.
        auto fence = []() __attribute__((always_inline)) {
          if (SDPA_DKDV_PIPE >= 2) __builtin_amdgcn_sched_barrier(0);
        };
        // (dropout) the keep bytes of each block, formed among the products
        // before its mask: the first block's among its own score products,
        // the second block's among the first block's dV products
        uint32_t kw0[8], kw1[8];
        const f32x16 s0 = scores(B0{}, [&](auto n) __attribute__((always_inline)) {
          if constexpr (DROP && decltype(n)::value == 0) keep_words(B0{}, kw0);
        });
        float nl[16], pv0[16], pv1[16];
        neg_lse(B0{}, nl);
        u32x4 oop0[2 * VB], oop1[2 * VB], pb[2];
        read_oop(B0{}, oop0);
        // the elements r with r N / 16 = n after the n-th of N products
        auto share = [&](auto n, auto nn, const f32x16& sc, float (&pv)[16]) __attribute__((always_inline)) {
          fence();
          static_for<16>([&](auto r) __attribute__((always_inline)) {
            if constexpr (decltype(r)::value * decltype(nn)::value / 16 == decltype(n)::value) pv[r] = exp_at(sc, nl, r);
          });
          fence();
        };
        const f32x16 s1 = scores(B1{}, [&](auto n) __attribute__((always_inline)) {
          share(n, std::integral_constant<int, KT>{}, s0, pv0);
        });
        finish(B0{}, pv0, kw0, pb);
        neg_lse(B1{}, nl);
        read_oop(B1{}, oop1);
        dv(oop0, pb, [&](auto n) __attribute__((always_inline)) {
          if constexpr (DROP && decltype(n)::value == 0) keep_words(B1{}, kw1);
          share(n, std::integral_constant<int, 2 * VB>{}, s1, pv1);
        });
        finish(B1{}, pv1, kw1, pb);
        dv(oop1, pb, none);
      } else {
        if (block_active(it.q0)) block(B0{});
        if (block_active(it.q0 + 32)) block(B1{});
      }
    }
  };

  // ---- role B: dP, dS, dBias, dK for tile i ---------------------------------
  auto stepB = [&](int i, int set, const Unit& u, Item it, const u32x4* reg, f32x16* acc)
      __attribute__((always_inline)) {
    const int b = u.b, sq = u.sq, skv = u.skv;
    const Band bd = u.bd;
    const int wk0 = u.kv0 + 32 * kb, kvr = wk0 + l32;
    const bool kv_ok = kvr < skv;
    // the same for one 32-row block starting at row q0
    auto block_active = [&](int q0) __attribute__((always_inline)) {
      return !BAND || (wk0 + 31 - q0 >= bd.lo && wk0 - (q0 + 31) <= bd.hi);
    };
    // (bitwise, so that evaluating it needs no branches)
    auto block_needs_mask = [&](int q0) __attribute__((always_inline)) {
      return (q0 + 32 > sq) | (wk0 + 31 >= skv) |
             (BAND & !((wk0 - (q0 + 31) >= bd.lo) & (wk0 + 31 - q0 <= bd.hi)));
    };
   static_for<QBLK>([&](auto qbc) __attribute__((always_inline)) {
    constexpr int QB2 = decltype(qbc)::value;
    static_assert(QBLK == 1 || !BIAS, "a skipped block would leave its dBias rows unwritten");
    const int q0 = it.q0 + 32 * QB2;
    if (QBLK > 1 && !block_active(q0)) return;
    uint16_t* dbg = want_dbias ? dbias_head(b, it.h) : nullptr;
    const auto vO = rdO.view(sO[set]);
    const auto vQt = rdQt.view(sQ[set]);
    // (in halves when the dK accumulator is large, to bound registers)
    constexpr int VH = QB > 4 ? VT / 2 : VT;
    u32x4 oop[VH];
    f32x16 dp = f32x16{};
    static_for<VT / VH>([&](auto hf) __attribute__((always_inline)) {
      static_for<VH>([&](auto j) __attribute__((always_inline)) {
        oop[j] = vO.template read<hf * VH + j>(32 * QB2);
      });
#pragma unroll
      for (int j = 0; j < VH; ++j) dp = mfma32<T>(oop[j], reg[hf * VH + j], dp);
    });
    // Q^T operands for dK (the first half of them when there are more than 8)
    constexpr int QH = QB > 4 ? QB / 2 : QB;
    u32x4 qtop[2 * QH];
    static_for<QH>([&](auto qb) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) qtop[tt * QH + qb] = vQt.template read<32 * qb>(16 * tt + 32 * QB2);
    });
    const uint32_t pa = p_lane + (uint32_t)(i & 1) * P_SLOT + 2048 * QB2;
    u32x4 pw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) pw[j] = lds_load16(pa + 1024 * j);
    const float* cD = sD[set] + 32 * QB2;
    u32x4 dsb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int lb = 16 * hh + 8 * g;
      const f32x4 D0 = *(const f32x4*)(cD + lb), D1 = *(const f32x4*)(cD + lb + 4);
      float ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * hh + e;
        const uint32_t wd = pw[hh][e >> 1];
        const uint32_t bits = (e & 1) ? wd >> 16 : wd & 0xffffu;
        const float Dq = e < 4 ? D0[e] : D1[e - 4];
        float p, dpz;
        if (DROP) {
          p = to_f32<T>((uint16_t)(bits & 0x7fffu));
          dpz = (bits >> 15) ? 0.f : dp[r] * rescale;
        } else {
          p = to_f32<T>((uint16_t)bits);
          dpz = dp[r];
        }
        ds[e] = p * (dpz - Dq);
        if (want_dbias && kv_ok) {
          const int qr = q0 + lb + e;
          if (qr < sq) dbg[(int64_t)qr * a.sdb_.s + kvr] = (uint16_t)(pack2<T>(ds[e], 0.f) & 0xffffu);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsb[hh][e] = pack2<T>(ds[2 * e], ds[2 * e + 1]);
    }
    // dK^T += Q^T dS
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int qb = 0; qb < QH; ++qb) acc[qb] = mfma32<T>(qtop[tt * QH + qb], dsb[tt], acc[qb]);
    if constexpr (QH < QB) {
      static_for<QB - QH>([&](auto j) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) qtop[tt * QH + j] = vQt.template read<32 * (QH + j)>(16 * tt + 32 * QB2);
      });
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < QB - QH; ++j) acc[QH + j] = mfma32<T>(qtop[tt * QH + j], dsb[tt], acc[QH + j]);
    }
   });
  };

  // Each role runs its own copy of the trip loop, so its stationary operands
  // and accumulators are sized for it alone; both copies meet the same
  // barriers.  Trip i: role A takes item i (and loads item i + 1), role B
  // item i - 1; over this workgroup's N items both make N + 1 trips.
  auto run = [&](auto is_a) __attribute__((always_inline)) {
    constexpr bool IS_A = decltype(is_a)::value;
    constexpr int NR = IS_A ? KT : VT, NA = IS_A ? VB : QB;
    u32x4 reg[NR];  // K^T (role A) or V^T (role B) as B operands
    f32x16 acc[NA];  // dV^T (role A) or dK^T (role B), one key per lane
    // entering a unit: its stationary operands, a zeroed accumulator and
    // (role B, banded dBias) zeros in the rows no query tile of it covers
    auto enter = [&](const Unit& u, const SeqPos& sp) __attribute__((always_inline)) {
      const int kvr = u.kv0 + 32 * kb + l32;
      const bool kv_ok = kvr < u.skv;
      // Lanes past the keys load the last key's row: finite values whose
      // P (role A's mask) is zero and whose dK / dV are not stored.  The
      // loads are unconditional, so nothing waits for them until the
      // products use them (see the trip loop's first wait).
      const int kvc = min(kvr, u.skv - 1);
      const T* src = IS_A ? base_ptr<T>(a.k, a.sk_, sp, u.hk, false) + (int64_t)kvc * a.sk_.s
                          : base_ptr<T>(a.v, a.sv_, sp, u.hk, false) + (int64_t)kvc * a.sv_.s;
#pragma unroll
      for (int t = 0; t < NR; ++t) reg[t] = *(const u32x4*)(src + 16 * t + 8 * g);
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[j] = f32x16{};
      if (!IS_A && BAND && want_dbias && kv_ok) {
        const int sq = u.sq;
        const int z_end = min(u.q_begin, sq), z_begin = min(u.q_begin + u.nq * BQ, sq);
        for (int jh = 0; jh < G; ++jh) {
          uint16_t* dbg = dbias_head(u.b, u.hk * G + jh);
          for (int r = g; r < z_end; r += 2) dbg[(int64_t)r * a.sdb_.s + kvr] = 0;
          for (int r = z_begin + g; r < sq; r += 2) dbg[(int64_t)r * a.sdb_.s + kvr] = 0;
        }
      }
    };
    // leaving a unit: dV = rescale * dV^T acc (role A), dK = scale * dK^T acc (role B)
    auto leave = [&](const Unit& u, const SeqPos& sp) __attribute__((always_inline)) {
      const int kvr = u.kv0 + 32 * kb + l32;
      if (kvr >= u.skv) return;
      T* dst = IS_A ? base_ptr_mut<T>(a.dv, a.sdv_, sp, u.hk, false) + (int64_t)kvr * a.sdv_.s
                    : base_ptr_mut<T>(a.dk, a.sdk_, sp, u.hk, false) + (int64_t)kvr * a.sdk_.s;
      const float f = IS_A ? rescale : a.scale;
#pragma unroll
      for (int db = 0; db < NA; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          int d = 32 * db + 8 * rr + 4 * g;
          u32x2 v2;
          v2[0] = pack2<T>(acc[db][4 * rr] * f, acc[db][4 * rr + 1] * f);
          v2[1] = pack2<T>(acc[db][4 * rr + 2] * f, acc[db][4 * rr + 3] * f);
          *(u32x2*)(dst + d) = v2;
        }
      }
    };

    int set_prev = NSET - 1, set_cur = 0, set_nxt = 1;
    auto rotate = [&]() __attribute__((always_inline)) {
      set_prev = set_cur;
      set_cur = set_nxt;
      set_nxt = set_nxt == NSET - 1 ? 0 : set_nxt + 1;
    };
    Unit u;
    if constexpr (!STREAM) {
      // one unit per workgroup (the launch gives each unit its own): trip i
      // loads item i + 1 (all eight waves), role A takes item i, role B i - 1
      if (find_unit(0, u) != 0) return;  // no keys of this tile here
      const SeqPos sp = resolve_seq(a.seq, u.b);
      enter(u, sp);
      const int n = u.n;
      Item prev{}, cur{u.hk * G, u.q_begin}, nxt = next_item(u, cur);
      issue(0, u, sp, cur);
      for (int i = 0; i <= n; ++i) {
        wait_all();
        __syncthreads();  // item i landed; P(i-1) written; set (i+1)%3 free
        if (i + 1 < n) issue(set_nxt, u, sp, nxt);
        if constexpr (IS_A) {
          if (i < n && tile_active(u, cur)) stepA(i, set_cur, u, cur, reg, acc);
        } else if (i >= 1) {
          if (tile_active(u, prev)) {
            stepB(i - 1, set_prev, u, prev, reg, acc);
          } else if (BAND && want_dbias && u.nq > 0) {
            // the whole item is hidden from my key
            const int kvr = u.kv0 + 32 * kb + l32;
            if (kvr < u.skv) {
              uint16_t* dbg = dbias_head(u.b, prev.h);
              for (int r = prev.q0 + g; r < min(prev.q0 + BQ, u.sq); r += 2) dbg[(int64_t)r * a.sdb_.s + kvr] = 0;
            }
          }
        }
        prev = cur;
        cur = nxt;
        nxt = next_item(u, nxt);
        rotate();
      }
      leave(u, sp);
    } else {
      // several units per workgroup, streamed: role A loads every tile; at a
      // unit's last item it finds the next unit and loads that unit's first
      int k = find_unit(0, u);
      SeqPos sp = resolve_seq(a.seq, k >= 0 ? u.b : 0);
      if (IS_A && k >= 0) issue(0, u, sp, Item{u.hk * G, u.q_begin});
      if (!IS_A) {
        wait_all();
        __syncthreads();  // trip 0: role B has no item yet
        rotate();
      }
      int gi = 0;  // this role's item number
      while (k >= 0) {
        Unit un;  // role A: the next unit
        SeqPos spn;
        int kn = -1;
        enter(u, sp);
        Item it{u.hk * G, u.q_begin};
        for (int j = 0; j < u.n; ++j, ++gi) {
          // On a unit's first trip the last NR vector loads of this wave are
          // its stationary operands (issued on entering the unit, after
          // every tile load and store): the barrier need not wait for them.
          if (SDPA_DKDV_ENTER_NOWAIT && j == 0)
            wait_vm_lds<NR>();
          else
            wait_all();
          __syncthreads();  // item gi landed; P(gi-1) written; set (gi+1)%3 free
          if constexpr (IS_A) {
            if (j + 1 < u.n) {
              issue(set_nxt, u, sp, next_item(u, it));
            } else {
              kn = find_unit(k + 1, un);
              if (kn >= 0) {
                spn = resolve_seq(a.seq, un.b);
                issue(set_nxt, un, spn, Item{un.hk * G, un.q_begin});
              }
            }
          }
          if (tile_active(u, it)) {
            if constexpr (IS_A) stepA(gi, set_cur, u, it, reg, acc);
            else stepB(gi, set_prev, u, it, reg, acc);
          } else if (!IS_A && BAND && want_dbias && u.nq > 0) {
            // the whole item is hidden from my key
            const int kvr = u.kv0 + 32 * kb + l32;
            if (kvr < u.skv) {
              uint16_t* dbg = dbias_head(u.b, it.h);
              for (int r = it.q0 + g; r < min(it.q0 + BQ, u.sq); r += 2) dbg[(int64_t)r * a.sdb_.s + kvr] = 0;
            }
          }
          it = next_item(u, it);
          rotate();
        }
        leave(u, sp);
        if constexpr (IS_A) {
          k = kn;
          u = un;
          sp = spn;
        } else {
          k = find_unit(k + 1, u);
          if (k >= 0) sp = resolve_seq(a.seq, u.b);
        }
      }
      if (IS_A) {
        wait_all();
        __syncthreads();  // the last trip: role B's last item
      }
    }
  };
  if (roleA) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 waves x 32 query rows; key tiles of 64.  Each wave keeps
// Q^T and dO^T of its rows in registers and, per key tile, forms
//   S^T = K Q^T,  dP^T = V dO^T   (A operands: K, V rows from LDS)
//   dS^T = P^T o (dP^T - D)       (one query row per lane)
//   dQ^T += K^T dS^T              (A = K^T via the transposing LDS read)
// Two waves per SIMD (256 registers) unless the head dims are wide.  With
// dropout the d 128 instances spill at that budget; the causal ones without
// bias still run faster at two waves (measured), the others keep one wave.
template <int DQK, int DV, bool DROP, bool BAND = false, bool BIAS = false> struct DqOcc {
  static constexpr int value =
      (DQK + DV > 256) || (DROP && DQK + DV > 128 && !(BAND && !BIAS)) ? 1 : 2;
};

//
// With PRE the kernel also does the preprocess for its rows: D from the O
// and dO rows it loads and LSE*log2(e) from the forward's LSE, both written
// to the stats for the dK/dV kernel, which then runs after it.
template <typename T, int DQK, int DV, bool BAND, bool BIAS, bool DROP, bool PRE>
__global__ void __launch_bounds__(256, (DqOcc<DQK, DV, DROP, BAND, BIAS>::value)) dq_mfma(const BwdArgs a) {
  constexpr int BR = 128, BC = 64;
  constexpr int KT = DQK / 16, VT = DV / 16, QB = DQK / 32;
  // each buffer its own object: the compiler orders a transposing LDS read
  // after every pending direct-to-LDS load into the same object, which
  // would make each tile wait for the next tile's prefetch
  __shared__ __attribute__((aligned(1024))) T sK0[BC * DQK];
  __shared__ __attribute__((aligned(1024))) T sK1[BC * DQK];
  __shared__ __attribute__((aligned(1024))) T sV0[BC * DV];
  __shared__ __attribute__((aligned(1024))) T sV1[BC * DV];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = wave_id();
  const int nqt = (a.seq.s_q + BR - 1) / BR;
  const WorkItem wi = xcd_work(nqt, a.H, a.B, a.dq_head_group, a.seq.cu_q != nullptr);
  if (!wi.valid) return;
  const int b = wi.b, h = wi.h;
  const int mt = BAND ? nqt - 1 - wi.tile : wi.tile;  // heaviest top-left causal tiles first
  const SeqPos sp = resolve_seq(a.seq, b);
  const int sq = sp.sq, skv = sp.skv;
  const int q0 = mt * BR;
  if (q0 >= sq) return;

  const T* qg = base_ptr<T>(a.q, a.sq_, sp, h, true);
  const T* kg = base_ptr<T>(a.k, a.sk_, sp, h / a.G, false);
  const T* vg = base_ptr<T>(a.v, a.sv_, sp, h / a.G, false);
  const T* dog = base_ptr<T>(a.dout, a.sdo_, sp, h, true);
  const uint16_t* bg = nullptr;
  if (BIAS) bg = (const uint16_t*)a.bias + (int64_t)b * a.sb_.b + (int64_t)h * a.sb_.h;
  const bool alibi = BIAS && a.alibi != nullptr;  // computed in place of the bias tensor
  const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sq, skv);

  // banded: the tile's rows see only keys [q0 + lo, r_last + hi]
  const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sq, skv);
  const int r_last = min(q0 + BR, sq) - 1;
  const int k_begin = BAND ? max(0, q0 + bd.lo) : 0;
  const int k_end = BAND ? (int)min((int64_t)r_last + bd.hi + 1, (int64_t)skv) : skv;
  const int t0 = k_begin / BC;
  const int nt = k_end > k_begin ? (k_end + BC - 1) / BC - t0 : 0;
  const int row = q0 + 32 * w + l32;
  const int wq0 = q0 + 32 * w;  // this wave's first row
  const bool row_ok = row < sq;

  u32x4 qreg[KT], doreg[VT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
    qreg[t] = row_ok ? *(const u32x4*)(qg + (int64_t)row * a.sq_.s + 16 * t + 8 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < VT; ++t)
    doreg[t] = row_ok ? *(const u32x4*)(dog + (int64_t)row * a.sdo_.s + 16 * t + 8 * g) : u32x4{0, 0, 0, 0};
  float lse2 = 0.f, Drow = 0.f;
  const int64_t st = row_stat_base(a.seq, sp, b, h, a.H, (int64_t)a.B * a.seq.s_q) + row;
  if (PRE) {
    // D_row = rowsum(dO o O): this lane holds chunks 2t + g of its row's dO
    // (the B-operand layout), so it dots the same chunks of O and adds the
    // other half from lane l ^ 32.
    float part = 0.f;
    if (row_ok) {
      const T* orow = base_ptr<T>(a.o, a.so_, sp, h, true) + (int64_t)row * a.so_.s;
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const u32x4 ov = *(const u32x4*)(orow + 16 * t + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part += to_f32<T>((uint16_t)(ov[e] & 0xffffu)) * to_f32<T>((uint16_t)(doreg[t][e] & 0xffffu));
          part += to_f32<T>((uint16_t)(ov[e] >> 16)) * to_f32<T>((uint16_t)(doreg[t][e] >> 16));
        }
      }
      const int64_t lb = row_stat_base(a.seq, sp, b, h, a.H, lse_group_rows(a.seq, a.B));
      lse2 = a.lse[lb + row] * kLog2e;
    }
    Drow = sum_pair32(part);
    if (row_ok && g == 0) {
      a.dvec[st] = Drow;
      a.lse2[st] = lse2;
    }
  } else if (row_ok) {
    lse2 = a.lse2[st];
    Drow = a.dvec[st];
  }

  DropKey dk{};
  const uint32_t bh = (uint32_t)(b * a.H + h);
  if (DROP) dk = drop_key(a.drop);
  const float rescale = DROP ? a.drop.rescale : 1.f;

  f32x16 dqacc[QB];
#pragma unroll
  for (int i = 0; i < QB; ++i) dqacc[i] = f32x16{};

  TileLoader<DQK, BC, T, 4, true> ldK;
  TileLoader<DV, BC, T, 4, true> ldV;
  ldK.init(kg, a.sk_.s, w, lane);
  ldV.init(vg, a.sv_.s, w, lane);
  if (nt > 0) {
    ldK.load(sK0, t0 * BC, skv, w, lane);
    ldV.load(sV0, t0 * BC, skv, w, lane);
  }
  RowReader<DQK, T> rdK;
  RowReader<DV, T> rdV;
  // (the transposed reads' offsets held in registers where they fit)
  TrReader<DQK, T, !BIAS && !DROP && DQK + DV <= 256> rdKt;
  rdK.init(lane);
  rdV.init(lane);
  rdKt.init(lane);
  const float c = a.scale_log2;

  // One key tile: `cK`, `cV` hold tile `it`, the next one is loaded into
  // `nK`, `nV`; alternate tiles swap the buffers so that LDS addresses are
  // compile-time offsets from per-lane bases.
  auto tile = [&](int it, const T* cK, const T* cV, T* nK, T* nV) __attribute__((always_inline)) {
    const int n0 = (t0 + it) * BC;
    wait_all();
    __syncthreads();
    // key - row over the tile's keys and this wave's rows spans
    // [n0 - (wq0 + 31), n0 + BC - 1 - wq0]
    const bool active = !BAND || (n0 - (wq0 + 31) <= bd.hi && n0 + BC - 1 - wq0 >= bd.lo);

    if (it + 1 < nt) {
      ldK.load(nK, n0 + BC, skv, w, lane);
      ldV.load(nV, n0 + BC, skv, w, lane);
    }
    if (!active) return;

    // S^T = K Q^T and dP^T = V dO^T for the tile's two 32-key blocks
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    static_for<KT>([&](auto t) __attribute__((always_inline)) {
      u32x4 ab[2];
      if constexpr (BIAS) {
        ab[0] = rdK.template read<t>(cK, 0);
        ab[1] = rdK.template read<t>(cK, 32);
      } else {
        rdK.template read_blocks<t>(cK, ab);  // one swizzled offset for both blocks
      }
      const u32x4 a0 = ab[0], a1 = ab[1];
      s[0] = mfma32<T>(a0, qreg[t], s[0]);
      s[1] = mfma32<T>(a1, qreg[t], s[1]);
    });
    // bias for this lane's row, runs of 8 consecutive keys: requested
    // between the two products, so that the dP products hide their latency
    // without the registers being held across the score products too
    uint32_t braw[4][4];
    if (BIAS && active && !alibi) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int kb = n0 + 16 * u + 8 * g;
        const uint16_t* p = bg + (int64_t)row * a.sb_.s + kb;
        if (row_ok && kb + 8 <= skv && a.bias_vec) {
          u32x4 x = *(const u32x4*)p;
          braw[u][0] = x[0]; braw[u][1] = x[1]; braw[u][2] = x[2]; braw[u][3] = x[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t lo = (row_ok && kb + 2 * e < skv) ? p[2 * e] : 0;
            uint32_t hi = (row_ok && kb + 2 * e + 1 < skv) ? p[2 * e + 1] : 0;
            braw[u][e] = lo | (hi << 16);
          }
        }
      }
    }
    static_for<VT>([&](auto t) __attribute__((always_inline)) {
      u32x4 ab[2];
      if constexpr (BIAS) {
        ab[0] = rdV.template read<t>(cV, 0);
        ab[1] = rdV.template read<t>(cV, 32);
      } else {
        rdV.template read_blocks<t>(cV, ab);  // one swizzled offset for both blocks
      }
      const u32x4 a0 = ab[0], a1 = ab[1];
      dp[0] = mfma32<T>(a0, doreg[t], dp[0]);
      dp[1] = mfma32<T>(a1, doreg[t], dp[1]);
    });

    uint32_t kw[8];
    if (DROP) {
      uint32_t var4[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) var4[k] = (uint32_t)((n0 + 16 * (k >> 1) + 8 * g) >> 2) + (k & 1);
      quad_keep_words<true>(var4, (uint32_t)row >> 2, bh, dk.off, dk.k0, dk.k1, lane, kw);
    }

    // P^T = exp2(scale log2e S^T (+ log2e bias) - LSE log2e).  Rows past s_q
    // have Q = dO = 0 and LSE = D = 0, so their dS is exactly 0 without a
    // mask; keys past s_kv or outside the band are zeroed on the tiles
    // that have them.
    if (BIAS && alibi) {
      keep_branch();
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = n0 + 32 * blk + 16 * (r >> 3) + 8 * g + (r & 7);
          const float x = __builtin_fmaf(s[blk][r], c, __builtin_fmaf(alibi_at(at, kv, row), kLog2e, -lse2));
          s[blk][r] = __builtin_amdgcn_exp2f(x);
        }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x;
          if (BIAS) {
            const int u = 2 * blk + (r >> 3), e = r & 7;
            const uint32_t bits = (braw[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            x = __builtin_fmaf(s[blk][r], c, __builtin_fmaf(to_f32<T>((uint16_t)bits), kLog2e, -lse2));
          } else {
            x = __builtin_fmaf(s[blk][r], c, -lse2);
          }
          s[blk][r] = __builtin_amdgcn_exp2f(x);
        }
    }
    const bool need_mask =
        (n0 + BC > skv) || (BAND && !(n0 - (wq0 + 31) >= bd.lo && n0 + BC - 1 - wq0 <= bd.hi));
    if (need_mask) {
      keep_branch();
      const TileWindow win = keys_of_row(row, bd, BAND, skv, n0 + 8 * g);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[blk][r] = win.has(32 * blk + 16 * (r >> 3) + (r & 7)) ? s[blk][r] : 0.f;
    }
    // dS^T = P^T o (dP^T o Z - D), packed as the B operand of dQ^T += K^T dS^T
    u32x4 dsb[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int blk = tt >> 1, r0 = 8 * (tt & 1);
      float ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = r0 + e;
        float dpz = dp[blk][r];
        if (DROP) {
          const int k = 4 * blk + 2 * (r >> 3) + ((r & 7) >> 2);
          const bool keep = ((kw[k] >> (8 * (r & 3))) & 0xffu) >= dk.thr;
          dpz = keep ? dpz * rescale : 0.f;
        }
        ds[e] = s[blk][r] * (dpz - Drow);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsb[tt][e] = pack2<T>(ds[2 * e], ds[2 * e + 1]);
    }
    static_for<QB>([&](auto qb) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        dqacc[qb] = mfma32<T>(rdKt.template read<32 * qb>(cK, 16 * tt), dsb[tt], dqacc[qb]);
    });
  };

  for (int it = 0; it < nt; it += 2) {
    tile(it, sK0, sV0, sK1, sV1);
    if (it + 1 < nt) tile(it + 1, sK1, sV1, sK0, sV0);
  }

  if (row_ok) {
    T* dqr = base_ptr_mut<T>(a.dq, a.sdq_, sp, h, true) + (int64_t)row * a.sdq_.s;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int d = 32 * qb + 8 * rr + 4 * g;
        u32x2 v2;
        v2[0] = pack2<T>(dqacc[qb][4 * rr] * a.scale, dqacc[qb][4 * rr + 1] * a.scale);
        v2[1] = pack2<T>(dqacc[qb][4 * rr + 2] * a.scale, dqacc[qb][4 * rr + 3] * a.scale);
        *(u32x2*)(dqr + d) = v2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 io: one wavefront per query row (dQ) or per key (dK, dV, dBias).
template <bool BAND, bool BIAS, bool DROP>
__global__ void __launch_bounds__(256) dq_f32(const BwdArgs a, int dqk, int dv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const SeqPos sp = resolve_seq(a.seq, b);
  const int i = blockIdx.x * 4 + w;
  if (i >= sp.sq) return;
  const float* qi = base_ptr<float>(a.q, a.sq_, sp, h, true) + (int64_t)i * a.sq_.s;
  const float* doi = base_ptr<float>(a.dout, a.sdo_, sp, h, true) + (int64_t)i * a.sdo_.s;
  const float* kg = base_ptr<float>(a.k, a.sk_, sp, h / a.G, false);
  const float* vg = base_ptr<float>(a.v, a.sv_, sp, h / a.G, false);
  const float* brow = (BIAS && a.bias) ? (const float*)a.bias + (int64_t)b * a.sb_.b +
                                            (int64_t)h * a.sb_.h + (int64_t)i * a.sb_.s
                                      : nullptr;
  const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sp.sq, sp.skv);
  DropKey dk{};
  if (DROP) dk = drop_key(a.drop);
  const uint32_t bh = (uint32_t)(b * a.H + h);
  const int64_t st = row_stat_base(a.seq, sp, b, h, a.H, (int64_t)a.B * a.seq.s_q) + i;
  const float lse2 = a.lse2[st];
  const float Di = a.dvec[st];
  float q[4], dO[4], acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    q[c] = d < dqk ? qi[d] : 0.f;
    dO[c] = d < dv ? doi[d] : 0.f;
    acc[c] = 0.f;
  }
  int first = 0, last = sp.skv - 1;
  if (BAND) {
    const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sp.sq, sp.skv);
    first = (int)max((int64_t)0, (int64_t)i + bd.lo);
    last = (int)min((int64_t)last, (int64_t)i + bd.hi);
  }
  for (int j = first; j <= last; ++j) {
    const float* kj = kg + (int64_t)j * a.sk_.s;
    const float* vj = vg + (int64_t)j * a.sv_.s;
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int d = lane + 64 * c;
      if (d < dqk) ps += q[c] * kj[d];
      if (d < dv) pd += dO[c] * vj[d];
    }
    float s = wave_sum(ps) * a.scale + (BIAS ? (brow ? brow[j] : alibi_at(at, j, i)) : 0.f);
    float dp = wave_sum(pd);
    float p = exp2f(s * kLog2e - lse2);
    float z = 1.f;
    if (DROP) z = keep_one(dk, bh, i, j) ? a.drop.rescale : 0.f;
    float ds = p * (dp * z - Di);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int d = lane + 64 * c;
      if (d < dqk) acc[c] += ds * kj[d];
    }
  }
  float* dqi = base_ptr_mut<float>(a.dq, a.sdq_, sp, h, true) + (int64_t)i * a.sdq_.s;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    if (d < dqk) dqi[d] = acc[c] * a.scale;
  }
}

template <bool BAND, bool BIAS, bool DROP>
__global__ void __launch_bounds__(256) dkdv_f32(const BwdArgs a, int dqk, int dv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z, hk = blockIdx.y;  // key/value head
  const SeqPos sp = resolve_seq(a.seq, b);
  const int j = blockIdx.x * 4 + w;
  if (j >= sp.skv) return;
  const float* kj = base_ptr<float>(a.k, a.sk_, sp, hk, false) + (int64_t)j * a.sk_.s;
  const float* vj = base_ptr<float>(a.v, a.sv_, sp, hk, false) + (int64_t)j * a.sv_.s;
  DropKey dk{};
  if (DROP) dk = drop_key(a.drop);
  float k[4], v[4], gk[4], gv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    k[c] = d < dqk ? kj[d] : 0.f;
    v[c] = d < dv ? vj[d] : 0.f;
    gk[c] = 0.f;
    gv[c] = 0.f;
  }
  // rows that see key j: [j - hi, j - lo] within the sequence
  int i0 = 0, i1 = sp.sq;
  if (BAND) {
    const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sp.sq, sp.skv);
    i0 = (int)min((int64_t)sp.sq, max((int64_t)0, (int64_t)j - bd.hi));
    i1 = (int)max((int64_t)i0, min((int64_t)sp.sq, (int64_t)j - bd.lo + 1));
  }
  // the query heads of this key/value head's group, in ascending order
  for (int h = hk * a.G; h < (hk + 1) * a.G; ++h) {
    const float* qg = base_ptr<float>(a.q, a.sq_, sp, h, true);
    const float* dog = base_ptr<float>(a.dout, a.sdo_, sp, h, true);
    const float* bcol = (BIAS && a.bias)
                            ? (const float*)a.bias + (int64_t)b * a.sb_.b + (int64_t)h * a.sb_.h + j
                            : nullptr;
    const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sp.sq, sp.skv);
    float* dbcol = (BIAS && a.dbias)
                       ? (float*)a.dbias + (int64_t)b * a.sdb_.b + (int64_t)h * a.sdb_.h + j
                       : nullptr;
    const uint32_t bh = (uint32_t)(b * a.H + h);
    const int64_t d_base = row_stat_base(a.seq, sp, b, h, a.H, (int64_t)a.B * a.seq.s_q);
    if (dbcol && lane == 0) {
      for (int i = 0; i < i0; ++i) dbcol[(int64_t)i * a.sdb_.s] = 0.f;
      for (int i = i1; i < sp.sq; ++i) dbcol[(int64_t)i * a.sdb_.s] = 0.f;
    }
    for (int i = i0; i < i1; ++i) {
      const float* qi = qg + (int64_t)i * a.sq_.s;
      const float* doi = dog + (int64_t)i * a.sdo_.s;
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int d = lane + 64 * c;
        if (d < dqk) ps += qi[d] * k[c];
        if (d < dv) pd += doi[d] * v[c];
      }
      float s = wave_sum(ps) * a.scale +
                (BIAS ? (bcol ? bcol[(int64_t)i * a.sb_.s] : alibi_at(at, j, i)) : 0.f);
      float dp = wave_sum(pd);
      float p = exp2f(s * kLog2e - a.lse2[d_base + i]);
      float z = 1.f;
      if (DROP) z = keep_one(dk, bh, i, j) ? a.drop.rescale : 0.f;
      float ds = p * (dp * z - a.dvec[d_base + i]);
      if (dbcol && lane == 0) dbcol[(int64_t)i * a.sdb_.s] = ds;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int d = lane + 64 * c;
        if (d < dqk) gk[c] += ds * qi[d];
        if (d < dv) gv[c] += p * z * doi[d];
      }
    }
  }
  float* dkj = base_ptr_mut<float>(a.dk, a.sdk_, sp, hk, false) + (int64_t)j * a.sdk_.s;
  float* dvj = base_ptr_mut<float>(a.dv, a.sdv_, sp, hk, false) + (int64_t)j * a.sdv_.s;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    if (d < dqk) dkj[d] = gk[c] * a.scale;
    if (d < dv) dvj[d] = gv[c];
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_bwd_pre(IoType t, int dv, const BwdArgs& a, hipStream_t st) {
  dim3 grid((a.seq.s_q + 15) / 16, a.H, a.B), block(256);
  log_launch("bwd_pre", t, 0, dv, false, false, false, "16 rows per workgroup, 16 lanes per row",
             grid, block);
  if (t == IoType::BF16) hipLaunchKernelGGL(bwd_pre<__bf16>, grid, block, 0, st, a, dv);
  else if (t == IoType::F16) hipLaunchKernelGGL(bwd_pre<_Float16>, grid, block, 0, st, a, dv);
  else hipLaunchKernelGGL(bwd_pre<float>, grid, block, 0, st, a, dv);
  return hipGetLastError();
}

#define SDPA_FLAG_SWITCH(LAUNCH)              \
  if (!causal && !bias && !drop) LAUNCH(false, false, false) \
  if (causal && !bias && !drop) LAUNCH(true, false, false)   \
  if (!causal && bias && !drop) LAUNCH(false, true, false)   \
  if (causal && bias && !drop) LAUNCH(true, true, false)     \
  if (!causal && !bias && drop) LAUNCH(false, false, true)   \
  if (causal && !bias && drop) LAUNCH(true, false, true)     \
  if (!causal && bias && drop) LAUNCH(false, true, true)     \
  if (causal && bias && drop) LAUNCH(true, true, true)

template <typename T, int DQK, int DV>
static hipError_t dkdv_dims(bool causal, bool bias, bool drop, const BwdArgs& a, hipStream_t st) {
  // one workgroup per compute unit (a multiple of 8, one per XCD in turn),
  // each streaming its share of the (batch, head, key tile) units
  dim3 grid = xcd_grid((a.seq.s_kv + 127) / 128, a.H / a.G, a.B), block(512);
  // (the bias and dropout instances take one unit per workgroup, and so do
  // packed variable-length batches, whose units differ too much in size for
  // a fixed split: no cap)
  if (!bias && !drop && a.seq.cu_q == nullptr) {
    const long cap = a.dkdv_grid_cap < 0 ? (long)(device_cus() / 8 * 8) : (long)a.dkdv_grid_cap;
    if (cap > 0 && (long)grid.x > cap) grid.x = (unsigned)cap;
  }
#define L(C, BI, DR)                                                                         \
  {                                                                                          \
    hipLaunchKernelGGL((dkdv_mfma<T, DQK, DV, C, BI, DR>), grid, block, 0, st, a);           \
    log_launch("dkdv_mfma", std::is_same<T, __bf16>::value ? IoType::BF16 : IoType::F16, DQK, DV, \
               C, BI, DR, "128-key units (8 waves, 2 roles) streamed per workgroup, 32/64-row query tiles, 3 LDS sets", grid, block); \
    return hipGetLastError();                                                                \
  }
  SDPA_FLAG_SWITCH(L)
#undef L
  return hipErrorInvalidValue;
}
template <typename T, int DQK, int DV>
static hipError_t dq_dims(bool causal, bool bias, bool drop, bool pre, const BwdArgs& a,
                          hipStream_t st) {
  dim3 grid = xcd_grid((a.seq.s_q + 127) / 128, a.H, a.B), block(256);
#define L(C, BI, DR)                                                                        \
  {                                                                                         \
    if (pre) hipLaunchKernelGGL((dq_mfma<T, DQK, DV, C, BI, DR, true>), grid, block, 0, st, a); \
    else hipLaunchKernelGGL((dq_mfma<T, DQK, DV, C, BI, DR, false>), grid, block, 0, st, a);    \
    log_launch(pre ? "dq_mfma+preprocess" : "dq_mfma",                                      \
               std::is_same<T, __bf16>::value ? IoType::BF16 : IoType::F16, DQK, DV, C, BI, DR,   \
               "128 query rows (4 waves x 32) x 64-key tiles, 2 LDS buffers", grid, block);     \
    return hipGetLastError();                                                               \
  }
  SDPA_FLAG_SWITCH(L)
#undef L
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dkdv_type(int dqk, int dv, bool causal, bool bias, bool drop, const BwdArgs& a,
                            hipStream_t st) {
  if (dqk == 64 && dv == 64) return dkdv_dims<T, 64, 64>(causal, bias, drop, a, st);
  if (dqk == 128 && dv == 128) return dkdv_dims<T, 128, 128>(causal, bias, drop, a, st);
  if (dqk == 192 && dv == 128) return dkdv_dims<T, 192, 128>(causal, bias, drop, a, st);
  return hipErrorInvalidValue;
}
template <typename T>
static hipError_t dq_type(int dqk, int dv, bool causal, bool bias, bool drop, bool pre,
                          const BwdArgs& a, hipStream_t st) {
  if (dqk == 64 && dv == 64) return dq_dims<T, 64, 64>(causal, bias, drop, pre, a, st);
  if (dqk == 128 && dv == 128) return dq_dims<T, 128, 128>(causal, bias, drop, pre, a, st);
  if (dqk == 192 && dv == 128) return dq_dims<T, 192, 128>(causal, bias, drop, pre, a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(IoType t, int dqk, int dv, bool causal, const BwdArgs& a, hipStream_t st) {
  const bool bias = a.bias != nullptr || a.alibi != nullptr, drop = a.drop.enabled != 0;
  if (t == IoType::BF16) return dkdv_type<__bf16>(dqk, dv, causal, bias, drop, a, st);
  if (t == IoType::F16) return dkdv_type<_Float16>(dqk, dv, causal, bias, drop, a, st);
  dim3 grid((a.seq.s_kv + 3) / 4, a.H / a.G, a.B), block(256);
#define L(C, BI, DR)                                                                   \
  {                                                                                    \
    hipLaunchKernelGGL((dkdv_f32<C, BI, DR>), grid, block, 0, st, a, dqk, dv);          \
    log_launch("dkdv_f32", IoType::F32, dqk, dv, C, BI, DR, "one wave per key", grid, block); \
    return hipGetLastError();                                                          \
  }
  SDPA_FLAG_SWITCH(L)
#undef L
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(IoType t, int dqk, int dv, bool causal, const BwdArgs& a, hipStream_t st,
                         bool with_pre) {
  const bool bias = a.bias != nullptr || a.alibi != nullptr, drop = a.drop.enabled != 0;
  if (t == IoType::BF16) return dq_type<__bf16>(dqk, dv, causal, bias, drop, with_pre, a, st);
  if (t == IoType::F16) return dq_type<_Float16>(dqk, dv, causal, bias, drop, with_pre, a, st);
  if (with_pre) return hipErrorInvalidValue;  // the fp32 path keeps the separate preprocess
  dim3 grid((a.seq.s_q + 3) / 4, a.H, a.B), block(256);
#define L(C, BI, DR)                                                                 \
  {                                                                                  \
    hipLaunchKernelGGL((dq_f32<C, BI, DR>), grid, block, 0, st, a, dqk, dv);          \
    log_launch("dq_f32", IoType::F32, dqk, dv, C, BI, DR, "one wave per query row", grid, block); \
    return hipGetLastError();                                                        \
  }
  SDPA_FLAG_SWITCH(L)
#undef L
  return hipErrorInvalidValue;
}

}  // namespace sdpa
