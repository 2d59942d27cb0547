// Forward attention kernels for gfx950.
//
// What is computed (Composable Kernel "fmha_bwd_kernel.hpp Source File",
// formula comment S, S', S'', P; PyTorch "MHA.cpp" run_cudnn_SDP_fprop for
// the O and fp32 stats outputs): O = softmax(scale * Q K^T + Bias, masked)
// (dropped out) V, and LSE = row log-sum-exp (natural log).
//
// MFMA kernel (16-bit io).  One workgroup = 4 wavefronts = 128 query rows of
// one (batch, head) - the query-stationary grid of oneDNN's execute_forward
// (q tiles x heads x batch).  Each wave keeps its 32 query rows of Q in
// registers as the B operand and computes the transposed score tile
// S^T = K Q^T (keys x queries) per 64-key tile, so a lane owns one query
// row: the row max and row sum are lane-local apart from one exchange with
// lane l^32.  With the keys fetched in sig-permuted order, the probabilities
// come out of the accumulators already in the B-operand layout of the second
// product O^T += V^T P^T, whose A operand is read from the natural [key][d]
// V tile in LDS with the gfx950 transposing LDS read.  Softmax runs in base
// 2 with log2(e) folded into the scale (CK stores scale*log2e beside the raw
// scale in its kernel arguments).
#include <type_traits>

#include "sdpa_kcommon.h"

#ifndef SDPA_FWD_NBLK
#define SDPA_FWD_NBLK 2
#endif
// heads whose tiles are interleaved rank-major on one XCD (see xcd_work)

namespace sdpa {

// Wide head dims (d_qk + d_v > 256) without dropout read their K and V
// operands as they use them (LEAN) instead of a whole tile's ahead: the
// prefetched operands alone (d 192/128: 96 + 64 registers) would hold the
// kernel at one wave per SIMD, where nothing hides the latency of its
// loads.  With LEAN the second wave on the SIMD hides it.
template <int DQK, int DV, bool DROP> struct FwdLean {
  static constexpr bool value = (DQK + DV > 256) && !DROP;
};
// workgroups per CU the register budget is sized for
// Two waves per SIMD (256 registers) unless the head dims are wide (and not
// LEAN).  With dropout the d 128 instances spill at that budget; the causal
// ones without bias still run faster at two waves (measured), the others
// keep one wave.
template <int DQK, int DV, bool DROP, bool BAND = false, bool BIAS = false> struct FwdOcc {
  static constexpr int value =
      ((DQK + DV > 256) && !FwdLean<DQK, DV, DROP>::value) ||
              (DROP && DQK + DV > 128 && !(BAND && !BIAS))
          ? 1
          : 2;
};

template <typename T, int DQK, int DV, bool BAND, bool BIAS, bool DROP>
__global__ void __launch_bounds__(256, (FwdOcc<DQK, DV, DROP, BAND, BIAS>::value)) fwd_mfma(const FwdArgs a) {
  constexpr int BR = 128;
  constexpr int NBLK = SDPA_FWD_NBLK;  // 32-key blocks per key tile
  constexpr int BC = 32 * NBLK;
  constexpr int KT = DQK / 16;  // 16-wide k-steps over d_qk
  constexpr int DB = DV / 32;   // 32-wide blocks of d_v
  // Lazy rescaling: the running max is only raised (and O, l rescaled) when
  // some row's max grows by more than TAU (log2 units); until then the
  // probabilities are exp2(x - m_run) <= 2^TAU, exact in fp32 and bf16.
  constexpr float TAU = 8.f;
  // STREAM: the launch may give a workgroup several units (problems without
  // bias or dropout, batch or group mode, whose grid is capped at two
  // workgroups per compute unit)
  constexpr bool STREAM = !BIAS && !DROP;
  __shared__ __attribute__((aligned(1024))) T sK[2][BC * DQK];  // double-buffered tiles
  __shared__ __attribute__((aligned(1024))) T sV[2][BC * DV];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = wave_id();
  const int nqt = (a.seq.s_q + BR - 1) / BR;
  const bool hmajor = a.seq.cu_q != nullptr;

  // One unit: 128 query rows of one (batch, head).
  auto unit = [&](const WorkItem wi) __attribute__((always_inline)) {
  if (!wi.valid) return;
  const int b = wi.b, h = wi.h;
  const int mt = BAND ? nqt - 1 - wi.tile : wi.tile;  // heaviest causal tiles first
  const SeqPos sp = resolve_seq(a.seq, b);
  const int sq = sp.sq, skv = sp.skv;
  const int q0 = mt * BR;
  if (q0 >= sq) return;

  const T* qg = base_ptr<T>(a.q, a.sq_, sp, h, true);
  T* og = base_ptr_mut<T>(a.o, a.so_, sp, h, true);
  const uint16_t* bg = nullptr;
  if (BIAS) bg = (const uint16_t*)a.bias + (int64_t)b * a.sb_.b + (int64_t)h * a.sb_.h;
  // ALiBi takes the bias path's place (computed, not loaded)
  const bool alibi = BIAS && a.alibi != nullptr;
  const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sp.sq, sp.skv);

  // keys visible from some row of this tile: [k_begin, k_end), in key
  // tiles t0 .. t0 + nt - 1
  const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sq, skv);
  const int r_last = min(q0 + BR, sq) - 1;
  const int k_begin = BAND ? max(0, q0 + bd.lo) : 0;
  const int k_end = BAND ? min(skv, (int)min((int64_t)r_last + bd.hi + 1, (int64_t)skv)) : skv;
  const int t0 = k_begin / BC;
  const int nt = k_end > k_begin ? (k_end + BC - 1) / BC - t0 : 0;
  const int wq0 = q0 + 32 * w;        // this wave's first query row
  const int row = wq0 + l32;          // this lane's query row
  const bool row_ok = row < sq;

  TileLoader<DQK, BC, T> ldK;
  TileLoader<DV, BC, T> ldV;
  ldK.init(base_ptr<T>(a.k, a.sk_, sp, h / a.G, false), a.sk_.s, w, lane);
  ldV.init(base_ptr<T>(a.v, a.sv_, sp, h / a.G, false), a.sv_.s, w, lane);
  if (nt > 0) {
    ldK.load(sK[0], t0 * BC, skv, w, lane);
    ldV.load(sV[0], t0 * BC, skv, w, lane);
  }

  u32x4 qreg[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
    qreg[t] = row_ok ? *(const u32x4*)(qg + (int64_t)row * a.sq_.s + 16 * t + 8 * g)
                     : u32x4{0, 0, 0, 0};

  DropKey dk{};
  const uint32_t bh = (uint32_t)(b * a.H + h);
  if (DROP) dk = drop_key(a.drop);
  const float c = a.scale_log2;
  // A zero scale makes every visible score equal; the exponent's FMA cannot
  // then hide a score with an infinity (0 * inf), so such tiles replace the
  // raw scores by 0 (visible) / -inf (hidden) and use an effective scale 1.
  const bool zs = c == 0.f;
  const float ce = zs ? 1.f : c;
  const bool pos = ce >= 0.f;  // uniform: which extreme of the raw scores is the max

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;  // m_run in scaled log2 units

  RowReader<DQK, T> rdK;
  // (registers to spare only at d <= 128 without bias or dropout)
  TrReader<DV, T, !BIAS && !DROP && DQK + DV <= 256> rdV;
  rdK.init(lane);
  rdV.init(lane);

  // Bias loads.  One-wave-per-SIMD instances (BIAS_PF) have the registers
  // to hold a second tile's bias and request it one tile ahead; the latency
  // of HBM loads is otherwise exposed there, with no other wave to run.
  constexpr bool BIAS_PF = BIAS && FwdOcc<DQK, DV, DROP, BAND, BIAS>::value == 1;
  uint32_t bq[BIAS_PF ? 2 : 1][2 * NBLK][4];
  auto load_bias = [&](uint32_t (&dst)[2 * NBLK][4], int nb) __attribute__((always_inline)) {
    if (!BIAS || alibi) return;
#pragma unroll
    for (int u = 0; u < 2 * NBLK; ++u) {
      int kb = nb + 16 * u + 8 * g;  // u = 2*blk + hh
      const uint16_t* p = bg + (int64_t)row * a.sb_.s + kb;
      if (row_ok && kb + 8 <= skv && a.bias_vec) {
        u32x4 x = *(const u32x4*)p;
        dst[u][0] = x[0]; dst[u][1] = x[1]; dst[u][2] = x[2]; dst[u][3] = x[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t lo = (row_ok && kb + 2 * e < skv) ? p[2 * e] : 0;
          uint32_t hi = (row_ok && kb + 2 * e + 1 < skv) ? p[2 * e + 1] : 0;
          dst[u][e] = lo | (hi << 16);
        }
      }
    }
  };
  if (BIAS_PF && nt > 0) load_bias(bq[0], t0 * BC);

  // One key tile: `cK`, `cV` hold tile `it`; the next tile is loaded into
  // `nK`, `nV`.  Called with the two buffers swapped on alternate tiles so
  // that every LDS address is a compile-time offset from a per-lane base
  // (PC, the tile's parity, likewise selects the bias registers).
  auto tile = [&](int it, const T* cK, const T* cV, T* nK, T* nV, auto pcc) __attribute__((always_inline)) {
    constexpr int PC = decltype(pcc)::value;
    const int n0 = (t0 + it) * BC;
    wait_all();       // this wave's part of tile `it` has landed
    __syncthreads();  // ... and everyone's; tile it-1 is fully consumed

    // a wave whose rows see none of this tile skips it (band mask): its rows
    // [wq0, wq0 + 31] see keys [wq0 + lo, wq0 + 31 + hi]
    const bool active = !BAND || (n0 <= wq0 + 31 + bd.hi && n0 + BC - 1 >= wq0 + bd.lo);

    // All K operands of this tile are requested first, so their LDS latency
    // overlaps the prefetch issue and the rest of the requests (LEAN: each
    // is read at its product).
    constexpr bool LEAN = FwdLean<DQK, DV, DROP>::value;
    u32x4 kop[LEAN ? 1 : NBLK * KT];
    if (!LEAN && active) {
      static_for<KT>([&](auto t) __attribute__((always_inline)) {
        u32x4 kb2[NBLK];
        rdK.template read_blocks<t>(cK, kb2);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) kop[NBLK * t + blk] = kb2[blk];
      });
    }

    // bias for this lane's row: runs of 8 consecutive keys.  With BIAS_PF
    // the next tile's are requested here (they land with its K/V tiles);
    // otherwise this tile's, before the next tile's prefetch so that
    // waiting for them does not wait for it.
    uint32_t braw_here[2 * NBLK][4];
    uint32_t (&braw)[2 * NBLK][4] = *(BIAS_PF ? &bq[PC % (BIAS_PF ? 2 : 1)] : &braw_here);
    if constexpr (BIAS_PF) {
      if (it + 1 < nt) load_bias(bq[(1 - PC) % (BIAS_PF ? 2 : 1)], n0 + BC);
    } else if (BIAS && active && !alibi) {
      load_bias(braw, n0);
    }
    if (it + 1 < nt) {
      ldK.load(nK, n0 + BC, skv, w, lane);
      ldV.load(nV, n0 + BC, skv, w, lane);
    }
    if (!active) return;

    // S^T = K Q^T for the tile's 32-key blocks
    f32x16 s[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) s[blk] = f32x16{};
    if constexpr (LEAN) {
      static_for<KT>([&](auto t) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
          s[blk] = mfma32<T>(rdK.template read<t>(cK, 32 * blk), qreg[t], s[blk]);
      });
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) s[blk] = mfma32<T>(kop[NBLK * t + blk], qreg[t], s[blk]);
    }

    // keep bytes (dropout): runs of 4 keys
    uint32_t kw[8];
    if (DROP) {
      uint32_t var4[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) var4[k] = (uint32_t)((n0 + 16 * (k >> 1) + 8 * g) >> 2) + (k & 1);
      quad_keep_words<true>(var4, (uint32_t)row >> 2, bh, dk.off, dk.k0, dk.k1, lane, kw);
    }

    // Scores in scaled log2 units.  Without bias the scale is folded into
    // the exponent's FMA and the row max is taken on the raw scores.
    // masked unless every (row, key) of the wave's tile lies inside the band
    const bool need_mask =
        (n0 + BC > skv) || (BAND && !(n0 - (wq0 + 31) >= bd.lo && n0 + BC - 1 - wq0 <= bd.hi));
    // key n0 + 8 g + o of this lane's row (o = 32 blk + 16 (r >> 3) + (r & 7))
    auto visible = [&](const TileWindow& win, int blk, int r) {
      return win.has(32 * blk + 16 * (r >> 3) + (r & 7));
    };
    float mrow;
    if (BIAS) {
      if (alibi) {
        keep_branch();
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = n0 + 32 * blk + 16 * (r >> 3) + 8 * g + (r & 7);
            s[blk][r] = __builtin_fmaf(s[blk][r], c, alibi_at(at, kv, row) * kLog2e);
          }
      } else {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int u = 2 * blk + (r >> 3), e = r & 7;
            uint32_t bits = (braw[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            s[blk][r] = __builtin_fmaf(s[blk][r], c, to_f32<T>((uint16_t)bits) * kLog2e);
          }
      }
      if (need_mask) {
        keep_branch();
        const TileWindow win = keys_of_row(row, bd, BAND, skv, n0 + 8 * g);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[blk][r] = visible(win, blk, r) ? s[blk][r] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
      mrow = max_pair32(mx);
    } else {
      const float hide = pos ? -INFINITY : INFINITY;
      if (need_mask || zs) {
        keep_branch();
        const TileWindow win = keys_of_row(row, bd, BAND, skv, n0 + 8 * g);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[blk][r] = visible(win, blk, r) ? (zs ? 0.f : s[blk][r]) : hide;
      }
      float mx = -INFINITY, mn = INFINITY;
      if (pos) {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
        mx = max_pair32(mx);
        mrow = mx == -INFINITY ? -INFINITY : mx * ce;
      } else {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mn = fminf(mn, s[blk][r]);
        mn = -max_pair32(-mn);
        mrow = mn == INFINITY ? -INFINITY : mn * ce;
      }
    }

    // all V^T operands of this tile, requested before the exponentials
    // (LEAN: each slice's, at the slice)
    u32x4 vop[LEAN ? DB : 2 * NBLK * DB];
    if constexpr (!LEAN) {
#pragma unroll
      for (int tt = 0; tt < 2 * NBLK; ++tt)
        static_for<DB>([&](auto db) __attribute__((always_inline)) {
          vop[tt * DB + db] = rdV.template read<32 * db>(cV, 16 * tt);
        });
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
    // Masked scores already hold -inf (scaled) / the hiding infinity (raw),
    // so the exponent loop has no branches.  One 16-key slice at a time: the
    // slice's P V products are issued as soon as it is packed, so they run
    // on the matrix cores while the next slice's exponentials are computed.
    float psum = 0.f;
    u32x4 pb[2 * NBLK];
    static_for<2 * NBLK>([&](auto tt) __attribute__((always_inline)) {
      constexpr int blk = tt / 2, r0 = 8 * (tt % 2);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = r0 + e;
        const float x = BIAS ? __builtin_amdgcn_exp2f(s[blk][r] - m_run)
                             : __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][r], ce, -m_run));
        psum += x;
        p[e] = x;
        if (DROP) {
          const int k = 4 * blk + 2 * (r >> 3) + ((r & 7) >> 2);
          const bool keep = ((kw[k] >> (8 * (r & 3))) & 0xffu) >= dk.thr;
          p[e] = keep ? x : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[tt][e] = pack2<T>(p[2 * e], p[2 * e + 1]);
      // O^T += V^T P^T for this slice
      if constexpr (LEAN) {
        static_for<DB>([&](auto db) __attribute__((always_inline)) {
          vop[db] = rdV.template read<32 * db>(cV, 16 * tt);
        });
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma32<T>(vop[db], pb[tt], oacc[db]);
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma32<T>(vop[tt * DB + db], pb[tt], oacc[db]);
      }
    });
    l_run += psum;

    if (DROP && a.keep && row_ok) {
      uint8_t* kp = a.keep + (((int64_t)b * a.H + h) * a.seq.s_q + row) * a.seq.s_kv;
#pragma unroll
      for (int k = 0; k < 4 * NBLK; ++k) {
        int kv0 = n0 + 16 * (k >> 1) + 8 * g + 4 * (k & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int kv = kv0 + e;
          if (kv < skv && (!BAND || (kv - row >= bd.lo && kv - row <= bd.hi)))
            kp[kv] = ((kw[k] >> (8 * e)) & 0xffu) >= dk.thr ? 1 : 0;
        }
      }
    }

  };

  for (int it = 0; it < nt; it += 2) {
    tile(it, sK[0], sV[0], sK[1], sV[1], std::integral_constant<int, 0>{});
    if (it + 1 < nt) tile(it + 1, sK[1], sV[1], sK[0], sV[0], std::integral_constant<int, 1>{});
  }

  // epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2
  const float l_row = sum_pair32(l_run);
  float fac = l_row > 0.f ? 1.f / l_row : 0.f;
  if (DROP) fac *= a.drop.rescale;
  if (row_ok) {
    T* orow = og + (int64_t)row * a.so_.s;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int d = 32 * db + 8 * rr + 4 * g;
        u32x2 v2;
        v2[0] = pack2<T>(oacc[db][4 * rr + 0] * fac, oacc[db][4 * rr + 1] * fac);
        v2[1] = pack2<T>(oacc[db][4 * rr + 2] * fac, oacc[db][4 * rr + 3] * fac);
        *(u32x2*)(orow + d) = v2;
      }
    }
    if (a.lse && g == 0) {
      int64_t base = row_stat_base(a.seq, sp, b, h, a.H, lse_group_rows(a.seq, a.B));
      a.lse[base + row] = l_row > 0.f ? (m_run + log2f(l_row)) * kLn2 : -INFINITY;
    }
  }
  };

  if (STREAM) {
    // The grid may be smaller than the number of units: workgroup p = 8 r + x
    // takes the units of XCD x at positions r, 2R-1-r, 2R+r, ... (R
    // workgroups per XCD, every other round reversed to even out the
    // heaviest-first order), one after another.
    const int R = (int)(gridDim.x >> 3), xg = (int)(blockIdx.x & 7), rg = (int)(blockIdx.x >> 3);
    const int npos = (int)(((int64_t)a.B * a.H + 7) / 8) * nqt;
    for (int k = 0;; ++k) {
      const int pos = k * R + ((k & 1) ? R - 1 - rg : rg);
      if (pos >= npos) break;
      const WorkItem wi = xcd_work_at(8 * pos + xg, nqt, a.H, a.B, a.head_group, hmajor);
      if (!wi.valid) break;  // (positions only grow)
      if (k > 0) __syncthreads();  // every wave is done with the last unit's tiles
      unit(wi);
    }
  } else {
    unit(xcd_work(nqt, a.H, a.B, a.head_group, hmajor));
  }
}

// fp32 io: one wavefront per query row, the head dims spread over lanes.
template <bool BAND, bool BIAS, bool DROP>
__global__ void __launch_bounds__(256) fwd_f32(const FwdArgs a, int dqk, int dv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const SeqPos sp = resolve_seq(a.seq, b);
  const int row = blockIdx.x * 4 + w;
  if (row >= sp.sq) return;
  const float* qg = base_ptr<float>(a.q, a.sq_, sp, h, true) + (int64_t)row * a.sq_.s;
  const float* kg = base_ptr<float>(a.k, a.sk_, sp, h / a.G, false);
  const float* vg = base_ptr<float>(a.v, a.sv_, sp, h / a.G, false);
  float* og = base_ptr_mut<float>(a.o, a.so_, sp, h, true) + (int64_t)row * a.so_.s;
  const float* brow = (BIAS && a.bias) ? (const float*)a.bias + (int64_t)b * a.sb_.b +
                                            (int64_t)h * a.sb_.h + (int64_t)row * a.sb_.s
                                      : nullptr;
  const AlibiTerm at = alibi_term(a.alibi, a.alibi_sb, a.alibi_br, b, h, sp.sq, sp.skv);
  DropKey dk{};
  if (DROP) dk = drop_key(a.drop);
  const uint32_t bh = (uint32_t)(b * a.H + h);
  float q[4], o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    q[c] = d < dqk ? qg[d] : 0.f;
    o[c] = 0.f;
  }
  int first = 0, last = sp.skv - 1;
  if (BAND) {
    const Band bd = seq_band(a.band_br, a.band_lo, a.band_hi, sp.sq, sp.skv);
    first = (int)max((int64_t)0, (int64_t)row + bd.lo);
    last = (int)min((int64_t)last, (int64_t)row + bd.hi);
  }
  float m = -INFINITY, l = 0.f;
  for (int j = first; j <= last; ++j) {
    const float* kj = kg + (int64_t)j * a.sk_.s;
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int d = lane + 64 * c;
      if (d < dqk) part += q[c] * kj[d];
    }
    float sc = wave_sum(part) * a.scale + (BIAS ? (brow ? brow[j] : alibi_at(at, j, row)) : 0.f);
    float mn = fmaxf(m, sc);
    float alpha = expf(m - mn);
    float p = expf(sc - mn);
    l = l * alpha + p;
    m = mn;
    float pz = p;
    if (DROP) {
      bool keep = keep_one(dk, bh, row, j);
      pz = keep ? p : 0.f;
      if (a.keep && lane == 0)
        a.keep[(((int64_t)b * a.H + h) * a.seq.s_q + row) * a.seq.s_kv + j] = keep ? 1 : 0;
    }
    const float* vj = vg + (int64_t)j * a.sv_.s;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int d = lane + 64 * c;
      o[c] = o[c] * alpha + (d < dv ? pz * vj[d] : 0.f);
    }
  }
  float fac = l > 0.f ? 1.f / l : 0.f;
  if (DROP) fac *= a.drop.rescale;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int d = lane + 64 * c;
    if (d < dv) og[d] = o[c] * fac;
  }
  if (a.lse && lane == 0) {
    int64_t base = row_stat_base(a.seq, sp, b, h, a.H, lse_group_rows(a.seq, a.B));
    a.lse[base + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV>
static hipError_t fwd_dispatch_flags(bool causal, bool bias, bool drop, const FwdArgs& a,
                                     hipStream_t st) {
  dim3 grid = xcd_grid((a.seq.s_q + 127) / 128, a.H, a.B), block(256);
  // the plain instances stream units: as many workgroups as run at once
  // (their occupancy times the compute units, a multiple of 8), in batch and
  // group mode alike (group mode: 0.70 -> 0.66 ms on 16 sequences of
  // U[64, 4096] tokens)
  const int cus = device_cus() / 8 * 8;
#define SDPA_FWD_CASE(C, BI, DR)                                                 \
  if (causal == C && bias == BI && drop == DR) {                                 \
    if (!BI && !DR) {                                                            \
      const long cap = a.grid_cap < 0 ? (long)cus * FwdOcc<DQK, DV, DR, C, BI>::value \
                                      : (long)a.grid_cap;                        \
      if (cap > 0 && (long)grid.x > cap) grid.x = (unsigned)cap;                 \
    }                                                                            \
    hipLaunchKernelGGL((fwd_mfma<T, DQK, DV, C, BI, DR>), grid, block, 0, st, a); \
    log_launch("fwd_mfma", std::is_same<T, __bf16>::value ? IoType::BF16 : IoType::F16, DQK, DV, \
               C, BI, DR, "128 query rows (4 waves x 32) x 64-key tiles, 2 LDS buffers", grid, block); \
    return hipGetLastError();                                                    \
  }
  SDPA_FWD_CASE(false, false, false)
  SDPA_FWD_CASE(true, false, false)
  SDPA_FWD_CASE(false, true, false)
  SDPA_FWD_CASE(true, true, false)
  SDPA_FWD_CASE(false, false, true)
  SDPA_FWD_CASE(true, false, true)
  SDPA_FWD_CASE(false, true, true)
  SDPA_FWD_CASE(true, true, true)
#undef SDPA_FWD_CASE
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t fwd_dispatch_dims(int dqk, int dv, bool causal, bool bias, bool drop,
                                    const FwdArgs& a, hipStream_t st) {
  if (dqk == 64 && dv == 64) return fwd_dispatch_flags<T, 64, 64>(causal, bias, drop, a, st);
  if (dqk == 128 && dv == 128) return fwd_dispatch_flags<T, 128, 128>(causal, bias, drop, a, st);
  if (dqk == 192 && dv == 128) return fwd_dispatch_flags<T, 192, 128>(causal, bias, drop, a, st);
  return hipErrorInvalidValue;
}

bool mfma_dims_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

hipError_t launch_fwd(IoType t, int dqk, int dv, bool causal, const FwdArgs& a, hipStream_t st) {
  const bool bias = a.bias != nullptr || a.alibi != nullptr, drop = a.drop.enabled != 0;
  if (t == IoType::BF16) return fwd_dispatch_dims<__bf16>(dqk, dv, causal, bias, drop, a, st);
  if (t == IoType::F16) return fwd_dispatch_dims<_Float16>(dqk, dv, causal, bias, drop, a, st);
  dim3 grid((a.seq.s_q + 3) / 4, a.H, a.B), block(256);
#define SDPA_F32_CASE(C, BI, DR)                                                       \
  if (causal == C && bias == BI && drop == DR) {                                       \
    hipLaunchKernelGGL((fwd_f32<C, BI, DR>), grid, block, 0, st, a, dqk, dv);           \
    log_launch("fwd_f32", IoType::F32, dqk, dv, C, BI, DR, "one wave per query row", grid, block); \
    return hipGetLastError();                                                          \
  }
  SDPA_F32_CASE(false, false, false)
  SDPA_F32_CASE(true, false, false)
  SDPA_F32_CASE(false, true, false)
  SDPA_F32_CASE(true, true, false)
  SDPA_F32_CASE(false, false, true)
  SDPA_F32_CASE(true, false, true)
  SDPA_F32_CASE(false, true, true)
  SDPA_F32_CASE(true, true, true)
#undef SDPA_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdpa
