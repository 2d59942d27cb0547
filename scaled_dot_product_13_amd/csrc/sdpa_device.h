// Device-side building blocks for the gfx950 attention kernels: MFMA
// wrappers, LDS tile layouts, transposing LDS reads, cross-lane reductions
// and the counter-based dropout generator.
//
// Register layouts used throughout (CDNA4 v_mfma_f32_32x32x16_{bf16,f16},
// one 64-lane wavefront; l32 = lane & 31, g = lane >> 5):
//   A operand (32 x 16, M x K):  lane holds A[m = l32][k = 8g + e], e = 0..7
//   B operand (16 x 32, K x N):  lane holds B[k = 8g + e][n = l32]
//   C/D (32 x 32, fp32 x 16):    lane holds C[8(r>>2) + 4g + (r&3)][l32], r = 0..15
// When an A operand's rows are fetched in the permuted order sig(m) (bits 2
// and 3 of m swapped), C element r of a lane lands on logical row
// 16(r>>3) + 8g + (r&7): the 8 values a lane needs as the K-slice of a
// following MFMA are then contiguous, so an accumulator tile feeds the next
// contraction straight from registers with no shuffle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sdpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F, int I = 0> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

__device__ __forceinline__ int sig(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// ---- MFMA ---------------------------------------------------------------
template <typename T> __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma32<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma32<_Float16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> one dword of two 16-bit io values, round to nearest even.
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
template <typename T> __device__ __forceinline__ float to_f32(uint16_t bits);
template <> __device__ __forceinline__ float to_f32<__bf16>(uint16_t bits) {
  return __uint_as_float(((uint32_t)bits) << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

// ---- cross-lane ---------------------------------------------------------
// value of lane l and of lane l^32 (same row, other half of the columns)
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);  // same order in both lanes
}
// lane ^ rho within a quad of lanes (DPP quad_perm)
template <int RHO> __device__ __forceinline__ uint32_t quad_xor(uint32_t v) {
  constexpr int ctrl = RHO == 1 ? 0xB1 : RHO == 2 ? 0x4E : 0x1B;
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}

// ---- LDS tile layouts ---------------------------------------------------
// A tile of rows of D 16-bit elements, rows unpadded, with the 16-byte chunks
// of each row XOR-swizzled so that both access patterns used here are free
// of LDS bank conflicts: 16 lanes reading the same chunk of 16 consecutive
// rows (ds_read_b128), and the transposing ds_read_b64_tr_b16 pattern (4
// consecutive rows x 4 consecutive chunks).  Rows of 128 (or 256) elements
// fill whole 64-bank lines and XOR the low 4 chunk bits; rows of 64 or 192
// elements alternate half lines and XOR the low 3 bits.  The XOR is its own
// inverse, so the same function maps logical to physical chunks and back.
template <int D> struct Lds {
  static_assert(D % 64 == 0, "head dims are multiples of 64");
  static constexpr int STRIDE = D;
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  __device__ __forceinline__ static int swz(int row) {
    if constexpr (D % 128 == 0) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
  __device__ __forceinline__ static int off(int row, int col) {  // col % 4 == 0
    return row * D + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// Fill a ROWS x D tile from global memory with gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at LDS base +
// 16 l).  Each of the 4 waves issues ROWS*D/8/256 such loads; lane l of load
// j covers physical chunk 64(4j + w) + l of the tile, and fetches the logical
// chunk that the swizzle puts there.  The per-lane byte offsets within a
// full tile are computed once; the tile's first row only moves a uniform
// base.  A tile that runs past `row_limit` takes a slow path that clamps rows
// to row_limit - 1 (callers mask those rows), so every address is valid;
// row_limit must be >= 1.  NW waves (w = 0 .. NW-1) share the loads; `w`
// must be wave-uniform.
// PIN: add each lane's 32-bit offset to the uniform tile base at the load
// (scalar-base addressing) rather than letting the compiler keep one 64-bit
// address per load live across the key loop; for kernels whose register
// budget is tight.
template <int D, int ROWS, typename T, int NW = 4, bool PIN = false> struct TileLoader {
  static constexpr int CPR = Lds<D>::CPR;
  static constexpr int PER_WAVE = ROWS * CPR / (64 * NW);
  static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split into whole wave loads");
  static constexpr int LOWMASK = (D % 128 == 0) ? 15 : 7;
  // When one load's 64 NW chunks are whole rows and a multiple of the
  // swizzle period (16 rows), load j covers load 0's pattern RSTEP j rows
  // further down: one per-lane offset serves all loads and the row step goes
  // into the uniform base.
  static constexpr bool AFFINE = (64 * NW) % CPR == 0 && (64 * NW / CPR) % 16 == 0;
  static constexpr int RSTEP = AFFINE ? 64 * NW / CPR : 0;
  const char* g;
  int64_t stride_b;  // row stride in bytes
  uint32_t voff[AFFINE ? 1 : PER_WAVE];

  __device__ __forceinline__ static void coords(int j, int w, int lane, int& row, int& c) {
    const int L = 64 * (NW * j + w) + lane;
    row = L / CPR;
    const int phys = L % CPR;
    c = (phys & ~LOWMASK) | ((phys ^ Lds<D>::swz(row)) & LOWMASK);
  }
  __device__ __forceinline__ void init(const T* g_, int64_t row_stride, int w, int lane) {
    g = (const char*)g_;
    stride_b = row_stride * (int64_t)sizeof(T);
#pragma unroll
    for (int j = 0; j < (AFFINE ? 1 : PER_WAVE); ++j) {
      int row, c;
      coords(j, w, lane, row, c);
      voff[j] = (uint32_t)(row * stride_b + 16 * c);
    }
  }
  __device__ __forceinline__ void load(T* tile, int row0, int row_limit, int w, int lane) const {
    if (row0 + ROWS <= row_limit) {
      const char* base = g + row0 * stride_b;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        uint32_t o = voff[AFFINE ? 0 : j];
        if (PIN) __asm__ volatile("" : "+v"(o));  // opaque: the add cannot be hoisted
        const char* bj = AFFINE ? base + (int64_t)(RSTEP * j) * stride_b : base;
        __builtin_amdgcn_global_load_lds((const void*)(bj + o),
                                         (lds_void*)(tile + 512 * (NW * j + w)), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        int row, c;
        coords(j, w, lane, row, c);
        int gr = row0 + row;
        gr = gr < row_limit ? gr : row_limit - 1;
        __builtin_amdgcn_global_load_lds((const void*)(g + gr * stride_b + 16 * c),
                                         (lds_void*)(tile + 512 * (NW * j + w)), 16, 0, 0);
      }
    }
  }
};

// wave index as a scalar (the compiler cannot prove threadIdx.x >> 6 uniform)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Wait for all of this wave's outstanding memory operations (including the
// direct-to-LDS loads) to complete; a barrier after it publishes the tile.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
// Wait until at most N vector memory operations of this wave are
// outstanding (they complete in issue order), leaving the LDS and export
// counters alone: gfx9 s_waitcnt packs vmcnt[3:0] at bits 3:0 and vmcnt[5:4]
// at bits 15:14, with expcnt (bits 6:4) and lgkmcnt (bits 11:8) at their
// no-wait maxima.
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most N vector memory operations and no LDS operation of this
// wave are outstanding.
template <int N> __device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
// Wait for every outstanding LDS read of this wave.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

// v ^ K as one v_xor_b32 that the compiler can neither hoist out of a loop
// nor merge with another: LDS offsets formed this way are recomputed at
// each use (one VALU op) instead of each holding a register for the whole
// loop.  K == 0 is v itself.
template <uint32_t K> __device__ __forceinline__ uint32_t xor_at_use(uint32_t v) {
  if constexpr (K == 0) {
    return v;
  } else {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(K), "v"(v));
    return r;
  }
}

// An empty side-effecting statement.  Placed inside a wave-uniform `if`, it
// keeps the compiler from if-converting the block into unconditional
// per-element selects (which it otherwise does for cheap-looking bodies):
// the branch stays a scalar branch and the skipped work costs nothing.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// A operand from a tile stored as X[m][k] (k contiguous), rows permuted by
// sig: lane gets X[mb + sig(l32)][kb + 8g + e].
template <int D, typename T>
__device__ __forceinline__ u32x4 lds_rowA(const T* buf, int mb, int kb, int lane) {
  int row = mb + sig(lane & 31);
  int col = kb + 8 * (lane >> 5);
  return *reinterpret_cast<const u32x4*>(buf + Lds<D>::off(row, col));
}

// A operand from a tile stored as X[k][m] (m contiguous) via the gfx950
// transposing read: lane gets X[kb + 8g + e][mb + l32], e = 0..7.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i & 3) of the 8-byte chunks addressed by lanes (i >> 2) + 4t, t = 0..3.
template <int D, typename T>
__device__ __forceinline__ u32x4 lds_trA(const T* buf, int kb, int mb, int lane) {
  int i = lane & 15, G = lane >> 4;
  int row = kb + 8 * (G >> 1) + (i >> 2);
  int col = mb + 16 * (G & 1) + 4 * (i & 3);
  const T* p0 = buf + Lds<D>::off(row, col);
  const T* p1 = buf + Lds<D>::off(row + 4, col);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// 32-bit LDS byte address of a pointer into __shared__ memory, and loads
// from such an address.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) { return *(const lds_u32x4*)(uintptr_t)addr; }
__device__ __forceinline__ s16x4 lds_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
}

// Register-lean readers for the two A-operand patterns above.  For rows of
// 64 or 128 elements the swizzled byte offset of every access a lane makes
// is (per-lane base) XOR (compile-time constant) plus a compile-time row
// offset: the XOR only touches bits below the row size and the per-lane
// base's row part has those bits clear.  So a lane keeps one (rows) or two
// (transposing) base registers, and each access costs at most one v_xor.
// Other widths use the general offset computation.
// refresh() is called once per loop trip: the XORed offsets are then formed
// once per trip (shared by every row block) and die within it.
template <int D, typename T> struct RowReader {
  static constexpr bool FAST = (D == 64 || D == 128);
  uint32_t pre;  // byte offset of (row sig(l32), chunk g), swizzled
  int lane_;
  __device__ __forceinline__ void init(int lane) {
    lane_ = lane;
    const int row = sig(lane & 31), g = lane >> 5;
    pre = (uint32_t)(row * D * 2 + 16 * (g ^ Lds<D>::swz(row)));
  }
  // A tile whose buffer changes from trip to trip: the buffer's address is
  // folded into the per-lane offset once (one VALU op) and each read then
  // costs at most one XOR.  Buffers must be 256-byte aligned, so that adding
  // the base leaves the XORed bits alone.
  struct View {
    uint32_t bp;
    const T* tile;
    int lane;
    template <int T_> __device__ __forceinline__ u32x4 read(int mb) const {
      if constexpr (FAST) return lds_load16(xor_at_use<32u * T_>(bp) + (uint32_t)(mb * D * 2));
      else return lds_rowA<D>(tile, mb, 16 * T_, lane);
    }
  };
  __device__ __forceinline__ View view(const T* tile) const {
    return View{lds_addr(tile) + pre, tile, lane_};
  }
  // read<T_>(tile, 32 b) for b = 0 .. NB-1, sharing the swizzled offset
  template <int T_, int NB>
  __device__ __forceinline__ void read_blocks(const T* tile, u32x4 (&out)[NB]) const {
    if constexpr (FAST) {
      const uint32_t off = xor_at_use<32u * T_>(pre);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        out[b] = *reinterpret_cast<const u32x4*>((const char*)tile + off + (uint32_t)(32 * b * D * 2));
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) out[b] = lds_rowA<D>(tile, 32 * b, 16 * T_, lane_);
    }
  }
  // X[mb + sig(l32)][16 t + 8g + e]; mb a multiple of 32
  template <int T_>
  __device__ __forceinline__ u32x4 read(const T* tile, int mb) const {
    if constexpr (FAST) {
      const uint32_t off = xor_at_use<32u * T_>(pre) + (uint32_t)(mb * D * 2);
      return *reinterpret_cast<const u32x4*>((const char*)tile + off);
    } else {
      return lds_rowA<D>(tile, mb, 16 * T_, lane_);
    }
  }
};

// HOIST: keep the swizzled offsets of every 32-column block in registers
// (2 D / 32 of them) instead of forming each with a v_xor at its read, for
// kernels with registers to spare and vector work to save.
template <int D, typename T, bool HOIST = false> struct TrReader {
  static constexpr bool FAST = (D == 64 || D == 128);
  static constexpr int NX = HOIST ? D / 32 : 1;
  uint32_t pre[2];  // byte offsets of the two 4-row halves at kb = mb = 0
  uint32_t px[NX][2];  // (HOIST) pre[h] ^ 64 m: the halves' offsets at MB = 32 m
  int lane_;
  __device__ __forceinline__ void init(int lane) {
    lane_ = lane;
    const int i = lane & 15, G = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * (G >> 1) + 4 * h + (i >> 2);
      const int col = 16 * (G & 1) + 4 * (i & 3);
      pre[h] = (uint32_t)(2 * Lds<D>::off(row, col));
#pragma unroll
      for (int m = 0; m < NX; ++m) px[m][h] = pre[h] ^ (uint32_t)(64 * m);
    }
  }
  struct View {
    uint32_t bp0, bp1;
    const T* tile;
    int lane;
    template <int MB> __device__ __forceinline__ u32x4 read(int kb) const {
      if constexpr (FAST) {
        constexpr uint32_t x = (uint32_t)(64 * (MB / 32));
        const uint32_t kbo = (uint32_t)(kb * D * 2);
        s16x4 lo = lds_tr8(xor_at_use<x>(bp0) + kbo), hi = lds_tr8(xor_at_use<x>(bp1) + kbo);
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      } else {
        return lds_trA<D>(tile, kb, MB, lane);
      }
    }
  };
  // as RowReader::view (256-byte aligned buffers)
  __device__ __forceinline__ View view(const T* tile) const {
    const uint32_t base = lds_addr(tile);
    return View{base + pre[0], base + pre[1], tile, lane_};
  }
  // X[kb + 8g + e][MB + l32], e = 0..7; kb a multiple of 16, MB of 32
  template <int MB>
  __device__ __forceinline__ u32x4 read(const T* tile, int kb) const {
    if constexpr (FAST) {
      const char* base = (const char*)tile + kb * D * 2;
      constexpr uint32_t x = (uint32_t)(64 * (MB / 32));
      const uint32_t o0 = HOIST ? px[MB / 32][0] : xor_at_use<x>(pre[0]);
      const uint32_t o1 = HOIST ? px[MB / 32][1] : xor_at_use<x>(pre[1]);
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o0));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o1));
      u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    } else {
      return lds_trA<D>(tile, kb, MB, lane_);
    }
  }
};

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw; SC'11) -------------------
struct Philox {
  __device__ __forceinline__ static void block(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1,
                                               uint32_t out[4]) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
      uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
      uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
      c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
  }
};

// Dropout keep bytes for 8 patches of 4x4 (query, key) positions shared by a
// quad of lanes.  The quad (lanes 4a..4a+3) shares the fixed coordinate's
// patch index `fix4` (= fixed >> 2); each of the quad's lanes computes two
// of the 8 patches and the results are exchanged with DPP so that every lane
// ends up with, for each patch k, the dword whose byte b belongs to varying
// coordinate 4*var4[k] + b:
//   ROW_FIXED (lane owns query row i, patches run along keys j):
//        counter (var4[k], fix4, bh, off); the lane needs word (i & 3).
//   !ROW_FIXED (lane owns key j, patches run along queries i):
//        counter (fix4, var4[k], bh, off); the lane needs byte (j & 3) of
//        each of the 4 words, packed into one dword.
template <bool ROW_FIXED>
__device__ __forceinline__ void quad_keep_words(const uint32_t var4[8], uint32_t fix4,
                                                uint32_t bh, uint32_t off, uint32_t k0,
                                                uint32_t k1, int lane, uint32_t out[8]) {
  const int c = lane & 3;  // my position in the quad = my fixed coordinate & 3
  // patches 2c and 2c+1 are computed here
  uint32_t w[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // var4[2c + s] by selects on register copies (the compiler turns a
    // lane-dependent index, or selects of array elements, into a load from
    // scratch memory)
    uint32_t a0 = var4[s], a1 = var4[2 + s], a2 = var4[4 + s], a3 = var4[6 + s];
    __asm__ volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    uint32_t v4 = (c == 1) ? a1 : a0;
    v4 = (c == 2) ? a2 : v4;
    v4 = (c == 3) ? a3 : v4;
    if (ROW_FIXED)
      Philox::block(v4, fix4, bh, off, k0, k1, w[s]);
    else
      Philox::block(fix4, v4, bh, off, k0, k1, w[s]);
  }
  // what a reader at quad position q wants from one patch
  auto want = [&](int s, int q) -> uint32_t {
    if (ROW_FIXED) {
      uint32_t x = w[s][0];
      x = (q == 1) ? w[s][1] : x;
      x = (q == 2) ? w[s][2] : x;
      x = (q == 3) ? w[s][3] : x;
      return x;
    } else {
      int sh = 8 * q;
      return ((w[s][0] >> sh) & 0xffu) | (((w[s][1] >> sh) & 0xffu) << 8) |
             (((w[s][2] >> sh) & 0xffu) << 16) | (((w[s][3] >> sh) & 0xffu) << 24);
    }
  };
  // round rho: reader c pulls from source c ^ rho, which computed patches
  // 2(c^rho) and 2(c^rho)+1 and sends the part meant for quad position c.
  uint32_t r0[2], r1[2], r2[2], r3[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    r0[s] = want(s, c);
    r1[s] = quad_xor<1>(want(s, c ^ 1));
    r2[s] = quad_xor<2>(want(s, c ^ 2));
    r3[s] = quad_xor<3>(want(s, c ^ 3));
  }
  // r_rho[s] holds patch 2(c^rho)+s
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int src = k >> 1, s = k & 1;
    int rho = src ^ c;
    uint32_t x = r0[s];
    x = (rho == 1) ? r1[s] : x;
    x = (rho == 2) ? r2[s] : x;
    x = (rho == 3) ? r3[s] : x;
    out[k] = x;
  }
}

}  // namespace sdpa
