// Kernel argument blocks and launcher declarations shared by the host API
// (sdpa_api.cpp) and the kernels (sdpa_*.hip).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

enum class IoType : int { F32 = 0, F16 = 1, BF16 = 2 };

// Strides in elements; the innermost dimension is contiguous.
struct Str {
  int64_t b, h, s;
};

// Where the sequences of one batch entry live.  In batch mode every entry
// has s_q / s_kv rows starting at row 0 of its (b, h) slice; in group mode
// the rows of sequence b start at token cu_q[b] (cu_kv[b]) of a packed
// tensor and the batch stride is unused.
struct SeqInfo {
  const int32_t* cu_q;   // null in batch mode
  const int32_t* cu_kv;
  int32_t s_q, s_kv;     // batch mode lengths (group mode: maxima, grid sizing only)
  int64_t t_q;           // group mode: row count of the LSE [h, t_q]; 0 = cu_q[b]
};

struct DropoutArgs {
  int32_t enabled;                  // p > 0
  uint32_t threshold;               // keep iff random byte >= threshold
  float rescale;                    // 1 / (1 - p)
  uint64_t seed, offset;            // used when seed_offset_dev is null
  const uint64_t* seed_offset_dev;  // optional device {seed, offset}
};

constexpr int32_t kBandInf = 1 << 30;

struct FwdArgs {
  const void *q, *k, *v, *bias;
  void* o;
  float* lse;       // nullable
  uint8_t* keep;    // nullable, dense [B,H,S_q,S_kv], batch mode only
  Str sq_, sk_, sv_, sb_, so_;
  int32_t bias_vec;  // bias rows 16-byte aligned: vector loads allowed
  int32_t B, H;
  int32_t G;           // query heads per key/value head (K/V head of h is h / G)
  // band mask: key j visible from row i iff lo <= j - i - off <= hi, with
  // off = s_kv - s_q (per sequence) when band_br, else 0; +-kBandInf = unbounded
  int32_t band_br, band_lo, band_hi;
  // ALiBi (nullable; then the BIAS kernels take it in place of the bias
  // tensor): s_ij += -alibi[b * alibi_sb + h] * |j - i - off|, off = s_kv -
  // s_q (per sequence) when alibi_br, else 0
  const float* alibi;
  int64_t alibi_sb;
  int32_t alibi_br;
  SeqInfo seq;
  float scale;         // scaling_factor
  float scale_log2;    // scaling_factor * log2(e)
  DropoutArgs drop;
  // launch configuration (LaunchConfig below): heads per L2 group in the
  // XCD placement, and the workgroup count of the streamed instances (host)
  int32_t head_group;
  int32_t grid_cap;
};

struct BwdArgs {
  const void *q, *k, *v, *bias, *o, *dout;
  const float* lse;  // forward stats (natural log), read by the preprocess only
  // backward stats written by the preprocess: D and LSE*log2(e), each dense
  // batch [B,H,S_q] or group [H, B*S_q]
  float* dvec;
  float* lse2;
  void *dq, *dk, *dv, *dbias;
  Str sq_, sk_, sv_, sb_, so_, sdo_, sdq_, sdk_, sdv_, sdb_;
  int32_t bias_vec;
  int32_t B, H;
  int32_t G;  // query heads per key/value head (K/V head of h is h / G)
  // band mask: key j visible from row i iff lo <= j - i - off <= hi, with
  // off = s_kv - s_q (per sequence) when band_br, else 0; +-kBandInf = unbounded
  int32_t band_br, band_lo, band_hi;
  // ALiBi, as in FwdArgs
  const float* alibi;
  int64_t alibi_sb;
  int32_t alibi_br;
  SeqInfo seq;
  float scale, scale_log2;
  DropoutArgs drop;
  // launch configuration (LaunchConfig below): heads per L2 group of the dQ
  // and dK/dV placements, and the dK/dV workgroup count when streamed (host)
  int32_t dq_head_group, dkdv_head_group;
  int32_t dkdv_grid_cap;
};

// Thin-query forward (split-KV).  Each split of the keys writes a normalised
// partial O and its natural-log LSE for every row, at row index st (the
// dense stats index: batch (b H + h) s_q + s, group h T + token) of slice
// `split`; a combine kernel merges them.  With ns == 1 the kernel writes O
// and LSE itself and no partials are used.
struct DecodeArgs {
  float* part_o;    // [ns][nr][d_v]
  float* part_lse;  // [ns][nr]
  int64_t nr;       // rows per slice: B * H * s_q
  int32_t ns;       // splits
  int32_t chunk;    // keys per split, a multiple of 128
  int32_t rg;       // 32-row groups of (query head of the group, position) pairs
  // quantized K/V (k_sc non-null; a.k, a.v then hold int8 codes, or 4-bit
  // codes two per byte, with byte strides): per (token, group of qgs
  // head-dim elements) fp32 scales and nullable int8 zero points, at element
  // strides ss (group index unit)
  const float *k_sc, *v_sc;
  const int8_t *k_zp, *v_zp;
  Str ss;
  int32_t qgs;
  int32_t qfmt;  // codes: 1 int8, 2 signed 4-bit, 3 unsigned 4-bit (0: 16-bit K/V)
};
struct DecodePlan {
  int32_t ns, chunk, rg;
};
// Splits for about `target_wgs` workgroups over B x (H / G) x row groups.
DecodePlan plan_decode(int64_t B, int64_t H, int32_t G, int64_t s_q, int64_t s_kv,
                       int64_t target_wgs);
constexpr int64_t kDecodeMaxSq = 16;  // thin-query path: s_q <= 16

// With SDPA_LOG set in the environment: one stderr line per kernel launch
// naming the kernel instance (io type, head dims, mask / bias / dropout
// flags), its tile shape and its grid, as oneDNN's SDPA driver prints the
// configuration it chose.  Host only.
// Launch configuration of the tile kernels.  The tile shapes are fixed by
// the compiled instances; what a launch chooses at run time is the XCD
// placement's head-group size (heads whose tiles share an L2 at a time) and
// how many workgroups the streamed instances (batch mode, no bias, no
// dropout) run: -1 = one per concurrent slot (occupancy x compute units),
// 0 = one unit per workgroup, n > 0 = n (a multiple of 8).  The defaults
// can be overridden through the environment, as oneDNN's SDPA_CONFIG and
// BWD_SDPA_CONFIG override its tile choices:
//   SDPA_FWD_CONFIG="heads=4,wgs=512"
//   SDPA_BWD_CONFIG="dq_heads=4,dkdv_heads=2,dkdv_wgs=256"
// (any subset of the keys).  Results do not depend on these settings.
// Packed variable-length batches (group mode) start from their own head
// groups (measured on 16 sequences of U[64, 4096] tokens, H16 d128, causal:
// forward 648 -> 569 us with 2, dQ 868 -> 702 us and dK/dV 1333 -> 1016 us
// with 1).
struct LaunchConfig {
  int fwd_heads = 4, fwd_wgs = -1;
  int dq_heads = 4;
  int dkdv_heads = 2, dkdv_wgs = -1;
  static LaunchConfig defaults(bool group_mode) {
    LaunchConfig c;
    if (group_mode) {
      c.fwd_heads = 2;
      c.dq_heads = 1;
      c.dkdv_heads = 1;
    }
    return c;
  }
};

bool log_enabled();
// Compute units of the current device (0 if the runtime cannot say); the
// persistent launches size their grids by it.  Host only.
int device_cus();
void log_launch(const char* kernel, IoType t, int dqk, int dv, bool band, bool bias, bool drop,
                const char* tile, dim3 grid, dim3 block);

// Launchers (each returns hipSuccess or the launch error).  `causal`,
// `bias` and `dropout` select template instances.
hipError_t launch_fwd(IoType t, int dqk, int dv, bool causal, const FwdArgs& a,
                      hipStream_t st);
hipError_t launch_bwd_pre(IoType t, int dv, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(IoType t, int dqk, int dv, bool causal, const BwdArgs& a,
                           hipStream_t st);
// with_pre: the dQ kernel also writes the stats (D, LSE*log2e) of its rows
// from o, dout and lse (16-bit io only)
hipError_t launch_bwd_dq(IoType t, int dqk, int dv, bool causal, const BwdArgs& a,
                         hipStream_t st, bool with_pre = false);
hipError_t launch_fwd_decode(IoType t, int dqk, int dv, bool band, const FwdArgs& a,
                             const DecodeArgs& d, hipStream_t st);
bool mfma_dims_supported(int dqk, int dv);

}  // namespace sdpa
