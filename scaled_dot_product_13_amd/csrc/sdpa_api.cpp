// Host side of the C ABI declared in include/sdpa.h: argument validation,
// workspace sizing and kernel launches on the caller's stream.
//
// Behaviour taken from the pages' host drivers:
//   - zero-element problems return success without launching (PyTorch
//     "MHA.cpp", run_cudnn_SDP_fprop / run_cudnn_SDP_bprop early return);
//   - the backward is a preprocess (D) plus main kernels, with a workspace
//     the caller provides (oneDNN micro SDPA host driver, init_scratchpad and
//     execute_backward; the cuDNN glue's workspace);
//   - errors are reported as status codes with a message (oneDNN's status
//     codes and VCHECK_SDPA_COND messages), never as exceptions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/sdpa.h"
#include "sdpa_params.h"

namespace {

thread_local char g_msg[512] = "";

sdpa_status_t fail(sdpa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  if (std::getenv("SDPA_LOG")) std::fprintf(stderr, "[sdpa] %s\n", g_msg);
  return st;
}

bool log_on() {
  static int on = std::getenv("SDPA_LOG") ? 1 : 0;
  return on != 0;
}

size_t elem_size(sdpa_dtype_t t) { return t == SDPA_F32 ? 4 : 2; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

sdpa_status_t check_problem(const sdpa_problem_t* p) {
  if (!p) return fail(SDPA_ERR_INVALID_ARG, "problem is null");
  if (p->struct_size != sizeof(sdpa_problem_t))
    return fail(SDPA_ERR_INVALID_ARG, "problem.struct_size is %u, expected %zu", p->struct_size,
                sizeof(sdpa_problem_t));
  if (p->dtype != SDPA_F32 && p->dtype != SDPA_F16 && p->dtype != SDPA_BF16)
    return fail(SDPA_ERR_INVALID_ARG, "unknown dtype %d", (int)p->dtype);
  if (p->b < 0 || p->h < 0 || p->s_q < 0 || p->s_kv < 0)
    return fail(SDPA_ERR_INVALID_ARG, "negative size (b=%lld h=%lld s_q=%lld s_kv=%lld)",
                (long long)p->b, (long long)p->h, (long long)p->s_q, (long long)p->s_kv);
  if (p->d_qk <= 0 || p->d_v <= 0)
    return fail(SDPA_ERR_INVALID_ARG, "head dims must be positive (d_qk=%lld d_v=%lld)",
                (long long)p->d_qk, (long long)p->d_v);
  if (p->b > 65535 || p->h > 65535 || p->s_q > (1 << 30) || p->s_kv > (1 << 30))
    return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the supported grid (b, h <= 65535)");
  if (!(p->dropout_probability >= 0.f && p->dropout_probability < 1.f))
    return fail(SDPA_ERR_INVALID_ARG, "dropout_probability %g outside [0, 1)",
                (double)p->dropout_probability);
  if (p->dropout_probability > 0.f) {
    // the 8-bit threshold round(256 p) must be in [1, 255]: p below 1/512
    // would keep every element (while still rescaling by 1/(1-p)), p above
    // 255/256 would saturate the threshold
    const double t = std::floor(256.0 * (double)p->dropout_probability + 0.5);
    if (t < 1.0 || (double)p->dropout_probability > 255.0 / 256.0)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "dropout_probability %g: the 8-bit keep threshold round(256 p) = %g must lie "
                  "in [1, 255] (p in [1/512, 255/256])", (double)p->dropout_probability, t);
  }
  if (p->total_q < 0) return fail(SDPA_ERR_INVALID_ARG, "total_q is negative");
  if (!std::isfinite(p->scaling_factor))
    return fail(SDPA_ERR_INVALID_ARG, "scaling_factor is not finite");
  if (p->h_kv < 0 || (p->h_kv > 0 && p->h % p->h_kv != 0))
    return fail(SDPA_ERR_INVALID_ARG, "h_kv=%lld must be 0 or divide h=%lld", (long long)p->h_kv,
                (long long)p->h);
  if (p->mask_flags & ~(SDPA_MASK_BOTTOM_RIGHT | SDPA_MASK_WINDOW))
    return fail(SDPA_ERR_INVALID_ARG, "unknown mask_flags bits 0x%x", p->mask_flags);
  if (p->alibi_slopes && p->alibi_batch_stride < 0)
    return fail(SDPA_ERR_INVALID_ARG, "alibi_batch_stride is negative");
  if (p->kv_quant != SDPA_KV_QUANT_NONE && p->kv_quant != SDPA_KV_QUANT_S8 &&
      p->kv_quant != SDPA_KV_QUANT_S4 && p->kv_quant != SDPA_KV_QUANT_U4)
    return fail(SDPA_ERR_INVALID_ARG, "unknown kv_quant %d", p->kv_quant);
  if ((p->cu_seqlens_q == nullptr) != (p->cu_seqlens_kv == nullptr))
    return fail(SDPA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_kv must both be set or both null");
  if (p->dtype == SDPA_F32) {
    if (p->d_qk > 256 || p->d_v > 256)
      return fail(SDPA_ERR_UNSUPPORTED, "fp32 head dims must be <= 256 (d_qk=%lld d_v=%lld)",
                  (long long)p->d_qk, (long long)p->d_v);
    if (p->d_v % 4 != 0)
      return fail(SDPA_ERR_UNSUPPORTED, "fp32 d_v must be a multiple of 4");
  } else if (!sdpa::mfma_dims_supported((int)p->d_qk, (int)p->d_v)) {
    return fail(SDPA_ERR_UNSUPPORTED,
                "no 16-bit kernel for d_qk=%lld d_v=%lld (compiled: 64/64, 128/128, 192/128)",
                (long long)p->d_qk, (long long)p->d_v);
  }
  return SDPA_OK;
}

// query heads per key/value head
int32_t kv_group(const sdpa_problem_t* p) { return p->h_kv > 0 ? (int32_t)(p->h / p->h_kv) : 1; }

// Band of the mask (see sdpa_problem_t): returns whether any key is masked
// by it; lo, hi are clamped to +-kBandInf (sequence lengths are <= 2^30).
bool band_of(const sdpa_problem_t* p, int32_t& br, int32_t& lo, int32_t& hi) {
  const int64_t inf = sdpa::kBandInf;
  const bool win = (p->mask_flags & SDPA_MASK_WINDOW) != 0;
  int64_t l = (win && p->window_left >= 0) ? -std::min(p->window_left, inf) : -inf;
  int64_t h = (win && p->window_right >= 0) ? std::min(p->window_right, inf) : inf;
  if (p->is_causal) h = std::min<int64_t>(h, 0);
  br = (p->mask_flags & SDPA_MASK_BOTTOM_RIGHT) ? 1 : 0;
  lo = (int32_t)l;
  hi = (int32_t)h;
  return l > -inf || h < inf;
}
// ALiBi alignment: the mask's, and bottom-right when there is no mask.
int32_t alibi_bottom_right(const sdpa_problem_t* p) {
  const bool masked = p->is_causal || (p->mask_flags & SDPA_MASK_WINDOW);
  return (!masked || (p->mask_flags & SDPA_MASK_BOTTOM_RIGHT)) ? 1 : 0;
}
template <typename Args> void fill_alibi(const sdpa_problem_t* p, Args& a) {
  a.alibi = p->alibi_slopes;
  a.alibi_sb = p->alibi_batch_stride;
  a.alibi_br = alibi_bottom_right(p);
}

bool banded(const sdpa_problem_t* p) {
  int32_t br, lo, hi;
  return band_of(p, br, lo, hi);
}

bool empty_problem(const sdpa_problem_t* p) {
  return p->b == 0 || p->h == 0 || p->s_q == 0 || p->s_kv == 0;
}

// A tensor operand: non-null, non-negative strides; for 16-bit io the
// vectorised kernels need 16-byte aligned rows.
sdpa_status_t check_tensor(const sdpa_problem_t* p, const void* ptr, sdpa_strides_t s,
                           const char* name, bool need_vec) {
  if (!ptr) return fail(SDPA_ERR_INVALID_ARG, "%s is null", name);
  if (s.batch < 0 || s.head < 0 || s.seq < 0)
    return fail(SDPA_ERR_INVALID_ARG, "%s has a negative stride", name);
  if (need_vec) {
    size_t es = elem_size(p->dtype);
    bool ok = ((uintptr_t)ptr % 16 == 0) && (s.head * es) % 16 == 0 && (s.seq * es) % 16 == 0 &&
              (p->cu_seqlens_q || (s.batch * es) % 16 == 0);
    if (!ok)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "%s: base pointer and batch/head/seq strides must be multiples of 16 bytes", name);
    // tile loaders keep 32-bit byte offsets within a 128-row tile
    if (s.seq * (int64_t)es > (int64_t)1 << 24)
      return fail(SDPA_ERR_UNSUPPORTED, "%s: row (seq) stride above 16 MiB", name);
  }
  return SDPA_OK;
}

sdpa::Str to_str(sdpa_strides_t s) { return sdpa::Str{s.batch, s.head, s.seq}; }

void fill_dropout(const sdpa_problem_t* p, sdpa::DropoutArgs& d) {
  float pr = p->dropout_probability;
  d.enabled = pr > 0.f ? 1 : 0;
  double t = std::floor(256.0 * (double)pr + 0.5);
  if (t > 255.0) t = 255.0;
  d.threshold = (uint32_t)t;
  d.rescale = pr > 0.f ? (float)(1.0 / (1.0 - (double)pr)) : 1.f;
  d.seed = p->dropout_seed;
  d.offset = p->dropout_offset;
  d.seed_offset_dev = p->dropout_seed_offset_dev;
}

sdpa::SeqInfo seq_info(const sdpa_problem_t* p) {
  sdpa::SeqInfo s;
  s.cu_q = p->cu_seqlens_q;
  s.cu_kv = p->cu_seqlens_kv;
  s.s_q = (int32_t)p->s_q;
  s.s_kv = (int32_t)p->s_kv;
  s.t_q = p->cu_seqlens_q ? p->total_q : 0;
  return s;
}

sdpa::IoType io(sdpa_dtype_t t) {
  return t == SDPA_F32 ? sdpa::IoType::F32 : t == SDPA_F16 ? sdpa::IoType::F16 : sdpa::IoType::BF16;
}

bool bias_vec_ok(const sdpa_problem_t* p, const void* bias, sdpa_strides_t s) {
  size_t es = elem_size(p->dtype);
  return bias && (uintptr_t)bias % 16 == 0 && (s.batch * es) % 16 == 0 &&
         (s.head * es) % 16 == 0 && (s.seq * es) % 16 == 0 && s.seq * (int64_t)es <= (int64_t)1 << 24;
}

// Backward stats: D = rowsum(dO o O), then LSE * log2(e), each n floats
// (n = b*h*s_q), the second array starting at the next 256-byte boundary.
size_t stats_half_bytes(const sdpa_problem_t* p) {
  return align_up(sizeof(float) * (size_t)p->b * (size_t)p->h * (size_t)p->s_q);
}
size_t d_workspace_bytes(const sdpa_problem_t* p) { return 2 * stats_half_bytes(p); }
float* stats_lse2(const sdpa_problem_t* p, const float* stats) {
  return (float*)((const char*)stats + stats_half_bytes(p));
}

// Thin-query forward: 16-bit io, at most kDecodeMaxSq query rows per
// sequence, no bias and no dropout (SDPA_DECODE=0 turns the path off).
bool decode_eligible(const sdpa_problem_t* p, bool has_bias) {
  static const bool off = [] {
    const char* e = std::getenv("SDPA_DECODE");
    return e && e[0] == '0';
  }();
  return !off && p->dtype != SDPA_F32 && !has_bias && p->dropout_probability == 0.f &&
         p->s_q <= sdpa::kDecodeMaxSq;
}
// Workgroups the split-KV plan aims for (SDPA_DECODE_WGS overrides).
int64_t decode_target_wgs() {
  static const int64_t n = [] {
    const char* e = std::getenv("SDPA_DECODE_WGS");
    const long long v = e ? std::atoll(e) : 0;
    return v > 0 ? (int64_t)v : (int64_t)256;
  }();
  return n;
}
// Quantized K/V: everything the thin-query kernel's quantized modes assume.
sdpa_status_t check_kv_quant(const sdpa_problem_t* p, bool has_bias, const void* k,
                             sdpa_strides_t k_s, const void* v, sdpa_strides_t v_s) {
  if (p->dtype == SDPA_F32 || has_bias || p->dropout_probability > 0.f || p->s_q > sdpa::kDecodeMaxSq)
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V needs a thin-query forward: 16-bit q, s_q <= %lld, "
                "no bias, ALiBi or dropout", (long long)sdpa::kDecodeMaxSq);
  if (!decode_eligible(p, false))
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V needs the thin-query kernel (SDPA_DECODE=0 is set)");
  if (p->d_qk != 128 || p->d_v != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V needs d_qk = d_v = 128");
  const int g = p->kv_group_size;
  const bool four = p->kv_quant != SDPA_KV_QUANT_S8;
  if (!(g == 32 || g == 64 || g == 128 || (g == 16 && !four)))
    return fail(SDPA_ERR_UNSUPPORTED, "kv_group_size %d not in {%s32, 64, 128}", g, four ? "" : "16, ");
  if (!p->k_scales || !p->v_scales) return fail(SDPA_ERR_INVALID_ARG, "k_scales / v_scales are null");
  if ((p->k_zero_points == nullptr) != (p->v_zero_points == nullptr))
    return fail(SDPA_ERR_INVALID_ARG, "k_zero_points and v_zero_points must both be set or both null");
  const sdpa_strides_t ss = p->kv_scale_strides;
  if (ss.batch < 0 || ss.head < 0 || ss.seq < 0)
    return fail(SDPA_ERR_INVALID_ARG, "kv_scale_strides has a negative stride");
  const bool group = p->cu_seqlens_q != nullptr;
  for (int i = 0; i < 2; ++i) {
    const void* t = i ? v : k;
    const sdpa_strides_t s = i ? v_s : k_s;
    if ((uintptr_t)t % 16 || s.head % 16 || s.seq % 16 || (!group && s.batch % 16))
      return fail(SDPA_ERR_UNSUPPORTED, "quantized %s: base and strides must be multiples of 16 bytes",
                  i ? "v" : "k");
  }
  return SDPA_OK;
}

sdpa::DecodePlan decode_plan(const sdpa_problem_t* p) {
  return sdpa::plan_decode(p->b, p->h, kv_group(p), p->s_q, p->s_kv, decode_target_wgs());
}
// Rows of one split-KV partial slice: the row index is the LSE index
// (batch (b H + h) s_q + s; group h total_q + token, where every token is
// below b s_q when total_q is not given).
int64_t decode_rows(const sdpa_problem_t* p) {
  if (p->cu_seqlens_q && p->total_q > 0) return p->h * p->total_q;
  return p->b * p->h * p->s_q;
}
// split-KV partials: O [ns][rows][d_v] fp32, then LSE [ns][rows]
size_t decode_part_o_bytes(const sdpa_problem_t* p, const sdpa::DecodePlan& pl) {
  return align_up(sizeof(float) * (size_t)pl.ns * (size_t)decode_rows(p) * (size_t)p->d_v);
}
size_t decode_workspace_bytes(const sdpa_problem_t* p, const sdpa::DecodePlan& pl) {
  if (pl.ns <= 1) return 0;
  return decode_part_o_bytes(p, pl) + align_up(sizeof(float) * (size_t)pl.ns * (size_t)decode_rows(p));
}

// ---- the no-allocation backward's stats array -------------------------------
// File-scope device memory, one copy per GPU: D then LSE*log2(e), each
// SDPA_NOALLOC_MAX_ROWS floats (the layout of the backward workspace for
// any problem within the limit: stats_half_bytes(p) <= 4 * MAX_ROWS).  Host
// code never uses the name `scratch` itself (on the host it is a stand-in,
// not a device address): its per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kNoAllocRows = SDPA_NOALLOC_MAX_ROWS;
__device__ __attribute__((aligned(256))) float scratch[2 * kNoAllocRows];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];

sdpa_status_t noalloc_stats(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SDPA_ERR_UNSUPPORTED, "device %d beyond the %d devices the library tracks", dev,
                kMaxDevices);
  void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SDPA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev].store(ptr, std::memory_order_release);  // same value if two threads race
  }
  *out = ptr;
  return SDPA_OK;
}

// One of SDPA_FWD_CONFIG / SDPA_BWD_CONFIG: comma-separated key=value with
// integer values, keys from `keys` (LaunchConfig in sdpa_params.h).
sdpa_status_t parse_config_env(const char* name, const char* const* keys, int* const* vals, int nk) {
  const char* s = std::getenv(name);
  if (!s || !*s) return SDPA_OK;
  const char* c = s;
  while (*c) {
    const char* eq = std::strchr(c, '=');
    const char* comma = std::strchr(c, ',');
    if (!eq || (comma && comma < eq))
      return fail(SDPA_ERR_INVALID_ARG, "%s: expected key=value items in \"%s\"", name, s);
    const size_t klen = (size_t)(eq - c);
    int idx = -1;
    for (int i = 0; i < nk; ++i)
      if (std::strlen(keys[i]) == klen && std::strncmp(keys[i], c, klen) == 0) idx = i;
    if (idx < 0) return fail(SDPA_ERR_INVALID_ARG, "%s: unknown key \"%.*s\"", name, (int)klen, c);
    char* end = nullptr;
    const long v = std::strtol(eq + 1, &end, 10);
    if (end == eq + 1 || (*end && *end != ',') || v < -1 || v > (1L << 20))
      return fail(SDPA_ERR_INVALID_ARG, "%s: bad value for %s in \"%s\"", name, keys[idx], s);
    *vals[idx] = (int)v;
    c = *end == ',' ? end + 1 : end;
  }
  return SDPA_OK;
}

// The launch configuration: the defaults (batch or group mode), then the
// environment overrides, validated (head groups 1 .. 64; workgroup counts
// -1, 0 or a positive multiple of 8).
sdpa_status_t launch_config(sdpa::LaunchConfig& cfg, bool group_mode) {
  cfg = sdpa::LaunchConfig::defaults(group_mode);
  static const char* const fk[] = {"heads", "wgs"};
  int* const fv[] = {&cfg.fwd_heads, &cfg.fwd_wgs};
  if (sdpa_status_t st = parse_config_env("SDPA_FWD_CONFIG", fk, fv, 2); st != SDPA_OK) return st;
  static const char* const bk[] = {"dq_heads", "dkdv_heads", "dkdv_wgs"};
  int* const bv[] = {&cfg.dq_heads, &cfg.dkdv_heads, &cfg.dkdv_wgs};
  if (sdpa_status_t st = parse_config_env("SDPA_BWD_CONFIG", bk, bv, 3); st != SDPA_OK) return st;
  for (int h : {cfg.fwd_heads, cfg.dq_heads, cfg.dkdv_heads})
    if (h < 1 || h > 64) return fail(SDPA_ERR_INVALID_ARG, "launch config: head groups must be 1 .. 64");
  for (int wgs : {cfg.fwd_wgs, cfg.dkdv_wgs})
    if (wgs > 0 && wgs % 8 != 0)
      return fail(SDPA_ERR_INVALID_ARG, "launch config: workgroup counts must be multiples of 8");
  return SDPA_OK;
}

}  // namespace

namespace sdpa {
bool log_enabled() { return log_on(); }
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
void log_launch(const char* kernel, IoType t, int dqk, int dv, bool band, bool bias, bool drop,
                const char* tile, dim3 grid, dim3 block) {
  if (!log_on()) return;
  static const char* names[] = {"f32", "f16", "bf16"};
  std::fprintf(stderr, "[sdpa] launch %s<%s, d %d/%d, band=%d bias=%d drop=%d> tile: %s grid %u x %u x %u, "
               "block %u\n", kernel, names[(int)t], dqk, dv, (int)band, (int)bias, (int)drop, tile,
               grid.x, grid.y, grid.z, block.x);
}
}  // namespace sdpa

extern "C" {

const char* sdpa_version(void) { return "0.1.0"; }

const char* sdpa_status_string(sdpa_status_t st) {
  switch (st) {
    case SDPA_OK: return "SDPA_OK";
    case SDPA_ERR_INVALID_ARG: return "SDPA_ERR_INVALID_ARG";
    case SDPA_ERR_UNSUPPORTED: return "SDPA_ERR_UNSUPPORTED";
    case SDPA_ERR_WORKSPACE: return "SDPA_ERR_WORKSPACE";
    case SDPA_ERR_HIP: return "SDPA_ERR_HIP";
  }
  return "SDPA_ERR_UNKNOWN";
}

const char* sdpa_last_error_message(void) { return g_msg; }

size_t sdpa_fwd_workspace_size(const sdpa_problem_t* p) {
  if (check_problem(p) != SDPA_OK || empty_problem(p) || !decode_eligible(p, false)) return 0;
  return decode_workspace_bytes(p, decode_plan(p));
}

size_t sdpa_bwd_workspace_size(const sdpa_problem_t* p) {
  if (check_problem(p) != SDPA_OK || empty_problem(p)) return 0;
  return d_workspace_bytes(p);
}

sdpa_status_t sdpa_fwd(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s, const void* k,
                       sdpa_strides_t k_s, const void* v, sdpa_strides_t v_s,
                       const void* attn_bias, sdpa_strides_t bias_s, void* o, sdpa_strides_t o_s,
                       float* softmax_lse, uint8_t* dropout_keep_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (empty_problem(p)) return SDPA_OK;
  const bool vec = p->dtype != SDPA_F32;
  if ((st = check_tensor(p, q, q_s, "q", vec)) != SDPA_OK) return st;
  const bool q8 = p->kv_quant != SDPA_KV_QUANT_NONE;  // quantized K/V codes
  if ((st = check_tensor(p, k, k_s, "k", vec && !q8)) != SDPA_OK) return st;
  if ((st = check_tensor(p, v, v_s, "v", vec && !q8)) != SDPA_OK) return st;
  if ((st = check_tensor(p, o, o_s, "o", vec)) != SDPA_OK) return st;
  const bool group = p->cu_seqlens_q != nullptr;
  if (attn_bias) {
    if (p->alibi_slopes)
      return fail(SDPA_ERR_UNSUPPORTED, "attn_bias and alibi_slopes cannot be combined");
    if (group) return fail(SDPA_ERR_UNSUPPORTED, "attn_bias is not supported in group (varlen) mode");
    if ((st = check_tensor(p, attn_bias, bias_s, "attn_bias", false)) != SDPA_OK) return st;
  }
  if (q8 && (st = check_kv_quant(p, attn_bias || p->alibi_slopes, k, k_s, v, v_s)) != SDPA_OK)
    return st;
  if (dropout_keep_out && group)
    return fail(SDPA_ERR_UNSUPPORTED, "dropout_keep_out is only available in batch mode");

  sdpa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.bias = attn_bias; a.o = o;
  a.lse = softmax_lse;
  a.keep = p->dropout_probability > 0.f ? dropout_keep_out : nullptr;
  a.sq_ = to_str(q_s); a.sk_ = to_str(k_s); a.sv_ = to_str(v_s);
  a.sb_ = to_str(bias_s); a.so_ = to_str(o_s);
  a.bias_vec = bias_vec_ok(p, attn_bias, bias_s) ? 1 : 0;
  a.B = (int32_t)p->b; a.H = (int32_t)p->h; a.G = kv_group(p);
  band_of(p, a.band_br, a.band_lo, a.band_hi);
  fill_alibi(p, a);
  a.seq = seq_info(p);
  a.scale = p->scaling_factor;
  a.scale_log2 = (float)((double)p->scaling_factor * 1.4426950408889634);
  fill_dropout(p, a.drop);
  {
    sdpa::LaunchConfig cfg;
    if ((st = launch_config(cfg, a.seq.cu_q != nullptr)) != SDPA_OK) return st;
    a.head_group = cfg.fwd_heads;
    a.grid_cap = cfg.fwd_wgs;
  }
  if (log_on())
    std::fprintf(stderr, "[sdpa] fwd dtype=%d b=%lld h=%lld s_q=%lld s_kv=%lld d=%lld/%lld causal=%d "
                 "bias=%d p=%g group=%d\n", (int)p->dtype, (long long)p->b, (long long)p->h,
                 (long long)p->s_q, (long long)p->s_kv, (long long)p->d_qk, (long long)p->d_v,
                 p->is_causal, attn_bias != nullptr, (double)p->dropout_probability, group);
  hipError_t e;
  if (decode_eligible(p, attn_bias != nullptr || p->alibi_slopes != nullptr)) {
    // thin query: split-KV when the workspace holds the partials, else one
    // split per (batch, key/value head, row group)
    sdpa::DecodePlan pl = decode_plan(p);
    const size_t need = decode_workspace_bytes(p, pl);
    if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16 != 0)) {
      pl.chunk = (int32_t)((p->s_kv + 127) / 128 * 128);
      pl.ns = 1;
    }
    sdpa::DecodeArgs d{};
    if (q8) {
      d.k_sc = p->k_scales;
      d.v_sc = p->v_scales;
      d.k_zp = p->k_zero_points;
      d.v_zp = p->v_zero_points;
      d.ss = to_str(p->kv_scale_strides);
      d.qgs = p->kv_group_size;
      d.qfmt = p->kv_quant == SDPA_KV_QUANT_S8 ? 1 : p->kv_quant == SDPA_KV_QUANT_S4 ? 2 : 3;
    }
    d.ns = pl.ns;
    d.chunk = pl.chunk;
    d.rg = pl.rg;
    d.nr = decode_rows(p);
    if (pl.ns > 1) {
      d.part_o = (float*)workspace;
      d.part_lse = (float*)((char*)workspace + decode_part_o_bytes(p, pl));
    }
    if (log_on())
      std::fprintf(stderr, "[sdpa] fwd thin-query path: splits=%d chunk=%d row_groups=%d\n", d.ns,
                   d.chunk, d.rg);
    e = sdpa::launch_fwd_decode(io(p->dtype), (int)p->d_qk, (int)p->d_v, banded(p), a, d,
                                (hipStream_t)stream);
  } else {
    e = sdpa::launch_fwd(io(p->dtype), (int)p->d_qk, (int)p->d_v, banded(p), a,
                         (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

static sdpa_status_t fill_bwd_args(const sdpa_problem_t* p, sdpa::BwdArgs& a) {
  sdpa::LaunchConfig cfg;
  if (sdpa_status_t st = launch_config(cfg, p->cu_seqlens_q != nullptr); st != SDPA_OK) return st;
  a.dq_head_group = cfg.dq_heads;
  a.dkdv_head_group = cfg.dkdv_heads;
  a.dkdv_grid_cap = cfg.dkdv_wgs;
  a.B = (int32_t)p->b; a.H = (int32_t)p->h; a.G = kv_group(p);
  band_of(p, a.band_br, a.band_lo, a.band_hi);
  fill_alibi(p, a);
  a.seq = seq_info(p);
  a.scale = p->scaling_factor;
  a.scale_log2 = (float)((double)p->scaling_factor * 1.4426950408889634);
  fill_dropout(p, a.drop);
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd_preprocess(const sdpa_problem_t* p, const void* o, sdpa_strides_t o_s,
                                  const void* d_o, sdpa_strides_t do_s, const float* softmax_lse,
                                  float* stats, void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (p->kv_quant != SDPA_KV_QUANT_NONE)
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V is a forward (inference) feature only");
  if (empty_problem(p)) return SDPA_OK;
  if ((st = check_tensor(p, o, o_s, "o", true)) != SDPA_OK) return st;
  if ((st = check_tensor(p, d_o, do_s, "d_o", true)) != SDPA_OK) return st;
  if (!stats) return fail(SDPA_ERR_INVALID_ARG, "stats is null");
  if (!softmax_lse) return fail(SDPA_ERR_INVALID_ARG, "softmax_lse is null");
  if (p->d_v % (16 / (int)elem_size(p->dtype)) != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "d_v must fill whole 16-byte chunks");
  sdpa::BwdArgs a{};
  if (sdpa_status_t fs = fill_bwd_args(p, a); fs != SDPA_OK) return fs;
  a.o = o; a.dout = d_o; a.so_ = to_str(o_s); a.sdo_ = to_str(do_s);
  a.lse = softmax_lse;
  a.dvec = stats;
  a.lse2 = stats_lse2(p, stats);
  hipError_t e = sdpa::launch_bwd_pre(io(p->dtype), (int)p->d_v, a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "preprocess launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s, const void* k,
                       sdpa_strides_t k_s, const void* v, sdpa_strides_t v_s,
                       const void* attn_bias, sdpa_strides_t bias_s, const void* o,
                       sdpa_strides_t o_s, const void* d_o, sdpa_strides_t do_s,
                       const float* softmax_lse, void* dq, sdpa_strides_t dq_s, void* dk,
                       sdpa_strides_t dk_s, void* dv, sdpa_strides_t dv_s, void* dbias,
                       sdpa_strides_t dbias_s, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (p->kv_quant != SDPA_KV_QUANT_NONE)
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V is a forward (inference) feature only");
  if (empty_problem(p)) return SDPA_OK;
  const bool vec = p->dtype != SDPA_F32;
  if ((st = check_tensor(p, q, q_s, "q", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, k, k_s, "k", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, v, v_s, "v", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, o, o_s, "o", true)) != SDPA_OK) return st;
  if ((st = check_tensor(p, d_o, do_s, "d_o", true)) != SDPA_OK) return st;
  if ((st = check_tensor(p, dq, dq_s, "dq", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, dk, dk_s, "dk", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, dv, dv_s, "dv", vec)) != SDPA_OK) return st;
  if (!softmax_lse) return fail(SDPA_ERR_INVALID_ARG, "softmax_lse is null (the backward needs the stats)");
  const bool group = p->cu_seqlens_q != nullptr;
  if (attn_bias) {
    if (p->alibi_slopes)
      return fail(SDPA_ERR_UNSUPPORTED, "attn_bias and alibi_slopes cannot be combined");
    if (group) return fail(SDPA_ERR_UNSUPPORTED, "attn_bias is not supported in group (varlen) mode");
    if ((st = check_tensor(p, attn_bias, bias_s, "attn_bias", false)) != SDPA_OK) return st;
  }
  if (dbias) {
    if (!attn_bias) return fail(SDPA_ERR_INVALID_ARG, "dbias requires attn_bias");
    if ((st = check_tensor(p, dbias, dbias_s, "dbias", false)) != SDPA_OK) return st;
  }
  if (p->d_v % (16 / (int)elem_size(p->dtype)) != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "d_v must fill whole 16-byte chunks");
  const size_t need = d_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace % 16 != 0)
    return fail(SDPA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  sdpa::BwdArgs a{};
  if (sdpa_status_t fs = fill_bwd_args(p, a); fs != SDPA_OK) return fs;
  a.q = q; a.k = k; a.v = v; a.bias = attn_bias; a.o = o; a.dout = d_o;
  a.lse = softmax_lse;
  a.dvec = (float*)workspace;
  a.lse2 = stats_lse2(p, (const float*)workspace);
  a.dq = dq; a.dk = dk; a.dv = dv; a.dbias = dbias;
  a.sq_ = to_str(q_s); a.sk_ = to_str(k_s); a.sv_ = to_str(v_s); a.sb_ = to_str(bias_s);
  a.so_ = to_str(o_s); a.sdo_ = to_str(do_s); a.sdq_ = to_str(dq_s); a.sdk_ = to_str(dk_s);
  a.sdv_ = to_str(dv_s); a.sdb_ = to_str(dbias_s);
  a.bias_vec = bias_vec_ok(p, attn_bias, bias_s) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  const sdpa::IoType t = io(p->dtype);
  const bool causal = banded(p);
  if (log_on())
    std::fprintf(stderr, "[sdpa] bwd dtype=%d b=%lld h=%lld s_q=%lld s_kv=%lld d=%lld/%lld causal=%d "
                 "bias=%d dbias=%d p=%g group=%d\n", (int)p->dtype, (long long)p->b,
                 (long long)p->h, (long long)p->s_q, (long long)p->s_kv, (long long)p->d_qk,
                 (long long)p->d_v, p->is_causal, attn_bias != nullptr, dbias != nullptr,
                 (double)p->dropout_probability, group);
  hipError_t e;
  if (t != sdpa::IoType::F32) {
    // 16-bit io: the dQ kernel does the preprocess for its rows, then dK/dV
    e = sdpa::launch_bwd_dq(t, (int)p->d_qk, (int)p->d_v, causal, a, s, true);
    if (e == hipSuccess) e = sdpa::launch_bwd_dkdv(t, (int)p->d_qk, (int)p->d_v, causal, a, s);
  } else {
    e = sdpa::launch_bwd_pre(t, (int)p->d_v, a, s);
    if (e == hipSuccess) e = sdpa::launch_bwd_dkdv(t, (int)p->d_qk, (int)p->d_v, causal, a, s);
    if (e == hipSuccess) e = sdpa::launch_bwd_dq(t, (int)p->d_qk, (int)p->d_v, causal, a, s);
  }
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd_noalloc(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s,
                               const void* k, sdpa_strides_t k_s, const void* v,
                               sdpa_strides_t v_s, const void* attn_bias, sdpa_strides_t bias_s,
                               const void* o, sdpa_strides_t o_s, const void* d_o,
                               sdpa_strides_t do_s, const float* softmax_lse, void* dq,
                               sdpa_strides_t dq_s, void* dk, sdpa_strides_t dk_s, void* dv,
                               sdpa_strides_t dv_s, void* dbias, sdpa_strides_t dbias_s,
                               void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (empty_problem(p)) return SDPA_OK;
  const int64_t rows = p->b * p->h * p->s_q;
  if (rows > kNoAllocRows)
    return fail(SDPA_ERR_WORKSPACE, "b*h*s_q = %lld exceeds the no-allocation limit of %lld rows",
                (long long)rows, (long long)kNoAllocRows);
  void* ws = nullptr;
  if ((st = noalloc_stats(&ws)) != SDPA_OK) return st;
  // the stats layout inside the array is the workspace layout of sdpa_bwd
  return sdpa_bwd(p, q, q_s, k, k_s, v, v_s, attn_bias, bias_s, o, o_s, d_o, do_s, softmax_lse,
                  dq, dq_s, dk, dk_s, dv, dv_s, dbias, dbias_s, ws,
                  sizeof(float) * 2 * (size_t)kNoAllocRows, stream);
}

// Shared checks of the operands the dK/dV and dQ kernels read.
static sdpa_status_t check_bwd_inputs(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s,
                                      const void* k, sdpa_strides_t k_s, const void* v,
                                      sdpa_strides_t v_s, const void* attn_bias,
                                      sdpa_strides_t bias_s, const void* d_o, sdpa_strides_t do_s,
                                      const float* stats) {
  sdpa_status_t st;
  if (p->kv_quant != SDPA_KV_QUANT_NONE)
    return fail(SDPA_ERR_UNSUPPORTED, "quantized K/V is a forward (inference) feature only");
  const bool vec = p->dtype != SDPA_F32;
  if ((st = check_tensor(p, q, q_s, "q", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, k, k_s, "k", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, v, v_s, "v", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, d_o, do_s, "d_o", true)) != SDPA_OK) return st;
  if (!stats) return fail(SDPA_ERR_INVALID_ARG, "stats is null (run sdpa_bwd_preprocess first)");
  if (attn_bias) {
    if (p->alibi_slopes)
      return fail(SDPA_ERR_UNSUPPORTED, "attn_bias and alibi_slopes cannot be combined");
    if (p->cu_seqlens_q) return fail(SDPA_ERR_UNSUPPORTED, "attn_bias is not supported in group (varlen) mode");
    if ((st = check_tensor(p, attn_bias, bias_s, "attn_bias", false)) != SDPA_OK) return st;
  }
  if (p->d_v % (16 / (int)elem_size(p->dtype)) != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "d_v must fill whole 16-byte chunks");
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd_dkdv(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s,
                            const void* k, sdpa_strides_t k_s, const void* v, sdpa_strides_t v_s,
                            const void* attn_bias, sdpa_strides_t bias_s, const void* d_o,
                            sdpa_strides_t do_s, const float* stats, void* dk,
                            sdpa_strides_t dk_s, void* dv, sdpa_strides_t dv_s, void* dbias,
                            sdpa_strides_t dbias_s, void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (empty_problem(p)) return SDPA_OK;
  if ((st = check_bwd_inputs(p, q, q_s, k, k_s, v, v_s, attn_bias, bias_s, d_o, do_s, stats)) != SDPA_OK)
    return st;
  const bool vec = p->dtype != SDPA_F32;
  if ((st = check_tensor(p, dk, dk_s, "dk", vec)) != SDPA_OK) return st;
  if ((st = check_tensor(p, dv, dv_s, "dv", vec)) != SDPA_OK) return st;
  if (dbias) {
    if (!attn_bias) return fail(SDPA_ERR_INVALID_ARG, "dbias requires attn_bias");
    if ((st = check_tensor(p, dbias, dbias_s, "dbias", false)) != SDPA_OK) return st;
  }
  sdpa::BwdArgs a{};
  if (sdpa_status_t fs = fill_bwd_args(p, a); fs != SDPA_OK) return fs;
  a.q = q; a.k = k; a.v = v; a.bias = attn_bias; a.dout = d_o;
  a.dvec = (float*)stats; a.lse2 = stats_lse2(p, stats);
  a.dk = dk; a.dv = dv; a.dbias = dbias;
  a.sq_ = to_str(q_s); a.sk_ = to_str(k_s); a.sv_ = to_str(v_s); a.sb_ = to_str(bias_s);
  a.sdo_ = to_str(do_s); a.sdk_ = to_str(dk_s); a.sdv_ = to_str(dv_s); a.sdb_ = to_str(dbias_s);
  a.bias_vec = bias_vec_ok(p, attn_bias, bias_s) ? 1 : 0;
  hipError_t e = sdpa::launch_bwd_dkdv(io(p->dtype), (int)p->d_qk, (int)p->d_v, banded(p),
                                       a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "dK/dV launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd_dq(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s,
                          const void* k, sdpa_strides_t k_s, const void* v, sdpa_strides_t v_s,
                          const void* attn_bias, sdpa_strides_t bias_s, const void* d_o,
                          sdpa_strides_t do_s, const float* stats, void* dq,
                          sdpa_strides_t dq_s, void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (empty_problem(p)) return SDPA_OK;
  if ((st = check_bwd_inputs(p, q, q_s, k, k_s, v, v_s, attn_bias, bias_s, d_o, do_s, stats)) != SDPA_OK)
    return st;
  if ((st = check_tensor(p, dq, dq_s, "dq", p->dtype != SDPA_F32)) != SDPA_OK) return st;
  sdpa::BwdArgs a{};
  if (sdpa_status_t fs = fill_bwd_args(p, a); fs != SDPA_OK) return fs;
  a.q = q; a.k = k; a.v = v; a.bias = attn_bias; a.dout = d_o;
  a.dvec = (float*)stats; a.lse2 = stats_lse2(p, stats);
  a.dq = dq;
  a.sq_ = to_str(q_s); a.sk_ = to_str(k_s); a.sv_ = to_str(v_s); a.sb_ = to_str(bias_s);
  a.sdo_ = to_str(do_s); a.sdq_ = to_str(dq_s);
  a.bias_vec = bias_vec_ok(p, attn_bias, bias_s) ? 1 : 0;
  hipError_t e = sdpa::launch_bwd_dq(io(p->dtype), (int)p->d_qk, (int)p->d_v, banded(p), a,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "dQ launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

sdpa_status_t sdpa_bwd_dq_preprocess(const sdpa_problem_t* p, const void* q, sdpa_strides_t q_s,
                                     const void* k, sdpa_strides_t k_s, const void* v,
                                     sdpa_strides_t v_s, const void* attn_bias,
                                     sdpa_strides_t bias_s, const void* o, sdpa_strides_t o_s,
                                     const void* d_o, sdpa_strides_t do_s,
                                     const float* softmax_lse, float* stats, void* dq,
                                     sdpa_strides_t dq_s, void* stream) {
  g_msg[0] = 0;
  sdpa_status_t st = check_problem(p);
  if (st != SDPA_OK) return st;
  if (empty_problem(p)) return SDPA_OK;
  if (p->dtype == SDPA_F32)
    return fail(SDPA_ERR_UNSUPPORTED, "the fused dQ + preprocess kernel is for 16-bit io; use "
                "sdpa_bwd_preprocess then sdpa_bwd_dq");
  if ((st = check_bwd_inputs(p, q, q_s, k, k_s, v, v_s, attn_bias, bias_s, d_o, do_s, stats)) != SDPA_OK)
    return st;
  if ((st = check_tensor(p, o, o_s, "o", true)) != SDPA_OK) return st;
  if ((st = check_tensor(p, dq, dq_s, "dq", true)) != SDPA_OK) return st;
  if (!softmax_lse) return fail(SDPA_ERR_INVALID_ARG, "softmax_lse is null");
  sdpa::BwdArgs a{};
  if (sdpa_status_t fs = fill_bwd_args(p, a); fs != SDPA_OK) return fs;
  a.q = q; a.k = k; a.v = v; a.bias = attn_bias; a.o = o; a.dout = d_o;
  a.lse = softmax_lse;
  a.dvec = stats; a.lse2 = stats_lse2(p, stats);
  a.dq = dq;
  a.sq_ = to_str(q_s); a.sk_ = to_str(k_s); a.sv_ = to_str(v_s); a.sb_ = to_str(bias_s);
  a.so_ = to_str(o_s); a.sdo_ = to_str(do_s); a.sdq_ = to_str(dq_s);
  a.bias_vec = bias_vec_ok(p, attn_bias, bias_s) ? 1 : 0;
  hipError_t e = sdpa::launch_bwd_dq(io(p->dtype), (int)p->d_qk, (int)p->d_v, banded(p), a,
                                     (hipStream_t)stream, true);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "dQ launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

}  // extern "C"
