// C ABI of the MACaQ online W4A4 linear layer (declared in include/macaq.h).
//
// Host side only: argument checks (pure host code, done before any HIP call),
// the device check, workspace carving and kernel dispatch. No call allocates,
// synchronizes or keeps state beyond a per-device architecture cache.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.hpp"
#include "macaq.h"

using namespace macaq;

namespace {

thread_local char g_last_error[512] = "";

macaq_status fail(macaq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
macaq_status fail(macaq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

macaq_status hip_fail(hipError_t e, const char* what) {
  return fail(MACAQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_block(int32_t b) { return b == 0 || b == 32 || b == 64 || b == 128; }

// c_b = RN32(1/sqrt(b)) (1 without a Hadamard): 1/b is exact in fp32 for a
// power of two and sqrtf rounds once.
float multiplier_cb(int32_t b) { return b > 0 ? std::sqrt(1.0f / (float)b) : 1.0f; }

// gfx950 check of the current device, cached per device id.
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::mutex g_arch_mu;
// Architecture name that replaces the device query when set (a test hook).
char g_arch_override[64];
bool g_arch_overridden = false;

macaq_status check_device() {
  {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_overridden) {
      if (std::strncmp(g_arch_override, "gfx950", 6) == 0) return MACAQ_OK;
      return fail(MACAQ_EUNSUPPORTED, "device is %s, not gfx950", g_arch_override);
    }
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MACAQ_EUNSUPPORTED, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MACAQ_EUNSUPPORTED, "device id %d out of range", dev);
  {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_ok[dev] == 1) return MACAQ_OK;
    if (g_arch_ok[dev] == -1) return fail(MACAQ_EUNSUPPORTED, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    g_arch_ok[dev] = ok ? 1 : -1;
  }
  if (!ok) return fail(MACAQ_EUNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return MACAQ_OK;
}

constexpr size_t kWsAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of the layer calls: the quantized activations in the GEMM layout,
// then call-specific extra space (split-K partial sums or the MoE tile map).
struct LinearWs {
  size_t codes_off, scales_off, extra_off, total;
};

LinearWs linear_ws(int64_t M, int64_t K, size_t extra_bytes) {
  LinearWs w;
  w.codes_off = 0;
  w.scales_off = round_up((size_t)tiled_codes_bytes(M, K), kWsAlign);
  w.extra_off = w.scales_off + round_up((size_t)tiled_scales_bytes(M, K), kWsAlign);
  w.total = w.extra_off + round_up(extra_bytes, kWsAlign);
  return w;
}

// The grouped layer's extra workspace: the tile map, then the expert of each
// row.
size_t grouped_map_bytes(int64_t max_mtiles) {
  return round_up(((size_t)max_mtiles * 2 + 1) * sizeof(int32_t), kWsAlign);
}
size_t grouped_extra_bytes(int64_t T, int64_t max_mtiles) {
  return grouped_map_bytes(max_mtiles) + (size_t)T * sizeof(int32_t);
}

// Scratch of macaq_linear_noalloc: the quantized activations and split-K
// partial sums of one call, in device memory the library owns (one copy per
// GPU, held until the process ends). Host code never uses the array's name
// as an address: each device's address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
uint8_t* g_scratch_at[kMaxDevices];  // per device, set on its first no-allocation call
std::mutex g_scratch_mu;

macaq_status scratch_address(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MACAQ_EUNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MACAQ_EHIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_at[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_at[dev];
  return MACAQ_OK;
}

// Flip-Refinement keeps a row's state in the registers of one workgroup (at most 1024 threads).
constexpr int64_t kMaxRefineK = 32768;

// The GEMM addresses each packed operand through a 32-bit buffer range.
constexpr int64_t kMaxOperandBytes = (int64_t(1) << 31) - (int64_t(1) << 20);
bool operand_fits(int64_t rows, int64_t K) { return tiled_codes_bytes(rows, K) <= kMaxOperandBytes; }

macaq_status check_quant_shape(int64_t M, int64_t K, int64_t ld, int32_t b, const char* who) {
  if (M < 0) return fail(MACAQ_EINVAL, "%s: M = %lld < 0", who, (long long)M);
  if (K < 32 || K % 32 != 0) return fail(MACAQ_EINVAL, "%s: K = %lld is not a positive multiple of 32", who, (long long)K);
  if (!valid_block(b)) return fail(MACAQ_EINVAL, "%s: Hadamard block %d not in {0, 32, 64, 128}", who, b);
  if (b > 0 && K % b != 0) return fail(MACAQ_EINVAL, "%s: K = %lld is not a multiple of b = %d", who, (long long)K, b);
  if (ld < K) return fail(MACAQ_EINVAL, "%s: leading dimension %lld < K = %lld", who, (long long)ld, (long long)K);
  return MACAQ_OK;
}

macaq_status check_out(const void* Y, macaq_dtype dt, int64_t N, int64_t ldy, const char* who) {
  if (!Y) return fail(MACAQ_EINVAL, "%s: Y is NULL", who);
  if (dt != MACAQ_BF16 && dt != MACAQ_F32) return fail(MACAQ_EINVAL, "%s: bad output dtype %d", who, (int)dt);
  if (ldy < N) return fail(MACAQ_EINVAL, "%s: ldy = %lld < N = %lld", who, (long long)ldy, (long long)N);
  if (!aligned(Y, dt == MACAQ_F32 ? 4 : 2)) return fail(MACAQ_EALIGN, "%s: Y not aligned to its element size", who);
  return MACAQ_OK;
}

// Workspace of the MoE calls, R = T*k rows: routing arrays (with the
// expert of each row) and the routing counts, the tile map of the grouped GEMMs, the gathered gate/up input, the
// down input and the bf16 expert rows.
struct MoeWs {
  size_t offsets, row_token, row_expert, pos, counts, map, map2, agu_codes, agu_scales, dn_codes, dn_scales, rows,
      total;
  int64_t max_mtiles;
};

size_t route_counts_bytes(int64_t n, int32_t E) { return (size_t)moe_route_chunks(n) * (size_t)E * 4; }

MoeWs moe_ws(int64_t T, int32_t k, int32_t E, int64_t H, int64_t F) {
  const int64_t R = T * k;
  const GemmPlan pg = plan_gemm_grouped(R, E, 2 * F, H, true), pd = plan_gemm_grouped(R, E, H, F);
  const int64_t bm = pg.bm < pd.bm ? pg.bm : pd.bm;
  MoeWs w;
  w.max_mtiles = (R + bm - 1) / bm + E;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += round_up(bytes, kWsAlign);
    return here;
  };
  w.offsets = take((size_t)(E + 1) * 4);
  w.row_token = take((size_t)R * 4);
  w.row_expert = take((size_t)R * 4);
  w.pos = take((size_t)R * 4);
  w.counts = take(route_counts_bytes(R, E));
  w.map = take(((size_t)w.max_mtiles * 2 + 1) * 4);
  w.map2 = take(((size_t)w.max_mtiles * 2 + 1) * 4);  // the down GEMM's, when its tile rows differ
  w.agu_codes = take((size_t)tiled_codes_bytes(R, H));
  w.agu_scales = take((size_t)tiled_scales_bytes(R, H));
  w.dn_codes = take((size_t)tiled_codes_bytes(R, F));
  w.dn_scales = take((size_t)tiled_scales_bytes(R, F));
  w.rows = take((size_t)R * H * 2);
  w.total = at;
  return w;
}

macaq_status check_moe_shape(int64_t T, int32_t k, int32_t E, int64_t H, int64_t F, int32_t b, const char* who) {
  if (T < 0) return fail(MACAQ_EINVAL, "%s: T = %lld < 0", who, (long long)T);
  if (k < 1) return fail(MACAQ_EINVAL, "%s: k = %d < 1", who, k);
  if (E < 1 || E > kMaxExperts) return fail(MACAQ_EINVAL, "%s: E = %d not in [1, %d]", who, E, kMaxExperts);
  if (H < 32 || H % 32 != 0) return fail(MACAQ_EINVAL, "%s: H = %lld is not a positive multiple of 32", who, (long long)H);
  if (F < 32 || F % 32 != 0) return fail(MACAQ_EINVAL, "%s: F = %lld is not a positive multiple of 32", who, (long long)F);
  if (!valid_block(b)) return fail(MACAQ_EINVAL, "%s: Hadamard block %d not in {0, 32, 64, 128}", who, b);
  if (b > 0 && (H % b != 0 || F % b != 0)) return fail(MACAQ_EINVAL, "%s: H and F must be multiples of b = %d", who, b);
  const int64_t R = T * (int64_t)k;
  if (R > 0x7FFFFFFF) return fail(MACAQ_EINVAL, "%s: T*k = %lld rows exceed int32", who, (long long)R);
  if (!operand_fits(R, H) || !operand_fits(R, F) || !operand_fits(2 * F, H) || !operand_fits(H, F))
    return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  return MACAQ_OK;
}

hipError_t moe_gate_up_launch(const void* X, int64_t T, int64_t H, int64_t ldx, int32_t k, const int32_t* row_token,
                              const int32_t* offsets, int32_t E, const float* a_gu, int32_t b,
                              const uint8_t* wgu_codes, const uint8_t* wgu_scales, int64_t F, const float* a_dn,
                              uint8_t* dn_codes, uint8_t* dn_scales, uint8_t* ws, const MoeWs& w, int32_t* map,
                              bool routed_here, hipStream_t s) {
  const int64_t R = T * k;
  // the expert of each row: written by the routing when it ran in this call,
  // else from the offsets
  int32_t* row_expert = reinterpret_cast<int32_t*>(ws + w.row_expert);
  if (a_gu && !routed_here) {
    const hipError_t e = launch_row_expert(offsets, E, R, row_expert, s);
    if (e != hipSuccess) return e;
  }
  QuantArgs q{};
  q.x = X;
  q.M = R;
  q.K = H;
  q.ldx = ldx;
  q.mult = a_gu;
  q.row_expert = a_gu ? row_expert : nullptr;
  q.codes = ws + w.agu_codes;
  q.scales = ws + w.agu_scales;
  q.tiled = true;
  q.kpad = pad_k(H);
  q.gather = row_token;
  q.src_rows = T;
  hipError_t e = launch_quant_rows(q, b, false, s);
  if (e != hipSuccess) return e;
  GemmArgs g{};
  g.a_codes = q.codes;
  g.a_scales = q.scales;
  g.b_codes = wgu_codes;
  g.b_scales = wgu_scales;
  g.M = R;
  g.N = 2 * F;
  g.K = H;
  g.splits = 1;
  g.offsets = offsets;
  g.tile_map = map;
  g.E = E;
  g.max_mtiles = w.max_mtiles;
  g.map_ready = routed_here;
  g.swiglu = true;
  g.q_codes = dn_codes;
  g.q_scales = dn_scales;
  g.q_mult = a_dn;
  g.q_F = F;
  g.q_b = b;
  return launch_gemm_grouped(g, plan_gemm_grouped(R, E, 2 * F, H, true), s);
}

hipError_t moe_down_combine_launch(const uint8_t* dn_codes, const uint8_t* dn_scales, const int32_t* offsets,
                                   const int32_t* pos, const float* w_route, int64_t T, int32_t k, int32_t E,
                                   const uint8_t* wdn_codes, const uint8_t* wdn_scales, int64_t H, int64_t F,
                                   void* Y, macaq_dtype y_dtype, int64_t ldy, uint8_t* ws, const MoeWs& w,
                                   int32_t* map, bool build_map, hipStream_t s) {
  const int64_t R = T * k;
  uint16_t* rows = reinterpret_cast<uint16_t*>(ws + w.rows);
  GemmArgs g{};
  g.a_codes = dn_codes;
  g.a_scales = dn_scales;
  g.b_codes = wdn_codes;
  g.b_scales = wdn_scales;
  g.M = R;
  g.N = H;
  g.K = F;
  g.y = rows;
  g.ldy = H;
  g.y_bf16 = true;
  g.splits = 1;
  g.offsets = offsets;
  g.tile_map = map;
  g.E = E;
  g.max_mtiles = w.max_mtiles;
  g.map_ready = !build_map;
  hipError_t e = launch_gemm_grouped(g, plan_gemm_grouped(R, E, H, F), s);
  if (e != hipSuccess) return e;
  return launch_moe_combine(rows, H, pos, w_route, T, k, Y, y_dtype == MACAQ_BF16, ldy, s);
}

}  // namespace

extern "C" {

const char* macaq_status_string(macaq_status s) {
  switch (s) {
    case MACAQ_OK: return "ok";
    case MACAQ_EINVAL: return "invalid argument";
    case MACAQ_EALIGN: return "misaligned pointer or leading dimension";
    case MACAQ_EWORKSPACE: return "workspace too small or misaligned";
    case MACAQ_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case MACAQ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* macaq_last_error(void) { return g_last_error; }

macaq_status macaq_calibrate_pow(const void* xcal, int64_t R, int64_t K, int64_t ldx, int32_t quarters, float* s,
                                 macaq_stream_t stream) {
  if (quarters != 0 && quarters != 1 && quarters != 2 && quarters != 4)
    return fail(MACAQ_EINVAL, "macaq_calibrate: quarters = %d not in {0, 1, 2, 4}", quarters);
  if (!xcal || !s) return fail(MACAQ_EINVAL, "macaq_calibrate: NULL pointer");
  if (R < 1 || K < 1 || ldx < K) return fail(MACAQ_EINVAL, "macaq_calibrate: need R >= 1, K >= 1, ldx >= K");
  if (!aligned(xcal, 2) || !aligned(s, 4)) return fail(MACAQ_EALIGN, "macaq_calibrate: misaligned pointer");
  macaq_status st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = launch_calibrate(xcal, R, K, ldx, quarters, s, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_calibrate launch");
}

macaq_status macaq_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, float* s, macaq_stream_t stream) {
  return macaq_calibrate_pow(xcal, R, K, ldx, 2, s, stream);
}

void macaq_debug_override_arch(const char* arch) {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  g_arch_overridden = arch != nullptr;
  if (arch) {
    std::strncpy(g_arch_override, arch, sizeof g_arch_override - 1);
    g_arch_override[sizeof g_arch_override - 1] = 0;
  }
}

void macaq_debug_limit_workgroups(int32_t n) { macaq::set_workgroup_cap(n); }

macaq_status macaq_debug_mfma_probe(const void* operands, int32_t workgroups, int32_t iters, float* out,
                                    macaq_stream_t stream) {
  const char* who = "macaq_debug_mfma_probe";
  if (!operands || !out) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (workgroups < 1 || workgroups > 65536 || iters < 1)
    return fail(MACAQ_EINVAL, "%s: workgroups = %d not in [1, 65536] or iters = %d < 1", who, workgroups, iters);
  if (!aligned(operands, 16) || !aligned(out, 4)) return fail(MACAQ_EALIGN, "%s: operands 16-byte aligned", who);
  macaq_status st = check_device();
  if (st != MACAQ_OK) return st;
  const hipError_t e =
      launch_mfma_probe(operands, workgroups, iters, out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_debug_mfma_probe launch");
}

macaq_status macaq_debug_read_probe(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                                    macaq_stream_t stream) {
  const char* who = "macaq_debug_read_probe";
  if (!src || !out) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (bytes < 16 || workgroups < 1 || workgroups > 65536)
    return fail(MACAQ_EINVAL, "%s: bytes = %lld < 16 or workgroups = %d not in [1, 65536]", who, (long long)bytes,
                workgroups);
  if (!aligned(src, 16) || bytes % 16 != 0 || !aligned(out, 4))
    return fail(MACAQ_EALIGN, "%s: src 16-byte aligned and bytes a multiple of 16", who);
  macaq_status st = check_device();
  if (st != MACAQ_OK) return st;
  const hipError_t e = launch_read_probe(src, bytes, workgroups, out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_debug_read_probe launch");
}

macaq_status macaq_make_multipliers(const float* s, int64_t K, int32_t b, float* a, float* r) {
  const char* who = "macaq_make_multipliers";
  if (!s || (!a && !r)) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (K < 1) return fail(MACAQ_EINVAL, "%s: K < 1", who);
  if (!valid_block(b)) return fail(MACAQ_EINVAL, "%s: block %d not in {0, 32, 64, 128}", who, b);
  if (!aligned(s, 4) || (a && !aligned(a, 4)) || (r && !aligned(r, 4)))
    return fail(MACAQ_EALIGN, "%s: misaligned pointer", who);
  for (int64_t k = 0; k < K; ++k)
    if (!(s[k] > 0.0f) || !std::isfinite(s[k]))
      return fail(MACAQ_EINVAL, "%s: s[%lld] = %g is not positive and finite", who, (long long)k, (double)s[k]);
  const float cb = multiplier_cb(b);
  // IEEE single precision: each quotient and product is rounded once
  // (this file is compiled without contraction)
  for (int64_t k = 0; k < K; ++k) {
    if (a) a[k] = cb / s[k];
    if (r) r[k] = cb * s[k];
  }
  return MACAQ_OK;
}

macaq_status macaq_make_multipliers_device(const float* s, int64_t K, int32_t b, float* a, float* r,
                                           macaq_stream_t stream) {
  const char* who = "macaq_make_multipliers_device";
  if (!s || (!a && !r)) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (K < 1) return fail(MACAQ_EINVAL, "%s: K < 1", who);
  if (!valid_block(b)) return fail(MACAQ_EINVAL, "%s: block %d not in {0, 32, 64, 128}", who, b);
  if (!aligned(s, 4) || (a && !aligned(a, 4)) || (r && !aligned(r, 4)))
    return fail(MACAQ_EALIGN, "%s: misaligned pointer", who);
  macaq_status st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = launch_multipliers(s, K, multiplier_cb(b), a, r, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_make_multipliers_device launch");
}

macaq_status macaq_prepare_weights(const void* W, macaq_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                                   const float* r, int32_t b, macaq_layout layout, uint8_t* w_codes,
                                   uint8_t* w_scales, macaq_stream_t stream) {
  const char* who = "macaq_prepare_weights";
  if (w_dtype != MACAQ_BF16 && w_dtype != MACAQ_F32) return fail(MACAQ_EINVAL, "%s: bad weight dtype", who);
  macaq_status st = check_quant_shape(N, K, ldw, b, who);
  if (st != MACAQ_OK) return st;
  if (layout != MACAQ_ROW_MAJOR && layout != MACAQ_GEMM_LAYOUT) return fail(MACAQ_EINVAL, "%s: bad layout", who);
  if (N == 0) return MACAQ_OK;
  if (!W || !w_codes || !w_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (layout == MACAQ_GEMM_LAYOUT && !operand_fits(N, K))
    return fail(MACAQ_EINVAL, "%s: packed weights over 2 GiB", who);
  const size_t esz = w_dtype == MACAQ_F32 ? 4 : 2;
  if (!aligned(W, 16) || (ldw * (int64_t)esz) % 16 != 0 || !aligned(w_codes, 16) || !aligned(w_scales, 16) ||
      (r && !aligned(r, 16)))
    return fail(MACAQ_EALIGN, "%s: W, r, w_codes, w_scales must be 16-byte aligned and rows of W 16-byte multiples", who);
  if (N == 0) return MACAQ_OK;
  st = check_device();
  if (st != MACAQ_OK) return st;
  QuantArgs q{};
  q.x = W;
  q.M = N;
  q.K = K;
  q.ldx = ldw;
  q.mult = r;
  q.codes = w_codes;
  q.scales = w_scales;
  q.tiled = layout == MACAQ_GEMM_LAYOUT;
  q.kpad = pad_k(K);
  hipError_t e = launch_quant_rows(q, b, w_dtype == MACAQ_F32, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_prepare_weights launch");
}

size_t macaq_packed_codes_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0) return 0;
  return (size_t)tiled_codes_bytes(rows, K);
}

size_t macaq_packed_scales_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0) return 0;
  return (size_t)tiled_scales_bytes(rows, K);
}

macaq_status macaq_quant_act(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                             macaq_layout layout, uint8_t* a_codes, uint8_t* a_scales, macaq_stream_t stream) {
  const char* who = "macaq_quant_act";
  macaq_status st = check_quant_shape(M, K, ldx, b, who);
  if (st != MACAQ_OK) return st;
  if (layout != MACAQ_ROW_MAJOR && layout != MACAQ_GEMM_LAYOUT) return fail(MACAQ_EINVAL, "%s: bad layout", who);
  if (layout == MACAQ_GEMM_LAYOUT && !operand_fits(M, K))
    return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  if (M == 0) return MACAQ_OK;
  if (!X || !a_codes || !a_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(a_codes, 16) || !aligned(a_scales, 16) || (a && !aligned(a, 16)))
    return fail(MACAQ_EALIGN, "%s: X, a, a_codes, a_scales must be 16-byte aligned and ldx a multiple of 8", who);
  if (M == 0) return MACAQ_OK;
  st = check_device();
  if (st != MACAQ_OK) return st;
  QuantArgs q{};
  q.x = X;
  q.M = M;
  q.K = K;
  q.ldx = ldx;
  q.mult = a;
  q.codes = a_codes;
  q.scales = a_scales;
  q.tiled = layout == MACAQ_GEMM_LAYOUT;
  q.kpad = pad_k(K);
  hipError_t e = launch_quant_rows(q, b, false, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_quant_act launch");
}

size_t macaq_gemm_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return round_up(plan_gemm(M, N, K).partial_bytes, kWsAlign);
}

size_t macaq_linear_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return linear_ws(M, K, plan_gemm(M, N, K).partial_bytes).total;
}

static macaq_status gemm_common(const uint8_t* ac, const uint8_t* as, int64_t M, int64_t K, const uint8_t* wc,
                                const uint8_t* ws, int64_t N, void* Y, macaq_dtype y_dtype, int64_t ldy,
                                float* partial, hipStream_t stream, const char* who) {
  GemmPlan p = plan_gemm(M, N, K);
  GemmArgs g{};
  g.a_codes = ac;
  g.a_scales = as;
  g.b_codes = wc;
  g.b_scales = ws;
  g.M = M;
  g.N = N;
  g.K = K;
  g.y = Y;
  g.ldy = ldy;
  g.y_bf16 = y_dtype == MACAQ_BF16;
  g.partial = partial;
  g.splits = p.splits;
  hipError_t e = launch_gemm(g, p, stream);
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, who);
}

macaq_status macaq_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, int64_t K, const uint8_t* w_codes,
                        const uint8_t* w_scales, int64_t N, void* Y, macaq_dtype y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_gemm";
  if (M < 0 || N < 1) return fail(MACAQ_EINVAL, "%s: need M >= 0, N >= 1", who);
  if (K < 32 || K % 32 != 0) return fail(MACAQ_EINVAL, "%s: K is not a positive multiple of 32", who);
  if (M == 0) return MACAQ_OK;
  if (!a_codes || !a_scales || !w_codes || !w_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!operand_fits(M, K) || !operand_fits(N, K)) return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  macaq_status st = check_out(Y, y_dtype, N, ldy, who);
  if (st != MACAQ_OK) return st;
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 16) || !aligned(w_scales, 16))
    return fail(MACAQ_EALIGN, "%s: code and scale arrays must be 16-byte aligned", who);
  if (M == 0) return MACAQ_OK;
  const size_t need = macaq_gemm_workspace_size(M, K, N);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign)))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, need);
  st = check_device();
  if (st != MACAQ_OK) return st;
  return gemm_common(a_codes, a_scales, M, K, w_codes, w_scales, N, Y, y_dtype, ldy, static_cast<float*>(workspace),
                     reinterpret_cast<hipStream_t>(stream), who);
}

// Argument checks of macaq_linear and its no-allocation variant (workspace
// aside); MACAQ_OK with *empty set when there is nothing to do.
static macaq_status linear_check(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, const void* Y,
                                 macaq_dtype y_dtype, int64_t ldy, const char* who, bool* empty) {
  *empty = false;
  macaq_status st = check_quant_shape(M, K, ldx, b, who);
  if (st != MACAQ_OK) return st;
  if (N < 1) return fail(MACAQ_EINVAL, "%s: N < 1", who);
  if (M == 0) {
    *empty = true;
    return MACAQ_OK;
  }
  if (!X || !w_codes || !w_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!operand_fits(M, K) || !operand_fits(N, K)) return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  st = check_out(Y, y_dtype, N, ldy, who);
  if (st != MACAQ_OK) return st;
  if (!aligned(X, 16) || ldx % 8 != 0 || (a && !aligned(a, 16)) || !aligned(w_codes, 16) || !aligned(w_scales, 16))
    return fail(MACAQ_EALIGN, "%s: X, a, w_codes, w_scales must be 16-byte aligned and ldx a multiple of 8", who);
  return MACAQ_OK;
}

// Quantize, then the GEMM, with the layout of linear_ws in `ws`.
static macaq_status linear_enqueue(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                                   const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y,
                                   macaq_dtype y_dtype, int64_t ldy, uint8_t* ws, const LinearWs& w, hipStream_t s,
                                   const char* who) {
  QuantArgs q{};
  q.x = X;
  q.M = M;
  q.K = K;
  q.ldx = ldx;
  q.mult = a;
  q.codes = ws + w.codes_off;
  q.scales = ws + w.scales_off;
  q.tiled = true;
  q.kpad = pad_k(K);
  hipError_t e = launch_quant_rows(q, b, false, s);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return gemm_common(q.codes, q.scales, M, K, w_codes, w_scales, N, Y, y_dtype, ldy,
                     reinterpret_cast<float*>(ws + w.extra_off), s, who);
}

macaq_status macaq_linear(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                          const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y, macaq_dtype y_dtype,
                          int64_t ldy, void* workspace, size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_linear";
  bool empty;
  macaq_status st = linear_check(X, M, K, ldx, a, b, w_codes, w_scales, N, Y, y_dtype, ldy, who, &empty);
  if (st != MACAQ_OK || empty) return st;
  const LinearWs w = linear_ws(M, K, plan_gemm(M, N, K).partial_bytes);
  if (!workspace || workspace_bytes < w.total || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, w.total);
  st = check_device();
  if (st != MACAQ_OK) return st;
  return linear_enqueue(X, M, K, ldx, a, b, w_codes, w_scales, N, Y, y_dtype, ldy, static_cast<uint8_t*>(workspace),
                        w, reinterpret_cast<hipStream_t>(stream), who);
}

macaq_status macaq_linear_noalloc(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y,
                                  macaq_dtype y_dtype, int64_t ldy, macaq_stream_t stream) {
  const char* who = "macaq_linear_noalloc";
  bool empty;
  macaq_status st = linear_check(X, M, K, ldx, a, b, w_codes, w_scales, N, Y, y_dtype, ldy, who, &empty);
  if (st != MACAQ_OK || empty) return st;
  const LinearWs w = linear_ws(M, K, plan_gemm(M, N, K).partial_bytes);
  if (w.total > kScratchBytes)
    return fail(MACAQ_EWORKSPACE,
                "%s: M = %lld, K = %lld, N = %lld need %zu bytes of scratch; the library's fixed scratch holds %zu "
                "(use macaq_linear with a workspace)",
                who, (long long)M, (long long)K, (long long)N, w.total, kScratchBytes);
  st = check_device();
  if (st != MACAQ_OK) return st;
  uint8_t* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MACAQ_OK) return st;
  return linear_enqueue(X, M, K, ldx, a, b, w_codes, w_scales, N, Y, y_dtype, ldy, ws, w,
                        reinterpret_cast<hipStream_t>(stream), who);
}

size_t macaq_linear_grouped_workspace_size(int64_t T, int32_t E, int64_t K, int64_t N) {
  if (T <= 0 || E < 1 || K <= 0 || N <= 0) return 0;
  const GemmPlan p = plan_gemm_grouped(T, E, N, K);
  const int64_t max_mtiles = (T + p.bm - 1) / p.bm + E;
  return linear_ws(T, K, grouped_extra_bytes(T, max_mtiles)).total;
}

macaq_status macaq_linear_grouped(const void* X, const int32_t* offsets, int32_t E, int64_t T, int64_t K,
                                  const float* a, int32_t b, const uint8_t* w_codes, const uint8_t* w_scales,
                                  int64_t N, void* Y, macaq_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                  macaq_stream_t stream) {
  const char* who = "macaq_linear_grouped";
  if (E < 1) return fail(MACAQ_EINVAL, "%s: E < 1", who);
  macaq_status st = check_quant_shape(T, K, K, b, who);
  if (st != MACAQ_OK) return st;
  if (N < 1) return fail(MACAQ_EINVAL, "%s: N < 1", who);
  if (T == 0) return MACAQ_OK;
  if (!X || !offsets || !w_codes || !w_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!operand_fits(T, K) || !operand_fits(N, K)) return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  st = check_out(Y, y_dtype, N, N, who);
  if (st != MACAQ_OK) return st;
  if (!aligned(X, 16) || (a && !aligned(a, 16)) || !aligned(w_codes, 16) || !aligned(w_scales, 16) ||
      !aligned(offsets, 4) || (K * (int64_t)sizeof(float)) % 16 != 0)
    return fail(MACAQ_EALIGN, "%s: X, a, w_codes, w_scales must be 16-byte aligned", who);
  if (T == 0) return MACAQ_OK;
  const size_t need = macaq_linear_grouped_workspace_size(T, E, K, N);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, need);
  st = check_device();
  if (st != MACAQ_OK) return st;
  const GemmPlan p = plan_gemm_grouped(T, E, N, K);
  const int64_t max_mtiles = (T + p.bm - 1) / p.bm + E;
  const LinearWs w = linear_ws(T, K, grouped_extra_bytes(T, max_mtiles));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* row_expert = reinterpret_cast<int32_t*>(ws + w.extra_off + grouped_map_bytes(max_mtiles));
  if (a) {
    const hipError_t e = launch_row_expert(offsets, E, T, row_expert, s);
    if (e != hipSuccess) return hip_fail(e, "macaq_linear_grouped row experts launch");
  }
  QuantArgs q{};
  q.x = X;
  q.M = T;
  q.K = K;
  q.ldx = K;
  q.mult = a;
  q.row_expert = a ? row_expert : nullptr;
  q.codes = ws + w.codes_off;
  q.scales = ws + w.scales_off;
  q.tiled = true;
  q.kpad = pad_k(K);
  hipError_t e = launch_quant_rows(q, b, false, s);
  if (e != hipSuccess) return hip_fail(e, "macaq_linear_grouped quantize launch");
  GemmArgs g{};
  g.a_codes = q.codes;
  g.a_scales = q.scales;
  g.b_codes = w_codes;
  g.b_scales = w_scales;
  g.M = T;
  g.N = N;
  g.K = K;
  g.y = Y;
  g.ldy = N;
  g.y_bf16 = y_dtype == MACAQ_BF16;
  g.splits = 1;
  g.offsets = offsets;
  g.tile_map = reinterpret_cast<int32_t*>(ws + w.extra_off);
  g.E = E;
  g.max_mtiles = max_mtiles;
  e = launch_gemm_grouped(g, p, s);
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_linear_grouped GEMM launch");
}

size_t macaq_moe_workspace_size(int64_t T, int32_t k, int32_t E, int64_t H, int64_t F) {
  if (T <= 0 || k < 1 || E < 1 || H < 32 || F < 32) return 0;
  return moe_ws(T, k, E, H, F).total;
}

size_t macaq_moe_route_workspace_size(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * (int64_t)k > 0x7FFFFFFF) return 0;
  return round_up(route_counts_bytes(T * k, E), kWsAlign);
}

macaq_status macaq_moe_route(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* offsets,
                             int32_t* row_token, int32_t* pos, void* workspace, size_t workspace_bytes,
                             macaq_stream_t stream) {
  const char* who = "macaq_moe_route";
  if (T < 0 || k < 1) return fail(MACAQ_EINVAL, "%s: T = %lld, k = %d", who, (long long)T, k);
  if (E < 1 || E > kMaxExperts) return fail(MACAQ_EINVAL, "%s: E = %d not in [1, %d]", who, E, kMaxExperts);
  if (T * (int64_t)k > 0x7FFFFFFF) return fail(MACAQ_EINVAL, "%s: T*k exceeds int32", who);
  // with no entries ids is never read (an empty tensor may have no storage)
  if ((!ids && T > 0) || !offsets || !row_token || !pos) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if ((ids && !aligned(ids, 16)) || !aligned(offsets, 4) || !aligned(row_token, 4) || !aligned(pos, 4))
    return fail(MACAQ_EALIGN, "%s: ids must be 16-byte aligned, the other int32 arrays 4-byte aligned", who);
  const size_t need = macaq_moe_route_workspace_size(T, k, E);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, need);
  macaq_status st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = launch_moe_route(ids, T, k, E, offsets, row_token, pos, static_cast<int32_t*>(workspace),
                                  RouteMaps{{nullptr, nullptr}, {0, 0}, 0}, nullptr,
                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_moe_route launch");
}

macaq_status macaq_moe_gate_up(const void* X, int64_t T, int64_t H, int64_t ldx, int32_t k, const int32_t* row_token,
                               const int32_t* offsets, int32_t E, const float* a_gu, int32_t b,
                               const uint8_t* wgu_codes, const uint8_t* wgu_scales, int64_t F, const float* a_dn,
                               uint8_t* dn_codes, uint8_t* dn_scales, void* workspace, size_t workspace_bytes,
                               macaq_stream_t stream) {
  const char* who = "macaq_moe_gate_up";
  macaq_status st = check_moe_shape(T, k, E, H, F, b, who);
  if (st != MACAQ_OK) return st;
  if (ldx < H) return fail(MACAQ_EINVAL, "%s: ldx = %lld < H", who, (long long)ldx);
  if (!X || !row_token || !offsets || !wgu_codes || !wgu_scales || !dn_codes || !dn_scales)
    return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if ((!a_gu || !a_dn) && b != 0) return fail(MACAQ_EINVAL, "%s: a_gu and a_dn are required when b > 0", who);
  if (!aligned(X, 16) || ldx % 8 != 0 || (a_gu && !aligned(a_gu, 16)) || (a_dn && !aligned(a_dn, 4)) ||
      !aligned(wgu_codes, 16) || !aligned(wgu_scales, 16) || !aligned(dn_codes, 16) || !aligned(dn_scales, 4) ||
      !aligned(row_token, 4) || !aligned(offsets, 4))
    return fail(MACAQ_EALIGN, "%s: X, a_gu, weights and dn_codes 16-byte aligned, ldx a multiple of 8", who);
  if (T == 0) return MACAQ_OK;
  const MoeWs w = moe_ws(T, k, E, H, F);
  if (!workspace || workspace_bytes < w.total || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, w.total);
  st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = moe_gate_up_launch(X, T, H, ldx, k, row_token, offsets, E, a_gu, b, wgu_codes, wgu_scales, F, a_dn,
                                    dn_codes, dn_scales, static_cast<uint8_t*>(workspace), w,
                                    reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + w.map), false,
                                    reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_moe_gate_up launch");
}

macaq_status macaq_moe_down_combine(const uint8_t* dn_codes, const uint8_t* dn_scales, const int32_t* offsets,
                                    const int32_t* pos, const float* w_route, int64_t T, int32_t k, int32_t E,
                                    const uint8_t* wdn_codes, const uint8_t* wdn_scales, int64_t H, int64_t F,
                                    void* Y, macaq_dtype y_dtype, int64_t ldy, void* workspace,
                                    size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_moe_down_combine";
  macaq_status st = check_moe_shape(T, k, E, H, F, 0, who);
  if (st != MACAQ_OK) return st;
  if (!dn_codes || !dn_scales || !offsets || !pos || !w_route || !wdn_codes || !wdn_scales)
    return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  st = check_out(Y, y_dtype, H, ldy, who);
  if (st != MACAQ_OK) return st;
  if (!aligned(dn_codes, 16) || !aligned(dn_scales, 16) || !aligned(wdn_codes, 16) || !aligned(wdn_scales, 16) ||
      !aligned(offsets, 4) || !aligned(pos, 4) || !aligned(w_route, 4))
    return fail(MACAQ_EALIGN, "%s: packed operands 16-byte aligned, int32/fp32 arrays 4-byte aligned", who);
  if (T == 0) return MACAQ_OK;
  const MoeWs w = moe_ws(T, k, E, H, F);
  if (!workspace || workspace_bytes < w.total || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, w.total);
  st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = moe_down_combine_launch(dn_codes, dn_scales, offsets, pos, w_route, T, k, E, wdn_codes, wdn_scales,
                                         H, F, Y, y_dtype, ldy, static_cast<uint8_t*>(workspace), w,
                                         reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + w.map), true,
                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_moe_down_combine launch");
}

macaq_status macaq_moe_block(const void* X, int64_t T, int64_t H, int64_t ldx, const int32_t* ids, const float* w_route,
                             int32_t k, int32_t E, const float* a_gu, const uint8_t* wgu_codes,
                             const uint8_t* wgu_scales, const float* a_dn, const uint8_t* wdn_codes,
                             const uint8_t* wdn_scales, int64_t F, int32_t b, void* Y, macaq_dtype y_dtype,
                             int64_t ldy, void* workspace, size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_moe_block";
  macaq_status st = check_moe_shape(T, k, E, H, F, b, who);
  if (st != MACAQ_OK) return st;
  if (ldx < H) return fail(MACAQ_EINVAL, "%s: ldx = %lld < H", who, (long long)ldx);
  if (!X || !ids || !w_route || !wgu_codes || !wgu_scales || !wdn_codes || !wdn_scales)
    return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if ((!a_gu || !a_dn) && b != 0) return fail(MACAQ_EINVAL, "%s: a_gu and a_dn are required when b > 0", who);
  st = check_out(Y, y_dtype, H, ldy, who);
  if (st != MACAQ_OK) return st;
  if (!aligned(X, 16) || ldx % 8 != 0 || (a_gu && !aligned(a_gu, 16)) || (a_dn && !aligned(a_dn, 4)) ||
      !aligned(wgu_codes, 16) || !aligned(wgu_scales, 16) || !aligned(wdn_codes, 16) || !aligned(wdn_scales, 16) ||
      !aligned(ids, 16) || !aligned(w_route, 4))
    return fail(MACAQ_EALIGN, "%s: X, a_gu, weights and ids 16-byte aligned, ldx a multiple of 8", who);
  if (T == 0) return MACAQ_OK;
  const MoeWs w = moe_ws(T, k, E, H, F);
  if (!workspace || workspace_bytes < w.total || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, w.total);
  st = check_device();
  if (st != MACAQ_OK) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + w.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + w.row_token);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + w.pos);
  // the routing also writes the tile maps of both grouped GEMMs (one map when
  // their tiles have the same rows)
  const int bm_gu = plan_gemm_grouped(T * k, E, 2 * F, H, true).bm, bm_dn = plan_gemm_grouped(T * k, E, H, F).bm;
  int32_t* map_gu = reinterpret_cast<int32_t*>(ws + w.map);
  int32_t* map_dn = bm_dn == bm_gu ? map_gu : reinterpret_cast<int32_t*>(ws + w.map2);
  const RouteMaps maps{{map_gu, bm_dn == bm_gu ? nullptr : map_dn}, {bm_gu, bm_dn}, w.max_mtiles};
  hipError_t e =
      launch_moe_route(ids, T, k, E, offsets, row_token, pos, reinterpret_cast<int32_t*>(ws + w.counts), maps,
                       reinterpret_cast<int32_t*>(ws + w.row_expert), s);
  if (e != hipSuccess) return hip_fail(e, "macaq_moe_block routing launch");
  e = moe_gate_up_launch(X, T, H, ldx, k, row_token, offsets, E, a_gu, b, wgu_codes, wgu_scales, F, a_dn,
                         ws + w.dn_codes, ws + w.dn_scales, ws, w, map_gu, true, s);
  if (e != hipSuccess) return hip_fail(e, "macaq_moe_block gate/up launch");
  e = moe_down_combine_launch(ws + w.dn_codes, ws + w.dn_scales, offsets, pos, w_route, T, k, E, wdn_codes,
                              wdn_scales, H, F, Y, y_dtype, ldy, ws, w, map_dn, false, s);
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_moe_block down/combine launch");
}

size_t macaq_hessian_workspace_size(int64_t R, int64_t K) {
  if (R <= 0 || K <= 0) return 0;
  return round_up((size_t)R * (size_t)K * sizeof(float), kWsAlign);
}

macaq_status macaq_hessian(const void* Xcal, int64_t R, int64_t K, int64_t ldx, const float* a, int32_t b, double* H,
                           void* workspace, size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_hessian";
  if (R < 1) return fail(MACAQ_EINVAL, "%s: R = %lld < 1", who, (long long)R);
  macaq_status st = check_quant_shape(R, K, ldx, b, who);
  if (st != MACAQ_OK) return st;
  if (K > kMaxRefineK) return fail(MACAQ_EINVAL, "%s: K = %lld > %lld", who, (long long)K, (long long)kMaxRefineK);
  if (!Xcal || !H) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!a && b != 0) return fail(MACAQ_EINVAL, "%s: a is required when b > 0", who);
  if (!aligned(Xcal, 16) || ldx % 8 != 0 || (a && !aligned(a, 16)) || !aligned(H, 16))
    return fail(MACAQ_EALIGN, "%s: Xcal, a and H must be 16-byte aligned and ldx a multiple of 8", who);
  const size_t need = macaq_hessian_workspace_size(R, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, need);
  st = check_device();
  if (st != MACAQ_OK) return st;
  hipError_t e = launch_hessian(Xcal, R, K, ldx, a, b, static_cast<float*>(workspace), H,
                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_hessian launch");
}

size_t macaq_flip_refine_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return 2 * round_up((size_t)N * (size_t)K * sizeof(double), kWsAlign) + round_up((size_t)K * sizeof(double), kWsAlign);
}

macaq_status macaq_flip_refine(const void* W, macaq_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, const float* r,
                               int32_t b, const double* H, int32_t max_flips, uint8_t* w_codes, const uint8_t* w_scales,
                               int32_t* flips, void* workspace, size_t workspace_bytes, macaq_stream_t stream) {
  const char* who = "macaq_flip_refine";
  if (N < 1) return fail(MACAQ_EINVAL, "%s: N = %lld < 1", who, (long long)N);
  macaq_status st = check_quant_shape(N, K, ldw, b, who);
  if (st != MACAQ_OK) return st;
  if (K > kMaxRefineK) return fail(MACAQ_EINVAL, "%s: K = %lld > %lld", who, (long long)K, (long long)kMaxRefineK);
  if (w_dtype != MACAQ_BF16 && w_dtype != MACAQ_F32) return fail(MACAQ_EINVAL, "%s: bad weight dtype", who);
  if (max_flips < 0) return fail(MACAQ_EINVAL, "%s: max_flips < 0", who);
  if (!W || !H || !w_codes || !w_scales) return fail(MACAQ_EINVAL, "%s: NULL pointer", who);
  if (!r && b != 0) return fail(MACAQ_EINVAL, "%s: r is required when b > 0", who);
  if (!operand_fits(N, K)) return fail(MACAQ_EINVAL, "%s: packed operand over 2 GiB", who);
  const int64_t vec = w_dtype == MACAQ_F32 ? 4 : 8;
  if (!aligned(W, 16) || ldw % vec != 0 || (r && !aligned(r, 16)) || !aligned(H, 16) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 16) || (flips && !aligned(flips, 4)))
    return fail(MACAQ_EALIGN, "%s: W, r, H and the packed weights 16-byte aligned, ldw a multiple of %lld", who,
                (long long)vec);
  const size_t need = macaq_flip_refine_workspace_size(N, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return fail(MACAQ_EWORKSPACE, "%s: need %zu workspace bytes, 256-byte aligned", who, need);
  st = check_device();
  if (st != MACAQ_OK) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t mat = round_up((size_t)N * (size_t)K * sizeof(double), kWsAlign);
  hipError_t e = launch_flip_refine(W, w_dtype == MACAQ_F32, N, K, ldw, r, b, H, max_flips, w_codes, w_scales, flips,
                                    reinterpret_cast<double*>(ws), reinterpret_cast<double*>(ws + mat),
                                    reinterpret_cast<double*>(ws + 2 * mat), reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MACAQ_OK : hip_fail(e, "macaq_flip_refine launch");
}

}  // extern "C"
