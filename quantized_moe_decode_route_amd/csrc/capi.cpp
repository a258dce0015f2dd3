// C ABI of libmoedecode: argument validation, workspace layout and launch
// sequencing.  No entry point allocates device memory; the few that
// synchronise their stream once per device say so in the header.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

// Workspace of moe_layer_decode_noalloc: a file-scope device array, one copy
// per GPU.  Host code never passes its name to a kernel (on the host the name
// is a stand-in, not a device address); it uses the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = (int)e;
  return MOE_ERR_HIP;
}

int arch_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hip_status(hipErrorNoDevice);
  // Cache per device: the answer cannot change for a device ordinal.
  static int cached[64] = {0};  // 0 unknown, 1 ok, 2 wrong arch
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev] == 1 ? MOE_OK : MOE_ERR_ARCH;
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_status(e);
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cached[dev] = ok ? 1 : 2;
  return ok ? MOE_OK : MOE_ERR_ARCH;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int block_len(int fmt) { return fmt == MOE_FMT_Q2K ? 256 : 32; }

int check_gemv(const void* w, int N, int K, const float* x, int B, float* y, int fmt) {
  if (!w || !x || !y) return MOE_ERR_ARG;
  if (N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (B < 1 || B > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
  if (K % block_len(fmt) != 0) return MOE_ERR_SHAPE;
  if (!aligned(x, 16)) return MOE_ERR_ALIGN;
  if (fmt == MOE_FMT_INT4G32 ? !aligned(w, 16) : !aligned(w, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Format of the down projection (enum moe_format), or -1 if invalid.
int down_fmt(const moe_layer_desc* L) {
  if (L->down_format == MOE_DOWN_SAME) return L->format;
  if (L->down_format < MOE_DOWN_MXFP4 || L->down_format > MOE_DOWN_INT4G32) return -1;
  return L->down_format - 1;
}

int check_layer(const moe_layer_desc* L, int B) {
  if (!L) return MOE_ERR_ARG;
  const int fg = L->format, fd = down_fmt(L);
  if (fg < MOE_FMT_MXFP4 || fg > MOE_FMT_INT4G32 || fd < 0) return MOE_ERR_ARG;
  if (!L->router_w || !L->gate || !L->up || !L->down) return MOE_ERR_ARG;
  if (L->n_experts < 1 || L->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (L->top_k < 1 || L->top_k > MOE_MAX_TOPK || L->top_k > L->n_experts) return MOE_ERR_SHAPE;
  if (B < 1 || B > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
  const int bl = block_len(fg) > block_len(fd) ? block_len(fg) : block_len(fd);
  if (L->d_model <= 0 || L->d_ff <= 0 || L->d_model % bl || L->d_ff % bl) return MOE_ERR_SHAPE;
  if (L->gate_stride < 0 || L->up_stride < 0 || L->down_stride < 0) return MOE_ERR_ARG;
  if (!aligned(L->router_w, 16)) return MOE_ERR_ALIGN;
  const uintptr_t wg = fg == MOE_FMT_INT4G32 ? 16 : 4, wd = fd == MOE_FMT_INT4G32 ? 16 : 4;
  if (!aligned(L->gate, wg) || !aligned(L->up, wg) || !aligned(L->down, wd)) return MOE_ERR_ALIGN;
  if (L->gate_stride % wg || L->up_stride % wg || L->down_stride % wd) return MOE_ERR_ALIGN;
  if (L->down_layout != MOE_LAYOUT_ROWS && L->down_layout != MOE_LAYOUT_TILE256 &&
      L->down_layout != MOE_LAYOUT_MFMA16)
    return MOE_ERR_ARG;
  if (L->down_layout == MOE_LAYOUT_MFMA16 && fd != MOE_FMT_MXFP4) return MOE_ERR_ARG;
  if (L->down_layout != MOE_LAYOUT_ROWS && L->d_ff % kTileCols) return MOE_ERR_SHAPE;
  if (L->down_layout == MOE_LAYOUT_MFMA16 && L->d_model % 16) return MOE_ERR_SHAPE;
  if (fg == MOE_FMT_INT4G32) {
    if (!L->gate_scale || !L->up_scale) return MOE_ERR_ARG;
    if (!aligned(L->gate_scale, 2) || !aligned(L->up_scale, 2)) return MOE_ERR_ALIGN;
    if (L->gate_scale_stride % 2 || L->up_scale_stride % 2) return MOE_ERR_ALIGN;
  }
  if (fd == MOE_FMT_INT4G32) {
    if (!L->down_scale) return MOE_ERR_ARG;
    if (!aligned(L->down_scale, 2) || L->down_scale_stride % 2) return MOE_ERR_ALIGN;
  }
  if (L->tid2eid) {
    if (L->vocab < 1) return MOE_ERR_ARG;
    if (!aligned(L->tid2eid, 4)) return MOE_ERR_ALIGN;
  }
  return MOE_OK;
}

// A hash-routed layer needs the tokens' ids.
int check_ids(const moe_layer_desc* L, const int32_t* token_ids) {
  if (L->tid2eid && !token_ids) return MOE_ERR_ARG;
  if (token_ids && !aligned(token_ids, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

WeightRef wref(const void* base, int64_t stride, const uint16_t* scale, int64_t scale_stride, int layout) {
  WeightRef w;
  w.base = static_cast<const uint8_t*>(base);
  w.stride = stride;
  w.scale = scale;
  w.scale_stride = scale_stride;
  w.layout = layout;
  return w;
}

// With hn set, the layer's activations are x = RMSNorm(hn) (bf16, eps): the
// single-launch kernel forms them itself when it can (hn must not alias y),
// otherwise the norm kernel writes them to xbuf first.
int layer_impl(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, const float* residual, void* ws,
               int32_t* idx_out, float* gw_out, void* const* events, hipStream_t s, uint64_t* trace = nullptr,
               const float* hn = nullptr, double eps = 0.0, uint16_t* xbuf = nullptr,
               const int32_t* token_ids = nullptr, const float* next_router = nullptr) {
  const HashRoute hr{L->tid2eid, token_ids, L->vocab};
  const int D = L->d_model, F = L->d_ff, E = L->n_experts, k = L->top_k;
  const WsLayout W = layer_ws_layout(B, D, F, E, k);
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto rec = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    return hipSuccess;
  };
  const WeightRef g = wref(L->gate, L->gate_stride, L->gate_scale, L->gate_scale_stride, MOE_LAYOUT_ROWS);
  const WeightRef u = wref(L->up, L->up_stride, L->up_scale, L->up_scale_stride, MOE_LAYOUT_ROWS);
  const WeightRef d = wref(L->down, L->down_stride, L->down_scale, L->down_scale_stride, L->down_layout);
  hipError_t e;
  if ((e = rec(0)) != hipSuccess) return hip_status(e);
  const int grid = fused_grid_size();
  int nx = xcd_count();
  if (nx == 0) nx = probe_xcd_count(reinterpret_cast<uint32_t*>(w + W.topo), grid, s);
  const int fd = down_fmt(L);
  const FusedShape sh = nx > 0 ? fused_shape(L->format, fd, B, k, D, F, grid, nx, L->down_layout) : FusedShape{};
  const bool fused = nx > 0 && sh.ok;
  // In-kernel norm for one token only: at B = 8 its redundant per-workgroup
  // work (every workgroup normalises the whole batch) costs more than the
  // separate norm kernel.
  if (hn && !(fused && sh.mfma && B == 1 && D <= kFusedNormMaxD && D % 8 == 0 && hn != y)) {
    if ((e = launch_rmsnorm_bf16(hn, B, D, eps, xbuf, s)) != hipSuccess) return hip_status(e);
    x_bf16 = xbuf;
    hn = nullptr;
  }
  if (fused) {
    e = launch_fused_layer(L->format, fd, L->router_w, x_bf16, hn, eps, g, u, d, E, D, F, k, B, w, W, y, residual,
                           idx_out, gw_out, trace, s, hr, next_router);
    if (e != hipSuccess) return hip_status(e);
  } else {
    if ((e = launch_route(L->router_w, E, D, x_bf16, B, k, w, W, idx_out, gw_out, nullptr, s, hr)) != hipSuccess)
      return hip_status(e);
    if ((e = launch_gate_up(L->format, g, u, D, F, B, k, w, W, s)) != hipSuccess) return hip_status(e);
    if ((e = launch_down(fd, d, D, F, B, k, w, W, s)) != hipSuccess) return hip_status(e);
    if ((e = launch_combine(D, B, k, w, W, y, residual, s)) != hipSuccess) return hip_status(e);
  }
  if ((e = rec(1)) != hipSuccess) return hip_status(e);
  return MOE_OK;
}

// The current device's copy of `scratch`, set up on the first call on that
// device: its address is looked up with that device current, and the array
// is cleared (counters, epoch and exchange words must start at zero) with
// the fill kernel; the stream is synchronised so that no later call on
// another stream can overtake the clearing.
std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[64];

int static_scratch(hipStream_t s, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= 64) return MOE_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_status(e);
    if (!p || !aligned(p, 256)) return MOE_ERR_WORKSPACE;
    static_assert(MOE_STATIC_SCRATCH_BYTES % 4 == 0 && MOE_STATIC_SCRATCH_BYTES / 4 < (1u << 30), "one fill launch");
    if ((e = launch_zero_u32(static_cast<uint32_t*>(p), (int)(MOE_STATIC_SCRATCH_BYTES / 4), s)) != hipSuccess)
      return hip_status(e);
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_status(e);
    g_scratch_dev[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  if (have < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int layer_entry(const moe_layer_desc* L, const int32_t* token_ids, const uint16_t* x_bf16, int B, float* y, void* ws,
                size_t ws_bytes, int32_t* idx_out, float* gw_out, void* const* events, void* stream) {
  int st = check_layer(L, B);
  if (st != MOE_OK) return st;
  if ((st = check_ids(L, token_ids)) != MOE_OK) return st;
  if (!x_bf16 || !y) return MOE_ERR_ARG;
  if (!aligned(x_bf16, 16) || !aligned(y, 16)) return MOE_ERR_ALIGN;
  const size_t need = layer_ws_layout(B, L->d_model, L->d_ff, L->n_experts, L->top_k).total;
  if ((st = check_ws(ws, ws_bytes, need)) != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  return layer_impl(L, x_bf16, B, y, nullptr, ws, idx_out, gw_out, events, (hipStream_t)stream, nullptr, nullptr,
                    0.0, nullptr, token_ids);
}
}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (null pointer or bad size)";
    case MOE_ERR_SHAPE: return "unsupported shape (block multiple, token count, top_k or expert count)";
    case MOE_ERR_ARCH: return "device is not gfx950";
    case MOE_ERR_HIP: return "HIP runtime error (see moe_last_hip_error)";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MOE_ERR_ALIGN: return "pointer or stride misaligned";
    case MOE_ERR_SCRATCH: return "the call needs more workspace than the library's static scratch holds";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip; }

int moe_device_check(void) { return arch_check(); }

int moe_expert_gemv_mxfp4(const uint8_t* blocks, int N, int K, const float* x, int B, float* y, void* stream) {
  int st = check_gemv(blocks, N, K, x, B, y, MOE_FMT_MXFP4);
  if (st != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  return hip_status(launch_gemv(MOE_FMT_MXFP4, blocks, nullptr, N, K, x, B, y, (hipStream_t)stream));
}

int moe_expert_gemv_q2k(const uint8_t* blocks, int N, int K, const float* x, int B, float* y, void* stream) {
  int st = check_gemv(blocks, N, K, x, B, y, MOE_FMT_Q2K);
  if (st != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  return hip_status(launch_gemv(MOE_FMT_Q2K, blocks, nullptr, N, K, x, B, y, (hipStream_t)stream));
}

int moe_expert_gemv_int4g32(const int32_t* q, const uint16_t* scale_bf16, int N, int K, const float* x, int B,
                            float* y, void* stream) {
  int st = check_gemv(q, N, K, x, B, y, MOE_FMT_INT4G32);
  if (st != MOE_OK) return st;
  if (!scale_bf16) return MOE_ERR_ARG;
  if (!aligned(scale_bf16, 2)) return MOE_ERR_ALIGN;
  if ((st = arch_check()) != MOE_OK) return st;
  return hip_status(launch_gemv(MOE_FMT_INT4G32, q, scale_bf16, N, K, x, B, y, (hipStream_t)stream));
}

int moe_q8k_quantize(const float* x, int B, int K, int8_t* q, float* d, void* stream) {
  if (!x || !q || !d) return MOE_ERR_ARG;
  if (B < 1 || K < 256 || K % 256 != 0) return MOE_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(d, 4)) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_q8k_quantize(x, B, K, q, d, (hipStream_t)stream));
}

int moe_expert_gemv_mxfp4_q8(const uint8_t* blocks, int N, int K, const int8_t* q, const float* d, int B, float* y,
                             void* stream) {
  if (!blocks || !q || !d || !y) return MOE_ERR_ARG;
  if (N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (B < 1 || B > MOE_MAX_TOKENS || K % 256 != 0) return MOE_ERR_SHAPE;
  if (!aligned(blocks, 4) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4)) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_gemv_q8(blocks, N, K, q, d, B, y, (hipStream_t)stream));
}

int moe_mxfp4_half_lut(uint16_t* lut, void* stream) {
  if (!lut) return MOE_ERR_ARG;
  if (!aligned(lut, 2)) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_half_lut(lut, (hipStream_t)stream));
}

int moe_expert_gemv_mxfp4_hlut(const uint8_t* blocks, int N, int K, const float* x, int B, float* y, void* stream) {
  int st = check_gemv(blocks, N, K, x, B, y, MOE_FMT_MXFP4);
  if (st != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  return hip_status(launch_gemv_hlut(blocks, N, K, x, B, y, (hipStream_t)stream));
}

size_t moe_route_workspace_bytes(int B, int D, int E, int top_k) {
  if (B < 1 || D < 1 || E < 1 || top_k < 1) return 0;
  // Routing uses the leading regions of a layer workspace, up to the
  // activation widened to fp32 (the region before h).
  return layer_ws_layout(B, D, 0, E, top_k).h;
}

int moe_route_topk(const float* router_w, int E, int D, const uint16_t* x_bf16, int B, int top_k, int32_t* idx,
                   float* gate_w, double* logits_out, void* ws, size_t ws_bytes, void* stream) {
  if (!router_w || !x_bf16 || !idx || !gate_w) return MOE_ERR_ARG;
  if (E < 1 || E > MOE_MAX_EXPERTS || D <= 0) return MOE_ERR_SHAPE;
  if (B < 1 || B > MOE_MAX_TOKENS || top_k < 1 || top_k > MOE_MAX_TOPK || top_k > E) return MOE_ERR_SHAPE;
  if (D % 4 != 0) return MOE_ERR_SHAPE;
  if (!aligned(router_w, 16) || !aligned(x_bf16, 8)) return MOE_ERR_ALIGN;
  // The route kernel also widens x into the xf region, which needs D.
  const WsLayout W = layer_ws_layout(B, D, 0, E, top_k);
  int st = check_ws(ws, ws_bytes, W.h);
  if (st != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  return hip_status(launch_route(router_w, E, D, x_bf16, B, top_k, static_cast<uint8_t*>(ws), W, idx, gate_w,
                                 logits_out, (hipStream_t)stream));
}

size_t moe_layer_workspace_bytes(int B, int D, int F, int E, int top_k) {
  if (B < 1 || D < 1 || F < 1 || E < 1 || top_k < 1) return 0;
  return layer_ws_layout(B, D, F, E, top_k).total;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 64 * sizeof(uint32_t) || !aligned(ws, 256) || ws_bytes % 4) return MOE_ERR_WORKSPACE;
  int st = arch_check();
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // First use on this device: check the workgroup placement the single-launch
  // layer relies on (synchronises the stream once), using the workspace as scratch.
  if (xcd_count() == 0 && ws_bytes >= 4096 * sizeof(uint32_t))
    probe_xcd_count(static_cast<uint32_t*>(ws), fused_grid_size(), s);
  // Zero everything: counters, epoch and every tagged exchange word.
  const size_t n = ws_bytes / 4;
  for (size_t off = 0; off < n; off += (size_t)1 << 30) {
    const size_t cnt = n - off < ((size_t)1 << 30) ? n - off : ((size_t)1 << 30);
    hipError_t e = launch_zero_u32(static_cast<uint32_t*>(ws) + off, (int)cnt, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return MOE_OK;
}


int moe_layer_decode(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, void* ws, size_t ws_bytes,
                     int32_t* idx_out, float* gw_out, void* stream) {
  return layer_entry(L, nullptr, x_bf16, B, y, ws, ws_bytes, idx_out, gw_out, nullptr, stream);
}

int moe_layer_decode_ids(const moe_layer_desc* L, const int32_t* token_ids, const uint16_t* x_bf16, int B, float* y,
                         void* ws, size_t ws_bytes, int32_t* idx_out, float* gw_out, void* stream) {
  return layer_entry(L, token_ids, x_bf16, B, y, ws, ws_bytes, idx_out, gw_out, nullptr, stream);
}

int moe_layer_decode_noalloc(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, int32_t* idx_out,
                             float* gw_out, void* stream) {
  int st = check_layer(L, B);
  if (st != MOE_OK) return st;
  if ((st = check_ids(L, nullptr)) != MOE_OK) return st;
  if (!x_bf16 || !y) return MOE_ERR_ARG;
  if (!aligned(x_bf16, 16) || !aligned(y, 16)) return MOE_ERR_ALIGN;
  if (layer_ws_layout(B, L->d_model, L->d_ff, L->n_experts, L->top_k).total > MOE_STATIC_SCRATCH_BYTES)
    return MOE_ERR_SCRATCH;
  if ((st = arch_check()) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = nullptr;
  if ((st = static_scratch(s, &ws)) != MOE_OK) return st;
  return layer_impl(L, x_bf16, B, y, nullptr, ws, idx_out, gw_out, nullptr, s);
}

int moe_workspace_flags(const void* ws, size_t ws_bytes, uint32_t* flags, void* stream) {
  if (!ws || !flags) return MOE_ERR_ARG;
  if (!aligned(ws, 256) || ws_bytes < (kCtrTimeout + 1) * sizeof(uint32_t)) return MOE_ERR_WORKSPACE;
  uint32_t c[2] = {0u, 0u};
  hipStream_t s = (hipStream_t)stream;
  const uint32_t* ctr = static_cast<const uint32_t*>(ws);  // the counters region comes first
  hipError_t e = hipMemcpyAsync(c, ctr + kCtrBadIds, sizeof(c), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  *flags = (c[1] ? 1u : 0u) | (c[0] ? 2u : 0u);
  return MOE_OK;
}

int moe_layer_decode_profiled(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, void* ws,
                              size_t ws_bytes, int32_t* idx_out, float* gw_out, void* const* events, void* stream) {
  return layer_entry(L, nullptr, x_bf16, B, y, ws, ws_bytes, idx_out, gw_out, events, stream);
}

int moe_layer_decode_traced(const moe_layer_desc* L, const uint16_t* x_bf16, int B, float* y, void* ws,
                            size_t ws_bytes, uint64_t* trace, int* trace_blocks, void* stream) {
  int st = check_layer(L, B);
  if (st != MOE_OK) return st;
  if ((st = check_ids(L, nullptr)) != MOE_OK) return st;
  if (!x_bf16 || !y || !trace_blocks) return MOE_ERR_ARG;
  if (!aligned(x_bf16, 16) || !aligned(y, 16)) return MOE_ERR_ALIGN;
  const size_t need = layer_ws_layout(B, L->d_model, L->d_ff, L->n_experts, L->top_k).total;
  if ((st = check_ws(ws, ws_bytes, need)) != MOE_OK) return st;
  if ((st = arch_check()) != MOE_OK) return st;
  const int grid = fused_grid_size();
  const int nx = xcd_count();
  const bool fused =
      nx > 0 && fused_shape(L->format, down_fmt(L), B, L->top_k, L->d_model, L->d_ff, grid, nx, L->down_layout).ok;
  *trace_blocks = fused ? grid : 0;
  if (!trace) return MOE_OK;  // size query
  return layer_impl(L, x_bf16, B, y, nullptr, ws, nullptr, nullptr, nullptr, (hipStream_t)stream, trace);
}

size_t moe_stack_workspace_bytes(int B, int D, int F, int E, int top_k) {
  const size_t layer = moe_layer_workspace_bytes(B, D, F, E, top_k);
  if (!layer) return 0;
  // + normalised activation (bf16) of the current layer, + one fp32 residual
  // state (layers alternate between it and h_out)
  return layer + align256((size_t)B * D * sizeof(uint16_t)) + align256((size_t)B * D * sizeof(float));
}

int moe_stack_decode(const moe_layer_desc* layers, int n_layers, const float* h_in, int B, float* h_out, double eps,
                     void* ws, size_t ws_bytes, void* stream) {
  return moe_stack_decode_ids(layers, n_layers, nullptr, h_in, B, h_out, eps, ws, ws_bytes, stream);
}

int moe_stack_decode_ids(const moe_layer_desc* layers, int n_layers, const int32_t* token_ids, const float* h_in,
                         int B, float* h_out, double eps, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 1 || !h_in || !h_out) return MOE_ERR_ARG;
  if (!(eps >= 0.0)) return MOE_ERR_ARG;
  int st;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_layer(&layers[l], B)) != MOE_OK) return st;
    if ((st = check_ids(&layers[l], token_ids)) != MOE_OK) return st;
    if (layers[l].d_model != layers[0].d_model || layers[l].d_ff != layers[0].d_ff ||
        layers[l].n_experts != layers[0].n_experts || layers[l].top_k != layers[0].top_k)
      return MOE_ERR_SHAPE;
  }
  if (!aligned(h_in, 16) || !aligned(h_out, 16)) return MOE_ERR_ALIGN;
  const int D = layers[0].d_model;
  const size_t layer_bytes = moe_layer_workspace_bytes(B, D, layers[0].d_ff, layers[0].n_experts, layers[0].top_k);
  if ((st = check_ws(ws, ws_bytes, moe_stack_workspace_bytes(B, D, layers[0].d_ff, layers[0].n_experts,
                                                            layers[0].top_k))) != MOE_OK)
    return st;
  if ((st = arch_check()) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* xb = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + layer_bytes);
  float* tmp = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + layer_bytes +
                                        align256((size_t)B * D * sizeof(uint16_t)));
  // Layer l reads h_l and writes h_{l+1} to another buffer (h_out for the
  // last layer, the two alternating backwards from it), so a layer that
  // normalises its own input never overwrites it.  If h_in aliases h_out
  // and layer 0 would write h_out, layer 0 takes the separate norm kernel.
  const float* cur = h_in;
  for (int l = 0; l < n_layers; ++l) {
    float* dst = (n_layers - 1 - l) % 2 == 0 ? h_out : tmp;
    // (layers of one stack share E and d_model, so layer l can pull its row
    // of layer l+1's router into L2)
    st = layer_impl(&layers[l], nullptr, B, dst, cur, ws, nullptr, nullptr, nullptr, s, nullptr, cur, eps, xb,
                    token_ids, l + 1 < n_layers ? layers[l + 1].router_w : nullptr);
    if (st != MOE_OK) return st;
    cur = dst;
  }
  return MOE_OK;
}

int moe_rmsnorm_bf16(const float* h, int B, int D, double eps, uint16_t* x_out, void* stream) {
  if (!h || !x_out || B < 1 || D < 1) return MOE_ERR_ARG;
  if (!(eps >= 0.0)) return MOE_ERR_ARG;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_rmsnorm_bf16(h, B, D, eps, x_out, (hipStream_t)stream));
}

int quantize_fp4_to_int4g32(const uint8_t* mxfp4, int N, int K, int32_t* q_out, uint16_t* scale_out, void* stream) {
  if (!mxfp4 || !q_out || !scale_out || N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (K % 32) return MOE_ERR_SHAPE;
  if (!aligned(mxfp4, 4) || !aligned(q_out, 16) || !aligned(scale_out, 2)) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_quantize_int4(mxfp4, (int64_t)N * (K / 32), q_out, scale_out, (hipStream_t)stream));
}

int moe_tile_weights(int format, const void* src, const uint16_t* src_scale, int N, int K, void* dst,
                     uint16_t* dst_scale, void* stream) {
  if (format < MOE_FMT_MXFP4 || format > MOE_FMT_INT4G32) return MOE_ERR_ARG;
  if (!src || !dst || N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (K % kTileCols) return MOE_ERR_SHAPE;
  const bool int4 = format == MOE_FMT_INT4G32;
  if (int4 && (!src_scale || !dst_scale)) return MOE_ERR_ARG;
  if (!int4 && (src_scale || dst_scale)) return MOE_ERR_ARG;
  if (!aligned(src, int4 ? 16 : 4) || !aligned(dst, int4 ? 16 : 4)) return MOE_ERR_ALIGN;
  if (int4 && (!aligned(src_scale, 2) || !aligned(dst_scale, 2))) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  const int tiles = K / kTileCols;
  hipStream_t s = (hipStream_t)stream;
  // Bytes of one row of one tile: 8 MXFP4 blocks, 1 Q2_K block, or 32 INT4
  // code words (+ 8 bfloat16 scales).
  const int tile_bytes = format == MOE_FMT_MXFP4 ? 8 * 17 : format == MOE_FMT_Q2K ? 84 : 128;
  hipError_t e = launch_tile_rows(src, dst, N, tiles, tile_bytes / 4, 4, s);
  if (e == hipSuccess && int4) e = launch_tile_rows(src_scale, dst_scale, N, tiles, kTileCols / 32, 2, s);
  return hip_status(e);
}

int moe_tile_weights_mfma16(const uint8_t* src, int N, int K, uint8_t* dst, void* stream) {
  if (!src || !dst || N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (K % kTileCols || N % 16) return MOE_ERR_SHAPE;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_tile_mfma16(src, dst, N, K, (hipStream_t)stream));
}

int moe_stream_read(const void* src, size_t bytes, int pattern, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0) return MOE_ERR_ARG;
  if (pattern != MOE_STREAM_DWORDX4 && pattern != MOE_STREAM_MXFP4) return MOE_ERR_ARG;
  if (pattern == MOE_STREAM_DWORDX4 ? (!aligned(src, 16) || bytes % 16) : (!aligned(src, 4) || bytes % 4))
    return MOE_ERR_ALIGN;
  if (pattern == MOE_STREAM_MXFP4 && bytes < 20) return MOE_ERR_SHAPE;
  if (!aligned(sink, 4)) return MOE_ERR_ALIGN;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_stream_read(src, (int64_t)bytes, pattern, sink, (hipStream_t)stream));
}

int moe_validate_mxfp4(const uint8_t* blocks, int64_t n_blocks, int32_t* bad_count_dev, void* stream) {
  if (!blocks || !bad_count_dev || n_blocks < 0) return MOE_ERR_ARG;
  int st = arch_check();
  if (st != MOE_OK) return st;
  return hip_status(launch_validate_mxfp4(blocks, n_blocks, bad_count_dev, (hipStream_t)stream));
}

}  // extern "C"
