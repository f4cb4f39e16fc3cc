// libvsa C ABI: host-side argument validation, then asynchronous launches on
// the caller's stream. No entry point allocates or frees device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "launch.h"
#include "vsa.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_err[0] = '\0';
  return VSA_OK;
}

constexpr int64_t kMaxGridX = 2147483647;
constexpr int64_t kMaxGridYZ = 65535;
// vsa_fwd addresses a 16-row tile quarter by a 32-bit byte offset from its head's first
// key row: one batch's k (Nkv * 64 rows of NH * D bf16) must span < 4 GiB.
constexpr uint64_t kMaxFwdKvBytes = 1ull << 32;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of (B, NH, D). Rows of NH*D bf16 are moved in 16-byte chunks;
// one cube's rows (64 * NH * D elements) are indexed with 32-bit offsets.
int32_t check_bhd(int32_t B, int32_t NH, int32_t D) {
  if (B <= 0 || NH <= 0 || D <= 0)
    return fail(VSA_ERR_SHAPE, "B=%d NH=%d D=%d must be positive", B, NH, D);
  if (D != 64 && D != 128)
    return fail(VSA_ERR_UNSUPPORTED, "D=%d not supported (64 or 128)", D);
  if (B > kMaxGridYZ) return fail(VSA_ERR_SHAPE, "B=%d exceeds %lld", B, (long long)kMaxGridYZ);
  if ((int64_t)NH * D * 64 > 2147483647LL)
    return fail(VSA_ERR_SHAPE, "NH*D*64 = %lld exceeds 2^31-1", (long long)NH * D * 64);
  return VSA_OK;
}

int32_t check_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  return VSA_OK;
}

int32_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VSA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

int64_t num_cubes64(int32_t T, int32_t H, int32_t W) {
  if (T <= 0 || H <= 0 || W <= 0) return -1;
  return (int64_t)((T + 3) / 4) * ((H + 3) / 4) * ((W + 3) / 4);
}

int32_t check_grid(int32_t T, int32_t H, int32_t W, int64_t* nc) {
  *nc = num_cubes64(T, H, W);
  if (*nc < 0) return fail(VSA_ERR_SHAPE, "grid %dx%dx%d must be positive", T, H, W);
  if (*nc * 4 > kMaxGridX) return fail(VSA_ERR_SHAPE, "too many cubes: %lld", (long long)*nc);
  return VSA_OK;
}

// Scratch of vsa_select_noalloc: the selector's workspace (pooled q and k,
// the cube scores) for as many (batch, head) pairs as fit, in a file-scope
// device array. Every GPU the library runs on holds its own copy of it until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: kernels and copies receive the per-device address that
// hipGetSymbolAddress returns, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int32_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VSA_ERR_UNSUPPORTED, "device %d above the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(VSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

int32_t vsa_abi_version(void) { return VSA_ABI_VERSION; }

const char* vsa_status_string(int32_t status) {
  switch (status) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_NULL: return "VSA_ERR_NULL";
    case VSA_ERR_SHAPE: return "VSA_ERR_SHAPE";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
    case VSA_ERR_RANGE: return "VSA_ERR_RANGE";
    case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE";
    case VSA_ERR_HIP: return "VSA_ERR_HIP";
    default: return "VSA_ERR_UNKNOWN";
  }
}

const char* vsa_last_error(void) { return g_err; }

int32_t vsa_num_cubes(int32_t T, int32_t H, int32_t W) {
  const int64_t n = num_cubes64(T, H, W);
  return (n < 0 || n > 2147483647LL) ? -1 : (int32_t)n;
}

int32_t vsa_vbs_host(int32_t T, int32_t H, int32_t W, int32_t* vbs, int32_t n_vbs) {
  if (vbs == nullptr) return fail(VSA_ERR_NULL, "vbs is NULL");
  const int64_t nc = num_cubes64(T, H, W);
  if (nc < 0) return fail(VSA_ERR_SHAPE, "grid %dx%dx%d must be positive", T, H, W);
  if (nc > n_vbs) return fail(VSA_ERR_SHAPE, "vbs holds %d entries, %lld needed", n_vbs, (long long)nc);
  const int Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  for (int64_t c = 0; c < nc; ++c) {
    const int cw = (int)(c % Nw), ch = (int)((c / Nw) % Nh), ct = (int)(c / ((int64_t)Nw * Nh));
    const int et = T - 4 * ct < 4 ? T - 4 * ct : 4;
    const int eh = H - 4 * ch < 4 ? H - 4 * ch : 4;
    const int ew = W - 4 * cw < 4 ? W - 4 * cw : 4;
    vbs[c] = et * eh * ew;
  }
  return ok();
}

int32_t vsa_tile(const vsa_bf16_t* x, vsa_bf16_t* x_tiled, int32_t* vbs, int32_t B,
                 int32_t T, int32_t H, int32_t W, int32_t NH, int32_t D,
                 vsa_stream_t stream) {
  if (x == nullptr || x_tiled == nullptr) return fail(VSA_ERR_NULL, "x or x_tiled is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  int64_t nc;
  if ((s = check_grid(T, H, W, &nc)) != VSA_OK) return s;
  if (!aligned16(x) || !aligned16(x_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "x and x_tiled must be 16-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_tile(x, x_tiled, vbs, nullptr, B, T, H, W, NH, D,
                                   static_cast<hipStream_t>(stream)), "tile");
}

int32_t vsa_untile(const vsa_bf16_t* y_tiled, vsa_bf16_t* y, int32_t B, int32_t T,
                   int32_t H, int32_t W, int32_t NH, int32_t D, vsa_stream_t stream) {
  if (y_tiled == nullptr || y == nullptr) return fail(VSA_ERR_NULL, "y_tiled or y is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  int64_t nc;
  if ((s = check_grid(T, H, W, &nc)) != VSA_OK) return s;
  if (!aligned16(y) || !aligned16(y_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "y and y_tiled must be 16-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_untile(y_tiled, y, nullptr, B, T, H, W, NH, D,
                                     static_cast<hipStream_t>(stream)), "untile");
}

int32_t vsa_cube_order_host(int32_t T, int32_t H, int32_t W, int32_t kind, int32_t* order,
                            int32_t n_order) {
  if (order == nullptr) return fail(VSA_ERR_NULL, "order is NULL");
  const int64_t nc = num_cubes64(T, H, W);
  if (nc < 0) return fail(VSA_ERR_SHAPE, "grid %dx%dx%d must be positive", T, H, W);
  if (nc > n_order)
    return fail(VSA_ERR_SHAPE, "order holds %d entries, %lld needed", n_order, (long long)nc);
  if (kind != VSA_ORDER_ROW_MAJOR && kind != VSA_ORDER_HILBERT)
    return fail(VSA_ERR_RANGE, "unknown cube order kind %d", kind);
  if (!vsa::cube_order(T, H, W, kind, order))
    return fail(VSA_ERR_UNSUPPORTED, "grid %dx%dx%d too large for a 63-bit Hilbert index", T, H,
                W);
  return ok();
}

int32_t vsa_tile_ordered(const vsa_bf16_t* x, vsa_bf16_t* x_tiled, int32_t* vbs,
                         const int32_t* order, int32_t B, int32_t T, int32_t H, int32_t W,
                         int32_t NH, int32_t D, vsa_stream_t stream) {
  if (order == nullptr) return fail(VSA_ERR_NULL, "order is NULL");
  if (x == nullptr || x_tiled == nullptr) return fail(VSA_ERR_NULL, "x or x_tiled is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  int64_t nc;
  if ((s = check_grid(T, H, W, &nc)) != VSA_OK) return s;
  if (!aligned16(x) || !aligned16(x_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "x and x_tiled must be 16-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_tile(x, x_tiled, vbs, order, B, T, H, W, NH, D,
                                   static_cast<hipStream_t>(stream)), "tile_ordered");
}

int32_t vsa_untile_ordered(const vsa_bf16_t* y_tiled, vsa_bf16_t* y, const int32_t* order,
                           int32_t B, int32_t T, int32_t H, int32_t W, int32_t NH, int32_t D,
                           vsa_stream_t stream) {
  if (order == nullptr) return fail(VSA_ERR_NULL, "order is NULL");
  if (y_tiled == nullptr || y == nullptr) return fail(VSA_ERR_NULL, "y_tiled or y is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  int64_t nc;
  if ((s = check_grid(T, H, W, &nc)) != VSA_OK) return s;
  if (!aligned16(y) || !aligned16(y_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "y and y_tiled must be 16-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_untile(y_tiled, y, order, B, T, H, W, NH, D,
                                     static_cast<hipStream_t>(stream)), "untile_ordered");
}

int32_t vsa_mask_to_lut(const uint8_t* block_mask, int32_t B, int32_t NH, int32_t Nq,
                        int32_t Nkv, int32_t max_kv, int32_t* kv_block_idx,
                        int32_t* valid_block_num, int32_t* n_truncated, vsa_stream_t stream) {
  if (block_mask == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr)
    return fail(VSA_ERR_NULL, "block_mask, kv_block_idx or valid_block_num is NULL");
  if (B <= 0 || NH <= 0 || Nq <= 0 || Nkv <= 0)
    return fail(VSA_ERR_SHAPE, "B=%d NH=%d Nq=%d Nkv=%d must be positive", B, NH, Nq, Nkv);
  if (max_kv < 1 || max_kv > Nkv) return fail(VSA_ERR_RANGE, "max_kv=%d outside [1, %d]", max_kv, Nkv);
  // four rows per workgroup: at most 4 * (2^31 - 1) rows; the mask (rows *
  // Nkv bytes) then stays far below 2^63
  const int64_t bh = (int64_t)B * NH;
  if (bh > 4 * kMaxGridX / Nq)
    return fail(VSA_ERR_SHAPE, "B*NH*Nq = %lld*%d rows exceed the grid", (long long)bh, Nq);
  const int64_t rows = bh * Nq;
  int32_t s = check_device();
  if (s != VSA_OK) return s;
  return launched(vsa::launch_mask_to_lut(block_mask, rows, Nkv, max_kv, kv_block_idx,
                                          valid_block_num, n_truncated,
                                          static_cast<hipStream_t>(stream)),
                  "mask_to_lut");
}

size_t vsa_select_workspace_bytes(int32_t B, int32_t NH, int32_t Nc, int32_t D) {
  if (B <= 0 || NH <= 0 || Nc <= 0 || D <= 0) return 0;
  return vsa::select_workspace(B, NH, Nc, D).total;
}

int32_t vsa_select(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                   const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                   int32_t topk, int32_t* topk_idx, void* workspace,
                   size_t workspace_bytes, vsa_stream_t stream) {
  if (q_tiled == nullptr || k_tiled == nullptr || vbs == nullptr || topk_idx == nullptr)
    return fail(VSA_ERR_NULL, "q_tiled, k_tiled, vbs or topk_idx is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nc <= 0) return fail(VSA_ERR_SHAPE, "Nc=%d must be positive", Nc);
  if (Nc > VSA_MAX_CUBES)
    return fail(VSA_ERR_UNSUPPORTED, "Nc=%d exceeds VSA_MAX_CUBES=%d", Nc, VSA_MAX_CUBES);
  if ((int64_t)B * NH > kMaxGridYZ)
    return fail(VSA_ERR_SHAPE, "B*NH=%lld exceeds %lld", (long long)B * NH, (long long)kMaxGridYZ);
  if (topk < 1 || topk > Nc) return fail(VSA_ERR_RANGE, "topk=%d outside [1, %d]", topk, Nc);
  if (!aligned16(q_tiled) || !aligned16(k_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "q_tiled and k_tiled must be 16-byte aligned");
  const size_t need = vsa::select_workspace(B, NH, Nc, D).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(VSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_select(q_tiled, k_tiled, vbs, B, Nc, NH, D, topk, topk_idx,
                                     nullptr, 0.0f, 0.0f, workspace,
                                     static_cast<hipStream_t>(stream)),
                  "select");
}

size_t vsa_select_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int32_t vsa_select_noalloc(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                           const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                           int32_t topk, int32_t* topk_idx, vsa_stream_t stream) {
  if (q_tiled == nullptr || k_tiled == nullptr || vbs == nullptr || topk_idx == nullptr)
    return fail(VSA_ERR_NULL, "q_tiled, k_tiled, vbs or topk_idx is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nc <= 0) return fail(VSA_ERR_SHAPE, "Nc=%d must be positive", Nc);
  if (Nc > VSA_MAX_CUBES)
    return fail(VSA_ERR_UNSUPPORTED, "Nc=%d exceeds VSA_MAX_CUBES=%d", Nc, VSA_MAX_CUBES);
  if (topk < 1 || topk > Nc) return fail(VSA_ERR_RANGE, "topk=%d outside [1, %d]", topk, Nc);
  if (!aligned16(q_tiled) || !aligned16(k_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "q_tiled and k_tiled must be 16-byte aligned");
  // heads per chunk: the most whose workspace fits the scratch
  const size_t one = vsa::select_workspace(1, 1, Nc, D).total;
  if (one > kNoAllocScratchBytes)
    return fail(VSA_ERR_UNSUPPORTED,
                "one head of Nc=%d cubes needs %zu bytes of scratch, above the %zu of "
                "vsa_select_noalloc (use vsa_select with a workspace)",
                Nc, one, kNoAllocScratchBytes);
  int32_t chunk = (int32_t)(kNoAllocScratchBytes / one);
  if (chunk > NH) chunk = NH;
  while (chunk > 1 && vsa::select_workspace(1, chunk, Nc, D).total > kNoAllocScratchBytes) --chunk;
  if ((s = check_device()) != VSA_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != VSA_OK) return s;
  const size_t row = (size_t)NH * D;  // elements per tiled token row
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h0 = 0; h0 < NH; h0 += chunk) {
      const int32_t nh = NH - h0 < chunk ? NH - h0 : chunk;
      const size_t off = (size_t)b * Nc * 64 * row + (size_t)h0 * D;
      int32_t* idx = topk_idx + ((size_t)b * NH + h0) * Nc * topk;
      const hipError_t e = vsa::launch_select(q_tiled + off, k_tiled + off, vbs, 1, Nc, nh, D,
                                              topk, idx, nullptr, 0.0f, 0.0f, ws,
                                              static_cast<hipStream_t>(stream), NH);
      if (e != hipSuccess) return launched(e, "select_noalloc");
    }
  return ok();
}

int32_t vsa_select_cdf(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                       const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                       int32_t max_k, float tau, float sm_scale, int32_t* kv_block_idx,
                       int32_t* valid_block_num, void* workspace, size_t workspace_bytes,
                       vsa_stream_t stream) {
  if (valid_block_num == nullptr) return fail(VSA_ERR_NULL, "valid_block_num is NULL");
  if (!(tau > 0.0f && tau <= 1.0f)) return fail(VSA_ERR_RANGE, "tau must be in (0, 1]");
  if (!isfinite(sm_scale)) return fail(VSA_ERR_RANGE, "sm_scale is not finite");
  if (q_tiled == nullptr || k_tiled == nullptr || vbs == nullptr || kv_block_idx == nullptr)
    return fail(VSA_ERR_NULL, "q_tiled, k_tiled, vbs or kv_block_idx is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nc <= 0) return fail(VSA_ERR_SHAPE, "Nc=%d must be positive", Nc);
  if (Nc > VSA_MAX_CUBES)
    return fail(VSA_ERR_UNSUPPORTED, "Nc=%d exceeds VSA_MAX_CUBES=%d", Nc, VSA_MAX_CUBES);
  if ((int64_t)B * NH > kMaxGridYZ)
    return fail(VSA_ERR_SHAPE, "B*NH=%lld exceeds %lld", (long long)B * NH, (long long)kMaxGridYZ);
  if (max_k < 1 || max_k > Nc) return fail(VSA_ERR_RANGE, "max_k=%d outside [1, %d]", max_k, Nc);
  if (!aligned16(q_tiled) || !aligned16(k_tiled))
    return fail(VSA_ERR_UNSUPPORTED, "q_tiled and k_tiled must be 16-byte aligned");
  const size_t need = vsa::select_workspace(B, NH, Nc, D).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(VSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (sm_scale <= 0.0f) sm_scale = 1.0f / sqrtf((float)D);
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_select(q_tiled, k_tiled, vbs, B, Nc, NH, D, max_k, kv_block_idx,
                                     valid_block_num, sm_scale, tau, workspace,
                                     static_cast<hipStream_t>(stream)),
                  "select_cdf");
}

size_t vsa_coarse_workspace_bytes(int32_t B, int32_t NH, int32_t Nc, int32_t D) {
  if (B <= 0 || NH <= 0 || Nc <= 0 || D <= 0) return 0;
  return vsa::coarse_workspace_bytes(B, NH, Nc, D);
}

int32_t vsa_coarse(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                   const vsa_bf16_t* v_tiled, const int32_t* vbs, int32_t B, int32_t Nc,
                   int32_t NH, int32_t D, int32_t topk, int32_t* topk_idx, float sm_scale,
                   float* o_coarse, void* workspace, size_t workspace_bytes,
                   vsa_stream_t stream) {
  if (q_tiled == nullptr || k_tiled == nullptr || v_tiled == nullptr || vbs == nullptr ||
      o_coarse == nullptr)
    return fail(VSA_ERR_NULL, "q_tiled, k_tiled, v_tiled, vbs or o_coarse is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nc <= 0) return fail(VSA_ERR_SHAPE, "Nc=%d must be positive", Nc);
  if (Nc > VSA_MAX_CUBES)
    return fail(VSA_ERR_UNSUPPORTED, "Nc=%d exceeds VSA_MAX_CUBES=%d", Nc, VSA_MAX_CUBES);
  if ((int64_t)B * NH > kMaxGridYZ)
    return fail(VSA_ERR_SHAPE, "B*NH=%lld exceeds %lld", (long long)B * NH, (long long)kMaxGridYZ);
  if (topk_idx != nullptr && (topk < 1 || topk > Nc))
    return fail(VSA_ERR_RANGE, "topk=%d outside [1, %d]", topk, Nc);
  if (!isfinite(sm_scale)) return fail(VSA_ERR_RANGE, "sm_scale is not finite");
  if (!aligned16(q_tiled) || !aligned16(k_tiled) || !aligned16(v_tiled) || !aligned16(o_coarse))
    return fail(VSA_ERR_UNSUPPORTED, "q_tiled, k_tiled, v_tiled and o_coarse must be 16-byte aligned");
  const size_t need = vsa::coarse_workspace_bytes(B, NH, Nc, D);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(VSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (sm_scale <= 0.0f) sm_scale = 1.0f / sqrtf((float)D);
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_coarse(q_tiled, k_tiled, v_tiled, vbs, B, Nc, NH, D, topk,
                                     topk_idx, sm_scale, o_coarse, workspace,
                                     static_cast<hipStream_t>(stream)),
                  "coarse");
}

int32_t vsa_gate_combine(const vsa_bf16_t* o_fine, const float* o_coarse,
                         const vsa_bf16_t* gate_coarse, const vsa_bf16_t* gate_fine,
                         vsa_bf16_t* out, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                         vsa_stream_t stream) {
  if (o_fine == nullptr || o_coarse == nullptr || gate_coarse == nullptr ||
      gate_fine == nullptr || out == nullptr)
    return fail(VSA_ERR_NULL, "o_fine, o_coarse, gate_coarse, gate_fine or out is NULL");
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nc <= 0) return fail(VSA_ERR_SHAPE, "Nc=%d must be positive", Nc);
  if ((int64_t)B * Nc * 64 > kMaxGridX)
    return fail(VSA_ERR_SHAPE, "B*Nc*64=%lld exceeds %lld", (long long)B * Nc * 64,
                (long long)kMaxGridX);
  if (!aligned16(o_fine) || !aligned16(o_coarse) || !aligned16(gate_coarse) ||
      !aligned16(gate_fine) || !aligned16(out))
    return fail(VSA_ERR_UNSUPPORTED, "all buffers must be 16-byte aligned");
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_gate_combine(o_fine, o_coarse, gate_coarse, gate_fine, out, B, Nc,
                                           NH, D, static_cast<hipStream_t>(stream)),
                  "gate_combine");
}

size_t vsa_fwd_workspace_bytes_ex(int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                                  int32_t topk, int32_t kv_splits) {
  if (B <= 0 || Nq <= 0 || Nkv <= 0 || NH <= 0 || D <= 0 || topk <= 0 || kv_splits < 0 ||
      kv_splits > vsa::kMaxSplits)
    return 0;
  return vsa::fwd_workspace(B, Nq, Nkv, NH, D, topk, kv_splits).total;
}

size_t vsa_fwd_workspace_bytes(int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                               int32_t topk) {
  return vsa_fwd_workspace_bytes_ex(B, Nq, Nkv, NH, D, topk, 0);
}

int32_t vsa_fwd_splits(int32_t Nkv, int32_t D, int32_t topk, int32_t kv_splits) {
  if (Nkv <= 0 || D <= 0 || topk <= 0 || topk > Nkv || kv_splits < 0 ||
      kv_splits > vsa::kMaxSplits)
    return 0;
  return vsa::fwd_splits(Nkv, D, topk, kv_splits);
}

namespace {
// Shared argument checks and launch of vsa_fwd and vsa_fwd_lut.
int32_t fwd_common(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                   const int32_t* idx, const int32_t* valid, const int32_t* vbs,
                   vsa_bf16_t* out, float* lse, float* max_prob, int32_t B, int32_t Nq,
                   int32_t Nkv, int32_t NH, int32_t D, int32_t row_len, float sm_scale,
                   int32_t kv_splits, void* workspace, size_t workspace_bytes,
                   vsa_stream_t stream) {
  int32_t s = check_bhd(B, NH, D);
  if (s != VSA_OK) return s;
  if (Nq <= 0 || Nkv <= 0) return fail(VSA_ERR_SHAPE, "Nq=%d Nkv=%d must be positive", Nq, Nkv);
  if (row_len < 1 || row_len > Nkv)
    return fail(VSA_ERR_RANGE, "index row length %d outside [1, %d]", row_len, Nkv);
  if (kv_splits < 0 || kv_splits > vsa::kMaxSplits)
    return fail(VSA_ERR_RANGE, "kv_splits=%d outside [0, %d]", kv_splits, vsa::kMaxSplits);
  const int splits = vsa::fwd_splits(Nkv, D, row_len, kv_splits);
  if ((int64_t)B * NH * Nq * splits > kMaxGridX)
    return fail(VSA_ERR_SHAPE, "B*NH*Nq*splits=%lld exceeds %lld",
                (long long)B * NH * Nq * splits, (long long)kMaxGridX);
  if (!isfinite(sm_scale)) return fail(VSA_ERR_RANGE, "sm_scale is not finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(VSA_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  if (B > kMaxGridYZ) return fail(VSA_ERR_SHAPE, "B=%d exceeds %lld", B, (long long)kMaxGridYZ);
  if ((uint64_t)Nkv * 64u * (uint64_t)NH * (uint64_t)D * 2u >= kMaxFwdKvBytes)
    return fail(VSA_ERR_UNSUPPORTED, "Nkv * 64 * NH * D * 2 = %llu bytes per batch must be < 2^32",
                (unsigned long long)Nkv * 64ull * NH * D * 2ull);
  const size_t need = vsa::fwd_workspace(B, Nq, Nkv, NH, D, row_len, kv_splits).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(VSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (sm_scale <= 0.0f) sm_scale = 1.0f / sqrtf((float)D);
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_fwd(q, k, v, idx, valid, vbs, out, lse, max_prob, B, Nq, Nkv, NH,
                                  D, row_len, sm_scale, kv_splits, workspace,
                                  static_cast<hipStream_t>(stream)),
                  "fwd");
}
}  // namespace

int32_t vsa_fwd(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                const int32_t* topk_idx, const int32_t* vbs, vsa_bf16_t* out, int32_t B,
                int32_t Nq, int32_t Nkv, int32_t NH, int32_t D, int32_t topk,
                float sm_scale, void* workspace, size_t workspace_bytes,
                vsa_stream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || topk_idx == nullptr ||
      vbs == nullptr || out == nullptr)
    return fail(VSA_ERR_NULL, "q, k, v, topk_idx, vbs or out is NULL");
  if (topk < 1 || topk > Nkv) return fail(VSA_ERR_RANGE, "topk=%d outside [1, %d]", topk, Nkv);
  return fwd_common(q, k, v, topk_idx, nullptr, vbs, out, nullptr, nullptr, B, Nq, Nkv, NH, D,
                    topk, sm_scale, 0, workspace, workspace_bytes, stream);
}

int32_t vsa_fwd_lut_ex(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                       const int32_t* kv_block_idx, const int32_t* valid_block_num,
                       const int32_t* vbs, vsa_bf16_t* out, float* lse, float* max_prob,
                       int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                       int32_t max_kv, float sm_scale, int32_t kv_splits, void* workspace,
                       size_t workspace_bytes, vsa_stream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || kv_block_idx == nullptr ||
      vbs == nullptr || out == nullptr)
    return fail(VSA_ERR_NULL, "q, k, v, kv_block_idx, vbs or out is NULL");
  if (max_kv < 1 || max_kv > Nkv)
    return fail(VSA_ERR_RANGE, "max_kv=%d outside [1, %d]", max_kv, Nkv);
  if ((lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) ||
      (max_prob != nullptr && (reinterpret_cast<uintptr_t>(max_prob) & 3u) != 0))
    return fail(VSA_ERR_UNSUPPORTED, "lse and max_prob must be 4-byte aligned");
  return fwd_common(q, k, v, kv_block_idx, valid_block_num, vbs, out, lse, max_prob, B, Nq,
                    Nkv, NH, D, max_kv, sm_scale, kv_splits, workspace, workspace_bytes, stream);
}

int32_t vsa_fwd_lut(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                    const int32_t* kv_block_idx, const int32_t* valid_block_num,
                    const int32_t* vbs, vsa_bf16_t* out, float* lse, float* max_prob,
                    int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                    int32_t max_kv, float sm_scale, void* workspace,
                    size_t workspace_bytes, vsa_stream_t stream) {
  return vsa_fwd_lut_ex(q, k, v, kv_block_idx, valid_block_num, vbs, out, lse, max_prob, B, Nq,
                        Nkv, NH, D, max_kv, sm_scale, 0, workspace, workspace_bytes, stream);
}

int32_t vsa_validate_topk(const int32_t* topk_idx, int32_t B, int32_t NH, int32_t Nq,
                          int32_t Nkv, int32_t topk, int32_t* bad_count,
                          vsa_stream_t stream) {
  if (topk_idx == nullptr || bad_count == nullptr)
    return fail(VSA_ERR_NULL, "topk_idx or bad_count is NULL");
  if (B <= 0 || NH <= 0 || Nq <= 0 || Nkv <= 0)
    return fail(VSA_ERR_SHAPE, "B, NH, Nq, Nkv must be positive");
  if (Nkv > VSA_MAX_CUBES)
    return fail(VSA_ERR_UNSUPPORTED, "Nkv=%d exceeds VSA_MAX_CUBES=%d", Nkv, VSA_MAX_CUBES);
  if ((int64_t)B * NH * Nq > kMaxGridX) return fail(VSA_ERR_SHAPE, "too many rows");
  if (topk < 1) return fail(VSA_ERR_RANGE, "topk=%d must be >= 1", topk);
  int32_t s;
  if ((s = check_device()) != VSA_OK) return s;
  return launched(vsa::launch_validate_topk(topk_idx, B, NH, Nq, Nkv, topk, bad_count,
                                            static_cast<hipStream_t>(stream)), "validate_topk");
}

}  // extern "C"
