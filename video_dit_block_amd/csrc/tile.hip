// Cube tiling of the latent token grid, and its inverse.
//
// VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs, section "Two-Stage Architecture" (Stage 1 groups tokens into (4, 4, 4)
// cubes of 64); Wan2.2 Production Values dataset card, section "Shapes" (the
// attention sequence is cube-major and padded: S_padded = Nc x 64, with vbs
// real tokens per cube).
//
// In BSHD the NH*D values of one token are contiguous (NH*D*2 bytes: 10 KiB
// for 40 heads of 128), so tiling is a gather of whole token rows. Each
// workgroup moves 16 slots of one cube; each wave copies one row at a time
// with 16-byte accesses across its 64 lanes, so every access instruction
// covers 1 KiB of contiguous memory. Padding slots are written as zeros and
// never read. The work is a pure copy and is bound by HBM bandwidth.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr int kSlotsPerBlock = 16;
constexpr int kSplit = kCube / kSlotsPerBlock;  // workgroups per cube
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Copy one row of `cpr` 16-byte chunks (src == nullptr: write zeros).
__device__ __forceinline__ void copy_row(const u32x4* __restrict__ src,
                                         u32x4* __restrict__ dst, int cpr,
                                         int lane) {
  if (src == nullptr) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int col = lane; col < cpr; col += 64) dst[col] = z;
    return;
  }
  int col = lane;
  for (; col + 64 * (kUnroll - 1) < cpr; col += 64 * kUnroll) {
    u32x4 t[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) t[i] = __builtin_nontemporal_load(src + col + 64 * i);
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) __builtin_nontemporal_store(t[i], dst + col + 64 * i);
  }
  for (; col < cpr; col += 64) __builtin_nontemporal_store(__builtin_nontemporal_load(src + col), dst + col);
}

// grid (Nc * kSplit, B), block kThreads. kInverse = false: natural -> tiled;
// true: tiled -> natural (padding slots skipped).
template <bool kInverse>
__global__ __launch_bounds__(kThreads) void tile_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int32_t* vbs_out,
    int T, int H, int W, int Nh, int Nw, int cpr) {
  const int c = blockIdx.x / kSplit;
  const int part = blockIdx.x - c * kSplit;
  const int b = blockIdx.y;
  const int cw = c % Nw;
  const int ch = (c / Nw) % Nh;
  const int ct = c / (Nw * Nh);
  const int eh = cube_extent(H, ch), ew = cube_extent(W, cw);
  const int n_real = cube_extent(T, ct) * eh * ew;
  if (!kInverse && vbs_out != nullptr && part == 0 && b == 0 && threadIdx.x == 0)
    vbs_out[c] = n_real;

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const size_t n_nat = (size_t)T * H * W;
  const size_t n_tiled = (size_t)gridDim.x / kSplit * kCube;
#pragma unroll 1
  for (int r = 0; r < kSlotsPerBlock / 4; ++r) {
    const int u = part * kSlotsPerBlock + r * 4 + wave;
    const size_t tiled_row = (size_t)b * n_tiled + (size_t)c * kCube + u;
    if (u < n_real) {
      const size_t nat_row =
          (size_t)b * n_nat + slot_token(u, ct, ch, cw, eh, ew, H, W);
      if (kInverse)
        copy_row(src + tiled_row * cpr, dst + nat_row * cpr, cpr, lane);
      else
        copy_row(src + nat_row * cpr, dst + tiled_row * cpr, cpr, lane);
    } else if (!kInverse) {
      copy_row(nullptr, dst + tiled_row * cpr, cpr, lane);
    }
  }
}

}  // namespace

hipError_t launch_tile(const uint16_t* x, uint16_t* x_tiled, int32_t* vbs, int B,
                       int T, int H, int W, int NH, int D, hipStream_t stream) {
  const int Nt = (T + 3) / 4, Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  const int cpr = NH * D * 2 / 16;
  dim3 grid(Nt * Nh * Nw * kSplit, B);
  hipLaunchKernelGGL(tile_kernel<false>, grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(x),
                     reinterpret_cast<u32x4*>(x_tiled), vbs, T, H, W, Nh, Nw, cpr);
  return hipGetLastError();
}

hipError_t launch_untile(const uint16_t* y_tiled, uint16_t* y, int B, int T,
                         int H, int W, int NH, int D, hipStream_t stream) {
  const int Nt = (T + 3) / 4, Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  const int cpr = NH * D * 2 / 16;
  dim3 grid(Nt * Nh * Nw * kSplit, B);
  hipLaunchKernelGGL(tile_kernel<true>, grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(y_tiled),
                     reinterpret_cast<u32x4*>(y), nullptr, T, H, W, Nh, Nw, cpr);
  return hipGetLastError();
}

}  // namespace vsa
