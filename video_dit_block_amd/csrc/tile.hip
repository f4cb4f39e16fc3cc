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
// workgroup moves 8 slots of one cube; each wave copies one row at a time
// with 16-byte accesses across its 64 lanes, so every access instruction
// covers 1 KiB of contiguous memory. Padding slots are written as zeros and
// never read. The work is a pure copy and is bound by HBM bandwidth.
//
// Cube order. By default tiled cube p is the cube with row-major id p,
// (ct * Nh + ch) * Nw + cw. An order table may instead place row-major cube
// order[p] at position p; cube_order() builds the row-major table or a 3D
// Hilbert curve over the cube grid. (The VSA blog, "Two-Stage Architecture",
// pre-stage: tokens are reordered along a 3D space-filling curve so that each
// block is a compact spatial-temporal region; the curve is not named. Here
// the 4x4x4 cube is the curve's leaf, so every block is compact by
// construction, and the curve orders the cubes.) The Hilbert index of (ct, ch, cw) follows J. Skilling, "Programming
// the Hilbert curve" (AIP Conf. Proc. 707, 2004): the axes-to-transpose
// transform, then the bits of the transposed coordinates interleaved, ct
// first, most significant bit first; cubes are sorted by that index inside
// the power-of-two box that holds the grid.
#include <algorithm>
#include <utility>
#include <vector>

#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr int kSlotsPerBlock = 8;
constexpr int kSplit = kCube / kSlotsPerBlock;  // workgroups per cube
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

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
// true: tiled -> natural (padding slots skipped). order == nullptr: tiled
// position p holds row-major cube p; otherwise order[p] (clamped into range,
// so a bad table gives wrong rows but never an access out of bounds).
template <bool kInverse>
__global__ __launch_bounds__(kThreads) void tile_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int32_t* vbs_out,
    const int32_t* __restrict__ order, int T, int H, int W, int Nh, int Nw, int cpr) {
  const int pos = blockIdx.x / kSplit;
  const int part = blockIdx.x - pos * kSplit;
  const int n_cubes = gridDim.x / kSplit;
  const int c = order == nullptr ? pos : min(max(order[pos], 0), n_cubes - 1);
  const int b = blockIdx.y;
  const int cw = c % Nw;
  const int ch = (c / Nw) % Nh;
  const int ct = c / (Nw * Nh);
  const int eh = cube_extent(H, ch), ew = cube_extent(W, cw);
  const int n_real = cube_extent(T, ct) * eh * ew;
  if (!kInverse && vbs_out != nullptr && part == 0 && b == 0 && threadIdx.x == 0)
    vbs_out[pos] = n_real;

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const size_t n_nat = (size_t)T * H * W;
  const size_t n_tiled = (size_t)gridDim.x / kSplit * kCube;
#pragma unroll 1
  for (int r = 0; r < kSlotsPerBlock / 4; ++r) {
    const int u = part * kSlotsPerBlock + r * 4 + wave;
    const size_t tiled_row = (size_t)b * n_tiled + (size_t)pos * kCube + u;
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

// Hilbert index of X[0..2] (each < 2^bits, bits <= 21): axes to transpose,
// then interleave.
uint64_t hilbert3(uint32_t x0, uint32_t x1, uint32_t x2, int bits) {
  uint32_t X[3] = {x0, x1, x2};
  const uint32_t top = 1u << (bits - 1);
  for (uint32_t q = top; q > 1; q >>= 1) {  // undo excess work
    const uint32_t p = q - 1;
    for (int i = 0; i < 3; ++i) {
      if (X[i] & q) {
        X[0] ^= p;  // invert the low bits of X[0]
      } else {
        const uint32_t t = (X[0] ^ X[i]) & p;  // exchange low bits of X[0], X[i]
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  for (int i = 1; i < 3; ++i) X[i] ^= X[i - 1];  // Gray encode
  uint32_t t = 0;
  for (uint32_t q = top; q > 1; q >>= 1)
    if (X[2] & q) t ^= q - 1;
  for (int i = 0; i < 3; ++i) X[i] ^= t;
  uint64_t h = 0;
  for (int bit = bits - 1; bit >= 0; --bit)
    for (int i = 0; i < 3; ++i) h = (h << 1) | ((X[i] >> bit) & 1u);
  return h;
}

}  // namespace

bool cube_order(int T, int H, int W, int kind, int32_t* order) {
  const int Nt = (T + 3) / 4, Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  const int64_t nc = (int64_t)Nt * Nh * Nw;
  if (kind == 0) {
    for (int64_t c = 0; c < nc; ++c) order[c] = (int32_t)c;
    return true;
  }
  int bits = 1;
  while ((1 << bits) < std::max(Nt, std::max(Nh, Nw))) ++bits;
  if (bits > 21) return false;
  std::vector<std::pair<uint64_t, int32_t>> keyed((size_t)nc);
  for (int64_t c = 0; c < nc; ++c) {
    const int cw = (int)(c % Nw), ch = (int)((c / Nw) % Nh), ct = (int)(c / ((int64_t)Nw * Nh));
    keyed[(size_t)c] = {hilbert3((uint32_t)ct, (uint32_t)ch, (uint32_t)cw, bits), (int32_t)c};
  }
  std::sort(keyed.begin(), keyed.end());
  for (int64_t c = 0; c < nc; ++c) order[c] = keyed[(size_t)c].second;
  return true;
}

hipError_t launch_tile(const uint16_t* x, uint16_t* x_tiled, int32_t* vbs,
                       const int32_t* order, int B, int T, int H, int W, int NH, int D,
                       hipStream_t stream) {
  const int Nt = (T + 3) / 4, Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  const int cpr = NH * D * 2 / 16;
  dim3 grid(Nt * Nh * Nw * kSplit, B);
  hipLaunchKernelGGL(tile_kernel<false>, grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(x),
                     reinterpret_cast<u32x4*>(x_tiled), vbs, order, T, H, W, Nh, Nw, cpr);
  return hipGetLastError();
}

hipError_t launch_untile(const uint16_t* y_tiled, uint16_t* y, const int32_t* order, int B,
                         int T, int H, int W, int NH, int D, hipStream_t stream) {
  const int Nt = (T + 3) / 4, Nh = (H + 3) / 4, Nw = (W + 3) / 4;
  const int cpr = NH * D * 2 / 16;
  dim3 grid(Nt * Nh * Nw * kSplit, B);
  hipLaunchKernelGGL(tile_kernel<true>, grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(y_tiled),
                     reinterpret_cast<u32x4*>(y), nullptr, order, T, H, W, Nh, Nw, cpr);
  return hipGetLastError();
}

}  // namespace vsa
