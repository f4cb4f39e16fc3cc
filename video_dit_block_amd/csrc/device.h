// Internal device helpers shared by the libvsa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

constexpr int kCube = 64;   // tokens per 4x4x4 cube
constexpr int kEdge = 4;    // cube edge
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, each with its own L2

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Workgroups are handed to the XCDs round-robin (workgroup id i runs on XCD
// i % 8). Map the hardware id to a logical work index so that each XCD walks a
// contiguous range of the logical index space: neighbouring work items, which
// read overlapping data, then share one L2. Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n / kNumXcd, r = n % kNumXcd;
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  return x * q + (x < r ? x : r) + i;
}

// Clipped extent of cube i along an axis of n tokens.
__device__ __forceinline__ int cube_extent(int n, int i) {
  const int e = n - kEdge * i;
  return e < kEdge ? e : kEdge;
}

// Natural token index of slot u (< et*eh*ew) of cube (ct, ch, cw): real tokens
// fill the cube row-major over its clipped extent.
__device__ __forceinline__ int slot_token(int u, int ct, int ch, int cw, int eh,
                                          int ew, int H, int W) {
  const int ehw = eh * ew;
  const int dt = u / ehw;
  const int rem = u - dt * ehw;
  const int dh = rem / ew;
  const int dw = rem - dh * ew;
  return ((kEdge * ct + dt) * H + kEdge * ch + dh) * W + kEdge * cw + dw;
}

}  // namespace vsa
