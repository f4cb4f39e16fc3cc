// Block mask -> lookup table compaction.
//
// VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs, section "Sparse Encoding in CK Tile": Jenga keeps a full M x M block
// relation matrix B and skips the cells with B[i][j] = 0, while VSA keeps only
// the selected key/value block ids plus a valid count per query block. This
// kernel turns the first encoding into the second, so that a mask (for
// instance a union of importance, condition and adjacency masks) can drive
// the LUT fine kernel.
//
// mask_to_lut_kernel: one wave per mask row. The wave reads 64 consecutive
// bytes per step (one per lane, coalesced), takes a ballot of the nonzero
// ones, and each set lane writes its id at (ids written so far) + (set lanes
// below it). Ids therefore come out in ascending order. Memory-bound: one
// byte read per cell, four bytes written per set cell.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kWavesPerBlock) void mask_to_lut_kernel(
    const uint8_t* __restrict__ mask, int64_t rows, int Nkv, int max_kv,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, int32_t* n_truncated) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / 64;
  if (row >= rows) return;
  const int lane = threadIdx.x % 64;
  const uint8_t* __restrict__ m = mask + row * Nkv;
  int32_t* __restrict__ out = idx + row * max_kv;
  const uint64_t below = (1ull << lane) - 1ull;
  int total = 0;
  for (int j0 = 0; j0 < Nkv; j0 += 64) {
    const int j = j0 + lane;
    const bool set = j < Nkv && m[j] != 0;
    const uint64_t bits = __ballot(set);
    const int pos = total + __popcll(bits & below);
    if (set && pos < max_kv) out[pos] = j;
    total += __popcll(bits);
  }
  if (lane == 0) {
    count[row] = min(total, max_kv);
    if (total > max_kv && n_truncated != nullptr) atomicAdd(n_truncated, 1);
  }
}

}  // namespace

hipError_t launch_mask_to_lut(const uint8_t* mask, int64_t rows, int Nkv, int max_kv,
                              int32_t* kv_block_idx, int32_t* valid_block_num,
                              int32_t* n_truncated, hipStream_t stream) {
  const int64_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(mask_to_lut_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, mask, rows, Nkv, max_kv, kv_block_idx, valid_block_num,
                     n_truncated);
  return hipGetLastError();
}

}  // namespace vsa
