// Device-side check of the fine stage's index precondition.
//
// VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs, section "Block-Sparse Encoding": the index list names, for each query
// block, the selected key/value blocks; an id outside [0, Nkv) or named twice
// in one row breaks that encoding. One wave per row marks ids in an LDS bitmap
// and counts the offending entries; one atomic add per row reports them.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr int kValidateThreads = 64;
constexpr int kMaxWords = 8192 / 32;  // VSA_MAX_CUBES bits

__global__ __launch_bounds__(kValidateThreads) void validate_kernel(
    const int32_t* __restrict__ topk_idx, int Nkv, int topk,
    int32_t* __restrict__ bad_count) {
  __shared__ uint32_t seen[kMaxWords];
  const int words = (Nkv + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kValidateThreads) seen[w] = 0u;
  __syncthreads();
  const int32_t* row = topk_idx + (size_t)blockIdx.x * topk;
  int bad = 0;
  for (int t = threadIdx.x; t < topk; t += kValidateThreads) {
    const int id = row[t];
    if (id < 0 || id >= Nkv) {
      ++bad;
    } else {
      const uint32_t bit = 1u << (id & 31);
      if (atomicOr(&seen[id >> 5], bit) & bit) ++bad;
    }
  }
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  if (threadIdx.x == 0 && bad > 0) atomicAdd(bad_count, bad);
}

}  // namespace

hipError_t launch_validate_topk(const int32_t* topk_idx, int B, int NH, int Nq,
                                int Nkv, int topk, int32_t* bad_count,
                                hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(B * NH * Nq), dim3(kValidateThreads), 0,
                     stream, topk_idx, Nkv, topk, bad_count);
  return hipGetLastError();
}

}  // namespace vsa
