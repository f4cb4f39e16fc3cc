// Coarse-stage output and the gated combine of the two stages.
//
// VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs, section "Two-Stage Architecture": the coarse stage works on
// mean-pooled cubes (the same pooling the selector uses) and the layer's output
// mixes the coarse-stage output with the fine-stage output through learnable
// gates; the comparison of VSA with Jenga in the same post lists that gate as a
// coarse/fine mix.
//
// Readings: the coarse output is dense attention of the pooled query cubes
// over the pooled key cubes, softmax(Qc Kc^T * sm_scale) Vc per (batch, head),
// over the key cubes that hold at least one real token; every token row of a
// cube receives its cube's row. The gates are caller-supplied tensors of the
// output's shape, applied elementwise.
//
// Kernels, after the selector's pool and score kernels (q and k) and one more
// pool over v:
//   coarse_attn_kernel  one workgroup per (16 query cubes, batch*head). Pass 1:
//                       each wave reduces the max and the exp-sum of 4 score
//                       rows. Pass 2: chunks of 256 key cubes; the workgroup
//                       writes the normalised weights of the chunk to LDS, then
//                       each lane (one channel d, a set of rows) accumulates
//                       w[r][j] * Vc[j][d] in fp32. Vc rows are read once per
//                       16 query cubes and are coalesced across lanes; the
//                       weight reads are wave-wide broadcasts. A tiny
//                       contraction (Nc^2 D per head), L2-resident.
//   combine_kernel      HBM-bound elementwise pass: one workgroup per token
//                       row, 16-byte vectors of o_fine and both gates; the
//                       cube's O_c row (fp32) is an L2 hit shared by 64 rows.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------- coarse attention

constexpr int kCoarseThreads = 256;  // 4 waves
constexpr int kCoarseRows = 16;      // query cubes per workgroup
constexpr int kChunk = kCoarseThreads;  // key cubes per LDS chunk

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// grid (ceil(Nc / 16), B*NH). s: unscaled scores [BH][Nc][Nc]; vc, oc:
// [BH][Nc][D] fp32. Rows past Nc (last workgroup) read row Nc-1 and are not
// written.
template <int D>
__global__ __launch_bounds__(kCoarseThreads) void coarse_attn_kernel(
    const float* __restrict__ s, const float* __restrict__ vc,
    const int32_t* __restrict__ vbs, float* __restrict__ oc, int Nc, float scale_log2) {
  constexpr int kGroups = kCoarseThreads / D;     // lanes sharing one channel d
  constexpr int kPerLane = kCoarseRows / kGroups;  // rows accumulated per lane
  __shared__ float w[kCoarseRows][kChunk];
  __shared__ float row_m[kCoarseRows], row_inv[kCoarseRows];

  const int bh = blockIdx.y, i0 = blockIdx.x * kCoarseRows;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const float* __restrict__ sb = s + (size_t)bh * Nc * Nc;

  // Pass 1: row max and sum of exp2((s - m) scale_log2) over real key cubes.
  constexpr int kRowsPerWave = kCoarseRows / (kCoarseThreads / 64);
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int r = wave * kRowsPerWave + rr;
    const float* __restrict__ srow = sb + (size_t)min(i0 + r, Nc - 1) * Nc;
    float m = -INFINITY;
    for (int j = lane; j < Nc; j += 64)
      if (vbs[j] > 0) m = fmaxf(m, srow[j]);
    m = wave_max(m);
    if (m == -INFINITY) m = 0.0f;  // no real key cube: every weight is 0
    float l = 0.0f;
    for (int j = lane; j < Nc; j += 64)
      if (vbs[j] > 0) l += __builtin_amdgcn_exp2f((srow[j] - m) * scale_log2);
    l = wave_sum(l);
    if (lane == 0) {
      row_m[r] = m;
      row_inv[r] = l > 0.0f ? 1.0f / l : 0.0f;
    }
  }
  __syncthreads();

  // Pass 2: o[r][d] = sum_j w[r][j] Vc[j][d].
  const int d = threadIdx.x % D, g = threadIdx.x / D;
  const float* __restrict__ vb = vc + (size_t)bh * Nc * D + d;
  float acc[kPerLane];
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) acc[e] = 0.0f;
  for (int j0 = 0; j0 < Nc; j0 += kChunk) {
    const int j = j0 + threadIdx.x;
    const bool real = j < Nc && vbs[j] > 0;
#pragma unroll 4
    for (int r = 0; r < kCoarseRows; ++r) {
      const float sv = real ? sb[(size_t)min(i0 + r, Nc - 1) * Nc + j] : 0.0f;
      w[r][threadIdx.x] =
          real ? __builtin_amdgcn_exp2f((sv - row_m[r]) * scale_log2) * row_inv[r] : 0.0f;
    }
    __syncthreads();
    const int n = min(kChunk, Nc - j0);
    int jj = 0;
    for (; jj + 8 <= n; jj += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = vb[(size_t)(j0 + jj + u) * D];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) acc[e] = fmaf(w[g + kGroups * e][jj + u], v[u], acc[e]);
    }
    for (; jj < n; ++jj) {
      const float v = vb[(size_t)(j0 + jj) * D];
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) acc[e] = fmaf(w[g + kGroups * e][jj], v, acc[e]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) {
    const int i = i0 + g + kGroups * e;
    if (i < Nc) oc[((size_t)bh * Nc + i) * D + d] = acc[e];
  }
}

// ---------------------------------------------------------------- gated combine

constexpr int kCombineThreads = 128;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// grid (B * Nc * 64 token rows). out may alias o_fine or a gate: every
// element is read and then written by the same lane. The sum is taken in
// fp32 as gc * oc + gf * of (one fma) and rounded to bf16 to nearest even.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const u32x4* o_fine, const float* __restrict__ oc, const u32x4* gate_c,
    const u32x4* gate_f, u32x4* out, int Nc, int NH) {
  const int row = blockIdx.x;  // b * Nc * 64 + token
  const int rows_per_b = Nc * kCube;
  const int b = row / rows_per_b, c = (row - b * rows_per_b) / kCube;
  const int cpr = NH * D / 8;  // 16-byte chunks per token row
  const size_t base = (size_t)row * cpr;
  for (int col = threadIdx.x; col < cpr; col += kCombineThreads) {
    const int h = col / (D / 8), d = (col % (D / 8)) * 8;
    const float* ocp = oc + (((size_t)b * NH + h) * Nc + c) * D + d;
    const floatx4 lo = *reinterpret_cast<const floatx4*>(ocp);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(ocp + 4);
    const float o8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const u32x4 f = o_fine[base + col], a = gate_c[base + col], z = gate_f[base + col];
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = fmaf(bf16_lo(a[e]), o8[2 * e], bf16_lo(z[e]) * bf16_lo(f[e]));
      const float x1 = fmaf(bf16_hi(a[e]), o8[2 * e + 1], bf16_hi(z[e]) * bf16_hi(f[e]));
      r[e] = pack_bf16x2(x0, x1);
    }
    out[base + col] = r;
  }
}

}  // namespace

size_t coarse_workspace_bytes(int B, int NH, int Nc, int D) {
  return select_workspace(B, NH, Nc, D).total +
         align_up((size_t)B * NH * Nc * D * sizeof(float));
}

hipError_t launch_coarse(const uint16_t* q_tiled, const uint16_t* k_tiled,
                         const uint16_t* v_tiled, const int32_t* vbs, int B, int Nc, int NH,
                         int D, int topk, int32_t* topk_idx, float scale, float* o_coarse,
                         void* workspace, hipStream_t stream) {
  const SelectWorkspace w = select_workspace(B, NH, Nc, D);
  char* ws = static_cast<char*>(workspace);
  const float* s = reinterpret_cast<const float*>(ws + w.s_off);
  float* vcp = reinterpret_cast<float*>(ws + w.total);

  hipError_t e = launch_pool_scores(q_tiled, k_tiled, vbs, B, Nc, NH, D, workspace, stream);
  if (e != hipSuccess) return e;
  if (topk_idx != nullptr) {
    e = launch_topk(s, B * NH, Nc, topk, topk_idx, nullptr, 0.0f, 0.0f, stream);
    if (e != hipSuccess) return e;
  }
  e = launch_pool(v_tiled, vbs, B, Nc, NH, D, vcp, stream);
  if (e != hipSuccess) return e;

  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((Nc + kCoarseRows - 1) / kCoarseRows, B * NH);
  if (D == 128)
    hipLaunchKernelGGL(coarse_attn_kernel<128>, grid, dim3(kCoarseThreads), 0, stream, s, vcp,
                       vbs, o_coarse, Nc, scale_log2);
  else
    hipLaunchKernelGGL(coarse_attn_kernel<64>, grid, dim3(kCoarseThreads), 0, stream, s, vcp,
                       vbs, o_coarse, Nc, scale_log2);
  return hipGetLastError();
}

hipError_t launch_gate_combine(const uint16_t* o_fine, const float* o_coarse,
                               const uint16_t* gate_c, const uint16_t* gate_f, uint16_t* out,
                               int B, int Nc, int NH, int D, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)B * Nc * kCube));
  auto cast = [](const uint16_t* p) { return reinterpret_cast<const u32x4*>(p); };
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kCombineThreads), 0, stream,
                       cast(o_fine), o_coarse, cast(gate_c), cast(gate_f),
                       reinterpret_cast<u32x4*>(out), Nc, NH);
  else
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kCombineThreads), 0, stream,
                       cast(o_fine), o_coarse, cast(gate_c), cast(gate_f),
                       reinterpret_cast<u32x4*>(out), Nc, NH);
  return hipGetLastError();
}

}  // namespace vsa
