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
//   coarse_attn_kernel  one workgroup per (32 query cubes, batch*head). Pass 1:
//                       the row maxima (loads for 8 rows in flight together,
//                       DPP wave reductions). Pass 2, chunks of 64 key cubes:
//                       the workgroup stages the chunk's Vc rows and weights in
//                       LDS, and the 4 waves multiply them on fp32 MFMA
//                       (v_mfma_f32_16x16x4_f32), each a 16-row x D/2 block;
//                       the row sums are reduced once at the end.
//                       A small contraction (2 Nc^2 D FLOP per head) on
//                       L2-resident data.
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
constexpr int kCoarseRows = 32;      // query cubes per workgroup
constexpr int kCoarseKeys = 64;      // key cubes per LDS chunk

// Wave-wide reductions on DPP lane moves (no LDS round trips): within each
// row of 16 lanes by quad permutes and mirrors, then across rows by the row
// broadcasts; lane 63 ends with the result, which is read back uniformly.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp(float x, float identity) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                               __builtin_bit_cast(int, x), kCtrl,
                                                               kRowMask, 0xF, false));
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float x, float identity, Op op) {
  x = op(x, dpp<0xB1, 0xF>(x, identity));   // quad_perm [1,0,3,2]
  x = op(x, dpp<0x4E, 0xF>(x, identity));   // quad_perm [2,3,0,1]
  x = op(x, dpp<0x141, 0xF>(x, identity));  // row_half_mirror
  x = op(x, dpp<0x140, 0xF>(x, identity));  // row_mirror
  x = op(x, dpp<0x142, 0xA>(x, identity));  // row_bcast:15 into rows 1, 3
  x = op(x, dpp<0x143, 0xC>(x, identity));  // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, 0.0f, [](float a, float b) { return a + b; });
}

// grid (ceil(Nc / 32), B*NH). s: unscaled scores [BH][Nc][Nc]; vc, oc:
// [BH][Nc][D] fp32. Rows past Nc (last workgroup) read row Nc-1 and are not
// written.
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// receives D[4(l/16) + r][l%16], r = 0..3. A = the weights of 16 query rows
// at 4 keys, B = Vc of those 4 keys at 16 channels. Wave w owns query rows
// 16 (w % 2) .. + 15 and channels (w / 2) D/2 .. + D/2 - 1 of the tile.
template <int D>
__global__ __launch_bounds__(kCoarseThreads) __attribute__((amdgpu_waves_per_eu(3))) void coarse_attn_kernel(
    const float* __restrict__ s, const float* __restrict__ vc,
    const int32_t* __restrict__ vbs, float* __restrict__ oc, int Nc, float scale_log2) {
  constexpr int kVStride = D + 16;           // floats per staged Vc row (spreads banks)
  constexpr int kPStride = kCoarseKeys + 4;  // floats per staged weight row
  constexpr int kCols = D / 2;               // channels per wave
  constexpr int kBlocks = kCols / 16;        // 16-wide channel blocks per wave
  __shared__ __attribute__((aligned(16))) float vs[kCoarseKeys * kVStride];
  __shared__ float ps[kCoarseRows * kPStride];
  __shared__ float row_m[kCoarseRows], row_l[kCoarseRows];

  const int bh = blockIdx.y, i0 = blockIdx.x * kCoarseRows;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const float* __restrict__ sb = s + (size_t)bh * Nc * Nc;
  const float* __restrict__ vb = vc + (size_t)bh * Nc * D;

  constexpr int kRowsPerWave = kCoarseRows / (kCoarseThreads / 64);  // row r: wave r % 4

  // Pass 1: each row's max over its real key cubes. Lanes hold 4 keys of each
  // of the wave's 8 rows per step, all 36 loads (with vbs) in flight at once.
  {
    float mx[kRowsPerWave];
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) mx[q] = -INFINITY;
    for (int jb = 0; jb < Nc; jb += 4 * 64) {
      bool real[4];
      float v[kRowsPerWave][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + 64 * u + lane, jc = min(j, Nc - 1);
        real[u] = j < Nc && vbs[jc] > 0;
#pragma unroll
        for (int q = 0; q < kRowsPerWave; ++q)
          v[q][u] = sb[(size_t)min(i0 + wave + 4 * q, Nc - 1) * Nc + jc];
      }
#pragma unroll
      for (int q = 0; q < kRowsPerWave; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) mx[q] = real[u] ? fmaxf(mx[q], v[q][u]) : mx[q];
    }
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
      const float m = wave_max(mx[q]);
      if (lane == 0) row_m[wave + 4 * q] = m > -INFINITY ? m : 0.0f;  // no real key: weights 0
    }
  }
  __syncthreads();

  // Pass 2: keys 64 at a time. The chunk's Vc rows and weights
  // exp2((s - m) scale_log2) are staged in LDS (the wave that owns a row
  // holds its 64 scores of the chunk, one per lane, and keeps a per-lane
  // partial of the row's sum l); the 4 waves multiply weights by Vc on fp32
  // MFMA. The next chunk's global loads are issued before this chunk's MFMAs.
  // O = acc / l at the end.
  constexpr int kVIters = kCoarseKeys * D / 4 / kCoarseThreads;  // float4 per lane
  const int rq = 16 * (wave & 1), c0 = (wave >> 1) * kCols;
  const int lr = lane % 16, lk = lane / 16;
  floatx4 acc[kBlocks];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) acc[cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float mrow[kRowsPerWave], lpart[kRowsPerWave];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
    mrow[q] = row_m[wave + 4 * q];
    lpart[q] = 0.0f;
  }
  floatx4 vreg[kVIters];
  float sreg[kRowsPerWave];
  // indices are clamped into range; out-of-range Vc rows become 0 and
  // out-of-range or non-real scores -inf
  auto load_chunk = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kVIters; ++it) {
      const int e = tid + kCoarseThreads * it;
      const int key = e / (D / 4), c4 = e - key * (D / 4);
      vreg[it] = *reinterpret_cast<const floatx4*>(vb + (size_t)min(j0 + key, Nc - 1) * D + 4 * c4);
      if (j0 + key >= Nc) vreg[it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int j = min(j0 + lane, Nc - 1);
    const bool real = j0 + lane < Nc && vbs[j] > 0;
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
      const float sv = sb[(size_t)min(i0 + wave + 4 * q, Nc - 1) * Nc + j];
      sreg[q] = real ? sv : -INFINITY;
    }
  };
  load_chunk(0);
  for (int j0 = 0; j0 < Nc; j0 += kCoarseKeys) {
#pragma unroll
    for (int it = 0; it < kVIters; ++it) {
      const int e = tid + kCoarseThreads * it;
      const int key = e / (D / 4), c4 = e - key * (D / 4);
      *reinterpret_cast<floatx4*>(&vs[key * kVStride + 4 * c4]) = vreg[it];
    }
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
      const float w = sreg[q] > -INFINITY ? __builtin_amdgcn_exp2f((sreg[q] - mrow[q]) * scale_log2)
                                          : 0.0f;
      ps[(wave + 4 * q) * kPStride + lane] = w;
      lpart[q] += w;
    }
    __syncthreads();
    if (j0 + kCoarseKeys < Nc) load_chunk(j0 + kCoarseKeys);
    // operands of 8 key steps are read ahead of their MFMAs
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      constexpr int kSteps = kCoarseKeys / 8;
      float a[kSteps], b[kSteps][kBlocks];
#pragma unroll
      for (int t = 0; t < kSteps; ++t) {
        const int ks = half * kSteps + t;
        a[t] = ps[(rq + lr) * kPStride + 4 * ks + lk];
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb) b[t][cb] = vs[(4 * ks + lk) * kVStride + c0 + 16 * cb + lr];
      }
#pragma unroll
      for (int t = 0; t < kSteps; ++t)
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t][cb], acc[cb], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
    const float l = wave_sum(lpart[q]);
    if (lane == 0) row_l[wave + 4 * q] = l;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = row_l[rq + 4 * lk + r];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // no real key cube: the row is 0
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb) acc[cb][r] *= inv;
  }
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + rq + 4 * lk + r;
      if (i < Nc) oc[((size_t)bh * Nc + i) * D + c0 + 16 * cb + lr] = acc[cb][r];
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
  // kBatch chunks per lane are loaded before any is stored (out may alias an
  // input, so loads cannot be moved above earlier stores by the compiler);
  // this keeps 3 x kBatch 16-byte loads in flight per lane
  constexpr int kBatch = 4;
  for (int col0 = threadIdx.x; col0 < cpr; col0 += kBatch * kCombineThreads) {
    u32x4 f[kBatch], a[kBatch], z[kBatch];
    floatx4 lo[kBatch], hi[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int col = min(col0 + i * kCombineThreads, cpr - 1);
      const int h = col / (D / 8), d = (col % (D / 8)) * 8;
      const float* ocp = oc + (((size_t)b * NH + h) * Nc + c) * D + d;
      lo[i] = *reinterpret_cast<const floatx4*>(ocp);
      hi[i] = *reinterpret_cast<const floatx4*>(ocp + 4);
      f[i] = o_fine[base + col];
      a[i] = gate_c[base + col];
      z[i] = gate_f[base + col];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int col = col0 + i * kCombineThreads;
      if (col >= cpr) break;
      const float o8[8] = {lo[i][0], lo[i][1], lo[i][2], lo[i][3],
                           hi[i][0], hi[i][1], hi[i][2], hi[i][3]};
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = fmaf(bf16_lo(a[i][e]), o8[2 * e], bf16_lo(z[i][e]) * bf16_lo(f[i][e]));
        const float x1 = fmaf(bf16_hi(a[i][e]), o8[2 * e + 1], bf16_hi(z[i][e]) * bf16_hi(f[i][e]));
        r[e] = pack_bf16x2(x0, x1);
      }
      out[base + col] = r;
    }
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
