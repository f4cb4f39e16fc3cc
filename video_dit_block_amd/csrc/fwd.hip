// Fine stage of Video Sparse Attention: non-causal block-sparse attention over
// the selected key/value cubes.
//
// Wan2.2 Production Values dataset card, section "Operator contract": for every
// (batch, head, query cube), out = softmax((q k_sel^T) / sqrt(D)) v_sel over the
// key/value cubes named by topk_idx, attending only the first vbs[c] tokens of
// cube c. VSA: Accelerating Video Diffusion Inference with Sparse Attention on
// AMD GPUs, sections "Two-Stage Architecture" (Stage 2: token-level attention
// only over the selected cubes), "Sparse Traversal" (the kernel walks the index
// list) and "Kernel Architecture" (QK GEMM with running max and sum, softmax,
// PV GEMM, accumulated over tiles).
//
// Design for gfx950
// -----------------
// * One workgroup = one (b, h, query cube): 64 query rows, 2 waves of 32 rows.
//   Work items are numbered head-major and remapped so each XCD walks a
//   contiguous range: concurrently resident query cubes are spatial
//   neighbours of one head and their selections overlap, so key/value cubes
//   are served from that XCD's L2.
// * Per selected cube, K (64 x D) and V (64 x D) are staged in LDS. The next
//   cube's rows are fetched into registers (16-byte global loads) while the
//   MFMAs run on the current one: one LDS buffer, register double-buffering.
//   Rows at or beyond vbs[j] are not read; zeros are staged instead, so pad
//   values (even NaN) never reach an MFMA.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the A operand is a K row slice read from LDS, the B operand is the wave's
//   Q held in registers for the whole loop. In the accumulator layout each
//   lane then holds 16 scores of ONE query row (row l%32; the other 16 of the
//   32-token tile sit in lane l^32), so the row max and row sum need one
//   cross-half swap (v_permlane32_swap) and the probabilities are already in
//   the B-operand layout of O^T = V^T P^T: they go from accumulator to MFMA
//   operand in registers. The contraction index of the PV product is
//   permuted to match the accumulator's token order (any fixed permutation
//   of a summation index leaves the sum unchanged).
// * V is stored transposed in LDS (V^T, d-major), so the PV A operand is two
//   8-byte LDS reads per lane. O^T accumulates in fp32, each lane holding
//   D/2 values of its own query row, so the online-softmax rescale is a
//   per-lane multiply.
// * fp32 online softmax in the exp2 domain: s * (sm_scale * log2 e), running
//   max m, running sum l, O rescaled by exp2(m_old - m_new). A fully masked
//   row keeps m = -inf; the subtraction then uses 0 so no (-inf) - (-inf)
//   arises. Tokens >= vbs[j] are set to -inf in registers before the max.
// * A cube with vbs[j] <= 32 skips its second 32-token half entirely.
// * Output: P is rounded to bf16 for the PV MFMA; O / l is rounded to bf16
//   (nearest even) and stored.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct FwdShape {
  static constexpr int kThreads = 128;              // 2 waves x 32 query rows
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kGroups = kThreads / kChunks;  // token groups per tile
  static constexpr int kTokPerThread = kCube / kGroups;  // rows each thread stages
  static constexpr int kKPitch = D + 8;             // LDS pitch of K rows (bf16)
  static constexpr int kVPitch = kCube + 8;         // LDS pitch of V^T rows (bf16)
  static constexpr int kQSteps = D / 16;            // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;           // 32-wide d blocks of O^T
  static_assert(kCube % kGroups == 0, "tile split");
};

// Both halves of the wave: returns {value of lane l%32, value of lane l%32+32}
// in an order that does not matter to the callers (they combine them
// symmetrically).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

template <int D>
__global__ __launch_bounds__(FwdShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ vbs, uint16_t* __restrict__ out, int Nq,
    int Nkv, int NH, int topk, float scale_log2, int n_units) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[kCube * S::kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * S::kVPitch];

  const int unit = xcd_remap(blockIdx.x, n_units);
  const int qc = unit % Nq;
  const int bh = unit / Nq;
  const int h = bh % NH, b = bh / NH;
  const size_t row_stride = (size_t)NH * D;  // elements between tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qr = lane & 31, g = lane >> 5;

  // ---- Q of this wave's 32 rows, in the B-operand layout of S^T = K Q^T:
  // lane (column qr, k-group g) holds q[row][16 ks + 8 g .. + 7].
  bf16x8 qf[S::kQSteps];
  {
    const uint16_t* qrow =
        q + ((size_t)b * Nq * kCube + (size_t)qc * kCube + 32 * wave + qr) * row_stride +
        (size_t)h * D;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * g);
  }

  // ---- staging map: thread stages chunk `ch` of tokens tg*kTokPerThread + i
  const int ch = tid % S::kChunks;
  const int tg = tid / S::kChunks;
  const size_t kv_batch = (size_t)b * Nkv * kCube;
  u32x4 kreg[S::kTokPerThread], vreg[S::kTokPerThread];

  // Per-thread part of the staging offsets (32-bit: one cube's rows span
  // 64 * NH * D elements); the per-cube base pointer is wave-uniform.
  const int rs = NH * D;
  const int toff = tg * S::kTokPerThread * rs + 8 * ch;
  auto fetch = [&](int j, int nv) {
    const size_t cube = (kv_batch + (size_t)j * kCube) * row_stride + (size_t)h * D;
    const uint16_t* kb = k + cube;
    const uint16_t* vb = v + cube;
#pragma unroll
    for (int i = 0; i < S::kTokPerThread; ++i) {
      const int tok = tg * S::kTokPerThread + i;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = z;
      vreg[i] = z;
      if (tok < nv) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kb + (toff + i * rs));
        vreg[i] = *reinterpret_cast<const u32x4*>(vb + (toff + i * rs));
      }
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < S::kTokPerThread; ++i) {
      const int tok = tg * S::kTokPerThread + i;
      *reinterpret_cast<u32x4*>(&ks[tok * S::kKPitch + 8 * ch]) = kreg[i];
    }
    // V^T: for each of the chunk's 8 d values, the thread's kTokPerThread
    // consecutive tokens form one contiguous run of a V^T row.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint32_t packed[S::kTokPerThread / 2];
#pragma unroll
      for (int i = 0; i < S::kTokPerThread / 2; ++i)
        packed[i] = __builtin_amdgcn_perm(vreg[2 * i + 1][e >> 1], vreg[2 * i][e >> 1], sel);
      uint16_t* dst = &vt[(8 * ch + e) * S::kVPitch + tg * S::kTokPerThread];
      if constexpr (S::kTokPerThread == 8) {
        const u32x4 w = {packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4*>(dst) = w;
      } else {
        const u32x2 w = {packed[0], packed[1]};
        *reinterpret_cast<u32x2*>(dst) = w;
      }
    }
  };

  floatx16 oacc[S::kDBlocks];
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;

  // Ids and counts are clamped into range: a violated precondition gives
  // unspecified values, never an out-of-bounds access.
  const int32_t* __restrict__ sel = topk_idx + (size_t)unit * topk;
  auto cube_id = [&](int it) { return min(max(sel[it], 0), Nkv - 1); };
  auto cube_len = [&](int jj) { return min(max(vbs[jj], 0), kCube); };
  int j = cube_id(0);
  int nv = cube_len(j);
  fetch(j, nv);

#pragma unroll 1
  for (int it = 0; it < topk; ++it) {
    const int nv_cur = nv;
    __syncthreads();  // every wave is done reading the previous tile
    stage();
    __syncthreads();
    if (it + 1 < topk) {
      j = cube_id(it + 1);
      nv = cube_len(j);
      fetch(j, nv);  // in flight during the MFMAs below
    }
    const bool two = nv_cur > 32;

    // ---- S^T = K Q^T for the (one or two) 32-token halves
    floatx16 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[tt][r] = 0.0f;
      if (tt == 1 && !two) break;
#pragma unroll
      for (int s = 0; s < S::kQSteps; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &ks[(32 * tt + qr) * S::kKPitch + 16 * s + 8 * g]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[tt], 0, 0, 0);
      }
    }

    // ---- mask, scale, running max
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = 32 * tt + 8 * (r >> 2) + 4 * g + (r & 3);
        const float x = tok < nv_cur ? sacc[tt][r] * scale_log2 : kNegInf;
        sacc[tt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float rs = 0.0f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        floatx8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(sacc[tt][8 * kk + e] - m_use);
          rs += p[e];
        }
        pb[tt][kk] = __builtin_convertvector(p, bf16x8);
      }
    rs = halves_sum(rs);
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // ---- O^T += V^T P^T; the k-slots of lane group g are tokens
    // base+4g+{0..3} and base+8+4g+{0..3}, matching the accumulator layout.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt == 1 && !two) break;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int base = 32 * tt + 16 * kk + 4 * g;
#pragma unroll
        for (int db = 0; db < S::kDBlocks; ++db) {
          const uint16_t* src = &vt[(32 * db + qr) * S::kVPitch + base];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
          const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, w), pb[tt][kk], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: lane holds O^T[d][row] for d = 32 db + 8 (r/4) + 4 g + r%4
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  uint16_t* orow =
      out + ((size_t)b * Nq * kCube + (size_t)qc * kCube + 32 * wave + qr) * row_stride +
      (size_t)h * D;
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x2 w = {pack_bf16x2(oacc[db][4 * r4] * inv_l, oacc[db][4 * r4 + 1] * inv_l),
                       pack_bf16x2(oacc[db][4 * r4 + 2] * inv_l, oacc[db][4 * r4 + 3] * inv_l)};
      *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * g) = w;
    }
}

}  // namespace

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* vbs, uint16_t* out,
                      int B, int Nq, int Nkv, int NH, int D, int topk,
                      float sm_scale, hipStream_t stream) {
  const int n_units = B * NH * Nq;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  if (D == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(n_units), dim3(FwdShape<128>::kThreads), 0,
                       stream, q, k, v, topk_idx, vbs, out, Nq, Nkv, NH, topk,
                       scale_log2, n_units);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(n_units), dim3(FwdShape<64>::kThreads), 0,
                       stream, q, k, v, topk_idx, vbs, out, Nq, Nkv, NH, topk,
                       scale_log2, n_units);
  return hipGetLastError();
}

}  // namespace vsa
