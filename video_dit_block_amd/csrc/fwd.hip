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
//   cube's rows are fetched into registers (16-byte raw buffer loads) while
//   the MFMAs run on the current one: one LDS buffer, register double-
//   buffering. The buffer range covers only the cube's vbs[j] real rows, so
//   the padding rows read as zeros: pad values (even NaN) never reach an
//   MFMA, with no branch.
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
// * V is stored transposed in LDS (V^T, d-major, fp16), so the PV A operand
//   is two 8-byte LDS reads per lane. O^T accumulates in fp32, each lane holding
//   D/2 values of its own query row, so the online-softmax rescale is a
//   per-lane multiply.
// * fp32 online softmax in the exp2 domain: p = exp2(s * c - m * c) with
//   c = sm_scale * log2 e (one FMA per score), running reference max m,
//   running sum l. The reference max is raised lazily: only when a tile's
//   row max exceeds it by more than 2^8 (log2 units: 8) does the wave
//   rescale O and l by exp2((m_old - m_new) c); otherwise p may reach 2^8,
//   which fp32 and fp16 hold exactly in range. A fully masked row keeps
//   m = -inf and uses 0 in the subtraction, so no (-inf) - (-inf) arises.
//   Tokens >= vbs[j] are set to -inf in registers before the max (partial
//   cubes only).
// * A cube with vbs[j] <= 32 skips its second 32-token half entirely.
// * The unit's cube ids are sorted ascending in LDS first (the result is
//   independent of their order), so the query cubes resident on one XCD
//   sweep the key/value cubes of their head in the same order.
// * Precision: QK^T is a bf16 MFMA with fp32 accumulation. The PV product
//   runs as an fp16 MFMA (v_mfma_f32_32x32x16_f16): P is rounded to fp16 and
//   V is converted to fp16 while it is transposed into LDS. fp16 keeps 3 more
//   significand bits than bf16, which matters for rows with few keys; V is
//   converted exactly for |v| <= 65504 (bf16 values are a subset of fp16 in
//   that range) and saturates to 65504 beyond it. O / l is rounded to bf16
//   (nearest even) and stored.
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct FwdShape {
  static constexpr int kThreads = 128;              // 2 waves x 32 query rows
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kGroups = kThreads / kChunks;  // token groups per tile
  static constexpr int kTokPerThread = kCube / kGroups;  // rows each thread stages
  static constexpr int kKPitch = D + 8;             // LDS pitch of K rows (bf16)
  static constexpr int kVPitch = kCube + 4;         // LDS pitch of V^T rows (bf16)
  static constexpr int kQSteps = D / 16;            // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;           // 32-wide d blocks of O^T
  static_assert(kCube % kGroups == 0, "tile split");
};

// Largest index row sorted in LDS; longer rows are walked in the given order.
constexpr int kSortCap = 1024;
// Lazy rescale threshold (log2 units): the running reference max is only
// raised when a tile's max exceeds it by more than this, so unnormalised
// probabilities stay <= 2^8.
constexpr float kRescaleThreshold = 8.0f;
constexpr int kBufferDword3 = 0x00020000;  // gfx9 raw buffer resource flags

// Both halves of the wave: combines the value of lane l%32 with that of lane
// l%32+32 (v_permlane32_swap exchanges the halves of two registers).
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
  __shared__ int32_t order[kSortCap];

  const int unit = xcd_remap(blockIdx.x, n_units);
  const int qc = unit % Nq;
  const int bh = unit / Nq;
  const int h = bh % NH, b = bh / NH;
  const size_t row_stride = (size_t)NH * D;  // elements between tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qr = lane & 31, g = lane >> 5;

  // ---- this unit's cube ids, sorted ascending in LDS (the result does not
  // depend on the order; a common ascending sweep lets concurrently resident
  // query cubes of a head reuse the same key/value cubes from L2). Ids are
  // clamped into range: a violated precondition gives unspecified values,
  // never an out-of-bounds access.
  const int32_t* __restrict__ sel = topk_idx + (size_t)unit * topk;
  const bool sorted = topk <= kSortCap;
  if (sorted) {
    int n2 = 1;
    while (n2 < topk) n2 <<= 1;
    for (int i = tid; i < n2; i += S::kThreads)
      order[i] = i < topk ? min(max(sel[i], 0), Nkv - 1) : 0x7FFFFFFF;
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __syncthreads();
        for (int t = tid; t < (n2 >> 1); t += S::kThreads) {
          const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
          const int a = order[lo], c = order[hi];
          if (((lo & size) == 0) == (a > c)) {
            order[lo] = c;
            order[hi] = a;
          }
        }
      }
    __syncthreads();
  }
  auto cube_id = [&](int it) -> int {
    const int j = sorted ? order[it] : min(max(sel[it], 0), Nkv - 1);
    return __builtin_amdgcn_readfirstlane(j);
  };
  auto cube_len = [&](int j) -> int {
    return __builtin_amdgcn_readfirstlane(min(max(vbs[j], 0), kCube));
  };

  // ---- Q of this wave's 32 rows, in the B-operand layout of S^T = K Q^T:
  // lane (column qr, k-group g) holds q[row][16 s + 8 g .. + 7].
  bf16x8 qf[S::kQSteps];
  {
    const uint16_t* qrow =
        q + ((size_t)b * Nq * kCube + (size_t)qc * kCube + 32 * wave + qr) * row_stride +
        (size_t)h * D;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * g);
  }

  // ---- staging maps. K: chunk-fast (16 lanes cover one 256-byte row), so
  // both the global reads and the LDS row writes are contiguous. V: token-
  // group-fast, so the transposed LDS writes of consecutive lanes are
  // consecutive. Each thread stages kTokPerThread rows of one chunk.
  const int rs = NH * D;
  const int k_ch = tid % S::kChunks, k_tg = tid / S::kChunks;
  const int v_tg = tid % S::kGroups, v_ch = tid / S::kGroups;
  // byte offsets: < 64 * NH * D * 2 <= 2^32 (checked by the host), so u32
  const uint32_t rs2 = (uint32_t)rs * 2u;
  const uint32_t k_off = (uint32_t)(k_tg * S::kTokPerThread) * rs2 + 16u * k_ch;
  const uint32_t v_off = (uint32_t)(v_tg * S::kTokPerThread) * rs2 + 16u * v_ch;
  const size_t kv_batch = (size_t)b * Nkv * kCube;
  u32x4 kreg[S::kTokPerThread], vreg[S::kTokPerThread];

  // Raw buffer loads with the range limited to the cube's real rows: rows at
  // or beyond vbs[j] lie outside the range and read as zeros, so padding is
  // never read and staged as 0 without branches.
  auto fetch = [&](int j, int nv) {
    const size_t cube = (kv_batch + (size_t)j * kCube) * row_stride + (size_t)h * D;
    // wave-uniform by construction; readfirstlane keeps the descriptor scalar
    const int bytes = __builtin_amdgcn_readfirstlane((int)((uint32_t)nv * rs2));
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + cube), (short)0, bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + cube), (short)0, bytes, kBufferDword3);
#pragma unroll
    for (int i = 0; i < S::kTokPerThread; ++i) {
      kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + i * rs2, 0, 0));
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off + i * rs2, 0, 0));
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < S::kTokPerThread; ++i)
      *reinterpret_cast<u32x4*>(&ks[(k_tg * S::kTokPerThread + i) * S::kKPitch + 8 * k_ch]) = kreg[i];
    // V^T in fp16: for each of the chunk's 8 d values, the thread's
    // kTokPerThread consecutive tokens form one contiguous run of a V^T row.
    // bf16 -> f32 is exact (a shift or a mask); f32 -> f16 truncation is exact
    // for every bf16 value of magnitude <= 65504 (fp16 has the wider
    // significand) and saturates to the largest fp16 above that.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = &vt[(8 * v_ch + e) * S::kVPitch + v_tg * S::kTokPerThread];
      auto f32 = [&](int t) {
        const uint32_t w = vreg[t][e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
      };
#pragma unroll
      for (int i = 0; i < S::kTokPerThread / 4; ++i) {
        const u32x2 w = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f32(4 * i), f32(4 * i + 1))),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f32(4 * i + 2), f32(4 * i + 3)))};
        *reinterpret_cast<u32x2*>(dst + 4 * i) = w;
      }
    }
  };

  floatx16 oacc[S::kDBlocks];
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  // m_ref: reference max (raw score units) the probabilities are taken
  // against; l_run: running sum of exp2((s - m_ref) * scale_log2).
  float m_ref = kNegInf, l_run = 0.0f;

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

    // ---- S^T = K Q^T for the (one or two) 32-token halves; each chain
    // starts from an inline zero accumulator
    floatx16 sacc[2];
    const floatx16 zero16 = {};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt == 1 && !two) break;
      const uint16_t* krow = &ks[(32 * tt + qr) * S::kKPitch + 8 * g];
      sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(krow), qf[0], zero16, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < S::kQSteps; ++s)
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(krow + 16 * s), qf[s], sacc[tt], 0, 0, 0);
    }

    // ---- mask tokens >= vbs (partial cubes only), tile max
    if (nv_cur < kCube) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (tt == 1 && !two) break;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = 32 * tt + 8 * (r >> 2) + 4 * g + (r & 3);
          if (tok >= nv_cur) sacc[tt][r] = kNegInf;
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
    if (two) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
    }
    mx = halves_max(mx);

    // ---- lazy rescale: only when some row's max passes the reference by
    // more than the threshold (wave-uniform decision)
    if (__builtin_amdgcn_ballot_w64(mx * scale_log2 > m_ref * scale_log2 + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_ref == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float mc = m_ref == kNegInf ? 0.0f : m_ref * scale_log2;

    // P in fp16 (round to nearest even); the row sum adds the same rounded
    // values (v_dot2_f32_f16 against 1.0), so numerator and denominator agree
    float rs_sum = 0.0f;
    halfx8 pb[2][2];
    const halfx2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt == 1 && !two) break;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        floatx8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * kk + e], scale_log2, -mc));
        pb[tt][kk] = __builtin_convertvector(p, halfx8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const halfx2 pair = {pb[tt][kk][e], pb[tt][kk][e + 1]};
          rs_sum = __builtin_amdgcn_fdot2(pair, ones, rs_sum, false);
        }
      }
    }
    l_run += halves_sum(rs_sum);

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
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(halfx8, w), pb[tt][kk], oacc[db], 0, 0, 0);
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
