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
// * Per selected cube, K (64 x D, bf16) and V (64 x D, fp16 copy made by a
//   pre-pass) are staged in LDS, one buffer each, loaded global -> LDS
//   directly (buffer_load ... lds). The two tensors form a two-stage
//   pipeline: V of cube j streams in while QK^T of cube j runs, K of cube
//   j+1 while PV of cube j runs, each tile's DMAs spread one per MFMA step.
//   The buffer range covers only the cube's vbs[j] real rows, so the padding
//   rows land as zeros: pad values (even NaN) never reach an MFMA, with no
//   branch.
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
// * V is stored row-major in LDS; the PV A operand (V^T) comes from two
//   transposing 8-byte LDS reads per lane (ds_read_b64_tr_b16). O^T
//   accumulates in fp32, each lane holding D/2 values of its own query row,
//   so the online-softmax rescale is a per-lane multiply.
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
//   V is converted to fp16 by the pre-pass. fp16 keeps 3 more
//   significand bits than bf16, which matters for rows with few keys; V is
//   converted exactly for |v| <= 65504 (bf16 values are a subset of fp16 in
//   that range) and saturates to 65504 beyond it. O / l is rounded to bf16
//   (nearest even) and stored.
#include <type_traits>

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
  static constexpr int kThreads = 128;                 // 2 waves x 32 query rows
  static constexpr int kRowBytes = 2 * D;              // one (token, head) row
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;  // rows one wave-wide DMA fills
  static constexpr int kLoadsPerWave = kCube * kRowBytes / 1024 / 2;  // per tile, per wave
  static constexpr int kQSteps = D / 16;               // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;              // 32-wide d blocks of O^T
  // one tile DMA per QK k-step and per PV (16-token half, d-block) step
  static_assert(kQSteps == kLoadsPerWave && 2 * kDBlocks == kLoadsPerWave, "DMA spread");
};

// XOR swizzles of the 16-byte chunk index inside an LDS row: chunk c of row r
// lives in slot c ^ swz(r). Chosen (by an exhaustive search over linear maps
// of the row's low 4 bits, with a 32- and a 64-bank model) so that the two
// read patterns below are free of bank conflicts:
//   K: 32 lanes read chunk c of rows r..r+31 (ds_read_b128);
//   V: the transposing read, 16-lane groups reading 8 bytes of 4
//      consecutive rows at 4 column blocks (ds_read_b64_tr_b16).
template <int D> __device__ __forceinline__ int swz_k(int r);
template <int D> __device__ __forceinline__ int swz_v(int r);
template <> __device__ __forceinline__ int swz_k<128>(int r) { return r & 15; }
template <> __device__ __forceinline__ int swz_v<128>(int r) {
  return ((r & 1) ? 10 : 0) ^ ((r & 2) ? 4 : 0);
}
template <> __device__ __forceinline__ int swz_k<64>(int r) {
  return ((r & 1) ? 1 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 2 : 0) ^ ((r & 8) ? 1 : 0);
}
template <> __device__ __forceinline__ int swz_v<64>(int r) {
  return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0);
}

// Largest index row sorted in LDS; longer rows are walked in the given order.
constexpr int kSortCap = 1024;
// Lazy rescale threshold (log2 units): the running reference max is only
// raised when a tile's max exceeds it by more than this, so unnormalised
// probabilities stay <= 2^8.
constexpr float kRescaleThreshold = 8.0f;
constexpr int kBufferDword3 = 0x00020000;  // gfx9 raw buffer resource flags

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef int32_t int32x4_t __attribute__((ext_vector_type(4)));

// One wave-wide 16-byte-per-lane global -> LDS load (buffer_load_dwordx4 ...
// lds): lane L's 16 bytes land at LDS byte lds_addr + 16 L. Issued as inline
// assembly so that the compiler does not guard every later LDS read with a
// wait for all outstanding loads; the kernel waits explicitly (wait_vmcnt)
// before the barrier that publishes a tile. M0 carries the LDS base; the
// s_nop covers the M0 -> LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used nowhere else
__device__ __forceinline__ void dma16(int32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// gfx9 raw buffer resource: base address, stride 0, num_records bytes.
__device__ __forceinline__ int32x4_t buffer_rsrc(const void* base, int num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = kBufferDword3;
  return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(size_t)(lds_void_ptr)(p);
}
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_t* lds_fp16x4_ptr;

// s_waitcnt with vmcnt <= n and the other counters unconstrained (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

// ---------------------------------------------------------------------------
// V -> fp16 pre-pass. Writes an fp16 copy of v (same tiled BSHD layout) into
// the workspace: real rows converted, padding rows zeroed. bf16 -> f32 is
// exact (the bf16 bits are the upper half of an f32); f32 -> f16 truncation
// is exact for |v| <= 65504, since every such bf16 value is an fp16 value,
// and saturates to 65504 beyond. HBM-bound: one read and one write of v.
constexpr int kCvtThreads = 256;
constexpr int kCvtSplit = 4;  // workgroups per cube (16 slots each)

__global__ __launch_bounds__(kCvtThreads) void v_to_fp16_kernel(
    const u32x4* __restrict__ v, u32x4* __restrict__ v16, const int32_t* __restrict__ vbs,
    int Nkv, int cpr) {
  const int c = blockIdx.x / kCvtSplit, part = blockIdx.x % kCvtSplit, b = blockIdx.y;
  const int nv = min(max(vbs[c], 0), kCube);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
#pragma unroll 1
  for (int r = 0; r < kCube / kCvtSplit / 4; ++r) {
    const int u = part * (kCube / kCvtSplit) + r * 4 + wave;
    const size_t row = ((size_t)b * Nkv + c) * kCube + u;
    const u32x4* __restrict__ src = v + row * cpr;
    u32x4* __restrict__ dst = v16 + row * cpr;
    if (u < nv) {
      for (int col = lane; col < cpr; col += 64) {
        const u32x4 w = src[col];
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                                   __uint_as_float(w[e] << 16),
                                                   __uint_as_float(w[e] & 0xFFFF0000u)));
        dst[col] = o;
      }
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int col = lane; col < cpr; col += 64) dst[col] = z;
    }
  }
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(FwdShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v16, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ vbs, uint16_t* __restrict__ out, int Nq,
    int Nkv, int NH, int topk, float scale_log2, int n_units) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t ksm[kCube * S::kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vsm[kCube * S::kRowBytes];
  __shared__ int32_t order[kSortCap];

  const int unit = xcd_remap(blockIdx.x, n_units);
  const int qc = unit % Nq;
  const int bh = unit / Nq;
  const int h = bh % NH, b = bh / NH;
  const size_t row_stride = (size_t)NH * D;  // elements between tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qr = lane & 31, g = lane >> 5;

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

  // ---- K and V tiles go global -> LDS directly (buffer_load ... lds): each
  // wave-wide load fills 1 KiB of LDS, lane L writing bytes [16 L, 16 L + 16).
  // The lane fetches the global chunk that the swizzle places in that slot.
  // The buffer range ends at the cube's vbs[j] real rows, so padding rows land
  // in LDS as zeros. Byte offsets are < 64 * NH * D * 2 <= 2^32 (host-checked).
  const uint32_t rs2 = (uint32_t)NH * D * 2u;
  uint32_t koff[S::kLoadsPerWave], voff[S::kLoadsPerWave];
#pragma unroll
  for (int n = 0; n < S::kLoadsPerWave; ++n) {
    const int row = (wave * S::kLoadsPerWave + n) * S::kRowsPerKiB + lane / S::kChunks;
    const int slot = lane % S::kChunks;
    koff[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_k<D>(row));
    voff[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_v<D>(row));
  }
  const size_t kv_batch = (size_t)b * Nkv * kCube;
  // Buffer resource and LDS base of one tile load; the kLoadsPerWave DMAs of
  // a tile are spread over the MFMA loop that runs while the tile is in
  // flight (one DMA after each MFMA step), so that no wave issues a burst of
  // loads and stalls behind a full memory pipeline.
  const uint32_t lds_wave = (uint32_t)(wave * S::kLoadsPerWave) * 1024u;
  auto tile_rsrc = [&](const uint16_t* base, int j, int nv) -> int32x4_t {
    const size_t cube = (kv_batch + (size_t)j * kCube) * row_stride + (size_t)h * D;
    return buffer_rsrc(base + cube, (int)((uint32_t)nv * rs2));
  };

  floatx16 oacc[S::kDBlocks];
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  // m_ref: reference max (raw score units) the probabilities are taken
  // against; l_run: running sum of exp2((s - m_ref) * scale_log2).
  float m_ref = kNegInf, l_run = 0.0f;
  const floatx16 zero16 = {};
  const halfx2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // The Q loads (issued before the index sort) must be complete here, so that
  // inside the loop the only outstanding vector-memory operations are the
  // K/V tile loads that the explicit waits below account for.
  //
  // Pipeline of one cube: K(it) landed -> barrier -> QK(it), with V(it)'s
  // DMAs issued between its MFMAs (the V buffer is free: every wave passed
  // the barrier after PV(it-1)) -> barrier -> softmax -> V(it) landed ->
  // barrier -> PV(it), with K(it+1)'s DMAs issued between its MFMAs (the K
  // buffer is free: every wave passed the barrier after QK(it)). At each
  // wait the tile about to be read is the only load in flight.
  wait_vmcnt<0>();
  int j = cube_id(0);
  int nv = cube_len(j);
  {
    const int32x4_t rsrc = tile_rsrc(k, j, nv);
    const uint32_t lds0 = lds_address(ksm) + lds_wave;
#pragma unroll
    for (int n = 0; n < S::kLoadsPerWave; ++n) dma16(rsrc, koff[n], lds0 + 1024u * n);
  }

#pragma unroll 1
  for (int it = 0; it < topk; ++it) {
    const int nv_cur = nv;
    const int j_cur = j;
    const bool more = it + 1 < topk;
    if (more) {
      j = cube_id(it + 1);
      nv = cube_len(j);
    }
    const bool two = nv_cur > 32;

    // ---- K of this cube has landed (this wave's loads), then every wave's
    // loads are visible
    wait_vmcnt<0>();
    __syncthreads();
    const int32x4_t vrsrc = tile_rsrc(v16, j_cur, nv_cur);
    const uint32_t vlds0 = lds_address(vsm) + lds_wave;

    // ---- S^T = K Q^T, one MFMA chain per 32-token half (the second half only
    // when the cube has more than 32 real tokens). The K operands are read
    // from LDS two k-steps ahead of the MFMAs that consume them. Each chain
    // starts from an inline zero accumulator. Keeping the second half an
    // additive block (rather than a second copy of the whole computation)
    // keeps the accumulators in the same registers on both paths.
    floatx16 sacc[2];
    auto qk_half = [&](int tt) {
      const uint8_t* krow = ksm + (32 * tt + qr) * S::kRowBytes;
      const int ksw = swz_k<D>(32 * tt + qr);
      bf16x8 a[3];
      auto rd = [&](int st) {
        a[st % 3] = *reinterpret_cast<const bf16x8*>(krow + 16 * ((2 * st + g) ^ ksw));
      };
      rd(0);
      rd(1);
#pragma unroll
      for (int st = 0; st < S::kQSteps; ++st) {
        if (st + 2 < S::kQSteps) rd(st + 2);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st % 3], qf[st],
                                                            st == 0 ? zero16 : sacc[tt], 0, 0, 0);
        if (tt == 0) dma16(vrsrc, voff[st], vlds0 + 1024u * st);  // kQSteps == kLoadsPerWave
      }
    };
    qk_half(0);
    if (two) qk_half(1);
    __syncthreads();  // every wave is done reading K
    const int32x4_t krsrc = tile_rsrc(k, j, nv);
    const uint32_t klds0 = lds_address(ksm) + lds_wave;

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

    // ---- V of this cube has landed, then every wave's loads are visible
    wait_vmcnt<0>();
    __syncthreads();

    // ---- O^T += V^T P^T. The A operand comes from the transposing read: in
    // each 16-lane group, lane i receives element i%4 of the 8 bytes that
    // lane 4e + i/4 addressed, for e = 0..3. Lane (group G, s) addresses row
    // base + 4(G/2) + s/4 at column block 32 db + 16 (G%2) + 4 (s%4), so lane
    // l receives d = 32 db + l%32 at tokens base + 4 (l/32) + e: the k-slots
    // of lane group g = l/32 are tokens base+4g+{0..3} and base+8+4g+{0..3},
    // matching the accumulator layout of P. Operands are read two MFMAs
    // ahead.
    {
      const int G = lane >> 4, s4 = lane & 15;
      const int trow = 4 * (G >> 1) + (s4 >> 2);
      const int dcol = 16 * (G & 1) + 4 * (s4 & 3);
      auto pv_half = [&](int tt) {
        constexpr int NSTEP = 2 * S::kDBlocks;  // (kk, db)
        u32x4 a[3];
        auto rd = [&](int st) {
          const int kk = st / S::kDBlocks, db = st % S::kDBlocks;
          const int r0 = 32 * tt + 16 * kk + trow, r1 = r0 + 8;
          const int d0 = 32 * db + dcol;
          const uint8_t* p0 = vsm + r0 * S::kRowBytes + 16 * ((d0 >> 3) ^ swz_v<D>(r0)) + 2 * (d0 & 7);
          const uint8_t* p1 = vsm + r1 * S::kRowBytes + 16 * ((d0 >> 3) ^ swz_v<D>(r1)) + 2 * (d0 & 7);
          const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p0)));
          const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p1)));
          a[st % 3] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        rd(0);
        rd(1);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
          if (st + 2 < NSTEP) rd(st + 2);
          const int kk = st / S::kDBlocks, db = st % S::kDBlocks;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a[st % 3]),
                                                            pb[tt][kk], oacc[db], 0, 0, 0);
          // the next cube's K, one DMA per step (2 kDBlocks == kLoadsPerWave)
          if (tt == 0 && more) dma16(krsrc, koff[st], klds0 + 1024u * st);
        }
      };
      pv_half(0);
      if (two) pv_half(1);
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

size_t fwd_workspace_bytes(int B, int Nkv, int NH, int D) {
  return (size_t)B * Nkv * kCube * NH * D * 2;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* vbs, uint16_t* out,
                      int B, int Nq, int Nkv, int NH, int D, int topk,
                      float sm_scale, void* workspace, hipStream_t stream) {
  uint16_t* v16 = static_cast<uint16_t*>(workspace);
  const int cpr = NH * D / 8;
  hipLaunchKernelGGL(v_to_fp16_kernel, dim3(Nkv * kCvtSplit, B), dim3(kCvtThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(v16), vbs, Nkv,
                     cpr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_units = B * NH * Nq;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  if (D == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(n_units), dim3(FwdShape<128>::kThreads), 0,
                       stream, q, k, v16, topk_idx, vbs, out, Nq, Nkv, NH, topk,
                       scale_log2, n_units);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(n_units), dim3(FwdShape<64>::kThreads), 0,
                       stream, q, k, v16, topk_idx, vbs, out, Nq, Nkv, NH, topk,
                       scale_log2, n_units);
  return hipGetLastError();
}

}  // namespace vsa
