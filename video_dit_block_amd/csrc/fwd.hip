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
// * Two pre-passes: (1) an fp16 copy of v (the PV product runs in fp16);
//   (2) per (b, h, query cube) "unit", the selected cube ids sorted ascending
//   and expanded into a list of 32-token half-tiles: half 0 of every cube with
//   a real token, half 1 of every cube with more than 32. Each entry holds the
//   half-tile's byte offset from the head's first key row and its real-row
//   count, so the fine kernel builds a load descriptor with two scalar adds
//   and never touches a half without real tokens. The result does not depend
//   on the order of topk_idx; the ascending sweep makes the units resident on
//   one XCD walk their head's key/value cubes in the same order.
// * One workgroup = one unit: 2 waves of 32 query rows, 4 workgroups per CU
//   (2 waves per SIMD; 32 KiB of LDS each). Units are numbered head-major and
//   remapped so each XCD walks a contiguous range. A third pre-pass orders
//   each head's query cubes by descending count of selected cubes, then by
//   ascending smallest selected id, and that order is the dispatch order
//   inside the head. Units that run side by side then start their ascending
//   sweeps close together and move at similar rates, so they keep sharing L2
//   lines (measured on the Wan tensors: top-78 4.23 -> 3.99 ms; a lookup
//   table at a 0.9 mass threshold 18.5 -> 14.1 ms).
// * K and V half-tiles stream through LDS, each double-buffered, loaded
//   global -> LDS directly (buffer_load ... lds, two 1 KiB loads per M0
//   write); every wave loads half of each tile. The buffer range of a load
//   ends at the half's real rows, so padding rows land in LDS as zeros: pad
//   values (even NaN) never reach an MFMA.
// * Software pipeline inside each wave (step j = half-tile j):
//     A(j): QK^T of half-tile j+1 (8 MFMAs) interleaved with the softmax
//           exponentials, fp16 conversion and row sums of half-tile j;
//     B(j): PV of half-tile j (8 MFMAs) interleaved with the mask and row
//           max of half-tile j+1.
//   Matrix and vector work of one wave thus overlap, and the second wave on
//   the SIMD fills the remaining gaps. Loads keep 1.5 steps of lead: A(j)
//   issues V(j+1), B(j) issues K(j+3).
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the A operand is a K row slice read from LDS, the B operand is the wave's
//   Q held in registers for the whole loop. In the accumulator layout each
//   lane then holds 16 scores of ONE query row (row l%32; the other 16 of the
//   32-token half sit in lane l^32), so the row max and row sum need one
//   cross-half swap (v_permlane32_swap) and the probabilities are already in
//   the B-operand layout of O^T = V^T P^T: they go from accumulator to MFMA
//   operand in registers. The contraction index of the PV product is
//   permuted to match the accumulator's token order (any fixed permutation
//   of a summation index leaves the sum unchanged); the V^T operand comes
//   from two transposing 8-byte LDS reads per lane (ds_read_b64_tr_b16) of
//   row-major V.
// * fp32 online softmax in the exp2 domain: p = exp2(s * c - m * c) with
//   c = sm_scale * log2 e (one FMA per score), reference max m, running sum
//   l. The reference max is raised lazily: only when a half's row max
//   exceeds it by more than 2^8 (log2 units: 8) does the wave rescale O and l
//   by exp2((m_old - m_new) c); otherwise p may reach 2^8, which fp32 and fp16
//   hold exactly in range. Tokens past a half's real rows are set to -inf in
//   registers before the max (partial halves only). O^T accumulates in fp32,
//   each lane holding D/2 values of its own query row, so the rescale is a
//   per-lane multiply.
// * Precision: QK^T is a bf16 MFMA with fp32 accumulation. The PV product
//   runs as an fp16 MFMA (v_mfma_f32_32x32x16_f16): P is rounded to fp16 and
//   V is converted to fp16 by the pre-pass. fp16 keeps 3 more
//   significand bits than bf16, which matters for rows with few keys; V is
//   converted exactly for 2^-14 <= |v| <= 65504 and 0 (there every bf16
//   value is an fp16 value), saturates to 65504 above, and below 2^-14 (fp16
//   subnormals) is truncated toward zero, an absolute error under 2^-24. O / l
//   is rounded to bf16 (nearest even) and stored.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kHalf = 32;  // tokens per half-tile

template <int D>
struct FwdShape {
  static constexpr int kThreads = 128;                  // 2 waves x 32 query rows
  static constexpr int kRowBytes = 2 * D;               // one (token, head) row
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;  // rows one wave-wide load fills
  static constexpr int kHalfBytes = kHalf * kRowBytes;  // one tensor of one half-tile
  static constexpr int kLoads = kHalfBytes / 1024 / 2;  // loads per wave, tensor and half-tile
  static constexpr int kQSteps = D / 16;                // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;               // 32-wide d blocks of O^T
  static_assert(kLoads % 2 == 0, "loads go in pairs");
};

// XOR swizzles of the 16-byte chunk index inside an LDS row: chunk c of row r
// lives in slot c ^ swz(r). Chosen (by an exhaustive search over linear maps
// of the row's low 4 bits, with a 32- and a 64-bank model) so that the two
// read patterns below are free of bank conflicts:
//   K: 32 lanes read chunk c of rows r..r+31 (ds_read_b128);
//   V: the transposing read, 16-lane groups reading 8 bytes of 4
//      consecutive rows at 4 column blocks (ds_read_b64_tr_b16).
// The V swizzle depends on the row's low 2 bits only.
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

// Lazy rescale threshold (log2 units): the running reference max is only
// raised when a tile's max exceeds it by more than this, so unnormalised
// probabilities stay <= 2^8.
constexpr float kRescaleThreshold = 8.0f;
constexpr int kBufferDword3 = 0x00020000;  // gfx9 raw buffer resource flags

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef int32_t int32x4_t __attribute__((ext_vector_type(4)));

// Two wave-wide 16-byte-per-lane global -> LDS loads (buffer_load_dwordx4 ...
// lds) into consecutive KiB of LDS with one M0 write: lane L's 16 bytes of
// the first load land at LDS byte lds_addr + 16 L, those of the second at
// lds_addr + 1024 + 16 L. The instruction offset (1024) applies to both the
// global and the LDS address, so the second lane offset comes pre-reduced by
// 1024. Issued as inline assembly so that the compiler does not guard every
// later LDS read with a wait for all outstanding loads; the kernel waits
// explicitly (wait_vmcnt) before the barrier that publishes a tile. The
// s_nop covers the M0 -> LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used nowhere else
__device__ __forceinline__ void dma16x2(int32x4_t rsrc, uint32_t voff0, uint32_t voff1m,
                                        uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
      :
      : "s"(lds_addr), "v"(voff0), "v"(voff1m), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

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

template <int N>
using IC = std::integral_constant<int, N>;

// ---------------------------------------------------------------------------
// V -> fp16 pre-pass. Writes an fp16 copy of v (same tiled BSHD layout) into
// the workspace: real rows converted, padding rows zeroed. bf16 -> f32 is
// exact (the bf16 bits are the upper half of an f32); f32 -> f16 with
// truncation is exact for 2^-14 <= |v| <= 65504 and 0, since every such bf16
// value is an fp16 value; it saturates to 65504 above, and below 2^-14 (fp16
// subnormals) it loses at most 2^-24. HBM-bound: one read and one write of v.
constexpr int kCvtThreads = 256;
constexpr int kCvtSplit = 8;   // workgroups per cube (8 slots each)
constexpr int kCvtUnroll = 8;  // 16-byte loads in flight per lane

__device__ __forceinline__ u32x4 bf16x8_to_fp16x8(const u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[e] << 16),
                                                                  __uint_as_float(w[e] & 0xFFFF0000u)));
  return o;
}

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
      int col = lane;
      for (; col + 64 * (kCvtUnroll - 1) < cpr; col += 64 * kCvtUnroll) {
        u32x4 w[kCvtUnroll];
#pragma unroll
        for (int i = 0; i < kCvtUnroll; ++i) w[i] = __builtin_nontemporal_load(src + col + 64 * i);
#pragma unroll
        for (int i = 0; i < kCvtUnroll; ++i) dst[col + 64 * i] = bf16x8_to_fp16x8(w[i]);
      }
      for (; col < cpr; col += 64) dst[col] = bf16x8_to_fp16x8(__builtin_nontemporal_load(src + col));
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int col = lane; col < cpr; col += 64) dst[col] = z;
    }
  }
}

// ---------------------------------------------------------------------------
// Half-tile list pre-pass: one wave per unit (b, h, query cube). The unit's
// selected ids (the first valid[unit] entries of its index row, or all of
// them; clamped into range: a violated precondition gives unspecified values,
// never an out-of-bounds access) are sorted ascending and expanded into
// 32-token half-tiles: half 0 of every cube with a real token, half 1 of
// every cube with more than 32. Entry = (byte offset of the half from the
// head's first key row, real rows of the half), two uint32; kListPad (0, 0)
// entries follow the last one. Rows with topk > kListSortCap keep the given
// order.
constexpr int kListSortCap = 1024;
constexpr int kListPad = 4;

__global__ __launch_bounds__(64) void halves_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ valid,
    const int32_t* __restrict__ vbs, uint32_t* __restrict__ list, int32_t* __restrict__ counts,
    int Nkv, int row_len, int stride, uint32_t rs2) {
  __shared__ int32_t keys[kListSortCap];
  const int unit = blockIdx.x, lane = threadIdx.x;
  const int32_t* __restrict__ sel = topk_idx + (size_t)unit * row_len;
  // the row's first `topk` ids are used: all of them, or valid[unit] (clamped)
  const int topk = valid == nullptr ? row_len : min(max(valid[unit], 0), row_len);
  uint32_t* __restrict__ out = list + (size_t)unit * stride * 2;
  const bool sorted = topk <= kListSortCap;
  auto id_at = [&](int i) __attribute__((always_inline)) -> int {
    return min(max(sel[i], 0), Nkv - 1);
  };
  if (sorted) {
    int n2 = 1;
    while (n2 < topk) n2 <<= 1;
    for (int i = lane; i < n2; i += 64) keys[i] = i < topk ? id_at(i) : 0x7FFFFFFF;
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride2 = size >> 1; stride2 > 0; stride2 >>= 1) {
        __syncthreads();
        for (int t = lane; t < (n2 >> 1); t += 64) {
          const int lo = 2 * t - (t & (stride2 - 1)), hi = lo + stride2;
          const int a = keys[lo], c = keys[hi];
          if (((lo & size) == 0) == (a > c)) {
            keys[lo] = c;
            keys[hi] = a;
          }
        }
      }
    __syncthreads();
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  for (int c0 = 0; c0 < topk; c0 += 64) {
    const int i = c0 + lane;
    int id = 0, nv = 0;
    if (i < topk) {
      id = sorted ? keys[i] : id_at(i);
      nv = min(max(vbs[id], 0), kCube);
    }
    const uint64_t b1 = __builtin_amdgcn_ballot_w64(nv > 0);
    const uint64_t b2 = __builtin_amdgcn_ballot_w64(nv > kHalf);
    const int pos = base + __builtin_popcountll(b1 & below) + __builtin_popcountll(b2 & below);
    const uint32_t off0 = (uint32_t)id * (uint32_t)kCube * rs2;
    if (nv > 0) {
      out[2 * pos] = off0;
      out[2 * pos + 1] = (uint32_t)min(nv, kHalf);
    }
    if (nv > kHalf) {
      out[2 * pos + 2] = off0 + (uint32_t)kHalf * rs2;
      out[2 * pos + 3] = (uint32_t)(nv - kHalf);
    }
    base += __builtin_popcountll(b1) + __builtin_popcountll(b2);
  }
  if (lane < 2 * kListPad) out[2 * base + lane] = 0u;
  if (lane == 0) counts[unit] = base;
}

// Dispatch order inside each (b, h): query cubes by descending count of
// selected cubes, then by ascending smallest selected id, then by cube id.
// Units that run side by side then sweep the ascending key ids from nearby
// starting points at similar rates, so their half-tile loads keep hitting the
// same L2 lines, and with per-row counts the longest units start first.
// Two passes: order_key_kernel writes one packed key per unit, a lane quad
// per unit; order_rank_kernel ranks each head's keys, grid (B*NH,
// ceil(Nq / 256)), dynamic LDS Nq uint64. Smallest ids are capped at 2^20 - 1
// in the key (the order stays valid, only less sharp, above that).
constexpr int kOrderThreads = 256;
constexpr int kOrderMaxNq = 4096;

// The key packs the order into one integer: 2^31 - 1 - count, then the
// smallest id (below 2^20), then the cube id (below kOrderMaxNq = 2^12).
__global__ __launch_bounds__(kOrderThreads) void order_key_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ valid, int row_len,
    int Nkv, int Nq, uint64_t* __restrict__ keys, int64_t n_units) {
  const int64_t i4 = (int64_t)blockIdx.x * kOrderThreads + threadIdx.x;
  const int64_t unit = i4 >> 2;
  const int part = (int)(i4 & 3);
  if (unit >= n_units) return;  // whole quads leave together (n_units * 4 lanes)
  const int n = valid == nullptr ? row_len : min(max(valid[unit], 0), row_len);
  const int32_t* __restrict__ sel = topk_idx + unit * row_len;
  int first = (1 << 20) - 1;
#pragma unroll 8
  for (int t = part; t < n; t += 4) first = min(first, min(max(sel[t], 0), Nkv - 1));
  first = min(first, __shfl_xor(first, 1, 64));
  first = min(first, __shfl_xor(first, 2, 64));
  if (part == 0)
    keys[unit] = ((uint64_t)(0x7FFFFFFF - n) << 32) | ((uint64_t)first << 12) |
                 (uint64_t)(unit % Nq);
}

__global__ __launch_bounds__(kOrderThreads) void order_rank_kernel(
    const uint64_t* __restrict__ keys, int32_t* __restrict__ order, int Nq) {
  extern __shared__ uint64_t key[];
  const size_t base = (size_t)blockIdx.x * Nq;
  for (int i = threadIdx.x; i < Nq; i += kOrderThreads) key[i] = keys[base + i];
  __syncthreads();
  const int i = blockIdx.y * kOrderThreads + threadIdx.x;
  if (i >= Nq) return;
  const uint64_t ki = key[i];
  int rank = 0;  // keys are distinct (the cube id is part of them)
#pragma unroll 8
  for (int j = 0; j < Nq; ++j) rank += key[j] < ki;
  order[base + rank] = i;
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(FwdShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v16, const uint32_t* __restrict__ list,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ order,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ max_prob, int Nq,
    int Nkv, int NH, int list_stride, float scale_log2, int n_units) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][S::kHalfBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][S::kHalfBytes];

  // XCD x runs a contiguous range of (b, h, rank); within a (b, h) the query
  // cube of a rank is the rank itself, or order[] for per-row counts
  const int lin = xcd_remap(blockIdx.x, n_units);
  const int bh = lin / Nq;
  const int qc = order == nullptr ? lin - bh * Nq : min(max(order[lin], 0), Nq - 1);
  const int unit = bh * Nq + qc;
  const int h = bh % NH, b = bh / NH;
  const size_t row_stride = (size_t)NH * D;  // elements between tokens
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qr = lane & 31, g = lane >> 5;
  const size_t qrow = ((size_t)b * Nq + qc) * kCube + 32 * wave + qr;

  // ---- Q of this wave's 32 rows, in the B-operand layout of S^T = K Q^T:
  // lane (column qr, k-group g) holds q[row][16 s + 8 g .. + 7].
  bf16x8 qf[S::kQSteps];
  {
    const uint16_t* q0 = q + qrow * row_stride + (size_t)h * D;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(q0 + 16 * s + 8 * g);
  }
  uint16_t* const orow = out + qrow * row_stride + (size_t)h * D;

  // ---- the unit's half-tiles; reads past the list (i >= n) see the (0, 0)
  // padding entries (i < n + kListPad)
  const uint32_t* __restrict__ lst = list + (size_t)unit * list_stride * 2;
  const int n = __builtin_amdgcn_readfirstlane(counts[unit]);
  auto ent = [&](int i) __attribute__((always_inline)) -> u32x2 {
    const u32x2 v = *reinterpret_cast<const u32x2*>(lst + 2 * __builtin_amdgcn_readfirstlane(i));
    return u32x2{(uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)v[1])};
  };
  // per-row statistics: row (b, h, c * 64 + 32 wave + qr), written by lane g = 0
  const size_t srow = ((size_t)bh * Nq + qc) * kCube + 32 * wave + qr;
  if (n == 0) {  // no real key in any selected cube: the rows are 0
#pragma unroll
    for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * g) = u32x2{0u, 0u};
    if (g == 0 && lse != nullptr) lse[srow] = kNegInf;
    if (g == 0 && max_prob != nullptr) max_prob[srow] = 0.0f;
    return;
  }

  // ---- loads: wave w fills KiB [L w, L w + L) of every half-tile buffer
  // (L = kLoads), lane L' writing bytes [16 L', 16 L' + 16) of a KiB; the
  // lane fetches the global chunk that the swizzle places in that slot.
  // Byte offsets stay below 2^32 (host-checked).
  constexpr int L = S::kLoads;
  const uint32_t rs2 = (uint32_t)NH * D * 2u;
  uint32_t koff[L], voff[L];
#pragma unroll
  for (int m = 0; m < L; ++m) {
    const int row = (wave * L + m) * S::kRowsPerKiB + lane / S::kChunks;
    const int slot = lane % S::kChunks;
    koff[m] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_k<D>(row)) - 1024u * (m & 1);
    voff[m] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_v<D>(row)) - 1024u * (m & 1);
  }
  const uint32_t lds_wave = (uint32_t)(wave * L) * 1024u;
  const size_t kv_head = (size_t)b * Nkv * kCube * row_stride + (size_t)h * D;
  const uint64_t kbase = reinterpret_cast<uint64_t>(k + kv_head);
  const uint64_t vbase = reinterpret_cast<uint64_t>(v16 + kv_head);
  // gfx9 raw buffer descriptor of one half-tile: base + offset, range = its
  // real rows (the loads of padding rows and of (0, 0) entries return zeros)
  auto mk_rsrc = [&](uint64_t base, const u32x2& e) __attribute__((always_inline)) -> int32x4_t {
    const uint64_t a = base + e[0];
    int32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)(e[1] * rs2));
    r[3] = kBufferDword3;
    return r;
  };
  const uint32_t kb0 = lds_address(kbuf), vb0 = lds_address(vbuf);
  // load pair p (0 <= p < L / 2) of a half-tile into buffer `buf`
  auto dma_k = [&](const int32x4_t& r, int buf, int p) __attribute__((always_inline)) {
    dma16x2(r, koff[2 * p], koff[2 * p + 1], kb0 + (uint32_t)buf * S::kHalfBytes + lds_wave + 2048u * p);
  };
  auto dma_v = [&](const int32x4_t& r, int buf, int p) __attribute__((always_inline)) {
    dma16x2(r, voff[2 * p], voff[2 * p + 1], vb0 + (uint32_t)buf * S::kHalfBytes + lds_wave + 2048u * p);
  };

  // ---- per-lane LDS read addresses in buffer 0 (buffer 1 is a constant
  // offset away). K: chunk 2 st + g of row qr. V^T: rows 16 kk + trow (+8),
  // columns 32 db + dcol; since the V swizzle depends on the row mod 4 only,
  // kk and the +8 rows are constant offsets too. The transposing read: in each
  // 16-lane group, lane i receives element i%4 of the 8 bytes that lane
  // 4e + i/4 addressed, for e = 0..3. Lane (group G, s) addresses row
  // base + 4(G/2) + s/4 at column block 32 db + 16 (G%2) + 4 (s%4), so lane l
  // receives d = 32 db + l%32 at tokens base + 4 (l/32) + e: the k-slots of
  // lane group g = l/32 are tokens base+4g+{0..3} and base+8+4g+{0..3},
  // matching the accumulator layout of P.
  const uint8_t* kl[S::kQSteps];
#pragma unroll
  for (int st = 0; st < S::kQSteps; ++st)
    kl[st] = &kbuf[0][0] + qr * S::kRowBytes + 16 * ((2 * st + g) ^ swz_k<D>(qr));
  const int Gq = lane >> 4, s4 = lane & 15;
  const int trow = 4 * (Gq >> 1) + (s4 >> 2);
  const int dcol = 16 * (Gq & 1) + 4 * (s4 & 3);
  const uint8_t* vl[S::kDBlocks];
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db) {
    const int d0 = 32 * db + dcol;
    vl[db] = &vbuf[0][0] + trow * S::kRowBytes + 16 * ((d0 >> 3) ^ swz_v<D>(trow)) + 2 * (d0 & 7);
  }

  floatx16 oacc[S::kDBlocks];
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  // m_ref: reference max (raw score units) the probabilities are taken
  // against; l_run: running sum of exp2((s - m_ref) * scale_log2); alpha and
  // need_rescale: the pending O rescale after a raise of m_ref
  float m_ref = kNegInf, l_run = 0.0f, alpha = 1.0f;
  float m_row = kNegInf;  // the row's largest score so far (for max_prob)
  bool need_rescale = false;
  const floatx16 zero16 = {};
  const halfx2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // S^T = K Q^T for the half-tile in K buffer kbi; V load pairs ride along
  auto qk = [&](int kbi, floatx16& s, const int32x4_t& vr, int vbi) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < S::kQSteps; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl[st] + kbi * S::kHalfBytes);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? zero16 : s, 0, 0, 0);
      if (vbi >= 0 && st % 2 == 1 && st / 2 < L / 2) dma_v(vr, vbi, st / 2);
    }
  };
  // O^T += V^T P^T for the half-tile in V buffer vbi; K load pairs ride along
  auto pv = [&](int vbi, const halfx8 (&pb)[2], const int32x4_t& kr, int kbi) __attribute__((always_inline)) {
    constexpr int NSTEP = 2 * S::kDBlocks;  // (kk, db)
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st / S::kDBlocks, db = st % S::kDBlocks;
      const uint8_t* p0 = vl[db] + vbi * S::kHalfBytes + kk * 16 * S::kRowBytes;
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p0)));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p0 + 8 * S::kRowBytes)));
      const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), pb[kk], oacc[db], 0, 0, 0);
      if (kbi >= 0 && st % 2 == 1 && st / 2 < L / 2) dma_k(kr, kbi, st / 2);
    }
  };
  // tokens >= the half's real rows set to -inf (partial halves only; the asm
  // keeps the compiler from flattening the branch into selects that every
  // half would execute), row max, lazy raise of the reference max
  // (wave-uniform decision)
  auto mask_max = [&](uint32_t nvh, floatx16& s) __attribute__((always_inline)) {
    if (nvh < (uint32_t)kHalf) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t tok = 8 * (r >> 2) + 4 * g + (r & 3);
        if (tok >= nvh) s[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    m_row = fmaxf(m_row, mx);
    const bool up = mx * scale_log2 > m_ref * scale_log2 + kRescaleThreshold;
    need_rescale = __builtin_amdgcn_ballot_w64(up) != 0;
    if (need_rescale) {
      const float m_new = up ? mx : m_ref;
      alpha = m_ref == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
      m_ref = m_new;
      l_run *= alpha;
    }
  };
  // P in fp16 (round to nearest even) and the row sums of the same rounded
  // values (v_dot2_f32_f16 against 1.0). Every row has a finite m_ref here:
  // the first half-tile of a unit holds at least one real token.
  auto exp_sum = [&](const floatx16& s, halfx8 (&pb)[2]) __attribute__((always_inline)) {
    const float mc = m_ref * scale_log2;
    float rs = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      floatx8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kk + e], scale_log2, -mc));
      pb[kk] = __builtin_convertvector(p, halfx8);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const halfx2 two = {pb[kk][e], pb[kk][e + 1]};
        rs = __builtin_amdgcn_fdot2(two, ones, rs, false);
      }
    }
    l_run += halves_sum(rs);
  };
  auto rescale = [&]() __attribute__((always_inline)) {
    if (need_rescale) {
#pragma unroll
      for (int db = 0; db < S::kDBlocks; ++db) oacc[db] *= alpha;
    }
  };

  // The Q loads must be complete before the first tile load is issued:
  // afterwards the only outstanding vector-memory operations are the tile
  // loads that the explicit waits account for. The empty asm makes the
  // compiler place its own wait for Q here rather than inside the loop.
#pragma unroll
  for (int s = 0; s < S::kQSteps; ++s) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qf[s])));

  // ---- prologue: K(0), K(1), V(0) in flight; QK(0) and its max
  floatx16 sA, sB;
  halfx8 pb[2];
  u32x2 e_n1 = ent(1), e_n2 = ent(2);
  {
    const u32x2 e0 = ent(0);
    const int32x4_t r0 = mk_rsrc(kbase, e0), r1 = mk_rsrc(kbase, e_n1), r2 = mk_rsrc(vbase, e0);
#pragma unroll
    for (int p = 0; p < L / 2; ++p) dma_k(r0, 0, p);
#pragma unroll
    for (int p = 0; p < L / 2; ++p) dma_k(r1, 1, p);
#pragma unroll
    for (int p = 0; p < L / 2; ++p) dma_v(r2, 0, p);
    wait_vmcnt<2 * L>();  // K(0): K(1), V(0) may be in flight
    __syncthreads();
    qk(0, sA, r0, -1);
    mask_max(e0[1], sA);
    need_rescale = false;  // O and l are still zero
  }

  // Step j (0 <= j < n - 1), parity P = j & 1: S(j) in sc, S(j+1) into sn.
  //   A(j): K(j+1) landed; O rescale; QK(j+1) with V(j+1)'s loads; P(j)
  //   B(j): V(j) landed; PV(j) with K(j+3)'s loads; mask and max of S(j+1)
  // K(i) and V(i) sit in buffer i & 1. K(j+3) reuses the buffer of K(j+1),
  // which every wave finished in A(j) (the barrier of B(j) certifies it);
  // V(j+1) reuses that of V(j-1), finished in B(j-1) (the barrier of A(j)).
  // Issue order: K0 K1 V0 | A(0): K2 V1 | B(0): K3 | A(1): V2 | B(1): K4 ...;
  // from A(1) on every wait leaves the two most recent tiles in flight.
  auto step = [&](auto Pc, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(Pc)::value;
    floatx16& sc = P ? sB : sA;
    floatx16& sn = P ? sA : sB;
    const u32x2 e_n3 = ent(j + 3);
    if (j == 0) {
      wait_vmcnt<L>();  // K(1): V(0) may be in flight
      __syncthreads();
      const int32x4_t r2 = mk_rsrc(kbase, e_n2);
#pragma unroll
      for (int p = 0; p < L / 2; ++p) dma_k(r2, 0, p);
    } else {
      wait_vmcnt<2 * L>();  // K(j+1)
      __syncthreads();
    }
    rescale();
    qk(P ^ 1, sn, mk_rsrc(vbase, e_n1), P ^ 1);
    exp_sum(sc, pb);
    wait_vmcnt<2 * L>();  // V(j)
    __syncthreads();
    pv(P, pb, mk_rsrc(kbase, e_n3), P ^ 1);
    mask_max(e_n1[1], sn);
    e_n1 = e_n2;
    e_n2 = e_n3;
  };
  int j = 0;
  if (n > 1) {
    step(IC<0>{}, 0);
    j = 1;
#pragma unroll 1
    while (j + 1 < n) {
      step(IC<1>{}, j);
      ++j;
      if (j + 1 >= n) break;
      step(IC<0>{}, j);
      ++j;
    }
  }
  // ---- the last step: P(n-1) and PV(n-1); V(n-1) sits in vbuf[(n-1) & 1]
  {
    rescale();
    exp_sum((j & 1) ? sB : sA, pb);
    wait_vmcnt<0>();
    __syncthreads();
    const int32x4_t none = mk_rsrc(kbase, u32x2{0u, 0u});
    if (j & 1)
      pv(1, pb, none, -1);
    else
      pv(0, pb, none, -1);
  }

  // ---- per-row statistics. l_run sums exp2((s - m_ref) c), so the natural
  // log-sum-exp of the scaled scores is (m_ref c + log2 l_run) ln 2, and the
  // largest softmax weight is 1 / sum exp2((s - m_row) c) =
  // exp2((m_row - m_ref) c) / l_run.
  if (g == 0 && lse != nullptr)
    lse[srow] = (m_ref * scale_log2 + __log2f(l_run)) * 0.69314718055994531f;
  if (g == 0 && max_prob != nullptr)
    max_prob[srow] = __builtin_amdgcn_exp2f((m_row - m_ref) * scale_log2) / l_run;

  // ---- epilogue: lane holds O^T[d][row] for d = 32 db + 8 (r/4) + 4 g + r%4
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
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

FwdWorkspace fwd_workspace(int B, int Nq, int Nkv, int NH, int D, int topk) {
  auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
  FwdWorkspace w;
  w.list_stride = 2 * topk + kListPad;  // entries per unit, 8 bytes each
  const size_t units = (size_t)B * NH * Nq;
  w.v16_off = 0;
  w.list_off = up((size_t)B * Nkv * kCube * NH * D * 2);
  w.count_off = w.list_off + up(units * w.list_stride * 8);
  w.order_off = w.count_off + up(units * 4);
  w.key_off = w.order_off + up(units * 4);
  w.total = w.key_off + up(units * 8);
  return w;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* valid, const int32_t* vbs,
                      uint16_t* out, float* lse, float* max_prob, int B, int Nq, int Nkv,
                      int NH, int D, int topk, float sm_scale, void* workspace,
                      hipStream_t stream) {
  const FwdWorkspace w = fwd_workspace(B, Nq, Nkv, NH, D, topk);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + w.v16_off);
  uint32_t* list = reinterpret_cast<uint32_t*>(ws + w.list_off);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.count_off);
  int32_t* order = nullptr;
  const int cpr = NH * D / 8;
  const int n_units = B * NH * Nq;
  hipLaunchKernelGGL(v_to_fp16_kernel, dim3(Nkv * kCvtSplit, B), dim3(kCvtThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(v16), vbs, Nkv,
                     cpr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The order pass runs ahead of the list pass: launched right before the
  // fine kernel it cost that kernel about 1 ms at 312 cubes per row
  // (measured, cause not established).
  if (Nq <= kOrderMaxNq) {
    order = reinterpret_cast<int32_t*>(ws + w.order_off);
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + w.key_off);
    const int64_t lanes = (int64_t)n_units * 4;
    hipLaunchKernelGGL(order_key_kernel, dim3((unsigned)((lanes + kOrderThreads - 1) / kOrderThreads)),
                       dim3(kOrderThreads), 0, stream, topk_idx, valid, topk, Nkv, Nq, keys,
                       (int64_t)n_units);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(order_rank_kernel, dim3(B * NH, (Nq + kOrderThreads - 1) / kOrderThreads),
                       dim3(kOrderThreads), (size_t)Nq * sizeof(uint64_t), stream, keys, order, Nq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(halves_kernel, dim3(n_units), dim3(64), 0, stream, topk_idx, valid, vbs,
                     list, counts, Nkv, topk, w.list_stride, (uint32_t)NH * D * 2u);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  if (D == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(n_units), dim3(FwdShape<128>::kThreads), 0, stream,
                       q, k, v16, list, counts, order, out, lse, max_prob, Nq, Nkv, NH,
                       w.list_stride, scale_log2, n_units);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(n_units), dim3(FwdShape<64>::kThreads), 0, stream,
                       q, k, v16, list, counts, order, out, lse, max_prob, Nq, Nkv, NH,
                       w.list_stride, scale_log2, n_units);
  return hipGetLastError();
}

}  // namespace vsa
