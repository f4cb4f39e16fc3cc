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
// * Pre-passes: (1) an fp16 copy of v (the PV product runs in fp16), exact
//   over the bf16 range through a per-head power-of-two scale where a head's
//   values leave fp16's normal range; (2) per (b, h, query cube) "unit", the
//   selected cube ids sorted ascending and cut into quarters of at most 16
//   real rows, consecutive quarters paired into 32-row tiles. Each quarter is
//   its byte offset from the head's first key row plus its real-row count, so
//   the fine kernel builds a load descriptor with two scalar operations and
//   never spends a tile on padding rows except where a cube's real count is
//   not a multiple of 16. The result does not depend on the order of
//   topk_idx; the ascending sweep makes the units resident on one XCD walk
//   their head's key/value cubes in the same order.
// * One workgroup = one unit: 2 waves of 32 query rows, 4 workgroups per CU
//   (2 waves per SIMD; 32 KiB of LDS each). Units are numbered head-major and
//   remapped so each XCD walks a contiguous range. A third pre-pass orders
//   each head's query cubes by descending count of selected cubes, then by
//   ascending smallest selected id, and that order is the dispatch order
//   inside the head. Units that run side by side then start their ascending
//   sweeps close together and move at similar rates, so they keep sharing L2
//   lines (measured on the Wan tensors: top-78 4.23 -> 3.99 ms; a lookup
//   table at a 0.9 mass threshold 18.5 -> 14.1 ms).
// * Key-range splits (split-KV) for heads whose K and fp16 V exceed about
//   32 MiB: each unit runs as S work items, item s over its selected cubes
//   in key range s, split-major inside each head, so that the items resident
//   on an XCD share one range of the head's keys; each item leaves a partial
//   online-softmax state and merge_kernel combines them (fwd_splits below).
// * K and V tiles stream through LDS, each double-buffered, loaded
//   global -> LDS directly (buffer_load ... lds, two 1 KiB loads per M0
//   write); wave w loads quarter w of each tile with its own descriptor. The
//   buffer range of a load ends at the quarter's real rows, so padding rows
//   land in LDS as zeros: pad values (even NaN) never reach an MFMA.
// * Software pipeline inside each wave (step j = tile j):
//     A(j): QK^T of tile j+1 (8 MFMAs) interleaved with the softmax
//           exponentials, fp16 conversion and row sums of tile j;
//     B(j): PV of tile j (8 MFMAs) interleaved with the mask and row
//           max of tile j+1.
//   Matrix and vector work of one wave thus overlap, and the second wave on
//   the SIMD fills the remaining gaps. Loads keep 1.5 steps of lead: A(j)
//   issues V(j+1), B(j) issues K(j+3).
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the A operand is a K row slice read from LDS, the B operand is the wave's
//   Q held in registers for the whole loop. In the accumulator layout each
//   lane then holds 16 scores of ONE query row (row l%32; the other 16 of the
//   32-token tile sit in lane l^32), so the row max and row sum need one
//   cross-half swap (v_permlane32_swap) and the probabilities are already in
//   the B-operand layout of O^T = V^T P^T: they go from accumulator to MFMA
//   operand in registers. The contraction index of the PV product is
//   permuted to match the accumulator's token order (any fixed permutation
//   of a summation index leaves the sum unchanged); the V^T operand comes
//   from two transposing 8-byte LDS reads per lane (ds_read_b64_tr_b16) of
//   row-major V.
// * fp32 online softmax in the exp2 domain: p = exp2(s * c - m * c + 7) with
//   c = sm_scale * log2 e (one FMA per score), reference max m, running sum
//   l. The reference max is raised lazily: only when a tile's row max
//   exceeds it by more than 2^8 (log2 units: 8) does the wave rescale O and l
//   by exp2((m_old - m_new) c); otherwise p may reach 2^8 * 2^7, which fp32
//   and fp16 hold in range. The constant 2^7 keeps weights down to 2^-21 of
//   the reference max normal in fp16; it cancels in O / l. Tokens past a
//   quarter's real rows are set to -inf in registers before the max (tiles
//   with a partial quarter only). O^T accumulates in fp32, each lane holding
//   D/2 values of its own query row, so the rescale is a per-lane multiply.
// * Precision: QK^T is a bf16 MFMA with fp32 accumulation. The PV product
//   runs as an fp16 MFMA (v_mfma_f32_32x32x16_f16): P is rounded to fp16 and
//   V is converted to fp16 by the pre-pass. fp16 keeps 3 more significand
//   bits than bf16, which matters for rows with few keys. Every bf16 value
//   with 2^-14 <= |v| <= 65504 (and 0) is an fp16 value; heads whose largest
//   |v| lies outside [2^-4, 65504] are converted scaled by a power of two
//   2^-e_h, undone in the epilogue, so the copy is exact over the bf16 range
//   up to fp16 subnormals (an absolute error under 2^-24 * 2^e_h, at most
//   2^-20 of the head's largest |v|). O / l * 2^e_h is rounded to bf16
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
constexpr int kTile = 32;  // tokens per tile (two quarters)

template <int D>
struct FwdShape {
  static constexpr int kThreads = 128;                  // 2 waves x 32 query rows
  static constexpr int kRowBytes = 2 * D;               // one (token, head) row
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;  // rows one wave-wide load fills
  static constexpr int kTileBytes = kTile * kRowBytes;  // one tensor of one tile
  static constexpr int kLoads = kTileBytes / 1024 / 2;  // loads per wave, tensor and tile
  static constexpr int kQSteps = D / 16;                // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;               // 32-wide d blocks of O^T
  static_assert(kLoads % 2 == 0, "loads go in pairs");
  static_assert(kLoads * kRowsPerKiB == 16, "each wave loads one 16-row quarter");
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
// Every probability is computed as 2^kPShift times its value relative to the
// reference max: p in (0, 2^15] instead of (0, 2^8], still inside fp16's range
// (65504), so that weights down to 2^-21 of the reference (not 2^-14) stay
// normal fp16 numbers when P enters the P.V product. O and l carry the same
// factor, which cancels in O / l; the row statistics remove it.
constexpr float kPShift = 7.0f;
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
  // one v_max_f32: fmaxf would first quieten both operands (a v_max of each
  // with itself); the values here are never NaN
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
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
// V -> fp16 pre-pass, exact over the bf16 range. Every bf16 value whose
// magnitude lies in [2^-14, 65504] (or is 0) is an fp16 value, so for the
// usual inputs the conversion is a plain copy into the narrower format. A
// head (b, h) whose largest |v| over its real rows is above 65504, or below
// 2^-4, is instead stored scaled by 2^-e_h, e_h = floor(log2 max|v|) - 14
// (clamped to [-90, 113]), which puts its largest magnitude in [2^14, 2^15);
// multiplying by a power of two is exact, and the fine kernel multiplies the
// head's output rows by 2^e_h. Three launches:
//   v_to_fp16_kernel: real rows converted with e = 0 (padding rows are never
//                     read, so not written), and the largest |v| of every
//                     (workgroup, head) written to vmax;
//   vscale_kernel:    per (b, h), e_h from the largest of those maxima;
//   vfix_kernel:      the rows of heads with e_h != 0 converted again, scaled.
// Only the first is HBM-bound (one read and one write of v); the other two
// read a few hundred KiB and, for in-range heads, return at once.
// Values below 2^-14 (times 2^e_h) become fp16 subnormals by truncation,
// an absolute error under 2^-24 (times 2^e_h): at most 2^-20 of the head's
// largest |v| when e_h = 0.
constexpr int kCvtThreads = 256;
constexpr int kCvtSplit = 8;    // workgroups per cube (8 slots each)
constexpr int kCvtColBlk = 4;   // 64-lane column blocks per pass (x 2 rows = 8 loads in flight)
constexpr int kVexpMin = -90, kVexpMax = 113;

__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const u32x4 w) {
  // largest |x| of 8 bf16 values as fp32 bits (non-negative floats order as
  // unsigned integers)
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max((w[e] << 16) & 0x7FFF0000u, w[e] & 0x7FFF0000u));
  return m;
}

__device__ __forceinline__ uint32_t cvt2_fp16(uint32_t w, int e) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e == 0 ? lo : ldexpf(lo, -e),
                                                                e == 0 ? hi : ldexpf(hi, -e)));
}

__device__ __forceinline__ u32x4 bf16x8_to_fp16x8(const u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = cvt2_fp16(w[e], 0);
  return o;
}

// grid (Nkv * kCvtSplit, B); wave w converts rows 8 part + w and 8 part + 4 + w
// of cube c. cph = 16-byte chunks per head (D / 8), cpr = per row (NH cph).
// vmax[b][blockIdx.x][h] = largest |v| (fp32 bits) of the workgroup's real rows.
__global__ __launch_bounds__(kCvtThreads) void v_to_fp16_kernel(
    const u32x4* __restrict__ v, u32x4* __restrict__ v16, const int32_t* __restrict__ vbs,
    uint32_t* __restrict__ vmax, int Nkv, int NH, int cph) {
  __shared__ uint32_t red[kCvtThreads / 64][kCvtColBlk * 64];
  const int c = blockIdx.x / kCvtSplit, part = blockIdx.x % kCvtSplit, b = blockIdx.y;
  const int nv = min(max(vbs[c], 0), kCube);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int cpr = NH * cph;
  const int u0 = part * (kCube / kCvtSplit) + wave, u1 = u0 + 4;
  const size_t row0 = ((size_t)b * Nkv + c) * kCube + u0;
  const u32x4* __restrict__ src0 = v + row0 * cpr;
  const u32x4* __restrict__ src1 = src0 + (size_t)4 * cpr;
  u32x4* __restrict__ dst0 = v16 + row0 * cpr;
  u32x4* __restrict__ dst1 = dst0 + (size_t)4 * cpr;
  uint32_t* __restrict__ vm = vmax + ((size_t)b * gridDim.x + blockIdx.x) * NH;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c0 = 0; c0 < cpr; c0 += 64 * kCvtColBlk) {
    u32x4 w0[kCvtColBlk], w1[kCvtColBlk];
#pragma unroll
    for (int i = 0; i < kCvtColBlk; ++i) {
      const int col = c0 + 64 * i + lane;
      w0[i] = (col < cpr && u0 < nv) ? __builtin_nontemporal_load(src0 + col) : z;
      w1[i] = (col < cpr && u1 < nv) ? __builtin_nontemporal_load(src1 + col) : z;
    }
#pragma unroll
    for (int i = 0; i < kCvtColBlk; ++i) {
      const int col = c0 + 64 * i + lane;
      // real rows only: the fine kernel's loads never reach padding rows
      // (a load's buffer range ends at its quarter's real rows)
      if (col < cpr && u0 < nv) dst0[col] = bf16x8_to_fp16x8(w0[i]);
      if (col < cpr && u1 < nv) dst1[col] = bf16x8_to_fp16x8(w1[i]);
      // largest |v| of the head's chunks in these two rows: reduce over the
      // cph lanes of each head (heads start at multiples of cph lanes)
      uint32_t m = max(bf16x8_absmax_bits(w0[i]), bf16x8_absmax_bits(w1[i]));
      for (int o = 1; o < cph; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
      red[wave][64 * i + lane] = m;
    }
    __syncthreads();
    // one lane per head of this pass combines the four waves
    const int heads = min(kCvtColBlk * 64, cpr - c0) / cph;
    if (wave == 0 && lane < heads) {
      const int t = lane * cph;
      const uint32_t m = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
      vm[c0 / cph + lane] = m;
    }
    __syncthreads();
  }
}

// grid (NH, B), 256 threads: e_h from the largest of the head's workgroup maxima.
__global__ __launch_bounds__(256) void vscale_kernel(const uint32_t* __restrict__ vmax,
                                                     int32_t* __restrict__ vexp, int n_wg, int NH) {
  __shared__ uint32_t red[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const uint32_t* __restrict__ vm = vmax + (size_t)b * n_wg * NH + h;
  uint32_t m = 0;
#pragma unroll 8  // several loads in flight per thread
  for (int i = threadIdx.x; i < n_wg; i += 256) m = max(m, vm[(size_t)i * NH]);
  for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float M = __uint_as_float(m);
    int e = 0;
    if (M > 65504.0f || (M > 0.0f && M < 0.0625f))
      e = min(max(ilogbf(M) - 14, kVexpMin), kVexpMax);
    vexp[(size_t)b * NH + h] = e;
  }
}

// grid (Nkv * kCvtSplit, B): the real rows of every head with e_h != 0,
// converted again with the scale 2^-e_h.
__global__ __launch_bounds__(kCvtThreads) void vfix_kernel(
    const uint32_t* __restrict__ v, uint32_t* __restrict__ v16, const int32_t* __restrict__ vbs,
    const int32_t* __restrict__ vexp, int Nkv, int NH, int D) {
  const int c = blockIdx.x / kCvtSplit, part = blockIdx.x % kCvtSplit, b = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  // the common case, no head of the batch scaled: one load per lane, leave
  bool any = false;
  for (int h0 = 0; h0 < NH; h0 += 64)
    any |= __builtin_amdgcn_ballot_w64(h0 + lane < NH && vexp[(size_t)b * NH + h0 + lane] != 0) != 0;
  if (!any) return;
  const int nv = min(max(vbs[c], 0), kCube);
  const int wpr = NH * D / 2;  // 32-bit words (bf16 pairs) per row
  for (int h = 0; h < NH; ++h) {
    const int e = vexp[(size_t)b * NH + h];
    if (e == 0) continue;
    for (int r = 0; r < kCube / kCvtSplit / 4; ++r) {
      const int u = part * (kCube / kCvtSplit) + r * 4 + wave;
      if (u >= nv) continue;
      const size_t row = ((size_t)b * Nkv + c) * kCube + u;
      for (int j = lane; j < D / 2; j += 64) {
        const size_t i = row * wpr + (size_t)h * (D / 2) + j;
        v16[i] = cvt2_fp16(v[i], e);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile list pre-pass: one wave per unit (b, h, query cube). The unit's
// selected ids (the first valid[unit] entries of its index row, or all of
// them; clamped into range: a violated precondition gives unspecified values,
// never an out-of-bounds access) are sorted ascending and every cube with
// real tokens is cut into quarters of at most 16 rows (ceil(vbs / 16) of
// them: rows 0-15, 16-31, ...). Consecutive quarters pair up into 32-row
// tiles, the unit of the fine kernel's loop: a cube of 16 or 8 real tokens
// shares its tile with the next cube's first quarter instead of leaving half
// a tile of padding (at the Wan shape this removes about 5% of the tiles).
// A quarter is one uint32: its byte offset from the head's first key row
// (a multiple of 16 row strides, so of 2048) OR its real-row count (1..16).
// Tile t = quarters 2t and 2t+1; an odd last quarter is paired with 0 (no
// rows), and kListPad all-zero tiles follow the last one. Rows with
// topk > kListSortCap keep the given order.
//
// With key-range splits (splits > 1, sorted rows only), the quarters of the
// cubes of split s (ids j with j * splits / Nkv == s) form tiles of their
// own: a split whose quarter count is odd ends with a zero quarter, so that
// no tile mixes two splits, and kListPad zero tiles follow every split.
// sbeg[unit][s] is the first tile of split s (of the list: s = 0) and
// sbeg[unit][splits] the end of the list, so split s has
// sbeg[s + 1] - sbeg[s] - kListPad tiles.
//
// Rotated sweeps (rank_of != NULL; sorted rows): the units resident
// on an XCD at one time are about kSweepWindow consecutive dispatch
// positions. Once their run times drift apart, units that started at
// different times sweep different parts of the key range, and their tiles
// stop sharing L2 lines. So a unit's ascending sweep starts at key id
// (p mod W) * Nkv / W, where p is its dispatch position on its XCD and
// W = kSweepWindow, and wraps around to the lower ids. A unit that starts
// when the one W positions earlier ends then meets the resident units at
// the same key position. On the Wan tensors this measured 3.85-3.91 ->
// 3.69 ms at top-78, 16.1-16.5 -> 14.3-14.5 ms at top-312 and 9.4 -> 8.6 ms
// at top-187. A row that selects every key cube (dense) keeps the plain
// sweep: such units never drift, and rotating them cost 5%. The rotation
// depends only on the row's ids, its count and the dispatch position, so a
// lookup-table row equal to a top-k row gives the same list. With key-range
// splits each split's sweep rotates the same way inside the split's range,
// by the item's own dispatch position.
constexpr int kListSortCap = 1024;
constexpr int kListRegSort = 256;  // rows up to this long sort in registers
constexpr int kListPad = 4;
constexpr int kQuarter = 16;  // rows per quarter
// fine-kernel units resident per XCD on MI355X: 32 CUs x 4 workgroups
constexpr int kSweepWindow = 128;

// Bitonic sort of 64 R keys held by one wave, key p = lane + 64 r in
// register r: a compare-exchange with a partner less than 64 positions away
// is a cross-lane swap (__shfl_xor), one 64 or more away is inside the lane.
// Ascending; no LDS and no barriers.
template <int R>
__device__ __forceinline__ void wave_bitonic_sort(int (&v)[R], int lane) {
#pragma unroll
  for (int size = 2; size <= 64 * R; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {
        const int rs = stride / 64;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & rs) continue;  // r is the lower position of its pair
          const int p = lane + 64 * r;
          const int a = v[r], c = v[r | rs];
          const bool asc = (p & size) == 0;
          v[r] = asc ? min(a, c) : max(a, c);
          v[r | rs] = asc ? max(a, c) : min(a, c);
        }
      } else {
        const bool lower = (lane & stride) == 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int p = lane + 64 * r;
          const int w = __shfl_xor(v[r], stride, 64);
          const bool take_min = lower == ((p & size) == 0);
          v[r] = take_min ? min(v[r], w) : max(v[r], w);
        }
      }
    }
  }
}

__global__ __launch_bounds__(64) void tiles_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ valid,
    const int32_t* __restrict__ vbs, uint32_t* __restrict__ list, int32_t* __restrict__ sbeg,
    int Nkv, int row_len, int stride, uint32_t rs2, int splits,
    const int32_t* __restrict__ rank_of, int Nq, int n_units) {
  __shared__ int32_t keys[kListSortCap];
  __shared__ int32_t qcount[kMaxSplits];  // quarters of split s
  __shared__ int32_t qpad[kMaxSplits];    // zero quarters placed before split s
  __shared__ int32_t qend[kMaxSplits];    // first quarter after split s's tiles
  __shared__ int32_t qbeg[kMaxSplits];    // first quarter of split s
  __shared__ int32_t qstart[kMaxSplits];  // key id split s's rotated sweep starts at
  __shared__ int32_t qbelow[kMaxSplits];  // quarters of split s below that id
  const int unit = blockIdx.x, lane = threadIdx.x;
  const int32_t* __restrict__ sel = topk_idx + (size_t)unit * row_len;
  // the row's first `topk` ids are used: all of them, or valid[unit] (clamped)
  const int topk = valid == nullptr ? row_len : min(max(valid[unit], 0), row_len);
  uint32_t* __restrict__ out = list + (size_t)unit * stride * 2;
  const bool sorted = topk <= kListSortCap;
  auto id_at = [&](int i) __attribute__((always_inline)) -> int {
    return min(max(sel[i], 0), Nkv - 1);
  };
  // rows of up to kListRegSort ids sort in registers (64, 128 or 256 keys,
  // padded with INT_MAX), longer ones through LDS
  auto reg_sort = [&](auto Rc) __attribute__((always_inline)) {
    constexpr int R = decltype(Rc)::value;
    int v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = lane + 64 * r < topk ? id_at(lane + 64 * r) : 0x7FFFFFFF;
    wave_bitonic_sort<R>(v, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) keys[lane + 64 * r] = v[r];
    __syncthreads();
  };
  if (sorted && topk <= 64) {
    reg_sort(std::integral_constant<int, 1>{});
  } else if (sorted && topk <= 128) {
    reg_sort(std::integral_constant<int, 2>{});
  } else if (sorted && topk <= kListRegSort) {
    reg_sort(std::integral_constant<int, 4>{});
  } else if (sorted) {
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
  int32_t* __restrict__ sb = sbeg + (size_t)unit * (splits + 1);
  auto split_of = [&](int id) __attribute__((always_inline)) -> int {
    return (int)(((int64_t)id * splits) / Nkv);
  };
  // dispatch position on its XCD of work item (unit, split sp): the items
  // run split-major inside each (b, h), in rank order, and xcd_remap hands
  // each XCD a contiguous range of them
  const bool rotate = rank_of != nullptr && sorted && topk > 0 && topk < Nkv;
  auto xcd_position = [&](int sp) __attribute__((always_inline)) -> int {
    const int n_items = n_units * splits;
    const int bh = unit / Nq;
    const int lin = (bh * splits + sp) * Nq + min(max(rank_of[unit], 0), Nq - 1);
    const int q8 = n_items / kNumXcd, r8 = n_items % kNumXcd;
    int x = 0;
    while (x < kNumXcd - 1 && lin >= (x + 1) * q8 + min(x + 1, r8)) ++x;
    return lin - (x * q8 + min(x, r8));
  };
  if (splits > 1) {  // the host allows splits only for sorted rows
    if (lane < kMaxSplits) {
      qcount[lane] = 0;
      qbelow[lane] = 0;
    }
    if (lane < splits) {  // split lane: ids [lo, hi); its sweep starts inside
      const int lo = (int)(((int64_t)lane * Nkv + splits - 1) / splits);
      const int hi = (int)(((int64_t)(lane + 1) * Nkv + splits - 1) / splits);
      qstart[lane] = rotate ? lo + (int)(((int64_t)(xcd_position(lane) % kSweepWindow) *
                                          (hi - lo)) / kSweepWindow)
                            : lo;
    }
    __syncthreads();
    for (int i = lane; i < topk; i += 64) {
      const int id = keys[i];
      const int nv = min(max(vbs[id], 0), kCube);
      const int sp = split_of(id), nq = (nv + kQuarter - 1) / kQuarter;
      atomicAdd(&qcount[sp], nq);
      if (id < qstart[sp]) atomicAdd(&qbelow[sp], nq);
    }
    __syncthreads();
    if (lane == 0) {
      int pad = 0, start = 0;  // start: first quarter of split s
      for (int sp = 0; sp < splits; ++sp) {
        const int qn = qcount[sp];
        qpad[sp] = pad;
        qbeg[sp] = start;
        sb[sp] = start / 2;
        qend[sp] = start + qn + (qn & 1);
        pad += (qn & 1) + 2 * kListPad;
        start = qend[sp] + 2 * kListPad;
      }
      sb[splits] = start / 2;
    }
    __syncthreads();
    // an odd split's completing zero quarter, then the split's zero tiles
    for (int sp = 0; sp < splits; ++sp)
      if (lane < 2 * kListPad + 1 && (lane > 0 || (qcount[sp] & 1)))
        out[qend[sp] - 1 + lane] = 0u;
  }
  // rotated sweep: the list starts at sorted position k0, the first id at
  // or above the unit's start key id
  int k0 = 0;
  if (rotate && splits == 1) {
    const int start = (int)(((int64_t)(xcd_position(0) % kSweepWindow) * Nkv) / kSweepWindow);
    int below_start = 0;
    for (int i = lane; i < topk; i += 64) below_start += keys[i] < start;
    for (int o = 32; o > 0; o >>= 1) below_start += __shfl_xor(below_start, o, 64);
    k0 = below_start == topk ? 0 : below_start;
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base = 0;  // quarters written so far, without the zero quarters
  for (int c0 = 0; c0 < topk; c0 += 64) {
    const int i = c0 + lane;
    int id = 0, nv = 0;
    if (i < topk) {
      id = sorted ? keys[k0 == 0 ? i : (i + k0) % topk] : id_at(i);
      nv = min(max(vbs[id], 0), kCube);
    }
    const int nq = (nv + kQuarter - 1) / kQuarter;  // 0..4
    const int sp = splits > 1 && i < topk ? split_of(id) : 0;
    int pos = base + (splits > 1 && i < topk ? qpad[sp] : 0), tot = 0;
#pragma unroll
    for (int k = 1; k <= kCube / kQuarter; ++k) {
      const uint64_t bk = __builtin_amdgcn_ballot_w64(nq >= k);
      pos += __builtin_popcountll(bk & below);
      tot += __builtin_popcountll(bk);
    }
    // split sp's quarters in rotated order: the cube's offset inside the
    // split, less the quarters below the split's start id, modulo the split
    if (splits > 1 && nq > 0 && qbelow[sp] > 0)
      pos = qbeg[sp] + (pos - qbeg[sp] - qbelow[sp] + qcount[sp]) % qcount[sp];
    const uint32_t off0 = (uint32_t)id * (uint32_t)kCube * rs2;
    for (int k = 0; k < nq; ++k)
      out[pos + k] = (off0 + (uint32_t)(kQuarter * k) * rs2) | (uint32_t)min(nv - kQuarter * k, kQuarter);
    base += tot;
  }
  if (splits > 1) return;
  const int n_tiles = (base + 1) / 2;
  if (lane == 0 && (base & 1)) out[base] = 0u;
  if (lane < 2 * kListPad) out[2 * n_tiles + lane] = 0u;
  if (lane == 0) {
    sb[0] = 0;
    sb[1] = n_tiles + kListPad;
  }
}

// Dispatch order inside each (b, h): query cubes by descending count of
// selected cubes, then by ascending smallest selected id, then by cube id.
// Units that run side by side then sweep the ascending key ids from nearby
// starting points at similar rates, so their tile loads keep hitting the
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
    const uint64_t* __restrict__ keys, int32_t* __restrict__ order, int32_t* __restrict__ rank_of,
    int Nq) {
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
  rank_of[base + i] = rank;
}

// ---------------------------------------------------------------------------
// kStats: the row statistics (lse, max_prob) are written; the plain forward
// skips the bookkeeping of the exact row maximum that only max_prob needs.
template <int D, bool kStats>
__global__ __launch_bounds__(FwdShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v16, const uint32_t* __restrict__ list,
    const int32_t* __restrict__ sbeg, const int32_t* __restrict__ order,
    const int32_t* __restrict__ vexp, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ max_prob, float* __restrict__ part, float4* __restrict__ pstat,
    int Nq, int Nkv, int NH, int list_stride, float scale_log2, int splits, int n_items) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][S::kTileBytes];

  // XCD x runs a contiguous range of (b, h, split, rank); within a (b, h)
  // the query cube of a rank is the rank itself, or order[]
  const int lin = xcd_remap(blockIdx.x, n_items);
  const int bh = lin / (Nq * splits);
  const int rem = lin - bh * Nq * splits;
  const int sp = rem / Nq, rank = rem - sp * Nq;
  const int qc = order == nullptr ? rank : min(max(order[bh * Nq + rank], 0), Nq - 1);
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

  // ---- the tiles (two quarters each) of this unit's split: n tiles from
  // tile t0 of the unit's list; reads past them (i >= n) see the split's
  // all-zero padding tiles (i < n + kListPad), whose loads fetch nothing
  const int32_t* __restrict__ sb = sbeg + (size_t)unit * (splits + 1) + sp;
  const int t0 = __builtin_amdgcn_readfirstlane(sb[0]);
  const int n = __builtin_amdgcn_readfirstlane(sb[1]) - t0 - kListPad;
  const uint32_t* __restrict__ lst = list + (size_t)unit * list_stride * 2 + 2 * (size_t)t0;
  auto ent = [&](int i) __attribute__((always_inline)) -> u32x2 {
    const u32x2 v = *reinterpret_cast<const u32x2*>(lst + 2 * __builtin_amdgcn_readfirstlane(i));
    return u32x2{(uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)v[1])};
  };
  // per-row statistics: row (b, h, c * 64 + 32 wave + qr), written by lane g = 0
  const size_t srow = ((size_t)bh * Nq + qc) * kCube + 32 * wave + qr;
  if (n == 0) {  // no real key in any selected cube: the rows are 0
    if (splits > 1) return;  // the merge skips empty splits
#pragma unroll
    for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * g) = u32x2{0u, 0u};
    if (g == 0 && lse != nullptr) lse[srow] = kNegInf;
    if (g == 0 && max_prob != nullptr) max_prob[srow] = 0.0f;
    return;
  }

  // ---- loads: wave w fills KiB [L w, L w + L) of every tile buffer
  // (L = kLoads), i.e. tile rows [16 w, 16 w + 16): quarter w of the tile;
  // lane L' writes bytes [16 L', 16 L' + 16) of a KiB and fetches the global
  // chunk that the swizzle places in that slot. Byte offsets stay below 2^32
  // (host-checked).
  constexpr int L = S::kLoads;
  const uint32_t rs2 = (uint32_t)NH * D * 2u;
  uint32_t koff[L], voff[L];
#pragma unroll
  for (int m = 0; m < L; ++m) {
    // LDS row of the tile, and its row inside this wave's quarter (the
    // descriptor's base is the quarter's first row)
    const int row = (wave * L + m) * S::kRowsPerKiB + lane / S::kChunks;
    const int qrow = row - kQuarter * wave;
    const int slot = lane % S::kChunks;
    koff[m] = (uint32_t)qrow * rs2 + 16u * (uint32_t)(slot ^ swz_k<D>(row)) - 1024u * (m & 1);
    voff[m] = (uint32_t)qrow * rs2 + 16u * (uint32_t)(slot ^ swz_v<D>(row)) - 1024u * (m & 1);
  }
  const uint32_t lds_wave = (uint32_t)(wave * L) * 1024u;
  const size_t kv_head = (size_t)b * Nkv * kCube * row_stride + (size_t)h * D;
  const uint64_t kbase = reinterpret_cast<uint64_t>(k + kv_head);
  const uint64_t vbase = reinterpret_cast<uint64_t>(v16 + kv_head);
  // gfx9 raw buffer descriptor of this wave's quarter of a tile: base +
  // offset, range = its real rows (the loads of padding rows and of empty
  // quarters return zeros)
  auto mk_rsrc = [&](uint64_t base, const u32x2& e) __attribute__((always_inline)) -> int32x4_t {
    const uint32_t qw = wave ? e[1] : e[0];
    const uint64_t a = base + (qw & ~31u);
    int32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)((qw & 31u) * rs2));
    r[3] = kBufferDword3;
    return r;
  };
  const uint32_t kb0 = lds_address(kbuf), vb0 = lds_address(vbuf);
  // load pair p (0 <= p < L / 2) of a tile into buffer `buf`
  auto dma_k = [&](const int32x4_t& r, int buf, int p) __attribute__((always_inline)) {
    dma16x2(r, koff[2 * p], koff[2 * p + 1], kb0 + (uint32_t)buf * S::kTileBytes + lds_wave + 2048u * p);
  };
  auto dma_v = [&](const int32x4_t& r, int buf, int p) __attribute__((always_inline)) {
    dma16x2(r, voff[2 * p], voff[2 * p + 1], vb0 + (uint32_t)buf * S::kTileBytes + lds_wave + 2048u * p);
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
  // a tile max above m_lim = m_ref + kRescaleThreshold / c raises m_ref
  float m_lim = kNegInf;
  float m_row = kNegInf;  // the row's largest score so far (for max_prob)
  bool need_rescale = false;
  const floatx16 zero16 = {};
  const halfx2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // S^T = K Q^T for the tile in K buffer kbi; V load pairs ride along
  auto qk = [&](int kbi, floatx16& s, const int32x4_t& vr, int vbi) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < S::kQSteps; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl[st] + kbi * S::kTileBytes);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? zero16 : s, 0, 0, 0);
      if (vbi >= 0 && st % 2 == 1 && st / 2 < L / 2) dma_v(vr, vbi, st / 2);
    }
  };
  // O^T += V^T P^T for the tile in V buffer vbi; K load pairs ride along
  auto pv = [&](int vbi, const halfx8 (&pb)[2], const int32x4_t& kr, int kbi) __attribute__((always_inline)) {
    constexpr int NSTEP = 2 * S::kDBlocks;  // (kk, db)
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st / S::kDBlocks, db = st % S::kDBlocks;
      const uint8_t* p0 = vl[db] + vbi * S::kTileBytes + kk * 16 * S::kRowBytes;
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p0)));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_ptr)(p0 + 8 * S::kRowBytes)));
      const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), pb[kk], oacc[db], 0, 0, 0);
      if (kbi >= 0 && st % 2 == 1 && st / 2 < L / 2) dma_k(kr, kbi, st / 2);
    }
  };
  // tokens past the real rows of their quarter set to -inf (tiles with a
  // partial quarter only; the asm keeps the compiler from flattening the
  // branch into selects that every tile would execute), row max, lazy raise
  // of the reference max (wave-uniform decision). Accumulator entry r holds
  // token 8 (r / 4) + 4 g + r % 4: entries 0-7 lie in quarter 0 (tokens
  // 0-15), entries 8-15 in quarter 1.
  auto mask_max = [&](const u32x2& e, floatx16& s) __attribute__((always_inline)) {
    const uint32_t na = e[0] & 31u, nb = e[1] & 31u;
    if ((na & nb) < (uint32_t)kQuarter) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t tok = 8 * (r >> 2) + 4 * g + (r & 3);
        if (r < 8 ? tok >= na : tok - kQuarter >= nb) s[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    if (kStats) m_row = fmaxf(m_row, mx);
    const bool up = mx > m_lim;
    need_rescale = __builtin_amdgcn_ballot_w64(up) != 0;
    if (need_rescale) {  // rare: a real branch (the asm keeps it from being flattened)
      asm volatile("");
      const float m_new = up ? mx : m_ref;
      alpha = m_ref == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
      m_ref = m_new;
      m_lim = m_ref + kRescaleThreshold / scale_log2;
      l_run *= alpha;
    }
  };
  // P in fp16 (round to nearest even) and the row sums of the same rounded
  // values (v_dot2_f32_f16 against 1.0). Every row has a finite m_ref here:
  // the first tile of a unit holds at least one real token.
  auto exp_sum = [&](const floatx16& s, halfx8 (&pb)[2]) __attribute__((always_inline)) {
    const float mc = m_ref * scale_log2 - kPShift;
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
    mask_max(e0, sA);
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
    mask_max(e_n1, sn);
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

  // ---- with key-range splits: the partial result of this split, O
  // unnormalised (fp32, [item][row][D]) and (m_ref, l_run, m_row) per row
  if (splits > 1) {
    const size_t item = (size_t)unit * splits + sp;
    const int row = 32 * wave + qr;
    float* __restrict__ po = part + (item * kCube + row) * D;
#pragma unroll
    for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * r4 + 4 * g) =
            float4{oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2],
                   oacc[db][4 * r4 + 3]};
    if (g == 0) pstat[item * kCube + row] = float4{m_ref, l_run, m_row, 0.0f};
    return;
  }

  // ---- per-row statistics. l_run sums exp2((s - m_ref) c + kPShift), so the
  // natural log-sum-exp of the scaled scores is (m_ref c - kPShift +
  // log2 l_run) ln 2, and the largest softmax weight is
  // 1 / sum exp2((s - m_row) c) = exp2((m_row - m_ref) c + kPShift) / l_run.
  if (g == 0 && lse != nullptr)
    lse[srow] = (m_ref * scale_log2 - kPShift + __log2f(l_run)) * 0.69314718055994531f;
  if (kStats && g == 0 && max_prob != nullptr)
    max_prob[srow] = __builtin_amdgcn_exp2f((m_row - m_ref) * scale_log2 + kPShift) / l_run;

  // ---- epilogue: lane holds O^T[d][row] for d = 32 db + 8 (r/4) + 4 g + r%4;
  // V entered the product scaled by 2^-e_h (0 for heads in fp16's range)
  const int ve = vexp == nullptr ? 0 : vexp[bh];
  const float inv_l = l_run > 0.0f ? ldexpf(1.0f / l_run, ve) : 0.0f;
#pragma unroll
  for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x2 w = {pack_bf16x2(oacc[db][4 * r4] * inv_l, oacc[db][4 * r4 + 1] * inv_l),
                       pack_bf16x2(oacc[db][4 * r4 + 2] * inv_l, oacc[db][4 * r4 + 3] * inv_l)};
      *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * g) = w;
    }
}

// ---------------------------------------------------------------------------
// Merge of the key-range splits: one workgroup of 256 threads per unit (b, h,
// query cube). With M the largest reference max over a row's non-empty
// splits and w_s = exp2((m_s - M) c), O = sum_s w_s O_s and l = sum_s w_s l_s
// (the online-softmax combination of partial states), out = O / l * 2^e_h
// rounded to bf16, and the statistics are the unsplit epilogue's with (M, l)
// and the largest row max. The kernel is bound by reading the partial
// states, so their reads are coalesced: an item's partial O (64 rows of D
// fp32) is read as float4 j = t + 256 i by thread t, consecutive threads on
// consecutive 16 bytes; thread t thus combines columns 4 (t % (D/4)) .. + 3
// of rows t / (D/4) + (1024 / D) i. kS > 0: exactly kS splits (their loads
// unrolled); kS = 0: any count.
template <int D, int kS>
__global__ __launch_bounds__(256) void merge_kernel(
    const float* __restrict__ part, const float4* __restrict__ pstat,
    const int32_t* __restrict__ sbeg, const int32_t* __restrict__ vexp,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ max_prob, int Nq,
    int NH, int splits, float scale_log2) {
  constexpr int kF4 = D / 4;             // float4 per row
  constexpr int kRowStep = 256 / kF4;    // rows apart between a thread's rows
  constexpr int kRows = kCube / kRowStep;  // rows per thread
  const int unit = blockIdx.x;
  const int bh = unit / Nq, qc = unit - bh * Nq, h = bh % NH, b = bh / NH;
  const int col4 = threadIdx.x % kF4, row0 = threadIdx.x / kF4;
  const int nsp = kS > 0 ? kS : splits;
  const int32_t* __restrict__ sb = sbeg + (size_t)unit * (nsp + 1);
  const float4* __restrict__ pst = pstat + (size_t)unit * nsp * kCube;
  const float4* __restrict__ po = reinterpret_cast<const float4*>(part) + (size_t)unit * nsp *
                                                                             kCube * kF4;
  float M[kRows], m_row[kRows], l[kRows];
  float4 acc[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    M[i] = kNegInf;
    m_row[i] = kNegInf;
    l[i] = 0.0f;
    acc[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // the row maxima, then the weighted sums
#pragma unroll 4
  for (int sp = 0; sp < nsp; ++sp) {
    if (sb[sp + 1] - sb[sp] == kListPad) continue;  // an empty split
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const float4 st = pst[sp * kCube + row0 + kRowStep * i];
      M[i] = fmaxf(M[i], st.x);
      m_row[i] = fmaxf(m_row[i], st.z);
    }
  }
#pragma unroll 4
  for (int sp = 0; sp < nsp; ++sp) {
    if (sb[sp + 1] - sb[sp] == kListPad) continue;
    float4 x[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) x[i] = po[(size_t)sp * kCube * kF4 + threadIdx.x + 256 * i];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const float4 st = pst[sp * kCube + row0 + kRowStep * i];
      const float w = __builtin_amdgcn_exp2f((st.x - M[i]) * scale_log2);
      l[i] = __builtin_fmaf(w, st.y, l[i]);
      acc[i].x = __builtin_fmaf(w, x[i].x, acc[i].x);
      acc[i].y = __builtin_fmaf(w, x[i].y, acc[i].y);
      acc[i].z = __builtin_fmaf(w, x[i].z, acc[i].z);
      acc[i].w = __builtin_fmaf(w, x[i].w, acc[i].w);
    }
  }
  const int ve = vexp == nullptr ? 0 : vexp[bh];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int row = row0 + kRowStep * i;
    const size_t srow = (size_t)unit * kCube + row;
    if (col4 == 0) {
      if (lse != nullptr)
        lse[srow] = l[i] > 0.0f
                        ? (M[i] * scale_log2 - kPShift + __log2f(l[i])) * 0.69314718055994531f
                        : kNegInf;
      if (max_prob != nullptr)
        max_prob[srow] = l[i] > 0.0f ? __builtin_amdgcn_exp2f((m_row[i] - M[i]) * scale_log2 +
                                                              kPShift) / l[i]
                                     : 0.0f;
    }
    const float inv_l = l[i] > 0.0f ? ldexpf(1.0f / l[i], ve) : 0.0f;
    uint16_t* __restrict__ orow = out + (((size_t)b * Nq + qc) * kCube + row) * (size_t)NH * D +
                                  (size_t)h * D + 4 * col4;
    *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(acc[i].x * inv_l, acc[i].y * inv_l),
                                            pack_bf16x2(acc[i].z * inv_l, acc[i].w * inv_l)};
  }
}

}  // namespace

// Key-range splits of the fine stage (split-KV). The units of a head that
// run side by side on an XCD sweep that head's keys; once one head's K and
// fp16 V exceed about 32 MiB (a few times the XCD's 4 MiB L2) their tiles are
// evicted before the other units reach them, and the kernel fetches many
// times its algorithmic bytes from beyond L2 (measured at the 720p shape
// before rotated sweeps: 65x, 29% L2 hits, 7.3 TB/s). Split into S key
// ranges of about 32 MiB, run split-major inside each head, the resident
// units share one range; each item leaves a partial state that merge_kernel
// combines. Measured at the 720p shape (63 MB per head) with rotated sweeps:
// S = 1 21.6 ms, 2 20.9, 3 21.2, 4 21.7, 8 24.1 (every split adds a partial
// state per unit). forced: 0 chooses, 1 turns splitting off, 2..kMaxSplits
// forces S. Rows longer than the sorted list pre-pass allows (kListSortCap
// ids) are never split.
int fwd_splits(int Nkv, int D, int topk, int forced) {
  if (topk > kListSortCap) return 1;
  if (forced > 0) return forced < kMaxSplits ? forced : kMaxSplits;
  const double kv_head = (double)Nkv * kCube * D * 4.0;  // K bf16 + V fp16
  const double mib = 1024.0 * 1024.0;
  if (kv_head <= 32.0 * mib) return 1;
  int sp = (int)ceil(kv_head / (32.0 * mib));
  sp = sp < topk / 8 ? sp : topk / 8;  // at least 8 selected cubes per item on average
  return sp < 2 ? 1 : (sp < kMaxSplits ? sp : kMaxSplits);
}

FwdWorkspace fwd_workspace(int B, int Nq, int Nkv, int NH, int D, int topk, int forced) {
  auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
  FwdWorkspace w;
  w.splits = fwd_splits(Nkv, D, topk, forced);
  // tiles per unit: at most 4 quarters per cube, two per tile, then
  // kListPad zero tiles; with splits a zero quarter and kListPad zero tiles
  // per split
  w.list_stride = 2 * topk + kListPad + (w.splits > 1 ? w.splits * (kListPad + 1) : 0);
  const size_t units = (size_t)B * NH * Nq;
  w.v16_off = 0;
  w.list_off = up((size_t)B * Nkv * kCube * NH * D * 2);
  w.sbeg_off = w.list_off + up(units * w.list_stride * 8);
  w.order_off = w.sbeg_off + up(units * (w.splits + 1) * 4);
  w.rank_off = w.order_off + up(units * 4);
  w.key_off = w.rank_off + up(units * 4);
  w.vmax_off = w.key_off + up(units * 8);
  w.vexp_off = w.vmax_off + up((size_t)B * Nkv * kCvtSplit * NH * 4);
  w.part_off = w.vexp_off + up((size_t)B * NH * 4);
  const size_t items = w.splits > 1 ? units * w.splits : 0;
  w.pstat_off = w.part_off + up(items * kCube * D * 4);
  w.total = w.pstat_off + up(items * kCube * 16);
  return w;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* valid, const int32_t* vbs,
                      uint16_t* out, float* lse, float* max_prob, int B, int Nq, int Nkv,
                      int NH, int D, int topk, float sm_scale, int forced_splits,
                      void* workspace, hipStream_t stream) {
  const FwdWorkspace w = fwd_workspace(B, Nq, Nkv, NH, D, topk, forced_splits);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + w.v16_off);
  uint32_t* list = reinterpret_cast<uint32_t*>(ws + w.list_off);
  int32_t* sbeg = reinterpret_cast<int32_t*>(ws + w.sbeg_off);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float4* pstat = reinterpret_cast<float4*>(ws + w.pstat_off);
  const int splits = w.splits;
  uint32_t* vmax = reinterpret_cast<uint32_t*>(ws + w.vmax_off);
  int32_t* vexp = reinterpret_cast<int32_t*>(ws + w.vexp_off);
  int32_t* order = nullptr;
  int32_t* rank_of = nullptr;
  const int n_units = B * NH * Nq;
  hipLaunchKernelGGL(v_to_fp16_kernel, dim3(Nkv * kCvtSplit, B), dim3(kCvtThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(v16), vbs, vmax,
                     Nkv, NH, D / 8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vscale_kernel, dim3(NH, B), dim3(256), 0, stream, vmax, vexp,
                     Nkv * kCvtSplit, NH);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vfix_kernel, dim3(Nkv * kCvtSplit, B), dim3(kCvtThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(v), reinterpret_cast<uint32_t*>(v16), vbs,
                     vexp, Nkv, NH, D);
  e = hipGetLastError();
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
    rank_of = reinterpret_cast<int32_t*>(ws + w.rank_off);
    hipLaunchKernelGGL(order_rank_kernel, dim3(B * NH, (Nq + kOrderThreads - 1) / kOrderThreads),
                       dim3(kOrderThreads), (size_t)Nq * sizeof(uint64_t), stream, keys, order,
                       rank_of, Nq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tiles_kernel, dim3(n_units), dim3(64), 0, stream, topk_idx, valid, vbs,
                     list, sbeg, Nkv, topk, w.list_stride, (uint32_t)NH * D * 2u, splits,
                     rank_of, Nq, n_units);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  const bool stats = lse != nullptr || max_prob != nullptr;
  const int n_items = n_units * splits;
#define VSA_FWD_LAUNCH(DD, ST)                                                                  \
  hipLaunchKernelGGL((fwd_kernel<DD, ST>), dim3(n_items), dim3(FwdShape<DD>::kThreads), 0, stream, \
                     q, k, v16, list, sbeg, order, vexp, out, lse, max_prob, part, pstat, Nq,    \
                     Nkv, NH, w.list_stride, scale_log2, splits, n_items)
  if (D == 128) {
    if (stats) VSA_FWD_LAUNCH(128, true);
    else VSA_FWD_LAUNCH(128, false);
  } else {
    if (stats) VSA_FWD_LAUNCH(64, true);
    else VSA_FWD_LAUNCH(64, false);
  }
#undef VSA_FWD_LAUNCH
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
#define VSA_MERGE_LAUNCH(DD, SS)                                                          \
  hipLaunchKernelGGL((merge_kernel<DD, SS>), dim3(n_units), dim3(256), 0, stream, part, pstat, \
                     sbeg, vexp, out, lse, max_prob, Nq, NH, splits, scale_log2)
#define VSA_MERGE_D(DD)                           \
  switch (splits) {                               \
    case 2: VSA_MERGE_LAUNCH(DD, 2); break;       \
    case 3: VSA_MERGE_LAUNCH(DD, 3); break;       \
    case 4: VSA_MERGE_LAUNCH(DD, 4); break;       \
    default: VSA_MERGE_LAUNCH(DD, 0); break;      \
  }
  if (D == 128) {
    VSA_MERGE_D(128)
  } else {
    VSA_MERGE_D(64)
  }
#undef VSA_MERGE_D
#undef VSA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace vsa
