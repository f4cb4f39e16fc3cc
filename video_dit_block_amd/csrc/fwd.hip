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
//   (2) per pair of neighbouring query cubes (2j, 2j+1) of one (b, h), the
//   sorted union of their selected cube ids, expanded into a list of 32-token
//   half-tiles: half 0 of every cube with a real token, half 1 of every cube
//   with more than 32. Each entry packs the cube id, which of the two query
//   cubes selected it, the half and its real-row count. Neighbouring query
//   cubes select overlapping sets (about a quarter of a pair's half-tiles are
//   shared on video workloads), and a shared half-tile is loaded once for
//   both. The result does not depend on the order of topk_idx; the ascending
//   sweep makes the pairs resident on one XCD walk their head's key/value
//   cubes in the same order, which keeps them in that XCD's L2, and no half
//   without real tokens is touched.
// * One workgroup = one pair: 4 waves of 32 query rows (waves 0-1 the first
//   query cube, 2-3 the second), 2 workgroups per CU. Pairs are numbered
//   head-major and remapped so each XCD walks a contiguous range.
// * The pair's half-tiles stream through LDS, K and V each double-buffered
//   (2 x 2 x 8 KiB at D = 128), loaded global -> LDS directly
//   (buffer_load ... lds), every wave loading a quarter of each half-tile:
//   V of half-tile i+1 streams in during QK^T of half-tile i, K of half-tile
//   i+2 during PV of half-tile i, each tile's DMAs spread one per MFMA step.
//   That gives every load well over a half-tile's compute of lead, which the
//   L2/MALL latency under load needs. The waves of a query cube that did not
//   select half-tile i only issue its loads and pass the barriers. The
//   buffer range of a load ends at the half's real rows, so padding rows land
//   as zeros: pad values (even NaN) never reach an MFMA, with no branch.
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
// * fp32 online softmax in the exp2 domain, one step per half-tile:
//   p = exp2(s * c - m * c) with c = sm_scale * log2 e (one FMA per score),
//   running reference max m, running sum l. The reference max is raised
//   lazily: only when a half's row max exceeds it by more than 2^8 (log2
//   units: 8) does the wave rescale O and l by exp2((m_old - m_new) c);
//   otherwise p may reach 2^8, which fp32 and fp16 hold exactly in range. A
//   fully masked row keeps m = -inf and uses 0 in the subtraction, so no
//   (-inf) - (-inf) arises. Tokens past a half's real rows are set to -inf in
//   registers before the max (partial halves only). O^T accumulates in fp32,
//   each lane holding D/2 values of its own query row, so the rescale is a
//   per-lane multiply.
// * Precision: QK^T is a bf16 MFMA with fp32 accumulation. The PV product
//   runs as an fp16 MFMA (v_mfma_f32_32x32x16_f16): P is rounded to fp16 and
//   V is converted to fp16 by the pre-pass. fp16 keeps 3 more
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
constexpr int kHalf = 32;  // tokens per half-tile

template <int D>
struct FwdShape {
  static constexpr int kThreads = 256;                  // 2 query cubes x 2 waves x 32 rows
  static constexpr int kRowBytes = 2 * D;               // one (token, head) row
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;  // rows one wave-wide DMA fills
  static constexpr int kHalfBytes = kHalf * kRowBytes;  // one tensor of one half-tile
  static constexpr int kLoads = kHalfBytes / 1024 / 4;  // DMAs per wave per tensor and half-tile
  static constexpr int kQSteps = D / 16;                // k-steps of the QK^T MFMAs
  static constexpr int kDBlocks = D / 32;               // 32-wide d blocks of O^T
  // a half-tile's DMAs are spread over the first kLoads MFMA steps of QK / PV
  static_assert(kLoads <= kQSteps && kLoads <= 2 * kDBlocks, "DMA spread");
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
// Step list pre-pass: one workgroup per pair of neighbouring query cubes
// (2j, 2j+1) of one (b, h). The two index rows are merged into their sorted
// union, each cube expanded into its 32-token half-tiles (half 0 if it has a
// real token, half 1 if it has more than 32), and the half-tiles are
// scheduled into steps of two slots (X for cube 2j, Y for cube 2j+1):
//   * a half-tile both cubes selected gets a step of its own, in both slots
//     (loaded once, used by all four waves);
//   * the k-th half-tile only cube 2j selected and the k-th only cube 2j+1
//     selected share a step (X and Y), so neither wave pair idles while the
//     other works; a side with fewer such half-tiles gets empty slots.
// Entry layout (uint32): (cube id << 8) | kValid | (half << 5) | (real rows
// of the half - 1); 0 is an empty slot. Steps are stored as (X, Y) pairs;
// kStepPad empty steps follow the last one so the fine kernel may read a few
// steps past the end. Rows with 2 topk > kListSortCap keep the given order
// and share nothing (all their half-tiles are one-sided).
constexpr int kListThreads = 256;
constexpr int kListSortCap = 4096;
constexpr int kStepPad = 8;
constexpr uint32_t kValid = 1u << 7;

__global__ __launch_bounds__(kListThreads) void steps_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ vbs,
    uint32_t* __restrict__ steps, int32_t* __restrict__ counts, int Nq, int Nkv, int topk,
    int stride, int n_pairs_q) {
  __shared__ int32_t keys[kListSortCap];
  __shared__ int32_t part[3][kListThreads / 64];
  const int pair = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int bh = pair / n_pairs_q, qc0 = 2 * (pair % n_pairs_q);
  const int32_t* __restrict__ sel = topk_idx + ((size_t)bh * Nq + qc0) * topk;
  uint32_t* __restrict__ out = steps + (size_t)pair * stride * 2;
  const int n = (qc0 + 1 < Nq ? 2 : 1) * topk;  // ids of both rows, row 2j first
  const bool sorted = n <= kListSortCap;
  // Ids are clamped into range: a violated precondition gives unspecified
  // values, never an out-of-bounds access. Key = (id << 1) | row.
  auto key_at = [&](int i) __attribute__((always_inline)) -> int {
    return (min(max(sel[i], 0), Nkv - 1) << 1) | (i >= topk ? 1 : 0);
  };
  if (sorted) {
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = tid; i < n2; i += kListThreads) keys[i] = i < n ? key_at(i) : 0x7FFFFFFF;
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride2 = size >> 1; stride2 > 0; stride2 >>= 1) {
        __syncthreads();
        for (int t = tid; t < (n2 >> 1); t += kListThreads) {
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
  // Two passes over the merged list: the first counts the half-tiles of each
  // class (1: cube 2j only, 2: cube 2j+1 only, 3: both), the second writes
  // them at their step. In sorted order a cube both rows selected appears as
  // (id, 0), (id, 1): the first of a run of equal ids carries the run's flags.
  int total[4] = {0, 0, 0, 0};
  for (int pass = 0; pass < 2; ++pass) {
    int base[4] = {0, 0, 0, 0};
    for (int c0 = 0; c0 < n; c0 += kListThreads) {
      const int i = c0 + tid;
      int id = 0, nv = 0, cls = 0;
      if (i < n) {
        const int key = sorted ? keys[i] : key_at(i);
        id = key >> 1;
        const bool head = !sorted || i == 0 || (keys[i - 1] >> 1) != id;
        if (head) {
          cls = 1 << (key & 1);
          if (sorted && i + 1 < n && (keys[i + 1] >> 1) == id) cls |= 1 << (keys[i + 1] & 1);
          nv = min(max(vbs[id], 0), kCube);
        }
      }
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int pre = 0;
#pragma unroll
      for (int c = 1; c <= 3; ++c) {
        const uint64_t b1 = __builtin_amdgcn_ballot_w64(cls == c && nv > 0);
        const uint64_t b2 = __builtin_amdgcn_ballot_w64(cls == c && nv > kHalf);
        if (cls == c) pre = __builtin_popcountll(b1 & below) + __builtin_popcountll(b2 & below);
        if (lane == 0) part[c - 1][wave] = __builtin_popcountll(b1) + __builtin_popcountll(b2);
      }
      __syncthreads();
      int off = 0, chunk[4] = {0, 0, 0, 0};
      for (int w = 0; w < kListThreads / 64; ++w) {
#pragma unroll
        for (int c = 1; c <= 3; ++c) {
          chunk[c] += part[c - 1][w];
          if (c == cls && w < wave) off += part[c - 1][w];
        }
      }
      if (pass == 1 && nv > 0) {
        const uint32_t tag = ((uint32_t)id << 8) | kValid;
        const int r = base[cls] + off + pre;  // rank of half 0 within its class
        const int s = cls == 3 ? r : total[3] + r;
        const int slot = cls == 2 ? 1 : 0;
        const uint32_t e0 = tag | (uint32_t)(min(nv, kHalf) - 1);
        const uint32_t e1 = tag | (1u << 5) | (uint32_t)(nv - kHalf - 1);
        if (cls == 3) {
          out[2 * s] = e0;
          out[2 * s + 1] = e0;
          if (nv > kHalf) {
            out[2 * s + 2] = e1;
            out[2 * s + 3] = e1;
          }
        } else {
          out[2 * s + slot] = e0;
          if (nv > kHalf) out[2 * s + 2 + slot] = e1;
        }
      }
#pragma unroll
      for (int c = 1; c <= 3; ++c) base[c] += chunk[c];
      __syncthreads();
    }
    if (pass == 0) {
#pragma unroll
      for (int c = 1; c <= 3; ++c) total[c] = base[c];
    }
  }
  // empty slots on the shorter one-sided list, then the padding steps
  const int n_one = max(total[1], total[2]);
  const int n_steps = total[3] + n_one;
  for (int r = total[1] + tid; r < n_one; r += kListThreads) out[2 * (total[3] + r)] = 0u;
  for (int r = total[2] + tid; r < n_one; r += kListThreads) out[2 * (total[3] + r) + 1] = 0u;
  for (int i = tid; i < 2 * kStepPad; i += kListThreads) out[2 * n_steps + i] = 0u;
  if (tid == 0) counts[pair] = n_steps;
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(FwdShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v16, const uint32_t* __restrict__ steps,
    const int32_t* __restrict__ counts, uint16_t* __restrict__ out, int Nq, int Nkv,
    int NH, int step_stride, float scale_log2, int n_pairs, int n_pairs_q) {
  using S = FwdShape<D>;
  // [buffer][slot X / Y][half-tile]
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][2][S::kHalfBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][S::kHalfBytes];

  const int pair = xcd_remap(blockIdx.x, n_pairs);
  const int bh = pair / n_pairs_q;
  const int h = bh % NH, b = bh / NH;
  const size_t row_stride = (size_t)NH * D;  // elements between tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = wave >> 1;  // which query cube of the pair this wave serves (slot X / Y)
  const int qc = 2 * (pair % n_pairs_q) + sub;
  const bool real_q = qc < Nq;  // false for the second cube of an odd tail
  const int qr = lane & 31, g = lane >> 5;
  const size_t qrow_idx = (size_t)b * Nq * kCube + (size_t)qc * kCube + 32 * (wave & 1) + qr;

  // ---- Q of this wave's 32 rows, in the B-operand layout of S^T = K Q^T:
  // lane (column qr, k-group g) holds q[row][16 s + 8 g .. + 7].
  bf16x8 qf[S::kQSteps];
  uint16_t* const orow = out + qrow_idx * row_stride + (size_t)h * D;
  if (real_q) {
    const uint16_t* qrow = q + qrow_idx * row_stride + (size_t)h * D;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * g);
  } else {
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s) qf[s] = bf16x8{};
  }

  // ---- the pair's step list (built by the pre-pass): step i holds the
  // entries of slots X and Y. Reads stay below n_steps + 3, inside the padded
  // list. Scalar loads: the index is made wave-uniform explicitly, since a
  // vector load here would be counted by the explicit vmcnt waits.
  const uint32_t* __restrict__ lst = steps + (size_t)pair * step_stride * 2;
  const int n_steps = __builtin_amdgcn_readfirstlane(counts[pair]);
  auto ent = [&](int i, int slot) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)lst[2 * __builtin_amdgcn_readfirstlane(i) + slot]);
  };
  if (n_steps == 0) {  // no real key in any cube either row selected: the rows are 0
    if (real_q) {
#pragma unroll
      for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * g) = u32x2{0u, 0u};
    }
    return;
  }

  // ---- DMA: each wave-wide load fills 1 KiB of a half-tile buffer, lane L
  // writing bytes [16 L, 16 L + 16); the lane fetches the global chunk that
  // the swizzle places in that slot. Wave w loads rows [8 w, 8 w + 8) of
  // both slots' half-tiles. The buffer range ends at the half's real rows,
  // so padding rows land in LDS as zeros; an empty slot, or slot Y of a
  // shared step, gets an empty range (its loads move no data and only write
  // zeros), which keeps the wait counts constant. Byte offsets are
  // < 32 * NH * D * 2 < 2^31 (host-checked).
  const uint32_t rs2 = (uint32_t)NH * D * 2u;
  uint32_t koff[S::kLoads], voff[S::kLoads];
#pragma unroll
  for (int n = 0; n < S::kLoads; ++n) {
    const int row = (wave * S::kLoads + n) * S::kRowsPerKiB + lane / S::kChunks;
    const int slot = lane % S::kChunks;
    koff[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_k<D>(row));
    voff[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(slot ^ swz_v<D>(row));
  }
  const uint32_t lds_wave = (uint32_t)(wave * S::kLoads) * 1024u;
  const size_t kv_head = (size_t)b * Nkv * kCube * row_stride + (size_t)h * D;
  auto half_rsrc = [&](const uint16_t* base, uint32_t e, bool real) __attribute__((always_inline)) -> int32x4_t {
    const uint16_t* p =
        base + kv_head + ((size_t)(e >> 8) * kCube + kHalf * ((e >> 5) & 1)) * row_stride;
    return buffer_rsrc(p, real ? (int)((((e & 31) + 1) * rs2)) : 0);
  };
  // resources of both slots of a step: X loads unless empty, Y loads unless
  // empty or equal to X
  struct Pair2 {
    int32x4_t x, y;
  };
  auto step_rsrc = [&](const uint16_t* base, uint32_t ex, uint32_t ey) __attribute__((always_inline)) -> Pair2 {
    return Pair2{half_rsrc(base, ex, (ex & kValid) != 0),
                 half_rsrc(base, ey, (ey & kValid) != 0 && ey != ex)};
  };
  // DMA j (0 <= j < 2 kLoads) of a step's tensor: the first kLoads fill slot
  // X, the rest slot Y
  auto dma_j = [&](const Pair2& r, uint32_t lds_buf, const uint32_t* off, int j) __attribute__((always_inline)) {
    if (j < S::kLoads)
      dma16(r.x, off[j], lds_buf + lds_wave + 1024u * j);
    else
      dma16(r.y, off[j - S::kLoads], lds_buf + (uint32_t)S::kHalfBytes + lds_wave + 1024u * (j - S::kLoads));
  };
  auto issue_all = [&](const Pair2& r, uint32_t lds_buf, const uint32_t* off) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2 * S::kLoads; ++j) dma_j(r, lds_buf, off, j);
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

  // The Q loads must be complete before the first DMA is issued: afterwards
  // the only outstanding vector-memory operations are the tile loads that
  // the explicit waits account for. The empty asm makes the compiler place
  // its own wait for Q here rather than inside the loop.
#pragma unroll
  for (int s = 0; s < S::kQSteps; ++s) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qf[s])));

  // ---- pipeline over steps. Buffers alternate: step i uses kbuf[i&1] and
  // vbuf[i&1]. V(i+1) streams in during QK(i) (its buffer held V(i-1), which
  // every wave finished before the first barrier of step i); K(i+2) streams
  // in during PV(i) (its buffer held K(i), which every wave finished before
  // the second barrier of step i). Each step's DMAs are spread one per MFMA
  // step; a wave whose slot is empty in step i issues them back to back and
  // skips the arithmetic. The prologue loads K(0), V(0) and K(1). Loads of
  // steps past the end of the list are issued with empty slots, so every
  // wait below leaves exactly the two younger steps' loads in flight.
  constexpr int kPerStep = 2 * S::kLoads;  // DMAs per wave, tensor and step
  const uint32_t kb0 = lds_address(kbuf), vb0 = lds_address(vbuf);
  constexpr uint32_t kBufBytes = 2u * S::kHalfBytes;
  uint32_t x_c = ent(0, 0), y_c = ent(0, 1), x_n1 = ent(1, 0), y_n1 = ent(1, 1);
  issue_all(step_rsrc(k, x_c, y_c), kb0, koff);
  issue_all(step_rsrc(k, x_n1, y_n1), kb0 + kBufBytes, koff);

  const int G = lane >> 4, s4 = lane & 15;
  const int trow = 4 * (G >> 1) + (s4 >> 2);
  const int dcol = 16 * (G & 1) + 4 * (s4 & 3);
  // this wave's entry of a step, and the slot its tiles sit in (slot X for a
  // shared step)
  auto my_entry = [&](uint32_t ex, uint32_t ey) __attribute__((always_inline)) -> uint32_t {
    return sub == 0 ? ex : ey;
  };
  auto my_slot = [&](uint32_t ex, uint32_t ey) __attribute__((always_inline)) -> uint32_t {
    return (sub == 0 || ex == ey) ? 0u : (uint32_t)S::kHalfBytes;
  };
  // Steps in which this wave's slot is empty run in the inner loop, which
  // only keeps the loads going; the accumulators are carried by the outer
  // loop alone.
  int i = 0;
#pragma unroll 1
  while (true) {
#pragma unroll 1
    while (i < n_steps && (my_entry(x_c, y_c) & kValid) == 0) {
      const uint32_t x_n2 = ent(i + 2, 0), y_n2 = ent(i + 2, 1);
      wait_vmcnt<kPerStep>();
      __syncthreads();
      issue_all(step_rsrc(v16, x_c, y_c), vb0, voff);
      wait_vmcnt<0>();
      __syncthreads();
      issue_all(step_rsrc(k, x_n2, y_n2), kb0 + kBufBytes * (uint32_t)(i & 1), koff);
      x_c = x_n1;
      y_c = y_n1;
      x_n1 = x_n2;
      y_n1 = y_n2;
      ++i;
    }
    if (i >= n_steps) break;
    const uint32_t x_n2 = ent(i + 2, 0), y_n2 = ent(i + 2, 1);
    const uint32_t e_c = my_entry(x_c, y_c);
    const uint32_t sl = my_slot(x_c, y_c);

    // ---- K(i) has landed (K(i+1) may be in flight), then every wave's
    // loads are visible; every wave has finished PV(i-1), so the V buffer is
    // free for V(i)
    wait_vmcnt<kPerStep>();
    __syncthreads();

    // ---- S^T = K Q^T over the half's 32 tokens; the K operands are read
    // from LDS two k-steps ahead of the MFMAs that consume them. V(i+1)'s
    // DMAs ride along.
    floatx16 sacc;
    {
      const Pair2 vr = step_rsrc(v16, x_c, y_c);
      const uint32_t vlds = vb0;
      const uint8_t* krow = &kbuf[i & 1][0][0] + sl + qr * S::kRowBytes;
      const int ksw = swz_k<D>(qr);
      bf16x8 a[3];
      auto rd = [&](int st) __attribute__((always_inline)) {
        a[st % 3] = *reinterpret_cast<const bf16x8*>(krow + 16 * ((2 * st + g) ^ ksw));
      };
      rd(0);
      rd(1);
#pragma unroll
      for (int st = 0; st < S::kQSteps; ++st) {
        if (st + 2 < S::kQSteps) rd(st + 2);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st % 3], qf[st], st == 0 ? zero16 : sacc,
                                                       0, 0, 0);
        if (st < kPerStep) dma_j(vr, vlds, voff, st);
      }
#pragma unroll
      for (int j = S::kQSteps; j < kPerStep; ++j) dma_j(vr, vlds, voff, j);
    }

    // ---- online softmax of the half: tokens >= its real rows set to -inf
    // (partial halves only; the asm keeps the compiler from flattening the
    // branch into selects that every half would execute), row max, lazy
    // raise of the reference max (wave-uniform), P in fp16 (round to nearest
    // even), row sum of the same rounded values (v_dot2_f32_f16 against 1.0).
    {
      const int nvh = (int)(e_c & 31u) + 1;
      if (nvh < kHalf) {
        asm volatile("");
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = 8 * (r >> 2) + 4 * g + (r & 3);
          if (tok >= nvh) sacc[r] = kNegInf;
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = halves_max(mx);
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
    halfx8 pb[2];
    float rs_sum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      floatx8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * kk + e], scale_log2, -mc));
      pb[kk] = __builtin_convertvector(p, halfx8);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const halfx2 two = {pb[kk][e], pb[kk][e + 1]};
        rs_sum = __builtin_amdgcn_fdot2(two, ones, rs_sum, false);
      }
    }
    l_run += halves_sum(rs_sum);

    // ---- V(i) (and K(i+1)) have landed, then every wave's loads are
    // visible; every wave has finished QK(i), so K(i)'s buffer is free for
    // K(i+2).
    wait_vmcnt<0>();
    __syncthreads();

    // ---- O^T += V^T P^T. The A operand comes from the transposing read: in
    // each 16-lane group, lane i receives element i%4 of the 8 bytes that
    // lane 4e + i/4 addressed, for e = 0..3. Lane (group G, s) addresses row
    // base + 4(G/2) + s/4 at column block 32 db + 16 (G%2) + 4 (s%4), so lane
    // l receives d = 32 db + l%32 at tokens base + 4 (l/32) + e: the k-slots
    // of lane group g = l/32 are tokens base+4g+{0..3} and base+8+4g+{0..3},
    // matching the accumulator layout of P. Operands are read two MFMAs
    // ahead. K(i+2)'s DMAs ride along.
    {
      const Pair2 kr = step_rsrc(k, x_n2, y_n2);
      const uint32_t klds = kb0 + kBufBytes * (uint32_t)(i & 1);
      const uint8_t* vb = &vbuf[0][0] + sl;
      constexpr int NSTEP = 2 * S::kDBlocks;  // (kk, db)
      u32x4 a[3];
      auto rd = [&](int st) __attribute__((always_inline)) {
        const int kk = st / S::kDBlocks, db = st % S::kDBlocks;
        const int r0 = 16 * kk + trow, r1 = r0 + 8;
        const int d0 = 32 * db + dcol;
        const uint8_t* p0 = vb + r0 * S::kRowBytes + 16 * ((d0 >> 3) ^ swz_v<D>(r0)) + 2 * (d0 & 7);
        const uint8_t* p1 = vb + r1 * S::kRowBytes + 16 * ((d0 >> 3) ^ swz_v<D>(r1)) + 2 * (d0 & 7);
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
                                                          pb[kk], oacc[db], 0, 0, 0);
        if (st < kPerStep) dma_j(kr, klds, koff, st);
      }
#pragma unroll
      for (int j = NSTEP; j < kPerStep; ++j) dma_j(kr, klds, koff, j);
    }
    x_c = x_n1;
    y_c = y_n1;
    x_n1 = x_n2;
    y_n1 = y_n2;
    ++i;
  }

  wait_vmcnt<0>();  // the empty loads of the last steps
  if (!real_q) return;

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
  w.list_stride = 2 * topk + kStepPad;  // steps per pair, 8 bytes each
  const size_t pairs = (size_t)B * NH * ((Nq + 1) / 2);
  w.v16_off = 0;
  w.list_off = up((size_t)B * Nkv * kCube * NH * D * 2);
  w.count_off = w.list_off + up(pairs * w.list_stride * 8);
  w.total = w.count_off + up(pairs * 4);
  return w;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* vbs, uint16_t* out,
                      int B, int Nq, int Nkv, int NH, int D, int topk,
                      float sm_scale, void* workspace, hipStream_t stream) {
  const FwdWorkspace w = fwd_workspace(B, Nq, Nkv, NH, D, topk);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + w.v16_off);
  uint32_t* steps = reinterpret_cast<uint32_t*>(ws + w.list_off);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.count_off);
  const int cpr = NH * D / 8;
  const int n_pairs_q = (Nq + 1) / 2;
  const int n_pairs = B * NH * n_pairs_q;
  hipLaunchKernelGGL(v_to_fp16_kernel, dim3(Nkv * kCvtSplit, B), dim3(kCvtThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(v16), vbs, Nkv,
                     cpr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(steps_kernel, dim3(n_pairs), dim3(kListThreads), 0, stream, topk_idx, vbs,
                     steps, counts, Nq, Nkv, topk, w.list_stride, n_pairs_q);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  if (D == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(n_pairs), dim3(FwdShape<128>::kThreads), 0,
                       stream, q, k, v16, steps, counts, out, Nq, Nkv, NH, w.list_stride,
                       scale_log2, n_pairs, n_pairs_q);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(n_pairs), dim3(FwdShape<64>::kThreads), 0,
                       stream, q, k, v16, steps, counts, out, Nq, Nkv, NH, w.list_stride,
                       scale_log2, n_pairs, n_pairs_q);
  return hipGetLastError();
}

}  // namespace vsa
