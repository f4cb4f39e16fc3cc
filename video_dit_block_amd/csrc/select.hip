// Coarse selector: cube mean-pool, cube-to-cube scores, per-row top-k.
//
// VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
// GPUs, section "Two-Stage Architecture", Stage 1 (each cube is mean-pooled,
// cube-to-cube scores are computed, and every query cube keeps the Top-K key
// cubes with the highest scores) and section "Generating Sparsity Patterns"
// (pooled einsum, then top-k along the key axis, largest first). Optimizing
// block-sparse INT8 attention and multi-expert step caching for Wan 2.2,
// section "Decoupling Block Selection from Sparse CUDA Kernels" (mean-pooled
// summaries scored by dot product).
//
// Three kernels on the caller's stream:
//   pool_kernel   HBM-bound: one workgroup per (cube, 128 column chunks,
//                 batch, tensor); each lane owns one 16-byte column chunk of
//                 the token row and sums the cube's real rows in fp32, 8 rows
//                 in flight; the mean divides by vbs[c].
//   score_kernel  fp32 MFMA (v_mfma_f32_16x16x4_f32): a 64x64 tile of
//                 S = Qc . Kc^T per workgroup, its 64 Kc rows staged once in
//                 LDS for the four waves (Wan shape: 57-62 us, against 91-97 us
//                 with every wave reading its Kc operands from L2). fp32
//                 inputs keep the ranking accurate to fp32 rounding (bf16
//                 inputs would perturb scores by ~2^-9 relative and reorder
//                 near-ties).
//   topk_wave_kernel (Nc <= 2048) one wave per score row, rows independent:
//                 the row's order-preserving score keys sit in registers; an
//                 8-bit radix select of up to 4 passes (LDS histogram per
//                 pass, a DPP prefix sum over the bins to find the digit;
//                 it stops once every key on the resolved prefix is in the
//                 top k) bounds the k-th largest key; the keys above it and
//                 the lowest-id keys equal to it are compacted with ballots,
//                 and only those k are sorted (64-bit keys: score bits, then
//                 the complemented cube id), descending: by counting for up
//                 to 128, by an LDS bitonic network beyond.
//   topk_kernel   (larger rows) one workgroup per score row: a bitonic sort of
//                 all of the row's 64-bit keys in LDS, descending; the first
//                 topk ids are written out.
//                 Both give equal scores by ascending cube id, so their outputs
//                 are identical.
//                 With a CDF threshold tau either also writes the row's count: the
//                 fewest leading cubes whose softmax mass (softmax over all Nc
//                 scores times `scale`) reaches tau, capped at topk (Wan INT8
//                 blog, same section: sort block scores per query block and
//                 keep key blocks by a cumulative distribution threshold).
#include "device.h"
#include "launch.h"

namespace vsa {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------- pool

constexpr int kPoolThreads = 128;
constexpr int kPoolUnroll = 8;  // rows in flight per lane

// Up to three tensors pooled by one launch; blockIdx.z picks one.
struct PoolArgs {
  const u32x4* x[3];
  float* xc[3];
};

// grid (Nc * splits, B, n_tensors), splits = ceil(cpr / kPoolThreads): each
// lane owns one 16-byte column chunk (8 channels of one head) of the cube's
// token rows and sums its real rows in fp32, kPoolUnroll rows in flight.
// The NH pooled heads are the first NH of each source row of row_cpr chunks
// (row_cpr = NH * D / 8 unless the source holds more heads). Output layout
// [B][NH][Nc][D] fp32.
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolArgs a, const int32_t* __restrict__ vbs,
                                                           int Nc, int NH, int D, int splits,
                                                           int row_cpr) {
  const int c = blockIdx.x / splits, split = blockIdx.x - c * splits, b = blockIdx.y;
  const int cpr = NH * D / 8;  // 16-byte chunks (8 bf16) of the pooled heads
  const int col = split * kPoolThreads + threadIdx.x;
  if (col >= cpr) return;
  const u32x4* __restrict__ x = a.x[blockIdx.z];
  float* __restrict__ xc = a.xc[blockIdx.z];
  const int n = min(max(vbs[c], 0), kCube);  // clamped: never reads past the cube
  const u32x4* __restrict__ base = x + ((size_t)b * Nc + c) * kCube * row_cpr + col;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](const u32x4 t) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(t[e] << 16);
      acc[2 * e + 1] += __uint_as_float(t[e] & 0xFFFF0000u);
    }
  };
  int u = 0;
  for (; u + kPoolUnroll <= n; u += kPoolUnroll) {
    u32x4 t[kPoolUnroll];
#pragma unroll
    for (int i = 0; i < kPoolUnroll; ++i) t[i] = __builtin_nontemporal_load(base + (size_t)(u + i) * row_cpr);
#pragma unroll
    for (int i = 0; i < kPoolUnroll; ++i) add(t[i]);
  }
  for (; u < n; ++u) add(__builtin_nontemporal_load(base + (size_t)u * row_cpr));
  const int elem = col * 8;
  const int h = elem / D, d = elem - h * D;
  float* dst = xc + (((size_t)b * NH + h) * Nc + c) * D + d;
  floatx4 lo, hi;
  for (int e = 0; e < 4; ++e) {
    lo[e] = n > 0 ? acc[e] / (float)n : 0.0f;
    hi[e] = n > 0 ? acc[4 + e] / (float)n : 0.0f;
  }
  *reinterpret_cast<floatx4*>(dst) = lo;
  *reinterpret_cast<floatx4*>(dst + 4) = hi;
}

hipError_t pool_launch(const PoolArgs& a, int n_tensors, const int32_t* vbs, int B, int Nc,
                       int NH, int D, hipStream_t stream, int row_nh) {
  const int cpr = NH * D / 8;
  const int splits = (cpr + kPoolThreads - 1) / kPoolThreads;
  hipLaunchKernelGGL(pool_kernel, dim3(Nc * splits, B, n_tensors), dim3(kPoolThreads), 0, stream,
                     a, vbs, Nc, NH, D, splits, row_nh * D / 8);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scores

constexpr int kScoreThreads = 256;  // 4 waves; wave w owns tile rows 16w..16w+15
constexpr int kScoreTile = 64;

// grid (ceil(Nc/64) [j tiles], ceil(Nc/64) [i tiles], B*NH).
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// receives D[4*(l/16) + r][l%16], r = 0..3. The contraction index is
// assigned so that lane group g = l/16 covers d in [g*D/4, (g+1)*D/4): every
// lane then reads D/4 contiguous floats of one Qc row and of one Kc row.
template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc,
    float* __restrict__ s, int Nc) {
  constexpr int kSeg = D / 4;  // contraction steps per MFMA chain
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * kScoreTile, j0 = blockIdx.x * kScoreTile;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int r = lane % 16, g = lane / 16;
  const float* __restrict__ qb = qc + (size_t)bh * Nc * D;
  const float* __restrict__ kb = kc + (size_t)bh * Nc * D;
  float* __restrict__ sb = s + (size_t)bh * Nc * Nc;

  const int qi = min(i0 + 16 * wave + r, Nc - 1);
  float a[kSeg];
#pragma unroll
  for (int t = 0; t < kSeg; t += 4) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(qb + (size_t)qi * D + g * kSeg + t);
    a[t] = v[0]; a[t + 1] = v[1]; a[t + 2] = v[2]; a[t + 3] = v[3];
  }
  // the tile's 64 Kc rows staged once in LDS for the four waves (row pitch
  // D + 4 floats)
  __shared__ __attribute__((aligned(16))) float ks[kScoreTile * (D + 4)];
  for (int i = threadIdx.x; i < kScoreTile * D / 4; i += kScoreThreads) {
    const int row = i / (D / 4), c4 = i - row * (D / 4);
    const int kj = min(j0 + row, Nc - 1);
    *reinterpret_cast<floatx4*>(ks + row * (D + 4) + 4 * c4) =
        *reinterpret_cast<const floatx4*>(kb + (size_t)kj * D + 4 * c4);
  }
  __syncthreads();
#pragma unroll
  for (int cb = 0; cb < kScoreTile / 16; ++cb) {
    const float* kr = ks + (16 * cb + r) * (D + 4) + g * kSeg;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kSeg; t += 4) {
      const floatx4 b = *reinterpret_cast<const floatx4*>(kr + t);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t + e], b[e], acc, 0, 0, 0);
    }
    const int col = j0 + 16 * cb + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = i0 + 16 * wave + 4 * g + e;
      if (row < Nc && col < Nc) sb[(size_t)row * Nc + col] = acc[e];
    }
  }
}

// ---------------------------------------------------------------- top-k

constexpr int kTopkThreads = 256;

// Order-preserving map of a float to u32 (larger float -> larger key); -0 is
// folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key.
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// grid (Nc rows, B*NH). Dynamic LDS: n_pow2 * 8 bytes.
// Key = order_key(score) << 32 | (0xFFFFFFFF - j). Real keys are > 0; the
// padding keys (0) sort below every real key. valid != nullptr selects the
// CDF count (scale, tau).
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ s, int32_t* __restrict__ topk_idx, int Nc,
    int n_pow2, int topk, int32_t* __restrict__ valid, float scale, float tau) {
  extern __shared__ uint64_t keys[];
  const size_t row = (size_t)blockIdx.y * Nc + blockIdx.x;
  const float* __restrict__ srow = s + row * Nc;
  for (int j = threadIdx.x; j < n_pow2; j += kTopkThreads)
    keys[j] = j < Nc ? ((uint64_t)order_key(srow[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j)
                     : 0ull;
  const int half = n_pow2 / 2;
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = threadIdx.x; t < half; t += kTopkThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const uint64_t a = keys[lo], b = keys[hi];
        // descending within blocks whose `size` bit is clear, ascending
        // otherwise; the last merge (size == n_pow2) is all descending
        const bool desc = (lo & size) == 0;
        if (desc ? (a < b) : (a > b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
    }
  }
  __syncthreads();
  int32_t* __restrict__ out = topk_idx + row * topk;
  for (int t = threadIdx.x; t < topk; t += kTopkThreads)
    out[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[t] & 0xFFFFFFFFull));
  if (valid == nullptr) return;

  // ---- CDF count. Weights w_i = exp((s_i - s_0) scale) over the sorted
  // scores (s_0 the row max), Z = sum_i w_i; the count is the smallest n with
  // w_0 + ... + w_{n-1} >= tau Z, at most topk. Thread t owns the ranks
  // [t per, t per + per); a scan of the per-thread sums gives every thread
  // its running sum at the start of its ranks.
  __shared__ float part[kTopkThreads];
  __shared__ int first;
  const int tid = threadIdx.x;
  const int per = (Nc + kTopkThreads - 1) / kTopkThreads;
  const int r0 = tid * per, r1 = min(r0 + per, Nc);
  const float s0 = key_score((uint32_t)(keys[0] >> 32));
  auto w = [&](int i) __attribute__((always_inline)) -> float {
    return __expf((key_score((uint32_t)(keys[i] >> 32)) - s0) * scale);
  };
  float loc = 0.0f;
  for (int i = r0; i < r1; ++i) loc += w(i);
  part[tid] = loc;
  if (tid == 0) first = 0x7FFFFFFF;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {  // inclusive scan
    const float add = tid >= off ? part[tid - off] : 0.0f;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const float thr = tau * part[kTopkThreads - 1];
  float run = tid > 0 ? part[tid - 1] : 0.0f;
  for (int i = r0; i < r1; ++i) {
    run += w(i);
    if (run >= thr) {
      atomicMin(&first, i);
      break;
    }
  }
  __syncthreads();
  if (tid == 0) valid[row] = first == 0x7FFFFFFF ? min(Nc, topk) : min(first + 1, topk);
}

// ---------------------------------------------------------------- top-k, one wave per row

constexpr int kWaveRowsMax = 4;  // rows (waves) per workgroup

// Inclusive prefix sum over the wave on DPP lane moves (no LDS round trips):
// within each row of 16 lanes by shifts of 1, 2, 4 and 8 (a lane without a
// source adds 0), then across rows by the row broadcasts of lanes 15 and 31.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// grid (ceil(rows / waves)), block 64 * waves; dynamic LDS per wave: 256 u32
// histogram bins + n2 u64 candidate keys (n2 = power of two >= topk). Each
// wave owns its LDS and its row; no workgroup barrier. Lane l holds the keys
// of cubes j = 64 i + l, i < KPL (Nc <= 64 KPL).
template <int KPL>
__global__ __launch_bounds__(64 * kWaveRowsMax) void topk_wave_kernel(
    const float* __restrict__ s, int32_t* __restrict__ topk_idx, int64_t rows, int Nc, int n2,
    int topk, int32_t* __restrict__ valid, float scale, float tau) {
  extern __shared__ uint32_t smem[];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + wave;
  if (row >= rows) return;
  uint32_t* bins = smem + (size_t)wave * (256 + 2 * n2);
  uint64_t* cand = reinterpret_cast<uint64_t*>(bins + 256);
  const float* __restrict__ srow = s + row * Nc;
  const uint64_t below = (1ull << lane) - 1ull;

  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = 64 * i + lane;
    key[i] = j < Nc ? order_key(srow[j]) : 0u;
  }

  // Radix select: after pass p the top 8(p+1) bits of the k-th largest key
  // are known; krem counts how many keys sharing that prefix still belong to
  // the top k.
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)topk;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = lane; b < 256; b += 64) bins[b] = 0u;
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (64 * i + lane < Nc && (key[i] & pmask) == prefix)
        atomicAdd(&bins[(key[i] >> shift) & 255u], 1u);
    wave_lds_fence();
    // lane l holds digits 4l .. 4l+3; suf = keys with digit >= 4l
    const uint32_t b0 = bins[4 * lane], b1 = bins[4 * lane + 1], b2 = bins[4 * lane + 2],
                   b3 = bins[4 * lane + 3];
    const uint32_t t = b0 + b1 + b2 + b3;
    const uint32_t pre = wave_prefix_sum(t);  // keys with digit < 4 (l + 1)
    const uint32_t suf = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + t;
    // the digit d is the largest with (keys with digit >= d) >= krem; its lane
    // is the one lane with suf >= krem > suf - t
    const uint64_t hit = __ballot(suf >= krem && suf - t < krem);
    const int L = __ffsll((unsigned long long)hit) - 1;
    uint32_t d = 0, above = 0, at = 0;  // above / at: keys with digit > d / == d
    if (lane == L) {
      const uint32_t c4 = suf - t, c3 = c4 + b3, c2 = c3 + b2, c1 = c2 + b1;
      if (c3 >= krem) {
        d = 4 * L + 3; above = c4; at = b3;
      } else if (c2 >= krem) {
        d = 4 * L + 2; above = c3; at = b2;
      } else if (c1 >= krem) {
        d = 4 * L + 1; above = c2; at = b1;
      } else {
        d = 4 * L; above = c1; at = b0;
      }
    }
    d = (uint32_t)__builtin_amdgcn_readlane((int)d, L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
    at = (uint32_t)__builtin_amdgcn_readlane((int)at, L);
    krem -= above;
    prefix |= d << shift;
    pmask |= 0xFFu << shift;
    // every key sharing the prefix belongs to the top k: the lower digits
    // need not be resolved (and no tie among them needs breaking)
    if (at == krem) break;
  }

  // Compact the top k: keys whose resolved bits are above the prefix, then
  // the krem lowest-id keys equal to it on those bits (ids ascend with
  // (i, lane)); after an early exit that is every key equal to it.
  const int n_gt = topk - (int)krem;
  int seen_gt = 0, seen_eq = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = 64 * i + lane;
    const bool ok = j < Nc;
    const bool gt = ok && (key[i] & pmask) > prefix, eq = ok && (key[i] & pmask) == prefix;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const uint64_t k64 = ((uint64_t)key[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    if (gt) cand[seen_gt + __popcll(bg & below)] = k64;
    const int r = seen_eq + __popcll(be & below);
    if (eq && r < (int)krem) cand[n_gt + r] = k64;
    seen_gt += __popcll(bg);
    seen_eq += __popcll(be);
  }
  for (int t = topk + lane; t < n2; t += 64) cand[t] = 0ull;

  // Sort the candidates, descending. Up to 128 of them: each lane holds two
  // and counts the candidates above each (the keys are distinct, so that
  // count is its place), then writes them back in place; the wave reads
  // every candidate once with a broadcast read, no dependent chain (Wan
  // shape, 78 of 624: 13 us less than the bitonic network). More: a bitonic
  // sort of the n2 candidates. One wave: its LDS accesses complete in order,
  // the fence keeps the compiler from moving them.
  if (topk <= 128) {
    wave_lds_fence();
    const bool h0 = lane < topk, h1 = lane + 64 < topk;
    const uint64_t c0 = h0 ? cand[lane] : 0ull, c1 = h1 ? cand[lane + 64] : 0ull;
    int r0 = 0, r1 = 0;
#pragma unroll 4
    for (int j = 0; j < topk; ++j) {
      const uint64_t cj = cand[j];
      r0 += cj > c0;
      r1 += cj > c1;
    }
    wave_lds_fence();
    if (h0) cand[r0] = c0;
    if (h1) cand[r1] = c1;
  } else {
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size / 2; stride > 0; stride >>= 1) {
        wave_lds_fence();
        for (int t = lane; t < n2 / 2; t += 64) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const uint64_t a = cand[lo], b = cand[hi];
          const bool desc = (lo & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            cand[lo] = b;
            cand[hi] = a;
          }
        }
      }
    }
  }
  wave_lds_fence();
  int32_t* __restrict__ out = topk_idx + row * topk;
  for (int t = lane; t < topk; t += 64)
    out[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)(cand[t] & 0xFFFFFFFFull));
  if (valid == nullptr) return;

  // CDF count: w_i = exp((s_i - s_0) scale) with s_0 the row maximum, Z the
  // sum over all Nc cubes; the count is the smallest n with w_0 + .. + w_{n-1}
  // >= tau Z over the sorted ids, at most topk.
  const float s0 = key_score((uint32_t)(cand[0] >> 32));
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    if (64 * i + lane < Nc) z += __expf((key_score(key[i]) - s0) * scale);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  const float thr = tau * z;
  float run = 0.0f;
  int first = -1;
  for (int t0 = 0; t0 < topk && first < 0; t0 += 64) {
    const int t = t0 + lane;
    float sc = t < topk ? __expf((key_score((uint32_t)(cand[t] >> 32)) - s0) * scale) : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(sc, off, 64);
      if (lane >= off) sc += o;
    }
    const uint64_t reached = __ballot(t < topk && run + sc >= thr);
    if (reached != 0ull) first = t0 + __ffsll((unsigned long long)reached) - 1;
    run += __shfl(sc, 63, 64);
  }
  if (lane == 0) valid[row] = first < 0 ? topk : first + 1;
}

}  // namespace

hipError_t launch_pool(const uint16_t* x_tiled, const int32_t* vbs, int B, int Nc, int NH,
                       int D, float* xc, hipStream_t stream) {
  PoolArgs a = {};
  a.x[0] = reinterpret_cast<const u32x4*>(x_tiled);
  a.xc[0] = xc;
  return pool_launch(a, 1, vbs, B, Nc, NH, D, stream, NH);
}

SelectWorkspace select_workspace(int B, int NH, int Nc, int D) {
  SelectWorkspace w;
  const size_t pooled = (size_t)B * NH * Nc * D * sizeof(float);
  w.qc_off = 0;
  w.kc_off = align_up(pooled);
  w.s_off = w.kc_off + align_up(pooled);
  w.total = w.s_off + align_up((size_t)B * NH * Nc * Nc * sizeof(float));
  return w;
}

hipError_t launch_pool_scores(const uint16_t* q_tiled, const uint16_t* k_tiled,
                              const int32_t* vbs, int B, int Nc, int NH, int D,
                              void* workspace, hipStream_t stream, int row_nh) {
  const SelectWorkspace w = select_workspace(B, NH, Nc, D);
  char* ws = static_cast<char*>(workspace);
  float* qc = reinterpret_cast<float*>(ws + w.qc_off);
  float* kc = reinterpret_cast<float*>(ws + w.kc_off);
  float* s = reinterpret_cast<float*>(ws + w.s_off);

  PoolArgs a = {};
  a.x[0] = reinterpret_cast<const u32x4*>(q_tiled);
  a.x[1] = reinterpret_cast<const u32x4*>(k_tiled);
  a.xc[0] = qc;
  a.xc[1] = kc;
  hipError_t e = pool_launch(a, 2, vbs, B, Nc, NH, D, stream, row_nh > 0 ? row_nh : NH);
  if (e != hipSuccess) return e;

  const int nt = (Nc + kScoreTile - 1) / kScoreTile;
  dim3 sgrid(nt, nt, B * NH);
  if (D == 128)
    hipLaunchKernelGGL(score_kernel<128>, sgrid, dim3(kScoreThreads), 0, stream, qc, kc, s, Nc);
  else
    hipLaunchKernelGGL(score_kernel<64>, sgrid, dim3(kScoreThreads), 0, stream, qc, kc, s, Nc);
  return hipGetLastError();
}

hipError_t launch_topk(const float* s, int BH, int Nc, int topk, int32_t* topk_idx,
                       int32_t* valid, float scale, float tau, hipStream_t stream) {
  if (Nc <= 64 * 32) {
    int n2 = 64;
    while (n2 < topk) n2 <<= 1;
    const int waves = n2 <= 1024 ? kWaveRowsMax : 2;
    const int64_t rows = (int64_t)BH * Nc;
    const dim3 grid((unsigned)((rows + waves - 1) / waves)), block(64 * waves);
    const size_t lds = (size_t)waves * (256 + 2 * n2) * sizeof(uint32_t);
#define VSA_TOPK_WAVE(K)                                                                      \
  hipLaunchKernelGGL(topk_wave_kernel<K>, grid, block, lds, stream, s, topk_idx, rows, Nc, n2, \
                     topk, valid, scale, tau)
    if (Nc <= 64) VSA_TOPK_WAVE(1);
    else if (Nc <= 128) VSA_TOPK_WAVE(2);
    else if (Nc <= 256) VSA_TOPK_WAVE(4);
    else if (Nc <= 512) VSA_TOPK_WAVE(8);
    else if (Nc <= 1024) VSA_TOPK_WAVE(16);
    else VSA_TOPK_WAVE(32);
#undef VSA_TOPK_WAVE
    return hipGetLastError();
  }
  int n_pow2 = 1;
  while (n_pow2 < Nc) n_pow2 <<= 1;
  if (n_pow2 < 2) n_pow2 = 2;
  hipLaunchKernelGGL(topk_kernel, dim3(Nc, BH), dim3(kTopkThreads),
                     (size_t)n_pow2 * sizeof(uint64_t), stream, s, topk_idx, Nc,
                     n_pow2, topk, valid, scale, tau);
  return hipGetLastError();
}

hipError_t launch_select(const uint16_t* q_tiled, const uint16_t* k_tiled,
                         const int32_t* vbs, int B, int Nc, int NH, int D,
                         int topk, int32_t* topk_idx, int32_t* valid, float scale, float tau,
                         void* workspace, hipStream_t stream, int row_nh) {
  hipError_t e = launch_pool_scores(q_tiled, k_tiled, vbs, B, Nc, NH, D, workspace, stream,
                                    row_nh);
  if (e != hipSuccess) return e;
  const float* s = reinterpret_cast<const float*>(static_cast<const char*>(workspace) +
                                                  select_workspace(B, NH, Nc, D).s_off);
  return launch_topk(s, B * NH, Nc, topk, topk_idx, valid, scale, tau, stream);
}

}  // namespace vsa
