// Measurement aids, not part of the VSA path. (1) A bounded loop of bf16 MFMAs
// (v_mfma_f32_32x32x16_bf16) whose operands are random bf16 values read from
// LDS, so that the matrix cores switch as they do on real data (operands that
// stay constant draw less power and let the engine clock run higher). It gives
// the bf16 MFMA rate the part sustains at the clock its power budget allows,
// the ceiling against which the fine kernel's rate is read beside the
// datasheet figure. (2) An engine-clock meter: small workgroups that wait on the
// 100 MHz real-time counter (s_memrealtime) for a fixed span while reading the
// shader cycle counter (s_memtime), launched on a second stream beside a timed
// loop; the ratio of the two counts is the clock the loop ran at. (3) An LDS
// read pattern with and without bank conflicts, a control for the profiler's
// bank-conflict counter. (4) The MFMA loop with the fine kernel's vector
// work beside its MFMAs, at the fine kernel's occupancy: the rate the matrix
// units reach with that instruction mix when nothing else (loads, barriers,
// dependent accumulators) holds them. Built into its own library
// (libvsa_probe.so), loaded only by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;        // 4 waves, one per SIMD
constexpr int kLdsBytes = 32768;     // per workgroup; 4 workgroups per CU
constexpr int kMfmaPerIter = 16;

// grid: any number of workgroups; every wave runs `iters` iterations of 16
// independent-accumulator MFMAs. `src` holds kLdsBytes of random bf16 bits
// per workgroup slot (src is read modulo n_src_slots).
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(const uint4* __restrict__ src,
                                                             int n_src_slots, int iters,
                                                             float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4* s = src + (size_t)(blockIdx.x % n_src_slots) * (kLdsBytes / 16);
  for (int i = tid; i < kLdsBytes / 16; i += kThreads) reinterpret_cast<uint4*>(lds)[i] = s[i];
  __syncthreads();
  // each wave reads 16-byte operands from its own 8 KiB quarter of the LDS
  const uint8_t* base = lds + wave * 8192 + lane * 16;
  floatx16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < kMfmaPerIter; ++m) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + ((m + it) & 3) * 1024);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(base + 4096 + ((m + 2 * it) & 3) * 1024);
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[j][i];
  out[(size_t)blockIdx.x * kThreads + tid] = r;
}

// One workgroup of one wave per slot: counts shader cycles over `ticks` of
// the 100 MHz real-time counter (the loop always ends: the counter only
// advances), sleeping between reads; lane 0 writes (cycles, ticks).
__global__ __launch_bounds__(64) void clock_meter_kernel(uint64_t ticks,
                                                         unsigned long long* __restrict__ out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r - r0;
  }
}

// LDS bank-conflict control for the profiler's conflict counter: every lane
// reads `width` bytes at byte (lane * stride * width + 4 * (it & 7)) of a
// 32 KiB LDS array, `iters` times. stride 1 gives contiguous, conflict-free
// reads; stride 8 puts the lanes of a read on few banks. All addresses stay
// below 64 * 8 * 16 + 28 bytes.
template <int kWidth>
__global__ __launch_bounds__(64) void lds_conflict_kernel(int stride, int iters,
                                                          float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float lds[8192];
  const int lane = threadIdx.x;
  for (int i = lane; i < 8192; i += 64) lds[i] = (float)(i & 255);
  __syncthreads();
  float acc = 0.0f;
  const int base = lane * stride * (kWidth / 4);
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // one LDS read per iteration, none hoisted
    const int w = base + (it & 7);
    if (kWidth == 16) {
      const float4 x = *reinterpret_cast<const float4*>(&lds[w & ~3]);
      acc += x.x + x.y + x.z + x.w;
    } else {
      acc += lds[w];
    }
  }
  out[(size_t)blockIdx.x * 64 + lane] = acc;
}

// (4): 2-wave workgroups holding 40 KiB of LDS each, so 4 workgroups and 2
// waves per SIMD share a CU as in the fine kernel. Per 16 MFMAs (the same
// operands and accumulators as mfma_peak_kernel) every lane also runs 16
// exp2 and 48 FMAs on 16 registers that no MFMA reads, about the vector work
// of one fine-kernel wave-step (16 exponentials and some 50 other vector
// instructions). `src` as for mfma_peak_kernel; out: blocks * 128 floats.
constexpr int kMixThreads = 128;
constexpr int kMixLdsBytes = 40960;
constexpr int kMixExp = 16, kMixFma = 48;

__global__ __launch_bounds__(kMixThreads) void mfma_mix_kernel(const uint4* __restrict__ src,
                                                               int n_src_slots, int iters,
                                                               float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMixLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4* s = src + (size_t)(blockIdx.x % n_src_slots) * (kLdsBytes / 16);
  for (int i = tid; i < kLdsBytes / 16; i += kMixThreads) reinterpret_cast<uint4*>(lds)[i] = s[i];
  if (tid == 0) lds[kMixLdsBytes - 1] = 1;  // the whole allocation is in use
  __syncthreads();
  // each wave reads 16-byte operands from 8 KiB in its own half of the random
  // 32 KiB
  const uint8_t* base = lds + wave * 16384 + lane * 16;
  floatx16 acc[4] = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.001f * (float)(lane + i);
  const float c = 0.9999f, d = -0.0001f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < kMfmaPerIter; ++m) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + ((m + it) & 3) * 1024);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(base + 4096 + ((m + 2 * it) & 3) * 1024);
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
      if (m < kMixExp) x[m] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[m], c, d));
#pragma unroll
      for (int f = 0; f < kMixFma / kMfmaPerIter; ++f)
        x[(m + 5 * f + 1) & 15] = __builtin_fmaf(x[(m + 5 * f + 1) & 15], c, d);
    }
  }
  float r = (float)lds[kMixLdsBytes - 1];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[j][i];
#pragma unroll
  for (int i = 0; i < 16; ++i) r += x[i];
  out[(size_t)blockIdx.x * kMixThreads + tid] = r;
}

}  // namespace

extern "C" {

// Launches `blocks` one-wave workgroups of the LDS conflict control on
// `stream`; width 4 or 16 bytes, stride 1..8; out: device float buffer of
// blocks * 64 entries.
int32_t vsa_probe_lds(int32_t width, int32_t stride, int32_t blocks, int32_t iters, float* out,
                      void* stream) {
  if (out == nullptr || (width != 4 && width != 16) || stride < 1 || stride > 8 || blocks <= 0 ||
      iters <= 0)
    return (int32_t)hipErrorInvalidValue;
  if (width == 4)
    hipLaunchKernelGGL(lds_conflict_kernel<4>, dim3(blocks), dim3(64), 0,
                       static_cast<hipStream_t>(stream), stride, iters, out);
  else
    hipLaunchKernelGGL(lds_conflict_kernel<16>, dim3(blocks), dim3(64), 0,
                       static_cast<hipStream_t>(stream), stride, iters, out);
  return (int32_t)hipGetLastError();
}

// Launches `slots` one-wave workgroups (8: one per XCD, as workgroups are
// dealt to the XCDs in turn) that each run for `ticks` of the 100 MHz
// real-time counter on `stream`; out: device buffer of 2 * slots uint64.
int32_t vsa_probe_clock(int32_t slots, uint64_t ticks, void* out, void* stream) {
  if (out == nullptr || slots <= 0 || ticks == 0 || ticks > 1000000000ull)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_meter_kernel, dim3(slots), dim3(64), 0,
                     static_cast<hipStream_t>(stream), ticks,
                     static_cast<unsigned long long*>(out));
  return (int32_t)hipGetLastError();
}

// FLOP of one launch: blocks * 4 waves * iters * 16 MFMAs * 32768.
double vsa_probe_mfma_flop(int32_t blocks, int32_t iters) {
  return (double)blocks * 4.0 * iters * kMfmaPerIter * 32.0 * 32.0 * 16.0 * 2.0;
}

// Launches the loop on `stream`. src: device buffer of n_src_slots * 32 KiB of
// random bf16 bits; out: device float buffer of blocks * 256 entries.
// Returns 0, or the hipError_t of the launch.
int32_t vsa_probe_mfma(const void* src, int32_t n_src_slots, int32_t blocks, int32_t iters,
                       float* out, void* stream) {
  if (src == nullptr || out == nullptr || n_src_slots <= 0 || blocks <= 0 || iters <= 0)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     n_src_slots, iters, out);
  return (int32_t)hipGetLastError();
}

// Launches the loop with vector work (4) on `stream`: `blocks` workgroups of
// 2 waves; src as for vsa_probe_mfma; out: device float buffer of blocks * 128
// entries. Returns 0, or the hipError_t of the launch.
int32_t vsa_probe_mfma_mix(const void* src, int32_t n_src_slots, int32_t blocks, int32_t iters,
                           float* out, void* stream) {
  if (src == nullptr || out == nullptr || n_src_slots <= 0 || blocks <= 0 || iters <= 0)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_mix_kernel, dim3(blocks), dim3(kMixThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     n_src_slots, iters, out);
  return (int32_t)hipGetLastError();
}

// MFMA FLOP of one launch of (4): blocks * 2 waves * iters * 16 MFMAs * 32768.
double vsa_probe_mfma_mix_flop(int32_t blocks, int32_t iters) {
  return (double)blocks * 2.0 * iters * kMfmaPerIter * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
