// Measurement probes for the benchmark (libdsa_bench.so; not part of the
// draft-and-verify path and not linked into libdsa.so):
//   * the dense bf16 MFMA rate this chip sustains on full-mantissa operands,
//     from register-only loops of v_mfma_f32_32x32x16_bf16 and of
//     v_mfma_f32_16x16x32_bf16, four independent accumulation chains per
//     wave and no memory traffic (the 16x16x32 form sustains more on such
//     data, where the chip clocks down under MFMA load);
//   * the HBM read and copy bandwidth it sustains: every workgroup streams
//     its own contiguous chunk with 16-byte non-temporal loads (and stores).
// The benchmark reports each kernel's rate against these measured peaks next
// to the datasheet figures.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kThreads = 256;   // four waves, one per SIMD

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Operands are pseudo-random bf16 values with full mantissas (the chip's
// sustained MFMA clock depends on the data; small integers run faster than
// the normal-distributed values the kernels see).
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = mix(threadIdx.x * 131u + blockIdx.x * 7919u + e * 17u);
    a[e] = (__bf16)(((float)(h & 0xffffu) / 32768.f - 1.f) * 1.7f);
    b[e] = (__bf16)(((float)(h >> 16) / 32768.f - 1.f) * 1.3f);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += (c0[e] + c1[e]) + (c2[e] + c3[e]);
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// 16x16x32: eight waves per workgroup, two per SIMD, accumulators in
// ArchVGPRs (the form the kernels use; the AGPR form sustains less here),
// eight distinct A and B operands cycling over four chains.
constexpr int kThreads16 = 512;
__global__ __launch_bounds__(kThreads16) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma16_peak_kernel(
    float* __restrict__ out, int iters) {
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = mix(threadIdx.x * 131u + blockIdx.x * 7919u + j * 17u + e);
      a[j][e] = (__bf16)(((float)(h & 0xffffu) / 32768.f - 1.f) * 1.7f);
      b[j][e] = (__bf16)(((float)(h >> 16) / 32768.f - 1.f) * 1.3f);
    }
  f32x4_t c[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j % 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(j + j % 4) & 7], b[(j / 4) & 7], c[j % 4], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += (c[k][0] + c[k][1]) + (c[k][2] + c[k][3]);
  out[(size_t)blockIdx.x * kThreads16 + threadIdx.x] = s;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamU = 8;     // 16-byte loads in flight per thread

// Workgroup g reads (and, with dst, writes) 16-byte words
// [g * per_wg, min((g + 1) * per_wg, n)); one sum per thread goes to out.
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const u32x4_t* __restrict__ src,
                                                                u32x4_t* __restrict__ dst, uint32_t* out,
                                                                long long n, long long per_wg) {
  const long long lo = (long long)blockIdx.x * per_wg;
  const long long hi = lo + per_wg < n ? lo + per_wg : n;
  uint32_t acc = 0;
  for (long long i = lo + threadIdx.x; i < hi; i += (long long)kStreamThreads * kStreamU) {
    u32x4_t v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long j = i + (long long)u * kStreamThreads;
      v[u] = j < hi ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long j = i + (long long)u * kStreamThreads;
      if (dst && j < hi) __builtin_nontemporal_store(v[u], dst + j);
      acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
  }
  out[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace

// Streams `bytes` (a multiple of 16) from src, and copies them to dst when
// dst is not NULL, with `blocks` workgroups; out: uint32 [blocks * 256].
// Returns a hipError_t code.
extern "C" int dsa_bench_stream(const void* src, void* dst, void* out, long long bytes, int blocks, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
  const long long n = bytes / 16;
  const long long per_wg = (n + blocks - 1) / blocks;
  hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), static_cast<uint32_t*>(out), n,
                     per_wg);
  return (int)hipGetLastError();
}

// FLOPs of one call: blocks * 8 waves * iters * 32 MFMAs * 2*16*16*32.
// out: fp32 [blocks * 512] device buffer.  Returns a hipError_t code.
extern "C" int dsa_bench_mfma16_peak(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma16_peak_kernel, dim3(blocks), dim3(kThreads16), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return (int)hipGetLastError();
}

// FLOPs of one call: blocks * 4 waves * iters * 4 MFMAs * 2*32*32*16.
// out: fp32 [blocks * 256] device buffer.  Returns a hipError_t code.
extern "C" int dsa_bench_mfma_peak(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return (int)hipGetLastError();
}
