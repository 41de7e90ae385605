// gdr_peaks.hip -- the copy and MFMA-loop probes of include/gdr_peaks.h.
//
// Copy: 16-byte non-temporal loads and stores (the data is touched once),
// each thread moving four 16-byte pieces per grid stride so that four loads
// are in flight before their stores; 32 workgroups per CU.  MFMA: independent
// accumulator chains per wave (eight 16x16 or four 32x32 tiles), enough to
// keep the matrix pipe of a SIMD issuing back to back with two or more waves
// per SIMD.  On gfx950 the 32x32x16 bf16 form reaches about twice the flop
// rate of the 16x16x32 form, so both are probed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gdr_peaks.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_peak_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_peak_mfma16(float* __restrict__ sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((threadIdx.x + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((threadIdx.x * 3 + j) & 7));
  }
  f32x4 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_peak_mfma32(float* __restrict__ sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((threadIdx.x + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((threadIdx.x * 3 + j) & 7));
  }
  f32x16 c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[k][e];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <typename F>
int timed(int reps, hipStream_t st, float* ms_out, F launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -4;
  int rc = 0;
  launch();   // untimed first launch (code load, clocks)
  if (hipEventRecord(e0, st) != hipSuccess) rc = -4;
  for (int r = 0; r < reps && rc == 0; ++r) launch();
  if (rc == 0 && hipGetLastError() != hipSuccess) rc = -4;
  if (rc == 0 && hipEventRecord(e1, st) != hipSuccess) rc = -4;
  float ms = 0.f;
  if (rc == 0 && (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess)) rc = -4;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc == 0) *ms_out = ms / (float)reps;
  return rc;
}

}  // namespace

extern "C" {

int gdr_peak_copy(const void* src, void* dst, size_t bytes, int reps, void* stream, float* ms_out) {
  if (!src || !dst || !ms_out || reps < 1 || bytes == 0 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  const unsigned grid = 256 * 32;
  return timed(reps, st, ms_out, [&] {
    hipLaunchKernelGGL(k_peak_copy, dim3(grid), dim3(256), 0, st, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
  });
}

int gdr_peak_mfma_bf16(float* sink, int tile, int iters, int workgroups, int reps, void* stream, float* ms_out) {
  if (!sink || !ms_out || (tile != 16 && tile != 32) || iters < 1 || workgroups < 1 || reps < 1) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return timed(reps, st, ms_out, [&] {
    if (tile == 16) hipLaunchKernelGGL(k_peak_mfma16, dim3(workgroups), dim3(256), 0, st, sink, iters);
    else hipLaunchKernelGGL(k_peak_mfma32, dim3(workgroups), dim3(256), 0, st, sink, iters);
  });
}

}  // extern "C"
