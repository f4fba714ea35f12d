// Ceiling kernels: what this chip reaches on the two resources the SATA path
// is bound by, measured with plain kernels of the same shapes.
//
//   HBM: a read + write copy, an in-place read-modify-write in the decode
//        step's access shape (blocks of 128 threads, two 16-byte vectors a
//        thread, one pass, non-temporal loads and stores) and a read-only
//        sum, each over a caller buffer.
//   MFMA: each wave issues eight independent accumulation chains of
//        16x16x32 bf16 (or 16x16x4 fp32) matrix instructions on register
//        operands, the instruction mix of the prefill's contractions with no
//        operand traffic.
//
// Built into its own library (libsata_ceilings.so): these are measurement
// tools beside the SATA path, not part of it.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sata_ceilings.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kCopyThreads = 256;
constexpr int kRmwThreads = 128, kRmwVec = 2;
constexpr int kReadThreads = 256, kReadVec = 4;
constexpr int kMfmaThreads = 512, kChains = 8;

__global__ __launch_bounds__(kCopyThreads) void ceil_copy(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                          int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kRmwThreads) void ceil_rmw(f32x4* p, int64_t n4) {
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * (kRmwThreads * kRmwVec) + threadIdx.x;
  f32x4 x[kRmwVec];
#pragma unroll
  for (int j = 0; j < kRmwVec; ++j) {
    const int64_t i = i0 + j * kRmwThreads;
    x[j] = i < n4 ? __builtin_nontemporal_load(p + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < kRmwVec; ++j) {
    const int64_t i = i0 + j * kRmwThreads;
    if (i < n4) __builtin_nontemporal_store(x[j] * 0.5f + 1.f, p + i);
  }
}

__global__ __launch_bounds__(kReadThreads) void ceil_read(const f32x4* __restrict__ src, int64_t n4,
                                                          float* __restrict__ partial) {
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * (kReadThreads * kReadVec) + threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kReadVec; ++j) {
    const int64_t i = i0 + j * kReadThreads;
    if (i < n4) acc += __builtin_nontemporal_load(src + i);
  }
  float s = acc[0] + acc[1] + acc[2] + acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  __shared__ float ws[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) t += ws[w];
    partial[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(kMfmaThreads) void ceil_mfma_bf16(float* out, int iters) {
  // small operands that differ by lane (the chains never overflow)
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x + j) & 7) * 0.0009765625f);
    b[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + j) & 7) * 0.0009765625f);
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<int64_t>(blockIdx.x) * kMfmaThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kMfmaThreads) void ceil_mfma_f32(float* out, int iters) {
  const float a = static_cast<float>(threadIdx.x & 7) * 0.0009765625f;
  const float b = static_cast<float>((threadIdx.x * 3) & 7) * 0.0009765625f;
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<int64_t>(blockIdx.x) * kMfmaThreads + threadIdx.x] = s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Grids stay within the 2^31 - 1 block limit.
bool grid_ok(int64_t blocks) { return blocks > 0 && blocks <= 0x7fffffff; }

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int sata_ceil_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(dst)) return -1;
  const int64_t n4 = static_cast<int64_t>(bytes / 16);
  const int64_t blocks = (n4 + kCopyThreads - 1) / kCopyThreads;
  if (!grid_ok(blocks)) return -1;
  ceil_copy<<<static_cast<unsigned>(blocks), kCopyThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n4);
  return status(hipGetLastError());
}

int sata_ceil_rmw(void* buf, size_t bytes, void* stream) {
  if (!buf || bytes == 0 || bytes % 16 || !aligned16(buf)) return -1;
  const int64_t n4 = static_cast<int64_t>(bytes / 16);
  const int64_t blocks = (n4 + kRmwThreads * kRmwVec - 1) / (kRmwThreads * kRmwVec);
  if (!grid_ok(blocks)) return -1;
  ceil_rmw<<<static_cast<unsigned>(blocks), kRmwThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<f32x4*>(buf), n4);
  return status(hipGetLastError());
}

int64_t sata_ceil_read_partials(size_t bytes) {
  const int64_t n4 = static_cast<int64_t>(bytes / 16);
  return (n4 + kReadThreads * kReadVec - 1) / (kReadThreads * kReadVec);
}

int sata_ceil_read(const void* src, size_t bytes, float* partial, void* stream) {
  if (!src || !partial || bytes == 0 || bytes % 16 || !aligned16(src)) return -1;
  const int64_t n4 = static_cast<int64_t>(bytes / 16);
  const int64_t blocks = sata_ceil_read_partials(bytes);
  if (!grid_ok(blocks)) return -1;
  ceil_read<<<static_cast<unsigned>(blocks), kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const f32x4*>(src), n4, partial);
  return status(hipGetLastError());
}

int sata_ceil_mfma(int dtype, int blocks, int iters, float* out, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (dtype != 0 && dtype != 1)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == 1)
    ceil_mfma_bf16<<<blocks, kMfmaThreads, 0, s>>>(out, iters);
  else
    ceil_mfma_f32<<<blocks, kMfmaThreads, 0, s>>>(out, iters);
  return status(hipGetLastError());
}

double sata_ceil_mfma_flops(int dtype, int blocks, int iters) {
  const double per = dtype == 1 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 4;
  return per * kChains * (kMfmaThreads / 64) * static_cast<double>(blocks) * iters;
}

}  // extern "C"
