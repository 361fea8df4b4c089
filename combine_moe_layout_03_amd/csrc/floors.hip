// Floor kernels: the same byte counts as the dispatch scatter and the combine
// gather, with every data-dependent step taken out, so the benchmark can state
// how far each real kernel is from the best this GPU does with its bytes at
// its size. They are measurement infrastructure, built into their own library
// (libmoe_floors.so), not part of the dispatch/combine interface.
//
//   moe_floor_empty   an empty kernel of a given grid: the cost of a launch
//                     and its drain, nothing else.
//   moe_floor_bcast   out[t*K + k] = x[t]: the dispatch's bytes (one row read,
//                     K row writes per token) with computed, sequential
//                     destinations -- no layout, no slot read, ideal write order.
//   moe_floor_gather  out[t] = bf16(sum over k of y[t*K + k]): the combine's
//                     bytes (K row reads, one row write per token) with
//                     computed row addresses -- no slot or weight read.
//   moe_floor_copy    a contiguous copy: the plain streaming rate.
//
// Launch shapes follow the real kernels: one wave per (token, 1 KiB of the
// row) in 256-thread workgroups for the broadcast (as the stand-alone
// scatter), one wave per (token, 512 B) in one-wave workgroups for the gather
// (as the combine); non-temporal loads and stores throughout. A wave's token
// comes from a host-computed reciprocal (an integer division per wave cost the
// gather 0.2 us).
#include <hip/hip_runtime.h>
#include <stdint.h>

#define FLOOR_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxK = 8;

__global__ void floor_empty_kernel() {}

// One wave per (token, 64 vectors of 16 bytes); t is wave-uniform.
__global__ __launch_bounds__(256) void floor_bcast_kernel(const u32x4 *__restrict__ x,
                                                          u32x4 *__restrict__ out, uint64_t magic,
                                                          int32_t T, int32_t K, int32_t nvec,
                                                          int32_t nchunk) {
  const int wid = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int t = (int)(((uint64_t)(uint32_t)wid * magic) >> 32);
  if (t >= T) return;
  const int v = (wid - t * nchunk) * 64 + (int)(threadIdx.x & 63);
  if (v >= nvec) return;
  const u32x4 val = __builtin_nontemporal_load(x + (int64_t)t * nvec + v);
  u32x4 *dst = out + (int64_t)t * K * nvec + v;
  for (int k = 0; k < K; ++k) __builtin_nontemporal_store(val, dst + (int64_t)k * nvec);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One wave per (token, 64 lanes of 8 bytes); rows t*K .. t*K + K-1.
__global__ __launch_bounds__(64) void floor_gather_kernel(const u32x2 *__restrict__ y,
                                                          u32x2 *__restrict__ out, uint64_t magic,
                                                          int32_t T, int32_t K, int32_t nq,
                                                          int32_t nchunk) {
  const int wid = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  const int t = (int)(((uint64_t)(uint32_t)wid * magic) >> 32);
  if (t >= T) return;
  const int v = (wid - t * nchunk) * 64 + (int)(threadIdx.x & 63);
  if (v >= nq) return;
  const u32x2 *src = y + (int64_t)t * K * nq + v;
  u32x2 val[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k)
    if (k < K) val[k] = __builtin_nontemporal_load(src + (int64_t)k * nq);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k >= K) break;
    a0 += __uint_as_float(val[k].x << 16);
    a1 += __uint_as_float(val[k].x & 0xffff0000u);
    a2 += __uint_as_float(val[k].y << 16);
    a3 += __uint_as_float(val[k].y & 0xffff0000u);
  }
  const u32x2 o = {bf16_rne(a0) | (bf16_rne(a1) << 16), bf16_rne(a2) | (bf16_rne(a3) << 16)};
  __builtin_nontemporal_store(o, out + (int64_t)t * nq + v);
}

// Grid-stride copy of n 16-byte vectors, four in flight per thread.
__global__ __launch_bounds__(256) void floor_copy_kernel(const u32x4 *__restrict__ src,
                                                         u32x4 *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(a[j], dst + i + j * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ceil(2^32 / d): (w * m) >> 32 == w / d for every w < waves while waves * d
// < 2^32 (the callers check it)
uint64_t recip(int32_t d) { return ((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d; }

int ok(hipError_t e) { return e == hipSuccess ? 0 : -7; }

}  // namespace

// Returns 0, -1 (NULL pointer), -2 (bad size), -5 (misaligned) or -7 (launch).
FLOOR_API int moe_floor_empty(int32_t workgroups, int32_t threads, hipStream_t s) {
  if (workgroups < 1 || threads < 1 || threads > 1024) return -2;
  hipLaunchKernelGGL(floor_empty_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0,
                     s);
  return ok(hipGetLastError());
}

// x [T, H] bf16 -> out [T*K, H] bf16; H % 8 == 0, 1 <= K <= 8.
FLOOR_API int moe_floor_bcast(const uint16_t *x, uint16_t *out, int32_t T, int32_t H, int32_t K,
                              hipStream_t s) {
  if (T < 1 || H < 8 || H % 8 != 0 || K < 1 || K > kMaxK) return -2;
  if ((int64_t)T * (H / 8) >= ((int64_t)1 << 31)) return -2;
  if (!x || !out) return -1;
  if (!aligned16(x) || !aligned16(out)) return -5;
  const int32_t nvec = H / 8, nchunk = (nvec + 63) / 64;
  const int64_t waves = (int64_t)T * nchunk;
  if ((waves + 3) / 4 * 4 * (int64_t)nchunk >= ((int64_t)1 << 32)) return -2;
  hipLaunchKernelGGL(floor_bcast_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(x), reinterpret_cast<u32x4 *>(out),
                     recip(nchunk), T, K, nvec, nchunk);
  return ok(hipGetLastError());
}

// y [T*K, H] bf16 -> out [T, H] bf16; H % 8 == 0, 1 <= K <= 8.
FLOOR_API int moe_floor_gather(const uint16_t *y, uint16_t *out, int32_t T, int32_t H,
                               int32_t K, hipStream_t s) {
  if (T < 1 || H < 8 || H % 8 != 0 || K < 1 || K > kMaxK) return -2;
  if ((int64_t)T * (H / 4) >= ((int64_t)1 << 31)) return -2;
  if (!y || !out) return -1;
  if (!aligned16(y) || !aligned16(out)) return -5;
  const int32_t nq = H / 4, nchunk = (nq + 63) / 64;
  const int64_t waves = (int64_t)T * nchunk;
  if (waves * (int64_t)nchunk >= ((int64_t)1 << 32)) return -2;
  hipLaunchKernelGGL(floor_gather_kernel, dim3((unsigned)waves), dim3(64), 0, s,
                     reinterpret_cast<const u32x2 *>(y), reinterpret_cast<u32x2 *>(out),
                     recip(nchunk), T, K, nq, nchunk);
  return ok(hipGetLastError());
}

// bytes % 16 == 0; src and dst 16-byte aligned, not overlapping.
FLOOR_API int moe_floor_copy(const void *src, void *dst, int64_t bytes, hipStream_t s) {
  if (bytes < 16 || bytes % 16 != 0) return -2;
  if (!src || !dst) return -1;
  if (!aligned16(src) || !aligned16(dst)) return -5;
  const int64_t n = bytes / 16;
  int64_t wgs = (n + 1023) / 1024;  // four vectors per thread
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(floor_copy_kernel, dim3((unsigned)wgs), dim3(256), 0, s,
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
  return ok(hipGetLastError());
}
