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
//   moe_floor_bcast_split  the same broadcast by S waves per 1 KiB chunk, wave
//                     j storing rows j, j + S, ... (the stand-alone scatter's
//                     shape).
//   moe_floor_copy    a contiguous copy: the plain streaming rate.
//
// Launch shapes: one wave per (token, 1 KiB of the row) in 256-thread
// workgroups for the broadcast (the copying waves of the fused layout +
// dispatch kernel store all K rows of a chunk so), one workgroup of S waves
// per (token, 1 KiB) for the split broadcast, one wave per (token, 512 B) in
// one-wave workgroups for the gather (as the combine; the gather split over
// two or four waves per chunk, each loading a share of the K rows and wave 0
// summing them through LDS, measured 4.76 / 4.81 against 4.59 us at 128 x 7168
// x 8); non-temporal stores throughout. A wave's token comes from a
// host-computed reciprocal (an integer division per wave cost the gather
// 0.2 us).
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

// One workgroup of kS waves per (token, 64 vectors of 16 bytes); wave j
// stores rows j, j + kS, ... The chunk is read by every wave (plain loads:
// after the first, from L2).
template <int kS>
__global__ __launch_bounds__(64 * kS) void floor_bcast_split_kernel(
    const u32x4 *__restrict__ x, u32x4 *__restrict__ out, uint64_t magic, int32_t T, int32_t K,
    int32_t nvec, int32_t nchunk) {
  const int b = blockIdx.x;
  const int t = (int)(((uint64_t)(uint32_t)b * magic) >> 32);
  if (t >= T) return;
  const int j = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int v = (b - t * nchunk) * 64 + (int)(threadIdx.x & 63);
  if (v >= nvec) return;
  const u32x4 val = x[(int64_t)t * nvec + v];
  u32x4 *dst = out + (int64_t)t * K * nvec + v;
  for (int k = j; k < K; k += kS) __builtin_nontemporal_store(val, dst + (int64_t)k * nvec);
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

// Copy of n 16-byte vectors, one per thread and grid stride, up to 65536
// workgroups. (Four vectors in flight per thread over at most 8192 workgroups
// streamed a 1 GiB copy at 5.0 TB/s; one per thread over 65536 workgroups at
// 5.9 TB/s.)
__global__ __launch_bounds__(256) void floor_copy_kernel(const u32x4 *__restrict__ src,
                                                         u32x4 *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
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

// The broadcast by S waves per chunk; S in {1, 2, 4, 8}.
FLOOR_API int moe_floor_bcast_split(const uint16_t *x, uint16_t *out, int32_t T, int32_t H,
                                    int32_t K, int32_t S, hipStream_t s) {
  if (T < 1 || H < 8 || H % 8 != 0 || K < 1 || K > kMaxK) return -2;
  if (S != 1 && S != 2 && S != 4 && S != 8) return -2;
  if ((int64_t)T * (H / 8) >= ((int64_t)1 << 31)) return -2;
  if (!x || !out) return -1;
  if (!aligned16(x) || !aligned16(out)) return -5;
  const int32_t nvec = H / 8, nchunk = (nvec + 63) / 64;
  const int64_t wgs = (int64_t)T * nchunk;
  if (wgs * (int64_t)nchunk >= ((int64_t)1 << 32)) return -2;
  const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
  u32x4 *ov = reinterpret_cast<u32x4 *>(out);
  const dim3 g((unsigned)wgs), w((unsigned)(64 * S));
  const uint64_t m = recip(nchunk);
  switch (S) {
    case 1: hipLaunchKernelGGL(floor_bcast_split_kernel<1>, g, w, 0, s, xv, ov, m, T, K, nvec, nchunk); break;
    case 2: hipLaunchKernelGGL(floor_bcast_split_kernel<2>, g, w, 0, s, xv, ov, m, T, K, nvec, nchunk); break;
    case 4: hipLaunchKernelGGL(floor_bcast_split_kernel<4>, g, w, 0, s, xv, ov, m, T, K, nvec, nchunk); break;
    default: hipLaunchKernelGGL(floor_bcast_split_kernel<8>, g, w, 0, s, xv, ov, m, T, K, nvec, nchunk);
  }
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
  int64_t wgs = (n + 255) / 256;  // one vector per thread
  if (wgs > 65536) wgs = 65536;
  hipLaunchKernelGGL(floor_copy_kernel, dim3((unsigned)wgs), dim3(256), 0, s,
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
  return ok(hipGetLastError());
}
