// FP8 dispatch kernels on gfx950, after the NeMo AutoModel page
// "nemo_automodel.components.moe.uccl_ep.buffer":
//  - Buffer.low_latency_dispatch with use_fp8 (round_scale, use_ue8m0): every
//    token row is cast once to E4M3 with one scale per 128 channels, and the
//    codes and scales go to the pair's padded row; the scale tensors keep the
//    page's column-major last two dimensions, [E][H/128][R*M] floats or
//    [E][H/512][R*M] packed UE8M0 words;
//  - Buffer.dispatch with x given as an (E4M3 [T, H], float [T, H/128]) tuple:
//    both members are copied to the pair's row;
//  - optionally (kFp8ScaleRows) the low-latency scales row-major, [rows][H/128]
//    or [rows][H/512]: each pair's scales then fill contiguous bytes of its
//    own row instead of one 4-byte entry in each of H/128 lines shared with
//    the expert's other tokens;
//  - the cast alone (the tuple that Buffer.dispatch takes), row-major scales.
//
// The decomposition is the bf16 scatter's: a wave owns 64 consecutive 16-byte
// vectors of one token row (wave-uniform token, scalar slot loads, one
// settled row load, K stores issued back to back). For the cast a wave's
// 512 channels are four scale groups of 16 lanes each (fp8.hpp); it writes
// 8 bytes of codes per lane and pair, and one scale per group and pair (or one
// packed word per pair).
#include "fp8.hpp"
#include "wave.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cast and scatter to the low-latency rows. Row s = (e*R + src)*M + j of the
// [E*R*M, H] union; its scales sit at (e*G + g)*RM + (s - e*RM).
template <int KT, int kFlags>
__global__ __launch_bounds__(256) void ll_quant_dispatch_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ slot, u32x2 *__restrict__ recv_q,
    float *__restrict__ recv_scale, uint32_t *__restrict__ recv_ue, int32_t T, int32_t Kr,
    int32_t nvec, int32_t nchunk, int64_t rows, int32_t RM, int32_t G, int32_t *status) {
  const int K = KT ? KT : Kr;
  int t;
  const int v = wave_token_chunk(nchunk, t);
  if (t >= T) return;
  const int lane = lane_id();
  const int chunk = (v - lane) >> 6;
  const bool lane_ok = v < nvec;
  const int32_t *srow = slot + (int64_t)t * K;
  // slots are int32: the unsigned compare against the row count clamped to
  // INT32_MAX stays scalar, and -1 never passes it
  const uint32_t rows32 = rows < 0x7fffffff ? (uint32_t)rows : 0x7fffffffu;
  constexpr int GS = (KT > 0 && KT < 8) ? KT : 8;
  // unconditional, clamped load (H % 128 == 0, so a 16-lane group is either
  // inside the row or wholly past its end and never stored)
  u32x4 val = __builtin_nontemporal_load(x + (int64_t)t * nvec + min(v, nvec - 1));
  int32_t s[GS];
#pragma unroll
  for (int g = 0; g < GS; ++g) s[g] = (g < K) ? srow[g] : -1;
  asm volatile("" : "+v"(val));
  const Fp8Lane q = fp8_cast_lane<kFlags>(val);
  const u32x2 codes = {q.lo, q.hi};
  const int grp = chunk * 4 + (lane >> 4);
  uint32_t word = 0;
  if (kFlags & kFp8Ue8m0) word = ue8m0_word(q.scale);
  int st = 0;
  for (int k0 = 0; k0 < K; k0 += GS) {
    if (k0 > 0) {
#pragma unroll
      for (int g = 0; g < GS; ++g) s[g] = (k0 + g < K) ? srow[k0 + g] : -1;
    }
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const int r = s[g];
      if ((uint32_t)r < rows32) {
        const int e = r / RM;  // scalar
        const int i = r - e * RM;
        if (lane_ok) __builtin_nontemporal_store(codes, recv_q + (int64_t)r * nvec + v);
        if (kFlags & kFp8Ue8m0) {
          if (lane == 0)
            recv_ue[(kFlags & kFp8ScaleRows) ? (int64_t)r * nchunk + chunk
                                             : ((int64_t)e * nchunk + chunk) * RM + i] = word;
        } else if ((lane & 15) == 0 && lane_ok) {
          recv_scale[(kFlags & kFp8ScaleRows) ? (int64_t)r * G + grp
                                              : ((int64_t)e * G + grp) * RM + i] = q.scale;
        }
      } else if (r != -1) {
        st |= kStBadSlot;
      }
    }
  }
  if (st && status && lane == 0) atomicOr(status, st);
}

// Cast only: q [T, H], scales [T, H/128] floats or [T, H/512] UE8M0 words.
template <int kFlags>
__global__ __launch_bounds__(256) void quantize_kernel(const u32x4 *__restrict__ x,
                                                       u32x2 *__restrict__ q_out,
                                                       float *__restrict__ scale,
                                                       uint32_t *__restrict__ ue, int32_t T,
                                                       int32_t nvec, int32_t nchunk, int32_t G) {
  int t;
  const int v = wave_token_chunk(nchunk, t);
  if (t >= T) return;
  const int lane = lane_id();
  const int chunk = (v - lane) >> 6;
  const bool lane_ok = v < nvec;
  u32x4 val = __builtin_nontemporal_load(x + (int64_t)t * nvec + min(v, nvec - 1));
  asm volatile("" : "+v"(val));
  const Fp8Lane q = fp8_cast_lane<kFlags>(val);
  if (lane_ok) q_out[(int64_t)t * nvec + v] = u32x2{q.lo, q.hi};
  if (kFlags & kFp8Ue8m0) {
    const uint32_t word = ue8m0_word(q.scale);
    if (lane == 0) ue[(int64_t)t * nchunk + chunk] = word;
  } else if ((lane & 15) == 0 && lane_ok) {
    scale[(int64_t)t * G + chunk * 4 + (lane >> 4)] = q.scale;
  }
}

// Tuple copy: a wave owns 1 KiB of codes (64 lanes x 16 codes, 8 scale
// groups); lanes 0..7 also carry the chunk's 8 scales.
template <int KT>
__global__ __launch_bounds__(256) void fp8_copy_dispatch_kernel(
    const u32x4 *__restrict__ xq, const float *__restrict__ xs, const int32_t *__restrict__ slot,
    u32x4 *__restrict__ rq, float *__restrict__ rs, int32_t T, int32_t Kr, int32_t nvec,
    int32_t nchunk, int32_t G, int64_t rows, int32_t *status) {
  const int K = KT ? KT : Kr;
  int t;
  const int v = wave_token_chunk(nchunk, t);
  if (t >= T) return;
  const int lane = lane_id();
  const int chunk = (v - lane) >> 6;
  const bool lane_ok = v < nvec;
  const int g = chunk * 8 + (lane & 7);
  const bool scale_ok = lane < 8 && g < G;
  const int32_t *srow = slot + (int64_t)t * K;
  // slots are int32: the unsigned compare against the row count clamped to
  // INT32_MAX stays scalar, and -1 never passes it
  const uint32_t rows32 = rows < 0x7fffffff ? (uint32_t)rows : 0x7fffffffu;
  constexpr int GS = (KT > 0 && KT < 8) ? KT : 8;
  u32x4 val = __builtin_nontemporal_load(xq + (int64_t)t * nvec + min(v, nvec - 1));
  float sc = xs[(int64_t)t * G + min(g, G - 1)];
  int32_t s[GS];
#pragma unroll
  for (int j = 0; j < GS; ++j) s[j] = (j < K) ? srow[j] : -1;
  asm volatile("" : "+v"(val), "+v"(sc));
  int st = 0;
  for (int k0 = 0; k0 < K; k0 += GS) {
    if (k0 > 0) {
#pragma unroll
      for (int j = 0; j < GS; ++j) s[j] = (k0 + j < K) ? srow[k0 + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      const int r = s[j];
      if ((uint32_t)r < rows32) {
        if (lane_ok) __builtin_nontemporal_store(val, rq + (int64_t)r * nvec + v);
        if (scale_ok) rs[(int64_t)r * G + g] = sc;
      } else if (r != -1) {
        st |= kStBadSlot;
      }
    }
  }
  if (st && status && lane == 0) atomicOr(status, st);
}

unsigned wave_blocks(int32_t T, int32_t nchunk) {
  const int64_t waves = (int64_t)T * nchunk;
  return (unsigned)((waves + 3) / 4);
}

template <int KT, int kFlags>
hipError_t ll_quant_k(const uint16_t *x, const int32_t *slot, const Fp8Out &o, int32_t T,
                      int32_t K, int32_t H, int64_t rows, int32_t *status, hipStream_t s) {
  const int32_t nvec = H / 8, nchunk = (nvec + 63) / 64;
  hipLaunchKernelGGL((ll_quant_dispatch_kernel<KT, kFlags>), dim3(wave_blocks(T, nchunk)),
                     dim3(256), 0, s, reinterpret_cast<const u32x4 *>(x), slot,
                     reinterpret_cast<u32x2 *>(o.q), static_cast<float *>(o.scale),
                     static_cast<uint32_t *>(o.scale), T, K, nvec, nchunk, rows,
                     o.rows_per_expert, H / kFp8Group, status);
  return hipGetLastError();
}

template <int KT>
hipError_t ll_quant_flags(const uint16_t *x, const int32_t *slot, const Fp8Out &o, int32_t T,
                          int32_t K, int32_t H, int64_t rows, int32_t *status, hipStream_t s) {
  constexpr int R1 = kFp8RoundScale, U = kFp8Ue8m0, SR = kFp8ScaleRows;
  switch (o.flags) {
    case 0: return ll_quant_k<KT, 0>(x, slot, o, T, K, H, rows, status, s);
    case R1: return ll_quant_k<KT, R1>(x, slot, o, T, K, H, rows, status, s);
    case R1 | U: return ll_quant_k<KT, R1 | U>(x, slot, o, T, K, H, rows, status, s);
    case SR: return ll_quant_k<KT, SR>(x, slot, o, T, K, H, rows, status, s);
    case SR | R1: return ll_quant_k<KT, SR | R1>(x, slot, o, T, K, H, rows, status, s);
    default: return ll_quant_k<KT, SR | R1 | U>(x, slot, o, T, K, H, rows, status, s);
  }
}

template <int KT>
hipError_t fp8_copy_k(const uint8_t *xq, const float *xs, const int32_t *slot, uint8_t *rq,
                      float *rs, int32_t T, int32_t K, int32_t H, int64_t rows, int32_t *status,
                      hipStream_t s) {
  const int32_t nvec = H / 16, nchunk = (nvec + 63) / 64;
  hipLaunchKernelGGL(fp8_copy_dispatch_kernel<KT>, dim3(wave_blocks(T, nchunk)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(xq), xs, slot, reinterpret_cast<u32x4 *>(rq),
                     rs, T, K, nvec, nchunk, H / kFp8Group, rows, status);
  return hipGetLastError();
}

template <int kFlags>
hipError_t quantize_k(const uint16_t *x, uint8_t *q, void *scale, int32_t T, int32_t H,
                      hipStream_t s) {
  const int32_t nvec = H / 8, nchunk = (nvec + 63) / 64;
  hipLaunchKernelGGL(quantize_kernel<kFlags>, dim3(wave_blocks(T, nchunk)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(x), reinterpret_cast<u32x2 *>(q),
                     static_cast<float *>(scale), static_cast<uint32_t *>(scale), T, nvec, nchunk,
                     H / kFp8Group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ll_quant_dispatch(const uint16_t *x, const int32_t *slot, const Fp8Out &o,
                                    int32_t T, int32_t K, int32_t H, int64_t rows,
                                    int32_t *status, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  switch (K) {
    case 1: return ll_quant_flags<1>(x, slot, o, T, K, H, rows, status, s);
    case 2: return ll_quant_flags<2>(x, slot, o, T, K, H, rows, status, s);
    case 4: return ll_quant_flags<4>(x, slot, o, T, K, H, rows, status, s);
    case 6: return ll_quant_flags<6>(x, slot, o, T, K, H, rows, status, s);
    case 8: return ll_quant_flags<8>(x, slot, o, T, K, H, rows, status, s);
    default: return ll_quant_flags<0>(x, slot, o, T, K, H, rows, status, s);
  }
}

hipError_t launch_fp8_copy_dispatch(const uint8_t *xq, const float *xs, const int32_t *slot,
                                    uint8_t *rq, float *rs, int32_t T, int32_t K, int32_t H,
                                    int64_t rows, int32_t *status, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  switch (K) {
    case 1: return fp8_copy_k<1>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
    case 2: return fp8_copy_k<2>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
    case 4: return fp8_copy_k<4>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
    case 6: return fp8_copy_k<6>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
    case 8: return fp8_copy_k<8>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
    default: return fp8_copy_k<0>(xq, xs, slot, rq, rs, T, K, H, rows, status, s);
  }
}

hipError_t launch_quantize_fp8(const uint16_t *x, uint8_t *q, void *scale, int32_t flags,
                               int32_t T, int32_t H, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  switch (flags & (kFp8RoundScale | kFp8Ue8m0)) {  // the cast alone is always row-major
    case 0: return quantize_k<0>(x, q, scale, T, H, s);
    case kFp8RoundScale: return quantize_k<kFp8RoundScale>(x, q, scale, T, H, s);
    default: return quantize_k<kFp8RoundScale | kFp8Ue8m0>(x, q, scale, T, H, s);
  }
}

}  // namespace moe
