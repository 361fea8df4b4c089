// Dispatch scatter and weighted combine on gfx950.
//
// Dispatch (NeMo AutoModel page "nemo_automodel.components.moe.uccl_ep.buffer",
// Buffer.dispatch and Buffer.low_latency_dispatch with bf16 x): every selected
// (token, k) pair receives a bit copy of the token's hidden row in its slot of
// the receive buffer.
// Combine (same page, Buffer.low_latency_combine "reduce with weights"; and
// Buffer.combine): each token's expert outputs are summed back, times their
// top-k weights, into a bf16 row. Optionally with an active-rank mask (the
// NIXL EP notes: the combine loops check each rank's mask entry): pairs whose
// expert lives on a masked rank are left out. The row loads do not wait for
// the mask -- they are issued from the slots as usual, and the (scalar) id and
// mask reads complete while the rows are in flight; the mask only gates the
// sum. In normal mode (one row per token and rank, slots = the [T, R] rank
// table) the first wave of each token also sums the received top-k weights of
// its rows back, lanes 0..Kw-1, loaded alongside the rows.
//
// Both are HBM-bound streams with no data reuse, so the design is about
// bytes in flight. Dispatch: a thread owns one 16-byte vector (8 bf16) of one
// token row, a workgroup one 1 KiB chunk of a row, and its two (or four)
// waves each read the chunk and store it to half (a quarter) of the token's K
// slots -- 896 workgroups of two waves at 128 x 7168 -- with non-temporal
// stores (the receive rows are not re-read by this kernel).
// Combine: a thread owns 8 bytes (4 bf16), a wave covers 512 bytes of a row,
// one wave per workgroup -- 3584 waves at 128 x 7168. (Measured per step at 128 x 7168 / at 8192 x 7168: 16-byte lanes
// 9.50 / 178 us, 8-byte lanes 9.31 / 171 us, 4-byte lanes 9.30 / 183 us; two
// 16-byte vectors per lane 10.0 us: more waves hide more of the gather
// latency.) It issues all K loads of its lane before it sums, so K requests
// per lane are in flight at once, then adds in ascending k in f32 with no
// fused multiply-add and rounds once to bf16 (round to nearest even, NaN ->
// 0x7FC0), stored non-temporally.
#include "wave.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; every NaN becomes 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// A lane of kDw dwords (2: 8 bytes, 4 bf16; 4: 16 bytes, 8 bf16).
template <int kDw> struct Lane;
template <> struct Lane<2> { typedef u32x2 T; };
template <> struct Lane<4> { typedef u32x4 T; };

// One workgroup per (token, 1 KiB chunk of its row) of kS waves; wave j stores
// the chunk to the token's slots j, j + kS, ... Every wave reads the chunk
// (a plain load: after the first wave's, from L2) and has K / kS stores per
// lane in flight instead of K. Against one wave per chunk storing all K (four
// chunks per workgroup): 8192 x 7168 rows to random slots 219 -> 181 us (two
// waves) / 179 us (four); the skewed 4096 x 4096 batch (K = 6) 45.5 -> 38.5 /
// 37.3 us; 128 x 7168 3.82 -> 3.71 / 3.97 us. The token of workgroup b is
// b / nchunk, by the host reciprocal tmagic where exact (0: a division).
template <int KT, int kS>
__global__ __launch_bounds__(64 * kS) void dispatch_kernel(
    const int32_t *__restrict__ slot, const u32x4 *__restrict__ x, uint64_t tmagic, int64_t rows,
    int32_t T, int32_t nvec, int32_t nchunk, int32_t Kr, u32x4 *__restrict__ recv,
    int32_t *status) {
  const int K = KT ? KT : Kr;
  const int b = blockIdx.x;
  const int t = tmagic ? (int)(((uint64_t)(uint32_t)b * tmagic) >> 32) : b / nchunk;
  if (t >= T) return;
  const int j = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int v = (b - t * nchunk) * 64 + (int)(threadIdx.x & 63);
  const bool lane_ok = v < nvec;
  const int32_t *srow = slot + (int64_t)t * K;
  // a 32-bit unsigned compare against the row count clamped to INT32_MAX
  // keeps the slot tests scalar (slots are int32; -1 never passes)
  const uint32_t rows32 = rows < 0x7fffffff ? (uint32_t)rows : 0x7fffffffu;
  // slots per wave and group: all of them for a compile-time K
  constexpr int G = KT > 0 ? (KT + kS - 1) / kS : 4;
  u32x4 val = x[(int64_t)t * nvec + min(v, nvec - 1)];
  int32_t s[G];
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = (j + g * kS < K) ? srow[j + g * kS] : -1;
  // Settle the row load once here: without this the compiler re-waits on it
  // before every (conditional) store, and on gfx950 such a wait also drains
  // the stores already issued, serialising the copies.
  asm volatile("" : "+v"(val));
  int st = 0;
  for (int k0 = j; k0 < K; k0 += G * kS) {
    if (k0 > j) {
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = (k0 + g * kS < K) ? srow[k0 + g * kS] : -1;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if ((uint32_t)s[g] < rows32) {
        if (lane_ok) __builtin_nontemporal_store(val, recv + (int64_t)s[g] * nvec + v);
      } else if (s[g] != -1) {
        st |= kStBadSlot;
      }
    }
  }
  if (st && status && (threadIdx.x & 63) == 0) atomicOr(status, st);
}

template <int KT, bool kWeights, bool kF32Out, bool kMask, bool kWsum, int kDw>
// One wave per workgroup; the token of wave b is b / nchunk, by the
// host-computed reciprocal tmagic where that is exact (0: a division). The
// arguments a wave needs before its first loads lead, so the launch preloads
// them into registers (14 dwords, up to w): a read of the argument buffer
// before the slot load put a round trip ahead of every row load.
__global__ __launch_bounds__(64) void combine_kernel(const int32_t *__restrict__ slot,
                                                     const typename Lane<kDw>::T *__restrict__ y,
                                                     uint64_t tmagic, int64_t rows, int32_t T,
                                                     int32_t nq, int32_t nchunk, int32_t Kr,
                                                     const float *__restrict__ w,
                                                     typename Lane<kDw>::T *__restrict__ out,
                                                     f32x4 *__restrict__ out_f32, CombineMask cm,
                                                     RowWeightSum ws, int32_t *status) {
#pragma clang fp contract(off)
  typedef typename Lane<kDw>::T VT;
  const int K = KT ? KT : Kr;
  const int b = blockIdx.x;
  const int t = __builtin_expect(tmagic != 0, 1) ? (int)(((uint64_t)(uint32_t)b * tmagic) >> 32)
                                                 : b / nchunk;
  if (t >= T) return;
  const int v = (b - t * nchunk) * 64 + (int)(threadIdx.x & 63);  // lane (kDw dwords) in the row
  const bool full = (b - t * nchunk + 1) * 64 <= nq;  // uniform: every lane in the row
  // slots are int32: a 32-bit unsigned compare against the row count (clamped
  // to INT32_MAX) keeps the validity tests scalar (a 64-bit compare went to
  // the vector unit: low-latency combine at 128 tokens 4.89 -> 4.72 us,
  // normal-mode combine 3.80 -> 3.73 us)
  const uint32_t rows32 = rows < 0x7fffffff ? (uint32_t)rows : 0x7fffffffu;
  const bool lane_ok = v < nq;
  const int32_t *srow = slot + (int64_t)t * K;
  const float *wrow = kWeights ? w + (int64_t)t * K : nullptr;
  float acc[2 * kDw];
#pragma unroll
  for (int j = 0; j < 2 * kDw; ++j) acc[j] = 0.0f;
  int st = 0;
  // normal mode: the first wave of the token (lanes < Kw) sums the rows'
  // weights. Every lane of that wave loads (lanes past Kw repeat the last
  // entry): a load under a per-lane condition makes the compiler merge its
  // result, i.e. wait for it, before the next row load goes out (0.9 us per
  // step here).
  const bool wsum_wave = kWsum && v < 64;  // uniform: chunk 0
  const bool wsum_lane = wsum_wave && (int)(threadIdx.x & 63) < ws.Kw;
  const int wl = kWsum ? min((int)(threadIdx.x & 63), ws.Kw - 1) : 0;
  float wacc = 0.0f;
  constexpr int G = (KT > 0 && KT < 8) ? KT : 8;
  for (int k0 = 0; k0 < K; k0 += G) {
    int32_t s[G];
    float wk[G];
    bool ok[G], off[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool in = k0 + g < K;
      s[g] = in ? srow[k0 + g] : -1;
      wk[g] = (kWeights && in) ? wrow[k0 + g] : 1.0f;
    }
    VT val[G];
    float rw[G];
    // With the weight sum, loads under uniform branches only (lanes past the
    // row end re-read its last lane, the same cache line, and store nothing):
    // there a per-lane condition made the compiler wait between the loads.
    // Without it the per-lane form measured slightly faster.
    const int vc = lane_ok ? v : nq - 1;
    bool all_ok = full;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ok[g] = (uint32_t)s[g] < rows32;  // -1 and negatives are never below it
      all_ok = all_ok && ok[g];
    }
    if (kMask && __builtin_expect(all_ok, 1)) {
      // masked combine, every slot valid and the whole chunk in the row
      // (uniform): the loads go out with no per-load mask (M = 16 / 128
      // low-latency batches 2.87 -> 2.65 / 5.08 -> 4.83 us; the plain
      // combine measured 0.03 us slower so)
#pragma unroll
      for (int g = 0; g < G; ++g) val[g] = __builtin_nontemporal_load(y + (int64_t)s[g] * nq + v);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        val[g] = VT(0u);
        if (kWsum) {
          if (ok[g]) val[g] = __builtin_nontemporal_load(y + (int64_t)s[g] * nq + vc);
        } else if (ok[g] && lane_ok) {
          val[g] = __builtin_nontemporal_load(y + (int64_t)s[g] * nq + v);
        }
      }
    }
    // the rows' weights after all row loads are out
#pragma unroll
    for (int g = 0; g < G; ++g) {
      rw[g] = 0.0f;
      if (kWsum && ok[g] && wsum_wave) rw[g] = ws.in[(int64_t)s[g] * ws.Kw + wl];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {  // masked ranks (scalar reads, rows already in flight)
      off[g] = false;
      if (kMask && k0 + g < K) {
        const int64_t e = cm.idx[(int64_t)t * K + k0 + g];
        off[g] = e >= 0 && e < cm.E && cm.mask[rank_of((int)e, cm.l_magic)] != 0;
      }
      if (!ok[g] && s[g] != -1 && !off[g]) st |= kStBadSlot;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g] || off[g]) continue;
      if (kWsum) wacc = wacc + rw[g];
      const float a = wk[g];
#pragma unroll
      for (int d = 0; d < kDw; ++d) {
        acc[2 * d] = acc[2 * d] + a * bf16_lo(val[g][d]);
        acc[2 * d + 1] = acc[2 * d + 1] + a * bf16_hi(val[g][d]);
      }
    }
  }
  if (kWsum && wsum_lane) ws.out[(int64_t)t * ws.Kw + wl] = wacc;
  if (lane_ok) {
    const int64_t i = (int64_t)t * nq + v;
    VT o;
#pragma unroll
    for (int d = 0; d < kDw; ++d) o[d] = to_bf16(acc[2 * d]) | (to_bf16(acc[2 * d + 1]) << 16);
    // non-temporal: the kernel does not read its output back (0.2 us per
    // step faster than a plain store at 128 x 7168)
    __builtin_nontemporal_store(o, out + i);
    if (kF32Out) {
#pragma unroll
      for (int d = 0; d < kDw / 2; ++d)
        __builtin_nontemporal_store(
            f32x4{acc[4 * d], acc[4 * d + 1], acc[4 * d + 2], acc[4 * d + 3]},
            out_f32 + (kDw / 2) * i + d);
    }
  }
  if (st && status && (threadIdx.x & 63) == 0) atomicOr(status, st);
}

// ceil(2^32 / d): (b * m) >> 32 == b / d for every b < waves while
// waves * d < 2^32 (the error b * (m - 2^32 / d) / 2^32 < b / 2^32 stays under
// 1 / d); 0 beyond, where the kernel divides.
uint64_t token_magic(int64_t waves, int32_t d) {
  if ((uint64_t)waves * (uint64_t)d >= (1ull << 32)) return 0;
  return ((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d;
}

// Four waves per chunk for K >= 4 from kWideChunks (token, chunk) pairs on,
// else two (one for K = 1).
constexpr int64_t kWideChunks = 8192;

template <int KT, int kS>
hipError_t dispatch_ks(const uint16_t *x, const int32_t *slot, uint16_t *recv, int32_t T,
                       int32_t K, int32_t nvec, int32_t nchunk, int64_t rows, int32_t *status,
                       hipStream_t s) {
  const int64_t wgs = (int64_t)T * nchunk;
  hipLaunchKernelGGL((dispatch_kernel<KT, kS>), dim3((unsigned)wgs), dim3(64 * kS), 0, s, slot,
                     reinterpret_cast<const u32x4 *>(x), token_magic(wgs, nchunk), rows, T, nvec,
                     nchunk, K, reinterpret_cast<u32x4 *>(recv), status);
  return hipGetLastError();
}

template <int KT>
hipError_t dispatch_k(const uint16_t *x, const int32_t *slot, uint16_t *recv, int32_t T,
                      int32_t K, int32_t nvec, int64_t rows, int32_t *status, hipStream_t s) {
  const int32_t nchunk = (nvec + 63) / 64;
  if (K >= 4 && (int64_t)T * nchunk >= kWideChunks)
    return dispatch_ks<KT, 4>(x, slot, recv, T, K, nvec, nchunk, rows, status, s);
  if (K >= 2) return dispatch_ks<KT, 2>(x, slot, recv, T, K, nvec, nchunk, rows, status, s);
  return dispatch_ks<KT, 1>(x, slot, recv, T, K, nvec, nchunk, rows, status, s);
}

template <int KT, bool kW, bool kF, bool kM>
hipError_t combine_k3(const uint16_t *y, int64_t rows, const int32_t *slot, const float *w,
                      uint16_t *out, float *out_f32, int32_t T, int32_t K, int32_t nvec,
                      const CombineMask &cm, int32_t *status, hipStream_t s) {
  // one wave per workgroup: measured faster than four (128 x 7168: 0.2 us per
  // step; 8192 x 7168: 2 us) -- the waves spread over the CUs evenly
  const int32_t nq = nvec * 2;  // 8-byte lanes per row
  const int32_t nchunk = (nq + 63) / 64;
  const int64_t waves = (int64_t)T * nchunk;
  const RowWeightSum none{nullptr, nullptr, 0};
  hipLaunchKernelGGL((combine_kernel<KT, kW, kF, kM, false, 2>), dim3((unsigned)waves), dim3(64), 0,
                     s, slot, reinterpret_cast<const u32x2 *>(y), token_magic(waves, nchunk), rows,
                     T, nq, nchunk, K, w, reinterpret_cast<u32x2 *>(out),
                     reinterpret_cast<f32x4 *>(out_f32), cm, none, status);
  return hipGetLastError();
}

template <int KT, bool kF, bool kWs>
hipError_t rank_combine_k(const uint16_t *y, int64_t rows, const int32_t *rank_slot,
                          uint16_t *out, float *out_f32, int32_t T, int32_t R, int32_t nvec,
                          const RowWeightSum &ws, int32_t *status, hipStream_t s) {
  // 8-byte lanes, as the weighted combine (128 x 7168: 4.07 us; 16-byte lanes
  // 4.18 us)
  const int32_t nq = nvec * 2, nchunk = (nq + 63) / 64;
  const int64_t waves = (int64_t)T * nchunk;
  const CombineMask none{nullptr, nullptr, 0, 0};
  hipLaunchKernelGGL((combine_kernel<KT, false, kF, false, kWs, 2>), dim3((unsigned)waves), dim3(64),
                     0, s, rank_slot, reinterpret_cast<const u32x2 *>(y),
                     token_magic(waves, nchunk), rows, T, nq, nchunk, R, nullptr,
                     reinterpret_cast<u32x2 *>(out), reinterpret_cast<f32x4 *>(out_f32), none, ws,
                     status);
  return hipGetLastError();
}

template <int KT>
hipError_t rank_combine_kt(const uint16_t *y, int64_t rows, const int32_t *rank_slot,
                           uint16_t *out, float *out_f32, int32_t T, int32_t R, int32_t nvec,
                           const RowWeightSum &ws, int32_t *status, hipStream_t s) {
  if (ws.in) {
    if (out_f32) return rank_combine_k<KT, true, true>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
    return rank_combine_k<KT, false, true>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
  }
  if (out_f32) return rank_combine_k<KT, true, false>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
  return rank_combine_k<KT, false, false>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
}

template <int KT, bool kM>
hipError_t combine_km(const uint16_t *y, int64_t rows, const int32_t *slot, const float *w,
                      uint16_t *out, float *out_f32, int32_t T, int32_t K, int32_t nvec,
                      const CombineMask &cm, int32_t *status, hipStream_t s) {
  if (w) {
    if (out_f32)
      return combine_k3<KT, true, true, kM>(y, rows, slot, w, out, out_f32, T, K, nvec, cm, status, s);
    return combine_k3<KT, true, false, kM>(y, rows, slot, w, out, out_f32, T, K, nvec, cm, status, s);
  }
  if (out_f32)
    return combine_k3<KT, false, true, kM>(y, rows, slot, w, out, out_f32, T, K, nvec, cm, status, s);
  return combine_k3<KT, false, false, kM>(y, rows, slot, w, out, out_f32, T, K, nvec, cm, status, s);
}

template <int KT>
hipError_t combine_k(const uint16_t *y, int64_t rows, const int32_t *slot, const float *w,
                     uint16_t *out, float *out_f32, int32_t T, int32_t K, int32_t nvec,
                     const CombineMask *mask, int32_t *status, hipStream_t s) {
  if (mask) return combine_km<KT, true>(y, rows, slot, w, out, out_f32, T, K, nvec, *mask, status, s);
  const CombineMask none{nullptr, nullptr, 0, 0};
  return combine_km<KT, false>(y, rows, slot, w, out, out_f32, T, K, nvec, none, status, s);
}

}  // namespace

hipError_t launch_dispatch(const uint16_t *x, const int32_t *slot, uint16_t *recv, int32_t T,
                           int32_t K, int32_t H, int64_t rows, int32_t *status, hipStream_t s) {
  if (T <= 0) return hipSuccess;  // nothing to launch
  const int32_t nvec = H / 8;
  switch (K) {
    case 1: return dispatch_k<1>(x, slot, recv, T, K, nvec, rows, status, s);
    case 2: return dispatch_k<2>(x, slot, recv, T, K, nvec, rows, status, s);
    case 4: return dispatch_k<4>(x, slot, recv, T, K, nvec, rows, status, s);
    case 6: return dispatch_k<6>(x, slot, recv, T, K, nvec, rows, status, s);
    case 8: return dispatch_k<8>(x, slot, recv, T, K, nvec, rows, status, s);
    default: return dispatch_k<0>(x, slot, recv, T, K, nvec, rows, status, s);
  }
}

hipError_t launch_combine(const uint16_t *y, int64_t rows, const int32_t *slot, const float *w,
                          uint16_t *out, float *out_f32, int32_t T, int32_t K, int32_t H,
                          const CombineMask *mask, int32_t *status, hipStream_t s) {
  if (T <= 0) return hipSuccess;  // nothing to launch
  const int32_t nvec = H / 8;
  switch (K) {
    case 1: return combine_k<1>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
    case 2: return combine_k<2>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
    case 4: return combine_k<4>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
    case 6: return combine_k<6>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
    case 8: return combine_k<8>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
    default: return combine_k<0>(y, rows, slot, w, out, out_f32, T, K, nvec, mask, status, s);
  }
}

hipError_t launch_rank_combine(const uint16_t *y, int64_t rows, const int32_t *rank_slot,
                               uint16_t *out, float *out_f32, int32_t T, int32_t R, int32_t H,
                               const RowWeightSum &ws, int32_t *status, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int32_t nvec = H / 8;
  switch (R) {
    case 4: return rank_combine_kt<4>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
    case 8: return rank_combine_kt<8>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
    default: return rank_combine_kt<0>(y, rows, rank_slot, out, out_f32, T, R, nvec, ws, status, s);
  }
}

}  // namespace moe
