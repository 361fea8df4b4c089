// Wave64 and workgroup helpers shared by the layout kernels (gfx950).
#pragma once

#include "kernels.hpp"

namespace moe {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// v with lane j replaced by the (uniform) value x
__device__ __forceinline__ int set_lane(int v, int j, int x) { return lane_id() == j ? x : v; }

// Inclusive prefix sum over the lanes of a wave (every lane must call it):
// a Hillis-Steele scan inside each 16-lane DPP row (row_shr by 1, 2, 4, 8),
// then row 1 and 3 add the last lane of the row before (row_bcast:15) and
// rows 2 and 3 the last lane of row 1 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

// Sum over the 64 lanes of a wave, wave-uniform (every lane must call it):
// rotations inside each 16-lane row (by 8, 4, 2, 1) give every lane its row's
// sum, then the four row sums are added.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xf, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 0) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 32) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
}

// Lanes of this wave holding the same key (only lanes with valid = true take
// part): one ballot per key bit, AND-ed -- gfx950 has no match instruction.
// Every lane of the wave must call this (the ballots are wave-wide).
__device__ __forceinline__ uint64_t match_peers(uint32_t key, bool valid, int bits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool one = (key >> b) & 1u;
    const uint64_t ones = __ballot(one);
    m &= one ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

// The lowest lane of a peer group speaks for it.
__device__ __forceinline__ bool is_leader(uint64_t peers) {
  return peers != 0ull && (__ffsll((unsigned long long)peers) - 1) == lane_id();
}

// Peers in lower lanes (earlier pairs, since lanes follow pair order).
__device__ __forceinline__ int below_me(uint64_t peers) {
  const uint64_t lt = (1ull << lane_id()) - 1ull;
  return __popcll(peers & lt);
}

// Workgroup barrier that orders LDS traffic only. Unlike __syncthreads() it
// does not wait for the wave's outstanding global loads, so a row load can
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave owns 64 consecutive vectors (16 bytes in the dispatch, 8 in the
// combine) of one token row, so the token index is wave-uniform: its K slots
// (and weights) arrive as scalar loads before any vector memory operation, and
// the row's K stores or loads are issued back to back without waiting on each
// other. Lanes past the row end (vectors per row not a multiple of 64) idle.
__device__ __forceinline__ int wave_token_chunk(int nchunk, int &t) {
  const int wid = __builtin_amdgcn_readfirstlane(
      (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
  t = wid / nchunk;
  return (wid - t * nchunk) * 64 + (int)(threadIdx.x & 63);
}

__device__ __forceinline__ int round_up(int c, int a) { return (c + a - 1) / a * a; }

// Exclusive scan of one int per thread over a workgroup of nwaves wave64s
// (s_wave holds at least nwaves ints). Every thread must call it. Its barriers
// order LDS only: the caller's outstanding global loads and stores stay in
// flight.
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave, int nwaves, int *total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
  if (lane == 63) s_wave[wave] = x;
  lds_barrier();
  int before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int s = s_wave[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  lds_barrier();
  *total = all;
  return before + x - v;
}

}  // namespace moe
