// Wave64 and workgroup helpers shared by the layout kernels (gfx950).
#pragma once

#include "kernels.hpp"

namespace moe {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

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

// A wave owns 64 consecutive 16-byte vectors of one token row, so the token
// index is wave-uniform: its K slots (and weights) arrive as scalar loads before
// any vector memory operation, and the row's K stores or loads are issued back
// to back without waiting on each other. Lanes past the row end (H/8 not a
// multiple of 64) idle.
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
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
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
