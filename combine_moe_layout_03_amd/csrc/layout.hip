// Dispatch layout on gfx950: per-expert counts, aligned prefix offsets and
// stable slots for every (token, k) pair, plus per-rank token sets.
//
// What is computed follows the NeMo AutoModel page
// "nemo_automodel.components.moe.uccl_ep.buffer": Buffer.get_dispatch_layout
// (num_tokens_per_rank, is_token_in_rank, num_tokens_per_expert), Buffer.dispatch
// (expert_alignment), Buffer.low_latency_dispatch (receive stripes of M rows per
// source rank and local expert). Rows inside an expert follow pair order t*K+k,
// which makes the layout unique.
//
// How: a wave64 finds the lanes holding the same expert id with one ballot per
// id bit (gfx950 has no match instruction), so a lane's rank among its peers is
// a popcount and one leader lane per (wave, expert) touches LDS -- no atomics on
// a hot expert's counter, whatever the skew. Each wave owns a contiguous segment
// of pairs and a private row of uint16 counters in LDS; a per-expert prefix over
// the 16 waves then gives every wave its starting rank. A batch of up to 1024
// pairs is done by one workgroup; larger batches take three launches (per-block
// counts and local ranks; one wave per expert for the prefix over blocks; a
// per-pair fix-up whose workgroups each scan the per-expert totals), with no
// inter-workgroup waiting. (Batches with alignment 1 of up to 4096 pairs take
// the counting kernel of fused.hip instead.)
#include "wave.hpp"

namespace moe {
namespace {

// One workgroup's share of the layout: tokens [t0, t1).
// kOneBlock: the workgroup holds the whole batch and writes final slots.
// Otherwise: it writes its per-expert totals and per-rank token counts to the
// workspace and its pairs' ranks inside the block to slot[]; the scan and
// fix-up kernels finish the job.
template <bool kOneBlock>
__global__ __launch_bounds__(kLayoutThreads) void layout_block_kernel(LayoutParams p) {
  __shared__ int16_t s_ids[kMaxPairsOneBlock];     // validated ids, -1 = none (16 KiB)
  __shared__ uint16_t s_wc[kLayoutWaves][kMaxExperts];  // per-wave counters (32 KiB)
  __shared__ int32_t s_base[kMaxExperts + 1];      // first slot of each expert (+ end)
  __shared__ int32_t s_cnt[kMaxExperts];           // pairs per expert in this block
  __shared__ int32_t s_rc[kMaxExperts];            // tokens per rank in this block
  __shared__ int32_t s_wave[kLayoutWaves];
  __shared__ int32_t s_status;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int E = p.E, R = p.R, K = p.K;
  const int t0 = blockIdx.x * p.tokens_per_block;
  const int t1 = min(p.T, t0 + p.tokens_per_block);
  const int nt = max(0, t1 - t0);
  const int np = nt * K;
  const int64_t p0 = (int64_t)t0 * K;
  int st = 0;

  for (int i = tid; i < kLayoutWaves * kMaxExperts; i += kLayoutThreads)
    (&s_wc[0][0])[i] = 0;
  for (int r = tid; r < R; r += kLayoutThreads) s_rc[r] = 0;
  if (tid == 0) s_status = 0;

  // Read the routing once; keep validated ids in LDS. A thread's (at most
  // kMaxPairsOneBlock / kLayoutThreads) loads are all issued before the first
  // is used (addresses clamped into the batch), so they cost one latency.
  constexpr int kIdsPerThread = kMaxPairsOneBlock / kLayoutThreads;
  if (np > 0) {
    int64_t v[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u)
      v[u] = p.idx[p0 + min(u * kLayoutThreads + tid, np - 1)];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = u * kLayoutThreads + tid;
      if (i < np) {
        const bool ok = v[u] >= 0 && v[u] < E;
        if (!ok && v[u] != -1) st |= kStBadExpert;
        s_ids[i] = ok ? (int16_t)v[u] : (int16_t)-1;
      }
    }
  }
  lds_barrier();

  // Per-wave counts over contiguous segments of 64-pair steps.
  const int seg = (((np + kLayoutWaves - 1) / kLayoutWaves) + 63) & ~63;
  const int s0 = wave * seg, s1 = min(np, s0 + seg);
  for (int b = s0; b < s1; b += 64) {
    const int i = b + lane;
    const int e = (i < s1) ? s_ids[i] : -1;
    const uint64_t peers = match_peers((uint32_t)e, e >= 0, p.id_bits);
    if (is_leader(peers)) s_wc[wave][e] += (uint16_t)__popcll(peers);
  }
  lds_barrier();

  // Exclusive prefix over waves for each expert; block totals.
  for (int e = tid; e < E; e += kLayoutThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int c = s_wc[w][e];
      s_wc[w][e] = (uint16_t)run;
      run += c;
    }
    s_cnt[e] = run;
  }
  lds_barrier();

  // First slot of each expert.
  if (kOneBlock) {
    const int e = tid;  // E <= 1024 = threads
    const int c = (e < E) ? s_cnt[e] : 0;
    const int padded = (p.mode == kModeContiguous) ? round_up(c, p.A) : 0;
    int total = 0;
    const int excl = block_exclusive_scan(padded, s_wave, kLayoutWaves, &total);
    if (e < E) {
      if (p.mode == kModeContiguous) {
        p.count[e] = c;
        if (p.recv_stats) p.recv_stats[e] += c;
        p.offset[e] = excl;
        if (e == E - 1) p.offset[E] = total;
        s_base[e] = excl;
        if (e == E - 1) s_base[E] = total;
      } else {
        const int base = (e * R + p.src) * p.M;
        p.count[e] = min(c, p.M);
        if (p.recv_stats) p.recv_stats[e] += min(c, p.M);
        if (c > p.M) st |= kStOverflow;
        if (p.offset) {
          p.offset[e] = base;
          if (e == E - 1) p.offset[E] = E * R * p.M;
        }
        s_base[e] = base;
      }
    }
    if (E == 0 && tid == 0 && p.mode == kModeContiguous) p.offset[0] = 0;
  } else {
    for (int e = tid; e < E; e += kLayoutThreads)
      p.ws_hist[(int64_t)e * p.nblocks + blockIdx.x] = s_cnt[e];
  }
  lds_barrier();

  // Stable ranks: walk the same segments again; a wave's running counter per
  // expert starts at the prefix of the waves before it.
  for (int b = s0; b < s1; b += 64) {
    const int i = b + lane;
    const bool in = i < s1;
    const int e = in ? s_ids[i] : -1;
    const uint64_t peers = match_peers((uint32_t)e, e >= 0, p.id_bits);
    if (in) {
      int out = -1;
      if (e >= 0) {
        const int j = (int)s_wc[wave][e] + below_me(peers);
        if (kOneBlock) {
          if (p.mode == kModeContiguous) {
            out = s_base[e] + j;
            if (p.row_src) p.row_src[out] = (int32_t)(p0 + i);
          } else if (j < p.M) {
            out = s_base[e] + j;
            if (p.row_src) p.row_src[(int64_t)e * p.M + j] = (int32_t)(p0 + i);
          } else {
            st |= kStOverflow;
          }
        } else {
          out = j;
        }
      }
      p.slot[p0 + i] = out;
    }
    if (is_leader(peers)) s_wc[wave][e] += (uint16_t)__popcll(peers);
  }

  // Which ranks each token reaches, and distinct tokens per rank.
  if (p.in_rank || p.rank_token_count) {
    const int n = nt * R;
    for (int b = 0; b < n; b += kLayoutThreads) {
      const int i = b + tid;
      bool hit = false;
      int r = 0;
      if (i < n) {
        const int tl = i / R;
        r = i - tl * R;
        // eight LDS reads in flight at a time (indexes clamped into the token)
        for (int k0 = 0; k0 < K; k0 += 8) {
          int e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = s_ids[tl * K + min(k0 + j, K - 1)];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            hit |= (e[j] >= 0) && (rank_of(e[j], p.l_magic) == r);
        }
        if (p.in_rank) p.in_rank[(int64_t)t0 * R + i] = hit ? 1 : 0;
      }
      const uint64_t peers = match_peers((uint32_t)r, hit, p.rank_bits);
      if (is_leader(peers)) atomicAdd(&s_rc[r], __popcll(peers));
    }
  }
  if (st) atomicOr(&s_status, st);
  lds_barrier();

  if (p.rank_token_count) {
    for (int r = tid; r < R; r += kLayoutThreads) {
      if (kOneBlock)
        p.rank_token_count[r] = s_rc[r];
      else
        p.ws_rcnt[(int64_t)r * p.nblocks + blockIdx.x] = s_rc[r];
    }
  }
  if (kOneBlock && p.row_src) {
    // Rows that hold no pair carry -1: the alignment padding after each
    // expert's rows, or the low-latency stripe rows past its received count.
    // Wave w takes experts w, w + 16, ...: its lanes read the experts' row
    // ranges at once, then store each range with consecutive lanes.
    for (int e0 = wave; e0 < E; e0 += kLayoutWaves * 64) {
      const int e = e0 + lane * kLayoutWaves;
      int lo = 0, hi = 0;
      if (e < E) {
        if (p.mode == kModeContiguous) {
          lo = s_base[e] + s_cnt[e];
          hi = s_base[e + 1];
        } else {
          lo = e * p.M + min(s_cnt[e], p.M);
          hi = (e + 1) * p.M;
        }
      }
      const int n = min(64, (E - e0 + kLayoutWaves - 1) / kLayoutWaves);
      for (int j = 0; j < n; ++j) {
        const int l = __builtin_amdgcn_readlane(lo, j), h = __builtin_amdgcn_readlane(hi, j);
        for (int r = l + lane; r < h; r += 64) p.row_src[r] = -1;
      }
    }
  }
  if (tid == 0 && s_status && p.status) atomicOr(p.status, s_status);
}

// Multi-block pass 2: one wave per expert (exclusive prefix of its per-block
// counts, in place, and its total) and one wave per rank (its token total).
__global__ __launch_bounds__(64) void layout_prefix_kernel(LayoutParams p) {
  const int lane = lane_id(), nb = p.nblocks;
  const int g = blockIdx.x;
  if (g < p.E) {
    // kPrefixLoads counts per lane are requested before the first is scanned
    // (one load latency per 64 * kPrefixLoads blocks), each 64 by a DPP scan
    constexpr int kPrefixLoads = 4;
    int32_t *h = p.ws_hist + (int64_t)g * nb;
    int carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 64 * kPrefixLoads) {
      int c[kPrefixLoads];
#pragma unroll
      for (int j = 0; j < kPrefixLoads; ++j) {
        const int b = b0 + 64 * j + lane;
        c[j] = b < nb ? h[b] : 0;
      }
#pragma unroll
      for (int j = 0; j < kPrefixLoads; ++j) {
        const int b = b0 + 64 * j + lane;
        const int x = wave_inclusive_sum(c[j]);
        if (b < nb) h[b] = carry + x - c[j];
        carry += __builtin_amdgcn_readlane(x, 63);
      }
    }
    if (lane == 0) p.ws_cnt[g] = carry;
  } else if (p.rank_token_count) {
    const int r = g - p.E;
    const int32_t *h = p.ws_rcnt + (int64_t)r * nb;
    int n = 0;
    for (int b = lane; b < nb; b += 64) n += h[b];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d, 64);
    if (lane == 0) p.rank_token_count[r] = n;
  }
}

// Multi-block pass 3: every workgroup scans the per-expert totals into the
// first row of each expert (cheap: E <= 1024), workgroup 0 writes the totals,
// the workgroups share the unfilled rows, then each thread fixes one pair:
// slot = first row of its expert + pairs of that expert in earlier blocks +
// its rank inside its own block.
constexpr int kFixupThreads = 256;

__global__ __launch_bounds__(kFixupThreads) void layout_fixup_kernel(LayoutParams p) {
  __shared__ int32_t s_base[kMaxExperts];
  __shared__ int32_t s_wave[kFixupThreads / 64];
  const int tid = threadIdx.x, E = p.E, R = p.R;
  const bool contiguous = p.mode == kModeContiguous;
  // this thread's pair: its id and in-block rank are requested first, so they
  // arrive while the expert totals are scanned (address clamped into the batch)
  const int64_t i = (int64_t)blockIdx.x * kFixupThreads + tid;
  const int64_t n = (int64_t)p.T * p.K;
  const int64_t ic = i < n ? i : n - 1;
  const int64_t v = p.idx[ic];
  const int32_t local = p.slot[ic];
  // aligned exclusive scan over experts (E/256 consecutive experts per thread)
  const int per = (E + kFixupThreads - 1) / kFixupThreads;
  const int e0 = tid * per;
  int sum = 0;
  for (int j = 0; j < per; ++j)
    if (e0 + j < E) sum += contiguous ? round_up(p.ws_cnt[e0 + j], p.A) : 0;
  int total = 0;
  int run = block_exclusive_scan(sum, s_wave, kFixupThreads / 64, &total);
  int st = 0;
  for (int j = 0; j < per; ++j) {
    const int e = e0 + j;
    if (e >= E) break;
    const int c = p.ws_cnt[e];
    const int base = contiguous ? run : (e * R + p.src) * p.M;
    s_base[e] = base;
    if (blockIdx.x == 0) {
      if (contiguous) {
        p.count[e] = c;
        if (p.recv_stats) p.recv_stats[e] += c;
        p.offset[e] = base;
      } else {
        p.count[e] = min(c, p.M);
        if (p.recv_stats) p.recv_stats[e] += min(c, p.M);
        if (c > p.M) st |= kStOverflow;
        if (p.offset) p.offset[e] = base;
      }
    }
    if (contiguous) run += round_up(c, p.A);
  }
  if (blockIdx.x == 0 && tid == 0 && p.offset) p.offset[E] = contiguous ? total : E * R * p.M;
  lds_barrier();

  // rows no pair fills carry -1 (alignment padding, or low-latency stripe rows
  // past the received count): expert e's go to workgroup e mod gridDim.x,
  // whose threads stride over them
  if (p.row_src) {
    for (int e = blockIdx.x; e < E; e += gridDim.x) {
      const int c = p.ws_cnt[e];
      if (contiguous) {
        const int hi = s_base[e] + round_up(c, p.A);
        for (int r = s_base[e] + c + tid; r < hi; r += kFixupThreads) p.row_src[r] = -1;
      } else {
        int32_t *stripe = p.row_src + (int64_t)e * p.M;
        for (int j2 = min(c, p.M) + tid; j2 < p.M; j2 += kFixupThreads) stripe[j2] = -1;
      }
    }
  }

  if (i < n) {
    if (v >= 0 && v < E) {  // other pairs already hold slot -1
      const int e = (int)v;
      const int b = (int)((i / p.K) / p.tokens_per_block);
      const int j = p.ws_hist[(int64_t)e * p.nblocks + b] + local;
      if (contiguous) {
        const int s = s_base[e] + j;
        p.slot[i] = s;
        if (p.row_src) p.row_src[s] = (int32_t)i;
      } else if (j < p.M) {
        p.slot[i] = s_base[e] + j;
        if (p.row_src) p.row_src[(int64_t)e * p.M + j] = (int32_t)i;
      } else {
        p.slot[i] = -1;
        st |= kStOverflow;
      }
    }
  }
  if (st && p.status) atomicOr(p.status, st);
}

// Per-expert load of the batch. Each workgroup histograms its share of the
// pairs in LDS (one leader lane per (wave, expert) per 64-pair step) and adds
// its non-zero bins to the output with global atomics; integer sums, so the
// result does not depend on their order. `zero` first clears the output.
constexpr int kLoadPairsPerBlock = 4096;

__global__ __launch_bounds__(kLayoutThreads) void load_zero_kernel(int32_t *load, int32_t E) {
  for (int e = threadIdx.x; e < E; e += kLayoutThreads) load[e] = 0;
}

__global__ __launch_bounds__(kLayoutThreads) void expert_load_kernel(const int64_t *idx,
                                                                     int32_t n, int32_t E,
                                                                     int32_t bits,
                                                                     int32_t *load,
                                                                     int32_t *status,
                                                                     int32_t per_block,
                                                                     int32_t accumulate) {
  __shared__ int32_t s_h[kMaxExperts];
  __shared__ int32_t s_status;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kLayoutThreads) s_h[e] = 0;
  if (tid == 0) s_status = 0;
  lds_barrier();
  int st = 0;
  const int i0 = blockIdx.x * per_block, i1 = min(n, i0 + per_block);
  for (int b = i0; b < i1; b += kLayoutThreads) {
    const int i = b + tid;
    int e = -1;
    if (i < i1) {
      const int64_t v = idx[i];
      if (v >= 0 && v < E)
        e = (int)v;
      else if (v != -1)
        st |= kStBadExpert;
    }
    const uint64_t peers = match_peers((uint32_t)e, e >= 0, bits);
    if (is_leader(peers)) atomicAdd(&s_h[e], __popcll(peers));
  }
  if (st) atomicOr(&s_status, st);
  lds_barrier();
  for (int e = tid; e < E; e += kLayoutThreads) {
    if (accumulate) {
      if (s_h[e]) atomicAdd(&load[e], s_h[e]);
    } else {
      load[e] = s_h[e];
    }
  }
  if (tid == 0 && s_status && status) atomicOr(status, s_status);
}

}  // namespace

hipError_t launch_layout_one_block(const LayoutParams &p, hipStream_t s) {
  hipLaunchKernelGGL(layout_block_kernel<true>, dim3(1), dim3(kLayoutThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_layout_multi_block(const LayoutParams &p, hipStream_t s) {
  hipLaunchKernelGGL(layout_block_kernel<false>, dim3(p.nblocks), dim3(kLayoutThreads), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(layout_prefix_kernel, dim3(p.E + p.R), dim3(64), 0, s, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = (int64_t)p.T * p.K;
  const int64_t blocks = (n + kFixupThreads - 1) / kFixupThreads;
  hipLaunchKernelGGL(layout_fixup_kernel, dim3((unsigned)blocks), dim3(kFixupThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_expert_load(const int64_t *idx, int32_t T, int32_t K, int32_t E,
                              int32_t id_bits, int32_t *load, int32_t *status, hipStream_t s) {
  const int32_t n = T * K;
  if (n <= kLoadPairsPerBlock) {  // one workgroup writes the result directly
    hipLaunchKernelGGL(expert_load_kernel, dim3(1), dim3(kLayoutThreads), 0, s, idx, n, E,
                       id_bits, load, status, kLoadPairsPerBlock, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(load_zero_kernel, dim3(1), dim3(kLayoutThreads), 0, s, load, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int blocks = (n + kLoadPairsPerBlock - 1) / kLoadPairsPerBlock;
  hipLaunchKernelGGL(expert_load_kernel, dim3(blocks), dim3(kLayoutThreads), 0, s, idx, n, E,
                     id_bits, load, status, kLoadPairsPerBlock, 1);
  return hipGetLastError();
}

}  // namespace moe
