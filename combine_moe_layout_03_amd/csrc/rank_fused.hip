// Normal-mode layout and dispatch in one launch, for batches of at most 1024
// tokens with K <= 8: the same results, bit for bit, as the rank layout
// followed by the rank scatter (ranks.hip, scatter.hip), after the NeMo
// AutoModel page "nemo_automodel.components.moe.uccl_ep.buffer"
// (Buffer.dispatch in normal mode: is_token_in_rank, num_tokens_per_rank,
// recv_topk_idx, recv_topk_weights and the per-expert receive counts).
//
// Rank r's rows follow the rows of every lower rank, in token order, so
//   row(t, r) = sum over r' < r of n(r')  +  #(tokens t' < t that reach r),
// with n(r') the number of tokens that reach rank r'. A lane holds the set of
// ranks of one token (two for batches above 512) as a 64-bit mask, so each
// term is one ballot of a mask bit and a popcount, and a workgroup serving
// token t derives its rows with no help from any other workgroup. As in the
// low-latency counting kernel (fused.hip), a row is split over workgroups of
// 8 waves (two for a 7168-wide row): each requests the routing, then its row
// chunk, counts while the chunk is in flight and stores it once per rank the
// token reaches. Each workgroup also counts the pairs of one or a few experts
// (the aligned receive counts; duty workgroups with no token take the rest
// when there are few tokens), and one more workgroup writes the rank offsets.
#include "wave.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRfThreads = 512;  // 8 waves; every wave counts
constexpr int kRfWaves = kRfThreads / 64;
constexpr int kRfChunks = 8;     // row chunks of 64 x 16 bytes per workgroup, at most
constexpr int kRfMaxK = 8;
constexpr int kRfMaxTokens = 2 * kRfThreads;  // two tokens per lane
constexpr int kRfDuties = 4;     // experts whose pairs one workgroup counts, at most

struct RankFusedParams {
  const int64_t *idx;  // [T*K]
  const float *w;      // [T*K] may be null
  int32_t T, K, E, R, L, A;
  uint64_t l_magic;
  int32_t *rank_slot;    // [T*R]
  int32_t *rank_offset;  // [R+1]
  int32_t *recv_src;     // [cap] may be null
  int64_t *recv_idx;     // [cap*K] may be null
  float *recv_w;         // [cap*K] may be null
  int32_t *recv_count;   // [E] may be null
  int64_t cap;
  int32_t *status;
  const u32x4 *x;  // [T, nvec]
  u32x4 *recv;     // [rows, nvec]
  int64_t rows;
  int32_t nvec, nchunk, chunks_per_wg, wg_per_token;
  uint64_t wpt_magic;  // ceil(2^32 / wg_per_token)
  int32_t token_wgs;  // [0, token_wgs) serve tokens
  int32_t count_wgs;  // [0, count_wgs) also count experts b, b + count_wgs, ... (at most
                      // kRfDuties each); workgroups [token_wgs, count_wgs) only do that;
                      // workgroup count_wgs writes the rank offsets
};

// The routing in two views. Read as it lies in memory -- pair i * 512 + tid
// in round i, one 8-byte load per pair, every wave taking part, so each load
// instruction covers 512 contiguous bytes -- a lane keeps its pairs' valid ids
// (for the receive counts) and writes their ranks, one byte each, into an LDS
// table with one 8-byte row per token. After a barrier a lane reads the rows
// of tokens tid + 512 j (j < kRounds) and holds those tokens' sets of ranks.
// (Each lane reading its own token's 64 bytes as four 16-byte loads, from
// two waves only, brought the routing in 0.36 us later and the row chunk,
// which returns behind it, as much later.) kPairRounds, the pair rounds
// compiled, is the launch's ceil(T * K / 512) rounded up to a power of two:
// the few-microsecond kernel pays for every instruction-cache line its waves
// run through, so no unused round is unrolled.
template <int kRounds, int kPairRounds>
struct LaneTokens {
  int64_t raw[kPairRounds];
  int pid[kPairRounds];  // the id of pair i * 512 + tid if valid, else -1
  uint64_t ranks[kRounds];

  // request the pairs (addresses clamped into the routing)
  __device__ __forceinline__ void issue(const int64_t *idx, int P) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPairRounds; ++i) {
      raw[i] = -1;
      if (i * kRfThreads < P) raw[i] = idx[min(i * kRfThreads + tid, P - 1)];  // uniform
    }
    // every id load stays ahead of whatever the caller issues next (a row load)
    __builtin_amdgcn_sched_barrier(0);
  }
  // validate the pairs (bad ids flagged) and write their rank bytes (0xff:
  // no expert) into row q / K, byte q mod K of the table
  __device__ __forceinline__ void settle(const RankFusedParams &p, int P, uint8_t *s_rk,
                                         int &st) {
    const int tid = threadIdx.x;
    // q / K by a multiply: the reciprocal's error times q stays under
    // 2^13 / 2^18 = 1/32 for q < P <= 2^13, below the 1/K >= 1/8 gap
    // between q / K and the next integer; q * kmag < 2^32
    const uint32_t kmag = (1u << 18) / (uint32_t)p.K + 1u;
#pragma unroll
    for (int i = 0; i < kPairRounds; ++i) {
      const int q = i * kRfThreads + tid;
      const bool in = q < P;
      const int64_t e = raw[i];
      const bool ok = in && e >= 0 && e < p.E;
      if (in && !ok && e != -1) st |= kStBadExpert;
      pid[i] = ok ? (int)e : -1;
      if (in) {
        const int tt = (int)(((uint32_t)q * kmag) >> 18);
        s_rk[tt * kRfMaxK + (q - tt * p.K)] =
            ok ? (uint8_t)rank_of((int)e, p.l_magic) : (uint8_t)0xffu;
      }
    }
  }
  // after the barrier that follows every settle: the sets of ranks
  __device__ __forceinline__ void gather(const RankFusedParams &p, const uint8_t *s_rk) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int tt = j * kRfThreads + (int)threadIdx.x;
      ranks[j] = tt < p.T ? rank_set(*reinterpret_cast<const uint64_t *>(s_rk + tt * kRfMaxK), p.K)
                          : 0ull;
    }
  }
  // the set of ranks of a token's row of rank bytes (the first K of them)
  static __device__ __forceinline__ uint64_t rank_set(uint64_t row, int K) {
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < kRfMaxK; ++k) {
      const uint32_t r = (uint32_t)(row >> (8 * k)) & 0xffu;
      if (k < K && r != 0xffu) m |= 1ull << r;
    }
    return m;
  }
};

// Bits 0..3 of x to bits 0, 8, 16, 24: four one-byte counters that a sum over
// a wave's lanes (at most 2 * 64 per byte here) cannot carry out of.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return (x * 0x00204081u) & 0x01010101u; }

// This wave's pairs on experts b, b + G, ... (lane j: the j-th of them; at
// most kRfDuties), for the aligned receive counts. Every lane of the wave must
// call it.
template <int kRounds, int kPR>
__device__ __forceinline__ int count_experts(const RankFusedParams &p,
                                             const LaneTokens<kRounds, kPR> &rt, int P, int b,
                                             int G, int &ne) {
  ne = b < p.E ? (p.E - 1 - b) / G + 1 : 0;
  int cv = 0;
  for (int j = 0; j < ne; ++j) {
    const int e = b + j * G;
    int n = 0;
#pragma unroll
    for (int i = 0; i < kPR; ++i)
      if (i * kRfThreads < P) n += __popcll(__ballot(rt.pid[i] == e));  // uniform
    cv = set_lane(cv, j, n);
  }
  return cv;
}

// kCopy false: the layout alone (no row chunk read or stored; one workgroup
// per token).
template <bool kCopy, int kRounds, int kPR>
__device__ void token_workgroup(const RankFusedParams &p, int b, int &st, int32_t *s_exp,
                                uint8_t *s_rk) {
  __shared__ int32_t s_cnt[64];  // per rank: tokens reaching it
  __shared__ int32_t s_pos[64];  // per rank: tokens before t reaching it
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // b / wg_per_token by the reciprocal (exact while b * wg_per_token < 2^32)
  const int t = (int)(((uint64_t)(uint32_t)b * p.wpt_magic) >> 32);  // < T
  const int part = b - t * p.wg_per_token;  // workgroup within the token
  const bool lead = part == 0;
  // the last wave writes the handle entries and reports bad rows: it copies
  // nothing for 7168-wide rows (7 chunks), so those stores do not queue behind
  // a row's stores
  constexpr int hw = kRfWaves - 1;
  const int K = p.K, P = p.T * K;
  if (tid < 64) {
    s_cnt[tid] = 0;
    s_pos[tid] = 0;
  }

  // 1. the routing first ...
  LaneTokens<kRounds, kPR> rt;
  rt.issue(p.idx, P);
  // 2. ... then the row chunk this wave copies, unconditionally (address
  //    clamped into the row), so it stays in flight while the rows are derived.
  //    Every wave's routing loads leave before any wave's row load (a barrier
  //    with no memory wait): routing loads issued after another wave's cold
  //    row load come back after it.
  u32x4 val = {0u, 0u, 0u, 0u};
  int v = 0;
  bool lane_ok = false;
  if (kCopy) {
    __builtin_amdgcn_s_barrier();
    const int chunk = part * p.chunks_per_wg + wave;
    v = chunk * 64 + lane;
    lane_ok = wave < p.chunks_per_wg && chunk < p.nchunk && v < p.nvec;
    val = __builtin_nontemporal_load(p.x + (int64_t)t * p.nvec + min(v, p.nvec - 1));
    __builtin_amdgcn_sched_barrier(0);  // nothing below waits before the row load is issued
  }

  // 3. the rank table; after the barrier each lane takes its tokens' sets of
  //    ranks, and every lane the row of token t: its set of ranks (uniform)
  //    and, in lane j, the rank of pair j mod K (-1: no expert)
  rt.settle(p, P, s_rk, st);
  lds_barrier();  // the rank table is whole, the LDS counters are zero
  rt.gather(p, s_rk);
  const int kl = lane % K;
  const uint64_t trow = *reinterpret_cast<const uint64_t *>(s_rk + t * kRfMaxK);
  const uint32_t trk = (uint32_t)(trow >> (8 * kl)) & 0xffu;
  const int tr = trk == 0xffu ? -1 : (int)trk;
  const uint64_t mt = LaneTokens<kRounds, kPR>::rank_set(trow, K);
  const int rhi = mt ? 63 - __builtin_clzll(mt) : 0;  // highest rank reached
  const int nc = (rhi >> 3) + 1;                       // 8-rank groups up to it

  // 4. per rank r of the first nc groups, this wave's tokens reaching r and
  //    its tokens before t reaching r: one byte counter per rank, summed over
  //    the wave by DPP; lane r takes rank r's counts. Waves that hold no token
  //    add nothing.
  if (wave * 64 < p.T) {  // uniform
    int cv = 0, pv = 0;
    for (int c = 0; c < nc; ++c) {
      uint32_t alo = 0, ahi = 0, elo = 0, ehi = 0;
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const uint32_t a = (uint32_t)(rt.ranks[i] >> (8 * c)) & 0xffu;
        const uint32_t e = (i * kRfThreads + tid < t) ? a : 0u;
        alo += spread4(a & 15u);
        ahi += spread4(a >> 4);
        elo += spread4(e & 15u);
        ehi += spread4(e >> 4);
      }
      const uint32_t sal = wave_sum(alo), sah = wave_sum(ahi);
      const uint32_t sel = wave_sum(elo), seh = wave_sum(ehi);
      if ((lane >> 3) == c) {
        const int sh = 8 * (lane & 3);
        cv = (int)(((lane & 4) ? sah : sal) >> sh & 0xffu);
        pv = (int)(((lane & 4) ? seh : sel) >> sh & 0xffu);
      }
    }
    if (lane < 8 * nc) {
      atomicAdd(&s_cnt[lane], cv);
      atomicAdd(&s_pos[lane], pv);
    }
  }
  {  // this workgroup's share of the receive counts (every wave holds pairs)
    int ne;
    const int ev = count_experts(p, rt, P, b, p.count_wgs, ne);
    if (lane < ne) atomicAdd(&s_exp[lane], ev);
  }
  lds_barrier();
  if (p.recv_count && tid < kRfDuties && b + tid * p.count_wgs < p.E)
    p.recv_count[b + tid * p.count_wgs] = round_up(s_exp[tid], p.A);

  // 5. row of (t, r) in lane r: the tokens of the ranks below r (a scan over
  //    the lanes) plus the tokens before t on r
  const int n = s_cnt[lane];
  int row = wave_inclusive_sum(n) - n + s_pos[lane];
  const bool hit = (mt >> lane) & 1ull;
  if (!hit) {
    row = -1;
  } else if (row >= p.cap) {  // receive arrays smaller than the layout needs
    if (lead && wave == hw) st |= kStBadSlot;
    row = -1;
  }

  // 6. the row chunk, once per rank reached (row -1 for the others; rows are
  //    int32, so one unsigned compare against the clamped row count)
  if (!kCopy) {
  } else if (p.R == 8) {  // the eight rows first, then the stores back to back
    asm volatile("" : "+v"(val));
    const uint32_t rows32 = p.rows < 0x7fffffff ? (uint32_t)p.rows : 0x7fffffffu;
    u32x4 *dst = p.recv + v;
    int sl[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) sl[r] = __builtin_amdgcn_readlane(row, r);
    if (lane_ok) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if ((uint32_t)sl[r] < rows32) __builtin_nontemporal_store(val, dst + (int64_t)sl[r] * p.nvec);
    }
    if (lead && wave == hw) {  // receive buffer smaller than the layout needs
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if ((uint32_t)sl[r] >= rows32 && sl[r] != -1) st |= kStBadSlot;
    }
  } else {
    asm volatile("" : "+v"(val));
    const uint32_t rows32 = p.rows < 0x7fffffff ? (uint32_t)p.rows : 0x7fffffffu;
    u32x4 *dst = p.recv + v;
    for (uint64_t rest = mt; rest; rest &= rest - 1ull) {
      const int s = __builtin_amdgcn_readlane(row, __ffsll((unsigned long long)rest) - 1);
      if ((uint32_t)s < rows32) {
        if (lane_ok) __builtin_nontemporal_store(val, dst + (int64_t)s * p.nvec);
      } else if (s != -1 && lead && wave == hw) {
        st |= kStBadSlot;  // receive buffer smaller than the layout needs
      }
    }
  }

  // 7. the token's handle entries; the pairs' ids and weights are read here,
  //    by this wave only (a CU returns loads in issue order, so read ahead of
  //    the routing they would hold it back)
  if (lead && wave == hw) {
    const int64_t te = p.idx[(int64_t)t * K + kl];
    if (lane < p.R) p.rank_slot[(int64_t)t * p.R + lane] = row;
    if (row >= 0 && p.recv_src) p.recv_src[row] = t;
    // entry (j, k) of the rows' local ids and weights in lane j*K + k (at
    // most 64 of them: a token reaches at most K ranks)
    const int jl = lane / K;
    int rj = -1, jr = -1, j = 0;
    for (uint64_t rest = mt; rest; rest &= rest - 1ull, ++j) {
      const int r = __ffsll((unsigned long long)rest) - 1;
      const int rr = __builtin_amdgcn_readlane(row, r);
      if (jl == j) {
        rj = r;
        jr = rr;
      }
    }
    if (jr >= 0) {
      const bool loc = tr == rj;  // the pair's expert lives on the row's rank
      if (p.recv_idx) p.recv_idx[(int64_t)jr * K + kl] = loc ? te - (int64_t)rj * p.L : -1;
      if (p.recv_w && p.w) p.recv_w[(int64_t)jr * K + kl] = loc ? p.w[(int64_t)t * K + kl] : 0.0f;
    }
  }
  st &= ~kStBadExpert;  // every workgroup reads every id; the duty workgroups report
}

// Workgroups with no token: receive counts (b < count_wgs, written by the
// kernel after its last barrier), or the rank offsets (b == count_wgs).
template <int kRounds, int kPR>
__device__ void duty_workgroup(const RankFusedParams &p, int b, int &st, int32_t *s_exp,
                               uint8_t *s_rk) {
  __shared__ int32_t s_c[kRfWaves][64];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = p.T * p.K;  // 0 for an empty batch: nothing is read
  LaneTokens<kRounds, kPR> rt;
  rt.issue(p.idx, P);
  rt.settle(p, P, s_rk, st);
  lds_barrier();  // the rank table is whole, s_exp is zero
  rt.gather(p, s_rk);
  if (b < p.count_wgs) {
    int ne;
    const int ev = count_experts(p, rt, P, b, p.count_wgs, ne);
    if (lane < ne) atomicAdd(&s_exp[lane], ev);
  } else {
    // rank offsets: exclusive sum of the tokens reaching each rank
    int cv = 0;
    for (int r = 0; r < p.R; ++r) {
      int n = 0;
#pragma unroll
      for (int i = 0; i < kRounds; ++i) n += __popcll(__ballot((rt.ranks[i] >> r) & 1ull));
      cv = set_lane(cv, r, n);
    }
    s_c[wave][lane] = cv;
    lds_barrier();
    if (wave == 0) {
      int n = 0;
      for (int w = 0; w < kRfWaves; ++w) n += s_c[w][lane];
      if (lane >= p.R) n = 0;
      const int incl = wave_inclusive_sum(n);
      if (lane < p.R) p.rank_offset[lane] = incl - n;
      if (lane == p.R - 1) p.rank_offset[p.R] = incl;
    }
  }
}

template <bool kCopy, int kRounds, int kPR>
__global__ __launch_bounds__(kRfThreads) void rank_layout_dispatch_kernel(RankFusedParams p) {
  __shared__ int32_t s_exp[kRfDuties];  // pairs on this workgroup's experts
  // per token its pairs' ranks, one byte each (0xff: no expert), 8 per row
  __shared__ __align__(8) uint8_t s_rk[kRfMaxTokens * kRfMaxK];
  const int tid = threadIdx.x, b = blockIdx.x;
  int st = 0;
  if (tid < kRfDuties) s_exp[tid] = 0;
  if (b < p.token_wgs) {  // uniform per workgroup
    token_workgroup<kCopy, kRounds, kPR>(p, b, st, s_exp, s_rk);
  } else {
    duty_workgroup<kRounds, kPR>(p, b, st, s_exp, s_rk);
    lds_barrier();  // every wave's receive counts are in s_exp
    if (b < p.count_wgs && p.recv_count && tid < kRfDuties && b + tid * p.count_wgs < p.E)
      p.recv_count[b + tid * p.count_wgs] = round_up(s_exp[tid], p.A);
  }
  // error bits (rare) go straight to the status word: no barrier ends a token
  // workgroup, so each wave leaves as soon as its own work is out
  if (st && p.status) atomicOr(p.status, st);
}

// The kernel instance for the batch: pair rounds ceil(T * K / 512) rounded up
// to a power of two (T * K <= 8192).
template <bool kCopy>
void launch_rounds(const RankFusedParams &p, dim3 grid, dim3 block, hipStream_t s) {
  const int pr = (p.T * p.K + kRfThreads - 1) / kRfThreads;
  if (p.T <= kRfThreads) {
    if (pr <= 1)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 1, 1>), grid, block, 0, s, p);
    else if (pr <= 2)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 1, 2>), grid, block, 0, s, p);
    else if (pr <= 4)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 1, 4>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 1, 8>), grid, block, 0, s, p);
  } else {
    if (pr <= 2)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 2, 2>), grid, block, 0, s, p);
    else if (pr <= 4)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 2, 4>), grid, block, 0, s, p);
    else if (pr <= 8)
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 2, 8>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((rank_layout_dispatch_kernel<kCopy, 2, 16>), grid, block, 0, s, p);
  }
}

}  // namespace

bool rank_layout_dispatch_fits(int32_t T, int32_t K, int32_t R) {
  return T <= kRfMaxTokens && K <= kRfMaxK && R <= 64;
}

hipError_t launch_rank_layout_dispatch(const int64_t *idx, const float *w, int32_t T, int32_t K,
                                       int32_t E, int32_t R, int32_t A, int32_t *rank_slot,
                                       int32_t *rank_offset, int32_t *recv_src,
                                       int64_t *recv_idx, float *recv_w, int32_t *recv_count,
                                       int64_t cap, int32_t *status, const uint16_t *x,
                                       uint16_t *recv, int64_t rows, int32_t H, hipStream_t s) {
  if (!rank_layout_dispatch_fits(T, K, R)) return hipErrorInvalidValue;
  RankFusedParams p;
  p.idx = idx;
  p.w = w;
  p.T = T;
  p.K = K;
  p.E = E;
  p.R = R;
  p.L = E / R;
  p.A = A;
  p.l_magic = ((1ull << 32) + (uint64_t)p.L - 1) / (uint64_t)p.L;
  p.rank_slot = rank_slot;
  p.rank_offset = rank_offset;
  p.recv_src = recv_src;
  p.recv_idx = recv_idx;
  p.recv_w = recv_w;
  p.recv_count = recv_count;
  p.cap = cap;
  p.status = status;
  p.x = reinterpret_cast<const u32x4 *>(x);
  p.recv = reinterpret_cast<u32x4 *>(recv);
  p.rows = rows;
  p.nvec = x ? H / 8 : 0;
  p.nchunk = (p.nvec + 63) / 64;
  const int groups = (p.nchunk + kRfChunks - 1) / kRfChunks;
  p.chunks_per_wg = x ? (p.nchunk + groups - 1) / groups : 0;  // <= kRfChunks = waves
  p.wg_per_token = x ? (p.nchunk + p.chunks_per_wg - 1) / p.chunks_per_wg : 1;
  p.wpt_magic = ((1ull << 32) + (uint64_t)p.wg_per_token - 1) / p.wg_per_token;
  p.token_wgs = T * p.wg_per_token;
  const int need = (E + kRfDuties - 1) / kRfDuties;
  p.count_wgs = p.token_wgs > need ? p.token_wgs : need;
  const dim3 grid((unsigned)(p.count_wgs + 1)), block(kRfThreads);
  if (x)
    launch_rounds<true>(p, grid, block, s);
  else
    launch_rounds<false>(p, grid, block, s);
  return hipGetLastError();
}

}  // namespace moe
