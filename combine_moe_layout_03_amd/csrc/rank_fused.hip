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
  int32_t token_wgs;  // [0, token_wgs) serve tokens
  int32_t count_wgs;  // [0, count_wgs) also count experts b, b + count_wgs, ... (at most
                      // kRfDuties each); workgroups [token_wgs, count_wgs) only do that;
                      // workgroup count_wgs writes the rank offsets
};

// The routing as one lane sees it: tokens tid + 512 i (i < kRounds), their
// valid ids (-1 otherwise) and their sets of ranks.
template <int kRounds>
struct LaneTokens {
  int64_t raw[kRounds][kRfMaxK];
  int id[kRounds][kRfMaxK];
  uint64_t ranks[kRounds];

  // request the ids (addresses clamped into the routing; T >= 1)
  __device__ __forceinline__ void issue(const RankFusedParams &p) {
    const int w0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x & ~63);
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int t = min(i * kRfThreads + (int)threadIdx.x, p.T - 1);
      const int64_t *row = p.idx + (int64_t)t * p.K;
#pragma unroll
      for (int k = 0; k < kRfMaxK; ++k) raw[i][k] = -1;
      // waves whose lanes hold no token (and ids past K) request nothing
      if (i * kRfThreads + w0 < p.T) {
        if (p.K == kRfMaxK) {  // the token's 64-byte row in four 16-byte loads
          typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
          const i64x2 *row2 = reinterpret_cast<const i64x2 *>(row);
#pragma unroll
          for (int k = 0; k < kRfMaxK / 2; ++k) {
            const i64x2 q = row2[k];
            raw[i][2 * k] = q.x;
            raw[i][2 * k + 1] = q.y;
          }
        } else {
#pragma unroll
          for (int k = 0; k < kRfMaxK; ++k)
            if (k < p.K) raw[i][k] = row[k];
        }
      }
    }
    // every id load stays ahead of whatever the caller issues next (a row load)
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void settle(const RankFusedParams &p, int &st) {
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const bool live = i * kRfThreads + (int)threadIdx.x < p.T;
      uint64_t m = 0;
#pragma unroll
      for (int k = 0; k < kRfMaxK; ++k) {
        const int64_t e = raw[i][k];
        const bool in = live && k < p.K;
        const bool ok = in && e >= 0 && e < p.E;
        if (in && !ok && e != -1) st |= kStBadExpert;
        id[i][k] = ok ? (int)e : -1;
        if (ok) m |= 1ull << rank_of((int)e, p.l_magic);
      }
      ranks[i] = m;
    }
  }
  __device__ __forceinline__ void empty() {
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      ranks[i] = 0;
#pragma unroll
      for (int k = 0; k < kRfMaxK; ++k) id[i][k] = -1;
    }
  }
};

// Bits 0..3 of x to bits 0, 8, 16, 24: four one-byte counters that a sum over
// a wave's lanes (at most 2 * 64 per byte here) cannot carry out of.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return (x * 0x00204081u) & 0x01010101u; }

// This wave's pairs on experts b, b + G, ... (lane j: the j-th of them; at
// most kRfDuties), for the aligned receive counts. Every lane of the wave must
// call it.
template <int kRounds>
__device__ __forceinline__ int count_experts(const RankFusedParams &p,
                                             const LaneTokens<kRounds> &rt, int b, int G,
                                             int &ne) {
  ne = b < p.E ? (p.E - 1 - b) / G + 1 : 0;
  int cv = 0;
  for (int j = 0; j < ne; ++j) {
    const int e = b + j * G;
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int k = 0; k < kRfMaxK; ++k) n += __popcll(__ballot(rt.id[i][k] == e));
    cv = set_lane(cv, j, n);
  }
  return cv;
}

template <int kRounds>
__device__ void token_workgroup(const RankFusedParams &p, int b, int &st, int32_t *s_exp) {
  __shared__ int32_t s_cnt[64];  // per rank: tokens reaching it
  __shared__ int32_t s_pos[64];  // per rank: tokens before t reaching it
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = b / p.wg_per_token;  // < T
  const bool lead = b % p.wg_per_token == 0;
  const int K = p.K;
  if (tid < 64) {
    s_cnt[tid] = 0;
    s_pos[tid] = 0;
  }

  // 1. pair (t, lane mod K) and its weight (lanes 0..K-1 hold the token's K
  //    pairs; without weights the load reads id bits, unused: no branch
  //    around it) ...
  const int kl = lane % K;
  const int64_t *trow = p.idx + (int64_t)t * K;
  const int64_t te = trow[kl];
  const float *wsrc = p.w ? p.w : reinterpret_cast<const float *>(p.idx);
  const float tw = wsrc[(int64_t)t * K + kl];
  // 2. ... the routing ...
  LaneTokens<kRounds> rt;
  rt.issue(p);
  // 3. ... then the row chunk this wave copies, unconditionally (address
  //    clamped into the row), so it stays in flight while the rows are derived.
  //    Every wave's routing loads leave before any wave's row load (a barrier
  //    with no memory wait): routing loads issued after another wave's cold
  //    row load come back after it.
  __builtin_amdgcn_s_barrier();
  const int chunk = (b % p.wg_per_token) * p.chunks_per_wg + wave;
  const int v = chunk * 64 + lane;
  const bool lane_ok = wave < p.chunks_per_wg && chunk < p.nchunk && v < p.nvec;
  u32x4 val = __builtin_nontemporal_load(p.x + (int64_t)t * p.nvec + min(v, p.nvec - 1));
  __builtin_amdgcn_sched_barrier(0);  // nothing below waits before the row load is issued

  // 4. the token's set of ranks (uniform)
  const bool tok = te >= 0 && te < p.E;
  const int tr = tok ? rank_of((int)te, p.l_magic) : -1;  // rank of pair `lane` (lane < K)
  uint64_t mt = 0;
  for (int k = 0; k < K; ++k) {
    const int rk = __builtin_amdgcn_readlane(tr, k);
    if (rk >= 0) mt |= 1ull << rk;
  }
  const int rhi = mt ? 63 - __builtin_clzll(mt) : 0;  // highest rank reached
  const int nc = (rhi >> 3) + 1;                       // 8-rank groups up to it
  lds_barrier();  // the LDS counters are zero
  rt.settle(p, st);

  // 5. per rank r of the first nc groups, this wave's tokens reaching r and
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
    // this workgroup's share of the receive counts
    int ne;
    const int ev = count_experts(p, rt, b, p.count_wgs, ne);
    if (lane < ne) atomicAdd(&s_exp[lane], ev);
  }
  lds_barrier();
  if (p.recv_count && tid < kRfDuties && b + tid * p.count_wgs < p.E)
    p.recv_count[b + tid * p.count_wgs] = round_up(s_exp[tid], p.A);

  // 6. row of (t, r) in lane r: the tokens of the ranks below r (a scan over
  //    the lanes) plus the tokens before t on r
  const int n = s_cnt[lane];
  int row = wave_inclusive_sum(n) - n + s_pos[lane];
  const bool hit = (mt >> lane) & 1ull;
  if (!hit) {
    row = -1;
  } else if (row >= p.cap) {  // receive arrays smaller than the layout needs
    if (lead && wave == 0) st |= kStBadSlot;
    row = -1;
  }

  // 7. the row chunk, once per rank reached (row -1 for the others; rows are
  //    int32, so one unsigned compare against the clamped row count)
  asm volatile("" : "+v"(val));
  const uint32_t rows32 = p.rows < 0x7fffffff ? (uint32_t)p.rows : 0x7fffffffu;
  u32x4 *dst = p.recv + v;
  if (p.R == 8) {  // the eight rows first, then the stores back to back
    int sl[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) sl[r] = __builtin_amdgcn_readlane(row, r);
    if (lane_ok) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if ((uint32_t)sl[r] < rows32) __builtin_nontemporal_store(val, dst + (int64_t)sl[r] * p.nvec);
    }
    if (lead && wave == 0) {  // receive buffer smaller than the layout needs
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if ((uint32_t)sl[r] >= rows32 && sl[r] != -1) st |= kStBadSlot;
    }
  } else {
    for (uint64_t rest = mt; rest; rest &= rest - 1ull) {
      const int s = __builtin_amdgcn_readlane(row, __ffsll((unsigned long long)rest) - 1);
      if ((uint32_t)s < rows32) {
        if (lane_ok) __builtin_nontemporal_store(val, dst + (int64_t)s * p.nvec);
      } else if (s != -1 && lead && wave == 0) {
        st |= kStBadSlot;  // receive buffer smaller than the layout needs
      }
    }
  }

  // 8. the token's handle entries
  if (lead && wave == 0) {
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
      if (p.recv_w && p.w) p.recv_w[(int64_t)jr * K + kl] = loc ? tw : 0.0f;
    }
  }
  st &= ~kStBadExpert;  // every workgroup reads every id; the duty workgroups report
}

// Workgroups with no token: receive counts (b < count_wgs, written by the
// kernel after its last barrier), or the rank offsets (b == count_wgs).
template <int kRounds>
__device__ void duty_workgroup(const RankFusedParams &p, int b, int &st, int32_t *s_exp) {
  __shared__ int32_t s_c[kRfWaves][64];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  LaneTokens<kRounds> rt;
  if (p.T > 0) {
    rt.issue(p);
    rt.settle(p, st);
  } else {
    rt.empty();
  }
  lds_barrier();  // s_exp is zero
  if (b < p.count_wgs) {
    int ne;
    const int ev = count_experts(p, rt, b, p.count_wgs, ne);
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

template <int kRounds>
__global__ __launch_bounds__(kRfThreads) void rank_layout_dispatch_kernel(RankFusedParams p) {
  __shared__ int32_t s_status;
  __shared__ int32_t s_exp[kRfDuties];  // pairs on this workgroup's experts
  const int tid = threadIdx.x, b = blockIdx.x;
  int st = 0;
  if (tid == 0) s_status = 0;
  if (tid < kRfDuties) s_exp[tid] = 0;
  if (b < p.token_wgs)  // uniform per workgroup
    token_workgroup<kRounds>(p, b, st, s_exp);
  else
    duty_workgroup<kRounds>(p, b, st, s_exp);
  if (st) atomicOr(&s_status, st);
  lds_barrier();
  if (tid == 0 && s_status && p.status) atomicOr(p.status, s_status);
  if (b >= p.token_wgs && b < p.count_wgs && p.recv_count && tid < kRfDuties &&
      b + tid * p.count_wgs < p.E)
    p.recv_count[b + tid * p.count_wgs] = round_up(s_exp[tid], p.A);
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
  p.nvec = H / 8;
  p.nchunk = (p.nvec + 63) / 64;
  const int groups = (p.nchunk + kRfChunks - 1) / kRfChunks;
  p.chunks_per_wg = (p.nchunk + groups - 1) / groups;  // <= kRfChunks = waves
  p.wg_per_token = (p.nchunk + p.chunks_per_wg - 1) / p.chunks_per_wg;
  p.token_wgs = T * p.wg_per_token;
  const int need = (E + kRfDuties - 1) / kRfDuties;
  p.count_wgs = p.token_wgs > need ? p.token_wgs : need;
  const dim3 grid((unsigned)(p.count_wgs + 1)), block(kRfThreads);
  if (T <= kRfThreads)
    hipLaunchKernelGGL(rank_layout_dispatch_kernel<1>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(rank_layout_dispatch_kernel<2>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
