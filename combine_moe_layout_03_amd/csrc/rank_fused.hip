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
// token reaches. A few duty workgroups write the totals: the aligned receive
// count of each expert, and the rank offsets.
#include "wave.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRfThreads = 512;  // 8 waves; every wave counts
constexpr int kRfWaves = kRfThreads / 64;
constexpr int kRfChunks = 8;     // row chunks of 64 x 16 bytes per workgroup, at most
constexpr int kRfMaxK = 8;
constexpr int kRfMaxTokens = 2 * kRfThreads;  // two tokens per lane
constexpr int kRfDuties = 4;     // experts whose receive counts one duty workgroup writes

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
  int32_t token_wgs;   // [0, token_wgs) serve tokens
  int32_t expert_wgs;  // then expert_wgs duty workgroups for the receive counts, then one
                       // for the rank offsets
};

__device__ __forceinline__ int set_lane(int v, int j, int x) { return lane_id() == j ? x : v; }

// The routing as one lane sees it: tokens tid + 512 i (i < kRounds), their
// valid ids (-1 otherwise) and their sets of ranks.
template <int kRounds>
struct LaneTokens {
  int64_t raw[kRounds][kRfMaxK];
  int id[kRounds][kRfMaxK];
  uint64_t ranks[kRounds];

  // request the ids (addresses clamped into the routing; T >= 1)
  __device__ __forceinline__ void issue(const RankFusedParams &p) {
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int t = min(i * kRfThreads + (int)threadIdx.x, p.T - 1);
      const int64_t *row = p.idx + (int64_t)t * p.K;
#pragma unroll
      for (int k = 0; k < kRfMaxK; ++k) raw[i][k] = row[min(k, p.K - 1)];
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

// Inclusive sum over the lanes of a wave (every lane must call it).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

template <int kRounds>
__device__ void token_workgroup(const RankFusedParams &p, int b, int &st) {
  __shared__ int32_t s_cnt[64];       // per rank below the token's highest: tokens reaching it
  __shared__ int32_t s_pos[kRfMaxK];  // per rank of the token: tokens before t reaching it
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = b / p.wg_per_token;  // < T
  const bool lead = b % p.wg_per_token == 0;
  const int K = p.K;
  if (tid < 64) s_cnt[tid] = 0;
  if (tid < kRfMaxK) s_pos[tid] = 0;

  // 1. the routing, and this token's ids and weights (lane k holds pair k) ...
  LaneTokens<kRounds> rt;
  rt.issue(p);
  const int kk = min(lane, K - 1);
  const int64_t te = p.idx[(int64_t)t * K + kk];
  // (without weights the load reads id bits, unused: no branch around it)
  const float *wsrc = p.w ? p.w : reinterpret_cast<const float *>(p.idx);
  const float tw = wsrc[(int64_t)t * K + kk];
  // 2. ... then the row chunk this wave copies, unconditionally (address
  //    clamped into the row), so it stays in flight while the rows are derived
  const int chunk = (b % p.wg_per_token) * p.chunks_per_wg + wave;
  const int v = chunk * 64 + lane;
  const bool lane_ok = wave < p.chunks_per_wg && chunk < p.nchunk && v < p.nvec;
  u32x4 val = __builtin_nontemporal_load(p.x + (int64_t)t * p.nvec + min(v, p.nvec - 1));
  lds_barrier();  // the LDS counters are zero
  rt.settle(p, st);

  // 3. the token's set of ranks (uniform), and the masks of earlier tokens
  const bool tk = lane < K && te >= 0 && te < p.E;
  const int tr = tk ? rank_of((int)te, p.l_magic) : -1;  // rank of pair `lane`
  uint64_t mt = 0;
  for (int k = 0; k < K; ++k) {
    const int rk = __builtin_amdgcn_readlane(tr, k);
    if (rk >= 0) mt |= 1ull << rk;
  }
  uint64_t early[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) early[i] = (i * kRfThreads + tid < t) ? rt.ranks[i] : 0ull;
  const int nj = __popcll(mt);
  const int rhi = mt ? 63 - __builtin_clzll(mt) : 0;  // ranks below the highest reached

  // 4. this wave's share of n(r') for r' < rhi (lane r'), and of the tokens
  //    before t on the token's j-th rank (lane j)
  int cv = 0;
  for (int r = 0; r < rhi; ++r) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) n += __popcll(__ballot((rt.ranks[i] >> r) & 1ull));
    cv = set_lane(cv, r, n);
  }
  int pv = 0, rjv = 0;
  uint64_t rest = mt;
  for (int j = 0; j < nj; ++j) {
    const int rj = __ffsll((unsigned long long)rest) - 1;
    rest &= rest - 1ull;
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) n += __popcll(__ballot((early[i] >> rj) & 1ull));
    pv = set_lane(pv, j, n);
    rjv = set_lane(rjv, j, rj);
  }
  if (lane < rhi) atomicAdd(&s_cnt[lane], cv);
  if (lane < nj) atomicAdd(&s_pos[lane], pv);
  lds_barrier();

  // 5. rows: lane r' sums the ranks below it; lane j gets the row on rank r_j
  const int c = lane < rhi ? s_cnt[lane] : 0;
  const int start = wave_inclusive_sum(c) - c;
  int row = 0;
  for (int j = 0; j < nj; ++j) row = set_lane(row, j, __builtin_amdgcn_readlane(start, __builtin_amdgcn_readlane(rjv, j)));
  if (lane < nj) {
    row += s_pos[lane];
    if (row >= p.cap) {  // receive arrays smaller than the layout needs
      if (lead && wave == 0) st |= kStBadSlot;
      row = -1;
    }
  } else {
    row = -1;
  }

  // 6. the row chunk, once per rank reached
  asm volatile("" : "+v"(val));
  for (int j = 0; j < nj; ++j) {
    const int s = __builtin_amdgcn_readlane(row, j);
    if (s >= 0 && s < p.rows) {
      if (lane_ok) __builtin_nontemporal_store(val, p.recv + (int64_t)s * p.nvec + v);
    } else if (s != -1 && lead && wave == 0) {
      st |= kStBadSlot;  // receive buffer smaller than the layout needs
    }
  }

  // 7. the token's handle entries (all 64 lanes of wave 0 take part in the
  //    shuffles)
  if (lead && wave == 0) {
    const int below = __popcll(mt & ((1ull << lane) - 1ull));  // lane = rank r
    const int rrow = __shfl(row, below, 64);
    if (lane < p.R) p.rank_slot[(int64_t)t * p.R + lane] = ((mt >> lane) & 1ull) ? rrow : -1;
    if (lane < nj && row >= 0 && p.recv_src) p.recv_src[row] = t;
    // entry (j, k) of the rows' local ids and weights in lane j*K + k (nj*K <= 64)
    const int j = lane / K, k = lane - j * K;
    const int jr = __shfl(row, j & 63, 64);
    const int rj = __shfl(rjv, j & 63, 64);
    const int rk = __shfl(tr, k, 64);
    const int ek = __shfl((int)te, k, 64);
    const float wk = __shfl(tw, k, 64);
    if (j < nj && jr >= 0) {
      const bool loc = rk == rj;  // the pair's expert lives on the row's rank
      if (p.recv_idx) p.recv_idx[(int64_t)jr * K + k] = loc ? (int64_t)(ek - rj * p.L) : -1;
      if (p.recv_w && p.w) p.recv_w[(int64_t)jr * K + k] = loc ? wk : 0.0f;
    }
  }
  st &= ~kStBadExpert;  // every workgroup reads every id; the duty workgroups report
}

template <int kRounds>
__device__ void duty_workgroup(const RankFusedParams &p, int d, int &st) {
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
  if (d < p.expert_wgs) {
    // receive counts of experts d, d + D, ... (pairs, duplicates included)
    const int D = p.expert_wgs;
    const int nd = d < p.E ? (p.E - 1 - d) / D + 1 : 0;  // <= kRfDuties
    int cv = 0;
    for (int j = 0; j < nd; ++j) {
      const int e = d + j * D;
      int n = 0;
#pragma unroll
      for (int i = 0; i < kRounds; ++i)
#pragma unroll
        for (int k = 0; k < kRfMaxK; ++k) n += __popcll(__ballot(rt.id[i][k] == e));
      cv = set_lane(cv, j, n);
    }
    s_c[wave][lane] = cv;
    lds_barrier();
    if (tid < nd && p.recv_count) {
      int n = 0;
      for (int w = 0; w < kRfWaves; ++w) n += s_c[w][tid];
      p.recv_count[d + tid * D] = round_up(n, p.A);
    }
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
  int st = 0;
  if (threadIdx.x == 0) s_status = 0;
  if ((int)blockIdx.x < p.token_wgs)  // uniform per workgroup
    token_workgroup<kRounds>(p, blockIdx.x, st);
  else
    duty_workgroup<kRounds>(p, blockIdx.x - p.token_wgs, st);
  if (st) atomicOr(&s_status, st);
  lds_barrier();
  if (threadIdx.x == 0 && s_status && p.status) atomicOr(p.status, s_status);
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
  p.expert_wgs = (E + kRfDuties - 1) / kRfDuties;
  const dim3 grid((unsigned)(p.token_wgs + p.expert_wgs + 1)), block(kRfThreads);
  if (T <= kRfThreads)
    hipLaunchKernelGGL(rank_layout_dispatch_kernel<1>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(rank_layout_dispatch_kernel<2>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
