// Normal-mode (high-throughput) layout on gfx950: one receive row per
// (token, rank reached), after the NeMo AutoModel page
// "nemo_automodel.components.moe.uccl_ep.buffer" (Buffer.dispatch:
// is_token_in_rank, num_tokens_per_rank, topk_idx, topk_weights,
// expert_alignment, and its returns recv_topk_idx, recv_topk_weights and the
// per-expert receive counts; Buffer.combine adds the rows back without
// weights). The scatter and the row sum are the pair kernels run over the
// [T, R] table of rank rows instead of the [T, K] table of expert slots.
//
// Layout (batches of more than 1024 tokens, or K > 8; smaller ones take the
// one-launch kernel of rank_fused.hip without its row copy): one workgroup
// per rank r. A thread takes one token per pass, reads
// its K ids and forms the set of ranks it reaches as a 64-bit mask (so
// duplicates collapse). Pass 1 sums, over all tokens, the ranks below r that
// each reaches (popcount of the masked bits) -- the start of rank r's rows --
// and counts the rank's local experts in LDS. Pass 2 block-scans "reaches r"
// in token order and writes the rows: no workgroup waits for another.
#include "wave.hpp"

namespace moe {
namespace {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / 64;

struct RankParams {
  const int64_t *idx;
  const float *w;  // may be null
  int32_t T, K, E, R, L, A;
  uint64_t l_magic;
  int32_t *rank_slot;     // [T*R]
  int32_t *rank_offset;   // [R+1]
  int32_t *recv_src;      // [cap] may be null
  int64_t *recv_idx;      // [cap*K] may be null
  float *recv_w;          // [cap*K] may be null
  int32_t *recv_count;    // [E] may be null
  int64_t cap;            // rows the recv arrays hold
  int32_t *status;
};

// A token's ids, 8 at a time: the 8 loads are issued together (addresses
// clamped into the row, so none waits behind a branch), then examined.
struct IdChunk {
  int64_t e[8];
  __device__ __forceinline__ void load(const RankParams &p, int t, int k0) {
    const int64_t *row = p.idx + (int64_t)t * p.K;
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = row[min(k0 + j, p.K - 1)];
  }
};

// Ranks reached by token t (bit r), the pairs of t whose expert lives on rank
// r (bit k), and, with s_cnt, one count per such pair into its local expert.
__device__ __forceinline__ uint64_t token_ranks(const RankParams &p, int t, int r, int &st,
                                                uint64_t *local, int32_t *s_cnt) {
  uint64_t m = 0, loc = 0;
  for (int k0 = 0; k0 < p.K; k0 += 8) {
    IdChunk c;
    c.load(p, t, k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t e = c.e[j];
      if (k0 + j >= p.K) break;
      if (e >= 0 && e < p.E) {
        const int rr = rank_of((int)e, p.l_magic);
        m |= 1ull << rr;
        if (rr == r) {
          loc |= 1ull << (k0 + j);
          if (s_cnt) atomicAdd(&s_cnt[(int)e - r * p.L], 1);
        }
      } else if (e != -1) {
        st |= kStBadExpert;
      }
    }
  }
  if (local) *local = loc;
  return m;
}

// Batches of more than 1024 tokens, or K > 8 (smaller ones take the
// layout-only instance of the one-launch kernel in rank_fused.hip).
__global__ __launch_bounds__(kRankThreads) void rank_layout_kernel(RankParams p) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_wave[kRankWaves];
  __shared__ int32_t s_status;
  const int tid = threadIdx.x, r = blockIdx.x;
  const uint64_t below = (1ull << r) - 1ull;  // r < 64
  int st = 0;
  if (tid == 0) s_status = 0;
  for (int l = tid; l < p.L; l += kRankThreads) s_cnt[l] = 0;
  lds_barrier();

  // pass 1: start of this rank's rows, local expert counts
  int before = 0;
  for (int t0 = 0; t0 < p.T; t0 += kRankThreads) {
    const int t = t0 + tid;
    int n = 0;
    if (t < p.T) n = __popcll(token_ranks(p, t, r, st, nullptr, s_cnt) & below);
    int total = 0;
    block_exclusive_scan(n, s_wave, kRankWaves, &total);
    before += total;
  }
  lds_barrier();
  if (p.recv_count)
    for (int l = tid; l < p.L; l += kRankThreads)
      p.recv_count[r * p.L + l] = round_up(s_cnt[l], p.A);

  // pass 2: rows of the tokens that reach r, in token order
  int run = before;
  for (int t0 = 0; t0 < p.T; t0 += kRankThreads) {
    const int t = t0 + tid;
    int hit = 0;
    uint64_t local = 0;
    if (t < p.T) hit = (int)((token_ranks(p, t, r, st, &local, nullptr) >> r) & 1ull);
    int total = 0;
    const int pos = block_exclusive_scan(hit, s_wave, kRankWaves, &total);
    if (t < p.T) {
      int row = hit ? run + pos : -1;
      if (row >= p.cap) {
        st |= kStBadSlot;  // receive arrays smaller than the layout needs
        row = -1;
      }
      p.rank_slot[(int64_t)t * p.R + r] = row;
      if (row >= 0) {
        if (p.recv_src) p.recv_src[row] = t;
        for (int k0 = 0; k0 < p.K; k0 += 8) {
          IdChunk c;
          c.load(p, t, k0);
          float wk[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            wk[j] = p.w ? p.w[(int64_t)t * p.K + min(k0 + j, p.K - 1)] : 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int k = k0 + j;
            if (k >= p.K) break;
            const bool loc = (local >> k) & 1ull;
            if (p.recv_idx) p.recv_idx[(int64_t)row * p.K + k] = loc ? c.e[j] - (int64_t)r * p.L : -1;
            if (p.recv_w && p.w) p.recv_w[(int64_t)row * p.K + k] = loc ? wk[j] : 0.0f;
          }
        }
      }
    }
    run += total;
  }
  if (tid == 0) {
    p.rank_offset[r] = before;
    if (r == p.R - 1) p.rank_offset[p.R] = run;
  }
  if (r != 0) st &= ~kStBadExpert;  // every workgroup sees the same ids; one reports
  if (st) atomicOr(&s_status, st);
  lds_barrier();
  if (tid == 0 && s_status && p.status) atomicOr(p.status, s_status);
}

}  // namespace

hipError_t launch_rank_layout(const int64_t *idx, const float *w, int32_t T, int32_t K,
                              int32_t E, int32_t R, int32_t A, int32_t *rank_slot,
                              int32_t *rank_offset, int32_t *recv_src, int64_t *recv_idx,
                              float *recv_w, int32_t *recv_count, int64_t cap, int32_t *status,
                              hipStream_t s) {
  // batches the one-launch normal-mode kernel takes: its layout-only instance
  // (one workgroup per token instead of one per rank)
  if (rank_layout_dispatch_fits(T, K, R))
    return launch_rank_layout_dispatch(idx, w, T, K, E, R, A, rank_slot, rank_offset, recv_src,
                                       recv_idx, recv_w, recv_count, cap, status, nullptr,
                                       nullptr, 0, 0, s);
  RankParams p;
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
  hipLaunchKernelGGL(rank_layout_kernel, dim3((unsigned)R), dim3(kRankThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
