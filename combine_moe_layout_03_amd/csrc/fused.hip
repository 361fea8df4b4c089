// Layout by counting, for small batches, with or without the dispatch copy in
// the same launch. Same results, bit for bit, as the layout kernels (and the
// scatter) for alignment 1 and for the low-latency stripes, as the NeMo
// AutoModel page "nemo_automodel.components.moe.uccl_ep.buffer" describes them
// for Buffer.get_dispatch_layout, Buffer.dispatch (topk_idx given, no handle)
// and Buffer.low_latency_dispatch.
//
// With alignment 1 the slot of pair (t, k) on expert e is
//   #(valid pairs with id < e) + #(pairs before token t with id e)
//   + #(earlier k of token t with id e),
// and in the low-latency layout it is (e*R + src)*M plus the last two terms.
// The three terms together count the pairs ordered before (t, k) by the key
// id * P + pair index, and the last two the keys in [e * P, e * P + tK + k),
// so a workgroup that serves token t needs one count per selected expert over
// the whole routing (low latency: over the pairs up to its own only), one
// compare per id -- no histogram, no scan, no cross-workgroup step.
// Each wave reads a few ids per lane (the routing is a few KiB and sits in
// L2 after the first touch) and turns them into counts with ballot +
// popcount, accumulated in scalar registers; the waves' partial counts meet
// in LDS once. The totals the handle also needs (count and offset per expert,
// tokens per rank, empty low-latency stripe rows) are computed the same way by
// extra "duty" workgroups that copy nothing (one per expert for batches of up
// to 2048 pairs), so the copying workgroups only derive their own K slots. The id loads are unrolled over a compile-time
// number of rounds (up to 8: 4096 pairs over 512 lanes) and every count is a
// compare or two + ballot + popcount: at this size the counting is bound by
// each wave's serial instruction latency, not by memory.
//
// With the copy, a workgroup of 8 waves owns up to 8 chunks (1 KiB each) of
// one token row (a 7168-wide row is two workgroups of 7 copying waves, so the
// row stores of 128 tokens leave from all 256 CUs; every wave also counts:
// 512 lanes read a 1024-pair routing in two rounds). It requests the routing
// first (every wave's, before any wave's row load) and the row second, derives
// its K slots while the (cold) row is still in flight, then stores the row K
// times, back to back -- as
// bf16, or (low-latency FP8 dispatch) cast once to E4M3 with per-128-channel
// scales (fp8.hpp) and stored as codes plus column-major (or row-major)
// scales.
#include "fp8.hpp"
#include "wave.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Every workgroup of the kernel has 8 waves: a copying workgroup owns at most
// 8 row chunks (one per wave, or two per wave for large batches), and every
// wave reads its share of the routing and counts. A compile-time block size
// spares the wave a load of the launch's block size and makes the lane
// arithmetic shifts.
constexpr int kCountWaves = 8;
constexpr int kCountThreads = 64 * kCountWaves;
constexpr int kCountMaxRounds = 8;  // ids per lane; the batch needs P <= 8 * 512
// Experts (and ranks) whose totals one duty workgroup writes: one each for
// batches of at most kManyPairs pairs -- the duty workgroups' last stores
// tend to end the kernel (they queue behind the row stores of the copying
// workgroup sharing the CU), and a shorter duty ends sooner (128 x 7168 with
// 1, 4, 8 experts each: 4.35, 4.65, 4.95 us); kMaxDuties each above, where
// every duty workgroup reading the whole routing from L2 is what costs. (The
// totals done by the token workgroups after their stores instead cost 1.3 us:
// that code then runs late, from cold instruction caches.)
constexpr int kMaxDuties = 4;
constexpr int kManyPairs = 2048;
constexpr int kNoId = -2;           // sentinel: matches no expert
constexpr int kAboveAll = 0x7fffffff;  // sentinel: not below any expert

struct CountParams {
  LayoutParams lp;
  const u32x4 *x;  // null: layout only
  u32x4 *recv;
  int64_t rows;
  int32_t nvec, nchunk, chunks_per_wg, wg_per_token;
  uint64_t wpt_magic;  // ceil(2^32 / wg_per_token): token of workgroup b = (b * magic) >> 32
  int32_t token_wgs;  // workgroups [0, token_wgs) serve tokens, the rest do duties
  int32_t duty_wgs;
  // FP8 output (kFp8 >= 0): codes, scales, rows per expert, scale groups per row
  u32x2 *q;
  float *scale;
  uint32_t *ue;
  int32_t RM, G;
};

__device__ __forceinline__ int valid_or_neg(int64_t v, int E, int &st) {
  const bool ok = v >= 0 && v < E;
  if (!ok && v != -1) st |= kStBadExpert;
  return ok ? (int)v : -1;
}

// The routing as seen by one lane: ids of pairs r*nthreads + tid for
// r < kRounds, in the three forms the counts compare against: any id
// (sentinel kNoId), valid ids for "below" tests (kAboveAll otherwise), and
// the key id * P + pair index (kAboveAll for no valid id), by which pairs
// order as the slots do: by expert, then by pair index.
template <int kRounds>
struct LaneIds {
  int64_t raw[kRounds];
  int any[kRounds], below[kRounds], key[kRounds];

  // request the ids of rounds r < nr (the rest read as "no id"); nothing
  // waits for them here
  __device__ __forceinline__ void issue(const int64_t *idx, int P, int nthreads, int nr = kRounds) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      raw[r] = -1;
      if (r == 0 || r < nr) raw[r] = idx[min(r * nthreads + (int)threadIdx.x, P - 1)];
    }
    // every id load stays ahead of whatever the caller issues next (a row load)
    __builtin_amdgcn_sched_barrier(0);
  }
  // wait for them and build the three forms; pairs [tok, tok + K) are also
  // written to s_tok (each pair is held by exactly one lane)
  __device__ __forceinline__ void settle(int P, int E, int nthreads, int tok,
                                         int K, int32_t *s_tok, int &st) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int i = r * nthreads + (int)threadIdx.x;
      const int e = i < P ? valid_or_neg(raw[r], E, st) : -1;
      any[r] = e >= 0 ? e : kNoId;
      below[r] = e >= 0 ? e : kAboveAll;
      key[r] = e >= 0 ? e * P + i : kAboveAll;
      if (s_tok && i >= tok && i < tok + K && i < P) s_tok[i - tok] = e;
    }
  }
  __device__ __forceinline__ void load(const int64_t *idx, int P, int E, int nthreads,
                                       int &st) {
    issue(idx, P, nthreads);
    settle(P, E, nthreads, 0, 0, nullptr, st);
  }
  // wave-wide counts, as scalars
  __device__ __forceinline__ int count_equal(int e) const {
    int n = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) n += __popcll(__ballot(any[r] == e));
    return n;
  }
  // pairs whose key lies in [lo, lo + width) (one unsigned compare each): with
  // lo = e * P and width = i, the pairs of e before pair i -- its row in e's
  // low-latency stripe
  __device__ __forceinline__ int count_keys_in(int lo, int width, int nr = kRounds) const {
    int n = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r)
      if (r == 0 || r < nr)  // (the first load round always counts)
        n += __popcll(__ballot((uint32_t)key[r] - (uint32_t)lo < (uint32_t)width));
    return n;
  }
  // pairs whose key is below k: with k = e * P + i, the valid pairs with an id
  // below e plus the pairs of e before pair i -- pair i's contiguous slot (A = 1)
  __device__ __forceinline__ int count_key_below(int k) const {
    int n = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) n += __popcll(__ballot(key[r] < k));
    return n;
  }
  __device__ __forceinline__ int count_below(int e) const {
    int n = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) n += __popcll(__ballot(below[r] < e));
    return n;
  }
};

// Totals the handle needs besides the slots, one workgroup per group of
// experts/ranks: count (and first row) of experts d, d+D, ...; distinct tokens
// of ranks d, d+D, ...; empty low-latency stripe rows.
template <int kRounds>
__device__ void duty_workgroup(const LayoutParams &p, int d, int D, int &st) {
  __shared__ int32_t s_c[kCountWaves][kMaxDuties];
  __shared__ int32_t s_l[kCountWaves][kMaxDuties];
  __shared__ int32_t s_r[kCountWaves][kMaxDuties];
  __shared__ uint8_t s_mark[kMaxPairsFused];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int nthreads = kCountThreads, nwaves = kCountWaves;
  const int E = p.E, R = p.R, K = p.K, T = p.T, P = T * K;
  const bool ll = p.mode == kModeLowLatency;
  LaneIds<kRounds> ids;
  if (P > 0) {
    ids.load(p.idx, P, E, nthreads, st);
  } else {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      ids.any[r] = kNoId;
      ids.below[r] = kAboveAll;
    }
  }
  const int ndx = d < E ? (E - 1 - d) / D + 1 : 0;
  // (ranks only when their token counts are asked for)
  const int ndr = (d < R && p.rank_token_count) ? (R - 1 - d) / D + 1 : 0;
  int cv = 0, lv = 0;  // lane j holds duty j's counts
  for (int j = 0; j < ndx; ++j) {
    const int ed = d + j * D;
    cv = set_lane(cv, j, ids.count_equal(ed));
    if (!ll) lv = set_lane(lv, j, ids.count_below(ed));
  }
  if (lane < ndx) {
    s_c[wave][lane] = cv;
    s_l[wave][lane] = lv;
  }
  for (int j = 0; j < ndr; ++j) {  // the same trip count for the whole workgroup
    const int rd = d + j * D;
    for (int t = tid; t < T; t += nthreads) s_mark[t] = 0;
    lds_barrier();
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int i = r * nthreads + tid;
      if (ids.any[r] >= 0 && rank_of(ids.any[r], p.l_magic) == rd) s_mark[i / K] = 1;
    }
    lds_barrier();
    int n = 0;
    for (int t0 = 0; t0 < T; t0 += nthreads) {
      const int t = t0 + tid;
      n += __popcll(__ballot(t < T && s_mark[t] != 0));
    }
    if (lane == 0) s_r[wave][j] = n;
    lds_barrier();
  }
  lds_barrier();
  if (tid < ndx) {
    const int ed = d + tid * D;
    int c = 0, lt = 0;
    for (int w = 0; w < nwaves; ++w) {
      c += s_c[w][tid];
      lt += s_l[w][tid];
    }
    if (!ll) {
      p.count[ed] = c;
      if (p.recv_stats) p.recv_stats[ed] += c;
      p.offset[ed] = lt;
      if (ed == E - 1) p.offset[E] = lt + c;
    } else {
      p.count[ed] = min(c, p.M);
      if (p.recv_stats) p.recv_stats[ed] += min(c, p.M);
      if (c > p.M) st |= kStOverflow;
      if (p.offset) {
        p.offset[ed] = (ed * R + p.src) * p.M;
        if (ed == E - 1) p.offset[E] = E * R * p.M;
      }
    }
  }
  if (tid < ndr && p.rank_token_count) {
    int n = 0;
    for (int w = 0; w < nwaves; ++w) n += s_r[w][tid];
    p.rank_token_count[d + tid * D] = n;
  }
  if (ll && p.row_src) {
    // stripe rows past the received count hold no pair
    for (int j = 0; j < ndx; ++j) {
      const int ed = d + j * D;
      int c = 0;
      for (int w = 0; w < nwaves; ++w) c += s_c[w][j];
      for (int jj = min(c, p.M) + tid; jj < p.M; jj += nthreads)
        p.row_src[(int64_t)ed * p.M + jj] = -1;
    }
  }
}

// v with lane j (a compile-time constant) replaced by the wave-uniform x
template <int j>
__device__ __forceinline__ int write_lane(int v, int x) {
  asm("v_writelane_b32 %0, %1, %2" : "=v"(v) : "s"(x), "i"(j), "0"(v));
  return v;
}

// Lane k < K: pair (pbeg + k)'s count over the wave's ids, thr holding its
// threshold key in lane k (see the kernel).
template <int kRounds>
__device__ __forceinline__ int token_counts(const LaneIds<kRounds> &ids, int thr, int K,
                                            int pbeg, bool ll, int nr) {
  int prev = 0;
  if (ll) {
    for (int k = 0; k < K; ++k)
      prev = set_lane(prev, k, ids.count_keys_in(__builtin_amdgcn_readlane(thr, k), pbeg + k, nr));
  } else {
    for (int k = 0; k < K; ++k)
      prev = set_lane(prev, k, ids.count_key_below(__builtin_amdgcn_readlane(thr, k)));
  }
  return prev;
}

// The same for K = 8, written so the eight thresholds are read first and each
// count lands in its lane with one v_writelane.
template <int kRounds>
__device__ __forceinline__ int token_counts8(const LaneIds<kRounds> &ids, int thr, int pbeg,
                                             bool ll, int nr) {
  int th[8], n[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) th[k] = __builtin_amdgcn_readlane(thr, k);
  // (the contiguous counting is laid out inline, the low-latency one after it:
  // fused kernel at 128 x 7168 4.37 -> 4.35 us)
  if (__builtin_expect(ll, 0)) {
    // rounds outermost: one uniform branch per round skips the rounds past
    // this token's pairs (with k outermost the test became a branch per
    // (k, round), most of them to out-of-line blocks and back: low-latency
    // layout + dispatch at 128 / 256 tokens 4.58 -> 4.49 / 7.31 -> 7.08 us)
#pragma unroll
    for (int k = 0; k < 8; ++k) n[k] = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      if (r == 0 || r < nr) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          n[k] += __popcll(__ballot((uint32_t)ids.key[r] - (uint32_t)th[k] <
                                    (uint32_t)(pbeg + k)));
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) n[k] = ids.count_key_below(th[k]);
  }
  int prev = 0;
  prev = write_lane<0>(prev, n[0]);
  prev = write_lane<1>(prev, n[1]);
  prev = write_lane<2>(prev, n[2]);
  prev = write_lane<3>(prev, n[3]);
  prev = write_lane<4>(prev, n[4]);
  prev = write_lane<5>(prev, n[5]);
  prev = write_lane<6>(prev, n[6]);
  prev = write_lane<7>(prev, n[7]);
  return prev;
}

// kFp8: -1 copies bf16 rows; otherwise the FP8 flags of the cast. kCpw: row
// chunks per copying wave (2 only for bf16 rows).
//
// The values a token workgroup needs before its first loads come first, as
// scalar arguments (copies of fields of f), so the launch can preload them
// into registers (the library is built with kernel-argument preloading): the
// routing and row loads need no round trip to the argument buffer. The launch
// preloads 14 dwords (up to hnchunk); hE is read after the row load is issued.
template <bool kCopy, int kRounds, int kFp8, int kCpw>
__global__ __launch_bounds__(kCountThreads) void count_layout_kernel(
    const int64_t *hidx, const u32x4 *hx, uint64_t hmagic, int32_t hT, int32_t hK,
    int32_t hmode, int32_t htoken_wgs, int32_t hwpt, int32_t hcpw, int32_t hnvec,
    int32_t hnchunk, int32_t hE, CountParams f) {
  __shared__ int32_t s_pre[64];  // per k: the slot (contiguous) or stripe row (low latency)
  __shared__ int32_t s_tok[64];   // this token's ids (-1 = none)

  const LayoutParams &p = f.lp;
  const int tid = threadIdx.x, lane = lane_id();
  const int b = blockIdx.x;
  int st = 0;

  // uniform per workgroup; the token path is laid out first, so a token
  // wave's first instructions follow the entry in the instruction cache
  if (__builtin_expect(b >= htoken_wgs, 0)) {
    duty_workgroup<kRounds>(p, b - htoken_wgs, f.duty_wgs, st);
  } else {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the last wave writes the token's handle entries and reports its bad
    // slots: with 7 row chunks in 8 waves it copies nothing, so those stores
    // do not queue behind a row's K stores
    constexpr int hw = kCountWaves - 1;
    // lanes that read the routing and count (all of them without the copy)
    constexpr int nthreads = kCountThreads;
    constexpr bool counting = true;
    const int E = hE, R = p.R, K = hK, T = hT;
    const int P = T * K;
    const bool ll = hmode == kModeLowLatency;
    // b / wg_per_token, exact while b * wg_per_token < 2^32
    const int t = kCopy ? (int)(((uint64_t)(uint32_t)b * hmagic) >> 32) : b;  // < T
    const int part = b - t * (kCopy ? hwpt : 1);  // workgroup within the token
    const bool token_lead = part == 0;
    const int pbeg = t * K;
    if (tid < 64) s_pre[tid] = 0;

    // 1. the routing first ...
    LaneIds<kRounds> ids;
    // A stripe row counts earlier pairs only, so in the low-latency layout
    // the ids past this token's pairs are neither requested nor counted (on
    // average half the routing); a contiguous slot counts every pair.
    const int nr = ll ? (pbeg + K + nthreads - 1) / nthreads : kRounds;
    if (counting) ids.issue(hidx, P, nthreads, nr);
    //    Every wave's id loads leave before any wave's row load (a barrier
    //    with no memory wait). Without it the routing reached a workgroup's
    //    last wave 0.5 us after its first -- id loads issued after another
    //    wave's cold row load came back after it -- and the barrier takes
    //    0.4 us off the 128 x 7168 batch.
    __builtin_amdgcn_s_barrier();
    // 2. ... then the row chunk this wave copies; it stays in flight while
    //    the slots are worked out. The load is unconditional (address clamped
    //    into the row): under a branch it would force an early wait.
    static_assert(kCpw == 1 || kFp8 < 0, "two chunks per wave for bf16 rows only");
    u32x4 val = {0u, 0u, 0u, 0u}, val2 = {0u, 0u, 0u, 0u};
    int v = 0, chunk = 0;
    bool lane_ok = false, lane_ok2 = false;
    if (kCopy) {
      chunk = part * hcpw + wave * kCpw;
      v = chunk * 64 + lane;
      lane_ok = wave * kCpw < hcpw && chunk < hnchunk && v < hnvec;
      val = __builtin_nontemporal_load(hx + (int64_t)t * hnvec + min(v, hnvec - 1));
      if (kCpw == 2) {  // the wave's second chunk, 64 vectors further
        lane_ok2 = wave * kCpw + 1 < hcpw && chunk + 1 < hnchunk && v + 64 < hnvec;
        val2 = __builtin_nontemporal_load(hx + (int64_t)t * hnvec + min(v + 64, hnvec - 1));
      }
    }
    if (counting) ids.settle(P, E, nthreads, pbeg, K, s_tok, st);
    lds_barrier();

    // 3. per pair k of this token: (contiguous layout) the pairs ordered
    //    before it by (expert, pair index), which is its slot; (low latency)
    //    the pairs of its expert before it, its stripe row. The token's ids
    //    sit in lanes 0..K-1 of tokv; each wave adds its counts for k into
    //    s_pre[k]. (An invalid ek = -1 gives an unused count, so it needs no
    //    branch.)
    const int tokv = lane < K ? s_tok[lane] : -1;
    if (counting) {  // uniform per wave
      // lane k: pair k's threshold key -- contiguous: e * P + pair index (its
      // slot counts the keys below); low latency: e * P (its row counts the
      // keys in [e * P, e * P + pair index)) -- so one lane read per k
      const int thr = tokv * P + (ll ? 0 : pbeg + lane);
      const int prev = K == 8 ? token_counts8(ids, thr, pbeg, ll, nr)
                              : token_counts(ids, thr, K, pbeg, ll, nr);
      if (lane < K) atomicAdd(&s_pre[lane], prev);
    }
    lds_barrier();

    // 4. slots of this token's pairs (lane k of every wave; wave 0 keeps them)
    int out = -1, j = 0;
    {
      const int e = tokv;
      if (lane < K && e >= 0) {
        j = s_pre[lane];  // contiguous: the slot; low latency: the stripe row
        if (!ll) {
          out = j;
        } else if (j < p.M) {
          out = (e * R + p.src) * p.M + j;
        } else if (wave == hw) {
          st |= kStOverflow;
        }
      }
    }

    // 5. the row, K times (slot k read from lane k)
    if (kCopy && kFp8 >= 0) {
      asm volatile("" : "+v"(val));
      // H % 128 == 0: a 16-lane scale group is inside the row or wholly past it
      const Fp8Lane q = fp8_cast_lane<(kFp8 < 0 ? 0 : kFp8)>(val);
      const u32x2 codes = {q.lo, q.hi};
      const int grp = chunk * 4 + (lane >> 4);
      uint32_t word = 0;
      if (kFp8 & kFp8Ue8m0) word = ue8m0_word(q.scale);
      const uint32_t rows32 = f.rows < 0x7fffffff ? (uint32_t)f.rows : 0x7fffffffu;
      // pair k's codes, and its scale (or packed UE8M0 word) by one lane per group
      auto put = [&](int s, int e) {
        const int i = s - e * f.RM;  // row within the expert's R*M rows
        __builtin_nontemporal_store(codes, f.q + (int64_t)s * hnvec + v);
        if (kFp8 & kFp8Ue8m0) {
          if (lane == 0)
            f.ue[(kFp8 & kFp8ScaleRows) ? (int64_t)s * hnchunk + chunk
                                        : ((int64_t)e * hnchunk + chunk) * f.RM + i] = word;
        } else if ((lane & 15) == 0) {
          f.scale[(kFp8 & kFp8ScaleRows) ? (int64_t)s * f.G + grp
                                         : ((int64_t)e * f.G + grp) * f.RM + i] = q.scale;
        }
      };
      if (K == 8) {  // the eight slots and experts first, then the stores back to back
        int sl[8], ex[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          sl[k] = __builtin_amdgcn_readlane(out, k);
          ex[k] = __builtin_amdgcn_readlane(tokv, k);
        }
        if (lane_ok) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((uint32_t)sl[k] < rows32) put(sl[k], ex[k]);
        }
        if (wave == hw) {  // receive buffer smaller than the layout needs
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((uint32_t)sl[k] >= rows32 && sl[k] != -1) st |= kStBadSlot;
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int sk = __builtin_amdgcn_readlane(out, k);
          if ((uint32_t)sk < rows32) {
            if (lane_ok) put(sk, __builtin_amdgcn_readlane(tokv, k));
          } else if (sk != -1 && wave == hw) {
            st |= kStBadSlot;  // receive buffer smaller than the layout needs
          }
        }
      }
    } else if (kCopy) {
      asm volatile("" : "+v"(val));
      if (kCpw == 2) asm volatile("" : "+v"(val2));
      // slots are int32, so a 32-bit unsigned compare against the row count
      // (clamped to INT32_MAX) tells valid slots (and -1 is never valid)
      const uint32_t rows32 = f.rows < 0x7fffffff ? (uint32_t)f.rows : 0x7fffffffu;
      u32x4 *dst = f.recv + v;
      if (K == 8) {  // the eight slots first, then the stores back to back
        int sl[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) sl[k] = __builtin_amdgcn_readlane(out, k);
        if (lane_ok) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((uint32_t)sl[k] < rows32)
              __builtin_nontemporal_store(val, dst + (int64_t)sl[k] * hnvec);
        }
        if (kCpw == 2 && lane_ok2) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((uint32_t)sl[k] < rows32)
              __builtin_nontemporal_store(val2, dst + (int64_t)sl[k] * hnvec + 64);
        }
        if (wave == hw) {  // receive buffer smaller than the layout needs
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((uint32_t)sl[k] >= rows32 && sl[k] != -1) st |= kStBadSlot;
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int sk = __builtin_amdgcn_readlane(out, k);
          if ((uint32_t)sk < rows32) {
            if (lane_ok) __builtin_nontemporal_store(val, dst + (int64_t)sk * hnvec);
            if (kCpw == 2 && lane_ok2)
              __builtin_nontemporal_store(val2, dst + (int64_t)sk * hnvec + 64);
          } else if (sk != -1 && wave == hw) {
            st |= kStBadSlot;  // receive buffer smaller than the layout needs
          }
        }
      }
    }

    // 6. this token's handle entries
    if (token_lead && wave == hw) {
      if (lane < K) {
        p.slot[pbeg + lane] = out;
        if (out >= 0 && p.row_src)
          p.row_src[ll ? (int64_t)tokv * p.M + j : (int64_t)out] = pbeg + lane;
      }
      if (p.in_rank) {
        const int rank_v = tokv >= 0 ? rank_of(tokv, p.l_magic) : -1;
        for (int r0 = 0; r0 < R; r0 += 64) {
          const int r = r0 + lane;
          bool hit = false;
          for (int k = 0; k < K; ++k) hit |= __builtin_amdgcn_readlane(rank_v, k) == r;
          if (r < R) p.in_rank[(int64_t)t * R + r] = hit ? 1 : 0;
        }
      }
    }
    // every workgroup reads every id; the duty workgroups report bad ones
    st &= ~kStBadExpert;
  }
  // error bits (rare) go straight to the status word: no barrier at the end,
  // so each wave leaves as soon as its own work is out
  if (st && p.status) atomicOr(p.status, st);
}

template <bool kCopy, int kFp8, int kCpw = 1>
hipError_t launch_rounds(int rounds, dim3 grid, dim3 block, hipStream_t s, const CountParams &f) {
#define MOE_COUNT_ARGS                                                                       \
  f.lp.idx, f.x, f.wpt_magic, f.lp.T, f.lp.K, f.lp.mode, f.token_wgs, f.wg_per_token,        \
      f.chunks_per_wg, f.nvec, f.nchunk, f.lp.E, f
  if (rounds <= 1)
    hipLaunchKernelGGL((count_layout_kernel<kCopy, 1, kFp8, kCpw>), grid, block, 0, s, MOE_COUNT_ARGS);
  else if (rounds <= 2)
    hipLaunchKernelGGL((count_layout_kernel<kCopy, 2, kFp8, kCpw>), grid, block, 0, s, MOE_COUNT_ARGS);
  else if (rounds <= 4)
    hipLaunchKernelGGL((count_layout_kernel<kCopy, 4, kFp8, kCpw>), grid, block, 0, s, MOE_COUNT_ARGS);
  else
    hipLaunchKernelGGL((count_layout_kernel<kCopy, 8, kFp8, kCpw>), grid, block, 0, s, MOE_COUNT_ARGS);
#undef MOE_COUNT_ARGS
  return hipGetLastError();
}

// Row chunks of a copying workgroup: at most 8, one per wave (for large
// batches 16, two per wave). Measured on the 128 x 7168, top-8 batch: 8 chunks
// in 8-wave workgroups beat one 16-wave workgroup per token (5.7 vs 6.1 us):
// twice the CUs issue the row stores, and the counting still takes two rounds.
constexpr int kCopyChunks = kCountWaves;
// From this many tokens on (bf16 rows), a copying wave takes two chunks, so a
// token's row needs half the workgroups: the batch's workgroups then fit the
// GPU at once and each token's routing is counted once, not twice (512
// low-latency tokens x 7168: 14.8 vs 15.9 us; at 256 tokens it measured
// slower, 8.1 vs 7.8 us).
#ifndef MOE_TWO_CHUNK_TOKENS
#define MOE_TWO_CHUNK_TOKENS 512
#endif

// Row chunks of one workgroup (cpw: chunks per copying wave).
int copy_chunks(int32_t H, int cpw = 1) {
  const int nchunk = (H / 8 + 63) / 64;
  const int groups = (nchunk + cpw * kCopyChunks - 1) / (cpw * kCopyChunks);
  return (nchunk + groups - 1) / groups;
}

}  // namespace

bool count_layout_fits(const LayoutParams &lp, int32_t H, bool copy) {
  if (lp.mode == kModeContiguous && lp.A != 1) return false;
  const int64_t P = (int64_t)lp.T * lp.K;
  if (P > kMaxPairsFused) return false;
  // the batch must fit kCountMaxRounds rounds of the 512 counting lanes
  return P <= (int64_t)kCountMaxRounds * kCountThreads;
}

hipError_t launch_count_layout(const LayoutParams &lp, const uint16_t *x, uint16_t *recv,
                               int64_t rows, int32_t H, const Fp8Out *fp8, hipStream_t s) {
  CountParams f;
  f.lp = lp;
  f.x = reinterpret_cast<const u32x4 *>(x);
  f.recv = reinterpret_cast<u32x4 *>(recv);
  f.rows = rows;
  f.q = fp8 ? reinterpret_cast<u32x2 *>(fp8->q) : nullptr;
  f.scale = fp8 ? static_cast<float *>(fp8->scale) : nullptr;
  f.ue = fp8 ? static_cast<uint32_t *>(fp8->scale) : nullptr;
  f.RM = fp8 ? fp8->rows_per_expert : 0;
  f.G = H / kFp8Group;
  const int need = (lp.E > lp.R ? lp.E : lp.R);
  const int duties = (int64_t)lp.T * lp.K > kManyPairs ? kMaxDuties : 1;
  f.duty_wgs = (need + duties - 1) / duties;
  const int P = lp.T * lp.K;
  if (x && lp.T > 0) {
    const int cpw = (!fp8 && lp.T >= MOE_TWO_CHUNK_TOKENS) ? 2 : 1;
    f.nvec = H / 8;
    f.nchunk = (f.nvec + 63) / 64;
    f.chunks_per_wg = copy_chunks(H, cpw);  // <= cpw * 8: one or two per wave
    f.wg_per_token = (f.nchunk + f.chunks_per_wg - 1) / f.chunks_per_wg;
    f.wpt_magic = ((1ull << 32) + (uint64_t)f.wg_per_token - 1) / f.wg_per_token;
    f.token_wgs = lp.T * f.wg_per_token;
    const int rounds = (P + kCountThreads - 1) / kCountThreads;
    const dim3 grid((unsigned)(f.token_wgs + f.duty_wgs)), block(kCountThreads);
    if (!fp8)
      return cpw == 2 ? launch_rounds<true, -1, 2>(rounds, grid, block, s, f)
                      : launch_rounds<true, -1>(rounds, grid, block, s, f);
    constexpr int R1 = kFp8RoundScale, U = kFp8Ue8m0, SR = kFp8ScaleRows;
    switch (fp8->flags) {
      case 0: return launch_rounds<true, 0>(rounds, grid, block, s, f);
      case R1: return launch_rounds<true, R1>(rounds, grid, block, s, f);
      case R1 | U: return launch_rounds<true, R1 | U>(rounds, grid, block, s, f);
      case SR: return launch_rounds<true, SR>(rounds, grid, block, s, f);
      case SR | R1: return launch_rounds<true, SR | R1>(rounds, grid, block, s, f);
      default: return launch_rounds<true, SR | R1 | U>(rounds, grid, block, s, f);
    }
  }
  f.nvec = f.nchunk = f.chunks_per_wg = 0;
  f.wg_per_token = 1;
  f.wpt_magic = 0;
  f.token_wgs = lp.T;
  const int rounds = (P + kCountThreads - 1) / kCountThreads;
  return launch_rounds<false, -1>(rounds, dim3((unsigned)(f.token_wgs + f.duty_wgs)),
                                  dim3(kCountThreads), s, f);
}

}  // namespace moe
