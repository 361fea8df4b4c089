// Internal launch interface between the C-ABI entry points (capi.hip) and the
// gfx950 kernels (layout.hip, scatter.hip, replica.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// One workgroup of the layout kernels: 16 wave64s.
constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / 64;
// Largest expert count (one expert per layout thread; per-wave counters in LDS).
constexpr int kMaxExperts = 1024;
// Batches of up to kMaxPairsFused pairs with alignment 1 (or low latency) are
// laid out by counting, with or without the dispatch in the same launch (every
// workgroup re-derives its slots from the routing in L2). Otherwise a batch of
// up to kMaxPairsOneBlock pairs is laid out by one workgroup, and a larger one
// by three launches whose first pass gives each workgroup about kPairsPerBlock
// pairs (one workgroup's serial work grows with its pairs: at 4096 and 8192
// pairs, the one-workgroup kernel took 18 and 27 us, three launches 15 and 13).
constexpr int kMaxPairsFused = 4096;
constexpr int kMaxPairsOneBlock = 1024;
constexpr int kPairsPerBlock = 256;

enum LayoutMode : int32_t {
  kModeContiguous = 0,  // aligned per-expert partitions of one receive buffer
  kModeLowLatency = 1,  // fixed stripes (e*R + src)*M + j
};

struct LayoutParams {
  const int64_t *idx;  // [T*K]
  int32_t T, K, E, R, L, A;
  int32_t mode;
  int32_t M, src;        // low-latency capacity and source rank
  int32_t id_bits;       // bits needed for an expert id in [0, E)
  int32_t rank_bits;     // bits needed for a rank id in [0, R)
  uint64_t l_magic;      // ceil(2^32 / L): rank of expert e = (e * l_magic) >> 32
  int32_t tokens_per_block;
  int32_t nblocks;
  int32_t *count;
  int32_t *offset;
  int32_t *rank_token_count;
  uint8_t *in_rank;
  int32_t *slot;
  int32_t *row_src;
  int32_t *status;
  int32_t *recv_stats;  // [E] cumulative receive counts (+= count), may be null
  int32_t *ws_hist;  // [E][nblocks]  multi-block path: pairs of e per block, then prefix
  int32_t *ws_rcnt;  // [R][nblocks]  multi-block path: tokens reaching r per block
  int32_t *ws_cnt;   // [E]           multi-block path: pairs per expert
};

// Rank that owns expert e: e / L by a 32.32 reciprocal (exact for e < 2^20, L <= 2^10).
__device__ __forceinline__ int rank_of(int e, uint64_t l_magic) {
  return (int)(((uint64_t)(uint32_t)e * l_magic) >> 32);
}

// Status bits (same values as the MOE_STATUS_* macros of the public header).
constexpr int32_t kStBadExpert = 1;
constexpr int32_t kStOverflow = 2;
constexpr int32_t kStBadSlot = 4;
constexpr int32_t kStBadReplica = 8;

// Launchers: return hipSuccess or the launch error.
hipError_t launch_layout_one_block(const LayoutParams &p, hipStream_t s);
hipError_t launch_layout_multi_block(const LayoutParams &p, hipStream_t s);
hipError_t launch_expert_load(const int64_t *idx, int32_t T, int32_t K, int32_t E,
                              int32_t id_bits, int32_t *load, int32_t *status, hipStream_t s);

// FP8 form of a low-latency receive buffer: E4M3 codes [rows, H] and the
// per-128-channel scales, stored [E][H/128][rows_per_expert] as floats, or
// [E][H/512][rows_per_expert] as packed UE8M0 words (flags has kFp8Ue8m0).
struct Fp8Out {
  int32_t flags;            // kFp8RoundScale | kFp8Ue8m0 bits (fp8.hpp)
  uint8_t *q;
  void *scale;
  int32_t rows_per_expert;  // R*M
};

// Layout by counting (alignment 1 or low latency, at most kMaxPairsFused
// pairs), optionally with the dispatch copy in the same launch (x != null):
// bf16 rows into recv, or, with fp8 != null (low latency only), the E4M3 cast.
bool count_layout_fits(const LayoutParams &p, int32_t H, bool copy);
hipError_t launch_count_layout(const LayoutParams &p, const uint16_t *x, uint16_t *recv,
                               int64_t rows, int32_t H, const Fp8Out *fp8, hipStream_t s);

// FP8 kernels (fp8.hip).
hipError_t launch_ll_quant_dispatch(const uint16_t *x, const int32_t *slot, const Fp8Out &o,
                                    int32_t T, int32_t K, int32_t H, int64_t rows,
                                    int32_t *status, hipStream_t s);
hipError_t launch_fp8_copy_dispatch(const uint8_t *xq, const float *xs, const int32_t *slot,
                                    uint8_t *rq, float *rs, int32_t T, int32_t K, int32_t H,
                                    int64_t rows, int32_t *status, hipStream_t s);
hipError_t launch_quantize_fp8(const uint16_t *x, uint8_t *q, void *scale, int32_t flags,
                               int32_t T, int32_t H, hipStream_t s);

hipError_t launch_dispatch(const uint16_t *x, const int32_t *slot, uint16_t *recv, int32_t T,
                           int32_t K, int32_t H, int64_t rows, int32_t *status, hipStream_t s);
// Active-rank mask of a combine: pairs whose expert e lives on a rank r with
// mask[r] != 0 are left out of the sum.
struct CombineMask {
  const int64_t *idx;   // [T*K] expert ids
  const int32_t *mask;  // [R]
  int32_t E;
  uint64_t l_magic;     // rank of e = (e * l_magic) >> 32
};
hipError_t launch_combine(const uint16_t *y, int64_t rows, const int32_t *slot, const float *w,
                          uint16_t *out, float *out_f32, int32_t T, int32_t K, int32_t H,
                          const CombineMask *mask, int32_t *status, hipStream_t s);

// Normal-mode layout, one row per (token, rank) (ranks.hip); R <= 64.
hipError_t launch_rank_layout(const int64_t *idx, const float *w, int32_t T, int32_t K,
                              int32_t E, int32_t R, int32_t A, int32_t *rank_slot,
                              int32_t *rank_offset, int32_t *recv_src, int64_t *recv_idx,
                              float *recv_w, int32_t *recv_count, int64_t cap, int32_t *status,
                              hipStream_t s);
// Normal-mode layout and dispatch in one launch (rank_fused.hip), for
// T <= 1024, K <= 8, R <= 64: the results of launch_rank_layout followed by
// the rank scatter. With x null, the layout alone (no row read or written).
bool rank_layout_dispatch_fits(int32_t T, int32_t K, int32_t R);
hipError_t launch_rank_layout_dispatch(const int64_t *idx, const float *w, int32_t T, int32_t K,
                                       int32_t E, int32_t R, int32_t A, int32_t *rank_slot,
                                       int32_t *rank_offset, int32_t *recv_src,
                                       int64_t *recv_idx, float *recv_w, int32_t *recv_count,
                                       int64_t cap, int32_t *status, const uint16_t *x,
                                       uint16_t *recv, int64_t rows, int32_t H, hipStream_t s);
// Normal-mode combine: the unweighted row sum over the [T, R] rank table, and
// (ws.in != null) the rows' top-k weights summed back per token.
struct RowWeightSum {
  const float *in;  // [rows*Kw]
  float *out;       // [T*Kw]
  int32_t Kw;
};
hipError_t launch_rank_combine(const uint16_t *y, int64_t rows, const int32_t *rank_slot,
                               uint16_t *out, float *out_f32, int32_t T, int32_t R, int32_t H,
                               const RowWeightSum &ws, int32_t *status, hipStream_t s);

hipError_t launch_replica_weight_sync(int32_t E, int32_t E_phys, int64_t S,
                                      const int32_t *replica_count, const int32_t *replica_phys,
                                      uint16_t *w, int32_t *status, hipStream_t s);
hipError_t launch_replica_grad_reduce(int32_t E, int32_t E_phys, int64_t S,
                                      const int32_t *replica_count, const int32_t *replica_phys,
                                      float *g, int32_t *status, hipStream_t s);
hipError_t launch_plan_replicas(int32_t E, int32_t R, int32_t C, const int32_t *load,
                                int32_t *replica_count, int32_t *replica_phys,
                                int32_t *phys_to_logical, hipStream_t s);
hipError_t launch_reroute(int32_t T, int32_t K, int32_t E, const int64_t *idx,
                          const int32_t *replica_count, const int32_t *replica_phys,
                          int32_t E_phys, int64_t *phys_idx, int32_t *status, hipStream_t s);

}  // namespace moe
