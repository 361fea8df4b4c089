// Replica planning and routing expansion on gfx950, after the
// "dots-infra/ultraep architecture" page (Overview: plan replicas from each
// layer's post-gating routing, then expand the routing before the experts;
// GPU operations: Placement planning, Routing expansion).
//
// Plan: one workgroup per expert. An expert's place in the order (load
// descending, id ascending) is the number of experts ahead of it, counted by
// the workgroup's threads over the E loads and summed; the first C get a
// second physical replica. Numbering: rank r holds L' = L + C/R physical experts,
// r*L' + l (l < L) is the primary of logical expert r*L + l, and the i-th
// hottest expert's replica is (i mod R)*L' + L + i/R, so replicas are dealt
// round-robin over the ranks.
// Reroute: one thread per (token, k) pair; the pair uses replica
// (t mod replica_count[e]) of its expert.
// Weight sync and gradient reduction (GPU operations: Replica weight sync,
// Replica gradient reduction): the physical expert buffer keeps each expert's
// master copy in its primary slot; the sync copies it into the replica slot,
// the reduction adds the replica's f32 gradient into the primary's. Grid: one
// row of workgroups per logical expert (the ones without a replica exit at
// once), each streaming its share of the S elements as 16-byte vectors, four
// in flight per thread.
#include "wave.hpp"

namespace moe {
namespace {

// One workgroup per expert e: its threads compare e against a share of the E
// loads and the counts meet in one block sum, so the E^2 comparisons are
// spread over E CUs instead of queuing on one.
__global__ __launch_bounds__(256) void plan_replicas_kernel(
    int32_t E, int32_t R, int32_t C, const int32_t *__restrict__ load,
    int32_t *__restrict__ replica_count, int32_t *__restrict__ replica_phys,
    int32_t *__restrict__ phys_to_logical) {
  __shared__ int32_t s_wave[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int mine = load[e];
  int ahead = 0;
  for (int f = tid; f < E; f += 256) {
    const int lf = load[f];
    ahead += (lf > mine) || (lf == mine && f < e);
  }
  int total = 0;
  block_exclusive_scan(ahead, s_wave, 4, &total);
  if (tid != 0) return;
  const int L = E / R, Lp = L + C / R;
  const int prim = (e / L) * Lp + (e - (e / L) * L);
  const bool hot = total < C;
  replica_count[e] = hot ? 2 : 1;
  replica_phys[2 * e] = prim;
  phys_to_logical[prim] = e;
  if (hot) {
    const int rep = (total % R) * Lp + L + total / R;
    replica_phys[2 * e + 1] = rep;
    phys_to_logical[rep] = e;
  } else {
    replica_phys[2 * e + 1] = -1;
  }
}

__global__ __launch_bounds__(256) void reroute_kernel(int32_t T, int32_t K, int32_t E,
                                                      const int64_t *__restrict__ idx,
                                                      const int32_t *__restrict__ replica_count,
                                                      const int32_t *__restrict__ replica_phys,
                                                      int32_t E_phys, int64_t *__restrict__ phys,
                                                      int32_t *status) {
  // The plan's tables go to LDS while the ids load, so each pair costs one
  // global read instead of three dependent ones.
  __shared__ int32_t s_count[kMaxExperts];
  __shared__ int32_t s_phys[2 * kMaxExperts];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < (int64_t)T * K;
  const int64_t v = live ? idx[i] : -1;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_count[e] = replica_count[e];
    s_phys[2 * e] = replica_phys[2 * e];
    s_phys[2 * e + 1] = replica_phys[2 * e + 1];
  }
  lds_barrier();
  if (!live) return;
  int64_t out = -1;
  int st = 0;
  if (v >= 0 && v < E) {
    const int e = (int)v;
    const int c = s_count[e];
    if (c == 1 || c == 2) {
      const int t = (int)(i / K);
      const int ph = s_phys[2 * e + (c == 2 ? (t & 1) : 0)];
      if (ph >= 0 && ph < E_phys)
        out = ph;
      else
        st |= kStBadReplica;
    } else {
      st |= kStBadReplica;
    }
  } else if (v != -1) {
    st |= kStBadExpert;
  }
  phys[i] = out;
  if (st && status) atomicOr(status, st);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Vectors in flight per thread: the copy is fastest at 4 (8: 329 vs 322 us
// per sync), the reduction, with two reads per write, at 8 (4: 1071 vs
// 1011 us; a plain grid-stride loop 1030 us).
constexpr int kSyncUnroll = 4;
constexpr int kReduceUnroll = 8;

template <bool kReduce>
__global__ __launch_bounds__(256) void replica_move_kernel(const int32_t *__restrict__ replica_count,
                                                           const int32_t *__restrict__ replica_phys,
                                                           int32_t E_phys, int64_t nvec,
                                                           void *buf, int32_t *status) {
  const int e = blockIdx.y;
  if (replica_count[e] != 2) return;  // wave-uniform
  const int prim = replica_phys[2 * e], rep = replica_phys[2 * e + 1];
  if (prim < 0 || prim >= E_phys || rep < 0 || rep >= E_phys) {
    if (status && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, kStBadReplica);
    return;
  }
  constexpr int kReplicaUnroll = kReduce ? kReduceUnroll : kSyncUnroll;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!kReduce) {
    const u32x4 *src = static_cast<const u32x4 *>(buf) + (int64_t)prim * nvec;
    u32x4 *dst = static_cast<u32x4 *>(buf) + (int64_t)rep * nvec;
    for (; v + (kReplicaUnroll - 1) * stride < nvec; v += kReplicaUnroll * stride) {
      u32x4 a[kReplicaUnroll];
#pragma unroll
      for (int j = 0; j < kReplicaUnroll; ++j) a[j] = __builtin_nontemporal_load(src + v + j * stride);
#pragma unroll
      for (int j = 0; j < kReplicaUnroll; ++j) __builtin_nontemporal_store(a[j], dst + v + j * stride);
    }
    for (; v < nvec; v += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
  } else {
#pragma clang fp contract(off)
    f32x4 *gp = static_cast<f32x4 *>(buf) + (int64_t)prim * nvec;
    const f32x4 *gr = static_cast<const f32x4 *>(buf) + (int64_t)rep * nvec;
    for (; v + (kReplicaUnroll - 1) * stride < nvec; v += kReplicaUnroll * stride) {
      f32x4 a[kReplicaUnroll], b[kReplicaUnroll];
#pragma unroll
      for (int j = 0; j < kReplicaUnroll; ++j) {
        a[j] = __builtin_nontemporal_load(gp + v + j * stride);
        b[j] = __builtin_nontemporal_load(gr + v + j * stride);
      }
#pragma unroll
      for (int j = 0; j < kReplicaUnroll; ++j) __builtin_nontemporal_store(a[j] + b[j], gp + v + j * stride);
    }
    for (; v < nvec; v += stride)
      __builtin_nontemporal_store(__builtin_nontemporal_load(gp + v) + __builtin_nontemporal_load(gr + v), gp + v);
  }
}

// Workgroups per expert: two unrolled steps per thread, at most 1024.
unsigned replica_wgs(int64_t nvec, int unroll) {
  const int64_t per = 256LL * unroll * 2;
  int64_t n = (nvec + per - 1) / per;
  return (unsigned)(n < 1 ? 1 : (n > 1024 ? 1024 : n));
}

}  // namespace

hipError_t launch_replica_weight_sync(int32_t E, int32_t E_phys, int64_t S,
                                      const int32_t *replica_count, const int32_t *replica_phys,
                                      uint16_t *w, int32_t *status, hipStream_t s) {
  const int64_t nvec = S / 8;  // bf16, 8 per vector
  hipLaunchKernelGGL(replica_move_kernel<false>, dim3(replica_wgs(nvec, kSyncUnroll), (unsigned)E), dim3(256),
                     0, s, replica_count, replica_phys, E_phys, nvec, static_cast<void *>(w),
                     status);
  return hipGetLastError();
}

hipError_t launch_replica_grad_reduce(int32_t E, int32_t E_phys, int64_t S,
                                      const int32_t *replica_count, const int32_t *replica_phys,
                                      float *g, int32_t *status, hipStream_t s) {
  const int64_t nvec = S / 4;  // f32, 4 per vector
  hipLaunchKernelGGL(replica_move_kernel<true>, dim3(replica_wgs(nvec, kReduceUnroll), (unsigned)E), dim3(256),
                     0, s, replica_count, replica_phys, E_phys, nvec, static_cast<void *>(g),
                     status);
  return hipGetLastError();
}

hipError_t launch_plan_replicas(int32_t E, int32_t R, int32_t C, const int32_t *load,
                                int32_t *replica_count, int32_t *replica_phys,
                                int32_t *phys_to_logical, hipStream_t s) {
  hipLaunchKernelGGL(plan_replicas_kernel, dim3((unsigned)E), dim3(256), 0, s, E, R, C, load,
                     replica_count, replica_phys, phys_to_logical);
  return hipGetLastError();
}

hipError_t launch_reroute(int32_t T, int32_t K, int32_t E, const int64_t *idx,
                          const int32_t *replica_count, const int32_t *replica_phys,
                          int32_t E_phys, int64_t *phys_idx, int32_t *status, hipStream_t s) {
  const int64_t n = (int64_t)T * K;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(reroute_kernel, dim3(blocks), dim3(256), 0, s, T, K, E, idx, replica_count,
                     replica_phys, E_phys, phys_idx, status);
  return hipGetLastError();
}

}  // namespace moe
