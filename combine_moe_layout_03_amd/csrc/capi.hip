// C-ABI entry points of libmoe_ep.so (declared and documented in moe_ep.h):
// host-side argument checks, then kernel launches on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <atomic>
#include <cstring>

#include "fp8.hpp"
#include "kernels.hpp"
#include "moe_ep.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace moe;

static_assert(MOE_FP8_ROUND_SCALE == kFp8RoundScale && MOE_FP8_UE8M0 == kFp8Ue8m0 &&
                  MOE_FP8_SCALE_ROWS == kFp8ScaleRows,
              "FP8 flag values of the header and the kernels differ");
static_assert(MOE_STATUS_BAD_EXPERT == kStBadExpert && MOE_STATUS_LL_OVERFLOW == kStOverflow &&
                  MOE_STATUS_BAD_SLOT == kStBadSlot && MOE_STATUS_BAD_REPLICA == kStBadReplica,
              "status bits of the header and the kernels differ");

constexpr int kMaxDevices = 64;
constexpr int kMaxRanksNormal = 64;  // a token's set of ranks is one 64-bit mask
std::atomic<int> g_arch[kMaxDevices];  // 0 = not checked yet, 1 = gfx950, 2 = other

// Layout workspace of moe_layout_dispatch_static, for callers that cannot
// allocate: one array per GPU, held until the process ends. In host code its
// name stands for no device address; the address comes from
// hipGetSymbolAddress, once per device, kept in g_scratch.
static_assert(MOE_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];
std::atomic<uintptr_t> g_scratch[kMaxDevices];  // 0 = not looked up yet

// The kernels are compiled for gfx950 only; refuse any other current device.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_DEVICE;
  int state = dev < kMaxDevices ? g_arch[dev].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < kMaxDevices) g_arch[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MOE_OK : MOE_ERR_ARCH;
}

// Device address of the current device's scratch array (looked up on the first
// call on each device, with that device current). NULL if the lookup fails.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uintptr_t a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    a = reinterpret_cast<uintptr_t>(ptr);
    g_scratch[dev].store(a, std::memory_order_release);
  }
  return reinterpret_cast<void *>(a);
}

int bits_for(int n) {  // bits needed to tell apart the values 0 .. n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// FP8 flag set and the hidden sizes it needs: scales cover 128 channels, and
// UE8M0 words pack four of them (and require power-of-two scales).
int check_fp8(int32_t H, int32_t flags) {
  const int cast = flags & ~MOE_FP8_SCALE_ROWS;
  if (flags < 0 || (flags & ~(MOE_FP8_ROUND_SCALE | MOE_FP8_UE8M0 | MOE_FP8_SCALE_ROWS)) ||
      (cast != 0 && cast != MOE_FP8_ROUND_SCALE && cast != (MOE_FP8_ROUND_SCALE | MOE_FP8_UE8M0)))
    return MOE_ERR_FLAGS;
  if (H % kFp8Group != 0) return MOE_ERR_SHAPE;
  if ((flags & MOE_FP8_UE8M0) && H % (4 * kFp8Group) != 0) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Shape checks shared by every call that takes a moe_shape.
int check_shape(const moe_shape *s, bool need_h) {
  if (!s) return MOE_ERR_NULL;
  if (s->T < 0 || s->K < 1 || s->K > 64 || s->E < 1 || s->E > kMaxExperts || s->R < 1 ||
      s->E % s->R != 0 || s->A < 1 || s->A > (1 << 16))
    return MOE_ERR_SHAPE;
  const int64_t worst = (int64_t)s->T * s->K + (int64_t)s->E * (s->A - 1);
  if (worst >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (need_h) {
    if (s->H < 8 || s->H > (1 << 20) || s->H % 8 != 0) return MOE_ERR_SHAPE;
    if ((int64_t)s->T * (s->H / 8) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

int tokens_per_block(int K) { return kPairsPerBlock / K > 0 ? kPairsPerBlock / K : 1; }

bool one_block(const moe_shape *s) { return (int64_t)s->T * s->K <= kMaxPairsOneBlock; }

// The counting kernel lays out batches of up to kMaxPairsFused pairs with
// alignment 1 (low-latency layouts ignore the alignment) without a workspace.
bool counted(const moe_shape *s, int mode) {
  return (int64_t)s->T * s->K <= kMaxPairsFused && (mode == kModeLowLatency || s->A == 1);
}

// Workspace of the three-launch layout; 0 when no call with this shape takes
// it (a low-latency call with A > 1 in the shape may be asked for one that it
// does not use).
size_t workspace_bytes(const moe_shape *s) {
  if (one_block(s) || counted(s, kModeContiguous)) return 0;
  const int64_t tpb = tokens_per_block(s->K);
  const int64_t nb = (s->T + tpb - 1) / tpb;
  const int64_t ints = nb * s->E + nb * s->R + s->E;
  return (size_t)((ints * 4 + 255) / 256 * 256);
}

// Checks a layout call's arguments and fills the kernel parameters.
int layout_params(const moe_shape *s, int mode, int32_t M, int32_t src, const int64_t *idx,
                  const moe_layout_t *out, void *ws, size_t ws_bytes, LayoutParams *p) {
  int rc = check_shape(s, false);
  if (rc) return rc;
  if (!out || !out->count || (s->T > 0 && !out->slot)) return MOE_ERR_NULL;
  if (mode == kModeContiguous && !out->offset) return MOE_ERR_NULL;
  if (s->T > 0 && !idx) return MOE_ERR_NULL;
  if (!aligned8(idx)) return MOE_ERR_ALIGN;
  if (mode == kModeLowLatency) {
    if (M < 1 || s->T > M || src < 0 || src >= s->R) return MOE_ERR_LL;
    if ((int64_t)s->E * s->R * M >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  }
  const bool multi = !one_block(s) && !counted(s, mode);
  const size_t need = multi ? workspace_bytes(s) : 0;
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;

  std::memset(p, 0, sizeof(*p));
  p->idx = idx;
  p->T = s->T;
  p->K = s->K;
  p->E = s->E;
  p->R = s->R;
  p->L = s->E / s->R;
  p->A = mode == kModeContiguous ? s->A : 1;
  p->mode = mode;
  p->M = M;
  p->src = src;
  p->id_bits = bits_for(s->E);
  p->rank_bits = bits_for(s->R);
  p->l_magic = ((1ull << 32) + (uint64_t)p->L - 1) / (uint64_t)p->L;
  p->count = out->count;
  p->offset = out->offset;
  p->rank_token_count = out->rank_token_count;
  p->in_rank = out->is_token_in_rank;
  p->slot = out->slot;
  p->row_src = out->row_src;
  p->status = out->status;
  p->recv_stats = out->recv_stats;
  if (!multi) {  // the counting kernel ignores these
    p->tokens_per_block = s->T > 0 ? s->T : 1;
    p->nblocks = 1;
  } else {
    p->tokens_per_block = tokens_per_block(s->K);
    p->nblocks = (s->T + p->tokens_per_block - 1) / p->tokens_per_block;
    p->ws_hist = static_cast<int32_t *>(ws);
    p->ws_rcnt = p->ws_hist + (int64_t)p->nblocks * s->E;
    p->ws_cnt = p->ws_rcnt + (int64_t)p->nblocks * s->R;
  }
  return MOE_OK;
}

hipError_t launch_layout(const LayoutParams &p, hipStream_t stream) {
  if (count_layout_fits(p, 0, false))
    return launch_count_layout(p, nullptr, nullptr, 0, 0, nullptr, stream);
  return p.nblocks == 1 && p.ws_hist == nullptr ? launch_layout_one_block(p, stream)
                                                 : launch_layout_multi_block(p, stream);
}

int layout_common(const moe_shape *s, int mode, int32_t M, int32_t src, const int64_t *idx,
                  const moe_layout_t *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  LayoutParams p;
  int rc = layout_params(s, mode, M, src, idx, out, ws, ws_bytes, &p);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  return launch_layout(p, stream) == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Layout + dispatch: bf16 rows into recv, or (fp8 != null, low latency) the
// E4M3 cast into fp8->q / fp8->scale.
int layout_dispatch_common(const moe_shape *s, int mode, int32_t M, int32_t src,
                           const int64_t *idx, const moe_layout_t *out, const uint16_t *x,
                           uint16_t *recv, int64_t rows, const Fp8Out *fp8, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s, true);
  if (rc) return rc;
  LayoutParams p;
  rc = layout_params(s, mode, M, src, idx, out, ws, ws_bytes, &p);
  if (rc) return rc;
  if (rows < 0) return MOE_ERR_CAPACITY;
  if (fp8) {
    rc = check_fp8(s->H, fp8->flags);
    if (rc) return rc;
    if (rows > (int64_t)s->E * s->R * M) return MOE_ERR_CAPACITY;
    if (s->T > 0 && (!x || (rows > 0 && (!fp8->q || !fp8->scale)))) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(fp8->q) || !aligned4(fp8->scale)) return MOE_ERR_ALIGN;
  } else {
    if (s->T > 0 && (!x || (!recv && rows > 0))) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(recv)) return MOE_ERR_ALIGN;
  }
  rc = check_device();
  if (rc) return rc;
  hipError_t err;
  if (count_layout_fits(p, s->H, true)) {
    err = launch_count_layout(p, x, recv, rows, s->H, fp8, stream);
  } else {
    err = launch_layout(p, stream);
    if (err == hipSuccess && s->T > 0) {
      err = fp8 ? launch_ll_quant_dispatch(x, p.slot, *fp8, s->T, s->K, s->H, rows, p.status,
                                           stream)
                : launch_dispatch(x, p.slot, recv, s->T, s->K, s->H, rows, p.status, stream);
    }
  }
  return err == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_CAPACITY: return "receive buffer size is invalid";
    case MOE_ERR_LL: return "low latency: T > M or src_rank outside [0, R)";
    case MOE_ERR_ALIGN: return "a pointer is not aligned as required (rows 16 bytes, ids 8)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_ARCH: return "current device is not gfx950";
    case MOE_ERR_DEVICE: return "HIP runtime query failed";
    case MOE_ERR_FLAGS: return "unsupported FP8 flag combination";
    case MOE_ERR_SCRATCH:
      return "shape needs a larger layout workspace than the static scratch holds";
    default: return "unknown error code";
  }
}

MOE_API int64_t moe_recv_rows_worst(const moe_shape *shape) {
  if (check_shape(shape, false)) return -1;
  return (int64_t)shape->T * shape->K + (int64_t)shape->E * (shape->A - 1);
}

MOE_API int64_t moe_ll_recv_rows(int32_t E, int32_t R, int32_t M) {
  if (E < 1 || R < 1 || M < 1 || E % R != 0) return -1;
  return (int64_t)E * R * M;
}

MOE_API size_t moe_layout_workspace_bytes(const moe_shape *shape) {
  if (check_shape(shape, false)) return 0;
  return workspace_bytes(shape);
}

MOE_API int moe_layout(const moe_shape *shape, const int64_t *topk_idx, const moe_layout_t *out,
                       void *ws, size_t ws_bytes, hipStream_t stream) {
  return layout_common(shape, kModeContiguous, 0, 0, topk_idx, out, ws, ws_bytes, stream);
}

MOE_API int moe_ll_layout(const moe_shape *shape, int32_t M, int32_t src_rank,
                          const int64_t *topk_idx, const moe_layout_t *out, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  return layout_common(shape, kModeLowLatency, M, src_rank, topk_idx, out, ws, ws_bytes, stream);
}

MOE_API int moe_layout_dispatch(const moe_shape *shape, const int64_t *topk_idx,
                                const moe_layout_t *out, const uint16_t *x, uint16_t *recv_x,
                                int64_t recv_rows, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  return layout_dispatch_common(shape, kModeContiguous, 0, 0, topk_idx, out, x, recv_x,
                                recv_rows, nullptr, ws, ws_bytes, stream);
}

MOE_API int moe_layout_dispatch_static(const moe_shape *shape, const int64_t *topk_idx,
                                       const moe_layout_t *out, const uint16_t *x,
                                       uint16_t *recv_x, int64_t recv_rows, hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  const size_t need = workspace_bytes(shape);
  if (need == 0)  // counted or one-workgroup layout: no scratch
    return layout_dispatch_common(shape, kModeContiguous, 0, 0, topk_idx, out, x, recv_x,
                                  recv_rows, nullptr, nullptr, 0, stream);
  if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  rc = check_device();
  if (rc) return rc;
  void *ws = device_scratch();
  if (!ws) return MOE_ERR_DEVICE;
  return layout_dispatch_common(shape, kModeContiguous, 0, 0, topk_idx, out, x, recv_x,
                                recv_rows, nullptr, ws, MOE_STATIC_SCRATCH_BYTES, stream);
}

MOE_API int moe_ll_layout_dispatch(const moe_shape *shape, int32_t M, int32_t src_rank,
                                   const int64_t *topk_idx, const moe_layout_t *out,
                                   const uint16_t *x, uint16_t *recv_x, int64_t recv_rows,
                                   void *ws, size_t ws_bytes, hipStream_t stream) {
  return layout_dispatch_common(shape, kModeLowLatency, M, src_rank, topk_idx, out, x, recv_x,
                                recv_rows, nullptr, ws, ws_bytes, stream);
}

MOE_API int moe_ll_layout_dispatch_fp8(const moe_shape *shape, int32_t M, int32_t src_rank,
                                       const int64_t *topk_idx, const moe_layout_t *out,
                                       const uint16_t *x, uint8_t *recv_q, void *recv_scale,
                                       int64_t recv_rows, int32_t flags, void *ws,
                                       size_t ws_bytes, hipStream_t stream) {
  if (!shape) return MOE_ERR_NULL;
  // R*M is validated (E*R*M < 2^31) by the layout checks before any use
  const int64_t rm = (int64_t)shape->R * (M > 0 ? M : 0);
  Fp8Out o{flags, recv_q, recv_scale, (int32_t)(rm < (1ll << 31) ? rm : 0)};
  return layout_dispatch_common(shape, kModeLowLatency, M, src_rank, topk_idx, out, x, nullptr,
                                recv_rows, &o, ws, ws_bytes, stream);
}

MOE_API int moe_ll_dispatch_fp8(const moe_shape *shape, int32_t M, const uint16_t *x,
                                const int32_t *slot, uint8_t *recv_q, void *recv_scale,
                                int64_t recv_rows, int32_t flags, int32_t *status,
                                hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  rc = check_fp8(shape->H, flags);
  if (rc) return rc;
  if (M < 1 || (int64_t)shape->E * shape->R * M >= ((int64_t)1 << 31)) return MOE_ERR_LL;
  if (recv_rows < 0 || recv_rows > (int64_t)shape->E * shape->R * M) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!x || !slot || (recv_rows > 0 && (!recv_q || !recv_scale))) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(recv_q) || !aligned4(recv_scale)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  const Fp8Out o{flags, recv_q, recv_scale, shape->R * M};
  return launch_ll_quant_dispatch(x, slot, o, shape->T, shape->K, shape->H, recv_rows, status,
                                  stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_dispatch_fp8(const moe_shape *shape, const uint8_t *x_q, const float *x_scale,
                             const int32_t *slot, uint8_t *recv_q, float *recv_scale,
                             int64_t recv_rows, int32_t *status, hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (shape->H % kFp8Group != 0) return MOE_ERR_SHAPE;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!x_q || !x_scale || !slot || (recv_rows > 0 && (!recv_q || !recv_scale)))
    return MOE_ERR_NULL;
  if (!aligned16(x_q) || !aligned16(recv_q) || !aligned4(x_scale) || !aligned4(recv_scale))
    return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_fp8_copy_dispatch(x_q, x_scale, slot, recv_q, recv_scale, shape->T, shape->K,
                                  shape->H, recv_rows, status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, void *scale,
                             int32_t flags, hipStream_t stream) {
  if (T < 0 || H < kFp8Group || H > (1 << 20)) return MOE_ERR_SHAPE;
  if ((int64_t)T * (H / 8) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  int rc = check_fp8(H, flags);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_quantize_fp8(x, q, scale, flags, T, H, stream) == hipSuccess ? MOE_OK
                                                                              : MOE_ERR_LAUNCH;
}

MOE_API int moe_expert_load(int32_t T, int32_t K, int32_t E, const int64_t *topk_idx,
                            int32_t *load, int32_t *status, hipStream_t stream) {
  if (T < 0 || K < 1 || K > 64 || E < 1 || E > kMaxExperts) return MOE_ERR_SHAPE;
  if ((int64_t)T * K >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (!load || (T > 0 && !topk_idx)) return MOE_ERR_NULL;
  if (!aligned8(topk_idx)) return MOE_ERR_ALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_expert_load(topk_idx, T, K, E, bits_for(E), load, status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *slot,
                         uint16_t *recv_x, int64_t recv_rows, int32_t *status,
                         hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!x || !slot || (!recv_x && recv_rows > 0)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(recv_x)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_dispatch(x, slot, recv_x, shape->T, shape->K, shape->H, recv_rows, status,
                         stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_combine(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                        const int32_t *slot, const float *topk_weights, uint16_t *out,
                        float *out_f32, int32_t *status, hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!slot || !out || (!y && recv_rows > 0)) return MOE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out) || !aligned16(out_f32)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_combine(y, recv_rows, slot, topk_weights, out, out_f32, shape->T, shape->K,
                        shape->H, nullptr, status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_combine_masked(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                               const int32_t *slot, const int64_t *topk_idx,
                               const float *topk_weights, const int32_t *rank_mask,
                               uint16_t *out, float *out_f32, int32_t *status,
                               hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!slot || !out || !topk_idx || !rank_mask || (!y && recv_rows > 0)) return MOE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out) || !aligned16(out_f32) || !aligned8(topk_idx))
    return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  const uint64_t L = (uint64_t)(shape->E / shape->R);
  const CombineMask cm{topk_idx, rank_mask, shape->E, ((1ull << 32) + L - 1) / L};
  return launch_combine(y, recv_rows, slot, topk_weights, out, out_f32, shape->T, shape->K,
                        shape->H, &cm, status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int64_t moe_rank_recv_rows_worst(const moe_shape *shape) {
  if (check_shape(shape, false)) return -1;
  return (int64_t)shape->T * (shape->K < shape->R ? shape->K : shape->R);
}

MOE_API int moe_rank_layout(const moe_shape *shape, const int64_t *topk_idx,
                            const float *topk_weights, const moe_rank_layout_t *out,
                            int64_t recv_cap, hipStream_t stream) {
  int rc = check_shape(shape, false);
  if (rc) return rc;
  if (shape->R > kMaxRanksNormal) return MOE_ERR_SHAPE;
  if (!out || !out->rank_offset || (shape->T > 0 && !out->rank_slot)) return MOE_ERR_NULL;
  if (shape->T > 0 && !topk_idx) return MOE_ERR_NULL;
  if (out->recv_topk_weights && !topk_weights && shape->T > 0) return MOE_ERR_NULL;
  if (!aligned8(topk_idx)) return MOE_ERR_ALIGN;
  if (recv_cap < 0) return MOE_ERR_CAPACITY;
  rc = check_device();
  if (rc) return rc;
  return launch_rank_layout(topk_idx, topk_weights, shape->T, shape->K, shape->E, shape->R,
                            shape->A, out->rank_slot, out->rank_offset, out->recv_src,
                            out->recv_topk_idx, out->recv_topk_weights, out->recv_expert_count,
                            recv_cap, out->status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_rank_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *rank_slot,
                              uint16_t *recv_x, int64_t recv_rows, int32_t *status,
                              hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (shape->R > kMaxRanksNormal) return MOE_ERR_SHAPE;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!x || !rank_slot || (!recv_x && recv_rows > 0)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(recv_x)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  // one row copy per (token, rank): the pair scatter over the [T, R] table
  return launch_dispatch(x, rank_slot, recv_x, shape->T, shape->R, shape->H, recv_rows, status,
                         stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_rank_layout_dispatch(const moe_shape *shape, const int64_t *topk_idx,
                                     const float *topk_weights, const moe_rank_layout_t *out,
                                     int64_t recv_cap, const uint16_t *x, uint16_t *recv_x,
                                     int64_t recv_rows, hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (shape->R > kMaxRanksNormal) return MOE_ERR_SHAPE;
  if (!out || !out->rank_offset || (shape->T > 0 && !out->rank_slot)) return MOE_ERR_NULL;
  if (shape->T > 0 && !topk_idx) return MOE_ERR_NULL;
  if (out->recv_topk_weights && !topk_weights && shape->T > 0) return MOE_ERR_NULL;
  if (recv_cap < 0 || recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T > 0 && (!x || (!recv_x && recv_rows > 0))) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(recv_x) || !aligned8(topk_idx)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  hipError_t e;
  if (rank_layout_dispatch_fits(shape->T, shape->K, shape->R)) {
    e = launch_rank_layout_dispatch(topk_idx, topk_weights, shape->T, shape->K, shape->E,
                                    shape->R, shape->A, out->rank_slot, out->rank_offset,
                                    out->recv_src, out->recv_topk_idx, out->recv_topk_weights,
                                    out->recv_expert_count, recv_cap, out->status, x, recv_x,
                                    recv_rows, shape->H, stream);
  } else {
    e = launch_rank_layout(topk_idx, topk_weights, shape->T, shape->K, shape->E, shape->R,
                           shape->A, out->rank_slot, out->rank_offset, out->recv_src,
                           out->recv_topk_idx, out->recv_topk_weights, out->recv_expert_count,
                           recv_cap, out->status, stream);
    if (e == hipSuccess && shape->T > 0)
      e = launch_dispatch(x, out->rank_slot, recv_x, shape->T, shape->R, shape->H, recv_rows,
                          out->status, stream);
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

MOE_API int moe_rank_combine(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                             const int32_t *rank_slot, const float *recv_topk_weights,
                             uint16_t *out, float *out_f32, float *out_topk_weights,
                             int32_t *status, hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (shape->R > kMaxRanksNormal) return MOE_ERR_SHAPE;
  if (recv_rows < 0) return MOE_ERR_CAPACITY;
  if (shape->T == 0) return MOE_OK;
  if (!rank_slot || !out || (!y && recv_rows > 0)) return MOE_ERR_NULL;
  if (out_topk_weights && !recv_topk_weights) return MOE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out) || !aligned16(out_f32)) return MOE_ERR_ALIGN;
  rc = check_device();
  if (rc) return rc;
  // the unweighted row sum over the [T, R] table, with the weights summed back
  const RowWeightSum ws{out_topk_weights ? recv_topk_weights : nullptr, out_topk_weights,
                        shape->K};
  return launch_rank_combine(y, recv_rows, rank_slot, out, out_f32, shape->T, shape->R,
                             shape->H, ws, status, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_plan_replicas(int32_t E, int32_t R, int32_t C, const int32_t *load,
                              int32_t *replica_count, int32_t *replica_phys,
                              int32_t *phys_to_logical, hipStream_t stream) {
  if (E < 1 || E > kMaxExperts || R < 1 || E % R != 0 || C < 0 || C > E || C % R != 0)
    return MOE_ERR_SHAPE;
  if (!load || !replica_count || !replica_phys || !phys_to_logical) return MOE_ERR_NULL;
  int rc = check_device();
  if (rc) return rc;
  return launch_plan_replicas(E, R, C, load, replica_count, replica_phys, phys_to_logical,
                              stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

namespace {
int replica_move_checks(int32_t E, int32_t E_phys, int64_t S, const int32_t *replica_count,
                        const int32_t *replica_phys, const void *buf) {
  if (E < 1 || E > 65535 || E_phys < E || S < 0 || S % 8 != 0) return MOE_ERR_SHAPE;
  if (S > 0 && (int64_t)E_phys * S / 4 >= ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  if (!replica_count || !replica_phys || (S > 0 && !buf)) return MOE_ERR_NULL;
  if (!aligned16(buf)) return MOE_ERR_ALIGN;
  return MOE_OK;
}
}  // namespace

MOE_API int moe_replica_weight_sync(int32_t E, int32_t E_phys, int64_t S,
                                    const int32_t *replica_count, const int32_t *replica_phys,
                                    uint16_t *w, int32_t *status, hipStream_t stream) {
  int rc = replica_move_checks(E, E_phys, S, replica_count, replica_phys, w);
  if (rc) return rc;
  if (S == 0) return MOE_OK;
  rc = check_device();
  if (rc) return rc;
  return launch_replica_weight_sync(E, E_phys, S, replica_count, replica_phys, w, status,
                                    stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_replica_grad_reduce(int32_t E, int32_t E_phys, int64_t S,
                                    const int32_t *replica_count, const int32_t *replica_phys,
                                    float *g, int32_t *status, hipStream_t stream) {
  int rc = replica_move_checks(E, E_phys, S, replica_count, replica_phys, g);
  if (rc) return rc;
  if (S == 0) return MOE_OK;
  rc = check_device();
  if (rc) return rc;
  return launch_replica_grad_reduce(E, E_phys, S, replica_count, replica_phys, g, status,
                                    stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API int moe_reroute(int32_t T, int32_t K, int32_t E, const int64_t *topk_idx,
                        const int32_t *replica_count, const int32_t *replica_phys,
                        int32_t E_phys, int64_t *phys_idx, int32_t *status, hipStream_t stream) {
  if (T < 0 || K < 1 || K > 64 || E < 1 || E > kMaxExperts || E_phys < 1) return MOE_ERR_SHAPE;
  if ((int64_t)T * K >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !replica_count || !replica_phys || !phys_idx) return MOE_ERR_NULL;
  if (!aligned8(topk_idx) || !aligned8(phys_idx)) return MOE_ERR_ALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_reroute(T, K, E, topk_idx, replica_count, replica_phys, E_phys, phys_idx, status,
                        stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}
