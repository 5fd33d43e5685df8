// fa_api.hip -- the C ABI declared in include/fa.h: argument validation,
// kernel-instance dispatch and launch on the caller's stream.  No call here
// allocates, copies or synchronises.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kMaxDevices = 64;

namespace {
std::atomic<int> g_device_cus[kMaxDevices];  // 0 until the device's count is read
}  // namespace

// Racing first calls on one device both read the same count and store it;
// every later call on that device reads the cached value.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int cached = g_device_cus[dev].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  g_device_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace fa

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int check_common(int B, int H, int N, int D, float scale, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const int64_t elems = (int64_t)B * H * N * D;
  if (elems > (int64_t)INT32_MAX) return FA_ERR_INVALID_ARG;
  // head dims some kernel serves; each launcher returns "unsupported" for
  // the ones it does not (the backward and the float32 forward: 64, 128, 256)
  if (D != 32 && D != 64 && D != 96 && D != 128 && D != 160 && D != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int map_launch(int rc) {
  if (rc == 0) return FA_OK;
  if (rc == -2) return FA_ERR_UNSUPPORTED;
  return FA_ERR_LAUNCH;
}

fa::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
                     float scale, int causal) {
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal;
  a.Nk = N;
  a.n_split = 1;
  a.part_o = nullptr;
  a.part_l = nullptr;
  a.block_mask = nullptr;
  a.mask_heads = 0;
  return a;
}

constexpr int kMaxSplits = 256;

// The vector decode kernel serves up to kDecodeMaxRows rows at D = 64, 128,
// 256 (a K row split over D/8 lanes must divide the wave); the rest runs on
// the matrix-core kernel.
bool use_decode(int Nq, int D) { return Nq <= fa::kDecodeMaxRows && (D == 64 || D == 128 || D == 256); }

// Key ranges per query block when the caller leaves the choice to the
// library.  Matrix-core path: enough (query block, key range) workgroups to
// give every CU its share of workgroups at once, and at least two key tiles
// of 64 per range.  Decode path (Nq <= 4): about one workgroup per CU (two
// for three or four rows), at least two ranges, each over at least 256 keys
// (measured: 256 to 512 decode workgroups beat both fewer and more).
int choose_splits(int B, int H, int Nq, int Nk, int D) {
  const int cus = fa::device_cus();
  if (use_decode(Nq, D)) {
    const int64_t heads = (int64_t)B * H;
    int64_t s = (cus + heads - 1) / heads;
    if (s < 2) s = 2;
    if (Nq > 2) s *= 2;
    const int64_t ranges = (Nk + 255) / 256;
    s = s < ranges ? s : ranges;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : (int)s;
  }
  const int64_t slots = (int64_t)cus * fa::fwd_workgroups_per_cu(D);
  const int rows = fa::fwd_rows_per_workgroup(D, Nq);
  const int64_t blocks = (int64_t)((Nq + rows - 1) / rows) * B * H;
  if (blocks >= slots) return 1;
  int64_t s = (slots + blocks - 1) / blocks;
  const int64_t tiles = (Nk + 63) / 64;
  s = s < tiles / 2 ? s : tiles / 2;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

size_t kv_workspace_bytes(int B, int H, int Nq, int D, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * B * H * Nq * (size_t)(D + 1) * sizeof(float);
}

int check_kv(int B, int H, int Nq, int Nk, int D, float scale, int causal) {
  if (Nk <= 0) return FA_ERR_INVALID_ARG;
  int rc = check_common(B, H, Nq, D, scale, causal);
  if (rc != FA_OK) return rc;
  if ((int64_t)B * H * Nk * D > (int64_t)INT32_MAX) return FA_ERR_INVALID_ARG;
  if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Checks shared by fa_fwd_kv and fa_fwd_kv_noalloc, and the range count.
// HIP's launch limit is on work-items (workgroups x threads per workgroup
// below 2^32), for the range kernel and for the merge: both are checked
// here, before anything is launched.
int kv_prepare(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
               float scale, int causal, int num_splits, int* splits_out) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const int rc = check_kv(B, H, Nq, Nk, D, scale, causal);
  if (rc != FA_OK) return rc;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  const int splits = num_splits == 0 ? choose_splits(B, H, Nq, Nk, D) : num_splits;
  const int64_t rows = (int64_t)B * H * Nq;
  int64_t workgroups, threads;
  if (use_decode(Nq, D)) {
    workgroups = (int64_t)B * H * splits;
    threads = fa::kDecodeThreads;
  } else {
    const int rows_wg = fa::fwd_rows_per_workgroup(D, Nq);
    workgroups = (int64_t)((Nq + rows_wg - 1) / rows_wg) * splits * B * H;
    threads = fa::fwd_threads_per_workgroup(D, Nq);
  }
  if (workgroups * threads > (int64_t)UINT32_MAX) return FA_ERR_INVALID_ARG;
  // the merge: one 256-thread workgroup per row for many ranges, else
  // 256-thread workgroups of 256 / (D/4) rows
  if (splits > 1) {
    const int64_t rows_per_wg = 256 / (D / 4);
    const int64_t merge_wgs = splits > fa::kMaxNarrowMerge ? rows : (rows + rows_per_wg - 1) / rows_per_wg;
    if (merge_wgs * 256 > (int64_t)UINT32_MAX) return FA_ERR_INVALID_ARG;
  }
  *splits_out = splits;
  return FA_OK;
}

int kv_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
           float scale, int causal, int splits, void* workspace, void* stream) {
  fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, Nq, D, scale, causal);
  a.Nk = Nk;
  a.n_split = splits;
  if (splits > 1) {
    a.part_o = (float*)workspace;
    a.part_l = (float*)workspace + (size_t)splits * B * H * Nq * D;
  }
  int lrc = use_decode(Nq, D) ? fa::launch_fwd_decode(a, (hipStream_t)stream)
                              : fa::launch_fwd_bf16_kv(a, (hipStream_t)stream);
  if (lrc == 0 && splits > 1) lrc = fa::launch_fwd_kv_merge(a, (hipStream_t)stream);
  return map_launch(lrc);
}

// Scratch of fa_fwd_kv_noalloc: the key-range partials of one call, in a
// fixed array that each device holds from the library's first use on it
// until the process ends.  In host code `scratch` only names the symbol;
// its device address is looked up once per device (with that device
// current) and kept in g_scratch.  Every call on one device shares the
// array, so calls that overlap on one device race.  Nothing in it has to
// start at zero: every range writes all of its partial rows.
std::atomic<void*> g_scratch[fa::kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[FA_FWD_KV_NOALLOC_MAX_BYTES];

namespace {

void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= fa::kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int fa_version(void) { return (1 << 16) | 0; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK:
      return "success";
    case FA_ERR_INVALID_ARG:
      return "invalid argument (null pointer, non-positive size, bad scale or causal flag, or size overflow)";
    case FA_ERR_UNSUPPORTED:
      return "unsupported shape (head dimension: 32, 64, 96, 128, 160 or 256 for the bf16 forward, 64, 128 or "
             "256 for the float32 forward, 32, 64, 96, 128 or 256 for the backward) or block-sparse sequence length "
             "above 262144";
    case FA_ERR_LAUNCH:
      return "kernel launch failed";
    default:
      return "unknown error code";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D, float scale,
           int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, D, scale, causal);
  if (rc != FA_OK) return rc;
  const fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, N, D, scale, causal);
  return map_launch(fa::launch_fwd_bf16(a, (hipStream_t)stream));
}

int fa_fwd_kv_splits(int B, int H, int Nq, int Nk, int D, int causal) {
  const int rc = check_kv(B, H, Nq, Nk, D, 1.0f, causal);
  if (rc != FA_OK) return rc;
  return choose_splits(B, H, Nq, Nk, D);
}

size_t fa_fwd_kv_workspace_bytes(int B, int H, int Nq, int D, int num_splits) {
  if (B <= 0 || H <= 0 || Nq <= 0 || D <= 0 || num_splits <= 0) return 0;
  return kv_workspace_bytes(B, H, Nq, D, num_splits);
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
              float scale, int causal, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int splits = 0;
  const int rc = kv_prepare(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, num_splits, &splits);
  if (rc != FA_OK) return rc;
  const size_t need = kv_workspace_bytes(B, H, Nq, D, splits);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15) != 0)) return FA_ERR_INVALID_ARG;
  return kv_run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, splits, workspace, stream);
}

int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                      int D, float scale, int causal, int num_splits, void* stream) {
  int splits = 0;
  const int rc = kv_prepare(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, num_splits, &splits);
  if (rc != FA_OK) return rc;
  const size_t need = kv_workspace_bytes(B, H, Nq, D, splits);
  if (need > FA_FWD_KV_NOALLOC_MAX_BYTES) return FA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr();
    if (!ws) return FA_ERR_LAUNCH;
  }
  return kv_run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, splits, ws, stream);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
                  float scale, int causal, const unsigned char* block_mask, int mask_heads, void* stream) {
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, D, scale, causal);
  if (rc != FA_OK) return rc;
  if (mask_heads != 1 && (int64_t)mask_heads != (int64_t)B * H) return FA_ERR_INVALID_ARG;
  const int64_t nb = ((int64_t)N + fa::kSparseBlock - 1) / fa::kSparseBlock;
  if (nb > fa::kSparseMaxTiles) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, N, D, scale, causal);
  a.block_mask = block_mask;
  a.mask_heads = mask_heads;
  return map_launch(fa::launch_fwd_bf16_sparse(a, (hipStream_t)stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int D,
               float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, D, scale, causal);
  if (rc != FA_OK) return rc;
  return map_launch(fa::launch_fwd_f32(fwd_args(q, k, v, o, lse, B, H, N, D, scale, causal), (hipStream_t)stream));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
              float* delta, void* dq, int B, int H, int N, int D, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !delta || !dq) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, D, scale, causal);
  if (rc != FA_OK) return rc;
  fa::BwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dO = dO;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal;
  return map_launch(fa::launch_bwd_dq(a, (hipStream_t)stream));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                void* dk, void* dv, int B, int H, int N, int D, float scale, int causal, void* stream) {
  if (!q || !k || !v || !dO || !lse || !delta || !dk || !dv) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, D, scale, causal);
  if (rc != FA_OK) return rc;
  fa::BwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse = lse;
  a.delta = const_cast<float*>(delta);
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal;
  return map_launch(fa::launch_bwd_dkdv(a, (hipStream_t)stream));
}

}  // extern "C"
