// C ABI of libwavealign: host-side argument validation and kernel launches.
// No entry point allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "wa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return WA_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(WA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

bool supported_shape(int head_dim, int block) {
  return (head_dim == 64 || head_dim == 128) && (block == 64 || block == 128);
}

// XCD (L2 domain) count of the device that runs `stream` (the current device for
// the null stream); 1 if the runtime does not report it.
hipError_t stream_xcds(hipStream_t stream, int* n_xcd) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int x = 0;
  e = hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev);
  *n_xcd = (e == hipSuccess && x >= 1) ? x : 1;
  return hipSuccess;
}

}  // namespace

extern "C" {

int wa_abi_version(void) { return 4; }

const char* wa_last_error(void) { return g_err; }

int wa_schedule_info(int device, int32_t head_dim, int32_t* n_xcd, int32_t* cus_per_xcd,
                     int32_t* wave) {
  if (!n_xcd || !cus_per_xcd || !wave) return fail(WA_ERR_INVALID_ARG, "null output pointer");
  if (head_dim != 64 && head_dim != 128)
    return fail(WA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  int cus = 0, xccs = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute(cu count)");
  e = hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, device);
  if (e != hipSuccess || xccs < 1) xccs = 1;
  *n_xcd = xccs;
  *cus_per_xcd = cus / xccs;
  *wave = (cus / xccs) * wa::attn_resident_wgs_per_cu(head_dim, 128);
  return ok();
}

int wa_build_block_index(const uint8_t* mask, int32_t H, int32_t MB, int32_t NB,
                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                         int32_t* row_nnz, int32_t* csc_ptr, int32_t* csc_idx,
                         int64_t csc_capacity, void* stream) {
  if (!mask || !row_ptr || !row_nnz || (!col_idx && col_capacity > 0))
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if ((int64_t)H * MB * NB >= (int64_t)1 << 31)
    return fail(WA_ERR_UNSUPPORTED, "H*MB*NB must be below 2^31");
  if (col_capacity < 0 || csc_capacity < 0)
    return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if (csc_ptr != nullptr && csc_idx == nullptr && csc_capacity > 0)
    return fail(WA_ERR_INVALID_ARG, "csc_idx is null but csc_ptr is set");
  return hip_status(wa::launch_block_index(mask, H, MB, NB, row_ptr, col_idx, col_capacity,
                                           row_nnz, csc_ptr, csc_idx, csc_capacity,
                                           static_cast<hipStream_t>(stream)),
                    "wa_build_block_index");
}

int wa_reorder_rows(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* csc_ptr,
                    const int32_t* csc_idx, int64_t capacity, const float* x0, int32_t H,
                    int32_t MB, int32_t NB,
                    int32_t block, int32_t head_dim, const wa_reorder_params* params,
                    int32_t* perm, int32_t* inv_perm, uint8_t* skipped, double* angles,
                    double* stats, void* stream) {
  if (!row_ptr || !col_idx || !x0 || !params || !perm || !inv_perm || !skipped)
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if (MB > WA_MAX_BLOCKS || NB > WA_MAX_BLOCKS)
    return fail(WA_ERR_UNSUPPORTED, "MB and NB must be <= %d", WA_MAX_BLOCKS);
  if ((!csc_ptr || !csc_idx) && wa::reorder_needs_csc(MB, NB))
    return fail(WA_ERR_INVALID_ARG, "csc_ptr and csc_idx are required for MB=%d, NB=%d", MB, NB);
  if (block < 1 || head_dim < 1) return fail(WA_ERR_UNSUPPORTED, "block and head_dim must be >= 1");
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  const wa_reorder_params& p = *params;
  if (p.wave < 1) return fail(WA_ERR_INVALID_ARG, "wave must be >= 1");
  if (p.n_slices < 1 || p.n_slices > 64) return fail(WA_ERR_INVALID_ARG, "n_slices must be in 1..64");
  if (p.iters < 0 || p.iters > 1000) return fail(WA_ERR_INVALID_ARG, "iters must be in 0..1000");
  if (p.skip_mode < WA_SKIP_ADAPTIVE || p.skip_mode > WA_SKIP_ALWAYS)
    return fail(WA_ERR_INVALID_ARG, "unknown skip_mode %d", p.skip_mode);
  if ((p.stage1 != 0 && p.stage1 != 1) || (p.stage2 != 0 && p.stage2 != 1))
    return fail(WA_ERR_INVALID_ARG, "stage1 and stage2 must be 0 or 1");
  return hip_status(wa::launch_reorder(row_ptr, col_idx, csc_ptr, csc_idx, capacity, x0, H, MB, NB, block,
                                       head_dim, p, perm, inv_perm, skipped, angles, stats,
                                       static_cast<hipStream_t>(stream)),
                    "wa_reorder_rows");
}

int wa_minhash_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t capacity, int32_t H,
                     int32_t MB, int32_t NB, const uint32_t* hash_a, const uint32_t* hash_b,
                     int32_t n_hash, int32_t wave, int32_t n_slices, int32_t stage2,
                     int32_t* perm, int32_t* inv_perm, void* stream) {
  if (!row_ptr || !col_idx || !hash_a || !hash_b || !perm || !inv_perm)
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if (MB > WA_MAX_BLOCKS || NB > WA_MAX_BLOCKS)
    return fail(WA_ERR_UNSUPPORTED, "MB and NB must be <= %d", WA_MAX_BLOCKS);
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if (n_hash != 1 && n_hash != 2) return fail(WA_ERR_INVALID_ARG, "n_hash must be 1 or 2");
  for (int i = 0; i < n_hash; ++i)
    if (hash_a[i] < 1 || hash_a[i] >= 0x7fffffffu || hash_b[i] >= 0x7fffffffu)
      return fail(WA_ERR_INVALID_ARG, "hash coefficients must satisfy 1 <= a < 2^31-1, b < 2^31-1");
  if (wave < 1) return fail(WA_ERR_INVALID_ARG, "wave must be >= 1");
  if (n_slices < 1 || n_slices > 64) return fail(WA_ERR_INVALID_ARG, "n_slices must be in 1..64");
  if (stage2 != 0 && stage2 != 1) return fail(WA_ERR_INVALID_ARG, "stage2 must be 0 or 1");
  return hip_status(wa::launch_minhash_order(row_ptr, col_idx, capacity, H, MB, NB, hash_a, hash_b,
                                             n_hash, wave, n_slices, stage2, perm, inv_perm,
                                             static_cast<hipStream_t>(stream)),
                    "wa_minhash_order");
}

int wa_lsh_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t capacity, int32_t H,
                 int32_t MB, int32_t NB, const uint32_t* hash_a, const uint32_t* hash_b,
                 int32_t n_bands, int32_t wave, int32_t n_slices, int32_t stage2,
                 int32_t* perm, int32_t* inv_perm, void* stream) {
  if (!row_ptr || !col_idx || !hash_a || !hash_b || !perm || !inv_perm)
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if (MB > WA_MAX_BLOCKS || NB > WA_MAX_BLOCKS)
    return fail(WA_ERR_UNSUPPORTED, "MB and NB must be <= %d", WA_MAX_BLOCKS);
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if (n_bands < 1 || n_bands > wa::kLshMaxBands)
    return fail(WA_ERR_INVALID_ARG, "n_bands must be in 1..%d", wa::kLshMaxBands);
  for (int i = 0; i < 2 * n_bands; ++i)
    if (hash_a[i] < 1 || hash_a[i] >= 0x7fffffffu || hash_b[i] >= 0x7fffffffu)
      return fail(WA_ERR_INVALID_ARG, "hash coefficients must satisfy 1 <= a < 2^31-1, b < 2^31-1");
  if (wave < 1) return fail(WA_ERR_INVALID_ARG, "wave must be >= 1");
  if (n_slices < 1 || n_slices > 64) return fail(WA_ERR_INVALID_ARG, "n_slices must be in 1..64");
  if (stage2 != 0 && stage2 != 1) return fail(WA_ERR_INVALID_ARG, "stage2 must be 0 or 1");
  return hip_status(wa::launch_lsh_order(row_ptr, col_idx, capacity, H, MB, NB, hash_a, hash_b,
                                         n_bands, wave, n_slices, stage2, perm, inv_perm,
                                         static_cast<hipStream_t>(stream)),
                    "wa_lsh_order");
}

int wa_reorder_needs_csc(int32_t MB, int32_t NB) {
  if (MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "MB and NB must be >= 1");
  if (MB > WA_MAX_BLOCKS || NB > WA_MAX_BLOCKS)
    return fail(WA_ERR_UNSUPPORTED, "MB and NB must be <= %d", WA_MAX_BLOCKS);
  ok();
  return wa::reorder_needs_csc(MB, NB) ? 1 : 0;
}

int wa_sparse_attn_workspace_size(int32_t H, int32_t L, int32_t head_dim, int32_t block,
                                  size_t* bytes) {
  if (!bytes) return fail(WA_ERR_INVALID_ARG, "null output pointer");
  if (H < 1 || L < 1) return fail(WA_ERR_INVALID_ARG, "H and L must be >= 1");
  if (!supported_shape(head_dim, block))
    return fail(WA_ERR_UNSUPPORTED, "head_dim %d / block %d not in {64, 128}", head_dim, block);
  const int MB = (L + block - 1) / block;
  *bytes = wa::attn_workspace_bytes(H, MB * block, head_dim);
  return ok();
}

// Host-side validation of an attention call; on success *n_xcd is the XCD count of
// the stream's device and nothing has been enqueued.
static int sparse_attn_check(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                             int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                             const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                             int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream,
                             int* n_xcd_out) {
  if (!q || !k || !v || !row_ptr || !col_idx || !o || !lse)
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || L < 1) return fail(WA_ERR_INVALID_ARG, "H and L must be >= 1");
  if (!supported_shape(head_dim, block))
    return fail(WA_ERR_UNSUPPORTED, "head_dim %d / block %d not in {64, 128}", head_dim, block);
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if (schedule != WA_SCHED_NATURAL && schedule != WA_SCHED_XCD_SLICED &&
      schedule != WA_SCHED_HEADS_INTERLEAVED && schedule != WA_SCHED_AUTO &&
      schedule != WA_SCHED_DEFAULT)
    return fail(WA_ERR_INVALID_ARG, "unknown schedule %d", schedule);
  if (!(scale > 0.0f) || !(scale < 1e30f)) return fail(WA_ERR_INVALID_ARG, "scale must be > 0");
  const int64_t MB = ((int64_t)L + block - 1) / block;
  if ((int64_t)H * MB * block * head_dim >= ((int64_t)1 << 40))
    return fail(WA_ERR_UNSUPPORTED, "tensor too large");
  if ((int64_t)H * MB * 8 >= ((int64_t)1 << 31))
    return fail(WA_ERR_UNSUPPORTED, "too many query blocks");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if (al % 16 != 0) return fail(WA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  const size_t need = wa::attn_workspace_bytes(H, (int)(MB * block), head_dim);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(WA_ERR_CAPACITY, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (perm_slices < 0 || perm_slices > 64)
    return fail(WA_ERR_INVALID_ARG, "perm_slices must be in 0..64");
  int n_xcd = 1;
  const hipError_t e = stream_xcds(static_cast<hipStream_t>(stream), &n_xcd);
  if (e != hipSuccess) return hip_status(e, "device of the stream");
  // The XCD-sliced schedule runs slice x of each head's order on XCD x, so a
  // permutation whose wave buckets were cut into another number of slices would
  // put its buckets across L2 domains.
  if (perm != nullptr && (schedule == WA_SCHED_XCD_SLICED || schedule == WA_SCHED_AUTO) &&
      perm_slices != n_xcd)
    return fail(WA_ERR_INVALID_ARG,
                "perm was built for %d slices but the XCD-sliced schedule runs %d (the device's "
                "XCD count)", perm_slices, n_xcd);
  *n_xcd_out = n_xcd;
  return WA_OK;
}

static int sparse_attn_common(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                              int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                              const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                              int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o,
                              float* lse, float* g, float* entropy, float* distance,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const char* name) {
  int n_xcd = 1;
  const int rc = sparse_attn_check(q, k, v, H, L, head_dim, block, row_ptr, col_idx, capacity,
                                   perm, perm_slices, schedule, scale, o, lse, workspace,
                                   workspace_bytes, stream, &n_xcd);
  if (rc != WA_OK) return rc;
  return hip_status(wa::launch_sparse_attn(q, k, v, H, L, head_dim, block, row_ptr, col_idx,
                                           capacity, perm, schedule, n_xcd, scale, o, lse, g,
                                           entropy, distance, workspace,
                                           static_cast<hipStream_t>(stream)),
                    name);
}

int wa_sparse_attn_fwd_noalloc(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                               int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                               const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                               int32_t perm_slices, int32_t schedule, const uint8_t* skipped,
                               float scale, wa_bf16* o, float* lse, float* g, void* stream) {
  if (schedule == WA_SCHED_AUTO && !skipped)
    return fail(WA_ERR_INVALID_ARG, "WA_SCHED_AUTO needs the skip flags");
  if (H < 1 || L < 1) return fail(WA_ERR_INVALID_ARG, "H and L must be >= 1");
  if (!supported_shape(head_dim, block))
    return fail(WA_ERR_UNSUPPORTED, "head_dim %d / block %d not in {64, 128}", head_dim, block);
  const int64_t MB = ((int64_t)L + block - 1) / block;
  if ((int64_t)H * MB * 8 >= ((int64_t)1 << 31))
    return fail(WA_ERR_UNSUPPORTED, "too many query blocks");
  const size_t need = wa::attn_workspace_bytes(H, (int)(MB * block), head_dim);
  if (need > wa::kStaticScratchBytes)
    return fail(WA_ERR_CAPACITY, "these sizes need %zu bytes of scratch; the static scratch "
                "holds %zu", need, wa::kStaticScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "device of the stream");
  void* scratch = nullptr;
  e = wa::static_scratch(dev, &scratch);
  if (e != hipSuccess) return hip_status(e, "static scratch address");
  int n_xcd = 1;
  const int rc = sparse_attn_check(q, k, v, H, L, head_dim, block, row_ptr, col_idx, capacity,
                                   perm, perm_slices, schedule, scale, o, lse, scratch,
                                   wa::kStaticScratchBytes, stream, &n_xcd);
  if (rc != WA_OK) return rc;
  if (schedule == WA_SCHED_AUTO) {
    // The schedule word is written whole by the selection kernel, so nothing has to
    // be cleared first.
    e = wa::launch_sched_select(skipped, H, scratch, s);
    if (e != hipSuccess) return hip_status(e, "wa_sparse_attn_fwd_noalloc (schedule)");
  }
  return hip_status(wa::launch_sparse_attn(q, k, v, H, L, head_dim, block, row_ptr, col_idx,
                                           capacity, perm, schedule, n_xcd, scale, o, lse, g,
                                           nullptr, nullptr, scratch, s),
                    "wa_sparse_attn_fwd_noalloc");
}

int wa_xcd_placement(int32_t n_wg, int32_t block, int32_t* xcd_out, void* stream) {
  if (!xcd_out) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (n_wg < 1) return fail(WA_ERR_INVALID_ARG, "n_wg must be >= 1");
  if (block != 64 && block != 128) return fail(WA_ERR_UNSUPPORTED, "block %d not in {64, 128}", block);
  return hip_status(wa::launch_xcd_placement(n_wg, block, xcd_out, static_cast<hipStream_t>(stream)),
                    "wa_xcd_placement");
}

int wa_default_schedule(int32_t L, int32_t head_dim, int32_t block, int32_t* schedule) {
  if (!schedule) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (L < 1) return fail(WA_ERR_INVALID_ARG, "L must be >= 1");
  if (!supported_shape(head_dim, block))
    return fail(WA_ERR_UNSUPPORTED, "head_dim %d / block %d not in {64, 128}", head_dim, block);
  *schedule = wa::default_schedule((int)(((int64_t)L + block - 1) / block), block, head_dim);
  return ok();
}

int wa_attn_schedule_select(const uint8_t* skipped, int32_t H, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!skipped || !workspace) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1) return fail(WA_ERR_INVALID_ARG, "H must be >= 1");
  const size_t need = wa::attn_workspace_bytes(H, 0, 0);
  if (workspace_bytes < need)
    return fail(WA_ERR_CAPACITY, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  return hip_status(wa::launch_sched_select(skipped, H, workspace, static_cast<hipStream_t>(stream)),
                    "wa_attn_schedule_select");
}

int wa_sparse_attn_fwd(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                       int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                       int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o, float* lse,
                       float* g, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_common(q, k, v, H, L, head_dim, block, row_ptr, col_idx, capacity, perm,
                            perm_slices, schedule, scale, o, lse, g, nullptr, nullptr, workspace,
                            workspace_bytes, stream, "wa_sparse_attn_fwd");
}

int wa_sparse_attn_fwd_diag(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                            int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                            const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                            int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o,
                            float* lse, float* g, float* entropy, float* distance,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!entropy && !distance)
    return fail(WA_ERR_INVALID_ARG, "entropy and distance are both null");
  return sparse_attn_common(q, k, v, H, L, head_dim, block, row_ptr, col_idx, capacity, perm,
                            perm_slices, schedule, scale, o, lse, g, entropy, distance, workspace,
                            workspace_bytes, stream, "wa_sparse_attn_fwd_diag");
}

int wa_block_importance(const float* g, const float* lse, const int32_t* row_ptr,
                        int64_t capacity, int32_t H, int32_t MB, int32_t L, int32_t block,
                        float* w, void* stream) {
  if (!g || !lse || !row_ptr || !w) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || L < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, L must be >= 1");
  if (block != 64 && block != 128) return fail(WA_ERR_UNSUPPORTED, "block %d not in {64, 128}", block);
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if ((int64_t)MB * block < L || (int64_t)(MB - 1) * block >= L)
    return fail(WA_ERR_INVALID_ARG, "MB must equal ceil(L / block)");
  return hip_status(wa::launch_block_importance(g, lse, row_ptr, capacity, H, MB, L, block, w,
                                                static_cast<hipStream_t>(stream)),
                    "wa_block_importance");
}

int wa_topp_select(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                   int64_t capacity, int32_t H, int32_t MB, int32_t NB, double p,
                   uint8_t* mask_out, void* stream) {
  if (!w || !row_ptr || !col_idx || !mask_out) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if (NB > WA_MAX_BLOCKS) return fail(WA_ERR_UNSUPPORTED, "NB must be <= %d", WA_MAX_BLOCKS);
  if (!(p > 0.0 && p <= 1.0)) return fail(WA_ERR_INVALID_ARG, "p must be in (0, 1]");
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  return hip_status(wa::launch_topp(w, row_ptr, col_idx, capacity, H, MB, NB, p, mask_out,
                                    static_cast<hipStream_t>(stream)),
                    "wa_topp_select");
}

int wa_mask_recall(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                   int64_t capacity, int32_t H, int32_t MB, int32_t NB, const uint8_t* mask,
                   float* recall_out, void* stream) {
  if (!w || !row_ptr || !col_idx || !mask || !recall_out)
    return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || NB < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, NB must be >= 1");
  if (NB > WA_MAX_BLOCKS) return fail(WA_ERR_UNSUPPORTED, "NB must be <= %d", WA_MAX_BLOCKS);
  if (capacity < 0) return fail(WA_ERR_INVALID_ARG, "negative capacity");
  if ((int64_t)H * MB >= ((int64_t)1 << 31)) return fail(WA_ERR_UNSUPPORTED, "too many rows");
  return hip_status(wa::launch_mask_recall(w, row_ptr, col_idx, capacity, H, MB, NB, mask,
                                           recall_out, static_cast<hipStream_t>(stream)),
                    "wa_mask_recall");
}

static int permute_common(const void* src, void* dst, const int32_t* perm, int32_t H, int32_t MB,
                          int64_t block_bytes, bool scatter, void* stream) {
  if (!src || !dst || !perm) return fail(WA_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1 || MB < 1 || block_bytes < 1) return fail(WA_ERR_INVALID_ARG, "H, MB, block_bytes must be >= 1");
  if ((int64_t)H * MB >= ((int64_t)1 << 31)) return fail(WA_ERR_UNSUPPORTED, "too many blocks");
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  const int64_t total = (int64_t)H * MB * block_bytes;
  if (s < d + total && d < s + total) return fail(WA_ERR_INVALID_ARG, "src and dst overlap");
  return hip_status(wa::launch_permute_blocks(src, dst, perm, H, MB, block_bytes, scatter,
                                              static_cast<hipStream_t>(stream)),
                    scatter ? "wa_scatter_blocks" : "wa_gather_blocks");
}

int wa_gather_blocks(const void* src, void* dst, const int32_t* perm, int32_t H, int32_t MB,
                     int64_t block_bytes, void* stream) {
  return permute_common(src, dst, perm, H, MB, block_bytes, false, stream);
}

int wa_scatter_blocks(const void* src, void* dst, const int32_t* perm, int32_t H, int32_t MB,
                      int64_t block_bytes, void* stream) {
  return permute_common(src, dst, perm, H, MB, block_bytes, true, stream);
}

}  // extern "C"
