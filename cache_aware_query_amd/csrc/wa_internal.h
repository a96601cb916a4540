// Internal declarations shared by the HIP translation units of libwavealign.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wavealign.h"

namespace wa {

// Launchers (defined next to their kernels).  They assume validated arguments and
// return the hipError_t of the launch.
hipError_t launch_block_index(const uint8_t* mask, int H, int MB, int NB, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_cap, int32_t* row_nnz,
                              int32_t* csc_ptr, int32_t* csc_idx, int64_t csc_cap,
                              hipStream_t s);

hipError_t launch_reorder(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* csc_ptr,
                          const int32_t* csc_idx, int64_t cap, const float* x0, int H, int MB, int NB,
                          int block, int head_dim, const wa_reorder_params& p, int32_t* perm,
                          int32_t* inv_perm, uint8_t* skipped, double* angles, double* stats,
                          hipStream_t s);
hipError_t launch_minhash_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap,
                                int H, int MB, int NB, const uint32_t* hash_a,
                                const uint32_t* hash_b, int n_hash, int wave, int n_slices,
                                int stage2, int32_t* perm, int32_t* inv_perm, hipStream_t s);

// Hash coefficients of the LSH comparator: two MinHash functions per band.
constexpr int kLshMaxBands = 4;
struct LshHashes {
  uint32_t a[2 * kLshMaxBands], b[2 * kLshMaxBands];
};
hipError_t launch_lsh_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap, int H,
                            int MB, int NB, const uint32_t* hash_a, const uint32_t* hash_b,
                            int n_bands, int wave, int n_slices, int stage2, int32_t* perm,
                            int32_t* inv_perm, hipStream_t s);
size_t lsh_lds_bytes(int MB, int n_bands);

// True if the reorder of an MB x NB mask cannot hold the mask as bitmasks in LDS
// and must read the transposed lists (CSC) instead.
bool reorder_needs_csc(int MB, int NB);

size_t attn_workspace_bytes(int H, int L_pad, int head_dim);
hipError_t launch_sched_select(const uint8_t* skipped, int H, void* workspace, hipStream_t s);
hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H,
                              int L, int head_dim, int block, const int32_t* row_ptr,
                              const int32_t* col_idx, int64_t cap, const int32_t* perm,
                              int schedule, int n_xcd, float scale, uint16_t* o, float* lse,
                              float* g, float* ent, float* dist, void* workspace, hipStream_t s);
hipError_t launch_xcd_placement(int n_wg, int block, int32_t* out, hipStream_t s);

// The static device scratch of wa_sparse_attn_fwd_noalloc: its size, and the device
// address of device `dev`'s copy (looked up once per device).
// The schedule WA_SCHED_DEFAULT resolves to for heads that keep their original order.
__host__ __device__ inline int default_schedule(int MB, int block, int head_dim) {
  return (unsigned long long)MB * block * head_dim * 4 <= WA_ALL_HEADS_MAX_KV_BYTES
             ? WA_SCHED_HEADS_INTERLEAVED
             : WA_SCHED_XCD_SLICED;
}

constexpr size_t kStaticScratchBytes = 256;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(int dev, void** out);
int attn_resident_wgs_per_cu(int head_dim, int block);

hipError_t launch_block_importance(const float* g, const float* lse, const int32_t* row_ptr,
                                   int64_t cap, int H, int MB, int L, int block, float* w, hipStream_t s);
hipError_t launch_mask_recall(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t cap, int H, int MB, int NB, const uint8_t* mask, float* out,
                              hipStream_t s);
hipError_t launch_topp(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t cap, int H,
                       int MB, int NB, double p, uint8_t* mask_out, hipStream_t s);

hipError_t launch_permute_blocks(const void* src, void* dst, const int32_t* perm, int H, int MB,
                                 int64_t block_bytes, bool scatter, hipStream_t s);


}  // namespace wa
