// Explicit block permutation (WaveAlign §V: gather query blocks and mask rows
// into the execution order before the kernel, put output rows back after it).
// One workgroup per (head, position); the copy width is the widest of 16, 4 or 1
// bytes that divides the block size and both base addresses.
#include "wa_internal.h"

namespace wa {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_permute(const T* __restrict__ src, T* __restrict__ dst,
                                                 const int32_t* __restrict__ perm, int MB,
                                                 int64_t elems, int scatter) {
  const int h = blockIdx.x / MB;
  const int s = blockIdx.x % MB;
  const int p = perm[(size_t)h * MB + s];
  if (p < 0 || p >= MB) return;  // out-of-range entries are ignored
  const size_t from = ((size_t)h * MB + (scatter ? s : p)) * elems;
  const size_t to = ((size_t)h * MB + (scatter ? p : s)) * elems;
  for (int64_t i = threadIdx.x; i < elems; i += 256) dst[to + i] = src[from + i];
}

}  // namespace

hipError_t launch_permute_blocks(const void* src, void* dst, const int32_t* perm, int H, int MB,
                                 int64_t block_bytes, bool scatter, hipStream_t s) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  const dim3 grid(H * MB), blk(256);
  if (block_bytes % 16 == 0 && a % 16 == 0) {
    hipLaunchKernelGGL(k_permute<uint4>, grid, blk, 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), perm, MB, block_bytes / 16, scatter ? 1 : 0);
  } else if (block_bytes % 4 == 0 && a % 4 == 0) {
    hipLaunchKernelGGL(k_permute<uint32_t>, grid, blk, 0, s, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), perm, MB, block_bytes / 4, scatter ? 1 : 0);
  } else {
    hipLaunchKernelGGL(k_permute<uint8_t>, grid, blk, 0, s, static_cast<const uint8_t*>(src),
                       static_cast<uint8_t*>(dst), perm, MB, block_bytes, scatter ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace wa
