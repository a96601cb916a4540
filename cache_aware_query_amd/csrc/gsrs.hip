// GSRS block importance (Phase 2) and Top-p block selection.
//
// "Sparse Attention for Video Generation Acceleration via Growing Sparsity and
// Reduced Search": §5.3 and Appendix A.2 define the block weight of query block u
// on evaluated key block v as the attention weight of u's rows on v's keys,
// normalised over the evaluated keys and averaged over u's rows; with the Phase-1
// block log-sum-exp G and the row LSE this is (1/B_u) sum_i exp(G_iv - LSE_i).
// Algorithm 3 keeps a row's blocks in descending weight until the cumulative
// weight exceeds p.
#include "wa_internal.h"

namespace wa {
namespace {

// One workgroup (4 wavefronts) per query-block row; each wavefront takes CSR
// entries in turn, each lane two rows of the block, and reduces with a fixed
// shuffle tree, so W is bitwise reproducible.
template <int BLOCK>
__global__ __launch_bounds__(256) void k_block_importance(const float* __restrict__ G,
                                                          const float* __restrict__ lse,
                                                          const int32_t* __restrict__ row_ptr,
                                                          int cap, int MB, int L,
                                                          float* __restrict__ W) {
  constexpr int kPer = BLOCK / 64;
  const int row = blockIdx.x;  // h * MB + u
  const int h = row / MB, u = row % MB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  const int nvalid = min(BLOCK, L - u * BLOCK);
  const size_t lp = (size_t)MB * BLOCK;
  float l[kPer];
  bool live[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int r = lane + 64 * j;
    const float x = r < nvalid ? lse[(size_t)h * lp + (size_t)u * BLOCK + r] : -INFINITY;
    live[j] = r < nvalid && x != -INFINITY;
    l[j] = x;
  }
  const float inv_b = 1.0f / (float)nvalid;
  for (int e = e0 + wave; e < e1; e += 4) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = lane + 64 * j;
      if (live[j]) s += expf(G[(size_t)e * BLOCK + r] - l[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) W[e] = s * inv_b;
  }
}

// One workgroup per query-block row: sort the candidates by (W descending, block
// id ascending) with a bitonic sort of 64-bit keys in LDS, then accumulate in fp64
// in that order on one lane (the order of the additions fixes the rounding of the
// running total, and the kept set depends on it).
__global__ __launch_bounds__(256) void k_topp(const float* __restrict__ W,
                                              const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col_idx, int cap,
                                              int NB, double p, uint8_t* __restrict__ mask_out) {
  __shared__ uint64_t key[WA_MAX_BLOCKS];
  const int row = blockIdx.x;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  const int n = min(e1 - e0, WA_MAX_BLOCKS);
  uint8_t* out = mask_out + (size_t)row * NB;
  for (int v = threadIdx.x; v < NB; v += 256) out[v] = 0;
  if (n <= 0) return;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256) {
    if (i < n) {
      float w = W[e0 + i];
      if (!(w >= 0.0f)) w = 0.0f;  // NaN or negative weights rank last
      const uint32_t wb = __float_as_uint(w);
      key[i] = ((uint64_t)(0x7FFFFFFFu - wb) << 32) | (uint32_t)col_idx[e0 + i];
    } else {
      key[i] = ~0ull;
    }
  }
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < (n2 >> 1); i += 256) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) {
      if (acc > p) break;
      const uint64_t k = key[i];
      const int v = (int)(uint32_t)(k & 0xFFFFFFFFu);
      const float w = __uint_as_float(0x7FFFFFFFu - (uint32_t)(k >> 32));
      if (v >= 0 && v < NB) out[v] = 1;
      acc += (double)w;
    }
  }
}

}  // namespace

hipError_t launch_block_importance(const float* g, const float* lse, const int32_t* row_ptr,
                                   int64_t cap64, int H, int MB, int L, int block, float* w,
                                   hipStream_t s) {
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  if (block == 128)
    hipLaunchKernelGGL(k_block_importance<128>, dim3(H * MB), dim3(256), 0, s, g, lse, row_ptr,
                       cap, MB, L, w);
  else
    hipLaunchKernelGGL(k_block_importance<64>, dim3(H * MB), dim3(256), 0, s, g, lse, row_ptr,
                       cap, MB, L, w);
  return hipGetLastError();
}

hipError_t launch_topp(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t cap64, int H, int MB, int NB, double p, uint8_t* mask_out,
                       hipStream_t s) {
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  hipLaunchKernelGGL(k_topp, dim3(H * MB), dim3(256), 0, s, w, row_ptr, col_idx, cap, NB, p,
                     mask_out);
  return hipGetLastError();
}

}  // namespace wa
