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

// One workgroup per query-block row u.  Eight consecutive threads share one CSR
// entry and each sums a fixed slice of BLOCK/8 rows of it, so a wavefront reads
// eight whole G rows (8 x BLOCK floats, contiguous in memory) with 16-byte loads;
// the eight partial sums are combined by a fixed shuffle tree, so W is bitwise
// reproducible.  exp(G - L) is evaluated as exp2((G - L) log2 e).
template <int BLOCK>
__global__ __launch_bounds__(256) void k_block_importance(const float* __restrict__ G,
                                                          const float* __restrict__ lse,
                                                          const int32_t* __restrict__ row_ptr,
                                                          int cap, int MB, int L,
                                                          float* __restrict__ W) {
  constexpr int kParts = 8;                // threads per CSR entry
  constexpr int kRows = BLOCK / kParts;    // rows per thread
  constexpr int kPerPass = 256 / kParts;   // entries per pass of the workgroup
  constexpr float kLog2e = 1.4426950408889634f;
  const int row = blockIdx.x;  // h * MB + u
  const int h = row / MB, u = row % MB;
  const int part = threadIdx.x % kParts, slot = threadIdx.x / kParts;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  const int nvalid = min(BLOCK, L - u * BLOCK);
  const size_t lp = (size_t)MB * BLOCK;
  float lsc[kRows];
  bool live[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int r = part * kRows + k;
    const float x = r < nvalid ? lse[(size_t)h * lp + (size_t)u * BLOCK + r] : -INFINITY;
    live[k] = r < nvalid && x != -INFINITY;
    lsc[k] = live[k] ? x * kLog2e : 0.0f;
  }
  const float inv_b = 1.0f / (float)nvalid;
  for (int e = e0 + slot; e < e1; e += kPerPass) {
    const float4* gp = reinterpret_cast<const float4*>(G + (size_t)e * BLOCK + part * kRows);
    float s = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < kRows / 4; ++k4) {
      const float4 v = gp[k4];
      const float gv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * k4 + j;
        if (live[k]) s += __builtin_amdgcn_exp2f(fmaf(gv[j], kLog2e, -lsc[k]));
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (part == 0) W[e] = s * inv_b;
  }
}

// One wavefront per query-block row: sort the candidates by (W descending, block
// id ascending) with a bitonic sort of 64-bit keys in LDS (n2 = the candidate count
// rounded up to a power of two), then walk them in that order with a wave-uniform
// fp64 running total (the order of the additions fixes the rounding of the total,
// and the kept set depends on it) and keep blocks while the total before them is
// at most p.
__global__ __launch_bounds__(64) void k_topp(const float* __restrict__ W,
                                             const int32_t* __restrict__ row_ptr,
                                             const int32_t* __restrict__ col_idx, int cap,
                                             int NB, double p, uint8_t* __restrict__ mask_out) {
  extern __shared__ uint64_t key[];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  int n2max = 1;  // LDS keys allocated by the launcher
  while (n2max < NB) n2max <<= 1;
  const int n = max(0, min(e1 - e0, n2max));  // a well-formed row has at most NB entries
  uint8_t* out = mask_out + (size_t)row * NB;
  for (int v = lane; v < NB; v += 64) out[v] = 0;
  if (n <= 0) return;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = lane; i < n2; i += 64) {
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
      for (int i = lane; i < (n2 >> 1); i += 64) {
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
  double acc = 0.0;
  for (int c = 0; c < n && !(acc > p); c += 64) {
    const uint64_t mine = c + lane < n ? key[c + lane] : ~0ull;
    const uint32_t klo = (uint32_t)mine, khi = (uint32_t)(mine >> 32);
    const int m = min(64, n - c);
    for (int j = 0; j < m; ++j) {
      if (acc > p) break;
      const uint32_t wv = 0x7FFFFFFFu - __builtin_amdgcn_readlane(khi, j);
      const int v = (int)__builtin_amdgcn_readlane(klo, j);
      if (lane == 0 && v >= 0 && v < NB) out[v] = 1;
      acc += (double)__uint_as_float(wv);
    }
  }
}

// Attention recall of a mask per query block: one wavefront per CSR row; lanes
// walk the row's entries 64 apart and add the weight of every entry whose block
// the mask keeps (in fp64), and a fixed shuffle tree adds the lanes.
__global__ __launch_bounds__(256) void k_mask_recall(const float* __restrict__ W,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col_idx, int cap,
                                                     int rows, int NB,
                                                     const uint8_t* __restrict__ mask,
                                                     float* __restrict__ out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int lo = min(row_ptr[r], cap), hi = min(row_ptr[r + 1], cap);
  const uint8_t* m = mask + (size_t)r * NB;
  double acc = 0.0;
  for (int k = lo + lane; k < hi; k += 64) {
    const int v = col_idx[k];
    if ((unsigned)v < (unsigned)NB && m[v] != 0) acc += (double)W[k];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) out[r] = (float)acc;
}

}  // namespace

hipError_t launch_mask_recall(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t cap64, int H, int MB, int NB, const uint8_t* mask,
                              float* out, hipStream_t s) {
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  const int rows = H * MB;
  hipLaunchKernelGGL(k_mask_recall, dim3((rows + 3) / 4), dim3(256), 0, s, w, row_ptr, col_idx,
                     cap, rows, NB, mask, out);
  return hipGetLastError();
}

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
  int n2 = 1;
  while (n2 < NB) n2 <<= 1;  // a row has at most NB candidates
  hipLaunchKernelGGL(k_topp, dim3(H * MB), dim3(64), (size_t)n2 * sizeof(uint64_t), s, w,
                     row_ptr, col_idx, cap, NB, p, mask_out);
  return hipGetLastError();
}

}  // namespace wa
