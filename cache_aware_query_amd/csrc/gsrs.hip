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

// Four consecutive query-block rows per workgroup, their CSR entries taken as one
// run: eight consecutive threads share an entry and 32 entries are in flight per
// pass, however the entries fall into the four rows, so long and short rows both
// keep the workgroup busy.  Thread p of the eight takes the rows 32*j + 4*p + i
// (i < 4) of its entry, so that each 16-byte load of the eight covers 128 contiguous
// bytes of the entry's G row and of its query block's LSEs (the same LSEs for every
// entry of a row, so they come from the cache).  Each thread sums its BLOCK/8 terms
// in a fixed order and a fixed shuffle tree adds the eight partial sums, so W is
// bitwise reproducible.  exp(G - L) is evaluated as exp2((G - L) log2 e).  UNROLL
// passes have their loads issued together: two when rows are long (more bytes in
// flight), one when they are short (fewer registers, more workgroups resident);
// the arithmetic of an entry, and so W, is the same either way.
template <int BLOCK, int UNROLL>
__global__ __launch_bounds__(256) void k_block_importance(const float* __restrict__ G,
                                                          const float* __restrict__ lse,
                                                          const int32_t* __restrict__ row_ptr,
                                                          int cap, int rows, int MB, int L,
                                                          float* __restrict__ W) {
  constexpr int kParts = 8;                // threads per CSR entry
  constexpr int kVec = BLOCK / 32;         // 16-byte loads per thread, entry and array
  constexpr int kPerPass = 256 / kParts;   // entries per pass of the workgroup
  constexpr int kUnroll = UNROLL;
  constexpr float kLog2e = 1.4426950408889634f;
  const int r0 = blockIdx.x * 4;  // rows r0 .. r0+3 (h * MB + u)
  const int part = threadIdx.x % kParts, slot = threadIdx.x / kParts;
  // entries of row r0 + k: [eb[k], eb[k + 1])
  int eb[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) eb[k] = min(row_ptr[min(r0 + k, rows)], cap);
  const size_t lp = (size_t)MB * BLOCK;
  for (int e = eb[0] + slot; e < eb[4]; e += kUnroll * kPerPass) {
    float4 gv[kUnroll][kVec], lv[kUnroll][kVec];
    int nvalid[kUnroll];
#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
      const int ex = e + x * kPerPass;
      const int k = (ex >= eb[1]) + (ex >= eb[2]) + (ex >= eb[3]);
      const int row = min(r0 + k, rows - 1);  // past the run: a valid row, not read
      const int h = row / MB, u = row - h * MB;
      nvalid[x] = min(BLOCK, L - u * BLOCK);
      const float* gp = G + (size_t)ex * BLOCK + 4 * part;
      const float* lr = lse + (size_t)h * lp + (size_t)u * BLOCK + 4 * part;
      const bool in = ex < eb[4];
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        gv[x][j] = in ? *reinterpret_cast<const float4*>(gp + 32 * j)
                      : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        // rows at or past L (padding, inside [0, L_pad)) are read but not used
        lv[x][j] = in ? *reinterpret_cast<const float4*>(lr + 32 * j)
                      : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
      const int ex = e + x * kPerPass;
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const float g4[4] = {gv[x][j].x, gv[x][j].y, gv[x][j].z, gv[x][j].w};
        const float l4[4] = {lv[x][j].x, lv[x][j].y, lv[x][j].z, lv[x][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool live = 32 * j + 4 * part + i < nvalid[x] && l4[i] != -INFINITY;
          if (live) s += __builtin_amdgcn_exp2f(fmaf(g4[i], kLog2e, -(l4[i] * kLog2e)));
        }
      }
      // the eight threads of a group share ex, so they shuffle together even past the
      // end of the run
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (part == 0 && ex < eb[4]) W[ex] = s * (1.0f / (float)nvalid[x]);
    }
  }
}

// Top-p key of a candidate: (W descending, block id ascending) as one unsigned
// 64-bit key, so that ascending key order is the selection order.  NaN and
// negative weights rank as zero; a real key is below 2^63, the padding key ~0.
__device__ inline uint64_t topp_key(float w, int32_t v) {
  if (!(w > 0.0f)) w = 0.0f;
  return ((uint64_t)(0x7FFFFFFFu - __float_as_uint(w)) << 32) | (uint32_t)v;
}

__device__ inline float topp_weight(uint64_t key) {
  return __uint_as_float(0x7FFFFFFFu - (uint32_t)(key >> 32));
}

// Rows up to kToppRegMax candidates are sorted in registers; longer rows (possible
// only when NB > kToppRegMax) take the LDS kernel below.
constexpr int kToppRegMax = 1024;

__device__ inline uint64_t shfl_xor_u64(uint64_t x, int m) {
  const int lo = __shfl_xor((int)(uint32_t)x, m), hi = __shfl_xor((int)(uint32_t)(x >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// One chunk of the walk: lane j holds the weight of the chunk's element j (m
// elements, zero beyond).  Adds them in lane order to the wave-uniform running
// total acc and returns false when every element is kept (acc then includes them
// all); otherwise returns true with j_kept = the elements kept before the first
// whose preceding total exceeds p (the cut; acc is then no longer needed).  A whole
// chunk is kept when the total before its last element is at most p, since a total
// of non-negative terms never decreases; only the chunk holding the cut, and a
// partial last chunk, are walked element by element.
__device__ __forceinline__ bool walk_chunk(double wd, int m, double p, double& acc, int& j_kept) {
  const int lo = __double2loint(wd), hi = __double2hiint(wd);
  auto lane_w = [&](int j) {
    return __hiloint2double(__builtin_amdgcn_readlane(hi, j), __builtin_amdgcn_readlane(lo, j));
  };
  if (m == 64) {
    double a = acc;
#pragma unroll 3
    for (int j = 0; j < 63; ++j) a += lane_w(j);
    const bool whole = !(a > p);
    a += lane_w(63);
    if (whole) {
      acc = a;
      return false;
    }
  }
  int j = 0;
  double a = acc;
  for (; j < m && !(a > p); ++j) a += lane_w(j);
  acc = a;
  j_kept = j;
  return j < m;
}

// Cross-lane stages of the register bitonic sort for one `size`: pairs `stride`
// lanes apart in the same register, stride = first, first/2, .., 1 (first <= 32).
// The direction of a pair follows bit `size` of its element index 64*r + lane,
// which comes from the lane when size < 64 and from r otherwise.
template <int R>
__device__ __forceinline__ void bitonic_across_lanes(uint64_t (&k)[R], int lane, int size,
                                                     int first) {
  const bool lane_asc = (lane & size) == 0;
#pragma unroll 1
  for (int stride = first; stride > 0; stride >>= 1) {
    const bool lower = (lane & stride) == 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool asc = lane_asc && ((64 * r) & size) == 0;
      const uint64_t o = shfl_xor_u64(k[r], stride);
      // the lower element of an ascending pair keeps the smaller key
      const bool take_other = (k[r] < o) != (lower == asc);
      k[r] = take_other ? o : k[r];
    }
  }
}

// Bitonic sort, ascending, of the 64*R keys held as element i = 64*r + lane in
// register r of each lane: pairs 64 or more elements apart (rs = stride/64
// registers) exchange within a lane, closer pairs across lanes.
template <int R>
__device__ __forceinline__ void bitonic_sort_reg(uint64_t (&k)[R], int lane) {
#pragma unroll 1
  for (int size = 2; size <= 64; size <<= 1) bitonic_across_lanes<R>(k, lane, size, size >> 1);
#pragma unroll
  for (int size = 128; size <= 64 * R; size <<= 1) {
#pragma unroll
    for (int rs = size / 128; rs >= 1; rs >>= 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r & rs) continue;
        const bool asc = ((64 * r) & size) == 0;
        const uint64_t a = k[r], b = k[r | rs];
        const bool sw = (b < a) == asc;  // equal keys may swap: nothing changes
        k[r] = sw ? b : a;
        k[r | rs] = sw ? a : b;
      }
    }
    bitonic_across_lanes<R>(k, lane, size, 32);
  }
}

// One row of n <= 64*R candidates on one wavefront: the keys are sorted in
// registers, then walked in sorted order chunk by chunk (chunk r is register r).
template <int R>
__device__ __forceinline__ void topp_row_reg(const float* __restrict__ W,
                                             const int32_t* __restrict__ col_idx, int e0, int n,
                                             int NB, double p, uint8_t* flags, int lane) {
  uint64_t k[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = 64 * r + lane;
    k[r] = i < n ? topp_key(W[e0 + i], col_idx[e0 + i]) : ~0ull;
  }
  bitonic_sort_reg<R>(k, lane);
  double acc = 0.0;
  int kept = n;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (64 * r >= n) break;
    const int m = min(64, n - 64 * r);
    const double wd = 64 * r + lane < n ? (double)topp_weight(k[r]) : 0.0;
    int j;
    if (walk_chunk(wd, m, p, acc, j)) {
      kept = 64 * r + j;
      break;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int v = (int)(uint32_t)k[r];
    if (64 * r + lane < kept && v >= 0 && v < NB) flags[v] = 1;
  }
}

// One wavefront per query-block row with at most kToppRegMax candidates (rows with
// more are left to k_topp_lds): the row's NB mask bytes are built in LDS and
// written once.
__global__ __launch_bounds__(64) void k_topp_reg(const float* __restrict__ W,
                                                 const int32_t* __restrict__ row_ptr,
                                                 const int32_t* __restrict__ col_idx, int cap,
                                                 int NB, double p, uint8_t* __restrict__ mask_out) {
  extern __shared__ uint8_t flags[];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  int n2max = 1;
  while (n2max < NB) n2max <<= 1;
  const int n = max(0, min(e1 - e0, n2max));  // a well-formed row has at most NB entries
  if (n > kToppRegMax) return;
  for (int v = lane; v < NB; v += 64) flags[v] = 0;
  __syncthreads();
  if (n > 512) topp_row_reg<16>(W, col_idx, e0, n, NB, p, flags, lane);
  else if (n > 256) topp_row_reg<8>(W, col_idx, e0, n, NB, p, flags, lane);
  else if (n > 128) topp_row_reg<4>(W, col_idx, e0, n, NB, p, flags, lane);
  else if (n > 64) topp_row_reg<2>(W, col_idx, e0, n, NB, p, flags, lane);
  else if (n > 0) topp_row_reg<1>(W, col_idx, e0, n, NB, p, flags, lane);
  __syncthreads();
  uint8_t* out = mask_out + (size_t)row * NB;
  for (int v = lane; v < NB; v += 64) out[v] = flags[v];
}

// Rows with more than kToppRegMax candidates: a bitonic sort of the 64-bit keys in
// LDS (n2 = the candidate count rounded up to a power of two), then the same walk
// one element at a time.
__global__ __launch_bounds__(64) void k_topp_lds(const float* __restrict__ W,
                                                 const int32_t* __restrict__ row_ptr,
                                                 const int32_t* __restrict__ col_idx, int cap,
                                                 int NB, double p, uint8_t* __restrict__ mask_out) {
  extern __shared__ uint64_t key[];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int e0 = min(row_ptr[row], cap), e1 = min(row_ptr[row + 1], cap);
  int n2max = 1;  // LDS keys allocated by the launcher
  while (n2max < NB) n2max <<= 1;
  const int n = max(0, min(e1 - e0, n2max));
  if (n <= kToppRegMax) return;  // k_topp_reg's row
  uint8_t* out = mask_out + (size_t)row * NB;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = lane; i < n2; i += 64) key[i] = i < n ? topp_key(W[e0 + i], col_idx[e0 + i]) : ~0ull;
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
  int kept = n;
  for (int c = 0; c < n; c += 64) {
    const int m = min(64, n - c);
    const double wd = c + lane < n ? (double)topp_weight(key[c + lane]) : 0.0;
    int j;
    if (walk_chunk(wd, m, p, acc, j)) {
      kept = c + j;
      break;
    }
  }
  uint8_t* flags = reinterpret_cast<uint8_t*>(key + n2max);
  for (int v = lane; v < NB; v += 64) flags[v] = 0;
  __syncthreads();
  for (int i = lane; i < kept; i += 64) {
    const int v = (int)(uint32_t)key[i];
    if (v >= 0 && v < NB) flags[v] = 1;
  }
  __syncthreads();
  for (int v = lane; v < NB; v += 64) out[v] = flags[v];
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
  const int rows = H * MB;
  const dim3 grid((rows + 3) / 4);
  // The capacity bounds the entries: at 16 or more per row the rows are long.
  const bool long_rows = cap >= 16LL * rows;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, g, lse, row_ptr, cap, rows, MB, L, w);
  };
  if (block == 128) {
    if (long_rows) launch(k_block_importance<128, 2>);
    else launch(k_block_importance<128, 1>);
  } else {
    if (long_rows) launch(k_block_importance<64, 2>);
    else launch(k_block_importance<64, 1>);
  }
  return hipGetLastError();
}

hipError_t launch_topp(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t cap64, int H, int MB, int NB, double p, uint8_t* mask_out,
                       hipStream_t s) {
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  int n2 = 1;
  while (n2 < NB) n2 <<= 1;  // a row has at most NB candidates
  hipLaunchKernelGGL(k_topp_reg, dim3(H * MB), dim3(64), (size_t)((NB + 3) & ~3), s, w, row_ptr,
                     col_idx, cap, NB, p, mask_out);
  if (n2 > kToppRegMax)  // keys, then the row's mask bytes
    hipLaunchKernelGGL(k_topp_lds, dim3(H * MB), dim3(64),
                       (size_t)n2 * sizeof(uint64_t) + (size_t)((NB + 3) & ~3), s, w, row_ptr,
                       col_idx, cap, NB, p, mask_out);
  return hipGetLastError();
}

}  // namespace wa
