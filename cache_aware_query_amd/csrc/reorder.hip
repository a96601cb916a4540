// WaveAlign two-stage query-row reordering on the GPU (WaveAlign §IV-C, §IV-D,
// §IV-E; Algorithms 1 and 2), one workgroup of 1024 threads per head.
//
//  1. statistics and the adaptive skip decision (§IV-E);
//  2. rank-2 embedding of the column-centered mask by matrix-free centered subspace
//     iteration (§IV-C-2, Algorithm 1): Y = M^T X - c (1^T X)/MB and
//     Z = M Y - 1 (c^T Y)/MB with the CSC and CSR lists (gathers only, so every sum
//     has a fixed order), modified Gram-Schmidt QR, then the Ritz rotation that
//     orders the basis by singular value;
//  3. polar angles (eq. (4)) and a stable ascending sort (Stage 1);
//  4. buckets of at most W positions inside contiguous slices, and a stable
//     NNZ-descending sort inside each bucket (§IV-D, Stage 2).
//
// Arithmetic is fp64 (MI355X runs fp64 vector code at half the fp32 rate; the
// whole stage is a few MFLOP per head), so the angles agree with an fp64 reference
// to rounding.  All reductions use a fixed tree (DPP and lane-swap steps inside a
// wavefront, then the wavefront sums in index order), so results are bitwise
// reproducible run to run.  The Stage-1 and Stage-2 orders are one sort each of
// distinct (key, index) pairs in LDS: wavefront rank sorts of 64, then pairwise
// merges by binary search.
#include <math.h>

#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kThreads = 1024;
// Dynamic LDS the bitmask form of the reorder may use (the rest of the 160 KiB is
// left to the kernel's static arrays).
constexpr size_t kBitsLdsLimit = 152 * 1024;
constexpr int kWaves = kThreads / 64;
// Mean row length from which the CSC-form statistics walk rows per wave.
constexpr long long kStatsWaveMin = 64;

// Orders one wave's LDS accesses across its lanes (the compiler may not move them
// past this point; the hardware keeps a wave's LDS operations in order).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr double kTwoPi = 6.283185307179586;

struct DevParams {
  int wave, n_slices, iters, stage1, stage2, skip_mode;
  double ws_min, flops_min, jac_max;
};

// One 32-bit lane move across the wavefront by a DPP pattern (all source lanes
// exist for the patterns used here).
template <int CTRL>
__device__ inline double dpp_move(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// x of this lane plus x of the lane 16 (or 32) rows away, with the two operands in
// the same order on both lanes of the pair.
__device__ inline double pair16_sum(double x) {
  const long long b = __double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false,
                                                   false);
  return __longlong_as_double(((long long)hi[0] << 32) | lo[0]) +
         __longlong_as_double(((long long)hi[1] << 32) | lo[1]);
}
__device__ inline double pair32_sum(double x) {
  const long long b = __double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false,
                                                   false);
  return __longlong_as_double(((long long)hi[0] << 32) | lo[0]) +
         __longlong_as_double(((long long)hi[1] << 32) | lo[1]);
}

// Wavefront sum, bitwise equal on every lane: each step adds a lane to its partner
// under a pairing that is its own inverse (xor 1, xor 2 inside quads, mirror inside
// rows and half rows, then across rows), and a + b == b + a exactly, so both
// partners always hold the same value.
__device__ inline double wave_sum(double x) {
  x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_move<0x140>(x);  // row_mirror
  x += dpp_move<0x141>(x);  // row_half_mirror
  x = pair16_sum(x);
  return pair32_sum(x);
}

// Block-wide sums through two alternating LDS slots: a slot is written again only
// two reductions later, after every thread has passed the barrier of the reduction
// in between, so one barrier per reduction suffices.  All threads call every
// reduction in the same order.
struct Reducer {
  double* buf;  // 2 slots of 4 * kWaves doubles
  int phase;
};

template <int N>
__device__ inline void block_sum_n(double (&v)[N], Reducer& r) {
  static_assert(N <= 4, "at most four sums per reduction");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double* slot = r.buf + r.phase * 4 * kWaves;
  r.phase ^= 1;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) slot[N * w + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = 0.0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j)
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += slot[N * j + i];
}

__device__ inline double2 block_sum2(double2 v, Reducer& r) {
  double a[2] = {v.x, v.y};
  block_sum_n(a, r);
  return make_double2(a[0], a[1]);
}

__device__ inline double block_sum(double v, Reducer& r) {
  double a[1] = {v};
  block_sum_n(a, r);
  return a[0];
}

__device__ inline long long block_sum_i64(long long v, long long* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  long long s = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
}

__device__ inline long long block_max_i64(long long v, long long* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (long long)__shfl_xor(v, off));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  long long s = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) s = max(s, red[i]);
  return s;
}

__device__ inline int block_min_i32(int v, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) s = min(s, red[i]);
  return s;
}

// Q factor of the MB x 2 block in x (in place): Gram-Schmidt with a positive
// diagonal; a second column whose orthogonalised norm is <= 1e-12 of the first
// column's norm becomes zero; a zero first column zeroes both.  The projection
// coefficient is taken as (x1 . x2) / |x1| from the same reduction as |x1|; the
// orthogonalised column's norm is summed from the new column itself.
__device__ void qr2_inplace(double2* x, int MB, Reducer& red) {
  const int t = threadIdx.x;
  double g[2] = {0.0, 0.0};
  for (int u = t; u < MB; u += kThreads) {
    const double2 xu = x[u];
    g[0] += xu.x * xu.x;
    g[1] += xu.x * xu.y;
  }
  block_sum_n(g, red);
  const double n1 = sqrt(g[0]);
  if (n1 == 0.0) {
    for (int u = t; u < MB; u += kThreads) x[u] = make_double2(0.0, 0.0);
    __syncthreads();
    return;
  }
  const double r12 = g[1] / n1;
  double s2 = 0.0;
  for (int u = t; u < MB; u += kThreads) {
    const double q1 = x[u].x / n1;
    const double w = x[u].y - r12 * q1;
    x[u] = make_double2(q1, w);
    s2 += w * w;
  }
  const double n2 = sqrt(block_sum(s2, red));
  const bool keep = n2 > 1e-12 * n1;
  for (int u = t; u < MB; u += kThreads) x[u].y = keep ? x[u].y / n2 : 0.0;
  __syncthreads();
}

// Sums over index lists in global memory: list r (entries ptr[r] .. ptr[r+1], cut
// at cap) adds src[idx[k]] over its entries.  G lanes share a list: lane j of the
// group takes entries j, j+G, ... with U loads in flight, and the G partial sums
// are added by a fixed shuffle tree, so every sum has a fixed order.
// emit(r, sum) runs on the group's first lane.
template <int G, int U, typename F>
__device__ void gather_lists(const double2* src, const int32_t* __restrict__ ptr,
                             const int32_t* __restrict__ idx, int cap, int n, F emit) {
  const int t = threadIdx.x, sub = t & (G - 1);
  for (int r0 = 0; r0 < n; r0 += kThreads / G) {
    const int r = r0 + t / G;
    double ax = 0.0, ay = 0.0;
    if (r < n) {
      const int lo = min(ptr[r], cap), hi = min(ptr[r + 1], cap);
      int k = lo + sub;
      for (; k + (U - 1) * G < hi; k += U * G) {
        int i[U];
#pragma unroll
        for (int j = 0; j < U; ++j) i[j] = idx[k + j * G];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const double2 a = src[i[j]];
          ax += a.x;
          ay += a.y;
        }
      }
      for (; k < hi; k += G) {
        const double2 a = src[idx[k]];
        ax += a.x;
        ay += a.y;
      }
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      ax += __shfl_xor(ax, off);
      ay += __shfl_xor(ay, off);
    }
    if (r < n && sub == 0) emit(r, ax, ay);
  }
}

// The same sums with the index lists read 16 bytes (four entries) per load, so that
// each load in flight brings four entries: the entries before the list's first
// 16-byte boundary and after its last one are taken one by one, the aligned
// four-entry chunks in between go to the G lanes in turn (chunk m to lane m mod G).
// Lane j adds its head entry (if any), its chunks in ascending order (each chunk's
// entries in order) and its tail entry (if any); then the same shuffle tree.  The
// index array must be 16-byte aligned.
template <int G, int U, typename F>
__device__ void gather_lists_v4(const double2* src, const int32_t* __restrict__ ptr,
                                const int32_t* __restrict__ idx, int cap, int n, F emit) {
  const int t = threadIdx.x, sub = t & (G - 1);
  for (int r0 = 0; r0 < n; r0 += kThreads / G) {
    const int r = r0 + t / G;
    double ax = 0.0, ay = 0.0;
    if (r < n) {
      const int lo = min(ptr[r], cap), hi = min(ptr[r + 1], cap);
      const int a = min((lo + 3) & ~3, hi);  // first 16-byte boundary in the list
      const int b = max(a, hi & ~3);         // last one
      for (int k = lo + sub; k < a; k += G) {
        const double2 v = src[idx[k]];
        ax += v.x;
        ay += v.y;
      }
      const int4* chunk = reinterpret_cast<const int4*>(idx + a);
      const int nch = (b - a) >> 2;
      int m = sub;
      for (; m + (U - 1) * G < nch; m += U * G) {
        int4 i[U];
#pragma unroll
        for (int j = 0; j < U; ++j) i[j] = chunk[m + j * G];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const double2 v0 = src[i[j].x], v1 = src[i[j].y], v2 = src[i[j].z], v3 = src[i[j].w];
          ax += v0.x;
          ay += v0.y;
          ax += v1.x;
          ay += v1.y;
          ax += v2.x;
          ay += v2.y;
          ax += v3.x;
          ay += v3.y;
        }
      }
      for (; m < nch; m += G) {
        const int4 i = chunk[m];
        const double2 v0 = src[i.x], v1 = src[i.y], v2 = src[i.z], v3 = src[i.w];
        ax += v0.x;
        ay += v0.y;
        ax += v1.x;
        ay += v1.y;
        ax += v2.x;
        ay += v2.y;
        ax += v3.x;
        ay += v3.y;
      }
      for (int k = b + sub; k < hi; k += G) {
        const double2 v = src[idx[k]];
        ax += v.x;
        ay += v.y;
      }
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      ax += __shfl_xor(ax, off);
      ay += __shfl_xor(ay, off);
    }
    if (r < n && sub == 0) emit(r, ax, ay);
  }
}

// Lanes per list from the mean list length (uniform across the workgroup): four
// lanes with eight loads each in flight unless the lists are very short (measured
// on MI355X over 929..2841 blocks per side and 0.4%..20% density).  Bit 3 of the
// result selects the four-entry loads (index arrays 16-byte aligned).
__device__ inline int gather_lanes(long long entries, int lists, bool aligned16) {
  return (lists > 0 && entries >= 8LL * lists ? 4 : 1) | (aligned16 ? 8 : 0);
}

template <typename F>
__device__ void gather_any(int lanes, const double2* src, const int32_t* ptr,
                           const int32_t* idx, int cap, int n, F emit) {
  switch (lanes) {
    case 12: gather_lists_v4<4, 4>(src, ptr, idx, cap, n, emit); break;
    case 9: gather_lists_v4<1, 4>(src, ptr, idx, cap, n, emit); break;
    case 4: gather_lists<4, 8>(src, ptr, idx, cap, n, emit); break;
    default: gather_lists<1, 8>(src, ptr, idx, cap, n, emit); break;
  }
}

// Y = M^T X - c (1^T X) / MB, reading X and writing Y (LDS), from the CSC lists.
__device__ void apply_mt(const double2* x, double2* y, const int32_t* __restrict__ cp,
                         const int32_t* __restrict__ ci, int cap, int MB, int NB, int lanes,
                         Reducer& red) {
  const int t = threadIdx.x;
  double2 s = make_double2(0.0, 0.0);
  for (int u = t; u < MB; u += kThreads) {
    s.x += x[u].x;
    s.y += x[u].y;
  }
  s = block_sum2(s, red);
  const double inv = 1.0 / (double)MB;
  gather_any(lanes, x, cp, ci, cap, NB, [&](int v, double ax, double ay) {
    const double c = (double)(min(cp[v + 1], cap) - min(cp[v], cap));
    y[v] = make_double2(ax - c * s.x * inv, ay - c * s.y * inv);
  });
  __syncthreads();
}

// Z = M Y - 1 (c^T Y) / MB from the CSR lists; calls f(u, z) once per row.
template <typename F>
__device__ void apply_m(const double2* y, const int32_t* __restrict__ cp,
                        const int32_t* __restrict__ rp, const int32_t* __restrict__ ci, int cap,
                        int MB, int NB, int lanes, Reducer& red, F f) {
  const int t = threadIdx.x;
  double2 s = make_double2(0.0, 0.0);
  for (int v = t; v < NB; v += kThreads) {
    const double c = (double)(cp[v + 1] - cp[v]);
    s.x += c * y[v].x;
    s.y += c * y[v].y;
  }
  s = block_sum2(s, red);
  const double inv = 1.0 / (double)MB;
  gather_any(lanes, y, rp, ci, cap, MB, [&](int u, double ax, double ay) {
    f(u, make_double2(ax - s.x * inv, ay - s.y * inv));
  });
}

// Z = M Y - 1 (c^T Y) / MB with the column counts c from LDS and the rows gathered
// from the CSR in global memory (faster than walking the row bitmasks).
template <typename F>
__device__ void apply_m_rows(const double2* y, const int32_t* cc, const int32_t* __restrict__ rp,
                             const int32_t* __restrict__ ci, int cap, int MB, int NB, int lanes,
                             Reducer& red, F f) {
  const int t = threadIdx.x;
  double2 s = make_double2(0.0, 0.0);
  for (int v = t; v < NB; v += kThreads) {
    const double c = (double)cc[v];
    s.x += c * y[v].x;
    s.y += c * y[v].y;
  }
  s = block_sum2(s, red);
  const double inv = 1.0 / (double)MB;
  gather_any(lanes, y, rp, ci, cap, MB, [&](int u, double ax, double ay) {
    f(u, make_double2(ax - s.x * inv, ay - s.y * inv));
  });
}

// The head's mask as column bitmasks in LDS: column v is cm[v*MW .. +MW) (bit u%32
// of word u/32 for row u); cc[v] is the column count.  Four lanes share a column,
// each summing every fourth word in ascending bit order, and the four partial sums
// are combined with a fixed shuffle tree (so every sum has a fixed order and the
// result is reproducible).  Row products read the CSR lists instead.
struct MaskBits {
  const uint32_t* cm;
  const int32_t* cc;
  int MW;
  int8_t* digits;  // room for the fixed-point digits of apply_mt_mfma, or null
};

// Y = M^T X - c (1^T X) / MB from the column bitmasks.
__device__ void apply_mt_bits(const double2* x, double2* y, const MaskBits& mb, int MB, int NB,
                              Reducer& red) {
  const int t = threadIdx.x;
  double2 s = make_double2(0.0, 0.0);
  for (int u = t; u < MB; u += kThreads) {
    s.x += x[u].x;
    s.y += x[u].y;
  }
  s = block_sum2(s, red);
  const double inv = 1.0 / (double)MB;
  const int sub = t & 3;
  for (int v = t >> 2; v < NB; v += kThreads / 4) {
    double ax = 0.0, ay = 0.0;
    const uint32_t* col = mb.cm + (size_t)v * mb.MW;
    for (int i = sub; i < mb.MW; i += 4) {
      uint32_t bits = col[i];
      while (bits != 0u) {
        const int u = 32 * i + __builtin_ctz(bits);
        bits &= bits - 1u;
        ax += x[u].x;
        ay += x[u].y;
      }
    }
    ax += __shfl_xor(ax, 1);
    ay += __shfl_xor(ay, 1);
    ax += __shfl_xor(ax, 2);
    ay += __shfl_xor(ay, 2);
    const double c = (double)mb.cc[v];
    if (sub == 0) y[v] = make_double2(ax - c * s.x * inv, ay - c * s.y * inv);
  }
  __syncthreads();
}


typedef int i32x16_t __attribute__((ext_vector_type(16)));

// Rows of the digit table of apply_mt_mfma (seven digits per basis vector).
constexpr int kDigits = 7;

// Bytes of that table: 2 * kDigits rows of max(MB, NB) rounded up to 16 bytes.
__host__ __device__ inline size_t mfma_digit_bytes(int MB, int NB) {
  return (size_t)2 * kDigits * (size_t)(((MB > NB ? MB : NB) + 15) & ~15);
}

// Y = M^T X - c (1^T X) / MB from the column bitmasks on the matrix cores, exactly.
// Each basis entry is taken in fixed point, r = x * 2^53 rounded to the nearest
// integer (|x| <= 1 for the orthonormal basis, so |r| <= 2^53), and written as seven
// signed base-256 digits d_k, r = sum_k d_k 256^k.  The products sum_u M[u][v] d_k[u]
// are int8 MFMAs (v_mfma_i32_32x32x16_i8: the 14 digit rows times a 16-row slice of
// 32 mask columns, the mask bits spread to 0/1 bytes), exact in int32, and the
// digits are recombined in 64-bit integers: sum_u M[u][v] r_u exactly (at most MB *
// 2^53 < 2^63), whatever the order.  Y is that sum times 2^-53.  A wavefront takes
// 32 columns at a time; lane l holds digit row l % 32 and mask column l % 32 of the
// tile, and rows 8 (l / 32) .. + 7 of each 16-row slice.
__device__ void apply_mt_mfma(const double2* x, double2* y, const MaskBits& mb, int MB, int NB,
                              Reducer& red) {
  const int t = threadIdx.x;
  double2 s = make_double2(0.0, 0.0);
  for (int u = t; u < MB; u += kThreads) {
    s.x += x[u].x;
    s.y += x[u].y;
  }
  s = block_sum2(s, red);
  const double inv = 1.0 / (double)MB;
  const int MBp = (MB + 15) & ~15;
  int8_t* dg = mb.digits;  // [2 * kDigits][MBp]
  for (int u = t; u < MBp; u += kThreads) {
    long long r0 = 0, r1 = 0;
    if (u < MB) {
      r0 = __double2ll_rn(x[u].x * 0x1p53);
      r1 = __double2ll_rn(x[u].y * 0x1p53);
    }
#pragma unroll
    for (int k = 0; k < kDigits; ++k) {
      const long long d0 = ((r0 + 128) & 255) - 128;
      const long long d1 = ((r1 + 128) & 255) - 128;
      dg[(size_t)k * MBp + u] = (int8_t)d0;
      dg[(size_t)(kDigits + k) * MBp + u] = (int8_t)d1;
      r0 = (r0 - d0) >> 8;
      r1 = (r1 - d1) >> 8;
    }
  }
  __syncthreads();
  const int w = t >> 6, l = t & 63;
  const int g = l >> 5, n = l & 31;
  const int tiles = (NB + 31) / 32;
  for (int ct = w; ct < tiles; ct += kWaves) {
    const int v = ct * 32 + n;
    // lanes past the last column read column NB - 1; their sums are not stored
    const uint32_t* col = mb.cm + (size_t)min(v, NB - 1) * mb.MW;
    const int8_t* arow = dg + (size_t)min(n, 2 * kDigits - 1) * MBp + 8 * g;
    // A: digits of row n of the table at rows u0 + 8 g .. + 7 (rows 14..31 are zero);
    // B: mask bits M[u0 + 8 g .. + 7][v] (bits of rows >= MB are 0), one per byte
    auto operands = [&](int u0, long& a, long& b) {
      a = n < 2 * kDigits ? *reinterpret_cast<const long*>(arow + u0) : 0l;
      const uint32_t byte = (col[(u0 + 8 * g) >> 5] >> ((u0 + 8 * g) & 31)) & 0xffu;
      const uint32_t lo = ((byte & 0xfu) * 0x00204081u) & 0x01010101u;
      const uint32_t hi = ((byte >> 4) * 0x00204081u) & 0x01010101u;
      b = (long)(((unsigned long)hi << 32) | lo);
    };
    // two accumulators (even and odd row slices) so that consecutive MFMAs do not
    // wait for each other; integer sums, so the split changes nothing
    i32x16_t acc = {}, acc1 = {};
    int u0 = 0;
    // four row slices per step, their operand reads issued together
    for (; u0 + 64 <= MBp; u0 += 64) {
      long a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) operands(u0 + 16 * q, a[q], b[q]);
      acc = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[0], b[0], acc, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[1], b[1], acc1, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[2], b[2], acc, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[3], b[3], acc1, 0, 0, 0);
    }
    for (; u0 < MBp; u0 += 16) {
      long a0, b0;
      operands(u0, a0, b0);
      acc = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, b0, acc, 0, 0, 0);
    }
    acc += acc1;
    // register r holds digit row 8 (r / 4) + 4 g + r % 4 of column v
    long long px = 0, py = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r / 4) + 4 * g + (r % 4);
      if (j < kDigits) px += (long long)acc[r] * (1ll << (8 * j));
      else if (j < 2 * kDigits) py += (long long)acc[r] * (1ll << (8 * (j - kDigits)));
    }
    px += __shfl_xor(px, 32);
    py += __shfl_xor(py, 32);
    if (g == 0 && v < NB) {
      const double c = (double)mb.cc[v];
      y[v] = make_double2((double)px * 0x1p-53 - c * s.x * inv,
                          (double)py * 0x1p-53 - c * s.y * inv);
    }
  }
  __syncthreads();
}

// Ascending sort of n (a power of two, at most 4 * kThreads) (key, val) pairs in
// LDS, ordered by key and then by val; the pairs must be distinct.  Runs of 64 are
// sorted inside one wavefront each (an element's rank is the number of smaller
// elements of its run, counted with lane reads), then runs are merged pairwise:
// an element's place in the merged run is its index in its own run plus the number
// of smaller elements in the partner run, found by a binary search of fixed depth.
__device__ inline bool pair_less(uint64_t ka, uint32_t va, uint64_t kb, uint32_t vb) {
  return ka < kb || (ka == kb && va < vb);
}

__device__ void sort_pairs(uint64_t* key, uint32_t* val, int n) {
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r0 = n < 64 ? n : 64;
  __syncthreads();
  for (int base = w * 64; base < n; base += kThreads) {
    const bool act = lane < r0;
    const uint64_t k = act ? key[base + lane] : ~0ull;
    const uint32_t v = act ? val[base + lane] : ~0u;
    const uint32_t klo = (uint32_t)k, khi = (uint32_t)(k >> 32);
    int rank = 0;
    for (int j = 0; j < r0; ++j) {
      const uint32_t jlo = __builtin_amdgcn_readlane(klo, j);
      const uint32_t jhi = __builtin_amdgcn_readlane(khi, j);
      const uint32_t jv = __builtin_amdgcn_readlane(v, j);
      rank += pair_less(((uint64_t)jhi << 32) | jlo, jv, k, v) ? 1 : 0;
    }
    if (act) {
      key[base + rank] = k;
      val[base + rank] = v;
    }
  }
  for (int r = r0; r < n; r <<= 1) {
    __syncthreads();
    uint64_t kk[4];
    uint32_t vv[4];
    int dst[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = t + c * kThreads;
      if (i < n) {
        const uint64_t k = key[i];
        const uint32_t v = val[i];
        const int own = i & ~(r - 1);
        const int part = own ^ r;
        // Largest m with part[m - 1] < (k, v): lifted bit by bit, then one last step.
        int m = 0;
        for (int step = r >> 1; step > 0; step >>= 1)
          if (pair_less(key[part + m + step - 1], val[part + m + step - 1], k, v)) m += step;
        if (pair_less(key[part + m], val[part + m], k, v)) ++m;
        dst[c] = (own & ~r) + (i - own) + m;
        kk[c] = k;
        vv[c] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (t + c * kThreads < n) {
        key[dst[c]] = kk[c];
        val[dst[c]] = vv[c];
      }
    }
  }
  __syncthreads();
}

// Stage 2 (§IV-D) on the Stage-1 order in val[0, MB) (key and val are the sort
// arrays, n2 >= MB a power of two): inside each wave bucket of each slice, rows by
// descending NNZ, ties in Stage-1 position; then perm[pos] = row and inv_perm[row] = pos.
__device__ void stage2_and_write(uint64_t* key, uint32_t* val, int n2, const int32_t* rp, int cap,
                                 int MB, int NB, int wave, int n_slices, bool stage2,
                                 int32_t* perm_h, int32_t* inv_h) {
  const int t = threadIdx.x;
  if (stage2 && wave <= 64) {
    // Buckets of at most 64 positions: one wavefront sorts a bucket by ranking its
    // (NB - nnz, position) keys across the lanes, the same order as the sort below.
    const int s = (MB + n_slices - 1) / n_slices;
    const int per_slice = (s + wave - 1) / wave;
    const int w = t >> 6, lane = t & 63;
    for (int bk = w; bk < n_slices * per_slice; bk += kWaves) {
      const int x = bk / per_slice, j = bk - x * per_slice;
      const int lo = x * s + j * wave;
      const int hi = min(min(lo + wave, (x + 1) * s), MB);
      const int n = hi - lo;  // uniform; <= 0 past the last row
      if (n <= 0) continue;
      const bool has = lane < n;
      const uint32_t row = has ? val[lo + lane] : 0u;
      const int nnz_row = has ? min(rp[row + 1], cap) - min(rp[row], cap) : 0;
      const uint64_t k = has ? ((uint64_t)(NB - nnz_row) << 32) | (uint32_t)(lo + lane) : ~0ull;
      const uint32_t klo = (uint32_t)k, khi = (uint32_t)(k >> 32);
      int rank = 0;
      for (int i = 0; i < n; ++i) {
        const uint64_t ki = ((uint64_t)__builtin_amdgcn_readlane(khi, i) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(klo, i);
        rank += ki < k;
      }
      if (has) val[lo + rank] = row;
    }
    __syncthreads();
  } else if (stage2) {
    const int s = (MB + n_slices - 1) / n_slices;
    const int per_slice = (s + wave - 1) / wave;
    for (int pos = t; pos < n2; pos += kThreads) {
      if (pos < MB) {
        const int row = (int)val[pos];
        const int nnz_row = min(rp[row + 1], cap) - min(rp[row], cap);
        const int x = pos / s;
        const int bucket = x * per_slice + (pos - x * s) / wave;
        key[pos] = ((uint64_t)bucket << 40) | ((uint64_t)(NB - nnz_row) << 20) | (uint64_t)pos;
      } else {
        key[pos] = ~0ull;
        val[pos] = (uint32_t)pos;
      }
    }
    sort_pairs(key, val, n2);
  }
  for (int pos = t; pos < MB; pos += kThreads) {
    const int row = (int)val[pos];
    perm_h[pos] = row;
    inv_h[row] = pos;
  }
}

// BITS: the head's mask is first expanded into row and column bitmasks in LDS and
// every product with M or M^T reads those (the CSC is not used); otherwise the
// products gather through the CSR and CSC lists in global memory.
template <bool BITS>
__global__ __launch_bounds__(kThreads) void k_reorder(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ csc_ptr, const int32_t* __restrict__ csc_idx, int cap,
    const float* __restrict__ x0, int MB, int NB, int block, int head_dim, DevParams p, int rowbits,
    int mfma,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, uint8_t* __restrict__ skipped,
    double* __restrict__ angles, double* __restrict__ stats) {
  extern __shared__ double2 lds[];
  __shared__ double red_buf[2 * 4 * kWaves];
  Reducer red{red_buf, 0};
  __shared__ long long redi[kWaves];
  __shared__ int redm[kWaves];
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const int32_t* rp = row_ptr + (size_t)h * MB;
  const int32_t* cp = BITS ? nullptr : csc_ptr + (size_t)h * NB;
  int32_t* perm_h = perm + (size_t)h * MB;
  int32_t* inv_h = inv_perm + (size_t)h * MB;
  double* ang_h = angles ? angles + (size_t)h * MB : nullptr;

  // ---- statistics and the skip decision (§IV-E) ----
  // The size and work rules need only NNZ counts: when they (or WA_SKIP_ALWAYS)
  // decide, the head is skipped at once and the adjacent-row similarity, which the
  // decision did not need, is reported as NaN.  The work rule looks at the heaviest
  // head of the launch: the heads are reordered side by side, one workgroup each, so
  // the launch costs what its slowest head costs, and once one head's work pays for
  // it the other heads are reordered at no extra cost.
  const long long nnz = (long long)rp[MB] - (long long)rp[0];
  const double ws = (double)NB * (double)block * (double)head_dim * 4.0;
  const double flops = 4.0 * (double)block * (double)block * (double)head_dim * (double)nnz;
  double call_flops = flops;
  if (p.skip_mode == WA_SKIP_ADAPTIVE) {
    long long most = 0;
    for (int hh = t; hh < (int)gridDim.x; hh += kThreads)
      most = max(most, (long long)row_ptr[(size_t)(hh + 1) * MB] - (long long)row_ptr[(size_t)hh * MB]);
    most = block_max_i64(most, redi);
    call_flops = 4.0 * (double)block * (double)block * (double)head_dim * (double)most;
  }
  auto skip_head = [&](double jac_) {
    if (stats != nullptr && t == 0) {
      double* s_ = stats + (size_t)h * 5;
      s_[0] = (double)nnz;
      s_[1] = (double)nnz / ((double)MB * (double)NB);
      s_[2] = ws;
      s_[3] = flops;
      s_[4] = jac_;
    }
    if (t == 0) skipped[h] = 1;
    for (int u = t; u < MB; u += kThreads) {
      perm_h[u] = u;
      inv_h[u] = u;
      if (ang_h) ang_h[u] = __longlong_as_double(0x7ff8000000000000ll);
    }
  };
  if (p.skip_mode == WA_SKIP_ALWAYS ||
      (p.skip_mode == WA_SKIP_ADAPTIVE && !(ws > p.ws_min && call_flops >= p.flops_min))) {
    skip_head(__longlong_as_double(0x7ff8000000000000ll));
    return;
  }

  MaskBits bits{};
  // BITS: this thread's part of the sum over adjacent row pairs of |R_u & R_u+1|,
  // read off the column bitmasks as pairs of neighbouring set bits.
  long long pair_inter = 0;
  if constexpr (BITS) {
    const int MW = (MB + 31) / 32;
    uint32_t* cm = reinterpret_cast<uint32_t*>(lds + MB + NB);
    int32_t* cc = reinterpret_cast<int32_t*>(cm + (size_t)NB * MW);
    // mfma: the launch left room after the bitmasks for the digit table of the
    // matrix-core product (16-byte aligned)
    const size_t digit_off =
        ((size_t)(MB + NB) * sizeof(double2) + ((size_t)NB * MW + NB) * 4 + 15) & ~(size_t)15;
    int8_t* digits = mfma ? reinterpret_cast<int8_t*>(reinterpret_cast<char*>(lds) + digit_off)
                          : nullptr;
    for (int i = t; i < NB * MW; i += kThreads) cm[i] = 0u;
    __syncthreads();
    // Each wavefront sets the bits of four of its rows at a time, the first 128 entries
    // of each of the four loaded together (the lists sit in L2: their latency, not
    // their bytes, is the cost); OR is order-free, so the bitmasks do not depend on it.
    const int w = t >> 6, lane = t & 63;
    for (int u = w; u < MB; u += 4 * kWaves) {
      int lo[4], hi[4], vv[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int uu = u + j * kWaves;
        lo[j] = uu < MB ? min(rp[uu], cap) : 0;
        hi[j] = uu < MB ? min(rp[uu + 1], cap) : 0;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int k = lo[j] + lane + 64 * m;
          vv[j][m] = k < hi[j] ? col_idx[k] : -1;
        }
      auto set_bit = [&](int uu, int v) {
        atomicOr(&cm[(size_t)v * MW + (uu >> 5)], 1u << (uu & 31));
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int uu = u + j * kWaves;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int v = vv[j][m];
          if ((unsigned)v < (unsigned)NB) set_bit(uu, v);
        }
        for (int k = lo[j] + 128 + lane; k < hi[j]; k += 64) {
          const int v = col_idx[k];
          if ((unsigned)v < (unsigned)NB) set_bit(uu, v);
        }
      }
    }
    __syncthreads();
    for (int v = t; v < NB; v += kThreads) {
      int c = 0;
      uint32_t prev = 0u;
      for (int i = 0; i < MW; ++i) {
        const uint32_t x = cm[(size_t)v * MW + i];
        c += __popc(x);
        pair_inter += __popc(x & (x >> 1)) + (int)((prev >> 31) & x & 1u);
        prev = x;
      }
      cc[v] = c;
    }
    __syncthreads();
    bits = MaskBits{cm, cc, MW, digits};
  }

  long long inter = 0, uni = 0;
  // Without the bitmasks of the BITS form, row bitmasks alone still fit in LDS for
  // moderate sizes (rowbits): built here from the lists, they only serve the pairs.
  const uint32_t* prm = reinterpret_cast<const uint32_t*>(lds);
  const int pnw = (NB + 31) / 32;
  if constexpr (!BITS) {
    if (rowbits) {
      uint32_t* rmw = reinterpret_cast<uint32_t*>(lds);
      for (int i = t; i < MB * pnw; i += kThreads) rmw[i] = 0u;
      __syncthreads();
      const int w = t >> 6, lane = t & 63;
      for (int u = w; u < MB; u += kWaves)
        for (int k = min(rp[u], cap) + lane, e = min(rp[u + 1], cap); k < e; k += 64) {
          const int v = col_idx[k];
          if ((unsigned)v < (unsigned)NB) atomicOr(&rmw[(size_t)u * pnw + (v >> 5)], 1u << (v & 31));
        }
      __syncthreads();
    }
  }
  if (BITS) {
    // pooled union = sum over pairs of |R_u| + |R_u+1| minus the intersections
    inter = pair_inter;
    uni = -pair_inter;
    if (t == 0) {
      const long long n0 = min(rp[1], cap) - min(rp[0], cap);
      const long long nl = min(rp[MB], cap) - min(rp[MB - 1], cap);
      uni += 2 * ((long long)min(rp[MB], cap) - min(rp[0], cap)) - n0 - nl;
    }
  } else if (rowbits || nnz < kStatsWaveMin * (long long)MB) {
    // One thread per adjacent pair: popcounts of the row bitmasks, else a merge of
    // the two sorted lists (short lists: cheaper than walking rows per wave).
    for (int u = t; u + 1 < MB; u += kThreads) {
      const int na = min(rp[u + 1], cap) - min(rp[u], cap);
      const int nb = min(rp[u + 2], cap) - min(rp[u + 1], cap);
      int common = 0;
      if (rowbits) {
        for (int i = 0; i < pnw; ++i)
          common += __popc(prm[(size_t)u * pnw + i] & prm[(size_t)(u + 1) * pnw + i]);
      } else {
        int a = min(rp[u], cap), ae = min(rp[u + 1], cap);
        int b = ae, be = min(rp[u + 2], cap);
        while (a < ae && b < be) {
          const int va = col_idx[a], vb = col_idx[b];
          common += va == vb;
          a += va <= vb;
          b += vb <= va;
        }
      }
      inter += common;
      uni += na + nb - common;
    }
  } else {
    // Each wave walks a run of consecutive rows, keeping the last two rows as bit
    // sets in its own LDS: row u+1's entries are tested against row u's bits and set
    // in the other buffer, so every list is read from memory once.
    const int NW = (NB + 31) / 32, w = t >> 6, lane = t & 63;
    uint32_t* bset = reinterpret_cast<uint32_t*>(lds) + (size_t)w * 2 * NW;
    const int pairs = MB - 1, run = (pairs + kWaves - 1) / kWaves;
    const int u0 = w * run, u1 = min(u0 + run, pairs);
    for (int i = lane; i < 2 * NW; i += 64) bset[i] = 0u;
    wave_sync();
    if (u0 < u1) {
      for (int k = min(rp[u0], cap) + lane, e = min(rp[u0 + 1], cap); k < e; k += 64) {
        const int v = col_idx[k];
        if ((unsigned)v < (unsigned)NB) atomicOr(&bset[(u0 & 1) * NW + (v >> 5)], 1u << (v & 31));
      }
      if (lane == 0) uni += min(rp[u0 + 1], cap) - min(rp[u0], cap);
    }
    for (int u = u0; u < u1; ++u) {
      uint32_t* cur = bset + (u & 1) * NW;
      uint32_t* nxt = bset + ((u + 1) & 1) * NW;
      wave_sync();
      const int lo = min(rp[u + 1], cap), hi = min(rp[u + 2], cap);
      int common = 0;
      int k = lo + lane;
      auto test_set = [&](int v) {
        if ((unsigned)v < (unsigned)NB) {
          common += (int)((cur[v >> 5] >> (v & 31)) & 1u);
          atomicOr(&nxt[v >> 5], 1u << (v & 31));
        }
      };
      for (; k + 192 < hi; k += 256) {
        const int v0 = col_idx[k], v1 = col_idx[k + 64], v2 = col_idx[k + 128], v3 = col_idx[k + 192];
        test_set(v0);
        test_set(v1);
        test_set(v2);
        test_set(v3);
      }
      for (; k < hi; k += 64) test_set(col_idx[k]);
      // row u's set is dead once every lane has tested against it
      wave_sync();
      for (int i = lane; i < NW; i += 64) cur[i] = 0u;
      inter += common;
      uni += (lane == 0 ? hi - lo : 0) - common;
      if (lane == 0 && u + 1 < u1) uni += hi - lo;
    }
  }
  inter = block_sum_i64(inter, redi);
  uni = block_sum_i64(uni, redi);
  const bool idx16 =
      ((reinterpret_cast<uintptr_t>(col_idx) | reinterpret_cast<uintptr_t>(csc_idx)) & 15) == 0;
  const int glists = gather_lanes(nnz, max(MB, NB), idx16);
  const double jac = uni == 0 ? 1.0 : (double)inter / (double)uni;
  if (p.skip_mode == WA_SKIP_ADAPTIVE && !(jac < p.jac_max)) {
    skip_head(jac);
    return;
  }
  if (stats != nullptr && t == 0) {
    double* s = stats + (size_t)h * 5;
    s[0] = (double)nnz;
    s[1] = (double)nnz / ((double)MB * (double)NB);
    s[2] = ws;
    s[3] = flops;
    s[4] = jac;
  }
  if (t == 0) skipped[h] = 0;

  // ---- Stage 1: spectral polar order ----
  double2* X = lds;        // [MB]
  double2* Y = lds + MB;   // [NB]
  bool varied = false;
  for (int v = t; v < NB; v += kThreads) {
    const int c = BITS ? bits.cc[v] : cp[v + 1] - cp[v];
    varied |= (c != 0 && c != MB);
  }
  const bool embed = p.stage1 && __syncthreads_or(varied);
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  uint64_t* key = reinterpret_cast<uint64_t*>(lds);    // [n2], after the embedding
  uint32_t* val = reinterpret_cast<uint32_t*>(key + n2);  // [n2]
  if (embed) {
    const float* xh = x0 + (size_t)h * MB * 2;
    for (int u = t; u < MB; u += kThreads)
      X[u] = make_double2((double)xh[2 * u], (double)xh[2 * u + 1]);
    __syncthreads();
    qr2_inplace(X, MB, red);
    for (int it = 0; it < p.iters; ++it) {
      if constexpr (BITS) {
        if (bits.digits) apply_mt_mfma(X, Y, bits, MB, NB, red);
        else apply_mt_bits(X, Y, bits, MB, NB, red);
        apply_m_rows(Y, bits.cc, rp, col_idx, cap, MB, NB, glists, red,
                     [&](int u, double2 z) { X[u] = z; });
      } else {
        apply_mt(X, Y, cp, csc_idx, cap, MB, NB, glists, red);
        apply_m(Y, cp, rp, col_idx, cap, MB, NB, glists, red, [&](int u, double2 z) { X[u] = z; });
      }
      __syncthreads();
      qr2_inplace(X, MB, red);
    }
    // Ritz rotation: B = X^T Z with Z = M~ M~^T X, symmetrised; rotate X onto the
    // eigenvectors of B, larger eigenvalue first.
    double b00 = 0.0, b01 = 0.0, b10 = 0.0, b11 = 0.0;
    auto ritz_acc = [&](int u, double2 z) {
      const double2 xu = X[u];
      b00 += xu.x * z.x;
      b01 += xu.x * z.y;
      b10 += xu.y * z.x;
      b11 += xu.y * z.y;
    };
    if constexpr (BITS) {
      if (bits.digits) apply_mt_mfma(X, Y, bits, MB, NB, red);
      else apply_mt_bits(X, Y, bits, MB, NB, red);
      apply_m_rows(Y, bits.cc, rp, col_idx, cap, MB, NB, glists, red, ritz_acc);
    } else {
      apply_mt(X, Y, cp, csc_idx, cap, MB, NB, glists, red);
      apply_m(Y, cp, rp, col_idx, cap, MB, NB, glists, red, ritz_acc);
    }
    const double2 bd = block_sum2(make_double2(b00, b11), red);
    const double2 bo = block_sum2(make_double2(b01, b10), red);
    const double boff = 0.5 * (bo.x + bo.y);
    const double theta = 0.5 * atan2(2.0 * boff, bd.x - bd.y);
    const double cs = cos(theta), sn = sin(theta);
    double cube0 = 0.0, cube1 = 0.0;
    for (int u = t; u < MB; u += kThreads) {
      const double2 xu = X[u];
      const double r0 = xu.x * cs + xu.y * sn;
      const double r1 = -xu.x * sn + xu.y * cs;
      X[u] = make_double2(r0, r1);
      cube0 += r0 * r0 * r0;
      cube1 += r1 * r1 * r1;
    }
    // Sign convention: positive sum of cubes; near zero, first entry > 1e-6 positive.
    const double2 cube = block_sum2(make_double2(cube0, cube1), red);
    int first0 = MB, first1 = MB;
    for (int u = t; u < MB; u += kThreads) {
      if (fabs(X[u].x) > 1e-6) first0 = min(first0, u);
      if (fabs(X[u].y) > 1e-6) first1 = min(first1, u);
    }
    first0 = block_min_i32(first0, redm);
    first1 = block_min_i32(first1, redm);
    bool flip0, flip1;
    if (fabs(cube.x) >= 1e-6) flip0 = cube.x < 0.0;
    else flip0 = first0 < MB && X[first0].x < 0.0;
    if (fabs(cube.y) >= 1e-6) flip1 = cube.y < 0.0;
    else flip1 = first1 < MB && X[first1].y < 0.0;
    __syncthreads();
    // Angles (eq. (4)) in [0, 2pi].
    double ang[WA_MAX_BLOCKS / kThreads];
    int nmine = 0;
    for (int u = t; u < MB; u += kThreads) {
      const double a0 = flip0 ? -X[u].x : X[u].x;
      const double a1 = flip1 ? -X[u].y : X[u].y;
      double a = atan2(a1, a0);
      if (a < 0.0) a += kTwoPi;
      a += 0.0;
      ang[nmine++] = a;
      if (ang_h) ang_h[u] = a;
    }
    __syncthreads();  // X is dead from here on; its LDS holds the sort arrays
    // A non-negative double's bit pattern sorts like its value, so sorting the pairs
    // (angle bits, row) is the stable ascending sort by angle.
    nmine = 0;
    for (int u = t; u < MB; u += kThreads) {
      key[u] = (uint64_t)__double_as_longlong(ang[nmine++]);
      val[u] = (uint32_t)u;
    }
    for (int u = MB + t; u < n2; u += kThreads) {
      key[u] = ~0ull;
      val[u] = (uint32_t)u;  // distinct padding, after every row
    }
    sort_pairs(key, val, n2);
  } else {
    if (ang_h)
      for (int u = t; u < MB; u += kThreads) ang_h[u] = __longlong_as_double(0x7ff8000000000000ll);
    for (int u = t; u < MB; u += kThreads) val[u] = (uint32_t)u;
    __syncthreads();
  }
  // val[pos] is the Stage-1 order.

  stage2_and_write(key, val, n2, rp, cap, MB, NB, p.wave, p.n_slices, p.stage2 != 0, perm_h,
                   inv_h);
}

// ---- The MinHash comparator order (WaveAlign Table II) ----
constexpr uint32_t kMinhashP = 0x7fffffffu;  // 2^31 - 1

// (a v + b) mod (2^31 - 1) for a, b < 2^31 and v < 2^12, by folding the high bits.
__device__ inline uint32_t minhash(uint32_t a, uint32_t b, int v) {
  const uint64_t x = (uint64_t)a * (uint32_t)v + b;
  uint32_t r = (uint32_t)(x & kMinhashP) + (uint32_t)(x >> 31);
  if (r >= kMinhashP) r -= kMinhashP;
  return r;
}

__device__ inline uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, off));
  return x;
}

// One workgroup per head: the MinHash signature of every row (a wavefront per row,
// minimum over the row's list), a sort of the rows by (signature, row), then the
// same Stage 2 and output as the spectral order.
__global__ __launch_bounds__(kThreads) void k_minhash_order(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int cap, int MB,
    int NB, uint32_t a0, uint32_t b0, uint32_t a1, uint32_t b1, int n_hash, int wave,
    int n_slices, int stage2, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ double2 lds[];
  const int h = blockIdx.x, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int32_t* rp = row_ptr + (size_t)h * MB;
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  uint64_t* key = reinterpret_cast<uint64_t*>(lds);
  uint32_t* val = reinterpret_cast<uint32_t*>(key + n2);
  for (int u = w; u < MB; u += kWaves) {
    uint32_t m0 = kMinhashP, m1 = kMinhashP;
    const int lo = min(rp[u], cap), hi = min(rp[u + 1], cap);
    for (int k = lo + lane; k < hi; k += 64) {
      const int v = col_idx[k];
      if ((unsigned)v < (unsigned)NB) {
        m0 = min(m0, minhash(a0, b0, v));
        m1 = min(m1, minhash(a1, b1, v));
      }
    }
    m0 = wave_min_u32(m0);
    m1 = wave_min_u32(m1);
    if (lane == 0) {
      key[u] = n_hash == 2 ? (((uint64_t)m0 << 31) | m1) : (uint64_t)m0;
      val[u] = (uint32_t)u;
    }
  }
  for (int u = MB + t; u < n2; u += kThreads) {
    key[u] = ~0ull;
    val[u] = (uint32_t)u;
  }
  sort_pairs(key, val, n2);
  stage2_and_write(key, val, n2, rp, cap, MB, NB, wave, n_slices, stage2 != 0,
                   perm + (size_t)h * MB, inv_perm + (size_t)h * MB);
}

// ---- The banded LSH comparator order (WaveAlign Table II) ----
// One workgroup per head.  Band b's bucket of a row is the pair of its MinHash values
// under hash functions 2b and 2b+1, as one 62-bit key.  Rows sorted by (key, row) put
// each bucket in one run whose first element is its lowest row; every row takes the
// lowest such row over the bands as its label (one owner per row and band, so no two
// threads update a label in the same band).  Rows are then ordered by (label, row)
// and the same Stage 2 follows.
__global__ __launch_bounds__(kThreads) void k_lsh_order(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int cap, int MB,
    int NB, LshHashes hs, int n_bands, int wave, int n_slices, int stage2,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ double2 lds[];
  const int h = blockIdx.x, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int32_t* rp = row_ptr + (size_t)h * MB;
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  uint64_t* key = reinterpret_cast<uint64_t*>(lds);
  uint32_t* val = reinterpret_cast<uint32_t*>(key + n2);
  int* label = reinterpret_cast<int*>(val + n2);
  for (int u = t; u < MB; u += kThreads) label[u] = u;
  for (int b = 0; b < n_bands; ++b) {
    const uint32_t a0 = hs.a[2 * b], b0 = hs.b[2 * b], a1 = hs.a[2 * b + 1], b1 = hs.b[2 * b + 1];
    for (int u = w; u < MB; u += kWaves) {
      uint32_t m0 = kMinhashP, m1 = kMinhashP;
      const int lo = min(rp[u], cap), hi = min(rp[u + 1], cap);
      for (int k = lo + lane; k < hi; k += 64) {
        const int v = col_idx[k];
        if ((unsigned)v < (unsigned)NB) {
          m0 = min(m0, minhash(a0, b0, v));
          m1 = min(m1, minhash(a1, b1, v));
        }
      }
      m0 = wave_min_u32(m0);
      m1 = wave_min_u32(m1);
      if (lane == 0) {
        key[u] = ((uint64_t)m0 << 31) | m1;
        val[u] = (uint32_t)u;
      }
    }
    for (int u = MB + t; u < n2; u += kThreads) {
      key[u] = ~0ull;
      val[u] = (uint32_t)u;
    }
    sort_pairs(key, val, n2);  // ends with a barrier
    for (int p = t; p < MB; p += kThreads) {
      // first position of the run of key[p]: the lowest row of its bucket
      const uint64_t k = key[p];
      int lo = 0, hi = p;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (key[mid] < k) lo = mid + 1;
        else hi = mid;
      }
      const int row = (int)val[p], first = (int)val[lo];
      if (first < label[row]) label[row] = first;
    }
    __syncthreads();  // the next band's keys overwrite the sorted ones
  }
  for (int u = t; u < n2; u += kThreads) {
    key[u] = u < MB ? ((uint64_t)label[u] << 32) | (uint32_t)u : ~0ull;
    val[u] = (uint32_t)u;
  }
  sort_pairs(key, val, n2);
  stage2_and_write(key, val, n2, rp, cap, MB, NB, wave, n_slices, stage2 != 0,
                   perm + (size_t)h * MB, inv_perm + (size_t)h * MB);
}

}  // namespace

size_t lsh_lds_bytes(int MB, int n_bands) {
  (void)n_bands;
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  return (size_t)n2 * (sizeof(uint64_t) + sizeof(uint32_t)) + (size_t)MB * sizeof(int);
}

hipError_t launch_lsh_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap64, int H,
                            int MB, int NB, const uint32_t* hash_a, const uint32_t* hash_b,
                            int n_bands, int wave, int n_slices, int stage2, int32_t* perm,
                            int32_t* inv_perm, hipStream_t s) {
  LshHashes hs{};
  for (int i = 0; i < 2 * n_bands; ++i) {
    hs.a[i] = hash_a[i];
    hs.b[i] = hash_b[i];
  }
  const size_t lds = lsh_lds_bytes(MB, n_bands);
  hipError_t e = hipFuncSetAttribute((const void*)k_lsh_order,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     160 * 1024 - 4096);
  if (e != hipSuccess) return e;
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  hipLaunchKernelGGL(k_lsh_order, dim3(H), dim3(kThreads), lds, s, row_ptr, col_idx, cap, MB, NB,
                     hs, n_bands, wave, n_slices, stage2, perm, inv_perm);
  return hipGetLastError();
}

size_t reorder_bits_lds_bytes(int MB, int NB) {
  const size_t MW = (MB + 31) / 32;
  return (size_t)(MB + NB) * sizeof(double2) + ((size_t)NB * MW + NB) * 4;
}

bool reorder_needs_csc(int MB, int NB) { return reorder_bits_lds_bytes(MB, NB) > kBitsLdsLimit; }

hipError_t launch_reorder(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* csc_ptr,
                          const int32_t* csc_idx, int64_t cap64, const float* x0, int H, int MB, int NB,
                          int block, int head_dim, const wa_reorder_params& p, int32_t* perm,
                          int32_t* inv_perm, uint8_t* skipped, double* angles, double* stats,
                          hipStream_t s) {
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  const bool use_bits = !reorder_needs_csc(MB, NB);
  const size_t stats_bytes = (size_t)kWaves * 2 * ((NB + 31) / 32) * sizeof(uint32_t);
  size_t embed_bytes = use_bits ? reorder_bits_lds_bytes(MB, NB)
                                : (size_t)(MB + NB) * sizeof(double2);
  // The column product on the matrix cores when its digit table fits beside the
  // bitmasks.
  const size_t mfma_bytes = ((embed_bytes + 15) & ~(size_t)15) + mfma_digit_bytes(MB, NB);
  const int mfma = use_bits && mfma_bytes <= kBitsLdsLimit ? 1 : 0;
  if (mfma) embed_bytes = mfma_bytes;
  if (!use_bits && stats_bytes > embed_bytes) embed_bytes = stats_bytes;
  // Row bitmasks for the pair statistics of the transposed-list form, when they fit.
  const size_t rowbits_bytes = (size_t)MB * ((NB + 31) / 32) * sizeof(uint32_t);
  const int rowbits = !use_bits && rowbits_bytes <= kBitsLdsLimit ? 1 : 0;
  if (rowbits && rowbits_bytes > embed_bytes) embed_bytes = rowbits_bytes;
  const size_t sort_bytes = (size_t)n2 * (sizeof(uint64_t) + sizeof(uint32_t));
  const size_t lds = embed_bytes > sort_bytes ? embed_bytes : sort_bytes;
  // The dynamic LDS limit is a function attribute of the current device; setting it
  // is idempotent and cheap, so every launch sets it (no state kept between calls).
  hipError_t e = hipFuncSetAttribute((const void*)(use_bits ? k_reorder<true> : k_reorder<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     160 * 1024 - 4096);
  if (e != hipSuccess) return e;
  DevParams dp{p.wave, p.n_slices, p.iters, p.stage1, p.stage2, p.skip_mode,
               p.ws_min_bytes, p.flops_min, p.jaccard_max};
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  if (use_bits) {
    hipLaunchKernelGGL(k_reorder<true>, dim3(H), dim3(kThreads), lds, s, row_ptr, col_idx, csc_ptr,
                       csc_idx, cap, x0, MB, NB, block, head_dim, dp, 0, mfma, perm, inv_perm, skipped,
                       angles, stats);
  } else {
    hipLaunchKernelGGL(k_reorder<false>, dim3(H), dim3(kThreads), lds, s, row_ptr, col_idx,
                       csc_ptr, csc_idx, cap, x0, MB, NB, block, head_dim, dp, rowbits, 0, perm,
                       inv_perm,
                       skipped, angles, stats);
  }
  return hipGetLastError();
}

hipError_t launch_minhash_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap64,
                                int H, int MB, int NB, const uint32_t* hash_a,
                                const uint32_t* hash_b, int n_hash, int wave, int n_slices,
                                int stage2, int32_t* perm, int32_t* inv_perm, hipStream_t s) {
  int n2 = 1;
  while (n2 < MB) n2 <<= 1;
  const size_t lds = (size_t)n2 * (sizeof(uint64_t) + sizeof(uint32_t));  // <= 48 KiB
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  hipLaunchKernelGGL(k_minhash_order, dim3(H), dim3(kThreads), lds, s, row_ptr, col_idx, cap, MB,
                     NB, hash_a[0], hash_b[0], n_hash > 1 ? hash_a[1] : 0u,
                     n_hash > 1 ? hash_b[1] : 0u, n_hash, wave, n_slices, stage2, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace wa
