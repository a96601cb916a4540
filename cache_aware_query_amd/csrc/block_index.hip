// Block index of a block mask: per-query-block K/V lists (CSR) and the transposed
// lists (CSC).  WaveAlign §II-B/§II-C: mask row i names the K/V blocks query block
// i visits in the kernel's inner loop; the row sum is its workload.
//
// Integer work, bit-exact by construction: row and column lists are emitted in
// ascending order with wavefront ballots, counts are exact and the prefix sums
// are single-workgroup scans.
#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kWave = 64;

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// The mask read four bytes per lane.  Words are counted from the 4-byte aligned
// address at or below the mask (o = misalignment); a word that does not lie wholly
// inside the mask is assembled from its in-range bytes, so no byte outside the
// buffer is read.  Row r covers bytes [o + r*NB, o + r*NB + NB) of that word space.
struct MaskWords {
  const uint32_t* aligned;
  const uint8_t* bytes;  // == aligned as bytes
  int64_t o, total;      // misalignment and mask size in bytes

  __device__ explicit MaskWords(const uint8_t* mask, int64_t size) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(mask);
    aligned = reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3);
    bytes = reinterpret_cast<const uint8_t*>(aligned);
    o = (int64_t)(a & 3);
    total = size;
  }
  __device__ uint32_t word(int64_t w) const {
    if (4 * w >= o && 4 * w + 4 <= o + total) return aligned[w];
    uint32_t x = 0;
    for (int b = 0; b < 4; ++b) {
      const int64_t i = 4 * w + b;
      if (i >= o && i < o + total) x |= (uint32_t)bytes[i] << (8 * b);
    }
    return x;
  }
};

// Flags (bit b) of the non-zero bytes of word w that belong to columns [0, NB) of
// the row starting at byte rs; *v0 receives the column of byte 0 of the word.
__device__ inline uint32_t row_word_flags(const MaskWords& mw, int64_t w, int64_t rs, int NB,
                                          int64_t* v0) {
  const uint32_t x = mw.word(w);
  const int64_t c0 = 4 * w - rs;
  uint32_t f = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t v = c0 + b;
    if (v >= 0 && v < NB && ((x >> (8 * b)) & 0xffu) != 0) f |= 1u << b;
  }
  *v0 = c0;
  return f;
}

// One wavefront per mask row: row_nnz[r] = number of non-zero bytes.
__global__ __launch_bounds__(256) void k_row_counts(const uint8_t* __restrict__ mask, int rows,
                                                    int NB, int32_t* __restrict__ row_nnz) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const MaskWords mw(mask, (int64_t)rows * NB);
  const int64_t rs = mw.o + (int64_t)r * NB;
  const int64_t w_end = (rs + NB + 3) / 4;
  int cnt = 0;
  for (int64_t w = rs / 4 + lane; w < w_end; w += kWave) {
    int64_t c0;
    cnt += __popc(row_word_flags(mw, w, rs, NB, &c0));
  }
  // wavefront sum (integers: exact in any order)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (lane == 0) row_nnz[r] = cnt;
}

// One workgroup of 16 wavefronts per (head, 64-column tile): lane l of every
// wavefront counts column v0 + l over the rows u = wave, wave + 16, ... (each row
// read is 64 contiguous bytes), and the 16 partial counts are added in LDS.
__global__ __launch_bounds__(1024) void k_col_counts(const uint8_t* __restrict__ mask, int H,
                                                     int MB, int NB, int32_t* __restrict__ cnt) {
  __shared__ int32_t part[16][64];
  const int tiles_per_head = (NB + 63) / 64;
  const int h = blockIdx.x / tiles_per_head;
  const int v0 = (blockIdx.x % tiles_per_head) * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int v = v0 + lane;
  const uint8_t* m = mask + (size_t)h * MB * NB + v;
  int c = 0;
  if (v < NB) {
    int u = wave;
    for (; u + 48 < MB; u += 64) {
      const uint8_t a = m[(size_t)u * NB], b = m[(size_t)(u + 16) * NB];
      const uint8_t d = m[(size_t)(u + 32) * NB], e = m[(size_t)(u + 48) * NB];
      c += (a != 0) + (b != 0) + (d != 0) + (e != 0);
    }
    for (; u < MB; u += 16) c += m[(size_t)u * NB] != 0;
  }
  part[wave][lane] = c;
  __syncthreads();
  if (wave == 0 && v < NB) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) s += part[w][lane];
    cnt[h * NB + v] = s;
  }
}

// Exclusive prefix sum of n counts into ptr[0..n] (ptr may alias cnt).  One
// workgroup of 1024 threads walks the array in tiles of 4096 counts: each thread
// holds four consecutive counts, wavefront shuffles and one LDS pass scan the
// tile, and the running total carries into the next tile, whose counts are
// loaded before the current tile is scanned.
__global__ __launch_bounds__(1024) void k_exclusive_scan(const int32_t* cnt, int32_t* ptr, int n) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  auto load4 = [&](int base) {
    int4 v = make_int4(0, 0, 0, 0);
    const int i = base + 4 * t;
    if (i < n) v.x = cnt[i];
    if (i + 1 < n) v.y = cnt[i + 1];
    if (i + 2 < n) v.z = cnt[i + 2];
    if (i + 3 < n) v.w = cnt[i + 3];
    return v;
  };
  int32_t carry = 0;
  int4 cur = load4(0);
  for (int base = 0; base < n; base += 4096) {
    const int4 nxt = base + 4096 < n ? load4(base + 4096) : make_int4(0, 0, 0, 0);
    const int32_t s4 = cur.x + cur.y + cur.z + cur.w;
    // Inclusive scan of the per-thread sums across the wavefront.
    int32_t incl = s4;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int32_t before = carry;
    int32_t total = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int32_t x = wsum[j];
      before += j < w ? x : 0;
      total += x;
    }
    __syncthreads();  // wsum is rewritten by the next tile
    int32_t run = before + incl - s4;  // exclusive prefix of this thread's first count
    const int i = base + 4 * t;
    if (i < n) ptr[i] = run;
    run += cur.x;
    if (i + 1 < n) ptr[i + 1] = run;
    run += cur.y;
    if (i + 2 < n) ptr[i + 2] = run;
    run += cur.z;
    if (i + 3 < n) ptr[i + 3] = run;
    carry += total;
    cur = nxt;
  }
  if (t == 0) ptr[n] = carry;
}

// One wavefront per row: ascending column ids of the non-zero bytes.
__global__ __launch_bounds__(256) void k_fill_rows(const uint8_t* __restrict__ mask, int rows,
                                                   int NB, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx, int64_t cap) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const uint8_t* m = mask + (size_t)r * NB;
  int64_t base = row_ptr[r];
  const uint64_t lt = lanemask_lt();
  for (int v0 = 0; v0 < NB; v0 += kWave) {
    const int v = v0 + lane;
    const bool bit = v < NB && m[v] != 0;
    const uint64_t b = __ballot(bit);
    if (bit) {
      const int64_t idx = base + __popcll(b & lt);
      if (idx < cap) col_idx[idx] = v;
    }
    base += __popcll(b);
  }
}

// One workgroup of 16 wavefronts per (head, 64-column tile): ascending row ids
// per column.  The mask is walked in tiles of 64 rows x 64 columns, staged in LDS
// so that global reads stay row-contiguous; the next tile is loaded into
// registers while the current one is scanned, and the two LDS buffers alternate
// so that one barrier per tile suffices.  Each wavefront owns 4 columns and walks
// them with ballots over the 64 rows of the tile.
__global__ __launch_bounds__(1024) void k_fill_cols(const uint8_t* __restrict__ mask, int H, int MB,
                                                    int NB, const int32_t* __restrict__ csc_ptr,
                                                    int32_t* __restrict__ csc_idx, int64_t cap) {
  __shared__ uint8_t tile[2][64][65];
  const int tiles_per_head = (NB + 63) / 64;
  const int h = blockIdx.x / tiles_per_head;
  const int v0 = (blockIdx.x % tiles_per_head) * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt = lanemask_lt();
  int64_t base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = v0 + wave + 16 * j;
    base[j] = v < NB ? csc_ptr[h * NB + v] : 0;
  }
  const uint8_t* mh = mask + (size_t)h * MB * NB;
  // Thread (wave, lane) stages rows wave + 16 k (k < 4) of column v0 + lane.
  const int sv = v0 + lane;
  uint8_t r[4];
  auto load = [&](int u0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = u0 + wave + 16 * k;
      r[k] = (u < MB && sv < NB) ? (mh[(size_t)u * NB + sv] != 0) : 0;
    }
  };
  load(0);
  int buf = 0;
  for (int u0 = 0; u0 < MB; u0 += 64) {
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[buf][wave + 16 * k][lane] = r[k];
    if (u0 + 64 < MB) load(u0 + 64);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vv = wave + 16 * j;
      const bool bit = tile[buf][lane][vv] != 0;
      const uint64_t b = __ballot(bit);
      if (bit) {
        const int64_t idx = base[j] + __popcll(b & lt);
        if (idx < cap) csc_idx[idx] = u0 + lane;
      }
      base[j] += __popcll(b);
    }
    buf ^= 1;
  }
}

}  // namespace

hipError_t launch_block_index(const uint8_t* mask, int H, int MB, int NB, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_cap, int32_t* row_nnz,
                              int32_t* csc_ptr, int32_t* csc_idx, int64_t csc_cap,
                              hipStream_t s) {
  const int rows = H * MB;
  hipLaunchKernelGGL(k_row_counts, dim3((rows + 3) / 4), dim3(256), 0, s, mask, rows, NB, row_nnz);
  hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(1024), 0, s, row_nnz, row_ptr, rows);
  hipLaunchKernelGGL(k_fill_rows, dim3((rows + 3) / 4), dim3(256), 0, s, mask, rows, NB, row_ptr,
                     col_idx, col_cap);
  if (csc_ptr != nullptr) {
    const int cols = H * NB;
    hipLaunchKernelGGL(k_col_counts, dim3(H * ((NB + 63) / 64)), dim3(1024), 0, s, mask, H, MB, NB,
                       csc_ptr);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(1024), 0, s, csc_ptr, csc_ptr, cols);
    hipLaunchKernelGGL(k_fill_cols, dim3(H * ((NB + 63) / 64)), dim3(1024), 0, s, mask, H, MB, NB,
                       csc_ptr, csc_idx, csc_cap);
  }
  return hipGetLastError();
}

}  // namespace wa
