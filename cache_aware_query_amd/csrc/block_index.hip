// Block index of a block mask: per-query-block K/V lists (CSR) and the transposed
// lists (CSC).  WaveAlign §II-B/§II-C: mask row i names the K/V blocks query block
// i visits in the kernel's inner loop; the row sum is its workload.
//
// Integer work, bit-exact by construction: row and column lists are emitted in
// ascending order with wavefront scans and ballots, counts are exact and the
// prefix sums are single-workgroup scans.
#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kWave = 64;

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// The mask read sixteen bytes per lane.  Chunks are counted from the 16-byte aligned
// address at or below the mask (o = misalignment); a chunk that does not lie wholly
// inside the mask is assembled from its in-range bytes, so no byte outside the
// buffer is read.  Row r covers bytes [o + r*NB, o + r*NB + NB) of that chunk space.
struct MaskChunks {
  const uint4* aligned;
  const uint8_t* bytes;  // == aligned as bytes
  int64_t o, total;      // misalignment and mask size in bytes

  __device__ explicit MaskChunks(const uint8_t* mask, int64_t size) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(mask);
    aligned = reinterpret_cast<const uint4*>(a & ~(uintptr_t)15);
    bytes = reinterpret_cast<const uint8_t*>(aligned);
    o = (int64_t)(a & 15);
    total = size;
  }
  __device__ uint4 chunk(int64_t c) const {
    if (16 * c >= o && 16 * c + 16 <= o + total) return aligned[c];
    uint32_t x[4] = {0, 0, 0, 0};
    for (int b = 0; b < 16; ++b) {
      const int64_t i = 16 * c + b;
      if (i >= o && i < o + total) x[b >> 2] |= (uint32_t)bytes[i] << (8 * (b & 3));
    }
    return make_uint4(x[0], x[1], x[2], x[3]);
  }
};

// Bit b of the result: byte b of x is non-zero (b < 4).
__device__ inline uint32_t nonzero_bytes4(uint32_t x) {
  x |= x >> 4;
  x |= x >> 2;
  x |= x >> 1;
  x &= 0x01010101u;
  return (x | (x >> 7) | (x >> 14) | (x >> 21)) & 0xfu;
}

// Flags (bit b) of the non-zero bytes of chunk c that belong to columns [0, NB) of
// the row starting at byte rs; *v0 receives the column of byte 0 of the chunk.
__device__ inline uint32_t row_chunk_flags(const MaskChunks& mc, int64_t c, int64_t rs, int NB,
                                           int64_t* v0) {
  const uint4 x = mc.chunk(c);
  uint32_t f = nonzero_bytes4(x.x) | (nonzero_bytes4(x.y) << 4) | (nonzero_bytes4(x.z) << 8) |
               (nonzero_bytes4(x.w) << 12);
  const int64_t c0 = 16 * c - rs;
  if (c0 < 0) f &= 0xffffu << (int)(-c0);            // bytes before the row's first column
  if (c0 + 16 > NB) f &= 0xffffu >> (int)(c0 + 16 - NB);  // bytes past its last column
  *v0 = c0;
  return f;
}

// One wavefront per mask row: row_nnz[r] = number of non-zero bytes.
__global__ __launch_bounds__(256) void k_row_counts(const uint8_t* __restrict__ mask, int rows,
                                                    int NB, int32_t* __restrict__ row_nnz) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const MaskChunks mc(mask, (int64_t)rows * NB);
  const int64_t rs = mc.o + (int64_t)r * NB;
  const int64_t c_end = (rs + NB + 15) / 16;
  int cnt = 0;
  for (int64_t c = rs / 16 + lane; c < c_end; c += kWave) {
    int64_t v0;
    cnt += __popc(row_chunk_flags(mc, c, rs, NB, &v0));
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
// workgroup of 1024 threads walks the array in tiles of 16,384 counts.  A tile is
// loaded with coalesced reads (thread t takes counts t, t + 1024, ...) into LDS,
// where thread t sums its contiguous run of sixteen; a wavefront shuffle scan and
// one LDS pass give each run its offset, the run's prefixes go back into LDS and
// leave with coalesced writes.  The next tile's counts are loaded into registers
// while the current one is scanned; tiles are disjoint and each count is read
// before its slot is written, so ptr may alias cnt.
__global__ __launch_bounds__(1024) void k_exclusive_scan(const int32_t* cnt, int32_t* ptr, int n) {
  constexpr int kPer = 16, kTile = 1024 * kPer;
  __shared__ int32_t tile[kTile];
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t nxt[kPer];
  auto load = [&](int base) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = base + j * 1024 + t;
      nxt[j] = i < n ? cnt[i] : 0;
    }
  };
  load(0);
  int32_t carry = 0;
  for (int base = 0; base < n; base += kTile) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) tile[j * 1024 + t] = nxt[j];
    if (base + kTile < n) load(base + kTile);
    __syncthreads();
    // this thread's run: tile[kPer*t .. kPer*t + kPer), read four at a time
    int32_t x[kPer];
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const int4 q = *reinterpret_cast<const int4*>(&tile[kPer * t + 4 * j]);
      x[4 * j + 0] = q.x;
      x[4 * j + 1] = q.y;
      x[4 * j + 2] = q.z;
      x[4 * j + 3] = q.w;
    }
    int32_t own = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) own += x[j];
    int32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int32_t run = carry + incl - own;
    int32_t total = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int32_t s = wsum[j];
      run += j < w ? s : 0;
      total += s;
    }
    int32_t pre[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      pre[j] = run;
      run += x[j];
    }
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j)
      *reinterpret_cast<int4*>(&tile[kPer * t + 4 * j]) =
          make_int4(pre[4 * j], pre[4 * j + 1], pre[4 * j + 2], pre[4 * j + 3]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = base + j * 1024 + t;
      if (i < n) ptr[i] = tile[j * 1024 + t];
    }
    carry += total;
    __syncthreads();  // tile and wsum are rewritten by the next tile
  }
  if (t == 0) ptr[n] = carry;
}

// One wavefront per row: ascending column ids of the non-zero bytes.  Each lane
// takes one 16-byte chunk of the row per pass; an exclusive shuffle scan of the
// lanes' counts places every lane's columns, in ascending order, after those of
// the lanes before it.  The pass's ids are first placed in the wavefront's own LDS
// run and then written out 64 consecutive ids per store, so that dense rows leave
// with coalesced stores.
__global__ __launch_bounds__(256) void k_fill_rows(const uint8_t* __restrict__ mask, int rows,
                                                   int NB, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx, int64_t cap) {
  __shared__ int32_t stage[4][kWave * 16];
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  int32_t* st = stage[threadIdx.x >> 6];
  const MaskChunks mc(mask, (int64_t)rows * NB);
  const int64_t rs = mc.o + (int64_t)r * NB;
  const int64_t c_first = rs / 16, c_end = (rs + NB + 15) / 16;
  int64_t base = row_ptr[r];
  for (int64_t c0 = c_first; c0 < c_end; c0 += kWave) {
    const int64_t c = c0 + lane;
    int64_t v0 = 0;
    uint32_t f = c < c_end ? row_chunk_flags(mc, c, rs, NB, &v0) : 0u;
    const int n = __popc(f);
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = incl - n;  // at most 16 * 63: inside the run
    while (f != 0) {
      const int b = __builtin_ctz(f);
      f &= f - 1;
      st[pos++] = (int32_t)(v0 + b);
    }
    const int total = __shfl(incl, 63);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < total; i += kWave)
      if (base + i < cap) col_idx[base + i] = st[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the run is rewritten by the next pass
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    base += total;
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
