// Block-sparse attention forward for CDNA4 (gfx950).
//
// What is computed (WaveAlign §II-C; GSRS §3): query block u of head h attends to
// the valid tokens of the K/V blocks listed in its CSR row, in ascending order,
// with an online softmax that keeps a running max and sum per query row; the
// output is normalised at the end and the row log-sum-exp is written beside it.
// A query block with an empty list gets O = 0 and LSE = -inf (GSRS, fully masked
// rows).  With `g` set, the kernel also writes the block log-sum-exp of every
// (row, evaluated block) pair, GSRS Phase 1 (§5.3): G = m_blk + ln sum exp(z - m_blk)
// with m_blk the block maximum.
//
// Mapping onto the hardware
// -------------------------
//  * One workgroup per query block: BLOCK/32 wavefronts, each owning 32 query rows.
//  * Both products are computed transposed with v_mfma_f32_32x32x16_bf16:
//      S^T = K Q^T   (A = K rows from LDS, B = this wave's Q rows in registers)
//      O^T = V^T P^T (A = V^T rows from LDS, B = P taken straight from S^T)
//    In both outputs a lane owns one query row (column of the 32x32 tile), so the
//    row max needs one cross-lane exchange (lanes l and l^32 hold the two halves of
//    a row) and the row sum needs none until the end.  The K rows feeding the A
//    operand of S^T are permuted (pi below) so that the accumulator registers of
//    S^T are, register for register, the B operand of the P.V product: no data
//    moves between the two products.
//  * K and V^T tiles are copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no
//    VGPR staging), in 16-byte chunks whose position inside a row is XOR-swizzled
//    so that the 16 lanes of an LDS read phase hit distinct banks.  V is
//    transposed once per call by a separate pass into the workspace.
//  * Workgroup -> query block: natural head-major order, or XCD-sliced: workgroup
//    w runs on XCD w % 8 (round-robin dispatch), and XCD x takes the x-th
//    contiguous slice of each head's execution order, so each XCD's L2 sees one
//    contiguous run of the (reordered) schedule and all XCDs stay on one head.
#include <math.h>

#include "wa_internal.h"

namespace wa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Position of the 16-byte chunk c of LDS row r (XOR swizzle inside the row).
template <int CHUNKS>
__device__ inline int swz_k(int r) {
  return ((r & 3) | ((r >> 1) & 4) | ((r << 1) & 8)) & (CHUNKS - 1);
}
template <int CHUNKS>
__device__ inline int swz_v(int r) {
  return r & (CHUNKS - 1);
}

// Key row of a 32-key tile that feeds A-operand row i of S^T, chosen so that
// accumulator register r of lane group g holds key 16*(r/8) + 8*g + (r%8).
__device__ inline int pi_row(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}

template <int BLOCK, int D>
struct Tile {
  static constexpr int kWaves = BLOCK / 32;
  static constexpr int kHalves = BLOCK / 64;   // 64-key halves of a K/V tile
  static constexpr int kKChunks = D / 8;       // 16-byte chunks per K row
  static constexpr int kVChunks = BLOCK / 8;   // 16-byte chunks per V^T row
  static constexpr int kSubBytes = 64 * D * 2; // one half of the K or V^T tile
  static constexpr int kSubInst = kSubBytes / 1024 / kWaves;  // DMA instructions per wave
  static constexpr int kKS = D / 16;           // contraction steps of S^T
  static constexpr int kDT = D / 32;           // d tiles of O^T
  // Outstanding vector-memory operations allowed while waiting for one sub-tile:
  // with two halves the three sub-tile loads issued after it (minus slack for one
  // G store, which only makes the wait stricter) may stay in flight.
  static constexpr int kWaitN = kHalves == 2 ? 2 * kSubInst : 0;
};

// Lazy softmax reference: the running maximum used as the exponent reference
// only moves when a new block maximum exceeds it by more than kTau (log2
// units), so most tiles need no rescale of the output accumulator; the
// probabilities stay below 2^kTau, far inside bf16 and fp32 range.
constexpr float kTau = 8.0f;
// A half tile whose maximum lies more than kLow below the reference takes its
// own maximum as reference, so that its block log-sum-exp keeps full precision.
constexpr float kLow = 64.0f;

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4,
// saddr form: wave-uniform base in SGPRs plus a per-lane 32-bit offset; the LDS
// destination is the wave-uniform lds_addr plus 16 bytes per lane).  Issued
// through inline assembly so that the compiler does not serialise the copy
// against later LDS reads of other buffers; completion is awaited explicitly with
// wait_vmcnt (vector-memory operations retire in issue order).  M0 is saved and
// restored around the copy.
__device__ inline void dma16(const char* base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(base)
      : "memory");
}

__device__ inline uint32_t lds_address(const char* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

template <int BLOCK, int D, bool WITH_G>
__global__ __launch_bounds__(BLOCK * 2) __attribute__((amdgpu_waves_per_eu(2)))
void k_sparse_attn(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ Vt, int H, int L, int MB,
                   const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                   int cap, const int32_t* __restrict__ perm, int schedule, float scale_log2,
                   uint16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ G) {
  using T = Tile<BLOCK, D>;
  // Four separate LDS objects (K and V^T halves) so that the compiler can tell the
  // asynchronous copies into one from the reads of another.
  __shared__ __attribute__((aligned(1024))) char sk0[T::kSubBytes];
  __shared__ __attribute__((aligned(1024))) char sk1[T::kHalves == 2 ? T::kSubBytes : 16];
  __shared__ __attribute__((aligned(1024))) char sv0[T::kSubBytes];
  __shared__ __attribute__((aligned(1024))) char sv1[T::kHalves == 2 ? T::kSubBytes : 16];

  const int Lp = MB * BLOCK;
  int h, pos;
  if (schedule == WA_SCHED_XCD_SLICED) {
    const int s = (MB + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    h = j / s;
    pos = x * s + j % s;
    if (pos >= MB) return;
  } else {
    h = blockIdx.x / MB;
    pos = blockIdx.x % MB;
  }
  const int u = perm ? perm[h * MB + pos] : pos;
  if ((unsigned)u >= (unsigned)MB) return;  // malformed permutation entry: nothing to run

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int i32 = lane & 31;
  const int qrow = u * BLOCK + wave * 32 + i32;  // the query row this lane owns
  const size_t head_off = (size_t)h * Lp * D;

  const int e0 = min(row_ptr[h * MB + u], cap);
  const int e1 = min(row_ptr[h * MB + u + 1], cap);
  if (e0 >= e1) {  // fully masked query block: O = 0, LSE = -inf
#pragma unroll
    for (int c = 0; c < D / 8; c += 2) {
      uint4* dst = reinterpret_cast<uint4*>(O + head_off + (size_t)qrow * D + (c + g) * 8);
      *dst = make_uint4(0, 0, 0, 0);
    }
    if (g == 0) lse[(size_t)h * Lp + qrow] = -INFINITY;
    return;
  }

  // Per-lane byte offsets of this wave's DMA chunks inside a K half (rows = keys)
  // and a V^T half (rows = d, 64 keys wide), relative to the half's global base.
  uint32_t koff[T::kSubInst], voff[T::kSubInst];
#pragma unroll
  for (int j = 0; j < T::kSubInst; ++j) {
    const int flat = (wave + j * T::kWaves) * 1024 + lane * 16;
    const int r = flat / (D * 2);
    const int ks = (flat % (D * 2)) / 16;
    koff[j] = (uint32_t)(r * D * 2 + ((ks ^ swz_k<T::kKChunks>(r)) * 16));
    const int d = flat / 128;  // a V^T half row is 64 keys = 128 bytes
    const int vs = (flat % 128) / 16;
    voff[j] = (uint32_t)((size_t)d * Lp * 2 + ((vs ^ swz_v<8>(d)) * 16));
  }
  const char* kbytes = reinterpret_cast<const char*>(K + head_off);
  const char* vbytes = reinterpret_cast<const char*>(Vt + head_off);
  const uint32_t lk[2] = {lds_address(sk0), lds_address(sk1)};
  const uint32_t lv[2] = {lds_address(sv0), lds_address(sv1)};
  auto issue_k = [&](int v, int half) {
    const char* base = kbytes + ((size_t)v * BLOCK + 64 * half) * D * 2;
#pragma unroll
    for (int j = 0; j < T::kSubInst; ++j)
      dma16(base, koff[j], lk[half] + (uint32_t)((wave + j * T::kWaves) * 1024));
  };
  auto issue_v = [&](int v, int half) {
    const char* base = vbytes + ((size_t)v * BLOCK + 64 * half) * 2;
#pragma unroll
    for (int j = 0; j < T::kSubInst; ++j)
      dma16(base, voff[j], lv[half] + (uint32_t)((wave + j * T::kWaves) * 1024));
  };
  // Block id of CSR entry e, or 0 for an entry outside [0, MB) (then copied but
  // not used, so that every iteration issues the same copies).  Read as a
  // wave-uniform value so that the copy bases stay in scalar registers.
  auto block_of = [&](int e) {
    const int v = __builtin_amdgcn_readfirstlane(col_idx[e]);
    return ((unsigned)v < (unsigned)MB) ? v : 0;
  };

  // Q fragment (B operand of S^T): lane holds q[qrow][16*ks + 8*g .. +7].
  bf16x8 qf[T::kKS];
  {
    const uint16_t* qp = Q + head_off + (size_t)qrow * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < T::kKS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * ks));
  }

  f32x16 acc_o[T::kDT];
#pragma unroll
  for (int dt = 0; dt < T::kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.0f;
  float m_run = -INFINITY;  // exponent reference (log2 units)
  float l_run = 0.0f;       // this lane's part of the running sum

  // Prologue: the first tile's K halves and first V half.
  int v_cur = block_of(e0);
  issue_k(v_cur, 0);
  if constexpr (T::kHalves == 2) {
    issue_v(v_cur, 0);
    issue_k(v_cur, 1);
  }

  for (int e = e0; e < e1; ++e) {
    const bool last = e + 1 == e1;
    const bool ok = (unsigned)col_idx[e] < (unsigned)MB;
    const int v_next = last ? 0 : block_of(e + 1);
    const int key0 = v_cur * BLOCK;
    const int valid = L - key0;  // valid keys in this tile (>= 1 for a valid block)
    float c_half[2] = {-INFINITY, -INFINITY};
    float r_half[2] = {0.0f, 0.0f};

#pragma unroll
    for (int hh = 0; hh < T::kHalves; ++hh) {
      // ---- wait for K half hh, then S^T for its 64 keys ----
      if (last) wait_vmcnt<0>(); else wait_vmcnt<T::kWaitN>();
      __syncthreads();
      // Copies issued once every wave has passed this barrier, i.e. finished
      // the previous P.V product: with two halves, V half 1 of this tile (hh = 0)
      // and V half 0 of the next tile (hh = 1); with one half, this tile's V.
      if constexpr (T::kHalves == 2) {
        if (hh == 0) issue_v(v_cur, 1);
        else if (!last) issue_v(v_next, 0);
      } else {
        issue_v(v_cur, 0);
      }
      const bool live = ok && valid > 64 * hh;  // uniform: the half holds valid keys
      f32x16 acc_s[2];
      const char* sk = hh ? sk1 : sk0;
      if (live) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_s[mt][r] = 0.0f;
          const int krow = mt * 32 + pi_row(i32);
          const char* base = sk + krow * (D * 2);
          const int sw = swz_k<T::kKChunks>(krow);
#pragma unroll
          for (int ks = 0; ks < T::kKS; ++ks) {
            const int c = 2 * ks + g;
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(base + 16 * (c ^ sw)));
            acc_s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc_s[mt], 0, 0, 0);
          }
        }
        // Keys past L in the last tile never enter the softmax.
        const int vh = valid - 64 * hh;
        if (vh < 64) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = mt * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
              if (key >= vh) acc_s[mt][r] = -INFINITY;
            }
        }
        // ---- online softmax over the half ----
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[mt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_h = mx * scale_log2;
        const bool grow = m_h > m_run + kTau;
        const float m_ref = grow ? m_h : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
        bool low = false;
        float c = m_ref;
        if constexpr (WITH_G) {
          low = m_h < m_ref - kLow;
          c = low ? m_h : m_ref;
        }
        float psum = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(acc_s[mt][r], scale_log2, -c));
            acc_s[mt][r] = pv;
            psum += pv;
          }
        float beta = 1.0f;
        if constexpr (WITH_G) {
          c_half[hh] = c;
          r_half[hh] = psum;
          if (__builtin_amdgcn_ballot_w64(low) != 0) {
            beta = low ? __builtin_amdgcn_exp2f(m_h - m_ref) : 1.0f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc_s[mt][r] *= beta;
          }
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
          for (int dt = 0; dt < T::kDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
        }
        l_run = l_run * alpha + psum * beta;
        m_run = m_ref;
      }
      if constexpr (WITH_G) {
        if (hh == T::kHalves - 1 && ok) {
          // Block log-sum-exp of the tile from the halves' (reference, sum) pairs.
          const float R0 = r_half[0] + __shfl_xor(r_half[0], 32);
          const float R1 = r_half[1] + __shfl_xor(r_half[1], 32);
          const float M = fmaxf(c_half[0], c_half[1]);
          const float sum = R0 * __builtin_amdgcn_exp2f(c_half[0] - M) +
                            R1 * __builtin_amdgcn_exp2f(c_half[1] - M);
          if (g == 0) G[(size_t)e * BLOCK + wave * 32 + i32] = (M + __log2f(sum)) * kLn2;
        }
      }

      // ---- wait for V^T half hh, then O^T += V^T P^T over its 64 keys ----
      if (last) wait_vmcnt<0>(); else wait_vmcnt<T::kWaitN>();
      __syncthreads();
      if (!last) issue_k(v_next, hh);
      if (live) {
        const char* sv = hh ? sv1 : sv0;
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = (__bf16)acc_s[ps >> 1][8 * (ps & 1) + j];
          const int c = 2 * ps + g;
#pragma unroll
          for (int dt = 0; dt < T::kDT; ++dt) {
            const int drow = dt * 32 + i32;
            const char* base = sv + drow * 128;
            const bf16x8 a = as_bf16x8(
                *reinterpret_cast<const uint4*>(base + 16 * (c ^ swz_v<8>(drow))));
            acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc_o[dt], 0, 0, 0);
          }
        }
      }
    }
    v_cur = v_next;
  }

  // Normalise and store.  Register r of d tile dt holds d = 32*dt + 8*(r/4) + 4*g + r%4.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_tot;
  uint16_t* op = O + head_off + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < T::kDT; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint2 packed;
      __bf16 b0 = (__bf16)(acc_o[dt][4 * rb + 0] * inv_l);
      __bf16 b1 = (__bf16)(acc_o[dt][4 * rb + 1] * inv_l);
      __bf16 b2 = (__bf16)(acc_o[dt][4 * rb + 2] * inv_l);
      __bf16 b3 = (__bf16)(acc_o[dt][4 * rb + 3] * inv_l);
      packed.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      packed.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      *reinterpret_cast<uint2*>(op + dt * 32 + 8 * rb + 4 * g) = packed;
    }
  if (g == 0) lse[(size_t)h * Lp + qrow] = (m_run + __log2f(l_tot)) * kLn2;
}

// V [H][Lp][D] -> V^T [H][D][Lp], 64 x 64 tiles through LDS.
template <int D>
__global__ __launch_bounds__(256) void k_transpose_v(const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ Vt, int Lp) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tiles_t = Lp / 64;
  const int h = blockIdx.x / (tiles_t * (D / 64));
  const int rem = blockIdx.x % (tiles_t * (D / 64));
  const int t0 = (rem / (D / 64)) * 64;
  const int d0 = (rem % (D / 64)) * 64;
  const uint16_t* src = V + (size_t)h * Lp * D;
  uint16_t* dst = Vt + (size_t)h * D * Lp;
  for (int c = threadIdx.x; c < 64 * 8; c += 256) {
    const int tt = c >> 3, dc = (c & 7) * 8;
    const uint4 val = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + tt) * D + d0 + dc);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[tt][dc + j] = pv[j];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 64 * 8; c += 256) {
    const int dd = c >> 3, tc = (c & 7) * 8;
    uint16_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = tile[tc + j][dd];
    *reinterpret_cast<uint4*>(dst + (size_t)(d0 + dd) * Lp + t0 + tc) =
        *reinterpret_cast<const uint4*>(w);
  }
}

template <int BLOCK, int D>
hipError_t launch_typed(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H, int L,
                        const int32_t* row_ptr, const int32_t* col_idx, int cap,
                        const int32_t* perm,
                        int schedule, float scale, uint16_t* o, float* lse, float* g,
                        uint16_t* vt, hipStream_t s) {
  const int MB = (L + BLOCK - 1) / BLOCK;
  const int Lp = MB * BLOCK;
  hipLaunchKernelGGL(k_transpose_v<D>, dim3(H * (Lp / 64) * (D / 64)), dim3(256), 0, s, v, vt, Lp);
  int grid = H * MB;
  if (schedule == WA_SCHED_XCD_SLICED) grid = H * kXcds * ((MB + kXcds - 1) / kXcds);
  const float sl2 = scale * kLog2e;
  if (g != nullptr) {
    hipLaunchKernelGGL((k_sparse_attn<BLOCK, D, true>), dim3(grid), dim3(BLOCK * 2), 0, s, q, k,
                       vt, H, L, MB, row_ptr, col_idx, cap, perm, schedule, sl2, o, lse, g);
  } else {
    hipLaunchKernelGGL((k_sparse_attn<BLOCK, D, false>), dim3(grid), dim3(BLOCK * 2), 0, s, q, k,
                       vt, H, L, MB, row_ptr, col_idx, cap, perm, schedule, sl2, o, lse, g);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int H, int L_pad, int head_dim) {
  return (size_t)H * (size_t)L_pad * (size_t)head_dim * sizeof(uint16_t);
}

int attn_resident_wgs_per_cu(int head_dim, int block) {
  (void)head_dim;
  (void)block;
  return 2;  // 64 KiB of LDS per workgroup, two waves per SIMD
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H,
                              int L, int head_dim, int block, const int32_t* row_ptr,
                              const int32_t* col_idx, int64_t cap64, const int32_t* perm,
                              int schedule, float scale, uint16_t* o, float* lse, float* g,
                              void* workspace, hipStream_t s) {
  uint16_t* vt = static_cast<uint16_t*>(workspace);
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  if (block == 128 && head_dim == 128)
    return launch_typed<128, 128>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, scale, o, lse,
                                  g, vt, s);
  if (block == 128 && head_dim == 64)
    return launch_typed<128, 64>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, scale, o, lse,
                                 g, vt, s);
  if (block == 64 && head_dim == 128)
    return launch_typed<64, 128>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, scale, o, lse,
                                 g, vt, s);
  return launch_typed<64, 64>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, scale, o, lse, g,
                              vt, s);
}

}  // namespace wa
