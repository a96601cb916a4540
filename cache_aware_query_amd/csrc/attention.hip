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
//  * One workgroup per query block: BLOCK/32 wavefronts, each owning 32 query rows;
//    two workgroups share a compute unit (two wavefronts per SIMD).
//  * Both products are computed transposed with v_mfma_f32_32x32x16_bf16:
//      S^T = K Q^T   (A = K rows from LDS, B = this wave's Q rows in registers)
//      O^T = V^T P^T (A = V^T rows read transposed from LDS, B = P taken straight
//                     from S^T)
//    In both outputs a lane owns one query row (column of the 32x32 tile), so the
//    row max needs one cross-lane exchange (lanes l and l^32 hold the two halves of
//    a row, swapped with v_permlane32_swap) and the row sum none until the end.
//    The K rows feeding the A operand of S^T are permuted (pi below) so that the
//    accumulator registers of S^T are, register for register, the B operand of the
//    P.V product: no data moves between the two products.  Row sums are taken from
//    the bf16 probabilities with dot products against 1.
//  * The list is walked in 32-key quarters, software-pipelined: the S^T product of
//    quarter q+1 is issued while the softmax of quarter q runs, then the P.V product
//    of quarter q.  The softmax first takes the probabilities against the running
//    (lazy) reference and takes the row maximum only when their sums show that the
//    reference must move or that a block sum would lose precision.
//  * K and V are copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging) in 64-key halves, double-buffered, in 16-byte chunks whose position
//    inside a row is XOR-swizzled so that the lanes of an LDS read phase hit
//    distinct banks.  V keeps its key-row layout: the V^T operand of the P.V
//    product is gathered with ds_read_b64_tr_b16 transposing reads, so no
//    transposed copy of V is ever written.  The query block's K/V list is staged
//    in LDS so that block ids never wait on scalar memory inside the loop.
//  * Workgroup -> query block: natural head-major order, or XCD-sliced: workgroup
//    w runs on XCD w % n_xcd (round-robin dispatch; n_xcd is the device's XCD
//    count, 8 on MI355X, and wa_xcd_placement records the placement), and XCD x
//    takes the x-th
//    contiguous slice of each head's execution order, so each XCD's L2 sees one
//    contiguous run of the (reordered) schedule and all XCDs stay on one head.  The
//    head-interleaved order (position w / H of head w % H) runs all heads at once,
//    the concurrent-head execution WaveAlign compares sequential heads with; the
//    default path for unreordered heads takes it for small heads and the
//    XCD-sliced original order for large ones (WA_SCHED_DEFAULT).
#include <math.h>

#include <mutex>
#include <type_traits>

#include "wa_internal.h"

// Scratch of the allocation-free entry point (wa_sparse_attn_fwd_noalloc): the
// schedule word WA_SCHED_AUTO reads, written on the device by k_sched_select.  Each
// GPU the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not the device array: kernels get the device
// address that static_scratch() looks up.
static __device__ __align__(256) int scratch[wa::kStaticScratchBytes / sizeof(int)];

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
// V rows (keys) are read with transposing LDS reads that take four consecutive
// rows per 16-lane group; the swizzle spreads those four rows over distinct banks.
template <int CHUNKS>
__device__ inline int swz_v(int r) {
  return CHUNKS == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane s names 4 consecutive 16-bit
// elements (a row segment); lane j receives element j % 4 of lanes j / 4, j / 4 + 4,
// j / 4 + 8 and j / 4 + 12, i.e. one column of the 4 x 16 block the group names.
__device__ inline i16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) const char*)p);
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
};

// Entries of a query block's K/V list staged in LDS.  With NB <= kListCap every
// list is staged and the loop reads block ids from LDS only; larger masks read
// them from global memory.
constexpr int kListCap = 2048;

// Lazy softmax reference: the running maximum used as the exponent reference
// only moves when a new block maximum exceeds it by more than kTau (log2
// units), so most tiles need no rescale of the output accumulator; the
// probabilities stay below 2^kTau, far inside bf16 and fp32 range (a row's sum of
// them, and its products with V, stay below 2^60 for any list length here).
constexpr float kTau = 32.0f;
// A quarter whose maximum lies more than kLow below the reference takes its
// own maximum as reference, so that its block log-sum-exp keeps full precision.
constexpr float kLow = 64.0f;
// Bounds on a lane's sum of one quarter's probabilities (16 keys) under which the
// quarter keeps the current reference without taking its maximum.
constexpr float kSumMax = 4294967296.0f;            // 2^kTau
constexpr float kSumMin = 1.2621774483536189e-29f;  // 2^-96

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Copies from global memory straight into LDS, 16 bytes per lane
// (global_load_lds_dwordx4, saddr form: wave-uniform base in SGPRs plus a per-lane
// 32-bit offset; the LDS destination is the wave-uniform M0 plus 16 bytes per lane).
// Issued through inline assembly so that the compiler does not serialise the copies
// against later LDS reads of other buffers; completion is awaited explicitly with
// wait_vmcnt (vector-memory loads retire in issue order).  M0 is declared clobbered.
//
template <int N>
__device__ inline void dma16_group(const char* base, const uint32_t (&off)[4], uint32_t lds_addr) {
  static_assert(N == 2 || N == 4, "copy groups of 2 or 4");
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
        "global_load_lds_dwordx4 %4, %5 offset:3072"
        :
        : "s"(lds_addr), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(base)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "global_load_lds_dwordx4 %2, %3 offset:1024"
        :
        : "s"(lds_addr), "v"(off[0]), "v"(off[1]), "s"(base)
        : "memory", "m0");
  }
}

__device__ inline uint32_t lds_address(const char* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// Sum (or maximum) of lane l and lane l ^ 32, returned to both lanes.  Lanes l and
// l ^ 32 hold the two key halves of the same query row in every product below.
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of v added to acc (two fp32 dot products with 1).
__device__ inline float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// Softmax bookkeeping for one 32-key quarter, fixed before its exponentials.
struct QuarterDecision {
  float m_h;    // maximum of the scaled scores (log2 units), -inf if none is valid
  float m_ref;  // exponent reference after this quarter
  float c;      // exponent offset used for the probabilities (finite)
  float c_g;    // the same offset as a block statistic (-inf if nothing is valid)
  float alpha;    // rescale of the previous output and sum
  bool any_grow;  // (wave-uniform) the reference moved on some lane
  bool any_low;   // (wave-uniform) some lane keeps its quarter maximum as offset (block
                  // LSE precision); per lane: m_h < m_ref - kLow
};

template <int BLOCK, int D, bool WITH_G, bool STAGED, bool DIAG>
__global__ __launch_bounds__(BLOCK * 2) __attribute__((amdgpu_waves_per_eu(2)))
void k_sparse_attn(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, int H, int L, int MB,
                   const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                   int cap, const int32_t* __restrict__ perm, int schedule, int n_xcd,
                   float scale_log2,
                   uint16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ G,
                   float* __restrict__ ENT, float* __restrict__ DIST,
                   const int* __restrict__ sched_ws) {
  using T = Tile<BLOCK, D>;
  // Two K and two V half-tile buffers in one LDS array, so that every operand read
  // is a loop-invariant per-lane address plus a constant offset.
  __shared__ __attribute__((aligned(1024))) char kvbuf[4 * T::kSubBytes];
  char* const sk0 = kvbuf;
  char* const sk1 = kvbuf + T::kSubBytes;
  char* const sv0 = kvbuf + 2 * T::kSubBytes;
  char* const sv1 = kvbuf + 3 * T::kSubBytes;
  __shared__ int32_t blist[STAGED ? kListCap + 4 : 4];

  const int Lp = MB * BLOCK;
  int h, pos;
  if (schedule == WA_SCHED_AUTO) {
    // the choice of k_sched_select: XCD-sliced in the reordered order, or the default
    // path when every head kept its order (the permutation is the identity, not read)
    if (sched_ws[0] == WA_SCHED_DEFAULT) {
      schedule = default_schedule(MB, BLOCK, D);
      perm = nullptr;
    } else {
      schedule = WA_SCHED_XCD_SLICED;
    }
  }
  if (schedule == WA_SCHED_XCD_SLICED) {
    const int s = (MB + n_xcd - 1) / n_xcd;
    const int x = blockIdx.x % n_xcd;
    const int j = blockIdx.x / n_xcd;
    h = j / s;
    pos = x * s + j % s;
    if (pos >= MB) return;
  } else if (schedule == WA_SCHED_HEADS_INTERLEAVED) {
    h = blockIdx.x % H;
    pos = blockIdx.x / H;
    if (pos >= MB) return;  // an AUTO launch has the larger XCD-sliced grid
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
    if (DIAG && ENT != nullptr && g == 0) ENT[(size_t)h * Lp + qrow] = 0.0f;
    if (DIAG && DIST != nullptr && g == 0) DIST[(size_t)h * Lp + qrow] = 0.0f;
    return;
  }

  // The query block's K/V list, staged in LDS (STAGED: the launch guarantees
  // NB <= kListCap) so that the loop reads block ids with LDS reads only: a read
  // from global memory there is a vector-memory load, and waiting for it waits
  // for every K/V copy in flight as well.
  const int ntiles = e1 - e0;
  // Q rows (the B operand of S^T): lane holds q[qrow][16*ks + 8*g .. +7], loaded in
  // the prologue below.
  bf16x8 qf[T::kKS];
  const uint16_t* qp = Q + head_off + (size_t)qrow * D + 8 * g;
  auto load_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < T::kKS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * ks));
  };
  // List entry of tile t (wave-uniform; t is clamped into the list).
  auto list_entry = [&](int t) {
    t = min(t, ntiles - 1);
    if constexpr (STAGED) {
      if (t < kListCap) return __builtin_amdgcn_readfirstlane(blist[t]);
    }
    return __builtin_amdgcn_readfirstlane(col_idx[e0 + t]);
  };

  // Copies of a K or V half (64 keys x D, 1 KiB chunks of whole rows): wave w copies
  // the kSubInst consecutive chunks from chunk w * kSubInst on, in groups of up to
  // four that share one scalar base and one M0 (the instruction offset j KiB moves
  // both the global and the LDS address).  The per-lane offsets inside chunk j of a
  // group carry the swizzle; it depends on the row modulo 16 only, and every group
  // starts at a multiple of 16 rows, so the offsets are the same for every group.
  constexpr int kGroup = T::kSubInst < 4 ? T::kSubInst : 4;
  constexpr int kRowsPerChunk = 1024 / (D * 2);
  constexpr int kLanesPerRow = (D * 2) / 16;
  static_assert((T::kSubInst * kRowsPerChunk) % 16 == 0 && (kGroup * kRowsPerChunk) % 16 == 0,
                "copy groups must start at a multiple of 16 rows");
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = lane / kLanesPerRow, ks = lane % kLanesPerRow;
    const int r = j * kRowsPerChunk + rr;  // row modulo 16 within the group
    koff[j] = (uint32_t)(rr * D * 2 + ((ks ^ swz_k<T::kKChunks>(r)) * 16));
    voff[j] = (uint32_t)(rr * D * 2 + ((ks ^ swz_v<T::kKChunks>(r)) * 16));
  }
  const char* kbytes = reinterpret_cast<const char*>(K + head_off) + wave * T::kSubInst * 1024;
  const char* vbytes = reinterpret_cast<const char*>(V + head_off) + wave * T::kSubInst * 1024;
  const uint32_t wl = (uint32_t)(wave * T::kSubInst * 1024);
  const uint32_t lk[2] = {lds_address(sk0) + wl, lds_address(sk1) + wl};
  const uint32_t lv[2] = {lds_address(sv0) + wl, lds_address(sv1) + wl};

  // The list is walked in 32-key quarters q = 0 .. NQ-1: quarter q is key tile q % 2
  // of half q / 2; half hh is part hh % kHalves of list tile hh / kHalves and
  // lives in K/V buffer hh % 2.
  const int NH = (e1 - e0) * T::kHalves;
  const int NQ = 2 * NH;
  // K/V block to copy for list entry v: an entry outside [0, MB) copies block 0,
  // which is then masked out, so that every half issues the same copies.  The
  // entry is wave-uniform, so the copy bases stay in scalar registers.
  auto copy_block = [&](int v) { return ((unsigned)v < (unsigned)MB) ? v : 0; };
  auto issue_k = [&](int v, int hh, int buf) {
    const char* base =
        kbytes + ((size_t)copy_block(v) * BLOCK + 64 * (hh % T::kHalves)) * D * 2;
#pragma unroll
    for (int gq = 0; gq < T::kSubInst / kGroup; ++gq)
      dma16_group<kGroup>(base + gq * 4096, koff, lk[buf] + (uint32_t)(gq * 4096));
  };
  auto issue_v = [&](int v, int hh, int buf) {
    const char* base =
        vbytes + ((size_t)copy_block(v) * BLOCK + 64 * (hh % T::kHalves)) * D * 2;
#pragma unroll
    for (int gq = 0; gq < T::kSubInst / kGroup; ++gq)
      dma16_group<kGroup>(base + gq * 4096, voff, lv[buf] + (uint32_t)(gq * 4096));
  };

  // K operands of the S^T product of one 32-key tile (key tile mt of the half in a
  // K buffer), then the product itself.
  auto load_k = [&](bf16x8(&ka)[T::kKS], const char* sk, int mt) {
    const int krow = mt * 32 + pi_row(i32);
    const char* base = sk + krow * (D * 2);
    const int sw = swz_k<T::kKChunks>(krow);
#pragma unroll
    for (int ks = 0; ks < T::kKS; ++ks)
      ka[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(base + 16 * ((2 * ks + g) ^ sw)));
  };
  auto mfma_s = [&](f32x16& acc, const bf16x8(&ka)[T::kKS]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < T::kKS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], acc, 0, 0, 0);
  };
  auto compute_s = [&](f32x16& acc, const char* sk, int mt) {
    bf16x8 ka[T::kKS];
    load_k(ka, sk, mt);
    mfma_s(acc, ka);
  };

  // Keys past L (last tile) and every key of an invalid list entry leave the softmax.
  auto mask_s = [&](f32x16& acc, int v, int q) {
    const int hh = q >> 1;
    const int vq = (unsigned)v < (unsigned)MB
                       ? L - v * BLOCK - 64 * (hh % T::kHalves) - 32 * (q & 1)
                       : 0;
    if (vq < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 16 * (r >> 3) + 8 * g + (r & 7);
        if (key >= vq) acc[r] = -INFINITY;
      }
    }
  };

  f32x16 acc_o[T::kDT];
#pragma unroll
  for (int dt = 0; dt < T::kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.0f;
  float m_run = -INFINITY;  // exponent reference (log2 units)
  float l_run = 0.0f;       // this lane's part of the running sum
  float es_run = 0.0f;      // DIAG: this lane's part of sum p * score, rescaled like l_run
  float ds_run = 0.0f;      // DIAG: this lane's part of sum p * |i - j|, rescaled like l_run
  constexpr int kQ = BLOCK / 32;  // quarters per list tile
  // Block statistics of the current tile: offset and this lane's part of the sum of
  // exp2(score - offset); quarters with another offset are rescaled into it.
  float blk_m = -INFINITY, blk_s = 0.0f;
  float g_pending = 0.0f;  // G of the last finished tile, stored at the next half start
  int e_pending = -1;

  // Row maximum of a masked quarter and the reference decisions that follow from it.
  auto decide = [&](const f32x16& acc) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
    QuarterDecision d;
    d.m_h = pair_max(mx) * scale_log2;
    const bool grow = d.m_h > m_run + kTau;
    d.any_grow = __builtin_amdgcn_ballot_w64(grow) != 0;
    d.m_ref = grow ? d.m_h : m_run;
    d.alpha = 1.0f;
    if (d.any_grow) {  // rare: only then is an exponential spent on the rescale
      if (d.m_h > m_run + kTau) d.alpha = __builtin_amdgcn_exp2f(m_run - d.m_h);
    }
    const bool low = WITH_G && d.m_h < d.m_ref - kLow;
    d.any_low = WITH_G && __builtin_amdgcn_ballot_w64(low) != 0;
    d.c_g = low ? d.m_h : d.m_ref;
    d.c = d.c_g == -INFINITY ? 0.0f : d.c_g;
    return d;
  };

  // Probabilities of a quarter against exponent offset c, packed to bf16 for P.V;
  // returns this lane's sum of the packed values.
  auto exps = [&](const f32x16& acc, float c, bf16x8(&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pb[ps][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(acc[8 * ps + j], scale_log2, -c));
    return sum8(pb[1], sum8(pb[0], 0.0f));
  };

  // Bookkeeping of quarter q once its probabilities are fixed: pb against the
  // running reference (lane sum lsum), and the lane sum psum of the same keys
  // against the block-statistic offset c_g.  Adds to the running sum and, at the
  // tile's last quarter, sets the pending block LSE of the tile.
  auto account = [&](const f32x16& acc, float c_g, float psum, float lsum, int v, int q,
                     const bf16x8(&pb)[2]) __attribute__((always_inline)) {
    if constexpr (WITH_G) {
      const int qi = q % kQ;
      if (qi == 0) {
        blk_m = c_g;
        blk_s = psum;
      } else if (__builtin_amdgcn_ballot_w64(c_g != blk_m) == 0) {
        blk_s += psum;  // the usual case: the tile keeps one offset
      } else {
        const float nm = fmaxf(blk_m, c_g);
        if (nm != -INFINITY)
          blk_s = blk_s * __builtin_amdgcn_exp2f(blk_m - nm) +
                  psum * __builtin_amdgcn_exp2f(c_g - nm);
        blk_m = nm;
      }
      if (qi == kQ - 1) {
        // An entry outside [0, MB) evaluates no key: its G is -inf, so that its block
        // weight is 0.
        const float bs = pair_sum(blk_s);
        g_pending = ((unsigned)v < (unsigned)MB && blk_m != -INFINITY)
                        ? (blk_m + __log2f(bs)) * kLn2
                        : -INFINITY;
        e_pending = e0 + q / kQ;
      }
    }
    if constexpr (DIAG) {
      // Masked keys have p = 0 and score -inf; clamping the score keeps 0 * score = 0.
      // Key 16*ps + j of the quarter sits at token key0 + 16*ps + j.
      const int vb = (unsigned)v < (unsigned)MB ? v : 0;
      const int key0 = vb * BLOCK + 64 * ((q >> 1) % T::kHalves) + 32 * (q & 1) + 8 * g;
      const float d0 = (float)(qrow - key0);
      float es = 0.0f, ds = 0.0f;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = (float)pb[ps][j];
          es = fmaf(p, fmaxf(acc[8 * ps + j], -3.0e38f), es);
          ds = fmaf(p, fabsf(d0 - (float)(16 * ps + j)), ds);
        }
      es_run += es;
      ds_run += ds;
    }
    l_run += lsum;
  };

  // Softmax of quarter q (S in acc, masked).  The probabilities are first taken
  // against the current reference, without the row maximum: if every lane's sum
  // of them lies in [kSumMin, 2^kTau], no probability exceeds 2^kTau (so the
  // reference would not move) and, with G, each lane's largest probability is at
  // least kSumMin / 16, a normal number whose block sum keeps full precision.  That
  // is the usual case after the first quarter.  Otherwise (the first quarter, a
  // rising maximum, a quarter far below the reference, masked keys) the wave takes
  // the row maximum and decides as above, recomputing the probabilities if the
  // offset changed, and rescales O^T if the reference moved.
  auto quarter = [&](const f32x16& acc, int v, int q, bf16x8(&pb)[2]) __attribute__((always_inline)) {
    const float c0 = m_run == -INFINITY ? 0.0f : m_run;
    float psum = exps(acc, c0, pb);
    float lsum = psum;
    float c_g = m_run;
    const bool bad = m_run == -INFINITY || !(psum <= kSumMax) || (WITH_G && psum < kSumMin);
    // Order of the region that also holds the next quarter's S^T product (its K
    // operands were read before the copies were issued): two of these VALU
    // instructions, then one MFMA per six VALU instructions.
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
#pragma unroll
    for (int i = 0; i < T::kKS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      const QuarterDecision d = decide(acc);
      if (d.any_grow) {  // the reference moved on some lane: rescale what it weighs
#pragma unroll
        for (int dt = 0; dt < T::kDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[dt][r] *= d.alpha;
        l_run *= d.alpha;
        if constexpr (DIAG) {
          es_run *= d.alpha;
          ds_run *= d.alpha;
        }
      }
      m_run = d.m_ref;
      c_g = d.c_g;
      if (__builtin_amdgcn_ballot_w64(d.c != c0) != 0) psum = exps(acc, d.c, pb);
      lsum = psum;
      if constexpr (WITH_G) {
        if (d.any_low) {
          // Lanes whose quarter sits far below the reference: their output share uses
          // the common reference (a value 2^-64 below it or smaller).
          if (d.m_h < d.m_ref - kLow) lsum = exps(acc, d.m_ref == -INFINITY ? 0.0f : d.m_ref, pb);
        }
      }
    }
    account(acc, c_g, psum, lsum, v, q, pb);
  };

  // O^T += V^T P^T over one quarter (key tile mt of the half in a V buffer).  The V
  // buffer holds key rows; the A operand (8 consecutive keys of one d row per lane)
  // is gathered by two transposing LDS reads of four keys each.
  const int tr_s = lane & 15, tr_grp = lane >> 4;
  const int tr_key = tr_s >> 2;  // key of the row segment this lane names (mod 4)
  int tr_off[T::kDT];
#pragma unroll
  for (int dt = 0; dt < T::kDT; ++dt) {
    const int chunk = dt * 4 + 2 * (tr_grp & 1) + ((tr_s & 3) >> 1);
    tr_off[dt] = (8 * g + tr_key) * (D * 2) + ((chunk ^ swz_v<T::kKChunks>(tr_key)) * 16) +
                 8 * (tr_s & 1);
  }
  auto pv = [&](const bf16x8(&pb)[2], const char* sv, int mt) {
    bf16x8 a[2][T::kDT];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const int ps = 2 * mt + p2;
#pragma unroll
      for (int dt = 0; dt < T::kDT; ++dt) {
        const char* base = sv + tr_off[dt] + 16 * ps * (D * 2);
        const i16x4 lo = lds_read_tr16(base);
        const i16x4 hi = lds_read_tr16(base + 4 * (D * 2));
        a[p2][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
      for (int dt = 0; dt < T::kDT; ++dt)
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p2][dt], pb[p2], acc_o[dt], 0, 0, 0);
    // Every V operand read is issued before the first MFMA, so that each MFMA waits
    // only for its own pair of reads, not for reads issued just before it.
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * T::kDT, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::kDT, 0);
  };
  auto store_pending_g = [&]() {
    if constexpr (WITH_G) {
      if (e_pending >= 0 && g == 0) G[(size_t)e_pending * BLOCK + wave * 32 + i32] = g_pending;
      e_pending = -1;
    }
  };

  // One quarter step.  On entry S of quarter q is in acc[MT], masked.
  // Copies: K of half hh+2 is issued at the middle of half hh (once K of half hh is
  // consumed) and V of half hh+1 at its start; each is awaited one half later, with
  // only the younger copies (loads retire in order) left in flight.
  f32x16 acc[2];
  bf16x8 pb[2];
  // ids[i] is the list entry of tile t0 + i, t0 the tile of the step's first half.
  auto step = [&](auto mt_c, auto buf_c, int q, int t0, const int (&ids)[4]) {
    constexpr int MT = decltype(mt_c)::value;   // key tile of quarter q inside its half
    constexpr int P = decltype(buf_c)::value;   // buffer of quarter q's half
    const int hh = q >> 1;
    const bool younger = hh + 1 < NH;
    if (younger) wait_vmcnt<T::kSubInst>();
    else wait_vmcnt<0>();
    __syncthreads();
    auto id_of_half = [&](int x) { return ids[x / T::kHalves - t0]; };
    // K operands of the S product of quarter q+1 (after the last quarter they come
    // from a stale buffer and are unused), read before the copies are issued.
    bf16x8 ka[T::kKS];
    if constexpr (MT == 0) load_k(ka, P ? sk1 : sk0, 1);
    else load_k(ka, P ? sk0 : sk1, 0);
    if constexpr (MT == 0) {
      store_pending_g();
      if (hh + 1 < NH) issue_v(id_of_half(hh + 1), hh + 1, 1 - P);
    } else {
      if (hh + 2 < NH) issue_k(id_of_half(hh + 2), hh + 2, P);
    }
    // S of quarter q+1 (after the last quarter the product reads a stale buffer and
    // is unused) while this quarter's softmax runs.
    if constexpr (MT == 0) mfma_s(acc[1], ka);
    else mfma_s(acc[0], ka);
    quarter(acc[MT], id_of_half(hh), q, pb);
    if (q + 1 < NQ) mask_s(acc[1 - MT], id_of_half((q + 1) >> 1), q + 1);
    pv(pb, P ? sv1 : sv0, MT);
  };

  // Prologue: K of halves 0 and 1 and V of half 0, the staged list and Q; S of
  // quarter 0.  The first list entries are read straight from the CSR so that the
  // first copies are issued before the list is staged and before Q is loaded: the
  // three transfers overlap, and since vector-memory loads retire in issue order,
  // Q having arrived means the copies have landed as well.  (The loop never waits
  // on a global load of its own: the list is in LDS and Q in registers.)
  int ids[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ids[i] = __builtin_amdgcn_readfirstlane(col_idx[e0 + min(i, ntiles - 1)]);
  issue_k(ids[0], 0, 0);
  issue_v(ids[0], 0, 0);
  if (NH > 1) issue_k(ids[1 / T::kHalves], 1, 1);
  if constexpr (STAGED) {
    // A well-formed row holds at most NB <= kListCap entries; entries past kListCap
    // (a malformed, longer row) are read from global memory instead.
    const int n_st = min(ntiles, kListCap);
    const int t0 = threadIdx.x;
    const int first = t0 < n_st ? col_idx[e0 + t0] : 0;
    load_q();
    if (t0 < n_st) blist[t0] = first;
    for (int i = t0 + BLOCK * 2; i < n_st; i += BLOCK * 2) blist[i] = col_idx[e0 + i];
  } else {
    load_q();
  }
#pragma unroll
  for (int ks = 0; ks < T::kKS; ++ks) asm volatile("" ::"v"(qf[ks]));
  wait_vmcnt<0>();
  __syncthreads();
  compute_s(acc[0], sk0, 0);
  mask_s(acc[0], ids[0], 0);

  // Each iteration runs two halves (four quarters); the list entries it needs
  // (tiles t0 .. t0+3 at most) are read one iteration ahead.
  constexpr int kTilesPerIter = 2 / T::kHalves;
  for (int q = 0; q < NQ; q += 4) {
    const int t0 = (q >> 1) / T::kHalves;
    int next[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) next[i] = list_entry(t0 + kTilesPerIter + i);
    step(std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), q, t0, ids);
    step(std::integral_constant<int, 1>(), std::integral_constant<int, 0>(), q + 1, t0, ids);
    if (q + 2 < NQ) {
      step(std::integral_constant<int, 0>(), std::integral_constant<int, 1>(), q + 2, t0, ids);
      step(std::integral_constant<int, 1>(), std::integral_constant<int, 1>(), q + 3, t0, ids);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ids[i] = next[i];
  }
  store_pending_g();

  // Normalise and store.  Register r of d tile dt holds d = 32*dt + 8*(r/4) + 4*g + r%4.
  // A row that evaluated no key (every list entry outside [0, MB)) has l_tot = 0:
  // it gets O = 0 and LSE = -inf, like an empty list.
  const float l_tot = pair_sum(l_run);
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
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
  const float lse_row = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (g == 0) lse[(size_t)h * Lp + qrow] = lse_row;
  if constexpr (DIAG) {
    // Entropy of the row's attention: LSE - E[z] with z = scale * q.k (natural log);
    // mean attention distance: E[|i - j|] in tokens.
    const float ez = pair_sum(es_run) * inv_l * (scale_log2 * kLn2);
    const float ed = pair_sum(ds_run) * inv_l;
    if (ENT != nullptr && g == 0) ENT[(size_t)h * Lp + qrow] = l_tot > 0.0f ? lse_row - ez : 0.0f;
    if (DIST != nullptr && g == 0) DIST[(size_t)h * Lp + qrow] = ed;
  }
}

template <int BLOCK, int D>
hipError_t launch_typed(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H, int L,
                        const int32_t* row_ptr, const int32_t* col_idx, int cap,
                        const int32_t* perm, int schedule, int n_xcd, float scale, uint16_t* o,
                        float* lse, float* g, float* ent, float* dist, const int* sched_ws,
                        hipStream_t s) {
  const int MB = (L + BLOCK - 1) / BLOCK;
  if (schedule == WA_SCHED_DEFAULT) {  // known from the sizes: resolved here
    schedule = default_schedule(MB, BLOCK, D);
    perm = nullptr;
  }
  int grid = H * MB;
  if (schedule == WA_SCHED_XCD_SLICED || schedule == WA_SCHED_AUTO)
    grid = H * n_xcd * ((MB + n_xcd - 1) / n_xcd);  // >= H * MB, the other schedules' grid
  const float sl2 = scale * kLog2e;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(BLOCK * 2), 0, s, q, k, v, H, L, MB, row_ptr,
                       col_idx, cap, perm, schedule, n_xcd, sl2, o, lse, g, ent, dist, sched_ws);
  };
  const bool staged = MB <= kListCap;  // NB = MB: every list fits in LDS
  auto pick = [&](auto diag) {
    constexpr bool E = decltype(diag)::value;
    if (g != nullptr) {
      if (staged) launch(k_sparse_attn<BLOCK, D, true, true, E>);
      else launch(k_sparse_attn<BLOCK, D, true, false, E>);
    } else {
      if (staged) launch(k_sparse_attn<BLOCK, D, false, true, E>);
      else launch(k_sparse_attn<BLOCK, D, false, false, E>);
    }
  };
  if (ent != nullptr || dist != nullptr) pick(std::true_type());
  else pick(std::false_type());
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int H, int L_pad, int head_dim) {
  (void)H;
  (void)L_pad;
  (void)head_dim;
  return 256;  // the schedule chosen for WA_SCHED_AUTO; K and V are read in place
}

namespace {
// One wavefront: WA_SCHED_DEFAULT if every head was skipped, else
// WA_SCHED_XCD_SLICED, into out[0].
__global__ __launch_bounds__(64) void k_sched_select(const uint8_t* __restrict__ skipped, int H,
                                                     int* __restrict__ out) {
  bool all = true;
  for (int i = threadIdx.x; i < H; i += 64) all = all && skipped[i] != 0;
  const bool some_reordered = __builtin_amdgcn_ballot_w64(!all) != 0;
  if (threadIdx.x == 0) out[0] = some_reordered ? WA_SCHED_XCD_SLICED : WA_SCHED_DEFAULT;
}
}  // namespace

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // Once per device, with that device current: the device address of its copy.
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_sched_select(const uint8_t* skipped, int H, void* workspace, hipStream_t s) {
  hipLaunchKernelGGL(k_sched_select, dim3(1), dim3(64), 0, s, skipped, H,
                     static_cast<int*>(workspace));
  return hipGetLastError();
}

int attn_resident_wgs_per_cu(int head_dim, int block) {
  (void)head_dim;
  (void)block;
  return 2;  // 64 KiB of K/V buffers per workgroup, two waves per SIMD
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H,
                              int L, int head_dim, int block, const int32_t* row_ptr,
                              const int32_t* col_idx, int64_t cap64, const int32_t* perm,
                              int schedule, int n_xcd, float scale, uint16_t* o, float* lse,
                              float* g, float* ent, float* dist, void* workspace, hipStream_t s) {
  const int* sched_ws = static_cast<const int*>(workspace);
  const int cap = cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
  if (block == 128 && head_dim == 128)
    return launch_typed<128, 128>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, n_xcd,
                                  scale, o, lse, g, ent, dist, sched_ws, s);
  if (block == 128 && head_dim == 64)
    return launch_typed<128, 64>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, n_xcd,
                                 scale, o, lse, g, ent, dist, sched_ws, s);
  if (block == 64 && head_dim == 128)
    return launch_typed<64, 128>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, n_xcd,
                                 scale, o, lse, g, ent, dist, sched_ws, s);
  return launch_typed<64, 64>(q, k, v, H, L, row_ptr, col_idx, cap, perm, schedule, n_xcd, scale,
                              o, lse, g, ent, dist, sched_ws, s);
}

namespace {
// Each workgroup (of the attention kernel's size for this block) records the XCD it
// runs on: bits [3:0] of the XCC_ID hardware register.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void k_xcd_placement(int32_t* __restrict__ out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;
}
}  // namespace

hipError_t launch_xcd_placement(int n_wg, int block, int32_t* out, hipStream_t s) {
  if (block == 128)
    hipLaunchKernelGGL(k_xcd_placement<256>, dim3(n_wg), dim3(256), 0, s, out);
  else
    hipLaunchKernelGGL(k_xcd_placement<128>, dim3(n_wg), dim3(128), 0, s, out);
  return hipGetLastError();
}

}  // namespace wa
