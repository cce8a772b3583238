// Tiled matrix-core GEMM for gfx950: C = A B^T with both operands stored
// K-contiguous ("NT"), fused epilogue.
//
// int8 mode is the quantised linear ("INT8 Convrot Safetensors", section
// "Runtime activation quantization"): A = Qx [M, K], B = Qw [N, K], exact
// int32 accumulation A[r, o] = sum_i Qx[r, i] Qw[o, i], then
// Y[r, o] = A * s_x[r] * s_w[o] + b[o] written as fp32 or bf16 (or the raw
// int32 accumulator).  bf16 mode is the unquantised linear that routed
// layers keep (sglang PR 34581 summary, kitchen_int8 routing): fp32
// accumulation of bf16 products, Y = acc + b.
//
// Design:
//  * 256 x (32 TN) output tile per 256-thread workgroup (TN in {4, 6, 8},
//    chosen per shape), 4 waves in a 2x2 grid, each wave owning a
//    128 x (16 TN) sub-tile: 8 x TN MFMA tiles of 16x16, i.e. up to 256
//    int32/fp32 accumulators per lane, held in AGPRs.  K advances in
//    128-byte slices.
//  * Both instruction kinds consume 16 bytes per lane per operand and cover
//    64 bytes of K (v_mfma_i32_16x16x64_i8: 64 int8; v_mfma_f32_16x16x32_bf16:
//    32 bf16), so the data movement is shared and only the MFMA differs.
//  * The weight tile feeds the MFMA "row" operand and the activation tile
//    the "column" operand, so each lane's four accumulators are four
//    consecutive output features of one output row (one 16-byte fp32 or
//    8-byte bf16 store).
//  * LDS holds three activation slices and two weight slices ([rows][128 B]
//    each; 160 KiB at TN = 8).  16-byte chunks are XOR-swizzled by
//    (row & 7), which makes both the coalesced row writes and the MFMA
//    fragment reads (16 rows, one chunk column) bank-conflict free.
//  * Slices move global -> LDS directly (global_load_lds_dwordx4, no
//    staging registers), two slices ahead of the MFMAs, spread between
//    them by a compile-time schedule, with one barrier per slice (see the
//    pipeline comment at the main loop).
//  * Workgroups are remapped so that each of the 8 XCDs (workgroup id mod 8
//    on dispatch) works on a contiguous range of tiles, and tiles are walked
//    in groups of 8 row-tiles so that concurrent workgroups on one XCD share
//    A and B panels in that XCD's L2.
//  * Integer accumulation is exact, so every tiling gives the same bits.
//  * Fused epilogues (int8 mode): an activation applied to Y (GELU in its erf
//    or tanh form), or a gated pair: two weights sharing the packed
//    activation, Y = act(gate) * up.  For the pair, each wave's half of the
//    B tile holds gate rows and the up rows of the same features, so a lane
//    ends with both results of an output in registers.
//
// This header holds the kernel template; the translation units that
// instantiate it (plain int8, bf16, fused epilogues) compile in parallel.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "device.h"
#include "epilogue.h"
#include "launchers.h"

namespace convrot {
namespace {

// Four consecutive outputs go out as one vector store when aligned for it.
template <typename T>
__device__ __forceinline__ bool vec_ok(const T* p) {
  return (reinterpret_cast<uintptr_t>(p) & (4 * sizeof(T) - 1)) == 0;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256;
constexpr int kBK = 128;  // bytes of K per LDS slice
constexpr int kWM = 128;
constexpr int kTM = kWM / 16;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kATileBytes = kBM * kBK;  // one A slice

// The MFMAs are issued through inline asm so that the accumulator is pinned
// to AGPRs and tied in/out ("+a"): with the builtins the register allocator
// spreads the 256 accumulators over both register files once two fragment
// sets are live and copies them every iteration.  The compiler does not see
// these as MFMAs, so the kernel pads the MFMA hazards itself (see s_nop uses
// below): a VALU write feeding an MFMA needs 2 wait states, and an MFMA
// result read by non-MFMA instructions needs up to 11 (8-pass) / 19 (16-pass).
template <bool I8>
struct Mfma;

//
// Statements that only make sense for the GPU target (AMDGPU register
// constraints, s_waitcnt) sit under __HIP_DEVICE_COMPILE__: the host pass of
// the same source must still see a well-formed kernel to emit its launch
// stub.
template <>
struct Mfma<true> {
  typedef i32x4 acc_t;
  static __device__ __forceinline__ void run(i32x4& c, const i32x4& a, const i32x4& b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
#endif
  }
};

template <>
struct Mfma<false> {
  typedef f32x4 acc_t;
  static __device__ __forceinline__ void run(f32x4& c, const i32x4& a, const i32x4& b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
#endif
  }
};

// s_waitcnt immediates (GFX9 layout: vmcnt [3:0] + [15:14], expcnt [6:4],
// lgkmcnt [11:8]): lgkmcnt(0) only, and vmcnt(0) lgkmcnt(0).
__device__ __forceinline__ void wait_lds() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xC07F);
#endif
}
__device__ __forceinline__ void wait_lds_and_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0070);
#endif
}
// Wait until at most N of this wave's vector-memory operations are
// outstanding (lgkmcnt and expcnt are not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}
// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4): lane
// l's 16 bytes land at lds + 16 l.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
#endif
}
// 16-byte LDS read into a fragment register, issued in program order (the
// caller retires it with wait_lds()).
template <int OFF>
__device__ __forceinline__ void lds_read16(i32x4& r, uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
#endif
}
__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(p)));
}
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}
// Keeps the compiler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}
// Hazard padding (wait states) as an ordered statement.
template <int N>
__device__ __forceinline__ void pad() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  static_assert(N == 5 || N == 16 || N == 24, "add the padding length needed");
  if constexpr (N == 5) {
    asm volatile("s_nop 4" ::);
  } else if constexpr (N == 16) {
    asm volatile("s_nop 7\n\ts_nop 7" ::);
  } else {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  }
  __builtin_amdgcn_sched_barrier(0);
#endif
}
// Keeps fragment registers allocated up to this point (no instruction).
// The MFMAs are inline asm, so the compiler does not know that an MFMA may
// still be reading its operands several cycles after issue; without this it
// may hand a register to an unrelated temporary right behind the last MFMA
// that reads it.
template <int N>
__device__ __forceinline__ void keep_live(const i32x4 (&r)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(r[i]));
#endif
}
// Marks an accumulator as rewritten here (no instruction).
template <typename T>
__device__ __forceinline__ void touch_acc(T& a) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+a"(a));
#endif
}
// Workgroup barrier without the memory fence of __syncthreads(), whose
// release semantics would add a wait for every outstanding vector-memory
// operation; callers wait for exactly what they need before it.
__device__ __forceinline__ void barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#endif
}
// Zero the B fragments of chunks past the end of K, then pad the VALU ->
// MFMA hazard; the asm operands keep the selects ahead of the padding.
template <int TN>
__device__ __forceinline__ void mask_tail(i32x4* fb, bool dead) {
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[j] = dead ? i32x4{0, 0, 0, 0} : fb[j];
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(TN == 4 || TN == 6 || TN == 8, "unsupported tile width");
  if constexpr (TN == 4) {
    asm volatile("s_nop 4" : "+v"(fb[0]), "+v"(fb[1]), "+v"(fb[2]), "+v"(fb[3]));
  } else if constexpr (TN == 6) {
    asm volatile("s_nop 4" : "+v"(fb[0]), "+v"(fb[1]), "+v"(fb[2]), "+v"(fb[3]), "+v"(fb[4]), "+v"(fb[5]));
  } else {
    asm volatile("s_nop 4" : "+v"(fb[0]), "+v"(fb[1]), "+v"(fb[2]), "+v"(fb[3]), "+v"(fb[4]), "+v"(fb[5]),
                 "+v"(fb[6]), "+v"(fb[7]));
  }
#endif
}

// Tile coordinates for this workgroup: XCD-contiguous ranges, then grouped
// row-major order inside each range.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, local = bid / 8;
  const int logical = xcd * q + min(xcd, r) + local;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// LDS: three A slices (the activation tile is re-filled one slice
// further ahead than the weight tile) and two B slices.
template <int TN>
constexpr int smem_bytes() {
  return 3 * kATileBytes + 2 * (32 * TN) * kBK;
}

// OUT: 0 = fp32, 1 = bf16, 2 = raw int32 accumulator.
// TN: 16-wide output tiles per wave along N; the workgroup tile is
// 256 x (32 TN), 4 waves in a 2 x 2 grid, each wave 128 x (16 TN).
// ACT: epilogue activation (see activation()).  GATED: the B tile of each
// wave column holds 8 TN gate rows then the 8 TN up rows of the same
// features, and the output tile is half as wide.
template <bool I8, int OUT, bool KTAIL, int TN, int ACT = 0, bool GATED = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, EpiArgs epi, int M,
    int N, int Kb, void* __restrict__ C, int64_t ldc, int tiles_m, int tiles_n, bool vec_cols, bool staged) {
  static_assert(!GATED || (I8 && TN % 2 == 0), "the gated pair is an int8 feature");
  static_assert((ACT == 0 && !GATED) || OUT != 2, "activations need a float output");
  const float* __restrict__ sa = epi.sa;
  const float* __restrict__ sb = epi.sb;
  const float* __restrict__ bias = epi.bias;
  constexpr int kBN = 32 * TN;
  constexpr int kWN = 16 * TN;
  constexpr int kTNo = GATED ? TN / 2 : TN;  // output 16-column tiles per wave
  constexpr int kWNo = 16 * kTNo;            // output columns per wave
  constexpr int kBNo = 2 * kWNo;             // output columns per tile
  constexpr int kBTileBytes = kBN * kBK;
  constexpr int kDmaA = kBM / 32;  // 1 KiB DMA instructions per slice and wave: A part
  constexpr int kDmas = kDmaA + kBN / 32;
  constexpr int kBBase = 3 * kATileBytes;  // LDS offset of the B slices
  static_assert(smem_bytes<TN>() <= 160 * 1024, "LDS budget");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using Op = Mfma<I8>;
  using acc_t = typename Op::acc_t;

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m_blk = tm * kBM;
  const int n_blk = tn * kBNo;  // first output feature of the tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = (wid & 1) * kWM;
  const int wn = (wid >> 1) * kWN;     // B-tile rows of the wave
  const int wno = (wid >> 1) * kWNo;   // output columns of the wave

  // Global -> LDS without registers (global_load_lds_dwordx4): one
  // instruction fills a contiguous 1 KiB LDS block, i.e. 8 swizzled rows of
  // a slice, lane l writing physical chunk l % 8 of row l / 8.  Wave w
  // fills blocks w, w + 4, ..., so each lane fetches logical chunk
  // (l % 8) ^ (l / 8) of rows 8 (w + 4 i) + l / 8.  Rows past the matrix edge
  // re-read the last row (their results are never stored).
  //
  // Issuing a DMA costs no vector ALU work inside the loop: the address is
  // a wave-uniform base (tile origin + slice offset, scalar registers) plus
  // a per-lane 32-bit offset computed once here, and the LDS destination
  // (M0) is derived from the wave-uniform wave id.  When K has a tail, the
  // last slice uses a second offset set in which chunks past the end of K
  // point at the row's first chunk (a valid address); fragments of such
  // chunks are zeroed when read.
  const uint8_t* a_tile = A + static_cast<int64_t>(m_blk) * lda;
  const uint8_t* b_tile = B + static_cast<int64_t>(n_blk) * ldb;
  const uint8_t* b2_tile = GATED ? epi.B2 + static_cast<int64_t>(n_blk) * epi.ldb2 : nullptr;
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  // B DMA instruction i of wave w covers B-tile rows 8 (w + 4 i) .. + 7: a
  // block of one matrix (gate or up) only, since 8 TN is a multiple of 8.
  // Its base (wave-uniform) and the feature of its first row:
  auto b_block = [&](int i, bool& up, int& feat) {
    const int row0 = 8 * (wid_u + 4 * i);
    if constexpr (GATED) {
      const int w = row0 % kWN;
      up = w >= kWN / 2;
      feat = (row0 / kWN) * (kWN / 2) + (up ? w - kWN / 2 : w);
    } else {
      up = false;
      feat = row0;
    }
  };
  const int dma_ch = (lane & 7) ^ (lane >> 3);
  const int nk = (Kb + kBK - 1) / kBK;
  const int k_last = (nk - 1) * kBK;
  uint32_t dma_off[kDmas], dma_off_tail[KTAIL ? kDmas : 1];
#pragma unroll
  for (int i = 0; i < kDmas; ++i) {
    const bool is_a = i < kBM / 32;
    bool up = false;
    int feat = 0;
    if (!is_a) b_block(i - kBM / 32, up, feat);
    const int row = is_a ? 8 * (wid + 4 * i) + (lane >> 3) : feat + (lane >> 3);
    const int rows = is_a ? M - m_blk : N - n_blk;
    const int64_t ld = is_a ? lda : (up ? epi.ldb2 : ldb);
    const uint32_t row_off = static_cast<uint32_t>(min(row, rows - 1)) * static_cast<uint32_t>(ld);
    dma_off[i] = row_off + dma_ch * 16;
    if constexpr (KTAIL) dma_off_tail[i] = row_off + (k_last + dma_ch * 16 < Kb ? k_last + dma_ch * 16 : 0);
  }
  // DMA instruction number s of the slice starting at byte k0; A blocks
  // (s < kDmaA) go to A slice buffer `buf` (of 3), B blocks to B slice
  // buffer `buf` (of 2).
  auto dma_block = [&](auto s_c, int buf, int k0, auto tail_c) {
    constexpr int s = decltype(s_c)::value;
    constexpr bool kTail = decltype(tail_c)::value;
    constexpr bool kIsA = s < kDmaA;
    constexpr int kBlk = kIsA ? s : s - kDmaA;
    uint8_t* lds = smem + (kIsA ? buf * kATileBytes : kBBase + buf * kBTileBytes) + (wid_u + 4 * kBlk) * 1024;
    const uint8_t* base = a_tile;
    if constexpr (!kIsA) {
      bool up = false;
      int feat = 0;
      b_block(kBlk, up, feat);
      base = up ? b2_tile : b_tile;
    }
    if constexpr (kTail) {
      dma16(base + dma_off_tail[s], lds);
    } else {
      dma16(base + k0 + dma_off[s], lds);
    }
  };
  // DMA instructions [FIRST, LAST) of the slice at k0 (A into A buffer
  // abuf, B into B buffer bbuf).
  auto issue = [&](auto first_c, auto last_c, int abuf, int bbuf, int k0) {
    constexpr int kFirst = decltype(first_c)::value;
    constexpr int kLast = decltype(last_c)::value;
    auto all = [&](auto tail_c) {
      static_for<kLast - kFirst>([&](auto i_c) {
        constexpr int s = kFirst + decltype(i_c)::value;
        dma_block(std::integral_constant<int, s>{}, s < kDmaA ? abuf : bbuf, k0, tail_c);
      });
    };
    if constexpr (KTAIL) {
      if (k0 == k_last) all(std::true_type{}); else all(std::false_type{});
    } else {
      all(std::false_type{});
    }
  };

  acc_t acc[kTM][TN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  // The zeroing above is VALU work read by the first MFMAs.
  pad<5>();

  // Fragment addresses: row (l & 15) of each 16-row tile, chunk (l >> 4) of
  // each 64-byte K step; the swizzle term depends on the lane only.
  const int frag_row = lane & 15;
  const int frag_ch = lane >> 4;
  int frag_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) frag_off[ks] = frag_row * kBK + (((4 * ks + frag_ch) ^ (frag_row & 7)) << 4);
  const uint32_t lds0 = lds_address(smem);
  auto addr_a = [&](int buf, int ks) -> uint32_t { return lds0 + buf * kATileBytes + wm * kBK + frag_off[ks]; };
  auto addr_b = [&](int buf, int ks) -> uint32_t {
    return lds0 + kBBase + buf * kBTileBytes + wn * kBK + frag_off[ks];
  };

  // Two register sets of fragments: one feeds the MFMAs while the other is
  // being read from LDS.
  i32x4 fa0[kTM], fb0[TN], fa1[kTM], fb1[TN];
  constexpr int kReads = kTM + TN;              // fragment reads per step
  // Fragment read number s of a step into (fa, fb).
  auto read_frag = [&](auto s_c, i32x4* fa, i32x4* fb, uint32_t aa, uint32_t ab) {
    constexpr int s = decltype(s_c)::value;
    if constexpr (s < kTM) {
      lds_read16<2048 * s>(fa[s], aa);
    } else {
      lds_read16<2048 * (s - kTM)>(fb[s - kTM], ab);
    }
  };
  // One 64-byte K step: the TM x TN MFMAs on (fa, fb), with op(0..NOPS-1)
  // spread evenly over all but the last 8 MFMAs, so that LDS and DMA
  // traffic trickles out while the matrix cores are busy instead of
  // queueing in front of them, and the last read has landed by the end.
  auto mfma_step = [&](const i32x4* fa, const i32x4* fb, auto nops_c, auto&& op) {
    constexpr int kOps = decltype(nops_c)::value;
    constexpr int kM = kTM * TN;
    constexpr int kSpread = kM - 8;
    static_assert(kOps <= kSpread, "more side operations than MFMA slots");
    static_for<kM>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      // Ops s with floor(s * kSpread / kOps) == m go right before MFMA m.
      constexpr int first = (m * kOps + kSpread - 1) / kSpread;
      constexpr int next = ((m + 1) * kOps + kSpread - 1) / kSpread;
      constexpr int count = (first < kOps ? (next < kOps ? next : kOps) - first : 0);
      static_for<count>([&](auto c_c) { op(std::integral_constant<int, first + decltype(c_c)::value>{}); });
      Op::run(acc[m / TN][m % TN], fb[m % TN], fa[m / TN]);
    });
  };
  auto tail_mask = [&](i32x4* fb, int k0, int ks) {
    if constexpr (KTAIL) mask_tail<TN>(fb, k0 + (4 * ks + frag_ch) * 16 >= Kb);
  };
  using no_ops = std::integral_constant<int, 0>;
  using read_ops = std::integral_constant<int, kReads>;
  using dma_read_ops = std::integral_constant<int, kDmas + kReads>;

  // Pipeline per 128-byte slice kt (two 64-byte steps).  Slice kt lives in
  // A buffer kt % 3 and B buffer kt % 2.  The vector-memory path moves at
  // most ~36 bytes per clock into a CU's LDS, so each phase carries half of
  // a slice's DMA: the A part of slice kt+2 in phase 1, the B part in
  // phase 2 (a 256 x 256 tile moves 32 KiB per phase, 32 bytes per clock at
  // the MFMA rate).  The third A buffer is what lets A go out a phase early.
  //   phase 1: MFMAs on set 0 | DMA A(kt+2) into A buffer (kt+2) % 3,
  //            reads of set 1 (slice kt, step 1)
  //   wait for own LDS reads and for own DMAs up to B(kt+1) (A(kt+2) may
  //   still fly); barrier
  //   phase 2: MFMAs on set 1 | DMA B(kt+2) into B buffer kt % 2, reads of
  //            set 0 (slice kt+1, step 0)
  // A buffer is refilled only after the barrier that follows the last read
  // of its previous slice: A buffer (kt+2) % 3 held slice kt-1 (last read
  // before barrier kt-1), B buffer kt % 2 holds slice kt (last read before
  // barrier kt).  Every slice runs the same code: DMAs of slices past the
  // end are skipped by uniform branches, and the reads that would feed
  // slice nk fetch stale LDS data that no MFMA uses.  The loop has one entry
  // and one exit: the MFMAs are opaque to the compiler, and a second path
  // into the epilogue would let it place accumulator copies right behind
  // the last MFMAs, before the hazard padding.
  using dma_a = std::integral_constant<int, 0>;
  using dma_mid = std::integral_constant<int, kDmaA>;
  using dma_end = std::integral_constant<int, kDmas>;
  issue(dma_a{}, dma_end{}, 0, 0, 0);
  if (nk > 1) issue(dma_a{}, dma_end{}, 1, 1, kBK);
  if (nk > 1) wait_vm<kDmas>(); else wait_vm<0>();
  wait_lds();
  barrier();
  static_for<kReads>([&](auto s_c) { read_frag(s_c, fa0, fb0, addr_a(0, 0), addr_b(0, 0)); });

  int kt = 0;
  int a_cur = 0;  // kt % 3
  do {
    const int b_cur = kt & 1;
    const int a_next = a_cur == 2 ? 0 : a_cur + 1;    // (kt+1) % 3
    const int a_after = a_next == 2 ? 0 : a_next + 1;  // (kt+2) % 3
    const int k0 = kt * kBK;
    const bool dma = kt + 2 < nk;
    wait_lds();
    tail_mask(fb0, k0, 0);
    {
      const uint32_t aa = addr_a(a_cur, 1), ab = addr_b(b_cur, 1);
      mfma_step(fa0, fb0, std::integral_constant<int, kDmaA + kReads>{}, [&](auto s_c) {
        constexpr int o = decltype(s_c)::value;
        if constexpr (o < kDmaA) {
          if (dma) {
            if constexpr (KTAIL) {
              if (k0 + 2 * kBK == k_last) {
                dma_block(s_c, a_after, k0 + 2 * kBK, std::true_type{});
              } else {
                dma_block(s_c, a_after, k0 + 2 * kBK, std::false_type{});
              }
            } else {
              dma_block(s_c, a_after, k0 + 2 * kBK, std::false_type{});
            }
          }
        } else {
          read_frag(std::integral_constant<int, o - kDmaA>{}, fa1, fb1, aa, ab);
        }
      });
    }
    // The operands of the last MFMAs may still be being read: release the
    // set's registers only after enough wait states (see keep_live).
    pad<16>();
    keep_live(fa0);
    keep_live(fb0);
    if (dma) wait_vm<kDmaA>(); else wait_vm<0>();
    wait_lds();
    barrier();
    tail_mask(fb1, k0, 1);
    {
      const uint32_t aa = addr_a(a_next, 0), ab = addr_b(b_cur ^ 1, 0);
      mfma_step(fa1, fb1, std::integral_constant<int, kDmas - kDmaA + kReads>{}, [&](auto s_c) {
        constexpr int o = decltype(s_c)::value;
        if constexpr (o < kDmas - kDmaA) {
          if (dma) {
            using blk = std::integral_constant<int, kDmaA + o>;
            if constexpr (KTAIL) {
              if (k0 + 2 * kBK == k_last) {
                dma_block(blk{}, b_cur, k0 + 2 * kBK, std::true_type{});
              } else {
                dma_block(blk{}, b_cur, k0 + 2 * kBK, std::false_type{});
              }
            } else {
              dma_block(blk{}, b_cur, k0 + 2 * kBK, std::false_type{});
            }
          }
        } else {
          read_frag(std::integral_constant<int, o - (kDmas - kDmaA)>{}, fa0, fb0, aa, ab);
        }
      });
    }
    pad<16>();
    keep_live(fa1);
    keep_live(fb1);
    a_cur = a_next;
    ++kt;
  } while (kt < nk);
  // The last reads fetched nothing that is used; let them retire.  Their
  // destination registers stay allocated until the wait has passed, so that
  // no epilogue value is placed in a register an LDS read is still writing.
  sched_fence();
  wait_lds();
  sched_fence();
  keep_live(fa0);
  keep_live(fb0);
  keep_live(fa1);
  keep_live(fb1);
  // MFMA results are read below by ordinary instructions: wait out the
  // longest MFMA write latency first.  The empty statements then redefine
  // every accumulator after the padding, so no copy of one (which the
  // register allocator is free to place anywhere after its last write) can
  // read an MFMA result before it is complete.
  pad<24>();
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) touch_acc(acc[i][j]);

  // Epilogue.  Lane holds, for tile (i, j), output row m = m0 + 16 i + (l & 15)
  // and the four consecutive output features n = n0 + 16 j + 4 (l >> 4) + r
  // (for the gated pair, tiles j and j + TN/2 are the gate and up results of
  // the same features).  Every scale and bias it needs is requested first,
  // in one batch (16-byte loads where the columns allow), so the tile pays
  // one memory round trip.
  const int n_lane = 4 * (lane >> 4);
  float s_row[kTM];
  f32x4 s_col[kTNo], b_col[kTNo], s_col2[GATED ? kTNo : 1], b_col2[GATED ? kTNo : 1];
  if constexpr (OUT != 2) {
    auto col_loads = [&](const float* s, const float* b, f32x4* sc, f32x4* bc) {
      if (vec_cols && n_blk + kBNo <= N) {  // uniform: the whole tile is inside N
#pragma unroll
        for (int j = 0; j < kTNo; ++j) {
          const int n = n_blk + wno + 16 * j + n_lane;
          sc[j] = I8 ? *reinterpret_cast<const f32x4*>(s + n) : f32x4{1.f, 1.f, 1.f, 1.f};
          bc[j] = b ? *reinterpret_cast<const f32x4*>(b + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      } else {
#pragma unroll
        for (int j = 0; j < kTNo; ++j) {
          const int n = n_blk + wno + 16 * j + n_lane;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int nn = min(n + r, N - 1);
            sc[j][r] = I8 ? s[nn] : 1.f;
            bc[j][r] = b ? b[nn] : 0.f;
          }
        }
      }
    };
    col_loads(sb, bias, s_col, b_col);
    if constexpr (GATED) col_loads(epi.sb2, epi.bias2, s_col2, b_col2);
#pragma unroll
    for (int i = 0; i < kTM; ++i) s_row[i] = I8 ? sa[min(m_blk + wm + 16 * i + frag_row, M - 1)] : 1.f;
  }
  // Output value r of tile (i, j), j < kTNo.
  auto value = [&](int i, int j, int r) -> float {
    float y;
    if constexpr (I8) {
      y = fmaf(static_cast<float>(acc[i][j][r]), s_row[i] * s_col[j][r], b_col[j][r]);
    } else {
      y = acc[i][j][r] + b_col[j][r];
    }
    if constexpr (GATED) {
      const float u = fmaf(static_cast<float>(acc[i][j + kTNo][r]), s_row[i] * s_col2[j][r], b_col2[j][r]);
      return activation<ACT>(y) * u;
    } else {
      return activation<ACT>(y);
    }
  };
  // fp32 / bf16 outputs leave through LDS when the destination allows
  // 16-byte stores: each wave writes one 16-row block of its results into a
  // private, padded LDS area and reads it back as 16-byte chunks, so that
  // consecutive lanes store consecutive bytes of an output row (whole cache
  // lines) instead of 32-byte pieces of 16 different rows.
  if constexpr (OUT != 2) {
    if (staged) {
      using out_t = typename std::conditional<OUT == 0, float, __bf16>::type;
      constexpr int kElt = sizeof(out_t);
      constexpr int kRowBytes = 16 * kTNo * kElt;  // one row of the wave's block
      constexpr int kPitch = kRowBytes + 32;       // padding spreads rows over banks
      constexpr int kSegs = kRowBytes / 16;        // 16-byte chunks per row
      constexpr int kChunks = 16 * kSegs;          // per 16-row block
      __syncthreads();  // every wave is done reading the slice buffers
      uint8_t* stage = smem + wid * 16 * kPitch;
      constexpr int kPasses = (kChunks + 63) / 64;
      const bool full = m_blk + kBM <= M && n_blk + kBNo <= N;  // uniform
      // Lane l's store of pass p in 16-row block 0 (blocks follow at
      // block_stride bytes).
      uint8_t* pass_base[kPasses];
      const int64_t block_stride = 16 * ldc * kElt;
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int c = min(64 * p + lane, kChunks - 1);
        const int row = c / kSegs, seg = c % kSegs;
        pass_base[p] = static_cast<uint8_t*>(C) +
                       (static_cast<int64_t>(m_blk + wm + row) * ldc + n_blk + wno) * kElt + seg * 16;
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int j = 0; j < kTNo; ++j) {
          float y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = value(i, j, r);
          uint8_t* dst = stage + frag_row * kPitch + (16 * j + n_lane) * kElt;
          if constexpr (OUT == 0) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{y[0], y[1], y[2], y[3]};
          } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<bf16x4*>(dst) = bf16x4{static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1]),
                                                     static_cast<__bf16>(y[2]), static_cast<__bf16>(y[3])};
          }
        }
        if (full) {
          // Whole tile inside the output: no bound checks, addresses step by
          // a uniform 16-row stride from the per-pass bases.
#pragma unroll
          for (int p = 0; p < kPasses; ++p) {
            const int c = 64 * p + lane;
            if (kChunks % 64 == 0 || c < kChunks) {
              const int row = c / kSegs, seg = c % kSegs;
              const i32x4 v = *reinterpret_cast<const i32x4*>(stage + row * kPitch + seg * 16);
              *reinterpret_cast<i32x4*>(pass_base[p] + static_cast<int64_t>(i) * block_stride) = v;
            }
          }
          continue;
        }
#pragma unroll
        for (int c0 = 0; c0 < kChunks; c0 += 64) {
          const int c = c0 + lane;
          if (kChunks % 64 == 0 || c < kChunks) {
            const int row = c / kSegs, seg = c % kSegs;
            const i32x4 v = *reinterpret_cast<const i32x4*>(stage + row * kPitch + seg * 16);
            const int m = m_blk + wm + 16 * i + row;
            const int n = n_blk + wno + seg * (16 / kElt);
            if (m < M) {
              out_t* out = static_cast<out_t*>(C) + static_cast<int64_t>(m) * ldc + n;
              if (n + 16 / kElt <= N) {
                *reinterpret_cast<i32x4*>(out) = v;
              } else {
                // ragged right edge: element r of the 16-byte piece, taken
                // with shifts (taking the vector's address would place it in
                // scratch memory for every piece, not only the ragged ones)
                for (int r = 0; r < 16 / kElt && n + r < N; ++r) {
                  if constexpr (OUT == 0) {
                    reinterpret_cast<int32_t*>(out)[r] = v[r];
                  } else {
                    reinterpret_cast<uint16_t*>(out)[r] = static_cast<uint16_t>(v[r >> 1] >> (16 * (r & 1)));
                  }
                }
              }
            }
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < kTNo; ++j) {
    const int n = n_blk + wno + 16 * j + n_lane;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int m = m_blk + wm + 16 * i + frag_row;
      if (m >= M) continue;
      if constexpr (OUT == 2) {
        const acc_t a = acc[i][j];
        int32_t* out = static_cast<int32_t*>(C) + static_cast<int64_t>(m) * ldc + n;
        if (n + 3 < N && vec_ok(out)) {
          *reinterpret_cast<i32x4*>(out) = a;
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) out[r] = a[r];
        }
      } else {
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = value(i, j, r);
        if constexpr (OUT == 0) {
          float* out = static_cast<float*>(C) + static_cast<int64_t>(m) * ldc + n;
          if (n + 3 < N && vec_ok(out)) {
            *reinterpret_cast<f32x4*>(out) = f32x4{y[0], y[1], y[2], y[3]};
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) out[r] = y[r];
          }
        } else {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          __bf16* out = static_cast<__bf16*>(C) + static_cast<int64_t>(m) * ldc + n;
          if (n + 3 < N && vec_ok(out)) {
            *reinterpret_cast<bf16x4*>(out) =
                bf16x4{static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1]), static_cast<__bf16>(y[2]),
                       static_cast<__bf16>(y[3])};
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) out[r] = static_cast<__bf16>(y[r]);
          }
        }
      }
    }
  }
}

inline int num_cus() { return device_cus(); }

// Output-tile width: the candidate minimising (rounds of one tile per CU) x
// (work per tile), i.e. the fewest idle CU-slots in the last round; ties go
// to the wider tile (less LDS traffic per MFMA).  `cols` counts B-tile
// columns (2 N for a gated pair).
inline int choose_tn(int64_t M, int64_t cols) {
  // CONVROT_GEMM_TN=4|6|8 pins the width (tuning and checking only).
  static const int forced = [] {
    const char* e = std::getenv("CONVROT_GEMM_TN");
    const int v = e ? std::atoi(e) : 0;
    return (v == 4 || v == 6 || v == 8) ? v : 0;
  }();
  if (forced) return forced;
  const int cands[] = {8, 6, 4};
  const int64_t cus = num_cus();
  int best = 8;
  int64_t best_cost = -1;
  for (int tn : cands) {
    const int64_t bn = 32 * tn;
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((cols + bn - 1) / bn);
    const int64_t cost = ((tiles + cus - 1) / cus) * bn;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = tn;
    }
  }
  return best;
}

template <bool I8, int OUT, bool KTAIL, int TN, int ACT, bool GATED>
hipError_t launch_typed(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const EpiArgs& epi, int64_t M,
                        int64_t N, int64_t Kb, void* C, int64_t ldc, hipStream_t stream) {
  auto kern = gemm_nt_kernel<I8, OUT, KTAIL, TN, ACT, GATED>;
  constexpr int kSmem = smem_bytes<TN>();
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kern), kSmem, lds_set);
  if (e != hipSuccess) return e;
  constexpr int kBNo = GATED ? 16 * TN : 32 * TN;
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBNo - 1) / kBNo);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
  // 16-byte scale/bias loads need 16-byte aligned vectors.
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec_cols = al16(epi.sb) && al16(epi.bias) && (!GATED || (al16(epi.sb2) && al16(epi.bias2)));
  // Staged stores need 16-byte aligned output rows.
  const int out_elt = OUT == 1 ? 2 : 4;
  const bool staged = al16(C) && (ldc * out_elt) % 16 == 0;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), kSmem, stream, A, lda, B, ldb, epi, static_cast<int>(M),
                     static_cast<int>(N), static_cast<int>(Kb), C, ldc, tiles_m, tiles_n, vec_cols, staged);
  return hipGetLastError();
}

template <bool I8, int OUT, int ACT, bool GATED>
hipError_t launch_gemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const EpiArgs& epi, int64_t M,
                       int64_t N, int64_t Kb, void* C, int64_t ldc, hipStream_t stream) {
  const int tn = choose_tn(M, GATED ? 2 * N : N);
  const bool tail = Kb % kBK != 0;
#define CONVROT_GEMM_CASE(TN_)                                                                             \
  case TN_:                                                                                                \
    return tail ? launch_typed<I8, OUT, true, TN_, ACT, GATED>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream) \
                : launch_typed<I8, OUT, false, TN_, ACT, GATED>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream);
  switch (tn) {
    CONVROT_GEMM_CASE(6)
    CONVROT_GEMM_CASE(4)
    default:
      CONVROT_GEMM_CASE(8)
  }
#undef CONVROT_GEMM_CASE
}

}  // namespace
}  // namespace convrot
