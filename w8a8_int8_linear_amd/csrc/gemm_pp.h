// Eight-wave "ping-pong" matrix-core GEMM for gfx950: C = A B^T, both
// operands K-contiguous, fused scale/bias (and activation) epilogue.  Same
// operation, modes and result bits as gemm_nt_kernel (gemm_kernel.h); it
// runs every linear with whole 128-byte K slices (the four-wave kernel keeps
// K tails and the gated pair).
//
// Why eight waves.  A wave issues in order, and a global -> LDS transfer
// (global_load_lds_dwordx4, 1 KiB) holds its wave's issue for about 50
// cycles, so MFMAs interleaved with transfers in one wave leave the matrix
// core idle a third of the time.  Transfers and LDS reads issued by
// *another* wave on the same SIMD do not slow that wave's MFMAs at all.  So
// each SIMD runs two waves that take turns: while one issues its memory
// phase (its share of the transfers and the LDS reads of its next
// fragments), the other runs a compute phase of MFMAs on fragments already
// in registers, and a workgroup barrier swaps the roles.  The second group
// starts one phase late (one extra barrier) and so stays a phase behind.
//
// Shapes.  Workgroup tile 256 (A rows, tokens) x 64 TN (B rows, features),
// TN in {2, 3, 4}; 8 waves, wave w owning tokens 64 (w % 4) .. + 63 and B
// rows 32 TN (w / 4) .. + 32 TN - 1, i.e. 4 x 2 TN MFMA tiles of 16 x 16
// (v_mfma_i32_16x16x64_i8, or v_mfma_f32_16x16x32_bf16 in bf16 mode; both
// take 16 bytes of K per lane and operand).  That is at most 128
// accumulators per lane, so two waves fit on a SIMD.  The 16 x 16 x 64
// form is used rather than 32 x 32 x 32 because on random int8 operands it
// runs at a higher clock under the power limit (2.06 against 1.68 GHz
// at the same utilisation): less energy per operation.
//
// Data movement.  K advances in 128-byte slices ([rows][128 B], 16-byte
// chunks XOR-swizzled by row & 7); one slice is two 64-byte steps, one step
// per memory/compute phase pair.  LDS holds three A slices and two B
// slices.  In the period of slice p each wave issues the B part of slice
// p + 1 in its first memory phase and the A part of slice p + 2 in its
// second, so every transfer has at least two phases to land; each wave
// waits for its own transfers (vmcnt) before the barrier that publishes
// them.  A buffer (p + 2) % 3 and B buffer (p + 1) % 2 held slices p - 1,
// whose last reads precede the barrier that opens period p.
//
// Epilogue.  Weights are the MFMA "row" operand, so each lane's four
// accumulators of a tile hold four consecutive output features of one
// token.  Scales and biases are loaded before the main loop.  The raw
// accumulators of each 16-token tile are staged as rows (16-byte chunks
// XOR-swizzled by row) in a private LDS area per wave and read back so
// that each lane finishes fixed 4-feature segments (conversion, both
// scales, bias, activation; the row scale taken from the lane that holds
// it) and stores whole row pieces (with the non-temporal hint when the
// output is larger than the 256 MB Infinity Cache).
//
// Walk.  The grid is one workgroup per CU; each takes every gridDim.x-th
// tile of an XCD-ordered tile list, and requests the next tile's scales
// and first slices before its current tile's epilogue.  With int8
// operands every other round runs K last slice first, so that it starts on
// the slices of the row group's A panels that the round before left in the
// XCD's L2.
//
// Producer fusion (ROWMAX, 256-wide tiles): the epilogue also computes, for
// the next layer's pack, the largest magnitude of every G-group (G <= 256)
// of each output row after the regular rotation R_G, from the output as
// stored.  The two waves that share 64 tokens (w and w + 4) stage their
// halves of the tile into one area, so that each finishes 16 whole
// 256-feature rows per 32 tokens, four features per lane.  The group's
// base-4 digits are the element (digit 0), lane bits 0-1 (digit 1) and the
// Gray codes of lane bits 2-3 and 4-5 (digits 2 and 3), so that every lane
// exchange of the rotation is the one the pack kernel uses (quad and row
// DPP, the 16- and 32-lane swizzles); the rotation takes the pack kernel's
// operations in the pack kernel's order (lanes.h), so the maxima equal the
// pack's own bit for bit.
#pragma once
#include "gemm_kernel.h"
#include "lanes.h"

namespace convrot {
namespace {

constexpr int kPPThreads = 512;

// Largest power of two dividing both v and 64.
constexpr int gcd_pow2_64(int v) { return (v & -v) < 64 ? (v & -v) : 64; }

template <int TN>
constexpr int pp_smem_bytes() {
  return 3 * kATileBytes + 2 * (64 * TN) * kBK;
}

// First of the four features lane l finishes in the ROWMAX epilogue: digit
// 1 of the feature index is lane bits 0-1, digits 2 and 3 the Gray codes of
// lane bits 2-3 and 4-5.
__device__ __forceinline__ int rowmax_col(int lane) {
  const int m2 = (lane >> 2) & 3, m3 = lane >> 4;
  return 4 * ((lane & 3) + 4 * (m2 ^ (m2 >> 1)) + 16 * (m3 ^ (m3 >> 1)));
}

// OUT: 0 = fp32, 1 = bf16, 2 = raw int32 accumulator (int8 mode only).
// ACT: epilogue activation (see activation() in epilogue.h).
// STREAM: output stores with the non-temporal hint (see launch_pp_typed).
template <bool I8, int OUT, int TN, int ACT, bool ROWMAX = false, bool STREAM = false>
__global__ __launch_bounds__(kPPThreads, 1) void gemm_pp_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, EpiArgs epi, int M,
    int N, int Kb, void* __restrict__ C, int64_t ldc, int tiles_m, int tiles_n, bool vec_cols, bool vec_out,
    RowmaxArgs rm) {
  static_assert(TN >= 2 && TN <= 4, "tile width");
  static_assert(I8 || OUT != 2, "raw accumulators are an int8 feature");
  static_assert(ACT == 0 || OUT != 2, "activations need a float output");
  static_assert(!ROWMAX || (TN == 4 && OUT != 2), "group maxima need 256-wide tiles and a float output");
  constexpr int kBN = 64 * TN;          // B-tile rows (output features)
  constexpr int kWN = 32 * TN;          // B rows per wave
  constexpr int kBTileBytes = kBN * kBK;
  constexpr int kBBase = 3 * kATileBytes;
  constexpr int kDmaA = kBM / 64;       // 1 KiB transfers per wave and slice: A part
  constexpr int kDmaB = kBN / 64;       // and B part
  static_assert(pp_smem_bytes<TN>() <= 160 * 1024, "LDS budget");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using Op = Mfma<I8>;
  using acc_t = typename Op::acc_t;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int grp = wid >> 2;            // 0: leads, 1: one phase behind
  const int wm = (wid & 3) * 64;       // tokens of the wave within the tile
  const int wn = grp * kWN;            // features of the wave within the tile
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const int grp_u = wid_u >> 2;
  const int total = tiles_m * tiles_n;
  const int nk = Kb / kBK;

  // Transfers: instruction i of wave w fills 1 KiB block w + 8 i of a slice
  // (8 rows; lane l writes physical chunk l % 8 of row l / 8, which holds
  // logical chunk (l % 8) ^ (l / 8)).  Rows past the matrix edge re-read
  // the last row; their results are never stored.
  const int dma_ch = (lane & 7) ^ (lane >> 3);
  // Per-tile state: the tile's corner, the operand panels and each lane's
  // transfer offsets within them.
  struct Tile {
    int m_blk, n_blk;
    const uint8_t* a;
    const uint8_t* b;
    uint32_t off_a[kDmaA], off_b[kDmaB];
    int kstep;  // bytes from one slice to the next: kBK, or -kBK when the tile runs K backwards
  };
  auto tile_at = [&](int id, Tile& T) {
    int tm, tn;
    tile_coords(id, tiles_m, tiles_n, tm, tn);
    // int8: every other round of the walk runs K backwards, so that it
    // starts on the slices the previous round (same row group on this XCD)
    // left in L2.  Exact integer sums do not depend on the order; float
    // sums keep one order so that their bits match the other kernels'.
    const bool rev = I8 && ((id / gridDim.x) & 1);
    const int k0 = rev ? (nk - 1) * kBK : 0;
    T.kstep = rev ? -kBK : kBK;
    T.m_blk = tm * kBM;
    T.n_blk = tn * kBN;
    T.a = A + static_cast<int64_t>(T.m_blk) * lda + k0;
    T.b = B + static_cast<int64_t>(T.n_blk) * ldb + k0;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
      const int row = 8 * (wid + 8 * i) + (lane >> 3);
      T.off_a[i] = static_cast<uint32_t>(min(row, M - T.m_blk - 1)) * static_cast<uint32_t>(lda) + dma_ch * 16;
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      const int row = 8 * (wid + 8 * i) + (lane >> 3);
      T.off_b[i] = static_cast<uint32_t>(min(row, N - T.n_blk - 1)) * static_cast<uint32_t>(ldb) + dma_ch * 16;
    }
  };
  auto dma_a = [&](const Tile& T, int slice, int buf) {
    const uint8_t* g = T.a + slice * T.kstep;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) dma16(g + T.off_a[i], smem + buf * kATileBytes + (wid_u + 8 * i) * 1024);
  };
  auto dma_b = [&](const Tile& T, int slice, int buf) {
    const uint8_t* g = T.b + slice * T.kstep;
#pragma unroll
    for (int i = 0; i < kDmaB; ++i)
      dma16(g + T.off_b[i], smem + kBBase + buf * kBTileBytes + (wid_u + 8 * i) * 1024);
  };

  // Fragment reads: lane l takes row l % 16 of a 16-row tile and 16-byte
  // chunk l / 16 of the 64-byte K step; step s of a slice is chunks 4 s ..
  // 4 s + 3.  The swizzle depends on the lane only, so there is one base
  // address per step and operand; tiles are immediate offsets (16 rows =
  // 2 KiB).
  const int frow = lane & 15;
  const int fk = lane >> 4;
  const uint32_t lds0 = lds_address(smem);
  uint32_t base_a[2], base_b[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t off = frow * kBK + (((4 * st + fk) ^ (frow & 7)) << 4);
    base_a[st] = lds0 + wm * kBK + off;
    base_b[st] = lds0 + kBBase + wn * kBK + off;
  }

  constexpr int kTF = 2 * TN;  // 16-feature tiles per wave
  acc_t acc[4][kTF];
  auto zero_acc = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int f = 0; f < kTF; ++f) acc[t][f] = acc_t{};
    pad<5>();  // the zeroing is VALU work read by the first MFMAs
  };

  // One fragment set: a wave reads it in a memory phase and consumes it in
  // the next phase; the overlap comes from the other wave on the SIMD.
  i32x4 fa[4], fb[kTF];
  auto read_step = [&](int st, int abuf, int bbuf) {
    const uint32_t aa = base_a[st] + abuf * kATileBytes, ab = base_b[st] + bbuf * kBTileBytes;
    static_for<4>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      lds_read16<2048 * t>(fa[t], aa);
    });
    static_for<kTF>([&](auto f_c) {
      constexpr int f = decltype(f_c)::value;
      lds_read16<2048 * f>(fb[f], ab);
    });
  };
  auto compute_step = [&]() {
    static_for<4>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      static_for<kTF>([&](auto f_c) {
        constexpr int f = decltype(f_c)::value;
        Op::run(acc[t][f], fb[f], fa[t]);
      });
    });
    // Keep the fragment registers allocated up to here: the MFMAs are opaque
    // to the compiler, which must not hand their source registers to a
    // temporary while they may still be read.  (The next writes to them are
    // LDS reads behind a barrier; the accumulators, read as SrcC, are only
    // touched again after the padding in front of the epilogue.)
    keep_live(fa);
    keep_live(fb);
  };

  // Epilogue operands of a tile, requested well before its epilogue (the
  // first tile's before its main loop, every later tile's before the
  // previous tile's epilogue).  Per lane: the row scale of its four tokens
  // (MFMA layout, token = l % 16 of each 16-token tile), and the column
  // scales and biases of the 4-feature output segments it finishes (row
  // layout, see the epilogue).
  constexpr int kSegs = kWN / 4;                       // 4-feature segments per wave row
  constexpr int kLaneSegs = kSegs / gcd_pow2_64(kSegs);  // distinct segments per lane
  struct Scales {
    float row[4];
    f32x4 col[kLaneSegs], bias[kLaneSegs];
  };
  auto load_scales = [&](const Tile& T, Scales& S) {
#pragma unroll
    for (int t = 0; t < 4; ++t) S.row[t] = 1.f;
    if constexpr (OUT != 2) {
      if constexpr (I8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) S.row[t] = epi.sa[min(T.m_blk + wm + 16 * t + frow, M - 1)];
      }
#pragma unroll
      for (int j = 0; j < kLaneSegs; ++j) {
        // (ROWMAX: the lane finishes 4 features of the whole tile, see rowmax_col)
        const int n = ROWMAX ? T.n_blk + rowmax_col(lane) : T.n_blk + wn + 4 * ((64 * j + lane) % kSegs);
        const bool vec = vec_cols && T.n_blk + kBN <= N;
        auto load4 = [&](const float* v, float dflt) -> f32x4 {
          if (v == nullptr) return f32x4{dflt, dflt, dflt, dflt};
          if (vec) return *reinterpret_cast<const f32x4*>(v + n);
          f32x4 r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = v[min(n + i, N - 1)];
          return r;
        };
        S.col[j] = I8 ? load4(epi.sb, 1.f) : f32x4{1.f, 1.f, 1.f, 1.f};
        S.bias[j] = load4(epi.bias, 0.f);
      }
    }
  };

  // Persistent walk: this workgroup takes tiles blockIdx.x, + gridDim.x, ...
  // of the XCD-ordered list (a grid of one workgroup per tile runs the body
  // once).  Before a tile's epilogue the next tile's scales and first three
  // slices (A 0, A 1 and B 0, buffers no wave reads any more once the main
  // loop has passed its last barrier) are requested, so their latency hides
  // behind the epilogue, whose staging uses A buffer 2 and B buffer 1 only.
  // The ROWMAX epilogue stages through most of LDS, and the raw int32
  // output (a checking mode) would spill registers holding the next tile's
  // state; both take one tile per workgroup.
  constexpr bool kPrefetch = !ROWMAX && OUT != 2;
  int tile = blockIdx.x;
  Tile cur;
  tile_at(tile, cur);
  Scales sc;
  load_scales(cur, sc);
  zero_acc();
  dma_a(cur, 0, 0);
  dma_b(cur, 0, 0);
  if (nk > 1) dma_a(cur, 1, 1);
  if (nk > 1) wait_vm<kDmaA>(); else wait_vm<0>();
  barrier();
  if (grp_u == 1) barrier();  // the second group runs one phase behind

  while (true) {
    int p = 0;
    int a_cur = 0;  // p % 3
    do {
      const int b_cur = p & 1;
      const int a_next = a_cur == 2 ? 0 : a_cur + 1;
      const int a_after = a_next == 2 ? 0 : a_next + 1;  // (p + 2) % 3
      // memory phase: fragments of step 0 of slice p, then the B part of
      // slice p + 1 (LDS reads queued behind transfers wait for them; in
      // this order the transfers issue while the reads are in flight)
      read_step(0, a_cur, b_cur);
      if (p + 1 < nk) dma_b(cur, p + 1, b_cur ^ 1);
      wait_lds();
      barrier();
      compute_step();
      barrier();
      // memory phase: fragments of step 1 of slice p, then the A part of
      // slice p + 2; every transfer but that A part must have landed before
      // the barrier
      read_step(1, a_cur, b_cur);
      if (p + 2 < nk) dma_a(cur, p + 2, a_after);
      if (p + 2 < nk) wait_vm<kDmaA>(); else wait_vm<0>();
      wait_lds();
      barrier();
      compute_step();
      if (grp_u == 0 || p + 1 < nk) barrier();
      a_cur = a_next;
      ++p;
    } while (p < nk);

    // MFMA results are read below by ordinary instructions: wait out the
    // longest MFMA write latency, then redefine every accumulator so no copy
    // of one can be placed before the padding.
    pad<24>();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int f = 0; f < kTF; ++f) touch_acc(acc[t][f]);

    const int next = tile + static_cast<int>(gridDim.x);
    const bool more = kPrefetch && next < total;  // uniform
    Tile nxt = cur;
    Scales sc_next = sc;
    if (more) {
      tile_at(next, nxt);
      load_scales(nxt, sc_next);
      dma_a(nxt, 0, 0);
      dma_b(nxt, 0, 0);
      if (nk > 1) dma_a(nxt, 1, 1);
    }

    const int m_blk = cur.m_blk, n_blk = cur.n_blk;
    const float* s_row = sc.row;
    const f32x4* s_col = sc.col;
    const f32x4* b_col = sc.bias;
    // Epilogue.  Lane l holds, for tile (t, f), token m = m0 + 16 t + l % 16
    // and features n = n0 + 16 f + 4 (l / 16) + r, r = 0..3.
    const int n_lane = 4 * fk;
    if constexpr (OUT == 2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m_blk + wm + 16 * t + frow;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < kTF; ++f) {
          const int n = n_blk + wn + 16 * f + n_lane;
          int32_t* out = static_cast<int32_t*>(C) + static_cast<int64_t>(m) * ldc + n;
          const i32x4 a = acc[t][f];
          if (n + 3 < N && vec_ok(out)) {
            *reinterpret_cast<i32x4*>(out) = a;
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) out[r] = a[r];
          }
        }
      }
    } else if constexpr (ROWMAX) {
      using namespace lanes;
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      constexpr int kRowPitch = kBN * 4 + 16;  // a staged row of the whole tile + its scale, padded across banks
      static_assert(4 * 32 * kRowPitch <= pp_smem_bytes<TN>(), "pair staging area");
      uint8_t* pst = smem + (wid & 3) * 32 * kRowPitch;  // shared by waves w and w + 4
      const int lg = rm.log2g;
      const float norm = __builtin_ldexpf(1.0f, -(lg / 2));
      const int col = rowmax_col(lane);
      const int n_seg = n_blk + col;
  #pragma unroll
      for (int u = 0; u < 2; ++u) {
        // Stage tokens 32 u .. 32 u + 31 of the pair: this wave's 128
        // features of each row, at column wn (every slice read of every wave
        // finished before the loop's last barrier; the previous pass over
        // this area finished before the barrier that ends it).
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 2 * u + h;
          uint8_t* row_ptr = pst + (16 * h + frow) * kRowPitch;
  #pragma unroll
          for (int f = 0; f < kTF; ++f) *reinterpret_cast<acc_t*>(row_ptr + (wn + 16 * f + n_lane) * 4) = acc[t][f];
          if (grp == 0 && fk == 0) *reinterpret_cast<float*>(row_ptr + kBN * 4) = s_row[t];
        }
        wait_lds();
        barrier();  // both halves of every staged row are in place
        // This wave finishes rows 16 grp .. 16 grp + 15 of the 32.
  #pragma unroll 2
        for (int pr = 0; pr < 16; ++pr) {
          const int r = 16 * grp + pr;
          const acc_t a = *reinterpret_cast<const acc_t*>(pst + r * kRowPitch + col * 4);
          const float sr = *reinterpret_cast<const float*>(pst + r * kRowPitch + kBN * 4);
          float y[4];
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = static_cast<float>(a[q]);
            const float z = I8 ? fmaf(v, sr * s_col[0][q], b_col[0][q]) : v + b_col[0][q];
            y[q] = activation<ACT>(z);
          }
          const int m = m_blk + wm + 32 * u + r;
          // the output as stored, the values the next pack reads
          float hv[4];
          if constexpr (OUT == 0) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = y[q];
            if (m < M)
              *reinterpret_cast<f32x4*>(static_cast<float*>(C) + static_cast<int64_t>(m) * ldc + n_seg) =
                  f32x4{y[0], y[1], y[2], y[3]};
          } else {
            const bf16x2 lo = __builtin_convertvector((f32x2{y[0], y[1]}), bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2{y[2], y[3]}), bf16x2);
            hv[0] = static_cast<float>(lo[0]);
            hv[1] = static_cast<float>(lo[1]);
            hv[2] = static_cast<float>(hi[0]);
            hv[3] = static_cast<float>(hi[1]);
            if (m < M)
              *reinterpret_cast<u32x2*>(static_cast<__bf16*>(C) + static_cast<int64_t>(m) * ldc + n_seg) =
                  u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
          // Unnormalised rotation, the pack kernel's stages in its order:
          // digit 0 in registers; digit 1 (lane bits 0-1) as the in-register
          // butterfly's sum and fused multiply-add over the quad; digits 2
          // and 3 (Gray-coded lane bits 2-3 and 4-5) as
          // (a_d - a_{3-d}) + (other pair's sum), the partner a row rotation
          // by 8 / lane ^ 32 away and the other pair a row rotation by 4 /
          // lane ^ 16 away.
          bfly4(hv[0], hv[1], hv[2], hv[3]);
          if (lg >= 4) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x = hv[q];
              const float pq = x + dpp<kQuadXor1>(x);
              const float s4 = pq + dpp<kQuadXor2>(pq);
              hv[q] = fmaf(-2.f, dpp<kQuadXor3>(x), s4);
            }
          }
          if (lg >= 6) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x = hv[q];
              const float us = x + dpp<kRowRor8>(x);
              hv[q] = (x - dpp<kRowRor8>(x)) + dpp<kRowRor4>(us);
            }
          }
          if (lg >= 8) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x = hv[q];
              const float xp = xor32(x);
              const float us = x + xp;
              hv[q] = (x - xp) + swz<kSwzXor16>(us);
            }
          }
          // Largest magnitude over the group's G / 4 lanes (a quad, a row of
          // 16, or the wavefront; bit patterns of non-negative values order
          // like unsigned integers).
          uint32_t bits = as_u(fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3]))));
          if (lg >= 8) {
            bits = wave_max_bits(bits);
          } else {
            if (lg >= 4) {
              bits = max(bits, dpp_u<kQuadXor1>(bits));
              bits = max(bits, dpp_u<kQuadXor2>(bits));
            }
            if (lg >= 6) {
              bits = max(bits, dpp_u<kRowRor4>(bits));
              bits = max(bits, dpp_u<kRowRor8>(bits));
            }
          }
          if (m < M && (lane & ((1 << (lg - 2)) - 1)) == 0)
            rm.out[static_cast<int64_t>(m) * rm.ld + (n_seg >> lg)] = as_f(bits) * norm;
        }
        barrier();  // every read of this area is done before it is staged again
      }
    } else {
      // Per 16-token tile: the raw accumulators go to a private LDS area of
      // the wave as rows (16-byte chunks XOR-swizzled by row, so that the
      // 16 rows a column of lanes writes, and the chunks of a row a pass
      // reads, fall in distinct banks); each lane then takes 4-feature
      // segments of those rows, whose column scale and bias it already
      // holds, fetches the row's scale from the lane that holds it
      // (ds_bpermute), converts, finishes them and stores whole row pieces.
      // The areas lie in A buffer 2 (waves 0-3) and B buffer 1 (waves 4-7),
      // which the next tile's first slices do not use; every slice read
      // finished before the main loop's last barrier.  The value is
      // fma(acc, s_x s_w, b), the same expression in the same precision as
      // the other linear kernels, so the result bits do not depend on which
      // kernel a shape runs on.
      using out_t = typename std::conditional<OUT == 0, float, __bf16>::type;
      constexpr int kPitch = kWN * 4;                  // one row of the wave's features
      constexpr int kSwz = kSegs % 16 == 0 ? 15 : 7;  // chunk swizzle: row bits within the row's chunk count
      constexpr int kPasses = 16 * kSegs / 64;
      static_assert((16 * kSegs) % 64 == 0, "whole passes per 16 rows");
      // Passes run in kRuns straight runs (see below); the erf GELU's
      // temporaries take quarter runs at the widest tile.
      constexpr int kRuns = (ACT == 1 && TN == 4) ? 4 : 2;
      constexpr int kRunPasses = kPasses / kRuns;
      static_assert(kPasses % kRuns == 0 && kRunPasses % kLaneSegs == 0, "runs repeat the segment pattern");
      static_assert(4 * 16 * kPitch <= kATileBytes && 4 * 16 * kPitch <= kBTileBytes, "staging areas");
      uint8_t* stage = wid_u < 4 ? smem + 2 * kATileBytes + wid_u * 16 * kPitch
                                 : smem + kBBase + kBTileBytes + (wid_u - 4) * 16 * kPitch;
      // Tiles wholly inside the output take a branch-free pass loop (so the
      // LDS reads of later passes can issue ahead of earlier stores): lane
      // l's segment and row in pass p repeat with period kLaneSegs, the row
      // advancing by kRowStep, so a few per-lane bases and uniform strides
      // give every address.
      const bool full = vec_out && m_blk + kBM <= M && n_blk + kBN <= N;  // uniform
      constexpr int kRowStep = 64 * kLaneSegs / kSegs;
      out_t* lane_base[kLaneSegs];
#pragma unroll
      for (int j = 0; j < kLaneSegs; ++j) {
        const int c = 64 * j + lane;
        lane_base[j] = static_cast<out_t*>(C) + static_cast<int64_t>(m_blk + wm + c / kSegs) * ldc + n_blk + wn +
                       4 * (c % kSegs);
      }
      // Segment of pass p: converted, scaled, biased and activated outputs
      // (row scale of token `row` of the tile: s_row of lane `row`).
      auto finish = [&](int p, int j, float s_tile, float y[4]) {
        const int c = 64 * p + lane;
        const int row = c / kSegs, seg = c % kSegs;
        const acc_t a = *reinterpret_cast<const acc_t*>(stage + row * kPitch + ((seg ^ (row & kSwz)) << 4));
        const float sr = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(row << 2, __builtin_bit_cast(int, s_tile)));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = static_cast<float>(a[r]);
          const float z = I8 ? fmaf(v, sr * s_col[j][r], b_col[j][r]) : v + b_col[j][r];
          y[r] = activation<ACT>(z);
        }
      };
      // STREAM (outputs larger than the 256 MB Infinity Cache): stores with
      // the non-temporal hint, which leave the L2 to the operand panels;
      // smaller outputs stay cached for the launch that reads them next.  (A
      // run-time choice between the two stores is merged into one plain
      // store by the compiler, hence the template parameter.)
      auto store4 = [](out_t* out, const float y[4]) {
        if constexpr (OUT == 0) {
          const f32x4 v = {y[0], y[1], y[2], y[3]};
          if constexpr (STREAM)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out));
          else
            *reinterpret_cast<f32x4*>(out) = v;
        } else {
          // Two pairs, each one packed round-to-nearest-even conversion.
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const bf16x2 lo = __builtin_convertvector((f32x2{y[0], y[1]}), bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2{y[2], y[3]}), bf16x2);
          const u32x2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          if constexpr (STREAM)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(out));
          else
            *reinterpret_cast<u32x2*>(out) = v;
        }
      };
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        {
          const int r0 = 16 * t;  // first token of the tile within the wave's 64
          {
            // chunk 4 f + fk of row frow: features 16 f + 4 fk .. + 3
            uint8_t* row_ptr = stage + frow * kPitch;
#pragma unroll
            for (int f = 0; f < kTF; ++f)
              *reinterpret_cast<acc_t*>(row_ptr + (((4 * f + fk) ^ (frow & kSwz)) << 4)) = acc[t][f];
          }
          // The passes run in kRuns straight runs (the column scales' index
          // p % kLaneSegs stays a constant); fewer reads in flight keep the
          // registers within the budget of two waves per SIMD.
          if (full) {
#pragma unroll 1
            for (int hp = 0; hp < kRuns; ++hp) {
#pragma unroll
              for (int q = 0; q < kRunPasses; ++q) {
                const int p = hp * kRunPasses + q;
                float y[4];
                finish(p, q % kLaneSegs, s_row[t], y);
                store4(lane_base[q % kLaneSegs] + static_cast<int64_t>(r0 + (p / kLaneSegs) * kRowStep) * ldc, y);
              }
            }
          } else {
#pragma unroll 1
            for (int hp = 0; hp < kRuns; ++hp) {
#pragma unroll
            for (int q = 0; q < kRunPasses; ++q) {
              const int p = hp * kRunPasses + q;
              float y[4];
              finish(p, q % kLaneSegs, s_row[t], y);
              const int c = 64 * p + lane;
              const int m = m_blk + wm + r0 + c / kSegs;
              const int n = n_blk + wn + 4 * (c % kSegs);
              if (m < M) {
                out_t* out = static_cast<out_t*>(C) + static_cast<int64_t>(m) * ldc + n;
                if (vec_out && n + 3 < N) {
                  store4(out, y);
                } else {
                  for (int r = 0; r < 4 && n + r < N; ++r) out[r] = static_cast<out_t>(y[r]);
                }
              }
            }
            }
          }
        }
      }
    }

    if (!more) break;
    // The next tile: its state, zeroed accumulators, and its first slices
    // landed (each wave waits for its own transfers, which the barrier then
    // publishes; the wait also covers this tile's stores).  The barrier also
    // ends every wave's epilogue before the next main loop writes A buffer 2
    // and B buffer 1 again.
    tile = next;
    cur = nxt;
    sc = sc_next;
    zero_acc();
    wait_vm<0>();
    barrier();
    if (grp_u == 1) barrier();  // the second group runs one phase behind
  }
}

// Tile width for the eight-wave kernel: the least estimated time, counted as
// rounds of tiles over the CUs times the tile width times a cost per output
// column that depends on the width.  Wider tiles read fewer LDS bytes per
// MFMA and spread the prologue and epilogue over more columns; measured with
// the same number of rounds (K = 3072 and 6144, M from 4096 to 32700), a
// column of a 192-wide tile costs 1.14-1.17x one of a 256-wide tile, and a
// 128-wide tile 1.39-1.40x.  Ties go to the wider tile.
inline int choose_tn_pp(int64_t M, int64_t cols) {
  constexpr int cands[] = {4, 3, 2};
  constexpr int64_t col_cost[] = {100, 116, 140};
  const int64_t cus = num_cus();
  int best = 4;
  int64_t best_cost = -1;
  for (int i = 0; i < 3; ++i) {
    const int64_t bn = 64 * cands[i];
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((cols + bn - 1) / bn);
    const int64_t cost = ((tiles + cus - 1) / cus) * bn * col_cost[i];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = cands[i];
    }
  }
  return best;
}

template <bool I8, int OUT, int TN, int ACT, bool ROWMAX = false>
hipError_t launch_pp_typed(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const EpiArgs& epi,
                           int64_t M, int64_t N, int64_t Kb, void* C, int64_t ldc, hipStream_t stream,
                           const RowmaxArgs& rm = RowmaxArgs{nullptr, 0, 0}) {
  // Outputs that cannot stay in the 256 MB Infinity Cache for their reader
  // are streamed out (large-M QKV 1.0-2.2% and its routed bf16 layer
  // 2.9-3.6% faster per launch, two boxes).  A smaller output keeps plain
  // stores: the DiT launch was 7% faster streaming its 100 MB, but the LoRA
  // correction that adds into that output in place made that step 4.7%
  // slower.
  constexpr bool kCanStream = !ROWMAX && OUT != 2;
  const int out_elt = OUT == 1 ? 2 : 4;
  const bool stream_out = kCanStream && M * N * out_elt > (int64_t{256} << 20);
  auto kern = stream_out ? gemm_pp_kernel<I8, OUT, TN, ACT, ROWMAX, kCanStream>
                         : gemm_pp_kernel<I8, OUT, TN, ACT, ROWMAX, false>;
  constexpr int kSmem = pp_smem_bytes<TN>();
  static std::atomic<uint64_t> lds_set{0}, lds_set_stream{0};
  const hipError_t e =
      set_lds_limit(reinterpret_cast<const void*>(kern), kSmem, stream_out ? lds_set_stream : lds_set);
  if (e != hipSuccess) return e;
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + 64 * TN - 1) / (64 * TN));
  // One workgroup per CU walking the tile list (one workgroup fits a CU);
  // the ROWMAX epilogue and the raw int32 output take one tile per
  // workgroup (the kernel does not walk for them).  CONVROT_GEMM_GRID=tiles
  // launches one workgroup per tile (same-box comparisons only).
  static const bool one_per_tile = [] {
    const char* e = std::getenv("CONVROT_GEMM_GRID");
    return e != nullptr && std::strcmp(e, "tiles") == 0;
  }();
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = (ROWMAX || OUT == 2 || one_per_tile) ? tiles : std::min<int64_t>(tiles, num_cus());
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec_cols = al16(epi.sb) && al16(epi.bias);
  // Four consecutive outputs go out as one store when rows keep them aligned.
  const bool vec_out = (reinterpret_cast<uintptr_t>(C) % (4 * out_elt)) == 0 && ldc % 4 == 0;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kPPThreads), kSmem, stream, A, lda, B,
                     ldb, epi, static_cast<int>(M), static_cast<int>(N), static_cast<int>(Kb), C, ldc, tiles_m,
                     tiles_n, vec_cols, vec_out, rm);
  return hipGetLastError();
}

// Whether the eight-wave kernel takes this shape: whole 128-byte K slices.
inline bool pp_eligible(int64_t Kb) { return Kb % kBK == 0 && Kb > 0; }

template <bool I8, int OUT, int ACT = 0>
hipError_t launch_gemm_pp(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const EpiArgs& epi, int64_t M,
                          int64_t N, int64_t Kb, void* C, int64_t ldc, hipStream_t stream) {
  switch (choose_tn_pp(M, N)) {
    case 2: return launch_pp_typed<I8, OUT, 2, ACT>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream);
    case 3: return launch_pp_typed<I8, OUT, 3, ACT>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream);
    default: return launch_pp_typed<I8, OUT, 4, ACT>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream);
  }
}

// The linear with an activation and the next layer's per-group maxima
// (ROWMAX): always 256-wide tiles; the caller guarantees N % 256 == 0,
// G = 2^log2g with log2g in {2, 4, 6, 8}, whole 128-byte K slices and
// output rows aligned for 4-element stores.
template <int OUT, int ACT>
hipError_t launch_gemm_pp_rowmax(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const EpiArgs& epi,
                                 int64_t M, int64_t N, int64_t Kb, void* C, int64_t ldc, const RowmaxArgs& rm,
                                 hipStream_t stream) {
  return launch_pp_typed<true, OUT, 4, ACT, true>(A, lda, B, ldb, epi, M, N, Kb, C, ldc, stream, rm);
}

}  // namespace
}  // namespace convrot
