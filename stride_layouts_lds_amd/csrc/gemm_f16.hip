// gemm_f16.hip -- D = A * B^T + C, fp16 operands, fp32 accumulation, fp16
// output, on the gfx950 matrix cores (v_mfma_f32_16x16x32_f16).
//
// Data flow, each stage a layout (the method of "CuTe 中 A、B 如何加载到
// MMA 寄存器" and "数据布局及其记号", redone for CDNA4):
//   HBM tile  --(LoaderKVec/LoaderMNVec/LoaderGeneric)-->  XOR-swizzled LDS
//   tile, two stages (double buffer)  --(ds_read_b128 at
//   fragment_lds_offset)-->  per-lane operand fragments in the instruction's
//   (lane, slot) layout  --(MFMA)-->  fp32 accumulators in the instruction's
//   D layout  --(epilogue: + C, round to fp16, predicated stores)-->  HBM.
//
// The instruction is issued with its operands swapped (instruction A = our
// B tile, instruction B = our A tile), so the accumulator layout puts four
// consecutive n of one output row m in each lane: 8-byte stores.
#include "sl_device.hpp"

namespace sl {
namespace {

// Epilogue: acc[i][j][r] is output (m, n) with
//   m = m_base + 16 i + lane % 16,  n = n_base + 16 j + 4 (lane / 16) + r
// D = fp16_rne(acc + C), stores predicated on m < M, n < N.
template <int FM, int FN, int DT = DT_F16>
__device__ __forceinline__ void epilogue(const floatx4 (&acc)[FM][FN], const GemmParams& p, int32_t batch,
                                         int64_t m_base, int64_t n_base, int32_t lane) {
  uint16_t* D = (uint16_t*)p.d + batch * p.d_bs;
  if (p.flags & F_HAS_C) {
    // every C load of the lane is issued before its first D store (C may
    // be D itself: each element is read before it is written)
    const uint16_t* C = (const uint16_t*)p.c + batch * p.c_bs;
    u16x4 cq[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        cq[i][j] = load_c_quad(p, C, m_base + 16 * i + (lane & 15), n_base + 16 * j + 4 * (lane >> 4));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        floatx4 v = acc[i][j];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += to_f32<DT>(cq[i][j][r]);
        store_d_quad<DT>(p, D, m_base + 16 * i + (lane & 15), n_base + 16 * j + 4 * (lane >> 4), v);
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        store_d_quad<DT>(p, D, m_base + 16 * i + (lane & 15), n_base + 16 * j + 4 * (lane >> 4), acc[i][j]);
  }
}

// Split-K partial: acc[i][j] (same layout as the epilogue's) goes to
// ws[split][batch][m][n] in fp32, 16-byte stores where the row allows.
template <int FM, int FN>
__device__ __forceinline__ void store_partial(const floatx4 (&acc)[FM][FN], const GemmParams& p, int32_t split,
                                              int32_t batch, int64_t m_base, int64_t n_base, int32_t lane) {
  float* W = p.ws + ((int64_t)split * p.batch + batch) * p.M * p.N;
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t m = m_base + 16 * i + (lane & 15);
      const int64_t n = n_base + 16 * j + 4 * (lane >> 4);
      if (m >= p.M || n >= p.N) continue;
      float* w = W + m * p.N + n;
      if (vec) {
        *(floatx4*)w = acc[i][j];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) w[r] = acc[i][j][r];
      }
    }
}

// Epilogue of a wave's 128 x 16 FN block (FN = 8 or 4) through a private
// LDS region of 64 rows x 16 FN fp32 (rows_load_c / rows_store_half): here
// the accumulator-order writes, 16 rows x one 16-byte chunk per instruction
// (accumulator (i, j) holds rows 16 i + lane % 16, columns 16 j + 4 (lane /
// 16) .. + 3).  NT: non-temporal D stores.
template <int DT, int FN, bool NT>
__device__ __forceinline__ void epilogue_rows(const floatx4 (&acc)[8][FN], const GemmParams& p, int32_t batch,
                                              int64_t m_base, int64_t n_base, int32_t lane, char* region) {
  constexpr int COLS = 16 * FN;
  const int32_t l0 = lane & 15, l1 = lane >> 4;
  u16x4 cq[2][COLS / 4];
  rows_load_c<COLS>(p, batch, m_base, n_base, lane, cq);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int32_t r = 16 * i + l0;
        *(floatx4*)(region + rows_chunk<COLS>(r, 4 * j + l1)) = acc[4 * h + i][j];
      }
    rows_store_half<DT, COLS, NT>(p, batch, m_base + 64 * h, n_base, lane, region, cq[h]);
  }
}

// the row epilogue's condition: every 256 x 256 tile full, D (and C if
// present) in contiguous 8-byte aligned rows
inline bool rows_epilogue_ok(const GemmParams& p) {
  return p.M % 256 == 0 && p.N % 256 == 0 && (p.flags & F_D_VEC) && (!(p.flags & F_HAS_C) || (p.flags & F_C_VEC));
}

// PIPE 0: per k-slice, read the fragments then issue the MFMAs (latency is
// covered by the other wave on the SIMD when WM*WN = 8).  PIPE 1: two
// fragment sets, the next slice is read while the current one computes.
// ROWS (8 waves of 128 x 64, PIPE 0): every tile is full and C and D rows
// are contiguous and 8-byte aligned, so the epilogue goes through LDS rows
// (epilogue_rows, a 16 KiB region per wave in the stage buffers); ROWS_NT:
// the same with non-temporal D stores, for grids of one round (every
// workgroup stores at once: 3-4% faster there, 1% slower on four rounds).
template <int BM, int BN, int WM, int WN, int ALOAD, int BLOAD, int SHIFT, int PIPE, int DT = DT_F16,
          bool ROWS = false, bool ROWS_NT = false>
__global__ __launch_bounds__(WM* WN * 64, (WM * WN + 3) / 4) void gemm_f16_kernel(const GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 instruction tiles per wave
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  static_assert(!ROWS || (FM == 8 && FN == 4 && PIPE == 0 && WM * WN * 64 * 64 * 4 <= 2 * STAGE),
                "the row epilogue: 128 x 64 wave blocks, one 16 KiB region each in the stage buffers");

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave % WM, wn = wave / WM;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  auto la = make_loader<ALOAD, BM, NT, SHIFT>(p, 0, tc.batch, m0, rows_a, wave, lane);
  auto lb = make_loader<BLOAD, BN, NT, SHIFT>(p, 1, tc.batch, n0, rows_b, wave, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  // operand fragments of one k-slice (32 of the tile's 64 K), two sets:
  // one feeds the MFMAs while the other is being read from LDS
  half8 fa0[FM], fb0[FN];
  [[maybe_unused]] half8 fa1[FM], fb1[FN];
  auto read_slice = [&](const char* buf, int ks, half8(&fa)[FM], half8(&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = read_frag<ALOAD, BM, SHIFT>(buf, lane, a_row0 + 16 * i, ks);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = read_frag<BLOAD, BN, SHIFT>(buf + ABYTES, lane, b_row0 + 16 * j, ks);
  };
  // instruction A = our B fragment, instruction B = our A fragment
  auto mfma_slice = [&](const half8(&fa)[FM], const half8(&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma16<DT>(fb[j], fa[i], acc[i][j]);
  };
  constexpr int NREAD = FM + FN;          // ds_read_b128 per slice
  constexpr int NMFMA = FM * FN;          // MFMAs per slice
  constexpr int PER = NMFMA / NREAD;      // MFMAs between two reads

  const int32_t T = p.k_tiles;
  if (T > 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    la.commit(smem);
    lb.commit(smem + ABYTES);
    wait_vmem();
    __syncthreads();
    if constexpr (PIPE == 1) read_slice(smem, 0, fa0, fb0);
  }

  // Past the last tile the loads are fully out of range (they write zeros
  // into the idle buffer) and the reads of the idle buffer are never
  // consumed.  With direct copies and every K-tile whole, the copies take
  // the path without vector arithmetic (issue_full), the one past the last
  // tile reloading the last tile (not with PIPE 1, whose second fragment
  // set leaves no registers for the loaders' offsets).
  constexpr bool direct = PIPE == 0 && (ALOAD == LOAD_KVEC || ALOAD == LOAD_MNDMA) &&
                          (BLOAD == LOAD_KVEC || BLOAD == LOAD_MNDMA);
  const bool kfull = direct && p.K % 64 == 0;
  for (int32_t t = 0; t < T; ++t) {
    char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    if constexpr (direct) {
      if (kfull) {
        const int32_t u = t + 1 < T ? t + 1 : T - 1;
#pragma unroll
        for (int j = 0; j < decltype(la)::ITERS; ++j) la.issue_full(u, nxt, j);
#pragma unroll
        for (int j = 0; j < decltype(lb)::ITERS; ++j) lb.issue_full(u, nxt + ABYTES, j);
      } else {
        la.issue(t + 1, nxt);
        lb.issue(t + 1, nxt + ABYTES);
      }
    } else {
      la.issue(t + 1, nxt);
      lb.issue(t + 1, nxt + ABYTES);
    }
    if constexpr (PIPE == 0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        read_slice(cur, ks, fa0, fb0);
        mfma_slice(fa0, fb0);
      }
      la.commit(nxt);
      lb.commit(nxt + ABYTES);
      wait_vmem();
      __syncthreads();
    } else {
      // first half: read slice 1 of tile t, compute slice 0
      read_slice(cur, 1, fa1, fb1);
      mfma_slice(fa0, fb0);
#pragma unroll
      for (int g = 0; g < NREAD; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one ds_read
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // PER MFMAs
      }
      la.commit(nxt);
      lb.commit(nxt + ABYTES);
      // tile t+1 is in LDS and every wave is done reading tile t's slice 0
      wait_vmem();
      __syncthreads();
      // second half: read slice 0 of tile t+1, compute slice 1 of tile t
      read_slice(nxt, 0, fa0, fb0);
      mfma_slice(fa1, fb1);
#pragma unroll
      for (int g = 0; g < NREAD; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
      }
    }
  }

  if constexpr (ROWS) {
    __syncthreads();  // every wave is done reading the stage buffers
    epilogue_rows<DT, FN, ROWS_NT>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane, smem + wave * 16384);
  } else {
    epilogue<FM, FN, DT>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// Multi-stage variant for K-contiguous operands: K-tiles of RB/2 fp16 (LDS
// rows of RB bytes), STAGES LDS buffers in a ring, the copy of tile
// t+STAGES-1 issued while tile t computes, so each tile's HBM->LDS copy has
// STAGES-1 tiles of compute to land.  One phase barrier per tile makes the
// landed tile visible to every wave and retires the buffer the next issue
// overwrites.  (A __syncthreads() here would wait for every copy in flight:
// its fence counts the direct-to-LDS copies as outstanding LDS writes.)
//
// With BM = 32, BN = 128 and 64-wide K-tiles this is the streaming kernel
// for outputs too small to fill the chip with big tiles (skinny N): one
// 32-row panel of A per workgroup, read once from HBM, against all of B,
// which every workgroup shares through L2.
template <int BM, int BN, int WM, int WN, int STAGES, int SHIFT, int RB = 64, int DT = DT_F16>
__global__ __launch_bounds__(WM* WN * 64, (WM * WN + 3) / 4) void gemm_f16_ms_kernel(const GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KT = RB / 2;   // fp16 of K per tile
  constexpr int KS = KT / 32;  // k-slices of the instruction per tile
  constexpr int ABYTES = BM * RB, BBYTES = BN * RB;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  using LA = LoaderKVec<BM, NT, SHIFT, 2, RB>;
  using LB = LoaderKVec<BN, NT, SHIFT, 2, RB>;
  constexpr int LOADS = LA::ITERS + LB::ITERS;  // vector-memory ops per tile per thread
  static_assert((STAGES - 2) * LOADS < 64, "vmcnt range");

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave % WM, wn = wave / WM;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);
  LA la(A, rows_a, p.a_rs, 1, p.K, wave, lane);
  LB lb(B, rows_b, p.b_rs, 1, p.K, wave, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;

  // K-tiles [t0, t0 + T) of this workgroup: all of K, or one split's share
  const int32_t T_all = (int32_t)((p.K + KT - 1) / KT);
  const int32_t t0 = tc.split * p.split_tiles;
  const int32_t T = p.splits > 1 ? (T_all - t0 < p.split_tiles ? T_all - t0 : p.split_tiles) : T_all;
  // the u-th tile of the range; past its end, a tile fully out of range
  auto ktile = [&](int32_t u) { return u < T ? t0 + u : T_all; };
  // prologue: tiles 0 .. STAGES-2 in flight, wait for tile 0
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    la.issue(ktile(s), smem + s * STAGE);
    lb.issue(ktile(s), smem + s * STAGE + ABYTES);
  }
  wait_vmem_n<(STAGES - 2) * LOADS>();
  phase_barrier();

  for (int32_t t = 0; t < T; ++t) {
    const char* cur = smem + (t % STAGES) * STAGE;
    char* fut = smem + ((t + STAGES - 1) % STAGES) * STAGE;
    // the buffer of tile t-1 is retired (barrier at the end of t-1): refill
    // it with tile t+STAGES-1 (fully out of range past the last tile)
    la.issue(ktile(t + STAGES - 1), fut);
    lb.issue(ktile(t + STAGES - 1), fut + ABYTES);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, ks, SHIFT, RB));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *(const half8*)(cur + ABYTES + fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, ks, SHIFT, RB));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma16<DT>(fb[j], fa[i], acc[i][j]);
    }
    // tile t+1 landed (this wave's part); the barrier publishes every
    // wave's part and, with this wave's LDS reads complete, retires tile t's
    // buffer
    wait_vmem_n<(STAGES - 2) * LOADS>();
    phase_barrier();
  }
  // the out-of-range copies past the last tile still target this
  // workgroup's LDS: let them land before the workgroup can end
  wait_vmem();
  if (p.splits > 1)
    store_partial<FM, FN>(acc, p, tc.split, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  else
    epilogue<FM, FN, DT>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
}

// The ring kernel reads fragment r of a slice (rows row0 + 16 r ...) at the
// lane's offset for r's parity plus 4096 (r / 2): with the chunk swizzle at
// shift 0 a row's swizzle depends on its low three bits and bit 4, i.e. on
// the lane and on r's parity when row0 is a multiple of 32.  Checked here
// for every lane and slice at the wave rows the kernel uses.
constexpr bool frag_offset_splits() {
  for (int32_t row0 : {0, 96, 128})
    for (int32_t lane = 0; lane < 64; ++lane)
      for (int32_t ks = 0; ks < 2; ++ks)
        for (int32_t r = 0; r < 8; ++r)
          if (fragment_lds_offset(MFMA16_F16, lane, 0, row0 + 16 * r, ks, 0) !=
              fragment_lds_offset(MFMA16_F16, lane, 0, row0 + 16 * (r & 1), ks, 0) + 4096 * (r >> 1))
            return false;
  return true;
}
static_assert(frag_offset_splits(), "fragment offsets split into a parity part and 4096 (r / 2)");

// MFMA whose accumulator is pinned to AGPRs (the "a" constraint): a
// 128x128 wave block needs 256 accumulator registers per lane, which only
// the AGPR file can hold beside the operand fragments.  The statement is
// opaque to the compiler, which therefore inserts no wait states before the
// result is read: a kernel using it reads its accumulators only after an
// explicit idle (see the end of gemm_f16_w4r_kernel).
template <int DT>
__device__ __forceinline__ void mfma_acc(floatx4& c, const half8& a, const half8& b) {
  if constexpr (DT == DT_F16)
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Four waves, one per SIMD, each computing a 128 x BN/2 block of the
// 256 x BN tile (8 x BN/32 MFMA tiles, accumulators in AGPRs, two sets of
// operand fragments in VGPRs).  With one wave per SIMD every latency is
// hidden in software: the LDS reads of the next k-slice and the HBM->LDS
// copies are interleaved one by one with the MFMAs of the current slice.
// LDS is a ring of five 32 KiB slots, each one operand K-tile of 64 K (the
// XOR-swizzled K-major layout, or for ALOAD / BLOAD = LOAD_MNDMA the
// M-major one read by transposing reads): operand tile q (A of K-tile q/2
// for even q, B for odd q) sits in slot q % 5, so the two tiles being read
// and three in flight fit the 160 KiB of a CU.  Requires at least one
// K-tile.  ROWS (BN = 256 only): every tile is full and C and D rows are
// contiguous and 8-byte aligned, so the epilogue goes through LDS
// (epilogue_rows, its D stores non-temporal: with every workgroup of a
// round storing at once this measured 1-6% faster on the one-round shapes
// and no different on the larger ones); otherwise the per-quad epilogue.
// KFULL (K-contiguous
// operands, K a multiple of 64): every K-tile is whole, so every copy is
// issue_full, with no vector arithmetic in front of it.
//
// Tile t: (1) reads of slice 0 into set 0, the second half of tile t-1's
// slice 1 on set 1, copy of B(t+1) into A(t-1)'s slot; (2) slice 0 on set
// 0, reads of slice 1 into set 1, copy of A(t+2) into B(t-1)'s slot; (3)
// the first half of slice 1; barrier.  Each copy has at least one K-tile of
// compute to land; at the barrier ending tile t only A(t+2) (and the C line
// load issued just before it) may still be in flight.  In the last eight
// K-tiles half the lanes also load one 128-byte line of the wave's C block
// each (4 bytes into LDS bytes that A(t+2)'s first copy overwrites next), so the
// epilogue's C reads find C in L2 or the Infinity Cache: all CUs finish
// their tiles together, and C read then from HBM is a burst at the end.
template <int SHIFT, int DT, bool ROWS, int ALOAD = LOAD_KVEC, int BLOAD = LOAD_KVEC, int BN = 256,
          bool KFULL = false>
__global__ __launch_bounds__(256, 1) void gemm_f16_w4r_kernel(const GemmParams p) {
  constexpr int BM = 256, FM = 8, FN = BN / 32;
  constexpr int SLOT = 256 * kRowBytes;
  static_assert(!ROWS || BN == 256, "the row epilogue covers 128-column wave blocks");
  __shared__ __attribute__((aligned(1024))) char smem[5 * SLOT];

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave & 1, wn = wave >> 1;
  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  auto la = make_loader<ALOAD, BM, 256, SHIFT>(p, 0, tc.batch, m0, rows_a, wave, lane);
  auto lb = make_loader<BLOAD, BN, 256, SHIFT>(p, 1, tc.batch, n0, rows_b, wave, lane);
  constexpr int LOADS = decltype(la)::ITERS;    // copy instructions per A tile
  constexpr int BLOADS = decltype(lb)::ITERS;   // ... per B tile
  static_assert(LOADS == 8 && BLOADS <= 8, "copy layout");
  static_assert(!KFULL || (ALOAD == LOAD_KVEC && BLOAD == LOAD_KVEC), "whole K-tiles: K-contiguous operands");
  static_assert(SHIFT == 0, "the fragment addresses are split for the shift-0 swizzle");

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * 128, b_row0 = wn * (BN / 2);
  const int32_t T = p.k_tiles;  // at least 1 (the planner's condition for this kernel)
  __builtin_assume(T >= 1);
  // K-tile u's copies; past the last K-tile the look-ahead copies are never
  // read: fully out of range, or with KFULL (every K-tile whole) the last
  // K-tile again, so that every copy takes the fast path
  auto kt = [&](int32_t u) { return u < T ? u : (KFULL ? T - 1 : T); };
  auto slot = [&](int32_t q) { return smem + q * SLOT; };
  auto copy_a = [&](int32_t u, char* dst, int j) {
    if constexpr (KFULL) la.issue_full(kt(u), dst, j);
    else la.issue_one(kt(u), dst, j);
  };
  auto copy_b = [&](int32_t u, char* dst, int j) {
    if constexpr (KFULL) lb.issue_full(kt(u), dst, j);
    else lb.issue_one(kt(u), dst, j);
  };
  half8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  // Fragment reads of K-contiguous tiles from precomputed LDS addresses:
  // fragment r of a slice sits at (lane part for r's parity and the slice)
  // + slot base + 4096 (r / 2) (frag_offset_splits), and the bases of a
  // K-tile are formed before the barrier that ends the previous one, so no
  // read waits on fresh vector arithmetic.  M-major tiles read as before.
  typedef __attribute__((address_space(3))) const half8 lds_h8;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)smem;
  uint32_t offA[2][2], offB[2][2], bA[2][2], bB[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      offA[ks][par] = lds0 + (uint32_t)fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * par, ks, SHIFT);
      offB[ks][par] = lds0 + (uint32_t)fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * par, ks, SHIFT);
    }
  auto bases = [&](int32_t qa, int32_t qb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        bA[ks][par] = offA[ks][par] + (uint32_t)(qa * SLOT);
        bB[ks][par] = offB[ks][par] + (uint32_t)(qb * SLOT);
      }
    // computed here, not next to the reads
    asm volatile("" : "+v"(bA[0][0]), "+v"(bA[0][1]), "+v"(bA[1][0]), "+v"(bA[1][1]));
    asm volatile("" : "+v"(bB[0][0]), "+v"(bB[0][1]), "+v"(bB[1][0]), "+v"(bB[1][1]));
  };
  // read r of a slice's FN + FM fragment reads (B's first)
  auto read = [&](const char* cA, const char* cB, int r, int ks, half8(&fa)[FM], half8(&fb)[FN]) {
    if (r < FN) {
      if constexpr (BLOAD == LOAD_KVEC)
        fb[r] = *(lds_h8*)(uintptr_t)(bB[ks][r & 1] + 4096u * (uint32_t)(r >> 1));
      else
        fb[r] = read_frag<BLOAD, BN, SHIFT>(cB, lane, b_row0 + 16 * r, ks);
    } else {
      const int i = r - FN;
      if constexpr (ALOAD == LOAD_KVEC)
        fa[i] = *(lds_h8*)(uintptr_t)(bA[ks][i & 1] + 4096u * (uint32_t)(i >> 1));
      else
        fa[i] = read_frag<ALOAD, BM, SHIFT>(cA, lane, a_row0 + 16 * i, ks);
    }
  };
  constexpr int NR = FN + FM;  // fragment reads per slice (at most 16)
  constexpr int NH = 4 * FN;   // MFMAs in half a slice

  // C of this wave's block, pulled into the caches during the last PF_TILES
  // K-tiles (one dword per 128-byte line; 16 rows, two lines each, per K-tile
  // on lanes 0-31): the epilogue's C reads then hit L2 / the Infinity Cache
  // instead of HBM.  Over eight K-tiles rather than four the C traffic meets
  // less of the operand traffic: 3-4% off a cold 4096^3 + C launch, the same
  // warm or at 8192^3.
  constexpr int32_t PF_TILES = 8, PF_ROWS = 128 / PF_TILES;
  const bool pf_on = (p.flags & F_HAS_C) && (p.flags & F_C_VEC);
  const int32_t pf_rows = rows_a - a_row0 < 128 ? rows_a - a_row0 : 128;
  const int32_t pf_cols = rows_b - b_row0 < BN / 2 ? rows_b - b_row0 : BN / 2;
  const uint16_t* pf_base = (const uint16_t*)p.c + (pf_on ? tc.batch * p.c_bs + (m0 + a_row0) * p.c_rs + n0 + b_row0 : 0);
  const __amdgpu_buffer_rsrc_t pf_rsrc =
      make_rsrc(pf_base, pf_on && pf_rows > 0 && pf_cols > 0 ? (uint32_t)(((pf_rows - 1) * p.c_rs + pf_cols) * 2) : 0u);
  const int32_t pf_r = lane >> 1, pf_c = 64 * (lane & 1);
  const uint32_t pf_off = (uint32_t)((pf_r * p.c_rs + pf_c) * 2);
  const uint32_t pf_step = (uint32_t)(PF_ROWS * p.c_rs * 2);
  // K-tile u's C-line offset, formed a K-tile ahead of its load
  auto pf_voff = [&](int32_t u) {
    const int32_t k = u - (T - PF_TILES);
    const bool in = k >= 0 && pf_r < PF_ROWS && PF_ROWS * k + pf_r < pf_rows && pf_c < pf_cols;
    uint32_t v = in ? pf_off + (uint32_t)k * pf_step : kOutOfRange;
    asm volatile("" : "+v"(v));
    return v;
  };

#pragma unroll
  for (int j = 0; j < LOADS; ++j) copy_a(0, slot(0), j);
#pragma unroll
  for (int j = 0; j < BLOADS; ++j) copy_b(0, slot(1), j);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) copy_a(1, slot(2), j);
  // the first tile's part (1) computes with zero fragments (adds nothing)
#pragma unroll
  for (int i = 0; i < FM; ++i) fa1[i] = half8{};
#pragma unroll
  for (int j = 0; j < FN; ++j) fb1[j] = half8{};
  wait_vmem_n<LOADS>();
  phase_barrier();

  int32_t sa = 0;  // slot of A(t); B(t) in the next one
  int32_t t = 0;
  bases(0, 1);
  uint32_t pf_v = pf_voff(0);
  // one copy of the loop body: a peeled or unswitched copy would give the
  // accumulators a second path to the epilogue
#pragma clang loop unroll(disable)
  do {  // T >= 1: one path into the epilogue keeps the accumulators in place
    const int32_t sb = sa == 4 ? 0 : sa + 1;
    const int32_t s3 = sa + 3 >= 5 ? sa - 2 : sa + 3, s4 = sa == 0 ? 4 : sa - 1;
    const char* cA = slot(sa);
    const char* cB = slot(sb);
    // (1)
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (g < NR) read(cA, cB, g, 0, fa0, fb0);
      if (!(g & 1) && g / 2 < BLOADS) copy_b(t + 1, slot(s3), g >> 1);
#pragma unroll
      for (int e = g * NH / 16; e < (g + 1) * NH / 16; ++e) {
        const int i = FM / 2 + e / FN, j = e % FN;
        mfma_acc<DT>(acc[i][j], fb1[j], fa1[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // (2)
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (g < NR) read(cA, cB, g, 1, fa1, fb1);
      if (g == 0) {
        // one C line per lane into the bytes A(t+2)'s first copy overwrites
        // next (loads return in order); out of range before the last eight
        // K-tiles, so the count of loads in flight stays fixed
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pf_rsrc, (lds_void_t*)(slot(s4) + wave * 1024), 4, pf_v, 0, 0, 0);
      }
      if (g & 1) copy_a(t + 2, slot(s4), g >> 1);
#pragma unroll
      for (int e = g * 2 * NH / 16; e < (g + 1) * 2 * NH / 16; ++e) {
        const int i = e / FN, j = e % FN;
        mfma_acc<DT>(acc[i][j], fb0[j], fa0[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // (3)
#pragma unroll
    for (int i = 0; i < FM / 2; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_acc<DT>(acc[i][j], fb1[j], fa1[i]);
    // the next K-tile's read bases and C-line offset
    {
      const int32_t na = sa + 2 >= 5 ? sa - 3 : sa + 2;
      bases(na, na == 4 ? 0 : na + 1);
      pf_v = pf_voff(t + 1);
    }
    // in flight after this: the C line load and A(t+2)'s copies
    wait_vmem_n<LOADS + 1>();
    phase_barrier();
    sa = sa + 2 >= 5 ? sa - 3 : sa + 2;
  } while (++t < T);
  // the last tile's second half of slice 1
#pragma unroll
  for (int i = FM / 2; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) mfma_acc<DT>(acc[i][j], fb1[j], fa1[i]);
  wait_vmem();
  // The MFMAs above are inline assembly, so the compiler inserts no wait
  // states before their results are read.  Empty volatile statements that
  // re-define every accumulator hold the MFMAs before an idle of 32 cycles
  // (more than the instruction's passes need) and every read after it
  // (volatile statements keep their order).
  auto pin = [&] {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; j += 2) asm volatile("" : "+a"(acc[i][j]), "+a"(acc[i][j + 1]));
  };
  pin();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  pin();
  if constexpr (ROWS) {
    // every wave's copies have landed and its reads of the ring are done:
    // the LDS is free for the per-wave epilogue regions
    __syncthreads();
    epilogue_rows<DT, 8, true>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane, smem + wave * 32768);
  } else {
    epilogue<FM, FN, DT>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// NVFP4 on the ring kernel's schedule: 4 waves, one per SIMD, each a
// 128 x 128 block (8 x 8 fp16 MFMA tiles, accumulators in AGPRs).  The
// decoding loaders (PAIRS: two K-tiles per fetch) bring K-tile t+2's packed
// E2M1 data and E4M3 scales into registers during K-tile t, and during K-tile
// t+1 decode them to fp16 (exact) and write the stage of the next K-tile, so
// every fetch has a K-tile of compute to land and LDS holds two fp16 stages
// (128 KiB).  Tile t: (1) reads of slice 0 into set 0, the second half of
// tile t-1's slice 1 on set 1, and the decode of A's K-tile t+1 into the
// idle stage one 16-byte piece at a time between the MFMAs, then the fetch
// of A's K-tile t+2; (2) slice 0 on set 0 with the reads of slice 1 and B's
// decode, then B's fetch; (3) the first half of slice 1; barrier.  (Decoding
// a whole tile at once stalls the one wave of the SIMD: 35% slower.)  ROWS: the
// row epilogue through LDS (full tiles, vector C/D).
template <int SHIFT, bool PAIRS, bool ROWS>
__global__ __launch_bounds__(256, 1) void gemm_nvfp4_w4r_kernel(const GemmParams p) {
  constexpr int BM = 256, BN = 256, FM = 8, FN = 8;
  constexpr int KIND = PAIRS ? LOAD_NVFP4_PAIRS : LOAD_NVFP4;
  constexpr int ABYTES = BM * kRowBytes, STAGE = ABYTES + BN * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave & 1, wn = wave >> 1;
  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  auto la = make_loader<KIND, BM, 256, SHIFT>(p, 0, tc.batch, m0, rows_a, wave, lane);
  auto lb = make_loader<KIND, BN, 256, SHIFT>(p, 1, tc.batch, n0, rows_b, wave, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * 128, b_row0 = wn * 128;
  const int32_t T = p.k_tiles;  // at least 1 (the planner's condition for this kernel)
  __builtin_assume(T >= 1);
  auto kt = [&](int32_t u) { return u < T ? u : T; };
  half8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto read = [&](const char* st, int r, int ks, half8(&fa)[FM], half8(&fb)[FN]) {
    if (r < FN)
      fb[r] = read_frag<KIND, BN, SHIFT>(st + ABYTES, lane, b_row0 + 16 * r, ks);
    else
      fa[r - FN] = read_frag<KIND, BM, SHIFT>(st, lane, a_row0 + 16 * (r - FN), ks);
  };

  // K-tile 0 into stage 0; K-tile 1 fetched
  la.issue(0, nullptr);
  lb.issue(0, nullptr);
  la.commit(smem);
  lb.commit(smem + ABYTES);
  la.issue(kt(1), nullptr);
  lb.issue(kt(1), nullptr);
  // the first tile's part (1) computes with zero fragments (adds nothing)
#pragma unroll
  for (int i = 0; i < FM; ++i) fa1[i] = half8{};
#pragma unroll
  for (int j = 0; j < FN; ++j) fb1[j] = half8{};
  phase_barrier();

  int32_t t = 0;
  do {  // T >= 1: one path into the epilogue keeps the accumulators in place
    const char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    // (1), with A's K-tile t+1 decoded piece by piece
    constexpr int PARTS = decltype(la)::PARTS;
    static_assert(PARTS <= 16, "decode pieces per part");
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      read(cur, g, 0, fa0, fb0);
      if (g * PARTS % 16 == 0) la.commit_part(nxt, g * PARTS / 16 / 4, g * PARTS / 16 % 4);
#pragma unroll
      for (int e = 2 * g; e < 2 * g + 2; ++e) {
        const int i = FM / 2 + e / FN, j = e % FN;
        mfma_acc<DT_F16>(acc[i][j], fb1[j], fa1[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    la.issue(kt(t + 2), nullptr);  // A's K-tile t+2 (past the end: fully out of range)
    // (2), with B's K-tile t+1 decoded piece by piece
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      read(cur, g, 1, fa1, fb1);
      if (g * PARTS % 16 == 0) lb.commit_part(nxt + ABYTES, g * PARTS / 16 / 4, g * PARTS / 16 % 4);
#pragma unroll
      for (int e = 4 * g; e < 4 * g + 4; ++e) {
        const int i = e / FN, j = e % FN;
        mfma_acc<DT_F16>(acc[i][j], fb0[j], fa0[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lb.issue(kt(t + 2), nullptr);
    // (3)
#pragma unroll
    for (int i = 0; i < FM / 2; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_acc<DT_F16>(acc[i][j], fb1[j], fa1[i]);
    phase_barrier();  // K-tile t+1 written by every wave; K-tile t's reads done
  } while (++t < T);
  // the last tile's second half of slice 1
#pragma unroll
  for (int i = FM / 2; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) mfma_acc<DT_F16>(acc[i][j], fb1[j], fa1[i]);
  wait_vmem();  // the fetches past the end
  auto pin = [&] {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; j += 2) asm volatile("" : "+a"(acc[i][j]), "+a"(acc[i][j + 1]));
  };
  pin();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  pin();
  if constexpr (ROWS) {
    __syncthreads();
    epilogue_rows<DT_F16, 8, false>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane, smem + wave * 32768);
  } else {
    epilogue<FM, FN, DT_F16>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// D = round(C + sum_s ws[s]) to D's format over every output, four
// consecutive n per thread (grid-stride).  The partial planes are
// [batch][M][N] fp32, contiguous.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmParams p) {
  const int64_t nq = (p.N + 3) / 4;
  const int64_t total = (int64_t)p.batch * p.M * nq;
  const int64_t plane = (int64_t)p.batch * p.M * p.N;
  const bool vec = (p.N & 3) == 0;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t n = (q % nq) * 4;
    const int64_t bm = q / nq;
    const int64_t m = bm % p.M;
    const int32_t b = (int32_t)(bm / p.M);
    const float* w = p.ws + (b * p.M + m) * p.N + n;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
      for (int32_t sp = 0; sp < p.splits; ++sp) v += *(const floatx4*)(w + sp * plane);
    } else {
      for (int32_t sp = 0; sp < p.splits; ++sp)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) v[r] += w[sp * plane + r];
    }
    uint16_t* D = (uint16_t*)p.d + b * p.d_bs;
    const uint16_t* C = (p.flags & F_HAS_C) ? (const uint16_t*)p.c + b * p.c_bs : nullptr;
    store_quad<DT>(p, C, D, m, n, v);
  }
}

// Ping-pong variant for K-contiguous operands, 256x256 tile, 8 waves.
// The waves form two groups of four, one wave of each group per SIMD, each
// wave owning a 128x64 block of the tile.  Every K-tile is two phases per
// wave: a memory phase M(t) (group 0 also issues the HBM->LDS copy of tile
// t+1; every wave reads all its fragments of tile t) and a compute phase
// C(t) (64 MFMAs back to back on registers).  Group 1 runs one phase behind
// group 0, so on every SIMD one wave computes while the other moves data;
// the phases are separated by phase barriers.
//   group 0:  b0 M(0) b1 C(0) b2 M(1) b3 C(1) ...  C(T-1) b2T  [epilogue] b2T+1
//   group 1:  b0 ---- b1 M(0) b2 C(0) b3 M(1) ...  M(T-1) b2T  C(T-1) b2T+1 [epilogue]
// Both groups pass 2T+2 barriers.  Tile t+1 is copied into the buffer of
// tile t-1 during M(t) of group 0; its last readers (M(t-1) of both groups)
// finished before barrier b2t.  Group 0 waits for the copy at the end of
// C(t), before barrier b2t+2, ahead of the first read in M(t+1).
template <int SHIFT>
__global__ __launch_bounds__(512, 2) void gemm_f16_pp_kernel(const GemmParams p) {
  constexpr int BM = 256, BN = 256;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t grp = wave >> 2;
  const int32_t wm = wave & 1, wn = wave >> 1;  // group 0: wn 0,1; group 1: wn 2,3

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);
  // the copy is done by the four group-0 waves
  LoaderKVec<BM, 256, SHIFT, 2> la(A, rows_a, p.a_rs, 1, p.K, wave & 3, lane);
  LoaderKVec<BN, 256, SHIFT, 2> lb(B, rows_b, p.b_rs, 1, p.K, wave & 3, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  half8 fa[2][FM], fb[2][FN];

  const int32_t T = p.k_tiles;
  if (grp == 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    wait_vmem();
  }
  phase_barrier();                 // b0: tile 0 in LDS
  if (grp == 1) phase_barrier();   // b1 for group 1: start one phase behind

  for (int32_t t = 0; t < T; ++t) {
    const char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    // ---- M(t)
    if (grp == 0) {
      la.issue(t + 1, nxt);       // fully out of range past the last tile
      lb.issue(t + 1, nxt + ABYTES);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[ks][i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, ks, SHIFT));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[ks][j] =
            *(const half8*)(cur + ABYTES + fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, ks, SHIFT));
    }
    phase_barrier();
    // ---- C(t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
    if (grp == 0) wait_vmem();   // tile t+1 landed before b2t+2
    phase_barrier();
  }
  if (grp == 0) {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
    phase_barrier();               // b2T+1: matches group 1's last barrier
  } else {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// Ping-pong with deep prefetch: the ping-pong schedule above on K-tiles of
// 32 (LDS rows of 64 bytes) held in STAGES buffers.  Group 0 issues the copy
// of tile t+STAGES-1 during M(t) into the buffer of tile t-1 (its last
// readers, M(t-1) of both groups, finished before barrier b2t), and at the
// end of C(t) waits only until tile t+1 has landed (the copies of tiles
// t+2 .. t+STAGES-1 stay in flight), so every copy has STAGES-1 tiles of
// compute to complete.
template <int STAGES, int SHIFT>
__global__ __launch_bounds__(512, 2) void gemm_f16_pps_kernel(const GemmParams p) {
  constexpr int BM = 256, BN = 256;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int RB = 64;
  constexpr int ABYTES = BM * RB, BBYTES = BN * RB;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  using LA = LoaderKVec<BM, 256, SHIFT, 2, RB>;
  using LB = LoaderKVec<BN, 256, SHIFT, 2, RB>;
  constexpr int LOADS = LA::ITERS + LB::ITERS;  // copy instructions per tile per group-0 wave

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t grp = wave >> 2;
  const int32_t wm = wave & 1, wn = wave >> 1;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);
  LA la(A, rows_a, p.a_rs, 1, p.K, wave & 3, lane);
  LB lb(B, rows_b, p.b_rs, 1, p.K, wave & 3, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  half8 fa[FM], fb[FN];

  const int32_t T = (int32_t)((p.K + 31) / 32);
  if (grp == 0) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
      la.issue(s, smem + s * STAGE);
      lb.issue(s, smem + s * STAGE + ABYTES);
    }
    wait_vmem_n<(STAGES - 2) * LOADS>();  // tile 0 landed
  }
  phase_barrier();               // b0
  if (grp == 1) phase_barrier(); // group 1 starts one phase behind

  for (int32_t t = 0; t < T; ++t) {
    const char* cur = smem + (t % STAGES) * STAGE;
    char* fut = smem + ((t + STAGES - 1) % STAGES) * STAGE;
    // ---- M(t)
    if (grp == 0) {
      la.issue(t + STAGES - 1, fut);  // fully out of range past the last tile
      lb.issue(t + STAGES - 1, fut + ABYTES);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, 0, SHIFT, RB));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = *(const half8*)(cur + ABYTES + fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, 0, SHIFT, RB));
    phase_barrier();
    // ---- C(t)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    if (grp == 0) wait_vmem_n<(STAGES - 2) * LOADS>();  // tile t+1 landed
    phase_barrier();
  }
  if (grp == 0) {
    wait_vmem();  // the out-of-range copies past the last tile
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
    phase_barrier();
  } else {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// Ping-pong with deep prefetch and a spread copy: as above, but every wave
// copies an eighth of each tile, and issues its copy instructions one per 8
// MFMAs inside its own compute phase (copy of tile t+STAGES-1 during C(t),
// into the buffer of tile t-1 whose last readers finished before b2t).  The
// memory phases hold only fragment reads, so both phases of every SIMD are
// balanced.  Before barrier b2t+2 both groups have their part of tile t+1
// landed: group 0 (at the end of C(t), copies issued up to tile t+S-1) allows
// S-2 tiles in flight, group 1 (at the end of M(t), copies up to tile
// t+S-2) allows S-3.
template <int STAGES, int SHIFT>
__global__ __launch_bounds__(512, 2) void gemm_f16_pps2_kernel(const GemmParams p) {
  static_assert(STAGES >= 3, "group 1 waits for S-3 tiles");
  constexpr int BM = 256, BN = 256;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int RB = 64;
  constexpr int ABYTES = BM * RB, BBYTES = BN * RB;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  using LA = LoaderKVec<BM, 512, SHIFT, 2, RB>;
  using LB = LoaderKVec<BN, 512, SHIFT, 2, RB>;
  constexpr int LOADS = LA::ITERS + LB::ITERS;  // copy instructions per tile per wave
  static_assert(LA::ITERS == 2 && LB::ITERS == 2, "copy layout");

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t grp = wave >> 2;
  const int32_t wm = wave & 1, wn = wave >> 1;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);
  LA la(A, rows_a, p.a_rs, 1, p.K, wave, lane);
  LB lb(B, rows_b, p.b_rs, 1, p.K, wave, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  half8 fa[FM], fb[FN];

  const int32_t T = (int32_t)((p.K + 31) / 32);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    la.issue(s, smem + s * STAGE);
    lb.issue(s, smem + s * STAGE + ABYTES);
  }
  wait_vmem_n<(STAGES - 2) * LOADS>();  // this wave's part of tile 0 landed
  phase_barrier();                       // b0
  if (grp == 1) phase_barrier();

  for (int32_t t = 0; t < T; ++t) {
    const char* cur = smem + (t % STAGES) * STAGE;
    char* fut = smem + ((t + STAGES - 1) % STAGES) * STAGE;
    // ---- M(t)
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, 0, SHIFT, RB));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = *(const half8*)(cur + ABYTES + fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, 0, SHIFT, RB));
    if (grp == 1) wait_vmem_n<(STAGES - 3) * LOADS>();  // group 1's part of tile t+1
    phase_barrier();
    // ---- C(t): 32 MFMAs with the 4 copy instructions of tile t+S-1 spread in
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      if (i % 2 == 1) {
        const int c = i / 2;  // 0..3
        if (c < 2)
          la.issue_one(t + STAGES - 1, fut, c);
        else
          lb.issue_one(t + STAGES - 1, fut + ABYTES, c - 2);
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // 8 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy instruction
    }
    if (grp == 0) wait_vmem_n<(STAGES - 2) * LOADS>();  // group 0's part of tile t+1
    phase_barrier();
  }
  wait_vmem();  // the out-of-range copies past the last tile
  if (grp == 0) {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
    phase_barrier();
  } else {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

// Ping-pong on 64-wide K-tiles (two LDS stages) where group 1 alone copies,
// spreading the copy instructions of tile t+2 over its compute phase C(t),
// one per 4 MFMAs; the memory phases hold only fragment reads.
//   group 0:  b0 M(0) b1 C(0) b2 M(1) b3 ...      C(T-1) b2T  [epilogue] b2T+1
//   group 1:  b0 copy(1) b1 M(0) b2 C(0)+copy(2) b3 M(1) b4 ... C(T-1) b2T+1
// Tile t+2 goes into the buffer of tile t during C(t) of group 1, i.e. after
// b2t+2, when M(t) of both groups (the buffer's last readers) is over.  Group
// 1 waits for the copy of tile t+1 at the end of its M(t), before b2t+2,
// ahead of the first read of tile t+1 (M(t+1) of group 0).  Tile 0 is copied
// by all waves before b0; tile 1 by group 1 in its first phase.
template <int SHIFT>
__global__ __launch_bounds__(512, 2) void gemm_f16_ppg_kernel(const GemmParams p) {
  constexpr int BM = 256, BN = 256;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  using LA = LoaderKVec<BM, 256, SHIFT, 2>;
  using LB = LoaderKVec<BN, 256, SHIFT, 2>;
  static_assert(LA::ITERS == 8 && LB::ITERS == 8, "copy layout");

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t grp = wave >> 2;
  const int32_t wm = wave & 1, wn = wave >> 1;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);
  // each group's four waves can copy a whole tile
  LA la(A, rows_a, p.a_rs, 1, p.K, wave & 3, lane);
  LB lb(B, rows_b, p.b_rs, 1, p.K, wave & 3, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  half8 fa[2][FM], fb[2][FN];

  const int32_t T = p.k_tiles;
  if (grp == 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    wait_vmem();
  }
  phase_barrier();  // b0: tile 0 in LDS
  if (grp == 1) {
    la.issue(1, smem + STAGE);  // out of range if there is no tile 1
    lb.issue(1, smem + STAGE + ABYTES);
    phase_barrier();  // b1
  }

  for (int32_t t = 0; t < T; ++t) {
    const char* cur = smem + (t & 1) * STAGE;
    char* cpy = smem + (t & 1) * STAGE;  // tile t+2 reuses tile t's buffer
    // ---- M(t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[ks][i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, ks, SHIFT));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[ks][j] =
            *(const half8*)(cur + ABYTES + fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, ks, SHIFT));
    }
    if (grp == 1) wait_vmem();  // the copy of tile t+1 landed (before b2t+2)
    phase_barrier();
    // ---- C(t): one MFMA sequence; group 1 issues a copy instruction of
    // tile t+2 after every 4 MFMAs (a wave-uniform branch)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
        if (grp == 1) {
          const int c = ks * FM + i;  // 0..15: eight A then eight B row blocks
          if (c < 8)
            la.issue_one(t + 2, cpy, c);
          else
            lb.issue_one(t + 2, cpy + ABYTES, c - 8);
        }
      }
    phase_barrier();
  }
  if (grp == 0) {
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
    phase_barrier();  // b2T+1
  } else {
    wait_vmem();  // the out-of-range copies past the last tile
    epilogue<FM, FN>(acc, p, tc.batch, m0 + a_row0, n0 + b_row0, lane);
  }
}

template <int BM, int BN, int WM, int WN, int AL, int BL, int PIPE, int DT>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.tiles_m * p.tiles_n;
  dim3 grid((uint32_t)total), block(WM * WN * 64);
  if constexpr (BM == 256 && BN == 256 && WM == 2 && WN == 4 && PIPE == 0) {
    if (rows_epilogue_ok(p)) {
      if (total <= kCUs)
        hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, AL, BL, 0, PIPE, DT, true, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, AL, BL, 0, PIPE, DT, true>), grid, block, 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, AL, BL, 0, PIPE, DT>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int STAGES, int RB, int DT>
hipError_t launch_ms(const GemmParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.splits * p.batch * p.tiles_m * p.tiles_n;
  dim3 grid((uint32_t)total), block(WM * WN * 64);
  hipLaunchKernelGGL((gemm_f16_ms_kernel<BM, BN, WM, WN, STAGES, 0, RB, DT>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int AL, int BL, int DT>
hipError_t launch_tile(const GemmParams& p, int32_t tile, hipStream_t s) {
  switch (tile) {
    case T256x256_W2x2: return launch_cfg<256, 256, 2, 2, AL, BL, 0, DT>(p, s);
    case T256x128_W2x2: return launch_cfg<256, 128, 2, 2, AL, BL, 0, DT>(p, s);
    case T128x256_W2x2: return launch_cfg<128, 256, 2, 2, AL, BL, 0, DT>(p, s);
    case T128x128_W2x2: return launch_cfg<128, 128, 2, 2, AL, BL, 0, DT>(p, s);
    case T256x256_W2x4: return launch_cfg<256, 256, 2, 4, AL, BL, 0, DT>(p, s);
    case T256x256_W2x4_P: return launch_cfg<256, 256, 2, 4, AL, BL, 1, DT>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// the ping-pong variants (fp16 only)
hipError_t launch_pingpong(const GemmParams& p, int32_t tile, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.tiles_m * p.tiles_n;
  const dim3 g((uint32_t)total), b(512);
  switch (tile) {
    case T256x256_PP: hipLaunchKernelGGL(gemm_f16_pp_kernel<0>, g, b, 0, s, p); break;
    case T256x256_PPS4: hipLaunchKernelGGL((gemm_f16_pps_kernel<4, 0>), g, b, 0, s, p); break;
    case T256x256_PPS5: hipLaunchKernelGGL((gemm_f16_pps_kernel<5, 0>), g, b, 0, s, p); break;
    case T256x256_PPC4: hipLaunchKernelGGL((gemm_f16_pps2_kernel<4, 0>), g, b, 0, s, p); break;
    case T256x256_PPC5: hipLaunchKernelGGL((gemm_f16_pps2_kernel<5, 0>), g, b, 0, s, p); break;
    case T256x256_PPG: hipLaunchKernelGGL(gemm_f16_ppg_kernel<0>, g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// the ring kernel (tiles 19 and 20): at least one K-tile, no K-split; the
// row epilogue when every 256 x 256 tile is full and C and D rows allow it;
// the whole-K-tile copies when both operands are K-contiguous and K is a
// multiple of the 64-wide K-tile
template <int DT, int AL, int BL, int BN>
hipError_t launch_ring(const GemmParams& p, hipStream_t s) {
  if (p.k_tiles < 1 || p.splits != 1) return hipErrorInvalidValue;
  const dim3 g((uint32_t)((int64_t)p.batch * p.tiles_m * p.tiles_n)), b(256);
  const bool rows = BN == 256 && rows_epilogue_ok(p);
  if constexpr (AL == LOAD_KVEC && BL == LOAD_KVEC) {
    if (p.K % 64 == 0) {
      if constexpr (BN == 256) {
        if (rows) {
          hipLaunchKernelGGL((gemm_f16_w4r_kernel<0, DT, true, AL, BL, BN, true>), g, b, 0, s, p);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((gemm_f16_w4r_kernel<0, DT, false, AL, BL, BN, true>), g, b, 0, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (BN == 256) {
    if (rows) {
      hipLaunchKernelGGL((gemm_f16_w4r_kernel<0, DT, true, AL, BL, BN>), g, b, 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_f16_w4r_kernel<0, DT, false, AL, BL, BN>), g, b, 0, s, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_typed(const GemmParams& p, int32_t tile, int32_t a_load, int32_t b_load, hipStream_t s) {
  if (a_load == LOAD_GENERIC || b_load == LOAD_GENERIC) {
    // one configuration for every stride pattern
    if (tile != T128x128_W2x2) return hipErrorInvalidValue;
    if (a_load == LOAD_GENERIC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_GENERIC, 0, DT>(p, s);
    if (a_load == LOAD_GENERIC && b_load == LOAD_KVEC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_KVEC, 0, DT>(p, s);
    if (a_load == LOAD_KVEC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_KVEC, LOAD_GENERIC, 0, DT>(p, s);
    if (a_load == LOAD_GENERIC && b_load == LOAD_MNVEC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_MNVEC, 0, DT>(p, s);
    if (a_load == LOAD_MNVEC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_MNVEC, LOAD_GENERIC, 0, DT>(p, s);
    return hipErrorInvalidValue;
  }
  if (a_load == LOAD_KVEC && b_load == LOAD_KVEC) {
    switch (tile) {
      case T256x256_W2x4_S3: return launch_ms<256, 256, 2, 4, 3, 64, DT>(p, s);
      case T256x256_W2x4_S4: return launch_ms<256, 256, 2, 4, 4, 64, DT>(p, s);
      case T256x256_W2x4_S5: return launch_ms<256, 256, 2, 4, 5, 64, DT>(p, s);
      case T32x128_STREAM: return launch_ms<32, 128, 1, 4, 6, 128, DT>(p, s);
      case T128x128_SPLITK: return launch_ms<128, 128, 2, 4, 3, 128, DT>(p, s);
      case T256x128_SPLITK: return launch_ms<256, 128, 4, 2, 3, 128, DT>(p, s);
      case T256x192_W2x4: return launch_cfg<256, 192, 2, 4, LOAD_KVEC, LOAD_KVEC, 0, DT>(p, s);
      case T256x256_W4R: return launch_ring<DT, LOAD_KVEC, LOAD_KVEC, 256>(p, s);
      case T256x192_W4R: return launch_ring<DT, LOAD_KVEC, LOAD_KVEC, 192>(p, s);
      case T256x256_PP:
      case T256x256_PPS4:
      case T256x256_PPS5:
      case T256x256_PPC4:
      case T256x256_PPC5:
      case T256x256_PPG:
        if constexpr (DT == DT_F16) return launch_pingpong(p, tile, s);
        return hipErrorInvalidValue;
      default: return launch_tile<LOAD_KVEC, LOAD_KVEC, DT>(p, tile, s);
    }
  }
  if (a_load == LOAD_NVFP4 || b_load == LOAD_NVFP4 || a_load == LOAD_NVFP4_PAIRS || b_load == LOAD_NVFP4_PAIRS) {
    // the dequantising loaders exist for the 4-wave ring schedule and the
    // 8-wave 256x256 fp16 kernel
    if constexpr (DT != DT_F16) return hipErrorInvalidValue;
    if (a_load != b_load) return hipErrorInvalidValue;
    if (tile == T256x256_W4R) {
      if (p.k_tiles < 1 || p.splits != 1) return hipErrorInvalidValue;
      const dim3 g((uint32_t)((int64_t)p.batch * p.tiles_m * p.tiles_n)), b(256);
      const bool rows = rows_epilogue_ok(p);
      const bool pairs = a_load == LOAD_NVFP4_PAIRS;
      if (pairs && rows) hipLaunchKernelGGL((gemm_nvfp4_w4r_kernel<0, true, true>), g, b, 0, s, p);
      if (pairs && !rows) hipLaunchKernelGGL((gemm_nvfp4_w4r_kernel<0, true, false>), g, b, 0, s, p);
      if (!pairs && rows) hipLaunchKernelGGL((gemm_nvfp4_w4r_kernel<0, false, true>), g, b, 0, s, p);
      if (!pairs && !rows) hipLaunchKernelGGL((gemm_nvfp4_w4r_kernel<0, false, false>), g, b, 0, s, p);
      return hipGetLastError();
    }
    if (tile != T256x256_W2x4) return hipErrorInvalidValue;
    if (a_load == LOAD_NVFP4_PAIRS) return launch_cfg<256, 256, 2, 4, LOAD_NVFP4_PAIRS, LOAD_NVFP4_PAIRS, 0, DT_F16>(p, s);
    return launch_cfg<256, 256, 2, 4, LOAD_NVFP4, LOAD_NVFP4, 0, DT_F16>(p, s);
  }

  if (a_load == LOAD_MNDMA || b_load == LOAD_MNDMA) {
    // the M-major direct-copy tiles exist for the 256x256 ring kernel and
    // the 8-wave 256x256 kernel
    if (tile == T256x256_W4R) {
      if (a_load == LOAD_MNDMA && b_load == LOAD_KVEC) return launch_ring<DT, LOAD_MNDMA, LOAD_KVEC, 256>(p, s);
      if (a_load == LOAD_KVEC && b_load == LOAD_MNDMA) return launch_ring<DT, LOAD_KVEC, LOAD_MNDMA, 256>(p, s);
      if (a_load == LOAD_MNDMA && b_load == LOAD_MNDMA) return launch_ring<DT, LOAD_MNDMA, LOAD_MNDMA, 256>(p, s);
      return hipErrorInvalidValue;
    }
    if (tile != T256x256_W2x4) return hipErrorInvalidValue;
    if (a_load == LOAD_MNDMA && b_load == LOAD_KVEC)
      return launch_cfg<256, 256, 2, 4, LOAD_MNDMA, LOAD_KVEC, 0, DT>(p, s);
    if (a_load == LOAD_KVEC && b_load == LOAD_MNDMA)
      return launch_cfg<256, 256, 2, 4, LOAD_KVEC, LOAD_MNDMA, 0, DT>(p, s);
    if (a_load == LOAD_MNDMA && b_load == LOAD_MNDMA)
      return launch_cfg<256, 256, 2, 4, LOAD_MNDMA, LOAD_MNDMA, 0, DT>(p, s);
    return hipErrorInvalidValue;
  }
  if (tile > T256x256_W2x4_P) return hipErrorInvalidValue;
  if (a_load == LOAD_MNVEC && b_load == LOAD_KVEC) return launch_tile<LOAD_MNVEC, LOAD_KVEC, DT>(p, tile, s);
  if (a_load == LOAD_KVEC && b_load == LOAD_MNVEC) return launch_tile<LOAD_KVEC, LOAD_MNVEC, DT>(p, tile, s);
  if (a_load == LOAD_MNVEC && b_load == LOAD_MNVEC) return launch_tile<LOAD_MNVEC, LOAD_MNVEC, DT>(p, tile, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_splitk_reduce(const GemmParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.M * ((p.N + 3) / 4);
  const int64_t blocks = (total + 255) / 256;
  const dim3 g((uint32_t)(blocks < 4096 ? blocks : 4096)), b(256);
  if (p.flags & F_BF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<DT_BF16>, g, b, 0, s, p);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<DT_F16>, g, b, 0, s, p);
  return hipGetLastError();
}

// An NVFP4 operand decoded to fp16 ahead of the product: rows x K packed
// E2M1 values (element (b, r, k) at byte (b bs + r rs + k) / 2, low nibble
// first) with one E4M3 scale per 16 K (at s + b sbs + r srs + (k / 16) sks)
// become fp16 rows of K contiguous values, batch after batch.  A thread turns
// one scale block (8 bytes, 16 values) into 32 bytes of fp16 with the fused
// loader's arithmetic (e2m1x8_to_half8, then an fp16 product with the
// decoded scale: exact), so the fp16 kernel that follows computes the same
// result bit for bit.  Consecutive threads take consecutive blocks of a row.
__global__ __launch_bounds__(256) void nvfp4_decode_kernel(const Nvfp4Decode d) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  auto mul = [](uint32_t x, _Float16 sc) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, x) * half2v{sc, sc});
  };
  const int64_t nb = d.K / 16;
  const int64_t total = (int64_t)d.batch * d.rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t kb = i % nb, rb = i / nb;  // rb = b rows + r
    const int64_t r = rb % d.rows, b = rb / d.rows;
    const u32x2 w = *(const u32x2*)(d.x + (b * d.bs + r * d.rs) / 2 + kb * 8);
    const _Float16 sc = e4m3_to_half(d.s[b * d.sbs + r * d.srs + kb * d.sks]);
    const u32x4 lo = e2m1x8_to_half8(w[0]);
    const u32x4 hi = e2m1x8_to_half8(w[1]);
    u32x4* out = (u32x4*)(d.out + rb * d.K + kb * 16);
    out[0] = u32x4{mul(lo[0], sc), mul(lo[1], sc), mul(lo[2], sc), mul(lo[3], sc)};
    out[1] = u32x4{mul(hi[0], sc), mul(hi[1], sc), mul(hi[2], sc), mul(hi[3], sc)};
  }
}

hipError_t launch_nvfp4_decode(const Nvfp4Decode& d, hipStream_t s) {
  const int64_t total = (int64_t)d.batch * d.rows * (d.K / 16);
  if (total <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(nvfp4_decode_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_gemm_f16(const GemmParams& p, int32_t tile, int32_t a_load, int32_t b_load, hipStream_t s) {
  if (p.flags & F_BF16) return launch_typed<DT_BF16>(p, tile, a_load, b_load, s);
  return launch_typed<DT_F16>(p, tile, a_load, b_load, s);
}

}  // namespace sl
