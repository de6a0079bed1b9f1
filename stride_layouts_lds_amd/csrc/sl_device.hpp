// sl_device.hpp -- device-side building blocks of the GEMM kernels: vector
// types, buffer resources, the XCD-aware tile order, and the three
// HBM -> LDS tile loaders.  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sl_kernels.hpp"
#include "sl_maps.hpp"

namespace sl {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// One 16x16x32 MFMA step on 16-bit operands of element type DT (the
// fragments travel as 16 raw bytes; fp16 and bf16 share the operand and
// accumulator layouts).
template <int DT>
__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// 16-bit element of type DT -> fp32 (exact), and fp32 -> DT rounded to
// nearest-even (overflow to infinity)
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (DT == DT_F16)
    return (float)__builtin_bit_cast(_Float16, bits);
  else
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float v) {
  if constexpr (DT == DT_F16)
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  else
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

using lds_void_t = __attribute__((address_space(3))) void;

// A buffer load whose offset is at or beyond the resource's byte count
// returns zero; every masked lane uses this offset.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts.
constexpr int32_t kRsrcWord3 = 0x00020000;

// The base and size are the same in every lane; reading them from the first
// lane tells the compiler so, and keeps the resource in scalar registers
// (a resource it cannot prove uniform is issued once per distinct value).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)u, (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}

// Wait until every vector-memory operation of this wave (including
// direct-to-LDS loads) has completed.  s_waitcnt vmcnt(0), other counters
// left at their maximum.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Phase barrier of the ping-pong schedule: this wave's LDS reads are
// complete (lgkmcnt(0)), then s_barrier.  Direct HBM->LDS copies stay in
// flight across it (a fence would wait for them: the hardware counts them
// with the vector-memory counter).  The memory clobber keeps the compiler
// from moving memory operations across it, the scheduling barriers keep it
// from moving anything else (MFMAs included), so the phases stay separate.
// A copy is made visible by the issuing wave's wait_vmem() before a later
// phase barrier.  The LDS wait is the builtin, not part of the assembly: the
// compiler's wait-count pass then knows that every earlier LDS read has
// completed (a wait inside inline assembly is invisible to it, and it put a
// full LDS wait, the read just issued included, before the first MFMAs after
// each barrier: 1-2% of the ring kernels' time).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), the other counters at their maximum
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still
// outstanding (they complete in issue order).  vmcnt is split over bits
// [3:0] and [15:14]; expcnt (bits [6:4]) and lgkmcnt ([11:8]) at maximum.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ---------------------------------------------------------------------------
// Tile order.  Workgroup IDs are handed to the 8 XCDs round-robin; remap so
// that each XCD owns a contiguous range of the logical order, then walk the
// output tiles in groups of `group_m` tile-rows so that the workgroups
// resident on one XCD share A rows and B columns in that XCD's L2.
// ---------------------------------------------------------------------------
struct TileCoord {
  int32_t batch, tm, tn, split;
};

// `total` workgroups hold `total / (batch * tiles_m * tiles_n)` K-splits of
// the output tiles; the splits are the slowest-varying index, so the
// workgroups of one split (which read the same K range of a shared
// operand) sit on neighbouring XCD ranges.
__device__ __forceinline__ TileCoord map_tile(int32_t bid, int32_t total, int32_t tiles_m, int32_t tiles_n,
                                              int32_t group_m, int32_t batch) {
  const int32_t x = bid & 7, local = bid >> 3;
  const int32_t q = total >> 3, r = total & 7;
  int32_t id = x * q + (x < r ? x : r) + local;
  const int32_t per_batch = tiles_m * tiles_n;
  const int32_t split = id / (batch * per_batch);
  id -= split * batch * per_batch;
  const int32_t b = id / per_batch;
  const int32_t t = id - b * per_batch;
  const int32_t span = group_m * tiles_n;
  const int32_t g = t / span;
  const int32_t first_m = g * group_m;
  const int32_t left = tiles_m - first_m;
  const int32_t gsz = left < group_m ? left : group_m;
  const int32_t in = t - g * span;
  return TileCoord{b, first_m + in % gsz, in / gsz, split};
}

// ---------------------------------------------------------------------------
// Epilogue store of four consecutive outputs (m, n..n+3) of one lane:
// D = round(v + C) to D's 16-bit type DT (nearest-even), predicated on
// m < M and n + r < N.  8-byte accesses
// when the row is contiguous and aligned (F_D_VEC / F_C_VEC) and all four
// columns are in range.
// ---------------------------------------------------------------------------
// C's four values at (m, n..n+3) as 16-bit codes (zero where out of range)
__device__ __forceinline__ u16x4 load_c_quad(const GemmParams& p, const uint16_t* C, int64_t m, int64_t n) {
  u16x4 cv = {0, 0, 0, 0};
  if (m >= p.M || n >= p.N) return cv;
  const uint16_t* cp = C + m * p.c_rs + n * p.c_cs;
  if (n + 3 < p.N && (p.flags & F_C_VEC)) return *(const u16x4*)cp;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (n + r < p.N) cv[r] = cp[r * p.c_cs];
  return cv;
}

// D(m, n..n+3) = round(v) to DT, predicated on m < M and n + r < N
template <int DT = DT_F16>
__device__ __forceinline__ void store_d_quad(const GemmParams& p, uint16_t* D, int64_t m, int64_t n, floatx4 v) {
  if (m >= p.M || n >= p.N) return;
  uint16_t* dp = D + m * p.d_rs + n * p.d_cs;
  if (n + 3 < p.N && (p.flags & F_D_VEC)) {
    *(u16x4*)dp = u16x4{from_f32<DT>(v[0]), from_f32<DT>(v[1]), from_f32<DT>(v[2]), from_f32<DT>(v[3])};
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < p.N) dp[r * p.d_cs] = from_f32<DT>(v[r]);
  }
}

template <int DT = DT_F16>
__device__ __forceinline__ void store_quad(const GemmParams& p, const uint16_t* C, uint16_t* D, int64_t m,
                                           int64_t n, floatx4 v) {
  if (p.flags & F_HAS_C) {
    const u16x4 cv = load_c_quad(p, C, m, n);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += to_f32<DT>(cv[r]);
  }
  store_d_quad<DT>(p, D, m, n, v);
}

// ---------------------------------------------------------------------------
// Row epilogue of a wave's 128 x COLS output block (COLS = 128 or 64), for
// full tiles with contiguous, 8-byte aligned C and D rows.  The block goes
// through a private LDS region of 64 rows x COLS fp32 (32 or 16 KiB) in two
// halves of 64 rows, row-major with the 16-byte chunk q of row r at chunk
// q ^ (r % 16) (rows_chunk): free of bank conflicts both for
// accumulator-order writes (16 rows at one chunk per 16 lanes) and for
// row-order reads.  Read back one row-contiguous 16-byte piece per lane
// (COLS / 4 lanes per row, 256 / COLS rows per instruction), added to C and
// stored as 8 bytes, every C load and D store instruction covers whole
// 128-byte row segments; in accumulator order one touches 16 rows.  All of
// the lane's C loads are issued first.  NT: the D stores carry the
// non-temporal hint (D is not read again).
// ---------------------------------------------------------------------------
template <int COLS = 128>
__device__ __forceinline__ int32_t rows_chunk(int32_t r, int32_t q) {
  static_assert(COLS == 128 || COLS == 64, "row epilogue block width");
  return r * (4 * COLS) + 16 * (q ^ (r & 15));
}

// C of the lane's row-order pieces of both halves (rows (256 / COLS) it +
// lane / (COLS / 4), columns 4 (lane % (COLS / 4)) .. + 3); nothing when
// there is no C
template <int COLS = 128>
__device__ __forceinline__ void rows_load_c(const GemmParams& p, int32_t batch, int64_t m_base, int64_t n_base,
                                            int32_t lane, u16x4 (&cq)[2][COLS / 4]) {
  constexpr int LPR = COLS / 4, RPI = 64 / LPR;
  if (!(p.flags & F_HAS_C)) return;
  const uint16_t* C = (const uint16_t*)p.c + batch * p.c_bs;
  const int32_t q = lane % LPR, rl = lane / LPR;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int it = 0; it < LPR; ++it)
      cq[h][it] = *(const u16x4*)(C + (m_base + 64 * h + RPI * it + rl) * p.c_rs + n_base + 4 * q);
}

// D rows m_base .. m_base + 63 from the region (+ C), one half
template <int DT, int COLS = 128, bool NT = false>
__device__ __forceinline__ void rows_store_half(const GemmParams& p, int32_t batch, int64_t m_base, int64_t n_base,
                                                int32_t lane, const char* region, const u16x4 (&cq)[COLS / 4]) {
  constexpr int LPR = COLS / 4, RPI = 64 / LPR;
  uint16_t* D = (uint16_t*)p.d + batch * p.d_bs;
  const bool has_c = p.flags & F_HAS_C;
  const int32_t q = lane % LPR, rl = lane / LPR;
#pragma unroll
  for (int it = 0; it < LPR; ++it) {
    const int32_t r = RPI * it + rl;
    floatx4 v = *(const floatx4*)(region + rows_chunk<COLS>(r, q));
    if (has_c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += to_f32<DT>(cq[it][e]);
    }
    const u16x4 d = u16x4{from_f32<DT>(v[0]), from_f32<DT>(v[1]), from_f32<DT>(v[2]), from_f32<DT>(v[3])};
    u16x4* dp = (u16x4*)(D + (m_base + r) * p.d_rs + n_base + 4 * q);
    if constexpr (NT)
      __builtin_nontemporal_store(d, dp);
    else
      *dp = d;
  }
}

// ---------------------------------------------------------------------------
// HBM -> LDS tile loaders.  A tile is ROWS rows (of A's m or B's n) by 128
// bytes of K (64 fp16 or 128 fp8 values), stored in LDS through
// lds_offset(row, byte, SHIFT).  Each loader exposes
//   issue(t, lds)  : start bringing K-tile t (direct loaders write LDS here)
//   commit(lds)    : finish writing K-tile t into LDS (staged loaders)
// Out-of-range rows and K positions read as zero (both operands must be
// zero past K: 0 * stale NaN would poison the sum).
// ---------------------------------------------------------------------------

// K-contiguous rows, 16-B aligned: each lane's 16-B chunk is fetched by a
// direct HBM->LDS buffer load.  One wave instruction fills 1 KiB of LDS,
// i.e. 1024/RB consecutive rows, lane l landing at byte 16*l of that block.
// The swizzle is therefore realised on the global side: the lane that
// lands in physical chunk p of row r fetches logical chunk p ^ swz(r).
// TB < RB: a K-tile is TB bytes of each row (packed 6-bit data: 128 values
// in 96 bytes); the row's chunks past TB are filled with zeros and never
// read, and K-tile t starts t*TB bytes into the row.
template <int ROWS, int NT, int SHIFT, int ELEM, int RB = kRowBytes, int TB = RB>
struct LoaderKVec {
  static constexpr int WAVES = NT / 64;
  static constexpr int CPR = RB / 16;          // chunks per row
  static constexpr int RPI = 1024 / RB;        // rows per wave instruction
  static constexpr int ITERS = ROWS * RB / (NT * 16);
  static constexpr int KT = TB / ELEM;         // K elements per tile
  static constexpr int CE = 16 / ELEM;         // K elements per 16-B chunk
  static constexpr int CT = TB / 16;           // chunks of a row that hold the tile
  static_assert(ITERS >= 1 && ROWS * RB % (NT * 16) == 0, "tile too small for the workgroup");
  static_assert(TB <= RB && TB % 16 == 0, "tile bytes per row");

  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_off;   // byte offset of this lane's row in instruction 0
  uint32_t row_step;  // bytes between the row blocks of consecutive instructions
  int32_t row0;       // this lane's tile row in instruction 0
  int32_t K;
  int32_t wave;
  int32_t lane;
  // this lane's byte offset in copy j of K-tile 0 (kOutOfRange for chunks
  // past the tile's bytes): loop-invariant, for issue_full
  uint32_t voff[ITERS];

  __device__ __forceinline__ LoaderKVec(const void* base, int32_t rows_valid, int64_t rs, int64_t /*ks*/,
                                        int64_t K_, int32_t wave_, int32_t lane_) {
    K = (int32_t)K_;
    wave = wave_;
    lane = lane_;
    const uint32_t bytes =
        rows_valid > 0 ? (uint32_t)(((int64_t)(rows_valid - 1) * rs + K_) * ELEM) : 0u;
    rsrc = make_rsrc(base, bytes);
    row0 = wave * RPI + lane / CPR;
    row_off = (uint32_t)(row0 * rs * ELEM);
    row_step = (uint32_t)(WAVES * RPI * rs * ELEM);
#pragma unroll
    for (int j = 0; j < ITERS; ++j) {
      const int32_t c = (lane % CPR) ^ swz(row0 + j * WAVES * RPI, SHIFT, RB);
      voff[j] = c < CT ? row_off + (uint32_t)j * row_step + (uint32_t)(c * 16) : kOutOfRange;
    }
  }

  // one copy instruction: j-th row block of K-tile t
  __device__ __forceinline__ void issue_one(int32_t t, char* lds, int j) const {
    // instruction j covers rows (j*WAVES + wave)*RPI + 0..RPI-1
    const int32_t row = row0 + j * WAVES * RPI;
    const int32_t c = (lane % CPR) ^ swz(row, SHIFT, RB);
    const uint32_t a = row_off + (uint32_t)j * row_step + (uint32_t)(c * 16) + (uint32_t)(t * TB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (j * WAVES + wave) * 1024), 16,
                                             (c < CT && t * KT + c * CE < K) ? a : kOutOfRange, 0, 0, 0);
  }

  // The same copy for a K-tile that lies wholly inside K (0 <= t and
  // (t + 1) * KT <= K): the per-lane offset is voff[j] and the K-tile's
  // start goes into the instruction's scalar offset, so the copy waits on
  // no vector arithmetic (next to the MFMA stream a vector result consumed
  // at once by a memory instruction stalls the wave).  Rows past the valid
  // ones still read zero: their offset alone is past the resource's bytes.
  // (The element is copied to a local first: the host compilation pass
  // drops the launch stubs of kernels that index the member array inside
  // the builtin's argument list.)
  __device__ __forceinline__ void issue_full(int32_t t, char* lds, int j) const {
    const uint32_t v = voff[j];
    const uint32_t s = (uint32_t)(t * TB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (j * WAVES + wave) * 1024), 16, v, s, 0, 0);
  }

  __device__ __forceinline__ void issue(int32_t t, char* lds) const {
#pragma unroll
    for (int j = 0; j < ITERS; ++j) issue_one(t, lds, j);
  }
  __device__ __forceinline__ void commit(char*) const {}
};

// Packed 6-bit K-tiles for the 4-wave MX kernel, copied as they lie: a
// row's K-tile (128 values, 96 bytes) is 6 consecutive 16-byte chunks of
// LDS, rows 96 bytes apart, so a K-tile of 256 rows takes 24 copy
// instructions (a wave's 64 lanes fill 64 consecutive chunks, 10 2/3 rows)
// where 128-byte LDS rows take 32.  On rows 16-31 of every 32 the chunk
// order is rotated by one (fp6_packed_chunk): the kernel's 16-byte fragment
// reads (one chunk of 32 rows, lanes paired as gfx950 serves them) then hit
// distinct banks; its 8-byte reads take two passes.  Every K-tile must lie
// inside K (the 4-wave MX kernel's condition: K a multiple of 512).
SL_HD constexpr int32_t fp6_packed_chunk(int32_t row, int32_t c) { return (c + ((row >> 4) & 1)) % 6; }

template <int ROWS, int NT>
struct LoaderFP6Packed {
  static constexpr int WAVES = NT / 64;
  static constexpr int TB = 96;                  // bytes of a row per K-tile
  static constexpr int KT = 128;                 // values per K-tile
  static constexpr int INSTR = ROWS * 6 / 64;    // copy instructions per K-tile
  static constexpr int ITERS = INSTR / WAVES;    // ... per wave
  static_assert(ROWS * 6 % 64 == 0 && INSTR % WAVES == 0, "tile rows for the workgroup");

  __amdgpu_buffer_rsrc_t rsrc;
  int32_t wave;
  uint32_t voff[ITERS];  // this lane's byte offset in copy j of K-tile 0

  __device__ __forceinline__ LoaderFP6Packed(const void* base, int32_t rows_valid, int64_t rs_bytes,
                                             int64_t K_elems, int32_t wave_, int32_t lane) {
    wave = wave_;
    const uint32_t bytes =
        rows_valid > 0 ? (uint32_t)((int64_t)(rows_valid - 1) * rs_bytes + K_elems / 4 * 3) : 0u;
    rsrc = make_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < ITERS; ++j) {
      // copy j of this wave fills chunks 64 (j * WAVES + wave) + lane of the
      // tile: physical chunk p of row `row`, holding the row's chunk c
      const int32_t g = 64 * (j * WAVES + wave) + lane;
      const int32_t row = g / 6, p = g % 6;
      const int32_t c = (p + 6 - ((row >> 4) & 1)) % 6;
      voff[j] = (uint32_t)(row * rs_bytes) + (uint32_t)(16 * c);
    }
  }

  // copy j of K-tile t, with no vector arithmetic: the lane's offset is
  // voff[j] and the K-tile's start goes into the scalar offset (rows past
  // the valid ones read zero: their offset alone is past the resource)
  __device__ __forceinline__ void issue_full(int32_t t, char* lds, int j) const {
    const uint32_t v = voff[j];
    const uint32_t s = (uint32_t)(t * TB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (j * WAVES + wave) * 1024), 16, v, s, 0, 0);
  }
};

// M- (or N-) contiguous fp16 rows, 16-B aligned: the tile is stored in HBM
// as K rows of ROWS contiguous values.  A thread fetches KB consecutive K
// rows of one 8-value block (8 x KB halves), transposes them in registers
// and writes 8 K-contiguous pieces of KB halves into the LDS tile.
template <int ROWS, int NT, int SHIFT>
struct LoaderMNVec {
  static constexpr int MB = ROWS / 8;        // 8-row blocks
  static constexpr int KB = 64 * MB / NT;    // K rows per thread
  static_assert(KB == 8 || KB == 4, "unsupported tile for the transposing loader");

  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off0;
  uint32_t kstep;  // bytes between consecutive K rows
  int32_t mb, kbase, K;
  bool row_ok;
  u32x4 stage[KB];

  __device__ __forceinline__ LoaderMNVec(const void* base, int32_t rows_valid, int64_t /*rs*/, int64_t ks,
                                         int64_t K_, int32_t /*wave*/, int32_t /*lane*/) {
    K = (int32_t)K_;
    const int32_t tid = threadIdx.x;
    mb = tid % MB;
    kbase = (tid / MB) * KB;
    row_ok = mb * 8 < rows_valid;
    const uint32_t bytes =
        (rows_valid > 0 && K_ > 0) ? (uint32_t)(((K_ - 1) * ks + rows_valid) * 2) : 0u;
    rsrc = make_rsrc(base, bytes);
    kstep = (uint32_t)(ks * 2);
    off0 = (uint32_t)(mb * 16) + (uint32_t)kbase * kstep;
  }

  __device__ __forceinline__ void issue(int32_t t, char*) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int32_t k = t * 64 + kbase + j;
      const uint32_t o = (row_ok && k < K) ? off0 + (uint32_t)(t * 64 + j) * kstep : kOutOfRange;
      stage[j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0);
    }
  }

  __device__ __forceinline__ void commit(char* lds) const {
    // stage[j] holds values (m = 8*mb + e, k = kbase + j), e = 0..7, two per
    // 32-bit word.  Row e of the output needs (m = 8*mb + e, k = kbase + j)
    // for j = 0..KB-1.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int32_t row = mb * 8 + e;
      const int32_t byte = kbase * 2;
      uint32_t w[KB / 2];
#pragma unroll
      for (int j = 0; j < KB; j += 2) {
        const uint32_t lo = stage[j][e >> 1], hi = stage[j + 1][e >> 1];
        // select the 16-bit half e&1 of each, pack (k = j) low, (k = j+1) high
        w[j / 2] = (e & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                           : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      char* dst = lds + lds_offset(row, byte, SHIFT);
      if constexpr (KB == 8) {
        *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        *(u32x2*)dst = u32x2{w[0], w[1]};
      }
    }
  }
};

// M- (N-) contiguous fp16 rows, 16-B aligned, copied straight into the
// M-major LDS tile (mn_lds_offset): K-row k of the tile is ROWS contiguous
// values at base + k*ks.  One wave instruction fills 1 KiB of LDS, i.e.
// RPI = 1024 / (2 ROWS) consecutive K-rows, lane l landing at byte 16 l of
// that block; the lane that lands in physical chunk p of K-row k fetches
// logical chunk p ^ mn_swz(k).
template <int ROWS, int NT>
struct LoaderMNDma {
  static constexpr int WAVES = NT / 64;
  static constexpr int CPR = ROWS / 8;             // 16-byte chunks per K-row
  static constexpr int RPI = 1024 / (2 * ROWS);    // K-rows per wave instruction
  static constexpr int ITERS = 64 * ROWS * 2 / (NT * 16);
  static_assert(ROWS >= 128 && RPI >= 1 && ITERS >= 1 && 64 * ROWS * 2 % (NT * 16) == 0, "unsupported tile");

  __amdgpu_buffer_rsrc_t rsrc;
  int32_t K, wave, lane, rows_valid;
  int64_t ks;
  uint32_t voff[ITERS];  // this lane's byte offset in copy j of K-tile 0 (issue_full)
  uint32_t kstep;        // bytes between K-tiles

  __device__ __forceinline__ LoaderMNDma(const void* base, int32_t rows_valid_, int64_t /*rs*/, int64_t ks_,
                                         int64_t K_, int32_t wave_, int32_t lane_) {
    K = (int32_t)K_;
    wave = wave_;
    lane = lane_;
    rows_valid = rows_valid_;
    ks = ks_;
    const uint32_t bytes =
        (rows_valid_ > 0 && K_ > 0) ? (uint32_t)(((K_ - 1) * ks_ + rows_valid_) * 2) : 0u;
    rsrc = make_rsrc(base, bytes);
    kstep = (uint32_t)(64 * ks_ * 2);
#pragma unroll
    for (int j = 0; j < ITERS; ++j) {
      const int32_t kr = (j * WAVES + wave) * RPI + lane / CPR;
      const int32_t c = (lane % CPR) ^ mn_swz(kr);
      voff[j] = c * 8 < rows_valid_ ? (uint32_t)(((int64_t)kr * ks_ + c * 8) * 2) : kOutOfRange;
    }
  }

  // the copy of issue_one for a K-tile inside K (0 <= t, 64 (t + 1) <= K),
  // with no vector arithmetic: the lane's offset is voff[j] and the K-tile's
  // start goes into the scalar offset (as LoaderKVec::issue_full)
  __device__ __forceinline__ void issue_full(int32_t t, char* lds, int j) const {
    const uint32_t v = voff[j];
    const uint32_t s = (uint32_t)t * kstep;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (j * WAVES + wave) * 1024), 16, v, s, 0, 0);
  }

  // one copy instruction: the j-th 1 KiB block of this wave in K-tile t
  __device__ __forceinline__ void issue_one(int32_t t, char* lds, int j) const {
    const int32_t blk = j * WAVES + wave;             // 1 KiB block of the tile
    const int32_t kr = blk * RPI + lane / CPR;        // K-row inside the tile
    const int32_t c = (lane % CPR) ^ mn_swz(kr);      // logical chunk this lane fetches
    const int32_t k = t * 64 + kr;
    const bool ok = k < K && c * 8 < rows_valid;
    const uint32_t off = (uint32_t)(((int64_t)k * ks + c * 8) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + blk * 1024), 16, ok ? off : kOutOfRange,
                                             0, 0, 0);
  }
  __device__ __forceinline__ void issue(int32_t t, char* lds) const {
#pragma unroll
    for (int j = 0; j < ITERS; ++j) issue_one(t, lds, j);
  }
  __device__ __forceinline__ void commit(char*) const {}
};

typedef short short4_t __attribute__((ext_vector_type(4)));

// One fp16 MFMA fragment (8 halves of one lane) of the 16-row tile at row0,
// k-slice ks, from an LDS tile of layout KIND: K-major (every loader but
// LOAD_MNDMA) by one ds_read_b128, M-major by two transposing reads.
template <int KIND, int ROWS, int SHIFT>
__device__ __forceinline__ half8 read_frag(const char* buf, int32_t lane, int32_t row0, int32_t ks) {
  if constexpr (KIND == LOAD_MNDMA) {
    typedef __attribute__((address_space(3))) short4_t lds_s4;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(buf + tr_read_offset(lane, 0, row0, ks, ROWS)));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(buf + tr_read_offset(lane, 1, row0, ks, ROWS)));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    return *(const half8*)(buf + fragment_lds_offset(MFMA16_F16, lane, 0, row0, ks, SHIFT));
  }
}

// Any strides: every element is fetched on its own (64-bit addressing).
template <int ROWS, int NT, int SHIFT>
struct LoaderGeneric {
  static constexpr int PER = ROWS * 64 / NT;
  const uint16_t* base;
  int64_t rs, ks;
  int32_t rows_valid, K;
  uint16_t stage[PER];

  __device__ __forceinline__ LoaderGeneric(const void* base_, int32_t rows_valid_, int64_t rs_, int64_t ks_,
                                           int64_t K_, int32_t, int32_t) {
    base = (const uint16_t*)base_;
    rs = rs_;
    ks = ks_;
    rows_valid = rows_valid_;
    K = (int32_t)K_;
  }

  __device__ __forceinline__ void issue(int32_t t, char*) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = j * NT + (int32_t)threadIdx.x;
      const int32_t r = e >> 6, k = t * 64 + (e & 63);
      stage[j] = (r < rows_valid && k < K) ? base[(int64_t)r * rs + (int64_t)k * ks] : (uint16_t)0;
    }
  }

  __device__ __forceinline__ void commit(char* lds) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = j * NT + (int32_t)threadIdx.x;
      *(uint16_t*)(lds + lds_offset(e >> 6, (e & 63) * 2, SHIFT)) = stage[j];
    }
  }
};

// NVFP4 operand: K-contiguous packed E2M1 (two per byte, even element in
// the low nibble) with one E4M3 scale per 16 K.  Each thread owns one
// (row, 32-wide half) of the 64-wide K-tile: one 16-byte load of 32 codes
// and two scale bytes, decoded in registers to fp16 and multiplied by the
// scale (E2M1 x E4M3 has at most 5 significant bits and lies in
// [2^-10, 2688]: exact in fp16), then written as four 16-byte chunks of
// the K-major fp16 LDS tile.  Past K, or past the valid rows, the copies
// read zero.
__device__ __forceinline__ _Float16 e4m3_to_half(uint32_t b) {
  // branch-free: both the normal and the subnormal reading, then selects
  const uint32_t s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  const float normal = __builtin_bit_cast(float, ((e + 120) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  const float sub = (float)m * 0x1p-9f;                                          // m/8 * 2^-6
  float f = e == 0 ? sub : normal;
  f = (e == 15 && m == 7) ? __builtin_nanf("") : f;
  return (_Float16)(s ? -f : f);
}

// 8 E2M1 codes (nibbles of w, element 0 in the low nibble) -> 8 fp16 bit
// patterns, two per dword.  Every E2M1 value has a zero low byte in fp16;
// the high byte comes from an 8-entry byte table selected with v_perm_b32,
// plus the sign.
__device__ __forceinline__ u32x4 e2m1x8_to_half8(uint32_t w) {
  constexpr uint32_t kTabLo = 0x3E3C3800u;  // 0, 0.5, 1, 1.5 (high bytes)
  constexpr uint32_t kTabHi = 0x46444240u;  // 2, 3, 4, 6
  const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
  const uint32_t he = __builtin_amdgcn_perm(kTabHi, kTabLo, ev & 0x07070707u) | ((ev & 0x08080808u) << 4);
  const uint32_t ho = __builtin_amdgcn_perm(kTabHi, kTabLo, od & 0x07070707u) | ((od & 0x08080808u) << 4);
  // dword i = (element 2i, element 2i+1) = bytes [0, he.b_i, 0, ho.b_i]
  return u32x4{__builtin_amdgcn_perm(ho, he, 0x040C000Cu), __builtin_amdgcn_perm(ho, he, 0x050C010Cu),
               __builtin_amdgcn_perm(ho, he, 0x060C020Cu), __builtin_amdgcn_perm(ho, he, 0x070C030Cu)};
}

template <int ROWS, int NT, int SHIFT, bool PAIRS>
struct LoaderNVFP4 {
  static constexpr int PER = ROWS * 2 / NT;  // (row, half) units per thread
  static_assert(PER >= 1 && ROWS * 2 % NT == 0, "tile too small for the workgroup");
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));

  // PAIRS: K-tiles are fetched in pairs.  A unit's two 16-byte pieces (its
  // half of K-tiles 2p and 2p+1) lie in one 128-byte line and are requested
  // back to back, and one 8-byte load brings the row's 8 scales of the pair
  // (scale rows of unit stride on 8-byte boundaries).  issue(t) for even t
  // loads the pair, for odd t nothing; commit() decodes the tile of the last
  // issue.  Without PAIRS: one piece and two scale bytes per unit per tile.
  static constexpr int NB = PAIRS ? 2 : 1;  // tiles held per unit
  __amdgpu_buffer_rsrc_t rd, rsf;
  int32_t K;
  uint32_t sks;
  int32_t cur;  // tile of the last issue
  uint32_t d_off[PER], s_off[PER];
  int32_t row[PER], half[PER];
  bool ok[PER];
  u32x4 data[PER][NB];
  u32x2 sc8[PER];        // PAIRS: scale bytes of blocks 4t .. 4t + 7
  uint32_t sc[PER][2];   // else: the unit's two scale bytes of tile t

  __device__ __forceinline__ LoaderNVFP4(const uint8_t* base, const uint8_t* sbase, int32_t rows_valid,
                                         int64_t rs, int64_t srs, int64_t sks_, int64_t K_) {
    K = (int32_t)K_;
    sks = (uint32_t)sks_;
    cur = 0;
    rd = make_rsrc(base, rows_valid > 0 ? (uint32_t)((rows_valid - 1) * (rs / 2) + K_ / 2) : 0u);
    rsf = make_rsrc(sbase, rows_valid > 0 ? (uint32_t)((rows_valid - 1) * srs + (K_ / 16 - 1) * sks_ + 1) : 0u);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int32_t id = u * NT + (int32_t)threadIdx.x;
      row[u] = id >> 1;
      half[u] = id & 1;
      ok[u] = row[u] < rows_valid;
      d_off[u] = (uint32_t)(row[u] * (rs / 2) + half[u] * 16);
      s_off[u] = (uint32_t)(row[u] * srs + (PAIRS ? 0 : half[u] * 2 * sks_));
    }
  }

  __device__ __forceinline__ void issue(int32_t t, char*) {
    cur = t;
    if (PAIRS && (t & 1)) return;  // fetched with the pair's first tile
#pragma unroll
    for (int u = 0; u < PER; ++u) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int32_t tq = t + q;
        const bool v = ok[u] && tq * 64 + half[u] * 32 < K;
        data[u][q] = __builtin_amdgcn_raw_buffer_load_b128(rd, v ? d_off[u] + (uint32_t)(tq * 32) : kOutOfRange, 0, 0);
      }
      const bool v = ok[u] && t * 64 + half[u] * 32 < K;
      if constexpr (PAIRS) {
        sc8[u] = __builtin_amdgcn_raw_buffer_load_b64(rsf, ok[u] && t * 64 < K ? s_off[u] + (uint32_t)(4 * t)
                                                                               : kOutOfRange, 0, 0);
      } else {
        const uint32_t s0 = s_off[u] + (uint32_t)(4 * t) * sks;
        sc[u][0] = __builtin_amdgcn_raw_buffer_load_b8(rsf, v ? s0 : kOutOfRange, 0, 0);
        sc[u][1] = __builtin_amdgcn_raw_buffer_load_b8(rsf, v ? s0 + sks : kOutOfRange, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ uint32_t mul_h2(uint32_t x, _Float16 s) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, x) * half2v{s, s});
  }

  // One 16-byte piece of the fp16 tile: unit u's 8 elements K = 32 half +
  // 8 j .. of tile `cur` (its scale: block 4 cur + 2 half + j / 2, with PAIRS
  // byte 4 q + 2 half + j / 2 of the pair's 8).  The four products are built
  // as separate values: an in-place loop over the vector's elements was
  // miscompiled into reuse of element 0.
  __device__ __forceinline__ void commit_part(char* lds, int u, int j) const {
    const int32_t q = PAIRS ? (cur & 1) : 0;
    uint32_t sb;
    if constexpr (PAIRS) {
      const uint32_t w = q ? sc8[u][1] : sc8[u][0];
      sb = (w >> (16 * half[u] + 8 * (j >> 1))) & 0xFF;
    } else {
      sb = sc[u][j >> 1];
    }
    const _Float16 s = e4m3_to_half(sb);
    const u32x4 d = q ? data[u][NB - 1] : data[u][0];
    const u32x4 h = e2m1x8_to_half8(d[j]);
    *(u32x4*)(lds + lds_offset(row[u], (half[u] * 32 + 8 * j) * 2, SHIFT)) =
        u32x4{mul_h2(h[0], s), mul_h2(h[1], s), mul_h2(h[2], s), mul_h2(h[3], s)};
  }
  static constexpr int PARTS = PER * 4;  // commit_part calls of one tile
  __device__ __forceinline__ void commit(char* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) commit_part(lds, u, j);
  }
};

template <int KIND, int ROWS, int NT, int SHIFT>
struct LoaderSel;
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_KVEC, ROWS, NT, SHIFT> {
  using type = LoaderKVec<ROWS, NT, SHIFT, 2>;
};
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_MNVEC, ROWS, NT, SHIFT> {
  using type = LoaderMNVec<ROWS, NT, SHIFT>;
};
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_GENERIC, ROWS, NT, SHIFT> {
  using type = LoaderGeneric<ROWS, NT, SHIFT>;
};
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_MNDMA, ROWS, NT, SHIFT> {
  using type = LoaderMNDma<ROWS, NT>;
};
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_NVFP4, ROWS, NT, SHIFT> {
  using type = LoaderNVFP4<ROWS, NT, SHIFT, false>;
};
template <int ROWS, int NT, int SHIFT>
struct LoaderSel<LOAD_NVFP4_PAIRS, ROWS, NT, SHIFT> {
  using type = LoaderNVFP4<ROWS, NT, SHIFT, true>;
};

// The loader of operand `op` (0: A rows from m0, 1: B rows from n0) of
// batch `batch`, `rows_valid` rows of the tile in range.
template <int KIND, int ROWS, int NT, int SHIFT>
__device__ __forceinline__ typename LoaderSel<KIND, ROWS, NT, SHIFT>::type make_loader(
    const GemmParams& p, int op, int32_t batch, int64_t row0, int32_t rows_valid, int32_t wave, int32_t lane) {
  const int64_t bs = op ? p.b_bs : p.a_bs, rs = op ? p.b_rs : p.a_rs, ks = op ? p.b_ks : p.a_ks;
  const uint8_t* x = (const uint8_t*)(op ? p.b : p.a);
  if constexpr (KIND == LOAD_NVFP4 || KIND == LOAD_NVFP4_PAIRS) {
    const int64_t sbs = op ? p.sb_bs : p.sa_bs, srs = op ? p.sb_rs : p.sa_rs, sks = op ? p.sb_ks : p.sa_ks;
    const uint8_t* sf = (op ? p.sfb : p.sfa) + batch * sbs + row0 * srs;
    return typename LoaderSel<KIND, ROWS, NT, SHIFT>::type(x + (batch * bs + row0 * rs) / 2, sf, rows_valid, rs,
                                                           srs, sks, p.K);
  } else {
    return typename LoaderSel<KIND, ROWS, NT, SHIFT>::type(x + 2 * (batch * bs + row0 * rs), rows_valid, rs, ks, p.K,
                                                           wave, lane);
  }
}

}  // namespace sl
