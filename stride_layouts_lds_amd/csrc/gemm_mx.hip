// gemm_mx.hip -- MXFP8 block-scaled GEMM on gfx950:
//   D = C + (A_low * SFA) (B_low * SFB)^T,  A_low, B_low FP8 E4M3,
//   one E8M0 scale per 32 consecutive K per row of A and of B,
// i.e. the block-scaled product of "数据布局及其记号", section
// "Replication 与 Offset", with B stored (N, K) and K_blk = 32.
//
// Same data flow as the fp16 kernel: a K-tile is 128 bytes = 128 E4M3
// values per row, loaded straight into the XOR-swizzled LDS tile.  Two
// kernels: a 4-wave one on v_mfma_scale_f32_16x16x128_f8f6f4 that takes
// any scale strides (scale lane l covers (row l % 16, K block l / 16) of
// its operand, so lane l fetches the byte SF[row0 + l % 16][4 t + l / 16]
// for K-tile t), and the 8-wave one below for dword-aligned scale rows.
#include <type_traits>

#include "sl_device.hpp"

namespace sl {
namespace {

constexpr int32_t kFmtE4M3 = 0;  // CBSZ/BLGP format code of FP8 E4M3
constexpr int32_t kFmtE2M3 = 2;  // ... of FP6 E2M3
constexpr int32_t kFmtE3M2 = 3;  // ... of FP6 E3M2
constexpr int32_t kFmtE2M1 = 4;  // ... of FP4 E2M1

template <int BM, int BN, int WM, int WN, int SHIFT>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_mx_kernel(const GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave % WM, wn = wave / WM;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  const char* A = (const char*)p.a + (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + (tc.batch * p.b_bs + n0 * p.b_rs);

  LoaderKVec<BM, NT, SHIFT, 1> la(A, rows_a, p.a_rs, 1, p.K, wave, lane);
  LoaderKVec<BN, NT, SHIFT, 1> lb(B, rows_b, p.b_rs, 1, p.K, wave, lane);

  // scale resources: rows [m0, m0 + rows) of SFA / SFB
  const int32_t kblocks = (int32_t)((p.K + 31) / 32);
  const uint8_t* SA = p.sfa + tc.batch * p.sa_bs + m0 * p.sa_rs;
  const uint8_t* SB = p.sfb + tc.batch * p.sb_bs + n0 * p.sb_rs;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(SA, rows_a > 0 ? (uint32_t)((rows_a - 1) * p.sa_rs + (kblocks - 1) * p.sa_ks + 1) : 0u);
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(SB, rows_b > 0 ? (uint32_t)((rows_b - 1) * p.sb_rs + (kblocks - 1) * p.sb_ks + 1) : 0u);
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  const int32_t sblk = lane >> 4;  // K block of this lane inside the instruction
  const uint32_t sa_lane = (uint32_t)((a_row0 + (lane & 15)) * p.sa_rs);
  const uint32_t sb_lane = (uint32_t)((b_row0 + (lane & 15)) * p.sb_rs);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t T = p.k_tiles;
  if (T > 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    wait_vmem();
    __syncthreads();
  }

  for (int32_t t = 0; t < T; ++t) {
    char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    const bool more = t + 1 < T;
    // this tile's scale bytes (masked past the last K block)
    const int32_t kb = 4 * t + sblk;
    const bool kb_ok = kb < kblocks;
    int32_t sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa[i] = __builtin_amdgcn_raw_buffer_load_b8(
          ra, kb_ok ? sa_lane + (uint32_t)(16 * i * p.sa_rs + kb * p.sa_ks) : kOutOfRange, 0, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      sb[j] = __builtin_amdgcn_raw_buffer_load_b8(
          rb, kb_ok ? sb_lane + (uint32_t)(16 * j * p.sb_rs + kb * p.sb_ks) : kOutOfRange, 0, 0);
    if (more) {
      la.issue(t + 1, nxt);
      lb.issue(t + 1, nxt + ABYTES);
    }
    i32x8 af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const u32x4 lo = *(const u32x4*)(cur + fragment_lds_offset(MFMA16_F8, lane, 0, a_row0 + 16 * i, 0, SHIFT));
      const u32x4 hi = *(const u32x4*)(cur + fragment_lds_offset(MFMA16_F8, lane, 1, a_row0 + 16 * i, 0, SHIFT));
      af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const u32x4 lo =
          *(const u32x4*)(cur + ABYTES + fragment_lds_offset(MFMA16_F8, lane, 0, b_row0 + 16 * j, 0, SHIFT));
      const u32x4 hi =
          *(const u32x4*)(cur + ABYTES + fragment_lds_offset(MFMA16_F8, lane, 1, b_row0 + 16 * j, 0, SHIFT));
      bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // operands swapped as in the fp16 kernel: instruction A = our B tile
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], kFmtE4M3, kFmtE4M3,
                                                                     0, sb[j], 0, sa[i]);
    wait_vmem();
    __syncthreads();
  }

  uint16_t* D = (uint16_t*)p.d + tc.batch * p.d_bs;
  const uint16_t* C = (p.flags & F_HAS_C) ? (const uint16_t*)p.c + tc.batch * p.c_bs : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      store_quad<DT_F16>(p, C, D, m0 + a_row0 + 16 * i + (lane & 15), n0 + b_row0 + 16 * j + 4 * (lane >> 4), acc[i][j]);
}

// 8 waves (2 along M x 4 along N) on a 256 x 256 output tile, each wave a
// 128 x 64 block as 4 x 2 tiles of v_mfma_scale_f32_32x32x64_f8f6f4; one
// 128-byte K-tile is two 64-wide k-slices.  The wider instruction halves the
// fragment registers of a slice (6 x 8 VGPRs) against the 16x16x128 form.
//
// Scales go through LDS with the data: for K-tile t a row of A or B owns
// the dword of SF holding its four E8M0 bytes for k-blocks 4t..4t+3.
//   SV = 1: that dword is copied per K-tile into the tile's stage by one
//           4-byte direct-to-LDS load per row (waves 0-3: A rows, 4-7: B).
//   SV = 4: every fourth K-tile, one 16-byte copy per row brings the dwords
//           of the next four K-tiles into one of two scale buffers.  A row's
//           scales are then one line request per four K-tiles instead of
//           one per K-tile, which matters because a CU's line requests in
//           flight bound its copy bandwidth.  Needs rows of a multiple of 16
//           blocks on 16-byte boundaries.
// Both need the scale rows K-contiguous, dword aligned and a whole number
// of dwords long; the planner checks it.  In slice s, scale lane l of an
// instruction tile wants block 2s + l / 32 of row l % 32: the lane reads
// its row's dword, shifts it right by 8 (l / 32) once per K-tile, and
// passes byte 2s of the result.
//
// FMT = E2M1 (MXFP4): the same tile with 256 packed fp4 per 128-byte K-tile
// row, four 64-wide k-slices, one 16-byte fragment per lane (its 32
// consecutive k, as the device probe of the operand map shows) and 8 scale bytes per row
// per K-tile (a 16-byte scale chunk covers two K-tiles; SV = 4 only).
//
// FMT = E2M3 or E3M2 (MXFP6): 128 values per K-tile row are 96 bytes of
// a 6-bit stream, held in the first 96 bytes of the 128-byte LDS row (the
// loader zero-fills the rest, which is never read).  Two 64-wide k-slices;
// a lane's 32 consecutive k (the probed operand order) are 24 bytes, read
// as one 16-byte and one 8-byte piece; 4 scale bytes per row per K-tile,
// as for E4M3.
template <int SHIFT, int SV, int FMT = 0>
__global__ __launch_bounds__(512, 2) void gemm_mx_w8_kernel(const GemmParams p) {
  constexpr bool F4 = FMT == kFmtE2M1;
  constexpr bool F6 = FMT == kFmtE2M3 || FMT == kFmtE3M2;
  constexpr int KS = F4 ? 4 : 2;     // 64-wide k-slices per K-tile
  constexpr int SBT = F4 ? 8 : 4;    // scale bytes per row per K-tile
  constexpr int TPC = 16 / SBT;      // K-tiles per 16-byte scale chunk
  constexpr int TB = F6 ? 96 : kRowBytes;  // bytes of a row per K-tile
  static_assert(!(F4 || F6) || SV == 4, "E2M1 and 6-bit data take 16-byte scale chunks");
  constexpr int BM = 256, BN = 256, WM = 2, NT = 512;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int SOFF = ABYTES + BBYTES;  // SV 1: A scale dwords, then B scale dwords
  constexpr int STAGE = SV == 1 ? SOFF + (BM + BN) * 4 : SOFF;
  constexpr int SBUF = SV == 1 ? 0 : (BM + BN) * 16;  // SV 4: one of the two scale buffers
  static_assert(SV == 1 || SV == 4, "scale copy width");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 2 * SBUF];

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave % WM, wn = wave / WM;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  // byte addressing: E2M1 elements are packed two per byte, 6-bit ones
  // four per three bytes (the planner makes strides and K multiples of
  // the packing)
  auto bytes = [](int64_t elems) -> int64_t { return F4 ? elems / 2 : F6 ? elems / 4 * 3 : elems; };
  const char* A = (const char*)p.a + bytes(tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + bytes(tc.batch * p.b_bs + n0 * p.b_rs);

  LoaderKVec<BM, NT, SHIFT, 1, kRowBytes, TB> la(A, rows_a, bytes(p.a_rs), 1, bytes(p.K), wave, lane);
  LoaderKVec<BN, NT, SHIFT, 1, kRowBytes, TB> lb(B, rows_b, bytes(p.b_rs), 1, bytes(p.K), wave, lane);

  // scale copy of this wave: operand (wave / 4), rows 64 (wave % 4) + lane
  const int32_t kb = (int32_t)((p.K + 31) / 32);  // scale bytes per row
  const bool s_is_b = wave >= 4;
  const uint8_t* S = s_is_b ? p.sfb + tc.batch * p.sb_bs + n0 * p.sb_rs : p.sfa + tc.batch * p.sa_bs + m0 * p.sa_rs;
  const int64_t s_rs = s_is_b ? p.sb_rs : p.sa_rs;
  const int32_t s_rows = s_is_b ? rows_b : rows_a;
  const __amdgpu_buffer_rsrc_t rs_ = make_rsrc(S, s_rows > 0 ? (uint32_t)((s_rows - 1) * s_rs + kb) : 0u);
  const int32_t s_row = 64 * (wave & 3) + lane;
  const uint32_t s_off = s_row < s_rows ? (uint32_t)(s_row * s_rs) : kOutOfRange;
  // SV 1: dword of K-tile t into the stage; SV 4: 16 bytes (K-tiles
  // TPC q .. TPC q + TPC - 1) into scale buffer q & 1
  auto issue_scales = [&](int32_t t, char* stage) {
    if constexpr (SV == 1) {
      const uint32_t off = (s_off != kOutOfRange && 4 * t < kb) ? s_off + 4u * (uint32_t)t : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (lds_void_t*)(stage + SOFF + (s_is_b ? BM * 4 : 0) + 256 * (wave & 3)),
                                               4, off, 0, 0, 0);
    } else {
      const int32_t q = t;  // chunk index
      const uint32_t off = (s_off != kOutOfRange && 16 * q < kb) ? s_off + 16u * (uint32_t)q : kOutOfRange;
      char* buf = smem + 2 * STAGE + (q & 1) * SBUF + (s_is_b ? BM * 16 : 0) + 1024 * (wave & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (lds_void_t*)buf, 16, off, 0, 0, 0);
    }
  };
  // SV 1: the scale dword of K-tile t for row `row` of operand `op` (0 A,
  // 1 B) in the tile's stage.  SV 4: the 16 bytes of K-tiles 4q..4q+3 of
  // that row, read into registers once per four K-tiles (one ds_read_b128
  // of 32 consecutive rows is free of bank conflicts; per-tile dword reads
  // 16 bytes apart are not).
  auto scale_word = [&](const char* cur, int32_t op, int32_t row) -> uint32_t {
    return *(const uint32_t*)(cur + SOFF + op * BM * 4 + 4 * row);
  };
  auto scale_chunk = [&](int32_t q, int32_t op, int32_t row) -> u32x4 {
    return *(const u32x4*)(smem + 2 * STAGE + (q & 1) * SBUF + op * BM * 16 + 16 * row);
  };
  auto pick = [](const u32x4& v, int32_t s) -> uint32_t {
    return s == 0 ? v[0] : s == 1 ? v[1] : s == 2 ? v[2] : v[3];
  };
  [[maybe_unused]] u32x4 sa4[FM], sb4[FN];

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;
  const int32_t half_sel = 8 * (lane >> 5);

  const int32_t T = p.k_tiles;
  if (T > 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    issue_scales(0, smem);
    wait_vmem();
    __syncthreads();
  }

  // Loop body without branches, as in the fp16 kernel: past the last tile
  // the copies are fully out of range and fill the idle stage with zeros.
  for (int32_t t = 0; t < T; ++t) {
    char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    la.issue(t + 1, nxt);
    lb.issue(t + 1, nxt + ABYTES);
    if constexpr (SV == 1) {
      issue_scales(t + 1, nxt);
    } else {
      // chunk t/TPC + 1 into the buffer chunk t/TPC - 1 used (retired by
      // the barrier that ended K-tile t - 1); it lands by K-tile t + TPC
      if ((t & (TPC - 1)) == 0) issue_scales(t / TPC + 1, nullptr);
    }
    // this K-tile's scale dwords of each lane's rows, shifted right by
    // 8 (lane / 32): byte 2 s' of dword s / 2 is then the scale of slice s
    // (s' = s % 2) for this lane
    uint32_t sa[FM][SBT / 4], sb[FN][SBT / 4];
    if constexpr (SV == 1) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i][0] = scale_word(cur, 0, a_row0 + 32 * i + (lane & 31)) >> half_sel;
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j][0] = scale_word(cur, 1, b_row0 + 32 * j + (lane & 31)) >> half_sel;
    } else {
      if ((t & (TPC - 1)) == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa4[i] = scale_chunk(t / TPC, 0, a_row0 + 32 * i + (lane & 31));
#pragma unroll
        for (int j = 0; j < FN; ++j) sb4[j] = scale_chunk(t / TPC, 1, b_row0 + 32 * j + (lane & 31));
      }
      const int32_t d0 = (t & (TPC - 1)) * (SBT / 4);
#pragma unroll
      for (int d = 0; d < SBT / 4; ++d) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i][d] = pick(sa4[i], d0 + d) >> half_sel;
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j][d] = pick(sb4[j], d0 + d) >> half_sel;
      }
    }
    // fragments of k-slice ks (operand maps as probed; see the format notes above)
    auto read_slice = [&](int ks, i32x8(&af)[FM], i32x8(&bf)[FN]) {
      if constexpr (F6) {
        // 24 bytes: the lane's 32 consecutive k, k = 32 (lane / 32) + v,
        // i.e. bytes [24 h, 24 h + 24) of the slice's 48 (h = lane / 32):
        // one 16-byte read of the aligned chunk inside it (bytes 0-15 or
        // 32-47) and one 8-byte read of the rest (16-23 or 24-31).  The
        // 8-byte read is served in passes of lanes 0-31 and 32-63, i.e. 32
        // rows at one half of one chunk, which a 128-byte row pitch can
        // spread over only 16 bank pairs (2-way); the 16-byte read is
        // conflict-free under the 32-row swizzle.
        const int32_t h = lane >> 5;
        const int32_t bq = 48 * ks + 32 * h, bd = 48 * ks + 16 + 8 * h;
        auto frag6 = [&](const char* tile, int32_t row) -> i32x8 {
          const u32x4 q = *(const u32x4*)(tile + lds_offset(row, bq, SHIFT));
          const u32x2 d = *(const u32x2*)(tile + lds_offset(row, bd, SHIFT));
          return h ? i32x8{(int)d[0], (int)d[1], (int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0}
                   : i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], (int)d[0], (int)d[1], 0, 0};
        };
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = frag6(cur, a_row0 + 32 * i + (lane & 31));
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = frag6(cur + ABYTES, b_row0 + 32 * j + (lane & 31));
      } else if constexpr (F4) {
        // 16 bytes: the lane's 32 consecutive k (k = 32 (lane / 32) + v)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const u32x4 v = *(const u32x4*)(cur + lds_offset(a_row0 + 32 * i + (lane & 31), 32 * ks + 16 * (lane >> 5), SHIFT));
          af[i] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 v =
              *(const u32x4*)(cur + ABYTES + lds_offset(b_row0 + 32 * j + (lane & 31), 32 * ks + 16 * (lane >> 5), SHIFT));
          bf[j] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const u32x4 lo = *(const u32x4*)(cur + fragment_lds_offset(MFMA32_F8, lane, 0, a_row0 + 32 * i, ks, SHIFT));
          const u32x4 hi = *(const u32x4*)(cur + fragment_lds_offset(MFMA32_F8, lane, 1, a_row0 + 32 * i, ks, SHIFT));
          af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 lo =
              *(const u32x4*)(cur + ABYTES + fragment_lds_offset(MFMA32_F8, lane, 0, b_row0 + 32 * j, ks, SHIFT));
          const u32x4 hi =
              *(const u32x4*)(cur + ABYTES + fragment_lds_offset(MFMA32_F8, lane, 1, b_row0 + 32 * j, ks, SHIFT));
          bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
      }
    };
    // instruction A = our B tile (its scales: sb), instruction B = our A tile
    auto mfma_slice = [&](int ks, const i32x8(&af)[FM], const i32x8(&bf)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[j], af[i], acc[i][j], FMT, FMT, 0, (int)((sb[j][ks >> 1] >> (16 * (ks & 1))) & 0xFFu), 0,
              (int)((sa[i][ks >> 1] >> (16 * (ks & 1))) & 0xFFu));
    };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x8 af[FM], bf[FN];
      read_slice(ks, af, bf);
      mfma_slice(ks, af, bf);
    }
    wait_vmem();
    __syncthreads();
  }

  // accumulator register r of tile (i, j): instruction row (our n)
  // 8 (r / 4) + 4 (lane / 32) + r % 4, instruction column (our m) lane % 32
  uint16_t* D = (uint16_t*)p.d + tc.batch * p.d_bs;
  const uint16_t* C = (p.flags & F_HAS_C) ? (const uint16_t*)p.c + tc.batch * p.c_bs : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + a_row0 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + b_row0 + 32 * j + 8 * g + 4 * (lane >> 5);
        const floatx16& a = acc[i][j];
        store_quad<DT_F16>(p, C, D, m, n, floatx4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]});
      }
  }
}

typedef int32_t i32x6 __attribute__((ext_vector_type(6)));

// Scaled 32x32x64 MFMA whose accumulator is pinned to AGPRs, as mfma_acc in
// the fp16 kernels: the compiler inserts no wait states for it, so a kernel
// reads its accumulators only after an explicit idle.  FMT is the data
// format of both operands (the cbsz / blgp fields; the operand holds 8, 6
// or 4 registers for 8-, 6- or 4-bit data).  Each scale register holds the
// lane's scale bytes of two k-slices; S selects byte 2S (the op_sel_hi bit
// of each scale operand).
#define SL_MFMA_SCALE(MODS)                                                                       \
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 " MODS : "+a"(c) : "v"(a), "v"(b), \
      "v"(sa), "v"(sb))
template <int FMT, int S>
__device__ __forceinline__ void mfma_scale_acc(floatx16& c, i32x8 a, i32x8 b, uint32_t sa, uint32_t sb) {
  if constexpr (FMT == kFmtE4M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0]");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0]");
  } else if constexpr (FMT == kFmtE2M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:2 blgp:2");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:2 blgp:2");
  } else if constexpr (FMT == kFmtE3M2) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:3 blgp:3");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:3 blgp:3");
  } else {
    static_assert(FMT == kFmtE2M1, "data format");
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:4 blgp:4");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:4 blgp:4");
  }
}
template <int FMT, int S>
__device__ __forceinline__ void mfma_scale_acc(floatx16& c, i32x6 a, i32x6 b, uint32_t sa, uint32_t sb) {
  if constexpr (FMT == kFmtE4M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0]");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0]");
  } else if constexpr (FMT == kFmtE2M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:2 blgp:2");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:2 blgp:2");
  } else if constexpr (FMT == kFmtE3M2) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:3 blgp:3");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:3 blgp:3");
  } else {
    static_assert(FMT == kFmtE2M1, "data format");
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:4 blgp:4");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:4 blgp:4");
  }
}
template <int FMT, int S>
__device__ __forceinline__ void mfma_scale_acc(floatx16& c, u32x4 a, u32x4 b, uint32_t sa, uint32_t sb) {
  if constexpr (FMT == kFmtE4M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0]");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0]");
  } else if constexpr (FMT == kFmtE2M3) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:2 blgp:2");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:2 blgp:2");
  } else if constexpr (FMT == kFmtE3M2) {
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:3 blgp:3");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:3 blgp:3");
  } else {
    static_assert(FMT == kFmtE2M1, "data format");
    if constexpr (S == 0) SL_MFMA_SCALE("op_sel_hi:[0,0,0] cbsz:4 blgp:4");
    else SL_MFMA_SCALE("op_sel_hi:[1,1,0] cbsz:4 blgp:4");
  }
}
#undef SL_MFMA_SCALE

// The MX formats on the fp16 ring kernel's schedule: 4 waves, one per SIMD,
// each a 128 x 128 block as 4 x 4 tiles of v_mfma_scale_f32_32x32x64 with
// the accumulators in AGPRs; LDS a ring of five 32 KiB operand K-tiles (256
// rows of 128 bytes: 128 E4M3, 128 6-bit values in the first 96 bytes, or
// 256 E2M1), operand tile q (A of K-tile q/2 for even q, B for odd q) in
// slot q % 5.  A K-tile is KS 64-wide k-slices (2, or 4 for E2M1); fragment
// sets 0 and 1 alternate between slices.  Per K-tile: (1) reads of slice 0,
// the second half of the previous tile's last slice, the copy of B(t+1);
// then every slice but the last with the reads of the next slice (and, in
// slice 0, the copy of A(t+2)) interleaved; the first half of the last
// slice; one barrier.  (E2M1 spreads its copies over more slices: see
// copies below.)  The ring takes all of the LDS, so the scales go
// straight to registers: per TPC K-tiles each lane loads the 16-byte scale
// chunk of each of its rows (4 of A, 4 of B; scale rows of a multiple of 16
// blocks on 16-byte boundaries) into a second register set, issued two
// K-tiles before their first use after that K-tile's copies (its barrier
// lets them stay in flight, the next one waits for them); the loop runs
// TPC K-tiles per iteration so that this load needs no branch (a branch in the loop made the compiler copy accumulators; past T
// the tiles are zero and add nothing).  Slice s takes dword s / 2 of its
// K-tile's scale bytes, shifted right by 8 (lane / 32): byte 2 (s % 2) is
// then the lane's scale.  ROWS: the row epilogue through LDS (full tiles,
// vector C/D).
// Lane part q (0..3) of the LDS byte address of a fragment read of the ring
// kernel, for the 32-row block starting at row0 (shift-0 swizzle): E2M1 one
// 16-byte read per k-slice (q = slice); E4M3 two 16-byte pieces per slice
// (q = 2 slice + piece).  6-bit data (packed rows, LoaderFP6Packed): lane
// half h = lane / 32 takes the row's 32-value blocks 2h (k-slice 0) and
// 2h + 1 (slice 1), bytes 48h .. 48h + 47 = chunks 3h .. 3h + 2: slice 0
// is chunk 3h (q = 0) and the low half of chunk 3h + 1 (q = 1), slice 1
// the high half of chunk 3h + 1 (q = 2) and chunk 3h + 2 (q = 3).  Block g
// of a wave reads at lane part + g mx_block_bytes (mx_offsets_split).
constexpr bool mx_f6(int fmt) { return fmt == kFmtE2M3 || fmt == kFmtE3M2; }
constexpr int32_t mx_block_bytes(int fmt) { return mx_f6(fmt) ? 32 * 96 : 32 * kRowBytes; }
constexpr int32_t mx_lane_off(int fmt, int32_t row0, int32_t lane, int q) {
  if (fmt == kFmtE2M1) return lds_offset(row0 + (lane & 31), 32 * q + 16 * (lane >> 5), 0);
  if (mx_f6(fmt)) {
    const int32_t row = row0 + (lane & 31), c = 3 * (lane >> 5) + (q + 1) / 2;
    return 96 * row + 16 * fp6_packed_chunk(row, c) + (q == 2 ? 8 : 0);
  }
  return fragment_lds_offset(MFMA32_F8, lane, q & 1, row0, q >> 1, 0);
}
constexpr bool mx_offsets_split() {
  for (int fmt : {(int)kFmtE4M3, (int)kFmtE2M1, (int)kFmtE2M3})
    for (int32_t row0 : {0, 128})
      for (int32_t lane = 0; lane < 64; ++lane)
        for (int q = 0; q < 4; ++q)
          for (int32_t g = 0; g < 4; ++g)
            if (mx_lane_off(fmt, row0 + 32 * g, lane, q) != mx_lane_off(fmt, row0, lane, q) + mx_block_bytes(fmt) * g)
              return false;
  return true;
}
static_assert(mx_offsets_split(), "a 32-row block's fragment addresses are block 0's plus a fixed step per block");

template <int SHIFT, bool ROWS, int FMT, bool KFULL = false>
__global__ __launch_bounds__(256, 1) void gemm_mx_w4r_kernel(const GemmParams p) {
  constexpr bool F4 = FMT == kFmtE2M1;
  constexpr bool F6 = FMT == kFmtE2M3 || FMT == kFmtE3M2;
  constexpr int KS = F4 ? 4 : 2;        // 64-wide k-slices per K-tile
  constexpr int SD = KS / 2;            // scale dwords per row per K-tile
  constexpr int TPC = 4 / SD;           // K-tiles per 16-byte scale chunk
  constexpr int TB = F6 ? 96 : kRowBytes;  // bytes of a row per K-tile
  using Frag = std::conditional_t<F4, u32x4, std::conditional_t<F6, i32x6, i32x8>>;
  constexpr int BM = 256, BN = 256, FM = 4, FN = 4;
  constexpr int SLOT = 256 * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char smem[5 * SLOT];
  using LD = std::conditional_t<F6, LoaderFP6Packed<256, 256>, LoaderKVec<256, 256, SHIFT, 1, kRowBytes, TB>>;
  constexpr int LOADS = LD::ITERS;  // copies per operand K-tile and wave: 8 (6 for packed 6-bit rows)
  static_assert(LOADS <= 8, "copy layout");
  static_assert(!F6 || KFULL, "packed 6-bit K-tiles are whole (K a multiple of 512)");
  static_assert(SHIFT == 0, "the fragment addresses are split for the shift-0 swizzle");

  const int32_t lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wm = wave & 1, wn = wave >> 1;
  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.batch);
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int32_t rows_a = (int32_t)(p.M - m0 < BM ? p.M - m0 : BM);
  const int32_t rows_b = (int32_t)(p.N - n0 < BN ? p.N - n0 : BN);
  // byte addressing: E2M1 packs two values per byte, 6-bit data four per
  // three bytes (the planner makes strides and K multiples of the packing)
  auto bytes = [](int64_t elems) -> int64_t { return F4 ? elems / 2 : F6 ? elems / 4 * 3 : elems; };
  const char* A = (const char*)p.a + bytes(tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + bytes(tc.batch * p.b_bs + n0 * p.b_rs);
  auto make_ld = [&](const char* base, int32_t rows, int64_t rs) {
    if constexpr (F6)
      return LD(base, rows, bytes(rs), p.K, wave, lane);
    else
      return LD(base, rows, bytes(rs), 1, bytes(p.K), wave, lane);
  };
  const LD la = make_ld(A, rows_a, p.a_rs);
  const LD lb = make_ld(B, rows_b, p.b_rs);
  const int32_t a_row0 = wm * 128, b_row0 = wn * 128;

  // scale chunks of the lane's rows a_row0 + 32 i + lane % 32 (and of B)
  const int32_t kb = (int32_t)((p.K + 31) / 32);
  const uint8_t* SA = p.sfa + tc.batch * p.sa_bs + m0 * p.sa_rs;
  const uint8_t* SB = p.sfb + tc.batch * p.sb_bs + n0 * p.sb_rs;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(SA, rows_a > 0 ? (uint32_t)((rows_a - 1) * p.sa_rs + kb) : 0u);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(SB, rows_b > 0 ? (uint32_t)((rows_b - 1) * p.sb_rs + kb) : 0u);
  uint32_t soa[FM], sob[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int32_t r = a_row0 + 32 * i + (lane & 31);
    soa[i] = r < rows_a ? (uint32_t)(r * p.sa_rs) : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int32_t r = b_row0 + 32 * j + (lane & 31);
    sob[j] = r < rows_b ? (uint32_t)(r * p.sb_rs) : kOutOfRange;
  }
  u32x4 sa4[FM], sb4[FN], na4[FM], nb4[FN];  // scale chunks in use and next
  auto load_chunk = [&](int32_t q, u32x4(&xa)[FM], u32x4(&xb)[FN]) {
    const bool in = 16 * q < kb;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      xa[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rsa, in && soa[i] != kOutOfRange ? soa[i] + 16u * (uint32_t)q : kOutOfRange, 0, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      xb[j] = __builtin_amdgcn_raw_buffer_load_b128(
          rsb, in && sob[j] != kOutOfRange ? sob[j] + 16u * (uint32_t)q : kOutOfRange, 0, 0);
  };
  // a lane's scale bytes of its blocks in k-slices 0 and 1 go to bytes 0
  // and 2 of its scale register: blocks h and h + 2 of the chunk's dword
  // (lane half h = lane / 32: a shift by 8 h), for packed 6-bit rows blocks
  // 2h and 2h + 1 (a byte permute)
  const int32_t half_sel = 8 * (lane >> 5);
  const uint32_t f6_sel = (lane >> 5) ? 0x03030202u : 0x01010000u;
  auto lane_scales = [&](uint32_t w4) -> uint32_t {
    if constexpr (F6) return __builtin_amdgcn_perm(0u, w4, f6_sel);
    else return w4 >> half_sel;
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};
  const int32_t T = p.k_tiles;  // at least 1 (the planner's condition for this kernel)
  __builtin_assume(T >= 1);
  // K-tile u's copies; past the last K-tile the look-ahead copies are never
  // read: fully out of range, or with KFULL (every K-tile whole) the last
  // K-tile again, so that every copy takes the path without vector
  // arithmetic (issue_full)
  auto kt = [&](int32_t u) { return u < T ? u : (KFULL ? T - 1 : T); };
  auto slot = [&](int32_t q) { return smem + q * SLOT; };
  auto copy = [&](const LD& ld, int32_t u, char* dst, int j) {
    if constexpr (KFULL) ld.issue_full(kt(u), dst, j);
    else ld.issue_one(kt(u), dst, j);
  };
  // the copies of step g of phase ph of K-tile t (phase 0: part (1), phase
  // s + 1: slice s with the reads of slice s + 1).  E4M3 and 6-bit data:
  // B(t+1) over part (1), A(t+2) over slice 0, one per step.  E2M1 has four
  // slices of 32-cycle MFMAs, so its part (1) holds a quarter of the MFMA
  // cycles of E4M3's: its copies go every other step, B(t+1) over part (1)
  // and slice 0, A(t+2) over slices 1 and 2 (2-3% faster; the same spread
  // made 6-bit data 2% slower).  B's copies always precede A's, so the
  // barrier's count of copies left in flight covers A's alone.
  auto copies = [&](int ph, int g, int32_t t, int32_t s3, int32_t s4) {
    if constexpr (F4) {
      if (g % 2 == 0) {
        if (ph <= 1) copy(lb, t + 1, slot(s3), 4 * ph + g / 2);
        else copy(la, t + 2, slot(s4), 4 * (ph - 2) + g / 2);
      }
    } else {
      if (ph == 0 && g < LOADS) copy(lb, t + 1, slot(s3), g);
      if (ph == 1 && g < LOADS) copy(la, t + 2, slot(s4), g);
    }
  };
  static_assert(!F4 || (LOADS == 8 && KS == 4), "E2M1 copy plan: 8 copies per operand over four slices");
  // fragment of k-slice ks for row block g of the wave (the probed operand
  // orders: E4M3 two 16-byte pieces K/2 apart; E2M1 the lane's 32
  // consecutive k in 16 bytes; 6-bit data its 32 consecutive k in 24 bytes,
  // block 2 (lane / 32) + ks of the packed K-tile: a 16-byte and an 8-byte
  // read, in an order fixed per k-slice, so the same registers on every
  // lane), read at the K-tile's precomputed bases (lane part + slot) + g
  // mx_block_bytes: the bases are formed before the barrier that ends the
  // previous K-tile, so no read waits on fresh vector arithmetic.  The MFMA
  // sums the same 64 values per k-slice pair either way; the 6-bit blocks'
  // order only moves which scale byte a lane passes (lane_scales)
  typedef __attribute__((address_space(3))) const u32x4 lds_u4;
  typedef __attribute__((address_space(3))) const u32x2 lds_u2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)smem;
  uint32_t offA[4], offB[4], bA[4], bB[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    offA[q] = lds0 + (uint32_t)mx_lane_off(FMT, a_row0, lane, q);
    offB[q] = lds0 + (uint32_t)mx_lane_off(FMT, b_row0, lane, q);
  }
  auto bases = [&](int32_t qa, int32_t qb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bA[q] = offA[q] + (uint32_t)(qa * SLOT);
      bB[q] = offB[q] + (uint32_t)(qb * SLOT);
    }
    asm volatile("" : "+v"(bA[0]), "+v"(bA[1]), "+v"(bA[2]), "+v"(bA[3]));
    asm volatile("" : "+v"(bB[0]), "+v"(bB[1]), "+v"(bB[2]), "+v"(bB[3]));
  };
  auto rd = [&](const uint32_t(&b)[4], int g, int ks) -> Frag {
    const uint32_t o = (uint32_t)mx_block_bytes(FMT) * (uint32_t)g;
    if constexpr (F4) {
      return *(lds_u4*)(uintptr_t)(b[ks] + o);
    } else if constexpr (F6) {
      // slice 0: 16 bytes then 8; slice 1: 8 bytes then 16 (the block's
      // bytes in order either way)
      if (ks == 0) {
        const u32x4 x = *(lds_u4*)(uintptr_t)(b[0] + o);
        const u32x2 y = *(lds_u2*)(uintptr_t)(b[1] + o);
        return i32x6{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1]};
      } else {
        const u32x2 y = *(lds_u2*)(uintptr_t)(b[2] + o);
        const u32x4 x = *(lds_u4*)(uintptr_t)(b[3] + o);
        return i32x6{(int)y[0], (int)y[1], (int)x[0], (int)x[1], (int)x[2], (int)x[3]};
      }
    } else {
      const u32x4 lo = *(lds_u4*)(uintptr_t)(b[2 * ks] + o);
      const u32x4 hi = *(lds_u4*)(uintptr_t)(b[2 * ks + 1] + o);
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  Frag fa[2][FM], fb[2][FN];  // fragment sets 0 and 1
  uint32_t sac[SD][FM], sbc[SD][FN];  // scale registers of this K-tile
  uint32_t sap[FM], sbp[FN];          // ... of the previous one's last dword
  // slice s of the current K-tile on set s % 2, tiles e0 .. e0 + n - 1 in
  // (i, j) order; S = s % 2 picks the byte
  auto mfma_range = [&](auto s_c, int e0, int n) {
    constexpr int s = decltype(s_c)::value;
#pragma unroll
    for (int e = e0; e < e0 + n; ++e) {
      const int i = e / FN, j = e % FN;
      mfma_scale_acc<FMT, s % 2>(acc[i][j], fb[s % 2][j], fa[s % 2][i], sbc[s / 2][j], sac[s / 2][i]);
    }
  };

  // Every MFMA operand written by a vector-ALU instruction (the zero
  // fragments and scales below, each K-tile's scale registers) is written
  // before an idle of 5 cycles that nothing crosses: the inline-assembly
  // MFMAs get no wait states from the compiler.
  auto valu_fence = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  load_chunk(0, sa4, sb4);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) copy(la, 0, slot(0), j);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) copy(lb, 0, slot(1), j);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) copy(la, 1, slot(2), j);
  bases(0, 1);
  // the first tile's part (1) computes with zero fragments (adds nothing)
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[1][i] = Frag{}, sap[i] = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[1][j] = Frag{}, sbp[j] = 0;
  wait_vmem_n<LOADS>();  // the first scale chunk, A(0), B(0)
  phase_barrier();

  const int32_t TT = (T + TPC - 1) / TPC * TPC;
  int32_t sa = 0;  // slot of A(t); B(t) in the next one
  int32_t t0 = 0;
  do {  // T >= 1: one path into the epilogue keeps the accumulators in place
#pragma unroll
    for (int d = 0; d < TPC; ++d) {
      const int32_t t = t0 + d;
      const int32_t s3 = sa + 3 >= 5 ? sa - 2 : sa + 3, s4 = sa == 0 ? 4 : sa - 1;
#pragma unroll
      for (int w = 0; w < SD; ++w) {
        auto pick = [](const u32x4& v, int k) -> uint32_t { return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3]; };
#pragma unroll
        for (int i = 0; i < FM; ++i) sac[w][i] = lane_scales(pick(sa4[i], SD * d + w));
#pragma unroll
        for (int j = 0; j < FN; ++j) sbc[w][j] = lane_scales(pick(sb4[j], SD * d + w));
        // opaque from here on, so that the compiler cannot recompute them
        // next to the MFMAs
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(sac[w][i]));
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(sbc[w][j]));
      }
      valu_fence();
      // (1): reads of slice 0, the previous K-tile's last slice (second half), copy of B(t+1)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g < 4)
          fb[0][g] = rd(bB, g, 0);
        else
          fa[0][g - 4] = rd(bA, g - 4, 0);
        copies(0, g, t, s3, s4);
        const int i = FM / 2 + g / FN, j = g % FN;
        mfma_scale_acc<FMT, 1>(acc[i][j], fb[1][j], fa[1][i], sbp[j], sap[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // every slice but the last, with the reads of the next one
      auto middle = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (g < 4)
            fb[(s + 1) % 2][g] = rd(bB, g, s + 1);
          else
            fa[(s + 1) % 2][g - 4] = rd(bA, g - 4, s + 1);
          copies(s + 1, g, t, s3, s4);
          mfma_range(s_c, 2 * g, 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      middle(std::integral_constant<int, 0>{});
      // the next chunk's scales, two K-tiles before their first use, after
      // this K-tile's copies: the barrier that ends it lets them (and the
      // copy of A(t+2)) stay in flight, the next one waits for them
      if (d == TPC - 2) load_chunk(t0 / TPC + 1, na4, nb4);
      if constexpr (KS == 4) {
        middle(std::integral_constant<int, 1>{});
        middle(std::integral_constant<int, 2>{});
      }
      // the last slice, first half
      mfma_range(std::integral_constant<int, KS - 1>{}, 0, 8);
      {
        // the next K-tile's read bases
        const int32_t na = sa + 2 >= 5 ? sa - 3 : sa + 2;
        bases(na, na == 4 ? 0 : na + 1);
      }
      if (d == TPC - 2)
        wait_vmem_n<LOADS + FM + FN>();
      else
        wait_vmem_n<LOADS>();
      phase_barrier();
#pragma unroll
      for (int i = 0; i < FM; ++i) sap[i] = sac[SD - 1][i];
#pragma unroll
      for (int j = 0; j < FN; ++j) sbp[j] = sbc[SD - 1][j];
      sa = sa + 2 >= 5 ? sa - 3 : sa + 2;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) sa4[i] = na4[i];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb4[j] = nb4[j];
    t0 += TPC;
  } while (t0 < TT);
  // the last tile's last slice, second half
#pragma unroll
  for (int i = FM / 2; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) mfma_scale_acc<FMT, 1>(acc[i][j], fb[1][j], fa[1][i], sbp[j], sap[i]);
  wait_vmem();
  // empty volatile statements re-defining every accumulator hold the MFMAs
  // before an idle of 32 cycles and every read after it
  auto pin = [&] {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
  };
  pin();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  pin();

  // accumulator register r of tile (i, j): instruction row (our n)
  // 8 (r / 4) + 4 (lane / 32) + r % 4, instruction column (our m) lane % 32
  if constexpr (ROWS) {
    __syncthreads();  // every copy landed, every read of the ring done
    char* region = smem + wave * 32768;
    const int64_t m_base = m0 + a_row0, n_base = n0 + b_row0;
    u16x4 cq[2][32];
    rows_load_c(p, tc.batch, m_base, n_base, lane, cq);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx16& a = acc[2 * h + ii][j];
            *(floatx4*)(region + rows_chunk(32 * ii + (lane & 31), 8 * j + 2 * g + (lane >> 5))) =
                floatx4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          }
      rows_store_half<DT_F16>(p, tc.batch, m_base + 64 * h, n_base, lane, region, cq[h]);
    }
  } else {
    uint16_t* D = (uint16_t*)p.d + tc.batch * p.d_bs;
    const uint16_t* C = (p.flags & F_HAS_C) ? (const uint16_t*)p.c + tc.batch * p.c_bs : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + a_row0 + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + b_row0 + 32 * j + 8 * g + 4 * (lane >> 5);
          const floatx16& a = acc[i][j];
          store_quad<DT_F16>(p, C, D, m, n, floatx4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]});
        }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.tiles_m * p.tiles_n;
  dim3 grid((uint32_t)total), block(WM * WN * 64);
  hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, 0>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmParams& p, int32_t tile, hipStream_t s) {
  switch (tile) {
    case T256x256_W2x2: return launch_cfg<256, 256, 2, 2>(p, s);
    case T256x128_W2x2: return launch_cfg<256, 128, 2, 2>(p, s);
    case T128x256_W2x2: return launch_cfg<128, 256, 2, 2>(p, s);
    case T128x128_W2x2: return launch_cfg<128, 128, 2, 2>(p, s);
    case T256x256_W2x4: {
      dim3 grid((uint32_t)((int64_t)p.batch * p.tiles_m * p.tiles_n)), block(512);
      if (p.flags & F_FP4)
        hipLaunchKernelGGL((gemm_mx_w8_kernel<0, 4, kFmtE2M1>), grid, block, 0, s, p);
      else if (p.flags & F_FP6)
        hipLaunchKernelGGL((gemm_mx_w8_kernel<0, 4, kFmtE2M3>), grid, block, 0, s, p);
      else if (p.flags & F_FP6_E3M2)
        hipLaunchKernelGGL((gemm_mx_w8_kernel<0, 4, kFmtE3M2>), grid, block, 0, s, p);
      else if (p.flags & F_SCALE16)
        hipLaunchKernelGGL((gemm_mx_w8_kernel<0, 4>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((gemm_mx_w8_kernel<0, 1>), grid, block, 0, s, p);
      return hipGetLastError();
    }
    case T256x256_W4R: {
      // 16-byte scale chunks and at least one K-tile
      if (p.k_tiles < 1 || !(p.flags & F_SCALE16)) return hipErrorInvalidValue;
      dim3 grid((uint32_t)((int64_t)p.batch * p.tiles_m * p.tiles_n)), block(256);
      const bool rows = p.M % 256 == 0 && p.N % 256 == 0 && (p.flags & F_D_VEC) &&
                        (!(p.flags & F_HAS_C) || (p.flags & F_C_VEC));
      // whole K-tiles (the copies without vector arithmetic): always for the
      // packed formats (K a multiple of 512), for E4M3 when K is a multiple
      // of its 128-wide K-tile
      auto go = [&](auto fmt) {
        constexpr int F = decltype(fmt)::value;
        if (F != kFmtE4M3 || p.K % 128 == 0) {
          if (rows)
            hipLaunchKernelGGL((gemm_mx_w4r_kernel<0, true, F, true>), grid, block, 0, s, p);
          else
            hipLaunchKernelGGL((gemm_mx_w4r_kernel<0, false, F, true>), grid, block, 0, s, p);
        } else if constexpr (F == kFmtE4M3) {
          if (rows)
            hipLaunchKernelGGL((gemm_mx_w4r_kernel<0, true, F>), grid, block, 0, s, p);
          else
            hipLaunchKernelGGL((gemm_mx_w4r_kernel<0, false, F>), grid, block, 0, s, p);
        }
      };
      if (p.flags & F_FP4)
        go(std::integral_constant<int, kFmtE2M1>{});
      else if (p.flags & F_FP6)
        go(std::integral_constant<int, kFmtE2M3>{});
      else if (p.flags & F_FP6_E3M2)
        go(std::integral_constant<int, kFmtE3M2>{});
      else
        go(std::integral_constant<int, kFmtE4M3>{});
      return hipGetLastError();
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sl
