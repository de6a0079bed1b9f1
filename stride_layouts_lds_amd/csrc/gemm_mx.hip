// gemm_mx.hip -- MXFP8 block-scaled GEMM on gfx950:
//   D = C + (A_low * SFA) (B_low * SFB)^T,  A_low, B_low FP8 E4M3,
//   one E8M0 scale per 32 consecutive K per row of A and of B,
// i.e. the block-scaled product of "数据布局及其记号", section
// "Replication 与 Offset", with B stored (N, K) and K_blk = 32.
//
// Same data flow as the fp16 kernel: a K-tile is 128 bytes = 128 E4M3
// values per row, loaded straight into the XOR-swizzled LDS tile; the
// instruction v_mfma_scale_f32_16x16x128_f8f6f4 consumes 32 bytes per lane
// (two ds_read_b128) and one scale byte per lane.  Its scale lane l covers
// (row l % 16, K block l / 16) of its operand, so lane l fetches the byte
// SF[row0 + l % 16][4 t + l / 16] for K-tile t.
#include "sl_device.hpp"

namespace sl {
namespace {

constexpr int32_t kFmtE4M3 = 0;  // CBSZ/BLGP format code of FP8 E4M3

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

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
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

  const bool has_c = p.flags & F_HAS_C;
  const bool d_vec = p.flags & F_D_VEC;
  const bool c_vec = p.flags & F_C_VEC;
  uint16_t* D = (uint16_t*)p.d + tc.batch * p.d_bs;
  const uint16_t* C = has_c ? (const uint16_t*)p.c + tc.batch * p.c_bs : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + a_row0 + 16 * i + (lane & 15);
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + b_row0 + 16 * j + 4 * (lane >> 4);
      if (n >= p.N) continue;
      floatx4 v = acc[i][j];
      const bool full = n + 3 < p.N;
      if (has_c) {
        const uint16_t* cp = C + m * p.c_rs + n * p.c_cs;
        if (full && c_vec) {
          const half4 cv = *(const half4*)cp;
          v[0] += (float)cv[0];
          v[1] += (float)cv[1];
          v[2] += (float)cv[2];
          v[3] += (float)cv[3];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) v[r] += (float)__builtin_bit_cast(_Float16, cp[r * p.c_cs]);
        }
      }
      uint16_t* dp = D + m * p.d_rs + n * p.d_cs;
      if (full && d_vec) {
        *(half4*)dp = half4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) dp[r * p.d_cs] = __builtin_bit_cast(uint16_t, (_Float16)v[r]);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmParams& p, int32_t shift, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.tiles_m * p.tiles_n;
  dim3 grid((uint32_t)total), block(WM * WN * 64);
  if (shift == 0)
    hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, 0>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, 1>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmParams& p, int32_t tile, int32_t shift, hipStream_t s) {
  switch (tile) {
    case T256x256_W2x2: return launch_cfg<256, 256, 2, 2>(p, shift, s);
    case T256x128_W2x2: return launch_cfg<256, 128, 2, 2>(p, shift, s);
    case T128x256_W2x2: return launch_cfg<128, 256, 2, 2>(p, shift, s);
    case T128x128_W2x2: return launch_cfg<128, 128, 2, 2>(p, shift, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sl
