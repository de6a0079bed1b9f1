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

template <int BM, int BN, int WM, int WN, int ALOAD, int BLOAD, int SHIFT>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_f16_kernel(const GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 instruction tiles per wave
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
  const char* A = (const char*)p.a + 2 * (tc.batch * p.a_bs + m0 * p.a_rs);
  const char* B = (const char*)p.b + 2 * (tc.batch * p.b_bs + n0 * p.b_rs);

  typename LoaderSel<ALOAD, BM, NT, SHIFT>::type la(A, rows_a, p.a_rs, p.a_ks, p.K, wave, lane);
  typename LoaderSel<BLOAD, BN, NT, SHIFT>::type lb(B, rows_b, p.b_rs, p.b_ks, p.K, wave, lane);

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Per-lane fragment offsets inside one stage, k-slice 0 of tile 0 of this
  // wave; the others differ by compile-time constants.
  const int32_t a_row0 = wm * TM, b_row0 = wn * TN;

  const int32_t T = p.k_tiles;
  if (T > 0) {
    la.issue(0, smem);
    lb.issue(0, smem + ABYTES);
    la.commit(smem);
    lb.commit(smem + ABYTES);
    wait_vmem();
    __syncthreads();
  }

  for (int32_t t = 0; t < T; ++t) {
    char* cur = smem + (t & 1) * STAGE;
    char* nxt = smem + ((t + 1) & 1) * STAGE;
    const bool more = t + 1 < T;
    if (more) {
      la.issue(t + 1, nxt);
      lb.issue(t + 1, nxt + ABYTES);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      half8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const half8*)(cur + fragment_lds_offset(MFMA16_F16, lane, 0, a_row0 + 16 * i, ks, SHIFT));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *(const half8*)(cur + ABYTES +
                                fragment_lds_offset(MFMA16_F16, lane, 0, b_row0 + 16 * j, ks, SHIFT));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.commit(nxt);
      lb.commit(nxt + ABYTES);
    }
    wait_vmem();
    __syncthreads();
  }

  // Epilogue.  acc[i][j][r] is output (m, n) with
  //   m = m0 + a_row0 + 16 i + lane % 16,  n = n0 + b_row0 + 16 j + 4 (lane / 16) + r
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

template <int BM, int BN, int WM, int WN, int AL, int BL>
hipError_t launch_cfg(const GemmParams& p, int32_t shift, hipStream_t s) {
  const int64_t total = (int64_t)p.batch * p.tiles_m * p.tiles_n;
  dim3 grid((uint32_t)total), block(WM * WN * 64);
  if (shift == 0)
    hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, AL, BL, 0>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, AL, BL, 1>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int AL, int BL>
hipError_t launch_tile(const GemmParams& p, int32_t tile, int32_t shift, hipStream_t s) {
  switch (tile) {
    case T256x256_W2x2: return launch_cfg<256, 256, 2, 2, AL, BL>(p, shift, s);
    case T256x128_W2x2: return launch_cfg<256, 128, 2, 2, AL, BL>(p, shift, s);
    case T128x256_W2x2: return launch_cfg<128, 256, 2, 2, AL, BL>(p, shift, s);
    case T128x128_W2x2: return launch_cfg<128, 128, 2, 2, AL, BL>(p, shift, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_f16(const GemmParams& p, int32_t tile, int32_t a_load, int32_t b_load,
                           int32_t shift, hipStream_t s) {
  if (a_load == LOAD_GENERIC || b_load == LOAD_GENERIC) {
    // one configuration for every stride pattern
    if (tile != T128x128_W2x2) return hipErrorInvalidValue;
    if (a_load == LOAD_GENERIC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_GENERIC>(p, shift, s);
    if (a_load == LOAD_GENERIC && b_load == LOAD_KVEC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_KVEC>(p, shift, s);
    if (a_load == LOAD_KVEC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_KVEC, LOAD_GENERIC>(p, shift, s);
    if (a_load == LOAD_GENERIC && b_load == LOAD_MNVEC)
      return launch_cfg<128, 128, 2, 2, LOAD_GENERIC, LOAD_MNVEC>(p, shift, s);
    if (a_load == LOAD_MNVEC && b_load == LOAD_GENERIC)
      return launch_cfg<128, 128, 2, 2, LOAD_MNVEC, LOAD_GENERIC>(p, shift, s);
    return hipErrorInvalidValue;
  }
  if (a_load == LOAD_KVEC && b_load == LOAD_KVEC) return launch_tile<LOAD_KVEC, LOAD_KVEC>(p, tile, shift, s);
  if (a_load == LOAD_MNVEC && b_load == LOAD_KVEC) return launch_tile<LOAD_MNVEC, LOAD_KVEC>(p, tile, shift, s);
  if (a_load == LOAD_KVEC && b_load == LOAD_MNVEC) return launch_tile<LOAD_KVEC, LOAD_MNVEC>(p, tile, shift, s);
  if (a_load == LOAD_MNVEC && b_load == LOAD_MNVEC)
    return launch_tile<LOAD_MNVEC, LOAD_MNVEC>(p, tile, shift, s);
  return hipErrorInvalidValue;
}

}  // namespace sl
