// sl_kernels.hpp -- parameters and launchers shared between the host
// dispatcher (api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sl {

// How one operand tile is brought from HBM into its K-contiguous LDS tile.
enum LoadKind : int32_t {
  LOAD_KVEC = 0,    // K contiguous, 16-B aligned: direct HBM->LDS 16-B buffer loads
  LOAD_MNVEC = 1,   // M (or N) contiguous, 16-B aligned: 16-B loads, 8x8 register transpose
  LOAD_GENERIC = 2, // any strides: element loads
  LOAD_MNDMA = 3,   // M (or N) contiguous, 16-B aligned: direct HBM->LDS into an M-major tile,
                    // fragments by transposing LDS reads (8-wave 256x256 kernel)
  LOAD_NVFP4_PAIRS = 5,  // the same, fetching two K-tiles per row at once (8-byte scale loads)
  LOAD_NVFP4 = 4    // packed E2M1 with E4M3 scales per 16 K: decoded and scaled in registers,
                    // written to the K-major fp16 tile (8-wave 256x256 kernel)
};

// Kernel families (sl_plan.kernel).
enum KernelKind : int32_t {
  K_F16 = 1,          // fp16, vector loaders
  K_F16_GENERIC = 2,  // fp16 with an element-wise loader on one side
  K_MX = 3,           // MXFP8, 4 waves, v_mfma_scale 16x16x128, scales by byte loads
  K_MX_W8 = 4,        // MXFP8, 8 waves, v_mfma_scale 32x32x64, scales staged in LDS
  K_NVFP4 = 5,        // NVFP4 dequantised to exact fp16 tiles, fp16 MFMA (8 waves)
  K_MXFP4 = 6,        // MXFP4, 8 waves, v_mfma_scale 32x32x64 with E2M1 data
  K_MXFP6 = 7,        // MXFP6, 8 waves, v_mfma_scale 32x32x64 with E2M3 or E3M2 data
  K_MX_W4R = 8        // MXFP8, 4 waves each 128x128, v_mfma_scale 32x32x64, LDS ring, scales in registers
};

// Tile configurations the dispatcher can choose: rows of A, rows of B,
// waves along M, waves along N, and whether the fragments are double-
// buffered in registers (pipe).
enum TileCfg : int32_t {
  T256x256_W2x2 = 0,    // 4 waves, each 128x128
  T256x128_W2x2 = 1,    // 4 waves, each 128x64
  T128x256_W2x2 = 2,    // 4 waves, each 64x128
  T128x128_W2x2 = 3,    // 4 waves, each 64x64
  T256x256_W2x4 = 4,    // 8 waves (2 per SIMD), each 128x64
  T256x256_W2x4_P = 5,  // 8 waves, double-buffered fragments
  T256x256_W2x4_S3 = 6, // 8 waves, K-tiles of 32, 3 LDS stages
  T256x256_W2x4_S4 = 7, // 8 waves, K-tiles of 32, 4 LDS stages
  T256x256_W2x4_S5 = 8, // 8 waves, K-tiles of 32, 5 LDS stages
  T256x256_PP = 9,      // 8 waves in two ping-pong groups, each wave 128x64
  T256x256_PPS4 = 10,   // ping-pong, K-tiles of 32, 4 LDS stages
  T256x256_PPS5 = 11,   // ping-pong, K-tiles of 32, 5 LDS stages
  T256x256_PPC4 = 12,   // ping-pong, 4 stages, copy spread over all waves' compute phases
  T256x256_PPC5 = 13,   // same with 5 stages
  T256x256_PPG = 14,    // ping-pong, 2 stages of 64-wide K-tiles, group 1 copies inside its compute phase
  T32x128_STREAM = 15,  // 4 waves along N, each 32x32; 6 stages of 64-wide K-tiles (skinny outputs)
  T128x128_SPLITK = 16, // 8 waves, each 64x32; 3 stages of 64-wide K-tiles; K split over workgroups
  T256x192_W2x4 = 17,   // 8 waves, each 128x48 (fills the chip on ~4000 x 3000 outputs)
  T256x128_SPLITK = 18, // 8 waves (4 along M), each 64x64; 3 stages; K split (tall skinny outputs)
  T256x256_W4R = 19,    // 4 waves, each 128x128 (AGPR accumulators); a ring of five operand K-tiles in LDS
  T256x192_W4R = 20,    // the same with 256x192 tiles, each wave 128x96
  T_COUNT = 21
};

struct TileShape {
  int32_t bm, bn, wm, wn, bk, stages;
};

constexpr TileShape kTiles[T_COUNT] = {
    {256, 256, 2, 2, 64, 2}, {256, 128, 2, 2, 64, 2}, {128, 256, 2, 2, 64, 2},
    {128, 128, 2, 2, 64, 2}, {256, 256, 2, 4, 64, 2}, {256, 256, 2, 4, 64, 2},
    {256, 256, 2, 4, 32, 3}, {256, 256, 2, 4, 32, 4}, {256, 256, 2, 4, 32, 5},
    {256, 256, 2, 4, 64, 2}, {256, 256, 2, 4, 32, 4}, {256, 256, 2, 4, 32, 5},
    {256, 256, 2, 4, 32, 4}, {256, 256, 2, 4, 32, 5}, {256, 256, 2, 4, 64, 2},
    {32, 128, 1, 4, 64, 6}, {128, 128, 2, 4, 64, 3}, {256, 192, 2, 4, 64, 2},
    {256, 128, 4, 2, 64, 3}, {256, 256, 2, 2, 64, 2}, {256, 192, 2, 2, 64, 2}};

struct GemmParams {
  const void* a;  // element (b, m, k) at a + b*a_bs + m*a_rs + k*a_ks
  const void* b;  // element (b, n, k) at b + b*b_bs + n*b_rs + k*b_ks
  const void* c;  // may be NULL
  void* d;
  const uint8_t* sfa;  // MX scales (NULL for fp16)
  const uint8_t* sfb;
  int64_t M, N, K;
  int64_t a_rs, a_ks, a_bs;
  int64_t b_rs, b_ks, b_bs;
  int64_t c_rs, c_cs, c_bs;
  int64_t d_rs, d_cs, d_bs;
  int64_t sa_rs, sa_ks, sa_bs;  // scale strides (elements = bytes)
  int64_t sb_rs, sb_ks, sb_bs;
  int32_t batch;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
  int32_t k_tiles;
  int32_t flags;
  // split-K: the grid holds `splits` copies of the output tiles, copy s
  // covering K-tiles [s*split_tiles, (s+1)*split_tiles); each writes fp32
  // partial sums to ws[s][batch][M][N] and a second kernel reduces them
  int32_t splits;       // 1: no split
  int32_t split_tiles;  // K-tiles per split
  float* ws;
};

// GemmParams.flags
constexpr int32_t F_HAS_C = 1;
constexpr int32_t F_D_VEC = 2;  // D rows contiguous and 8-B aligned: 4-half stores
constexpr int32_t F_C_VEC = 4;  // C rows contiguous and 8-B aligned: 4-half loads
constexpr int32_t F_SCALE16 = 8;  // MX scale rows 16-B aligned, a multiple of 16 blocks long
constexpr int32_t F_BF16 = 16;    // A, B, C and D are bf16 (else fp16)
constexpr int32_t F_FP4 = 32;     // MX operands are packed E2M1 (MXFP4), else E4M3
constexpr int32_t F_FP6 = 64;     // MX operands are packed 6-bit E2M3 (MXFP6)
constexpr int32_t F_FP6_E3M2 = 128;  // MX operands are packed 6-bit E3M2 (MXFP6)
constexpr int32_t kCUs = 256;     // compute units of an MI355X: one round of single-workgroup-per-CU tiles

// element type of the 16-bit GEMM kernels (template argument)
constexpr int DT_F16 = 0;
constexpr int DT_BF16 = 1;

// Launchers (each returns the launch's hipError_t).  The 16-bit kernels
// take their element type from GemmParams.flags (F_BF16).
hipError_t launch_gemm_f16(const GemmParams& p, int32_t tile, int32_t a_load, int32_t b_load,
                           hipStream_t stream);
// D = C + sum over splits of ws (the second kernel of a split-K GEMM).
hipError_t launch_splitk_reduce(const GemmParams& p, hipStream_t stream);
// An NVFP4 operand decoded to fp16 rows (K contiguous, batch after batch)
// ahead of an fp16 product: packed E2M1 x with strides rs, bs (elements)
// and E4M3 scales s with strides srs, sks, sbs (one per 16 K); K % 32 == 0,
// rows 16 bytes apart at least (rs % 32 == 0), x on a 16-byte boundary.
struct Nvfp4Decode {
  const uint8_t* x;
  const uint8_t* s;
  uint16_t* out;
  int64_t rows, K, rs, bs, srs, sks, sbs;
  int32_t batch;
};
hipError_t launch_nvfp4_decode(const Nvfp4Decode& d, hipStream_t stream);
hipError_t launch_gemm_mx(const GemmParams& p, int32_t tile, hipStream_t stream);

// The static device scratch behind sl_gemm_no_alloc (scratch.hip): its size
// bounds the split-K workspace that entry point can serve, and its device
// address on the current GPU comes from scratch_address().
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(void** out);

hipError_t launch_probe_mfma(int32_t instr, int32_t mode, float* out, int64_t cases, hipStream_t stream);
hipError_t launch_probe_lds(int32_t mode, const void* src, const int32_t* perm, void* out,
                            hipStream_t stream);

}  // namespace sl
