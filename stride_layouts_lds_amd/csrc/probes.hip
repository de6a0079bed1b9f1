// probes.hip -- device probes that observe, on the hardware, the operand
// maps of the matrix-core instructions and the LDS data paths the GEMM
// relies on.  They compute nothing the GEMM computes; each writes raw
// register or LDS contents for the host to compare against the maps.
#include "sl_device.hpp"

namespace sl {
namespace {

constexpr uint8_t kE4M3One = 0x38;  // 1.0
constexpr uint8_t kCodeBase = 0x20; // lane/slot-coded E4M3 values start here (0.125)
constexpr int kFmtE2M3 = 2;         // CBSZ/BLGP format codes: FP6 E2M3,
constexpr int kFmtE3M2 = 3;         // BF6 E3M2,
constexpr int kFmtE2M1 = 4;         // FP4 E2M1

// One wave per case.  f16 instructions: case = (lane, slot) of the one-hot
// operand; the other operand holds lane*8 + slot + 1.
template <int INSTR>
__global__ __launch_bounds__(64) void probe_mfma_f16(int32_t mode, float* out) {
  constexpr int REGS = instr_acc_regs(INSTR);
  const int32_t lane = threadIdx.x;
  const int32_t c = blockIdx.x;
  const int32_t hl = c / 8, hs = c % 8;
  half8 onehot, coded;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    onehot[v] = (lane == hl && v == hs) ? (_Float16)1.0f : (_Float16)0.0f;
    coded[v] = (_Float16)(float)(lane * 8 + v + 1);
  }
  const half8 a = mode == 0 ? onehot : coded;
  const half8 b = mode == 0 ? coded : onehot;
  float r[REGS];
  if constexpr (INSTR == MFMA16_F16) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = acc[i];
  } else {
    floatx16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = acc[i];
  }
#pragma unroll
  for (int i = 0; i < REGS; ++i) out[((int64_t)c * 64 + lane) * REGS + i] = r[i];
}

// Scaled E4M3 instructions: case = (lane, byte) of the one-hot operand.
//   mode 0/1: A one-hot, B byte = base + lane / base + byte, unit scales
//   mode 2/3: B one-hot, A byte = base + lane / base + byte, unit scales
//   mode 4:   A one-hot, B = 1, A scale of lane l = 127 + l - 32
//   mode 5:   B one-hot, A = 1, B scale of lane l = 127 + l - 32
//   mode 6/7: A in E2M1 (format 4): case = (lane, nibble) of a one-hot 1.0
//             among the lane's 32 nibbles (16 bytes, low nibble first);
//             B in E4M3 with byte = base + lane / base + byte, unit scales
template <int INSTR>
__global__ __launch_bounds__(64) void probe_mfma_f8(int32_t mode, float* out) {
  constexpr int REGS = instr_acc_regs(INSTR);
  const int32_t lane = threadIdx.x;
  const int32_t c = blockIdx.x;
  const int32_t hl = c / 32, hs = c % 32;
  uint32_t wa[8], wb[8];
  const bool a_hot = mode == 0 || mode == 1 || mode == 4;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t hot = 0, other = 0;
#pragma unroll
    for (int bidx = 0; bidx < 4; ++bidx) {
      const int32_t s = 4 * w + bidx;
      const uint32_t hb = (lane == hl && s == hs) ? kE4M3One : 0u;
      uint32_t ob;
      if (mode == 4 || mode == 5)
        ob = kE4M3One;
      else if (mode == 0 || mode == 2)
        ob = kCodeBase + lane;
      else
        ob = kCodeBase + s;
      hot |= hb << (8 * bidx);
      other |= ob << (8 * bidx);
    }
    wa[w] = a_hot ? hot : other;
    wb[w] = a_hot ? other : hot;
  }
  const i32x8 a = {(int)wa[0], (int)wa[1], (int)wa[2], (int)wa[3], (int)wa[4], (int)wa[5], (int)wa[6], (int)wa[7]};
  const i32x8 b = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3], (int)wb[4], (int)wb[5], (int)wb[6], (int)wb[7]};
  const int32_t sa = mode == 4 ? 127 + lane - 32 : 127;
  const int32_t sb = mode == 5 ? 127 + lane - 32 : 127;
  // mode 6/7: A one-hot E2M1 1.0 (code 0x2) at nibble hs of lane hl
  uint32_t w4[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) w4[w] = (lane == hl && hs / 8 == w) ? (0x2u << (4 * (hs % 8))) : 0u;
  const i32x8 a4 = {(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3], 0, 0, 0, 0};
  uint32_t wb4[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t v = 0;
#pragma unroll
    for (int bidx = 0; bidx < 4; ++bidx) v |= (uint32_t)(kCodeBase + (mode == 6 ? lane : 4 * w + bidx)) << (8 * bidx);
    wb4[w] = v;
  }
  const i32x8 b4 = {(int)wb4[0], (int)wb4[1], (int)wb4[2], (int)wb4[3],
                    (int)wb4[4], (int)wb4[5], (int)wb4[6], (int)wb4[7]};
  const bool fp4 = mode == 6 || mode == 7;
  // mode 8-11: A one-hot 1.0 in a 6-bit format at value hs of lane hl, the
  // 32 values of a lane packed as one little-endian bit stream (value v at
  // bits 6v .. 6v+5 of six dwords): E2M3 (modes 8/9, 1.0 = 0b001000) or
  // E3M2 (modes 10/11, 1.0 = 0b001100); B as in modes 6/7
  const bool fp6 = mode >= 8;
  const uint32_t one6 = mode >= 10 ? 0x0Cu : 0x08u;
  const int32_t bit = 6 * hs;
  uint32_t w6[6];
#pragma unroll
  for (int w = 0; w < 6; ++w) {
    uint32_t v = 0;
    if (lane == hl) {
      if (bit / 32 == w) v |= one6 << (bit % 32);
      if (bit / 32 + 1 == w && bit % 32 > 26) v |= one6 >> (32 - bit % 32);
    }
    w6[w] = v;
  }
  const i32x8 a6 = {(int)w6[0], (int)w6[1], (int)w6[2], (int)w6[3], (int)w6[4], (int)w6[5], 0, 0};
  uint32_t wb6[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t v = 0;
#pragma unroll
    for (int bidx = 0; bidx < 4; ++bidx)
      v |= (uint32_t)(kCodeBase + ((mode & 1) == 0 ? lane : 4 * w + bidx)) << (8 * bidx);
    wb6[w] = v;
  }
  const i32x8 b6 = {(int)wb6[0], (int)wb6[1], (int)wb6[2], (int)wb6[3],
                    (int)wb6[4], (int)wb6[5], (int)wb6[6], (int)wb6[7]};
  float r[REGS];
  if constexpr (INSTR == MFMA16_F8) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (fp4)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a4, b4, acc, kFmtE2M1, 0, 0, 127, 0, 127);
    else if (fp6 && mode >= 10)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a6, b6, acc, kFmtE3M2, 0, 0, 127, 0, 127);
    else if (fp6)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a6, b6, acc, kFmtE2M3, 0, 0, 127, 0, 127);
    else
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = acc[i];
  } else {
    floatx16 acc = {};
    if (fp4)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, acc, kFmtE2M1, 0, 0, 127, 0, 127);
    else if (fp6 && mode >= 10)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a6, b6, acc, kFmtE3M2, 0, 0, 127, 0, 127);
    else if (fp6)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a6, b6, acc, kFmtE2M3, 0, 0, 127, 0, 127);
    else
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = acc[i];
  }
#pragma unroll
  for (int i = 0; i < REGS; ++i) out[((int64_t)c * 64 + lane) * REGS + i] = r[i];
}

// LDS data paths, one wave, 4 KiB of LDS.
__global__ __launch_bounds__(64) void probe_lds(int32_t mode, const uint8_t* src, const int32_t* perm,
                                                uint8_t* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4096];
  const int32_t lane = threadIdx.x;
  if (mode == 0 || mode == 1 || mode == 3) {
#pragma unroll
    for (int i = 0; i < 4096 / 64 / 4; ++i) ((uint32_t*)lds)[i * 64 + lane] = 0xA5A5A5A5u;
    __syncthreads();
    const int32_t p = perm[lane] & 63;
    if (mode == 0) {
      // a negative perm entry makes the lane's offset out of range
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src, 1024u);
      const uint32_t off = perm[lane] < 0 ? kOutOfRange : (uint32_t)(16 * p);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, off, 0, 0, 0);
    } else if (mode == 3) {
      // 4-byte direct-to-LDS buffer load: lane l fetches src + 4*perm[l]
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src, 1024u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, (uint32_t)(4 * (perm[lane] & 255)), 0, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds((const void*)(src + 16 * p), (lds_void_t*)lds, 16, 0, 0);
    }
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4096 / 64 / 4; ++i) ((uint32_t*)out)[i * 64 + lane] = ((uint32_t*)lds)[i * 64 + lane];
  } else {
#pragma unroll
    for (int i = 0; i < 4096 / 64 / 4; ++i) ((uint32_t*)lds)[i * 64 + lane] = ((const uint32_t*)src)[i * 64 + lane];
    __syncthreads();
    const int32_t a = perm[lane] & (4096 - 8) & ~7;
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(lds + a));
    *(s4*)(out + 8 * lane) = v;
  }
}

}  // namespace

hipError_t launch_probe_mfma(int32_t instr, int32_t mode, float* out, int64_t cases, hipStream_t s) {
  dim3 grid((uint32_t)cases), block(64);
  switch (instr) {
    case MFMA16_F16: hipLaunchKernelGGL(probe_mfma_f16<MFMA16_F16>, grid, block, 0, s, mode, out); break;
    case MFMA32_F16: hipLaunchKernelGGL(probe_mfma_f16<MFMA32_F16>, grid, block, 0, s, mode, out); break;
    case MFMA16_F8: hipLaunchKernelGGL(probe_mfma_f8<MFMA16_F8>, grid, block, 0, s, mode, out); break;
    case MFMA32_F8: hipLaunchKernelGGL(probe_mfma_f8<MFMA32_F8>, grid, block, 0, s, mode, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_lds(int32_t mode, const void* src, const int32_t* perm, void* out, hipStream_t s) {
  hipLaunchKernelGGL(probe_lds, dim3(1), dim3(64), 0, s, mode, (const uint8_t*)src, perm, (uint8_t*)out);
  return hipGetLastError();
}

}  // namespace sl
