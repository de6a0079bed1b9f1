// sl_maps.hpp -- the layouts every stage of the GEMM uses, as constexpr
// functions callable from host and device.  The kernels compute their LDS
// and fragment addresses with these functions, and the host query entry
// points dump them, so what is exported is what runs.
//
// Notation follows "数据布局及其记号" (shape:stride layouts, section
// "Shape-Stride 模型"; XOR swizzle, section "Swizzle Layout") and the TV
// (thread, value) maps of "CuTe 中 A、B 如何加载到 MMA 寄存器", section 2:
// a lane index l and a value (slot) index v are unflattened first-mode-
// fastest and the map returns the operand tile coordinate.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SL_HD __host__ __device__ __forceinline__
#else
#define SL_HD inline
#endif

namespace sl {

// ---------------------------------------------------------------------------
// Matrix-core operand maps (CDNA4 / gfx950).
//
// v_mfma_f32_16x16x32_f16: lane l = l0 + 16*l1 (l0 < 16, l1 < 4), slot v < 8
//   A (16 x 32):  m = l0, k = 8*l1 + v        TV ((16,4),8):((1,128),16), q = m + 16k
//   B (16 x 32):  n = l0, k = 8*l1 + v        (same form)
//   D (16 x 16):  n = l0, m = 4*l1 + v (v<4)   TV ((16,4),4):((16,4),1),  q = m + 16n
// v_mfma_f32_32x32x16_f16: lane l = l0 + 32*l1 (l0 < 32, l1 < 2)
//   A (32 x 16):  m = l0, k = 8*l1 + v
//   D (32 x 32):  n = l0, m = 8*(v/4) + 4*l1 + v%4  (v < 16)
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3): slot v = v0 + 16*v1 < 32 (bytes)
//   A (16 x 128): m = l0, k = 16*l1 + v0 + 64*v1; scale lane l -> (m = l0, block l1)
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3):
//   A (32 x 64):  m = l0, k = 16*l1 + v0 + 32*v1; scale lane l -> (m = l0, block l1)
// (the blocks of 32 consecutive k are the ones whose bytes share a scale lane)
// ---------------------------------------------------------------------------

// (the same scaled instructions with E2M1 data, 16 bytes = 32 nibbles per
// lane: nibble v of lane l holds row l0, k = 32*l1 + v, 32 consecutive k)
// (and with 6-bit E2M3 / E3M2 data, 32 values per lane as one little-endian
// 6-bit stream over six dwords: value v of lane l holds row l0, k = 32*l1 +
// v, the same order as E2M1)
enum Instr : int32_t {
  MFMA16_F16 = 0, MFMA32_F16 = 1, MFMA16_F8 = 2, MFMA32_F8 = 3, MFMA16_F4 = 4, MFMA32_F4 = 5,
  MFMA16_F6 = 6, MFMA32_F6 = 7
};
enum Operand : int32_t { OP_A = 0, OP_B = 1, OP_D = 2, OP_SCALE = 3 };

struct Coord {
  int32_t row, col;
};

SL_HD constexpr int32_t instr_rows(int32_t instr) {
  return (instr == MFMA16_F16 || instr == MFMA16_F8 || instr == MFMA16_F4 || instr == MFMA16_F6) ? 16 : 32;
}
SL_HD constexpr int32_t instr_k(int32_t instr) {
  return instr == MFMA16_F16                                                ? 32
         : instr == MFMA32_F16                                              ? 16
         : (instr == MFMA16_F8 || instr == MFMA16_F4 || instr == MFMA16_F6) ? 128
                                                                            : 64;
}
// input slots per lane (elements) for A/B
SL_HD constexpr int32_t instr_in_slots(int32_t instr) { return (instr == MFMA16_F16 || instr == MFMA32_F16) ? 8 : 32; }
// accumulator registers per lane
SL_HD constexpr int32_t instr_acc_regs(int32_t instr) { return instr_rows(instr) == 16 ? 4 : 16; }

// (lane, slot) -> (row, col) of operand A or B.
//   f16:  row = l0, col = 8*l1 + v
//   f8:   row = l0, col = 16*l1 + v%16 + (K/2)*(v/16)
//   f4, f6: row = l0, col = 32*l1 + v
SL_HD constexpr Coord operand_map(int32_t instr, int32_t lane, int32_t slot) {
  const int32_t R = instr_rows(instr);
  if (instr_in_slots(instr) == 8) return Coord{lane % R, 8 * (lane / R) + slot};
  if (instr == MFMA16_F4 || instr == MFMA32_F4 || instr == MFMA16_F6 || instr == MFMA32_F6)
    return Coord{lane % R, 32 * (lane / R) + slot};
  return Coord{lane % R, 16 * (lane / R) + slot % 16 + (instr_k(instr) / 2) * (slot / 16)};
}

// (lane, reg) -> (m, n) of the accumulator.
SL_HD constexpr Coord acc_map(int32_t instr, int32_t lane, int32_t reg) {
  return instr_rows(instr) == 16 ? Coord{4 * (lane / 16) + reg, lane % 16}
                                 : Coord{8 * (reg / 4) + 4 * (lane / 32) + reg % 4, lane % 32};
}

// scale lane -> (row, K block of 32) for the scaled f8 instructions
SL_HD constexpr Coord scale_map(int32_t instr, int32_t lane) {
  const int32_t R = instr_rows(instr);
  return Coord{lane % R, lane / R};
}

// ---------------------------------------------------------------------------
// LDS tile layout: a K-contiguous tile of `rows` x RB bytes (RB = 128: one
// 64-wide fp16 K-tile per row; RB = 64: a 32-wide one).  Logical byte
// (row, b) lives in 16-byte chunk c = b/16 of its row; the chunk index is
// XOR-swizzled with bits of the row so that the lanes of one ds_read_b128
// pass land on distinct banks:
//   offset(row, b) = row*RB + 16*(c ^ swz(row)) + b%16
// with swz(row) = ((row >> shift) ^ ((row >> (shift + 4)) & 1)) & (RB/16 - 1).
// For RB = 128 and shift 0 the first term is the pages' SWIZZLE_128B rule
// (row-in-8 XOR the 16-byte chunk, Swizzle<3,4,3> on byte offsets); the
// second flips chunk bit 0 on rows 16-31 of every 32 (Swizzle<1,4,7>
// composed on top).  gfx950 serves a ds_read_b128 in passes that pair
// lanes 0-7 with 16-23 (and 8-15 with 24-31, ...) over 64 banks of 4 bytes;
// the 32-row instructions put rows r and r + 16 of one chunk into one pass,
// which SWIZZLE_128B alone sends to the same banks (a 2-way conflict on
// every fragment read, seen in the LDS conflict counter).  The extra flip
// separates them and leaves the 16-row patterns conflict-free.  Any per-row
// XOR is a bijection on the row's chunks, and the writer (loader) and the
// reader (fragment load) call this one function.
// ---------------------------------------------------------------------------

constexpr int32_t kRowBytes = 128;

SL_HD constexpr int32_t swz(int32_t row, int32_t shift, int32_t row_bytes = kRowBytes) {
  return ((row >> shift) ^ ((row >> (shift + 4)) & 1)) & (row_bytes / 16 - 1);
}

SL_HD constexpr int32_t lds_offset(int32_t row, int32_t byte_in_row, int32_t shift,
                                   int32_t row_bytes = kRowBytes) {
  return row * row_bytes + 16 * (((byte_in_row >> 4) ^ swz(row, shift, row_bytes)) & (row_bytes / 16 - 1)) +
         (byte_in_row & 15);
}

// Byte offset in the LDS tile that lane `lane` reads, for its 16-byte
// fragment piece `piece` (f16: 1 piece of 8 halves; f8: 2 pieces of 16
// bytes), of the MFMA tile whose first row is `row0`, at k-slice `ks` (in
// units of the instruction's K).
SL_HD constexpr int32_t fragment_lds_offset(int32_t instr, int32_t lane, int32_t piece, int32_t row0,
                                            int32_t ks, int32_t shift, int32_t row_bytes = kRowBytes) {
  const Coord c = operand_map(instr, lane, piece * 16 / (instr_in_slots(instr) == 8 ? 2 : 1));
  const int32_t elem_bytes = instr_in_slots(instr) == 8 ? 2 : 1;
  const int32_t byte = (ks * instr_k(instr) + c.col) * elem_bytes;
  return lds_offset(row0 + c.row, byte, shift, row_bytes);
}

// ---------------------------------------------------------------------------
// M- (N-) major LDS tile, for operands stored with M (or N) contiguous: the
// tile keeps the global orientation, 64 K-rows of `rows` fp16 each, so the
// HBM -> LDS copy moves whole 16-byte chunks along M with no register
// transpose.  16-byte chunk c of K-row k sits at physical chunk
//   c ^ mn_swz(k),  mn_swz(k) = 2 * ((k & 3) | ((k >> 3) & 1) << 2)
// (an XOR on chunk bits 1-3; rows >= 128 keeps it inside the row).
//
// The MFMA fragment (lane l = l0 + 16 l1 wants element (row l0, k 8 l1 + v))
// is read with two ds_read_b64_tr_b16: in such a read the 16 lanes of group
// l1 each supply the address of one 8-byte block (4 consecutive rows at one
// k), the group's 16 blocks form a 4 x 16 matrix (row j = blocks of lanes
// 4j .. 4j+3) and lane i receives its column i.  Lane p of group l1 in read
// r therefore supplies the block of rows row0 + 4 (p % 4) .. + 3 at
// k = 32 ks + 8 l1 + 4 r + p / 4, and lane i receives rows row0 + i at
// k = 32 ks + 8 l1 + 4 r + j, j = 0..3: slots 4 r .. 4 r + 3 of its
// fragment.  With the swizzle above the 8 K-rows that one 32-lane half of
// the read touches land on 16 distinct 16-byte bank groups.
// ---------------------------------------------------------------------------

SL_HD constexpr int32_t mn_swz(int32_t k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

SL_HD constexpr int32_t mn_lds_offset(int32_t k, int32_t row, int32_t rows) {
  return k * rows * 2 + 16 * ((row >> 3) ^ mn_swz(k)) + (row & 7) * 2;
}

// byte address lane `lane` supplies to transposing read r (0, 1) of the
// fragment of the 16-row MFMA tile at `row0`, k-slice `ks` (32 wide)
SL_HD constexpr int32_t tr_read_offset(int32_t lane, int32_t r, int32_t row0, int32_t ks, int32_t rows) {
  return mn_lds_offset(32 * ks + 8 * (lane / 16) + 4 * r + (lane % 16) / 4, row0 + 4 * (lane % 4), rows);
}

}  // namespace sl
