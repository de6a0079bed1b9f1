// describe.cpp -- the plan trace: every stage of the planned GEMM written as
// a shape:stride layout ("数据布局及其记号", section "Shape-Stride 模型"),
// each one computed from the previous ones with the host layout algebra the
// way "CuTe 中 A、B 如何加载到 MMA 寄存器" builds its views: the operand
// divided into workgroup tiles, the tile in LDS, the instruction's TV map,
// the wave's partition of the LDS tile (composition of the tile with the TV
// slice, section 2), the registers that hold it (make_fragment_like,
// section 3), and the accumulator's partition of D.
//
// Units: A, B, C, D layouts count elements of their dtype (E2M1 elements
// are nibbles, two per byte); LDS tile layouts count elements of the LDS
// tile (fp16 / bf16 halves, fp8 bytes, fp4 nibbles) before the XOR
// swizzle, which is stated next to them; copy layouts count LDS bytes.
// Instruction TV layouts map (lane, slot) to row + R * k of the R x K_I
// instruction tile (D: m + R * n).
#include "describe.hpp"

#include <cstdarg>
#include <cstdio>
#include <functional>
#include <vector>

#include "layout_algebra.hpp"
#include "sl_kernels.hpp"
#include "sl_maps.hpp"

namespace sl {
namespace {

using la::Layout;

Layout S(int64_t s, int64_t d) { return Layout::mode(s, d); }         // compile-time constant
Layout R(int64_t s, int64_t d) { return Layout::mode(s, d, false); }  // run-time value
Layout T(std::vector<Layout> k) { return Layout::tuple(std::move(k)); }

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

int log2i(int64_t v) {
  int r = 0;
  while ((int64_t(1) << (r + 1)) <= v) ++r;
  return r;
}

struct Out {
  std::string s;
  void note(const std::string& t) { s += "# " + t + "\n"; }
  void line(const std::string& name, const Layout& l, const std::string& why = "") {
    s += name + ": " + la::to_string(l);
    if (!why.empty()) s += "  # " + why;
    s += "\n";
  }
  // a stage computed with the algebra; an undefined case prints its reason
  void stage(const std::string& name, const std::function<Layout()>& f, const std::string& why = "") {
    try {
      line(name, f(), why);
    } catch (const la::Error& e) {
      s += "# " + name + ": not one layout (" + e.what + ")\n";
    }
  }
};

// The matrix-core instruction of a kernel family.
struct InstrInfo {
  int32_t id;        // sl::Instr
  std::string name;  // mnemonic and data format
  int32_t rows;      // R: rows of A and of B per instruction
  int32_t k;         // K_I: K per instruction (elements)
  int32_t kl;        // K elements per lane group (lanes l0 + R*l1 share l1)
};

InstrInfo instr_of(const DescribeInput& in) {
  const bool bf16 = in.flags & F_BF16;
  switch (in.kernel) {
    case K_MX: return {MFMA16_F8, "v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 data, E8M0 scales)", 16, 128, 16};
    case K_MX_W8:
    case K_MX_W4R: return {MFMA32_F8, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 data, E8M0 scales)", 32, 64, 16};
    case K_MXFP4: return {MFMA32_F4, "v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 data, E8M0 scales)", 32, 64, 32};
    case K_MXFP6:
      return {MFMA32_F6,
              std::string("v_mfma_scale_f32_32x32x64_f8f6f4 (") + ((in.flags & F_FP6) ? "E2M3" : "E3M2") +
                  " data, E8M0 scales)",
              32, 64, 32};
    default:
      return {MFMA16_F16, bf16 ? "v_mfma_f32_16x16x32_bf16" : "v_mfma_f32_16x16x32_f16", 16, 32, 8};
  }
}

// slot modes of one lane's operand values, as steps of `unit` per unit of k
// (unit R: the instruction tile's coordinate row + R k; unit BM: a tile's)
Layout slot_modes(const InstrInfo& I, int64_t unit) {
  switch (I.id) {
    case MFMA16_F8:
    case MFMA32_F8: return T({S(16, unit), S(2, unit * (I.k / 2))});  // two 16-byte pieces, K_I/2 apart
    case MFMA16_F4:
    case MFMA32_F4:
    case MFMA16_F6:
    case MFMA32_F6: return T({S(32, unit)});
    default: return T({S(8, unit)});
  }
}

Layout lane_modes(const InstrInfo& I, int64_t unit) { return T({S(I.rows, 1), S(64 / I.rows, unit * I.kl)}); }

// accumulator (lane, reg) -> m + unit * n in our (m, n): the kernels issue
// the instruction with the B tile first, so its rows are our n
Layout acc_lane(const InstrInfo& I, int64_t unit) {
  return I.rows == 16 ? T({S(16, 1), S(4, 4 * unit)}) : T({S(32, 1), S(2, 4 * unit)});
}
Layout acc_regs(const InstrInfo& I, int64_t unit) {
  return I.rows == 16 ? T({S(4, unit)}) : T({S(4, unit), S(4, 8 * unit)});
}

const char* load_name(int32_t l) {
  switch (l) {
    case LOAD_KVEC: return "K-contiguous 16-byte direct HBM->LDS loads";
    case LOAD_MNVEC: return "M-contiguous 16-byte loads, 8x8 register transpose, K-major LDS writes";
    case LOAD_GENERIC: return "element loads (any strides)";
    case LOAD_MNDMA: return "M-contiguous 16-byte direct HBM->LDS loads into an M-major tile";
    case LOAD_NVFP4: return "packed E2M1 16-byte loads, decoded and scaled to fp16 in registers";
    case LOAD_NVFP4_PAIRS:
      return "packed E2M1 16-byte loads of two K-tiles at once, 8-byte scale loads, decoded and scaled to fp16 in "
             "registers";
    default: return "?";
  }
}

const char* kernel_name(int32_t k) {
  switch (k) {
    case K_F16: return "16-bit GEMM, vector loaders";
    case K_F16_GENERIC: return "16-bit GEMM, element loader on one side";
    case K_MX: return "MXFP8 GEMM, 4 waves";
    case K_MX_W8: return "MXFP8 GEMM, 8 waves, scales staged in LDS";
    case K_NVFP4: return "NVFP4 GEMM, dequantised to fp16 tiles";
    case K_MXFP4: return "MXFP4 GEMM, scaled 32x32x64 instruction on E2M1 data";
    case K_MXFP6: return "MXFP6 GEMM, scaled 32x32x64 instruction on 6-bit data";
    case K_MX_W4R: return "MXFP8 GEMM, 4 waves, scales loaded into registers";
    default: return "?";
  }
}

// (rows, cols[, batch]) view of an operand
Layout view(int64_t rows, int64_t cols, int64_t rs, int64_t cs, bool batched, int64_t batch, int64_t bs) {
  if (batched) return T({R(rows, rs), R(cols, cs), R(batch, bs)});
  return T({R(rows, rs), R(cols, cs)});
}

void operand(Out& o, const DescribeInput& in, const InstrInfo& I, char name, int32_t load) {
  const bool isA = name == 'A';
  const int64_t rows = isA ? in.M : in.N;
  const int64_t rs = isA ? in.a_rs : in.b_rs, cs = isA ? in.a_cs : in.b_cs, bs = isA ? in.a_bs : in.b_bs;
  const bool batched = isA ? in.a_batched : in.b_batched;
  const int32_t BR = isA ? in.bm : in.bn;                 // tile rows
  const int32_t W = isA ? in.wm : in.wn;                  // waves along these rows
  const int32_t TR = BR / W;                              // wave tile rows
  const int32_t F = TR / I.rows;                          // instruction repeats
  const int32_t KS = in.bk / I.k;                         // K slices per K-tile
  const bool fp4 = in.kernel == K_MXFP4;
  const bool fp6 = in.kernel == K_MXFP6;
  const bool fp8 = in.kernel == K_MX || in.kernel == K_MX_W8 || in.kernel == K_MX_W4R;
  // the 4-wave MX kernel packs 6-bit K-tiles: rows 96 bytes apart in LDS
  // (LoaderFP6Packed); the 8-wave one pads them to 128-byte rows
  const bool packed = fp6 && in.ring;
  const int32_t RB = fp4 ? in.bk / 2 : packed ? 96 : fp6 ? 128 : fp8 ? in.bk : in.bk * 2;  // LDS bytes per tile row
  const std::string n(1, name);
  const Layout X = view(rows, in.K, rs, cs, batched, in.batch, bs);

  o.line(n, X, isA ? "element (m, k[, batch])" : "element (n, k[, batch])");
  o.stage(n + "_tiles", [&] { return la::zipped_divide(T({R(rows, rs), R(in.K, cs)}), T({S(BR, 1), S(in.bk, 1)})); },
          fmt("zipped_divide by the %dx%d workgroup tile: ((tile), (tile index)); a ragged last tile is "
              "completed with zeros by the loads",
              BR, in.bk));
  o.note(n + " loader: " + load_name(load));

  const bool mmajor = load == LOAD_MNDMA;
  // 6-bit data is counted in bits (an element is 6 of them)
  const Layout tile = mmajor ? T({S(BR, 1), S(in.bk, BR)})
                      : fp6  ? T({S(BR, 8 * RB), S(in.bk, 6)})
                             : T({S(BR, in.bk), S(in.bk, 1)});
  if (packed) {
    o.line(n + "_lds", tile,
           fmt("bits: a K-tile's %d values are the %d bytes of a row, rows %d bytes apart, as 6 chunks of 16 "
               "bytes; chunk c of row r sits at chunk (c + ((r >> 4) & 1)) mod 6 of the row",
               in.bk, RB, RB));
  } else if (fp6) {
    const int b = log2i(RB / 16), sh = log2i(RB);
    o.line(n + "_lds", tile,
           fmt("bits: a K-tile's %d values are the first %d bytes of a %d-byte row (the rest zero, never "
               "read); byte b of row r at r*%d + 16((b/16) ^ swz(r)) + b%%16, swz(r) = (r ^ (r>>4)&1) & %d: "
               "Swizzle<%d,4,%d> then Swizzle<1,4,%d> on byte offsets",
               in.bk, in.bk * 6 / 8, RB, RB, RB / 16 - 1, b, sh - 4, sh));
  } else if (mmajor) {
    o.line(n + "_lds", tile,
           fmt("M-major: K-row k of %d elements; its 16-byte chunk c at c ^ 2((k&3)|((k>>3)&1)<<2)", BR));
  } else {
    const int b = log2i(RB / 16), sh = log2i(RB);
    o.line(n + "_lds", tile,
           fmt("byte b of row r at r*%d + 16((b/16) ^ swz(r)) + b%%16, swz(r) = (r ^ (r>>4)&1) & %d: "
               "Swizzle<%d,4,%d> then Swizzle<1,4,%d> on byte offsets",
               RB, RB / 16 - 1, b, sh - 4, sh));
  }
  if (load == LOAD_KVEC || load == LOAD_MNDMA) {
    const int32_t NT = in.wm * in.wn * 64, WV = NT / 64;
    const int32_t tile_bytes = mmajor ? in.bk * BR * 2 : BR * RB;
    const int32_t iters = tile_bytes / (NT * 16);
    if (iters >= 1)
      o.line(n + "_copy", T({S(64, 16), S(WV, 1024), S(iters, 1024 * WV)}),
             mmajor ? "LDS bytes filled by (lane, wave, instruction); the lane landing in chunk p of K-row k "
                      "loads chunk p ^ swz(k) of that row"
             : packed ? "LDS bytes filled by (lane, wave, instruction); the lane landing in chunk p of row r "
                        "loads chunk (p - ((r >> 4) & 1)) mod 6 of the row's K-tile"
                      : "LDS bytes filled by (lane, wave, instruction); the lane landing in chunk p of row r "
                        "loads chunk p ^ swz(r) of that row");
  }
  // wave partition of the LDS tile: (lane, ((slots), repeats, K slices)),
  // first in the tile's coordinates (row + BR * k), then through the tile
  const Layout slots = slot_modes(I, BR);
  // packed 6-bit rows: lane half h takes the K-tile's 32-value blocks 2h
  // (K slice 0) and 2h + 1 (slice 1), so the lane-half mode steps 64
  // values and the slice mode 32
  const int64_t slice_k = packed ? 32 : I.k;
  std::vector<Layout> vals{slots, S(F, I.rows), S(KS, (int64_t)BR * slice_k)};
  const Layout lanes = packed ? T({S(I.rows, 1), S(64 / I.rows, (int64_t)BR * 64)}) : lane_modes(I, BR);
  const Layout part = T({lanes, T(vals)});
  o.stage(n + "_wave", [&] { return la::composition(tile, part); },
          fmt("(lane, ((slot), %c repeat, K slice)) -> element of the LDS tile; wave w starts at row %d*(w%s%d)",
              isA ? 'M' : 'N', TR, isA ? " % " : " / ", in.wm));
  const Layout lane0 = T({slots, S(F, I.rows), S(KS, (int64_t)BR * slice_k)});
  o.stage(n + "_lane0", [&] { return la::composition(tile, lane0); }, "lane 0's values (the wave partition at lane 0)");
  if (packed)
    o.note(n + " fragments: lane half h = lane / 32 takes blocks 2h and 2h + 1 of the K-tile (its 32 values, "
                 "24 bytes, per K slice): slice 0 one 16-byte read (chunk 3h) and one 8-byte read (the low half "
                 "of chunk 3h + 1), slice 1 one 8-byte read (its high half) and one 16-byte read (chunk 3h + 2); "
                 "the 16-byte reads are free of bank conflicts, the 8-byte reads take two passes");
  else if (fp6)
    o.note(n + " fragments: one 16-byte and one 8-byte LDS read per lane per instruction tile (its 32 values, "
                 "24 bytes)");
  o.stage(n + "_frag", [&] { return la::fragment_like(la::composition(tile, T({slots, S(F, I.rows)}))); },
          fmt("fragment_like of one K slice: the registers the lane reads it into (%d values x %d), reloaded "
              "per K slice",
              (int)la::size(slots), F));
  if (mmajor)
    o.note(n + " fragments: two ds_read_b64_tr_b16 per instruction tile, slots 4r..4r+3 from read r "
               "(the slot stride above is a whole K-row)");
}

void workgroup_map(Out& o, const DescribeInput& in) {
  const int64_t total = in.workgroups;
  const int64_t q = total / 8;
  o.note(fmt("workgroup b -> XCD x = b %% 8 takes the contiguous range x*%lld.. of the tile order; the order walks "
             "groups of %d tile-rows column by column",
             (long long)q, in.group_m));
  if (total % 8 == 0 && in.batch == 1 && in.splits == 1 && in.tiles_m % in.group_m == 0) {
    const Layout xcd = T({S(8, q), S(q, 1)});
    const Layout order = T({S(in.group_m, 1), S(in.tiles_n, in.tiles_m), S(in.tiles_m / in.group_m, in.group_m)});
    o.line("tile_order", order, "order index -> tm + tiles_m*tn");
    o.stage("workgroup_tile", [&] { return la::composition(order, xcd); },
            "tile_order o (8, b/8):(range, 1): workgroup b -> tm + tiles_m*tn");
  } else {
    o.note("workgroup -> tile is not one layout for this grid (ragged group, batch or split index); the formula "
           "above applies");
  }
}

void accumulators(Out& o, const DescribeInput& in, const InstrInfo& I) {
  const int32_t TM = in.bm / in.wm, TN = in.bn / in.wn;
  const int32_t FM = TM / I.rows, FN = TN / I.rows;
  const int32_t regs = I.rows == 16 ? 4 : 16;
  o.line("D_instr", T({acc_lane(I, I.rows), acc_regs(I, I.rows)}),
         fmt("accumulator (lane, reg) -> m + %d n of the instruction tile", I.rows));
  o.line("acc", T({S(regs, 1), S(FM, regs * FN), S(FN, regs)}), "fp32 registers acc[i][j][r] as (r, i, j)");
  const Layout dtile = T({R(in.bm, in.d_rs), R(in.bn, in.d_cs)});
  const Layout slice = T({acc_regs(I, in.bm), S(FM, I.rows), S(FN, (int64_t)I.rows * in.bm)});
  o.stage("D_lane0", [&] { return la::composition(dtile, slice); },
          fmt("D elements of lane 0's (r, i, j) from the wave's corner; lane l adds row l %% %d and column "
              "4 (l / %d)",
              I.rows, I.rows));
  o.note(std::string("epilogue: 4 consecutive n of one m per store; ") +
         ((in.flags & F_D_VEC) ? "one 8-byte store (D rows contiguous and aligned)" : "element stores") +
         (in.has_c ? ((in.flags & F_C_VEC) ? ", C read as 8 bytes" : ", C read by elements") : ", no C"));
}

}  // namespace

std::string describe_plan(const DescribeInput& in) {
  Out o;
  const InstrInfo I = instr_of(in);
  const int32_t NT = in.wm * in.wn * 64;
  if (in.ring)
    o.note(fmt("kernel %d: %s; tile %dx%dx%d, %d waves (%d x %d), wave tile %dx%d with accumulators in AGPRs; LDS "
               "a ring of five operand K-tiles (operand tile q = A of K-tile q/2 for even q, B for odd q, in slot "
               "q %% 5), %d LDS bytes",
               in.kernel, kernel_name(in.kernel), in.bm, in.bn, in.bk, NT / 64, in.wm, in.wn, in.bm / in.wm,
               in.bn / in.wn, in.lds_bytes));
  else
    o.note(fmt("kernel %d: %s; tile %dx%dx%d, %d waves (%d x %d), wave tile %dx%d, %d LDS stages, %d LDS bytes",
               in.kernel, kernel_name(in.kernel), in.bm, in.bn, in.bk, NT / 64, in.wm, in.wn, in.bm / in.wm,
               in.bn / in.wn, in.stages, in.lds_bytes));
  o.note(fmt("M=%lld N=%lld K=%lld batch=%lld: %lld workgroups of %d threads, split_k %d", (long long)in.M,
             (long long)in.N, (long long)in.K, (long long)in.batch, (long long)in.workgroups, NT, in.splits));
  o.note("instruction: " + I.name + " (issued with the B tile as its first operand)");
  o.line("A_instr", T({lane_modes(I, I.rows), slot_modes(I, I.rows)}),
         fmt("(lane, slot) -> m + %d k of the %dx%d A operand (B: n for m)", I.rows, I.rows, I.k));
  operand(o, in, I, 'A', in.a_load);
  operand(o, in, I, 'B', in.b_load);
  if (in.kernel == K_MX || in.kernel == K_MX_W8 || in.kernel == K_MX_W4R || in.kernel == K_MXFP4 ||
      in.kernel == K_MXFP6 || in.kernel == K_NVFP4) {
    const int64_t kb = (in.K + in.block_k - 1) / in.block_k;
    const char* fmt_s = in.kernel == K_NVFP4 ? "E4M3" : "E8M0";
    o.line("SFA", T({R(in.M, in.sa_rs), R(kb, in.sa_cs)}), fmt("%s scale of A(m, %d j .. %d j + %d)", fmt_s,
                                                                in.block_k, in.block_k, in.block_k - 1));
    o.line("SFB", T({R(in.N, in.sb_rs), R(kb, in.sb_cs)}), fmt("%s scale of B(n, block)", fmt_s));
    if (in.kernel == K_NVFP4 && in.nv_decoded) {
      const int64_t bytes_a = in.batch * in.M * in.K * 2;
      o.line("A_decoded", T({R(in.M, in.K), R(in.K, 1), R(in.batch, in.M * in.K)}),
             "fp16 (m, k, batch) in the workspace from byte 0: a first kernel turns each 16-value block into "
             "E2M1 x its E4M3 scale (exact in fp16)");
      o.line("B_decoded", T({R(in.N, in.K), R(in.K, 1), R(in.batch, in.N * in.K)}),
             fmt("fp16 (n, k, batch) in the workspace from byte %lld; the stages above read these rows, not the "
                 "packed operands", (long long)((bytes_a + 255) / 256 * 256)));
    } else if (in.kernel == K_NVFP4) {
      o.note("NVFP4: each lane decodes 8 E2M1 values and multiplies them by their E4M3 scale into exact fp16 "
             "before the LDS write; the fp16 path follows");
    } else {
      o.line("scale_instr", T({S(I.rows, 1), S(64 / I.rows, I.rows)}),
             fmt("scale lane -> row + %d (K block of 32) of the instruction", I.rows));
      if (in.ring)
        o.note(fmt("scales: one 16-byte load per row per %d K-tiles straight into registers (the LDS holds the "
                   "ring); slice s takes dword s / 2 of its K-tile's scale bytes, shifted right by 8 (lane / 32)",
                   in.kernel == K_MXFP4 ? 2 : 4));
      else if (in.kernel != K_MX)
        o.note((in.flags & F_SCALE16)
                   ? fmt("scales: one 16-byte chunk per row per %d K-tiles, staged in two LDS buffers of %d bytes",
                         in.kernel == K_MXFP4 ? 2 : 4, (in.bm + in.bn) * 16)
                   : std::string("scales: one dword per row per K-tile, staged with the data"));
      else
        o.note("scales: byte loads from HBM per K-tile");
    }
  }
  accumulators(o, in, I);
  o.line("D", view(in.M, in.N, in.d_rs, in.d_cs, in.d_batched, in.batch, in.d_bs), "element (m, n[, batch])");
  if (in.has_c) o.line("C", view(in.M, in.N, in.c_rs, in.c_cs, in.c_batched, in.batch, in.c_bs));
  o.stage("D_tiles", [&] { return la::zipped_divide(T({R(in.M, in.d_rs), R(in.N, in.d_cs)}), T({S(in.bm, 1), S(in.bn, 1)})); },
          "zipped_divide by the output tile");
  workgroup_map(o, in);
  if (in.splits > 1) {
    const int64_t mn = in.M * in.N;
    o.line("workspace", T({R(in.M, in.N), R(in.N, 1), R(in.batch, mn), R(in.splits, in.batch * mn)}),
           fmt("fp32 partial sums (m, n, batch, split); split s covers K-tiles [%d s, %d s + %d); a second kernel "
               "writes D = C + their sum",
               in.split_tiles, in.split_tiles, in.split_tiles));
  }
  return o.s;
}

}  // namespace sl
