// describe.hpp -- text trace of the layouts every stage of a planned GEMM
// uses, computed with the host layout algebra.
#pragma once
#include <stdint.h>

#include <string>

namespace sl {

struct DescribeInput {
  int32_t kernel;          // KernelKind
  int32_t a_load, b_load;  // LoadKind
  int32_t bm, bn, bk;      // workgroup tile (bk in elements)
  int32_t wm, wn, stages;  // waves along M and N, LDS stages
  int32_t splits, split_tiles, group_m, tiles_m, tiles_n;
  int64_t workgroups, batch, M, N, K;
  // element strides (batch, row, col); *_batched: the operand is rank 3
  int64_t a_bs, a_rs, a_cs, b_bs, b_rs, b_cs, c_bs, c_rs, c_cs, d_bs, d_rs, d_cs;
  int64_t sa_rs, sa_cs, sb_rs, sb_cs;
  bool a_batched, b_batched, c_batched, d_batched, has_c;
  int32_t flags;    // GemmParams flags
  int32_t block_k;  // scale block (MX 32, NVFP4 16)
  int32_t lds_bytes;
  bool ring;  // LDS as a ring of five operand K-tiles (the 4-wave 256x256 kernel)
  bool nv_decoded;  // NVFP4 operands decoded to fp16 rows in the workspace by a first kernel
};

// One line per stage: "name: layout  # note" (the layout parses back with
// the algebra's parser) or "# note" lines.
std::string describe_plan(const DescribeInput& in);

}  // namespace sl
