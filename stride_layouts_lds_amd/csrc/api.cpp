// api.cpp -- the C ABI of include/sl.h: descriptor validation and
// classification (host only), kernel selection, launch, and the map
// queries / device probes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>

#include "../../include/sl.h"
#include "describe.hpp"
#include "layout_algebra.hpp"
#include "sl_kernels.hpp"
#include "sl_maps.hpp"

namespace {

thread_local std::string g_msg;

sl_status fail(sl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sl_status fail(sl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

int elem_size(int32_t dt) {
  switch (dt) {
    case SL_F16: return 2;
    case SL_BF16: return 2;
    case SL_F32: return 4;
    case SL_F8_E4M3: return 1;
    case SL_E8M0: return 1;
    case SL_F4_E2M1: return 1;  // two elements per byte: byte_range halves the span
    case SL_F6_E2M3:
    case SL_F6_E3M2: return 1;  // four elements per three bytes: byte_range scales the span
    default: return 0;
  }
}

// A matrix view (batch stride, row stride, column stride) of a descriptor.
struct View {
  const sl_tensor* t;
  int64_t batch;  // 1 for rank 2
  int64_t rows, cols;
  int64_t bs, rs, cs;
  bool present;
};

sl_status make_view(const char* name, const sl_tensor& t, View* v) {
  v->t = &t;
  v->present = true;
  const sl_layout& L = t.layout;
  if (L.rank != 2 && L.rank != 3) return fail(SL_ERR_LAYOUT, "%s: rank %d (expected 2 or 3)", name, L.rank);
  for (int i = 0; i < L.rank; ++i) {
    if (L.shape[i] < 0) return fail(SL_ERR_SHAPE, "%s: negative size %lld", name, (long long)L.shape[i]);
    if (L.stride[i] < 0) return fail(SL_ERR_LAYOUT, "%s: negative stride %lld", name, (long long)L.stride[i]);
  }
  if (L.rank == 3) {
    v->batch = L.shape[0];
    v->rows = L.shape[1];
    v->cols = L.shape[2];
    v->bs = L.stride[0];
    v->rs = L.stride[1];
    v->cs = L.stride[2];
  } else {
    v->batch = 1;
    v->rows = L.shape[0];
    v->cols = L.shape[1];
    v->bs = 0;
    v->rs = L.stride[0];
    v->cs = L.stride[1];
  }
  return SL_OK;
}

// [lo, hi) byte range a view can touch, for `batch` batches.
void byte_range(const View& v, int64_t batch, uintptr_t* lo, uintptr_t* hi) {
  const int es = elem_size(v.t->dtype);
  const int64_t nb = v.t->layout.rank == 3 ? batch : 1;
  int64_t last = 0;
  if (nb > 0 && v.rows > 0 && v.cols > 0) last = (nb - 1) * v.bs + (v.rows - 1) * v.rs + (v.cols - 1) * v.cs;
  *lo = (uintptr_t)v.t->data;
  if (v.t->dtype == SL_F4_E2M1)
    *hi = (uintptr_t)v.t->data + (uintptr_t)(last / 2 + 1);
  else if (v.t->dtype == SL_F6_E2M3 || v.t->dtype == SL_F6_E3M2)
    *hi = (uintptr_t)v.t->data + (uintptr_t)((6 * last + 5) / 8 + 1);
  else
    *hi = (uintptr_t)v.t->data + (uintptr_t)((last + 1) * es);
}

// Distinct (batch, row, col) must map to distinct addresses.
bool injective(const View& v, int64_t batch) {
  struct Dim {
    int64_t n, s;
  } d[3] = {{batch, v.bs}, {v.rows, v.rs}, {v.cols, v.cs}};
  Dim live[3];
  int k = 0;
  for (auto& x : d)
    if (x.n > 1) live[k++] = x;
  std::sort(live, live + k, [](const Dim& a, const Dim& b) { return a.s < b.s; });
  int64_t span = 0;  // largest offset reached by the faster dims
  for (int i = 0; i < k; ++i) {
    if (live[i].s <= span) return false;
    span += live[i].s * (live[i].n - 1);
  }
  return true;
}

bool same_layout(const sl_tensor& x, const sl_tensor& y) {
  if (x.layout.rank != y.layout.rank) return false;
  for (int i = 0; i < x.layout.rank; ++i)
    if (x.layout.shape[i] != y.layout.shape[i] || x.layout.stride[i] != y.layout.stride[i]) return false;
  return true;
}

struct Plan {
  sl_plan pub;
  sl::GemmParams p;
  int32_t tile;
  bool mx;
  bool empty;
  size_t ws_bytes;  // workspace: split-K partial sums, or NVFP4 operands decoded to fp16 (0: none)
  bool nv_dec;      // NVFP4 decoded ahead into the workspace, then the fp16 ring kernel
  sl::Nvfp4Decode dec[2];  // A and B (out set at launch)
  size_t dec_off_b, dec_bytes;  // B's offset in the workspace, and the total
  // byte ranges of the operands with data, for the workspace overlap check
  uintptr_t lo[6], hi[6];
  int32_t nranges;
};

int32_t env_int(const char* name, int32_t dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return (int32_t)strtol(s, nullptr, 10);
}

// Loader for one operand: rows x K with strides (rs along rows, ks along K).
int32_t choose_load(const View& v, int64_t K, int64_t tile_rows, int es) {
  const uintptr_t addr = (uintptr_t)v.t->data;
  const int64_t vec = 16 / es;  // elements per 16 bytes
  const bool base16 = addr % 16 == 0 && (v.t->layout.rank == 2 || v.bs % vec == 0);
  const int64_t limit = (int64_t)1 << 31;
  if (v.cs == 1 && base16 && v.rs % vec == 0 && K % vec == 0 &&
      ((tile_rows - 1) * v.rs + K) * es < limit)
    return sl::LOAD_KVEC;
  if (es == 2 && v.rs == 1 && base16 && v.cs % vec == 0 && v.rows % 8 == 0 &&
      ((K > 0 ? K - 1 : 0) * v.cs + tile_rows) * es < limit)
    return sl::LOAD_MNVEC;
  return sl::LOAD_GENERIC;
}

// Estimated relative cost of one tile shape: the number of workgroup waves
// over the 256 CUs times the time of one wave, where `per_cu` co-resident
// workgroups share a CU, with an efficiency factor that favours big tiles
// (fewer LDS bytes per MFMA).
double tile_cost(const sl::TileShape& t, int64_t batch, int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = batch * ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  const int64_t lds = (int64_t)t.stages * (t.bm + t.bn) * t.bk * 2;
  const int64_t per_cu = lds <= 80 * 1024 ? 2 : 1;
  const int64_t slots = 256 * per_cu;
  const int64_t waves = (tiles + slots - 1) / slots;
  // the streaming tile moves 5x the L2 bytes per MFMA of a 256x256 tile:
  // worth it only where the big tiles leave most of the chip idle
  const double eff = (t.bm == 256 && t.bn == 256) ? 1.0
                     : (t.bm == 256 && t.bn == 192) ? 0.96
                     : (t.bm * t.bn == 256 * 128) ? 0.92
                     : (t.bm * t.bn == 128 * 128) ? 0.80
                                                  : 0.50;
  return (double)waves * (double)t.bm * (double)t.bn * (double)std::max<int64_t>(K, 64) * per_cu / eff;
}

sl_status plan_gemm(const sl_gemm_args* args, Plan* out, bool allow_decode = true) {
  g_msg.clear();
  if (!args) return fail(SL_ERR_NULL, "args is NULL");
  const bool fp4 = args->a.dtype == SL_F4_E2M1;
  // E2M1 data: NVFP4 (E4M3 scales per 16) or MXFP4 (E8M0 scales per 32)
  const bool nvfp4 = fp4 && args->sfa.dtype == SL_F8_E4M3;
  const bool mxfp4 = fp4 && !nvfp4;
  // 6-bit data: MXFP6 (E8M0 scales per 32)
  const bool mxfp6 = args->a.dtype == SL_F6_E2M3 || args->a.dtype == SL_F6_E3M2;
  const bool mx = args->a.dtype == SL_F8_E4M3 || fp4 || mxfp6;
  // dtypes
  if (mxfp6) {
    if (args->b.dtype != args->a.dtype) return fail(SL_ERR_DTYPE, "b must have a's 6-bit format");
    if (args->sfa.dtype != SL_E8M0 || args->sfb.dtype != SL_E8M0 || args->block_k != 32)
      return fail(SL_ERR_DTYPE, "6-bit operands take e8m0 sfa and sfb with block_k 32");
  } else if (nvfp4) {
    if (args->b.dtype != SL_F4_E2M1) return fail(SL_ERR_DTYPE, "b must be f4_e2m1 when a is");
    if (args->sfb.dtype != SL_F8_E4M3 || args->block_k != 16)
      return fail(SL_ERR_DTYPE, "NVFP4 takes f8_e4m3 sfa and sfb with block_k 16");
  } else if (mxfp4) {
    if (args->b.dtype != SL_F4_E2M1) return fail(SL_ERR_DTYPE, "b must be f4_e2m1 when a is");
    if (args->sfa.dtype != SL_E8M0 || args->sfb.dtype != SL_E8M0 || args->block_k != 32)
      return fail(SL_ERR_DTYPE,
                  "f4_e2m1 operands take f8_e4m3 scales with block_k 16 (NVFP4) or e8m0 with block_k 32 (MXFP4)");
  } else if (mx) {
    if (args->b.dtype != SL_F8_E4M3) return fail(SL_ERR_DTYPE, "b must be f8_e4m3 when a is");
    if (args->sfa.dtype != SL_E8M0 || args->sfb.dtype != SL_E8M0)
      return fail(SL_ERR_DTYPE, "MX operands need e8m0 sfa and sfb");
    if (args->block_k != 32) return fail(SL_ERR_SHAPE, "block_k must be 32 for MXFP8 (got %d)", args->block_k);
  } else {
    if (!((args->a.dtype == SL_F16 && args->b.dtype == SL_F16) || (args->a.dtype == SL_BF16 && args->b.dtype == SL_BF16)))
      return fail(SL_ERR_DTYPE, "a and b must both be f16, both bf16, or both f8_e4m3 with scales");
    if (args->sfa.data || args->sfb.data) return fail(SL_ERR_DTYPE, "scales given for 16-bit operands");
  }
  // D (and C) are bf16 for bf16 operands, f16 otherwise
  const bool bf16 = args->a.dtype == SL_BF16;
  const int32_t out_dt = bf16 ? SL_BF16 : SL_F16;
  if (args->d.dtype != out_dt) return fail(SL_ERR_DTYPE, "d must be %s", bf16 ? "bf16" : "f16");
  const bool has_c = args->c.data != nullptr;
  if (has_c && args->c.dtype != out_dt) return fail(SL_ERR_DTYPE, "c must be %s", bf16 ? "bf16" : "f16");

  View A, B, C{}, D, SA{}, SB{};
  sl_status s;
  if ((s = make_view("a", args->a, &A)) != SL_OK) return s;
  if ((s = make_view("b", args->b, &B)) != SL_OK) return s;
  if ((s = make_view("d", args->d, &D)) != SL_OK) return s;
  if (has_c && (s = make_view("c", args->c, &C)) != SL_OK) return s;
  if (mx) {
    if ((s = make_view("sfa", args->sfa, &SA)) != SL_OK) return s;
    if ((s = make_view("sfb", args->sfb, &SB)) != SL_OK) return s;
  }

  const int64_t batch = D.batch;
  const int64_t M = A.rows, K = A.cols, N = B.rows;
  if (B.cols != K) return fail(SL_ERR_SHAPE, "b is (%lld,%lld) but a has K=%lld", (long long)B.rows,
                               (long long)B.cols, (long long)K);
  if (D.rows != M || D.cols != N)
    return fail(SL_ERR_SHAPE, "d is (%lld,%lld), expected (%lld,%lld)", (long long)D.rows, (long long)D.cols,
                (long long)M, (long long)N);
  if (has_c && (C.rows != M || C.cols != N))
    return fail(SL_ERR_SHAPE, "c is (%lld,%lld), expected (%lld,%lld)", (long long)C.rows, (long long)C.cols,
                (long long)M, (long long)N);
  const View* ins[5] = {&A, &B, has_c ? &C : nullptr, mx ? &SA : nullptr, mx ? &SB : nullptr};
  const char* names[5] = {"a", "b", "c", "sfa", "sfb"};
  for (int i = 0; i < 5; ++i)
    if (ins[i] && ins[i]->t->layout.rank == 3 && ins[i]->batch != batch)
      return fail(SL_ERR_SHAPE, "%s has batch %lld, d has %lld", names[i], (long long)ins[i]->batch,
                  (long long)batch);
  const int64_t kb = nvfp4 ? (K + 15) / 16 : mx ? (K + 31) / 32 : 0;  // scale blocks per row
  if (mx) {
    if (SA.rows != M || SA.cols != kb)
      return fail(SL_ERR_SHAPE, "sfa is (%lld,%lld), expected (%lld,%lld)", (long long)SA.rows,
                  (long long)SA.cols, (long long)M, (long long)kb);
    if (SB.rows != N || SB.cols != kb)
      return fail(SL_ERR_SHAPE, "sfb is (%lld,%lld), expected (%lld,%lld)", (long long)SB.rows,
                  (long long)SB.cols, (long long)N, (long long)kb);
  }
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim || batch >= lim) return fail(SL_ERR_SHAPE, "a dimension exceeds 2^31-1");
  // Every kernel addresses an operand from its tile's first row with 64-bit
  // pointer arithmetic and 32-bit offsets inside the tile (at most 256
  // rows): only one tile's span must stay below 2^31 bytes, not the whole
  // operand's.  `row_bytes` and `k_bytes` are the packed byte counts of the
  // row stride and of K.
  auto tile_span_ok = [&](const View& X, int64_t row_bytes, int64_t k_bytes) {
    return (std::min<int64_t>(X.rows, 256) - 1) * row_bytes + k_bytes < lim;
  };
  auto scale_span_ok = [&](const View& S) {
    return (std::min<int64_t>(S.rows, 256) - 1) * S.rs + (kb - 1) * S.cs + 1 < lim;
  };

  Plan& P = *out;
  memset(&P, 0, sizeof P);
  P.mx = mx;
  P.pub.batch = batch;
  P.pub.m = M;
  P.pub.n = N;
  P.pub.k = K;
  P.empty = batch == 0 || M == 0 || N == 0;
  if (P.empty) {
    P.pub.kernel = nvfp4 ? sl::K_NVFP4 : mxfp4 ? sl::K_MXFP4 : mxfp6 ? sl::K_MXFP6 : mx ? sl::K_MX : sl::K_F16;
    return SL_OK;
  }

  // pointers and alignment
  const View* all[6] = {&A, &B, has_c ? &C : nullptr, &D, mx ? &SA : nullptr, mx ? &SB : nullptr};
  const char* all_names[6] = {"a", "b", "c", "d", "sfa", "sfb"};
  for (int i = 0; i < 6; ++i) {
    if (!all[i]) continue;
    const bool needs_data = !(i == 0 || i == 1 || i == 4 || i == 5) || K > 0;
    if (!all[i]->t->data) {
      if (needs_data) return fail(SL_ERR_NULL, "%s.data is NULL", all_names[i]);
      continue;
    }
    const int es = elem_size(all[i]->t->dtype);
    if ((uintptr_t)all[i]->t->data % es != 0)
      return fail(SL_ERR_ALIGN, "%s.data is not aligned to its %d-byte element", all_names[i], es);
  }
  // D must not broadcast; D must not overlap an input except C == D exactly
  if (!injective(D, batch)) return fail(SL_ERR_LAYOUT, "d's strides map distinct elements to one address");
  uintptr_t dlo, dhi;
  byte_range(D, batch, &dlo, &dhi);
  P.nranges = 0;
  for (int i = 0; i < 6; ++i) {
    if (!all[i] || !all[i]->t->data || ((i <= 1 || i >= 4) && K == 0)) continue;
    byte_range(*all[i], batch, &P.lo[P.nranges], &P.hi[P.nranges]);
    ++P.nranges;
  }
  for (int i = 0; i < 6; ++i) {
    if (!all[i] || i == 3 || !all[i]->t->data) continue;
    if (i == 2 && args->c.data == args->d.data && same_layout(args->c, args->d)) continue;
    if (i <= 1 && K == 0) continue;
    uintptr_t lo, hi;
    byte_range(*all[i], batch, &lo, &hi);
    if (lo < dhi && dlo < hi) return fail(SL_ERR_ALIAS, "d overlaps %s", all_names[i]);
  }

  // kernel selection
  sl::GemmParams& p = P.p;
  p.a = args->a.data;
  p.b = args->b.data;
  p.c = has_c ? args->c.data : nullptr;
  p.d = args->d.data;
  p.M = M;
  p.N = N;
  p.K = K;
  p.a_rs = A.rs, p.a_ks = A.cs, p.a_bs = A.t->layout.rank == 3 ? A.bs : 0;
  p.b_rs = B.rs, p.b_ks = B.cs, p.b_bs = B.t->layout.rank == 3 ? B.bs : 0;
  if (has_c) p.c_rs = C.rs, p.c_cs = C.cs, p.c_bs = C.t->layout.rank == 3 ? C.bs : 0;
  p.d_rs = D.rs, p.d_cs = D.cs, p.d_bs = D.t->layout.rank == 3 ? D.bs : 0;
  p.batch = (int32_t)batch;
  p.flags = has_c ? sl::F_HAS_C : 0;
  if (D.cs == 1 && D.rs % 4 == 0 && (uintptr_t)D.t->data % 8 == 0 && (batch == 1 || p.d_bs % 4 == 0))
    p.flags |= sl::F_D_VEC;
  if (has_c && C.cs == 1 && C.rs % 4 == 0 && (uintptr_t)C.t->data % 8 == 0 && (batch == 1 || p.c_bs % 4 == 0))
    p.flags |= sl::F_C_VEC;
  p.splits = 1;
  p.split_tiles = 0;
  if (bf16) p.flags |= sl::F_BF16;
  p.group_m = std::max(1, env_int("SL_GROUP_M", 8));

  int32_t tile = env_int("SL_TILE", -1);
  if (nvfp4) {
    // packed along K: each row of a K-tile is 32 bytes at a 16-byte aligned
    // address; K a multiple of 32 so every 16-byte piece is whole
    auto packed_ok = [&](const View& X) {
      return X.cs == 1 && X.rs % 32 == 0 && (uintptr_t)X.t->data % 16 == 0 &&
             (X.t->layout.rank == 2 || X.bs % 32 == 0);
    };
    if (!packed_ok(A) || !packed_ok(B) || K % 32 != 0)
      return fail(SL_ERR_LAYOUT,
                  "NVFP4 operands must be K-contiguous (packed) with rows a multiple of 32 elements apart, "
                  "16-byte aligned, and K %% 32 == 0");
    if (!tile_span_ok(A, A.rs / 2, K / 2) || !tile_span_ok(B, B.rs / 2, K / 2) || !scale_span_ok(SA) ||
        !scale_span_ok(SB))
      return fail(SL_ERR_SHAPE, "a 256-row tile of an operand spans 2^31 bytes or more");
    p.sfa = (const uint8_t*)args->sfa.data;
    p.sfb = (const uint8_t*)args->sfb.data;
    p.sa_rs = SA.rs, p.sa_ks = SA.cs, p.sa_bs = SA.t->layout.rank == 3 ? SA.bs : 0;
    p.sb_rs = SB.rs, p.sb_ks = SB.cs, p.sb_bs = SB.t->layout.rank == 3 ? SB.bs : 0;
    // one 8-byte load for a row's scales of two K-tiles when the scale rows
    // are K-contiguous on 8-byte boundaries
    auto pair_rows = [&](const View& S) {
      return S.cs == 1 && S.rs % 8 == 0 && (uintptr_t)S.t->data % 8 == 0 &&
             (S.t->layout.rank == 2 || S.bs % 8 == 0);
    };
    const bool pairs = pair_rows(SA) && pair_rows(SB) && env_int("SL_NV_PAIRS", 1);
    // Products of 2048^3 and more: both operands decoded to fp16 rows in the
    // caller's workspace by a first kernel, then the fp16 4-wave ring kernel
    // on them (the fused 8-wave kernel below decodes in its loader and runs
    // at the 8-wave kernel's pace; 8192^3 took 1006 us fused against 755
    // decoded ahead).  SL_NV_DECODE=0 / 1 forbids / forces it; an SL_TILE
    // choice keeps the fused kernels; sl_gemm_no_alloc never decodes ahead.
    const int32_t dec_env = env_int("SL_NV_DECODE", -1);
    const bool dec_ok = allow_decode && K > 0 && K % 64 == 0 && (int64_t)256 * K * 2 < ((int64_t)1 << 31);
    const bool dec = dec_ok && (dec_env == 1 || (dec_env < 0 && tile < 0 &&
                                                 (double)batch * (double)M * (double)N * (double)K >= 0x1p33));
    if (dec) {
      auto dec_of = [&](const View& X, const View& S, int64_t rows) {
        sl::Nvfp4Decode d{};
        d.x = (const uint8_t*)X.t->data;
        d.s = (const uint8_t*)S.t->data;
        d.rows = rows, d.K = K, d.rs = X.rs, d.bs = X.t->layout.rank == 3 ? X.bs : 0;
        d.srs = S.rs, d.sks = S.cs, d.sbs = S.t->layout.rank == 3 ? S.bs : 0;
        d.batch = (int32_t)batch;
        return d;
      };
      P.nv_dec = true;
      P.dec[0] = dec_of(A, SA, M);
      P.dec[1] = dec_of(B, SB, N);
      P.dec_off_b = ((size_t)batch * (size_t)M * (size_t)K * 2 + 255) & ~(size_t)255;
      P.dec_bytes = P.dec_off_b + (size_t)batch * (size_t)N * (size_t)K * 2;
      // the fp16 product over the decoded rows (pointers set at launch)
      p.sfa = p.sfb = nullptr;
      p.a_rs = K, p.a_ks = 1, p.a_bs = M * K;
      p.b_rs = K, p.b_ks = 1, p.b_bs = N * K;
      tile = sl::T256x256_W4R;
      P.pub.kernel = sl::K_NVFP4;
      P.pub.a_load = P.pub.b_load = sl::LOAD_KVEC;
      P.pub.tile_k = 64;
      p.k_tiles = (int32_t)(K / 64);
    } else {
      // the 8-wave kernel; the 4-wave ring schedule (tile 19, K > 0) only when
      // asked for: with one wave per SIMD the decode between the MFMAs made
      // it 25% slower on 8192^3
      tile = K > 0 && tile == sl::T256x256_W4R ? sl::T256x256_W4R : sl::T256x256_W2x4;
      P.pub.kernel = sl::K_NVFP4;
      P.pub.a_load = P.pub.b_load = pairs ? sl::LOAD_NVFP4_PAIRS : sl::LOAD_NVFP4;
      P.pub.tile_k = 64;
      p.k_tiles = (int32_t)((K + 63) / 64);
    }
  } else if (mxfp6) {
    // packed 6-bit rows in the 8-wave scaled-MFMA kernel: K-contiguous rows
    // a multiple of 64 elements (48 bytes) apart on 16-byte boundaries, so
    // every row and K-tile (128 values, 96 bytes) starts on a 16-byte chunk;
    // 16-byte scale chunks as for MXFP4: K a multiple of 512
    auto packed_ok = [&](const View& X) {
      return X.cs == 1 && X.rs % 64 == 0 && (uintptr_t)X.t->data % 16 == 0 &&
             (X.t->layout.rank == 2 || X.bs % 64 == 0);
    };
    auto chunk_rows = [&](const View& S) {
      return S.cs == 1 && S.rs % 16 == 0 && (uintptr_t)S.t->data % 16 == 0 &&
             (S.t->layout.rank == 2 || S.bs % 16 == 0);
    };
    if (!packed_ok(A) || !packed_ok(B) || K % 512 != 0 || !chunk_rows(SA) || !chunk_rows(SB))
      return fail(SL_ERR_LAYOUT,
                  "MXFP6 operands must be K-contiguous (packed) with rows a multiple of 64 elements apart, "
                  "16-byte aligned, K %% 512 == 0, and scale rows K-contiguous, 16-byte aligned");
    if (!tile_span_ok(A, A.rs / 4 * 3, K / 4 * 3) || !tile_span_ok(B, B.rs / 4 * 3, K / 4 * 3) ||
        !scale_span_ok(SA) || !scale_span_ok(SB))
      return fail(SL_ERR_SHAPE, "a 256-row tile of an operand spans 2^31 bytes or more");
    p.sfa = (const uint8_t*)args->sfa.data;
    p.sfb = (const uint8_t*)args->sfb.data;
    p.sa_rs = SA.rs, p.sa_ks = SA.cs, p.sa_bs = SA.t->layout.rank == 3 ? SA.bs : 0;
    p.sb_rs = SB.rs, p.sb_ks = SB.cs, p.sb_bs = SB.t->layout.rank == 3 ? SB.bs : 0;
    p.flags |= (args->a.dtype == SL_F6_E2M3 ? sl::F_FP6 : sl::F_FP6_E3M2) | sl::F_SCALE16;
    // the 4-wave ring kernel unless K = 0 (or the 8-wave tile is asked for)
    tile = K > 0 && tile != sl::T256x256_W2x4 ? sl::T256x256_W4R : sl::T256x256_W2x4;
    P.pub.kernel = sl::K_MXFP6;
    P.pub.a_load = P.pub.b_load = sl::LOAD_KVEC;
    P.pub.tile_k = 128;
    p.k_tiles = (int32_t)(K / 128);
  } else if (mxfp4) {
    // packed E2M1 in the 8-wave scaled-MFMA kernel: the NVFP4 packing rules,
    // and 16-byte scale chunks (rows of a multiple of 16 blocks, 16-byte
    // aligned): K a multiple of 512
    auto packed_ok = [&](const View& X) {
      return X.cs == 1 && X.rs % 32 == 0 && (uintptr_t)X.t->data % 16 == 0 &&
             (X.t->layout.rank == 2 || X.bs % 32 == 0);
    };
    auto chunk_rows = [&](const View& S) {
      return S.cs == 1 && S.rs % 16 == 0 && (uintptr_t)S.t->data % 16 == 0 &&
             (S.t->layout.rank == 2 || S.bs % 16 == 0);
    };
    if (!packed_ok(A) || !packed_ok(B) || K % 512 != 0 || !chunk_rows(SA) || !chunk_rows(SB))
      return fail(SL_ERR_LAYOUT,
                  "MXFP4 operands must be K-contiguous (packed) with rows a multiple of 32 elements apart, "
                  "16-byte aligned, K %% 512 == 0, and scale rows K-contiguous, 16-byte aligned");
    if (!tile_span_ok(A, A.rs / 2, K / 2) || !tile_span_ok(B, B.rs / 2, K / 2) || !scale_span_ok(SA) ||
        !scale_span_ok(SB))
      return fail(SL_ERR_SHAPE, "a 256-row tile of an operand spans 2^31 bytes or more");
    p.sfa = (const uint8_t*)args->sfa.data;
    p.sfb = (const uint8_t*)args->sfb.data;
    p.sa_rs = SA.rs, p.sa_ks = SA.cs, p.sa_bs = SA.t->layout.rank == 3 ? SA.bs : 0;
    p.sb_rs = SB.rs, p.sb_ks = SB.cs, p.sb_bs = SB.t->layout.rank == 3 ? SB.bs : 0;
    p.flags |= sl::F_FP4 | sl::F_SCALE16;
    // the 4-wave ring kernel unless K = 0 (or the 8-wave tile is asked for)
    tile = K > 0 && tile != sl::T256x256_W2x4 ? sl::T256x256_W4R : sl::T256x256_W2x4;
    P.pub.kernel = sl::K_MXFP4;
    P.pub.a_load = P.pub.b_load = sl::LOAD_KVEC;
    P.pub.tile_k = 256;
    p.k_tiles = (int32_t)(K / 256);
  } else if (mx) {
    p.sfa = (const uint8_t*)args->sfa.data;
    p.sfb = (const uint8_t*)args->sfb.data;
    p.sa_rs = SA.rs, p.sa_ks = SA.cs, p.sa_bs = SA.t->layout.rank == 3 ? SA.bs : 0;
    p.sb_rs = SB.rs, p.sb_ks = SB.cs, p.sb_bs = SB.t->layout.rank == 3 ? SB.bs : 0;
    const int32_t la = choose_load(A, K, 256, 1), lb = choose_load(B, K, 256, 1);
    if (la != sl::LOAD_KVEC || lb != sl::LOAD_KVEC)
      return fail(SL_ERR_LAYOUT,
                  "MXFP8 operands must be K-contiguous with 16-byte aligned rows and K %% 16 == 0");
    if (!scale_span_ok(SA) || !scale_span_ok(SB))
      return fail(SL_ERR_SHAPE, "a 256-row tile of a scale tensor spans 2^31 bytes or more");
    // The 8-wave kernel copies one dword of scales per row and K-tile: the
    // scale rows must be K-contiguous, 4-byte aligned, and hold a multiple
    // of four blocks.
    auto dword_rows = [&](const View& S) {
      return S.cs == 1 && S.rs % 4 == 0 && (uintptr_t)S.t->data % 4 == 0 &&
             (S.t->layout.rank == 2 || S.bs % 4 == 0);
    };
    const bool wide_ok = kb % 4 == 0 && dword_rows(SA) && dword_rows(SB);
    auto chunk_rows = [&](const View& S) {
      return S.cs == 1 && S.rs % 16 == 0 && (uintptr_t)S.t->data % 16 == 0 &&
             (S.t->layout.rank == 2 || S.bs % 16 == 0);
    };
    if (kb % 16 == 0 && chunk_rows(SA) && chunk_rows(SB) && env_int("SL_SCALE16", 1)) p.flags |= sl::F_SCALE16;
    // the 4-wave ring kernel: 16-byte scale chunks and at least one K-tile
    const bool ring_ok = (p.flags & sl::F_SCALE16) && K > 0;
    const bool valid = tile == sl::T256x256_W2x4  ? wide_ok
                       : tile == sl::T256x256_W4R ? ring_ok
                                                  : tile >= 0 && tile <= sl::T128x128_W2x2;
    if (!valid) {
      tile = sl::T256x128_W2x2;
      double best = 1e300;
      for (int t : {sl::T256x256_W2x4, sl::T256x128_W2x2, sl::T128x256_W2x2, sl::T128x128_W2x2}) {
        if (t == sl::T256x256_W2x4 && !wide_ok) continue;
        const double c = tile_cost(sl::kTiles[t], batch, M, N, K);
        if (c < best) best = c, tile = t;
      }
      if (tile == sl::T256x256_W2x4 && ring_ok) tile = sl::T256x256_W4R;
    }
    P.pub.kernel = tile == sl::T256x256_W4R   ? sl::K_MX_W4R
                   : tile == sl::T256x256_W2x4 ? sl::K_MX_W8
                                               : sl::K_MX;
    P.pub.a_load = P.pub.b_load = sl::LOAD_KVEC;
    P.pub.tile_k = 128;
    p.k_tiles = (int32_t)((K + 127) / 128);
  } else {
    int32_t la = choose_load(A, K, 256, 2), lb = choose_load(B, K, 256, 2);
    const bool generic = la == sl::LOAD_GENERIC || lb == sl::LOAD_GENERIC;
    if (generic) {
      // one 128x128 configuration, instantiated for every pair that has a
      // generic side: (G,G) (G,K) (K,G) (G,MN) (MN,G)
      tile = sl::T128x128_W2x2;
      P.pub.kernel = sl::K_F16_GENERIC;
    } else {
      // the multi-stage, ping-pong, streaming and split-K variants exist
      // for K-contiguous operands only; the 8-wave 256x256 kernel also for
      // M- (N-) contiguous ones, and among the automatic choices it
      // replaces the 4-wave 256x256 one
      const bool kk = la == sl::LOAD_KVEC && lb == sl::LOAD_KVEC;
      // Split-K for outputs that leave most of the chip idle even in
      // 128x128 tiles (a skinny N, a small M x N with a long K): up to 8
      // K-splits, each at least 4 K-tiles of 64, towards 256 workgroups.
      const int64_t T_all = (K + 63) / 64;
      const int64_t t128 = batch * ((M + 127) / 128) * ((N + 127) / 128);
      const int64_t auto_splits =
          std::max<int64_t>(1, std::min<int64_t>({8, 256 / std::max<int64_t>(1, t128), T_all / 4}));
      if (kk && tile < 0 && t128 < 128 && auto_splits >= 2) tile = sl::T128x128_SPLITK;
      const bool split_tile = tile == sl::T128x128_SPLITK || tile == sl::T256x128_SPLITK;
      if (split_tile && kk) {
        const sl::TileShape& st = sl::kTiles[tile];
        const int64_t tt = batch * ((M + st.bm - 1) / st.bm) * ((N + st.bn - 1) / st.bn);
        const int64_t tile_splits =
            std::max<int64_t>(1, std::min<int64_t>({8, 256 / std::max<int64_t>(1, tt), T_all / 4}));
        int64_t splits = env_int("SL_SPLITK", 0) > 0 ? env_int("SL_SPLITK", 0) : tile_splits;
        splits = std::max<int64_t>(1, std::min<int64_t>(splits, std::max<int64_t>(T_all, 1)));
        const int64_t per = (std::max<int64_t>(T_all, 1) + splits - 1) / splits;
        p.split_tiles = (int32_t)per;
        p.splits = (int32_t)((std::max<int64_t>(T_all, 1) + per - 1) / per);
      }
      // the ping-pong variants (tiles 9-14) are fp16 only
      const bool pingpong = tile >= sl::T256x256_PP && tile <= sl::T256x256_PPG;
      // the 4-wave ring kernels need at least one K-tile and K- or M/N-
      // contiguous vector operands (the 256x192 one K-contiguous ones).
      // With M/N-contiguous operands the 8-wave kernel is the automatic
      // choice: on the batched 64 x 512^3 shapes the ring kernel's
      // transposing fragment reads made it 20-50% slower.
      const bool vec = (la == sl::LOAD_KVEC || la == sl::LOAD_MNVEC) && (lb == sl::LOAD_KVEC || lb == sl::LOAD_MNVEC);
      const bool ring_ok = vec && K > 0;
      const bool ring = tile == sl::T256x256_W4R || tile == sl::T256x192_W4R;
      if (tile < 0 || tile >= sl::T_COUNT || (!kk && tile > sl::T256x256_W2x4_P && !ring) ||
          (bf16 && pingpong) || (ring && !ring_ok) || (tile == sl::T256x192_W4R && !kk)) {
        const int32_t big = ring_ok && kk ? sl::T256x256_W4R : sl::T256x256_W2x4;
        const int32_t wide = kk && K > 0 ? sl::T256x192_W4R : sl::T256x192_W2x4;
        tile = big;
        double best = 1e300;
        for (int t : {big, wide, (int32_t)sl::T256x128_W2x2, (int32_t)sl::T128x256_W2x2,
                      (int32_t)sl::T128x128_W2x2, (int32_t)sl::T32x128_STREAM}) {
          if ((t == sl::T32x128_STREAM || t == wide) && !kk) continue;
          const double c = tile_cost(sl::kTiles[t], batch, M, N, K);
          if (c < best) best = c, tile = t;
        }
      }
      P.pub.kernel = sl::K_F16;
    }
    // M- (N-) contiguous operands of the 256x256 ring kernel and of the
    // 8-wave 256x256 kernel are copied straight into an M-major LDS tile
    // (SL_MN_LOADER=1 keeps the register-transposing loader on the latter)
    if (tile == sl::T256x256_W4R || (tile == sl::T256x256_W2x4 && env_int("SL_MN_LOADER", 3) == 3)) {
      if (la == sl::LOAD_MNVEC) la = sl::LOAD_MNDMA;
      if (lb == sl::LOAD_MNVEC) lb = sl::LOAD_MNDMA;
    }
    P.pub.a_load = la;
    P.pub.b_load = lb;
    P.pub.tile_k = sl::kTiles[tile].bk;
    p.k_tiles = (int32_t)((K + P.pub.tile_k - 1) / P.pub.tile_k);
  }
  const sl::TileShape& ts = sl::kTiles[tile];
  P.tile = tile;
  p.tiles_m = (int32_t)((M + ts.bm - 1) / ts.bm);
  p.tiles_n = (int32_t)((N + ts.bn - 1) / ts.bn);
  const int64_t total = batch * p.tiles_m * p.tiles_n * p.splits;
  if (total >= lim) return fail(SL_ERR_SHAPE, "too many output tiles (%lld)", (long long)total);
  P.pub.tile_m = ts.bm;
  P.pub.tile_n = ts.bn;
  P.pub.threads = ts.wm * ts.wn * 64;
  P.pub.split_k = p.splits;
  P.pub.workgroups = total;
  P.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)batch * (size_t)M * (size_t)N * sizeof(float) : P.dec_bytes;
  P.pub.workspace_bytes = (int64_t)P.ws_bytes;
  P.pub.lds_bytes = ts.stages * (ts.bm + ts.bn) * P.pub.tile_k * (mx && !nvfp4 ? 1 : 2);
  if (P.pub.kernel == sl::K_MXFP4 || P.pub.kernel == sl::K_MXFP6)
    P.pub.lds_bytes = ts.stages * (ts.bm + ts.bn) * 128 + 2 * (ts.bm + ts.bn) * 16;
  if (P.pub.kernel == sl::K_MX_W8)
    P.pub.lds_bytes += (p.flags & sl::F_SCALE16) ? 2 * (ts.bm + ts.bn) * 16 : ts.stages * (ts.bm + ts.bn) * 4;
  if (tile == sl::T256x256_W4R || tile == sl::T256x192_W4R)
    P.pub.lds_bytes = nvfp4 && !P.nv_dec ? 2 * 512 * 128   // two fp16 stages (the packed data waits in registers)
                                         : 5 * 256 * 128;  // five 32 KiB operand K-tile slots
  return SL_OK;
}

// The caller's workspace (split-K partial sums, or NVFP4 operands decoded
// to fp16): present, large enough, 16-byte aligned (it is written 16 bytes
// at a time) and apart from every operand (it is read while D is written).
sl_status check_workspace(const sl_gemm_args* args, const Plan& P) {
  if (!P.ws_bytes) return SL_OK;
  if (!args->workspace)
    return fail(SL_ERR_NULL, "the plan needs a workspace of %zu bytes (%s); workspace is NULL", P.ws_bytes,
                P.nv_dec ? "NVFP4 operands decoded to fp16" : "split-K partial sums");
  if (args->workspace_bytes < 0 || (uint64_t)args->workspace_bytes < (uint64_t)P.ws_bytes)
    return fail(SL_ERR_SHAPE, "workspace of %lld bytes, the plan needs %zu", (long long)args->workspace_bytes,
                P.ws_bytes);
  const uintptr_t lo = (uintptr_t)args->workspace, hi = lo + P.ws_bytes;
  if (lo % 16 != 0) return fail(SL_ERR_ALIGN, "workspace is not on a 16-byte boundary");
  for (int32_t i = 0; i < P.nranges; ++i)
    if (P.lo[i] < hi && lo < P.hi[i]) return fail(SL_ERR_ALIAS, "workspace overlaps an operand");
  return SL_OK;
}

// gfx950 check, cached per device
sl_status check_arch() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SL_ERR_LAUNCH, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SL_ERR_ARCH, "device index %d out of range", dev);
  std::lock_guard<std::mutex> g(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(SL_ERR_LAUNCH, "hipGetDeviceProperties failed");
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (known[dev] < 0) return fail(SL_ERR_ARCH, "device %d is not gfx950", dev);
  return SL_OK;
}

// Copies `text` into the caller's buffer; *needed gets its size with the
// terminating NUL.  A buffer too small for it returns SL_ERR_SHAPE.
sl_status emit_text(const std::string& text, char* out, int64_t capacity, int64_t* needed) {
  const int64_t n = (int64_t)text.size() + 1;
  if (needed) *needed = n;
  if (!out) return fail(SL_ERR_NULL, "out is NULL");
  if (capacity < n) {
    if (capacity > 0) out[0] = '\0';
    return fail(SL_ERR_SHAPE, "output buffer of %lld bytes, %lld needed", (long long)capacity, (long long)n);
  }
  memcpy(out, text.c_str(), (size_t)n);
  return SL_OK;
}

// "layout" text, or a shape tuple alone (strides 0)
sl::la::Layout parse_any(const char* text) {
  const std::string t(text);
  return t.find(':') == std::string::npos ? sl::la::parse_shape(t) : sl::la::parse(t);
}

// an order tuple "(_2048,(144,288))" (or a layout, whose strides are the
// order values) as a layout whose strides carry the values
sl::la::Layout parse_order(const char* text) {
  const std::string t(text);
  if (t.find(':') != std::string::npos) return sl::la::parse(t);
  std::function<sl::la::Layout(const sl::la::Layout&)> mv = [&](const sl::la::Layout& l) {
    if (l.leaf) {
      sl::la::Layout m = sl::la::Layout::mode(1, l.shape);
      m.stride_static = l.shape_static;
      return m;
    }
    std::vector<sl::la::Layout> k;
    for (const auto& x : l.kids) k.push_back(mv(x));
    return sl::la::Layout::tuple(std::move(k));
  };
  return mv(sl::la::parse_shape(t));
}

int64_t parse_int(const char* text) {
  char* end = nullptr;
  const long long v = strtoll(text, &end, 10);
  if (end == text || *end != '\0') throw sl::la::Error{std::string("expected an integer, got \"") + text + "\""};
  return v;
}

// The plan's kernels on `stream`; a split-K plan's partial sums, or the
// decoded NVFP4 operands, go to `ws`.
sl_status launch_plan(Plan& P, void* ws, hipStream_t st) {
  hipError_t e;
  if (P.nv_dec) {
    sl::Nvfp4Decode da = P.dec[0], db = P.dec[1];
    da.out = (uint16_t*)ws;
    db.out = (uint16_t*)((char*)ws + P.dec_off_b);
    P.p.a = da.out;
    P.p.b = db.out;
    e = sl::launch_nvfp4_decode(da, st);
    if (e == hipSuccess) e = sl::launch_nvfp4_decode(db, st);
    if (e == hipSuccess) e = sl::launch_gemm_f16(P.p, P.tile, P.pub.a_load, P.pub.b_load, st);
  } else if (P.pub.kernel == sl::K_NVFP4) {
    e = sl::launch_gemm_f16(P.p, P.tile, P.pub.a_load, P.pub.b_load, st);
  } else if (P.mx) {
    e = sl::launch_gemm_mx(P.p, P.tile, st);
  } else if (P.ws_bytes) {
    P.p.ws = (float*)ws;
    e = sl::launch_gemm_f16(P.p, P.tile, P.pub.a_load, P.pub.b_load, st);
    if (e == hipSuccess) e = sl::launch_splitk_reduce(P.p, st);
  } else {
    e = sl::launch_gemm_f16(P.p, P.tile, P.pub.a_load, P.pub.b_load, st);
  }
  if (e != hipSuccess) return fail(SL_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SL_OK;
}

}  // namespace

extern "C" {

int32_t sl_abi_version(void) { return SL_ABI_VERSION; }

const char* sl_last_error_message(void) { return g_msg.c_str(); }

const char* sl_status_string(int32_t s) {
  switch (s) {
    case SL_OK: return "ok";
    case SL_ERR_NULL: return "null pointer";
    case SL_ERR_DTYPE: return "unsupported dtype";
    case SL_ERR_SHAPE: return "shape mismatch or size limit";
    case SL_ERR_LAYOUT: return "unsupported layout";
    case SL_ERR_ALIGN: return "misaligned pointer";
    case SL_ERR_ALIAS: return "output overlaps an input";
    case SL_ERR_ARCH: return "device is not gfx950";
    case SL_ERR_LAUNCH: return "HIP launch error";
    case SL_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

sl_status sl_gemm_plan(const sl_gemm_args* args, sl_plan* plan) {
  Plan P;
  const sl_status s = plan_gemm(args, &P);
  if (s != SL_OK) return s;
  if (plan) *plan = P.pub;
  return SL_OK;
}

sl_status sl_gemm_workspace_bytes(const sl_gemm_args* args, int64_t* bytes) {
  if (!bytes) return fail(SL_ERR_NULL, "bytes is NULL");
  Plan P;
  const sl_status s = plan_gemm(args, &P);
  if (s != SL_OK) return s;
  *bytes = P.empty ? 0 : (int64_t)P.ws_bytes;
  return SL_OK;
}

sl_status sl_gemm(const sl_gemm_args* args, void* stream) {
  Plan P;
  sl_status s = plan_gemm(args, &P);
  if (s != SL_OK) return s;
  if (P.empty) return SL_OK;
  if ((s = check_workspace(args, P)) != SL_OK) return s;
  if ((s = check_arch()) != SL_OK) return s;
  return launch_plan(P, args->workspace, (hipStream_t)stream);
}

static_assert(sl::kScratchBytes == (size_t)SL_NO_ALLOC_SCRATCH_BYTES, "one scratch size");

sl_status sl_gemm_no_alloc(const sl_gemm_args* args, void* stream) {
  Plan P;
  sl_status s = plan_gemm(args, &P, false);  // NVFP4: the fused kernels, no decoded copies
  if (s != SL_OK) return s;
  if (P.empty) return SL_OK;
  if (P.ws_bytes > sl::kScratchBytes)
    return fail(SL_ERR_SHAPE, "the plan splits K %d ways into %zu bytes of partial sums; the static scratch holds %zu",
                P.pub.split_k, P.ws_bytes, sl::kScratchBytes);
  if ((s = check_arch()) != SL_OK) return s;
  void* ws = nullptr;
  if (P.ws_bytes) {
    const hipError_t e = sl::scratch_address(&ws);
    if (e != hipSuccess) return fail(SL_ERR_LAUNCH, "scratch address: %s", hipGetErrorString(e));
  }
  return launch_plan(P, ws, (hipStream_t)stream);
}

sl_status sl_query_fragment_map(int32_t instr, int32_t operand, int32_t* lane, int32_t* slot, int32_t* row,
                                int32_t* col, int64_t capacity, int64_t* count) {
  g_msg.clear();
  if (instr < 0 || instr > 7) return fail(SL_ERR_ARG, "instr %d", instr);
  if (operand < 0 || operand > 3) return fail(SL_ERR_ARG, "operand %d", operand);
  if ((operand == sl::OP_SCALE) && instr < 2) return fail(SL_ERR_ARG, "instr %d has no scale operand", instr);
  const int32_t slots = operand == sl::OP_D ? sl::instr_acc_regs(instr) : operand == sl::OP_SCALE ? 1
                                                                                                  : sl::instr_in_slots(instr);
  int64_t n = 0;
  for (int32_t l = 0; l < 64; ++l)
    for (int32_t v = 0; v < slots; ++v, ++n) {
      if (n >= capacity) continue;
      sl::Coord c = operand == sl::OP_D       ? sl::acc_map(instr, l, v)
                    : operand == sl::OP_SCALE ? sl::scale_map(instr, l)
                                              : sl::operand_map(instr, l, v);
      if (lane) lane[n] = l;
      if (slot) slot[n] = v;
      if (row) row[n] = c.row;
      if (col) col[n] = c.col;
    }
  if (count) *count = n;
  return SL_OK;
}

// query id of the M-major LDS tile (LOAD_MNDMA operands), next to the
// kernel family ids
constexpr int32_t kMnTile = 5;

// the kernels are built with the row-shift 0 swizzle (swz)
static int32_t current_shift() { return 0; }

sl_status sl_query_lds_map(int32_t variant, int32_t operand, int64_t* offsets, int64_t capacity, int32_t* rows,
                           int32_t* cols, int32_t* elem_bytes) {
  g_msg.clear();
  if (variant < sl::K_F16 || variant > kMnTile) return fail(SL_ERR_ARG, "variant %d", variant);
  if (operand < 0 || operand > 1) return fail(SL_ERR_ARG, "operand %d", operand);
  if (variant == kMnTile) {
    int64_t n = 0;
    for (int32_t r = 0; r < 256; ++r)
      for (int32_t k = 0; k < 64; ++k, ++n)
        if (offsets && n < capacity) offsets[n] = sl::mn_lds_offset(k, r, 256);
    if (rows) *rows = 256;
    if (cols) *cols = 64;
    if (elem_bytes) *elem_bytes = 2;
    return SL_OK;
  }
  const int32_t R = variant == sl::K_F16_GENERIC ? 128 : 256;
  const int32_t es = variant >= sl::K_MX ? 1 : 2;
  const int32_t Cn = sl::kRowBytes / es;
  const int32_t sh = current_shift();
  int64_t n = 0;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t k = 0; k < Cn; ++k, ++n)
      if (offsets && n < capacity) offsets[n] = sl::lds_offset(r, k * es, sh);
  if (rows) *rows = R;
  if (cols) *cols = Cn;
  if (elem_bytes) *elem_bytes = es;
  return SL_OK;
}

sl_status sl_query_fragment_addresses(int32_t variant, int32_t operand, int64_t* addr, int64_t capacity,
                                      int64_t* count) {
  g_msg.clear();
  if (variant < sl::K_F16 || variant > kMnTile) return fail(SL_ERR_ARG, "variant %d", variant);
  if (operand < 0 || operand > 1) return fail(SL_ERR_ARG, "operand %d", operand);
  if (variant == kMnTile) {
    // the address each lane supplies to the two transposing reads
    int64_t n = 0;
    for (int32_t l = 0; l < 64; ++l)
      for (int32_t r = 0; r < 2; ++r, ++n)
        if (addr && n < capacity) addr[n] = sl::tr_read_offset(l, r, 0, 0, 256);
    if (count) *count = n;
    return SL_OK;
  }
  const int32_t instr = variant == sl::K_MX_W8 ? sl::MFMA32_F8 : variant == sl::K_MX ? sl::MFMA16_F8 : sl::MFMA16_F16;
  const int32_t slots = sl::instr_in_slots(instr);
  const int32_t es = variant >= sl::K_MX ? 1 : 2;
  const int32_t sh = current_shift();
  int64_t n = 0;
  for (int32_t l = 0; l < 64; ++l)
    for (int32_t v = 0; v < slots; ++v, ++n) {
      if (!addr || n >= capacity) continue;
      // the kernels read 16-byte pieces at fragment_lds_offset; slot v sits
      // (v % (16/es)) elements into piece v / (16/es)
      const int32_t per = 16 / es;
      addr[n] = sl::fragment_lds_offset(instr, l, v / per, 0, 0, sh) + (v % per) * es;
    }
  if (count) *count = n;
  return SL_OK;
}

sl_status sl_probe_mfma(int32_t instr, int32_t mode, float* out, int64_t capacity, int64_t* cases,
                        void* stream) {
  g_msg.clear();
  if (instr < 0 || instr > 3) return fail(SL_ERR_ARG, "instr %d", instr);
  const bool f8 = instr >= 2;
  if (mode < 0 || mode > (f8 ? 11 : 1)) return fail(SL_ERR_ARG, "mode %d", mode);
  const int64_t nc = 64 * (int64_t)sl::instr_in_slots(instr);
  const int64_t need = nc * 64 * sl::instr_acc_regs(instr);
  if (cases) *cases = nc;
  if (!out) return fail(SL_ERR_NULL, "out is NULL");
  if (capacity < need) return fail(SL_ERR_SHAPE, "out holds %lld floats, needs %lld", (long long)capacity,
                                   (long long)need);
  sl_status s = check_arch();
  if (s != SL_OK) return s;
  const hipError_t e = sl::launch_probe_mfma(instr, mode, out, nc, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SL_ERR_LAUNCH, "probe launch failed: %s", hipGetErrorString(e));
  return SL_OK;
}

sl_status sl_probe_lds(int32_t mode, const void* src, const int32_t* perm, void* out, void* stream) {
  g_msg.clear();
  if (mode < 0 || mode > 3) return fail(SL_ERR_ARG, "mode %d", mode);
  if (!src || !perm || !out) return fail(SL_ERR_NULL, "src, perm and out are required");
  if ((uintptr_t)src % 16 || (uintptr_t)out % 16) return fail(SL_ERR_ALIGN, "src and out must be 16-byte aligned");
  sl_status s = check_arch();
  if (s != SL_OK) return s;
  const hipError_t e = sl::launch_probe_lds(mode, src, perm, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SL_ERR_LAUNCH, "probe launch failed: %s", hipGetErrorString(e));
  return SL_OK;
}

sl_status sl_layout_op(int32_t op, const char* a, const char* b, char* out, int64_t capacity, int64_t* needed) {
  g_msg.clear();
  namespace la = sl::la;
  if (!a) return fail(SL_ERR_NULL, "a is NULL");
  const bool mark = (op & SL_LA_MARK_STATIC) != 0;
  op &= ~SL_LA_MARK_STATIC;
  const bool binary = op == SL_LA_COMPOSITION || op == SL_LA_COMPLEMENT || op == SL_LA_ZIPPED_DIVIDE ||
                      op == SL_LA_MAKE_ORDERED || op == SL_LA_LOGICAL_PRODUCT || op == SL_LA_TILED_PRODUCT ||
                      op == SL_LA_EVAL;
  if (binary && !b) return fail(SL_ERR_NULL, "b is NULL");
  std::string r;
  try {
    switch (op) {
      case SL_LA_PARSE: r = la::to_string(parse_any(a), mark); break;
      case SL_LA_COALESCE: r = la::to_string(la::coalesce(la::parse(a)), mark); break;
      case SL_LA_COMPOSITION: r = la::to_string(la::composition(la::parse(a), la::parse(b)), mark); break;
      case SL_LA_COMPLEMENT: r = la::to_string(la::complement(la::parse(a), parse_int(b)), mark); break;
      case SL_LA_RIGHT_INVERSE: r = la::to_string(la::right_inverse(la::parse(a)), mark); break;
      case SL_LA_ZIPPED_DIVIDE: r = la::to_string(la::zipped_divide(la::parse(a), la::parse(b)), mark); break;
      case SL_LA_FILTER_ZEROS: r = la::to_string(la::filter_zeros(la::parse(a)), mark); break;
      case SL_LA_COMPACT_LEFT: r = la::to_string(la::compact_left(parse_any(a)), mark); break;
      case SL_LA_MAKE_ORDERED: r = la::to_string(la::make_ordered(parse_any(a), parse_order(b)), mark); break;
      case SL_LA_LOGICAL_PRODUCT: r = la::to_string(la::logical_product(la::parse(a), la::parse(b)), mark); break;
      case SL_LA_TILED_PRODUCT: r = la::to_string(la::tiled_product(la::parse(a), la::parse(b)), mark); break;
      case SL_LA_FRAGMENT_LIKE: r = la::to_string(la::fragment_like(la::parse(a)), mark); break;
      case SL_LA_TENSOR_LIKE: r = la::to_string(la::tensor_like(la::parse(a)), mark); break;
      case SL_LA_EVAL: {
        const int64_t i = parse_int(b);
        const la::Layout l = la::parse(a);
        if (i < 0 || i >= la::size(l)) return fail(SL_ERR_SHAPE, "index %lld outside [0, %lld)", (long long)i, (long long)la::size(l));
        r = std::to_string(la::eval(l, i));
        break;
      }
      case SL_LA_SIZE: r = std::to_string(la::size(parse_any(a))); break;
      case SL_LA_COSIZE: r = std::to_string(la::cosize(la::parse(a))); break;
      default: return fail(SL_ERR_ARG, "unknown layout op %d", op);
    }
  } catch (const la::Error& e) {
    return fail(SL_ERR_LAYOUT, "%s", e.what.c_str());
  } catch (const std::exception& e) {
    return fail(SL_ERR_LAYOUT, "%s", e.what());
  }
  return emit_text(r, out, capacity, needed);
}

sl_status sl_describe_plan(const sl_gemm_args* args, char* out, int64_t capacity, int64_t* needed) {
  Plan P;
  const sl_status s = plan_gemm(args, &P);
  if (s != SL_OK) return s;
  if (P.empty) return emit_text("# empty product: nothing is launched\n", out, capacity, needed);
  const sl::TileShape& ts = sl::kTiles[P.tile];
  const sl::GemmParams& p = P.p;
  sl::DescribeInput in{};
  in.kernel = P.pub.kernel;
  in.a_load = P.pub.a_load;
  in.b_load = P.pub.b_load;
  in.bm = ts.bm, in.bn = ts.bn, in.bk = P.pub.tile_k;
  in.wm = ts.wm, in.wn = ts.wn, in.stages = ts.stages;
  in.ring = P.tile == sl::T256x256_W4R || P.tile == sl::T256x192_W4R;
  in.nv_decoded = P.nv_dec;
  in.splits = p.splits, in.split_tiles = p.split_tiles, in.group_m = p.group_m;
  in.tiles_m = p.tiles_m, in.tiles_n = p.tiles_n;
  in.workgroups = P.pub.workgroups, in.batch = P.pub.batch, in.M = p.M, in.N = p.N, in.K = p.K;
  in.a_bs = p.a_bs, in.a_rs = p.a_rs, in.a_cs = p.a_ks;
  in.b_bs = p.b_bs, in.b_rs = p.b_rs, in.b_cs = p.b_ks;
  in.c_bs = p.c_bs, in.c_rs = p.c_rs, in.c_cs = p.c_cs;
  in.d_bs = p.d_bs, in.d_rs = p.d_rs, in.d_cs = p.d_cs;
  in.sa_rs = p.sa_rs, in.sa_cs = p.sa_ks, in.sb_rs = p.sb_rs, in.sb_cs = p.sb_ks;
  in.a_batched = args->a.layout.rank == 3, in.b_batched = args->b.layout.rank == 3;
  in.c_batched = args->c.layout.rank == 3, in.d_batched = args->d.layout.rank == 3;
  in.has_c = (p.flags & sl::F_HAS_C) != 0;
  in.flags = p.flags;
  in.block_k = args->block_k;
  in.lds_bytes = P.pub.lds_bytes;
  std::string text;
  try {
    text = sl::describe_plan(in);
  } catch (const std::exception& e) {
    return fail(SL_ERR_LAYOUT, "%s", e.what());
  }
  return emit_text(text, out, capacity, needed);
}

}  // extern "C"
