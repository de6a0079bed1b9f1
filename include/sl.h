/*
 * sl.h -- C ABI of libstride_layouts_lds.so, a strided-layout GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * The one operation:  D = A * B^T + C   (optionally block-scaled).
 *
 *  - "CuTe 中 A、B 如何加载到 MMA 寄存器", section 1: the matrix-core
 *    instruction computes D = A x B + C with A indexed (M,K) and B indexed
 *    (N,K); D may reuse C's storage.
 *  - "数据布局及其记号", section "Shape-Stride 模型": a tensor is flat storage
 *    plus a layout S[(shape):(strides)]; the element at index (i,j,...) is at
 *    the dot product of the index with the strides, counted in ELEMENTS (not
 *    bytes).  A transpose is a stride swap; no data moves.
 *  - same page, section "Replication 与 Offset": the block-scaled product
 *    A_real[m,k] = A_low[m,k] * SFA[m, k/K_blk], B_real[n,k] = B_low[n,k] *
 *    SFB[n, k/K_blk], D = C + A_real x B_real^T.  MXFP8: FP8 E4M3 data, one
 *    E8M0 scale per 32 consecutive K elements (K_blk = 32).
 *
 * Every operand is passed as a device pointer plus such a layout, so
 * row-major, column-major, transposed and batched strided views all go
 * through the one entry point sl_gemm().
 *
 * Conventions
 *  - All shapes and strides are int64 counts of ELEMENTS.  Strides must be
 *    >= 0.  A rank-2 layout is (rows, cols); a rank-3 layout is
 *    (batch, rows, cols).  A rank-2 input is the same matrix for every batch.
 *  - A: (batch?, M, K); B: (batch?, N, K); C and D: (batch?, M, N);
 *    SFA: (batch?, M, ceil(K/block_k)); SFB: (batch?, N, ceil(K/block_k)).
 *  - Batch counts of rank-3 operands must equal D's batch count; an input
 *    may broadcast along the batch with batch stride 0.  A zero stride
 *    inside the matrix dimensions of an input is also accepted (every index
 *    along it reads the same element).  D must not broadcast: its strides
 *    must map distinct (batch, m, n) to distinct addresses.
 *  - C may be absent (data == NULL: C = 0) or be exactly D (same pointer and
 *    same layout: the update is done in place).  Any other overlap of D's
 *    address range with A, B, C or the scales returns SL_ERR_ALIAS.
 *  - M == 0 or N == 0 (or batch == 0) is a no-op returning SL_OK.  K == 0
 *    gives D = C (or D = 0).
 *  - Ownership: the caller owns every buffer, the library allocates no
 *    device memory, and sl_gemm() keeps no pointer after it returns.  A
 *    plan with sl_plan.workspace_bytes > 0 (also given by
 *    sl_gemm_workspace_bytes()) needs that much workspace, which the
 *    caller passes in sl_gemm_args.workspace: device memory, 16-byte
 *    aligned, overlapping no operand, and not used by anything else until
 *    the call's kernels have finished on `stream`.  Two kinds of plan have
 *    one: a split-K plan (sl_plan.split_k > 1) keeps its fp32 partial sums
 *    there, and an NVFP4 plan that decodes its operands ahead (kernel 5
 *    with a_load 0) keeps A and B there as fp16 rows of K contiguous
 *    values (batch * M * K * 2 bytes of A, then B from the next 256-byte
 *    boundary: about (M + N) * K * 2 bytes per batch).  Other plans ignore
 *    the workspace fields.
 *  - Execution: validation runs on the host before any HIP call; a failure
 *    returns a negative sl_status and sets the thread-local message.  On
 *    success the kernel is launched asynchronously on `stream` (a
 *    hipStream_t; NULL is the default stream) and the call returns without
 *    waiting.  Errors reported by the launch return SL_ERR_LAUNCH.  A
 *    split-K plan launches two kernels (partial sums, then D = C + their
 *    sum) on the same stream.
 *  - Numerics: fp16 (bf16) products are accumulated in fp32; the result
 *    (plus C, added in fp32) is rounded to fp16 (bf16) to nearest-even,
 *    overflow to +-inf.  bf16 inputs take bf16 C and D.
 *    A split-K plan sums each K-split in fp32 and then adds the splits in
 *    fp32 (a different summation order, same precision).
 */
#ifndef STRIDE_LAYOUTS_LDS_SL_H
#define STRIDE_LAYOUTS_LDS_SL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SL_ABI_VERSION 2

typedef enum {
  SL_F16 = 1,     /* IEEE binary16 */
  SL_F32 = 2,     /* IEEE binary32 (accepted for nothing but reported) */
  SL_F8_E4M3 = 3, /* OCP MX E4M3 (bias 7, max 448, S.1111.111 = NaN) */
  SL_E8M0 = 4,    /* OCP MX E8M0 scale: 2^(b-127), 255 = NaN */
  SL_BF16 = 5,    /* bfloat16: binary32's sign and 8-bit exponent, 7 stored significand bits */
  SL_F4_E2M1 = 6, /* OCP MX E2M1 (bias 1, max 6), packed two per byte along the unit-stride
                     (K) axis: element offset o is byte o/2, low nibble for even o */
  SL_F6_E2M3 = 7, /* OCP MX FP6 E2M3 (bias 1, 3 significand bits, max 7.5), packed as one
                     little-endian bit stream along the unit-stride (K) axis: element offset
                     o occupies bits 6o .. 6o+5, bit 0 = least significant bit of byte 0 */
  SL_F6_E3M2 = 8  /* OCP MX FP6 E3M2 (bias 3, 2 significand bits, max 28), packed as E2M3 */
} sl_dtype;

typedef enum {
  SL_OK = 0,
  SL_ERR_NULL = -1,   /* required pointer is NULL */
  SL_ERR_DTYPE = -2,  /* unsupported dtype or dtype combination */
  SL_ERR_SHAPE = -3,  /* shapes disagree, negative sizes, or size limits */
  SL_ERR_LAYOUT = -4, /* rank, negative stride, or a broadcasting D */
  SL_ERR_ALIGN = -5,  /* a pointer not aligned to its element size */
  SL_ERR_ALIAS = -6,  /* D overlaps an input (other than C == D exactly) */
  SL_ERR_ARCH = -7,   /* the current device is not gfx950 */
  SL_ERR_LAUNCH = -8, /* the HIP runtime reported an error */
  SL_ERR_ARG = -9     /* an invalid enum or query argument */
} sl_status;

/* A shape:stride layout S[(shape):(stride)], counted in elements. */
typedef struct {
  int32_t rank;      /* 2: (rows, cols)   3: (batch, rows, cols) */
  int64_t shape[3];
  int64_t stride[3];
} sl_layout;

/* Device pointer + dtype + layout.  data == NULL marks an absent operand. */
typedef struct {
  void* data;
  int32_t dtype; /* sl_dtype */
  sl_layout layout;
} sl_tensor;

typedef struct {
  sl_tensor a;     /* (batch?, M, K)  f16, bf16, f8_e4m3 or f4_e2m1 (scaled) */
  sl_tensor b;     /* (batch?, N, K)  same dtype as a                      */
  sl_tensor c;     /* (batch?, M, N)  D's dtype; data == NULL means C = 0  */
  sl_tensor d;     /* (batch?, M, N)  bf16 for bf16 a/b, else f16 output  */
  sl_tensor sfa;   /* (batch?, M, ceil(K/block_k)) e8m0 (MXFP8) or f8_e4m3 (NVFP4) */
  sl_tensor sfb;   /* (batch?, N, ceil(K/block_k)) same dtype as sfa       */
  int32_t block_k; /* 32 for MXFP8, 16 for NVFP4; ignored for f16 / bf16   */
  void* workspace;          /* device memory for a plan's workspace: split-K
                               fp32 partial sums or decoded NVFP4 operands
                               (NULL when the plan needs none) */
  int64_t workspace_bytes;  /* its size in bytes */
} sl_gemm_args;

/* What sl_gemm would launch for these arguments (host only, no HIP call). */
typedef struct {
  int32_t kernel;     /* kernel family: 1 fp16/bf16 fast, 2 fp16/bf16 with an
                         element loader, 3 mxfp8 (4 waves, 16x16x128
                         instruction), 4 mxfp8 (8 waves, 32x32x64 instruction,
                         scales staged in LDS), 5 nvfp4 (decoded to fp16 in
                         the loader, fp16 instruction; from 2048^3 on, or
                         with SL_NV_DECODE=1, and K % 64 == 0: decoded
                         ahead into the workspace by a first kernel, then
                         the fp16 4-wave ring kernel, a_load 0), 6 mxfp4 and 7 mxfp6
                         (32x32x64 scaled instruction with E2M1 or 6-bit
                         data: 4 waves on an LDS ring, scales in registers;
                         8 waves when K == 0 or tile 4 is asked for),
                         8 mxfp8 (4 waves, 32x32x64 instruction,
                         LDS ring, scales in registers: scale rows of a
                         multiple of 16 blocks on 16-byte boundaries) */
  int32_t a_load;     /* 0 K-contiguous vector, 1 M-contiguous vector (register
                         transpose), 2 generic, 3 M-contiguous direct copy into
                         an M-major LDS tile read by transposing reads, 4 NVFP4
                         decoding loader, 5 the same fetching two K-tiles per
                         row at once (scale rows K-contiguous on 8-byte
                         boundaries) */
  int32_t b_load;     /* same, for B */
  int32_t tile_m, tile_n, tile_k;
  int32_t threads;    /* per workgroup */
  int32_t split_k;    /* K partitions (1: none); > 1 needs a workspace of
                         split_k * batch * m * n fp32 and adds a reduction
                         kernel */
  int64_t workgroups; /* total workgroups launched */
  int32_t lds_bytes;  /* LDS per workgroup */
  int64_t batch, m, n, k;
  int64_t workspace_bytes; /* bytes of workspace sl_gemm needs (0: none) */
} sl_plan;

/*
 * D = A * B^T + C over the strided descriptors above (f16 x f16 -> f16 or
 * bf16 x bf16 -> bf16, with fp32 accumulation), or the MXFP8 block-scaled
 * form when a and b are SL_F8_E4M3 and sfa/sfb are SL_E8M0 with
 * block_k == 32 (the matrix product of "CuTe 中 A、B 如何加载到 MMA 寄存器",
 * section 1, and the block-scaled product of "数据布局及其记号", section
 * "Replication 与 Offset"), or its NVFP4 form named on the same page: a and
 * b SL_F4_E2M1 (packed, K-contiguous, row strides multiples of 32, 16-byte
 * aligned, K % 32 == 0), sfa/sfb SL_F8_E4M3, block_k == 16, D f16.  bf16
 * is the same product in another 16-bit format; the pages name fp16 only.
 * MXFP4 (a, b SL_F4_E2M1 with SL_E8M0 scales, block_k 32) and MXFP6 (a, b
 * both SL_F6_E2M3 or both SL_F6_E3M2, SL_E8M0 scales, block_k 32) are the
 * block-scaled product with 4- and 6-bit data: packed K-contiguous rows on
 * 16-byte boundaries (row strides multiples of 32 (fp4) or 64 (fp6)
 * elements), K % 512 == 0, and scale rows K-contiguous on 16-byte
 * boundaries with row strides multiples of 16.
 * Sizes: M, N, K and the batch count below 2^31 (else SL_ERR_SHAPE).  An
 * operand may span any number of bytes; 256 of its rows (one tile) must
 * span fewer than 2^31 bytes for the vector loaders of 16-bit operands
 * (else the slower element loader runs), and for packed 4/6-bit data and
 * scale tensors (else SL_ERR_SHAPE).
 * A plan with a workspace reads args->workspace: NULL returns SL_ERR_NULL, fewer
 * than the plan's workspace bytes SL_ERR_SHAPE, an address not on a 16-byte
 * boundary SL_ERR_ALIGN, and a range overlapping an operand SL_ERR_ALIAS,
 * all before any HIP call.
 * `stream` is a hipStream_t.  Asynchronous; see Conventions.
 */
sl_status sl_gemm(const sl_gemm_args* args, void* stream);

/*
 * sl_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same validation, plans and kernels, but a split-K plan keeps its fp32
 * partial sums in a static device array of the library instead of the
 * caller's workspace (args->workspace and workspace_bytes are ignored), and
 * NVFP4 always runs the fused kernels (no decoded copies; its plan can
 * differ from sl_gemm_plan's, with the same result bit for bit).
 * The call allocates nothing.  The array holds SL_NO_ALLOC_SCRATCH_BYTES
 * bytes on each GPU the library runs on and is held until the process ends;
 * a plan needing more (sl_plan.workspace_bytes) returns SL_ERR_SHAPE before
 * any HIP call.  Every call on one GPU shares that GPU's array and finds
 * the previous call's contents there (every partial sum a plan reads is
 * written by the same call first, so nothing needs clearing); calls that
 * overlap in time on one GPU, e.g. on two streams, race on it.
 */
#define SL_NO_ALLOC_SCRATCH_BYTES (32LL << 20)
sl_status sl_gemm_no_alloc(const sl_gemm_args* args, void* stream);

/*
 * Planner overrides, read from the environment on every planning call (by
 * sl_gemm, sl_gemm_no_alloc, sl_gemm_plan and the calls built on it).  They
 * exist for measurement and tests; unset, the planner's own choices hold.
 * A value a shape cannot use is replaced by the planner's choice.
 *   SL_TILE=n       the library's tile configuration n, 0-20 (4: the 8-wave
 *                   256x256 kernel, 19: the 4-wave 256x256 ring kernel, 20:
 *                   the 256x192 ring kernel); the plan reports its tile_m/n/k
 *   SL_GROUP_M=n    output-tile rows per group in each XCD's tile order
 *                   (default 8, at least 1)
 *   SL_SPLITK=n     split count of the split-K tiles (default: from the grid)
 *   SL_SCALE16=0    MXFP8: no 16-byte scale chunks (so no 4-wave ring kernel)
 *   SL_NV_PAIRS=0   NVFP4: fetch one K-tile per load instead of two
 *   SL_MN_LOADER=1  8-wave 256x256 kernel: M/N-contiguous operands through
 *                   the register-transposing loader instead of direct copies
 *   SL_NV_DECODE=0  NVFP4: never decode ahead into the workspace (=1: always,
 *                   when K % 64 == 0; unset: from 2048^3 on, without SL_TILE)
 */

/* Validation and kernel selection only: fills *plan, launches nothing and
 * makes no HIP call.  Same status codes as sl_gemm, except that the
 * workspace fields are not checked. */
sl_status sl_gemm_plan(const sl_gemm_args* args, sl_plan* plan);

/* Bytes of workspace sl_gemm needs for these arguments (0 when the plan has
 * no K-split), from the same validation and kernel selection as
 * sl_gemm_plan; host only.  Errors as sl_gemm_plan, SL_ERR_NULL for a NULL
 * `bytes`. */
sl_status sl_gemm_workspace_bytes(const sl_gemm_args* args, int64_t* bytes);

/* Static text for a status code (never NULL). */
const char* sl_status_string(int32_t status);

/* Thread-local text of the last failure in this thread ("" if none); valid
 * until the next call into the library from the same thread. */
const char* sl_last_error_message(void);

int32_t sl_abi_version(void);

/*
 * Matrix-core operand maps used by the kernels, dumped from the same
 * constexpr tables the kernels are compiled from.  Each entry is one
 * (lane, slot) -> (row, col) of the operand tile.
 *   instr:   0 v_mfma_f32_16x16x32_f16      1 v_mfma_f32_32x32x16_f16
 *            2 v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)
 *            3 v_mfma_scale_f32_32x32x64_f8f6f4  (E4M3)
 *            4 / 5 the same two with E2M1 data (32 nibbles per lane)
 *            6 / 7 the same two with 6-bit E2M3 or E3M2 data (32 values per lane)
 *   operand: 0 A (row = m, col = k)   1 B (row = n, col = k)
 *            2 D accumulator (row = m, col = n)
 *            3 scale (row = operand row, col = K block of 32; slot 0 only)
 * Arrays receive up to `capacity` entries; *count gets the number of
 * entries of the map.  Host only; no HIP call.
 */
sl_status sl_query_fragment_map(int32_t instr, int32_t operand, int32_t* lane, int32_t* slot,
                                int32_t* row, int32_t* col, int64_t capacity, int64_t* count);

/*
 * LDS tile layout of a kernel variant: for each logical element (row, k) of
 * one operand's tile, its byte offset inside the tile's LDS buffer.
 * `variant` is the sl_plan.kernel id, or 5 for the M-major tile that an
 * operand with a_load / b_load == 3 uses (256 rows, one 64-wide K-tile,
 * M contiguous); `operand` 0 = A, 1 = B.  Writes
 * rows*cols offsets row-major (index row*cols + k) into `offsets` (up to
 * `capacity`), and the tile's rows, cols and element bytes into the three
 * outputs.  Host only.
 */
sl_status sl_query_lds_map(int32_t variant, int32_t operand, int64_t* offsets, int64_t capacity,
                           int32_t* rows, int32_t* cols, int32_t* elem_bytes);

/*
 * The LDS byte address each (lane, slot) of a fragment load reads for
 * MFMA tile 0, k-slice 0 of wave 0, i.e. the composition of the LDS tile
 * layout with the instruction's operand map.  `variant`/`operand` as in
 * sl_query_lds_map.  `addr` receives lanes*slots entries (lane-major).
 * For variant 5 it receives, per lane, the two addresses the lane supplies
 * to the fragment's two ds_read_b64_tr_b16 reads (lane-major, 128 entries).
 */
sl_status sl_query_fragment_addresses(int32_t variant, int32_t operand, int64_t* addr,
                                      int64_t capacity, int64_t* count);

/*
 * Device probe of one matrix-core instruction's operand maps: launches one
 * wave per case on `stream` and writes every accumulator register.
 * f16 instructions (instr 0/1), case c = (lane, slot) = (c / 8, c % 8):
 *   mode 0: A (lane, slot) holds 1.0, every other A slot 0; B slot (l, s)
 *           holds l*8 + s + 1.
 *   mode 1: the same with the roles of A and B swapped.
 * Scaled E4M3 instructions (instr 2/3), case c = (lane, byte) = (c / 32,
 * c % 32), unit (127) scales unless stated:
 *   mode 0/1: A one-hot 1.0; B byte = E4M3 code 0x20 + lane (0) or
 *             0x20 + byte (1).
 *   mode 2/3: the same with A and B swapped.
 *   mode 4:   A one-hot, B = 1.0, A scale of lane l = 127 + l - 32.
 *   mode 5:   B one-hot, A = 1.0, B scale of lane l = 127 + l - 32.
 *   mode 6/7: A in E2M1 (format 4): case = (lane, nibble) of a one-hot 1.0
 *             among the lane's 32 nibbles (16 bytes, low nibble first); B in
 *             E4M3 coded as in mode 0 (6) or mode 1 (7).
 *   mode 8/9, 10/11: A in FP6 E2M3 (format 2; modes 8, 9) or E3M2 (format
 *             3; modes 10, 11): case = (lane, value) of a one-hot 1.0 among
 *             the lane's 32 values, packed as one little-endian 6-bit stream
 *             over six dwords; B coded as in mode 0 (even) or mode 1 (odd).
 * `out` (device, fp32) receives cases * 64 * regs values laid out
 * [case][lane][reg].  Returns the case count through *cases.
 */
sl_status sl_probe_mfma(int32_t instr, int32_t mode, float* out, int64_t capacity,
                        int64_t* cases, void* stream);

/*
 * Device probe of the LDS data paths: each of 64 lanes of one wave writes
 * through the path under test and every byte of a 4096-byte LDS buffer is
 * copied to `out` (device, 4096 bytes), or for mode 2 the registers read.
 *   mode 0: LDS is first filled with the byte 0xA5; then one direct-to-LDS
 *           16-byte buffer load per lane: lane l loads the 16 bytes at
 *           src + 16*(perm[l] & 63), or, when perm[l] < 0, an out-of-range
 *           offset (src: 1024 device bytes, perm: device int32[64]).
 *   mode 1: as mode 0 with the global (non-buffer) direct-to-LDS load
 *           (perm[l] & 63 always).
 *   mode 2: ds_read_b64_tr_b16: LDS is filled with src (4096 bytes), lane l
 *           reads at byte address perm[l]; out receives 64 lanes x 8 bytes.
 *   mode 3: as mode 0 with a 4-byte direct-to-LDS buffer load: lane l loads
 *           the 4 bytes at src + 4*(perm[l] & 255).
 */
sl_status sl_probe_lds(int32_t mode, const void* src, const int32_t* perm, void* out, void* stream);

/*
 * Host layout algebra on shape:stride layouts given as text, the notation
 * of "数据布局及其记号" (section "Shape-Stride 模型": "(shape):(stride)",
 * nested tuples, a coordinate's offset is its dot product with the strides,
 * coordinates unflattened first-mode-fastest) and the operations
 * "CuTe 中 A、B 如何加载到 MMA 寄存器" derives its views and fragments with
 * (sections 2 and 3 and its closing source notes).  Host only, no HIP call.
 *
 * Text: "(4,(2,2)):(1,(4,8))", "8:1", "((_2,_2),_4):((_1,72),_2048)".  As in
 * that page's printed traces, a leading '_' marks a compile-time (static)
 * integer and a bare one a run-time value.  The distinction decides two
 * operations only: filter_zeros treats a stride as a broadcast only when it
 * is a static 0, and make_ordered takes static order values first (by
 * value) and run-time ones after them, in the order they appear.  Results
 * print without '_' unless `op` carries SL_LA_MARK_STATIC.
 *
 *   op                     a                 b              result
 *   SL_LA_PARSE            layout or shape   -              a, normalised
 *   SL_LA_COALESCE         layout            -              size-1 modes dropped, contiguous modes merged
 *   SL_LA_COMPOSITION      layout A          layout B       A o B (B's hierarchy; A(B(i)) for every i)
 *   SL_LA_COMPLEMENT       layout            integer N      the modes filling [0, N) around a's image
 *   SL_LA_RIGHT_INVERSE    layout            -              R with a(R(i)) == i on [0, size(R))
 *   SL_LA_ZIPPED_DIVIDE    layout            tiler layout   ((tile), (rest)); tiler mode i divides mode i
 *   SL_LA_FILTER_ZEROS     layout            -              static-0-stride leaves get shape 1
 *   SL_LA_COMPACT_LEFT     layout or shape   -              compact first-mode-fastest strides,
 *                                                           size-1 modes stride 0
 *   SL_LA_MAKE_ORDERED     layout or shape   order tuple    compact strides in the order of b's values
 *                                                           (or of b's strides if b is a layout)
 *   SL_LA_LOGICAL_PRODUCT  block             rest           (block, complement(block, size*cosize(rest)) o rest)
 *   SL_LA_TILED_PRODUCT    block             rest           the same, rest's modes lifted beside block
 *   SL_LA_FRAGMENT_LIKE    partition         -              make_fragment_like: mode 0 compacted
 *                                                           left (broadcasts kept), modes 1.. ordered
 *                                                           by their strides, tiled_product of the two
 *   SL_LA_TENSOR_LIKE      partition         -              make_ordered over all modes
 *   SL_LA_EVAL             layout            index          offset of the flat index (decimal)
 *   SL_LA_SIZE             layout or shape   -              number of coordinates (decimal)
 *   SL_LA_COSIZE           layout            -              1 + largest offset (decimal)
 *
 * The result text (NUL-terminated) goes to `out`; *needed (if not NULL)
 * gets its size in bytes including the NUL.  Errors: SL_ERR_NULL (a, b or
 * out NULL), SL_ERR_ARG (unknown op), SL_ERR_LAYOUT (text that does not
 * parse, or an operation undefined for its operands, e.g. a composition
 * whose strides do not divide), SL_ERR_SHAPE (out smaller than *needed, or
 * an EVAL index outside the layout).  The message says which.
 */
enum {
  SL_LA_PARSE = 0,
  SL_LA_COALESCE = 1,
  SL_LA_COMPOSITION = 2,
  SL_LA_COMPLEMENT = 3,
  SL_LA_RIGHT_INVERSE = 4,
  SL_LA_ZIPPED_DIVIDE = 5,
  SL_LA_FILTER_ZEROS = 6,
  SL_LA_COMPACT_LEFT = 7,
  SL_LA_MAKE_ORDERED = 8,
  SL_LA_LOGICAL_PRODUCT = 9,
  SL_LA_TILED_PRODUCT = 10,
  SL_LA_FRAGMENT_LIKE = 11,
  SL_LA_TENSOR_LIKE = 12,
  SL_LA_EVAL = 13,
  SL_LA_SIZE = 14,
  SL_LA_COSIZE = 15,
  SL_LA_MARK_STATIC = 256
};
sl_status sl_layout_op(int32_t op, const char* a, const char* b, char* out, int64_t capacity, int64_t* needed);

/*
 * Trace of the plan sl_gemm would run for `args` (host only: validation and
 * kernel selection as sl_gemm_plan, no HIP call): every stage's layout,
 * computed with the algebra above, one line each as "name: layout  # note",
 * plus "# note" lines.  The stages follow how "CuTe 中 A、B 如何加载到 MMA
 * 寄存器" walks one operand from memory to the instruction (section 2: the
 * TV map of the instruction, the thread's partition of the shared-memory
 * tile as a composition, its register fragment by make_fragment_like in
 * section 3), applied to this library's kernels:
 *   A_instr          (lane, slot) -> m + R k of the instruction's A operand
 *   A, A_tiles       the operand view, zipped_divide by the workgroup tile
 *   A_lds, A_copy    the LDS tile before its XOR swizzle (stated beside
 *                    it), the LDS bytes each copy instruction fills
 *   A_wave, A_lane0  the wave's (lane, ((slot), repeat, K slice)) partition
 *                    of the LDS tile, and lane 0's part of it
 *   A_frag           fragment_like of one K slice: the lane's registers
 *   (B the same), SFA / SFB / scale_instr for scaled formats,
 *   D_instr, acc, D_lane0   accumulator TV map, register order, and the D
 *                    elements of lane 0's registers
 *   D, C, D_tiles, tile_order, workgroup_tile, workspace (split-K).
 * Output and errors as sl_layout_op (plus sl_gemm_plan's validation
 * statuses); pointers in args are only checked, never dereferenced.
 */
sl_status sl_describe_plan(const sl_gemm_args* args, char* out, int64_t capacity, int64_t* needed);

#ifdef __cplusplus
}
#endif
#endif /* STRIDE_LAYOUTS_LDS_SL_H */
