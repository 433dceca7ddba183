/*
 * trt.h -- C ABI of the MI355X (gfx950) register-tile GEMM library, libtrt.so.
 *
 * One operation, as defined by the NineToothed page "Named layouts" (the GEMM
 * arrangement at the top of the page, and sections "Contract" and "Runtime
 * and compilation"):
 *
 *     C[M,N] = epilogue( A[M,K] . B[K,N] )
 *
 * computed by a grid of workgroups, each owning one logical [BM,BN] tile of C
 * and consuming [BM,BK] / [BK,BN] operand tiles per K step.  Products are
 * accumulated in fp32 and cast once, at the end, to the output dtype.  The
 * epilogue, when requested, is  y = relu(acc * row_scale[m] + bias[n]) + R[m,n]
 * with each term optional, evaluated in fp32 before the single cast.
 *
 * The library has no global mutable state and never allocates: all buffers
 * belong to the caller.  Every call validates its arguments on the host
 * before any device work (an error leaves C untouched) and then enqueues its
 * kernels on the caller's stream (one, or two for trt_gemm_ws's split K);
 * the result is valid once that stream has synchronised.  No pointer is
 * kept after a call returns.
 */
#ifndef TRT_H
#define TRT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRT_ABI_VERSION 13

/* Status codes.  Every entry point returns one of these. */
typedef enum {
  TRT_OK = 0,
  TRT_ERR_SIZE = 1,        /* a size out of range, an extent that overflows,
                              or more than 2^31-1 workgroups in one launch     */
  TRT_ERR_STRIDE = 2,      /* an input leading dimension < 1, or ldc < N       */
  TRT_ERR_NULL = 3,        /* A, B or C is NULL (or a required output buffer)  */
  TRT_ERR_ALIGN = 4,       /* a pointer not aligned to its element             */
  TRT_ERR_OVERLAP = 5,     /* C's byte range meets an input's byte range       */
  TRT_ERR_DTYPE = 6,       /* unsupported input/output dtype combination       */
  TRT_ERR_UNSUPPORTED = 7, /* no compiled kernel for the requested tile / map  */
  TRT_ERR_HIP = 8,         /* the HIP runtime reported an error (see message)  */
  TRT_ERR_ARG = 9          /* any other invalid argument (op flag, map id...)  */
} trt_status;

/* Element types: IEEE binary16, bfloat16 or binary32, for the inputs (A and
 * B share one dtype) and, independently, for the output C and the epilogue
 * operands (bias, residual, row scale), which share the output dtype.
 * binary32 inputs run on their own 128x128x32 tile. */
typedef enum { TRT_F16 = 1, TRT_BF16 = 2, TRT_F32 = 3 } trt_dtype;

/* Storage of an operand.  An operand is never transposed implicitly
 * ("Named layouts", section "Contract": a transpose is explicit):
 *   A, TRT_OP_N: A(m,k) = A[m*lda + k]   (row-major [M][lda])
 *   A, TRT_OP_T: A(m,k) = A[k*lda + m]   (A^T stored row-major [K][lda])
 *   B, TRT_OP_N: B(k,n) = B[k*ldb + n]   (row-major [K][ldb])
 *   B, TRT_OP_T: B(k,n) = B[n*ldb + k]   (B^T stored row-major [N][ldb])
 * C(m,n) = C[m*ldc + n] and R(m,n) = R[m*ldr + n].  Leading dimensions are
 * in elements, not bytes. */
typedef enum { TRT_OP_N = 0, TRT_OP_T = 1 } trt_op;

/* Optional same-output-domain postprocessing ("Named layouts", section
 * "Contract": bias / ReLU / residual on the output's own domain; a column
 * bias spans the n axis only and broadcasts over m, a row scale spans the m
 * axis only and broadcasts over n).  With acc the fp32 sum of products:
 *   y = acc * row_scale[m]   (if row_scale)
 *   y = y + bias[n]          (if bias)
 *   y = max(y, 0)            (if relu)
 *   y = y + R(m,n)           (if residual)
 * bias: [N] elements of out_dtype, or NULL.  row_scale: [M] elements of
 * out_dtype, or NULL.  residual: R(m,n) = residual[m*ldr + n] of out_dtype,
 * or NULL.  Passing NULL for the whole struct means a plain GEMM. */
typedef struct {
  const void* bias;
  int32_t relu;
  const void* residual;
  int64_t ldr;
  const void* row_scale;
} trt_epilogue;

/* A workgroup tile: the logical [bm, bn] output tile and the K step bk.
 * The physical thread shape (wavefronts of 64 lanes) and the per-lane
 * register shape of each compiled tile are reported by trt_tile_at(). */
typedef struct {
  int32_t bm, bn, bk;
} trt_tile;

/*
 * trt_gemm -- C = epilogue(A . B) with a tile chosen by the library.
 *
 * M, N, K >= 1 ("Named layouts", section "Runtime and compilation": logical
 * sizes are positive).  lda, ldb and (when a residual is given) ldr >= 1:
 * input strides are positive; input rows may overlap.  ldc >= N: output
 * writes never overlap each other.  C's byte range must not meet the byte
 * range of A, B, bias, residual or row_scale -- an in-place residual is
 * rejected, since safety that cannot be proven is an error.  A, B, C must be
 * non-NULL; A and B aligned to the input element, C and the epilogue operands
 * to the output element (2 or 4 bytes).  in_dtype and out_dtype are each
 * TRT_F16, TRT_BF16 or TRT_F32 (otherwise TRT_ERR_DTYPE).  M, N, K <= 2^30
 * and at most 2^31-1 output tiles for the chosen tile (TRT_ERR_SIZE).
 * Elements of C outside [0,M) x [0,N) (the ldc padding) are never written.
 * Elements of A and B outside the logical operands (the lda/ldb padding)
 * never influence C, and no byte outside an operand's extent ((rows-1)*ld +
 * cols elements from its base) is ever read.
 *
 * stream: a hipStream_t (NULL = the default stream).  The call enqueues one
 * kernel and returns; TRT_ERR_HIP means that launch failed (the status the
 * runtime returned for it, not an error left by an earlier HIP call), with
 * the runtime's message in trt_last_error().  Pointers are device (or
 * device-accessible) addresses owned by the caller.
 */
trt_status trt_gemm(int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda, int32_t opA,
                    const void* B, int64_t ldb, int32_t opB,
                    void* C, int64_t ldc,
                    int32_t in_dtype, int32_t out_dtype,
                    const trt_epilogue* epi, void* stream);

/*
 * trt_gemm_tiled -- trt_gemm with an explicit workgroup tile.  The tile is
 * the layout's own parameter: "Named layouts" fixes BM, BN, BK = 16, 64, 32
 * in its GEMM arrangement, and its section "Contract" has declared tile
 * sizes belong to the layout rather than to a backend's preset list, with
 * the target's real restrictions still applying.  Here the target's
 * restriction is what is compiled: tile must name a compiled instance (see
 * trt_tile_at; 16x64x32 is the page's), otherwise TRT_ERR_UNSUPPORTED and
 * nothing is enqueued.  tile == NULL behaves as trt_gemm.  With binary32
 * inputs the tile must be NULL or 128x128x32: that path has one kernel, a
 * 2x2-wave tile of 16x16x4 f32 matrix-core fragments, double-buffered
 * through LDS (not listed by trt_tile_at).  Arguments, ownership, stream
 * and errors otherwise as trt_gemm.
 */
trt_status trt_gemm_tiled(int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, int32_t opA,
                          const void* B, int64_t ldb, int32_t opB,
                          void* C, int64_t ldc,
                          int32_t in_dtype, int32_t out_dtype,
                          const trt_epilogue* epi, const trt_tile* tile,
                          void* stream);

/*
 * trt_gemm_workspace_size -- the bytes of workspace trt_gemm_ws uses for an
 * M x N x K problem with these storage orders and input dtype, or 0 when its
 * kernels need none; -1 on an argument error (sizes outside [1, 2^30], an
 * unknown op flag or dtype; message in trt_last_error()).  Host only, no HIP
 * call.  Nonzero only for the streaming shapes (M <= 16, A and B both
 * TRT_OP_N, 16-bit inputs, K % 8 == 0, N % 4 == 0) whose K is long enough to
 * split over workgroups: splits * M * N * 4 bytes of fp32 partial sums.
 */
int64_t trt_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t opA,
                                int32_t opB, int32_t in_dtype);

/*
 * trt_gemm_ws -- trt_gemm with a caller workspace.  The operation, arguments,
 * validation and errors are trt_gemm's ("Named layouts": the GEMM
 * arrangement and section "Contract"); the page's loop fixes the
 * accumulation over K blocks as one sum, which any order of fp32 additions
 * implements within the accumulation's rounding.  For the streaming shapes
 * of trt_gemm_workspace_size, when the operands also allow the streaming
 * kernel's vector loads (A 16-byte and B 8-byte aligned, lda % 8 == 0,
 * ldb % 4 == 0), K is split into slices over workgroups: each writes fp32
 * partial sums of its slice to the workspace, and a second kernel, on the
 * same stream, adds them in slice order (the result does not depend on
 * timing) and applies the epilogue; otherwise the call is trt_gemm and the
 * workspace is not touched.
 * workspace: device memory of at least trt_gemm_workspace_size(...) bytes
 * owned by the caller, 16-byte aligned, disjoint from A, B, C, bias,
 * residual and row_scale; it may be NULL (with any workspace_bytes) for
 * calls that need none.  Its contents on entry do not matter and are
 * unspecified afterwards; the library keeps no pointer to it.  Errors, before
 * any HIP call: trt_gemm's, and TRT_ERR_NULL / TRT_ERR_SIZE / TRT_ERR_ALIGN /
 * TRT_ERR_OVERLAP for a missing, short, misaligned or overlapping workspace.
 */
trt_status trt_gemm_ws(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, int32_t opA,
                       const void* B, int64_t ldb, int32_t opB,
                       void* C, int64_t ldc,
                       int32_t in_dtype, int32_t out_dtype,
                       const trt_epilogue* epi, void* workspace,
                       int64_t workspace_bytes, void* stream);

/*
 * trt_gemm_noalloc -- trt_gemm_ws for callers that cannot allocate (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same operation, arguments, validation, kernels and results (bit for bit),
 * with the workspace taken from a device array of TRT_NOALLOC_SCRATCH_BYTES
 * that the library's code object holds on each GPU it runs on, for the life
 * of the process; the call allocates and frees nothing.  Every split plan
 * needs at most 16,744,448 bytes (16 rows, at most ceil(512 / p) slices of p
 * column panels), so all fit; a call that needed more would fail with
 * TRT_ERR_SIZE.  The array's address on a device is looked up on the first
 * call on that device (the device of `stream`).  All calls on one GPU share
 * its array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that may overlap in time on one GPU -- on different
 * streams, or from several threads -- race and must be serialised by the
 * caller.  Errors: trt_gemm's; TRT_ERR_HIP if the array's address or the
 * stream's device cannot be read.
 */
#define TRT_NOALLOC_SCRATCH_BYTES 16777216
trt_status trt_gemm_noalloc(int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, int32_t opA,
                            const void* B, int64_t ldb, int32_t opB,
                            void* C, int64_t ldc,
                            int32_t in_dtype, int32_t out_dtype,
                            const trt_epilogue* epi, void* stream);

/*
 * trt_validate -- the host-side checks of trt_gemm_tiled, alone: returns the
 * status the call would return before any device work.  Makes no HIP call,
 * dereferences no pointer, and is safe on a machine without a GPU.
 */
trt_status trt_validate(int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda, int32_t opA,
                        const void* B, int64_t ldb, int32_t opB,
                        const void* C, int64_t ldc,
                        int32_t in_dtype, int32_t out_dtype,
                        const trt_epilogue* epi, const trt_tile* tile);

/*
 * trt_choose_tile -- the workgroup tile trt_gemm uses for an M x N output
 * with inputs of in_dtype (host only, no HIP call): for M <= 16 the
 * streaming tile 16x64 (K step 256); otherwise, when either 256-wide
 * pipelined tile gives the 256 compute units at least 192 workgroups, the
 * one of 256x256x32 and 256x192x32 with fewer rounds of 256 workgroups
 * times tile area; otherwise the pipelined 128x128x32 if it gives at least
 * 64 workgroups, else 64x64x64; binary32 inputs always 128x128x32 (the
 * binary32 kernel's tile).  Whether the pipelined
 * kernel or the generic one runs a pipelined tile also depends on the
 * operands' alignment and extents (see trt_gemm).  Errors: TRT_ERR_NULL,
 * TRT_ERR_SIZE (M or N outside [1, 2^30]), TRT_ERR_DTYPE.
 */
trt_status trt_choose_tile(int64_t M, int64_t N, int32_t in_dtype, trt_tile* tile);

/* Number of compiled workgroup tiles. */
int32_t trt_tile_count(void);

/*
 * trt_tile_at -- describe compiled tile i (0 <= i < trt_tile_count()):
 * its logical tile, its physical thread shape as waves_m x waves_n
 * wavefronts of 64 lanes, the accumulator registers each lane owns, and the
 * edge (16 or 32) of the square matrix-core fragments those registers are
 * grouped in ("My Triton From Scratch, Part 16: Register Tiles", section
 * "Three coordinate spaces": logical shape vs. thread shape vs. register
 * shape).  Any output pointer may be NULL.  TRT_ERR_ARG if i is out of range.
 */
trt_status trt_tile_at(int32_t i, trt_tile* tile, int32_t* waves_m,
                       int32_t* waves_n, int32_t* regs_per_lane, int32_t* frag);

/* Maps that trt_layout_dump can enumerate. */
typedef enum {
  /* C ownership: input index x = (wave*64 + lane)*REGS + reg, output
   * (row, col) of the tile element that accumulator register holds. */
  TRT_MAP_C_OWNER = 0,
  /* LDS operand slot: x = row*G + g (G = bk/8 chunks of 8 k per row),
   * output (slot, 0): the swizzled 16-byte chunk slot of chunk (row, g). */
  TRT_MAP_LDS_SLOT_A = 1,
  TRT_MAP_LDS_SLOT_B = 2,
  /* Cooperative copy, k-contiguous operand rows of the A tile:
   * x = iteration*THREADS + thread, output (row, g) of the 16-byte chunk
   * it moves, or (-1, -1) for an inactive tail lane. */
  TRT_MAP_COPY_KCONTIG_A = 3,
  /* Cooperative copy, row-contiguous storage of the A tile: output (rb, g)
   * of the 8x8 block it moves (rows 8rb..8rb+7, k = 8g..8g+7), or (-1,-1). */
  TRT_MAP_COPY_MNCONTIG_A = 4,
  TRT_MAP_COPY_KCONTIG_B = 5,
  TRT_MAP_COPY_MNCONTIG_B = 6,
  /* Direct-to-LDS tiles of the pipelined kernel (tiles with bk == 32).
   * k-contiguous operand tile: x = r*4 + g (chunk g of 8 k of row r),
   * output (slot, 0).  Rows-contiguous operand tile: x = k*(R/8) + c
   * (chunk c of 8 rows of k row k), output (slot, 0).  R = bm for A, bn
   * for B; the rows-contiguous maps need R >= 128. */
  TRT_MAP_DMA_KC_SLOT_A = 7,
  TRT_MAP_DMA_KC_SLOT_B = 8,
  TRT_MAP_DMA_MN_SLOT_A = 9,
  TRT_MAP_DMA_MN_SLOT_B = 10
} trt_map;

/*
 * trt_layout_dump -- evaluate map `map_id` of compiled tile `tile` on the
 * device, with the very device functions the GEMM kernels use (the C
 * ownership map is the one their epilogues store through), for inputs
 * x = 0..n-1, writing rows[x] and cols[x] (device buffers of n int32, owned
 * by the caller, not read).  "My Triton From Scratch, Part 16: Register
 * Tiles", section "Tests cover the mapping as a contract": every stage has to
 * agree on one ownership mapping; this call lets a test read the mapping the
 * device evaluates and compare it with the host's and with the oracle's.
 * n must equal trt_layout_size(map_id, tile).  Errors before any HIP call:
 * TRT_ERR_NULL, TRT_ERR_UNSUPPORTED (tile not compiled), TRT_ERR_ARG (map
 * not defined for the tile), TRT_ERR_SIZE; TRT_ERR_HIP if the launch fails.
 * Enqueued on `stream`.
 */
trt_status trt_layout_dump(int32_t map_id, const trt_tile* tile,
                           int32_t* rows, int32_t* cols, int64_t n,
                           void* stream);

/* The same maps evaluated on the host (no HIP call; host buffers). */
trt_status trt_layout_dump_host(int32_t map_id, const trt_tile* tile,
                                int32_t* rows, int32_t* cols, int64_t n);

/* Number of inputs of map `map_id` for tile `tile`, or -1 if unsupported. */
int64_t trt_layout_size(int32_t map_id, const trt_tile* tile);

/*
 * trt_layout_rank -- GF(2) rank of the C ownership map of a compiled tile
 * (the rank of its (register, lane, wave) -> (row, col) basis matrix), and
 * the number of its input and output bits.  Exactly-once ownership means
 * rank == in_bits == out_bits ("Triton LinearLayout", section
 * "Surjectivity, injectivity, and broadcasts").  Host only.
 */
trt_status trt_layout_rank(const trt_tile* tile, int32_t* rank,
                           int32_t* in_bits, int32_t* out_bits);

/*
 * trt_mfma_probe -- run one matrix-core instruction on one wave, shape 16
 * (16x16x32) or 32 (32x32x16): lane l passes a[l*8 .. l*8+7] as its first
 * operand register and b[l*8 ..] as its second (raw 16-bit values of
 * `dtype`), starting from a zero accumulator, and writes its R result
 * registers to c[l*R .. l*R+R-1] (fp32), R = 4 (shape 16) or 16 (shape 32).
 * a, b are device buffers of 512 elements, c of 64*R.  Used to confirm the
 * hardware fragment layouts the ownership maps are built on.
 */
trt_status trt_mfma_probe(int32_t dtype, int32_t shape, const void* a,
                          const void* b, float* c, void* stream);

/*
 * trt_hbm_read_probe -- measurement yardstick, not part of the GEMM: a plain
 * streaming read of `bytes` bytes at device address x (16-byte aligned,
 * bytes a positive multiple of 16), enqueued on `stream`.  The kernel runs
 * TRT_READ_PROBE_SINK_BYTES / 16 workgroups; workgroup w writes the XOR of
 * the 16-byte words it read to sink[16w .. 16w+15] (device buffer owned by
 * the caller, at least TRT_READ_PROBE_SINK_BYTES, 16-byte aligned, disjoint
 * from x), so the XOR of all sink words equals the XOR of all words of x.
 * Timing it gives the HBM read bandwidth a simple kernel reaches, the
 * context for the memory-bound (M <= 16) GEMM.  Errors: TRT_ERR_NULL,
 * TRT_ERR_SIZE, TRT_ERR_ALIGN, TRT_ERR_OVERLAP, before any HIP call;
 * TRT_ERR_HIP if the launch fails.
 */
#define TRT_READ_PROBE_SINK_BYTES 32768
trt_status trt_hbm_read_probe(const void* x, int64_t bytes, void* sink,
                              int64_t sink_bytes, void* stream);

/*
 * trt_mfma_loop_probe -- measurement yardstick, not part of the GEMM: 256
 * workgroups of 4 waves (one wave per SIMD) each run `iters` rounds of
 * matrix-core products and no other work in the loop, the instruction the
 * GEMM kernels issue: for dtype TRT_F16 or TRT_BF16, 64 v_mfma_f32_16x16x32
 * per round on 64 independent accumulators, 2^14 * 64 * 1024 * iters FLOP
 * per launch; for TRT_F32, 32 v_mfma_f32_16x16x4_f32 per round on 16
 * accumulators, 2^11 * 32 * 1024 * iters FLOP.  Operand registers come from
 * `operands` (device buffer of TRT_MFMA_PROBE_OPERAND_BYTES, 16-byte
 * aligned; lane l of every wave reads 16-byte words l, 64+l, ..., 960+l);
 * thread x of workgroup w writes 16 fp32 sums of its accumulators to
 * sink[16*(256w + x) ..] (device
 * buffer of at least TRT_MFMA_PROBE_SINK_BYTES, 64-byte aligned, disjoint
 * from the operands).  Timing it gives the matrix-core rate the part
 * sustains on such data, the context for the GEMM's fraction of peak.
 * Errors: TRT_ERR_NULL, TRT_ERR_DTYPE, TRT_ERR_ARG (iters < 1), TRT_ERR_SIZE,
 * TRT_ERR_ALIGN, TRT_ERR_OVERLAP, before any HIP call; TRT_ERR_HIP if the
 * launch fails.
 */
#define TRT_MFMA_PROBE_OPERAND_BYTES 16384
#define TRT_MFMA_PROBE_SINK_BYTES 4194304
trt_status trt_mfma_loop_probe(int32_t dtype, const void* operands, int32_t iters,
                               float* sink, int64_t sink_bytes, void* stream);

/*
 * trt_clock_probe -- measurement yardstick, not part of the GEMM: 256
 * workgroups of one wave each read the shader-cycle counter and the
 * constant-rate real-time counter, wait until the real-time counter has
 * advanced by `ticks` (1 <= ticks <= 2^27), and read both again; workgroup w
 * writes the shader cycles that passed to sink[2w] and the real-time ticks
 * to sink[2w+1] (uint64; device buffer owned by the caller, at least
 * TRT_CLOCK_PROBE_SINK_BYTES, 8-byte aligned).  cycles / ticks times the
 * real-time counter's rate is the shader clock while the probe ran: timed
 * right before and right after a measured region, it records the clock the
 * part ran at around it.  The rate itself follows from timing a long probe.
 * Errors: TRT_ERR_NULL, TRT_ERR_ARG, TRT_ERR_SIZE, TRT_ERR_ALIGN before any
 * HIP call; TRT_ERR_HIP if the launch fails.  Enqueued on `stream`.
 */
#define TRT_CLOCK_PROBE_SINK_BYTES 4096
trt_status trt_clock_probe(int64_t ticks, void* sink, int64_t sink_bytes, void* stream);

/*
 * The GF(2) layout algebra of the layout module ("Triton LinearLayout",
 * sections "Combining layouts" and "invertAndCompose: derive data
 * movement"), on caller arrays, host only (no HIP call).  The library derives
 * the inverse copy maps of its pipelined kernel with the same code at build
 * time.  A map of nin input bits to nout output bits (0 <= nin, nout <= 32)
 * is given by its nin columns: cols[i] is the image of input bit i, a word
 * with no bit at or above nout; the image of x is the XOR of the columns of
 * x's set bits.  Output arrays belong to the caller.  Errors: TRT_ERR_ARG
 * (bit counts out of range, a column beyond nout, mismatched sizes),
 * TRT_ERR_NULL, TRT_ERR_SIZE (a product beyond 32 bits).
 */
/* GF(2) rank of the map, or -1 on an argument error. */
int32_t trt_gf2_rank(int32_t nin, int32_t nout, const uint32_t* cols);
/* out (inner_nin columns of outer_nout bits) = outer o inner; outer_nin
 * must equal inner_nout. */
trt_status trt_gf2_compose(int32_t outer_nin, int32_t outer_nout, const uint32_t* outer,
                           int32_t inner_nin, int32_t inner_nout, const uint32_t* inner,
                           uint32_t* out);
/* out (a_nin + b_nin columns) = the direct sum of a and b: input bits of a
 * then of b, output bits of a then of b (b's columns shifted by a_nout). */
trt_status trt_gf2_product(int32_t a_nin, int32_t a_nout, const uint32_t* a,
                           int32_t b_nin, int32_t b_nout, const uint32_t* b,
                           uint32_t* out);
/* out = the map restricted to the input bits set in in_mask and projected
 * onto the output bits set in out_mask (kept bits in order, packed); its
 * sizes go to *out_nin and *out_nout. */
trt_status trt_gf2_sublayout(int32_t nin, int32_t nout, const uint32_t* cols,
                             uint32_t in_mask, uint32_t out_mask, uint32_t* out,
                             int32_t* out_nin, int32_t* out_nout);
/* q (r_nin columns of s_nin bits) with S(q(x)) == R(x) for every x, where
 * R: r_nin -> t_bits and S: s_nin -> t_bits; S may be non-injective (the
 * solution then uses only the columns of S independent of earlier ones).
 * TRT_ERR_ARG if some value of R is not a value of S. */
trt_status trt_gf2_invert_and_compose(int32_t r_nin, int32_t t_bits, const uint32_t* r,
                                      int32_t s_nin, const uint32_t* s, uint32_t* q);

/*
 * Register tiles of any logical shape ("My Triton From Scratch, Part 16:
 * Register Tiles").  A logical [lm, ln] C tile is computed by a physical
 * thread shape [tm, tn], each thread holding a register tile of
 * [lm/tm, ln/tn] accumulators.
 *
 * trt_regtile_thread_shape -- the deterministic thread-shape policy (section
 * "Choosing the physical thread shape"): of the pairs (a, b) with a dividing
 * lm, b dividing ln and a*b <= max_threads, the largest by (a*b, min(a, b),
 * b).  max_threads = 32 gives the pages' one-warp results, for example
 * (3, 17) -> (1, 17) and (16, 32) -> (4, 8); the GEMM below allows up to one
 * 64-lane wavefront.  Host only.  Errors: TRT_ERR_NULL, TRT_ERR_SIZE (lm or
 * ln < 1), TRT_ERR_ARG (max_threads < 1).
 */
trt_status trt_regtile_thread_shape(int32_t lm, int32_t ln, int32_t max_threads,
                                    int32_t* tm, int32_t* tn);

/*
 * trt_regtile_owner -- the strided ownership of a register tile (section "A
 * strided ownership rule"): thread t = ti*tn + tj, register r = ri*rn + rj
 * (rn = ln/tn) owns logical (ti + ri*tm, tj + rj*tn); writes rows[x],
 * cols[x] for x = t*(lm/tm * ln/tn) + r (caller arrays of n = lm*ln) and
 * checks that every logical element is owned exactly once.  Host only; it
 * is the map the register-tile GEMM's kernel evaluates.  Errors:
 * TRT_ERR_SIZE (a shape < 1, lm*ln > 2^24, n != lm*ln), TRT_ERR_ARG (tm does
 * not divide lm or tn does not divide ln), TRT_ERR_NULL.
 */
trt_status trt_regtile_owner(int32_t lm, int32_t ln, int32_t tm, int32_t tn,
                             int32_t* rows, int32_t* cols, int64_t n);

/*
 * trt_gemm_regtile -- trt_gemm computed with a register tile of logical
 * shape [lm, ln] on general-purpose vector lanes instead of the matrix
 * cores (section "Register-valued loop-carried accumulators"): one 64-lane
 * wavefront per output tile, thread shape trt_regtile_thread_shape(lm, ln,
 * max_threads), each thread accumulating its registers with fp32 fused
 * multiply-adds over K, then the same fused epilogue and rounding as
 * trt_gemm.  Any positive lm, ln (no power of two needed) with at most 8
 * registers per axis: lm/tm <= 8 and ln/tn <= 8, otherwise
 * TRT_ERR_UNSUPPORTED.  max_threads in [1, 64] (TRT_ERR_ARG).  Arguments,
 * dtypes, validation and errors otherwise as trt_gemm; enqueued on `stream`.
 */
trt_status trt_gemm_regtile(int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, int32_t opA,
                            const void* B, int64_t ldb, int32_t opB,
                            void* C, int64_t ldc,
                            int32_t in_dtype, int32_t out_dtype,
                            const trt_epilogue* epi, int32_t lm, int32_t ln,
                            int32_t max_threads, void* stream);

/*
 * trt_block_reduce -- the rank-1 block reduction ("My Triton From Scratch,
 * Part 12: CUDA Tile Layouts", section "Output shape is not always thread
 * shape"): out[b] = op over x[b*block .. min(n, (b+1)*block) - 1] for every
 * block b = 0 .. ceil(n / block) - 1 (the last block may be partial; its
 * missing elements are masked off).  x: n contiguous elements of dtype
 * (TRT_F16, TRT_BF16 or TRT_F32), aligned to its element; out: ceil(n/block)
 * binary32 results, 4-byte aligned, disjoint from x; both device buffers
 * owned by the caller.  op: TRT_REDUCE_SUM (accumulated in binary32, in an
 * order of the library's choosing), TRT_REDUCE_MAX or TRT_REDUCE_MIN (an
 * element of the block; NaN if any element is NaN; +0 and -0 compare
 * equal).  n, block >= 1, n <= 2^40.  Errors before any HIP call:
 * TRT_ERR_SIZE, TRT_ERR_DTYPE, TRT_ERR_ARG (op), TRT_ERR_NULL,
 * TRT_ERR_ALIGN, TRT_ERR_OVERLAP; TRT_ERR_HIP if the launch fails.
 * Enqueued on `stream`.
 */
typedef enum { TRT_REDUCE_SUM = 0, TRT_REDUCE_MAX = 1, TRT_REDUCE_MIN = 2 } trt_reduce_op;
trt_status trt_block_reduce(const void* x, int64_t n, int64_t block, int32_t dtype,
                            int32_t op, float* out, void* stream);

/*
 * trt_abi_version -- the ABI version of the loaded library (TRT_ABI_VERSION
 * at build time).  "Named layouts", section "Runtime and compilation": the
 * launch ABI keeps versioned layout obligations so that caching and reload
 * cannot drop checks; a caller compares this number with the header it was
 * built against before it calls anything else.  No error.
 */
int32_t trt_abi_version(void);

/*
 * trt_last_error -- a message describing the last failed call on the calling
 * thread ("" after a call that succeeded).  The pointer stays valid until the
 * thread's next call into the library; the text belongs to the library.  No
 * page defines it: it is this library's way to carry a runtime message with
 * TRT_ERR_HIP and to say which check an argument failed.
 */
const char* trt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRT_H */
