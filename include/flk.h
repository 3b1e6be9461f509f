/*
 * flk.h -- C ABI of the MI355X packed-KV codec (FlashLoop INT4 base + cross-loop residuals).
 *
 * The codec stores one request/layer's logical [token, KV head, channel] BF16 K or V tensor
 * as a quantized base plus successive cross-loop residuals, each encoded against the
 * reconstructed predecessor, and rebuilds the tensor at any depth from the packed streams.
 * It follows the FlashLoop integration RFC (vllm-rlt issue #156), section 3.3 "Quantized base
 * and cross-loop KV residuals", and the standalone codec of vllm-rlt pull request #166
 * ("Purpose": INT4 codes two per byte, FP16 minimum and scale, group 64, K grouped across
 * compact token rows per head/channel, V across channels per token/head, subtraction and
 * addition in the compute dtype, partial groups allowed).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensors live in device memory (HBM) unless a parameter says "host".  Every pointer is
 *    a plain device address (for example torch.Tensor.data_ptr()).  The caller allocates and
 *    owns every buffer, including workspace; the library never allocates, frees, or keeps a
 *    pointer after the call returns (the RFC, section 4: the runner owns the tensors, kernels
 *    borrow them).
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  Work is
 *    enqueued on it and the call returns without synchronizing; buffers must stay untouched
 *    until that stream work has completed.  The library never reads device data on the host
 *    (the RFC, section 6.2: no GPU-to-CPU readback to prepare asynchronous work).
 *  - Validation happens on the host before anything is enqueued.  On any status other than
 *    FLK_OK nothing has been launched and no output byte has been written (the RFC, section 4:
 *    explicit incompatible choices fail clearly).  No C++ exception crosses the ABI.
 *  - BF16 tensors are [rows, H, D] row-major with channels contiguous.  Element (r, h, c) is
 *    at index (r*H + h)*D + c.  BF16 data, codes and params must be 16-byte aligned, rows
 *    4-byte aligned.  Every BF16 tensor a call describes stays below 4 GiB
 *    (T*H*D < 2^31 elements); larger sizes are FLK_E_SHAPE.
 *  - Preconditions not checked on the host: `rows` arrays strictly ascending with values in
 *    [0, T); inputs finite.  Non-finite inputs, FP16 overflow of a group's minimum or scale
 *    and rows entries outside [0, T) are reported through the optional device status word
 *    (below); outputs are then undefined, but no kernel addresses memory outside the
 *    buffers the call describes.
 *
 * Packed stream layout (one loop of one tensor, n compact rows)
 * -------------------------------------------------------------
 *  codes   uint8 [n][H][D/2]: byte j of (row, head) holds channel 2j in its low nibble and
 *          channel 2j+1 in its high nibble (PR #166 lists nibble order among its tests).
 *  params  uint32, one per group: FP16 minimum in bits 0..15, FP16 scale in bits 16..31.
 *          K, compact-row groups (FLK_KGROUP_ROWS): [ceil(n/64)][H][D], group g of channel
 *          (h, c) covers compact rows 64g..64g+63.
 *          K, tile groups (FLK_KGROUP_TILE): [ceil(T/64)][H][D], group t of channel (h, c)
 *          covers the compact rows whose positions lie in [64t, 64t+64) (0 to 64 rows; an
 *          empty tile's params are 0).  A dense stream is the same in both forms.
 *          V: [n][H][ceil(D/64)]  (group g of (row, h) covers channels 64g..64g+63).
 *          The last group along the axis may be partial (statistics over its real elements).
 *  rows    int32 [n], ascending logical positions of the compact rows (compact row ->
 *          logical position); NULL for a dense stream (n == T).  A position a residual
 *          stream does not list inherits its predecessor (an absent residual is not a
 *          code-0 residual, RFC section 3.3).
 *  tile_start  int32 [ceil(T/64) + 1], the inverse map at 64-position granularity:
 *          tile_start[t] = number of rows < 64*t, so the compact rows of positions
 *          [64t, 64t+64) are tile_start[t] .. tile_start[t+1]-1 (and tile_start[last] = n).
 *          Compact streams only (NULL for dense).  Together with rows it is the RFC's
 *          explicit logical-position <-> compact-row mapping (section 3.3); readers use it
 *          instead of searching rows.  flk_encode_residual writes it; it depends on rows and
 *          T alone, so the K and V streams of one loop may share one array.
 *  Codes and params for a group are computed with the FP16-rounded minimum and scale:
 *    scale32 = (max - min) / 15 (binary32), min16 = fp16(min), scale16 = fp16(scale32),
 *    code = clamp(round_half_even((x - min16) / scale16), 0, 15), or 0 when scale16 == 0
 *    (the constant group), and decoding is bf16(min16 + scale16 * code).  Min and max use
 *    the total order in which -0 < +0.
 */
#ifndef FLK_H
#define FLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLK_ABI_VERSION 2
#define FLK_GROUP 64       /* group size (PR #166 "Purpose": default group size 64)        */
#define FLK_MAX_LOOPS 8    /* longest chain (base + residuals) one call accepts             */
#define FLK_MAX_HEAD_DIM 512

typedef enum flk_status {
    FLK_OK = 0,
    FLK_E_NULL = 1,        /* a required pointer is NULL                                      */
    FLK_E_SHAPE = 2,       /* a size is out of range (T, n_rows, H, D, n_loops, heads ...)     */
    FLK_E_ALIGN = 3,       /* a pointer is not aligned as documented                           */
    FLK_E_DESC = 4,        /* descriptor fields not recognised (version/format/kind/group ...) */
    FLK_E_UNSUPPORTED = 5, /* a valid request this library does not implement                  */
    FLK_E_WORKSPACE = 6,   /* workspace missing or smaller than flk_workspace_bytes()          */
    FLK_E_LAUNCH = 7       /* the HIP runtime rejected a kernel launch                         */
} flk_status;

/* Which tensor a stream encodes; it selects the group axis and is recorded in the
 * descriptor (the PR #166 review asks for format, axis and group size in the descriptor). */
enum { FLK_KIND_K = 0, FLK_KIND_V = 1 };
enum { FLK_FMT_INT4_AFFINE = 1, FLK_FMT_NVFP4 = 2, FLK_FMT_MXFP4 = 3 };
enum { FLK_PARAM_FP16_MIN_SCALE = 1, FLK_PARAM_E4M3_BLOCK_F32_STREAM = 2, FLK_PARAM_E8M0_BLOCK = 3 };
enum { FLK_NIBBLE_LOW_EVEN = 1 };

/* The NVFP4 variant (PR #166 review, item 2: E2M1 codes, one E4M3 scale per 16 elements and
 * one FP32 scale per tensor, about 4.5 bits per element, symmetric).  Descriptor: format
 * FLK_FMT_NVFP4, group FLK_FP4_BLOCK, param_dtype FLK_PARAM_E4M3_BLOCK_F32_STREAM,
 * k_grouping FLK_KGROUP_ROWS, D % 16 == 0.  Blocks run along the 16 consecutive channels of one
 * (row, head) for K and V alike.  Per stream of n rows:
 *   codes   [n][H][D/2] bytes, low nibble = even channel; a nibble is sign (bit 3) and the
 *           E2M1 magnitude 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)
 *   params  a 16-byte header {s_g, amax, 0, 0} (binary32) then the E4M3 block scales
 *           [n][H][D/16] bytes (flk_params_bytes = 16 + n*H*D/16)
 * The stream scale is s_g = RN32(amax / 2688) over the magnitudes the stream encodes (X for a
 * base loop, the BF16 residual for a residual loop), or 1 when amax is 0.  A block's scale is
 * E4M3(RN32(amax_b / RN32(6 * s_g))), nearest-even and saturated at 448, and its binary32 value
 * bs = RN32(e4m3 * s_g).  Each code is the E2M1 value nearest (ties to even) to RN32(x / bs),
 * saturated at 6; a value that rounds to zero keeps its sign; a block with bs == 0 has codes
 * +0.  Decoding gives RN32(e2m1 * bs), rounded to BF16.  The residual chain is the INT4 one:
 * residuals are rounded to BF16 before encoding and added in binary32, rounded to BF16. */
#define FLK_FP4_BLOCK 16

/* The MXFP4 variant (OCP Microscaling Formats specification v1.0, section 6: E2M1 elements
 * sharing one E8M0 power-of-two scale per block of 32; the pages name NVFP4 only, and MX-scaled
 * FP4 only as an instruction's name).  Descriptor: format FLK_FMT_MXFP4, group FLK_MX_BLOCK,
 * param_dtype FLK_PARAM_E8M0_BLOCK, k_grouping FLK_KGROUP_ROWS, D % 32 == 0.  Blocks run along
 * the 32 consecutive channels of one (row, head) for K and V alike.  Per stream of n rows:
 *   codes   as NVFP4's: [n][H][D/2] bytes, low nibble = even channel, sign in bit 3
 *   params  the E8M0 block scales [n][H][D/32] bytes, no header (flk_params_bytes = n*H*D/32)
 * A block's scale is X = 2^e with e = floor(log2(amax_b)) - 2, clamped to [-127, 127] (-127 for
 * a block of zeros); its byte is e + 127.  Each code is the E2M1 value nearest (ties to even) to
 * x / X, saturated at 6 (amax_b / X lies in [4, 8), so values above 6 X are clipped); a value
 * that rounds to zero keeps its sign.  Decoding gives e2m1 * X, exact in BF16.  4.25 bits per
 * element.  The residual chain is the INT4 one. */
#define FLK_MX_BLOCK 32

/* Who owns a K group (the PR #166 review, item 3 "Group ownership vs 16-token pages": K
 * groups that follow compact-row order can put rows of distant positions, on different
 * pages, under one minimum and scale, so no page can be freed, offloaded, transferred or
 * shared without re-encoding its group).
 *   FLK_KGROUP_ROWS  64 consecutive compact rows (the default; the fewest groups).
 *   FLK_KGROUP_TILE  the compact rows of one 64-position tile, i.e. of four whole 16-token
 *                    pages: a tile's codes and params depend on that tile's tokens alone,
 *                    and whole tiles can be appended to a stream (flk_append_residual).
 * V groups lie within one token row, so they are page-local in either form. */
enum { FLK_KGROUP_ROWS = 0, FLK_KGROUP_TILE = 1 };

/* Bits of the optional device status word (a uint32 in device memory the caller zeroes).
 * Encode kernels OR these in with a device atomic; they never clear it. */
#define FLK_DEV_NONFINITE 1u  /* a group held an Inf or NaN value                           */
#define FLK_DEV_RANGE 2u      /* a group's minimum or scale overflowed FP16                 */
#define FLK_DEV_ROWS 4u       /* a rows entry lay outside [0, T); that row was skipped      */
#define FLK_DEV_COUNT 8u      /* token selection: the windows' budgets do not add up to n_out */
#define FLK_DEV_CLASS 16u     /* row partition: a class value other than FLK_ROW_*; the row
                                 was left out as inactive                                  */

/* Versioned encoding descriptor (the RFC, section 6.5: bit width, group axes and sizes and
 * depth representation travel with the data).  Fill with flk_desc_init(). */
typedef struct flk_desc {
    uint16_t abi_version;   /* FLK_ABI_VERSION                                             */
    uint8_t format;         /* FLK_FMT_INT4_AFFINE, FLK_FMT_NVFP4 or FLK_FMT_MXFP4         */
    uint8_t kind;           /* FLK_KIND_K or FLK_KIND_V                                    */
    uint16_t group;         /* FLK_GROUP (64) INT4, FLK_FP4_BLOCK (16) NVFP4, FLK_MX_BLOCK (32) MXFP4 */
    uint8_t param_dtype;    /* FLK_PARAM_FP16_MIN_SCALE (INT4), FLK_PARAM_E4M3_BLOCK_F32_STREAM
                               (NVFP4), FLK_PARAM_E8M0_BLOCK (MXFP4)                      */
    uint8_t nibble_order;   /* FLK_NIBBLE_LOW_EVEN                                         */
    int32_t n_heads;        /* H >= 1                                                      */
    int32_t head_dim;       /* D: 8 <= D <= FLK_MAX_HEAD_DIM, D % 8 == 0                   */
    uint8_t k_grouping;     /* FLK_KGROUP_ROWS or FLK_KGROUP_TILE (no effect on V)         */
    uint8_t reserved[3];    /* must be 0                                                   */
} flk_desc;

/* One encoded loop of one tensor, as the host describes it to the library.  The struct is
 * host memory; the pointers inside are device addresses. */
typedef struct flk_stream {
    int32_t n_rows;         /* compact rows n (n == T for a dense stream)                  */
    int32_t reserved;       /* must be 0                                                   */
    const int32_t* rows;    /* device, n ascending positions in [0, T), or NULL = dense    */
    const uint8_t* codes;   /* device, flk_codes_bytes(desc, n) bytes, 16-byte aligned     */
    const uint32_t* params; /* device, flk_params_bytes(desc, n) bytes, 16-byte aligned    */
    const int32_t* tile_start; /* device, flk_tile_index_bytes(T) bytes; NULL = dense      */
} flk_stream;
/* A stream with n_rows == 0 (an empty loop) contributes nothing; its pointers are ignored. */

/* ---------------------------------------------------------------- host-only helpers --- */

/* Fill a descriptor with the only format this ABI version defines and compact-row K groups
 * (set k_grouping afterwards to choose tile groups). */
void flk_desc_init(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim);

/* Fill a descriptor for NVFP4 streams.  NVFP4 descriptors are accepted by flk_desc_check, the
 * stream size functions, flk_encode_base, flk_encode_residual, flk_reconstruct,
 * flk_reconstruct_mixed, flk_decode_attn_mixed and the two sparse *_mixed calls; every other
 * entry point answers FLK_E_UNSUPPORTED. */
void flk_desc_init_nvfp4(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim);

/* Fill a descriptor for MXFP4 streams; accepted by the same entry points as NVFP4's. */
void flk_desc_init_mxfp4(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim);

/* FLK_OK if the descriptor is well formed, else FLK_E_NULL / FLK_E_DESC / FLK_E_SHAPE. */
flk_status flk_desc_check(const flk_desc* d);

/* Storage of one stream with n compact rows (the RFC, section 7.4: the allocator budgets
 * payload, quantization parameters and maps).  0 for a malformed descriptor or n < 0.   */
size_t flk_codes_bytes(const flk_desc* d, int32_t n_rows);   /* n*H*D/2                    */
size_t flk_params_bytes(const flk_desc* d, int32_t n_rows, int32_t T); /* 4 * groups; T is
                                       the stream's positions (read for tile-grouped K only);
                                       NVFP4: 16 + n*H*D/16; MXFP4: n*H*D/32               */
size_t flk_rows_bytes(int32_t n_rows, int sparse);            /* 4*n if sparse, else 0      */
size_t flk_tile_index_bytes(int32_t T);                       /* 4*(ceil(T/64) + 1)         */
/* Everything one stream stores: codes + params + rows + tile index (sparse streams), with
 * the padding of partially filled groups and, for tile-grouped K, one parameter row per
 * tile whatever its occupancy (the RFC, section 7.4: small residual streams pay for their
 * partially filled groups; resource queries report the format's actual cost). */
size_t flk_stream_bytes(const flk_desc* d, int32_t n_rows, int32_t T, int sparse);

/* Rolling BF16 tail (the RFC, section 3.3, last paragraph: the tail keeps at least 64 recent
 * tokens and flushes whole 64-token groups, so it holds 64 to 127 tokens after a step).
 * Returns how many leading positions of an n_tokens sequence a rolling cache keeps packed:
 * the largest multiple of 64 that leaves at least 64 tokens in the tail (0 below 128
 * tokens, and 0 for n_tokens < 0).  Positions [prefix, n_tokens) stay in BF16. */
int32_t flk_rolling_prefix(int32_t n_tokens);

/* Workspace of flk_decode_attn_packed and flk_decode_attn_rolling: enough for every call over
 * at most T attended tokens in all (packed plus BF16 tail, T >= 0) with n_q_heads query heads
 * (other calls need none); non-decreasing in T, so a buffer sized for the longest context
 * serves every shorter one.  0 for malformed arguments. */
size_t flk_attn_workspace_bytes(const flk_desc* k_desc, int32_t T, int32_t n_q_heads);

const char* flk_status_string(flk_status s);
int flk_abi_version(void);

/* ---------------------------------------------------------------- codec calls --------- */

/* Loop 1: X_hat[1] = dequantize(quantize(X[1])) (RFC section 3.3; loop 1 is dense, section
 * 3.1).  x: BF16 [T, H, D] (input).  codes/params: the base stream (outputs, dense, n = T).
 * recon: BF16 [T, H, D] (output) receives X_hat[1], the predecessor of loop 2.
 * dev_status: optional device uint32 (may be NULL), see FLK_DEV_*.
 * Errors: FLK_E_NULL, FLK_E_DESC, FLK_E_SHAPE (T < 1), FLK_E_ALIGN, FLK_E_LAUNCH.       */
flk_status flk_encode_base(const flk_desc* d, const void* x, int32_t T, uint8_t* codes,
                           uint32_t* params, void* recon, uint32_t* dev_status, void* stream);

/* Loop r >= 2 (RFC section 3.3): delta[j] = bf16(X[r][j] - X_hat[r-1][p_j]) with
 * p_j = rows[j] (or j when rows == NULL), encoded with K groups over compact rows j; then
 * X_hat[r][p_j] = bf16(X_hat[r-1][p_j] + dequantize(quantize(delta))[j]); positions not in
 * rows are left untouched (inheritance).
 * x_rows: BF16 [n_rows, H, D], X[r] at the active positions only (input).
 * rows: device int32 [n_rows] ascending positions, or NULL for a dense loop (n_rows == T).
 * recon: BF16 [T, H, D], X_hat[r-1] on entry, X_hat[r] on exit (updated in place).
 * codes/params: the residual stream (outputs).  tile_start: output, required when rows is
 * not NULL (flk_tile_index_bytes(T) bytes, 4-byte aligned), ignored for a dense loop.
 * n_rows == 0 (an empty loop) is allowed, ignores x_rows, rows, codes, params and
 * tile_start, and writes nothing.
 * Errors: as flk_encode_base, plus FLK_E_SHAPE when n_rows > T or rows == NULL with
 * n_rows != T.                                                                            */
flk_status flk_encode_residual(const flk_desc* d, const void* x_rows, const int32_t* rows,
                               int32_t n_rows, int32_t T, void* recon, uint8_t* codes,
                               uint32_t* params, int32_t* tile_start, uint32_t* dev_status,
                               void* stream);

/* Rebuild X_hat[n_loops] from the packed chain alone (RFC section 3.3: a loop-4 read of t1
 * resolves to base + delta2, of t2 to base + delta2 + delta3, of t4 to the full chain).
 * chain: host array of n_loops streams; chain[0] is the dense base, chain[l] the residual of
 * loop l+1.  Each step adds in binary32 and rounds to BF16, as the encoder did, so the
 * result equals the encoder's in-place reconstruction bit for bit.
 * out: BF16 [T, H, D] (output).  1 <= n_loops <= FLK_MAX_LOOPS.
 * Errors: FLK_E_NULL, FLK_E_DESC, FLK_E_SHAPE, FLK_E_ALIGN, FLK_E_LAUNCH.                */
flk_status flk_reconstruct(const flk_desc* d, int32_t T, const flk_stream* chain,
                           int32_t n_loops, void* out, void* stream);

/* flk_reconstruct for a chain whose base (chain[0]) is described by base_desc and whose
 * residual loops by resid_desc: an INT4 base with FP4 residuals (the PR #166 review's "INT4
 * base plus NVFP4 residuals", and likewise with MXFP4), NVFP4 or MXFP4 throughout, or INT4
 * throughout.  Both descriptors must agree on kind, H and D.  An FP4 base with INT4 residuals,
 * and NVFP4 mixed with MXFP4, are FLK_E_UNSUPPORTED.
 * Errors: those of flk_reconstruct, plus FLK_E_DESC when the descriptors disagree. */
flk_status flk_reconstruct_mixed(const flk_desc* base_desc, const flk_desc* resid_desc, int32_t T,
                                 const flk_stream* chain, int32_t n_loops, void* out, void* stream);

/* Single-token decode attention read directly from the packed chains (RFC section 3.3:
 * optimized readers consume packed base/residual tiles during QK/PV instead of building a
 * BF16 shadow cache).  out[i] = sum_t softmax_t(scale * q[i] . K_hat[t, h]) V_hat[t, h] with
 * h = i / (n_q_heads / H) (grouped-query attention), K_hat/V_hat the chains' final depth.
 * q: BF16 [n_q_heads, D].  out: BF16 [n_q_heads, D].  Accumulation is binary32; the
 * result agrees with exact attention over the reconstructed BF16 K/V to about 1e-2
 * relative, not bit for bit.  workspace: device, >= flk_attn_workspace_bytes().
 * Requires k_desc kind K, v_desc kind V, equal H and D, D == 128, n_q_heads % H == 0,
 * n_q_heads / H <= 16, and both chains with the same T and n_loops.
 * Errors: FLK_E_NULL, FLK_E_DESC, FLK_E_SHAPE, FLK_E_ALIGN, FLK_E_UNSUPPORTED,
 * FLK_E_WORKSPACE, FLK_E_LAUNCH.                                                          */
flk_status flk_decode_attn_packed(const flk_desc* k_desc, const flk_desc* v_desc, int32_t T,
                                  const void* q, int32_t n_q_heads, const flk_stream* k_chain,
                                  const flk_stream* v_chain, int32_t n_loops,
                                  float softmax_scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Largest scratch area flk_decode_attn_packed_noalloc uses: a device array of this many bytes,
 * one copy per GPU the library runs on, held until the process ends. */
#define FLK_NOALLOC_SCRATCH_BYTES (64u << 20)

/* flk_decode_attn_packed without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The per-split partial results go to the library's own device array of
 * FLK_NOALLOC_SCRATCH_BYTES bytes on the current device (located on the first call on that
 * device); the call allocates nothing.  Every call on one GPU uses the same array, which keeps
 * the last call's contents (each call writes every partial it reads): calls that may overlap
 * in time on one GPU (streams not ordered with each other) race, and their outputs are then
 * undefined.  Arguments as flk_decode_attn_packed.
 * Errors: those of flk_decode_attn_packed; FLK_E_WORKSPACE when the call needs more than
 * FLK_NOALLOC_SCRATCH_BYTES (flk_attn_workspace_bytes(k_desc, T, n_q_heads) bounds the need;
 * 131072 tokens, 8 KV heads and 32 query heads need about 21.5 MB); FLK_E_LAUNCH when the
 * array cannot be located on the current device or a launch fails.                         */
flk_status flk_decode_attn_packed_noalloc(const flk_desc* k_desc, const flk_desc* v_desc, int32_t T,
                                          const void* q, int32_t n_q_heads, const flk_stream* k_chain,
                                          const flk_stream* v_chain, int32_t n_loops, float softmax_scale,
                                          void* out, void* stream);

/* flk_decode_attn_packed over chains whose streams are INT4 throughout, an INT4 base with FP4
 * residual loops, or FP4 throughout, the FP4 loops all NVFP4 or all MXFP4 (PR #166 review,
 * item 2: the comparison that counts is speed and accuracy with dequantization and residual
 * reconstruction fused into attention).  The base loop of the K chain is described by kd_base,
 * its residual loops by kd_resid; V likewise.  K and V must use the same combination; an FP4
 * base with INT4 residuals, NVFP4 mixed with MXFP4, and tile-grouped K with FP4 residuals are
 * FLK_E_UNSUPPORTED.  An FP4 value is the E2M1 code times the block's binary32 scale, rounded
 * to BF16, as flk_reconstruct decodes it.
 * Errors: those of flk_decode_attn_packed, plus FLK_E_DESC when a descriptor's kind is not the
 * tensor's. */
flk_status flk_decode_attn_mixed(const flk_desc* kd_base, const flk_desc* kd_resid, const flk_desc* vd_base,
                                 const flk_desc* vd_resid, int32_t T, const void* q, int32_t n_q_heads,
                                 const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops,
                                 float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------------------
 * Appending whole tiles: the flush of a rolling BF16 tail (the RFC, section 3.3, last
 * paragraph).  Decode-time tokens stay in BF16 until a whole 64-token group can leave the
 * tail; the flush encodes positions [p0, p0 + n_pos) of every loop and appends them to
 * streams that already hold positions [0, p0).  Because groups never straddle a tile (V
 * groups lie in one row; K groups are tile groups, or dense), the streams afterwards are
 * exactly those of encoding [0, p0 + n_pos) in one call, and the bytes already written are
 * never touched.
 * Common rules: p0 and n_pos are multiples of 64, n_pos >= 64, and (p0 + n_pos)*H*D < 2^31.
 * codes / params / tile_start point at the START of the stream's buffers, which must hold
 * the stream after the append (flk_codes_bytes(d, rows_before + n_rows), flk_params_bytes(
 * d, rows_before + n_rows, p0 + n_pos), flk_tile_index_bytes(p0 + n_pos)); the call writes
 * only the window's part of them.  recon is the window's own reconstruction, BF16
 * [n_pos, H, D]: row i is position p0 + i.
 * --------------------------------------------------------------------------------------- */

/* Loop 1 of the window: x is X[1] at positions [p0, p0 + n_pos), BF16 [n_pos, H, D]; recon
 * receives X_hat[1] of the window.  Writes codes rows p0.. and the window's params.
 * Errors: those of flk_encode_base, plus FLK_E_SHAPE for p0 or n_pos not as above.      */
flk_status flk_append_base(const flk_desc* d, const void* x, int32_t p0, int32_t n_pos, uint8_t* codes,
                           uint32_t* params, void* recon, uint32_t* dev_status, void* stream);

/* Loop r >= 2 of the window.  rows: device int32 [n_rows], the stream's row entries for the
 * window -- ascending absolute positions in [p0, p0 + n_pos) -- or NULL for a dense loop
 * (n_rows == n_pos, rows_before == p0).  rows_before: the stream's compact rows at
 * positions < p0 (rows_before <= p0).  x_rows: BF16 [n_rows, H, D], X[r] at those rows.
 * recon: X_hat[r-1] of the window on entry, X_hat[r] on exit.  A compact loop writes
 * codes rows rows_before.., its tile parameters (tile-grouped K) or row parameters (V), and
 * tile_start[p0/64 .. (p0+n_pos)/64] = rows_before + (rows of the window below each tile).
 * n_rows == 0 writes only those tile_start entries and, for K, zero params of the window's
 * tiles.  Compact K loops need k_grouping == FLK_KGROUP_TILE (compact-row groups would
 * have to merge with the stream's last, partially filled group): FLK_E_UNSUPPORTED
 * otherwise.
 * Errors: those of flk_encode_residual, plus FLK_E_SHAPE for a window or rows_before out
 * of range, FLK_E_UNSUPPORTED as above.                                                  */
flk_status flk_append_residual(const flk_desc* d, const void* x_rows, const int32_t* rows, int32_t n_rows,
                               int32_t p0, int32_t n_pos, int32_t rows_before, void* recon, uint8_t* codes,
                               uint32_t* params, int32_t* tile_start, uint32_t* dev_status, void* stream);

/* Decode attention over a rolling cache: the packed chains hold positions [0, T) (T may be
 * 0, then the chains are not read) and the BF16 tail holds positions [T, T + tail_len)
 * (RFC section 3.3: the recent BF16 tail is part of the cache).  k_tail / v_tail: BF16
 * [tail_len, H, D] at the final depth (each token's last-exited version); its tiles are
 * read as stored, in the same launch as the packed tiles.  Otherwise as
 * flk_decode_attn_packed; T + tail_len >= 1; workspace >= flk_attn_workspace_bytes(k_desc,
 * T + tail_len, n_q_heads).
 * Errors: those of flk_decode_attn_packed, plus FLK_E_NULL for a missing tail with
 * tail_len > 0.                                                                            */
flk_status flk_decode_attn_rolling(const flk_desc* k_desc, const flk_desc* v_desc, int32_t T, const void* q,
                                   int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                   int32_t n_loops, const void* k_tail, const void* v_tail, int32_t tail_len,
                                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------------------
 * Sparse decode attention (RFC section 3.2).  Loop 2 is the reference: it runs full attention
 * and keeps, per query head, the k keys with the highest reference probabilities (S, equal
 * scores by the lower position), their probability mass m, the full output O_ref and the
 * selected keys' weighted value sum C_ref.  A later loop r attends to the keys of S alone, read
 * from the packed chains at depth r, and corrects the reference output:
 *   p_local = softmax(scale * q_r . K_hat_r[S]),  O_r = O_ref - C_ref + m * (p_local . V_hat_r[S]).
 * Mass and accumulation are binary32 (RFC section 5).  Shapes as flk_decode_attn_packed (D ==
 * 128, n_q_heads / H <= 16); 1 <= k <= T; both calls take the packed chains of positions
 * [0, T) without a BF16 tail.
 * --------------------------------------------------------------------------------------- */

/* Workspace of both sparse calls for T packed tokens, n_q_heads query heads, k keys per head
 * and chains of at most n_loops loops (the reference call's scores take 4*T*n_q_heads bytes).
 * 0 for malformed arguments. */
size_t flk_sparse_workspace_bytes(const flk_desc* k_desc, int32_t T, int32_t n_q_heads, int32_t k, int32_t n_loops);

/* The reference loop over chains of n_loops loops (the reference depth).
 * q: BF16 [n_q_heads, D].  out: BF16 [n_q_heads, D], the reference loop's attention output.
 * sel: device int32 [n_q_heads, k], S in ascending position order.  mass: device float
 * [n_q_heads].  o_ref, c_ref: device float [n_q_heads, D].  All outputs.
 * Errors: those of flk_decode_attn_packed, plus FLK_E_SHAPE for k out of range.            */
flk_status flk_sparse_attn_reference(const flk_desc* k_desc, const flk_desc* v_desc, int32_t T, const void* q,
                                     int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                     int32_t n_loops, int32_t k, float softmax_scale, void* out, int32_t* sel,
                                     float* mass, float* o_ref, float* c_ref, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* A later loop over chains of n_loops loops (its depth).  q: BF16 [n_q_heads, D] of this loop;
 * sel, mass, o_ref, c_ref: the reference call's outputs (inputs here); out: BF16
 * [n_q_heads, D].  Entries of sel outside [0, T) are a precondition violation: they are
 * skipped.
 * Errors: those of flk_sparse_attn_reference.                                              */
flk_status flk_sparse_attn_loop(const flk_desc* k_desc, const flk_desc* v_desc, int32_t T, const void* q,
                                int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                int32_t n_loops, int32_t k, float softmax_scale, const int32_t* sel,
                                const float* mass, const float* o_ref, const float* c_ref, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* flk_sparse_attn_reference and flk_sparse_attn_loop over chains of FP4 streams (the PR #166
 * review, item 2, asks for the consumers' speed and accuracy with FP4 residual reconstruction
 * fused in; RFC section 3.2 for the method): the K chain's base loop is described by kd_base,
 * its residual loops by kd_resid, V likewise, with the combinations flk_decode_attn_mixed
 * accepts (INT4 throughout; an INT4 base with NVFP4 or MXFP4 residuals; NVFP4 or MXFP4
 * throughout; the same for K and V).  The keys the later loops gather are decoded from the
 * FP4 streams as flk_reconstruct decodes them.  The workspace is flk_sparse_workspace_bytes of
 * an INT4 descriptor with the same H and D (the size does not depend on the stream format).
 * Errors: those of the INT4 calls, plus FLK_E_DESC / FLK_E_UNSUPPORTED as for
 * flk_decode_attn_mixed. */
flk_status flk_sparse_attn_reference_mixed(const flk_desc* kd_base, const flk_desc* kd_resid,
                                           const flk_desc* vd_base, const flk_desc* vd_resid, int32_t T,
                                           const void* q, int32_t n_q_heads, const flk_stream* k_chain,
                                           const flk_stream* v_chain, int32_t n_loops, int32_t k,
                                           float softmax_scale, void* out, int32_t* sel, float* mass,
                                           float* o_ref, float* c_ref, void* workspace, size_t workspace_bytes,
                                           void* stream);
flk_status flk_sparse_attn_loop_mixed(const flk_desc* kd_base, const flk_desc* kd_resid, const flk_desc* vd_base,
                                      const flk_desc* vd_resid, int32_t T, const void* q, int32_t n_q_heads,
                                      const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops,
                                      int32_t k, float softmax_scale, const int32_t* sel, const float* mass,
                                      const float* o_ref, const float* c_ref, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Token selection for sparse prefill (RFC section 3.1, "Token-sparse prefill", and its fixed
 * selection windows; section 6.2 for the row partition).  Loops 1 and 2 run densely; before
 * loop r >= 3 every token active at loop r-1 gets the change score
 *   score = ||H[r-1] - H[r-2]|| / max(||H[r-1]||, eps)
 * and each selection window keeps its highest-scoring tokens, equal scores by the lower
 * position.  Windows are [w*window, min((w+1)*window, T)); a window's budget is
 * ceil(pct * len / 100) for its own length len (budgets refer to the original window, not to
 * the tokens still active), and never more than its tokens still active, so active sets are
 * nested.  The score is binary32: each difference, square, addition, the square roots and the
 * quotient are rounded once, and each sum of squares is taken in pairwise order (the complete
 * binary tree over the channel index, zero-padded to a power of two), so a score depends on
 * its row alone: not on the batch, the packing or the launch.  Nothing is read back to the host;
 * the counts the caller needs follow from T, window and the budgets (flk_select_count).
 * --------------------------------------------------------------------------------------- */

/* Tokens active after the budgets pct[0..n_budgets) are applied in turn, from a dense loop, to
 * every window (the n_out of the last of them).  -1 for a malformed argument (T < 0,
 * window < 1, a pct outside [0, 100], n_budgets < 0 or pct NULL with n_budgets > 0). */
int32_t flk_select_count(int32_t T, int32_t window, const int32_t* pct, int32_t n_budgets);

/* Workspace of flk_select_rows: 4 * (ceil(T / window) + 1) bytes rounded up to 256; 0 for a
 * malformed argument. */
size_t flk_select_workspace_bytes(int32_t T, int32_t window);

/* Loop r's active set from H[r-1] and H[r-2].
 * h_prev:    device BF16 [T, d], H[r-1] indexed by position; 16-byte aligned.
 * h_prev2:   device BF16 [T, d], H[r-2] (the rows active at loop r-1 kept from before that loop
 *            overwrote them; RFC: two aliases of one tensor give no change score); 16-byte
 *            aligned, not the same buffer as h_prev.
 * rows_prev: device int32 [n_prev], the positions active at loop r-1, strictly ascending in
 *            [0, T); NULL when loop r-1 was dense (then n_prev == T) or selected nothing
 *            (n_prev == 0).
 * window, pct: the selection window length (>= 1) and loop r's budget in percent (0..100).
 * eps:       a positive finite binary32.
 * scores:    device float [n_prev], written with the score of rows_prev[j] (or of position j)
 *            when 0 < pct < 100; pct 0 and 100 select without scores (the RFC asks that 100 %
 *            retention and all-off skip the selection work) and leave it untouched.
 * rows_out:  device int32 [n_out], written: loop r's active positions, ascending (may be NULL
 *            when n_out == 0).
 * n_out:     flk_select_count for this loop's budgets; if the windows' budgets add up to
 *            another number (rows_prev not made by the same budgets), FLK_DEV_COUNT is set and
 *            no entry at or past n_out is written.
 * slot:      optional device int32 [T], written: slot[p] = index of p in rows_out, else -1.
 * workspace: device, at least flk_select_workspace_bytes(T, window) bytes, 4-byte aligned.
 * dev_status: optional device uint32: FLK_DEV_NONFINITE when a score is not finite (inputs
 *            whose squares overflow), FLK_DEV_COUNT as above.
 * Errors: FLK_E_NULL, FLK_E_SHAPE (T < 1, d < 8, d % 8 != 0, d > 16384, T * d >= 2^31,
 * n_prev outside [0, T] or not 0 or T without rows_prev, window < 1, pct outside [0, 100],
 * n_out outside [0, n_prev], eps not positive and finite, h_prev == h_prev2), FLK_E_ALIGN,
 * FLK_E_WORKSPACE, FLK_E_LAUNCH.                                                           */
flk_status flk_select_rows(const void* h_prev, const void* h_prev2, int32_t T, int32_t d, const int32_t* rows_prev,
                           int32_t n_prev, int32_t window, int32_t pct, float eps, float* scores,
                           int32_t* rows_out, int32_t n_out, int32_t* slot, void* workspace,
                           size_t workspace_bytes, uint32_t* dev_status, void* stream);

/* Classes of a submission's execution rows for flk_partition_rows. */
enum { FLK_ROW_INACTIVE = 0, FLK_ROW_ACTIVE = 1, FLK_ROW_DECODE = 2 };

/* Gather indices of a mixed submission by stable partition (RFC section 6.2): the decode rows
 * in their order, then the active prefill rows in their order; inactive prefill rows are left
 * out (they keep their state).  E.g. [P0, D0, P1, P2, D1, P3] with P1 and P3 active gives
 * [D0, D1 | P1, P3] and the split offset 2.
 * cls:     device uint8 [n], FLK_ROW_* per row; another value counts as inactive and sets
 *          FLK_DEV_CLASS.
 * gather:  device int32 [n], written: entries [0, counts[1]) are row indices, the rest -1.
 * scatter: device int32 [n], written: the index of row i in gather, or -1.
 * counts:  device int32 [2], written: {decode rows (the split offset), gathered rows}.
 * One workgroup scans the rows, sized for a submission's rows (tens of thousands).
 * Errors: FLK_E_NULL, FLK_E_SHAPE (n < 0), FLK_E_LAUNCH.                                    */
flk_status flk_partition_rows(const uint8_t* cls, int32_t n, int32_t* gather, int32_t* scatter, int32_t* counts,
                              uint32_t* dev_status, void* stream);

/* ---------------------------------------------------------------------------------------
 * Batched calls.  A serving step encodes or rebuilds many tensors at once -- every layer's K
 * and V of a request, or of many requests -- and one kernel launch covering them avoids a
 * launch (and a ramp-up and drain of the GPU) per tensor; the RFC, section 6.2, asks for the
 * codec to join the runtime's batched submissions.  Each unit is one (request, layer, K or V)
 * tensor; units are independent and may differ in T, n_rows and kind.  The results are
 * exactly those of the single call applied to each unit.  No two units may write the same
 * buffer, except that units whose rows arrays are equal may share one tile_start array.
 * k_desc / v_desc describe every K / V unit (either may be NULL when no unit has that kind).
 * The unit tables are host memory; every unit is validated on the host before anything is
 * launched, so on an error nothing has been written.  n_units == 0 is a no-op.
 * --------------------------------------------------------------------------------------- */

/* One tensor of a batched encode; the pointers are device addresses as in the single calls. */
typedef struct flk_unit {
  const void* x;            /* BF16 [n_rows, H, D]: X[1] (base) or X[r] at the active rows    */
  const int32_t* rows;      /* ascending positions of a compact loop, NULL for a dense one     */
  void* recon;              /* BF16 [T, H, D]: written by a base, updated by a residual        */
  uint8_t* codes;           /* output stream of this loop                                     */
  uint32_t* params;
  int32_t* tile_start;      /* output tile index of a compact loop, else NULL                 */
  int32_t n_rows;           /* == T for a base or dense loop; 0 = an empty residual loop      */
  int32_t T;
  int32_t kind;             /* FLK_KIND_K or FLK_KIND_V                                       */
  int32_t reserved;         /* must be 0                                                      */
} flk_unit;

/* flk_encode_base for every unit (rows must be NULL and n_rows == T).
 * Errors: those of flk_encode_base for any unit, FLK_E_NULL for a NULL table or a missing
 * descriptor, FLK_E_DESC for a bad kind or reserved field, FLK_E_SHAPE for n_units < 0.     */
flk_status flk_encode_base_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_unit* units,
                                 int32_t n_units, uint32_t* dev_status, void* stream);

/* flk_encode_residual for every unit (dense and compact units may be mixed).
 * Errors: those of flk_encode_residual for any unit, plus those of flk_encode_base_batch.   */
flk_status flk_encode_residual_batch(const flk_desc* k_desc, const flk_desc* v_desc,
                                     const flk_unit* units, int32_t n_units, uint32_t* dev_status,
                                     void* stream);

/* One tensor of a batched reconstruct. */
typedef struct flk_recon_unit {
  const flk_stream* chain;  /* host array of n_loops streams, chain[0] the dense base         */
  void* out;                /* BF16 [T, H, D] output                                          */
  int32_t T;
  int32_t n_loops;
  int32_t kind;             /* FLK_KIND_K or FLK_KIND_V                                       */
  int32_t reserved;         /* must be 0                                                      */
} flk_recon_unit;

/* flk_reconstruct for every unit.
 * Errors: those of flk_reconstruct for any unit, plus those of flk_encode_base_batch.       */
flk_status flk_reconstruct_batch(const flk_desc* k_desc, const flk_desc* v_desc,
                                 const flk_recon_unit* units, int32_t n_units, void* stream);

/* One window of a batched append (the arguments of flk_append_base / flk_append_residual).
 * Loop 1 (flk_append_base_batch): rows NULL, n_rows == n_pos, rows_before == p0. */
typedef struct flk_append_unit {
  const void* x;            /* BF16 [n_rows, H, D]: X[1] of the window, or X[r] at its rows     */
  const int32_t* rows;      /* the window's row entries (absolute positions), NULL when dense   */
  void* recon;              /* BF16 [n_pos, H, D]: the window's reconstruction                  */
  uint8_t* codes;           /* the stream's buffers, at their start                             */
  uint32_t* params;
  int32_t* tile_start;      /* compact loops (and empty compact windows), else NULL             */
  int32_t n_rows;
  int32_t p0;               /* first position of the window, a multiple of 64                   */
  int32_t n_pos;            /* positions in the window, a multiple of 64                        */
  int32_t rows_before;      /* the stream's compact rows at positions < p0                      */
  int32_t kind;             /* FLK_KIND_K or FLK_KIND_V                                         */
  int32_t reserved;         /* must be 0                                                        */
} flk_append_unit;

/* The flush of a decode step that fills whole tiles of many tensors at once (every layer's
 * K and V of a request, or of several requests): flk_append_base / flk_append_residual for
 * every unit, in one launch per loop type where the shapes allow.
 * Errors: those of the single calls for any unit, plus those of flk_encode_base_batch.     */
flk_status flk_append_base_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_append_unit* units,
                                 int32_t n_units, uint32_t* dev_status, void* stream);
flk_status flk_append_residual_batch(const flk_desc* k_desc, const flk_desc* v_desc,
                                     const flk_append_unit* units, int32_t n_units, uint32_t* dev_status,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLK_H */
