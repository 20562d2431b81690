/*
 * moe.h -- C ABI of the quantized routed mixture-of-experts layer for AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes (the pages describe it in prose only):
 *   a router scores every token against E experts, keeps the top k, and a
 *   block-sparse kernel streams only the activated experts' quantised
 *   weights, dequantising them on the fly ("antirez ds4: DeepSeek Metal
 *   inference", ainews.cool, section 技术深度解析 -- 64 fine-grained experts,
 *   top-2 routing, custom dequantisation kernels); the routed count k is a
 *   run-time choice (Anemll/ds4-ssd README, section "Experimental Pro
 *   Support", --moe-expert-topk); experts come as native MXFP4 packs
 *   (ds4-ssd README, section "Run SSD Sidecar Mode") or 2-bit asymmetric
 *   packs ("DwarfStar 4 (ds4) | Mac Studio ... 完整指南", res.pawin.top,
 *   section on q2 asymmetric quantisation).
 *
 *   1. logits[t][e] = sum_i float(x[t][i]) * w_router[e][i] + bias[e]     (fp32)
 *   2. topk_ids[t][0..k) = the k largest logits, ordered by (logit desc,
 *      expert id asc); topk_w[t][j] = softmax over the k selected logits
 *   3. stable counting sort of the pairs p = t*k + j by topk_ids:
 *      offsets[E+1], perm[r] = pair at sorted row r, inv[p] = row of pair p
 *   4. for sorted row r of expert e, token t = perm[r] / k:
 *      act[r][n] = bf16_rne( silu(Wg[e][n,:] . x[t]) * (Wu[e][n,:] . x[t]) )
 *   5. y[r][m] = Wd[e][m,:] . act[r]                                          (fp32)
 *   6. out[t][m] = sum_{j=0..k-1} topk_w[t][j] * y[inv[t*k+j]][m]  (j order) (fp32)
 *
 * Entry points: moe_route_topk (1-2), moe_dispatch (3), moe_expert_ffn (4-5),
 * moe_combine (6) and moe_layer (1-6 in one call); moe_pack_qmat lays
 * weights out for the kernels.  Beside the layer: moe_layer_shared (an
 * always-on shared expert), moe_expert_ffn_mx8 / moe_layer_mx8 and
 * moe_expert_ffn_mx4 / moe_layer_mx4 (MXFP8 or MXFP4 activations on the
 * block-scaled matrix cores), and the slot bank
 * (moe_bank_reset / moe_bank_plan / moe_bank_fetch / moe_layer_banked:
 * N device expert slots paged from host memory).
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer (HBM of the current HIP
 *     device) unless stated otherwise; `moe_shape` / `moe_experts` structs are
 *     read on the host during the call and may be freed after it returns.
 *   - bf16 and fp16 values are passed as their uint16 bit patterns.
 *   - Row-major everywhere; the last index is contiguous.
 *   - Alignment: x, y, out, logits, every pack pointer and ws must be 16-byte
 *     aligned; int32 arrays 4-byte aligned.
 *   - The caller owns and allocates every buffer (inputs, outputs and the
 *     workspace).  The library allocates and frees nothing and keeps no
 *     mutable global state: calls on different streams with different
 *     buffers are independent.
 *   - Every call only ENQUEUES work on `stream` and returns; buffers must stay
 *     valid until the stream has passed that work.  Nothing synchronises the
 *     host except moe_read_device_status and moe_read_device_status_bits.
 *   - Host-side validation runs before any HIP call; a negative return code
 *     means nothing was enqueued.  The library never prints, aborts or throws.
 *   - T == 0 is valid and enqueues nothing.
 *
 * Shape limits: 1 <= k <= E <= 64; d and f positive multiples of 32;
 * T >= 0; T*k*max(d, f) < 2^31.
 */
#ifndef QUANTIZED_ROUTED_MOE_AMD_MOE_H
#define QUANTIZED_ROUTED_MOE_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (return values). */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* shape outside the limits above */
    MOE_ERR_FORMAT = -3,      /* unknown, mixed or mislaid pack format / layout */
    MOE_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
    MOE_ERR_WORKSPACE = -5,   /* ws_bytes < moe_workspace_bytes(shape) */
    MOE_ERR_UNSUPPORTED = -6, /* valid request the library cannot serve */
    MOE_ERR_HIP = -7,         /* a HIP call (launch, copy) failed */
    MOE_ERR_DEVICE = -8       /* a kernel flagged bad device data (see below) */
};

/* Device status bits, OR-ed into the workspace header by the kernels. */
enum moe_device_status_bits {
    MOE_DEV_BAD_EXPERT_ID = 1, /* a topk id outside [0, E) reached moe_dispatch */
    MOE_DEV_BAD_SLOT = 2,      /* slot_of_expert[e] outside [0, num_slots) for a routed e */
    MOE_DEV_CHAIN_TIMEOUT = 4  /* prefill FFN: a down tile gave up waiting for its gate/up tiles
                                  (its y rows then hold NaN, never a product of unfinished act rows) */
};

/* The single-launch prefill FFN (T*k >= 256 with d % 512 == 0 and
   f % 256 == 0, every pack format, and the MXFP8 / MXFP4-activation entry
   points) hands act from its gate/up
   tiles to its down tiles through ready flags with a bounded wait (about a
   third of a second).  A wait that gives up makes that tile's y rows NaN and
   raises MOE_DEV_CHAIN_TIMEOUT; a caller that must not consume such a
   result reads the status word (moe_read_device_status) after the call.
   Workspace header word 32 (bytes 128..131; zero after moe_workspace_init),
   when it holds w != 0, limits each wait to w - 1 polls (w = 1: give up at
   once): a test hook that forces the timeout path from the host. */

typedef struct moe_shape {
    int32_t T; /* tokens in the call */
    int32_t d; /* hidden size (model dimension) */
    int32_t E; /* routed experts */
    int32_t k; /* experts per token (top-k) */
    int32_t f; /* expert FFN (intermediate) size */
} moe_shape;

/* Expert weight pack formats (the quantisation of one row; the layout of the
   rows in memory is given separately by enum moe_layout). */
enum moe_format {
    /* MXFP4 (OCP Microscaling v1.0): 4-bit e2m1 codes, element 2i of a row in
       the LOW nibble of byte i, element 2i+1 in the HIGH nibble (bit 3 of a
       code is its sign); one e8m0 scale byte per 32 consecutive elements
       along K (value 2^(byte-127); byte 255 is not allowed). */
    MOE_FMT_MXFP4 = 1,
    /* 2-bit group-asymmetric: w = scale * q + min, q in {0,1,2,3}; element 4i+j
       of a row is bits (2j, 2j+1) of byte i; one fp16 scale and one fp16 min per
       32 consecutive elements along K. */
    MOE_FMT_Q2G32 = 2,
    /* 4-bit group-asymmetric: w = scale * q + min, q in {0..15}; element 2i
       of a row is the LOW nibble of byte i, element 2i+1 the HIGH nibble; one
       fp16 scale and one fp16 min per 32 consecutive elements along K (the
       4-bit "GPTQ-style" pack of "antirez ds4: DeepSeek Metal inference",
       section 技术深度解析, read as the affine form of the 2-bit pack). */
    MOE_FMT_Q4G32 = 3
};

/* Memory layouts of a quantised matrix of n rows x K elements per slot
   (n a multiple of 16, K a multiple of 32; G = K/32 groups per row).

   MOE_LAYOUT_ROWS -- the interchange layout (input of moe_pack_qmat only):
     MXFP4: codes uint8 [slots][n][K/2], scales uint8 [slots][n][G], mins NULL.
     Q2:    codes uint8 [slots][n][K/4], scales and mins fp16 bits
            uint16 [slots][n][G].
     Q4:    codes uint8 [slots][n][K/2], scales and mins fp16 bits
            uint16 [slots][n][G].

   MOE_LAYOUT_TILES -- the layout the expert FFN reads (moe_pack_qmat writes
   it).  Rows are cut into tiles of 16 and K into steps of 128 elements (four
   groups; S = ceil(K/128) steps, the groups past G of the last step are
   padding).  One (tile, step) block holds 64 "pieces"; piece L covers row
   16*tile + L%16.  Blocks are stored [slots][n/16][S] (step fastest), so
   one piece array of a block is contiguous and a 64-lane wave reads a
   whole block in one instruction.
     MXFP4: piece L = group 4*step + L/16 of its row:
            codes  [slots][n/16][S][64][16 B]  the group's 16 code bytes
                                                (padding: 0)
            scales [slots][n/16][S][64] uint8  its e8m0 scale (padding: 127)
            mins   NULL
     Q2:    codes  [slots][n/16][S][64][8 B]   elements 8g..8g+7 (g = L/16)
                                                of each of the step's four
                                                groups (padding: 0), as two
                                                little-endian uint32; word t
                                                holds groups a = 4*step+2t and
                                                b = a+1: bits 0-7 elements
                                                8g, 8g+2, 8g+4, 8g+6 of a (2
                                                bits each, ascending), bits
                                                8-15 the same of b, bits 16-23
                                                elements 8g+1, +3, +5, +7 of
                                                a, bits 24-31 the same of b
            scales [slots][n/16][S][16][4] uint32  row-major: word (r, j) =
                                                fp16 scale | fp16 min << 16 of
                                                row 16*tile + r, group
                                                4*step + j (padding 0)
            mins   NULL (the mins live in scales)
     Q4:    codes  [slots][n/16][S][64][16 B]  elements 8g..8g+7 (g = L/16)
                                                of each of the step's four
                                                groups (padding: 0), as four
                                                little-endian uint32; word j
                                                holds group 4*step+j: bits
                                                4h..4h+3 element 8g+2h and
                                                bits 16+4h..19+4h element
                                                8g+2h+1 (h = 0..3)
            scales as Q2
            mins   NULL (the mins live in scales)
   Sizes: moe_qmat_bytes. */
enum moe_layout {
    MOE_LAYOUT_ROWS = 0,
    MOE_LAYOUT_TILES = 1
};

/* One quantised matrix, n rows of K elements, for every slot. */
typedef struct moe_qmat {
    int32_t fmt;        /* enum moe_format */
    int32_t layout;     /* enum moe_layout */
    const void* codes;  /* device */
    const void* scales; /* device */
    const void* mins;   /* device; Q2 in MOE_LAYOUT_ROWS only, else NULL */
} moe_qmat;

/* Bytes of each array of a (fmt, layout) matrix of `slots` x n x K (any of
   the out pointers may be NULL).  Returns the total, or 0 (all outputs 0)
   when the request is invalid: unknown fmt or layout, slots < 1, n not a
   positive multiple of 16, K not a positive multiple of 32. */
size_t moe_qmat_bytes(int32_t fmt, int32_t layout, int32_t slots, int32_t n, int32_t K,
                      size_t* codes_bytes, size_t* scales_bytes, size_t* mins_bytes);

/* Re-lays `src` (MOE_LAYOUT_ROWS) into `dst` (MOE_LAYOUT_TILES, same fmt,
   arrays of moe_qmat_bytes size, caller-allocated, not overlapping src) on
   `stream`: a bit-exact copy of every code, scale and min.  Meant to run once
   when the weights are loaded.  Errors: MOE_ERR_NULL, MOE_ERR_FORMAT (fmt or
   layout mismatch), MOE_ERR_SHAPE (as moe_qmat_bytes), MOE_ERR_ALIGN (codes
   16-byte, scales and mins 4-byte aligned), MOE_ERR_HIP. */
int moe_pack_qmat(const moe_qmat* src, const moe_qmat* dst, int32_t slots, int32_t n, int32_t K,
                  hipStream_t stream);

/* The experts of one layer.  gate and up are n=f rows of K=d; down is n=d
   rows of K=f.  All three use the same format and MOE_LAYOUT_TILES.  Expert e lives in pack slot
   slot_of_expert[e] (device int32 [E]) or, when slot_of_expert is NULL, in
   slot e (then num_slots >= E is required).
   slot_of_expert[e] == MOE_SLOT_SKIP leaves expert e out of the call and
   raises no status.  moe_expert_ffn / moe_expert_ffn_mx8 then leave its y
   rows untouched (a slot-bank pass that computes other experts, y filling
   up over several calls); the one-call layers (moe_layer, moe_layer_shared,
   moe_layer_mx8) treat it as contributing zero (its y rows are zeroed, or
   with the combine fused into the down projection nothing is added).
   A routed expert whose slot is otherwise outside [0, num_slots) is not
   computed: its y rows are written as zeros and MOE_DEV_BAD_SLOT is raised.

   Slot placement: with slot_bytes == 0 every array holds its slots back to
   back (slot s of an array starts s * (its moe_qmat_bytes for one slot)
   bytes past its pointer).  With slot_bytes != 0 (a multiple of 256) slot s
   of EVERY array starts s * slot_bytes bytes past that array's pointer: the
   six arrays of one expert can then share one contiguous slab per slot
   (moe_slab_layout), which the slot bank copies in one transfer. */
enum { MOE_SLOT_SKIP = -2 };
typedef struct moe_experts {
    moe_qmat gate, up, down;
    const int32_t* slot_of_expert;
    int32_t num_slots;
    uint64_t slot_bytes;      /* 0, or the stride between slots of every array (slabs) */
} moe_experts;

/* Slab layout of one expert of format fmt (hidden size d, expert size f):
   the byte offsets of its six tile-layout arrays inside one slab, in the
   order gate codes, gate scales, up codes, up scales, down codes, down
   scales (offsets[6], HOST; may be NULL), each a multiple of 256.  Returns
   the slab size (a multiple of 256) -- the moe_experts.slot_bytes of a slab
   pack whose array pointers are base + offsets[i] -- or 0 for an invalid
   request (unknown fmt; d or f not a positive multiple of 32). */
size_t moe_slab_layout(int32_t fmt, int32_t d, int32_t f, size_t* offsets);

/* Workspace bytes moe_dispatch / moe_expert_ffn / moe_layer need for `shape`
   (a 256-byte header holding the device status word, then the bf16 SwiGLU
   intermediate act[T*k][f], then, when f % 256 == 0, the ready flags of the
   single-launch prefill FFN: 8 bytes per 128-row m-tile and 256 rows of f,
   for the ceil(T*k/128) + min(E, T*k) m-tiles there can be, that count
   rounded up to a multiple of 4; every
   launch writes a value of its own into them, so they never need clearing;
   then, for shapes that take that launch (T*k >= 256, d % 512 == 0,
   f % 256 == 0), the per-32-element group sums the 2-bit and 4-bit packs'
   launch uses for their min term: u32 [T][d/32] and [T*k][f/32], each word
   the sum as two fp16 halves, so a group's sum must stay below 65504 in
   magnitude -- beyond it the outputs become NaN, never finite and wrong).
   Returns 0 for an invalid shape.  The header must be zeroed once before
   first use (moe_workspace_init does it).  A workspace serves one call at a
   time: calls that overlap on one workspace race. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Clears the workspace header (device status word) on `stream`. */
int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1-2.  x bf16 [T][d]; w_router fp32 [E][d]; bias fp32 [E] or NULL.
   If w_router != NULL the logits are computed and written to logits fp32
   [T][E]; if w_router == NULL, logits is an INPUT (given router logits) and
   bias must be NULL.  Logits must be finite (NaN gives unspecified routing).
   Out: topk_ids int32 [T][k] in selection order, topk_w fp32 [T][k].
   Ties between equal logits go to the lower expert id; -0.0 == +0.0. */
int moe_route_topk(const moe_shape* shape, const uint16_t* x, const float* w_router,
                   const float* bias, float* logits, int32_t* topk_ids, float* topk_w,
                   hipStream_t stream);

/* Step 3.  topk_ids int32 [T][k] (any source).  Out: offsets int32 [E+1]
   (offsets[0] = 0, offsets[E] = number of valid pairs = T*k when all ids are
   valid), perm int32 [T*k], inv int32 [T*k].  Pairs of one expert keep
   ascending pair order (stable).  Ids outside [0, E) raise
   MOE_DEV_BAD_EXPERT_ID and are sorted after every valid pair.  Uses the
   workspace header only. */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_ids, int32_t* offsets,
                 int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps 4-5.  x bf16 [T][d]; offsets/perm as produced by moe_dispatch.
   Out: y fp32 [T*k][d] in sorted-row order (rows at or past offsets[E] are
   zero).  The bf16 intermediate act lives in ws.  Only experts with at least
   one row are read from HBM. */
int moe_expert_ffn(const moe_shape* shape, const uint16_t* x, const moe_experts* experts,
                   const int32_t* offsets, const int32_t* perm, float* y, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* Step 6.  y fp32 [T*k][d], inv int32 [T*k], topk_w fp32 [T][k].
   Out: out fp32 [T][d].  Fixed summation order j = 0..k-1 (deterministic). */
int moe_combine(const moe_shape* shape, const float* y, const int32_t* inv,
                const float* topk_w, float* out, hipStream_t stream);

/* Steps 1-6 in one call; identical (bit for bit) to moe_route_topk,
   moe_dispatch, moe_expert_ffn and moe_combine in sequence.  offsets, perm,
   inv and y are carved from `ws`, which must hold
   moe_layer_workspace_bytes(shape) bytes. */
size_t moe_layer_workspace_bytes(const moe_shape* shape);
int moe_layer(const moe_shape* shape, const uint16_t* x, const float* w_router,
              const float* bias, float* logits, const moe_experts* experts,
              int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* ---- moe_layer without a workspace argument, for callers that cannot
   allocate: code under HIP graph capture, tight serving loops, harnesses
   that forbid hipMalloc.

   The same computation and launches as moe_layer (identical results), with
   the workspace taken from a file-scope device array of
   MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
   the process ends.  The call allocates nothing (no hipMalloc, hipFree or
   allocating library routine); its first call on a device looks the
   array's address up once.  Shapes whose moe_layer_workspace_bytes exceed
   MOE_NOALLOC_SCRATCH_BYTES are rejected with MOE_ERR_WORKSPACE (at
   d = 4096, f = 2048, k = 2 that is about 400 tokens: decode, verify and
   short batches, not a 2048-token prefill chunk -- use moe_layer there).
   status: DEVICE uint32 (4-byte aligned) into which device-detected faults
   are OR-ed as by the workspace status word (see moe_device_status_bits;
   the caller zeroes it and reads it after the call), or NULL to ignore
   them.  Every call on one GPU shares that GPU's array: calls that overlap
   on one GPU (on different streams or host threads) race.  Nothing in the
   array needs to start at zero.  Other arguments and errors as moe_layer. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int moe_layer_noalloc(const moe_shape* shape, const uint16_t* x, const float* w_router,
                      const float* bias, float* logits, const moe_experts* experts,
                      int32_t* topk_ids, float* topk_w, float* out, uint32_t* status,
                      hipStream_t stream);

/* ---- MXFP8 activations: the block-scaled fp4 x fp8 matrix cores.

   A faster mode that changes the rounding points, as the pages' engine
   keeps fast reduced-precision accelerator paths beside a switch that
   turns them off for quality (Anemll/ds4-ssd README, section "Experimental
   Pro Support": --no-int8 / --quality).  The token rows and the SwiGLU
   output are quantised to MXFP8 (OCP Microscaling Formats v1.0: E4M3
   elements, one E8M0 scale per 32 along the contraction axis, the scale
   2^(floor(log2 amax) - 8), elements rounded to nearest even and saturated
   at 448) instead of being kept in / rounded to bf16; MXFP4 weights and
   MXFP8 activations then meet in the gfx950 32x32x64 block-scaled matrix
   instruction with fp32 accumulation.  Steps 4-5 become
     xq[r] = MXFP8(x[perm[r] / k]),  act_q[r] = MXFP8(silu(Wg xq[r]) * (Wu xq[r])),
     y[r]  = Wd act_q[r]                                              (fp32)
   MXFP4 weights only, and shapes the grouped FFN takes (d % 512 == 0,
   f % 256 == 0); otherwise MOE_ERR_UNSUPPORTED.  Arguments as
   moe_expert_ffn / moe_layer; the workspace also holds the quantised rows
   (moe_workspace_bytes_mx8, moe_layer_mx8_workspace_bytes): after a call,
   act_q codes u8 [T*k][f] start at byte 256 of ws. */
size_t moe_workspace_bytes_mx8(const moe_shape* shape);
int moe_expert_ffn_mx8(const moe_shape* shape, const uint16_t* x, const moe_experts* experts,
                       const int32_t* offsets, const int32_t* perm, float* y, void* ws,
                       size_t ws_bytes, hipStream_t stream);
size_t moe_layer_mx8_workspace_bytes(const moe_shape* shape);
int moe_layer_mx8(const moe_shape* shape, const uint16_t* x, const float* w_router,
                  const float* bias, float* logits, const moe_experts* experts,
                  int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* ---- MXFP4 activations: the block-scaled fp4 x fp4 matrix cores.

   The same mode as the MXFP8 calls above with E2M1 activations (the other
   activation format the gfx950 block-scaled instruction takes beside E4M3,
   at twice its rate): the token rows and the SwiGLU output are quantised to
   MXFP4 (OCP Microscaling Formats v1.0: E2M1 elements, one E8M0 scale per
   32 along the contraction axis, the scale 2^(floor(log2 amax) - 2),
   elements rounded to nearest, ties to even, magnitudes above 6 clamped to
   6, zero stored as +0).  Steps 4-5 become
     xq[r] = MXFP4(x[perm[r] / k]),  act_q[r] = MXFP4(silu(Wg xq[r]) * (Wu xq[r])),
     y[r]  = Wd act_q[r]                                              (fp32)
   E2M1 keeps one mantissa bit: out moves by tens of per cent (relative L2)
   from the bf16 layer; parity is against the oracle's MXFP4 layer.  Shapes,
   formats, arguments and errors as the MXFP8 calls; after a call, act_q
   codes u8 [T*k][f/2] (two per byte, the even column in the low nibble)
   start at byte 256 of ws. */
size_t moe_workspace_bytes_mx4(const moe_shape* shape);
int moe_expert_ffn_mx4(const moe_shape* shape, const uint16_t* x, const moe_experts* experts,
                       const int32_t* offsets, const int32_t* perm, float* y, void* ws,
                       size_t ws_bytes, hipStream_t stream);
size_t moe_layer_mx4_workspace_bytes(const moe_shape* shape);
int moe_layer_mx4(const moe_shape* shape, const uint16_t* x, const float* w_router,
                  const float* bias, float* logits, const moe_experts* experts,
                  int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* ---- Shared expert: one always-on SwiGLU expert beside the routed ones.

   DeepSeek blocks add a shared expert that every token passes through; the
   pages name it only through a decode knob that prefetches its down
   projection (Anemll/ds4-ssd README, section "Experimental Pro Support",
   shared-down decode prefetch).  Reading taken: weight 1, same SwiGLU and
   rounding points as a routed expert, added after the routed terms:
     out[t][m] = sum_{j<k} topk_w[t][j] * y[inv[t*k+j]][m] + ys[t][m]
     ys[t] = Wd_s . bf16_rne( silu(Wg_s . x[t]) * (Wu_s . x[t]) )
   `shared` is a pack of the same format and layout as `experts` (slot 0 is
   used; its slot_of_expert is ignored).  Its rows are computed in the same
   launches as the routed experts' (its T rows follow the T*k routed rows in
   act and y, and its down weights are prefetched with theirs at decode).
   The workspace is moe_layer_shared_workspace_bytes(shape) (offsets, perm,
   inv and y carved from it).  Errors: as moe_layer, plus MOE_ERR_FORMAT /
   MOE_ERR_NULL / MOE_ERR_ALIGN for the shared pack. */
size_t moe_layer_shared_workspace_bytes(const moe_shape* shape);
int moe_layer_shared(const moe_shape* shape, const uint16_t* x, const float* w_router,
                     const float* bias, float* logits, const moe_experts* experts,
                     const moe_experts* shared, int32_t* topk_ids, float* topk_w, float* out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Slot bank: N < E resident expert slots in HBM, paged from a host pool.

   The pages' SSD sidecar keeps the routed experts outside the dense model
   and pages them through a bounded cache of expert slots, whose size trades
   memory for fewer reads (Anemll/ds4-ssd README, sections "Run SSD Sidecar
   Mode": --moe-slot-bank caps the resident routed-expert slots, --ssd-cache
   sizes the bank in bytes; the 10100.com article on ds4-ssd, section 核心功能:
   routed experts paged through a slot-bank cache).  Here the pool of all E
   experts sits in pinned host memory (standing in for the sidecar files) and
   the bank is a moe_experts pack of num_slots slots in HBM; misses are copied
   host -> device by the DMA engines.  The pages name no replacement policy;
   this library evicts the least recently used slot.

   moe_bank is host-side bookkeeping; the caller allocates its arrays (and,
   for copies that overlap the expert FFN, a copy stream and two events). */
typedef struct moe_bank {
    int32_t E;                /* experts in the pool, 1..64 */
    int32_t num_slots;        /* N, 1..E: slots of the device bank */
    int32_t* slot_of_expert;  /* HOST int32 [E]: slot holding expert e, or -1 */
    int32_t* expert_of_slot;  /* HOST int32 [N]: expert held by slot s, or -1 (empty) */
    uint64_t* last_use;       /* HOST uint64 [N]: request stamp of the slot's last use */
    uint64_t clock;           /* request stamps handed out so far */
    /* moe_layer_banked only.  NULL: the copies run on the call's stream, in
       order with its kernels.  Otherwise the copies run on copy_stream (a
       stream of the same device, default priority), and ev_copied /
       ev_computed (events created by the caller, e.g. hipEventCreateWithFlags
       with hipEventDisableTiming) order them against the FFN launches:
       the FFN of a pass's resident experts runs while its misses are
       copied, and copies into a slot wait for the FFN that last read it. */
    hipStream_t copy_stream;
    hipEvent_t ev_copied;
    hipEvent_t ev_computed;
} moe_bank;

/* Slots of a bank sized like the pages' --ssd-cache: a byte budget, or
   `auto` (budget_bytes == 0) from the memory still free, clamped so that the
   largest call the caller will make (prefill_shape, e.g. a prefill chunk)
   still finds its layer workspace:
     avail = free_bytes - reserve_bytes - moe_layer_workspace_bytes(prefill_shape)
     bytes = budget_bytes ? min(budget_bytes, avail) : avail
     *num_slots = min(prefill_shape->E, bytes / moe_slab_layout(fmt, d, f, NULL))
   free_bytes is the caller's reading of free device memory (hipMemGetInfo);
   reserve_bytes covers the caller's other buffers of that call (x, out,
   logits ...).  HOST only, no HIP call.  Errors: MOE_ERR_NULL,
   MOE_ERR_SHAPE / MOE_ERR_FORMAT (invalid shape or fmt), MOE_ERR_WORKSPACE
   (not even one slot fits; *num_slots = 0). */
int moe_bank_slots(int32_t fmt, const moe_shape* prefill_shape, uint64_t budget_bytes, uint64_t free_bytes,
                   uint64_t reserve_bytes, int32_t* num_slots);

/* Empties the bank (every slot -1, stamps and clock 0).  Errors:
   MOE_ERR_NULL, MOE_ERR_SHAPE (E outside 1..64, N outside 1..E). */
int moe_bank_reset(moe_bank* bank);

/* Plans one pass over the distinct experts want[0..n_want) (HOST int32,
   ids in [0, E), no repeats, n_want <= num_slots):
     - a wanted expert already resident is a hit;
     - each miss, in `want` order, takes the lowest-numbered empty slot, else
       the least recently used slot whose expert is not wanted in this pass
       (the evicted expert's slot_of_expert becomes -1);
     - then every wanted expert's slot is stamped ++clock, in `want` order.
   Out (HOST): load_expert / load_slot int32 [n_want], the misses in order,
   and *n_load, their count.  The bank state is updated; the copies are the
   caller's (moe_bank_fetch).  Errors (bank unchanged): MOE_ERR_NULL,
   MOE_ERR_SHAPE (n_want outside 0..num_slots, an id outside [0, E) or
   repeated). */
int moe_bank_plan(moe_bank* bank, const int32_t* want, int32_t n_want, int32_t* load_expert,
                  int32_t* load_slot, int32_t* n_load);

/* Enqueues on `stream` the host -> device copies of the planned loads:
   expert load_expert[i] of `pool` into slot load_slot[i] of `slots`, for
   i < n_load (HOST arrays), every array of gate, up and down.  pool: the
   packs of all E experts in HOST memory (pinned, e.g. hipHostMalloc, for
   asynchronous DMA; num_slots = E, slot_of_expert NULL); slots: the device
   bank (num_slots = N); same fmt, MOE_LAYOUT_TILES, hidden size d and
   expert size f.  When both packs are slab packs of the same layout
   (slot_bytes == moe_slab_layout(fmt, d, f, offsets) and every array at
   gate.codes + offsets[i]), each load is ONE copy of the whole slab;
   otherwise six (codes and scales of each matrix).  Errors: MOE_ERR_NULL,
   MOE_ERR_SHAPE, MOE_ERR_FORMAT, MOE_ERR_HIP. */
int moe_bank_fetch(const moe_experts* pool, const moe_experts* slots, int32_t d, int32_t f,
                   const int32_t* load_expert, const int32_t* load_slot, int32_t n_load,
                   hipStream_t stream);

/* Counters of one moe_layer_banked call (HOST). */
typedef struct moe_bank_stats {
    int32_t active;           /* distinct routed experts */
    int32_t hits;             /* of them already resident */
    int32_t misses;           /* paged in */
    int32_t passes;           /* FFN passes (ceil(active / N), at least 1) */
    int64_t bytes_paged;      /* host -> device bytes enqueued */
} moe_bank_stats;

/* moe_layer over a slot bank.  Every argument is validated first (nothing
   is enqueued and the bank is unchanged on an error).  Routes and
   dispatches on the device, then SYNCHRONISES `stream` to read the
   per-expert row counts.  The active experts, resident ones first, then in
   id order, are split into passes of at most N; each pass plans
   (moe_bank_plan) and pages its misses in (moe_bank_fetch).  Its resident
   experts' FFN (moe_expert_ffn on the bank with `slot_map`, DEVICE int32
   [E], holding only their slots) runs first, then -- once the copies have
   landed -- its misses' FFN; one combine follows.  Without a copy stream
   all of it is enqueued on `stream` in that order; with one (moe_bank) the
   copies overlap the resident experts' FFN, and a pass's copies wait for
   the previous pass's FFN (they may overwrite the slots it reads).  `slots`
   is the device bank (its slot_of_expert is ignored); `ws` as for
   moe_layer.  Results equal moe_layer's bit for bit (an expert's rows do
   not depend on its slot or pass).  stats may be NULL.  If a HIP call fails
   midway, MOE_ERR_HIP is returned and the bank is reset (moe_bank_reset):
   its books no longer claim slots whose copies may not have run. */
int moe_layer_banked(const moe_shape* shape, const uint16_t* x, const float* w_router,
                     const float* bias, float* logits, const moe_experts* pool, moe_bank* bank,
                     const moe_experts* slots, int32_t* slot_map, int32_t* topk_ids, float* topk_w,
                     float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                     moe_bank_stats* stats);

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(int status);

/* Synchronises `stream`, then reads the workspace's device status word.
   Returns MOE_OK, MOE_ERR_DEVICE (some bit set) or MOE_ERR_HIP;
   MOE_ERR_NULL / MOE_ERR_ALIGN for a null or misaligned ws.  The word stays
   set until moe_workspace_init. */
int moe_read_device_status(const void* ws, hipStream_t stream);
/* The same, also storing the word (the MOE_DEV_* bits) in *bits when
   bits != NULL. */
int moe_read_device_status_bits(const void* ws, uint32_t* bits, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QUANTIZED_ROUTED_MOE_AMD_MOE_H */
