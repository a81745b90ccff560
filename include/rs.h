/*
 * rs.h — RaggedShard / DBuffer layout transforms on one MI355X (gfx950).
 *
 * A group of N tensors shares one flat buffer of V*S elements; logical rank k
 * owns the slice [k*S, (k+1)*S). Tensor i occupies the contiguous interval
 * [s_i, s_i + n_i); intervals are disjoint and padding lives only between
 * them; a rank boundary that falls inside a tensor falls between two of its
 * atomic blocks ("veScale-FSDP: flexible, structure-aware sharding at
 * 10K-GPU scale", feynmanwiki walkthrough: the paragraphs on RaggedShard's
 * forbidden cut and on the planner as a packing problem). The V ranks are
 * slices of one GPU buffer: nothing here runs a collective.
 *
 * Calls (all extern "C", all return rs_status unless noted):
 *   rs_plan_build       host planner: S and the starts s_i
 *   rs_plan_load        validate a plan and lower it to device work lists
 *   rs_plan_info / rs_plan_free
 *   rs_unpack_gathered  gathered flat buffer -> N full tensors
 *   rs_pack_scatter     N full gradients -> flat buffer, fused scale/add/zero
 *   rs_block_quant      per-block absmax 8-bit quantisation of the flat buffer
 *   rs_block_quant_noalloc  the same from the plan as data, with its work list
 *                       in static device memory (no allocation)
 *   rs_block_dequant    the inverse of rs_block_quant
 *   rs_unpack_dequant   gathered codes + scales -> the quantised full tensors
 *   rs_adam8_step       one AdamW step on block-quantised int8 / uint8 state
 *   rs_last_error       text of the calling thread's last error
 *
 * Conventions
 *   - Sizes and offsets are in elements unless a name says bytes; all int64.
 *   - Device pointers come from the caller (e.g. torch tensors' data_ptr())
 *     and stay owned by the caller. The library owns rs_plan and the device
 *     tables it allocates once in rs_plan_load; no transform call allocates.
 *     rs_block_quant_noalloc allocates nothing at all: its work list goes
 *     into a static device array.
 *   - `stream` is a hipStream_t passed as void* (torch's current stream on
 *     ROCm). Transform calls are asynchronous and ordered on that stream.
 *   - Every check happens before any launch: on error nothing is enqueued,
 *     the status is returned and rs_last_error() says why. No C++ exception
 *     crosses this boundary.
 *   - A plan caches the per-tensor pointer tables it last saw and uploads a
 *     new table on `stream` only when they change; kernels read the table
 *     when they run. The upload is ordered with the work on `stream` only.
 *     A plan is therefore not safe to use from two threads at once; and when
 *     its calls go to more than one stream, a call with new tensor pointers
 *     must be ordered after every earlier call on the other streams, and the
 *     later calls on other streams after it (an event or a synchronisation).
 *   - HIP graphs: the transform calls may be captured (hipStreamBeginCapture
 *     on `stream`) once a call with the same tensor pointers has run outside
 *     the capture and is ordered before the replays. The graph then holds
 *     kernel launches only; they read the plan's pointer table when they run.
 *     A call whose pointers differ from the plan's last call returns
 *     RS_EINVAL while its stream is capturing, and launches nothing. Calls
 *     with other pointers between replays change the tables the replays
 *     read: keep them fixed while such a graph is in use, or use a second
 *     plan for other tensors.
 *   - Floating-point inputs must be finite; NaN or Inf inside a quantisation
 *     block gives unspecified codes (padding is never read, so it may hold
 *     anything).
 */
#ifndef RS_H
#define RS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rs_status {
  RS_OK = 0,
  RS_EINVAL = -1,   /* bad argument: null pointer, n < 1, V < 1, unknown enum ... */
  RS_EPLAN = -2,    /* the plan breaks a constraint, or no plan exists */
  RS_EALIGN = -3,   /* a pointer is not 16-byte aligned, or S / a start not a multiple of 16 */
  RS_EDTYPE = -4,   /* dtype or code format not supported by this call */
  RS_ENOMEM = -5,   /* host or device allocation failed (rs_plan_load only) */
  RS_EHIP = -6,     /* a HIP runtime call or a kernel launch failed */
  RS_ERANGE = -7    /* int64 overflow, or R_mat outside [R_used, V] */
} rs_status;

typedef enum rs_dtype {
  RS_F32 = 0,
  RS_BF16 = 1,
  RS_E4M3 = 2,      /* OCP FP8 E4M3 (largest finite 448, no infinities) */
  RS_I8 = 3,        /* signed, symmetric [-127, 127] */
  RS_U8 = 4         /* unsigned [0, 255] */
} rs_dtype;

/* Atomic block of a tensor: the unit a rank boundary may never cut
 * (feynmanwiki walkthrough, RaggedShard paragraphs: one element, rows, or a
 * larger custom block). The flat block size g follows from the kind:
 *   RS_ELEM        one element                        g = 1
 *   RS_ROWS(k)     k whole rows                       g = k * cols
 *   RS_TILE(br,bc) br x bc tiles of the row-major tensor; a rank boundary may
 *                  only fall between br-row bands (the walkthrough's 8-bit
 *                  Adam: 32x32 blocks at 32-row granularity)   g = br * cols
 *   RS_FLAT(b)     b consecutive elements             g = b
 *   RS_WHOLE       the whole tensor (one matrix per rank, as Muon wants)
 *                                                     g = rows * cols
 *   RS_TILEMAJOR(br,bc) br x bc tiles stored tile by tile: in the flat buffer
 *                  the tensor is its tiles in tile-row-major order, each tile
 *                  contiguous and row-major inside, so a rank boundary may
 *                  fall between any two tiles (the walkthrough's 2-D blocks
 *                  distributed asymmetrically)           g = br * bc
 *                  Needs rows % br == 0, cols % bc == 0, br*bc % 16 == 0 and
 *                  bc <= 8192. Unpack and pack reorder between this layout and
 *                  the row-major tensor (staged through LDS on the GPU).
 * The last block of a tensor may be partial. TILE, TILEMAJOR and FLAT
 * tensors are the ones rs_block_quant quantises (tiles / flat blocks); the
 * others are not. */
typedef enum rs_block_kind {
  RS_ELEM = 0, RS_ROWS = 1, RS_TILE = 2, RS_FLAT = 3, RS_WHOLE = 4, RS_TILEMAJOR = 5
} rs_block_kind;

/* One tensor of the group. A 1-D tensor of n elements is rows = n, cols = 1.
 * p0: ROWS k, TILE br, FLAT b; p1: TILE bc; unused fields must be 0.
 * Limits: rows * cols <= 2^40; a tile (br * bc) or a flat block (b) holds at
 * most 2^24 elements. */
typedef struct rs_tensor_spec {
  int64_t rows;
  int64_t cols;
  int32_t kind;      /* rs_block_kind */
  int32_t reserved;  /* must be 0 */
  int64_t p0;
  int64_t p1;
} rs_tensor_spec;

typedef struct rs_plan rs_plan;   /* opaque, owned by the library */

enum { RS_ORDER_BEST = 0, RS_ORDER_DEFAULT = 1, RS_ORDER_BLOCK_SIZE = 2, RS_ORDER_SHAPE = 3 };
enum { RS_ORDER_KIND_DEFAULT = 0, RS_ORDER_KIND_BLOCK = 1, RS_ORDER_KIND_SHAPE = 2 };

/* Host planner (feynmanwiki walkthrough: the planner paragraphs on the
 * tensor order, on one candidate per-device size and on the search over
 * sizes; bud-325 summary, Method (2)).
 * For each tensor order tried — the caller's order, block size descending,
 * shape descending (element count, then rows), all stable — find the
 * smallest S that is a multiple of `align` and at least
 *   LB = align_up(max(ceil(sum n_i / V), max_i min(g_i, n_i)), align)
 * for which placing each tensor at its earliest valid start after the
 * previous tensor's end fits inside V*S. Keep the order with the smallest S,
 * then the smallest end max(s_i + n_i), then the one listed first.
 * policy: RS_ORDER_BEST tries the three orders; RS_ORDER_DEFAULT,
 * RS_ORDER_BLOCK_SIZE or RS_ORDER_SHAPE plans with that one order (to compare
 * the orders). align >= 1 (16 for plans that rs_plan_load accepts).
 * Outputs (caller-owned host arrays): *S_out; starts_out[n] in the caller's
 * tensor order; order_out[n] the placement order (a permutation of 0..n-1);
 * *order_kind_out one of RS_ORDER_KIND_*. order_out / order_kind_out may be
 * NULL. Host only: touches no GPU.
 * Errors: RS_EINVAL (null, n < 1, V < 1, align < 1, bad spec), RS_ERANGE
 * (int64 overflow). */
int rs_plan_build(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t align,
                  int32_t policy, int64_t* S_out, int64_t* starts_out,
                  int64_t* order_out, int32_t* order_kind_out);

/* Validate a plan and build its device work lists on `device` (the pages'
 * persistent per-tensor address mapping, made once).
 * R_mat: number of rank slices actually allocated by the caller, with
 * R_used = ceil(max(s_i + n_i) / S) <= R_mat <= V; ranks at or past R_mat
 * hold only padding and are never touched.
 * Checks (RS_EPLAN unless noted): S > 0 and S % 16 == 0 and every
 * s_i % 16 == 0 (RS_EALIGN); intervals disjoint and inside [0, V*S); no
 * rank boundary inside a tensor except at a multiple of g_i from s_i;
 * R_mat in [R_used, V] (RS_ERANGE); V*S fits int64 (RS_ERANGE);
 * R_mat*S <= 2^39 elements and fewer than 2^32 work items per launch
 * (RS_ERANGE; neither limit is reached by a group one device can hold).
 * Environment read here, once per plan: RS_E4M3_ENCODER=sw selects the
 * integer E4M3 encoder instead of gfx950's conversion instruction;
 * RS_TM_KERNEL=direct runs the tile-major reorder of unpack / pack with
 * direct per-lane kernels instead of staging it through LDS. Both give
 * identical results.
 * On success *out owns host memory and one device allocation, released by
 * rs_plan_free. Errors: the above, RS_ENOMEM, RS_EHIP. */
int rs_plan_load(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                 const int64_t* starts, int64_t R_mat, int32_t device, rs_plan** out);

/* Plan facts; any output pointer may be NULL. n_qblocks is the number of
 * quantisation blocks, i.e. the length of rs_block_quant's scale array:
 * tensors in the caller's order; within a TILE tensor its tiles row-major,
 * within a FLAT tensor its blocks in order. padding_elems counts the
 * positions of [0, R_mat*S) that belong to no tensor. */
int rs_plan_info(const rs_plan* plan, int64_t* R_used, int64_t* n_qblocks,
                 int64_t* padding_elems);

void rs_plan_free(rs_plan* plan);   /* NULL is a no-op; waits for the device */

/* Unpack after the (simulated) AllGather: T_i[e] = gathered[s_i + e] for
 * every tensor i and 0 <= e < n_i, bit for bit (for a TILEMAJOR tensor,
 * element (r, c) is read from its place in its tile) (feynmanwiki walkthrough,
 * DBuffer paragraphs: a tensor is its planned slice; this call does the
 * Copy-Out of FSDP2's Copy-Out / Copy-In paragraph in one launch).
 * gathered: device, R_mat*S elements of `dt`, 16-byte aligned.
 * dst: HOST array of n device pointers, each a contiguous row-major tensor of
 * n_i elements of `dt`, 16-byte aligned. dt: RS_F32, RS_BF16 or any 1-byte
 * dtype (RS_E4M3 / RS_I8 / RS_U8). Padding of `gathered` is never read.
 * Errors: RS_EINVAL, RS_EALIGN, RS_EDTYPE, RS_EHIP. */
int rs_unpack_gathered(rs_plan* plan, const void* gathered, int32_t dt,
                       void* const* dst, void* stream);

enum { RS_SCALE_INV_V = 0, RS_SCALE_GIVEN = 1 };

/* Pack before the (simulated) ReduceScatter, with the group-fused pre-
 * communication ops (feynmanwiki walkthrough, DBuffer paragraph on add,
 * scale, zero and copy fused at group level):
 *   sigma = fl32(1/V) for RS_SCALE_INV_V, else `scale`;
 *   y = fl32(src_i[e] * sigma);
 *   packed[s_i + e] = prev ? fl32(prev[s_i + e] + y) : y
 * (for a TILEMAJOR tensor, element (r, c) goes to its place in its tile)
 * (scale first, then add: two IEEE round-to-nearest-even operations, never a
 * fused multiply-add), and packed[p] = +0.0 at every padding position p in
 * [0, R_mat*S). Padding of `prev` is never read. With packed_dt = RS_BF16
 * (a bf16 ReduceScatter, as in mixed-precision training) each fp32 result
 * is rounded once to the nearest bf16, ties to even.
 * src: HOST array of n device pointers to contiguous gradients (src_dt
 * RS_F32 or RS_BF16, 16-byte aligned). prev: device fp32 R_mat*S or NULL (no
 * accumulation); it may equal `packed` (in-place accumulation) only when
 * packed_dt is RS_F32 (otherwise RS_EINVAL), and must not overlap it in any
 * other way. packed: device R_mat*S elements of packed_dt (RS_F32 or
 * RS_BF16), 16-byte aligned.
 * Errors: RS_EINVAL, RS_EALIGN, RS_EDTYPE, RS_EHIP. */
int rs_pack_scatter(rs_plan* plan, const void* const* src, int32_t src_dt,
                    const float* prev, void* packed, int32_t packed_dt, int32_t scale_mode,
                    float scale, void* stream);

/* Block-wise quantisation of every locally whole block (feynmanwiki
 * walkthrough, block-quantisation paragraph: all codes of a block depend on
 * one per-block scale, so a rank boundary must never split a block; and the
 * 8-bit Adam paragraph). For each block B
 * (a br x bc tile of a TILE tensor, partial at the edges, or a b-element
 * block of a FLAT tensor):
 *   amax = max |x| over B;  Q = 448 (RS_E4M3), 127 (RS_I8), 255 (RS_U8);
 *   amax == 0: scale[B] = 1.0 and every code is 0;
 *   amax NaN (a NaN in B; NaN wins the max) or +inf (an infinity in B):
 *   scale[B] = quiet NaN 0x7FC00000 or +inf and every code is 0, so the
 *   block dequantises to NaN everywhere (the pages assume finite values);
 *   otherwise scale[B] = fl32(amax / Q), r = min(fl32(Q / amax), FLT_MAX),
 *   code = enc(fl32(x * r)), enc being round-to-nearest-even with saturation
 *   (E4M3: to +-448, sign kept, -0 -> 0x80; I8: to [-127,127]; U8: [0,255]).
 * Every byte of q outside all blocks (padding, untiled tensors) is 0x00.
 * E4M3 codes come from gfx950's FP8 conversion instructions unless the
 * environment variable RS_E4M3_ENCODER=sw is set when the plan is loaded
 * (then an integer encoder is used); both give identical codes.
 * src: device, R_mat*S elements of src_dt (RS_F32 or RS_BF16), 16-byte
 * aligned. q: device, R_mat*S bytes, 16-byte aligned. scales: device fp32
 * [n_qblocks] (rs_plan_info), ordered by tensor, then tile row-major or flat
 * block index.
 * Errors: RS_EINVAL, RS_EALIGN, RS_EDTYPE, RS_EHIP. */
int rs_block_quant(rs_plan* plan, const void* src, int32_t src_dt, void* q, int32_t q_dt,
                   float* scales, void* stream);

/* Allocation-free variant of rs_block_quant, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * allocation). It takes the plan as data (the arguments of rs_plan_load)
 * instead of a loaded plan: it validates the plan, builds the quant work list
 * on the host and copies it into a static device array of 16 MiB that each GPU
 * holds for the life of the process: at most 262,144 work items, one per
 * tile, per pair of flat blocks and per 65,536 positions outside all blocks.
 * It calls no hipMalloc, hipFree or other allocating HIP routine. Codes and
 * scales equal those of rs_block_quant on the same plan, bit for bit.
 * The work list is copied on `stream`, after the work already queued there,
 * and the call waits for `stream` before it launches. Every call on one GPU
 * shares that GPU's array: calls in order on one stream are safe; calls that
 * may overlap on one GPU (other streams, other host threads) race, and the
 * caller must serialise them.
 * specs, n, V, S, starts, R_mat: as for rs_plan_load; the current device runs
 * the call. src, src_dt, q, q_dt: as for rs_block_quant. scales: device fp32,
 * scales_len entries, at least the plan's number of blocks.
 * Errors: the plan's validation errors as for rs_plan_load, RS_EDTYPE,
 * RS_EALIGN, RS_EINVAL (null buffer, scales too short), RS_ERANGE (work list
 * larger than the static array: load the plan and call rs_block_quant),
 * RS_EHIP. Nothing is launched on an error. */
int rs_block_quant_noalloc(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                           const int64_t* starts, int64_t R_mat, const void* src, int32_t src_dt,
                           void* q, int32_t q_dt, float* scales, int64_t scales_len, void* stream);

/* Inverse of rs_block_quant: out[p] = fl32(dec(q[p]) * scale[B]) inside
 * block B, +0.0 everywhere else in [0, R_mat*S). Arguments as in
 * rs_block_quant; out: device fp32 R_mat*S, 16-byte aligned. */
int rs_block_dequant(rs_plan* plan, const void* q, int32_t q_dt, const float* scales,
                     float* out, void* stream);

/* Gather side of block-wise FP8 training, fused (bud-325 summary, TL;DR and
 * Key claims: DeepSeek-V3-style block-wise FP8; feynmanwiki walkthrough,
 * block-quantisation paragraph): after the codes and scales of every rank
 * slice are all-gathered, rebuild each quantised tensor straight from them:
 *   T_i[e] = fl32(dec(q[s_i + e]) * scale[B])   for e in block B of T_i,
 * rounded to bf16 (nearest, ties to even) when dst_dt is RS_BF16. This is
 * rs_block_dequant followed by rs_unpack_gathered (and a cast), in one pass
 * that reads each code once and writes each value once.
 * q, q_dt, scales: as produced by rs_block_quant (device, R_mat*S bytes,
 * 16-byte aligned; fp32 [n_qblocks]). dst: HOST array of n device pointers;
 * entries of TILE, TILEMAJOR and FLAT tensors point to contiguous row-major tensors of
 * n_i elements of dst_dt (RS_BF16 or RS_F32), 16-byte aligned; entries of
 * other tensors are ignored and may be NULL. Codes 0x7F / 0xFF (E4M3 NaN)
 * give unspecified values. Errors: RS_EINVAL, RS_EALIGN, RS_EDTYPE, RS_EHIP. */
int rs_unpack_dequant(rs_plan* plan, const void* q, int32_t q_dt, const float* scales,
                      void* const* dst, int32_t dst_dt, void* stream);

/* Hyper-parameters of one Adam step; step counts from 1. */
typedef struct rs_adam_hparams {
  float lr;
  float beta1;         /* in [0, 1) */
  float beta2;         /* in [0, 1) */
  float eps;           /* >= 0 */
  float weight_decay;  /* decoupled (AdamW); 0 for plain Adam */
  int32_t reserved;    /* must be 0 */
  int64_t step;        /* >= 1 */
} rs_adam_hparams;

/* One 8-bit Adam step on every quantisation block of the plan, in place
 * (feynmanwiki walkthrough, 8-bit Adam paragraph: optimizer state quantised
 * in blocks that stay whole on their device, so each device updates and
 * requantises its own blocks with no scale exchange). The pages give no
 * update formula; this is AdamW. Host scalars, computed in double from the
 * fp32 hyper-parameters and rounded once to fp32:
 *   c1 = 1 - b1, c2 = 1 - b2, step_size = lr / (1 - b1^t),
 *   inv_bc2_sqrt = 1 / sqrt(1 - b2^t), decay = 1 - lr*wd.
 * Per element of a block B, each operation one fp32 round-to-nearest-even
 * step (no fused multiply-add):
 *   m0 = dec_i8(q_m) * s_m[B]        v0 = dec_u8(q_v) * s_v[B]
 *   m1 = b1*m0 + c1*g                v1 = b2*v0 + c2*(g*g)
 *   den = sqrt(v1)*inv_bc2_sqrt + eps
 *   param = param*decay - step_size*(m1/den)
 * then m1 and v1 are requantised per block exactly as rs_block_quant does
 * (int8 and uint8). Positions outside quantisation blocks are not touched.
 * param: device fp32 R_mat*S (in place); grad: device fp32 R_mat*S (the
 * packed gradient, e.g. from rs_pack_scatter); q_m / q_v: device int8 / uint8
 * codes, R_mat*S bytes, in place; s_m / s_v: device fp32 [n_qblocks], in
 * place. All 16-byte aligned. hp: host pointer.
 * Errors: RS_EINVAL (null, step < 1, beta outside [0,1), eps < 0, non-finite
 * lr / wd), RS_EALIGN, RS_EHIP. */
int rs_adam8_step(rs_plan* plan, float* param, const float* grad, void* q_m, float* s_m,
                  void* q_v, float* s_v, const rs_adam_hparams* hp, void* stream);

/* Message for the calling thread's last failed call ("" if none). The
 * pointer stays valid until the thread's next rs_* call. */
const char* rs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RS_H */
