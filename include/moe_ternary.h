/*
 * moe_ternary.h - C ABI of the MI355X (gfx950) ternary-expert MoE block.
 *
 * The library computes the forward pass of one mixture-of-experts block whose
 * expert weights are ternary {-1, 0, +1} times one fp16 scale per group of 128
 * weights, stored in one of two containers:
 *
 *   PQ2_0  (id 142): 34 bytes per 128 weights, 2.125 bits per weight.
 *          Scion-35B-A3B card, "Weight Representation: ternary PQ2_0 + trained
 *          corrections" and "About the Hub's quant chip" (2-bit codes plus one
 *          fp16 group scale per 128; the legacy Q1_0_g128 name has the same
 *          byte layout).
 *          bytes 0..31: weight j in byte j/4, bits 2(j%4)..2(j%4)+1, LSB first;
 *          code 00 = 0, 01 = +1, 11 = -1 (10 is invalid);
 *          bytes 32..33: the scale, IEEE binary16, little-endian.
 *
 *   PTQ1_0 (id 143): 28 bytes per 128 weights, 1.75 bits per weight.
 *          Scion-FlashNext-176B-A6B card, "Weight Representation: ternary
 *          PTQ1_0 + trained corrections + Q4_0 PLE" (24 bytes of 5-trit data,
 *          2 bytes holding the remaining trits, the 2-byte group scale) and
 *          "Highlights" (5 trits per byte, about 10% over the 1.585 bpw entropy).
 *          bytes 0..23: byte b holds weights 5b..5b+4 as sum_i d_i 3^i (<= 242);
 *          bytes 24..25: byte 24+m holds weights 120+4m..123+4m as sum_i d_i 3^i
 *          (<= 80); digit d = t mod 3 (0 -> 0, 1 -> +1, 2 -> -1);
 *          bytes 26..27: the scale, IEEE binary16, little-endian.
 *
 *   The format ids are the type ids the fork gives the two containers
 *   (35B-A3B card, "Quickstart": GGML_TYPE_PQ2_0 = 142; FlashNext card,
 *   "About the Hub's quant chip": PTQ1_0 is type id 143).  A weight's value is
 *   scale * t.  Groups of 128 run along the input (K) dimension of each row.
 *
 * The forward pass (Scion project README, "The idea" and "Serving notes";
 * FlashNext card, "Model Overview"):
 *   l = (W_r + dW_r) x                       router logits plus router delta
 *   s_1..s_k = top-k of l                    ties go to the lower expert index
 *   w_i = softmax over the k selected logits
 *   grouping of (token, slot) pairs per expert
 *   o(t, e) = W_down,e (silu(W_gate,e x_t) * (W_up,e x_t))   ternary SwiGLU expert
 *   y_t = sum_i w_i o(t, s_i) + sum_shared o(t, shared) + B (A x_t)
 * The last term is the rank-r correction branch on the MoE block output, on the
 * residual stream (README, "What the experiments established": the placement
 * rule; 35B-A3B card, "Weight Representation": rank-512 branches and exact
 * router deltas).
 *
 * Numerics: activations x and y are bfloat16; all products accumulate in fp32 on
 * matrix cores; the intermediate h = silu(g) * u and z = A x are rounded to
 * bfloat16; router, router delta, A and B (fp16) enter the matrix cores as an
 * exact two-term bfloat16 split (the router and its delta are first summed in
 * fp32).  Gate weights use fp32 exp.
 *
 * Ownership and ordering: the caller allocates and frees every buffer.  The
 * library allocates no device memory and keeps no caller pointer after a call
 * returns, except the stage events handed to moe_set_stage_events; besides
 * those it holds only a thread-local error message and the device's compute
 * unit count, read once.  Device entry points are ordered on the given stream
 * (a hipStream_t; NULL means the null stream) and return once the work is
 * enqueued: inputs must stay alive and unchanged until the stream reaches the
 * call, and concurrent streams need separate workspaces.
 *
 * Errors: every argument, shape and format check happens on the host before the
 * first launch, so a call that returns an error has enqueued nothing.  A failed
 * launch returns MOE_E_DEVICE.  No C++ exception crosses this interface.
 */
#ifndef MOE_TERNARY_H
#define MOE_TERNARY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_PQ2_0 = 142, MOE_PTQ1_0 = 143 };

enum {
  MOE_OK = 0,
  MOE_E_ARG = -1,        /* NULL pointer or out-of-range scalar argument       */
  MOE_E_FORMAT = -2,     /* unknown container id                                 */
  MOE_E_SHAPE = -3,      /* a dimension is not a multiple of 128, or k > E       */
  MOE_E_CODE = -4,       /* invalid code byte (2-bit 10, base-3 byte too large)  */
  MOE_E_NONFINITE = -5,  /* NaN or Inf group scale                                */
  MOE_E_SPACE = -6,      /* destination or workspace too small                    */
  MOE_E_DEVICE = -7      /* a HIP launch or runtime call failed                   */
};

/* Bytes per 128-weight group: 34 (PQ2_0), 28 (PTQ1_0), -1 for an unknown id. */
int64_t moe_block_bytes(int32_t fmt);

/* Container bytes for n_weights weights; -1 if fmt is unknown or n_weights is
 * negative or not a multiple of 128. */
int64_t moe_packed_bytes(int32_t fmt, int64_t n_weights);

/* Host: pack n_weights trits (int8 in {-1,0,+1}) and n_weights/128 fp16 scale
 * bit patterns into dst (dst_bytes >= moe_packed_bytes).  Errors: MOE_E_FORMAT,
 * MOE_E_SHAPE (n % 128), MOE_E_ARG (NULL, trit outside {-1,0,1}),
 * MOE_E_NONFINITE (NaN/Inf scale), MOE_E_SPACE. */
int32_t moe_pack(int32_t fmt, const int8_t* trits, const uint16_t* scales_f16,
                 int64_t n_weights, uint8_t* dst, int64_t dst_bytes);

/* Host: validate and unpack a container into trits and scale bits.  An invalid
 * code byte returns MOE_E_CODE and the message names the group and byte. */
int32_t moe_unpack(int32_t fmt, const uint8_t* src, int64_t src_bytes, int8_t* trits,
                   uint16_t* scales_f16, int64_t n_weights);

/* Device: decode a container already in device memory (d_src) into device
 * trits (int8, n_weights) and scale bits (uint16, n_weights/128) with the same
 * in-register decoders the expert kernels use.  No code validation: the
 * container must come from moe_pack or have passed moe_unpack. */
int32_t moe_unpack_device(int32_t fmt, const uint8_t* d_src, int64_t n_weights, int8_t* d_trits,
                          uint16_t* d_scales, void* stream);

/* Quantizer rules for a group of 128 weights (project README, "What the
 * experiments established": the ternary Lloyd quantizer over groups of 128
 * that the released experts use beats one-shot absmean; Scion-35B-A3B
 * discussion thread, its list of findings). */
enum { MOE_QUANT_ABSMEAN = 0, MOE_QUANT_LLOYD = 1 };

/* Device: quantize n_weights bfloat16 weights (d_w, device memory, row-major,
 * groups of 128 along each row) into a container at d_dst (device memory,
 * moe_packed_bytes(fmt, n_weights) bytes, groups in the order of the input).
 *   MOE_QUANT_ABSMEAN  s = mean |w|; t = sign(w) where 2|w| > s, else 0.
 *   MOE_QUANT_LLOYD    from the absmean codes, alternate s = mean |w| over the
 *                      weights with t != 0 and t = sign(w) where 2|w| > s until
 *                      the codes repeat, at most 32 rounds; s is then the mean
 *                      |w| over the final nonzero codes (0 if there are none).
 * Every comparison and sum is fp32, each group sum a balanced tree over adjacent
 * pairs (weights 2m and 2m+1 first); the scale is rounded to binary16, nearest
 * even, saturating at 65504.  Weights must be finite (otherwise the codes and
 * scales of their groups are unspecified).  The result is a pure function of
 * the input bits.  d_rounds (device memory, n_weights/128 bytes, or NULL)
 * receives per group the Lloyd rounds taken, the round that repeats the codes
 * included (32 if none does); 0 for absmean.  d_w must be 16-byte and d_dst
 * 4-byte aligned; the buffers must not overlap.  Ordered on `stream`; nothing
 * is allocated.
 * Errors: MOE_E_FORMAT, MOE_E_ARG (unknown method, NULL d_w or d_dst,
 * misaligned, overlapping), MOE_E_SHAPE (n_weights negative, not a multiple of
 * 128, or too large for one launch: above 2^31 - 1 blocks of 16 groups),
 * MOE_E_DEVICE. */
int32_t moe_quantize_device(int32_t fmt, int32_t method, const uint16_t* d_w, int64_t n_weights,
                            uint8_t* d_dst, uint8_t* d_rounds, void* stream);

/* Device: gather rows of a Q4_0 table and decode them to fp32.  The FlashNext
 * release keeps its n-gram table (320,001,536 rows of 160 values, 28.8 GB) as
 * one Q4_0 tensor with groups of 32 along each row, decoded per row
 * (Scion-FlashNext-176B-A6B card, "Model Overview" and "Weight Representation:
 * ternary PTQ1_0 + trained corrections + Q4_0 PLE").  The format is read as
 * ggml's Q4_0 block: 18 bytes per 32 values, a binary16 scale d (little-
 * endian), then 16 code bytes whose low nibbles hold values 0..15 and high
 * nibbles values 16..31; value = d * (nibble - 8).  Rows of row_len values
 * (a multiple of 32) lie back to back, row_len / 32 * 18 bytes each.
 *   d_table  device, n_rows rows, 2-byte aligned
 *   d_idx    device int64 row numbers, n_idx of them, 8-byte aligned
 *   d_out    device fp32 [n_idx x row_len], 16-byte aligned; row i = decoded
 *            row d_idx[i] (exact: every d * (nibble - 8) is an fp32 value).
 *            An index outside [0, n_rows) gives a row of quiet NaN and reads
 *            nothing; duplicates are allowed.
 * Ordered on `stream`; nothing is allocated.  Errors: MOE_E_SHAPE (row_len not
 * a positive multiple of 32, negative counts), MOE_E_ARG (NULL, misaligned),
 * MOE_E_DEVICE. */
int32_t moe_ple_gather_q4_0(const uint8_t* d_table, int64_t n_rows, int32_t row_len, const int64_t* d_idx,
                            int64_t n_idx, float* d_out, void* stream);

/* Device: the rank-r branch on its own, y = y_in + B (A x), for the other
 * tensor the releases correct the same way: rank-512 branches sit on the
 * attention output as well as on the MoE block output (Scion-35B-A3B card,
 * "Weight Representation"; project README, "The idea").
 *   x           device bf16 [n_tokens x d] (the branch input), 16-byte aligned
 *   y_in        device bf16 [n_tokens x d], or NULL for zero; y may equal y_in
 *               (an in-place update of the residual stream)
 *   A / A_q     fp16 [r x d] or a ternary PQ2_0 container of it (row-major
 *               groups); exactly one of the two
 *   B / B_q     fp16 [d x r] or PQ2_0 (then r % 128 == 0); exactly one
 *   y           device bf16 [n_tokens x d], 16-byte aligned, not x
 *   workspace   >= moe_lowrank_workspace_bytes(n_tokens, d, r), 256-byte aligned
 * The numerics are the block's correction: fp32 products on matrix cores, z =
 * A x rounded to bf16, y summed in fp32 as (B z) + y_in and rounded to bf16.
 * With r >= 2048 and fp16 A, A x adds its K steps in another order from 33 to
 * 256 tokens than below 33, so results can differ in their last bits between
 * such batches (the block's own projection keeps one order for every batch).
 * d % 128 == 0, r % 8 == 0, r <= 4096.  Errors: MOE_E_SHAPE, MOE_E_ARG,
 * MOE_E_SPACE, MOE_E_DEVICE. */
int64_t moe_lowrank_workspace_bytes(int64_t n_tokens, int32_t d, int32_t r);
int32_t moe_lowrank_apply(const uint16_t* x, const uint16_t* y_in, int64_t n_tokens, int32_t d,
                          const uint16_t* A, const uint8_t* A_q, const uint16_t* B, const uint8_t* B_q,
                          int32_t r, uint16_t* y, void* workspace, int64_t workspace_bytes, void* stream);

/* Device: the k=1 draft head that ships beside the 35B-A3B release, an fp16
 * fc1 / gelu / fc2 head over the model's own hidden state and the next token's
 * embedding (Scion-35B-A3B card, "Shipped Components" and "Highlights"):
 *   x = [hidden ; emb]  (hidden first, 2h values)
 *   y = W2 gelu(W1 x + b1) + b2,   gelu(v) = v (1 + erf(v / sqrt 2)) / 2
 *   hidden, emb  device bf16 [n_tokens x h] (bit patterns), row-major, 16-byte aligned
 *   w1           device fp16 [m x 2h], b1 fp16 [m] or NULL (no bias)
 *   w2           device fp16 [h x m],  b2 fp16 [h] or NULL
 *   y            device bf16 [n_tokens x h]
 *   workspace    device, >= moe_draft_head_workspace_bytes(...), 256-byte aligned
 * h and m are multiples of 128 (h = 2048, m = 4096 is the card's 50 MB).
 * Products accumulate in fp32 on matrix cores (fp16 weights as exact bf16
 * pairs); gelu(W1 x + b1) and y are rounded to bf16.  From 33 to 256 tokens a
 * product of 2048 or more rows adds its K steps in another order than below 33
 * tokens, so a token's y can differ in its last bits between such batches.
 * n_tokens = 0 is a no-op.
 * Errors: MOE_E_SHAPE, MOE_E_ARG (NULL, misaligned), MOE_E_SPACE, MOE_E_DEVICE. */
int64_t moe_draft_head_workspace_bytes(int64_t n_tokens, int32_t hidden, int32_t inner);
int32_t moe_draft_head(const uint16_t* hidden, const uint16_t* emb, int64_t n_tokens, int32_t h, int32_t m,
                       const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2,
                       uint16_t* y, void* workspace, int64_t workspace_bytes, void* stream);

/* Host: reorder the blocks of a [rows x cols] container (rows % 16 == 0,
 * cols % 128 == 0) between the row-major order moe_pack writes and the
 * tile-major order the expert kernels read.  With G = cols / 128, block
 * (row n, group g) has row-major index n G + g and tile-major index
 * ((n / 16) G + g) 16 + n % 16: the 16 blocks of one group of a 16-row tile are
 * adjacent, so one wave-wide load reads 16 consecutive blocks.  Every block
 * keeps its bytes; only their order changes.  src and dst must not overlap.
 * Errors: MOE_E_FORMAT, MOE_E_SHAPE, MOE_E_ARG (NULL, overlap), MOE_E_SPACE. */
int32_t moe_tile_container(int32_t fmt, const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                           int64_t dst_bytes);
int32_t moe_untile_container(int32_t fmt, const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                             int64_t dst_bytes);

/* One layer's expert banks: E routed experts, then S always-on shared experts
 * (FlashNext card, "Model Overview": top-10 routed + 1 shared).  Bank e starts
 * at byte offsets[e] of `banks` and holds three containers back to back:
 * gate [d_ff x d_model], up [d_ff x d_model], down [d_model x d_ff], groups of
 * 128 along each row, all in format formats[e], each in the tile-major block
 * order of moe_tile_container.  Offsets must be multiples of 16 (the kernels
 * read each group of a 16-row tile with aligned 16-byte loads), and the buffer
 * must extend at least MOE_BANK_SLACK bytes past the end of every bank (the
 * expert kernels read each block with one 12-byte load that can run 2 bytes
 * past the block); the slack's content is ignored. */
enum { MOE_BANK_SLACK = 16 };
/* Block order of the containers in a moe_expert_banks.  The expert kernels read
 * only the tile-major order; the field makes the caller state it, so banks
 * straight from moe_pack (row-major) are refused with MOE_E_ARG instead of
 * being read in the wrong order. */
enum { MOE_BANKS_ROW_MAJOR = 1, MOE_BANKS_TILE_MAJOR = 2 };
typedef struct moe_expert_banks {
  int32_t d_model;              /* d: multiple of 128                              */
  int32_t d_ff;                 /* f: multiple of 128                              */
  int32_t n_experts;            /* E >= 1 routed experts                           */
  int32_t n_shared;             /* S >= 0 shared experts (weight 1, no gate)       */
  const uint8_t* banks;         /* device: all containers                          */
  int64_t banks_bytes;          /* size of `banks` in bytes, slack included        */
  const int64_t* offsets;       /* device int64[E+S]                               */
  const uint8_t* formats;       /* device uint8[E+S]: 142 or 143                   */
  const int64_t* offsets_host;  /* host copy of offsets (validation)               */
  const uint8_t* formats_host;  /* host copy of formats (validation, dispatch)     */
  int32_t layout;               /* must be MOE_BANKS_TILE_MAJOR                    */
} moe_expert_banks;

/* Workspace bytes moe_ternary_forward needs for n_tokens tokens. */
int64_t moe_workspace_bytes(const moe_expert_banks* banks, int64_t n_tokens, int32_t top_k,
                            int32_t corr_rank);

/* The block's forward pass.
 *   x            device bf16 [n_tokens x d_model] (bit patterns), row-major
 *   router       device fp16 [E x d_model]
 *   router_delta device fp16 [E x d_model], or NULL for a zero delta
 *   corr_A       device fp16 [corr_rank x d_model], corr_B fp16 [d_model x corr_rank];
 *                both NULL with corr_rank = 0 for the uncorrected block
 *   top_k        1 <= top_k <= E
 *   y            device bf16 [n_tokens x d_model]; must not alias x
 *   workspace    device, >= moe_workspace_bytes(...) bytes, 256-byte aligned
 * n_tokens = 0 is a no-op.  The banks must come from moe_pack (codes are not
 * re-validated on the device). */
int32_t moe_ternary_forward(const uint16_t* x, int64_t n_tokens, const uint16_t* router,
                            const uint16_t* router_delta, const moe_expert_banks* banks,
                            const uint16_t* corr_A, const uint16_t* corr_B, int32_t corr_rank,
                            int32_t top_k, uint16_t* y, void* workspace, int64_t workspace_bytes,
                            void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward pass as moe_ternary_forward, with its workspace taken from a
 * library-owned device array of MOE_NOALLOC_SCRATCH_BYTES bytes (one per GPU,
 * loaded with the library and held until the process ends) instead of a
 * caller buffer.  The call allocates nothing.  The caller still passes every
 * input and y, with moe_ternary_forward's layouts; results equal
 * moe_ternary_forward's bit for bit.  A batch whose moe_workspace_bytes exceeds
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_E_SPACE before any launch (decode
 * batches of up to 256 tokens fit at every layer shape of the releases).  All
 * calls on one GPU share its array and nothing in it needs clearing between
 * calls (every byte a call reads it wrote first), so calls that overlap on one
 * GPU (concurrent streams, or threads) race; serialise them.  Errors: those of
 * moe_ternary_forward, MOE_E_SPACE as above, MOE_E_DEVICE if the array's device
 * address cannot be resolved. */
#define MOE_NOALLOC_SCRATCH_BYTES (64ll << 20)
int32_t moe_ternary_forward_noalloc(const uint16_t* x, int64_t n_tokens, const uint16_t* router,
                                    const uint16_t* router_delta, const moe_expert_banks* banks,
                                    const uint16_t* corr_A, const uint16_t* corr_B, int32_t corr_rank,
                                    int32_t top_k, uint16_t* y, void* stream);

/* The same forward pass with the router delta and the correction stored as
 * ternary PQ2_0 containers, the way the 35B-A3B release ships them (Scion-
 * 35B-A3B card, "Weight Representation" and "Shipped Components": the
 * rank-512 corrections and the exact router deltas in the legacy q1_0_g128
 * container, whose bytes are PQ2_0's).
 *   router_delta_q  device PQ2_0 [E x d_model], or NULL for a zero delta
 *   corr_A_q        device PQ2_0 [corr_rank x d_model], corr_B_q PQ2_0
 *                   [d_model x corr_rank] (corr_rank a multiple of 128); both
 *                   NULL with corr_rank = 0
 * The containers are in moe_pack's row-major group order, 2-byte aligned.  A
 * code times its group scale is an fp16 value, and the kernels expand the
 * codes into exactly those fp16 operands, so the result equals bit for bit that
 * of moe_ternary_forward given the fp16 matrices s * t; only 34 bytes per 128
 * weights are read instead of 256.  Other arguments, the workspace and the
 * errors are those of moe_ternary_forward; codes are not re-validated. */
int32_t moe_ternary_forward_q(const uint16_t* x, int64_t n_tokens, const uint16_t* router,
                              const uint8_t* router_delta_q, const moe_expert_banks* banks,
                              const uint8_t* corr_A_q, const uint8_t* corr_B_q, int32_t corr_rank,
                              int32_t top_k, uint16_t* y, void* workspace, int64_t workspace_bytes,
                              void* stream);

/* The same forward pass with the router delta given as two low-rank factors,
 * the way the FlashNext release ships it (Scion-FlashNext-176B-A6B card,
 * "Weight Representation": rank-512 F16 factors for the router deltas): the
 * logits are W_r x + U (V x).
 *   delta_U     device fp16 [E x delta_rank], 16-byte aligned
 *   delta_V     device fp16 [delta_rank x d_model], 4-byte aligned
 *   delta_rank  a positive multiple of 8, at most 1024
 * V x is computed as the router's own product (fp32 on matrix cores, fp16
 * weights as exact bf16 pairs) and kept in fp32; U (V x) accumulates in fp32
 * and joins the router logits before the top-k.  The workspace is
 * moe_workspace_bytes_factored's; corrections are fp16 (or NULL), and the
 * other arguments and the errors are moe_ternary_forward's (MOE_E_SHAPE for a
 * bad delta_rank). */
int64_t moe_workspace_bytes_factored(const moe_expert_banks* banks, int64_t n_tokens, int32_t top_k,
                                     int32_t corr_rank, int32_t delta_rank);
int32_t moe_ternary_forward_factored(const uint16_t* x, int64_t n_tokens, const uint16_t* router,
                                     const uint16_t* delta_U, const uint16_t* delta_V, int32_t delta_rank,
                                     const moe_expert_banks* banks, const uint16_t* corr_A,
                                     const uint16_t* corr_B, int32_t corr_rank, int32_t top_k, uint16_t* y,
                                     void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes moe_route needs. */
int64_t moe_route_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t n_experts,
                                  int32_t top_k);

/* The routing half of the forward pass, with every intermediate exported
 * (device buffers):
 *   logits  fp32 [n_tokens x E]       the same fp32 logits the forward pass uses
 *   topk_idx int32 [n_tokens x k]     selected experts in rank order
 *   topk_w  fp32 [n_tokens x k]       softmax over the selected logits
 *   counts  int32 [E]                 slots per expert
 *   offsets int32 [E+1]               exclusive scan of counts
 *   perm    int32 [n_tokens * k]      flat slot ids t*k+i ordered by (expert, token)
 * Runs the same kernels as moe_ternary_forward on the same inputs. */
int32_t moe_route(const uint16_t* x, int64_t n_tokens, int32_t d_model, int32_t n_experts,
                  const uint16_t* router, const uint16_t* router_delta, int32_t top_k,
                  float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
                  int32_t* offsets, int32_t* perm, void* workspace, int64_t workspace_bytes,
                  void* stream);

/* The routing half of moe_ternary_forward_factored, with every intermediate
 * exported: the router delta as fp16 factors U [E x delta_rank] (16-byte
 * aligned) and V [delta_rank x d_model] (4-byte aligned), logits W_r x + U (V x)
 * (FlashNext card, "Weight Representation": rank-512 F16 factors for the
 * router deltas).  Outputs and their layouts are moe_route's; the kernels and
 * their summation order are those moe_ternary_forward_factored runs, so the
 * exported choice is the one the forward pass makes for the same tokens.  The
 * workspace is moe_route_workspace_bytes_factored's.  Errors: moe_route's, and
 * MOE_E_SHAPE for a delta_rank that is not a positive multiple of 8 up to 1024. */
int64_t moe_route_workspace_bytes_factored(int64_t n_tokens, int32_t d_model, int32_t n_experts,
                                           int32_t top_k, int32_t delta_rank);
int32_t moe_route_factored(const uint16_t* x, int64_t n_tokens, int32_t d_model, int32_t n_experts,
                           const uint16_t* router, const uint16_t* delta_U, const uint16_t* delta_V,
                           int32_t delta_rank, int32_t top_k, float* logits, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                           void* workspace, int64_t workspace_bytes, void* stream);

/* Measurement hook.  With events != NULL (n_events >= 2 * MOE_N_STAGES
 * hipEvent_t handles created by the caller), every later moe_ternary_forward
 * call on this thread records events[2s] before and events[2s+1] after stage s
 * on the call's stream (a NULL entry skips that record); NULL events (or
 * n_events = 0) turn recording off.  Stages:
 * 0 router/correction projection, 1 routing (top-k, ranking, scan, scatter),
 * 2 gate/up experts, 3 down experts, 4 combine.  moe_draft_head records
 * events[0], [1] around its fc1 product and [2], [3] around its fc2 product;
 * moe_lowrank_apply [0], [1] around the product A x (up to 256 tokens its fp32
 * slices, added up after events[1]) and [2], [3] around B z + y_in.
 * The library keeps the pointer until it is replaced; the caller keeps the
 * events alive meanwhile. */
enum { MOE_N_STAGES = 5 };
int32_t moe_set_stage_events(void** events, int32_t n_events);

/* Message of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TERNARY_H */
