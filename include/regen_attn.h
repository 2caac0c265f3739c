/*
 * regen_attn: 3D-RoPE exact self-attention for the ReGenVC diffusion
 * transformer decoder, on AMD Instinct MI355X (gfx950).
 *
 * The operation. The ReGenVC decoder is a four-step distilled diffusion
 * transformer (arXiv 2607.28144; index page, "Abstract") whose blocks attend
 * over the video-latent token sequence of one decode window, split into
 * attention heads (blog summary, "Methodology - deep read", the USP
 * paragraph: Ulysses reshuffles the sequence into heads). The pages require
 * the attention to stay exact (blog summary, "Technical innovations", USP
 * bullet) and cite FlashAttention / FlashAttention-2 (index page, "Builds
 * on"). For every head and query token m this library computes
 *
 *     o_m = sum_n softmax_n( sm_scale * <R(m) q_m, R(n) k_n> ) v_n
 *
 * over all tokens n of the window (non-causal), where R(n) is a rotary
 * position embedding over the token's (t, h, w) latent coordinates. The
 * pages give no rotary convention; this library fixes it as follows:
 *   - token n of the T x H x W grid sits at t = n / (H W), h = (n / W) % H,
 *     w = n % W (row-major, t slowest), with origin 0 on every axis;
 *   - the head_dim/2 pairs (x[2i], x[2i+1]) are split into consecutive
 *     chunks of pairs_t, pairs_h, pairs_w pairs for the t, h, w axes;
 *   - pair j of axis a turns counter-clockwise by pos_a * base^(-j/P_a).
 *
 * Numerics: inputs and output are bf16; rotated Q and K are rounded to bf16,
 * both products use bf16 MFMA with fp32 accumulation, the softmax runs in
 * fp32 (exp2 with the scale folded in), probabilities are rounded to bf16
 * for the P V product, and the output is rounded to bf16
 * (round-to-nearest-even throughout).
 *
 * Layout: q, k, v, o are contiguous bf16 tensors [heads][T*H*W][head_dim]
 * in device memory, 16-byte aligned, owned by the caller; with the flag
 * REGEN_ATTN_TOKEN_MAJOR they are [T*H*W][heads][head_dim] instead, the
 * layout a Ulysses all-to-all delivers and expects back (see
 * regen_ulysses_pack).
 *
 * Threading: a handle is bound to the HIP device that was current at
 * create, and is read-only for the caller after create: calls on one handle
 * may be issued from any host thread, on any streams, with no ordering
 * between them. The handle owns two sets of the device buffers a call writes
 * besides its output (rotated K, transposed V, split-tile partials, and for
 * an attention block its projection outputs). A call takes the set its
 * stream used last, else an unused one, else the least recently used one,
 * after making its stream wait (hipStreamWaitEvent) for the last call that
 * used that set; after enqueueing, it records the set's event on its stream.
 * So calls on two streams run at the same time, and a third stream is
 * ordered behind one of them. A stream handle must not be destroyed and
 * re-created at the same address while calls on it are in flight (the
 * library tells streams apart by their handle value). Distinct handles are
 * independent.
 */
#ifndef REGEN_ATTN_H
#define REGEN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum regen_status {
    REGEN_OK = 0,
    REGEN_ERR_INVALID_ARGUMENT = 1, /* a NULL, out-of-range or misaligned argument */
    REGEN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head_dim, device) */
    REGEN_ERR_NO_DEVICE = 3,        /* no usable HIP device */
    REGEN_ERR_OUT_OF_MEMORY = 4,    /* device or host allocation failed */
    REGEN_ERR_HIP = 5               /* a HIP runtime call failed; see regen_attn_last_error */
} regen_status;

/* Flags for regen_attn_desc.flags. */
#define REGEN_ATTN_NO_ROPE 0x1u /* skip the rotation (plain exact attention) */
#define REGEN_ATTN_PROFILE 0x2u /* record HIP events around each kernel (see
                                   regen_attn_profile_read) */
#define REGEN_ATTN_TOKEN_MAJOR 0x4u /* q, k, v, o are [tokens][heads][head_dim]
                                       (lse stays [heads][tokens]) */

/*
 * Problem description. Zero in an optional field selects its default.
 *   struct_size : sizeof(regen_attn_desc) (version check)
 *   heads       : attention heads, >= 1
 *   head_dim    : 64 or 128
 *   grid_t/h/w  : latent grid; tokens = grid_t * grid_h * grid_w, >= 1
 *   pairs_t/h/w : rotary pairs per axis; all three 0 selects the default
 *                 split (h and w get floor(head_dim/6) each, t the rest:
 *                 22/21/21 at head_dim 128, 12/10/10 at 64); otherwise each
 *                 must be >= 1 and they must sum to head_dim / 2
 *   rope_base   : rotary base, > 0 (0 selects 10000)
 *   sm_scale    : softmax scale, > 0 (0 selects 1/sqrt(head_dim))
 *   flags       : REGEN_ATTN_* bits
 */
typedef struct regen_attn_desc {
    uint32_t struct_size;
    int32_t heads;
    int32_t head_dim;
    int32_t grid_t;
    int32_t grid_h;
    int32_t grid_w;
    int32_t pairs_t;
    int32_t pairs_h;
    int32_t pairs_w;
    float rope_base;
    float sm_scale;
    uint32_t flags;
} regen_attn_desc;

typedef struct regen_attn *regen_attn_t;

/*
 * Create a handle for one problem shape on the current HIP device.
 * Allocates the handle, the per-axis rotary tables (fp64 on the host,
 * stored as fp32 cos/sin) and two sets (see Threading above) of: a device
 * workspace of 2 * heads * ceil(tokens/128)*128 * head_dim * 2 bytes
 * (rotated K and transposed V; see regen_attn_workspace_size) and a scratch
 * area for query tiles whose keys are split over several workgroups of the
 * persistent attention kernel: 2 * P * 256 * (2 * head_dim + 8) bytes (bf16
 * O/l and fp32 (m, l) per row), P = resident workgroups of the device (one
 * per compute unit on MI355X: 33 MiB at head_dim 128), plus a 4-byte counter
 * of the leftover pieces workgroups claim.
 * On success *out receives the handle; on any failure *out is set to NULL
 * (when out is not NULL) and the status says why:
 *   INVALID_ARGUMENT (NULL desc/out, wrong struct_size, heads/grid < 1,
 *   bad pairs split, base or scale < 0, unknown flags, tokens > 2^30, one
 *   head's rotated K reaching 2^31 bytes: ceil(tokens/128)*128 * head_dim *
 *   2 >= 2^31, or heads * ceil(tokens/256) * ceil(tokens/64) >= 2^31: the
 *   attention schedule numbers its (query tile, key block) pairs in 31 bits),
 *   UNSUPPORTED (head_dim not 64/128, current device is not gfx950),
 *   NO_DEVICE, OUT_OF_MEMORY, HIP.
 */
regen_status regen_attn_create(const regen_attn_desc *desc, regen_attn_t *out);

/*
 * Enqueue one attention call on `stream` (a hipStream_t; NULL = the null
 * stream) and return without waiting. q, k, v (inputs) and o (output) are
 * device pointers to contiguous bf16 [heads][tokens][head_dim] tensors,
 * 16-byte aligned; o must not overlap q, k or v. The buffer sizes cannot be
 * checked from raw pointers: each must hold heads * tokens * head_dim bf16
 * values. The same inputs give bit-identical outputs on every call: query
 * tiles whose keys are split over workgroups are cut at fixed key blocks and
 * merged in a fixed order, whichever workgroup computed a part (workgroups
 * claim the last parts as they finish, since the device's parts do not all
 * run at one clock). Errors: INVALID_ARGUMENT (NULL or destroyed handle,
 * NULL or misaligned pointer, o overlapping an input), HIP (launch failure;
 * detail in regen_attn_last_error). Faults during execution surface at the
 * caller's next synchronization.
 */
regen_status regen_attn_forward(regen_attn_t h, const void *q, const void *k,
                                const void *v, void *o, void *stream);

/*
 * Attention of a run of query tokens against a run of key tokens of the
 * handle's window, with the log-sum-exp of every row's scores. This is the
 * piece of Ring-style sequence parallelism that one GPU computes (blog
 * summary, "Methodology - deep read", USP paragraph: Ring circulates key and
 * value blocks while each device keeps its queries; "Technical innovations":
 * the split attention stays exact): results over separate key runs combine
 * exactly with regen_attn_merge.
 *   q     : [heads][q_count][head_dim] bf16, row m = token q_begin + m
 *   k, v  : [heads][kv_count][head_dim] bf16, row n = token kv_begin + n
 *   o     : [heads][q_count][head_dim] bf16, attention over those keys only
 *   lse   : [heads][q_count] fp32, lse_m = log sum_n exp(sm_scale <R(m)q_m,
 *           R(n)k_n>) (natural log), or NULL to skip it
 * Each token is rotated at its own place on the latent grid (token index as
 * in the file comment). Ranges must satisfy 0 <= begin, 1 <= count,
 * begin + count <= grid_t*grid_h*grid_w. Pointers: device memory, o 16-byte
 * aligned and not overlapping q, k, v; lse 4-byte aligned and not
 * overlapping any other buffer. regen_attn_forward(h, q, k, v,
 * o, s) equals this call with both ranges covering the window and lse NULL.
 * Errors: INVALID_ARGUMENT (bad handle, range, pointer, alignment or
 * overlap), HIP (launch failure).
 */
regen_status regen_attn_forward_range(regen_attn_t h, const void *q, int64_t q_begin,
                                      int64_t q_count, const void *k, const void *v,
                                      int64_t kv_begin, int64_t kv_count, void *o, float *lse,
                                      void *stream);

/*
 * Cross-attention of the window's tokens to conditioning tokens (the text /
 * image encoder context a DiT block attends to besides its own tokens; the
 * pages name the encoders, not the context length): for every head and
 * window token m, o_m = sum_j softmax_j(sm_scale <q_m, c_j>) w_j over the
 * ctx_len context keys c_j and values w_j. Nothing is rotated.
 *   q      : all window tokens, layout as for regen_attn_forward
 *   k_ctx, v_ctx : [heads][ctx_len][head_dim] bf16 ([ctx_len][heads]
 *            [head_dim] with REGEN_ATTN_TOKEN_MAJOR)
 *   o      : like q;  lse : [heads][tokens] fp32 or NULL
 * 1 <= ctx_len <= grid_t*grid_h*grid_w (the workspace is sized by the
 * window). Same pointer rules and errors as regen_attn_forward_range. A context of at most 256 tokens is held whole in
 * on-chip memory by one kernel that reads k_ctx and v_ctx directly (the
 * handle's workspace is not touched); longer ones go through the workspace
 * like regen_attn_forward.
 */
regen_status regen_attn_forward_cross(regen_attn_t h, const void *q, const void *k_ctx,
                                      const void *v_ctx, int64_t ctx_len, void *o, float *lse,
                                      void *stream);

/*
 * Combine nparts attention results over disjoint key sets into the result
 * over their union (the exact combination Ring-style key splitting relies
 * on; blog summary, "Methodology - deep read", USP paragraph):
 *     lse = log sum_i exp(lse_i),   o = sum_i exp(lse_i - lse) o_i.
 *   o_parts   : host array of nparts device pointers, each bf16
 *               [heads][rows][head_dim], 16-byte aligned
 *   lse_parts : host array of nparts device pointers, each fp32
 *               [heads][rows], 4-byte aligned (-inf marks a part with no keys)
 *   o         : bf16 [heads][rows][head_dim] output, 16-byte aligned
 *   lse       : fp32 [heads][rows] output, or NULL
 * 1 <= nparts <= 8; head_dim 64 or 128. Outputs must not overlap inputs. A
 * row whose parts are all -inf gets o = 0 and lse = -inf. Needs no handle;
 * enqueued on `stream` (the current device's). Errors: INVALID_ARGUMENT,
 * UNSUPPORTED (head_dim), NO_DEVICE, HIP.
 */
regen_status regen_attn_merge(const void *const *o_parts, const float *const *lse_parts,
                              int nparts, int heads, int64_t rows, int head_dim, void *o,
                              float *lse, void *stream);

/*
 * The on-device halves of a Ulysses all-to-all (blog summary, "Methodology -
 * deep read", USP paragraph: Ulysses reshuffles the sequence into attention
 * heads; with G devices each holds tokens_local = N/G tokens of every head
 * before attention and all N tokens of heads/G heads during it).
 *
 * regen_ulysses_pack: x [tokens_local][heads][head_dim] (this device's
 * token shard, all heads) -> send [groups][tokens_local][heads/groups]
 * [head_dim], so that block g (heads g*heads/groups ..) is one contiguous
 * piece for device g. After the all-to-all, the piece received from device
 * s is tokens s*tokens_local .. of this device's head group, i.e. the receive
 * buffer is [N][heads/groups][head_dim] token-major: attention takes it as
 * is with REGEN_ATTN_TOKEN_MAJOR (rotation fused into its loads) and writes
 * O in the same layout, which is the send buffer of the reverse all-to-all.
 *
 * regen_ulysses_unpack: recv [groups][tokens_local][heads/groups][head_dim]
 * (piece g from the device holding head group g) -> y [tokens_local][heads]
 * [head_dim], this device's token shard with all heads again.
 *
 * bf16 elements; heads must be a multiple of groups and (heads/groups) *
 * head_dim * 2 a multiple of 16; buffers 16-byte aligned, not overlapping.
 * Enqueued on `stream` of the current device. Errors: INVALID_ARGUMENT,
 * NO_DEVICE, HIP.
 */
regen_status regen_ulysses_pack(const void *x, void *send, int64_t tokens_local, int heads,
                                int head_dim, int groups, void *stream);
regen_status regen_ulysses_unpack(const void *recv, void *y, int64_t tokens_local, int heads,
                                  int head_dim, int groups, void *stream);

/*
 * A linear layer without bias, y = x w^T: x [rows][in_features], w
 * [out_features][in_features] (the usual [out][in] weight layout), y
 * [rows][out_features]; bf16 in and out, fp32 accumulation (MFMA), y
 * rounded to nearest even. in_features must be a multiple of 64; every
 * operand under 4 GiB; device pointers, 16-byte aligned, y not overlapping
 * x or w. Enqueued on `stream` of the current device. Errors:
 * INVALID_ARGUMENT, UNSUPPORTED (in_features), NO_DEVICE, HIP.
 */
regen_status regen_linear(const void *x, const void *w, void *y, int64_t rows, int in_features,
                          int out_features, void *stream);

/*
 * One self-attention block of the diffusion transformer around this
 * attention (index page, "Abstract": the decoder is a DiT; the projection
 * sizes follow the heads x head_dim of the description, hidden = heads *
 * head_dim, no biases):
 *     [Q | K | V] = X W_qkv^T,   O = attention(R Q, R K, V),   Y = O W_o^T.
 *   x     : [tokens][hidden] bf16, token-major hidden states of the window
 *   w_qkv : [3 hidden][hidden] bf16 ([out][in]); output rows 0..hidden-1
 *           give Q, the next hidden give K, the last hidden give V; head h
 *           uses rows h*head_dim .. h*head_dim + head_dim - 1 of each
 *   w_o   : [hidden][hidden] bf16 ([out][in])
 *   y     : [tokens][hidden] bf16 output (must not overlap the inputs)
 * The projections run as regen_linear; the attention reads Q, K and V in
 * place out of the projection output (a strided token-major view) and
 * applies the rotation while loading. All pointers are device memory,
 * 16-byte aligned, owned by the caller. regen_block_create takes the same
 * description as regen_attn_create (without REGEN_ATTN_TOKEN_MAJOR or
 * REGEN_ATTN_PROFILE) and allocates two sets of the attention workspace,
 * the projection output (tokens * 3 hidden bf16) and the attention output
 * (tokens * hidden bf16); like an attention handle, a block is read-only
 * after create and may be used from several streams and threads at once.
 * Errors as for the attention calls.
 */
typedef struct regen_block *regen_block_t;
regen_status regen_block_create(const regen_attn_desc *desc, regen_block_t *out);
regen_status regen_block_forward(regen_block_t b, const void *x, const void *w_qkv,
                                 const void *w_o, void *y, void *stream);
regen_status regen_block_destroy(regen_block_t b);

/*
 * Free the handle, its tables and workspace, after waiting for the last
 * call on each of its buffer sets. No call on the handle may be issued
 * during or after destroy. NULL is a no-op
 * returning REGEN_OK; a handle that is not live gives INVALID_ARGUMENT.
 */
regen_status regen_attn_destroy(regen_attn_t h);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as regen_attn_create + regen_attn_forward + regen_attn_destroy
 * with the same q, k, v, o arguments and rules, but with no handle and no
 * allocation. The rotary table (built on the device by a kernel), the rotated
 * K / transposed V and the split-tile partials live in one static device
 * array of REGEN_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on
 * each device it runs on until the process ends; the first call on a device
 * looks its address up. Problems that need more than that (the table, 2 *
 * heads * ceil(tokens/128)*128 * head_dim * 2 bytes of workspace and
 * 2 * P * 256 * (2 * head_dim + 8) bytes of partials, P = resident
 * workgroups, and a piece counter, each at a 256-byte boundary) are rejected with UNSUPPORTED: the 25-frame window (12 x 10920
 * x 128, about 102 MB) fits, the 77-frame clip (12 x 31200 x 128) does not.
 * Every call on a device shares its one array, and each call leaves its
 * contents behind: calls that overlap in time on one device (different
 * streams, or host threads without ordering) race and give wrong results,
 * so order them. No buffer needs clearing between calls (each call writes
 * everything it reads). REGEN_ATTN_PROFILE is rejected. Errors as for
 * regen_attn_create and regen_attn_forward, plus UNSUPPORTED for the size.
 */
#define REGEN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
regen_status regen_attn_forward_noalloc(const regen_attn_desc *desc, const void *q, const void *k,
                                        const void *v, void *o, void *stream);

/* Static, human-readable name of a status code. Never NULL; do not free. */
const char *regen_attn_status_string(regen_status s);

/*
 * Detail of the last failure on the calling thread (thread-local storage;
 * empty string if none). Valid until the next library call on this thread.
 */
const char *regen_attn_last_error(void);

/*
 * Kernel timing for handles created with REGEN_ATTN_PROFILE. Each forward
 * then records HIP events on its stream around each of its three kernels
 * (the K-rotation / V-transpose pass, the attention kernel, the merge of
 * tiles split across workgroups; a short-context cross-attention call runs
 * one kernel, counted as the attention kernel). This call waits for the events of every
 * forward issued since the last read, adds their durations (milliseconds)
 * to *prep_ms, *attn_ms, *merge_ms and the number of forwards to *calls
 * (each output may be NULL), and forgets them.
 * Errors: INVALID_ARGUMENT (handle not live, or created without the flag),
 * HIP (event failure).
 */
regen_status regen_attn_profile_read(regen_attn_t h, double *prep_ms, double *attn_ms,
                                     double *merge_ms, int64_t *calls);

/*
 * Measurement aid: the GPU core clock under a pure bf16 MFMA load (one
 * workgroup of 8 waves per compute unit, every wave issuing iters rounds of
 * four independent 32x32x16 MFMAs). Enqueues one kernel on `stream` that
 * writes, from one wave, counters[0..1] = core cycle counter at the start
 * and end of its loop and counters[2..3] = constant-rate counter at start
 * and end (counters: device memory, 5 int64, 8-byte aligned, caller-owned;
 * counters[4] is scratch). *wall_clock_khz receives the constant counter's
 * rate. After the stream has finished: clock = (c1 - c0) / ((c3 - c2) /
 * (wall_clock_khz * 1e3)). Errors: INVALID_ARGUMENT, HIP.
 */
regen_status regen_clock_probe(int iters, int64_t *counters, double *wall_clock_khz, void *stream);

/*
 * Bytes of the rotated-K / transposed-V workspace regen_attn_create would
 * allocate for desc (the device-dependent split-tile scratch not included),
 * or 0 if the description is invalid. Touches no device.
 */
size_t regen_attn_workspace_size(const regen_attn_desc *desc);

#ifdef __cplusplus
}
#endif

#endif /* REGEN_ATTN_H */
