/*
 * hsw.h -- C ABI of the hybrid sliding-window attention core (libhsw.so),
 * hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The method (MiMo-V2.6 Flash/Pro attention, as described on the pages):
 *  - colibri "MiMo-V2.6 (Xiaomi)", section "What the engine implements":
 *    layers are windowed (128-position ring, 8 KV heads on Flash, RoPE theta
 *    1e4, a per-head sink logit that joins the softmax denominator only) or
 *    full attention (4 KV heads on Flash, theta 1e7, no sink); partial
 *    rotate-half RoPE on the first 64 of 192 q/k dims; values 128 wide; the
 *    value scale (0.707 Flash, 0.612 Pro) multiplies values before attention.
 *  - colibri, section "System One mode and prompt reuse": position p lives in
 *    ring slot p mod 128; full layers keep K/V rows by position.
 *  - gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", section "What was built":
 *    the decode window is exactly the last 128 positions; the sink must count
 *    once per sequence, not once per KV block; section "Tiled global-attention
 *    prefill": softmax is per query row, so query tiles need no merge.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked "host".  Scalars are host
 *    values.  Tensor pointers must be 16-byte aligned.
 *  - All tensors are dense, row-major (last index fastest), in `dtype`
 *    (HSW_BF16 or HSW_F32) unless stated.  Positions and lengths are int64.
 *  - The caller allocates and owns every buffer; the library allocates and
 *    frees nothing.  Every output element of a call is overwritten (nothing is
 *    accumulated into).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise.  They are re-entrant and may be issued
 *    from several host threads on different streams.
 *  - Errors: arguments are validated on the host before any launch.  A
 *    failure returns an HSW_E_* code, launches nothing and writes nothing;
 *    hsw_last_error() then describes it (thread-local).  Sizes of zero return
 *    HSW_OK without a launch.  A launch failure reported by the runtime gives
 *    HSW_E_LAUNCH.  Device-resident values (positions, lengths, bases) are not
 *    read on the host; kernels skip, without writing, any K/V row whose
 *    destination or source falls outside the capacities passed in.  The
 *    contract on them (stated per call, collected under "Device-resident
 *    argument checks" below) is checked on the device only by builds with
 *    HSW_CHECK_DEVICE=1 (libhsw_checked.so).
 *  - Positions are 0-based int64.  A window of W positions at position p
 *    holds p-W+1 .. p (the token itself and the W-1 before it).  Windowed
 *    calls take any position below 2^53 (the RoPE angle is formed in double;
 *    ring slots need only its low bits).  Full-attention positions index pool
 *    rows (base + position < pool_rows), and pool_rows must be below 2^31
 *    (HSW_E_SHAPE otherwise): no pool that fits in one GPU comes near it.
 *  - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *  - No C++ exception crosses this boundary.
 */
#ifndef HSW_H_
#define HSW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hsw_stream_t; /* identical to hipStream_t */

typedef int32_t hsw_status;
enum {
    HSW_OK = 0,
    HSW_E_NULL = 1,      /* a required pointer is NULL */
    HSW_E_SHAPE = 2,     /* inconsistent or unsupported sizes */
    HSW_E_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
    HSW_E_DTYPE = 4,     /* unsupported dtype combination */
    HSW_E_WORKSPACE = 5, /* workspace smaller than required */
    HSW_E_LAUNCH = 6,    /* the HIP runtime rejected a launch */
    HSW_E_CAPACITY = 7,  /* a KV pool (ring slots, pool rows, snapshots) lacks room */
    HSW_E_STALE = 8,     /* a snapshot was released (its rows were rewritten) */
    HSW_E_DEVICE_INPUT = 9 /* checked builds: a device-resident argument broke the contract */
};

enum { HSW_BF16 = 0, HSW_F32 = 1 };

/* Destination of K/V rows written by hsw_rope_partial_kv_write. */
enum {
    HSW_DST_RING = 0,    /* k_dst [n_seqs][Hkv][window][d_qk], slot = pos mod window */
    HSW_DST_POOL = 1,    /* k_dst [rows][Hkv][d_qk], row = seq_base[seq] + pos      */
    HSW_DST_STAGING = 2  /* k_dst [n_tokens][Hkv][d_qk], row = token index          */
};

/* Per-layer attention shape.
 *   n_q_heads, n_kv_heads: GQA; n_q_heads % n_kv_heads == 0 (MFMA kernels
 *   take groups of 1, 2, 4, 8 or 16; other groups use a generic kernel).
 *   d_qk: q/k head width (192; multiple of 8, <= 256).  d_v: value width
 *   (128; multiple of 8, <= 256).  rope_dim: rotated leading dims of each
 *   q/k head (64; multiple of 16, <= d_qk).  The MFMA kernels take
 *   d_qk = 192, d_v = 128 (and window 128 on windowed layers) in bf16; other
 *   shapes and fp32 storage run on a generic wave-per-row kernel.  window: ring / window length in
 *   positions (128) for windowed layers, 0 for full attention.
 *   softmax_scale: multiplies q.k (1/sqrt(192) for these heads).
 *   value_scale: multiplies values before attention (0.707 Flash).
 *   rope_theta: 1e4 windowed, 1e7 full.
 *   dtype: storage type of q, k, v, q_rot and the K/V caches.
 *   out_dtype: type of attention outputs. */
typedef struct hsw_attn_shape {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t d_qk;
    int32_t d_v;
    int32_t rope_dim;
    int32_t window;
    float softmax_scale;
    float value_scale;
    double rope_theta;
    int32_t dtype;
    int32_t out_dtype;
} hsw_attn_shape;

const char *hsw_status_str(hsw_status s);
const char *hsw_last_error(void);
const char *hsw_version(void);

/* ------------------------------------------------------------------
 * Device-resident argument checks.
 *
 * The calls never read device-resident arguments on the host (that would
 * need a synchronisation), so release builds trust them.  A build with
 * HSW_CHECK_DEVICE=1 (libhsw_checked.so, same ABI) launches a check kernel
 * ahead of each call's kernels on the call's stream; it tests every element
 * against the contract below and records the first violation it sees in a
 * flag held in the library's module memory, one per device (nothing is
 * allocated).  Every kernel of that and every later call on the device then
 * returns without reading or writing anything, until the flag is cleared.
 * The contract per call (codes HSW_DEV_*):
 *   RoPE:        pos[t] >= 0 (POSITION); ring: 0 <= seq[t] < dst_capacity
 *                (RING_SEQ); pool: seq[t] >= 0 and 0 <= seq_base[seq[t]] +
 *                pos[t] < dst_capacity, staging: t < dst_capacity
 *                (DST_RANGE).  seq[t] must also index seq_base, which no
 *                build can check (its length is not passed).
 *   prefills:    cu_seqlens[0] >= 0, non-decreasing, every length <=
 *                max_seqlen (CU_SEQLENS), and cu_seqlens[n_seqs] at most the
 *                rows of q / staging / out (not checkable); start_pos >= 0
 *                (POSITION); full: 0 <= seq_base and seq_base + start_pos +
 *                length <= pool_rows (POOL_RANGE).
 *   SWA decode:  pos >= 0 (POSITION).
 *   full decode: 1 <= ctx_len <= max_ctx (CTX_LEN); 0 <= seq_base and
 *                seq_base + ctx_len <= pool_rows (POOL_RANGE).
 *   ViT:         cu_seqlens as for the prefills with max_len; every order
 *                entry inside its picture (ORDER).
 * Calls on several streams of one device share the flag.
 */
enum {
    HSW_DEV_OK = 0,
    HSW_DEV_POSITION = 1,
    HSW_DEV_CU_SEQLENS = 2,
    HSW_DEV_POOL_RANGE = 3,
    HSW_DEV_RING_SEQ = 4,
    HSW_DEV_CTX_LEN = 5,
    HSW_DEV_ORDER = 6,
    HSW_DEV_DST_RANGE = 7
};

/* 1 in a build with HSW_CHECK_DEVICE=1, else 0. */
int32_t hsw_device_checks_enabled(void);

/* Synchronise `stream`, then read the current device's check flag: HSW_OK
 * with *code = HSW_DEV_OK and *index = -1 when no violation was recorded;
 * HSW_E_DEVICE_INPUT with *code the HSW_DEV_* code and *index the element
 * (token, sequence or picture) that broke it, after which the flag is
 * cleared.  In a release build nothing is checked: HSW_OK with *code = -1
 * and *index = -1, no synchronisation.  code and index may be NULL. */
hsw_status hsw_device_check_status(hsw_stream_t stream, int32_t *code, int64_t *index);

/*
 * Partial rotate-half RoPE on q and k, plus the K/V write.
 * Follows colibri "What the engine implements" (rotate-half on the first
 * rope_dim dims, theta per layer kind) and gaudi-cookbook "The RoPE fix for
 * large positions" (angles must stay exact at large positions: each angle
 * pos * theta^(-2i/rope_dim) is formed and reduced in double precision, then
 * rotated in fp32).  Values are written unscaled: the value scale is applied
 * to the attention output, which equals scaling values first by linearity.
 *
 *   q [n_tokens][Hq][d_qk], k [n_tokens][Hkv][d_qk], v [n_tokens][Hkv][d_v]
 *      in dtype; pos [n_tokens] int64 (>= 0); seq [n_tokens] int32 (the
 *      token's sequence; may be NULL for HSW_DST_STAGING; for HSW_DST_POOL
 *      every seq[t] must index seq_base).
 *   dst_kind: HSW_DST_RING / POOL / STAGING (see the enum for layouts; V is
 *      the same with d_v).  dst_capacity: sequences in the ring, rows in the
 *      pool, or rows in staging.  seq_base [n_seqs] int64: POOL only.
 *   q_rot [n_tokens][Hq][d_qk] in dtype (written).  q and q_rot may both be
 *      NULL: then only K/V are rotated and written (for the *_qrope calls,
 *      which rotate q themselves); one of them NULL alone is HSW_E_NULL.
 *   v and v_dst may both be NULL for HSW_DST_STAGING: then only K is
 *      written (V staging has v's own layout [n_tokens][Hkv][d_v], so the
 *      windowed prefill can take v itself as its V staging); one of them
 *      NULL alone, or either NULL for RING / POOL, is HSW_E_NULL.
 *   dst_index_out [n_tokens] int64 or NULL: the slot / row written for each
 *      token, or -1 when its destination was outside dst_capacity.
 */
hsw_status hsw_rope_partial_kv_write(const hsw_attn_shape *sh, int64_t n_tokens,
                                     const void *q, const void *k, const void *v,
                                     const int64_t *pos, const int32_t *seq,
                                     int32_t dst_kind, void *k_dst, void *v_dst,
                                     int64_t dst_capacity, const int64_t *seq_base,
                                     void *q_rot, int64_t *dst_index_out,
                                     hsw_stream_t stream);

/*
 * Banded sliding-window prefill with a per-head sink, then the ring commit.
 * Follows gaudi-cookbook "What was built" (banded tiles, fp32 softmax that
 * includes the sink) and colibri "What the engine implements" (window of
 * sh->window positions, sink in the denominator only, value scale).
 *
 *   Sequence s owns chunk tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 at
 *   positions start_pos[s] + t.  Keys at positions < start_pos[s] come from
 *   the ring (slot = pos mod window), which must hold positions
 *   start_pos[s]-window+1 .. start_pos[s]-1 (those >= 0); keys inside the
 *   chunk come from the staging buffers.
 *   cu_seqlens [n_seqs+1], start_pos [n_seqs] int64; max_seqlen (host) bounds
 *   every chunk length.  q_rot [T][Hq][d_qk]; k_stage [T][Hkv][d_qk];
 *   v_stage [T][Hkv][d_v]; k_ring [n_seqs][Hkv][window][d_qk];
 *   v_ring [n_seqs][Hkv][window][d_v]; sinks [Hq] fp32 or NULL;
 *   out [T][Hq][d_v] in out_dtype.
 *   After the attention, the last min(len, window) chunk rows of each
 *   sequence are copied into their ring slots (a second, stream-ordered
 *   launch), so the ring then holds the chunk's final positions.
 */
hsw_status hsw_swa_prefill(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                           const int64_t *cu_seqlens, const int64_t *start_pos,
                           const void *q_rot, const void *k_stage, const void *v_stage,
                           void *k_ring, void *v_ring, const float *sinks, void *out,
                           hsw_stream_t stream);

/*
 * Sliding-window decode of one new token per sequence over its ring.
 * Follows colibri "System One mode and prompt reuse" (slot t holds position
 * P - ((P - t) mod window); slots holding positions < 0 are skipped) and
 * gaudi-cookbook "What was built" (exactly the last `window` positions, the
 * sink counted once).
 *
 *   pos [n_seqs] int64: the new token's position (already in the ring).
 *   q_rot [n_seqs][Hq][d_qk]; k_ring / v_ring as in hsw_swa_prefill;
 *   sinks [Hq] fp32 or NULL; out [n_seqs][Hq][d_v] in out_dtype.
 */
hsw_status hsw_swa_decode(const hsw_attn_shape *sh, int32_t n_seqs, const int64_t *pos,
                          const void *q_rot, const void *k_ring, const void *v_ring,
                          const float *sinks, void *out, hsw_stream_t stream);

/*
 * hsw_swa_prefill with the q-RoPE fused in: q is the unrotated query
 * [T][Hq][d_qk] (the K/V staging rows must already be rotated, e.g. by
 * hsw_rope_partial_kv_write with q = q_rot = NULL), and the kernel rotates q
 * as it loads it (colibri "What the engine implements": rotate-half on the
 * first rope_dim dims; gaudi-cookbook "The RoPE fix for large positions":
 * the angle is formed and reduced in double) at positions start_pos[s] + t.
 * The rotation and its bf16 rounding are those of hsw_rope_partial_kv_write,
 * so out is bit-identical to that call followed by hsw_swa_prefill; no q_rot
 * is written or read.  Every other argument, the ring commit and the error
 * behaviour are those of hsw_swa_prefill.  Supported shapes: bf16 in and
 * out, d_qk 192, d_v 128, rope_dim 64, window 128, 2/4/8/16 query heads per
 * KV head; others give HSW_E_SHAPE.
 */
hsw_status hsw_swa_prefill_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                 const int64_t *cu_seqlens, const int64_t *start_pos, const void *q,
                                 const void *k_stage, const void *v_stage, void *k_ring, void *v_ring,
                                 const float *sinks, void *out, hsw_stream_t stream);

/*
 * hsw_swa_decode with the q-RoPE fused in: q [n_seqs][Hq][d_qk] is
 * unrotated and is rotated at pos[s] in the kernel (same sources as
 * hsw_swa_prefill_qrope).  The rotated rotary dims are kept in fp32 (split
 * into bf16 hi + lo for the products), so the result is at least as accurate
 * as RoPE to a bf16 q_rot followed by hsw_swa_decode, without q_rot's bytes.
 * The ring must already hold the new token's K/V (hsw_rope_partial_kv_write
 * with q = q_rot = NULL).  Supported shapes: bf16 in and out, d_qk 192, d_v
 * 128, rope_dim 64, window 128, n_q_heads <= 256, 1/2/4/8/16 query heads per
 * KV head; others give HSW_E_SHAPE.  Other arguments and errors as
 * hsw_swa_decode.
 */
hsw_status hsw_swa_decode_qrope(const hsw_attn_shape *sh, int32_t n_seqs, const int64_t *pos,
                                const void *q, const void *k_ring, const void *v_ring,
                                const float *sinks, void *out, hsw_stream_t stream);

/*
 * Full-attention decode, split over key chunks with a log-sum-exp combine.
 * Follows colibri "System One mode and prompt reuse" (rows by position) and
 * gaudi-cookbook "What was built" / "What it taught about Gaudi" (per-block
 * decode partials; a sink, if given, is added exactly once, in the combine).
 *
 *   ctx_len [n_seqs] int64 (keys 0 .. ctx_len-1, the new token last, at
 *   row seq_base[s] + ctx_len - 1); seq_base [n_seqs] int64; max_ctx (host)
 *   bounds every ctx_len (keys past max_ctx are not read).  q_rot [n_seqs][Hq][d_qk];
 *   k_pool [pool_rows][Hkv][d_qk], v_pool [pool_rows][Hkv][d_v] with
 *   pool_rows (host) rows; sinks [Hq] fp32 or NULL; chunk: keys per split
 *   (multiple of 64, e.g. 2048).  ws: device workspace of ws_bytes bytes,
 *   at least hsw_full_decode_workspace_bytes(...).  out [n_seqs][Hq][d_v].
 */
size_t hsw_full_decode_workspace_bytes(const hsw_attn_shape *sh, int32_t n_seqs,
                                       int64_t max_ctx, int32_t chunk);
hsw_status hsw_full_decode_splitk(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                  const int64_t *ctx_len, const int64_t *seq_base,
                                  const void *q_rot, const void *k_pool, const void *v_pool,
                                  int64_t pool_rows, const float *sinks, int32_t chunk,
                                  void *ws, size_t ws_bytes, void *out, hsw_stream_t stream);

/*
 * hsw_full_decode_splitk without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split-K partials go to a scratch
 * array in the library's module memory, HSW_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per device, held until the process ends; the call allocates and frees
 * nothing.  Every other argument, the result and the error behaviour are
 * those of hsw_full_decode_splitk (bit for bit the same output).  A call
 * whose partials, hsw_full_decode_workspace_bytes(sh, n_seqs, max_ctx,
 * chunk), exceed the scratch returns HSW_E_WORKSPACE and launches nothing
 * (64 sequences x 64 heads at 131072 keys fit with chunk 8192).  All calls
 * on one device share the scratch: calls that overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the caller.
 */
#define HSW_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hsw_status hsw_full_decode_splitk_noalloc(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                          const int64_t *ctx_len, const int64_t *seq_base, const void *q_rot,
                                          const void *k_pool, const void *v_pool, int64_t pool_rows,
                                          const float *sinks, int32_t chunk, void *out, hsw_stream_t stream);

/*
 * Full-attention chunked prefill over prior rows plus the chunk (causal).
 * Follows gaudi-cookbook "Tiled global-attention prefill" (query tiles, no
 * materialised mask, no cross-tile merge since softmax is per row) and
 * colibri "System One mode and prompt reuse" (rows by position).
 *
 *   Sequence s: chunk tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 at positions
 *   start_pos[s] + t; its rows seq_base[s] + 0 .. seq_base[s] + start_pos[s]
 *   + len - 1 are already in the pool (RoPE appended the chunk).
 *   q_rot [T][Hq][d_qk]; pools as in hsw_full_decode_splitk; sinks [Hq] or
 *   NULL; out [T][Hq][d_v] in out_dtype.
 */
hsw_status hsw_full_prefill_chunk(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                  const int64_t *cu_seqlens, const int64_t *start_pos,
                                  const int64_t *seq_base, const void *q_rot,
                                  const void *k_pool, const void *v_pool, int64_t pool_rows,
                                  const float *sinks, void *out, hsw_stream_t stream);

/*
 * hsw_full_prefill_chunk with the q-RoPE fused in: q [T][Hq][d_qk] is
 * unrotated (the chunk's K/V rows must already be in the pool, e.g. by
 * hsw_rope_partial_kv_write with q = q_rot = NULL) and is rotated in the
 * kernel at positions start_pos[s] + t with the RoPE call's own arithmetic
 * (colibri "What the engine implements"; gaudi-cookbook "The RoPE fix for
 * large positions"), so out is bit-identical to that call followed by
 * hsw_full_prefill_chunk; no q_rot is written or read.  Supported shapes:
 * bf16 in and out, d_qk 192, d_v 128, rope_dim 64, 2/4/8/16 query heads per
 * KV head (HSW_E_SHAPE otherwise); other arguments and errors as
 * hsw_full_prefill_chunk.
 */
hsw_status hsw_full_prefill_chunk_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                        const int64_t *cu_seqlens, const int64_t *start_pos,
                                        const int64_t *seq_base, const void *q, const void *k_pool,
                                        const void *v_pool, int64_t pool_rows, const float *sinks, void *out,
                                        hsw_stream_t stream);

/*
 * hsw_full_decode_splitk with the q-RoPE fused in: q [n_seqs][Hq][d_qk] is
 * unrotated and is rotated in the kernel at each sequence's new position
 * ctx_len[s] - 1; the rotated rotary dims stay fp32 (bf16 hi + lo in the
 * products).  The pool must already hold the new token's K/V.  Supported
 * shapes: bf16 in and out, d_qk 192, d_v 128, rope_dim 64, 1/2/4/8/16 query
 * heads per KV head (HSW_E_SHAPE otherwise); other arguments, the workspace
 * and errors as hsw_full_decode_splitk.
 */
hsw_status hsw_full_decode_splitk_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                        const int64_t *ctx_len, const int64_t *seq_base, const void *q,
                                        const void *k_pool, const void *v_pool, int64_t pool_rows,
                                        const float *sinks, int32_t chunk, void *ws, size_t ws_bytes, void *out,
                                        hsw_stream_t stream);

/*
 * KV-cache bytes (host arithmetic).  kind HSW_DST_RING: every sequence holds
 * `window` positions whatever ctx is (the O(W) ring of colibri "What the
 * engine implements"); HSW_DST_POOL: ctx positions.  Per position and layer:
 * n_kv_heads * (d_qk + d_v_stored) * elem_bytes.  Returns -1 on bad input.
 */
int64_t hsw_kv_bytes(int32_t kind, int64_t n_seqs, int64_t ctx, int32_t window,
                     int32_t n_kv_heads, int32_t d_qk, int32_t d_v_stored,
                     int32_t elem_bytes, int32_t n_layers);

/*
 * Dual-pool KV manager (host bookkeeping over caller-owned device pools).
 *
 * gokawiil "Full-Pipeline Inference Optimization for MiMo-V2.5 Series",
 * section 2.1 "SWA KVCache Management": the full-attention layers and the
 * windowed layers keep separate pools -- full layers O(N) rows per sequence,
 * windowed layers O(W) (here the 128-slot ring of each sequence) -- and a
 * request is admitted only if both pools have room; prefix reuse is clipped
 * to a "window-safe length", where the windowed layers' last W positions are
 * still held.  colibri "MiMo-V2.6 (Xiaomi)", section "System One mode and
 * prompt reuse": a snapshot keeps the full layers' rows in place (nothing
 * after it writes below its position; the token ids are recorded and checked
 * before resuming, and a sequence that diverged below it releases it), copies
 * every windowed layer's ring into the snapshot and back, and records its
 * position.
 *
 * Layout the manager assumes (the same the attention calls use):
 *   windowed layer l: K ring swa_k[l] [ring_seqs][swa_kv_heads][window][d_qk],
 *                     V ring swa_v[l] [ring_seqs][swa_kv_heads][window][d_v];
 *   full layers: pool rows [pool_rows][full_kv_heads][d], a sequence owning
 *                rows seq_base .. seq_base + max_len - 1 (row = seq_base + pos);
 *   snapshot k: bytes [k * S, (k+1) * S) of snap_buf, S =
 *                hsw_kvm_snapshot_bytes(cfg), holding per windowed layer the
 *                sequence's K ring block then its V ring block.
 * The manager allocates no device memory; its host state is allocated by
 * hsw_kvm_create and freed by hsw_kvm_destroy.  One handle must not be used
 * from two host threads at once.  Snapshot and restore are stream-ordered
 * copies on `stream`; bookkeeping calls only touch host state.
 */
typedef struct hsw_kvm hsw_kvm;

typedef struct {
    int32_t n_swa_layers;   /* windowed layers (1..128) */
    int32_t swa_kv_heads;
    int32_t window;         /* ring slots per sequence and layer */
    int32_t d_qk, d_v;      /* head widths (multiples of 8) */
    int32_t elem_bytes;     /* 2 (bf16) or 4 (fp32) */
    int32_t ring_seqs;      /* sequences each ring buffer holds */
    int64_t pool_rows;      /* rows each full-layer pool holds */
    int32_t max_snapshots;  /* snapshots snap_buf holds */
} hsw_kvm_config;

/* Bytes of one snapshot: n_swa_layers * swa_kv_heads * window * (d_qk + d_v)
 * * elem_bytes (colibri: "about 50 MB per snapshot on Flash" in fp32; 25.6 MB
 * in bf16).  0 on bad input. */
size_t hsw_kvm_snapshot_bytes(const hsw_kvm_config *cfg);

/* swa_k, swa_v: host arrays of n_swa_layers device pointers (16-byte
 * aligned); snap_buf: device, at least max_snapshots * snapshot bytes
 * (HSW_E_WORKSPACE otherwise; may be NULL when max_snapshots is 0). */
hsw_status hsw_kvm_create(const hsw_kvm_config *cfg, void *const *swa_k, void *const *swa_v,
                          void *snap_buf, size_t snap_buf_bytes, hsw_kvm **out);
void hsw_kvm_destroy(hsw_kvm *kvm);

/* Admit a sequence that will hold at most max_len positions: takes a free ring
 * slot and the first free run of max_len pool rows, or takes nothing and
 * returns HSW_E_CAPACITY when either pool lacks room.  *seq (ring slot and
 * sequence id) and *seq_base (first pool row) are written on success. */
hsw_status hsw_kvm_admit(hsw_kvm *kvm, int64_t max_len, int32_t *seq, int64_t *seq_base);
/* Return the sequence's ring slot and pool rows; its snapshots are released. */
hsw_status hsw_kvm_release(hsw_kvm *kvm, int32_t seq);

/* Record host token ids for positions len .. len+n-1 of the sequence (the
 * caller then writes their K/V with hsw_rope_partial_kv_write and runs the
 * attention at *start_pos = len, which puts each of these positions into its
 * ring slot p mod window; the manager records that the slots now hold them).
 * HSW_E_CAPACITY past max_len.  A token that differs from the one its row
 * held before releases the sequence's snapshots at positions above it. */
hsw_status hsw_kvm_append(hsw_kvm *kvm, int32_t seq, const int32_t *tokens, int64_t n, int64_t *start_pos);
/* Move the sequence's length back to new_len <= len (the rows beyond keep
 * their contents and token ids until rewritten; the ring slots keep the
 * positions they hold, so the windowed state at new_len exists only if they
 * still hold its window -- hsw_kvm_window_safe_length says where it does). */
hsw_status hsw_kvm_truncate(hsw_kvm *kvm, int32_t seq, int64_t new_len);
/* Length, first pool row and capacity of a sequence. */
hsw_status hsw_kvm_info(hsw_kvm *kvm, int32_t seq, int64_t *len, int64_t *seq_base, int64_t *max_len);
/* Free ring slots, largest free run of pool rows, free snapshot slots. */
hsw_status hsw_kvm_free_space(hsw_kvm *kvm, int32_t *ring_slots, int64_t *pool_run, int32_t *snapshots);

/* Copy the sequence's ring of every windowed layer into a free snapshot slot
 * (one launch on `stream`) and record (sequence, position = len, the token
 * ids below it).  HSW_E_CAPACITY when every slot is taken. */
hsw_status hsw_kvm_snapshot(hsw_kvm *kvm, int32_t seq, int32_t *snap, hsw_stream_t stream);
/* Copy the snapshot's rings back into its sequence's ring slot (one launch)
 * and set the sequence's length to the snapshot's position.  HSW_E_STALE if
 * the snapshot was released (the sequence diverged below its position). */
hsw_status hsw_kvm_restore(hsw_kvm *kvm, int32_t snap, hsw_stream_t stream);
hsw_status hsw_kvm_drop_snapshot(hsw_kvm *kvm, int32_t snap);

/* Window-safe reuse length of `tokens` (host, n ids) against the sequence:
 * the longest L <= the common prefix of tokens and the sequence's recorded
 * ids at which the windowed layers' state is available.  The state at L
 * exists where ring slots hold every position the window of the token at L
 * reads from the ring, max(0, L - window + 1) .. L - 1 (each slot holds the
 * last position appended into it, or the one a restored snapshot held).
 * Candidates: every L <= the live length under the live rings (truncate to
 * L, then append; for a sequence longer than the window that is the live
 * length itself and the one below it, unless a truncate and re-append left
 * other runs), and each live snapshot at its own position when its copied
 * rings hold that window (*snap set to it; restore before use); 0 always.
 * The live state wins over a snapshot of the same length.  *snap = -1 unless
 * a snapshot is needed.  Returns -1 on bad arguments. */
int64_t hsw_kvm_window_safe_length(hsw_kvm *kvm, int32_t seq, const int32_t *tokens, int64_t n, int32_t *snap);

/* ==================================================================
 * Vision encoder (ViT) attention.
 * colibri "MiMo-V2.6 (Xiaomi)", the model description's "vision" entry: 2D
 * RoPE, grouped-query attention, full attention in 4 of 28 blocks and a 1D
 * window of 64 tokens in the others, row and column order of the 2x2 merge
 * units alternating; the window blocks add a sink at their leading key; its
 * "Verifying it": the gateway's patches equal the Qwen2-VL processor's.
 * Readings: a picture's tokens come in merge-unit order (the 4 patches of a
 * 2x2 unit consecutive: top-left, top-right, bottom-left, bottom-right;
 * units row by row); attention is bidirectional within a picture; a window
 * block cuts the picture's tokens, in its order, into consecutive windows of
 * 64 (the last may be shorter) and each token attends to its window and to
 * the sink key, the picture's first token in that order.
 * ================================================================== */

/*
 * Host arithmetic (no device access): for an h x w patch grid (h, w > 0 and
 * even) in merge-unit order, row[t] and col[t] are token t's patch
 * coordinates and col_order[j] is the token at position j of the column
 * order (units column by column, a unit's 4 patches still consecutive).
 * Host arrays of h*w int32 each; any of them may be NULL (not written).
 * HSW_E_SHAPE on a bad grid.
 */
hsw_status hsw_vit_layout(int32_t h, int32_t w, int32_t *row, int32_t *col, int32_t *col_order);

/*
 * 2D rotate-half RoPE of whole heads: pair (i, i + d/2), i < d/2, turns by
 * row * f(i) for i < d/4 and by col * f(i - d/4) above, with
 * f(j) = rope_theta^(-j / (d/4)) (the frequencies of a 1D rotary of width
 * d/2; the angle formed and reduced in double, the rotation in fp32).
 *   q [n_tokens][Hq][d], k [n_tokens][Hkv][d] bf16 (d = sh->d_qk, a multiple
 *   of 32, <= 128; sh->rope_dim == d); row, col [n_tokens] int32 patch
 *   coordinates (hsw_vit_layout); q_out, k_out like q, k (may equal them:
 *   in place is allowed).  q and q_out both given or both NULL, likewise k
 *   and k_out; at least one pair.
 * Errors: HSW_E_NULL, HSW_E_SHAPE (d, rope_dim), HSW_E_DTYPE (not bf16),
 * HSW_E_ALIGN.
 */
hsw_status hsw_vit_rope_2d(const hsw_attn_shape *sh, int64_t n_tokens, const void *q, const void *k,
                           const int32_t *row, const int32_t *col, void *q_out, void *k_out,
                           hsw_stream_t stream);

/*
 * ViT attention over n_images pictures packed by cu_seqlens [n_images + 1]
 * (int64, token rows; picture s is rows cu[s] .. cu[s+1]-1, at most max_len
 * long).  q [T][Hq][64], k, v [T][Hkv][64] bf16 (rotated q and k), out
 * [T][Hq][64] bf16, all by token row.
 *   sh->window == 0: every token attends to its whole picture (full block).
 *   sh->window == 64: window block: the picture's tokens in the block's
 *     order -- order[cu[s] + j] (int32, picture-local) is the token at
 *     position j, or order == NULL for the tokens' own order -- cut into
 *     consecutive 64-token windows; a token attends to its window and, if
 *     sink_key != 0, to the token at position 0 of the order (once).
 *   sinks [Hq] fp32 or NULL: learned sink logits, in the denominator only.
 * softmax_scale multiplies q.k (1/8 for 64-wide heads); value_scale must be
 * 1.  Supported: bf16 in and out, d_qk = d_v = 64, 1/2/4/8/16 query heads per
 * KV head (HSW_E_SHAPE otherwise).  Every output row of a picture is
 * written.  Order entries are not checked on the host; the kernel clamps
 * them into the picture (wrong rows, never out-of-bounds accesses).
 * Errors: HSW_E_NULL, HSW_E_SHAPE, HSW_E_ALIGN (q, k, v, out 16 B;
 * cu_seqlens 8 B; order, sinks 4 B).
 */
hsw_status hsw_vit_attention(const hsw_attn_shape *sh, int32_t n_images, int64_t max_len,
                             const int64_t *cu_seqlens, const int32_t *order, int32_t sink_key, const void *q,
                             const void *k, const void *v, const float *sinks, void *out, hsw_stream_t stream);

/*
 * A ViT window block with its 2D RoPE fused: hsw_vit_rope_2d of q and k
 * (rope_theta of sh, row and col as there) followed by hsw_vit_attention with
 * window 64, in one call that reads the unrotated q and k and writes only
 * out -- no rotated copy of q or k goes through memory.  Follows colibri
 * "MiMo-V2.6 (Xiaomi)", the model description's "vision" entry (2D RoPE;
 * 64-token windows with a sink on the first key), read as for the two calls
 * it joins.  Each workgroup forms the angles of its window's tokens once and
 * rotates with the 2D RoPE call's own arithmetic, so out is bit-identical to
 * the two calls made in turn.
 *   Arguments as hsw_vit_attention, with q [T][Hq][64] and k [T][Hkv][64]
 *   unrotated, and row, col [T] int32 patch coordinates by token row
 *   (hsw_vit_layout).  Requires sh->window == 64 and d_qk == d_v ==
 *   rope_dim == 64 (HSW_E_SHAPE otherwise); full blocks (window 0) rotate
 *   once with hsw_vit_rope_2d instead, since every query block of a picture
 *   reads every key.
 * Errors: HSW_E_NULL (cu_seqlens, row, col, q, k, v, out), HSW_E_SHAPE,
 * HSW_E_ALIGN (q, k, v, out 16 B; cu_seqlens 8 B; order, sinks, row, col 4 B).
 */
hsw_status hsw_vit_window_attention_rope(const hsw_attn_shape *sh, int32_t n_images, int64_t max_len,
                                         const int64_t *cu_seqlens, const int32_t *order, int32_t sink_key,
                                         const int32_t *row, const int32_t *col, const void *q, const void *k,
                                         const void *v, const float *sinks, void *out, hsw_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HSW_H_ */
