// hsw_launch.h -- internal launch interface between the C ABI (hsw_abi.hip)
// and the kernels.  Argument structs are passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsw {

struct RopeArgs {
    const void *q, *k, *v;
    const int64_t *pos;
    const int32_t *seq;
    const int64_t *seq_base;
    void *k_dst, *v_dst, *q_rot;
    int64_t *dst_index_out;
    const unsigned long long *dev_flag;  // checked builds: nonzero once an argument broke the contract
    int64_t n_tokens, dst_capacity;
    int hq, hkv, dqk, dv, rope_dim, window, dst_kind;
    double inv_freq[128];      // theta^(-2i/rope_dim), i < rope_dim/2
};

// Attention call kinds served by the generic (any dtype / shape) kernel.
enum AttnKind { kSwaPrefill = 0, kSwaDecode = 1, kFullPrefill = 2, kFullDecode = 3 };

struct AttnArgs {
    const void *q;             // q_rot
    const void *k_main;        // staging (SWA prefill) / ring (SWA decode) / pool (full)
    const void *v_main;
    const void *k_ring;        // ring (SWA prefill only)
    const void *v_ring;
    const float *sinks;        // [Hq] or null
    const int64_t *cu_seqlens; // prefill kinds
    const int64_t *start_pos;  // prefill kinds
    const int64_t *pos;        // SWA decode: position of the new token
    const int64_t *ctx_len;    // full decode
    const int64_t *seq_base;   // full kinds
    void *out;
    void *ws;                  // full decode partials
    const unsigned long long *dev_flag;  // checked builds: nonzero once an argument broke the contract
    int64_t n_rows;            // query rows (tokens or sequences)
    int64_t max_seqlen;        // prefill: bound on chunk length; full decode: max_ctx
    int64_t pool_rows;         // full kinds: rows in the pool
    int n_seqs, hq, hkv, dqk, dv, window, chunk, n_chunks;
    float scale, value_scale;
    int kind;
    int qrope;                 // 1: q is unrotated; the kernel applies RoPE to it
    int rope_dim;
    double inv_freq[32];       // theta^(-2i/rope_dim), i < min(rope_dim/2, 32)
};

// Record an error message for hsw_last_error() and return st (hsw_abi.hip).
int32_t fail(int32_t st, const char *fmt, ...);

// Ring snapshots: copy one sequence's ring block of every windowed layer into
// a snapshot (to_snap) or back (kv_manager.hip).
constexpr int kMaxRingLayers = 128;
struct RingCopyArgs {
    char *k[kMaxRingLayers], *v[kMaxRingLayers];  // ring buffers, already offset to the sequence
    char *snap;                                    // the snapshot's first byte
    int64_t kb, vb;                                // K / V block bytes per layer (multiples of 16)
    int n_layers, to_snap;
};
hipError_t launch_ring_copy(const RingCopyArgs &a, hipStream_t s);

// Vision-encoder attention (vit.hip).
struct VitArgs {
    const void *q, *k, *v;
    const int64_t *cu_seqlens;  // [n_images + 1]
    const int32_t *order;       // picture-local token at each position of the order, or null
    const float *sinks;         // learned sink logits [Hq], or null
    void *out;
    const unsigned long long *dev_flag;  // checked builds: nonzero once an argument broke the contract
    int n_images, hq, hkv, window, sink_key;
    float scale;
    // fused 2D RoPE of q and k (window blocks): rope != 0, patch coordinates
    // per token row, and the frequencies theta^(-j / 16), j < 16
    int rope;
    const int32_t *row, *col;
    double rope_f[16];
};
struct VitRopeArgs {
    const void *q, *k;          // either may be null (then not rotated)
    void *q_out, *k_out;
    const int32_t *row, *col;
    int64_t n_tokens;
    int hq, hkv, d;
    double inv_freq[32];        // theta^(-j / (d/4)), j < d/4
};
bool vit_attn_ok(const VitArgs &a, int d_qk, int d_v, int dtype, int out_dtype);
int vit_block_tokens(int G);
hipError_t launch_vit_attn(const VitArgs &a, int64_t max_len, hipStream_t s);
hipError_t launch_vit_rope(const VitRopeArgs &a, hipStream_t s);

hipError_t launch_rope(const RopeArgs &a, int dtype, hipStream_t s);
hipError_t launch_generic_attn(const AttnArgs &a, int dtype, int out_dtype, hipStream_t s);
hipError_t launch_ring_commit(const AttnArgs &a, int dtype, hipStream_t s);
bool swa_decode_fast_ok(const AttnArgs &a, int dtype, int out_dtype);
bool swa_qrope_ok(const AttnArgs &a, int dtype, int out_dtype, bool prefill);
bool full_qrope_ok(const AttnArgs &a, int dtype, int out_dtype, bool prefill);
hipError_t launch_swa_decode(const AttnArgs &a, hipStream_t s);
bool swa_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype);
hipError_t launch_swa_prefill(const AttnArgs &a, hipStream_t s);
bool full_decode_fast_ok(const AttnArgs &a, int dtype, int out_dtype);
hipError_t launch_full_decode(const AttnArgs &a, hipStream_t s);
size_t full_decode_ws_bytes(int64_t n_seqs, int64_t hq, int64_t n_chunks, int64_t dv);
bool full_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype);
hipError_t launch_full_prefill(const AttnArgs &a, hipStream_t s);

}  // namespace hsw
