// dev_check.h -- the contract on device-resident arguments (positions,
// lengths, bases, orders) that include/hsw.h states for each call, as one
// predicate per checked element.
//
// Builds with HSW_CHECK_DEVICE=1 run these predicates in a check kernel
// launched ahead of each call's kernels (check_kernel in hsw_abi.hip); every
// kernel of the call then returns at once when a violation was recorded, so
// nothing reads or writes outside the buffers an out-of-contract value would
// point it to.  Release builds do not check: reading device values on the
// host would need a synchronisation.  The header is plain C++ as well, so a
// host program built with g++ runs the same predicates (the CPU contract
// test).
//
// The rules: positions are 0-based and >= 0 (colibri "MiMo-V2.6 (Xiaomi)",
// "System One mode and prompt reuse": position p lives in ring slot p mod W
// and in pool row base + p); a chunk's rows are cu_seqlens[s] ..
// cu_seqlens[s+1]-1 with lengths in [0, max_seqlen]; a full-attention
// sequence's rows base + 0 .. base + its last position lie inside the pool;
// a decode context length is in [1, max_ctx].
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define HSW_HD __host__ __device__
#else
#define HSW_HD
#endif

namespace hsw {
namespace devcheck {

// Violation codes (the HSW_DEV_* values of include/hsw.h).
enum : int32_t {
    kOk = 0,
    kPosition = 1,    // a position < 0
    kCuSeqlens = 2,   // cu_seqlens[0] < 0, a decreasing entry, or a length > max_seqlen
    kPoolRange = 3,   // a full-attention sequence's rows (base + position) outside [0, pool_rows)
    kRingSeq = 4,     // a ring sequence index outside [0, ring sequences)
    kCtxLen = 5,      // a decode context length outside [1, max_ctx]
    kOrder = 6,       // a vision order entry outside its picture
    kDstRange = 7,    // a RoPE destination row outside dst_capacity, or a negative sequence index
};

// Which call's arguments are checked.
enum : int32_t { kRope = 0, kSwaPrefill = 1, kSwaDecode = 2, kFullDecode = 3, kFullPrefill = 4, kVit = 5 };

struct Inputs {
    int32_t call;
    int32_t dst_kind;           // kRope: 0 ring, 1 pool, 2 staging
    int64_t n;                  // elements: tokens (kRope), sequences, pictures (kVit)
    const int64_t *pos;         // kRope, kSwaDecode
    const int32_t *seq;         // kRope ring / pool
    const int64_t *seq_base;    // kRope pool, kFullDecode, kFullPrefill
    const int64_t *cu_seqlens;  // prefill kinds, kVit
    const int64_t *start_pos;   // prefill kinds
    const int64_t *ctx_len;     // kFullDecode
    const int32_t *order;       // kVit, may be null
    int64_t max_seqlen;         // prefill kinds, kVit (max_len)
    int64_t pool_rows;          // full kinds
    int64_t dst_capacity;       // kRope
    int64_t max_ctx;            // kFullDecode
};

// Contract of element i (token, sequence or picture).  Returns kOk or the
// violation found first, in the order the rules are listed per call.
HSW_HD inline int32_t check_element(const Inputs &in, int64_t i) {
    switch (in.call) {
        case kRope: {
            const int64_t p = in.pos[i];
            if (p < 0) return kPosition;
            if (in.dst_kind == 0) {
                const int64_t s = in.seq[i];
                if (s < 0 || s >= in.dst_capacity) return kRingSeq;
            } else if (in.dst_kind == 1) {
                const int64_t s = in.seq[i];
                if (s < 0) return kDstRange;
                const int64_t r = in.seq_base[s] + p;
                if (r < 0 || r >= in.dst_capacity) return kDstRange;
            } else if (i >= in.dst_capacity) {
                return kDstRange;
            }
            return kOk;
        }
        case kSwaDecode:
            return in.pos[i] < 0 ? kPosition : kOk;
        case kFullDecode: {
            const int64_t L = in.ctx_len[i], b = in.seq_base[i];
            if (L < 1 || L > in.max_ctx) return kCtxLen;
            if (b < 0 || b + L > in.pool_rows) return kPoolRange;
            return kOk;
        }
        case kSwaPrefill:
        case kFullPrefill:
        case kVit: {
            const int64_t c0 = in.cu_seqlens[i], c1 = in.cu_seqlens[i + 1];
            if ((i == 0 && c0 < 0) || c1 < c0 || c1 - c0 > in.max_seqlen) return kCuSeqlens;
            if (in.call == kVit) {
                if (in.order)
                    for (int64_t j = c0; j < c1; ++j)
                        if (in.order[j] < 0 || in.order[j] >= c1 - c0) return kOrder;
                return kOk;
            }
            const int64_t st = in.start_pos[i];
            if (st < 0) return kPosition;
            if (in.call == kFullPrefill) {
                const int64_t b = in.seq_base[i];
                if (b < 0 || b + st + (c1 - c0) > in.pool_rows) return kPoolRange;
            }
            return kOk;
        }
        default:
            return kOk;
    }
}

}  // namespace devcheck
}  // namespace hsw
