// vit.hip -- attention of the vision encoder (ViT): 2D RoPE and
// bidirectional attention over whole pictures or 64-token windows with a
// sink key (bf16 storage, MFMA).
//
// colibri "MiMo-V2.6 (Xiaomi)", the model description's "vision" entry: 2D
// RoPE, grouped-query attention, full attention in 4 of 28 blocks and a 1D
// window of 64 tokens in the others, row and column order of the 2x2 merge
// units alternating; the window blocks add a sink at their leading key.  Read
// here as: a picture's tokens come in merge-unit order; a window block takes
// the tokens in its order (row order = that order, or an index array such
// as the column order of the units), cuts them into consecutive windows of
// 64 and lets each token attend to its window plus the picture's first
// token in that order (the sink key); a full block attends to the whole
// picture; pictures never see each other.  2D RoPE is rotate-half over the
// whole head: pair (i, i + d/2) turns by row * f(i) for i < d/4 and by
// col * f(i - d/4) above, f(j) = theta^(-j / (d/4)).
//
// Attention: one workgroup per (picture, KV head, query block); a block's
// 32 * waves rows are (rows / G) tokens x the G query heads of the KV head
// (heads are the 16-wide MFMA columns, two column tiles per wave), all in one
// window.  Keys stream through LDS 64 at a time (one chunk for a window, the
// whole picture for a full block, double-buffered through registers):
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16 (K from LDS in fragment order)
//   softmax          online in log2 units, the reference max raised only when
//                    a chunk's max exceeds it by more than 2^8
//   O^T += V^T P^T   v_mfma_f32_16x16x32_f16: fp16 P times V converted to
//                    fp16 as it is staged; a chunk holding a value of
//                    magnitude 65536 or more (or a non-finite one) is staged
//                    in bf16 instead and takes P as bf16 hi + lo (two bf16
//                    MFMAs), chosen block-wide.  V^T is read from row-major V
//                    fragments by ds_read_b64_tr_b16.
// The sink key is a fifth 16-key tile (its first row; the rest zero and
// masked) and a third PV step, only in windows after the first.  Queries and
// keys are fetched through the order array, so a block in column order reads
// its rows where they are: no permuted copy of q, k, v or the output.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int D = 64;                 // q, k and v head width
constexpr int STEPS = D / 32;         // k-steps of the S^T product
constexpr int DT = D / 16;            // output tiles of the O^T product
constexpr int KC = 64;                // keys per chunk (= the window)
constexpr int K_TILES = KC / 16 + 1;  // + the sink tile
constexpr int V_HALVES = KC / 16 + 2; // + the sink PV step (two 16-key halves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float quad_max_swap(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float quad_sum_swap(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}
// Consecutive blocks of one (picture, KV head) on one XCD, so the blocks that
// read the same keys share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int full = (total / 8) * 8;
    if (bid >= full) return bid;
    return (bid % 8) * (total / 8) + bid / 8;
}

// ---------------------------------------------------------------- 2D RoPE
// One thread per (token, head, 8-dim piece of the first half): dims
// 8p .. 8p+7 and their partners d/2 + 8p .. (a piece never straddles d/4).
__global__ __launch_bounds__(256) void vit_rope_kernel(VitRopeArgs a) {
    const int pieces = a.d / 16;
    const int nhq = a.q ? a.hq : 0, nhk = a.k ? a.hkv : 0;
    const int64_t per_tok = (int64_t)(nhq + nhk) * pieces;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.n_tokens * per_tok) return;
    const int64_t t = idx / per_tok;
    const int rem = (int)(idx % per_tok);
    const int h = rem / pieces, p = rem % pieces;
    const uint16_t *x;
    uint16_t *y;
    if (h < nhq) {
        x = (const uint16_t *)a.q + (t * a.hq + h) * (int64_t)a.d;
        y = (uint16_t *)a.q_out + (t * a.hq + h) * (int64_t)a.d;
    } else {
        x = (const uint16_t *)a.k + (t * a.hkv + (h - nhq)) * (int64_t)a.d;
        y = (uint16_t *)a.k_out + (t * a.hkv + (h - nhq)) * (int64_t)a.d;
    }
    const int half = a.d / 2, quarter = a.d / 4;
    u32x4 lo = ld16(x + 8 * p), hi = ld16(x + half + 8 * p);
    const bool by_row = 8 * p < quarter;
    const int64_t coord = by_row ? a.row[t] : a.col[t];
    const int f0 = by_row ? 8 * p : 8 * p - quarter;
    float c[8], s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_cos_sin(coord, a.inv_freq[f0 + e], c[e], s[e]);
    rope_rotate_bf16x8(lo, hi, c, s);
    // (non-temporal: the rotated q and k of a whole batch of pictures are
    // larger than the last-level cache, so keeping them there buys nothing)
    __builtin_nontemporal_store(lo, reinterpret_cast<u32x4 *>(y + 8 * p));
    __builtin_nontemporal_store(hi, reinterpret_cast<u32x4 *>(y + half + 8 * p));
}

// -------------------------------------------------------------- attention
// WIN: a window block (one 64-key chunk, the sink tile, one LDS stage);
// otherwise a full block (the picture in 128-key chunks, each computed as two
// 64-key halves, two stages, the next chunk's loads in flight while one is
// computed).
template <int G, bool WIN, bool ROPE = false>
__global__ __launch_bounds__((G == 1 ? 2 : 4) * 64, WIN ? 4 : 2) void vit_attn_kernel(VitArgs a, int nqb) {
    static_assert(!ROPE || WIN, "the fused 2D RoPE is for window blocks");
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    constexpr int NW = G == 1 ? 2 : 4;        // waves: 64 tokens per block at G = 1
    constexpr int NT = NW * 64;
    constexpr int BQ = 32 * NW / G;           // tokens per block; divides 64
    constexpr int KCS = WIN ? KC : 2 * KC;    // keys per stage
    constexpr int PIECES = KCS * D / 8;       // 16-byte pieces of one K (or V) chunk
    constexpr int LOADS = PIECES / NT;        // per thread and tensor
    constexpr int NSTG = WIN ? 1 : 2;
    constexpr int KT = WIN ? K_TILES : KCS / 16;   // 16-key K tiles per stage
    constexpr int VH = WIN ? V_HALVES : KCS / 16;  // 16-key V halves per stage
    static_assert(64 % BQ == 0 && PIECES % NT == 0, "block shape");
    // A stage holds K in MFMA fragment order (16-byte unit (h * STEPS + st) *
    // 64 + lane = K[16h + lane % 16][32st + 8 (lane / 16) ..]) and V in
    // transposing-read order (8-byte unit (hh * DT + dt) * 64 + 16q + 4k + m
    // = V[16hh + 4q + k][16dt + 4m .. +3]), V as fp16 unless the chunk holds
    // a value fp16 cannot (then bf16): every read is one contiguous run in
    // lane order.
    __shared__ __attribute__((aligned(1024))) uint16_t ks[NSTG][KT * 16 * D];
    __shared__ __attribute__((aligned(1024))) uint16_t vs[NSTG][VH * 16 * D];
    // ROPE: (cos, sin) of every rotary pair i < 32 of the window's 64 tokens
    // and the sink token (slot 64), [slot][i][2]
    __shared__ __attribute__((aligned(16))) float rtab[ROPE ? (KC + 1) * 32 * 2 : 2];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int quad = lane >> 4, col = lane & 15;
    const int total = a.n_images * a.hkv * nqb;
    const int bid = xcd_remap((int)__builtin_amdgcn_workgroup_id_x(), total);
    const int qb = bid % nqb;
    const int g = (bid / nqb) % a.hkv;
    const int s = bid / (nqb * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int len = (int)(a.cu_seqlens[s + 1] - tok0);
    if (qb * BQ >= len) return;
    const int32_t *ord = a.order ? a.order + tok0 : nullptr;
    // token row at position j of the block's order (entries clamped into the
    // picture, so a bad index array reads wrong rows but never out of bounds)
    auto row_of = [&](int j) -> int64_t {
        const int t = ord ? min(max(ord[j], 0), len - 1) : j;
        return tok0 + t;
    };
    const int klo = WIN ? (qb * BQ / KC) * KC : 0;
    const int khi = WIN ? min(len, klo + KC) : len;
    const bool has_sink = WIN && a.sink_key && klo > 0;
    const int nch = WIN ? 1 : (len + KCS - 1) / KCS;

    // ROPE: the angles of the window's tokens (slot t: position klo + t of
    // the order, clamped into the picture as the K loads are; slot 64: the
    // sink key at position 0).  Pair i (dims i, i + 32) turns by row * f(i)
    // for i < 16 and by col * f(i - 16) above, formed and reduced as the
    // 2D RoPE call does it, so the rotated bf16 q and k are the bytes that
    // call writes.  Entry u = (slot, quarter qq) holds pairs 8 qq .. 8 qq + 7,
    // which share one coordinate; thread tid takes entries tid + NT m.  The
    // coordinates are loaded after q (table_coords) and the angles formed
    // once the window's K/V loads are in flight (table_angles); the barrier
    // before the first staging publishes them.
    constexpr int TE = (KC + 1) * 4, TM = (TE + NT - 1) / NT;
    int32_t tcoord[ROPE ? TM : 1];   // (32-bit until used: no wait where it lands)
    int tq[2], tkv[WIN ? LOADS : 1], tsk = 0, ttab[ROPE ? TM : 1];   // tokens by order position, below
    const int32_t *rowp = a.row, *colp = a.col;
    auto table_coords = [&]() {
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            // (every thread loads, entries past the table too (token 0 of the
            // order): a load under a branch is waited for where the branch
            // ends; the array is picked as a value, since a pick between two
            // fields of the argument block loads the pointer per lane first)
            const int32_t *coords = ((tid + NT * m) & 3) < 2 ? rowp : colp;
            tcoord[m] = coords[tok0 + ttab[m]];
        }
    };
    auto table_angles = [&]() {
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const int u = tid + NT * m;
            if (u < TE) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 8 * (u & 3) + e;
                    // f(i & 15) = f(8 (u & 1) + e): a pick between two
                    // values the whole workgroup shares (an index per lane
                    // would load from the argument block per lane, behind
                    // the K/V loads)
                    const double f_lo = a.rope_f[e], f_hi = a.rope_f[8 + e];
                    float c, sn;
                    rope_cos_sin((int64_t)tcoord[m], (u & 1) ? f_hi : f_lo, c, sn);
                    rtab[2 * ((u >> 2) * 32 + i)] = c;
                    rtab[2 * ((u >> 2) * 32 + i) + 1] = sn;
                }
            }
        }
    };
    // ROPE: rotate a 16-byte piece of a head row of window slot `slot`:
    // piece p < 4 holds dims 8p .. 8p+7 (the first of each pair), p >= 4 the
    // partners 32 + 8(p - 4) ..; `other` is the partner piece.
    auto rotate_piece = [&](u32x4 mine, u32x4 other, int p, int slot) {
        const bool first = p < 4;
        const u32x4 lo = first ? mine : other, hi = first ? other : mine;
        const float *cs = &rtab[2 * (slot * 32 + 8 * (p & 3))];
        u32x4 y;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            float yl0, yh0, yl1, yh1;
            rope_rotate(__uint_as_float(lo[w2] << 16), __uint_as_float(hi[w2] << 16), cs[4 * w2], cs[4 * w2 + 1],
                        yl0, yh0);
            rope_rotate(__uint_as_float(lo[w2] & 0xffff0000u), __uint_as_float(hi[w2] & 0xffff0000u),
                        cs[4 * w2 + 2], cs[4 * w2 + 3], yl1, yh1);
            y[w2] = first ? pack_bf16x2(yl0, yl1) : pack_bf16x2(yh0, yh1);
        }
        return y;
    };
    auto partner = [&](const u32x4 &x) {   // the piece of lane ^ 4 (piece p ^ 4 of the same key)
        u32x4 o;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) o[w2] = (uint32_t)__shfl_xor((int)x[w2], 4, 64);
        return o;
    };

    const uint16_t *kg = (const uint16_t *)a.k + g * D;
    const uint16_t *vg = (const uint16_t *)a.v + g * D;
    const int64_t rs = (int64_t)a.hkv * D;   // elements per token row of k / v

    // Load i of lane l in wave w moves 16-byte piece p of key `key` of the
    // chunk, b = NW i + w.  Window blocks (HBM-bound): 8 keys x 8 pieces per
    // load for K and V alike (key 8 b + l / 8, piece l % 8), whole 128-byte
    // rows.  Full blocks (bound by issue, where LDS bank conflicts of the
    // staging writes showed): for K, 16 keys x 4 pieces per load (key
    // 16 (b >> 1) + l % 16, piece 4 (b & 1) + l / 16); for V, 8 keys x 8
    // pieces (key 8 b + 4 ((l >> 3) & 1) + ((l >> 1) & 3), piece 2 (l >> 4) +
    // (l & 1)), so the lanes of each 8- and 16-lane group write different LDS
    // bank groups in put (a K unit's bank group is its key mod 16; a V unit's
    // is 8 (key >> 2 & 1) + 2 (key & 3) + (piece & 1)).
    auto k_piece = [&](int i, int &key, int &p) {
        const int b = NW * i + w;
        if constexpr (WIN) {
            key = 8 * b + (lane >> 3);
            p = lane & 7;
        } else {
            key = 16 * (b >> 1) + (lane & 15);
            p = 4 * (b & 1) + (lane >> 4);
        }
    };
    auto v_piece = [&](int i, int &key, int &p) {
        const int b = NW * i + w;
        if constexpr (WIN) {
            key = 8 * b + (lane >> 3);
            p = lane & 7;
        } else {
            key = 8 * b + 4 * ((lane >> 3) & 1) + ((lane >> 1) & 3);
            p = 2 * (lane >> 4) + (lane & 1);
        }
    };
    // The block's tokens by order position, every lookup issued before any
    // is used: with an index array, a lookup whose row feeds a load at once
    // makes the compiler wait for every load in flight after each one, so
    // the block's q, K/V, sink and table loads would each wait a memory
    // latency behind the one before.  tq: q / output rows (n = 0, 1);
    // window blocks: tkv the K/V pieces of the window, tsk the sink (order
    // position 0), ttab the RoPE table's entries (declared with tcoord).
    {
        int jq[2], jkv[WIN ? LOADS : 1], jt[ROPE ? TM : 1];
#pragma unroll
        for (int n = 0; n < 2; ++n) jq[n] = min(qb * BQ + (32 * w + 16 * n + col) / G, len - 1);
        if constexpr (WIN) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                int key, p;
                k_piece(i, key, p);
                jkv[i] = min(klo + key, khi - 1);
            }
        }
        if constexpr (ROPE) {
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                const int u = tid + NT * m, slot = u >> 2;
                jt[m] = u < TE && slot < KC ? min(klo + slot, khi - 1) : 0;
            }
        }
        auto clampt = [&](int t) { return min(max(t, 0), len - 1); };
        if (ord) {
#pragma unroll
            for (int n = 0; n < 2; ++n) tq[n] = ord[jq[n]];
            if constexpr (WIN) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) tkv[i] = ord[jkv[i]];
                tsk = ord[0];
            }
            if constexpr (ROPE) {
#pragma unroll
                for (int m = 0; m < TM; ++m) ttab[m] = ord[jt[m]];
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) tq[n] = clampt(tq[n]);
#pragma unroll
            for (int i = 0; i < (WIN ? LOADS : 0); ++i) tkv[i] = clampt(tkv[i]);
            tsk = clampt(tsk);
#pragma unroll
            for (int m = 0; m < (ROPE ? TM : 0); ++m) ttab[m] = clampt(ttab[m]);
        } else {
#pragma unroll
            for (int n = 0; n < 2; ++n) tq[n] = jq[n];
#pragma unroll
            for (int i = 0; i < (WIN ? LOADS : 0); ++i) tkv[i] = jkv[i];
#pragma unroll
            for (int m = 0; m < (ROPE ? TM : 0); ++m) ttab[m] = jt[m];
        }
    }

    // q of this wave's rows: row r = 32w + 16n + col is token qb*BQ + r/G,
    // head g*G + r%G (rows past the picture read its last token, never stored)
    u32x4 qv[2][STEPS];
    const uint16_t *qg = (const uint16_t *)a.q;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = 32 * w + 16 * n + col;
        const uint16_t *qrow = qg + ((tok0 + tq[n]) * a.hq + g * G + r % G) * (int64_t)D;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) qv[n][st] = ld16(qrow + 32 * st + 8 * quad);
    }

    u32x4 kr[LOADS], vr[LOADS];
    auto fetch = [&](int c) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            int key, p;
            k_piece(i, key, p);
            const int64_t r = WIN ? tok0 + tkv[i] : row_of(min(klo + c * KCS + key, khi - 1));
            kr[i] = ld16(kg + r * rs + 8 * p);
            if constexpr (WIN) {
                vr[i] = ld16(vg + r * rs + 8 * p);  // the same piece of V: one lookup of the order
            } else {
                v_piece(i, key, p);
                vr[i] = ld16(vg + row_of(min(klo + c * KCS + key, khi - 1)) * rs + 8 * p);
            }
        }
    };
    // Any value of V pieces beyond fp16: bf16 magnitude bits at or above
    // 0x4780 (|v| >= 65536, the first bf16 value fp16 cannot hold; infinity
    // and NaN above it), from a packed 16-bit maximum of the magnitude bits
    // (two instructions per word).
    auto mag_max = [&](u16x2 mx, const u32x4 &x) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, x[e] & 0x7fff7fffu));
        return mx;
    };
    auto beyond_f16 = [&](u16x2 mx) { return mx[0] >= 0x4780 || mx[1] >= 0x4780; };
    auto v_big = [&](const u32x4 &x) { return beyond_f16(mag_max(u16x2{0, 0}, x)); };
    auto to_f16 = [&](u32x4 x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16x2_to_f16x2(x[e]);
        return x;
    };
    auto k_unit = [](int key, int p) { return ((key >> 4) * STEPS + (p >> 2)) * 64 + 16 * (p & 3) + (key & 15); };
    auto v_unit = [](int key, int p) {
        return ((key >> 4) * DT + (p >> 1)) * 64 + 16 * ((key & 15) >> 2) + 4 * (key & 3) + 2 * (p & 1);
    };
    auto put = [&](int stg, bool f16) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            int key, p;
            k_piece(i, key, p);
            if constexpr (ROPE) kr[i] = rotate_piece(kr[i], partner(kr[i]), p, key);
            *reinterpret_cast<u32x4 *>(&ks[stg][k_unit(key, p) * 8]) = kr[i];
            v_piece(i, key, p);
            *reinterpret_cast<u32x4 *>(&vs[stg][v_unit(key, p) * 4]) = f16 ? to_f16(vr[i]) : vr[i];
        }
    };
    auto chunk_big = [&](bool extra) {
        u16x2 mx = u16x2{0, 0};
#pragma unroll
        for (int i = 0; i < LOADS; ++i) mx = mag_max(mx, vr[i]);
        return extra || beyond_f16(mx);
    };

    // First chunk (and, in a window after the first, the sink key: slot 64 =
    // the picture's first token in the block's order; slots 65..79 of K and
    // 65..95 of V zero).
    if constexpr (ROPE) table_coords();
    u32x4 sk = u32x4{0, 0, 0, 0}, svv = u32x4{0, 0, 0, 0};
    if (has_sink && tid < 8) {
        const int64_t r0 = tok0 + tsk;
        sk = ld16(kg + r0 * rs + 8 * tid);
        svv = ld16(vg + r0 * rs + 8 * tid);
    }
    fetch(0);
    if constexpr (ROPE) table_angles();
    bool f16 = !__syncthreads_or(chunk_big(has_sink && tid < 8 && v_big(svv)));
    if constexpr (ROPE) {
        // q: lane (quad, col) holds dims 8 quad .. (step 0) and their
        // partners 32 + 8 quad .. (step 1) of its rows' tokens
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int r = 32 * w + 16 * n + col;
            const int slot = min(qb * BQ + r / G, len - 1) - klo;
            const u32x4 lo = qv[n][0];
            qv[n][0] = rotate_piece(lo, qv[n][1], quad, slot);
            qv[n][1] = rotate_piece(qv[n][1], lo, quad + 4, slot);
        }
        // the sink key's pieces (threads 0..7 of wave 0, piece tid)
        const u32x4 sko = partner(sk);
        if (has_sink && tid < 8) sk = rotate_piece(sk, sko, tid, KC);
    }
    put(0, f16);
    if (WIN && has_sink) {
        for (int pi = tid; pi < 32 * 8; pi += NT) {
            const int kk = pi >> 3, p = pi & 7;
            const u32x4 z = u32x4{0, 0, 0, 0};
            if (kk < 16) *reinterpret_cast<u32x4 *>(&ks[0][k_unit(KC + kk, p) * 8]) = kk == 0 ? sk : z;
            *reinterpret_cast<u32x4 *>(&vs[0][v_unit(KC + kk, p) * 4]) = kk == 0 ? (f16 ? to_f16(svv) : svv) : z;
        }
    }
    __syncthreads();

    const float scale2 = a.scale * kLog2e;
    f32x4 oacc[2][DT];
    float m[2], l[2];
    // full blocks: row sums of the same P the PV product takes, from an MFMA
    // of P against an all-ones operand (every lane then holds its column's
    // whole sum), instead of a VALU add per score
    f32x4 lacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        m[n] = -INFINITY;
        l[n] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[n][dt] = f32x4{0, 0, 0, 0};
    }

    // A window: the wave's two column tiles one after the other (fewer live
    // registers: four waves per SIMD), the sink tile when the window has one.
    auto compute = [&](int stg, int c, bool sink, bool vf16) {
        const uint16_t *ksc = ks[stg];
        const uint16_t *vsc = vs[stg];
        const int nvalid = khi - (klo + c * KC);   // keys of this chunk in range (>= 1)
        const bool interior = nvalid >= KC;
        const int nsteps = sink ? 3 : 2;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float sv[K_TILES][4];
#pragma unroll
            for (int h = 0; h < K_TILES; ++h) {
                if (h == K_TILES - 1 && !sink) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[h][j] = -INFINITY;
                    continue;
                }
                f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
                    acc = mfma_16x16x32_bf16(*reinterpret_cast<const u32x4 *>(ksc + ((h * STEPS + st) * 64 + lane) * 8),
                                             qv[n][st], acc);
                if (h == K_TILES - 1) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[h][j] = (quad == 0 && j == 0) ? acc[j] : -INFINITY;
                } else if (interior) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[h][j] = acc[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[h][j] = 16 * h + 4 * quad + j < nvalid ? acc[j] : -INFINITY;
                }
            }
            float cm = -INFINITY;
#pragma unroll
            for (int h = 0; h < K_TILES; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) cm = fmaxf(cm, sv[h][j]);
            cm = quad_max_swap(cm) * scale2;
            const bool raise = cm > m[n] + kRescale;
            if (__any(raise)) {
                const float mn = raise ? cm : m[n];
                if (__any(raise && m[n] != -INFINITY)) {
                    const float f = (m[n] == -INFINITY) ? 0.0f : exp2f(m[n] - mn);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[n][dt] *= f;
                    l[n] *= f;
                }
                m[n] = mn;
            }
            const float mu = m[n] == -INFINITY ? 0.0f : -m[n];
            float pv[K_TILES + 1][4];   // + a zero half pairing with the sink tile
#pragma unroll
            for (int h = 0; h < K_TILES; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pv[h][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[h][j], scale2, mu));
                    l[n] += pv[h][j];
                }
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[K_TILES][j] = 0.0f;
            // O^T += V^T P^T over 32-key steps: slots 0-3 of a quad are keys
            // 4quad.. of the step's first 16-key half, slots 4-7 of its
            // second half, on both operands.  fp16 P (<= 2^8) x fp16 V, or,
            // for a chunk kept in bf16, P as bf16 hi + lo x bf16 V.
#pragma unroll
            for (int s2 = 0; s2 < 3; ++s2) {
                if (s2 >= nsteps) break;
                const float *p0 = pv[2 * s2], *p1 = pv[2 * s2 + 1];
                if (vf16) {
                    const u32x4 pf = u32x4{pack_f16x2(p0[0], p0[1]), pack_f16x2(p0[2], p0[3]),
                                           pack_f16x2(p1[0], p1[1]), pack_f16x2(p1[2], p1[3])};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const u32x2 a0 = ds_read_tr16(vsc + ((2 * s2 * DT + dt) * 64 + lane) * 4);
                        const u32x2 a1 = ds_read_tr16(vsc + (((2 * s2 + 1) * DT + dt) * 64 + lane) * 4);
                        oacc[n][dt] = mfma_16x16x32_f16(u32x4{a0[0], a0[1], a1[0], a1[1]}, pf, oacc[n][dt]);
                    }
                } else {
                    u32x2 h0, l0, h1, l1;
                    split_hi_lo(p0, h0, l0);
                    split_hi_lo(p1, h1, l1);
                    const u32x4 ph = u32x4{h0[0], h0[1], h1[0], h1[1]};
                    const u32x4 pl = u32x4{l0[0], l0[1], l1[0], l1[1]};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const u32x2 a0 = ds_read_tr16(vsc + ((2 * s2 * DT + dt) * 64 + lane) * 4);
                        const u32x2 a1 = ds_read_tr16(vsc + (((2 * s2 + 1) * DT + dt) * 64 + lane) * 4);
                        const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
                        oacc[n][dt] = mfma_16x16x32_bf16(av, ph, oacc[n][dt]);
                        oacc[n][dt] = mfma_16x16x32_bf16(av, pl, oacc[n][dt]);
                    }
                }
            }
        }
    };

    // A full block's chunk: both column tiles together, so every K and V^T
    // fragment read from LDS feeds two MFMAs; four key tiles, no sink.
    auto compute_full = [&](int stg, int c, int hf, bool vf16) {
        constexpr int NKT = KC / 16;
        const uint16_t *ksc = ks[stg] + hf * (NKT * STEPS * 64 * 8);   // the half's K tiles
        const uint16_t *vsc = vs[stg] + hf * (NKT * DT * 64 * 4);      // and V halves
        const int nvalid = khi - (klo + c * KCS + hf * KC);
        const bool interior = nvalid >= KC;
        float sv[2][NKT][4];
#pragma unroll
        for (int h = 0; h < NKT; ++h) {
            u32x4 ak[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
                ak[st] = *reinterpret_cast<const u32x4 *>(ksc + ((h * STEPS + st) * 64 + lane) * 8);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < STEPS; ++st) acc = mfma_16x16x32_bf16(ak[st], qv[n][st], acc);
                if (interior) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[n][h][j] = acc[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[n][h][j] = 16 * h + 4 * quad + j < nvalid ? acc[j] : -INFINITY;
                }
            }
        }
        float pv[2][NKT][4];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float cm = -INFINITY;
#pragma unroll
            for (int h = 0; h < NKT; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) cm = fmaxf(cm, sv[n][h][j]);
            cm = quad_max_swap(cm) * scale2;
            const bool raise = cm > m[n] + kRescale;
            if (__any(raise)) {
                const float mn = raise ? cm : m[n];
                if (__any(raise && m[n] != -INFINITY)) {
                    const float f = (m[n] == -INFINITY) ? 0.0f : exp2f(m[n] - mn);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[n][dt] *= f;
                    lacc[n] *= f;
                }
                m[n] = mn;
            }
            const float mu = m[n] == -INFINITY ? 0.0f : -m[n];
#pragma unroll
            for (int h = 0; h < NKT; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) pv[n][h][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[n][h][j], scale2, mu));
        }
        constexpr uint32_t kOnesF16 = 0x3c003c00u, kOnesBf16 = 0x3f803f80u;
#pragma unroll
        for (int s2 = 0; s2 < NKT / 2; ++s2) {
            if (vf16) {
                u32x4 pf[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const float *p0 = pv[n][2 * s2], *p1 = pv[n][2 * s2 + 1];
                    pf[n] = u32x4{pack_f16x2(p0[0], p0[1]), pack_f16x2(p0[2], p0[3]), pack_f16x2(p1[0], p1[1]),
                                  pack_f16x2(p1[2], p1[3])};
                }
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    lacc[n] = mfma_16x16x32_f16(u32x4{kOnesF16, kOnesF16, kOnesF16, kOnesF16}, pf[n], lacc[n]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2 a0 = ds_read_tr16(vsc + ((2 * s2 * DT + dt) * 64 + lane) * 4);
                    const u32x2 a1 = ds_read_tr16(vsc + (((2 * s2 + 1) * DT + dt) * 64 + lane) * 4);
                    const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(av, pf[n], oacc[n][dt]);
                }
            } else {
                u32x4 ph[2], pl[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    u32x2 h0, l0, h1, l1;
                    split_hi_lo(pv[n][2 * s2], h0, l0);
                    split_hi_lo(pv[n][2 * s2 + 1], h1, l1);
                    ph[n] = u32x4{h0[0], h0[1], h1[0], h1[1]};
                    pl[n] = u32x4{l0[0], l0[1], l1[0], l1[1]};
                    const u32x4 ones = u32x4{kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
                    lacc[n] = mfma_16x16x32_bf16(ones, ph[n], lacc[n]);
                    lacc[n] = mfma_16x16x32_bf16(ones, pl[n], lacc[n]);
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2 a0 = ds_read_tr16(vsc + ((2 * s2 * DT + dt) * 64 + lane) * 4);
                    const u32x2 a1 = ds_read_tr16(vsc + (((2 * s2 + 1) * DT + dt) * 64 + lane) * 4);
                    const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        oacc[n][dt] = mfma_16x16x32_bf16(av, ph[n], oacc[n][dt]);
                        oacc[n][dt] = mfma_16x16x32_bf16(av, pl[n], oacc[n][dt]);
                    }
                }
            }
        }
    };

    if constexpr (WIN) {
        compute(0, 0, has_sink, f16);
    } else {
        for (int c = 0; c < nch; ++c) {
            const int stg = c & 1;
            if (c + 1 < nch) fetch(c + 1);
            compute_full(stg, c, 0, f16);
            if (c * KCS + KC < len) compute_full(stg, c, 1, f16);
            if (c + 1 < nch) {
                f16 = !__syncthreads_or(chunk_big(false));
                put(stg ^ 1, f16);
            }
            __syncthreads();
        }
    }

    // Epilogue: learned sink (if any) in the denominator, normalise, bf16.
    uint16_t *og = (uint16_t *)a.out;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = 32 * w + 16 * n + col;
        const int j = qb * BQ + r / G;
        const int head = r % G;
        float ll = WIN ? quad_sum_swap(l[n]) : lacc[n][0];
        float fac = 1.0f;
        if (a.sinks) {
            const float sk2 = a.sinks[g * G + head] * kLog2e;
            const float mf = fmaxf(m[n], sk2);
            fac = exp2f(m[n] - mf);
            ll = ll * fac + exp2f(sk2 - mf);
        }
        const float sc = fac / ll;
        if (j < len) {
            uint16_t *orow = og + ((tok0 + tq[n]) * a.hq + g * G + head) * (int64_t)D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o = oacc[n][dt];
                *reinterpret_cast<u32x2 *>(orow + 16 * dt + 4 * quad) =
                    u32x2{pack_bf16x2(o[0] * sc, o[1] * sc), pack_bf16x2(o[2] * sc, o[3] * sc)};
            }
        }
    }
}

}  // namespace

bool vit_attn_ok(const VitArgs &a, int d_qk, int d_v, int dtype, int out_dtype) {
    const int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && d_qk == D && d_v == D && (a.window == 0 || a.window == KC) &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

int vit_block_tokens(int G) { return G == 1 ? 64 : 128 / G; }

hipError_t launch_vit_attn(const VitArgs &a, int64_t max_len, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const int BQ = vit_block_tokens(G);
    const int nqb = (int)((max_len + BQ - 1) / BQ);
    dim3 grid((unsigned)((int64_t)a.n_images * a.hkv * nqb));
    if (a.rope) {   // window blocks only (the caller checks)
        switch (G) {
            case 1: hipLaunchKernelGGL((vit_attn_kernel<1, true, true>), grid, dim3(128), 0, s, a, nqb); break;
            case 2: hipLaunchKernelGGL((vit_attn_kernel<2, true, true>), grid, dim3(256), 0, s, a, nqb); break;
            case 4: hipLaunchKernelGGL((vit_attn_kernel<4, true, true>), grid, dim3(256), 0, s, a, nqb); break;
            case 8: hipLaunchKernelGGL((vit_attn_kernel<8, true, true>), grid, dim3(256), 0, s, a, nqb); break;
            default: hipLaunchKernelGGL((vit_attn_kernel<16, true, true>), grid, dim3(256), 0, s, a, nqb); break;
        }
    } else if (a.window > 0) {
        switch (G) {
            case 1: hipLaunchKernelGGL((vit_attn_kernel<1, true>), grid, dim3(128), 0, s, a, nqb); break;
            case 2: hipLaunchKernelGGL((vit_attn_kernel<2, true>), grid, dim3(256), 0, s, a, nqb); break;
            case 4: hipLaunchKernelGGL((vit_attn_kernel<4, true>), grid, dim3(256), 0, s, a, nqb); break;
            case 8: hipLaunchKernelGGL((vit_attn_kernel<8, true>), grid, dim3(256), 0, s, a, nqb); break;
            default: hipLaunchKernelGGL((vit_attn_kernel<16, true>), grid, dim3(256), 0, s, a, nqb); break;
        }
    } else {
        switch (G) {
            case 1: hipLaunchKernelGGL((vit_attn_kernel<1, false>), grid, dim3(128), 0, s, a, nqb); break;
            case 2: hipLaunchKernelGGL((vit_attn_kernel<2, false>), grid, dim3(256), 0, s, a, nqb); break;
            case 4: hipLaunchKernelGGL((vit_attn_kernel<4, false>), grid, dim3(256), 0, s, a, nqb); break;
            case 8: hipLaunchKernelGGL((vit_attn_kernel<8, false>), grid, dim3(256), 0, s, a, nqb); break;
            default: hipLaunchKernelGGL((vit_attn_kernel<16, false>), grid, dim3(256), 0, s, a, nqb); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_vit_rope(const VitRopeArgs &a, hipStream_t s) {
    const int64_t per_tok = (int64_t)((a.q ? a.hq : 0) + (a.k ? a.hkv : 0)) * (a.d / 16);
    const int64_t n = a.n_tokens * per_tok;
    hipLaunchKernelGGL(vit_rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hsw
