// prefill_attn.hip -- chunked prefill attention (bf16 storage, MFMA):
// the banded sliding-window prefill with a per-head sink, and the same tile
// machinery over a full-attention pool (causal over all prior rows).
//
// gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", "What was built": windowed
// prefill runs as banded tiles with an fp32 softmax that includes the sink;
// "Tiled global-attention prefill": softmax is per query row, so query tiles
// need no merge.  colibri "MiMo-V2.6 (Xiaomi)", "What the engine implements":
// each query sees the last 128 positions (itself included), the sink logit
// joins the denominator only, values carry the value scale (applied to the
// fp32 output).  colibri "System One mode and prompt reuse": keys before the
// chunk start come from ring slot p mod 128.
//
// Work unit: one workgroup per (sequence, KV head, block of 128/G query
// positions).  The block's G heads x 128/G positions form 128 query rows =
// eight 16-row MFMA column tiles; wave w owns rows [32w, 32w+32).  Keys are
// streamed in 16-position tiles aligned to multiples of 16: a block touches
// at most ceil((128/G + 127)/16) + 1 tiles, 9 for G = 8 (144 keys computed
// for the 128 each query needs).  Per tile:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, K from LDS, Q held in VGPRs
//   online softmax   fp32 in log2 units, max over the tile's keys per row
//   O^T += V^T P^T   v_mfma_f32_16x16x16_bf16, P as bf16 hi + lo (two MFMAs)
// K/V tiles are double-buffered in LDS (next tile's global loads in flight
// while the current tile computes); V is stored transposed so each MFMA
// A operand is one 8-byte LDS read.  Block ids are remapped so that
// consecutive query blocks of one (sequence, KV head) run on the same XCD and
// re-read the overlapping band from that XCD's L2.
//
// Full-attention layers (FULL = true; gaudi-cookbook "Tiled global-attention
// prefill": query tiles against all keys, causality from the positions, no
// materialised mask or score matrix) take keys 0 .. p of the sequence from
// pool rows seq_base + position and have no sink unless one is passed.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128, W = 128;
constexpr int STEPS = DQK / 32;
constexpr int DT = DV / 16;
constexpr int KT = 16;                     // keys per tile
constexpr int K_CHUNKS = KT * DQK / 8;     // 16-byte chunks per K tile (384)
constexpr int V_CHUNKS = KT * DV / 8;      // 16-byte chunks per V tile (256)
constexpr int VT_STRIDE = KT + 4;          // bf16 per transposed V row (16 keys + pad)
constexpr int KS_STRIDE = DQK + 8;         // bf16 per K row in LDS (pad spreads banks)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct TileRegs {
    u32x4 k0, k1, v;
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int full = (total / 8) * 8;
    if (bid >= full) return bid;
    return (bid % 8) * (total / 8) + bid / 8;
}

template <int G, bool FULL>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(AttnArgs a) {
    constexpr int BQ = 128 / G;  // query positions per block
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][KT * KS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t vts[2][DV * VT_STRIDE];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int quad = lane >> 4, col = lane & 15;
    const int nqb = (int)((a.max_seqlen + BQ - 1) / BQ);
    const int total = a.n_seqs * a.hkv * nqb;
    const int bid = xcd_remap(blockIdx.x, total);
    const int qblk = bid % nqb;
    const int g = (bid / nqb) % a.hkv;
    const int s = bid / (nqb * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int64_t len = a.cu_seqlens[s + 1] - tok0;
    const int64_t local0 = (int64_t)qblk * BQ;
    if (local0 >= len) return;  // whole block past this sequence's chunk
    const int64_t start = a.start_pos[s];
    const int64_t p0 = start + local0;                 // first query position
    const int64_t plast = start + min(len, local0 + BQ) - 1;

    const uint16_t *qg = (const uint16_t *)a.q;
    const uint16_t *kst = (const uint16_t *)a.k_main;
    const uint16_t *vst = (const uint16_t *)a.v_main;
    const uint16_t *kring = FULL ? nullptr : (const uint16_t *)a.k_ring + ((int64_t)(s * a.hkv + g) * W) * DQK;
    const uint16_t *vring = FULL ? nullptr : (const uint16_t *)a.v_ring + ((int64_t)(s * a.hkv + g) * W) * DV;
    const int64_t pool_base = FULL ? a.seq_base[s] : 0;

    // This wave's two column tiles: row r = 32w + 16n + col -> (position, head).
    int64_t qpos[2];
    bool qvalid[2];
    u32x4 qb[2][STEPS];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        int r = 32 * w + 16 * n + col;
        int off = r / G, head = r % G;
        qpos[n] = p0 + off;
        qvalid[n] = local0 + off < len;
        const uint16_t *qrow = qg + ((tok0 + local0 + off) * a.hq + g * G + head) * (int64_t)DQK;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            qb[n][st] = qvalid[n] ? ld16(qrow + 32 * st + 8 * quad) : u32x4{0, 0, 0, 0};
    }
    // Positions this wave's rows span, for skipping tiles wholly outside.
    const int64_t wpos_lo = p0 + (32 * w) / G;
    const int64_t wpos_hi = p0 + (32 * w + 31) / G;

    // Key tiles covering positions max(0, p0-W+1) .. plast (0 .. plast when full).
    int64_t first = FULL ? 0 : p0 - (W - 1);
    if (first < 0) first = 0;
    const int64_t t_lo = first / KT, t_hi = plast / KT;

    // Source of the key at position kp: ring before the chunk, staging inside.
    auto load_tile = [&](int64_t t, TileRegs &r) {
        const int64_t kbase = t * KT;
        {
            int c = threadIdx.x;  // K chunk c: key c / 24, 16-byte piece c % 24
            int key = c / (DQK / 8), piece = c % (DQK / 8);
            int64_t kp = kbase + key;
            const uint16_t *src = nullptr;
            if (FULL) {
                int64_t row = pool_base + kp;
                if (kp >= 0 && kp <= plast && row >= 0 && row < a.pool_rows) src = kst + (row * a.hkv + g) * (int64_t)DQK;
            } else if (kp >= 0 && kp < start) {
                src = kring + (kp % W) * DQK;
            } else if (kp >= start && kp <= plast) {
                src = kst + ((tok0 + kp - start) * a.hkv + g) * (int64_t)DQK;
            }
            r.k0 = src ? ld16(src + 8 * piece) : u32x4{0, 0, 0, 0};
        }
        if (threadIdx.x < K_CHUNKS - kThreads) {
            int c = threadIdx.x + kThreads;
            int key = c / (DQK / 8), piece = c % (DQK / 8);
            int64_t kp = kbase + key;
            const uint16_t *src = nullptr;
            if (FULL) {
                int64_t row = pool_base + kp;
                if (kp >= 0 && kp <= plast && row >= 0 && row < a.pool_rows) src = kst + (row * a.hkv + g) * (int64_t)DQK;
            } else if (kp >= 0 && kp < start) {
                src = kring + (kp % W) * DQK;
            } else if (kp >= start && kp <= plast) {
                src = kst + ((tok0 + kp - start) * a.hkv + g) * (int64_t)DQK;
            }
            r.k1 = src ? ld16(src + 8 * piece) : u32x4{0, 0, 0, 0};
        }
        {
            int c = threadIdx.x;  // V chunk c: key c / 16, 8 dims at 8 * (c % 16)
            int key = c / (DV / 8), piece = c % (DV / 8);
            int64_t kp = kbase + key;
            const uint16_t *src = nullptr;
            if (FULL) {
                int64_t row = pool_base + kp;
                if (kp >= 0 && kp <= plast && row >= 0 && row < a.pool_rows) src = vst + (row * a.hkv + g) * (int64_t)DV;
            } else if (kp >= 0 && kp < start) {
                src = vring + (kp % W) * DV;
            } else if (kp >= start && kp <= plast) {
                src = vst + ((tok0 + kp - start) * a.hkv + g) * (int64_t)DV;
            }
            r.v = src ? ld16(src + 8 * piece) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf, const TileRegs &r) {
        {
            int c = threadIdx.x;
            *reinterpret_cast<u32x4 *>(&ks[buf][(c / (DQK / 8)) * KS_STRIDE + 8 * (c % (DQK / 8))]) = r.k0;
        }
        if (threadIdx.x < K_CHUNKS - kThreads) {
            int c = threadIdx.x + kThreads;
            *reinterpret_cast<u32x4 *>(&ks[buf][(c / (DQK / 8)) * KS_STRIDE + 8 * (c % (DQK / 8))]) = r.k1;
        }
        int key = threadIdx.x / (DV / 8), dv0 = 8 * (threadIdx.x % (DV / 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t word = r.v[e >> 1];
            vts[buf][(dv0 + e) * VT_STRIDE + key] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
        }
    };

    f32x4 oacc[2][DT];
    float m[2], l[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        m[n] = -INFINITY;
        l[n] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[n][dt] = f32x4{0, 0, 0, 0};
    }
    const float scale2 = a.scale * kLog2e;

    TileRegs regs;
    load_tile(t_lo, regs);
    store_tile(0, regs);
    __syncthreads();
    int buf = 0;
    for (int64_t t = t_lo; t <= t_hi; ++t) {
        const bool more = t < t_hi;
        if (more) load_tile(t + 1, regs);
        const int64_t kbase = t * KT;
        // Skip a tile that no row of this wave can see (wave-uniform).
        const bool use = kbase <= wpos_hi && (FULL || kbase + KT - 1 > wpos_lo - W);
        if (use) {
            u32x4 ak[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
                ak[st] = *reinterpret_cast<const u32x4 *>(&ks[buf][col * KS_STRIDE + 32 * st + 8 * quad]);
            u32x2 av[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                av[dt] = *reinterpret_cast<const u32x2 *>(&vts[buf][(16 * dt + col) * VT_STRIDE + 4 * quad]);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f32x4 sacc = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < STEPS; ++st) sacc = mfma_16x16x32_bf16(ak[st], qb[n][st], sacc);
                float sv[4], mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int64_t kp = kbase + 4 * quad + i;
                    bool ok = kp <= qpos[n] && (FULL || kp > qpos[n] - W) && kp >= 0;
                    sv[i] = ok ? sacc[i] * scale2 : -INFINITY;
                    mx = fmaxf(mx, sv[i]);
                }
                mx = quad_max(mx);
                float mn = fmaxf(m[n], mx);
                float mu = mn == -INFINITY ? 0.0f : mn;
                float corr = exp2f(m[n] - mu);
                float pv[4], ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = exp2f(sv[i] - mu);
                    ps += pv[i];
                }
                ps = quad_sum(ps);
                l[n] = l[n] * corr + ps;
                m[n] = mn;
                u32x2 hi, lo;
                split_hi_lo(pv, hi, lo);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    oacc[n][dt] *= corr;
                    oacc[n][dt] = mfma_16x16x16_bf16(av[dt], hi, oacc[n][dt]);
                    oacc[n][dt] = mfma_16x16x16_bf16(av[dt], lo, oacc[n][dt]);
                }
            }
        }
        if (more) {
            // buf ^ 1 was last read in iteration t - 1, before the barrier
            // that ended it, so it can be refilled without another barrier.
            store_tile(buf ^ 1, regs);
            __syncthreads();
            buf ^= 1;
        }
    }

    // Epilogue: the sink joins the denominator once; scale; store bf16.
    uint16_t *outg = (uint16_t *)a.out;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        if (!qvalid[n]) continue;
        int r = 32 * w + 16 * n + col;
        int off = r / G, head = r % G;
        float mm = m[n], ll = l[n], fac = 1.0f;
        if (a.sinks) {
            float sk = a.sinks[g * G + head] * kLog2e;
            float mf = fmaxf(mm, sk);
            fac = exp2f(mm - mf);
            ll = ll * fac + exp2f(sk - mf);
        }
        float rs = a.value_scale * fac / ll;
        uint16_t *orow = outg + ((tok0 + local0 + off) * a.hq + g * G + head) * (int64_t)DV;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 o = oacc[n][dt];
            u32x2 pk = u32x2{(uint32_t)f2bf(o[0] * rs) | ((uint32_t)f2bf(o[1] * rs) << 16),
                             (uint32_t)f2bf(o[2] * rs) | ((uint32_t)f2bf(o[3] * rs) << 16)};
            *reinterpret_cast<u32x2 *>(orow + 16 * dt + 4 * quad) = pk;
        }
    }
}

}  // namespace

bool swa_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == W &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

template <bool FULL>
static hipError_t launch_prefill(const AttnArgs &a, hipStream_t s) {
    int G = a.hq / a.hkv;
    int BQ = 128 / G;
    int64_t nqb = (a.max_seqlen + BQ - 1) / BQ;
    dim3 grid((unsigned)(a.n_seqs * a.hkv * nqb)), block(kThreads);
    switch (G) {
        case 1: hipLaunchKernelGGL((prefill_kernel<1, FULL>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<2, FULL>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<4, FULL>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<8, FULL>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((prefill_kernel<16, FULL>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_swa_prefill(const AttnArgs &a, hipStream_t s) { return launch_prefill<false>(a, s); }

}  // namespace hsw
