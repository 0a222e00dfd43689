// full_prefill.hip -- full-attention chunked prefill (bf16 storage, MFMA):
// each query attends causally to every prior row of its sequence plus the
// chunk rows up to itself.
//
// gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", "Tiled global-attention
// prefill": the chunk's queries are split into tiles, each against all keys,
// causality from positions (no materialised bias or mask) and no cross-tile
// merge since softmax is per query row.  colibri "MiMo-V2.6 (Xiaomi)",
// "System One mode and prompt reuse": full layers keep K/V rows by position;
// "What the engine implements": no sink on full layers (one may be passed),
// values carry the value scale (applied to the fp32 output).
//
// MFMA-bound (~6.6e4 flop/B for an 8192-token chunk after 131072 rows).
// One workgroup (4 waves) per (sequence, KV head, 128/G query positions):
// 128 query rows = the G heads of each position as 16-wide MFMA columns, two
// column tiles per wave.  Keys stream through LDS in 32-row chunks, double
// buffered (the next chunk's global loads are in flight while the current one
// computes; one barrier per chunk):
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16 (K rows from LDS, q in VGPRs)
//   softmax          online, log2 units; the reference max is raised only when
//                    a chunk's max exceeds it by more than 2^8 (P <= 256), so
//                    the O rescale is rare
//   O^T += V^T P^T   v_mfma_f32_16x16x32_f16 on fp16 P and fp16 V; the V^T
//                    operand comes straight from row-major V in LDS through the
//                    gfx950 transposing read (ds_read_b64_tr_b16).
// V is converted bf16 -> fp16 once per chunk when it enters LDS (exact for
// |v| < 65520).  A bf16 copy is kept beside it: a chunk holding a value
// outside fp16 range is computed exactly instead, with bf16 V^T and P split
// into bf16 hi + lo (two MFMAs).
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128;
constexpr int STEPS = DQK / 32;
constexpr int DT = DV / 16;
constexpr int KC = 32;                     // keys per chunk
constexpr int KS_STRIDE = DQK + 8;         // bf16 per K row in LDS
constexpr int VS_STRIDE = DV + 16;         // 16-bit elements per V row in LDS
constexpr int K_STAGE = KC * KS_STRIDE;
constexpr int V_STAGE = KC * VS_STRIDE;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(uintptr_t)(const void *)p);
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int full = (total / 8) * 8;
    if (bid >= full) return bid;
    return (bid % 8) * (total / 8) + bid / 8;
}

struct ChunkRegs {
    u32x4 k[3];  // 768 K chunks (32 keys x 24) over 256 threads
    u32x4 v[2];  // 512 V chunks (32 keys x 16)
};

template <int G>
__global__ __launch_bounds__(kThreads, 2) void full_prefill_kernel(AttnArgs a) {
    constexpr int BQ = 128 / G;
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][K_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t vs16[2][V_STAGE];  // fp16
    __shared__ __attribute__((aligned(16))) uint16_t vsbf[2][V_STAGE];  // bf16

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
    const int quad = lane >> 4, col = lane & 15;
    const int nqb = (int)((a.max_seqlen + BQ - 1) / BQ);
    const int total = a.n_seqs * a.hkv * nqb;
    const int bid = xcd_remap(blockIdx.x, total);
    const int qblk = bid % nqb;
    const int g = (bid / nqb) % a.hkv;
    const int s = bid / (nqb * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int len = (int)(a.cu_seqlens[s + 1] - tok0);
    const int local0 = qblk * BQ;
    if (local0 >= len) return;
    const int start = (int)a.start_pos[s];
    const int p0 = start + local0;
    const int plast = start + min(len, local0 + BQ) - 1;  // last query position of the block
    const int64_t base = a.seq_base[s];
    // Keys are rows base + 0 .. base + plast, clamped to the pool.
    int nkeys = plast + 1;
    if (base + nkeys > a.pool_rows) nkeys = (int)(a.pool_rows - base);
    if (base < 0) nkeys = 0;

    const uint16_t *qg = (const uint16_t *)a.q;
    // Uniform per-workgroup bases of this sequence's K/V rows for KV head g;
    // per-thread 32-bit byte offsets from them (row stride hkv * 384 / 256 B;
    // the host bounds contexts so the offsets fit).
    const char *kseq = (const char *)a.k_main + ((base < 0 ? 0 : base) * a.hkv + g) * (int64_t)(DQK * 2);
    const char *vseq = (const char *)a.v_main + ((base < 0 ? 0 : base) * a.hkv + g) * (int64_t)(DV * 2);
    const uint32_t krow = (uint32_t)a.hkv * DQK * 2, vrow = (uint32_t)a.hkv * DV * 2;

    // q of this wave's rows (row r = 32w + 16n + col -> position r / G, head r % G),
    // from a clamped row so the load is unconditional.
    u32x4 qb[2][STEPS];
    int qpos[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        int r = 32 * w + 16 * n + col;
        int local = min(local0 + r / G, len - 1);
        qpos[n] = p0 + r / G;
        const uint16_t *qrow = qg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DQK;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) qb[n][st] = ld16(qrow + 32 * st + 8 * quad);
    }
    const int wpos_lo = p0 + (32 * w) / G, wpos_hi = p0 + (32 * w + 31) / G;
    const int nchunks = (nkeys + KC - 1) / KC;

    auto load_chunk = [&](int c, ChunkRegs &r) {
        const int k0 = c * KC;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            int cc = threadIdx.x + kThreads * i;
            uint32_t key = (uint32_t)min(k0 + cc / (DQK / 8), nkeys - 1);
            r.k[i] = ld16(kseq + (key * krow + 16u * (uint32_t)(cc % (DQK / 8))));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int cc = threadIdx.x + kThreads * i;
            uint32_t key = (uint32_t)min(k0 + cc / (DV / 8), nkeys - 1);
            r.v[i] = ld16(vseq + (key * vrow + 16u * (uint32_t)(cc % (DV / 8))));
        }
    };
    // Returns true if this thread's V values include one outside fp16 range.
    auto store_chunk = [&](int buf, const ChunkRegs &r) -> bool {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            int cc = threadIdx.x + kThreads * i;
            *reinterpret_cast<u32x4 *>(&ks[buf][(cc / (DQK / 8)) * KS_STRIDE + 8 * (cc % (DQK / 8))]) = r.k[i];
        }
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int cc = threadIdx.x + kThreads * i;
            int off = (cc / (DV / 8)) * VS_STRIDE + 8 * (cc % (DV / 8));
            *reinterpret_cast<u32x4 *>(&vsbf[buf][off]) = r.v[i];
            u32x4 h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = bf16x2_to_f16x2(r.v[i][j]);
                bad |= ((h[j] & 0x7c00u) == 0x7c00u) | ((h[j] & 0x7c000000u) == 0x7c000000u);
            }
            *reinterpret_cast<u32x4 *>(&vs16[buf][off]) = h;
        }
        return bad;
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
    // transposing-read lane roles: within a quad's 16 lanes, lane 4k + mm
    // supplies row (4 quad + k) of a 16-key half, dims (16 dt + 4 mm) .. + 3
    const int tr_row = 4 * quad + (col >> 2), tr_col = 4 * (col & 3);

    ChunkRegs regs;
    bool bad = false;
    if (nchunks > 0) {
        load_chunk(0, regs);
        bad = store_chunk(0, regs);
    }
    bool chunk_bad = __syncthreads_or(bad);
    int buf = 0;
    for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        if (more) load_chunk(c + 1, regs);
        const int k0 = c * KC;
        // chunk wholly above every row of this wave: nothing to do (wave-uniform)
        if (k0 <= wpos_hi) {
            const bool interior = k0 + KC - 1 <= wpos_lo && k0 + KC <= nkeys;
            float sv[2][2][4];  // [16-key half][n][j]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 ak[STEPS];
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
                    ak[st] = *reinterpret_cast<const u32x4 *>(&ks[buf][(16 * h + col) * KS_STRIDE + 32 * st + 8 * quad]);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
                    for (int st = 0; st < STEPS; ++st) acc = mfma_16x16x32_bf16(ak[st], qb[n][st], acc);
                    if (interior) {  // wave-uniform: no per-element mask
#pragma unroll
                        for (int j = 0; j < 4; ++j) sv[h][n][j] = acc[j];
                    } else {
                        const int d = min(qpos[n], nkeys - 1) - (k0 + 16 * h + 4 * quad);  // key j visible iff j <= d
#pragma unroll
                        for (int j = 0; j < 4; ++j) sv[h][n][j] = j <= d ? acc[j] : -INFINITY;
                    }
                }
            }
            u32x4 bhi[2], blo[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                float cm = fmaxf(fmaxf(fmaxf(sv[0][n][0], sv[0][n][1]), fmaxf(sv[0][n][2], sv[0][n][3])),
                                 fmaxf(fmaxf(sv[1][n][0], sv[1][n][1]), fmaxf(sv[1][n][2], sv[1][n][3])));
                cm = quad_max(cm) * scale2;
                const bool raise = cm > m[n] + kRescale;
                if (__any(raise)) {
                    const float mn = raise ? cm : m[n];
                    const float f = (m[n] == -INFINITY) ? 0.0f : exp2f(m[n] - mn);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[n][dt] *= f;
                    l[n] *= f;
                    m[n] = mn;
                }
                const float mu = m[n] == -INFINITY ? 0.0f : -m[n];
                float pv[8];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pv[4 * h + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[h][n][j], scale2, mu));
                        l[n] += pv[4 * h + j];
                    }
                if (!chunk_bad) {
                    bhi[n] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]), pack_f16x2(pv[4], pv[5]),
                                   pack_f16x2(pv[6], pv[7])};
                } else {
                    u32x2 h0, l0, h1, l1;
                    split_hi_lo(pv, h0, l0);
                    split_hi_lo(pv + 4, h1, l1);
                    bhi[n] = u32x4{h0[0], h0[1], h1[0], h1[1]};
                    blo[n] = u32x4{l0[0], l0[1], l1[0], l1[1]};
                }
            }
            // O^T += V^T P^T: slots 0-3 of a quad are keys 4quad.. of the first
            // 16-key half, slots 4-7 the same keys of the second half, on both
            // operands.
            if (!chunk_bad) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    u32x2 a0 = ds_read_tr16(&vs16[buf][tr_row * VS_STRIDE + 16 * dt + tr_col]);
                    u32x2 a1 = ds_read_tr16(&vs16[buf][(16 + tr_row) * VS_STRIDE + 16 * dt + tr_col]);
                    u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(av, bhi[n], oacc[n][dt]);
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    u32x2 a0 = ds_read_tr16(&vsbf[buf][tr_row * VS_STRIDE + 16 * dt + tr_col]);
                    u32x2 a1 = ds_read_tr16(&vsbf[buf][(16 + tr_row) * VS_STRIDE + 16 * dt + tr_col]);
                    u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        oacc[n][dt] = mfma_16x16x32_bf16(av, bhi[n], oacc[n][dt]);
                        oacc[n][dt] = mfma_16x16x32_bf16(av, blo[n], oacc[n][dt]);
                    }
                }
            }
        }
        if (more) {
            // buf ^ 1 was last read in iteration c - 1, before the barrier that ended it
            bad = store_chunk(buf ^ 1, regs);
            chunk_bad = __syncthreads_or(bad);
            buf ^= 1;
        }
    }

    // Epilogue: an optional sink joins the denominator once; scale; store bf16.
    uint16_t *outg = (uint16_t *)a.out;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        int r = 32 * w + 16 * n + col;
        int local = local0 + r / G;
        float ll = quad_sum(l[n]);
        if (local >= len) continue;
        int head = r % G;
        float mm = m[n], fac = 1.0f;
        if (a.sinks) {
            float sk = a.sinks[g * G + head] * kLog2e;
            float mf = fmaxf(mm, sk);
            fac = exp2f(mm - mf);
            ll = ll * fac + exp2f(sk - mf);
        }
        float rs = ll > 0.0f ? a.value_scale * fac / ll : 0.0f;
        uint16_t *orow = outg + ((tok0 + local) * a.hq + g * G + head) * (int64_t)DV;
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

bool full_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == 0 &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_full_prefill(const AttnArgs &a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const int BQ = 128 / G;
    const int64_t nqb = (a.max_seqlen + BQ - 1) / BQ;
    dim3 grid((unsigned)(a.n_seqs * a.hkv * nqb)), block(kThreads);
    switch (G) {
        case 1: hipLaunchKernelGGL(full_prefill_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(full_prefill_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(full_prefill_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(full_prefill_kernel<8>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(full_prefill_kernel<16>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
