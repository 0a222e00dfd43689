// swa_decode.hip -- sliding-window decode over the 128-slot ring (bf16, MFMA).
//
// colibri "MiMo-V2.6 (Xiaomi)", "System One mode and prompt reuse": a
// windowed layer keeps position p in ring slot p mod 128, so at decode
// position P slot t holds position P - ((P - t) mod 128); slots whose
// position would be negative (P < 127) are skipped.  gaudi-cookbook
// "MiMo-V2.6-Flash on Gaudi 2", "What was built": the window is exactly the
// last 128 positions and the sink counts once per sequence.  colibri "What
// the engine implements": the sink logit joins the denominator only, values
// are scaled by the value scale (applied here to the fp32 output).
//
// HBM-bound: each (sequence, KV head) -- an "item" -- reads its 48 KiB K ring
// and 32 KiB V ring exactly once.  Persistent workgroups (two per CU, 4 waves)
// walk the items with the next item's bytes always in flight: at the top of
// item i the workgroup issues every load of item i + grid (K and q into a
// second register set, V by direct global->LDS loads into a second LDS
// buffer), then waits only for item i's.  Wave w owns ring slots
// [32w, 32w+32) of an item:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, K rows straight from HBM as the
//                    A operand, the G query heads as the 16 B columns (heads
//                    past G repeat real ones and are never stored);
//   softmax          per wave over its 32 slots, in log2 units;
//   O^T = V^T P^T    v_mfma_f32_16x16x32_bf16 on P split into bf16 hi + lo (P
//                    keeps ~16 bits), V^T read from LDS by ds_read_b64_tr_b16
//                    (V is placed in MFMA fragment order by the loads);
// then the four waves' (max, sum, O) partials meet in LDS (in the V buffer the
// wave has finished with) and are combined with the sink, scaled and stored.
//
// With QROPE the kernel reads unrotated q and applies the rotate-half RoPE
// itself (colibri "What the engine implements"; angle formed and reduced in
// double as the gaudi-cookbook "The RoPE fix for large positions" requires):
// the rotated rotary dims stay fp32 and enter S^T as bf16 hi + lo (two MFMAs
// on those two of the six steps), so q loses nothing to a bf16 q_rot and no
// q_rot is written or read.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128, W = 128;
constexpr int STEPS = DQK / 32;       // 16x16x32 MFMA steps over q/k dims
constexpr int DT = DV / 16;           // 16-wide value tiles
constexpr int kThreads = 256;
constexpr int KEYS = W / 4;           // ring slots per wave
constexpr int K_LOADS = 2 * STEPS;    // per wave per item: K, 16 bytes a lane
constexpr int Q_LOADS = STEPS;        // q
constexpr int V_LOADS = KEYS * DV * 2 / (64 * 16);  // V, direct to LDS (8)
constexpr int LOADS = K_LOADS + Q_LOADS + V_LOADS + 1;  // 27 (+ the position)
constexpr int VBUF = 4 * KEYS * DV;   // bf16 per V buffer (32 KiB)
constexpr int MAX_HQ = 256;           // sinks staged in LDS
constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) alone, and lgkmcnt(0) alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The item loads are inline asm so the compiler does not track them (it would
// otherwise wait for all of them, the next item's included, before the first
// use of any); their completion is awaited explicitly with s_waitcnt vmcnt.
// Vector-memory loads complete in issue order, so "at most LOADS outstanding"
// right after the next item's LOADS were issued means this item's have landed.
__device__ __forceinline__ void load16(u32x4 &v, const void *src) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "+v"(v) : "v"(src) : "memory");
}
__device__ __forceinline__ void load8(u32x2 &v, const void *src) {
    asm volatile("global_load_dwordx2 %0, %1, off" : "+v"(v) : "v"(src) : "memory");
}
// Direct global -> LDS load: lane i's 16 bytes land at lds_wave_base + 16 i.
__device__ __forceinline__ void load_lds16(const void *src, const void *lds_wave_base) {
    const uint32_t m = (uint32_t)(uintptr_t)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

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

__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <int G, bool QROPE>
__global__ __launch_bounds__(kThreads, 2) void swa_decode_kernel(AttnArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    // V of the current and the next item, each wave's 32 slots in its own
    // 8 KiB; after a wave's PV it holds that wave's O partial [G][DV] fp32,
    // 16-byte unit u of head row h stored at unit u ^ (h & 15), so the 16
    // lanes of a quad (16 heads, one unit) write 16 different bank groups.
    __shared__ __attribute__((aligned(1024))) uint16_t vb0[VBUF], vb1[VBUF];
    __shared__ float ml[2][4][16][2];  // (max, sum) per buffer, wave, head
    __shared__ float sk[MAX_HQ];       // sinks in log2 units
    __shared__ float qcs[QROPE ? 4 : 1][64];  // per wave: cos, sin of the item's 32 angles

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int quad = lane >> 4, col = lane & 15;
    const int n_items = a.n_seqs * a.hkv;

    for (int i = threadIdx.x; i < a.hq; i += kThreads) sk[i] = a.sinks ? a.sinks[i] * kLog2e : -INFINITY;
    // frequency (lane mod 32) of the rotary pairs
    // (pinned here, before the first untracked load: see pin_loaded)
    const double invf = QROPE ? pin_loaded(a.inv_freq[lane & 31]) : 0.0;

    // Per-lane constant parts of the load addresses.  K: A operand of the
    // S^T MFMA, lane (quad, col) takes slot 32w + 16h + col, dims 32st + 8quad.
    // V: load i fills 8-byte units (2i + (lane >> 5)) * 64 + (2u, 2u + 1),
    // u = lane & 31, i.e. what lane (quad', 4k + mm) supplies to the
    // transposing read of key half hh = i / 4, tile dt = 2 (i % 4) + (lane >> 5):
    // slot 32w + 16hh + 4 (u >> 3) + ((u >> 1) & 3), bytes 64 (i % 4) +
    // 32 (lane >> 5) + 16 (u & 1).
    const int u = lane & 31;
    const uint32_t koff = (uint32_t)((32 * w + col) * DQK * 2 + 16 * quad);
    const uint32_t voff = (uint32_t)((32 * w + 4 * (u >> 3) + ((u >> 1) & 3)) * DV * 2 + 32 * (lane >> 5) + 16 * (u & 1));
    const uint32_t qoff = (uint32_t)((col % G) * DQK * 2 + 16 * quad);

    auto issue = [&](int item, u32x4 (&ka)[2][STEPS], u32x4 (&qb)[STEPS], uint16_t *vb, u32x2 &pos) {
        const int s = item / a.hkv, g = item % a.hkv;
        load8(pos, a.pos + s);
        const char *K = (const char *)a.k_main + (int64_t)item * W * DQK * 2;
        const char *V = (const char *)a.v_main + (int64_t)item * W * DV * 2;
        const char *Q = (const char *)a.q + ((int64_t)s * a.hq + g * G) * DQK * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int st = 0; st < STEPS; ++st) load16(ka[h][st], K + koff + 16 * h * DQK * 2 + 64 * st);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) load16(qb[st], Q + qoff + 64 * st);
        const char *vw = (const char *)vb + w * KEYS * DV * 2;
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i)
            load_lds16(V + voff + 16 * (i / 4) * DV * 2 + 64 * (i % 4), vw + i * 1024);
    };

    const float scale2 = a.scale * kLog2e;
    auto compute = [&](int item, const u32x4 (&ka)[2][STEPS], const u32x4 (&qb)[STEPS], uint16_t *vb,
                       float (&mlb)[4][16][2], u32x2 pos) {
        const int s = item / a.hkv, g = item % a.hkv;
        const int64_t P = (int64_t)(((uint64_t)pos[1] << 32) | pos[0]);
        const int pc = P < W - 1 ? (int)P : W - 1;  // slot positions >= 0 iff (P - slot) mod W <= pc

        f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
        if constexpr (QROPE) {
            // The item's 32 (cos, sin) pairs through the wave's LDS row, then
            // lane (quad, col) rotates dims 8 quad .. +7 (step 0) against
            // their partners 32 + 8 quad .. (step 1) in fp32 and splits the
            // results into bf16 hi + lo.
            float cv, sv;
            rope_cos_sin(P, invf, cv, sv);
            if (lane < 32) {
                qcs[w][lane] = cv;
                qcs[w][32 + lane] = sv;
            }
            const f32x4 c0 = *reinterpret_cast<const f32x4 *>(&qcs[w][8 * quad]);
            const f32x4 c1 = *reinterpret_cast<const f32x4 *>(&qcs[w][8 * quad + 4]);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&qcs[w][32 + 8 * quad]);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&qcs[w][32 + 8 * quad + 4]);
            const float cc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            const float ss[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            float yl[8], yh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wl = qb[0][e >> 1], wh = qb[1][e >> 1];
                const float xl = __uint_as_float((e & 1) ? (wl & 0xffff0000u) : (wl << 16));
                const float xh = __uint_as_float((e & 1) ? (wh & 0xffff0000u) : (wh << 16));
                rope_rotate(xl, xh, cc[e], ss[e], yl[e], yh[e]);
            }
            u32x2 lh0, ll0, lh1, ll1, hh0, hl0, hh1, hl1;
            split_hi_lo(yl, lh0, ll0);
            split_hi_lo(yl + 4, lh1, ll1);
            split_hi_lo(yh, hh0, hl0);
            split_hi_lo(yh + 4, hh1, hl1);
            const u32x4 q0h = u32x4{lh0[0], lh0[1], lh1[0], lh1[1]}, q0l = u32x4{ll0[0], ll0[1], ll1[0], ll1[1]};
            const u32x4 q1h = u32x4{hh0[0], hh0[1], hh1[0], hh1[1]}, q1l = u32x4{hl0[0], hl0[1], hl1[0], hl1[1]};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                sacc[h] = mfma_16x16x32_bf16(ka[h][0], q0h, sacc[h]);
                sacc[h] = mfma_16x16x32_bf16(ka[h][0], q0l, sacc[h]);
                sacc[h] = mfma_16x16x32_bf16(ka[h][1], q1h, sacc[h]);
                sacc[h] = mfma_16x16x32_bf16(ka[h][1], q1l, sacc[h]);
            }
#pragma unroll
            for (int st = 2; st < STEPS; ++st)
#pragma unroll
                for (int h = 0; h < 2; ++h) sacc[h] = mfma_16x16x32_bf16(ka[h][st], qb[st], sacc[h]);
        } else {
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
#pragma unroll
                for (int h = 0; h < 2; ++h) sacc[h] = mfma_16x16x32_bf16(ka[h][st], qb[st], sacc[h]);
        }

        float sv[8], mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int slot = 32 * w + 16 * h + 4 * quad + j;
                const int back = ((int)(P & (W - 1)) - slot) & (W - 1);  // (P - slot) mod W, any int64 P
                const float v = back <= pc ? sacc[h][j] * scale2 : -INFINITY;
                sv[4 * h + j] = v;
                mx = fmaxf(mx, v);
            }
        mx = quad_max_swap(mx);
        const float mu = mx == -INFINITY ? 0.0f : mx;
        float pv[8], lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(sv[e] - mu);
            lsum += pv[e];
        }
        lsum = quad_sum_swap(lsum);
        u32x2 h0, l0, h1, l1;
        split_hi_lo(pv, h0, l0);
        split_hi_lo(pv + 4, h1, l1);
        const u32x4 bhi = u32x4{h0[0], h0[1], h1[0], h1[1]};
        const u32x4 blo = u32x4{l0[0], l0[1], l1[0], l1[1]};

        // O^T = V^T P^T over the wave's 32 slots: operand slots 0-3 of a quad
        // are keys 4quad.. of the first 16-key half, slots 4-7 of the second.
        uint16_t *vw = vb + w * KEYS * DV;
        f32x4 oacc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x2 a0 = ds_read_tr16(vw + (dt * 64 + lane) * 4);
            const u32x2 a1 = ds_read_tr16(vw + ((DT + dt) * 64 + lane) * 4);
            const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
            oacc[dt] = mfma_16x16x32_bf16(av, bhi, f32x4{0, 0, 0, 0});
            oacc[dt] = mfma_16x16x32_bf16(av, blo, oacc[dt]);
        }
        // The wave's partial over its own V slots (its reads of them are done:
        // LDS accesses of one wave are performed in order).
        float *part = reinterpret_cast<float *>(vw);
        if (col < G) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4 *>(part + col * DV + 4 * ((4 * dt + quad) ^ col)) = oacc[dt];
            if (quad == 0) {
                mlb[w][col][0] = mx;
                mlb[w][col][1] = lsum;
            }
        }
        lds_barrier();

        // Combine the four waves; the sink joins the denominator once.
        uint16_t *out = (uint16_t *)a.out + ((int64_t)s * a.hq + g * G) * DV;
        const float *pbase = reinterpret_cast<const float *>(vb);
        for (int idx = threadIdx.x; idx < G * (DV / 4); idx += kThreads) {
            const int hd = idx / (DV / 4), d4 = 4 * (idx % (DV / 4));
            const float sink2 = sk[g * G + hd];
            float mw[4], M = sink2;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                mw[ww] = mlb[ww][hd][0];
                M = fmaxf(M, mw[ww]);
            }
            float L = __builtin_amdgcn_exp2f(sink2 - M);  // 0 without a sink
            f32x4 o = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float f = __builtin_amdgcn_exp2f(mw[ww] - M);
                L += f * mlb[ww][hd][1];
                o += f * *reinterpret_cast<const f32x4 *>(pbase + ww * (KEYS * DV / 2) + hd * DV +
                                                          4 * ((d4 / 4) ^ (hd & 15)));
            }
            const float r = a.value_scale / L;
            const u32x2 pk = u32x2{pack_bf16x2(o[0] * r, o[1] * r), pack_bf16x2(o[2] * r, o[3] * r)};
            *reinterpret_cast<u32x2 *>(out + hd * DV + d4) = pk;
        }
        // Every wave is done with this buffer before the loads of the item
        // after next are issued into it.
        lds_barrier();
    };

    u32x4 kaA[2][STEPS], kaB[2][STEPS], qbA[STEPS], qbB[STEPS];
    u32x2 pA = u32x2{0, 0}, pB = u32x2{0, 0};
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        qbA[st] = qbB[st] = u32x4{0, 0, 0, 0};
        kaA[0][st] = kaA[1][st] = kaB[0][st] = kaB[1][st] = u32x4{0, 0, 0, 0};
    }
    lds_barrier();  // sinks staged (their global loads were awaited by the compiler)

    int item = blockIdx.x;
    const int grid = gridDim.x;
    issue(item, kaA, qbA, vb0, pA);
    while (true) {
        bool more = item + grid < n_items;
        if (more) {
            issue(item + grid, kaB, qbB, vb1, pB);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __asm__ volatile("" ::: "memory");
        compute(item, kaA, qbA, vb0, ml[0], pA);
        item += grid;
        if (!more) break;
        more = item + grid < n_items;
        if (more) {
            issue(item + grid, kaA, qbA, vb0, pA);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __asm__ volatile("" ::: "memory");
        compute(item, kaB, qbB, vb1, ml[1], pB);
        item += grid;
        if (!more) break;
    }
}

int cu_count() {
    static int n[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (n[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        n[dev] = c;
    }
    return n[dev];
}

}  // namespace

bool swa_decode_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == W && a.hq <= MAX_HQ &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_swa_decode(const AttnArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.n_seqs * a.hkv;
    const int64_t nb = items < 2 * cu_count() ? items : 2 * cu_count();
    dim3 grid((unsigned)nb), block(kThreads);
    if (a.qrope) {
        switch (a.hq / a.hkv) {
            case 1: hipLaunchKernelGGL((swa_decode_kernel<1, true>), grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL((swa_decode_kernel<2, true>), grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL((swa_decode_kernel<4, true>), grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL((swa_decode_kernel<8, true>), grid, block, 0, s, a); break;
            default: hipLaunchKernelGGL((swa_decode_kernel<16, true>), grid, block, 0, s, a); break;
        }
        return hipGetLastError();
    }
    switch (a.hq / a.hkv) {
        case 1: hipLaunchKernelGGL((swa_decode_kernel<1, false>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((swa_decode_kernel<2, false>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((swa_decode_kernel<4, false>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((swa_decode_kernel<8, false>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((swa_decode_kernel<16, false>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
