// full_decode.hip -- full-attention decode over the contiguous pool, split
// over key chunks, with a log-sum-exp combine (bf16 storage, MFMA).
//
// colibri "MiMo-V2.6 (Xiaomi)", "System One mode and prompt reuse": full
// layers keep K/V rows by position.  gaudi-cookbook "MiMo-V2.6-Flash on
// Gaudi 2", "What was built" and "What it taught about Gaudi": decode runs as
// per-block partials, and a sink must count once per sequence, not once per
// block -- so partials carry no sink and the combine adds it exactly once.
// Full layers of MiMo have no sink (colibri "What the engine implements"),
// but one may be passed.
//
// Pass 1: one workgroup per (sequence, KV head, chunk of `chunk` keys); wave
// w takes a contiguous quarter of the chunk in steps of 32 keys.  The G query
// heads of the group are the 16 B columns of S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16, K rows loaded from HBM straight into the A
// operand); an online softmax in log2 units; O^T += V^T P^T
// (v_mfma_f32_16x16x32_bf16, P as bf16 hi + lo; V loaded in MFMA fragment
// order, put in a per-wave LDS tile by 16-byte writes and read back
// transposed by ds_read_b64_tr_b16, free of bank conflicts).  The four
// waves merge in LDS and write one
// (m, l, acc[128]) fp32 partial per (sequence, head, chunk).
// Pass 2: one wave per (sequence, head) merges the chunks:
//   M = max m_c,  Z = sum 2^(m_c - M) l_c (+ 2^(sink - M) once),
//   o = value_scale * sum 2^(m_c - M) acc_c / Z.
// HBM-bound: every K/V row is read exactly once.
//
// With QROPE the partial kernel reads unrotated q and rotates it at the new
// token's position ctx_len - 1 (colibri "What the engine implements"; angle
// in double per the gaudi-cookbook "The RoPE fix for large positions"); the
// rotated rotary dims stay fp32 and enter S^T as bf16 hi + lo, so no bf16
// q_rot is written, read or rounded.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128;
constexpr int STEPS = DQK / 32;
constexpr int DT = DV / 16;
constexpr int KS = 32;                 // keys per wave step
constexpr int VSTEP = KS * DV;         // bf16 of one wave's V tile (8 KiB)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

struct StepRegs {
    u32x4 k[2][STEPS];
    u32x4 v[8];
};

template <int G, bool QROPE>
__global__ __launch_bounds__(kThreads, 2) void full_decode_partial_kernel(AttnArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    __shared__ __attribute__((aligned(1024))) uint16_t vt[4 * VSTEP];
    __shared__ float red_m[4][16], red_l[4][16];
    __shared__ float qcs[QROPE ? 4 : 1][64];  // per wave: cos, sin of the 32 angles

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int quad = lane >> 4, col = lane & 15;
    // (sequence, chunk, KV head) with the head fastest: consecutive
    // workgroups go to the XCDs in turn, so every XCD gets an even share of
    // each sequence's chunks whatever the context lengths (grouping a
    // sequence's chunks on one XCD left the busiest XCD 13% over the mean
    // for contexts spread over 32768 .. 131072)
    const int bid = blockIdx.x;
    const int g = bid % a.hkv;
    const int c = (bid / a.hkv) % a.n_chunks;
    const int s = bid / (a.n_chunks * a.hkv);

    const int64_t L = a.ctx_len[s];
    const int64_t c0 = (int64_t)c * a.chunk;
    if (c0 >= L) return;
    const int64_t base = a.seq_base[s];
    const int per_wave = a.chunk / 4;
    const int64_t w0 = c0 + (int64_t)w * per_wave;
    int64_t w1 = w0 + per_wave;
    if (w1 > L) w1 = L;
    if (base + w1 > a.pool_rows) w1 = a.pool_rows - base;  // never read past the pool
    if (base < 0) w1 = w0;                                   // nor before it
    const int nsteps = w1 > w0 ? (int)((w1 - w0 + KS - 1) / KS) : 0;

    const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)s * a.hq + g * G) * DQK;
    const uint16_t *Kp = (const uint16_t *)a.k_main;
    const uint16_t *Vp = (const uint16_t *)a.v_main;
    u32x4 qb[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
        qb[st] = col < G ? ld16(Q + col * DQK + 32 * st + 8 * quad) : u32x4{0, 0, 0, 0};
    // QROPE: steps 0 and 1 (dims 8 quad .. and their partners 32 + 8 quad ..)
    // become the rotated values split into bf16 hi (qb) + lo (ql).
    u32x4 ql[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    if constexpr (QROPE) {
        float cv, sv;
        rope_cos_sin(L - 1, a.inv_freq[lane & 31], cv, sv);
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
        if (col < G) {
            qb[0] = u32x4{lh0[0], lh0[1], lh1[0], lh1[1]};
            ql[0] = u32x4{ll0[0], ll0[1], ll1[0], ll1[1]};
            qb[1] = u32x4{hh0[0], hh0[1], hh1[0], hh1[1]};
            ql[1] = u32x4{hl0[0], hl0[1], hl1[0], hl1[1]};
        }
    }

    const int u = lane & 31;
    const int vkey = 4 * (u >> 3) + ((u >> 1) & 3), vbyte = 32 * (lane >> 5) + 16 * (u & 1);
    auto load_step = [&](int i, StepRegs &r) {
        const int64_t k0 = w0 + (int64_t)i * KS;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            int64_t key = k0 + 16 * kt + col;
            bool ok = key < w1;
            const uint16_t *src = Kp + ((base + key) * a.hkv + g) * (int64_t)DQK + 8 * quad;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) r.k[kt][st] = ok ? ld16(src + 32 * st) : u32x4{0, 0, 0, 0};
        }
        // V in the fragment order of the transposing reads: piece i of lane
        // (u = lane & 31) is key 16 (i / 4) + 4 (u >> 3) + ((u >> 1) & 3) of
        // the step, bytes 64 (i % 4) + 32 (lane >> 5) + 16 (u & 1) of its
        // row, and goes to bytes 1024 i + 16 lane of the wave's tile.
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int64_t key = k0 + 16 * (it / 4) + vkey;
            r.v[it] = key < w1 ? ld16((const char *)(Vp + ((base + key) * a.hkv + g) * (int64_t)DV) + 64 * (it % 4) +
                                      vbyte)
                               : u32x4{0, 0, 0, 0};
        }
    };

    uint16_t *vtw = vt + w * VSTEP;
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0, 0, 0, 0};
    float m = -INFINITY, l = 0.0f;
    const float scale2 = a.scale * kLog2e;

    StepRegs cur;
    for (int i = 0; i < nsteps; ++i) {
        load_step(i, cur);
        const int64_t k0 = w0 + (int64_t)i * KS;
        f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) sacc[kt] = mfma_16x16x32_bf16(cur.k[kt][st], qb[st], sacc[kt]);
        if constexpr (QROPE) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) sacc[kt] = mfma_16x16x32_bf16(cur.k[kt][st], ql[st], sacc[kt]);
        }
        // V of this step into the wave's LDS tile (DS ops of one wave run in
        // order, so the reads below see these writes and the writes of the
        // next step come after these reads).
#pragma unroll
        for (int it = 0; it < 8; ++it) *reinterpret_cast<u32x4 *>(vtw + it * 512 + 8 * lane) = cur.v[it];
        __builtin_amdgcn_wave_barrier();
        float sv[8], mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int64_t key = k0 + 16 * kt + 4 * quad + j;
                float v = key < w1 ? sacc[kt][j] * scale2 : -INFINITY;
                sv[4 * kt + j] = v;
                mx = fmaxf(mx, v);
            }
        mx = quad_max(mx);
        float mn = fmaxf(m, mx);
        float mu = mn == -INFINITY ? 0.0f : mn;
        float corr = exp2f(m - mu);
        float pv[8], ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = exp2f(sv[e] - mu);
            ps += pv[e];
        }
        ps = quad_sum(ps);
        l = l * corr + ps;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= corr;
        // O^T += V^T P^T over the step's 32 keys: operand slots 0-3 of a
        // quad are keys 4quad.. of the first 16-key half, slots 4-7 of the
        // second.
        u32x2 h0, l0, h1, l1;
        split_hi_lo(pv, h0, l0);
        split_hi_lo(pv + 4, h1, l1);
        const u32x4 bhi = u32x4{h0[0], h0[1], h1[0], h1[1]};
        const u32x4 blo = u32x4{l0[0], l0[1], l1[0], l1[1]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x2 a0 = ds_read_tr16(vtw + (dt * 64 + lane) * 4);
            const u32x2 a1 = ds_read_tr16(vtw + ((DT + dt) * 64 + lane) * 4);
            const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
            oacc[dt] = mfma_16x16x32_bf16(av, bhi, oacc[dt]);
            oacc[dt] = mfma_16x16x32_bf16(av, blo, oacc[dt]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // Merge the four waves of this chunk.
    if (quad == 0) {
        red_m[w][col] = m;
        red_l[w][col] = l;
    }
    __syncthreads();  // all waves done with their V tiles: reuse vt for partials
    // [4][16][DV]; 16-byte unit u of head row h at unit u ^ h (the 16 lanes
    // of a quad write 16 different bank groups)
    float *opart = reinterpret_cast<float *>(vt);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4 *>(opart + (w * 16 + col) * DV + 4 * ((4 * dt + quad) ^ col)) = oacc[dt];
    __syncthreads();
    float *ws_ml = (float *)a.ws;
    float *ws_acc = ws_ml + ((2 * (int64_t)a.n_seqs * a.hq * a.n_chunks + 3) & ~(int64_t)3);
    for (int idx = threadIdx.x; idx < G * DV / 4; idx += kThreads) {
        int h = idx / (DV / 4), d4 = 4 * (idx % (DV / 4));
        float mc = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
        float mu = mc == -INFINITY ? 0.0f : mc;
        f32x4 o = f32x4{0, 0, 0, 0};
        float lc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            float f = exp2f(red_m[ww][h] - mu);
            o += f * *reinterpret_cast<const f32x4 *>(opart + (ww * 16 + h) * DV + 4 * ((d4 / 4) ^ h));
            lc += f * red_l[ww][h];
        }
        int64_t slot = ((int64_t)s * a.hq + g * G + h) * a.n_chunks + c;
        *reinterpret_cast<f32x4 *>(ws_acc + slot * DV + d4) = o;
        if (d4 == 0) {
            ws_ml[2 * slot] = mc;
            ws_ml[2 * slot + 1] = lc;
        }
    }
}

// One wave per (sequence, q head); lane owns value dims 2*lane, 2*lane+1.
__global__ __launch_bounds__(kThreads) void full_decode_combine_kernel(AttnArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)a.n_seqs * a.hq) return;
    const int s = (int)(wid / a.hq), h = (int)(wid % a.hq);
    const int64_t L = a.ctx_len[s];
    int64_t nc64 = (L + a.chunk - 1) / a.chunk;
    const int nc = (int)(nc64 < a.n_chunks ? nc64 : a.n_chunks);  // ctx_len beyond max_ctx is clipped
    const float *ws_ml = (const float *)a.ws;
    const float *ws_acc = ws_ml + ((2 * (int64_t)a.n_seqs * a.hq * a.n_chunks + 3) & ~(int64_t)3);
    const int64_t slot0 = wid * a.n_chunks;
    // (m, l) of chunk c in lane c mod 64 of pass c / 64: the maximum and the
    // factors come from one coalesced load per 64 chunks, then each chunk's
    // accumulator loads are independent of one another (eight in flight).
    float M = -INFINITY;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        if (c < nc) M = fmaxf(M, ws_ml[2 * (slot0 + c)]);
    }
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
    M = fmaxf(M, sink2);
    const float mu = M == -INFINITY ? 0.0f : M;
    float z = a.sinks ? exp2f(sink2 - mu) : 0.0f;
    float o0 = 0.0f, o1 = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        float f = 0.0f, lz = 0.0f;
        if (c < nc) {
            f = exp2f(ws_ml[2 * (slot0 + c)] - mu);
            lz = f * ws_ml[2 * (slot0 + c) + 1];
        }
        for (int off = 32; off > 0; off >>= 1) lz += __shfl_xor(lz, off, 64);
        z += lz;
        const int n = min(64, nc - c0);
        int j = 0;
        for (; j + 8 <= n; j += 8) {
            float2 v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = *reinterpret_cast<const float2 *>(ws_acc + (slot0 + c0 + j + e) * DV + 2 * lane);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float fe = __shfl(f, j + e, 64);
                o0 += fe * v[e].x;
                o1 += fe * v[e].y;
            }
        }
        for (; j < n; ++j) {
            const float2 v = *reinterpret_cast<const float2 *>(ws_acc + (slot0 + c0 + j) * DV + 2 * lane);
            const float fe = __shfl(f, j, 64);
            o0 += fe * v.x;
            o1 += fe * v.y;
        }
    }
    float r = z > 0.0f ? a.value_scale / z : 0.0f;
    uint16_t *out = (uint16_t *)a.out + wid * DV + 2 * lane;
    *reinterpret_cast<uint32_t *>(out) = pack_bf16x2(o0 * r, o1 * r);
}

}  // namespace

bool full_decode_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.chunk % 128 == 0 &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_full_decode(const AttnArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.n_seqs * a.hkv * a.n_chunks)), block(kThreads);
    if (a.qrope) {
        switch (a.hq / a.hkv) {
            case 1: hipLaunchKernelGGL((full_decode_partial_kernel<1, true>), grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL((full_decode_partial_kernel<2, true>), grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL((full_decode_partial_kernel<4, true>), grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL((full_decode_partial_kernel<8, true>), grid, block, 0, s, a); break;
            default: hipLaunchKernelGGL((full_decode_partial_kernel<16, true>), grid, block, 0, s, a); break;
        }
    } else {
        switch (a.hq / a.hkv) {
            case 1: hipLaunchKernelGGL((full_decode_partial_kernel<1, false>), grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL((full_decode_partial_kernel<2, false>), grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL((full_decode_partial_kernel<4, false>), grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL((full_decode_partial_kernel<8, false>), grid, block, 0, s, a); break;
            default: hipLaunchKernelGGL((full_decode_partial_kernel<16, false>), grid, block, 0, s, a); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t waves = (int64_t)a.n_seqs * a.hq;
    dim3 grid2((unsigned)((waves + 3) / 4));
    hipLaunchKernelGGL(full_decode_combine_kernel, grid2, block, 0, s, a);
    return hipGetLastError();
}

// Workspace: (m, l) pairs then acc[DV] per (sequence, head, chunk), fp32.
size_t full_decode_ws_bytes(int64_t n_seqs, int64_t hq, int64_t n_chunks, int64_t dv) {
    int64_t ml = (2 * n_seqs * hq * n_chunks + 3) & ~(int64_t)3;
    return (size_t)(ml + n_seqs * hq * n_chunks * dv) * sizeof(float);
}

}  // namespace hsw
