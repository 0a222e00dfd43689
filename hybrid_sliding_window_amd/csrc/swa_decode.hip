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
// HBM-bound: each (sequence, KV head) reads its 48 KiB K ring and 32 KiB V
// ring exactly once.  One workgroup (4 waves) per (sequence, KV head); wave w
// owns ring slots [32w, 32w+32).  The G query heads of the group share every
// K/V load: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K rows straight from
// HBM into the A operand, the G heads as the 16 B columns, zero-padded), an
// fp32 softmax reduced across quads and waves, then O^T = V^T P^T with
// v_mfma_f32_16x16x16_bf16 on P split into bf16 hi + lo (so P keeps ~16 bits;
// a single bf16 P costs too much accuracy), V transposed through LDS.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128, W = 128;
constexpr int STEPS = DQK / 32;       // 16x16x32 MFMA steps over q/k dims
constexpr int DT = DV / 16;           // 16-wide value tiles
constexpr int VT_STRIDE = 36;         // bf16 per transposed V row (32 keys + pad)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <int G>
__global__ __launch_bounds__(kThreads) void swa_decode_kernel(AttnArgs a) {
    // LDS: per-wave transposed V tile [DV][32 keys], later reused for the
    // per-wave output partials [16 heads][DV] fp32.
    __shared__ __attribute__((aligned(16))) uint16_t vt[4 * DV * VT_STRIDE];
    __shared__ float red_m[4][16], red_l[4][16], m_fin[16];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int quad = lane >> 4, col = lane & 15;
    const int s = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
    const int64_t P = a.pos[s];

    const uint16_t *K = (const uint16_t *)a.k_main + ((int64_t)(s * a.hkv + g) * W) * DQK;
    const uint16_t *V = (const uint16_t *)a.v_main + ((int64_t)(s * a.hkv + g) * W) * DV;
    const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)s * a.hq + g * G) * DQK;

    // Issue every global load of this wave up front.
    u32x4 qb[STEPS], ka[2][STEPS], vr[8];
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
        qb[st] = col < G ? ld16(Q + col * DQK + 32 * st + 8 * quad) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            ka[kt][st] = ld16(K + (32 * w + 16 * kt + col) * DQK + 32 * st + 8 * quad);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        int c = it * 64 + lane;  // 16-byte chunk of this wave's 32 x DV tile
        vr[it] = ld16(V + (32 * w + (c >> 4)) * DV + 8 * (c & 15));
    }

    // S^T[key][head] for the wave's two 16-key tiles.
    f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt] = mfma_16x16x32_bf16(ka[kt][st], qb[st], sacc[kt]);

    // V transposed into LDS: vt[w][dv][key].
    uint16_t *vtw = vt + w * DV * VT_STRIDE;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        int c = it * 64 + lane, key = c >> 4, dv0 = 8 * (c & 15);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t word = vr[it][e >> 1];
            vtw[(dv0 + e) * VT_STRIDE + key] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
        }
    }

    // Scaled logits in log2 units, masked where the slot holds a position < 0.
    const float scale2 = a.scale * kLog2e;
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int slot = 32 * w + 16 * kt + 4 * quad + i;
            int64_t back = (P - slot) & (W - 1);
            float v = back <= P ? sacc[kt][i] * scale2 : -INFINITY;
            sv[4 * kt + i] = v;
            mx = fmaxf(mx, v);
        }
    mx = quad_max(mx);
    if (quad == 0) red_m[w][col] = mx;
    __syncthreads();
    float m = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
    const bool has_sink = a.sinks != nullptr && col < G;
    const float sink2 = has_sink ? a.sinks[g * G + col] * kLog2e : -INFINITY;
    m = fmaxf(m, sink2);  // finite: the current position is always in the ring
    float pv[8], lsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pv[e] = exp2f(sv[e] - m);
        lsum += pv[e];
    }
    lsum = quad_sum(lsum);
    if (quad == 0) red_l[w][col] = lsum;
    if (w == 0 && quad == 0) m_fin[col] = m;

    // O^T[dv][head] = V^T P^T over this wave's 32 keys.
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        u32x2 hi, lo;
        split_hi_lo(pv + 4 * kt, hi, lo);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2 av = *reinterpret_cast<const u32x2 *>(vtw + (16 * dt + col) * VT_STRIDE + 16 * kt + 4 * quad);
            oacc[dt] = mfma_16x16x16_bf16(av, hi, oacc[dt]);
            oacc[dt] = mfma_16x16x16_bf16(av, lo, oacc[dt]);
        }
    }
    __syncthreads();  // every wave is done with vt: reuse it for the partials
    float *opart = reinterpret_cast<float *>(vt);  // [4][16][DV]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4 *>(opart + (w * 16 + col) * DV + 16 * dt + 4 * quad) = oacc[dt];
    __syncthreads();

    // Combine the four waves, add the sink to the denominator, scale, store.
    uint16_t *out = (uint16_t *)a.out + ((int64_t)s * a.hq + g * G) * DV;
    for (int idx = threadIdx.x; idx < G * DV / 4; idx += kThreads) {
        int h = idx / (DV / 4), d4 = 4 * (idx % (DV / 4));
        f32x4 o = *reinterpret_cast<const f32x4 *>(opart + h * DV + d4);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) o += *reinterpret_cast<const f32x4 *>(opart + (ww * 16 + h) * DV + d4);
        float l = red_l[0][h] + red_l[1][h] + red_l[2][h] + red_l[3][h];
        if (a.sinks) l += exp2f(a.sinks[g * G + h] * kLog2e - m_fin[h]);
        float r = a.value_scale / l;
        u32x2 pk = u32x2{(uint32_t)f2bf(o[0] * r) | ((uint32_t)f2bf(o[1] * r) << 16),
                         (uint32_t)f2bf(o[2] * r) | ((uint32_t)f2bf(o[3] * r) << 16)};
        *reinterpret_cast<u32x2 *>(out + h * DV + d4) = pk;
    }
}

}  // namespace

bool swa_decode_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == W &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_swa_decode(const AttnArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.n_seqs * a.hkv)), block(kThreads);
    switch (a.hq / a.hkv) {
        case 1: hipLaunchKernelGGL(swa_decode_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(swa_decode_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(swa_decode_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(swa_decode_kernel<8>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(swa_decode_kernel<16>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
