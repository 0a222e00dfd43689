// generic_attn.hip -- wave-per-(row, head) attention for any dtype and shape,
// plus the ring commit that follows a windowed prefill.
//
// This is the path for fp32 storage and for shapes the MFMA kernels do not
// take (other head widths, windows or group sizes).  One wave owns one
// (query row, q head): the wave reduces each q.k across its 64 lanes and
// keeps an online softmax, each lane accumulating a slice of the value dims.
// The key sets are those of the method:
//  - windowed prefill: positions max(0, p-W+1) .. p, keys before the chunk
//    start from ring slot (pos mod W), the rest from staging (colibri
//    "System One mode and prompt reuse"; gaudi-cookbook "What was built");
//  - windowed decode: every ring slot t, holding position
//    P - ((P - t) mod W), used when that position is >= 0;
//  - full prefill / decode: pool rows seq_base + 0 .. seq_base + p.
// The sink joins the denominator only (colibri "What the engine implements").
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kMaxDim = 256;
constexpr int kSlices = kMaxDim / kWave;

template <typename T, typename TO>
__global__ __launch_bounds__(kThreads) void generic_attn_kernel(AttnArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    const int lane = threadIdx.x % kWave;
    const int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (wid >= a.n_rows * a.hq) return;
    int64_t row = wid / a.hq;  // prefill kinds: s * max_seqlen + local token
    const int h = (int)(wid % a.hq);
    const int g = h / (a.hq / a.hkv);

    // Resolve the query position and the key range [j0, j1] (positions).
    int s = 0;
    int64_t p = 0, j0 = 0, j1 = -1, start = 0, tok0 = 0;
    if (a.kind == kSwaPrefill || a.kind == kFullPrefill) {
        s = (int)(row / a.max_seqlen);
        const int64_t local = row % a.max_seqlen;
        tok0 = a.cu_seqlens[s];
        if (local >= a.cu_seqlens[s + 1] - tok0) return;
        row = tok0 + local;  // chunk token index
        start = a.start_pos[s];
        p = start + local;
        j1 = p;
        j0 = (a.kind == kSwaPrefill) ? p - a.window + 1 : 0;
        if (j0 < 0) j0 = 0;
    } else if (a.kind == kSwaDecode) {
        s = (int)row;
        p = a.pos[s];
        j0 = 0;
        j1 = a.window - 1;  // iterate slots
    } else {
        s = (int)row;
        p = a.ctx_len[s] - 1;
        j0 = 0;
        j1 = p;
    }

    const T *qrow = (const T *)a.q + (row * a.hq + h) * (int64_t)a.dqk;
    float qv[kSlices];
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
        int d = lane + kWave * i;
        qv[i] = d < a.dqk ? Elem<T>::load(qrow + d) : 0.0f;
    }
    float acc[kSlices] = {0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    for (int64_t j = j0; j <= j1; ++j) {
        const T *kr;
        const T *vr;
        if (a.kind == kSwaPrefill) {
            if (j < start) {
                int64_t slot = j % a.window;
                int64_t base = ((int64_t)s * a.hkv + g) * a.window + slot;
                kr = (const T *)a.k_ring + base * a.dqk;
                vr = (const T *)a.v_ring + base * a.dv;
            } else {
                int64_t r = tok0 + (j - start);
                kr = (const T *)a.k_main + (r * a.hkv + g) * (int64_t)a.dqk;
                vr = (const T *)a.v_main + (r * a.hkv + g) * (int64_t)a.dv;
            }
        } else if (a.kind == kSwaDecode) {
            int64_t back = (p - j) % a.window;
            if (back < 0) back += a.window;
            if (p - back < 0) continue;
            int64_t base = ((int64_t)s * a.hkv + g) * a.window + j;
            kr = (const T *)a.k_main + base * a.dqk;
            vr = (const T *)a.v_main + base * a.dv;
        } else {
            int64_t r = a.seq_base[s] + j;
            if (r < 0 || r >= a.pool_rows) continue;
            kr = (const T *)a.k_main + (r * a.hkv + g) * (int64_t)a.dqk;
            vr = (const T *)a.v_main + (r * a.hkv + g) * (int64_t)a.dv;
        }
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < kSlices; ++i) {
            int d = lane + kWave * i;
            if (d < a.dqk) dot += qv[i] * Elem<T>::load(kr + d);
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, kWave);
        float sc = dot * a.scale;
        float mn = fmaxf(m, sc);
        float corr = expf(m - mn);   // 0 on the first key (m = -inf)
        float pj = expf(sc - mn);
        l = l * corr + pj;
#pragma unroll
        for (int i = 0; i < kSlices; ++i) {
            int d = lane + kWave * i;
            float vv = d < a.dv ? Elem<T>::load(vr + d) : 0.0f;
            acc[i] = acc[i] * corr + pj * vv;
        }
        m = mn;
    }
    if (a.sinks) {
        float sk = a.sinks[h];
        float mn = fmaxf(m, sk);
        float corr = expf(m - mn);
        l = l * corr + expf(sk - mn);
#pragma unroll
        for (int i = 0; i < kSlices; ++i) acc[i] *= corr;
    }
    float inv = l > 0.0f ? a.value_scale / l : 0.0f;
    TO *orow = (TO *)a.out + (row * a.hq + h) * (int64_t)a.dv;
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
        int d = lane + kWave * i;
        if (d < a.dv) Elem<TO>::store(orow + d, acc[i] * inv);
    }
}

// Copy the last min(len, W) chunk rows of each sequence into ring slot
// (pos mod W).  One block per (sequence, ring row).
template <typename T>
__global__ __launch_bounds__(kThreads) void ring_commit_kernel(AttnArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    const int s = blockIdx.y;
    const int i = blockIdx.x;
    const int64_t tok0 = a.cu_seqlens[s];
    const int64_t len = a.cu_seqlens[s + 1] - tok0;
    const int64_t n = len < a.window ? len : a.window;
    if (i >= n) return;
    const int64_t t = len - n + i;
    const int64_t p = a.start_pos[s] + t;
    if (p < 0) return;
    const int64_t slot = p % a.window;
    const int kchunks = a.dqk * (int)sizeof(T) / 16, vchunks = a.dv * (int)sizeof(T) / 16;
    for (int c = threadIdx.x; c < a.hkv * (kchunks + vchunks); c += kThreads) {
        int h = c / (kchunks + vchunks);
        int e = c % (kchunks + vchunks);
        int64_t ring_row = ((int64_t)s * a.hkv + h) * a.window + slot;
        int64_t src_row = (tok0 + t) * a.hkv + h;
        if (e < kchunks) {
            const char *src = (const char *)a.k_main + src_row * a.dqk * sizeof(T) + 16 * e;
            char *dst = (char *)a.k_ring + ring_row * a.dqk * sizeof(T) + 16 * e;
            st16(dst, ld16(src));
        } else {
            e -= kchunks;
            const char *src = (const char *)a.v_main + src_row * a.dv * sizeof(T) + 16 * e;
            char *dst = (char *)a.v_ring + ring_row * a.dv * sizeof(T) + 16 * e;
            st16(dst, ld16(src));
        }
    }
}

}  // namespace

hipError_t launch_generic_attn(const AttnArgs &a, int dtype, int out_dtype, hipStream_t s) {
    int64_t waves = a.n_rows * a.hq;
    dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)), block(kThreads);
    if (dtype == 0 && out_dtype == 0)
        hipLaunchKernelGGL((generic_attn_kernel<uint16_t, uint16_t>), grid, block, 0, s, a);
    else if (dtype == 0)
        hipLaunchKernelGGL((generic_attn_kernel<uint16_t, float>), grid, block, 0, s, a);
    else if (out_dtype == 0)
        hipLaunchKernelGGL((generic_attn_kernel<float, uint16_t>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((generic_attn_kernel<float, float>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ring_commit(const AttnArgs &a, int dtype, hipStream_t s) {
    dim3 grid((unsigned)a.window, (unsigned)a.n_seqs), block(kThreads);
    if (dtype == 0)
        hipLaunchKernelGGL(ring_commit_kernel<uint16_t>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(ring_commit_kernel<float>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace hsw
