// rope_kv.hip -- partial rotate-half RoPE on q and k plus the K/V write.
//
// colibri "MiMo-V2.6 (Xiaomi)", "What the engine implements": rotate-half on
// the first rope_dim (64) of each 192-wide q/k head, theta 1e4 on windowed
// layers and 1e7 on full layers; values pass through (the value scale is
// applied to the attention output instead, equal by linearity).
// gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", "The RoPE fix for large
// positions": an fp32 angle is wrong at large positions, so every angle
// pos * theta^(-2i/R) is formed and reduced modulo pi/2 in double precision
// (rope_cos_sin); sin/cos of the reduced angle and the rotation are fp32.
// colibri "System One mode and prompt reuse": K/V of position p go to ring
// slot p mod window (windowed layers) or to row seq_base + p (full layers).
//
// HBM-bound (~2 flop per 4 bytes).  One workgroup per token: the token's
// rope_dim/2 angles are computed once into LDS and shared by all of its
// q and k heads.  Each thread then walks "items" of 8 contiguous elements:
// a rotation item covers dims [8j, 8j+8) and their partners [8j+R/2, ...),
// a pass-through item copies 8 dims unchanged (bit-exact).
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHalf = 128;

template <typename T> struct Chunk8;
template <> struct Chunk8<uint16_t> {  // 8 bf16 = 16 bytes
    u32x4 r;
    __device__ void load(const uint16_t *p) { r = ld16(p); }
    __device__ void store(uint16_t *p) const { st16(p, r); }
    __device__ float get(int i) const {
        uint32_t w = r[i >> 1];
        return bf2f((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
    }
    __device__ void set_all(const float f[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    }
};
template <> struct Chunk8<float> {  // 8 fp32 = 32 bytes
    u32x4 r0, r1;
    __device__ void load(const float *p) { r0 = ld16(p); r1 = ld16(p + 4); }
    __device__ void store(float *p) const { st16(p, r0); st16(p + 4, r1); }
    __device__ float get(int i) const { return __uint_as_float(i < 4 ? r0[i] : r1[i - 4]); }
    __device__ void set_all(const float f[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r0[i] = __float_as_uint(f[i]);
            r1[i] = __float_as_uint(f[i + 4]);
        }
    }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kv_kernel(RopeArgs a) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    __shared__ float cs[kMaxHalf], sn[kMaxHalf];
    __shared__ int64_t dst_row;  // element row of head 0: ring (seq*Hkv)*window + slot; pool/staging row*Hkv
    const int64_t t = blockIdx.x;
    const int half = a.rope_dim / 2;
    const int64_t p = a.pos[t];

    if (threadIdx.x < half) {
        // angle = p * theta^(-2i/R) formed and reduced in double
        float c, s;
        rope_cos_sin(p, a.inv_freq[threadIdx.x], c, s);
        cs[threadIdx.x] = c;
        sn[threadIdx.x] = s;
    }
    if (threadIdx.x == 0) {
        int64_t idx = -1, row = -1;
        if (a.dst_kind == 2) {  // staging
            if (t < a.dst_capacity) { idx = t; row = t * a.hkv; }
        } else {
            int64_t s = a.seq[t];
            if (a.dst_kind == 0) {  // ring
                if (s >= 0 && s < a.dst_capacity && p >= 0) {
                    int64_t slot = p % a.window;
                    idx = slot;
                    row = s * (int64_t)a.hkv * a.window + slot;
                }
            } else {  // pool
                if (s >= 0 && p >= 0) {
                    int64_t r = a.seq_base[s] + p;
                    if (r >= 0 && r < a.dst_capacity) { idx = r; row = r * a.hkv; }
                }
            }
        }
        dst_row = row;
        if (a.dst_index_out) a.dst_index_out[t] = idx;
    }
    __syncthreads();

    const int units = half / 8;                      // rotation items per head
    const int pass = (a.dqk - a.rope_dim) / 8;       // pass-through items per q/k head
    const int per_qk = units + pass;
    const int per_v = a.dv / 8;
    // q == NULL: K/V only (the attention call rotates q itself); v == NULL
    // (staging only): K only (the windowed prefill reads V where it is)
    const int n_q = a.q ? a.hq * per_qk : 0, n_k = a.hkv * per_qk, n_v = a.v ? a.hkv * per_v : 0;
    const int64_t row = dst_row;
    // K/V row stride between heads: ring rows interleave (head, slot).
    const int64_t head_stride = (a.dst_kind == 0) ? (int64_t)a.window : 1;

    for (int it = threadIdx.x; it < n_q + n_k + n_v; it += kThreads) {
        const T *src;
        T *dst;
        int item;
        if (it < n_q + n_k) {
            int h, is_k = it >= n_q;
            int j = is_k ? it - n_q : it;
            h = j / per_qk;
            item = j % per_qk;
            if (!is_k) {
                src = (const T *)a.q + (t * a.hq + h) * (int64_t)a.dqk;
                dst = (T *)a.q_rot + (t * a.hq + h) * (int64_t)a.dqk;
            } else {
                if (row < 0) continue;
                src = (const T *)a.k + (t * a.hkv + h) * (int64_t)a.dqk;
                dst = (T *)a.k_dst + (row + h * head_stride) * (int64_t)a.dqk;
            }
            if (item < units) {
                Chunk8<T> lo, hi;
                lo.load(src + 8 * item);
                hi.load(src + 8 * item + half);
                float ylo[8], yhi[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    rope_rotate(lo.get(e), hi.get(e), cs[8 * item + e], sn[8 * item + e], ylo[e], yhi[e]);
                lo.set_all(ylo);
                hi.set_all(yhi);
                lo.store(dst + 8 * item);
                hi.store(dst + 8 * item + half);
            } else {
                int off = a.rope_dim + 8 * (item - units);
                Chunk8<T> x;
                x.load(src + off);
                x.store(dst + off);
            }
        } else {
            if (row < 0) continue;
            int j = it - n_q - n_k;
            int h = j / per_v;
            item = j % per_v;
            src = (const T *)a.v + (t * a.hkv + h) * (int64_t)a.dv;
            dst = (T *)a.v_dst + (row + h * head_stride) * (int64_t)a.dv;
            Chunk8<T> x;
            x.load(src + 8 * item);
            x.store(dst + 8 * item);
        }
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, int dtype, hipStream_t s) {
    dim3 grid((unsigned)a.n_tokens), block(kThreads);
    if (dtype == 0)
        hipLaunchKernelGGL(rope_kv_kernel<uint16_t>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(rope_kv_kernel<float>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace hsw
