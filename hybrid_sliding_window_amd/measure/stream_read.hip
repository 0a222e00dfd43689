// stream_read.hip -- measurement only, not part of the attention path: a plain
// read of item-shaped blocks from three arrays (per item, one block of each),
// loads only, with nothing computed on the data.  bench.py times it on the
// windowed decode's own bytes in the decode's layout (per (sequence, KV head):
// the 48 KiB K ring, the 32 KiB V ring and the 3 KiB of its query heads), so
// the decode kernel's time can be set beside what a bare stream of the same
// bytes takes on the same GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

// One workgroup per item; every 16-byte unit of the item's three blocks is
// loaded once (consecutive threads, consecutive units) and folded into an
// XOR that is stored only if it equals a value no input here produces, so
// the loads cannot be removed.  KU, VU, QU: the blocks' sizes in 16-byte
// units when known at compile time (every load of the item is then issued
// before the first is used), else 0 and the runtime sizes are looped over.
template <int KU, int VU, int QU>
__global__ __launch_bounds__(kThreads) void read_items_kernel(const u32x4 *k, const u32x4 *v, const u32x4 *q,
                                                             int64_t ku, int64_t vu, int64_t qu,
                                                             unsigned int *sink) {
    const int64_t it = blockIdx.x;
    const int t = threadIdx.x;
    uint32_t acc = 0;
    if constexpr (KU > 0) {
        static_assert(KU % kThreads == 0 && VU % kThreads == 0, "whole rounds of K and V units");
        constexpr int NK = KU / kThreads, NV = VU / kThreads, NQ = (QU + kThreads - 1) / kThreads;
        const u32x4 *kb = k + it * KU, *vb = v + it * VU, *qb = q + it * QU;
        u32x4 r[NK + NV + NQ];
#pragma unroll
        for (int i = 0; i < NK; ++i) r[i] = kb[i * kThreads + t];
#pragma unroll
        for (int i = 0; i < NV; ++i) r[NK + i] = vb[i * kThreads + t];
#pragma unroll
        for (int i = 0; i < NQ; ++i)
            r[NK + NV + i] = i * kThreads + t < QU ? qb[i * kThreads + t] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NK + NV + NQ; ++i) acc ^= r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3];
    } else {
        const u32x4 *kb = k + it * ku, *vb = v + it * vu, *qb = q + it * qu;
        for (int64_t i = t; i < ku; i += kThreads) {
            const u32x4 x = kb[i];
            acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
        }
        for (int64_t i = t; i < vu; i += kThreads) {
            const u32x4 x = vb[i];
            acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
        }
        for (int64_t i = t; i < qu; i += kThreads) {
            const u32x4 x = qb[i];
            acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
        }
    }
    if (acc == 0x9e3779b9u) sink[it & 1023] = acc;
}

}  // namespace

// Launch one read of n_items items on `stream`.  k, v, q: device arrays of
// n_items blocks of k_bytes, v_bytes, q_bytes each (multiples of 16, 16-byte
// aligned); sink: device memory of 1024 unsigned ints (written only in the
// case described above).  Returns 0, 1 for bad arguments (nothing launched),
// or 2 + the HIP error code of a failed launch.
extern "C" int hsw_measure_read_items(const void *k, const void *v, const void *q, int32_t n_items,
                                      int64_t k_bytes, int64_t v_bytes, int64_t q_bytes, unsigned int *sink,
                                      void *stream) {
    if (!k || !v || !q || !sink || n_items <= 0 || k_bytes <= 0 || v_bytes < 0 || q_bytes < 0 ||
        k_bytes % 16 || v_bytes % 16 || q_bytes % 16 || ((uintptr_t)k | (uintptr_t)v | (uintptr_t)q) % 16)
        return 1;
    const dim3 grid((unsigned)n_items), block(kThreads);
    const u32x4 *kp = (const u32x4 *)k, *vp = (const u32x4 *)v, *qp = (const u32x4 *)q;
    const int64_t ku = k_bytes / 16, vu = v_bytes / 16, qu = q_bytes / 16;
    // the windowed decode's items: 128 ring slots of K (192 bf16) and V (128
    // bf16), and the query heads of one KV head (8 or 16 x 192 bf16)
    if (ku == 3072 && vu == 2048 && qu == 192)
        hipLaunchKernelGGL((read_items_kernel<3072, 2048, 192>), grid, block, 0, (hipStream_t)stream, kp, vp, qp,
                           ku, vu, qu, sink);
    else if (ku == 3072 && vu == 2048 && qu == 384)
        hipLaunchKernelGGL((read_items_kernel<3072, 2048, 384>), grid, block, 0, (hipStream_t)stream, kp, vp, qp,
                           ku, vu, qu, sink);
    else
        hipLaunchKernelGGL((read_items_kernel<0, 0, 0>), grid, block, 0, (hipStream_t)stream, kp, vp, qp, ku, vu,
                           qu, sink);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : 2 + (int)e;
}
