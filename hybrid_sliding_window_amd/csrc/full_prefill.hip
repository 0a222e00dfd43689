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
// Sixteen query heads per KV head (both models' full layers) take the
// 8-wave kernel at the end of this file, whose two wave halves alternate
// between MFMA and VALU work; the smaller groups take the kernel described
// here.  One workgroup (4 waves) per query block: 128 rows = 128/G positions x the G
// query heads of one KV head (the heads are the 16-wide MFMA columns), two
// column tiles per wave.  The block's keys (pool rows base + 0 .. base +
// its last position) stream through LDS in 32-key chunks with a three-stage
// pipeline: chunk c+2 is fetched by direct global->LDS 16-byte loads (no VGPR
// staging) while chunk c is computed, one barrier per chunk; each wave skips
// chunks past its rows' positions.  Per chunk:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16 (K rows from LDS, q in VGPRs)
//   softmax          online in log2 units; the reference max is raised only
//                    when a chunk's max exceeds it by more than 2^8 (P <= 256),
//                    so the O rescale is rare
//   O^T += V^T P^T   v_mfma_f32_16x16x32_f16: P rounded to fp16 (11
//                    significant bits; P <= 256 keeps it in range) times V
//                    converted to fp16 in LDS, exact for every bf16 value of
//                    magnitude below 65536.  A 32-column block of a chunk
//                    holding a larger or non-finite value stays bf16 and takes
//                    the fp16-rounded P split exactly into bf16 hi + lo
//                    (v_mfma_f32_16x16x32_bf16 twice).  The V^T operand is
//                    read from row-major V by ds_read_b64_tr_b16.
// LDS holds K and V in MFMA fragment order (the load side places each
// 16-byte piece where a lane will read it), so every LDS read is a contiguous
// run in lane order, free of bank conflicts.  Block ids are remapped so
// consecutive query blocks of one (sequence, KV head) run on one XCD and
// stream the same keys through its L2.
//
// With QROPE the kernel reads unrotated q and applies the rotate-half RoPE
// itself (colibri "What the engine implements"; the angle in double as the
// gaudi-cookbook "The RoPE fix for large positions" requires) with the RoPE
// kernel's helpers and rounding, so the output is bit-identical to RoPE
// followed by the plain kernel, without q_rot's write and re-read.
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128;
constexpr int STEPS = DQK / 32;
constexpr int DT = DV / 16;
constexpr int KC = 32;                      // keys per chunk
constexpr int K_PIECES = KC * DQK / 8;      // 16-byte pieces per K stage (768)
constexpr int V_PIECES = KC * DV / 8;       // per V stage (512)
constexpr int kThreads = 256;
constexpr int K_LOADS = K_PIECES / kThreads;  // 3 per thread
constexpr int V_LOADS = V_PIECES / kThreads;  // 2 per thread
constexpr int LOADS = K_LOADS + V_LOADS;      // vector-memory ops per chunk per thread
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;

// s_waitcnt immediates (gfx9 encoding): wait until at most N vector-memory
// ops of this wave are outstanding; expcnt and lgkmcnt left unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0) alone

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds_wave_base + 16 i (lds_wave_base is wave-uniform, passed in m0; said
// so, for code where the compiler cannot tell).  Issued
// as inline asm so the compiler does not track it: it would otherwise add
// waits of its own before some LDS reads, for more of these loads than the
// read needs.  Completion is awaited explicitly (s_waitcnt vmcnt) before the
// barrier that publishes a stage; m0 is used by nothing else in this kernel.
__device__ __forceinline__ void load_lds16(const void *src, const void *lds_wave_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(src) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane
// offset: no per-lane address arithmetic.
__device__ __forceinline__ void load_lds16_s(const void *sbase, uint32_t voff, const void *lds_wave_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m), "v"(voff), "s"(sbase) : "memory", "m0");
}

// 16-byte global load into v, untracked like the loads above (v keeps its
// register; the first wait of the pipeline covers it, as it was issued first).
__device__ __forceinline__ void load_q16(u32x4 &v, const void *src) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "+v"(v) : "v"(src) : "memory");
}

// Max / sum over the four quads (lanes c, c+16, c+32, c+48) with the gfx950
// half-wave and row swaps (VALU, no LDS round trip).
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

// Transposing LDS read.  The pointer is cast straight to the LDS address
// space (not through an integer) so the read keeps the alias scope of its LDS
// array: the compiler then makes it wait only for loads into that array, not
// for the loads in flight to the other stages.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// A pointer every lane holds, said to be wave-uniform (SGPRs), as the
// scalar base of a load must be.
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int full = (total / 8) * 8;
    if (bid >= full) return bid;
    return (bid % 8) * (total / 8) + bid / 8;
}

template <int G, bool QROPE>
__global__ __launch_bounds__(kThreads, 2) void full_prefill_kernel(AttnArgs a, int nqb) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    constexpr int BQ = 128 / G;
    // Three stages, each its own LDS object so the compiler can tell that a
    // read of one stage does not depend on the loads in flight to another.
    __shared__ __attribute__((aligned(1024))) uint16_t ks0[KC * DQK], ks1[KC * DQK], ks2[KC * DQK];
    __shared__ __attribute__((aligned(1024))) uint16_t vs0[KC * DV], vs1[KC * DV], vs2[KC * DV];
    // per stage and wave: 1 if the wave's block of V columns stayed bf16
    // (a value beyond the fp16 range), 0 if it was converted to fp16
    __shared__ int vflag[3][4];
    // Raw bf16 copies of the V column blocks kept out of fp16 (rare), by
    // chunk parity: the stage itself then holds zeros there, so the fp16
    // product of every tile runs unconditionally and a kept block's tiles are
    // added from here afterwards.  convert_v of chunk c runs after every wave
    // passed the barrier of chunk c-1, so no wave still reads chunk c-2's copy.
    __shared__ __attribute__((aligned(1024))) uint16_t vbk[2][KC * DV];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();  // the intrinsics, so no library call is needed
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int quad = lane >> 4, col = lane & 15;
    const int total = a.n_seqs * a.hkv * nqb;
    const int bid = xcd_remap((int)__builtin_amdgcn_workgroup_id_x(), total);
    const int qb = bid % nqb;
    const int g = (bid / nqb) % a.hkv;
    const int s = bid / (nqb * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int len = (int)(a.cu_seqlens[s + 1] - tok0);
    if (qb * BQ >= len) return;
    // Positions index pool rows (base + position < pool_rows < 2^31, checked
    // on the host), so they fit in an int; an out-of-contract start is
    // clamped into [0, pool_rows] and its keys to the pool below.
    const int64_t start64 = a.start_pos[s];
    const int start = (int)(start64 < 0 ? 0 : start64 > a.pool_rows ? a.pool_rows : start64);
    const int p0 = start + qb * BQ;                         // first query position
    const int plast = start + min(len, qb * BQ + BQ) - 1;   // last query position
    const int64_t base = a.seq_base[s];
    // Keys are pool rows base + 0 .. base + plast, clamped to the pool.
    int nkeys = plast + 1;
    if (base + nkeys > a.pool_rows) nkeys = (int)(a.pool_rows - base);
    if (base < 0 || nkeys < 0) nkeys = 0;
    const int klast = max(nkeys - 1, 0);
    const int nch = max((nkeys + KC - 1) / KC, 1);

    // this lane's rotary frequency (fused q-RoPE), loaded before any
    // untracked load
    const double invf = QROPE ? pin_loaded(a.inv_freq[lane & 31]) : 0.0;
    // q of this wave's rows (row r = 32w + 16n + col -> position r / G, head
    // r % G), from a clamped row so the load is unconditional; rows past the
    // block only affect their own column and are never stored.
    u32x4 qv[2][STEPS];
    const uint16_t *qg = (const uint16_t *)a.q;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        int r = 32 * w + 16 * n + col;
        int local = min(qb * BQ + r / G, len - 1);
        const uint16_t *qrow = qg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DQK;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            // (tracked when the kernel rotates q: its first use, the
            // rotation, then waits for it before the loop; untracked ones
            // could be copied or reused by the register allocator before
            // the rotation's wait)
            if constexpr (QROPE) {
                qv[n][st] = ld16(qrow + 32 * st + 8 * quad);
            } else {
                qv[n][st] = u32x4{0, 0, 0, 0};
                load_q16(qv[n][st], qrow + 32 * st + 8 * quad);
            }
        }
    }

    // This sequence's K/V rows for KV head g.
    const int64_t b0 = base < 0 ? 0 : base;
    const char *kseq = (const char *)a.k_main + (b0 * a.hkv + g) * (int64_t)(DQK * 2);
    const char *vseq = (const char *)a.v_main + (b0 * a.hkv + g) * (int64_t)(DV * 2);
    const int64_t krow = (int64_t)a.hkv * DQK * 2, vrow = (int64_t)a.hkv * DV * 2;

    // LDS layout: fragment order.  K: 16-byte unit (h * 6 + st) * 64 + lane
    // holds what lane (quad, col) feeds the S^T MFMA of key half h, step st:
    // K[16h + col][pieces 4st + quad].  V: 8-byte unit (hh * 8 + dt) * 64 +
    // lane holds what lane (quad, 4k + mm) supplies to the transposing read of
    // key half hh, output tile dt: V[16hh + 4quad + k][16dt + 4mm .. +3].  The
    // i-th 16-byte load of wave w fills units (4i + w) * 64 + lane:
    //   K load i: j = 4i + w, h = j / 6, st = j % 6: key 16h + col, bytes
    //             64 st + 16 quad.
    //   V load i: j = 4i + w, hh = j / 4, tiles 2 (j % 4) + (lane >> 5); with
    //             u = lane & 31: row 16hh + 4 (u >> 3) + ((u >> 1) & 3), bytes
    //             64 (j % 4) + 32 (lane >> 5) + 16 (u & 1).
    const int u = lane & 31;
    const int vrow_l = 4 * (u >> 3) + ((u >> 1) & 3);
    const int vbyte_l = 32 * (lane >> 5) + 16 * (u & 1);
    // per-lane byte offsets of the unclamped loads (within 16 pool rows)
    const uint32_t koff_l = (uint32_t)(col * krow + 16 * quad);
    const uint32_t voff_l = (uint32_t)(vrow_l * vrow + vbyte_l);

    // Chunk c's loads.  Keys past the last one are clamped to it (finite
    // data, masked); past the band a dummy set (the first row, again) keeps
    // the number of loads per step constant.
    // Wave-uniform byte offsets of this wave's loads within a chunk (key
    // half and 64-byte column of each), computed once: an interior chunk's
    // load is then its chunk base plus one of these.
    int64_t kl_off[K_LOADS], vl_off[V_LOADS];
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
        const int j = 4 * i + w;
        kl_off[i] = (int64_t)(16 * (j / STEPS)) * krow + 64 * (j % STEPS);
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
        const int j = 4 * i + w;
        vl_off[i] = (int64_t)(16 * (j / 4)) * vrow + 64 * (j % 4);
    }
    // kco / vco: byte offset from kseq / vseq of chunk c's first row, carried
    // as running sums by the loop.
    auto issue = [&](int c, uint16_t *ksd, uint16_t *vsd, int64_t kco, int64_t vco) {
        const int k0 = c * KC;
        const char *ksrc[K_LOADS], *vsrc[V_LOADS];
        if (c < nch && k0 + KC - 1 <= klast) {
            // whole chunk inside the band: uniform base + per-lane offset
            const char *kb = kseq + kco, *vb = vseq + vco;
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i)
                load_lds16_s(vb + vl_off[i], voff_l, (const char *)vsd + (4 * i + w) * 1024);
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i)
                load_lds16_s(kb + kl_off[i], koff_l, (const char *)ksd + (4 * i + w) * 1024);
            return;
        }
        if (c >= nch) {
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i) ksrc[i] = kseq;
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) vsrc[i] = vseq;
        } else {
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i) {
                const int j = 4 * i + w, h = j / STEPS, st = j % STEPS;
                const int kp = min(k0 + 16 * h + col, klast);
                ksrc[i] = kseq + (int64_t)kp * krow + 64 * st + 16 * quad;
            }
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                const int j = 4 * i + w, hh = j / 4;
                const int kp = min(k0 + 16 * hh + vrow_l, klast);
                vsrc[i] = vseq + (int64_t)kp * vrow + 64 * (j % 4) + vbyte_l;
            }
        }
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i) load_lds16(vsrc[i], (const char *)vsd + (4 * i + w) * 1024);
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) load_lds16(ksrc[i], (const char *)ksd + (4 * i + w) * 1024);
    };

    // Each wave converts the V pieces it loaded for a chunk (columns 32w ..
    // 32w+31 of the chunk's 32 keys) from bf16 to fp16 in place, unless one
    // of them is beyond the fp16 range (|v| >= 65536, the first bf16 value
    // fp16 cannot hold): then they stay bf16 and the wave's flag says so.
    // The wave's own loads of those pieces must have landed; the barrier
    // after it publishes the result (the flags are read after it too).
    auto convert_v = [&](uint16_t *vst, int (&vf)[4], uint16_t *vb) {
        u32x4 raw[V_LOADS];
        float big = 0.0f;
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i) {
            raw[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(vst) + (4 * i + w) * 1024 + lane * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                big = fmaxf(big, fmaxf(fabsf(__uint_as_float(raw[i][e] << 16)),
                                       fabsf(__uint_as_float(raw[i][e] & 0xffff0000u))));
        }
        const bool keep = __any(big >= 65536.0f);
        if (!keep) {
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                u32x4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(raw[i][e]);
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(vst) + (4 * i + w) * 1024 + lane * 16) = h;
            }
        } else {
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                const int off = (4 * i + w) * 1024 + lane * 16;
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(vb) + off) = raw[i];
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(vst) + off) = u32x4{0, 0, 0, 0};
            }
        }
        if (lane == 0) vf[w] = keep ? 1 : 0;
    };

    const float scale2 = a.scale * kLog2e;
    f32x4 oacc[2][DT];
    float m[2], l[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        m[n] = -INFINITY;
        l[n] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[n][dt] = f32x4{0, 0, 0, 0};
    }
    const int wpos_lo = p0 + (32 * w) / G, wpos_hi = p0 + (32 * w + 31) / G;
    // last key visible to the wave's rows / to its first row
    const int vis_hi = min(wpos_hi, nkeys - 1), vis_lo = min(wpos_lo, nkeys - 1);

    auto step = [&](int c, const uint16_t *ksc, uint16_t *vsc, uint16_t *ksn, uint16_t *vsn, int (&vf)[4],
                    int64_t kco_next, int64_t vco_next) {
        // Own loads of chunk c done (chunk c+1's, the last LOADS issued, may
        // still fly); the wave converts its V pieces of chunk c; the barrier
        // makes every wave's K, V and flags visible.  The stage chunk c+2
        // goes to was last read in step c-1, which every wave has finished
        // once past this barrier.
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        __asm__ volatile("" ::: "memory");
        uint16_t *vbc = vbk[c & 1];
        convert_v(vsc, vf, vbc);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        issue(c + 2, ksn, vsn, kco_next, vco_next);

        const int k0 = c * KC;
        // skip a chunk no row of this wave can see (wave-uniform)
        if (k0 > vis_hi) return;
        // every key of the chunk visible to every row: no mask
        const bool interior = k0 + KC - 1 <= vis_lo;
        // S^T for both 16-key halves and both row tiles: four independent
        // accumulation chains, so consecutive MFMAs never wait on each other.
        float sv[2][2][4];  // [16-key half][n][j]
        {
            u32x4 ak[2][STEPS];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
                    ak[h][st] = *reinterpret_cast<const u32x4 *>(ksc + ((h * STEPS + st) * 64 + lane) * 8);
            f32x4 acc[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[h][n] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc[h][n] = mfma_16x16x32_bf16(ak[h][st], qv[n][st], acc[h][n]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    if (interior) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) sv[h][n][j] = acc[h][n][j];
                    } else {
                        // key j of this lane is visible iff key <= min(qpos, nkeys - 1)
                        const int d = min(p0 + (32 * w + 16 * n + col) / G, nkeys - 1) - (k0 + 16 * h + 4 * quad);
#pragma unroll
                        for (int j = 0; j < 4; ++j) sv[h][n][j] = j <= d ? acc[h][n][j] : -INFINITY;
                    }
                }
        }
        // V column blocks kept in bf16 (rare): their tiles take P as bf16
        // hi + lo; the others fp16 P x fp16 V.
        const int kept = vf[0] | (vf[1] << 1) | (vf[2] << 2) | (vf[3] << 3);
        u32x4 pf16[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float cm = fmaxf(fmaxf(fmaxf(sv[0][n][0], sv[0][n][1]), fmaxf(sv[0][n][2], sv[0][n][3])),
                             fmaxf(fmaxf(sv[1][n][0], sv[1][n][1]), fmaxf(sv[1][n][2], sv[1][n][3])));
            cm = quad_max_swap(cm) * scale2;
            const bool raise = cm > m[n] + kRescale;
            if (__any(raise)) {
                const float mn = raise ? cm : m[n];
                // rows that have seen no key yet hold zeros: nothing to rescale
                if (__any(raise && m[n] != -INFINITY)) {
                    const float f = (m[n] == -INFINITY) ? 0.0f : exp2f(m[n] - mn);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[n][dt] *= f;
                    l[n] *= f;
                }
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
            // P <= 2^8, so fp16 holds it with 11 significant bits
            pf16[n] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]), pack_f16x2(pv[4], pv[5]),
                            pack_f16x2(pv[6], pv[7])};
        }
        // O^T += V^T P^T: slots 0-3 of a quad are keys 4quad.. of the first
        // 16-key half, slots 4-7 the same keys of the second half, on both
        // operands.
        // fp16 product of every tile (a kept block reads zeros here)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2 a0 = ds_read_tr16(vsc + (dt * 64 + lane) * 4);
            u32x2 a1 = ds_read_tr16(vsc + ((DT + dt) * 64 + lane) * 4);
            u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
            for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(av, pf16[n], oacc[n][dt]);
        }
        if (kept) {
            // A kept block's tiles add the same fp16-rounded P, split exactly
            // into bf16 hi + lo (11 significant bits fit in two bf16), times
            // the raw bf16 V saved by convert_v.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if ((kept >> (dt / 2)) & 1) {
                    u32x2 a0 = ds_read_tr16(vbc + (dt * 64 + lane) * 4);
                    u32x2 a1 = ds_read_tr16(vbc + ((DT + dt) * 64 + lane) * 4);
                    u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        float pf[8];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // (copied out first: a bit cast of a vector element in place
                            // reads element 0 with this compiler)
                            const uint32_t word = pf16[n][e];
                            const f16x2 hp = __builtin_bit_cast(f16x2, word);
                            pf[2 * e] = (float)hp[0];
                            pf[2 * e + 1] = (float)hp[1];
                        }
                        u32x2 h0, l0, h1, l1;
                        split_hi_lo(pf, h0, l0);
                        split_hi_lo(pf + 4, h1, l1);
                        oacc[n][dt] = mfma_16x16x32_bf16(av, u32x4{h0[0], h0[1], h1[0], h1[1]}, oacc[n][dt]);
                        oacc[n][dt] = mfma_16x16x32_bf16(av, u32x4{l0[0], l0[1], l1[0], l1[1]}, oacc[n][dt]);
                    }
                }
            }
        }
    };

    // No key row in the pool (base outside it): no load at all.
    if (nkeys > 0) {
        const int64_t kchunk = (int64_t)KC * krow, vchunk = (int64_t)KC * vrow;
        issue(0, ks0, vs0, 0, 0);
        issue(1, ks1, vs1, kchunk, vchunk);
        if constexpr (QROPE) {
            // Rotate the unrotated q in registers with the RoPE kernel's own
            // helpers (so the result equals RoPE then this kernel, bit for
            // bit).  The wave's 32 rows cover NP positions; entry e = 32 i + f
            // of the table is frequency f at position pw + i (cos in ks2, sin
            // in vs2: the first loads into either are issued after the first
            // step's barrier, which each wave reaches after these reads).
            constexpr int NP = 32 / G;
            static_assert(4 * NP * 32 <= KC * DQK / 2 && 4 * NP * 32 <= KC * DV / 2, "cos/sin table too large");
            float *tc = reinterpret_cast<float *>(ks2) + w * (NP * 32);
            float *ts = reinterpret_cast<float *>(vs2) + w * (NP * 32);
            const int pw = p0 + (32 * w) / G;
#pragma unroll
            for (int e = lane; e < NP * 32; e += 64) {
                float cv, sv;
                rope_cos_sin((int64_t)(pw + e / 32), invf, cv, sv);
                tc[e] = cv;
                ts[e] = sv;
            }
            // (q's loads are tracked here: the compiler waits for them
            // before the first use below; the table was built while they flew)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int pi = (16 * n + col) / G;
                const f32x4 c0 = *reinterpret_cast<const f32x4 *>(tc + 32 * pi + 8 * quad);
                const f32x4 c1 = *reinterpret_cast<const f32x4 *>(tc + 32 * pi + 8 * quad + 4);
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(ts + 32 * pi + 8 * quad);
                const f32x4 s1 = *reinterpret_cast<const f32x4 *>(ts + 32 * pi + 8 * quad + 4);
                const float cc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                const float ss[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                rope_rotate_bf16x8(qv[n][0], qv[n][1], cc, ss);
            }
            settle_q(qv);   // every q load has landed before the loop
        }
        int64_t kco = 2 * kchunk, vco = 2 * vchunk;   // chunk 2, the first one a step issues
        // Unrolled by the three stages; nested so that each step is reached
        // only through the one before it (the compiler then knows which loads
        // into a stage have landed).
        for (int c = 0; c < nch; c += 3) {
            step(c, ks0, vs0, ks2, vs2, vflag[0], kco, vco);
            if (c + 1 < nch) {
                step(c + 1, ks1, vs1, ks0, vs0, vflag[1], kco + kchunk, vco + vchunk);
                if (c + 2 < nch) step(c + 2, ks2, vs2, ks1, vs1, vflag[2], kco + 2 * kchunk, vco + 2 * vchunk);
            }
            kco += 3 * kchunk;
            vco += 3 * vchunk;
        }
        // The dummy loads past the band must land before a stage is reused
        // below (and before the workgroup's LDS is released).
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
    } else {
        wait_vmcnt_q<0>(qv);  // the q loads, before their registers may be reused
    }

    // Epilogue: an optional sink joins the denominator once; scale; bf16.
    // Each wave turns its 32 x 128 output tile around in LDS so that the
    // stores cover whole 256-byte rows, four per instruction.  Tile row
    // stride 256 B, 16-byte units xor-swizzled by (row & 15).
    uint16_t *ep = (w == 0) ? ks0 : (w == 1) ? ks1 : (w == 2) ? ks2 : vs0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = 32 * w + 16 * n + col;
        float ll = quad_sum_swap(l[n]);
        const int head = r % G;
        float mm = m[n], fac = 1.0f;
        if (a.sinks) {
            float sk = a.sinks[g * G + head] * kLog2e;
            float mf = fmaxf(mm, sk);
            fac = exp2f(mm - mf);
            ll = ll * fac + exp2f(sk - mf);
        }
        const float rs = a.value_scale * fac / ll;
        const int row = 16 * n + col;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = oacc[n][dt];
            const u32x2 pk = u32x2{pack_bf16x2(o[0] * rs, o[1] * rs), pack_bf16x2(o[2] * rs, o[3] * rs)};
            const int unit = (2 * dt + (quad >> 1)) ^ (row & 15);
            *reinterpret_cast<u32x2 *>(ep + row * DV + unit * 8 + 4 * (quad & 1)) = pk;
        }
    }
    uint16_t *outg = (uint16_t *)a.out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + (lane >> 4), c = lane & 15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + row * DV + ((c ^ (row & 15)) * 8));
        const int r = 32 * w + row;
        const int local = qb * BQ + r / G;
        if (local < len)
            st16(outg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DV + 8 * c, v);
    }
}

// ---------------------------------------------------------------------
// G = 16 (16 query heads per KV head, both models' full layers): one 8-wave
// workgroup per CU over 256 query rows (16 positions x 16 heads), keys in
// 64-key chunks.  The two halves of the workgroup (waves 0-3: rows 0-127,
// waves 4-7: rows 128-255) share every K/V chunk in LDS and take turns on
// each SIMD: between two workgroup barriers one half issues MFMAs (PV of the
// previous chunk, then S^T of this one, at raised wave priority) while the
// other runs the softmax and the fp16 conversion of V (VALU), then they
// swap, so the two waves of a SIMD keep its matrix and vector units busy at
// once.  Per chunk c, both halves:
//   barrier; issue the loads of chunk c+2;
//   half 0: PV(c-1), S^T(c)          | half 1: softmax(c-1), convert V(c)
//   barrier;
//   half 0: softmax(c), convert V(c) | half 1: PV(c-1), S^T(c)
//   wait for chunk c+1's loads; note its V range.
// K of chunk c is read in iteration c (three K stages), V of chunk c in
// iteration c+1 (four V stages).  V goes to fp16 in place (fp16 P x fp16 V,
// P <= 2^8 by the lazy rescale).  A chunk holding a finite value of
// magnitude 65536 or more (fp16 cannot hold it) sends the workgroup, before
// it has written anything, to a second pass over its keys in which such a
// chunk keeps bf16 V and takes P split exactly into bf16 hi + lo; the common
// loop carries no code for that form.
constexpr int PP_KC = 64;                               // keys per chunk
constexpr int PP_THREADS = 512;
constexpr int PP_WAVES = PP_THREADS / 64;
constexpr int PP_KT = PP_KC / 16;                       // 16-key tiles per chunk
constexpr int PP_K_LOADS = PP_KC * DQK / 8 / PP_THREADS;  // 3 per thread
constexpr int PP_V_LOADS = PP_KC * DV / 8 / PP_THREADS;   // 2 per thread
constexpr int PP_LOADS = PP_K_LOADS + PP_V_LOADS;
constexpr int PP_KSTAGES = 3, PP_VSTAGES = 4;
constexpr int PP_KSTAGE = PP_KC * DQK, PP_VSTAGE = PP_KC * DV;  // bf16 elements
static_assert(PP_K_LOADS * PP_THREADS * 8 == PP_KSTAGE && PP_V_LOADS * PP_THREADS * 8 == PP_VSTAGE,
              "chunk loads must cover the stages exactly");

#define AI __attribute__((always_inline))


// LDS of the G = 16 kernel, at namespace scope so that its two bodies (the
// common one and the general one) share one allocation.
__shared__ __attribute__((aligned(1024))) uint16_t pp_kst[PP_KSTAGES][PP_KSTAGE];
__shared__ __attribute__((aligned(1024))) uint16_t pp_vst[PP_VSTAGES][PP_VSTAGE];
// per V stage and wave: 1 if the wave's V pieces hold a finite value beyond
// the fp16 range (the chunk then stays bf16), else 0
__shared__ __attribute__((aligned(16))) int pp_vbig[PP_VSTAGES][PP_WAVES];

// One workgroup's work.  GEN false: the common body, without the bf16 PV;
// it returns false, having written nothing, at the first chunk that needs
// that form (every wave at the same barrier, all loads landed).  GEN true:
// the general body, either form per chunk.
template <bool QROPE, bool GEN>
__device__ __forceinline__ bool pp_body(const AttnArgs &a, int nqb) {
    constexpr int G = 16, BQ = 256 / G;
    auto &kst = pp_kst;
    auto &vst = pp_vst;
    auto &vbig = pp_vbig;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = w >> 2;
    const int quad = lane >> 4, col = lane & 15;
    const int total = a.n_seqs * a.hkv * nqb;
    const int bid = xcd_remap((int)__builtin_amdgcn_workgroup_id_x(), total);
    const int qb = bid % nqb;
    const int g = (bid / nqb) % a.hkv;
    const int s = bid / (nqb * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int len = (int)(a.cu_seqlens[s + 1] - tok0);
    if (qb * BQ >= len) return true;
    // Positions index pool rows (base + position < pool_rows < 2^31, checked
    // on the host), so they fit in an int; an out-of-contract start is
    // clamped into [0, pool_rows] and its keys to the pool below.
    const int64_t start64 = a.start_pos[s];
    const int start = (int)(start64 < 0 ? 0 : start64 > a.pool_rows ? a.pool_rows : start64);
    const int p0 = start + qb * BQ;
    const int plast = start + min(len, qb * BQ + BQ) - 1;
    const int64_t base = a.seq_base[s];
    int nkeys = plast + 1;
    if (base + nkeys > a.pool_rows) nkeys = (int)(a.pool_rows - base);
    if (base < 0 || nkeys < 0) nkeys = 0;
    const int klast = max(nkeys - 1, 0);
    const int nch = max((nkeys + PP_KC - 1) / PP_KC, 1);

    const double invf = QROPE ? pin_loaded(a.inv_freq[lane & 31]) : 0.0;
    // q of the wave's rows r = 32w + 16n + col (position r / 16, head r % 16)
    u32x4 qv[2][STEPS];
    const uint16_t *qg = (const uint16_t *)a.q;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int r = 32 * w + 16 * n + col;
        const int local = min(qb * BQ + r / G, len - 1);
        const uint16_t *qrow = qg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DQK;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            qv[n][st] = ld16(qrow + 32 * st + 8 * quad);
        }
    }

    // With no key in the pool (out of contract) every chunk is masked and
    // the loads read the pool's first row (the launcher takes this kernel
    // only for pools of at least one row).
    const int64_t b0 = nkeys == 0 ? 0 : base;
    const char *kseq = (const char *)a.k_main + (b0 * a.hkv + g) * (int64_t)(DQK * 2);
    const char *vseq = (const char *)a.v_main + (b0 * a.hkv + g) * (int64_t)(DV * 2);
    const int64_t krow = (int64_t)a.hkv * DQK * 2, vrow = (int64_t)a.hkv * DV * 2;

    // LDS fragment order as in full_prefill_kernel, for 64 keys: K unit
    // (kt * 6 + st) * 64 + lane (16 B) = K[16kt + col][pieces 4st + quad];
    // V 8-byte unit (hh * 8 + dt) * 64 + lane, hh = 16-key tile.  The i-th
    // 16-byte load of wave w fills 1 KB block j = 8i + w (j wave-uniform).
    const int u = lane & 31;
    const int vrow_l = 4 * (u >> 3) + ((u >> 1) & 3);
    const uint32_t vbyte_l = 32 * (lane >> 5) + 16 * (u & 1), kbyte_l = 16 * quad;
    // 32-bit per-lane offsets: 64 rows of either pool span less than 2^31
    // bytes (the launcher checks).
    const uint32_t krow32 = (uint32_t)krow, vrow32 = (uint32_t)vrow;
    // Chunk c's loads into K stage c % 3 and V stage c % 4.  Rows past the
    // last key are clamped to it (finite data, masked); past the band a
    // dummy chunk (the first one again) keeps the count per iteration
    // constant.
    auto issue = [&](int c) AI {
        uint16_t *ksd = kst[c % PP_KSTAGES], *vsd = vst[c % PP_VSTAGES];
        const int kb0 = c < nch ? c * PP_KC : 0;
        const int lim = klast - kb0;   // the chunk's last existing row, >= 0
        const char *kb = kseq + (int64_t)kb0 * krow, *vb = vseq + (int64_t)kb0 * vrow;
#pragma unroll
        for (int i = 0; i < PP_V_LOADS; ++i) {
            const int j = PP_WAVES * i + w;
            const uint32_t row = (uint32_t)min(16 * (j / 4) + vrow_l, lim);
            load_lds16_s(uniform_ptr(vb + 64 * (j % 4)), row * vrow32 + vbyte_l, (const char *)vsd + j * 1024);
        }
#pragma unroll
        for (int i = 0; i < PP_K_LOADS; ++i) {
            const int j = PP_WAVES * i + w;
            const uint32_t row = (uint32_t)min(16 * (j / STEPS) + col, lim);
            load_lds16_s(uniform_ptr(kb + 64 * (j % STEPS)), row * krow32 + kbyte_l, (const char *)ksd + j * 1024);
        }
    };

    // Whether the wave's V pieces of chunk c (landed) hold a finite value of
    // magnitude 65536 or more (bf16 magnitude bits 0x4780 up to, not
    // including, the non-finite 0x7f80): the fp16 conversion would overflow.
    // Non-finite values convert to themselves and do not count.
    auto note_big = [&](int c) AI {
        const char *vsd = (const char *)vst[c % PP_VSTAGES];
        // per 16-bit half: magnitude - 0x4780 (wrapping) < 0x3800 is the
        // range test; the minimum over the pieces decides it
        u16x2 mn = u16x2{0xffff, 0xffff};
#pragma unroll
        for (int i = 0; i < PP_V_LOADS; ++i) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(vsd + (PP_WAVES * i + w) * 1024 + lane * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t mag = raw[e] & 0x7fff7fffu;
                mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2, mag) - u16x2{0x4780, 0x4780});
            }
        }
        const bool any = __any(mn[0] < 0x3800 || mn[1] < 0x3800);
        if (lane == 0) vbig[c % PP_VSTAGES][w] = any ? 1 : 0;
    };
    // Whether chunk c stays bf16 (every wave's note published by a barrier).
    auto chunk_big = [&](int c) AI {
        const u32x4 f0 = *reinterpret_cast<const u32x4 *>(&vbig[c % PP_VSTAGES][0]);
        const u32x4 f1 = *reinterpret_cast<const u32x4 *>(&vbig[c % PP_VSTAGES][4]);
        // the same in every lane: said so, so that a branch on it is scalar
        return __builtin_amdgcn_readfirstlane((f0[0] | f0[1] | f0[2] | f0[3]) | (f1[0] | f1[1] | f1[2] | f1[3])) != 0;
    };
    // Convert the wave's V pieces of chunk c to fp16 in place (exact for
    // bf16 values from 2^-14 up to 65536; smaller ones are rounded to fp16's
    // absolute step 2^-24).  A chunk that stays bf16 is left as loaded.
    auto convert_v = [&](int c, bool big) AI {
        if (big) return;
        char *vsd = (char *)vst[c % PP_VSTAGES];
#pragma unroll
        for (int i = 0; i < PP_V_LOADS; ++i) {
            u32x4 *pp = reinterpret_cast<u32x4 *>(vsd + (PP_WAVES * i + w) * 1024 + lane * 16);
            const u32x4 raw = *pp;
            u32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(raw[e]);
            *pp = h;
        }
    };
    // P (packed fp16) as bf16 hi + lo with hi + lo == P exactly: fp16's 11
    // significant bits are bf16's 8 plus at most 3.
    auto split_p = [&](const u32x4 &p, u32x4 &hi, u32x4 &lo) AI {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // (the element through a scalar: a bit cast of a vector element
            // taken in place reads element 0 whatever the index)
            const uint32_t word = p[e];
            const f16x2 v = __builtin_bit_cast(f16x2, word);
            const float x = (float)v[0], y = (float)v[1];
            const uint32_t xh = __float_as_uint(x) & 0xffff0000u, yh = __float_as_uint(y) & 0xffff0000u;
            hi[e] = (xh >> 16) | yh;
            lo[e] = pack_bf16x2(x - __uint_as_float(xh), y - __uint_as_float(yh));
        }
    };

    const float scale2 = a.scale * kLog2e;
    f32x4 oacc[2][DT];
    // m: reference max per row; lacc: the row sums of the fp16 P the PV
    // products take, formed by the same MFMA with an all-ones V^T operand
    // (every element of a row's lacc holds the sum)
    float m[2];
    f32x4 lacc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        m[n] = -INFINITY;
        lacc[n] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[n][dt] = f32x4{0, 0, 0, 0};
    }
    const u32x4 ones_f16 = u32x4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
    const int wpos_lo = p0 + (32 * w) / G, wpos_hi = p0 + (32 * w + 31) / G;
    const int vis_hi = min(wpos_hi, nkeys - 1), vis_lo = min(wpos_lo, nkeys - 1);
    auto visible = [&](int c) AI { return c >= 0 && c < nch && c * PP_KC <= vis_hi; };

    // S^T of chunk c (accumulators), P of the chunk before (fp16, per row
    // tile and 32-key half)
    f32x4 sacc[PP_KT][2];
    u32x4 pf[2][2];
    // a rescale of O the softmax found needed, applied before the next PV
    bool rs_pend = false;
    float rs_f[2] = {1.0f, 1.0f};
#pragma unroll
    for (int n = 0; n < 2; ++n) pf[n][0] = pf[n][1] = u32x4{0, 0, 0, 0};

    // MFMA phase: PV of chunk c-1 (V stage, P from the softmax), then S^T of c.
    auto mfma_phase = [&](int c, bool bigprev) AI {
        if (visible(c - 1)) {
            const uint16_t *vsc = vst[(c - 1) % PP_VSTAGES];
            if (rs_pend) {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    lacc[n] *= rs_f[n];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[n][dt] *= rs_f[n];
                }
            }
            // row sums of P (both forms of the PV take the same fp16 P)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int n = 0; n < 2; ++n) lacc[n] = mfma_16x16x32_f16(ones_f16, pf[n][kh], lacc[n]);
            if (!bigprev) {
                // 16 tiles (kh, dt) in 4 groups of 4; the V^T reads of group
                // g+1 are issued before the MFMAs of group g (fenced, so the
                // scheduler keeps them a group ahead of their use)
                u32x2 vb[2][4][2];
                auto vread = [&](int g, u32x2 (&d)[4][2]) AI {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kh = (4 * g + i) / DT, dt = (4 * g + i) % DT;
                        d[i][0] = ds_read_tr16(vsc + ((2 * kh * 8 + dt) * 64 + lane) * 4);
                        d[i][1] = ds_read_tr16(vsc + (((2 * kh + 1) * 8 + dt) * 64 + lane) * 4);
                    }
                };
                vread(0, vb[0]);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if (g + 1 < 4) vread(g + 1, vb[(g + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kh = (4 * g + i) / DT, dt = (4 * g + i) % DT;
                        const u32x4 av = u32x4{vb[g & 1][i][0][0], vb[g & 1][i][0][1], vb[g & 1][i][1][0],
                                               vb[g & 1][i][1][1]};
#pragma unroll
                        for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(av, pf[n][kh], oacc[n][dt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // bf16 V times P split exactly into bf16 hi + lo
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    u32x4 ph[2], pl[2];
#pragma unroll
                    for (int n = 0; n < 2; ++n) split_p(pf[n][kh], ph[n], pl[n]);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const u32x2 a0 = ds_read_tr16(vsc + ((2 * kh * 8 + dt) * 64 + lane) * 4);
                        const u32x2 a1 = ds_read_tr16(vsc + (((2 * kh + 1) * 8 + dt) * 64 + lane) * 4);
                        const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                        for (int n = 0; n < 2; ++n) {
                            oacc[n][dt] = mfma_16x16x32_bf16(av, ph[n], oacc[n][dt]);
                            oacc[n][dt] = mfma_16x16x32_bf16(av, pl[n], oacc[n][dt]);
                        }
                    }
                }
            }
        }
        if (visible(c)) {
            const uint16_t *ksc = kst[c % PP_KSTAGES];
#pragma unroll
            for (int kt = 0; kt < PP_KT; ++kt)
#pragma unroll
                for (int n = 0; n < 2; ++n) sacc[kt][n] = f32x4{0, 0, 0, 0};
            // the K reads of step st+1 are issued before the MFMAs of step st
            u32x4 kb[2][PP_KT];
            auto kread = [&](int st, u32x4 (&d)[PP_KT]) AI {
#pragma unroll
                for (int kt = 0; kt < PP_KT; ++kt)
                    d[kt] = *reinterpret_cast<const u32x4 *>(ksc + ((kt * STEPS + st) * 64 + lane) * 8);
            };
            kread(0, kb[0]);
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                if (st + 1 < STEPS) kread(st + 1, kb[(st + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < PP_KT; ++kt)
#pragma unroll
                    for (int n = 0; n < 2; ++n) sacc[kt][n] = mfma_16x16x32_bf16(kb[st & 1][kt], qv[n][st], sacc[kt][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // VALU phase: online softmax of chunk c's S^T into P (fp16).
    auto softmax = [&](int c) AI {
        if (!visible(c)) return;
        const int k0 = c * PP_KC;
        if (k0 + PP_KC - 1 > vis_lo) {
            // key 16 kt + 4 quad + j of the chunk is visible to row r iff it
            // is at most min(position of r, nkeys - 1)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int d = min(p0 + (32 * w + 16 * n + col) / G, nkeys - 1) - (k0 + 4 * quad);
#pragma unroll
                for (int kt = 0; kt < PP_KT; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * kt + j > d) sacc[kt][n][j] = -INFINITY;
            }
        }
        // New reference maxima first; the O rescale (rare) after P, so that
        // it does not overlap the exponentials.
        float fr[2] = {1.0f, 1.0f};
        bool resc = false;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float cm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < PP_KT; ++kt)
                cm = fmaxf(cm, fmaxf(fmaxf(sacc[kt][n][0], sacc[kt][n][1]), fmaxf(sacc[kt][n][2], sacc[kt][n][3])));
            cm = quad_max_swap(cm) * scale2;
            const bool raise = cm > m[n] + kRescale;
            if (__any(raise)) {
                const float mn = raise ? cm : m[n];
                if (__any(raise && m[n] != -INFINITY)) {
                    fr[n] = (m[n] == -INFINITY) ? 0.0f : exp2f(m[n] - mn);
                    resc = true;
                }
                m[n] = mn;
            }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const float mu = m[n] == -INFINITY ? 0.0f : -m[n];
            float pv[PP_KT][4];
#pragma unroll
            for (int kt = 0; kt < PP_KT; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pv[kt][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][n][j], scale2, mu));
            // P <= 2^8: fp16 keeps 11 significant bits.  32-key half kh takes
            // tiles 2kh (slots 0-3) and 2kh + 1 (slots 4-7).
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                pf[n][kh] = u32x4{pack_f16x2(pv[2 * kh][0], pv[2 * kh][1]), pack_f16x2(pv[2 * kh][2], pv[2 * kh][3]),
                                  pack_f16x2(pv[2 * kh + 1][0], pv[2 * kh + 1][1]),
                                  pack_f16x2(pv[2 * kh + 1][2], pv[2 * kh + 1][3])};
        }
        rs_pend = resc;
        rs_f[0] = fr[0];
        rs_f[1] = fr[1];
    };
    auto barrier = [&]() AI {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    // Epilogue: an optional sink joins the denominator once; scale; bf16.
    // Each wave turns its 32 x 128 output tile around in LDS (8 KB of the K
    // stages each) so that the stores cover whole 256-byte rows.
    auto finish = [&]() AI {
        uint16_t *ep = &kst[0][0] + w * (32 * DV);
    #pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int r = 32 * w + 16 * n + col;
            float ll = lacc[n][0];
            const int head = r % G;
            float mm = m[n], fac = 1.0f;
            if (a.sinks) {
                float sk = a.sinks[g * G + head] * kLog2e;
                float mf = fmaxf(mm, sk);
                fac = exp2f(mm - mf);
                ll = ll * fac + exp2f(sk - mf);
            }
            const float rs = a.value_scale * fac / ll;
            const int row = 16 * n + col;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o = oacc[n][dt];
                const u32x2 pk = u32x2{pack_bf16x2(o[0] * rs, o[1] * rs), pack_bf16x2(o[2] * rs, o[3] * rs)};
                const int unit = (2 * dt + (quad >> 1)) ^ (row & 15);
                *reinterpret_cast<u32x2 *>(ep + row * DV + unit * 8 + 4 * (quad & 1)) = pk;
            }
        }
        uint16_t *outg = (uint16_t *)a.out;
    #pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4), c = lane & 15;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + row * DV + ((c ^ (row & 15)) * 8));
            const int r = 32 * w + row;
            const int local = qb * BQ + r / G;
            if (local < len)
                st16(outg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DV + 8 * c, v);
        }
    };

    {
        issue(0);
        issue(1);
        if constexpr (QROPE) {
            // Rotate q in registers with the RoPE kernel's helpers (bit for
            // bit RoPE then this kernel).  The wave's 32 rows cover 2
            // positions; table entry e = 32 i + f is frequency f at position
            // pw + i, cos then sin, in V stage 3 (first loaded in iteration 1).
            float *tc = reinterpret_cast<float *>(vst[3]) + w * 64;
            float *ts = reinterpret_cast<float *>(vst[3]) + PP_WAVES * 64 + w * 64;
            const int pw = p0 + (32 * w) / G;
            {
                float cv, sv;
                rope_cos_sin((int64_t)(pw + lane / 32), invf, cv, sv);
                tc[lane] = cv;
                ts[lane] = sv;
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int pi = (16 * n + col) / G;
                const f32x4 c0 = *reinterpret_cast<const f32x4 *>(tc + 32 * pi + 8 * quad);
                const f32x4 c1 = *reinterpret_cast<const f32x4 *>(tc + 32 * pi + 8 * quad + 4);
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(ts + 32 * pi + 8 * quad);
                const f32x4 s1 = *reinterpret_cast<const f32x4 *>(ts + 32 * pi + 8 * quad + 4);
                const float cc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                const float ss[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                rope_rotate_bf16x8(qv[n][0], qv[n][1], cc, ss);
            }
            settle_q(qv);
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PP_LOADS));
            __asm__ volatile("" ::: "memory");
        } else {
            // q landed here once (the compiler's wait for it, counting only
            // its own loads, is for everything: chunks 0 and 1 too), not at
            // first use inside the loop
            settle_q(qv);
        }
        // The chunk loop, one copy per half.  Half 0 runs the MFMA phase of
        // chunk c first, half 1 its VALU phase; half 1's loop is rotated to
        // start at the second barrier, so that in both copies only P (not
        // S^T) is live across an iteration.
        auto mfma_hi = [&](int c, bool bigprev) AI {
            __builtin_amdgcn_s_setprio(1);
            mfma_phase(c, bigprev);
            __builtin_amdgcn_s_setprio(0);
        };
        auto await_next = [&](int c) AI {   // chunk c+1 landed; its V noted
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PP_LOADS));
            __asm__ volatile("" ::: "memory");
            if (c + 1 < nch) note_big(c + 1);
        };
        auto leave = [&]() AI {   // every load landed and every wave here
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __asm__ volatile("" ::: "memory");
            barrier();
        };
        // Without GEN the loops leave at the first chunk that needs the
        // bf16 PV (known to every wave after the same barrier).
        note_big(0);
        bool bailed = false;
        if (half == 0) {
            bool big_this = false;
#pragma clang loop unroll(disable)
            for (int c = 0; c <= nch; ++c) {
                barrier();                     // chunk c's K, V and V note visible; iteration c-1 done
                issue(c + 2);
                const bool big_prev = big_this;  // chunk c-1, whose PV runs now
                if (c < nch) big_this = chunk_big(c);
                if (!GEN && big_this) {
                    bailed = true;
                    break;
                }
                mfma_hi(c, GEN && big_prev);
                barrier();
                softmax(c);
                if (c < nch) {
                    convert_v(c, GEN && big_this);
                    await_next(c);
                }
            }
        } else {
            barrier();
            issue(2);
            bool big_this = chunk_big(0), big_prev = false;
            if (!GEN && big_this) {
                leave();
                return false;
            }
            convert_v(0, GEN && big_this);
#pragma clang loop unroll(disable)
            for (int c = 0;; ++c) {
                barrier();
                mfma_hi(c, GEN && big_prev);
                if (c == nch) break;
                await_next(c);
                barrier();                     // chunk c+1's K, V and V note visible
                issue(c + 3);
                big_prev = big_this;
                if (c + 1 < nch) big_this = chunk_big(c + 1);
                if (!GEN && big_this) {
                    bailed = true;
                    break;
                }
                softmax(c);
                if (c + 1 < nch) convert_v(c + 1, GEN && big_this);
            }
        }
        leave();   // every load landed (the dummy ones too) before LDS is reused
        if (!GEN && bailed) return false;
        finish();
        return true;
    }
}

template <bool QROPE>
__global__ __launch_bounds__(PP_THREADS, 1) void full_prefill_pp_kernel(AttnArgs a, int nqb) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    // The common body; a workgroup that met a chunk needing the bf16 PV
    // starts over in the general one (its loop comes after the common loop
    // and shares none of its registers).
    if (pp_body<QROPE, false>(a, nqb)) return;
    pp_body<QROPE, true>(a, nqb);
}

}  // namespace

bool full_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == 0 &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

// Shapes the full-attention kernels that rotate q themselves take: the bf16
// fast shapes with a 64-dim rotary part, and (prefill, for the per-wave
// cos/sin table) at least two query heads per KV head.
bool full_qrope_ok(const AttnArgs &a, int dtype, int out_dtype, bool prefill) {
    const int G = a.hq / a.hkv;
    const bool fast = prefill ? full_prefill_fast_ok(a, dtype, out_dtype) : full_decode_fast_ok(a, dtype, out_dtype);
    return fast && a.rope_dim == 64 && (!prefill || G >= 2);
}

hipError_t launch_full_prefill(const AttnArgs &a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    if (G == 16 && a.pool_rows > 0 && (int64_t)a.hkv * DQK * 2 * PP_KC < (int64_t(1) << 31)) {
        const int64_t nqb = (a.max_seqlen + 15) / 16;
        dim3 grid((unsigned)((int64_t)a.n_seqs * a.hkv * nqb)), block(PP_THREADS);
        if (a.qrope)
            hipLaunchKernelGGL((full_prefill_pp_kernel<true>), grid, block, 0, s, a, (int)nqb);
        else
            hipLaunchKernelGGL((full_prefill_pp_kernel<false>), grid, block, 0, s, a, (int)nqb);
        return hipGetLastError();
    }
    const int BQ = 128 / G;
    const int64_t nqb = (a.max_seqlen + BQ - 1) / BQ;
    dim3 grid((unsigned)((int64_t)a.n_seqs * a.hkv * nqb)), block(kThreads);
    const int nq = (int)nqb;
    if (a.qrope) {
        switch (G) {
            case 2: hipLaunchKernelGGL((full_prefill_kernel<2, true>), grid, block, 0, s, a, nq); break;
            case 4: hipLaunchKernelGGL((full_prefill_kernel<4, true>), grid, block, 0, s, a, nq); break;
            case 8: hipLaunchKernelGGL((full_prefill_kernel<8, true>), grid, block, 0, s, a, nq); break;
            default: hipLaunchKernelGGL((full_prefill_kernel<16, true>), grid, block, 0, s, a, nq); break;
        }
        return hipGetLastError();
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((full_prefill_kernel<1, false>), grid, block, 0, s, a, nq); break;
        case 2: hipLaunchKernelGGL((full_prefill_kernel<2, false>), grid, block, 0, s, a, nq); break;
        case 4: hipLaunchKernelGGL((full_prefill_kernel<4, false>), grid, block, 0, s, a, nq); break;
        case 8: hipLaunchKernelGGL((full_prefill_kernel<8, false>), grid, block, 0, s, a, nq); break;
        default: hipLaunchKernelGGL((full_prefill_kernel<16, false>), grid, block, 0, s, a, nq); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
