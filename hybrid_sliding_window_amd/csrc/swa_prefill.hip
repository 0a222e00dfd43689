// swa_prefill.hip -- banded sliding-window prefill with a per-head sink
// (bf16 storage, MFMA).  The ring commit that follows it is ring_commit_kernel
// (generic_attn.hip), launched after it on the same stream.
//
// gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", "What was built": windowed
// prefill as banded tiles with an fp32 softmax that includes the sink;
// "Tiled global-attention prefill": softmax is per query row, so query tiles
// need no merge.  colibri "MiMo-V2.6 (Xiaomi)", "What the engine implements":
// each query sees the last 128 positions (itself included), the sink logit
// joins the denominator only, values carry the value scale (applied to the
// fp32 output); "System One mode and prompt reuse": keys before the chunk
// start come from ring slot p mod 128.
//
// 8 or 16 query heads per KV head take swa_sweep_kernel (end of file), which
// sweeps consecutive query blocks with the window's keys held in LDS.  For
// 1, 2 or 4 heads, one workgroup (4 waves) per query block: 128 rows = 128/G
// positions x the G query heads of one KV head (the heads are the 16-wide
// MFMA columns), two column tiles per wave.  The block's band (positions
// max(0, p0-127) .. its last position) streams through LDS in 32-key chunks
// with a three-stage pipeline: chunk c+2 is fetched by direct global->LDS
// 16-byte loads (no VGPR staging) while chunk c is computed, one barrier per
// chunk; each wave skips chunks outside its rows' windows.  Per chunk:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16 (K rows from LDS, q in VGPRs)
//   softmax          online in log2 units over logits only (the sink joins the
//                    denominator at the end); the reference max is raised only
//                    when a chunk's max exceeds it by more than 2^8 (P <= 256)
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
// run in lane order, free of bank conflicts.  Block ids are remapped so consecutive query
// blocks of one (sequence, KV head) run on one XCD and re-read their
// overlapping bands from its L2.
//
// With QROPE the kernel reads unrotated q and applies the rotate-half RoPE
// itself (colibri "What the engine implements"; the angle in double as the
// gaudi-cookbook "The RoPE fix for large positions" requires), with the same
// helpers and rounding as the RoPE kernel, so the rotated q -- and therefore
// the output -- is bit-identical to RoPE followed by the plain kernel, without
// q_rot's write and re-read.  Each wave puts the cos/sin of its rows'
// positions into its own part of the third pipeline stage, which no load
// reaches before the first step's barrier.
#include "hsw_device.h"
#include "hsw_launch.h"

#include <algorithm>

namespace hsw {
namespace {

constexpr int DQK = 192, DV = 128, W = 128;
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

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds_wave_base + 16 i (lds_wave_base is wave-uniform, passed in m0).  Issued
// as inline asm so the compiler does not track it (it would otherwise add
// waits of its own before LDS reads, for more of these loads than a read
// needs); completion is awaited explicitly (s_waitcnt vmcnt) before the
// barrier that publishes a stage.  m0 is used by nothing else here.
__device__ __forceinline__ void load_lds16(const void *src, const void *lds_wave_base) {
    const uint32_t m = (uint32_t)(uintptr_t)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(src) : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane
// offset: no per-lane address arithmetic.
__device__ __forceinline__ void load_lds16_s(const void *sbase, uint32_t voff, const void *lds_wave_base) {
    const uint32_t m = (uint32_t)(uintptr_t)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m), "v"(voff), "s"(sbase) : "memory", "m0");
}

// 16-byte global load into v, untracked like the loads above: were the
// compiler to track q, its waits for it (merged over the chunk loop) would be
// vmcnt(0) inside every step and drain the chunk pipeline.  The first wait of
// the pipeline covers q, as q is issued first; v keeps its register.
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

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int full = (total / 8) * 8;
    if (bid >= full) return bid;
    return (bid % 8) * (total / 8) + bid / 8;
}

// LDS placement, in 16-byte pieces.
// K: key row r(key) = key ^ ((key >> 3) & 1), piece lp ^ (key & 7) of 24.  A
//    quad's 16 lanes read keys 16h .. 16h+15 at one logical piece: the xor
//    spreads 8 consecutive keys over 8 different 16-byte bank groups and the
//    row swap puts keys k and k+8 on opposite halves of a 256-byte bank line.
// V: row key, piece lp ^ 2 (key & 7) of 16.  A transposing read takes rows
//    4q .. 4q+3 (16 lanes) / 8 rows (32 lanes) at two logical pieces; the xor
//    gives each row its own pair of pieces.

template <int G, bool QROPE>
__global__ __launch_bounds__(kThreads, 2) void swa_prefill_kernel(AttnArgs a, int nqb) {
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
    // Positions are taken relative to the chunk start (its first token is 0),
    // so every position the block handles fits in an int whatever the int64
    // start: relative key kp < 0 is absolute start + kp, which exists iff
    // >= 0, and lives in ring slot (start + kp) mod W.
    const int64_t start = a.start_pos[s];
    const int kmin = start < W - 1 ? -(int)start : -(W - 1);  // lowest relative key that exists
    const int smod = (int)(start & (W - 1));                   // ring slot of relative position 0
    const int p0 = qb * BQ;                         // first query position
    const int plast = min(len, qb * BQ + BQ) - 1;
    const int kstart = max(kmin, p0 - (W - 1));     // band: kstart .. plast
    const int nch = max((plast - kstart + KC) / KC, 1);  // >= 1 (stated so the compiler knows the loop runs)

    // this lane's rotary frequency (fused q-RoPE), loaded before any
    // untracked load
    const double invf = QROPE ? pin_loaded(a.inv_freq[lane & 31]) : 0.0;
    // q of this wave's rows (row r = 32w + 16n + col -> position r / G, head
    // r % G), from a clamped row so the load is unconditional; rows past the
    // chunk only affect their own column and are never stored.
    u32x4 qv[2][STEPS];
    int qpos[2];
    const uint16_t *qg = (const uint16_t *)a.q;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        int r = 32 * w + 16 * n + col;
        int local = min(qb * BQ + r / G, len - 1);
        qpos[n] = p0 + r / G;
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

    // Sources: this sequence's staging rows and ring for KV head g.
    const char *kst = (const char *)a.k_main + (tok0 * a.hkv + g) * (int64_t)(DQK * 2);
    const char *vst = (const char *)a.v_main + (tok0 * a.hkv + g) * (int64_t)(DV * 2);
    const char *kring = (const char *)a.k_ring + ((int64_t)(s * a.hkv + g) * W) * (DQK * 2);
    const char *vring = (const char *)a.v_ring + ((int64_t)(s * a.hkv + g) * W) * (DV * 2);
    const int64_t krow = (int64_t)a.hkv * DQK * 2, vrow = (int64_t)a.hkv * DV * 2;

    // LDS layout: fragment order.  K: 16-byte unit (h * 6 + st) * 64 + lane
    // holds what lane (quad, col) feeds the S^T MFMA of key half h, step st:
    // K[16h + col][pieces 4st + quad].  V: 8-byte unit (hh * 8 + dt) * 64 +
    // lane holds what lane (quad, 4k + mm) supplies to the transposing read of
    // key half hh, output tile dt: V[16hh + 4quad + k][16dt + 4mm .. +3].  So
    // every LDS read is one contiguous 1 KB (K) or 512 B (V) run in lane
    // order: no bank conflicts, and the address is the lane offset plus an
    // immediate.  The load side picks each lane's global source to match: the
    // i-th 16-byte load of wave w fills units (4i + w) * 64 + lane.
    //   K load i: j = 4i + w, h = j / 6, st = j % 6: key 16h + col, bytes
    //             64 st + 16 quad.
    //   V load i: j = 4i + w, hh = j / 4, tiles 2 (j % 4) + (lane >> 5); with
    //             u = lane & 31: row 16hh + 4 (u >> 3) + ((u >> 1) & 3), bytes
    //             64 (j % 4) + 32 (lane >> 5) + 16 (u & 1).
    const int u = lane & 31;
    const int vrow_l = 4 * (u >> 3) + ((u >> 1) & 3);
    const int vbyte_l = 32 * (lane >> 5) + 16 * (u & 1);
    // Interior chunks (all keys from staging, none past plast): source =
    // scalar base + this lane's constant offset.
    const uint32_t koff_l = (uint32_t)(col * krow + 16 * quad);
    const uint32_t voff_l = (uint32_t)(vrow_l * vrow + vbyte_l);

    // Key at relative band position kp: ring slot (start + kp) mod W before
    // the chunk start, staging row kp from it; positions past plast are
    // clamped to plast (finite data, masked).
    auto key_src = [&](int kp, const char *st_base, const char *ring_base, int64_t row_bytes,
                       int ring_row_bytes) -> const char * {
        return kp >= 0 ? st_base + (int64_t)kp * row_bytes
                       : ring_base + (int64_t)((smod + kp) & (W - 1)) * ring_row_bytes;
    };
    auto issue = [&](int c, uint16_t *ksd, uint16_t *vsd) {
        const int k0 = kstart + c * KC;
        if (k0 >= 0 && k0 + KC - 1 <= plast) {
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i) {
                const int j = 4 * i + w, h = j / STEPS, st = j % STEPS;
                load_lds16_s(kst + (int64_t)(k0 + 16 * h) * krow + 64 * st, koff_l,
                             (const char *)ksd + j * 1024);
            }
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                const int j = 4 * i + w, hh = j / 4;
                load_lds16_s(vst + (int64_t)(k0 + 16 * hh) * vrow + 64 * (j % 4), voff_l,
                             (const char *)vsd + j * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i) {
                const int j = 4 * i + w, h = j / STEPS, st = j % STEPS;
                const int kp = min(k0 + 16 * h + col, plast);
                load_lds16(key_src(kp, kst, kring, krow, DQK * 2) + 64 * st + 16 * quad,
                           (const char *)ksd + j * 1024);
            }
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                const int j = 4 * i + w, hh = j / 4;
                const int kp = min(k0 + 16 * hh + vrow_l, plast);
                load_lds16(key_src(kp, vst, vring, vrow, DV * 2) + 64 * (j % 4) + vbyte_l,
                           (const char *)vsd + j * 1024);
            }
        }
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

    auto step = [&](int c, const uint16_t *ksc, uint16_t *vsc, uint16_t *ksn, uint16_t *vsn, int (&vf)[4]) {
        // Own loads of chunk c done (chunk c+1's may still fly); the wave
        // converts its V pieces of chunk c; the barrier makes every wave's K,
        // V and flags visible.  The stage chunk c+2 goes to was last read in
        // step c-1, which every wave has finished once past this barrier.
        __asm__ volatile("" ::: "memory");
        if (c + 1 < nch)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __asm__ volatile("" ::: "memory");
        uint16_t *vbc = vbk[c & 1];
        convert_v(vsc, vf, vbc);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (c + 2 < nch) issue(c + 2, ksn, vsn);

        const int k0 = kstart + c * KC;
        // skip a chunk no row of this wave can see (wave-uniform)
        if (!(k0 <= wpos_hi && k0 + KC - 1 > wpos_lo - W)) return;
        // every key of the chunk inside every row's window: no mask
        const bool interior = k0 + KC - 1 <= wpos_lo && k0 > wpos_hi - W && k0 + KC - 1 <= plast;
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
                        // key j of this lane is visible iff 0 <= qpos - kp < W (kp <= plast follows)
                        const int d = qpos[n] - (k0 + 16 * h + 4 * quad);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            sv[h][n][j] = (unsigned)(d - j) < (unsigned)W ? acc[h][n][j] : -INFINITY;
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

    issue(0, ks0, vs0);
    if (nch > 1) issue(1, ks1, vs1);
    if constexpr (QROPE) {
        // The wave's 32 rows cover NP positions; table entry e = 32 i + f is
        // frequency f at position pw + i (cos in ks2, sin in vs2; the first
        // loads into either are issued after the first step's barrier, which
        // each wave reaches only after its reads below have completed).
        constexpr int NP = 32 / G;
        static_assert(4 * NP * 32 <= KC * DQK / 2 && 4 * NP * 32 <= KC * DV / 2, "cos/sin table too large");
        float *tc = reinterpret_cast<float *>(ks2) + w * (NP * 32);
        float *ts = reinterpret_cast<float *>(vs2) + w * (NP * 32);
        const int pw = p0 + (32 * w) / G;
#pragma unroll
        for (int e = lane; e < NP * 32; e += 64) {
            float cv, sv;
            rope_cos_sin(start + pw + e / 32, invf, cv, sv);
            tc[e] = cv;
            ts[e] = sv;
        }
        // (q's loads are tracked here: the compiler waits for them before
        // the first use below; the table above was built while they flew)
        // Lane (quad, col) holds dims 8 quad .. +7 (step 0) and their
        // partners 32 + 8 quad .. (step 1) of row 32w + 16n + col.
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
    for (int c = 0; c < nch; c += 3) {
        step(c, ks0, vs0, ks2, vs2, vflag[0]);
        if (c + 1 < nch) step(c + 1, ks1, vs1, ks0, vs0, vflag[1]);
        if (c + 2 < nch) step(c + 2, ks2, vs2, ks1, vs1, vflag[2]);
    }

    // Epilogue: the sink joins the denominator once; scale; bf16.  Each wave
    // turns its 32 x 128 output tile around in LDS (a stage no wave reads any
    // more: only the last chunk's stage is still in use) so that the stores
    // cover whole 256-byte rows, four per instruction.  Tile row stride 256 B,
    // 16-byte units xor-swizzled by (row & 15): conflict-free both ways.
    const int sl = (nch - 1) % 3;
    const int fs = (w & 1) ? (sl + 2) % 3 : (sl + 1) % 3;
    uint16_t *ep = (w < 2) ? (fs == 0 ? ks0 : fs == 1 ? ks1 : ks2) : (fs == 0 ? vs0 : fs == 1 ? vs1 : vs2);
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
// 8 or 16 query heads per KV head (both models' windowed layers): a
// workgroup sweeps a segment of consecutive query blocks of one (sequence,
// KV head) and keeps the keys of the moving window in two LDS rings of six
// 32-key chunks (relative keys 32c .. 32c+31 in slot c mod 6), one for K and
// one for V, so each key's K/V is loaded, and its V converted to fp16, once
// per segment rather than once for every block whose window holds it.  A
// block is 128 rows = 128/G positions x G heads, 32 rows per wave; the
// windows of a wave's rows lie in the 5 chunks ending with the one holding
// the block's last position, which the wave takes whole:
//   S^T = K Q^T (v_mfma_f32_16x16x32_bf16), the exact row max over the 5
//   chunks (so no online rescale), P = exp2 relative to it (P <= 1, fp16),
//   its row sums by an MFMA with a 1.0 operand per existing key, and O^T += V^T P^T
//   (v_mfma_f32_16x16x32_f16 with V in fp16; a column block holding a finite
//   V beyond the fp16 range stays bf16 and takes P split exactly into bf16
//   hi + lo).
// The waves are software-pipelined over blocks: block b+1's S^T (matrix
// cores, K from LDS) runs in the same straight-line code as block b's
// exponentials and P V (VALU and matrix cores), so neither unit waits for
// the other.  Hence K runs two blocks ahead (a K chunk is loaded while the
// block before the one that first needs it computes) and V one block ahead.
// Keys outside a row's window are masked; a slot holding another chunk (or
// none yet: the rings start zeroed) only ever meets a mask, so its finite
// contents never count, and no slot a block reads is being loaded.  The
// next block's q loads as soon as S^T has read each step of it; a block's
// output is staged in LDS and stored at the start of the next block, so the
// wait there never covers a store issued just before it.
#define AI __attribute__((always_inline))  // lambdas called from two sites stay inline
constexpr int kSweepGroups = 256;  // workgroups the sweep aims for (one per CU)
constexpr int SW_SLOTS = 6;        // chunk slots of each ring: a band's 5 and the one loading
constexpr int SW_WIN = 5;          // chunks a wave reads per block

__device__ __forceinline__ float pin_f(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int G, bool QROPE>
__global__ __launch_bounds__(kThreads, 1) void swa_sweep_kernel(AttnArgs a, int nbw, int nseg) {
    if (checks_failed(a.dev_flag)) return;  // (checked builds only)
    constexpr int BQ = 128 / G;
    // a block's band p0-127 .. p0+BQ-1 (p0 a multiple of BQ, which divides
    // 16) lies in chunks (p0>>5)-4 .. p0>>5, and every row of a wave (4 or 2
    // consecutive positions, aligned) in chunk p0>>5
    static_assert(16 % BQ == 0 && W % 32 == 0 && W / 32 + 1 == SW_WIN && SW_WIN < SW_SLOTS, "band and ring");
    __shared__ __attribute__((aligned(1024))) uint16_t kr[SW_SLOTS][KC * DQK];
    __shared__ __attribute__((aligned(1024))) uint16_t vr[SW_SLOTS][KC * DV];
    // per wave: the output tile of the block before (32 rows x 128)
    __shared__ __attribute__((aligned(1024))) uint16_t stg[4][32 * DV];
    // per wave: the cos/sin table of the fused q-RoPE (32 / G positions)
    __shared__ __attribute__((aligned(16))) float rtab[4][QROPE ? 2 * (32 / G) * 32 : 4];
    // per V slot and wave: 1 if the wave's column block of the chunk's V
    // (dims 32w .. 32w+31) stayed bf16
    __shared__ __attribute__((aligned(16))) int vbig[SW_SLOTS][4];
    // per V slot: the fp16 A operand of the row-sum MFMA for each quad, 1.0
    // for a key of the chunk that exists (>= kmin), 0 for one that does not
    __shared__ __attribute__((aligned(16))) uint32_t vvalid[SW_SLOTS][4][4];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int quad = lane >> 4, col = lane & 15;
    const int bid = (int)__builtin_amdgcn_workgroup_id_x();
    const int seg = bid % nseg;
    const int g = (bid / nseg) % a.hkv;
    const int s = bid / (nseg * a.hkv);

    const int64_t tok0 = a.cu_seqlens[s];
    const int len = (int)(a.cu_seqlens[s + 1] - tok0);
    const int b_begin = seg * nbw, b_end = min((len + BQ - 1) / BQ, b_begin + nbw);
    if (b_begin >= b_end) return;
    // Relative positions (the chunk's first token is 0): key kp < 0 is
    // absolute position start + kp, which exists iff kp >= kmin, and lives in
    // ring slot (start + kp) mod W.
    const int64_t start = a.start_pos[s];
    const int kmin = start < W - 1 ? -(int)start : -(W - 1);
    const int smod = (int)(start & (W - 1));
    const int plast = len - 1;
    auto band_lo = [&](int b) AI { return max(kmin, b * BQ - (W - 1)); };
    auto band_hi = [&](int b) AI { return min(plast, b * BQ + BQ - 1); };
    // the last chunk of block b's window (it holds the block's stored rows)
    auto top_chunk = [&](int b) AI { return band_hi(b) >> 5; };

    const double invf = QROPE ? pin_loaded(a.inv_freq[lane & 31]) : 0.0;
    float sk2[2] = {0.0f, 0.0f};  // the rows' sink logits in log2 units
    if (a.sinks) {
#pragma unroll
        for (int n = 0; n < 2; ++n) sk2[n] = pin_f(a.sinks[g * G + (32 * w + 16 * n + col) % G] * kLog2e);
    }

    const uint16_t *qg = (const uint16_t *)a.q;
    // q step st of the wave's rows r = 32w + 16n + col (position r / G,
    // head r % G) of block b; rows past the sequence read its last row
    // (their outputs are not stored).  Ordinary loads: the first use follows
    // the wait at the next block's start, where the compiler's wait costs
    // nothing.
    auto load_q_step = [&](int b, int st, u32x4 (&qv)[2][STEPS]) AI {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int r = 32 * w + 16 * n + col;
            const int local = min(b * BQ + r / G, plast);
            qv[n][st] = ld16(qg + ((tok0 + local) * a.hq + g * G + r % G) * (int64_t)DQK + 32 * st + 8 * quad);
        }
    };

    const char *kst = (const char *)a.k_main + (tok0 * a.hkv + g) * (int64_t)(DQK * 2);
    const char *vst = (const char *)a.v_main + (tok0 * a.hkv + g) * (int64_t)(DV * 2);
    const char *kring = (const char *)a.k_ring + ((int64_t)(s * a.hkv + g) * W) * (DQK * 2);
    const char *vring = (const char *)a.v_ring + ((int64_t)(s * a.hkv + g) * W) * (DV * 2);
    const int64_t krow = (int64_t)a.hkv * DQK * 2, vrow = (int64_t)a.hkv * DV * 2;
    // A chunk's LDS layout is the fragment order of swa_prefill_kernel: K
    // 16-byte unit (h * 6 + st) * 64 + lane, V 8-byte unit (hh * 8 + dt) *
    // 64 + lane; the i-th load of wave w fills 1 KB unit group 4i + w, so
    // wave w's V pieces are the chunk's column block w (tiles 2w, 2w+1).
    const int u = lane & 31;
    const int vrow_l = 4 * (u >> 3) + ((u >> 1) & 3);
    const int vbyte_l = 32 * (lane >> 5) + 16 * (u & 1);
    auto slot_of = [&](int c) AI { return (c + 8 * SW_SLOTS) % SW_SLOTS; };  // c >= -48
    // K or V of chunk c (relative keys 32c .. 32c+31, each clamped into
    // kmin .. plast: finite data, masked where outside a window) into its slot
    auto issue_k = [&](int c) AI {
        const int k0 = 32 * c;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int j = 4 * i + w, h = j / STEPS, st = j % STEPS;
            const int kp = min(max(k0 + 16 * h + col, kmin), plast);
            const char *src = kp >= 0 ? kst + (int64_t)kp * krow : kring + (int64_t)((smod + kp) & (W - 1)) * (DQK * 2);
            load_lds16(src + 64 * st + 16 * quad, (const char *)kr[slot_of(c)] + j * 1024);
        }
    };
    auto issue_v = [&](int c) AI {
        const int k0 = 32 * c;
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i) {
            const int j = 4 * i + w, hh = j / 4;
            const int kp = min(max(k0 + 16 * hh + vrow_l, kmin), plast);
            const char *src = kp >= 0 ? vst + (int64_t)kp * vrow : vring + (int64_t)((smod + kp) & (W - 1)) * (DV * 2);
            load_lds16(src + 64 * (j % 4) + vbyte_l, (const char *)vr[slot_of(c)] + j * 1024);
        }
    };
    // The wave's column block of chunk c's V (landed) to fp16 in place, or,
    // if it holds a finite value of magnitude 65536 or more (bf16 magnitude
    // bits 0x4780 up to, not including, 0x7f80), left bf16 and flagged.  fp16
    // holds every other bf16 value exactly from 2^-14 up, smaller magnitudes
    // to its absolute step 2^-24.
    auto settle_v = [&](int c) AI {
        char *vsd = (char *)vr[slot_of(c)];
        u32x4 raw[V_LOADS];
        bool big = false;
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i) {
            raw[i] = *reinterpret_cast<const u32x4 *>(vsd + (4 * i + w) * 1024 + lane * 16);
            // (a key that does not exist: V row zero; the piece is one key's)
            if (32 * c + 16 * i + vrow_l < kmin) {
                raw[i] = u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4 *>(vsd + (4 * i + w) * 1024 + lane * 16) = raw[i];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t word = raw[i][e];
                const uint32_t lo = word & 0x7fffu, hi = (word >> 16) & 0x7fffu;
                big |= (lo - 0x4780u < 0x3800u) || (hi - 0x4780u < 0x3800u);
            }
        }
        const bool keep = __any(big);
        if (!keep) {
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                u32x4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(raw[i][e]);
                *reinterpret_cast<u32x4 *>(vsd + (4 * i + w) * 1024 + lane * 16) = h;
            }
        }
        if (lane == 0) vbig[slot_of(c)][w] = keep ? 1 : 0;
        // slots 0-3 of quad q: keys 4q .. 4q+3 of the first 16-key half,
        // slots 4-7 the same keys of the second half (P's slot order)
        if (w == 0 && lane < 16) {
            const int q = lane >> 2, e = lane & 3;
            const int k0 = 32 * c + 4 * q + (e < 2 ? 2 * e : 16 + 2 * (e - 2));
            vvalid[slot_of(c)][q][e] = (k0 >= kmin ? 0x3c00u : 0u) | (k0 + 1 >= kmin ? 0x3c000000u : 0u);
        }
    };
    auto barrier = [&]() AI {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    uint16_t *ep = &stg[w][0];
    uint16_t *obase = (uint16_t *)a.out + (tok0 * a.hq + g * G) * (int64_t)DV;
    // Store the wave's rows of block b staged in ep, in 8 parts: in part i,
    // lane (lane >> 4, c) stores 16 bytes c of tile row 4i + (lane >> 4), i.e.
    // wave row r = 32w + 4i + (lane >> 4), at position (32w + 4i) / G of the
    // block (the same for the part's 4 rows: G is 8 or 16), head (4i) % G +
    // (lane >> 4); rows past the sequence not.  Tile row stride 256 B,
    // 16-byte units xor-swizzled by row & 15.
    // (all eight parts read first, so their LDS latency is paid once)
    auto store_out = [&](int b) AI {
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4), c = lane & 15;
            v[i] = *reinterpret_cast<const u32x4 *>(ep + row * DV + ((c ^ (row & 15)) * 8));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rq = (32 * w + 4 * i) / G;
            if (b * BQ + rq < len) {
                uint16_t *ob = obase + (int64_t)(b * BQ + rq) * a.hq * DV;
                // (non-temporal: nothing here reads the output again)
                __builtin_nontemporal_store(
                    v[i], reinterpret_cast<u32x4 *>(ob + (uint32_t)((((4 * i) % G) + (lane >> 4)) * DV + 8 * (lane & 15))));
            }
        }
    };
    // The fused q-RoPE of block b's q: cos/sin of the wave's NP positions in
    // its table, then rotate-half of dims 0 .. 63.
    auto rope_q = [&](int b, u32x4 (&qv)[2][STEPS]) AI {
        constexpr int NP = 32 / G;
        float *tc = &rtab[w][0];
        float *ts = tc + NP * 32;
        const int pw = b * BQ + (32 * w) / G;
#pragma unroll
        for (int e = lane; e < NP * 32; e += 64) {
            float cv, sv;
            rope_cos_sin(start + pw + e / 32, invf, cv, sv);
            tc[e] = cv;
            ts[e] = sv;
        }
        // lane (quad, col) holds dims 8 quad .. +7 (step 0) and their
        // rotation partners 32 + 8 quad .. (step 1) of row 32w + 16n + col
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
    };

    // the rings start zeroed: a slot not loaded yet holds finite values
    {
        constexpr int KU = SW_SLOTS * KC * DQK / 8, VU = SW_SLOTS * KC * DV / 8;
        for (int i = tid; i < KU; i += kThreads) reinterpret_cast<u32x4 *>(&kr[0][0])[i] = u32x4{0, 0, 0, 0};
        for (int i = tid; i < VU; i += kThreads) reinterpret_cast<u32x4 *>(&vr[0][0])[i] = u32x4{0, 0, 0, 0};
        if (tid < SW_SLOTS * 4) reinterpret_cast<u32x4 *>(&vvalid[0][0][0])[tid] = u32x4{0, 0, 0, 0};
        barrier();
    }

    const float scale2 = a.scale * kLog2e;
    int ck_next = band_lo(b_begin) >> 5;  // next K chunk to load
    int cv_next = ck_next;                // next V chunk to load
    int cv_conv = cv_next;                // next landed V chunk to settle
    int slotkept = 0;                     // 4 bits per V slot: column blocks kept bf16
    u32x4 qv[2][STEPS];

    // S^T = K Q^T of block b (q in qv, landed): lane (quad, col) gets keys
    // 4 quad .. +3 of each 16-key half of each window chunk against row
    // 32w + 16n + col.  Step-major, so each step's q registers are free
    // early: block b+1's q for that step loads right away (its rows clamped
    // into the sequence, so past the segment it loads rows it does not use).
    auto s_phase = [&](int b, f32x4 (&sacc)[SW_WIN][2][2]) AI {
        const int ct = top_chunk(b);
#pragma unroll
        for (int i = 0; i < SW_WIN; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int n = 0; n < 2; ++n) sacc[i][h][n] = f32x4{0, 0, 0, 0};
        // K operands one step ahead of the MFMAs that take them (a fence per
        // step keeps that order, so each read has a step's MFMAs to land)
        u32x4 kb[2][SW_WIN][2];
        auto read_k = [&](int st, u32x4 (&dst)[SW_WIN][2]) AI {
#pragma unroll
            for (int i = 0; i < SW_WIN; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    dst[i][h] = *reinterpret_cast<const u32x4 *>(kr[slot_of(ct - (SW_WIN - 1) + i)] +
                                                                 ((h * STEPS + st) * 64 + lane) * 8);
        };
        read_k(0, kb[0]);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (st + 1 < STEPS) read_k(st + 1, kb[(st + 1) & 1]);
#pragma unroll
            for (int i = 0; i < SW_WIN; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int n = 0; n < 2; ++n) sacc[i][h][n] = mfma_16x16x32_bf16(kb[st & 1][i][h], qv[n][st], sacc[i][h][n]);
            load_q_step(b + 1, st, qv);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Softmax numerators of block b from its S^T: every stored row's
    // position lies in chunk ct (a wave's rows are 4 or 2 aligned positions
    // of one block), so chunks 1 .. 3 of the window are inside each row's
    // window and only chunk 0 (keys below pos - 127) and chunk 4 (keys past
    // pos) take a mask.  A key below kmin does not exist; where it falls in
    // chunks 1 .. 3 (a block near the start of a sequence with fewer than
    // W-1 earlier positions) its K is key kmin's, which lies in every row's
    // window, so it leaves the row max as it is; its V is zero and the row
    // sums leave it out (vvalid), so it adds nothing.  Then the exact row max m (in log2 units) and P = exp2(s scale2
    // - m) <= 1 in fp16 (slots 0-3: keys 4 quad.. of the first 16-key half,
    // 4-7 of the second, as V^T's slots).  In pieces, to interleave with
    // other work: t = 0 .. 9 mask and max of chunk t % 5 for rows n = t / 5;
    // t = 10, 11 the row max of n = t - 10; t = 12 .. 21 the numerators of
    // chunk (t - 12) % 5 for n = (t - 12) / 5.
    constexpr int SM_PIECES = 4 * SW_WIN + 2;
    auto softmax_piece = [&](int t, int b, f32x4 (&sacc)[SW_WIN][2][2], u32x4 (&pf)[SW_WIN][2], float (&mx)[2],
                             float (&mrow)[2]) AI {
        if (t < 2 * SW_WIN) {
            const int i = t % SW_WIN, n = t / SW_WIN;
            const int pos = b * BQ + (32 * w + 16 * n + col) / G;
            const int klo = pos - (W - 1);
            const int ct = top_chunk(b);
            if (i == 0) mx[n] = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = 32 * (ct - (SW_WIN - 1) + i) + 16 * h + 4 * quad;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (i == 0) sacc[i][h][n][j] = kk + j >= klo ? sacc[i][h][n][j] : -INFINITY;
                    if (i == SW_WIN - 1) sacc[i][h][n][j] = kk + j <= pos ? sacc[i][h][n][j] : -INFINITY;
                    mx[n] = fmaxf(mx[n], sacc[i][h][n][j]);
                }
            }
        } else if (t < 2 * SW_WIN + 2) {
            const int n = t - 2 * SW_WIN;
            // (every row sees at least key min(pos, plast): finite)
            mrow[n] = quad_max_swap(mx[n]) * scale2;
        } else {
            const int i = (t - 2 * SW_WIN - 2) % SW_WIN, n = (t - 2 * SW_WIN - 2) / SW_WIN;
            float pv[8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pv[4 * h + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i][h][n][j], scale2, -mrow[n]));
            pf[i][n] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]), pack_f16x2(pv[4], pv[5]),
                             pack_f16x2(pv[6], pv[7])};
        }
    };
    auto softmax = [&](int b, f32x4 (&sacc)[SW_WIN][2][2], u32x4 (&pf)[SW_WIN][2], float (&mrow)[2]) AI {
        float mx[2];
#pragma unroll
        for (int t = 0; t < SM_PIECES; ++t) softmax_piece(t, b, sacc, pf, mx, mrow);
    };

    // Block b, whose P is in pcur: block b+1's S^T, then block b+1's softmax
    // (VALU) alongside block b's P V (matrix cores), then block b's output.
    auto block = [&](int b, u32x4 (&pcur)[SW_WIN][2], float (&mcur)[2], u32x4 (&pnext)[SW_WIN][2],
                     float (&mnext)[2]) AI {
        // every load and store of this wave done: q of b+1, the K chunk for
        // block b+1's band, the V chunk for block b's, the stores of b-2
        wait_vmcnt_q<0>(qv);
        for (int c = cv_conv; c < cv_next; ++c) settle_v(c);
        // every wave's chunks, conversions and flags in; every wave past block b-1
        barrier();
        for (int c = cv_conv; c < cv_next; ++c) {
            const u32x4 f = *reinterpret_cast<const u32x4 *>(&vbig[slot_of(c)][0]);
            const int bits = (f[0] ? 1 : 0) | (f[1] ? 2 : 0) | (f[2] ? 4 : 0) | (f[3] ? 8 : 0);
            const int sh = 4 * slot_of(c);
            slotkept = (slotkept & ~(15 << sh)) | (__builtin_amdgcn_readfirstlane(bits) << sh);
        }
        cv_conv = cv_next;
        if (b > b_begin) store_out(b - 1);
        // The slot a new chunk goes to last held the chunk 6 before it: for
        // K, below block b+1's window (the one read now); for V, below block
        // b's.
        if (b + 2 < b_end && ck_next <= top_chunk(b + 2)) {
            issue_k(ck_next);
            ++ck_next;
        }
        if (b + 1 < b_end && cv_next <= top_chunk(b + 1)) {
            issue_v(cv_next);
            ++cv_next;
        }
        if constexpr (QROPE) rope_q(b + 1, qv);
        f32x4 sacc[SW_WIN][2][2];
        s_phase(b + 1, sacc);

        // O^T = V^T P^T; the row sums of the fp16 P by an MFMA whose A
        // operand is 1.0 for each key that exists (every element of
        // lacc[n]'s column is row col's sum)
        const int ct = top_chunk(b);
        f32x4 oacc[2][DT], lacc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            lacc[n] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[n][dt] = f32x4{0, 0, 0, 0};
        }
        // the row-sum operand of window chunk i (all 1.0 where every key exists)
        auto valid_op = [&](int i) AI {
            return *reinterpret_cast<const u32x4 *>(&vvalid[slot_of(ct - (SW_WIN - 1) + i)][quad][0]);
        };
        int kept_any = 0;
#pragma unroll
        for (int i = 0; i < SW_WIN; ++i) kept_any |= (slotkept >> (4 * slot_of(ct - (SW_WIN - 1) + i))) & 15;
        if (kept_any == 0) {
            // 20 groups: each issues the V^T reads of the P V units two
            // groups on (unit u: chunk u / 8, tile u % 8), takes two units'
            // MFMAs and one piece of block b+1's softmax; a fence per group
            // keeps the interleave
            constexpr int UNITS = SW_WIN * DT, GROUPS = UNITS / 2;
            static_assert(GROUPS + 2 == SM_PIECES, "one softmax piece per group, two after");
            u32x4 vb[6];
            auto read_v = [&](int u2) AI {
                const uint16_t *vsc = vr[slot_of(ct - (SW_WIN - 1) + u2 / DT)];
                const int dt = u2 % DT;
                const u32x2 a0 = ds_read_tr16(vsc + (dt * 64 + lane) * 4);
                const u32x2 a1 = ds_read_tr16(vsc + ((DT + dt) * 64 + lane) * 4);
                vb[u2 % 6] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            };
            float mx[2];
#pragma unroll
            for (int u2 = 0; u2 < 4; ++u2) read_v(u2);
#pragma unroll
            for (int gi = 0; gi < GROUPS; ++gi) {
                if (2 * gi + 4 < UNITS) read_v(2 * gi + 4);
                if (2 * gi + 5 < UNITS) read_v(2 * gi + 5);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    const int u2 = 2 * gi + uu, i = u2 / DT, dt = u2 % DT;
#pragma unroll
                    for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(vb[u2 % 6], pcur[i][n], oacc[n][dt]);
                }
                if (gi % 4 == 0) {
#pragma unroll
                    for (int n = 0; n < 2; ++n) lacc[n] = mfma_16x16x32_f16(valid_op(gi / 4), pcur[gi / 4][n], lacc[n]);
                }
                softmax_piece(gi, b + 1, sacc, pnext, mx, mnext);
                __builtin_amdgcn_sched_barrier(0);
            }
            softmax_piece(GROUPS, b + 1, sacc, pnext, mx, mnext);
            softmax_piece(GROUPS + 1, b + 1, sacc, pnext, mx, mnext);
        } else {
            softmax(b + 1, sacc, pnext, mnext);
#pragma unroll
            for (int i = 0; i < SW_WIN; ++i) {
                const int sl = slot_of(ct - (SW_WIN - 1) + i);
                const uint16_t *vsc = vr[sl];
                const int kept = (slotkept >> (4 * sl)) & 15;
#pragma unroll
                for (int n = 0; n < 2; ++n) lacc[n] = mfma_16x16x32_f16(valid_op(i), pcur[i][n], lacc[n]);
                // a kept column block's tiles take the fp16-rounded P split
                // exactly into bf16 hi + lo (11 significant bits fit in two
                // bf16) times its raw bf16 V
                u32x4 ph[2], pl[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    float pr[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // (copied out first: a bit cast of a vector element in
                        // place reads element 0 with this compiler)
                        const uint32_t word = pcur[i][n][e];
                        const f16x2 hp = __builtin_bit_cast(f16x2, word);
                        pr[2 * e] = (float)hp[0];
                        pr[2 * e + 1] = (float)hp[1];
                    }
                    u32x2 h0, l0, h1, l1;
                    split_hi_lo(pr, h0, l0);
                    split_hi_lo(pr + 4, h1, l1);
                    ph[n] = u32x4{h0[0], h0[1], h1[0], h1[1]};
                    pl[n] = u32x4{l0[0], l0[1], l1[0], l1[1]};
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2 a0 = ds_read_tr16(vsc + (dt * 64 + lane) * 4);
                    const u32x2 a1 = ds_read_tr16(vsc + ((DT + dt) * 64 + lane) * 4);
                    const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
                    if ((kept >> (dt / 2)) & 1) {
#pragma unroll
                        for (int n = 0; n < 2; ++n) {
                            oacc[n][dt] = mfma_16x16x32_bf16(av, ph[n], oacc[n][dt]);
                            oacc[n][dt] = mfma_16x16x32_bf16(av, pl[n], oacc[n][dt]);
                        }
                    } else {
#pragma unroll
                        for (int n = 0; n < 2; ++n) oacc[n][dt] = mfma_16x16x32_f16(av, pcur[i][n], oacc[n][dt]);
                    }
                }
            }
        }
        // Epilogue: the sink joins the denominator once; value scale; bf16
        // into the staging tile, stored at the start of the next block.
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float ll = lacc[n][0], fac = 1.0f;
            if (a.sinks) {
                const float mf = fmaxf(mcur[n], sk2[n]);
                fac = __builtin_amdgcn_exp2f(mcur[n] - mf);
                ll = ll * fac + __builtin_amdgcn_exp2f(sk2[n] - mf);
            }
            const float rs = a.value_scale * fac * __builtin_amdgcn_rcpf(ll);
            const int row = 16 * n + col;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o = oacc[n][dt];
                const u32x2 pk = u32x2{pack_bf16x2(o[0] * rs, o[1] * rs), pack_bf16x2(o[2] * rs, o[3] * rs)};
                const int unit = (2 * dt + (quad >> 1)) ^ (row & 15);
                *reinterpret_cast<u32x2 *>(ep + row * DV + unit * 8 + 4 * (quad & 1)) = pk;
            }
        }
    };

    // Prologue: q of the first block; K of the first two blocks' bands (at
    // most 6 chunks), V of the first's; the first block's S^T and softmax.
#pragma unroll
    for (int st = 0; st < STEPS; ++st) load_q_step(b_begin, st, qv);
    for (; ck_next <= top_chunk(min(b_begin + 1, b_end - 1)); ++ck_next) issue_k(ck_next);
    for (; cv_next <= top_chunk(b_begin); ++cv_next) issue_v(cv_next);
    wait_vmcnt_q<0>(qv);
    barrier();
    if constexpr (QROPE) rope_q(b_begin, qv);
    u32x4 pa[SW_WIN][2], pb[SW_WIN][2];
    float ma[2], mb[2];
    {
        f32x4 sacc[SW_WIN][2][2];
        s_phase(b_begin, sacc);
        softmax(b_begin, sacc, pa, ma);
    }
#pragma unroll 1
    for (int b = b_begin; b < b_end; b += 2) {
        block(b, pa, ma, pb, mb);
        if (b + 1 < b_end) block(b + 1, pb, mb, pa, ma);
    }
    wait_vmcnt_q<0>(qv);
    store_out(b_end - 1);
}

}  // namespace

bool swa_prefill_fast_ok(const AttnArgs &a, int dtype, int out_dtype) {
    int G = a.hq / a.hkv;
    return dtype == 0 && out_dtype == 0 && a.dqk == DQK && a.dv == DV && a.window == W &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

// Shapes the kernels that rotate q themselves take: the bf16 fast shapes with
// a 64-dim rotary part, and (prefill, for the per-wave cos/sin table) at least
// two query heads per KV head.
bool swa_qrope_ok(const AttnArgs &a, int dtype, int out_dtype, bool prefill) {
    const int G = a.hq / a.hkv;
    const bool fast = prefill ? swa_prefill_fast_ok(a, dtype, out_dtype) : swa_decode_fast_ok(a, dtype, out_dtype);
    return fast && a.rope_dim == 64 && (!prefill || G >= 2);
}

hipError_t launch_swa_prefill(const AttnArgs &a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const int BQ = 128 / G;
    const int64_t nqb = (a.max_seqlen + BQ - 1) / BQ;
    if (G >= 8) {
        // segments of nbw query blocks: about one workgroup per CU
        const int64_t pairs = (int64_t)a.n_seqs * a.hkv;
        const int64_t want = std::max<int64_t>(1, std::min<int64_t>(nqb, (kSweepGroups + pairs - 1) / pairs));
        const int nbw = (int)((nqb + want - 1) / want);
        const int nseg = (int)((nqb + nbw - 1) / nbw);
        dim3 grid((unsigned)(pairs * nseg)), block(kThreads);
        if (G == 8) {
            if (a.qrope) hipLaunchKernelGGL((swa_sweep_kernel<8, true>), grid, block, 0, s, a, nbw, nseg);
            else hipLaunchKernelGGL((swa_sweep_kernel<8, false>), grid, block, 0, s, a, nbw, nseg);
        } else {
            if (a.qrope) hipLaunchKernelGGL((swa_sweep_kernel<16, true>), grid, block, 0, s, a, nbw, nseg);
            else hipLaunchKernelGGL((swa_sweep_kernel<16, false>), grid, block, 0, s, a, nbw, nseg);
        }
        return hipGetLastError();
    }
    // 1, 2 or 4 query heads per KV head: a workgroup per query block
    dim3 grid((unsigned)((int64_t)a.n_seqs * a.hkv * nqb)), block(kThreads);
    const int nq = (int)nqb;
    if (a.qrope) {
        if (G == 2) hipLaunchKernelGGL((swa_prefill_kernel<2, true>), grid, block, 0, s, a, nq);
        else hipLaunchKernelGGL((swa_prefill_kernel<4, true>), grid, block, 0, s, a, nq);
        return hipGetLastError();
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((swa_prefill_kernel<1, false>), grid, block, 0, s, a, nq); break;
        case 2: hipLaunchKernelGGL((swa_prefill_kernel<2, false>), grid, block, 0, s, a, nq); break;
        default: hipLaunchKernelGGL((swa_prefill_kernel<4, false>), grid, block, 0, s, a, nq); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
