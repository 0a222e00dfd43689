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
// One workgroup (4 waves) per query block: 128 rows = 128/G positions x the G
// query heads of one KV head (the heads are the 16-wide MFMA columns), two
// column tiles per wave.  The block's band (positions max(0, p0-127) .. its
// last position, <= 143 keys for G = 8) streams through LDS in 32-key chunks
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
    dim3 grid((unsigned)((int64_t)a.n_seqs * a.hkv * nqb)), block(kThreads);
    const int nq = (int)nqb;
    if (a.qrope) {
        switch (G) {
            case 2: hipLaunchKernelGGL((swa_prefill_kernel<2, true>), grid, block, 0, s, a, nq); break;
            case 4: hipLaunchKernelGGL((swa_prefill_kernel<4, true>), grid, block, 0, s, a, nq); break;
            case 8: hipLaunchKernelGGL((swa_prefill_kernel<8, true>), grid, block, 0, s, a, nq); break;
            default: hipLaunchKernelGGL((swa_prefill_kernel<16, true>), grid, block, 0, s, a, nq); break;
        }
        return hipGetLastError();
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((swa_prefill_kernel<1, false>), grid, block, 0, s, a, nq); break;
        case 2: hipLaunchKernelGGL((swa_prefill_kernel<2, false>), grid, block, 0, s, a, nq); break;
        case 4: hipLaunchKernelGGL((swa_prefill_kernel<4, false>), grid, block, 0, s, a, nq); break;
        case 8: hipLaunchKernelGGL((swa_prefill_kernel<8, false>), grid, block, 0, s, a, nq); break;
        default: hipLaunchKernelGGL((swa_prefill_kernel<16, false>), grid, block, 0, s, a, nq); break;
    }
    return hipGetLastError();
}

}  // namespace hsw
