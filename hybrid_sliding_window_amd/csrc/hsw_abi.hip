// hsw_abi.hip -- the C ABI of libhsw: host-side argument checks and dispatch.
//
// Every entry point validates its arguments before any launch; on failure it
// returns an HSW_E_* code, records a message for hsw_last_error() and
// launches nothing.  Zero-sized calls return HSW_OK without a launch.  No C++
// exception crosses the boundary.  Device-resident values (positions,
// lengths, bases) are never read here: the kernels bound their own accesses.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/hsw.h"
#include "dev_check.h"
#include "hsw_launch.h"

#ifndef HSW_CHECK_DEVICE
#define HSW_CHECK_DEVICE 0
#endif

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace hsw {
hsw_status vfail(hsw_status st, const char *fmt, va_list ap) {
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    return st;
}
hsw_status fail(hsw_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace hsw

namespace {
using hsw::fail;
namespace dc = hsw::devcheck;

// Pool rows are addressed by int positions in the kernels; no pool that fits
// in one GPU's memory comes near this many rows.
constexpr int64_t kMaxPoolRows = 0x7fffffffLL;

// Module memory is per device: each GPU holds its own copy of a __device__
// variable at its own address.  Host code takes that address once per device
// (with the device current) and uses only it.
constexpr int kMaxDevices = 64;
std::mutex g_symbol_mu;

hsw_status symbol_address(const void *symbol, void *(&cache)[kMaxDevices], void **out, const char *what) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(HSW_E_LAUNCH, "device %d is beyond the %d this library keeps %s for", dev, kMaxDevices, what);
    std::lock_guard<std::mutex> lock(g_symbol_mu);
    if (!cache[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, symbol);
        if (e != hipSuccess) return fail(HSW_E_LAUNCH, "hipGetSymbolAddress(%s): %s", what, hipGetErrorString(e));
        cache[dev] = p;
    }
    *out = cache[dev];
    return HSW_OK;
}

// ------------------------------------------------ the no-allocation call
// Scratch of hsw_full_decode_splitk_noalloc: its split-K partials, in module
// memory (nothing is allocated; each GPU the library runs on holds this
// array until the process ends).  Every call on a device shares the one
// array: calls that overlap on one GPU race.  The partial pass writes every
// slot the combine pass reads, so nothing has to start at zero.
static __device__ __align__(256) unsigned char scratch[HSW_NOALLOC_SCRATCH_BYTES];
void *g_scratch_ptr[kMaxDevices];

// ------------------------------------------------------------ device checks
#if HSW_CHECK_DEVICE
// Per device: [0] the code of a contract violation found (0: none), [1] the
// index of the element that broke it.  Module memory of the checked build:
// nothing is allocated.  Host code takes its address once per device with
// hipGetSymbolAddress and uses only that address.
__device__ __align__(16) unsigned long long g_dev_check[2];

__global__ __launch_bounds__(256) void check_kernel(dc::Inputs in, unsigned long long *flag) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < in.n; i += (int64_t)gridDim.x * 256) {
        const int32_t c = dc::check_element(in, i);
        if (c != 0 && atomicCAS(&flag[0], 0ull, (unsigned long long)c) == 0ull) flag[1] = (unsigned long long)i;
    }
}

void *g_flag_ptr[kMaxDevices];

// The current device's flag.
hsw_status device_flag(unsigned long long **out) {
    void *p = nullptr;
    hsw_status st = symbol_address(HIP_SYMBOL(g_dev_check), g_flag_ptr, &p, "the check flag");
    *out = static_cast<unsigned long long *>(p);
    return st;
}
#endif

// Checked builds: launch the check of a call's device-resident arguments on
// `s`, ahead of the call's kernels, and hand back the flag those kernels
// test.  Release builds: no launch, flag NULL.
hsw_status device_checks(const dc::Inputs &in, hipStream_t s, const unsigned long long **flag) {
    *flag = nullptr;
#if HSW_CHECK_DEVICE
    unsigned long long *f = nullptr;
    hsw_status st = device_flag(&f);
    if (st) return st;
    if (in.n > 0) {
        int64_t blocks = (in.n + 255) / 256;
        if (blocks > 1024) blocks = 1024;
        hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, f);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(HSW_E_LAUNCH, "device check: %s", hipGetErrorString(e));
    }
    *flag = f;
#else
    (void)in;
    (void)s;
#endif
    return HSW_OK;
}

dc::Inputs check_inputs(int32_t call, int64_t n) {
    dc::Inputs in;
    memset(&in, 0, sizeof in);
    in.call = call;
    in.n = n;
    return in;
}

bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

int elem_bytes(int32_t dtype) { return dtype == HSW_BF16 ? 2 : 4; }

// Shape checks shared by all calls.  want_window: 1 = windowed (> 0),
// 0 = full (== 0), -1 = either.
hsw_status check_shape(const hsw_attn_shape *sh, int want_window) {
    if (!sh) return fail(HSW_E_NULL, "shape pointer is NULL");
    if (sh->n_q_heads <= 0 || sh->n_kv_heads <= 0 || sh->n_q_heads % sh->n_kv_heads != 0)
        return fail(HSW_E_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                    sh->n_q_heads, sh->n_kv_heads);
    if (sh->d_qk < 8 || sh->d_qk > 256 || sh->d_qk % 8 != 0)
        return fail(HSW_E_SHAPE, "d_qk (%d) must be a multiple of 8 in [8, 256]", sh->d_qk);
    if (sh->d_v < 8 || sh->d_v > 256 || sh->d_v % 8 != 0)
        return fail(HSW_E_SHAPE, "d_v (%d) must be a multiple of 8 in [8, 256]", sh->d_v);
    if (sh->rope_dim < 0 || sh->rope_dim > sh->d_qk || sh->rope_dim % 16 != 0)
        return fail(HSW_E_SHAPE, "rope_dim (%d) must be a multiple of 16 in [0, d_qk]", sh->rope_dim);
    if (sh->window < 0) return fail(HSW_E_SHAPE, "window (%d) must be >= 0", sh->window);
    if (want_window == 1 && sh->window == 0)
        return fail(HSW_E_SHAPE, "a windowed call needs window > 0");
    if (want_window == 0 && sh->window != 0)
        return fail(HSW_E_SHAPE, "a full-attention call needs window == 0");
    if (sh->dtype != HSW_BF16 && sh->dtype != HSW_F32)
        return fail(HSW_E_DTYPE, "dtype %d is not HSW_BF16 or HSW_F32", sh->dtype);
    if (sh->out_dtype != HSW_BF16 && sh->out_dtype != HSW_F32)
        return fail(HSW_E_DTYPE, "out_dtype %d is not HSW_BF16 or HSW_F32", sh->out_dtype);
    if (!(sh->softmax_scale > 0.0f) || !isfinite(sh->softmax_scale) || !isfinite(sh->value_scale))
        return fail(HSW_E_SHAPE, "softmax_scale must be finite and > 0, value_scale finite");
    if (sh->rope_dim > 0 && !(sh->rope_theta > 0.0))
        return fail(HSW_E_SHAPE, "rope_theta must be > 0");
    return HSW_OK;
}

#define REQUIRE_PTR(p) \
    do { if (!(p)) return fail(HSW_E_NULL, "%s is NULL", #p); } while (0)
#define REQUIRE_ALIGN(p, n) \
    do { if ((p) && !aligned((p), (n))) return fail(HSW_E_ALIGN, "%s is not %d-byte aligned", #p, (int)(n)); } while (0)

hsw_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return HSW_OK;
}

// theta^(-2i/rope_dim) in double (colibri "What the engine implements"),
// computed once per call on the host and handed to the kernels.
double inv_freq(const hsw_attn_shape *sh, int i) {
    return pow(sh->rope_theta, -2.0 * (double)i / (double)sh->rope_dim);
}

hsw::AttnArgs base_args(const hsw_attn_shape *sh) {
    hsw::AttnArgs a;
    memset(&a, 0, sizeof a);
    a.hq = sh->n_q_heads;
    a.hkv = sh->n_kv_heads;
    a.dqk = sh->d_qk;
    a.dv = sh->d_v;
    a.window = sh->window;
    a.scale = sh->softmax_scale;
    a.value_scale = sh->value_scale;
    a.rope_dim = sh->rope_dim;
    for (int i = 0; i < sh->rope_dim / 2 && i < 32; ++i) a.inv_freq[i] = inv_freq(sh, i);
    return a;
}

}  // namespace

namespace {
// noalloc: ws / ws_bytes are ignored; the partials go to `scratch`.
hsw_status full_decode_impl(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx, const int64_t *ctx_len,
                            const int64_t *seq_base, const void *q, const void *k_pool, const void *v_pool,
                            int64_t pool_rows, const float *sinks, int32_t chunk, void *ws, size_t ws_bytes,
                            void *out, hipStream_t s, bool qrope, const char *what, bool noalloc = false) {
    hsw_status st = check_shape(sh, 0);
    if (st) return st;
    if (n_seqs < 0 || max_ctx < 0 || pool_rows < 0)
        return fail(HSW_E_SHAPE, "n_seqs, max_ctx and pool_rows must be >= 0");
    if (pool_rows > kMaxPoolRows) return fail(HSW_E_SHAPE, "pool_rows exceeds 2^31 - 1");
    if (chunk <= 0 || chunk % 128 != 0) return fail(HSW_E_SHAPE, "chunk (%d) must be a positive multiple of 128", chunk);
    if (!q) return fail(HSW_E_NULL, qrope ? "q is NULL" : "q_rot is NULL");
    REQUIRE_PTR(ctx_len); REQUIRE_PTR(seq_base); REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_pool, 16); REQUIRE_ALIGN(v_pool, 16);
    REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(ws, 16); REQUIRE_ALIGN(ctx_len, 8);
    REQUIRE_ALIGN(seq_base, 8); REQUIRE_ALIGN(sinks, 4);
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kFullDecode;
    a.qrope = qrope ? 1 : 0;
    a.chunk = chunk;
    if (qrope && !hsw::full_qrope_ok(a, sh->dtype, sh->out_dtype, false))
        return fail(HSW_E_SHAPE, "full_decode_splitk_qrope needs bf16 in and out, d_qk 192, d_v 128, rope_dim 64 "
                                 "and 1, 2, 4, 8 or 16 query heads per KV head");
    if (n_seqs == 0) return HSW_OK;
    size_t need = hsw_full_decode_workspace_bytes(sh, n_seqs, max_ctx, chunk);
    if (noalloc) {
        if (need > (size_t)HSW_NOALLOC_SCRATCH_BYTES)
            return fail(HSW_E_WORKSPACE, "the partials need %zu bytes; the no-allocation call holds %zu "
                                         "(use a larger chunk or fewer sequences per call)",
                        need, (size_t)HSW_NOALLOC_SCRATCH_BYTES);
        if (max_ctx == 0) return HSW_OK;
        if ((st = symbol_address(HIP_SYMBOL(scratch), g_scratch_ptr, &ws, "the scratch array"))) return st;
        ws_bytes = HSW_NOALLOC_SCRATCH_BYTES;
    }
    if (!ws || ws_bytes < need)
        return fail(HSW_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, need);
    if (max_ctx == 0) return HSW_OK;
    int64_t nc = (max_ctx + chunk - 1) / chunk;
    if ((int64_t)n_seqs * sh->n_kv_heads * nc > 0x7fffffffLL || (int64_t)n_seqs * sh->n_q_heads > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "grid too large");
    a.q = q; a.k_main = k_pool; a.v_main = v_pool; a.sinks = sinks; a.ctx_len = ctx_len;
    a.seq_base = seq_base; a.out = out; a.ws = ws; a.n_seqs = n_seqs; a.n_rows = n_seqs;
    a.max_seqlen = max_ctx; a.pool_rows = pool_rows; a.n_chunks = (int)nc;
    dc::Inputs ci = check_inputs(dc::kFullDecode, n_seqs);
    ci.ctx_len = ctx_len; ci.seq_base = seq_base; ci.max_ctx = max_ctx; ci.pool_rows = pool_rows;
    if ((st = device_checks(ci, s, &a.dev_flag))) return st;
    hipError_t e = (qrope || hsw::full_decode_fast_ok(a, sh->dtype, sh->out_dtype))
                       ? hsw::launch_full_decode(a, s)
                       : hsw::launch_generic_attn(a, sh->dtype, sh->out_dtype, s);
    return launched(e, what);
}

hsw_status full_prefill_impl(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                             const int64_t *cu_seqlens, const int64_t *start_pos, const int64_t *seq_base,
                             const void *q, const void *k_pool, const void *v_pool, int64_t pool_rows,
                             const float *sinks, void *out, hipStream_t s, bool qrope, const char *what) {
    hsw_status st = check_shape(sh, 0);
    if (st) return st;
    if (n_seqs < 0 || max_seqlen < 0 || pool_rows < 0)
        return fail(HSW_E_SHAPE, "n_seqs, max_seqlen and pool_rows must be >= 0");
    if (pool_rows > kMaxPoolRows) return fail(HSW_E_SHAPE, "pool_rows exceeds 2^31 - 1");
    if (!q) return fail(HSW_E_NULL, qrope ? "q is NULL" : "q_rot is NULL");
    REQUIRE_PTR(cu_seqlens); REQUIRE_PTR(start_pos); REQUIRE_PTR(seq_base);
    REQUIRE_PTR(k_pool); REQUIRE_PTR(v_pool); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_pool, 16); REQUIRE_ALIGN(v_pool, 16);
    REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(cu_seqlens, 8); REQUIRE_ALIGN(start_pos, 8);
    REQUIRE_ALIGN(seq_base, 8); REQUIRE_ALIGN(sinks, 4);
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kFullPrefill;
    a.qrope = qrope ? 1 : 0;
    if (qrope && !hsw::full_qrope_ok(a, sh->dtype, sh->out_dtype, true))
        return fail(HSW_E_SHAPE, "full_prefill_chunk_qrope needs bf16 in and out, d_qk 192, d_v 128, rope_dim 64 "
                                 "and 2, 4, 8 or 16 query heads per KV head");
    if (n_seqs == 0 || max_seqlen == 0) return HSW_OK;
    if ((int64_t)n_seqs * max_seqlen * sh->n_q_heads > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "n_seqs * max_seqlen * n_q_heads exceeds 2^31 - 1");
    a.q = q; a.k_main = k_pool; a.v_main = v_pool; a.sinks = sinks; a.cu_seqlens = cu_seqlens;
    a.start_pos = start_pos; a.seq_base = seq_base; a.out = out; a.n_seqs = n_seqs;
    a.max_seqlen = max_seqlen; a.n_rows = (int64_t)n_seqs * max_seqlen; a.pool_rows = pool_rows;
    dc::Inputs ci = check_inputs(dc::kFullPrefill, n_seqs);
    ci.cu_seqlens = cu_seqlens; ci.start_pos = start_pos; ci.seq_base = seq_base;
    ci.max_seqlen = max_seqlen; ci.pool_rows = pool_rows;
    if ((st = device_checks(ci, s, &a.dev_flag))) return st;
    hipError_t e = (qrope || hsw::full_prefill_fast_ok(a, sh->dtype, sh->out_dtype))
                       ? hsw::launch_full_prefill(a, s)
                       : hsw::launch_generic_attn(a, sh->dtype, sh->out_dtype, s);
    return launched(e, what);
}
}  // namespace

extern "C" {

const char *hsw_status_str(hsw_status s) {
    switch (s) {
        case HSW_OK: return "HSW_OK";
        case HSW_E_NULL: return "HSW_E_NULL: a required pointer is NULL";
        case HSW_E_SHAPE: return "HSW_E_SHAPE: inconsistent or unsupported sizes";
        case HSW_E_ALIGN: return "HSW_E_ALIGN: a tensor pointer is misaligned";
        case HSW_E_DTYPE: return "HSW_E_DTYPE: unsupported dtype";
        case HSW_E_WORKSPACE: return "HSW_E_WORKSPACE: workspace too small";
        case HSW_E_LAUNCH: return "HSW_E_LAUNCH: kernel launch failed";
        case HSW_E_CAPACITY: return "HSW_E_CAPACITY: a KV pool lacks room";
        case HSW_E_STALE: return "HSW_E_STALE: the snapshot was released";
        case HSW_E_DEVICE_INPUT: return "HSW_E_DEVICE_INPUT: a device-resident argument broke the contract";
        default: return "unknown hsw_status";
    }
}

const char *hsw_last_error(void) { return g_err; }

const char *hsw_version(void) { return HSW_CHECK_DEVICE ? "hsw 0.2 gfx950 checked" : "hsw 0.2 gfx950"; }

int32_t hsw_device_checks_enabled(void) { return HSW_CHECK_DEVICE ? 1 : 0; }

hsw_status hsw_device_check_status(hsw_stream_t stream, int32_t *code, int64_t *index) {
    if (code) *code = -1;
    if (index) *index = -1;
#if HSW_CHECK_DEVICE
    unsigned long long *f = nullptr;
    hsw_status st = device_flag(&f);
    if (st) return st;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "hipStreamSynchronize: %s", hipGetErrorString(e));
    unsigned long long h[2] = {0, 0};
    e = hipMemcpy(h, f, sizeof h, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "reading the check flag: %s", hipGetErrorString(e));
    if (code) *code = (int32_t)h[0];
    if (index) *index = h[0] ? (int64_t)h[1] : -1;
    if (h[0] == 0) return HSW_OK;
    const unsigned long long zero[2] = {0, 0};
    e = hipMemcpy(f, zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "clearing the check flag: %s", hipGetErrorString(e));
    return fail(HSW_E_DEVICE_INPUT, "device check code %d at element %lld", (int)h[0], (long long)h[1]);
#else
    (void)stream;
    return HSW_OK;
#endif
}

hsw_status hsw_rope_partial_kv_write(const hsw_attn_shape *sh, int64_t n_tokens, const void *q,
                                     const void *k, const void *v, const int64_t *pos,
                                     const int32_t *seq, int32_t dst_kind, void *k_dst, void *v_dst,
                                     int64_t dst_capacity, const int64_t *seq_base, void *q_rot,
                                     int64_t *dst_index_out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, -1);
    if (st) return st;
    if (n_tokens < 0) return fail(HSW_E_SHAPE, "n_tokens (%lld) < 0", (long long)n_tokens);
    if (dst_kind != HSW_DST_RING && dst_kind != HSW_DST_POOL && dst_kind != HSW_DST_STAGING)
        return fail(HSW_E_SHAPE, "dst_kind %d is not RING, POOL or STAGING", dst_kind);
    if (dst_kind == HSW_DST_RING && sh->window <= 0)
        return fail(HSW_E_SHAPE, "a ring destination needs window > 0");
    if (dst_capacity < 0) return fail(HSW_E_SHAPE, "dst_capacity < 0");
    if (sh->rope_dim / 2 > 128) return fail(HSW_E_SHAPE, "rope_dim > 256 is not supported");
    if (n_tokens > 0x7fffffffLL) return fail(HSW_E_SHAPE, "n_tokens exceeds 2^31 - 1");
    // q and q_rot both NULL: write K/V only (for the calls that rotate q
    // themselves); one without the other is an error.
    if (!q != !q_rot) return fail(HSW_E_NULL, "%s is NULL (q and q_rot must both be given, or both NULL)",
                                  q ? "q_rot" : "q");
    // v and v_dst both NULL (staging only): K alone is written; the windowed
    // prefill then reads V from v itself, whose layout is the staging one.
    if (dst_kind == HSW_DST_STAGING && !v && !v_dst) {
    } else {
        REQUIRE_PTR(v); REQUIRE_PTR(v_dst);
    }
    REQUIRE_PTR(k); REQUIRE_PTR(pos);
    REQUIRE_PTR(k_dst);
    if (dst_kind != HSW_DST_STAGING) REQUIRE_PTR(seq);
    if (dst_kind == HSW_DST_POOL) REQUIRE_PTR(seq_base);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(k_dst, 16);
    REQUIRE_ALIGN(v_dst, 16); REQUIRE_ALIGN(q_rot, 16); REQUIRE_ALIGN(pos, 8);
    REQUIRE_ALIGN(seq, 4); REQUIRE_ALIGN(seq_base, 8); REQUIRE_ALIGN(dst_index_out, 8);
    if (n_tokens == 0) return HSW_OK;
    hsw::RopeArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.pos = pos; a.seq = seq; a.seq_base = seq_base;
    a.k_dst = k_dst; a.v_dst = v_dst; a.q_rot = q_rot; a.dst_index_out = dst_index_out;
    a.n_tokens = n_tokens; a.dst_capacity = dst_capacity;
    for (int i = 0; i < sh->rope_dim / 2; ++i) a.inv_freq[i] = inv_freq(sh, i);
    a.hq = sh->n_q_heads; a.hkv = sh->n_kv_heads; a.dqk = sh->d_qk; a.dv = sh->d_v;
    a.rope_dim = sh->rope_dim; a.window = sh->window; a.dst_kind = dst_kind;
    dc::Inputs ci = check_inputs(dc::kRope, n_tokens);
    ci.dst_kind = dst_kind; ci.pos = pos; ci.seq = seq; ci.seq_base = seq_base; ci.dst_capacity = dst_capacity;
    if ((st = device_checks(ci, (hipStream_t)stream, &a.dev_flag))) return st;
    return launched(hsw::launch_rope(a, sh->dtype, (hipStream_t)stream), "rope_partial_kv_write");
}

hsw_status hsw_swa_prefill(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                           const int64_t *cu_seqlens, const int64_t *start_pos, const void *q_rot,
                           const void *k_stage, const void *v_stage, void *k_ring, void *v_ring,
                           const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, 1);
    if (st) return st;
    if (n_seqs < 0 || max_seqlen < 0) return fail(HSW_E_SHAPE, "n_seqs and max_seqlen must be >= 0");
    if ((int64_t)n_seqs * max_seqlen * sh->n_q_heads > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "n_seqs * max_seqlen * n_q_heads exceeds 2^31 - 1");
    REQUIRE_PTR(cu_seqlens); REQUIRE_PTR(start_pos); REQUIRE_PTR(q_rot); REQUIRE_PTR(k_stage);
    REQUIRE_PTR(v_stage); REQUIRE_PTR(k_ring); REQUIRE_PTR(v_ring); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q_rot, 16); REQUIRE_ALIGN(k_stage, 16); REQUIRE_ALIGN(v_stage, 16);
    REQUIRE_ALIGN(k_ring, 16); REQUIRE_ALIGN(v_ring, 16); REQUIRE_ALIGN(out, 16);
    REQUIRE_ALIGN(cu_seqlens, 8); REQUIRE_ALIGN(start_pos, 8); REQUIRE_ALIGN(sinks, 4);
    if (n_seqs == 0 || max_seqlen == 0) return HSW_OK;
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kSwaPrefill;
    a.q = q_rot; a.k_main = k_stage; a.v_main = v_stage; a.k_ring = k_ring; a.v_ring = v_ring;
    a.sinks = sinks; a.cu_seqlens = cu_seqlens; a.start_pos = start_pos; a.out = out;
    a.n_seqs = n_seqs; a.max_seqlen = max_seqlen; a.n_rows = (int64_t)n_seqs * max_seqlen;
    hipStream_t s = (hipStream_t)stream;
    dc::Inputs ci = check_inputs(dc::kSwaPrefill, n_seqs);
    ci.cu_seqlens = cu_seqlens; ci.start_pos = start_pos; ci.max_seqlen = max_seqlen;
    if ((st = device_checks(ci, s, &a.dev_flag))) return st;
    hipError_t e = hsw::swa_prefill_fast_ok(a, sh->dtype, sh->out_dtype)
                       ? hsw::launch_swa_prefill(a, s)
                       : hsw::launch_generic_attn(a, sh->dtype, sh->out_dtype, s);
    if ((st = launched(e, "swa_prefill"))) return st;
    // The ring commit overwrites slots the attention above read, so it is a
    // second launch, ordered after it on the same stream.
    return launched(hsw::launch_ring_commit(a, sh->dtype, s), "swa_prefill ring commit");
}

hsw_status hsw_swa_decode(const hsw_attn_shape *sh, int32_t n_seqs, const int64_t *pos,
                          const void *q_rot, const void *k_ring, const void *v_ring,
                          const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, 1);
    if (st) return st;
    if (n_seqs < 0) return fail(HSW_E_SHAPE, "n_seqs < 0");
    if ((int64_t)n_seqs * sh->n_q_heads > 0x7fffffffLL) return fail(HSW_E_SHAPE, "n_seqs * n_q_heads exceeds 2^31 - 1");
    REQUIRE_PTR(pos); REQUIRE_PTR(q_rot); REQUIRE_PTR(k_ring); REQUIRE_PTR(v_ring); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q_rot, 16); REQUIRE_ALIGN(k_ring, 16); REQUIRE_ALIGN(v_ring, 16);
    REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(pos, 8); REQUIRE_ALIGN(sinks, 4);
    if (n_seqs == 0) return HSW_OK;
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kSwaDecode;
    a.q = q_rot; a.k_main = k_ring; a.v_main = v_ring; a.sinks = sinks; a.pos = pos; a.out = out;
    a.n_seqs = n_seqs; a.n_rows = n_seqs;
    hipStream_t s = (hipStream_t)stream;
    dc::Inputs ci = check_inputs(dc::kSwaDecode, n_seqs);
    ci.pos = pos;
    if ((st = device_checks(ci, s, &a.dev_flag))) return st;
    hipError_t e = hsw::swa_decode_fast_ok(a, sh->dtype, sh->out_dtype)
                       ? hsw::launch_swa_decode(a, s)
                       : hsw::launch_generic_attn(a, sh->dtype, sh->out_dtype, s);
    return launched(e, "swa_decode");
}

hsw_status hsw_swa_prefill_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                 const int64_t *cu_seqlens, const int64_t *start_pos, const void *q,
                                 const void *k_stage, const void *v_stage, void *k_ring, void *v_ring,
                                 const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, 1);
    if (st) return st;
    if (n_seqs < 0 || max_seqlen < 0) return fail(HSW_E_SHAPE, "n_seqs and max_seqlen must be >= 0");
    if ((int64_t)n_seqs * max_seqlen * sh->n_q_heads > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "n_seqs * max_seqlen * n_q_heads exceeds 2^31 - 1");
    REQUIRE_PTR(cu_seqlens); REQUIRE_PTR(start_pos); REQUIRE_PTR(q); REQUIRE_PTR(k_stage);
    REQUIRE_PTR(v_stage); REQUIRE_PTR(k_ring); REQUIRE_PTR(v_ring); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_stage, 16); REQUIRE_ALIGN(v_stage, 16);
    REQUIRE_ALIGN(k_ring, 16); REQUIRE_ALIGN(v_ring, 16); REQUIRE_ALIGN(out, 16);
    REQUIRE_ALIGN(cu_seqlens, 8); REQUIRE_ALIGN(start_pos, 8); REQUIRE_ALIGN(sinks, 4);
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kSwaPrefill;
    a.qrope = 1;
    if (!hsw::swa_qrope_ok(a, sh->dtype, sh->out_dtype, true))
        return fail(HSW_E_SHAPE, "swa_prefill_qrope needs bf16 in and out, d_qk 192, d_v 128, rope_dim 64, "
                                 "window 128 and 2, 4, 8 or 16 query heads per KV head");
    if (n_seqs == 0 || max_seqlen == 0) return HSW_OK;
    a.q = q; a.k_main = k_stage; a.v_main = v_stage; a.k_ring = k_ring; a.v_ring = v_ring;
    a.sinks = sinks; a.cu_seqlens = cu_seqlens; a.start_pos = start_pos; a.out = out;
    a.n_seqs = n_seqs; a.max_seqlen = max_seqlen; a.n_rows = (int64_t)n_seqs * max_seqlen;
    hipStream_t s = (hipStream_t)stream;
    dc::Inputs ci = check_inputs(dc::kSwaPrefill, n_seqs);
    ci.cu_seqlens = cu_seqlens; ci.start_pos = start_pos; ci.max_seqlen = max_seqlen;
    if ((st = device_checks(ci, s, &a.dev_flag))) return st;
    if ((st = launched(hsw::launch_swa_prefill(a, s), "swa_prefill_qrope"))) return st;
    return launched(hsw::launch_ring_commit(a, sh->dtype, s), "swa_prefill_qrope ring commit");
}

hsw_status hsw_swa_decode_qrope(const hsw_attn_shape *sh, int32_t n_seqs, const int64_t *pos,
                                const void *q, const void *k_ring, const void *v_ring,
                                const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, 1);
    if (st) return st;
    if (n_seqs < 0) return fail(HSW_E_SHAPE, "n_seqs < 0");
    if ((int64_t)n_seqs * sh->n_q_heads > 0x7fffffffLL) return fail(HSW_E_SHAPE, "n_seqs * n_q_heads exceeds 2^31 - 1");
    REQUIRE_PTR(pos); REQUIRE_PTR(q); REQUIRE_PTR(k_ring); REQUIRE_PTR(v_ring); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_ring, 16); REQUIRE_ALIGN(v_ring, 16);
    REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(pos, 8); REQUIRE_ALIGN(sinks, 4);
    hsw::AttnArgs a = base_args(sh);
    a.kind = hsw::kSwaDecode;
    a.qrope = 1;
    if (!hsw::swa_qrope_ok(a, sh->dtype, sh->out_dtype, false))
        return fail(HSW_E_SHAPE, "swa_decode_qrope needs bf16 in and out, d_qk 192, d_v 128, rope_dim 64, "
                                 "window 128, n_q_heads <= 256 and 1, 2, 4, 8 or 16 query heads per KV head");
    if (n_seqs == 0) return HSW_OK;
    a.q = q; a.k_main = k_ring; a.v_main = v_ring; a.sinks = sinks; a.pos = pos; a.out = out;
    a.n_seqs = n_seqs; a.n_rows = n_seqs;
    dc::Inputs ci = check_inputs(dc::kSwaDecode, n_seqs);
    ci.pos = pos;
    if ((st = device_checks(ci, (hipStream_t)stream, &a.dev_flag))) return st;
    return launched(hsw::launch_swa_decode(a, (hipStream_t)stream), "swa_decode_qrope");
}

size_t hsw_full_decode_workspace_bytes(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                       int32_t chunk) {
    if (!sh || n_seqs < 0 || max_ctx < 0 || chunk <= 0) return 0;
    int64_t nc = (max_ctx + chunk - 1) / chunk;
    return hsw::full_decode_ws_bytes(n_seqs, sh->n_q_heads, nc, sh->d_v);
}


hsw_status hsw_full_decode_splitk(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                  const int64_t *ctx_len, const int64_t *seq_base,
                                  const void *q_rot, const void *k_pool, const void *v_pool,
                                  int64_t pool_rows, const float *sinks, int32_t chunk, void *ws,
                                  size_t ws_bytes, void *out, hsw_stream_t stream) {
    return full_decode_impl(sh, n_seqs, max_ctx, ctx_len, seq_base, q_rot, k_pool, v_pool, pool_rows, sinks, chunk,
                            ws, ws_bytes, out, (hipStream_t)stream, false, "full_decode_splitk");
}

hsw_status hsw_full_decode_splitk_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                        const int64_t *ctx_len, const int64_t *seq_base, const void *q,
                                        const void *k_pool, const void *v_pool, int64_t pool_rows,
                                        const float *sinks, int32_t chunk, void *ws, size_t ws_bytes, void *out,
                                        hsw_stream_t stream) {
    return full_decode_impl(sh, n_seqs, max_ctx, ctx_len, seq_base, q, k_pool, v_pool, pool_rows, sinks, chunk,
                            ws, ws_bytes, out, (hipStream_t)stream, true, "full_decode_splitk_qrope");
}

hsw_status hsw_full_decode_splitk_noalloc(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_ctx,
                                          const int64_t *ctx_len, const int64_t *seq_base, const void *q_rot,
                                          const void *k_pool, const void *v_pool, int64_t pool_rows,
                                          const float *sinks, int32_t chunk, void *out, hsw_stream_t stream) {
    return full_decode_impl(sh, n_seqs, max_ctx, ctx_len, seq_base, q_rot, k_pool, v_pool, pool_rows, sinks, chunk,
                            nullptr, 0, out, (hipStream_t)stream, false, "full_decode_splitk_noalloc", true);
}

hsw_status hsw_full_prefill_chunk(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                  const int64_t *cu_seqlens, const int64_t *start_pos,
                                  const int64_t *seq_base, const void *q_rot, const void *k_pool,
                                  const void *v_pool, int64_t pool_rows, const float *sinks,
                                  void *out, hsw_stream_t stream) {
    return full_prefill_impl(sh, n_seqs, max_seqlen, cu_seqlens, start_pos, seq_base, q_rot, k_pool, v_pool,
                             pool_rows, sinks, out, (hipStream_t)stream, false, "full_prefill_chunk");
}

hsw_status hsw_full_prefill_chunk_qrope(const hsw_attn_shape *sh, int32_t n_seqs, int64_t max_seqlen,
                                        const int64_t *cu_seqlens, const int64_t *start_pos,
                                        const int64_t *seq_base, const void *q, const void *k_pool,
                                        const void *v_pool, int64_t pool_rows, const float *sinks, void *out,
                                        hsw_stream_t stream) {
    return full_prefill_impl(sh, n_seqs, max_seqlen, cu_seqlens, start_pos, seq_base, q, k_pool, v_pool,
                             pool_rows, sinks, out, (hipStream_t)stream, true, "full_prefill_chunk_qrope");
}

int64_t hsw_kv_bytes(int32_t kind, int64_t n_seqs, int64_t ctx, int32_t window, int32_t n_kv_heads,
                     int32_t d_qk, int32_t d_v_stored, int32_t elem_bytes, int32_t n_layers) {
    if (n_seqs < 0 || ctx < 0 || n_kv_heads < 0 || d_qk < 0 || d_v_stored < 0 || elem_bytes <= 0 ||
        n_layers < 0)
        return -1;
    int64_t positions;
    if (kind == HSW_DST_RING) {
        if (window <= 0) return -1;
        positions = window;
    } else if (kind == HSW_DST_POOL) {
        positions = ctx;
    } else {
        return -1;
    }
    return (int64_t)n_layers * n_seqs * positions * n_kv_heads * (int64_t)(d_qk + d_v_stored) * elem_bytes;
}

// ------------------------------------------------------------------ vision
hsw_status hsw_vit_layout(int32_t h, int32_t w, int32_t *row, int32_t *col, int32_t *col_order) {
    if (h <= 0 || w <= 0 || h % 2 || w % 2 || (int64_t)h * w > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "h (%d) and w (%d) must be positive and even, h * w < 2^31", h, w);
    const int uh = h / 2, uw = w / 2;
    const int n = h * w;
    for (int t = 0; t < n; ++t) {
        const int u = t >> 2, e = t & 3;
        if (row) row[t] = 2 * (u / uw) + (e >> 1);
        if (col) col[t] = 2 * (u % uw) + (e & 1);
        if (col_order) {
            const int uc = t >> 2;  // position t of the column order: unit uc taken column by column
            col_order[t] = 4 * ((uc % uh) * uw + uc / uh) + e;
        }
    }
    return HSW_OK;
}

hsw_status hsw_vit_rope_2d(const hsw_attn_shape *sh, int64_t n_tokens, const void *q, const void *k,
                           const int32_t *row, const int32_t *col, void *q_out, void *k_out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, -1);
    if (st) return st;
    if (sh->dtype != HSW_BF16) return fail(HSW_E_DTYPE, "vit_rope_2d takes bf16 q and k");
    if (sh->d_qk % 32 != 0 || sh->d_qk > 128 || sh->rope_dim != sh->d_qk)
        return fail(HSW_E_SHAPE, "vit_rope_2d rotates whole heads: d_qk (%d) a multiple of 32, <= 128, "
                                 "rope_dim == d_qk (is %d)", sh->d_qk, sh->rope_dim);
    if (n_tokens < 0) return fail(HSW_E_SHAPE, "n_tokens must be >= 0");
    if (!q != !q_out) return fail(HSW_E_NULL, "q and q_out must both be given or both be NULL");
    if (!k != !k_out) return fail(HSW_E_NULL, "k and k_out must both be given or both be NULL");
    if (!q && !k) return fail(HSW_E_NULL, "neither q nor k is given");
    REQUIRE_PTR(row); REQUIRE_PTR(col);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(q_out, 16); REQUIRE_ALIGN(k_out, 16);
    REQUIRE_ALIGN(row, 4); REQUIRE_ALIGN(col, 4);
    if (n_tokens == 0) return HSW_OK;
    const int64_t per_tok = (int64_t)((q ? sh->n_q_heads : 0) + (k ? sh->n_kv_heads : 0)) * (sh->d_qk / 16);
    if (n_tokens * per_tok / 256 + 1 > 0x7fffffffLL) return fail(HSW_E_SHAPE, "grid too large");
    hsw::VitRopeArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.q_out = q_out; a.k_out = k_out; a.row = row; a.col = col;
    a.n_tokens = n_tokens; a.hq = sh->n_q_heads; a.hkv = sh->n_kv_heads; a.d = sh->d_qk;
    const int quarter = sh->d_qk / 4;
    for (int j = 0; j < quarter; ++j) a.inv_freq[j] = pow(sh->rope_theta, -(double)j / (double)quarter);
    return launched(hsw::launch_vit_rope(a, (hipStream_t)stream), "vit_rope_2d");
}

hsw_status hsw_vit_attention(const hsw_attn_shape *sh, int32_t n_images, int64_t max_len,
                             const int64_t *cu_seqlens, const int32_t *order, int32_t sink_key, const void *q,
                             const void *k, const void *v, const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, -1);
    if (st) return st;
    hsw::VitArgs a;
    memset(&a, 0, sizeof a);
    a.hq = sh->n_q_heads; a.hkv = sh->n_kv_heads; a.window = sh->window; a.sink_key = sink_key ? 1 : 0;
    a.scale = sh->softmax_scale;
    if (!hsw::vit_attn_ok(a, sh->d_qk, sh->d_v, sh->dtype, sh->out_dtype))
        return fail(HSW_E_SHAPE, "vit_attention needs bf16 in and out, d_qk = d_v = 64, window 0 or 64 and "
                                 "1, 2, 4, 8 or 16 query heads per KV head");
    if (sh->value_scale != 1.0f) return fail(HSW_E_SHAPE, "vit_attention has no value scale (must be 1)");
    if (n_images < 0 || max_len < 0) return fail(HSW_E_SHAPE, "n_images and max_len must be >= 0");
    if (max_len > 0x7fffffffLL) return fail(HSW_E_SHAPE, "max_len exceeds 2^31 - 1");
    REQUIRE_PTR(cu_seqlens); REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(out, 16);
    REQUIRE_ALIGN(cu_seqlens, 8); REQUIRE_ALIGN(order, 4); REQUIRE_ALIGN(sinks, 4);
    if (n_images == 0 || max_len == 0) return HSW_OK;
    const int BQ = hsw::vit_block_tokens(sh->n_q_heads / sh->n_kv_heads);
    if ((int64_t)n_images * sh->n_kv_heads * ((max_len + BQ - 1) / BQ) > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "grid too large");
    a.q = q; a.k = k; a.v = v; a.out = out; a.cu_seqlens = cu_seqlens; a.order = order; a.sinks = sinks;
    a.n_images = n_images;
    dc::Inputs ci = check_inputs(dc::kVit, n_images);
    ci.cu_seqlens = cu_seqlens; ci.order = order; ci.max_seqlen = max_len;
    if ((st = device_checks(ci, (hipStream_t)stream, &a.dev_flag))) return st;
    return launched(hsw::launch_vit_attn(a, max_len, (hipStream_t)stream), "vit_attention");
}

hsw_status hsw_vit_window_attention_rope(const hsw_attn_shape *sh, int32_t n_images, int64_t max_len,
                                         const int64_t *cu_seqlens, const int32_t *order, int32_t sink_key,
                                         const int32_t *row, const int32_t *col, const void *q, const void *k,
                                         const void *v, const float *sinks, void *out, hsw_stream_t stream) {
    hsw_status st = check_shape(sh, -1);
    if (st) return st;
    hsw::VitArgs a;
    memset(&a, 0, sizeof a);
    a.hq = sh->n_q_heads; a.hkv = sh->n_kv_heads; a.window = sh->window; a.sink_key = sink_key ? 1 : 0;
    a.scale = sh->softmax_scale;
    if (sh->window != 64 || !hsw::vit_attn_ok(a, sh->d_qk, sh->d_v, sh->dtype, sh->out_dtype) ||
        sh->rope_dim != sh->d_qk)
        return fail(HSW_E_SHAPE, "vit_window_attention_rope needs window 64, bf16 in and out, d_qk = d_v = "
                                 "rope_dim = 64 and 1, 2, 4, 8 or 16 query heads per KV head");
    if (sh->value_scale != 1.0f) return fail(HSW_E_SHAPE, "vit_window_attention_rope has no value scale (must be 1)");
    if (n_images < 0 || max_len < 0) return fail(HSW_E_SHAPE, "n_images and max_len must be >= 0");
    if (max_len > 0x7fffffffLL) return fail(HSW_E_SHAPE, "max_len exceeds 2^31 - 1");
    REQUIRE_PTR(cu_seqlens); REQUIRE_PTR(row); REQUIRE_PTR(col); REQUIRE_PTR(q); REQUIRE_PTR(k);
    REQUIRE_PTR(v); REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(out, 16);
    REQUIRE_ALIGN(cu_seqlens, 8); REQUIRE_ALIGN(order, 4); REQUIRE_ALIGN(sinks, 4);
    REQUIRE_ALIGN(row, 4); REQUIRE_ALIGN(col, 4);
    if (n_images == 0 || max_len == 0) return HSW_OK;
    const int BQ = hsw::vit_block_tokens(sh->n_q_heads / sh->n_kv_heads);
    if ((int64_t)n_images * sh->n_kv_heads * ((max_len + BQ - 1) / BQ) > 0x7fffffffLL)
        return fail(HSW_E_SHAPE, "grid too large");
    a.q = q; a.k = k; a.v = v; a.out = out; a.cu_seqlens = cu_seqlens; a.order = order; a.sinks = sinks;
    a.n_images = n_images;
    a.rope = 1; a.row = row; a.col = col;
    const int quarter = sh->d_qk / 4;   // the frequencies of hsw_vit_rope_2d
    for (int j = 0; j < quarter; ++j) a.rope_f[j] = pow(sh->rope_theta, -(double)j / (double)quarter);
    dc::Inputs ci = check_inputs(dc::kVit, n_images);
    ci.cu_seqlens = cu_seqlens; ci.order = order; ci.max_seqlen = max_len;
    if ((st = device_checks(ci, (hipStream_t)stream, &a.dev_flag))) return st;
    return launched(hsw::launch_vit_attn(a, max_len, (hipStream_t)stream), "vit_window_attention_rope");
}

}  // extern "C"
