// kv_manager.hip -- the dual-pool KV manager: host bookkeeping over the
// caller's device pools, and the kernel that copies a sequence's rings of
// every windowed layer into a snapshot and back.
//
// gokawiil "Full-Pipeline Inference Optimization for MiMo-V2.5 Series",
// section 2.1 "SWA KVCache Management": separate full and windowed pools, a
// request admitted only when both have room, prefix reuse clipped to the
// window-safe length.  colibri "MiMo-V2.6 (Xiaomi)", section "System One mode
// and prompt reuse": a snapshot leaves the full layers' rows in place
// (recording the token ids they hold, released when the sequence diverges
// below its position), copies every windowed layer's ring into the snapshot
// and back, and records its position.
//
// Pool rows are handed out as contiguous runs (first fit over an address-
// ordered free list, neighbours merged on release), since the attention calls
// address a sequence's rows as seq_base + position.
#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "../../include/hsw.h"
#include "hsw_device.h"
#include "hsw_launch.h"

namespace hsw {
namespace {

constexpr int kCopyThreads = 256;

// Grid-stride copy of 16-byte units: unit u of layer l is byte 16 r of the
// layer's K block (r < kb / 16) or of its V block; the snapshot holds per
// layer the K block then the V block.
__global__ __launch_bounds__(kCopyThreads) void ring_copy_kernel(RingCopyArgs a) {
    const int64_t uk = a.kb / 16, per_layer = (a.kb + a.vb) / 16;
    const int64_t total = per_layer * a.n_layers;
    for (int64_t u = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * kCopyThreads) {
        const int l = (int)(u / per_layer);
        const int64_t r = u - (int64_t)l * per_layer;
        char *ring = r < uk ? a.k[l] + 16 * r : a.v[l] + 16 * (r - uk);
        char *snap = a.snap + 16 * u;
        if (a.to_snap)
            st16(snap, ld16(ring));
        else
            st16(ring, ld16(snap));
    }
}

}  // namespace

hipError_t launch_ring_copy(const RingCopyArgs &a, hipStream_t s) {
    const int64_t units = (a.kb + a.vb) / 16 * a.n_layers;
    int64_t blocks = (units + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(ring_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hsw

struct hsw_kvm {
    struct Seq {
        bool used = false;
        int64_t base = 0, max_len = 0, len = 0;
        std::vector<int32_t> tok;       // token id each row holds (rows 0 .. tok.size()-1 written)
        std::vector<int64_t> slot_pos;  // position each ring slot holds (-1: none yet)
    };
    struct Snap {
        int32_t seq;
        int64_t pos;
        int32_t slot;
        std::vector<int64_t> slot_pos;  // what the copied rings held
    };
    hsw_kvm_config cfg;
    std::vector<char *> k, v;
    char *snap_buf = nullptr;
    size_t snap_bytes = 0;
    std::vector<Seq> seqs;
    std::map<int64_t, int64_t> free_rows;   // start -> length, address order
    std::map<int32_t, Snap> snaps;          // live snapshots by id
    std::vector<bool> slot_used;
    int32_t next_snap_id = 0;
};

namespace {

using hsw::fail;

size_t snapshot_bytes(const hsw_kvm_config &c) {
    return (size_t)c.n_swa_layers * c.swa_kv_heads * c.window * (size_t)(c.d_qk + c.d_v) * c.elem_bytes;
}

bool config_ok(const hsw_kvm_config *c) {
    return c && c->n_swa_layers >= 1 && c->n_swa_layers <= hsw::kMaxRingLayers && c->swa_kv_heads >= 1 &&
           c->window >= 1 && c->d_qk >= 8 && c->d_qk % 8 == 0 && c->d_v >= 8 && c->d_v % 8 == 0 &&
           (c->elem_bytes == 2 || c->elem_bytes == 4) && c->ring_seqs >= 1 && c->pool_rows >= 0 &&
           c->max_snapshots >= 0;
}

hsw_status check_seq(hsw_kvm *kvm, int32_t seq) {
    if (!kvm) return fail(HSW_E_NULL, "kvm is NULL");
    if (seq < 0 || seq >= (int32_t)kvm->seqs.size() || !kvm->seqs[seq].used)
        return fail(HSW_E_SHAPE, "sequence %d is not admitted", seq);
    return HSW_OK;
}

// The largest length L <= lim whose window the rings hold: the token at L
// reads positions max(0, L - W + 1) .. L - 1 from the ring (colibri "System
// One mode and prompt reuse": position p in slot p mod W).  The positions the
// slots hold form runs of consecutive values; a run [a, b] serves L iff
// L - 1 <= b and it reaches down to the window's first position: a == 0, or
// a <= L - W + 1.  L = 0 needs nothing, and neither does any L when W = 1
// (the token then attends to itself only).
int64_t longest_held_window(const std::vector<int64_t> &slot_pos, int64_t lim) {
    const int64_t W = (int64_t)slot_pos.size();
    if (W == 1) return lim > 0 ? lim : 0;
    std::vector<int64_t> held;
    held.reserve(slot_pos.size());
    for (int64_t p : slot_pos)
        if (p >= 0) held.push_back(p);
    std::sort(held.begin(), held.end());
    int64_t best = 0;
    for (size_t i = 0; i < held.size();) {
        size_t j = i;
        while (j + 1 < held.size() && held[j + 1] == held[j] + 1) ++j;
        const int64_t a = held[i], b = held[j];
        const int64_t lo = a == 0 ? 1 : a + W - 1, hi = b + 1 < lim ? b + 1 : lim;
        if (hi >= lo && hi > best) best = hi;
        i = j + 1;
    }
    return best;
}

void drop_snaps_above(hsw_kvm *kvm, int32_t seq, int64_t pos) {
    for (auto it = kvm->snaps.begin(); it != kvm->snaps.end();) {
        if (it->second.seq == seq && it->second.pos > pos) {
            kvm->slot_used[it->second.slot] = false;
            it = kvm->snaps.erase(it);
        } else {
            ++it;
        }
    }
}

hsw_status copy_rings(hsw_kvm *kvm, int32_t seq, int32_t slot, bool to_snap, hipStream_t s) {
    const hsw_kvm_config &c = kvm->cfg;
    hsw::RingCopyArgs a;
    a.kb = (int64_t)c.swa_kv_heads * c.window * c.d_qk * c.elem_bytes;
    a.vb = (int64_t)c.swa_kv_heads * c.window * c.d_v * c.elem_bytes;
    for (int l = 0; l < c.n_swa_layers; ++l) {
        a.k[l] = kvm->k[l] + (int64_t)seq * a.kb;
        a.v[l] = kvm->v[l] + (int64_t)seq * a.vb;
    }
    a.snap = kvm->snap_buf + (size_t)slot * kvm->snap_bytes;
    a.n_layers = c.n_swa_layers;
    a.to_snap = to_snap ? 1 : 0;
    hipError_t e = hsw::launch_ring_copy(a, s);
    if (e != hipSuccess) return fail(HSW_E_LAUNCH, "ring copy: %s", hipGetErrorString(e));
    return HSW_OK;
}

}  // namespace

extern "C" {

size_t hsw_kvm_snapshot_bytes(const hsw_kvm_config *cfg) {
    return config_ok(cfg) ? snapshot_bytes(*cfg) : 0;
}

hsw_status hsw_kvm_create(const hsw_kvm_config *cfg, void *const *swa_k, void *const *swa_v, void *snap_buf,
                          size_t snap_buf_bytes, hsw_kvm **out) {
    if (!cfg || !swa_k || !swa_v || !out) return fail(HSW_E_NULL, "cfg, swa_k, swa_v and out must be non-NULL");
    *out = nullptr;
    if (!config_ok(cfg))
        return fail(HSW_E_SHAPE, "kvm config: 1..128 windowed layers, heads/window/ring_seqs >= 1, d_qk and d_v "
                                 "multiples of 8, elem_bytes 2 or 4, pool_rows and max_snapshots >= 0");
    for (int l = 0; l < cfg->n_swa_layers; ++l) {
        if (!swa_k[l] || !swa_v[l]) return fail(HSW_E_NULL, "ring pointer of layer %d is NULL", l);
        if ((uintptr_t)swa_k[l] % 16 || (uintptr_t)swa_v[l] % 16)
            return fail(HSW_E_ALIGN, "ring pointer of layer %d is not 16-byte aligned", l);
    }
    const size_t sb = snapshot_bytes(*cfg);
    if (cfg->max_snapshots > 0) {
        if (!snap_buf) return fail(HSW_E_NULL, "snap_buf is NULL with max_snapshots > 0");
        if ((uintptr_t)snap_buf % 16) return fail(HSW_E_ALIGN, "snap_buf is not 16-byte aligned");
        if (snap_buf_bytes < sb * (size_t)cfg->max_snapshots)
            return fail(HSW_E_WORKSPACE, "snap_buf holds %zu bytes, %d snapshots need %zu", snap_buf_bytes,
                        cfg->max_snapshots, sb * (size_t)cfg->max_snapshots);
    }
    hsw_kvm *kvm = new (std::nothrow) hsw_kvm;
    if (!kvm) return fail(HSW_E_CAPACITY, "out of host memory");
    try {
        kvm->cfg = *cfg;
        kvm->k.assign((char *const *)swa_k, (char *const *)swa_k + cfg->n_swa_layers);
        kvm->v.assign((char *const *)swa_v, (char *const *)swa_v + cfg->n_swa_layers);
        kvm->snap_buf = (char *)snap_buf;
        kvm->snap_bytes = sb;
        kvm->seqs.resize(cfg->ring_seqs);
        if (cfg->pool_rows > 0) kvm->free_rows[0] = cfg->pool_rows;
        kvm->slot_used.assign(cfg->max_snapshots, false);
    } catch (...) {
        delete kvm;
        return fail(HSW_E_CAPACITY, "out of host memory");
    }
    *out = kvm;
    return HSW_OK;
}

void hsw_kvm_destroy(hsw_kvm *kvm) { delete kvm; }

hsw_status hsw_kvm_admit(hsw_kvm *kvm, int64_t max_len, int32_t *seq, int64_t *seq_base) {
    if (!kvm || !seq || !seq_base) return fail(HSW_E_NULL, "kvm, seq and seq_base must be non-NULL");
    if (max_len < 1) return fail(HSW_E_SHAPE, "max_len (%lld) must be >= 1", (long long)max_len);
    int32_t slot = -1;
    for (int32_t i = 0; i < (int32_t)kvm->seqs.size(); ++i)
        if (!kvm->seqs[i].used) { slot = i; break; }
    auto run = kvm->free_rows.end();
    for (auto it = kvm->free_rows.begin(); it != kvm->free_rows.end(); ++it)
        if (it->second >= max_len) { run = it; break; }
    // both pools are checked before anything is taken
    if (slot < 0 && run == kvm->free_rows.end())
        return fail(HSW_E_CAPACITY, "no free ring slot and no run of %lld free pool rows", (long long)max_len);
    if (slot < 0) return fail(HSW_E_CAPACITY, "no free ring slot (%d sequences)", (int)kvm->seqs.size());
    if (run == kvm->free_rows.end())
        return fail(HSW_E_CAPACITY, "no run of %lld free pool rows", (long long)max_len);
    const int64_t start = run->first, len = run->second;
    try {
        kvm->seqs[slot].slot_pos.assign(kvm->cfg.window, -1);   // (an unused slot: nothing to undo)
        if (len > max_len) kvm->free_rows[start + max_len] = len - max_len;
    } catch (...) {
        return fail(HSW_E_CAPACITY, "out of host memory");
    }
    kvm->free_rows.erase(start);
    hsw_kvm::Seq &s = kvm->seqs[slot];
    s.used = true;
    s.base = start;
    s.max_len = max_len;
    s.len = 0;
    s.tok.clear();
    *seq = slot;
    *seq_base = start;
    return HSW_OK;
}

hsw_status hsw_kvm_release(hsw_kvm *kvm, int32_t seq) {
    hsw_status st = check_seq(kvm, seq);
    if (st) return st;
    hsw_kvm::Seq &s = kvm->seqs[seq];
    drop_snaps_above(kvm, seq, -1);
    int64_t start = s.base, len = s.max_len;
    auto next = kvm->free_rows.lower_bound(start);
    if (next != kvm->free_rows.end() && next->first == start + len) {
        len += next->second;
        kvm->free_rows.erase(next);
    }
    auto prev = kvm->free_rows.lower_bound(start);
    if (prev != kvm->free_rows.begin()) {
        --prev;
        if (prev->first + prev->second == start) {
            start = prev->first;
            len += prev->second;
            kvm->free_rows.erase(prev);
        }
    }
    try {
        kvm->free_rows[start] = len;
    } catch (...) {
        return fail(HSW_E_CAPACITY, "out of host memory");
    }
    s = hsw_kvm::Seq();
    return HSW_OK;
}

hsw_status hsw_kvm_append(hsw_kvm *kvm, int32_t seq, const int32_t *tokens, int64_t n, int64_t *start_pos) {
    hsw_status st = check_seq(kvm, seq);
    if (st) return st;
    if (n < 0) return fail(HSW_E_SHAPE, "n (%lld) < 0", (long long)n);
    if (n > 0 && !tokens) return fail(HSW_E_NULL, "tokens is NULL");
    hsw_kvm::Seq &s = kvm->seqs[seq];
    if (s.len + n > s.max_len)
        return fail(HSW_E_CAPACITY, "sequence %d: %lld + %lld positions exceed its %lld rows", seq, (long long)s.len,
                    (long long)n, (long long)s.max_len);
    try {
        if (s.len + n > (int64_t)s.tok.size()) s.tok.reserve(s.len + n);
    } catch (...) {
        return fail(HSW_E_CAPACITY, "out of host memory");
    }
    if (start_pos) *start_pos = s.len;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t p = s.len + i;
        if (p < (int64_t)s.tok.size()) {
            if (s.tok[p] != tokens[i]) {
                drop_snaps_above(kvm, seq, p);  // row p now holds another history
                s.tok[p] = tokens[i];
            }
        } else {
            s.tok.push_back(tokens[i]);
        }
    }
    // the caller's attention calls over the appended tokens write each
    // position into its ring slot; only the last W of them stay
    const int64_t W = (int64_t)s.slot_pos.size();
    for (int64_t p = (n > W ? s.len + n - W : s.len); p < s.len + n; ++p) s.slot_pos[p % W] = p;
    s.len += n;
    return HSW_OK;
}

hsw_status hsw_kvm_truncate(hsw_kvm *kvm, int32_t seq, int64_t new_len) {
    hsw_status st = check_seq(kvm, seq);
    if (st) return st;
    hsw_kvm::Seq &s = kvm->seqs[seq];
    if (new_len < 0 || new_len > s.len)
        return fail(HSW_E_SHAPE, "new_len (%lld) must be in [0, %lld]", (long long)new_len, (long long)s.len);
    s.len = new_len;
    return HSW_OK;
}

hsw_status hsw_kvm_info(hsw_kvm *kvm, int32_t seq, int64_t *len, int64_t *seq_base, int64_t *max_len) {
    hsw_status st = check_seq(kvm, seq);
    if (st) return st;
    const hsw_kvm::Seq &s = kvm->seqs[seq];
    if (len) *len = s.len;
    if (seq_base) *seq_base = s.base;
    if (max_len) *max_len = s.max_len;
    return HSW_OK;
}

hsw_status hsw_kvm_free_space(hsw_kvm *kvm, int32_t *ring_slots, int64_t *pool_run, int32_t *snapshots) {
    if (!kvm) return fail(HSW_E_NULL, "kvm is NULL");
    int32_t r = 0, sn = 0;
    for (const auto &s : kvm->seqs) r += s.used ? 0 : 1;
    for (bool u : kvm->slot_used) sn += u ? 0 : 1;
    int64_t run = 0;
    for (const auto &f : kvm->free_rows) run = f.second > run ? f.second : run;
    if (ring_slots) *ring_slots = r;
    if (pool_run) *pool_run = run;
    if (snapshots) *snapshots = sn;
    return HSW_OK;
}

hsw_status hsw_kvm_snapshot(hsw_kvm *kvm, int32_t seq, int32_t *snap, hsw_stream_t stream) {
    hsw_status st = check_seq(kvm, seq);
    if (st) return st;
    if (!snap) return fail(HSW_E_NULL, "snap is NULL");
    int32_t slot = -1;
    for (int32_t i = 0; i < (int32_t)kvm->slot_used.size(); ++i)
        if (!kvm->slot_used[i]) { slot = i; break; }
    if (slot < 0) return fail(HSW_E_CAPACITY, "every snapshot slot (%d) is taken", (int)kvm->slot_used.size());
    const int32_t id = kvm->next_snap_id;
    try {
        kvm->snaps[id] = hsw_kvm::Snap{seq, kvm->seqs[seq].len, slot, kvm->seqs[seq].slot_pos};
    } catch (...) {
        return fail(HSW_E_CAPACITY, "out of host memory");
    }
    if ((st = copy_rings(kvm, seq, slot, true, (hipStream_t)stream))) {
        kvm->snaps.erase(id);
        return st;
    }
    kvm->slot_used[slot] = true;
    ++kvm->next_snap_id;
    *snap = id;
    return HSW_OK;
}

hsw_status hsw_kvm_restore(hsw_kvm *kvm, int32_t snap, hsw_stream_t stream) {
    if (!kvm) return fail(HSW_E_NULL, "kvm is NULL");
    auto it = kvm->snaps.find(snap);
    if (it == kvm->snaps.end()) return fail(HSW_E_STALE, "snapshot %d was released", snap);
    const hsw_kvm::Snap sn = it->second;
    hsw_kvm::Seq &s = kvm->seqs[sn.seq];
    hsw_status st = copy_rings(kvm, sn.seq, sn.slot, false, (hipStream_t)stream);
    if (st) return st;
    s.len = sn.pos;
    s.slot_pos = it->second.slot_pos;   // same size: no allocation
    return HSW_OK;
}

hsw_status hsw_kvm_drop_snapshot(hsw_kvm *kvm, int32_t snap) {
    if (!kvm) return fail(HSW_E_NULL, "kvm is NULL");
    auto it = kvm->snaps.find(snap);
    if (it == kvm->snaps.end()) return fail(HSW_E_STALE, "snapshot %d was released", snap);
    kvm->slot_used[it->second.slot] = false;
    kvm->snaps.erase(it);
    return HSW_OK;
}

int64_t hsw_kvm_window_safe_length(hsw_kvm *kvm, int32_t seq, const int32_t *tokens, int64_t n, int32_t *snap) {
    if (snap) *snap = -1;
    if (check_seq(kvm, seq) || n < 0 || (n > 0 && !tokens)) return -1;
    const hsw_kvm::Seq &s = kvm->seqs[seq];
    // common prefix with the rows' recorded ids (rows past len still hold
    // theirs, which snapshots above len rely on)
    int64_t lcp = 0;
    const int64_t lim = n < (int64_t)s.tok.size() ? n : (int64_t)s.tok.size();
    while (lcp < lim && s.tok[lcp] == tokens[lcp]) ++lcp;
    // live rings: any length up to the live one (a truncate reaches it)
    int64_t best = longest_held_window(s.slot_pos, lcp < s.len ? lcp : s.len);
    // a snapshot: its own position, if its copied rings hold that window
    for (const auto &kv : kvm->snaps) {
        const hsw_kvm::Snap &sn = kv.second;
        if (sn.seq == seq && sn.pos <= lcp && sn.pos > best && longest_held_window(sn.slot_pos, sn.pos) == sn.pos) {
            best = sn.pos;
            if (snap) *snap = kv.first;
        }
    }
    return best;
}

}  // extern "C"
