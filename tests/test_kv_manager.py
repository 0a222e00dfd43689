"""Dual-pool KV manager, host bookkeeping (CPU; no call here launches).

The reference model (oracle/kv_rules.py) is pinned first by hand-worked
scenarios whose expected values follow from the rules as the pages state them
(gokawiil section 2.1: both pools checked at admission, window-safe reuse
length; colibri "System One mode and prompt reuse": rows stay in place,
divergence below a snapshot releases it).  The C manager is then compared
with the model on random operation sequences: every admission result (error
or sequence / first row), length, free space and window-safe length must be
identical.  Snapshot copies need the GPU: those cases are in
tests/test_gpu_kv_manager.py.
"""
from __future__ import annotations

import random

import pytest

from oracle.kv_rules import KvModel

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw",
                          reason="libhsw.so not built (python -m hybrid_sliding_window_amd.build)")

FAKE = 0x10000  # 16-byte aligned device address, never dereferenced by bookkeeping calls


def manager(ring_seqs=4, pool_rows=10, layers=2, window=8):
    cfg = hsw.KvmConfig(layers, 2, window, 16, 8, 2, ring_seqs, pool_rows, 0)
    return hsw.KvManager(cfg, [FAKE] * layers, [FAKE] * layers, None)


def status(fn, *a):
    try:
        return fn(*a)
    except hsw.HswError as e:
        return {7: KvModel.CAPACITY, 8: KvModel.STALE, 2: KvModel.SHAPE}.get(e.status, e.status)


# ---------------------------------------------------------------- model pins
def test_model_admission_by_hand():
    m = KvModel(ring_seqs=2, pool_rows=10, max_snapshots=1)
    assert m.admit(4) == (0, 0)          # rows 0..3
    assert m.admit(3) == (1, 4)          # rows 4..6
    assert m.admit(1) == KvModel.CAPACITY     # ring pool full (rows 7..9 are free)
    assert m.release(0) is None
    assert m.free_space() == (1, 4, 1)   # free runs 0..3 and 7..9
    assert m.admit(5) == KvModel.CAPACITY     # a free slot, but no run of 5 rows
    assert m.admit(4) == (0, 0)
    assert m.release(1) is None
    assert m.free_space() == (1, 6, 1)   # 4..9 merged
    assert m.admit(0) == KvModel.SHAPE


def test_model_reuse_and_release_by_hand():
    """A 4-slot ring, so that the window matters after a few tokens: the state
    at L needs positions max(0, L - 3) .. L - 1 in their slots p mod 4."""
    m = KvModel(ring_seqs=1, pool_rows=16, max_snapshots=2, window=4)
    s, _ = m.admit(16)
    assert m.append(s, [1, 2, 3]) == 0                              # slots hold 0 1 2 -
    sid = m.snapshot(s)                                             # at position 3
    assert m.append(s, [4, 5]) == 3                                 # slots hold 4 1 2 3
    assert m.window_safe_length(s, [1, 2, 3, 4, 5, 6]) == (5, -1)   # live: 2 3 4 held
    assert m.window_safe_length(s, [1, 2, 3, 4]) == (4, -1)         # live: 1 2 3 held
    assert m.window_safe_length(s, [1, 2, 3, 9]) == (3, sid)        # 0 was overwritten: only the snapshot
    assert m.window_safe_length(s, [1, 2, 9]) == (0, -1)            # below every state
    assert m.truncate(s, 2) is None
    assert m.append(s, [3]) == 2                                    # same id: the snapshot stays
    assert m.window_safe_length(s, [1, 2, 3, 4, 5]) == (3, sid)     # live slot 0 still holds 4
    assert m.append(s, [7]) == 3                                    # row 3 held 4: above-3 snapshots only
    assert sid in m.snaps
    assert m.truncate(s, 1) is None
    assert m.append(s, [8]) == 1                                    # row 1 held 2: the snapshot at 3 goes
    assert m.restore(sid) == KvModel.STALE
    assert m.append(s, list(range(100, 115))) == KvModel.CAPACITY  # 2 + 15 > 16
    assert m.append(s, list(range(100, 114))) == 2                 # 2 + 14 = 16 fits


def truncate_scenario(window_safe_length, append, truncate):
    """A 300-token sequence on 128-slot rings (colibri 'System One mode':
    position p in slot p mod 128), so the rings hold 172..299; the state at L
    needs max(0, L - 127) .. L - 1.  Returns the reuse lengths seen."""
    ids = list(range(1000, 1300))
    seen = []
    assert append(ids) == 0
    seen.append(window_safe_length(ids))                          # 300: the live length
    seen.append(window_safe_length(ids[:299] + [7]))              # 299: needs 172..298, held
    seen.append(window_safe_length(ids[:298] + [7]))              # 298 needs 171 (slot 43 holds 299): 0
    truncate(250)
    seen.append(window_safe_length(ids))                          # 250 needs 123 (slot 123 holds 251): 0
    assert append(ids[250:260]) == 250                            # rewrites slots of 250..259 only
    seen.append(window_safe_length(ids))                          # 260 needs 133 (slot 5 holds 261): 0
    assert append(ids[260:300]) == 260
    seen.append(window_safe_length(ids))                          # 300 again: every slot rewritten
    truncate(40)                                                  # inside the first 128: slots 0..39 lost
    seen.append(window_safe_length(ids))
    return seen


TRUNCATE_WANT = [300, 299, 0, 0, 0, 300, 0]


def test_model_truncate_of_a_long_sequence_by_hand():
    m = KvModel(ring_seqs=1, pool_rows=400, max_snapshots=0, window=128)
    s, _ = m.admit(400)
    got = truncate_scenario(lambda t: m.window_safe_length(s, t)[0], lambda t: m.append(s, t),
                            lambda n: m.truncate(s, n))
    assert got == TRUNCATE_WANT


def test_model_short_sequence_reuses_any_prefix():
    """Up to 128 positions nothing has been overwritten: every prefix of the
    live length is window-safe."""
    m = KvModel(ring_seqs=1, pool_rows=200, max_snapshots=0, window=128)
    s, _ = m.admit(200)
    ids = list(range(100))
    m.append(s, ids)
    assert m.window_safe_length(s, ids[:40] + [-1]) == (40, -1)
    assert m.truncate(s, 40) is None
    assert m.window_safe_length(s, ids) == (40, -1)


# ------------------------------------------------ C manager against the model
def test_manager_truncate_of_a_long_sequence():
    """The C manager on the same scenario: a truncate below the last two
    positions of a sequence longer than the window leaves no windowed state
    until the positions are rewritten."""
    cfg = hsw.KvmConfig(2, 2, 128, 16, 8, 2, 1, 400, 0)
    kv = hsw.KvManager(cfg, [FAKE] * 2, [FAKE] * 2, None)
    s, _ = kv.admit(400)
    got = truncate_scenario(lambda t: kv.window_safe_length(s, t)[0], lambda t: kv.append(s, t),
                            lambda n: kv.truncate(s, n))
    assert got == TRUNCATE_WANT
    kv.close()


def test_manager_admission_matches_by_hand_values():
    kv = manager(ring_seqs=2, pool_rows=10)
    assert kv.admit(4) == (0, 0)
    assert kv.admit(3) == (1, 4)
    assert status(kv.admit, 1) == KvModel.CAPACITY
    kv.release(0)
    assert kv.free_space() == (1, 4, 0)
    assert status(kv.admit, 5) == KvModel.CAPACITY
    assert kv.admit(4) == (0, 0)
    kv.release(1)
    assert kv.free_space() == (1, 6, 0)
    assert status(kv.admit, 0) == KvModel.SHAPE
    kv.close()


@pytest.mark.parametrize("seed", range(9))
def test_manager_matches_model_on_random_operations(seed):
    rng = random.Random(seed)
    ring_seqs, pool_rows = rng.choice([(3, 40), (5, 64), (8, 200)])
    window = (8, 1, 3)[seed % 3]          # window 1: the token attends to itself only
    kv = manager(ring_seqs, pool_rows, window=window)
    m = KvModel(ring_seqs, pool_rows, 0, window=window)
    vocab = [1, 2, 3]                      # few ids: shared prefixes and rewrites are common
    for step in range(400):
        op = rng.choice(["admit", "admit", "release", "append", "append", "append", "truncate", "wsl", "info"])
        live = sorted(m.seqs)
        seq = rng.choice(live) if live and rng.random() < 0.9 else rng.randrange(ring_seqs + 1)
        if op == "admit":
            n = rng.randint(0, pool_rows // 2)
            assert status(kv.admit, n) == m.admit(n), (seed, step)
        elif op == "release":
            assert status(kv.release, seq) == m.release(seq), (seed, step)
        elif op == "append":
            toks = [rng.choice(vocab) for _ in range(rng.randint(0, 6))]
            assert status(kv.append, seq, toks) == m.append(seq, toks), (seed, step)
        elif op == "truncate":
            ln = m.seqs[seq]["len"] if seq in m.seqs else 8
            n = rng.choice([rng.randint(-1, 8), ln - 1, ln - 2, ln - rng.randint(0, 2 * window + 2)])
            assert status(kv.truncate, seq, n) == m.truncate(seq, n), (seed, step)
        elif op == "info":
            assert status(kv.info, seq) == m.info(seq), (seed, step)
        elif seq in m.seqs:
            toks = m.seqs[seq]["rows"][:rng.randint(0, 8)] + [rng.choice(vocab) for _ in range(rng.randint(0, 4))]
            assert kv.window_safe_length(seq, toks) == m.window_safe_length(seq, toks), (seed, step)
        assert kv.free_space() == m.free_space(), (seed, step)
    # every admitted sequence's rows are disjoint and inside the pool
    rows = set()
    for s in m.seqs:
        ln, base, mx = kv.info(s)
        span = set(range(base, base + mx))
        assert not rows & span and base + mx <= pool_rows
        rows |= span
    kv.close()


def test_manager_argument_errors():
    cfg = hsw.KvmConfig(2, 2, 8, 16, 8, 2, 4, 10, 0)
    bad = hsw.KvmConfig(0, 2, 8, 16, 8, 2, 4, 10, 0)
    with pytest.raises(hsw.HswError) as e:
        hsw.KvManager(bad, [], [], None)
    assert e.value.status == 2
    with pytest.raises(hsw.HswError) as e:
        hsw.KvManager(cfg, [FAKE + 8, FAKE], [FAKE, FAKE], None)
    assert e.value.status == 3
    snap_cfg = hsw.KvmConfig(2, 2, 8, 16, 8, 2, 4, 10, 2)
    with pytest.raises(hsw.HswError) as e:
        hsw.KvManager(snap_cfg, [FAKE] * 2, [FAKE] * 2, None)
    assert e.value.status == 1
    kv = manager()
    assert status(kv.restore, 0) == KvModel.STALE
    assert status(kv.drop_snapshot, 3) == KvModel.STALE
    assert status(kv.append, 2, [1]) == KvModel.SHAPE      # not admitted
    with pytest.raises(hsw.HswError):
        kv.window_safe_length(1, [1])
    kv.close()


def test_snapshot_bytes_are_the_pages_ring_size():
    """colibri 'System One mode': a Flash snapshot is 39 rings x 128 slots x 8
    heads x (192 + 128) values, about 50 MB in fp32."""
    f32 = hsw.KvmConfig(39, 8, 128, 192, 128, 4, 1, 0, 1)
    assert hsw.hsw_kvm_snapshot_bytes(f32) == 39 * 128 * 8 * 320 * 4 == 51_118_080
    bf16 = hsw.KvmConfig(39, 8, 128, 192, 128, 2, 1, 0, 1)
    assert hsw.hsw_kvm_snapshot_bytes(bf16) == 51_118_080 // 2
    assert hsw.hsw_kvm_snapshot_bytes(hsw.KvmConfig(0, 8, 128, 192, 128, 2, 1, 0, 1)) == 0
