"""The expert slot bank on the host (no GPU needed).

The oracle (oracle/bank.py) is pinned to least-recently-used replacement by
a textbook reference string, by the LRU stack-distance property and by a
multi-expert case worked out by hand; the library's moe_bank_plan must then
equal it exactly (integer work) on random pass sequences, and reject every
invalid request with the documented status."""

import ctypes

import numpy as np
import pytest

import quantized_routed_moe_amd as qm
from oracle import bank as ob

A16 = 0x10000          # fake, aligned "device" addresses (never dereferenced)


# ---------------------------------------------------------------- oracle pins

def test_oracle_textbook_reference_string():
    # The classic 20-reference string of the operating-systems textbooks
    # (Silberschatz, Galvin, Gagne, "Operating System Concepts", page
    # replacement): with 3 frames LRU takes 12 faults (FIFO 15, OPT 9).
    refs = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
    b = ob.SlotBank(8, 3)
    faults = sum(len(b.plan([e])) for e in refs)
    assert faults == 12
    assert sorted(e for e in b.holder) == [0, 1, 7]


def test_oracle_lru_stack_distance():
    # A reference hits an LRU cache of N slots iff fewer than N distinct
    # other keys were referenced since its previous reference.
    rng = np.random.default_rng(5)
    for N in (1, 2, 3, 5, 8):
        refs = [int(v) for v in rng.integers(0, 12, size=400)]
        b = ob.SlotBank(12, N)
        for i, e in enumerate(refs):
            hit = len(b.plan([e])) == 0
            prev = [j for j in range(i) if refs[j] == e]
            expect = bool(prev) and len(set(refs[prev[-1] + 1:i])) < N
            assert hit == expect, (N, i)


def test_oracle_hand_worked_passes():
    # E = 6, N = 3; loads derived by hand from the rules in oracle/bank.py.
    calls = [[0, 1], [2], [3, 0], [4, 5], [0, 1, 2, 3]]
    got = ob.run_layer_calls(6, 3, calls)
    assert [c["loads"] for c in got] == [
        [[(0, 0), (1, 1)]],
        [[(2, 2)]],
        [[(3, 1)]],
        [[(4, 2), (5, 0)]],
        [[(0, 2), (1, 0)], [(2, 1)]],     # 3 resident first: passes [3, 0, 1] and [2]
    ]
    assert [c["hits"] for c in got] == [0, 0, 1, 0, 1]
    assert got[-1]["holder"] == [1, 2, 0]


def test_oracle_invariants():
    rng = np.random.default_rng(9)
    E = 16
    seen = set()
    big = ob.SlotBank(E, E)
    misses = 0
    for _ in range(200):
        want = [int(v) for v in rng.choice(E, size=int(rng.integers(1, 5)), replace=False)]
        seen |= set(want)
        misses += len(big.plan(want))
    assert misses == len(seen)            # N >= E: compulsory misses only
    for N in (2, 4, 7):
        b = ob.SlotBank(E, N)
        for _ in range(300):
            want = [int(v) for v in rng.choice(E, size=int(rng.integers(0, N + 1)), replace=False)]
            before = list(b.holder)
            loads = b.plan(want)
            held = [e for e in b.holder if e is not None]
            assert len(held) == len(set(held))
            assert set(want) <= set(held)
            for e, s in loads:
                assert before[s] not in want
            assert len(loads) == len([e for e in want if e not in before])


# ------------------------------------------------- library against the oracle

@pytest.mark.parametrize("E,N", [(8, 1), (8, 3), (16, 5), (64, 8), (64, 64), (33, 32)])
def test_plan_equals_oracle(E, N):
    rng = np.random.default_rng(1000 * E + N)
    lib_b = qm.BankState(E, N)
    ora = ob.SlotBank(E, N)
    for step in range(400):
        n = int(rng.integers(0, N + 1))
        want = [int(v) for v in rng.choice(E, size=n, replace=False)]
        assert lib_b.plan(want) == ora.plan(want), step
        holder = [-1 if h is None else h for h in ora.holder]
        assert lib_b.expert_of_slot.tolist() == holder
        for e in range(E):
            s = ora.slot_of(e)
            assert lib_b.slot_of_expert[e] == (-1 if s is None else s)


def test_layer_pass_order_is_the_oracles():
    # moe_layer_banked plans its passes with moe_bank_plan over the active
    # experts, resident first, then the rest, in id order (the oracle's
    # layer_passes); replay that on the host with the library's planner.
    rng = np.random.default_rng(3)
    E, N = 64, 8
    lib_b = qm.BankState(E, N)
    calls = [sorted(set(int(v) for v in rng.integers(0, E, size=int(rng.integers(1, 40))))) for _ in range(60)]
    expect = ob.run_layer_calls(E, N, calls)
    for c, ex in zip(calls, expect):
        res = [e for e in c if lib_b.slot_of_expert[e] >= 0]
        order = res + [e for e in c if lib_b.slot_of_expert[e] < 0]
        passes = [order[i:i + N] for i in range(0, len(order), N)]
        assert [lib_b.plan(p) for p in passes] == ex["loads"]


# ----------------------------------------------------------------- validation

def _bank(E=8, N=3):
    return qm.BankState(E, N)


def test_plan_rejects_bad_requests():
    b = _bank()
    L = qm.lib()
    le = (ctypes.c_int32 * 8)()
    ls = (ctypes.c_int32 * 8)()
    n = ctypes.c_int32(-5)

    def plan(ids, count=None):
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        return L.moe_bank_plan(ctypes.byref(b.c), arr, len(ids) if count is None else count, le, ls,
                               ctypes.byref(n))

    before = (b.slot_of_expert.copy(), b.expert_of_slot.copy(), b.last_use.copy(), b.c.clock)
    assert plan([1, 1]) == qm.MOE_ERR_SHAPE          # repeated id
    assert plan([8]) == qm.MOE_ERR_SHAPE             # id >= E
    assert plan([-1]) == qm.MOE_ERR_SHAPE
    assert plan([0, 1, 2, 3]) == qm.MOE_ERR_SHAPE    # more than N
    assert plan([0], count=-1) == qm.MOE_ERR_SHAPE
    assert L.moe_bank_plan(ctypes.byref(b.c), None, 1, le, ls, ctypes.byref(n)) == qm.MOE_ERR_NULL
    assert L.moe_bank_plan(ctypes.byref(b.c), None, 0, None, None, None) == qm.MOE_ERR_NULL
    assert L.moe_bank_plan(None, None, 0, None, None, ctypes.byref(n)) == qm.MOE_ERR_NULL
    after = (b.slot_of_expert, b.expert_of_slot, b.last_use, b.c.clock)
    assert all(np.array_equal(x, y) for x, y in zip(before[:3], after[:3])) and before[3] == after[3]
    assert plan([], count=0) == qm.MOE_OK and n.value == 0


@pytest.mark.parametrize("E,N", [(0, 1), (65, 8), (8, 0), (8, 9)])
def test_bank_shape_limits(E, N):
    st = qm.moe_bank(E, N, A16, A16, A16, 0)
    assert qm.lib().moe_bank_reset(ctypes.byref(st)) == qm.MOE_ERR_SHAPE


def test_bank_null_arrays():
    st = qm.moe_bank(8, 2, None, A16, A16, 0)
    assert qm.lib().moe_bank_reset(ctypes.byref(st)) == qm.MOE_ERR_NULL
    assert qm.lib().moe_bank_reset(None) == qm.MOE_ERR_NULL


def _qm(fmt=qm.MOE_FMT_MXFP4, layout=qm.MOE_LAYOUT_TILES, codes=A16, scales=A16, mins=None):
    return qm.moe_qmat(fmt, layout, codes, scales, mins)


def _ex(num_slots, **kw):
    return qm.moe_experts(_qm(**kw), _qm(**kw), _qm(**kw), None, num_slots)


def test_fetch_validation():
    L = qm.lib()
    pool, slots = _ex(8), _ex(3)
    le = (ctypes.c_int32 * 1)(0)
    ls = (ctypes.c_int32 * 1)(0)
    assert L.moe_bank_fetch(None, ctypes.byref(slots), 256, 128, le, ls, 1, None) == qm.MOE_ERR_NULL
    assert L.moe_bank_fetch(ctypes.byref(_ex(8, fmt=qm.MOE_FMT_Q2G32)), ctypes.byref(slots), 256, 128, le, ls, 1,
                            None) == qm.MOE_ERR_FORMAT
    assert L.moe_bank_fetch(ctypes.byref(_ex(8, layout=qm.MOE_LAYOUT_ROWS)), ctypes.byref(slots), 256, 128, le, ls,
                            1, None) == qm.MOE_ERR_FORMAT
    assert L.moe_bank_fetch(ctypes.byref(pool), ctypes.byref(slots), 256, 100, le, ls, 1, None) == qm.MOE_ERR_SHAPE
    bad_e = (ctypes.c_int32 * 1)(8)
    bad_s = (ctypes.c_int32 * 1)(3)
    assert L.moe_bank_fetch(ctypes.byref(pool), ctypes.byref(slots), 256, 128, bad_e, ls, 1, None) == qm.MOE_ERR_SHAPE
    assert L.moe_bank_fetch(ctypes.byref(pool), ctypes.byref(slots), 256, 128, le, bad_s, 1, None) == qm.MOE_ERR_SHAPE
    assert L.moe_bank_fetch(ctypes.byref(pool), ctypes.byref(slots), 256, 128, None, ls, 1, None) == qm.MOE_ERR_NULL
    assert L.moe_bank_fetch(ctypes.byref(pool), ctypes.byref(slots), 256, 128, le, ls, 0, None) == qm.MOE_OK


def test_layer_banked_validation():
    L = qm.lib()
    b = _bank(8, 3)
    shape = qm.moe_shape(4, 256, 8, 2, 128)
    pool, slots = _ex(8), _ex(3)
    st = qm.moe_bank_stats()

    def call(shape=shape, pool=pool, slots=slots, bank=b.c, slot_map=A16, ws_bytes=1 << 30, ws=A16):
        return L.moe_layer_banked(ctypes.byref(shape), A16, A16, None, A16, ctypes.byref(pool), ctypes.byref(bank),
                                  ctypes.byref(slots), slot_map, A16, A16, A16, ws, ws_bytes, None, ctypes.byref(st))

    assert call(slot_map=None) == qm.MOE_ERR_NULL
    assert call(ws=None) == qm.MOE_ERR_NULL
    assert call(slot_map=A16 + 2) == qm.MOE_ERR_ALIGN
    assert call(shape=qm.moe_shape(4, 256, 16, 2, 128)) == qm.MOE_ERR_SHAPE       # bank E != shape E
    assert call(shape=qm.moe_shape(4, 250, 8, 2, 128)) == qm.MOE_ERR_SHAPE        # invalid shape
    assert call(slots=_ex(4)) == qm.MOE_ERR_SHAPE                                  # bank N != slots
    assert call(pool=_ex(7)) == qm.MOE_ERR_SHAPE                                   # pool smaller than E
    assert call(ws_bytes=1024) == qm.MOE_ERR_WORKSPACE
    assert call(shape=qm.moe_shape(0, 256, 8, 2, 128)) == qm.MOE_OK               # T = 0: nothing
    assert (st.active, st.hits, st.misses, st.passes, st.bytes_paged) == (0, 0, 0, 0, 0)


def test_layer_banked_rejects_before_touching_the_bank():
    """Every argument is checked before the first HIP call and before any
    planning: a rejected call leaves the bank's books exactly as they were
    (a bank that claimed slots whose copies never ran would later compute
    with wrong slot contents)."""
    L = qm.lib()
    b = _bank(8, 3)
    b.plan([2, 5])                                   # some residents and stamps
    before = (b.slot_of_expert.copy(), b.expert_of_slot.copy(), b.last_use.copy(), b.c.clock)
    shape = qm.moe_shape(4, 256, 8, 2, 128)
    st = qm.moe_bank_stats()

    def call(pool=_ex(8), slots=_ex(3), x=A16, ws=A16, out=A16):
        return L.moe_layer_banked(ctypes.byref(shape), x, A16, None, A16, ctypes.byref(pool), ctypes.byref(b.c),
                                  ctypes.byref(slots), A16, A16, A16, out, ws, 1 << 30, None, ctypes.byref(st))

    assert call(x=A16 + 2) == qm.MOE_ERR_ALIGN                                   # route arguments
    assert call(slots=_ex(3, fmt=qm.MOE_FMT_Q2G32)) == qm.MOE_ERR_FORMAT          # bank pack vs pool
    assert call(slots=_ex(3, codes=A16 + 8)) == qm.MOE_ERR_ALIGN                  # FFN alignment of the bank
    assert call(out=None) == qm.MOE_ERR_NULL
    bad = _ex(3)
    bad.slot_bytes = 1000                                                         # not a multiple of 256
    assert call(slots=bad) == qm.MOE_ERR_ALIGN
    b.c.copy_stream = A16                                                         # a copy stream needs its events
    assert call() == qm.MOE_ERR_NULL
    b.c.copy_stream = None
    after = (b.slot_of_expert, b.expert_of_slot, b.last_use, b.c.clock)
    for x0, x1 in zip(before[:3], after[:3]):
        assert np.array_equal(x0, x1)
    assert before[3] == after[3]


# ------------------------------------------------------------------ sizing

def _slab(fmt, d, f):
    off = (ctypes.c_size_t * 6)()
    n = qm.lib().moe_slab_layout(fmt, d, f, off)
    return int(n), list(off)


@pytest.mark.parametrize("fmt,per_expert", [(qm.MOE_FMT_MXFP4, 13_369_344), (qm.MOE_FMT_Q2G32, 9_437_184),
                                            (qm.MOE_FMT_Q4G32, 15_728_640)])
def test_slab_layout_at_the_expert_shape(fmt, per_expert):
    """At d = 4096, f = 2048 every array is a multiple of 256 bytes, so a
    slab holds exactly one expert's bytes: MXFP4 3 d f (1/2 + 1/32), Q2
    3 d f (1/4 + 4/32), Q4 3 d f (1/2 + 4/32)."""
    n, off = _slab(fmt, 4096, 2048)
    assert n == per_expert
    sizes = []
    for name, rows, K in (("gate", 2048, 4096), ("up", 2048, 4096), ("down", 4096, 2048)):
        c, s_, _ = qm.moe_qmat_bytes(fmt, qm.MOE_LAYOUT_TILES, 1, rows, K)
        sizes += [c, s_]
    assert off == list(np.cumsum([0] + sizes[:-1]))
    assert sum(sizes) == n


def test_slab_layout_rounds_each_array_to_256():
    n, off = _slab(qm.MOE_FMT_MXFP4, 96, 32)          # tiny: scale arrays of a few dozen bytes
    assert all(o % 256 == 0 for o in off) and n % 256 == 0
    assert off == sorted(off) and len(set(off)) == 6
    assert _slab(9, 96, 32)[0] == 0 and _slab(qm.MOE_FMT_MXFP4, 100, 32)[0] == 0


def _slots(fmt, shape, budget, free, reserve=0):
    n = ctypes.c_int32(-1)
    rc = qm.lib().moe_bank_slots(fmt, ctypes.byref(shape), budget, free, reserve, ctypes.byref(n))
    return rc, n.value


def test_bank_slots_budget_auto_and_clamp():
    L = qm.lib()
    pre = qm.moe_shape(2048, 4096, 64, 2, 2048)         # a prefill chunk
    slab = 13_369_344
    ws = L.moe_layer_workspace_bytes(ctypes.byref(pre))
    GiB = 1 << 30
    # explicit budget: budget / slab, whatever the free memory beyond it
    assert _slots(qm.MOE_FMT_MXFP4, pre, 8 * slab + 5, 200 * GiB) == (qm.MOE_OK, 8)
    # capped at E
    assert _slots(qm.MOE_FMT_MXFP4, pre, 100 * GiB, 200 * GiB) == (qm.MOE_OK, 64)
    # auto: what is free after the prefill workspace and the reserve
    free = ws + 3 * GiB + 10 * slab
    assert _slots(qm.MOE_FMT_MXFP4, pre, 0, free, 3 * GiB) == (qm.MOE_OK, 10)
    # the clamp: a budget larger than what is free shrinks to fit
    assert _slots(qm.MOE_FMT_MXFP4, pre, 50 * slab, free, 3 * GiB) == (qm.MOE_OK, 10)
    # not one slot fits
    assert _slots(qm.MOE_FMT_MXFP4, pre, 0, ws + slab - 1) == (qm.MOE_ERR_WORKSPACE, 0)
    assert _slots(qm.MOE_FMT_MXFP4, pre, slab - 1, 200 * GiB) == (qm.MOE_ERR_WORKSPACE, 0)
    # other formats use their own slab size
    assert _slots(qm.MOE_FMT_Q2G32, pre, 10 * 9_437_184, 200 * GiB) == (qm.MOE_OK, 10)
    # validation
    assert _slots(7, pre, 0, 200 * GiB)[0] == qm.MOE_ERR_FORMAT
    assert _slots(qm.MOE_FMT_MXFP4, qm.moe_shape(1, 100, 64, 2, 2048), 0, 200 * GiB)[0] == qm.MOE_ERR_SHAPE
    n = ctypes.c_int32(0)
    assert L.moe_bank_slots(qm.MOE_FMT_MXFP4, None, 0, 1, 0, ctypes.byref(n)) == qm.MOE_ERR_NULL
    assert L.moe_bank_slots(qm.MOE_FMT_MXFP4, ctypes.byref(pre), 0, 1, 0, None) == qm.MOE_ERR_NULL


def test_bank_slots_python_helper_uses_the_same_rule():
    pre = qm.Shape(16, 4096, 64, 2, 2048)
    n = qm.bank_slots("q2", pre, budget_bytes=0, reserve_bytes=0, free_bytes=1 << 40)
    assert n == 64
    assert qm.bank_slots("q2", pre, budget_bytes=3 * 9_437_184, free_bytes=1 << 40) == 3
