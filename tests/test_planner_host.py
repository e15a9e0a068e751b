"""Owner planner and packed-tail layout (host only, through the C ABI).

Pins of the reference (oracle.planner_ref):
* a hand-worked schedule: costs 7,5,4,3,3,2 on two owners go
  {7,3,2} / {5,4,3}, makespan 12 = total / 2 (optimal);
* Graham's bound: the LPT makespan is within (4/3 - 1/(3R)) of the optimum,
  the optimum found by trying every assignment of small instances;
* the byte cap and a schedule that the cap changes, worked by hand, and the
  rule for an item that no owner can take under the cap;
* tail layout offsets worked by hand.
The library must then give exactly the reference's assignment (same greedy
rule and tie breaks) on random instances, with and without a binding byte cap.
"""

import numpy as np
import pytest

import matrix_optimizer_step_owner_amd as mf
import oracle
from matrix_optimizer_step_owner_amd import _lib

ref = oracle.planner_ref


def test_hand_worked_schedule():
    cost = [7, 5, 4, 3, 3, 2]
    owner, load, used = ref.lpt_owners(cost, [1] * 6, 2, 10.0)
    assert owner == [0, 1, 1, 0, 1, 0] and load == [12.0, 12.0]
    assert ref.optimal_makespan(cost, 2) == 12.0
    assert mf.plan_owners(cost, [1] * 6, 2, byte_slack=10.0) == (owner, load, used)


def test_byte_cap_hand_worked():
    # cap = ceil((1 + slack) * max(total / R, largest item))
    assert ref.byte_cap([1, 10, 10, 1], 2, 0.0) == 11
    assert ref.byte_cap([3, 4], 2, 0.5) == 6          # largest item binds: 4 * 1.5
    assert ref.byte_cap([5, 5, 5], 2, 0.1) == 9       # ceil(7.5 * 1.1 = 8.25)


def test_binding_cap_changes_the_schedule():
    # costs 6,5,4,3 with bytes 1,10,10,1 on two owners, cap 11 (worked by hand):
    #   6 -> owner 0 (tie, lower rank)     loads 6,0   bytes 1,0
    #   5 -> owner 1 (less loaded)         loads 6,5   bytes 1,10
    #   4 -> owner 1 would hold 20 > 11: owner 0       loads 10,5  bytes 11,10
    #   3 -> owner 0 would hold 12 > 11: owner 1       loads 10,8  bytes 11,11
    cost, nbytes = [6, 5, 4, 3], [1, 10, 10, 1]
    want = ([0, 1, 0, 1], [10.0, 8.0], [11, 11])
    assert ref.lpt_owners(cost, nbytes, 2, 0.0) == want
    assert mf.plan_owners(cost, nbytes, 2, byte_slack=0.0) == want
    # without a binding cap LPT puts both 10-byte items on owner 1
    assert ref.lpt_owners(cost, nbytes, 2, 10.0) == ([0, 1, 1, 0], [9.0, 9.0], [2, 20])


def test_no_owner_under_the_cap_goes_to_fewest_bytes():
    # three 10-byte items on two owners, cap ceil(max(15, 10)) = 15:
    #   3 -> owner 0; 2 -> owner 1 (owner 0 would hold 20);
    #   1 -> neither stays under 15: the owner with the fewest bytes, tie 10/10
    #        to the lower rank, owner 0
    want = ([0, 1, 0], [4.0, 2.0], [20, 10])
    assert ref.lpt_owners([3, 2, 1], [10, 10, 10], 2, 0.0) == want
    assert mf.plan_owners([3, 2, 1], [10, 10, 10], 2, byte_slack=0.0) == want


@pytest.mark.parametrize("seed", range(12))
def test_graham_bound_and_library_equals_reference(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    R = int(rng.integers(2, 4))
    cost = [float(x) for x in rng.integers(1, 20, n)]
    nbytes = [int(x) for x in rng.integers(1, 1000, n)]
    owner, load, used = ref.lpt_owners(cost, nbytes, R, 1e9)   # cap never binds
    opt = ref.optimal_makespan(cost, R)
    assert opt <= max(load) <= (4 / 3 - 1 / (3 * R)) * opt + 1e-12
    assert mf.plan_owners(cost, nbytes, R, byte_slack=1e9) == (owner, load, used)


@pytest.mark.parametrize("seed", range(12))
def test_byte_cap_and_ties(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(5, 40))
    R = int(rng.integers(2, 9))
    # few distinct costs (ties) and skewed bytes so that the cap binds
    cost = [float(x) for x in rng.choice([1.0, 2.0, 5.0], n)]
    nbytes = [int(x) for x in (rng.pareto(1.5, n) * 1000 + 1)]
    slack = float(rng.choice([0.0, 0.05, 0.25]))
    got = mf.plan_owners(cost, nbytes, R, byte_slack=slack)
    want = ref.lpt_owners(cost, nbytes, R, slack)
    assert got == want
    owner, load, used = got
    for r in range(R):
        assert load[r] == pytest.approx(sum(c for c, o in zip(cost, owner) if o == r))
        assert used[r] == sum(b for b, o in zip(nbytes, owner) if o == r)
    assert sorted(set(owner)) <= list(range(R))


def test_planner_validation():
    lib = _lib.load()
    with pytest.raises(_lib.MfsdpError):
        mf.plan_owners([1.0], [1], 0)
    with pytest.raises(_lib.MfsdpError):
        mf.plan_owners([-1.0], [1], 2)
    with pytest.raises(_lib.MfsdpError):
        mf.plan_owners([float("nan")], [1], 2)
    with pytest.raises(_lib.MfsdpError):
        mf.plan_owners([1.0], [-5], 2)
    with pytest.raises(_lib.MfsdpError):
        mf.plan_owners([1.0], [5], 2, byte_slack=-0.1)
    assert mf.plan_owners([], [], 3) == ([], [0.0, 0.0, 0.0], [0, 0, 0])
    assert lib.mfsdp_plan_owners(None, None, 0, 1, 0.0, None, None, None) != 0


def test_tail_layout_hand_worked():
    assert ref.tail_layout([5, 0, 8, 3]) == ([0, 8, 8, 16], 20)
    assert mf.tail_layout([5, 0, 8, 3]) == ([0, 8, 8, 16], 20)
    assert mf.tail_layout([]) == ([], 0)
    rng = np.random.default_rng(3)
    sizes = [int(x) for x in rng.integers(0, 5000, 50)]
    assert mf.tail_layout(sizes) == ref.tail_layout(sizes)
    with pytest.raises(_lib.MfsdpError):
        mf.tail_layout([3, -1])


def _tail_call(fn, ptrs, numel, offsets, packed, packed_numel):
    import ctypes
    n = len(numel)
    P = (ctypes.c_void_p * max(n, 1))(*ptrs)
    N = (ctypes.c_int64 * max(n, 1))(*numel)
    O = (ctypes.c_int64 * max(n, 1))(*offsets)
    lib = _lib.load()
    if fn == "pack":
        return lib.mfsdp_tail_pack(P, N, O, n, packed, packed_numel, None)
    return lib.mfsdp_tail_unpack(packed, packed_numel, P, N, O, n, None)


@pytest.mark.parametrize("fn", ["pack", "unpack"])
def test_tail_copy_validation(fn):
    # invalid calls only: the library rejects them before any device work, so
    # the fake (never dereferenced) addresses below are safe
    A, B, PK = 0x10000, 0x20000, 0x40000
    inv, alias = 1, 4
    assert _tail_call(fn, [A], [5], [2], PK, 64) == inv            # offset not a multiple of 4
    assert _tail_call(fn, [A], [5], [60], PK, 64) == inv           # segment past the end
    assert _tail_call(fn, [None], [5], [0], PK, 64) == inv         # null tensor
    assert _tail_call(fn, [A + 2], [5], [0], PK, 64) == inv        # not 4-byte aligned
    assert _tail_call(fn, [A], [5], [0], PK + 4, 64) == inv        # packed not 16-byte aligned
    assert _tail_call(fn, [A, B], [5, 4], [0, 4], PK, 64) == alias  # segments overlap
    assert _tail_call(fn, [PK + 8], [4], [16], PK, 64) == alias     # tensor inside the buffer
    assert _tail_call(fn, [A], [-1], [0], PK, 64) == inv
    assert _tail_call(fn, [], [], [], PK, 0) == 0                  # nothing to copy
    # an empty tensor at the same offset as another one overlaps nothing; the
    # call then fails only on the (deliberately) misplaced third segment
    assert _tail_call(fn, [A, None, B], [5, 0, 4], [0, 8, 4], PK, 64) == alias
    if fn == "unpack":
        assert _tail_call(fn, [A, A + 8], [4, 4], [0, 8], PK, 64) == alias  # destinations overlap
