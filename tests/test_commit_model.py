"""The host model of the token-commit protocol (oracle/commit.py) against
hand-worked sequences of commits, each expected state written out from the
protocol (Arc PR #217, "What this does", step 3, and its fault handling)."""

from oracle import commit as cm


def test_publishes_in_order_and_wraps():
    m = cm.CommitModel(B=2, V=10, capacity=2)
    assert m.commit([1, 2]) and m.commit([3, 4])
    assert (m.position, m.published, m.fault) == (2, 2, cm.FAULT_NONE)
    assert m.ring == [[1, 2], [3, 4]] and m.next_input == [3, 4]
    m.drained = 1  # the host consumed step 0: its slot is free again
    assert m.commit([5, 6])
    assert m.ring == [[5, 6], [3, 4]] and (m.position, m.published) == (3, 3)


def test_overrun_latches_and_blocks_until_cleared():
    m = cm.CommitModel(B=1, V=10, capacity=2)
    assert m.commit([1]) and m.commit([2])
    assert not m.commit([3])  # slot 0 still holds step 0
    assert m.fault == cm.FAULT_RING_OVERRUN and (m.position, m.published) == (2, 2)
    assert m.ring == [[1], [2]] and m.next_input == [2]
    m.drained = 2
    assert not m.commit([3])  # drained, but the fault word is still set
    assert m.fault == cm.FAULT_RING_OVERRUN
    m.fault = cm.FAULT_NONE
    assert m.commit([3]) and m.ring == [[3], [2]] and m.position == 3


def test_token_range_and_refused_rows():
    m = cm.CommitModel(B=3, V=5, capacity=4)
    assert m.commit([0, -1, 4])  # -1 marks a refused row: published, no fault
    assert m.ring[0] == [0, -1, 4] and m.fault == cm.FAULT_NONE
    for bad in ([0, 5, 1], [-2, 0, 1]):
        assert not m.commit(bad)
        assert m.fault == cm.FAULT_TOKEN_RANGE and m.position == 1
        m.fault = cm.FAULT_NONE
    # the first fault stays: a later overrun does not replace it
    m2 = cm.CommitModel(B=1, V=5, capacity=1)
    assert m2.commit([1])
    assert not m2.commit([9]) and m2.fault == cm.FAULT_TOKEN_RANGE
    assert not m2.commit([1]) and m2.fault == cm.FAULT_TOKEN_RANGE
