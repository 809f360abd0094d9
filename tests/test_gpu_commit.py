"""GPU tests of arcs_commit_tokens: one step's tokens published into a pinned
host ring that the host drains by polling, with no HIP call in between; the
sticky fault word for out-of-range tokens and ring overruns; refused rows;
and the commit captured with the keyed sampler in a HIP graph.  After every
commit the device and host words are compared with the host model of the
protocol (oracle/commit.py), and sampled tokens with the sampling oracle."""

import time

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from oracle import commit as cm
from oracle import sampler as oracle
from workloads import make_params, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def arcs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


class Ring:
    def __init__(self, B, capacity, V=None):
        import torch
        self.model = cm.CommitModel(B, V, capacity) if V is not None else None
        self.ring = torch.full((capacity, B), -7, dtype=torch.int32).pin_memory()
        self.published = torch.zeros(1, dtype=torch.int64).pin_memory()
        self.drained = torch.zeros(1, dtype=torch.int64).pin_memory()
        self.fault = torch.zeros(1, dtype=torch.int32).pin_memory()
        self.position = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.next_input = torch.full((B,), -1, dtype=torch.int32, device="cuda")

    def commit(self, arcs, ids, V, check=True):
        arcs.commit_tokens(ids, V, self.position, self.ring, self.published, self.drained, self.fault,
                           next_input=self.next_input)
        if self.model is not None and check:
            import torch
            torch.cuda.synchronize()
            self.model.drained = int(self.drained[0])
            self.model.commit(ids.cpu().tolist())
            self.check()

    def check(self):
        m = self.model
        assert int(self.position.item()) == m.position
        assert int(self.published[0]) == m.published
        assert int(self.fault[0]) == m.fault
        assert self.ring.tolist() == m.ring
        if m.next_input is not None:
            assert self.next_input.cpu().tolist() == m.next_input

    def host_clears_fault(self):
        self.fault[0] = 0
        if self.model is not None:
            self.model.fault = cm.FAULT_NONE

    def host_drains(self, n):
        self.drained[0] = n
        if self.model is not None:
            self.model.drained = n

    def wait_published(self, count, seconds=10.0):
        # plain reads of pinned host memory: no stream synchronisation
        deadline = time.time() + seconds
        while int(self.published[0]) < count and time.time() < deadline:
            pass
        return int(self.published[0])


def _setup(arcs, B=6, V=4096):
    w = make_workload("normal_b4_bf16", B=B, V=V)
    logits = to_device_logits(w.logits, "bf16")
    params = arcs.params_to_device(make_params(B, temperature=1.0, top_p=0.9))
    return logits, params


def _oracle_ids(B, V, seed, step, params):
    w = make_workload("normal_b4_bf16", B=B, V=V)
    return np.array([r.id for r in oracle.sample(w.logits, "bf16", params, None, None, seed, step)])


def test_commit_publishes_each_step(arcs):
    import torch
    B, V, steps, seed = 6, 4096, 3, 3
    logits, params = _setup(arcs, B, V)
    r = Ring(B, capacity=4)
    key = arcs.make_key(seed, 0)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    got = []
    for _ in range(steps):
        arcs.sample_keyed(logits, params, key, out=out)
        r.commit(arcs, out, V)
        got.append(out.clone())
    assert r.wait_published(steps) == steps
    torch.cuda.synchronize()
    want = [arcs.sample(logits, params, seed=seed, step=s).cpu().numpy() for s in range(steps)]
    ph = make_params(B, temperature=1.0, top_p=0.9)
    for s in range(steps):
        assert np.array_equal(got[s].cpu().numpy(), want[s])
        assert np.array_equal(r.ring[s].numpy(), want[s])
        assert np.array_equal(want[s], _oracle_ids(B, V, seed, s, ph)), s
    assert (r.ring[steps:] == -7).all()
    assert int(r.fault[0]) == 0 and int(r.position.item()) == steps
    assert np.array_equal(r.next_input.cpu().numpy(), want[-1])


def test_commit_ring_overrun_and_drain(arcs):
    import torch
    B, V = 5, 4096
    logits, params = _setup(arcs, B, V)
    r = Ring(B, capacity=2, V=V)
    ids = [arcs.sample(logits, params, seed=1, step=s) for s in range(4)]
    r.commit(arcs, ids[0], V)
    r.commit(arcs, ids[1], V)
    r.commit(arcs, ids[2], V)  # slot 0 still holds step 0: refused, fault latched
    torch.cuda.synchronize()
    assert int(r.published[0]) == 2 and int(r.position.item()) == 2
    assert int(r.fault[0]) == 2
    assert np.array_equal(r.ring[0].numpy(), ids[0].cpu().numpy())
    assert np.array_equal(r.next_input.cpu().numpy(), ids[1].cpu().numpy())
    # the host drains both steps but leaves the fault set: still refused
    r.host_drains(2)
    r.commit(arcs, ids[2], V)
    torch.cuda.synchronize()
    assert int(r.published[0]) == 2 and int(r.fault[0]) == 2
    # cleared: the step goes into slot 0
    r.host_clears_fault()
    r.commit(arcs, ids[2], V)
    r.commit(arcs, ids[3], V)
    assert r.wait_published(4) == 4
    torch.cuda.synchronize()
    assert np.array_equal(r.ring[0].numpy(), ids[2].cpu().numpy())
    assert np.array_equal(r.ring[1].numpy(), ids[3].cpu().numpy())
    assert int(r.fault[0]) == 0 and int(r.position.item()) == 4


def test_commit_refuses_out_of_range_tokens(arcs):
    import torch
    B, V = 4, 100
    r = Ring(B, capacity=3, V=V)
    good = torch.tensor([0, 99, 5, 42], dtype=torch.int32, device="cuda")
    r.commit(arcs, good, V)
    for bad in ([0, 100, 5, 42], [-2, 3, 5, 42], [7, 3, -100, 2**31 - 1]):
        r.commit(arcs, torch.tensor(bad, dtype=torch.int32, device="cuda"), V)
        torch.cuda.synchronize()
        assert int(r.fault[0]) == 1
        assert int(r.published[0]) == 1 and int(r.position.item()) == 1
        assert (r.ring[1] == -7).all()
        assert r.next_input.cpu().tolist() == good.cpu().tolist()
        r.host_clears_fault()


def test_commit_publishes_rows_the_sampler_refused(arcs):
    """A batch with a row of invalid parameters: the sampler gives that row
    -1 and its status; the commit publishes the step (the other rows' tokens
    and the -1) without latching a fault."""
    import torch
    B, V, seed = 6, 4096, 5
    w = make_workload("normal_b4_bf16", B=B, V=V)
    logits = to_device_logits(w.logits, "bf16")
    p = make_params(B, temperature=1.0, top_p=0.9)
    p[2]["temperature"] = -1.0
    p[4]["top_p"] = 0.0
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    ids = arcs.sample(logits, arcs.params_to_device(p), seed=seed, step=0, out_status=status)
    refs = oracle.sample(w.logits, "bf16", p, None, None, seed, 0)
    assert ids.cpu().tolist() == [r.id for r in refs]
    assert status.cpu().tolist() == [r.status for r in refs] == [0, 0, 1, 0, 2, 0]
    r = Ring(B, capacity=2, V=V)
    r.commit(arcs, ids, V)
    assert r.wait_published(1) == 1
    assert r.ring[0].tolist() == [r_.id for r_ in refs] and int(r.fault[0]) == 0


def test_commit_in_a_graph_with_the_keyed_sampler(arcs):
    import torch
    B, V, seed, reps = 8, 4096, 11, 5
    logits, params = _setup(arcs, B, V)
    want = [arcs.sample(logits, params, seed=seed, step=s).cpu().numpy() for s in range(reps + 1)]
    r = Ring(B, capacity=8, V=V)
    key = arcs.make_key(seed, 0)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch outside the capture (no commit)
        arcs.sample_keyed(logits, params, key, advance=False, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        arcs.sample_keyed(logits, params, key, out=out)
        r.commit(arcs, out, V, check=False)
    torch.cuda.synchronize()
    assert int(r.published[0]) == 0  # capture runs nothing
    for i in range(reps):
        g.replay()
        if i == 2:
            torch.cuda.synchronize()  # eager work between replays
            assert int(r.published[0]) == 3
    assert r.wait_published(reps) == reps
    torch.cuda.synchronize()
    ph = make_params(B, temperature=1.0, top_p=0.9)
    for s in range(reps):
        assert np.array_equal(r.ring[s].numpy(), want[s]), s
        assert np.array_equal(want[s], _oracle_ids(B, V, seed, s, ph)), s
        r.model.commit(want[s].tolist())  # the host model, step by step
    r.check()
    assert int(r.fault[0]) == 0 and int(r.position.item()) == reps
