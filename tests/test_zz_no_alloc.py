"""arcs_sample_noalloc (the entry point that allocates nothing, with the
library's own per-GPU scratch) against arcs_sample with a caller workspace:
the same ids, bit for bit, on two calls in a row, the second with a
smaller batch (the scratch keeps the first call's partials, which the
second must not read), and on a shape that needs no scratch."""

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from workloads import f32_to_bf16_bits, make_params

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def arcs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _batch(B, V, seed):
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 3.0, (B, V)).astype(np.float32)
    p = make_params(B, temperature=1.0)
    for b in range(B):
        kind = b % 4
        if kind == 0:
            p[b]["temperature"] = 0.0
        elif kind == 1:
            p[b]["temperature"] = float(rng.uniform(0.3, 1.5))
        elif kind == 2:
            p[b]["top_k"] = 50
            p[b]["top_p"] = 0.9
        # kind 3: temperature 1, no filter
    return f32_to_bf16_bits(z), p


@pytest.mark.parametrize("shapes", [((16, 129_280), (4, 129_280)), ((64, 50_000), (3, 8192)),
                                    ((300, 20_000), (5, 131_072))])
def test_noalloc_matches_the_workspace_entry_point(arcs, shapes):
    import torch
    for i, (B, V) in enumerate(shapes):
        bits, p = _batch(B, V, 1000 * i + B)
        logits = to_device_logits(bits, "bf16")
        params = arcs.params_to_device(p)
        need = arcs.workspace_bytes(B, V, arcs.DTYPE_BF16)
        assert need <= arcs.NOALLOC_SCRATCH_BYTES
        for step in (0, 1):
            out = torch.full((B,), -5, dtype=torch.int32, device="cuda")
            status = torch.full((B,), -5, dtype=torch.int32, device="cuda")
            arcs.sample_noalloc(logits, params, seed=77, step=step, out=out, out_status=status)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            ref_status = torch.empty(B, dtype=torch.int32, device="cuda")
            ref = arcs.sample(logits, params, seed=77, step=step, out_status=ref_status, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), (B, V, step)
            assert np.array_equal(status.cpu().numpy(), ref_status.cpu().numpy()), (B, V, step)
            assert (status.cpu().numpy() == 0).all()
