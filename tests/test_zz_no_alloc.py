"""The clip entry point that allocates nothing (qblk_clip_grad_norm_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point qblk_clip_grad_norm: the same kernels, so norm, scale and the clipped
gradients agree bit for bit, on two calls in a row (the second smaller,
so the static array holds the first call's partial sums when it starts)."""
import numpy as np
import pytest
import torch

from bwd_rmsnorm_qkv_amd import qblk
from bwd_rmsnorm_qkv_amd.runtime import byte_buffer, dev, empty
from gpu_util import announce, need_gpu

pytestmark = pytest.mark.gpu


def _case(rng, sizes, std):
    return [(rng.standard_normal(s) * std).astype(np.float32) for s in sizes]


@pytest.mark.parametrize("apply", [0, 1])
def test_clip_noalloc_matches_workspace_entry_point(apply):
    need_gpu()
    rng = np.random.default_rng(40 + apply)
    # first: 70 tensors (3 chunks), clipped; second: 5 small tensors, below the limit
    calls = [(_case(rng, [(1000,), (64, 130), (5001,), (3,), (300, 301)] * 14, 0.05), 1.0),
             (_case(rng, [(17,), (256,), (4096,), (4097,), (9,)], 1e-3), 1.0)]
    for i, (gs, max_norm) in enumerate(calls):
        announce(f"clip noalloc call {i}: {len(gs)} tensors, apply={apply}")
        ga = [dev(g) for g in gs]
        gb = [dev(g) for g in gs]
        na, sa, nb, sb = empty(1), empty(1), empty(1), empty(1)
        ws = byte_buffer(qblk.clip_workspace_size(ga))
        qblk.clip_grad_norm(ga, max_norm, apply, na, sa, ws)
        qblk.clip_grad_norm_noalloc(gb, max_norm, apply, nb, sb)
        torch.cuda.synchronize()
        assert torch.equal(na, nb) and torch.equal(sa, sb), (na.item(), nb.item(), sa.item(), sb.item())
        for a, b in zip(ga, gb):
            assert torch.equal(a, b)
        # and against the plain definition in fp64 on the host (norm within fp32 rounding)
        ref = np.sqrt(sum(float(np.sum(g.astype(np.float64) ** 2)) for g in gs))
        assert abs(nb.item() - ref) <= 1e-6 * ref
        assert (sb.item() < 1.0) == (ref > max_norm)


def test_clip_noalloc_rejects_too_many_tensors():
    need_gpu()
    g = empty(16)
    with pytest.raises(qblk.QblkError) as e:
        qblk.clip_grad_norm_noalloc([g] * 2049, 1.0, 0, empty(1), empty(1))
    assert e.value.code == qblk.QBLK_EINVAL
