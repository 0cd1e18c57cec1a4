"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate: its scratch is
the library's per-GPU static array) against moe_dispatch with a caller workspace,
through the C ABI: every output bit for bit, on two calls in a row, the second with a
smaller batch (the scratch keeps the first call's contents), plus the size limit."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_forward_amd import _binding as B
from sparse_mixture_experts_forward_amd.layer import workspace

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()


def _idx(rng, n, E, k, skew):
    """Distinct experts per token, experts 0..3 favoured when skew (so capacity bites)."""
    w = np.ones(E)
    if skew:
        w[:4] = 12.0
    w /= w.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(n)]).astype(np.int32)


def _outputs(n, k, E, d, dev):
    i32 = torch.int32
    return dict(expert_offsets=torch.full((E + 1,), -5, dtype=i32, device=dev),
                row_token=torch.full((max(n * k, 1),), -7, dtype=i32, device=dev),
                slot_row=torch.full((n, k), -9, dtype=i32, device=dev),
                kept_count=torch.full((E,), -3, dtype=i32, device=dev),
                n_dropped=torch.full((1,), -2, dtype=i32, device=dev),
                x_perm=torch.zeros((max(n * k, 1), d), dtype=torch.bfloat16, device=dev),
                row_weight=torch.full((max(n * k, 1),), -1.5, dtype=torch.float32, device=dev))


def _run(noalloc, idx, w, x, E, cap):
    n, k = idx.shape
    o = _outputs(n, k, E, x.shape[1], DEV)
    args = (idx, E, cap, x, o["expert_offsets"], o["row_token"], o["slot_row"], o["kept_count"],
            o["n_dropped"], o["x_perm"])
    if noalloc:
        B.moe_dispatch_noalloc(*args, topk_w=w, row_weight=o["row_weight"])
    else:
        ws = workspace(B.moe_dispatch_workspace_size(n, k, E), DEV)
        B.moe_dispatch(*args, ws, topk_w=w, row_weight=o["row_weight"])
    torch.cuda.synchronize()
    return {key: t.cpu() for key, t in o.items()}


@pytest.mark.parametrize("E,k,cap", [(64, 2, 40), (160, 6, -1), (512, 8, 3)])
def test_noalloc_dispatch_matches_workspace_dispatch(E, k, cap):
    rng = np.random.default_rng(E + k)
    d = 256
    for n in (4096, 777):  # the second call is smaller
        idx = torch.from_numpy(_idx(rng, n, E, k, cap >= 0)).to(DEV)
        w = torch.from_numpy(rng.random((n, k)).astype(np.float32)).to(DEV)
        x = torch.randn((n, d), device=DEV).to(torch.bfloat16)
        ref = _run(False, idx, w, x, E, cap)
        got = _run(True, idx, w, x, E, cap)
        for key in ref:
            if ref[key].dtype == torch.bfloat16:
                assert torch.equal(got[key].view(torch.int16), ref[key].view(torch.int16)), (n, key)
            else:
                assert torch.equal(got[key], ref[key]), (n, key)
        kept = int(ref["expert_offsets"][-1])
        assert kept == int(ref["kept_count"].sum()) and kept > 0


def test_noalloc_dispatch_refuses_batches_beyond_its_scratch():
    L = B.lib()
    fake = 4096  # never dereferenced: the size check fails before any device work
    n, k, E = 1 << 22, 16, 512
    assert B.moe_dispatch_workspace_size(n, k, E) > B.MOE_NOALLOC_SCRATCH_BYTES
    st = L.moe_dispatch_noalloc(None, fake, n, k, E, -1, None, 0, 0, fake, fake, fake, None,
                                None, None, None, None)
    assert st == B.MOE_ERR_UNSUPPORTED
    assert "scratch" in L.moe_last_error().decode()
    # the largest expert count at a batch that fits
    assert B.moe_dispatch_workspace_size(65536, 8, 512) <= B.MOE_NOALLOC_SCRATCH_BYTES
