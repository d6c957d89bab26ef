"""moe_permute_noalloc (the permutation on the library's static scratch, for
callers that cannot allocate) against moe_permute with a caller workspace,
through the C ABI: bit-exact on every output array (integer work), on calls
in a row that reuse the scratch, the later ones with smaller inputs, plus the
oracle's counting sort; and the size limit rejected before any launch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _outputs(T, E, k, cuda):
    return (torch.full((E,), -7, dtype=torch.int32, device=cuda),
            torch.full((E + 1,), -7, dtype=torch.int32, device=cuda),
            torch.full((T * k,), -7, dtype=torch.int32, device=cuda),
            torch.full((T, k), -7, dtype=torch.int32, device=cuda))


# larger first, then smaller: the second call finds the first one's contents
# in the scratch array
CASES = [(4096, 512, 8), (300, 64, 4), (700, 1024, 16), (1, 4, 1)]


def test_noalloc_permute_matches_workspace_permute(cuda):
    for i, (T, E, k) in enumerate(CASES):
        idx = _routing(T, E, k, 100 + i)
        t_idx = torch.from_numpy(idx).to(cuda)
        ref = _outputs(T, E, k, cuda)
        ws = torch.empty(moe.moe_workspace_bytes(1, T, 64, 64, E, k, 64), dtype=torch.uint8,
                         device=cuda)
        moe.moe_permute(t_idx, E, *ref, ws)
        got = _outputs(T, E, k, cuda)
        U.log(f"[no-alloc permute] call {i}: T={T} E={E} k={k}")
        moe.moe_permute_noalloc(t_idx, E, *got)
        torch.cuda.synchronize()
        want = oracle.permute(idx, E)
        for n, a, b in zip(("expert_counts", "expert_offsets", "row_token", "assign_row"), got, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=n)
            np.testing.assert_array_equal(a.cpu().numpy().reshape(want[n].shape), want[n],
                                          err_msg=n)


def test_noalloc_permute_empty_and_limit(cuda):
    E = 16
    counts, offsets, _, _ = _outputs(0, E, 2, cuda)
    empty = torch.empty(0, dtype=torch.int32, device=cuda)
    moe.moe_permute_noalloc(torch.empty((0, 2), dtype=torch.int32, device=cuda), E, counts,
                            offsets, empty, empty)
    torch.cuda.synchronize()
    assert (counts == 0).all() and (offsets == 0).all()
    # 2 * ceil(T / 256) * E int32 beyond the 2^21 of the static array: rejected
    T, E, k = 600_000, 512, 1
    idx = torch.zeros((T, k), dtype=torch.int32, device=cuda)
    outs = _outputs(T, E, k, cuda)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_permute_noalloc(idx, E, *outs)
    assert ei.value.code == -2
    torch.cuda.synchronize()
    assert (outs[0] == -7).all() and (outs[2] == -7).all()   # nothing was launched
