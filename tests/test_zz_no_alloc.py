"""attn_fwd_splitk_noalloc (the split-K workspace in the library's static device array) against
attn_fwd_splitk with a caller-owned workspace: the same kernels on the same inputs, so the
outputs must be bitwise equal.  Two calls in a row on the one array, the second smaller (and in
another dtype and depth), so the second runs over what the first left behind; then a size past
the array's limit is rejected with nothing written."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def _run_both(sa, q, k, v, P, mask=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    out_na = torch.full_like(qd, 7.0)
    lse_na = torch.full(qd.shape[:3], 7.0, dtype=torch.float32, device=DEV)
    sa.attn_fwd_splitk_noalloc(qd, kd, vd, P, out_na, lse_na, mask=md)
    _, _, out_ws, lse_ws = sa.splitk(qd, kd, vd, P, mask=md)
    torch.cuda.synchronize()
    return out_na, lse_na, out_ws, lse_ws


def test_noalloc_two_calls_match_caller_workspace(sa):
    # 1: the decode shape (B8 H32 Nq1 Nkv32768 D128 bf16) at P = 37: 4.9 MB of workspace
    q, k, v = si.decode_inputs()
    out_na, lse_na, out_ws, lse_ws = _run_both(sa, q, k, v, 37)
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws)
    rows = np.unique(si.rng_for(96, 0).integers(0, 256, 32))
    ref, ref_lse = oracle.attn_dense(q, k, v, rows=rows)
    o = out_na.reshape(256, -1)[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    assert np.abs(o - ref).max() <= 2e-2
    # 2: smaller, fp16, depth 64, several queries per head (the matrix-core producer) and a mask
    rng = si.rng_for(96, 1)
    q, k, v = (si.cast(x, "f16") for x in si.draw_qkv(rng, (2, 77, 3, 64), (2, 1000, 3, 64)))
    mask, _ = si.bernoulli_mask(rng, 77, 1000, 2)
    out_na, lse_na, out_ws, lse_ws = _run_both(sa, q, k, v, 5, mask)
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws)
    ref, ref_lse = oracle.attn_dense(q, k, v, mask=mask)
    assert np.abs(out_na.reshape(-1, 64).float().cpu().numpy() - ref).max() <= 5e-3
    empty = ref_lse == -np.inf
    assert empty.sum() == 2 * 2 * 3
    assert bool(torch.isneginf(lse_na.reshape(-1)[torch.from_numpy(np.nonzero(empty)[0]).to(DEV)]).all())


def test_noalloc_rejects_past_the_limit(sa):
    q = torch.zeros((1, 509, 1, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 3.0)
    with pytest.raises(sa.AttnError) as e:
        sa.attn_fwd_splitk_noalloc(q, q, q, 256, out)      # 256 * 509 * 129 * 4 B > 64 MiB
    assert e.value.code == 5
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
