"""The allocation-free selection (tg_topk_select_noalloc) against the
workspace-taking tg_topk_select, through the C ABI: identical kept indices and
status flags (bit for bit) on two calls in a row that both use the library's
scratch, the second on a smaller batch, and against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import say
from learned_token_pruning_post_amd import binding as tg
from learned_token_pruning_post_amd.workloads import scores_with_ties

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.lib()  # raises loudly if the HIP library is missing


def _case(seed, N, K, F):
    rng = np.random.default_rng(seed)
    T_in = sum(N)
    cu_in = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    s = scores_with_ties(seed, T_in, 17)
    mask = np.zeros(T_in, np.uint8)
    for b in range(len(N)):
        f = min(F, N[b])
        mask[cu_in[b + 1] - f:cu_in[b + 1]] = 1  # forced tail
    s[cu_in[0] + rng.choice(N[0], 30, replace=False)] = np.nan
    return s, mask, cu_in, cu_k


def _both(s, mask, cu_in, cu_k, max_n):
    dev = "cuda"
    B = len(cu_in) - 1
    T = int(cu_k[-1])
    d_s = torch.from_numpy(s).to(dev)
    d_m = torch.from_numpy(mask).to(dev)
    d_ci = torch.from_numpy(cu_in).to(dev)
    d_ck = torch.from_numpy(cu_k).to(dev)
    need = tg.lib().tg_topk_select_workspace_size(B, s.size, max_n)
    assert 0 < need <= tg.SELECT_NOALLOC_SCRATCH_BYTES  # the call runs on the scratch
    # existing entry point, workspace from the caller
    kept_ws = torch.full((T,), -7, dtype=torch.int32, device=dev)
    st_ws = torch.full((B,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    tg.topk_select(d_s, d_m, d_ci, d_ck, T, max_n, kept=kept_ws, status=st_ws, ws=ws)
    # allocation-free entry point
    kept_na = torch.full((T,), -9, dtype=torch.int32, device=dev)
    st_na = torch.full((B,), -9, dtype=torch.int32, device=dev)
    tg.topk_select_noalloc(d_s, d_m, d_ci, d_ck, T, max_n, kept_na, st_na)
    torch.cuda.synchronize()
    return (kept_ws.cpu().numpy(), st_ws.cpu().numpy(), kept_na.cpu().numpy(), st_na.cpu().numpy())


def test_noalloc_select_matches_workspace_select_twice():
    calls = [
        ("first", 71, [70001, 45000, 9000], [6000, 45000, 700], 512, 70001),
        ("second, smaller", 72, [40000], [3000], 256, 40000),
        # sequences of at most 32768 tokens (one chunk size), then a smaller call
        ("third, short sequences", 73, [30000, 2000, 9000], [3000, 500, 9000], 128, 30000),
        ("fourth, smaller", 74, [5000], [700], 64, 5000),
    ]
    for what, seed, N, K, F, max_n in calls:
        print("noalloc select:", what, "N", N, "K", K, "max_n", max_n, flush=True)
        s, mask, cu_in, cu_k = _case(seed, N, K, F)
        kept_ws, st_ws, kept_na, st_na = _both(s, mask, cu_in, cu_k, max_n)
        assert np.array_equal(st_na, st_ws), what
        assert np.array_equal(kept_na, kept_ws), what
        ref, flags = O.topk_select(s, mask, cu_in, cu_k)
        assert np.array_equal(st_na, flags.astype(np.int32)), what
        assert np.array_equal(kept_na, ref.astype(np.int32)), what
        say("  %s call: %d kept, status %s, equal to the workspace call and the oracle"
            % (what, kept_na.size, st_na.tolist()))


def test_noalloc_select_rejects_oversized_batch():
    """Beyond the scratch size the call fails synchronously, before any launch."""
    dev = "cuda"
    B, n = 200, 40000
    s = torch.zeros(B * n, dtype=torch.float32, device=dev)
    cu = torch.arange(0, B + 1, dtype=torch.int32, device=dev) * n
    ck = torch.arange(0, B + 1, dtype=torch.int32, device=dev) * 10
    kept = torch.empty(B * 10, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    with pytest.raises(tg.TokenGateError) as e:
        tg.topk_select_noalloc(s, None, cu, ck, B * 10, n, kept, st)
    assert e.value.status == 3  # TG_ERR_WORKSPACE
