"""switch_dispatch_noalloc, the dispatch for callers that cannot allocate
device memory, against switch_dispatch with a workspace: every output bit
for bit, over calls in a row whose sizes shrink, so whatever an earlier call
left in the shared scratch cannot reach a later result."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_order_amd as sw
import workloads
from tests.gpu_helpers import bits_to_dev, i32_dev, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(T, d, E, C):
    t = dict(position=torch.empty(T, dtype=torch.int32, device=DEV),
             keep=torch.empty(T, dtype=torch.uint8, device=DEV),
             counts=torch.empty(E, dtype=torch.int32, device=DEV),
             accepted=torch.empty(E, dtype=torch.int32, device=DEV),
             slot_token=torch.empty((E, C), dtype=torch.int32, device=DEV),
             buf=torch.empty((E, C, d), dtype=torch.bfloat16, device=DEV))
    for v in t.values():
        v.view(torch.uint8).fill_(0xFF)
    return t


def _case(T, d, E, C, seed, skew):
    """bf16 tokens and expert ids with a hot expert (ids drawn with weights
    proportional to 1 / (e + 1)^skew)."""
    rng = np.random.default_rng(seed)
    w = 1.0 / (np.arange(E) + 1.0) ** skew
    expert = rng.choice(E, size=T, p=w / w.sum()).astype(np.int32)
    return bits_to_dev(workloads.random_bf16((T, d), seed)), i32_dev(expert)


# (T, d, E, C, skew): the largest first, then smaller ones
CASES = [(65536, 64, 2048, 32, 0.3), (16384, 768, 128, 128, 1.0), (3000, 64, 37, 50, 1.5), (700, 128, 5, 100, 0.0),
         (1, 64, 3, 1, 0.0)]


def test_noalloc_dispatch_matches_workspace_dispatch():
    assert sw.switch_dispatch_noalloc_max_scratch_bytes() == 4 << 20
    for i, (T, d, E, C, skew) in enumerate(CASES):
        say(f"noalloc dispatch T={T} d={d} E={E} C={C}")
        x, expert = _case(T, d, E, C, 900 + i, skew)
        ref = _outputs(T, d, E, C)
        ws = torch.empty(max(256, sw.switch_dispatch_workspace_bytes(T, E)), dtype=torch.uint8, device=DEV)
        sw.switch_dispatch(x, expert, T, d, E, C, ref["position"], ref["keep"], ref["counts"], ref["accepted"],
                           ref["slot_token"], ref["buf"], ws)
        got = _outputs(T, d, E, C)
        sw.switch_dispatch_noalloc(x, expert, T, d, E, C, got["position"], got["keep"], got["counts"],
                                   got["accepted"], got["slot_token"], got["buf"])
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(ref[name].view(torch.uint8), got[name].view(torch.uint8)), (name, T, E)
        assert int(got["accepted"].sum()) == int(got["keep"].sum())
        del ref, got, ws


def test_noalloc_dispatch_rejects_sizes_above_its_scratch():
    T, E = 1 << 18, 4096   # 1024 tiles x 4096 experts x 4 bytes = 16 MiB
    with pytest.raises(sw.SwitchError) as ei:
        sw.switch_dispatch_noalloc(None, None, T, 64, E, 1, None, None, None, None, None, None)
    assert ei.value.status == sw.SWITCH_E_UNSUPPORTED
    assert "scratch" in str(ei.value)
