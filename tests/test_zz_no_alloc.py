"""rtn_quantize_noalloc (the library's fixed per-device scratch in place of a
workspace, for callers that cannot allocate) against rtn_quantize_ex with a
caller workspace: identical codes, scales and qerr, over consecutive calls that
shrink, so that a call cannot lean on what an earlier one left in the scratch."""
import numpy as np
import pytest
import torch

import synthgen as g

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    m.lib()
    return m


def _both(gq, W, imp, G, flags, want_qerr=True):
    N, K = W.shape
    c1 = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    s1 = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.rtn_quantize_workspace_size(N, K, G), DEV)
    q1 = gq.rtn_quantize_ex(c1, s1, W, imp, G, flags, ws, want_qerr=want_qerr)
    c2 = torch.full((N, K // 2), 0xA5, dtype=torch.uint8, device=DEV)
    s2 = torch.full((N, K // G), -1.0, dtype=torch.float32, device=DEV)
    q2 = gq.rtn_quantize_noalloc(c2, s2, W, imp, G, flags, want_qerr=want_qerr)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert q1 == q2
    return q2


def test_noalloc_matches_workspace_call(gq):
    # 1: the attention shape's weights (10240 x 5120, G = 128), importance given
    wl = g.WORKLOADS["attn5120"]
    W = g.weights(wl, device=DEV)
    imp = (torch.exp(g.normal_tensor(3, g.S_S, (wl.K,), device=DEV)) ).float()
    assert gq.rtn_quantize_workspace_size(wl.N[0], wl.K, wl.group) <= gq.NOALLOC_SCRATCH_BYTES
    q_big = _both(gq, W, imp, wl.group, 0)
    assert 0.0 < q_big < 1.0
    # 2: smaller, NF4, no importance
    Ws = W[:300, :1024].contiguous()
    _both(gq, Ws, None, 64, gq.GQ_NF4)
    # 3: smaller still and ragged (the per-element kernel: K not a multiple of 8)
    Wr = g.uniform_weights(9, 33, 130, device=DEV)
    _both(gq, Wr, None, 2, 0)
    # 4: qerr not requested
    _both(gq, Wr[:5].contiguous(), None, 2, 0, want_qerr=False)


def test_noalloc_refuses_bad_arguments(gq):
    W = g.uniform_weights(1, 4, 64, device=DEV)
    c = torch.empty(4, 32, dtype=torch.uint8, device=DEV)
    s = torch.empty(4, 1, dtype=torch.float32, device=DEV)
    with pytest.raises(gq.GQError) as e:
        gq.rtn_quantize_noalloc(c, s, W, None, 48)                 # not a power of two
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    with pytest.raises(gq.GQError) as e:
        gq.rtn_quantize_noalloc(c, s, W, None, 64, 8)              # unknown flag bit
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    Wn = W.clone()
    Wn[1, 3] = float("nan")
    with pytest.raises(gq.GQError) as e:
        gq.rtn_quantize_noalloc(c, s, Wn, None, 64)
    assert e.value.status == gq.GQ_ERR_NONFINITE
    # the scratch keeps the last call's contents: the next good call still matches
    _both(gq, W, None, 64, 0)
