"""The HFQM package around the device path: a Hessian accumulated and packed on
the GPU goes into a package (with its imatrix, the stored exact diagonal), comes
back from the file, and unpacks on the GPU to exactly the matrix the unpacked
blob gives directly; the package bytes are the oracle writer's for the same
entries.  At the bench workload's size (K = 5120) and at K = 1024."""
import os

import numpy as np
import pytest
import torch

import oracle.hfqm as ohf
import synthgen as g

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


@pytest.mark.parametrize("wl_name", ["stored1024", "attn5120"])
def test_hfqm_roundtrip_through_device(gq, wl_name, tmp_path):
    wl = g.WORKLOADS[wl_name]
    K = wl.K
    X = g.x_chunk(wl, device=DEV)
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_accumulate(H, X)
    blob = torch.empty(gq.hessian_tril_bytes(K), dtype=torch.uint8, device=DEV)
    gq.hessian_pack_tril(blob, H)
    imat = blob[: 4 * K].view(torch.float32)
    name = f"blk.{wl_name}.proj"
    ents = [(name + ".hessian", gq.GQ_HFQM_HESSIAN, (K, K), 0, blob),
            (name + ".imatrix", gq.GQ_HFQM_F32, (K,), 0, imat)]
    p = str(tmp_path / "pkg.calib.hfq")
    gq.hfqm_write(p, 1, '{"workload":"%s","tokens":%d}' % (wl_name, wl.T), ents)
    arch, meta, idx = gq.hfqm_read(p)
    assert [e[0] for e in idx] == [name + ".hessian", name + ".imatrix"]
    assert idx[0][1:5] == (130, (K, K), 0, gq.hessian_tril_bytes(K))
    payload = gq.hfqm_read_payload(p, 0, idx[0][4])
    back = torch.from_numpy(payload).to(DEV)
    A = torch.empty(K, K, dtype=torch.float32, device=DEV)
    B = torch.empty(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_unpack_tril(A, blob)
    gq.hessian_unpack_tril(B, back)
    torch.cuda.synchronize()
    assert torch.equal(A.view(torch.int32), B.view(torch.int32))
    assert np.array_equal(gq.hfqm_read_payload(p, 1, 4 * K).view(np.float32), imat.cpu().numpy())
    q = str(tmp_path / "orc.calib.hfq")
    ohf.write(q, 1, meta, [(e[0], e[1], e[2], e[3], e[4].cpu().numpy().tobytes()) for e in ents])
    assert open(p, "rb").read() == open(q, "rb").read()
