"""Writes tests/golden/hfqm_tiny.calib.hfq.hex (the package's bytes as hex text,
32 bytes a line) with the oracle's HFQM writer: two
tensors (K = 5 and K = 3), each a stored Hessian (the oracle's tril packing of a
seeded symmetric matrix) and its imatrix (the diagonal), under arch_id 7 and a
small JSON metadata object.  Run from the repository root:
    python tests/golden/make_hfqm_golden.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle                       # noqa: E402
import oracle.hfqm as hfqm          # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hfqm_tiny.calib.hfq.hex")


def entries():
    rng = np.random.default_rng(20260818)
    out = []
    for name, K in (("blk.0.attn_qkv", 5), ("blk.0.ffn_down", 3)):
        A = rng.standard_normal((K, K)).astype(np.float32)
        H = (A @ A.T).astype(np.float32)
        out.append((name + ".hessian", hfqm.QT_HESSIAN, (K, K), 0, oracle.pack_tril(H).tobytes()))
        out.append((name + ".imatrix", hfqm.QT_F32, (K,), 0, np.diag(H).astype(np.float32).tobytes()))
    return out


ARCH_ID = 7
METADATA = '{"producer":"golden","tensors":2}'


if __name__ == "__main__":
    import tempfile
    oracle.build()
    with tempfile.TemporaryDirectory() as d:
        tmp = os.path.join(d, "tiny.calib.hfq")
        hfqm.write(tmp, ARCH_ID, METADATA, entries())
        data = open(tmp, "rb").read()
    with open(OUT, "w") as f:
        for i in range(0, len(data), 32):
            f.write(data[i:i + 32].hex() + "\n")
    print(OUT, len(data), "bytes")
