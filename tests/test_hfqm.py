"""HFQM calibration package (.calib.hfq): the library's writer and reader (host
code, no GPU) against the oracle's, the golden package, and the card's layout.

Pins from the pages (hipfire-calib-data, ".calib.hfq — HFQM calibration
package", tests/golden/pages_values.json "hfqm_layout"): the header is 32 bytes
and its six fields, at the widths the card lists, fill exactly those 32; a
tensor contributes two entries (496 tensors, 992 entries); a Hessian payload is
K*4 + K*(K-1)/2*2 bytes of quant_type 130, the tril blob.  The golden package
(tests/golden/hfqm_tiny.calib.hfq.hex) was written by
tests/golden/make_hfqm_golden.py with the oracle's writer only.
"""
import json
import os
import struct

import numpy as np
import pytest

import oracle.hfqm as ohf

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    m.lib()
    return m


def _golden_bytes():
    with open(os.path.join(GOLD, "hfqm_tiny.calib.hfq.hex")) as f:
        return bytes.fromhex("".join(line.strip() for line in f))


def _layout():
    return json.load(open(os.path.join(GOLD, "pages_values.json")))["hfqm_layout"]


def test_card_layout_pins(orc, gq, tmp_path):
    L = _layout()
    # magic 4 + version 4 + arch_id 4 + n_entries 4 + metadata_offset 8 + data_offset 8
    assert struct.calcsize("<4sIIIQQ") == L["header_bytes"] == ohf.HEADER.size
    # two entries per tensor: a package of L["tensors"] tiny tensors has L["entries"] entries
    ents = []
    for t in range(L["tensors"]):
        ents.append((f"t{t}.hessian", L["hessian_quant_type"], (1, 1), 0, b"\x00\x00\x80\x3f"))
        ents.append((f"t{t}.imatrix", 0, (1,), 0, b"\x00\x00\x80\x3f"))
    p = str(tmp_path / "many.calib.hfq")
    gq.hfqm_write(p, 0, "{}", ents)
    arch, meta, idx = gq.hfqm_read(p)
    assert len(idx) == L["entries"]
    raw = open(p, "rb").read()
    assert raw[:4] == L["magic"].encode() and struct.unpack_from("<I", raw, 4)[0] == L["version"]
    assert struct.unpack_from("<I", raw, 12)[0] == L["entries"]
    # the Hessian payload is the tril blob, K*4 + K*(K-1)/2*2 bytes
    for K in (1, 2, 5, 77, 5120):
        assert orc.tril_bytes(K) == K * 4 + K * (K - 1) // 2 * 2 == gq.hessian_tril_bytes(K)


def test_golden_read_by_library_and_oracle(gq, tmp_path):
    data = _golden_bytes()
    p = str(tmp_path / "golden.calib.hfq")
    open(p, "wb").write(data)
    arch, meta, idx = gq.hfqm_read(p)
    oarch, ometa, oents = ohf.read(p)
    assert arch == oarch == 7
    assert meta == ometa == '{"producer":"golden","tensors":2}'
    assert [e[0] for e in idx] == [e[0] for e in oents] == [
        "blk.0.attn_qkv.hessian", "blk.0.attn_qkv.imatrix", "blk.0.ffn_down.hessian", "blk.0.ffn_down.imatrix"]
    data_off = struct.unpack_from("<Q", data, 24)[0]
    off = data_off
    for i, (e, o) in enumerate(zip(idx, oents)):
        name, qt, shape, group, size, offset = e
        assert (qt, shape, group, size) == (o[1], o[2], o[3], len(o[4]))
        assert offset == off
        off += size
        assert gq.hfqm_read_payload(p, i, size).tobytes() == o[4]
    assert off == len(data)
    # the Hessian entries are K x K tril blobs, the imatrix entries K f32
    assert idx[0][1:4] == (130, (5, 5), 0) and idx[0][4] == 5 * 4 + 10 * 2
    assert idx[1][1:4] == (0, (5,), 0) and idx[1][4] == 5 * 4


def test_golden_written_by_library(gq, tmp_path):
    data = _golden_bytes()
    p = str(tmp_path / "g.calib.hfq")
    open(p, "wb").write(data)
    arch, meta, oents = ohf.read(p)
    q = str(tmp_path / "again.calib.hfq")
    gq.hfqm_write(q, arch, meta, oents)
    assert open(q, "rb").read() == data


def test_roundtrip_and_oracle_bytes(gq, tmp_path):
    rng = np.random.default_rng(3)
    ents = [
        ("模型.层.0.hessian", 130, (4, 4), 0, rng.integers(0, 256, 4 * 4 + 6 * 2, dtype=np.uint8).tobytes()),
        ("模型.层.0.imatrix", 0, (4,), 0, rng.standard_normal(4).astype(np.float32).tobytes()),
        ("empty", 0, (0,), 0, b""),
        ("four.dims", 7, (2, 3, 4, 5), 32, bytes(range(120))),
    ]
    meta = '{"note":"braces } and [ inside \\" strings","list":[{"a":1},{"b":[2,3]}]}'
    p, q = str(tmp_path / "lib.hfq"), str(tmp_path / "orc.hfq")
    gq.hfqm_write(p, 123456, meta, ents)
    ohf.write(q, 123456, meta, ents)
    assert open(p, "rb").read() == open(q, "rb").read()
    arch, m2, idx = gq.hfqm_read(p)
    assert (arch, m2) == (123456, meta)
    for i, (e, r) in enumerate(zip(ents, idx)):
        assert r[:4] == e[:4]
        assert gq.hfqm_read_payload(p, i, r[4]).tobytes() == e[4]
    # an empty package
    gq.hfqm_write(p, 0, "[]", [])
    assert gq.hfqm_read(p) == (0, "[]", [])


def _corrupt(data, off, raw):
    b = bytearray(data)
    b[off:off + len(raw)] = raw
    return bytes(b)


def test_malformed_packages(gq, tmp_path):
    data = _golden_bytes()
    meta_end = 32 + len('{"producer":"golden","tensors":2}')
    cases = {
        "magic": _corrupt(data, 0, b"HFQX"),
        "version": _corrupt(data, 4, struct.pack("<I", 2)),
        "count": _corrupt(data, 12, struct.pack("<I", 5)),
        "index_count": _corrupt(data, meta_end, struct.pack("<I", 3)),
        "metadata": _corrupt(data, 32, b"x"),
        "offsets": _corrupt(data, 24, struct.pack("<Q", len(data) + 1)),
        "truncated": data[:-3],
        "short_header": data[:20],
    }
    for name, raw in cases.items():
        p = str(tmp_path / f"{name}.hfq")
        open(p, "wb").write(raw)
        with pytest.raises(gq.GQError) as e:
            gq.hfqm_read(p)
        assert e.value.status == gq.GQ_ERR_IO, name
    with pytest.raises(gq.GQError) as e:
        gq.hfqm_read(str(tmp_path / "missing.hfq"))
    assert e.value.status == gq.GQ_ERR_IO


def test_write_argument_errors(gq, tmp_path):
    p = str(tmp_path / "x.hfq")
    for meta in ("", " {}", "{} ", "{}{}", '"text"', "{"):
        with pytest.raises(gq.GQError) as e:
            gq.hfqm_write(p, 0, meta, [])
        assert e.value.status == gq.GQ_ERR_INVALID_ARG, meta
    with pytest.raises(ValueError):
        gq.hfqm_write(p, 0, "{}", [("five", 0, (1, 1, 1, 1, 1), 0, b"1234")])
    with pytest.raises(gq.GQError) as e:
        gq.hfqm_write(p, 0, "{}", [("x" * 70000, 0, (1,), 0, b"1234")])
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    gq.hfqm_write(p, 0, "{}", [("ok", 0, (1,), 0, b"1234")])
    _, _, idx = gq.hfqm_read(p)
    with pytest.raises(gq.GQError) as e:
        gq.hfqm_read_payload(p, 0, 3)                  # destination smaller than the payload
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    with pytest.raises(gq.GQError) as e:
        gq.hfqm_read_payload(p, 1, 4)                  # no entry 1
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
