"""Reference writer and reader of the HFQM calibration package (.calib.hfq).

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`: the tests and the golden
script use it; the product library never does, and it shares no code with the
library's own writer and reader (csrc/hfqm.hip).

The layout is the one the hipfire-calib-data dataset card gives under
".calib.hfq — HFQM calibration package", little-endian:

    header (32 bytes)  magic b"HFQM", version u32 (1), arch_id u32, n_entries u32,
                       metadata_offset u64, data_offset u64
    metadata           one self-delimited JSON value at metadata_offset
    index              n_entries u32, then per entry: name_len u16, name,
                       quant_type u8, n_dims u8, shape[n_dims] u32,
                       group_size u32, data_size u64
    payloads           concatenated in index order from data_offset

The card leaves two positions implicit; the reading taken here is the listing's
order with nothing in between: metadata right after the header, the index right
after the metadata value, the payloads right after the index.  Each tensor gives
two entries, "<name>.hessian" (quant_type 130, the Bf16TrilDiagF32 blob) and
"<name>.imatrix" (f32 values; the card names no type code for it, 0 is used).
"""
from __future__ import annotations

import json
import struct

MAGIC = b"HFQM"
HEADER = struct.Struct("<4sIIIQQ")          # magic, version, arch_id, n_entries, metadata_offset, data_offset
QT_F32 = 0
QT_HESSIAN = 130                             # Bf16TrilDiagF32


def write(path, arch_id: int, metadata, entries):
    """entries: (name, quant_type, shape, group_size, payload bytes) in index order.
    metadata: a JSON string (written as given) or an object (dumped compactly)."""
    meta = metadata if isinstance(metadata, str) else json.dumps(metadata, separators=(",", ":"))
    meta_b = meta.encode()
    index = bytearray(struct.pack("<I", len(entries)))
    for name, qt, shape, group, payload in entries:
        nb = name.encode()
        index += struct.pack("<H", len(nb)) + nb
        index += struct.pack("<BB", qt, len(shape))
        index += b"".join(struct.pack("<I", d) for d in shape)
        index += struct.pack("<IQ", group, len(payload))
    meta_off = HEADER.size
    data_off = meta_off + len(meta_b) + len(index)
    with open(path, "wb") as f:
        f.write(HEADER.pack(MAGIC, 1, arch_id, len(entries), meta_off, data_off))
        f.write(meta_b)
        f.write(index)
        for *_, payload in entries:
            f.write(bytes(payload))


def _json_end(buf: bytes, start: int) -> int:
    """End (exclusive) of the JSON object or array starting at buf[start]."""
    dec = json.JSONDecoder()
    text = buf[start:].decode("utf-8", errors="surrogateescape")
    value, end = dec.raw_decode(text)
    if not isinstance(value, (dict, list)):
        raise ValueError("metadata is not a JSON object or array")
    return start + len(text[:end].encode("utf-8", errors="surrogateescape"))


def read(path):
    """(arch_id, metadata JSON text, [(name, quant_type, shape, group_size, payload bytes)])."""
    with open(path, "rb") as f:
        buf = f.read()
    magic, version, arch_id, n, meta_off, data_off = HEADER.unpack_from(buf, 0)
    if magic != MAGIC or version != 1:
        raise ValueError("not an HFQM version 1 package")
    mend = _json_end(buf, meta_off)
    meta = buf[meta_off:mend].decode()
    pos = mend
    (n2,) = struct.unpack_from("<I", buf, pos)
    pos += 4
    if n2 != n:
        raise ValueError("index entry count differs from the header's")
    entries, off = [], data_off
    for _ in range(n):
        (nl,) = struct.unpack_from("<H", buf, pos)
        pos += 2
        name = buf[pos:pos + nl].decode()
        pos += nl
        qt, nd = struct.unpack_from("<BB", buf, pos)
        pos += 2
        shape = struct.unpack_from("<" + "I" * nd, buf, pos)
        pos += 4 * nd
        group, size = struct.unpack_from("<IQ", buf, pos)
        pos += 12
        entries.append((name, qt, tuple(shape), group, buf[off:off + size]))
        off += size
    if off > len(buf):
        raise ValueError("payloads run past the end of the file")
    return arch_id, meta, entries
