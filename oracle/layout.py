"""Independent packer/parser of the packed slot layout.

Written from the layout specification of the library (the header
``include/stepq.h`` states it field by field); it shares no code with the
library.  The pages fix only what a slot must hold: integer codes, FP16 row
and column scales and FP16 pivots (STEPQuant appendix D and F.1), or the
window's INT8 boundary, float32 smoothing/column scales and records
(LeapQuant notes Sec. 3.1 and 4.5).  The bit order is the library's choice.

Specification in brief:

* A slot holds the heads in order; head h starts at byte head_off[h], every
  head is padded to a multiple of 256 bytes and slot_bytes = head_off[H].
  All multi-byte values are little-endian.
* Tile-uniform code regions (uniform heads, STEP GDN heads including FP16
  pivot heads, the window's INT8 boundary) use a column-pair blocked order:
  row block rb = 32 rows, column pair p; the chunk (rb, p) holds value
  n = 2m + c = element (32 rb + m, 2 p + c) at bits [n b, n b + b) of a
  little-endian bit stream of 8 b bytes, cut into b/2 pieces of 16 bytes;
  piece q sits at byte (rb (b/2) (d_v/2) + q (d_v/2) + p) 16 of the region.
  KDA rows are stored row-major: a code row of d_v codes at b bits takes
  d_v*b/8 bytes, code j at bits [j*b, j*b+b).  Codes are b-bit two's
  complement; b = 16 stores binary16 values.
* uniform head: code region, then d_k FP16 row scales s.
* STEP GDN head (b in {2,4,6,8}): code region, d_k FP16 r, d_v FP16 c.
  Pivot head (b = 16): the region of FP16 values and nothing else.
* STEP KDA head: storage rows ordered by width (ascending, ties by key row),
  so FP16 pivot rows come last; then d_k FP16 r in storage order (0 for a
  pivot row) and d_v FP16 c.
* window head: int32 l at byte 0 (bytes 4..15 zero), float32 alpha[p] at
  byte 16, INT8 Z [d_k, d_v] (blocked order) at round_up(16 + 4p, 128), then
  float32 C[d_k],
  float32 B[d_v], float32 K~[p, d_k], float32 U[p, d_v]; with r compensator
  pairs, then FP16 K~c[r, d_k] and FP16 U~c[r, d_v].
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

PIVOT_BITS = 16


def round_up(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def row_bytes(d_v: int, bits: int) -> int:
    return 2 * d_v if bits == PIVOT_BITS else d_v * bits // 8


def kda_storage_order(row_bits: np.ndarray) -> np.ndarray:
    """perm[s] = key row held by storage row s (ascending width, then index)."""
    return np.array(sorted(range(len(row_bits)), key=lambda i: (int(row_bits[i]), i)),
                    dtype=np.int64)


def head_fields(desc: dict, h: int) -> Dict[str, int]:
    """Byte offsets of the fields of head h and its padded size."""
    mode, d_k, d_v = desc["mode"], desc["d_k"], desc["d_v"]
    f: Dict[str, int] = {}
    if mode == "uniform":
        b = int(desc["bits"])
        f["codes"] = 0
        f["s"] = d_k * row_bytes(d_v, b)
        end = f["s"] + 2 * d_k
    elif mode == "step" and desc["kind"] == "gdn":
        b = int(desc["head_bits"][h])
        f["codes"] = 0
        if b == PIVOT_BITS:
            end = d_k * row_bytes(d_v, b)
        else:
            f["r"] = d_k * row_bytes(d_v, b)
            f["c"] = f["r"] + 2 * d_k
            end = f["c"] + 2 * d_v
    elif mode == "step":
        rb = np.asarray(desc["row_bits"][h])
        f["codes"] = 0
        f["r"] = int(sum(row_bytes(d_v, int(b)) for b in rb))
        f["c"] = f["r"] + 2 * d_k
        end = f["c"] + 2 * d_v
    elif mode == "window":
        p = int(desc["p"])
        f["ell"] = 0
        f["alpha"] = 16
        f["Z"] = round_up(16 + 4 * p, 128)
        f["C"] = f["Z"] + d_k * d_v
        f["B"] = f["C"] + 4 * d_k
        f["K"] = f["B"] + 4 * d_v
        f["U"] = f["K"] + 4 * p * d_k
        r = int(desc.get("rank", 0))
        f["Kc"] = f["U"] + 4 * p * d_v
        f["Uc"] = f["Kc"] + 2 * r * d_k
        end = f["Uc"] + 2 * r * d_v
    else:
        raise ValueError(mode)
    f["used"] = end
    f["bytes"] = round_up(end, 256)
    return f


def slot_layout(desc: dict) -> dict:
    offs: List[int] = []
    off = 0
    fields = []
    for h in range(desc["heads"]):
        f = head_fields(desc, h)
        offs.append(off)
        fields.append(f)
        off += f["bytes"]
    return {"head_off": np.array(offs, dtype=np.int64), "slot_bytes": off, "fields": fields}


# ------------------------------------------------------------- bit streams
def pack_code_row(z: np.ndarray, bits: int) -> bytes:
    z = np.asarray(np.rint(z), dtype=np.int64)
    vals = z & ((1 << bits) - 1)
    bitarr = ((vals[:, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bitarr, bitorder="little").tobytes()


def unpack_code_row(buf: bytes, bits: int, n: int) -> np.ndarray:
    arr = np.unpackbits(np.frombuffer(buf, dtype=np.uint8), bitorder="little")
    arr = arr[: n * bits].reshape(n, bits).astype(np.int64)
    vals = (arr << np.arange(bits)).sum(-1)
    return np.where(vals >= (1 << (bits - 1)), vals - (1 << bits), vals).astype(np.float64)


# ------------------------------------------------------- blocked code region
def _field_bits(vals: np.ndarray, bits: int) -> np.ndarray:
    """b-bit fields of integer codes (two's complement) or binary16 values."""
    if bits == PIVOT_BITS:
        return np.asarray(vals, dtype=np.float64).astype("<f2").view("<u2").astype(np.int64)
    return np.asarray(np.rint(vals), dtype=np.int64) & ((1 << bits) - 1)


def _from_fields(f: np.ndarray, bits: int) -> np.ndarray:
    if bits == PIVOT_BITS:
        return f.astype("<u2").view("<f2").astype(np.float64)
    return np.where(f >= (1 << (bits - 1)), f - (1 << bits), f).astype(np.float64)


def pack_blocked(vals: np.ndarray, bits: int) -> bytes:
    """Column-pair blocked region of a d_k x d_v tile of codes (or FP16 values)."""
    d_k, d_v = vals.shape
    P = d_v // 2
    half = bits // 2                                  # pieces per chunk
    fields = _field_bits(vals, bits)
    out = bytearray(d_k * d_v * bits // 8)
    for rb in range(d_k // 32):
        for p in range(P):
            blk = fields[32 * rb:32 * rb + 32, 2 * p:2 * p + 2].reshape(-1)  # n = 2m + c
            bitarr = ((blk[:, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
            chunk = np.packbits(bitarr, bitorder="little").tobytes()
            for q in range(half):
                o = (rb * half * P + q * P + p) * 16
                out[o:o + 16] = chunk[16 * q:16 * q + 16]
    return bytes(out)


def parse_blocked(buf: bytes, bits: int, d_k: int, d_v: int) -> np.ndarray:
    P = d_v // 2
    half = bits // 2
    out = np.zeros((d_k, d_v))
    for rb in range(d_k // 32):
        for p in range(P):
            chunk = b"".join(buf[(rb * half * P + q * P + p) * 16:
                                 (rb * half * P + q * P + p) * 16 + 16] for q in range(half))
            arr = np.unpackbits(np.frombuffer(chunk, dtype=np.uint8), bitorder="little")
            arr = arr[:64 * bits].reshape(64, bits).astype(np.int64)
            f = (arr << np.arange(bits)).sum(-1)
            out[32 * rb:32 * rb + 32, 2 * p:2 * p + 2] = _from_fields(f, bits).reshape(32, 2)
    return out


def _f16_bytes(x: np.ndarray) -> bytes:
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype("<f2").tobytes()


def _f16(buf: bytes) -> np.ndarray:
    return np.frombuffer(buf, dtype="<f2").astype(np.float64)


# ------------------------------------------------------------ head packers
def pack_head(desc: dict, h: int, st: dict) -> bytes:
    """Bytes of head h from a state in key-row order (z, r, c, h / s /
    window fields)."""
    f = head_fields(desc, h)
    out = bytearray(f["bytes"])
    d_k, d_v = desc["d_k"], desc["d_v"]
    mode = desc["mode"]
    if mode == "uniform":
        b = int(desc["bits"])
        out[0:f["s"]] = pack_blocked(st["z"], b)
        out[f["s"]:f["s"] + 2 * d_k] = _f16_bytes(st["s"])
    elif mode == "step" and desc["kind"] == "gdn":
        b = int(desc["head_bits"][h])
        if b == PIVOT_BITS:
            out[0:2 * d_k * d_v] = pack_blocked(st["h"], PIVOT_BITS)
        else:
            out[0:f["r"]] = pack_blocked(st["z"], b)
            out[f["r"]:f["r"] + 2 * d_k] = _f16_bytes(st["r"])
            out[f["c"]:f["c"] + 2 * d_v] = _f16_bytes(st["c"])
    elif mode == "step":
        rbits = np.asarray(desc["row_bits"][h])
        perm = kda_storage_order(rbits)
        off = 0
        r_store = np.zeros(d_k)
        for s, i in enumerate(perm):
            b = int(rbits[i])
            n = row_bytes(d_v, b)
            if b == PIVOT_BITS:
                out[off:off + n] = _f16_bytes(st["h"][i])
            else:
                out[off:off + n] = pack_code_row(st["z"][i], b)
                r_store[s] = st["r"][i]
            off += n
        out[f["r"]:f["r"] + 2 * d_k] = _f16_bytes(r_store)
        out[f["c"]:f["c"] + 2 * d_v] = _f16_bytes(st["c"])
    elif mode == "window":
        p = int(desc["p"])
        out[0:4] = np.int32(st["ell"]).tobytes()
        out[f["alpha"]:f["alpha"] + 4 * p] = np.asarray(st["alpha"], "<f4").tobytes()
        out[f["Z"]:f["Z"] + d_k * d_v] = pack_blocked(st["Z"], 8)
        out[f["C"]:f["C"] + 4 * d_k] = np.asarray(st["C"], "<f4").tobytes()
        out[f["B"]:f["B"] + 4 * d_v] = np.asarray(st["B"], "<f4").tobytes()
        out[f["K"]:f["K"] + 4 * p * d_k] = np.asarray(st["kt"], "<f4").tobytes()
        out[f["U"]:f["U"] + 4 * p * d_v] = np.asarray(st["u"], "<f4").tobytes()
        r = int(desc.get("rank", 0))
        if r:
            out[f["Kc"]:f["Kc"] + 2 * r * d_k] = _f16_bytes(np.asarray(st["Kc"]).reshape(-1))
            out[f["Uc"]:f["Uc"] + 2 * r * d_v] = _f16_bytes(np.asarray(st["Uc"]).reshape(-1))
    return bytes(out)


def parse_head(desc: dict, h: int, buf: bytes) -> dict:
    """State of head h in key-row order from its bytes."""
    f = head_fields(desc, h)
    d_k, d_v = desc["d_k"], desc["d_v"]
    mode = desc["mode"]
    st: Dict[str, np.ndarray] = {}
    if mode == "uniform":
        b = int(desc["bits"])
        st["z"] = parse_blocked(buf[0:f["s"]], b, d_k, d_v)
        st["s"] = _f16(buf[f["s"]:f["s"] + 2 * d_k])
    elif mode == "step" and desc["kind"] == "gdn":
        b = int(desc["head_bits"][h])
        if b == PIVOT_BITS:
            st["h"] = parse_blocked(buf[0:2 * d_k * d_v], PIVOT_BITS, d_k, d_v)
            st["z"] = np.zeros((d_k, d_v))
            st["r"] = np.zeros(d_k)
            st["c"] = np.zeros(d_v)
        else:
            st["z"] = parse_blocked(buf[0:f["r"]], b, d_k, d_v)
            st["r"] = _f16(buf[f["r"]:f["r"] + 2 * d_k])
            st["c"] = _f16(buf[f["c"]:f["c"] + 2 * d_v])
            st["h"] = np.zeros((d_k, d_v))
    elif mode == "step":
        rbits = np.asarray(desc["row_bits"][h])
        perm = kda_storage_order(rbits)
        r_store = _f16(buf[f["r"]:f["r"] + 2 * d_k])
        z = np.zeros((d_k, d_v))
        hv = np.zeros((d_k, d_v))
        r = np.zeros(d_k)
        off = 0
        for s, i in enumerate(perm):
            b = int(rbits[i])
            n = row_bytes(d_v, b)
            if b == PIVOT_BITS:
                hv[i] = _f16(buf[off:off + n])
            else:
                z[i] = unpack_code_row(buf[off:off + n], b, d_v)
                r[i] = r_store[s]
            off += n
        st.update(z=z, r=r, h=hv, c=_f16(buf[f["c"]:f["c"] + 2 * d_v]))
    elif mode == "window":
        p = int(desc["p"])
        st["ell"] = int(np.frombuffer(buf[0:4], "<i4")[0])
        st["alpha"] = np.frombuffer(buf[f["alpha"]:f["alpha"] + 4 * p], "<f4").astype(np.float64)
        st["Z"] = parse_blocked(buf[f["Z"]:f["Z"] + d_k * d_v], 8, d_k, d_v)
        st["C"] = np.frombuffer(buf[f["C"]:f["C"] + 4 * d_k], "<f4").astype(np.float64)
        st["B"] = np.frombuffer(buf[f["B"]:f["B"] + 4 * d_v], "<f4").astype(np.float64)
        st["kt"] = np.frombuffer(buf[f["K"]:f["K"] + 4 * p * d_k], "<f4").astype(
            np.float64).reshape(p, d_k)
        st["u"] = np.frombuffer(buf[f["U"]:f["U"] + 4 * p * d_v], "<f4").astype(
            np.float64).reshape(p, d_v)
        r = int(desc.get("rank", 0))
        if r:
            st["Kc"] = _f16(buf[f["Kc"]:f["Kc"] + 2 * r * d_k]).reshape(r, d_k)
            st["Uc"] = _f16(buf[f["Uc"]:f["Uc"] + 2 * r * d_v]).reshape(r, d_v)
    return st


def pack_slot(desc: dict, states: List[dict]) -> bytes:
    lay = slot_layout(desc)
    out = bytearray(lay["slot_bytes"])
    for h, st in enumerate(states):
        b = pack_head(desc, h, st)
        o = int(lay["head_off"][h])
        out[o:o + len(b)] = b
    return bytes(out)


def parse_slot(desc: dict, buf: bytes) -> List[dict]:
    lay = slot_layout(desc)
    return [parse_head(desc, h, buf[int(lay["head_off"][h]):
                                    int(lay["head_off"][h]) + lay["fields"][h]["bytes"]])
            for h in range(desc["heads"])]


def state_from_encoding(desc: dict, h: int, enc: dict, row_bits: Optional[np.ndarray] = None
                        ) -> dict:
    """Keep only the stored fields of a quantizer result."""
    if desc["mode"] == "uniform":
        return {"z": enc["z"], "s": enc["s"]}
    if desc["mode"] == "window":
        keys = ("Z", "C", "B", "ell", "alpha", "kt", "u") + (
            ("Kc", "Uc") if int(desc.get("rank", 0)) else ())
        return {k: enc[k] for k in keys}
    return {"z": enc["z"], "r": enc["r"], "c": enc["c"], "h": enc["h"]}
