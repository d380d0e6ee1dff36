"""Block *encoders* used by the tests to build blocks from chosen quants and scales.

Encoding is the inverse direction of what the oracle and the GPU library do
(decoding), written independently of both, so "decode(encode(params))" compared
with values computed straight from params pins the decoders to the format reading
stated in oracle/oracle.h. Also parses tests/golden/q4k_q8_0_blocks.txt.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q4k_q8_0_blocks.txt")
GOLDEN_Q6K = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q6k_blocks.txt")


def half_bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def pack_scales(sc, m) -> np.ndarray:
    """Sixteen 6-bit fields -> 12 bytes (the layout's bit placement, built field by field)."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    assert all(0 <= v < 64 for v in sc + m)
    s = [0] * 12
    for j in range(4):
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)        # sc[j] bits 0-5, sc[j+4] bits 4-5 on top
        s[j + 4] = m[j] | ((m[j + 4] >> 4) << 6)      # m[j] bits 0-5, m[j+4] bits 4-5 on top
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return np.array(s, dtype=np.uint8)


def pack_nibbles(q) -> np.ndarray:
    """256 quants (0..15) -> 128 bytes: byte 32g+l = q[64g+l] | q[64g+32+l] << 4."""
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 15
    out = np.zeros(128, dtype=np.uint8)
    for g in range(4):
        for l in range(32):
            out[32 * g + l] = q[64 * g + l] | (q[64 * g + 32 + l] << 4)
    return out


def q4k_block(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    blk = np.zeros(144, dtype=np.uint8)
    blk[0:2] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    blk[2:4] = np.array([dmin_bits], dtype=np.uint16).view(np.uint8)
    blk[4:16] = pack_scales(sc, m)
    blk[16:] = pack_nibbles(q)
    return blk


def q8_0_block(d_bits: int, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (32,) and q.min() >= -128 and q.max() <= 127
    blk = np.zeros(34, dtype=np.uint8)
    blk[0:2] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    blk[2:] = q.astype(np.int8).view(np.uint8)
    return blk


def q6k_block(d_bits: int, sc, q) -> np.ndarray:
    """Q6_K block from 16 int8 scales and 256 six-bit quants, built byte by byte:
    ql byte b of half h = b // 64 holds (low nibble) the low bits of the quant of
    weight 128h + 32(r // 32) + r % 32 and (high nibble) those of the weight 64
    further, r = b % 64; qh byte b of half h = b // 32 packs, two bits each from
    bit 0 up, the high bits of weights 128h + l, +32, +64, +96, l = b % 32."""
    sc = np.asarray(sc, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    assert sc.shape == (16,) and sc.min() >= -128 and sc.max() <= 127
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 63
    blk = np.zeros(210, dtype=np.uint8)
    for b in range(128):
        h, r = divmod(b, 64)
        first = 128 * h + 32 * (r // 32) + r % 32
        blk[b] = (q[first] & 15) | ((q[first + 64] & 15) << 4)
    for b in range(64):
        h, l = divmod(b, 32)
        v = 0
        for p in range(4):
            v |= (q[128 * h + 32 * p + l] >> 4) << (2 * p)
        blk[128 + b] = v
    blk[192:208] = sc.astype(np.int8).view(np.uint8)
    blk[208:210] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    return blk


def q6k_weights(d: float, sc, q) -> np.ndarray:
    """Weights straight from the parameters (no bytes involved)."""
    j = np.arange(256) // 16
    return d * np.asarray(sc, np.float64)[j] * (np.asarray(q, np.float64) - 32)


def golden_q6k() -> dict:
    """name -> dict(block=uint8[210], sum=float, w={index: value})."""
    fields: dict[str, dict[str, str]] = {}
    with open(GOLDEN_Q6K) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split("=", 1))
            name, attr = key.split(".")
            fields.setdefault(name, {})[attr] = val
    out = {}
    for name, fl in fields.items():
        ql = _rule(fl["ql_rule"], 128)
        qh = _rule(fl["qh_rule"], 64)
        assert ql.min() >= 0 and ql.max() <= 255 and qh.min() >= 0 and qh.max() <= 255
        blk = np.concatenate([ql.astype(np.uint8), qh.astype(np.uint8), _hex(fl["scales"]), _hex(fl["d"])])
        assert blk.size == 210
        w = {}
        for item in fl["w"].split():
            i, v = item.split(":")
            w[int(i)] = float(v)
        out[name] = {"block": blk, "sum": float(fl["sum"]), "w": w}
    return out


def q4k_weights(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Weights straight from the parameters (no bytes involved)."""
    j = np.arange(256) // 32
    return d * np.asarray(sc, np.float64)[j] * np.asarray(q, np.float64) - dmin * np.asarray(m, np.float64)[j]


def random_q4k_params(rng: np.random.Generator):
    d = float(np.float16(rng.uniform(0.001, 0.02)))
    dmin = float(np.float16(rng.uniform(0.001, 0.02)))
    sc = rng.integers(0, 64, 8)
    m = rng.integers(0, 64, 8)
    q = rng.integers(0, 16, 256)
    return d, dmin, sc, m, q


def _hex(s: str) -> np.ndarray:
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


def _rule(expr: str, n: int) -> np.ndarray:
    return np.array([eval(expr, {"__builtins__": {}}, {"i": i}) for i in range(n)], dtype=np.int64)


def golden() -> dict:
    """name -> dict(block=uint8 bytes, sum=float, w={index: value}, sc=, m=)."""
    fields: dict[str, dict[str, str]] = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split("=", 1))
            name, attr = key.split(".")
            fields.setdefault(name, {})[attr] = val
    out = {}
    for name, fl in fields.items():
        hdr = _hex(fl["header"])
        if "qs_rule" in fl:
            qs = _rule(fl["qs_rule"], 128)
            assert qs.min() >= 0 and qs.max() <= 255
            blk = np.concatenate([hdr, _hex(fl["scales"]), qs.astype(np.uint8)])
            assert blk.size == 144
        else:
            q = _rule(fl["q_rule"], 32)
            blk = np.concatenate([hdr, q.astype(np.int8).view(np.uint8)])
            assert blk.size == 34
        w = {}
        for item in fl["w"].split():
            i, v = item.split(":")
            w[int(i)] = float(v)
        ent = {"block": blk, "sum": float(fl["sum"]), "w": w}
        if "sc" in fl:
            ent["sc"] = [int(t) for t in fl["sc"].split()]
            ent["m"] = [int(t) for t in fl["m"].split()]
        out[name] = ent
    return out
