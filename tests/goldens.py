"""Readers for the hand-worked fixtures in tests/golden/ (see each file's header
for the page passages they are worked from)."""

from __future__ import annotations

import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def hex_f32(h: str) -> np.float32:
    return np.float32(struct.unpack("<f", struct.pack("<I", int(h, 16)))[0])


def _expand_bytes(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            b, n = t.split("*")
            out += [int(b, 16)] * int(n)
        else:
            out.append(int(t, 16))
    return bytes(out)


def pack_cases():
    cases, cur = [], None
    for line in _lines("pack_layout.txt"):
        head, _, rest = line.partition(" ")
        if head == "case":
            name, *kv = rest.split(" ")
            d = dict(x.split("=", 1) for x in kv)
            rows, K = int(d["rows"]), int(d["K"])
            w = np.full((rows, K), int(d["fill"]), dtype=np.int8)
            if d["set"]:
                for item in d["set"].split(","):
                    r, k, v = (int(t) for t in item.split(":"))
                    w[r, k] = v
            cur = {"name": name, "w": w, "ws": hex_f32(d["ws_hex"])}
            cases.append(cur)
        elif head == "bytes":
            cur["bytes"] = _expand_bytes(rest.split())
        elif head == "scale":
            cur["scale"] = bytes.fromhex(rest)
    return cases


def quantize_cases():
    cases, cur = [], None
    for line in _lines("quantize_vectors.txt"):
        head, _, rest = line.partition(" ")
        if head == "case":
            name, kv = rest.split(" ")
            K = int(kv.split("=")[1])
            cur = {"name": name, "K": K}
            cases.append(cur)
        elif head == "x_hex":
            lead = [hex_f32(t) for t in rest.split()]
            x = np.zeros(cur["K"], dtype=np.float32)
            x[: len(lead)] = lead
            cur["x"] = x
        elif head == "q":
            lead = [int(t) for t in rest.split()]
            q = np.zeros(cur["K"], dtype=np.int8)
            q[: len(lead)] = lead
            cur["q"] = q
        elif head == "scale_hex":
            cur["scale"] = hex_f32(rest)
        elif head == "row_sum":
            cur["row_sum"] = int(rest)
    return cases


def headroom():
    d = {}
    for line in _lines("headroom.txt"):
        k, v = line.split()
        d[k] = v
    return {
        "K": int(d["K"]),
        "ws": hex_f32(d["ws_hex"]),
        "scale": hex_f32(d["scale_hex"]),
        "row_sum": int(d["row_sum"]),
        "dot": int(d["dot"]),
        "y_bits": int(d["y_hex"], 16),
    }


def bias_add():
    """Hand-worked bias-add values (tests/golden/bias_add.txt), by key; *_hex
    entries are returned as binary32 bit patterns (int)."""
    out = {}
    for line in _lines("bias_add.txt"):
        k, v = line.split()
        out[k] = int(v, 16)
    return out


def i8s_mul_mat_add():
    """Hand-worked mul_mat_add cases (tests/golden/i8s_mul_mat_add.txt):
    (shared, cases) where shared holds OC, IC, N, w, ws, x, xs, acc and each
    case holds name, bias (f32), relu, q and scale_bits."""
    shared, cases, cur = {}, [], None
    for line in _lines("i8s_mul_mat_add.txt"):
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
            continue
        tgt = shared if cur is None else cur
        if key in ("OC", "IC", "N", "relu"):
            tgt[key] = int(vals[0])
        elif key in ("w", "x", "q"):
            tgt[key] = np.array([int(v) for v in vals], dtype=np.int8)
        elif key == "acc":
            tgt[key] = np.array([int(v) for v in vals], dtype=np.int32)
        elif key in ("ws_hex", "xs_hex"):
            tgt[key[:2]] = hex_f32(vals[0])
        elif key == "bias_hex":
            tgt["bias"] = np.array([hex_f32(v) for v in vals], dtype=np.float32)
        elif key == "scale_hex":
            tgt["scale_bits"] = int(vals[0], 16)
        else:
            raise ValueError(f"unknown key {key}")
    return shared, cases


def w8a8_rounding():
    """The hand-worked W8A8 rounding row (tests/golden/w8a8_rounding.txt):
    x (f32[16]), weight_q, act_q (int8[16]) and the scale (f32)."""
    d = {}
    for line in _lines("w8a8_rounding.txt"):
        key, *vals = line.split()
        d[key] = vals
    x = np.zeros(16, np.float32)
    x[: len(d["x_hex"])] = [hex_f32(v) for v in d["x_hex"]]
    wq = np.zeros(16, np.int8)
    wq[: len(d["weight_q"])] = [int(v) for v in d["weight_q"]]
    aq = np.zeros(16, np.int8)
    aq[: len(d["act_q"])] = [int(v) for v in d["act_q"]]
    return {"x": x, "weight_q": wq, "act_q": aq, "scale": hex_f32(d["scale_hex"][0])}
