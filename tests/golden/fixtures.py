"""Readers for the hand-written fixtures in this folder (plain text)."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _lines(name):
    with open(os.path.join(HERE, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                yield ln.split()


def q2k_blocks():
    """{name: (bytes uint8[84], {i: value})}"""
    out, cur = {}, None
    for tok in _lines("q2k_blocks.txt"):
        if tok[0] == "block":
            cur = tok[1]
            out[cur] = [None, {}]
        elif tok[0] == "bytes":
            out[cur][0] = np.array([int(b, 16) for b in tok[1:]], np.uint8)
        elif tok[0] == "expect":
            out[cur][1][int(tok[1])] = float(tok[2])
    return {k: (v[0], v[1]) for k, v in out.items()}


def vq2_row():
    cb = np.zeros((256, 4), np.int8)
    d, idx, exp = None, np.zeros(128, np.uint8), {}
    for tok in _lines("vq2_row.txt"):
        if tok[0] == "cb":
            cb[int(tok[1])] = [int(v) for v in tok[2:6]]
        elif tok[0] == "d":
            d = np.array([int(v, 16) for v in tok[1:]], np.uint16)
        elif tok[0] == "idx_fill":
            idx[int(tok[1]):int(tok[2])] = int(tok[3])
        elif tok[0] == "expect":
            exp[int(tok[1])] = float(tok[2])
    return cb, d, idx, exp


def mxfp4_row():
    vals = scales = None
    exp = {}
    for tok in _lines("mxfp4_row.txt"):
        if tok[0] == "bytes":
            vals = np.array([int(b, 16) for b in tok[1:]], np.uint8)
        elif tok[0] == "scales":
            scales = np.array([int(b, 16) for b in tok[1:]], np.uint8)
        elif tok[0] == "expect":
            exp[int(tok[1])] = float(tok[2])
    return vals, scales, exp


def splitmix64_vectors():
    return [(int(a, 16), int(b, 16)) for a, b in _lines("splitmix64.txt")]
