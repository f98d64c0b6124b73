"""Readers for the hand-derived text fixtures under tests/golden/."""
import configparser
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODES = {"DELTA": 0, "LITERAL": 1, "OFF": 2}


def load_ini(name):
    cp = configparser.ConfigParser(inline_comment_prefixes=None)
    cp.read(os.path.join(GOLDEN, name))
    return {sec: dict(cp[sec]) for sec in cp.sections()}


def floats(s):
    return np.array([float(v) for v in s.split()], dtype=np.float32)


def hexbytes(s):
    return np.array([int(v, 16) for v in s.split()], dtype=np.uint8)


def ints(s):
    return np.array([int(v) for v in s.split()], dtype=np.int64)


def hexwords(s, dtype):
    return np.array([int(v, 16) for v in s.split()], dtype=dtype)


def to_bf16_bits(values):
    """Exact fp32 -> bf16 bit patterns for values known to be representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "fixture value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)
