"""Brute-force reference for the oracle's pins: pure Python on tiny inputs,
every sum a correctly rounded math.fsum, float64 sqrt / exp / log, each
output rounded once to float32 (through numpy). Shares nothing with the
oracle's C code; the definitions are the textbook ones the oracle states."""
import math

import numpy as np


def _f32(v):
    return float(np.float32(v))


def rmsnorm(x, w, eps):
    out = []
    for row in x:
        row = [float(v) for v in row]
        ms = math.fsum(v * v for v in row) / len(row)
        d = math.sqrt(ms + float(np.float32(eps)))
        out.append([_f32(v * float(wc) / d) for v, wc in zip(row, w)])
    return np.array(out, np.float32)


def row_sum(x):
    return np.array([_f32(math.fsum(float(v) for v in row)) for row in x], np.float32)


def softmax(x):
    out = []
    for row in x:
        row = [float(v) for v in row]
        m = max(row)
        e = [math.exp(v - m) for v in row]
        z = math.fsum(e)
        out.append([_f32(v / z) for v in e])
    return np.array(out, np.float32)


def layernorm(h, gamma, beta, eps):
    out = []
    for row in h:
        row = [float(v) for v in row]
        n = len(row)
        mean = math.fsum(row) / n
        var = math.fsum((v - mean) ** 2 for v in row) / n
        d = math.sqrt(var + float(np.float32(eps)))
        out.append([_f32((v - mean) / d * float(g) + float(b)) for v, g, b in zip(row, gamma, beta)])
    return np.array(out, np.float32)


def residual_layernorm(x, r, gamma, beta, eps):
    h = (np.asarray(x, np.float32) + np.asarray(r, np.float32)).astype(np.float32)
    return layernorm(h, gamma, beta, eps), h


def cross_entropy(x, targets):
    out = []
    for row, t in zip(x, targets):
        row = [float(v) for v in row]
        if not 0 <= int(t) < len(row):
            out.append(float("nan"))
            continue
        m = max(row)
        z = math.fsum(math.exp(v - m) for v in row)
        out.append(_f32(math.log(z) + m - row[int(t)]))
    return np.array(out, np.float32)
