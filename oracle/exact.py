"""Independent brute force of the layer for tiny shapes: pure Python, exact integer arithmetic.

Test infrastructure only. It exists to pin ``oracle.moe`` and shares none of its code:

* FP4 values come from the integer map of the paper "DeepSeek-V4-Flash on AMD gfx90a" (section 6.1: E2M1 times two is one of
  0, +-1, +-2, +-3, +-4, +-6, +-8, +-12), not from the E2M1 table in ``oracle.formats``;
* E4M3 values come from the OCP bit fields as integers times 2^-9, and E4M3 encoding is a nearest
  search over all codes rather than arithmetic rounding;
* every dot product is an exact Python-integer sum, rounded to bf16 or fp32 by integer arithmetic;
* fp32 operations are Python float operations rounded to fp32 through ``struct`` (one rounding of an
  exact or fp64 result; for fp32 operands this equals the correctly rounded fp32 operation);
* the top-k is a full sort of (-score, id) tuples.

Scale: a few hundred thousand Python operations per (token, expert); meant for the tiny config.
"""
from __future__ import annotations

import math
import struct

EXP0 = 400  # values are held as integers times 2^-EXP0

_FP4_X2 = [0, 1, 2, 3, 4, 6, 8, 12]   # "DeepSeek-V4-Flash on AMD gfx90a", section 6.1


def fp4_int(nib: int) -> tuple[int, int]:
    """E2M1 nibble -> (integer, exponent) with value integer * 2^exponent."""
    v = _FP4_X2[nib & 7]
    return (-v if nib & 8 else v), -1


def e4m3_int(code: int) -> tuple[int, int]:
    """E4M3fn byte -> (integer, exponent); value = integer * 2^exponent."""
    if code & 0x7F == 0x7F:
        raise ValueError("E4M3 NaN")
    e, m = (code >> 3) & 15, code & 7
    v = m if e == 0 else (8 + m) << (e - 1)
    return (-v if code & 0x80 else v), -9


def bf16_int(bits: int) -> tuple[int, int]:
    """bf16 bit pattern -> (integer, exponent)."""
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        raise ValueError("bf16 inf/nan")
    v, ex = (m, -133) if e == 0 else (128 + m, e - 127 - 7)
    return (-v if bits & 0x8000 else v), ex


def f32_int(x: float) -> tuple[int, int]:
    """fp32-representable float -> (integer, exponent), exact."""
    fr = float(x).as_integer_ratio()
    num, den = fr
    ex = -(den.bit_length() - 1)
    return num, ex


def to_fixed(v: int, ex: int) -> int:
    return v << (ex + EXP0)


def round_fixed(S: int, bits: int, min_exp: int) -> float:
    """Round S * 2^-EXP0 to ``bits`` significant bits (ties to even), quantum at least 2^min_exp."""
    if S == 0:
        return 0.0
    sign = -1 if S < 0 else 1
    a = abs(S)
    lead = a.bit_length() - 1 - EXP0          # exponent of the leading bit
    q_exp = max(lead - (bits - 1), min_exp)    # quantum exponent
    shift = q_exp + EXP0
    if shift <= 0:
        return sign * math.ldexp(a, -EXP0)
    q, rem = a >> shift, a & ((1 << shift) - 1)
    half = 1 << (shift - 1)
    if rem > half or (rem == half and (q & 1)):
        q += 1
    return sign * math.ldexp(q, q_exp)


def to_bf16(S: int) -> float:
    r = round_fixed(S, 8, -133)
    if abs(r) >= 2.0 ** 128:
        return math.copysign(math.inf, r)
    return r


def to_f32(S: int) -> float:
    return round_fixed(S, 24, -149)


def f32(x: float) -> float:
    """Round a Python float to fp32 (RNE); finite values beyond the fp32 range become +-inf."""
    try:
        return struct.unpack("f", struct.pack("f", x))[0]
    except OverflowError:
        return math.copysign(math.inf, x)


def bf16_of_f32(x: float) -> float:
    """fp32 value -> bf16 RNE (exact integer route)."""
    if x == 0.0:
        return x
    v, ex = f32_int(x)
    return to_bf16(to_fixed(v, ex))


def bits_of_bf16(x: float) -> int:
    return struct.unpack("I", struct.pack("f", x))[0] >> 16


def e4m3_nearest(v: float) -> int:
    """Nearest E4M3fn code to |v| <= 448 by search over all codes; ties to the even code."""
    a = abs(v)
    best, bd = 0, None
    for c in range(0x7F):
        iv, ex = e4m3_int(c)
        d = abs(math.ldexp(iv, ex) - a)
        if bd is None or d < bd or (d == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, d
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    return best | sign


def qdq_row(vals: list[float]) -> tuple[list[int], list[int], list[tuple[int, int]]]:
    """QDQ one bf16 row per 32: returns codes, scale bytes and dequantized (int, exp) values."""
    codes, scales, deq = [], [], []
    inv448 = f32(1.0 / 448.0)
    for b in range(0, len(vals), 32):
        blk = vals[b:b + 32]
        amax = max(max(abs(v) for v in blk), f32(1e-4))
        v = f32(amax * inv448)
        fr, p = math.frexp(v)            # v = fr * 2^p, fr in [0.5, 1)
        E = p - 1 if fr == 0.5 else p    # ceil(log2 v)
        scales.append(127 + E)
        for x in blk:
            q = x / math.ldexp(1.0, E)
            q = max(-448.0, min(448.0, q))
            c = e4m3_nearest(q)
            codes.append(c)
            iv, ex = e4m3_int(c)
            deq.append((iv, ex + E))
    return codes, scales, deq


def dot_fixed(a: list[tuple[int, int]], b: list[tuple[int, int]]) -> int:
    return sum(to_fixed(ai * bi, ae + be) for (ai, ae), (bi, be) in zip(a, b))


def mxfp4_row(wrow, srow) -> list[tuple[int, int]]:
    out = []
    for j, byte in enumerate(wrow):
        sc = int(srow[(2 * j) // 32]) - 127
        for nib in (int(byte) & 15, int(byte) >> 4):
            v, ex = fp4_int(nib)
            out.append((v, ex + sc))
    return out


def fp8_row(wrow, srow_blocks) -> list[tuple[int, int]]:
    out = []
    for j, c in enumerate(wrow):
        v, ex = e4m3_int(int(c))
        out.append((v, ex + int(srow_blocks[j // 32]) - 127))
    return out


def swiglu_f32(g: float, u: float, rw: float | None) -> float:
    g = min(g, 10.0)
    u = max(-10.0, min(10.0, u))
    try:
        e = f32(math.exp(-g))
    except OverflowError:
        e = math.inf
    d = f32(1.0 + e)
    sg = f32(g / d)
    h = f32(sg * u)
    if rw is not None:
        h = f32(rw * h)
    return bf16_of_f32(h)


def expert(xdeq, rw, w1_rows, w3_rows, w2_rows):
    """One (token, expert): returns g, u, h16 (floats), hq codes, hs bytes, y (bf16 floats)."""
    g = [to_bf16(dot_fixed(xdeq, r)) for r in w1_rows]
    u = [to_bf16(dot_fixed(xdeq, r)) for r in w3_rows]
    h16 = [swiglu_f32(gi, ui, rw) for gi, ui in zip(g, u)]
    hq, hs, hdeq = qdq_row(h16)
    y = [to_bf16(dot_fixed(hdeq, r)) for r in w2_rows]
    return dict(g=g, u=u, h16=h16, hq=hq, hs=hs, y=y)


def layer(inp: dict, cfg) -> dict:
    """The whole layer by brute force (tiny shapes only)."""
    M, H, E, I, k = cfg.M, cfg.H, cfg.E, cfg.I, cfg.k
    x = inp["x"]
    xint = [[bf16_int(int(b)) for b in x[t]] for t in range(M)]
    W = [[f32_int(float(w)) for w in inp["gate_w"][e]] for e in range(E)]
    bias = [float(b) for b in inp["gate_b"]]
    res = dict(ids=[], rw=[], logits=[], scores=[], xq=[], xs=[], slot_y=[], out=[], g=[], u=[],
               h16=[], shared_y=[])
    dec = {}

    def weights(e):
        if e not in dec:
            dec[e] = ([mxfp4_row(inp["w1"][e][n], inp["s1"][e][n]) for n in range(I)],
                      [mxfp4_row(inp["w3"][e][n], inp["s3"][e][n]) for n in range(I)],
                      [mxfp4_row(inp["w2"][e][n], inp["s2"][e][n]) for n in range(H)])
        return dec[e]

    shared = None
    if "sw1" in inp:
        shared = ([fp8_row(inp["sw1"][n], inp["ss1"][n // 32]) for n in range(I)],
                  [fp8_row(inp["sw3"][n], inp["ss3"][n // 32]) for n in range(I)],
                  [fp8_row(inp["sw2"][n], inp["ss2"][n // 32]) for n in range(H)])
    for t in range(M):
        logits = [to_f32(dot_fixed(xint[t], W[e])) for e in range(E)]
        scores = [f32(math.sqrt(math.log1p(math.exp(l)))) for l in logits]
        sel = [f32(s + b) for s, b in zip(scores, bias)]
        ranked = sorted(range(E), key=lambda e: (-sel[e], e))
        ids = ranked[:k]
        w = [scores[e] for e in ids]
        acc = 0.0
        for wj in w:
            acc = f32(acc + wj)
        den = f32(acc + f32(1e-20))
        rw = [f32(f32(wj / den) * f32(cfg.route_scale)) for wj in w]
        xvals = [math.ldexp(v, ex) for v, ex in xint[t]]
        xq, xs, xdeq = qdq_row(xvals)
        slots = []
        for j, e in enumerate(ids):
            o = expert(xdeq, rw[j], *weights(e))
            slots.append(o)
        sh = expert(xdeq, None, *shared) if shared is not None else None
        acc = [0.0] * H
        for j in sorted(range(k), key=lambda j: ids[j]):
            acc = [f32(a + y) for a, y in zip(acc, slots[j]["y"])]
        if sh is not None:
            acc = [f32(a + y) for a, y in zip(acc, sh["y"])]
        out = [bf16_of_f32(a) for a in acc]
        res["ids"].append(ids); res["rw"].append(rw); res["logits"].append(logits)
        res["scores"].append(scores); res["xq"].append(xq); res["xs"].append(xs)
        res["slot_y"].append([o["y"] for o in slots]); res["g"].append([o["g"] for o in slots])
        res["u"].append([o["u"] for o in slots]); res["h16"].append([o["h16"] for o in slots])
        res["shared_y"].append(sh["y"] if sh is not None else None); res["out"].append(out)
    return res
