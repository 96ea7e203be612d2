"""The routed-MoE FFN layer, step by step, on the CPU (test infrastructure only).

Follows the page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)":
section 2 "Official semantics" (quantized linear, activation QDQ, gate, expert, MoE)
and section 4 "Kernel contract" (the per-(token, slot) math of the routed expert).

Precision: every linear output is the exact dot product of exactly decoded values, rounded once to
bf16 (RNE). NumPy's fp64 BLAS is exact here because every product is exact in fp64 and the partial
sums stay inside fp64's 53 bits for these formats and ranges (pinned against the brute force in
``oracle.exact``). The steps the page fixes in fp32 (router logits, scores, normalisation, SwiGLU) are
emulated in fp32 with correctly rounded operations.

Readings of open points (where the pages leave a step open, the plainest reading the rest supports):
* top-k order: descending selection score, ties to the lower expert id;
* normalisation: fp32 sum of the k weights in slot order, plus 1e-20, IEEE fp32 division, times the
  route scale;
* SwiGLU: fp32 chain g / (1 + exp(-g)) * u, then times the route weight, exp correctly rounded;
* clamps apply to the bf16-rounded g and u.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

TIE_WINDOW = 1e-6
QDQ_BLOCK = 32
AMAX_FLOOR = np.float32(1e-4)
INV_448 = np.float32(1.0 / 448.0)


# ----------------------------------------------------------------------------------------------
# router (section 2, "Gate")
# ----------------------------------------------------------------------------------------------
def router_logits(x_bits: np.ndarray, gate_w: np.ndarray) -> np.ndarray:
    """fp32 gate logits l[t, e] = fp32(sum_h x[t, h] * W[e, h]) on the raw (un-QDQ'd) bf16 x.

    Products of a bf16 and an fp32 value are exact in fp64; the fp64 sum is rounded once to fp32.
    gate_temp is 1.0 (identity). Pinned by the brute force (exact integer sum, one rounding).
    """
    x = F.bf16_from_bits(x_bits)
    return F.f32(x @ gate_w.astype(np.float64).T)


def router_scores(logits: np.ndarray) -> np.ndarray:
    """s = fp32(sqrt(softplus(l))), softplus = log(1 + exp(l)) evaluated in fp64."""
    l64 = logits.astype(np.float64)
    return F.f32(np.sqrt(np.log1p(np.exp(l64))))


def route(x_bits: np.ndarray, gate_w: np.ndarray, gate_b: np.ndarray, k: int,
          route_scale: float) -> dict:
    """Gate: scores, biased top-k, gathered and normalised route weights (section 2, "Gate").

    ``sel = fp32(s + bias)`` selects only; ``ids`` are the k largest ``sel`` in descending order,
    ties to the lower expert id. ``w = s[ids]``; ``rw = fp32(fp32(w / fp32(sum(w) + 1e-20)) * scale)``
    with the fp32 sum taken in slot order ((w0 + w1) + w2) + ...

    Also returns ``tie``: a token is flagged when its k-th and (k+1)-th selection scores, or two of
    its neighbouring selected scores, are within 1e-6 (a set or order decided by fp32 noise).
    Pinned by a full-sort brute force and by the sum-to-scale invariant.
    """
    logits = router_logits(x_bits, gate_w)
    s = router_scores(logits)
    sel = F.f32(s.astype(np.float64) + gate_b.astype(np.float64))
    M, E = sel.shape
    # stable sort on (-sel, id): descending score, ties to the lower id
    order = np.lexsort((np.broadcast_to(np.arange(E), (M, E)), -sel.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    w = np.take_along_axis(s, ids, axis=1)
    acc = np.zeros(M, dtype=np.float32)
    for j in range(k):
        acc = (acc + w[:, j]).astype(np.float32)
    denom = (acc + np.float32(1e-20)).astype(np.float32)
    rw = (w / denom[:, None]).astype(np.float32)
    rw = (rw * np.float32(route_scale)).astype(np.float32)
    srt = np.take_along_axis(sel, order, axis=1).astype(np.float64)
    gaps = np.abs(np.diff(srt[:, : min(k + 1, E)], axis=1))
    tie = np.any(gaps <= TIE_WINDOW, axis=1) if gaps.size else np.zeros(M, dtype=bool)
    return dict(logits=logits, scores=s, sel=sel, ids=ids, rw=rw, tie=tie)


# ----------------------------------------------------------------------------------------------
# activation QDQ (section 2, "Quantized linear": act_quant per 32 with a ue8m0 scale)
# ----------------------------------------------------------------------------------------------
def qdq_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """E with s = 2^E = 2^ceil(log2(fp32(max(amax, 1e-4) * fp32(1/448)))), taken from the fp32 bits.

    Pinned exhaustively over every finite bf16 amax against exact rational arithmetic.
    """
    a = np.maximum(np.asarray(amax, dtype=np.float32), AMAX_FLOOR)
    v = (a * INV_448).astype(np.float32)
    bits = v.view(np.uint32).astype(np.int64)
    e = ((bits >> 23) & 0xFF) - 127
    mant = bits & 0x7FFFFF
    return (e + (mant != 0)).astype(np.int64)


def act_qdq(vals: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """QDQ bf16 rows per 32 consecutive columns.

    ``vals``: fp64 array [R, n] of bf16-exact values, n a multiple of 32. Returns the E4M3 codes
    [R, n], the E8M0 scale bytes [R, n/32] and the dequantized values ``q * s`` (exact in bf16).
    ``q = e4m3_rne(clamp(x / s, -448, 448))``.
    """
    R, n = vals.shape
    blocks = vals.reshape(R, n // QDQ_BLOCK, QDQ_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    E = qdq_scale_exponent(amax)
    s = np.ldexp(1.0, E)[:, :, None]
    q = np.clip(blocks / s, -F.E4M3_MAX, F.E4M3_MAX)
    codes = F.e4m3_encode_rne(q)
    deq = F.e4m3_decode(codes) * s
    scale_bytes = (E + 127).astype(np.uint8)
    return codes.reshape(R, n), scale_bytes, deq.reshape(R, n)


# ----------------------------------------------------------------------------------------------
# expert FFN (section 2, "Expert"; section 4, math per (t, j))
# ----------------------------------------------------------------------------------------------
def swiglu_f32(g: np.ndarray, u: np.ndarray, rw: np.ndarray | None) -> np.ndarray:
    """The fp32 value h = rw * ((g / (1 + exp(-g))) * u) with the clamps u in [-10, 10], g <= 10.

    g and u are bf16 values; every operation is an fp32 operation (exp correctly rounded);
    ``rw`` (one per row) is None for the shared expert (no route weight). Returns an fp32 array.
    """
    g32 = np.minimum(g, 10.0).astype(np.float32)
    u32 = np.clip(u, -10.0, 10.0).astype(np.float32)
    with np.errstate(over="ignore"):
        e = F.f32(np.exp(-g32.astype(np.float64)))
    d = (np.float32(1.0) + e).astype(np.float32)
    sg = (g32 / d).astype(np.float32)
    h = (sg * u32).astype(np.float32)
    if rw is not None:
        h = (np.asarray(rw, dtype=np.float32)[:, None] * h).astype(np.float32)
    return h


def swiglu(g: np.ndarray, u: np.ndarray, rw: np.ndarray | None) -> np.ndarray:
    """h16 = bf16(swiglu_f32(g, u, rw)) (RNE), returned as fp64 values."""
    return F.bf16_rne(swiglu_f32(g, u, rw).astype(np.float64))


def expert_ffn(xhat: np.ndarray, rw: np.ndarray | None, w1: np.ndarray, w3: np.ndarray,
               w2: np.ndarray) -> dict:
    """One expert on R rows of QDQ'd activations.

    ``xhat`` fp64 [R, H] (exact q*s values), ``w1``/``w3`` fp64 [I, H], ``w2`` fp64 [H, I] (decoded).
    g = bf16(x w1^T), u = bf16(x w3^T); h16 = swiglu; (h_q, h_s) = QDQ(h16); y = bf16(h_hat w2^T).
    """
    g = F.bf16_rne(xhat @ w1.T)
    u = F.bf16_rne(xhat @ w3.T)
    h16 = swiglu(g, u, rw)
    hq, hs, hhat = act_qdq(h16)
    y = F.bf16_rne(hhat @ w2.T)
    return dict(g=g, u=u, h16=h16, hq=hq, hs=hs, y=y)


class ExpertWeights:
    """Decoded weights of the routed experts, decoded lazily per expert.

    ``arm="packed"`` decodes MXFP4 straight to fp64; ``arm="decoded"`` first expands each matrix to
    bf16 storage (``uint16``), the decoded-BF16 arm's own weights, and computes from those.
    ``cache=False`` keeps no expert after use (128 decoded experts of the full-size layer would take
    36 GB of fp64).
    """

    def __init__(self, inp: dict, arm: str = "packed", cache: bool = True):
        if arm not in ("packed", "decoded"):
            raise ValueError(arm)
        self.inp, self.arm, self.cache, self.keep = inp, arm, {}, cache

    def expand_bf16(self, e: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Expanded bf16 bit patterns of expert e: w1, w3 [I, H] and w2 [H, I] (exact)."""
        i = self.inp
        return (F.bf16_bits(F.decode_mxfp4(i["w1"][e], i["s1"][e])),
                F.bf16_bits(F.decode_mxfp4(i["w3"][e], i["s3"][e])),
                F.bf16_bits(F.decode_mxfp4(i["w2"][e], i["s2"][e])))

    def get(self, e: int):
        if e not in self.cache:
            i = self.inp
            if self.arm == "packed":
                w = (F.decode_mxfp4(i["w1"][e], i["s1"][e]), F.decode_mxfp4(i["w3"][e], i["s3"][e]),
                     F.decode_mxfp4(i["w2"][e], i["s2"][e]))
            else:
                w = tuple(F.bf16_from_bits(b) for b in self.expand_bf16(e))
            if not self.keep:
                return w
            self.cache[e] = w
        return self.cache[e]


def shared_weights(inp: dict):
    """Decoded FP8 shared expert: w1, w3 [I, H], w2 [H, I] (E8M0 per 32x32 block)."""
    return (F.decode_fp8_blocks(inp["sw1"], inp["ss1"]), F.decode_fp8_blocks(inp["sw3"], inp["ss3"]),
            F.decode_fp8_blocks(inp["sw2"], inp["ss2"]))


# ----------------------------------------------------------------------------------------------
# dense FP8 linear (section 4, "Dense")
# ----------------------------------------------------------------------------------------------
def fp8_linear(x_bits: np.ndarray, w: np.ndarray, s: np.ndarray) -> dict:
    """y = bf16(act_qdq(x) W^T): the page's dense projection family, W FP8 E4M3 [N, K] with one E8M0
    per 32x32 block ``s`` [N/32, K/32], x bf16 bits [M, K] QDQ'd per 32 along K (section 2
    "Quantized linear"). Returns the QDQ codes and scales, the exact sums ``acc`` (fp64) and y (fp64
    values of bf16)."""
    xq, xs, xhat = act_qdq(F.bf16_from_bits(x_bits))
    acc = xhat @ F.decode_fp8_blocks(w, s).T
    return dict(xq=xq, xs=xs, acc=acc, y=F.bf16_rne(acc))


# ----------------------------------------------------------------------------------------------
# combine (section 2, "MoE") and the whole layer
# ----------------------------------------------------------------------------------------------
def combine(ids: np.ndarray, slot_y: np.ndarray, shared_y: np.ndarray | None) -> np.ndarray:
    """out = bf16(fp32 sum of the token's expert outputs in ascending expert id, then the shared).

    ``ids`` [R, k], ``slot_y`` fp64 bf16 values [R, k, H] (slot order), ``shared_y`` [R, H] or None.
    Every add is an fp32 add starting from 0.
    """
    R, k = ids.shape
    order = np.argsort(ids, axis=1, kind="stable")
    acc = np.zeros((R, slot_y.shape[2]), dtype=np.float32)
    for j in range(k):
        yj = np.take_along_axis(slot_y, order[:, j][:, None, None], axis=1)[:, 0, :]
        acc = (acc + yj.astype(np.float32)).astype(np.float32)
    if shared_y is not None:
        acc = (acc + shared_y.astype(np.float32)).astype(np.float32)
    return F.bf16_rne(acc.astype(np.float64))


def moe_forward(inp: dict, cfg, tokens=None, ids=None, rw=None, arm: str = "packed",
                weights: ExpertWeights | None = None, with_shared: bool | None = None) -> dict:
    """The whole layer for the rows ``tokens`` (default all), as the MoE section defines it.

    ``ids``/``rw`` given (rows matching ``tokens``) run the experts on that routing instead of the
    oracle's own (conditioned mode, for tie-flagged tokens). Returns routing, QDQ'd x, the per-slot
    expert outputs, the shared output and the final bf16 output (fp64 values), plus intermediates.
    """
    M = inp["x"].shape[0]
    tok = np.arange(M) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xb = inp["x"][tok]
    r = route(xb, inp["gate_w"], inp["gate_b"], cfg.k, cfg.route_scale)
    use_ids = r["ids"] if ids is None else np.asarray(ids, dtype=np.int32)
    use_rw = r["rw"] if rw is None else np.asarray(rw, dtype=np.float32)
    xq, xs, xhat = act_qdq(F.bf16_from_bits(xb))
    W = weights if weights is not None else ExpertWeights(inp, arm, cache=False)
    R, k = use_ids.shape
    H, I = cfg.H, cfg.I
    slot_y = np.zeros((R, k, H))
    g_all = np.zeros((R, k, I)); u_all = np.zeros((R, k, I)); h_all = np.zeros((R, k, I))
    hq_all = np.zeros((R, k, I), dtype=np.uint8); hs_all = np.zeros((R, k, I // 32), dtype=np.uint8)
    for e in np.unique(use_ids):
        rows, slots = np.nonzero(use_ids == e)
        w1, w3, w2 = W.get(int(e))
        o = expert_ffn(xhat[rows], use_rw[rows, slots], w1, w3, w2)
        slot_y[rows, slots] = o["y"]
        g_all[rows, slots] = o["g"]; u_all[rows, slots] = o["u"]; h_all[rows, slots] = o["h16"]
        hq_all[rows, slots] = o["hq"]; hs_all[rows, slots] = o["hs"]
    shared_y = None
    if with_shared is None:
        with_shared = "sw1" in inp
    if with_shared:
        sw1, sw3, sw2 = shared_weights(inp)
        so = expert_ffn(xhat, None, sw1, sw3, sw2)
        shared_y = so["y"]
    out = combine(use_ids, slot_y, shared_y)
    return dict(tokens=tok, route=r, ids=use_ids, rw=use_rw, xq=xq, xs=xs, xhat=xhat, slot_y=slot_y,
                g=g_all, u=u_all, h16=h_all, hq=hq_all, hs=hs_all, shared_y=shared_y, out=out)


def permute(ids: np.ndarray, E: int) -> dict:
    """Token-to-expert permutation: a stable counting sort of the (t, j) pairs by expert id.

    counts[e] = #pairs routed to e; offsets = exclusive prefix sum (E + 1 entries); pairs lists
    t * k + j grouped by expert in ascending (t, j) order; inv[t, j] = position of pair (t, j);
    active = expert ids with counts > 0, ascending, padded with -1 to E entries.
    """
    M, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pairs = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty(M * k, dtype=np.int32)
    inv[pairs] = np.arange(M * k, dtype=np.int32)
    act = np.nonzero(counts)[0].astype(np.int32)
    active = np.full(E, -1, dtype=np.int32)
    active[: act.size] = act
    return dict(counts=counts, offsets=offsets, pairs=pairs, inv=inv.reshape(M, k), active=active,
                n_active=int(act.size))
