"""Plain CPU oracle of one MoE layer, forward and backward.

Test infrastructure only: the GPU library never imports, links or calls it;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.

Everything is computed in fp64 with numpy; a library matmul or sort is used
as a step where the definition is a plain product or a stable sort.  The
rounding points (fp32 for accumulator values, bf16 for stored activations,
the MX quantiser for MXFP8 operands) are applied where the layer stores a
value, and can be switched off (``exact=True``) for finite-difference tests.

Sources (the pages give prose only; every formula below is a reading of it):
  [KC] kucoin.com news flash "O MoK do Cursor alcança aumento de desempenho
       de 2,37x no NVIDIA GB300 NVL72": §01 "O imposto sobre comunicações do
       MoE", §02 (pull dispatch, megakernel, ring buffer), §03 (benchmark).
  [NA] noticiai.com.br "Cursor abre código do Mixture-of-Kittens: kernel MoE
       que acelera treinamento em GPUs Blackwell em até 2,37×", section
       "As três decisões de design que fazem a diferença".
  [DD] deepdigest.ru article on MoK (one untitled body).

The layer, as [KC §03] lists its measured parts: Schedule (routing and
layout), Dispatch, Expert FFN, Combine and the final weighted fusion.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .mx import mx_quantize, mx_roundtrip, mx_rows_roundtrip
from .numerics import bf16, bf16_bits, bf16_to_f64, f32, identity


class _Round:
    """The rounding points; ``exact`` turns every one of them off."""

    def __init__(self, exact: bool):
        self.f32 = identity if exact else f32
        self.bf16 = identity if exact else bf16


def _val(a):
    """bf16 bit patterns (uint16) -> values; anything else -> fp64."""
    if a is None:
        return None
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# Schedule: router and layout


def router_logits(x, w_router, bias=None, exact=False):
    """L[t,e] = fp32(sum_h x[t,h] W_r[h,e]) (+ bias[e], in fp32).

    The router re-decides each step which experts a token visits [KC §01];
    the pages give no formula, so the scoring is a plain linear map of the
    token's hidden vector.
    """
    R = _Round(exact)
    L = R.f32(_val(x) @ _val(w_router))
    if bias is not None:
        L = R.f32(L + _val(bias)[None, :])
    return L


def topk_softmax(logits, k, exact=False):
    """Top-k experts per token and their renormalised softmax weights.

    Each token picks a few experts [KC §01].  Reading: experts are ordered by
    descending logit, equal logits in ascending expert index (a stable sort of
    the negated logits; -0 and +0 compare equal); slot j holds the j-th
    expert of that order.  The weights are the softmax over the k selected
    logits (equal to the full softmax restricted to the selection and
    renormalised), computed in fp64 with the largest selected logit
    subtracted, then held in fp32.
    """
    R = _Round(exact)
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("topk_softmax needs 1 <= k <= E")
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = R.f32(ex / ex.sum(axis=1, keepdims=True))
    return idx, w


def layout(topk_idx, E):
    """Per-expert count, prefix-sum offsets and the expert-contiguous order.

    The layout step counts the tokens of each expert, decides where each one
    goes and keeps the rows of one expert together so that a grouped GEMM gets
    ordered input [KC §01].  Rows are the flat (token, slot) indices
    f = t*k + j; within an expert they stay in ascending f (a stable counting
    sort).  Returns counts[E], offsets[E+1], perm[R] (sorted row r holds flat
    index perm[r]) and inv_perm[R] (flat index f sits at row inv_perm[f]).
    """
    idx = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("layout: expert index out of range")
    counts = np.bincount(idx, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.concatenate([np.flatnonzero(idx == e) for e in range(E)]
                          + [np.zeros(0, np.int64)]).astype(np.int32)
    inv = np.empty(idx.size, dtype=np.int32)
    inv[perm] = np.arange(idx.size, dtype=np.int32)
    return counts, offsets, perm, inv


# ----------------------------------------------------------------------------
# Dispatch


def dispatch(x, perm, k, mx=False):
    """Gather-permute: sorted row r is a copy of token perm[r] div k.

    The destination side reads the rows it needs knowing only where each one
    sits in the source data [KC §02], so the gather is driven by the sorted
    row.  With MXFP8 the copy is quantised along the hidden axis as it is made
    (quantisation fused into dispatch [KC §02]).
    Returns bf16 bits [R,H], or (codes uint8 [R,H], scales uint8 [R,H/32]).
    """
    rows = np.asarray(x)[np.asarray(perm) // k]
    if not mx:
        return rows if rows.dtype == np.uint16 else bf16_bits(rows)
    return mx_quantize(_val(rows), axis=1)


# ----------------------------------------------------------------------------
# Expert FFN (SwiGLU)


def _swiglu_rows(Xhat, Wg, Wu, Wd, mx, R):
    """One expert on the rows Xhat: a = silu(X Wg) * (X Wu); Y = a Wd.

    SwiGLU is named as the expert activation [KC §02]; reading: the gate
    projection goes through silu, multiplies the up projection, and the down
    projection follows, with no biases.  The layer's precision is bf16
    storage with fp32 accumulation, so g and u are fp32 values and a, an
    elementwise function of them, is formed at that same precision before it
    is stored: as bf16, or with MXFP8 quantised along the intermediate axis
    (the SwiGLU path quantises [KC §02]).  Y is stored as bf16.
    """
    g = R.f32(Xhat @ Wg)
    u = R.f32(Xhat @ Wu)
    a = R.f32(silu(g) * u)
    ahat = mx_roundtrip(a, axis=1) if mx else R.bf16(a)
    Y = R.bf16(ahat @ Wd)
    return g, u, ahat, Y


def expert_weights(w_gate, w_up, w_down, mx, backward=False, wfmt="e4m3"):
    """One expert's weights as one direction's GEMMs see them.

    With MX operands every GEMM operand is quantised along that GEMM's
    contraction axis.  The forward contracts gate/up ([H, I]) over H and down
    ([I, H]) over I: axis -2 of each.  The backward data gradients contract
    gate/up over I (dX = dg W_gate^T) and down over H (dA = dY W_down^T):
    axis -1.  ``wfmt`` is the weights' element format: E4M3 (MXFP8
    throughout), or a lower-precision one (FP4 E2M1, FP6 E2M3 / E3M2) for
    lower-precision experts whose activations stay MXFP8.
    Returns dict(g, u, d) in fp64.
    """
    Wg, Wu, Wd = _val(w_gate), _val(w_up), _val(w_down)
    if not mx:
        return dict(g=Wg, u=Wu, d=Wd)
    ax = -1 if backward else -2
    return dict(g=mx_roundtrip(Wg, axis=ax, fmt=wfmt), u=mx_roundtrip(Wu, axis=ax, fmt=wfmt),
                d=mx_roundtrip(Wd, axis=ax, fmt=wfmt))


class ExpertWeights:
    """The routed (or shared) experts' weights, decoded one expert at a time
    on request: a 256-expert layer's decoded weights would not fit in host
    memory at once.  ``fwd(e)`` / ``bwd(e)`` give dict(g, u, d) as the
    forward / backward data-gradient GEMMs see them."""

    def __init__(self, inp, mx, shared=False, wfmt="e4m3"):
        if shared:
            self.src = (inp["ws_gate"][None], inp["ws_up"][None], inp["ws_down"][None])
        else:
            self.src = (inp["w_gate"], inp["w_up"], inp["w_down"])
        self.mx = mx
        self.wfmt = wfmt
        self.E = self.src[0].shape[0]

    def fwd(self, e):
        return expert_weights(self.src[0][e], self.src[1][e], self.src[2][e], self.mx,
                              wfmt=self.wfmt)

    def bwd(self, e):
        return expert_weights(self.src[0][e], self.src[1][e], self.src[2][e], self.mx,
                              backward=True, wfmt=self.wfmt)


THREADS = min(16, os.cpu_count() or 1)


def _each(fn, items):
    """fn(item) for every item, on a pool of THREADS threads (numpy's large
    array operations release the interpreter lock).  Every call writes only
    its own expert's rows or gradients, so the results do not depend on the
    order the calls run in."""
    items = list(items)
    if THREADS <= 1 or len(items) <= 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(min(THREADS, len(items))) as ex:
        list(ex.map(fn, items))


# ----------------------------------------------------------------------------
# Whole layer


def forward(inp, k, mx=False, exact=False, routing=None, logits=None, wfmt="e4m3"):
    """The layer's forward pass; returns every intermediate the backward needs.

    ``inp`` holds x, the expert weights and either a router (w_router, bias)
    or supplied routing (topk_idx, topk_w); the optional shared expert
    (ws_gate, ws_up, ws_down) runs densely on every token with weight one.
    ``logits`` (fp32 [T, E]) replaces the router's logits as the input of the
    selection and the weights: the selection is defined given the fp32
    logits, so a check of another implementation's routing passes that
    implementation's logits here (the router backward still runs).
    ``routing`` (idx, w) overrides the router altogether (used by the
    exact-mode gradient tests, where the selection must stay fixed).
    ``wfmt`` (with ``mx``) is the expert weights' MX element format (see
    :func:`expert_weights`); the activations are MXFP8 either way.
    """
    if exact and mx:
        raise ValueError("exact mode has no quantiser")
    R = _Round(exact)
    x = _val(inp["x"])
    T, H = x.shape
    W = ExpertWeights(inp, mx, wfmt=wfmt)
    E = W.E
    I = inp["w_gate"].shape[2]
    if routing is not None:
        idx, w = np.asarray(routing[0], np.int32), np.asarray(routing[1], np.float64)
    elif logits is not None:
        logits = np.asarray(logits, np.float64)
        if logits.shape != (T, E) or not np.array_equal(logits, f32(logits)):
            raise ValueError("forward: logits must be fp32 values of shape [T, E]")
        idx, w = topk_softmax(logits, k, exact)
    elif inp.get("topk_idx") is None:
        logits = router_logits(x, inp["w_router"], inp.get("bias"), exact)
        idx, w = topk_softmax(logits, k, exact)
    else:
        idx = np.asarray(inp["topk_idx"], np.int32)
        w = _val(inp["topk_w"])
    counts, offsets, perm, inv = layout(idx, E)
    src = perm.astype(np.int64) // k
    xhat_tok = mx_roundtrip(x, axis=1) if mx else x     # quantised per row
    Xhat = xhat_tok[src]                                   # dispatch
    Rn = T * k
    g = np.zeros((Rn, I)); u = np.zeros((Rn, I))
    ahat = np.zeros((Rn, I)); Y = np.zeros((Rn, H))

    def one(e):
        rs = slice(int(offsets[e]), int(offsets[e + 1]))
        We = W.fwd(e)
        g[rs], u[rs], ahat[rs], Y[rs] = _swiglu_rows(Xhat[rs], We["g"], We["u"], We["d"], mx, R)
    _each(one, [e for e in range(E) if counts[e]])
    WS = ExpertWeights(inp, mx, shared=True, wfmt=wfmt) if inp.get("ws_gate") is not None \
        else None
    shared = None
    if WS is not None:
        Ws = WS.fwd(0)
        gs, us, as_, ys = _swiglu_rows(xhat_tok, Ws["g"], Ws["u"], Ws["d"], mx, R)
        shared = dict(g=gs, u=us, ahat=as_, y=ys)
    out = combine(Y, w, inv, k, None if shared is None else shared["y"], exact)
    return dict(k=k, mx=mx, wfmt=wfmt, exact=exact, x=x, xhat_tok=xhat_tok, logits=logits,
                idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv,
                Xhat=Xhat, g=g, u=u, ahat=ahat, Y=Y, shared=shared, out=out, W=W, WS=WS)


def combine(Y, w, inv, k, y_shared=None, exact=False):
    """Combine and final weighted fusion.

    Each result goes back to its token's original position [KC §01] and the
    token's output is the weighted sum of its k expert rows (the weighted
    fusion that closes the measured layer [KC §03]), in ascending slot order,
    plus the shared expert's row with weight one; summed in fp64 and stored
    as bf16.
    """
    R = _Round(exact)
    w = np.asarray(w, dtype=np.float64)
    T = w.shape[0]
    rows = np.asarray(inv).reshape(T, k)
    acc = np.zeros((T, Y.shape[1]))
    for j in range(k):
        acc += w[:, j:j + 1] * Y[rows[:, j]]
    if y_shared is not None:
        acc += y_shared
    return R.bf16(acc)


def _swiglu_rows_bwd(Xhat, g, u, ahat, dY, Wb, mx, R, mx_wgrad=False):
    """Backward of one expert's SwiGLU FFN given its rows' output gradient dY.

    ``Wb`` holds the expert's weights as the backward data-gradient GEMMs see
    them (:meth:`ExpertWeights.bwd`).  ``g`` and ``u`` are the forward's fp32
    accumulator values; they reach the backward as the layer stores its
    activations, as bf16 (the layer's precision is bf16 activations with fp32
    accumulation), and the SwiGLU backward uses those stored values.

    dA = dY' Wd^T; dg = dA u silu'(g); du = dA silu(g) (stored as bf16);
    dWd = ahat^T dY; dWg = Xhat^T dg; dWu = Xhat^T du (fp32);
    dX = dg' Wg^T + du' Wu^T (bf16).  With MXFP8 the data-gradient GEMM
    operands dY' and dg', du' are the MX round trips of the stored bf16
    tensors (along H and along I); the weight-gradient GEMMs use the bf16
    tensors -- or, with mx_wgrad, MX round trips of them quantised along the
    rows, i.e. along those GEMMs' contraction axis, in 32-row blocks starting
    at the expert's first row (the last block zero-padded).
    silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
    """
    g, u = R.bf16(g), R.bf16(u)              # stored activations
    dYq = mx_roundtrip(dY, axis=1) if mx else dY
    dA = R.f32(dYq @ Wb["d"].T)
    s = sigmoid(g)
    dg = R.bf16(dA * u * s * (1.0 + g * (1.0 - s)))
    du = R.bf16(dA * g * s)
    if mx and mx_wgrad:
        aw, dYw = mx_rows_roundtrip(ahat), mx_rows_roundtrip(dY)
        Xw, dgw, duw = mx_rows_roundtrip(Xhat), mx_rows_roundtrip(dg), mx_rows_roundtrip(du)
    else:
        aw, dYw, Xw, dgw, duw = ahat, dY, Xhat, dg, du
    dWd = R.f32(aw.T @ dYw)
    dWg = R.f32(Xw.T @ dgw)
    dWu = R.f32(Xw.T @ duw)
    dgq = mx_roundtrip(dg, axis=1) if mx else dg
    duq = mx_roundtrip(du, axis=1) if mx else du
    dX = R.bf16(dgq @ Wb["g"].T + duq @ Wb["u"].T)
    return dict(dA=dA, dg=dg, du=du, dWd=dWd, dWg=dWg, dWu=dWu, dX=dX)


def backward(inp, fw, dout=None, mx_wgrad=False):
    """The layer's backward pass, mirroring the forward's data movement.

    Training adds two more exchange rounds in the opposite direction [KC §01]:
    reverse-combine (each sorted row pulls its token's output gradient times
    the slot weight) and reverse-dispatch (each token sums the gradients of
    its k rows) [KC §02].  Returns dY, dw, per-expert dg/du, dX, dW_gate,
    dW_up, dW_down, the router's dL/dW_r (router routing) and dx.  With
    MXFP8 and mx_wgrad the weight-gradient GEMMs also take MX operands
    (see _swiglu_rows_bwd); the shared expert's too.
    """
    k, mx, exact = fw["k"], fw["mx"], fw["exact"]
    R = _Round(exact)
    dout = _val(inp["dout"] if dout is None else dout)
    T, H = dout.shape
    perm, inv, offsets = fw["perm"], fw["inv"], fw["offsets"]
    w = np.asarray(fw["w"], dtype=np.float64)
    E = len(offsets) - 1
    I = fw["g"].shape[1]
    src = perm.astype(np.int64) // k
    # reverse-combine: dY[r] = w[f] dOut[t]; dw[t,j] = <dOut[t], Y[row of (t,j)]>
    dY = R.bf16(w.reshape(-1)[perm][:, None] * dout[src])
    rows = inv.reshape(T, k)
    dw = np.empty((T, k))
    for j in range(k):
        dw[:, j] = np.einsum("th,th->t", dout, fw["Y"][rows[:, j]])
    dw = R.f32(dw)
    Rn = T * k
    dg = np.zeros((Rn, I)); du = np.zeros((Rn, I)); dX = np.zeros((Rn, H))
    dWg = np.zeros((E, H, I)); dWu = np.zeros((E, H, I)); dWd = np.zeros((E, I, H))
    W = fw["W"]
    counts = np.diff(offsets)

    def one(e):
        rs = slice(int(offsets[e]), int(offsets[e + 1]))
        b = _swiglu_rows_bwd(fw["Xhat"][rs], fw["g"][rs], fw["u"][rs], fw["ahat"][rs],
                             dY[rs], W.bwd(e), mx, R, mx_wgrad)
        dg[rs], du[rs], dX[rs] = b["dg"], b["du"], b["dX"]
        dWg[e], dWu[e], dWd[e] = b["dWg"], b["dWu"], b["dWd"]
    _each(one, [e for e in range(E) if counts[e]])
    out = dict(dY=dY, dw=dw, dg=dg, du=du, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd)
    acc = np.zeros((T, H))
    for j in range(k):
        acc += dX[rows[:, j]]
    if fw["logits"] is not None:
        dsel, dL, dWr, dxr = router_backward(fw["x"], inp["w_router"], fw["idx"], w, dw,
                                             E, exact)
        out.update(dsel=dsel, dL=dL, dWr=dWr)
        acc += dxr
    if fw["shared"] is not None:
        sh = fw["shared"]
        b = _swiglu_rows_bwd(fw["xhat_tok"], sh["g"], sh["u"], sh["ahat"], dout,
                             fw["WS"].bwd(0), mx, R, mx_wgrad)
        out.update(dWsg=b["dWg"], dWsu=b["dWu"], dWsd=b["dWd"], dXs=b["dX"])
        acc += b["dX"]
    out["dx"] = R.bf16(acc)
    return out


def router_backward(x, w_router, idx, w, dw, E, exact=False):
    """Gradient through the renormalised top-k softmax and the router map.

    With w = softmax over the selected logits, dL[t,idx_j] = w_j (dw_j -
    sum_j' w_j' dw_j') and 0 for unselected experts (selection itself has no
    gradient); dW_r = x^T dL and the token-side term is dL W_r^T.
    """
    R = _Round(exact)
    x = _val(x)
    Wr = _val(w_router)
    w = np.asarray(w, np.float64)
    dw = np.asarray(dw, np.float64)
    s = np.sum(w * dw, axis=1, keepdims=True)
    dsel = R.f32(w * (dw - s))
    dL = np.zeros((x.shape[0], E))
    np.put_along_axis(dL, np.asarray(idx, np.int64), dsel, axis=1)
    dWr = R.f32(x.T @ dL)
    return dsel, dL, dWr, dL @ Wr.T


# ----------------------------------------------------------------------------
# Brute force per token: no layout, no permutation


class _LazyWeights:
    """Per-expert weights of both directions, dict(fwd=..., bwd=...) as
    :class:`ExpertWeights` gives them, decoded on first use and kept for the
    ``keep`` most recently used experts: the sampled evaluators touch only a
    few experts."""

    def __init__(self, inp, mx, shared=False, keep=16, wfmt="e4m3"):
        self.src = ExpertWeights(inp, mx, shared, wfmt)
        self.keep = keep
        self.cache = {}

    def _decode(self, e):
        return dict(fwd=self.src.fwd(e), bwd=self.src.bwd(e))

    def prefetch(self, experts, threads=8):
        """Decode several experts at once (numpy releases the GIL in the
        elementwise work, so threads overlap); the cache grows to hold them."""
        todo = [int(e) for e in dict.fromkeys(experts) if int(e) not in self.cache]
        self.keep = max(self.keep, len(self.cache) + len(todo))
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for e, We in zip(todo, ex.map(self._decode, todo)):
                self.cache[e] = We

    def __getitem__(self, e):
        if e in self.cache:
            self.cache[e] = self.cache.pop(e)          # most recently used last
        else:
            if len(self.cache) >= self.keep:
                self.cache.pop(next(iter(self.cache)))
            self.cache[e] = self._decode(e)
        return self.cache[e]


class TokenEvaluator:
    """Evaluate chosen tokens' outputs and gradients one token at a time.

    Nothing here uses counts, offsets or permutations: token t's output is
    sum_j w[t,j] FFN_{idx[t,j]}(x_t) (+ the shared expert), each FFN applied
    to the single row x_t.  It serves as the brute-force check of the layer
    and as the sampled oracle at sizes the full oracle cannot finish.
    Rounding points and quantisation are those of :func:`forward`.
    """

    def __init__(self, inp, k, mx=False, wfmt="e4m3"):
        self.inp, self.k, self.mx = inp, k, mx
        self.R = _Round(False)
        self.x = _val(inp["x"])
        self.W = _LazyWeights(inp, mx, wfmt=wfmt)
        self.WS = _LazyWeights(inp, mx, shared=True, wfmt=wfmt)[0] \
            if inp.get("ws_gate") is not None else None
        if inp.get("topk_idx") is None:
            self.routing = None
        else:
            self.routing = (np.asarray(inp["topk_idx"], np.int32), _val(inp["topk_w"]))

    def route(self, t):
        if self.routing is not None:
            return self.routing[0][t], self.routing[1][t]
        L = router_logits(self.x[t:t + 1], self.inp["w_router"], self.inp.get("bias"))
        i, w = topk_softmax(L, self.k)
        return i[0], w[0]

    def _xhat(self, t):
        xt = self.x[t:t + 1]
        return mx_roundtrip(xt, axis=1) if self.mx else xt

    def token(self, t):
        """Forward of token t: dict(idx, w, slots=[per-slot g,u,ahat,Y], shared, out)."""
        idx, w = self.route(t)
        xh = self._xhat(t)
        slots = []
        acc = np.zeros(self.x.shape[1])
        for j in range(self.k):
            e = int(idx[j])
            We = self.W[e]["fwd"]
            g, u, ah, Y = _swiglu_rows(xh, We["g"], We["u"], We["d"], self.mx, self.R)
            slots.append(dict(e=e, g=g, u=u, ahat=ah, Y=Y[0]))
            acc += w[j] * Y[0]
        ys = None
        if self.WS is not None:
            Ws = self.WS["fwd"]
            ys = _swiglu_rows(xh, Ws["g"], Ws["u"], Ws["d"], self.mx, self.R)
            acc += ys[3][0]
        return dict(idx=idx, w=w, slots=slots, shared=ys, xhat=xh, out=self.R.bf16(acc))

    def token_grad(self, t, dout_t):
        """Backward of token t given its output gradient: dw[k] and dx[H]."""
        fw = self.token(t)
        dout_t = np.asarray(dout_t, np.float64)
        w = np.asarray(fw["w"], np.float64)
        dw = self.R.f32(np.array([dout_t @ s["Y"] for s in fw["slots"]]))
        acc = np.zeros_like(dout_t)
        for j, s in enumerate(fw["slots"]):
            We = self.W[s["e"]]["bwd"]
            dY = self.R.bf16(w[j] * dout_t)[None, :]
            b = _swiglu_rows_bwd(fw["xhat"], s["g"], s["u"], s["ahat"], dY, We, self.mx, self.R)
            acc += b["dX"][0]
        if self.routing is None:
            E = self.inp["w_gate"].shape[0]
            _, _, _, dxr = router_backward(self.x[t:t + 1], self.inp["w_router"],
                                           fw["idx"][None], w[None], dw[None], E)
            acc += dxr[0]
        if fw["shared"] is not None:
            gs, us, as_, _ = fw["shared"]
            b = _swiglu_rows_bwd(fw["xhat"], gs, us, as_, dout_t[None, :], self.WS["bwd"],
                                 self.mx, self.R)
            acc += b["dX"][0]
        return dict(dw=dw, dx=self.R.bf16(acc))


def expert_weight_grad_columns(inp, k, mx, e, cols, dout=None, shared=False, weights=None,
                               logits=None, wfmt="e4m3"):
    """dW_down[e, i, :], dW_gate[e, :, i], dW_up[e, :, i] for chosen columns i.

    Sums over the rows routed to expert e (found from the routing by
    :func:`layout`), recomputing only the 32-column blocks of g, u, a and dA
    that the chosen columns fall in.  For sampled checks at full size.
    Router routing is evaluated in full (it is cheap), from ``logits`` when
    given (as :func:`forward` takes them); the FFN is not.
    With ``shared`` the expert is the shared one: every token, weight one.
    ``weights`` may pass the expert's decoded weights, dict(fwd=..., bwd=...)
    (as a TokenEvaluator holds them), to skip decoding them again.
    """
    R = _Round(False)
    x = _val(inp["x"])
    dout = _val(inp["dout"] if dout is None else dout)
    if shared:
        We = weights if weights is not None else _LazyWeights(inp, mx, True, wfmt=wfmt)[0]
        t = np.arange(x.shape[0])
        wrow = np.ones(x.shape[0])
    else:
        We = weights if weights is not None else _LazyWeights(inp, mx, wfmt=wfmt)[e]
        if logits is not None:
            idx, w = topk_softmax(logits, k)
        elif inp.get("topk_idx") is None:
            L = router_logits(x, inp["w_router"], inp.get("bias"))
            idx, w = topk_softmax(L, k)
        else:
            idx, w = np.asarray(inp["topk_idx"]), _val(inp["topk_w"])
        E = inp["w_gate"].shape[0]
        _, offsets, perm, _ = layout(idx, E)
        f = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
        t = f // k
        wrow = np.asarray(w, np.float64).reshape(-1)[f]
    Wf, Wb = We["fwd"], We["bwd"]
    xh = mx_roundtrip(x[t], axis=1) if mx else x[t]
    dY = R.bf16(wrow[:, None] * dout[t])
    cols = np.asarray(cols)
    blocks = np.unique(cols // 32)
    bc = np.concatenate([np.arange(b * 32, b * 32 + 32) for b in blocks])
    g = R.f32(xh @ Wf["g"][:, bc])
    u = R.f32(xh @ Wf["u"][:, bc])
    a = R.f32(silu(g) * u)
    ah = mx_roundtrip(a, axis=1) if mx else R.bf16(a)
    dYq = mx_roundtrip(dY, axis=1) if mx else dY
    dA = R.f32(dYq @ Wb["d"][bc, :].T)
    g, u = R.bf16(g), R.bf16(u)              # stored activations (see _swiglu_rows_bwd)
    s = sigmoid(g)
    dg = R.bf16(dA * u * s * (1.0 + g * (1.0 - s)))
    du = R.bf16(dA * g * s)
    pos = np.searchsorted(bc, cols)
    return dict(
        dWd=R.f32(ah[:, pos].T @ dY),          # [len(cols), H]
        dWg=R.f32(xh.T @ dg[:, pos]).T,        # [len(cols), H]
        dWu=R.f32(xh.T @ du[:, pos]).T,        # [len(cols), H]
        rows=int(t.size))
