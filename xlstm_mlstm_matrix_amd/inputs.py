"""Seeded synthetic inputs for the mLSTM cell workloads.

This module only draws random numbers and casts them; it holds none of the
cell's arithmetic, so the float64 oracle and the HIP path can both be fed from
it without sharing any of the method.

Recipe (every value is drawn in float64 from numpy's PCG64, then cast once to
the I/O dtype; bf16 casts round to nearest even):

* per (b, h) pair of a prefill workload a child generator seeded with
  ``SeedSequence([seed, b, h])`` draws, in this order and in C order,
  q[T, d_qk], k[T, d_qk], v[T, d_v], i_pre[T], f_raw[T], o_pre[T, d_v],
  then C0[d_qk, d_v], n0[d_qk], m0 (when the workload has an initial state);
* k is multiplied by 1/sqrt(d_qk) and the log forget gate input is
  f_pre = logsigmoid(f_raw), i.e. the forget gate handed to the cell is already
  in log space (the cell itself applies exp, never a sigmoid);
* a decode workload draws tensor j of step t from ``SeedSequence([seed, 1, t,
  j])`` (so any single step is reproducible alone) and batch row b of its
  initial state from ``SeedSequence([seed, 0, b])``;
* a layer workload draws batch row b of its input x[T, d_model] from
  ``SeedSequence([seed, 2, b])``, weight tensor j (W_q, W_k, W_v, W_o, W_i,
  W_f, b_q, b_k, b_v, b_o, b_i, b_f) from ``SeedSequence([seed, 3, j])`` and
  the initial state of cell (h, b) from ``SeedSequence([seed, 4, h, b])``.
  x ~ N(0, 1); W_q, W_v, W_o ~ N(0, 1/d_model) and W_k ~ N(0, 1/(d_model
  d_qk)), so q, v, o~ come out near N(0, 1) and k near N(0, 1/d_qk) as in the
  cell workloads; W_i ~ N(0, i_std^2/d_model) with b_i ~ N(i_mean, 0.1^2);
  W_f ~ N(0, f_std^2/d_model) with b_f ~ N(f_mean, 0.01^2), the forget input
  being the log forget gate directly; the other biases ~ N(0, 0.1^2) (b_k
  scaled by 1/sqrt(d_qk));
* an sLSTM workload draws the input pre-activations gx[T, 4, d] of group
  (b, h) from ``SeedSequence([seed, 5, b, h])`` (z~ ~ N(0, 1), i~ ~
  N(i_mean, i_std), f~ = logsigmoid(N(f_mean, f_std)), o~ ~ N(0, 1)), the
  recurrent weights R[h] [4, d, d] ~ N(0, r_scale^2/d) from
  ``SeedSequence([seed, 6, h])`` and the state of group (b, h) from
  ``SeedSequence([seed, 7, b, h])`` (c0 ~ N(0, 0.5), n0 ~ U(0.5, 1.5), m0 ~
  U(-1, 1), h0 ~ N(0, 0.3)).

Because the draws are per (b, h) (prefill) or per step (decode), a subset of
the pairs or steps can be regenerated without drawing the rest, which is how
the oracle is fed a bounded sample of a large workload.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "gen_prefill", "gen_decode_state",
           "gen_decode_step", "to_io_dtype", "logsigmoid", "LayerWorkload", "LAYER_WORKLOADS",
           "layer_workload", "gen_layer", "SlstmWorkload", "SLSTM_WORKLOADS", "slstm_workload",
           "gen_slstm"]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, I/O dtype and input distributions."""
    name: str
    seed: int
    kind: str                  # "prefill" or "decode"
    B: int
    H: int
    T: int                     # tokens (prefill) or consecutive steps (decode)
    d_qk: int
    d_v: int
    chunk: int                 # prefill chunk length (0 for decode)
    io: str                    # "f32" or "bf16": dtype of q, k, v, o_pre and h
    i_mean: float
    i_std: float
    f_mean: float              # f_pre = logsigmoid(N(f_mean, f_std))
    f_std: float
    init_state: Optional[Dict[str, Tuple[str, float, float]]] = None
    # init_state entries: name -> ("normal", mean, std) | ("uniform", lo, hi) | ("zero", 0, 0)
    description: str = ""


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_f32", 1, "prefill", 1, 1, 64, 16, 16, 16, "f32",
             0.0, 1.0, 3.0, 1.0, None,
             "Tiny mLSTM fwd, fp32: B=1 H=1 T=64 d_qk=d_v=16 chunk=16, zero initial state"),
    Workload("small_f32", 2, "prefill", 4, 4, 1024, 64, 64, 64, "f32",
             0.0, 1.0, 3.0, 1.0,
             {"C0": ("normal", 0.0, 0.1), "n0": ("normal", 0.0, 0.1), "m0": ("zero", 0.0, 0.0)},
             "Small mLSTM fwd, fp32: B=4 H=4 T=1024 d_qk=d_v=64 chunk=64, random initial state"),
    Workload("prefill_7b_bf16", 3, "prefill", 8, 8, 4096, 256, 512, 64, "bf16",
             -2.0, 1.0, 4.0, 1.5, None,
             "7B-layer-shaped prefill, bf16 I/O, fp32 state: B=8 H=8 T=4096 d_qk=256 d_v=512 chunk=64"),
    Workload("prefill_long_bf16", 4, "prefill", 1, 8, 65536, 256, 512, 128, "bf16",
             -2.0, 1.0, 4.0, 1.5, None,
             "Long-context prefill, bf16 I/O, fp32 state: B=1 H=8 T=65536 d_qk=256 d_v=512 chunk=128"),
    Workload("decode_bf16", 5, "decode", 256, 8, 1024, 256, 512, 0, "bf16",
             -2.0, 1.0, 4.0, 1.5,
             {"C0": ("normal", 0.0, 0.05), "n0": ("normal", 0.0, 0.05), "m0": ("uniform", -1.0, 1.0)},
             "Recurrent decode, bf16 q/k/v, fp32 state: B=256 H=8 d_qk=256 d_v=512, 1024 steps"),
]}


def workload(name: str, **override) -> Workload:
    """Return a named workload, optionally with some fields replaced (e.g. a
    reduced B for a parity test)."""
    w = WORKLOADS[name]
    if override:
        d = dict(w.__dict__)
        d.update(override)
        w = Workload(**d)
    return w


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """log(1/(1+e^{-x})) evaluated without overflow, in float64.

    Part of the input recipe (the forget-gate input is drawn as the log of a
    sigmoid), not of the cell."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def to_io_dtype(x: np.ndarray, io: str):
    """Cast a float64 array to the workload's I/O dtype.

    Returns a torch CPU tensor (float32 or bfloat16, the latter rounded to
    nearest even from the float32 value; float64 -> float32 is itself RNE and
    float32 -> bfloat16 RNE of it is what every consumer sees)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if io == "f32":
        return t
    if io == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown io dtype {io!r}")


def _draw_state(rng: np.random.Generator, spec, shape):
    kind, a, b = spec
    if kind == "normal":
        return rng.normal(a, b, size=shape)
    if kind == "uniform":
        return rng.uniform(a, b, size=shape)
    if kind == "zero":
        return np.zeros(shape)
    raise ValueError(kind)


def _draw_pair(w: Workload, b: int, h: int, T: int):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, h])))
    q = rng.standard_normal((T, w.d_qk))
    k = rng.standard_normal((T, w.d_qk)) * (1.0 / math.sqrt(w.d_qk))
    v = rng.standard_normal((T, w.d_v))
    i_pre = rng.normal(w.i_mean, w.i_std, size=T)
    f_pre = logsigmoid(rng.normal(w.f_mean, w.f_std, size=T))
    o_pre = rng.standard_normal((T, w.d_v))
    st = None
    if w.init_state is not None:
        C0 = _draw_state(rng, w.init_state["C0"], (w.d_qk, w.d_v))
        n0 = _draw_state(rng, w.init_state["n0"], (w.d_qk,))
        m0 = _draw_state(rng, w.init_state["m0"], ())
        st = (C0, n0, np.float64(m0))
    return q, k, v, i_pre, f_pre, o_pre, st


def gen_prefill(w: Workload, pairs: Optional[Sequence[Tuple[int, int]]] = None,
                T: Optional[int] = None, threads: int = 8):
    """Draw a prefill workload.

    Returns a dict of torch CPU tensors: q, k [P, T, d_qk], v, o_pre [P, T, d_v]
    in the I/O dtype, i_pre, f_pre [P, T] float32, and C0 [P, d_qk, d_v], n0
    [P, d_qk], m0 [P] float32 (None when the workload starts from the zero
    state), where P runs over ``pairs`` (default: every (b, h) in b-major
    order, so P = B*H and a reshape to [B, H, ...] is free).  ``T`` truncates
    the sequence (the first T tokens of each pair are identical to those of
    the full workload)."""
    import torch
    if pairs is None:
        pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    T = w.T if T is None else T
    P = len(pairs)
    cast = torch.bfloat16 if w.io == "bf16" else torch.float32
    out = {
        "q": torch.empty((P, T, w.d_qk), dtype=cast),
        "k": torch.empty((P, T, w.d_qk), dtype=cast),
        "v": torch.empty((P, T, w.d_v), dtype=cast),
        "i_pre": torch.empty((P, T), dtype=torch.float32),
        "f_pre": torch.empty((P, T), dtype=torch.float32),
        "o_pre": torch.empty((P, T, w.d_v), dtype=cast),
    }
    has_state = w.init_state is not None
    if has_state:
        out["C0"] = torch.empty((P, w.d_qk, w.d_v), dtype=torch.float32)
        out["n0"] = torch.empty((P, w.d_qk), dtype=torch.float32)
        out["m0"] = torch.empty((P,), dtype=torch.float32)

    def work(p):
        b, h = pairs[p]
        q, k, v, i_pre, f_pre, o_pre, st = _draw_pair(w, b, h, w.T)
        out["q"][p] = to_io_dtype(q[:T], w.io)
        out["k"][p] = to_io_dtype(k[:T], w.io)
        out["v"][p] = to_io_dtype(v[:T], w.io)
        out["o_pre"][p] = to_io_dtype(o_pre[:T], w.io)
        out["i_pre"][p] = torch.from_numpy(i_pre[:T].astype(np.float32))
        out["f_pre"][p] = torch.from_numpy(f_pre[:T].astype(np.float32))
        if has_state:
            out["C0"][p] = torch.from_numpy(st[0].astype(np.float32))
            out["n0"][p] = torch.from_numpy(st[1].astype(np.float32))
            out["m0"][p] = float(np.float32(st[2]))

    if threads > 1 and P > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(P)))
    else:
        for p in range(P):
            work(p)
    if not has_state:
        out["C0"] = out["n0"] = out["m0"] = None
    return out


_DECODE_TENSORS = {"q": 0, "k": 1, "v": 2, "i_pre": 3, "f_pre": 4, "o_pre": 5}


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def gen_decode_state(w: Workload, B: Optional[int] = None, threads: int = 8):
    """Initial state of a decode workload: C0 [B,H,d_qk,d_v], n0 [B,H,d_qk],
    m0 [B,H], float32 torch CPU tensors.  Batch row b is drawn (C0, then n0,
    then m0) from its own generator ``SeedSequence([seed, 0, b])``, so a
    reduced ``B`` is a prefix of the full workload."""
    import torch
    B = w.B if B is None else B
    C0 = torch.empty((B, w.H, w.d_qk, w.d_v), dtype=torch.float32)
    n0 = torch.empty((B, w.H, w.d_qk), dtype=torch.float32)
    m0 = torch.empty((B, w.H), dtype=torch.float32)

    def row(b):
        rng = _rng(w.seed, 0, b)
        C0[b] = torch.from_numpy(_draw_state(rng, w.init_state["C0"], (w.H, w.d_qk, w.d_v)).astype(np.float32))
        n0[b] = torch.from_numpy(_draw_state(rng, w.init_state["n0"], (w.H, w.d_qk)).astype(np.float32))
        m0[b] = torch.from_numpy(np.asarray(_draw_state(rng, w.init_state["m0"], (w.H,))).astype(np.float32))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(row, range(B)))
    return C0, n0, m0


def gen_decode_step(w: Workload, t: int, B: Optional[int] = None):
    """Inputs of decode step t: q, k [B,H,d_qk], v, o_pre [B,H,d_v] in the I/O
    dtype, i_pre, f_pre [B,H] float32 (torch CPU tensors).  Each tensor of
    each step comes from its own generator ``SeedSequence([seed, 1, t, j])``
    (j = 0..5 for q, k, v, i_pre, f_pre, o_pre), drawn in C order, so a
    reduced ``B`` is a prefix of the full step's batch."""
    import torch
    B = w.B if B is None else B
    H = w.H
    j = _DECODE_TENSORS
    q = _rng(w.seed, 1, t, j["q"]).standard_normal((B, H, w.d_qk))
    k = _rng(w.seed, 1, t, j["k"]).standard_normal((B, H, w.d_qk)) * (1.0 / math.sqrt(w.d_qk))
    v = _rng(w.seed, 1, t, j["v"]).standard_normal((B, H, w.d_v))
    i_pre = _rng(w.seed, 1, t, j["i_pre"]).normal(w.i_mean, w.i_std, size=(B, H))
    f_pre = logsigmoid(_rng(w.seed, 1, t, j["f_pre"]).normal(w.f_mean, w.f_std, size=(B, H)))
    o_pre = _rng(w.seed, 1, t, j["o_pre"]).standard_normal((B, H, w.d_v))
    return {
        "q": to_io_dtype(q, w.io), "k": to_io_dtype(k, w.io), "v": to_io_dtype(v, w.io),
        "i_pre": torch.from_numpy(i_pre.astype(np.float32)),
        "f_pre": torch.from_numpy(f_pre.astype(np.float32)),
        "o_pre": to_io_dtype(o_pre, w.io),
    }


def gen_decode_steps(w: Workload, steps: Sequence[int], B: Optional[int] = None, threads: int = 8):
    """Several decode steps stacked on a leading step axis (dict of torch CPU
    tensors of shape [S, B, H, ...]), drawn in parallel threads."""
    import torch
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        parts = list(ex.map(lambda t: gen_decode_step(w, t, B), steps))
    return {key: torch.stack([p[key] for p in parts]) for key in parts[0]}


@dataclass(frozen=True)
class LayerWorkload:
    """A synthetic mLSTM layer workload (input projections + cell)."""
    name: str
    seed: int
    B: int
    T: int
    d_model: int
    H: int
    d_qk: int
    d_v: int
    chunk: int
    io: str
    i_mean: float = -2.0
    i_std: float = 1.0
    f_mean: float = -0.05      # log forget gate: b_f ~ N(f_mean, 0.01^2)
    f_std: float = 0.05        # std of W_f x
    init_state: Optional[Dict[str, Tuple[str, float, float]]] = None
    description: str = ""


LAYER_WORKLOADS: Dict[str, LayerWorkload] = {w.name: w for w in [
    LayerWorkload("layer_small", 6, 2, 100, 64, 2, 16, 32, 32, "f32",
                  init_state={"C0": ("normal", 0.0, 0.1), "n0": ("normal", 0.0, 0.1),
                              "m0": ("uniform", -1.0, 1.0)},
                  description="Small mLSTM layer: B=2 T=100 d_model=64 H=2 d_qk=16 d_v=32, random state"),
    LayerWorkload("layer_7b_bf16", 7, 8, 4096, 4096, 8, 256, 512, 64, "bf16",
                  description="7B-shaped mLSTM layer, bf16: B=8 T=4096 d_model=4096 H=8 d_qk=256 d_v=512 "
                              "chunk=64, zero initial state"),
]}


def layer_workload(name: str, **override) -> LayerWorkload:
    w = LAYER_WORKLOADS[name]
    if override:
        d = dict(w.__dict__)
        d.update(override)
        w = LayerWorkload(**d)
    return w


def gen_layer(w: LayerWorkload, batches: Optional[Sequence[int]] = None, T: Optional[int] = None,
              threads: int = 8):
    """Draw a layer workload: a dict of torch CPU tensors x [len(batches), T,
    d_model] (default: every batch row), W_q, W_k [H, d_qk, d_model], W_v, W_o
    [H, d_v, d_model], W_i, W_f [H, d_model] in the I/O dtype, float32 biases
    b_q, b_k [H, d_qk], b_v, b_o [H, d_v], b_i, b_f [H], and the initial state
    C0 [H, nb, d_qk, d_v], n0 [H, nb, d_qk], m0 [H, nb] (float32, head-major,
    None for the zero state).  ``T`` truncates every row to its first T
    tokens."""
    import torch
    batches = list(range(w.B)) if batches is None else list(batches)
    T = w.T if T is None else T
    D, H, dk, dv = w.d_model, w.H, w.d_qk, w.d_v
    cast = torch.bfloat16 if w.io == "bf16" else torch.float32
    out = {"x": torch.empty((len(batches), T, D), dtype=cast)}

    def row(j):
        x = _rng(w.seed, 2, batches[j]).standard_normal((w.T, D))
        out["x"][j] = to_io_dtype(x[:T], w.io)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(row, range(len(batches))))
    sd = 1.0 / math.sqrt(D)
    specs = [("W_q", (H, dk, D), 0.0, sd), ("W_k", (H, dk, D), 0.0, sd / math.sqrt(dk)),
             ("W_v", (H, dv, D), 0.0, sd), ("W_o", (H, dv, D), 0.0, sd),
             ("W_i", (H, D), 0.0, w.i_std * sd), ("W_f", (H, D), 0.0, w.f_std * sd),
             ("b_q", (H, dk), 0.0, 0.1), ("b_k", (H, dk), 0.0, 0.1 / math.sqrt(dk)),
             ("b_v", (H, dv), 0.0, 0.1), ("b_o", (H, dv), 0.0, 0.1),
             ("b_i", (H,), w.i_mean, 0.1), ("b_f", (H,), w.f_mean, 0.01)]
    for j, (name, shape, mean, std) in enumerate(specs):
        a = _rng(w.seed, 3, j).normal(mean, std, size=shape)
        if name.startswith("W_"):
            out[name] = to_io_dtype(a, w.io)
        else:
            out[name] = torch.from_numpy(a.astype(np.float32))
    if w.init_state is None:
        out["C0"] = out["n0"] = out["m0"] = None
    else:
        nb = len(batches)
        C0 = torch.empty((H, nb, dk, dv), dtype=torch.float32)
        n0 = torch.empty((H, nb, dk), dtype=torch.float32)
        m0 = torch.empty((H, nb), dtype=torch.float32)
        for h in range(H):
            for j, b in enumerate(batches):
                rng = _rng(w.seed, 4, h, b)
                C0[h, j] = torch.from_numpy(_draw_state(rng, w.init_state["C0"], (dk, dv)).astype(np.float32))
                n0[h, j] = torch.from_numpy(_draw_state(rng, w.init_state["n0"], (dk,)).astype(np.float32))
                m0[h, j] = float(np.float32(_draw_state(rng, w.init_state["m0"], ())))
        out["C0"], out["n0"], out["m0"] = C0, n0, m0
    return out


@dataclass(frozen=True)
class SlstmWorkload:
    """A synthetic sLSTM cell workload."""
    name: str
    seed: int
    B: int
    H: int
    T: int
    d: int
    io: str
    state: bool
    i_mean: float = -2.0
    i_std: float = 1.0
    f_mean: float = 3.0        # f~ = logsigmoid(N(f_mean, f_std))
    f_std: float = 1.0
    r_scale: float = 1.0
    description: str = ""


SLSTM_WORKLOADS: Dict[str, SlstmWorkload] = {w.name: w for w in [
    SlstmWorkload("slstm_small", 8, 2, 2, 100, 32, "f32", True,
                  description="Small sLSTM cell: B=2 H=2 T=100 d=32 float32, random state"),
    SlstmWorkload("slstm_bf16", 9, 16, 8, 4096, 128, "bf16", False,
                  description="sLSTM cell, bf16 I/O: B=16 H=8 T=4096 d=128, zero state"),
]}


def slstm_workload(name: str, **override) -> SlstmWorkload:
    w = SLSTM_WORKLOADS[name]
    if override:
        d = dict(w.__dict__)
        d.update(override)
        w = SlstmWorkload(**d)
    return w


def gen_slstm(w: SlstmWorkload, groups: Optional[Sequence[Tuple[int, int]]] = None,
              T: Optional[int] = None, threads: int = 8):
    """Draw an sLSTM workload: gx [B, H, T, 4, d] (I/O dtype), R [H, 4, d, d]
    (I/O dtype) and the state c0, n0, m0, h0 [B, H, d] float32 (None for the
    zero state), as torch CPU tensors.  ``groups`` restricts gx and the state
    to those (b, h) groups, returned as [1, len(groups), ...] (R stays
    [H, ...]; group p uses head groups[p][1])."""
    import torch
    T = w.T if T is None else T
    d = w.d
    cast = torch.bfloat16 if w.io == "bf16" else torch.float32
    if groups is None:
        groups = [(b, h) for b in range(w.B) for h in range(w.H)]
        shape = (w.B, w.H)
    else:
        shape = (1, len(groups))
    gx = torch.empty((len(groups), T, 4, d), dtype=cast)
    st = [torch.empty((len(groups), d), dtype=torch.float32) for _ in range(4)] if w.state else None

    def group(p):
        b, h = groups[p]
        rng = _rng(w.seed, 5, b, h)
        z = rng.standard_normal((w.T, d))
        i = rng.normal(w.i_mean, w.i_std, size=(w.T, d))
        f = logsigmoid(rng.normal(w.f_mean, w.f_std, size=(w.T, d)))
        o = rng.standard_normal((w.T, d))
        gx[p] = to_io_dtype(np.stack([z, i, f, o], axis=1)[:T], w.io)
        if st is not None:
            r2 = _rng(w.seed, 7, b, h)
            vals = (r2.normal(0.0, 0.5, d), r2.uniform(0.5, 1.5, d), r2.uniform(-1.0, 1.0, d),
                    r2.normal(0.0, 0.3, d))
            for x, v in zip(st, vals):
                x[p] = torch.from_numpy(v.astype(np.float32))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(group, range(len(groups))))
    R = torch.stack([to_io_dtype(_rng(w.seed, 6, h).normal(0.0, w.r_scale / math.sqrt(d), (4, d, d)), w.io)
                     for h in range(w.H)])
    out = {"gx": gx.reshape(*shape, T, 4, d), "R": R}
    names = ("c0", "n0", "m0", "h0")
    for k, x in zip(names, st or (None,) * 4):
        out[k] = None if x is None else x.reshape(*shape, d)
    return out
