"""Seeded synthetic inputs for the once-per-block sparse selection path.

This module only draws numbers. It holds none of the selection or attention
arithmetic: both the CPU oracle (through the tests) and the HIP library read the
exact bits produced here, so the two sides see identical inputs.

The workloads stand in for the attention-layer shapes of the long-context runs
the HERALD pages report on (8B-style 32/8/128 GQA, 7B-style 28/4/128, contexts
16K-128K, K=1024 budget; HERALD arXiv 2606.21633 v3 abstract, SparDA arXiv
2606.04511 Experiment section). No benchmark item is reproduced: every tensor is
a seeded draw.

Recipe (every draw is fp32 from ``numpy.random.Generator(PCG64)`` and is then
rounded to bf16 with round-to-nearest-even, except in fp32 workloads):

* Each sequence ``s`` of a workload gets its own ``SeedSequence(seed_base + s)``,
  split with ``spawn`` into named child streams, so no tensor depends on the
  order in which the others were drawn.
* ``gaussian``: Q, K, V ~ N(0, 1).
* ``channel_scaled``: as ``gaussian``, each tensor multiplied per channel by a
  scale vector ~ U(0.5, 2), one vector per head per tensor (Q, K, V separately).
* ``drift``: K[j] = z_j + w_j with z ~ N(0, 1) and a random walk
  w_0 = 0, w_j = w_{j-1} + 0.01 * N(0, 1) per (KV head, channel), summed in fp64.
* Planted keys (``planted`` per KV head, positions uniform without replacement):
  k <- 4 * |k| * u_g, where u_g is the unit vector of the sum of the block's
  queries over b and over the query heads of group g. This makes them score high
  for every query head of the group.
* Outliers (``outlier_frac`` of the keys of each (sequence, KV head), positions
  uniform without replacement): k <- 3 * k (norm x3, direction kept).
* Per denoising step t: Q_t ~ law of Q, Kb_t ~ law of K without drift or
  planting, Vb_t ~ law of V. Q_0 is also the query the selection merges and the
  refine stage uses.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "Batch",
    "make_batch",
    "make_blocks",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + (((u >> 16) & 1) + 0x7FFF)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""

    name: str
    nseq: int
    L: int                       # context length, or the upper bound when ragged
    Hq: int
    Hkv: int
    d: int
    dtype: str                   # "f32" or "bf16"
    B: int                       # block size (queries per block)
    C: int                       # candidates kept by the merged-query scan
    topk: int                    # final budget
    T: int                       # denoising steps per block
    law: str = "gaussian"        # "gaussian" | "channel_scaled" | "drift"
    planted: int = 0             # planted high-score keys per (sequence, KV head)
    outlier_frac: float = 0.0    # fraction of keys scaled x3 per (sequence, KV head)
    L_min: Optional[int] = None  # ragged lengths ~ U{L_min..L} (inclusive) when set
    seed_base: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Names say what they are; sizes are in the fields.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_L4096", nseq=1, L=4096, Hq=4, Hkv=1, d=64, dtype="f32",
                 B=32, C=512, topk=256, T=4, law="gaussian", planted=16, seed_base=1000),
        Workload("gqa32x8_L32768_b1", nseq=1, L=32768, Hq=32, Hkv=8, d=128, dtype="bf16",
                 B=32, C=4096, topk=1024, T=8, law="channel_scaled", planted=64, seed_base=2000),
        Workload("gqa32x8_L32768_b16", nseq=16, L=32768, Hq=32, Hkv=8, d=128, dtype="bf16",
                 B=32, C=4096, topk=1024, T=8, law="channel_scaled", planted=64, seed_base=3000),
        Workload("gqa32x8_L131072_b4_drift", nseq=4, L=131072, Hq=32, Hkv=8, d=128, dtype="bf16",
                 B=32, C=8192, topk=1024, T=8, law="drift", planted=64, seed_base=4000),
        Workload("gqa28x4_ragged16k-64k_b8", nseq=8, L=65536, L_min=16384, Hq=28, Hkv=4, d=128,
                 dtype="bf16", B=32, C=4096, topk=2048, T=32, law="gaussian",
                 outlier_frac=0.01, seed_base=5000),
    ]
}


@dataclasses.dataclass
class Batch:
    """One batch of inputs. Float tensors hold uint16 bf16 bits, or float32 for fp32 workloads.

    Layouts (row-major, head_dim fastest):
      seq_start  int64 [nseq+1]      token offsets into the packed cache
      q0         [nseq][B][Hq][d]    the block's queries (merged for the scan, used by refine)
      k_cache    [sumL][Hkv][d]
      v_cache    [sumL][Hkv][d]
      q_steps    [T][nseq][B][Hq][d] per-step queries; q_steps[0] is q0
      kb_steps   [T][nseq][B][Hkv][d] per-step in-block keys
      vb_steps   [T][nseq][B][Hkv][d] per-step in-block values
      planted    list over s of int64 [Hkv][n] sequence-local positions of planted keys
    """

    wl: Workload
    seq_start: np.ndarray
    q0: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q_steps: np.ndarray
    kb_steps: np.ndarray
    vb_steps: np.ndarray
    planted: list

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.seq_start)

    def as_f64(self, name: str) -> np.ndarray:
        """A tensor widened exactly to float64 (the values every consumer computes on)."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _channel_scales(wl: Workload, gen: np.random.Generator):
    """Per-channel scales of Q, K and V (one vector per head per tensor), ones unless channel_scaled."""
    if wl.law == "channel_scaled":
        sq = gen.uniform(0.5, 2.0, size=(wl.Hq, wl.d)).astype(np.float32)
        sk = gen.uniform(0.5, 2.0, size=(wl.Hkv, wl.d)).astype(np.float32)
        sv = gen.uniform(0.5, 2.0, size=(wl.Hkv, wl.d)).astype(np.float32)
        return sq, sk, sv
    return (np.ones((wl.Hq, wl.d), np.float32), np.ones((wl.Hkv, wl.d), np.float32),
            np.ones((wl.Hkv, wl.d), np.float32))


def _lengths(wl: Workload) -> np.ndarray:
    if wl.L_min is None:
        return np.full(wl.nseq, wl.L, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed_base, 999_999])))
    return rng.integers(wl.L_min, wl.L, size=wl.nseq, endpoint=True).astype(np.int64)


def make_batch(wl: Workload, steps: Optional[int] = None) -> Batch:
    """Draw one batch for workload ``wl``. ``steps`` overrides the number of per-step draws (default T)."""
    T = wl.T if steps is None else steps
    lengths = _lengths(wl)
    seq_start = np.zeros(wl.nseq + 1, dtype=np.int64)
    seq_start[1:] = np.cumsum(lengths)
    total = int(seq_start[-1])
    bf16 = wl.dtype == "bf16"
    store = np.uint16 if bf16 else np.float32

    def finish(x: np.ndarray) -> np.ndarray:
        return f32_to_bf16_bits(x) if bf16 else x.astype(np.float32)

    def widen(x: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(x) if bf16 else x

    k_cache = np.empty((total, wl.Hkv, wl.d), dtype=store)
    v_cache = np.empty((total, wl.Hkv, wl.d), dtype=store)
    q0 = np.empty((wl.nseq, wl.B, wl.Hq, wl.d), dtype=store)
    q_steps = np.empty((T, wl.nseq, wl.B, wl.Hq, wl.d), dtype=store)
    kb_steps = np.empty((T, wl.nseq, wl.B, wl.Hkv, wl.d), dtype=store)
    vb_steps = np.empty((T, wl.nseq, wl.B, wl.Hkv, wl.d), dtype=store)
    planted = []

    for s in range(wl.nseq):
        L = int(lengths[s])
        names = ["q", "k", "v", "scale", "plant", "outlier", "drift", "steps"]
        streams = dict(zip(names, np.random.SeedSequence(wl.seed_base + s).spawn(len(names))))
        gen = {n: np.random.Generator(np.random.PCG64(ss)) for n, ss in streams.items()}

        sq, sk, sv = _channel_scales(wl, gen["scale"])

        qs = finish(gen["q"].standard_normal((wl.B, wl.Hq, wl.d), dtype=np.float32) * sq)
        q0[s] = qs

        k = gen["k"].standard_normal((L, wl.Hkv, wl.d), dtype=np.float32) * sk
        if wl.law == "drift":
            walk = np.zeros((L, wl.Hkv * wl.d), dtype=np.float64)
            walk[1:] = np.cumsum(0.01 * gen["drift"].standard_normal((L - 1, wl.Hkv * wl.d)), axis=0)
            k += walk.reshape(L, wl.Hkv, wl.d).astype(np.float32)
            del walk

        pos_s = np.zeros((wl.Hkv, 0), dtype=np.int64)
        if wl.planted:
            qw = widen(qs).astype(np.float64)  # [B][Hq][d]
            G = wl.G
            pos_s = np.empty((wl.Hkv, wl.planted), dtype=np.int64)
            for g in range(wl.Hkv):
                u = qw[:, g * G:(g + 1) * G, :].sum(axis=(0, 1))
                u /= np.linalg.norm(u)
                pos = np.sort(gen["plant"].choice(L, size=wl.planted, replace=False))
                pos_s[g] = pos
                norms = np.linalg.norm(k[pos, g, :].astype(np.float64), axis=1)
                k[pos, g, :] = (4.0 * norms[:, None] * u[None, :]).astype(np.float32)
        if wl.outlier_frac > 0:
            n_out = int(round(wl.outlier_frac * L))
            for g in range(wl.Hkv):
                pos = gen["outlier"].choice(L, size=n_out, replace=False)
                k[pos, g, :] *= np.float32(3.0)
        planted.append(pos_s)

        a, b = int(seq_start[s]), int(seq_start[s + 1])
        k_cache[a:b] = finish(k)
        del k
        v_cache[a:b] = finish(gen["v"].standard_normal((L, wl.Hkv, wl.d), dtype=np.float32) * sv)

        st = gen["steps"]
        for t in range(T):
            if t == 0:
                q_steps[0, s] = qs
            else:
                q_steps[t, s] = finish(st.standard_normal((wl.B, wl.Hq, wl.d), dtype=np.float32) * sq)
            kb_steps[t, s] = finish(st.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32) * sk)
            vb_steps[t, s] = finish(st.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32) * sv)

    return Batch(wl, seq_start, q0, k_cache, v_cache, q_steps, kb_steps, vb_steps, planted)


def make_blocks(wl: Workload, batch: Batch, nblocks: int) -> list:
    """Inputs of nblocks consecutive blocks over the batch's cache: block 0 is the batch's own
    (q0, q_steps, kb_steps, vb_steps); block i >= 1 draws its own queries and per-step
    in-block keys and values, with the sequence's channel scales, from a stream named by
    (seed_base + s, block i). The cache is the same for every block. Each entry is a dict
    with "q0" [nseq][B][Hq][d] and "q_steps", "kb_steps", "vb_steps" [T][nseq][B][H][d]."""
    blocks = [{"q0": batch.q0, "q_steps": batch.q_steps, "kb_steps": batch.kb_steps, "vb_steps": batch.vb_steps}]
    bf16 = wl.dtype == "bf16"
    T = batch.q_steps.shape[0]

    def finish(x: np.ndarray) -> np.ndarray:
        return f32_to_bf16_bits(x) if bf16 else x.astype(np.float32)

    for i in range(1, nblocks):
        q0 = np.empty_like(batch.q0)
        q_steps, kb_steps, vb_steps = (np.empty_like(a) for a in (batch.q_steps, batch.kb_steps, batch.vb_steps))
        for s in range(wl.nseq):
            names = ["q", "k", "v", "scale", "plant", "outlier", "drift", "steps"]
            scale_ss = np.random.SeedSequence(wl.seed_base + s).spawn(len(names))[names.index("scale")]
            sq, sk, sv = _channel_scales(wl, np.random.Generator(np.random.PCG64(scale_ss)))
            st = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed_base + s, 7_000_000 + i])))
            q0[s] = finish(st.standard_normal((wl.B, wl.Hq, wl.d), dtype=np.float32) * sq)
            for t in range(T):
                q_steps[t, s] = q0[s] if t == 0 else finish(st.standard_normal((wl.B, wl.Hq, wl.d),
                                                                               dtype=np.float32) * sq)
                kb_steps[t, s] = finish(st.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32) * sk)
                vb_steps[t, s] = finish(st.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32) * sv)
        blocks.append({"q0": q0, "q_steps": q_steps, "kb_steps": kb_steps, "vb_steps": vb_steps})
    return blocks
