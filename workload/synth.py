"""Seeded synthetic Q/K/V for the H2O workloads.

Inputs only: nothing here computes attention, scores or evictions, so the GPU
path and the CPU oracle can both draw from it without sharing any of the
method's arithmetic.

Two generators produce inputs with the same recipe (N(0, 1) entries, anchor bias
on keys, the anchor direction added to queries, RNE rounding to the storage type):

* ``unit_qkv`` / ``batch_qkv`` (NumPy, Philox keyed by
  (config, layer, batch, head, stream, chunk of 1024 positions)).  Any unit or
  position range can be regenerated alone, bit for bit.  Used wherever the
  oracle checks every unit.
* ``torch_qkv`` (PyTorch generator on a device, keyed by (config, layer, stream,
  chunk of 4096 positions)).  Fast enough for the 32-layer and 4 M-token
  workloads; the oracle reads the generated tensors back for the units it samples.

Anchor layouts, directions and strengths come from NumPy in both cases.
"""
from __future__ import annotations

import numpy as np

from .configs import ROOT_SEED, Workload

STREAM_ID = {"q": 0, "k": 1, "v": 2}
NP_CHUNK = 1024
TORCH_CHUNK = 4096


# ----------------------------------------------------------------------------- rounding
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 result."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """The upper 16 bits (the bfloat16 encoding) of already-rounded float32 values."""
    return (np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32)
            >> np.uint32(16)).astype(np.uint16)


def round_storage(w: Workload, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_to_bf16(x) if w.dtype == "bf16" else x


# ----------------------------------------------------------------------------- anchors
def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(ROOT_SEED, spawn_key=key)))


def direction(w: Workload, layer: int, head: int, epoch: int = 0) -> np.ndarray:
    """Unit-norm float32 anchor direction of one head (and drift epoch)."""
    key = (w.cid, layer, head, 9) if epoch == 0 else (w.cid, layer, head, 9, epoch)
    u = _rng(*key).standard_normal(w.head_dim)
    return (u / np.linalg.norm(u)).astype(np.float32)


def n_drift_epochs(w: Workload) -> int:
    if w.anchor != "drift":
        return 0
    return -(-w.decode_steps // w.drift_every)


def anchors(w: Workload, layer: int, b: int):
    """Per-sequence anchor layout.

    Returns ``(alpha, key_epoch, query_epoch)``: float32 key-bias strength per
    position ``[N]``, the direction epoch used by each key ``[N]`` and by each
    query ``[N]`` (all zero unless the layout drifts).
    """
    n = w.n_positions
    g = _rng(w.cid, layer, b, 8)
    alpha = np.zeros(n, dtype=np.float32)
    key_epoch = np.zeros(n, dtype=np.int64)
    query_epoch = np.zeros(n, dtype=np.int64)
    if w.anchor == "fixed":
        pos = g.choice(n, size=min(w.n_anchors, n), replace=False)
        alpha[pos] = np.float32(w.alpha)
    elif w.anchor == "zipf":
        rho = g.permutation(n).astype(np.float64) + 1.0
        alpha[:] = (w.alpha * rho ** (-w.zipf_s)).astype(np.float32)
    elif w.anchor == "drift":
        pos0 = g.choice(w.prompt_len, size=min(w.n_anchors, w.prompt_len), replace=False)
        alpha[pos0] = np.float32(w.alpha)
        m_total = n_drift_epochs(w)
        offs = g.integers(0, w.drift_every, size=m_total)
        starts = w.prompt_len + w.drift_every * np.arange(m_total) + offs
        starts = starts[starts < n]
        for m, p in enumerate(starts, start=1):
            alpha[p] = np.float32(w.alpha)
            key_epoch[p] = m
        # queries follow the latest anchor at or before their own position
        if len(starts):
            query_epoch[:] = np.searchsorted(starts, np.arange(n), side="right")
    elif w.anchor == "none":
        pass
    else:
        raise ValueError(f"unknown anchor layout {w.anchor!r}")
    return alpha, key_epoch, query_epoch


def _dirs(w: Workload, layer: int, head: int, epochs: np.ndarray) -> np.ndarray:
    uniq = np.unique(epochs)
    table = {int(e): direction(w, layer, head, int(e)) for e in uniq}
    return np.stack([table[int(e)] for e in epochs]) if len(epochs) else np.zeros((0, w.head_dim), np.float32)


# ----------------------------------------------------------------------------- NumPy path
def _normals(w: Workload, layer: int, b: int, h: int, stream: str, start: int, stop: int) -> np.ndarray:
    out = np.empty((stop - start, w.head_dim), dtype=np.float32)
    c0, c1 = start // NP_CHUNK, (stop - 1) // NP_CHUNK if stop > start else start // NP_CHUNK - 1
    for c in range(c0, c1 + 1):
        blk = _rng(w.cid, layer, b, h, STREAM_ID[stream], c).standard_normal(
            (NP_CHUNK, w.head_dim), dtype=np.float32)
        lo, hi = max(start, c * NP_CHUNK), min(stop, (c + 1) * NP_CHUNK)
        out[lo - start:hi - start] = blk[lo - c * NP_CHUNK:hi - c * NP_CHUNK]
    return out


def unit_qkv(w: Workload, layer: int, b: int, h: int, start: int = 0, stop: int | None = None,
             _anchor_cache: dict | None = None):
    """Q, K, V of one unit over positions ``[start, stop)``: float32 ``[n, d]``,
    already rounded to the storage type (so float64 copies are exact)."""
    stop = w.n_positions if stop is None else stop
    if _anchor_cache is not None and (layer, b) in _anchor_cache:
        alpha, ke, qe = _anchor_cache[(layer, b)]
    else:
        alpha, ke, qe = anchors(w, layer, b)
        if _anchor_cache is not None:
            _anchor_cache[(layer, b)] = (alpha, ke, qe)
    sl = slice(start, stop)
    q = _normals(w, layer, b, h, "q", start, stop)
    k = _normals(w, layer, b, h, "k", start, stop)
    v = _normals(w, layer, b, h, "v", start, stop)
    if w.anchor != "none":
        k = k + alpha[sl, None] * _dirs(w, layer, h, ke[sl])
        q = q + _dirs(w, layer, h, qe[sl])
    return round_storage(w, q), round_storage(w, k), round_storage(w, v)


def batch_qkv(w: Workload, layer: int, start: int = 0, stop: int | None = None):
    """All units of one layer: float32 ``[B, H, n, d]`` each (rounded)."""
    stop = w.n_positions if stop is None else stop
    shape = (w.batch, w.heads, stop - start, w.head_dim)
    Q, K, V = (np.empty(shape, np.float32) for _ in range(3))
    cache: dict = {}
    for b in range(w.batch):
        for h in range(w.heads):
            Q[b, h], K[b, h], V[b, h] = unit_qkv(w, layer, b, h, start, stop, cache)
    return Q, K, V


# ----------------------------------------------------------------------------- torch path
def _torch_seed(*key: int) -> int:
    st = np.random.SeedSequence(ROOT_SEED, spawn_key=key).generate_state(2, np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def torch_qkv(w: Workload, layer: int, start: int, stop: int, device, out_dtype=None):
    """All units of one layer over positions ``[start, stop)`` as torch tensors
    ``[B, H, n, d]`` in the storage type, generated on ``device``."""
    import torch

    if out_dtype is None:
        out_dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    B, H, d, n = w.batch, w.heads, w.head_dim, stop - start
    res = []
    for stream in ("q", "k", "v"):
        x = torch.empty((B, H, n, d), dtype=torch.float32, device=device)
        c0, c1 = start // TORCH_CHUNK, (stop - 1) // TORCH_CHUNK
        for c in range(c0, c1 + 1):
            g = torch.Generator(device=device)
            g.manual_seed(_torch_seed(w.cid, layer, STREAM_ID[stream], c, 77))
            blk = torch.randn((B, H, TORCH_CHUNK, d), generator=g, dtype=torch.float32, device=device)
            lo, hi = max(start, c * TORCH_CHUNK), min(stop, (c + 1) * TORCH_CHUNK)
            x[:, :, lo - start:hi - start] = blk[:, :, lo - c * TORCH_CHUNK:hi - c * TORCH_CHUNK]
            del blk
        res.append(x)
    q, k, v = res
    if w.anchor != "none":
        al, ke, qe = [], [], []
        for b in range(B):
            a_, k_, q_ = anchors(w, layer, b)
            al.append(a_[start:stop]); ke.append(k_[start:stop]); qe.append(q_[start:stop])
        alpha = torch.from_numpy(np.stack(al)).to(device)  # [B, n]
        if w.anchor == "drift":
            epochs = np.unique(np.concatenate(ke + qe))
            idx = {int(e): i for i, e in enumerate(epochs)}
            U = torch.from_numpy(np.stack([[direction(w, layer, h, int(e)) for h in range(H)]
                                           for e in epochs])).to(device)  # [E, H, d]
            kei = torch.from_numpy(np.vectorize(idx.get)(np.stack(ke)).astype(np.int64)).to(device)
            qei = torch.from_numpy(np.vectorize(idx.get)(np.stack(qe)).astype(np.int64)).to(device)
            uk = U[kei].permute(0, 2, 1, 3)  # [B, H, n, d]
            uq = U[qei].permute(0, 2, 1, 3)
            k += alpha[:, None, :, None] * uk
            q += uq
        else:
            U = torch.from_numpy(np.stack([direction(w, layer, h) for h in range(H)])).to(device)
            k += alpha[:, None, :, None] * U[None, :, None, :]
            q += U[None, :, None, :]
    return q.to(out_dtype), k.to(out_dtype), v.to(out_dtype)


def to_torch(w: Workload, x_rounded: np.ndarray, device="cpu"):
    """Upload rounded float32 values in the storage type (exact)."""
    import torch

    if w.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x_rounded, np.float32)).to(device)
    bits = bf16_bits(x_rounded).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).to(device)
