"""Grouped + residual streaming KV cache state machine (oracle; test infrastructure only).

KIVI page, paragraph on the recent-token window: per-channel key groups need 32 tokens, tokens arrive one at a
time, so the newest tokens (up to R = 128) stay in full precision and are quantized in blocks when the window
fills. synthetic.wiki "Keys are harder than values", last bullet: the key cache is split into a grouped part and a
residual part.

Readings taken where the pages are silent:
- the window covers keys and values alike;
- the flush is lazy: when a token arrives and the window already holds R tokens, the whole window is quantized
  (keys per channel in groups of 32 tokens, values per token) and emptied, then the token is stored; after any
  append the window therefore holds 1..R tokens;
- appending T tokens at once equals T single appends, so a prefill leaves the same state as a token-by-token
  decode (a flushed block is bit-identical to quantizing the same tokens at prefill);
- the flushed block is quantized with the same group quantizer as everywhere else.

A ``SliceCache`` holds any number S of independent (batch row, KV head) slices that share their lengths.

KVQuant variant (``sink=True``; synthetic.wiki "KV cache quantization", section "What they report", on the
attention sink: the first token's keys stay in full
precision). Reading taken: token 0 is held apart as the sink, its key in float16 and
its value quantized per token like any other value; the grouped and residual parts start at token 1, so key
groups cover tokens 1..32, 33..64, and so on, and the window logic above applies to the tokens after the sink.

Dense-and-sparse groups (``sparse=True``, ``oracle.sparse``): every flushed group, and the sink's value groups, keep
their largest-magnitude element apart (value and index) and quantize the rest; ``outliers()`` returns them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import quant, sparse as dsq


@dataclass
class SliceCache:
    """Logical state of S cache slices: quantized part (codes, scales, zeros) plus the fp16 residual window."""
    slices: int
    head_dim: int = 128
    residual_cap: int = 128
    group: int = 32
    bits: int = 2
    # quantized part, kept as lists of blocks and joined on demand
    _kq: list = field(default_factory=list)
    _ks: list = field(default_factory=list)
    _kz: list = field(default_factory=list)
    _vq: list = field(default_factory=list)
    _vs: list = field(default_factory=list)
    _vz: list = field(default_factory=list)
    n_quant: int = 0
    k_res: np.ndarray = None
    v_res: np.ndarray = None
    sink: bool = False
    k_sink: np.ndarray = None          # float16 [S, D] once the sink holds token 0
    v_sink: tuple = None               # (codes uint8 [S, D], scale float16 [S, D/32], zero float16 [S, D/32])
    sparse: bool = False               # per-vector dense-and-sparse groups (oracle.sparse)
    v_sink_out: tuple = None           # sparse: (outlier values float16 [S, D/32], channels uint8 [S, D/32])
    _ko: list = field(default_factory=list)
    _ki: list = field(default_factory=list)
    _vo: list = field(default_factory=list)
    _vi: list = field(default_factory=list)

    def __post_init__(self):
        if self.residual_cap % self.group:
            raise ValueError("residual capacity must be a multiple of the group size")
        if self.k_res is None:
            self.k_res = np.zeros((self.slices, 0, self.head_dim), np.float16)
            self.v_res = np.zeros((self.slices, 0, self.head_dim), np.float16)

    @property
    def n_resid(self) -> int:
        return self.k_res.shape[1]

    @property
    def n_sink(self) -> int:
        return 0 if self.k_sink is None else 1

    @property
    def n_tokens(self) -> int:
        return self.n_sink + self.n_quant + self.n_resid

    def _take_sink(self, k_tok: np.ndarray, v_tok: np.ndarray):
        """Token 0 of a sink cache: key kept as float16, value quantized per token."""
        self.k_sink = np.asarray(k_tok, np.float16).copy()
        v1 = np.asarray(v_tok, np.float16)[:, None, :]
        if self.sparse:
            vq, vs, vz, vo, vi = dsq.quantize_values_per_token_sparse(v1, self.group, self.bits)
            self.v_sink_out = (vo[:, 0], vi[:, 0])
        else:
            vq, vs, vz = quant.quantize_values_per_token(v1, self.group, self.bits)
        self.v_sink = (vq[:, 0], vs[:, 0], vz[:, 0])

    def quantized(self):
        """(k_codes [S,n_q,D], k_scale [S,n_q/32,D], k_zero, v_codes [S,n_q,D], v_scale [S,n_q,D/32], v_zero)."""
        S, D, g = self.slices, self.head_dim, self.group
        if not self._kq:
            e = np.zeros((S, 0, D), np.uint8)
            return (e, np.zeros((S, 0, D), np.float16), np.zeros((S, 0, D), np.float16),
                    e.copy(), np.zeros((S, 0, D // g), np.float16), np.zeros((S, 0, D // g), np.float16))
        if len(self._kq) > 1:
            for name in ("_kq", "_ks", "_kz", "_vq", "_vs", "_vz"):
                setattr(self, name, [np.concatenate(getattr(self, name), axis=1)])
        return self._kq[0], self._ks[0], self._kz[0], self._vq[0], self._vs[0], self._vz[0]

    def outliers(self):
        """Sparse caches: (key outlier values float16 [S, n_q/32, D], their tokens uint8, value outlier values
        float16 [S, n_q, D/32], their channels uint8)."""
        S, D, g = self.slices, self.head_dim, self.group
        if not self._ko:
            return (np.zeros((S, 0, D), np.float16), np.zeros((S, 0, D), np.uint8),
                    np.zeros((S, 0, D // g), np.float16), np.zeros((S, 0, D // g), np.uint8))
        if len(self._ko) > 1:
            for name in ("_ko", "_ki", "_vo", "_vi"):
                setattr(self, name, [np.concatenate(getattr(self, name), axis=1)])
        return self._ko[0], self._ki[0], self._vo[0], self._vi[0]

    def _push_quantized(self, k_tok: np.ndarray, v_tok: np.ndarray):
        if self.sparse:
            kq, ks, kz, ko, ki = dsq.quantize_keys_per_channel_sparse(k_tok, self.group, self.bits)
            vq, vs, vz, vo, vi = dsq.quantize_values_per_token_sparse(v_tok, self.group, self.bits)
            self._ko.append(ko); self._ki.append(ki); self._vo.append(vo); self._vi.append(vi)
        else:
            kq, ks, kz = quant.quantize_keys_per_channel(k_tok, self.group, self.bits)
            vq, vs, vz = quant.quantize_values_per_token(v_tok, self.group, self.bits)
        self._kq.append(kq); self._ks.append(ks); self._kz.append(kz)
        self._vq.append(vq); self._vs.append(vs); self._vz.append(vz)
        self.n_quant += k_tok.shape[1]

    def flush(self):
        """Quantize the whole residual window into the grouped part and empty the window."""
        if self.n_resid == 0:
            return
        self._push_quantized(self.k_res, self.v_res)
        self.k_res = self.k_res[:, :0]
        self.v_res = self.v_res[:, :0]

    def append_token(self, k_tok: np.ndarray, v_tok: np.ndarray):
        """One token per slice (float16 ``[S, D]``): flush a full window first, then store the token (the first
        token of a sink cache goes to the sink)."""
        if self.sink and self.k_sink is None:
            self._take_sink(k_tok, v_tok)
            return
        if self.n_resid == self.residual_cap:
            self.flush()
        self.k_res = np.concatenate([self.k_res, np.asarray(k_tok, np.float16)[:, None, :]], axis=1)
        self.v_res = np.concatenate([self.v_res, np.asarray(v_tok, np.float16)[:, None, :]], axis=1)

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """Append ``T`` tokens per slice (float16 ``[S, T, D]``) as ``T`` single appends, in order."""
        for i in range(k_new.shape[1]):
            self.append_token(k_new[:, i], v_new[:, i])


def flushed_tokens(n_resid0: int, t_new: int, residual_cap: int = 128) -> int:
    """Tokens that T single appends flush, starting from a window of ``n_resid0`` tokens.

    A flush happens at the i-th append exactly when the window is full before it, i.e. when n_resid0 + i - 1 is a
    positive multiple of R (1-based i); every flush empties R tokens. Counting them gives
    R * floor((n_resid0 + T - 1) / R) for T >= 1.
    """
    if t_new <= 0:
        return 0
    return residual_cap * ((n_resid0 + t_new - 1) // residual_cap)


def append_block(cache: SliceCache, k_new: np.ndarray, v_new: np.ndarray):
    """Same state as :meth:`SliceCache.append`, reached in one step.

    The flushed tokens are the first F of (window, new tokens) with F from :func:`flushed_tokens`; they are cut into
    blocks of R, each quantized as one flush would; the remaining tokens form the new window.
    """
    t = k_new.shape[1]
    if t == 0:
        return
    if cache.sink and cache.k_sink is None:
        cache._take_sink(k_new[:, 0], v_new[:, 0])
        k_new, v_new, t = k_new[:, 1:], v_new[:, 1:], t - 1
        if t == 0:
            return
    f = flushed_tokens(cache.n_resid, t, cache.residual_cap)
    k_all = np.concatenate([cache.k_res, np.asarray(k_new, np.float16)], axis=1)
    v_all = np.concatenate([cache.v_res, np.asarray(v_new, np.float16)], axis=1)
    if f:
        cache._push_quantized(k_all[:, :f], v_all[:, :f])
    cache.k_res = k_all[:, f:]
    cache.v_res = v_all[:, f:]
