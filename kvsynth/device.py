"""Copy synthetic workload tensors to the GPU (generation on the host, one batch row at a time)."""
from __future__ import annotations

import numpy as np
import torch

from . import K_ID, V_ID, Workload, kv_tensor, query


def kv_to_device(w: Workload, tensor_id: int, t0: int, t1: int, device="cuda", threads=None) -> torch.Tensor:
    """Tokens ``[t0, t1)`` of K (``K_ID``, with outlier channels) or V (``V_ID``) as a device float16 tensor
    ``[B, Hkv, t1 - t0, 128]``; the host holds one batch row at a time."""
    n_out, factor = (w.k_outliers, w.k_factor) if tensor_id == K_ID else (0, 1.0)
    out = torch.empty((w.batch, w.kv_heads, t1 - t0, w.head_dim), dtype=torch.float16, device=device)
    host = np.empty((1, w.kv_heads, t1 - t0, w.head_dim), dtype=np.float16)
    for b in range(w.batch):
        kv_tensor_row(w, tensor_id, b, t0, t1, n_out, factor, host, threads)
        out[b].copy_(torch.from_numpy(host[0]))
    return out


def kv_tensor_row(w, tensor_id, b, t0, t1, n_out, factor, host, threads):
    from concurrent.futures import ThreadPoolExecutor
    from . import slice_tokens

    def one(h):
        host[0, h] = slice_tokens(w.seed, tensor_id, b, h, t0, t1, w.head_dim, n_out, factor)

    if threads == 1 or w.kv_heads == 1:
        for h in range(w.kv_heads):
            one(h)
    else:
        import os
        n = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(one, range(w.kv_heads)))


def queries_to_device(w: Workload, steps, device="cuda") -> torch.Tensor:
    """Decode queries of the given step indices as a device float16 tensor ``[len(steps), B, Hq, 128]``."""
    return torch.from_numpy(np.stack([query(w.seed, s, w.batch, w.q_heads, w.head_dim) for s in steps])).to(device)


__all__ = ["kv_to_device", "queries_to_device", "K_ID", "V_ID", "kv_tensor"]
