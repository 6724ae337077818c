"""Move generated inputs between numpy storage and torch device tensors.

Plumbing only: bf16 bit patterns become ``torch.bfloat16`` tensors and back,
integer arrays become int32 tensors.  No model arithmetic happens here.
"""

from __future__ import annotations

from typing import Dict

import numpy as np
import torch


def to_torch(arr: np.ndarray, dtype: str = None, device="cuda") -> torch.Tensor:
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:          # bf16 bits
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    elif arr.dtype == np.float32:
        t = torch.from_numpy(arr)
    elif np.issubdtype(arr.dtype, np.integer):
        t = torch.from_numpy(arr.astype(np.int32))
    else:
        raise TypeError(arr.dtype)
    return t.to(device)


def from_torch(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload_weights(weights: Dict, device="cuda") -> Dict:
    out = {}
    for k, v in weights.items():
        if k == "layers":
            out[k] = [{n: to_torch(a, device=device) for n, a in lw.items()} for lw in v]
        else:
            out[k] = to_torch(v, device=device)
    return out


def upload_batch(batch, device="cuda") -> Dict:
    d = dict(query_lens=to_torch(batch.query_lens, device=device),
             target_ids=to_torch(batch.target_ids, device=device),
             target_pos=to_torch(batch.target_pos, device=device),
             num_accepted=to_torch(batch.num_accepted, device=device),
             bonus_ids=to_torch(batch.bonus_ids, device=device),
             target_hidden=to_torch(batch.target_hidden, device=device),
             block_table=to_torch(batch.block_table, device=device))
    d["k_cache"] = [to_torch(k, device=device) for k in batch.k_cache]
    d["v_cache"] = [to_torch(v, device=device) for v in batch.v_cache]
    return d
