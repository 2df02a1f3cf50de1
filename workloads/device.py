"""Copy a drawn batch to device tensors (lossless: every value is already
exactly representable in the workload's element type)."""
from __future__ import annotations

import numpy as np
import torch

from .inputs import Batch


def torch_dtype(batch: Batch) -> torch.dtype:
    return torch.bfloat16 if batch.workload.dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dtype)


def upload(batch: Batch, device="cuda") -> dict:
    dt = torch_dtype(batch)
    return {
        "q_nope": to_dev(batch.q_nope, dt, device),
        "q_rope": to_dev(batch.q_rope, dt, device),
        "w_uk": to_dev(batch.w_uk, dt, device),
        "w_uv": to_dev(batch.w_uv, dt, device),
        "q_abs": to_dev(batch.q_abs, dt, device),
        "pool": to_dev(batch.pool, dt, device),
        "block_table": torch.from_numpy(batch.block_table).to(device),
        "lengths": torch.from_numpy(batch.lengths).to(device),
        "seq_lens": torch.from_numpy(batch.seq_lens).to(device),
        "new_rows": to_dev(batch.new_rows, dt, device),
    }
