"""Device-side helpers for the GPU tests: numpy <-> torch marshalling and one-call wrappers
around the C-ABI binding.  Nothing here computes attention."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_gqa_attention_decode_amd as pa

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives output capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """numpy -> contiguous device tensor; uint16 arrays are reinterpreted as f16/bf16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dtype])
    else:
        t = torch.from_numpy(a)
    return t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DecodeRun:
    """Device copies of a DecodeCase plus workspace; `step` runs write -> decode -> combine."""

    def __init__(self, case, num_splits=None, window=None):
        self.case = case
        self.S = int(num_splits or case.num_splits)
        self.window = int(case.window if window is None else window)
        dt = case.dtype
        self.q = dev(case.q)
        self.kp = dev(case.k_pages, dt)
        self.vp = dev(case.v_pages, dt)
        self.table = dev(case.page_table)
        self.ctx = dev(case.context_lens)
        self.k_new = dev(case.k_new, dt)
        self.v_new = dev(case.v_new, dt)
        self.owner = dev(case.token_table_index)
        self.pos = dev(case.token_position)
        B, Hq, D = case.q.shape
        self.po = torch.full((B, Hq, self.S, D), float("nan"), device=DEV)
        self.pml = torch.full((B, Hq, self.S, 2), float("nan"), device=DEV)
        self.out = torch.full((B, Hq, D), float("nan"), device=DEV)

    def write(self):
        pa.kv_page_write(self.k_new, self.v_new, self.kp, self.vp, self.table, self.owner,
                         self.pos)

    def decode(self):
        pa.paged_attn_decode(self.q, self.kp, self.vp, self.table, self.ctx, self.case.scale,
                             self.po, self.pml, window=self.window)
        pa.paged_attn_combine(self.po, self.pml, self.out)

    def step(self):
        self.write()
        self.decode()
        torch.cuda.synchronize()
        return host(self.out)

    def fused_step(self):
        """The same step as one launch (paged_attn_decode_fused)."""
        if not hasattr(self, "counters"):
            B, Hq, D = self.case.q.shape
            n = pa.paged_attn_decode_fused_counters(B, Hq, self.case.k_pages.shape[2])
            self.counters = torch.zeros(n, dtype=torch.int32, device=DEV)
        pa.paged_attn_decode_fused(self.q, self.k_new, self.v_new, self.kp, self.vp, self.table,
                                   self.ctx, self.case.scale, self.po, self.pml, self.counters,
                                   self.out, window=self.window)
        torch.cuda.synchronize()
        return host(self.out)
