"""Shared helpers of the GPU tests: build inputs from the seeded workloads,
run the library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl
from oracle import checker

EPS = wl.EPS
CANARY = 0x7F7F  # a bf16 NaN pattern no result can take


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_bits(t: torch.Tensor) -> np.ndarray:
    return wl.bits(t)


class Case:
    """Host inputs of one call plus their device copies."""

    def __init__(self, w: wl.Workload, set_index: int = 0, M: int | None = None,
                 W: torch.Tensor | None = None, rope: bool = True):
        self.w = w
        self.nkv = w.nkv
        self.N = w.N
        self.x, self.positions, self.slots = wl.make_tokens(w, set_index, M=M)
        self.M = self.x.shape[0]
        self.W = wl.make_weights(w, set_index) if W is None else W
        self.cos_sin = wl.rope_table(w.table_rows) if rope else None
        self.cache = wl.make_cache(w)

    def device(self):
        dev = "cuda"
        g = {
            "x": self.x.to(dev), "W": self.W.to(dev), "positions": self.positions.to(dev),
            "slots": self.slots.to(dev),
            "cos_sin": None if self.cos_sin is None else self.cos_sin.to(dev),
            "kv_cache": self.cache.to(dev),
        }
        y = torch.empty(self.M, self.N, dtype=torch.bfloat16, device=dev)
        y.view(torch.int16).fill_(CANARY)
        g["y"] = y
        return g


def run_gpu(case: Case, g=None, label: str = "") -> dict:
    g = case.device() if g is None else g
    say(f"{label or case.w.name} M={case.M} nkv={case.nkv} N={case.N}")
    qf.prepare(case.N, case.nkv, case.M)
    qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"],
           M=case.M)
    torch.cuda.synchronize()
    assert qf.device_fault() == 0, "a call gave up waiting for a partial"
    return g


def check(case: Case, g, oracle_state=None) -> dict:
    return checker.check_front(
        to_bits(case.x), to_bits(case.W), case.positions.numpy(), case.slots.numpy(),
        None if case.cos_sin is None else case.cos_sin.numpy(), case.nkv, EPS,
        to_bits(case.cache), to_bits(g["y"]), to_bits(g["kv_cache"]),
        nthreads=oracle_threads(), oracle_state=oracle_state)
