"""Helpers for the GPU tests: run a problem through the C ABI and compare with
the fp64 oracle at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np

from lora_workloads import bf16_bits_to_f32
from segmented_gather_gemm_lora_amd import binding as B

# |gpu - ref| <= rel * (|ref| + floor)
TOL = {"f32": (1e-5, 1.0), "bf16": (2e-2, 1e-2)}


def say(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    B.load()
    return torch


def decode(arr, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).reshape(arr.shape).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def within_tol(gpu, ref, dtype):
    rel, floor = TOL[dtype]
    err = np.abs(gpu - ref)
    bound = rel * (np.abs(ref) + floor)
    ok = err <= bound
    return bool(ok.all()), float(np.max(err / bound)) if err.size else 0.0


def assert_close(gpu, ref, dtype, what=""):
    ok, worst = within_tol(gpu, ref, dtype)
    assert ok, f"{what}: worst |err|/bound = {worst:.3g}"
    return worst


def v_bound(prob, rows_x, ids_rows):
    """Rigorous fp32 summation bound for v rows: (d_in + 1) * 2^-24 * sum_k |x_k A_jk|."""
    x = np.abs(decode(prob.x, prob.dtype))
    rows_x = np.asarray(rows_x, dtype=np.int64)
    ids_rows = np.asarray(ids_rows)
    out = np.zeros((len(rows_x), max(prob.max_rank, 1)))
    for a in np.unique(ids_rows[ids_rows >= 0]):
        sel = np.nonzero(ids_rows == a)[0]
        A = np.abs(decode(prob.A(a), prob.dtype))
        out[sel, : A.shape[0]] = x[rows_x[sel]] @ A.T
    return (prob.d_in + 1) * 2.0**-24 * out + 1e-30


class GpuCase:
    """Device copies of one problem."""

    def __init__(self, prob, y_init="stored"):
        import torch

        self.torch = torch
        self.prob = prob
        self.dt = prob.dtype
        self.pool = B.DevicePool.from_problem(prob)
        self.x = B.to_device(prob.x, self.dt)
        if isinstance(y_init, str) and y_init == "stored":
            y = prob.y_base()
        elif isinstance(y_init, str) and y_init == "zero":
            y = np.zeros((prob.T, prob.d_out), dtype=np.uint16 if self.dt == "bf16" else np.float32)
        else:
            y = y_init
        self.y_host_in = y
        self.y = B.to_device(y, self.dt) if prob.T else None
        self.ids_dev = torch.from_numpy(np.ascontiguousarray(prob.ids, dtype=np.int32)).cuda()
        self.ldv = B.v_pitch(max(prob.max_rank, 1))

    def y_out(self):
        return decode(B.to_host_bits(self.y, self.dt), self.dt)

    def run_sgmv(self, stream=None):
        torch = self.torch
        plan = B.Plan(max(self.prob.T, 1)).build(self.prob.ids, self.pool).upload(stream)
        h = plan.header()
        v = torch.full((max(h["num_sorted"], 1), self.ldv), float("nan"), device="cuda")
        B.sgmv_shrink(self.x, plan, v, self.dt, stream=stream)
        B.sgmv_expand(v, plan, self.y, self.dt, stream=stream)
        torch.cuda.synchronize()
        self.plan = plan
        return v.cpu().numpy().astype(np.float64), plan

    def run(self, path, stream=None):
        """path: sgmv / bgmv (one combined call) or sgmv_split / bgmv_split
        (separate shrink and expand calls).  Returns (v or None, plan or None)."""
        if path == "sgmv_split":
            return self.run_sgmv(stream)
        if path == "bgmv_split":
            return self.run_bgmv(stream), None
        torch = self.torch
        p = self.prob
        if path == "sgmv":
            plan = B.Plan(max(p.T, 1)).build(p.ids, self.pool).upload(stream)
            ws = B.workspace(B.LORA_OP_SGMV, max(p.T, 1), p.d_in, p.d_out, max(p.max_rank, 1))
            B.sgmv(self.x, plan, self.y, ws, self.dt, stream=stream)
            torch.cuda.synchronize()
            self.plan = plan
            return None, plan
        if path == "bgmv":
            ws = B.workspace(B.LORA_OP_BGMV, max(p.T, 1), p.d_in, p.d_out, max(p.max_rank, 1))
            B.bgmv(self.x, self.ids_dev, self.pool, self.y, ws, self.dt, stream=stream)
            torch.cuda.synchronize()
            return None, None
        raise ValueError(path)

    def run_bgmv(self, stream=None):
        torch = self.torch
        v = torch.full((max(self.prob.T, 1), self.ldv), float("nan"), device="cuda")
        B.bgmv_shrink(self.x, self.ids_dev, self.pool, v, self.dt, stream=stream)
        B.bgmv_expand(v, self.ids_dev, self.pool, self.y, self.dt, stream=stream)
        torch.cuda.synchronize()
        return v.cpu().numpy().astype(np.float64)
