#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

Default workload: Qwen3-0.6B-shaped single-layer decode, bf16 (batch 64, 16
query heads over 8 KV heads, head_dim 128, page_size 1 through a
token-granular req_to_token table of width 8192, KV lengths uniform in
[512, 4096], slots a seeded shuffle of a 400k-token pool).  One step is one
pass of the hot path over the batch: the KV append of the 64 new tokens
(kv_store) followed by paged decode attention (split-K partial kernel plus
the log-sum-exp merge).  Inputs are resident in HBM before timing starts.

Prints one JSON line with the whole-step throughput (algorithmic HBM bytes
per second), decode tokens/s, the roofline of the dominant kernel (the
split-K decode kernel, timed with HIP events on the launch stream) and the
oracle's CPU throughput on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published


# ---------------------------------------------------------------------------
# HIP events straight from the runtime, so the timer sits on the stream the
# library launches on.
# ---------------------------------------------------------------------------
class HipEvents:
    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self) -> int:
        e = C.c_void_p()
        assert self.hip.hipEventCreate(C.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(C.c_void_p(b)) == 0
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(C.c_void_p(e))


def i32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
class DecodeBench:
    """Decode step: optional kv_store of this step's tokens, optional
    build_kv_indices, then paged decode attention."""

    def __init__(self, case, fmt: str, dev="cuda"):
        import torch
        import paged_kv_cache_38_amd as P
        import workloads as W

        self.case, self.P, self.torch = case, P, torch
        g = case.geom
        dt = torch.float32 if g.dtype == "f32" else torch.bfloat16
        self.vals = W.make_values(case, device=dev)
        kb, vb = P.kv_pool_bytes(1, g.num_pages, g.page_size, g.num_kv_heads, g.head_dim_qk,
                                 g.head_dim_v, dt, g.latent)
        self.k_buf = self.vals["pool_k"].reshape(-1)
        self.v_buf = None if g.latent else self.vals["pool_v"].reshape(-1)
        assert self.k_buf.numel() * dt.itemsize == kb
        self.pool = P.kv_pool_create(self.k_buf, self.v_buf, num_layers=1, num_pages=g.num_pages,
                                     page_size=g.page_size, num_kv_heads=g.num_kv_heads, head_dim_qk=g.head_dim_qk,
                                     head_dim_v=g.head_dim_v, latent=g.latent)
        r = case.regions["self"]
        self.kv_lens = i32(r.kv_lens, dev)
        self.kv_start = i32(r.kv_start, dev)
        self.rpi = i32(case.req_pool_indices, dev)
        self.table = i32(case.req_to_token, dev)
        self.out_loc = i32(case.out_loc, dev)
        self.k_new = self.vals["k_new"]
        self.v_new = self.vals["v_new"]
        self.q = self.vals["q"]["self"]
        self.max_len = int(r.kv_lens.max())
        self.fmt = fmt
        ps = g.page_size
        per = -(-self.max_len // ps)
        if fmt == "token_table":
            self.map = P.make_kv_map(P.PKV_MAP_TOKEN_TABLE, self.kv_lens, self.max_len, req_to_token=self.table,
                                     req_pool_indices=self.rpi, kv_start=self.kv_start)
        elif fmt == "csr":
            self.indptr = torch.empty(case.bs + 1, dtype=torch.int32, device=dev)
            self.indices = torch.empty(case.bs * per, dtype=torch.int32, device=dev)
            self.map = P.make_kv_map(P.PKV_MAP_CSR, self.kv_lens, self.max_len, kv_indptr=self.indptr,
                                     kv_indices=self.indices)
        else:
            self.bt = torch.empty((case.bs, per), dtype=torch.int32, device=dev)
            self.map = P.make_kv_map(P.PKV_MAP_BLOCK_TABLE, self.kv_lens, self.max_len, block_table=self.bt)
        self.out = torch.empty((case.bs, g.num_q_heads, g.head_dim_v), dtype=dt, device=dev)
        self.lse = torch.empty((case.bs, g.num_q_heads), dtype=torch.float32, device=dev)
        nb = P.paged_decode_workspace_bytes(self.pool, case.bs, g.num_q_heads, self.max_len)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

    def step(self):
        P, c = self.P, self.case
        if c.n_new:
            P.kv_store(self.pool, 0, self.k_new, self.v_new, self.out_loc)
        ps = c.geom.page_size
        if self.fmt == "csr":
            P.build_kv_indices(P.PKV_MAP_CSR, self.table, self.rpi, self.kv_start, self.kv_lens, ps, self.max_len,
                               self.indptr, self.indices)
        elif self.fmt == "block_table":
            P.build_kv_indices(P.PKV_MAP_BLOCK_TABLE, self.table, self.rpi, self.kv_start, self.kv_lens, ps,
                               self.max_len, None, self.bt)
        P.paged_decode_attn(self.pool, 0, self.q, self.map, c.sm_scale, self.out, self.lse, self.ws)

    # algorithmic bytes ----------------------------------------------------
    def kernel_bytes(self) -> int:
        """Decode split kernel: each live token's K and V rows (all KV
        heads) once, its slot/page index, and the queries."""
        c, g = self.case, self.case.geom
        tok = int(c.regions["self"].kv_lens.sum())
        row = g.num_kv_heads * (g.head_dim_qk + (0 if g.latent else g.head_dim_v)) * g.elem_bytes
        idx = 4 if g.page_size == 1 or self.fmt == "token_table" else 4.0 / g.page_size
        return int(tok * (row + idx) + c.bs * g.num_q_heads * g.head_dim_qk * g.elem_bytes)

    def step_bytes(self) -> int:
        c, g = self.case, self.case.geom
        out_b = c.bs * g.num_q_heads * g.head_dim_v * g.elem_bytes
        row = g.num_kv_heads * (g.head_dim_qk + (0 if g.latent else g.head_dim_v)) * g.elem_bytes
        store_b = c.n_new * (2 * row + 4)
        return self.kernel_bytes() + out_b + store_b

    def kernel_flops(self) -> int:
        c, g = self.case, self.case.geom
        tok = int(c.regions["self"].kv_lens.sum())
        return 2 * tok * g.num_q_heads * (g.head_dim_qk + g.head_dim_v)

    def decode_tokens(self) -> int:
        return self.case.bs

    # CPU baseline: the oracle on a bounded sample --------------------------
    def cpu_baseline(self, budget_s: float = 15.0):
        import oracle
        from workloads.cases import to_numpy_bits

        c, g = self.case, self.case.geom
        r = c.regions["self"]
        self.torch.cuda.synchronize()
        pk = to_numpy_bits(self.pool.flat("k", 0))  # pool after this run's stores
        pv = None if g.latent else to_numpy_bits(self.pool.flat("v", 0))
        q = to_numpy_bits(self.q)
        slots = [oracle.slots_from_token_table(c.req_to_token, c.req_pool_indices[i], r.kv_start[i], r.kv_lens[i])
                 for i in range(c.bs)]
        # whole passes over the batch (request by request) until the budget is
        # spent, so the rate is measured over ~budget_s of oracle work
        reqs, toks, t0 = 0, 0, time.perf_counter()
        while True:
            for i in range(c.bs):
                oracle.paged_attention(q, c.q_lens, pk, pv, g.dtype, slots, c.sm_scale, True,
                                       head_dim_v=g.head_dim_v, requests=[i])
                reqs += 1
                toks += int(r.kv_lens[i])
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        row = g.num_kv_heads * (g.head_dim_qk + (0 if g.latent else g.head_dim_v)) * g.elem_bytes
        gbs = toks * (row + 4) / dt / 1e9
        return {"value": round(gbs, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
                "decode_tokens_per_s": round(reqs / dt, 3),
                "sample": f"{reqs} request decodes ({reqs / c.bs:.2f} passes over the {c.bs}-request batch, "
                          f"{toks} KV tokens) by the numpy fp64 oracle (gather + BLAS matmul per request), "
                          f"{dt:.1f} s"}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def build_workload(name: str):
    import workloads as W
    if name == "qwen3_decode":
        return W.qwen3_decode(seed=0), "token_table", {
            "workload": "qwen3_0.6b_decode_bf16", "batch": 64, "num_q_heads": 16, "num_kv_heads": 8,
            "head_dim": 128, "page_size": 1, "kv_len": "U[512,4096]", "pool_tokens": 400000,
            "table": "req_to_token [65, 8192]", "step": "kv_store + paged_decode_attn"}
    if name.startswith("gqa_prefix_share_ps"):
        ps = int(name[len("gqa_prefix_share_ps"):])
        return W.gqa_prefix_share(ps, seed=0), "csr", {
            "workload": f"gqa_prefix_share_decode_bf16_ps{ps}", "batch": 256, "num_q_heads": 32,
            "num_kv_heads": 8, "head_dim": 128, "page_size": ps, "kv_len": "lognormal(2048, 1) clip [64, 32768]",
            "prefix_share": "groups of 8 share 2048 tokens", "step": "build_kv_indices(CSR) + paged_decode_attn"}
    if name == "tiny_decode":
        return W.tiny_decode(seed=0), "csr", {"workload": "tiny_decode_f32", "batch": 4, "page_size": 16}
    raise SystemExit(f"unknown workload {name}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 256 MiB device copy three times (a known-size reference "
                         "for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.init()
    case, fmt, cfg = build_workload(args.workload)
    b = DecodeBench(case, fmt)
    ev = HipEvents()
    import paged_kv_cache_38_amd as P

    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        P.pkv_set_kernel_timer(*pairs[k])
        b.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [ev.elapsed_ms(a, z) for a, z in pairs]
    for a, z in pairs:
        ev.destroy(a)
        ev.destroy(z)

    ms_step = wall * 1e3 / args.steps
    k_ms = float(np.mean(kern_ms))
    step_gbs = b.step_bytes() / (ms_step * 1e-3) / 1e9
    kern_gbs = b.kernel_bytes() / (k_ms * 1e-3) / 1e9
    res = {
        "metric": "paged decode attn: achieved HBM GB/s (% of peak) + decode tokens/s, 1 GPU",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.geom.dtype,
        "data": "synthetic (seeded; N(0,1) values)",
        "config": cfg,
        "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(b.decode_tokens() / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": "decode split-K partial (paged_decode_attn)",
            "bound": "hbm",
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel_ms": round(k_ms, 5),
            "kernel_bytes": b.kernel_bytes(),
            "kernel_tflops": round(b.kernel_flops() / (k_ms * 1e-3) / 1e12, 3),
        },
    }
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = b.cpu_baseline(args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
