#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

Default workload (the headline line): large-batch paged GQA decode with
prefix sharing, bf16 -- batch 256, 32 query heads over 8 KV heads, head_dim
128, page_size 16, KV lengths lognormal (median 2048, sigma 1, clipped to
[64, 32768]), groups of 8 requests reading the same physical pages for a
common 2048-token prefix, pool of 1.2x the pages needed in a seeded
free-list order.  One step is one pass of the hot path over the batch:
build_kv_indices (CSR) then paged_decode_attn (shared-prefix detection,
planner, the stream and shared-prefix work in one split-K launch,
log-sum-exp merge).  Inputs are resident in HBM before timing starts.  This
is the largest of the decode workloads that fit one GPU; the roofline
counts each distinct K/V row once.

Other workloads (--workload): qwen3_decode (Qwen3-0.6B-shaped decode: batch
64, 16 / 8 heads, head_dim 128, page_size 1 through a token table of width
8192, lengths U[512, 4096], the step's KV append in the planner launch),
gqa_prefix_share_ps64 (page size 64; the _cascade variants pass the
prefix groups to the cascade decode), mla_decode (latent 576/512, 128
heads, page_size 64), mla_verify (the same pool, 32 heads x 4 draft tokens
verified per request), encdec_extend (Whisper-shaped causal + cross extend
over a paged prefix), encdec_extend_ragged (the same through kv_gather and
contiguous K/V), mixed_spans_extend / _softcap (rows of a causal text span
and a full image span run as per-segment-flagged requests, without and with
softcap 30), tiny_decode (fp32 correctness shape), serving_alloc_decode /
serving_alloc_extend (one step of the device slot allocator: alloc, row
write and free; integer work bound by launch latency).

Prints one JSON line: whole-step throughput (algorithmic HBM bytes per
second), tokens per second, the roofline of the dominant kernel and the
oracle's CPU throughput on a bounded sample of the same workload.  The K
timed steps run with nothing else on the stream; the dominant kernel's
time comes from K more steps with HIP events recorded on the launch stream
around it.

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
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ROOT = os.path.dirname(os.path.abspath(__file__))


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel, from the
    FETCH_SIZE / WRITE_SIZE counter passes summarised under profiles/ (each
    scaled by what the counter reads for a plain copy of known size). None
    when no record exists or when the kernel's sources changed since the
    counters were taken (the record carries their sha256)."""
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("traffic_record: "):
                    continue
                rec = json.loads(line[len("traffic_record: "):])
                if rec.get("workload") != workload:
                    continue
                h = hashlib.sha256()
                try:
                    for src in rec["sources"]:
                        with open(os.path.join(ROOT, src), "rb") as sf:
                            h.update(sf.read())
                except OSError:
                    return None
                if h.hexdigest() != rec["sources_sha256"]:
                    return None
                return int(rec["traffic_bytes"])
    return None


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


def i32(a, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


_LIMITER = None


def _cpu_cores() -> dict:
    """The host cores this process may run on (its CPU affinity), with the
    BLAS pool set to that many threads; both are reported."""
    global _LIMITER
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        _LIMITER = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        pass
    return {"cores": cores, "blas_threads": _blas_threads()}


def _row_bytes(g) -> int:
    """One token's K and V rows over all KV heads (a latent row once)."""
    return g.num_kv_heads * (g.head_dim_qk + (0 if g.latent else g.head_dim_v)) * g.elem_bytes


def _make_pool(case, vals):
    """Pool built over the generated values (one layer)."""
    import paged_kv_cache_38_amd as P
    g = case.geom
    return P.kv_pool_create(vals["pool_k"].reshape(-1), None if g.latent else vals["pool_v"].reshape(-1),
                            num_layers=1, num_pages=g.num_pages, page_size=g.page_size, num_kv_heads=g.num_kv_heads,
                            head_dim_qk=g.head_dim_qk, head_dim_v=g.head_dim_v, latent=g.latent)


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------
class DecodeBench:
    """Decode step: kv_store of this step's tokens (if any), build_kv_indices
    (page-granular formats), then paged decode attention."""

    kernel_name = "paged decode split-K kernel (stream split)"
    attn_calls = 1
    tokens_label = "decode_tokens_per_s"

    def __init__(self, case, fmt: str, dev="cuda"):
        import torch
        import paged_kv_cache_38_amd as P
        import workloads as W

        self.case, self.P, self.torch = case, P, torch
        g = case.geom
        dt = torch.float32 if g.dtype == "f32" else torch.bfloat16
        self.vals = W.make_values(case, device=dev)
        self.pool = _make_pool(case, self.vals)
        r = case.regions["self"]
        self.kv_lens = i32(r.kv_lens, dev)
        self.kv_start = i32(r.kv_start, dev)
        self.rpi = i32(case.req_pool_indices, dev)
        self.table = i32(case.req_to_token, dev)
        self.out_loc = i32(case.out_loc, dev)
        self.k_new, self.v_new = self.vals["k_new"], self.vals["v_new"]
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
        # requests that share prefix pages read the same K/V rows: HBM has to
        # deliver each distinct row once (the rest can come from cache)
        self.logical_tokens = int(r.kv_lens.sum())
        slots = [np.repeat(np.asarray(pl, np.int64) * ps, ps)[:L] + np.tile(np.arange(ps), len(pl))[:L]
                 for pl, L in zip(r.page_lists, r.kv_lens.tolist())]
        self.unique_tokens = int(np.unique(np.concatenate(slots)).size) if slots else 0

    # the step's KV append rides in the decode call (its planner launch);
    # --separate-append issues kv_store on its own first
    fused_append = True

    def step(self, timers=None):
        P, c = self.P, self.case
        fused = c.n_new and self.fused_append
        if c.n_new and not fused:
            P.kv_store(self.pool, 0, self.k_new, self.v_new, self.out_loc)
        ps = c.geom.page_size
        if self.fmt == "csr":
            P.build_kv_indices(P.PKV_MAP_CSR, self.table, self.rpi, self.kv_start, self.kv_lens, ps, self.max_len,
                               self.indptr, self.indices)
        elif self.fmt == "block_table":
            P.build_kv_indices(P.PKV_MAP_BLOCK_TABLE, self.table, self.rpi, self.kv_start, self.kv_lens, ps,
                               self.max_len, None, self.bt)
        if timers:
            P.pkv_set_kernel_timer(*timers[0])
        if fused:
            P.paged_decode_attn_append(self.pool, 0, self.q, self.map, self.k_new, self.v_new, self.out_loc,
                                       c.sm_scale, self.out, self.lse, self.ws)
        else:
            P.paged_decode_attn(self.pool, 0, self.q, self.map, c.sm_scale, self.out, self.lse, self.ws)

    def kernel_bytes(self, logical: bool = False) -> int:
        """Decode kernel: the K/V rows of every distinct live slot once
        (every live token's, when logical), a slot id (or page id share) per
        token, and the queries."""
        c, g = self.case, self.case.geom
        idx = 4 if g.page_size == 1 or self.fmt == "token_table" else 4.0 / g.page_size
        rows = self.logical_tokens if logical else self.unique_tokens
        return int(rows * _row_bytes(g) + self.logical_tokens * idx +
                   c.bs * g.num_q_heads * g.head_dim_qk * g.elem_bytes)

    def step_bytes(self) -> int:
        c, g = self.case, self.case.geom
        out_b = c.bs * g.num_q_heads * g.head_dim_v * g.elem_bytes
        return self.kernel_bytes() + out_b + c.n_new * (2 * _row_bytes(g) + 4)

    def kernel_flops(self) -> int:
        c, g = self.case, self.case.geom
        tok = int(c.regions["self"].kv_lens.sum())
        return 2 * tok * g.num_q_heads * (g.head_dim_qk + g.head_dim_v)

    def tokens_per_step(self) -> int:
        return self.case.bs

    def cpu_baseline(self, budget_s: float):
        import oracle
        from workloads.cases import to_numpy_bits

        cpu = _cpu_cores()
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
        while time.perf_counter() - t0 <= budget_s:
            for i in range(c.bs):
                oracle.paged_attention(q, c.q_lens, pk, pv, g.dtype, slots, c.sm_scale, True,
                                       head_dim_v=g.head_dim_v, requests=[i])
                reqs += 1
                toks += int(r.kv_lens[i])
                if time.perf_counter() - t0 > budget_s:
                    break
        dt = time.perf_counter() - t0
        gbs = toks * (_row_bytes(g) + 4) / dt / 1e9
        return {"value": round(gbs, 4), "unit": "GB/s", **cpu, "kind": "oracle",
                "decode_tokens_per_s": round(reqs / dt, 3),
                "sample": f"{reqs} request decodes ({reqs / c.bs:.2f} passes over the {c.bs}-request batch, "
                          f"{toks} KV tokens) by the numpy fp64 oracle (gather + BLAS matmul per request), "
                          f"{dt:.1f} s"}


class CascadeBench(DecodeBench):
    """Decode step with the prefix groups known: build_kv_indices (CSR) then
    paged_decode_attn_cascade (each group's shared prefix read once, the own
    keys by the split-K kernel in the same launch, one log-sum-exp merge)."""

    kernel_name = "cascade decode: split-K kernel over own keys and the groups' shared prefixes (one launch)"

    def __init__(self, case, dev="cuda"):
        super().__init__(case, "csr", dev)
        g = case.geom
        indptr, plen = case.prefix_groups
        self.groups = self.P.make_prefix_groups(i32(indptr, dev), i32(plen, dev), int(np.diff(indptr).max()),
                                                int(plen.max()))
        nb = self.P.paged_decode_cascade_workspace_bytes(self.pool, case.bs, g.num_q_heads, self.max_len,
                                                         self.groups)
        self.ws = self.torch.empty(max(nb, 256), dtype=self.torch.uint8, device=dev)

    def step(self, timers=None):
        P, c = self.P, self.case
        P.build_kv_indices(P.PKV_MAP_CSR, self.table, self.rpi, self.kv_start, self.kv_lens, c.geom.page_size,
                           self.max_len, self.indptr, self.indices)
        if timers:
            P.pkv_set_kernel_timer(*timers[0])
        P.paged_decode_attn_cascade(self.pool, 0, self.q, self.map, self.groups, c.sm_scale, self.out, self.lse,
                                    self.ws)


class VerifyBench(DecodeBench):
    """Target-verification step over the MLA pool: kv_store of the drafts,
    build_kv_indices (block table), then paged_verify_attn (drafts folded
    into heads, bottom-right causal among them)."""

    kernel_name = "MLA decode kernel, target verification (drafts folded into heads)"
    tokens_label = "verified_tokens_per_s"

    def __init__(self, case, n_draft: int, dev="cuda"):
        super().__init__(case, "block_table", dev)
        g = case.geom
        self.n = n_draft
        self.qv = self.q.view(case.bs, n_draft, g.num_q_heads, g.head_dim_qk)
        self.out = self.torch.empty((case.bs, n_draft, g.num_q_heads, g.head_dim_v), dtype=self.torch.bfloat16,
                                    device=dev)
        self.lse = self.torch.empty((case.bs, n_draft, g.num_q_heads), dtype=self.torch.float32, device=dev)
        nb = self.P.paged_decode_workspace_bytes(self.pool, case.bs, n_draft * g.num_q_heads, self.max_len)
        self.ws = self.torch.empty(max(nb, 256), dtype=self.torch.uint8, device=dev)

    def step(self, timers=None):
        P, c = self.P, self.case
        if not self.fused_append:
            P.kv_store(self.pool, 0, self.k_new, self.v_new, self.out_loc)
        P.build_kv_indices(P.PKV_MAP_BLOCK_TABLE, self.table, self.rpi, self.kv_start, self.kv_lens,
                           c.geom.page_size, self.max_len, None, self.bt)
        if timers:
            P.pkv_set_kernel_timer(*timers[0])
        if self.fused_append:
            P.paged_verify_attn_append(self.pool, 0, self.qv, self.map, self.k_new, self.out_loc, c.sm_scale,
                                       self.out, self.lse, self.ws)
        else:
            P.paged_verify_attn(self.pool, 0, self.qv, self.map, c.sm_scale, self.out, self.lse, self.ws)

    def kernel_bytes(self, logical: bool = False) -> int:
        """Every distinct latent row once, a page id share per token, and the
        queries of every draft."""
        c, g = self.case, self.case.geom
        return int(self.unique_tokens * _row_bytes(g) + self.logical_tokens * 4.0 / g.page_size +
                   c.bs * self.n * g.num_q_heads * g.head_dim_qk * g.elem_bytes)

    def step_bytes(self) -> int:
        c, g = self.case, self.case.geom
        out_b = c.bs * self.n * g.num_q_heads * g.head_dim_v * g.elem_bytes
        return self.kernel_bytes() + out_b + c.n_new * (2 * _row_bytes(g) + 4)

    def kernel_flops(self) -> int:
        """Draft j of a request sees L - n + j + 1 keys."""
        c, g = self.case, self.case.geom
        L = c.regions["self"].kv_lens.astype(np.int64)
        pairs = int(np.sum(self.n * L - self.n * (self.n - 1) // 2))
        return 2 * pairs * g.num_q_heads * (g.head_dim_qk + g.head_dim_v)

    def tokens_per_step(self) -> int:
        return self.case.bs * self.n

    def cpu_baseline(self, budget_s: float):
        import oracle
        from workloads.cases import to_numpy_bits

        cpu = _cpu_cores()
        c, g = self.case, self.case.geom
        r = c.regions["self"]
        self.torch.cuda.synchronize()
        pk = to_numpy_bits(self.pool.flat("k", 0))
        q = to_numpy_bits(self.q)
        slots = [oracle.slots_from_token_table(c.req_to_token, c.req_pool_indices[i], r.kv_start[i], r.kv_lens[i])
                 for i in range(c.bs)]
        reqs, toks, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            for i in range(c.bs):
                oracle.paged_attention(q, c.q_lens, pk, None, g.dtype, slots, c.sm_scale, True,
                                       head_dim_v=g.head_dim_v, requests=[i])
                reqs += 1
                toks += int(r.kv_lens[i])
                if time.perf_counter() - t0 > budget_s:
                    break
        dt = time.perf_counter() - t0
        return {"value": round(toks * _row_bytes(g) / dt / 1e9, 4), "unit": "GB/s", **cpu,
                "kind": "oracle", "verified_tokens_per_s": round(reqs * self.n / dt, 3),
                "sample": f"{reqs} request verifications of {self.n} drafts ({toks} KV tokens) by the numpy fp64 "
                          f"oracle, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# extend workload (encoder-decoder)
# ---------------------------------------------------------------------------
class ExtendBench:
    """Extend step: kv_store of the new decoder tokens, CSR build for the
    decoder and encoder regions, causal extend over the decoder region and
    non-causal extend over the encoder region (ragged: kv_gather of both
    regions, then extend over the contiguous copies)."""

    attn_calls = 2
    tokens_label = "extend_tokens_per_s"

    def __init__(self, case, ragged: bool, softcap: float = 0.0, dev="cuda"):
        import torch
        import paged_kv_cache_38_amd as P
        import workloads as W

        self.case, self.P, self.torch, self.ragged, self.softcap = case, P, torch, ragged, softcap
        self.kernel_name = "paged extend attention kernel" + (" (contiguous K/V after kv_gather)" if ragged else "")
        if softcap:
            self.kernel_name += f" (softcap {softcap:g})"
        g = case.geom
        self.vals = W.make_values(case, device=dev)
        self.pool = _make_pool(case, self.vals)
        self.rpi = i32(case.req_pool_indices, dev)
        self.table = i32(case.req_to_token, dev)
        self.out_loc = i32(case.out_loc, dev)
        self.qo = i32(np.concatenate([[0], np.cumsum(case.q_lens)]), dev)
        self.max_q = int(case.q_lens.max())
        self.total_q = int(case.q_lens.sum())
        self.regions = {}
        for name, r in case.regions.items():
            maxl = int(r.kv_lens.max())
            per = max(-(-maxl // g.page_size), 1)
            d = {"kv_start": i32(r.kv_start, dev), "kv_lens": i32(r.kv_lens, dev), "max": maxl,
                 "flags": None if r.causal_flags is None else i32(r.causal_flags, dev),
                 "indptr": torch.empty(case.bs + 1, dtype=torch.int32, device=dev),
                 "indices": torch.empty(case.bs * per, dtype=torch.int32, device=dev),
                 "q": self.vals["q"][name], "causal": r.causal,
                 "out": torch.empty((self.total_q, g.num_q_heads, g.head_dim_v), dtype=torch.bfloat16, device=dev),
                 "lse": torch.empty((self.total_q, g.num_q_heads), dtype=torch.float32, device=dev)}
            d["map"] = P.make_kv_map(P.PKV_MAP_CSR, d["kv_lens"], maxl, kv_indptr=d["indptr"],
                                     kv_indices=d["indices"])
            if ragged:
                cu = np.concatenate([[0], np.cumsum(r.kv_lens)]).astype(np.int64)
                tot = int(cu[-1])
                d["cu"] = i32(cu, dev)
                d["k"] = torch.empty((max(tot, 1), g.num_kv_heads, g.head_dim_qk), dtype=torch.bfloat16, device=dev)
                d["v"] = torch.empty_like(d["k"])
                d["cmap"] = P.make_kv_map(P.PKV_MAP_CONTIGUOUS, d["kv_lens"], maxl, k=d["k"][:tot], v=d["v"][:tot],
                                          cu_seqlens_k=d["cu"])
            self.regions[name] = d

    def step(self, timers=None):
        P, c = self.P, self.case
        P.kv_store(self.pool, 0, self.vals["k_new"], self.vals["v_new"], self.out_loc)
        for k, (name, d) in enumerate(self.regions.items()):
            P.build_kv_indices(P.PKV_MAP_CSR, self.table, self.rpi, d["kv_start"], d["kv_lens"], c.geom.page_size,
                               d["max"], d["indptr"], d["indices"])
            m = d["map"]
            if self.ragged:
                P.kv_gather(self.pool, 0, m, d["cu"], d["k"], d["v"])
                m = d["cmap"]
            if timers:
                P.pkv_set_kernel_timer(*timers[k])
            if d["flags"] is None and not self.softcap:
                P.paged_extend_attn(self.pool, 0, d["q"], self.qo, self.max_q, m, d["causal"], c.sm_scale,
                                    d["out"], d["lse"])
            else:
                P.paged_extend_attn_ex(self.pool, 0, d["q"], self.qo, self.max_q, m, c.sm_scale, d["out"],
                                       d["lse"], causal=d["causal"], causal_flags=d["flags"], softcap=self.softcap)

    def _pairs(self, name) -> int:
        """Unmasked (query, key) pairs of one region."""
        c = self.case
        r = c.regions[name]
        n = c.q_lens.astype(np.int64)
        L = r.kv_lens.astype(np.int64)
        causal = np.full(len(n), bool(r.causal)) if r.causal_flags is None else r.causal_flags != 0
        # a causal request's query j sees L - n + j + 1 keys, a full one sees L
        return int(np.sum(np.where(causal, n * (L - n) + n * (n + 1) // 2, n * L)))

    def kernel_flops(self) -> int:
        g = self.case.geom
        return sum(self._pairs(nm) for nm in self.case.regions) * g.num_q_heads * 2 * (g.head_dim_qk + g.head_dim_v)

    def kernel_bytes(self, logical: bool = False) -> int:
        """Both extend calls: every key row of both regions once, the queries
        and the outputs of both calls (no row is shared between requests, so
        logical and distinct bytes are the same)."""
        c, g = self.case, self.case.geom
        rows = sum(int(r.kv_lens.sum()) for r in c.regions.values())
        qo = 2 * self.total_q * g.num_q_heads * g.head_dim_qk * g.elem_bytes
        return rows * _row_bytes(g) + 2 * qo

    def step_bytes(self) -> int:
        c, g = self.case, self.case.geom
        b = self.kernel_bytes() + c.n_new * (2 * _row_bytes(g) + 4)
        if self.ragged:
            rows = sum(int(r.kv_lens.sum()) for r in c.regions.values())
            b += 2 * rows * _row_bytes(g)  # gather reads and writes every row once more
        return b

    def tokens_per_step(self) -> int:
        return self.total_q

    def cpu_baseline(self, budget_s: float):
        import oracle
        from workloads.cases import to_numpy_bits

        cpu = _cpu_cores()
        c, g = self.case, self.case.geom
        self.torch.cuda.synchronize()
        pk, pv = to_numpy_bits(self.pool.flat("k", 0)), to_numpy_bits(self.pool.flat("v", 0))
        qs = {nm: to_numpy_bits(self.vals["q"][nm]) for nm in c.regions}
        reqs, toks, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            for i in range(c.bs):
                for nm, r in c.regions.items():
                    slots = [oracle.slots_from_token_table(c.req_to_token, c.req_pool_indices[i], r.kv_start[i],
                                                           r.kv_lens[i]) if j == i else np.zeros(0, np.int64)
                             for j in range(c.bs)]
                    causal = r.causal if r.causal_flags is None else [bool(f) for f in r.causal_flags]
                    oracle.paged_attention(qs[nm], c.q_lens, pk, pv, g.dtype, slots, c.sm_scale, causal,
                                           requests=[i], softcap=self.softcap)
                reqs += 1
                toks += int(c.q_lens[i])
                if time.perf_counter() - t0 > budget_s:
                    break
        dt = time.perf_counter() - t0
        return {"value": round(toks / dt, 2), "unit": "extend tokens/s", **cpu, "kind": "oracle",
                "sample": f"{reqs} request extends ({' + '.join(c.regions)}; {reqs / c.bs:.2f} passes over the "
                          f"{c.bs}-request batch, {toks} new tokens) by the numpy fp64 oracle, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# encoder-embedding block cache workload
# ---------------------------------------------------------------------------
class EncCacheBench:
    """Encoder cache step at the Neuron notes' Qwen3-VL geometry: the encoder's
    8 output blocks scattered into the cache (6 items + 2 padding blocks to
    the scratch block), then 8 blocks gathered and merged into the batch's
    hidden rows by the position map (2865 real tokens of 40 KiB)."""

    attn_calls = 1
    dtype = "bf16"
    tokens_label = "merged_tokens_per_s"
    kernel_name = "encoder cache: enc_write_kernel + enc_merge_kernel"

    def __init__(self, dev="cuda"):
        import torch
        import paged_kv_cache_38_amd as P
        from workloads.enc_cache import enc_cache_case

        self.P, self.torch, self.case = P, torch, None
        self.w = w = enc_cache_case(seed=0)
        g = torch.Generator(device=dev).manual_seed(w.value_seed)
        shape = (w.block_size, w.fat_dim)
        self.buf = torch.randn((w.num_blocks, *shape), generator=g, device=dev).to(torch.bfloat16)
        self.src = torch.randn((len(w.write_ids), *shape), generator=g, device=dev).to(torch.bfloat16)
        self.hidden = torch.zeros((w.num_tokens, w.fat_dim), dtype=torch.bfloat16, device=dev)
        self.write_ids = i32(w.write_ids, dev)
        self.gather_ids = i32(w.gather_ids, dev)
        self.pos = torch.from_numpy(w.positions).to(dev)
        self.row = w.fat_dim * 2
        self.stream = torch.cuda.current_stream().cuda_stream
        self.hip = HipEvents().hip
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def step(self, timers=None):
        P = self.P
        if timers:
            assert self.hip.hipEventRecord(C.c_void_p(timers[0][0]), C.c_void_p(self.stream)) == 0
        P.enc_cache_write(self.buf, self.src, self.write_ids)
        P.enc_cache_merge(self.buf, self.gather_ids, self.pos, self.hidden)
        if timers:
            assert self.hip.hipEventRecord(C.c_void_p(timers[0][1]), C.c_void_p(self.stream)) == 0

    def kernel_bytes(self, logical: bool = False) -> int:
        """Every written block read and written once, every real gathered
        token's row read and written once, plus the position map."""
        w = self.w
        return (2 * len(w.write_ids) * w.block_size * self.row + 2 * w.real_tokens * self.row +
                w.positions.size * 8 + 4 * (len(w.write_ids) + len(w.gather_ids)))

    def step_bytes(self) -> int:
        return self.kernel_bytes()

    def kernel_flops(self) -> int:
        return 0

    def tokens_per_step(self) -> int:
        return self.w.real_tokens

    def cpu_baseline(self, budget_s: float):
        import oracle
        from workloads.cases import to_numpy_bits

        cpu = _cpu_cores()
        w = self.w
        self.torch.cuda.synchronize()
        buf = to_numpy_bits(self.buf)
        src = to_numpy_bits(self.src)
        hidden = to_numpy_bits(self.hidden)
        steps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            b2 = oracle.write_blocks(buf, src, w.write_ids)
            oracle.merge_blocks(b2, w.gather_ids, w.positions, hidden, w.num_tokens)
            steps += 1
        dt = time.perf_counter() - t0
        return {"value": round(steps * self.kernel_bytes() / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                "cores_available": cpu["cores"],
                "kind": "oracle", "merged_tokens_per_s": round(steps * w.real_tokens / dt, 1),
                "sample": f"{steps} whole write + merge steps by the numpy oracle (a full buffer copy per write), "
                          f"{dt:.1f} s"}


# ---------------------------------------------------------------------------
# slot allocation workload
# ---------------------------------------------------------------------------
class AllocBench:
    """Slot allocation step: kv_alloc_decode (or kv_alloc_extend) of the
    batch, write_req_to_token of the new slots into the requests' rows, then
    kv_free of the same slots, which returns exactly the pages just taken
    (every prefix is page aligned), so every step does the same work."""

    attn_calls = 1
    dtype = "int32"
    tokens_label = "new_slots_per_s"
    metric = "slot allocation step (alloc + row write + free): new slots per second, 1 GPU"
    unit = "slots/s"

    def __init__(self, decode: bool, dev="cuda"):
        import torch
        import paged_kv_cache_38_amd as P
        from workloads.alloc import serving_alloc

        self.P, self.torch, self.decode = P, torch, decode
        self.kernel_name = ("allocation step: " + ("kv_alloc_decode" if decode else "kv_alloc_extend") +
                            " + write_req_to_token + kv_free (6 launches)")
        self.w = w = serving_alloc(decode)
        self.case = None
        self.bs = len(w.seq_lens)
        self.new = int((w.seq_lens - w.prefix_lens).sum())
        self.pages = int(sum(-(-int(s) // w.page_size) - int(p) // w.page_size
                             for p, s in zip(w.prefix_lens, w.seq_lens)))
        self.fl = P.kv_free_list_create(w.page_size, w.num_pages, device=dev)
        self.prefix, self.seq, self.rpi = i32(w.prefix_lens, dev), i32(w.seq_lens, dev), i32(w.req_pool_indices, dev)
        self.last = i32(np.full(self.bs, -1), dev)
        self.out = torch.empty(self.new, dtype=torch.int32, device=dev)
        self.table = torch.zeros((self.bs + 1, w.table_width), dtype=torch.int32, device=dev)
        self.max_seq = int(w.seq_lens.max())
        self.stream = torch.cuda.current_stream().cuda_stream
        self.hip = HipEvents().hip
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def step(self, timers=None):
        P = self.P
        if timers:
            assert self.hip.hipEventRecord(C.c_void_p(timers[0][0]), C.c_void_p(self.stream)) == 0
        if self.decode:
            P.kv_alloc_decode(self.fl, self.seq, self.last, self.out)
        else:
            P.kv_alloc_extend(self.fl, self.prefix, self.seq, self.last, self.out)
        P.write_req_to_token(self.table, self.rpi, self.prefix, self.seq, self.out, self.max_seq)
        P.kv_free(self.fl, self.out)
        if timers:
            assert self.hip.hipEventRecord(C.c_void_p(timers[0][1]), C.c_void_p(self.stream)) == 0

    def check(self):
        """Every step must be granted: the free list is back at full size."""
        self.torch.cuda.synchronize()
        st = int(self.fl.status.item())
        size = int(self.fl.state[1].item())
        if st != 0 or size != self.w.num_pages:
            raise SystemExit(f"allocation step left status {st}, free size {size} (expected 0, {self.w.num_pages})")

    def kernel_bytes(self, logical: bool = False) -> int:
        """Lengths read by the allocator and the row writer, the ring entries
        taken and given back, the new slots written, read back by the row
        writer and by the free, the table cells written, and the free's page
        bitmap cleared, marked and read."""
        words = (self.w.num_pages + 31) // 32
        lens = self.bs * (4 if self.decode else 8) + self.bs * 12
        return lens + 2 * self.pages * 4 + 4 * self.new * 4 + 3 * words * 4

    def step_bytes(self) -> int:
        return self.kernel_bytes()

    def kernel_flops(self) -> int:
        return 0

    def tokens_per_step(self) -> int:
        return self.new

    def value(self, ms_step: float) -> float:
        return self.new / (ms_step * 1e-3)

    def cpu_baseline(self, budget_s: float):
        import oracle

        w = self.w
        ring = oracle.FreeRing(list(range(w.num_pages)), w.num_pages)
        table = np.zeros((self.bs + 1, w.table_width), np.int64)
        last = [-1] * self.bs
        steps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            slots = oracle.alloc_extend(ring, w.page_size, w.prefix_lens, w.seq_lens, last)
            table = oracle.write_req_to_token(table, w.req_pool_indices, w.prefix_lens, w.seq_lens, slots)
            oracle.free_pages(ring, oracle.pages_of_slots(slots, w.page_size))
            steps += 1
        dt = time.perf_counter() - t0
        return {"value": round(steps * self.new / dt, 1), "unit": "slots/s", "cores": 1,
                "cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
                "sample": f"{steps} whole allocation steps ({steps * self.new} slots) by the Python oracle, "
                          f"{dt:.1f} s"}


def build_workload(name: str):
    import workloads as W
    if name == "qwen3_decode":
        return DecodeBench(W.qwen3_decode(seed=0), "token_table"), {
            "workload": "qwen3_0.6b_decode_bf16", "batch": 64, "num_q_heads": 16, "num_kv_heads": 8,
            "head_dim": 128, "page_size": 1, "kv_len": "U[512,4096]", "pool_tokens": 400000,
            "table": "req_to_token [65, 8192]", "step": "kv_store + paged_decode_attn"}
    if name.startswith("gqa_prefix_share_ps") and name.endswith("_cascade"):
        ps = int(name[len("gqa_prefix_share_ps"):-len("_cascade")])
        return CascadeBench(W.gqa_prefix_share(ps, seed=0)), {
            "workload": f"gqa_prefix_share_decode_bf16_ps{ps}_cascade", "batch": 256, "num_q_heads": 32,
            "num_kv_heads": 8, "head_dim": 128, "page_size": ps, "kv_len": "lognormal(2048, 1) clip [64, 32768]",
            "prefix_share": "groups of 8 share 2048 tokens, passed as prefix groups",
            "step": "build_kv_indices(CSR) + paged_decode_attn_cascade"}
    if name.startswith("gqa_prefix_share_ps"):
        ps = int(name[len("gqa_prefix_share_ps"):])
        return DecodeBench(W.gqa_prefix_share(ps, seed=0), "csr"), {
            "workload": f"gqa_prefix_share_decode_bf16_ps{ps}", "batch": 256, "num_q_heads": 32,
            "num_kv_heads": 8, "head_dim": 128, "page_size": ps, "kv_len": "lognormal(2048, 1) clip [64, 32768]",
            "prefix_share": "groups of 8 share 2048 tokens", "step": "build_kv_indices(CSR) + paged_decode_attn"}
    if name == "mla_decode":
        return DecodeBench(W.mla_decode(seed=0), "block_table"), {
            "workload": "mla_decode_bf16", "batch": 128, "num_q_heads": 128, "head_dim_qk": 576, "head_dim_v": 512,
            "page_size": 64, "kv_len": "U[4096,16384]",
            "step": "kv_store + build_kv_indices(BLOCK_TABLE) + paged_decode_attn"}
    if name == "mla_verify":
        return VerifyBench(W.mla_decode(seed=0, num_q_heads=32, num_draft=4), 4), {
            "workload": "mla_target_verify_bf16", "batch": 128, "num_q_heads": 32, "num_draft": 4,
            "rows_per_request": 128, "head_dim_qk": 576, "head_dim_v": 512, "page_size": 64,
            "kv_len": "U[4096,16384] including the drafts",
            "step": "kv_store (drafts) + build_kv_indices(BLOCK_TABLE) + paged_verify_attn"}
    if name in ("encdec_extend", "encdec_extend_ragged"):
        ragged = name.endswith("ragged")
        return ExtendBench(W.encdec_extend(seed=0), ragged), {
            "workload": "whisper_encdec_extend_bf16" + ("_ragged" if ragged else ""), "batch": 32, "num_heads": 20,
            "head_dim": 64, "page_size": 16, "encoder_len": 1500, "decoder_prefix": "U{0..448}",
            "new_tokens": "U{1..512}",
            "step": "kv_store + build_kv_indices(CSR) x2 + " + ("kv_gather x2 + " if ragged else "")
                    + "paged_extend_attn (causal self + cross)"}
    if name == "enc_cache_qwen3vl":
        return EncCacheBench(), {
            "workload": "encoder_cache_qwen3vl_bf16", "num_blocks": 33, "block_size": 512, "fat_dim": 20480,
            "written_blocks": "8 (6 items + 2 padding to the scratch block)", "gathered_blocks": 8,
            "real_tokens": 2865, "num_tokens": 8192, "step": "enc_cache_write + enc_cache_merge"}
    if name in ("serving_alloc_decode", "serving_alloc_extend"):
        dec = name.endswith("decode")
        return AllocBench(dec), {
            "workload": name, "batch": 4096 if dec else 64, "page_size": 16, "pool_pages": 65536,
            "prefix": "page aligned, " + ("U[512,4096)" if dec else "U[0,4096)"),
            "new_tokens": "1 (every request opens a page)" if dec else "U[1,2048]",
            "step": ("kv_alloc_decode" if dec else "kv_alloc_extend") + " + write_req_to_token + kv_free"}
    if name in ("mixed_spans_extend", "mixed_spans_extend_softcap"):
        cap = 30.0 if name.endswith("softcap") else 0.0
        b = ExtendBench(W.mixed_spans(seed=0), False, softcap=cap)
        b.attn_calls = 1
        return b, {
            "workload": name, "rows": 4, "spans": "causal text 128 + full image 2048 per row, one segment each",
            "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16, "softcap": cap,
            "step": "kv_store of every row token + build_kv_indices(CSR) + paged_extend_attn_ex "
                    "(per-segment causal flags)"}
    if name == "tiny_decode":
        return DecodeBench(W.tiny_decode(seed=0), "csr"), {"workload": "tiny_decode_f32", "batch": 4, "page_size": 16}
    raise SystemExit(f"unknown workload {name}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_prefix_share_ps16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="after the timed steps, time the kernel this many more times with the caches "
                         "cleared (a 1 GiB read) before each step; reported as roofline.kernel_ms_cold")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode and verification workloads: launch kv_store on its own before the attention "
                         "call instead of passing the append to paged_decode_attn_append / "
                         "paged_verify_attn_append")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the plain 1 GiB device copy and the 8192^3 bf16 GEMM that report "
                         "roofline.attainable_copy_gbs and roofline.attainable_gemm_tflops")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 256 MiB device copy three times (a known-size reference "
                         "for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.init()
    b, cfg = build_workload(args.workload)
    if isinstance(b, DecodeBench) and b.case.n_new:
        b.fused_append = not args.separate_append
        if b.fused_append and "step" in cfg:
            cfg["step"] = cfg["step"].replace("kv_store (drafts) + ", "").replace("kv_store + ", "").replace(
                "paged_decode_attn", "paged_decode_attn_append (the kv_store runs in its planner launch)").replace(
                "paged_verify_attn", "paged_verify_attn_append (the drafts' kv_store runs in its planner launch)")
    ev = HipEvents()
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    # the timed region: exactly K steps and nothing else on the stream
    t0 = time.perf_counter()
    for _ in range(args.steps):
        b.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel times: K more steps with HIP events recorded around the
    # attention call(s) (event records between launches cost the stream a
    # few microseconds, so they stay out of the timed steps above)
    pairs = [[(ev.create(), ev.create()) for _ in range(b.attn_calls)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        b.step(pairs[k])
    torch.cuda.synchronize()
    call_ms = [[ev.elapsed_ms(a, z) for a, z in step] for step in pairs]
    kern_ms = [sum(c) for c in call_ms]
    for step in pairs:
        for a, z in step:
            ev.destroy(a)
            ev.destroy(z)

    ms_step = wall * 1e3 / args.steps
    k_ms = float(np.mean(kern_ms))
    step_gbs = b.step_bytes() / (ms_step * 1e-3) / 1e9
    kern_gbs = b.kernel_bytes() / (k_ms * 1e-3) / 1e9
    kern_tf = b.kernel_flops() / (k_ms * 1e-3) / 1e12
    # the roof that bounds the kernel at its arithmetic intensity: HBM below
    # the ridge point (peak flop/s / peak bytes/s = 312.5 flop/B), MFMA above
    intensity = b.kernel_flops() / max(b.kernel_bytes(), 1)
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kern_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(kern_tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kern_tf / BF16_PEAK_TFLOPS, 4)}
    roof.update({"traffic": measured_traffic(args.workload), "kernel": b.kernel_name, "kernel_ms": round(k_ms, 5),
                 "kernel_bytes": b.kernel_bytes(), "kernel_gbs": round(kern_gbs, 2),
                 "kernel_hbm_frac": round(kern_gbs / HBM_PEAK_GBS, 4), "kernel_tflops": round(kern_tf, 3),
                 "kernel_mfma_frac": round(kern_tf / BF16_PEAK_TFLOPS, 4),
                 "flop_per_byte": round(intensity, 2),
                 "kernel_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(kern_ms, [10, 50, 90])]})
    if b.attn_calls > 1:
        roof["call_ms"] = [round(float(np.mean([c[k] for c in call_ms])), 5) for k in range(b.attn_calls)]
    if b.kernel_bytes(logical=True) != b.kernel_bytes():
        # shared prefix pages: the kernel reads more rows than there are
        # distinct ones; the roofline counts each distinct row once
        lb = b.kernel_bytes(logical=True)
        roof.update({"kernel_logical_bytes": lb, "kernel_logical_gbs": round(lb / (k_ms * 1e-3) / 1e9, 2)})
    if args.cold_steps > 0:
        # the same kernel with the caches cleared first: a 1 GiB buffer is
        # read before each step (MALL and L2 are smaller; reading leaves no
        # dirty lines to write back during the kernel), outside the events
        # that time the kernel
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        cold = [[(ev.create(), ev.create()) for _ in range(b.attn_calls)] for _ in range(args.cold_steps)]
        for k in range(args.cold_steps):
            flush.sum()
            b.step(cold[k])
        torch.cuda.synchronize()
        cold_ms = float(np.mean([sum(ev.elapsed_ms(a, z) for a, z in st) for st in cold]))
        for st in cold:
            for a, z in st:
                ev.destroy(a)
                ev.destroy(z)
        del flush
        cold_gbs = b.kernel_bytes() / (cold_ms * 1e-3) / 1e9
        roof.update({"kernel_ms_cold": round(cold_ms, 5), "kernel_gbs_cold": round(cold_gbs, 2),
                     "kernel_hbm_frac_cold": round(cold_gbs / HBM_PEAK_GBS, 4)})
    res = {
        "metric": getattr(b, "metric", "paged decode attn: achieved HBM GB/s (% of peak) + decode tokens/s, 1 GPU"),
        "value": round(b.value(ms_step), 1) if hasattr(b, "value") else round(step_gbs, 2),
        "unit": getattr(b, "unit", "GB/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.case.geom.dtype if b.case is not None else b.dtype,
        "data": "synthetic (seeded; N(0,1) values)",
        "config": cfg,
        "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        b.tokens_label: round(b.tokens_per_step() / (ms_step * 1e-3), 1),
        # the same count over the timed kernel(s) alone (attention only for the
        # decode and extend workloads: no append, planner or merge)
        b.tokens_label + "_kernel_only": round(b.tokens_per_step() / (k_ms * 1e-3), 1),
        "roofline": roof,
    }
    if not args.no_attainable and not args.calibrate_copy:
        # the attainable HBM rate on this machine: a plain 1 GiB device-to-device
        # copy (read + write bytes over its event time), beside the 8 TB/s peak
        # (left out of counter runs, whose known-size copy must stay the largest)
        a_src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        a_dst = torch.empty_like(a_src)
        a_dst.copy_(a_src)
        e0, e1 = ev.create(), ev.create()
        hip_rec = ev.hip.hipEventRecord
        hip_rec.argtypes = [C.c_void_p, C.c_void_p]
        cur = torch.cuda.current_stream().cuda_stream
        hip_rec(C.c_void_p(e0), C.c_void_p(cur))
        for _ in range(5):
            a_dst.copy_(a_src)
        hip_rec(C.c_void_p(e1), C.c_void_p(cur))
        copy_ms = ev.elapsed_ms(e0, e1) / 5
        ev.destroy(e0)
        ev.destroy(e1)
        del a_src, a_dst
        roof["attainable_copy_gbs"] = round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1)
        if roof["unit"] == "GB/s":
            roof["frac_of_attainable_copy"] = round(kern_gbs / roof["attainable_copy_gbs"], 4)
        # the attainable bf16 MFMA rate: a plain 8192^3 bf16 GEMM from the
        # vendor BLAS (contiguous 2-D operands), beside the 2.5 PFLOP/s peak
        g_n = 8192
        g_a = torch.randn(g_n, g_n, device="cuda").to(torch.bfloat16)
        g_b = torch.randn(g_n, g_n, device="cuda").to(torch.bfloat16).contiguous()
        g_c = torch.matmul(g_a, g_b)
        for _ in range(3):
            torch.matmul(g_a, g_b, out=g_c)
        e0, e1 = ev.create(), ev.create()
        hip_rec(C.c_void_p(e0), C.c_void_p(cur))
        for _ in range(10):
            torch.matmul(g_a, g_b, out=g_c)
        hip_rec(C.c_void_p(e1), C.c_void_p(cur))
        gemm_ms = ev.elapsed_ms(e0, e1) / 10
        ev.destroy(e0)
        ev.destroy(e1)
        del g_a, g_b, g_c
        roof["attainable_gemm_tflops"] = round(2 * g_n ** 3 / (gemm_ms * 1e-3) / 1e12, 1)
        roof["frac_of_attainable_gemm"] = round(kern_tf / roof["attainable_gemm_tflops"], 4)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = src.numel()
    if hasattr(b, "check"):
        b.check()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = b.cpu_baseline(args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
