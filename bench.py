"""Benchmark of the paged-KV attention step on one MI355X.

One step = one pass of the whole path over one batch. Prefill: device-side metadata (slots, prefix sums) and
store_kvcache of the new tokens in one launch (two with --separate-store), then attention over the paged cache in
one pass. Decode: pa_decode_append, whose balanced pass computes each new token's slot from the block table,
stores its K/V rows and attends over the cache, then merges cut sequences (two launches); with --no-append, the
metadata + store launch and pa_decode as for prefill.

Main line: the decode workload with Qwen3-0.6B attention shape (64 sequences, 16 query / 8 KV heads, head_dim
128, bf16, block_size 256, contexts U[128, 4096]). Consecutive steps use different per-layer cache pools (the
same block tables, as in an engine whose pool is [2, num_layers, num_blocks, block_size, Hkv, D]), so the KV a
step reads was not touched by the previous few steps and cannot sit in the 256 MB last-level cache.

Printed: one JSON line with the whole-step throughput (`value`, GB/s of algorithmic bytes over the wall time of
K uninstrumented steps), the roofline of the decode attention call (its duration from HIP events recorded on
the launch stream in a second pass of K steps), the oracle's CPU throughput on a bounded sample, and secondary
entries for the prefill workloads (varlen, a 2048-row chunk and a 256-row chunk over a long prefix) and the
long-context decode workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "decode paged-attn KV GB/s (% HBM peak); prefill attn TFLOP/s (% MFMA peak)"


# ---------------------------------------------------------------------------------------------- workload sizes


def algorithmic_work(wl, step, out_bytes: int):
    """Bytes (decode, store, metadata) and flops (prefill) the method must move or compute for one step.

    Decode: each needed KV row once (2 * Hkv * D * elem bytes per token), Q, O, the used block-table entries and
    the context lengths; shared prefix blocks of one call are counted once. Store: the new K/V rows read and
    written plus slot_mapping. Prefill flops: 4 * D * Hq per unmasked (query, key) pair.
    """
    E = wl.elem_bytes
    kv_tok = 2 * wl.num_kv_heads * wl.head_dim * E
    B = step.batch
    k_len = (step.num_cached + step.num_new).astype(np.int64)
    q_len = step.num_new.astype(np.int64)
    T = int(q_len.sum())
    shared = wl.notes.get("shared", [])
    shared_tokens = sum(n * wl.block_size for _, _, n in shared)
    n_tbl = int(sum(-(-int(n) // wl.block_size) for n in k_len))
    kv_bytes = (int(k_len.sum()) - shared_tokens) * kv_tok
    q_bytes = T * wl.num_heads * wl.head_dim * E
    o_bytes = T * wl.num_heads * wl.head_dim * out_bytes
    attn_bytes = kv_bytes + q_bytes + o_bytes + 4 * n_tbl + 4 * B
    store_bytes = 2 * T * kv_tok + 4 * T
    append_bytes = 2 * T * kv_tok
    meta_bytes = 4 * (3 * B + n_tbl) + 4 * (3 * B + 2 + 2 * T)
    past = k_len - q_len
    pairs = int(np.sum(q_len * past + q_len * (q_len + 1) // 2))
    flops = 4 * wl.head_dim * wl.num_heads * pairs
    return {"kv_bytes": kv_bytes, "attn_bytes": attn_bytes, "store_bytes": store_bytes, "meta_bytes": meta_bytes,
            "append_bytes": append_bytes,
            "pairs": pairs, "flops": flops, "sum_k": int(k_len.sum()), "tokens": T}


# ---------------------------------------------------------------------------------------------- GPU timing


# Sources of the attention kernels each workload kind runs, and the kernels of one attention call: a traffic
# summary taken on other sources is stale and not reported.
ATTN_SOURCES = {"decode": ("pa_decode_stream.hip", "pa_decode_tile.h", "pa_dpp.h", "pa_common.h", "pa_api.hip"),
                "prefill": ("pa_prefill.hip", "pa_prefill_tile.h", "pa_dpp.h", "pa_common.h", "pa_api.hip")}
ATTN_KERNELS = {"decode": ("decode_stream_kernel", "decode_stream_merge_kernel"),
                "prefill": ("prefill_mfma_kernel", "prefill_merge_kernel")}
ATTN_KERNELS_OPTIONAL = {"prefill_merge_kernel"}  # launched only by calls that split their keys


def _code_text(src: str) -> str:
    """A source file without its comments, trailing spaces and blank lines: what a counter summary is tied to
    (a change of wording in a comment does not make the measured kernels stale)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def _src_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_111_amd", "csrc", n), encoding="utf-8") as f:
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _traffic(profile_name: str, sha: str):
    """HBM bytes per launch from a committed counter summary, or None if absent or taken on other sources."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    with open(p, encoding="utf-8") as f:
        d = json.load(f)
    if d.get("source_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def write_traffic_summary(workload: str, fetch_csv: str, write_csv: str) -> dict:
    """profiles/<workload>_hbm_traffic.json from two rocprofv3 --pmc runs of this script with --calibrate-copy
    (one with FETCH_SIZE, one with WRITE_SIZE, counter values in KiB per dispatch). Each counter is scaled by
    known / measured on the plain copy kernel of the same run (torch.mul over 1 GiB of fp16: reads 1 GiB, writes
    1 GiB); HBM bytes per launch = sum over the attention call's kernels of the scaled means."""
    import collections
    import csv

    from workloads import make_config

    kind = make_config(workload, fill=False).steps[-1].kind

    def load(path):
        agg = collections.defaultdict(list)
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    fetch, write = load(fetch_csv), load(write_csv)

    def mean(agg, part):
        keys = [k for k in agg if part in k]
        if not keys:
            raise SystemExit(f"no dispatch of a kernel named like {part!r} in the counter file")
        vals = [v for k in keys for v in agg[k]]
        return sum(vals) / len(vals), len(vals)

    known_kib = (1 << 30) / 1024.0
    copy_f, _ = mean(fetch, COPY_KERNEL)
    copy_w, _ = mean(write, COPY_KERNEL)
    fscale, wscale = known_kib / copy_f, known_kib / copy_w
    per, total = {}, 0.0
    for kn in ATTN_KERNELS[kind]:
        if kn in ATTN_KERNELS_OPTIONAL and not any(kn in k for k in fetch):
            continue
        fk, n = mean(fetch, kn)
        wk, _ = mean(write, kn)
        b = (fk * fscale + wk * wscale) * 1024
        per[kn] = {"FETCH_SIZE_KiB": round(fk, 1), "WRITE_SIZE_KiB": round(wk, 1), "hbm_bytes": int(b),
                   "dispatches": n}
        total += b
    out = {
        "workload": workload,
        "what": "HBM bytes per launch of the attention call from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                "dispatch, mean over the profiled dispatches), each scaled by known / measured of the same counter "
                "on a plain copy kernel (torch.mul over 1 GiB of fp16: reads 1 GiB, writes 1 GiB)",
        "commands": [f"cd /tmp && rocprofv3 --pmc {c} -d gpurun_out/pmc_{c}_{workload} -o pmc --output-format csv "
                     f"-- python /root/repo/bench.py --only {workload} --no-cpu-baseline --steps 5 --warmup 2 "
                     f"--prewarm 0 --calibrate-copy" for c in ("FETCH_SIZE", "WRITE_SIZE")]
                    + [f"python bench.py --only {workload} --traffic-summary "
                       f"gpurun_out/pmc_FETCH_SIZE_{workload}/pmc_counter_collection.csv "
                       f"gpurun_out/pmc_WRITE_SIZE_{workload}/pmc_counter_collection.csv"],
        "copy_kernel": {"FETCH_SIZE_KiB": round(copy_f, 1), "WRITE_SIZE_KiB": round(copy_w, 1),
                        "known_read_KiB": known_kib, "known_write_KiB": known_kib,
                        "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)},
        "kernels": per,
        "hbm_bytes_per_launch": int(total),
        "source_files": list(ATTN_SOURCES[kind]),
        "source_sha": _src_sha(*ATTN_SOURCES[kind]),
    }
    with open(os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json"), "w", encoding="utf-8") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


SQ_PASSES = {
    "A": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES "
         "SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE",
    "B": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_LDS SQ_WAIT_INST_LDS "
         "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
}
N_SIMDS = 256 * 4


def write_sq_summary(workload: str, csv_a: str, csv_b: str) -> dict:
    """profiles/<workload>_sq_counters.json from two rocprofv3 --pmc runs of this script (the counter sets of
    SQ_PASSES, eight counters per run at most): the attention kernel's mean counters per dispatch and the
    fractions they give. GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the kernel's cycles are an eighth of it; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)."""
    import collections
    import csv

    from workloads import make_config

    kind = make_config(workload, fill=False).steps[-1].kind
    kern = ATTN_KERNELS[kind][0]
    vals = {}
    for path in (csv_a, csv_b):
        agg = collections.defaultdict(list)
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if kern in r["Kernel_Name"]:
                    agg[r["Counter_Name"]].append(float(r["Counter_Value"]))
        if not agg:
            raise SystemExit(f"no dispatch of {kern} in {path}")
        for k, v in agg.items():
            vals.setdefault(k, sum(v) / len(v))
    cycles = vals["GRBM_GUI_ACTIVE"] / 8
    frac = {
        "mfma_busy": vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMDS),
        "mfma_valu_coexec_per_mfma_busy": vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / vals["SQ_VALU_MFMA_BUSY_CYCLES"],
        "valu_insts_per_mfma": vals["SQ_INSTS_VALU"] / vals["SQ_INSTS_MFMA"],
        "trans_f32_per_mfma": vals["SQ_INSTS_VALU_TRANS_F32"] / vals["SQ_INSTS_MFMA"],
        "valu_active_per_wave_cycle": vals["SQ_ACTIVE_INST_VALU"] / vals["SQ_WAVE_CYCLES"],
        "lds_wait_per_wave_cycle": vals["SQ_WAIT_INST_LDS"] / vals["SQ_WAVE_CYCLES"],
        "any_wait_per_wave_cycle": vals["SQ_WAIT_INST_ANY"] / vals["SQ_WAVE_CYCLES"],
        "lds_bank_conflict_per_lds_active": vals["SQ_LDS_BANK_CONFLICT"] / max(1.0, vals["SQ_LDS_IDX_ACTIVE"]),
    }
    out = {
        "workload": workload,
        "kernel": kern,
        "what": "SQ counters of the attention kernel, mean per dispatch (totals over the GPU), and fractions: MFMA "
                "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)",
        "commands": [f"cd /tmp && rocprofv3 --pmc {SQ_PASSES[p]} -d gpurun_out/sq{p}_{workload} -o pmc "
                     f"--output-format csv -- python /root/repo/bench.py --only {workload} --no-cpu-baseline "
                     f"--steps 5 --warmup 2 --prewarm 0" for p in ("A", "B")]
                    + [f"python bench.py --only {workload} --sq-summary gpurun_out/sqA_{workload}/"
                       f"pmc_counter_collection.csv gpurun_out/sqB_{workload}/pmc_counter_collection.csv"],
        "counters": {k: round(v, 1) for k, v in sorted(vals.items())},
        "kernel_cycles": round(cycles, 1),
        "fractions": {k: round(v, 4) for k, v in frac.items()},
        "source_files": list(ATTN_SOURCES[kind]),
        "source_sha": _src_sha(*ATTN_SOURCES[kind]),
    }
    with open(os.path.join(ROOT, "profiles", f"{workload}_sq_counters.json"), "w", encoding="utf-8") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


class GpuWorkload:
    """A workload's inputs on the device, with n_layers independent cache pools holding the same contents."""

    def __init__(self, wl, n_layers: int, out_dtype, fused_store: bool = True, append: bool = True):
        import torch

        self.torch = torch
        self.wl = wl
        self.step = wl.steps[-1]
        self.fused_store = fused_store
        self.append = append and self.step.kind == "decode"
        dev = "cuda:0"

        def up(a):
            if wl.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

        k0, v0 = up(wl.k_cache), up(wl.v_cache)
        self.k_layers = [k0] + [k0.clone() for _ in range(n_layers - 1)]
        self.v_layers = [v0] + [v0.clone() for _ in range(n_layers - 1)]
        st = self.step
        self.block_table = i32(st.block_table)
        self.num_cached = i32(st.num_cached)
        self.num_new = i32(st.num_new)
        self.q, self.k, self.v = up(st.q), up(st.k), up(st.v)
        self.total_q = int(st.num_new.sum())
        self.max_q = int(st.num_new.max())
        self.max_k = int((st.num_cached + st.num_new).max())
        self.out = torch.empty((st.num_tokens, wl.num_heads, wl.head_dim), dtype=out_dtype, device=dev)
        import paged_kv_cache_111_amd as pa

        self.pa = pa
        if st.kind == "decode":
            need = pa.decode_workspace_bytes(st.batch, wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                             st.block_table.shape[1], wl.block_size, 0)
        else:
            need = pa.prefill_workspace_bytes(st.batch, wl.num_heads, wl.head_dim, self.max_q, self.max_k)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def run_attention(self, layer: int):
        """The attention call of the step alone (decode with append: the whole pa_decode_append call, whose store
        rewrites the same rows; prefill and decode: the attention over the cache the step's store filled)."""
        pa, wl, st = self.pa, self.wl, self.step
        kc, vc = self.k_layers[layer], self.v_layers[layer]
        if self.append:
            pa.decode_append(self.q, self.k, self.v, kc, vc, self.num_cached, self.block_table, wl.scale,
                             out=self.out, workspace=self.ws, fallback=False)
        elif st.kind == "decode":
            pa.decode(self.q, kc, vc, self.meta["context_lens"], self.block_table, wl.scale, out=self.out,
                      workspace=self.ws)
        else:
            pa.prefill_varlen(self.q, kc, vc, self.meta["cu_seqlens_q"], self.meta["cu_seqlens_k"],
                              self.block_table, self.max_q, self.max_k, wl.scale, out=self.out, workspace=self.ws)

    def run(self, layer: int, ev=None):
        """One step on layer `layer`'s pool; ev = (e0, e1, e2, e3) events around metadata, store, attention (with
        the fused launch, e0..e1 spans metadata and store, and e1..e2 is empty; with append, the decode call
        computes its slots and stores the new rows itself, and e0..e2 is empty)."""
        pa, wl, st = self.pa, self.wl, self.step
        kc, vc = self.k_layers[layer], self.v_layers[layer]
        if ev:
            ev[0].record()
        if self.append:
            if ev:
                ev[1].record()
                ev[2].record()
            pa.decode_append(self.q, self.k, self.v, kc, vc, self.num_cached, self.block_table, wl.scale,
                             out=self.out, workspace=self.ws, fallback=False)
            if ev:
                ev[3].record()
            return
        if self.fused_store:
            meta = pa.build_metadata_store(self.num_cached, self.num_new, self.block_table, self.total_q, self.k,
                                           self.v, kc, vc)
            if ev:
                ev[1].record()
        else:
            meta = pa.build_metadata(self.num_cached, self.num_new, self.block_table, self.total_q,
                                     wl.num_blocks, wl.block_size)
            if ev:
                ev[1].record()
            pa.store_kvcache(self.k, self.v, kc, vc, meta["slot_mapping"])
        if ev:
            ev[2].record()
        self.meta = meta
        if st.kind == "decode":
            pa.decode(self.q, kc, vc, meta["context_lens"], self.block_table, wl.scale, out=self.out,
                      workspace=self.ws)
        else:
            pa.prefill_varlen(self.q, kc, vc, meta["cu_seqlens_q"], meta["cu_seqlens_k"], self.block_table,
                              self.max_q, self.max_k, wl.scale, out=self.out, workspace=self.ws)
        if ev:
            ev[3].record()


PREWARM_S = 0.3  # seconds of the workload's own steps run before the warmup steps


def time_workload(g: GpuWorkload, steps: int, warmup: int, n_layers: int):
    """Two passes of `steps` steps after `warmup` untimed ones. The first carries no events: its wall time (between
    two synchronisations) gives the step time. The second records events around each launch on the launch stream
    and gives the per-kernel durations (recording an event costs a few microseconds of GPU time, so the
    instrumented pass is not used for the step time).

    Before the warmup steps the workload's steps run for PREWARM_S seconds: a GPU that was idle runs its first
    milliseconds of work at lower clocks (the first few prefill steps measured 10-15% slower), and ten steps of
    a 0.1 ms decode are far shorter than that."""
    torch = g.torch
    t_pre = time.perf_counter()
    i = 0
    while time.perf_counter() - t_pre < PREWARM_S:
        g.run(i % n_layers)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        g.run(i % n_layers)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        g.run(i % n_layers)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t1 = time.perf_counter()
    for i in range(steps):
        g.run(i % n_layers, evs[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    # third pass: the attention call alone, K calls back to back between one pair of events on the launch stream
    # (no event between launches): the kernel time the roofline uses
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_a.record()
    for i in range(steps):
        g.run_attention(i % n_layers)
    e_b.record()
    torch.cuda.synchronize()
    launch_ms = e_a.elapsed_time(e_b) / steps
    meta_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    store_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    attn_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    return {"wall_ms_per_step": 1e3 * wall / steps, "wall_ms_per_step_with_events": 1e3 * wall_ev / steps,
            "step_ms": float(np.mean(step_ms)), "meta_ms": float(np.mean(meta_ms)),
            "store_ms": float(np.mean(store_ms)), "attn_ms": float(np.mean(attn_ms)),
            "attn_ms_median": float(np.median(attn_ms)), "attn_ms_min": float(np.min(attn_ms)),
            "launch_ms": launch_ms}


# The batch sizes the engine captures its decode step for: 1, 2, 4, 8, then every multiple of 16 up to 512 (larger
# batches run eagerly), "一个 prompt 的一生" §2.2.4 and §3.3.2.
GRAPH_LADDER = [1, 2, 4, 8] + list(range(16, 513, 16))


def graph_ladder(batches, iters: int = 200):
    """Host launch overhead of a decode step (store_kvcache + decode, and pa_decode_append on the same data: the
    new rows at position length - 1) at the Qwen3-0.6B attention shape: wall
    time per step of eager calls through the binding against one replay of the same calls captured in a HIP
    graph, for a ladder of batch sizes (contexts U{128..4096}, block size 256, one pool, synthetic data). The
    engine captures its decode step per batch size for exactly this overhead ("一个 prompt 的一生：nano-vllm 从起服务到吐出
    token" §2.2.4)."""
    import torch

    import paged_kv_cache_111_amd as pa

    dev = "cuda:0"
    Hq, Hkv, D, bs, mbps = 16, 8, 128, 256, 16
    rows = []
    for B in batches:
        rng = np.random.default_rng(7000 + B)
        nb = B * mbps
        table = rng.permutation(nb).astype(np.int32).reshape(B, mbps)
        lens = rng.integers(128, mbps * bs + 1, size=B)
        pos = lens - 1
        slots = (table[np.arange(B), pos // bs].astype(np.int64) * bs + pos % bs).astype(np.int32)
        gen = torch.Generator(device=dev).manual_seed(B)
        kc = torch.randn((nb, bs, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        vc = torch.randn((nb, bs, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        q = torch.randn((B, Hq, D), device=dev, generator=gen).to(torch.bfloat16)
        k_new = torch.randn((B, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        v_new = torch.randn((B, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        ctx = torch.from_numpy(lens.astype(np.int32)).to(dev)
        sl = torch.from_numpy(slots).to(dev)
        bt = torch.from_numpy(table).to(dev)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, pa.decode_workspace_bytes(B, Hq, Hkv, D, mbps, bs, 0)), dtype=torch.uint8,
                         device=dev)
        scale = 1.0 / np.sqrt(D)

        cached = torch.from_numpy((lens - 1).astype(np.int32)).to(dev)

        def step():
            pa.store_kvcache(k_new, v_new, kc, vc, sl)
            pa.decode(q, kc, vc, ctx, bt, scale, out=out, workspace=ws)

        def step_append():
            pa.decode_append(q, k_new, v_new, kc, vc, cached, bt, scale, out=out, workspace=ws, fallback=False)

        def eager_and_graph(fn):
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(iters):
                fn()
            torch.cuda.synchronize()
            eager = (time.perf_counter() - t0) / iters
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for _ in range(10):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(iters):
                g.replay()
            torch.cuda.synchronize()
            graph = (time.perf_counter() - t0) / iters
            del g
            return eager, graph

        eager, graph = eager_and_graph(step)
        a_eager, a_graph = eager_and_graph(step_append)
        kv = float(lens.sum()) * 2 * Hkv * D * 2
        rows.append({"batch": B, "eager_us": round(eager * 1e6, 2), "graph_us": round(graph * 1e6, 2),
                     "kv_GBps_eager": round(kv / eager / 1e9, 1), "kv_GBps_graph": round(kv / graph / 1e9, 1),
                     "append_eager_us": round(a_eager * 1e6, 2), "append_graph_us": round(a_graph * 1e6, 2)})
        print(f"[bench] graph ladder {rows[-1]}", file=sys.stderr, flush=True)
        del kc, vc
        torch.cuda.empty_cache()
    return rows


def store_sweep(tokens=(64, 2048, 16384, 131072), iters: int = 50):
    """store_kvcache bandwidth at the Qwen3-0.6B cache shape (Hkv 8, D 128, bf16, block size 256) over token
    counts: decode-size stores are launch-bound, large ones HBM-bound. Bytes = 2·T·Hkv·D·2 read + the same
    written + 4T of slots; slots are a random permutation of a pool twice the size (no duplicates). Beside it,
    the fused q/k norm + rotary embedding + store step with 16 query heads."""
    import torch

    import paged_kv_cache_111_amd as pa

    dev = "cuda:0"
    Hkv, D, bs = 8, 128, 256
    rows = []
    for T in tokens:
        nb = max(8, (2 * T + bs - 1) // bs)
        rng = np.random.default_rng(5000 + T)
        slots = torch.from_numpy(rng.permutation(nb * bs)[:T].astype(np.int32)).to(dev)
        gen = torch.Generator(device=dev).manual_seed(T)
        k = torch.randn((T, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        v = torch.randn((T, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        kc = torch.zeros((nb, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        for _ in range(5):
            pa.store_kvcache(k, v, kc, vc, slots)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            pa.store_kvcache(k, v, kc, vc, slots)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        nbytes = 2 * (2 * T * Hkv * D * 2) + 4 * T
        # the fused pre-attention step at the same shape with Q (16 query heads): reads q, k, v, a table row and
        # the position of each token, writes the rotated q, K and V
        Hq = 16
        q = torch.randn((T, Hq, D), device=dev, generator=gen).to(torch.bfloat16)
        q_out = torch.empty_like(q)
        kw = torch.ones(D, dtype=torch.bfloat16, device=dev)
        pos = torch.from_numpy(rng.integers(0, 4096, size=T).astype(np.int32)).to(dev)
        ang = torch.arange(4096, device=dev, dtype=torch.float64)[:, None] * \
            (1e6 ** (-torch.arange(0, D, 2, device=dev, dtype=torch.float64) / D))[None, :]
        cs = torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).float().contiguous()

        def fused():
            pa.norm_rope_store_kvcache(k, v, kc, vc, slots, kw, pos, cs, 1e-6, q=q, q_norm_weight=kw, q_out=q_out)

        for _ in range(5):
            fused()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fused()
        e1.record()
        torch.cuda.synchronize()
        us_f = e0.elapsed_time(e1) * 1e3 / iters
        fbytes = 2 * T * (2 * Hkv + Hq) * D * 2 + T * D * 4 + 8 * T
        rows.append({"tokens": T, "us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                     "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                     "norm_rope_store_us": round(us_f, 2), "norm_rope_store_GBps": round(fbytes / us_f / 1e3, 1)})
        print(f"[bench] store sweep {rows[-1]}", file=sys.stderr, flush=True)
        del kc, vc, k, v, q, q_out
        torch.cuda.empty_cache()
    return rows


STORE_PROFILE_TOKENS = 131072  # the large store of the store profile (0.6B cache shape: 2 KiB K + 2 KiB V per token)


def store_profile(iters: int = 20):
    """The store kernels alone, for the store counters: pa_store_kvcache of STORE_PROFILE_TOKENS tokens at the
    Qwen3-0.6B cache shape (random distinct slots of a pool twice that size), then the varlen prefill workload's
    metadata + store launch (pa_build_metadata_store) and its separate store (pa_store_kvcache), each `iters`
    calls after 3 untimed ones. Returns per call: mean time between events around the calls and the algorithmic
    bytes (K and V rows read and written, slots, and for the fused launch the metadata arrays)."""
    import torch

    import paged_kv_cache_111_amd as pa
    from workloads import make_config

    dev = "cuda:0"
    res = {}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    Hkv, D, bs, T = 8, 128, 256, STORE_PROFILE_TOKENS
    nb = 2 * T // bs
    rng = np.random.default_rng(5000 + T)
    slots = torch.from_numpy(rng.permutation(nb * bs)[:T].astype(np.int32)).to(dev)
    gen = torch.Generator(device=dev).manual_seed(T)
    k = torch.randn((T, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
    kc = torch.zeros((nb, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    us = timed(lambda: pa.store_kvcache(k, v, kc, vc, slots))
    nbytes = 2 * (2 * T * Hkv * D * 2) + 4 * T
    res["store_kvcache_131072"] = {"kernel": "store_kvcache_kernel", "us": round(us, 2), "bytes": nbytes,
                                   "GBps": round(nbytes / us / 1e3, 1)}
    del k, v, kc, vc, slots
    torch.cuda.empty_cache()

    wl = make_config("prefill_qwen3_8b")
    g = GpuWorkload(wl, 1, torch.float32)
    st = g.step
    kc, vc = g.k_layers[0], g.v_layers[0]
    work = algorithmic_work(wl, st, 4)
    us = timed(lambda: pa.build_metadata_store(g.num_cached, g.num_new, g.block_table, g.total_q, g.k, g.v, kc, vc))
    nbytes = work["store_bytes"] + work["meta_bytes"]
    res["metadata_store_prefill_qwen3_8b"] = {"kernel": "metadata_store_kernel", "us": round(us, 2),
                                              "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                                              "tokens": work["tokens"]}
    meta = pa.build_metadata(g.num_cached, g.num_new, g.block_table, g.total_q, wl.num_blocks, wl.block_size)
    us = timed(lambda: pa.store_kvcache(g.k, g.v, kc, vc, meta["slot_mapping"]))
    nbytes = work["store_bytes"]
    res["store_kvcache_prefill_qwen3_8b"] = {"kernel": "store_kvcache_kernel", "us": round(us, 2), "bytes": nbytes,
                                             "GBps": round(nbytes / us / 1e3, 1), "tokens": work["tokens"]}
    return res


STORE_KERNELS = ("store_kvcache_kernel", "metadata_store_kernel")
COPY_KERNEL = "MulFunctor"  # torch.mul over 1 GiB of fp16: the plain copy the byte counters are scaled by
STORE_SOURCES = ("pa_meta_store.hip", "pa_dpp.h", "pa_common.h", "pa_api.hip")


def _kernel_calls(path: str, names):
    """Per dispatch, in order, the counter value of each kernel whose name contains one of `names`."""
    import collections
    import csv

    out = collections.defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            for n in names:
                if n in r["Kernel_Name"]:
                    out[n].append(float(r["Counter_Value"]))
    return out


def write_store_traffic_summary(fetch_csv: str, write_csv: str, trace_csv: str) -> dict:
    """profiles/store_hbm_traffic.json from three rocprofv3 runs of `bench.py --store-profile`: FETCH_SIZE and
    WRITE_SIZE (--pmc, with --calibrate-copy) and a kernel trace. For each store launch: the mean kernel duration (trace),
    its algorithmic bytes (K/V rows read and written, slots, and the metadata arrays of the fused launch) over that
    duration, and HBM bytes per launch (counters scaled by the 1 GiB copy's known / measured, as for the attention
    kernels). The profile runs, in order: 3 + 20 store_kvcache calls of STORE_PROFILE_TOKENS tokens at the 0.6B
    cache shape, 3 + 20 metadata + store launches of the varlen prefill step, 3 + 20 stores of that step's tokens;
    the 3 untimed calls of each group are left out of the means."""
    import csv

    from workloads import make_config

    names = (COPY_KERNEL,) + STORE_KERNELS
    fetch, write = _kernel_calls(fetch_csv, names), _kernel_calls(write_csv, names)
    known_kib = (1 << 30) / 1024.0
    fscale = known_kib / (sum(fetch[COPY_KERNEL]) / len(fetch[COPY_KERNEL]))
    wscale = known_kib / (sum(write[COPY_KERNEL]) / len(write[COPY_KERNEL]))
    dur = {n: [] for n in STORE_KERNELS}
    with open(trace_csv, newline="") as f:
        for r in sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"])):
            for n in STORE_KERNELS:
                if n in r["Kernel_Name"]:
                    dur[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)  # ns -> us

    def split(v):  # [large store x 23, prefill-step store x 23] for store_kvcache_kernel
        h = len(v) // 2
        return v[:h], v[h:]

    wl = make_config("prefill_qwen3_8b", fill=False)
    work = algorithmic_work(wl, wl.steps[-1], 4)
    T, row = STORE_PROFILE_TOKENS, 8 * 128 * 2
    algo = {"store_kvcache_131072": 2 * (2 * T * row) + 4 * T,
            "store_kvcache_prefill_qwen3_8b": work["store_bytes"],
            "metadata_store_prefill_qwen3_8b": work["store_bytes"] + work["meta_bytes"]}
    sk_f, sk_w, sk_d = split(fetch["store_kvcache_kernel"]), split(write["store_kvcache_kernel"]), \
        split(dur["store_kvcache_kernel"])
    groups = {"store_kvcache_131072": ("store_kvcache_kernel", sk_f[0], sk_w[0], sk_d[0]),
              "store_kvcache_prefill_qwen3_8b": ("store_kvcache_kernel", sk_f[1], sk_w[1], sk_d[1]),
              "metadata_store_prefill_qwen3_8b": ("metadata_store_kernel", fetch["metadata_store_kernel"],
                                                  write["metadata_store_kernel"], dur["metadata_store_kernel"])}
    launches = {}
    for key, (kern, fv, wv, dv) in groups.items():
        fk, wk = sum(fv[3:]) / len(fv[3:]), sum(wv[3:]) / len(wv[3:])
        us = sum(dv[3:]) / len(dv[3:])
        hbm = (fk * fscale + wk * wscale) * 1024
        launches[key] = {"kernel": kern, "kernel_us": round(us, 2), "algorithmic_bytes": algo[key],
                         "GBps": round(algo[key] / us / 1e3, 1),
                         "frac_hbm_peak": round(algo[key] / us / 1e3 / HBM_PEAK_GBS, 4),
                         "FETCH_SIZE_KiB": round(fk, 1), "WRITE_SIZE_KiB": round(wk, 1), "hbm_bytes": int(hbm),
                         "hbm_over_algorithmic": round(hbm / algo[key], 3), "dispatches": len(dv) - 3}
    out = {
        "what": "store launches: algorithmic bytes (K/V rows read and written, slots, metadata arrays) over the mean "
                "kernel duration from the kernel trace, and HBM bytes per launch from rocprofv3 FETCH_SIZE and "
                "WRITE_SIZE scaled by a plain 1 GiB copy's known / measured",
        "commands": [f"cd /tmp && rocprofv3 --pmc {c} -d gpurun_out/pmc_{c}_store -o pmc --output-format csv -- "
                     f"python /root/repo/bench.py --store-profile --calibrate-copy" for c in ("FETCH_SIZE",
                                                                                             "WRITE_SIZE")]
                    + ["cd /tmp && rocprofv3 --kernel-trace --stats -d gpurun_out/kt_store -o kt --output-format csv "
                       "-- python /root/repo/bench.py --store-profile",
                       "python bench.py --store-traffic-summary gpurun_out/pmc_FETCH_SIZE_store/"
                       "pmc_counter_collection.csv gpurun_out/pmc_WRITE_SIZE_store/pmc_counter_collection.csv "
                       "gpurun_out/kt_store/kt_kernel_trace.csv"],
        "copy_kernel": {"FETCH_SIZE_KiB": round(sum(fetch[COPY_KERNEL]) / len(fetch[COPY_KERNEL]), 1),
                        "WRITE_SIZE_KiB": round(sum(write[COPY_KERNEL]) / len(write[COPY_KERNEL]), 1),
                        "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)},
        "launches": launches,
        "source_files": list(STORE_SOURCES),
        "source_sha": _src_sha(*STORE_SOURCES),
    }
    with open(os.path.join(ROOT, "profiles", "store_hbm_traffic.json"), "w", encoding="utf-8") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def write_kernel_stats_summary(name: str, stats_csv: str, command: str) -> str:
    """profiles/<name>_kernel_stats.txt from a rocprofv3 --kernel-trace --stats kernel_stats.csv: calls, mean,
    min and max duration and share per kernel, with the command that made the file."""
    import csv

    rows = list(csv.DictReader(open(stats_csv, newline="")))
    lines = ["# rocprofv3 kernel statistics", f"# command: {command}", "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share_%':>8s}"]
    for r in rows:
        n = re.sub(r"\(.*", "", r["Name"]).replace("void ", "")
        lines.append(f"{n[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"{name}_kernel_stats.txt"), "w", encoding="utf-8") as f:
        f.write(text)
    return text


def sample_sweep(batches=(1, 64, 256), vocab: int = 151936, iters: int = 50):
    """pa_sample at the Qwen3 vocabulary: time per call (events over back-to-back calls) and the rate at which
    it consumes logits (B·V·4 bytes; the uniforms are generated in the kernel, not read)."""
    import torch

    import paged_kv_cache_111_amd as pa

    dev = "cuda:0"
    rows = []
    for B in batches:
        gen = torch.Generator(device=dev).manual_seed(B)
        logits = 3.0 * torch.randn((B, vocab), device=dev, generator=gen)
        temps = torch.full((B,), 0.8, device=dev)
        toks = torch.empty(B, dtype=torch.int32, device=dev)
        ws = torch.empty(max(8, pa.sample_workspace_bytes(B, vocab)), dtype=torch.uint8, device=dev)
        for i in range(5):
            pa.sample(logits, temps, 1, i, tokens=toks, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            pa.sample(logits, temps, 1, i, tokens=toks, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        rows.append({"batch": B, "vocab": vocab, "us": round(us, 2),
                     "logits_GBps": round(B * vocab * 4 / us / 1e3, 1),
                     "Gsamples_per_s": round(B * vocab / us / 1e3, 1)})
        print(f"[bench] sample sweep {rows[-1]}", file=sys.stderr, flush=True)
    return rows


# ---------------------------------------------------------------------------------------------- CPU baseline


def cpu_baseline(wl, budget_s: float):
    """The oracle (as it stands) on the host: metadata, store and attention of the same step.

    Work units are whole sequences for decode and chunks of CPU_ROWS query rows of a sequence for prefill (a
    single long chunk, like the 2048 rows over 32768 keys, would otherwise take tens of seconds). Units are
    visited in the step's order, over repeated passes, until the time budget is spent; the rate counts the keys
    (decode) or unmasked (query, key) pairs (prefill) of the units computed. The oracle's store writes the same
    rows on every pass, so it runs in place on the workload's host pools.
    """
    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = 1
    st = wl.steps[-1]
    k_len = st.num_cached + st.num_new
    units = []  # (sequence, rows or None)
    for s in range(st.batch):
        ql = int(st.num_new[s])
        if st.kind == "decode" or ql <= CPU_ROWS:
            units.append((s, None))
        else:
            units.extend((s, np.arange(r0, min(ql, r0 + CPU_ROWS))) for r0 in range(0, ql, CPU_ROWS))
    secs, keys, pairs, units_done, passes = 0.0, 0, 0, 0, 0
    while secs < budget_s:
        t0 = time.perf_counter()
        meta = oracle.build_metadata(st.block_table, st.num_cached, st.num_new, wl.block_size)
        oracle.store_kvcache(wl.k_cache, wl.v_cache, st.k, st.v, meta["slot_mapping"])
        secs += time.perf_counter() - t0
        for s, rows in units:
            t1 = time.perf_counter()
            if st.kind == "decode":
                oracle.decode(st.q, wl.k_cache, wl.v_cache, meta["context_lens"], st.block_table, wl.scale,
                              wl.dtype, seqs=[s])
            else:
                oracle.prefill_varlen(st.q, wl.k_cache, wl.v_cache, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                      st.block_table, wl.scale, wl.dtype, seqs=[s],
                                      rows=None if rows is None else {s: rows})
            secs += time.perf_counter() - t1
            units_done += 1
            keys += int(k_len[s])
            ql = int(st.num_new[s])
            past = int(k_len[s]) - ql
            r = np.arange(ql) if rows is None else rows
            pairs += int(np.sum(past + r + 1))
            if secs > budget_s:
                break
        passes += 1
    kv_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    if st.kind == "decode":
        value, unit = keys * kv_tok / secs / 1e9, "GB/s"
        what = f"{units_done} sequence decodes ({keys} keys)"
    else:
        value, unit = 4 * wl.head_dim * wl.num_heads * pairs / secs / 1e12, "TFLOP/s"
        what = f"{units_done} units of up to {CPU_ROWS} query rows of a sequence ({pairs} query-key pairs)"
    return {"value": round(value, 6), "unit": unit, "cores": int(blas), "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{passes} pass(es) of oracle metadata + store + float64 attention over the same step; "
                      f"{what} in {secs:.1f} s; cores = BLAS threads"}


CPU_ROWS = 128  # query rows per unit of the prefill CPU baseline


# ---------------------------------------------------------------------------------------------- main


def bench_one(name: str, steps: int, warmup: int, n_layers: int, out_dtype_name: str, fused_store: bool = True,
              append: bool = True):
    import torch

    from workloads import make_config

    wl = make_config(name)
    out_dtype = torch.bfloat16 if out_dtype_name == "bf16" else torch.float32
    g = GpuWorkload(wl, n_layers, out_dtype, fused_store, append)
    t = time_workload(g, steps, warmup, n_layers)
    work = algorithmic_work(wl, g.step, 2 if out_dtype == torch.bfloat16 else 4)
    res = {"workload": name, "kind": g.step.kind, "timing": t, "work": work, "append": g.append}
    if g.step.kind == "decode":
        # with append the decode launch also moves the new rows (read and written); no slot or metadata arrays
        launch_bytes = work["attn_bytes"] + (work["append_bytes"] if g.append else 0)
        step_bytes = launch_bytes if g.append else work["attn_bytes"] + work["store_bytes"] + work["meta_bytes"]
        res["launch_bytes"] = launch_bytes
        res["attn_GBps"] = launch_bytes / (t["launch_ms"] * 1e-3) / 1e9
        res["attn_frac_hbm"] = res["attn_GBps"] / HBM_PEAK_GBS
        res["step_GBps"] = step_bytes / (t["wall_ms_per_step"] * 1e-3) / 1e9
    else:
        res["attn_TFLOPs"] = work["flops"] / (t["launch_ms"] * 1e-3) / 1e12
        res["attn_frac_mfma"] = res["attn_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        res["step_TFLOPs"] = work["flops"] / (t["wall_ms_per_step"] * 1e-3) / 1e12
    if not g.append and fused_store:
        res["meta_store_GBps"] = (work["store_bytes"] + work["meta_bytes"]) / (t["meta_ms"] * 1e-3) / 1e9
    elif not g.append:
        res["store_GBps"] = work["store_bytes"] / (t["store_ms"] * 1e-3) / 1e9
    del g
    torch.cuda.empty_cache()
    return wl, res


def roofline_of(name: str, r: dict) -> dict:
    """The roofline object of one workload's attention call: algorithmic bytes (decode) or flops (prefill) per
    launch over the launch time of the uninstrumented attention-only pass, against the MI355X peak; traffic = HBM
    bytes per launch from the committed counter summary of the same kernel sources (None if absent or stale)."""
    t = r["timing"]
    traffic = _traffic(f"{name}_hbm_traffic.json", _src_sha(*ATTN_SOURCES[r["kind"]]))
    if r["kind"] == "decode":
        return {"bound": "hbm", "achieved": round(r["attn_GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["attn_frac_hbm"], 4), "traffic": traffic,
                "kernel": ("pa_decode_append (" if r["append"] else "pa_decode (") +
                          " + ".join(ATTN_KERNELS["decode"]) + ")",
                "bytes_per_launch": r["launch_bytes"], "launch_ms": round(t["launch_ms"], 5)}
    return {"bound": "mfma", "achieved": round(r["attn_TFLOPs"], 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(r["attn_frac_mfma"], 4), "traffic": traffic,
            "kernel": "pa_prefill_varlen (" + " + ".join(ATTN_KERNELS["prefill"]) + ")",
            "flops_per_launch": r["work"]["flops"], "launch_ms": round(t["launch_ms"], 5)}


def _step_text(is_dec: bool, append: bool, fused: bool) -> str:
    if append:
        return "decode with the new K/V rows stored in its own pass (balanced pass + merge; slots from the tables)"
    return (("metadata and store_kvcache in one launch + " if fused else "metadata + store_kvcache + ") +
            ("decode (balanced pass + merge)" if is_dec else "prefill"))


def _store_rate(r) -> dict:
    if r["append"]:
        return {"store": "in the decode launch"}
    if "store_GBps" in r:
        return {"store_GBps": round(r["store_GBps"], 1)}
    return {"metadata_store_GBps": round(r["meta_store_GBps"], 1)}


def main() -> int:
    global PREWARM_S
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=8, help="cache pools cycled through by consecutive steps")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--only", default=None, help="run one workload only (no secondary entries)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--secondary-cpu-budget", type=float, default=5.0,
                    help="seconds of oracle work for each secondary workload's CPU baseline")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write the HBM traffic summary of --only's workload from two rocprofv3 counter files "
                         "(no GPU needed) and exit")
    ap.add_argument("--sq-summary", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"), default=None,
                    help="write the SQ counter summary of --only's workload from two rocprofv3 counter files "
                         "(no GPU needed) and exit")
    ap.add_argument("--store-profile", action="store_true",
                    help="only run the store launches of the store counter summary (large store, the varlen "
                         "prefill step's metadata + store and its separate store)")
    ap.add_argument("--store-traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "TRACE_CSV"),
                    default=None, help="write profiles/store_hbm_traffic.json (no GPU needed) and exit")
    ap.add_argument("--stats-summary", nargs=3, metavar=("NAME", "STATS_CSV", "COMMAND"), default=None,
                    help="write profiles/NAME_kernel_stats.txt from a rocprofv3 kernel_stats.csv (no GPU needed)")
    ap.add_argument("--store-sweep", action="store_true",
                    help="only time store_kvcache at the 0.6B cache shape for 64 .. 131072 tokens")
    ap.add_argument("--sample-sweep", action="store_true",
                    help="only time the sampler at the Qwen3 vocabulary for batch 1, 64, 256")
    ap.add_argument("--graph-ladder", action="store_true",
                    help="only time a decode step eager vs captured in a HIP graph over the batch sizes the engine "
                         "captures (1, 2, 4, 8, 16, 32, ..., 512)")
    ap.add_argument("--prewarm", type=float, default=PREWARM_S,
                    help="seconds of untimed steps before the warmup steps (0 for counter runs)")
    ap.add_argument("--separate-store", action="store_true",
                    help="metadata and store as two launches (pa_build_metadata, pa_store_kvcache) instead of one "
                         "(pa_build_metadata_store)")
    ap.add_argument("--no-append", action="store_true",
                    help="decode: metadata + store launch before pa_decode instead of pa_decode_append (which "
                         "stores the new rows inside the decode pass)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB copy kernel (reference for the HBM byte counters)")
    args = ap.parse_args()
    PREWARM_S = args.prewarm
    if args.traffic_summary:
        if not args.only:
            ap.error("--traffic-summary needs --only WORKLOAD")
        print(json.dumps(write_traffic_summary(args.only, *args.traffic_summary), indent=1))
        return 0
    if args.sq_summary:
        if not args.only:
            ap.error("--sq-summary needs --only WORKLOAD")
        print(json.dumps(write_sq_summary(args.only, *args.sq_summary), indent=1))
        return 0
    if args.store_traffic_summary:
        print(json.dumps(write_store_traffic_summary(*args.store_traffic_summary), indent=1))
        return 0
    if args.stats_summary:
        print(write_kernel_stats_summary(*args.stats_summary))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the attention step runs "
              "on one GPU's share and has no cross-GPU exchange)", file=sys.stderr)
        return 2
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.store_sweep:
        print(json.dumps({"store_sweep": store_sweep()}))
        return 0
    if args.store_profile:
        if args.calibrate_copy:
            x = torch.empty(1 << 29, dtype=torch.float16, device="cuda:0").normal_()
            y = torch.empty_like(x)
            for _ in range(3):
                torch.mul(x, 1.0, out=y)  # reads 1 GiB, writes 1 GiB
            torch.cuda.synchronize()
            del x, y
        print(json.dumps({"store_profile": store_profile()}))
        return 0
    if args.sample_sweep:
        print(json.dumps({"sample_sweep": sample_sweep()}))
        return 0
    if args.graph_ladder:
        print(json.dumps({"graph_ladder": graph_ladder(GRAPH_LADDER)}))
        return 0
    main_name = args.only or "decode_qwen3_0p6b"
    fused = not args.separate_store
    append = not args.no_append
    wl, main = bench_one(main_name, args.steps, args.warmup, args.layers, args.out_dtype, fused, append)
    print(f"[bench] {main_name}: {json.dumps(main['timing'])}", file=sys.stderr, flush=True)
    secondary = []
    if not args.only and not args.no_secondary:
        for name in ("prefill_qwen3_8b", "chunked_qwen3_8b", "chunk256_qwen3_8b", "decode_qwen3_32b"):
            layers = 1 if name == "decode_qwen3_32b" else args.layers
            swl, r = bench_one(name, max(10, args.steps // 2), max(2, args.warmup // 2), layers, args.out_dtype,
                               fused, append)
            print(f"[bench] {name}: {json.dumps(r['timing'])}", file=sys.stderr, flush=True)
            entry = {"workload": name, "attn_ms": round(r["timing"]["launch_ms"], 4),
                     "step_ms": round(r["timing"]["wall_ms_per_step"], 4)}
            entry.update(_store_rate(r))
            if r["kind"] == "decode":
                entry.update({"attn_GBps": round(r["attn_GBps"], 1), "frac_hbm": round(r["attn_frac_hbm"], 4),
                              "kv_bytes": r["work"]["kv_bytes"]})
            else:
                entry.update({"attn_TFLOPs": round(r["attn_TFLOPs"], 1),
                              "frac_mfma": round(r["attn_frac_mfma"], 4), "flops": r["work"]["flops"]})
            entry["roofline"] = roofline_of(name, r)
            if not args.no_cpu_baseline:
                entry["cpu_baseline"] = cpu_baseline(swl, args.secondary_cpu_budget)
            del swl
            secondary.append(entry)
    if args.calibrate_copy:
        x = torch.empty(1 << 29, dtype=torch.float16, device="cuda:0").normal_()
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del x, y

    t = main["timing"]
    work = main["work"]
    is_dec = main["kind"] == "decode"
    roof = roofline_of(main_name, main)
    if is_dec:
        value = main["step_GBps"]
        unit = "GB/s"
    else:
        value = work["flops"] / (t["wall_ms_per_step"] * 1e-3) / 1e12
        unit = "TFLOP/s"
    st = wl.steps[-1]
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "prewarm_s": PREWARM_S, "ms_per_step": round(t["wall_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": main_name, "batch": st.batch, "num_heads": wl.num_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "sum_context": work["sum_k"], "new_tokens": work["tokens"], "seed": wl.seed,
                   "out_dtype": args.out_dtype, "layers_cycled": args.layers,
                   "step": _step_text(is_dec, main["append"], fused)},
        "breakdown_ms": ({} if main["append"] else {"metadata_store": round(t["meta_ms"], 5)} if fused else
                         {"metadata": round(t["meta_ms"], 5), "store": round(t["store_ms"], 5)}) |
                        {"attention_alone": round(t["launch_ms"], 5),
                         "attention_with_events": round(t["attn_ms"], 5),
                         "attention_with_events_median": round(t["attn_ms_median"], 5),
                         "events_step": round(t["step_ms"], 5),
                         "wall_step_with_events": round(t["wall_ms_per_step_with_events"], 5)},
        **_store_rate(main),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    if secondary:
        line["secondary"] = secondary
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
