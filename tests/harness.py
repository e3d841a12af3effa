"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP path through the C ABI, compare with
the oracle. Nothing here computes the method: the HIP side is paged_kv_cache_111_amd, the reference is oracle/.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_cache_111_amd as pa

# Attention tolerance against the float64 oracle, over the whole output tensor of one call (bf16 inputs,
# float32 accumulation and output).
MAX_ABS = 2e-2
REL_RMS = 5e-3

DEV = "cuda:0"


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw stored values on the host: uint16 bf16 bits or float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class DevStep:
    """One step's inputs on the device."""

    def __init__(self, step, dtype: str):
        self.step = step
        self.block_table = i32(step.block_table)
        self.num_cached = i32(step.num_cached)
        self.num_new = i32(step.num_new)
        self.q = to_dev(step.q, dtype)
        self.k = to_dev(step.k, dtype)
        self.v = to_dev(step.v, dtype)
        self.total_q = int(step.num_new.sum())
        self.max_q = int(step.num_new.max()) if step.batch else 0
        self.max_k = int((step.num_cached + step.num_new).max()) if step.batch else 0


def hip_step(wl, ds: DevStep, kc: torch.Tensor, vc: torch.Tensor, out_dtype=torch.float32, split_tokens=0,
             fused_store=False, append=False):
    """The whole path on the GPU: metadata, store, attention (metadata and store in one launch with fused_store;
    with append, a decode step stores and attends in pa_decode_append and the metadata call only computes the
    arrays compared with the oracle's). Returns (metadata tensors, output tensor)."""
    if append and ds.step.kind == "decode":
        meta = pa.build_metadata(ds.num_cached, ds.num_new, ds.block_table, ds.total_q, wl.num_blocks,
                                 wl.block_size)
        out = pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale,
                               out_dtype=out_dtype, fallback=False)
        return meta, out
    if fused_store:
        meta = pa.build_metadata_store(ds.num_cached, ds.num_new, ds.block_table, ds.total_q, ds.k, ds.v, kc, vc)
    else:
        meta = pa.build_metadata(ds.num_cached, ds.num_new, ds.block_table, ds.total_q, wl.num_blocks,
                                 wl.block_size)
        pa.store_kvcache(ds.k, ds.v, kc, vc, meta["slot_mapping"])
    if ds.step.kind == "prefill":
        out = pa.prefill_varlen(ds.q, kc, vc, meta["cu_seqlens_q"], meta["cu_seqlens_k"], ds.block_table, ds.max_q,
                                ds.max_k, wl.scale, out_dtype=out_dtype)
    else:
        out = pa.decode(ds.q, kc, vc, meta["context_lens"], ds.block_table, wl.scale, out_dtype=out_dtype,
                        split_tokens=split_tokens)
    return meta, out


def compare_metadata(meta_dev: dict, meta_ref: dict) -> None:
    for key in ("cu_seqlens_q", "cu_seqlens_k", "context_lens", "positions", "slot_mapping"):
        got = meta_dev[key].cpu().numpy()
        assert np.array_equal(got, meta_ref[key]), f"{key} differs"


def attention_errors(out: torch.Tensor, ref: np.ndarray, rows=None):
    """(max_abs, rel_rms) over the rows the oracle computed (all rows by default)."""
    got = out.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(ref))
    assert np.all(np.isfinite(got)), "non-finite output"
    err = got - ref
    max_abs = float(np.max(np.abs(err)))
    rel_rms = float(np.sqrt(np.sum(err * err) / np.sum(ref * ref)))
    return max_abs, rel_rms


def bf16_half_ulp(got: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp in the binade of |got| (elementwise): an upper bound on |got - x| for any float x whose
    round-to-nearest-even to bf16 is got. bf16 has an 8-bit significand, so the half ulp of [2^e, 2^(e+1)) is
    2^(e-8); a value rounded up across a power of two lies in the binade below, whose half ulp is smaller."""
    a = np.maximum(np.abs(got), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 8)


def assert_close(out: torch.Tensor, ref: np.ndarray, rows=None, what: str = "") -> tuple:
    """Attention tolerance against the float64 oracle. A float32 output must meet MAX_ABS and REL_RMS. A bf16
    output is the float32 result x the kernel computed, rounded to nearest even: |got - x| <= h = half a bf16 ulp
    of got (bf16_half_ulp), so x meeting the tolerance implies, elementwise, |got - ref| <= MAX_ABS + h, and over
    the tensor ||got - ref|| <= REL_RMS ||ref|| + ||h|| (triangle inequality). Those two bounds are what a bf16
    output is graded with here; the parity runs also check the bf16 output bit for bit against the rounding of
    the float32 output of the same call (assert_bf16_is_rounded_f32)."""
    max_abs, rel_rms = attention_errors(out, ref, rows)
    if out.dtype == torch.bfloat16:
        got = out.detach().float().cpu().numpy().astype(np.float64)
        r = ref if rows is None else ref[rows]
        g = got if rows is None else got[rows]
        h = bf16_half_ulp(g)
        assert np.all(np.abs(g - r) <= MAX_ABS + h), f"{what}: bf16 output off by more than tol + half an ulp"
        rms_bound = REL_RMS + float(np.sqrt(np.sum(h * h) / np.sum(r * r)))
        assert rel_rms <= rms_bound, f"{what}: rel_rms {rel_rms:.3g} > {rms_bound:.3g}"
    else:
        assert max_abs <= MAX_ABS, f"{what}: max_abs {max_abs:.3g} > {MAX_ABS}"
        assert rel_rms <= REL_RMS, f"{what}: rel_rms {rel_rms:.3g} > {REL_RMS}"
    return max_abs, rel_rms


def assert_bf16_is_rounded_f32(out_bf16: torch.Tensor, out_f32: torch.Tensor, what: str = "") -> None:
    """The bf16 output of a call equals, bit for bit, the round-to-nearest-even of the float32 output of the same
    call on the same inputs (torch's CPU conversion rounds to nearest even)."""
    want = out_f32.detach().cpu().to(torch.bfloat16)
    assert torch.equal(out_bf16.detach().cpu().view(torch.int16), want.view(torch.int16)), \
        f"{what}: bf16 output is not the rounded float32 output"


def oracle_step(wl, step, kc_host: np.ndarray, vc_host: np.ndarray, seqs=None, rows=None):
    """Oracle metadata, store (in place on the host pools) and attention for one step."""
    return oracle.run_step(step, kc_host, vc_host, wl.block_size, wl.scale, wl.dtype, seqs=seqs, rows=rows)


def flat_rows(meta_ref: dict, seqs, rows_by_seq=None):
    """Flattened output rows covered by the given sequences (and row subsets)."""
    cu = meta_ref["cu_seqlens_q"]
    out = []
    for s in seqs:
        if rows_by_seq is not None and s in rows_by_seq:
            out.extend(int(cu[s]) + np.asarray(rows_by_seq[s]))
        else:
            out.extend(range(int(cu[s]), int(cu[s + 1])))
    return np.asarray(out, dtype=np.int64)
