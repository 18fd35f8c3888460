"""The kernels read no workspace they have not written in the same call.

Every workspace the binding allocates is filled with 0xFF bytes first (NaN as bf16, fp16 and
fp32, -1 as int32), and the results must be bitwise those of a run on a fresh workspace.  A
kernel that read a part of the workspace no earlier kernel of the call wrote (the visibility
bounds, delta, the sink partials, the 16-bit or fp32 dU blocks, the head-split dK/dV partials,
the full or head-summed dbias of a broadcast bias) would turn NaN or a wrong bound into its
results.
"""
import numpy as np
import pytest
import torch

import attention_tanh_logit_amd.ops as ops
import harness
from harness import TOL, as_dense_mask, as_k_start, case, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

CASES = {
    "du_blocks_segments": dict(dtype="bf16", D=128, B=2, S=200, Hq=4, Hkv=2, segments=[[45, 70, 190], [128]],
                               sink_mode="learnable"),
    "head_split_d64": dict(dtype="bf16", D=64, B=1, S=203, Hq=8, Hkv=2, sink_mode="learnable"),
    "bias_heads_partials": dict(dtype="bf16", D=128, B=2, S=200, Hq=4, Hkv=2, bias=True, bias_bcast="heads",
                                softcap=50.0),
    "bias_batch_fp32": dict(dtype="fp32", D=128, B=2, S=131, Hq=4, Hkv=2, bias=True, bias_bcast="batch"),
    "du_blocks_fp32": dict(dtype="fp32", D=256, B=2, S=200, Hq=4, Hkv=2, segments=[[45, 70, 190], [128]],
                           sink_mode="learnable", window=50),
    "du_blocks_fp32_d64_dropout": dict(dtype="fp32", D=64, B=2, S=203, Hq=4, Hkv=2, dropout_p=0.2),
    "dense_mask": dict(dtype="bf16", D=128, B=2, S=200, Hq=4, Hkv=2, segments=[[45, 70, 190], [128]]),
    "k_start": dict(dtype="bf16", D=256, B=2, S=200, Hq=4, Hkv=2, segments=[[45, 70, 190], [128]]),
    "dropout": dict(dtype="bf16", D=128, B=2, S=203, Hq=4, Hkv=2, dropout_p=0.2, sink_mode="learnable"),
    "wide_d512": dict(dtype="bf16", D=512, B=1, S=150, Hq=2, Hkv=1, sink_mode="learnable"),
    "wide_d512_bias": dict(dtype="bf16", D=512, B=2, S=200, Hq=4, Hkv=2, bias=True, softcap=50.0,
                           segments=[[45, 70, 190], [128]]),
}


def _poisoned(nbytes, device):
    if nbytes == 0:
        return None
    return torch.full((nbytes,), 255, dtype=torch.uint8, device=device)


@pytest.mark.parametrize("name", list(CASES))
def test_results_do_not_depend_on_the_workspace_contents(name, monkeypatch):
    c = case(**CASES[name])
    if name == "dense_mask":
        c = as_dense_mask(c)
    elif name == "k_start":
        c = as_k_start(c)
    print(f"workspace poisoning: {name}", flush=True)
    clean = run_gpu(c)
    monkeypatch.setattr(ops, "_workspace", _poisoned)
    dirty = run_gpu(c)
    for n, x in clean.items():
        if x is None:
            assert dirty[n] is None, n
            continue
        assert not np.isnan(x).any(), f"{name}: {n} has NaN on a fresh workspace"
        assert x.tobytes() == dirty[n].tobytes(), f"{name}: {n} depends on the workspace contents"


# Sq > Sk + window - 1 without a causal mask: the last queries see no key, whole 32-query waves
# of them, and Sk is not a multiple of 32, so their empty key intervals sit inside the last
# 32-key block.  dk/dv writes no dU block for those waves; the dq kernels must read none.
BLIND = {
    "bf16_d128": dict(dtype="bf16", D=128, B=1, S=252, Sk=56, Hq=2, Hkv=1, causal=False, window=47),
    "bf16_d512": dict(dtype="bf16", D=512, B=1, S=184, Sk=59, Hq=2, Hkv=1, causal=False, window=42),
    "fp16_d64": dict(dtype="fp16", D=64, B=1, S=300, Sk=33, Hq=2, Hkv=1, causal=False, window=5),
    "fp32_d128": dict(dtype="fp32", D=128, B=2, S=171, Sk=89, Hq=2, Hkv=1, causal=False, window=38,
                      bias=True, bias_bcast="batch"),
}


@pytest.mark.parametrize("name", list(BLIND))
def test_queries_that_see_no_key_get_zero_dq_from_the_du_blocks(name, monkeypatch):
    c = case(**BLIND[name])
    Sk, window = c["k"].shape[1], c["window"]
    blind = np.arange(c["q"].shape[1]) >= Sk + window - 1
    assert any(blind[32 * w:32 * w + 32].all() for w in range(len(blind) // 32)), "no whole blind wave"
    print(f"blind query waves: {name}", flush=True)
    monkeypatch.setattr(ops, "_workspace", _poisoned)
    gpu = run_gpu(c, dq_mode="du_blocks")
    assert (gpu["dq"][:, blind] == 0).all(), f"{name}: dq of queries that see no key is not zero"
    assert (gpu["out"][:, blind] == 0).all()
    errs = compare(gpu, run_oracle(c), c["dtype"], per_head=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[c["dtype"]]}
    assert not bad, f"over tolerance {TOL[c['dtype']]}: {bad}"


# The 16-bit dk/dv kernels stage the bias tile of an item in LDS.  In the last key block some
# keys lie past Sk; their chunks must read as zeros, not as the next row's keys and, after the
# last row, not as whatever follows the bias in memory (here NaN): the dU blocks carry those
# keys' values to the dq kernel, which multiplies them by zero K rows.
BIAS_TAIL = {
    "d128": dict(dtype="bf16", D=128, B=2, S=200, Hq=4, Hkv=2, bias=True, softcap=50.0),
    "d256": dict(dtype="bf16", D=256, B=2, S=200, Hq=4, Hkv=1, bias=True, softcap=30.0),
    "d128_fp16_noncausal": dict(dtype="fp16", D=128, B=1, S=136, Hq=2, Hkv=1, bias=True, causal=False),
}


@pytest.mark.parametrize("name", list(BIAS_TAIL))
def test_bias_tiles_read_nothing_past_the_last_key(name):
    c = case(**BIAS_TAIL[name])
    print(f"NaN after the bias: {name}", flush=True)
    clean = run_gpu(c, dq_mode="du_blocks")
    tail = run_gpu(c, dq_mode="du_blocks", nan_after_bias=True)
    for n, x in clean.items():
        if x is None:
            continue
        assert not np.isnan(tail[n]).any(), f"{name}: {n} picked up the NaN after the bias"
        assert x.tobytes() == tail[n].tobytes(), f"{name}: {n} depends on the memory after the bias"


# Every uploaded input (q, k, v, dO, bias) at the start of a buffer whose tail is NaN: no kernel
# may read past an input's last element.
TAILS = {
    "bf16_d128_segments_bias": dict(dtype="bf16", D=128, B=2, S=200, Hq=4, Hkv=2, bias=True,
                                    segments=[[45, 70, 190], [128]], sink_mode="learnable"),
    "bf16_d512_bias_dropout": dict(dtype="bf16", D=512, B=1, S=200, Hq=2, Hkv=1, bias=True, dropout_p=0.1),
    "fp32_d256_window": dict(dtype="fp32", D=256, B=2, S=131, Hq=4, Hkv=2, window=40, bias=True,
                             bias_bcast="heads"),
    "fp16_d64_cross": dict(dtype="fp16", D=64, B=2, S=150, Sk=97, Hq=4, Hkv=1, causal=False, window=30),
}


@pytest.mark.parametrize("name", list(TAILS))
def test_no_kernel_reads_past_an_input(name, monkeypatch):
    c = case(**TAILS[name])
    print(f"NaN after every input: {name}", flush=True)
    clean = run_gpu(c, dq_mode="du_blocks")
    orig = harness.to_dev

    def to_dev_tail(x, dtype, device="cuda"):
        t = orig(x, dtype, device)
        buf = torch.full((t.numel() + 8192,), float("nan"), dtype=t.dtype, device=t.device)
        buf[:t.numel()] = t.reshape(-1)
        return buf[:t.numel()].view(t.shape)

    monkeypatch.setattr(harness, "to_dev", to_dev_tail)
    tail = run_gpu(c, dq_mode="du_blocks")
    for n, x in clean.items():
        if x is None:
            continue
        assert x.tobytes() == tail[n].tobytes(), f"{name}: {n} depends on the memory after the inputs"
