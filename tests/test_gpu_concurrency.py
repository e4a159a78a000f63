"""Concurrent use of the library: launches interleaved on two streams, and calls from two
host threads, each checked against the oracle (the library keeps no state between calls,
so independent calls must not interfere)."""

import sys
import threading

import numpy as np
import pytest
import torch

import gpu_util as G
from residual_add_rmsnorm_fp32_amd import binding as B
from residual_add_rmsnorm_fp32_amd import workloads as wk

pytestmark = pytest.mark.gpu

CASES = [  # (seed, P, T, H, quant): a decode-shaped and a prefill-shaped call
    (101, 8, 80, 4096, "none"),
    (102, 2, 512, 5120, "dynamic"),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _device_inputs(inp):
    return ([G.to_dev(p, "bf16") for p in inp["partials"]], G.to_dev(inp["residual"], "bf16"),
            G.to_dev(inp["gamma"], "bf16"))


def _check(outs, inp, quant, tag):
    ref = G.run_oracle(inp, "bf16", 1e-6, 0.0, quant)
    H = inp["gamma"].shape[-1]
    got = {"new_residual": G.codes_of(outs[1]).reshape(-1, H)}
    if quant == "none":
        got["norm_out"] = G.codes_of(outs[0]).reshape(-1, H)
    else:
        got["quant_out"] = G.codes_of(outs[0]).reshape(-1, H)
        got["scale_out"] = G.codes_of(outs[2]).reshape(-1)
    return G.compare(got, ref, "bf16", quant, inp, tag=tag)


def test_interleaved_streams():
    """Two streams at the default priority, launches alternating between them, each
    stream rewriting its own outputs; the last result on each must equal the oracle's."""
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    inputs = [wk.random_case(s, P, T, H) for s, P, T, H, _ in CASES]
    dev = [_device_inputs(inp) for inp in inputs]
    torch.cuda.synchronize()
    outs = [None, None]
    for it in range(20):
        for i, (st, (parts, res, gam)) in enumerate(zip(streams, dev)):
            quant = CASES[i][4]
            with torch.cuda.stream(st):
                outs[i] = B.fused_add_rmsnorm(parts, res, gam, 1e-6, 0.0,
                                              quant=None if quant == "none" else quant)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs):
        _say(f"[concurrency] stream {i} case {CASES[i]}")
        _check(outs[i], inp, CASES[i][4], f"stream {i}")


def test_two_host_threads():
    """Two host threads, each on its own stream, calling the library at the same time."""
    inputs = [wk.random_case(s + 100, P, T, H) for s, P, T, H, _ in CASES]
    results = [None, None]
    errors = []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                parts, res, gam = _device_inputs(inputs[i])
                quant = CASES[i][4]
                for _ in range(20):
                    out = B.fused_add_rmsnorm(parts, res, gam, 1e-6, 0.0,
                                              quant=None if quant == "none" else quant)
                st.synchronize()
                results[i] = out
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for i, inp in enumerate(inputs):
        _say(f"[concurrency] thread {i} case {CASES[i]}")
        _check(results[i], inp, CASES[i][4], f"thread {i}")

