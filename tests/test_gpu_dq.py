"""GPU parity of the 4-bit form with double-quantised block constants (8-bit
absmax codes through a 256-level table, one fp32 scale per 256 blocks, one
offset) against the float64 oracle: the standalone decode bit-exact, and
every entry point that takes a base weight within the bf16 tolerance, in
both workspace strategies (decoded copy, or decode inside the GEMM)."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_linear, gen_mlp

from gpu_helpers import check, dev, host, linear_weight, log
from test_gpu_merge import _sync
from test_gpu_parity import WS_MODES, check_linear, check_mlp
from test_gpu_qkv import make_qkv, run_and_check

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# (n, k): one 256-block group; a partial last group (360 blocks); many groups
@pytest.mark.parametrize("nk", [(1, 64), (72, 320), (4096, 1024)], ids=str)
def test_decode_weight_dq_bit_exact(nk):
    n, k = nk
    log(f"decode dq n={n} k={k}")
    q = gen_linear(1, k, n, 1, 1.0, "bf16", seed=n + k, q4="dq").q4
    out = L.lora_decode_weight(L.to_device_q4(q))
    _sync()
    ref = oracle.decode_q4dq_bits(q.codes, q.absmax_codes, q.absmax_codebook, q.absmax_scale,
                                  q.absmax_offset, q.codebook, n, k)
    assert np.array_equal(_bits(out), ref)


def test_decode_weight_plain_q4_matches_dequant4():
    q = L.to_device_q4(gen_linear(1, 320, 264, 1, 1.0, "bf16", seed=4, q4=True).q4)
    a, b = L.lora_decode_weight(q), L.lora_dequant4(q)
    _sync()
    assert np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("ws", WS_MODES)
def test_linear_q4dq(ws):
    log(f"linear q4dq ws={ws}")
    check_linear(gen_linear(300, 320, 264, 16, 16.0, "bf16", seed=31, q4="dq"), ws=ws)
    check_linear(gen_linear(77, 128, 136, 16, 16.0, "bf16", seed=32, q4="dq", b_std=1.0), ws=ws)


@pytest.mark.parametrize("ws", WS_MODES)
def test_mlp_q4dq(ws):
    log(f"mlp q4dq T=300 d=256 f=576 r=16 ws={ws}")
    check_mlp(gen_mlp(300, 256, 576, 16, 16.0, "bf16", seed=33, q4="dq"), ws=ws)
    check_mlp(gen_mlp(70, 128, 192, 16, 16.0, "bf16", seed=34, q4="dq", b_std=1.0), ws=ws)


@pytest.mark.parametrize("ws", WS_MODES)
@pytest.mark.parametrize("form", [True, "dq"], ids=["q4", "q4dq"])
def test_mlp_gate_up_distinct_tables(form, ws):
    """Gate and up weights with different 16-level codebooks (and, double
    quantised, different 256-level tables and offsets): the fused gate/up
    GEMM and the stacked dX GEMM must decode each with its own."""
    log(f"mlp gate/up distinct tables form={form} ws={ws}")
    mi = gen_mlp(260, 192, 320, 8, 16.0, "bf16", seed=35, q4=form)
    up = mi.q4["up"]
    up.codebook = (up.codebook[::-1] * np.float32(-0.5)).astype(np.float32)
    if form == "dq":
        up.absmax_codebook = (up.absmax_codebook * np.float32(0.75)).astype(np.float32)
        up.absmax_offset = 0.05
    check_mlp(mi, ws=ws)


def test_merge_q4dq():
    li = gen_linear(1, 256, 136, 16, 16.0, "bf16", seed=36, q4="dq", b_std=0.5)
    s = oracle.scaling(li.alpha, li.r)
    Wd, Wref = linear_weight(li)
    A, B = dev(li.A, "bf16"), dev(li.B, "bf16")
    out = L.lora_merge(Wd, A, B, li.alpha)
    _sync()
    check("W' (double-quantised 4-bit base)", host(out),
          oracle.merged_weight(Wref, li.A, li.B, s), "bf16")


@pytest.mark.parametrize("ws", WS_MODES)
def test_qkv_q4dq(ws):
    log(f"qkv q4dq ws={ws}")
    run_and_check(make_qkv(130, 256, 512, 256, 16, seed=37, q4="dq"), ws=ws)
