"""Planted mistakes in a copy of the CPU oracle: every one must fail a pin.

Each case below edits one expression of oracle/lora_ref.py the way a plausible
slip would (a dropped term or scale, a wrong sign, a transposed operand, a
wrong index or nibble order, a rounding mode), loads the edited source as a
separate module, and runs every pin of tests/test_oracle_pins.py against it.
The case passes when at least one pin fails (an assertion or an exception,
e.g. a shape error).  The unedited copy must pass every pin, so the failures
come from the planted mistake alone.  The real oracle module is never
modified.
"""
import importlib.util
import inspect
import os
import types
import warnings

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "lora_ref.py")

# (case, exact text in the oracle, replacement)
MUTANTS = [
    # LoRA linear forward: Y = X W^T + s (X A^T) B^T
    ("fwd_scale_dropped", "    return X @ W.T + s * (H @ B.T)", "    return X @ W.T + (H @ B.T)"),
    ("fwd_lora_sign", "    return X @ W.T + s * (H @ B.T)", "    return X @ W.T - s * (H @ B.T)"),
    ("fwd_base_weight_transposed", "    return X @ W.T + s * (H @ B.T)",
     "    return X @ W + s * (H @ B.T)"),
    ("scaling_inverted", "    return float(alpha) / float(r)", "    return float(r) / float(alpha)"),
    ("trainable_params_wrong", "    return r * n + r * k", "    return r * n + k"),
    ("merge_scale_dropped", "    return _f64(W) + s * (_f64(B) @ _f64(A))",
     "    return _f64(W) + (_f64(B) @ _f64(A))"),
    # LoRA linear backward
    ("dx_lora_term_dropped", "    dX = dY @ W + s * (G @ A) if want_dx else None",
     "    dX = dY @ W if want_dx else None"),
    ("dx_lora_scale_dropped", "    dX = dY @ W + s * (G @ A) if want_dx else None",
     "    dX = dY @ W + (G @ A) if want_dx else None"),
    ("dA_scale_dropped", "    dA = s * (G.T @ X)", "    dA = (G.T @ X)"),
    ("dB_scale_dropped", "    dB = s * (dY.T @ H)", "    dB = (dY.T @ H)"),
    # SwiGLU and its derivative
    ("sigmoid_sign", "        return 1.0 / (1.0 + np.exp(-z))", "        return 1.0 / (1.0 + np.exp(z))"),
    ("glu_instead_of_swiglu", "    return e * sigmoid(e) * g", "    return sigmoid(e) * g"),
    ("silu_derivative_sign", "    de = dh * g * sg * (1.0 + e * (1.0 - sg))",
     "    de = dh * g * sg * (1.0 - e * (1.0 - sg))"),
    ("de_missing_g", "    de = dh * g * sg * (1.0 + e * (1.0 - sg))",
     "    de = dh * sg * (1.0 + e * (1.0 - sg))"),
    ("dg_missing_e", "    dg = dh * e * sg", "    dg = dh * sg"),
    # MLP composition
    ("down_reads_e_not_h", '    Y = linear_fwd(h, W["down"], A["down"], B["down"], s)',
     '    Y = linear_fwd(e, W["down"], A["down"], B["down"], s)'),
    ("gate_up_swapped_in_bwd", "    de, dg = swiglu_bwd(e, g, dh)", "    de, dg = swiglu_bwd(g, e, dh)"),
    ("dx_up_branch_dropped", '        out["dX"] = dXg + dXu', '        out["dX"] = dXg'),
    # bf16 rounding and the 4-bit decode
    ("bf16_round_half_up", "    rounded = (u + 0x7FFF + lsb) >> 16", "    rounded = (u + 0x8000) >> 16"),
    ("bf16_truncate", "    rounded = (u + 0x7FFF + lsb) >> 16", "    rounded = u >> 16"),
    ("nibble_order_swapped", "    nib[0::2] = flat & 0x0F\n    nib[1::2] = flat >> 4",
     "    nib[0::2] = flat >> 4\n    nib[1::2] = flat & 0x0F"),
    ("absmax_block_index", "np.repeat(am, blocksize)", "np.tile(am, blocksize)"),
    ("dq_offset_sign", "    return (m + np.float32(absmax_offset)).astype(np.float32)",
     "    return (m - np.float32(absmax_offset)).astype(np.float32)"),
    ("dq_scale_group_index", "    group = np.arange(nblocks) // blocksize2",
     "    group = np.arange(nblocks) % sc.size"),
    # RMSNorm
    ("rmsnorm_sum_not_mean", "    rstd = 1.0 / np.sqrt(np.mean(X * X, axis=1) + float(eps))",
     "    rstd = 1.0 / np.sqrt(np.sum(X * X, axis=1) + float(eps))"),
    ("rmsnorm_eps_dropped", "    rstd = 1.0 / np.sqrt(np.mean(X * X, axis=1) + float(eps))",
     "    rstd = 1.0 / np.sqrt(np.mean(X * X, axis=1))"),
    ("rmsnorm_bwd_projection_dropped", "    return r[:, None] * g - (r ** 3 * dot / d)[:, None] * X",
     "    return r[:, None] * g"),
    ("rmsnorm_bwd_missing_1_over_d", "    return r[:, None] * g - (r ** 3 * dot / d)[:, None] * X",
     "    return r[:, None] * g - (r ** 3 * dot)[:, None] * X"),
    ("rmsnorm_bwd_weight_dropped", "    g = dY * w[None, :]", "    g = dY"),
    # comparator and the 4-bit container dispatch
    ("rel_fro_norm_difference", "    num = np.linalg.norm((x - ref).ravel())",
     "    num = abs(np.linalg.norm(x.ravel()) - np.linalg.norm(ref.ravel()))"),
    ("rel_fro_max_abs", "    num = np.linalg.norm((x - ref).ravel())",
     "    num = np.max(np.abs(x - ref))"),
    ("rel_fro_no_ratio", "    return float(num / den)", "    return float(num)"),
    ("rel_fro_squared", "    return float(num / den)", "    return float((num / den) ** 2)"),
    ("rel_fro_denominator_x", "    den = np.linalg.norm(ref.ravel())",
     "    den = np.linalg.norm(x.ravel())"),
    ("rel_fro_zero_reference_passes", '        return 0.0 if num == 0.0 else float("inf")',
     "        return 0.0"),
    ("rel_fro_sum_not_difference", "    num = np.linalg.norm((x - ref).ravel())",
     "    num = np.linalg.norm((x + ref).ravel())"),
    ("dispatch_dims_swapped", "q.absmax_offset, q.codebook, q.n, q.k, q.blocksize,",
     "q.absmax_offset, q.codebook, q.k, q.n, q.blocksize,"),
    ("dispatch_plain_dims_swapped", "    return decode_q4(q.codes, q.absmax, q.codebook, q.n, q.k, q.blocksize)",
     "    return decode_q4(q.codes, q.absmax, q.codebook, q.k, q.n, q.blocksize)"),
    ("dispatch_dq_ignored", '    if getattr(q, "absmax_codes", None) is not None:',
     '    if getattr(q, "absmax", None) is None and False:'),
]


def _source():
    with open(ORACLE_SRC) as fh:
        return fh.read()


def _module_from(src, name):
    mod = types.ModuleType(name)
    mod.__file__ = ORACLE_SRC
    exec(compile(src, ORACLE_SRC, "exec"), mod.__dict__)
    return mod


def _pins_module():
    # a private instance of the pins module, so that its `oracle` name can be
    # pointed at a variant without touching the module pytest collected
    spec = importlib.util.spec_from_file_location("_pins_under_mutation",
                                                  os.path.join(HERE, "test_oracle_pins.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_PINS = None


def _failing_pins(oracle_variant):
    global _PINS
    if _PINS is None:
        _PINS = _pins_module()
    tests = [(n, f) for n, f in vars(_PINS).items()
             if n.startswith("test_") and callable(f) and not inspect.signature(f).parameters]
    assert len(tests) >= 25
    saved = _PINS.oracle
    _PINS.oracle = oracle_variant
    failed = []
    try:
        for n, f in tests:
            try:
                with warnings.catch_warnings():
                    warnings.simplefilter("ignore")
                    f()
            except Exception:   # an assertion, or an error the mistake causes
                failed.append(n)
    finally:
        _PINS.oracle = saved
    return failed


def test_unmodified_copy_passes_every_pin():
    assert _failing_pins(_module_from(_source(), "oracle_copy")) == []


@pytest.mark.parametrize("case,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(case, old, new):
    src = _source()
    assert src.count(old) == 1, f"{case}: the edited text must occur once in the oracle"
    failed = _failing_pins(_module_from(src.replace(old, new), "oracle_" + case))
    assert failed, f"no pin catches the planted mistake {case}"
