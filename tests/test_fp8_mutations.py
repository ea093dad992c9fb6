"""Planted mistakes in copies of the FP8 pre-pass oracle (oracle/fp8.py) must each fail a pin.

Each mutation is a plausible slip in the pre-pass: a rounding tie broken the wrong way, an
exponent off by one, a scale factor or the sign diagonal dropped, the sign of an exact zero
kept, V rotated too, the per-tensor amax taken over one block or one sequence, packed
sequences quantised on blocks of the packed axis, the scale floor lost or not shifted for K.
The altered source is loaded as a module of its own and the pins of tests/test_fp8_oracle.py
are run against it; the test passes only if some pin rejects it.
"""
import importlib.util
import inspect
import os

import pytest

import oracle
from tests import test_fp8_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fp8.py")

MUTATIONS = {
    "ties_to_odd": ("((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    "exponent_off_by_one": ("return ex - 9 if m <= 0.875 else ex - 8", "return ex - 8 if m <= 0.875 else ex - 7"),
    "rotation_without_signs": ("return (x * np.asarray(signs, dtype=np.float64)) @ hadamard(d)",
                               "return x @ hadamard(d)"),
    "k_scale_without_1_over_d": ("to_scale(ek - shift_k)", "to_scale(ek)"),
    "v_rotated": ("v8, ev = quant(np.asarray(v, dtype=np.float64), block)",
                  "v8, ev = quant(rotate(v, signs), block)"),
    "tensor_amax_from_first_block": ("e = max(block_exponent(float(np.max(np.abs(y))) if y.size else 0.0), e_floor)",
                                     "e = max(block_exponent(float(np.max(np.abs(y[:, :block])))), e_floor)"),
    "block_scale_without_floor": (
        "exps[b, h, j] = max(block_exponent(float(np.max(np.abs(blk))) if blk.size else 0.0), e_floor)",
        "exps[b, h, j] = block_exponent(float(np.max(np.abs(blk))) if blk.size else 0.0)"),
    "k_floor_not_shifted": ("SCALE_EXP_MIN + shift_k)", "SCALE_EXP_MIN)"),
    "varlen_tensor_amax_from_first_sequence": (
        "e_tensor = max(block_exponent(float(np.max(np.abs(y))) if y.size else 0.0), floor)",
        "e_tensor = max(block_exponent(float(np.max(np.abs(y[:cu[1]])))), floor)"),
    "varlen_blocks_not_restarted": ("c, e = quantize_blocks(seq, block, floor)",
                                    "c, e = quantize_blocks(y[None, :cu[b + 1]], block, floor)\n"
                                    "                c = c[:, cu[b]:]"),
    "rope_sin_sign": ("r0 = (x0 * c) - (x1 * s)", "r0 = (x0 * c) + (x1 * s)"),
    "rope_half_split_pairs": ("x0 = x[..., 0::2].astype(np.float32)", "x0 = x[..., 1::2].astype(np.float32)"),
    "rope_positions_from_packed_axis": (
        "pos = np.concatenate([np.arange(cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]).astype(np.int64)",
        "pos = np.arange(cu[-1])"),
    "bf16_ties_up": ("r = ((u + 0x7FFF + keep_lsb) >> 16) << 16", "r = ((u + 0x8000) >> 16) << 16"),
    "signed_zero_kept": ("-int(exps[b, h, j])) + 0.0)", "-int(exps[b, h, j])))"),
    "dequantize_next_block": ("tok_blk = np.arange(N) // block", "tok_blk = np.minimum(np.arange(N) // block + 1, "
                              "scales.shape[2] - 1)"),
}

# every parametrised pin runs with each of these arguments
_ARGS = {"per_tensor": (False, True), "d": (16,)}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        if not params:
            calls.append((name, fn, {}))
        else:
            (p,) = params
            calls.extend((f"{name}[{a}]", fn, {p: a}) for a in _ARGS[p])
    return calls


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_fp8_mutation_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "fp8_mutated.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("fp8_mutated", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(pins, "fp8", mod)
    for pin_name, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except (AssertionError, ValueError, IndexError):
            return  # caught
    pytest.fail(f"no pin caught the planted mistake {name}")
