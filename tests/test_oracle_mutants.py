"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each of them. This is what makes the pins meaningful:
a pin set that passes a broken oracle would not pin anything."""
import inspect
import types

import pytest

import oracle.paged_attention as pa
from oracle_pins import PINS

MUTANTS = {
    "gqa_mapping_modulo": ("h = j // group", "h = j % Hkv"),
    "scale_dropped": ("z = scale * (ks[:, h, :] @ qf[s, j])", "z = (ks[:, h, :] @ qf[s, j])"),
    "gather_block_offset_swapped": ("return rows.reshape(", "return rows.transpose(1, 0, 2, 3).reshape("),
    "gather_off_by_one": ("[:length]\n", "[1:length + 1]\n"),
    "softmax_unnormalised": ("w = e / e.sum()", "w = e"),
    "reads_k_as_v": ("out[s, j] = w @ vs[:, h, :]", "out[s, j] = w @ ks[:, h, :]"),
    "bf16_widen_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "fp16_as_bf16": ("return bits.view(np.float16).astype(np.float64)",
                     "return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)"),
    "merge_no_rescale": ("w = np.array([l * math.exp(m - big_m)", "w = np.array([l * 1.0"),
    "merge_unweighted": ("out[s, j] = (w[:, None] * np.array(os_)).sum(axis=0) / w.sum()",
                         "out[s, j] = np.array(os_).mean(axis=0)"),
    "cache_slot_divmod_swapped": ("blk, off = divmod(int(slot), block_size)",
                                  "off, blk = divmod(int(slot), block_size)"),
    "cache_negative_not_skipped": ("if slot < 0:\n            continue", "if False:\n            continue"),
    "mq_no_causal_mask": ("visible = length - n_new + i + 1", "visible = length"),
    "mq_causal_off_by_one": ("visible = length - n_new + i + 1", "visible = length - n_new + i + 2"),
    "mq_positions_from_start": ("visible = length - n_new + i + 1", "visible = i + 1"),
    "mq_query_rows_reversed": ("row = first + i\n", "row = first + n_new - 1 - i\n"),
    "prefill_not_causal": ("row + 1", "hi"),
    "prefill_crosses_prompts": ("lo:row + 1", "0:row + 1"),
    "prefill_head_mapping": ("                h = j // group\n                z = scale * (kf",
                             "                h = j % key.shape[1]\n                z = scale * (kf"),
    "length_ignores_last_token": ("length = int(context_lens[s])\n        if length <= 0:\n            weights",
                                  "length = int(context_lens[s]) - 1\n        if length <= 0:\n            weights"),
}


def make_mutant(old, new):
    src = inspect.getsource(pa)
    assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mutant = make_mutant(*MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
