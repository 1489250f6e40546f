"""Pin the oracle's closed-form storage counts to the figures the pages print.

The fixture ``tests/golden/page_figures.json`` holds each printed number with
its citation and the tolerance its wording ("about", "~") allows.
"""

import json
import os

import pytest

from oracle import accounting

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
GB = 1e9


def _close(value, key):
    ref = GOLD[key]
    tol = ref["tol"]
    if isinstance(ref["value"], list):
        lo, hi = ref["value"]
        return lo <= value <= hi
    return abs(value - ref["value"]) <= tol * abs(ref["value"])


@pytest.mark.parametrize("key,value", [
    ("lora_params_r8_d4096", accounting.lora_param_count(8, 4096, 4096)),
    ("full_params_d4096", 4096 * 4096),
    ("fp32_constant_bits", accounting.constant_bits_per_param(double_quant=False)),
    ("dq_constant_bits", accounting.constant_bits_per_param(double_quant=True)),
    ("dq_saving_bits", accounting.constant_bits_per_param(False) - accounting.constant_bits_per_param(True)),
    ("dq_saving_65B_GB", accounting.dq_saving_bytes(65e9) / GB),
    ("dq_saving_70B_GB", accounting.dq_saving_bytes(70e9) / GB),
    ("blocks_70B", 70e9 / 64),
    ("fp32_constants_70B_GB", accounting.first_level_constant_bytes(int(70e9)) / GB),
    ("fp16_70B_GB", 70e9 * 2 / GB),
    ("nf4_70B_GB", accounting.code_bytes(int(70e9)) / GB),
    ("fp16_65B_GB", 65e9 * 2 / GB),
    ("nf4_65B_GB_range", 65e9 * accounting.bits_per_param() / 8 / GB),
])
def test_page_figure(key, value):
    assert _close(value, key), (key, value, GOLD[key])


def test_exact_storage_of_the_format():
    assert accounting.bits_per_param() == 4 + 8 / 64 + 64 / 16384 == 4.12890625
    assert accounting.stored_bytes(4096, 4096) == 4096 * 4096 // 2 + 4096 * 64 + 8 * 1024
    # the small-M weight stream of a 4096 -> 11008 linear (codes, int8 constants, fp32 scale+offset)
    assert accounting.stored_bytes(11008, 4096) == 22544384 + 704512 + 8 * 2752
