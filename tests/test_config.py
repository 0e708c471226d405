"""DeepSpeed-style config reading (host only).

Pins: the two configuration examples the pages print (tests/golden/README.md
names their sources), the batch identity of [Deep dive] "Let the engine own
the microstep" (64 = 2 x 8 x 4 data ranks; eight ranks with the same three
fields is inconsistent), and rejection of malformed fields.
"""
import json
import os

import pytest

import bench
from zero_sharded_optimizer_owned_amd.config import step_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(name):
    return os.path.join(GOLDEN, name)


def test_stage3_fp16_example():
    c = step_config(_cfg("ds_config_stage3_fp16.json"))
    assert c["hyper"] == {"lr": 1e-3, "beta1": 0.8, "beta2": 0.999, "eps": 1e-8, "weight_decay": 3e-7,
                          "adamw": True}
    assert (c["param_dtype"], c["stage"], c["gradient_accumulation_steps"], c["data_parallel"]) == \
        ("fp16", 3, 1, None)
    # the benchmark's optimizer settings are this example's
    assert c["hyper"] == bench.HP


def test_stage2_bf16_example_gives_four_data_ranks():
    c = step_config(_cfg("ds_config_stage2_bf16.json"))
    assert c["hyper"] == {"lr": 2e-5, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.01,
                          "adamw": True}
    assert c["param_dtype"] == "bf16" and c["grad_accum_dtype"] == "fp32"
    assert (c["stage"], c["gradient_accumulation_steps"], c["reduce_bucket_size"]) == (2, 8, 200_000_000)
    assert c["data_parallel"] == 4
    assert step_config(_cfg("ds_config_stage2_bf16.json"), ranks=4)["data_parallel"] == 4
    with pytest.raises(ValueError):
        step_config(_cfg("ds_config_stage2_bf16.json"), ranks=8)


def test_bucket_bytes_follow_the_element_width():
    """[Deep dive] "Let the engine own the microstep": the bucket size counts elements;
    2e8 of them take 400 MB at two bytes and 800 MB at four."""
    c = step_config(_cfg("ds_config_stage2_bf16.json"))
    assert c["reduce_bucket_size"] * 2 == 400_000_000
    assert c["reduce_bucket_size"] * 4 == 800_000_000


def test_two_batch_fields_and_the_rank_count_fix_the_third():
    base = json.load(open(_cfg("ds_config_stage2_bf16.json")))
    for drop in ("train_batch_size", "train_micro_batch_size_per_gpu", "gradient_accumulation_steps"):
        c = dict(base)
        del c[drop]
        assert step_config(c, ranks=8)["data_parallel"] == 8
    c = dict(base)
    del c["gradient_accumulation_steps"]
    assert step_config(c, ranks=8)["gradient_accumulation_steps"] == 4   # 64 = 2 x 4 x 8
    with pytest.raises(ValueError):
        step_config(c, ranks=5)                                           # 64 / (2 x 5) is not whole


def test_json_text_and_adam_variants():
    text = json.dumps({"optimizer": {"type": "Adam", "params": {"lr": 0.01, "weight_decay": 0.1}}})
    c = step_config(text)
    assert c["hyper"]["adamw"] is False and c["hyper"]["lr"] == 0.01
    assert (c["hyper"]["beta1"], c["hyper"]["beta2"], c["hyper"]["eps"]) == (0.9, 0.999, 1e-8)
    assert c["param_dtype"] == "fp32" and c["gradient_accumulation_steps"] == 1
    c = step_config({"optimizer": {"type": "Adam", "params": {"adam_w_mode": True}}})
    assert c["hyper"]["adamw"] is True


@pytest.mark.parametrize("bad", [
    {},
    {"optimizer": {"type": "SGD"}},
    {"optimizer": {"type": "AdamW", "params": {"betas": [0.9]}}},
    {"optimizer": {"type": "AdamW", "params": {"betas": [0.9, 1.0]}}},
    {"optimizer": {"type": "AdamW", "params": {"lr": "0.1"}}},
    {"optimizer": {"type": "AdamW", "params": {"lr": -1.0}}},
    {"optimizer": {"type": "AdamW", "params": {"adam_w_mode": 1}}},
    {"optimizer": {"type": "AdamW"}, "fp16": {"enabled": True}, "bf16": {"enabled": True}},
    {"optimizer": {"type": "AdamW"}, "zero_optimization": {"stage": 4}},
    {"optimizer": {"type": "AdamW"}, "train_batch_size": 10, "train_micro_batch_size_per_gpu": 3,
     "gradient_accumulation_steps": 1},
    {"optimizer": {"type": "AdamW"}, "gradient_accumulation_steps": 0},
    {"optimizer": {"type": "AdamW"}, "data_types": {"grad_accum_dtype": "int8"}},
])
def test_rejects_malformed(bad):
    with pytest.raises(ValueError):
        step_config(bad)
