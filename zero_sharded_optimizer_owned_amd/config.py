"""The optimizer-step settings of a DeepSpeed-style JSON training config.

[ZeRO-3 docs] (the configuration examples of the stage list) and [Deep dive]
"Let the engine own the microstep" show configs whose `optimizer` block names
AdamW with lr, betas, eps and weight_decay, next to the precision switch
(`fp16` / `bf16` enabled), `data_types.grad_accum_dtype`, the ZeRO stage, the
bucket size and the three batch fields.  This module reads exactly those
fields into the arguments of the owner step; everything else in a config is
ignored.

The batch fields obey train_batch_size = train_micro_batch_size_per_gpu *
gradient_accumulation_steps * data-parallel degree ([Deep dive] "Let the
engine own the microstep": the batch counts the samples of one update across
all data ranks); given all three, the data-parallel degree follows, and a rank
count that disagrees with it is an error.
"""
from __future__ import annotations

import json
import os
from typing import Any

_ADAM_TYPES = {"adam": False, "adamw": True}
_DTYPES = {"fp16": "fp16", "float16": "fp16", "half": "fp16", "bf16": "bf16", "bfloat16": "bf16",
           "fp32": "fp32", "float32": "fp32", "float": "fp32"}


def _load(cfg: Any) -> dict:
    if isinstance(cfg, dict):
        return cfg
    if isinstance(cfg, (str, os.PathLike)):
        text = str(cfg)
        if not text.lstrip().startswith("{") and os.path.exists(text):
            with open(text) as f:
                text = f.read()
        return json.loads(text)
    raise TypeError("config must be a dict, JSON text or a path to a JSON file")


def _pos_int(d: dict, key: str):
    v = d.get(key)
    if v is None:
        return None
    if isinstance(v, bool) or not isinstance(v, int) or v <= 0:
        raise ValueError(f"{key} must be a positive integer, got {v!r}")
    return v


def _number(params: dict, key: str, default: float) -> float:
    v = params.get(key, default)
    if isinstance(v, bool) or not isinstance(v, (int, float)):
        raise ValueError(f"optimizer params.{key} must be a number, got {v!r}")
    return float(v)


def step_config(cfg: Any, ranks: int | None = None) -> dict:
    """Owner-step settings of a DeepSpeed-style config (dict, JSON text or path).

    Returns {"hyper": {lr, beta1, beta2, eps, weight_decay, adamw} (the keyword
    set OwnerShard.adam_step takes), "param_dtype": "fp16" | "bf16" | "fp32",
    "grad_accum_dtype": dtype name or None, "stage": int or None,
    "gradient_accumulation_steps": int (1 when absent), "reduce_bucket_size":
    int or None, "data_parallel": int or None}.

    Readings: optimizer type "AdamW" decouples the weight decay and "Adam"
    adds it to the gradient (an explicit boolean "adam_w_mode" in params
    overrides either); missing params take torch's defaults (lr 1e-3, betas
    0.9/0.999, eps 1e-8, weight_decay 0).  Raises ValueError for an unknown
    optimizer type, malformed values, fp16 and bf16 both enabled, or batch
    fields that disagree with each other or with `ranks`.
    """
    c = _load(cfg)
    opt = c.get("optimizer")
    if not isinstance(opt, dict):
        raise ValueError("config has no optimizer block")
    kind = str(opt.get("type", "")).lower()
    if kind not in _ADAM_TYPES:
        raise ValueError(f"optimizer type {opt.get('type')!r} is not Adam or AdamW")
    params = opt.get("params", {})
    if not isinstance(params, dict):
        raise ValueError("optimizer params must be an object")
    adamw = _ADAM_TYPES[kind]
    if "adam_w_mode" in params:
        if not isinstance(params["adam_w_mode"], bool):
            raise ValueError("adam_w_mode must be true or false")
        adamw = params["adam_w_mode"]
    betas = params.get("betas", [0.9, 0.999])
    if not isinstance(betas, (list, tuple)) or len(betas) != 2 or not all(
            isinstance(b, (int, float)) and not isinstance(b, bool) for b in betas):
        raise ValueError(f"betas must be two numbers, got {betas!r}")
    hyper = {"lr": _number(params, "lr", 1e-3), "beta1": float(betas[0]), "beta2": float(betas[1]),
             "eps": _number(params, "eps", 1e-8), "weight_decay": _number(params, "weight_decay", 0.0),
             "adamw": adamw}
    if hyper["lr"] < 0 or hyper["eps"] < 0 or hyper["weight_decay"] < 0:
        raise ValueError("lr, eps and weight_decay must be >= 0")
    if not (0 <= hyper["beta1"] < 1 and 0 <= hyper["beta2"] < 1):
        raise ValueError("betas must lie in [0, 1)")

    def enabled(key):
        blk = c.get(key)
        return isinstance(blk, dict) and bool(blk.get("enabled", False))

    if enabled("fp16") and enabled("bf16"):
        raise ValueError("fp16 and bf16 are both enabled")
    param_dtype = "fp16" if enabled("fp16") else "bf16" if enabled("bf16") else "fp32"
    gad = (c.get("data_types") or {}).get("grad_accum_dtype")
    if gad is not None:
        if str(gad).lower() not in _DTYPES:
            raise ValueError(f"unknown grad_accum_dtype {gad!r}")
        gad = _DTYPES[str(gad).lower()]
    zero = c.get("zero_optimization") or {}
    stage = zero.get("stage")
    if stage is not None and (isinstance(stage, bool) or stage not in (0, 1, 2, 3)):
        raise ValueError(f"zero_optimization.stage must be 0-3, got {stage!r}")
    bucket = _pos_int(zero, "reduce_bucket_size")

    tbs = _pos_int(c, "train_batch_size")
    micro = _pos_int(c, "train_micro_batch_size_per_gpu")
    gas = _pos_int(c, "gradient_accumulation_steps")
    dp = None
    if tbs is not None and micro is not None and gas is not None:
        if tbs % (micro * gas):
            raise ValueError(f"train_batch_size {tbs} is not a multiple of micro batch {micro} x "
                             f"accumulation {gas}")
        dp = tbs // (micro * gas)
    elif ranks is not None and sum(x is not None for x in (tbs, micro, gas)) == 2:
        # two fields and the rank count fix the third
        if tbs is None:
            tbs = micro * gas * ranks
        elif micro is None:
            if tbs % (gas * ranks):
                raise ValueError("batch fields disagree with the rank count")
            micro = tbs // (gas * ranks)
        else:
            if tbs % (micro * ranks):
                raise ValueError("batch fields disagree with the rank count")
            gas = tbs // (micro * ranks)
        dp = ranks
    if ranks is not None and dp is not None and dp != ranks:
        raise ValueError(f"the batch fields give {dp} data-parallel ranks, not {ranks}")
    return {"hyper": hyper, "param_dtype": param_dtype, "grad_accum_dtype": gad, "stage": stage,
            "gradient_accumulation_steps": gas or 1, "reduce_bucket_size": bucket, "data_parallel": dp}
