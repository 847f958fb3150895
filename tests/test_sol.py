"""Bytes-per-step and speed-of-light: the oracle's calculator against the pages' numbers."""
import json
import os

import oracle as O
from fixtures import workload

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sol_worked_examples.json")))


def test_megakernel_page_worked_numbers():
    g = GOLD["megakernel_h100"]
    sol = O.speed_of_light(g["weight_bytes"] + g["kv_bytes_8k"], g["bandwidth_Bps"])
    assert abs(sol - g["sol_tok_s_about"]) < 5          # 471.8 ~ "about 470"
    assert round(100 * g["vllm_tok_s"] / g["sol_tok_s_about"]) == g["vllm_frac_sol_pct"]
    assert round(100 * g["megakernel_tok_s"] / g["sol_tok_s_about"]) == g["megakernel_frac_sol_pct"]
    assert round(g["megakernel_tok_s"] / g["vllm_tok_s"], 2) == g["speedup_over_vllm"]


def test_kinetic_bandwidth_wall():
    g = GOLD["kinetic_bandwidth_wall"]
    sol = O.speed_of_light(g["model_bytes"], g["bandwidth_Bps"])
    assert abs(sol - g["tok_s_near"]) < 5                # 107 ~ "near 110"


def test_moe48_parameter_counts_match_the_page():
    g = GOLD["megakernel_h100"]
    total, active = O.param_counts(workload("moe48_b1_8k")["model"])
    assert abs(total / g["params_total_about"] - 1) < 0.03     # 30.5B ~ "30B"
    assert abs(active / g["params_active_about"] - 1) < 0.03   # 3.35B ~ "3.3B"
    assert abs(2 * active / g["weight_bytes"] - 1) < 0.03      # 6.7 GB ~ "6.6 GB"


def test_moe48_step_bytes():
    m = workload("moe48_b1_8k")["model"]
    w, kr, kw = O.step_bytes(m, [8192])
    assert abs(w / 1e9 - 6.084) < 0.002
    assert abs((kr + kw) / 1e9 - 0.805) < 0.002
    sol = O.speed_of_light(w + kr + kw, 8.0e12)
    assert abs(sol - 1161) < 2
    w5, kr5, kw5 = O.step_bytes(m, [262144])
    assert abs(kr5 / 1e9 - 25.77) < 0.01            # "about 25 GB" of paged KV
    # dense tiny decoder: every FFN weight is read
    t = workload("tiny_dense")["model"]
    wt, _, _ = O.step_bytes(t, [128])
    assert wt == 2 * (2 * (256 * 512 + 256 * 256 + 3 * 256 * 512) + 1024 * 256 + 256 + 5 * 256)
