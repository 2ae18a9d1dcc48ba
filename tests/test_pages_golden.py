"""Values the pages print, checked against the configuration, the flat
parameter layout and the synthetic workload (tests/golden/pages_d20.json)."""
import json
import math
import os

import numpy as np
import pytest

import synthdata

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_d20.json")))


def g(k):
    return GOLD[k]["value"]


def test_d20_shape_matches_pages():
    cfg = synthdata.get_config("d20")
    assert cfg.n_layer == g("n_layer")
    assert cfg.d_model == g("d_model")
    assert cfg.n_head == g("n_head") and cfg.head_dim == g("head_dim")
    assert cfg.n_head * cfg.head_dim == cfg.d_model
    assert cfg.batch == g("rows_per_gpu") and cfg.seq_len == g("seq_len")
    assert cfg.batch * cfg.seq_len * g("n_gpu") == g("tokens_per_step") == 2 ** 19


def test_d20_param_count_and_chinchilla_arithmetic():
    cfg = synthdata.get_config("d20")
    P = synthdata.param_count(cfg)
    # 12 L d^2 (no biases, no norm parameters) + untied embedding and unembedding
    assert P == 12 * cfg.n_layer * cfg.d_model ** 2 + 2 * cfg.vocab * cfg.d_model == 560_988_160
    assert P == pytest.approx(g("params_approx"), rel=GOLD["params_approx"]["rel_tol"])
    tokens = g("chinchilla_ratio") * P
    assert tokens == pytest.approx(g("train_tokens_approx"), rel=GOLD["train_tokens_approx"]["rel_tol"])
    # the arithmetic closes exactly at vocab 65,536: 20 P = 21,400 x 2^19
    assert tokens == 21_400 * g("tokens_per_step")
    assert tokens / g("tokens_per_step") == pytest.approx(g("steps_approx"), rel=GOLD["steps_approx"]["rel_tol"])
    # the other vocabularies the pages mention would not give ~560M
    for V in (50257, 100277):
        other = 12 * cfg.n_layer * cfg.d_model ** 2 + 2 * V * cfg.d_model
        assert abs(other / g("params_approx") - 1) > 0.05


def test_flop_convention_reproduces_4e19():
    from decoder_only_transformer_d20_amd.flops import flops_per_token
    cfg = synthdata.get_config("d20")
    total = flops_per_token(cfg) * g("chinchilla_ratio") * synthdata.param_count(cfg)
    assert total == pytest.approx(g("train_flops_approx"), rel=GOLD["train_flops_approx"]["rel_tol"])


def test_synthetic_bytes_per_token_mean():
    cfg = synthdata.get_config("d20")
    tb = synthdata.make_token_bytes(cfg)
    assert tb.min() >= 1
    assert tb.mean() == pytest.approx(g("chars_per_token"), rel=GOLD["chars_per_token"]["rel_tol"])


def test_synthetic_tokens_follow_zipf():
    cfg = synthdata.get_config("small")
    idx, tgt = synthdata.make_tokens(cfg)
    assert idx.dtype == np.int32 and idx.shape == (cfg.batch, cfg.seq_len)
    np.testing.assert_array_equal(idx[:, 1:], tgt[:, :-1])
    assert idx.min() >= 0 and idx.max() < cfg.vocab
    p0 = 1.0 / np.sum(np.arange(1, cfg.vocab + 1, dtype=np.float64) ** -1.1)
    assert np.mean(idx == 0) == pytest.approx(p0, abs=0.02)
    # same seed -> same draw; a prefix of rows is the same rows
    idx2, _ = synthdata.make_tokens(cfg, rows=3)
    np.testing.assert_array_equal(idx2, idx[:3])


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0, 1e-40], dtype=np.float32)
    r = synthdata.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even
    assert r[2] == 1.0 + 2 ** -6             # tie -> even (upwards)
    assert r[3] == -2.5
    assert np.all(synthdata.round_to_bf16(r) == r)
    assert math.isclose(float(r[4]), 65536.0)
