"""Model-FLOP accounting for the d20 training step (forward + backward).

Per token: 6 * (weight-matmul parameters) for the forward and the two
backward products of every weight matrix (the 12*L*d^2 layer matrices and
the d x V unembedding; the embedding is a gather and costs nothing), plus
12*L*d*T for the attention score and value products (2 * 2 * d * T per layer
in the forward, twice that in the backward), counted over the full T x T
square.  This is the convention that reproduces the pages' "about 4e19
FLOPs" for 11.2B tokens of d20 (speedrun walkthrough, Pretraining) and the
"nearly half" MFU at 0.5 s per 2^19-token step on the node they used.
Recomputation is never counted.
"""


def flops_per_token(cfg) -> float:
    L, d, V, T = cfg.n_layer, cfg.d_model, cfg.vocab, cfg.seq_len
    return 6.0 * (12 * L * d * d + V * d) + 12.0 * L * d * T


def flops_per_token_causal(cfg) -> float:
    """Same, with the attention products counted over the causal half."""
    L, d, V, T = cfg.n_layer, cfg.d_model, cfg.vocab, cfg.seq_len
    return 6.0 * (12 * L * d * d + V * d) + 6.0 * L * d * T


def flops_per_step(cfg) -> float:
    return flops_per_token(cfg) * cfg.batch * cfg.seq_len


# bf16 dense MFMA peak of one MI355X: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz
PEAK_BF16_FLOPS = 256 * 4096 * 2.4e9
PEAK_HBM_BYTES = 8.0e12
