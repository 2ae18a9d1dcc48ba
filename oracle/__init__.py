"""fp64 CPU oracle for one training step of the d20 decoder-only Transformer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(the HIP library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product.

Parity pinning: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, invariants, special cases that reduce to textbook
routines, values the pages print, and fp64 finite differences.  The
optimiser step (``optim.py``: AdamW, Muon, the schedule) is checked by
``tests/test_oracle_optim.py`` against torch's AdamW, the singular-value
form of the Newton-Schulz iteration and closed forms of the first two Muon
steps.  Three
readings are fixed by contract rather than by the pages (RMSNorm epsilon,
the rotary pairing convention and the weight-init law); those are
"parity unpinned" as far as the pages go: both sides implement the same
stated reading, and no page value checks it.
"""
from .model import (  # noqa: F401
    rmsnorm, rmsnorm_bwd, rope_angles, rope, causal_attention,
    causal_attention_bwd, relu2, cross_entropy, cross_entropy_grad,
    block_forward, block_backward, model_forward_row, model_backward_row,
    train_step, block_step, loss_bpb, weighted_loss, sample_next, zero_grads,
)
from . import optim  # noqa: F401
