"""CPU oracle (test infrastructure only; see lce_oracle's header)."""
from .lce_oracle import (IGNORE_INDEX, apply_softcap, backward, bad_mask,  # noqa: F401
                         dW_vocab_rows, dX_rows, forward, logit_gradient, logits,
                         backward_rows, logsumexp_by_vocab_tiles, mean_loss_value,
                         row_logsumexp, softcap_derivative, valid_mask)
