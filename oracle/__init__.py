"""fp64 CPU oracle (test infrastructure only; never used by the product path)."""
from .ttt_oracle import (Model, TTTResult, as_f64, ce_stats, chunk_loss_and_grads, clip_scale, decode_ttt,
                         forward, gelu, gelu_prime, logits, logsumexp_rows, passage_loss, run_ttt,
                         settle_step, static_losses, token_losses)

__all__ = ["Model", "TTTResult", "as_f64", "ce_stats", "chunk_loss_and_grads", "clip_scale", "decode_ttt",
           "forward", "gelu", "gelu_prime", "logits", "logsumexp_rows", "passage_loss", "run_ttt",
           "settle_step", "static_losses", "token_losses"]
