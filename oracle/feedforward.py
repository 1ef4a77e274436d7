"""CPU fp64 oracle for the blockwise feedforward of the Blockwise Transformer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the library
in ``long_context_exact_ra_amd`` never does, and this module imports nothing
from it.

Sources (cited by page title and section):

* "Ring Attention with Blockwise Transformers for Near-Infinite Context",
  section 三 "核心公式": the position-wise feedforward network
  FFN(x) = max(0, x W1 + b1) W2 + b2.
* "Blockwise Feedforward网络详解 ... RingAttention如何实现内存高效的前向传播",
  sections "核心技术原理" and "技术实现细节": the sequence is cut into
  fixed-size chunks ((batch, seq, hidden) -> (batch, num_chunks, chunk,
  hidden)), the feedforward runs on one chunk at a time in order (a scan
  over the chunks), and the chunk outputs are put back in sequence order,
  so only one chunk's intermediate activations exist at a time.

Readings where the pages are silent (also listed in the design notes):
the chunk size must divide the sequence length (the reshape requires it);
the hidden width of the feedforward is a parameter of the weights.

Everything is float64; inputs are upcast exactly.  Matrix products are
library primitives used as single steps.
"""

from __future__ import annotations

import numpy as np

__all__ = ["ffn", "blockwise_ffn"]


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _relu(z: np.ndarray) -> np.ndarray:
    """max(0, z) of the feedforward equation."""
    return np.maximum(z, 0.0)


def ffn(x, w1, b1, w2, b2) -> np.ndarray:
    """FFN(x) = max(0, x W1 + b1) W2 + b2 on the last axis of x.

    x [..., hidden]; w1 [hidden, ffn]; b1 [ffn]; w2 [ffn, hidden]; b2 [hidden].
    """
    x, w1, b1, w2, b2 = (_as_f64(t) for t in (x, w1, b1, w2, b2))
    return _relu(x @ w1 + b1) @ w2 + b2


def blockwise_ffn(x, w1, b1, w2, b2, chunk_size: int) -> np.ndarray:
    """The feedforward applied one sequence chunk at a time.

    x [batch, seq, hidden] is viewed as [batch, seq / chunk, chunk, hidden];
    the chunks are processed in order and their outputs written back to
    their places in the sequence.
    """
    x = _as_f64(x)
    B, L, H = x.shape
    if chunk_size <= 0 or L % chunk_size:
        raise ValueError("chunk_size must divide the sequence length")
    xc = x.reshape(B, L // chunk_size, chunk_size, H)
    out = np.empty_like(xc)
    for c in range(L // chunk_size):
        out[:, c] = ffn(xc[:, c], w1, b1, w2, b2)
    return out.reshape(B, L, H)
