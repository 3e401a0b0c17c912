"""Joint vector quantization across loop steps and decode over it (LoopVQ-style).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Float64 after the
stored fp16 codewords and bf16 inputs, which are exact in float64.

Source
------
"LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers",
abstract (概要, mlinfo page; also on the fugumt page): keys and values
change little from one loop step to the next, so one codebook entry can
stand for a group of channels of all loop steps at once; the paper tunes
its codebooks and stores half a bit per element.

Readings where the pages are silent:
* for one layer, token and head, the joint vector of channel group j is the
  concatenation over loops r = 0..R-1 of channels [4j, 4j+4) of loop r's
  key (or value): 4R numbers;
* each group j has its own codebook of 256 codewords (an 8-bit index), per
  layer, shared by the heads, separately for keys and values; with R = 4
  that is 8 bits per 16 elements = 0.5 bit per element;
* encoding picks the codeword nearest in squared Euclidean distance (ties:
  lowest index); decoding loop r reads slice [4r, 4r+4) of the codeword;
* attention of loop r is plain softmax attention over the decoded keys and
  values with that loop's own query (no tau, no planes);
* codebooks are inputs (fine-tuning needs a model and data, out of scope).

Pins (tests/test_oracle_loopvq.py): a codebook that holds every joint
vector exactly gives lossless coding; brute force over every codeword on a
tiny case; decode equals torch SDPA (float64) over the decoded tensors;
the index is invariant to scaling data and codebook together.
"""
from __future__ import annotations

import numpy as np

SUB = 4          # channels per loop in one joint vector
N_CODES = 256    # codewords per codebook (8-bit index)


def joint_vectors(x_loops):
    """x_loops float [R][T][D] (one head) -> joint vectors [T][D/4][4R]."""
    x = np.asarray(x_loops, np.float64)
    R, T, D = x.shape
    g = x.reshape(R, T, D // SUB, SUB)               # [R][T][G][4]
    return g.transpose(1, 2, 0, 3).reshape(T, D // SUB, R * SUB)


def encode(x_loops, codebook):
    """Nearest-codeword indices [T][G] (int) of one head's keys or values.

    x_loops float [R][T][D]; codebook float [G][256][4R].
    """
    jv = joint_vectors(x_loops)                      # [T][G][J]
    cb = np.asarray(codebook, np.float64)            # [G][N][J]
    T, G, J = jv.shape
    idx = np.empty((T, G), np.int64)
    for j in range(G):
        d = ((jv[:, j, None, :] - cb[j][None, :, :]) ** 2).sum(-1)   # [T][N]
        idx[:, j] = np.argmin(d, axis=1)             # first minimum = lowest index
    return idx


def distances(x_loops, codebook):
    """Squared distances [T][G][256] (for checking a chosen index)."""
    jv = joint_vectors(x_loops)
    cb = np.asarray(codebook, np.float64)
    return ((jv[:, :, None, :] - cb[None, :, :, :]) ** 2).sum(-1)


def decode_loop(idx, codebook, loop):
    """Decoded [T][D] of loop `loop` from indices [T][G]."""
    cb = np.asarray(codebook, np.float64)
    T, G = idx.shape
    out = np.empty((T, G, SUB))
    for j in range(G):
        out[:, j, :] = cb[j, idx[:, j], SUB * loop:SUB * (loop + 1)]
    return out.reshape(T, G * SUB)


def attend(q, k_hat, v_hat, sm_scale=1.0):
    """Softmax attention of one query [D] over [T][D] keys / values (float64)."""
    q = np.asarray(q, np.float64)
    if k_hat.shape[0] == 0:
        return np.zeros(q.shape[0])
    s = sm_scale * (k_hat @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ v_hat
