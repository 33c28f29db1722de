"""Seeded synthetic inputs for the STCA forward workloads.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``target_cross_attention_amd``).  It only draws random numbers and lays them
out; it holds none of the method's arithmetic.  Both sides therefore consume
bit-identical inputs.

Workloads (stand-ins for the internal Douyin logs the STCA papers train and
serve on; no public data set exists):

* ``tiny``      1 user, L=256, 4 targets, d=64, h=4, M=1, r=2, fp32
* ``uniform``   256 users x L=2048, 8 targets each, d=128, h=8, M=2, r=2, bf16
* ``ragged``    512 users, L ~ log-normal (median 1500, unclipped mean 2000)
                clipped to [64, 10000], targets 1+Poisson(5), d=256, h=8, M=3,
                r=4, bf16
* ``dense10k``  1024 users x L=10000, 16 targets each, d=256, h=8, M=3, r=4,
                bf16, ~10% of history tokens are copies of a token at most 3
                positions earlier (same-ID repeats)
* ``stress20k`` 256 users x L=20000, 32 targets each, d=512, h=16, M=4, r=4,
                bf16

Random streams (numpy PCG64 through ``SeedSequence(seed, spawn_key=...)``):

* ``(0,)``   layout: per-user history lengths, then per-user target counts
* ``(1, u)`` history of user ``u`` (and its duplicate pattern)
* ``(2,)``   target embeddings x_t for all targets, in user order
* ``(3,)``   weights, layer-major
* ``(4,)``   prediction-token weights (W_Z and its SwiGLU FFN)
* ``(5,)``   stochastic-length draws (Beta variates, truncation order)

Values are drawn in float32.  For bf16 workloads every drawn value is rounded
to the nearest bf16 (ties to even) and kept as a float32 array holding
bf16-representable values; ``bf16_bits`` gives the raw 16-bit patterns to
upload.  X and x_t ~ N(0, 1); every weight matrix ~ N(0, 1/fan_in) where
fan_in is its number of rows; LayerNorm gamma = 1, beta = 0 unless
``random_ln`` is asked for.
"""
from .configs import CONFIGS, Config, get_config, scaled
from .generate import (
    Inputs,
    PredictWeights,
    Weights,
    batch_layout,
    bf16_bits,
    bf16_round,
    bits_to_f32,
    make_inputs,
    make_predict_weights,
    make_sl_draws,
    make_weights,
    offsets,
    user_history,
    targets,
)

__all__ = [
    "CONFIGS", "Config", "get_config", "scaled", "Inputs", "PredictWeights", "Weights",
    "batch_layout", "bf16_bits", "bf16_round", "bits_to_f32", "make_inputs",
    "make_predict_weights", "make_sl_draws", "make_weights", "offsets", "user_history", "targets",
]
