"""MI355X (gfx950) DFlash 2 path selector.

The compute path is the HIP library libdflash2.so (C ABI: include/dflash2.h);
`binding` marshals torch tensors into it.  `synth` draws seeded synthetic
inputs.  Importing the package does not load the library: the first call
does, and raises if it has not been built.
"""
from .binding import (PreparedSelect, SelectorError, conv2, device_error, lmhead_topk, load,
                      pair_scores, philox_uniforms, philox_uniforms_next, plan,
                      plan_override, project, release, sample_walk, select, select_sample, topk, version,
                      viterbi, walk)

__all__ = ["PreparedSelect", "SelectorError", "conv2", "device_error", "lmhead_topk", "load",
           "pair_scores", "philox_uniforms", "philox_uniforms_next", "plan",
           "plan_override", "project", "release", "sample_walk", "select", "select_sample", "topk", "version",
           "viterbi", "walk"]
