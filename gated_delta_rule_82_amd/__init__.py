"""MI355X-native KDA decode: the HIP library libkda and its thin binding.

    from gated_delta_rule_82_amd import kda      # ctypes binding (needs torch)
    kda.decode(out, q, k, v, raw_gate, beta_logits, a_log, dt_bias,
               cu_seqlens, state_pool, state_indices, gate_mode="softplus")

``workloads`` draws the seeded synthetic inputs; ``build`` compiles the
library for gfx950.
"""
__all__ = ["kda", "workloads", "build"]
