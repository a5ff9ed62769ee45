"""Jagged (variable-length) multi-head attention for AMD Instinct MI355X.

Forward and backward of softmax attention and of GDPA (silu(scale*q.k)/L_kv)
over packed sequences addressed by offsets, with no padding, computed by the
hand-written gfx950 HIP kernels of libjfa.so (C ABI in include/jfa.h).

  from jagged_attention_ads_amd import jfa
  out, lse = jfa.forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, causal=True)
  dq, dk, dv = jfa.backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, causal=True)
"""

__all__ = ["jfa", "workloads"]
