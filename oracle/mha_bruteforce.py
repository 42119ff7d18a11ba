"""Brute-force un-absorbed multi-head attention for tiny MLA shapes (numpy fp64).

TEST INFRASTRUCTURE ONLY.  It pins the absorbed oracle against the model it
stands for.  The pages fix the DeepSeek-R1 MLA head dims as 128 no-rope +
64 rope for keys and 128 for values (vLLM PR #41778 digest, "Risks and
impact" item 4); the 512-wide latent plus 64-wide rope per cached token is
what the split-KV partial width kv_lora_rank + 1 counts (vLLM PR #46819
digest, "Key code excerpt").  Each head h owns up-projections
W_UK[h], W_UV[h] in R^{128 x 512}; for cached latent c_j and rope r_j:

    k_{h,j} = [ W_UK[h] c_j ; r_j ]      (192 wide)
    v_{h,j} =   W_UV[h] c_j              (128 wide)

and a query head is q_h = [ q_nope_h (128) ; q_pe_h (64) ].  Plain attention
over the same visible list gives o_h = sum_j softmax_j(scale * q_h . k_{h,j}) v_{h,j}.
Absorbing W_UK into the query (q_abs = W_UK[h]^T q_nope_h) turns this into
attention against the shared latent; W_UV[h] applied to the latent-space
output must give o_h back, with the same log-sum-exp.
"""
from __future__ import annotations

import numpy as np

QK_NOPE, QK_ROPE, V_HEAD = 128, 64, 128


def mha_decode(q_nope_heads, q_pe, latents, ropes, w_uk, w_uv, scale, visible):
    """Un-absorbed decode.

    q_nope_heads [H,128], q_pe [H,64]: one query token's heads.
    latents [L,512], ropes [L,64]: the sequence's cached tokens, in order.
    w_uk, w_uv [H,128,512].  visible: list of token positions attended.
    Returns (o [H,128], lse [H]).
    """
    H = q_nope_heads.shape[0]
    o = np.zeros((H, V_HEAD))
    lse = np.full((H,), -np.inf)
    if len(visible) == 0:
        return o, lse
    c = latents[visible]                       # [n, 512]
    r = ropes[visible]                         # [n, 64]
    for h in range(H):
        k_nope = c @ w_uk[h].T                 # [n, 128]
        keys = np.concatenate([k_nope, r], axis=1)           # [n, 192]
        vals = c @ w_uv[h].T                   # [n, 128]
        q = np.concatenate([q_nope_heads[h], q_pe[h]])       # [192]
        s = scale * (keys @ q)
        m = s.max()
        p = np.exp(s - m)
        o[h] = (p @ vals) / p.sum()
        lse[h] = m + np.log(p.sum())
    return o, lse


def absorb_query(q_nope_heads, w_uk):
    """q_abs[h] = W_UK[h]^T q_nope_h  ->  [H, 512]."""
    return np.einsum("hdk,hd->hk", w_uk, q_nope_heads)


def project_output(out_latent, w_uv):
    """o[h] = W_UV[h] out_latent[h]  ->  [H, 128]."""
    return np.einsum("hdk,hk->hd", w_uv, out_latent)
