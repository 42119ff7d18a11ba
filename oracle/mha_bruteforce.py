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


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (8 significant bits,
    ties to even), in one step from the float64 value: x = m 2^e with
    m in [0.5, 1) has quantum 2^(e-8), and below the smallest normal
    (2^-126) the quantum stays 2^-133.  Magnitudes beyond the bf16 range
    are not expected here and are left to the arithmetic."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.where(x == 0, x, np.ldexp(np.rint(np.ldexp(x, -q)), q))


def mha_decode(q_nope_heads, q_pe, latents, ropes, w_uk, w_uv, scale, visible, expanded="f64"):
    """Un-absorbed decode.

    q_nope_heads [H,128], q_pe [H,64]: one query token's heads.
    latents [L,512], ropes [L,64]: the sequence's cached tokens, in order.
    w_uk, w_uv [H,128,512].  visible: list of token positions attended.
    expanded: "f64" keeps the up-projected keys and values exact; "bf16"
    rounds them to bfloat16, as a route that materialises them as the
    model's activations does (the pages leave that type open; bf16 is the
    model's activation type).
    Returns (o [H,128], lse [H]).
    """
    if expanded not in ("f64", "bf16"):
        raise ValueError("expanded must be f64 or bf16")
    rnd = round_bf16 if expanded == "bf16" else (lambda a: a)
    H = q_nope_heads.shape[0]
    o = np.zeros((H, V_HEAD))
    lse = np.full((H,), -np.inf)
    if len(visible) == 0:
        return o, lse
    c = latents[visible]                       # [n, 512]
    r = ropes[visible]                         # [n, 64]
    for h in range(H):
        k_nope = rnd(c @ w_uk[h].T)            # [n, 128]
        keys = np.concatenate([k_nope, r], axis=1)           # [n, 192]
        vals = rnd(c @ w_uv[h].T)              # [n, 128]
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


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) to float64: the bf16 value is the float32
    whose top 16 bits they are."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def mha_paged(q_nope, q_pe, kv_cache, block_table, seq_lens, w_uk, w_uv, scale, rows=None, expanded="f64"):
    """Un-absorbed attention of every (b, t, h) over a paged latent cache
    (fp64), causal as the decode calls are: query t of a q_len-T call sees
    positions 0 .. L_b - T + t.  q_nope [B,T,H,128], q_pe [B,T,H,64],
    kv_cache [NB,P,576] and w_uk / w_uv [H,128,512] as float64;
    block_table [B,MB], seq_lens [B].  Returns (out [n,128], lse [n]) for the
    flattened rows (b*T + t)*H + h, all when rows is None.  ``expanded`` as
    in mha_decode."""
    B, T, H, _ = q_nope.shape
    P = kv_cache.shape[1]
    want = None if rows is None else set(int(r) for r in rows)
    outs, lses = {}, {}
    for b in range(B):
        L = int(seq_lens[b])
        if L > 0:
            pages = [int(block_table[b, i]) for i in range((L + P - 1) // P)]
            toks = np.concatenate([kv_cache[pg] for pg in pages], axis=0)[:L]
        else:
            toks = np.zeros((0, kv_cache.shape[2]))
        for t in range(T):
            keep = [h for h in range(H) if want is None or ((b * T + t) * H + h) in want]
            if not keep:
                continue
            n = max(0, L - T + t + 1)
            o, lse = mha_decode(q_nope[b, t][keep], q_pe[b, t][keep], toks[:, :512], toks[:, 512:], w_uk[keep],
                                w_uv[keep], scale, list(range(n)), expanded)
            for k, h in enumerate(keep):
                outs[(b * T + t) * H + h] = o[k]
                lses[(b * T + t) * H + h] = lse[k]
    order = sorted(outs) if rows is None else [int(r) for r in rows]
    return np.stack([outs[r] for r in order]), np.array([lses[r] for r in order])
