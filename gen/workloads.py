"""Workload recipes: shapes and value distributions of the five parity /
benchmark configurations of the MXFP4 routed-expert path.

C1  one MXFP4 GEMV, W 256x1024, x fp32 N(0,1)
C2  one routed SwiGLU expert, hidden 7168, inter 1536, x bf16 N(0,1)
C3  one decode token through a 896-expert layer, top-16, bf16 router N(0,0.02)
C4  64 decode tokens, Zipf(s=1.1)-skewed router logits, top-16
C5  2048 prefill tokens, uniform router logits, top-16

Codes are uniform over the 16 E2M1 codes; exponent bytes uniform in
[120, 134] (one per 32 along K). Every tensor is drawn from its own
counter-based stream keyed by (seed, config, kind, a, b), so any expert or
token can be regenerated alone.
"""
from . import (KIND_BIAS, KIND_LOGITS, KIND_ROUTER, KIND_SHARED, KIND_TOKENS, expert, key,
               mxfp4_matrix, normal_bf16, normal_f32, uniform_f32, zipf_logits)

HIDDEN, INTER, N_EXPERTS, TOPK = 7168, 1536, 896, 16
ELO, EHI = 120, 134
# Supplementary exponent range that puts SwiGLU's gate in its curved region.
ELO_CURVED, EHI_CURVED = 114, 120

C1, C2, C3, C4, C5 = 1, 2, 3, 4, 5


def c1_inputs(seed=0, rows=256, cols=1024, elo=ELO, ehi=EHI):
    nib, sc = mxfp4_matrix(seed, C1, rows, cols, elo, ehi)
    x = normal_f32(key(seed, C1, KIND_TOKENS, 0, 0), cols)
    return nib, sc, x


def expert_weights(seed, cfg, e, hidden=HIDDEN, inter=INTER, elo=ELO, ehi=EHI):
    return expert(seed, cfg, e, hidden, inter, elo, ehi)


def tokens_bf16(seed, cfg, T, hidden=HIDDEN, batch=0):
    """T activation rows bf16 N(0,1); `batch` selects a fresh batch."""
    return normal_bf16(key(seed, cfg, KIND_TOKENS, batch, 0), T * hidden).reshape(T, hidden)


def router_bf16(seed, cfg=C3, n_experts=N_EXPERTS, hidden=HIDDEN):
    return normal_bf16(key(seed, cfg, KIND_ROUTER, 0, 0), n_experts * hidden,
                       0.0, 0.02).reshape(n_experts, hidden)


def zipf_router_logits(seed, T, n_experts=N_EXPERTS, s=1.1, cfg=C4, batch=0):
    return zipf_logits(seed, cfg, T, n_experts, s, batch)


def uniform_router_logits(seed, T, n_experts=N_EXPERTS, cfg=C5, batch=0):
    return uniform_f32(key(seed, cfg, KIND_LOGITS, batch, 0), T * n_experts).reshape(T, n_experts)


N_SHARED = 2
SHARED_SIGMA = 0.02


def shared_experts_bf16(seed, cfg=C3, n_shared=N_SHARED, hidden=HIDDEN, inter=INTER,
                        sigma=SHARED_SIGMA):
    """n_shared shared experts: dicts gate/up [inter][hidden], down
    [hidden][inter], bf16 N(0, sigma) (the router's distribution)."""
    out = []
    for s in range(n_shared):
        def m(i, rows, cols):
            return normal_bf16(key(seed, cfg, KIND_SHARED, s, i), rows * cols, 0.0,
                               sigma).reshape(rows, cols)
        out.append({"gate": m(0, inter, hidden), "up": m(1, inter, hidden),
                    "down": m(2, hidden, inter)})
    return out


def routing_bias(seed, n_experts=N_EXPERTS, scale=0.1, cfg=C3):
    return normal_f32(key(seed, cfg, KIND_BIAS, 0, 0), n_experts, 0.0, scale)
