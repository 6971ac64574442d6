"""Seeded synthetic inputs for the hybrid compressed attention workloads.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no pooling, no RoPE, no quantisation, no scoring).
Both the CPU oracle and the GPU library are fed from it.

Distributions follow the workload statements: hidden states and projected
tensors N(0, 1); projection weights N(0, 1/hidden); learned positional biases
N(0, 0.1); sink logits 0; indexer head weights N(0, 1/H_I). N(0, v) names the
variance v. Projected tensors of the large workloads are drawn directly as
N(0, 1), which is their distribution when hidden ~ N(0,1) and W ~ N(0,1/d);
only the tiny workload forms the host projections literally.

bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even from
float32), everything else as numpy float32 / int32.
"""
import numpy as np

__all__ = ["rng", "normal", "to_bf16", "bf16_to_f32", "WORKLOADS", "make"]


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(g, shape, var=1.0):
    """float32 draws from N(0, var)."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


def to_bf16(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs).

    Large arrays use torch's CPU cast (also round-to-nearest-even) for speed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size > (1 << 22):
        try:
            import torch
            return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        except ImportError:
            pass
    u = x.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_normal(g, shape, var=1.0):
    return to_bf16(normal(g, shape, var))


# --------------------------------------------------------------- workloads
# Each recipe returns a dict of numpy arrays plus scalar parameters. Seeds
# are fixed per workload; keyword overrides of the size arguments (B, S, ctx)
# shrink a workload for fast parity cases and keep everything else.

WORKLOADS = {
    "tiny_csa_prefill": dict(seed=1),
    "hca_prefill_16k": dict(seed=2),
    "csa_decode_128k": dict(seed=3),
    "csa_prefill_64k": dict(seed=4),
    "decode_1m_pair": dict(seed=5),
}


def tiny_csa_prefill(seed=1, S=256, hidden=256):
    """Batch 1, seq 256, hidden 256; one KV head dim 64 (last 32 RoPE), 4
    query heads dim 64; m=4; indexer 2 heads dim 32 in fp32; top-k 8;
    window 32; one sink logit 0 per head. Host projections in float64,
    rounded to float32."""
    g = rng(seed)
    h = normal(g, (S, hidden)).astype(np.float64)

    def proj(cols):
        W = normal(g, (hidden, cols), 1.0 / hidden).astype(np.float64)
        return (h @ W).astype(np.float32)

    H, D, HI, dI, m = 4, 64, 2, 32, 4
    d = dict(
        B=1, S=S, H=H, D=D, dv=D, d_rope=32, rope_base=10000.0, m=m, HI=HI, dI=dI, k=8, W=32,
        scale=float(np.float32(1.0 / np.sqrt(D))), dtype="f32",
    )
    d["q"] = proj(H * D).reshape(1, S, H, D)
    d["ca"], d["za"], d["cb"], d["zb"] = (proj(D).reshape(1, S, D) for _ in range(4))
    d["kv_w"] = proj(D).reshape(1, S, D)
    d["qI"] = proj(HI * dI).reshape(1, S, HI, dI)
    d["w"] = proj(HI).reshape(1, S, HI)
    d["ia"], d["iza"], d["ib"], d["izb"] = (proj(dI).reshape(1, S, dI) for _ in range(4))
    d["bias_a"], d["bias_b"] = normal(g, (m, D), 0.1), normal(g, (m, D), 0.1)
    d["ibias_a"], d["ibias_b"] = normal(g, (m, dI), 0.1), normal(g, (m, dI), 0.1)
    d["sink"] = np.zeros(H, np.float32)
    d["q_pos"] = np.arange(S, dtype=np.int32).reshape(1, S)
    d["w_pos0"] = np.zeros(1, np.int32)
    return d


def hca_prefill_16k(seed=2, S=16384):
    """Batch 1, seq 16384, m'=128 (128 entries); 16 query heads dim 128 over
    one shared KV head dim 128 (last 64 RoPE, base 10000); window 128; sink
    0; bf16 inputs."""
    g = rng(seed)
    H, D, m = 16, 128, 128
    d = dict(B=1, S=S, H=H, D=D, dv=D, d_rope=64, rope_base=10000.0, m=m, W=128,
             scale=float(np.float32(1.0 / np.sqrt(D))), dtype="bf16")
    d["q"] = _bf16_normal(g, (1, S, H, D))
    d["c"] = _bf16_normal(g, (1, S, D))
    d["z"] = _bf16_normal(g, (1, S, D))
    d["kv_w"] = _bf16_normal(g, (1, S, D))
    d["bias"] = normal(g, (m, D), 0.1)
    d["sink"] = np.zeros(H, np.float32)
    d["q_pos"] = np.arange(S, dtype=np.int32).reshape(1, S)
    d["w_pos0"] = np.zeros(1, np.int32)
    return d


def _decode_common(g, B, ctx, H, D, HI, dI, m, W):
    N = ctx // m
    d = {}
    d["kv_c"] = _bf16_normal(g, (B, N, D))
    d["kv_w"] = _bf16_normal(g, (B, W, D))
    d["q"] = _bf16_normal(g, (B, 1, H, D))
    d["kI"] = normal(g, (B, N, dI))          # quantised to MXFP4 by the method
    d["qI"] = normal(g, (B, 1, HI, dI))      # quantised to MXFP4 by the method
    d["w"] = normal(g, (B, 1, HI), 1.0 / HI)
    d["q_pos"] = np.full((B, 1), ctx - 1, np.int32)
    d["w_pos0"] = np.full(B, ctx - W, np.int32)
    d["n_entries"] = np.full(B, N, np.int32)
    d["sink"] = np.zeros(H, np.float32)
    return d


def csa_decode_128k(seed=3, B=32, ctx=131072):
    """Batch 32, context 131072 -> 32768 CSA entries; KV dim 512 + 64 RoPE;
    64 query heads; indexer 64 heads dim 128 on MXFP4; top-k 2048; window
    128; sink; KV cache and queries N(0,1). The cache content stands for
    already-rotated entries."""
    g = rng(seed)
    d = dict(B=B, ctx=ctx, H=64, D=576, dv=512, d_rope=64, rope_base=10000.0, m=4, HI=64, dI=128,
             k=2048, W=128, scale=float(np.float32(1.0 / np.sqrt(576))), dtype="bf16")
    d.update(_decode_common(g, B, ctx, 64, 576, 64, 128, 4, 128))
    return d


def csa_prefill_64k(seed=4, S=65536):
    """Batch 1, seq 65536 -> 16384 entries; 64 query heads; KV dim 512 + 64
    RoPE; indexer 64 heads dim 128 on MXFP4, top-k 2048 causal; window 128.
    Projected tensors drawn directly as N(0,1) bf16."""
    g = rng(seed)
    H, D, HI, dI, m = 64, 576, 64, 128, 4
    d = dict(B=1, S=S, H=H, D=D, dv=512, d_rope=64, rope_base=10000.0, m=m, HI=HI, dI=dI, k=2048,
             W=128, scale=float(np.float32(1.0 / np.sqrt(D))), dtype="bf16")
    d["ca"], d["za"], d["cb"], d["zb"] = (_bf16_normal(g, (1, S, D)) for _ in range(4))
    d["ia"], d["iza"], d["ib"], d["izb"] = (_bf16_normal(g, (1, S, dI)) for _ in range(4))
    d["bias_a"], d["bias_b"] = normal(g, (m, D), 0.1), normal(g, (m, D), 0.1)
    d["ibias_a"], d["ibias_b"] = normal(g, (m, dI), 0.1), normal(g, (m, dI), 0.1)
    d["q"] = _bf16_normal(g, (1, S, H, D))
    d["qI"] = normal(g, (1, S, HI, dI))
    d["w"] = normal(g, (1, S, HI), 1.0 / HI)
    d["kv_w"] = _bf16_normal(g, (1, S, D))
    d["sink"] = np.zeros(H, np.float32)
    d["q_pos"] = np.arange(S, dtype=np.int32).reshape(1, S)
    d["w_pos0"] = np.zeros(1, np.int32)
    return d


def decode_1m_pair(seed=5, B=4, ctx=1048576):
    """Interleaved CSA + HCA layer pair at context 1048576, batch 4. CSA:
    262144 entries (KV 512+64, MXFP4 indexer 64x128, top-k 2048); HCA: 8192
    entries, dense; 64 query heads per layer; window 128 and sink on both.
    Also the newest source tokens that complete one CSA entry (8 tokens,
    two series) and one HCA entry (128 tokens), with their biases."""
    g = rng(seed)
    H, D, HI, dI = 64, 576, 64, 128
    d = dict(B=B, ctx=ctx, H=H, D=D, dv=512, d_rope=64, rope_base=10000.0, m=4, m_h=128, HI=HI, dI=dI,
             k=2048, W=128, scale=float(np.float32(1.0 / np.sqrt(D))), dtype="bf16")
    d.update(_decode_common(g, B, ctx, H, D, HI, dI, 4, 128))
    Nh = ctx // 128
    d["kv_h"] = _bf16_normal(g, (B, Nh, D))
    d["q_h"] = _bf16_normal(g, (B, 1, H, D))
    d["kv_w_h"] = _bf16_normal(g, (B, 128, D))
    d["n_entries_h"] = np.full(B, Nh, np.int32)
    d["sink_h"] = np.zeros(H, np.float32)
    # newest sources: CSA entry N-1 pools tokens [ctx-8, ctx); HCA entry Nh-1 pools [ctx-128, ctx)
    d["src_ca"], d["src_za"], d["src_cb"], d["src_zb"] = (_bf16_normal(g, (B, 8, D)) for _ in range(4))
    d["src_ia"], d["src_iza"], d["src_ib"], d["src_izb"] = (_bf16_normal(g, (B, 8, dI)) for _ in range(4))
    d["src_c"], d["src_z"] = _bf16_normal(g, (B, 128, D)), _bf16_normal(g, (B, 128, D))
    d["bias_a"], d["bias_b"] = normal(g, (4, D), 0.1), normal(g, (4, D), 0.1)
    d["ibias_a"], d["ibias_b"] = normal(g, (4, dI), 0.1), normal(g, (4, dI), 0.1)
    d["bias_h"] = normal(g, (128, D), 0.1)
    return d


_RECIPES = {
    "tiny_csa_prefill": tiny_csa_prefill,
    "hca_prefill_16k": hca_prefill_16k,
    "csa_decode_128k": csa_decode_128k,
    "csa_prefill_64k": csa_prefill_64k,
    "decode_1m_pair": decode_1m_pair,
}


def make(name, **overrides):
    """Build a workload by name; keyword overrides shrink its sizes."""
    fn = _RECIPES[name]
    kw = dict(seed=WORKLOADS[name]["seed"])
    kw.update(overrides)
    return fn(**kw)


def out_proj(seed, R, H, dv, g, dg, d):
    """Grouped output projection inputs: attention outputs o [R, H*dv] bf16
    N(0,1) (heads consecutive), group weights w1 [g, dg, (H/g)*dv] bf16
    N(0, 1/((H/g)*dv)), hidden weights w2 [d, g*dg] bf16 N(0, 1/(g*dg))
    (projection weights N(0, 1/fan_in), so every output is about N(0,1))."""
    gen = rng(seed)
    K1 = H // g * dv
    return dict(o=_bf16_normal(gen, (R, H * dv)), w1=_bf16_normal(gen, (g, dg, K1), 1.0 / K1),
                w2=_bf16_normal(gen, (d, g * dg), 1.0 / (g * dg)), R=R, H=H, dv=dv, g=g, dg=dg, d=d)


def projection(seed, B, S, hidden, D, csa, m):
    """Projection-then-compression inputs: hidden states x [B,S,hidden] bf16
    N(0,1); series weights w [4 or 2, D, hidden] bf16 N(0, 1/hidden)
    (CSA: W_ca, W_za, W_cb, W_zb; HCA: W_c, W_z); positional biases
    [m, D] N(0, 0.1); RMSNorm scale gamma [D] N(1, 0.01)."""
    gen = rng(seed)
    ns = 4 if csa else 2
    d = dict(x=_bf16_normal(gen, (B, S, hidden)), w=_bf16_normal(gen, (ns, D, hidden), 1.0 / hidden),
             bias_a=normal(gen, (m, D), 0.1), bias_b=normal(gen, (m, D), 0.1))
    d["gamma"] = (1.0 + normal(gen, (D,), 0.01)).astype(np.float32)
    return d
