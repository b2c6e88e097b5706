"""Seeded synthetic inputs for the MXFP8 MoE expert path.

Shared by the tests, the benchmark and the oracle checks.  This module only
draws random inputs; it performs none of the method's arithmetic (no
quantization, no scale rule, no permutation).  Generators:
``numpy.random.Generator(PCG64(SeedSequence([cfg, tag, chunk])))``, so any
tensor (or one expert's slice of it) can be regenerated on its own.

bf16 tensors are returned as uint16 bit patterns, drawn in fp32 and rounded
to bf16 by round-to-nearest-even.  Outliers are elements multiplied by 1000
(in fp32, then rounded to bf16).

Workloads (the MoE expert computation of the MXFP8 MoE training digest and
pytorch/ao PR #3203; shapes echo that PR's (n, 8192, 5120) benchmark
inputs):

1. tiny forward   E=4,  K=256,  N=512,  T=2048, group sizes 32*Multinomial(64, 1/4)
2. mid fwd+bwd    E=8,  K=2048, N=1408, T=16384, Zipf(1.2) group sizes, not
                  multiples of 32
3. large fwd+bwd  T=8192 tokens, top-2 of E=16, K=5120, N=8192, one expert
                  forced empty, 0.1% outliers x1000 in X, W and dY
4. quantize bandwidth  [16*8192, 5120], 1% all-zero 32x32 tiles, 1%
                  subnormal 32x32 tiles, 0.1% outliers x1000
5. SwiGLU expert FFN layer  T=32768 tokens, top-8 of E=64, hidden 7168,
                  expert ffn 2048 (``layer_inputs``: drawn on the GPU)
"""

import numpy as np

BLOCK = 32
TAGS = {"x": 1, "w": 2, "dy": 3, "logits": 4, "sizes": 5, "tiles": 6, "outl": 7, "perm": 8, "gate": 9}


def rng(cfg, tag, chunk=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(cfg), TAGS[tag], int(chunk)])))


def f32_to_bf16_bits(x):
    """Round fp32 samples to bf16 bit patterns (nearest, ties to even).  The
    samples are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g, shape, std=1.0, outlier_p=0.0, outlier_g=None):
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    b = f32_to_bf16_bits(x)
    if outlier_p:
        og = outlier_g if outlier_g is not None else g
        m = og.random(shape, dtype=np.float32) < outlier_p
        b[m] = f32_to_bf16_bits(bf16_bits_to_f32(b[m]) * np.float32(1000.0))
    return b


def capacity(T, topk, E):
    """Rows of a padded permuted buffer: the worst case T*topk + 31*E rounded
    up to a multiple of 32 (columnwise blocks run along these rows)."""
    n = T * topk + (BLOCK - 1) * E
    return -(-n // BLOCK) * BLOCK


def ids_from_sizes(sizes):
    """expert_ids [T, 1] of tokens that arrive already sorted by expert."""
    return np.repeat(np.arange(len(sizes)), sizes).astype(np.int32)[:, None]


def topk_route(logits, topk):
    """Top-k experts per token (ties to the lower expert id) and softmax
    weights renormalised over the k chosen logits."""
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    w = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def zipf_sizes(cfg, T, E, s=1.2):
    g = rng(cfg, "sizes")
    p = np.arange(1, E + 1, dtype=np.float64) ** -s
    p /= p.sum()
    m = g.multinomial(T, p)
    m = m[g.permutation(E)]
    while np.any(m % BLOCK == 0):
        e = int(np.nonzero(m % BLOCK == 0)[0][0])
        big = int(np.argmax(m))
        m[big] -= 1
        m[e] += 1
    return m.astype(np.int64)


def moe_case(cfg, T, K, N, E, topk=1, sizes=None, x_std=1.0, w_std=0.02, dy_std=1.0,
             outlier_p=0.0, empty_experts=(), with_dy=True, w_outliers=None):
    """A MoE expert-GEMM workload.

    Routing is either given group sizes (tokens sorted by expert, topk=1) or
    top-``topk`` of seeded N(0,1) router logits with ``empty_experts`` forced
    to -inf.  Returns a dict with bf16 bit tensors x [T,K], w [E,N,K] and
    dy_full [T*topk + 31E, N] (rows of the padded permuted layout; the caller
    zeroes the pad rows), int32 expert_ids [T, topk] and fp32 weights.
    """
    out = {"cfg": cfg, "T": T, "K": K, "N": N, "E": E, "topk": topk}
    if sizes is not None:
        sizes = np.asarray(sizes, dtype=np.int64)
        assert sizes.sum() == T and topk == 1
        out["expert_ids"] = ids_from_sizes(sizes)
        out["weights"] = np.ones((T, 1), np.float32)
    else:
        lg = rng(cfg, "logits").standard_normal((T, E), dtype=np.float32)
        for e in empty_experts:
            lg[:, e] = -np.inf
        ids, wts = topk_route(lg, topk)
        out["logits"] = lg
        out["expert_ids"] = ids
        out["weights"] = wts
    out["x"] = normal_bf16(rng(cfg, "x"), (T, K), x_std, outlier_p)
    wo = outlier_p if w_outliers is None else w_outliers
    out["w"] = np.stack([normal_bf16(rng(cfg, "w", e), (N, K), w_std, wo) for e in range(E)])
    cap = capacity(T, topk, E)
    out["capacity"] = cap
    if with_dy:
        out["dy_full"] = normal_bf16(rng(cfg, "dy"), (cap, N), dy_std, outlier_p)
    return out


def config(n, with_dy=True):
    """Workload n (1-4) at its full size."""
    if n == 1:
        g = rng(1, "sizes")
        sizes = BLOCK * g.multinomial(64, [0.25] * 4)
        return moe_case(1, 2048, 256, 512, 4, 1, sizes=sizes, with_dy=False)
    if n == 2:
        return moe_case(2, 16384, 2048, 1408, 8, 1, sizes=zipf_sizes(2, 16384, 8), with_dy=with_dy)
    if n == 3:
        empty = [int(rng(3, "gate").integers(0, 16))]
        return moe_case(3, 8192, 5120, 8192, 16, 2, x_std=1.0, w_std=1.0, outlier_p=0.001,
                        empty_experts=empty, with_dy=with_dy)
    raise ValueError(n)


def quant_tensor(cfg, rows, cols, zero_p=0.01, sub_p=0.01, outlier_p=0.001, chunk=0):
    """Workload-4 style bf16 tensor [rows, cols]: N(0,1) values; in the grid of
    aligned 32x32 tiles a seeded fraction ``zero_p`` is all zero and a
    disjoint fraction ``sub_p`` holds bf16 subnormals (exponent field 0,
    random sign, random nonzero 7-bit mantissa); outliers x1000 elsewhere."""
    g = rng(cfg, "x", chunk)
    x = normal_bf16(g, (rows, cols))
    tg = rng(cfg, "tiles", chunk)
    tr, tc = rows // BLOCK, cols // BLOCK
    u = tg.random((tr, tc))
    zero = u < zero_p
    sub = (u >= zero_p) & (u < zero_p + sub_p)
    og = rng(cfg, "outl", chunk)
    om = og.random((rows, cols), dtype=np.float32) < outlier_p
    tile_any = np.repeat(np.repeat(zero | sub, BLOCK, 0), BLOCK, 1)
    om &= ~tile_any
    x[om] = f32_to_bf16_bits(bf16_bits_to_f32(x[om]) * np.float32(1000.0))
    xv = x.reshape(tr, BLOCK, tc, BLOCK)
    zt = np.repeat(np.repeat(zero, BLOCK, 0), BLOCK, 1).reshape(tr, BLOCK, tc, BLOCK)
    xv[zt] = 0
    st = np.repeat(np.repeat(sub, BLOCK, 0), BLOCK, 1).reshape(tr, BLOCK, tc, BLOCK)
    nsub = int(st.sum())
    mant = tg.integers(1, 128, nsub).astype(np.uint16)
    sign = (tg.integers(0, 2, nsub).astype(np.uint16) << 15)
    xv[st] = mant | sign
    return x




def layer_inputs(device="cuda:0", seed=5, T=32768, H=7168, F=2048, E=64, topk=8):
    """SwiGLU layer inputs (T=32768 tokens, hidden 7168, ffn 2048, top-8 of 64
    experts by default) drawn on the GPU with a seeded torch generator (the
    weights alone are 5.6 G elements): router logits fp32 N(0,1) [T, E]; X
    and dOut bf16 N(0,1) [T, H]; W1 [E, 2F, H] (gate rows then up rows) and
    W2 [E, H, F] bf16 0.02 * N(0,1).  Samples are fp32, scaled, then rounded
    to bf16 (RNE, torch's conversion)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal_bf16_gpu(shape, std):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1)
        ch = 1 << 26               # chunked: keeps the fp32 temporary small
        for i in range(0, flat.numel(), ch):
            n = min(ch, flat.numel() - i)
            flat[i:i + n] = (torch.randn(n, generator=g, device=device) * std).to(torch.bfloat16)
        return out

    logits = torch.randn((T, E), generator=g, device=device)
    return {
        "T": T, "H": H, "F": F, "E": E, "topk": topk,
        "logits": logits,
        "x": normal_bf16_gpu((T, H), 1.0),
        "dout": normal_bf16_gpu((T, H), 1.0),
        "w1": normal_bf16_gpu((E, 2 * F, H), 0.02),
        "w2": normal_bf16_gpu((E, H, F), 0.02),
    }
