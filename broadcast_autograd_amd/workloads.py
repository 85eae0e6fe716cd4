"""Seeded synthetic inputs for the five workloads of the broadcasting path.

This module only draws numbers: it holds none of the operators' arithmetic,
so both the HIP path and the CPU oracle can be fed from it.  Every array is
drawn on the host in float32 with numpy's PCG64 (``default_rng(seed)``):

  N(mu, sigma) = standard_normal(float32) * sigma + mu   (sigma = std. dev.)
  U(lo, hi)    = random(float32) * (hi - lo) + lo

The causal mask follows the GPT chapter of the "Zero" book (section
"attention"): 0 on and below the diagonal, a large negative constant above it
(j > i).  The workloads use -1e9 as that constant.
"""
import numpy as np

# workload name -> description
WORKLOADS = {
    "xy_plus_x": "z = x*y + x, x[64,128,256], y[128,1]",
    "mlp_bias_gelu": "y = GeLU(act[4096,1024] + bias[1024])",
    "attn_scale_mask": "scores[8,16,1024,1024] * scale[1,16,1,1] + mask[1,1,1024,1024]",
    "strided_highrank": "a[4096,4096] strides [1,4096] * b[4096]; a[2..9] / b[1,3,1,5,1,7,1,9]",
    "gpt_residual": "h[16,2048,4096] * gamma[4096] + resid[16,2048,4096]",
    "gpt_loss_mean_clip": "mean of the per-token loss[64*256] and its gradient; "
                          "ClipGradNorm(1.0) over the GPT configuration's 76 gradients",
    "gpt_row_stats": "LayerNorm row mean/variance of x[64*256, 384]; softmax row max / "
                     "sum exp of causal scores[64*6*256, 256]",
}


def normal(shape, seed, mu=0.0, sigma=1.0):
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape, dtype=np.int64))
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if mu != 0.0:
        x += np.float32(mu)
    return x.reshape(shape)


def uniform(shape, seed, lo, hi):
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape, dtype=np.int64))
    x = rng.random(n, dtype=np.float32)
    x *= np.float32(hi - lo)
    x += np.float32(lo)
    return x.reshape(shape)


def causal_mask(t, neg=-1e9):
    """[1,1,t,t]: 0 where j <= i, ``neg`` where j > i."""
    m = np.zeros((t, t), dtype=np.float32)
    m[np.triu_indices(t, k=1)] = np.float32(neg)
    return m.reshape(1, 1, t, t)


def xy_plus_x(scale=1):
    """x[64,128,256], y[128,1], g[64,128,256]; ``scale`` < 1 shrinks the
    leading dim for quick checks."""
    d0 = max(1, int(64 * scale))
    return dict(x=normal((d0, 128, 256), 1001), y=normal((128, 1), 1002),
                g=normal((d0, 128, 256), 1003))


def mlp_bias_gelu(rows=4096, cols=1024):
    return dict(act=normal((rows, cols), 2001),
                bias=normal((cols,), 2002, 0.0, 0.02),
                g=normal((rows, cols), 2003))


def attn_scale_mask(b=8, h=16, t=1024):
    return dict(scores=normal((b, h, t, t), 3001),
                scale=uniform((1, h, 1, 1), 3002, 0.5, 2.0),
                mask=causal_mask(t),
                g=normal((b, h, t, t), 3003))


def attn_mask_grad(b=8, h=16, t=1024):
    """Upstream gradient of the attention scores, to be summed back to the
    causal mask's shape [1, 1, t, t] (same seed as attn_scale_mask's g)."""
    return dict(g=normal((b, h, t, t), 3003))


def strided_transposed(n=4096):
    """Storage S[n*n] U(-1,1); a = S viewed [n,n] and transposed, i.e.
    sizes [n,n], strides [1,n]; b[n] U(-1,1); g[n,n] N(0,1)."""
    return dict(a_storage=uniform((n * n,), 4001, -1.0, 1.0),
                a_sizes=(n, n), a_strides=(1, n),
                b=uniform((n,), 4002, -1.0, 1.0),
                g=normal((n, n), 4003))


def rank8(shape_a=(2, 3, 4, 5, 6, 7, 8, 9), shape_b=(1, 3, 1, 5, 1, 7, 1, 9)):
    return dict(a=uniform(shape_a, 4101, 0.5, 2.0),
                b=uniform(shape_b, 4102, 0.5, 2.0),
                g=normal(shape_a, 4103))


def gpt_residual(b=16, t=2048, c=4096):
    return dict(h=normal((b, t, c), 5001), gamma=normal((c,), 5002, 1.0, 0.1),
                resid=normal((b, t, c), 5003), g=normal((b, t, c), 5004))


def gpt_param_shapes(vocab=4096, ctx=256, c=384, blocks=6):
    """Parameter shapes of the GPT training configuration of the GPT chapter
    ("training configuration": hidden size 384, 6 blocks, sequence length
    256), in list order: token embedding [V, C] (the output layer reuses it
    transposed), position embedding [T, C]; per block LayerNorm weight and
    bias, the attention's QKV projection [C, 3C] and bias, its output
    projection [C, C] and bias, a second LayerNorm, the FFN's [C, 4C] and
    bias and [4C, C] and bias; a final LayerNorm.  The vocabulary size is
    the corpus's and is not printed; 4096 is assumed."""
    shapes = [(vocab, c), (ctx, c)]
    for _ in range(blocks):
        shapes += [(c,), (c,), (c, 3 * c), (3 * c,), (c, c), (c,),
                   (c,), (c,), (c, 4 * c), (4 * c,), (4 * c, c), (c,)]
    shapes += [(c,), (c,)]
    return shapes


def grad_arena_offsets(shapes, align=64):
    """Element offsets of each tensor in one flat gradient buffer, each
    rounded up to ``align`` elements (256 bytes), and the buffer's size."""
    offs, pos = [], 0
    for s in shapes:
        offs.append(pos)
        n = int(np.prod(s, dtype=np.int64))
        pos += (n + align - 1) // align * align
    return offs, pos


def gpt_loss_mean_clip(b=64, t=256):
    """Per-token loss[b*t] U(0, 10) (positive, like cross-entropy values);
    the parameter gradients as one flat buffer N(0, 0.01) laid out by
    grad_arena_offsets (padding included); the loss's upstream gradient 1."""
    shapes = gpt_param_shapes(ctx=t)
    _, total = grad_arena_offsets(shapes)
    return dict(loss=uniform((b * t,), 6001, 0.0, 10.0),
                grads=normal((total,), 6002, 0.0, 0.01),
                g=np.array(1.0, dtype=np.float32))


def gpt_row_stats(b=64, t=256, c=384, heads=6):
    """LayerNorm input x[b*t, c] N(0,1) and attention scores [b*heads*t, t]
    N(0,1) with the causal mask added (row i of each t x t block: -1e9 for
    j > i), i.e. the masked scores the softmax reduces."""
    x = normal((b * t, c), 7001)
    s = normal((b * heads, t, t), 7002)
    s += causal_mask(t).reshape(1, t, t)
    return dict(x=x, scores=s.reshape(b * heads * t, t))
