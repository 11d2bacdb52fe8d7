"""Oracle for the kernel-generation (KG) transformer: plain NumPy, float64.

TEST INFRASTRUCTURE, like the rest of this package (only tests/, the smoke
check and the CPU-baseline leg of bench.py may use it).

What it computes, and the readings taken (GKDT model card, "Architecture"
bullet; the paper summary's four-step pipeline; the Chinese analysis page,
"key mechanisms" paragraph and its discussion of the SA/CA ablation):

* The KG transformer turns the visual and the text keypoint prototypes into
  the kernels the detection head convolves with. It has 2 blocks of
  self-attention (SA) over the prototypes, cross-attention (CA) from the
  prototypes to the query image's features, and a feed-forward net of
  width d_ff = 1024, plus a learned mask token.
* Sequence (reading): the 2R slots [visual row 0..R-1, text row 0..R-1] of
  one crop. A slot whose row has no prompt of that kind holds the mask
  token. The pages say strong-modality prototypes calibrate weak ones, so
  both sets sit in one SA sequence.
* Keys (reading): SA keys are the slots of rows that carry at least one
  prompt; the slots of padding rows are queries only, so a crop's valid
  outputs do not depend on how far its rows are padded. A crop without a
  single prompted row gets a zero attention output. CA keys and values
  are the H*W query-feature tokens.
* Block (reading: torch's decoder layer in its default post-norm form,
  which the model card's converter notes match by splitting a packed
  q/k/v in_proj): x = LN1(x + SA(x)); x = LN2(x + CA(x, F));
  x = LN3(x + W2 relu(W1 x + b1) + b2); LayerNorm eps 1e-5, dropout off.
* Heads (reading): 64-wide heads, C/64 of them (16 at C = 1024, as in the
  ViT-L tower the features come from), scores scaled by 1/sqrt(64).
* Output: [B, 2R, C], the visual kernels in slots 0..R-1 and the text
  kernels in slots R..2R-1.

Weights come as one flat array in this order: mask token [C]; then per
block: SA in_proj weight [3C, C] and bias [3C], SA out_proj weight [C, C]
and bias [C], LN1 weight and bias [C] each, CA in_proj weight [3C, C] and
bias [3C], CA out_proj weight [C, C] and bias [C], LN2 weight and bias, FFN
W1 [d_ff, C] and b1 [d_ff], W2 [C, d_ff] and b2 [C], LN3 weight and bias.
torch.nn.Linear stores weights as [out, in]; y = x W^T + b.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 64
LN_EPS = 1e-5


def block_size(C: int, d_ff: int) -> int:
    """Elements of one block's weights in the flat array."""
    return 8 * C * C + 2 * d_ff * C + 15 * C + d_ff


def unpack(weights, C: int, d_ff: int, n_blocks: int):
    """Split the flat weight array into the mask token and per-block dicts."""
    w = np.asarray(weights, dtype=np.float64).ravel()
    if w.size != C + n_blocks * block_size(C, d_ff):
        raise ValueError("weight array has the wrong size")
    pos = 0

    def take(*shape):
        nonlocal pos
        n = int(np.prod(shape))
        out = w[pos:pos + n].reshape(shape)
        pos += n
        return out

    mask_token = take(C)
    blocks = []
    for _ in range(n_blocks):
        b = {}
        b["sa_in_w"], b["sa_in_b"] = take(3 * C, C), take(3 * C)
        b["sa_out_w"], b["sa_out_b"] = take(C, C), take(C)
        b["ln1_w"], b["ln1_b"] = take(C), take(C)
        b["ca_in_w"], b["ca_in_b"] = take(3 * C, C), take(3 * C)
        b["ca_out_w"], b["ca_out_b"] = take(C, C), take(C)
        b["ln2_w"], b["ln2_b"] = take(C), take(C)
        b["ff1_w"], b["ff1_b"] = take(d_ff, C), take(d_ff)
        b["ff2_w"], b["ff2_b"] = take(C, d_ff), take(C)
        b["ln3_w"], b["ln3_b"] = take(C), take(C)
        blocks.append(b)
    return mask_token, blocks


def layer_norm(x, w, b):
    """LayerNorm over the last axis: biased variance, eps inside the root."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + LN_EPS) * w + b


def softmax_rows(s, key_ok):
    """Softmax over the last axis, restricted to the keys with key_ok; a row
    with no allowed key gives all zeros."""
    s = np.where(key_ok, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(key_ok, np.exp(s - m), 0.0)
    z = e.sum(axis=-1, keepdims=True)
    return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def attention(x, mem, in_w, in_b, out_w, out_b, key_ok):
    """Multi-head attention of the rows of x [T, C] over mem [S, C]; key_ok
    [S] marks the keys that may be attended to."""
    C = x.shape[1]
    nh = C // HEAD_DIM
    q = x @ in_w[:C].T + in_b[:C]
    k = mem @ in_w[C:2 * C].T + in_b[C:2 * C]
    v = mem @ in_w[2 * C:].T + in_b[2 * C:]
    out = np.empty_like(q)
    for h in range(nh):
        cs = slice(h * HEAD_DIM, (h + 1) * HEAD_DIM)
        s = (q[:, cs] @ k[:, cs].T) / np.sqrt(HEAD_DIM)
        out[:, cs] = softmax_rows(s, key_ok[None, :]) @ v[:, cs]
    return out @ out_w.T + out_b


def kg_block(x, mem, b, key_ok):
    """One post-norm block: SA, then CA to mem, then the ReLU FFN."""
    x = layer_norm(x + attention(x, x, b["sa_in_w"], b["sa_in_b"], b["sa_out_w"],
                                 b["sa_out_b"], key_ok), b["ln1_w"], b["ln1_b"])
    all_keys = np.ones(mem.shape[0], dtype=bool)
    x = layer_norm(x + attention(x, mem, b["ca_in_w"], b["ca_in_b"], b["ca_out_w"],
                                 b["ca_out_b"], all_keys), b["ln2_w"], b["ln2_b"])
    h = np.maximum(x @ b["ff1_w"].T + b["ff1_b"], 0.0)
    return layer_norm(x + h @ b["ff2_w"].T + b["ff2_b"], b["ln3_w"], b["ln3_b"])


def kg_sequence(vis, mask_vis, txt, mask_txt, mask_token):
    """The 2R input slots of one crop and its SA key mask."""
    R, C = mask_vis.shape[0], mask_token.shape[0]
    x = np.empty((2 * R, C))
    for r in range(R):
        x[r] = vis[r] if mask_vis[r] else mask_token
        x[R + r] = txt[r] if mask_txt[r] else mask_token
    row_ok = mask_vis | mask_txt
    return x, np.concatenate([row_ok, row_ok])


def kg_transformer(vis, mask_vis, txt, mask_txt, query, weights, n_blocks=2, d_ff=1024,
                   tokens=False):
    """Kernels [B, 2R, C] (float64) from the prototypes.

    vis, txt: [B, R, C] prototypes (None when that modality is absent);
    mask_vis, mask_txt: [B, R] (None: no row has that prompt);
    query: [B, C, H, W], or [B, H*W, C] tokens when tokens is set;
    weights: the flat array described in the module docstring."""
    query = np.asarray(query, dtype=np.float64)
    B = query.shape[0]
    C = query.shape[2] if tokens else query.shape[1]
    mem_all = query if tokens else query.reshape(B, C, -1).transpose(0, 2, 1)
    R = (mask_vis if mask_vis is not None else mask_txt).shape[1]
    zeros = np.zeros((B, R, C))
    no = np.zeros((B, R), dtype=bool)
    vis = zeros if vis is None else np.asarray(vis, dtype=np.float64)
    txt = zeros if txt is None else np.asarray(txt, dtype=np.float64)
    mv = no if mask_vis is None else np.asarray(mask_vis).astype(bool)
    mt = no if mask_txt is None else np.asarray(mask_txt).astype(bool)
    mask_token, blocks = unpack(weights, C, d_ff, n_blocks)
    out = np.empty((B, 2 * R, C))
    for bi in range(B):
        x, key_ok = kg_sequence(vis[bi], mv[bi], txt[bi], mt[bi], mask_token)
        for b in blocks:
            x = kg_block(x, mem_all[bi], b, key_ok)
        out[bi] = x
    return out
