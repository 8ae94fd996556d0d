"""Workloads of the parity tests: seeded matrices and activations (from
block_quant_weight_amd.synth), laid out as the file holds them by the
oracle's own span rule, plus small GPU helpers."""
import os

import numpy as np

import oracle as O
from block_quant_weight_amd import synth

Q8, Q4 = 1, 2
THREADS = max(1, min(16, os.cpu_count() or 1))


def make_image(config, matrix, wtype, sf16, rows, cols, lo=1e-3, hi=1e-2):
    gq = synth.rng(config, matrix, synth.STREAM_QUANTS)
    gd = synth.rng(config, matrix, synth.STREAM_SCALES)
    q = synth.q8_quants(gq, rows, cols) if wtype == Q8 else synth.q4_quants(gq, rows, cols)
    d = synth.scales(gd, rows * cols // 32, bool(sf16), lo, hi)
    return O.layout(wtype, sf16, rows, cols, q, d)


def make_x(config, matrix, batch, cols):
    return synth.act_f32(synth.rng(config, matrix, synth.STREAM_ACT), batch, cols)


def make_xb(config, matrix, batch, cols):
    return synth.act_bf16(synth.rng(config, matrix, synth.STREAM_ACT), batch, cols)


# The mixed-precision decode layer: dim 4096, 32 heads, 8 KV heads, head_dim
# 128 (q_dim 4096, kv_dim 1024), FFN 11008; q8_mask = 8 | 64; f16 scales.
# (name, class bit, rows, cols)
LAYER = [("wq", 4, 4096, 4096), ("wk", 4, 1024, 4096), ("wv", 8, 1024, 4096),
         ("wo", 16, 4096, 4096), ("w1", 32, 11008, 4096), ("w3", 32, 11008, 4096),
         ("w2", 64, 4096, 11008)]
LAYER_Q8_MASK = 8 | 64

# Shared classifier: vocab 248320, hidden 1024, Q8_0 with f16 scales.
VOCAB, HIDDEN = 248320, 1024


def sample_rows(rows, n, seed=0, tile=128):
    """First and last rows, rows around tile edges, and a seeded sample."""
    g = np.random.default_rng(seed)
    fixed = {0, 1, rows - 1, rows - 2}
    for t in range(tile, rows, tile * max(1, rows // (tile * 8))):
        fixed.update({t - 1, t})
    extra = g.choice(rows, size=min(n, rows), replace=False)
    sel = sorted(r for r in fixed.union(extra.tolist()) if 0 <= r < rows)
    return np.array(sel, dtype=np.int64)


# ---- GPU side -------------------------------------------------------------

def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload(img, wtype, sf16, rows, cols):
    from block_quant_weight_amd import qmv as Q
    h = Q.qmv_create(wtype, sf16, rows, cols)
    Q.qmv_upload(h, img)
    return h


def gpu_gemv(h, x):
    import torch
    from block_quant_weight_amd import qmv as Q
    xd = dev(x.astype(np.float32))
    y = torch.empty((x.shape[0], h.rows), dtype=torch.float32, device="cuda")
    Q.qmv_gemv(h, xd, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_gemm(h, xb):
    import torch
    from block_quant_weight_amd import qmv as Q
    xd = dev(xb.view(np.int16)).view(torch.bfloat16)
    y = torch.empty((xb.shape[0], h.rows), dtype=torch.float32, device="cuda")
    Q.qmv_gemm(h, xd, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_embed(h, ids):
    import torch
    from block_quant_weight_amd import qmv as Q
    idd = dev(np.asarray(ids, dtype=np.int32))
    out = torch.empty((len(ids), h.cols), dtype=torch.float32, device="cuda")
    Q.qmv_embed_rows(h, idd, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()
