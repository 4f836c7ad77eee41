"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

These stand in for the pages' models and datasets (LLaMA-3.1-8B, LongBench,
RULER, MATH-500, ...), which are not available: every tensor is drawn from a
seeded ``torch.Generator`` on the requested device and rounded to bf16 with
round-to-nearest-even.  The same tensors feed the HIP library and the CPU
oracle.

Recipe (one stream = one batch entry x one kv head):

* ``u`` -- a unit direction per stream: a standard normal vector, normalised.
* queries (window and decode, every q head of the group):
  ``q = sqrt(1 - rho^2) z + rho sqrt(D) u`` with ``rho = 1/2``.
* keys ``K = z`` (plus the per-4096-token drifting mean of the million-token
  workload), then 4 outlier channels per stream, drawn without replacement,
  scaled by 10 (the MosaicKV page, Fig. 2 text: outliers sit in few channels).
* heavy tokens (the pages' observation that importance is concentrated):
  ``k = kappa sqrt(D) u + z/4`` with ``kappa = 1.5``.
* values ``V = z``.

Draw order per call: u, outlier channels, heavy positions, K noise, V noise,
window-query noise, decode-query noise (drifting mean between heavy positions
and K noise for the million-token workload).  Large workloads are drawn one
batch entry at a time in that order.
"""
import math

import numpy as np
import torch

D = 128
RHO = 0.5
KAPPA = 1.5
N_OUTLIER = 4
OUTLIER_SCALE = 10.0


def table9(S):
    """The nine strategies {100, 50, 25}% tokens x {128, 64, 32} channels, in that
    order, as (T, c) integers with T = pct*S/100 rounded half up."""
    out = []
    for pct in (100, 50, 25):
        for c in (128, 64, 32):
            out.append(((pct * S + 50) // 100, c))
    return out


def budget_bytes(pct, S):
    """Per-segment byte cap: pct of the dense K+V bytes of the segment."""
    return (pct * 4 * S * D) // 100


# The five workloads.  W (window queries per q head) for the three large
# configurations is a choice of this implementation; the pages do not give it.
CONFIGS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, N=4096, S=64, W=32, budget_pct=33, heavy="count",
                 heavy_n=16),
    "llama8b": dict(B=1, Hq=32, Hkv=8, N=32768, S=128, W=64, budget_pct=33, heavy="frac",
                    heavy_frac=0.005),
    "batched128k": dict(B=16, Hq=32, Hkv=8, N=131072, S=128, W=64, budget_pct=25,
                        heavy="segment", heavy_dmax=0.02),
    "million": dict(B=1, Hq=32, Hkv=8, N=1048576, S=256, W=64, budget_pct=20, heavy=None,
                    drift_block=4096, drift_sigma=0.1),
}

# Kara-style sliding-window workload (events every `delta` steps).
KARA = dict(B=64, Hq=32, Hkv=8, prompt=16384, gen=8192, window=512, retention_pct=20,
            gamma=16, alpha=3, page=16, delta=64, protect=64, spans=32, span_min=4, span_max=16)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(g, shape, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _rand(g, shape, device):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def _queries(g, u_rep, n, device):
    """u_rep: [Hq, D] direction of each q head's kv head."""
    Hq = u_rep.shape[0]
    z = _randn(g, (Hq, n, D), device)
    q = math.sqrt(1.0 - RHO * RHO) * z + RHO * math.sqrt(D) * u_rep[:, None, :]
    return q.to(torch.bfloat16)


def _outliers(g, Hkv, device):
    return _rand(g, (Hkv, D), device).argsort(dim=-1)[:, :N_OUTLIER]


def _keys(z, u, heavy, outl):
    """z: [Hkv, N, D] noise (already carrying any drift); heavy: [Hkv, N] bool."""
    k = torch.where(heavy[..., None], KAPPA * math.sqrt(D) * u[:, None, :] + 0.25 * z, z)
    scale = torch.ones(u.shape[0], D, device=z.device)
    scale.scatter_(1, outl, OUTLIER_SCALE)
    return (k * scale[:, None, :]).to(torch.bfloat16)


def make_workload(cfg, seed=0, device="cpu", N=None, B=None, with_decode_query=True):
    """Inputs of one workload.

    Returns dict K, V [B,Hkv,N,D] bf16, Qw [B,Hq,W,D] bf16, q [B,Hq,D] bf16 and
    ``heavy`` [B,Hkv,N] bool.  ``N``/``B`` override the config's sizes (for the
    small cases the oracle finishes quickly); the structure stays the same.
    """
    c = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    Hq, Hkv, S, W = c["Hq"], c["Hkv"], c["S"], c["W"]
    G = Hq // Hkv
    g = _gen(seed, device)
    K = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    Qw = torch.empty((B, Hq, W, D), dtype=torch.bfloat16, device=device)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=device)
    heavy_all = torch.zeros((B, Hkv, N), dtype=torch.bool, device=device)
    for b in range(B):
        z = _randn(g, (Hkv, D), device)
        u = z / z.norm(dim=-1, keepdim=True)
        outl = _outliers(g, Hkv, device)
        kind = c.get("heavy")
        if kind == "count":
            r = _rand(g, (Hkv, N), device)
            heavy = r.argsort(dim=-1).argsort(dim=-1) < c["heavy_n"]
        elif kind == "frac":
            cnt = int(round(c["heavy_frac"] * N))
            r = _rand(g, (Hkv, N), device)
            heavy = r.argsort(dim=-1).argsort(dim=-1) < cnt
        elif kind == "segment":
            nseg = N // S
            d = _rand(g, (Hkv, nseg), device) * c["heavy_dmax"]
            cnt = torch.round(d * S)
            r = _rand(g, (Hkv, nseg, S), device)
            heavy = (r.argsort(dim=-1).argsort(dim=-1) < cnt[..., None]).reshape(Hkv, N)
        else:
            heavy = torch.zeros((Hkv, N), dtype=torch.bool, device=device)
        zk = _randn(g, (Hkv, N, D), device)
        if c.get("drift_block"):
            nb = (N + c["drift_block"] - 1) // c["drift_block"]
            steps = c["drift_sigma"] * _randn(g, (Hkv, nb, D), device)
            steps[:, 0, :] = 0.0
            mu = steps.cumsum(dim=1)
            zk = zk + mu.repeat_interleave(c["drift_block"], dim=1)[:, :N, :]
        K[b] = _keys(zk, u, heavy, outl)
        del zk
        V[b] = _randn(g, (Hkv, N, D), device).to(torch.bfloat16)
        u_rep = u.repeat_interleave(G, dim=0)
        Qw[b] = _queries(g, u_rep, W, device)
        if with_decode_query:
            q[b] = _queries(g, u_rep, 1, device)[:, 0, :]
        heavy_all[b] = heavy
    return dict(K=K, V=V, Qw=Qw, q=q, heavy=heavy_all, S=S, W=W, G=G, B=B, N=N, Hq=Hq,
                Hkv=Hkv, budget_pct=c["budget_pct"])


def make_kara(seed=0, device="cpu", B=None, prompt=None, gen=None):
    """Kara-style workload: K, V [B,Hkv,L,D] and queries at every position
    Qall [B,Hq,L,D] (L = prompt + gen), with 32 planted heavy spans of length
    4..16 per stream inside the generated region; decode query q [B,Hq,D]."""
    c = dict(KARA)
    B = c["B"] if B is None else B
    prompt = c["prompt"] if prompt is None else prompt
    gen = c["gen"] if gen is None else gen
    Hq, Hkv = c["Hq"], c["Hkv"]
    G = Hq // Hkv
    L = prompt + gen
    g = _gen(seed, device)
    K = torch.empty((B, Hkv, L, D), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    Qall = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=device)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=device)
    for b in range(B):
        z = _randn(g, (Hkv, D), device)
        u = z / z.norm(dim=-1, keepdim=True)
        outl = _outliers(g, Hkv, device)
        lens = torch.randint(c["span_min"], c["span_max"] + 1, (Hkv, c["spans"]), generator=g,
                             device=device)
        starts = (_rand(g, (Hkv, c["spans"]), device) * (gen - lens + 1).float()).long()
        pos = torch.arange(gen, device=device)
        inside = (pos[None, None, :] >= starts[..., None]) & (pos[None, None, :] < (starts + lens)[..., None])
        heavy = torch.zeros((Hkv, L), dtype=torch.bool, device=device)
        heavy[:, prompt:] = inside.any(dim=1)
        K[b] = _keys(_randn(g, (Hkv, L, D), device), u, heavy, outl)
        V[b] = _randn(g, (Hkv, L, D), device).to(torch.bfloat16)
        u_rep = u.repeat_interleave(G, dim=0)
        Qall[b] = _queries(g, u_rep, L, device)
        q[b] = _queries(g, u_rep, 1, device)[:, 0, :]
    return dict(K=K, V=V, Qall=Qall, q=q, B=B, L=L, prompt=prompt, gen=gen, Hq=Hq, Hkv=Hkv, G=G)


def offaxis_blocks(X, block, seed=1):
    """X: [B, Hkv, N, D] bf16 -> a copy in which every `block`-token block of
    every stream is multiplied by its own seeded random orthogonal matrix
    (QR of a Gaussian matrix) and rounded to bf16 again.  The outlier
    channels and heavy-token directions of the recipe then sit along
    directions that differ from block to block instead of along channels
    (an input transformation only)."""
    B, H, N, _ = X.shape
    g = _gen(seed, X.device)
    out = torch.empty_like(X)
    nb = (N + block - 1) // block
    for b in range(B):
        Q, _ = torch.linalg.qr(_randn(g, (H * nb, D, D), X.device).cpu())
        Q = Q.to(X.device).view(H, nb, D, D)
        for j in range(nb):
            t0, t1 = j * block, min(N, (j + 1) * block)
            out[b, :, t0:t1] = (X[b, :, t0:t1].float() @ Q[:, j]).to(torch.bfloat16)
    return out


def u16(t):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_u16(a, device="cpu"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
