"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random numbers and shapes them; it holds none of the
recurrence's arithmetic, so both the GPU library's tests and the CPU oracle can
consume the same bytes.

Distributions (the workload descriptions; draws on a CPU ``torch.Generator``):
  * q, k ~ N(0, 1), then L2-normalised per token in fp32, then cast to the input dtype;
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1));
  * log alpha = -a_h * softplus(N(0, 1)) with a_h = exp(A_h), A_h = log U(1, 16) drawn once
    per value head (the "tiny_gdn/fugue.py" page draws A_log = log U(1, 16) per head and
    direction; the "sparse-delta-memory layer.py" page, ``compute_gates``, has the same
    -exp(A) * softplus(.) form);
  * h0 ~ sigma * N(0, 1) in fp32 (sigma read as a standard deviation).

Draw order per case: per-head A, q, k, v, the decay normals, the beta normals, then h0.
The segment lengths of a packed case are drawn first, with their own seed offset.

Extra gate regimes (for tests that must see the carried state, which the workload
gates erase within a few tokens):
  * "zero":  log alpha = 0 (pure delta rule, alpha = 1);
  * "p5":    alpha ~ U(0.5, 1) (the "Prizma seq/delta.py" page's self-test regime);
  * "slow":  log alpha = -U(0, 0.05).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

GATE_REGIMES = ("config", "zero", "p5", "slow")


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, std=1.0):
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _l2_normalise(x):
    return torch.nn.functional.normalize(x, dim=-1, eps=1e-12)


def _gates(g, A_head, lead_shape, regime):
    """log_alpha, beta of shape lead_shape = (..., Hv, T); A_head has shape (Hv,)."""
    z = _normal(g, lead_shape)
    zb = _normal(g, lead_shape)
    beta = torch.sigmoid(zb)
    if regime == "config":
        a = torch.exp(A_head).view(*([1] * (len(lead_shape) - 2)), -1, 1)
        log_alpha = -a * torch.nn.functional.softplus(z)
    elif regime == "zero":
        log_alpha = torch.zeros(lead_shape)
    elif regime == "p5":
        log_alpha = torch.log(0.5 + 0.5 * torch.rand(tuple(lead_shape), generator=g))
    elif regime == "slow":
        log_alpha = -0.05 * torch.rand(tuple(lead_shape), generator=g)
    else:
        raise ValueError("unknown gate regime %r (choose from %s)" % (regime, GATE_REGIMES))
    return log_alpha.contiguous(), beta.contiguous()


@dataclass
class ChunkCase:
    """Inputs of one chunked-forward call (CPU tensors)."""
    q: torch.Tensor            # [B, Hk, T, dk]
    k: torch.Tensor            # [B, Hk, T, dk]
    v: torch.Tensor            # [B, Hv, T, dv]
    log_alpha: torch.Tensor    # [B, Hv, T] fp32
    beta: torch.Tensor         # [B, Hv, T] fp32
    h0: torch.Tensor | None    # [nseq, Hv, dk, dv] fp32
    cu_seqlens: torch.Tensor | None   # [nseq + 1] int32
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return int(self.q.shape[0] * self.q.shape[2])


def chunk_case(*, B=1, T=256, Hk=2, Hv=None, dk=64, dv=64, dtype=torch.float32, seed=0,
               h0_std=0.0, regime="config", lengths=None) -> ChunkCase:
    """Draw one chunked-forward case. ``lengths`` (list of ints) packs segments into B=1."""
    Hv = Hk if Hv is None else Hv
    g = _gen(seed)
    cu = None
    if lengths is not None:
        B = 1
        lengths = [int(x) for x in lengths]
        T = sum(lengths)
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    nseq = B if cu is None else len(lengths)
    A_head = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=g))
    q = _l2_normalise(_normal(g, (B, Hk, T, dk))).to(dtype).contiguous()
    k = _l2_normalise(_normal(g, (B, Hk, T, dk))).to(dtype).contiguous()
    v = _normal(g, (B, Hv, T, dv)).to(dtype).contiguous()
    log_alpha, beta = _gates(g, A_head, (B, Hv, T), regime)
    h0 = _normal(g, (nseq, Hv, dk, dv), h0_std).contiguous() if h0_std > 0 else None
    return ChunkCase(q, k, v, log_alpha, beta, h0, cu)


def segment_lengths(n, lo, hi, seed) -> list[int]:
    """n integer lengths drawn uniformly from [lo, hi], both ends included."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


@dataclass
class DecodeCase:
    q: torch.Tensor          # [steps, N, Hk, dk]
    k: torch.Tensor          # [steps, N, Hk, dk]
    v: torch.Tensor          # [steps, N, Hv, dv]
    log_alpha: torch.Tensor  # [steps, N, Hv] fp32
    beta: torch.Tensor       # [steps, N, Hv] fp32
    state: torch.Tensor      # [N, Hv, dk, dv] fp32


def decode_case(*, N=4, Hk=2, Hv=4, dk=128, dv=128, steps=1, dtype=torch.bfloat16, seed=0,
                state_std=0.05, regime="config") -> DecodeCase:
    g = _gen(seed)
    A_head = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=g))
    q = _l2_normalise(_normal(g, (steps, N, Hk, dk))).to(dtype).contiguous()
    k = _l2_normalise(_normal(g, (steps, N, Hk, dk))).to(dtype).contiguous()
    v = _normal(g, (steps, N, Hv, dv)).to(dtype).contiguous()
    # gates laid out [steps, N, Hv] with the per-head A broadcast along the head axis
    la, beta = _gates(g, A_head, (steps * N, Hv, 1), regime)
    log_alpha = la.view(steps, N, Hv).contiguous()
    beta = beta.view(steps, N, Hv).contiguous()
    state = _normal(g, (N, Hv, dk, dv), state_std).contiguous()
    return DecodeCase(q, k, v, log_alpha, beta, state)


# ---------------------------------------------------------------------------
# The five workloads. Seeds are 1000 + workload index.

@dataclass
class RawCase:
    """Inputs of the fused prologue: raw q, k (rows of varied length), raw gate inputs a, b
    and per-value-head gate parameters A_log, dt_bias."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    h0: torch.Tensor | None
    cu_seqlens: torch.Tensor | None


def raw_case(*, B=1, T=256, Hk=2, Hv=None, dk=64, dv=64, dtype=torch.float32, seed=0,
             h0_std=0.0, lengths=None) -> RawCase:
    """q, k ~ N(0, 1) times a per-row length factor U(0.25, 4) (not normalised); v ~ N(0, 1);
    a, b ~ N(0, 1); A_log = log U(1, 16) and dt_bias ~ U(-4, 1) per value head (the range
    softplus(a + dt_bias) takes at the pages' dt_bias initialisation, 0.001..0.1, and above)."""
    Hv = Hk if Hv is None else Hv
    g = _gen(seed + 50000)
    cu = None
    if lengths is not None:
        assert B == 1
        T = int(sum(lengths))
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    nseq = B if cu is None else len(lengths)
    A_log = torch.log(torch.rand(Hv, generator=g) * 15.0 + 1.0)
    dt_bias = torch.rand(Hv, generator=g) * 5.0 - 4.0
    q = (_normal(g, (B, Hk, T, dk)) * (torch.rand(B, Hk, T, 1, generator=g) * 3.75 + 0.25)).to(dtype).contiguous()
    k = (_normal(g, (B, Hk, T, dk)) * (torch.rand(B, Hk, T, 1, generator=g) * 3.75 + 0.25)).to(dtype).contiguous()
    v = _normal(g, (B, Hv, T, dv)).to(dtype).contiguous()
    a = _normal(g, (B, Hv, T)).contiguous()
    b = _normal(g, (B, Hv, T)).contiguous()
    h0 = _normal(g, (nseq, Hv, dk, dv), h0_std).contiguous() if h0_std > 0 else None
    return RawCase(q, k, v, a, b, A_log.contiguous(), dt_bias.contiguous(), h0, cu)


@dataclass
class Gdn2Case:
    q: torch.Tensor          # [B, Hk, T, dk]
    k: torch.Tensor          # [B, Hk, T, dk]
    v: torch.Tensor          # [B, Hv, T, dv]
    g: torch.Tensor          # [B, Hk, T, dk] fp32 log decay per key channel
    b: torch.Tensor          # [B, Hk, T, dk] erase gate
    w: torch.Tensor          # [B, Hv, T, dv] write gate
    h0: torch.Tensor | None  # [S, Hv, dk, dv] fp32
    cu_seqlens: torch.Tensor | None = None


GDN2_REGIMES = ("page", "weak", "strong", "mixed")


def gdn2_case(*, B=1, T=256, Hk=2, Hv=None, dk=64, dv=64, dtype=torch.float32, seed=0, h0_std=0.0,
              lengths=None, regime="page", unit_rows=True) -> Gdn2Case:
    """GDN-2 inputs with the distributions of the BidirectionalGatedDeltaNet2 layer on the
    "tiny_gdn/fugue.py" page at its initialisation:
      * "page": g = -A_h softplus(f + dt_bias_c), A_h ~ U(1, 16) per key head, dt_bias_c the
        inverse softplus of dt ~ logU(0.001, 0.1) per key channel, f ~ N(0, 1) per token and channel;
      * "weak": g = -U(0, 0.05) (long memory); "strong": g = -U(2, 10) (every 16-token block decays
        by more than e^-60 on some channel); "mixed": "page", with g = -U(2, 10) on every fourth
        key channel of the tokens t with (t // 16) % 3 == 0 (strong and weak blocks side by side);
      * b = 2 sigmoid(N(0, 1)) (the allow_neg_eigval range (0, 2)), w = sigmoid(N(0, 1));
      * q, k ~ N(0, 1), L2-normalised per row in fp32 when ``unit_rows``, otherwise times a
        per-row length factor U(0.25, 4); v ~ N(0, 1); h0 ~ h0_std N(0, 1).
    Draw order: A, dt, q, k, v, f (or the uniform g), b, w, row factors, h0."""
    assert regime in GDN2_REGIMES, regime
    Hv = Hk if Hv is None else Hv
    g = _gen(seed + 70000)
    cu = None
    if lengths is not None:
        assert B == 1
        T = int(sum(lengths))
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    nseq = B if cu is None else len(lengths)
    A = torch.rand(Hk, generator=g) * 15.0 + 1.0
    dt = torch.exp(torch.rand(dk, generator=g) * (math.log(0.1) - math.log(0.001)) + math.log(0.001))
    dt_bias = dt + torch.log(-torch.expm1(-dt))
    q = _normal(g, (B, Hk, T, dk))
    k = _normal(g, (B, Hk, T, dk))
    v = _normal(g, (B, Hv, T, dv)).to(dtype).contiguous()
    if regime == "page":
        f = _normal(g, (B, Hk, T, dk))
        gate = -A[None, :, None, None] * torch.nn.functional.softplus(f + dt_bias)
    elif regime == "mixed":
        f = _normal(g, (B, Hk, T, dk))
        gate = -A[None, :, None, None] * torch.nn.functional.softplus(f + dt_bias)
        strong = -(torch.rand(B, Hk, T, dk, generator=g) * 8.0 + 2.0)
        sel = ((torch.arange(T) // 16) % 3 == 0)[:, None] & (torch.arange(dk) % 4 == 0)[None, :]
        gate = torch.where(sel, strong, gate)
    elif regime == "weak":
        gate = -torch.rand(B, Hk, T, dk, generator=g) * 0.05
    else:
        gate = -(torch.rand(B, Hk, T, dk, generator=g) * 8.0 + 2.0)
    b = (2.0 * torch.sigmoid(_normal(g, (B, Hk, T, dk)))).to(dtype).contiguous()
    w = torch.sigmoid(_normal(g, (B, Hv, T, dv))).to(dtype).contiguous()
    if unit_rows:
        q, k = _l2_normalise(q), _l2_normalise(k)
    else:
        q = q * (torch.rand(B, Hk, T, 1, generator=g) * 3.75 + 0.25)
        k = k * (torch.rand(B, Hk, T, 1, generator=g) * 3.75 + 0.25)
    h0 = _normal(g, (nseq, Hv, dk, dv), h0_std).contiguous() if h0_std > 0 else None
    return Gdn2Case(q.to(dtype).contiguous(), k.to(dtype).contiguous(), v, gate.float().contiguous(), b, w, h0, cu)


@dataclass
class DeltaProductCase:
    q: torch.Tensor          # [B, Hk, T, dk]
    k: torch.Tensor          # [B, Hk, T, n, dk]
    v: torch.Tensor          # [B, Hv, T, n, dv]
    log_alpha: torch.Tensor  # [B, Hv, T] fp32
    beta: torch.Tensor       # [B, Hv, T, n] fp32
    h0: torch.Tensor | None  # [S, Hv, dk, dv] fp32
    cu_seqlens: torch.Tensor | None = None


def delta_product_case(*, B=1, T=256, n=2, Hk=2, Hv=None, dk=64, dv=64, dtype=torch.float32, seed=0,
                       h0_std=0.0, lengths=None, regime="config") -> DeltaProductCase:
    """DeltaProduct inputs: the distributions of ``chunk_case`` with n keys, values and betas per
    token (every sub-step's key L2-normalised in fp32) and one decay per token. Draw order: A, q,
    k, v, the decay normals (or uniforms), the beta normals, h0."""
    Hv = Hk if Hv is None else Hv
    g = _gen(seed + 90000)
    cu = None
    if lengths is not None:
        assert B == 1
        T = int(sum(lengths))
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    nseq = B if cu is None else len(lengths)
    A = torch.log(torch.rand(Hv, generator=g) * 15.0 + 1.0)
    q = _l2_normalise(_normal(g, (B, Hk, T, dk))).to(dtype).contiguous()
    k = _l2_normalise(_normal(g, (B, Hk, T, n, dk))).to(dtype).contiguous()
    v = _normal(g, (B, Hv, T, n, dv)).to(dtype).contiguous()
    log_alpha, _ = _gates(g, A, (B, Hv, T), regime)
    beta = torch.sigmoid(_normal(g, (B, Hv, T, n))).contiguous()
    h0 = _normal(g, (nseq, Hv, dk, dv), h0_std).contiguous() if h0_std > 0 else None
    return DeltaProductCase(q, k, v, log_alpha, beta, h0, cu)


WORKLOADS = {
    0: "gdr-fwd-fp32-B1-H2-T256-d64-c64",
    1: "gdr-chunk-fwd-bf16-B4-H16-T4096-d128-c64",
    2: "gdr-varlen-bf16-8seg-512..8192-H32-d128-c64",
    3: "gdr-decode-bf16-N256-Hk16-Hv32-d128-64steps",
    4: "gdr-bidir-pre-bf16-4x4096-H16-d128-c64",
}


def workload0(regime="config") -> ChunkCase:
    return chunk_case(B=1, T=256, Hk=2, dk=64, dv=64, dtype=torch.float32, seed=1000,
                      h0_std=0.0, regime=regime)


def workload1(regime="config", T=4096) -> ChunkCase:
    return chunk_case(B=4, T=T, Hk=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
                      h0_std=0.1, regime=regime)


def workload2(regime="config", lengths=None) -> ChunkCase:
    if lengths is None:
        lengths = segment_lengths(8, 512, 8192, seed=1002 + 7919)
    return chunk_case(Hk=32, dk=128, dv=128, dtype=torch.bfloat16, seed=1002, h0_std=0.1,
                      regime=regime, lengths=lengths)


def workload3(regime="config", N=256, steps=64) -> DecodeCase:
    return decode_case(N=N, Hk=16, Hv=32, dk=128, dv=128, steps=steps, dtype=torch.bfloat16,
                       seed=1003, state_std=0.05, regime=regime)


def workload4(regime="config", seg_len=4096, nseg=4, H=16):
    """Bidirectional case: shared q, k, v; one gate set per direction; h0 = 0."""
    lengths = [seg_len] * nseg
    g = _gen(1004)
    T = sum(lengths)
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    A_dir = torch.log(1.0 + 15.0 * torch.rand(2, H, generator=g))
    q = _l2_normalise(_normal(g, (1, H, T, 128))).to(torch.bfloat16).contiguous()
    k = _l2_normalise(_normal(g, (1, H, T, 128))).to(torch.bfloat16).contiguous()
    v = _normal(g, (1, H, T, 128)).to(torch.bfloat16).contiguous()
    la_f, b_f = _gates(g, A_dir[0], (1, H, T), regime)
    la_b, b_b = _gates(g, A_dir[1], (1, H, T), regime)
    case = ChunkCase(q, k, v, la_f, b_f, None, cu)
    case.extra = {"log_alpha_bwd": la_b, "beta_bwd": b_b}
    return case
