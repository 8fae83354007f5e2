"""Seeded synthetic inputs of the decode-batch front's workloads.

This module only draws inputs: it holds none of the front's arithmetic and
imports neither the library nor any checker, so the HIP path and the CPU
oracle can both be fed from it.

Shapes and distributions (qkv_front page, module summary, for 1 <= M <= 16;
cute_ops page, split_qkv and the attn2 contract for widths and the cache):
  x         bf16 [M, 8192] ~ N(0, 1), optionally with outlier rows x30;
  W         bf16 [N, 8192] ~ N(0, 0.011^2), N = 1152 * nkv;
  positions int64 [M], slots int64 [M] (distinct), per workload;
  cos_sin   fp32 [rows, 64]: row p holds cos(p * f_i) in column i and
            sin(p * f_i) in column 32 + i, f_i = theta^(-2i/64), theta 10000
            (the interleaved rotary table's usual construction);
  kv_cache  bf16 [pages, nkv, 16, 128] prefilled with random bits.

attn2 (cute_ops page, attn2 contract: 8 query rows per request, any L >= 8,
head_dim 64, 8 q heads per KV head, an optional window):
  y         bf16 [8 R, 1152 nkv] ~ N(0, 1), the front's output rows whose q
            and gate columns attn2 reads (q and k heads come out of the
            front's norm with RMS 1, and v = x W_v has unit variance for
            x ~ N(0, 1), W ~ N(0, 0.011^2), K = 8192), optionally q scaled
            for peakier softmax;
  kv_cache  bf16 [pages, nkv, 16, 128] ~ N(0, 1);
  block_table int32 [R, ceil(max_model_len / 16)]: request r owns a random
            set of distinct pages (disjoint across requests and sets), the
            unused tail of each row points at page 0;
  seq_lens  int32 [R], per workload.

MuseRouting (cute_ops page, MuseRouting entry; 256 experts, top 8):
  logits    fp32 [b, 256] ~ N(0, 2^2) (router logits of b <= 8 tokens);
  bias      fp32 [256] ~ N(0, 0.05^2) (the correction bias); route_scale 2.5.

LayerFront (layer_front page, LayerFront.run; rows of 8192):
  x         bf16 or fp32 [rows, 8192] ~ N(0, 1) (the embedded tokens; the
            bf16 path is the eager embedding, the fp32 one the in-graph one);
  weight    bf16 [8192] = 1 + 0.1 N(0, 1) (the pre-QKV norm's gain), or none.
"""
from __future__ import annotations

import dataclasses
import math

import torch

HIDDEN = 8192
HEAD_DIM = 64
QHEADS_PER_KV = 8
PAGE_SLOTS = 16
SLOT_WIDTH = 128
EPS = 1e-6
ROPE_THETA = 10000.0
W_STD = 0.011


def n_cols(nkv: int) -> int:
    return 2 * (QHEADS_PER_KV * nkv + nkv) * HEAD_DIM


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    nkv: int
    pages: int
    table_rows: int
    pos_mode: str          # "uniform" | "consecutive"
    pos_lo: int
    pos_hi: int            # exclusive
    slot_mode: str         # "uniform" (one token) | "consecutive" | "distinct"
    slot_hi: int           # exclusive bound for the first / random slots
    wsets: int             # weight sets rotated per call
    outlier_p: float = 0.0  # probability that an x row is scaled x30
    force_outlier: bool = False
    index: int = 0

    @property
    def N(self) -> int:
        return n_cols(self.nkv)

    def algorithmic_bytes(self) -> int:
        """Bytes the front must move once per call: W, x, y, the cos|sin
        rows, positions + slots, and the K|V slots written."""
        M, N = self.M, self.N
        return (2 * N * HIDDEN + 2 * M * HIDDEN + 2 * M * N + 4 * HEAD_DIM * M
                + 16 * M + 2 * SLOT_WIDTH * M * self.nkv)


# The five workloads the front is measured and checked on.
C1 = Workload("m1_nkv1_n1152", M=1, nkv=1, pages=64, table_rows=4096,
              pos_mode="uniform", pos_lo=0, pos_hi=4096,
              slot_mode="uniform", slot_hi=1024, wsets=1, index=1)
C2 = Workload("m8_nkv2_n2304_draft", M=8, nkv=2, pages=512, table_rows=4104,
              pos_mode="consecutive", pos_lo=8, pos_hi=4096,
              slot_mode="consecutive", slot_hi=512 * 16 - 7, wsets=1, index=2)
C3 = Workload("m8_nkv8_n9216", M=8, nkv=8, pages=8192, table_rows=131072,
              pos_mode="uniform", pos_lo=0, pos_hi=131072,
              slot_mode="distinct", slot_hi=8192 * 16, wsets=4, index=3)
C4 = Workload("m16_nkv8_n9216_outliers", M=16, nkv=8, pages=16384,
              table_rows=32768, pos_mode="uniform", pos_lo=0, pos_hi=32768,
              slot_mode="distinct", slot_hi=16384 * 16, wsets=4,
              outlier_p=0.01, force_outlier=True, index=4)
WORKLOADS = {w.name: w for w in (C1, C2, C3, C4)}

SWEEP_M = (1, 2, 3, 4, 5, 8, 12, 16)
SWEEP_NKV = (1, 2, 4, 8)


def sweep(M: int, nkv: int, wsets: int = 32) -> Workload:
    """One point of the M x KV-heads sweep: cache of 64K slots, positions
    uniform in [0, 131072), random distinct slots."""
    return Workload(f"sweep_m{M}_nkv{nkv}", M=M, nkv=nkv, pages=4096,
                    table_rows=131072, pos_mode="uniform", pos_lo=0,
                    pos_hi=131072, slot_mode="distinct", slot_hi=4096 * 16,
                    wsets=wsets, index=5)


def seed_of(w: Workload, set_index: int) -> int:
    return 1000 * w.index + set_index


def rope_table(rows: int, theta: float = ROPE_THETA) -> torch.Tensor:
    """fp32 [rows, 64]: 32 cos | 32 sin, built in float64, stored as fp32."""
    pos = torch.arange(rows, dtype=torch.float64)[:, None]
    i = torch.arange(HEAD_DIM // 2, dtype=torch.float64)[None, :]
    ang = pos * torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * i / HEAD_DIM)
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).contiguous()


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_weights(w: Workload, set_index: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [N, 8192] ~ N(0, 0.011^2), drawn on the CPU (reproducible)."""
    g = _gen(seed_of(w, set_index) * 7919 + 1)
    W = torch.randn(w.N, HIDDEN, generator=g, dtype=torch.float32) * W_STD
    return W.to(torch.bfloat16).to(device)


def make_weights_on_device(w: Workload, set_index: int, device) -> torch.Tensor:
    """Same distribution drawn by the device's own generator (fast, for
    large rotated weight pools that are never checked element by element)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(w, set_index) * 7919 + 2)
    W = torch.empty(w.N, HIDDEN, dtype=torch.bfloat16, device=device)
    W.normal_(0.0, W_STD, generator=g)
    return W


def make_tokens(w: Workload, set_index: int = 0, device="cpu", M: int | None = None):
    """x, positions, slots for one call."""
    M = w.M if M is None else M
    g = _gen(seed_of(w, set_index) * 7919 + 3)
    x = torch.randn(M, HIDDEN, generator=g, dtype=torch.float32)
    if w.outlier_p > 0:
        hit = torch.rand(M, generator=g) < w.outlier_p
        if w.force_outlier:
            hit[int(torch.randint(0, M, (1,), generator=g))] = True
        x[hit] *= 30.0
    x = x.to(torch.bfloat16)
    if w.pos_mode == "consecutive":
        p0 = int(torch.randint(w.pos_lo, w.pos_hi, (1,), generator=g))
        positions = torch.arange(p0, p0 + M, dtype=torch.int64)
    else:
        positions = torch.randint(w.pos_lo, w.pos_hi, (M,), generator=g, dtype=torch.int64)
    if w.slot_mode == "consecutive":
        s0 = int(torch.randint(0, w.slot_hi, (1,), generator=g))
        slots = torch.arange(s0, s0 + M, dtype=torch.int64)
    elif w.slot_mode == "uniform":
        slots = torch.randint(0, w.slot_hi, (M,), generator=g, dtype=torch.int64)
    else:
        slots = torch.randperm(w.slot_hi, generator=g)[:M].to(torch.int64)
    assert int(positions.max()) < w.table_rows
    assert int(slots.max()) < w.pages * PAGE_SLOTS
    return x.to(device), positions.to(device), slots.to(device)


def make_cache(w: Workload, device="cpu", seed: int | None = None) -> torch.Tensor:
    """bf16 [pages, nkv, 16, 128] filled with random bit patterns."""
    g = _gen((seed_of(w, 0) if seed is None else seed) * 7919 + 4)
    n = w.pages * w.nkv * PAGE_SLOTS * SLOT_WIDTH
    bits = torch.randint(-32768, 32768, (n,), generator=g, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16).reshape(w.pages, w.nkv, PAGE_SLOTS, SLOT_WIDTH).to(device)


def bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 tensor's bit patterns (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def describe(w: Workload) -> dict:
    return {"workload": w.name, "M": w.M, "num_kv_heads": w.nkv, "N": w.N,
            "K": HIDDEN, "weight_sets": w.wsets, "cache_pages": w.pages,
            "table_rows": w.table_rows}


def rope_angle(pos: int, pair: int, theta: float = ROPE_THETA) -> float:
    """The rotation angle the table above encodes for (position, pair)."""
    return pos * math.pow(theta, -2.0 * pair / HEAD_DIM)


# ---------------------------------------------------------------- attn2 --

@dataclasses.dataclass(frozen=True)
class Attn2Workload:
    name: str
    nkv: int
    max_model_len: int
    lens: tuple            # context length L of each request (>= 8)
    window: int = 0        # 0: no sliding window
    sets: int = 1          # request sets on disjoint pages, rotated per call
    q_scale: float = 1.0
    index: int = 0

    @property
    def R(self) -> int:
        return len(self.lens)

    @property
    def pages_per_req(self) -> int:
        return (max(self.lens) + PAGE_SLOTS - 1) // PAGE_SLOTS

    @property
    def pages(self) -> int:
        return 1 + self.sets * self.R * self.pages_per_req

    @property
    def table_width(self) -> int:
        return (self.max_model_len + PAGE_SLOTS - 1) // PAGE_SLOTS

    @property
    def eff_window(self) -> int:
        """The window that matters: none when it covers max_model_len."""
        return 0 if self.window >= self.max_model_len else self.window

    def first_key(self, L: int) -> int:
        """Earliest key any of the request's 8 rows attends."""
        w = self.eff_window
        return max(0, L - 8 - w + 1) if w > 0 else 0

    def algorithmic_bytes(self) -> int:
        """Bytes one call must move: q and gate rows read, the output
        written, the K|V slots of every attended key read once per KV head,
        the block-table entries of the pages they sit in, and seq_lens."""
        nq = QHEADS_PER_KV * self.nkv
        rows = 8 * self.R
        b = 3 * rows * nq * HEAD_DIM * 2 + 4 * self.R
        for L in self.lens:
            lo = self.first_key(L)
            b += (L - lo) * self.nkv * SLOT_WIDTH * 2
            b += 4 * ((L + PAGE_SLOTS - 1) // PAGE_SLOTS - lo // PAGE_SLOTS)
        return b


# attn2 workloads: the verify step of one request (8 rows) with the 8 KV
# heads of the M = 8 front at 32K and at the full 128K context, two requests
# (M = 16) with mixed lengths, the 2-KV-head draft with a short context, and
# a sliding-window layer.
A1 = Attn2Workload("attn2_r1_nkv8_L32768", nkv=8, max_model_len=131072, lens=(32768,),
                   sets=16, index=11)
A2 = Attn2Workload("attn2_r2_nkv8_L30000_9001", nkv=8, max_model_len=32768,
                   lens=(30000, 9001), sets=12, index=12)
A3 = Attn2Workload("attn2_r1_nkv2_L1500_draft", nkv=2, max_model_len=2048, lens=(1500,),
                   sets=64, index=13)
A4 = Attn2Workload("attn2_r2_nkv8_win4096", nkv=8, max_model_len=131072, lens=(20000, 4100),
                   window=4096, sets=32, index=14)
A5 = Attn2Workload("attn2_r1_nkv8_L131072", nkv=8, max_model_len=131072, lens=(131072,),
                   sets=3, index=15)
A0 = Attn2Workload("attn2_r3_nkv2_small", nkv=2, max_model_len=4096, lens=(300, 41, 8),
                   q_scale=3.0, index=10)
ATTN2_WORKLOADS = {a.name: a for a in (A0, A1, A2, A3, A4, A5)}


def make_attn2_y(a: Attn2Workload, set_index: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [8 R, 1152 nkv] rows of the front's output; q columns scaled by
    q_scale."""
    g = _gen((1000 * a.index + set_index) * 7919 + 5)
    y = torch.randn(8 * a.R, n_cols(a.nkv), generator=g, dtype=torch.float32)
    y[:, :QHEADS_PER_KV * a.nkv * HEAD_DIM] *= a.q_scale
    return y.to(torch.bfloat16).to(device)


def attn2_views(y: torch.Tensor, nkv: int):
    """(q, gate) column views of the front's output rows: [q | k | v | gate]."""
    nq = QHEADS_PER_KV * nkv * HEAD_DIM
    g0 = nq + 2 * nkv * HEAD_DIM
    return y[:, :nq], y[:, g0:g0 + nq]


def make_attn2_cache(a: Attn2Workload, device="cpu") -> torch.Tensor:
    """bf16 [pages, nkv, 16, 128] ~ N(0, 1); on a device, drawn there."""
    shape = (a.pages, a.nkv, PAGE_SLOTS, SLOT_WIDTH)
    if str(device) == "cpu":
        return torch.randn(shape, generator=_gen(1000 * a.index * 7919 + 6)).to(torch.bfloat16)
    g = torch.Generator(device=device)
    g.manual_seed(1000 * a.index * 7919 + 7)
    c = torch.empty(shape, dtype=torch.bfloat16, device=device)
    c.normal_(0.0, 1.0, generator=g)
    return c


def make_attn2_table(a: Attn2Workload, set_index: int = 0) -> torch.Tensor:
    """int32 [R, table_width]: set s, request r owns pages drawn without
    replacement from its own disjoint block, in random order."""
    g = _gen(1000 * a.index * 7919 + 8)
    perm = torch.randperm(a.pages - 1, generator=g) + 1   # page 0 is the filler
    P = a.pages_per_req
    bt = torch.zeros(a.R, a.table_width, dtype=torch.int32)
    for r in range(a.R):
        start = (set_index * a.R + r) * P
        bt[r, :P] = perm[start:start + P].to(torch.int32)
    return bt


def make_attn2_lens(a: Attn2Workload) -> torch.Tensor:
    assert all(8 <= L <= a.max_model_len for L in a.lens)
    return torch.tensor(a.lens, dtype=torch.int32)


def describe_attn2(a: Attn2Workload) -> dict:
    return {"workload": a.name, "requests": a.R, "query_rows": 8 * a.R, "num_kv_heads": a.nkv,
            "seq_lens": list(a.lens), "max_model_len": a.max_model_len, "window": a.window,
            "cache_pages": a.pages}


# ---------------------------------------------------------- LayerFront --

@dataclasses.dataclass(frozen=True)
class LayerFrontWorkload:
    name: str
    rows: int
    fp32_input: bool
    weight: bool = True
    aux: bool = True
    index: int = 0

    def algorithmic_bytes(self) -> int:
        """x read, stream (+ aux) written as fp32, out written as bf16, the
        weight read once."""
        n = self.rows * HIDDEN
        return (n * (4 if self.fp32_input else 2) + n * 4 * (2 if self.aux else 1) + n * 2
                + (2 * HIDDEN if self.weight else 0))


LF1 = LayerFrontWorkload("lf_m16_bf16_w_aux", rows=16, fp32_input=False, index=21)
LF2 = LayerFrontWorkload("lf_m8_f32_w", rows=8, fp32_input=True, aux=False, index=22)
LF3 = LayerFrontWorkload("lf_m1_bf16_w", rows=1, fp32_input=False, aux=False, index=23)
LAYER_FRONT_WORKLOADS = {w.name: w for w in (LF1, LF2, LF3)}


def make_lf_x(w: LayerFrontWorkload, set_index: int = 0, device="cpu") -> torch.Tensor:
    g = _gen((1000 * w.index + set_index) * 7919 + 9)
    x = torch.randn(w.rows, HIDDEN, generator=g)
    return (x if w.fp32_input else x.to(torch.bfloat16)).to(device)


def make_lf_weight(w: LayerFrontWorkload, device="cpu"):
    if not w.weight:
        return None
    g = _gen(1000 * w.index * 7919 + 10)
    return (1.0 + 0.1 * torch.randn(HIDDEN, generator=g)).to(torch.bfloat16).to(device)


def describe_layer_front(w: LayerFrontWorkload) -> dict:
    return {"workload": w.name, "rows": w.rows, "hidden": HIDDEN,
            "x_dtype": "fp32" if w.fp32_input else "bf16", "weight": w.weight, "aux": w.aux}


# ------------------------------------------------------------- routing --

@dataclasses.dataclass(frozen=True)
class RouteWorkload:
    name: str
    tokens: int
    route_scale: float = 2.5
    index: int = 0

    def algorithmic_bytes(self) -> int:
        """logits and bias read, ids and weights written."""
        return 4 * 256 * self.tokens + 4 * 256 + 2 * 4 * 8 * self.tokens


RT1 = RouteWorkload("route_b8", tokens=8, index=31)
RT2 = RouteWorkload("route_b1", tokens=1, index=32)
ROUTE_WORKLOADS = {w.name: w for w in (RT1, RT2)}


def make_route_inputs(w: RouteWorkload, set_index: int = 0, device="cpu"):
    g = _gen((1000 * w.index + set_index) * 7919 + 11)
    logits = torch.randn(w.tokens, 256, generator=g) * 2.0
    bias = torch.randn(256, generator=g) * 0.05
    return logits.to(device), bias.to(device)
