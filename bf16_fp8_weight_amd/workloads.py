"""Seeded synthetic workloads for parameter preparation.

This module holds the five workload shapes, their seeded input generators and
the packing helper that assigns destination offsets (the part of the
controller's static transfer schedule that says where each output lands). It
holds none of the preparation arithmetic: no amax, no scale, no FP8 cast. The
GPU library and the CPU oracle both receive exactly the bytes made here.

Sources for the shapes: the page "Weight transfer for RL post-training in
under 2 seconds" (section "Task pipeline": each parameter tensor is a task;
preparation rebuilds the full weight from FSDP shards, fuses projections and
quantizes; section "GPU memory usage control") names Kimi-K2 and BF16 -> FP8
but gives no per-tensor shapes; the shapes below are the standard
architectures named by the workloads (a hidden-1024 dense layer, a 7B-shaped
dense model, one GPU's share of a Kimi-K2 MoE layer, a ragged stress set, and
a Kimi-K2 MLA attention stack with many small tensors).

Values are N(0, 0.02) drawn in fp32 and rounded to BF16 (round to nearest
even, torch's conversion) unless a workload says otherwise. FSDP placement is
read as a dim-0 split in rank order, torch.chunk style: ceil(R / n) rows per
shard, trailing shards smaller or empty.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

FP8 = "fp8"    # quantized to E4M3 with one fp32 scale per 128x128 tile
BF16 = "bf16"  # copied byte for byte

TILE = 128


@dataclass
class Part:
    """One source tensor (a fusion component) as its dim-0 shards."""

    name: str
    rows: int
    shards: List[torch.Tensor] = field(default_factory=list)
    shard_rows: List[int] = field(default_factory=list)


@dataclass
class OutputSpec:
    """One output tensor: components concatenated along dim 0, then packed."""

    name: str
    kind: str
    cols: int
    parts: List[Part]
    dst_offset: int = 0
    scale_offset: int = 0

    @property
    def rows(self) -> int:
        return sum(p.rows for p in self.parts)

    @property
    def elems(self) -> int:
        return self.rows * self.cols

    @property
    def n_tiles(self) -> int:
        return ceil_div(self.rows, TILE) * ceil_div(self.cols, TILE) if self.kind == FP8 else 0

    @property
    def data_bytes(self) -> int:
        return self.elems * (1 if self.kind == FP8 else 2)

    @property
    def scale_bytes(self) -> int:
        return 4 * self.n_tiles


@dataclass
class Workload:
    name: str
    outputs: List[OutputSpec]
    dst_bytes: int = 0
    shard_mem: str = "device"  # "device" or "host" (pinned)
    seed: int = 0
    arena: Optional[torch.Tensor] = None  # pinned host arena holding every shard (host workloads)

    @property
    def input_bytes(self) -> int:
        return sum(2 * o.elems for o in self.outputs)

    @property
    def fp8_elems(self) -> int:
        return sum(o.elems for o in self.outputs if o.kind == FP8)

    @property
    def copy_elems(self) -> int:
        return sum(o.elems for o in self.outputs if o.kind == BF16)

    @property
    def n_tiles(self) -> int:
        return sum(o.n_tiles for o in self.outputs)

    @property
    def output_bytes(self) -> int:
        return sum(o.data_bytes + o.scale_bytes for o in self.outputs)

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes that must cross HBM once: BF16 read + FP8/BF16 written + scales written."""
        return self.input_bytes + self.output_bytes


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def split_rows(rows: int, n: int) -> List[int]:
    """torch.chunk-style dim-0 split into exactly n shards (trailing may be empty)."""
    per = ceil_div(rows, n) if rows else 0
    out = []
    left = rows
    for _ in range(n):
        r = min(per, left)
        out.append(r)
        left -= r
    return out


def align_up(x: int, a: int) -> int:
    return ceil_div(x, a) * a


def pack(outputs: List[OutputSpec], align: int = 256, start: int = 0) -> int:
    """Assigns dst_offset / scale_offset back to back (data, then scales, per
    output, each aligned to `align` bytes). Returns the region size."""
    off = start
    for o in outputs:
        off = align_up(off, align)
        o.dst_offset = off
        off += o.data_bytes
        if o.kind == FP8:
            off = align_up(off, max(align, 4) if align >= 4 else 4)
            o.scale_offset = off
            off += o.scale_bytes
    return align_up(off, max(align, 1))


def metadata(wl: "Workload", with_ptrs: bool = True):
    """The metadata the controller collects for a workload: training
    parameters (name, shape, number of FSDP shards, where they live) and
    inference tensors (name, the training parameters fused into it, dtype).
    A training parameter is named "<inference tensor>/<component>"."""
    params, dsts = [], []
    for o in wl.outputs:
        comps = []
        for p in o.parts:
            nm = f"{o.name}/{p.name}"
            d = {"name": nm, "rows": p.rows, "cols": o.cols, "n_shards": len(p.shard_rows),
                 "shard_mem": 1 if wl.shard_mem == "host" else 0}
            if with_ptrs and p.shards:
                d["shard_ptrs"] = [s.data_ptr() if r else 0 for s, r in zip(p.shards, p.shard_rows)]
            params.append(d)
            comps.append(nm)
        dsts.append({"name": o.name, "components": comps, "dtype": 0 if o.kind == FP8 else 1})
    return params, dsts


# ---------------------------------------------------------------- generators
def _gen(device: str, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16(shape, g, device, std=0.02) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x.to(torch.bfloat16)


def _student_t3_bf16(shape, g, device, scale=0.02) -> torch.Tensor:
    # t(3) = Z / sqrt(chi2(3) / 3), chi2(3) a sum of three squared normals.
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    c = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        c.addcmul_(n, n)
    t = z / torch.sqrt(c / 3.0)
    return (t * scale).to(torch.bfloat16)


def _shard_into(part: Part, full: torch.Tensor, n_shards: int, alloc) -> None:
    """Splits a full tensor into dim-0 shards, each in its own allocation."""
    part.shard_rows = split_rows(part.rows, n_shards)
    r = 0
    part.shards = []
    for k in range(n_shards):
        rk = part.shard_rows[k]
        part.shards.append(alloc(full[r:r + rk]))
        r += rk


def _materialize(wl: Workload, device: str, fill) -> Workload:
    """Allocates and fills every shard. `fill(output, part, g)` returns the full
    BF16 tensor of the part; shards are then split off."""
    g = _gen(device if wl.shard_mem == "device" else "cpu", wl.seed)
    if wl.shard_mem == "host":
        # One pinned arena, shards laid out in table order (as an offloaded
        # flat parameter would be), each shard start aligned to 256 bytes.
        total = 0
        for o in wl.outputs:
            for p in o.parts:
                for rk in p.shard_rows:
                    total = align_up(total, 256) + 2 * rk * o.cols
        arena = torch.empty(max(total, 256), dtype=torch.uint8)
        if torch.cuda.is_available():
            arena = arena.pin_memory()
        wl.arena = arena
        cursor = [0]

        def host_alloc(src: torch.Tensor) -> torch.Tensor:
            n = src.numel() * 2
            off = align_up(cursor[0], 256)
            view = arena[off:off + n].view(torch.bfloat16).view(src.shape)
            view.copy_(src)
            cursor[0] = off + n
            return view

        alloc = host_alloc
        gen_device = "cpu"
    else:
        def alloc(src: torch.Tensor) -> torch.Tensor:
            return src.clone()

        gen_device = device
    for o in wl.outputs:
        for p in o.parts:
            full = fill(o, p, g, gen_device)
            n = len(p.shard_rows)
            _shard_into(p, full, n, alloc)
            del full
    return wl


def _matrix_parts(names, rows, n_shards):
    ps = []
    for nm, r in zip(names, rows):
        p = Part(nm, r)
        p.shard_rows = split_rows(r, n_shards)
        ps.append(p)
    return ps


# ---------------------------------------------------------------- workloads
def dense_layer_h1024(device="cpu", materialize=True) -> Workload:
    """One dense transformer layer, hidden 1024: Wq, Wk, Wv [1024x1024] fused to
    qkv [3072x1024]; gate, up [2816x1024] fused to gate_up [5632x1024];
    down [1024x2816]; 4 row shards each; packed back to back."""
    outs = [
        OutputSpec("qkv", FP8, 1024, _matrix_parts(["Wq", "Wk", "Wv"], [1024] * 3, 4)),
        OutputSpec("gate_up", FP8, 1024, _matrix_parts(["gate", "up"], [2816] * 2, 4)),
        OutputSpec("down", FP8, 2816, _matrix_parts(["down"], [1024], 4)),
    ]
    wl = Workload("dense_layer_h1024", outs, seed=1001)
    wl.dst_bytes = pack(outs)
    if materialize:
        _materialize(wl, device, lambda o, p, g, d: _normal_bf16((p.rows, o.cols), g, d))
    return wl


def dense_7b(device="cpu", materialize=True, layers=32) -> Workload:
    """7B-shaped dense model: hidden 4096, intermediate 11008; per layer qkv
    [12288x4096] (fused), o [4096x4096], gate_up [22016x4096] (fused), down
    [4096x11008]; 8 row shards; two RMSNorm [4096] per layer plus the final
    norm are BF16 pass-through copies."""
    outs = []
    for l in range(layers):
        outs.append(OutputSpec(f"l{l}.qkv", FP8, 4096, _matrix_parts(["q", "k", "v"], [4096] * 3, 8)))
        outs.append(OutputSpec(f"l{l}.o", FP8, 4096, _matrix_parts(["o"], [4096], 8)))
        outs.append(OutputSpec(f"l{l}.gate_up", FP8, 4096, _matrix_parts(["gate", "up"], [11008] * 2, 8)))
        outs.append(OutputSpec(f"l{l}.down", FP8, 11008, _matrix_parts(["down"], [4096], 8)))
        outs.append(OutputSpec(f"l{l}.attn_norm", BF16, 1, _matrix_parts(["w"], [4096], 8)))
        outs.append(OutputSpec(f"l{l}.mlp_norm", BF16, 1, _matrix_parts(["w"], [4096], 8)))
    outs.append(OutputSpec("final_norm", BF16, 1, _matrix_parts(["w"], [4096], 8)))
    wl = Workload(f"dense_7b_{layers}l", outs, seed=1002)
    wl.dst_bytes = pack(outs)
    if materialize:
        _materialize(wl, device, lambda o, p, g, d: _normal_bf16((p.rows, o.cols), g, d))
    return wl


def kimi_k2_expert_share(device="cpu", materialize=True, experts=96) -> Workload:
    """One GPU's share of a Kimi-K2-shaped MoE layer: per expert, w1 and w3
    [2048x7168] fused to gate_up [4096x7168] and w2 [7168x2048]; 8 row shards
    per tensor; per-expert packed slots [gate_up][scales][w2][scales]."""
    outs = []
    for e in range(experts):
        outs.append(OutputSpec(f"e{e}.gate_up", FP8, 7168, _matrix_parts(["w1", "w3"], [2048, 2048], 8)))
        outs.append(OutputSpec(f"e{e}.w2", FP8, 2048, _matrix_parts(["w2"], [7168], 8)))
    wl = Workload(f"kimi_k2_moe_{experts}experts", outs, seed=1003)
    wl.dst_bytes = pack(outs)
    if materialize:
        _materialize(wl, device, lambda o, p, g, d: _normal_bf16((p.rows, o.cols), g, d))
    return wl


def _draw_dim(g: torch.Generator, hi: int) -> int:
    while True:
        v = int(torch.randint(1, hi + 1, (1,), generator=g).item())
        if v % TILE != 0:
            return v


def e4m3_grid() -> List[float]:
    """The 127 non-negative finite E4M3 magnitudes (OCP FP8 E4M3: bias 7,
    S.1111.111 is NaN), ascending. Used only to plant exact grid points and
    midpoints in stress inputs."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for E in range(1, 16):
        for m in range(8):
            if E == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (E - 7))
    return vals


def ragged_stress(device="cpu", materialize=True, n_tensors=512, max_dim=3000, seed=1004) -> Workload:
    """Quantization stress set: n_tensors unfused tensors with rows, cols drawn
    uniformly from 1..max_dim (redrawn on multiples of 128); shard count from
    {1, 2, 3, 4, 8}; values Student-t(3) x 0.02 with 0.1% outliers x100; 2% of
    tiles zeroed; about 1% of tiles planted with amax = 448 * 2^k (k in
    [-20, 0]) plus exact E4M3 midpoints and values at and just below amax."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    outs = []
    for t in range(n_tensors):
        r = _draw_dim(g, max_dim)
        c = _draw_dim(g, max_dim)
        n = [1, 2, 3, 4, 8][int(torch.randint(0, 5, (1,), generator=g).item())]
        outs.append(OutputSpec(f"t{t}", FP8, c, _matrix_parts(["w"], [r], n)))
    wl = Workload(f"ragged_stress_{n_tensors}", outs, seed=seed)
    wl.dst_bytes = pack(outs)
    if materialize:
        grid = torch.tensor(e4m3_grid(), dtype=torch.float64)
        mids = ((grid[1:] + grid[:-1]) / 2).to(torch.float32)  # exact in fp32 and bf16

        def fill(o, p, gg, d):
            x = _student_t3_bf16((p.rows, o.cols), gg, d).to(torch.float32)
            out_mask = torch.rand((p.rows, o.cols), generator=gg, device=d) < 0.001
            x = torch.where(out_mask, x * 100.0, x)
            tr, tc = ceil_div(p.rows, TILE), ceil_div(o.cols, TILE)
            u = torch.rand((tr, tc), generator=gg, device=d)
            ks = torch.randint(-20, 1, (tr, tc), generator=gg, device=d)
            zero_t = (u < 0.02).nonzero().tolist()
            plant_t = ((u >= 0.02) & (u < 0.03)).nonzero().tolist()
            for (i, j) in zero_t:
                x[i * TILE:(i + 1) * TILE, j * TILE:(j + 1) * TILE] = 0.0
            md = mids.to(d)
            for (i, j) in plant_t:
                k = int(ks[i, j].item())
                blk = x[i * TILE:(i + 1) * TILE, j * TILE:(j + 1) * TILE]
                amax = 448.0 * 2.0 ** k
                # rescale the tile strictly inside (-amax, amax), then plant
                peak = float(blk.abs().max().item())
                if peak > 0:
                    blk.mul_(0.9 * amax / peak)
                vals = torch.cat([
                    torch.tensor([amax, -amax], device=d),
                    md * 2.0 ** k,
                    -md[:16] * 2.0 ** k,
                ])
                # one BF16 ulp below amax, both signs
                below = torch.tensor([amax], dtype=torch.float32, device=d).to(torch.bfloat16)
                below = (below.view(torch.int16) - 1).view(torch.bfloat16).to(torch.float32)
                vals = torch.cat([vals, below, -below])
                n_el = blk.numel()
                m = min(n_el, vals.numel())
                idx = torch.randperm(n_el, generator=gg, device=d)
                flat = blk.reshape(-1).clone()
                flat[idx[:m]] = vals[:m]
                flat[idx[0]] = amax  # the tile's amax is present even in tiny tiles
                blk.copy_(flat.reshape(blk.shape))
            return x.to(torch.bfloat16)

        # materialize per output with the shared generator (device draws)
        gdev = _gen(device, seed + 7)
        for o in outs:
            for p in o.parts:
                full = fill(o, p, gdev, device)
                _shard_into(p, full, len(p.shard_rows), lambda s: s.clone())
    return wl


def mla_many_small(device="cpu", materialize=True, layers=8, n_small=4000, host=True) -> Workload:
    """Kimi-K2-style MLA attention stack: per layer q_a [1536x7168], q_b
    [12288x1536], kv_a [576x7168], kv_b [16384x512], o [7168x8192] quantized,
    plus n_small small BF16 pass-through tensors: one router [384x7168] per
    layer and the rest [7168] norm/bias vectors; 8 row shards each; shards in
    pinned host memory when host=True (CPU-offloaded FSDP)."""
    outs = []
    n_vec = n_small - layers
    per_layer = [n_vec // layers + (1 if l < n_vec % layers else 0) for l in range(layers)]
    for l in range(layers):
        for nm, r, c in [("q_a", 1536, 7168), ("q_b", 12288, 1536), ("kv_a", 576, 7168),
                         ("kv_b", 16384, 512), ("o", 7168, 8192)]:
            outs.append(OutputSpec(f"l{l}.{nm}", FP8, c, _matrix_parts([nm], [r], 8)))
        outs.append(OutputSpec(f"l{l}.router", BF16, 7168, _matrix_parts(["router"], [384], 8)))
        for v in range(per_layer[l]):
            outs.append(OutputSpec(f"l{l}.vec{v}", BF16, 1, _matrix_parts(["w"], [7168], 8)))
    wl = Workload(f"mla_{layers}l_{n_small}small", outs, seed=1005, shard_mem="host" if host else "device")
    wl.dst_bytes = pack(outs)
    if materialize:
        _materialize(wl, device, lambda o, p, g, d: _normal_bf16((p.rows, o.cols), g, d))
    return wl


# ------------------------------------------------------- token activations
@dataclass
class ActWorkload:
    """Token activations for block-scaled FP8 quantization (dispatch sender).

    x: [tokens, hidden] BF16. index: int32 output-row -> token map (None: row
    i is token i). Outputs: n_out rows; with `interleaved` each row is one
    send-buffer slot of `slot` bytes holding the row's FP8 codes then its
    scales, else codes and scales are separate dense arrays."""

    name: str
    tokens: int
    hidden: int
    x: Optional[torch.Tensor]
    index: Optional[torch.Tensor]
    n_out: int
    interleaved: bool
    seed: int

    @property
    def nb(self) -> int:
        return ceil_div(self.hidden, TILE)

    @property
    def q_stride(self) -> int:
        return self.slot if self.interleaved else self.hidden

    @property
    def s_stride(self) -> int:
        return self.slot if self.interleaved else 4 * self.nb

    @property
    def slot(self) -> int:
        return align_up(self.hidden + 4 * self.nb, 16)

    @property
    def input_bytes(self) -> int:
        return 2 * self.n_out * self.hidden

    @property
    def algorithmic_bytes(self) -> int:
        """Per output row: its BF16 token read, FP8 codes and scales written,
        plus its 4-byte index when rows are gathered."""
        return self.n_out * (3 * self.hidden + 4 * self.nb + (4 if self.index is not None else 0))


def _activations(shape, g, device, outlier_channels=8) -> torch.Tensor:
    """Student-t(3) values of unit scale with a few outlier channels x50 (the
    heavy-tailed, channel-outlier shape of transformer hidden states)."""
    t = _student_t3_bf16(shape, g, device, scale=1.0).float()
    ch = torch.randint(0, shape[1], (outlier_channels,), generator=g, device=device)
    t[:, ch] *= 50.0
    return t.to(torch.bfloat16)


def act_dispatch(device="cpu", tokens=128, hidden=7168, topk=8, n_experts=384, seed=2001,
                 interleaved=True, materialize=True) -> ActWorkload:
    """MoE dispatch sender: each token goes to topk distinct experts drawn
    uniformly; output rows are (token, expert) pairs grouped by expert, so a
    token's activations appear topk times, each copy quantized into its slot."""
    g = _gen(device, seed)
    x = idx = None
    if materialize:
        x = _activations((tokens, hidden), g, device)
        experts = torch.rand((tokens, n_experts), generator=g, device=device).topk(topk, dim=1).indices
        order = torch.sort(experts.flatten(), stable=True).indices
        idx = (order // topk).to(torch.int32)
    wl = ActWorkload(f"act_dispatch_t{tokens}_top{topk}_h{hidden}", tokens, hidden, x, idx, tokens * topk,
                     interleaved, seed)
    if not materialize:
        wl.index = torch.empty(0, dtype=torch.int32)  # marks a gathered workload
    return wl


def act_tokens(device="cpu", tokens=4096, hidden=7168, seed=2002, materialize=True) -> ActWorkload:
    """A plain batch of tokens (no gather), codes and scales in separate arrays."""
    g = _gen(device, seed)
    x = _activations((tokens, hidden), g, device) if materialize else None
    return ActWorkload(f"act_tokens_t{tokens}_h{hidden}", tokens, hidden, x, None, tokens, False, seed)


WORKLOADS = {
    "dense_layer_h1024": dense_layer_h1024,
    "dense_7b": dense_7b,
    "kimi_k2_moe": kimi_k2_expert_share,
    "ragged_stress": ragged_stress,
    "mla_many_small": mla_many_small,
}


def custom(shapes, kind=FP8, n_shards=1, seed=7, device="cpu", fused=False, dist="normal",
           align=256) -> Workload:
    """Small ad-hoc workload: `shapes` is a list of (rows, cols) components.
    With fused=True they form one output (same cols required)."""
    if fused:
        cols = shapes[0][1]
        assert all(c == cols for _, c in shapes)
        outs = [OutputSpec("fused", kind, cols, _matrix_parts([f"c{i}" for i in range(len(shapes))],
                                                              [r for r, _ in shapes], n_shards))]
    else:
        outs = [OutputSpec(f"t{i}", kind, c, _matrix_parts(["w"], [r], n_shards)) for i, (r, c) in enumerate(shapes)]
    wl = Workload("custom", outs, seed=seed)
    wl.dst_bytes = pack(outs, align=align)
    gen = _normal_bf16 if dist == "normal" else _student_t3_bf16
    _materialize(wl, device, lambda o, p, g, d: gen((p.rows, o.cols), g, d))
    return wl
