"""Workload registry: the five video-shaped VSA2 problems.

Grids are (T, Y, X) latent cells; tokens are stored in cube-tiled order (4x4x4
cubes of 64 tokens, each made of eight 2x2x2 sub-cubes of 8 tokens).  A grid
whose sides are not multiples of 4 is padded up to whole cubes; L counts the
slots of the padded grid.  ``topk`` is the average number of KV cubes per query cube, so the
per-head budget is nb * topk selected (query cube, KV cube) pairs
(paper "Improving Video Sparse Attention with Fine-grained Router and Sparse
Rebasing", §2.2 Eq.(8)-(9)).
"""

from dataclasses import dataclass, field

CUBE = 64          # tokens per 4x4x4 cube (block size of the block-sparse attention)
SUB = 8            # tokens per 2x2x2 router pooling sub-cube
G = CUBE // SUB    # pooled tokens per cube


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    grid: tuple            # (T, Y, X)
    batch: int
    heads: int
    head_dim: int
    dtype: str             # "f32" or "bf16"
    topk: int
    gen: str               # "sinusoid" or "lowrank"
    alpha: float = 0.5     # weight of the structured component
    skew: bool = False     # heavy-tailed per-query-cube scale
    train: bool = False    # forward + backward
    extra_topk: tuple = field(default_factory=tuple)
    block: int = 64        # attention block: 64 (a 4x4x4 cube) or 128 (4x4x8, two x-adjacent cubes)
    text: int = 0          # MMDiT text tokens joining the fine branch (rows after the video slots)
    router: str = "vsa2"   # "vsa2" (fine-grained, per-sequence TopK) or "vsa" (coarse scores, TopK per row)

    @property
    def pgrid(self):
        """The grid padded up to whole attention blocks along each axis (§2.2
        "Kernel Implementation"); equal to ``grid`` when it divides."""
        mult = (4, 4, 4 * (self.block // CUBE))
        return tuple(-(-n // m) * m for n, m in zip(self.grid, mult))

    @property
    def padded(self):
        return self.pgrid != tuple(self.grid)

    @property
    def L(self):
        """Token slots per (batch, head): the padded grid's size."""
        t, y, x = self.pgrid
        return t * y * x

    @property
    def rows(self):
        """Token rows per (batch, head) of the attention tensors: the video
        slots, then the text tokens padded to a multiple of 64."""
        return self.L + 64 * -(-self.text // 64)

    @property
    def L_real(self):
        """Real tokens per (batch, head) (pad slots excluded)."""
        t, y, x = self.grid
        return t * y * x

    @property
    def nb(self):
        """4x4x4 cubes per (batch, head)."""
        return self.L // CUBE

    @property
    def nblk(self):
        """Attention blocks per (batch, head): the rows and columns of the
        router scores and of the selection."""
        return self.L // self.block

    @property
    def d_model(self):
        return self.heads * self.head_dim

    def budget(self, topk=None):
        k = self.topk if topk is None else topk
        return min(self.nblk * k, self.nblk * self.nblk)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, (8, 16, 16), 1, 2, 64, "f32", 8, "sinusoid", alpha=1.0),
        Workload("short", 2, (16, 32, 64), 1, 20, 128, "bf16", 64, "lowrank"),
        Workload("train480", 3, (28, 32, 52), 1, 20, 128, "bf16", 64, "lowrank", train=True),
        Workload("infer720", 4, (44, 48, 104), 1, 20, 128, "bf16", 64, "lowrank", extra_topk=(128,)),
        Workload("train720", 5, (44, 48, 104), 1, 20, 128, "bf16", 64, "lowrank", skew=True, train=True),
        # the 720p training problem on a grid one short of whole cubes along
        # every axis: padded to the same 44 x 48 x 104 slots (3.5% pad slots)
        Workload("train720pad", 6, (43, 47, 103), 1, 20, 128, "bf16", 64, "lowrank", skew=True, train=True),
        # the 720p training problem with 128-token blocks (4x4x8, two
        # x-adjacent cubes; G = 16): the blog's inferred setting, top64
        Workload("train720b128", 7, (44, 48, 104), 1, 20, 128, "bf16", 64, "lowrank", skew=True, train=True,
                 block=128),
        # the 720p training problem with 512 MMDiT text tokens in the fine branch
        Workload("train720text", 8, (44, 48, 104), 1, 20, 128, "bf16", 64, "lowrank", skew=True, train=True,
                 text=512),
        # the 720p training problem under the VSA router the paper compares
        # against: coarse scores, top128 per query block
        Workload("train720vsa", 9, (44, 48, 104), 1, 20, 128, "bf16", 128, "lowrank", skew=True, train=True,
                 router="vsa"),
    ]
}


def text_pairs(w: Workload):
    """64 x 64 tile pairs the MMDiT text rows add per (batch, head): every video
    query cube against every text cube, every text query cube against every
    video and text cube."""
    ntc = -(-w.text // 64)
    return 2 * w.nb * ntc + ntc * ntc


def flops(w: Workload, topk=None):
    """Algorithmic FLOPs of one call of each op, counting selected blocks only.

    Fine branch: 4 * B^2 * d per selected block pair forward (QK^T and PV),
    2.5x that backward (five BxBxd GEMMs).  Router: two pooled GEMMs (LSE pass
    and score pass), each 2 * (L/8)^2 * d, as in the paper's App. B cost model.
    Coarse: dense attention over the nb block tokens, 4 * nb^2 * d forward.
    MMDiT text rows add their 64 x 64 tile pairs (text_pairs) to the fine
    branch.
    """
    k = w.budget(topk)
    bh = w.batch * w.heads
    d = w.head_dim
    lr = w.L // SUB
    pair = 4 * w.block * w.block * d
    tpair = text_pairs(w) * 4 * CUBE * CUBE * d
    # the VSA router's two passes run over the nb coarse tokens
    rt = w.nblk if w.router == "vsa" else lr
    return {
        "fine_fwd": bh * (k * pair + tpair),
        "fine_bwd": bh * (k * pair + tpair) * 5 // 2,
        "router": bh * 2 * 2 * rt * rt * d,
        "coarse_fwd": bh * 4 * w.nblk * w.nblk * d,
        "coarse_bwd": bh * 10 * w.nblk * w.nblk * d,
        "gate_fwd": 2 * w.batch * w.L * w.d_model * w.heads,
        "gate_bwd": 4 * w.batch * w.L * w.d_model * w.heads,
    }


def kernel_flops(w: Workload, topk=None):
    """Algorithmic FLOPs credited to each timed kernel of one call.

    The fine backward's five GEMMs per selected block pair are split between
    its two kernels: the dK/dV kernel computes S^T, dP^T, dV and dK (four of
    them, 8 * B^2 * d); the dQ kernel is credited with the dQ GEMM only
    (2 * B^2 * d), its recomputation of S and dP is not counted.  Each router
    pass is one pooled GEMM of 2 * (L/8)^2 * d per (batch, head).
    """
    k = w.budget(topk)
    bh = w.batch * w.heads
    d = w.head_dim
    lr = w.L // SUB
    gemm = 2 * w.block * w.block * d
    tg = text_pairs(w) * 2 * CUBE * CUBE * d      # text tile pairs, one GEMM each
    rt = w.nblk if w.router == "vsa" else lr
    return {
        "fine_fwd": bh * (k * 2 * gemm + 2 * tg),
        "bwd_dkdv": bh * (k * 4 * gemm + 4 * tg),
        "bwd_dq": bh * (k * gemm + tg),
        "router_lse": bh * 2 * rt * rt * d,
        "router_scores": bh * 2 * rt * rt * d,
    }


def gather_bytes(w: Workload, topk=None):
    """Bytes one launch of each timed kernel gathers when no tile is reused.

    This is a property of the tile-gathering design, not a floor: the fine
    kernels gather one B-row tile of two operands per selected block pair (K
    and V for the forward and the dQ kernel, Q and dO plus the B rows' (lse,
    delta) pairs for the dK/dV kernel), plus the index entry, and read or
    write the per-token tensors that stay with the block once.  The dK/dV and
    dQ kernels also read the coarse branch's per-block gradient rows.  A
    router pass reads the pooled Q_r and K_r once and writes the per-row LSE;
    the score pass also writes the nb x nb cube scores.
    """
    k = w.budget(topk)
    bh = w.batch * w.heads
    d = w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    tile = w.block * d * esz
    tok = w.rows * d * esz       # one per-token tensor of one (batch, head), text rows included
    ptr = (w.nblk + 1) * 4
    lr = w.L // SUB
    tp = text_pairs(w)           # text tile pairs: one 64-row tile of each of two operands
    t64 = CUBE * d * esz
    return {
        "fine_fwd": bh * (k * (2 * tile + 4) + tp * 2 * t64 + 2 * tok + w.rows * 4 + ptr),
        "bwd_dkdv": bh * (k * (2 * tile + w.block * 8 + 4) + tp * (2 * t64 + CUBE * 8) + 4 * tok
                          + 2 * w.nblk * d * 4 + ptr),
        "bwd_dq": bh * (k * (2 * tile + 4) + tp * 2 * t64 + 3 * tok + w.rows * 8 + w.nblk * d * 4 + ptr),
        "router_lse": bh * (2 * lr * d * esz + lr * 4),
        "router_scores": bh * (2 * lr * d * esz + lr * 4 + w.nblk * w.nblk * 4),
    }


def compulsory_bytes(w: Workload, topk=None):
    """Bytes one launch of each timed kernel must move at least: every input
    read once and every output written once, whatever the tiling.

    Forward: Q, K, V read, O_f and the LSE written, the CSR read.  dK/dV: Q,
    K, V, dO and the per-row (lse, delta) pairs read, dK and dV written, the
    CSC and the coarse per-block dK_c, dV_c rows read.  dQ: Q, K, V, dO, O_f
    and the LSE read, dQ and the per-row pairs written, the CSR and dQ_c read.
    Router passes as in gather_bytes (they read each pooled operand once).
    """
    k = w.budget(topk)
    bh = w.batch * w.heads
    d = w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.rows * d * esz
    idx = k * 4 + (w.nblk + 1) * 4
    crow = w.nblk * d * 4
    g = gather_bytes(w, topk)
    return {
        "fine_fwd": bh * (4 * tok + w.rows * 4 + idx),
        "bwd_dkdv": bh * (6 * tok + w.rows * 8 + idx + 2 * crow),
        "bwd_dq": bh * (6 * tok + w.rows * 4 + w.rows * 8 + idx + crow),
        "router_lse": g["router_lse"],
        "router_scores": g["router_scores"],
    }


def op_bytes(w: Workload, topk=None):
    """Bytes the memory-bound calls move, as implemented (each pass counted).

    route: both router passes (gather_bytes of each).  topk: the per-sequence
    TopK reads the nb x nb fp32 scores five times (three radix histogram
    passes, the per-row count and the compaction), writes the CSR and the
    selection bitmap, then reads the bitmap twice and writes the CSC (the
    per-row TopK of the VSA router baseline also reads every score five times:
    four 8-bit radix passes per row and the compaction).  A forward-only
    workload calls TopK without the CSC, which then builds no bitmap and no
    CSC: the five score passes and the CSR only.  pool: Q, K, V read once,
    the router and coarse operands written.
    """
    k = w.budget(topk)
    bh = w.batch * w.heads
    d = w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    nb = w.nblk
    scores = nb * nb * 4
    csc = w.train  # the CSC side (bitmap, column lists) feeds only the backward
    bitmap = nb * 2 * ((nb + 63) // 64) * 4 if csc else 0
    lists = (2 if csc else 1) * (k * 4 + (nb + 1) * 4)
    passes = 5
    g = gather_bytes(w, topk)
    nbp = -(-nb // 64) * 64
    return {
        "route": g["router_lse"] + g["router_scores"],
        "topk": bh * (passes * scores + 3 * bitmap + lists),
        "pool": bh * (3 * w.L * d * esz + (2 * (w.L // SUB) + 3 * nbp) * d * esz),
    }
