"""Thin ctypes binding of libvsa2.so (include/vsa2.h).

Functions keep the C names and only marshal arguments: torch tensors become
device pointers, the stream defaults to torch's current stream, and a non-zero
status raises.  All computation happens in the HIP library; there is no other
code path.  Loading fails loudly if the library has not been built.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa2.so")

VSA2_OK, VSA2_E_ARG, VSA2_E_SHAPE, VSA2_E_WORKSPACE, VSA2_E_HIP, VSA2_E_UNSUPPORTED, VSA2_E_SCRATCH = range(7)
VSA2_F32, VSA2_BF16 = 0, 1
OP_POOL, OP_ROUTE, OP_TOPK, OP_PLAN, OP_FWD, OP_BWD, OP_COARSE, OP_COARSE_BWD, OP_ROUTE_COARSE, OP_TOPK_ROW = range(10)
K_FINE_FWD, K_BWD_DKDV, K_BWD_DQ, K_ROUTER_LSE, K_ROUTER_SCORES = range(5)


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("lat_t", ctypes.c_int32),
        ("lat_y", ctypes.c_int32),
        ("lat_x", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("block_tokens", ctypes.c_int32),
        ("text_tokens", ctypes.c_int32),
        ("router_pool", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_PP = ctypes.POINTER(Problem)

_SIGS = {
    "vsa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vsa2_workspace_size": (ctypes.c_int, [_PP, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "vsa2_pooled_size": (ctypes.c_int, [_PP, ctypes.POINTER(_SZ)]),
    "vsa2_saved_size": (ctypes.c_int, [_PP, ctypes.POINTER(_SZ)]),
    "vsa2_budget": (ctypes.c_int, [_PP, _I32, ctypes.POINTER(ctypes.c_int64)]),
    "vsa2_pool": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "vsa2_route": (ctypes.c_int, [_PP, _P, _P, _P, _SZ, _P]),
    "vsa2_route_noalloc": (ctypes.c_int, [_PP, _P, _P, _P]),
    "vsa2_route_noalloc_limit": (ctypes.c_int, [ctypes.POINTER(_SZ)]),
    "vsa2_sched_size": (ctypes.c_int, [_PP, _I32, ctypes.POINTER(_SZ)]),
    "vsa2_topk_per_seq": (ctypes.c_int, [_PP, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "vsa2_route_coarse": (ctypes.c_int, [_PP, _P, _P, _P, _SZ, _P]),
    "vsa2_topk_per_row": (ctypes.c_int, [_PP, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "vsa2_plan_from_csr": (ctypes.c_int, [_PP, _I32, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "vsa2_sparse_attn_fwd": (ctypes.c_int, [_PP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "vsa2_sparse_attn_bwd": (ctypes.c_int, [_PP, _I32] + [_P] * 16 + [_SZ, _P]),
    "vsa2_coarse_gate": (ctypes.c_int, [_PP, _P, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "vsa2_coarse_gate_bwd": (ctypes.c_int, [_PP, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "vsa2_kernel_timer_start": (ctypes.c_int, [_I32, _I32]),
    "vsa2_kernel_timer_stop": (ctypes.c_int, [_I32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I32)]),
}

_lib = None


def lib():
    """The loaded library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m video_dit_trainable_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


class Vsa2Error(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({lib().vsa2_status_string(code).decode()})")


def _check(fn, code):
    if code != VSA2_OK:
        raise Vsa2Error(fn, code)


def problem(batch, heads, head_dim, grid, dtype, softmax_scale=0.0, block=64, text=0, router_pool=2):
    t, y, x = grid
    dt = {"bf16": VSA2_BF16, "f32": VSA2_F32, torch.bfloat16: VSA2_BF16, torch.float32: VSA2_F32}[dtype]
    return Problem(batch, heads, head_dim, t, y, x, dt, softmax_scale, block, text, router_pool)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _size(fn, *args):
    out = _SZ(0)
    _check(fn, getattr(lib(), fn)(*args, ctypes.byref(out)))
    return out.value


def workspace_size(p, op, topk=1, d_model=0):
    return _size("vsa2_workspace_size", ctypes.byref(p), op, topk, d_model)


def pooled_size(p):
    return _size("vsa2_pooled_size", ctypes.byref(p))


def saved_size(p):
    return _size("vsa2_saved_size", ctypes.byref(p))


def budget(p, topk):
    out = ctypes.c_int64(0)
    _check("vsa2_budget", lib().vsa2_budget(ctypes.byref(p), topk, ctypes.byref(out)))
    return out.value


def vsa2_pool(p, q, k, v, pooled, stream=None):
    _check("vsa2_pool", lib().vsa2_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pooled), _stream(stream)))


def vsa2_route(p, pooled, scores, ws, stream=None):
    _check("vsa2_route", lib().vsa2_route(ctypes.byref(p), _ptr(pooled), _ptr(scores), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vsa2_route_noalloc(p, pooled, scores, stream=None):
    _check("vsa2_route_noalloc", lib().vsa2_route_noalloc(ctypes.byref(p), _ptr(pooled), _ptr(scores),
                                                          _stream(stream)))


def route_noalloc_limit():
    out = _SZ(0)
    _check("vsa2_route_noalloc_limit", lib().vsa2_route_noalloc_limit(ctypes.byref(out)))
    return out.value


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def sched_size(p, topk):
    out = _SZ(0)
    _check("vsa2_sched_size", lib().vsa2_sched_size(ctypes.byref(p), topk, ctypes.byref(out)))
    return out.value


def vsa2_topk_per_seq(p, scores, topk, row_ptr, col_idx, col_ptr, row_idx, ws, stream=None, sched=None):
    _check("vsa2_topk_per_seq", lib().vsa2_topk_per_seq(
        ctypes.byref(p), _ptr(scores), topk, _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
        _ptr(sched), _nbytes(sched), _ptr(ws), _nbytes(ws), _stream(stream)))


def vsa2_route_coarse(p, pooled, scores, ws, stream=None):
    _check("vsa2_route_coarse", lib().vsa2_route_coarse(ctypes.byref(p), _ptr(pooled), _ptr(scores), _ptr(ws),
                                                        0 if ws is None else ws.numel() * ws.element_size(),
                                                        _stream(stream)))


def vsa2_topk_per_row(p, scores, topk, row_ptr, col_idx, col_ptr, row_idx, ws, stream=None, sched=None):
    _check("vsa2_topk_per_row", lib().vsa2_topk_per_row(
        ctypes.byref(p), _ptr(scores), topk, _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
        _ptr(sched), _nbytes(sched), _ptr(ws), _nbytes(ws), _stream(stream)))


def vsa2_plan_from_csr(p, topk, row_ptr, col_idx, col_ptr, row_idx, ws, stream=None, sched=None):
    _check("vsa2_plan_from_csr", lib().vsa2_plan_from_csr(
        ctypes.byref(p), topk, _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
        _ptr(sched), _nbytes(sched), _ptr(ws), _nbytes(ws), _stream(stream)))


def vsa2_sparse_attn_fwd(p, topk, q, k, v, row_ptr, col_idx, o_f, lse, ws=None, stream=None, sched=None):
    _check("vsa2_sparse_attn_fwd", lib().vsa2_sparse_attn_fwd(
        ctypes.byref(p), topk, _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx), _ptr(sched), _ptr(o_f),
        _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)))


def vsa2_sparse_attn_bwd(p, topk, q, k, v, o_f, lse, d_o, row_ptr, col_idx, col_ptr, row_idx, dqkv_c,
                         dq, dk, dv, ws, stream=None, sched=None):
    _check("vsa2_sparse_attn_bwd", lib().vsa2_sparse_attn_bwd(
        ctypes.byref(p), topk, _ptr(q), _ptr(k), _ptr(v), _ptr(o_f), _ptr(lse), _ptr(d_o), _ptr(row_ptr),
        _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx), _ptr(sched), _ptr(dqkv_c), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def vsa2_coarse_gate(p, pooled, x, d_model, w_g, o_f, o, saved, ws, stream=None):
    _check("vsa2_coarse_gate", lib().vsa2_coarse_gate(
        ctypes.byref(p), _ptr(pooled), _ptr(x), d_model, _ptr(w_g), _ptr(o_f), _ptr(o), _ptr(saved),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vsa2_coarse_gate_bwd(p, pooled, x, d_model, w_g, saved, d_o, dqkv_c, dx, dw_g, ws, stream=None):
    _check("vsa2_coarse_gate_bwd", lib().vsa2_coarse_gate_bwd(
        ctypes.byref(p), _ptr(pooled), _ptr(x), d_model, _ptr(w_g), _ptr(saved), _ptr(d_o), _ptr(dqkv_c),
        _ptr(dx), _ptr(dw_g), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def kernel_timer_start(kernel, capacity=256):
    _check("vsa2_kernel_timer_start", lib().vsa2_kernel_timer_start(kernel, capacity))


def kernel_timer_stop(kernel):
    """(summed milliseconds, launches) of the timed launches of `kernel`."""
    ms, n = ctypes.c_float(0.0), _I32(0)
    _check("vsa2_kernel_timer_stop", lib().vsa2_kernel_timer_stop(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------------------
# buffer bookkeeping for a full layer call (allocation + the call sequence)
# ---------------------------------------------------------------------------
def _ws(nbytes, device):
    # workspaces are 256-byte aligned (torch's caching allocator gives >= 512)
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Layer:
    """Device buffers for one (problem, topk, d_model) and the call sequence of
    the layer: pool -> route -> topk -> fine fwd -> coarse+gate, and the
    backward coarse+gate bwd -> fine bwd."""

    def __init__(self, p, topk, d_model, device="cuda"):
        self.p, self.topk, self.d_model, self.device = p, topk, d_model, device
        bh = p.batch * p.heads
        # token slots of the grid padded up to whole blocks (4x4x4 cubes, or
        # 4x4x8 pairs of cubes for 128-token blocks); nb counts blocks
        block = p.block_tokens or 64
        per = block // 64
        L = 64 * -(-p.lat_t // 4) * -(-p.lat_y // 4) * (-(-p.lat_x // (4 * per)) * per)
        nb = L // block
        self.L, self.nb, self.bh, self.block = L, nb, bh, block
        # MMDiT text rows follow the video slots of every per-token attention tensor
        self.rows = L + 64 * -(-p.text_tokens // 64)
        self.ntc = (self.rows - L) // 64  # text cubes
        self.k = budget(p, topk)
        self.sdt = torch.bfloat16 if p.dtype == VSA2_BF16 else torch.float32
        i32 = dict(dtype=torch.int32, device=device)
        self.pooled = _ws(pooled_size(p), device)
        self.scores = torch.empty((p.batch, p.heads, nb, nb), dtype=torch.float32, device=device)
        self.row_ptr = torch.empty((p.batch, p.heads, nb + 1), **i32)
        self.col_idx = torch.empty((p.batch, p.heads, self.k), **i32)
        self.col_ptr = torch.empty((p.batch, p.heads, nb + 1), **i32)
        self.row_idx = torch.empty((p.batch, p.heads, self.k), **i32)
        shp = (p.batch, p.heads, self.rows, p.head_dim)
        self.o_f = torch.empty(shp, dtype=self.sdt, device=device)
        self.o = torch.empty(shp, dtype=self.sdt, device=device)
        self.lse = torch.empty((p.batch, p.heads, self.rows), dtype=torch.float32, device=device)
        self.saved = _ws(saved_size(p), device)
        ws_need = max(workspace_size(p, op, topk, d_model)
                      for op in (OP_ROUTE, OP_TOPK, OP_PLAN, OP_FWD, OP_BWD, OP_COARSE, OP_COARSE_BWD,
                                 OP_ROUTE_COARSE, OP_TOPK_ROW))
        self.ws = _ws(ws_need, device)
        # the fine branch's work schedule (None when the problem needs none)
        ss = sched_size(p, topk)
        self.sched = _ws(ss, device) if ss else None
        self._grads = None

    def forward(self, q, k, v, x, w_g, route=True, stream=None, router="vsa2"):
        """router: "vsa2" (fine-grained router, per-sequence TopK) or "vsa"
        (the coarse-score router with a TopK per query block)."""
        p = self.p
        vsa2_pool(p, q, k, v, self.pooled, stream)
        if route and router == "vsa":
            vsa2_route_coarse(p, self.pooled, self.scores, self.ws, stream)
            vsa2_topk_per_row(p, self.scores, self.topk, self.row_ptr, self.col_idx, self.col_ptr,
                              self.row_idx, self.ws, stream, sched=self.sched)
        elif route:
            vsa2_route(p, self.pooled, self.scores, self.ws, stream)
            vsa2_topk_per_seq(p, self.scores, self.topk, self.row_ptr, self.col_idx, self.col_ptr,
                              self.row_idx, self.ws, stream, sched=self.sched)
        vsa2_sparse_attn_fwd(p, self.topk, q, k, v, self.row_ptr, self.col_idx, self.o_f, self.lse, self.ws, stream,
                             sched=self.sched)
        vsa2_coarse_gate(p, self.pooled, x, self.d_model, w_g, self.o_f, self.o, self.saved, self.ws, stream)
        return self.o

    def set_selection(self, row_ptr, col_idx, stream=None):
        self.row_ptr.copy_(row_ptr)
        self.col_idx.copy_(col_idx)
        vsa2_plan_from_csr(self.p, self.topk, self.row_ptr, self.col_idx, self.col_ptr, self.row_idx, self.ws, stream,
                           sched=self.sched)

    def grads(self):
        """Gradient buffers (allocated on first use): dq, dk, dv, dx, dw_g, dqkv_c."""
        p = self.p
        if self._grads is None:
            shp = (p.batch, p.heads, self.rows, p.head_dim)
            self._grads = dict(
                dq=torch.empty(shp, dtype=self.sdt, device=self.device),
                dk=torch.empty(shp, dtype=self.sdt, device=self.device),
                dv=torch.empty(shp, dtype=self.sdt, device=self.device),
                dx=torch.empty((p.batch, self.L, self.d_model), dtype=self.sdt, device=self.device),
                dw_g=torch.empty((self.d_model, p.heads), dtype=torch.float32, device=self.device),
                dqkv_c=torch.empty((3, p.batch, p.heads, self.nb, p.head_dim), dtype=torch.float32,
                                   device=self.device),
            )
        return self._grads

    def backward(self, q, k, v, x, w_g, d_o, stream=None):
        p = self.p
        g = self.grads()
        vsa2_coarse_gate_bwd(p, self.pooled, x, self.d_model, w_g, self.saved, d_o, g["dqkv_c"], g["dx"],
                             g["dw_g"], self.ws, stream)
        vsa2_sparse_attn_bwd(p, self.topk, q, k, v, self.o_f, self.lse, d_o, self.row_ptr, self.col_idx,
                             self.col_ptr, self.row_idx, g["dqkv_c"], g["dq"], g["dk"], g["dv"], self.ws, stream,
                             sched=self.sched)
        return g

    def saved_views(self):
        """(O_hat_c [B,H,nb,d], lse_c [B,H,nb], G [B,H,L]) views of the saved buffer."""
        p = self.p
        f = self.saved.view(torch.float32)
        n1 = self.bh * self.nb * p.head_dim
        n2 = self.bh * self.nb
        return (f[:n1].view(p.batch, p.heads, self.nb, p.head_dim), f[n1:n1 + n2].view(p.batch, p.heads, self.nb),
                f[n1 + n2:n1 + n2 + self.bh * self.L].view(p.batch, p.heads, self.L))

    def pooled_views(self):
        """(Q_r, K_r [B,H,L/8,d], Q_c, K_c, V_c [B,H,nbp,d]) views of the pooled buffer."""
        p = self.p
        flat = self.pooled.view(self.sdt)
        lr, nbp, d = self.L // 8, (self.nb + 63) // 64 * 64, p.head_dim
        n_r, n_c = self.bh * lr * d, self.bh * nbp * d
        sh_r, sh_c = (p.batch, p.heads, lr, d), (p.batch, p.heads, nbp, d)
        return (flat[:n_r].view(sh_r), flat[n_r:2 * n_r].view(sh_r), flat[2 * n_r:2 * n_r + n_c].view(sh_c),
                flat[2 * n_r + n_c:2 * n_r + 2 * n_c].view(sh_c), flat[2 * n_r + 2 * n_c:2 * n_r + 3 * n_c].view(sh_c))
