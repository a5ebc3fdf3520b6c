"""Torch-facing wrapper of libra_attn.so.

PyTorch supplies device memory (tensors) and the stream; every step of the
attention runs in the library's HIP kernels.  Nothing here computes the method.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import native
from .native import check, lib

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _stream_ptr(stream=None, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """A validated problem (shape + options) with its RoPE tables.

    q, k, v, out are [B, N, H, D] contiguous CUDA tensors, N = F*H*W tokens in
    (f, h, w) order.  rot: 'none' | 'interleaved' | 'half' | 'full'; prec:
    'int4' | 'bf16'; in_dtype/out_dtype: 'bf16' | 'f32'.  Creating a plan
    copies its small RoPE tables to the current device; the calls then
    allocate nothing on the library side.
    """

    def __init__(self, batch, heads, head_dim, grid, seg, rot="half", prec="int4",
                 in_dtype="bf16", out_dtype="f32", rope_theta=10000.0, softmax_scale=0.0,
                 p_mode=0, v_hadamard=0):
        self.batch, self.heads, self.head_dim = int(batch), int(heads), int(head_dim)
        self.grid = tuple(int(x) for x in grid)
        self.seg = tuple(int(x) for x in seg)
        self.rot, self.prec, self.in_dtype, self.out_dtype = rot, prec, in_dtype, out_dtype
        self.tokens = self.grid[0] * self.grid[1] * self.grid[2]
        self._shape = native.make_shape(self.batch, self.heads, self.head_dim, self.grid, self.seg)
        self._opts = native.make_opts(rot, prec, in_dtype, out_dtype, rope_theta, softmax_scale,
                                      p_mode, v_hadamard)
        h = ctypes.c_void_p()
        check(lib().ra_plan_create(ctypes.byref(self._shape), ctypes.byref(self._opts),
                                   ctypes.byref(h)), "ra_plan_create")
        self._h = h
        n = ctypes.c_size_t()
        check(lib().ra_plan_workspace_size(self._h, ctypes.byref(n)), "ra_plan_workspace_size")
        self.workspace_bytes = n.value

    # -- lifetime -----------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            lib().ra_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- buffers ------------------------------------------------------------
    @property
    def io_shape(self):
        return (self.batch, self.tokens, self.heads, self.head_dim)

    def workspace(self, device="cuda"):
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def empty_out(self, device="cuda"):
        return torch.empty(self.io_shape, dtype=_TORCH_DT[self.out_dtype], device=device)

    def _check_in(self, *ts):
        want = _TORCH_DT[self.in_dtype]
        for t in ts:
            if tuple(t.shape) != self.io_shape or t.dtype != want or not t.is_contiguous() or not t.is_cuda:
                raise ValueError("input must be a contiguous CUDA %s tensor of shape %s (got %s %s)"
                                 % (want, self.io_shape, t.dtype, tuple(t.shape)))

    def _check_out(self, out, device):
        want = _TORCH_DT[self.out_dtype]
        if (tuple(out.shape) != self.io_shape or out.dtype != want or not out.is_contiguous()
                or not out.is_cuda or out.device != device):
            raise ValueError("out must be a contiguous %s tensor of shape %s on %s (got %s %s on %s)"
                             % (want, self.io_shape, device, out.dtype, tuple(out.shape), out.device))

    def _ws(self, workspace, device):
        if workspace is None:
            workspace = self.workspace(device)
        if (workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not workspace.is_cuda
                or workspace.device != device):
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % device)
        return workspace

    # -- calls --------------------------------------------------------------
    def forward(self, q, k, v, out=None, workspace=None, stream=None):
        self._check_in(q, k, v)
        out = self.empty_out(q.device) if out is None else out
        self._check_out(out, q.device)
        ws = self._ws(workspace, q.device)
        check(lib().ra_attn_fwd(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                ws.numel(), _stream_ptr(stream, q.device)), "ra_attn_fwd")
        return out

    __call__ = forward

    def forward_noalloc(self, q, k, v, out=None, stream=None):
        """ra_attn_fwd_noalloc: the same forward with the library's fixed
        device-resident workspace (for plans of at most
        RA_NOALLOC_WORKSPACE_BYTES; calls on one GPU share it)."""
        self._check_in(q, k, v)
        out = self.empty_out(q.device) if out is None else out
        self._check_out(out, q.device)
        check(lib().ra_attn_fwd_noalloc(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _stream_ptr(stream, q.device)), "ra_attn_fwd_noalloc")
        return out

    def prologue(self, q, k, v, workspace, stream=None):
        self._check_in(q, k, v)
        workspace = self._ws(workspace, q.device)
        check(lib().ra_attn_prologue(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                                     workspace.numel(), _stream_ptr(stream, q.device)),
              "ra_attn_prologue")

    def main(self, out, workspace, stream=None):
        self._check_out(out, out.device)
        workspace = self._ws(workspace, out.device)
        check(lib().ra_attn_main(self._h, _ptr(out), _ptr(workspace), workspace.numel(),
                                 _stream_ptr(stream, out.device)), "ra_attn_main")
        return out

    def upload(self):
        """Copy the plan's tables to the current device (needed before using
        the plan on a device other than the one current at creation)."""
        check(lib().ra_plan_upload(self._h), "ra_plan_upload")

    # -- parity exports -----------------------------------------------------
    def debug_prologue(self, q, k, v, workspace=None):
        self._check_in(q, k, v)
        ws = self._ws(workspace, q.device)
        B, N, H, D = self.io_shape
        nblk = (N + 63) // 64
        qc = np.empty((B, H, N, D), np.int8)
        kc = np.empty((B, H, N, D), np.int8)
        vc = np.empty((B, H, N, D), np.int8)
        sq = np.empty((B, H, nblk), np.float32)
        sk = np.empty((B, H, nblk), np.float32)
        sv = np.empty((B, H, D), np.float32)
        P = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        check(lib().ra_debug_prologue(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(ws), ws.numel(),
                                      P(qc), P(sq), P(kc), P(sk), P(vc), P(sv),
                                      _stream_ptr(None, q.device)), "ra_debug_prologue")
        return dict(q_codes=qc, s_q=sq, k_codes=kc, s_k=sk, v_codes=vc, s_v=sv)

    def debug_tile(self, workspace, b, h, q_blk, kv_blk):
        D = self.head_dim
        s_int = np.empty((64, 64), np.int32)
        p_code = np.empty((64, 64), np.int8)
        pv = np.empty((64, D), np.int32)
        m = np.empty(64, np.float32)
        P = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        check(lib().ra_debug_tile(self._h, _ptr(workspace), workspace.numel(), b, h, q_blk, kv_blk,
                                  P(s_int), P(p_code), P(pv), P(m),
                                  _stream_ptr(None, workspace.device)), "ra_debug_tile")
        return dict(s_int=s_int, p_code=p_code, pv_int=pv, m_after=m)

    def row_digests(self, workspace, out=None):
        """Stage 2 through the parity variant of the INT4 kernel (f32
        output): returns (out, rows) with rows [B, H, N, 4] uint32 = (final
        running max bits, sum of u, sum of u * h(j) mod 2^32, row-sum bits)."""
        B, N, H, D = self.io_shape
        out = self.empty_out(workspace.device) if out is None else out
        self._check_out(out, workspace.device)
        workspace = self._ws(workspace, workspace.device)
        rows = torch.empty((B, H, N, 4), dtype=torch.int32, device=workspace.device)
        check(lib().ra_debug_row_digests(self._h, _ptr(out), _ptr(workspace), workspace.numel(), _ptr(rows),
                                         _stream_ptr(None, workspace.device)), "ra_debug_row_digests")
        return out, rows

    def tables(self, seg: int):
        npos = self.grid[seg]
        half = self.seg[seg] // 2
        cs = np.empty((npos, half), np.float32)
        sn = np.empty((npos, half), np.float32)
        check(lib().ra_debug_tables(self._h, seg, cs.ctypes.data_as(ctypes.c_void_p),
                                    sn.ctypes.data_as(ctypes.c_void_p)), "ra_debug_tables")
        return cs, sn


def attn_fwd(q, k, v, grid, seg, rot="half", prec="int4", out_dtype="f32", workspace=None,
             stream=None):
    """One-shot forward through ra_attn_fwd_simple (plans cached in the library)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, D] (got %s)" % (tuple(q.shape),))
    B, N, H, D = q.shape
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must be bfloat16 or float32 (got %s)" % q.dtype)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("%s must be a %s tensor of shape %s on %s like q (got %s %s on %s)"
                             % (name, q.dtype, tuple(q.shape), q.device, t.dtype, tuple(t.shape), t.device))
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous CUDA tensor" % name)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()
                                  or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % q.device)
    in_dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[q.dtype]
    shape = native.make_shape(B, H, D, grid, seg)
    opts = native.make_opts(rot, prec, in_dtype, out_dtype)
    n = ctypes.c_size_t()
    check(lib().ra_workspace_size(ctypes.byref(shape), ctypes.byref(opts), ctypes.byref(n)),
          "ra_workspace_size")
    ws = workspace if workspace is not None else torch.empty(n.value, dtype=torch.uint8, device=q.device)
    out = torch.empty((B, N, H, D), dtype=_TORCH_DT[out_dtype], device=q.device)
    check(lib().ra_attn_fwd_simple(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, D, *grid, *seg,
                                   native.ROT[rot], native.PREC[prec], native.DT[in_dtype],
                                   native.DT[out_dtype], _ptr(ws), ws.numel(),
                                   _stream_ptr(stream, q.device)), "ra_attn_fwd_simple")
    return out


def schedule_pick(sched, step, n_steps, block, n_blocks) -> str:
    """'bf16' on the head/tail steps or blocks of `sched` = (steps_head,
    steps_tail, blocks_head, blocks_tail), else 'int4'."""
    s = native.RaSchedule(*[int(x) for x in sched])
    return "bf16" if lib().ra_schedule_pick(ctypes.byref(s), step, n_steps, block, n_blocks) else "int4"


def pmap_device(d: torch.Tensor, p_mode: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """The attention kernels' P map on exponents d = log2 p (float32 CUDA
    tensor) -> u = round(15 2^d) = code + 8 (p_mode 0) or round(7 2^d) = code
    (p_mode 1), uint8."""
    if d.dtype != torch.float32 or not d.is_cuda:
        raise ValueError("d must be a float32 CUDA tensor")
    d = d.contiguous()
    u = torch.empty(d.shape, dtype=torch.uint8, device=d.device) if out is None else out
    if u.dtype != torch.uint8 or u.numel() != d.numel() or not u.is_contiguous() or u.device != d.device:
        raise ValueError("out must be a contiguous uint8 tensor with d's size on its device")
    check(lib().ra_debug_pmap(_ptr(d), _ptr(u), d.numel(), int(p_mode), _stream_ptr(None, d.device)),
          "ra_debug_pmap")
    return u


def copy(dst: torch.Tensor, src: torch.Tensor, nbytes: int | None = None, stream=None):
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    check(lib().ra_copy(_ptr(dst), _ptr(src), nbytes, _stream_ptr(stream, src.device)), "ra_copy")


def pmap_thresholds(p_mode: int = 0) -> np.ndarray:
    """The library's P-map thresholds T_k (binary32): u = #{k : d >= T_k}."""
    T = np.empty(15 if p_mode == 0 else 7, np.float32)
    check(lib().ra_pmap_thresholds(int(p_mode), T.ctypes.data_as(ctypes.c_void_p)), "ra_pmap_thresholds")
    return T


def pmap_table(p_mode: int = 0):
    """The byte table the INT4 kernels look P codes up in (entries, then 16
    8-byte records; see ra_pmap_table) and its top cell."""
    buf = np.zeros(RA_PMAP_TABLE_BYTES, np.uint8)
    top = ctypes.c_int32(0)
    check(lib().ra_pmap_table(int(p_mode), buf.ctypes.data_as(ctypes.c_void_p), buf.size, ctypes.byref(top)),
          "ra_pmap_table")
    return buf, int(top.value)


RA_PMAP_TABLE_BYTES = 20240

PEAK_KINDS = {"i8": 0, "fp8": 1, "fp6": 2, "fp6_fp8": 3, "bf16": 4}


def mfma_peak(kind: str, iters: int = 20000, blocks: int = 768, stream=None):
    """Sustained matrix-core throughput of one operand type through
    ra_bench_mfma_peak: returns (T ops/s, engine clock in GHz over the launch).
    768 workgroups of 4 waves put 3 waves on each SIMD of the 256 CUs."""
    dev = torch.device("cuda", torch.cuda.current_device())
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    ops = ctypes.c_double()
    st = _stream_ptr(stream, dev)
    s = torch.cuda.current_stream(dev) if stream is None else stream

    def launch():
        check(lib().ra_bench_mfma_peak(PEAK_KINDS[kind], int(iters), int(blocks), _ptr(sink), _ptr(clk),
                                       ctypes.byref(ops), st), "ra_bench_mfma_peak")

    launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    launch()
    e1.record(s)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1)
    c = clk.cpu().tolist()
    ghz = (c[1] - c[0]) / max(1, c[3] - c[2]) * 0.1
    return ops.value / (ms * 1e-3) / 1e12, ghz
