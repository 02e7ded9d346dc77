"""ctypes binding of the C ABI declared in include/bi_gemm.h, include/bi_moe.h,
include/bi_norm.h and include/bi_attn.h.

Argument marshalling only: every step of the GEMM runs in the HIP library
``libbigemm.so``.  Tensors are PyTorch device tensors (PyTorch provides device
memory and streams); their pointers and sizes go straight to the C calls.
There is no fallback: if the library is missing or the call fails, this
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# BI_GEMM_LIB may name another build of the same library (the CPU tests'
# AddressSanitizer copy); there is no other implementation to fall back to
LIB_PATH = os.environ.get("BI_GEMM_LIB") or os.path.join(HERE, "libbigemm.so")
PIN_TABLE = os.path.join(HERE, "pins", "gfx950.txt")

STATUS = {
    0: "BI_OK",
    1: "BI_ERR_INVALID_ARGUMENT",
    2: "BI_ERR_MISALIGNED",
    3: "BI_ERR_NO_PIN",
    4: "BI_ERR_UNSUPPORTED_DEVICE",
    5: "BI_ERR_OUT_OF_MEMORY",
    6: "BI_ERR_HIP",
    7: "BI_ERR_BAD_PIN_TABLE",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}


MAX_TILINGS = 12  # BI_MAX_TILINGS
INT32_MAX = 2 ** 31 - 1

# bi_kernel_kind_t, by index; the names are the pin table's
KERNEL_KINDS = ("stream_mb1", "stream_mb2", "stream_mb4", "tiled_64x32", "tiled_64x64", "tiled_128x64",
                "tiled_128x64_deep", "tiled_128x128", "tiled_128x128_deep", "tiled4_128x256", "tiled4_256x256",
                "tiled4_160x256", "tiled4_192x256", "stream_mb2_n2", "stream_mb4_n2", "stream_mb2_n4",
                "stream_mb4_n4")


CONCURRENT_SPLITS = 0x100  # BI_KERNEL_CONCURRENT_SPLITS; "+cs" in a kind's name


def kind_value(kind) -> int:
    """A kind name ("tiled_64x64", "tiled_64x64+cs") or value -> its tile_kernel value."""
    if not isinstance(kind, str):
        return int(kind)
    if kind.endswith("+cs"):
        return KERNEL_KINDS.index(kind[:-3]) | CONCURRENT_SPLITS
    return KERNEL_KINDS.index(kind)


def kind_name(value: int) -> str:
    return KERNEL_KINDS[value & ~CONCURRENT_SPLITS] + ("+cs" if value & CONCURRENT_SPLITS else "")


class BiPinInfo(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n", "k", "experts", "mfma_m", "mfma_n", "mfma_k", "k_map", "splits", "split_len",
        "fold", "stream_max_m", "from_table", "table_version", "tilings")] + [
        ("tile_m_max", ctypes.c_int32 * MAX_TILINGS), ("tile_kernel", ctypes.c_int32 * MAX_TILINGS),
        ("split_ws_rows", ctypes.c_int32)]

    def as_dict(self):
        d = {name: int(getattr(self, name)) for name, t in self._fields_ if t is ctypes.c_int32}
        d["tiling"] = [(int(self.tile_m_max[i]), kind_name(self.tile_kernel[i])) for i in range(self.tilings)]
        return d

    def set_tiling(self, tiling):
        """tiling: [(m_max, kind name or value), ...], the last m_max None or
        INT32_MAX (every larger M)."""
        if len(tiling) > MAX_TILINGS:
            raise ValueError("at most %d tiling entries" % MAX_TILINGS)
        self.tilings = len(tiling)
        for i, (m, kind) in enumerate(tiling):
            self.tile_m_max[i] = INT32_MAX if m is None else int(m)
            self.tile_kernel[i] = kind_value(kind)


class BiGemmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__("%s: %s" % (self.name, detail))


_lock = threading.Lock()
_lib = None


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    S = ctypes.c_int  # bi_status_t
    sig = {
        "bi_gemm_load_pins": ([ctypes.c_char_p], S),
        "bi_gemm_tree_id": ([], ctypes.c_char_p),
        "bi_gemm_kernel_kind_name": ([I], ctypes.c_char_p),
        "bi_gemm_set_strict": ([I], None),
        "bi_gemm_create": ([I, I, P, ctypes.POINTER(P)], S),
        "bi_gemm_create_pinned": ([I, I, P, ctypes.POINTER(BiPinInfo), ctypes.POINTER(P)], S),
        "bi_gemm_run": ([P, P, I, P, P], S),
        "bi_gemm_run_splitk": ([P, P, I, P, I, I, P, P], S),
        "bi_grouped_gemm_create": ([I, I, I, P, ctypes.POINTER(P)], S),
        "bi_grouped_gemm_run": ([P, P, P, I, P, P], S),
        "bi_gemm_destroy": ([P], None),
        "bi_gemm_get_pin": ([P, ctypes.POINTER(BiPinInfo)], S),
        "bi_status_string": ([S], ctypes.c_char_p),
        "bi_gemm_kernel_name": ([P, I], ctypes.c_char_p),
        "bi_last_error": ([], ctypes.c_char_p),
        "bi_grouped_gemm_run_indexed": ([P, P, I, P, P, I, P, P], S),
        "bi_moe_topk": ([P, I, I, I, P, P, P], S),
        "bi_moe_permute": ([P, I, I, I, P, P, P, P], S),
        "bi_gather_rows": ([P, I, P, I, I, P, P], S),
        "bi_swiglu": ([P, I, I, P, P], S),
        "bi_moe_combine": ([P, I, P, P, P, I, I, I, P, P], S),
        "bi_moe_create": ([I, I, I, I, P, P, P, I, ctypes.POINTER(P)], S),
        "bi_moe_run": ([P, P, I, P, P], S),
        "bi_moe_destroy": ([P], None),
        "bi_rmsnorm": ([P, P, I, I, ctypes.c_float, P, P], S),
        "bi_rmsnorm_gemm_run": ([P, P, P, ctypes.c_float, I, P, P, P], S),
        "bi_rmsnorm_gemm_kernel_name": ([P, I], ctypes.c_char_p),
        "bi_attn_create": ([I, I, I, I, I, I, ctypes.POINTER(P)], S),
        "bi_attn_decode": ([P, P, P, P, P, I, I, ctypes.c_float, P, P], S),
        "bi_attn_destroy": ([P], None),
        "bi_attn_decode_noalloc": ([I, I, I, I, I, P, P, P, P, I, I, ctypes.c_float, P, P], S),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def load(path: str = LIB_PATH, pins: str | None = PIN_TABLE):
    """Load the HIP library (once) and its pin table.  Raises if missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    "the HIP library %s is not built; run __graft_entry__.build() "
                    "or python invariant_bi_gemm_amd/build.py" % path)
            lib = _declare(ctypes.CDLL(path))
            if pins and not os.environ.get("BI_GEMM_PINS"):
                st = lib.bi_gemm_load_pins(pins.encode())
                if st != 0:
                    raise BiGemmError(st, lib.bi_last_error().decode())
            _lib = lib
    return _lib


def last_error() -> str:
    return load().bi_last_error().decode()


def check(status: int):
    if status != 0:
        raise BiGemmError(status, last_error())


def status_string(status: int) -> str:
    return load().bi_status_string(status).decode()


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _need(t, dtype, ndim, what):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if t.dtype != dtype or t.dim() != ndim or not t.is_cuda:
        raise TypeError("%s must be a %d-d %s CUDA tensor, got %s %s on %s" % (what, ndim, dtype, t.dtype, tuple(t.shape), t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)


class Gemm:
    """A dense layer handle: ``y = x @ W.T`` with batch-invariant rows.

    ``W`` is a contiguous bf16 [N, K] CUDA tensor.  The C library packs its
    own copy at create, so W may be freed or changed afterwards.  ``pin``
    (optional) is a dict with ``splits``, ``stream_max_m`` and ``tiling``
    ([(m_max, kind), ...], the last m_max None) to override the pin table.
    """

    def __init__(self, W, pin: dict | None = None):
        import torch

        lib = load()
        _need(W, torch.bfloat16, 2, "W")
        self.n, self.k = (int(v) for v in W.shape)
        self._lib = lib
        h = ctypes.c_void_p()
        with torch.cuda.device(W.device):
            if pin is None:
                st = lib.bi_gemm_create(self.n, self.k, ctypes.c_void_p(W.data_ptr()), ctypes.byref(h))
            else:
                p = BiPinInfo()
                p.splits = int(pin.get("splits", 1))
                p.stream_max_m = int(pin.get("stream_max_m", 16))
                p.set_tiling(pin.get("tiling", []))
                st = lib.bi_gemm_create_pinned(self.n, self.k, ctypes.c_void_p(W.data_ptr()),
                                               ctypes.byref(p), ctypes.byref(h))
        check(st)
        self._h = h

    @property
    def pin(self) -> dict:
        info = BiPinInfo()
        check(self._lib.bi_gemm_get_pin(self._h, ctypes.byref(info)))
        return info.as_dict()

    def kernel_name(self, m: int) -> str:
        """The kernel a call with ``m`` rows launches (no launch)."""
        return self._lib.bi_gemm_kernel_name(self._h, int(m)).decode()

    def __call__(self, x, out=None, stream=None):
        import torch

        _need(x, torch.bfloat16, 2, "x")
        if x.shape[1] != self.k:
            raise ValueError("x has K=%d, the layer has K=%d" % (x.shape[1], self.k))
        m = int(x.shape[0])
        if out is None:
            out = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, torch.float32, 2, "out")
            if tuple(out.shape) != (m, self.n):
                raise ValueError("out must be [%d, %d]" % (m, self.n))
        self.run_ptr(x.data_ptr(), m, out.data_ptr(), stream)
        return out

    def run_ptr(self, x_ptr: int, m: int, y_ptr: int, stream=None):
        """Raw call: device pointers and the row count, as the C ABI takes them."""
        check(self._lib.bi_gemm_run(self._h, ctypes.c_void_p(x_ptr), int(m), ctypes.c_void_p(y_ptr),
                                    _stream_ptr(stream)))

    def run_splitk(self, x, kind, splits, out=None, workspace=None, stream=None):
        """The NON-invariant comparison GEMM (include/bi_gemm_ref.h): kernel
        ``kind`` (a name of KERNEL_KINDS or its index) over ``splits``
        concurrent K splits.  ``workspace``: fp32 with at least
        (splits-1)*M*N elements (allocated here when None)."""
        import torch

        _need(x, torch.bfloat16, 2, "x")
        if x.shape[1] != self.k:
            raise ValueError("x has K=%d, the layer has K=%d" % (x.shape[1], self.k))
        m = int(x.shape[0])
        if out is None:
            out = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        if workspace is None and splits > 1:
            workspace = torch.empty((splits - 1) * m * self.n, dtype=torch.float32, device=x.device)
        if workspace is not None and workspace.numel() < (splits - 1) * m * self.n:
            raise ValueError("workspace too small")
        k = KERNEL_KINDS.index(kind) if isinstance(kind, str) else int(kind)
        check(self._lib.bi_gemm_run_splitk(self._h, ctypes.c_void_p(x.data_ptr()), m, ctypes.c_void_p(out.data_ptr()),
                                           k, int(splits),
                                           ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0),
                                           _stream_ptr(stream)))
        return out

    def rmsnorm_run(self, x, gain, eps, out=None, rstd=None, stream=None):
        """``RMSNorm(x) * gain @ W.T`` with the norm in the GEMM's prologue
        (bi_rmsnorm_gemm_run): x raw bf16 [M, K], gain bf16 [K].  Returns
        (y, rstd)."""
        import torch

        _need(x, torch.bfloat16, 2, "x")
        _need(gain, torch.bfloat16, 1, "gain")
        if x.shape[1] != self.k or gain.shape[0] != self.k:
            raise ValueError("x and gain must have K=%d" % self.k)
        m = int(x.shape[0])
        if out is None:
            out = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, torch.float32, 2, "out")
            if tuple(out.shape) != (m, self.n):
                raise ValueError("out must be [%d, %d]" % (m, self.n))
        if rstd is None:
            rstd = torch.empty(m, dtype=torch.float32, device=x.device)
        else:
            _need(rstd, torch.float32, 1, "rstd")
            if rstd.shape[0] != m:
                raise ValueError("rstd must hold M values")
        check(self._lib.bi_rmsnorm_gemm_run(self._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(gain.data_ptr()),
                                            ctypes.c_float(eps), m, ctypes.c_void_p(rstd.data_ptr()),
                                            ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out, rstd

    def rmsnorm_kernel_name(self, m: int) -> str:
        return self._lib.bi_rmsnorm_gemm_kernel_name(self._h, int(m)).decode()

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bi_gemm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 (interpreter shutdown)
            pass


class GroupedGemm:
    """MoE experts: ``W`` is bf16 [E, N, K] (copied at create); rows of x are
    grouped by expert."""

    def __init__(self, W):
        import torch

        lib = load()
        _need(W, torch.bfloat16, 3, "W")
        self.e, self.n, self.k = (int(v) for v in W.shape)
        self._lib = lib
        h = ctypes.c_void_p()
        with torch.cuda.device(W.device):
            st = lib.bi_grouped_gemm_create(self.e, self.n, self.k, ctypes.c_void_p(W.data_ptr()), ctypes.byref(h))
        check(st)
        self._h = h

    @property
    def pin(self) -> dict:
        info = BiPinInfo()
        check(self._lib.bi_gemm_get_pin(self._h, ctypes.byref(info)))
        return info.as_dict()

    def kernel_name(self, rows: int) -> str:
        """The kernels a call with ``rows`` rows in all launches (no launch)."""
        return self._lib.bi_gemm_kernel_name(self._h, int(rows)).decode()

    def __call__(self, x, expert_offsets, out=None, stream=None):
        import torch

        _need(x, torch.bfloat16, 2, "x")
        _need(expert_offsets, torch.int32, 1, "expert_offsets")
        if x.shape[1] != self.k or expert_offsets.shape[0] != self.e + 1:
            raise ValueError("shape mismatch")
        r = int(x.shape[0])
        if out is None:
            out = torch.empty((r, self.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, torch.float32, 2, "out")
            if tuple(out.shape) != (r, self.n):
                raise ValueError("out must be [%d, %d]" % (r, self.n))
        check(self._lib.bi_grouped_gemm_run(self._h, ctypes.c_void_p(x.data_ptr()),
                                            ctypes.c_void_p(expert_offsets.data_ptr()), r,
                                            ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def run_indexed(self, x, row_index, expert_offsets, out=None, stream=None):
        """``y[i] = x[row_index[i]] @ W[e].T`` for the rows i of expert e: the
        gather into expert order done by the kernels' loads."""
        import torch

        _need(x, torch.bfloat16, 2, "x")
        _need(row_index, torch.int32, 1, "row_index")
        _need(expert_offsets, torch.int32, 1, "expert_offsets")
        if x.shape[1] != self.k or expert_offsets.shape[0] != self.e + 1:
            raise ValueError("shape mismatch")
        r = int(row_index.shape[0])
        if out is None:
            out = torch.empty((r, self.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, torch.float32, 2, "out")
        check(self._lib.bi_grouped_gemm_run_indexed(self._h, ctypes.c_void_p(x.data_ptr()), int(x.shape[0]),
                                                    ctypes.c_void_p(row_index.data_ptr()),
                                                    ctypes.c_void_p(expert_offsets.data_ptr()), r,
                                                    ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bi_gemm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass


# ---- the MoE layer around the grouped GEMM (include/bi_moe.h) ----------------

def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def moe_topk(logits, k: int, stream=None):
    """Top-k routing of fp32 logits [T, E]: ``(ids int32 [T,k], weights fp32 [T,k])``."""
    import torch

    lib = load()
    _need(logits, torch.float32, 2, "logits")
    t, e = (int(v) for v in logits.shape)
    ids = torch.empty((t, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((t, k), dtype=torch.float32, device=logits.device)
    check(lib.bi_moe_topk(_p(logits), t, e, int(k), _p(ids), _p(w), _stream_ptr(stream)))
    return ids, w


def moe_permute(ids, experts: int, stream=None):
    """Stable grouping of the (token, slot) pairs by expert:
    ``(offsets [E+1], token_of_row [T*k], row_of [T,k])``, int32."""
    import torch

    lib = load()
    _need(ids, torch.int32, 2, "ids")
    t, k = (int(v) for v in ids.shape)
    dev = ids.device
    off = torch.empty(experts + 1, dtype=torch.int32, device=dev)
    tok = torch.empty(t * k, dtype=torch.int32, device=dev)
    row_of = torch.empty((t, k), dtype=torch.int32, device=dev)
    check(lib.bi_moe_permute(_p(ids), t, int(experts), k, _p(off), _p(tok), _p(row_of), _stream_ptr(stream)))
    return off, tok, row_of


def gather_rows(src, idx, stream=None):
    """``src[idx]`` for bf16 rows (an index outside the rows gives zeros)."""
    import torch

    lib = load()
    _need(src, torch.bfloat16, 2, "src")
    _need(idx, torch.int32, 1, "idx")
    r, kk = int(idx.shape[0]), int(src.shape[1])
    out = torch.empty((r, kk), dtype=torch.bfloat16, device=src.device)
    check(lib.bi_gather_rows(_p(src), int(src.shape[0]), _p(idx), r, kk, _p(out), _stream_ptr(stream)))
    return out


def swiglu(h, stream=None):
    """bf16 ``silu(h[:, :I]) * h[:, I:]`` of an fp32 up projection h [R, 2I]."""
    import torch

    lib = load()
    _need(h, torch.float32, 2, "h")
    r, i2 = (int(v) for v in h.shape)
    if i2 % 2:
        raise ValueError("h must have an even number of columns")
    out = torch.empty((r, i2 // 2), dtype=torch.bfloat16, device=h.device)
    check(lib.bi_swiglu(_p(h), r, i2 // 2, _p(out), _stream_ptr(stream)))
    return out


def moe_combine(o, ids, weights, row_of, stream=None):
    """``y[t] = sum_j weights[t,j] * o[row_of[t,j]]`` in ascending expert id."""
    import torch

    lib = load()
    _need(o, torch.float32, 2, "o")
    _need(ids, torch.int32, 2, "ids")
    _need(weights, torch.float32, 2, "weights")
    _need(row_of, torch.int32, 2, "row_of")
    t, k = (int(v) for v in ids.shape)
    if tuple(weights.shape) != (t, k) or tuple(row_of.shape) != (t, k):
        raise ValueError("ids, weights and row_of must all be [T, k]")
    r, hdim = (int(v) for v in o.shape)
    y = torch.empty((t, hdim), dtype=torch.float32, device=o.device)
    check(lib.bi_moe_combine(_p(o), r, _p(ids), _p(weights), _p(row_of), t, k, hdim, _p(y),
                             _stream_ptr(stream)))
    return y


class MoeLayer:
    """The expert layer: router, top-k, grouping, up projection, SwiGLU, down
    projection and the weighted combine, every token's output independent of
    the batch.  ``W_router`` bf16 [E, H], ``W_up`` bf16 [E, 2I, H] (gate rows
    then up rows), ``W_down`` bf16 [E, H, I]; the handle packs its own copies
    at create."""

    def __init__(self, W_router, W_up, W_down, k: int, max_tokens: int):
        import torch

        lib = load()
        _need(W_router, torch.bfloat16, 2, "W_router")
        _need(W_up, torch.bfloat16, 3, "W_up")
        _need(W_down, torch.bfloat16, 3, "W_down")
        self.e, self.h = (int(v) for v in W_router.shape)
        self.i = int(W_down.shape[2])
        self.k, self.max_tokens = int(k), int(max_tokens)
        if tuple(W_up.shape) != (self.e, 2 * self.i, self.h) or tuple(W_down.shape) != (self.e, self.h, self.i):
            raise ValueError("W_up must be [E, 2I, H] and W_down [E, H, I]")
        self._lib = lib
        h = ctypes.c_void_p()
        with torch.cuda.device(W_router.device):
            st = lib.bi_moe_create(self.e, self.k, self.h, self.i, _p(W_router), _p(W_up), _p(W_down),
                                   self.max_tokens, ctypes.byref(h))
        check(st)
        self._h = h

    def __call__(self, x, out=None, stream=None):
        import torch

        _need(x, torch.bfloat16, 2, "x")
        t = int(x.shape[0])
        if int(x.shape[1]) != self.h:
            raise ValueError("x must be [T, %d]" % self.h)
        if out is None:
            out = torch.empty((t, self.h), dtype=torch.float32, device=x.device)
        else:
            _need(out, torch.float32, 2, "out")
        check(self._lib.bi_moe_run(self._h, _p(x), t, _p(out), _stream_ptr(stream)))
        return out

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bi_moe_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass


# ---- RMSNorm (include/bi_norm.h) -----------------------------------------------

def rmsnorm(x, gain, eps: float = 1e-5, out=None, stream=None):
    """bf16 ``x * gain / sqrt(mean(x^2) + eps)`` per row of a bf16 [T, H]
    tensor, each row reduced by a tree fixed by H alone."""
    import torch

    lib = load()
    _need(x, torch.bfloat16, 2, "x")
    _need(gain, torch.bfloat16, 1, "gain")
    t, h = (int(v) for v in x.shape)
    if int(gain.shape[0]) != h:
        raise ValueError("gain must have H = %d entries" % h)
    if out is None:
        out = torch.empty((t, h), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, 2, "out")
        if tuple(out.shape) != (t, h):
            raise ValueError("out must be [%d, %d]" % (t, h))
    check(lib.bi_rmsnorm(_p(x), _p(gain), t, h, float(eps), _p(out), _stream_ptr(stream)))
    return out


# ---- decode attention (include/bi_attn.h) --------------------------------------

class DecodeAttention:
    """Decode attention with a pinned split size: one query token per
    sequence against its KV cache, grouped-query heads, D = 128.  The handle
    owns the split workspace for up to ``max_batch`` sequences of up to
    ``max_seq_len`` keys."""

    def __init__(self, hq: int, hkv: int, split: int, max_batch: int, max_seq_len: int, head_dim: int = 128,
                 device=None):
        import torch

        lib = load()
        self.hq, self.hkv, self.d, self.split = int(hq), int(hkv), int(head_dim), int(split)
        self.max_batch, self.max_seq_len = int(max_batch), int(max_seq_len)
        self._lib = lib
        h = ctypes.c_void_p()
        with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
            st = lib.bi_attn_create(self.hq, self.hkv, self.d, self.split, self.max_batch, self.max_seq_len,
                                    ctypes.byref(h))
        check(st)
        self._h = h

    def __call__(self, q, k, v, seq_start, scale=None, out=None, stream=None):
        """q bf16 [B, Hq, D]; k, v bf16 [Ntok, Hkv, D]; seq_start int32 [B+1] on
        the device.  Returns fp32 [B, Hq, D]."""
        import torch

        _need(q, torch.bfloat16, 3, "q")
        _need(k, torch.bfloat16, 3, "k")
        _need(v, torch.bfloat16, 3, "v")
        _need(seq_start, torch.int32, 1, "seq_start")
        b = int(q.shape[0])
        if tuple(q.shape[1:]) != (self.hq, self.d) or tuple(k.shape[1:]) != (self.hkv, self.d) \
                or k.shape != v.shape or int(seq_start.shape[0]) != b + 1:
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / float(self.d) ** 0.5
        if out is None:
            out = torch.empty((b, self.hq, self.d), dtype=torch.float32, device=q.device)
        else:
            _need(out, torch.float32, 3, "out")
        check(self._lib.bi_attn_decode(self._h, _p(q), _p(k), _p(v), _p(seq_start), b, int(k.shape[0]),
                                       float(scale), _p(out), _stream_ptr(stream)))
        return out

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bi_attn_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass
