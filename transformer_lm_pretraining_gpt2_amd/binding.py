"""ctypes binding of libgpt2mi.so (the C ABI in include/gpt2.h).

Argument marshalling only: every step of the training step runs in the HIP
library.  torch supplies device memory and the stream.  There is no CPU
fallback: if the library is missing, `lib()` raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgpt2mi.so")

GPT2_FP32, GPT2_BF16 = 0, 1
GPT2_RECOMPUTE_GELU = 0x100  # OR into the precision: MLP activation recompute
GPT2_FP8_FWD = 0x200  # OR into the precision (bf16 only): forward products on FP8 E4M3 copies
ERRORS = {0: "GPT2_OK", -1: "GPT2_ERR_CONFIG", -2: "GPT2_ERR_SHAPE", -3: "GPT2_ERR_ARG", -4: "GPT2_ERR_HIP",
          -5: "GPT2_ERR_TOKEN_RANGE", -6: "GPT2_ERR_NONFINITE", -7: "GPT2_ERR_WORKSPACE"}


class Gpt2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class CConfig(ctypes.Structure):
    _fields_ = [("vocab_size", ctypes.c_int32), ("padded_vocab_size", ctypes.c_int32), ("n_layer", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_embd", ctypes.c_int32), ("max_seq_len", ctypes.c_int32)]


class CTensorDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_int64), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("decay", ctypes.c_int32)]


# (name, restype, argtypes) of every exported function
_P, _I, _I64, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
_CFG = ctypes.POINTER(CConfig)
SIGNATURES = [
    ("gpt2_num_params", _I64, [_CFG]),
    ("gpt2_num_decay_params", _I64, [_CFG]),
    ("gpt2_param_layout", _I, [_CFG, ctypes.POINTER(CTensorDesc), _I]),
    ("gpt2_workspace_bytes", _I64, [_CFG, _I, _I, _I]),
    ("gpt2_check_shapes", _I, [_CFG, _I, _I]),
    ("gpt2_init", _I, [ctypes.POINTER(_P), _CFG, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I64, _P]),
    ("gpt2_destroy", None, [_P]),
    ("gpt2_refresh_params", _I, [_P]),
    ("gpt2_set_stream", _I, [_P, _P]),
    ("gpt2_set_overlap", _I, [_P, _I]),
    ("gpt2_forward", _I, [_P, _P, _P, _P, _P]),
    ("gpt2_eval", _I, [_P, _P, _P, _P, _P]),
    ("gpt2_residual", _I, [_P, _I, ctypes.POINTER(_P)]),
    ("gpt2_backward", _I, [_P, _I, _I]),
    ("gpt2_adamw_step", _I, [_P, _I, _F, _F, _F, _F, _F, _F, _P]),
    ("gpt2_adamw_step_noalloc", _I, [_P, _P, _P, _P, _P, _I64, _I64, _I, _F, _F, _F, _F, _F, _F, _P, _P]),
    ("gpt2_sync_status", _I, [_P]),
    ("gpt2_last_error", ctypes.c_char_p, [_P]),
    ("gpt2_strerror", ctypes.c_char_p, [_I]),
    ("gpt2_kernel_count", _I, []),
    ("gpt2_kernel_name", ctypes.c_char_p, [_I]),
    ("gpt2_timing_enable", _I, [_P, _I, _I]),
    ("gpt2_timing_read", _I, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_double)]),
]

_lib = None


def lib():
    """Loads the HIP library; raises if it has not been built.

    torch is imported first: its bundled HIP runtime has the same soname
    (libamdhip64.so.7) as the one the library links, so the loader binds the
    library to torch's runtime and the process has a single HIP runtime
    (device memory and streams from torch are then valid in the library)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (must precede the CDLL below)

        path = os.environ.get("GPT2MI_LIBRARY", LIB_PATH)  # another build of the same library, if given
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(make -C transformer_lm_pretraining_gpt2_amd/csrc)")
        L = ctypes.CDLL(path)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def cconfig(m):
    return CConfig(m.vocab_size, m.padded_vocab_size, m.n_layer, m.n_head, m.n_embd, m.max_seq_len)


def num_params(m):
    return int(lib().gpt2_num_params(ctypes.byref(cconfig(m))))


def num_decay_params(m):
    return int(lib().gpt2_num_decay_params(ctypes.byref(cconfig(m))))


def param_layout(m):
    c = cconfig(m)
    n = lib().gpt2_param_layout(ctypes.byref(c), None, 0)
    if n < 0:
        raise Gpt2Error(n, "param_layout")
    arr = (CTensorDesc * n)()
    lib().gpt2_param_layout(ctypes.byref(c), arr, n)
    return [dict(name=d.name.decode(), offset=int(d.offset), rows=int(d.rows), cols=int(d.cols), decay=int(d.decay))
            for d in arr]


def workspace_bytes(m, B, T, precision):
    return int(lib().gpt2_workspace_bytes(ctypes.byref(cconfig(m)), B, T, precision))


def check_shapes(m, B, T):
    return int(lib().gpt2_check_shapes(ctypes.byref(cconfig(m)), B, T))


def adamw_step_noalloc(params, params_lp, grads, m, v, n_decay, step, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                       weight_decay=0.1, grad_clip=1.0, grad_norm=None, stream=None):
    """gpt2_adamw_step_noalloc on torch device tensors (fp32 [n] params, grads,
    m, v; bf16 [n] params_lp or None; fp32 [1] grad_norm), enqueued on `stream`
    (default: torch's current stream).  Raises Gpt2Error on a refused call."""
    import torch

    st = stream if stream is not None else torch.cuda.current_stream()
    p = lambda t: t.data_ptr() if t is not None else None
    rc = lib().gpt2_adamw_step_noalloc(p(params), p(params_lp), p(grads), p(m), p(v), params.numel(), n_decay, step, lr,
                                       beta1, beta2, eps, weight_decay, grad_clip, p(grad_norm), st.cuda_stream)
    if rc != 0:
        raise Gpt2Error(rc, "adamw_step_noalloc")


def kernel_names():
    return [lib().gpt2_kernel_name(i).decode() for i in range(lib().gpt2_kernel_count())]


class TrainStep:
    """Device buffers plus a library handle for micro-batches of B x T tokens.

    params/grads/m/v are fp32 torch tensors [N] on the device; params_lp is the
    bf16 copy (bf16 precision only); workspace is a uint8 tensor.
    """

    def __init__(self, model, B, T, precision, device="cuda", stream=None, recompute=False, fp8=False):
        import torch

        self.torch = torch
        self.model, self.B, self.T = model, B, T
        self.precision = GPT2_BF16 if precision in ("bf16", GPT2_BF16) else GPT2_FP32
        self.recompute = bool(recompute)
        self.fp8 = bool(fp8)
        flags = self.precision | (GPT2_RECOMPUTE_GELU if self.recompute else 0) | (GPT2_FP8_FWD if self.fp8 else 0)
        self.N = num_params(model)
        if self.N < 0:
            raise Gpt2Error(self.N, "invalid config")
        ws = workspace_bytes(model, B, T, flags)
        if ws < 0:
            raise Gpt2Error(ws, "invalid shapes")
        f32 = dict(dtype=torch.float32, device=device)
        self.params = torch.zeros(self.N, **f32)
        self.grads = torch.zeros(self.N, **f32)
        self.m = torch.zeros(self.N, **f32)
        self.v = torch.zeros(self.N, **f32)
        self.params_lp = torch.zeros(self.N, dtype=torch.bfloat16, device=device) if self.precision == GPT2_BF16 else None
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.layout = param_layout(model)
        h = ctypes.c_void_p()
        rc = lib().gpt2_init(ctypes.byref(h), ctypes.byref(cconfig(model)), flags, B, T,
                             self.params.data_ptr(), self.params_lp.data_ptr() if self.params_lp is not None else None,
                             self.grads.data_ptr(), self.m.data_ptr(), self.v.data_ptr(), self.workspace.data_ptr(),
                             ws, self.stream.cuda_stream)
        if rc != 0:
            raise Gpt2Error(rc, "gpt2_init")
        self.h = h

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and _lib is not None:
            _lib.gpt2_destroy(h)
            self.h = None

    def _check(self, rc, what):
        if rc != 0:
            raise Gpt2Error(rc, f"{what}: {lib().gpt2_last_error(self.h).decode()}")

    def set_params(self, flat):
        """Copies host parameters (numpy fp32 [N]) in and refreshes the bf16 copy."""
        t = self.torch.from_numpy(np.ascontiguousarray(flat, dtype=np.float32))
        self.params.copy_(t)
        self.m.zero_()
        self.v.zero_()
        self.torch.cuda.current_stream().synchronize()
        self._check(lib().gpt2_refresh_params(self.h), "refresh_params")

    def forward(self, ids, targets=None, loss=None, loss_rows=None):
        p = lambda t: t.data_ptr() if t is not None else None
        self._check(lib().gpt2_forward(self.h, p(ids), p(targets), p(loss), p(loss_rows)), "forward")

    def evaluate(self, ids, targets, loss=None, loss_rows=None):
        """Forward-only loss (no backward state kept)."""
        p = lambda t: t.data_ptr() if t is not None else None
        self._check(lib().gpt2_eval(self.h, p(ids), p(targets), p(loss), p(loss_rows)), "eval")

    def residual_ptr(self, layer):
        """Device address of the fp32 residual stream [B*T, C] saved at the input
        of block `layer` by the last forward (layer n_layer: the final LayerNorm's
        input; layer 0: the embedding output)."""
        ptr = ctypes.c_void_p()
        self._check(lib().gpt2_residual(self.h, layer, ctypes.byref(ptr)), "residual")
        return int(ptr.value)

    def residual(self, layer):
        """Copy of that residual stream as a float32 torch tensor [B*T, C] on the device."""
        torch = self.torch
        n = self.B * self.T * self.model.n_embd
        off = self.residual_ptr(layer) - self.workspace.data_ptr()
        assert 0 <= off and off + 4 * n <= self.workspace.numel()
        return self.workspace[off:off + 4 * n].view(torch.float32).view(self.B * self.T, self.model.n_embd).clone()

    def backward(self, micro_step=0, grad_accum_steps=1):
        self._check(lib().gpt2_backward(self.h, micro_step, grad_accum_steps), "backward")

    def adamw_step(self, step, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_clip=1.0, grad_norm=None):
        self._check(lib().gpt2_adamw_step(self.h, step, lr, beta1, beta2, eps, weight_decay, grad_clip,
                                          grad_norm.data_ptr() if grad_norm is not None else None), "adamw_step")

    def sync_status(self):
        """Returns the deferred status code (0 = ok) after synchronising."""
        return int(lib().gpt2_sync_status(self.h))

    def set_stream(self, stream):
        """Stream later calls enqueue on (a torch.cuda.Stream)."""
        self._check(lib().gpt2_set_stream(self.h, stream.cuda_stream), "set_stream")
        self.stream = stream

    def set_overlap(self, enable=True):
        """Weight-gradient products on the handle's second stream (default) or all on one stream."""
        self._check(lib().gpt2_set_overlap(self.h, 1 if enable else 0), "set_overlap")

    def timing_enable(self, kernel_name, enable=True):
        kid = kernel_names().index(kernel_name)
        self._check(lib().gpt2_timing_enable(self.h, kid, 1 if enable else 0), "timing_enable")

    def timing_read(self):
        ms, n, fl = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double()
        self._check(lib().gpt2_timing_read(self.h, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl)), "timing_read")
        return ms.value, n.value, fl.value
