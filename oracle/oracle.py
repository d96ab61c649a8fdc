"""ctypes wrapper of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The product library never imports it.

Arrays are numpy; `R` selects the real type of the oracle instantiation
(np.float64 for parity references and finite differences, np.float32 for the
plain fp32 variant).  A config is any object with vocab_size,
padded_vocab_size, n_layer, n_head, n_embd and max_seq_len attributes, or a
6-tuple in that order.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=False):
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["make", "-s", "-C", _HERE] + (["-B"] if force else []), check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_num_params.restype = i64
        L.oracle_num_params.argtypes = [P]
        L.oracle_num_tensors.restype = ctypes.c_int
        L.oracle_num_tensors.argtypes = [P]
        L.oracle_tensor.restype = ctypes.c_int
        L.oracle_tensor.argtypes = [P, ctypes.c_int, ctypes.c_char_p, P, P, P, P]
        for sfx, R in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
            f = getattr(L, f"oracle_{sfx}_fwd_bwd")
            f.restype = R
            f.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, R, P, P]
            f = getattr(L, f"oracle_{sfx}_grad_norm")
            f.restype = R
            f.argtypes = [P, i64]
            f = getattr(L, f"oracle_{sfx}_clip_grads")
            f.restype = R
            f.argtypes = [P, i64, R]
            f = getattr(L, f"oracle_{sfx}_adamw")
            f.restype = ctypes.c_int
            f.argtypes = [P, P, P, P, P, ctypes.c_int, R, R, R, R, R]
            getattr(L, f"oracle_{sfx}_linear").argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int]
            getattr(L, f"oracle_{sfx}_linear_bwd").argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int]
            getattr(L, f"oracle_{sfx}_layernorm").argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, R]
            getattr(L, f"oracle_{sfx}_layernorm_bwd").argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int]
            getattr(L, f"oracle_{sfx}_gelu").argtypes = [P, P, P, i64]
            getattr(L, f"oracle_{sfx}_attention").argtypes = [P, P, P] + [ctypes.c_int] * 4
            getattr(L, f"oracle_{sfx}_attention_bwd").argtypes = [P, P, P] + [ctypes.c_int] * 4
            getattr(L, f"oracle_{sfx}_cross_entropy").argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, R]
        for fn in ("linear", "linear_bwd", "layernorm", "layernorm_bwd", "gelu", "attention", "attention_bwd", "cross_entropy"):
            for sfx in ("f64", "f32"):
                getattr(L, f"oracle_{sfx}_{fn}").restype = None
        _lib = L
    return _lib


def _cfg_arr(cfg):
    if hasattr(cfg, "vocab_size"):
        t = (cfg.vocab_size, cfg.padded_vocab_size, cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.max_seq_len)
    else:
        t = tuple(cfg)
    return np.asarray(t, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _sfx(R):
    R = np.dtype(R)
    if R == np.float64:
        return "f64"
    if R == np.float32:
        return "f32"
    raise ValueError(R)


def _chk(a, R, name):
    if a is None:
        return None
    if a.dtype != np.dtype(R) or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name} must be a C-contiguous {np.dtype(R)} array")
    return a


def num_params(cfg):
    return int(lib().oracle_num_params(_p(_cfg_arr(cfg))))


def param_layout(cfg):
    """List of dicts {name, offset, rows, cols, decay} in flat order."""
    c = _cfg_arr(cfg)
    n = lib().oracle_num_tensors(_p(c))
    out = []
    name = ctypes.create_string_buffer(32)
    off, r, cc, d = np.zeros(1, np.int64), np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(1, np.int32)
    for i in range(n):
        if lib().oracle_tensor(_p(c), i, name, _p(off), _p(r), _p(cc), _p(d)) != 0:
            raise RuntimeError("oracle_tensor failed")
        out.append(dict(name=name.value.decode(), offset=int(off[0]), rows=int(r[0]), cols=int(cc[0]), decay=int(d[0])))
    return out


def fwd_bwd(cfg, B, T, params, ids, tgt, grad_scale=1.0, grads=None, row_loss=None, R=np.float64):
    """Mean loss of one micro-batch; adds grad_scale * dloss/dparams into `grads` if given."""
    s = _sfx(R)
    _chk(params, R, "params"); _chk(grads, R, "grads"); _chk(row_loss, R, "row_loss")
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    tgt = np.ascontiguousarray(tgt, dtype=np.int32)
    assert ids.size == B * T and tgt.size == B * T
    f = getattr(lib(), f"oracle_{s}_fwd_bwd")
    return float(f(_p(_cfg_arr(cfg)), B, T, _p(params), _p(ids), _p(tgt), grad_scale, _p(grads), _p(row_loss)))


def grad_norm(g, R=np.float64):
    return float(getattr(lib(), f"oracle_{_sfx(R)}_grad_norm")(_p(_chk(g, R, "g")), g.size))


def clip_grads(g, clip, R=np.float64):
    """Scales g in place when its global norm exceeds clip; returns the pre-clip norm."""
    return float(getattr(lib(), f"oracle_{_sfx(R)}_clip_grads")(_p(_chk(g, R, "g")), g.size, clip))


def adamw(cfg, p, g, m, v, t, lr, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, R=np.float64):
    for a, nm in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _chk(a, R, nm)
    rc = getattr(lib(), f"oracle_{_sfx(R)}_adamw")(_p(_cfg_arr(cfg)), _p(p), _p(g), _p(m), _p(v), t, lr, b1, b2, eps, wd)
    if rc != 0:
        raise ValueError("oracle adamw rejected its arguments")


def train_step(cfg, micro_batches, params, m, v, step, lr, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, clip=1.0, R=np.float64):
    """One optimizer step over K micro-batches [(ids[B,T], tgt[B,T]), ...].

    Updates params, m, v in place.  Returns (mean loss over micro-batches,
    pre-clip grad norm, grads after clipping, per-micro-batch row losses)."""
    K = len(micro_batches)
    grads = np.zeros_like(params)
    losses, rows = [], []
    for ids, tgt in micro_batches:
        B, T = ids.shape
        rl = np.zeros(B * T, dtype=R)
        losses.append(fwd_bwd(cfg, B, T, params, ids, tgt, 1.0 / K, grads, rl, R=R))
        rows.append(rl)
    norm = clip_grads(grads, clip, R=R)
    adamw(cfg, params, grads, m, v, step, lr, b1, b2, eps, wd, R=R)
    return float(np.mean(losses)), norm, grads, rows


# ---- building blocks, exposed for the pin tests ---------------------------------

def linear(x, W, b=None, R=np.float64):
    M, K = x.shape
    N = W.shape[0]
    y = np.zeros((M, N), dtype=R)
    getattr(lib(), f"oracle_{_sfx(R)}_linear")(_p(y), _p(_chk(x, R, "x")), _p(_chk(W, R, "W")), _p(_chk(b, R, "b")), M, N, K)
    return y


def linear_bwd(dy, x, W, R=np.float64):
    M, N = dy.shape
    K = x.shape[1]
    dx = np.zeros((M, K), dtype=R)
    dW = np.zeros((N, K), dtype=R)
    db = np.zeros(N, dtype=R)
    getattr(lib(), f"oracle_{_sfx(R)}_linear_bwd")(_p(dx), _p(dW), _p(db), _p(_chk(dy, R, "dy")), _p(_chk(x, R, "x")), _p(_chk(W, R, "W")), M, N, K)
    return dx, dW, db


def layernorm(x, g, b, eps=1e-5, R=np.float64):
    M, C = x.shape
    y = np.zeros_like(x)
    mean = np.zeros(M, dtype=R)
    rstd = np.zeros(M, dtype=R)
    getattr(lib(), f"oracle_{_sfx(R)}_layernorm")(_p(y), _p(mean), _p(rstd), _p(_chk(x, R, "x")), _p(_chk(g, R, "g")), _p(_chk(b, R, "b")), M, C, eps)
    return y, mean, rstd


def layernorm_bwd(dy, x, mean, rstd, g, R=np.float64):
    M, C = x.shape
    dx = np.zeros_like(x)
    dg = np.zeros(C, dtype=R)
    db = np.zeros(C, dtype=R)
    getattr(lib(), f"oracle_{_sfx(R)}_layernorm_bwd")(_p(dx), _p(dg), _p(db), _p(_chk(dy, R, "dy")), _p(x), _p(mean), _p(rstd), _p(g), M, C)
    return dx, dg, db


def gelu(x, R=np.float64):
    x = _chk(np.ascontiguousarray(x, dtype=R), R, "x")
    y = np.zeros_like(x)
    d = np.zeros_like(x)
    getattr(lib(), f"oracle_{_sfx(R)}_gelu")(_p(y), _p(d), _p(x), x.size)
    return y, d


def attention(qkv, B, T, NH, hd, want_probs=False, R=np.float64):
    C = NH * hd
    y = np.zeros((B * T, C), dtype=R)
    probs = np.zeros((B, NH, T, T), dtype=R) if want_probs else None
    getattr(lib(), f"oracle_{_sfx(R)}_attention")(_p(y), _p(probs), _p(_chk(qkv, R, "qkv")), B, T, NH, hd)
    return (y, probs) if want_probs else y


def attention_bwd(dy, qkv, B, T, NH, hd, R=np.float64):
    dqkv = np.zeros_like(qkv)
    getattr(lib(), f"oracle_{_sfx(R)}_attention_bwd")(_p(dqkv), _p(_chk(dy, R, "dy")), _p(_chk(qkv, R, "qkv")), B, T, NH, hd)
    return dqkv


def cross_entropy(logits, tgt, V, scale=1.0, want_grad=True, R=np.float64):
    M, ld = logits.shape
    rl = np.zeros(M, dtype=R)
    dz = np.zeros_like(logits) if want_grad else None
    tgt = np.ascontiguousarray(tgt, dtype=np.int32)
    getattr(lib(), f"oracle_{_sfx(R)}_cross_entropy")(_p(rl), _p(dz), _p(_chk(logits, R, "logits")), _p(tgt), M, V, ld, scale)
    return (rl, dz) if want_grad else rl
