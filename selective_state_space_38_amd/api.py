"""PyTorch-facing binding of the selective-scan C ABI.

Argument marshalling only: every tensor must already be a contiguous tensor on
the current HIP device with the documented dtype; the functions pass raw
device pointers and the current stream to the library and raise
RuntimeError with the library's status text on failure.  No arithmetic of the
method happens here.
"""

import ctypes

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.SSM_F32, torch.bfloat16: _lib.SSM_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raise(rc):
    if rc != 0:
        raise RuntimeError(_lib.status_string(rc))


def fwd_plan(batch, seqlen, dim, dstate, dtype=torch.float32):
    """Launch plan the forward uses for these sizes (host-only query)."""
    lib = _lib.load()
    dims = _lib.SsmDims(batch, seqlen, dim, dstate, _DTYPES[dtype])
    plan = _lib.SsmFwdPlan()
    _raise(lib.ssm_fwd_plan_for(ctypes.byref(dims), ctypes.byref(plan)))
    return {f: getattr(plan, f) for f, _ in plan._fields_}


def _bbar_code(bbar):
    codes = {"delta": _lib.SSM_BBAR_DELTA, "zoh": _lib.SSM_BBAR_ZOH}
    if bbar not in codes:
        raise ValueError(f"bbar must be 'delta' or 'zoh', not {bbar!r}")
    return codes[bbar]


def _check_record_buffer(rec, dims, dev):
    if rec.device != dev or not rec.is_contiguous():
        raise ValueError("rec must be a contiguous tensor on the same device")
    if rec.numel() * rec.element_size() < _lib.load().ssm_fwd_record_bytes(ctypes.byref(dims)):
        raise ValueError("rec is too small (use record_buffer)")


def ckpt_buffer(u, dstate):
    """A float32 device buffer for the training pair's checkpoints (the state
    before every 8th step of every block of 64 channels) of activations u."""
    bsz, L, dim = u.shape
    dims = _lib.SsmDims(bsz, L, dim, dstate, _DTYPES[u.dtype])
    nbytes = _lib.load().ssm_ckpt_bytes(ctypes.byref(dims))
    _raise(nbytes if nbytes < 0 else 0)
    return torch.empty(nbytes // 4, dtype=torch.float32, device=u.device)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=True, return_last_state=False, h0=None,
                       out=None, last_state=None, bbar="delta", ckpt=None, no_alloc=False,
                       rec=None):
    """Selective-scan forward on the GPU.

    u, delta, z: [batch, L, dim]; B, C: [batch, L, dstate] (float32 or
    bfloat16, all the same); A: [dim, dstate], D, delta_bias: [dim] and
    h0: [batch, dim, dstate] float32.  Returns out (same dtype as u) and, with
    return_last_state, the float32 final state [batch, dim, dstate].
    bbar: "delta" (Bbar = Delta*B) or "zoh" (exact zero-order hold,
    (exp(Delta A) - 1)/A * B).  ckpt: a buffer from ckpt_buffer() to keep the
    backward's checkpoints (training mode; pass the same bbar to the backward).  no_alloc: use the
    entry point that allocates nothing (selective_scan_fwd_noalloc: its carry
    scratch is a static per-device array, so overlapping calls on one GPU
    race; Delta*B only, no checkpoints).  rec: a record_buffer filled by
    selective_scan_fwd_aggregate(rec=...) on the same inputs and bbar: every
    inner segment then starts from its kept carry (selective_scan_fwd_from_rec).
    """
    code = _bbar_code(bbar)
    if no_alloc and (ckpt is not None or code != _lib.SSM_BBAR_DELTA):
        raise ValueError("no_alloc covers the Delta*B forward without checkpoints only")
    if u.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {u.dtype}")
    bsz, L, dim = u.shape
    dstate = A.shape[1]
    dev = u.device
    act = u.dtype
    _check(u, "u", act, (bsz, L, dim), dev)
    _check(delta, "delta", act, (bsz, L, dim), dev)
    _check(z, "z", act, (bsz, L, dim), dev)
    _check(B, "B", act, (bsz, L, dstate), dev)
    _check(C, "C", act, (bsz, L, dstate), dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _check(h0, "h0", torch.float32, (bsz, dim, dstate), dev)
    if out is None:
        out = torch.empty_like(u)
    _check(out, "out", act, (bsz, L, dim), dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((bsz, dim, dstate), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", torch.float32, (bsz, dim, dstate), dev)
    dims = _lib.SsmDims(bsz, L, dim, dstate, _DTYPES[act])
    lib = _lib.load()
    if ckpt is not None:
        if ckpt.dtype != torch.float32 or ckpt.device != dev or not ckpt.is_contiguous():
            raise ValueError("ckpt must be a contiguous float32 tensor on the same device")
        if ckpt.numel() * 4 < lib.ssm_ckpt_bytes(ctypes.byref(dims)):
            raise ValueError("ckpt is too small (use ckpt_buffer)")
    if rec is not None:
        if ckpt is not None or no_alloc:
            raise ValueError("rec excludes ckpt and no_alloc")
        _check_record_buffer(rec, dims, dev)
    with torch.cuda.device(dev):
        if rec is not None:
            rc = lib.selective_scan_fwd_from_rec(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), code, _ptr(rec),
                _ptr(out), _ptr(last_state), ctypes.byref(dims), _stream(dev))
        elif ckpt is not None and code != _lib.SSM_BBAR_DELTA:
            rc = lib.selective_scan_fwd_train_ex(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), code, _ptr(out),
                _ptr(last_state), _ptr(ckpt), ctypes.byref(dims), _stream(dev))
        elif ckpt is not None:
            rc = lib.selective_scan_fwd_train(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), _ptr(out),
                _ptr(last_state), _ptr(ckpt), ctypes.byref(dims), _stream(dev))
        elif no_alloc:
            rc = lib.selective_scan_fwd_noalloc(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), _ptr(out),
                _ptr(last_state), ctypes.byref(dims), _stream(dev))
        elif code == _lib.SSM_BBAR_DELTA:
            rc = lib.selective_scan_fwd_h0(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), _ptr(out),
                _ptr(last_state), ctypes.byref(dims), _stream(dev))
        else:
            rc = lib.selective_scan_fwd_ex(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), code, _ptr(out),
                _ptr(last_state), ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return (out, last_state) if return_last_state else out


def record_buffer(u, dstate):
    """A device buffer for selective_scan_fwd_aggregate(rec=...) and
    selective_scan_fwd(rec=...) on activations u (the launch plan's inner
    segment carries)."""
    bsz, L, dim = u.shape
    dims = _lib.SsmDims(bsz, L, dim, dstate, _DTYPES[u.dtype])
    nbytes = _lib.load().ssm_fwd_record_bytes(ctypes.byref(dims))
    _raise(nbytes if nbytes < 0 else 0)
    return torch.empty(nbytes, dtype=torch.uint8, device=u.device)


def selective_scan_fwd_aggregate(u, delta, A, B, delta_bias=None, delta_softplus=True,
                                 h0=None, bbar="delta", sum_delta=None, state=None, rec=None):
    """Carry record of a sequence segment on the GPU: (sum of Delta
    [batch, dim], state after the last step [batch, dim, dstate]), both
    float32, from h0 (zeros when None).  Shapes and dtypes as
    selective_scan_fwd; C, D and z play no part.  rec (a record_buffer; h0
    must be None) also keeps the carries inside the segment for
    selective_scan_fwd(rec=...)."""
    code = _bbar_code(bbar)
    if rec is not None and h0 is not None:
        raise ValueError("a kept record starts from zero: h0 must be None")
    if u.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {u.dtype}")
    bsz, L, dim = u.shape
    dstate = A.shape[1]
    dev = u.device
    act = u.dtype
    _check(u, "u", act, (bsz, L, dim), dev)
    _check(delta, "delta", act, (bsz, L, dim), dev)
    _check(B, "B", act, (bsz, L, dstate), dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _check(h0, "h0", torch.float32, (bsz, dim, dstate), dev)
    if sum_delta is None:
        sum_delta = torch.empty((bsz, dim), dtype=torch.float32, device=dev)
    if state is None:
        state = torch.empty((bsz, dim, dstate), dtype=torch.float32, device=dev)
    _check(sum_delta, "sum_delta", torch.float32, (bsz, dim), dev)
    _check(state, "state", torch.float32, (bsz, dim, dstate), dev)
    dims = _lib.SsmDims(bsz, L, dim, dstate, _DTYPES[act])
    lib = _lib.load()
    if rec is not None:
        _check_record_buffer(rec, dims, dev)
    with torch.cuda.device(dev):
        if rec is not None:
            rc = lib.selective_scan_fwd_aggregate_rec(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(delta_bias),
                1 if delta_softplus else 0, code, _ptr(sum_delta), _ptr(state), _ptr(rec),
                ctypes.byref(dims), _stream(dev))
        else:
            rc = lib.selective_scan_fwd_aggregate(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(delta_bias),
                1 if delta_softplus else 0, _ptr(h0), code, _ptr(sum_delta), _ptr(state),
                ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return sum_delta, state


def selective_scan_carry_combine(sum_delta, agg, A, h0=None, h_in=None, h_out=None):
    """Start states of S consecutive segments from their carry records:
    sum_delta [S, batch, dim], agg [S, batch, dim, dstate] (float32, each
    from selective_scan_fwd_aggregate with h0=None).  Returns (h_in
    [S, batch, dim, dstate], h_out [batch, dim, dstate]): every segment's
    start state from h0 (zeros when None) and the state after the last."""
    S, bsz, dim, dstate = agg.shape
    dev = agg.device
    _check(sum_delta, "sum_delta", torch.float32, (S, bsz, dim), dev)
    _check(agg, "agg", torch.float32, (S, bsz, dim, dstate), dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(h0, "h0", torch.float32, (bsz, dim, dstate), dev)
    if h_in is None:
        h_in = torch.empty_like(agg)
    if h_out is None:
        h_out = torch.empty((bsz, dim, dstate), dtype=torch.float32, device=dev)
    _check(h_in, "h_in", torch.float32, (S, bsz, dim, dstate), dev)
    _check(h_out, "h_out", torch.float32, (bsz, dim, dstate), dev)
    dims = _lib.SsmDims(bsz, 1, dim, dstate, _lib.SSM_F32)
    lib = _lib.load()
    with torch.cuda.device(dev):
        rc = lib.selective_scan_carry_combine(
            _ptr(sum_delta), _ptr(agg), _ptr(A), _ptr(h0), _ptr(h_in), _ptr(h_out), S,
            ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return h_in, h_out


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dlast=None, ckpt=None, bbar="delta"):
    """Backward of selective_scan_fwd on the GPU (either input discretisation:
    bbar "delta" or "zoh", as the forward's).

    Inputs as in the forward, plus dout [batch, L, dim] (activation dtype),
    the gradient of the output, and dlast [batch, dim, dstate] float32
    (optional), the gradient of the final state.  Returns a dict of gradients:
    du, ddelta (of the raw dt), dz (if z is given) in the activation dtype;
    dB, dC [batch, L, dstate] in the activation dtype; dA [dim, dstate] and,
    for given D / delta_bias / h0, dD, ddt_bias, dh0 in float32.  ckpt: the
    buffer a training-mode selective_scan_fwd filled on the same inputs and
    the same bbar (the backward then skips its own forward pass).
    """
    code = _bbar_code(bbar)
    if u.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {u.dtype}")
    bsz, L, dim = u.shape
    dstate = A.shape[1]
    dev = u.device
    act = u.dtype
    for t, name, dt_, shp in ((u, "u", act, (bsz, L, dim)), (delta, "delta", act, (bsz, L, dim)),
                              (z, "z", act, (bsz, L, dim)), (dout, "dout", act, (bsz, L, dim)),
                              (B, "B", act, (bsz, L, dstate)), (C, "C", act, (bsz, L, dstate)),
                              (A, "A", torch.float32, (dim, dstate)),
                              (D, "D", torch.float32, (dim,)),
                              (delta_bias, "delta_bias", torch.float32, (dim,)),
                              (h0, "h0", torch.float32, (bsz, dim, dstate)),
                              (dlast, "dlast", torch.float32, (bsz, dim, dstate))):
        _check(t, name, dt_, shp, dev)
    if dout is None:
        raise ValueError("dout is required")
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
             dA=torch.empty((dim, dstate), dtype=torch.float32, device=dev),
             dB=torch.empty_like(B), dC=torch.empty_like(C))
    if D is not None:
        g["dD"] = torch.empty((dim,), dtype=torch.float32, device=dev)
    if z is not None:
        g["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        g["ddt_bias"] = torch.empty((dim,), dtype=torch.float32, device=dev)
    if h0 is not None:
        g["dh0"] = torch.empty((bsz, dim, dstate), dtype=torch.float32, device=dev)
    dims = _lib.SsmDims(bsz, L, dim, dstate, _DTYPES[act])
    lib = _lib.load()
    if ckpt is not None:
        if ckpt.dtype != torch.float32 or ckpt.device != dev or not ckpt.is_contiguous():
            raise ValueError("ckpt must be a contiguous float32 tensor on the same device")
        if ckpt.numel() * 4 < lib.ssm_ckpt_bytes(ctypes.byref(dims)):
            raise ValueError("ckpt is too small (use ckpt_buffer)")
    with torch.cuda.device(dev):
        head = [_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0), _ptr(dout), _ptr(dlast)]
        tail = [_ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddt_bias")),
                _ptr(g.get("dh0")), ctypes.byref(dims), _stream(dev)]
        if code != _lib.SSM_BBAR_DELTA:
            rc = lib.selective_scan_bwd_ex(*head[:10], code, *head[10:], _ptr(ckpt), *tail)
        elif ckpt is not None:
            rc = lib.selective_scan_bwd_ckpt(*head, _ptr(ckpt), *tail)
        else:
            rc = lib.selective_scan_bwd(*head, *tail)
    _raise(rc)
    return g


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           dt_softplus=True, out=None, bbar="delta"):
    """One decode step on the GPU, updating ``state`` in place.

    state: [batch, dim, dstate] float32; x, dt, z: [batch, dim] and
    B, C: [batch, dstate] (float32 or bfloat16, all the same); A, D, dt_bias
    and bbar as in the forward.  Returns out [batch, dim] in the activation
    dtype.
    """
    code = _bbar_code(bbar)
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    bsz, dim = x.shape
    dstate = A.shape[1]
    dev = x.device
    act = x.dtype
    _check(state, "state", torch.float32, (bsz, dim, dstate), dev)
    _check(x, "x", act, (bsz, dim), dev)
    _check(dt, "dt", act, (bsz, dim), dev)
    _check(z, "z", act, (bsz, dim), dev)
    _check(B, "B", act, (bsz, dstate), dev)
    _check(C, "C", act, (bsz, dstate), dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", act, (bsz, dim), dev)
    dims = _lib.SsmDims(bsz, 1, dim, dstate, _DTYPES[act])
    lib = _lib.load()
    with torch.cuda.device(dev):
        if code == _lib.SSM_BBAR_DELTA:
            rc = lib.selective_state_update(
                _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(dt_bias), 1 if dt_softplus else 0, _ptr(out), ctypes.byref(dims),
                _stream(dev))
        else:
            rc = lib.selective_state_update_ex(
                _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                _ptr(dt_bias), 1 if dt_softplus else 0, code, _ptr(out), ctypes.byref(dims),
                _stream(dev))
    _raise(rc)
    return out


def _act_code(activation):
    if activation not in ("silu", None):
        raise ValueError(f"activation must be 'silu' or None, not {activation!r}")
    return 1 if activation == "silu" else 0


def causal_conv1d_fwd(x, weight, bias=None, state_in=None, activation="silu",
                      return_final_state=False, out=None, state_out=None):
    """Causal depthwise conv1d (+ SiLU) on the GPU.

    x: [batch, L, dim] (float32 or bfloat16); weight: [dim, width] float32
    (width 1..4); bias: [dim]; state_in: [batch, dim, width - 1] float32, the
    inputs before t = 0 (zeros if None).  Returns out (same dtype as x) and,
    with return_final_state, the last width - 1 inputs [batch, dim, width - 1].
    """
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    bsz, L, dim = x.shape
    width = weight.shape[1]
    dev = x.device
    _check(x, "x", x.dtype, (bsz, L, dim), dev)
    _check(weight, "weight", torch.float32, (dim, width), dev)
    _check(bias, "bias", torch.float32, (dim,), dev)
    _check(state_in, "state_in", torch.float32, (bsz, dim, width - 1), dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", x.dtype, (bsz, L, dim), dev)
    if return_final_state and state_out is None:
        state_out = torch.empty((bsz, dim, width - 1), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", torch.float32, (bsz, dim, width - 1), dev)
    dims = _lib.SsmDims(bsz, L, dim, 1, _DTYPES[x.dtype])
    with torch.cuda.device(dev):
        rc = _lib.load().causal_conv1d_fwd(
            _ptr(x), _ptr(weight), _ptr(bias), _ptr(state_in), width, _act_code(activation),
            _ptr(out), _ptr(state_out) if state_out is not None and width > 1 else None,
            ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return (out, state_out) if return_final_state else out


def causal_conv1d_update(state, x, weight, bias=None, activation="silu", out=None):
    """One decode step of the causal conv1d on the GPU, shifting ``state``
    ([batch, dim, width - 1] float32) by one input in place.  x: [batch, dim].
    Returns out [batch, dim] in x's dtype."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    bsz, dim = x.shape
    width = weight.shape[1]
    dev = x.device
    _check(state, "state", torch.float32, (bsz, dim, width - 1), dev)
    _check(x, "x", x.dtype, (bsz, dim), dev)
    _check(weight, "weight", torch.float32, (dim, width), dev)
    _check(bias, "bias", torch.float32, (dim,), dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", x.dtype, (bsz, dim), dev)
    dims = _lib.SsmDims(bsz, 1, dim, 1, _DTYPES[x.dtype])
    with torch.cuda.device(dev):
        rc = _lib.load().causal_conv1d_update(
            _ptr(state) if width > 1 else None, _ptr(x), _ptr(weight), _ptr(bias), width,
            _act_code(activation), _ptr(out), ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return out


BLOCK_WEIGHTS = ("in_x", "in_z", "conv_w", "conv_b", "x_dt", "x_B", "x_C", "dt", "dt_bias",
                 "A", "D", "out")


def mamba_block_fwd(x_in, weights, out=None):
    """Forward of one Mamba block on the GPU (projections on hipBLASLt, conv1d
    + SiLU and the gated selective scan in this library's kernels).

    x_in: [batch, L, d_model] (float32 or bfloat16).  ``weights``: dict with
    the projection weights in the layout of a linear layer's weight,
    [out, in]: in_x, in_z [d_inner, d_model], x_dt [r, d_inner], x_B, x_C
    [N, d_inner], dt [d_inner, r], out [d_model, d_inner] in x_in's dtype;
    and conv_w [d_inner, K], A [d_inner, N], optional conv_b, dt_bias, D
    [d_inner] in float32.  Returns out [batch, L, d_model].
    """
    if x_in.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x_in.dtype}")
    bsz, L, dm = x_in.shape
    dev = x_in.device
    act = x_in.dtype
    di = weights["in_x"].shape[0]
    n = weights["A"].shape[1]
    r = weights["x_dt"].shape[0]
    k = weights["conv_w"].shape[1]
    shapes = dict(in_x=((di, dm), act), in_z=((di, dm), act), conv_w=((di, k), torch.float32),
                  conv_b=((di,), torch.float32), x_dt=((r, di), act), x_B=((n, di), act),
                  x_C=((n, di), act), dt=((di, r), act), dt_bias=((di,), torch.float32),
                  A=((di, n), torch.float32), D=((di,), torch.float32), out=((dm, di), act))
    _check(x_in, "x_in", act, (bsz, L, dm), dev)
    for name, (shp, dt_) in shapes.items():
        if weights.get(name) is None and name not in ("conv_b", "dt_bias", "D"):
            raise ValueError(f"weight {name} is required")
        _check(weights.get(name), name, dt_, shp, dev)
    if out is None:
        out = torch.empty_like(x_in)
    _check(out, "out", act, (bsz, L, dm), dev)
    wts = _lib.MambaBlockWeights(*[None if weights.get(nm) is None else weights[nm].data_ptr()
                                   for nm in BLOCK_WEIGHTS])
    dims = _lib.MambaBlockDims(bsz, L, dm, di, n, r, k, _DTYPES[act])
    with torch.cuda.device(dev):
        rc = _lib.load().mamba_block_fwd(_ptr(x_in), ctypes.byref(wts), _ptr(out),
                                         ctypes.byref(dims), _stream(dev))
    _raise(rc)
    return out


def check_device_errors(device=None):
    """Synchronises the current stream and raises if a carry wait timed out."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    _raise(_lib.load().ssm_check_device_errors(_stream(dev)))
