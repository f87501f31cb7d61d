"""MI355X-native 4-bit weight-only GEMM (INT4 group-wise asymmetric and NF4).

Python face of the C ABI in ``include/w4a16.h``; each function here has the
name of the C entry point it calls and only marshals torch tensors (device
memory) and the current stream into it.  All arithmetic runs in the HIP
kernels of ``libw4a16.so`` -- there is no CPU or PyTorch fallback: calling
anything without the built library (or without a GPU) raises.

Typical flow (weights quantized at load time, repacked once, then many calls):

    qw, sc, qz = w4a16_quantize_rtn(W, group_size=128, g_idx=g_idx, perm=perm)
    packed = w4a16_repack(qw, sc, qz, g_idx)       # dict of device tensors
    y = w4a16_gemm(x, packed)                      # y = x @ dequant(W)^T
"""

import ctypes

import torch

from . import _lib
from ._lib import W4A16Error  # noqa: F401

F16, BF16 = 0, 1
GROUP = 128

_DT = {torch.float16: F16, torch.bfloat16: BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, numel=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))


def version():
    return _lib.lib().w4a16_version()


def w4a16_set_timing_events(start_event, stop_event):
    """Attach raw hipEvent_t handles (ints) to the next GEMM kernel launch."""
    _lib.check(_lib.lib().w4a16_set_timing_events(ctypes.c_void_p(start_event),
                                                  ctypes.c_void_p(stop_event)),
               "w4a16_set_timing_events")


def w4a16_repacked_bytes(K, N, group_size=GROUP, bits=4):
    L = _lib.lib()
    if bits == 4:
        out = [L.w4a16_repacked_bytes(K, N, group_size, w) for w in (0, 1, 2)]
    else:
        out = [L.w4a16_repacked_bytes_bits(K, N, group_size, bits, w) for w in (0, 1, 2)]
    if min(out) < 0:
        raise W4A16Error("w4a16_repacked_bytes: invalid shape K=%d N=%d G=%d" % (K, N, group_size))
    return tuple(out)


def w4a16_workspace_bytes(M, N, K, group_size=GROUP):
    return int(_lib.lib().w4a16_workspace_bytes(M, N, K, group_size))


def nf4_workspace_bytes(M, N, K, blocksize=64):
    return int(_lib.lib().nf4_workspace_bytes(M, N, K, blocksize))


def _names(fn, *args):
    buf = ctypes.create_string_buffer(1024)
    n = ctypes.c_int64(0)
    _lib.check(fn(*args, buf, len(buf), ctypes.byref(n)), fn.__name__)
    return buf.value.decode()


def w4a16_gemm_plan(M, N, K, group_size=GROUP, bits=4, dtype=torch.float16, perm=False,
                    x_scale=False, workspace=True):
    """Kernels a w4a16_gemm call of this shape launches (host-only query): a
    list of instantiation names as the profiler reports them, in launch order."""
    s = _names(_lib.lib().w4a16_gemm_plan, M, N, K, group_size, bits, _DT[dtype], int(perm),
               int(x_scale), int(workspace))
    return s.split(" + ")


def nf4_gemm_plan(M, N, K, blocksize=64, dtype=torch.bfloat16, workspace=True):
    """Kernels an nf4_gemm call of this shape launches (host-only query)."""
    return _names(_lib.lib().nf4_gemm_plan, M, N, K, blocksize, _DT[dtype],
                  int(workspace)).split(" + ")


def workspace(nbytes, device="cuda"):
    """A zero-filled workspace of at least ``nbytes`` (None when 0)."""
    if nbytes <= 0:
        return None
    return torch.zeros((nbytes + 255) // 256 * 64, dtype=torch.int32, device=device)


def w4a16_make_perm(g_idx, group_size=GROUP, stream=None):
    _need(g_idx, torch.int32, "g_idx")
    perm = torch.empty_like(g_idx)
    nt = ctypes.c_int32(0)
    _lib.check(_lib.lib().w4a16_make_perm(_ptr(g_idx), g_idx.numel(), group_size, _ptr(perm),
                                          ctypes.byref(nt), _stream(stream)), "w4a16_make_perm")
    return perm, bool(nt.value)


def _group(K, group_size):
    """The group size in elements (-1 is per-channel: one group of K)."""
    return K if group_size == -1 else group_size


def w4a16_quantize_rtn(W, group_size=GROUP, g_idx=None, perm=None, sym=False, bits=4,
                       stream=None):
    """RTN group quantization of W [N, K] fp32 -> (qweight, scales, qzeros), with
    ``bits``-bit codes (3, 4 or 8) in the canonical packing.

    ``sym=True``: symmetric codes (zero point fixed, stored offset by
    2^(bits-1)) and qzeros = None."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    G = _group(K, group_size)
    if g_idx is not None and perm is None:
        perm, _ = w4a16_make_perm(g_idx, group_size, stream)
    dev = W.device
    qweight = torch.empty((K * bits // 32, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // G, N), dtype=torch.float16, device=dev)
    qzeros = (None if sym else
              torch.empty((K // G, N * bits // 32), dtype=torch.int32, device=dev))
    L = _lib.lib()
    args = (_ptr(qweight), _ptr(scales), _ptr(qzeros), _stream(stream))
    if bits == 4:
        _lib.check(L.w4a16_quantize_rtn(_ptr(W), _ptr(g_idx), _ptr(perm), N, K, group_size,
                                        *args), "w4a16_quantize_rtn")
    else:
        _lib.check(L.w4a16_quantize_rtn_bits(_ptr(W), _ptr(g_idx), _ptr(perm), N, K, group_size,
                                             bits, *args), "w4a16_quantize_rtn_bits")
    return qweight, scales, qzeros


def w4a16_repack(qweight, scales, qzeros, g_idx=None, group_size=GROUP, bits=4, stream=None):
    """Repack canonical tensors of ``bits``-bit codes; returns dict(codes, scales,
    zeros, perm, K, N, group_size, bits).

    ``qzeros=None`` is a symmetric weight: the result then has zeros = None."""
    _need(qweight, torch.int32, "qweight")
    Kw, N = qweight.shape
    K = Kw * 32 // bits
    G = _group(K, group_size)
    _need(scales, torch.float16, "scales", (K // G) * N)
    if qzeros is not None:
        _need(qzeros, torch.int32, "qzeros", (K // G) * (N * bits // 32))
    nc, ns, nz = w4a16_repacked_bytes(K, N, group_size, bits)
    dev = qweight.device
    codes_r = torch.empty(nc, dtype=torch.uint8, device=dev)
    scales_r = torch.empty(ns // 2, dtype=torch.float16, device=dev)
    zeros_r = None if qzeros is None else torch.empty(nz // 4, dtype=torch.int32, device=dev)
    perm = None
    if g_idx is not None:
        _need(g_idx, torch.int32, "g_idx", K)
        perm = torch.empty(K, dtype=torch.int32, device=dev)
    used = ctypes.c_int32(0)
    L = _lib.lib()
    head = (_ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(g_idx), K, N, group_size)
    tail = (_ptr(codes_r), _ptr(scales_r), _ptr(zeros_r), _ptr(perm), ctypes.byref(used),
            _stream(stream))
    if bits == 4:
        _lib.check(L.w4a16_repack(*head, *tail), "w4a16_repack")
    else:
        _lib.check(L.w4a16_repack_bits(*head, bits, *tail), "w4a16_repack_bits")
    return {"codes": codes_r, "scales": scales_r, "zeros": zeros_r,
            "perm": perm if used.value else None, "K": K, "N": N, "group_size": group_size,
            "bits": bits}


def w4a16_gemm(x, packed, out=None, workspace=None, use_workspace=True, stream=None):
    """y = x @ dequant(W)^T for x [M, K] fp16/bf16 (weights from w4a16_repack)."""
    return _int4_gemm(x, None, packed, out, workspace, use_workspace, stream)


def w4a16_gemm_xscale(x, x_scale, packed, out=None, workspace=None, use_workspace=True,
                      stream=None):
    """y = (x / s) @ dequant(W)^T: AWQ input scales s [K] (x's dtype) applied
    by the GEMM itself."""
    _need(x_scale, x.dtype, "x_scale", packed["K"])
    return _int4_gemm(x, x_scale, packed, out, workspace, use_workspace, stream)


def _int4_gemm(x, x_scale, packed, out, workspace, use_workspace, stream):
    if x.dtype not in _DT:
        raise TypeError("x must be float16 or bfloat16")
    _need(x, x.dtype, "x")
    K, N, G = packed["K"], packed["N"], packed["group_size"]
    M = x.numel() // K
    if x.shape[-1] != K:
        raise ValueError("x last dim %d != K %d" % (x.shape[-1], K))
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _need(out, x.dtype, "out", M * N)
    ws_bytes = 0
    if use_workspace:
        need = w4a16_workspace_bytes(M, N, K, G)
        if workspace is None and need > 0:
            workspace = _ws_cache(x.device, need, stream)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    else:
        workspace = None
    L = _lib.lib()
    bits = packed.get("bits", 4)
    wts = (_ptr(packed["codes"]), _ptr(packed["scales"]), _ptr(packed["zeros"]),
           _ptr(packed["perm"]), G)
    rest = (_ptr(out), M, N, K, _DT[x.dtype], _ptr(workspace), ws_bytes, _stream(stream))
    if bits != 4:
        _lib.check(L.w4a16_gemm_bits(_ptr(x), _ptr(x_scale), *wts, bits, *rest),
                   "w4a16_gemm_bits")
    elif x_scale is None:
        _lib.check(L.w4a16_gemm(_ptr(x), *wts, *rest), "w4a16_gemm")
    else:
        _lib.check(L.w4a16_gemm_xscale(_ptr(x), _ptr(x_scale), *wts, *rest), "w4a16_gemm_xscale")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def w4a16_gemm_noalloc(x, packed, x_scale=None, out=None, stream=None):
    """y = (x [/ s]) @ dequant(W)^T through the entry point that allocates
    nothing (the library's fixed per-GPU scratch instead of a workspace);
    ``out`` may be given to avoid the output allocation here too."""
    if x.dtype not in _DT:
        raise TypeError("x must be float16 or bfloat16")
    _need(x, x.dtype, "x")
    K, N, G = packed["K"], packed["N"], packed["group_size"]
    M = x.numel() // K
    if x_scale is not None:
        _need(x_scale, x.dtype, "x_scale", K)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _need(out, x.dtype, "out", M * N)
    _lib.check(_lib.lib().w4a16_gemm_noalloc(
        _ptr(x), _ptr(x_scale), _ptr(packed["codes"]), _ptr(packed["scales"]),
        _ptr(packed["zeros"]), _ptr(packed["perm"]), G, packed.get("bits", 4), _ptr(out), M, N,
        K, _DT[x.dtype], _stream(stream)), "w4a16_gemm_noalloc")
    return out


def w4a16_dequant(packed, dtype=torch.float16, stream=None, out=None):
    """Dequantized weights [N, K] (permuted column order) via the device routine."""
    K, N = packed["K"], packed["N"]
    if out is None:
        w = torch.empty((N, K), dtype=dtype, device=packed["codes"].device)
    else:
        _need(out, dtype, "out", N * K)
        w = out
    bits = packed.get("bits", 4)
    arrays = (_ptr(packed["codes"]), _ptr(packed["scales"]), _ptr(packed["zeros"]), K, N,
              packed["group_size"])
    if bits == 4:
        _lib.check(_lib.lib().w4a16_dequant(*arrays, _DT[dtype], _ptr(w), _stream(stream)),
                   "w4a16_dequant")
    else:
        _lib.check(_lib.lib().w4a16_dequant_bits(*arrays, bits, _DT[dtype], _ptr(w),
                                                 _stream(stream)), "w4a16_dequant_bits")
    return w


def nf4_codebook():
    buf = (ctypes.c_float * 16)()
    _lib.check(_lib.lib().nf4_codebook(ctypes.cast(buf, ctypes.c_void_p)), "nf4_codebook")
    return [float(v) for v in buf]


def nf4_quantize(W, blocksize=64, stream=None):
    """NF4 + double quant of W [N, K] fp32 -> dict(qweight, absmax_q, absmax_scale, N, K)."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    nb = N * K // blocksize
    dev = W.device
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    aq = torch.empty(nb, dtype=torch.uint8, device=dev)
    sc = torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev)
    _lib.check(_lib.lib().nf4_quantize(_ptr(W), N, K, blocksize, _ptr(q), _ptr(aq), _ptr(sc),
                                       _stream(stream)), "nf4_quantize")
    return {"qweight": q, "absmax_q": aq, "absmax_scale": sc, "N": N, "K": K,
            "blocksize": blocksize}


def nf4_repack(nf4, stream=None):
    """The NF4 codes re-laid into 1 KB tiles (once per layer): a copy of the
    weight dict with "qweight_r" added, which nf4_gemm then uses."""
    N, K, bs = nf4["N"], nf4["K"], nf4["blocksize"]
    nb = int(_lib.lib().nf4_repacked_bytes(N, K, bs))
    if nb < 0:
        raise ValueError("nf4_repack: unsupported shape N=%d K=%d" % (N, K))
    r = torch.empty(nb, dtype=torch.uint8, device=nf4["qweight"].device)
    _lib.check(_lib.lib().nf4_repack(_ptr(nf4["qweight"]), N, K, bs, _ptr(r), _stream(stream)),
               "nf4_repack")
    out = dict(nf4)
    out["qweight_r"] = r
    return out


def nf4_gemm_repacked_plan(M, N, K, blocksize=64, dtype=torch.bfloat16, workspace=True):
    """Kernels an nf4_gemm_repacked call of this shape launches (host-only query)."""
    return _names(_lib.lib().nf4_gemm_repacked_plan, M, N, K, blocksize, _DT[dtype],
                  int(workspace)).split(" + ")


def nf4_gemm(x, nf4, out=None, workspace=None, use_workspace=True, stream=None):
    """y = x @ dequant_nf4(W)^T for x [M, K] fp16/bf16 (on the repacked codes
    when the dict carries them, see nf4_repack)."""
    if x.dtype not in _DT:
        raise TypeError("x must be float16 or bfloat16")
    _need(x, x.dtype, "x")
    K, N, bs = nf4["K"], nf4["N"], nf4["blocksize"]
    M = x.numel() // K
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _need(out, x.dtype, "out", M * N)
    ws_bytes = 0
    if use_workspace:
        need = nf4_workspace_bytes(M, N, K, bs)
        if workspace is None and need > 0:
            workspace = _ws_cache(x.device, need, stream)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    else:
        workspace = None
    rp = "qweight_r" in nf4
    fn = _lib.lib().nf4_gemm_repacked if rp else _lib.lib().nf4_gemm
    _lib.check(fn(_ptr(x), _ptr(nf4["qweight_r" if rp else "qweight"]), _ptr(nf4["absmax_q"]),
                  _ptr(nf4["absmax_scale"]), bs, _ptr(out), M, N, K, _DT[x.dtype],
                  _ptr(workspace), ws_bytes, _stream(stream)),
               "nf4_gemm_repacked" if rp else "nf4_gemm")
    return out


def nf4_dequant(nf4, dtype=torch.bfloat16, stream=None):
    K, N = nf4["K"], nf4["N"]
    w = torch.empty((N, K), dtype=dtype, device=nf4["qweight"].device)
    _lib.check(_lib.lib().nf4_dequant(_ptr(nf4["qweight"]), _ptr(nf4["absmax_q"]),
                                      _ptr(nf4["absmax_scale"]), N, K, nf4["blocksize"],
                                      _DT[dtype], _ptr(w), _stream(stream)), "nf4_dequant")
    return w


# One workspace per (device, stream), grown on demand and reused by later
# calls on that stream (calls on one stream run in order; the kernels write
# every workspace byte they read, so its contents do not matter).
_WS = {}


def _ws_cache(device, nbytes, stream=None):
    st = torch.cuda.current_stream() if stream is None else stream
    key = (str(device), st.cuda_stream)
    cur = _WS.get(key)
    if cur is None or cur.numel() * 4 < nbytes:
        st.synchronize()
        cur = workspace(max(nbytes, 1 << 20), device)
        _WS[key] = cur
    return cur
