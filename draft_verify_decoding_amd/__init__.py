"""Python binding of libisd.so, the MI355X (gfx950) ISD step library.

Argument marshalling only: every step of the path runs in the HIP kernels of
libisd.so; torch is used for device memory and the current stream. The
names mirror the C ABI in include/isd.h. There is no fallback: if the
library is missing, importing works but every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libisd.so")

ISD_BF16 = 1
ISD_F32 = 2
PROPOSE = {"sample": 0, "argmax": 1}
PAGE_SIZE = 16

DEV_PAGE_OOB = 1
DEV_CAPACITY = 2
DEV_NONFINITE = 4
DEV_TOKEN_OOB = 8
DEV_STATE = 16

_DTYPES = {torch.bfloat16: ISD_BF16, torch.float32: ISD_F32}


class IsdError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where}: {strerror(code)} (code {code})")
        self.code = code


# ------------------------------------------------------------------ C types
class IsdKvCache(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("table_stride", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class IsdSeqState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("n_draft", "drafts", "q_x", "q_m", "q_s", "q_row")]


class IsdAcceptArgs(ctypes.Structure):
    _fields_ = [
        ("C", ctypes.c_int32), ("N", ctypes.c_int32), ("V", ctypes.c_int32),
        ("rows", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("logits", ctypes.c_void_p), ("prev_logits", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("in_", IsdSeqState), ("out", IsdSeqState),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint64),
        ("accepted", ctypes.c_void_p), ("n_emit", ctypes.c_void_p),
        ("emit", ctypes.c_void_p), ("kv_commit", ctypes.c_void_p),
        ("ctx", ctypes.c_void_p),
        ("p_x", ctypes.c_void_p), ("resid_mass", ctypes.c_void_p),
        ("row_m", ctypes.c_void_p), ("row_s", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("dev_err", ctypes.c_void_p),
        ("proposal", ctypes.c_int32),
        ("step_dev", ctypes.c_void_p),
        ("chunk_stats", ctypes.c_void_p),
    ]


_lib = None

_SIGNATURES = {
    "isd_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "isd_version": (ctypes.c_int, []),
    "isd_kv_write": (ctypes.c_int, [ctypes.POINTER(IsdKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "isd_attention_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                       ctypes.POINTER(IsdKvCache), ctypes.c_int, ctypes.c_int]),
    "isd_attention": (ctypes.c_int, [ctypes.POINTER(IsdKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    "isd_attention_with_block": (ctypes.c_int, [ctypes.POINTER(IsdKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                ctypes.c_void_p, ctypes.c_void_p]),
    "isd_kv_write_layers": (ctypes.c_int, [ctypes.POINTER(IsdKvCache), ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "isd_accept_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "isd_accept": (ctypes.c_int, [ctypes.POINTER(IsdAcceptArgs), ctypes.c_void_p]),
    "isd_accept_noalloc_max_workspace": (ctypes.c_size_t, []),
    "isd_accept_noalloc": (ctypes.c_int, [ctypes.POINTER(IsdAcceptArgs), ctypes.c_void_p]),
    "isd_block_assemble": (ctypes.c_int, [ctypes.POINTER(IsdSeqState), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "isd_linear": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "isd_lora_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int]),
    "gated_lora_apply": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "isd_linear_gated": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "isd_rmsnorm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "isd_cast_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
    "isd_swiglu": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "isd_lm_head_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int]),
    "isd_lm_head": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]),
}


def lib():
    """The loaded library; raises if libisd.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python draft_verify_decoding_amd/build.py (no CPU fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code):
    return lib().isd_strerror(int(code)).decode()


def _check(rc, where):
    if rc != 0:
        raise IsdError(rc, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


# ------------------------------------------------------------------ KV cache
class KVCache:
    """Device page pools in the library's layout plus a block table.

    k_pages/v_pages hold num_pages * Hkv * D * 16 elements each; the layout
    of a page is documented in include/isd.h.
    """

    def __init__(self, num_pages, num_kv_heads, head_dim, dtype, block_table, device="cuda", pools=None):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.dtype = dtype
        n = num_pages * num_kv_heads * head_dim * PAGE_SIZE
        if pools is None:
            self.k_pages = torch.zeros(n, dtype=dtype, device=device)
            self.v_pages = torch.zeros(n, dtype=dtype, device=device)
        else:  # views into storage the caller owns (see stacked)
            self.k_pages, self.v_pages = pools
        self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()

    @classmethod
    def stacked(cls, layers, num_pages, num_kv_heads, head_dim, dtype, block_table, device="cuda"):
        """One cache per layer in a single [layers, pool] allocation with a
        shared block table, for isd_kv_write_layers. Returns (caches,
        layer_stride in elements)."""
        n = num_pages * num_kv_heads * head_dim * PAGE_SIZE
        k_all = torch.zeros((layers, n), dtype=dtype, device=device)
        v_all = torch.zeros((layers, n), dtype=dtype, device=device)
        table = block_table.to(device=device, dtype=torch.int32).contiguous()
        caches = [cls(num_pages, num_kv_heads, head_dim, dtype, table, device, pools=(k_all[l], v_all[l]))
                  for l in range(layers)]
        return caches, n

    def c_struct(self):
        return IsdKvCache(
            self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.block_table.data_ptr(),
            self.block_table.shape[1], self.num_pages, PAGE_SIZE, self.num_kv_heads,
            self.head_dim, _DTYPES[self.dtype])


def isd_kv_write(kv, k, v, pos0, nrows=None, dev_err=None, stream=None):
    """Write k, v [C, rows, Hkv, D] at positions pos0[b] + r (r < nrows[b])."""
    C, rows = k.shape[0], k.shape[1]
    s = kv.c_struct()
    rc = lib().isd_kv_write(ctypes.byref(s), _p(k), _p(v), _p(pos0), _p(nrows), C, rows,
                            _p(dev_err), _stream(stream))
    _check(rc, "isd_kv_write")


def isd_kv_write_layers(kv, layer_stride, k, v, pos0, nrows=None, dev_err=None, stream=None):
    """isd_kv_write for every layer: k, v [layers, C, rows, Hkv, D]; layer l's
    pools start l * layer_stride elements after kv's (layer 0's)."""
    layers, C, rows = k.shape[0], k.shape[1], k.shape[2]
    s = kv.c_struct()
    rc = lib().isd_kv_write_layers(ctypes.byref(s), layers, int(layer_stride), _p(k), _p(v), _p(pos0), _p(nrows), C,
                                   rows, _p(dev_err), _stream(stream))
    _check(rc, "isd_kv_write_layers")


def attn_invariant(chunk_tiles):
    """`slices` value of the batch-invariant split (ISD_ATTN_INVARIANT)."""
    return -int(chunk_tiles)


def isd_attention_workspace_size(kv, C, rows, num_q_heads, max_len, slices=0):
    s = kv.c_struct()
    return int(lib().isd_attention_workspace_size(C, rows, num_q_heads, ctypes.byref(s), max_len, slices))


def isd_attention(kv, q, ctx, max_len, scale=None, slices=0, out=None, ws=None, dev_err=None, stream=None,
                  k_blk=None, v_blk=None, odtype=torch.float32):
    """out [C, rows, Hq, D] (fp32, or bf16: `odtype` or the dtype of a given
    out) = causal attention of q over the pages; with k_blk, v_blk
    ([C, rows, Hkv, D]) the block's own keys come from those rows
    (isd_attention_with_block)."""
    C, rows, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((C, rows, Hq, D), dtype=odtype, device=q.device)
    need = isd_attention_workspace_size(kv, C, rows, Hq, max_len, slices)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    s = kv.c_struct()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    if k_blk is None:
        rc = lib().isd_attention(ctypes.byref(s), _p(q), _p(ctx), C, rows, Hq, float(scale), int(max_len),
                                 int(slices), _p(out), _dtype_code(out), _p(ws), nbytes, _p(dev_err),
                                 _stream(stream))
        _check(rc, "isd_attention")
    else:
        rc = lib().isd_attention_with_block(ctypes.byref(s), _p(k_blk), _p(v_blk), _p(q), _p(ctx), C, rows, Hq,
                                            float(scale), int(max_len), int(slices), _p(out), _dtype_code(out),
                                            _p(ws), nbytes, _p(dev_err), _stream(stream))
        _check(rc, "isd_attention_with_block")
    return out


# -------------------------------------------------------------------- accept
class SeqState:
    """Per-sequence decoding state on the device (see isd_seq_state)."""

    def __init__(self, C, N, device="cuda"):
        nd = N - 1
        self.C, self.N = C, N
        self.n_draft = torch.zeros(C, dtype=torch.int32, device=device)
        self.drafts = torch.full((C, nd), -1, dtype=torch.int32, device=device)
        self.q_x = torch.zeros((C, nd), dtype=torch.float32, device=device)
        self.q_m = torch.zeros((C, nd), dtype=torch.float32, device=device)
        self.q_s = torch.zeros((C, nd), dtype=torch.float32, device=device)
        self.q_row = torch.zeros(C, dtype=torch.int32, device=device)

    def c_struct(self):
        return IsdSeqState(*(t.data_ptr() for t in
                             (self.n_draft, self.drafts, self.q_x, self.q_m, self.q_s, self.q_row)))

    def copy_(self, other):
        for name in ("n_draft", "drafts", "q_x", "q_m", "q_s", "q_row"):
            getattr(self, name).copy_(getattr(other, name))
        return self


def isd_accept_workspace_size(C, N, V, rows):
    return int(lib().isd_accept_workspace_size(C, N, V, rows))


def accept_workspace(C, N, V, rows, device="cuda"):
    """An isd_accept workspace (its contents on entry are ignored)."""
    return torch.empty(isd_accept_workspace_size(C, N, V, rows), dtype=torch.uint8, device=device)


class AcceptOutputs:
    def __init__(self, C, N, rows, device, diag):
        self.accepted = torch.empty(C, dtype=torch.int32, device=device)
        self.n_emit = torch.empty(C, dtype=torch.int32, device=device)
        self.emit = torch.empty((C, N), dtype=torch.int32, device=device)
        self.kv_commit = torch.empty(C, dtype=torch.int32, device=device)
        self.p_x = self.resid_mass = self.row_m = self.row_s = None
        if diag:
            self.p_x = torch.empty((C, N - 1), dtype=torch.float32, device=device)
            self.resid_mass = torch.empty(C, dtype=torch.float32, device=device)
            self.row_m = torch.empty((C, rows), dtype=torch.float32, device=device)
            self.row_s = torch.empty((C, rows), dtype=torch.float32, device=device)


def isd_accept(logits, prev_logits, state_in, state_out, N, seed, step, V=None, out=None, ws=None,
               diag=False, dev_err=None, ctx=None, stream=None, proposal="sample", step_dev=None,
               chunk_stats=None, noalloc=False):
    """One accept step. logits [C, rows, ld] (bf16 or fp32); returns the
    AcceptOutputs (device tensors) and writes state_out. If ctx (int32 [C])
    is given, the kernel adds kv_commit to it. proposal: "sample" or
    "argmax" (drafts = argmax of the MASK rows). step_dev: optional int64
    device tensor [1] holding the step number (then `step` is ignored), for
    calls captured in a graph. chunk_stats: optional fp32 [C, rows, nch, 2]
    from isd_lm_head (then the statistics pass is skipped). noalloc: call
    isd_accept_noalloc, whose workspace is the library's fixed device array
    (ws is then ignored and none is allocated)."""
    C, rows, ld = logits.shape
    V = ld if V is None else V
    if out is None:
        out = AcceptOutputs(C, N, rows, logits.device, diag)
    if ws is None and not noalloc:
        ws = accept_workspace(C, N, V, rows, logits.device)
    args = IsdAcceptArgs()
    args.C, args.N, args.V, args.rows = C, N, V, rows
    args.dtype = _dtype_code(logits)
    args.logits = logits.data_ptr()
    args.prev_logits = None if prev_logits is None else prev_logits.data_ptr()
    args.ld = ld
    args.in_ = state_in.c_struct()
    args.out = state_out.c_struct()
    args.seed, args.step = int(seed), int(step)
    args.accepted, args.n_emit = out.accepted.data_ptr(), out.n_emit.data_ptr()
    args.emit, args.kv_commit = out.emit.data_ptr(), out.kv_commit.data_ptr()
    args.ctx = None if ctx is None else ctx.data_ptr()
    for name in ("p_x", "resid_mass", "row_m", "row_s"):
        t = getattr(out, name)
        setattr(args, name, None if t is None else t.data_ptr())
    args.ws = None if ws is None else ws.data_ptr()
    args.ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    args.dev_err = None if dev_err is None else dev_err.data_ptr()
    args.proposal = PROPOSE[proposal]
    args.step_dev = None if step_dev is None else step_dev.data_ptr()
    args.chunk_stats = None if chunk_stats is None else chunk_stats.data_ptr()
    if noalloc:
        _check(lib().isd_accept_noalloc(ctypes.byref(args), _stream(stream)), "isd_accept_noalloc")
    else:
        _check(lib().isd_accept(ctypes.byref(args), _stream(stream)), "isd_accept")
    return out


def isd_block_assemble(state, emit, n_emit, ctx, N, mask_id, tokens=None, positions=None, is_mask=None,
                       dev_err=None, stream=None):
    """The next step's block [C, 2N] from the state and outputs isd_accept
    wrote: newest emitted token, pending drafts, MASK rows. Returns
    (tokens, positions, is_mask); positions and is_mask are made when ctx is
    given or when passed in."""
    C = emit.shape[0]
    dev = emit.device
    if tokens is None:
        tokens = torch.empty((C, 2 * N), dtype=torch.int32, device=dev)
    if positions is None and ctx is not None:
        positions = torch.empty((C, 2 * N), dtype=torch.int32, device=dev)
    if is_mask is None:
        is_mask = torch.empty((C, 2 * N), dtype=torch.uint8, device=dev)
    s = state.c_struct()
    _check(lib().isd_block_assemble(ctypes.byref(s), _p(emit), _p(n_emit), _p(ctx), C, N, int(mask_id), _p(tokens),
                                    _p(positions), _p(is_mask), _p(dev_err), _stream(stream)),
           "isd_block_assemble")
    return tokens, positions, is_mask


# --------------------------------------------------------------- projections
def isd_linear(x, W, y=None, stream=None, ydtype=torch.float32):
    """y = x W^T; y fp32 or bf16 (`ydtype`, or the dtype of a given y)."""
    M, K = x.shape
    Nout = W.shape[0]
    if y is None:
        y = torch.empty((M, Nout), dtype=ydtype, device=x.device)
    _check(lib().isd_linear(_p(x), _p(W), M, K, Nout, _p(y), _dtype_code(y), _stream(stream)), "isd_linear")
    return y


def isd_lora_workspace_size(M, r):
    return int(lib().isd_lora_workspace_size(M, r))


def lora_workspace(M, r, device="cuda"):
    """A LoRA workspace, zero-filled as the library requires before its first
    use (every call returns its counters to zero)."""
    return torch.zeros(isd_lora_workspace_size(M, r), dtype=torch.uint8, device=device)


def gated_lora_apply(x, A, B, is_mask, y, scale=1.0, ws=None, stream=None):
    M, K = x.shape
    r, Nout = A.shape[0], B.shape[0]
    if ws is None:
        ws = lora_workspace(M, r, x.device)
    rc = lib().gated_lora_apply(_p(x), _p(A), _p(B), _p(is_mask), M, K, Nout, r, float(scale), _p(y),
                                _dtype_code(y), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gated_lora_apply")
    return y


def isd_linear_gated(x, W, A, B, is_mask, scale=1.0, y=None, ws=None, stream=None, ydtype=torch.float32):
    M, K = x.shape
    r, Nout = A.shape[0], W.shape[0]
    if y is None:
        y = torch.empty((M, Nout), dtype=ydtype, device=x.device)
    if ws is None:
        ws = lora_workspace(M, r, x.device)
    rc = lib().isd_linear_gated(_p(x), _p(W), _p(A), _p(B), _p(is_mask), M, K, Nout, r, float(scale), _p(y),
                                _dtype_code(y), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "isd_linear_gated")
    return y


def isd_lm_head_workspace_size(M, V):
    return int(lib().isd_lm_head_workspace_size(M, V))


def isd_lm_head(h, W, logits=None, chunk_stats=None, ws=None, stream=None):
    """logits [M, ld] (torch.bfloat16) = h W^T, rounded to nearest even, and
    their chunk statistics [M, nch, 2] fp32 (nch = ceil(V / 8192))."""
    M, K = h.shape
    V = W.shape[0]
    if logits is None:
        logits = torch.empty((M, V), dtype=torch.bfloat16, device=h.device)
    nch = (V + 8191) // 8192
    if chunk_stats is None:
        chunk_stats = torch.empty((M, nch, 2), dtype=torch.float32, device=h.device)
    if ws is None:
        ws = torch.empty(isd_lm_head_workspace_size(M, V), dtype=torch.uint8, device=h.device)
    rc = lib().isd_lm_head(_p(h), _p(W), M, K, V, _p(logits), logits.stride(-2), _p(chunk_stats), _p(ws),
                           ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "isd_lm_head")
    return logits, chunk_stats


def prepare_lm_head(h, W, logits, chunk_stats, ws, stream=None):
    M, K = h.shape
    V = W.shape[0]
    return Prepared("isd_lm_head", _p(h), _p(W), M, K, V, _p(logits), logits.stride(-2), _p(chunk_stats), _p(ws),
                    ws.numel() * ws.element_size(), _stream(stream), keep=(h, W, logits, chunk_stats, ws))


# ---------------------------------------------------------- decoder block
def isd_rmsnorm(h, gamma, out=None, delta=None, eps=1e-6, stream=None):
    """h [M, H] fp32 (updated in place with h += delta when delta is given);
    returns out [M, H] bf16 = rmsnorm(h) * gamma."""
    M, H = h.shape
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=h.device)
    _check(lib().isd_rmsnorm(_p(h), _p(delta), _p(gamma), M, H, float(eps), _p(out), _stream(stream)), "isd_rmsnorm")
    return out


def isd_cast_bf16(src, outs, stream=None):
    """Columns of src [M, ld] fp32 split into the bf16 tensors outs (each
    [M, w] contiguous, or any tensor of M * w elements), in order."""
    M, ld = src.shape[0], src.stride(0)
    widths = [o.numel() // M for o in outs]
    w_arr = (ctypes.c_int * len(outs))(*widths)
    d_arr = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    _check(lib().isd_cast_bf16(_p(src), ld, M, len(outs), w_arr, d_arr, _stream(stream)), "isd_cast_bf16")
    return outs


def isd_swiglu(gu, out=None, stream=None):
    """gu [M, 2I] fp32 (gate | up) -> out [M, I] bf16 = silu(gate) * up."""
    M, I2 = gu.shape
    if out is None:
        out = torch.empty((M, I2 // 2), dtype=torch.bfloat16, device=gu.device)
    _check(lib().isd_swiglu(_p(gu), M, I2 // 2, _p(out), _stream(stream)), "isd_swiglu")
    return out


# ------------------------------------------------------- prepared calls
class Prepared:
    """One library call with its arguments marshalled once, for loops that
    issue the same call many times (the arguments' tensors must stay alive
    and in place). Calling it runs the call and raises on an error code."""

    def __init__(self, name, *args, keep=()):
        self.name = name
        self.fn = getattr(lib(), name)
        self.args = args
        self.keep = keep

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise IsdError(rc, self.name)


def prepare_kv_write(kv, k, v, pos0, nrows=None, dev_err=None, stream=None):
    s = kv.c_struct()
    return Prepared("isd_kv_write", ctypes.byref(s), _p(k), _p(v), _p(pos0), _p(nrows), k.shape[0], k.shape[1],
                    _p(dev_err), _stream(stream), keep=(s, kv, k, v, pos0, nrows, dev_err))


def prepare_kv_write_layers(kv, layer_stride, k, v, pos0, nrows=None, dev_err=None, stream=None):
    s = kv.c_struct()
    return Prepared("isd_kv_write_layers", ctypes.byref(s), k.shape[0], int(layer_stride), _p(k), _p(v), _p(pos0),
                    _p(nrows), k.shape[1], k.shape[2], _p(dev_err), _stream(stream),
                    keep=(s, kv, k, v, pos0, nrows, dev_err))


def prepare_attention(kv, q, ctx, max_len, out, ws=None, slices=0, scale=None, dev_err=None, stream=None,
                      k_blk=None, v_blk=None):
    C, rows, Hq, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    s = kv.c_struct()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    if k_blk is not None:
        return Prepared("isd_attention_with_block", ctypes.byref(s), _p(k_blk), _p(v_blk), _p(q), _p(ctx), C, rows,
                        Hq, float(scale), int(max_len), int(slices), _p(out), _dtype_code(out), _p(ws), nbytes,
                        _p(dev_err), _stream(stream), keep=(s, kv, k_blk, v_blk, q, ctx, out, ws, dev_err))
    return Prepared("isd_attention", ctypes.byref(s), _p(q), _p(ctx), C, rows, Hq, float(scale), int(max_len),
                    int(slices), _p(out), _dtype_code(out), _p(ws), nbytes, _p(dev_err), _stream(stream),
                    keep=(s, kv, q, ctx, out, ws, dev_err))


def prepare_linear(x, W, y, stream=None):
    M, K = x.shape
    return Prepared("isd_linear", _p(x), _p(W), M, K, W.shape[0], _p(y), _dtype_code(y), _stream(stream),
                    keep=(x, W, y))


def prepare_linear_gated(x, W, A, B, is_mask, y, ws, scale=1.0, stream=None):
    M, K = x.shape
    return Prepared("isd_linear_gated", _p(x), _p(W), _p(A), _p(B), _p(is_mask), M, K, W.shape[0], A.shape[0],
                    float(scale), _p(y), _dtype_code(y), _p(ws), ws.numel() * ws.element_size(), _stream(stream),
                    keep=(x, W, A, B, is_mask, y, ws))


def prepare_rmsnorm(h, gamma, out, delta=None, eps=1e-6, stream=None):
    M, H = h.shape
    return Prepared("isd_rmsnorm", _p(h), _p(delta), _p(gamma), M, H, float(eps), _p(out), _stream(stream),
                    keep=(h, gamma, out, delta))


def prepare_cast_bf16(src, outs, stream=None):
    M, ld = src.shape[0], src.stride(0)
    w_arr = (ctypes.c_int * len(outs))(*[o.numel() // M for o in outs])
    d_arr = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    return Prepared("isd_cast_bf16", _p(src), ld, M, len(outs), w_arr, d_arr, _stream(stream),
                    keep=(src, tuple(outs), w_arr, d_arr))


def prepare_swiglu(gu, out, stream=None):
    M, I2 = gu.shape
    return Prepared("isd_swiglu", _p(gu), M, I2 // 2, _p(out), _stream(stream), keep=(gu, out))


def prepare_accept(logits, prev_logits, state_in, state_out, N, seed, out, ws, V=None, ctx=None, dev_err=None,
                   proposal="sample", step_dev=None, chunk_stats=None, stream=None):
    """isd_accept with its arguments marshalled once; the returned call takes
    the step number."""
    C, rows, ld = logits.shape
    args = IsdAcceptArgs()
    args.C, args.N, args.V, args.rows = C, N, ld if V is None else V, rows
    args.dtype = _dtype_code(logits)
    args.logits = logits.data_ptr()
    args.prev_logits = None if prev_logits is None else prev_logits.data_ptr()
    args.ld = ld
    args.in_ = state_in.c_struct()
    args.out = state_out.c_struct()
    args.seed = int(seed)
    args.accepted, args.n_emit = out.accepted.data_ptr(), out.n_emit.data_ptr()
    args.emit, args.kv_commit = out.emit.data_ptr(), out.kv_commit.data_ptr()
    args.ctx = None if ctx is None else ctx.data_ptr()
    for name in ("p_x", "resid_mass", "row_m", "row_s"):
        t = getattr(out, name)
        setattr(args, name, None if t is None else t.data_ptr())
    args.ws = ws.data_ptr()
    args.ws_bytes = ws.numel() * ws.element_size()
    args.dev_err = None if dev_err is None else dev_err.data_ptr()
    args.proposal = PROPOSE[proposal]
    args.step_dev = None if step_dev is None else step_dev.data_ptr()
    args.chunk_stats = None if chunk_stats is None else chunk_stats.data_ptr()
    fn = lib().isd_accept
    stream_p = _stream(stream)
    keep = (logits, prev_logits, state_in, state_out, out, ws, ctx, dev_err, step_dev, chunk_stats)

    def call(step):
        args.step = int(step)
        rc = fn(ctypes.byref(args), stream_p)
        if rc != 0:
            raise IsdError(rc, "isd_accept")
    call.keep = keep
    call.args = args
    return call
