"""ctypes binding of libpkv.so (the C ABI declared in include/pkv.h).

Argument marshalling only: every step of the path (slot mapping, allocator bookkeeping, work
planning, the KV scatter and the attention kernels) runs inside the library. Device buffers
are torch tensors (PyTorch is used for device memory and streams); host metadata are int32
numpy arrays or CPU tensors. Importing this module does not need a GPU; calling a device entry
point does. If libpkv.so is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence, Tuple

import numpy as np

LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "pkv.h")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_POOL_EXHAUSTED = -2
PKV_ERR_DOUBLE_FREE = -3
PKV_ERR_SHARED_WRITE = -4
PKV_ERR_UNSUPPORTED = -5
PKV_ERR_HIP = -6
PKV_ERR_INCONSISTENT = -7
PKV_F32 = 0
PKV_BF16 = 1
PKV_E4M3 = 2
PKV_ATTN_PHASE_CONSISTENT = 1


class PkvError(RuntimeError):
    status = None

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


class InvalidArgument(PkvError):
    pass


class PoolExhausted(PkvError):
    pass


class DoubleFree(PkvError):
    pass


class SharedWrite(PkvError):
    pass


class Unsupported(PkvError):
    pass


class HipError(PkvError):
    pass


class Inconsistent(PkvError):
    pass


_ERRORS = {
    PKV_ERR_INVALID: InvalidArgument, PKV_ERR_POOL_EXHAUSTED: PoolExhausted,
    PKV_ERR_DOUBLE_FREE: DoubleFree, PKV_ERR_SHARED_WRITE: SharedWrite,
    PKV_ERR_UNSUPPORTED: Unsupported, PKV_ERR_HIP: HipError, PKV_ERR_INCONSISTENT: Inconsistent,
}

_lib = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_version": ([], ctypes.c_char_p),
    "pkv_alloc_create": ([_i32, ctypes.POINTER(_vp)], _i32),
    "pkv_alloc_destroy": ([_vp], None),
    "pkv_alloc_allocate": ([_vp, _i32, _pi32], _i32),
    "pkv_alloc_incref": ([_vp, _i32, _pi32], _i32),
    "pkv_alloc_free": ([_vp, _i32, _pi32], _i32),
    "pkv_alloc_refcount": ([_vp, _i32], _i32),
    "pkv_alloc_num_free": ([_vp], _i32),
    "pkv_alloc_num_blocks": ([_vp], _i32),
    "pkv_alloc_check_consistent": ([_vp], _i32),
    "pkv_alloc_snapshot": ([_vp, _pi32, _pi32], _i32),
    "pkv_slot_mapping": ([_vp, _pi32, _i32, _i32, _i32, _i32, _pi32], _i32),
    "pkv_slot_mapping_step": ([_vp, _pi32, _i32, _i32, _i32, _pi32, _pi32, _pi32], _i32),
    "pkv_validate_slots": ([_pi32, _i32, _i64], _i32),
    "pkv_sched_create": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp)], _i32),
    "pkv_sched_destroy": ([_vp], None),
    "pkv_sched_allocator": ([_vp], _vp),
    "pkv_sched_add": ([_vp, _i32, _i32, _i32], _i32),
    "pkv_sched_step": ([_vp, _pi32, _pi32, _pi32, _pi32], _i32),
    "pkv_sched_plan": ([_vp, _pi32, _pi32, _pi32, _pi32, _pi32, _pi32, _pi32, _pi32], _i32),
    "pkv_sched_complete": ([_vp, _pi32, _i32, _pi32, _pi32], _i32),
    "pkv_sched_trim": ([_vp, _i32, _i32], _i32),
    "pkv_sched_fork": ([_vp, _i32, _i32], _i32),
    "pkv_sched_seq_info": ([_vp, _i32, _pi32, _pi32, _pi32, _pi32], _i32),
    "pkv_sched_seq_blocks": ([_vp, _i32, _pi32], _i32),
    "pkv_sched_stats": ([_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), _pi32, _pi32], _i32),
    "pkv_sched_check": ([_vp], _i32),
    "pkv_copy_blocks": ([_vp, _vp, _pi32, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                         ctypes.c_size_t, _vp], _i32),
    "pkv_write_kv": ([_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "pkv_attention_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      ctypes.POINTER(ctypes.c_size_t)], _i32),
    "pkv_attention_workspace_size_ex": ([_pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)],
                                        _i32),
    "pkv_attention_ex": ([_vp, _vp, _vp, _vp, _i32, _pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, ctypes.c_float, _i32, _i32, ctypes.c_uint32, _vp, _vp,
                          ctypes.c_size_t, _vp], _i32),
    "pkv_attention": ([_vp, _vp, _vp, _vp, _i32, _pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                       _i32, _i32, ctypes.c_float, _i32, _i32, _vp, _vp, ctypes.c_size_t, _vp],
                      _i32),
    "pkv_write_kv_attention_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                                               _i32, ctypes.c_uint32, _i32,
                                               ctypes.POINTER(ctypes.c_size_t)], _i32),
    "pkv_write_kv_attention": ([_vp, _vp, _vp, _pi32, _i32, _vp, _vp, _vp, _i32, _pi32, _pi32,
                                _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32,
                                _i32, ctypes.c_uint32, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "pkv_write_kv_attention_shared_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32,
                                                      _i32, _i32, ctypes.c_uint32, _i32, _pi32,
                                                      _i32, _i32,
                                                      ctypes.POINTER(ctypes.c_size_t)], _i32),
    "pkv_write_kv_attention_shared": ([_vp, _vp, _vp, _pi32, _i32, _vp, _vp, _vp, _pi32, _i32,
                                       _pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       ctypes.c_float, _i32, _i32, ctypes.c_uint32, _vp, _vp,
                                       ctypes.c_size_t, _vp], _i32),
    "pkv_write_kv_attention_shared_fp8_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32,
                                                          _i32, ctypes.c_uint32, _i32, _pi32,
                                                          _i32, _i32,
                                                          ctypes.POINTER(ctypes.c_size_t)],
                                                         _i32),
    "pkv_write_kv_attention_shared_fp8": ([_vp, _vp, _vp, _pi32, _i32, _vp, _vp, _vp, _pi32,
                                           _i32, _pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, _i32, ctypes.c_uint32, _vp, _vp,
                                           ctypes.c_size_t, _vp], _i32),
    "pkv_write_kv_fp8": ([_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                          ctypes.c_float, ctypes.c_float, _vp], _i32),
    "pkv_attention_fp8_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                                          ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)],
                                         _i32),
    "pkv_attention_fp8": ([_vp, _vp, _vp, _vp, _i32, _pi32, _pi32, _i32, _i32, _i32, _i32,
                           _i32, _i32, _i32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                           _i32, ctypes.c_uint32, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "pkv_write_kv_attention_fp8_workspace_size": ([_pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
                                                   ctypes.c_uint32, _i32,
                                                   ctypes.POINTER(ctypes.c_size_t)], _i32),
    "pkv_write_kv_attention_fp8": ([_vp, _vp, _vp, _pi32, _i32, _vp, _vp, _vp, _i32, _pi32,
                                    _pi32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                    ctypes.c_float, ctypes.c_float, ctypes.c_float, _i32,
                                    ctypes.c_uint32, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "pkv_profile_set_kinds": ([ctypes.c_uint32], _i32),
    "pkv_staging_info": ([ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_i64)], _i32),
    "pkv_attention_noalloc": ([_vp, _vp, _vp, _vp, _i32, _pi32, _pi32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, ctypes.c_float, _i32, _i32, ctypes.c_uint32,
                               _vp, _vp], _i32),
    "pkv_profile_enable": ([_i32], _i32),
    "pkv_profile_read": ([_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)], _i32),
    "pkv_profile_read_span": ([ctypes.c_uint32, ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(_i64)], _i32),
}

KERNEL_KINDS = {"write_kv": 0, "prefill": 1, "decode": 2, "merge": 3, "decode_group": 4}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m prefill_slot_mapping_amd.build` (no fallback path)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def header_functions() -> List[str]:
    """Names of every function declared in include/pkv.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def _check(status: int) -> int:
    if status >= 0:
        return status
    msg = lib().pkv_last_error().decode("utf-8", "replace")
    raise _ERRORS.get(status, PkvError)(status, msg)


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        if x.device.type != "cpu":
            raise ValueError("host metadata must be CPU arrays")
        x = x.detach().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_pi32)


def version() -> str:
    return lib().pkv_version().decode()


# ---- host allocator ----------------------------------------------------------------------

class BlockAllocator:
    """Handle on the library's LIFO + refcount block allocator (see include/pkv.h)."""

    def __init__(self, num_blocks: int):
        h = _vp()
        _check(lib().pkv_alloc_create(int(num_blocks), ctypes.byref(h)))
        self._h = h

    @classmethod
    def _view(cls, handle, owner):
        """A non-owning view of an allocator that another handle owns (kept alive by it)."""
        a = cls.__new__(cls)
        a._h = handle
        a._owner = owner
        return a

    def close(self):
        if getattr(self, "_h", None) and getattr(self, "_owner", None) is None:
            lib().pkv_alloc_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return _check(lib().pkv_alloc_num_blocks(self._h))

    def num_free(self) -> int:
        return _check(lib().pkv_alloc_num_free(self._h))

    def allocate(self, n: int) -> List[int]:
        out = np.zeros(max(int(n), 1), dtype=np.int32)
        _check(lib().pkv_alloc_allocate(self._h, int(n), _ptr(out)))
        return out[:int(n)].tolist()

    def incref(self, ids: Sequence[int]) -> None:
        a = _host_i32(list(ids))
        _check(lib().pkv_alloc_incref(self._h, a.size, _ptr(a)))

    def free(self, ids: Sequence[int]) -> None:
        a = _host_i32(list(ids))
        _check(lib().pkv_alloc_free(self._h, a.size, _ptr(a)))

    def refcount(self, block: int) -> int:
        return _check(lib().pkv_alloc_refcount(self._h, int(block)))

    def check_consistent(self) -> bool:
        st = lib().pkv_alloc_check_consistent(self._h)
        if st == PKV_ERR_INCONSISTENT:
            return False
        _check(st)
        return True

    def snapshot(self) -> Tuple[List[int], List[int]]:
        nf, nb = self.num_free(), self.num_blocks
        stack = np.zeros(max(nf, 1), dtype=np.int32)
        rc = np.zeros(max(nb, 1), dtype=np.int32)
        _check(lib().pkv_alloc_snapshot(self._h, _ptr(stack), _ptr(rc)))
        return stack[:nf].tolist(), rc[:nb].tolist()

    def slots(self, block_table_row, start_pos: int, n_new: int, block_size: int) -> np.ndarray:
        row = _host_i32(block_table_row)
        out = np.zeros(max(int(n_new), 1), dtype=np.int32)
        _check(lib().pkv_slot_mapping(self._h, _ptr(row), row.size, int(block_size),
                                      int(start_pos), int(n_new), _ptr(out)))
        return out[:int(n_new)]


# ---- host step builder ------------------------------------------------------------------

class SchedPlan:
    """One step built by the scheduler (fields as pkv_sched_plan, as Python lists)."""
    __slots__ = ("seq_ids", "n_new", "ctx_lens", "cu_seqlens", "block_tables", "slots",
                 "copies", "preempted")

    def __init__(self, **kw):
        for k in self.__slots__:
            setattr(self, k, kw[k])


class Scheduler:
    """Handle on the library's host step builder (pkv_sched_* in include/pkv.h)."""

    def __init__(self, num_blocks: int, block_size: int, chunk_size: int, token_budget: int,
                 max_num_seqs: int, max_blocks_per_seq: int, prefix_sharing: bool = False):
        h = _vp()
        _check(lib().pkv_sched_create(int(num_blocks), int(block_size), int(chunk_size),
                                      int(token_budget), int(max_num_seqs),
                                      int(max_blocks_per_seq), 1 if prefix_sharing else 0,
                                      ctypes.byref(h)))
        self._h = h
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        self.allocator = BlockAllocator._view(_vp(lib().pkv_sched_allocator(h)), self)

    def close(self):
        if getattr(self, "_h", None):
            lib().pkv_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, seq_id: int, prompt_len: int, group: int = -1) -> None:
        _check(lib().pkv_sched_add(self._h, int(seq_id), int(prompt_len), int(group)))

    def step(self) -> SchedPlan:
        B, T, nc, npre = (ctypes.c_int32(0) for _ in range(4))
        _check(lib().pkv_sched_step(self._h, ctypes.byref(B), ctypes.byref(T), ctypes.byref(nc),
                                    ctypes.byref(npre)))
        b, t, c, pr = B.value, T.value, nc.value, npre.value
        mb = self.max_blocks_per_seq
        ids, nn, ctx = (np.zeros(max(b, 1), np.int32) for _ in range(3))
        cu = np.zeros(b + 1, np.int32)
        bt = np.zeros(max(b, 1) * mb, np.int32)
        sl = np.zeros(max(t, 1), np.int32)
        cp = np.zeros(max(2 * c, 1), np.int32)
        pp = np.zeros(max(pr, 1), np.int32)
        _check(lib().pkv_sched_plan(self._h, _ptr(ids), _ptr(nn), _ptr(ctx), _ptr(cu), _ptr(bt),
                                    _ptr(sl), _ptr(cp), _ptr(pp)))
        bt = bt[:b * mb].reshape(b, mb)
        tables = [[int(x) for x in row if x >= 0] for row in bt]
        return SchedPlan(seq_ids=ids[:b].tolist(), n_new=nn[:b].tolist(),
                         ctx_lens=ctx[:b].tolist(), cu_seqlens=cu.tolist(), block_tables=tables,
                         slots=sl[:t].tolist(),
                         copies=[(int(cp[2 * i]), int(cp[2 * i + 1])) for i in range(c)],
                         preempted=pp[:pr].tolist())

    def complete(self, finished: Sequence[int] = ()) -> List[int]:
        fin = _host_i32(list(finished) or [0])
        n = len(list(finished))
        _, _, _, running = self.stats_tuple()
        out = np.zeros(max(running, 1), np.int32)
        ns = ctypes.c_int32(0)
        _check(lib().pkv_sched_complete(self._h, _ptr(fin), n, _ptr(out), ctypes.byref(ns)))
        return out[:ns.value].tolist()

    def trim(self, seq_id: int, n_tokens: int) -> None:
        _check(lib().pkv_sched_trim(self._h, int(seq_id), int(n_tokens)))

    def fork(self, src_id: int, new_id: int) -> None:
        _check(lib().pkv_sched_fork(self._h, int(src_id), int(new_id)))

    def seq_info(self, seq_id: int) -> Tuple[int, int, int, int]:
        v = [ctypes.c_int32(0) for _ in range(4)]
        _check(lib().pkv_sched_seq_info(self._h, int(seq_id), *[ctypes.byref(x) for x in v]))
        return tuple(x.value for x in v)

    def seq_blocks(self, seq_id: int) -> List[int]:
        n = self.seq_info(seq_id)[3]
        out = np.zeros(max(n, 1), np.int32)
        _check(lib().pkv_sched_seq_blocks(self._h, int(seq_id), _ptr(out)))
        return out[:n].tolist()

    def stats_tuple(self) -> Tuple[int, int, int, int]:
        pre, sh = _i64(0), _i64(0)
        run, wait = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pkv_sched_stats(self._h, ctypes.byref(pre), ctypes.byref(sh),
                                     ctypes.byref(run), ctypes.byref(wait)))
        return pre.value, sh.value, wait.value, run.value

    def check(self) -> bool:
        st = lib().pkv_sched_check(self._h)
        if st == PKV_ERR_INCONSISTENT:
            return False
        _check(st)
        return True


def slot_mapping_step(allocator: "BlockAllocator", block_tables, block_size: int, start_pos,
                      n_new, out: Optional[np.ndarray] = None) -> np.ndarray:
    """pkv_slot_mapping_step: the slots of every sequence's new positions, in sequence order."""
    bt = _host_i32(block_tables)
    st = _host_i32(start_pos)
    nn = _host_i32(n_new)
    total = int(nn.sum())
    if out is None or out.size < total or out.dtype != np.int32:
        out = np.zeros(max(total, 1), dtype=np.int32)
    _check(lib().pkv_slot_mapping_step(allocator._h, _ptr(bt), bt.shape[0],
                                       bt.shape[1] if bt.ndim == 2 else 0, int(block_size),
                                       _ptr(st), _ptr(nn), _ptr(out)))
    return out[:total]


def validate_slots(slots, num_slots: int) -> None:
    a = _host_i32(slots)
    _check(lib().pkv_validate_slots(_ptr(a), a.size, int(num_slots)))


# ---- device entry points -------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise Unsupported(PKV_ERR_UNSUPPORTED, f"element type {t.dtype} (float32 or bfloat16)")


def _stream_ptr(t, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _on_stream(stream):
    """Context in which the wrappers allocate their temporaries (device copies of host slots,
    workspaces, outputs): the stream the library enqueues on. Memory the caching allocator
    hands out there is only reused by work ordered after ours on that stream, and a host-slot
    copy made there runs before the kernel that reads it."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need_cuda(*ts):
    for t in ts:
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("device arguments must be contiguous GPU tensors")


def write_kv(k_new, v_new, slots, k_cache, v_cache, stream=None) -> None:
    """pkv_write_kv: scatter rows of k_new / v_new [T_w, Hkv, D] into the pools through slots.

    ``slots`` is a device int32 tensor, or a host array that is validated with
    pkv_validate_slots (range and duplicates) and then copied to the device.
    """
    import torch
    _need_cuda(k_new, v_new, k_cache, v_cache)
    nb, bs, hkv, d = k_cache.shape
    with _on_stream(stream):
        if hasattr(slots, "is_cuda") and slots.is_cuda:
            sl = slots
        else:
            host = _host_i32(slots)
            validate_slots(host, nb * bs)
            sl = torch.from_numpy(host).to(k_cache.device)
        if sl.dtype != torch.int32 or not sl.is_contiguous():
            raise ValueError("slots must be a contiguous int32 tensor")
        _check(lib().pkv_write_kv(k_new.data_ptr(), v_new.data_ptr(), sl.data_ptr(),
                                  int(k_new.shape[0]), k_cache.data_ptr(), v_cache.data_ptr(), nb,
                                  bs, hkv, d, _dtype_code(k_cache), _stream_ptr(k_cache, stream)))


def copy_blocks(pairs, k_cache, v_cache, workspace=None, stream=None) -> None:
    """pkv_copy_blocks: for each (src, dst) pair, dst block of both pools := src block."""
    import torch
    _need_cuda(k_cache, v_cache)
    pr = _host_i32(np.asarray(list(pairs), dtype=np.int32).reshape(-1))
    n = pr.size // 2
    if n == 0:
        return
    nb, bs, hkv, d = k_cache.shape
    need = (8 * n + 255) // 256 * 256
    dt = PKV_E4M3 if k_cache.dtype == torch.uint8 else _dtype_code(k_cache)
    with _on_stream(stream):
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=k_cache.device)
        _check(lib().pkv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), _ptr(pr), n, nb, bs,
                                     hkv, d, dt, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream_ptr(k_cache, stream)))


def attention_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int, num_kv_heads: int,
                             head_dim: int, kv_split: int = 512, dtype: int = PKV_BF16,
                             phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_attention_workspace_size_ex(_ptr(ctx), _ptr(cu), ctx.size, int(num_q_heads),
                                                 int(num_kv_heads), int(head_dim), int(kv_split),
                                                 int(dtype), flags, ctypes.byref(out)))
    return int(out.value)


def attention(q, k_cache, v_cache, block_tables, ctx_lens, cu_seqlens_q, scale: float,
              out=None, workspace=None, kv_split: int = 512, stream=None,
              phase_consistent: bool = False):
    """pkv_attention over a flat ragged step; returns out (float32 [T, Hq, D]).

    q [T, Hq, D], pools [NB, BS, Hkv, D] (same element type), block_tables int32 [B, MB] on
    the device; ctx_lens [B] and cu_seqlens_q [B + 1] on the host. phase_consistent=True calls
    pkv_attention_ex with PKV_ATTN_PHASE_CONSISTENT (decode rows on the prefill tile path).
    """
    import torch
    _need_cuda(q, k_cache, v_cache, block_tables)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or q.dtype != k_cache.dtype:
        raise ValueError("q / pool shape or dtype mismatch")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    dt = _dtype_code(q)
    need = attention_workspace_size(ctx, cu, hq, hkv, d, kv_split, dt, phase_consistent)
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        args = [q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
                float(scale), int(kv_split), dt]
        tail = [out.data_ptr(), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)]
        if phase_consistent:
            _check(lib().pkv_attention_ex(*args, PKV_ATTN_PHASE_CONSISTENT, *tail))
        else:
            _check(lib().pkv_attention(*args, *tail))
    return out


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # PKV_NOALLOC_SCRATCH_BYTES of include/pkv.h


def attention_noalloc(q, k_cache, v_cache, block_tables, ctx_lens, cu_seqlens_q, scale: float,
                      out, kv_split: int = 512, stream=None, phase_consistent: bool = False):
    """pkv_attention_noalloc: pkv_attention_ex over the library's own device scratch (no
    workspace argument, no allocation after the first call on a device). ``out`` (float32
    [T, Hq, D]) is required: this wrapper allocates nothing either."""
    import torch
    _need_cuda(q, k_cache, v_cache, block_tables, out)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or q.dtype != k_cache.dtype:
        raise ValueError("q / pool shape or dtype mismatch")
    if out.dtype != torch.float32 or tuple(out.shape) != (T, hq, d):
        raise ValueError("out must be float32 [T, Hq, D]")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_attention_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb, float(scale),
        int(kv_split), _dtype_code(q), flags, out.data_ptr(), _stream_ptr(q, stream)))
    return out


def write_kv_attention_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int,
                                     num_kv_heads: int, head_dim: int, n_rows: int,
                                     kv_split: int = 512, dtype: int = PKV_BF16,
                                     phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_write_kv_attention_workspace_size(
        _ptr(ctx), _ptr(cu), ctx.size, int(num_q_heads), int(num_kv_heads), int(head_dim),
        int(kv_split), int(dtype), flags, int(n_rows), ctypes.byref(out)))
    return int(out.value)


def write_kv_attention(q, k_new, v_new, slots, k_cache, v_cache, block_tables, ctx_lens,
                       cu_seqlens_q, scale: float, out=None, workspace=None, kv_split: int = 512,
                       stream=None, phase_consistent: bool = False):
    """pkv_write_kv_attention: the KV append of k_new / v_new [T_w, Hkv, D] through host slots
    [T_w] and the attention over the step in one call (one host-to-device copy); returns out.
    """
    import torch
    _need_cuda(q, k_new, v_new, k_cache, v_cache, block_tables)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    sl = slots if isinstance(slots, np.ndarray) and slots.dtype == np.int32 and \
        slots.flags.c_contiguous else _host_i32(slots)
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or q.dtype != k_cache.dtype:
        raise ValueError("q / pool shape or dtype mismatch")
    n_rows = int(k_new.shape[0])
    if sl.size != n_rows or v_new.shape != k_new.shape:
        raise ValueError("slots / k_new / v_new row counts differ")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    dt = _dtype_code(q)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if workspace is None:
            need = write_kv_attention_workspace_size(ctx, cu, hq, hkv, d, n_rows, kv_split, dt,
                                                     phase_consistent)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            ws_have = workspace.numel()
        _check(lib().pkv_write_kv_attention(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), _ptr(sl), n_rows,
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
            float(scale), int(kv_split), dt, flags, out.data_ptr(), workspace.data_ptr(), ws_have,
            _stream_ptr(q, stream)))
    return out


def write_kv_attention_shared_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int,
                                            num_kv_heads: int, head_dim: int, n_rows: int,
                                            block_tables_host, block_size: int,
                                            kv_split: int = 512, dtype: int = PKV_BF16,
                                            phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    bt = _host_i32(block_tables_host)
    mb = int(bt.shape[1]) if bt.ndim == 2 else 0
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_write_kv_attention_shared_workspace_size(
        _ptr(ctx), _ptr(cu), ctx.size, int(num_q_heads), int(num_kv_heads), int(head_dim),
        int(kv_split), int(dtype), flags, int(n_rows), _ptr(bt), mb, int(block_size),
        ctypes.byref(out)))
    return int(out.value)


def write_kv_attention_shared(q, k_new, v_new, slots, k_cache, v_cache, block_tables,
                              block_tables_host, ctx_lens, cu_seqlens_q, scale: float, out=None,
                              workspace=None, kv_split: int = 512, stream=None,
                              phase_consistent: bool = False):
    """pkv_write_kv_attention_shared: pkv_write_kv_attention with a host copy of the block
    tables ([B, max_blocks], the device tables' entries), so that decode splits shared by
    several rows are read once per group of rows; same output bits. Returns out."""
    import torch
    _need_cuda(q, k_new, v_new, k_cache, v_cache, block_tables)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    sl = slots if isinstance(slots, np.ndarray) and slots.dtype == np.int32 and \
        slots.flags.c_contiguous else _host_i32(slots)
    bth = _host_i32(block_tables_host)
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or q.dtype != k_cache.dtype:
        raise ValueError("q / pool shape or dtype mismatch")
    n_rows = int(k_new.shape[0])
    if sl.size != n_rows or v_new.shape != k_new.shape:
        raise ValueError("slots / k_new / v_new row counts differ")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B or bth.ndim != 2 or \
            bth.shape[0] != B or bth.shape[1] != block_tables.shape[1]:
        raise ValueError("block_tables (device and host) must be [B, max_blocks]")
    dt = _dtype_code(q)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        if workspace is None:
            need = write_kv_attention_shared_workspace_size(ctx, cu, hq, hkv, d, n_rows, bth, bs,
                                                            kv_split, dt, phase_consistent)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check(lib().pkv_write_kv_attention_shared(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), _ptr(sl), n_rows,
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), _ptr(bth),
            int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
            float(scale), int(kv_split), dt, flags, out.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)))
    return out


# ---- FP8 (E4M3) pools with per-tensor scales ----------------------------------------------

def _need_fp8_pools(k_cache, v_cache):
    import torch
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("E4M3 pools are uint8 tensors of codes")
    if v_cache.shape != k_cache.shape or k_cache.dim() != 4:
        raise ValueError("pools must both be [num_blocks, block_size, num_kv_heads, head_dim]")


def write_kv_fp8(k_new, v_new, slots, k_cache, v_cache, k_scale: float, v_scale: float,
                 stream=None) -> None:
    """pkv_write_kv_fp8: quantise bfloat16 rows of k_new / v_new [T_w, Hkv, D] to E4M3 codes
    (value / scale, saturating, ties to even) and scatter them into the uint8 pools."""
    import torch
    _need_cuda(k_new, v_new, k_cache, v_cache)
    _need_fp8_pools(k_cache, v_cache)
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new / v_new must be bfloat16")
    nb, bs, hkv, d = k_cache.shape
    with _on_stream(stream):
        if hasattr(slots, "is_cuda") and slots.is_cuda:
            sl = slots
        else:
            host = _host_i32(slots)
            validate_slots(host, nb * bs)
            sl = torch.from_numpy(host).to(k_cache.device)
        if sl.dtype != torch.int32 or not sl.is_contiguous():
            raise ValueError("slots must be a contiguous int32 tensor")
        _check(lib().pkv_write_kv_fp8(k_new.data_ptr(), v_new.data_ptr(), sl.data_ptr(),
                                      int(k_new.shape[0]), k_cache.data_ptr(), v_cache.data_ptr(),
                                      nb, bs, hkv, d, float(k_scale), float(v_scale),
                                      _stream_ptr(k_cache, stream)))


def attention_fp8_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int, num_kv_heads: int,
                                 head_dim: int, kv_split: int = 512,
                                 phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_attention_fp8_workspace_size(_ptr(ctx), _ptr(cu), ctx.size,
                                                  int(num_q_heads), int(num_kv_heads),
                                                  int(head_dim), int(kv_split), flags,
                                                  ctypes.byref(out)))
    return int(out.value)


def attention_fp8(q, k_cache, v_cache, block_tables, ctx_lens, cu_seqlens_q, scale: float,
                  k_scale: float, v_scale: float, out=None, workspace=None,
                  kv_split: int = 512, stream=None, phase_consistent: bool = False):
    """pkv_attention_fp8: the ragged step over E4M3 pools (uint8 [NB, BS, Hkv, D]) with
    per-tensor scales; q bfloat16 [T, Hq, D]; returns out (float32 [T, Hq, D]).
    phase_consistent=True sets PKV_ATTN_PHASE_CONSISTENT (every row on the tile path)."""
    import torch
    _need_cuda(q, k_cache, v_cache, block_tables)
    _need_fp8_pools(k_cache, v_cache)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("q / pool head_dim mismatch")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    need = attention_fp8_workspace_size(ctx, cu, hq, hkv, d, kv_split, phase_consistent)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check(lib().pkv_attention_fp8(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
            float(scale), float(k_scale), float(v_scale), int(kv_split), flags, out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_ptr(q, stream)))
    return out


def write_kv_attention_fp8_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int,
                                         num_kv_heads: int, head_dim: int, n_rows: int,
                                         kv_split: int = 512,
                                         phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_write_kv_attention_fp8_workspace_size(
        _ptr(ctx), _ptr(cu), ctx.size, int(num_q_heads), int(num_kv_heads), int(head_dim),
        int(kv_split), flags, int(n_rows), ctypes.byref(out)))
    return int(out.value)


def write_kv_attention_fp8(q, k_new, v_new, slots, k_cache, v_cache, block_tables, ctx_lens,
                           cu_seqlens_q, scale: float, k_scale: float, v_scale: float, out=None,
                           workspace=None, kv_split: int = 512, stream=None,
                           phase_consistent: bool = False):
    """pkv_write_kv_attention_fp8: the E4M3 append of bfloat16 k_new / v_new [T_w, Hkv, D]
    through host slots [T_w] and the attention over the step in one call; returns out."""
    import torch
    _need_cuda(q, k_new, v_new, k_cache, v_cache, block_tables)
    _need_fp8_pools(k_cache, v_cache)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    if q.dtype != torch.bfloat16 or k_new.dtype != torch.bfloat16 or \
            v_new.dtype != torch.bfloat16:
        raise ValueError("q, k_new and v_new must be bfloat16")
    sl = slots if isinstance(slots, np.ndarray) and slots.dtype == np.int32 and \
        slots.flags.c_contiguous else _host_i32(slots)
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("q / pool head_dim mismatch")
    n_rows = int(k_new.shape[0])
    if sl.size != n_rows or v_new.shape != k_new.shape:
        raise ValueError("slots / k_new / v_new row counts differ")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        if workspace is None:
            need = write_kv_attention_fp8_workspace_size(ctx, cu, hq, hkv, d, n_rows, kv_split,
                                                         phase_consistent)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check(lib().pkv_write_kv_attention_fp8(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), _ptr(sl), n_rows,
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
            float(scale), float(k_scale), float(v_scale), int(kv_split), flags, out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_ptr(q, stream)))
    return out


def write_kv_attention_shared_fp8_workspace_size(ctx_lens, cu_seqlens_q, num_q_heads: int,
                                                num_kv_heads: int, head_dim: int, n_rows: int,
                                                block_tables_host, block_size: int,
                                                kv_split: int = 512,
                                                phase_consistent: bool = False) -> int:
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    bt = _host_i32(block_tables_host)
    mb = int(bt.shape[1]) if bt.ndim == 2 else 0
    out = ctypes.c_size_t(0)
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    _check(lib().pkv_write_kv_attention_shared_fp8_workspace_size(
        _ptr(ctx), _ptr(cu), ctx.size, int(num_q_heads), int(num_kv_heads), int(head_dim),
        int(kv_split), flags, int(n_rows), _ptr(bt), mb, int(block_size), ctypes.byref(out)))
    return int(out.value)


def write_kv_attention_shared_fp8(q, k_new, v_new, slots, k_cache, v_cache, block_tables,
                                  block_tables_host, ctx_lens, cu_seqlens_q, scale: float,
                                  k_scale: float, v_scale: float, out=None, workspace=None,
                                  kv_split: int = 512, stream=None,
                                  phase_consistent: bool = False):
    """pkv_write_kv_attention_shared_fp8: pkv_write_kv_attention_fp8 with a host copy of the
    block tables, so that decode splits shared by several rows are read once per group of
    rows; same output bits. Returns out."""
    import torch
    _need_cuda(q, k_new, v_new, k_cache, v_cache, block_tables)
    _need_fp8_pools(k_cache, v_cache)
    if block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32")
    if q.dtype != torch.bfloat16 or k_new.dtype != torch.bfloat16 or \
            v_new.dtype != torch.bfloat16:
        raise ValueError("q, k_new and v_new must be bfloat16")
    sl = slots if isinstance(slots, np.ndarray) and slots.dtype == np.int32 and \
        slots.flags.c_contiguous else _host_i32(slots)
    bth = _host_i32(block_tables_host)
    ctx = _host_i32(ctx_lens)
    cu = _host_i32(cu_seqlens_q)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("q / pool head_dim mismatch")
    n_rows = int(k_new.shape[0])
    if sl.size != n_rows or v_new.shape != k_new.shape:
        raise ValueError("slots / k_new / v_new row counts differ")
    B = ctx.size
    if block_tables.dim() != 2 or block_tables.shape[0] != B or bth.ndim != 2 or \
            bth.shape[0] != B or bth.shape[1] != block_tables.shape[1]:
        raise ValueError("block_tables (device and host) must be [B, max_blocks]")
    flags = PKV_ATTN_PHASE_CONSISTENT if phase_consistent else 0
    with _on_stream(stream):
        if out is None:
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
        _need_cuda(out)
        if workspace is None:
            need = write_kv_attention_shared_fp8_workspace_size(
                ctx, cu, hq, hkv, d, n_rows, bth, bs, kv_split, phase_consistent)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check(lib().pkv_write_kv_attention_shared_fp8(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), _ptr(sl), n_rows,
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), _ptr(bth),
            int(block_tables.shape[1]), _ptr(ctx), _ptr(cu), B, T, hq, hkv, d, bs, nb,
            float(scale), float(k_scale), float(v_scale), int(kv_split), flags, out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_ptr(q, stream)))
    return out


# ---- diagnostics ---------------------------------------------------------------------------

def profile_enable(on: bool = True) -> None:
    """Start (clearing old records) or stop per-kernel HIP-event timing inside the library."""
    _check(lib().pkv_profile_enable(1 if on else 0))


def profile_set_kinds(kinds: Sequence[str]) -> None:
    """Bracket only these kernel kinds from now on while profiling is enabled."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS[k]
    _check(lib().pkv_profile_set_kinds(mask))


def profile_read(kind: str) -> Tuple[float, int]:
    """(summed device ms, launch count) of one kernel kind since profile_enable(True)."""
    ms = ctypes.c_double(0.0)
    n = _i64(0)
    _check(lib().pkv_profile_read(KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def staging_info() -> Tuple[int, int]:
    """(bytes per staging slot, arena allocations so far) on the current device."""
    sb = ctypes.c_size_t(0)
    n = _i64(0)
    _check(lib().pkv_staging_info(ctypes.byref(sb), ctypes.byref(n)))
    return int(sb.value), int(n.value)


def profile_read_span(kinds: Sequence[str]) -> Tuple[float, int]:
    """(summed per-call span in ms, call count) of the bracketed launches of these kinds: for
    each attention call, from the earliest start to the latest end among them."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS[k]
    ms = ctypes.c_double(0.0)
    n = _i64(0)
    _check(lib().pkv_profile_read_span(mask, ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
