"""Python binding of libmbd (include/mbd.h): weight-only low-bit decode GEMV on MI355X.

The functions keep the C names and only marshal arguments: numpy arrays for the
CPU packer, torch device tensors (memory and streams) for the GPU calls.  Every
computation runs in libmbd; if the library is not built, importing the native
symbols raises.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._native import (  # noqa: F401
    MBD_CASSANDRA, MBD_EALIGN, MBD_EFORMAT, MBD_EHIP, MBD_EINVAL, MBD_ENOMEM, MBD_ERANGE,
    MBD_CASSANDRA_MX, MBD_ESHAPE, MBD_INT4_G128, MBD_MX32, MBD_OK, MBD_TERNARY_B128, MBD_TERNARY_SKIP, MbdDWeights, MbdError,
    MbdEncodePlan, MbdPackParams, MbdSection, MbdStats, check, lib,
)

SECTION_NAMES = {
    MBD_TERNARY_B128: ["codes", "scales"],
    MBD_INT4_G128: ["codes", "scales"],
    MBD_CASSANDRA: ["bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix", "lo_nib", "pruned"],
    MBD_MX32: ["mx_exp", "mx_sign", "mx_mag"],
    MBD_TERNARY_SKIP: ["codes", "scales", "slabs", "tile_base"],
    MBD_CASSANDRA_MX: ["bitmap", "mx_nib", "mx_sign", "mx_exp", "kprefix"],
}
SPEC_SECTIONS = ("bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix")


class Packed:
    """Owns an mbd_packed handle (host sections written by the C++ packer)."""

    def __init__(self, handle: ctypes.c_void_p, fmt: int, M: int, K: int, n_mats: int = 1):
        self._h = handle
        self._free = lib().mbd_packed_free        # the library that allocated the handle frees it
        self.fmt, self.M, self.K, self.n_mats = fmt, M, K, n_mats

    def __del__(self):
        h, free = getattr(self, "_h", None), getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            self._h = None

    def sections(self) -> dict:
        """name -> (uint8 copy of the padded section, meaningful byte count)."""
        L = lib()
        n = ctypes.c_int32(0)
        check(L.mbd_packed_sections(self._h, None, 0, ctypes.byref(n)), "mbd_packed_sections")
        arr = (MbdSection * n.value)()
        check(L.mbd_packed_sections(self._h, arr, n.value, ctypes.byref(n)), "mbd_packed_sections")
        out = {}
        for s in arr:
            buf = (ctypes.c_uint8 * s.padded_bytes).from_address(s.data)
            out[s.name.decode()] = (np.frombuffer(buf, dtype=np.uint8).copy(), int(s.bytes))
        return out

    def section(self, name: str, dtype) -> np.ndarray:
        """Meaningful bytes of one section viewed as ``dtype``."""
        raw, nbytes = self.sections()[name]
        return raw[:nbytes].view(dtype)

    def stats(self) -> MbdStats:
        st = MbdStats()
        check(lib().mbd_packed_stats(self._h, ctypes.byref(st)), "mbd_packed_stats")
        return st

    def validate(self) -> None:
        check(lib().mbd_validate(self._h), "mbd_validate")


def mbd_pack(fmt: int, w_bits: np.ndarray, act_norm: np.ndarray | None = None,
             keep_num: int = 3, keep_den: int = 10, n_mats: int = 1) -> Packed:
    """Pack bf16 bits [M][K] (numpy uint16) on the CPU; n_mats > 1 packs the rows as
    that many stacked matrices (ternary / INT4, for the expert GEMV)."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("w_bits must be 2-D [M][K]")
    M, K = w.shape
    nrm = None
    if act_norm is not None:
        nrm = np.ascontiguousarray(act_norm, dtype=np.float32)
    params = MbdPackParams(keep_num, keep_den, n_mats)
    h = ctypes.c_void_p()
    st = lib().mbd_pack(fmt, w.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), M, K,
                        None if nrm is None else nrm.ctypes.data, ctypes.byref(params), ctypes.byref(h))
    check(st, "mbd_pack")
    return Packed(h, fmt, M, K, n_mats)


class DeviceWeights:
    """Device copies (torch uint8 tensors) of packed sections plus the mbd_dweights
    descriptor that points at them.  ``n_mats`` > 1 describes stacked matrices."""

    def __init__(self, packed: Packed, device="cuda", n_mats: int = 1, only=None):
        import torch
        secs = packed.sections()
        names = SECTION_NAMES[packed.fmt]
        st = packed.stats()
        self.tensors = {}
        self.desc = MbdDWeights()
        self.desc.fmt = packed.fmt
        self.desc.n_sym = st.n_sym
        if packed.M % n_mats:
            raise ValueError("rows not divisible by n_mats")
        if n_mats != packed.n_mats and packed.fmt in (MBD_TERNARY_B128, MBD_INT4_G128):
            raise ValueError("packed as %d matrices, described as %d: pack with mbd_pack(..., n_mats=%d)"
                             % (packed.n_mats, n_mats, n_mats))
        self.desc.M = packed.M // n_mats
        self.desc.K = packed.K
        self.desc.n_kept = st.n_kept
        self.desc.n_mats = n_mats
        self.bytes = {}
        for i, name in enumerate(names):
            raw, nbytes = secs[name]
            self.bytes[name] = nbytes
            if only is not None and name not in only:
                self.desc.sec[i] = None
                continue
            t = torch.from_numpy(raw).to(device)
            self.tensors[name] = t
            self.desc.sec[i] = t.data_ptr()
        self.fmt, self.M, self.K, self.n_mats = packed.fmt, self.desc.M, packed.K, n_mats

    def ref(self):
        return ctypes.byref(self.desc)


def to_device(packed: Packed, device="cuda", n_mats: int = 1, only=None) -> DeviceWeights:
    return DeviceWeights(packed, device, n_mats, only)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def mbd_gemv(dw: DeviceWeights, x, y, stream=None) -> None:
    """y [B][M] fp32 = W x for bf16 x [B][K] (torch tensors on the device)."""
    check(lib().mbd_gemv(dw.ref(), _ptr(x), int(x.shape[0]), _ptr(y), _stream(stream)), "mbd_gemv")


def mbd_dequant(dw: DeviceWeights, out, stream=None) -> None:
    check(lib().mbd_dequant(dw.ref(), _ptr(out), _stream(stream)), "mbd_dequant")


def mbd_moe_workspace_bytes(n_mats: int, T: int, k: int) -> int:
    b = ctypes.c_uint64(0)
    check(lib().mbd_moe_workspace_bytes(n_mats, T, k, ctypes.byref(b)), "mbd_moe_workspace_bytes")
    return int(b.value)


def mbd_moe_gemv(dw: DeviceWeights, route, x, x_per_pair: bool, y, ws, stream=None) -> None:
    T, k = int(route.shape[0]), int(route.shape[1])
    check(lib().mbd_moe_gemv(dw.ref(), _ptr(route), T, k, _ptr(x), int(bool(x_per_pair)), _ptr(y),
                             _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)), "mbd_moe_gemv")


def mbd_moe_gemv_noalloc(dw: DeviceWeights, route, x, x_per_pair: bool, y, stream=None) -> None:
    """mbd_moe_gemv without a workspace (the library's static device scratch)."""
    T, k = int(route.shape[0]), int(route.shape[1])
    check(lib().mbd_moe_gemv_noalloc(dw.ref(), _ptr(route), T, k, _ptr(x), int(bool(x_per_pair)), _ptr(y),
                                     _stream(stream)), "mbd_moe_gemv_noalloc")


def mbd_spec_decode(dw: DeviceWeights, out, stream=None) -> None:
    check(lib().mbd_spec_decode(dw.ref(), _ptr(out), _stream(stream)), "mbd_spec_decode")


def mbd_spec_gemv(dw: DeviceWeights, x, y, stream=None) -> None:
    check(lib().mbd_spec_gemv(dw.ref(), _ptr(x), int(x.shape[0]), _ptr(y), _stream(stream)), "mbd_spec_gemv")


def mbd_verify_restore(dw: DeviceWeights, out, stream=None) -> None:
    check(lib().mbd_verify_restore(dw.ref(), _ptr(out), _stream(stream)), "mbd_verify_restore")


def mbd_encode_workspace_bytes(M: int) -> int:
    n = ctypes.c_uint64(0)
    check(lib().mbd_encode_workspace_bytes(M, ctypes.byref(n)), "mbd_encode_workspace_bytes")
    return int(n.value)


def mbd_encode_plan(w, act_norm, keep_num: int, keep_den: int, ws, stream=None) -> MbdEncodePlan:
    """Device encoder, first call (synchronises the stream): section sizes of the
    Cassandra sections of device bf16 w [M][K] (int16 tensor) and fp32 act_norm."""
    M, K = w.shape
    plan = MbdEncodePlan()
    check(lib().mbd_encode_plan(_ptr(w), _ptr(act_norm), M, K, keep_num, keep_den, _ptr(ws), ws.numel() * ws.element_size(),
                                ctypes.byref(plan), _stream(stream)), "mbd_encode_plan")
    return plan


def mbd_encode_cassandra(w, act_norm, keep_num: int, keep_den: int, plan: MbdEncodePlan, sections, ws, stream=None) -> None:
    """Device encoder, second call: writes the eight sections into ``sections``
    (device uint8 tensors of at least plan.padded_bytes[i] bytes each)."""
    M, K = w.shape
    arr = (ctypes.c_void_p * 8)(*[t.data_ptr() for t in sections])
    check(lib().mbd_encode_cassandra(_ptr(w), _ptr(act_norm), M, K, keep_num, keep_den, ctypes.byref(plan), arr, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "mbd_encode_cassandra")


def mbd_probe_stream_read(src, sink, blocks: int, threads: int, stream=None) -> None:
    """Streaming-read probe over the whole of ``src`` (a device tensor); measurement aid."""
    check(lib().mbd_probe_stream_read(_ptr(src), int(src.numel() * src.element_size()), _ptr(sink), int(blocks),
                                      int(threads), _stream(stream)), "mbd_probe_stream_read")
