"""Python binding of libecw.so: entropy-coded weights decoded inside a batch-1 GEMV.

Argument marshalling only.  Every step of the path (table building, rANS encoding,
validation, decoding and the fused GEMV) runs in the C-ABI library; PyTorch only
provides device memory and the current HIP stream.

    c = Coding(payload=INT_CODES, rows=N, cols=K, weights_per_symbol=2, code_bits=4,
               log2_m=11, tile_cols=256)
    blob = encode(c, codes, scales)          # numpy uint8, format v1
    t = CompressedTensor(blob)               # device copy + validated descriptor
    y = t.gemv(x)                            # x: cuda fp16/bf16 [batch, K] -> fp32 [batch, N]
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch  # noqa: F401  (load torch's HIP runtime first so the library binds to it)

INT_CODES, BF16_EXP, FP8_E4M3, E8_LATTICE = 1, 2, 3, 4
DT_F16, DT_BF16, DT_F32, DT_I8, DT_FP8_E4M3 = 1, 2, 3, 4, 5
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "CORRUPT", 4: "BUFFER_TOO_SMALL", 5: "HIP"}

ABI_VERSION = 3          # layout of the structs below
MAX_TUPLES = 4096
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libecw.so")


class Coding(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "payload", "rows", "cols", "weights_per_symbol", "code_bits", "log2_m",
        "tile_rows", "tile_cols", "recon_dtype", "stored_tuples")]

    def __init__(self, payload, rows, cols, weights_per_symbol=1, code_bits=0, log2_m=12,
                 tile_cols=256, recon_dtype=0, tile_rows=64, stored_tuples=0):
        super().__init__(payload, rows, cols, weights_per_symbol, code_bits, log2_m,
                         tile_rows, tile_cols, recon_dtype, stored_tuples)


class Tables(ctypes.Structure):
    _fields_ = [("n_tables", ctypes.c_uint32),
                ("alphabet", ctypes.c_uint32 * 17),
                ("value_offset", ctypes.c_int32 * 17),
                ("freq", (ctypes.c_uint16 * 256) * 17),
                ("count", (ctypes.c_uint64 * 256) * 17),
                ("pair_values", ctypes.c_uint8 * 16),
                ("escapes", ctypes.c_uint64),
                ("n_tuples", ctypes.c_uint32),
                ("tuples", ctypes.c_uint16 * MAX_TUPLES),
                ("tuple_freq", ctypes.c_uint16 * MAX_TUPLES),
                ("tuple_count", ctypes.c_uint64 * MAX_TUPLES)]

    def freq_array(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.freq)[: self.n_tables].astype(np.int64)

    def count_array(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.count)[: self.n_tables].astype(np.int64)


class Tensor(ctypes.Structure):
    _fields_ = [("coding", Coding)] + [(n, ctypes.c_uint32) for n in (
        "n_tables", "n_row_groups", "n_slices", "n_tiles", "steps_full", "steps_last",
        "lut_entry_bytes", "waves_per_block", "tiles_per_wave", "streams_per_wave",
                                         "row_groups_per_block")] + [
        ("blob_bytes", ctypes.c_uint64), ("bytes_words", ctypes.c_uint64),
        ("bytes_raw", ctypes.c_uint64), ("bytes_tile_meta", ctypes.c_uint64),
        ("bytes_tables", ctypes.c_uint64), ("bytes_scales", ctypes.c_uint64),
        ("device_blob", ctypes.c_void_p)] + [(n, ctypes.c_uint64) for n in (
            "off_tables", "off_lut", "off_states", "off_offsets", "off_words", "off_raw",
            "off_scales")]


EXPORTS = ["enc_build_tables", "enc_encode", "dec_prepare", "dec_gemv_workspace_size",
           "dec_gemv", "dec_gemv_group_workspace_size", "dec_gemv_group", "dec_materialize",
           "dec_dequantize", "ecw_last_error", "ecw_abi_version"]

_lib = None


class EcwError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.ecw_last_error().decode() if _lib is not None else ""
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def lib():
    """Load libecw.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} missing: run __graft_entry__.build() (or "
                          "python entropy_coded_weight_amd/build.py) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, i32, sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_size_t
    P = ctypes.POINTER
    L.enc_build_tables.argtypes = [P(Coding), vp, P(Tables)]
    L.enc_encode.argtypes = [P(Coding), P(Tables), vp, vp, vp, P(sz)]
    L.enc_e8_nearest.argtypes = [vp, sz, vp]
    L.dec_prepare.argtypes = [vp, sz, vp, P(Tensor)]
    L.dec_gemv_workspace_size.argtypes = [P(Tensor), i32, P(sz)]
    L.dec_gemv.argtypes = [vp, P(Tensor), vp, i32, vp, i32, vp, sz]
    L.dec_gemv_noalloc.argtypes = [vp, P(Tensor), vp, i32, vp, i32]
    L.dec_materialize.argtypes = [vp, P(Tensor), vp, vp, vp]
    L.dec_dequantize.argtypes = [vp, P(Tensor), vp, i32]
    L.dec_gemv_group_workspace_size.argtypes = [P(P(Tensor)), i32, i32, P(sz)]
    L.dec_gemv_group.argtypes = [vp, P(P(Tensor)), i32, vp, i32, P(vp), i32, vp, sz]
    L.dec_gemv_group_geometry.argtypes = [P(P(Tensor)), i32, i32, i32, P(u32), P(u32), P(sz)]
    L.dec_tune_launch.argtypes = [vp, P(Tensor), vp, i32, vp, i32, vp, sz, P(u32), i32, i32,
                                  P(ctypes.c_float)]
    L.dec_time_group.argtypes = [vp, P(P(Tensor)), i32, vp, i32, P(vp), i32, vp, sz, i32,
                                 P(ctypes.c_float)]
    L.ecw_probe_stream_read.argtypes = [vp, vp, sz, vp, u32]
    L.ecw_probe_lds_lookup.argtypes = [vp, u32, u32, u32, u32, u32, vp]
    L.ecw_probe_tile_stream.argtypes = [vp, vp, sz, u32, u32, u32, u32, vp]
    L.ecw_probe_clock.argtypes = [vp, u32, u32, vp, P(u32)]
    for f in ("enc_build_tables", "enc_encode", "enc_e8_nearest", "dec_prepare", "dec_gemv_workspace_size",
              "dec_gemv", "dec_gemv_noalloc", "dec_gemv_group_workspace_size", "dec_gemv_group",
              "dec_gemv_group_geometry", "dec_materialize", "dec_dequantize",
              "dec_tune_launch", "dec_time_group", "ecw_probe_stream_read", "ecw_probe_lds_lookup",
              "ecw_probe_tile_stream",
              "ecw_probe_clock"):
        getattr(L, f).restype = ctypes.c_int
    L.ecw_last_error.argtypes = []
    L.ecw_last_error.restype = ctypes.c_char_p
    L.ecw_abi_version.argtypes = []
    L.ecw_abi_version.restype = u32
    if L.ecw_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {L.ecw_abi_version()}, the binding expects "
                          f"{ABI_VERSION}: rebuild the library")
    _lib = L
    return L


def _check(status, where):
    if status != 0:
        raise EcwError(status, where)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _host_logical(coding: Coding, w: np.ndarray) -> np.ndarray:
    dt = {INT_CODES: np.int8, BF16_EXP: np.uint16, FP8_E4M3: np.uint8, E8_LATTICE: np.int8}[coding.payload]
    w = np.ascontiguousarray(w, dtype=dt)
    if w.shape != (coding.rows, coding.cols):
        raise ValueError(f"weights shape {w.shape} != ({coding.rows}, {coding.cols})")
    return w


# ------------------------------------------------------------------ host calls
def build_tables(coding: Coding, w: np.ndarray) -> Tables:
    w = _host_logical(coding, w)
    t = Tables()
    _check(lib().enc_build_tables(ctypes.byref(coding), _ptr(w), ctypes.byref(t)), "enc_build_tables")
    return t


def encode(coding: Coding, w: np.ndarray, scales=None, tables: Tables | None = None) -> np.ndarray:
    w = _host_logical(coding, w)
    if tables is None:
        tables = build_tables(coding, w)
    sc = None
    if scales is not None:
        sc = np.ascontiguousarray(scales, dtype=np.float16).view(np.uint16)
    n = ctypes.c_size_t(0)
    L = lib()
    _check(L.enc_encode(ctypes.byref(coding), ctypes.byref(tables), _ptr(w),
                        _ptr(sc) if sc is not None else None, None, ctypes.byref(n)), "enc_encode")
    buf = np.zeros(n.value, dtype=np.uint8)
    _check(L.enc_encode(ctypes.byref(coding), ctypes.byref(tables), _ptr(w),
                        _ptr(sc) if sc is not None else None, _ptr(buf), ctypes.byref(n)), "enc_encode")
    return buf[: n.value].copy()


def e8_nearest(u: np.ndarray) -> np.ndarray:
    """Nearest E8 lattice point of each block of eight values (enc_e8_nearest):
    u float64 [n, 8] -> doubled coordinates 2v int8 [n, 8]."""
    u = np.ascontiguousarray(u, dtype=np.float64).reshape(-1, 8)
    out = np.empty(u.shape, dtype=np.int8)
    _check(lib().enc_e8_nearest(_ptr(u), u.shape[0], _ptr(out)), "enc_e8_nearest")
    return out


def prepare(blob: np.ndarray, device_ptr: int | None = None) -> Tensor:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    t = Tensor()
    _check(lib().dec_prepare(_ptr(blob), blob.size, device_ptr, ctypes.byref(t)), "dec_prepare")
    return t


def workspace_size(t: Tensor, batch: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dec_gemv_workspace_size(ctypes.byref(t), batch, ctypes.byref(n)), "dec_gemv_workspace_size")
    return n.value


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def gemv_raw(t: Tensor, x: torch.Tensor, y: torch.Tensor, workspace: torch.Tensor | None, stream=None):
    """dec_gemv on caller-provided device buffers (x [batch, K] fp16/bf16, y [batch, N] fp32)."""
    if x.dtype == torch.float16:
        xd = DT_F16
    elif x.dtype == torch.bfloat16:
        xd = DT_BF16
    else:
        raise TypeError("x must be float16 or bfloat16")
    if y.dtype != torch.float32 or not y.is_contiguous() or not x.is_contiguous():
        raise TypeError("y must be contiguous float32; x contiguous")
    batch = x.shape[0]
    ws = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dec_gemv(_stream(stream), ctypes.byref(t), x.data_ptr(), xd, y.data_ptr(), batch,
                          ws, wsb), "dec_gemv")


def _tensor_array(ts):
    arr = (ctypes.POINTER(Tensor) * len(ts))(*[ctypes.pointer(t) for t in ts])
    return arr


def group_workspace_size(ts, batch: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dec_gemv_group_workspace_size(_tensor_array(ts), len(ts), batch, ctypes.byref(n)),
           "dec_gemv_group_workspace_size")
    return n.value


def group_geometry(ts, batch: int, x_dtype: int = None):
    """dec_gemv_group_geometry: (grid threads, block threads, dynamic LDS bytes) of the
    launch dec_gemv_group makes for tensors ts (no GPU needed)."""
    g, b, l = ctypes.c_uint32(0), ctypes.c_uint32(0), ctypes.c_size_t(0)
    _check(lib().dec_gemv_group_geometry(_tensor_array(ts), len(ts), batch, DT_F16 if x_dtype is None else x_dtype,
                                         ctypes.byref(g), ctypes.byref(b), ctypes.byref(l)),
           "dec_gemv_group_geometry")
    return g.value, b.value, l.value


def gemv_group_raw(ts, x: torch.Tensor, ys, workspace: torch.Tensor | None, stream=None):
    """dec_gemv_group: tensors ts share x [batch, K]; ys[i] fp32 [batch, N_i]."""
    xd = DT_F16 if x.dtype == torch.float16 else DT_BF16 if x.dtype == torch.bfloat16 else None
    if xd is None:
        raise TypeError("x must be float16 or bfloat16")
    yarr = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    ws = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dec_gemv_group(_stream(stream), _tensor_array(ts), len(ts), x.data_ptr(), xd, yarr,
                                x.shape[0], ws, wsb), "dec_gemv_group")


class GemvGroup:
    """Compressed tensors sharing one activation vector, run as one launch."""

    def __init__(self, tensors):
        self.tensors = list(tensors)
        self._ws = {}

    def workspace(self, batch: int):
        n = group_workspace_size([c.t for c in self.tensors], batch)
        if n == 0:
            return None
        key = (batch > 1, tuple((c.t.waves_per_block, c.t.tiles_per_wave) for c in self.tensors))
        ws = self._ws.get(key)
        if ws is None or ws.numel() < n:
            ws = torch.zeros(n, dtype=torch.uint8, device=self.tensors[0].dev.device)
            self._ws[key] = ws
        return ws

    def gemv(self, x: torch.Tensor, ys=None, stream=None):
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if ys is None:
            ys = [torch.empty((x.shape[0], c.rows), dtype=torch.float32, device=x.device) for c in self.tensors]
        gemv_group_raw([c.t for c in self.tensors], x, ys, self.workspace(x.shape[0]), stream)
        return ys


def materialize_raw(t: Tensor, symbols, w_out, status, stream=None):
    _check(lib().dec_materialize(_stream(stream), ctypes.byref(t),
                                 symbols.data_ptr() if symbols is not None else None,
                                 w_out.data_ptr() if w_out is not None else None,
                                 status.data_ptr() if status is not None else None), "dec_materialize")


def dequantize_raw(t: Tensor, w_out: torch.Tensor, stream=None):
    """dec_dequantize into a caller-provided device tensor [rows, cols] of fp16/bf16."""
    dt = DT_F16 if w_out.dtype == torch.float16 else DT_BF16 if w_out.dtype == torch.bfloat16 else None
    if dt is None:
        raise ValueError("w_out must be float16 or bfloat16")
    _check(lib().dec_dequantize(_stream(stream), ctypes.byref(t), w_out.data_ptr(), dt), "dec_dequantize")


# ------------------------------------------------------------------ roofline probes
def probe_stream_read(buf: torch.Tensor, blocks: int = 2048, reps: int = 5, region_bytes: int | None = None) -> float:
    """Achievable streaming-read GB/s over the device buffer `buf` (median of reps).
    With region_bytes, each rep reads another region of that size of `buf`, so that
    no rep finds its bytes cached: the rate one launch of that size can reach."""
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    total = buf.numel() * buf.element_size() // 16 * 16
    nbytes = total if region_bytes is None else region_bytes // 16 * 16
    if nbytes <= 0 or nbytes > total:
        raise ValueError("region larger than the buffer")
    nreg = total // nbytes
    s = torch.cuda.current_stream()
    times = []
    for r in range(reps + 1):
        base = buf.data_ptr() + (r % nreg) * nbytes
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(lib().ecw_probe_stream_read(_stream(None), base, nbytes, sink.data_ptr(), blocks),
               "ecw_probe_stream_read")
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    t = sorted(times[1:])[len(times[1:]) // 2]
    return nbytes / (t * 1e-3) / 1e9


def probe_tile_stream(buf: torch.Tensor, kib_per_wave: int, waves: int, waves_per_block: int = 16,
                      inflight: int = 1, reps: int = 5) -> float:
    """GB/s of `waves` per-wave streams of kib_per_wave KiB each (ecw_probe_tile_stream),
    median of reps; every rep reads another region of `buf`, so none is cached."""
    region = waves * kib_per_wave * 1024
    total = buf.numel() * buf.element_size()
    if region > total:
        raise ValueError("buffer smaller than one region")
    nreg = total // region
    sink = torch.empty(waves * 64, dtype=torch.int32, device=buf.device)
    s = torch.cuda.current_stream()
    times = []
    for r in range(reps + 1):
        base = buf.data_ptr() + (r % nreg) * region
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(lib().ecw_probe_tile_stream(_stream(None), base, region, kib_per_wave, waves, waves_per_block,
                                           inflight, sink.data_ptr()), "ecw_probe_tile_stream")
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    t = sorted(times[1:])[len(times[1:]) // 2]
    return region / (t * 1e-3) / 1e9


def probe_lds_lookup(log2_m: int, entry_bytes: int, steps: int = 4096, blocks: int = 512,
                     waves: int = 16) -> float:
    """Dependent LDS table lookups per second over the whole device (median of 3)."""
    sink = torch.empty(blocks * waves * 64, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    times = []
    for _ in range(4):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(lib().ecw_probe_lds_lookup(_stream(None), log2_m, entry_bytes, steps, blocks, waves,
                                          sink.data_ptr()), "ecw_probe_lds_lookup")
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    t = sorted(times[1:])[1]
    return blocks * waves * 64 * steps / (t * 1e-3)


class ClockProbe:
    """The shader clock while other work runs: start() launches ecw_probe_clock on a
    side stream (blocks one-wave blocks busy for duration_us), mhz() waits for it and
    returns the median clock over the blocks in MHz."""

    def __init__(self, duration_us: int = 3000, blocks: int = 8):
        self.duration_us, self.blocks = duration_us, blocks
        self.sink = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
        self.stream = torch.cuda.Stream()
        self.khz = ctypes.c_uint32(0)

    def start(self):
        self.stream.wait_stream(torch.cuda.current_stream())
        _check(lib().ecw_probe_clock(ctypes.c_void_p(self.stream.cuda_stream), self.duration_us, self.blocks,
                                     self.sink.data_ptr(), ctypes.byref(self.khz)), "ecw_probe_clock")

    def mhz(self) -> float:
        self.stream.synchronize()
        v = self.sink.view(-1, 2).cpu().numpy().astype(np.float64)
        f = v[:, 0] / np.maximum(v[:, 1], 1) * self.khz.value / 1e3
        return float(np.median(f))


# ------------------------------------------------------------------ device tensor
class CompressedTensor:
    """A blob resident in device memory plus its validated descriptor."""

    def __init__(self, blob: np.ndarray, device: str = "cuda", waves_per_block=None, tiles_per_wave=None,
                 streams_per_wave=None, row_groups_per_block=None):
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        self.host_blob = blob
        self.dev = torch.from_numpy(blob).to(device)
        if self.dev.data_ptr() % 256:
            raise RuntimeError("device allocation is not 256-byte aligned")
        self.t = prepare(blob, self.dev.data_ptr())
        if waves_per_block is not None:
            self.t.waves_per_block = waves_per_block
        if tiles_per_wave is not None:
            self.t.tiles_per_wave = tiles_per_wave
        if streams_per_wave is not None:
            self.t.streams_per_wave = streams_per_wave
        if row_groups_per_block is not None:
            self.t.row_groups_per_block = row_groups_per_block
        self._ws = {}

    @property
    def rows(self):
        return self.t.coding.rows

    @property
    def cols(self):
        return self.t.coding.cols

    def set_launch(self, waves_per_block: int, tiles_per_wave: int, streams_per_wave: int = 1,
                   row_groups_per_block: int = 1):
        self.t.waves_per_block = waves_per_block
        self.t.tiles_per_wave = tiles_per_wave
        self.t.streams_per_wave = streams_per_wave
        self.t.row_groups_per_block = row_groups_per_block

    def stored_bytes(self) -> int:
        t = self.t
        return t.bytes_words + t.bytes_raw + t.bytes_tile_meta + t.bytes_tables + t.bytes_scales

    def workspace(self, batch: int):
        key = (batch > 1, self.t.waves_per_block, self.t.tiles_per_wave)
        n = workspace_size(self.t, batch)
        if n == 0:
            return None
        ws = self._ws.get(key)
        if ws is None or ws.numel() < n:
            ws = torch.zeros(n, dtype=torch.uint8, device=self.dev.device)
            self._ws[key] = ws
        return ws

    def gemv(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if y is None:
            y = torch.empty((x.shape[0], self.rows), dtype=torch.float32, device=x.device)
        gemv_raw(self.t, x, y, self.workspace(x.shape[0]), stream)
        return y

    def dequantize(self, dtype=torch.float16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """The real weight values as a dense [rows, cols] fp16/bf16 matrix (dec_dequantize)."""
        shape = (self.rows, self.t.coding.cols)
        if out is None:
            out = torch.empty(shape, dtype=dtype, device=self.dev.device)
        elif tuple(out.shape) != shape or not out.is_contiguous() or out.device != self.dev.device:
            raise ValueError(f"out must be a contiguous {shape} tensor on {self.dev.device}")
        dequantize_raw(self.t, out, stream)
        return out

    def gemm(self, x: torch.Tensor, w_buf: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """y = x W^T in fp32 for any batch: up to 4 rows of x the fused decode-GEMV;
        more rows decode W once into a dense matrix (w_buf, if given, is reused) and
        multiply with the library GEMM (hipBLASLt through torch), fp32 output."""
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.shape[-1] != self.t.coding.cols:
            raise ValueError(f"x has {x.shape[-1]} columns, the tensor {self.t.coding.cols}")
        if x.shape[0] <= 4:
            return self.gemv(x, stream=stream)
        w = self.dequantize(x.dtype, w_buf, stream)
        s = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            return torch.mm(x, w.t(), out_dtype=torch.float32)

    def materialize(self, want_symbols=True, want_weights=True, stream=None):
        c = self.t.coding
        n_sym = {INT_CODES: c.cols // max(c.weights_per_symbol, 1), BF16_EXP: c.cols // max(c.weights_per_symbol, 1),
                 FP8_E4M3: c.cols, E8_LATTICE: c.cols // 8 * 9}[c.payload]
        dev = self.dev.device
        sym = torch.zeros((c.rows, n_sym), dtype=torch.int16, device=dev) if want_symbols else None
        wdt = {INT_CODES: torch.int8, BF16_EXP: torch.int16, FP8_E4M3: torch.uint8,
               E8_LATTICE: torch.int8 if c.recon_dtype == DT_I8 else torch.uint8}[c.payload]
        w = torch.zeros((c.rows, c.cols), dtype=wdt, device=dev) if want_weights else None
        st = torch.full((max(self.t.n_tiles, 1),), 0xFFFF, dtype=torch.int32, device=dev)
        materialize_raw(self.t, sym, w, st, stream)
        return sym, w, st[: self.t.n_tiles]
