"""ctypes binding of the streaming-read probe (stream_read.hip): the HBM read
ceiling that bench.py reports beside the library's own rate.  Measurement
only; the skinny-GEMM library does not use it."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

ORDER_WAVES = 0
ORDER_WORKGROUPS = 1


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libskinny_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.skinny_probe_stream_read.restype = ctypes.c_int
        L.skinny_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong,
                                               ctypes.c_longlong, ctypes.c_longlong, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p]
        L.skinny_probe_stream_read_tiles.restype = ctypes.c_int
        L.skinny_probe_stream_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_longlong,
                                                     ctypes.c_longlong, ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_void_p, ctypes.c_void_p]
        L.skinny_probe_tiles_writes.restype = ctypes.c_int
        L.skinny_probe_tiles_writes.argtypes = [ctypes.c_void_p, ctypes.c_longlong,
                                                ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong,
                                                ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


WRITE_MODES = {0: "no stores", 1: "4 fp32 stores per lane per unit (0.8% of the bytes)",
               2: "1 fp32 store per lane per unit (0.2%)", 3: "the 4 as nontemporal stores",
               4: "the 4 into a 64 KB region (cache-resident)",
               5: "the 4 hidden from the compiler's wait analysis",
               6: "the 4 every 4th unit only (mode 2's bytes in rarer bursts)",
               7: "16 every 16th unit (mode 1's bytes in rarer bursts)"}


def measure_tiles_writes(buf, row_bytes: int, mode: int, workgroups: int, lds_bytes: int,
                         reps: int = 5) -> float:
    """GB/s read by the tile pattern with writes added at the end of each unit
    of 128 rows (mode: WRITE_MODES)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    nbytes -= nbytes % (128 * row_bytes)
    units = nbytes // row_bytes // 128
    out = torch.empty(max(8192 * units, 16384), dtype=torch.float32, device=buf.device)
    sink = torch.zeros(workgroups, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()

    def go():
        rc = lib().skinny_probe_tiles_writes(buf.data_ptr(), nbytes, row_bytes, workgroups, mode,
                                             lds_bytes, out.data_ptr(), out.numel(),
                                             sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"skinny_probe_tiles_writes failed ({rc})")
    for _ in range(2):
        go()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        go()
    e1.record(stream)
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def measure_tiles(buf, row_bytes: int, wpb: int, ksplit: bool, workgroups_per_cu: int,
                  reps: int = 5, nontemporal: bool = False) -> float:
    """GB/s of the matrix-core kernel's read pattern over the whole of buf."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    nbytes -= nbytes % (16 * wpb * row_bytes)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    workgroups = cus * workgroups_per_cu
    sink = torch.zeros(workgroups, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()

    def go():
        rc = lib().skinny_probe_stream_read_tiles(buf.data_ptr(), nbytes, row_bytes, wpb,
                                                  int(ksplit), workgroups, int(nontemporal),
                                                  sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"skinny_probe_stream_read_tiles failed ({rc})")
    for _ in range(2):
        go()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        go()
    e1.record(stream)
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def stream_read(buf, nbytes: int, row_bytes: int, order: int, u: int, workgroups: int, sink,
                stream: int, read_bytes: int | None = None, nontemporal: bool = False):
    """Enqueue one read of the first nbytes of the device tensor buf (of each
    row, its first read_bytes; default the whole row)."""
    rc = lib().skinny_probe_stream_read(buf.data_ptr(), nbytes, row_bytes, read_bytes or row_bytes,
                                        order, u, workgroups, int(nontemporal), sink.data_ptr(),
                                        stream)
    if rc != 0:
        raise RuntimeError(f"skinny_probe_stream_read failed ({rc})")


def measure(buf, row_bytes: int, order: int, u: int, waves_per_cu: int, reps: int = 5,
            cus: int | None = None, read_bytes: int | None = None,
            nontemporal: bool = False) -> float:
    """GB/s read by `reps` back-to-back reads of buf (of each row, its first
    read_bytes; HIP events on the current stream, after two untimed reads)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    nbytes -= nbytes % row_bytes
    read = read_bytes or row_bytes
    if cus is None:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
    workgroups = cus * waves_per_cu // 4
    sink = torch.zeros(workgroups, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        stream_read(buf, nbytes, row_bytes, order, u, workgroups, sink, stream.cuda_stream, read,
                    nontemporal)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        stream_read(buf, nbytes, row_bytes, order, u, workgroups, sink, stream.cuda_stream, read,
                    nontemporal)
    e1.record(stream)
    torch.cuda.synchronize()
    return nbytes // row_bytes * read * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
