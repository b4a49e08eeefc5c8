"""Sweeps of the streaming-read probe on one GPU; prints one table per sweep.

    python -m gemv_skinny_gemm_amd.probe depth    order x row size x batch x waves per CU
    python -m gemv_skinny_gemm_amd.probe stride   1-2 KB read from the start of every row of a
                                                  given stride (32 GiB buffer)
    python -m gemv_skinny_gemm_amd.probe tiles    the matrix-core kernel's read pattern
    python -m gemv_skinny_gemm_amd.probe nt       plain against nontemporal loads, the fastest
                                                  patterns of the sweeps above and the tiles one
    python -m gemv_skinny_gemm_amd.probe writes   the tiles pattern with stores added at the end
                                                  of every unit (writes in the read stream)

Every figure is GB/s read from an 8 GiB buffer (GiB = 2^30 bytes), best of
three measurements of five passes each.  Measurement only.
"""
import sys

import torch

from gemv_skinny_gemm_amd import probe

GIB = 1 << 30


def best(fn, n=3):
    return max(fn() for _ in range(n))


def depth(buf):
    print("| order | row | KB per batch | waves/CU | GB/s |")
    print("|---|---|---|---|---|")
    for order, rows in ((probe.ORDER_WAVES, (2, 4, 8, 16, 64, 1024)),
                        (probe.ORDER_WORKGROUPS, (16, 32, 128, 512, 2048))):
        for row_kb in rows:
            for u in (1, 2, 4, 8):
                if row_kb % (2 * u):
                    continue
                for wpc in (4, 8, 12, 16, 32):
                    g = best(lambda: probe.measure(buf, row_kb << 10, order, u, wpc))
                    name = "to waves" if order == probe.ORDER_WAVES else "to workgroups"
                    print(f"| {name} | {row_kb} KB | {u} | {wpc} | {g:.0f} |", flush=True)


def stride(buf):
    """1 or 2 KB read from the start of every row of `stride` bytes, rows
    dealt to waves: the requests in flight sit `stride` apart (a 32 GiB
    buffer, so even the widest stride reads 128 MB per pass)."""
    del buf
    big = torch.ones(32 * GIB // 8, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    print("| stride | read per row | waves/CU | GB/s |")
    print("|---|---|---|---|")
    for sk in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        for read_kb, u in ((1, 1), (2, 2)):
            if read_kb > sk:
                continue
            for wpc in (8, 16):
                g = best(lambda: probe.measure(big, sk << 10, probe.ORDER_WAVES, u, wpc,
                                               read_bytes=read_kb << 10))
                print(f"| {sk} KB | {read_kb} KB | {wpc} | {g:.0f} |", flush=True)


def tiles(buf):
    print("| row | waves/workgroup | K split | workgroups/CU | GB/s |")
    print("|---|---|---|---|---|")
    for rb in (8192, 16384, 57344):
        for wpb, wgpc in ((4, 1), (4, 2), (8, 1)):
            for ks in (False, True):
                g = best(lambda: probe.measure_tiles(buf, rb, wpb, ks, wgpc))
                print(f"| {rb >> 10} KB | {wpb} | {int(ks)} | {wgpc} | {g:.0f} |", flush=True)


def nontemporal(buf):
    """The same patterns with plain and with nontemporal loads (the hint the
    library's weight loads carry)."""
    print("| pattern | plain GB/s | nontemporal GB/s |")
    print("|---|---|---|")
    for name, order, row_kb, u, wpc in (
            ("8 KB rows to waves, 2 KB batches, 8 waves/CU", probe.ORDER_WAVES, 8, 2, 8),
            ("32 KB rows to workgroups, 2 KB batches, 8 waves/CU", probe.ORDER_WORKGROUPS, 32, 2, 8),
            ("16 KB rows to waves, 1 KB batches, 16 waves/CU", probe.ORDER_WAVES, 16, 1, 16),
            ("16 KB rows to waves, 4 KB batches, 8 waves/CU", probe.ORDER_WAVES, 16, 4, 8),
            ("16 KB rows to waves, 8 KB batches, 16 waves/CU", probe.ORDER_WAVES, 16, 8, 16),
            ("8 KB rows to waves, 1 KB batches, 8 waves/CU", probe.ORDER_WAVES, 8, 1, 8)):
        g = [best(lambda: probe.measure(buf, row_kb << 10, order, u, wpc, nontemporal=nt))
             for nt in (False, True)]
        print(f"| {name} | {g[0]:.0f} | {g[1]:.0f} |", flush=True)
    for rb in (8192, 16384):
        for wpb, wgpc in ((4, 2), (8, 1)):
            g = [best(lambda: probe.measure_tiles(buf, rb, wpb, False, wgpc, nontemporal=nt))
                 for nt in (False, True)]
            print(f"| tiles: {rb >> 10} KB rows, {wpb}-wave workgroups x {wgpc} per CU | "
                  f"{g[0]:.0f} | {g[1]:.0f} |", flush=True)


def writes(buf):
    """The tile pattern (8 KB rows, nontemporal loads, 252 workgroups of 8
    waves with 160 KB of LDS each, as the 8-wave tile kernel's grid) with
    writes added at the end of every 128-row unit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg = cus - cus % 12     # 252 on 256 CUs: that kernel's grid when it splits K in 2 and 6
    print("| stores at the end of each 1 MB unit | GB/s read |")
    print("|---|---|")
    for mode, name in probe.WRITE_MODES.items():
        g = best(lambda: probe.measure_tiles_writes(buf, 8192, mode, wg, 160 * 1024))
        print(f"| {name} | {g:.0f} |", flush=True)
    g = best(lambda: probe.measure_tiles_writes(buf, 8192, 0, cus, 160 * 1024))
    print(f"| no stores, {cus} workgroups | {g:.0f} |", flush=True)


def main():
    what = sys.argv[1] if len(sys.argv) > 1 else "depth"
    buf = torch.ones(8 * GIB // 8, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    print(f"# {what} sweep, {torch.cuda.get_device_name(0)}", flush=True)
    {"depth": depth, "stride": stride, "tiles": tiles, "nt": nontemporal,
     "writes": writes}[what](buf)


if __name__ == "__main__":
    main()
