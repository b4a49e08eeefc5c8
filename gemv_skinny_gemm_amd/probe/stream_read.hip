// stream_read.hip - arithmetic-free streaming reads of a device buffer, the
// HBM read ceiling the decode-phase linear layer is measured against.
//
// Decode streams every weight byte once per step and is bound by HBM
// bandwidth ("Developing a custom Qwen2.5 72B inference engine from scratch
// - what is the real bottleneck?", section 6.1 "Decode GEMV: already near
// the roofline"); this kernel does nothing but those reads, so its rate is
// what a weight-streaming kernel can reach on this GPU at best.  Measurement
// only: the skinny-GEMM library neither links nor calls it.
//
// The buffer is cut into rows of `row_chunks` 16-byte chunks, of which the
// first `read_chunks` (a multiple of 64 U: whole batches) are read; reading
// less than the whole row gives a strided pattern.  A wave reads a row front
// to back in 1 KB wave loads (lane l takes chunk 64 s + l of segment s), U
// segments per batch and two batches in flight.  Rows are dealt to the
// waves in one of two orders:
//   ORDER_WAVES      wave w of the grid takes rows w, w + W, ... (every wave
//                    its own stream, all waves within a moving window),
//   ORDER_WORKGROUPS workgroup b takes rows b, b + G, ... and its waves
//                    split each row's batches between them.
// Every loaded word is XOR-folded into a value that is written out only if
// it equals a sentinel the data never produces, so no load can be dropped.
// NT: the loads carry the nontemporal hint (streamed data, not to be kept in
// the caches), as the library's weight loads do.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                 // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int ORDER_WAVES = 0;
constexpr int ORDER_WORKGROUPS = 1;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int U, int ORDER, bool NT>
__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* buf, long long rows,
                                                         int row_chunks, int read_chunks,
                                                         unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int batches = read_chunks / (64 * U);  // batches read per row
  long long first, step;
  int b0, bstep;                               // batches of a row this wave reads
  if (ORDER == ORDER_WAVES) {
    first = (long long)blockIdx.x * kWaves + wv;
    step = (long long)gridDim.x * kWaves;
    b0 = 0;
    bstep = 1;
  } else {
    first = blockIdx.x;
    step = gridDim.x;
    b0 = wv;
    bstep = kWaves;
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long long r = first; r < rows; r += step) {
    const u32x4* row = buf + r * (long long)row_chunks + lane;
    u32x4 a[U], b[U];
    int k = b0;
    if (k >= batches) continue;
#pragma unroll
    for (int v = 0; v < U; ++v) a[v] = ld<NT>(row + (k * U + v) * 64);
    for (; k + bstep < batches; k += 2 * bstep) {
#pragma unroll
      for (int v = 0; v < U; ++v) b[v] = ld<NT>(row + ((k + bstep) * U + v) * 64);
#pragma unroll
      for (int v = 0; v < U; ++v) acc ^= a[v];
      if (k + 2 * bstep < batches) {
#pragma unroll
        for (int v = 0; v < U; ++v) a[v] = ld<NT>(row + ((k + 2 * bstep) * U + v) * 64);
      }
#pragma unroll
      for (int v = 0; v < U; ++v) acc ^= b[v];
    }
    if (k < batches) {
#pragma unroll
      for (int v = 0; v < U; ++v) acc ^= a[v];
    }
  }
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

// The matrix-core kernel's access pattern: units of 16 WPB rows of
// `row_chunks` chunks, dealt round robin to the workgroups.  A wave load
// covers 512 bytes of each of two rows (lanes 0-31 one row, 32-63 the
// next), a segment 512 bytes of each of 16 rows (8 loads), one segment in
// flight ahead of the one being folded.  KSPLIT = false: wave i takes rows
// 16 i .. 16 i + 15 of the unit, all of K; KSPLIT = true: the unit is 16
// rows and wave i takes segments i, i + WPB, ... of them (the waves split K).
template <int WPB, bool KSPLIT, bool NT>
__global__ __launch_bounds__(64 * WPB) void stream_read_tiles(const u32x4* buf, long long rows,
                                                              int row_chunks, unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  constexpr int kUnitRows = KSPLIT ? 16 : 16 * WPB;
  const int segs = row_chunks / 32;            // 512-byte segments per row
  const long long units = rows / kUnitRows;
  const int lrow = lane >> 5, lchunk = lane & 31;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const long long row0 = u * kUnitRows + (KSPLIT ? 0 : 16 * wv);
    const u32x4* base = buf + (row0 + lrow) * (long long)row_chunks + lchunk;
    const int s0 = KSPLIT ? wv : 0;
    const int sstep = KSPLIT ? WPB : 1;
    if (s0 >= segs) continue;
    u32x4 a[8], b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = ld<NT>(base + 2 * q * (long long)row_chunks + s0 * 32);
    int s = s0;
    for (; s + sstep < segs; s += 2 * sstep) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        b[q] = ld<NT>(base + 2 * q * (long long)row_chunks + (s + sstep) * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= a[q];
      if (s + 2 * sstep < segs) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          a[q] = ld<NT>(base + 2 * q * (long long)row_chunks + (s + 2 * sstep) * 32);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= b[q];
    }
    if (s < segs) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= a[q];
    }
  }
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}


// The matrix-core kernel's pattern with writes added (stream_read_tiles,
// KSPLIT = false, nontemporal loads, 8 waves): at the end of every unit
// (128 rows of the whole row) each lane stores floats, as a kernel that
// writes its outputs in the middle of its weight stream does.  MODE 0 no
// stores; 1 four stores per lane, each wave writing 256 contiguous bytes per
// store; 2 one such store; 3 the four as nontemporal stores; 4 the four into
// the first 64 KB of out (a region that stays in the cache); 5 the four as
// stores the compiler's wait analysis does not see (inline asm), so they
// change none of its waits; 6 the four every fourth unit only (the bytes of
// mode 2 in rarer, larger bursts); 7 sixteen every sixteenth unit (the bytes
// of mode 1).
template <int MODE>
__global__ __launch_bounds__(512) void stream_read_tiles_writes(const u32x4* buf, long long rows,
                                                               int row_chunks, float* out,
                                                               unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  constexpr int kUnitRows = 128;
  const int segs = row_chunks / 32;
  const long long units = rows / kUnitRows;
  const int lrow = lane >> 5, lchunk = lane & 31;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const u32x4* base = buf + (u * kUnitRows + 16 * wv + lrow) * (long long)row_chunks + lchunk;
    u32x4 a[8], b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = ld<true>(base + 2 * q * (long long)row_chunks);
    int s = 0;
    for (; s + 1 < segs; s += 2) {
#pragma unroll
      for (int q = 0; q < 8; ++q) b[q] = ld<true>(base + 2 * q * (long long)row_chunks + (s + 1) * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= a[q];
      if (s + 2 < segs) {
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = ld<true>(base + 2 * q * (long long)row_chunks + (s + 2) * 32);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= b[q];
    }
    if (s < segs) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= a[q];
    }
    if (MODE == 6 && (u / gridDim.x) % 4 != 3) continue;
    if (MODE == 7 && (u / gridDim.x) % 16 != 15) continue;
    if (MODE != 0) {
      const float v = (float)(acc.x & 0xFFFF);
      constexpr int kStores = MODE == 2 ? 1 : MODE == 7 ? 16 : 4;
#pragma unroll
      for (int i = 0; i < kStores; ++i) {
        long long idx = ((u * 16 + i) * 8 + wv) * 64 + lane;
        if (MODE == 4) idx &= 16383;
        if (MODE == 3) {
          __builtin_nontemporal_store(v, out + idx);
        } else if (MODE == 5) {
          asm volatile("global_store_dword %0, %1, off" : : "v"(out + idx), "v"(v));
        } else {
          out[idx] = v;
        }
      }
    }
  }
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}
typedef void (*writes_fn)(const u32x4*, long long, int, float*, unsigned*);

typedef void (*probe_fn)(const u32x4*, long long, int, int, unsigned*);
typedef void (*tiles_fn)(const u32x4*, long long, int, unsigned*);

template <int ORDER, bool NT>
probe_fn pick(int u) {
  switch (u) {
    case 1: return stream_read<1, ORDER, NT>;
    case 2: return stream_read<2, ORDER, NT>;
    case 4: return stream_read<4, ORDER, NT>;
    case 8: return stream_read<8, ORDER, NT>;
    case 16: return stream_read<16, ORDER, NT>;
    default: return nullptr;
  }
}

template <bool NT>
probe_fn pick_order(int order, int u) {
  return order == ORDER_WAVES ? pick<ORDER_WAVES, NT>(u)
         : order == ORDER_WORKGROUPS ? pick<ORDER_WORKGROUPS, NT>(u)
                                     : nullptr;
}

constexpr int kMaxProbeThreads = 512;

}  // namespace

extern "C" {

// Reads the first read_bytes of every row_bytes of the first `bytes` of `buf`
// (16-byte aligned device memory) once: rows dealt in `order` (0 = to waves,
// 1 = to workgroups), U KB per batch, `workgroups` workgroups of 4 waves,
// nontemporal loads if `nontemporal` is nonzero.  Requirements: u in {1, 2,
// 4, 8, 16}; read_bytes a multiple of U KB and at most row_bytes; bytes a
// multiple of row_bytes; sink device memory of >= 4 * workgroups bytes
// (written only on the sentinel).  Returns 0, or -1 for invalid arguments
// (nothing enqueued), or -2 if the launch failed.
int skinny_probe_stream_read(const void* buf, long long bytes, long long row_bytes,
                             long long read_bytes, int order, int u, int workgroups,
                             int nontemporal, unsigned* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || row_bytes <= 0 || read_bytes <= 0 || workgroups < 1)
    return -1;
  if (((uintptr_t)buf & 15) != 0) return -1;
  const probe_fn fn = nontemporal ? pick_order<true>(order, u) : pick_order<false>(order, u);
  if (!fn) return -1;
  if (read_bytes % (u * 1024LL) != 0 || read_bytes > row_bytes || bytes % row_bytes != 0)
    return -1;
  if (row_bytes % 16 != 0 || row_bytes / 16 > (1LL << 30)) return -1;
  hipLaunchKernelGGL(fn, dim3(workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / row_bytes, (int)(row_bytes / 16),
                     (int)(read_bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// The matrix-core kernel's pattern (stream_read_tiles): `bytes` of buf read
// as rows of row_bytes (a multiple of 512; bytes a multiple of 16 * wpb *
// row_bytes), wpb in {4, 8} waves per workgroup, ksplit 0 or 1, nontemporal
// loads if `nontemporal` is nonzero.  Same returns and sink rule as
// skinny_probe_stream_read.
int skinny_probe_stream_read_tiles(const void* buf, long long bytes, long long row_bytes,
                                   int wpb, int ksplit, int workgroups, int nontemporal,
                                   unsigned* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || row_bytes <= 0 || workgroups < 1) return -1;
  if (((uintptr_t)buf & 15) != 0 || row_bytes % 512 != 0) return -1;
  if (bytes % (16LL * wpb * row_bytes) != 0 || row_bytes / 16 > (1LL << 30)) return -1;
  tiles_fn fn = nullptr;
  if (nontemporal) {
    if (wpb == 4) fn = ksplit ? stream_read_tiles<4, true, true> : stream_read_tiles<4, false, true>;
    if (wpb == 8) fn = ksplit ? stream_read_tiles<8, true, true> : stream_read_tiles<8, false, true>;
  } else {
    if (wpb == 4) fn = ksplit ? stream_read_tiles<4, true, false> : stream_read_tiles<4, false, false>;
    if (wpb == 8) fn = ksplit ? stream_read_tiles<8, true, false> : stream_read_tiles<8, false, false>;
  }
  if (!fn || 64 * wpb > kMaxProbeThreads) return -1;
  hipLaunchKernelGGL(fn, dim3(workgroups), dim3(64 * wpb), 0, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / row_bytes, (int)(row_bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}


// The tile pattern with writes (stream_read_tiles_writes): mode 0-7 as
// there; `workgroups` workgroups of 8 waves, each asking for lds_bytes of
// LDS (0 - 160 KB; more per workgroup means fewer per CU); out: device
// floats, out_floats >= 8192 * (bytes / row_bytes / 128) (16384 for mode 4).
// Requirements and returns as skinny_probe_stream_read_tiles; -2 also when
// the LDS size cannot be set.
int skinny_probe_tiles_writes(const void* buf, long long bytes, long long row_bytes,
                              int workgroups, int mode, int lds_bytes, float* out,
                              long long out_floats, unsigned* sink, void* stream) {
  if (!buf || !out || !sink || bytes <= 0 || row_bytes <= 0 || workgroups < 1) return -1;
  if (((uintptr_t)buf & 15) != 0 || row_bytes % 512 != 0) return -1;
  if (bytes % (128LL * row_bytes) != 0 || row_bytes / 16 > (1LL << 30)) return -1;
  if (lds_bytes < 0 || lds_bytes > 160 * 1024) return -1;
  const long long units = bytes / row_bytes / 128;
  if (out_floats < (mode == 4 ? 16384 : 8192 * units)) return -1;
  writes_fn fn = nullptr;
  switch (mode) {
    case 0: fn = stream_read_tiles_writes<0>; break;
    case 1: fn = stream_read_tiles_writes<1>; break;
    case 2: fn = stream_read_tiles_writes<2>; break;
    case 3: fn = stream_read_tiles_writes<3>; break;
    case 4: fn = stream_read_tiles_writes<4>; break;
    case 5: fn = stream_read_tiles_writes<5>; break;
    case 6: fn = stream_read_tiles_writes<6>; break;
    case 7: fn = stream_read_tiles_writes<7>; break;
    default: return -1;
  }
  if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds_bytes) != hipSuccess)
    return -2;
  hipLaunchKernelGGL(fn, dim3(workgroups), dim3(512), lds_bytes, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / row_bytes, (int)(row_bytes / 16), out, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
}  // extern "C"
