// skinny_gemm.hip - gfx950 kernels and C ABI for the decode-phase linear layer
// y[M x N] = x[M x K] . W^T, M = 1..16, bf16 or FP8-E4M3 (128 x 128 block
// scales) weights, bf16 activations and outputs, fp32 accumulation.
//
// Why the kernels look the way they do:
//   Decode streams every weight byte once per step and is bound by HBM
//   bandwidth ("Developing a custom Qwen2.5 72B inference engine from scratch
//   - what is the real bottleneck?", sections 2 and 6.1).  At skinny sizes a
//   launch of one workgroup per output tile leaves most compute units idle;
//   splitting the long K dimension lets the whole chip stream weights ("9%
//   faster GLM-5.3-Flash prefill with GPU-to-GPU IPC (and why TileLang didn't
//   help)", section "TileLang: twice as fast, and no faster").  The page
//   splits K into fixed slices per block; here a persistent grid deals the
//   work units (row group, K-chunk) of all linears in the launch round robin
//   to its workgroups, so one launch streams a whole stack with a single ramp
//   and tail, and a launch too small to fill the chip is cut into more
//   K-chunks.
//
// Two main kernels share that decomposition and the second pass:
//
//   skinny_rows  (VECTOR variant, small M): wave i of a workgroup streams
//     its rows of the row group front to back, lane l reading bytes
//     [16 l, 16 l + 16) of each 1 KB segment; x of the current K-chunk sits in
//     LDS, shared by the workgroup.  v_dot2_f32_bf16 accumulates in fp32 and
//     a 64-lane butterfly ends each row.  Measured on MI355X, one contiguous
//     stream per wave sustains ~6.3 TB/s.  Its MoE form serves one-token
//     slices, whose few chosen experts' rows its 8-row units spread over
//     more workgroups than the tile kernel's.
//
//   skinny_tiles (MFMA variant): each wave streams 16 rows in whole cache
//     lines (512 contiguous bytes per row per load), turns them around
//     through a private LDS tile into the B-operand layout of
//     v_mfma_f32_16x16x32_bf16, and reads the A operand (x, token = lane % 16)
//     from LDS.  The matrix cores make the arithmetic per weight independent
//     of M, which the vector path's is not.  Workgroups of 4 waves (two per
//     CU) or, for large FP8 launches, 8 waves with all of the CU's LDS in an
//     exact-fit layout (swizzled instead of padded) that holds x of six
//     tokens of K = 8192 whole.  Its MoE form takes the units of each chosen
//     expert's slice of routes.
//
//   x windows are copied from global memory straight into LDS (no
//   registers) while a unit's first weights load.  A linear cut into
//   K-chunks has each unit write fp32 partial sums to its own workspace
//   slot; skinny_combine adds a row's slots in chunk order.  The second pass
//   is deterministic and uses no atomics.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "skinny_gemm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;          // rows of one MFMA B operand
constexpr int kSegChunks = 64;          // 16-byte chunks per 1 KB row segment (skinny_rows)
constexpr int kCombineThreads = 256;
constexpr int kMaxWaves = 8192;         // 256 CUs x 32 resident waves
constexpr int kMaxLdsBytes = 160 * 1024;  // LDS of one CU
constexpr int kScaleBlock = 128;
constexpr int kRowsMaxKBlocks = 256;    // skinny_rows FP8: K <= 32768
// skinny_rows shape, measured on MI355X over the Qwen2.5-72B shapes: 8 waves
// per workgroup share one copy of x, 8 segments per wave in flight, up to 32
// waves per CU.
constexpr int kRowsWavesPerBlock = 8;
constexpr int kTargetRowsWavesPerCU = 32;

struct LinDesc {
  const u32x4* w;        // W rows as 16-byte chunks
  const float* scale;    // FP8 block scales (NULL for bf16)
  const u32x4* x;        // x rows as 16-byte chunks (8 bf16 each)
  __bf16* y;             // y[M][N]
  int N;
  int K;
  int cpr;               // 16-byte chunks per W row
  int spt;               // segments per W row (1 KB for skinny_rows, 512 B for skinny_tiles)
  int kblocks;           // ceil(K / 128)
  int chunks;            // K-chunks per row group (1 = not split)
  long long unit_base;   // index of this linear's first unit in the launch
  long long slot_base;   // first partial slot of a split linear
  int act;               // kActNone, or kActSwiGLU: x is [M][2K] = [gate | up], the
                         // linear's input is silu(gate) * up
  int sub;               // skinny_tiles: x windows per K-chunk, walked in turn by the
                         // unit's workgroup with its sums kept in registers
};

constexpr int kActNone = 0;
constexpr int kActSwiGLU = 1;

// Mixture-of-experts launch (skinny_tiles<DT, WPB, true>): lin[0] describes
// one expert (w, scale: expert 0; x, y: the routes' rows).  Work units are
// (slice, row group, K-chunk); a slice is up to `cap` routes of one expert,
// found on the device from the router's choices (see moe_setup).
struct MoeArgs {
  const int* ids;        // [routes] expert of route r = t * topk + j
  int* table;            // slice table copy for the second pass (NULL: unsplit)
  long long w_stride;    // 16-byte chunks of one expert's W
  long long s_stride;    // scales of one expert
  int E;
  int routes;
  int topk;
  int cap;               // routes per slice (the token count)
  int per_route;         // x holds a row per route (else a row per token)
  int max_slices;        // slices the routes can make, at most
  int units_per_slice;
  int table_lds;         // LDS offset of the slice table
};

// Greedy-token reduction ("Developing a custom Qwen2.5 72B inference engine
// from scratch - what is the real bottleneck?", section 5, third lever):
// pairs (value, index) ordered by value, then by lower index, so the result
// does not depend on the reduction order.  NaN ranks below every number,
// -inf included: a NaN is never taken, and a pair that has seen no number
// keeps the index N, which loses to every real index.
struct ArgmaxPair {
  float v;
  int i;
};

__device__ __forceinline__ void argmax_take(float v, int i, float& bv, int& bi) {
  if (v != v) return;
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

struct LaunchArgs {
  int nlin;
  int M;
  int G;                 // workgroups of the persistent grid
  int band_rows;         // rows per row group
  long long S;           // units of the launch
  float* slots;          // fp32 partial sums [slot][M][band_rows], one slot per split unit
  int x_lds_bytes;       // LDS bytes for x; the kernel's other LDS follows
  int pad;
  ArgmaxPair* pairs;     // skinny_rows, one unsplit linear: [M][G] greedy pairs, or NULL
  MoeArgs moe;
  LinDesc lin[SKINNY_MAX_LINEARS_PER_LAUNCH];
  const LinDesc* table;  // the nlin descriptors in device memory, or NULL: lin[] above
};

// The kernels read descriptors through a constant-address-space pointer, so
// every read is a scalar load (its own counter, never a wait on the weight
// stream's vector loads): the kernel arguments' own array, or for launches of
// more linears than it holds a table in the workspace, copied there ahead of
// the launch on its stream and not written while the launch runs.
typedef __attribute__((address_space(4))) const LinDesc KLinDesc;

__device__ __forceinline__ KLinDesc* launch_lins(const LaunchArgs& a) {
  return a.table ? (KLinDesc*)a.table : (KLinDesc*)a.lin;
}
// Mixture-of-experts launches describe one expert in lin[0] and never take a table.
__device__ __forceinline__ const LinDesc* moe_lins(const LaunchArgs& a) { return a.lin; }

// Weight loads are nontemporal: every weight byte is read once per call and
// never again soon, and on MI355X the streaming-read probe reads 7.2 TB/s
// with nontemporal 16-byte loads against 6.5 TB/s with plain ones (same
// patterns, 8 GiB).  x, the FP8 scales and everything shared stay plain.
__device__ __forceinline__ u32x4 ldw(const u32x4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ bf16x2 as_bf16x2(unsigned u) {
  return __builtin_bit_cast(bf16x2, u);
}

// 8 bf16 x 8 bf16 dot product into an fp32 accumulator (four v_dot2 ops).
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

// Two e4m3 bytes of v (bytes 0-1, or bytes 2-3 when HIGH) -> two bf16 in one
// dword.  Exact: every e4m3 value is also a bf16 value.
template <bool HIGH>
__device__ __forceinline__ unsigned e4m3x2_to_bf16(unsigned v) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HIGH));
}

// 16 e4m3 weights (one chunk) -> two chunks of 8 bf16, in order.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 q, u32x4& b0, u32x4& b1) {
  b0 = u32x4{e4m3x2_to_bf16<false>(q.x), e4m3x2_to_bf16<true>(q.x),
             e4m3x2_to_bf16<false>(q.y), e4m3x2_to_bf16<true>(q.y)};
  b1 = u32x4{e4m3x2_to_bf16<false>(q.z), e4m3x2_to_bf16<true>(q.z),
             e4m3x2_to_bf16<false>(q.w), e4m3x2_to_bf16<true>(q.w)};
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight gated-MLP inputs: bf16(silu(g) * u) for the bf16 pairs of g and u,
// in fp32 (silu(g) = g / (1 + e^-g)), rounded to nearest even ("Multi-GPU
// Inference and Serving at Scale", Example 3: the MLP's activation sits
// between its two linears; Qwen2.5's is the SiLU-gated unit).
__device__ __forceinline__ u32x4 swiglu8(u32x4 g, u32x4 u) {
  const bf16x8 gv = __builtin_bit_cast(bf16x8, g);
  const bf16x8 uv = __builtin_bit_cast(bf16x8, u);
  bf16x8 h;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float a = (float)gv[k];
    h[k] = (__bf16)(a / (1.0f + expf(-a)) * (float)uv[k]);
  }
  return __builtin_bit_cast(u32x4, h);
}

// x[m][xw0, xw0 + wlen) of tokens m < M into dst[m * stride + c], several
// loads in flight per thread.  With kActSwiGLU the linear's x holds [gate |
// up] per token (2 xcpr chunks) and the staged value is swiglu8(gate, up).
// GATHER: staged row m is x's row rows[m].
template <int THREADS, bool GATHER>
__device__ __forceinline__ void stage_x(const u32x4* X, int act, int M, int xcpr, int xw0,
                                        int wlen, u32x4* dst, int stride,
                                        const unsigned char* rows) {
  const int n = M * wlen;
  if (act == kActNone) {
    for (int b = threadIdx.x; b < n; b += 8 * THREADS) {
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = min(b + q * THREADS, n - 1);
        const int m = i / wlen;
        const int src = GATHER ? rows[m] : m;
        v[q] = X[(size_t)src * xcpr + xw0 + (i - m * wlen)];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = b + q * THREADS;
        const int m = i / wlen;
        if (i < n) dst[m * stride + (i - m * wlen)] = v[q];
      }
    }
  } else {
    for (int b = threadIdx.x; b < n; b += 4 * THREADS) {
      u32x4 g[4], u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = min(b + q * THREADS, n - 1);
        const int m = i / wlen;
        const int src = GATHER ? rows[m] : m;
        const u32x4* row = X + (size_t)src * 2 * xcpr + xw0 + (i - m * wlen);
        g[q] = row[0];
        u[q] = row[xcpr];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = b + q * THREADS;
        const int m = i / wlen;
        if (i < n) dst[m * stride + (i - m * wlen)] = swiglu8(g[q], u[q]);
      }
    }
  }
}

template <int THREADS, bool GATHER>
__device__ __forceinline__ void stage_x_direct(const u32x4* X, int M, int xcpr, int xw0, int wlen,
                                               u32x4* dst, int stride, const unsigned char* rows) {
  const int lane = threadIdx.x & 63;
  const int pieces = (wlen + 63) / 64;
  for (int p = threadIdx.x >> 6; p < M * pieces; p += THREADS / 64) {
    const int m = p / pieces;
    const int c0 = (p - m * pieces) * 64;
    const int src = GATHER ? rows[m] : m;
    if (c0 + lane < wlen)
      __builtin_amdgcn_global_load_lds(
          X + (size_t)src * xcpr + xw0 + c0 + lane,
          (__attribute__((address_space(3))) void*)(dst + m * stride + c0), 16, 0, 0);
  }
}

// The exact-fit form of stage_x_direct: window slot s of token m holds chunk
// s ^ (m % 8), so lane l of a 64-slot piece copies chunk c0 + (l ^ (m % 8));
// slots whose chunk lies past the window's data (wlen) are zeroed by the lane
// that owns them, so no slot is written twice.  win is a multiple of 8.
template <int THREADS>
__device__ __forceinline__ void stage_x_fit(const u32x4* X, int M, int xcpr, int xw0, int wlen,
                                            int win, u32x4* dst) {
  const int lane = threadIdx.x & 63;
  const int pieces = (win + 63) / 64;
  for (int p = threadIdx.x >> 6; p < M * pieces; p += THREADS / 64) {
    const int m = p / pieces;
    const int c0 = (p - m * pieces) * 64;
    const int c = c0 + (lane ^ (m & 7));
    if (c0 + lane < win) {
      if (c < wlen)
        __builtin_amdgcn_global_load_lds(
            X + (size_t)m * xcpr + xw0 + c,
            (__attribute__((address_space(3))) void*)(dst + m * win + c0), 16, 0, 0);
      else
        dst[m * win + c0 + lane] = zero4();
    }
  }
}

// ---------------------------------------------------------------------------
// Mixture-of-experts slices.  A router sends token t to topk experts; route r
// = t * topk + j goes to expert ids[r] ("Multi-GPU Inference and Serving at
// Scale", Example 8).  The routes of one expert share its weights, so the
// launch streams each chosen expert's W once for all of its routes: slice s
// is up to `cap` routes of one expert, slices ordered by expert, routes by
// index.  Every workgroup derives the same table from ids at its start (one
// thread per route, two passes over the routes in LDS), so the routing needs
// neither a host round trip nor a launch of its own.  Routes whose expert is
// outside [0, E) belong to no slice; their y rows are zeroed.
constexpr int kMoeMaxRoutes = 256;
constexpr int kMoeMlpMaxRoutes = 16;      // routes of the one-token fused MLP (top-k)
constexpr int kMoeMaxCap = 16;

struct MoeTable {
  int* head;             // [2]: slices, invalid routes
  int* expert;           // [max_slices]
  int* rows;             // [max_slices] routes in the slice
  unsigned char* yrow;   // [max_slices][16] route of slice row m (= its y row)
  unsigned char* xrow;   // [max_slices][16] x row of slice row m
  unsigned char* inv;    // [routes] routes with no expert
};

__device__ __forceinline__ MoeTable moe_table(unsigned char* base, int max_slices) {
  MoeTable t;
  t.head = reinterpret_cast<int*>(base);
  t.expert = t.head + 2;
  t.rows = t.expert + max_slices;
  t.yrow = reinterpret_cast<unsigned char*>(t.rows + max_slices);
  t.xrow = t.yrow + max_slices * kMoeMaxCap;
  t.inv = t.xrow + max_slices * kMoeMaxCap;
  return t;
}

// Builds the table in LDS (scratch: 2 x kMoeMaxRoutes ints, free until the
// caller's next barrier).  Needs THREADS >= routes.
template <int THREADS>
__device__ void moe_setup(const MoeArgs& mo, const MoeTable& tb, int* scratch) {
  static_assert(THREADS >= kMoeMaxRoutes, "one thread per route");
  int* ids = scratch;
  int* head = scratch + kMoeMaxRoutes;
  const int r = threadIdx.x;
  int e = -1;
  if (r < mo.routes) {
    const int v = mo.ids[r];
    e = v >= 0 && v < mo.E ? v : -1;
    ids[r] = e;
  }
  __syncthreads();
  int rank = 0, count = 0, inv_rank = 0;
  if (r < mo.routes) {
    for (int q = 0; q < mo.routes; ++q) {
      const int f = ids[q];
      count += f == e;
      rank += f == e && q < r;
      inv_rank += f < 0 && q < r;
    }
    head[r] = e >= 0 && rank % mo.cap == 0;        // first route of a slice
  }
  __syncthreads();
  if (r < mo.routes) {
    int before = 0, slices = 0, invalid = 0;
    for (int q = 0; q < mo.routes; ++q) {
      const int h = head[q];
      const int f = ids[q];
      before += h && f < e;                        // slices of lower experts
      slices += h;
      invalid += f < 0;
    }
    if (e >= 0) {
      const int sl = before + rank / mo.cap;
      const int m = rank % mo.cap;
      if (sl < mo.max_slices) {
        tb.yrow[sl * kMoeMaxCap + m] = (unsigned char)r;
        tb.xrow[sl * kMoeMaxCap + m] = (unsigned char)(mo.per_route ? r : r / mo.topk);
        if (m == 0) {
          tb.expert[sl] = e;
          tb.rows[sl] = min(mo.cap, count - rank);
        }
      }
    } else {
      tb.inv[inv_rank] = (unsigned char)r;
    }
    if (r == 0) {
      tb.head[0] = min(slices, mo.max_slices);
      tb.head[1] = invalid;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// skinny_rows: a workgroup of WPB waves streams row groups of WPB x R rows;
// wave i takes the R adjacent rows starting at row (WPB g + i) R.  Lanes run
// along K: lane l reads bytes [16 l, 16 l + 16) of each 1 KB segment of a
// row, so each wave reads its rows front to back in 1 KB coalesced loads, U
// segments per batch and two batches in flight.  Work units (row group,
// K-chunk) are dealt round robin: workgroup b takes units b, b + G, ..., so
// at any moment all workgroups read neighbouring rows - measured on MI355X
// this compact moving window streams faster than giving each workgroup its
// own contiguous share.  As in skinny_tiles, units are row-group-major and
// the chunk count divides the grid, so a workgroup keeps one K-chunk per
// linear.  LDS holds x[M][window] of the current (linear, chunk), restaged
// between two barriers when it changes, and per wave the FP8 scale row of
// the current 128-row block, prefetched one unit ahead.  One x read from LDS
// serves the wave's R rows.
template <int DT, int R, int U>
struct RowBatch {
  u32x4 w[U][R];
};

// The bf16 M <= 2 instances keep 16 waves per CU (<= 128 VGPRs); the others
// have the registers they need.
//
// MoE form (MOE): lin[0] describes one expert as in skinny_tiles; units are
// (slice, row group) with the K dimension unsplit, and a slice's x rows are
// gathered into LDS by the slice table, which sits at a.moe.table_lds inside
// the x budget.
template <int DT, int MT, int U, int R, int WPB, bool MOE = false>
__global__ __launch_bounds__(64 * WPB)
__attribute__((amdgpu_waves_per_eu((DT == SKINNY_BF16 && MT <= 2) ? 4 : 1))) void skinny_rows(
    const LaunchArgs a) {
  const auto lins = [&] {
    if constexpr (MOE) return moe_lins(a); else return launch_lins(a);
  }();
  constexpr int kThreads = 64 * WPB;
  constexpr int kGroupRows = WPB * R;
  constexpr int XC = DT == SKINNY_BF16 ? 1 : 2;        // x chunks per W chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  float* ss = reinterpret_cast<float*>(lds + a.x_lds_bytes) + wv * kRowsMaxKBlocks;
  float spre[kRowsMaxKBlocks / 64];
  long long S = a.S;
  MoeTable tb{};
  if constexpr (MOE) {
    // The slice table (built in the x region, free until the first staging),
    // then this workgroup's share of the zero rows.
    const MoeArgs& mo = a.moe;
    const auto& L = lins[0];
    tb = moe_table(lds + mo.table_lds, mo.max_slices);
    moe_setup<kThreads>(mo, tb, reinterpret_cast<int*>(lds));
    const long long zeros = (long long)tb.head[1] * L.N;
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < zeros;
         i += (long long)a.G * kThreads) {
      const int q = (int)(i / L.N);
      L.y[(size_t)tb.inv[q] * L.N + (i - (long long)q * L.N)] = (__bf16)0.0f;
    }
    S = (long long)tb.head[0] * mo.units_per_slice;
  }
  // MoE: l is the unit's slice and e its expert; the linear is lin[0].
  auto unit_of = [&](long long u, int& l, int& grp, int& chunk, int& e) {
    long long local;
    if constexpr (MOE) {
      l = (int)(u / a.moe.units_per_slice);
      local = u - (long long)l * a.moe.units_per_slice;
      e = __builtin_amdgcn_readfirstlane(tb.expert[l]);
    } else {
      while (l + 1 < a.nlin && lins[l + 1].unit_base <= u) ++l;
      local = u - lins[l].unit_base;
      e = 0;
    }
    const auto& L = lins[MOE ? 0 : l];
    grp = (int)(local / L.chunks);
    chunk = (int)(local - (long long)grp * L.chunks);
  };
  auto prefetch_scales = [&](long long u, int l) {
    if (DT == SKINNY_FP8_BS128 && u < S) {
      int grp, chunk, e;
      unit_of(u, l, grp, chunk, e);
      const auto& L = lins[MOE ? 0 : l];
      // The row group lies in one 128-row scale block (kGroupRows divides 128).
      const float* scale = MOE ? L.scale + (size_t)e * a.moe.s_stride : L.scale;
      const float* src = scale + (size_t)((grp * kGroupRows) / kScaleBlock) * L.kblocks;
#pragma unroll
      for (int i = 0; i < kRowsMaxKBlocks / 64; ++i) {
        const int k = 64 * i + lane;
        spre[i] = k < L.kblocks ? src[k] : 0.0f;
      }
    }
  };
  auto store_scales = [&]() {
    if (DT == SKINNY_FP8_BS128) {
#pragma unroll
      for (int i = 0; i < kRowsMaxKBlocks / 64; ++i) ss[64 * i + lane] = spre[i];
    }
  };
  int l = 0;
  int staged_l = -1;
  int staged_c = -1;
  long long u = blockIdx.x;
  // Greedy token of the rows this wave writes (a.pairs: one unsplit linear):
  // the best bf16 output per token, kept by lane 0.
  float gbv[MT];
  int gbi[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    gbv[m] = -__builtin_inff();
    gbi[m] = lins[0].N;
  }
  prefetch_scales(u, 0);
  store_scales();
  for (; u < S; u += a.G) {
    int grp, chunk, e;
    unit_of(u, l, grp, chunk, e);
    const auto& L = lins[MOE ? 0 : l];
    const int mt = MOE ? __builtin_amdgcn_readfirstlane(tb.rows[l]) : MT;   // tokens of the unit
    // Chunk c holds segments [c spt / chunks, (c + 1) spt / chunks).
    const int spc = (L.spt + L.chunks - 1) / L.chunks;          // window, in segments
    const int j0 = (int)((long long)chunk * L.spt / L.chunks);
    const int j1 = (int)((long long)(chunk + 1) * L.spt / L.chunks);
    const int xcpr = L.K >> 3;                                   // x chunks per token row
    const int win = spc * kSegChunks * XC;                       // x chunks per token in LDS
    const int xw0 = j0 * kSegChunks * XC;                        // first x chunk of the window
    const int row0 = grp * kGroupRows + wv * R;
    // Rows past N read row N - 1 instead; their sums are not written.
    const u32x4* w = MOE ? L.w + (size_t)e * a.moe.w_stride : L.w;
    const u32x4* wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wrow[r] = w + (size_t)min(row0 + r, L.N - 1) * (size_t)L.cpr;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
    // A batch of U whole segments: plain loads (no selects, so the compiler
    // keeps them unconditional and the waits exact) ...
    auto load = [&](RowBatch<DT, R, U>& b, int j) {
#pragma unroll
      for (int v = 0; v < U; ++v)
#pragma unroll
        for (int r = 0; r < R; ++r) b.w[v][r] = ldw(wrow[r] + (j + v) * kSegChunks + lane);
      __builtin_amdgcn_sched_barrier(0);
    };
    // ... and its products.  OK marks the chunks inside the row (a ragged end).
    auto consume = [&](const RowBatch<DT, R, U>& b, int j, auto masked) {
      constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int cw = (j + v) * kSegChunks + lane;
        const bool ok = !kMasked || ((j + v < j1) && cw < L.cpr);
        const int xl = cw * XC - xw0;                            // chunk index in the window
        if (DT == SKINNY_BF16) {
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 xv = ok ? xs[m * win + xl] : zero4();
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = dot8(xv, b.w[v][r], acc[r][m]);
          }
        } else {
          // W chunk cw holds k in [16 cw, 16 cw + 16): scale block cw / 8.
          const float sc = ok ? ss[cw >> 3] : 0.0f;
          u32x4 b0[R], b1[R];
#pragma unroll
          for (int r = 0; r < R; ++r) e4m3x16_to_bf16(b.w[v][r], b0[r], b1[r]);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 x0 = ok ? xs[m * win + xl] : zero4();
            const u32x4 x1 = ok ? xs[m * win + xl + 1] : zero4();
#pragma unroll
            for (int r = 0; r < R; ++r)
              acc[r][m] = __builtin_fmaf(sc, dot8(x1, b1[r], dot8(x0, b0[r], 0.0f)), acc[r][m]);
          }
        }
      }
    };
    using Plain = std::false_type;
    using Masked = std::true_type;
    // Whole batches [j0, jb) run two deep; the rest of the chunk (a short
    // batch or the row's ragged end) takes the masked path.  The first
    // batch's loads go out before x is staged, so the two fetches overlap.
    const int jf = (j1 == L.spt && L.cpr % kSegChunks != 0) ? j1 - 1 : j1;   // whole segments
    const int nb = (jf - j0) / U;
    const int jb = j0 + nb * U;
    RowBatch<DT, R, U> b0, b1;
    if (nb > 0) load(b0, j0);
    if (l != staged_l || chunk != staged_c) {                    // same for all waves
      __syncthreads();                                           // all done with the old window
      // MoE: the slice's rows of x (rows past mt keep stale values; their
      // sums are not written).
      const unsigned char* rows = MOE ? tb.xrow + l * kMoeMaxCap : nullptr;
      if (L.act == kActNone) {
        // Straight into LDS, no registers; the wait also covers the batch.
        stage_x_direct<kThreads, MOE>(L.x, mt, xcpr, xw0, min(win, xcpr - xw0), xs, win, rows);
        __builtin_amdgcn_s_waitcnt(0);
      } else {
        stage_x<kThreads, MOE>(L.x, L.act, mt, xcpr, xw0, min(win, xcpr - xw0), xs, win, rows);
      }
      __syncthreads();
      staged_l = l;
      staged_c = chunk;
    }
    prefetch_scales(u + a.G, l);
    if (nb > 0) {
      int b = 0;
      for (; b + 2 < nb; b += 2) {
        load(b1, j0 + (b + 1) * U);
        consume(b0, j0 + b * U, Plain{});
        load(b0, j0 + (b + 2) * U);
        consume(b1, j0 + (b + 1) * U, Plain{});
      }
      if (b + 2 == nb) {
        load(b1, j0 + (b + 1) * U);
        consume(b0, j0 + b * U, Plain{});
        consume(b1, j0 + (b + 1) * U, Plain{});
      } else {
        consume(b0, j0 + b * U, Plain{});
      }
    }
    for (int j = jb; j < j1; j += U) {
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int cw = (j + v) * kSegChunks + lane;
        const bool ok = (j + v < j1) && cw < L.cpr;
#pragma unroll
        for (int r = 0; r < R; ++r) b1.w[v][r] = ok ? ldw(wrow[r] + (ok ? cw : 0)) : zero4();
      }
      consume(b1, j, Masked{});
    }
    // This wave's reads of the current scales are done: install the next unit's.
    store_scales();
    // 64-lane butterflies; lane 0's sums have a fixed order.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[r][m] += __shfl_xor(acc[r][m], off);
    if (lane == 0) {
      const long long slot = L.slot_base + (long long)grp * L.chunks + chunk;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if constexpr (MOE) {                                   // unsplit: chunks == 1
            if (m < mt && row0 + r < L.N)
              L.y[(size_t)tb.yrow[l * kMoeMaxCap + m] * L.N + row0 + r] = (__bf16)acc[r][m];
          } else if (L.chunks == 1) {
            if (row0 + r < L.N) {
              const __bf16 yv = (__bf16)acc[r][m];
              L.y[(size_t)m * L.N + row0 + r] = yv;
              if (a.pairs) argmax_take((float)yv, row0 + r, gbv[m], gbi[m]);
            }
          } else {
            a.slots[((size_t)slot * MT + m) * kGroupRows + wv * R + r] = acc[r][m];
          }
        }
    }
  }
  if (!MOE && a.pairs) {
    // The workgroup's pair per token, from its waves' in wave order (the
    // order does not change the result), into pairs[m][workgroup].
    __syncthreads();                                             // every wave is done with x
    ArgmaxPair* red = reinterpret_cast<ArgmaxPair*>(lds);
    if (lane == 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wv * MT + m] = ArgmaxPair{gbv[m], gbi[m]};
    __syncthreads();
    if (threadIdx.x < MT) {
      const int m = threadIdx.x;
      float bv = -__builtin_inff();
      int bi = lins[0].N;
      for (int w = 0; w < WPB; ++w) argmax_take(red[w * MT + m].v, red[w * MT + m].i, bv, bi);
      a.pairs[(size_t)m * a.G + blockIdx.x] = ArgmaxPair{bv, bi};
    }
  }
}

// ---------------------------------------------------------------------------
// skinny_rows_flat: the row kernel for MT = 1-4 tokens with every wave's
// loads running as one stream across its units.  In skinny_rows a wave's
// pipeline fills at the start of each unit and drains at its end, so a short
// row (8 KB of FP8 at K = 8192) leaves the wave with little in flight for a
// good part of its time; here the wave keeps P slots of U 1 KB row segments
// in flight and, near the end of a unit, the loads already reach into its
// next unit (the next row group of the same or a later linear).  An FP8 scale
// travels with each load (the lane's 16 weights lie in one 128 x 128 block),
// so no scale row has to be staged between units.  Units are (row group of 8
// rows, whole K), dealt round robin as in skinny_rows; wave i takes row
// 8 g + i.  x of the current linear sits whole in LDS and is restaged between
// two barriers when the consumed unit moves to the next linear (all waves of
// a workgroup walk the same units, so they meet there).
//
// Every load is issued unconditionally, so the waits between a load and its
// products stay exact: loads past a ragged row end re-read the row's last
// chunk (those lanes do not add their products) and loads past the last unit
// re-read its last segment (never consumed).  Outputs are collected in LDS
// and written when x is restaged, when the buffer is full and at the end:
// loads and stores may complete out of order with each other, so a store in
// flight among the loads would turn the next wait into a full drain.  A wave
// keeps one sum per token; the per-lane arithmetic is that of skinny_rows,
// and the lane sum has its own fixed order (wave_sum_rows).
constexpr int kFlatYBytes = 16 * 1024;  // LDS for outputs waiting to be written

// Sum over the 64 lanes in a fixed order, without a round trip through LDS:
// each 16-lane row folds itself with rotations (DPP), then the four row sums
// are read out and added as (r0 + r1) + (r2 + r3).  The result is in every
// lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_rows(float v) {
  v += dpp_f32<0x128>(v);                              // row_ror:8
  v += dpp_f32<0x124>(v);                              // row_ror:4
  v += dpp_f32<0x122>(v);                              // row_ror:2
  v += dpp_f32<0x121>(v);                              // row_ror:1
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

template <int U>
struct FlatSlot {
  u32x4 w[U];            // 16 weight bytes of lane l in each of U segments of the row
  float s[U];            // FP8: their block scales
};

template <int DT, int MT, int P, int U>
__global__ __launch_bounds__(64 * kRowsWavesPerBlock) void skinny_rows_flat(const LaunchArgs a) {
  const auto lins = launch_lins(a);
  constexpr int WPB = kRowsWavesPerBlock;
  constexpr int kThreads = 64 * WPB;
  constexpr bool kFp8 = DT == SKINNY_FP8_BS128;
  constexpr int kYUnits = kFlatYBytes / (MT * WPB * 2);         // units whose outputs ybuf holds
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);                  // [token][K / 8]
  __bf16* ybuf = reinterpret_cast<__bf16*>(lds + a.x_lds_bytes);   // [unit][token][wave]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long S = a.S;
  if ((long long)blockIdx.x >= S) {
    if (a.pairs && threadIdx.x < MT)
      a.pairs[(size_t)threadIdx.x * a.G + blockIdx.x] = ArgmaxPair{-__builtin_inff(), lins[0].N};
    return;
  }
  auto linear_of = [&](long long u, int l) {
    while (l + 1 < a.nlin && lins[l + 1].unit_base <= u) ++l;
    return l;
  };
  // Load cursor: unit lu of linear ll, next segment lj of the wave's row.
  long long lu = blockIdx.x;
  int ll = linear_of(lu, 0);
  int lj = 0;
  const u32x4* lw = nullptr;
  const float* ls = nullptr;
  int lspt = 0, lcpr = 0;
  auto enter_load = [&]() {
    const auto& L = lins[ll];
    const int row = min((int)(lu - L.unit_base) * WPB + wv, L.N - 1);
    lw = L.w + (size_t)row * L.cpr;
    if (kFp8) ls = L.scale + (size_t)(row / kScaleBlock) * L.kblocks;
    lspt = (L.spt + U - 1) / U;
    lcpr = L.cpr;
  };
  auto load_next = [&](FlatSlot<U>& q) {
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const int c = min((lj * U + v) * kSegChunks + lane, lcpr - 1);
      q.w[v] = ldw(lw + c);
      if (kFp8) q.s[v] = ls[c >> 3];              // chunk c: k in [16 c, 16 c + 16)
    }
    if (++lj == lspt) {
      if (lu + a.G < S) {
        lu += a.G;
        ll = linear_of(lu, ll);
        enter_load();
        lj = 0;
      } else {
        lj = lspt - 1;
      }
    }
  };
  // Consume cursor: unit cu of linear cl, segment cj; rows of cfull whole
  // segments end with a ragged one; x has cxs chunks per token.  The outputs
  // of the units yfirst, yfirst + G, ... (ny of them) wait in ybuf.
  long long cu = blockIdx.x;
  int cl = ll;
  int cj = 0, crow = 0, cspt = 0, ccpr = 0, cfull = 0, cxs = 0;
  long long yfirst = cu;
  int ny = 0;
  float acc[MT];
  float gbv[MT];
  int gbi[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc[m] = 0.0f;
    gbv[m] = -__builtin_inff();
    gbi[m] = lins[0].N;
  }
  auto enter_consume = [&]() {
    const auto& L = lins[cl];
    crow = (int)(cu - L.unit_base) * WPB + wv;
    cspt = (L.spt + U - 1) / U;
    ccpr = L.cpr;
    cfull = L.cpr / (U * kSegChunks);
    cxs = L.K >> 3;
  };
  // Writes the buffered outputs of linear cl (after a barrier: every wave's
  // entries are in).  The caller waits for the stores and barriers again
  // before ybuf is reused.
  auto flush_y = [&]() {
    __syncthreads();
    const auto& L = lins[cl];
    const bool vec = (reinterpret_cast<size_t>(L.y) & 15) == 0 && L.N % 8 == 0;
    for (int i = threadIdx.x; i < ny * MT; i += kThreads) {
      const int t = i / MT, m = i - t * MT;
      const int row0 = (int)(yfirst + (long long)t * a.G - L.unit_base) * WPB;
      const __bf16* src = ybuf + i * WPB;
      __bf16* dst = L.y + (size_t)m * L.N + row0;
      if (vec && row0 + WPB <= L.N) {
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      } else {
        for (int e = 0; e < WPB && row0 + e < L.N; ++e) dst[e] = src[e];
      }
    }
    ny = 0;
  };
  auto stage = [&]() {
    __syncthreads();                                       // all done with the old x
    const auto& L = lins[cl];
    const int xcpr = L.K >> 3;
    stage_x_direct<kThreads, false>(L.x, MT, xcpr, 0, xcpr, xs, xcpr, nullptr);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Products of one slot; true when the wave has no unit left.
  auto consume = [&](const FlatSlot<U>& q) -> bool {
    if (cj < cfull) {
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int c = (cj * U + v) * kSegChunks + lane;
        if (kFp8) {
          u32x4 b0, b1;
          e4m3x16_to_bf16(q.w[v], b0, b1);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4* x = xs + m * cxs;
            acc[m] = __builtin_fmaf(q.s[v], dot8(x[2 * c + 1], b1, dot8(x[2 * c], b0, 0.0f)),
                                    acc[m]);
          }
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[m] = dot8(xs[m * cxs + c], q.w[v], acc[m]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int c = (cj * U + v) * kSegChunks + lane;
        const bool ok = c < ccpr;
        const int cx = ok ? c : 0;
        if (kFp8) {
          u32x4 b0, b1;
          e4m3x16_to_bf16(q.w[v], b0, b1);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4* x = xs + m * cxs;
            const float t =
                __builtin_fmaf(q.s[v], dot8(x[2 * cx + 1], b1, dot8(x[2 * cx], b0, 0.0f)), acc[m]);
            acc[m] = ok ? t : acc[m];
          }
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float t = dot8(xs[m * cxs + cx], q.w[v], acc[m]);
            acc[m] = ok ? t : acc[m];
          }
        }
      }
    }
    if (++cj < cspt) return false;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[m] = wave_sum_rows(acc[m]);
      if (lane == 0) {
        const __bf16 yv = (__bf16)acc[m];
        ybuf[(ny * MT + m) * WPB + wv] = yv;
        if (a.pairs && crow < lins[cl].N) argmax_take((float)yv, crow, gbv[m], gbi[m]);
      }
      acc[m] = 0.0f;
    }
    cj = 0;
    ++ny;
    if (cu + a.G >= S) return true;
    cu += a.G;
    const int nl = linear_of(cu, cl);
    if (nl != cl) {
      flush_y();                                           // stage() waits and barriers
      cl = nl;
      yfirst = cu;
      enter_consume();
      stage();
    } else {
      if (ny == kYUnits) {
        flush_y();
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        yfirst = cu;
      }
      enter_consume();
    }
    return false;
  };
  FlatSlot<U> q[P];
  enter_load();
  enter_consume();
  {
    // The first x goes out ahead of the first P - 1 slots, so one wait that
    // leaves those slots' loads in flight (loads complete in issue order)
    // covers it: the start does not drain the stream.
    const auto& L = lins[cl];
    const int xcpr = L.K >> 3;
    stage_x_direct<kThreads, false>(L.x, MT, xcpr, 0, xcpr, xs, xcpr, nullptr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < P - 1; ++s) load_next(q[s]);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kSlotLoads = (P - 1) * U * (kFp8 ? 2 : 1);
    static_assert(kSlotLoads < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((kSlotLoads & 0xF) | ((kSlotLoads >> 4) << 14) | 0x3F70);
    // A plain barrier: the compiler would put a wait for every outstanding
    // load in front of __syncthreads() here (the x copies write LDS), which
    // the wait above already covers for x.
    asm volatile("s_barrier" ::: "memory");
  }
  // P steps per pass: load the slot consumed last, consume the oldest.  Every
  // pass issues the same loads in the same order, the last one included (a
  // finished wave only skips its products), so each wait counts exactly the
  // loads that may still be in flight.
  bool done = false;
  for (;;) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      load_next(q[(s + P - 1) % P]);
      if (!done) done = consume(q[s]);
    }
    if (done) break;
  }
  flush_y();
  if (a.pairs) {
    // The workgroup's pair per token, from its waves' (in wave order; the
    // order does not change the result), into pairs[m][workgroup].
    __syncthreads();
    ArgmaxPair* red = reinterpret_cast<ArgmaxPair*>(ybuf);
    if (lane == 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wv * MT + m] = ArgmaxPair{gbv[m], gbi[m]};
    __syncthreads();
    if (threadIdx.x < MT) {
      const int m = threadIdx.x;
      float bv = -__builtin_inff();
      int bi = lins[0].N;
      for (int w = 0; w < WPB; ++w) argmax_take(red[w * MT + m].v, red[w * MT + m].i, bv, bi);
      a.pairs[(size_t)m * a.G + blockIdx.x] = ArgmaxPair{bv, bi};
    }
  }
}

// ---------------------------------------------------------------------------
// skinny_tiles: matrix cores fed by rows streamed front to back.
//
// The MFMA B operand wants lane l to hold 16 bytes of W row (l % 16), so
// loading it straight from HBM gives 64-byte pieces of 16 rows per wave
// instruction: half cache lines, measured on MI355X to stream at most
// ~5.8 TB/s.  Here every global load covers whole lines of two rows (lanes
// 0-31 one row, 32-63 the next, 512 contiguous bytes each) and each wave
// turns its 16 rows around through a private LDS tile, skewed by 16 bytes
// per row so the operand reads hit 16 different bank groups.
//
// A workgroup of WPB waves handles a row group of 16 WPB rows (inside one
// 128-row FP8 scale block); wave i owns the 16 rows from 16 i.  Work units
// (row group, K-chunk) are dealt round robin over the workgroups as in
// skinny_rows, with x[M][window] of the current (linear, K-chunk) in LDS
// (token rows padded by one chunk, then a zero row for absent tokens).  A
// segment is 512 bytes of each of the wave's rows: 8 loads, 8 LDS writes,
// then 8 k-steps of one operand read each; bf16 needs one MFMA per k-step,
// FP8 two (its 16-byte chunk holds 16 k) and the block scale is applied in
// fp32 to each 128-k partial sum.  Loads run one segment ahead of the
// products, across unit boundaries too: the last segment of a unit is
// consumed after the next unit's first loads are out, so the stream never
// drains between units and the x staging hides under those loads.
//
// Shape measured on MI355X over the Qwen2.5-72B shapes (TP=1 layers and the
// TP=8 layer, M = 1..16): 512-byte segments beat 256- and 1024-byte ones, and
// 4 waves per workgroup, two workgroups per CU, beat 8-wave workgroups on a
// single layer; large FP8 launches take the 8-wave shape (tiles_large).
constexpr int kSegBytesT = 512;                       // bytes of one row per segment
constexpr int kSegChunksT = kSegBytesT / 16;          // chunks
constexpr int kRowStrideT = kSegBytesT + 16;          // LDS bytes per staged row
constexpr int kLoadsT = kTileRows * kSegChunksT / 64; // wave loads per segment
constexpr int kLanesPerRowT = kSegChunksT;            // lanes of a load on one row
constexpr int kRowsPerLoadT = 64 / kLanesPerRowT;
constexpr int kStepsT = kSegChunksT / 4;              // k-steps per segment
constexpr int kSegBlocksT = kSegBytesT / kScaleBlock; // FP8 scale blocks per segment
// Two workgroup shapes: 4 waves with 80 KB of LDS (two per CU) or 8 waves
// with all 160 KB (one per CU, twice the x window).
constexpr int kTilesWavesSmall = 4;
constexpr int kTilesWavesLarge = 8;
constexpr int tiles_lds(int wpb) { return wpb == kTilesWavesLarge ? 160 * 1024 : 80 * 1024; }
constexpr int tiles_w_bytes(int wpb) { return wpb * kTileRows * kRowStrideT; }
constexpr int tiles_x_budget(int wpb) { return tiles_lds(wpb) - tiles_w_bytes(wpb); }
constexpr int kTilesXBudget = tiles_x_budget(kTilesWavesSmall);
// Exact-fit layout (FIT): W tiles of 512-byte rows and x rows without the pad
// chunk or the zero row, both XOR-swizzled in 16-byte slots instead of padded
// (slot c of W tile row r at c ^ (r % 16), chunk c of x token m at c ^ (m % 8),
// so the operand reads still hit distinct bank groups), and absent tokens
// read token 0 (their outputs are never written).  The 8-wave workgroup then
// holds x of six tokens of K = 8192 whole: 6 x 16 KB + 8 x 8 KB is all of the
// CU's 160 KB of LDS.
constexpr int tiles_w_bytes_fit(int wpb) { return wpb * kTileRows * kSegBytesT; }
constexpr int tiles_x_budget_fit(int wpb) { return tiles_lds(wpb) - tiles_w_bytes_fit(wpb); }
// The K-split form keeps its waves' partial tiles, two halves of WPB x 64
// lanes x 16 bytes, between the W tiles and the end of its LDS.
constexpr int tiles_red_bytes(int wpb) { return 2 * wpb * 64 * 16; }
constexpr int tiles_x_budget_ks(int wpb) { return tiles_x_budget(wpb) - tiles_red_bytes(wpb); }

template <int DT>
struct TileSeg {
  u32x4 w[kLoadsT];
  float sc;              // FP8: lane i holds the scale of the segment's block i % kSegBlocksT
};

// One work unit as every wave of the workgroup sees it (uniform values).
struct TileUnit {
  int l;                 // linear
  int grp;               // row group
  int chunk;             // K-chunk
  int sub;               // x window of the chunk
  int j0, j1;            // segments [j0, j1) of each row
  int spc;               // x window, in segments
  int slice;             // MoE: slice (else the linear)
  int e;                 // MoE: expert
  int m;                 // tokens (MoE: routes of the slice)
};

// KS (K split inside the workgroup): a unit is one 16-row tile, and the
// workgroup's waves take its segments round robin (wave i: segments j0 + i,
// j0 + i + WPB, ...), so every wave of the workgroup loads at once even
// where a row has only a few segments.  A window may then hold no segment
// for some waves.  The waves' partial tiles are added in LDS in wave order
// at the end of the unit (deterministic).
template <int DT, int WPB, bool MOE, bool KS = false, bool FIT = false>
__global__ __launch_bounds__(64 * WPB) void skinny_tiles(const LaunchArgs a) {
  static_assert(!FIT || (!MOE && !KS), "the exact-fit layout is for dense launches");
  const auto lins = [&] {
    if constexpr (MOE) return moe_lins(a); else return launch_lins(a);
  }();
  constexpr int kStride = FIT ? kSegBytesT : kRowStrideT;   // W tile bytes per row
  constexpr int kThreads = 64 * WPB;
  constexpr int kGroupRows = KS ? kTileRows : kTileRows * WPB;
  constexpr int kSegStep = KS ? WPB : 1;               // between a wave's segments
  constexpr int XC = DT == SKINNY_BF16 ? 1 : 2;        // x chunks per W chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int seg_off = KS ? wv : 0;                     // this wave's first segment of a window
  const int wrow = KS ? 0 : wv * kTileRows;            // this wave's first row of the group
  unsigned char* wt = lds + a.x_lds_bytes + wv * (kTileRows * kStride);
  // KS: partial tiles [2][WPB][64 lanes], alternate halves on alternate units.
  f32x4* red = reinterpret_cast<f32x4*>(lds + a.x_lds_bytes + WPB * kTileRows * kStride);
  // W tile slot of chunk c in tile row r (FIT: swizzled).
  auto wslot = [](int c, int r) { return FIT ? (c ^ (r & 15)) : c; };
  int red_half = 0;
  const int n = lane & 15;                             // operand row: token (A) / W row (B)
  const int g = lane >> 4;                             // operand k-group
  const int lrow = lane / kLanesPerRowT;               // load q: row q kRowsPerLoadT + lrow
  const int lchunk = lane % kLanesPerRowT;             // load: chunk of the segment

  long long S = a.S;
  MoeTable tb{};
  if constexpr (MOE) {
    // The slice table, then this workgroup's share of the zero rows; the
    // first workgroup also leaves the table for the second pass.
    const MoeArgs& mo = a.moe;
    const auto& L = lins[0];
    tb = moe_table(lds + mo.table_lds, mo.max_slices);
    moe_setup<kThreads>(mo, tb, reinterpret_cast<int*>(lds + a.x_lds_bytes));
    const int slices = tb.head[0];
    if (blockIdx.x == 0 && mo.table) {
      for (int i = threadIdx.x; i < slices; i += kThreads) mo.table[1 + i] = tb.rows[i];
      for (int i = threadIdx.x; i < slices * kMoeMaxCap; i += kThreads)
        mo.table[1 + mo.max_slices + i] = tb.yrow[i];
      if (threadIdx.x == 0) mo.table[0] = slices;
    }
    const long long zeros = (long long)tb.head[1] * L.N;
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < zeros;
         i += (long long)a.G * kThreads) {
      const int q = (int)(i / L.N);
      L.y[(size_t)tb.inv[q] * L.N + (i - (long long)q * L.N)] = (__bf16)0.0f;
    }
    S = (long long)slices * mo.units_per_slice;
  }

  // Units are row-group-major: with the chunk count dividing the grid,
  // workgroup b keeps K-chunk (b - base) % chunks all linear long.
  // Chunk c holds segments [c spt / chunks, (c + 1) spt / chunks): none is
  // empty (chunks <= spt) and none is longer than the window.
  int ldec = 0;
  auto decode = [&](long long u, int sub) {
    TileUnit t;
    long long local;
    if constexpr (MOE) {
      const int sl = (int)(u / a.moe.units_per_slice);
      local = u - (long long)sl * a.moe.units_per_slice;
      t.l = 0;
      t.slice = sl;
      t.e = __builtin_amdgcn_readfirstlane(tb.expert[sl]);
      t.m = __builtin_amdgcn_readfirstlane(tb.rows[sl]);
    } else {
      while (ldec + 1 < a.nlin && lins[ldec + 1].unit_base <= u) ++ldec;
      local = u - lins[ldec].unit_base;
      t.l = ldec;
      t.slice = ldec;
      t.e = 0;
      t.m = a.M;
    }
    const auto& L = lins[t.l];
    t.grp = (int)(local / L.chunks);
    t.chunk = (int)(local - (long long)t.grp * L.chunks);
    // Window `sub` of chunk c: [c0 + sub len / L.sub, c0 + (sub + 1) len / L.sub)
    // of the chunk's segments [c0, c0 + len).
    const int c0 = (int)((long long)t.chunk * L.spt / L.chunks);
    const int len = (int)((long long)(t.chunk + 1) * L.spt / L.chunks) - c0;
    t.sub = sub;
    t.spc = ((L.spt + L.chunks - 1) / L.chunks + L.sub - 1) / L.sub;
    t.j0 = c0 + sub * len / L.sub;
    t.j1 = c0 + (sub + 1) * len / L.sub;
    return t;
  };
  // Segment j of unit t into s.  Rows past N read row N - 1 (a B column only
  // feeds its own output, which is not written) and chunks past the row's
  // end read its last chunk (zeroed in LDS before use), so every load is
  // unconditional and in bounds and the compiler's waits stay exact.
  auto load = [&](TileSeg<DT>& s, const TileUnit& t, int j) {
    const auto& L = lins[t.l];
    const int row0 = t.grp * kGroupRows + wrow;
    const int c = min(j * kSegChunksT + lchunk, L.cpr - 1);
    const u32x4* w = MOE ? L.w + (size_t)t.e * a.moe.w_stride : L.w;
#pragma unroll
    for (int q = 0; q < kLoadsT; ++q) {
      const int row = min(row0 + kRowsPerLoadT * q + lrow, L.N - 1);
      s.w[q] = ldw(w + (size_t)row * L.cpr + c);
    }
    if (DT == SKINNY_FP8_BS128) {
      // The row group lies in one 128-row scale block.  Blocks past K cover
      // only zeroed weights; clamping keeps the read in bounds.
      const float* scale = MOE ? L.scale + (size_t)t.e * a.moe.s_stride : L.scale;
      const float* srow = scale + (size_t)((t.grp * kGroupRows) / kScaleBlock) * L.kblocks;
      s.sc = srow[min(kSegBlocksT * j + lane % kSegBlocksT, L.kblocks - 1)];
    }
    // Keep the loads ahead of the previous segment's work.
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int xw0 = 0, xstride = 1;                            // x window of the current unit
  const u32x4* xrow = xs;
  int xsw = 0;                                         // FIT: this lane's token's swizzle
  auto consume = [&](const TileSeg<DT>& s, const TileUnit& t, int j) {
    const auto& L = lins[t.l];
#pragma unroll
    for (int q = 0; q < kLoadsT; ++q)
      *reinterpret_cast<u32x4*>(wt + (kRowsPerLoadT * q + lrow) * kStride +
                                wslot(lchunk, kRowsPerLoadT * q + lrow) * 16) = s.w[q];
    if ((j + 1) * kSegChunksT > L.cpr && j * kSegChunksT + lchunk >= L.cpr) {
      // The row's ragged end: zero the chunks past it (written after the
      // clamped data, so these writes win).
#pragma unroll
      for (int q = 0; q < kLoadsT; ++q)
        *reinterpret_cast<u32x4*>(wt + (kRowsPerLoadT * q + lrow) * kStride +
                                  wslot(lchunk, kRowsPerLoadT * q + lrow) * 16) = zero4();
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < kStepsT; ++st) {
      const u32x4 b =
          *reinterpret_cast<const u32x4*>(wt + n * kStride + wslot(4 * st + g, n) * 16);
      const int xc = (j * kSegChunksT + 4 * st + g) * XC - xw0;  // x chunk in the window
      if (DT == SKINNY_BF16) {
        acc = mfma_bf16(xrow[xc ^ xsw], b, acc);
      } else {
        const u32x4 x0 = xrow[xc ^ xsw];
        const u32x4 x1 = xrow[(xc + 1) ^ xsw];
        u32x4 b0, b1;
        e4m3x16_to_bf16(b, b0, b1);
        p = mfma_bf16(x0, b0, p);
        p = mfma_bf16(x1, b1, p);
        if (st & 1) {
          // Steps 2 i and 2 i + 1 cover the 128 k of the segment's block i.
          const float sc = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.sc), st >> 1));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, p[i], acc[i]);
          p = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // x[M][window] of unit t into LDS, between two barriers, if it is not
  // there already (the same decision in every wave).
  int staged_l = -1, staged_c = -1, staged_s = -1;
  auto stage = [&](const TileUnit& t) {
    const auto& L = lins[t.l];
    const int win = t.spc * kSegChunksT * XC;                    // x chunks per token in LDS
    xstride = FIT ? win : win + 1;
    xw0 = t.j0 * kSegChunksT * XC;
    if (FIT) {
      const int tok = n < t.m ? n : 0;
      xrow = xs + tok * xstride;
      xsw = tok & 7;
    } else {
      xrow = xs + (n < t.m ? n : t.m) * xstride;
    }
    if (t.slice == staged_l && t.chunk == staged_c && t.sub == staged_s) return;
    staged_l = t.slice;
    staged_c = t.chunk;
    staged_s = t.sub;
    const int xcpr = L.K >> 3;                                   // x chunks per token
    __syncthreads();                                             // all done with the old window
    // Token rows 0..M-1, zeros past K, then a zero row that lanes of absent
    // tokens read.
    const int wlen = min(win, xcpr - xw0);
    if constexpr (FIT) {
      // Token rows 0..M-1 only, swizzled, zeros past K (plain x: the host
      // takes this form only for linears without an activation).
      stage_x_fit<kThreads>(L.x, t.m, xcpr, xw0, wlen, win, xs);
    } else {
      const unsigned char* rows = MOE ? tb.xrow + t.slice * kMoeMaxCap : nullptr;
      if (L.act == kActNone)
        stage_x_direct<kThreads, MOE>(L.x, t.m, xcpr, xw0, wlen, xs, xstride, rows);
      else
        stage_x<kThreads, MOE>(L.x, L.act, t.m, xcpr, xw0, wlen, xs, xstride, rows);
      const int pad = win - wlen;
      for (int i = threadIdx.x; i < t.m * pad; i += kThreads) {
        const int m = i / pad;
        xs[m * xstride + wlen + (i - m * pad)] = zero4();
      }
      for (int c = threadIdx.x; c < win; c += kThreads) xs[t.m * xstride + c] = zero4();
    }
    __builtin_amdgcn_s_waitcnt(0);                               // direct loads landed
    __syncthreads();
  };
  auto epilogue = [&](const TileUnit& t) {
    if constexpr (KS) {
      // The waves' partial tiles, added by wave 0 in wave order.  The other
      // half of `red` takes the next unit's, so one barrier per unit
      // suffices: a wave writes this half again only after passing the next
      // unit's barrier, which wave 0 reaches after these reads.
      f32x4* r = red + red_half * (WPB * 64);
      red_half ^= 1;
      r[wv * 64 + lane] = acc;
      __syncthreads();
      if (wv != 0) {
        acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        return;
      }
      f32x4 sum = r[lane];
#pragma unroll
      for (int w = 1; w < WPB; ++w) sum += r[w * 64 + lane];
      acc = sum;
    }
    // Lane (n, g) holds D[4 g + i][n]: token 4 g + i, row row0 + n.
    const auto& L = lins[t.l];
    const int row = t.grp * kGroupRows + wrow + n;
    const long long slot = (MOE ? (long long)t.slice * a.moe.units_per_slice : L.slot_base) +
                           (long long)t.grp * L.chunks + t.chunk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < t.m) {
        if (L.chunks == 1) {
          const int yr = MOE ? tb.yrow[t.slice * kMoeMaxCap + m] : m;
          if (row < L.N) L.y[(size_t)yr * L.N + row] = (__bf16)acc[i];
        } else {
          a.slots[((size_t)slot * a.M + m) * kGroupRows + wrow + n] = acc[i];
        }
      }
    }
    acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  // The segments of unit t, the first of which is already loading into A.
  // Ends with the first segment of unit nx (if has_next) loading into A when
  // t has an even number of segments, into B when odd; returns which.
  // This wave's segments of t are j0 + seg_off, then every kSegStep-th; in
  // the K-split form a window may hold none for this wave, and then nothing
  // was loaded for it.
  auto run_unit = [&](TileSeg<DT>& A, TileSeg<DT>& B, const TileUnit& t, const TileUnit& nx,
                      bool has_next) {
    const bool next = has_next && nx.j0 + seg_off < nx.j1;
    int j = t.j0 + seg_off;
    if (KS && j >= t.j1) {
      if (next) load(A, nx, nx.j0 + seg_off);
      return 0;
    }
    for (; j + 2 * kSegStep < t.j1; j += 2 * kSegStep) {
      load(B, t, j + kSegStep);
      consume(A, t, j);
      load(A, t, j + 2 * kSegStep);
      consume(B, t, j + kSegStep);
    }
    if (j + kSegStep < t.j1) {
      load(B, t, j + kSegStep);
      consume(A, t, j);
      if (next) load(A, nx, nx.j0 + seg_off);
      consume(B, t, j + kSegStep);
      return 0;
    }
    if (next) load(B, nx, nx.j0 + seg_off);
    consume(A, t, j);
    return 1;
  };
  long long u = blockIdx.x;
  if (u >= S) return;
  TileSeg<DT> s0, s1;
  TileUnit cur = decode(u, 0);
  if (cur.j0 + seg_off < cur.j1) load(s0, cur, cur.j0 + seg_off);
  int in_b = 0;                                         // the current unit's first segment is in s1
  for (;;) {
    // A unit's x windows in turn (its sums stay in acc), then the next unit.
    const bool last = cur.sub + 1 == lins[cur.l].sub;
    const bool has_next = !last || u + a.G < S;
    const TileUnit nx = !last ? decode(u, cur.sub + 1) : has_next ? decode(u + a.G, 0) : cur;
    stage(cur);
    const int flip = in_b ? run_unit(s1, s0, cur, nx, has_next)
                          : run_unit(s0, s1, cur, nx, has_next);
    if (last) epilogue(cur);
    if (!has_next) break;
    in_b ^= flip;
    cur = nx;
    if (last) u += a.G;
  }
}

// ---------------------------------------------------------------------------
// Second pass: for every output of a split linear, the sum of its K-chunks'
// partial results in chunk order.  blockIdx.y is the linear; thread t of
// the grid row takes four adjacent rows (one 16-byte slot read per chunk; a
// row group's height is a multiple of four) of one token.
constexpr int kCombineRows = 4;
constexpr int kCombineBatch = 8;

// p[0] + p[stride] + ... + p[(n - 1) stride], added in that order.  Loads go
// out kCombineBatch at a time (the last batch's past n re-read chunk n - 1
// and are not added), so a thread waits once per batch instead of once per
// chunk.
__device__ __forceinline__ f32x4 sum_chunks(const f32x4* p, size_t stride, int n) {
  f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < n; c += kCombineBatch) {
    f32x4 v[kCombineBatch];
#pragma unroll
    for (int q = 0; q < kCombineBatch; ++q) v[q] = p[(size_t)min(c + q, n - 1) * stride];
#pragma unroll
    for (int q = 0; q < kCombineBatch; ++q)
      if (c + q < n)
#pragma unroll
        for (int r = 0; r < kCombineRows; ++r) sum[r] += v[q][r];
  }
  return sum;
}
__global__ __launch_bounds__(kCombineThreads) void skinny_combine(const LaunchArgs a) {
  KLinDesc& L = launch_lins(a)[blockIdx.y];
  if (L.chunks == 1) return;
  const int R = a.band_rows;
  const int quads = (L.N + kCombineRows - 1) / kCombineRows;   // per token
  const int i = blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= a.M * quads) return;
  const int m = i / quads;
  const int row = (i - m * quads) * kCombineRows;
  const int grp = row / R;
  const int rr = row - grp * R;
  const f32x4* p = reinterpret_cast<const f32x4*>(
      a.slots + ((size_t)(L.slot_base + (long long)grp * L.chunks) * a.M + m) * R + rr);
  const size_t stride = (size_t)a.M * R / kCombineRows;        // one chunk's slot, in f32x4
  const f32x4 sum = sum_chunks(p, stride, L.chunks);
  __bf16* y = L.y + (size_t)m * L.N + row;
#pragma unroll
  for (int r = 0; r < kCombineRows; ++r)
    if (row + r < L.N) y[r] = (__bf16)sum[r];
}

// Second pass of a split MoE launch: grid row y is a slice, the table the
// first workgroup of the main kernel left in the workspace names its routes.
__global__ __launch_bounds__(kCombineThreads) void skinny_moe_combine(const LaunchArgs a) {
  const LinDesc& L = moe_lins(a)[0];
  const int* tb = a.moe.table;
  const int sl = blockIdx.y;
  if (sl >= tb[0]) return;
  const int M = tb[1 + sl];
  const int R = a.band_rows;
  const int quads = (L.N + kCombineRows - 1) / kCombineRows;
  const int i = blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= M * quads) return;
  const int m = i / quads;
  const int row = (i - m * quads) * kCombineRows;
  const int grp = row / R;
  const int rr = row - grp * R;
  const long long slot0 = (long long)sl * a.moe.units_per_slice + (long long)grp * L.chunks;
  const f32x4* p =
      reinterpret_cast<const f32x4*>(a.slots + ((size_t)slot0 * a.M + m) * R + rr);
  const size_t stride = (size_t)a.M * R / kCombineRows;
  const f32x4 sum = sum_chunks(p, stride, L.chunks);
  __bf16* y = L.y + (size_t)tb[1 + a.moe.max_slices + sl * kMoeMaxCap + m] * L.N + row;
#pragma unroll
  for (int r = 0; r < kCombineRows; ++r)
    if (row + r < L.N) y[r] = (__bf16)sum[r];
}

// ---------------------------------------------------------------------------
// The experts' gated MLP for one token in one launch: gate_up of each chosen
// expert, the SiLU-gated product, then down ("Multi-GPU Inference and
// Serving at Scale", Example 8: a router sends the token to its top-k
// experts; Example 3: an MLP's activation sits between its two linears).
// Route r uses expert ids[r]; routes whose id is outside [0, E) have zero
// outputs.  With one token each expert is read for one route, and two
// dependent launches cost more than their bytes (a launch's start, its first
// loads and its tail, twice); here the workgroups pass gate_up's outputs to
// each other within the launch.  Each output pair is written as one 64-bit
// word carrying the call's number, and a workgroup that computes down rows
// reads the words of its route until all carry this call's number: the data
// is its own signal, with no counter to wait on between the linears.  The
// call's number is the count of finished workgroups over all earlier calls
// divided by G, plus one; each workgroup adds itself to that count as it
// ends, and reads it at its start (at most G - 1 others of the same call can
// have ended by then, which leaves the quotient unchanged).  The grid is the
// resident one, so every workgroup whose outputs are waited for is running;
// the wait gives up after `spin` polls and then sets a flag word, so it never
// hangs.
//
// Units are 8 rows of one route (one row per wave): gate_up units dealt round
// robin over the grid, down units of each route over a group of workgroups
// (so each reads the outputs of one route).  A wave issues the loads of all
// its gate_up rows at its start and of all its down rows once its gate_up
// products are done (MA and MB slots of U 1 KB segments, unconditional, in a
// straight line so the waits stay exact), so down's weights arrive while the
// outputs of gate_up are passed on.
struct MoeMlpArgs {
  const u32x4* wg;       // gate_up experts [E][N1][K1], 16-byte chunks
  const float* sg;       // their FP8 scales [E][ceil(N1/128)][ceil(K1/128)]
  const u32x4* wd;       // down experts [E][N2][K2]
  const float* sd;
  long long wg_stride, sg_stride, wd_stride, sd_stride;   // per expert
  int E, R;              // experts; routes (top-k of the one token)
  int N1, K1, cpr1, spt1, kb1;   // gate_up: N1 = 2 K2 rows ([gate | up]) of K1
  int N2, K2, cpr2, spt2, kb2;   // down: N2 rows of K2
  const int* ids;        // [R]
  const u32x4* x;        // [K1] bf16
  unsigned long long* gu;         // [R][N1 / 2] gate_up outputs: call number << 32 | 2 x bf16
  __bf16* y;             // [R][N2] bf16
  unsigned long long* ended;      // workgroups finished, over all calls
  int* gave_up;          // set when a wait gives up
  long long spin;        // polls before a wait gives up; < 0: do not wait
  int G;
  int hs_off, ya_off, yb_off, tab_off;   // LDS: x at 0, h, the output buffers, the route table
};

// A workgroup's walk over its units of one linear: unit t is b + t G, in
// route k (of the valid routes) at row group grp; slot item j.
struct MlpCursor {
  int t, j, k, grp;
};

__device__ __forceinline__ MlpCursor mlp_cursor(int u, int g) {
  return MlpCursor{0, 0, u / g, u % g};
}

__device__ __forceinline__ void mlp_advance(MlpCursor& c, int items, int g, int G) {
  if (++c.j < items) return;
  c.j = 0;
  ++c.t;
  c.grp += G;
  while (c.grp >= g) {
    c.grp -= g;
    ++c.k;
  }
}

template <int DT, int MA, int MB, int U>
__global__ __launch_bounds__(64 * kRowsWavesPerBlock) void skinny_moe_mlp1(const MoeMlpArgs a) {
  constexpr int WPB = kRowsWavesPerBlock;
  constexpr int kThreads = 64 * WPB;
  constexpr bool kFp8 = DT == SKINNY_FP8_BS128;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  u32x4* hs = reinterpret_cast<u32x4*>(lds + a.hs_off);      // h of route kb: [K2 / 8]
  __bf16* ya = reinterpret_cast<__bf16*>(lds + a.ya_off);    // [gate_up unit][wave]
  __bf16* yb = reinterpret_cast<__bf16*>(lds + a.yb_off);    // [down unit][wave]
  int* tab = reinterpret_cast<int*>(lds + a.tab_off);        // nv, route[16], expert[16], call
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int G = a.G;
  // x into LDS and the router's choices, with one wait for both.
  const int n1x = a.K1 >> 3;
  for (int p = wv; p * 64 < n1x; p += WPB)
    __builtin_amdgcn_global_load_lds(a.x + min(p * 64 + lane, n1x - 1),
                                     (__attribute__((address_space(3))) void*)(xs + p * 64), 16,
                                     0, 0);
  int e = -1;
  if (wv == 0 && lane < a.R) e = a.ids[lane];
  unsigned long long ended = 0;
  if (threadIdx.x == 0)
    ended = __hip_atomic_load(a.ended, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  if (wv == 0) {                         // valid routes, in route order
    const bool ok = lane < a.R && e >= 0 && e < a.E;
    const unsigned long long m = __ballot(ok);
    if (ok) {
      const int pos = __popcll(m & ((1ull << lane) - 1));
      tab[1 + pos] = lane;
      tab[1 + kMoeMlpMaxRoutes + pos] = e;
    }
    if (lane == 0) {
      tab[0] = __popcll(m);
      tab[1 + 2 * kMoeMlpMaxRoutes] = (int)(unsigned)(ended / G + 1);
    }
  }
  __syncthreads();
  const int nv = __builtin_amdgcn_readfirstlane(tab[0]);
  const int gA = (a.N1 + WPB - 1) / WPB, gB = (a.N2 + WPB - 1) / WPB;
  const int UA = nv * gA;
  const int nua = b < UA ? (UA - 1 - b) / G + 1 : 0;     // this workgroup's gate_up units
  // down: the workgroups are split into one group per valid route, so each
  // stages h of one route only (half the reads of the intermediate at top-2,
  // which all workgroups read at once); workgroup b takes row groups
  // lb, lb + Gk, ... of route kb.
  const int kb = nv > 0 ? b * nv / G : 0;
  const int wg0 = nv > 0 ? (kb * G + nv - 1) / nv : 0;
  const int Gk = nv > 0 ? ((kb + 1) * G + nv - 1) / nv - wg0 : 1;
  const int lb = b - wg0;
  const int nub = nv > 0 && lb < gB ? (gB - 1 - lb) / Gk + 1 : 0;
  const int ia = (a.spt1 + U - 1) / U, ib = (a.spt2 + U - 1) / U;   // slots per unit
  const int k2c = a.K2 >> 3;                                          // h chunks per route

  // Every slot is loaded, all at the start: the slots of a linear walk the
  // workgroup's units item by item; slots past its units re-read its last
  // item (or x, if it has none), and their products are skipped.
  auto load_slot = [&](FlatSlot<U>& q, const MlpCursor& c, int n, bool down) {
    const u32x4* w = a.x;
    const float* sc = a.sg;
    int cpr = 1, j = 0;
    if (n > 0) {
      MlpCursor d = c;
      if (c.t >= n) {                    // the last unit's last item
        if (down) {
          d = MlpCursor{n - 1, ib - 1, kb, lb + (n - 1) * Gk};
        } else {
          d = mlp_cursor(b + (n - 1) * G, gA);
          d.j = ia - 1;
        }
      }
      j = d.j;
      const int N = down ? a.N2 : a.N1;
      const int row = min(d.grp * WPB + wv, N - 1);
      const int ex = __builtin_amdgcn_readfirstlane(tab[1 + kMoeMlpMaxRoutes + d.k]);
      cpr = down ? a.cpr2 : a.cpr1;
      w = (down ? a.wd + (size_t)ex * a.wd_stride : a.wg + (size_t)ex * a.wg_stride) +
          (size_t)row * cpr;
      if (kFp8)
        sc = (down ? a.sd + (size_t)ex * a.sd_stride : a.sg + (size_t)ex * a.sg_stride) +
             (size_t)(row / kScaleBlock) * (down ? a.kb2 : a.kb1);
    }
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const int c = min((j * U + v) * kSegChunks + lane, cpr - 1);
      q.w[v] = ldw(w + c);
      if (kFp8) q.s[v] = sc[c >> 3];
    }
  };
  FlatSlot<U> qa[MA], qb[MB];
  {
    MlpCursor c = mlp_cursor(b, gA);
#pragma unroll
    for (int s = 0; s < MA; ++s) {
      load_slot(qa[s], c, nua, false);
      mlp_advance(c, ia, gA, G);
    }
  }
  auto down_cursor = [&]() { return MlpCursor{0, 0, kb, lb}; };
  auto down_advance = [&](MlpCursor& c) {
    if (++c.j < ib) return;
    c.j = 0;
    ++c.t;
    c.grp += Gk;
  };
  auto load_down = [&]() {
    MlpCursor c = down_cursor();
#pragma unroll
    for (int s = 0; s < MB; ++s) {
      load_slot(qb[s], c, nub, true);
      down_advance(c);
    }
  };

  float acc = 0.0f;
  // Products of one slot at cursor c, from src; at a unit's last item the
  // row's sum goes to the LDS buffer.
  auto consume = [&](const FlatSlot<U>& q, const MlpCursor& c, int n, bool down,
                     const u32x4* src) {
    if (c.t >= n) return;
    const int cpr = down ? a.cpr2 : a.cpr1;
    const int j = c.j;
    if ((j + 1) * U * kSegChunks <= cpr) {
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int ci = (j * U + v) * kSegChunks + lane;
        if (kFp8) {
          u32x4 b0, b1;
          e4m3x16_to_bf16(q.w[v], b0, b1);
          acc = __builtin_fmaf(q.s[v], dot8(src[2 * ci + 1], b1, dot8(src[2 * ci], b0, 0.0f)),
                               acc);
        } else {
          acc = dot8(src[ci], q.w[v], acc);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int ci = (j * U + v) * kSegChunks + lane;
        const bool ok = ci < cpr;
        const int cx = ok ? ci : 0;
        float tv;
        if (kFp8) {
          u32x4 b0, b1;
          e4m3x16_to_bf16(q.w[v], b0, b1);
          tv = __builtin_fmaf(q.s[v], dot8(src[2 * cx + 1], b1, dot8(src[2 * cx], b0, 0.0f)),
                              acc);
        } else {
          tv = dot8(src[cx], q.w[v], acc);
        }
        acc = ok ? tv : acc;
      }
    }
    if (j == (down ? ib : ia) - 1) {
      acc = wave_sum_rows(acc);
      if (lane == 0) (down ? yb : ya)[c.t * WPB + wv] = (__bf16)acc;
      acc = 0.0f;
    }
  };
  {
    MlpCursor c = mlp_cursor(b, gA);
#pragma unroll
    for (int s = 0; s < MA; ++s) {
      consume(qa[s], c, nua, false, xs);
      mlp_advance(c, ia, gA, G);
    }
  }

  // Wave 0 writes gate_up's outputs, tagged with the call's number, then every
  // wave loads its down rows while the outputs are passed on (loading them
  // earlier, before the outputs are out, measured slower: 15.6 against
  // 14.5 us).  The words are relaxed device-scope atomic accesses, which the
  // hardware keeps coherent across the chip without cache-wide write-backs or
  // invalidations (release and acquire fences cost one of those per
  // workgroup, measured at tens of microseconds over the grid).
  __syncthreads();
  const unsigned call = (unsigned)tab[1 + 2 * kMoeMlpMaxRoutes];
  if (wv == 0) {
    for (int i = lane; i < nua * (WPB / 2); i += 64) {
      const int t = i / (WPB / 2), w = i - t * (WPB / 2);
      const int u = b + t * G;
      const int k = u / gA;
      const unsigned lo = __builtin_bit_cast(unsigned short, ya[t * WPB + 2 * w]);
      const unsigned hi = __builtin_bit_cast(unsigned short, ya[t * WPB + 2 * w + 1]);
      __hip_atomic_store(a.gu + ((size_t)tab[1 + k] * a.N1 + (u - k * gA) * WPB) / 2 + w,
                         ((unsigned long long)call << 32) | lo | (hi << 16), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  load_down();
  // h of route kb: every word read until it carries this call's number.
  // Each workgroup starts at a different chunk, so that the workgroups
  // reading one route at once spread over its lines.
  if (nub > 0) {
    const unsigned long long* row = a.gu + (size_t)tab[1 + kb] * (a.N1 / 2);
    const int rot = (int)(((long long)b * 67) % k2c);
    bool gave_up = a.spin < 0;
    for (int i = threadIdx.x; i < k2c; i += kThreads) {
      const int c = i + rot < k2c ? i + rot : i + rot - k2c;
      unsigned long long wd[8];
      long long polls = 0;
      for (;;) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wd[q] = __hip_atomic_load(row + 4 * c + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          wd[4 + q] = __hip_atomic_load(row + 4 * (k2c + c) + q, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        }
        bool ready = true;
#pragma unroll
        for (int q = 0; q < 8; ++q) ready = ready && (unsigned)(wd[q] >> 32) == call;
        if (ready || gave_up) break;
        if (++polls > a.spin) gave_up = true;
        __builtin_amdgcn_s_sleep(1);
      }
      u32x4 g, v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        g[q] = (unsigned)wd[q];
        v[q] = (unsigned)wd[4 + q];
      }
      hs[c] = swiglu8(g, v);
    }
    if (gave_up) __hip_atomic_store(a.gave_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  {
    MlpCursor c = down_cursor();
#pragma unroll
    for (int s = 0; s < MB; ++s) {
      consume(qb[s], c, nub, true, hs);
      down_advance(c);
    }
  }

  // Down outputs, then the zero rows of routes with no expert.
  __syncthreads();
  for (int i = threadIdx.x; i < nub * WPB; i += kThreads) {
    const int row = (lb + (i / WPB) * Gk) * WPB + (i % WPB);
    if (row < a.N2) a.y[(size_t)tab[1 + kb] * a.N2 + row] = yb[i];
  }
  if (nv < a.R) {
    for (int r = 0, k = 0; r < a.R; ++r) {
      if (k < nv && tab[1 + k] == r) {
        ++k;
        continue;
      }
      for (int i = b * kThreads + threadIdx.x; i < a.N2; i += G * kThreads)
        a.y[(size_t)r * a.N2 + i] = (__bf16)0.0f;
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(a.ended, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Greedy next token: for each token, the smallest index of the largest logit
// ("Developing a custom Qwen2.5 72B inference engine from scratch - what is
// the real bottleneck?", section 5, third lever: pick the next token on the
// GPU instead of copying the logits to the host).  Two passes, no atomics:
// workgroup (b, m) of the first reduces slice b of row m (kArgmaxSlice
// logits) to one (value, index) pair in the workspace; the second reduces
// each row's pairs.  Pairs are ordered by value, then by lower index, so
// the result does not depend on the reduction order.  NaN ranks below every
// number, -inf included: a NaN is never taken, and a pair that has seen no
// number keeps the index N, which loses to every real index; a row of NaNs
// ends with N and gives 0.
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxSlice = 4096;                    // logits per first-pass workgroup
constexpr int kArgmaxMaxSlices = 1 << 20;


// (value, index) of the workgroup into lane 0 of wave 0.
__device__ __forceinline__ void argmax_block(float& bv, int& bi) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    argmax_take(ov, oi, bv, bi);
  }
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wv] = bv;
    si[wv] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < kArgmaxThreads / 64; ++w) argmax_take(sv[w], si[w], bv, bi);
}

// VEC: N % 8 == 0 and 16-byte aligned rows, 8 logits per load.
template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads) void skinny_argmax_slices(const __bf16* y, int N,
                                                                       ArgmaxPair* pairs) {
  const int m = blockIdx.y;
  const int n0 = blockIdx.x * kArgmaxSlice;
  const int n1 = min(n0 + kArgmaxSlice, N);
  const __bf16* row = y + (size_t)m * N;
  float bv = -__builtin_inff();
  int bi = N;                                         // loses to any element
  if constexpr (VEC) {
    const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
    constexpr int kPer = kArgmaxSlice / 8 / kArgmaxThreads;   // loads per thread
    u32x4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) v[q] = r4[min((n0 / 8) + q * kArgmaxThreads + (int)threadIdx.x,
                                                  N / 8 - 1)];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = n0 / 8 + q * kArgmaxThreads + threadIdx.x;
      if (8 * c < n1) {
        const bf16x8 e = __builtin_bit_cast(bf16x8, v[q]);
#pragma unroll
        for (int k = 0; k < 8; ++k) argmax_take((float)e[k], 8 * c + k, bv, bi);
      }
    }
  } else {
    for (int n = n0 + threadIdx.x; n < n1; n += kArgmaxThreads) argmax_take((float)row[n], n, bv, bi);
  }
  argmax_block(bv, bi);
  if (threadIdx.x == 0) pairs[(size_t)m * gridDim.x + blockIdx.x] = ArgmaxPair{bv, bi};
}

__global__ __launch_bounds__(kArgmaxThreads) void skinny_argmax_rows(const ArgmaxPair* pairs,
                                                                     int slices, int N, int* idx) {
  const int m = blockIdx.x;
  float bv = -__builtin_inff();
  int bi = N;
  for (int b = threadIdx.x; b < slices; b += kArgmaxThreads) {
    const ArgmaxPair p = pairs[(size_t)m * slices + b];
    argmax_take(p.v, p.i, bv, bi);
  }
  argmax_block(bv, bi);
  if (threadIdx.x == 0) idx[m] = bi < N ? bi : 0;
}

// ---------------------------------------------------------------------------
// Host side.

struct DeviceInfo {
  int cus = 0;
  bool gfx950 = false;
  bool valid = false;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

skinny_status device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SKINNY_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_dev[dev].valid) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return SKINNY_ERR_HIP;
    g_dev[dev].cus = p.multiProcessorCount;
    g_dev[dev].gfx950 = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].valid = true;
  }
  *out = g_dev[dev];
  return SKINNY_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// allow_act: the library's own chained linears carry their input activation
// in `reserved` (kActSwiGLU); a caller's linear must have 0 there.
skinny_status check_linear(const skinny_linear& L, int M, bool allow_act = false) {
  if (L.dtype != SKINNY_BF16 && L.dtype != SKINNY_FP8_BS128) return SKINNY_ERR_INVALID_ARG;
  if (L.reserved != 0 && !(allow_act && L.reserved == kActSwiGLU)) return SKINNY_ERR_INVALID_ARG;
  if (M < 1 || M > SKINNY_MAX_M || L.N < 1 || L.K < 1) return SKINNY_ERR_INVALID_ARG;
  if (!L.w || !L.x || !L.y) return SKINNY_ERR_INVALID_ARG;
  if (L.dtype == SKINNY_FP8_BS128 && !L.w_scale) return SKINNY_ERR_INVALID_ARG;
  if (L.dtype == SKINNY_BF16 && L.w_scale) return SKINNY_ERR_INVALID_ARG;
  if (L.K % (L.dtype == SKINNY_BF16 ? 8 : 16) != 0) return SKINNY_ERR_UNSUPPORTED;
  if (!aligned(L.w, 16) || !aligned(L.x, 16) || !aligned(L.y, 16)) return SKINNY_ERR_UNSUPPORTED;
  if (L.w_scale && !aligned(L.w_scale, 4)) return SKINNY_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels is 32-bit per band, per row and per
  // (token, row) output of a linear.
  if (L.N > (1 << 26) || L.K > (1 << 28)) return SKINNY_ERR_UNSUPPORTED;
  return SKINNY_OK;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// The buffers a call writes (every y and the workspace) must not overlap
// anything else it reads or writes.
skinny_status check_outputs(const skinny_linear* lin, int count, int M, const void* ws,
                            size_t ws_bytes) {
  const Range wsr{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  for (int i = 0; i < count; ++i) {
    const skinny_linear& L = lin[i];
    Range y{(uintptr_t)L.y, (uintptr_t)L.y + (size_t)M * L.N * 2};
    if (overlap(y, wsr)) return SKINNY_ERR_INVALID_ARG;
    {
      const size_t wbytes = (size_t)L.N * L.K * (L.dtype == SKINNY_BF16 ? 2 : 1);
      const size_t xbytes = (size_t)M * L.K * 2 * (L.reserved == kActSwiGLU ? 2 : 1);
      if (overlap(wsr, Range{(uintptr_t)L.x, (uintptr_t)L.x + xbytes}) ||
          overlap(wsr, Range{(uintptr_t)L.w, (uintptr_t)L.w + wbytes}))
        return SKINNY_ERR_INVALID_ARG;
      if (L.w_scale) {
        const size_t sb = (size_t)((L.N + 127) / 128) * ((L.K + 127) / 128) * 4;
        if (overlap(wsr, Range{(uintptr_t)L.w_scale, (uintptr_t)L.w_scale + sb}))
          return SKINNY_ERR_INVALID_ARG;
      }
    }
    for (int j = 0; j < count; ++j) {
      const skinny_linear& O = lin[j];
      const size_t wbytes = (size_t)O.N * O.K * (O.dtype == SKINNY_BF16 ? 2 : 1);
      const size_t xbytes = (size_t)M * O.K * 2 * (O.reserved == kActSwiGLU ? 2 : 1);
      Range x{(uintptr_t)O.x, (uintptr_t)O.x + xbytes};
      Range w{(uintptr_t)O.w, (uintptr_t)O.w + wbytes};
      if (overlap(y, x) || overlap(y, w)) return SKINNY_ERR_INVALID_ARG;
      if (O.w_scale) {
        const size_t sb = (size_t)((O.N + 127) / 128) * ((O.K + 127) / 128) * 4;
        Range s{(uintptr_t)O.w_scale, (uintptr_t)O.w_scale + sb};
        if (overlap(y, s)) return SKINNY_ERR_INVALID_ARG;
      }
      if (j != i) {
        Range y2{(uintptr_t)O.y, (uintptr_t)O.y + (size_t)M * O.N * 2};
        if (overlap(y, y2)) return SKINNY_ERR_INVALID_ARG;
      }
    }
  }
  return SKINNY_OK;
}

// skinny_rows shape per M: R rows per wave (one LDS read of x serves R weight
// loads, so LDS traffic stays at <= 2 x reads per weight load up to M = 8) and
// U segments per batch, R x U = 8 loads (bf16) or 4 (FP8, whose conversion
// needs the registers) per batch, two batches in flight.  bf16 at M = 2 takes
// half batches, which fit the 128 VGPRs of two workgroups per CU: as many
// loads in flight per CU as one workgroup of full batches, and measured on
// MI355X 42.0 against 47.4 us on the TP=8 layer (TP=1 stacks within +-1.5%).
constexpr int rows_r(int M) { return M <= 2 ? 1 : M <= 4 ? 2 : 4; }
constexpr int rows_u(int M, int dtype) {
  return (dtype == SKINNY_BF16 ? (M == 2 ? 4 : 8) : 4) / rows_r(M);
}
// The lean instance for large bf16 launches: 2 KB batches (2 / R segments
// of R rows) and one 8-wave workgroup per CU, so about 32 KB of loads are in
// flight per CU instead of ~6x that.  Measured on MI355X with an
// arithmetic-free read probe, HBM reads stream fastest (6.5 TB/s) with about
// 32 KB in flight per CU: less leaves latency exposed, more loses ~5% (the
// memory system serves a wider window of addresses at once).  On an 8-layer
// TP=1 launch the lean instance streams 6.49 against 6.20 TB/s (M = 1) and
// 6.38 against 6.09 (M = 2); a launch too small to fill the chip needs the
// deeper instance to cover latency (TP=8 layer at M = 1: 48.0 against 40.9
// us), hence a minimum launch size.
constexpr int rows_u_lean(int M) { return M <= 2 ? 2 : M <= 4 ? 1 : 0; }
constexpr int kRowsLeanWavesPerCU = 8;
constexpr double kRowsLeanLaunchBytes = 0.4e9;     // weight bytes of one launch
constexpr int kRowsXBudget = 64 * 1024;   // LDS for x per workgroup: two workgroups per CU
constexpr int kRowsMaxM = 8;
// Units per workgroup below which a launch cuts K into more chunks for
// parallelism.  Measured on MI355X (TP=8 layer, QKV GEMV): for the row kernel
// the second pass a split needs costs more than the idle workgroups (GEMV
// 10.7 -> 8.0 us without it); the tile kernel's units are 64 rows high and
// it gains from the split (TP=8 layer at M = 1: 52.8 -> 45.5 us).
constexpr int kRowsUnitsPerWorker = 0;
constexpr int kTilesUnitsPerWorker = 16;

// Fewest K-chunks of a linear whose x window (M tokens x chunk) fits the budget.
int rows_lds_chunks(int dtype, int M, int K, int budget = kRowsXBudget) {
  const int xc = dtype == SKINNY_BF16 ? 1 : 2;
  const int cpr = K / (dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunks - 1) / kSegChunks;
  const long long seg_bytes = (long long)M * kSegChunks * xc * 16;   // x bytes per segment
  const int max_spc = (int)(budget / seg_bytes);
  if (max_spc < 1) return -1;
  return (spt + max_spc - 1) / max_spc;
}

// K-chunks of a linear with spt segments: at least c_lds (LDS) and, up to
// spt / min_segs, par (parallelism of a small launch), rounded up to a power
// of two or, when the x window sets the count, to 3 x a power of two if that
// is closer (fewer partial sums, longer runs per row: +1.3-2.4% on the TP=1
// stacks at FP8 M = 1 and 6 and bf16 M = 8, measured on MI355X; parallelism
// splits keep powers of two, which measured better on the TP=8 layer).  The
// grid is then trimmed to a multiple of every count (grid_for_chunks), so
// every workgroup keeps one K-chunk - one x window - for the whole linear.
int chunk_count(int spt, int c_lds, long long par, int min_segs) {
  int c_par = spt / min_segs;
  if (c_par < 1) c_par = 1;
  if (par < c_par) c_par = (int)par;
  const int need = c_par > c_lds ? c_par : c_lds;
  int c = 1;
  while (c < need) c *= 2;
  if (c_lds >= c_par && c > 3 && 3 * (c / 4) >= need) c = 3 * (c / 4);
  return c <= spt ? c : need;
}

int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

// The persistent grid trimmed to a multiple of every K-chunk count of the
// launch (3 x 2^k at most: at most a few percent of the workgroups), so each
// workgroup keeps one chunk per linear; unchanged if no such multiple fits.
int grid_for_chunks(int G, const LinDesc* lin, int count) {
  int l = 1;
  for (int i = 0; i < count; ++i) {
    const int c = lin[i].chunks;
    l = l / gcd(l, c) * c;
    if (l > G) return G;
  }
  return G / l * l;
}

int rows_chunks(int dtype, int M, int K, long long par) {
  const int cpr = K / (dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunks - 1) / kSegChunks;
  return chunk_count(spt, rows_lds_chunks(dtype, M, K), par, rows_u(M, dtype));
}

// Most K-chunks the planner may give a linear: bounds the workspace slots.
int rows_max_chunks(int dtype, int M, int K) { return rows_chunks(dtype, M, K, 1LL << 40); }

bool rows_supported(const skinny_linear& L, int M) {
  if (M > kRowsMaxM) return false;
  if (L.dtype == SKINNY_FP8_BS128 && (L.K + kScaleBlock - 1) / kScaleBlock > kRowsMaxKBlocks)
    return false;
  return rows_lds_chunks(L.dtype, M, L.K) > 0;
}

// skinny_tiles: fewest K-chunks of a linear whose x window fits the LDS
// budget (token rows padded by one chunk), or -1 if not even one segment fits.
constexpr int kTilesMinSegs = 4;          // segments per chunk when splitting for parallelism
// Most segments an x window of M tokens may span within the budget.
// fit: the exact-fit layout (M token rows, no pad chunk).
int tiles_max_spc(int dtype, int M, int budget, bool fit = false) {
  const int xc = dtype == SKINNY_BF16 ? 1 : 2;
  if (fit) return budget / (16 * M) / (kSegChunksT * xc);
  return (budget / (16 * (M + 1)) - 1) / (kSegChunksT * xc);
}

int tiles_lds_chunks(int dtype, int M, int K, int budget = kTilesXBudget, bool fit = false) {
  const int cpr = K / (dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunksT - 1) / kSegChunksT;
  const int max_spc = tiles_max_spc(dtype, M, budget, fit);
  if (max_spc < 1) return -1;
  return (spt + max_spc - 1) / max_spc;
}

int tiles_chunks(int dtype, int M, int K, long long par, int budget = kTilesXBudget) {
  const int cpr = K / (dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunksT - 1) / kSegChunksT;
  return chunk_count(spt, tiles_lds_chunks(dtype, M, K, budget), par, kTilesMinSegs);
}


// skinny_tiles split of one linear: K-chunks, each a unit with its own
// partial slot (enough for the x window to fit the budget, more for a small
// launch's parallelism) or, with `windows` and when parallelism asks for no
// split, one chunk whose x windows the unit's workgroup walks in turn with its
// sums kept in registers: no partial sums and no second pass, but x restaged
// per unit.  The split's partial sums grow with M (M + 1) per weight byte (M
// outputs, a window of M + 1 rows), the walk's restaging with M, so the walk
// wins at large M: MoE launches always walk, dense launches from
// kTilesWalkMinM* tokens on (below).
void tiles_split(int dtype, int M, int K, long long par, int budget, bool windows, int* chunks,
                 int* sub, bool fit = false) {
  const int cpr = K / (dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunksT - 1) / kSegChunksT;
  const int c_lds = tiles_lds_chunks(dtype, M, K, budget, fit);
  *chunks = chunk_count(spt, c_lds, par, kTilesMinSegs);
  *sub = 1;
  if (windows && c_lds > 1 && chunk_count(spt, 1, par, kTilesMinSegs) == 1) {
    *chunks = 1;
    *sub = c_lds;                          // windows of <= spt / c_lds segments each
  }
}

bool tiles_supported(const skinny_linear& L, int M) {
  return tiles_lds_chunks(L.dtype, M, L.K) > 0;
}

// Workspace slots of one launch group: every linear at the most K-chunks the
// planner may give it, for the kernel of this variant (rows per row group) and,
// for the tile kernel, workgroup shape.
size_t group_slots_bytes(const skinny_linear* const* lin, int count, int M, int variant,
                         int wpb = kTilesWavesSmall) {
  const int rows = variant == SKINNY_VARIANT_MFMA ? kTileRows * wpb
                                                  : kRowsWavesPerBlock * rows_r(M);
  long long slots = 0;
  for (int i = 0; i < count; ++i) {
    const int c = variant == SKINNY_VARIANT_MFMA
                      ? tiles_chunks(lin[i]->dtype, M, lin[i]->K, 1LL << 40, tiles_x_budget(wpb))
                      : rows_max_chunks(lin[i]->dtype, M, lin[i]->K);
    if (c > 1) slots += (long long)((lin[i]->N + rows - 1) / rows) * c;
  }
  return (size_t)slots * M * rows * sizeof(float);
}

// Variant choice, measured on MI355X over the Qwen2.5-72B shapes (TP=1 layers
// and stacks of 1-8 layers per launch, the TP=8 layer, single linears).  Row
// streaming keeps one contiguous stream per wave, but its vector work per
// weight grows with M (and FP8 adds a half-rate conversion); the matrix-core
// kernel's does not.  bf16, rows vs tiles: M = 1 and 2 rows everywhere (TP=1
// stacks +2-10% at M = 2, TP=8 layer 42.0 / 44.7 us) but for short rows
// (8192 x 1024: 8.3 / 7.6 us); M = 3 and 4 rows only for launches of >= 2
// TP=1 layers (+2-7%; one layer, 1.76 GB, -1%, the TP=8 layer -3 to -7%:
// above two resident workgroups per CU the row kernel's fixed cost per launch
// is larger); M = 5 and 6 within a few percent either way, M = 8 tiles.  FP8
// at every M tiles (TP=1 stack at M = 1: 5.85 / 5.93 TB/s).
constexpr int kRowsMaxAutoMBf16 = 2;
constexpr int kRowsMaxAutoMBf16Large = 4;
constexpr double kRowsLargeLaunchBytes = 2.5e9;   // weight bytes of one launch
constexpr int kRowsMaxAutoMFp8 = 0;

int auto_variant(const skinny_linear* const* lin, int count, int M) {
  int cap = kRowsMaxAutoMFp8;
  if (lin[0]->dtype == SKINNY_BF16) {
    double bytes = 0;
    for (int i = 0; i < count; ++i) bytes += 2.0 * lin[i]->N * lin[i]->K;
    cap = bytes >= kRowsLargeLaunchBytes ? kRowsMaxAutoMBf16Large : kRowsMaxAutoMBf16;
  }
  if (M > cap) return SKINNY_VARIANT_MFMA;
  for (int i = 0; i < count; ++i)
    if (!rows_supported(*lin[i], M)) return SKINNY_VARIANT_MFMA;
  return SKINNY_VARIANT_VECTOR;
}

typedef void (*main_fn)(LaunchArgs);

struct KernelChoice {
  main_fn fn = nullptr;
  int band_rows = 0;           // rows per row group
  int wpb = 0;                 // waves per workgroup
  bool tiles = false;          // skinny_tiles (else skinny_rows)
  bool flat = false;           // skinny_rows_flat
  bool fit = false;            // skinny_tiles in the exact-fit layout
  int waves_per_cu = kTargetRowsWavesPerCU;   // cap on the persistent grid
  int id = SKINNY_KERNEL_NONE; // enum skinny_kernel
};

template <int DT, int WPB>
KernelChoice tiles_kernel() {
  static_assert(kScaleBlock % (kTileRows * WPB) == 0, "a row group must sit in one scale block");
  static_assert((kTileRows * WPB) % kCombineRows == 0, "second-pass quads");
  KernelChoice k;
  k.fn = skinny_tiles<DT, WPB, false>;
  k.band_rows = kTileRows * WPB;
  k.wpb = WPB;
  k.tiles = true;
  k.id = WPB == kTilesWavesSmall ? SKINNY_KERNEL_TILES : SKINNY_KERNEL_TILES_WIDE;
  return k;
}

// The 8-wave shape in the exact-fit layout (FP8 launches of plain linears).
template <int DT>
KernelChoice tiles_kernel_fit() {
  KernelChoice k = tiles_kernel<DT, kTilesWavesLarge>();
  k.fn = skinny_tiles<DT, kTilesWavesLarge, false, false, true>;
  k.fit = true;
  return k;
}

template <int DT, int MT>
KernelChoice rows_kernel() {
  constexpr int WPB = kRowsWavesPerBlock;
  constexpr int R = rows_r(MT);
  static_assert(kScaleBlock % (WPB * R) == 0, "a row group must sit in one scale block");
  static_assert((WPB * R) % kCombineRows == 0, "second-pass quads");
  KernelChoice k;
  k.fn = skinny_rows<DT, MT, rows_u(MT, DT), R, WPB>;
  k.band_rows = WPB * R;
  k.wpb = WPB;
  k.id = SKINNY_KERNEL_ROWS;
  return k;
}

template <int MT>
KernelChoice rows_kernel_lean() {
  static_assert(rows_u_lean(MT) > 0, "lean instances exist for M <= 4");
  KernelChoice k = rows_kernel<SKINNY_BF16, MT>();
  k.fn = skinny_rows<SKINNY_BF16, MT, rows_u_lean(MT), rows_r(MT), kRowsWavesPerBlock>;
  k.waves_per_cu = kRowsLeanWavesPerCU;
  k.id = SKINNY_KERNEL_ROWS_LEAN;
  return k;
}

// bf16 row-kernel launches of at least kRowsLeanLaunchBytes of weights at
// M <= 4 take the lean instance.
bool rows_lean(const skinny_linear* const* lin, int count, int M) {
  if (lin[0]->dtype != SKINNY_BF16 || rows_u_lean(M) == 0) return false;
  double bytes = 0;
  for (int i = 0; i < count; ++i) bytes += 2.0 * lin[i]->N * lin[i]->K;
  return bytes >= kRowsLeanLaunchBytes;
}

KernelChoice pick_lean(int M) {
  switch (M) {
    case 1: return rows_kernel_lean<1>();
    case 2: return rows_kernel_lean<2>();
    case 3: return rows_kernel_lean<3>();
    case 4: return rows_kernel_lean<4>();
    default: return KernelChoice{};
  }
}

// One-token launches on skinny_rows_flat: FP8 with 2 slots of 2 KB per wave,
// bf16 with 4 of 1 KB.  Measured on MI355X against the kernels they replace
// (same process, interleaved):
// - FP8 launches of at least kFlatLaunchBytes, one 8-wave workgroup per CU:
//   8-layer TP=1 launch 6.22 -> 6.29-6.30 TB/s (tile kernel before), FP8
//   vocabulary projection 225 -> 217 us; one FP8 TP=1 layer (0.87 GB) -0.6%,
//   hence the launch size; other shapes (1 KB slots, 3-8 deep, 16 waves per
//   CU) 0.3-3% slower.  bf16 launches of that size are as fast on the lean
//   skinny_rows instance (8-layer launch 6.50 vs 6.51 TB/s), which they keep.
// - Launches under kFlatSmallBytes (a TP=8 layer, its QKV GEMV), two
//   workgroups per CU: TP=8 layer 39.8 -> 38.7 us (bf16) and 26.1 -> 24.2 us
//   (FP8), QKV GEMV 7.4 -> 7.0 us, against the deep skinny_rows instance and
//   the tile kernel; at one workgroup per CU they were 1-3% slower than those.
//   With several tokens, against skinny_rows (M = 2) and the tile kernel: bf16
//   TP=8 layer 42.6 / 44.2 / 44.5 -> 40.3 / 40.9 / 42.6 us at M = 2 / 3 / 4,
//   QKV GEMV 8.1 / 11.3 -> 7.4 / 8.4 us at M = 2 / 4; FP8 TP=8 layer 26.8 ->
//   26.2 us at M = 2 but 27.4 -> 32.5 us at M = 4, where each 16-byte weight
//   chunk takes two x reads from LDS per token (LDS-bound), hence
//   flat_max_m.  bf16 x of K = 8192 fits the LDS for up to 4 tokens; with a
//   128 KB x budget (one workgroup, 8 waves per CU) it fits 5-8 tokens, but
//   the TP=8 layer then took 50.1 / 54.5 / 64.8 us at M = 5 / 6 / 8 against
//   the tile kernel's 45.1 / 45.3 / 45.6 (two waves per SIMD do not cover the
//   LDS reads and products of 5-8 tokens), so the tile kernel keeps them.
// Neither leaving x staged across linears nor dropping the FP8 scale loads
// (timing-only builds) moved the FP8 rate of the large launches, so it is not
// the staging drains or the extra loads that hold it below the bf16 rate.
constexpr int flat_depth(int dtype) { return dtype == SKINNY_BF16 ? 4 : 2; }
constexpr int flat_segs(int dtype) { return dtype == SKINNY_BF16 ? 1 : 2; }
constexpr int kFlatWavesPerCU = 8;
constexpr int kFlatWavesPerCUSmall = 16;
constexpr double kFlatLaunchBytes = 1.0e9;     // FP8 launches of at least this: flat
constexpr double kFlatSmallBytes = 0.4e9;      // launches under this: flat, 16 waves per CU
constexpr int flat_max_m(int dtype) { return dtype == SKINNY_BF16 ? 4 : 2; }

template <int DT, int MT>
KernelChoice flat_kernel() {
  KernelChoice k;
  k.fn = skinny_rows_flat<DT, MT, flat_depth(DT), flat_segs(DT)>;
  k.band_rows = kRowsWavesPerBlock;
  k.wpb = kRowsWavesPerBlock;
  k.flat = true;
  k.waves_per_cu = kFlatWavesPerCU;
  k.id = SKINNY_KERNEL_ROWS_FLAT;
  return k;
}

template <int DT>
KernelChoice flat_kernel_m(int M) {
  static_assert(flat_max_m(DT) == 2 || flat_max_m(DT) == 4, "instances for 2 or 4 tokens");
  if (M == 1) return flat_kernel<DT, 1>();
  if (M == 2) return flat_kernel<DT, 2>();
  if constexpr (flat_max_m(DT) == 4) {
    if (M == 3) return flat_kernel<DT, 3>();
    if (M == 4) return flat_kernel<DT, 4>();
  }
  return KernelChoice{};
}

// The flat kernel takes a launch of up to flat_max_m tokens whose linears all
// read a plain x that fits whole in its LDS (every segment of the longest row
// included, for each token).
bool flat_fits(const skinny_linear* const* lin, int count, int M) {
  if (M < 1 || M > flat_max_m(lin[0]->dtype)) return false;
  for (int i = 0; i < count; ++i) {
    const skinny_linear& L = *lin[i];
    if (L.reserved != kActNone) return false;
    const int xc = L.dtype == SKINNY_BF16 ? 1 : 2;
    const int cpr = L.K / (L.dtype == SKINNY_BF16 ? 8 : 16);
    const long long spt = (cpr + kSegChunks - 1) / kSegChunks;
    if (spt * kSegChunks * xc * 16 * M > kRowsXBudget) return false;
  }
  return true;
}

// A workgroup of the flat kernel restages x, between two barriers that drain
// its loads, each time its units move to another linear.  Many linears of
// few rows each make that happen at nearly every unit.  With more than one
// linear the automatic variant therefore asks for at least this many weight
// bytes per workgroup and switch (count - 1 switches at most).  Measured on
// MI355X, launches of eight equal linears against the next automatic
// choice: FP8 4096 x 1536 (14 KB per switch) 21.3 us flat against 12.5 on
// the tile kernel at M = 1 (23.4 against 12.6 at M = 2); bf16 4096 x 1536 at
// M = 2 (28 KB) 26.2 flat against 30.4 on skinny_rows; FP8 3072 x 4096 at
// M = 1 (28 KB) 22.1 flat against 24.4 tiles; the TP=8 layer (143 KB) gains.
constexpr double kFlatMinBytesPerSwitch = 24 * 1024;

// Waves per CU of the flat kernel for this launch, or 0 if it does not take
// it.  Automatic variant: launches under kFlatSmallBytes of weights (16 waves
// per CU) and one-token FP8 launches of at least kFlatLaunchBytes (8), given
// kFlatMinBytesPerSwitch; a forced VECTOR variant takes it for one token
// whenever it fits.
int use_flat(const skinny_linear* const* lin, int count, int M, int requested, int cus) {
  if (requested == SKINNY_VARIANT_MFMA || !flat_fits(lin, count, M)) return 0;
  double bytes = 0;
  for (int i = 0; i < count; ++i)
    bytes += (lin[i]->dtype == SKINNY_BF16 ? 2.0 : 1.0) * lin[i]->N * lin[i]->K;
  const int waves = bytes < kFlatSmallBytes ? kFlatWavesPerCUSmall : kFlatWavesPerCU;
  if (requested == SKINNY_VARIANT_VECTOR) return M == 1 ? waves : 0;
  const double workgroups = (double)cus * waves / kRowsWavesPerBlock;
  if (count > 1 && bytes / (workgroups * (count - 1)) < kFlatMinBytesPerSwitch) return 0;
  if (bytes < kFlatSmallBytes) return waves;
  return M == 1 && lin[0]->dtype != SKINNY_BF16 && bytes >= kFlatLaunchBytes ? waves : 0;
}

KernelChoice pick_flat(int dtype, int M, int waves_per_cu) {
  KernelChoice k = dtype == SKINNY_BF16 ? flat_kernel_m<SKINNY_BF16>(M)
                                        : flat_kernel_m<SKINNY_FP8_BS128>(M);
  k.waves_per_cu = waves_per_cu;
  return k;
}

template <int DT, int MT>
KernelChoice moe_rows_kernel() {
  KernelChoice k = rows_kernel<DT, MT>();
  k.fn = skinny_rows<DT, MT, rows_u(MT, DT), rows_r(MT), kRowsWavesPerBlock, true>;
  return k;
}

template <int DT>
KernelChoice pick_dt(int variant, int M) {
  if (variant == SKINNY_VARIANT_MFMA) return tiles_kernel<DT, kTilesWavesSmall>();
  switch (M) {
    case 1: return rows_kernel<DT, 1>();
    case 2: return rows_kernel<DT, 2>();
    case 3: return rows_kernel<DT, 3>();
    case 4: return rows_kernel<DT, 4>();
    case 5: return rows_kernel<DT, 5>();
    case 6: return rows_kernel<DT, 6>();
    case 7: return rows_kernel<DT, 7>();
    case 8: return rows_kernel<DT, 8>();
    default: return KernelChoice{};
  }
}

KernelChoice pick(int dtype, int variant, int M) {
  return dtype == SKINNY_BF16 ? pick_dt<SKINNY_BF16>(variant, M)
                              : pick_dt<SKINNY_FP8_BS128>(variant, M);
}

// Persistent grid size: every worker must be resident at once for the equal
// shares to finish together, so take what the occupancy query allows for the
// kernel (and its LDS), capped at kTargetRowsWavesPerCU waves per CU.  Query
// results are cached per (device, kernel, LDS bytes).
constexpr int kOccCache = 256;
struct OccEntry {
  int dev;
  const void* fn;
  int lds;
  int blocks_per_cu;
};
OccEntry g_occ[kOccCache];
int g_occ_n = 0;
std::mutex g_occ_mu;

skinny_status blocks_per_cu(const void* fn, int lds, int threads, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
  {
    std::lock_guard<std::mutex> lock(g_occ_mu);
    for (int i = 0; i < g_occ_n; ++i)
      if (g_occ[i].dev == dev && g_occ[i].fn == fn && g_occ[i].lds == lds) {
        *out = g_occ[i].blocks_per_cu;
        return SKINNY_OK;
      }
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) !=
      hipSuccess)
    return SKINNY_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_occ_mu);
  if (g_occ_n < kOccCache) g_occ[g_occ_n++] = OccEntry{dev, fn, lds, n};
  *out = n;
  return SKINNY_OK;
}

// Dynamic LDS above the default limit must be granted per kernel; the
// largest size granted so far is remembered per (device, kernel).
struct LdsEntry {
  int dev;
  const void* fn;
  int bytes;
};
LdsEntry g_lds[kOccCache];
int g_lds_n = 0;

skinny_status ensure_lds(const void* fn, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_occ_mu);
  int slot = -1;
  for (int i = 0; i < g_lds_n; ++i)
    if (g_lds[i].dev == dev && g_lds[i].fn == fn) slot = i;
  if (slot >= 0 && g_lds[slot].bytes >= bytes) return SKINNY_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) !=
      hipSuccess)
    return SKINNY_ERR_HIP;
  if (slot >= 0) g_lds[slot].bytes = bytes;
  else if (g_lds_n < kOccCache) g_lds[g_lds_n++] = LdsEntry{dev, fn, bytes};
  return SKINNY_OK;
}

// Workgroups of the persistent grid: as many as are resident at once.
skinny_status auto_workers(const DeviceInfo& d, const KernelChoice& k, int lds, int* workers) {
  int bpc = 0;
  skinny_status st = blocks_per_cu((const void*)k.fn, lds, 64 * k.wpb, &bpc);
  if (st != SKINNY_OK) return st;
  if (bpc < 1) return SKINNY_ERR_UNSUPPORTED;
  int waves_per_cu = bpc * k.wpb;
  if (waves_per_cu > k.waves_per_cu) waves_per_cu = k.waves_per_cu < k.wpb ? k.wpb : k.waves_per_cu;
  long long g = (long long)d.cus * waves_per_cu;
  if (g > kMaxWaves) g = kMaxWaves;
  *workers = (int)(g / k.wpb);
  return SKINNY_OK;
}

// LDS bytes a main kernel is launched with.  skinny_rows: the x budget plus one
// FP8 scale row per wave; the occupancy query uses the full budget so the grid
// does not depend on the shapes of the launch.
int kernel_lds(const KernelChoice& k, int dtype) {
  if (k.tiles) return tiles_lds(k.wpb);
  if (k.flat) return kRowsXBudget + kFlatYBytes;
  return kRowsXBudget +
         (dtype == SKINNY_FP8_BS128 ? k.wpb * kRowsMaxKBlocks * (int)sizeof(float) : 0);
}

// The 8-wave tile workgroup (one per CU, twice the x window: fewer K-chunks,
// one x copy per CU) for FP8 launches of M >= 2 tokens (bf16: M >= 5) with at least 8 of its
// 128-row groups per CU.  Measured on MI355X against the 4-wave shape: FP8
// TP=1 stack (8-layer launches) +3 / +2 / +6 / +7 / +7% at M = 2 / 4 / 6 / 8 /
// 16 but -3% at M = 1; a single FP8 gate_up (462 groups) -11% at M = 6, the
// fewer, larger units leaving a tail; bf16 stacks within +-3%, the TP=8 layer
// -4 to -6%.
constexpr int kTilesLargeGroupsPerCU = 8;
bool tiles_large(const skinny_linear* const* lin, int count, int M, int cus) {
  // bf16 from M = 5 (its tile launches): with a whole stack in one launch
  // the 8-wave shape gained +1.0 / +1.4 / +1.6% at M = 6 / 8 / 16 (80-layer
  // bf16 stack, same process, outputs bitwise equal).
  if (M < 2 || (lin[0]->dtype == SKINNY_BF16 && M < 5)) return false;
  long long groups = 0;
  for (int i = 0; i < count; ++i)
    groups += (lin[i]->N + kTileRows * kTilesWavesLarge - 1) / (kTileRows * kTilesWavesLarge);
  return groups >= (long long)kTilesLargeGroupsPerCU * cus;
}

// The 8-wave kernel of a large launch: for FP8 linears without an
// activation in the exact-fit layout, whose larger x window leaves K = 8192
// unsplit up to M = 6 (no partial sums, no second pass for those linears).
// Writes that reach memory in the middle of the weight stream cost about ten
// times their bytes in read rate (measured on MI355X with the read probe:
// 0.8% of the bytes written as fp32 stores, 6.88 -> 6.25 TB/s; the same
// stores into a cache-resident region, no loss), and the split's partial
// sums were most of this kernel's writes.  Measured against the padded
// layout, same process, 16-layer FP8 TP=1 launches: +0.3-0.7% at M = 6,
// +0.3% at M = 5 and 8, even at M = 2 and 16.
KernelChoice tiles_large_kernel(const skinny_linear* const* lin, int count) {
  if (lin[0]->dtype == SKINNY_BF16) return tiles_kernel<SKINNY_BF16, kTilesWavesLarge>();
  for (int i = 0; i < count; ++i)
    if (lin[i]->reserved != kActNone) return tiles_kernel<SKINNY_FP8_BS128, kTilesWavesLarge>();
  return tiles_kernel_fit<SKINNY_FP8_BS128>();
}

// Dense tile launches walk their x windows instead of splitting K for them
// from these token counts on.  Measured on MI355X (8-layer TP=1 stack
// launches, walk vs split): bf16 +0.8 / +2.8 / +1.7 / +5.7 / +10.5% at M = 5 /
// 6 / 8 / 10 / 16; FP8 (8-wave) -3.0 / -0.8% at M = 5 / 6, even at 7 and 8,
// +2.4 / +10.4 / +7.0% at 10 / 12 / 16 (the walk costs 1.8% at M = 1).
constexpr int kTilesWalkMinMBf16 = 5;
constexpr int kTilesWalkMinMFp8 = 9;
// The 8-wave FP8 shape walks from 4 tokens: its launches are the large ones
// (a whole stack in one launch), whose split would write partial sums for
// every split linear before one second pass reads them back.  Measured on
// MI355X, 80-layer FP8 TP=1 stack in one launch, walk vs split (same
// process, interleaved; with the exact-fit layout only down walks up to six
// tokens): -0.3 / -0.1 / +0.7 / +1.4 / +2.3 / +6.7 / +10.4% at M = 2 / 3 / 4 /
// 5 / 6 / 7 / 8.
constexpr int kTilesWalkMinMFp8Large = 4;

// K-chunks per linear (either kernel): enough for the x window to fit the LDS
// budget and, when the launch is too small to give every workgroup the
// kernel's units per worker, more - but never fewer segments per chunk than
// a wave keeps in flight.  Assigns the partial slots of the split linears and
// returns how many the launch uses.  The chunk counts only grow with the grid.
long long plan_chunks(LinDesc* lin, int count, int M, int rows, int x_lds_bytes, int G, int dtype,
                      bool tiles, bool fit = false) {
  long long groups = 0;
  for (int i = 0; i < count; ++i) groups += (lin[i].N + rows - 1) / rows;
  const long long want = (long long)(tiles ? kTilesUnitsPerWorker : kRowsUnitsPerWorker) * G;
  const long long par = (want + groups - 1) / groups;
  long long slots = 0;
  for (int i = 0; i < count; ++i) {
    LinDesc& d = lin[i];
    int c, w = 1;
    const bool walk = M >= (dtype == SKINNY_BF16                      ? kTilesWalkMinMBf16
                            : rows == kTileRows * kTilesWavesLarge ? kTilesWalkMinMFp8Large
                                                                   : kTilesWalkMinMFp8);
    if (tiles) tiles_split(dtype, M, d.K, par, x_lds_bytes, walk, &c, &w, fit);
    else c = rows_chunks(dtype, M, d.K, par);
    d.chunks = c;
    d.sub = w;
    d.slot_base = slots;
    if (c > 1) slots += (long long)((d.N + rows - 1) / rows) * c;
  }
  return slots;
}

constexpr size_t kWorkspaceAlign = 256;
size_t align_ws(size_t b) { return (b + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign; }

// Descriptor of linear L as kernel k reads it (chunks, windows and slots unplanned).
LinDesc describe(const skinny_linear& L, const KernelChoice& k) {
  LinDesc d;
  memset(&d, 0, sizeof d);
  d.w = (const u32x4*)L.w;
  d.scale = L.w_scale;
  d.x = (const u32x4*)L.x;
  d.y = (__bf16*)L.y;
  d.N = L.N;
  d.K = L.K;
  d.cpr = L.K / (L.dtype == SKINNY_BF16 ? 8 : 16);
  d.spt = k.tiles ? (d.cpr + kSegChunksT - 1) / kSegChunksT : (d.cpr + kSegChunks - 1) / kSegChunks;
  d.kblocks = (L.K + kScaleBlock - 1) / kScaleBlock;
  d.chunks = 1;
  d.sub = 1;
  d.act = L.reserved;
  return d;
}

int x_lds_budget(const KernelChoice& k) {
  return k.fit ? tiles_x_budget_fit(k.wpb) : k.tiles ? tiles_x_budget(k.wpb) : kRowsXBudget;
}

// Partial-sum bytes one launch of all these linears may use: every kernel
// shape the launch can take, planned at the largest grid any launch runs
// (kMaxWaves waves), which bounds the plan at every smaller grid.
size_t launch_slots_bound(const skinny_linear* const* lin, int count, int M) {
  const int dtype = lin[0]->dtype;
  const bool bf16 = dtype == SKINNY_BF16;
  const KernelChoice shapes[] = {
      pick(dtype, SKINNY_VARIANT_VECTOR, M), pick(dtype, SKINNY_VARIANT_MFMA, M),
      bf16 ? pick_lean(M) : KernelChoice{},
      bf16 ? tiles_kernel<SKINNY_BF16, kTilesWavesLarge>()
           : tiles_kernel<SKINNY_FP8_BS128, kTilesWavesLarge>(),
      bf16 ? KernelChoice{} : tiles_kernel_fit<SKINNY_FP8_BS128>()};
  std::vector<LinDesc> d(count);
  size_t most = 0;
  for (const KernelChoice& k : shapes) {
    if (!k.fn) continue;
    for (int i = 0; i < count; ++i) d[i] = describe(*lin[i], k);
    const long long slots = plan_chunks(d.data(), count, M, k.band_rows, x_lds_budget(k),
                                        kMaxWaves / k.wpb, dtype, k.tiles, k.fit);
    const size_t b = (size_t)slots * M * k.band_rows * sizeof(float);
    if (b > most) most = b;
  }
  return most;
}

// Enqueues one launch over a group of same-dtype linears.  workers = 0 sizes
// the persistent grid from occupancy; otherwise it is the number of waves to
// run (rounded down to whole workgroups, at least one).  The partial sums
// start at ws.  A group of more than SKINNY_MAX_LINEARS_PER_LAUNCH linears
// passes its descriptors in a table placed in the workspace after the partial
// sums, copied there on the stream ahead of the launch.
//
// pairs (optional): for a launch of one linear on the row kernel with K
// unsplit, the kernel also writes each workgroup's greedy pair per token to
// pairs[M][grid] and *pairs_grid is set to the grid; otherwise 0.
skinny_status launch_group(const DeviceInfo& dev, const skinny_linear* const* lin, int count,
                           int M, int variant, int workers, void* ws, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after,
                           ArgmaxPair* pairs = nullptr, int* pairs_grid = nullptr) {
  const int dtype = lin[0]->dtype;
  const int requested = variant;
  if (variant == SKINNY_VARIANT_AUTO) variant = auto_variant(lin, count, M);
  KernelChoice k = pick(dtype, variant, M);
  if (!k.fn) return SKINNY_ERR_UNSUPPORTED;
  if (!k.tiles && rows_lean(lin, count, M)) k = pick_lean(M);
  if (const int fw = use_flat(lin, count, M, requested, dev.cus)) k = pick_flat(dtype, M, fw);
  if (k.tiles && tiles_large(lin, count, M, dev.cus)) k = tiles_large_kernel(lin, count);
  LaunchArgs a;
  memset(&a, 0, sizeof a);
  a.nlin = count;
  a.M = M;
  a.slots = (float*)ws;
  a.band_rows = k.band_rows;
  for (int i = 0; i < count; ++i)
    if (!(k.tiles ? tiles_supported(*lin[i], M) : rows_supported(*lin[i], M)))
      return SKINNY_ERR_UNSUPPORTED;
  const int lds = kernel_lds(k, dtype);
  a.x_lds_bytes = x_lds_budget(k);
  skinny_status st = ensure_lds((const void*)k.fn, lds);
  if (st != SKINNY_OK) return st;
  const bool table = count > SKINNY_MAX_LINEARS_PER_LAUNCH;
  std::vector<LinDesc> big(table ? count : 0);
  LinDesc* D = table ? big.data() : a.lin;
  for (int i = 0; i < count; ++i) D[i] = describe(*lin[i], k);
  int G = workers;
  if (G == 0) {
    st = auto_workers(dev, k, lds, &G);
    if (st != SKINNY_OK) return st;
  } else {
    G = G / k.wpb > 0 ? G / k.wpb : 1;
  }
  if (G > kMaxWaves / k.wpb) G = kMaxWaves / k.wpb;       // the grid the slot bound assumes
  const long long slots = plan_chunks(D, count, M, k.band_rows, a.x_lds_bytes, G, dtype, k.tiles,
                                      k.fit);
  if (k.flat)
    for (int i = 0; i < count; ++i)
      if (D[i].chunks != 1) return SKINNY_ERR_UNSUPPORTED;   // x fits: never split
  G = grid_for_chunks(G, D, count);
  long long S = 0;
  for (int i = 0; i < count; ++i) {
    LinDesc& d = D[i];
    d.unit_base = S;
    S += (long long)((d.N + a.band_rows - 1) / a.band_rows) * d.chunks;
  }
  a.S = S;
  if (G > S) G = (int)S;
  if (G < 1) G = 1;
  a.G = G;
  if (pairs_grid) *pairs_grid = 0;
  if (pairs && !k.tiles && count == 1 && D[0].chunks == 1) {
    a.pairs = pairs;
    if (pairs_grid) *pairs_grid = G;
  }
  if (table) {
    // The table after the partial sums this plan uses (within the bound the
    // workspace size was checked against; checked again here).
    const size_t off = align_ws((size_t)slots * M * k.band_rows * sizeof(float));
    const size_t bytes = (size_t)count * sizeof(LinDesc);
    if (off + bytes > ws_bytes) return SKINNY_ERR_WORKSPACE;
    LinDesc* t = (LinDesc*)((char*)ws + off);
    if (hipMemcpyAsync(t, D, bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
      return SKINNY_ERR_HIP;
    a.table = t;
  }
  if (ev_before && hipEventRecord(ev_before, stream) != hipSuccess) return SKINNY_ERR_HIP;
  hipLaunchKernelGGL(k.fn, dim3(G), dim3(64 * k.wpb), lds, stream, a);
  if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  if (ev_after && hipEventRecord(ev_after, stream) != hipSuccess) return SKINNY_ERR_HIP;
  // Second pass over the split linears (grid row y = linear; unsplit ones return).
  long long most = 0;
  for (int i = 0; i < count; ++i) {
    const long long quads = (long long)M * ((D[i].N + kCombineRows - 1) / kCombineRows);
    if (D[i].chunks > 1 && quads > most) most = quads;
  }
  if (most > 0) {
    const long long cblocks = (most + kCombineThreads - 1) / kCombineThreads;
    hipLaunchKernelGGL(skinny_combine, dim3((unsigned)cblocks, count), dim3(kCombineThreads), 0,
                       stream, a);
    if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  }
  return SKINNY_OK;
}

// Launch groups: the linears of each dtype, in call order, make one launch
// (their descriptors in a table in the workspace when there are more than
// SKINNY_MAX_LINEARS_PER_LAUNCH), or, with max_group = that number, launches
// of at most that many (descriptors in the kernel arguments only: the form
// for streams under graph capture and for the static-buffer entry point).
// Measured on MI355X (16 TP=1 layers, one process, interleaved, 2 to 16
// launches): every launch costs ~9.5 us of ramp and tail (bf16 and FP8 at
// M = 1) to ~16 us (FP8 at M = 6, with its second pass); copying a 5 KB
// table ahead of a launch costs 0-10 us.  A table holds at most
// kTableLinearsMax descriptors (320 KB; the second pass's grid has a row per
// linear), so a call of more linears of one dtype makes more launches.
constexpr int kTableLinearsMax = 4096;
constexpr int kGroupsUncapped = kTableLinearsMax;

int launch_count(const skinny_linear* lin, int count, int max_group) {
  int launches = 0;
  for (int dt = SKINNY_BF16; dt <= SKINNY_FP8_BS128; ++dt) {
    int n = 0;
    for (int i = 0; i < count; ++i) n += lin[i].dtype == dt;
    launches += (n + max_group - 1) / max_group;
  }
  return launches;
}

// Calls fn(group, n) for each launch group (above).  Stops at the first error.
template <typename Fn>
skinny_status for_each_group(const skinny_linear* lin, int count, int max_group, Fn&& fn) {
  std::vector<const skinny_linear*> group;
  group.reserve(count < max_group ? count : max_group);
  for (int dt = SKINNY_BF16; dt <= SKINNY_FP8_BS128; ++dt) {
    group.clear();
    for (int i = 0; i < count; ++i) {
      if (lin[i].dtype != dt) continue;
      group.push_back(&lin[i]);
      if ((int)group.size() == max_group) {
        skinny_status st = fn(group.data(), (int)group.size());
        if (st != SKINNY_OK) return st;
        group.clear();
      }
    }
    if (!group.empty()) {
      skinny_status st = fn(group.data(), (int)group.size());
      if (st != SKINNY_OK) return st;
    }
  }
  return SKINNY_OK;
}

// Workspace a call over these linears needs (pure host arithmetic), never less
// than SKINNY_MIN_WORKSPACE_BYTES: for launches of at most
// SKINNY_MAX_LINEARS_PER_LAUNCH linears (always possible), the largest
// group's partial slots under either variant at the most K-chunks the planner
// may give each linear; unless max_group caps the groups there, also each
// larger group's partial sums (bounded at the largest grid) plus its table.
size_t required_workspace(const skinny_linear* lin, int count, int M,
                          int max_group = kGroupsUncapped) {
  size_t need = SKINNY_MIN_WORKSPACE_BYTES;
  for_each_group(lin, count, SKINNY_MAX_LINEARS_PER_LAUNCH,
                 [&](const skinny_linear* const* g, int n) {
    for (int v = SKINNY_VARIANT_VECTOR; v <= SKINNY_VARIANT_MFMA; ++v) {
      const size_t b = group_slots_bytes(g, n, M, v);
      if (b > need) need = b;
    }
    const size_t b = group_slots_bytes(g, n, M, SKINNY_VARIANT_MFMA, kTilesWavesLarge);
    if (b > need) need = b;
    return SKINNY_OK;
  });
  if (max_group <= SKINNY_MAX_LINEARS_PER_LAUNCH) return need;
  for_each_group(lin, count, max_group, [&](const skinny_linear* const* g, int n) {
    if (n <= SKINNY_MAX_LINEARS_PER_LAUNCH) return SKINNY_OK;
    const size_t b = align_ws(launch_slots_bound(g, n, M)) + (size_t)n * sizeof(LinDesc);
    if (b > need) need = b;
    return SKINNY_OK;
  });
  return need;
}

skinny_status run(const skinny_linear* lin, int count, int M, const skinny_plan* plan,
                  void* ws, size_t ws_bytes, void* stream, void* const* events = nullptr,
                  int event_count = 0, bool allow_act = false, ArgmaxPair* pairs = nullptr,
                  int* pairs_grid = nullptr, int max_group = kGroupsUncapped) {
  if (!lin || count < 1) return SKINNY_ERR_INVALID_ARG;
  if (M < 1 || M > SKINNY_MAX_M) return SKINNY_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    skinny_status st = check_linear(lin[i], M, allow_act);
    if (st != SKINNY_OK) return st;
  }
  int variant = SKINNY_VARIANT_AUTO;
  int waves = 0;
  if (plan) {
    for (int i = 0; i < 5; ++i)
      if (plan->reserved[i] != 0) return SKINNY_ERR_INVALID_ARG;
    variant = plan->variant;
    waves = plan->waves;
    if (variant < SKINNY_VARIANT_AUTO || variant > SKINNY_VARIANT_MFMA) return SKINNY_ERR_INVALID_ARG;
    if (waves < 0 || waves > kMaxWaves) return SKINNY_ERR_INVALID_ARG;
  }
  if (variant == SKINNY_VARIANT_VECTOR && M > kRowsMaxM) return SKINNY_ERR_UNSUPPORTED;
  if (!ws) return SKINNY_ERR_WORKSPACE;
  if (max_group > SKINNY_MAX_LINEARS_PER_LAUNCH) {
    // A table copy recorded into a graph would read this call's host memory
    // at every replay: under capture, launches of kernel-argument size only.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess ||
        cs != hipStreamCaptureStatusNone)
      max_group = SKINNY_MAX_LINEARS_PER_LAUNCH;
  }
  if (ws_bytes < required_workspace(lin, count, M, max_group)) return SKINNY_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return SKINNY_ERR_UNSUPPORTED;
  skinny_status st = check_outputs(lin, count, M, ws, ws_bytes);
  if (st != SKINNY_OK) return st;
  if (events && event_count < 2 * launch_count(lin, count, max_group)) return SKINNY_ERR_INVALID_ARG;
  // A plan the chosen kernel cannot run is rejected before anything is enqueued
  // (AUTO falls back to the matrix-core kernel where the row kernel cannot run).
  for (int i = 0; i < count; ++i) {
    if (variant == SKINNY_VARIANT_VECTOR && !rows_supported(lin[i], M))
      return SKINNY_ERR_UNSUPPORTED;
    if (variant != SKINNY_VARIANT_VECTOR && !tiles_supported(lin[i], M))
      return SKINNY_ERR_UNSUPPORTED;
  }
  DeviceInfo d;
  st = device_info(&d);
  if (st != SKINNY_OK) return st;
  if (!d.gfx950) return SKINNY_ERR_UNSUPPORTED;
  int launch = 0;
  return for_each_group(lin, count, max_group, [&](const skinny_linear* const* g, int n) {
    hipEvent_t before = events ? (hipEvent_t)events[2 * launch] : nullptr;
    hipEvent_t after = events ? (hipEvent_t)events[2 * launch + 1] : nullptr;
    ++launch;
    return launch_group(d, g, n, M, variant, waves, ws, ws_bytes, (hipStream_t)stream, before,
                        after, pairs, pairs_grid);
  });
}

int argmax_slices(int N) { return (N + kArgmaxSlice - 1) / kArgmaxSlice; }

size_t argmax_workspace(int M, int N) {
  const size_t b = (size_t)M * argmax_slices(N) * sizeof(ArgmaxPair);
  return b > SKINNY_MIN_WORKSPACE_BYTES ? b : SKINNY_MIN_WORKSPACE_BYTES;
}

// The greedy pairs the row kernel's epilogue writes: one per workgroup and token.
size_t argmax_fused_workspace(int M) {
  return (size_t)M * (kMaxWaves / kRowsWavesPerBlock) * sizeof(ArgmaxPair);
}

skinny_status launch_argmax(const void* y, int M, int N, int* idx, void* ws, hipStream_t stream) {
  const int slices = argmax_slices(N);
  ArgmaxPair* pairs = (ArgmaxPair*)ws;
  if (N % 8 == 0 && aligned(y, 16))
    hipLaunchKernelGGL(skinny_argmax_slices<true>, dim3(slices, M), dim3(kArgmaxThreads), 0,
                       stream, (const __bf16*)y, N, pairs);
  else
    hipLaunchKernelGGL(skinny_argmax_slices<false>, dim3(slices, M), dim3(kArgmaxThreads), 0,
                       stream, (const __bf16*)y, N, pairs);
  if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  hipLaunchKernelGGL(skinny_argmax_rows, dim3(M), dim3(kArgmaxThreads), 0, stream,
                     (const ArgmaxPair*)pairs, slices, N, idx);
  return hipGetLastError() == hipSuccess ? SKINNY_OK : SKINNY_ERR_HIP;
}

// y, idx and the workspace: present, aligned, within limits and disjoint.
skinny_status check_argmax(const void* y, int M, int N, const int* idx, const void* ws,
                           size_t ws_bytes) {
  if (!y || !idx || M < 1 || M > SKINNY_MAX_M || N < 1) return SKINNY_ERR_INVALID_ARG;
  if (argmax_slices(N) > kArgmaxMaxSlices) return SKINNY_ERR_UNSUPPORTED;
  if (!aligned(y, 2) || !aligned(idx, 4)) return SKINNY_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < argmax_workspace(M, N)) return SKINNY_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return SKINNY_ERR_UNSUPPORTED;
  const Range yr{(uintptr_t)y, (uintptr_t)y + (size_t)M * N * 2};
  const Range ir{(uintptr_t)idx, (uintptr_t)idx + (size_t)M * 4};
  const Range wr{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  if (overlap(yr, ir) || overlap(yr, wr) || overlap(ir, wr)) return SKINNY_ERR_INVALID_ARG;
  return SKINNY_OK;
}

// The two linears of a gated MLP: gate_up writes [gate | up] into the
// intermediate buffer `gu`, down reads it through the fused activation.
size_t mlp_gu_bytes(const skinny_mlp& P, int M) {
  const size_t b = (size_t)M * 2 * P.I * 2;
  return (b + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign;
}

void mlp_linears(const skinny_mlp& P, void* gu, skinny_linear* gate_up, skinny_linear* down) {
  memset(gate_up, 0, sizeof *gate_up);
  gate_up->dtype = P.dtype;
  gate_up->N = 2 * P.I;
  gate_up->K = P.H;
  gate_up->w = P.w_gate_up;
  gate_up->w_scale = P.s_gate_up;
  gate_up->x = P.x;
  gate_up->y = gu;
  memset(down, 0, sizeof *down);
  down->dtype = P.dtype;
  down->N = P.H;
  down->K = P.I;
  down->reserved = kActSwiGLU;
  down->w = P.w_down;
  down->w_scale = P.s_down;
  down->x = gu;
  down->y = P.y;
}

size_t mlp_workspace(const skinny_mlp& P, int M) {
  // Shapes only: stand-in non-null pointers keep the planner's checks quiet.
  skinny_linear g, d;
  mlp_linears(P, (void*)kWorkspaceAlign, &g, &d);
  const size_t a = required_workspace(&g, 1, M);
  const size_t b = required_workspace(&d, 1, M);
  return mlp_gu_bytes(P, M) + (a > b ? a : b);
}

// ---------------------------------------------------------------------------
// Mixture-of-experts launches (skinny_tiles or skinny_rows in its MoE form).

// An MoE launch whose unsplit units would keep fewer than 1/kMoeSplitBelow of
// the workers busy is cut into K-chunks for parallelism; otherwise each unit
// walks its x windows in turn and no second pass runs.  Measured on MI355X
// (verify step, 8 experts, top 2): splitting K for parallelism as the dense
// planner does cost 1-9% at 1, 6 and 16 tokens, the second pass included.
constexpr int kMoeSplitBelow = 8;

struct MoePlan {
  int cap;               // routes per slice: the token count
  int routes;
  int active;            // experts the routes can reach: min(E, routes)
  int max_slices;
  int groups;            // row groups per expert
  bool rows;             // skinny_rows (unsplit K), else skinny_tiles
  int wpb;               // workgroup shape (waves)
  int table_lds;         // LDS bytes of the slice table
  int x_budget;          // LDS bytes left for x; the table follows them
  size_t table_bytes;    // workspace bytes of the table copy (256-aligned)
  bool ks = false;       // skinny_tiles' K-split form (16-row groups)
  int band = 0;          // rows per row group
};

// Slices: an expert with c routes makes ceil(c / cap) of them, so n active
// experts over `routes` routes make at most n + (routes - n) / cap, which
// grows with n (<= min(E, routes)).
MoePlan moe_plan_base(const skinny_experts& ex, int T, int topk) {
  MoePlan p;
  p.cap = T;
  p.routes = T * topk;
  p.active = ex.E < p.routes ? ex.E : p.routes;
  p.max_slices = p.active + (p.routes - p.active) / p.cap;
  const int tb = 2 * 4 + p.max_slices * (2 * 4 + 2 * kMoeMaxCap) + p.routes;
  p.table_lds = (tb + 15) / 16 * 16;
  const size_t tg = (size_t)(1 + p.max_slices * (1 + kMoeMaxCap)) * sizeof(int);
  p.table_bytes = (tg + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign;
  return p;
}

MoePlan moe_plan_for(const skinny_experts& ex, int T, int topk, int wpb, bool ks = false) {
  MoePlan p = moe_plan_base(ex, T, topk);
  p.rows = false;
  p.wpb = wpb;
  p.ks = ks;
  p.band = ks ? kTileRows : kTileRows * wpb;
  p.groups = (ex.N + p.band - 1) / p.band;
  p.x_budget = (ks ? tiles_x_budget_ks(wpb) : tiles_x_budget(wpb)) - p.table_lds;
  return p;
}

// The row kernel's plan: the table takes the top of its x region (the slice
// setup's 2 KB of scratch at the bottom stays clear of it); usable only if the
// whole of K fits the rest and a row spans at least kMoeRowsMinSegs 1 KB
// segments (a wave's whole unit is one row: shorter rows leave too few loads
// in flight per unit).
constexpr int kMoeRowsMinSegs = 4;
MoePlan moe_plan_rows(const skinny_experts& ex, int T, int topk) {
  MoePlan p = moe_plan_base(ex, T, topk);
  p.wpb = kRowsWavesPerBlock;
  p.band = kRowsWavesPerBlock * rows_r(T);
  p.groups = (ex.N + p.band - 1) / p.band;
  p.x_budget = kRowsXBudget - p.table_lds;
  const int cpr = ex.K / (ex.dtype == SKINNY_BF16 ? 8 : 16);
  p.rows = T <= kRowsMaxM && p.x_budget >= 2 * kMoeMaxRoutes * (int)sizeof(int) &&
           (cpr + kSegChunks - 1) / kSegChunks >= kMoeRowsMinSegs &&
           (ex.dtype == SKINNY_BF16 || (ex.K + kScaleBlock - 1) / kScaleBlock <= kRowsMaxKBlocks) &&
           rows_lds_chunks(ex.dtype, T, ex.K, p.x_budget) == 1;
  return p;
}

// The 8-wave workgroup (twice the x window) when the 4-wave one would walk at
// least kMoeLargeWindows x windows per unit.  Measured on MI355X (verify step,
// 8 experts, top 2): 16 tokens +13% (FP8) and +4% (bf16); 6 tokens even; one
// token 27-37% slower (its few units leave most of the half-as-many
// workgroups idle).
constexpr int kMoeLargeWindows = 4;
// The row kernel for one-token slices: its 8-row units give the few chosen
// experts' rows to many more workgroups than the tile kernel's 64-row units.
// Measured on MI355X (verify step, 8 experts, top 2, one token): gate_up
// (K = 4096) 11.8 -> 11.0 us FP8 and 15.9 -> 13.3 us bf16; the down linear
// (K = 1536: 1.5 or 3 KB rows) 8.7 -> 13.3 and 10.1 -> 12.0 us, hence the
// minimum row length; two-token slices 15.2 -> 23.0 and 23.2 -> 24.6 us on
// gate_up (the two-token row instance's registers leave one workgroup per CU).
constexpr int kMoeRowsMaxCap = 1;
// One-token slices whose rows are too short for the row kernel take the tile
// kernel's K-split form: 16-row units (four times as many as 64-row ones,
// every workgroup busy) whose few segments all waves load at once.  Measured
// on MI355X (verify step, 8 experts, top 2, one token, down: K = 1536):
// 7.87 -> 7.68 us FP8, 10.09 -> 9.13 us bf16.  For gate_up (K = 4096) it was
// no faster than the row kernel (FP8 11.07 -> 10.95, bf16 13.33 -> 13.74 us),
// and at two or more tokens no faster than one tile per wave.
constexpr int kMoeKsMaxCap = 1;
MoePlan moe_plan(const skinny_experts& ex, int T, int topk) {
  if (T <= kMoeRowsMaxCap) {
    const MoePlan r = moe_plan_rows(ex, T, topk);
    if (r.rows) return r;
  }
  if (T <= kMoeKsMaxCap) return moe_plan_for(ex, T, topk, kTilesWavesSmall, true);
  const MoePlan p = moe_plan_for(ex, T, topk, kTilesWavesSmall);
  if (tiles_lds_chunks(ex.dtype, p.cap, ex.K, p.x_budget) >= kMoeLargeWindows)
    return moe_plan_for(ex, T, topk, kTilesWavesLarge);
  return p;
}

size_t moe_workspace(const skinny_experts& ex, const MoePlan& p) {
  const int c = p.rows ? 1 : tiles_chunks(ex.dtype, p.cap, ex.K, 1LL << 40, p.x_budget);
  const size_t slots = c > 1 ? (size_t)p.max_slices * p.groups * c * p.cap * p.band * sizeof(float)
                             : 0;
  const size_t b = p.table_bytes + slots;
  return b > SKINNY_MIN_WORKSPACE_BYTES ? b : SKINNY_MIN_WORKSPACE_BYTES;
}

skinny_status check_experts(const skinny_experts* ex, int T, int topk, int flags) {
  if (!ex) return SKINNY_ERR_INVALID_ARG;
  if (ex->dtype != SKINNY_BF16 && ex->dtype != SKINNY_FP8_BS128) return SKINNY_ERR_INVALID_ARG;
  if (ex->E < 1 || ex->N < 1 || ex->K < 1 || !ex->w) return SKINNY_ERR_INVALID_ARG;
  if ((ex->dtype == SKINNY_FP8_BS128) != (ex->w_scale != nullptr)) return SKINNY_ERR_INVALID_ARG;
  if (T < 1 || T > SKINNY_MAX_M || topk < 1 || topk > SKINNY_MAX_TOPK) return SKINNY_ERR_INVALID_ARG;
  if (flags & ~(SKINNY_MOE_X_PER_ROUTE | SKINNY_MOE_SWIGLU)) return SKINNY_ERR_INVALID_ARG;
  if (ex->K % (ex->dtype == SKINNY_BF16 ? 8 : 16) != 0) return SKINNY_ERR_UNSUPPORTED;
  if (ex->N > (1 << 26) || ex->K > (1 << 28)) return SKINNY_ERR_UNSUPPORTED;
  if (!aligned(ex->w, 16) || (ex->w_scale && !aligned(ex->w_scale, 4))) return SKINNY_ERR_UNSUPPORTED;
  const MoePlan p = moe_plan(*ex, T, topk);
  if (p.routes > kMoeMaxRoutes || p.cap > kMoeMaxCap) return SKINNY_ERR_UNSUPPORTED;
  if (!p.rows && tiles_lds_chunks(ex->dtype, p.cap, ex->K, p.x_budget) < 1)
    return SKINNY_ERR_UNSUPPORTED;
  return SKINNY_OK;
}

skinny_status moe_run(const skinny_experts* ex, const void* x, const int* ids, int T, int topk,
                      int flags, void* y, void* ws, size_t ws_bytes, void* stream,
                      void* const* events) {
  skinny_status st = check_experts(ex, T, topk, flags);
  if (st != SKINNY_OK) return st;
  if (!x || !ids || !y) return SKINNY_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4)) return SKINNY_ERR_UNSUPPORTED;
  const MoePlan p = moe_plan(*ex, T, topk);
  if (!ws) return SKINNY_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return SKINNY_ERR_UNSUPPORTED;
  if (ws_bytes < moe_workspace(*ex, p)) return SKINNY_ERR_WORKSPACE;
  const int dtype = ex->dtype;
  const size_t eb = dtype == SKINNY_BF16 ? 2 : 1;
  const size_t nb = (size_t)((ex->N + 127) / 128) * ((ex->K + 127) / 128);
  const int xrows = flags & SKINNY_MOE_X_PER_ROUTE ? p.routes : T;
  const Range yr{(uintptr_t)y, (uintptr_t)y + (size_t)p.routes * ex->N * 2};
  const Range xr{(uintptr_t)x,
                 (uintptr_t)x + (size_t)xrows * ex->K * 2 * (flags & SKINNY_MOE_SWIGLU ? 2 : 1)};
  const Range ir{(uintptr_t)ids, (uintptr_t)ids + (size_t)p.routes * 4};
  const Range wr{(uintptr_t)ex->w, (uintptr_t)ex->w + (size_t)ex->E * ex->N * ex->K * eb};
  const Range sr{(uintptr_t)ex->w_scale,
                 (uintptr_t)ex->w_scale + (ex->w_scale ? (size_t)ex->E * nb * 4 : 0)};
  const Range kr{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  if (overlap(yr, xr) || overlap(yr, ir) || overlap(yr, wr) || overlap(yr, sr) ||
      overlap(yr, kr) || overlap(kr, xr) || overlap(kr, ir) || overlap(kr, wr) || overlap(kr, sr))
    return SKINNY_ERR_INVALID_ARG;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != SKINNY_OK) return st;
  if (!dev.gfx950) return SKINNY_ERR_UNSUPPORTED;

  KernelChoice k;
  if (p.rows) {
    static_assert(kMoeRowsMaxCap == 1, "row-kernel MoE instances");
    k = dtype == SKINNY_BF16 ? moe_rows_kernel<SKINNY_BF16, 1>()
                             : moe_rows_kernel<SKINNY_FP8_BS128, 1>();
  } else {
    if (p.ks)
      k.fn = dtype == SKINNY_BF16 ? skinny_tiles<SKINNY_BF16, kTilesWavesSmall, true, true>
                                  : skinny_tiles<SKINNY_FP8_BS128, kTilesWavesSmall, true, true>;
    else if (p.wpb == kTilesWavesLarge)
      k.fn = dtype == SKINNY_BF16 ? skinny_tiles<SKINNY_BF16, kTilesWavesLarge, true>
                                  : skinny_tiles<SKINNY_FP8_BS128, kTilesWavesLarge, true>;
    else
      k.fn = dtype == SKINNY_BF16 ? skinny_tiles<SKINNY_BF16, kTilesWavesSmall, true>
                                  : skinny_tiles<SKINNY_FP8_BS128, kTilesWavesSmall, true>;
    k.band_rows = p.band;
    k.wpb = p.wpb;
    k.tiles = true;
  }
  const int lds = kernel_lds(k, dtype);
  st = ensure_lds((const void*)k.fn, lds);
  if (st != SKINNY_OK) return st;
  int G = 0;
  st = auto_workers(dev, k, lds, &G);
  if (st != SKINNY_OK) return st;

  LaunchArgs a;
  memset(&a, 0, sizeof a);
  a.nlin = 1;
  a.M = p.cap;
  a.band_rows = k.band_rows;
  a.x_lds_bytes = p.rows ? kRowsXBudget : p.x_budget;
  LinDesc& d = a.lin[0];
  d.w = (const u32x4*)ex->w;
  d.scale = ex->w_scale;
  d.x = (const u32x4*)x;
  d.y = (__bf16*)y;
  d.N = ex->N;
  d.K = ex->K;
  d.cpr = ex->K / (dtype == SKINNY_BF16 ? 8 : 16);
  d.spt = p.rows ? (d.cpr + kSegChunks - 1) / kSegChunks : (d.cpr + kSegChunksT - 1) / kSegChunksT;
  d.kblocks = (ex->K + kScaleBlock - 1) / kScaleBlock;
  d.act = flags & SKINNY_MOE_SWIGLU ? kActSwiGLU : kActNone;
  // K-chunks and x windows, planned for `active` experts' row groups.
  const long long units = (long long)kMoeSplitBelow * p.active * p.groups;
  d.chunks = 1;
  d.sub = 1;
  if (!p.rows)
    tiles_split(dtype, p.cap, ex->K, (G + units - 1) / units, p.x_budget, true, &d.chunks, &d.sub);
  MoeArgs& mo = a.moe;
  mo.ids = ids;
  mo.table = d.chunks > 1 ? (int*)ws : nullptr;
  mo.w_stride = (long long)ex->N * d.cpr;
  mo.s_stride = dtype == SKINNY_BF16 ? 0 : (long long)nb;
  mo.E = ex->E;
  mo.routes = p.routes;
  mo.topk = topk;
  mo.cap = p.cap;
  mo.per_route = flags & SKINNY_MOE_X_PER_ROUTE ? 1 : 0;
  mo.max_slices = p.max_slices;
  mo.units_per_slice = p.groups * d.chunks;
  // The tile kernel's LDS: x, the W tiles, (K-split: the partial tiles,)
  // then the table.
  mo.table_lds = p.rows ? p.x_budget
                        : p.x_budget + tiles_w_bytes(p.wpb) + (p.ks ? tiles_red_bytes(p.wpb) : 0);
  a.slots = (float*)((char*)ws + p.table_bytes);
  a.S = (long long)p.max_slices * mo.units_per_slice;
  G = grid_for_chunks(G, a.lin, a.nlin);
  if (G > a.S) G = (int)a.S;
  a.G = G;
  hipStream_t s = (hipStream_t)stream;
  if (events && hipEventRecord((hipEvent_t)events[0], s) != hipSuccess) return SKINNY_ERR_HIP;
  hipLaunchKernelGGL(k.fn, dim3(G), dim3(64 * k.wpb), lds, s, a);
  if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  if (events && hipEventRecord((hipEvent_t)events[1], s) != hipSuccess) return SKINNY_ERR_HIP;
  if (d.chunks > 1) {
    const long long quads = (long long)p.cap * ((ex->N + kCombineRows - 1) / kCombineRows);
    const long long cblocks = (quads + kCombineThreads - 1) / kCombineThreads;
    hipLaunchKernelGGL(skinny_moe_combine, dim3((unsigned)cblocks, p.max_slices),
                       dim3(kCombineThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  }
  return SKINNY_OK;
}

// ---------------------------------------------------------------------------
// Split-K partial sums without a caller's workspace: a static device buffer
// of SKINNY_STATIC_SCRATCH_BYTES that every GPU the library runs on holds
// from the code object's load until the process ends.  In host code the
// array's name is not a device address: its address on a device comes from
// hipGetSymbolAddress with that device current, resolved on the first call
// on the device and kept per device; only that address is passed to kernels.
// The partial-sum slots are written before the second pass reads them, so
// the buffer needs no clearing between calls.
static __device__ __align__(256) unsigned char scratch[SKINNY_STATIC_SCRATCH_BYTES];
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

skinny_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SKINNY_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKINNY_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SKINNY_OK;
}

}  // namespace

extern "C" {

size_t skinny_workspace_bytes(int dtype, int M, int N, int K) {
  if (dtype != SKINNY_BF16 && dtype != SKINNY_FP8_BS128) return 0;
  if (M < 1 || M > SKINNY_MAX_M || N < 1 || K < 1) return 0;
  skinny_linear L;
  memset(&L, 0, sizeof L);
  L.dtype = dtype;
  L.N = N;
  L.K = K;
  return required_workspace(&L, 1, M);
}

size_t skinny_stack_workspace_bytes(const skinny_linear* linears, int count, int M) {
  if (!linears || count < 1 || M < 1 || M > SKINNY_MAX_M) return 0;
  for (int i = 0; i < count; ++i) {
    const skinny_linear& L = linears[i];
    if (L.dtype != SKINNY_BF16 && L.dtype != SKINNY_FP8_BS128) return 0;
    if (L.N < 1 || L.K < 1) return 0;
  }
  return required_workspace(linears, count, M);
}

skinny_status skinny_gemm_bf16(const void* x, const void* w, void* y, int M, int N, int K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  skinny_linear L;
  memset(&L, 0, sizeof L);
  L.dtype = SKINNY_BF16;
  L.N = N;
  L.K = K;
  L.w = w;
  L.x = x;
  L.y = y;
  return run(&L, 1, M, nullptr, workspace, workspace_bytes, stream);
}

skinny_status skinny_gemm_fp8_bs128(const void* x, const void* w_fp8, const float* w_scale,
                                    void* y, int M, int N, int K, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  skinny_linear L;
  memset(&L, 0, sizeof L);
  L.dtype = SKINNY_FP8_BS128;
  L.N = N;
  L.K = K;
  L.w = w_fp8;
  L.w_scale = w_scale;
  L.x = x;
  L.y = y;
  if (!w_scale) return SKINNY_ERR_INVALID_ARG;
  return run(&L, 1, M, nullptr, workspace, workspace_bytes, stream);
}

skinny_status decode_linear_stack(const skinny_linear* linears, int count, int M,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return run(linears, count, M, nullptr, workspace, workspace_bytes, stream);
}

skinny_status decode_linear_stack_noalloc(const skinny_linear* linears, int count, int M,
                                          void* stream) {
  // Argument and size errors are returned before any device call.
  if (!linears || count < 1 || M < 1 || M > SKINNY_MAX_M) return SKINNY_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    skinny_status st = check_linear(linears[i], M);
    if (st != SKINNY_OK) return st;
  }
  // Its launches hold at most SKINNY_MAX_LINEARS_PER_LAUNCH linears each.
  if (required_workspace(linears, count, M, SKINNY_MAX_LINEARS_PER_LAUNCH) >
      (size_t)SKINNY_STATIC_SCRATCH_BYTES)
    return SKINNY_ERR_WORKSPACE;
  DeviceInfo d;
  skinny_status st = device_info(&d);
  if (st != SKINNY_OK) return st;
  if (!d.gfx950) return SKINNY_ERR_UNSUPPORTED;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SKINNY_OK) return st;
  // Descriptors in the kernel arguments only: nothing to copy into the buffer.
  return run(linears, count, M, nullptr, ws, SKINNY_STATIC_SCRATCH_BYTES, stream, nullptr, 0,
             false, nullptr, nullptr, SKINNY_MAX_LINEARS_PER_LAUNCH);
}

skinny_status skinny_linear_run(const skinny_linear* linears, int count, int M,
                                const skinny_plan* plan, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return run(linears, count, M, plan, workspace, workspace_bytes, stream);
}

int skinny_band_rows(int dtype, int variant, int M) {
  if (dtype != SKINNY_BF16 && dtype != SKINNY_FP8_BS128) return 0;
  if (M < 1 || M > SKINNY_MAX_M) return 0;
  if (variant != SKINNY_VARIANT_VECTOR && variant != SKINNY_VARIANT_MFMA) return 0;
  return pick(dtype, variant, M).band_rows;
}

int skinny_launch_count(const skinny_linear* linears, int count) {
  if (!linears || count < 1) return 0;
  for (int i = 0; i < count; ++i)
    if (linears[i].dtype != SKINNY_BF16 && linears[i].dtype != SKINNY_FP8_BS128) return 0;
  return launch_count(linears, count, kGroupsUncapped);
}

skinny_status skinny_linear_run_timed(const skinny_linear* linears, int count, int M,
                                      const skinny_plan* plan, void* const* events,
                                      int event_count, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!events) return SKINNY_ERR_INVALID_ARG;
  return run(linears, count, M, plan, workspace, workspace_bytes, stream, events, event_count);
}

skinny_status skinny_plan_query(const skinny_linear* linears, int count, int M,
                                skinny_plan* out) {
  if (!linears || count < 1 || !out) return SKINNY_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    skinny_status st = check_linear(linears[i], M);
    if (st != SKINNY_OK) return st;
  }
  // The plan of the first launch group: every linear of the first one's dtype.
  std::vector<const skinny_linear*> lins;
  for (int i = 0; i < count; ++i)
    if (linears[i].dtype == linears[0].dtype) lins.push_back(&linears[i]);
  const skinny_linear* const* group = lins.data();
  const int n = (int)lins.size();
  DeviceInfo d;
  skinny_status st = device_info(&d);
  if (st != SKINNY_OK) return st;
  memset(out, 0, sizeof *out);
  out->variant = auto_variant(group, n, M);
  KernelChoice k = pick(linears[0].dtype, out->variant, M);
  if (!k.fn) return SKINNY_ERR_INVALID_ARG;
  if (!k.tiles && rows_lean(group, n, M)) k = pick_lean(M);
  if (const int fw = use_flat(group, n, M, SKINNY_VARIANT_AUTO, d.cus)) {
    out->variant = SKINNY_VARIANT_VECTOR;
    k = pick_flat(linears[0].dtype, M, fw);
  }
  if (k.tiles && tiles_large(group, n, M, d.cus)) k = tiles_large_kernel(group, n);
  out->kernel = k.id;
  const int lds = kernel_lds(k, linears[0].dtype);
  st = ensure_lds((const void*)k.fn, lds);
  if (st != SKINNY_OK) return st;
  int workers = 0;
  st = auto_workers(d, k, lds, &workers);
  out->waves = workers * k.wpb;
  return st;
}

size_t skinny_argmax_workspace_bytes(int M, int N) {
  if (M < 1 || M > SKINNY_MAX_M || N < 1) return 0;
  return argmax_workspace(M, N);
}

skinny_status skinny_argmax_bf16(const void* y, int M, int N, int* idx, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  skinny_status st = check_argmax(y, M, N, idx, workspace, workspace_bytes);
  if (st != SKINNY_OK) return st;
  DeviceInfo d;
  st = device_info(&d);
  if (st != SKINNY_OK) return st;
  if (!d.gfx950) return SKINNY_ERR_UNSUPPORTED;
  return launch_argmax(y, M, N, idx, workspace, (hipStream_t)stream);
}

size_t skinny_lm_head_workspace_bytes(const skinny_linear* head, int M) {
  if (!head || M < 1 || M > SKINNY_MAX_M) return 0;
  const size_t lin = skinny_stack_workspace_bytes(head, 1, M);
  if (lin == 0) return 0;
  size_t am = argmax_workspace(M, head->N);
  if (argmax_fused_workspace(M) > am) am = argmax_fused_workspace(M);
  return lin > am ? lin : am;
}

skinny_status skinny_lm_head_argmax(const skinny_linear* head, int M, int* next_token,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!head) return SKINNY_ERR_INVALID_ARG;
  skinny_status st = check_linear(*head, M);
  if (st != SKINNY_OK) return st;
  st = check_argmax(head->y, M, head->N, next_token, workspace, workspace_bytes);
  if (st != SKINNY_OK) return st;
  // next_token must not overlap any operand of the linear either.
  const Range ir{(uintptr_t)next_token, (uintptr_t)next_token + (size_t)M * 4};
  const size_t wbytes = (size_t)head->N * head->K * (head->dtype == SKINNY_BF16 ? 2 : 1);
  const Range others[] = {
      {(uintptr_t)head->x, (uintptr_t)head->x + (size_t)M * head->K * 2},
      {(uintptr_t)head->w, (uintptr_t)head->w + wbytes}};
  for (const Range& r : others)
    if (overlap(ir, r)) return SKINNY_ERR_INVALID_ARG;
  if (head->w_scale) {
    const size_t sb = (size_t)((head->N + 127) / 128) * ((head->K + 127) / 128) * 4;
    if (overlap(ir, Range{(uintptr_t)head->w_scale, (uintptr_t)head->w_scale + sb}))
      return SKINNY_ERR_INVALID_ARG;
  }
  if (workspace_bytes < argmax_fused_workspace(M)) return SKINNY_ERR_WORKSPACE;
  // On the row kernel with K unsplit, the linear's launch also leaves each
  // workgroup's greedy pair per token at the start of the workspace (it needs
  // no partial sums then), and one pass reduces them.  Otherwise the
  // workspace serves the linear's partial sums, then (stream order: the
  // linear is done with them) the two argmax passes over the logits.
  int grid = 0;
  st = run(head, 1, M, nullptr, workspace, workspace_bytes, stream, nullptr, 0, false,
           (ArgmaxPair*)workspace, &grid);
  if (st != SKINNY_OK) return st;
  if (grid == 0) return launch_argmax(head->y, M, head->N, next_token, workspace, (hipStream_t)stream);
  hipLaunchKernelGGL(skinny_argmax_rows, dim3(M), dim3(kArgmaxThreads), 0, (hipStream_t)stream,
                     (const ArgmaxPair*)workspace, grid, head->N, next_token);
  return hipGetLastError() == hipSuccess ? SKINNY_OK : SKINNY_ERR_HIP;
}

size_t skinny_mlp_workspace_bytes(const skinny_mlp* mlp, int M) {
  if (!mlp || M < 1 || M > SKINNY_MAX_M || mlp->H < 1 || mlp->I < 1) return 0;
  if (mlp->dtype != SKINNY_BF16 && mlp->dtype != SKINNY_FP8_BS128) return 0;
  if ((long long)2 * mlp->I > (1 << 26)) return 0;
  return mlp_workspace(*mlp, M);
}

skinny_status skinny_mlp_swiglu(const skinny_mlp* mlp, int M, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!mlp || mlp->reserved != 0) return SKINNY_ERR_INVALID_ARG;
  const skinny_mlp& P = *mlp;
  if (M < 1 || M > SKINNY_MAX_M || P.H < 1 || P.I < 1) return SKINNY_ERR_INVALID_ARG;
  if (P.dtype != SKINNY_BF16 && P.dtype != SKINNY_FP8_BS128) return SKINNY_ERR_INVALID_ARG;
  if ((long long)2 * P.I > (1 << 26)) return SKINNY_ERR_UNSUPPORTED;
  if (!workspace) return SKINNY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SKINNY_ERR_UNSUPPORTED;
  if (workspace_bytes < mlp_workspace(P, M)) return SKINNY_ERR_WORKSPACE;
  skinny_linear g, d;
  mlp_linears(P, workspace, &g, &d);
  skinny_status st = check_linear(g, M);
  if (st == SKINNY_OK) st = check_linear(d, M, true);
  if (st != SKINNY_OK) return st;
  // y must not overlap the MLP's input, weights or the workspace; x must not
  // overlap the workspace (the intermediate is written there).
  const Range yr{(uintptr_t)P.y, (uintptr_t)P.y + (size_t)M * P.H * 2};
  const Range xr{(uintptr_t)P.x, (uintptr_t)P.x + (size_t)M * P.H * 2};
  const Range wr{(uintptr_t)workspace, (uintptr_t)workspace + workspace_bytes};
  const size_t eb = P.dtype == SKINNY_BF16 ? 2 : 1;
  const Range gw{(uintptr_t)P.w_gate_up, (uintptr_t)P.w_gate_up + (size_t)2 * P.I * P.H * eb};
  const Range dw{(uintptr_t)P.w_down, (uintptr_t)P.w_down + (size_t)P.H * P.I * eb};
  if (overlap(yr, xr) || overlap(yr, wr) || overlap(yr, gw) || overlap(yr, dw) || overlap(xr, wr))
    return SKINNY_ERR_INVALID_ARG;
  if (P.s_gate_up) {
    const size_t sb = (size_t)((2 * P.I + 127) / 128) * ((P.H + 127) / 128) * 4;
    if (overlap(yr, Range{(uintptr_t)P.s_gate_up, (uintptr_t)P.s_gate_up + sb}))
      return SKINNY_ERR_INVALID_ARG;
  }
  if (P.s_down) {
    const size_t sb = (size_t)((P.H + 127) / 128) * ((P.I + 127) / 128) * 4;
    if (overlap(yr, Range{(uintptr_t)P.s_down, (uintptr_t)P.s_down + sb}))
      return SKINNY_ERR_INVALID_ARG;
  }
  // gate_up, then down through the fused activation; the partial-sum slots
  // follow the intermediate in the workspace.
  const size_t gub = mlp_gu_bytes(P, M);
  void* slots = (char*)workspace + gub;
  st = run(&g, 1, M, nullptr, slots, workspace_bytes - gub, stream);
  if (st != SKINNY_OK) return st;
  return run(&d, 1, M, nullptr, slots, workspace_bytes - gub, stream, nullptr, 0, true);
}

size_t skinny_moe_workspace_bytes(const skinny_experts* experts, int T, int topk, int flags) {
  if (check_experts(experts, T, topk, flags) != SKINNY_OK) return 0;
  return moe_workspace(*experts, moe_plan(*experts, T, topk));
}

skinny_status skinny_moe_linear(const skinny_experts* experts, const void* x, const int* ids,
                                int T, int topk, int flags, void* y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return moe_run(experts, x, ids, T, topk, flags, y, workspace, workspace_bytes, stream, nullptr);
}

skinny_status skinny_moe_linear_timed(const skinny_experts* experts, const void* x,
                                      const int* ids, int T, int topk, int flags, void* y,
                                      void* const* events, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!events) return SKINNY_ERR_INVALID_ARG;
  return moe_run(experts, x, ids, T, topk, flags, y, workspace, workspace_bytes, stream, events);
}

// ---------------------------------------------------------------------------
// The experts' gated MLP (skinny_moe_mlp_swiglu).  Workspace: kMoeMlpCtrBytes
// of counters (zero before the first call, left zero by every call), the
// gate_up outputs [T * topk][2I] bf16, then what the two skinny_moe_linear
// launches of the general path need.
constexpr int kMoeMlpMaxGrid = 1 << 20;
constexpr size_t kMoeMlpCtrBytes = 256;
static_assert(kMoeMlpCtrBytes == SKINNY_MOE_MLP_COUNTER_BYTES, "the header's layout");
constexpr int kMoeMlpSegs = 2;           // 1 KB segments per slot of the one-token kernel
std::atomic<long long> g_moe_mlp_spin{1LL << 22};

// The gate_up outputs: bf16, or (one launch) 64-bit words of two bf16 and a tag.
size_t moe_mlp_gu_bytes(const skinny_experts& gu, int T, int topk) {
  return ((size_t)T * topk * gu.N * 4 + 255) / 256 * 256;
}

skinny_status check_moe_mlp(const skinny_experts* gu, const skinny_experts* dn, int T, int topk) {
  skinny_status st = check_experts(gu, T, topk, 0);
  if (st != SKINNY_OK) return st;
  st = check_experts(dn, T, topk, SKINNY_MOE_X_PER_ROUTE | SKINNY_MOE_SWIGLU);
  if (st != SKINNY_OK) return st;
  if (gu->E != dn->E || gu->N != 2 * dn->K) return SKINNY_ERR_INVALID_ARG;
  return SKINNY_OK;
}

size_t moe_mlp_workspace(const skinny_experts& gu, const skinny_experts& dn, int T, int topk) {
  const size_t a = moe_workspace(gu, moe_plan(gu, T, topk));
  const size_t b = moe_workspace(dn, moe_plan(dn, T, topk));
  return kMoeMlpCtrBytes + moe_mlp_gu_bytes(gu, T, topk) + (a > b ? a : b);
}

// LDS of the one-token kernel for G workgroups, or 0 if it does not apply.
struct MoeMlpLds {
  int hs_off, ya_off, yb_off, tab_off, bytes;
};
MoeMlpLds moe_mlp1_lds(const skinny_experts& gu, const skinny_experts& dn, int topk, int G) {
  MoeMlpLds l{};
  const long long xchunks = ((gu.K / 8 + 63) / 64) * 64;
  const long long gA = (gu.N + kRowsWavesPerBlock - 1) / kRowsWavesPerBlock;
  const long long gB = (dn.N + kRowsWavesPerBlock - 1) / kRowsWavesPerBlock;
  const long long ua = (topk * gA + G - 1) / G, ub = (gB + G / topk - 1) / (G / topk);
  long long off = xchunks * 16;
  l.hs_off = (int)off;
  off += (long long)(dn.K / 8) * 16;
  l.ya_off = (int)off;
  off += (ua * kRowsWavesPerBlock * 2 + 15) / 16 * 16;
  l.yb_off = (int)off;
  off += (ub * kRowsWavesPerBlock * 2 + 15) / 16 * 16;
  l.tab_off = (int)off;
  off += (2 + 2 * kMoeMlpMaxRoutes) * 4;
  if (off > kMaxLdsBytes) return MoeMlpLds{};
  l.bytes = (int)off;
  return l;
}

// The one-token kernel's instances: slots per wave for gate_up and down.  A
// call takes the first whose slots hold every workgroup's rows (units per
// workgroup x slots per unit, for the most routes the call can have), with
// one workgroup per CU: two per CU measured slower on the verify step (FP8
// 18.7 against 16.2 us, bf16 24.0 against 22.0 us).
struct MoeMlpInst {
  int dtype, ma, mb;
  void (*fn)(MoeMlpArgs);
};
const MoeMlpInst kMoeMlpInsts[] = {
    {SKINNY_FP8_BS128, 4, 2, skinny_moe_mlp1<SKINNY_FP8_BS128, 4, 2, kMoeMlpSegs>},
    {SKINNY_FP8_BS128, 6, 4, skinny_moe_mlp1<SKINNY_FP8_BS128, 6, 4, kMoeMlpSegs>},
    {SKINNY_FP8_BS128, 8, 8, skinny_moe_mlp1<SKINNY_FP8_BS128, 8, 8, kMoeMlpSegs>},
    {SKINNY_BF16, 8, 4, skinny_moe_mlp1<SKINNY_BF16, 8, 4, kMoeMlpSegs>},
    {SKINNY_BF16, 12, 8, skinny_moe_mlp1<SKINNY_BF16, 12, 8, kMoeMlpSegs>},
};

// Slots a wave needs for one linear: gate_up units are dealt over all G
// workgroups, down units of a route over its group of at least G / topk.
long long moe_mlp1_slots(const skinny_experts& e, int topk, int G, bool down) {
  const long long groups = (e.N + kRowsWavesPerBlock - 1) / kRowsWavesPerBlock;
  const long long units = down ? (groups + G / topk - 1) / (G / topk)
                               : (topk * groups + G - 1) / G;
  const int cpr = e.K / (e.dtype == SKINNY_BF16 ? 8 : 16);
  const int spt = (cpr + kSegChunks - 1) / kSegChunks;
  return units * ((spt + kMoeMlpSegs - 1) / kMoeMlpSegs);
}

struct MoeMlpChoice {
  const MoeMlpInst* inst = nullptr;
  int G = 0;
  MoeMlpLds lds{};
};

// The one-token kernel's instance and grid for this call, or none.
skinny_status moe_mlp1_choose(const skinny_experts& gu, const skinny_experts& dn, int T, int topk,
                              int cus, MoeMlpChoice* out) {
  *out = MoeMlpChoice{};
  if (T != 1 || topk > kMoeMlpMaxRoutes || gu.dtype != dn.dtype) return SKINNY_OK;
  const int G = cus;
  if (G < topk) return SKINNY_OK;
  if (G > kMoeMlpMaxGrid) return SKINNY_OK;
  const MoeMlpLds l = moe_mlp1_lds(gu, dn, topk, G);
  if (l.bytes == 0) return SKINNY_OK;
  for (const MoeMlpInst& in : kMoeMlpInsts) {
    if (in.dtype != gu.dtype || moe_mlp1_slots(gu, topk, G, false) > in.ma ||
        moe_mlp1_slots(dn, topk, G, true) > in.mb)
      continue;
    skinny_status st = ensure_lds((const void*)in.fn, l.bytes);
    if (st != SKINNY_OK) return st;
    int bpc = 0;
    st = blocks_per_cu((const void*)in.fn, l.bytes, 64 * kRowsWavesPerBlock, &bpc);
    if (st != SKINNY_OK) return st;
    if (bpc < 1) continue;
    *out = MoeMlpChoice{&in, G, l};
    return SKINNY_OK;
  }
  return SKINNY_OK;
}

skinny_status moe_mlp_run(const skinny_experts* gu, const skinny_experts* dn, const void* x,
                          const int* ids, int T, int topk, void* y, void* ws, size_t ws_bytes,
                          void* stream, void* const* events) {
  skinny_status st = check_moe_mlp(gu, dn, T, topk);
  if (st != SKINNY_OK) return st;
  if (!x || !ids || !y) return SKINNY_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4)) return SKINNY_ERR_UNSUPPORTED;
  if (!ws) return SKINNY_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SKINNY_ERR_UNSUPPORTED;
  if (ws_bytes < moe_mlp_workspace(*gu, *dn, T, topk)) return SKINNY_ERR_WORKSPACE;
  const int routes = T * topk;
  auto wrange = [](const skinny_experts* e) {
    return Range{(uintptr_t)e->w, (uintptr_t)e->w + (size_t)e->E * e->N * e->K *
                                                      (e->dtype == SKINNY_BF16 ? 2 : 1)};
  };
  auto srange = [](const skinny_experts* e) {
    const size_t nb = (size_t)((e->N + 127) / 128) * ((e->K + 127) / 128);
    return Range{(uintptr_t)e->w_scale,
                 (uintptr_t)e->w_scale + (e->w_scale ? (size_t)e->E * nb * 4 : 0)};
  };
  const Range yr{(uintptr_t)y, (uintptr_t)y + (size_t)routes * dn->N * 2};
  const Range xr{(uintptr_t)x, (uintptr_t)x + (size_t)T * gu->K * 2};
  const Range ir{(uintptr_t)ids, (uintptr_t)ids + (size_t)routes * 4};
  const Range kr{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  const Range in[] = {xr, ir, wrange(gu), srange(gu), wrange(dn), srange(dn)};
  for (const Range& r : in)
    if (overlap(yr, r) || overlap(kr, r)) return SKINNY_ERR_INVALID_ARG;
  if (overlap(yr, kr)) return SKINNY_ERR_INVALID_ARG;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != SKINNY_OK) return st;
  if (!dev.gfx950) return SKINNY_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  __bf16* gub = (__bf16*)((char*)ws + kMoeMlpCtrBytes);
  void* rest = (char*)ws + kMoeMlpCtrBytes + moe_mlp_gu_bytes(*gu, T, topk);
  const size_t rest_bytes = ws_bytes - kMoeMlpCtrBytes - moe_mlp_gu_bytes(*gu, T, topk);

  MoeMlpChoice ch;
  st = moe_mlp1_choose(*gu, *dn, T, topk, dev.cus, &ch);
  if (st != SKINNY_OK) return st;
  if (ch.inst) {
    const int dtype = gu->dtype;
    const MoeMlpLds& l = ch.lds;
    MoeMlpArgs a;
    memset(&a, 0, sizeof a);
    const int kpc = dtype == SKINNY_BF16 ? 8 : 16;       // K per 16-byte chunk
    a.wg = (const u32x4*)gu->w;
    a.sg = gu->w_scale;
    a.wd = (const u32x4*)dn->w;
    a.sd = dn->w_scale;
    a.E = gu->E;
    a.R = topk;
    a.N1 = gu->N;
    a.K1 = gu->K;
    a.cpr1 = gu->K / kpc;
    a.spt1 = (a.cpr1 + kSegChunks - 1) / kSegChunks;
    a.kb1 = (gu->K + kScaleBlock - 1) / kScaleBlock;
    a.N2 = dn->N;
    a.K2 = dn->K;
    a.cpr2 = dn->K / kpc;
    a.spt2 = (a.cpr2 + kSegChunks - 1) / kSegChunks;
    a.kb2 = (dn->K + kScaleBlock - 1) / kScaleBlock;
    a.wg_stride = (long long)a.N1 * a.cpr1;
    a.wd_stride = (long long)a.N2 * a.cpr2;
    a.sg_stride = dtype == SKINNY_BF16 ? 0 : (long long)((a.N1 + 127) / 128) * a.kb1;
    a.sd_stride = dtype == SKINNY_BF16 ? 0 : (long long)((a.N2 + 127) / 128) * a.kb2;
    a.ids = ids;
    a.x = (const u32x4*)x;
    a.gu = (unsigned long long*)gub;
    a.y = (__bf16*)y;
    a.ended = (unsigned long long*)ws;
    a.gave_up = (int*)((char*)ws + 8);
    a.spin = g_moe_mlp_spin.load();
    a.G = ch.G;
    a.hs_off = l.hs_off;
    a.ya_off = l.ya_off;
    a.yb_off = l.yb_off;
    a.tab_off = l.tab_off;
    if (events && hipEventRecord((hipEvent_t)events[0], s) != hipSuccess) return SKINNY_ERR_HIP;
    hipLaunchKernelGGL(ch.inst->fn, dim3(ch.G), dim3(64 * kRowsWavesPerBlock), l.bytes, s, a);
    if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
    if (events && hipEventRecord((hipEvent_t)events[1], s) != hipSuccess) return SKINNY_ERR_HIP;
    return SKINNY_OK;
  }
  // Two launches: gate_up into the workspace, then down through the SwiGLU.
  st = moe_run(gu, x, ids, T, topk, 0, gub, rest, rest_bytes, stream, events);
  if (st != SKINNY_OK) return st;
  return moe_run(dn, gub, ids, T, topk, SKINNY_MOE_X_PER_ROUTE | SKINNY_MOE_SWIGLU, y, rest,
                 rest_bytes, stream, nullptr);
}

size_t skinny_moe_mlp_workspace_bytes(const skinny_experts* gate_up, const skinny_experts* down,
                                      int T, int topk) {
  if (check_moe_mlp(gate_up, down, T, topk) != SKINNY_OK) return 0;
  return moe_mlp_workspace(*gate_up, *down, T, topk);
}

skinny_status skinny_moe_mlp_swiglu(const skinny_experts* gate_up, const skinny_experts* down,
                                    const void* x, const int* ids, int T, int topk, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return moe_mlp_run(gate_up, down, x, ids, T, topk, y, workspace, workspace_bytes, stream,
                     nullptr);
}

skinny_status skinny_moe_mlp_swiglu_timed(const skinny_experts* gate_up,
                                          const skinny_experts* down, const void* x,
                                          const int* ids, int T, int topk, void* y,
                                          void* const* events, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!events) return SKINNY_ERR_INVALID_ARG;
  return moe_mlp_run(gate_up, down, x, ids, T, topk, y, workspace, workspace_bytes, stream,
                     events);
}

void skinny_moe_mlp_set_spin_limit(long long polls) { g_moe_mlp_spin.store(polls); }

skinny_status skinny_moe_mlp_plan_query(const skinny_experts* gate_up, const skinny_experts* down,
                                        int T, int topk, skinny_plan* out) {
  if (!out) return SKINNY_ERR_INVALID_ARG;
  skinny_status st = check_moe_mlp(gate_up, down, T, topk);
  if (st != SKINNY_OK) return st;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != SKINNY_OK) return st;
  MoeMlpChoice ch;
  st = moe_mlp1_choose(*gate_up, *down, T, topk, dev.cus, &ch);
  if (st != SKINNY_OK) return st;
  if (ch.inst) {
    memset(out, 0, sizeof *out);
    out->variant = SKINNY_VARIANT_VECTOR;
    out->waves = ch.G * kRowsWavesPerBlock;
    out->kernel = SKINNY_KERNEL_MOE_MLP1;
    return SKINNY_OK;
  }
  return skinny_moe_plan_query(gate_up, T, topk, 0, out);
}

skinny_status skinny_moe_plan_query(const skinny_experts* experts, int T, int topk, int flags,
                                    skinny_plan* out) {
  if (!out) return SKINNY_ERR_INVALID_ARG;
  const skinny_status st = check_experts(experts, T, topk, flags);
  if (st != SKINNY_OK) return st;
  memset(out, 0, sizeof *out);
  const MoePlan p = moe_plan(*experts, T, topk);
  out->variant = p.rows ? SKINNY_VARIANT_VECTOR : SKINNY_VARIANT_MFMA;
  out->kernel = p.rows ? SKINNY_KERNEL_ROWS
                : p.ks ? SKINNY_KERNEL_TILES_KSPLIT
                : p.wpb == kTilesWavesSmall ? SKINNY_KERNEL_TILES : SKINNY_KERNEL_TILES_WIDE;
  return SKINNY_OK;
}

const char* skinny_status_string(int status) {
  switch (status) {
    case SKINNY_OK: return "ok";
    case SKINNY_ERR_INVALID_ARG: return "invalid argument";
    case SKINNY_ERR_UNSUPPORTED: return "unsupported shape, alignment or device";
    case SKINNY_ERR_WORKSPACE: return "workspace missing or too small";
    case SKINNY_ERR_HIP: return "HIP call failed";
    default: return "unknown status";
  }
}

int skinny_abi_version(void) { return SKINNY_ABI_VERSION; }

}  // extern "C"
