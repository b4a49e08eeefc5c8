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
//   splits K into fixed slices per block; here every wave of a persistent
//   grid takes an equal share of all (tile, k-step) work of all linears in the
//   launch, so one launch streams a whole stack with a single ramp and tail.
//
// Work decomposition:
//   tile  = 16 consecutive rows of one linear's W
//   band  = T consecutive tiles (16 T rows), T in {1, 2, 4}; one wave streams
//           a band so that each activation chunk it loads serves T weight loads
//   chunk = 16 bytes of a W row (8 bf16 or 16 e4m3 weights)
//   step  = one k-step of a band: per tile, 16 rows x 4 consecutive chunks;
//           lane l reads row (l % 16), chunk 4*j + (l / 16) of every tile.
//           This is exactly the B-operand layout of v_mfma_f32_16x16x32_bf16,
//           and the vector path uses it too.
//   Steps are numbered globally (linear, band, step-in-band); wave w of G
//   streams steps [w*S/G, (w+1)*S/G).  A band whose steps a single wave
//   covers is written straight to y.  A band cut by a wave boundary has each
//   contributing wave write fp32 partial sums to a fixed workspace slot
//   (slot 2w for the wave's first band, 2w+1 for its last), and a second
//   pass adds the slots in wave order: deterministic, no atomics.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "skinny_gemm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;
constexpr int kMaxBandTiles = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = 64 * kWavesPerBlock;
constexpr int kMaxWaves = 8192;         // 256 CUs x 32 resident waves
constexpr int kSlotsPerWave = 2;
constexpr int kScaleBlock = 128;

struct LinDesc {
  const u32x4* w;        // W rows as 16-byte chunks
  const float* scale;    // FP8 block scales (NULL for bf16)
  const u32x4* x;        // x rows as 16-byte chunks (8 bf16 each)
  __bf16* y;             // y[M][N]
  int N;
  int K;
  int cpr;               // 16-byte chunks per W row
  int spt;               // steps per band = ceil(cpr / 4)
  int kblocks;           // ceil(K / 128)
  int pad;
  long long step_base;   // global index of this linear's first step
};

struct LaunchArgs {
  int nlin;
  int M;
  int G;                 // waves of the main launch
  int band_rows;         // 16 T
  long long S;           // total steps of the launch
  float* slots;          // [2 G][M][band_rows] fp32 partial sums
  LinDesc lin[SKINNY_MAX_LINEARS_PER_LAUNCH];
};

__device__ __forceinline__ long long wave_start(long long w, long long S, long long G) {
  return w * S / G;
}

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

// ---------------------------------------------------------------------------
// Steps [j0, j1) of one band.  Per lane: row r = lane % 16 of each tile and
// chunk group g = lane / 16; step j reads chunk 4 j + g of those rows.  A
// batch of U steps is loaded (W for all T tiles, x once) before it is used;
// with PIPE the next batch's loads are issued before the current batch is
// consumed.  XC = 16-byte x chunks per W chunk (1 for bf16, 2 for e4m3).

template <int DT, int M, int T, int U>
struct Batch {
  static constexpr int XC = DT == SKINNY_BF16 ? 1 : 2;
  u32x4 w[U][T];
  u32x4 x[U][M][XC];
};

template <int DT, int XM, int T, int U>
__device__ __forceinline__ void load_batch(Batch<DT, XM, T, U>& b, const LinDesc& L,
                                           const u32x4* const (&wrow)[T], const bool (&rowok)[T],
                                           const u32x4* const (&xrow)[XM], const bool (&tokok)[XM],
                                           int j, int j1, int g) {
  constexpr int XC = Batch<DT, XM, T, U>::XC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = (j + u) * 4 + g;
    const bool ok = (j + u < j1) && (c < L.cpr);
#pragma unroll
    for (int t = 0; t < T; ++t) b.w[u][t] = (ok && rowok[t]) ? wrow[t][c] : zero4();
#pragma unroll
    for (int m = 0; m < XM; ++m)
#pragma unroll
      for (int h = 0; h < XC; ++h) b.x[u][m][h] = (ok && tokok[m]) ? xrow[m][XC * c + h] : zero4();
  }
}

// Vector path: lane keeps T x MT running sums (tile, token) for its row of
// each tile; the four lanes of a row are added at the end.
template <int DT, int MT, int T, int U>
__device__ __forceinline__ void compute_vector(const Batch<DT, MT, T, U>& b, float (&acc)[T][MT],
                                               const float* srow, int j, int j1) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (DT == SKINNY_BF16) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[t][m] = dot8(b.x[u][m][0], b.w[u][t], acc[t][m]);
    } else {
      const float s = (j + u < j1) ? srow[(j + u) >> 1] : 0.0f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        u32x4 b0, b1;
        e4m3x16_to_bf16(b.w[u][t], b0, b1);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float p = dot8(b.x[u][m][1], b1, dot8(b.x[u][m][0], b0, 0.0f));
          acc[t][m] = __builtin_fmaf(s, p, acc[t][m]);
        }
      }
    }
  }
}

// MFMA path: D[m][n] += x[m][k] W[n][k] over 32 k per instruction; A is the
// token tile (lane l supplies token l % 16, zero for tokens >= M), B a weight
// tile.  Lane l ends holding D[4 (l / 16) + i][l % 16], i = 0..3, per tile.
template <int DT, int T, int U>
__device__ __forceinline__ void compute_mfma(const Batch<DT, 1, T, U>& b, f32x4 (&acc)[T],
                                             const float* srow, int j, int j1) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (DT == SKINNY_BF16) {
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = mfma_bf16(b.x[u][0][0], b.w[u][t], acc[t]);
    } else {
      const float s = (j + u < j1) ? srow[(j + u) >> 1] : 0.0f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        u32x4 b0, b1;
        e4m3x16_to_bf16(b.w[u][t], b0, b1);
        f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
        p = mfma_bf16(b.x[u][0][0], b0, p);
        p = mfma_bf16(b.x[u][0][1], b1, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(s, p[i], acc[t][i]);
      }
    }
  }
}

// One band's steps [j0, j1).  VAR = vector: acc is float[T][MT]; MFMA: f32x4[T].
template <int DT, int VAR, int MT, int T, int U, bool PIPE, typename Acc>
__device__ __forceinline__ void run_band(const LinDesc& L, int M, int band, int j0, int j1,
                                         Acc& acc, int lane) {
  constexpr int XM = VAR == SKINNY_VARIANT_VECTOR ? MT : 1;   // x rows a lane loads
  const int r = lane & 15;
  const int g = lane >> 4;
  const int xcpr = L.K >> 3;                                   // x chunks per token row
  const u32x4* wrow[T];
  bool rowok[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int row = band * (kTileRows * T) + t * kTileRows + r;
    rowok[t] = row < L.N;
    wrow[t] = L.w + (size_t)(rowok[t] ? row : 0) * (size_t)L.cpr;
  }
  const u32x4* xrow[XM];
  bool tokok[XM];
#pragma unroll
  for (int m = 0; m < XM; ++m) {
    const int tok = (VAR == SKINNY_VARIANT_VECTOR) ? m : r;    // MFMA: A row = lane % 16
    tokok[m] = tok < M;
    xrow[m] = L.x + (size_t)(tokok[m] ? tok : 0) * xcpr;
  }
  // All rows of a band lie in one 128-row scale block (16 T divides 128).
  const float* srow = (DT == SKINNY_FP8_BS128)
                          ? L.scale + (size_t)((band * kTileRows * T) / kScaleBlock) * L.kblocks
                          : nullptr;
  auto compute = [&](const Batch<DT, XM, T, U>& bt, int j) {
    if constexpr (VAR == SKINNY_VARIANT_VECTOR) compute_vector<DT, MT, T, U>(bt, acc, srow, j, j1);
    else compute_mfma<DT, T, U>(bt, acc, srow, j, j1);
  };
  if constexpr (PIPE) {
    Batch<DT, XM, T, U> b0, b1;
    load_batch(b0, L, wrow, rowok, xrow, tokok, j0, j1, g);
    for (int j = j0; j < j1; j += 2 * U) {
      load_batch(b1, L, wrow, rowok, xrow, tokok, j + U, j1, g);
      compute(b0, j);
      load_batch(b0, L, wrow, rowok, xrow, tokok, j + 2 * U, j1, g);
      compute(b1, j + U);
    }
  } else {
    for (int j = j0; j < j1; j += U) {
      Batch<DT, XM, T, U> b0;
      load_batch(b0, L, wrow, rowok, xrow, tokok, j, j1, g);
      compute(b0, j);
    }
  }
}

// Main pass: wave w streams its equal share of the launch's steps.
template <int DT, int VAR, int MT, int T, int U, bool PIPE>
__global__ __launch_bounds__(kBlockThreads) void skinny_main(const LaunchArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (w >= a.G) return;
  const long long s0 = wave_start(w, a.S, a.G);
  const long long s1 = wave_start(w + 1, a.S, a.G);
  if (s0 >= s1) return;
  const int M = (VAR == SKINNY_VARIANT_VECTOR) ? MT : a.M;
  constexpr int kBandRows = kTileRows * T;
  const int r = lane & 15;
  const int g = lane >> 4;
  int l = 0;
  long long s = s0;
  bool first = true;
  while (s < s1) {
    while (l + 1 < a.nlin && a.lin[l + 1].step_base <= s) ++l;
    const LinDesc& L = a.lin[l];
    const long long local = s - L.step_base;
    const int band = (int)(local / L.spt);
    const int j0 = (int)(local - (long long)band * L.spt);
    const long long band_end = L.step_base + (long long)(band + 1) * L.spt;
    const int j1 = (int)((s1 < band_end ? s1 : band_end) - (L.step_base + (long long)band * L.spt));
    const bool whole = (j0 == 0) && (j1 == L.spt);
    float* slot = a.slots + (size_t)(2 * w + (first ? 0 : 1)) * M * kBandRows;
    if constexpr (VAR == SKINNY_VARIANT_VECTOR) {
      float acc[T][MT];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[t][m] = 0.0f;
      run_band<DT, VAR, MT, T, U, PIPE>(L, M, band, j0, j1, acc, lane);
      // Add the four lanes that share a row (r, r+16, r+32, r+48), fixed order.
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[t][m] += __shfl_xor(acc[t][m], 16);
          acc[t][m] += __shfl_xor(acc[t][m], 32);
        }
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int rr = t * kTileRows + r;
          const int row = band * kBandRows + rr;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (whole) {
              if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)acc[t][m];
            } else {
              slot[m * kBandRows + rr] = acc[t][m];
            }
          }
        }
      }
    } else {
      f32x4 acc[T];
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      run_band<DT, VAR, 1, T, U, PIPE>(L, M, band, j0, j1, acc, lane);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int rr = t * kTileRows + r;
        const int row = band * kBandRows + rr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * g + i;
          if (m < M) {
            if (whole) {
              if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)acc[t][i];
            } else {
              slot[m * kBandRows + rr] = acc[t][i];
            }
          }
        }
      }
    }
    s = band_end < s1 ? band_end : s1;
    first = false;
  }
}

// Second pass: block w handles the band that contains wave w's first step if
// that step lies strictly inside the band and no earlier wave boundary does.
// Its threads add, for every (token, row) of the band, the contributing
// waves' slots in increasing wave order and write y.
__global__ __launch_bounds__(kBlockThreads) void skinny_combine(const LaunchArgs a) {
  const int w = blockIdx.x;
  if (w == 0 || w >= a.G) return;
  const long long b = wave_start(w, a.S, a.G);
  if (b >= a.S) return;
  int l = 0;
  while (l + 1 < a.nlin && a.lin[l + 1].step_base <= b) ++l;
  const LinDesc& L = a.lin[l];
  const long long local = b - L.step_base;
  const int band = (int)(local / L.spt);
  const long long bstart = L.step_base + (long long)band * L.spt;
  const long long bend = bstart + L.spt;
  if (b == bstart) return;
  if (wave_start(w - 1, a.S, a.G) > bstart) return;
  const int R = a.band_rows;
  for (int idx = threadIdx.x; idx < a.M * R; idx += blockDim.x) {
    const int m = idx / R;
    const int rr = idx - m * R;
    float sum = 0.0f;
    for (int v = w - 1; v < a.G; ++v) {
      const long long sv = wave_start(v, a.S, a.G);
      if (sv >= bend) break;
      const long long ev = wave_start(v + 1, a.S, a.G);
      if (ev <= sv) continue;                     // empty wave
      const int slot = 2 * v + (sv >= bstart ? 0 : 1);
      sum += a.slots[((size_t)slot * a.M + m) * R + rr];
    }
    const int row = band * R + rr;
    if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)sum;
  }
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

skinny_status check_linear(const skinny_linear& L, int M) {
  if (L.dtype != SKINNY_BF16 && L.dtype != SKINNY_FP8_BS128) return SKINNY_ERR_INVALID_ARG;
  if (L.reserved != 0) return SKINNY_ERR_INVALID_ARG;
  if (M < 1 || M > SKINNY_MAX_M || L.N < 1 || L.K < 1) return SKINNY_ERR_INVALID_ARG;
  if (!L.w || !L.x || !L.y) return SKINNY_ERR_INVALID_ARG;
  if (L.dtype == SKINNY_FP8_BS128 && !L.w_scale) return SKINNY_ERR_INVALID_ARG;
  if (L.dtype == SKINNY_BF16 && L.w_scale) return SKINNY_ERR_INVALID_ARG;
  if (L.K % (L.dtype == SKINNY_BF16 ? 8 : 16) != 0) return SKINNY_ERR_UNSUPPORTED;
  if (!aligned(L.w, 16) || !aligned(L.x, 16) || !aligned(L.y, 16)) return SKINNY_ERR_UNSUPPORTED;
  if (L.w_scale && !aligned(L.w_scale, 4)) return SKINNY_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels is 32-bit per tile and per row.
  if (L.N > (1 << 30) || L.K > (1 << 28)) return SKINNY_ERR_UNSUPPORTED;
  return SKINNY_OK;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

skinny_status check_outputs(const skinny_linear* lin, int count, int M, const void* ws,
                            size_t ws_bytes) {
  for (int i = 0; i < count; ++i) {
    const skinny_linear& L = lin[i];
    Range y{(uintptr_t)L.y, (uintptr_t)L.y + (size_t)M * L.N * 2};
    Range wsr{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
    if (overlap(y, wsr)) return SKINNY_ERR_INVALID_ARG;
    for (int j = 0; j < count; ++j) {
      const skinny_linear& O = lin[j];
      const size_t wbytes = (size_t)O.N * O.K * (O.dtype == SKINNY_BF16 ? 2 : 1);
      Range x{(uintptr_t)O.x, (uintptr_t)O.x + (size_t)M * O.K * 2};
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

size_t workspace_for(int M) {
  return (size_t)kMaxWaves * kSlotsPerWave * (size_t)M * kTileRows * kMaxBandTiles *
         sizeof(float);
}

// Measured on MI355X (80-layer TP=1 shapes, M = 1..16, bf16 and FP8): the
// MFMA path streams faster than the v_dot2 path at every M, because one MFMA
// replaces four dot2 per chunk plus the cross-lane reduction and its A-operand
// load serves all tokens.  The vector path stays available through the plan.
int auto_variant(int dtype, int M) {
  (void)dtype;
  (void)M;
  return SKINNY_VARIANT_MFMA;
}

// Shape of the main loop per (dtype, variant, M): T tiles per band (x reuse),
// U steps per batch, PIPE = issue the next batch before using this one.
// Register use grows with T*U (weights) and U*M (activations), and the
// persistent grid needs enough waves resident to cover HBM latency.
struct LoopShape {
  int T, U;
  bool pipe;
};

template <int DT, int VAR, int MT>
constexpr LoopShape loop_shape() {
  if (VAR == SKINNY_VARIANT_MFMA) return LoopShape{2, 8, false};
  if (MT <= 1) return LoopShape{4, 2, true};
  if (MT <= 2) return LoopShape{2, 2, true};
  return LoopShape{1, 2, false};
}

typedef void (*main_fn)(LaunchArgs);

struct KernelChoice {
  main_fn fn = nullptr;
  int T = 1;
};

template <int DT, int VAR, int MT>
KernelChoice main_kernel() {
  constexpr LoopShape ls = loop_shape<DT, VAR, MT>();
  static_assert(ls.T >= 1 && ls.T <= kMaxBandTiles && (ls.T & (ls.T - 1)) == 0, "bad band");
  KernelChoice k;
  k.fn = skinny_main<DT, VAR, MT, ls.T, ls.U, ls.pipe>;
  k.T = ls.T;
  return k;
}

template <int DT>
KernelChoice pick_main(int variant, int M) {
  if (variant == SKINNY_VARIANT_MFMA) return main_kernel<DT, SKINNY_VARIANT_MFMA, 0>();
  switch (M) {
    case 1: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 1>();
    case 2: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 2>();
    case 3: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 3>();
    case 4: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 4>();
    case 5: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 5>();
    case 6: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 6>();
    case 7: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 7>();
    case 8: return main_kernel<DT, SKINNY_VARIANT_VECTOR, 8>();
    default: return KernelChoice{};
  }
}

KernelChoice pick(int dtype, int variant, int M) {
  return dtype == SKINNY_BF16 ? pick_main<SKINNY_BF16>(variant, M)
                              : pick_main<SKINNY_FP8_BS128>(variant, M);
}

// Persistent grid size: every wave must be resident at once for the equal
// shares to finish together, so take what the occupancy query allows for
// this kernel, capped at kTargetWavesPerCU waves per CU.  The query result is
// cached per (device, kernel).
constexpr int kTargetWavesPerCU = 16;
constexpr int kOccCache = 128;
struct OccEntry {
  int dev;
  main_fn fn;
  int blocks_per_cu;
};
OccEntry g_occ[kOccCache];
int g_occ_n = 0;
std::mutex g_occ_mu;

skinny_status auto_waves(const DeviceInfo& d, main_fn fn, int* waves) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
  int blocks_per_cu = -1;
  {
    std::lock_guard<std::mutex> lock(g_occ_mu);
    for (int i = 0; i < g_occ_n; ++i)
      if (g_occ[i].dev == dev && g_occ[i].fn == fn) blocks_per_cu = g_occ[i].blocks_per_cu;
  }
  if (blocks_per_cu < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_per_cu, (const void*)fn,
                                                     kBlockThreads, 0) != hipSuccess)
      return SKINNY_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_occ_mu);
    if (g_occ_n < kOccCache) g_occ[g_occ_n++] = OccEntry{dev, fn, blocks_per_cu};
  }
  int per_cu = blocks_per_cu * kWavesPerBlock;
  if (per_cu > kTargetWavesPerCU) per_cu = kTargetWavesPerCU;
  if (per_cu < kWavesPerBlock) per_cu = kWavesPerBlock;
  long long g = (long long)d.cus * per_cu;
  if (g > kMaxWaves) g = kMaxWaves;
  *waves = (int)g;
  return SKINNY_OK;
}

// Enqueues one group of same-dtype linears (at most SKINNY_MAX_LINEARS_PER_LAUNCH).
// G = 0 sizes the persistent grid from occupancy.
skinny_status launch_group(const DeviceInfo& dev, const skinny_linear* const* lin, int count,
                           int M, int variant, int G, float* slots, hipStream_t stream,
                           hipEvent_t ev_before, hipEvent_t ev_after) {
  const int dtype = lin[0]->dtype;
  const KernelChoice k = pick(dtype, variant, M);
  if (!k.fn) return SKINNY_ERR_INVALID_ARG;
  LaunchArgs a;
  memset(&a, 0, sizeof a);
  a.nlin = count;
  a.M = M;
  a.slots = slots;
  a.band_rows = kTileRows * k.T;
  long long S = 0;
  for (int i = 0; i < count; ++i) {
    const skinny_linear& L = *lin[i];
    LinDesc& d = a.lin[i];
    d.w = (const u32x4*)L.w;
    d.scale = L.w_scale;
    d.x = (const u32x4*)L.x;
    d.y = (__bf16*)L.y;
    d.N = L.N;
    d.K = L.K;
    d.cpr = L.K / (dtype == SKINNY_BF16 ? 8 : 16);
    d.spt = (d.cpr + 3) / 4;
    d.kblocks = (L.K + kScaleBlock - 1) / kScaleBlock;
    d.step_base = S;
    const long long bands = (L.N + a.band_rows - 1) / a.band_rows;
    S += bands * d.spt;
  }
  a.S = S;
  main_fn fn = k.fn;
  if (G == 0) {
    skinny_status st = auto_waves(dev, fn, &G);
    if (st != SKINNY_OK) return st;
  }
  if (G > S) G = (int)S;
  if (G < 1) G = 1;
  a.G = G;
  const int blocks = (G + kWavesPerBlock - 1) / kWavesPerBlock;
  if (ev_before && hipEventRecord(ev_before, stream) != hipSuccess) return SKINNY_ERR_HIP;
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kBlockThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  if (ev_after && hipEventRecord(ev_after, stream) != hipSuccess) return SKINNY_ERR_HIP;
  if (G > 1) {
    hipLaunchKernelGGL(skinny_combine, dim3(G), dim3(kBlockThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  }
  return SKINNY_OK;
}

int launch_count(const skinny_linear* lin, int count) {
  int launches = 0;
  for (int dt = SKINNY_BF16; dt <= SKINNY_FP8_BS128; ++dt) {
    int n = 0;
    for (int i = 0; i < count; ++i) n += lin[i].dtype == dt;
    launches += (n + SKINNY_MAX_LINEARS_PER_LAUNCH - 1) / SKINNY_MAX_LINEARS_PER_LAUNCH;
  }
  return launches;
}

skinny_status run(const skinny_linear* lin, int count, int M, const skinny_plan* plan,
                  void* ws, size_t ws_bytes, void* stream, void* const* events = nullptr,
                  int event_count = 0) {
  if (!lin || count < 1) return SKINNY_ERR_INVALID_ARG;
  if (M < 1 || M > SKINNY_MAX_M) return SKINNY_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    skinny_status st = check_linear(lin[i], M);
    if (st != SKINNY_OK) return st;
  }
  int variant = SKINNY_VARIANT_AUTO;
  int waves = 0;
  if (plan) {
    for (int i = 0; i < 6; ++i)
      if (plan->reserved[i] != 0) return SKINNY_ERR_INVALID_ARG;
    variant = plan->variant;
    waves = plan->waves;
    if (variant < SKINNY_VARIANT_AUTO || variant > SKINNY_VARIANT_MFMA) return SKINNY_ERR_INVALID_ARG;
    if (waves < 0 || waves > kMaxWaves) return SKINNY_ERR_INVALID_ARG;
  }
  if (variant == SKINNY_VARIANT_VECTOR && M > 8) return SKINNY_ERR_UNSUPPORTED;
  if (!ws) return SKINNY_ERR_WORKSPACE;
  if (ws_bytes < workspace_for(M)) return SKINNY_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return SKINNY_ERR_UNSUPPORTED;
  skinny_status st = check_outputs(lin, count, M, ws, ws_bytes);
  if (st != SKINNY_OK) return st;
  if (events && event_count < 2 * launch_count(lin, count)) return SKINNY_ERR_INVALID_ARG;
  DeviceInfo d;
  st = device_info(&d);
  if (st != SKINNY_OK) return st;
  if (!d.gfx950) return SKINNY_ERR_UNSUPPORTED;
  int launch = 0;
  auto ev = [&](int k) { return events ? (hipEvent_t)events[2 * launch + k] : (hipEvent_t) nullptr; };
  // Group by dtype, in call order, SKINNY_MAX_LINEARS_PER_LAUNCH per launch.
  for (int dt = SKINNY_BF16; dt <= SKINNY_FP8_BS128; ++dt) {
    const int var = variant == SKINNY_VARIANT_AUTO ? auto_variant(dt, M) : variant;
    const skinny_linear* group[SKINNY_MAX_LINEARS_PER_LAUNCH];
    int n = 0;
    for (int i = 0; i < count; ++i) {
      if (lin[i].dtype != dt) continue;
      group[n++] = &lin[i];
      if (n == SKINNY_MAX_LINEARS_PER_LAUNCH) {
        st = launch_group(d, group, n, M, var, waves, (float*)ws, (hipStream_t)stream, ev(0),
                          ev(1));
        if (st != SKINNY_OK) return st;
        ++launch;
        n = 0;
      }
    }
    if (n > 0) {
      st = launch_group(d, group, n, M, var, waves, (float*)ws, (hipStream_t)stream, ev(0),
                        ev(1));
      if (st != SKINNY_OK) return st;
      ++launch;
    }
  }
  return SKINNY_OK;
}

}  // namespace

extern "C" {

size_t skinny_workspace_bytes(int dtype, int M, int N, int K) {
  if (dtype != SKINNY_BF16 && dtype != SKINNY_FP8_BS128) return 0;
  if (M < 1 || M > SKINNY_MAX_M || N < 1 || K < 1) return 0;
  return workspace_for(M);
}

size_t skinny_stack_workspace_bytes(const skinny_linear* linears, int count, int M) {
  if (!linears || count < 1 || M < 1 || M > SKINNY_MAX_M) return 0;
  for (int i = 0; i < count; ++i)
    if (skinny_workspace_bytes(linears[i].dtype, M, linears[i].N, linears[i].K) == 0) return 0;
  return workspace_for(M);
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

skinny_status skinny_linear_run(const skinny_linear* linears, int count, int M,
                                const skinny_plan* plan, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return run(linears, count, M, plan, workspace, workspace_bytes, stream);
}

int skinny_band_rows(int dtype, int variant, int M) {
  if (dtype != SKINNY_BF16 && dtype != SKINNY_FP8_BS128) return 0;
  if (M < 1 || M > SKINNY_MAX_M) return 0;
  if (variant < SKINNY_VARIANT_AUTO || variant > SKINNY_VARIANT_MFMA) return 0;
  const int var = variant == SKINNY_VARIANT_AUTO ? auto_variant(dtype, M) : variant;
  const KernelChoice k = pick(dtype, var, M);
  return k.fn ? kTileRows * k.T : 0;
}

int skinny_launch_count(const skinny_linear* linears, int count) {
  if (!linears || count < 1) return 0;
  for (int i = 0; i < count; ++i)
    if (linears[i].dtype != SKINNY_BF16 && linears[i].dtype != SKINNY_FP8_BS128) return 0;
  return launch_count(linears, count);
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
  DeviceInfo d;
  skinny_status st = device_info(&d);
  if (st != SKINNY_OK) return st;
  memset(out, 0, sizeof *out);
  out->variant = auto_variant(linears[0].dtype, M);
  const KernelChoice k = pick(linears[0].dtype, out->variant, M);
  if (!k.fn) return SKINNY_ERR_INVALID_ARG;
  return auto_waves(d, k.fn, &out->waves);
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
