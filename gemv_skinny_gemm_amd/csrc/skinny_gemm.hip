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
//   chunk = 16 bytes of a W row (8 bf16 or 16 e4m3 weights)
//   step  = one 16-byte load per lane: 16 rows x 4 consecutive chunks, lane
//           l reads row (l % 16), chunk 4*j + (l / 16).  This is exactly the
//           B-operand layout of v_mfma_f32_16x16x32_bf16, and the vector path
//           uses it too.
//   Steps are numbered globally (linear, tile, step-in-tile); wave w of G
//   streams steps [w*T/G, (w+1)*T/G).  A tile whose steps a single wave
//   covers is written straight to y.  A tile cut by a wave boundary has each
//   contributing wave write fp32 partial sums to a fixed workspace slot
//   (slot 2w for the wave's first tile, 2w+1 for its last), and a second
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
  int spt;               // steps per tile = ceil(cpr / 4)
  int kblocks;           // ceil(K / 128)
  int pad;
  long long step_base;   // global index of this linear's first step
};

struct LaunchArgs {
  int nlin;
  int M;
  int G;                 // waves of the main launch
  int pad;
  long long T;           // total steps of the launch
  float* slots;          // [2 G][M][16] fp32 partial sums
  LinDesc lin[SKINNY_MAX_LINEARS_PER_LAUNCH];
};

__device__ __forceinline__ long long wave_start(long long w, long long T, long long G) {
  return w * T / G;
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

// ---------------------------------------------------------------------------
// Steps [j0, j1) of one tile.  Per lane: row r = lane % 16 of the tile and
// chunk group g = lane / 16; step j reads chunk 4 j + g of that row.

// Vector path: each lane keeps MT running sums (one per token) for its row;
// the four lanes of a row are added at the end.
template <int DT, int MT, int U>
__device__ __forceinline__ void tile_vector(const LinDesc& L, int tile, int j0, int j1,
                                            float (&acc)[MT], int lane) {
  const int r = lane & 15;
  const int g = lane >> 4;
  const int row = tile * kTileRows + r;
  const bool rowok = row < L.N;
  const u32x4* wrow = L.w + (size_t)(rowok ? row : 0) * (size_t)L.cpr;
  const int xcpr = L.K >> 3;                       // x chunks per token row
  const float* srow = (DT == 1) ? L.scale + (size_t)(tile >> 3) * L.kblocks : nullptr;
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  for (int j = j0; j < j1; j += U) {
    u32x4 wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + u) * 4 + g;
      const bool ok = rowok && (j + u < j1) && (c < L.cpr);
      wv[u] = ok ? __builtin_nontemporal_load(wrow + c) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + u) * 4 + g;
      const bool ok = (j + u < j1) && (c < L.cpr);
      if (DT == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 xv = ok ? L.x[(size_t)m * xcpr + c] : zero4();
          acc[m] = dot8(xv, wv[u], acc[m]);
        }
      } else {
        u32x4 b0, b1;
        e4m3x16_to_bf16(wv[u], b0, b1);
        const float s = (j + u < j1) ? srow[(j + u) >> 1] : 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 x0 = ok ? L.x[(size_t)m * xcpr + 2 * c] : zero4();
          const u32x4 x1 = ok ? L.x[(size_t)m * xcpr + 2 * c + 1] : zero4();
          const float p = dot8(x1, b1, dot8(x0, b0, 0.0f));
          acc[m] = __builtin_fmaf(s, p, acc[m]);
        }
      }
    }
  }
  // Add the four lanes that share a row (lanes r, r+16, r+32, r+48), fixed order.
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc[m] += __shfl_xor(acc[m], 16);
    acc[m] += __shfl_xor(acc[m], 32);
  }
}

// MFMA path: D[m][n] += x[m][k] W[n][k] over 32 k per instruction.  A is the
// token tile (rows m >= M are zero), B the weight tile.  Lane l ends holding
// D[4 (l / 16) + i][l % 16] for i = 0..3.
template <int DT, int U>
__device__ __forceinline__ f32x4 tile_mfma(const LinDesc& L, int M, int tile, int j0, int j1,
                                           int lane) {
  const int r = lane & 15;
  const int g = lane >> 4;
  const int row = tile * kTileRows + r;
  const bool rowok = row < L.N;
  const u32x4* wrow = L.w + (size_t)(rowok ? row : 0) * (size_t)L.cpr;
  const int xcpr = L.K >> 3;
  const bool tokok = r < M;                       // A-operand row m = r
  const u32x4* xrow = L.x + (size_t)(tokok ? r : 0) * xcpr;
  const float* srow = (DT == 1) ? L.scale + (size_t)(tile >> 3) * L.kblocks : nullptr;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = j0; j < j1; j += U) {
    u32x4 wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + u) * 4 + g;
      const bool ok = rowok && (j + u < j1) && (c < L.cpr);
      wv[u] = ok ? __builtin_nontemporal_load(wrow + c) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + u) * 4 + g;
      const bool ok = tokok && (j + u < j1) && (c < L.cpr);
      if (DT == 0) {
        const u32x4 xv = ok ? xrow[c] : zero4();
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv),
                                                      __builtin_bit_cast(bf16x8, wv[u]), acc,
                                                      0, 0, 0);
      } else {
        const u32x4 x0 = ok ? xrow[2 * c] : zero4();
        const u32x4 x1 = ok ? xrow[2 * c + 1] : zero4();
        u32x4 b0, b1;
        e4m3x16_to_bf16(wv[u], b0, b1);
        f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x0),
                                                    __builtin_bit_cast(bf16x8, b0), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x1),
                                                    __builtin_bit_cast(bf16x8, b1), t, 0, 0, 0);
        const float s = (j + u < j1) ? srow[(j + u) >> 1] : 0.0f;
        acc.x = __builtin_fmaf(s, t.x, acc.x);
        acc.y = __builtin_fmaf(s, t.y, acc.y);
        acc.z = __builtin_fmaf(s, t.z, acc.z);
        acc.w = __builtin_fmaf(s, t.w, acc.w);
      }
    }
  }
  return acc;
}

// Main pass: wave w streams its equal share of the launch's steps.
// VAR 1 = vector (MT = M at compile time), VAR 2 = MFMA (MT unused).
template <int DT, int VAR, int MT, int U>
__global__ __launch_bounds__(kBlockThreads) void skinny_main(const LaunchArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (w >= a.G) return;
  const long long s0 = wave_start(w, a.T, a.G);
  const long long s1 = wave_start(w + 1, a.T, a.G);
  if (s0 >= s1) return;
  int l = 0;
  while (l + 1 < a.nlin && a.lin[l + 1].step_base <= s0) ++l;
  const int M = (VAR == 1) ? MT : a.M;
  long long s = s0;
  bool first = true;
  while (s < s1) {
    while (l + 1 < a.nlin && a.lin[l + 1].step_base <= s) ++l;
    const LinDesc& L = a.lin[l];
    const long long local = s - L.step_base;
    const int tile = (int)(local / L.spt);
    const int j0 = (int)(local - (long long)tile * L.spt);
    const long long tile_end = L.step_base + (long long)(tile + 1) * L.spt;
    const int j1 = (int)((s1 < tile_end ? s1 : tile_end) - (L.step_base + (long long)tile * L.spt));
    const bool whole = (j0 == 0) && (j1 == L.spt);
    float* slot = a.slots + (size_t)(2 * w + (first ? 0 : 1)) * M * kTileRows;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int row = tile * kTileRows + r;
    if (VAR == 1) {
      float acc[MT > 0 ? MT : 1];
      tile_vector<DT, (MT > 0 ? MT : 1), U>(L, tile, j0, j1, acc, lane);
      if (g == 0) {
#pragma unroll
        for (int m = 0; m < (MT > 0 ? MT : 1); ++m) {
          if (whole) {
            if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)acc[m];
          } else {
            slot[m * kTileRows + r] = acc[m];
          }
        }
      }
    } else {
      const f32x4 acc = tile_mfma<DT, U>(L, M, tile, j0, j1, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) {
          const float v = acc[i];
          if (whole) {
            if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)v;
          } else {
            slot[m * kTileRows + r] = v;
          }
        }
      }
    }
    s = tile_end < s1 ? tile_end : s1;
    first = false;
  }
}

// Second pass: block w handles the tile that contains wave w's first step if
// that step lies strictly inside the tile and no earlier wave boundary does.
// Thread t adds token m = t / 16, row r = t % 16 over the contributing waves
// in increasing order and writes y.
__global__ __launch_bounds__(kBlockThreads) void skinny_combine(const LaunchArgs a) {
  const int w = blockIdx.x;
  if (w == 0 || w >= a.G) return;
  const long long b = wave_start(w, a.T, a.G);
  if (b >= a.T) return;
  int l = 0;
  while (l + 1 < a.nlin && a.lin[l + 1].step_base <= b) ++l;
  const LinDesc& L = a.lin[l];
  const long long local = b - L.step_base;
  const int tile = (int)(local / L.spt);
  const long long tstart = L.step_base + (long long)tile * L.spt;
  const long long tend = tstart + L.spt;
  if (b == tstart) return;
  if (wave_start(w - 1, a.T, a.G) > tstart) return;
  const int m = threadIdx.x >> 4;
  const int r = threadIdx.x & 15;
  if (m >= a.M) return;
  float sum = 0.0f;
  for (int v = w - 1; v < a.G; ++v) {
    const long long sv = wave_start(v, a.T, a.G);
    if (sv >= tend) break;
    const long long ev = wave_start(v + 1, a.T, a.G);
    if (ev <= sv) continue;                       // empty wave
    const int slot = 2 * v + (sv >= tstart ? 0 : 1);
    sum += a.slots[((size_t)slot * a.M + m) * kTileRows + r];
  }
  const int row = tile * kTileRows + r;
  if (row < L.N) L.y[(size_t)m * L.N + row] = (__bf16)sum;
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
  return (size_t)kMaxWaves * kSlotsPerWave * (size_t)M * kTileRows * sizeof(float);
}

int auto_variant(int dtype, int M) {
  (void)dtype;
  return M <= 4 ? SKINNY_VARIANT_VECTOR : SKINNY_VARIANT_MFMA;
}

// Loads in flight per lane per batch.  The vector path keeps M x-chunks per
// step live, so its unroll shrinks as M grows to hold occupancy.
template <int DT, int VAR, int MT>
constexpr int unroll_for() {
  if (VAR == SKINNY_VARIANT_MFMA) return 8;
  if (DT == SKINNY_BF16) return MT <= 1 ? 8 : MT <= 2 ? 4 : 2;
  return MT <= 1 ? 4 : 2;
}

typedef void (*main_fn)(LaunchArgs);

template <int DT, int VAR, int MT>
main_fn main_kernel() {
  return skinny_main<DT, VAR, MT, unroll_for<DT, VAR, MT>()>;
}

template <int DT>
main_fn pick_main(int variant, int M) {
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
    default: return nullptr;
  }
}

main_fn pick(int dtype, int variant, int M) {
  return dtype == SKINNY_BF16 ? pick_main<SKINNY_BF16>(variant, M)
                              : pick_main<SKINNY_FP8_BS128>(variant, M);
}

// Persistent grid size: every wave must be resident at once for the equal
// shares to finish together, so take what the occupancy query allows for
// this kernel, capped at kTargetWavesPerCU waves per CU.
constexpr int kTargetWavesPerCU = 16;

skinny_status auto_waves(const DeviceInfo& d, main_fn fn, int* waves) {
  int blocks_per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_per_cu, (const void*)fn,
                                                   kBlockThreads, 0) != hipSuccess)
    return SKINNY_ERR_HIP;
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
                           int M, int variant, int G, float* slots, hipStream_t stream) {
  LaunchArgs a;
  memset(&a, 0, sizeof a);
  a.nlin = count;
  a.M = M;
  a.slots = slots;
  const int dtype = lin[0]->dtype;
  long long T = 0;
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
    d.step_base = T;
    const long long tiles = (L.N + kTileRows - 1) / kTileRows;
    T += tiles * d.spt;
  }
  a.T = T;
  main_fn fn = pick(dtype, variant, M);
  if (!fn) return SKINNY_ERR_INVALID_ARG;
  if (G == 0) {
    skinny_status st = auto_waves(dev, fn, &G);
    if (st != SKINNY_OK) return st;
  }
  if (G > T) G = (int)T;
  if (G < 1) G = 1;
  a.G = G;
  const int blocks = (G + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kBlockThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  if (G > 1) {
    hipLaunchKernelGGL(skinny_combine, dim3(G), dim3(kBlockThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SKINNY_ERR_HIP;
  }
  return SKINNY_OK;
}

skinny_status run(const skinny_linear* lin, int count, int M, const skinny_plan* plan,
                  void* ws, size_t ws_bytes, void* stream) {
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
  DeviceInfo d;
  st = device_info(&d);
  if (st != SKINNY_OK) return st;
  if (!d.gfx950) return SKINNY_ERR_UNSUPPORTED;
  // Group by dtype, in call order, SKINNY_MAX_LINEARS_PER_LAUNCH per launch.
  for (int dt = SKINNY_BF16; dt <= SKINNY_FP8_BS128; ++dt) {
    const int var = variant == SKINNY_VARIANT_AUTO ? auto_variant(dt, M) : variant;
    const skinny_linear* group[SKINNY_MAX_LINEARS_PER_LAUNCH];
    int n = 0;
    for (int i = 0; i < count; ++i) {
      if (lin[i].dtype != dt) continue;
      group[n++] = &lin[i];
      if (n == SKINNY_MAX_LINEARS_PER_LAUNCH) {
        st = launch_group(d, group, n, M, var, waves, (float*)ws, (hipStream_t)stream);
        if (st != SKINNY_OK) return st;
        n = 0;
      }
    }
    if (n > 0) {
      st = launch_group(d, group, n, M, var, waves, (float*)ws, (hipStream_t)stream);
      if (st != SKINNY_OK) return st;
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
  main_fn fn = pick(linears[0].dtype, out->variant, M);
  if (!fn) return SKINNY_ERR_INVALID_ARG;
  return auto_waves(d, fn, &out->waves);
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
