// synth_gpu.hip - the seeded input generator of synth/__init__.py, on the GPU.
//
// Input generation only: it shares no code with the linear-layer kernels and
// computes nothing of y = x . W^T.  It exists so that weights of the size of
// the whole 80-layer stack (140 GB) can be made in device memory in well under
// a second.  It must agree bit for bit with the numpy generator, which the
// tests check:
//   * Philox4x32-10 (Salmon et al., SC'11): element i takes word i % 4 of
//     philox(counter = (i / 4 low, i / 4 high, 0, 0), key = (seed, stream)).
//   * bf16 normal: bit 31 = sign, bits 0..30 = uniform u; the magnitude code
//     is codes[j] for the first j with u < thresholds[j] (integer search).
//   * FP8 block quantizer: per 128 x 128 block, s = fp32(fp64(amax) / 448),
//     code = nearest E4M3FN value to fp64(w) / fp64(s), ties to even,
//     saturated to +-448; an all-zero block gets s = 0 and codes 0.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

struct u32x4s {
  uint32_t v[4];
};

__device__ __forceinline__ u32x4s philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t p0 = (uint64_t)kM0 * c0;
    const uint64_t p1 = (uint64_t)kM1 * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return u32x4s{{c0, c1, c2, c3}};
}

__device__ __forceinline__ uint16_t word_to_bf16(uint32_t word, const uint32_t* thr,
                                                 const uint16_t* codes, int n) {
  const uint32_t mag = word & 0x7FFFFFFFu;
  // First j with mag < thr[j]; thr[n-1] = 2^31 > mag, so j < n.
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (thr[mid] > mag) hi = mid; else lo = mid + 1;
  }
  const uint16_t c = codes[lo];
  const uint16_t sign = (c != 0 && (word >> 31)) ? 0x8000 : 0;
  return (uint16_t)(c | sign);
}

constexpr int kMaxTable = 8192;

// Grid-stride over blocks of 4 elements; the table is staged in LDS.
__global__ __launch_bounds__(256) void normal_bf16_kernel(uint16_t* out, long long start,
                                                          long long count, uint32_t seed,
                                                          uint32_t stream, const uint32_t* thr,
                                                          const uint16_t* codes, int n) {
  __shared__ uint32_t s_thr[kMaxTable];
  __shared__ uint16_t s_codes[kMaxTable];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    s_thr[i] = thr[i];
    s_codes[i] = codes[i];
  }
  __syncthreads();
  const long long b0 = start >> 2;
  const long long b1 = (start + count - 1) >> 2;
  for (long long b = b0 + blockIdx.x * (long long)blockDim.x + threadIdx.x; b <= b1;
       b += (long long)gridDim.x * blockDim.x) {
    const u32x4s r = philox((uint32_t)b, (uint32_t)(b >> 32), 0u, 0u, seed, stream);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long long i = b * 4 + q;
      if (i >= start && i < start + count) out[i - start] = word_to_bf16(r.v[q], s_thr, s_codes, n);
    }
  }
}

__device__ __forceinline__ double bf16_value(uint16_t c) {
  return (double)__uint_as_float((uint32_t)c << 16);
}

// Nearest E4M3FN code to r, ties to even, saturating at +-448.
__device__ __forceinline__ uint8_t encode_e4m3(double r) {
  double a = fabs(r);
  if (a > 448.0) a = 448.0;
  int ex = 0;
  (void)frexp(a, &ex);                     // a = f 2^ex, f in [0.5, 1)
  int e = ex - 1;
  if (e < -6) e = -6;
  if (e > 8) e = 8;
  const double quantum = ldexp(1.0, e - 3);
  const double val = rint(a / quantum) * quantum;
  uint32_t code = 0;
  if (val != 0.0) {
    int ex2 = 0;
    const double f = frexp(val, &ex2);
    const int ebias = ex2 - 1 + 7;
    if (ebias >= 1) {
      code = ((uint32_t)ebias << 3) | (uint32_t)rint((2.0 * f - 1.0) * 8.0);
    } else {
      code = (uint32_t)rint(val / ldexp(1.0, -9));
    }
    if (r < 0) code |= 0x80u;
  }
  return (uint8_t)code;
}

// One workgroup per 128 x 128 block.
__global__ __launch_bounds__(256) void quantize_bs128_kernel(const uint16_t* w, uint8_t* q,
                                                             float* scale, int N, int K) {
  const int kb = (K + 127) / 128;
  const int bi = blockIdx.x / kb, bj = blockIdx.x % kb;
  const int r0 = bi * 128, c0 = bj * 128;
  const int rows = min(128, N - r0), cols = min(128, K - c0);
  __shared__ float s_max[256];
  float m = 0.0f;
  for (int t = threadIdx.x; t < rows * cols; t += blockDim.x) {
    const int r = t / cols, c = t % cols;
    m = fmaxf(m, fabsf(__uint_as_float((uint32_t)w[(size_t)(r0 + r) * K + c0 + c] << 16)));
  }
  s_max[threadIdx.x] = m;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) s_max[threadIdx.x] = fmaxf(s_max[threadIdx.x], s_max[threadIdx.x + h]);
    __syncthreads();
  }
  const float amax = s_max[0];
  const float s = (float)((double)amax / 448.0);
  if (threadIdx.x == 0) scale[(size_t)bi * kb + bj] = s;
  for (int t = threadIdx.x; t < rows * cols; t += blockDim.x) {
    const int r = t / cols, c = t % cols;
    const size_t i = (size_t)(r0 + r) * K + c0 + c;
    q[i] = (s == 0.0f) ? (uint8_t)0 : encode_e4m3(bf16_value(w[i]) / (double)s);
  }
}

}  // namespace

extern "C" {

// out[0 .. count) = elements start .. start+count-1 of the (seed, stream) bf16
// normal sequence described by (thr, codes, n) (device arrays).  0 on success.
int synth_normal_bf16(void* out, long long start, long long count, unsigned seed,
                      unsigned stream, const void* thr, const void* codes, int n,
                      void* hip_stream) {
  if (count <= 0) return 0;
  if (!out || !thr || !codes || n < 1 || n > kMaxTable || start < 0) return 1;
  const long long blocks4 = ((start + count - 1) >> 2) - (start >> 2) + 1;
  long long grid = (blocks4 + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(normal_bf16_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)hip_stream, (uint16_t*)out, start, count, seed, stream,
                     (const uint32_t*)thr, (const uint16_t*)codes, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// bf16 w[N][K] -> e4m3 q[N][K] and fp32 scale[ceil(N/128)][ceil(K/128)].
int synth_quantize_bs128(const void* w, void* q, void* scale, int N, int K, void* hip_stream) {
  if (!w || !q || !scale || N < 1 || K < 1) return 1;
  const long long blocks = (long long)((N + 127) / 128) * ((K + 127) / 128);
  if (blocks > 0x7FFFFFFF) return 1;
  hipLaunchKernelGGL(quantize_bs128_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)hip_stream, (const uint16_t*)w, (uint8_t*)q, (float*)scale, N, K);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
