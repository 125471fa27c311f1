// Achievable peaks of the device: dense MFMA rates from registers (bf16
// v_mfma_f32_32x32x16_bf16, fp32 v_mfma_f32_32x32x2f32, fp64
// v_mfma_f64_16x16x4f64; short launches, fixed operands), the bf16 rate
// held over a long launch on random operands (32x32x16 and 16x16x32 forms),
// and an HBM copy rate (float4 grid-stride copy of 1 GiB, bytes read +
// written).  A measurement aid for the rooflines of the
// library's kernels, not part of the library.  Prints one JSON object.
//
//     peak_probe            (built next to libpwq.so)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;

constexpr int NACC = 8;   // independent accumulators per wave

__global__ __launch_bounds__(512) void mfma_bf16(float* out, int iters) {
  f32x16_t c[NACC];
  for (int i = 0; i < NACC; ++i)
    for (int r = 0; r < 16; ++r) c[i][r] = 0.0f;
  bf16x8_t x, y;
  for (int e = 0; e < 8; ++e) {
    x[e] = (short)(0x3f80 + (threadIdx.x & 7));
    y[e] = (short)(0x3f00 + e);
  }
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NACC; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c[i], 0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < NACC; ++i) s += c[i][threadIdx.x & 15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same rate held for a long launch on random operands that change with
// every MFMA (four operand sets per lane, loaded from `src`), as in a real
// product: the datapath toggles and the chip settles at the clock its power
// limit allows.
__global__ __launch_bounds__(512) void mfma_bf16_random(const bf16x8_t* __restrict__ src,
                                                        float* out, int iters) {
  f32x16_t c[NACC];
  for (int i = 0; i < NACC; ++i)
    for (int r = 0; r < 16; ++r) c[i][r] = 0.0f;
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t x[4], y[4];
  for (int s = 0; s < 4; ++s) {
    x[s] = src[8 * g + s];
    y[s] = src[8 * g + 4 + s];
  }
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[(i + s) & 3], y[((i >> 1) + s) & 3], c[i],
                                                       0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < NACC; ++i) s += c[i][threadIdx.x & 15];
  out[g] = s;
}

// The same work as v_mfma_f32_16x16x32_bf16 (twice the instructions, a
// quarter of the accumulator data each).
__global__ __launch_bounds__(512) void mfma_bf16_random_16(const bf16x8_t* __restrict__ src,
                                                           float* out, int iters) {
  f32x4_t c[2 * NACC];
  for (int i = 0; i < 2 * NACC; ++i)
    for (int r = 0; r < 4; ++r) c[i][r] = 0.0f;
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t x[4], y[4];
  for (int s = 0; s < 4; ++s) {
    x[s] = src[8 * g + s];
    y[s] = src[8 * g + 4 + s];
  }
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2 * NACC; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[(i + s) & 3], y[((i >> 2) + s) & 3], c[i],
                                                       0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < 2 * NACC; ++i) s += c[i][threadIdx.x & 3];
  out[g] = s;
}

__global__ __launch_bounds__(512) void mfma_f32(float* out, int iters) {
  f32x16_t c[NACC];
  for (int i = 0; i < NACC; ++i)
    for (int r = 0; r < 16; ++r) c[i][r] = 0.0f;
  const float x = 1.0f + (float)(threadIdx.x & 7), y = 0.5f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NACC; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c[i], 0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < NACC; ++i) s += c[i][threadIdx.x & 15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(512) void mfma_f64(float* out, int iters) {
  f64x4_t c[NACC];
  for (int i = 0; i < NACC; ++i)
    for (int r = 0; r < 4; ++r) c[i][r] = 0.0;
  const double x = 1.0 + (double)(threadIdx.x & 7), y = 0.5;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NACC; ++i) c[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, c[i], 0, 0, 0);
  double s = 0.0;
  for (int i = 0; i < NACC; ++i) s += c[i][threadIdx.x & 3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

__global__ __launch_bounds__(256) void copy4(const float4* __restrict__ src, float4* __restrict__ dst,
                                             size_t count) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    dst[i] = src[i];
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "peak_probe: %s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

// TFLOP/s of `kern` on 2 workgroups of 512 threads per CU, best of 3.
template <typename K>
double mfma_rate(K kern, int cus, int iters, double flop_per_wave_iter, float* out) {
  const int wgs = 2 * cus, thr = 512;
  hipEvent_t a, b;
  check(hipEventCreate(&a), "event");
  check(hipEventCreate(&b), "event");
  kern<<<wgs, thr>>>(out, 16);
  check(hipDeviceSynchronize(), "warmup");
  double best = 0.0;
  for (int r = 0; r < 3; ++r) {
    check(hipEventRecord(a), "record");
    kern<<<wgs, thr>>>(out, iters);
    check(hipEventRecord(b), "record");
    check(hipEventSynchronize(b), "sync");
    float ms = 0.0f;
    check(hipEventElapsedTime(&ms, a, b), "elapsed");
    const double tf = flop_per_wave_iter * iters * (thr / 64) * wgs / (ms * 1e-3) / 1e12;
    if (tf > best) best = tf;
  }
  check(hipEventDestroy(a), "event");
  check(hipEventDestroy(b), "event");
  return best;
}

}  // namespace

int main() {
  int dev = 0;
  check(hipGetDevice(&dev), "device");
  hipDeviceProp_t prop;
  check(hipGetDeviceProperties(&prop, dev), "properties");
  const int cus = prop.multiProcessorCount;
  float* out = nullptr;
  check(hipMalloc(&out, (size_t)2 * cus * 512 * sizeof(float)), "malloc");
  // per wave and iteration: NACC MFMAs of 2 M N K flop
  const double bf16 = mfma_rate(mfma_bf16, cus, 4000, NACC * 2.0 * 32 * 32 * 16, out);
  const double f32 = mfma_rate(mfma_f32, cus, 2000, NACC * 2.0 * 32 * 32 * 2, out);
  const double f64 = mfma_rate(mfma_f64, cus, 2000, NACC * 2.0 * 16 * 16 * 4, out);

  // sustained: one launch of 0.1 - 0.2 s on random bf16 operands (a
  // xorshift stream of N(0, 1)-like values: sign, exponent 2^-3 .. 2^2,
  // random mantissa)
  const int wgs = 2 * cus, thr = 512;
  const size_t nvec = (size_t)wgs * thr * 8;
  unsigned short* host = (unsigned short*)std::malloc(nvec * 16);
  if (host == nullptr) check(hipErrorOutOfMemory, "host buffer");
  unsigned long long st = 0x9e3779b97f4a7c15ull;
  for (size_t e = 0; e < nvec * 8; ++e) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    const unsigned sign = (unsigned)(st >> 63) << 15;
    const unsigned expo = 124u + (unsigned)((st >> 40) % 6u);
    host[e] = (unsigned short)(sign | (expo << 7) | (unsigned)(st & 0x7f));
  }
  bf16x8_t* rnd = nullptr;
  check(hipMalloc(&rnd, nvec * 16), "malloc");
  check(hipMemcpy(rnd, host, nvec * 16, hipMemcpyHostToDevice), "copy");
  std::free(host);
  double bf16_sus = 0.0, bf16_sus16 = 0.0;
  {
    const int iters = 50000;   // per iteration 4 NACC MFMAs of 32x32x16 or 8 NACC of 16x16x32
    const double flop = 4.0 * NACC * 2.0 * 32 * 32 * 16 * iters * (thr / 64) * wgs;
    hipEvent_t a, b;
    check(hipEventCreate(&a), "event");
    check(hipEventCreate(&b), "event");
    mfma_bf16_random<<<wgs, thr>>>(rnd, out, 16);
    mfma_bf16_random_16<<<wgs, thr>>>(rnd, out, 16);
    check(hipDeviceSynchronize(), "warmup");
    for (int v = 0; v < 2; ++v) {
      check(hipEventRecord(a), "record");
      if (v == 0)
        mfma_bf16_random<<<wgs, thr>>>(rnd, out, iters);
      else
        mfma_bf16_random_16<<<wgs, thr>>>(rnd, out, iters);
      check(hipEventRecord(b), "record");
      check(hipEventSynchronize(b), "sync");
      float ms = 0.0f;
      check(hipEventElapsedTime(&ms, a, b), "elapsed");
      (v == 0 ? bf16_sus : bf16_sus16) = flop / (ms * 1e-3) / 1e12;
    }
    check(hipEventDestroy(a), "event");
    check(hipEventDestroy(b), "event");
  }
  check(hipFree(rnd), "free");
  check(hipFree(out), "free");

  const size_t bytes = (size_t)1 << 30;
  float4 *src = nullptr, *dst = nullptr;
  check(hipMalloc(&src, bytes), "malloc");
  check(hipMalloc(&dst, bytes), "malloc");
  check(hipMemset(src, 0, bytes), "memset");
  const size_t count = bytes / sizeof(float4);
  const unsigned grid = (unsigned)(cus * 16);
  hipEvent_t a, b;
  check(hipEventCreate(&a), "event");
  check(hipEventCreate(&b), "event");
  copy4<<<grid, 256>>>(src, dst, count);
  check(hipDeviceSynchronize(), "copy warmup");
  double copy_gbs = 0.0;
  for (int r = 0; r < 5; ++r) {
    check(hipEventRecord(a), "record");
    copy4<<<grid, 256>>>(src, dst, count);
    check(hipEventRecord(b), "record");
    check(hipEventSynchronize(b), "sync");
    float ms = 0.0f;
    check(hipEventElapsedTime(&ms, a, b), "elapsed");
    const double gbs = 2.0 * bytes / (ms * 1e-3) / 1e9;
    if (gbs > copy_gbs) copy_gbs = gbs;
  }
  check(hipFree(src), "free");
  check(hipFree(dst), "free");
  std::printf(
      "{\"device\": \"%s\", \"cus\": %d, \"mfma_bf16_tflops\": %.1f, \"mfma_f32_tflops\": %.1f, "
      "\"mfma_f64_tflops\": %.1f, \"copy_gbs\": %.1f, \"mfma_bf16_sustained_random_tflops\": %.1f, "
      "\"mfma_bf16_16x16x32_sustained_random_tflops\": %.1f}\n",
      prop.gcnArchName, cus, bf16, f32, f64, copy_gbs, bf16_sus, bf16_sus16);
  return 0;
}
