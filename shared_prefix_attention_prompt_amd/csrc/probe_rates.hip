// Issue-rate probe of one MI355X (gfx950): what the attention kernels' inner loops can reach.
//
// A standalone program (not part of libaugtree.so), built next to the library by build.py and
// run as `shared_prefix_attention_prompt_amd/probe_rates`. Every kernel runs 8 waves per
// workgroup (two per SIMD), 4 workgroups per compute unit over the whole chip, and loops over
// independent chains held in registers; the only global memory access is one store per thread
// into a buffer of exactly grid x 512 floats, and LDS reads stay inside a 64 KB array.
//
// Part 1, vector issue: wave64 v_fma_f32, v_exp_f32 and two polynomial exp2 (round to nearest,
// Horner on the fraction, exponent added as an integer: the textbook range reduction), alone
// and mixed, reported in FMA issue slots per instruction (one FMA = 1), so no clock is needed.
// Part 2, matrix rate: v_mfma_f32_32x32x16_bf16 chains with register operands, with 1, 1.25 or 2
// 1 KB LDS operand reads per matrix op (ds_read_b128, conflict-free, double buffered), and
// with vector work beside them in the same wave or in the other wave of the SIMD.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 512;

// 2^x for x in the softmax range: x = n + f, n = rint(x), |f| <= 1/2, 2^f by its Taylor
// polynomial of degree DEG (coefficients (ln 2)^k / k!), 2^n added to the exponent field.
template <int DEG>
__device__ inline float exp2_poly(float x) {
  const float n = __builtin_rintf(x);
  const float f = x - n;
  float p;
  if constexpr (DEG == 3) {
    p = __builtin_fmaf(0.0555041086648216f, f, 0.2402265069591007f);
    p = __builtin_fmaf(p, f, 0.6931471805599453f);
    p = __builtin_fmaf(p, f, 1.0f);
  } else {
    p = __builtin_fmaf(0.0013333558146428443f, f, 0.009618129107628477f);
    p = __builtin_fmaf(p, f, 0.0555041086648216f);
    p = __builtin_fmaf(p, f, 0.2402265069591007f);
    p = __builtin_fmaf(p, f, 0.6931471805599453f);
    p = __builtin_fmaf(p, f, 1.0f);
  }
  return __builtin_bit_cast(float, __builtin_bit_cast(int, p) + ((int)n << 23));
}

// Vector chains. KIND: 0 = fma, 1 = v_exp_f32, 2 = degree-3 polynomial, 3 = degree-5
// polynomial, 4 = NV v_exp_f32 chains and 2*NV fma chains.
template <int KIND, int NV>
__global__ __launch_bounds__(kThreads, 1) void vector_chains(float* out, int iters, float a, float b) {
  const int tid = threadIdx.x;
  float x[NV], y[2 * NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = -0.1f * (tid & 7) - 0.01f * i;
#pragma unroll
  for (int i = 0; i < 2 * NV; ++i) y[i] = 0.2f * (tid & 3) + 0.03f * i;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if constexpr (KIND == 0) x[i] = __builtin_fmaf(x[i], a, b);
      if constexpr (KIND == 1 || KIND == 4) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      if constexpr (KIND == 2) x[i] = exp2_poly<3>(-x[i]);
      if constexpr (KIND == 3) x[i] = exp2_poly<5>(-x[i]);
    }
    if constexpr (KIND == 4) {
#pragma unroll
      for (int i = 0; i < 2 * NV; ++i) y[i] = __builtin_fmaf(y[i], a, b);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) s += x[i];
  if constexpr (KIND == 4) {
#pragma unroll
    for (int i = 0; i < 2 * NV; ++i) s += y[i];
  }
  out[blockIdx.x * kThreads + tid] = s;
}

// Matrix chains: 8 matrix ops per iteration over 4 accumulators. NR = LDS operand reads per 8
// ops (0: register operands). VEC: 0 none; 1 = 8 v_exp_f32 and 8 fma per iteration in the same
// wave; 2 = the same vector work in the other wave of each SIMD (waves 4..7), which issues no
// matrix ops.
template <int NR, int VEC>
__global__ __launch_bounds__(kThreads, 1) void matrix_chains(float* out, int iters, float a, float b) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 65536 / 4; i += kThreads) reinterpret_cast<float*>(lds)[i] = 1e-3f * (i & 31);
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  bf16x8 fr, fb;
#pragma unroll
  for (int r = 0; r < 8; ++r) { fr[r] = (__bf16)(0.001f * (tid & 15)); fb[r] = (__bf16)(0.002f * r); }
  float x[8], y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { x[i] = -0.1f * (tid & 7) - 0.01f * i; y[i] = 0.2f * (tid & 3) + 0.03f * i; }
  const bool mat = VEC != 2 || w < 4;
  const bool vec = VEC == 1 || (VEC == 2 && w >= 4);
  // LDS reads: 64 lanes x 16 B = one 1 KB slot each, slots taken in turn from 64 (wrapping)
  const char* base = lds + lane * 16;
  int slot = w * 4;
  auto load = [&](bf16x8 (&d)[16]) {
#pragma unroll
    for (int j = 0; j < NR; ++j) d[j] = *reinterpret_cast<const bf16x8*>(base + (((slot + j) & 63) << 10));
    slot = (slot + NR + 1) & 63;
  };
  auto ops = [&](const bf16x8 (&d)[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x8 fa = fr, fbb = fb;
      if constexpr (NR == 8) fa = d[i];
      if constexpr (NR == 10) { fa = d[i]; if (i < 2) fbb = d[8 + i]; }
      if constexpr (NR == 16) { fa = d[2 * i]; fbb = d[2 * i + 1]; }
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fbb, acc[i & 3], 0, 0, 0);
    }
  };
  auto vwork = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) { x[i] = __builtin_amdgcn_exp2f(-x[i]); y[i] = __builtin_fmaf(y[i], a, b); }
  };
  bf16x8 f[16], g[16];
  if (mat) load(f);
  for (int it = 0; it < iters; it += 2) {
    if (mat) {
      load(g);
      __builtin_amdgcn_sched_barrier(0);
      ops(f);
    }
    if (vec) vwork();
    __builtin_amdgcn_sched_barrier(0);
    if (mat) {
      load(f);
      __builtin_amdgcn_sched_barrier(0);
      ops(g);
    }
    if (vec) vwork();
    __builtin_amdgcn_sched_barrier(0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + y[i];
  out[blockIdx.x * kThreads + tid] = s;
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

// Average milliseconds of one launch over 3 timed launches after one warm-up launch.
template <typename K>
float time_ms(K kernel, float* out, int grid, int iters) {
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, 0, out, iters, 0.5f, 0.25f);
  check(hipGetLastError(), "launch");
  check(hipEventRecord(e0, 0), "record");
  for (int r = 0; r < 3; ++r) hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, 0, out, iters, 0.5f, 0.25f);
  check(hipGetLastError(), "launch");
  check(hipEventRecord(e1, 0), "record");
  check(hipEventSynchronize(e1), "sync");
  float ms = 0.f;
  check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
  check(hipEventDestroy(e0), "event");
  check(hipEventDestroy(e1), "event");
  return ms / 3;
}

}  // namespace

int main() {
  int dev = 0;
  check(hipGetDevice(&dev), "device");
  hipDeviceProp_t prop;
  check(hipGetDeviceProperties(&prop, dev), "properties");
  const int cus = prop.multiProcessorCount;
  const int grid = cus * 4;
  float* out = nullptr;
  check(hipMalloc(&out, (size_t)grid * kThreads * sizeof(float)), "alloc");
  std::printf("device %s, %d compute units, %d workgroups of %d threads\n\n", prop.gcnArchName, cus, grid, kThreads);

  // Part 1: per wave instruction, in FMA issue slots (8 chains of 20000 iterations)
  const int vi = 20000;
  const double fma = time_ms(vector_chains<0, 8>, out, grid, vi) / 8;
  std::printf("vector issue per wave64 instruction, in v_fma_f32 slots\n");
  std::printf("  %-52s %6.2f\n", "v_fma_f32", 1.0);
  std::printf("  %-52s %6.2f\n", "v_exp_f32", time_ms(vector_chains<1, 8>, out, grid, vi) / 8 / fma);
  std::printf("  %-52s %6.2f\n", "exp2, degree-3 polynomial (7 instructions)", time_ms(vector_chains<2, 8>, out, grid, vi) / 8 / fma);
  std::printf("  %-52s %6.2f\n", "exp2, degree-5 polynomial (9 instructions)", time_ms(vector_chains<3, 8>, out, grid, vi) / 8 / fma);
  std::printf("  %-52s %6.2f\n", "v_exp_f32 + 2 v_fma_f32 (mixed; sum if serial: exp + 2)",
              time_ms(vector_chains<4, 8>, out, grid, vi) / 8 / fma);

  // Part 2: matrix ops (8 per iteration, 4000 iterations)
  const int mi = 4000;
  const double flops = (double)grid * 8 * mi * 8 * (2.0 * 32 * 32 * 16);
  auto tf = [&](float ms) { return flops / (ms * 1e-3) / 1e12; };
  std::printf("\nv_mfma_f32_32x32x16_bf16, all 8 waves issuing matrix ops (TFLOP/s over the chip)\n");
  const float m0 = time_ms(matrix_chains<0, 0>, out, grid, mi);
  std::printf("  %-52s %8.1f\n", "register operands", tf(m0));
  std::printf("  %-52s %8.1f\n", "1 KB LDS operand read per matrix op", tf(time_ms(matrix_chains<8, 0>, out, grid, mi)));
  std::printf("  %-52s %8.1f\n", "1.25 KB LDS operand reads per matrix op", tf(time_ms(matrix_chains<10, 0>, out, grid, mi)));
  std::printf("  %-52s %8.1f\n", "2 KB LDS operand reads per matrix op", tf(time_ms(matrix_chains<16, 0>, out, grid, mi)));
  std::printf("  %-52s %8.1f\n", "register operands + 1 v_exp_f32, 1 fma per op, same wave",
              tf(time_ms(matrix_chains<0, 1>, out, grid, mi)));
  // split: only waves 0..3 issue matrix ops, so the chip-wide matrix work is half
  const float ms_split = time_ms(matrix_chains<0, 2>, out, grid, mi);
  std::printf("  %-52s %8.1f  (matrix pipe busy %.0f%% of the all-wave rate)\n",
              "one wave per SIMD matrix ops, the other the vector work", tf(ms_split) / 2, 100.0 * m0 / (2.0 * ms_split));
  std::printf("\nclock-free ratios: the fma slot above is 4 cycles per wave64 instruction by the ISA\n");
  check(hipFree(out), "free");
  std::printf("done\n");
  return 0;
}
