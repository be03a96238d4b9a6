// Memory-bound kernels around the attention kernels: transposed operand copies, the exact
// merge of partial softmax states, the backward row statistic, and the fixed-order sum of
// split partial gradients.
#include "kernels.hpp"

namespace augtree {

// X [rows][H][D] -> X^T, tile-major: column col of head h, row d sits at
// dst[((h * (cols / tw) + col / tw) * D + d) * tw + col % tw], so that one tw-column tile of
// the consumer (all D rows) is a single contiguous block. One workgroup moves 64 sequence
// positions of one segment (the prompt, a prompt key range, or one branch) and one head.
// Position i of the segment lands in column pad[seg] + (i & ~15) + tpos(i & 15); the padding
// columns of a segment's last tile are zero.
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  constexpr int PITCH = D + 4 / (int)sizeof(T);  // elements per LDS row: odd word stride
  constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                    // chunks per source row
  constexpr int CPC = 64 / EPC;                   // chunks per 64 output columns
  __shared__ __attribute__((aligned(16))) T lds[64 * PITCH];
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int b = a.nseg == 1 ? 0 : branch_of_tile(a.seg, tile);
  const int col0 = tile * 64;
  const int r0 = a.seg.off[b] + (col0 - a.seg.pad[b]);
  const int rend = a.seg.off[b + 1];
  for (int i = tid; i < 64 * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < rend)
      v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.src) +
                                          (((int64_t)(r0 + r) * a.H + h) * D + ch * EPC) * sizeof(T));
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds + r * PITCH + ch * EPC);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  }
  __syncthreads();
  for (int i = tid; i < D * CPC; i += 256) {
    const int d = i / CPC, cc = i % CPC;
    union { T e[EPC]; u32x4 v; } out;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int p = cc * EPC + e;
      out.e[e] = lds[((p & ~15) | tpos<T>(p & 15)) * PITCH + d];
    }
    const int col = col0 + cc * EPC;  // EPC consecutive columns never straddle a tile
    const int64_t idx = (((int64_t)h * (a.cols / a.tw) + col / a.tw) * D + d) * a.tw + col % a.tw;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.dst) + idx * sizeof(T)) = out.v;
  }
}

// Row statistics of the backward in the column layout of the transposed copies, for the
// key-stationary kernels: out[h][col] = lse * log2(e) and out[H + h][col] = rowdot of the
// row held in that column (segment rows in natural order, every segment padded to 64
// columns); padding columns get lse = +inf and rowdot = 0, so they carry zero probability.
__global__ __launch_bounds__(256) void statpack_kernel(StatPackArgs a) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (col >= a.cols) return;
  const int tile = col / kSeg;
  const int b = a.nseg == 1 ? 0 : branch_of_tile(a.seg, tile);
  const int row = a.seg.off[b] + (col - a.seg.pad[b]);
  const bool ok = row < a.seg.off[b + 1];
  const int64_t src = (int64_t)h * a.rows + a.row0 + row;
  a.out[(int64_t)h * a.cols + col] = ok ? a.lse[src] * kLog2e : kInf;
  a.out[(int64_t)(a.H + h) * a.cols + col] = ok ? a.rowdot[src] : 0.f;
}

// Merge of the replay partial states of each (row, head), e.g. the prompt part and the
// response-local part, or the parts of several prompt K/V shards. Each part is a normalised
// output with its LSE; the combined LSE is m + log(sum_i e^(lse_i - m)) with m = max_i lse_i,
// and the combined output is the e^(lse_i - lse)-weighted sum of the parts, which equals
// merging the unnormalised (m, l, O_acc) states ("Splitting Prompt Prefill from Response
// Replay ...", §3.3, Fig. 8). Parts are visited in index order. D/4 lanes handle one
// (row, head), four fp32 elements per lane.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t idx = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int sub = tid % LPR;
  if (idx >= (int64_t)a.rows * a.Hq) return;
  const int64_t row = idx / a.Hq;
  const int h = (int)(idx % a.Hq);
  const int64_t li = (int64_t)h * a.rows + row;
  float l[kMaxParts];
  float mx = -kInf;
#pragma unroll
  for (int i = 0; i < kMaxParts; ++i) {
    l[i] = i < a.nparts ? a.lse_part[i][li] : -kInf;
    mx = fmaxf(mx, l[i]);
  }
  const int64_t off = idx * D + sub * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -kInf;
  if (mx != -kInf) {
    float e[kMaxParts];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      e[i] = i < a.nparts ? __builtin_amdgcn_exp2f((l[i] - mx) * kLog2e) : 0.f;
      s += e[i];
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      if (i < a.nparts && e[i] > 0.f) {
        const float wgt = e[i] * inv;
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.o_part[i] + off);
        acc[0] += wgt * x[0]; acc[1] += wgt * x[1]; acc[2] += wgt * x[2]; acc[3] += wgt * x[3];
      }
    }
    lse = mx + __builtin_amdgcn_logf(s) * kLn2;
  }
  store4<T>(reinterpret_cast<T*>(a.o) + off, acc[0], acc[1], acc[2], acc[3]);
  if (sub == 0) a.lse[li] = lse;
}

// rowdot[h][r] = sum_d dO[r][h][d] * O[r][h][d]; D*sizeof(T)/16 lanes per (row, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(RowDotArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LPR = D / EPC;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t idx = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int sub = tid % LPR;
  const bool valid = idx < (int64_t)a.rows * a.Hq;
  float acc = 0.f;
  if (valid) {
    const int64_t off = idx * D + sub * EPC;
    const T* o = reinterpret_cast<const T*>(a.o) + off;
    const T* d = reinterpret_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int e = 0; e < EPC; e += 4) {
      const f32x4 x = load4f<T>(o + e), y = load4f<T>(d + e);
      acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (valid && sub == 0) {
    const int64_t row = idx / a.Hq;
    const int h = (int)(idx % a.Hq);
    a.rowdot[(int64_t)h * a.rows + row] = acc;
  }
}

// out[i] = part[0][i] + part[1][i] + ... in part order (fixed, so reproducible).
__global__ __launch_bounds__(256) void split_reduce_kernel(SplitReduceArgs a) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= a.n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.part + i4);
  for (int s = 1; s < a.nsplit; ++s) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part + s * a.n + i4);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  *reinterpret_cast<f32x4*>(a.out + i4) = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillReduceArgs a) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= a.n) return;
  const int key = (int)(i4 / a.row_elems);
  const int zmin = (key / kDkdvKeysPerWG * 8) / a.zc;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int z = zmin; z < a.nz; ++z) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part + z * a.n + i4);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  if (a.init != nullptr) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.init + i4);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  store4<T>(reinterpret_cast<T*>(a.out) + i4, acc[0], acc[1], acc[2], acc[3]);
}

// ---------------------------------------------------------------------------------------
hipError_t launch_prefill_reduce(int dtype, const PrefillReduceArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.n % 4 != 0 || a.row_elems % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n / 4 + 255) / 256));
  if (dtype == 1) hipLaunchKernelGGL(prefill_reduce_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(prefill_reduce_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_statpack(const StatPackArgs& a, hipStream_t s) {
  if (a.cols == 0) return hipSuccess;
  hipLaunchKernelGGL(statpack_kernel, dim3((a.cols + 255) / 256, a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, int D, const TransposeArgs& a, hipStream_t s) {
  if (a.cols == 0) return hipSuccess;
  if ((a.tw != 32 && a.tw != 64) || a.cols % 64 != 0) return hipErrorInvalidValue;
  dim3 grid(a.cols / 64, a.H), block(256);
  if (dtype == 1 && D == 128) hipLaunchKernelGGL((transpose_kernel<bf16, 128>), grid, block, 0, s, a);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((transpose_kernel<bf16, 64>), grid, block, 0, s, a);
  else if (dtype == 0 && D == 64) hipLaunchKernelGGL((transpose_kernel<float, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_merge_t(const MergeArgs& a, hipStream_t s) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t n = (int64_t)a.rows * a.Hq;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((n + RPB - 1) / RPB)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int D, const MergeArgs& a, hipStream_t s) {
  if ((int64_t)a.rows * a.Hq == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_merge_t<bf16, 128>(a, s);
  if (dtype == 1 && D == 64) return launch_merge_t<bf16, 64>(a, s);
  if (dtype == 0 && D == 64) return launch_merge_t<float, 64>(a, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_rowdot_t(const RowDotArgs& a, hipStream_t s) {
  constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
  const int64_t n = (int64_t)a.rows * a.Hq;
  hipLaunchKernelGGL((rowdot_kernel<T, D>), dim3((unsigned)((n + RPB - 1) / RPB)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowdot(int dtype, int D, const RowDotArgs& a, hipStream_t s) {
  if ((int64_t)a.rows * a.Hq == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_rowdot_t<bf16, 128>(a, s);
  if (dtype == 1 && D == 64) return launch_rowdot_t<bf16, 64>(a, s);
  if (dtype == 0 && D == 64) return launch_rowdot_t<float, 64>(a, s);
  return hipErrorInvalidValue;
}

// Fixed-order sum of float32 partial sums (e.g. the dQ partials of several prompt-K/V shards
// and of the rows' own branch keys), rounded once to the output type. Four elements per lane.
template <typename T>
__global__ __launch_bounds__(256) void sum_parts_kernel(SumPartsArgs a) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= a.n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.part[0] + i4);
  for (int p = 1; p < a.nparts; ++p) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part[p] + i4);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  store4<T>(reinterpret_cast<T*>(a.out) + i4, acc[0], acc[1], acc[2], acc[3]);
}

hipError_t launch_sum_parts(int dtype, const SumPartsArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n / 4 + 255) / 256));
  if (dtype == 1) hipLaunchKernelGGL(sum_parts_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(sum_parts_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Query-tile table of the prompt K/V gradient walk (see WalkTableArgs): one thread per tile.
__global__ __launch_bounds__(256) void walk_table_kernel(WalkTableArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.ntiles) return;
  const int b = branch_of_tile(a.bt, t);
  const int j = t - a.bt.tile_prefix[b];
  const int row0 = a.bt.off[b] + j * kDkdvBM;
  const int64_t off = (int64_t)row0 * a.row_bytes;
  int32_t* e = a.out + 4 * (int64_t)t;
  e[0] = (int32_t)(uint32_t)(uint64_t)off;
  e[1] = (int32_t)((uint64_t)off >> 32);
  e[2] = a.bt.pad[b] + j * kDkdvBM;
  e[3] = min(kDkdvBM, a.bt.off[b + 1] - row0);
}

hipError_t launch_walk_table(const WalkTableArgs& a, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL(walk_table_kernel, dim3((unsigned)((a.ntiles + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const SplitReduceArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int64_t n4 = a.n / 4;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace augtree
