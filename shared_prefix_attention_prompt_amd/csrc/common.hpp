// Building blocks shared by the gfx950 attention kernels: MFMA wrappers, the 32x32
// accumulator layout, and global -> LDS staging in natural and transposed form.
//
// Matrix-core conventions (one wave = 64 lanes, lane l: c = l & 31, g = l >> 5):
//   A operand (M x K): lane holds row c and E consecutive "k slots" of half g.
//   B operand (K x N): lane holds column c and the same E k slots of half g.
//   C / D (32 x 32 fp32, 16 registers): lane holds column c; register r holds row
//   crow(r, g) = 8*(r/4) + 4*g + r%4.
// Only the pairing of A's and B's k slots matters for a contraction, so a k slot may map to
// any k index as long as both operands use the same map. Two maps are used:
//   natural: slot (step s, half g, element i) -> k = s*K + g*E + i (contiguous loads),
//   C map:   slot (s, g, i) -> k = crow(s*E + i, g), i.e. the row order in which an
//            accumulator holds its rows, so that an fp32 accumulator tile can be reused as
//            the next MFMA's operand (softmax probabilities, dS) without any lane exchange.
// An operand paired with a C-map operand is staged transposed in LDS, with its rows
// permuted inside every 16-row group (bits 2 and 3 of the row index swapped, bf16 only)
// so that the E elements one lane needs are contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace augtree {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 waves per workgroup everywhere
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_inff();
constexpr int kMaxBranches = 128;

// Host-built table of the branches, passed by value as a kernel argument.
struct BranchTable {
  int32_t G;
  int32_t off[kMaxBranches + 1];          // packed row offsets of the branches
  int32_t tile_prefix[kMaxBranches + 1];  // first tile index of each branch
};

// Branch owning tile t (tile_prefix[b] <= t < tile_prefix[b+1]).
__device__ inline int branch_of_tile(const BranchTable& bt, int t) {
  int lo = 0, hi = bt.G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (bt.tile_prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int K = 16;  // contraction length of one instruction
  static constexpr int E = 8;   // elements per lane per operand
  using frag = bf16x8;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int K = 2;
  static constexpr int E = 1;
  using frag = float;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __host__ constexpr int crow(int r, int g) { return ((r >> 2) << 3) + (g << 2) + (r & 3); }

// Position of row `k` inside a transposed LDS tile (see header comment).
template <typename T> __device__ constexpr int tpos(int k);
template <> __device__ constexpr int tpos<bf16>(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }
template <> __device__ constexpr int tpos<float>(int k) { return k; }

// First position, inside a 32-row block of a transposed tile, of the elements that step s
// of half g reads (C map).
template <typename T> __device__ constexpr int tread(int s, int g);
template <> __device__ constexpr int tread<bf16>(int s, int g) { return s * 16 + g * 8; }
template <> __device__ constexpr int tread<float>(int s, int g) { return crow(s, g); }

// ---- fragment loads ----
template <typename T> __device__ inline typename Mma<T>::frag load_frag(const T* p);
template <> __device__ inline bf16x8 load_frag<bf16>(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
template <> __device__ inline float load_frag<float>(const float* p) { return *p; }

template <typename T> __device__ inline typename Mma<T>::frag zero_frag();
template <> __device__ inline bf16x8 zero_frag<bf16>() { bf16x8 z; for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f; return z; }
template <> __device__ inline float zero_frag<float>() { return 0.f; }

// Elements s*E .. s*E+E-1 of an accumulator as an operand fragment (C map).
template <typename T> __device__ inline typename Mma<T>::frag acc_frag(const f32x16& a, int s);
template <> __device__ inline bf16x8 acc_frag<bf16>(const f32x16& a, int s) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)a[s * 8 + i];
  return f;
}
template <> __device__ inline float acc_frag<float>(const f32x16& a, int s) { return a[s]; }

__device__ inline f32x16 zero16() { f32x16 z; for (int i = 0; i < 16; ++i) z[i] = 0.f; return z; }

// ---- output stores of an accumulator run of 4 consecutive elements ----
template <typename T> __device__ inline void store4(T* p, float a, float b, float c, float d);
template <> __device__ inline void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v; v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ inline void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v; v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T> __device__ inline f32x4 load4f(const T* p);
template <> __device__ inline f32x4 load4f<bf16>(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  f32x4 r; r[0] = (float)v[0]; r[1] = (float)v[1]; r[2] = (float)v[2]; r[3] = (float)v[3];
  return r;
}
template <> __device__ inline f32x4 load4f<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

__device__ inline float wave_swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// ---------------------------------------------------------------------------------------
// Staging of a ROWS x D tile (rows of a [rows][H][D] tensor, row stride `ld` elements) into
// LDS. Rows at or beyond `nvalid` are filled with zeros.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int ROWS>
struct Stage {
  static constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  static constexpr int CH = D / EPC;               // chunks per row
  static constexpr int NP = D + EPC;               // natural pitch (elements), 16 B pad
  static constexpr int TP = ROWS + EPC;            // transposed pitch (elements), 16 B pad
  static constexpr int NAT_ELEMS = ROWS * NP;
  static constexpr int TR_ELEMS = D * TP;
  static constexpr int NAT_UNITS = ROWS * CH;         // 16 B chunks
  static constexpr int TR_UNITS = (ROWS / 4) * CH;    // 4-row groups
  static constexpr int NAT_PER_THREAD = (NAT_UNITS + kThreads - 1) / kThreads;
  static constexpr int TR_PER_THREAD = (TR_UNITS + kThreads - 1) / kThreads;
  static_assert(NAT_UNITS % kThreads == 0 || NAT_UNITS < kThreads, "natural staging split");
  static_assert(TR_UNITS % kThreads == 0 || TR_UNITS < kThreads, "transposed staging split");

  struct NatRegs { u32x4 v[NAT_PER_THREAD]; };
  struct TrRegs { u32x4 v[TR_PER_THREAD][4]; };

  // natural: chunk c = tid + i*256 -> row c / CH, chunk c % CH (16 lanes span a row)
  __device__ static inline void load_nat(NatRegs& r, const T* src, int64_t ld, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < NAT_PER_THREAD; ++i) {
      int c = tid + i * kThreads;
      int row = c / CH, cc = c % CH;
      if (c < NAT_UNITS && row < nvalid) r.v[i] = *reinterpret_cast<const u32x4*>(src + row * ld + cc * EPC);
      else r.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ static inline void store_nat(const NatRegs& r, T* lds, int tid) {
#pragma unroll
    for (int i = 0; i < NAT_PER_THREAD; ++i) {
      int c = tid + i * kThreads;
      int row = c / CH, cc = c % CH;
      if (c < NAT_UNITS) *reinterpret_cast<u32x4*>(lds + row * NP + cc * EPC) = r.v[i];
    }
  }
  // transposed: group q = tid + i*256 -> rows 4m..4m+3 with m = q % (ROWS/4), chunk q / (ROWS/4)
  __device__ static inline void load_tr(TrRegs& r, const T* src, int64_t ld, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < TR_PER_THREAD; ++i) {
      int q = tid + i * kThreads;
      int m = q % (ROWS / 4), cc = q / (ROWS / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int row = 4 * m + j;
        if (q < TR_UNITS && row < nvalid) r.v[i][j] = *reinterpret_cast<const u32x4*>(src + row * ld + cc * EPC);
        else r.v[i][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // Writes the rows held as 4-row groups (load_tr) in natural layout, so that one set of
  // global loads feeds both LDS copies of a tile.
  __device__ static inline void store_nat_from_tr(const TrRegs& r, T* lds, int tid) {
#pragma unroll
    for (int i = 0; i < TR_PER_THREAD; ++i) {
      int q = tid + i * kThreads;
      int m = q % (ROWS / 4), cc = q / (ROWS / 4);
      if (q >= TR_UNITS) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(lds + (4 * m + j) * NP + cc * EPC) = r.v[i][j];
    }
  }
  // Writes each 4-row group transposed: LDS row (chunk*EPC + e) receives elements e of
  // rows 4m..4m+3 at position tpos(4m) (4 contiguous elements: 8 B for bf16, 16 B for f32).
  __device__ static inline void store_tr(const TrRegs& r, T* lds, int tid) {
#pragma unroll
    for (int i = 0; i < TR_PER_THREAD; ++i) {
      int q = tid + i * kThreads;
      int m = q % (ROWS / 4), cc = q / (ROWS / 4);
      int col = tpos<T>(4 * m);
      if (q >= TR_UNITS) continue;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = (r.v[i][j][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          u32x2 out;
          out[0] = w[0] | (w[1] << 16);
          out[1] = w[2] | (w[3] << 16);
          *reinterpret_cast<u32x2*>(lds + (cc * 8 + e) * TP + col) = out;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 out;
#pragma unroll
          for (int j = 0; j < 4; ++j) out[j] = r.v[i][j][e];
          *reinterpret_cast<u32x4*>(lds + (cc * 4 + e) * TP + col) = out;
        }
      }
    }
  }
};

}  // namespace augtree
