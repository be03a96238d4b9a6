// Building blocks shared by the gfx950 attention kernels: matrix-core wrappers and the
// 32x32 accumulator layout, the transposed operand layout, padded LDS tiles filled by direct
// global->LDS copies (per-wave copy plans), the LDS stage pipeline, and small wave-level
// helpers.
//
// Matrix-core conventions (one wave = 64 lanes, lane l: c = l & 31, g = l >> 5):
//   A operand (M x K): lane holds row c and E consecutive "k slots" of half g.
//   B operand (K x N): lane holds column c and the same E k slots of half g.
//   C / D (32 x 32 fp32, 16 registers): lane holds column c; register r holds row
//   crow(r, g) = 8*(r/4) + 4*g + r%4.
// Only the pairing of A's and B's k slots matters for a contraction, so a k slot may map to
// any k index as long as both operands use the same map. Two maps are used:
//   natural: slot (step s, half g, element i) -> k = s*K + g*E + i (contiguous loads),
//   C map:   slot (s, g, i) -> k = crow(s*E + i, g), the row order in which an accumulator
//            holds its rows, so that an fp32 accumulator tile (softmax probabilities, dS)
//            is reused as the next product's operand without any lane exchange.
// The operand paired with a C-map operand must hold, per lane, the E values of one row at
// the k indices of the C map. Such operands come from "transposed copies" written by the
// transpose kernel: X^T[h][d][col] with the sequence index along col, permuted inside every
// 16-column group by tpos() (bits 2 and 3 swapped, bf16) so that the 8 values one lane needs
// are contiguous, and every segment (the prompt, or one branch) padded with zeros to a
// multiple of 64 columns so that tiles never straddle segments. The copies are stored tile by
// tile ([H][cols / tw][D][tw], tw = the consumer's tile width), so one LDS tile of a
// transposed copy is a single contiguous block of memory.
//
// Tiles are copied from global memory into LDS by the direct-to-LDS load (each lane moves 16
// bytes; the 64 lanes of one instruction fill 1 KB of LDS in lane order). A tile row of RB
// bytes is stored at a pitch of RB + 16 bytes, which keeps the 16-byte fragment reads of 16
// consecutive rows on distinct LDS banks and every read address an immediate offset from one
// per-lane base; the lane whose 16 bytes land on a row's pad slot copies any valid chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace augtree {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_inff();
constexpr int kMaxBranches = 128;
constexpr int kSeg = 64;  // padding granule of transposed copies (columns)

// Host-built table of the branches, passed by value as a kernel argument.
struct BranchTable {
  int32_t G;
  int32_t off[kMaxBranches + 1];          // packed row offsets of the branches
  int32_t pad[kMaxBranches + 1];          // column offsets in transposed copies (64-aligned)
  int32_t tile_prefix[kMaxBranches + 1];  // first tile index of each branch (kernel's tile size)
};

// Branch owning tile t (tile_prefix[b] <= t < tile_prefix[b+1]).
__device__ inline int branch_of_tile(const BranchTable& bt, int t) {
  int lo = 0, hi = bt.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bt.tile_prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Dispatch hands consecutive workgroup ids to the 8 XCDs in turn; renumber them so that
// each XCD runs one contiguous range of logical ids, whose tiles share K/V in its L2.
__device__ inline int xcd_remap(int id, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = id & 7, slot = id >> 3;
  return x * per + min(x, rem) + slot;
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

// Column of sequence index i (inside a 64-aligned tile) in a transposed copy.
template <typename T> __device__ __host__ constexpr int tpos(int i);
template <> __device__ __host__ constexpr int tpos<bf16>(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
template <> __device__ __host__ constexpr int tpos<float>(int i) { return i; }

// First column, inside a 32-column block of a transposed tile, of the values that step s of
// half g reads as its C-map k slots.
template <typename T> __device__ constexpr int tread(int s, int g);
template <> __device__ constexpr int tread<bf16>(int s, int g) { return s * 16 + g * 8; }
template <> __device__ constexpr int tread<float>(int s, int g) { return crow(s, g); }

// ---- LDS tiles: RB-byte rows at a pitch of RB + 16 bytes ----
template <int RB>
constexpr int pitch() {
  static_assert(RB % 16 == 0 && RB >= 64 && RB <= 256, "tile rows of 64..256 bytes");
  return RB + 16;
}
// 1 KB blocks a padded tile of ROWS rows occupies.
template <int ROWS, int RB>
constexpr int tile_blocks() { return (ROWS * pitch<RB>() + 1023) / 1024; }
// Byte offset of byte `b` of row `row`.
template <int RB>
__device__ constexpr int tile_off(int row, int b) { return row * pitch<RB>() + b; }

template <typename T> __device__ inline typename Mma<T>::frag lds_frag(const char* tile_base, int off);
template <> __device__ inline bf16x8 lds_frag<bf16>(const char* p, int off) {
  return *reinterpret_cast<const bf16x8*>(p + off);
}
template <> __device__ inline float lds_frag<float>(const char* p, int off) {
  return *reinterpret_cast<const float*>(p + off);
}

// Operand fragment of row `row`, elements [e, e + E) of a natural or transposed LDS tile.
template <typename T, int RB>
__device__ inline typename Mma<T>::frag tile_frag(const char* tile, int row, int e) {
  return lds_frag<T>(tile, tile_off<RB>(row, e * (int)sizeof(T)));
}

// One direct-to-LDS copy: each lane moves 16 bytes from gptr to lds_block + 16 * lane
// (lds_block is the same for the whole wave). It is issued as an opaque instruction: the
// kernels order every copy themselves (explicit waits on the vector-memory counter, then a
// barrier, before any wave reads the stage), and the compiler's own, coarser tracking of
// such copies would otherwise wait for all of them before every LDS read.
__device__ inline void dma16(const void* gptr, char* lds_block) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((LDS_PTR char*)lds_block));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gptr) : "memory", "m0");
}

// Global source of the 16 bytes that lane `lane` lands at byte 1024 b + 16 lane of a padded
// tile whose row r is read from src + min(r, nvalid - 1) * ld (rows past the valid range
// repeat the last valid one and are masked by the callers; pad slots and the slack after the
// last row receive a valid chunk that is never read).
template <int RB>
__device__ inline const char* block_src(const char* src, uint32_t ld, int nvalid, int b, int lane) {
  constexpr int P = pitch<RB>();
  // The per-lane offsets are cheap to recompute; hiding the lane index from the optimiser
  // keeps it from hoisting them out of the tile loop into registers the MFMA loop needs.
  asm volatile("" : "+v"(lane));
  const int byte = b * 1024 + lane * 16;
  const int r = byte / P;
  int o = byte - r * P;
  o = o < RB ? o : 0;
  const uint32_t sr = (uint32_t)min(r, nvalid - 1);
  return src + (sr * ld + (uint32_t)o);
}

// A padded tile to copy: ROWS rows of RB bytes, row r read from src + min(r, nvalid - 1) * ld.
template <int ROWS_, int RB_>
struct TileSrc {
  static constexpr int ROWS = ROWS_, RB = RB_;
  static constexpr int NB = tile_blocks<ROWS, RB>();
  const char* src;
  uint32_t ld;
  int nvalid;
};

template <int OFF>
__device__ __forceinline__ void dma_block_of(char*, int, int) {}
template <int OFF, int ROWS, int RB, typename... Rest>
__device__ __forceinline__ void dma_block_of(char* stage, int k, int lane, const TileSrc<ROWS, RB>& t,
                                             const Rest&... rest) {
  constexpr int NB = TileSrc<ROWS, RB>::NB;
  if (k < OFF + NB) {
    dma16(block_src<RB>(t.src, t.ld, t.nvalid, k - OFF, lane), stage + k * 1024);
    return;
  }
  dma_block_of<OFF + NB>(stage, k, lane, rest...);
}

// 1 KB blocks of a stage made of the given tiles laid out back to back, and the copies each
// of NW waves issues for it.
template <typename... Tiles>
constexpr int stage_blocks() { return (Tiles::NB + ...); }
template <int NW, typename... Tiles>
constexpr int stage_copies() { return (stage_blocks<Tiles...>() + NW - 1) / NW; }

// This wave's share of the copies of one stage: blocks k = w + i * NW (i < stage_copies),
// wrapping past the last block, so every wave issues the same count (two waves landing the
// same block write identical bytes). w must be uniform across the wave.
template <int NW, typename... Tiles>
__device__ __forceinline__ void dma_stage(char* stage, int w, int lane, const Tiles&... tiles) {
  constexpr int TOT = stage_blocks<Tiles...>();
#pragma unroll
  for (int i = 0; i < stage_copies<NW, Tiles...>(); ++i) {
    int k = w + i * NW;
    // opaque here, so that the block tests are not hoisted out of a tile loop (into scalar
    // registers the loop needs)
    asm volatile("" : "+s"(k));
    if (k >= TOT) k -= TOT * (k / TOT);
    dma_block_of<0>(stage, k, lane, tiles...);
  }
}

// ---- copy plans: the same copies, with per-lane offsets computed once per kernel ----
// Block sizes and positions of a stage's tiles (compile time).
template <typename... Tiles>
struct StageLayout {
  static constexpr int N = sizeof...(Tiles);
  static constexpr int nb[N] = {Tiles::NB...};
  static constexpr int TOT = (Tiles::NB + ...);
  static constexpr int first(int t) {
    int s = 0;
    for (int i = 0; i < t; ++i) s += nb[i];
    return s;
  }
  static constexpr int tile_of(int k) {
    int t = 0;
    while (t < N - 1 && k >= first(t + 1)) ++t;
    return t;
  }
};

// Direct copy from a wave-uniform base plus a per-lane 32-bit offset (the scalar-base form
// of the load: no 64-bit address arithmetic per lane).
__device__ inline void dma16_sbase(const char* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(off), "s"(base)
               : "memory", "m0");
}

template <int J, uint32_t MASK, int N>
__device__ __forceinline__ const char* pick_base(int t, const char* const (&b)[N], const char* acc) {
  if constexpr (J == N) {
    return acc;
  } else if constexpr (((MASK >> J) & 1u) == 0) {
    return pick_base<J + 1, MASK>(t, b, acc);
  } else if constexpr ((MASK & ((1u << J) - 1u)) == 0) {
    return pick_base<J + 1, MASK>(t, b, b[J]);  // lowest candidate: the default
  } else {
    return pick_base<J + 1, MASK>(t, b, t == J ? b[J] : acc);
  }
}

// The copies one wave issues per stage (blocks k = w + i * NW, wrapping, as dma_stage) with
// the tile and LDS block of each fixed at kernel start. A stage whose tiles are all complete
// (nvalid >= ROWS) is then issued with one scalar-base load per copy; a stage with a partial
// tile falls back to dma_stage, which clamps rows per lane. HOLD: keep each copy's per-lane
// source offset in a register (one per copy) or, where registers are short, recompute it
// at every issue (a few integer operations per copy).
template <int NW, bool HOLD, typename... Tiles>
struct CopyPlan {
  using L = StageLayout<Tiles...>;
  static constexpr int N = L::N, TOT = L::TOT, DPT = (TOT + NW - 1) / NW;
  static constexpr uint32_t cand(int i) {
    uint32_t m = 0;
    for (int w = 0; w < NW; ++w) m |= 1u << L::tile_of((w + i * NW) % TOT);
    return m;
  }
  int w;
  int tile[DPT];           // wave-uniform
  int kofs[DPT];           // wave-uniform: LDS byte offset of the block in the stage
  uint32_t off[HOLD ? DPT : 1];  // per lane (HOLD)
  uint32_t ld[N];          // wave-uniform (recomputing plans)

  // Source offset of this lane's 16 bytes of block b of tile J (unsigned 24-bit arithmetic:
  // row pitches of tiles with more than two rows are below 2^24 bytes; two-row tiles select).
  template <int J>
  __device__ __forceinline__ static uint32_t tile_lane_off(int b, int lane, uint32_t ld_) {
    using TJ = std::tuple_element_t<J, std::tuple<Tiles...>>;
    constexpr uint32_t P = pitch<TJ::RB>();
    const uint32_t byte = (uint32_t)b * 1024u + (uint32_t)lane * 16u;
    const uint32_t q = byte / P;
    const uint32_t r = q < (uint32_t)(TJ::ROWS - 1) ? q : (uint32_t)(TJ::ROWS - 1);
    uint32_t o = byte - q * P;
    o = o < (uint32_t)TJ::RB ? o : 0u;
    if constexpr (TJ::ROWS <= 2) return (r != 0 ? ld_ : 0u) + o;
    else return (r & 0xffffffu) * (ld_ & 0xffffffu) + o;
  }
  // The same for a tile t known to be one of the tiles in MASK (bit J: tile J).
  template <uint32_t MASK, int J = 0>
  __device__ __forceinline__ static uint32_t lane_off(int t, int b, int lane, const uint32_t (&ld_)[N]) {
    if constexpr (((MASK >> J) & 1u) == 0) {
      return lane_off<MASK, J + 1>(t, b, lane, ld_);
    } else if constexpr ((MASK >> (J + 1)) == 0) {
      return tile_lane_off<J>(b, lane, ld_[J]);  // the last candidate
    } else {
      if (t == J) return tile_lane_off<J>(b, lane, ld_[J]);
      return lane_off<MASK, J + 1>(t, b, lane, ld_);
    }
  }

  __device__ __forceinline__ int first_of(int t) const {
    int f = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) f = t == j ? L::first(j) : f;
    return f;
  }

  template <int I = 0>
  __device__ __forceinline__ void init_slots(int lane, const uint32_t (&ld_)[N]) {
    if constexpr (I < DPT) {
      const int k = (w + I * NW) % TOT;
      int t = 0;
#pragma unroll
      for (int j = 1; j < N; ++j) t += k >= L::first(j) ? 1 : 0;
      tile[I] = t;
      kofs[I] = k * 1024;
      if constexpr (HOLD) off[I] = lane_off<cand(I)>(t, k - first_of(t), lane, ld_);
      init_slots<I + 1>(lane, ld_);
    }
  }

  // ld_[t]: bytes between source rows of tile t.
  __device__ __forceinline__ void init(int w_, int lane, const uint32_t (&ld_)[N]) {
    w = w_;
#pragma unroll
    for (int j = 0; j < N; ++j) ld[j] = ld_[j];
    init_slots(lane, ld_);
  }

  template <int I = 0>
  __device__ __forceinline__ void issue_fast(uint32_t lds, int lane, const char* const (&b)[N]) const {
    if constexpr (I < DPT) {
      // slots that never wrap sit at w + I * NW blocks: one uniform base plus an immediate
      const uint32_t k = (I * NW + NW - 1 < TOT) ? (uint32_t)(w * 1024 + I * NW * 1024) : (uint32_t)kofs[I];
      uint32_t o;
      if constexpr (HOLD) {
        o = off[I];
      } else {
        // hidden from the optimiser, so that it is not hoisted out of the tile loop
        asm volatile("" : "+v"(lane));
        constexpr uint32_t C = cand(I);
        if constexpr ((C & (C - 1)) == 0 && I * NW + NW - 1 < TOT) {
          // a single candidate tile and no wrap: block w + I * NW - first of that tile
          constexpr int J = __builtin_ctz(C);
          o = tile_lane_off<J>(w + I * NW - L::first(J), lane, ld[J]);
        } else {
          o = lane_off<C>(tile[I], kofs[I] / 1024 - first_of(tile[I]), lane, ld);
        }
      }
      dma16_sbase(pick_base<0, cand(I)>(tile[I], b, nullptr), o, lds + k);
      issue_fast<I + 1>(lds, lane, b);
    }
  }

  __device__ __forceinline__ void issue(char* stage, int lane, const Tiles&... tiles) const {
    const bool full = ((tiles.nvalid >= Tiles::ROWS) && ...);
    if (full) {
      const char* const b[N] = {tiles.src...};
      const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((LDS_PTR char*)stage));
      issue_fast(lds, lane, b);
    } else {
      dma_stage<NW>(stage, w, lane, tiles...);
    }
  }
};

// Waits for this wave's outstanding global loads, the direct-to-LDS copies included.
__device__ inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N of this wave's vector-memory loads are outstanding (they complete
// in issue order): vmcnt is bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] stay at
// their maxima.
template <int N>
__device__ inline void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS pipelines: the caller has already waited for the copies and
// LDS reads it needs, so no memory fence is attached (a fence would also wait for the copies
// still in flight for later stages). The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(integral_constant<S>) for S = 0 .. NS-1 (compile-time stage indices).
template <int NS, int S = 0, typename F>
__device__ __forceinline__ void for_stages(F&& f) {
  if constexpr (S < NS) {
    f(std::integral_constant<int, S>{});
    for_stages<NS, S + 1>(f);
  }
}

// Software pipeline over n >= 1 tiles and NS LDS stages: tile it lives in stage it % NS. At
// the start of iteration it the copies of tile it + NS - 1 are issued; before the barrier
// that ends iteration it, this wave's copies of tiles up to it + 1 + LA must have landed, so
// iteration it may read tiles it .. it + LA (LA: how far compute looks ahead). DPT is the
// number of copies one wave issues per tile. Past the last tile the free stage receives a
// repeat of tile n - 1 (never read), so every iteration issues the same number of copies and
// every wait is the same: at most (NS - 2 - LA) * DPT copies in flight. issue(it, stage) and
// compute(it, stage) take the stage as an integral_constant so that each stage is its own
// LDS object.
template <int NS, int DPT, int LA = 0, typename Issue, typename Compute>
__device__ __forceinline__ void run_pipeline(int n, Issue&& issue, Compute&& compute) {
  static_assert(NS >= 2 + LA && (NS - 2 - LA) * DPT < 64, "pipeline depth");
  wait_vm();  // the caller's own loads are done: inside, only copies count on vmcnt
  for_stages<NS - 1>([&](auto S) { issue(min((int)S, n - 1), S); });
  wait_vm_le<(NS - 2 - LA) * DPT>();
  stage_barrier();
  for (int base = 0; base < n; base += NS) {
    for_stages<NS>([&](auto S) {
      constexpr int st = decltype(S)::value;
      const int it = base + st;
      if (it >= n) return;
      issue(min(it + NS - 1, n - 1), std::integral_constant<int, (st + NS - 1) % NS>{});
      compute(it, S);
      wait_vm_le<(NS - 2 - LA) * DPT>();
      stage_barrier();
    });
  }
  wait_vm();  // repeats still landing must finish before the workgroup's LDS is released
}

// ---- accumulator helpers ----
// Elements s*E .. s*E+E-1 of an accumulator as an operand fragment (C map).
template <typename T> __device__ inline typename Mma<T>::frag acc_frag(const f32x16& a, int s);
template <> __device__ inline bf16x8 acc_frag<bf16>(const f32x16& a, int s) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)a[s * 8 + i];
  return f;
}
template <> __device__ inline float acc_frag<float>(const f32x16& a, int s) { return a[s]; }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Value of the same lane index in the other half of the wave, combined: f(x, x^32).
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the 8 bf16 values of a fragment (as the matrix cores see them) added to acc.
__device__ inline float frag_sum(const bf16x8& f, float acc) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {f[2 * i], f[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
  return acc;
}
__device__ inline float frag_sum(float f, float acc) { return acc + f; }

// ---- output stores of an accumulator run of 4 consecutive elements ----
template <typename T> __device__ inline void store4(T* p, float a, float b, float c, float d);
template <> __device__ inline void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ inline void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T> __device__ inline f32x4 load4f(const T* p);
template <> __device__ inline f32x4 load4f<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ inline f32x4 load4f<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Operand fragment straight from global memory (E consecutive elements).
template <typename T> __device__ inline typename Mma<T>::frag gload_frag(const T* p);
template <> __device__ inline bf16x8 gload_frag<bf16>(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
template <> __device__ inline float gload_frag<float>(const float* p) { return *p; }
template <typename T> __device__ inline typename Mma<T>::frag zero_frag();
template <> __device__ inline bf16x8 zero_frag<bf16>() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}
template <> __device__ inline float zero_frag<float>() { return 0.f; }

}  // namespace augtree
