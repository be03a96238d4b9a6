// Kernel argument blocks and host-side launchers of the gfx950 kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/augtree.h"
#include "common.hpp"

namespace augtree {

// ---- transposed copies: X [rows][H][D] -> X^T, tile-major (see common.hpp) ----
struct TransposeArgs {
  const void* src;      // [rows][H][D]
  void* dst;            // [H][cols / tw][D][tw]
  int32_t H;
  int32_t cols;         // padded columns (multiple of 64)
  int32_t tw;           // columns per tile (32 or 64): the consumer's LDS tile width
  int32_t nseg;         // segments: 1 (prompt or a prompt key range) or G (branches)
  BranchTable seg;      // off: source row offsets; pad: column offsets; tile_prefix: pad/64
};

// ---- backward row statistics in transposed-copy column order (see statpack_kernel) ----
struct StatPackArgs {
  const float* lse;     // [H][rows]
  const float* rowdot;  // [H][rows]
  float* out;           // [2][H][cols]
  int32_t H, rows;
  int32_t row0;         // first row of segment 0 in lse/rowdot
  int32_t cols;
  int32_t nseg;
  BranchTable seg;      // as for TransposeArgs
};

// ---- forward: query rows x HG heads per workgroup, 64-key LDS stages ----
enum FwdMode { kFwdPrefill = 0, kFwdReplayPrompt = 1, kFwdReplayLocal = 2 };
constexpr int kFwdBN = 64;   // keys per LDS stage
constexpr int kFwdWaves = 8;  // waves per workgroup

struct FwdArgs {
  const void* q;      // [nq_rows][Hq][D]
  const void* k;      // [nkv_rows][Hkv][D]
  const void* vt;     // transposed copy of V, 64-column tiles: [Hkv][vt_cols / 64][D][64]
  void* o;            // [nq_rows][Hq][D], dtype (prefill) or float32 (replay partials)
  float* lse;         // [Hq][nq_rows]
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows;
  int32_t vt_cols;
  int32_t ntiles;     // query tiles per head slot
  int32_t nwg;        // workgroups in the grid
  float scale_log2;   // softmax scale * log2(e)
  BranchTable bt;     // replay-local: branch offsets, transposed-copy offsets, tile prefix
};

// ---- merge of partial states (normalised output + LSE) per (row, head) ----
constexpr int kMaxParts = 8;
struct MergeArgs {
  const float* o_part[kMaxParts];    // [T][Hq][D] each
  const float* lse_part[kMaxParts];  // [Hq][T] each
  int32_t nparts;
  void* o;            // [T][Hq][D] dtype
  float* lse;         // [Hq][T]
  int32_t rows, Hq;
};

// ---- backward ----
struct RowDotArgs {   // Dv[h][r] = sum_d dO[r][h][d] * O[r][h][d]
  const void* o; const void* dout;
  float* rowdot;      // [Hq][rows]
  int32_t rows, Hq;
};

enum DkdvMode { kDkdvPromptFromReplay = 0, kDkdvLocal = 1, kDkdvPrefill = 2 };
constexpr int kDkdvBM = 32;   // query rows per LDS stage

struct DkdvArgs {
  const void* q; const void* dout;         // [nq_rows][Hq][D]
  const void* qt; const void* dot;         // transposed copies, 32-column tiles [Hq][qt_cols / 32][D][32]
  const float* stats;                      // [2][Hq][qt_cols]: lse * log2(e), rowdot (statpack)
  const void* k; const void* v;            // [nkv_rows][Hkv][D]
  void* dk; void* dv;                      // [nkv_rows][Hkv][D]: dtype, or float32 partials
  const float* init_dk; const float* init_dv;  // prefill: float32 [nkv][Hkv][D] added, or NULL
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows, qt_cols;
  int32_t nktiles;    // workgroups per kv head: key tiles (prefill split: key tile x chunk units)
  int32_t nqtiles;    // prompt-from-replay: query tiles (32-row tiles of every branch)
  int32_t nsplit;     // prompt-from-replay: query tile range split count; prefill: row-tile
                      // chunks (1: unsplit; > 1: float partials per chunk, summed afterwards)
  int32_t zc;         // prefill split: row tiles per chunk (a multiple of 8, whole key blocks)
  int32_t causal;     // 1: a key only sees queries at or after it (branch and prefill walks)
  int32_t nwg;
  int64_t split_stride;  // elements between split partial buffers
  const int32_t* walk;   // prompt-from-replay: per query tile {row byte offset lo, hi, column, rows}
  float scale, scale_log2;
  BranchTable bt;     // branches: offsets, padded offsets, tile prefix (query tiles for
                      // prompt-from-replay, key tiles for the branch walk)
};

// Table of the query tiles of every branch (32-row tiles, branches in order) for the walk of
// the prompt K/V gradient over all branch rows: entry t = {low and high word of row0 * row_bytes,
// column of the tile in the transposed copies, valid rows}. Written by walk_table_kernel.
struct WalkTableArgs {
  int32_t* out;        // [ntiles][4]
  int32_t ntiles;
  int64_t row_bytes;   // bytes between query rows (Hq * D * element size)
  BranchTable bt;      // tile_prefix in 32-row tiles
};

enum DqMode { kDqResponse = 0, kDqPrefill = 1 };
constexpr int kDqBN = 64;

struct DqArgs {
  const void* q; const void* dout;         // [nq_rows][Hq][D]
  const float* lse; const float* rowdot;   // [Hq][nq_rows]
  const void* k; const void* v;            // own keys: prompt (prefill) or response (response)
  const void* kt;                          // transposed own keys, 64-column tiles [Hkv][kt_cols / 64][D][64]
  const void* kp; const void* vp;          // response mode: the prompt keys/values
  const void* kpt;                         // response mode: transposed prompt keys
  void* dq;                                // [nq_rows][Hq][D]
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows, nprompt, kt_cols, kpt_cols;
  int32_t ntiles;
  int32_t nwg;
  int32_t own;        // response mode: 1 = also walk each row's own branch keys (causal)
  float scale, scale_log2;
  BranchTable bt;
};

// Prefill dK/dV from chunk partials: out[i] = (sum_{z >= zmin(key)} part[z][i]) + init[i],
// z ascending, rounded once to the output type; zmin(key) = (key / 256 * 8) / zc is the
// first chunk holding rows the key can see.
struct PrefillReduceArgs {
  const float* part;       // [nz][P][Hkv][D]
  const float* init;       // [P][Hkv][D] or NULL
  void* out;               // [P][Hkv][D] dtype
  int64_t n;               // P * Hkv * D
  int32_t row_elems;       // Hkv * D
  int32_t nz, zc;
};

struct SumPartsArgs {      // out[i] = sum_p part[p][i], p = 0..nparts-1 in order, rounded once
  const float* part[kMaxParts];
  int32_t nparts;
  void* out;              // dtype
  int64_t n;              // elements (a multiple of 4)
};

struct SplitReduceArgs {   // out[i] = sum_s part[s][i], s = 0..nsplit-1 in order
  const float* part;
  float* out;
  int64_t n;              // elements per partial
  int32_t nsplit;
};

// Heads per workgroup of the query-stationary kernels (the waves of a workgroup cover that
// many query heads of one kv group) and query rows per workgroup (8 waves of 32 rows over those
// heads): the dQ kernel, and the forward kernel per mode (FwdMode).
int heads_per_wg(int group);
int rows_per_wg(int group);
int fwd_heads_per_wg(int group, int mode);
int fwd_rows_per_wg(int group, int mode);

// Records `msg` as the calling thread's last error (augtree_last_error) and returns st.
augtree_status set_error(augtree_status st, const char* msg);

hipError_t launch_transpose(int dtype, int D, const TransposeArgs& a, hipStream_t s);
hipError_t launch_statpack(const StatPackArgs& a, hipStream_t s);
hipError_t launch_attn_fwd(int dtype, int D, int mode, const FwdArgs& a, hipStream_t s);
hipError_t launch_merge(int dtype, int D, const MergeArgs& a, hipStream_t s);
hipError_t launch_rowdot(int dtype, int D, const RowDotArgs& a, hipStream_t s);
hipError_t launch_dkdv(int dtype, int D, int mode, const DkdvArgs& a, hipStream_t s);
// f32_out: write float32 partial sums (response mode) instead of dtype
hipError_t launch_dq(int dtype, int D, int mode, bool f32_out, const DqArgs& a, hipStream_t s);
hipError_t launch_sum_parts(int dtype, const SumPartsArgs& a, hipStream_t s);
hipError_t launch_split_reduce(const SplitReduceArgs& a, hipStream_t s);
hipError_t launch_walk_table(const WalkTableArgs& a, hipStream_t s);
hipError_t launch_prefill_reduce(int dtype, const PrefillReduceArgs& a, hipStream_t s);

constexpr int kDkdvKeysPerWG = 256;  // 8 waves x 32 keys

}  // namespace augtree
