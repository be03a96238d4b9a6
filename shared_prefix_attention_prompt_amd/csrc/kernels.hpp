// Kernel argument blocks and host-side launchers of the gfx950 kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace augtree {

// ---- forward: one Q tile of 128 rows x one query head per workgroup ----
enum FwdMode { kFwdPrefill = 0, kFwdReplayPrompt = 1, kFwdReplayLocal = 2 };
constexpr int kFwdBM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kFwdBN = 64;   // keys per LDS stage

struct FwdArgs {
  const void* q;      // [nq_rows][Hq][D]
  const void* k;      // [nkv_rows][Hkv][D]
  const void* v;
  void* o;            // [nq_rows][Hq][D], dtype (prefill) or float32 (replay partials)
  float* lse;         // [Hq][nq_rows]
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows;
  int32_t ntiles;     // query tiles per head
  float scale_log2;   // softmax scale * log2(e)
  BranchTable bt;     // replay-local only: branch offsets and per-branch tile prefix
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
constexpr int kDkdvBN = 128;  // keys per workgroup (4 waves x 32)
constexpr int kDkdvBM = 64;   // query rows per LDS stage

struct DkdvArgs {
  const void* q; const void* dout;         // [nq_rows][Hq][D]
  const float* lse; const float* rowdot;   // [Hq][nq_rows]
  const void* k; const void* v;            // [nkv_rows][Hkv][D]
  void* dk; void* dv;                      // [nkv_rows][Hkv][D]: dtype, or float32 partials
  const float* init_dk; const float* init_dv;  // prefill: float32 [nkv][Hkv][D] added, or NULL
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows;
  int32_t nktiles;    // key tiles per kv head
  int32_t nsplit;     // prompt-from-replay: query range split count
  int64_t split_stride;  // elements between split partial buffers
  float scale, scale_log2;
  BranchTable bt;     // local only (tile_prefix in units of kDkdvBN keys)
};

enum DqMode { kDqResponse = 0, kDqPrefill = 1 };
constexpr int kDqBM = 128;
constexpr int kDqBN = 64;

struct DqArgs {
  const void* q; const void* dout;         // [nq_rows][Hq][D]
  const float* lse; const float* rowdot;   // [Hq][nq_rows]
  const void* k; const void* v;            // own keys: prompt (prefill) or response (response)
  const void* kp; const void* vp;          // response mode: the prompt keys/values
  void* dq;                                // [nq_rows][Hq][D]
  int32_t Hq, Hkv;
  int32_t nq_rows, nkv_rows, nprompt;
  int32_t ntiles;
  float scale, scale_log2;
  BranchTable bt;
};

struct SplitReduceArgs {   // out[i] = sum_s part[s][i], s = 0..nsplit-1 in order
  const float* part;
  float* out;
  int64_t n;              // elements per partial
  int32_t nsplit;
};

hipError_t launch_attn_fwd(int dtype, int D, int mode, const FwdArgs& a, hipStream_t s);
hipError_t launch_merge(int dtype, int D, const MergeArgs& a, hipStream_t s);
hipError_t launch_rowdot(int dtype, int D, const RowDotArgs& a, hipStream_t s);
hipError_t launch_dkdv(int dtype, int D, int mode, const DkdvArgs& a, hipStream_t s);
hipError_t launch_dq(int dtype, int D, int mode, const DqArgs& a, hipStream_t s);
hipError_t launch_split_reduce(const SplitReduceArgs& a, int nsplit_pairs, hipStream_t s);

}  // namespace augtree
