// Host side of the C ABI declared in include/augtree.h: argument validation, workspace
// layout, branch tables, transposed operand copies and the launch sequence of each entry
// point. Nothing here allocates, frees or synchronises; all work goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/augtree.h"
#include "kernels.hpp"

// Scratch of augtree_replay_fwd_noalloc: one copy per GPU, allocated when the library's code
// object is loaded on that GPU and held until the process ends. In host code this name only
// stands for the symbol; its device address comes from hipGetSymbolAddress (noalloc_scratch).
static __device__ __align__(256) char scratch[AUGTREE_NOALLOC_SCRATCH_BYTES];

namespace augtree {
namespace {

thread_local std::string t_last_error;

augtree_status fail(augtree_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
augtree_status fail(augtree_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return st;
}

struct Shape {
  int P = 0, G = 0, Hq = 0, Hkv = 0, D = 0, dtype = 0, T = 0;
  float scale = 0.f;
  int off[kMaxBranches + 1] = {};
  int pad[kMaxBranches + 1] = {};  // branch column offsets in transposed copies
  size_t esz() const { return dtype == AUGTREE_BF16 ? 2 : 4; }
  int Tp() const { return pad[G]; }  // padded columns of a response transposed copy
};

int pad64(int n) { return (n + kSeg - 1) / kSeg * kSeg; }

augtree_status check_dims(const augtree_dims* d, Shape* s) {
  if (d == nullptr) return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->prompt_len < 1) return fail(AUGTREE_ERR_INVALID_ARGUMENT, "prompt_len %d < 1", d->prompt_len);
  if (d->num_branches < 1 || d->num_branches > AUGTREE_MAX_BRANCHES)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "num_branches %d outside [1, %d]", d->num_branches,
                AUGTREE_MAX_BRANCHES);
  if (d->branch_offsets == nullptr) return fail(AUGTREE_ERR_INVALID_ARGUMENT, "branch_offsets is NULL");
  if (d->branch_offsets[0] != 0)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "branch_offsets[0] = %d, must be 0", d->branch_offsets[0]);
  for (int i = 0; i < d->num_branches; ++i)
    if (d->branch_offsets[i + 1] <= d->branch_offsets[i])
      return fail(AUGTREE_ERR_INVALID_ARGUMENT,
                  "branch_offsets not strictly increasing at branch %d (%d -> %d); every branch needs >= 1 token",
                  i, d->branch_offsets[i], d->branch_offsets[i + 1]);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hkv=%d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "num_q_heads %d not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim < 1) return fail(AUGTREE_ERR_INVALID_ARGUMENT, "head_dim %d < 1", d->head_dim);
  if (!(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale))
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (d->dtype != AUGTREE_F32 && d->dtype != AUGTREE_BF16)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dtype %d is not AUGTREE_F32 or AUGTREE_BF16", d->dtype);
  if (d->dtype == AUGTREE_BF16 && d->head_dim != 64 && d->head_dim != 128)
    return fail(AUGTREE_ERR_UNSUPPORTED, "bf16 head_dim %d not built (64 or 128)", d->head_dim);
  if (d->dtype == AUGTREE_F32 && d->head_dim != 64)
    return fail(AUGTREE_ERR_UNSUPPORTED, "f32 head_dim %d not built (64)", d->head_dim);
  // the tile copies compute per-lane source offsets as row x row-pitch in 24-bit arithmetic
  const int64_t pitch = (int64_t)d->num_q_heads * d->head_dim * (d->dtype == AUGTREE_BF16 ? 2 : 4);
  if (pitch >= (int64_t)1 << 24)
    return fail(AUGTREE_ERR_UNSUPPORTED, "num_q_heads x head_dim x element size = %lld bytes per row, "
                "must be below 2^24", (long long)pitch);
  // every index of the kernels (elements of one tensor, rows x heads) stays in 32 bits
  const int64_t T = d->branch_offsets[d->num_branches];
  const int64_t rows = T > d->prompt_len ? T : d->prompt_len;
  if ((rows + (int64_t)kSeg * d->num_branches) * d->num_q_heads * d->head_dim > INT32_MAX)
    return fail(AUGTREE_ERR_UNSUPPORTED, "rows x heads x head_dim beyond 2^31 elements");
  s->P = d->prompt_len;
  s->G = d->num_branches;
  s->Hq = d->num_q_heads;
  s->Hkv = d->num_kv_heads;
  s->D = d->head_dim;
  s->dtype = d->dtype;
  s->scale = d->softmax_scale;
  s->pad[0] = 0;
  for (int i = 0; i <= s->G; ++i) s->off[i] = d->branch_offsets[i];
  for (int i = 0; i < s->G; ++i) s->pad[i + 1] = s->pad[i] + pad64(s->off[i + 1] - s->off[i]);
  s->T = s->off[s->G];
  return AUGTREE_OK;
}

augtree_status check_ptr(const void* p, const char* name, bool may_be_null = false) {
  if (p == nullptr) {
    if (may_be_null) return AUGTREE_OK;
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  }
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return AUGTREE_OK;
}

#define CHECK(expr)                              \
  do {                                           \
    augtree_status st__ = (expr);                \
    if (st__ != AUGTREE_OK) return st__;         \
  } while (0)

#define LAUNCH(expr, what)                                                                   \
  do {                                                                                       \
    hipError_t e__ = (expr);                                                                 \
    if (e__ != hipSuccess) return fail(AUGTREE_ERR_HIP, "%s: %s", what, hipGetErrorString(e__)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- workspace pieces ----
// Transposed copies: [H][D][cols] of dtype.
size_t tr_bytes(const Shape& s, int H, int cols) { return align_up((size_t)H * s.D * cols * s.esz()); }
size_t tr_prompt(const Shape& s, int H) { return tr_bytes(s, H, pad64(s.P)); }
size_t tr_resp(const Shape& s, int H) { return tr_bytes(s, H, s.Tp()); }
// Row statistics of the key-stationary kernels: [2][Hq][cols] float32.
size_t st_prompt(const Shape& s) { return align_up((size_t)2 * s.Hq * pad64(s.P) * sizeof(float)); }
size_t st_resp(const Shape& s) { return align_up((size_t)2 * s.Hq * s.Tp() * sizeof(float)); }

// Split count of the prompt dK/dV pass over the branches' rows for `nkeys` prompt keys. One
// workgroup runs per compute unit at a time (LDS-bound), so a grid of W workgroups takes
// ceil(W / 256) rounds; a fractional last round leaves units idle. Among n = 1..16 parts
// (never more than the query tiles) giving at least two rounds of workgroups where that is
// possible, the count with the least modelled time is taken: ceil(wgs n / 256) rounds of
// T_R / n rows each, plus writing and re-reading the n float32 partial sums (two tensors of
// nkeys x Hkv x D, at about 5 TB/s against about 4.3 TFLOP/s per compute unit on the
// products, i.e. nkeys * Hkv * 0.0067 / group row-walks per part).
int prompt_split(const Shape& s, int nkeys) {
  const int64_t wgs = (int64_t)((nkeys + kDkdvKeysPerWG - 1) / kDkdvKeysPerWG) * s.Hkv;
  int64_t qtiles = 0;
  for (int i = 0; i < s.G; ++i) qtiles += (s.off[i + 1] - s.off[i] + kDkdvBM - 1) / kDkdvBM;
  const int64_t nmax = std::max<int64_t>(1, std::min<int64_t>(16, qtiles));
  const double reduce = (double)nkeys * s.Hkv * 0.0067 / (s.Hq / s.Hkv);
  int best = 1;
  double best_cost = 0.0;
  bool best_fills = false;
  for (int64_t n = 1; n <= nmax; ++n) {
    const int64_t w = wgs * n;
    const bool fills = w >= 512 || n == nmax;
    const double cost = (double)((w + 255) / 256) * (double)((s.T + n - 1) / n) + (n > 1 ? (double)n * reduce : 0.0);
    if (n == 1 || (fills && !best_fills) || (fills == best_fills && cost < best_cost)) {
      best = (int)n;
      best_cost = cost;
      best_fills = fills;
    }
  }
  return best;
}

// Row-tile chunks of the prefill dK/dV walk. When the key blocks fill the GPU (about two
// rounds of one-per-CU workgroups), long prompts are cut into chunks of about 8192 rows so that
// concurrent walks share rows in L2; otherwise the chunk count (whole key blocks of rows each,
// at most 16) is the one with the least modelled time. A key block only has units for the
// chunks holding rows it can see.
struct PrefillSplit { int nz, zc, units; };
PrefillSplit prefill_split(const Shape& s) {
  const int nt = (s.P + kDkdvBM - 1) / kDkdvBM;
  const int nk = (s.P + kDkdvKeysPerWG - 1) / kDkdvKeysPerWG;
  constexpr int kTilesPerKeyBlock = kDkdvKeysPerWG / kDkdvBM;
  PrefillSplit best{1, nt, nk};
  if ((int64_t)nk * s.Hkv >= 512) {
    // Enough key blocks to fill the GPU. Long prompts are still cut into (at most 8) chunks of
    // about kLockstepTiles row tiles: a key block's causal walk then starts at its chunk's end
    // together with the other key blocks of that chunk instead of at the prompt's end at
    // whatever time its workgroup starts, so the rows stay shared in L2.
    constexpr int kLockstepTiles = 256;
    if (nt < 2 * kLockstepTiles) return best;
    const int want = std::min(8, nt / kLockstepTiles);
    const int per = (nt + want - 1) / want;
    const int zc = (per + kTilesPerKeyBlock - 1) / kTilesPerKeyBlock * kTilesPerKeyBlock;
    const int nz = (nt + zc - 1) / zc;
    int units = 0;
    for (int kb = 0; kb < nk; ++kb) units += nz - (kb * kTilesPerKeyBlock) / zc;
    return PrefillSplit{nz, zc, units};
  }
  // Too few key blocks to fill the GPU: the fewest-cost chunk count. Units are uneven (a key
  // block sees only the rows after it), so the pass takes about the average work per compute
  // unit plus half the longest unit; each chunk adds its float32 partial sums (written once,
  // read once by the reduce, at about 5 TB/s). Times in row-tile walks of one workgroup
  // (32 rows x 256 keys per query head, about 2 us at the measured matrix rate).
  const int group = s.Hq / s.Hkv;
  const double tile_us = 1.95 * group;
  double best_cost = 1e300;
  for (int want = 1; want <= 16; ++want) {
    const int per = (nt + want - 1) / want;
    const int zc = (per + kTilesPerKeyBlock - 1) / kTilesPerKeyBlock * kTilesPerKeyBlock;
    const int nz = (nt + zc - 1) / zc;
    if (want > 1 && nz <= best.nz) continue;
    int units = 0;
    int64_t tiles = 0;
    int longest = 0;
    for (int kb = 0; kb < nk; ++kb) {
      for (int z = (kb * kTilesPerKeyBlock) / zc; z < nz; ++z) {
        const int len = std::min(nt, (z + 1) * zc) - std::max(kb * kTilesPerKeyBlock, z * zc);
        ++units;
        tiles += len;
        longest = std::max(longest, len);
      }
    }
    const double pass = ((double)tiles * s.Hkv / 256.0 + 0.5 * longest) * tile_us;
    const double partial = nz > 1 ? (double)nz * s.P * s.Hkv * s.D * 16.0 / 5e6 : 0.0;
    if (pass + partial < best_cost) {
      best_cost = pass + partial;
      best = PrefillSplit{nz, nz > 1 ? zc : nt, units};
    }
  }
  return best;
}

size_t prefill_split_ws(const Shape& s) {
  const PrefillSplit ps = prefill_split(s);
  return ps.nz > 1 ? align_up((size_t)2 * ps.nz * s.P * s.Hkv * s.D * sizeof(float)) : 0;
}

// Key rows of split partials (parts x keys) reserved for augtree_replay_prompt_bwd: the
// largest parts x keys over ranges of whole 256-key blocks (the whole prompt included). A
// range of any other length takes at most this many (split_for_range clamps its part count),
// so the reserve depends on the dims alone.
int64_t prompt_split_cap(const Shape& s) {
  int64_t best = 0;
  const int nkt = (s.P + kDkdvKeysPerWG - 1) / kDkdvKeysPerWG;
  for (int t = 1; t <= nkt; ++t) {
    const int nk = t == nkt ? s.P : t * kDkdvKeysPerWG;
    const int n = prompt_split(s, nk);
    if (n > 1) best = std::max<int64_t>(best, (int64_t)n * nk);
  }
  return best;
}

// Split count of the prompt dK/dV pass over `nkeys` keys: the modelled best, lowered where
// n x nkeys would exceed the reserve (a choice of summation grouping only: any count gives the
// same sums up to fp32 rounding, and it depends on dims and range alone, so results stay
// bitwise reproducible).
int split_for_range(const Shape& s, int nkeys, int64_t cap_keys) {
  int n = prompt_split(s, nkeys);
  if (n > 1 && (int64_t)n * nkeys > cap_keys) n = (int)(cap_keys / nkeys);
  return n > 1 ? n : 1;
}

// Bytes of split partials (dK and dV) for a reserve of cap_keys key rows.
size_t split_bytes(const Shape& s, int64_t cap_keys) {
  return align_up((size_t)2 * cap_keys * s.Hkv * s.D * sizeof(float));
}

// Reserve of the composite backward, which only runs the range [0, P).
int64_t prompt_split_cap_whole(const Shape& s) {
  const int n = prompt_split(s, s.P);
  return n > 1 ? (int64_t)n * s.P : 0;
}

// Query-tile walk table of the prompt K/V gradient over all branch rows: 16 bytes per 32-row tile.
size_t walk_bytes(const Shape& s) {
  int64_t t = 0;
  for (int i = 0; i < s.G; ++i) t += (s.off[i + 1] - s.off[i] + kDkdvBM - 1) / kDkdvBM;
  return align_up((size_t)t * 16);
}

// Layout of a workspace as consecutive 256-byte aligned pieces.
struct Layout {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t at = total;
    total += align_up(bytes);
    return at;
  }
};

struct ReplayFwdWs { size_t o_a, o_b, lse_a, lse_b, vpt, vrt, total; };
ReplayFwdWs replay_fwd_ws(const Shape& s) {
  ReplayFwdWs w;
  Layout l;
  w.o_a = l.add((size_t)s.T * s.Hq * s.D * sizeof(float));
  w.o_b = l.add((size_t)s.T * s.Hq * s.D * sizeof(float));
  w.lse_a = l.add((size_t)s.T * s.Hq * sizeof(float));
  w.lse_b = l.add((size_t)s.T * s.Hq * sizeof(float));
  w.vpt = l.add(tr_prompt(s, s.Hkv));
  w.vrt = l.add(tr_resp(s, s.Hkv));
  w.total = l.total;
  return w;
}

struct ReplayBwdWs { size_t rowdot, qrt, dort, stats, kpt, krt, walk, split, total; };
ReplayBwdWs replay_bwd_ws(const Shape& s) {
  ReplayBwdWs w;
  Layout l;
  w.rowdot = l.add((size_t)s.T * s.Hq * sizeof(float));
  w.qrt = l.add(tr_resp(s, s.Hq));
  w.dort = l.add(tr_resp(s, s.Hq));
  w.stats = l.add(st_resp(s));
  w.kpt = l.add(tr_prompt(s, s.Hkv));
  w.krt = l.add(tr_resp(s, s.Hkv));
  w.walk = l.add(walk_bytes(s));
  w.split = l.add(split_bytes(s, prompt_split_cap_whole(s)));
  w.total = l.total;
  return w;
}

struct PrefillBwdWs { size_t rowdot, qpt, dopt, stats, kpt, split, total; };
PrefillBwdWs prefill_bwd_ws(const Shape& s) {
  PrefillBwdWs w;
  Layout l;
  w.rowdot = l.add((size_t)s.P * s.Hq * sizeof(float));
  w.qpt = l.add(tr_prompt(s, s.Hq));
  w.dopt = l.add(tr_prompt(s, s.Hq));
  w.stats = l.add(st_prompt(s));
  w.kpt = l.add(tr_prompt(s, s.Hkv));
  w.split = l.add(prefill_split_ws(s));
  w.total = l.total;
  return w;
}

size_t op_workspace(const Shape& s, int op) {
  switch (op) {
    case AUGTREE_OP_PREFILL_FWD: return tr_prompt(s, s.Hkv);
    case AUGTREE_OP_REPLAY_FWD: return replay_fwd_ws(s).total;
    case AUGTREE_OP_REPLAY_BWD: return replay_bwd_ws(s).total;
    case AUGTREE_OP_PREFILL_BWD: return prefill_bwd_ws(s).total;
    case AUGTREE_OP_REPLAY_PROMPT_BWD:
      return 2 * tr_resp(s, s.Hq) + st_resp(s) + walk_bytes(s) + split_bytes(s, prompt_split_cap(s));
    case AUGTREE_OP_REPLAY_PROMPT_FWD: return tr_prompt(s, s.Hkv);
    case AUGTREE_OP_REPLAY_LOCAL_FWD: return tr_resp(s, s.Hkv);
    case AUGTREE_OP_REPLAY_LOCAL_BWD: return 2 * tr_resp(s, s.Hq) + st_resp(s);
    case AUGTREE_OP_REPLAY_DQ: return tr_prompt(s, s.Hkv) + tr_resp(s, s.Hkv);
    case AUGTREE_OP_PREFILL_KV_BWD: return 2 * tr_prompt(s, s.Hq) + st_prompt(s) + prefill_split_ws(s);
    case AUGTREE_OP_PREFILL_DQ: return tr_prompt(s, s.Hkv);
    case AUGTREE_OP_REPLAY_PROMPT_DQ: return tr_prompt(s, s.Hkv);
    case AUGTREE_OP_REPLAY_LOCAL_DQ: return tr_resp(s, s.Hkv);
  }
  return 0;
}

// Workspace of a call over prompt keys [kb, ke) (ops that take a key range; others: op_workspace).
size_t range_workspace(const Shape& s, int op, int kb, int ke) {
  const int nkeys = ke - kb;
  switch (op) {
    case AUGTREE_OP_REPLAY_PROMPT_FWD:
    case AUGTREE_OP_REPLAY_PROMPT_DQ: return tr_bytes(s, s.Hkv, pad64(nkeys));
    case AUGTREE_OP_REPLAY_PROMPT_BWD: {
      const int n = split_for_range(s, nkeys, prompt_split_cap(s));
      return 2 * tr_resp(s, s.Hq) + st_resp(s) + walk_bytes(s) + (n > 1 ? split_bytes(s, (int64_t)n * nkeys) : 0);
    }
  }
  return op_workspace(s, op);
}

augtree_status check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return AUGTREE_OK;
  if (ws == nullptr) return fail(AUGTREE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (have < need) return fail(AUGTREE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(AUGTREE_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
  return AUGTREE_OK;
}

// Table of the branches; tile_prefix counts tiles of `tile` rows per branch.
BranchTable branch_table(const Shape& s, int tile) {
  BranchTable bt;
  memset(&bt, 0, sizeof(bt));
  bt.G = s.G;
  int acc = 0;
  for (int i = 0; i <= s.G; ++i) {
    bt.off[i] = s.off[i];
    bt.pad[i] = s.pad[i];
    bt.tile_prefix[i] = acc;
    if (i < s.G) acc += (s.off[i + 1] - s.off[i] + tile - 1) / tile;
  }
  return bt;
}

int total_tiles(const BranchTable& bt) { return bt.tile_prefix[bt.G]; }

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---- transposed copies ----
// rows [r0, r0 + n) of x [rows][H][D] (one segment) -> [H][pad64(n) / tw][D][tw].
augtree_status transpose_range(const Shape& s, const void* x, int H, int r0, int n, int tw, void* dst,
                               hipStream_t st) {
  TransposeArgs a;
  memset(&a, 0, sizeof(a));
  a.tw = tw;
  a.src = static_cast<const char*>(x) + (size_t)r0 * H * s.D * s.esz();
  a.dst = dst;
  a.H = H;
  a.cols = pad64(n);
  a.nseg = 1;
  a.seg.G = 1;
  a.seg.off[0] = 0;
  a.seg.off[1] = n;
  a.seg.pad[0] = 0;
  a.seg.pad[1] = a.cols;
  a.seg.tile_prefix[0] = 0;
  a.seg.tile_prefix[1] = a.cols / kSeg;
  LAUNCH(launch_transpose(s.dtype, s.D, a, st), "transposed copy");
  return AUGTREE_OK;
}

// all branches of x [T_R][H][D] -> [H][Tp / tw][D][tw], every branch padded to 64 columns.
augtree_status transpose_branches(const Shape& s, const void* x, int H, int tw, void* dst, hipStream_t st) {
  TransposeArgs a;
  memset(&a, 0, sizeof(a));
  a.tw = tw;
  a.src = x;
  a.dst = dst;
  a.H = H;
  a.cols = s.Tp();
  a.nseg = s.G;
  a.seg.G = s.G;
  for (int i = 0; i <= s.G; ++i) {
    a.seg.off[i] = s.off[i];
    a.seg.pad[i] = s.pad[i];
    a.seg.tile_prefix[i] = s.pad[i] / kSeg;
  }
  LAUNCH(launch_transpose(s.dtype, s.D, a, st), "transposed copy (branches)");
  return AUGTREE_OK;
}

// Row statistics (lse * log2(e), rowdot) of the prompt rows or the branch rows in the
// column order of the matching transposed copies.
augtree_status pack_stats_prompt(const Shape& s, const float* lse, const float* rowdot, float* out, hipStream_t st) {
  StatPackArgs a;
  memset(&a, 0, sizeof(a));
  a.lse = lse; a.rowdot = rowdot; a.out = out;
  a.H = s.Hq; a.rows = s.P; a.row0 = 0; a.cols = pad64(s.P); a.nseg = 1;
  a.seg.G = 1; a.seg.off[1] = s.P; a.seg.pad[1] = a.cols; a.seg.tile_prefix[1] = a.cols / kSeg;
  LAUNCH(launch_statpack(a, st), "row statistics (prompt)");
  return AUGTREE_OK;
}

augtree_status pack_stats_branches(const Shape& s, const float* lse, const float* rowdot, float* out,
                                   hipStream_t st) {
  StatPackArgs a;
  memset(&a, 0, sizeof(a));
  a.lse = lse; a.rowdot = rowdot; a.out = out;
  a.H = s.Hq; a.rows = s.T; a.row0 = 0; a.cols = s.Tp(); a.nseg = s.G;
  a.seg.G = s.G;
  for (int i = 0; i <= s.G; ++i) {
    a.seg.off[i] = s.off[i];
    a.seg.pad[i] = s.pad[i];
    a.seg.tile_prefix[i] = s.pad[i] / kSeg;
  }
  LAUNCH(launch_statpack(a, st), "row statistics (branches)");
  return AUGTREE_OK;
}

// ---------------------------------------------------------------------------------------
// Single steps on validated shapes (no argument checks here). Transposed copies are passed
// in, already written.
// ---------------------------------------------------------------------------------------
// head slots of the dQ kernel's grid (query heads / heads per workgroup)
int heads_slots(const Shape& s) { return s.Hq / heads_per_wg(s.Hq / s.Hkv); }

augtree_status step_prefill_fwd(const Shape& s, const void* q_p, const void* k_p, const void* vpt, void* o_p,
                                float* lse_p, hipStream_t st) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_p; a.k = k_p; a.vt = vpt; a.o = o_p; a.lse = lse_p;
  a.Hq = s.Hq; a.Hkv = s.Hkv;
  a.nq_rows = s.P; a.nkv_rows = s.P; a.vt_cols = pad64(s.P);
  const int rt = fwd_rows_per_wg(s.Hq / s.Hkv, kFwdPrefill);
  a.ntiles = (s.P + rt - 1) / rt;
  a.nwg = a.ntiles * (s.Hq / fwd_heads_per_wg(s.Hq / s.Hkv, kFwdPrefill));
  a.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdPrefill, a, st), "prefill forward");
  return AUGTREE_OK;
}

// vt: transposed copy of prompt V rows [kb, ke) (pad64(ke - kb) columns)
augtree_status step_replay_prompt_fwd(const Shape& s, const void* k_p, const void* vt, const void* q_r, int kb,
                                      int ke, float* o_part, float* lse_part, hipStream_t st) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_r;
  a.k = static_cast<const char*>(k_p) + (size_t)kb * s.Hkv * s.D * s.esz();
  a.vt = vt;
  a.o = o_part; a.lse = lse_part;
  a.Hq = s.Hq; a.Hkv = s.Hkv;
  a.nq_rows = s.T; a.nkv_rows = ke - kb; a.vt_cols = pad64(ke - kb);
  const int rt = fwd_rows_per_wg(s.Hq / s.Hkv, kFwdReplayPrompt);
  a.ntiles = (s.T + rt - 1) / rt;
  a.nwg = a.ntiles * (s.Hq / fwd_heads_per_wg(s.Hq / s.Hkv, kFwdReplayPrompt));
  a.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdReplayPrompt, a, st), "replay forward (prompt keys)");
  return AUGTREE_OK;
}

augtree_status step_replay_local_fwd(const Shape& s, const void* q_r, const void* k_r, const void* vrt,
                                     float* o_part, float* lse_part, hipStream_t st) {
  FwdArgs b;
  memset(&b, 0, sizeof(b));
  b.q = q_r; b.k = k_r; b.vt = vrt; b.o = o_part; b.lse = lse_part;
  b.Hq = s.Hq; b.Hkv = s.Hkv;
  b.nq_rows = s.T; b.nkv_rows = s.T; b.vt_cols = s.Tp();
  b.bt = branch_table(s, fwd_rows_per_wg(s.Hq / s.Hkv, kFwdReplayLocal));
  b.ntiles = total_tiles(b.bt);
  b.nwg = b.ntiles * (s.Hq / fwd_heads_per_wg(s.Hq / s.Hkv, kFwdReplayLocal));
  b.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdReplayLocal, b, st), "replay forward (branch keys)");
  return AUGTREE_OK;
}

augtree_status step_merge(const Shape& s, int n, const float* const* o_parts, const float* const* lse_parts,
                          void* o_r, float* lse_r, hipStream_t st) {
  MergeArgs m;
  memset(&m, 0, sizeof(m));
  for (int i = 0; i < n; ++i) {
    m.o_part[i] = o_parts[i];
    m.lse_part[i] = lse_parts[i];
  }
  m.nparts = n;
  m.o = o_r; m.lse = lse_r; m.rows = s.T; m.Hq = s.Hq;
  LAUNCH(launch_merge(s.dtype, s.D, m, st), "merge of partial states");
  return AUGTREE_OK;
}

augtree_status step_row_dot(const Shape& s, int rows, const void* o, const void* d_o, float* rowdot,
                            hipStream_t st) {
  RowDotArgs r;
  r.o = o; r.dout = d_o; r.rowdot = rowdot; r.rows = rows; r.Hq = s.Hq;
  LAUNCH(launch_rowdot(s.dtype, s.D, r, st), "row dot");
  return AUGTREE_OK;
}

// qrt/dort: transposed branch copies of q_r / do_r; split: split-partial workspace
// walk: walk-table region (walk_bytes); split: split-partial region of split_have bytes;
// cap_keys: the reserve the split count is clamped to (parts x keys)
augtree_status step_replay_prompt_bwd(const Shape& s, const void* k_p, const void* v_p, const void* q_r,
                                      const void* qrt, const float* stats, const void* do_r, const void* dort,
                                      int kb, int ke, float* dk_acc, float* dv_acc, void* walk, void* split,
                                      size_t split_have, int64_t cap_keys, hipStream_t st) {
  const int nkeys = ke - kb;
  const int nsplit = split_for_range(s, nkeys, cap_keys);
  if (nsplit > 1 && (size_t)2 * nsplit * nkeys * s.Hkv * s.D * sizeof(float) > split_have)
    return fail(AUGTREE_ERR_WORKSPACE, "prompt dK/dV split partials of %d parts x %d keys exceed the %zu bytes "
                "left in the workspace", nsplit, nkeys, split_have);
  const size_t koff = (size_t)kb * s.Hkv * s.D;
  const int64_t part = (int64_t)nkeys * s.Hkv * s.D;
  float* part_dk = static_cast<float*>(split);
  float* part_dv = part_dk + (nsplit > 1 ? (int64_t)nsplit * part : 0);
  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_r; p.dout = do_r; p.qt = qrt; p.dot = dort; p.stats = stats;
  p.k = static_cast<const char*>(k_p) + koff * s.esz();
  p.v = static_cast<const char*>(v_p) + koff * s.esz();
  p.nsplit = nsplit;
  p.causal = 0;
  p.dk = nsplit > 1 ? static_cast<void*>(part_dk) : static_cast<void*>(dk_acc + koff);
  p.dv = nsplit > 1 ? static_cast<void*>(part_dv) : static_cast<void*>(dv_acc + koff);
  p.split_stride = part;
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.T; p.nkv_rows = nkeys; p.qt_cols = s.Tp();
  p.nktiles = (nkeys + kDkdvKeysPerWG - 1) / kDkdvKeysPerWG;
  p.bt = branch_table(s, kDkdvBM);
  p.nqtiles = total_tiles(p.bt);
  p.nwg = p.nktiles * s.Hkv * nsplit;
  p.walk = static_cast<const int32_t*>(walk);
  WalkTableArgs wt;
  memset(&wt, 0, sizeof(wt));
  wt.out = static_cast<int32_t*>(walk);
  wt.ntiles = p.nqtiles;
  wt.row_bytes = (int64_t)s.Hq * s.D * s.esz();
  wt.bt = p.bt;
  LAUNCH(launch_walk_table(wt, st), "walk table (prompt dK/dV)");
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPromptFromReplay, p, st), "prompt dK/dV from branches");
  if (nsplit > 1) {
    SplitReduceArgs sr;
    sr.n = part;
    sr.nsplit = nsplit;
    sr.part = part_dk;
    sr.out = dk_acc + koff;
    LAUNCH(launch_split_reduce(sr, st), "split reduce (dK)");
    sr.part = part_dv;
    sr.out = dv_acc + koff;
    LAUNCH(launch_split_reduce(sr, st), "split reduce (dV)");
  }
  return AUGTREE_OK;
}

augtree_status step_replay_local_bwd(const Shape& s, const void* q_r, const void* qrt, const void* k_r,
                                     const void* v_r, const float* stats, const void* do_r, const void* dort,
                                     void* dk_r, void* dv_r, hipStream_t st) {
  DkdvArgs l;
  memset(&l, 0, sizeof(l));
  l.q = q_r; l.dout = do_r; l.qt = qrt; l.dot = dort; l.stats = stats;
  l.k = k_r; l.v = v_r; l.dk = dk_r; l.dv = dv_r;
  l.Hq = s.Hq; l.Hkv = s.Hkv;
  l.nq_rows = s.T; l.nkv_rows = s.T; l.qt_cols = s.Tp();
  l.bt = branch_table(s, kDkdvKeysPerWG);
  l.nktiles = total_tiles(l.bt);
  l.nsplit = 1;
  l.causal = 1;
  l.nwg = l.nktiles * s.Hkv;
  l.scale = s.scale; l.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvLocal, l, st), "branch dK/dV");
  return AUGTREE_OK;
}

augtree_status step_replay_dq(const Shape& s, const void* k_p, const void* kpt, const void* v_p, const void* q_r,
                              const void* k_r, const void* krt, const void* v_r, const float* lse_r,
                              const float* rowdot_r, const void* do_r, void* dq_r, hipStream_t st) {
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_r; q.dout = do_r; q.lse = lse_r; q.rowdot = rowdot_r;
  q.k = k_r; q.v = v_r; q.kt = krt; q.kp = k_p; q.vp = v_p; q.kpt = kpt; q.dq = dq_r;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.T; q.nkv_rows = s.T; q.nprompt = s.P;
  q.kt_cols = s.Tp(); q.kpt_cols = pad64(s.P);
  q.bt = branch_table(s, rows_per_wg(s.Hq / s.Hkv));
  q.ntiles = total_tiles(q.bt);
  q.nwg = q.ntiles * heads_slots(s);
  q.own = 1;
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqResponse, false, q, st), "branch dQ");
  return AUGTREE_OK;
}

// float32 dQ partial of every branch row over prompt keys [kb, ke) only; kpt: transposed copy
// of the range's K (pad64(ke - kb) columns)
augtree_status step_replay_prompt_dq(const Shape& s, const void* k_p, const void* kpt, const void* v_p,
                                     const void* q_r, const float* lse_r, const float* rowdot_r, const void* do_r,
                                     int kb, int ke, float* dq_part, hipStream_t st) {
  const size_t koff = (size_t)kb * s.Hkv * s.D * s.esz();
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_r; q.dout = do_r; q.lse = lse_r; q.rowdot = rowdot_r;
  q.kp = static_cast<const char*>(k_p) + koff;
  q.vp = static_cast<const char*>(v_p) + koff;
  q.kpt = kpt;
  q.k = q.kp; q.v = q.vp; q.kt = kpt;  // own keys are not walked
  q.dq = dq_part;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.T; q.nkv_rows = s.T; q.nprompt = ke - kb;
  q.kt_cols = pad64(ke - kb); q.kpt_cols = pad64(ke - kb);
  q.bt = branch_table(s, rows_per_wg(s.Hq / s.Hkv));
  q.ntiles = total_tiles(q.bt);
  q.nwg = q.ntiles * heads_slots(s);
  q.own = 0;
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqResponse, true, q, st), "branch dQ partial (prompt key range)");
  return AUGTREE_OK;
}

// float32 dQ partial of every branch row over its own branch keys (causal)
augtree_status step_replay_local_dq(const Shape& s, const void* q_r, const void* k_r, const void* krt,
                                    const void* v_r, const float* lse_r, const float* rowdot_r, const void* do_r,
                                    float* dq_part, hipStream_t st) {
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_r; q.dout = do_r; q.lse = lse_r; q.rowdot = rowdot_r;
  q.k = k_r; q.v = v_r; q.kt = krt; q.kp = k_r; q.vp = v_r; q.kpt = krt;  // no prompt keys walked
  q.dq = dq_part;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.T; q.nkv_rows = s.T; q.nprompt = 0;
  q.kt_cols = s.Tp(); q.kpt_cols = s.Tp();
  q.bt = branch_table(s, rows_per_wg(s.Hq / s.Hkv));
  q.ntiles = total_tiles(q.bt);
  q.nwg = q.ntiles * heads_slots(s);
  q.own = 1;
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqResponse, true, q, st), "branch dQ partial (own branch keys)");
  return AUGTREE_OK;
}

// split: chunk-partial workspace (prefill_split_ws bytes; unused when unsplit)
augtree_status step_prefill_kv_bwd(const Shape& s, const void* q_p, const void* qpt, const void* k_p,
                                   const void* v_p, const float* stats, const void* do_p, const void* dopt,
                                   const float* dk_acc, const float* dv_acc, void* dk_p, void* dv_p,
                                   void* split, hipStream_t st) {
  const PrefillSplit ps = prefill_split(s);
  const int64_t part = (int64_t)s.P * s.Hkv * s.D;
  float* part_dk = static_cast<float*>(split);
  float* part_dv = part_dk + (ps.nz > 1 ? (int64_t)ps.nz * part : 0);
  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_p; p.dout = do_p; p.qt = qpt; p.dot = dopt; p.stats = stats;
  p.k = k_p; p.v = v_p;
  if (ps.nz > 1) {
    p.dk = part_dk; p.dv = part_dv;  // float partials; the reduce adds dk_acc/dv_acc
  } else {
    p.dk = dk_p; p.dv = dv_p;
    p.init_dk = dk_acc; p.init_dv = dv_acc;
  }
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.P; p.nkv_rows = s.P; p.qt_cols = pad64(s.P);
  p.nktiles = ps.units;
  p.nsplit = ps.nz;
  p.zc = ps.zc;
  p.split_stride = part;
  p.causal = 1;
  p.nwg = ps.units * s.Hkv;
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPrefill, p, st), "prefill dK/dV");
  if (ps.nz > 1) {
    PrefillReduceArgs r;
    r.n = part; r.row_elems = s.Hkv * s.D; r.nz = ps.nz; r.zc = ps.zc;
    r.part = part_dk; r.init = dk_acc; r.out = dk_p;
    LAUNCH(launch_prefill_reduce(s.dtype, r, st), "prefill chunk reduce (dK)");
    r.part = part_dv; r.init = dv_acc; r.out = dv_p;
    LAUNCH(launch_prefill_reduce(s.dtype, r, st), "prefill chunk reduce (dV)");
  }
  return AUGTREE_OK;
}

augtree_status step_prefill_dq(const Shape& s, const void* q_p, const void* k_p, const void* kpt, const void* v_p,
                               const float* lse_p, const float* rowdot_p, const void* do_p, void* dq_p,
                               hipStream_t st) {
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_p; q.dout = do_p; q.lse = lse_p; q.rowdot = rowdot_p;
  q.k = k_p; q.v = v_p; q.kt = kpt; q.dq = dq_p;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.P; q.nkv_rows = s.P; q.nprompt = 0;
  q.kt_cols = pad64(s.P);
  const int rt = rows_per_wg(s.Hq / s.Hkv);
  q.ntiles = (s.P + rt - 1) / rt;
  q.nwg = q.ntiles * heads_slots(s);
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqPrefill, false, q, st), "prefill dQ");
  return AUGTREE_OK;
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept; the only mutable state of the library.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

augtree_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AUGTREE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(AUGTREE_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(AUGTREE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AUGTREE_OK;
}

// augtree_replay_fwd on validated shapes with a workspace of replay_fwd_ws(s).total bytes
augtree_status replay_fwd_on(const Shape& s, const void* k_p, const void* v_p, const void* q_r, const void* k_r,
                             const void* v_r, void* o_r, float* lse_r, void* ws, hipStream_t st) {
  const ReplayFwdWs w = replay_fwd_ws(s);
  float* o_parts[2] = {reinterpret_cast<float*>(at(ws, w.o_a)), reinterpret_cast<float*>(at(ws, w.o_b))};
  float* l_parts[2] = {reinterpret_cast<float*>(at(ws, w.lse_a)), reinterpret_cast<float*>(at(ws, w.lse_b))};
  CHECK(transpose_range(s, v_p, s.Hkv, 0, s.P, 64, at(ws, w.vpt), st));
  CHECK(transpose_branches(s, v_r, s.Hkv, 64, at(ws, w.vrt), st));
  // (1) every branch row against the whole, unmasked prompt K/V: partial state a
  CHECK(step_replay_prompt_fwd(s, k_p, at(ws, w.vpt), q_r, 0, s.P, o_parts[0], l_parts[0], st));
  // (2) every branch row against its own branch, causally: partial state b
  CHECK(step_replay_local_fwd(s, q_r, k_r, at(ws, w.vrt), o_parts[1], l_parts[1], st));
  // (3) log-sum-exp merge of a and b
  const float* co[2] = {o_parts[0], o_parts[1]};
  const float* cl[2] = {l_parts[0], l_parts[1]};
  return step_merge(s, 2, co, cl, o_r, lse_r, st);
}

augtree_status check_key_range(const Shape& s, int kb, int ke) {
  if (kb < 0 || ke > s.P || kb >= ke)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "prompt key range [%d, %d) not inside [0, %d) or empty", kb, ke, s.P);
  return AUGTREE_OK;
}

}  // namespace

augtree_status set_error(augtree_status st, const char* msg) {
  t_last_error = msg;
  return st;
}

}  // namespace augtree

using namespace augtree;

#define PTR(p) CHECK(check_ptr((p), #p))
#define PTR_OR_NULL(p) CHECK(check_ptr((p), #p, true))

extern "C" {

int augtree_abi_version(void) { return AUGTREE_ABI_VERSION; }

const char* augtree_status_string(augtree_status st) {
  switch (st) {
    case AUGTREE_OK: return "AUGTREE_OK";
    case AUGTREE_ERR_INVALID_ARGUMENT: return "AUGTREE_ERR_INVALID_ARGUMENT";
    case AUGTREE_ERR_UNSUPPORTED: return "AUGTREE_ERR_UNSUPPORTED";
    case AUGTREE_ERR_WORKSPACE: return "AUGTREE_ERR_WORKSPACE";
    case AUGTREE_ERR_HIP: return "AUGTREE_ERR_HIP";
  }
  return "AUGTREE_ERR_UNKNOWN";
}

const char* augtree_last_error(void) { return t_last_error.c_str(); }

size_t augtree_range_workspace_bytes(const augtree_dims* dims, int op, int32_t key_begin, int32_t key_end) {
  Shape s;
  const std::string saved = t_last_error;
  if (check_dims(dims, &s) != AUGTREE_OK || key_begin < 0 || key_end > s.P || key_begin >= key_end) {
    t_last_error = saved;
    return 0;
  }
  return range_workspace(s, op, key_begin, key_end);
}

size_t augtree_workspace_bytes(const augtree_dims* dims, int op) {
  Shape s;
  const std::string saved = t_last_error;
  if (check_dims(dims, &s) != AUGTREE_OK) {
    t_last_error = saved;
    return 0;
  }
  return op_workspace(s, op);
}

// ---- single steps ----

augtree_status augtree_replay_prompt_fwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                         const void* q_r, int32_t key_begin, int32_t key_end, float* o_part,
                                         float* lse_part, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_key_range(s, key_begin, key_end));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(o_part); PTR(lse_part);
  CHECK(check_ws(ws, ws_bytes, range_workspace(s, AUGTREE_OP_REPLAY_PROMPT_FWD, key_begin, key_end)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_range(s, v_p, s.Hkv, key_begin, key_end - key_begin, 64, ws, st));
  return step_replay_prompt_fwd(s, k_p, ws, q_r, key_begin, key_end, o_part, lse_part, st);
}

augtree_status augtree_replay_local_fwd(const augtree_dims* dims, const void* q_r, const void* k_r,
                                        const void* v_r, float* o_part, float* lse_part, void* ws,
                                        size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_part); PTR(lse_part);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_REPLAY_LOCAL_FWD)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_branches(s, v_r, s.Hkv, 64, ws, st));
  return step_replay_local_fwd(s, q_r, k_r, ws, o_part, lse_part, st);
}

augtree_status augtree_merge_partials(const augtree_dims* dims, int32_t num_parts, const float* const* o_parts,
                                      const float* const* lse_parts, void* o_r, float* lse_r, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  if (num_parts < 1 || num_parts > AUGTREE_MAX_PARTS)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "num_parts %d outside [1, %d]", num_parts, AUGTREE_MAX_PARTS);
  if (o_parts == nullptr || lse_parts == nullptr)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "o_parts and lse_parts must be host arrays");
  for (int i = 0; i < num_parts; ++i) {
    CHECK(check_ptr(o_parts[i], "o_parts[i]"));
    CHECK(check_ptr(lse_parts[i], "lse_parts[i]"));
  }
  PTR(o_r); PTR(lse_r);
  return step_merge(s, num_parts, o_parts, lse_parts, o_r, lse_r, static_cast<hipStream_t>(stream));
}

augtree_status augtree_row_dot(const augtree_dims* dims, int32_t rows, const void* o, const void* d_o,
                               float* rowdot, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  if (rows != s.P && rows != s.T)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "rows %d is neither P=%d nor T_R=%d", rows, s.P, s.T);
  PTR(o); PTR(d_o); PTR(rowdot);
  return step_row_dot(s, rows, o, d_o, rowdot, static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_prompt_bwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                         const void* q_r, const float* lse_r, const float* rowdot_r,
                                         const void* do_r, int32_t key_begin, int32_t key_end, float* dk_p_acc,
                                         float* dv_p_acc, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_key_range(s, key_begin, key_end));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dk_p_acc); PTR(dv_p_acc);
  CHECK(check_ws(ws, ws_bytes, range_workspace(s, AUGTREE_OP_REPLAY_PROMPT_BWD, key_begin, key_end)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* qrt = ws;
  void* dort = at(ws, tr_resp(s, s.Hq));
  float* stats = reinterpret_cast<float*>(at(ws, 2 * tr_resp(s, s.Hq)));
  void* walk = at(ws, 2 * tr_resp(s, s.Hq) + st_resp(s));
  void* split = at(ws, 2 * tr_resp(s, s.Hq) + st_resp(s) + walk_bytes(s));
  const size_t split_have = ws_bytes - (2 * tr_resp(s, s.Hq) + st_resp(s) + walk_bytes(s));
  CHECK(transpose_branches(s, q_r, s.Hq, 32, qrt, st));
  CHECK(transpose_branches(s, do_r, s.Hq, 32, dort, st));
  CHECK(pack_stats_branches(s, lse_r, rowdot_r, stats, st));
  return step_replay_prompt_bwd(s, k_p, v_p, q_r, qrt, stats, do_r, dort, key_begin, key_end, dk_p_acc, dv_p_acc,
                                walk, split, split_have, prompt_split_cap(s), st);
}

augtree_status augtree_replay_local_bwd(const augtree_dims* dims, const void* q_r, const void* k_r,
                                        const void* v_r, const float* lse_r, const float* rowdot_r,
                                        const void* do_r, void* dk_r, void* dv_r, void* ws, size_t ws_bytes,
                                        void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_r); PTR(k_r); PTR(v_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dk_r); PTR(dv_r);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_REPLAY_LOCAL_BWD)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* qrt = ws;
  void* dort = at(ws, tr_resp(s, s.Hq));
  float* stats = reinterpret_cast<float*>(at(ws, 2 * tr_resp(s, s.Hq)));
  CHECK(transpose_branches(s, q_r, s.Hq, 32, qrt, st));
  CHECK(transpose_branches(s, do_r, s.Hq, 32, dort, st));
  CHECK(pack_stats_branches(s, lse_r, rowdot_r, stats, st));
  return step_replay_local_bwd(s, q_r, qrt, k_r, v_r, stats, do_r, dort, dk_r, dv_r, st);
}

augtree_status augtree_replay_dq(const augtree_dims* dims, const void* k_p, const void* v_p, const void* q_r,
                                 const void* k_r, const void* v_r, const float* lse_r, const float* rowdot_r,
                                 const void* do_r, void* dq_r, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dq_r);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_REPLAY_DQ)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* kpt = ws;
  void* krt = at(ws, tr_prompt(s, s.Hkv));
  CHECK(transpose_range(s, k_p, s.Hkv, 0, s.P, 64, kpt, st));
  CHECK(transpose_branches(s, k_r, s.Hkv, 64, krt, st));
  return step_replay_dq(s, k_p, kpt, v_p, q_r, k_r, krt, v_r, lse_r, rowdot_r, do_r, dq_r, st);
}

augtree_status augtree_replay_prompt_dq(const augtree_dims* dims, const void* k_p, const void* v_p,
                                        const void* q_r, const float* lse_r, const float* rowdot_r,
                                        const void* do_r, int32_t key_begin, int32_t key_end, float* dq_part,
                                        void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_key_range(s, key_begin, key_end));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dq_part);
  CHECK(check_ws(ws, ws_bytes, range_workspace(s, AUGTREE_OP_REPLAY_PROMPT_DQ, key_begin, key_end)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_range(s, k_p, s.Hkv, key_begin, key_end - key_begin, 64, ws, st));
  return step_replay_prompt_dq(s, k_p, ws, v_p, q_r, lse_r, rowdot_r, do_r, key_begin, key_end, dq_part, st);
}

augtree_status augtree_replay_local_dq(const augtree_dims* dims, const void* q_r, const void* k_r, const void* v_r,
                                       const float* lse_r, const float* rowdot_r, const void* do_r, float* dq_part,
                                       void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_r); PTR(k_r); PTR(v_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dq_part);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_REPLAY_LOCAL_DQ)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_branches(s, k_r, s.Hkv, 64, ws, st));
  return step_replay_local_dq(s, q_r, k_r, ws, v_r, lse_r, rowdot_r, do_r, dq_part, st);
}

augtree_status augtree_sum_parts(const augtree_dims* dims, int32_t rows, int32_t num_parts, const float* const* parts,
                                 void* out, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  if (rows != s.P && rows != s.T)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "rows %d is neither P=%d nor T_R=%d", rows, s.P, s.T);
  if (num_parts < 1 || num_parts > AUGTREE_MAX_PARTS)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "num_parts %d outside [1, %d]", num_parts, AUGTREE_MAX_PARTS);
  if (parts == nullptr) return fail(AUGTREE_ERR_INVALID_ARGUMENT, "parts must be a host array");
  for (int i = 0; i < num_parts; ++i) CHECK(check_ptr(parts[i], "parts[i]"));
  PTR(out);
  SumPartsArgs a;
  memset(&a, 0, sizeof(a));
  for (int i = 0; i < num_parts; ++i) a.part[i] = parts[i];
  a.nparts = num_parts;
  a.out = out;
  a.n = (int64_t)rows * s.Hq * s.D;
  LAUNCH(launch_sum_parts(s.dtype, a, static_cast<hipStream_t>(stream)), "sum of partials");
  return AUGTREE_OK;
}

augtree_status augtree_prefill_kv_bwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                      const void* v_p, const float* lse_p, const float* rowdot_p,
                                      const void* do_p, const float* dk_p_acc, const float* dv_p_acc, void* dk_p,
                                      void* dv_p, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(lse_p); PTR(rowdot_p); PTR(do_p);
  PTR_OR_NULL(dk_p_acc); PTR_OR_NULL(dv_p_acc);
  if ((dk_p_acc == nullptr) != (dv_p_acc == nullptr))
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dk_p_acc and dv_p_acc must both be set or both be NULL");
  PTR(dk_p); PTR(dv_p);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_PREFILL_KV_BWD)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* qpt = ws;
  void* dopt = at(ws, tr_prompt(s, s.Hq));
  float* stats = reinterpret_cast<float*>(at(ws, 2 * tr_prompt(s, s.Hq)));
  CHECK(transpose_range(s, q_p, s.Hq, 0, s.P, 32, qpt, st));
  CHECK(transpose_range(s, do_p, s.Hq, 0, s.P, 32, dopt, st));
  CHECK(pack_stats_prompt(s, lse_p, rowdot_p, stats, st));
  void* split = at(ws, 2 * tr_prompt(s, s.Hq) + st_prompt(s));
  return step_prefill_kv_bwd(s, q_p, qpt, k_p, v_p, stats, do_p, dopt, dk_p_acc, dv_p_acc, dk_p, dv_p, split, st);
}

augtree_status augtree_prefill_dq(const augtree_dims* dims, const void* q_p, const void* k_p, const void* v_p,
                                  const float* lse_p, const float* rowdot_p, const void* do_p, void* dq_p,
                                  void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(lse_p); PTR(rowdot_p); PTR(do_p); PTR(dq_p);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_PREFILL_DQ)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_range(s, k_p, s.Hkv, 0, s.P, 64, ws, st));
  return step_prefill_dq(s, q_p, k_p, ws, v_p, lse_p, rowdot_p, do_p, dq_p, st);
}

// ---- compositions ----

augtree_status augtree_prefill_fwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                   const void* v_p, void* o_p, float* lse_p, void* ws,
                                   size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(o_p); PTR(lse_p);
  CHECK(check_ws(ws, ws_bytes, op_workspace(s, AUGTREE_OP_PREFILL_FWD)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(transpose_range(s, v_p, s.Hkv, 0, s.P, 64, ws, st));
  return step_prefill_fwd(s, q_p, k_p, ws, o_p, lse_p, st);
}

augtree_status augtree_replay_fwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                  const void* q_r, const void* k_r, const void* v_r, void* o_r,
                                  float* lse_r, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_r); PTR(lse_r);
  CHECK(check_ws(ws, ws_bytes, replay_fwd_ws(s).total));
  return replay_fwd_on(s, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, ws, static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_fwd_noalloc(const augtree_dims* dims, const void* k_p, const void* v_p,
                                          const void* q_r, const void* k_r, const void* v_r, void* o_r,
                                          float* lse_r, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_r); PTR(lse_r);
  const size_t need = replay_fwd_ws(s).total;
  if (need > (size_t)AUGTREE_NOALLOC_SCRATCH_BYTES)
    return fail(AUGTREE_ERR_WORKSPACE, "this tree needs %zu bytes of scratch; the static scratch of the "
                "no-allocation entry point holds %zu", need, (size_t)AUGTREE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(noalloc_scratch(&ws));
  return replay_fwd_on(s, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, ws, static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_bwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                  const void* q_r, const void* k_r, const void* v_r,
                                  const void* o_r, const float* lse_r, const void* do_r,
                                  void* dq_r, void* dk_r, void* dv_r, float* dk_p_acc,
                                  float* dv_p_acc, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_r); PTR(lse_r); PTR(do_r);
  PTR(dq_r); PTR(dk_r); PTR(dv_r); PTR(dk_p_acc); PTR(dv_p_acc);
  const ReplayBwdWs w = replay_bwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rowdot = reinterpret_cast<float*>(at(ws, w.rowdot));
  CHECK(step_row_dot(s, s.T, o_r, do_r, rowdot, st));
  CHECK(transpose_branches(s, q_r, s.Hq, 32, at(ws, w.qrt), st));
  CHECK(transpose_branches(s, do_r, s.Hq, 32, at(ws, w.dort), st));
  CHECK(transpose_range(s, k_p, s.Hkv, 0, s.P, 64, at(ws, w.kpt), st));
  CHECK(transpose_branches(s, k_r, s.Hkv, 64, at(ws, w.krt), st));
  float* stats = reinterpret_cast<float*>(at(ws, w.stats));
  CHECK(pack_stats_branches(s, lse_r, rowdot, stats, st));
  // prompt keys x all branches' rows (no mask): the branch sum of the prompt gradient
  CHECK(step_replay_prompt_bwd(s, k_p, v_p, q_r, at(ws, w.qrt), stats, do_r, at(ws, w.dort), 0, s.P, dk_p_acc,
                               dv_p_acc, at(ws, w.walk), at(ws, w.split), w.total - w.split, prompt_split_cap_whole(s),
                               st));
  // branch keys x own-branch rows (causal)
  CHECK(step_replay_local_bwd(s, q_r, at(ws, w.qrt), k_r, v_r, stats, do_r, at(ws, w.dort), dk_r, dv_r, st));
  // dQ of every branch row: prompt keys, then own-branch keys
  return step_replay_dq(s, k_p, at(ws, w.kpt), v_p, q_r, k_r, at(ws, w.krt), v_r, lse_r, rowdot, do_r, dq_r, st);
}

augtree_status augtree_prefill_bwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                   const void* v_p, const void* o_p, const float* lse_p,
                                   const void* do_p, const float* dk_p_acc,
                                   const float* dv_p_acc, void* dq_p, void* dk_p, void* dv_p,
                                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(o_p); PTR(lse_p); PTR(do_p);
  PTR_OR_NULL(dk_p_acc); PTR_OR_NULL(dv_p_acc);
  if ((dk_p_acc == nullptr) != (dv_p_acc == nullptr))
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dk_p_acc and dv_p_acc must both be set or both be NULL");
  PTR(dq_p); PTR(dk_p); PTR(dv_p);
  const PrefillBwdWs w = prefill_bwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rowdot = reinterpret_cast<float*>(at(ws, w.rowdot));
  CHECK(step_row_dot(s, s.P, o_p, do_p, rowdot, st));
  CHECK(transpose_range(s, q_p, s.Hq, 0, s.P, 32, at(ws, w.qpt), st));
  CHECK(transpose_range(s, do_p, s.Hq, 0, s.P, 32, at(ws, w.dopt), st));
  CHECK(transpose_range(s, k_p, s.Hkv, 0, s.P, 64, at(ws, w.kpt), st));
  float* stats = reinterpret_cast<float*>(at(ws, w.stats));
  CHECK(pack_stats_prompt(s, lse_p, rowdot, stats, st));
  CHECK(step_prefill_kv_bwd(s, q_p, at(ws, w.qpt), k_p, v_p, stats, do_p, at(ws, w.dopt), dk_p_acc, dv_p_acc, dk_p,
                            dv_p, at(ws, w.split), st));
  return step_prefill_dq(s, q_p, k_p, at(ws, w.kpt), v_p, lse_p, rowdot, do_p, dq_p, st);
}

}  // extern "C"
