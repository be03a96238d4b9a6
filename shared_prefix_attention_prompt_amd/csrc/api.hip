// Host side of the C ABI declared in include/augtree.h: argument validation, workspace
// layout, branch tables and the launch sequence of each entry point. Nothing here
// allocates, frees or synchronises; all work goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/augtree.h"
#include "kernels.hpp"

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
};

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
  s->P = d->prompt_len;
  s->G = d->num_branches;
  s->Hq = d->num_q_heads;
  s->Hkv = d->num_kv_heads;
  s->D = d->head_dim;
  s->dtype = d->dtype;
  s->scale = d->softmax_scale;
  for (int i = 0; i <= s->G; ++i) s->off[i] = d->branch_offsets[i];
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

// Split count of the prompt dK/dV pass over the branches' rows for `nkeys` prompt keys:
// enough workgroups to give every compute unit about two, never more parts than query
// tiles, at most 16.
int prompt_split(const Shape& s, int nkeys) {
  const int64_t wgs = (int64_t)((nkeys + kDkdvBN - 1) / kDkdvBN) * s.Hkv;
  const int64_t target = 512;
  int64_t n = (target + wgs - 1) / wgs;
  const int64_t qtiles = (s.T + kDkdvBM - 1) / kDkdvBM;
  if (n > qtiles) n = qtiles;
  if (n > 16) n = 16;
  if (n < 1) n = 1;
  return (int)n;
}

// Float count of the split partials for a key range (split * keys * Hkv * D per tensor).
size_t prompt_split_floats(const Shape& s, int nkeys) {
  const int n = prompt_split(s, nkeys);
  return n > 1 ? (size_t)n * nkeys * s.Hkv * s.D : 0;
}

// Workspace of augtree_replay_prompt_bwd: sized for the largest key range a call may use
// (any range needs at most what some range of whole tiles needs; the maximum is taken
// over the tile counts, which is cheap for any realistic prompt).
size_t prompt_bwd_ws(const Shape& s) {
  size_t best = 0;
  const int nkt = (s.P + kDkdvBN - 1) / kDkdvBN;
  for (int t = 1; t <= nkt; ++t) {
    const int nk = t == nkt ? s.P : t * kDkdvBN;
    const size_t f = prompt_split_floats(s, nk);
    if (f > best) best = f;
    if (prompt_split(s, nk) == 1) break;  // larger ranges do not split
  }
  return align_up(2 * best * sizeof(float));
}

struct ReplayFwdWs { size_t o_a, o_b, lse_a, lse_b, total; };
ReplayFwdWs replay_fwd_ws(const Shape& s) {
  ReplayFwdWs w;
  const size_t o = align_up((size_t)s.T * s.Hq * s.D * sizeof(float));
  const size_t l = align_up((size_t)s.T * s.Hq * sizeof(float));
  w.o_a = 0;
  w.o_b = o;
  w.lse_a = 2 * o;
  w.lse_b = 2 * o + l;
  w.total = 2 * o + 2 * l;
  return w;
}

struct ReplayBwdWs { size_t rowdot, prompt, total; };
ReplayBwdWs replay_bwd_ws(const Shape& s) {
  ReplayBwdWs w;
  const size_t rd = align_up((size_t)s.T * s.Hq * sizeof(float));
  w.rowdot = 0;
  w.prompt = rd;
  w.total = rd + prompt_bwd_ws(s);
  return w;
}

size_t prefill_bwd_ws(const Shape& s) { return align_up((size_t)s.P * s.Hq * sizeof(float)); }

augtree_status check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return AUGTREE_OK;
  if (ws == nullptr) return fail(AUGTREE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (have < need) return fail(AUGTREE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(AUGTREE_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
  return AUGTREE_OK;
}

// Table of the branches for kernels that tile each branch separately.
BranchTable branch_table(const Shape& s, int tile) {
  BranchTable bt;
  memset(&bt, 0, sizeof(bt));
  bt.G = s.G;
  int acc = 0;
  for (int i = 0; i <= s.G; ++i) {
    bt.off[i] = s.off[i];
    bt.tile_prefix[i] = acc;
    if (i < s.G) acc += (s.off[i + 1] - s.off[i] + tile - 1) / tile;
  }
  return bt;
}

int total_tiles(const BranchTable& bt) { return bt.tile_prefix[bt.G]; }

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---------------------------------------------------------------------------------------
// Single steps on validated shapes (no argument checks here).
// ---------------------------------------------------------------------------------------
augtree_status step_prefill_fwd(const Shape& s, const void* q_p, const void* k_p, const void* v_p,
                                void* o_p, float* lse_p, hipStream_t st) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_p; a.k = k_p; a.v = v_p; a.o = o_p; a.lse = lse_p;
  a.Hq = s.Hq; a.Hkv = s.Hkv;
  a.nq_rows = s.P; a.nkv_rows = s.P;
  a.ntiles = (s.P + kFwdBM - 1) / kFwdBM;
  a.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdPrefill, a, st), "prefill forward");
  return AUGTREE_OK;
}

augtree_status step_replay_prompt_fwd(const Shape& s, const void* k_p, const void* v_p, const void* q_r,
                                      int kb, int ke, float* o_part, float* lse_part, hipStream_t st) {
  const size_t esz = s.dtype == AUGTREE_BF16 ? 2 : 4;
  const size_t koff = (size_t)kb * s.Hkv * s.D * esz;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_r;
  a.k = static_cast<const char*>(k_p) + koff;
  a.v = static_cast<const char*>(v_p) + koff;
  a.o = o_part; a.lse = lse_part;
  a.Hq = s.Hq; a.Hkv = s.Hkv;
  a.nq_rows = s.T; a.nkv_rows = ke - kb;
  a.ntiles = (s.T + kFwdBM - 1) / kFwdBM;
  a.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdReplayPrompt, a, st), "replay forward (prompt keys)");
  return AUGTREE_OK;
}

augtree_status step_replay_local_fwd(const Shape& s, const void* q_r, const void* k_r, const void* v_r,
                                     float* o_part, float* lse_part, hipStream_t st) {
  FwdArgs b;
  memset(&b, 0, sizeof(b));
  b.q = q_r; b.k = k_r; b.v = v_r; b.o = o_part; b.lse = lse_part;
  b.Hq = s.Hq; b.Hkv = s.Hkv;
  b.nq_rows = s.T; b.nkv_rows = s.T;
  b.bt = branch_table(s, kFwdBM);
  b.ntiles = total_tiles(b.bt);
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

augtree_status step_replay_prompt_bwd(const Shape& s, const void* k_p, const void* v_p, const void* q_r,
                                      const float* lse_r, const float* rowdot_r, const void* do_r, int kb,
                                      int ke, float* dk_acc, float* dv_acc, void* ws, hipStream_t st) {
  const int nkeys = ke - kb;
  const int nsplit = prompt_split(s, nkeys);
  const size_t esz = s.dtype == AUGTREE_BF16 ? 2 : 4;
  const size_t koff = (size_t)kb * s.Hkv * s.D;
  const int64_t part = (int64_t)nkeys * s.Hkv * s.D;
  float* part_dk = static_cast<float*>(ws);
  float* part_dv = part_dk + (nsplit > 1 ? (int64_t)nsplit * part : 0);
  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_r; p.dout = do_r; p.lse = lse_r; p.rowdot = rowdot_r;
  p.k = static_cast<const char*>(k_p) + koff * esz;
  p.v = static_cast<const char*>(v_p) + koff * esz;
  p.nsplit = nsplit;
  p.dk = nsplit > 1 ? static_cast<void*>(part_dk) : static_cast<void*>(dk_acc + koff);
  p.dv = nsplit > 1 ? static_cast<void*>(part_dv) : static_cast<void*>(dv_acc + koff);
  p.split_stride = part;
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.T; p.nkv_rows = nkeys;
  p.nktiles = (nkeys + kDkdvBN - 1) / kDkdvBN;
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPromptFromReplay, p, st), "prompt dK/dV from branches");
  if (nsplit > 1) {
    SplitReduceArgs sr;
    sr.n = part;
    sr.nsplit = nsplit;
    sr.part = part_dk;
    sr.out = dk_acc + koff;
    LAUNCH(launch_split_reduce(sr, 1, st), "split reduce (dK)");
    sr.part = part_dv;
    sr.out = dv_acc + koff;
    LAUNCH(launch_split_reduce(sr, 1, st), "split reduce (dV)");
  }
  return AUGTREE_OK;
}

augtree_status step_replay_local_bwd(const Shape& s, const void* q_r, const void* k_r, const void* v_r,
                                     const float* lse_r, const float* rowdot_r, const void* do_r, void* dk_r,
                                     void* dv_r, hipStream_t st) {
  DkdvArgs l;
  memset(&l, 0, sizeof(l));
  l.q = q_r; l.dout = do_r; l.lse = lse_r; l.rowdot = rowdot_r;
  l.k = k_r; l.v = v_r; l.dk = dk_r; l.dv = dv_r;
  l.Hq = s.Hq; l.Hkv = s.Hkv;
  l.nq_rows = s.T; l.nkv_rows = s.T;
  l.bt = branch_table(s, kDkdvBN);
  l.nktiles = total_tiles(l.bt);
  l.nsplit = 1;
  l.scale = s.scale; l.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvLocal, l, st), "branch dK/dV");
  return AUGTREE_OK;
}

augtree_status step_replay_dq(const Shape& s, const void* k_p, const void* v_p, const void* q_r,
                              const void* k_r, const void* v_r, const float* lse_r, const float* rowdot_r,
                              const void* do_r, void* dq_r, hipStream_t st) {
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_r; q.dout = do_r; q.lse = lse_r; q.rowdot = rowdot_r;
  q.k = k_r; q.v = v_r; q.kp = k_p; q.vp = v_p; q.dq = dq_r;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.T; q.nkv_rows = s.T; q.nprompt = s.P;
  q.bt = branch_table(s, kDqBM);
  q.ntiles = total_tiles(q.bt);
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqResponse, q, st), "branch dQ");
  return AUGTREE_OK;
}

augtree_status step_prefill_kv_bwd(const Shape& s, const void* q_p, const void* k_p, const void* v_p,
                                   const float* lse_p, const float* rowdot_p, const void* do_p,
                                   const float* dk_acc, const float* dv_acc, void* dk_p, void* dv_p,
                                   hipStream_t st) {
  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_p; p.dout = do_p; p.lse = lse_p; p.rowdot = rowdot_p;
  p.k = k_p; p.v = v_p; p.dk = dk_p; p.dv = dv_p;
  p.init_dk = dk_acc; p.init_dv = dv_acc;
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.P; p.nkv_rows = s.P;
  p.nktiles = (s.P + kDkdvBN - 1) / kDkdvBN;
  p.nsplit = 1;
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPrefill, p, st), "prefill dK/dV");
  return AUGTREE_OK;
}

augtree_status step_prefill_dq(const Shape& s, const void* q_p, const void* k_p, const void* v_p,
                               const float* lse_p, const float* rowdot_p, const void* do_p, void* dq_p,
                               hipStream_t st) {
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_p; q.dout = do_p; q.lse = lse_p; q.rowdot = rowdot_p;
  q.k = k_p; q.v = v_p; q.dq = dq_p;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.P; q.nkv_rows = s.P; q.nprompt = 0;
  q.ntiles = (s.P + kDqBM - 1) / kDqBM;
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqPrefill, q, st), "prefill dQ");
  return AUGTREE_OK;
}

augtree_status check_key_range(const Shape& s, int kb, int ke) {
  if (kb < 0 || ke > s.P || kb >= ke)
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "prompt key range [%d, %d) not inside [0, %d) or empty", kb, ke, s.P);
  return AUGTREE_OK;
}

}  // namespace
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

size_t augtree_workspace_bytes(const augtree_dims* dims, int op) {
  Shape s;
  const std::string saved = t_last_error;
  if (check_dims(dims, &s) != AUGTREE_OK) {
    t_last_error = saved;
    return 0;
  }
  switch (op) {
    case AUGTREE_OP_PREFILL_FWD: return 0;
    case AUGTREE_OP_REPLAY_FWD: return replay_fwd_ws(s).total;
    case AUGTREE_OP_REPLAY_BWD: return replay_bwd_ws(s).total;
    case AUGTREE_OP_PREFILL_BWD: return prefill_bwd_ws(s);
    case AUGTREE_OP_REPLAY_PROMPT_BWD: return prompt_bwd_ws(s);
  }
  return 0;
}

// ---- single steps ----

augtree_status augtree_replay_prompt_fwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                         const void* q_r, int32_t key_begin, int32_t key_end, float* o_part,
                                         float* lse_part, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_key_range(s, key_begin, key_end));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(o_part); PTR(lse_part);
  return step_replay_prompt_fwd(s, k_p, v_p, q_r, key_begin, key_end, o_part, lse_part,
                                static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_local_fwd(const augtree_dims* dims, const void* q_r, const void* k_r,
                                        const void* v_r, float* o_part, float* lse_part, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_part); PTR(lse_part);
  return step_replay_local_fwd(s, q_r, k_r, v_r, o_part, lse_part, static_cast<hipStream_t>(stream));
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
  CHECK(check_ws(ws, ws_bytes, prompt_bwd_ws(s)));
  return step_replay_prompt_bwd(s, k_p, v_p, q_r, lse_r, rowdot_r, do_r, key_begin, key_end, dk_p_acc,
                                dv_p_acc, ws, static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_local_bwd(const augtree_dims* dims, const void* q_r, const void* k_r,
                                        const void* v_r, const float* lse_r, const float* rowdot_r,
                                        const void* do_r, void* dk_r, void* dv_r, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_r); PTR(k_r); PTR(v_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dk_r); PTR(dv_r);
  return step_replay_local_bwd(s, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dk_r, dv_r,
                               static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_dq(const augtree_dims* dims, const void* k_p, const void* v_p, const void* q_r,
                                 const void* k_r, const void* v_r, const float* lse_r, const float* rowdot_r,
                                 const void* do_r, void* dq_r, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(lse_r); PTR(rowdot_r); PTR(do_r); PTR(dq_r);
  return step_replay_dq(s, k_p, v_p, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dq_r,
                        static_cast<hipStream_t>(stream));
}

augtree_status augtree_prefill_kv_bwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                      const void* v_p, const float* lse_p, const float* rowdot_p,
                                      const void* do_p, const float* dk_p_acc, const float* dv_p_acc, void* dk_p,
                                      void* dv_p, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(lse_p); PTR(rowdot_p); PTR(do_p);
  PTR_OR_NULL(dk_p_acc); PTR_OR_NULL(dv_p_acc);
  if ((dk_p_acc == nullptr) != (dv_p_acc == nullptr))
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dk_p_acc and dv_p_acc must both be set or both be NULL");
  PTR(dk_p); PTR(dv_p);
  return step_prefill_kv_bwd(s, q_p, k_p, v_p, lse_p, rowdot_p, do_p, dk_p_acc, dv_p_acc, dk_p, dv_p,
                             static_cast<hipStream_t>(stream));
}

augtree_status augtree_prefill_dq(const augtree_dims* dims, const void* q_p, const void* k_p, const void* v_p,
                                  const float* lse_p, const float* rowdot_p, const void* do_p, void* dq_p,
                                  void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(lse_p); PTR(rowdot_p); PTR(do_p); PTR(dq_p);
  return step_prefill_dq(s, q_p, k_p, v_p, lse_p, rowdot_p, do_p, dq_p, static_cast<hipStream_t>(stream));
}

// ---- compositions ----

augtree_status augtree_prefill_fwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                   const void* v_p, void* o_p, float* lse_p, void* ws,
                                   size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(q_p); PTR(k_p); PTR(v_p); PTR(o_p); PTR(lse_p);
  return step_prefill_fwd(s, q_p, k_p, v_p, o_p, lse_p, static_cast<hipStream_t>(stream));
}

augtree_status augtree_replay_fwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                  const void* q_r, const void* k_r, const void* v_r, void* o_r,
                                  float* lse_r, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  PTR(k_p); PTR(v_p); PTR(q_r); PTR(k_r); PTR(v_r); PTR(o_r); PTR(lse_r);
  const ReplayFwdWs w = replay_fwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float* o_parts[2] = {reinterpret_cast<float*>(at(ws, w.o_a)), reinterpret_cast<float*>(at(ws, w.o_b))};
  const float* l_parts[2] = {reinterpret_cast<float*>(at(ws, w.lse_a)), reinterpret_cast<float*>(at(ws, w.lse_b))};
  // (1) every branch row against the whole, unmasked prompt K/V: partial state a
  CHECK(step_replay_prompt_fwd(s, k_p, v_p, q_r, 0, s.P, const_cast<float*>(o_parts[0]),
                               const_cast<float*>(l_parts[0]), st));
  // (2) every branch row against its own branch, causally: partial state b
  CHECK(step_replay_local_fwd(s, q_r, k_r, v_r, const_cast<float*>(o_parts[1]), const_cast<float*>(l_parts[1]),
                              st));
  // (3) log-sum-exp merge of a and b
  return step_merge(s, 2, o_parts, l_parts, o_r, lse_r, st);
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
  // prompt keys x all branches' rows (no mask): the branch sum of the prompt gradient
  CHECK(step_replay_prompt_bwd(s, k_p, v_p, q_r, lse_r, rowdot, do_r, 0, s.P, dk_p_acc, dv_p_acc,
                               at(ws, w.prompt), st));
  // branch keys x own-branch rows (causal)
  CHECK(step_replay_local_bwd(s, q_r, k_r, v_r, lse_r, rowdot, do_r, dk_r, dv_r, st));
  // dQ of every branch row: prompt keys, then own-branch keys
  return step_replay_dq(s, k_p, v_p, q_r, k_r, v_r, lse_r, rowdot, do_r, dq_r, st);
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
  CHECK(check_ws(ws, ws_bytes, prefill_bwd_ws(s)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rowdot = static_cast<float*>(ws);
  CHECK(step_row_dot(s, s.P, o_p, do_p, rowdot, st));
  CHECK(step_prefill_kv_bwd(s, q_p, k_p, v_p, lse_p, rowdot, do_p, dk_p_acc, dv_p_acc, dk_p, dv_p, st));
  return step_prefill_dq(s, q_p, k_p, v_p, lse_p, rowdot, do_p, dq_p, st);
}

}  // extern "C"
