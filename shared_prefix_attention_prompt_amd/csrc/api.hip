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

// Split count of the prompt dK/dV pass over the branches' rows: enough workgroups to give
// every compute unit about two, never more parts than query tiles.
int prompt_split(const Shape& s) {
  const int64_t wgs = (int64_t)((s.P + kDkdvBN - 1) / kDkdvBN) * s.Hkv;
  const int64_t target = 512;
  int64_t n = (target + wgs - 1) / wgs;
  const int64_t qtiles = (s.T + kDkdvBM - 1) / kDkdvBM;
  if (n > qtiles) n = qtiles;
  if (n > 16) n = 16;
  if (n < 1) n = 1;
  return (int)n;
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

struct ReplayBwdWs { size_t rowdot, part_dk, part_dv, total; int nsplit; };
ReplayBwdWs replay_bwd_ws(const Shape& s) {
  ReplayBwdWs w;
  w.nsplit = prompt_split(s);
  const size_t rd = align_up((size_t)s.T * s.Hq * sizeof(float));
  const size_t part = w.nsplit > 1 ? align_up((size_t)w.nsplit * s.P * s.Hkv * s.D * sizeof(float)) : 0;
  w.rowdot = 0;
  w.part_dk = rd;
  w.part_dv = rd + part;
  w.total = rd + 2 * part;
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

}  // namespace
}  // namespace augtree

using namespace augtree;

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
  if (check_dims(dims, &s) != AUGTREE_OK) return 0;
  t_last_error = saved;
  switch (op) {
    case AUGTREE_OP_PREFILL_FWD: return 0;
    case AUGTREE_OP_REPLAY_FWD: return replay_fwd_ws(s).total;
    case AUGTREE_OP_REPLAY_BWD: return replay_bwd_ws(s).total;
    case AUGTREE_OP_PREFILL_BWD: return prefill_bwd_ws(s);
  }
  return 0;
}

augtree_status augtree_prefill_fwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                   const void* v_p, void* o_p, float* lse_p, void* ws,
                                   size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_ptr(q_p, "q_p"));
  CHECK(check_ptr(k_p, "k_p"));
  CHECK(check_ptr(v_p, "v_p"));
  CHECK(check_ptr(o_p, "o_p"));
  CHECK(check_ptr(lse_p, "lse_p"));
  hipStream_t st = static_cast<hipStream_t>(stream);
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

augtree_status augtree_replay_fwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                  const void* q_r, const void* k_r, const void* v_r, void* o_r,
                                  float* lse_r, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_ptr(k_p, "k_p"));
  CHECK(check_ptr(v_p, "v_p"));
  CHECK(check_ptr(q_r, "q_r"));
  CHECK(check_ptr(k_r, "k_r"));
  CHECK(check_ptr(v_r, "v_r"));
  CHECK(check_ptr(o_r, "o_r"));
  CHECK(check_ptr(lse_r, "lse_r"));
  const ReplayFwdWs w = replay_fwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* o_a = reinterpret_cast<float*>(at(ws, w.o_a));
  float* o_b = reinterpret_cast<float*>(at(ws, w.o_b));
  float* lse_a = reinterpret_cast<float*>(at(ws, w.lse_a));
  float* lse_b = reinterpret_cast<float*>(at(ws, w.lse_b));

  // (1) every branch row against the whole, unmasked prompt K/V: partial state a
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_r; a.k = k_p; a.v = v_p; a.o = o_a; a.lse = lse_a;
  a.Hq = s.Hq; a.Hkv = s.Hkv;
  a.nq_rows = s.T; a.nkv_rows = s.P;
  a.ntiles = (s.T + kFwdBM - 1) / kFwdBM;
  a.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdReplayPrompt, a, st), "replay forward (prompt part)");

  // (2) every branch row against its own branch, causally: partial state b
  FwdArgs b;
  memset(&b, 0, sizeof(b));
  b.q = q_r; b.k = k_r; b.v = v_r; b.o = o_b; b.lse = lse_b;
  b.Hq = s.Hq; b.Hkv = s.Hkv;
  b.nq_rows = s.T; b.nkv_rows = s.T;
  b.bt = branch_table(s, kFwdBM);
  b.ntiles = total_tiles(b.bt);
  b.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_attn_fwd(s.dtype, s.D, kFwdReplayLocal, b, st), "replay forward (branch part)");

  // (3) log-sum-exp merge of a and b
  MergeArgs m;
  m.o_a = o_a; m.lse_a = lse_a; m.o_b = o_b; m.lse_b = lse_b;
  m.o = o_r; m.lse = lse_r; m.rows = s.T; m.Hq = s.Hq;
  LAUNCH(launch_merge(s.dtype, s.D, m, st), "replay merge");
  return AUGTREE_OK;
}

augtree_status augtree_replay_bwd(const augtree_dims* dims, const void* k_p, const void* v_p,
                                  const void* q_r, const void* k_r, const void* v_r,
                                  const void* o_r, const float* lse_r, const void* do_r,
                                  void* dq_r, void* dk_r, void* dv_r, float* dk_p_acc,
                                  float* dv_p_acc, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_ptr(k_p, "k_p"));
  CHECK(check_ptr(v_p, "v_p"));
  CHECK(check_ptr(q_r, "q_r"));
  CHECK(check_ptr(k_r, "k_r"));
  CHECK(check_ptr(v_r, "v_r"));
  CHECK(check_ptr(o_r, "o_r"));
  CHECK(check_ptr(lse_r, "lse_r"));
  CHECK(check_ptr(do_r, "do_r"));
  CHECK(check_ptr(dq_r, "dq_r"));
  CHECK(check_ptr(dk_r, "dk_r"));
  CHECK(check_ptr(dv_r, "dv_r"));
  CHECK(check_ptr(dk_p_acc, "dk_p_acc"));
  CHECK(check_ptr(dv_p_acc, "dv_p_acc"));
  const ReplayBwdWs w = replay_bwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rowdot = reinterpret_cast<float*>(at(ws, w.rowdot));

  RowDotArgs r;
  r.o = o_r; r.dout = do_r; r.rowdot = rowdot; r.rows = s.T; r.Hq = s.Hq;
  LAUNCH(launch_rowdot(s.dtype, s.D, r, st), "replay backward row dot");

  // prompt keys x all branches' rows (no mask): the branch sum of the prompt gradient
  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_r; p.dout = do_r; p.lse = lse_r; p.rowdot = rowdot;
  p.k = k_p; p.v = v_p;
  p.nsplit = w.nsplit;
  p.dk = w.nsplit > 1 ? static_cast<void*>(at(ws, w.part_dk)) : static_cast<void*>(dk_p_acc);
  p.dv = w.nsplit > 1 ? static_cast<void*>(at(ws, w.part_dv)) : static_cast<void*>(dv_p_acc);
  p.split_stride = (int64_t)s.P * s.Hkv * s.D;
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.T; p.nkv_rows = s.P;
  p.nktiles = (s.P + kDkdvBN - 1) / kDkdvBN;
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPromptFromReplay, p, st), "replay backward prompt dK/dV");
  if (w.nsplit > 1) {
    SplitReduceArgs sr;
    sr.n = p.split_stride;
    sr.nsplit = w.nsplit;
    sr.part = reinterpret_cast<const float*>(at(ws, w.part_dk));
    sr.out = dk_p_acc;
    LAUNCH(launch_split_reduce(sr, 1, st), "replay backward split reduce (dK)");
    sr.part = reinterpret_cast<const float*>(at(ws, w.part_dv));
    sr.out = dv_p_acc;
    LAUNCH(launch_split_reduce(sr, 1, st), "replay backward split reduce (dV)");
  }

  // response keys x own-branch rows (causal)
  DkdvArgs l;
  memset(&l, 0, sizeof(l));
  l.q = q_r; l.dout = do_r; l.lse = lse_r; l.rowdot = rowdot;
  l.k = k_r; l.v = v_r; l.dk = dk_r; l.dv = dv_r;
  l.Hq = s.Hq; l.Hkv = s.Hkv;
  l.nq_rows = s.T; l.nkv_rows = s.T;
  l.bt = branch_table(s, kDkdvBN);
  l.nktiles = total_tiles(l.bt);
  l.nsplit = 1;
  l.scale = s.scale; l.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvLocal, l, st), "replay backward branch dK/dV");

  // dQ of every branch row: prompt keys, then own-branch keys
  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_r; q.dout = do_r; q.lse = lse_r; q.rowdot = rowdot;
  q.k = k_r; q.v = v_r; q.kp = k_p; q.vp = v_p; q.dq = dq_r;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.T; q.nkv_rows = s.T; q.nprompt = s.P;
  q.bt = branch_table(s, kDqBM);
  q.ntiles = total_tiles(q.bt);
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqResponse, q, st), "replay backward dQ");
  return AUGTREE_OK;
}

augtree_status augtree_prefill_bwd(const augtree_dims* dims, const void* q_p, const void* k_p,
                                   const void* v_p, const void* o_p, const float* lse_p,
                                   const void* do_p, const float* dk_p_acc,
                                   const float* dv_p_acc, void* dq_p, void* dk_p, void* dv_p,
                                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  CHECK(check_dims(dims, &s));
  CHECK(check_ptr(q_p, "q_p"));
  CHECK(check_ptr(k_p, "k_p"));
  CHECK(check_ptr(v_p, "v_p"));
  CHECK(check_ptr(o_p, "o_p"));
  CHECK(check_ptr(lse_p, "lse_p"));
  CHECK(check_ptr(do_p, "do_p"));
  CHECK(check_ptr(dk_p_acc, "dk_p_acc", true));
  CHECK(check_ptr(dv_p_acc, "dv_p_acc", true));
  if ((dk_p_acc == nullptr) != (dv_p_acc == nullptr))
    return fail(AUGTREE_ERR_INVALID_ARGUMENT, "dk_p_acc and dv_p_acc must both be set or both be NULL");
  CHECK(check_ptr(dq_p, "dq_p"));
  CHECK(check_ptr(dk_p, "dk_p"));
  CHECK(check_ptr(dv_p, "dv_p"));
  const size_t need = prefill_bwd_ws(s);
  CHECK(check_ws(ws, ws_bytes, need));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rowdot = static_cast<float*>(ws);

  RowDotArgs r;
  r.o = o_p; r.dout = do_p; r.rowdot = rowdot; r.rows = s.P; r.Hq = s.Hq;
  LAUNCH(launch_rowdot(s.dtype, s.D, r, st), "prefill backward row dot");

  DkdvArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q_p; p.dout = do_p; p.lse = lse_p; p.rowdot = rowdot;
  p.k = k_p; p.v = v_p; p.dk = dk_p; p.dv = dv_p;
  p.init_dk = dk_p_acc; p.init_dv = dv_p_acc;
  p.Hq = s.Hq; p.Hkv = s.Hkv;
  p.nq_rows = s.P; p.nkv_rows = s.P;
  p.nktiles = (s.P + kDkdvBN - 1) / kDkdvBN;
  p.nsplit = 1;
  p.scale = s.scale; p.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dkdv(s.dtype, s.D, kDkdvPrefill, p, st), "prefill backward dK/dV");

  DqArgs q;
  memset(&q, 0, sizeof(q));
  q.q = q_p; q.dout = do_p; q.lse = lse_p; q.rowdot = rowdot;
  q.k = k_p; q.v = v_p; q.dq = dq_p;
  q.Hq = s.Hq; q.Hkv = s.Hkv;
  q.nq_rows = s.P; q.nkv_rows = s.P; q.nprompt = 0;
  q.ntiles = (s.P + kDqBM - 1) / kDqBM;
  q.scale = s.scale; q.scale_log2 = s.scale * kLog2e;
  LAUNCH(launch_dq(s.dtype, s.D, kDqPrefill, q, st), "prefill backward dQ");
  return AUGTREE_OK;
}

}  // extern "C"
