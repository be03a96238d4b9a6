// Backward kernels for the loss sum(O * dO) of shared-prefix attention.
//
// With P = softmax(scale * Q K^T + M) recomputed from the saved row LSE, the gradients are
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowdot),  dQ = scale dS K,  dK = scale dS^T Q,
// where rowdot[r] = sum_d dO[r, d] O[r, d] (equal to sum_j P[r, j] dP[r, j]).
//
// dK/dV are computed key-stationary: a workgroup of 8 waves owns 256 keys of one key/value
// head (32 per wave; K and the dK/dV accumulators in registers, V in LDS) and walks every query
// tile that can see them, for every query head mapped to that kv head, in a fixed order. For
// the prompt keys this walk runs over all branches' rows at once, so the prompt gradient of
// every branch is summed inside one accumulator ("Splitting Prompt Prefill from Response
// Replay ...", §3.2: the prompt K/V gradient is the sum over branches) without atomics. When
// the keys alone cannot fill the GPU, the query tiles are split into a fixed number of parts
// (the prompt walk over the branches) or row-tile chunks (the causal prefill walk; long
// prompts are chunked too, so that concurrent workgroups walk the same rows) whose fp32
// partial sums are added afterwards in a fixed order, so results stay bitwise reproducible.
// Causal walks run from the last query tile down to the key block's own, so the workgroups of
// one kv head, whose walks start at different rows, read the same rows at the same time.
//
// dQ is computed query-stationary in its own pass (it recomputes S and dP), which keeps it
// free of atomics as well. For one stationary prompt-K/V shard (a prompt key range) the pass
// writes float32 partial sums over the range; the partials of the shards and of the rows' own
// branch keys are then added in a fixed order (aux.hip, sum_parts_kernel).
//
// Query tiles (dK/dV) and key tiles (dQ) are copied global -> LDS by direct loads through a
// ring of LDS stages, both in natural layout and from the transposed copies (the operands of
// the products that contract over the sequence; stored tile by tile, so each transposed LDS
// tile is one contiguous block in memory).
#include "kernels.hpp"

namespace augtree {


template <typename T, typename OT, int D, int MODE>
__global__ __launch_bounds__(512, 2) void dkdv_kernel(DkdvArgs a) {
  using M = Mma<T>;
  constexpr int NW = 8;
  constexpr int NSTAGE = 2;  // with the workgroup's V rows resident, two stages fit in LDS
  constexpr int ESZ = sizeof(T);
  constexpr int BM = kDkdvBM;
  constexpr int RBN = D * ESZ;   // natural tile row bytes
  constexpr int RBT = BM * ESZ;  // transposed tile row bytes
  using TN = TileSrc<BM, RBN>;      // Q or dO tile, natural
  using TT = TileSrc<D, RBT>;       // Q^T or dO^T tile, transposed
  using TS = TileSrc<2, BM * 4>;    // row statistics: lse * log2(e), rowdot
  using TVR = TileSrc<32 * NW, RBN>;  // the workgroup's V rows
  constexpr int O_DO = TN::NB * 1024, O_QT = 2 * TN::NB * 1024, O_DOT = O_QT + TT::NB * 1024;
  constexpr int O_ST = O_DOT + TT::NB * 1024;
  constexpr int SB = O_ST + TS::NB * 1024;  // bytes per stage
  constexpr int RD = pitch<BM * 4>() / 4;   // float offset of the rowdot row
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K;
  constexpr int KPW = 32 * NW;

  __shared__ __attribute__((aligned(1024))) char lv[TVR::NB * 1024];  // this workgroup's V rows
  // one LDS object per stage: Q, dO (natural), Q^T, dO^T (transposed), row statistics
  __shared__ __attribute__((aligned(1024))) char ls0[SB];
  __shared__ __attribute__((aligned(1024))) char ls1[SB];
  auto stage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return ls0; else return ls1;
  };

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lid = xcd_remap(blockIdx.x, a.nwg);
  // workgroups per kv head: key tiles x splits (prompt walk), units (prefill chunks)
  const int per_kvh = MODE == kDkdvPrefill ? a.nktiles : a.nktiles * a.nsplit;
  const int kvh = lid / per_kvh;
  int z = MODE == kDkdvPrefill ? 0 : (lid % per_kvh) / a.nktiles;
  const int kti = lid % a.nktiles;
  const int group = a.Hq / a.Hkv;

  // keys [k0, k1); query tiles [t_lo, t_hi) (meaning depends on the mode)
  int k0, k1, t_lo, t_hi, b = 0;
  // Causality is read from the arguments (set for the branch and prefill walks) rather than
  // fixed per mode: with a compile-time "never" the scheduler packs the unmasked loop too
  // tightly for the register budget.
  const bool causal = a.causal != 0;
  if constexpr (MODE == kDkdvPromptFromReplay) {
    k0 = kti * KPW;
    k1 = min(k0 + KPW, a.nkv_rows);
    const int nqt = a.nqtiles;
    const int per = (nqt + a.nsplit - 1) / a.nsplit;
    t_lo = min(nqt, z * per);
    t_hi = min(nqt, (z + 1) * per);
  } else if constexpr (MODE == kDkdvLocal) {
    b = branch_of_tile(a.bt, kti);
    const int bs = a.bt.off[b], be = a.bt.off[b + 1];
    k0 = bs + (kti - a.bt.tile_prefix[b]) * KPW;
    k1 = min(k0 + KPW, be);
    t_lo = (k0 - bs) / BM;
    t_hi = (be - bs + BM - 1) / BM;
  } else if (a.nsplit == 1) {
    k0 = kti * KPW;
    k1 = min(k0 + KPW, a.nkv_rows);
    t_lo = k0 / BM;
    t_hi = (a.nq_rows + BM - 1) / BM;
  } else {
    // unit u of this kv head: row-tile chunk z, the last chunk first, and inside it the key
    // blocks that see the chunk (first row before its end), in order; the workgroups that run
    // at the same time then walk the same rows of one chunk together and share them in L2
    const int nt = (a.nq_rows + BM - 1) / BM;
    const int nk = (a.nkv_rows + KPW - 1) / KPW;
    int u = lid % a.nktiles, zz = a.nsplit - 1;
    for (;;) {
      const int cnt = min(nk, ((zz + 1) * a.zc + KPW / BM - 1) / (KPW / BM));
      if (u < cnt || zz == 0) break;
      u -= cnt;
      --zz;
    }
    const int kb = u;
    z = zz;
    k0 = kb * KPW;
    k1 = min(k0 + KPW, a.nkv_rows);
    t_lo = max(k0 / BM, zz * a.zc);
    t_hi = min(nt, (zz + 1) * a.zc);
  }

  const uint32_t qld = (uint32_t)(a.Hq * D * ESZ);   // bytes between query rows
  constexpr uint32_t tld = RBT;  // transposed tiles are contiguous [D][BM] blocks
  const int key = k0 + w * 32 + c;
  const bool kvalid = key < k1;
  const int wk_lo = k0 + w * 32;

  // V rows of the workgroup's keys go to LDS once (landed before the pipeline's first
  // barrier); K stays in registers.
  dma_stage<NW>(lv, w, lane,
                TVR{reinterpret_cast<const char*>(a.v) + ((int64_t)k0 * a.Hkv + kvh) * D * ESZ,
                    (uint32_t)(a.Hkv * D * ESZ), k1 - k0});
  typename M::frag kf[KS];
  {
    const T* kp = reinterpret_cast<const T*>(a.k) + ((int64_t)key * a.Hkv + kvh) * D + g * M::E;
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = kvalid ? gload_frag<T>(kp + s * M::K) : zero_frag<T>();
  }
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) { dkt[db] = zero16(); dvt[db] = zero16(); }
  const float sl2 = a.scale_log2;

  const int ntile = t_hi > t_lo ? t_hi - t_lo : 0;
  const int niter = ntile * group;

  // Query tiles are walked head by head (the group's query heads in turn), tiles t_lo ..
  // t_hi - 1 of each. The walk is a cursor advanced by one tile per issued stage (issue is
  // called with consecutive iterations), so no iteration needs a division; over the branches'
  // rows each tile's place comes from the per-launch walk table (one scalar load). The first
  // row of each stage's tile is kept for the causal tests of compute.
  struct Tile { int hq, row0, col0, nval; int64_t rowoff; };
  Tile cur{kvh * group, 0, 0, 0, 0};
  int cur_it = -1, cur_t = t_lo - 1;
  auto advance = [&]() {
    ++cur_it;
    bool restart = cur_it == 0;
    if (!restart && ++cur_t == t_hi) {
      ++cur.hq;
      restart = true;
    }
    if (restart) cur_t = t_lo;
    if constexpr (MODE == kDkdvPromptFromReplay) {
      // one scalar load of the tile's entry in the walk table (the branch walk is done once
      // per launch by walk_table_kernel, not by every wave at every stage)
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(4))) const i32x4 const_i32x4;
      const i32x4 e = ((const_i32x4*)a.walk)[cur_t];
      cur.rowoff = (int64_t)(((uint64_t)(uint32_t)e[1] << 32) | (uint32_t)e[0]);
      cur.col0 = e[2];
      cur.nval = e[3];
    } else {
      // causal walks run from the last row tile down to the key block's own, so the
      // workgroups of one kv head (their key blocks start at different rows) walk the same
      // rows at the same time and share them in L2
      const int tt = t_lo + t_hi - 1 - cur_t;
      if constexpr (MODE == kDkdvLocal) {
        cur.row0 = a.bt.off[b] + tt * BM;
        cur.col0 = a.bt.pad[b] + tt * BM;
        cur.nval = min(BM, a.bt.off[b + 1] - cur.row0);
      } else {
        cur.row0 = tt * BM;
        cur.col0 = tt * BM;
        cur.nval = min(BM, a.nq_rows - cur.row0);
      }
    }
  };
  int stage_row0[NSTAGE];

  CopyPlan<NW, true, TN, TN, TT, TT, TS> plan;  // lane offsets held in registers
  {
    const uint32_t ld[5] = {qld, qld, tld, tld, (uint32_t)((int64_t)a.Hq * a.qt_cols * 4)};
    plan.init(w, lane, ld);
  }
  auto issue = [&](int it, auto S) {
    if (cur_it < it) advance();
    const Tile& tl = cur;
    stage_row0[decltype(S)::value] = tl.row0;
    int64_t nat;
    if constexpr (MODE == kDkdvPromptFromReplay) nat = tl.rowoff + (int64_t)tl.hq * (D * ESZ);
    else nat = ((int64_t)tl.row0 * a.Hq + tl.hq) * D * ESZ;
    const int64_t tr = ((int64_t)tl.hq * a.qt_cols + tl.col0) * D * ESZ;  // tile-major copies
    plan.issue(stage(S), lane, TN{reinterpret_cast<const char*>(a.q) + nat, qld, tl.nval},
                  TN{reinterpret_cast<const char*>(a.dout) + nat, qld, tl.nval},
                  TT{reinterpret_cast<const char*>(a.qt) + tr, tld, D},
                  TT{reinterpret_cast<const char*>(a.dot) + tr, tld, D},
                  TS{reinterpret_cast<const char*>(a.stats + (int64_t)tl.hq * a.qt_cols + tl.col0),
                     (uint32_t)((int64_t)a.Hq * a.qt_cols * 4), 2});
  };

  auto compute = [&](int it, auto S) {
    const char* q_ = stage(S);
    const char* o_ = q_ + O_DO;
    const char* qt_ = q_ + O_QT;
    const char* ot_ = q_ + O_DOT;
    const float* st = reinterpret_cast<const float*>(q_ + O_ST);
    const int row0 = stage_row0[decltype(S)::value];
    if (causal && row0 + 31 < wk_lo) return;  // every query of the tile precedes every key
    f32x16 sacc = zero16(), pacc = zero16();
    if constexpr (M::E == 8) {
      // Q, dO and V fragments read one step (two matrix ops) ahead
      auto fq = [&](int s) { return tile_frag<T, RBN>(q_, c, s * M::K + g * M::E); };
      auto fo = [&](int s) { return tile_frag<T, RBN>(o_, c, s * M::K + g * M::E); };
      auto fv = [&](int s) { return tile_frag<T, RBN>(lv, w * 32 + c, s * M::K + g * M::E); };
      typename M::frag q0 = fq(0), o0 = fo(0), v0 = fv(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        typename M::frag q1 = q0, o1 = o0, v1 = v0;
        if (s + 1 < KS) { q1 = fq(s + 1); o1 = fo(s + 1); v1 = fv(s + 1); }
        sacc = M::run(q0, kf[s], sacc);
        pacc = M::run(o0, v0, pacc);
        __builtin_amdgcn_sched_barrier(0);
        q0 = q1; o0 = o1; v0 = v1;
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = M::run(tile_frag<T, RBN>(q_, c, s * M::K + g * M::E), kf[s], sacc);
        pacc = M::run(tile_frag<T, RBN>(o_, c, s * M::K + g * M::E),
                      tile_frag<T, RBN>(lv, w * 32 + c, s * M::K + g * M::E), pacc);
      }
    }
    auto softmax_grad = [&](auto masked) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = r4 * 8 + g * 4;
        const f32x4 L = *reinterpret_cast<const f32x4*>(st + qi);
        const f32x4 R = *reinterpret_cast<const f32x4*>(st + RD + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r4 * 4 + j;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -L[j]));
          if constexpr (decltype(masked)::value) {
            if (key > row0 + qi + j) p = 0.f;
          }
          pacc[r] = p * (pacc[r] - R[j]);
          sacc[r] = p;
        }
      }
    };
    if (causal && row0 < wk_lo + 31) softmax_grad(std::true_type{});  // the diagonal tile
    else softmax_grad(std::false_type{});
    if constexpr (M::E == 8) {
      // dO^T and Q^T fragments read two matrix ops ahead through a ring of three
      constexpr int NP = NS * DB * 2;
      const typename M::frag pf0 = acc_frag<T>(sacc, 0), pf1 = acc_frag<T>(sacc, 1);
      const typename M::frag df0 = acc_frag<T>(pacc, 0), df1 = acc_frag<T>(pacc, 1);
      auto ft = [&](int i) {
        return tile_frag<T, RBT>((i & 1) ? qt_ : ot_, ((i >> 1) % DB) * 32 + c, tread<T>((i >> 1) / DB, g));
      };
      typename M::frag fr[3];
      fr[0] = ft(0);
      fr[1] = ft(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + 2 < NP) fr[(i + 2) % 3] = ft(i + 2);
        const int db = (i >> 1) % DB, s = (i >> 1) / DB;
        if (i & 1) dkt[db] = M::run(fr[i % 3], s == 0 ? df0 : df1, dkt[db]);
        else dvt[db] = M::run(fr[i % 3], s == 0 ? pf0 : pf1, dvt[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const typename M::frag pf = acc_frag<T>(sacc, s);
        const typename M::frag df = acc_frag<T>(pacc, s);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvt[db] = M::run(tile_frag<T, RBT>(ot_, db * 32 + c, tread<T>(s, g)), pf, dvt[db]);
          dkt[db] = M::run(tile_frag<T, RBT>(qt_, db * 32 + c, tread<T>(s, g)), df, dkt[db]);
        }
      }
    }
  };

  if (niter > 0)
    run_pipeline<NSTAGE, stage_copies<NW, TN, TN, TT, TT, TS>()>(niter, issue, compute);
  else
    wait_vm();  // the V copy must land before the workgroup's LDS is released

  if (!kvalid) return;
  int64_t obase = ((int64_t)key * a.Hkv + kvh) * D;
  if constexpr (MODE != kDkdvLocal) obase += (int64_t)z * a.split_stride;  // split partials
  OT* dk = reinterpret_cast<OT*>(a.dk) + obase;
  OT* dv = reinterpret_cast<OT*>(a.dv) + obase;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + r4 * 8 + g * 4;
      float k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k4[j] = dkt[db][r4 * 4 + j] * a.scale;
        v4[j] = dvt[db][r4 * 4 + j];
      }
      if constexpr (MODE == kDkdvPrefill) {
        if (a.init_dk != nullptr) {
          const f32x4 ik = *reinterpret_cast<const f32x4*>(a.init_dk + obase + d0);
          const f32x4 iv = *reinterpret_cast<const f32x4*>(a.init_dv + obase + d0);
#pragma unroll
          for (int j = 0; j < 4; ++j) { k4[j] += ik[j]; v4[j] += iv[j]; }
        }
      }
      store4<OT>(dk + d0, k4[0], k4[1], k4[2], k4[3]);
      store4<OT>(dv + d0, v4[0], v4[1], v4[2], v4[3]);
    }
}

template <typename T, typename OT, int D, int MODE, int HG>
__global__ __launch_bounds__(512, 2) void dq_kernel(DqArgs a) {
  using M = Mma<T>;
  constexpr int NW = 8;
  constexpr int ESZ = sizeof(T);
  constexpr int BN = kDqBN;
  constexpr int RBN = D * ESZ, RBT = BN * ESZ;
  using TN = TileSrc<BN, RBN>;  // K or V tile, natural
  using TT = TileSrc<D, RBT>;   // K^T tile, transposed
  constexpr int O_V = TN::NB * 1024, O_KT = 2 * TN::NB * 1024;
  constexpr int SB = O_KT + TT::NB * 1024;  // bytes per stage
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K, KB = BN / 32;
  constexpr int RT = 32 * (NW / HG);

  constexpr int NSTAGE = 3;
  // one LDS object per stage: K tile, V tile, K^T tile
  __shared__ __attribute__((aligned(1024))) char ls0[SB];
  __shared__ __attribute__((aligned(1024))) char ls1[SB];
  __shared__ __attribute__((aligned(1024))) char ls2[SB];
  auto stage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return ls0; else if constexpr (st == 1) return ls1; else return ls2;
  };

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lid = xcd_remap(blockIdx.x, a.nwg);
  const int hs = lid / a.ntiles;
  int tile = lid % a.ntiles;
  const int h = hs * HG + (w % HG);
  const int kvh = (hs * HG) / (a.Hq / a.Hkv);
  const int rb = w / HG;

  int q0, q1, n0 = 0, kb0, kb1, pcol0 = 0;
  if constexpr (MODE == kDqResponse) {
    const int b = branch_of_tile(a.bt, tile);
    const int bs = a.bt.off[b], be = a.bt.off[b + 1];
    q0 = bs + (tile - a.bt.tile_prefix[b]) * RT;
    q1 = min(q0 + RT, be);
    n0 = (a.nprompt + BN - 1) / BN;
    kb0 = bs;
    kb1 = a.own ? q1 : bs;  // own branch keys, or none (a prompt key range alone)
    pcol0 = a.bt.pad[b];
  } else {
    tile = a.ntiles - 1 - tile;  // longest causal row range first
    q0 = tile * RT;
    q1 = min(q0 + RT, a.nq_rows);
    kb0 = 0;
    kb1 = q1;
  }
  const int nkt = n0 + (kb1 - kb0 + BN - 1) / BN;

  const int64_t qld = (int64_t)a.Hq * D;
  const uint32_t kld = (uint32_t)(a.Hkv * D * ESZ);
  const int wq0 = q0 + rb * 32;
  const int qrow = wq0 + c;
  const bool qvalid = qrow < q1;
  const int wq_hi = min(q1, wq0 + 32) - 1;
  const bool wave_has_rows = wq0 < q1;

  typename M::frag qf[KS], of[KS];
  {
    const int64_t off = (int64_t)qrow * qld + (int64_t)h * D + g * M::E;
    const T* qp = reinterpret_cast<const T*>(a.q) + off;
    const T* op = reinterpret_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = qvalid ? gload_frag<T>(qp + s * M::K) : zero_frag<T>();
      of[s] = qvalid ? gload_frag<T>(op + s * M::K) : zero_frag<T>();
    }
  }
  const float lse2 = qvalid ? a.lse[(int64_t)h * a.nq_rows + qrow] * kLog2e : kInf;
  const float rdv = qvalid ? a.rowdot[(int64_t)h * a.nq_rows + qrow] : 0.f;
  const float sl2 = a.scale_log2;

  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = zero16();

  // key tile it: prompt tiles first (response mode, no mask), then own causal tiles
  auto tile_src = [&](int it, const char*& kp, const char*& vp, const char*& ktp, uint32_t& ktld, int& kstart,
                      int& nval, bool& cz) {
    if (it < n0) {
      kstart = it * BN;
      nval = a.nprompt - kstart;
      kp = reinterpret_cast<const char*>(a.kp) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      vp = reinterpret_cast<const char*>(a.vp) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      ktld = RBT;
      ktp = reinterpret_cast<const char*>(a.kpt) + ((int64_t)kvh * a.kpt_cols + kstart) * D * ESZ;
      cz = false;
    } else {
      const int i = it - n0;
      kstart = kb0 + i * BN;
      nval = kb1 - kstart;
      kp = reinterpret_cast<const char*>(a.k) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      vp = reinterpret_cast<const char*>(a.v) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      ktld = RBT;
      ktp = reinterpret_cast<const char*>(a.kt) + ((int64_t)kvh * a.kt_cols + pcol0 + i * BN) * D * ESZ;
      cz = true;
    }
  };

  CopyPlan<NW, true, TN, TN, TT> plan;
  {
    const uint32_t ld[3] = {kld, kld, (uint32_t)RBT};
    plan.init(w, lane, ld);
  }
  auto issue = [&](int it, auto S) {
    const char *kp, *vp, *ktp;
    uint32_t ktld;
    int ks, nv;
    bool cz;
    tile_src(it, kp, vp, ktp, ktld, ks, nv, cz);
    plan.issue(stage(S), lane, TN{kp, kld, nv}, TN{vp, kld, nv}, TT{ktp, ktld, D});
  };

  auto compute = [&](int it, auto S) {
    const char* k_ = stage(S);
    const char* v_ = k_ + O_V;
    const char* kt_ = k_ + O_KT;
    const char *kp, *vp, *ktp;
    uint32_t ktld;
    int kt, nv;
    bool cz;
    tile_src(it, kp, vp, ktp, ktld, kt, nv, cz);
    if (!wave_has_rows || (cz && kt > wq_hi)) return;
    const int kend = kt + min(nv, BN);
    const bool need_mask = (kt + BN > kend) || (cz && kt + BN - 1 > wq0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 sacc = zero16(), pacc = zero16();
      if constexpr (M::E == 8) {
        // K and V fragments read two matrix ops ahead through a ring of three (scheduling
        // barriers keep the order)
        constexpr int NI = 2 * KS;
        auto fkv = [&](int i) {
          return tile_frag<T, RBN>((i & 1) ? v_ : k_, kb * 32 + c, (i >> 1) * M::K + g * M::E);
        };
        typename M::frag fr[3];
        fr[0] = fkv(0);
        fr[1] = fkv(1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i + 2 < NI) fr[(i + 2) % 3] = fkv(i + 2);
          if (i & 1) pacc = M::run(fr[i % 3], of[i >> 1], pacc);
          else sacc = M::run(fr[i % 3], qf[i >> 1], sacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc = M::run(tile_frag<T, RBN>(k_, kb * 32 + c, s * M::K + g * M::E), qf[s], sacc);
          pacc = M::run(tile_frag<T, RBN>(v_, kb * 32 + c, s * M::K + g * M::E), of[s], pacc);
        }
      }
      // the mask test is taken once per tile, not per element, so that the unmasked
      // element loop is one straight block
      // key kt + kb * 32 + crow(r, g) is masked beyond the last valid key and, for the rows'
      // own keys, beyond the row: one per-lane limit against compile-time key offsets
      const int lim = min(kend - 1, cz ? qrow : INT32_MAX) - kt - kb * 32 - 4 * g;
      auto softmax_grad = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -lse2));
          if constexpr (decltype(masked)::value) {
            if (crow(r, 0) > lim) p = 0.f;
          }
          pacc[r] = p * (pacc[r] - rdv);
        }
      };
      if (need_mask) softmax_grad(std::true_type{});
      else softmax_grad(std::false_type{});
      if constexpr (M::E == 8) {
        // K^T fragments read two matrix ops ahead through a ring of three
        constexpr int NQ = NS * DB;
        const typename M::frag df0 = acc_frag<T>(pacc, 0);
        const typename M::frag df1 = acc_frag<T>(pacc, 1);
        auto fk = [&](int i) { return tile_frag<T, RBT>(kt_, (i % DB) * 32 + c, kb * 32 + tread<T>(i / DB, g)); };
        typename M::frag fr[3];
        fr[0] = fk(0);
        fr[1] = fk(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          if (i + 2 < NQ) fr[(i + 2) % 3] = fk(i + 2);
          dqt[i % DB] = M::run(fr[i % 3], i < DB ? df0 : df1, dqt[i % DB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const typename M::frag df = acc_frag<T>(pacc, s);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqt[db] = M::run(tile_frag<T, RBT>(kt_, db * 32 + c, kb * 32 + tread<T>(s, g)), df, dqt[db]);
        }
      }
    }
  };

  run_pipeline<NSTAGE, stage_copies<NW, TN, TN, TT>()>(nkt, issue, compute);

  if (!qvalid) return;
  OT* out = reinterpret_cast<OT*>(a.dq) + (int64_t)qrow * qld + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      store4<OT>(out + db * 32 + r4 * 8 + g * 4, dqt[db][r4 * 4] * a.scale, dqt[db][r4 * 4 + 1] * a.scale,
                dqt[db][r4 * 4 + 2] * a.scale, dqt[db][r4 * 4 + 3] * a.scale);
}

// ---------------------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_dkdv_t(int mode, const DkdvArgs& a, hipStream_t s) {
  dim3 grid(a.nwg), block(512);
  switch (mode) {
    case kDkdvPromptFromReplay:
      hipLaunchKernelGGL((dkdv_kernel<T, float, D, kDkdvPromptFromReplay>), grid, block, 0, s, a);
      break;
    case kDkdvLocal: hipLaunchKernelGGL((dkdv_kernel<T, T, D, kDkdvLocal>), grid, block, 0, s, a); break;
    case kDkdvPrefill:
      if (a.nsplit > 1) hipLaunchKernelGGL((dkdv_kernel<T, float, D, kDkdvPrefill>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dkdv_kernel<T, T, D, kDkdvPrefill>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dkdv(int dtype, int D, int mode, const DkdvArgs& a, hipStream_t s) {
  if (a.nwg == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_dkdv_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_dkdv_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_dkdv_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

template <typename T, int D, int HG>
static hipError_t launch_dq_hg(int mode, bool f32_out, const DqArgs& a, hipStream_t s) {
  dim3 grid(a.nwg), block(512);
  switch (mode) {
    case kDqResponse:
      if (f32_out) hipLaunchKernelGGL((dq_kernel<T, float, D, kDqResponse, HG>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dq_kernel<T, T, D, kDqResponse, HG>), grid, block, 0, s, a);
      break;
    case kDqPrefill:
      if (f32_out) return hipErrorInvalidValue;
      hipLaunchKernelGGL((dq_kernel<T, T, D, kDqPrefill, HG>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_t(int mode, bool f32_out, const DqArgs& a, hipStream_t s) {
  switch (heads_per_wg(a.Hq / a.Hkv)) {
    case 4: return launch_dq_hg<T, D, 4>(mode, f32_out, a, s);
    case 2: return launch_dq_hg<T, D, 2>(mode, f32_out, a, s);
    default: return launch_dq_hg<T, D, 1>(mode, f32_out, a, s);
  }
}

hipError_t launch_dq(int dtype, int D, int mode, bool f32_out, const DqArgs& a, hipStream_t s) {
  if (a.nwg == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_dq_t<bf16, 128>(mode, f32_out, a, s);
  if (dtype == 1 && D == 64) return launch_dq_t<bf16, 64>(mode, f32_out, a, s);
  if (dtype == 0 && D == 64) return launch_dq_t<float, 64>(mode, f32_out, a, s);
  return hipErrorInvalidValue;
}

}  // namespace augtree
