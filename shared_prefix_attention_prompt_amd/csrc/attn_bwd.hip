// Backward kernels for the loss sum(O * dO) of shared-prefix attention.
//
// With P = softmax(scale * Q K^T + M) recomputed from the saved row LSE, the gradients are
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowdot),  dQ = scale dS K,  dK = scale dS^T Q,
// where rowdot[r] = sum_d dO[r, d] O[r, d] (equal to sum_j P[r, j] dP[r, j]).
//
// dK/dV are computed key-stationary: a workgroup of 8 waves owns 256 keys of one key/value
// head (32 per wave, kept in registers with their dK/dV accumulators) and walks every query
// tile that can see them, for every query head mapped to that kv head, in a fixed order. For
// the prompt keys this walk runs over all branches' rows at once, so the prompt gradient of
// every branch is summed inside one accumulator ("Splitting Prompt Prefill from Response
// Replay ...", §3.2: the prompt K/V gradient is the sum over branches) without atomics. When
// the prompt has too few key tiles to fill the GPU, the query tiles are split into a fixed
// number of parts whose fp32 partial sums are added afterwards in part order, so results
// stay bitwise reproducible.
//
// dQ is computed query-stationary in its own pass (it recomputes S and dP), which keeps it
// free of atomics as well.
//
// Query tiles (dK/dV) and key tiles (dQ) of 64 positions are copied global -> LDS by direct
// loads, double buffered, both in natural layout and from the transposed copies (the
// operands of the products that contract over the sequence).
#include "kernels.hpp"

namespace augtree {

template <typename T, typename OT, int D, int MODE>
__global__ __launch_bounds__(512, 2) void dkdv_kernel(DkdvArgs a) {
  using M = Mma<T>;
  constexpr int NW = 8;
  constexpr int ESZ = sizeof(T);
  constexpr int BM = kDkdvBM;
  constexpr int RBN = D * ESZ;   // natural tile row bytes
  constexpr int RBT = BM * ESZ;  // transposed tile row bytes
  constexpr int NT = BM * RBN, TT = D * RBT;
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K;
  constexpr int KPW = 32 * NW;

  __shared__ __attribute__((aligned(1024))) char lv[KPW * RBN];  // this workgroup's V rows
  __shared__ __attribute__((aligned(1024))) char lq0[NT];
  __shared__ __attribute__((aligned(1024))) char lq1[NT];
  __shared__ __attribute__((aligned(1024))) char lo0[NT];
  __shared__ __attribute__((aligned(1024))) char lo1[NT];
  __shared__ __attribute__((aligned(1024))) char lqt0[TT];
  __shared__ __attribute__((aligned(1024))) char lqt1[TT];
  __shared__ __attribute__((aligned(1024))) char lot0[TT];
  __shared__ __attribute__((aligned(1024))) char lot1[TT];
  __shared__ __attribute__((aligned(16))) float ls0[2 * BM];  // lse * log2(e), then rowdot
  __shared__ __attribute__((aligned(16))) float ls1[2 * BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int lid = xcd_remap(blockIdx.x, a.nwg);
  const int per_kvh = a.nktiles * a.nsplit;
  const int kvh = lid / per_kvh;
  const int z = (lid % per_kvh) / a.nktiles;
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
  } else {
    k0 = kti * KPW;
    k1 = min(k0 + KPW, a.nkv_rows);
    t_lo = k0 / BM;
    t_hi = (a.nq_rows + BM - 1) / BM;
  }

  const uint32_t qld = (uint32_t)(a.Hq * D * ESZ);   // bytes between query rows
  const uint32_t tld = (uint32_t)(a.qt_cols * ESZ);  // bytes between transposed rows
  const uint32_t kld = (uint32_t)(a.Hkv * D * ESZ);  // bytes between key rows
  const int key = k0 + w * 32 + c;
  const bool kvalid = key < k1;
  const int wk_lo = k0 + w * 32;

  // V rows of the workgroup's keys go to LDS once; K stays in registers.
  dma_tile<KPW, RBN, NW>(lv, reinterpret_cast<const char*>(a.v) + ((int64_t)k0 * a.Hkv + kvh) * D * ESZ, kld,
                         k1 - k0, w, lane);
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

  // Query tiles in walk order: for each query head of the group, tiles t_lo .. t_hi - 1.
  // The tile being issued is tracked incrementally (branch of the tile included); compute
  // reads what issue recorded for its stage.
  struct Tile { int hq, row0, col0, nval; };
  int it_head = 0, it_t = t_lo, it_b = b;
  if constexpr (MODE == kDkdvPromptFromReplay) it_b = t_lo < t_hi ? branch_of_tile(a.bt, t_lo) : 0;
  const int b_first = it_b;
  auto next_tile = [&]() {
    Tile tl;
    tl.hq = kvh * group + it_head;
    if constexpr (MODE == kDkdvPromptFromReplay) {
      while (it_t >= a.bt.tile_prefix[it_b + 1]) ++it_b;
      const int j = it_t - a.bt.tile_prefix[it_b];
      tl.row0 = a.bt.off[it_b] + j * BM;
      tl.col0 = a.bt.pad[it_b] + j * BM;
      tl.nval = min(BM, a.bt.off[it_b + 1] - tl.row0);
    } else if constexpr (MODE == kDkdvLocal) {
      tl.row0 = a.bt.off[b] + it_t * BM;
      tl.col0 = a.bt.pad[b] + it_t * BM;
      tl.nval = min(BM, a.bt.off[b + 1] - tl.row0);
    } else {
      tl.row0 = it_t * BM;
      tl.col0 = it_t * BM;
      tl.nval = min(BM, a.nq_rows - tl.row0);
    }
    if (++it_t == t_hi) { it_t = t_lo; it_b = b_first; ++it_head; }
    return tl;
  };

  // Row statistics of the next tile: wave 0 lanes 0..31 hold lse * log2(e), lanes 32..63
  // rowdot, one row per lane. Rows past the tile's valid range get lse = +inf, so their
  // probabilities are 0.
  float stat = 0.f;
  auto issue = [&](const Tile& tl, char* q_, char* o_, char* qt_, char* ot_) {
    const char* nat_q = reinterpret_cast<const char*>(a.q) + ((int64_t)tl.row0 * a.Hq + tl.hq) * D * ESZ;
    const char* nat_o = reinterpret_cast<const char*>(a.dout) + ((int64_t)tl.row0 * a.Hq + tl.hq) * D * ESZ;
    const int64_t tr = ((int64_t)tl.hq * D * a.qt_cols + tl.col0) * ESZ;
    dma_tile<BM, RBN, NW>(q_, nat_q, qld, tl.nval, w, lane);
    dma_tile<BM, RBN, NW>(o_, nat_o, qld, tl.nval, w, lane);
    dma_tile<D, RBT, NW>(qt_, reinterpret_cast<const char*>(a.qt) + tr, tld, D, w, lane);
    dma_tile<D, RBT, NW>(ot_, reinterpret_cast<const char*>(a.dot) + tr, tld, D, w, lane);
    if (w == 0) {
      const bool ok = c < tl.nval;
      const int64_t si = (int64_t)tl.hq * a.nq_rows + tl.row0 + min(c, tl.nval - 1);
      stat = g == 0 ? (ok ? a.lse[si] * kLog2e : kInf) : (ok ? a.rowdot[si] : 0.f);
    }
  };
  auto publish_stat = [&](float* st) {
    if (w == 0) st[lane] = stat;
  };

  auto compute = [&](const Tile& tl, const char* q_, const char* o_, const char* qt_, const char* ot_,
                     const float* st) {
    const int row0 = tl.row0;
    if (causal && row0 + 31 < wk_lo) return;  // every query of the tile precedes every key
    const bool need_mask = causal && row0 < wk_lo + 31;  // the diagonal tile
    f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sacc = M::run(tile_frag<T, RBN>(q_, c, s * M::K + g * M::E), kf[s], sacc);
      pacc = M::run(tile_frag<T, RBN>(o_, c, s * M::K + g * M::E), tile_frag<T, RBN>(lv, w * 32 + c, s * M::K + g * M::E),
                    pacc);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int qi = r4 * 8 + g * 4;
      const f32x4 L = *reinterpret_cast<const f32x4*>(st + qi);
      const f32x4 R = *reinterpret_cast<const f32x4*>(st + BM + qi);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r4 * 4 + j;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -L[j]));
        if (need_mask && key > row0 + qi + j) p = 0.f;
        pacc[r] = p * (pacc[r] - R[j]);
        sacc[r] = p;
      }
    }
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
  };

  Tile t0 = {0, 0, 0, 1}, t1 = {0, 0, 0, 1};
  if (niter > 0) {
    t0 = next_tile();
    issue(t0, lq0, lo0, lqt0, lot0);
    publish_stat(ls0);
  }
  wait_vm();
  __syncthreads();
  for (int it = 0; it < niter; it += 2) {
    if (it + 1 < niter) {
      t1 = next_tile();
      issue(t1, lq1, lo1, lqt1, lot1);
    }
    compute(t0, lq0, lo0, lqt0, lot0, ls0);
    if (it + 1 < niter) publish_stat(ls1);
    wait_vm();
    __syncthreads();
    if (it + 1 >= niter) break;
    if (it + 2 < niter) {
      t0 = next_tile();
      issue(t0, lq0, lo0, lqt0, lot0);
    }
    compute(t1, lq1, lo1, lqt1, lot1, ls1);
    if (it + 2 < niter) publish_stat(ls0);
    wait_vm();
    __syncthreads();
  }

  if (!kvalid) return;
  int64_t obase = ((int64_t)key * a.Hkv + kvh) * D;
  if constexpr (MODE == kDkdvPromptFromReplay) obase += (int64_t)z * a.split_stride;
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

template <typename T, int D, int MODE, int HG>
__global__ __launch_bounds__(512, 2) void dq_kernel(DqArgs a) {
  using M = Mma<T>;
  constexpr int NW = 8;
  constexpr int ESZ = sizeof(T);
  constexpr int BN = kDqBN;
  constexpr int RBN = D * ESZ, RBT = BN * ESZ;
  constexpr int NT = BN * RBN, TT = D * RBT;
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K, KB = BN / 32;
  constexpr int RT = 32 * (NW / HG);

  __shared__ __attribute__((aligned(1024))) char lk0[NT];
  __shared__ __attribute__((aligned(1024))) char lk1[NT];
  __shared__ __attribute__((aligned(1024))) char lv0[NT];
  __shared__ __attribute__((aligned(1024))) char lv1[NT];
  __shared__ __attribute__((aligned(1024))) char lkt0[TT];
  __shared__ __attribute__((aligned(1024))) char lkt1[TT];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
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
    kb1 = q1;
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
      ktld = (uint32_t)(a.kpt_cols * ESZ);
      ktp = reinterpret_cast<const char*>(a.kpt) + (int64_t)kvh * D * ktld + (int64_t)kstart * ESZ;
      cz = false;
    } else {
      const int i = it - n0;
      kstart = kb0 + i * BN;
      nval = kb1 - kstart;
      kp = reinterpret_cast<const char*>(a.k) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      vp = reinterpret_cast<const char*>(a.v) + (int64_t)kstart * kld + (int64_t)kvh * D * ESZ;
      ktld = (uint32_t)(a.kt_cols * ESZ);
      ktp = reinterpret_cast<const char*>(a.kt) + (int64_t)kvh * D * ktld + (int64_t)(pcol0 + i * BN) * ESZ;
      cz = true;
    }
  };

  auto issue = [&](int it, char* k_, char* v_, char* kt_) {
    const char *kp, *vp, *ktp;
    uint32_t ktld;
    int ks, nv;
    bool cz;
    tile_src(it, kp, vp, ktp, ktld, ks, nv, cz);
    dma_tile<BN, RBN, NW>(k_, kp, kld, nv, w, lane);
    dma_tile<BN, RBN, NW>(v_, vp, kld, nv, w, lane);
    dma_tile<D, RBT, NW>(kt_, ktp, ktld, D, w, lane);
  };

  auto compute = [&](int it, const char* k_, const char* v_, const char* kt_) {
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
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = M::run(tile_frag<T, RBN>(k_, kb * 32 + c, s * M::K + g * M::E), qf[s], sacc);
        pacc = M::run(tile_frag<T, RBN>(v_, kb * 32 + c, s * M::K + g * M::E), of[s], pacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -lse2));
        if (need_mask) {
          const int kk = kt + kb * 32 + crow(r, g);
          if (kk >= kend || (cz && kk > qrow)) p = 0.f;
        }
        pacc[r] = p * (pacc[r] - rdv);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const typename M::frag df = acc_frag<T>(pacc, s);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dqt[db] = M::run(tile_frag<T, RBT>(kt_, db * 32 + c, kb * 32 + tread<T>(s, g)), df, dqt[db]);
      }
    }
  };

  issue(0, lk0, lv0, lkt0);
  wait_vm();
  __syncthreads();
  for (int it = 0; it < nkt; it += 2) {
    if (it + 1 < nkt) issue(it + 1, lk1, lv1, lkt1);
    compute(it, lk0, lv0, lkt0);
    wait_vm();
    __syncthreads();
    if (it + 1 >= nkt) break;
    if (it + 2 < nkt) issue(it + 2, lk0, lv0, lkt0);
    compute(it + 1, lk1, lv1, lkt1);
    wait_vm();
    __syncthreads();
  }

  if (!qvalid) return;
  T* out = reinterpret_cast<T*>(a.dq) + (int64_t)qrow * qld + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      store4<T>(out + db * 32 + r4 * 8 + g * 4, dqt[db][r4 * 4] * a.scale, dqt[db][r4 * 4 + 1] * a.scale,
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
    case kDkdvPrefill: hipLaunchKernelGGL((dkdv_kernel<T, T, D, kDkdvPrefill>), grid, block, 0, s, a); break;
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
static hipError_t launch_dq_hg(int mode, const DqArgs& a, hipStream_t s) {
  dim3 grid(a.nwg), block(512);
  switch (mode) {
    case kDqResponse: hipLaunchKernelGGL((dq_kernel<T, D, kDqResponse, HG>), grid, block, 0, s, a); break;
    case kDqPrefill: hipLaunchKernelGGL((dq_kernel<T, D, kDqPrefill, HG>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_t(int mode, const DqArgs& a, hipStream_t s) {
  switch (heads_per_wg(a.Hq / a.Hkv)) {
    case 4: return launch_dq_hg<T, D, 4>(mode, a, s);
    case 2: return launch_dq_hg<T, D, 2>(mode, a, s);
    default: return launch_dq_hg<T, D, 1>(mode, a, s);
  }
}

hipError_t launch_dq(int dtype, int D, int mode, const DqArgs& a, hipStream_t s) {
  if (a.nwg == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_dq_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_dq_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_dq_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

}  // namespace augtree
