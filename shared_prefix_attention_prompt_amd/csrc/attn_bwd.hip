// Backward kernels for the loss sum(O * dO) of shared-prefix attention.
//
// With P = softmax(scale * Q K^T + M) recomputed from the saved row LSE, the gradients are
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowdot),  dQ = scale dS K,  dK = scale dS^T Q,
// where rowdot[r] = sum_d dO[r, d] O[r, d] (equal to sum_j P[r, j] dP[r, j]).
//
// dK/dV are computed key-stationary: a workgroup owns 128 keys of one key/value head
// (32 per wave, kept in registers) and walks every query tile that can see them, for every
// query head mapped to that kv head, in a fixed order. For the prompt keys this walk runs
// over all branches' rows at once, so the prompt gradient of every branch is summed inside
// one accumulator ("Splitting Prompt Prefill from Response Replay ...", §3.2: the prompt K/V
// gradient is the sum over branches) without atomics. When the prompt has too few key tiles
// to fill the GPU, the row range is split into a fixed number of parts whose fp32 partial
// sums are added afterwards in part order, so results stay bitwise reproducible.
//
// dQ is computed query-stationary in its own pass (it recomputes S and dP), which keeps it
// free of atomics as well.
#include "kernels.hpp"

namespace augtree {

// rowdot[h][r] = sum_d dO[r][h][d] * O[r][h][d]; D*sizeof(T)/16 lanes per (row, head).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rowdot_kernel(RowDotArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LPR = D / EPC;
  constexpr int RPB = kThreads / LPR;
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

template <typename T, typename OT, int D, int MODE>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(DkdvArgs a) {
  using M = Mma<T>;
  constexpr int BN = kDkdvBN, BM = kDkdvBM;
  using SQ = Stage<T, D, BM>;
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K, QB = BM / 32;

  __shared__ __attribute__((aligned(16))) T lds_q[SQ::NAT_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_qt[SQ::TR_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do[SQ::NAT_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_dot[SQ::TR_ELEMS];
  __shared__ __attribute__((aligned(16))) float lds_lse[BM];
  __shared__ __attribute__((aligned(16))) float lds_rd[BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int kvh = blockIdx.y;
  const int group = a.Hq / a.Hkv;

  int k0, k1, q_lo, q_hi;
  bool causal;
  if constexpr (MODE == kDkdvPromptFromReplay) {
    k0 = blockIdx.x * BN;
    k1 = min(k0 + BN, a.nkv_rows);
    const int nqt = (a.nq_rows + BM - 1) / BM;
    const int per = (nqt + a.nsplit - 1) / a.nsplit;
    q_lo = min(nqt, (int)blockIdx.z * per) * BM;
    q_hi = min(a.nq_rows, min(nqt, ((int)blockIdx.z + 1) * per) * BM);
    causal = false;
  } else if constexpr (MODE == kDkdvLocal) {
    const int b = branch_of_tile(a.bt, blockIdx.x);
    const int be = a.bt.off[b + 1];
    k0 = a.bt.off[b] + (blockIdx.x - a.bt.tile_prefix[b]) * BN;
    k1 = min(k0 + BN, be);
    q_lo = k0;
    q_hi = be;
    causal = true;
  } else {
    k0 = blockIdx.x * BN;
    k1 = min(k0 + BN, a.nkv_rows);
    q_lo = k0;
    q_hi = a.nq_rows;
    causal = true;
  }

  const int64_t qld = (int64_t)a.Hq * D;
  const int64_t kld = (int64_t)a.Hkv * D;
  const int key = k0 + w * 32 + c;
  const bool kvalid = key < k1;
  const int wk_lo = k0 + w * 32;  // first key of this wave

  typename M::frag kf[KS], vf[KS];
  {
    const T* kb = reinterpret_cast<const T*>(a.k) + (int64_t)kvh * D + key * kld;
    const T* vb = reinterpret_cast<const T*>(a.v) + (int64_t)kvh * D + key * kld;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = kvalid ? load_frag<T>(kb + s * M::K + g * M::E) : zero_frag<T>();
      vf[s] = kvalid ? load_frag<T>(vb + s * M::K + g * M::E) : zero_frag<T>();
    }
  }
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) { dkt[db] = zero16(); dvt[db] = zero16(); }
  const float sl2 = a.scale_log2;

  const int nqt = q_hi > q_lo ? (q_hi - q_lo + BM - 1) / BM : 0;
  const int niter = nqt * group;
  typename SQ::TrRegs qr, dr;
  float lse_r = 0.f, rd_r = 0.f;

  // iteration it -> (query head j = it / nqt, tile it % nqt)
  auto load_iter = [&](int it) {
    const int hq = kvh * group + it / nqt;
    const int qt = q_lo + (it % nqt) * BM;
    const int nval = q_hi - qt;
    const T* qs = reinterpret_cast<const T*>(a.q) + (int64_t)hq * D + qt * qld;
    const T* ds = reinterpret_cast<const T*>(a.dout) + (int64_t)hq * D + qt * qld;
    SQ::load_tr(qr, qs, qld, nval, tid);
    SQ::load_tr(dr, ds, qld, nval, tid);
    if (tid < BM) {
      const bool v = tid < nval;
      lse_r = v ? a.lse[(int64_t)hq * a.nq_rows + qt + tid] * kLog2e : kInf;
      rd_r = v ? a.rowdot[(int64_t)hq * a.nq_rows + qt + tid] : 0.f;
    }
  };

  if (niter > 0) load_iter(0);
  for (int it = 0; it < niter; ++it) {
    const int qt = q_lo + (it % nqt) * BM;
    __syncthreads();  // every wave is done with the previous tile
    SQ::store_nat_from_tr(qr, lds_q, tid);
    SQ::store_tr(qr, lds_qt, tid);
    SQ::store_nat_from_tr(dr, lds_do, tid);
    SQ::store_tr(dr, lds_dot, tid);
    if (tid < BM) { lds_lse[tid] = lse_r; lds_rd[tid] = rd_r; }
    __syncthreads();
    if (it + 1 < niter) load_iter(it + 1);

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qa = qt + qb * 32;
      if (causal && qa + 31 < wk_lo) continue;  // every query of the block precedes every key
      const bool need_mask = causal && qa < wk_lo + 31;
      f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = M::run(load_frag<T>(lds_q + (qb * 32 + c) * SQ::NP + s * M::K + g * M::E), kf[s], sacc);
        pacc = M::run(load_frag<T>(lds_do + (qb * 32 + c) * SQ::NP + s * M::K + g * M::E), vf[s], pacc);
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = qb * 32 + r4 * 8 + g * 4;
        const f32x4 L = *reinterpret_cast<const f32x4*>(lds_lse + qi);
        const f32x4 R = *reinterpret_cast<const f32x4*>(lds_rd + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r4 * 4 + j;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -L[j]));
          if (need_mask && key > qt + qi + j) p = 0.f;
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
          dvt[db] = M::run(load_frag<T>(lds_dot + (db * 32 + c) * SQ::TP + qb * 32 + tread<T>(s, g)), pf, dvt[db]);
          dkt[db] = M::run(load_frag<T>(lds_qt + (db * 32 + c) * SQ::TP + qb * 32 + tread<T>(s, g)), df, dkt[db]);
        }
      }
    }
  }

  if (!kvalid) return;
  int64_t obase = key * kld + (int64_t)kvh * D;
  if constexpr (MODE == kDkdvPromptFromReplay) obase += (int64_t)blockIdx.z * a.split_stride;
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

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void dq_kernel(DqArgs a) {
  using M = Mma<T>;
  constexpr int BM = kDqBM, BN = kDqBN;
  using SK = Stage<T, D, BN>;
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K, KB = BN / 32;

  __shared__ __attribute__((aligned(16))) T lds_k[2][SK::NAT_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_kt[2][SK::TR_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[2][SK::NAT_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int h = blockIdx.y;
  const int kvh = h / (a.Hq / a.Hkv);
  int tile = blockIdx.x;

  int q0, q1;          // query rows
  int n0 = 0;          // prompt key tiles walked first (response mode)
  int kb0, kb1;        // own-sequence key range walked (causal)
  if constexpr (MODE == kDqResponse) {
    const int b = branch_of_tile(a.bt, tile);
    const int bs = a.bt.off[b], be = a.bt.off[b + 1];
    q0 = bs + (tile - a.bt.tile_prefix[b]) * BM;
    q1 = min(q0 + BM, be);
    n0 = (a.nprompt + BN - 1) / BN;
    kb0 = bs;
    kb1 = q1;
  } else {
    tile = a.ntiles - 1 - tile;  // longest causal row range first
    q0 = tile * BM;
    q1 = min(q0 + BM, a.nq_rows);
    kb0 = 0;
    kb1 = q1;
  }
  const int n1 = (kb1 - kb0 + BN - 1) / BN;
  const int nkt = n0 + n1;

  const int64_t qld = (int64_t)a.Hq * D;
  const int64_t kld = (int64_t)a.Hkv * D;
  const int qrow = q0 + w * 32 + c;
  const bool qvalid = qrow < q1;
  const int wq_lo = q0 + w * 32;
  const int wq_hi = min(q1, wq_lo + 32) - 1;
  const bool wave_has_rows = wq_lo < q1;

  typename M::frag qf[KS], of[KS];
  {
    const T* qb = reinterpret_cast<const T*>(a.q) + (int64_t)h * D + qrow * qld;
    const T* ob = reinterpret_cast<const T*>(a.dout) + (int64_t)h * D + qrow * qld;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = qvalid ? load_frag<T>(qb + s * M::K + g * M::E) : zero_frag<T>();
      of[s] = qvalid ? load_frag<T>(ob + s * M::K + g * M::E) : zero_frag<T>();
    }
  }
  const float lse2 = qvalid ? a.lse[(int64_t)h * a.nq_rows + qrow] * kLog2e : kInf;
  const float rdv = qvalid ? a.rowdot[(int64_t)h * a.nq_rows + qrow] : 0.f;
  const float sl2 = a.scale_log2;

  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = zero16();

  // key tile it: prompt tiles first (response mode, no mask), then own causal tiles
  auto tile_src = [&](int it, const T*& kp, const T*& vp, int& kstart, int& nval, bool& cz) {
    if (it < n0) {
      kstart = it * BN;
      nval = a.nprompt - kstart;
      kp = reinterpret_cast<const T*>(a.kp) + (int64_t)kvh * D + kstart * kld;
      vp = reinterpret_cast<const T*>(a.vp) + (int64_t)kvh * D + kstart * kld;
      cz = false;
    } else {
      kstart = kb0 + (it - n0) * BN;
      nval = kb1 - kstart;
      kp = reinterpret_cast<const T*>(a.k) + (int64_t)kvh * D + kstart * kld;
      vp = reinterpret_cast<const T*>(a.v) + (int64_t)kvh * D + kstart * kld;
      cz = true;
    }
  };

  typename SK::TrRegs kr;
  typename SK::NatRegs vr;
  if (nkt > 0) {
    const T *kp, *vp;
    int ks, nv;
    bool cz;
    tile_src(0, kp, vp, ks, nv, cz);
    SK::load_tr(kr, kp, kld, nv, tid);
    SK::load_nat(vr, vp, kld, nv, tid);
    SK::store_nat_from_tr(kr, lds_k[0], tid);
    SK::store_tr(kr, lds_kt[0], tid);
    SK::store_nat(vr, lds_v[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < nkt; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < nkt;
    const T *kp, *vp;
    int kt, nv;
    bool cz;
    tile_src(it, kp, vp, kt, nv, cz);
    const int kend = kt + min(nv, BN);
    if (more) {
      const T *kp2, *vp2;
      int ks2, nv2;
      bool cz2;
      tile_src(it + 1, kp2, vp2, ks2, nv2, cz2);
      SK::load_tr(kr, kp2, kld, nv2, tid);
      SK::load_nat(vr, vp2, kld, nv2, tid);
    }
    if (wave_has_rows && !(cz && kt > wq_hi)) {
      const T* lk = lds_k[buf];
      const T* lkt = lds_kt[buf];
      const T* lv = lds_v[buf];
      f32x16 sacc[KB], pacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = zero16();
        pacc[kb] = zero16();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[kb] = M::run(load_frag<T>(lk + (kb * 32 + c) * SK::NP + s * M::K + g * M::E), qf[s], sacc[kb]);
          pacc[kb] = M::run(load_frag<T>(lv + (kb * 32 + c) * SK::NP + s * M::K + g * M::E), of[s], pacc[kb]);
        }
      }
      const bool need_mask = (kt + BN > kend) || (cz && kt + BN - 1 > wq_lo);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], sl2, -lse2));
          if (need_mask) {
            const int kk = kt + kb * 32 + crow(r, g);
            if (kk >= kend || (cz && kk > qrow)) p = 0.f;
          }
          pacc[kb][r] = p * (pacc[kb][r] - rdv);
        }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const typename M::frag df = acc_frag<T>(pacc[kb], s);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqt[db] = M::run(load_frag<T>(lkt + (db * 32 + c) * SK::TP + kb * 32 + tread<T>(s, g)), df, dqt[db]);
        }
    }
    if (more) {
      SK::store_nat_from_tr(kr, lds_k[buf ^ 1], tid);
      SK::store_tr(kr, lds_kt[buf ^ 1], tid);
      SK::store_nat(vr, lds_v[buf ^ 1], tid);
    }
    __syncthreads();
  }

  if (!qvalid) return;
  T* out = reinterpret_cast<T*>(a.dq) + qrow * qld + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      store4<T>(out + db * 32 + r4 * 8 + g * 4, dqt[db][r4 * 4] * a.scale, dqt[db][r4 * 4 + 1] * a.scale,
                dqt[db][r4 * 4 + 2] * a.scale, dqt[db][r4 * 4 + 3] * a.scale);
}

// out[i] = part[0][i] + part[1][i] + ... in part order (fixed, so reproducible).
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(SplitReduceArgs a) {
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= a.n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.part + i4);
  for (int s = 1; s < a.nsplit; ++s) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part + s * a.n + i4);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  *reinterpret_cast<f32x4*>(a.out + i4) = acc;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_rowdot_t(const RowDotArgs& a, hipStream_t s) {
  constexpr int RPB = kThreads / (D / (16 / (int)sizeof(T)));
  const int64_t n = (int64_t)a.rows * a.Hq;
  hipLaunchKernelGGL((rowdot_kernel<T, D>), dim3((unsigned)((n + RPB - 1) / RPB)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowdot(int dtype, int D, const RowDotArgs& a, hipStream_t s) {
  if ((int64_t)a.rows * a.Hq == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_rowdot_t<bf16, 128>(a, s);
  if (dtype == 1 && D == 64) return launch_rowdot_t<bf16, 64>(a, s);
  if (dtype == 0 && D == 64) return launch_rowdot_t<float, 64>(a, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_dkdv_t(int mode, const DkdvArgs& a, hipStream_t s) {
  dim3 block(kThreads);
  switch (mode) {
    case kDkdvPromptFromReplay:
      hipLaunchKernelGGL((dkdv_kernel<T, float, D, kDkdvPromptFromReplay>), dim3(a.nktiles, a.Hkv, a.nsplit), block, 0, s, a);
      break;
    case kDkdvLocal:
      hipLaunchKernelGGL((dkdv_kernel<T, T, D, kDkdvLocal>), dim3(a.nktiles, a.Hkv, 1), block, 0, s, a);
      break;
    case kDkdvPrefill:
      hipLaunchKernelGGL((dkdv_kernel<T, T, D, kDkdvPrefill>), dim3(a.nktiles, a.Hkv, 1), block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dkdv(int dtype, int D, int mode, const DkdvArgs& a, hipStream_t s) {
  if (a.nktiles == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_dkdv_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_dkdv_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_dkdv_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_dq_t(int mode, const DqArgs& a, hipStream_t s) {
  dim3 grid(a.ntiles, a.Hq), block(kThreads);
  switch (mode) {
    case kDqResponse: hipLaunchKernelGGL((dq_kernel<T, D, kDqResponse>), grid, block, 0, s, a); break;
    case kDqPrefill: hipLaunchKernelGGL((dq_kernel<T, D, kDqPrefill>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dq(int dtype, int D, int mode, const DqArgs& a, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_dq_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_dq_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_dq_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(const SplitReduceArgs& a, int, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int64_t n4 = a.n / 4;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace augtree
