// Forward kernels: causal prompt prefill, replay against the stationary prompt K/V,
// response-local causal replay, and the log-sum-exp merge of the two replay partials.
//
// Attention per head is O = softmax(scale * Q K^T + M) V ("Splitting Prompt Prefill from
// Response Replay ...", §2.2), evaluated tile by tile with an online softmax: each K/V
// tile updates a running row maximum m, normaliser l and unnormalised output (the partial
// state S = (m, l, O_acc) of §3.3, Fig. 8). Each workgroup owns 128 query rows of one
// query head (one wave per 32 rows); K/V tiles of 64 keys are staged in LDS, double
// buffered, with the next tile's global loads in flight during the current tile's math.
//
// Per wave and tile: S^T = K Q^T on the matrix cores (32x32x16 bf16, or 32x32x2 f32), so
// the accumulator holds one query per lane and the softmax statistics are per lane;
// P^T = exp2(S^T * scale*log2e - m) is then fed straight back as the B operand of
// O^T += V^T P^T, with V staged transposed in LDS.
#include "kernels.hpp"

namespace augtree {

template <typename T, typename OT, int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdArgs a) {
  using M = Mma<T>;
  constexpr int BM = kFwdBM, BN = kFwdBN;
  using SK = Stage<T, D, BN>;
  constexpr int KS = D / M::K;   // MFMA steps over head_dim
  constexpr int DB = D / 32;     // 32-wide blocks of head_dim
  constexpr int NS = 32 / M::K;  // MFMA steps per 32-key block
  constexpr int KB = BN / 32;    // 32-key blocks per tile

  __shared__ __attribute__((aligned(16))) T lds_k[2][SK::NAT_ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_vt[2][SK::TR_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int h = blockIdx.y;
  const int kvh = h / (a.Hq / a.Hkv);
  int tile = blockIdx.x;

  int q0, q1, k0, k1;
  bool causal;
  if constexpr (MODE == kFwdPrefill) {
    tile = a.ntiles - 1 - tile;  // longest causal row range first
    q0 = tile * BM;
    q1 = min(q0 + BM, a.nq_rows);
    k0 = 0;
    k1 = q1;
    causal = true;
  } else if constexpr (MODE == kFwdReplayPrompt) {
    q0 = tile * BM;
    q1 = min(q0 + BM, a.nq_rows);
    k0 = 0;
    k1 = a.nkv_rows;
    causal = false;
  } else {
    const int b = branch_of_tile(a.bt, tile);
    const int bs = a.bt.off[b], be = a.bt.off[b + 1];
    q0 = bs + (tile - a.bt.tile_prefix[b]) * BM;
    q1 = min(q0 + BM, be);
    k0 = bs;
    k1 = q1;
    causal = true;
  }

  const int64_t qld = (int64_t)a.Hq * D;
  const int64_t kld = (int64_t)a.Hkv * D;
  const T* qbase = reinterpret_cast<const T*>(a.q) + (int64_t)h * D;
  const T* kbase = reinterpret_cast<const T*>(a.k) + (int64_t)kvh * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (int64_t)kvh * D;

  const int qrow = q0 + w * 32 + c;
  const bool qvalid = qrow < q1;
  const int wq_lo = q0 + w * 32;
  const int wq_hi = min(q1, wq_lo + 32) - 1;
  const bool wave_has_rows = wq_lo < q1;

  typename M::frag qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qvalid ? load_frag<T>(qbase + qrow * qld + s * M::K + g * M::E) : zero_frag<T>();

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = zero16();
  float m_run = -kInf, l_run = 0.f;
  const float sl2 = a.scale_log2;

  const int nkt = (k1 - k0 + BN - 1) / BN;
  typename SK::NatRegs kr;
  typename SK::TrRegs vr;
  SK::load_nat(kr, kbase + k0 * kld, kld, k1 - k0, tid);
  SK::load_tr(vr, vbase + k0 * kld, kld, k1 - k0, tid);
  SK::store_nat(kr, lds_k[0], tid);
  SK::store_tr(vr, lds_vt[0], tid);
  __syncthreads();

  for (int it = 0; it < nkt; ++it) {
    const int kt = k0 + it * BN;
    const int buf = it & 1;
    const bool more = it + 1 < nkt;
    if (more) {
      SK::load_nat(kr, kbase + (kt + BN) * kld, kld, k1 - (kt + BN), tid);
      SK::load_tr(vr, vbase + (kt + BN) * kld, kld, k1 - (kt + BN), tid);
    }
    if (wave_has_rows && !(causal && kt > wq_hi)) {
      const T* lk = lds_k[buf];
      const T* lv = lds_vt[buf];
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int s = 0; s < KS; ++s)
          sacc[kb] = M::run(load_frag<T>(lk + (kb * 32 + c) * SK::NP + s * M::K + g * M::E), qf[s], sacc[kb]);
      }
      const bool need_mask = (kt + BN > k1) || (causal && kt + BN - 1 > wq_lo);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + kb * 32 + crow(r, g);
            if (key >= k1 || (causal && key > qrow)) sacc[kb][r] = -kInf;
          }
      }
      float mt = -kInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = fmaxf(mt, wave_swap_halves(mt));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == -kInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * sl2);
      const float msc = m_use * sl2;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], sl2, -msc));
          sacc[kb][r] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const typename M::frag pf = acc_frag<T>(sacc[kb], s);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = M::run(load_frag<T>(lv + (db * 32 + c) * SK::TP + kb * 32 + tread<T>(s, g)), pf, oacc[db]);
        }
    }
    if (more) {
      SK::store_nat(kr, lds_k[buf ^ 1], tid);
      SK::store_tr(vr, lds_vt[buf ^ 1], tid);
    }
    __syncthreads();
  }

  const float l = l_run + wave_swap_halves(l_run);
  if (qvalid) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    OT* ob = reinterpret_cast<OT*>(a.o) + qrow * qld + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4<OT>(ob + db * 32 + r4 * 8 + g * 4, oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv,
                   oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv);
    if (g == 0)
      a.lse[(int64_t)h * a.nq_rows + qrow] =
          l > 0.f ? (m_run * sl2 + __builtin_amdgcn_logf(l)) * kLn2 : -kInf;
  }
}

// Merge of the replay partial states of each (row, head), e.g. the prompt part and the
// response-local part, or the parts of several prompt K/V shards. Each part is a normalised
// output with its LSE; the combined LSE is m + log(sum_i e^(lse_i - m)) with m = max_i lse_i,
// and the combined output is the e^(lse_i - lse)-weighted sum of the parts, which equals
// merging the unnormalised (m, l, O_acc) states (§3.3, Fig. 8). Parts are visited in index
// order. D/4 lanes handle one (row, head), four fp32 elements per lane.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPB = kThreads / LPR;
  const int tid = threadIdx.x;
  const int64_t idx = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int sub = tid % LPR;
  if (idx >= (int64_t)a.rows * a.Hq) return;
  const int64_t row = idx / a.Hq;
  const int h = (int)(idx % a.Hq);
  const int64_t li = (int64_t)h * a.rows + row;
  float l[kMaxParts];
  float mx = -kInf;
#pragma unroll
  for (int i = 0; i < kMaxParts; ++i) {
    l[i] = i < a.nparts ? a.lse_part[i][li] : -kInf;
    mx = fmaxf(mx, l[i]);
  }
  const int64_t off = idx * D + sub * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -kInf;
  if (mx != -kInf) {
    float e[kMaxParts];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      e[i] = i < a.nparts ? __builtin_amdgcn_exp2f((l[i] - mx) * kLog2e) : 0.f;
      s += e[i];
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      if (i < a.nparts && e[i] > 0.f) {
        const float wgt = e[i] * inv;
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.o_part[i] + off);
        acc[0] += wgt * x[0]; acc[1] += wgt * x[1]; acc[2] += wgt * x[2]; acc[3] += wgt * x[3];
      }
    }
    lse = mx + __builtin_amdgcn_logf(s) * kLn2;
  }
  store4<T>(reinterpret_cast<T*>(a.o) + off, acc[0], acc[1], acc[2], acc[3]);
  if (sub == 0) a.lse[li] = lse;
}

template <typename T, int D>
static hipError_t launch_fwd_t(int mode, const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.ntiles, a.Hq), block(kThreads);
  switch (mode) {
    case kFwdPrefill: hipLaunchKernelGGL((attn_fwd_kernel<T, T, D, kFwdPrefill>), grid, block, 0, s, a); break;
    case kFwdReplayPrompt: hipLaunchKernelGGL((attn_fwd_kernel<T, float, D, kFwdReplayPrompt>), grid, block, 0, s, a); break;
    case kFwdReplayLocal: hipLaunchKernelGGL((attn_fwd_kernel<T, float, D, kFwdReplayLocal>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(int dtype, int D, int mode, const FwdArgs& a, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_fwd_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_fwd_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_fwd_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_merge_t(const MergeArgs& a, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 4);
  const int64_t n = (int64_t)a.rows * a.Hq;
  dim3 grid((unsigned)((n + RPB - 1) / RPB)), block(kThreads);
  hipLaunchKernelGGL((merge_kernel<T, D>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int D, const MergeArgs& a, hipStream_t s) {
  if ((int64_t)a.rows * a.Hq == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_merge_t<bf16, 128>(a, s);
  if (dtype == 1 && D == 64) return launch_merge_t<bf16, 64>(a, s);
  if (dtype == 0 && D == 64) return launch_merge_t<float, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace augtree
