// Forward kernels: causal prompt prefill, replay against the stationary prompt K/V, and
// response-local causal replay.
//
// Attention per head is O = softmax(scale * Q K^T + M) V ("Splitting Prompt Prefill from
// Response Replay ...", §2.2), evaluated tile by tile with an online softmax: each K/V tile
// updates a running row maximum m, normaliser l and unnormalised output (the partial state
// S = (m, l, O_acc) of §3.3, Fig. 8).
//
// A workgroup is 8 waves of 32 query rows (two per SIMD); its waves cover HG query heads of
// one key/value group (HG = 4 for grouped-query heads, so one staged K/V tile serves four
// heads; HG = 7 for seven heads per kv head in the branch-local mode, one wave idle). K/V tiles of 64 keys go global -> LDS by direct loads through a 4-stage ring: while
// tile i is used, tile i + 1 is resident too (its scores are computed one iteration early,
// interleaved with tile i's softmax) and two more are in flight.
//
// Per wave and tile: S^T = K Q^T on the matrix cores, so the accumulator holds one query per
// lane and the softmax statistics are per lane; P^T = exp2(S^T * scale*log2e - m) is fed
// straight back as the B operand of O^T += V^T P^T, with V^T read from the transposed copy
// (stored tile by tile, so each 64-key V^T tile is one contiguous block).
// The running maximum is only raised when some row's tile maximum exceeds it by more than
// 2^8 (in exp2 units); below that the stale maximum is kept, probabilities stay <= 2^8 and
// the output accumulator is not rescaled. The result is the same softmax: the normaliser and
// the accumulator always share one reference maximum.
#include "kernels.hpp"

namespace augtree {

constexpr float kRescaleGap = 8.f;  // log2 of the largest unnormalised probability kept

template <typename T, typename OT, int D, int MODE, int HG>
__global__ __launch_bounds__(kFwdWaves * 64, 2) void attn_fwd_kernel(FwdArgs a) {
  using M = Mma<T>;
  constexpr int NW = kFwdWaves;
  constexpr int NSTAGE = 4;  // LDS stages
  constexpr int ESZ = sizeof(T);
  constexpr int BN = kFwdBN;
  constexpr int RBK = D * ESZ;   // bytes of a natural K tile row
  constexpr int RBV = BN * ESZ;  // bytes of a transposed V tile row
  using TK = TileSrc<BN, RBK>;  // K tile, natural
  using TV = TileSrc<D, RBV>;   // V^T tile, from the transposed copy
  constexpr int VOFF = TK::NB * 1024;
  constexpr int SB = (TK::NB + TV::NB) * 1024;  // bytes per stage
  constexpr int KS = D / M::K, DB = D / 32, NS = 32 / M::K, KB = BN / 32;
  constexpr int RT = 32 * (NW / HG);  // query rows per workgroup

  // one LDS object per stage (K tile, then V^T tile): distinct objects keep the stages apart
  // for the compiler
  __shared__ __attribute__((aligned(1024))) char ls0[SB];
  __shared__ __attribute__((aligned(1024))) char ls1[SB];
  __shared__ __attribute__((aligned(1024))) char ls2[SB];
  __shared__ __attribute__((aligned(1024))) char ls3[SB];
  auto stage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return ls0; else if constexpr (st == 1) return ls1; else if constexpr (st == 2) return ls2; else return ls3;
  };

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lid = xcd_remap(blockIdx.x, a.nwg);
  const int hs = lid / a.ntiles;
  int tile = lid % a.ntiles;
  const int h = hs * HG + (w % HG);
  const int kvh = (hs * HG) / (a.Hq / a.Hkv);
  const int rb = w / HG;

  int q0, q1, k0, k1, vcol0;
  bool causal;
  if constexpr (MODE == kFwdPrefill) {
    tile = a.ntiles - 1 - tile;  // longest causal row range first
    q0 = tile * RT;
    q1 = min(q0 + RT, a.nq_rows);
    k0 = 0;
    k1 = q1;
    vcol0 = 0;
    causal = true;
  } else if constexpr (MODE == kFwdReplayPrompt) {
    q0 = tile * RT;
    q1 = min(q0 + RT, a.nq_rows);
    k0 = 0;
    k1 = a.nkv_rows;
    vcol0 = 0;
    causal = false;
  } else {
    const int b = branch_of_tile(a.bt, tile);
    const int bs = a.bt.off[b], be = a.bt.off[b + 1];
    q0 = bs + (tile - a.bt.tile_prefix[b]) * RT;
    q1 = min(q0 + RT, be);
    k0 = bs;
    k1 = q1;
    vcol0 = a.bt.pad[b];
    causal = true;
  }

  const uint32_t kld = (uint32_t)(a.Hkv * D * ESZ);  // bytes between key rows
  constexpr uint32_t vld = RBV;  // V^T tiles are contiguous [D][BN] blocks
  const char* kbase = reinterpret_cast<const char*>(a.k) + (int64_t)kvh * D * ESZ;
  const char* vbase = reinterpret_cast<const char*>(a.vt) + (int64_t)kvh * a.vt_cols * D * ESZ;

  const int wq0 = q0 + rb * 32;
  const int qrow = wq0 + c;
  const bool qvalid = qrow < q1;
  const int wq_hi = min(q1, wq0 + 32) - 1;
  const bool wave_has_rows = wq0 < q1;

  typename M::frag qf[KS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((int64_t)qrow * a.Hq + h) * D + g * M::E;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qvalid ? gload_frag<T>(qp + s * M::K) : zero_frag<T>();
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = zero16();
  float m_run = -kInf, l_run = 0.f;
  const float sl2 = a.scale_log2;
  const int nkt = (k1 - k0 + BN - 1) / BN;

  CopyPlan<NW, true, TK, TV> plan;
  {
    const uint32_t ld[2] = {kld, vld};
    plan.init(w, lane, ld);
  }
  auto issue = [&](int it, auto S) {
    const int kt = k0 + it * BN;
    plan.issue(stage(S), lane, TK{kbase + (int64_t)kt * kld, kld, k1 - kt},
               TV{vbase + (int64_t)(vcol0 + it * BN) * D * ESZ, vld, D});
  };

  // Scores of tile it are computed one iteration early (while tile it - 1's softmax runs on
  // the vector ALUs), into one of two register buffers chosen by the stage parity.
  f32x16 sbuf[2][KB];
  auto active = [&](int it) { return wave_has_rows && !(causal && k0 + it * BN > wq_hi); };
  auto scores = [&](auto S, f32x16 (&sacc)[KB]) {
    const char* lk = stage(S);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = zero16();
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[kb] = M::run(tile_frag<T, RBK>(lk, kb * 32 + c, s * M::K + g * M::E), qf[s], sacc[kb]);
    }
  };

  auto compute = [&](int it, auto S) {
    constexpr int st = decltype(S)::value;
    constexpr int nst = (st + 1) % NSTAGE;
    static_assert(NSTAGE % 2 == 0, "buffer parity follows the stage");
    f32x16 (&sacc)[KB] = sbuf[st & 1];
    f32x16 (&snext)[KB] = sbuf[nst & 1];
    // a wave is active on a prefix of the tiles (the causal limit only grows), so an inactive
    // wave needs no further scores
    if (!active(it)) return;
    if (it == 0) scores(S, sacc);
    const char* lv = stage(S) + VOFF;
    const int kt = k0 + it * BN;
    if ((kt + BN > k1) || (causal && kt + BN - 1 > wq0)) {
      // key kt + kb * 32 + crow(r, g) is masked beyond the last valid key and, causally, beyond
      // the row: one per-lane limit per tile against compile-time key offsets
      const int lim = min(k1 - 1, causal ? qrow : INT32_MAX) - kt - 4 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + crow(r, 0) > lim) sacc[kb][r] = -kInf;
    }
    // The next tile's scores go to the matrix cores (its stage has landed; past the last
    // tile it holds a repeat, whose scores are never used) interleaved, instruction by
    // instruction, with this tile's maximum and probabilities (taken against the running
    // maximum and redone in the rare case that it is raised). Scheduling barriers keep the
    // order; K fragments are read two matrix ops ahead.
    {
      constexpr int NI = KB * KS;  // score matrix ops
      constexpr int NE = KB * 16;  // softmax elements per lane
      const char* lk = stage(std::integral_constant<int, nst>{});
      auto kfrag = [&](int i) { return tile_frag<T, RBK>(lk, (i % KB) * 32 + c, (i / KB) * M::K + g * M::E); };
      const float msc = m_run == -kInf ? 0.f : m_run * sl2;
      typename M::frag fr[3];
      fr[0] = kfrag(0);
      fr[1] = kfrag(1);
      float mt = -kInf;
      f32x16 pacc[KB];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i + 2 < NI) fr[(i + 2) % 3] = kfrag(i + 2);
        const int kb = i % KB, s_ = i / KB;
        snext[kb] = M::run(fr[i % 3], qf[s_], s_ == 0 ? zero16() : snext[kb]);
#pragma unroll
        for (int j = i * NE / NI; j < (i + 1) * NE / NI; ++j) {
          const float x = sacc[j / 16][j % 16];
          mt = fmaxf(mt, x);
          pacc[j / 16][j % 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, sl2, -msc));
          asm volatile("" : "+v"(pacc[j / 16][j % 16]));  // computed here, not sunk into a branch
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mt = halves_max(mt);
      if (__builtin_amdgcn_ballot_w64(mt * sl2 > m_run * sl2 + kRescaleGap) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -kInf ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        l_run *= alpha;
        m_run = m_new;
        const float msc2 = m_run == -kInf ? 0.f : m_run * sl2;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) pacc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], sl2, -msc2));
      }
      if constexpr (M::E == 8) {
        // V^T fragments read two matrix ops ahead through a ring of three
        constexpr int NP = KB * NS * DB;
        auto fv = [&](int i) {
          const int db = i % DB, ks = i / DB;  // ks = kb * NS + s
          return tile_frag<T, RBV>(lv, db * 32 + c, (ks / NS) * 32 + tread<T>(ks % NS, g));
        };
        typename M::frag pfs[KB * NS];
#pragma unroll
        for (int ks = 0; ks < KB * NS; ++ks) {
          pfs[ks] = acc_frag<T>(pacc[ks / NS], ks % NS);
          l_run = frag_sum(pfs[ks], l_run);
        }
        typename M::frag fr[3];
        fr[0] = fv(0);
        fr[1] = fv(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          if (i + 2 < NP) fr[(i + 2) % 3] = fv(i + 2);
          oacc[i % DB] = M::run(fr[i % 3], pfs[i / DB], oacc[i % DB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const typename M::frag pf = acc_frag<T>(pacc[kb], s);
            l_run = frag_sum(pf, l_run);
#pragma unroll
            for (int db = 0; db < DB; ++db)
              oacc[db] = M::run(tile_frag<T, RBV>(lv, db * 32 + c, kb * 32 + tread<T>(s, g)), pf, oacc[db]);
          }
      }
    }
  };

  run_pipeline<NSTAGE, stage_copies<NW, TK, TV>(), 1>(nkt, issue, compute);

  const float l = halves_sum(l_run);
  if (qvalid) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    OT* ob = reinterpret_cast<OT*>(a.o) + ((int64_t)qrow * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4<OT>(ob + db * 32 + r4 * 8 + g * 4, oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv,
                   oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv);
    if (g == 0)
      a.lse[(int64_t)h * a.nq_rows + qrow] = l > 0.f ? (m_run * sl2 + __builtin_amdgcn_logf(l)) * kLn2 : -kInf;
  }
}

int heads_per_wg(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }
int rows_per_wg(int group) { return 32 * (kFwdWaves / heads_per_wg(group)); }

// Seven query heads per kv head (a prime group): the branch-local forward takes one 32-row
// block of all seven heads per workgroup, the eighth wave idle, so that every wave walks the
// same short causal key range (one head over eight row blocks leaves the waves near the
// diagonal waiting at the stage barriers). The long walks keep one head per workgroup: there
// the lone wave of the idle wave's SIMD, with no second wave to overlap its softmax with the
// products, would set the pace at every barrier.
int fwd_heads_per_wg(int group, int mode) {
  return group == 7 && mode == kFwdReplayLocal ? 7 : heads_per_wg(group);
}
int fwd_rows_per_wg(int group, int mode) { return 32 * (kFwdWaves / fwd_heads_per_wg(group, mode)); }

template <typename T, int D, int HG>
static hipError_t launch_fwd_hg(int mode, const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.nwg), block(kFwdWaves * 64);
  switch (mode) {
    case kFwdPrefill: hipLaunchKernelGGL((attn_fwd_kernel<T, T, D, kFwdPrefill, HG>), grid, block, 0, s, a); break;
    case kFwdReplayPrompt: hipLaunchKernelGGL((attn_fwd_kernel<T, float, D, kFwdReplayPrompt, HG>), grid, block, 0, s, a); break;
    case kFwdReplayLocal: hipLaunchKernelGGL((attn_fwd_kernel<T, float, D, kFwdReplayLocal, HG>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_t(int mode, const FwdArgs& a, hipStream_t s) {
  switch (fwd_heads_per_wg(a.Hq / a.Hkv, mode)) {
    case 4: return launch_fwd_hg<T, D, 4>(mode, a, s);
    case 2: return launch_fwd_hg<T, D, 2>(mode, a, s);
    case 7:
      hipLaunchKernelGGL((attn_fwd_kernel<T, float, D, kFwdReplayLocal, 7>), dim3(a.nwg), dim3(kFwdWaves * 64), 0, s, a);
      return hipGetLastError();
    default: return launch_fwd_hg<T, D, 1>(mode, a, s);
  }
}

hipError_t launch_attn_fwd(int dtype, int D, int mode, const FwdArgs& a, hipStream_t s) {
  if (a.nwg == 0) return hipSuccess;
  if (dtype == 1 && D == 128) return launch_fwd_t<bf16, 128>(mode, a, s);
  if (dtype == 1 && D == 64) return launch_fwd_t<bf16, 64>(mode, a, s);
  if (dtype == 0 && D == 64) return launch_fwd_t<float, 64>(mode, a, s);
  return hipErrorInvalidValue;
}

}  // namespace augtree
