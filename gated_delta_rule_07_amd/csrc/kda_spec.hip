// Speculative decoding for KDA on gfx950: verify K draft tokens without
// touching the state, then commit the accepted prefix.
//
// A KDA layer keeps one state per (sequence, head) and each decode step
// overwrites it, so the tokens a draft model proposed cannot simply be cut off
// again when the target model rejects them (the "Kimi 모델 분석" write-up on
// rlaope.github.io, serving section, on speculative decoding; the "Kimi K3
// Technical Report review" on jw9603.github.io, section 13, lists restoring the
// state after rejected draft tokens).  Here the K tokens are split in two passes
// over the state:
//
//   verify  the recurrence of section 3.3 of the technical report review,
//             Sbar_t = Diag(alpha_t) S_{t-1},  u_t = beta_t (v_t - Sbar_t^T k_t),
//             S_t = Sbar_t + k_t u_t^T,        o_t = S_t^T q_t,
//           unrolled over the draft.  With P_t = prod_{r<=t} alpha_r and
//           G_ts = prod_{s<r<=t} alpha_r (per key channel; tokens t = 0 .. K-1),
//             Sbar_t = Diag(P_t) S + sum_{s<t} Diag(G_ts) k_s u_s^T,
//           so every product with the state is one of 2K vectors,
//             x_t = S^T (P_t k_t) + sum_{s<t} c_ts u_s,   c_ts = sum_i k_s G_ts k_t,
//             u_t = beta_t (v_t - x_t),
//             o_t = S^T (P_t q_t) + sum_{s<t} d_ts u_s + d_tt u_t,
//                                                      d_ts = sum_i k_s G_ts q_t
//           (G_tt = 1).  S is read once and multiplied by all 2K vectors in one
//           pass; the K-step substitution then runs on each value column with
//           the scalars c and d, which depend only on k, q and alpha and are
//           formed while the state is in flight.  o_t and the write vectors
//           u_t are stored; S in memory is untouched.
//   commit  with j accepted tokens, the state after them has the closed form
//             S_j = Diag(P_j) S + sum_{t<j} Diag(P_j / P_{t+1}) k_t u_t^T,
//           P_m = prod_{s<m} alpha_s (per key channel),
//           which one streaming pass over S computes (j = 0 leaves S as it is).
//
// Both kernels: one workgroup per (sequence, head).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Commit: each thread owns a float4 column group and DK/RG rows.
template <int DK, int DV>
struct SCfg {
  static constexpr int NCG = DV / 4;                            // float4 column groups
  static constexpr int RG = (256 / NCG < DK) ? 256 / NCG : DK;  // row groups
  static constexpr int NT = NCG * RG;
  static constexpr int RPT = DK / RG;                           // rows per thread
  static constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NT <= 256, "block shape");
};

// Verify: wave w owns 4 CGW value columns of the state; lane (rg, cg) of it
// holds rows rg + RGW r (r < RPT) of its float4 column group, so a sum over the
// rows of the state is a sum within the wave.  A pass over the state forms the
// products with RGW vectors at a time, one per row-group lane after the sum.
template <int DK, int DV>
struct VCfg {
  static constexpr int CGW = DV >= 32 ? 8 : DV / 4;  // float4 column groups per wave
  static constexpr int RGW = 64 / CGW;               // row groups per wave
  static constexpr int VPP = 4;                      // vectors per pass over the state
  static constexpr int NW = DV / (4 * CGW);
  static constexpr int NT = 64 * NW;
  static constexpr int RPT = DK / RGW;                 // state rows per lane
  static constexpr int CPI = DK < 16 ? DK : 16;        // key channels per coefficient work item
  static constexpr int NCB = DK / CPI;
  static_assert(RPT >= 1 && DK % RGW == 0 && DV % (4 * CGW) == 0, "verify block shape");
  static_assert(RGW >= 2 * VPP && RGW * CGW == 64, "a pass's vectors reduce over the row-group lanes");
};

// The verify kernel's LDS (floats, every region a multiple of 4), for K drafts.
// xs (the 2K state products) reuses the space of k, q and alpha, which are last
// read before it is written.
struct VLay {
  int nvp, np;                   // vectors padded to whole passes; token pairs s <= t
  int k, q, a, xs, v, b, pv, cp, dp, cc, dd, total;
  __host__ __device__ static int r4(int n) { return (n + 3) & ~3; }
  __host__ __device__ VLay(int K, int dk, int dv, int vpp, int ncb) {
    nvp = (2 * K + vpp - 1) / vpp * vpp;
    np = K * (K + 1) / 2;
    k = 0;
    q = k + r4(K * dk);
    a = q + r4(K * dk);
    xs = 0;
    int o = a + r4(K * dk);
    if (o < xs + nvp * dv) o = xs + nvp * dv;
    v = o;
    b = v + r4(K * dv);
    pv = b + r4(K);
    cp = pv + dk * nvp;
    dp = cp + r4(np * ncb);
    cc = dp + r4(np * ncb);
    dd = cc + r4(np);
    total = dd + r4(np);
  }
};

// Sums 2N vectors over lanes that differ in bit M and the bits below it down
// to the row-group bits: at each step a lane keeps half of its vectors (the
// upper half where its bit M is set) and adds its partner's copy of that half.
template <int N, int M>
__device__ __forceinline__ void reduce_scatter(f32x4* acc, int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const f32x4 keep = up ? acc[N + e] : acc[e];
    const f32x4 send = up ? acc[e] : acc[N + e];
    f32x4 got;
#pragma unroll
    for (int c = 0; c < 4; ++c) got[c] = __shfl_xor(send[c], M);
    acc[e] = keep + got;
  }
  if constexpr (N > 1) reduce_scatter<N / 2, M / 2>(acc, lane);
}

__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// NS states per workgroup, (b, h) = NS blockIdx.x + st: a workgroup that
// streams two 64 KB states reads HBM faster than two workgroups that stream one
// each.  MAXK bounds the drafts (the registers the drafts' inputs take while
// the states are in flight).
template <typename IO, int DK, int DV, int MAXK, int NS>
__global__ __launch_bounds__((VCfg<DK, DV>::NT)) void kda_verify_kernel(VerifyParams p) {
  using C = VCfg<DK, DV>;
  extern __shared__ f32x4 verify_lds[];
  const int K = p.K;
  const VLay L(K, DK, DV, C::VPP, C::NCB);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int nbh = p.B * p.H, bh0 = blockIdx.x * NS;
  // a state past the last (an odd count): its loads repeat the last state's, its results are not stored
  float* smb[NS];
  size_t row0[NS];  // row (b, t, h) of the [B][K][H][d] inputs is row0 + t H
  int bhs[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    smb[st] = reinterpret_cast<float*>(verify_lds) + st * L.total;
    bhs[st] = min(bh0 + st, nbh - 1);
    row0[st] = (size_t)(bhs[st] / p.H) * K * p.H + bhs[st] % p.H;
  }

  // the drafts' keys, queries, decays, values and betas, then the states: all
  // loads in flight at once (small indices clamped into range, so no branch
  // splits them); storing the small ones to LDS waits only for them
  constexpr int EK = (MAXK * DK + C::NT - 1) / C::NT, EV = (MAXK * DV + C::NT - 1) / C::NT;
  const int nk = K * DK, nv = K * DV;
  IO rk[NS][EK], rq[NS][EK], rv[NS][EV];
  float ra[NS][EK], rb[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
#pragma unroll
    for (int j = 0; j < EK; ++j) {
      const int e = min(tid + j * C::NT, nk - 1);
      const size_t at = (row0[st] + (size_t)(e / DK) * p.H) * DK + e % DK;
      rk[st][j] = static_cast<const IO*>(p.k)[at];
      rq[st][j] = static_cast<const IO*>(p.q)[at];
      ra[st][j] = p.alpha[at];
    }
#pragma unroll
    for (int j = 0; j < EV; ++j) {
      const int e = min(tid + j * C::NT, nv - 1);
      rv[st][j] = static_cast<const IO*>(p.v)[(row0[st] + (size_t)(e / DV) * p.H) * DV + e % DV];
    }
    rb[st] = p.beta[row0[st] + (size_t)min(tid, K - 1) * p.H];
  }
  __builtin_amdgcn_sched_barrier(0);  // (the loads are counted in order: keep the small ones first)

  const int cg = lane % C::CGW, rg = lane / C::CGW;
  const int col = 4 * (C::CGW * wave + cg);
  f32x4 s[NS][C::RPT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float* S = p.S + (size_t)bhs[st] * DK * DV + col;
#pragma unroll
    for (int r = 0; r < C::RPT; ++r)
      s[st][r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + C::RGW * r) * DV));
  }
  __builtin_amdgcn_sched_barrier(0);

  // (unconditional stores: a clamped index stores the value already there, and
  // no load is moved after the states')
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    float* sm = smb[st];
#pragma unroll
    for (int j = 0; j < EK; ++j) {
      const int e = min(tid + j * C::NT, nk - 1);
      sm[L.k + e] = to_f32(rk[st][j]);
      sm[L.q + e] = to_f32(rq[st][j]);
      sm[L.a + e] = ra[st][j];
    }
#pragma unroll
    for (int j = 0; j < EV; ++j) sm[L.v + min(tid + j * C::NT, nv - 1)] = to_f32(rv[st][j]);
    sm[L.b + min(tid, K - 1)] = rb[st];
  }
  block_sync_lds();

  // while the states are in flight: the 2K vectors P_t k_t and P_t q_t, one key
  // channel of one state per work item ...
  for (int e = tid; e < NS * DK; e += C::NT) {
    const float* sm = smb[0] + (e / DK) * L.total;
    const int i = e % DK;
    float P = 1.0f;
    float* pv = const_cast<float*>(sm) + L.pv + i * L.nvp;
    for (int t = 0; t < K; ++t) {
      P *= sm[L.a + t * DK + i];
      pv[t] = P * sm[L.k + t * DK + i];
      pv[K + t] = P * sm[L.q + t * DK + i];
    }
    for (int j = 2 * K; j < L.nvp; ++j) pv[j] = 0.0f;
  }
  // ... and c_ts, d_ts for every pair s <= t, in partial sums over CPI channels
  const int npc = L.np * C::NCB;
  for (int e2 = tid; e2 < NS * npc; e2 += C::NT) {
    float* sm = smb[0] + (e2 / npc) * L.total;
    const int e = e2 % npc;
    const int pr = e / C::NCB, cb = e % C::NCB;
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= pr) ++t;
    const int s0 = pr - t * (t + 1) / 2;
    float cs = 0.0f, ds = 0.0f;
#pragma unroll 1
    for (int ii = 0; ii < C::CPI; ++ii) {
      const int i = cb + C::NCB * ii;
      float g = sm[L.k + s0 * DK + i];  // k_s G_ts
      for (int r = s0 + 1; r <= t; ++r) g *= sm[L.a + r * DK + i];
      cs += g * sm[L.k + t * DK + i];
      ds += g * sm[L.q + t * DK + i];
    }
    sm[L.cp + e] = cs;
    sm[L.dp + e] = ds;
  }
  block_sync_lds();
  for (int e = tid; e < NS * L.np; e += C::NT) {
    float* sm = smb[0] + (e / L.np) * L.total;
    const int pr = e % L.np;
    float cs = 0.0f, ds = 0.0f;
    for (int cb = 0; cb < C::NCB; ++cb) {
      cs += sm[L.cp + pr * C::NCB + cb];
      ds += sm[L.dp + pr * C::NCB + cb];
    }
    sm[L.cc + pr] = cs;
    sm[L.dd + pr] = ds;
  }

  // one pass over a state per VPP = 4 vectors: the lane's rows, then a
  // reduce-scatter over lane bits 5 and 4 and a sum over the row-group bits
  // below them, after which the lanes with those bits clear hold the sum for
  // vector g0 + lane / 16 (the first state's passes wait only for its loads)
  static_assert(C::VPP == 4, "the reduce-scatter below takes four vectors");
  const int vec = lane / 16;
  const bool writer = (rg & (C::RGW / C::VPP - 1)) == 0;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    float* sm = smb[st];
    for (int g0 = 0; g0 < L.nvp; g0 += C::VPP) {
      f32x4 acc[C::VPP];
#pragma unroll
      for (int j = 0; j < C::VPP; ++j) acc[j] = (f32x4)0.0f;
#pragma unroll
      for (int r = 0; r < C::RPT; ++r) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(sm + L.pv + (rg + C::RGW * r) * L.nvp + g0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] += w[jj] * s[st][r];
      }
      reduce_scatter<C::VPP / 2, 32>(acc, lane);
#pragma unroll
      for (int m = 8; m >= C::CGW; m /= 2)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[0][c] += __shfl_xor(acc[0][c], m);
      if (writer) *reinterpret_cast<f32x4*>(sm + L.xs + (g0 + vec) * DV + col) = acc[0];
    }
  }
  block_sync_lds();

  // the substitution over the draft, one value column of one state per work item
  for (int e = tid; e < NS * DV; e += C::NT) {
    const int st = e / DV, c = e % DV;
    if (bh0 + st >= nbh) continue;
    const float* sm = smb[0] + st * L.total;
    const int bh = bh0 + st;
    const size_t r0 = (size_t)(bh / p.H) * K * p.H + bh % p.H;
    float u[MAXK];
#pragma unroll
    for (int t = 0; t < MAXK; ++t) {
      if (t >= K) continue;
      const int pt = t * (t + 1) / 2;
      float x = sm[L.xs + t * DV + c];
      float y = sm[L.xs + (K + t) * DV + c];
#pragma unroll
      for (int s0 = 0; s0 < t; ++s0) {
        x += sm[L.cc + pt + s0] * u[s0];
        y += sm[L.dd + pt + s0] * u[s0];
      }
      u[t] = sm[L.b + t] * (sm[L.v + t * DV + c] - x);
      y += sm[L.dd + pt + t] * u[t];
      const size_t orow = r0 + (size_t)t * p.H;
      if (p.o_f32) static_cast<float*>(p.o)[orow * DV + c] = y;
      else static_cast<__bf16*>(p.o)[orow * DV + c] = (__bf16)y;
      p.u[((size_t)bh * K + t) * DV + c] = u[t];
    }
  }
}

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void kda_commit_kernel(CommitParams p) {
  using C = SCfg<DK, DV>;
  __shared__ float coef[kMaxDraft][DK];  // k_t * P_j / P_{t+1}
  __shared__ float pj[DK];               // P_j
  const int tid = threadIdx.x;
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const int cg = tid % C::NCG, rg = tid / C::NCG;
  const int K = p.K;
  const int j = min(max(p.n_accept[b], 0), K);
  if (j == 0) return;  // nothing accepted: the state stays as it is

  float* S = p.S + (size_t)bh * DK * DV;
  // plain loads with the non-temporal stores below: faster than non-temporal both ways
  f32x4 s[C::RPT];
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) s[r] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg + C::RG * r) * DV + 4 * cg);
  for (int i = tid; i < DK; i += C::NT) {
    float run = 1.0f;  // product of the decays after token t
    for (int t = j - 1; t >= 0; --t) {
      const size_t row = ((size_t)b * K + t) * p.H + h;
      coef[t][i] = to_f32(static_cast<const IO*>(p.k)[row * DK + i]) * run;
      run *= p.alpha[row * DK + i];
    }
    pj[i] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) s[r] *= pj[rg + C::RG * r];
  for (int t = 0; t < j; ++t) {
    const f32x4 ut = *reinterpret_cast<const f32x4*>(p.u + ((size_t)bh * K + t) * DV + 4 * cg);
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) s[r] += coef[t][rg + C::RG * r] * ut;
  }
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
    __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(S + (size_t)(rg + C::RG * r) * DV + 4 * cg));
}

// Up to kVerifyPairK drafts: two states per workgroup; more: one.
constexpr int kVerifyPairK = 4;
template <typename IO, int DK, int DV>
hipError_t verify_one(const VerifyParams& p, hipStream_t s) {
  using C = VCfg<DK, DV>;
  const size_t lds = (size_t)VLay(p.K, DK, DV, C::VPP, C::NCB).total * sizeof(float);
  const long long nbh = (long long)p.B * p.H;
  if (p.K <= kVerifyPairK)
    hipLaunchKernelGGL((kda_verify_kernel<IO, DK, DV, kVerifyPairK, 2>), dim3((unsigned)((nbh + 1) / 2)), dim3(C::NT),
                       2 * lds, s, p);
  else
    hipLaunchKernelGGL((kda_verify_kernel<IO, DK, DV, kMaxDraft, 1>), dim3((unsigned)nbh), dim3(C::NT), lds, s, p);
  return hipGetLastError();
}
template <typename IO, int DK, int DV>
hipError_t commit_one(const CommitParams& p, hipStream_t s) {
  hipLaunchKernelGGL((kda_commit_kernel<IO, DK, DV>), dim3((unsigned)(p.B * p.H)), dim3(SCfg<DK, DV>::NT), 0, s, p);
  return hipGetLastError();
}

template <class P>
using spec_fn = hipError_t (*)(const P&, hipStream_t);

template <typename IO, int DK, int DV>
struct VerifyF {
  static constexpr spec_fn<VerifyParams> fn = &verify_one<IO, DK, DV>;
};
template <typename IO, int DK, int DV>
struct CommitF {
  static constexpr spec_fn<CommitParams> fn = &commit_one<IO, DK, DV>;
};

template <class P, template <typename, int, int> class F, typename IO, int DK>
spec_fn<P> pick_dv(int dv) {
  switch (dv) {
    case 16: return F<IO, DK, 16>::fn;
    case 32: return F<IO, DK, 32>::fn;
    case 64: return F<IO, DK, 64>::fn;
    case 128: return F<IO, DK, 128>::fn;
    default: return nullptr;
  }
}

template <class P, template <typename, int, int> class F, typename IO>
spec_fn<P> pick_dk(int dk, int dv) {
  switch (dk) {
    case 16: return pick_dv<P, F, IO, 16>(dv);
    case 32: return pick_dv<P, F, IO, 32>(dv);
    case 64: return pick_dv<P, F, IO, 64>(dv);
    case 128: return pick_dv<P, F, IO, 128>(dv);
    default: return nullptr;
  }
}

template <class P, template <typename, int, int> class F>
spec_fn<P> pick(int io_dtype, int dk, int dv) {
  if (io_dtype == 1) return pick_dk<P, F, __bf16>(dk, dv);
  if (io_dtype == 0) return pick_dk<P, F, float>(dk, dv);
  return nullptr;
}

}  // namespace

bool spec_supported(int io_dtype, int dk, int dv) {
  return pick<VerifyParams, VerifyF>(io_dtype, dk, dv) != nullptr;
}

hipError_t launch_verify(const VerifyParams& p, int io_dtype, hipStream_t s) {
  const spec_fn<VerifyParams> f = pick<VerifyParams, VerifyF>(io_dtype, p.dk, p.dv);
  if (!f || p.K < 1 || p.K > kMaxDraft) return hipErrorInvalidValue;
  return f(p, s);
}

hipError_t launch_commit(const CommitParams& p, int io_dtype, hipStream_t s) {
  const spec_fn<CommitParams> f = pick<CommitParams, CommitF>(io_dtype, p.dk, p.dv);
  if (!f || p.K < 1 || p.K > kMaxDraft) return hipErrorInvalidValue;
  return f(p, s);
}

}  // namespace kda
