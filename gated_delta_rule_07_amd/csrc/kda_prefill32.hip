// KDA prefill on 32x32x16 matrix-core tiles (gfx950), bf16 q/k/v, d_k in {64, 128},
// chunk 64, 32 state columns per workgroup.
//
// Same chunkwise method as kda_prefill.hip (the "Kimi 모델 분석" chunkwise form on
// rlaope.github.io: WY representation, UT transform, state carried between
// chunks), arranged for the full-rate 32x32x16 fp16 MFMA:
//
//   KG = K o e^{G},  QG = Q o e^{G},  KC = K o e^{-G}      (chunk-start reference)
//   L  = strict_tril(diag(beta) KG KC^T)   P = tril(QG KC^T)
//   T  = (I + L)^{-1} diag(beta)
//   X  = V - KG S      U = T X      O = QG S + P U
//   S' = Diag(e^{G_C}) (S + KC^T U)
//
// Every matrix-core operand is fp16 and every accumulation fp32.  KG, QG, KC are
// in fp16 range with full precision as long as the chunk's total decay in every
// channel is at least e^{-10}; a range that decays faster is regrouped into
// 16-token and then 2-token sub-chunks (alpha >= e^{-5}, the lower bound of
// section 3.5 of the "Kimi K3 Technical Report review", makes any 2 tokens
// safe), which computes the same recurrence.  Values (S, V, X, U) are rescaled
// by a power of two per state column and chunk.
//
// LDS layout.  The K-side matrices are stored [row][column] with the columns of
// each 16-group in quad order {0,2,1,3}; one 16-byte read then yields exactly
// the slots a 32x32x16 A operand needs when its B partner comes straight from a
// C tile held in registers (rows 4h..4h+3 and 8+4h..8+4h+3 of a 16-row step).
#include "kda_device.h"
#include "kda_launch.h"

#ifndef KDA_PHASE_MARK
#define KDA_PHASE_MARK(i)
#endif

namespace kda {
namespace {

typedef _Float16 h16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Storage column of logical column c: quads of each 16-group in order {0,2,1,3}.
__device__ __forceinline__ int spos(int c) {
  const int q = (c >> 2) & 3;
  return (c & ~15) | (((q & 1) << 1 | (q >> 1)) << 2) | (c & 3);
}

template <int DK_>
struct G {
  static constexpr int DK = DK_, CS = 64, J = 32;
  static constexpr int NT = 320, NW = 5;          // wave 0: state; waves 1-4: prep
  static constexpr int NP = 256;                  // prep threads
  static constexpr int NKT = DK / 32;            // 32-row channel tiles
  static constexpr int NKS = DK / 16;            // K16 steps over channels
  static constexpr int LDK = DK + 8;             // fp16 [64][DK]
  static constexpr int LDC = CS + 8;             // fp16 [rows][64]
  static constexpr int LDL = CS + 4;             // fp32 [64][64]
  static constexpr int LDB = 16 + 8;             // fp16 16x16 blocks
  static constexpr int NCQ = DK / 4;             // channel quads
  static constexpr int TGS = NCQ * 8 / 32 > 4 ? 8 : 4;  // tokens per scan thread
  static constexpr int NTG = CS / TGS;
  static_assert(NCQ * NTG == NP, "scan mapping covers the prep waves");
};

template <class C>
struct Smem32 {
  alignas(16) h16 kg[C::CS * C::LDK];    // K o e^{G}      [t][spos(c)]
  alignas(16) h16 qg[C::CS * C::LDK];    // Q o e^{G}      [t][spos(c)]
  alignas(16) h16 kc[C::CS * C::LDK];    // K o e^{-G}     [t][spos(c)]
  alignas(16) h16 kct[C::DK * C::LDC];   // (K o e^{-G})^T [c][spos(t)]
  alignas(16) h16 t[C::CS * C::LDC];     // T              [t][spos(s)]
  alignas(16) h16 p[C::CS * C::LDC];     // P              [t][spos(s)]
  alignas(16) h16 tt[C::CS * C::LDC];    // T^T            [s][t]   (solve)
  alignas(16) h16 ad[4][16 * C::LDB];    // diagonal blocks of (I+L)^{-1}
  alignas(16) h16 y[4][16 * C::LDB];     // per-prep-wave scratch (solve)
  alignas(16) __bf16 v[C::CS * C::J];    // V slab         [t][j]
  alignas(16) float l[C::CS * C::LDL];   // L (beta folded, strictly lower) [t][i]
  alignas(16) float tot[C::NTG * C::DK];
  alignas(16) float beta[C::CS];
  alignas(16) float gam[C::DK];
};

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16 mma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 ld8(const h16* p) { return *reinterpret_cast<const f16x8*>(p); }

// fp16 B operand from 8 accumulator values (a 16-row step of a 32x32 C tile).
__device__ __forceinline__ f16x8 bfrag(const f32x16& t, int half, float scale) {
  f16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (h16)(t[8 * half + e] * scale);
  return f;
}

__device__ __forceinline__ f16x8 neg8(f16x8 f) {
  u32x4 u = __builtin_bit_cast(u32x4, f);
  u ^= 0x80008000u;
  return __builtin_bit_cast(f16x8, u);
}

// Per-lane values routed through an empty asm so address arithmetic built on them
// is redone inside each loop iteration instead of being hoisted into registers
// for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Raw buffer resource over [base, base + bytes); stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}

template <class C>
struct Raw32 {
  f32x4 a[C::TGS];   // alpha, 4 channels per token
  u32x2 k[C::TGS];   // 4 bf16
  u32x2 q[C::TGS];
  u32x4 v;           // 8 bf16 of the V slab (64 rows x 32 columns = 256 x 16 bytes)
  float beta;
};

struct Ctx32 {
  PrefillParams p;
  int bh, b, h, col0;
};

__device__ __forceinline__ void unpack_bf16x4(const u32x2& w, float (&f)[4]) {
  f[0] = __builtin_bit_cast(float, w.x << 16);
  f[1] = __builtin_bit_cast(float, w.x & 0xffff0000u);
  f[2] = __builtin_bit_cast(float, w.y << 16);
  f[3] = __builtin_bit_cast(float, w.y & 0xffff0000u);
}

// Loads chunk t0's inputs for this thread.  Rows past the sequence end read as
// zeros (buffer range check); the segment bounds keep them out of the recurrence.
template <class C>
__device__ __forceinline__ void load_raw32(Raw32<C>& raw, const Ctx32& cx, int t0, int tid) {
  const PrefillParams& p = cx.p;
  const int cq = opaque(tid % C::NCQ), tg = opaque(tid / C::NCQ);
  const size_t row0 = ((size_t)cx.b * p.T + t0) * p.H + cx.h;  // token t0 of this (sequence, head)
  const int rows = min(C::CS, p.T - t0);
  const int tstride = p.H * C::DK;  // elements between tokens
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(const_cast<float*>(p.alpha) + row0 * C::DK, rows * tstride * 4);
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(const_cast<__bf16*>(static_cast<const __bf16*>(p.k)) + row0 * C::DK, rows * tstride * 2);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(const_cast<__bf16*>(static_cast<const __bf16*>(p.q)) + row0 * C::DK, rows * tstride * 2);
  const int e0 = tg * C::TGS * tstride + 4 * cq;  // element offset of the thread's first token
#pragma unroll
  for (int i = 0; i < C::TGS; ++i) {
    raw.a[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, 4 * e0, 4 * i * tstride, 0));
    raw.k[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, 2 * e0, 2 * i * tstride, 0));
    raw.q[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rq, 2 * e0, 2 * i * tstride, 0));
  }
  {
    const int vstride = p.H * p.dv;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(
        const_cast<__bf16*>(static_cast<const __bf16*>(p.v)) + row0 * p.dv + cx.col0, rows * vstride * 2);
    // 4 threads per V row of 32 bf16
    raw.v = __builtin_bit_cast(u32x4,
                               __builtin_amdgcn_raw_buffer_load_b128(rv, 2 * ((tid / 4) * vstride + 8 * (tid % 4)), 0, 0));
  }
  {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(const_cast<float*>(p.beta) + row0, rows * p.H * 4);
    raw.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * min(tid, C::CS - 1) * p.H, 0, 0));
  }
}

// ---- scan: decay products and the fp16 operand matrices ---------------------
// Tokens outside [lo, hi) act as identity steps.  With `check`, returns true
// (uniformly, writing nothing) if some channel decays below e^{-10} over [lo, hi).
template <class C>
__device__ bool scan32(Smem32<C>& sm, const Raw32<C>& raw, int lo, int hi, bool check, int tid) {
  tid = opaque(tid);
  const int cq = tid % C::NCQ, tg = tid / C::NCQ;
  float lp[C::TGS][4];  // inclusive prefix within the thread's tokens
  float run[4] = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
  for (int i = 0; i < C::TGS; ++i) {
    const int t = tg * C::TGS + i;
    const bool in = t >= lo && t < hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      run[e] *= in ? raw.a[i][e] : 1.0f;
      lp[i][e] = run[e];
    }
  }
  *reinterpret_cast<f32x4*>(&sm.tot[tg * C::DK + 4 * cq]) = f32x4{run[0], run[1], run[2], run[3]};
  KDA_PHASE_MARK(11);
  block_sync_lds();
  KDA_PHASE_MARK(12);
  float ep[4] = {1.0f, 1.0f, 1.0f, 1.0f}, sp[4] = {1.0f, 1.0f, 1.0f, 1.0f}, gm[4];
#pragma unroll
  for (int g2 = 0; g2 < C::NTG; ++g2) {
    const f32x4 tv = *reinterpret_cast<const f32x4*>(&sm.tot[g2 * C::DK + 4 * cq]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (g2 < tg) ep[e] *= tv[e];
      if (g2 > tg) sp[e] *= tv[e];
    }
  }
  KDA_PHASE_MARK(13);
  int steep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gm[e] = ep[e] * run[e] * sp[e];
    steep |= !(gm[e] >= 4.5399930e-05f);  // e^{-10}
  }
  if (check) {
    if (__syncthreads_or(steep)) return true;
  }
  KDA_PHASE_MARK(14);
  float ig[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ig[e] = sp[e] * __builtin_amdgcn_rcpf(gm[e]);  // prod_{later groups} / e^{G_C}
  // exclusive suffix inside the thread's tokens: 1/pre_t = suffix_t * ig
  float suf[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  h16 kct[4][C::TGS];
#pragma unroll
  for (int i = C::TGS - 1; i >= 0; --i) {
    const int t = tg * C::TGS + i;
    const bool in = t >= lo && t < hi;
    float kf[4], qf[4];
    unpack_bf16x4(raw.k[i], kf);
    unpack_bf16x4(raw.q[i], qf);
    f16x4 kgv, qgv, kcv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pre = ep[e] * lp[i][e];
      const float inv = suf[e] * ig[e];
      const float kk = in ? kf[e] : 0.0f, qq = in ? qf[e] : 0.0f;
      kgv[e] = (h16)(kk * pre);
      qgv[e] = (h16)(qq * pre);
      kcv[e] = (h16)(kk * inv);
      kct[e][i] = kcv[e];
      suf[e] *= in ? raw.a[i][e] : 1.0f;
    }
    const int col = spos(4 * cq);
    *reinterpret_cast<f16x4*>(&sm.kg[t * C::LDK + col]) = kgv;
    *reinterpret_cast<f16x4*>(&sm.qg[t * C::LDK + col]) = qgv;
    *reinterpret_cast<f16x4*>(&sm.kc[t * C::LDK + col]) = kcv;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int i4 = 0; i4 < C::TGS; i4 += 4) {
      const f16x4 w = {kct[e][i4], kct[e][i4 + 1], kct[e][i4 + 2], kct[e][i4 + 3]};
      *reinterpret_cast<f16x4*>(&sm.kct[(4 * cq + e) * C::LDC + spos(tg * C::TGS + i4)]) = w;
    }
  if (tg == 0) *reinterpret_cast<f32x4*>(&sm.gam[4 * cq]) = f32x4{gm[0], gm[1], gm[2], gm[3]};
  if (tid < C::CS) sm.beta[tid] = (tid >= lo && tid < hi) ? raw.beta : 0.0f;
  *reinterpret_cast<u32x4*>(&sm.v[(tid / 4) * C::J + 8 * (tid % 4)]) = raw.v;
  return false;
}

// P tile (token tile a, column s): keep the lower part including the diagonal.
template <class C>
__device__ __forceinline__ void store_p_tile(Smem32<C>& sm, const f32x16& acc, int a, int h, int s) {
  h16* prow = &sm.p[(32 * a + 4 * h) * C::LDC + spos(s)];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 32 * a + 8 * j + 4 * h + r;
      prow[(8 * j + r) * C::LDC] = (h16)(t >= s ? acc[4 * j + r] : 0.0f);
    }
}

// ---- L = beta K K^T and P = Q K^T (32x32 tiles (a, b), b <= a) -------------
// wave 0: L00 and P00; wave 1: L10 and P10; wave 2: L11; wave 3: P11.  `wave`
// is uniform, so the selections below are scalar.
template <class C>
__device__ void lp32(Smem32<C>& sm, int wave, int lane) {
  const int h = opaque(lane / 32), m = opaque(lane % 32);
  const int a = (wave == 0) ? 0 : 1;
  const int b = (wave == 1) ? 0 : a;
  const bool two = wave < 2;
  const h16* A1 = (wave == 3) ? sm.qg : sm.kg;  // first product: L (P on wave 3)
  f32x16 acc1 = (f32x16)0.0f, acc2 = (f32x16)0.0f;
  const h16* brow = &sm.kc[(32 * b + m) * C::LDK + 8 * h];
  const h16* arow1 = &A1[(32 * a + m) * C::LDK + 8 * h];
  const h16* arow2 = &sm.qg[(32 * a + m) * C::LDK + 8 * h];
  if (two) {
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) {
      const f16x8 B = ld8(brow + 16 * s);
      acc1 = mma32(ld8(arow1 + 16 * s), B, acc1);
      acc2 = mma32(ld8(arow2 + 16 * s), B, acc2);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) acc1 = mma32(ld8(arow1 + 16 * s), ld8(brow + 16 * s), acc1);
  }
  KDA_PHASE_MARK(17);
  // rows t = 32a + 8j + 4h + r hold element 4j + r; column s = 32b + m
  const int s = 32 * b + m;
  if (wave != 3) {  // acc1 holds L: keep the strictly lower part, scaled by beta_t
    float* lrow = &sm.l[(32 * a + 4 * h) * C::LDL + s];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[32 * a + 8 * j + 4 * h]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 32 * a + 8 * j + 4 * h + r;
        lrow[(8 * j + r) * C::LDL] = t > s ? acc1[4 * j + r] * bt[r] : 0.0f;
      }
    }
  } else {
    store_p_tile<C>(sm, acc1, a, h, s);
  }
  if (two) store_p_tile<C>(sm, acc2, a, h, s);
}

// ---- T = (I + L)^{-1} diag(beta) ----------------------------------------------
template <class C>
__device__ void solve32(Smem32<C>& sm, int wave, int lane) {
  // Diagonal 16x16 block a = wave: lane (s = column, qd = row quarter) keeps
  // rows 4qd..4qd+3 of column s of (I + L_aa)^{-1}; forward substitution over u
  // with x[u] broadcast from the lane that owns row u.
  {
    const int a = wave, s = opaque(lane % 16), qd = opaque(lane / 16);
    const float* Lb = &sm.l[(16 * a + 4 * qd) * C::LDL + 16 * a];
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (4 * qd + r == s) ? 1.0f : 0.0f;
#pragma unroll
    for (int u4 = 0; u4 < 16; u4 += 4) {
      f32x4 Lr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) Lr[r] = *reinterpret_cast<const f32x4*>(Lb + r * C::LDL + u4);
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int u = u4 + uu;
        const float xu = __shfl(x[u & 3], (u >> 2) * 16 + s);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] -= Lr[r][uu] * xu;  // L is zero on and above the diagonal
      }
    }
    const float bs = sm.beta[16 * a + s];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * qd + r;
      sm.ad[a][t * C::LDB + s] = (h16)x[r];
      const h16 tv = (h16)(x[r] * bs);
      sm.t[(16 * a + t) * C::LDC + spos(16 * a + s)] = tv;
      sm.tt[(16 * a + s) * C::LDC + 16 * a + t] = tv;
    }
  }
  KDA_PHASE_MARK(18);
  block_sync_lds();
  KDA_PHASE_MARK(19);
  // Off-diagonal blocks: T_ab = -(I+L_aa)^{-1} sum_{c=b}^{a-1} L_ac T_cb (16x16x32 steps).
  const int g = opaque(lane / 16), m = opaque(lane % 16);
  for (int d = 1; d < 4; ++d) {
    const int a = d + wave;
    if (a < 4) {
      const int b = a - d;
      f32x4 y = (f32x4)0.0f;
      for (int kb = 16 * b; kb < 16 * a; kb += 32) {
        Frag<h16> A, B;
        const Frag<float> lf = lds_frag(sm.l, C::LDL, 16 * a + m, kb + 8 * g, 16 * a);
#pragma unroll
        for (int e = 0; e < 8; ++e) A.v[e] = (h16)lf.v[e];
        B = lds_frag(sm.tt, C::LDC, 16 * b + m, kb + 8 * g, 16 * a);
        y = mma(A, B, y);
      }
      h16* ys = sm.y[wave];
#pragma unroll
      for (int r = 0; r < 4; ++r) ys[m * C::LDB + 4 * g + r] = (h16)y[r];
      wave_lds_sync();
      const Frag<h16> A = lds_frag(sm.ad[a], C::LDB, m, 8 * g, 16);
      const Frag<h16> B = lds_frag(ys, C::LDB, m, 8 * g, 16);
      const f32x4 z = mma(A, B, (f32x4)0.0f);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const h16 tv = (h16)(-z[r]);
        const int t = 16 * a + 4 * g + r, s = 16 * b + m;
        sm.t[t * C::LDC + spos(s)] = tv;
        sm.tt[s * C::LDC + t] = tv;
      }
    }
    KDA_PHASE_MARK(20);
    block_sync_lds();
    KDA_PHASE_MARK(21);
  }
}

// ---- state update: one wave, 32 columns ----------------------------------------
template <class C>
__device__ __forceinline__ float vload(const Smem32<C>& sm, int a, int i, int h, int n) {
  return (float)sm.v[(32 * a + 8 * (i / 4) + 4 * h + (i % 4)) * C::J + n];
}

template <class C>
__device__ void state32(Smem32<C>& sm, f32x16 (&S)[C::NKT], int lane, const Ctx32& cx, int t0, int lo, int hi) {
  const int h = opaque(lane / 32), n = opaque(lane % 32);
  // per-column power-of-two scale of the values (S, V)
  float mx = 0.0f;
#pragma unroll
  for (int ct = 0; ct < C::NKT; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(S[ct][i]));
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(vload(sm, a, i, h, n)));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const int ex = (mx > 0.0f) ? __builtin_amdgcn_frexp_expf(mx) : 0;
  const float scale = __builtin_amdgcn_ldexpf(1.0f, -ex);
  const float unscale = __builtin_amdgcn_ldexpf(1.0f, ex);

  // X = V - KG S and O = QG S in one pass over the channels (each S fragment
  // feeds four products)
  f32x16 X0, X1, O0 = (f32x16)0.0f, O1 = (f32x16)0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    X0[i] = vload(sm, 0, i, h, n) * scale;
    X1[i] = vload(sm, 1, i, h, n) * scale;
  }
#pragma unroll
  for (int s = 0; s < C::NKS; ++s) {
    const f16x8 B = bfrag(S[s / 2], s % 2, scale);
    const f16x8 nB = neg8(B);
    const int col = 16 * s + 8 * h;
    X0 = mma32(ld8(&sm.kg[n * C::LDK + col]), nB, X0);
    X1 = mma32(ld8(&sm.kg[(32 + n) * C::LDK + col]), nB, X1);
    O0 = mma32(ld8(&sm.qg[n * C::LDK + col]), B, O0);
    O1 = mma32(ld8(&sm.qg[(32 + n) * C::LDK + col]), B, O1);
  }
  KDA_PHASE_MARK(8);
  const f16x8 xf0 = bfrag(X0, 0, 1.0f), xf1 = bfrag(X0, 1, 1.0f);
  const f16x8 xf2 = bfrag(X1, 0, 1.0f), xf3 = bfrag(X1, 1, 1.0f);
  // U = T X (T lower triangular: token tile 0 needs steps 0-1, tile 1 steps 0-3)
  f32x16 U0 = (f32x16)0.0f, U1 = (f32x16)0.0f;
  U0 = mma32(ld8(&sm.t[n * C::LDC + 8 * h]), xf0, U0);
  U1 = mma32(ld8(&sm.t[(32 + n) * C::LDC + 8 * h]), xf0, U1);
  U0 = mma32(ld8(&sm.t[n * C::LDC + 16 + 8 * h]), xf1, U0);
  U1 = mma32(ld8(&sm.t[(32 + n) * C::LDC + 16 + 8 * h]), xf1, U1);
  U1 = mma32(ld8(&sm.t[(32 + n) * C::LDC + 32 + 8 * h]), xf2, U1);
  U1 = mma32(ld8(&sm.t[(32 + n) * C::LDC + 48 + 8 * h]), xf3, U1);
  const f16x8 uf0 = bfrag(U0, 0, 1.0f), uf1 = bfrag(U0, 1, 1.0f);
  const f16x8 uf2 = bfrag(U1, 0, 1.0f), uf3 = bfrag(U1, 1, 1.0f);
  KDA_PHASE_MARK(9);
  // O += P U
  O0 = mma32(ld8(&sm.p[n * C::LDC + 8 * h]), uf0, O0);
  O1 = mma32(ld8(&sm.p[(32 + n) * C::LDC + 8 * h]), uf0, O1);
  O0 = mma32(ld8(&sm.p[n * C::LDC + 16 + 8 * h]), uf1, O0);
  O1 = mma32(ld8(&sm.p[(32 + n) * C::LDC + 16 + 8 * h]), uf1, O1);
  O1 = mma32(ld8(&sm.p[(32 + n) * C::LDC + 32 + 8 * h]), uf2, O1);
  O1 = mma32(ld8(&sm.p[(32 + n) * C::LDC + 48 + 8 * h]), uf3, O1);
  {
    // rows of this chunk in o: [t0, t0 + rows); row t of the chunk, column n at
    // byte t*rs + 4n (fp32) or 2n (bf16); rows outside [lo, hi) are masked by an
    // out-of-range offset, rows past the sequence end by the resource size
    const int rows = min(C::CS, cx.p.T - t0);
    const int esz = cx.p.o_f32 ? 4 : 2;
    const int rs = cx.p.H * cx.p.dv * esz;
    char* ob = static_cast<char*>(cx.p.o) +
               ((((size_t)cx.b * cx.p.T + t0) * cx.p.H + cx.h) * cx.p.dv + cx.col0) * esz;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(ob, rows * rs);
    const int vbase = 4 * h * rs + n * esz;
    int voff[2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 32 * a + 8 * (i / 4) + (i % 4) + 4 * h;
        voff[a][i] = vbase + ((unsigned)(t - lo) < (unsigned)(hi - lo) ? 0 : 0x40000000);
      }
    if (cx.p.o_f32) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tr = 32 * a + 8 * (i / 4) + (i % 4);  // row without the half-wave term
          const float ov = (a ? O1[i] : O0[i]) * unscale;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ov), rsrc, voff[a][i], tr * rs, 0);
        }
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tr = 32 * a + 8 * (i / 4) + (i % 4);
          const float ov = (a ? O1[i] : O0[i]) * unscale;
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)ov), rsrc, voff[a][i], tr * rs, 0);
        }
    }
  }
  KDA_PHASE_MARK(10);
  // S' = Diag(e^{G_C}) (S + KC^T U)
#pragma unroll
  for (int ct = 0; ct < C::NKT; ++ct) {
    f32x16 acc = S[ct] * scale;
    const int row = (32 * ct + n) * C::LDC + 8 * h;
    acc = mma32(ld8(&sm.kct[row]), uf0, acc);
    acc = mma32(ld8(&sm.kct[row + 16]), uf1, acc);
    acc = mma32(ld8(&sm.kct[row + 32]), uf2, acc);
    acc = mma32(ld8(&sm.kct[row + 48]), uf3, acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) S[ct][i] = acc[i] * unscale * sm.gam[32 * ct + 8 * (i / 4) + 4 * h + (i % 4)];
  }
}

// Barrier sequence shared by both roles for one segment [lo, hi) of a chunk:
//   B0 | scan part 1 | B1 | scan part 2 | B2 (steep vote, when checked)
//   | outputs, prefetch | B3 | L, P | B4 | diagonal solve | B5 | 3 merge rounds (B6-B8)
//   | state update (wave 0) | next segment's B0
// Prep waves (1-4) do everything before the state update; wave 0 only the update.

template <class C>
__device__ bool prep_segment(Smem32<C>& sm, Raw32<C>& raw, const Ctx32& cx, int lo, int hi, bool check,
                             int prefetch_t0, int ptid, int pwave, int lane) {
  block_sync_lds();  // B0
  KDA_PHASE_MARK(0);
  if (scan32<C>(sm, raw, lo, hi, check, ptid)) return false;  // B1, B2 inside
  KDA_PHASE_MARK(15);
  if (prefetch_t0 >= 0) load_raw32<C>(raw, cx, prefetch_t0, ptid);
  KDA_PHASE_MARK(16);
  block_sync_lds();  // B3
  KDA_PHASE_MARK(1);
  lp32<C>(sm, pwave, lane);
  block_sync_lds();  // B4
  KDA_PHASE_MARK(2);
  solve32<C>(sm, pwave, lane);  // B5..B8 inside
  KDA_PHASE_MARK(3);
  return true;
}

template <class C>
__device__ bool state_segment(Smem32<C>& sm, f32x16 (&S)[C::NKT], const Ctx32& cx, int t0, int lo, int hi,
                              bool check, int lane) {
  block_sync_lds();  // B0
  KDA_PHASE_MARK(0);
  block_sync_lds();  // B1
  if (check) {
    if (__syncthreads_or(0)) return false;  // B2
  }
#pragma unroll
  for (int i = 0; i < 6; ++i) block_sync_lds();  // B3..B8
  KDA_PHASE_MARK(3);
  state32<C>(sm, S, lane, cx, t0, lo, hi);
  KDA_PHASE_MARK(4);
  return true;
}

template <class C>
__global__ __launch_bounds__(320, 1) void kda_prefill32_kernel(PrefillParams p) {
  __shared__ Smem32<C> sm;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: scalar branches
  const int nslab = p.dv / C::J;
  const int Gn = gridDim.x;
  int lid = blockIdx.x;
  if (Gn % 8 == 0) lid = (blockIdx.x % 8) * (Gn / 8) + blockIdx.x / 8;  // slabs of a head on one XCD
  Ctx32 cx;
  cx.p = p;
  cx.bh = lid / nslab;
  cx.b = cx.bh / p.H;
  cx.h = cx.bh % p.H;
  cx.col0 = (lid % nslab) * C::J;
  // T's upper 16x16 blocks inside its diagonal 32x32 tiles are read as zeros
  // by U = T X and never written.
  for (int i = tid; i < C::CS * C::LDC; i += C::NT) sm.t[i] = (h16)0.0f;
  const int nchunks = (p.T + C::CS - 1) / C::CS;

  // Each chunk is processed as [0, 64); if some channel decays below e^{-10}
  // over a segment, the segment is regrouped (exactly) into 16-token and then
  // 2-token segments.  Both roles walk the same segments.
  if (wave == 0) {
    const int h = lane / 32, n = lane % 32;
    f32x16 S[C::NKT];
    const size_t sbase = (size_t)cx.bh * C::DK * p.dv + cx.col0;
#pragma unroll
    for (int ct = 0; ct < C::NKT; ++ct) S[ct] = (f32x16)0.0f;
    if (p.S0) {
#pragma unroll
      for (int ct = 0; ct < C::NKT; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * ct + 8 * (i / 4) + 4 * h + (i % 4);
          S[ct][i] = p.S0[sbase + c * p.dv + n];
        }
    }
    for (int c = 0; c < nchunks; ++c) {
      const int cend = min(C::CS, p.T - c * C::CS);
      int lo = 0, size = C::CS;
      while (lo < cend) {
        const int hi = min(lo + size, cend);
        if (!state_segment<C>(sm, S, cx, c * C::CS, lo, hi, size > 2, lane)) {
          size = (size == C::CS) ? 16 : 2;
          continue;
        }
        lo = hi;
        if (size == 2 && (lo & 15) == 0) size = 16;
      }
    }
    if (p.S_T) {
#pragma unroll
      for (int ct = 0; ct < C::NKT; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * ct + 8 * (i / 4) + 4 * h + (i % 4);
          p.S_T[sbase + c * p.dv + n] = S[ct][i];
        }
    }
  } else {
    const int ptid = tid - 64, pwave = wave - 1;
    Raw32<C> raw;
    if (nchunks > 0) load_raw32<C>(raw, cx, 0, ptid);
    for (int c = 0; c < nchunks; ++c) {
      const int next = (c + 1 < nchunks) ? (c + 1) * C::CS : -1;
      const int cend = min(C::CS, p.T - c * C::CS);
      int lo = 0, size = C::CS;
      while (lo < cend) {
        const int hi = min(lo + size, cend);
        if (!prep_segment<C>(sm, raw, cx, lo, hi, size > 2, hi == cend ? next : -1, ptid, pwave, lane)) {
          size = (size == C::CS) ? 16 : 2;
          continue;
        }
        lo = hi;
        if (size == 2 && (lo & 15) == 0) size = 16;
      }
    }
  }
}

template <int DK>
hipError_t launch32(const PrefillParams& p, hipStream_t s) {
  using C = G<DK>;
  const unsigned grid = (unsigned)(p.B * p.H * (p.dv / C::J));
  hipLaunchKernelGGL((kda_prefill32_kernel<C>), dim3(grid), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool prefill32_supported(int io_dtype, int dk, int dv, int chunk, int H) {
  // per-chunk buffer ranges (64 tokens of every head) must fit 31 bits
  const long long chunk_bytes = 64LL * H * (dk > dv ? dk : dv) * 4;
  return io_dtype == 1 && (dk == 64 || dk == 128) && dv % 32 == 0 && chunk == 64 && chunk_bytes < (1LL << 31);
}

hipError_t launch_prefill32(const PrefillParams& p, hipStream_t s) {
  if (p.dk == 128) return launch32<128>(p, s);
  if (p.dk == 64) return launch32<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
