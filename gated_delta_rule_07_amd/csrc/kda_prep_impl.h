// KDA prefill, stage 1 of 2 (gfx950; bf16 q/k/v, d_k in {64, 128}), device
// code: the chunk-local operands of the chunkwise form for one (sequence, head,
// 32-token chunk) per wave.  Stage 2 (the chain kernel) only streams these
// records through the sequential state update, so nothing here sits on the
// serial path.  Used by the stage-1 kernel (kda_prep.hip) and by the launch that
// runs the chain over one block of chunks beside stage 1 of the next block
// (kda_prefill_pipe.hip).
//
// Method: the chunkwise (WY/UT) form of the recurrence ("Kimi 모델 분석",
// rlaope.github.io, section on putting the recurrence on the GPU; the per-token
// rule is section 3.2 of the "Kimi K3 Technical Report review" on
// jw9603.github.io).  With a_t the decay of token t (per channel), the products
// pre_t = prod_{s<=t} a_s from the chunk start, suf_t = prod_{s>t} a_s to the
// chunk end and gamma = pre_31:
//
//   KG = K o pre   QG = Q o pre   KH = K o suf
//   L_ij = beta_i sum_c k_ic k_jc r_c(i,j)  (j < i)     r_c(i,j) = prod_{j<s<=i} a_sc
//   P_ij =        sum_c q_ic k_jc r_c(i,j)  (j <= i)
//   T = (I + L)^{-1} diag(beta),  and the output's intra-chunk operator P T
//
// Bounded factors for L and P.  Every ratio r(i,j) is a product of decays, at
// most 1, but factoring it as pre_i / pre_j (one product per side) needs 1/pre,
// which leaves any finite range once a channel decays fast.  Instead each pair
// (i, j) is factored at a block boundary between them: with b the highest bit in
// which i and j differ (so i has it set and both lie in one aligned block of
// 2^{b+1} tokens, i in its upper half), r(i,j) = up_b(i) lo_b(j) where
//   up_b(i) = prod of a_s from the start of i's half up to i,
//   lo_b(j) = prod of a_s after j up to the end of j's half,
// both in [0, 1].  For each level b = 0..4 one 16x16 product of the 16 tokens
// with bit b set (rows) against the 16 with it clear (columns) yields every pair
// of that level on its block diagonal; the five levels cover each pair exactly
// once.  All matrix-core operands are then bounded by |k| or |q| (fp16), and no
// chunk is ever regrouped, whatever the decay.
//
// One wave per chunk record, no barriers: four waves of a workgroup serve four
// records independently, each with its own LDS.  A lane holds CPT = d_k/64
// adjacent channels of all 32 tokens, so the products along the chunk are plain
// running products in registers.
#pragma once
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace prep {
namespace {


typedef _Float16 h16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

constexpr int CS = kPipeChunk;
constexpr int kPrepWaves = 4;

template <int DK_>
struct PCfg {
  static constexpr int DK = DK_;
  static constexpr int CPT = DK / 64;  // channels per lane
  static constexpr int NKB = DK / 32;  // 32-channel reduction steps
  static constexpr int LDF = DK + 8;   // factor rows (fp16): the pad keeps row reads conflict-free
  static constexpr int LDL = CS + 1;   // D_L rows (fp32), read along rows and along columns
  static constexpr int LDP = CS + 4;   // D_P rows (fp32), read as 16-byte runs
  using R = ChunkRec<DK>;
};

template <class C>
struct PrepLds {
  alignas(16) h16 f[CS * C::LDF];    // rows 0..15: A operand, rows 16..31: B operand
  alignas(16) float dl[CS * C::LDL];  // sum_c k_i k_j r(i,j), i > j
  alignas(16) float dp[CS * C::LDP];  // sum_c q_i k_j r(i,j), i >= j
  alignas(16) float beta[CS];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// A 16-byte record store.  A buffer store of more than 8 bytes reads its data
// registers after it issues, so they must not be rewritten in the next two wait
// states; the compiler inserts that wait only when the store's scalar offset is
// not a register, so every offset here goes in the vector offset and the scalar
// offset is the constant 0.
__device__ __forceinline__ void st16(u32x4 d, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, 0);
}
__device__ __forceinline__ float lo16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two fp16 products in one register, each rounded once: the low half is
// fp16(xa[SA] * ra), the high half fp16(xb[SB] * rb), with xa, xb pairs of
// fp16 (index 1 = the high half) and ra, rb fp32 (mixed-precision FMA with a
// zero addend: one instruction per product).
template <int SA, int SB>
__device__ __forceinline__ uint32_t mul2(uint32_t xa, float ra, uint32_t xb, float rb) {
  uint32_t d;
  if constexpr (SA) asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(xa), "v"(ra));
  else asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(xa), "v"(ra));
  if constexpr (SB) asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(d) : "v"(xb), "v"(rb));
  else asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "+v"(d) : "v"(xb), "v"(rb));
  return d;
}
// fp16(x[0] * r) in the low half (the high half undefined)
__device__ __forceinline__ uint32_t mul1(uint32_t x, float r) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(x), "v"(r));
  return d;
}
// The CPT channels of a lane for one token, as fp16 products x[e] * r[e].
template <int CPT>
__device__ __forceinline__ uint32_t mul_ch(uint32_t x, const float (&r)[CPT]) {
  if constexpr (CPT == 2) return mul2<0, 1>(x, r[0], x, r[1]);
  else return mul1(x, r[0]);
}
__device__ __forceinline__ f16x8 ld8(const h16* p) { return *reinterpret_cast<const f16x8*>(p); }

// One swap step of a 4x4 transpose over four lanes: the lane whose bit (of the
// two that name its rank) is b gives its partner the elements whose index bit
// is 1 - b and takes the partner's elements whose index bit is b in their
// place.  DPP: quad_perm [1,0,3,2] is lane ^ 1, row_ror:8 is lane ^ 8.
template <int CTRL, int P0, int P1>
__device__ __forceinline__ void xswap(u32x4& x, bool b) {
  const uint32_t send = b ? x[P0] : x[P1];
  const uint32_t recv = __builtin_amdgcn_update_dpp(0u, send, CTRL, 0xf, 0xf, true);
  if (b) x[P0] = recv;
  else x[P1] = recv;
}
// Lanes of rank r = (lane bit 0) + 2 (lane bit 3) in a group of four hold x_r;
// afterwards the lane of rank r holds element r of every lane of its group,
// element s from the lane of rank s.
__device__ __forceinline__ u32x4 xpose4(u32x4 x, int lane) {
  const bool b0 = lane & 1, b3 = (lane >> 3) & 1;
  xswap<0xb1, 0, 1>(x, b0);
  xswap<0xb1, 2, 3>(x, b0);
  xswap<0x128, 0, 2>(x, b3);
  xswap<0x128, 1, 3>(x, b3);
  return x;
}

// Row of token t among the 16 tokens of its side at level b (bit b removed).
__device__ __forceinline__ constexpr int side_row(int t, int b) {
  return ((t >> (b + 1)) << b) | (t & ((1 << b) - 1));
}

// The record rec (= slot * H + h) by one wave with its own LDS.
template <class C, bool G>
__device__ __forceinline__ void prep_record(const PrefillParams& p, long long rec, PrepLds<C>& sm, int lane) {
  constexpr int CPT = C::CPT, DK = C::DK, NKB = C::NKB;
  using R = typename C::R;
  const int h = (int)(rec % p.H);
  const long long slot = rec / p.H;

  // ---- the chunk of this record -------------------------------------------------
  int b, c;
  if (!p.cu) {
    b = (int)(slot / p.rec_nc);
    c = p.rec_c0 + (int)(slot % p.rec_nc);
    if (b >= p.B) return;
  } else {
    // sequence b owns the slots from cu[b] / 32 + b on (strictly increasing in b)
    auto start = [&](int i) { return (long long)(min(max(p.cu[i], 0), p.T) / CS) + i; };
    if (slot < start(0)) return;
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (start(mid) <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    c = (int)(slot - start(b));
  }
  long long tok0;
  int len;
  seq_range(p, b, tok0, len);
  const int rows = min(CS, len - c * CS);
  if (rows <= 0) return;
  const long long row0 = (tok0 + (long long)c * CS) * p.H + h;  // token row of the chunk's first token
  const int rs = p.H * DK;                                       // elements between token rows

  // ---- inputs: CPT channels of all 32 tokens per lane (rows past the end read 0) ----
  uint32_t kw[CS], qw[CS];  // CPT channels each: bf16 as loaded, then fp16
  float a[CS][CPT];
  float beta;
  {
    const char* kb = static_cast<const char*>(p.k) + row0 * DK * 2;
    const char* qb = static_cast<const char*>(p.q) + row0 * DK * 2;
    const __amdgpu_buffer_rsrc_t rk = rsrc_of(kb, rows * rs * 2);
    const __amdgpu_buffer_rsrc_t rq = rsrc_of(qb, rows * rs * 2);
    const int vo = CPT * lane * 2;
    uint32_t zw[CS];
    __amdgpu_buffer_rsrc_t ra;
    if constexpr (G) ra = rsrc_of(static_cast<const char*>(p.z) + row0 * DK * 2, rows * rs * 2);
    else ra = rsrc_of(reinterpret_cast<const char*>(p.alpha + row0 * DK), rows * rs * 4);
#pragma unroll
    for (int t = 0; t < CS; ++t) {
      const int so = t * rs * 2;
      if constexpr (CPT == 2) {
        kw[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, vo, so, 0);
        qw[t] = __builtin_amdgcn_raw_buffer_load_b32(rq, vo, so, 0);
        if constexpr (G) {
          zw[t] = __builtin_amdgcn_raw_buffer_load_b32(ra, vo, so, 0);
        } else {
          // Reinterpret the loaded vector as a whole: single elements of the
          // integer vector a buffer load returns, reinterpreted as float, are
          // miscompiled by this toolchain (both read one dword).
          const f32x2v av = __builtin_bit_cast(f32x2v, __builtin_amdgcn_raw_buffer_load_b64(ra, 2 * vo, 2 * so, 0));
          a[t][0] = av[0];
          a[t][1] = av[1];
        }
      } else {
        kw[t] = __builtin_amdgcn_raw_buffer_load_b16(rk, vo, so, 0);
        qw[t] = __builtin_amdgcn_raw_buffer_load_b16(rq, vo, so, 0);
        if constexpr (G) zw[t] = __builtin_amdgcn_raw_buffer_load_b16(ra, vo, so, 0);
        else a[t][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, 2 * vo, 2 * so, 0));
      }
    }
    const __amdgpu_buffer_rsrc_t rb = rsrc_of(p.beta + row0, rows * p.H * 4);
    beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * p.H * 4, 0, 0));
    const float eA = G ? __expf(p.A[h]) : 1.0f;
    // tokens past the end are identity steps: decay 1 (k, q and beta read as 0)
#pragma unroll
    for (int t = 0; t < CS; ++t)
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        if constexpr (G) a[t][e] = gate_retention(eA * (e ? hi16(zw[t]) : lo16(zw[t])));
        if (t >= rows) a[t][e] = 1.0f;
      }
    // keys and queries as fp16, in place (exact: a bf16 value in fp16's normal
    // range has no bits fp16 cannot hold; the products below are rounded to
    // fp16 anyway)
#pragma unroll
    for (int t = 0; t < CS; ++t) {
      if constexpr (CPT == 2) {
        kw[t] = __builtin_bit_cast(uint32_t, f16x2{(h16)lo16(kw[t]), (h16)hi16(kw[t])});
        qw[t] = __builtin_bit_cast(uint32_t, f16x2{(h16)lo16(qw[t]), (h16)hi16(qw[t])});
      } else {
        kw[t] = __builtin_bit_cast(uint16_t, (h16)lo16(kw[t]));
        qw[t] = __builtin_bit_cast(uint16_t, (h16)lo16(qw[t]));
      }
    }
  }

  const __amdgpu_buffer_rsrc_t rr = rsrc_of(p.rec + rec * R::BYTES, R::BYTES);
  const int ch = CPT * lane;  // first channel of this lane
  const int g = lane / 16, n = lane % 16;

  // ---- KG, QG (forward products), gamma --------------------------------------------
  {
    // fragment position of channel ch: step kb, lane group gc, slot ec
    const int kb = ch >> 5, cc = ch & 31, gc = (cc & 15) >> 2, ec = (cc & 3) + 4 * (cc >> 4);
    const int vo = kb * 1024 + gc * 256 + 2 * ec;
    float run[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) run[e] = 1.0f;
    if constexpr (CPT == 2) {
      // The four dwords of a token's 16-byte fragment unit sit in the four lanes
      // that differ in lane bits 0 and 3 (dword = bit 0 + 2 * bit 3).  A 4x4
      // transpose over those lanes, per four tokens, gives each lane whole
      // units (token 4m + rank), stored 16 bytes at a time.
      const int sr = (lane & 1) | ((lane >> 2) & 2);
      const int uo = (lane >> 4) * 1024 + ((lane & 7) >> 1) * 256 + sr * 16;
#pragma unroll
      for (int m = 0; m < CS / 4; ++m) {
        u32x4 xk, xq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * m + i;
#pragma unroll
          for (int e = 0; e < CPT; ++e) run[e] *= a[t][e];
          xk[i] = mul_ch<CPT>(kw[t], run);
          xq[i] = mul_ch<CPT>(qw[t], run);
        }
        xk = xpose4(xk, lane);
        xq = xpose4(xq, lane);
        const int to = (m >> 2) * NKB * 1024 + (m & 3) * 64;
        st16(xk, rr, uo + R::KG + to);
        st16(xq, rr, uo + R::QG + to);
      }
    } else {
#pragma unroll
      for (int t = 0; t < CS; ++t) {
        run[0] *= a[t][0];
        const uint32_t kg = mul_ch<CPT>(kw[t], run), qg = mul_ch<CPT>(qw[t], run);
        const int to = (t >> 4) * NKB * 1024 + (t & 15) * 16;
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)kg, rr, vo, R::KG + to, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)qg, rr, vo, R::QG + to, 0);
      }
    }
    if constexpr (CPT == 2)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2v{run[0], run[1]}), rr, ch * 4, R::GAM, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, run[0]), rr, ch * 4, R::GAM, 0);
  }

  // ---- -KH^T (backward products): 16 bytes per (channel, tokens t4..t4+3 and
  //      t4+16..t4+19); the later run's 8 bytes are held until the earlier's ---------
  {
    u32x2 wh[4][CPT];
    float run[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) run[e] = -1.0f;  // the sign of -KH rides on the products
#pragma unroll
    for (int t4 = CS - 4; t4 >= 0; t4 -= 4) {
      float r[CPT][4];  // the backward product of channel e at token t4 + j
#pragma unroll
      for (int t = t4 + 3; t >= t4; --t)
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          r[e][t - t4] = run[e];
          run[e] *= a[t][e];
        }
      // tokens t4..t4+3 fill slots 0..3 (t4 < 16) or 4..7 of lane group (t4 % 16) / 4
      const int so = R::KH + 16 * ((t4 & 15) >> 2) * 16;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const int c = ch + e;
        u32x2 w;
        if (e == 0) {
          w[0] = mul2<0, 0>(kw[t4], r[0][0], kw[t4 + 1], r[0][1]);
          w[1] = mul2<0, 0>(kw[t4 + 2], r[0][2], kw[t4 + 3], r[0][3]);
        } else {
          w[0] = mul2<1, 1>(kw[t4], r[CPT - 1][0], kw[t4 + 1], r[CPT - 1][1]);
          w[1] = mul2<1, 1>(kw[t4 + 2], r[CPT - 1][2], kw[t4 + 3], r[CPT - 1][3]);
        }
        if (t4 >= 16) {
          wh[(t4 - 16) >> 2][e] = w;
        } else {
          const u32x2 wl = wh[t4 >> 2][e];
          st16(u32x4{w[0], w[1], wl[0], wl[1]}, rr, ((c >> 4) * 64 + (c & 15)) * 16 + so);
        }
      }
    }
  }

  // ---- the diagonal of P: q_t . k_t (fp16 products, exact) ---------------------------
  h16* fr = sm.f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (CPT == 2) {
        *reinterpret_cast<uint32_t*>(&fr[r * C::LDF + ch]) = qw[16 * hh + r];
        *reinterpret_cast<uint32_t*>(&fr[(16 + r) * C::LDF + ch]) = kw[16 * hh + r];
      } else {
        fr[r * C::LDF + ch] = __builtin_bit_cast(h16, (uint16_t)qw[16 * hh + r]);
        fr[(16 + r) * C::LDF + ch] = __builtin_bit_cast(h16, (uint16_t)kw[16 * hh + r]);
      }
    }
    wave_lds_sync();
    f32x4 acc = (f32x4)0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      acc = mma16x32(ld8(&fr[n * C::LDF + 32 * kb + 8 * g]), ld8(&fr[(16 + n) * C::LDF + 32 * kb + 8 * g]), acc);
    }
    const int jd = n - 4 * g;  // lane (g, n) holds rows 4g..4g+3 of column n
    if (jd >= 0 && jd < 4) {
      const float d = jd == 0 ? acc[0] : jd == 1 ? acc[1] : jd == 2 ? acc[2] : acc[3];
      sm.dp[(16 * hh + n) * C::LDP + 16 * hh + n] = d;
    }
  }

  // ---- the five levels of L and P ------------------------------------------------------
#pragma unroll
  for (int lv = 0; lv < 5; ++lv) {
    const int hb = 1 << lv;
    // up rows: x_t times the product from the start of t's half up to t, for the
    // tokens with bit lv set (x = k for L, x = q for P)
    auto up_rows = [&](bool use_q) {
      float run[CPT];
#pragma unroll
      for (int t = 0; t < CS; ++t)
        if (t & hb) {
          const int r = side_row(t, lv);
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            if ((t & (hb - 1)) == 0) run[e] = 1.0f;  // the first token of its half
            run[e] *= a[t][e];
          }
          const uint32_t x = mul_ch<CPT>(use_q ? qw[t] : kw[t], run);
          if constexpr (CPT == 2) *reinterpret_cast<uint32_t*>(&fr[r * C::LDF + ch]) = x;
          else fr[r * C::LDF + ch] = __builtin_bit_cast(h16, (uint16_t)x);
        }
    };
    wave_lds_sync();  // the previous readers of the factor rows are done
    up_rows(false);
    {
      float run[CPT];
#pragma unroll
      for (int t = CS - 1; t >= 0; --t)
        if (!(t & hb)) {
          const int r = 16 + side_row(t, lv);
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            if ((t & (hb - 1)) == hb - 1) run[e] = 1.0f;  // the last token of its half
          }
          const uint32_t x = mul_ch<CPT>(kw[t], run);
          if constexpr (CPT == 2) *reinterpret_cast<uint32_t*>(&fr[r * C::LDF + ch]) = x;
          else fr[r * C::LDF + ch] = __builtin_bit_cast(h16, (uint16_t)x);
#pragma unroll
          for (int e = 0; e < CPT; ++e) run[e] *= a[t][e];
        }
    }
    wave_lds_sync();
    f16x8 af[NKB], bfr[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      af[kb] = ld8(&fr[n * C::LDF + 32 * kb + 8 * g]);
      bfr[kb] = ld8(&fr[(16 + n) * C::LDF + 32 * kb + 8 * g]);
    }
    f32x4 accL = (f32x4)0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) accL = mma16x32(af[kb], bfr[kb], accL);
    wave_lds_sync();
    up_rows(true);
    wave_lds_sync();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) af[kb] = ld8(&fr[n * C::LDF + 32 * kb + 8 * g]);
    f32x4 accP = (f32x4)0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) accP = mma16x32(af[kb], bfr[kb], accP);
    // keep the block-diagonal entries: row 4g + j, column n of this level
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g + j, s = n;
      if ((r >> lv) == (s >> lv)) {
        const int i = ((r >> lv) << (lv + 1)) | hb | (r & (hb - 1));
        const int jj = ((s >> lv) << (lv + 1)) | (s & (hb - 1));
        sm.dl[i * C::LDL + jj] = accL[j];
        sm.dp[i * C::LDP + jj] = accP[j];
      }
    }
  }

  // ---- T = (I + L)^{-1} diag(beta) on 16x16 blocks ----------------------------------------
  if (lane < CS) sm.beta[lane] = beta;
  wave_lds_sync();
  const f32x4 b_r0 = *reinterpret_cast<const f32x4*>(&sm.beta[4 * g]);
  const f32x4 b_r1 = *reinterpret_cast<const f32x4*>(&sm.beta[16 + 4 * g]);
  const float b_c0 = sm.beta[n], b_c1 = sm.beta[16 + n];
  // N = -L (strictly lower) and N^T for both diagonal blocks, L_10, the identity
  f32x4 n0, n0t, n1, n1t, l10, eye;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g + j;
    const bool lower = r > n, upper = n > r;
    n0[j] = lower ? -sm.dl[r * C::LDL + n] * b_r0[j] : 0.0f;
    n0t[j] = upper ? -sm.dl[n * C::LDL + r] * b_c0 : 0.0f;
    n1[j] = lower ? -sm.dl[(16 + r) * C::LDL + 16 + n] * b_r1[j] : 0.0f;
    n1t[j] = upper ? -sm.dl[(16 + n) * C::LDL + 16 + r] * b_c1 : 0.0f;
    l10[j] = sm.dl[(16 + r) * C::LDL + n] * b_r1[j];
    eye[j] = (r == n) ? 1.0f : 0.0f;
  }
  f32x4 d0, d0t, d1, d1t;
  unit_lower_inverse(n0, n0t, eye, d0, d0t);
  unit_lower_inverse(n1, n1t, eye, d1, d1t);
  // T_10 = -D_1 L_10 D_0 diag(beta): carried as (D_1 L_10 D_0)^T = D_0^T (L_10^T D_1^T)
  const f32x4 y = mma16x16(h4(l10), h4(d1t), (f32x4)0.0f);
  const f32x4 zt = mma16x16(h4(d0), h4(y), (f32x4)0.0f);
  // fragments: lane (g, n) holds row 16 rt + n, columns {4g + j} and {16 + 4g + j}
  {
    f16x8 t0, t1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t0[j] = (h16)(d0t[j] * b_r0[j]);
      t0[4 + j] = (h16)0.0f;
      t1[j] = (h16)(-zt[j] * b_r0[j]);
      t1[4 + j] = (h16)(d1t[j] * b_r1[j]);
    }
    st16(__builtin_bit_cast(u32x4, t0), rr, lane * 16 + R::TT);
    st16(__builtin_bit_cast(u32x4, t1), rr, lane * 16 + R::TT + 1024);
  }
  // -P T: the output's intra-chunk operator, applied in the chain to Xn (one
  // fp16 rounding of the product, instead of one each of P, T and Un).  T in
  // fp32 to the D_L buffer (free after the solve), then the lower 16x16 tiles of
  // P T from fp16 high/low parts of both factors (three products per tile:
  // fp32-grade, the low-by-low term is below fp32 rounding), into the factor
  // buffer (free as well) as fp32 rows.
  float* tl = sm.dl;                               // T [row][col], stride LDL
  float* pt = reinterpret_cast<float*>(sm.f);      // P T [row][col], stride LDP
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tl[n * C::LDL + 4 * g + j] = d0t[j] * b_r0[j];
    tl[n * C::LDL + 16 + 4 * g + j] = 0.0f;
    tl[(16 + n) * C::LDL + 4 * g + j] = -zt[j] * b_r0[j];
    tl[(16 + n) * C::LDL + 16 + 4 * g + j] = d1t[j] * b_r1[j];
  }
  wave_lds_sync();
  auto split = [](float x, h16& hi) { hi = (h16)x; return (h16)(x - (float)hi); };
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct <= rt; ++ct) {
      // A: P rows 16 rt + n, k = 8g .. 8g + 7; B: T rows k, column 16 ct + n (natural packing)
      const int row = 16 * rt + n;
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&sm.dp[row * C::LDP + 8 * g]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&sm.dp[row * C::LDP + 8 * g + 4]);
      f16x8 ah, al, bh, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 8 * g + e;
        const float pv = kk <= row ? (e < 4 ? p0[e] : p1[e - 4]) : 0.0f;
        h16 hp, ht;
        al[e] = split(pv, hp);
        ah[e] = hp;
        bl[e] = split(tl[kk * C::LDL + 16 * ct + n], ht);
        bh[e] = ht;
      }
      f32x4 acc = mma16x32(ah, bh, (f32x4)0.0f);
      acc = mma16x32(ah, bl, acc);
      acc = mma16x32(al, bh, acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) pt[(16 * rt + 4 * g + j) * C::LDP + 16 * ct + n] = acc[j];
    }
  wave_lds_sync();
  // -P T fragments, lower triangle with the diagonal, as fp16 high and low parts
  // (the output's intra-chunk term is the largest part of a fast-forgetting
  // head's output; one fp16 rounding of it dominated the error there)
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = 16 * rt + n;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(&pt[row * C::LDP + 4 * g]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(&pt[row * C::LDP + 16 + 4 * g]);
    f16x8 pf, pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = (4 * g + j <= row) ? -lo[j] : 0.0f;
      const float a1 = (16 + 4 * g + j <= row) ? -hi[j] : 0.0f;
      pf[j] = (h16)a0;
      pf[4 + j] = (h16)a1;
      pl[j] = (h16)(a0 - (float)pf[j]);
      pl[4 + j] = (h16)(a1 - (float)pf[4 + j]);
    }
    st16(__builtin_bit_cast(u32x4, pf), rr, lane * 16 + R::PP + 1024 * rt);
    st16(__builtin_bit_cast(u32x4, pl), rr, lane * 16 + R::PL + 1024 * rt);
  }
}

}  // namespace
}  // namespace prep
}  // namespace kda
