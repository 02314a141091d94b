// KDA prefill as a warp-specialised pipeline (gfx950): bf16 q/k/v, d_k in
// {64, 128}, 32 state columns per workgroup, 32-token chunks.
//
// Method: the chunkwise form of the recurrence (the "Kimi 모델 분석" write-up on
// rlaope.github.io, chunkwise/WY section; the per-token rule is section 3.2 of the
// "Kimi K3 Technical Report review" on jw9603.github.io).  With decay products
// taken from the start of the chunk (pre_t = prod_{s<=t} alpha_s per channel,
// gamma = pre at the chunk end):
//
//   KG = K o pre   QG = Q o pre   KC = K o pre^{-1}   KH = K o (gamma / pre)
//   L  = strict_tril(diag(beta) KG KC^T)      P = tril(QG KC^T)
//   T  = (I + L)^{-1} diag(beta)
//   U  = T (V - KG S)      O = QG S + P U      S' = Diag(gamma) S + KH^T U
//
// Eight waves per workgroup, each with one job, advance together one pipeline
// step per barrier; a step moves every item (a chunk, or a segment of one)
// forward by one stage:
//
//   waves 4-7  scan   item n+2: decay products, KG/QG/KC/KH, V, beta, gamma
//   wave 1     L,T    item n+1: L = beta KG KC^T, then T = (I+L)^{-1} diag(beta)
//   wave 2     P      item n+1: P = QG KC^T
//   wave 0     state  item n:   U = T (V - KG S), S' (the only serial chain)
//   wave 3     output item n:   QG S;  item n-1: + P U, store O
//
// Stage outputs live in LDS rings indexed by item number.  Products run on the
// 32x32x16 fp16 matrix cores with fp32 accumulation; the state itself stays
// fp32 in registers and is rounded to fp16 (times a power-of-two scale per state
// column) only as an operand.  KG, QG and KH are bounded by |k|, |q|; KC grows
// as 1/pre, so an item in which some channel's decay falls below e^{-10}, or
// whose KC would leave fp16 range, is redone as a shorter segment: the scan
// votes the first token out of range, the segment ends before it, and the rest
// of the chunk proceeds in segments of that length (alpha >= e^{-5}, the lower
// bound in section 3.5 of the technical report review, keeps any 2 tokens
// within range).  This regrouping is exact.
//
// Sign conventions that save negations: the scan stores -KH, the P wave stores
// -P, and the state wave computes Xn = KG S - V = -(V - KG S), so Un = T Xn = -U,
// S' = gamma S + (-KH)^T Un and O = QG S + (-P) Un.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_prep_impl.h"


namespace kda {
namespace {

typedef _Float16 h16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

constexpr int CS = kPipeChunk;  // tokens per chunk
constexpr float STEEP = 4.5399930e-05f;  // e^{-10}

template <int DK_, int NST_>
struct Cfg4 {
  static constexpr int DK = DK_;
  static constexpr int NST = NST_;       // state waves, 16 state columns each (two here)
  static constexpr int J = 16 * NST;     // state columns per workgroup
  static_assert(NST == 2, "the role layout has two state waves (waves 0 and 1)");
  static constexpr int NKS = DK / 16;   // 16-channel reduction steps (32x32x16 products)
  static constexpr int NKT = DK / 16;   // 16-row channel tiles of a state wave's S
  static constexpr int NKB = DK / 32;   // 32-channel reduction steps (16x16x32 products)
  static constexpr int LDK = DK + 8;    // fp16 [token][channel] row stride
  static constexpr int LDC = CS + 8;    // fp16 [row][token] row stride
  static constexpr int LDV = CS + 4;    // bf16 V^T row stride
  static constexpr int NSW = 4;         // scan waves
  static constexpr int NW = 4 + NSW;    // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int CPW = DK / NSW;  // channels per scan wave
  // A scan lane holds CPL adjacent channels of TPL consecutive tokens; its
  // inputs arrive in TPL loads per tensor, each CPL elements wide.
  static constexpr int CPL = DK == 128 ? 4 : 2;
  static constexpr int PPW = CPW / CPL;  // channel groups per scan wave
  static constexpr int TQ = 64 / PPW;    // token groups per channel group
  static constexpr int TPL = CS / TQ;    // tokens per scan lane
  static_assert(TQ == 8 && TPL == 4, "scan layout");
  // the V slab (CS x J bf16) comes in 16-byte loads, J / 8 lanes per token row,
  // from the last J / 16 scan waves
  static constexpr int VLW = J / 16;
  static constexpr int VW0 = NSW - VLW;  // first V-loading scan wave
  static_assert(CS * J * 2 == VLW * 64 * 16, "V slab split");
};

// Storage position of logical index c (a channel, or a token of the chunk)
// within its block of 32: the eight quads of 4 are stored in the order
// {0, 4, 1, 5, 2, 6, 3, 7}.  A 16-byte read at offset 8g of a block then holds
// indices {4g..4g+3, 16+4g..16+4g+3}: the reduction slots of a 16x16x32 operand
// whose partner is built from two vertically adjacent C tiles in registers
// (lane group g of a C tile holds rows 4g..4g+3).
__device__ __forceinline__ int spos(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

template <class C>
struct ScanSlot {
  alignas(16) h16 kg[CS * C::LDK];    // KG      [t][spos(c)]
  alignas(16) h16 qg[CS * C::LDK];    // QG      [t][spos(c)]
  alignas(16) h16 kh[C::DK * C::LDC]; // -KH^T   [c][spos(t)]
  alignas(16) __bf16 v[C::J * C::LDV];  // V slab transposed [j][t]
  alignas(16) float gam[C::DK];       // gamma per channel
  alignas(16) float beta[CS];         // beta (0 outside the item's segment)
};

template <class C>
struct Smem4 {
  ScanSlot<C> ss[3];
  alignas(16) h16 kc[2][CS * C::LDK];      // KC [t][spos(c)]
  alignas(16) h16 t[2][CS * C::LDC];       // T  [t][spos(s)]
  alignas(16) h16 p[2][CS * C::LDC];       // -P [t][spos(s)]
  alignas(16) float xch[C::NSW][64][4];    // scan: token-group totals per wave
  alignas(16) int flags[2][C::NSW];        // scan: regroup votes per wave
  alignas(16) float scol[2][16];           // state waves: 1/scale of each of their columns
};

// s_waitcnt immediate for "vector memory counter at 0" (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x16 mma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 ld8(const h16* p) { return *reinterpret_cast<const f16x8*>(p); }

// fp16 B operand from one 16-row half of a 32x32 C tile.
__device__ __forceinline__ f16x8 bfrag(const f32x16& t, int half) {
  f16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (h16)t[8 * half + e];
  return f;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---- the item sequence ---------------------------------------------------------
// An item is the token range [lo, hi) of chunk c (tokens of the chunk outside it
// act as identity steps).  Every wave advances the same sequence from the same
// regroup votes, so all agree on every stage's item.
struct Item {
  int seq;  // < 0: no item
  int c, lo, hi, size;
};

__device__ __forceinline__ int chunk_end(int c, int T) { return min(CS, T - c * CS); }

// The item after `it`: the next segment of the same length (size), or the next
// chunk whole.
__device__ __forceinline__ Item next_item(const Item& it, int T, int nchunks) {
  Item n = it;
  n.seq = it.seq + 1;
  n.lo = it.hi;
  if (n.lo >= chunk_end(it.c, T)) {
    n.c = it.c + 1;
    n.lo = 0;
    n.size = CS;
    if (n.c >= nchunks) n.seq = -1;
  }
  n.hi = min(n.lo + n.size, chunk_end(n.c, T));
  return n;
}

// `it` redone as the segment that ends before its first out-of-range token
// `first` (a chunk position in [lo, hi)): between 2 tokens and one token fewer
// than `it` (the scan votes only for items longer than 2 tokens), so every
// split makes progress.
__device__ __forceinline__ Item split_item(const Item& it, int first) {
  Item n = it;
  n.hi = it.lo + min(max(first - it.lo, 2), it.hi - it.lo - 1);
  n.size = n.hi - n.lo;
  return n;
}

struct Ctx4 {
  PrefillParams p;
  int bh, b, h, col0, nchunks;
  int T;           // this sequence's (or part's) length
  long long tok0;  // its first token in the [.][H][d] token rows
  float eA;        // fused gate: e^{A_h}
  bool v_on;       // false: V reads as zeros (transition columns)
  bool o_on;       // false: o is not written
  int ident;       // >= 0: the state starts as columns ident.. of the identity
  const float* s0; // else: this slab's initial state (null: zeros), row stride s0_ld
  int s0_ld;
  float* st;       // this slab's final state (null: not written), row stride st_ld
  int st_ld;
};

// ---- scan waves --------------------------------------------------------------------
constexpr int BW = 1;   // the scan wave that loads beta
// Each load's result is kept as the vector it arrives in: the step loop then
// carries whole register tuples from one step's prefetch to the next step's
// scan.  (Kept as separate words, the tuples were reassembled by register
// copies right after the prefetch, which waited for the loads to land.)
template <class C>
struct Raw4 {
  typedef float AV __attribute__((ext_vector_type(C::CPL)));         // CPL fp32
  typedef uint32_t WV __attribute__((ext_vector_type(C::CPL / 2)));  // CPL bf16
  AV a[C::TPL];  // alpha of this lane's channels, per token
  WV k[C::TPL];
  WV q[C::TPL];
  WV z[C::TPL];  // fused gate: z in place of alpha
  u32x4 v;       // 8 bf16 of the V slab (scan waves VW0.. only)
  float beta;
};

// Where a scan lane's inputs lie: the byte address of chunk 0 of this
// (sequence, head) in each tensor, the bytes per chunk and per token row, and
// the lane's own offsets.  Formed once per wave, so a chunk's addresses cost one
// 64-bit product (chunk index x bytes per chunk) per tensor family rather than
// the whole (token x heads + head) x width arithmetic per tensor, which a scan
// wave otherwise issues as ~60 scalar instructions every step (a wave issues
// at most one instruction per turn of its SIMD, scalar or vector).
struct ScanSrc {
  const char* a;  // alpha (fp32) or the gate's z (bf16)
  const char* k;
  const char* q;
  const char* v;  // this slab's first column (or any address when V is off)
  const char* b;  // beta
  int kc;         // bytes per chunk of k and q (alpha: kc << ash)
  int ash;        // 1: alpha is fp32, 0: z is bf16
  int vc, bc;     // bytes per chunk of v and beta
  int kr, vr, br; // bytes per token row of k, v (0: V off) and beta
  int ts2;        // bytes between a lane's consecutive tokens in k (alpha: ts2 << ash)
  int vo_k, vo_v, vo_b;  // this lane's byte offsets in k, v and beta
};

template <class C, bool G>
__device__ ScanSrc scan_src(const Ctx4& cx, int sw, int lane) {
  const PrefillParams& p = cx.p;
  const int cp = lane % C::PPW, tq = lane / C::PPW;
  const size_t row0 = (size_t)cx.tok0 * p.H + cx.h;
  const int ts = p.H * C::DK;  // elements between tokens
  ScanSrc r;
  r.ash = G ? 0 : 1;
  r.a = G ? reinterpret_cast<const char*>(static_cast<const __bf16*>(p.z) + row0 * C::DK)
          : reinterpret_cast<const char*>(p.alpha + row0 * C::DK);
  r.k = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + row0 * C::DK);
  r.q = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.q) + row0 * C::DK);
  r.v = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + row0 * p.dv + (cx.v_on ? cx.col0 : 0));
  r.b = reinterpret_cast<const char*>(p.beta + row0);
  r.kr = ts * 2;
  r.kc = CS * r.kr;
  r.vr = cx.v_on ? p.H * p.dv * 2 : 0;  // a zero-length range reads as zeros: the transition columns have V = 0
  r.vc = CS * p.H * p.dv * 2;
  r.br = p.H * 4;
  r.bc = CS * r.br;
  r.ts2 = ts * 2;
  r.vo_k = 2 * (tq * C::TPL * ts + C::CPW * sw + C::CPL * cp);
  // V row vt / (J/8), columns 8 (vt % (J/8)) .. + 7 (scan waves VW0.. only)
  const int vt = 64 * (sw - C::VW0) + lane;
  r.vo_v = 2 * ((vt / (C::J / 8)) * p.H * p.dv + 8 * (vt % (C::J / 8)));
  r.vo_b = 4 * (lane % CS) * p.H;  // beta of token l is kept by lane l
  return r;
}

// Loads chunk c's inputs for scan lane (sw, lane): channels CPL*cp .. of the
// wave's slice, tokens tq*TPL ..  Rows past the sequence end read as zeros
// (buffer range check).  One load per token and tensor: the load count, not
// the byte count, sets what the scan waits for here.  The V slab and beta are
// loaded by the last scan waves, so the first one, which shares its SIMD with
// the state wave, does none of that work.
template <class C, bool G>
__device__ void load_raw4(Raw4<C>& raw, const Ctx4& cx, const ScanSrc& src, int c, int sw) {
  const int rows = min(CS, cx.T - c * CS);
  const size_t ok = (size_t)(unsigned)c * (unsigned)src.kc;  // chunk offset in k and q
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(src.a + (ok << src.ash), (rows * src.kr) << src.ash);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(src.k + ok, rows * src.kr);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(src.q + ok, rows * src.kr);
  const int vk = src.vo_k, va = src.vo_k << src.ash;
  typedef typename Raw4<C>::AV AV;
  typedef typename Raw4<C>::WV WV;
#pragma unroll
  for (int i = 0; i < C::TPL; ++i) {
    // Reinterpret each loaded vector as a whole: taking single elements of the
    // integer vector a buffer load returns and reinterpreting them as float is
    // miscompiled by this toolchain (both read one narrowed dword).
    const int sk = i * src.ts2, sa = sk << src.ash;
    if constexpr (C::CPL == 4) {
      if constexpr (G) raw.z[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b64(ra, va, sa, 0));
      else raw.a[i] = __builtin_bit_cast(AV, __builtin_amdgcn_raw_buffer_load_b128(ra, va, sa, 0));
      raw.k[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b64(rk, vk, sk, 0));
      raw.q[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b64(rq, vk, sk, 0));
    } else {
      if constexpr (G) raw.z[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b32(ra, va, sa, 0));
      else raw.a[i] = __builtin_bit_cast(AV, __builtin_amdgcn_raw_buffer_load_b64(ra, va, sa, 0));
      raw.k[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b32(rk, vk, sk, 0));
      raw.q[i] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b32(rq, vk, sk, 0));
    }
  }
  if (sw >= C::VW0) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(src.v + (size_t)(unsigned)c * (unsigned)src.vc, rows * src.vr);
    raw.v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, src.vo_v, 0, 0));
  }
  if (sw == BW) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(src.b + (size_t)(unsigned)c * (unsigned)src.bc, rows * src.br);
    raw.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, src.vo_b, 0, 0));
  }
}

// What a scan lane takes from its raw inputs: decays (alpha, or alpha formed from
// the gate), keys and queries as fp32, the V words and beta.  Read in one place,
// before the next chunk is loaded into the same registers.
template <class C>
struct ScanIn {
  float a[C::TPL][C::CPL];
  float kf[C::TPL][C::CPL];
  float qf[C::TPL][C::CPL];
};

// Makes the values read from raw count as used here, so the compiler computes
// them before a following load overwrites raw.
template <class C>
__device__ __forceinline__ void pin(ScanIn<C>& in) {
#pragma unroll
  for (int i = 0; i < C::TPL; ++i)
#pragma unroll
    for (int e = 0; e < C::CPL; ++e) asm volatile("" : "+v"(in.a[i][e]), "+v"(in.kf[i][e]), "+v"(in.qf[i][e]));
}

// Also stores the item's V slab (transposed) and beta to its ring slot, which
// need nothing else.
template <class C, bool G>
__device__ __forceinline__ void scan_read(ScanIn<C>& in, Smem4<C>& sm, const Raw4<C>& raw, const Item& it, float eA,
                                          int sw, int lane) {
  ScanSlot<C>& sl = sm.ss[it.seq % 3];
  if (sw >= C::VW0) {
    // V^T: this lane holds row vt / (J/8), columns 8 (vt % (J/8)) .. + 7
    const int vt = 64 * (sw - C::VW0) + lane;
    const int vr = vt / (C::J / 8), vc = 8 * (vt % (C::J / 8));
    const uint32_t w[4] = {raw.v.x, raw.v.y, raw.v.z, raw.v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sl.v[(vc + e) * C::LDV + vr] = __builtin_bit_cast(__bf16, (uint16_t)(w[e / 2] >> (16 * (e % 2))));
  }
  if (sw == BW && lane < CS) sl.beta[lane] = (lane >= it.lo && lane < it.hi) ? raw.beta : 0.0f;
#pragma unroll
  for (int i = 0; i < C::TPL; ++i) {
#pragma unroll
    for (int e = 0; e < C::CPL; ++e) {
      if constexpr (G) {  // alpha = exp(-5 sigmoid(e^A z)) from the bf16 gate input
        const uint32_t zw = raw.z[i][e / 2];
        in.a[i][e] = gate_retention(eA * ((e & 1) ? bf16_hi(zw) : bf16_lo(zw)));
      } else {
        in.a[i][e] = raw.a[i][e];
      }
    }
#pragma unroll
    for (int j = 0; j < C::CPL / 2; ++j) {
      in.kf[i][2 * j] = bf16_lo(raw.k[i][j]);
      in.kf[i][2 * j + 1] = bf16_hi(raw.k[i][j]);
      in.qf[i][2 * j] = bf16_lo(raw.q[i][j]);
      in.qf[i][2 * j + 1] = bf16_hi(raw.q[i][j]);
    }
  }
}

// Scan of item `it` by scan wave sw (one channel pair and TPL consecutive tokens
// per lane): writes ring slot it.seq % 3, KC slot it.seq % 2 and this wave's
// regroup vote.  FULL: the item is the whole chunk (no token is masked).
template <class C, bool FULL>
__device__ void scan4_body(Smem4<C>& sm, const ScanIn<C>& sin, const Item& it, int sw, int lane, int par) {
  constexpr int L = C::CPL, TP = C::TPL;
  ScanSlot<C>& sl = sm.ss[it.seq % 3];
  h16* kc = sm.kc[it.seq % 2];
  const int cp = opaque(lane % C::PPW), tq = opaque(lane / C::PPW);
  const int ch = C::CPW * sw + L * cp;  // this lane's first channel
  const int tb = tq * TP;               // first of this lane's tokens
  const int lo = it.lo, hi = it.hi;
  auto in = [&](int i) { return FULL || (tb + i >= lo && tb + i < hi); };

  float a[TP][L], gt[L];
#pragma unroll
  for (int e = 0; e < L; ++e) gt[e] = 1.0f;
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int e = 0; e < L; ++e) {
      a[i][e] = in(i) ? sin.a[i][e] : 1.0f;
      gt[e] *= a[i][e];
    }
  // keys and queries, zero outside the item
  float kf[TP][L], qf[TP][L];
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int e = 0; e < L; ++e) {
      kf[i][e] = in(i) ? sin.kf[i][e] : 0.0f;
      qf[i][e] = in(i) ? sin.qf[i][e] : 0.0f;
    }
  // Token-group products of every channel, exchanged within the wave.  Each
  // lane runs the product over the groups in order, keeps the partial product
  // reached at its own group (the groups before it), and takes the groups
  // after it from the total.
  if constexpr (L == 4) *reinterpret_cast<f32x4*>(&sm.xch[sw][lane][0]) = f32x4{gt[0], gt[1], gt[2], gt[3]};
  else *reinterpret_cast<f32x2*>(&sm.xch[sw][lane][0]) = f32x2{gt[0], gt[1]};
  wave_lds_sync();
  float run[L], ep[L];
#pragma unroll
  for (int e = 0; e < L; ++e) run[e] = ep[e] = 1.0f;
#pragma unroll
  for (int g = 0; g < C::TQ; ++g) {
    float v[L];
    if constexpr (L == 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(&sm.xch[sw][g * C::PPW + cp][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = w[e];
    } else {
      const f32x2 w = *reinterpret_cast<const f32x2*>(&sm.xch[sw][g * C::PPW + cp][0]);
      v[0] = w.x;
      v[1] = w.y;
    }
    const bool mine = g == tq;
#pragma unroll
    for (int e = 0; e < L; ++e) {
      ep[e] = mine ? run[e] : ep[e];
      run[e] *= v[e];
    }
  }
  float gam[L], rg[L], sp[L];
#pragma unroll
  for (int e = 0; e < L; ++e) {
    gam[e] = run[e];
    rg[e] = __builtin_amdgcn_rcpf(gam[e]);
    // gamma >= e^-10 for every item whose results are used (steeper ones are
    // regrouped), so this quotient neither underflows nor loses precision
    sp[e] = gam[e] * __builtin_amdgcn_rcpf(ep[e] * gt[e]);
  }
  // pre_t (prefix through t) and -gamma/pre_t (minus the suffix after t)
  float pre[TP][L], ns[TP][L];
#pragma unroll
  for (int e = 0; e < L; ++e) {
    float r = ep[e];
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      r *= a[i][e];
      pre[i][e] = r;
    }
    float sf = -sp[e];
#pragma unroll
    for (int i = TP - 1; i >= 0; --i) {
      ns[i][e] = sf;
      sf *= a[i][e];
    }
  }
  float kmax = 0.0f;
  h16 khv[L][TP];
  const int col = spos(ch);
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    h16 kg[L], qg[L], kcv[L];
#pragma unroll
    for (int e = 0; e < L; ++e) {
      kmax = fmaxf(kmax, fabsf(kf[i][e]));
      // fused multiply rounded once to fp16 (a mixed-precision fma): one
      // instruction per element instead of a multiply and half a conversion
      kg[e] = (h16)__builtin_fmaf(kf[i][e], pre[i][e], 0.0f);
      qg[e] = (h16)__builtin_fmaf(qf[i][e], pre[i][e], 0.0f);
      const float kh = kf[i][e] * ns[i][e];  // -KH
      khv[e][i] = (h16)kh;
      kcv[e] = (h16)__builtin_fmaf(kh, -rg[e], 0.0f);  // KC = KH / gamma
    }
    const int r = (tb + i) * C::LDK + col;  // CPL adjacent channels keep adjacent positions
    if constexpr (L == 4) {
      *reinterpret_cast<f16x4*>(&sl.kg[r]) = f16x4{kg[0], kg[1], kg[2], kg[3]};
      *reinterpret_cast<f16x4*>(&sl.qg[r]) = f16x4{qg[0], qg[1], qg[2], qg[3]};
      *reinterpret_cast<f16x4*>(&kc[r]) = f16x4{kcv[0], kcv[1], kcv[2], kcv[3]};
    } else {
      *reinterpret_cast<f16x2*>(&sl.kg[r]) = f16x2{kg[0], kg[1]};
      *reinterpret_cast<f16x2*>(&sl.qg[r]) = f16x2{qg[0], qg[1]};
      *reinterpret_cast<f16x2*>(&kc[r]) = f16x2{kcv[0], kcv[1]};
    }
  }
#pragma unroll
  for (int e = 0; e < L; ++e)
    *reinterpret_cast<f16x4*>(&sl.kh[(ch + e) * C::LDC + spos(tb)]) = f16x4{khv[e][0], khv[e][1], khv[e][2], khv[e][3]};
  if (tq == 0) {
    if constexpr (L == 4) *reinterpret_cast<f32x4*>(&sl.gam[ch]) = f32x4{gam[0], gam[1], gam[2], gam[3]};
    else *reinterpret_cast<f32x2*>(&sl.gam[ch]) = f32x2{gam[0], gam[1]};
  }
  // Regroup vote: the first token (chunk position) at which some channel's
  // prefix decay falls below e^{-10} or KC = k/pre would leave fp16 range; CS
  // when there is none.  A bound over the whole item (smallest gamma, largest
  // |k| times largest 1/gamma) clears almost every item, so only a wave that
  // fails it looks at the tokens one by one.  Items of 2 tokens are never split.
  float gmin = gam[0], rgm = rg[0];
#pragma unroll
  for (int e = 1; e < L; ++e) {
    gmin = fminf(gmin, gam[e]);
    rgm = fmaxf(rgm, rg[e]);
  }
  const bool rough = !(gmin >= STEEP) || !(kmax * rgm < 32768.0f);
  int vote = CS;
  if (hi - lo > 2 && __builtin_amdgcn_ballot_w64(rough) != 0) {
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      bool bad = false;
#pragma unroll
      for (int j = 0; j < L / 2; ++j) {
        const float k0 = fabsf(kf[i][2 * j]), k1 = fabsf(kf[i][2 * j + 1]);
        const float p0 = pre[i][2 * j], p1 = pre[i][2 * j + 1];
        bad = bad || !(p0 >= STEEP) || !(k0 < 32768.0f * p0) || !(p1 >= STEEP) || !(k1 < 32768.0f * p1);
      }
      // lanes are ordered by token group, so the lowest voting lane holds the
      // earliest such token among this token slot's lanes
      const uint64_t m = __builtin_amdgcn_ballot_w64(bad && in(i));
      if (m != 0) vote = min(vote, (int)(__builtin_ctzll(m) / C::PPW) * TP + i);
    }
    // gamma, a product in another order, may round below the bound although
    // no prefix does: drop the last token
    if (vote >= hi && __builtin_amdgcn_ballot_w64(!(gmin >= STEEP)) != 0) vote = hi - 1;
  }
  if (lane == 0) sm.flags[par][sw] = vote;
}

template <class C>
__device__ void scan4(Smem4<C>& sm, const ScanIn<C>& sin, const Item& it, int sw, int lane, int par) {
  if (it.lo == 0 && it.hi == CS) scan4_body<C, true>(sm, sin, it, sw, lane, par);
  else scan4_body<C, false>(sm, sin, it, sw, lane, par);
}

// ---- L, T wave -------------------------------------------------------------------------
// 16x16 matrix-core steps on C tiles (lane g = l/16, n = l%16 holds rows 4g+j of
// column n); the helpers are in kda_device.h.
template <class C>
__device__ void solve4(Smem4<C>& sm, const Item& it, int lane) {
  const ScanSlot<C>& sl = sm.ss[it.seq % 3];
  const h16* kc = sm.kc[it.seq % 2];
  h16* tt = sm.t[it.seq % 2];
  const int g = opaque(lane / 16), n = opaque(lane % 16);
  // K fragments of token rows n and 16+n over the channel steps (same storage
  // order on both sides of every product)
  f16x8 kg0[C::NKS / 2], kg1[C::NKS / 2], kc0[C::NKS / 2], kc1[C::NKS / 2];
#pragma unroll
  for (int s = 0; s < C::NKS / 2; ++s) {
    const int off = n * C::LDK + 32 * s + 8 * g;
    kg0[s] = ld8(&sl.kg[off]);
    kg1[s] = ld8(&sl.kg[off + 16 * C::LDK]);
    kc0[s] = ld8(&kc[off]);
    kc1[s] = ld8(&kc[off + 16 * C::LDK]);
  }
  f32x4 a00 = (f32x4)0.0f, a00t = a00, a11 = a00, a11t = a00, a10t = a00;
#pragma unroll
  for (int s = 0; s < C::NKS / 2; ++s) {
    a00 = mma16x32(kg0[s], kc0[s], a00);   // (KG KC^T)[4g+j][n]         block (0,0)
    a00t = mma16x32(kc0[s], kg0[s], a00t); // (KG KC^T)[n][4g+j]         transposed
    a11 = mma16x32(kg1[s], kc1[s], a11);   // block (1,1)
    a11t = mma16x32(kc1[s], kg1[s], a11t);
    a10t = mma16x32(kc0[s], kg1[s], a10t); // (KG KC^T)[16+n][4g+j]      block (1,0), transposed
  }
  const f32x4 b_r0 = *reinterpret_cast<const f32x4*>(&sl.beta[4 * g]);
  const f32x4 b_r1 = *reinterpret_cast<const f32x4*>(&sl.beta[16 + 4 * g]);
  const float b_c0 = sl.beta[n], b_c1 = sl.beta[16 + n];
  // N = -L (strictly lower, beta of the row folded in) and N^T for both diagonal
  // blocks; L_10^T; the identity tile
  f32x4 n0, n0t, n1, n1t, l10t, eye;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g + j;
    const bool lower = r > n, upper = n > r;
    n0[j] = lower ? -a00[j] * b_r0[j] : 0.0f;
    n0t[j] = upper ? -a00t[j] * b_c0 : 0.0f;
    n1[j] = lower ? -a11[j] * b_r1[j] : 0.0f;
    n1t[j] = upper ? -a11t[j] * b_c1 : 0.0f;
    l10t[j] = a10t[j] * b_c1;
    eye[j] = (r == n) ? 1.0f : 0.0f;
  }
  f32x4 d0, d0t, d1, d1t;
  unit_lower_inverse(n0, n0t, eye, d0, d0t);
  unit_lower_inverse(n1, n1t, eye, d1, d1t);
  // T_10 = -D_1 L_10 D_0 diag(beta)
  const f32x4 y = mma16x16(h4(l10t), h4(d0), (f32x4)0.0f);  // L_10 D_0
  const f32x4 z = mma16x16(h4(d1t), h4(y), (f32x4)0.0f);    // D_1 (L_10 D_0)
  // T = (I + L)^{-1} diag(beta): rows 4g+j (+16), column n (+16)
  const int c0 = spos(n), c1 = spos(16 + n);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g + j;
    tt[r * C::LDC + c0] = (h16)(d0[j] * b_c0);
    tt[(16 + r) * C::LDC + c1] = (h16)(d1[j] * b_c1);
    tt[(16 + r) * C::LDC + c0] = (h16)(-z[j] * b_c0);
  }
}

// ---- P wave ----------------------------------------------------------------------------
template <class C>
__device__ void pmat4(Smem4<C>& sm, const Item& it, int lane) {
  const ScanSlot<C>& sl = sm.ss[it.seq % 3];
  const h16* kc = sm.kc[it.seq % 2];
  h16* pp = sm.p[it.seq % 2];
  const int h = opaque(lane / 32), m = opaque(lane % 32);
  f32x16 acc = (f32x16)0.0f;
#pragma unroll
  for (int s = 0; s < C::NKS; ++s) {
    const int off = m * C::LDK + 16 * s + 8 * h;
    acc = mma32(ld8(&sl.qg[off]), ld8(&kc[off]), acc);
  }
  h16* prow = &pp[(4 * h) * C::LDC + spos(m)];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 8 * j + 4 * h + r;
      prow[(8 * j + r) * C::LDC] = (h16)(t >= m ? -acc[4 * j + r] : 0.0f);
    }
}

// ---- state waves ---------------------------------------------------------------------------
// Two waves, each owning 16 of the workgroup's 32 state columns, run the chain on
// 16x16x32 fp16 matrix cores: lane l (g = l / 16, n = l % 16) holds rows 4g + r
// of column n of every C tile.  Each also forms the output of its columns, so S
// and Un never leave its registers:
//   Xn = KG S - V,  Un = T Xn,  S' = gamma S + (-KH)^T Un,
//   O^T = S^T QG^T + Un^T (-P)^T      (the transposed output: a lane holds four
//                                      adjacent columns of one token)
// Every product's reduction slots are in the stacked order of two C tiles, so
// operands built from C tiles in registers (S, Xn, Un) pair with rows read from
// LDS in spos order in one 16-byte read.
template <class C>
struct StateRegs {
  f32x4 S[C::NKT];   // the state times sc (per column): rows 16 it + 4g + r, column n
  f16x8 Sf[C::NKB];  // fp16 S for reduction step kb (channels 32 kb ..)
  f32x4 vn[2];       // -V * sc of the item: tokens 16 rt + 4g + r
  float sc;          // 2^-e, this lane's column scale
  f32x4 usc;         // 1/sc of columns 4g .. 4g + 3 (the output rows this lane holds)
};

__device__ __forceinline__ f32x4 mma16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// fp16 operand in stacked order from two C tiles (slots 0..3 from the first)
__device__ __forceinline__ f16x8 stack2(const f32x4& lo, const f32x4& hi) {
  return f16x8{(h16)lo[0], (h16)lo[1], (h16)lo[2], (h16)lo[3], (h16)hi[0], (h16)hi[1], (h16)hi[2], (h16)hi[3]};
}

// Stores a state wave's output tiles (token 16 rt + n, columns 4g .. 4g + 3 of the
// wave's 16, times their column scales usc) of item `it`.
__device__ __forceinline__ void store_out(const Ctx4& cx, const Item& it, const f32x4 (&O)[2], const f32x4& usc, int w,
                                          int lane) {
  const int g = opaque(lane / 16), n = opaque(lane % 16);
  const PrefillParams& p = cx.p;
  const int rows = chunk_end(it.c, cx.T);
  const int esz = p.o_f32 ? 4 : 2;
  const int rs = p.H * p.dv * esz;
  char* ob = static_cast<char*>(p.o) +
             (((size_t)(cx.tok0 + it.c * CS) * p.H + cx.h) * p.dv + (cx.o_on ? cx.col0 + 16 * w : 0)) * esz;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(ob, cx.o_on ? rows * rs : 0);  // zero-length: stores dropped
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int t = 16 * rt + n;
    // tokens outside the item are pushed past the range, so their stores are dropped
    const int voff = t * rs + 4 * g * esz + ((unsigned)(t - it.lo) < (unsigned)(it.hi - it.lo) ? 0 : 0x40000000);
    const f32x4 y = O[rt] * usc;
    if (p.o_f32) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), rsrc, voff, 0, 0);
    } else {
      // reinterpret the whole vector (single elements are miscompiled)
      const bf16x4 b = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), rsrc, voff, 0, 0);
    }
  }
}

// One item of the chain for state wave w (columns 16w .. 16w + 15 of the slab),
// with the output of those columns stored.
template <class C>
__device__ void state_step(Smem4<C>& sm, StateRegs<C>& R, const Item& it, const Ctx4& cx, int w, int lane) {
  const ScanSlot<C>& sl = sm.ss[it.seq % 3];
  const h16* tt = sm.t[it.seq % 2];
  const h16* pp = sm.p[it.seq % 2];
  const int g = opaque(lane / 16), n = opaque(lane % 16);
  // operands first, so their reads overlap the products
  f16x8 A[2][C::NKB], Q[2][C::NKB], Tf[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      A[rt][kb] = ld8(&sl.kg[(16 * rt + n) * C::LDK + 32 * kb + 8 * g]);
      Q[rt][kb] = ld8(&sl.qg[(16 * rt + n) * C::LDK + 32 * kb + 8 * g]);
    }
    Tf[rt] = ld8(&tt[(16 * rt + n) * C::LDC + 8 * g]);
  }
  // Xn = KG S - V (scaled), and the first output term S^T QG^T
  f32x4 X[2] = {R.vn[0], R.vn[1]};
  f32x4 O[2] = {(f32x4)0.0f, (f32x4)0.0f};
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      X[rt] = mma16(A[rt][kb], R.Sf[kb], X[rt]);
      O[rt] = mma16(R.Sf[kb], Q[rt][kb], O[rt]);
    }
  // decay the state in place while the products run
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) R.S[i] *= *reinterpret_cast<const f32x4*>(&sl.gam[16 * i + 4 * g]);
  f16x8 KH[C::NKT];
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) KH[i] = ld8(&sl.kh[(16 * i + n) * C::LDC + 8 * g]);
  f16x8 Pf[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) Pf[rt] = ld8(&pp[(16 * rt + n) * C::LDC + 8 * g]);
  // Un = T Xn
  const f16x8 xf = stack2(X[0], X[1]);
  f32x4 U[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) U[rt] = mma16(Tf[rt], xf, (f32x4)0.0f);
  const f16x8 uf = stack2(U[0], U[1]);
  // S' = gamma S + (-KH)^T Un;  O^T += Un^T (-P)^T
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) R.S[i] = mma16(KH[i], uf, R.S[i]);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) O[rt] = mma16(uf, Pf[rt], O[rt]);

  store_out(cx, it, O, R.usc, w, lane);
}

// Maximum over the four lanes l % 16 == n (the four lane groups of a C-tile
// column): lane swaps across halves and across rows, no trip through LDS.
__device__ __forceinline__ float column_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);    // lanes l and l ^ 32
  float y, z;
  asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(h[0]), "v"(h[1]));
  const unsigned v = __float_as_uint(y);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);    // lanes l and l ^ 16
  asm("v_max_f32 %0, %1, %2" : "=v"(z) : "v"(r[0]), "v"(r[1]));
  return z;
}

// Column scale of a state wave for its next item, given the item's V values vf
// (tokens 16 rt + 4g + r of column n), and the fp16 fragments of S and -V * sc.
// scol: the wave's 16 column reciprocals in LDS.
template <class C>
__device__ __forceinline__ void state_rescale(StateRegs<C>& R, const float (&vf)[2][4], float* scol, int g, int n) {
  // this lane's maxima of |S| (a tree, not a chain) and of |V| times the scale
  float t[C::NKT];
#pragma unroll
  for (int i = 0; i < C::NKT; ++i)
    t[i] = fmaxf(fmaxf(fabsf(R.S[i][0]), fabsf(R.S[i][1])), fmaxf(fabsf(R.S[i][2]), fabsf(R.S[i][3])));
#pragma unroll
  for (int w = C::NKT / 2; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
  const float mv = fmaxf(fmaxf(fmaxf(fabsf(vf[0][0]), fabsf(vf[0][1])), fmaxf(fabsf(vf[0][2]), fabsf(vf[0][3]))),
                         fmaxf(fmaxf(fabsf(vf[1][0]), fabsf(vf[1][1])), fmaxf(fabsf(vf[1][2]), fabsf(vf[1][3]))));
  // Keep the scaled column maximum within [2^-4, 2^4]; rescale rarely.  The
  // scale is capped at 2^64: a column whose values have decayed below 2^-68
  // with no value input (a transition column, or an all-zero V column) stays
  // there, so the scale never overflows to infinity (0 * inf would be NaN).
  // (The four lanes of a column share its scale, so the maximum is taken once.)
  const float m = column_max(fmaxf(t[0], mv * R.sc));
  const bool bad = m > 16.0f || (m > 0.0f && m < 0.0625f && R.sc < 0x1p64f);
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {
    float f = 1.0f;
    if (bad) {
      const int ex = __builtin_amdgcn_frexp_expf(m);  // m = frac * 2^ex, frac in [0.5, 1)
      f = fminf(__builtin_amdgcn_ldexpf(1.0f, -ex), 0x1p64f / R.sc);  // powers of two: exact
    }
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] *= f;
    R.sc *= f;
    // the output rows a lane holds are columns 4g .. 4g + 3: exchange the scales
    if (g == 0) scol[n] = __builtin_amdgcn_rcpf(R.sc);
    wave_lds_sync();
    R.usc = *reinterpret_cast<const f32x4*>(&scol[4 * g]);
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) R.vn[rt][r] = -vf[rt][r] * R.sc;
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) R.Sf[kb] = stack2(R.S[2 * kb], R.S[2 * kb + 1]);
}

// Prepares item `it` (next for the state wave): column scale, fp16 fragments of
// S and -V * sc.
template <class C>
__device__ void state_prepare(Smem4<C>& sm, StateRegs<C>& R, const Item& it, int w, int lane) {
  const ScanSlot<C>& sl = sm.ss[it.seq % 3];
  const int g = opaque(lane / 16), n = opaque(lane % 16);
  float vf[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {  // tokens 16 rt + 4g .. + 3 of column 16w + n
    const u32x2 v2 = *reinterpret_cast<const u32x2*>(&sl.v[(16 * w + n) * C::LDV + 16 * rt + 4 * g]);
    vf[rt][0] = __builtin_bit_cast(float, v2.x << 16);
    vf[rt][1] = __builtin_bit_cast(float, v2.x & 0xffff0000u);
    vf[rt][2] = __builtin_bit_cast(float, v2.y << 16);
    vf[rt][3] = __builtin_bit_cast(float, v2.y & 0xffff0000u);
  }
  state_rescale<C>(R, vf, sm.scol[w], g, n);
}

// ---- kernel ---------------------------------------------------------------------------------
enum Role { SCAN, SOLVE, PMAT, STATE };

// Writes state wave w's S (16 columns; S = R.S / R.sc) to the [d_k][d_v]
// matrix whose slab starts at dst.  Buffer stores with a per-lane offset and a
// scalar row offset: no 64-bit address per element, and the stride is pinned
// here so nothing of it is hoisted into the step loop around a call.
template <class C>
__device__ void store_state(float* dst, const StateRegs<C>& R, int dv_, int w, int lane) {
  const int dv = __builtin_amdgcn_readfirstlane(opaque(dv_));
  const int g = lane / 16, n = lane % 16;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, C::DK * dv * 4);
  const int voff = (4 * g * dv + 16 * w + n) * 4;
  const float usc = __builtin_amdgcn_rcpf(R.sc);
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) {
    // Reinterpret the scaled tile as a whole: reinterpreting single elements of
    // a vector is miscompiled by this toolchain (every element reads element 0).
    const u32x4 v = __builtin_bit_cast(u32x4, R.S[i] * usc);
#pragma unroll
    for (int r = 0; r < 4; ++r) __builtin_amdgcn_raw_buffer_store_b32(v[r], rs, voff, (16 * i + r) * dv * 4, 0);
  }
}

// One wave's whole life: its own copy of the item sequence and its own
// registers (each role is a separate loop, so no role pays for another's live
// values).  Every role executes exactly one barrier per step.
template <class C, Role ROLE, bool G>
__device__ void run_role(Smem4<C>& sm, const Ctx4& cx, const SnapList& snap, int lane, int sw) {
  const PrefillParams& p = cx.p;
  StateRegs<C> R;
  // Scan inputs: the scan reads what it needs of chunk c out of raw first and
  // then loads chunk c + 1 into it, so the loads have most of a step to land.
  // rc: the chunk raw holds (a chunk regrouped into segments after that
  // prefetch is loaded again).
  Raw4<C> raw;
  int rc = -1;
  if constexpr (ROLE == STATE) {
    // state wave sw owns columns 16 sw .. 16 sw + 15 of the slab
    const int g = lane / 16, n = lane % 16, col = 16 * sw + n;
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] = (f32x4)0.0f;
    if (cx.ident >= 0) {
#pragma unroll
      for (int i = 0; i < C::NKT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) R.S[i][r] = (16 * i + 4 * g + r == cx.ident + col) ? 1.0f : 0.0f;
    } else if (cx.s0) {
#pragma unroll
      for (int i = 0; i < C::NKT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) R.S[i][r] = cx.s0[(size_t)(16 * i + 4 * g + r) * cx.s0_ld + col];
    }
    // Wait for the state loads once, here: otherwise the step loop carries a
    // wait before each write to a state register (no-op waits on the chain).
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    R.sc = 1.0f;
    R.usc = (f32x4)1.0f;
  }
  ScanSrc src{};
  if constexpr (ROLE == SCAN) {
    src = scan_src<C, G>(cx, sw, lane);
    if (cx.nchunks > 0) {
      load_raw4<C, G>(raw, cx, src, 0, sw);
      rc = 0;
    }
  }
  block_sync_lds();  // the zeroed T ring is visible

  const Item none = {-1, 0, 0, 0, 0};
  Item sI = none, bI = none, stI = none;
  if (cx.nchunks > 0) sI = Item{0, 0, 0, chunk_end(0, cx.T), CS};
  int par = 0;
  int ns = 0;  // state role: next recorded position
  while (sI.seq >= 0 || bI.seq >= 0 || stI.seq >= 0) {
    if constexpr (ROLE == SCAN) {
      if (sI.seq >= 0) {
        ScanIn<C> sin;
        if (rc == sI.c) {
          scan_read<C, G>(sin, sm, raw, sI, cx.eA, sw, lane);
          // raw is read: the item that ends its chunk fetches the next chunk
          // into it (the values read are pinned first, so no read of raw is
          // moved after the loads that overwrite it)
          if (sI.hi == chunk_end(sI.c, cx.T) && sI.c + 1 < cx.nchunks) {
            pin(sin);
            load_raw4<C, G>(raw, cx, src, sI.c + 1, sw);
            rc = sI.c + 1;
          }
          scan4<C>(sm, sin, sI, sw, lane, par);
        } else {
          // a chunk regrouped after its successor was fetched (rare): loaded
          // again into a buffer of its own, so raw keeps a single load site
          Raw4<C> again;
          load_raw4<C, G>(again, cx, src, sI.c, sw);
          scan_read<C, G>(sin, sm, again, sI, cx.eA, sw, lane);
          scan4<C>(sm, sin, sI, sw, lane, par);
        }
      }
    } else if constexpr (ROLE == SOLVE) {
      if (bI.seq >= 0) solve4<C>(sm, bI, lane);
    } else if constexpr (ROLE == PMAT) {
      if (bI.seq >= 0) pmat4<C>(sm, bI, lane);
    } else {
      if (stI.seq >= 0) {
        state_step<C>(sm, R, stI, cx, sw, lane);
        // record the state after a listed number of tokens
        if (ns < p.nsnap && stI.hi == chunk_end(stI.c, cx.T) && snap.pos[ns] == stI.c * CS + stI.hi) {
          store_state<C>(p.snaps + ((size_t)cx.bh * p.nsnap + ns) * C::DK * p.dv + cx.col0, R, p.dv, sw, lane);
          ++ns;
          // Drain the stores here, on this rare path: otherwise the next steps
          // carry a wait for them before every write to a register they might
          // still read.
          __builtin_amdgcn_s_waitcnt(kVmcnt0);
        }
      }
      if (bI.seq >= 0) state_prepare<C>(sm, R, bI, sw, lane);
    }
    // The scan item's successor is formed before the barrier, so after it only
    // the regroup vote remains to be read.
    Item nI = none;
    if (sI.seq >= 0) nI = next_item(sI, cx.T, cx.nchunks);
    block_sync_lds();
    int first = CS;  // the scan waves' earliest out-of-range token, CS: none
    if (sI.seq >= 0) {
#pragma unroll
      for (int w4 = 0; w4 < C::NSW; w4 += 4) {
        const int4 f = *reinterpret_cast<const int4*>(&sm.flags[par][w4]);
        first = min(first, min(min(f.x, f.y), min(f.z, f.w)));
      }
      first = __builtin_amdgcn_readfirstlane(first);
    }
    const bool steep = first < CS;
    stI = bI;
    bI = (sI.seq >= 0 && !steep) ? sI : none;
    if (sI.seq >= 0) sI = steep ? split_item(sI, first) : nI;
    par ^= 1;
  }

  if constexpr (ROLE == STATE) {
    if (cx.st) store_state<C>(cx.st, R, cx.st_ld, sw, lane);
  }
}

template <class C, bool G>
__global__ __launch_bounds__(C::NT, 1) void kda_prefill_pipe_kernel(PrefillParams p, SnapList snap) {
  __shared__ Smem4<C> sm;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  int task, slab;
  task_of_block((p.split == 1 ? p.dv + C::DK : p.dv) / C::J, task, slab);
  __shared__ int seq_lens[kMaxRankedSeqs], seq_pick;
  Ctx4 cx;
  cx.p = p;
  cx.h = task % p.H;
  cx.col0 = slab * C::J;
  cx.eA = G ? __expf(p.A[cx.h]) : 1.0f;
  const size_t mat = (size_t)C::DK * p.dv;  // elements of one state
  if (p.split) {
    // task = (b, part, h); part j covers tokens [j part_len, (j+1) part_len) of sequence b
    const int np = p.split == 1 ? p.nparts - 1 : p.nparts;
    const int part = (task / p.H) % np;
    cx.b = task / p.H / np;
    cx.bh = cx.b * p.H + cx.h;
    const long long start = (long long)part * p.part_len;
    cx.tok0 = (long long)cx.b * p.T + start;
    cx.T = (int)max(0LL, min((long long)p.part_len, (long long)p.T - start));
    if (p.split == 1) {
      cx.v_on = cx.col0 < p.dv;
      cx.o_on = false;
      cx.ident = cx.col0 < p.dv ? -1 : cx.col0 - p.dv;
      cx.s0 = nullptr;
      cx.s0_ld = 0;
      cx.st_ld = p.dv + C::DK;
      cx.st = p.ws_trans + ((size_t)(cx.b * (p.nparts - 1) + part) * p.H + cx.h) * C::DK * cx.st_ld + cx.col0;
    } else {
      cx.v_on = cx.o_on = true;
      cx.ident = -1;
      cx.s0_ld = cx.st_ld = p.dv;
      cx.s0 = p.ws_in + ((size_t)(cx.b * p.nparts + part) * p.H + cx.h) * mat + cx.col0;
      cx.st = (part == p.nparts - 1 && p.S_T) ? p.S_T + (size_t)cx.bh * mat + cx.col0 : nullptr;
    }
  } else {
    cx.b = __builtin_amdgcn_readfirstlane(seq_by_length_rank(p.cu, p.B, p.T, task / p.H, seq_lens, &seq_pick));
    cx.bh = cx.b * p.H + cx.h;
    seq_range(p, cx.b, cx.tok0, cx.T);
    cx.v_on = cx.o_on = true;
    cx.ident = -1;
    cx.s0_ld = cx.st_ld = p.dv;
    cx.s0 = p.S0 ? p.S0 + (size_t)cx.bh * mat + cx.col0 : nullptr;
    cx.st = p.S_T ? p.S_T + (size_t)cx.bh * mat + cx.col0 : nullptr;
  }
  cx.nchunks = (cx.T + CS - 1) / CS;
  // T's upper-right 16x16 block is read as zeros and never written
  for (int i = tid; i < 2 * CS * C::LDC; i += C::NT) (&sm.t[0][0])[i] = (h16)0.0f;
  // Waves w and w + 4 share a SIMD: the two state waves (SIMDs 0 and 1) and the
  // L/T and P waves (SIMDs 2 and 3) each share one with a scan wave.  The scan
  // and state waves carry the step's critical path, so they issue first.
  if (wave >= 4) {
    __builtin_amdgcn_s_setprio(3);
    run_role<C, SCAN, G>(sm, cx, snap, lane, wave - 4);
  } else if (wave < 2) {
    __builtin_amdgcn_s_setprio(3);
    run_role<C, STATE, G>(sm, cx, snap, lane, wave);
  } else if (wave == 2) {
    run_role<C, SOLVE, G>(sm, cx, snap, lane, 0);
  } else {
    run_role<C, PMAT, G>(sm, cx, snap, lane, 0);
  }
}

template <int DK, int NST>
hipError_t launch_pipe(const PrefillParams& p, const SnapList& snap, hipStream_t s) {
  using C = Cfg4<DK, NST>;
  const int tasks = p.B * p.H * (p.split == 1 ? p.nparts - 1 : p.split == 2 ? p.nparts : 1);
  const unsigned grid = (unsigned)(tasks * ((p.split == 1 ? p.dv + DK : p.dv) / C::J));
  if (p.z) hipLaunchKernelGGL((kda_prefill_pipe_kernel<C, true>), dim3(grid), dim3(C::NT), 0, s, p, snap);
  else hipLaunchKernelGGL((kda_prefill_pipe_kernel<C, false>), dim3(grid), dim3(C::NT), 0, s, p, snap);
  return hipGetLastError();
}


// ---- two-stage prefill, stage 2: the chain kernel ---------------------------------------
// The records of stage 1 (kda_prep.hip: KG, QG, T, -P T and -KH^T as
// matrix-core fragments, and gamma) and the V slab stream into LDS by
// direct-to-LDS loads from two loader waves: each record's state part (KG, T,
// -KH^T, gamma, with the V slab) into one ring and its output part (QG, -P T)
// into another, every part LAT steps ahead of the step that reads it.
// The state waves run only the serial part, the output waves the output:
//   Xn = KG S - V,  Un = T Xn,  S' = gamma S + (-KH)^T Un,
//   O^T = S^T QG^T + Xn^T (-P T)^T    (P U = -(P T) Xn, the product formed in stage 1)
// One barrier per chunk.  Every chunk is one item: stage 1 needs no regrouping.
template <int DK_, int NST_>
struct CfgC {
  static constexpr int DK = DK_, NST = NST_, J = 16 * NST;
  static constexpr int NKT = DK / 16, NKB = DK / 32;
  using R = ChunkRec<DK>;
  static constexpr int RECS = (R::OUT + 1023) / 1024;             // 1 KB transfers: a record's state part
  static constexpr int RECO = (R::BYTES - R::OUT + 1023) / 1024;  // ... and its output part
  static constexpr int VROW = J * 2;                              // bytes of one token's row of the V slab
  static constexpr int VK = CS * VROW / 1024;                     // 1 KB transfers per V slab
  static constexpr int NKS = RECS + VK, NKO = RECO;               // transfers into a state / output slot
  static constexpr int SLOTS = NKS * 1024, SLOTO = NKO * 1024;
  static constexpr int NL = 2;        // loader waves
  static constexpr int LAT = 3;       // steps each transfer has to land
  static constexpr int RING = LAT + 1;  // slots of each ring: LAT in flight, one being read
  static constexpr int NW = 2 * NST + NL, NT = 64 * NW;  // state, output and loader waves
  static constexpr int HAND = (NKB + 2) * 1024;        // state -> output handoff per wave: Sf, Xn, 1/scale
  // transfers of loader lw per state part, per output part, per step
  static constexpr int nks_of(int lw) { return (NKS - lw + NL - 1) / NL; }
  static constexpr int nko_of(int lw) { return (NKO - lw + NL - 1) / NL; }
  static constexpr int nk_of(int lw) { return nks_of(lw) + nko_of(lw); }
  static_assert(VROW % 16 == 0 && (CS * VROW) % 1024 == 0, "V slab transfers");
  static_assert((R::BYTES - R::OUT) % 1024 == 0 && R::OUT % 16 == 0, "output part: whole transfers");
  static_assert(LAT * (nks_of(0) + nko_of(0)) <= 63, "transfers in flight fit the wait counter");
};

// Barriers each wave of a chain workgroup passes over nchunks chunks.
__device__ __forceinline__ int chain_barriers(int nchunks) { return nchunks > 0 ? nchunks + 2 : 1; }

template <class C>
struct SmemC {
  alignas(16) char sring[C::RING][C::SLOTS];  // state parts (with V) of chunk c in slot c % RING
  alignas(16) char oring[C::RING][C::SLOTO];  // output parts
  alignas(16) char hand[2][C::NST][C::HAND];  // by chunk parity
  alignas(16) float scol[C::NST][16];         // state waves: 1/scale of each of their columns
};

// s_waitcnt immediate for "at most n vector memory operations outstanding".
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

typedef __attribute__((address_space(3))) void lds_void;

// Where a task's chunks lie.
struct ChainSrc {
  const char* rec;     // record of the task's first chunk
  long long rec_step;  // bytes between the records of consecutive chunks
  const char* v;       // the slab's V at the task's first token
  int vrow;            // bytes between V token rows
  int nchunks, T;
};

// Loader wave LW's share (every NL-th 1 KB transfer) of chunk c's state part
// and V slab, or of its output part, into `slot`.  A chunk past the end is a
// zero-length range (reads zeros), so every step has the same number of
// transfers in flight and one wait count fits all steps.
template <class C, int LW>
__device__ __forceinline__ void chain_issue_state(char* slot, const ChainSrc& q, int c, int lane) {
  const bool on = c < q.nchunks;
  const int rows = on ? min(CS, q.T - c * CS) : 0;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(q.rec + (on ? (long long)c * q.rec_step : 0), on ? C::R::OUT : 0);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(q.v + (on ? (long long)c * CS * q.vrow : 0), rows * q.vrow);
#pragma unroll
  for (int i = LW; i < C::NKS; i += C::NL) {
    if (i < C::RECS) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)(slot + 1024 * i), 16, 16 * lane, 1024 * i, 0, 0);
    } else {
      // V rows of VROW bytes, LPR lanes each: LDS holds the slab row-major
      constexpr int LPR = C::VROW / 16;
      const int row = (i - C::RECS) * (64 / LPR) + lane / LPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(slot + 1024 * i), 16, row * q.vrow + 16 * (lane % LPR),
                                               0, 0, 0);
    }
  }
}
template <class C, int LW>
__device__ __forceinline__ void chain_issue_out(char* slot, const ChainSrc& q, int c, int lane) {
  const bool on = c < q.nchunks;
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc(q.rec + C::R::OUT + (on ? (long long)c * q.rec_step : 0), on ? C::R::BYTES - C::R::OUT : 0);
#pragma unroll
  for (int i = LW; i < C::NKO; i += C::NL)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)(slot + 1024 * i), 16, 16 * lane, 1024 * i, 0, 0);
}

// The state waves read chunk c's state part during step c - 1 (chunk 0's
// before barrier 0, after an opening barrier) and the output waves its output
// part during step c.  At barrier n the loaders refill the slots of chunk n's
// state part and chunk n - 1's output part with the state part of chunk
// n + LAT + 1 and the output part of chunk n + LAT, both needed LAT barriers
// later; every wait leaves the newest LAT - 1 steps' transfers in flight.
template <class C, int LW>
__device__ void chain_loader(SmemC<C>& sm, const ChainSrc& q, int lane) {
  static_assert(C::LAT >= 2 && C::RING == C::LAT + 1, "LAT slots in flight plus the one being read");
  constexpr int L = C::LAT;
  constexpr int WAIT = vmcnt_imm((L - 1) * C::nk_of(LW));
  if (q.nchunks <= 0) {
    block_sync_lds();  // the closing barrier of every wave
    return;
  }
  // in the order the parts are needed: state 0, then output 0 and state 1
  // (barrier 0), then output c and state c + 1 (barrier c)
  chain_issue_state<C, LW>(sm.sring[0], q, 0, lane);
#pragma unroll
  for (int c = 0; c < L; ++c) {
    chain_issue_out<C, LW>(sm.oring[c], q, c, lane);
    chain_issue_state<C, LW>(sm.sring[c + 1], q, c + 1, lane);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(L * C::nk_of(LW)));  // state 0
  block_sync_lds();                                           // the opening barrier
  __builtin_amdgcn_s_waitcnt(WAIT);
  for (int n = 0; n < q.nchunks; ++n) {
    block_sync_lds();  // barrier n
    chain_issue_out<C, LW>(sm.oring[(n + L) % C::RING], q, n + L, lane);
    chain_issue_state<C, LW>(sm.sring[(n + L + 1) % C::RING], q, n + L + 1, lane);
    __builtin_amdgcn_s_waitcnt(WAIT);
  }
  block_sync_lds();  // the closing barrier of every wave
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
}

template <class C>
__device__ __forceinline__ f16x8 slot_frag(const char* lb, int off, int f) {
  return *reinterpret_cast<const f16x8*>(lb + off + f * 1024);
}

// max(|a|, |b|, |c|): one instruction where the operands come straight from
// arithmetic in the same block (known canonical, so no quieting maximum is added)
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)), __builtin_fabsf(c));
}

// max |S| over this lane's values: four chains over the tiles' rows
template <class C>
__device__ __forceinline__ float lane_smax(const StateRegs<C>& R) {
  static_assert(C::NKT >= 3, "three tiles at least");
  float m[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = max3_abs(R.S[0][r], R.S[1][r], R.S[2][r]);
#pragma unroll
    for (int i = 3; i < C::NKT; i += 2) m[r] = max3_abs(m[r], R.S[i][r], R.S[i + 1 < C::NKT ? i + 1 : i][r]);
  }
  return max3_abs(m[0], m[1], max3_abs(m[2], m[3], m[3]));
}

template <class C>
__device__ __forceinline__ void pack_sf(StateRegs<C>& R) {
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) R.Sf[kb] = stack2(R.S[2 * kb], R.S[2 * kb + 1]);
}

// A state wave's operands of one chunk, read from the chunk's ring slot.
template <class C>
struct ChainFrags {
  f16x8 A[2][C::NKB], Tf[2], KH[C::NKT];  // KG, T and -KH^T fragments
  f32x4 gam[C::NKT];                      // gamma of rows 16 i + 4g ..
  s16x4 va[2];                            // V as bf16 A operands: token 16 rt + n, columns 4g .. 4g + 3
  f32x4 x0[2];                            // -V * sc in the C layout of X (tokens 16 rt + 4g + r, column n)
};

template <class C>
__device__ __forceinline__ void chain_fetch(const SmemC<C>& sm, int c, int w, int lane, ChainFrags<C>& F) {
  using RC = typename C::R;
  const char* sb = sm.sring[c % C::RING];
  const char* lb = sb + 16 * opaque(lane);
  const int gg = opaque(lane / 16), nn = opaque(lane % 16);
  // V first: the column-scale check that follows waits only for it
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    F.va[rt] = *reinterpret_cast<const s16x4*>(sb + C::RECS * 1024 + (16 * rt + nn) * C::VROW + (16 * w + 4 * gg) * 2);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) F.A[rt][kb] = slot_frag<C>(lb, RC::KG, rt * C::NKB + kb);
    F.Tf[rt] = slot_frag<C>(lb, RC::TT, rt);
  }
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) F.KH[i] = slot_frag<C>(lb, RC::KH, i);
#pragma unroll
  for (int i = 0; i < C::NKT; ++i) F.gam[i] = *reinterpret_cast<const f32x4*>(sb + RC::GAM + (16 * i + 4 * gg) * 4);
}

// -sc times the identity as a bf16 B operand (lane (g, n) holds rows 4g .. 4g + 3
// of column n): V times it is -V * sc in the C layout, exactly (sc is a power of two).
__device__ __forceinline__ s16x4 neg_scaled_eye(float sc, int g, int n) {
  const uint32_t h = __float_as_uint(-sc) >> 16;
  const int j = n - 4 * g;  // the row of this lane's four that is on the diagonal, if any
  const uint32_t w0 = j == 0 ? h : j == 1 ? h << 16 : 0u;
  const uint32_t w1 = j == 2 ? h : j == 3 ? h << 16 : 0u;
  return __builtin_bit_cast(s16x4, u32x2{w0, w1});
}

// State wave w: the serial part of every chunk -- Xn = KG S - V, Un = T Xn,
// S' = gamma S + (-KH)^T Un -- and nothing else.  The fp16 S and Xn it used and
// the column scales go to output wave w through the handoff buffer of the
// chunk's parity.  Everything that does not depend on the new state -- reading
// the next chunk's operands out of LDS, and -V * sc on the matrix cores -- is
// issued right after the state update, so it overlaps the matrix-core
// products; the state's maximum, fp16 copy and column scale for the next chunk
// follow, ahead of the barrier.
template <class C>
__device__ void chain_state(SmemC<C>& sm, const Ctx4& cx, const SnapList& snap, int pos0, int w, int lane) {
  const PrefillParams& p = cx.p;
  StateRegs<C> R;
  const int g = lane / 16, n16 = lane % 16;
  {
    const int col = 16 * w + n16;
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] = (f32x4)0.0f;
    if (cx.s0) {
#pragma unroll
      for (int i = 0; i < C::NKT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) R.S[i][r] = cx.s0[(size_t)(16 * i + 4 * g + r) * cx.s0_ld + col];
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    R.sc = 1.0f;
    R.usc = (f32x4)1.0f;
  }
  s16x4 neye = neg_scaled_eye(R.sc, g, n16);
  int ns = 0;  // next listed position (positions up to pos0 belong to earlier blocks)
  while (ns < p.nsnap && snap.pos[ns] <= pos0) ++ns;
  float ms = lane_smax<C>(R);
  pack_sf<C>(R);
  // -V * sc of the next chunk, then its column scale: keep the scaled column
  // maximum of S and V within [2^-4, 2^4] (rarely changed; capped at 2^64 so a
  // column that has decayed to nothing with no value input never scales to
  // infinity, where 0 * inf would be NaN).  A lane whose own maximum is in range
  // proves its column is not too large, and not too small either unless all
  // four lanes of the column are small, so the per-column maximum is formed
  // only when some lane is out of range.
  auto start_chunk = [&](ChainFrags<C>& F) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) F.x0[rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(F.va[rt], neye, (f32x4)0.0f, 0, 0, 0);
    const float lm = max3_abs(max3_abs(ms, F.x0[0][0], F.x0[0][1]), max3_abs(F.x0[0][2], F.x0[0][3], F.x0[1][0]),
                              max3_abs(F.x0[1][1], F.x0[1][2], F.x0[1][3]));
    // (bitwise operators: straight-line compares, no branches)
    const bool room = R.sc < 0x1p64f;
    if (__builtin_amdgcn_ballot_w64((lm > 16.0f) | ((lm < 0.0625f) & room)) == 0) return;
    const float m = column_max(lm);
    const bool bad = (m > 16.0f) | ((m > 0.0f) & (m < 0.0625f) & room);
    if (__builtin_amdgcn_ballot_w64(bad) == 0) return;
    float f = 1.0f;
    if (bad) {
      const int ex = __builtin_amdgcn_frexp_expf(m);  // m = frac * 2^ex, frac in [0.5, 1)
      f = fminf(__builtin_amdgcn_ldexpf(1.0f, -ex), 0x1p64f / R.sc);  // powers of two: exact
    }
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] *= f;
    F.x0[0] *= f;
    F.x0[1] *= f;
    R.sc *= f;
    neye = neg_scaled_eye(R.sc, g, n16);
    if (g == 0) sm.scol[w][n16] = __builtin_amdgcn_rcpf(R.sc);  // output rows are columns 4g .. 4g + 3
    wave_lds_sync();
    R.usc = *reinterpret_cast<const f32x4*>(&sm.scol[w][4 * g]);
    pack_sf<C>(R);
  };
  ChainFrags<C> F;
  if (cx.nchunks > 0) {
    block_sync_lds();  // the opening barrier: chunk 0's state part is in its slot
    chain_fetch<C>(sm, 0, w, lane, F);
    start_chunk(F);
  }
  for (int n = 0; n < cx.nchunks; ++n) {
    block_sync_lds();  // chunk n + 1's state part is in its slot; the handoff of chunk n - 2 is free
    const Item it = {n, n, 0, chunk_end(n, cx.T), CS};
    char* hb = sm.hand[n & 1][w] + 16 * lane;
    f32x4 X[2] = {F.x0[0], F.x0[1]};
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) X[rt] = mma16(F.A[rt][kb], R.Sf[kb], X[rt]);
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) *reinterpret_cast<f16x8*>(hb + kb * 1024) = R.Sf[kb];
    *reinterpret_cast<f32x4*>(hb + (C::NKB + 1) * 1024) = R.usc;
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] *= F.gam[i];
    const f16x8 xf = stack2(X[0], X[1]);
    f32x4 U[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) U[rt] = mma16(F.Tf[rt], xf, (f32x4)0.0f);
    const f16x8 uf = stack2(U[0], U[1]);
#pragma unroll
    for (int i = 0; i < C::NKT; ++i) R.S[i] = mma16(F.KH[i], uf, R.S[i]);
    *reinterpret_cast<f16x8*>(hb + C::NKB * 1024) = xf;
    // (after the last chunk this reads a slot the loaders filled with zeros: no
    // branch, so the maxima below see the products' results directly)
    chain_fetch<C>(sm, n + 1, w, lane, F);
    ms = lane_smax<C>(R);
    pack_sf<C>(R);
    start_chunk(F);
    if (ns < p.nsnap && snap.pos[ns] == pos0 + n * CS + it.hi) {
      store_state<C>(p.snaps + ((size_t)cx.bh * p.nsnap + ns) * C::DK * p.dv + cx.col0, R, p.dv, w, lane);
      ++ns;
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }
  }
  block_sync_lds();  // the last handoff is complete
  if (cx.st) store_state<C>(cx.st, R, cx.st_ld, w, lane);
}

// Lane l of the result takes x from lane l - 1 (SHL false) or l + 1 (SHL true)
// of its 16-lane row.
template <bool SHL>
__device__ __forceinline__ f32x4 row_shift1(const f32x4& x) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_update_dpp(0u, u[i], SHL ? 0x101 : 0x111, 0xf, 0xf, true);
  return __builtin_bit_cast(f32x4, r);
}

// Output wave r: tokens 16 r .. 16 r + 15 of chunk n - 1 during step n, for every
// column of the slab, from the handoffs of both state waves and the chunk's QG
// and -P T fragments of those tokens, read into registers during step n - 1
// (its slot is refilled in step n):
//   O^T = S^T QG^T + Xn^T (-P T)^T.
// Lane (g, n) ends with columns 16 w + 4g .. + 3 of token 16 r + n for state
// wave w.  A shift by one lane within each 16-lane row gives each even lane the
// other half of its token's row and each odd lane its neighbour's, so that every
// store instruction writes whole rows of the slab: 8 tokens per instruction.
template <class C>
__device__ void chain_output(SmemC<C>& sm, const Ctx4& cx, int r, int lane) {
  static_assert(C::NST == 2, "a token's row of the slab: the columns of two state waves");
  using RC = typename C::R;
  const PrefillParams& p = cx.p;
  const int g = opaque(lane / 16), n = opaque(lane % 16);
  const bool odd = (n & 1) != 0;
  f16x8 Q[C::NKB], Pf, Pl;
  auto emit = [&](int c) {  // the output of chunk c
    f32x4 O[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const char* hb = sm.hand[c & 1][w] + 16 * lane;
      f16x8 Sf[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) Sf[kb] = *reinterpret_cast<const f16x8*>(hb + kb * 1024);
      const f16x8 xf = *reinterpret_cast<const f16x8*>(hb + C::NKB * 1024);
      const f32x4 usc = *reinterpret_cast<const f32x4*>(hb + (C::NKB + 1) * 1024);
      O[w] = (f32x4)0.0f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) O[w] = mma16(Sf[kb], Q[kb], O[w]);
      O[w] = mma16(xf, Pl, O[w]);
      O[w] = mma16(xf, Pf, O[w]) * usc;
    }
    // even tokens: the even lane's own first half and the odd lane's copy of the
    // second half; odd tokens: the odd lane's own second half and the even
    // lane's copy of the first half
    const f32x4 prev1 = row_shift1<false>(O[1]), next0 = row_shift1<true>(O[0]);
    const f32x4 a = odd ? prev1 : O[0];
    const f32x4 b = odd ? O[1] : next0;
    const int col = (odd ? 16 : 0) + 4 * g;
    const int te = 16 * r + (n & ~1), to = 16 * r + (n | 1);
    const int rows = chunk_end(c, cx.T);
    const int esz = p.o_f32 ? 4 : 2;
    const int rs = p.H * p.dv * esz;
    char* ob = static_cast<char*>(p.o) + (((size_t)(cx.tok0 + c * CS) * p.H + cx.h) * p.dv + cx.col0) * esz;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(ob, rows * rs);  // tokens past the end: dropped
    if (p.o_f32) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), rsrc, te * rs + col * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), rsrc, to * rs + col * 4, 0, 0);
    } else {
      // reinterpret whole vectors (single elements are miscompiled)
      const bf16x4 ah = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
      const bf16x4 bh = {(__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ah), rsrc, te * rs + col * 2, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, bh), rsrc, to * rs + col * 2, 0, 0);
    }
  };
  if (cx.nchunks > 0) block_sync_lds();  // the opening barrier
  for (int n = 0; n < cx.nchunks; ++n) {
    block_sync_lds();  // chunk n's output part is in its slot
    if (n > 0) emit(n - 1);
    const char* lb = sm.oring[n % C::RING] + 16 * opaque(lane);
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) Q[kb] = slot_frag<C>(lb, RC::QG - RC::OUT, r * C::NKB + kb);
    Pf = slot_frag<C>(lb, RC::PP - RC::OUT, r);
    Pl = slot_frag<C>(lb, RC::PL - RC::OUT, r);
  }
  block_sync_lds();
  if (cx.nchunks > 0) emit(cx.nchunks - 1);
}

// Workgroup bi of a chain launch over G workgroups (one per slab task).  Waves
// past the chain's NW (a launch shared with stage 1 has more) only take part in
// its barriers.
template <class C>
__device__ __forceinline__ void chain_block(SmemC<C>& sm, int* seq_lens, int* seq_pick, const PrefillParams& p,
                                            const SnapList& snap, int G, int bi) {
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  int task, slab;
  task_of_index(p.dv / C::J, G, bi, task, slab);
  Ctx4 cx;
  cx.p = p;
  cx.h = task % p.H;
  cx.col0 = slab * C::J;
  cx.eA = 1.0f;
  cx.b = __builtin_amdgcn_readfirstlane(seq_by_length_rank(p.cu, p.B, p.T, task / p.H, seq_lens, seq_pick));
  cx.bh = cx.b * p.H + cx.h;
  long long slot0;
  int pos0 = 0;
  if (p.cu) {
    seq_range(p, cx.b, cx.tok0, cx.T);
    slot0 = cx.tok0 / CS + cx.b;
  } else {
    pos0 = p.rec_c0 * CS;
    cx.tok0 = (long long)cx.b * p.T + pos0;
    cx.T = max(0, min(p.T - pos0, p.rec_nc * CS));
    slot0 = (long long)cx.b * p.rec_nc;
  }
  cx.nchunks = (cx.T + CS - 1) / CS;
  cx.v_on = cx.o_on = true;
  cx.ident = -1;
  cx.s0_ld = cx.st_ld = p.dv;
  const size_t mat = (size_t)C::DK * p.dv;
  cx.s0 = p.S0 ? p.S0 + (size_t)cx.bh * mat + cx.col0 : nullptr;
  cx.st = p.S_T ? p.S_T + (size_t)cx.bh * mat + cx.col0 : nullptr;
  // waves 0 .. NST-1: state (SIMDs 0 and 1), NST .. 2 NST-1: output (SIMDs 2
  // and 3), then the two loaders, which share the state waves' SIMDs and give
  // way to them
  if (wave >= C::NST && wave < 2 * C::NST) {
    __builtin_amdgcn_s_setprio(3);
    chain_state<C>(sm, cx, snap, pos0, wave - C::NST, lane);
  } else if (wave < C::NST) {
    chain_output<C>(sm, cx, wave, lane);
  } else if (wave < C::NW) {
    ChainSrc q;
    q.rec = p.rec + (slot0 * p.H + cx.h) * C::R::BYTES;
    q.rec_step = (long long)p.H * C::R::BYTES;
    q.vrow = p.H * p.dv * 2;
    q.v = static_cast<const char*>(p.v) + ((cx.tok0 * p.H + cx.h) * p.dv + cx.col0) * 2;
    q.nchunks = cx.nchunks;
    q.T = cx.T;
    if (wave == 2 * C::NST) chain_loader<C, 0>(sm, q, lane);
    else chain_loader<C, 1>(sm, q, lane);
  } else {
    for (int n = chain_barriers(cx.nchunks); n > 0; --n) block_sync_lds();  // as many barriers as every role
  }
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void kda_chain_kernel(PrefillParams p, SnapList snap) {
  __shared__ SmemC<C> sm;
  __shared__ int seq_lens[kMaxRankedSeqs], seq_pick;
  chain_block<C>(sm, seq_lens, &seq_pick, p, snap, gridDim.x, blockIdx.x);
}

// One launch for two blocks of chunks of a long batch: workgroups 0 .. G-1 run
// the chain over block k (records written by the previous launch), the rest
// run stage 1 of block k + 1 into the other record buffer, eight records each.
// The chain's workgroups come first, so they are placed first (one per
// compute unit); stage 1 runs on the compute units the chain leaves free and
// refills them as its workgroups finish.  Every workgroup reserves the larger
// of the two roles' LDS, which for stage 1 is that of eight waves.
constexpr int kFusedWaves = 8;
template <class C, class PC, bool G>
__global__ __launch_bounds__(64 * kFusedWaves, 1) void kda_chain_prep_kernel(PrefillParams pc, PrefillParams pp,
                                                                           SnapList snap, int chain_grid,
                                                                           long long nrec) {
  static_assert(C::NW <= kFusedWaves, "chain waves fit the launch");
  constexpr size_t LC = sizeof(SmemC<C>), LP = kFusedWaves * sizeof(prep::PrepLds<PC>);
  __shared__ __attribute__((aligned(16))) char smem[LC > LP ? LC : LP];
  __shared__ int seq_lens[kMaxRankedSeqs], seq_pick;
  if ((int)blockIdx.x < chain_grid) {
    chain_block<C>(*reinterpret_cast<SmemC<C>*>(smem), seq_lens, &seq_pick, pc, snap, chain_grid, blockIdx.x);
  } else {
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const long long rec = (long long)(blockIdx.x - chain_grid) * kFusedWaves + wave;
    if (rec < nrec) prep::prep_record<PC, G>(pp, rec, reinterpret_cast<prep::PrepLds<PC>*>(smem)[wave], lane);
  }
}

template <int DK, int NST>
hipError_t launch_chain(const PrefillParams& p, const SnapList& snap, hipStream_t s) {
  using C = CfgC<DK, NST>;
  const long long grid = (long long)p.B * p.H * (p.dv / C::J);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((kda_chain_kernel<C>), dim3((unsigned)grid), dim3(C::NT), 0, s, p, snap);
  return hipGetLastError();
}

template <int DK, int NST>
hipError_t launch_chain_prep(const PrefillParams& pc, const PrefillParams& pp, long long nslots, const SnapList& snap,
                             hipStream_t s) {
  using C = CfgC<DK, NST>;
  using PC = prep::PCfg<DK>;
  const long long chain_grid = (long long)pc.B * pc.H * (pc.dv / C::J);
  const long long nrec = nslots * pp.H;
  const long long grid = chain_grid + (nrec + kFusedWaves - 1) / kFusedWaves;
  if (chain_grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (pp.z)
    hipLaunchKernelGGL((kda_chain_prep_kernel<C, PC, true>), dim3((unsigned)grid), dim3(64 * kFusedWaves), 0, s, pc, pp,
                       snap, (int)chain_grid, nrec);
  else
    hipLaunchKernelGGL((kda_chain_prep_kernel<C, PC, false>), dim3((unsigned)grid), dim3(64 * kFusedWaves), 0, s, pc,
                       pp, snap, (int)chain_grid, nrec);
  return hipGetLastError();
}
}  // namespace

bool prefill_pipe_supported(int io_dtype, int dk, int dv, int chunk, int H) {
  // per-chunk buffer ranges (32 tokens of every head) must fit 31 bits
  const long long chunk_bytes = (long long)CS * H * (dk > dv ? dk : dv) * 4;
  return io_dtype == 1 && (dk == 64 || dk == 128) && dv % 32 == 0 && (chunk == 32 || chunk == 64) &&
         chunk_bytes < (1LL << 31);
}

hipError_t launch_prefill_pipe(const PrefillParams& p, const SnapList& snap, hipStream_t s) {
  if (p.dk == 128) return launch_pipe<128, 2>(p, snap, s);
  if (p.dk == 64) return launch_pipe<64, 2>(p, snap, s);
  return hipErrorInvalidValue;
}

bool prefill_chain_supported(int io_dtype, int dk, int dv, int chunk, int H) {
  return prefill_pipe_supported(io_dtype, dk, dv, chunk, H);
}

hipError_t launch_prefill_chain(const PrefillParams& p, const SnapList& snap, hipStream_t s) {
  if (p.dk == 128) return launch_chain<128, 2>(p, snap, s);
  if (p.dk == 64) return launch_chain<64, 2>(p, snap, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_chain_prep(const PrefillParams& pc, const PrefillParams& pp, long long nslots,
                                     const SnapList& snap, hipStream_t s) {
  if (pc.dk == 128) return launch_chain_prep<128, 2>(pc, pp, nslots, snap, s);
  if (pc.dk == 64) return launch_chain_prep<64, 2>(pc, pp, nslots, snap, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
