// libkda C ABI: argument validation, dispatch and error mapping.
//
// Every check runs before any HIP call, so invalid arguments return a status
// without touching the device.  Kernels are enqueued on the caller's stream and
// the calls return without synchronising.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kVersion = 200;  // 0.2.0

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// A C caller may pass any int where the header says kda_dtype or kda_status;
// reading such a value as the C++ enum type is undefined, so it is read as the
// integer it is.
// (Taken by reference: passing it by value would already read it as the enum.)
template <typename E>
int raw_enum(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum size");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}
bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }
int io_of(int d) { return d == KDA_BF16 ? 1 : 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Element counts fit in size_t and every row index used by the kernels fits in
// an int64; the kernels index tokens with 64-bit arithmetic.
bool sizes_ok(long long B, long long T, long long H, long long dk, long long dv) {
  const long long lim = (1LL << 40);
  if (B * H > (1LL << 26)) return false;
  if (B * T * H > lim / 128) return false;
  (void)dk;
  (void)dv;
  return true;
}

// Prefill kernel choice.  bf16 q/k/v with d_k in {64,128}, d_v % 32 == 0 and
// chunk 32 or 64 run 32-token chunks: by the two-stage prefill (chunk records
// for all chunks at once, then the chain), or by the single-kernel pipeline
// where the records' workspace cannot be had (and for split calls).  The
// generic 16x16-tile kernel serves everything else, with 16 state columns per
// workgroup unless 32-column slabs still give one workgroup per compute unit.
enum PrefillImpl { IMPL_GENERIC, IMPL_PIPE, IMPL_CHAIN };
struct PrefillPlan {
  PrefillImpl impl;
  int slab;
};

#ifdef KDA_TEST_HOOKS
// Test builds only (libkda_testhooks.so): a process-wide override of the kernel
// choice, so tests can run the generic kernel on shapes the pipeline kernel
// would take and pick its slab width.  The product library has no such state.
int g_force_impl = -1;  // -1: the library's choice; 0: generic; 1: pipeline; 2: two-stage
int g_force_slab = 0;   // 0: the library's choice; 16 or 32
size_t g_rec_cap = 0;   // 0: the library's cap on the two-stage workspace
int g_force_overlap = -1;  // -1: the library's choice; 0: never; 1: for every blocked batch
#endif

PrefillPlan plan_prefill(int B, int H, int dk, int dv, int chunk, int io) {
  int impl = -1, forced = 0;
#ifdef KDA_TEST_HOOKS
  impl = g_force_impl;
  if ((g_force_slab == 16 || g_force_slab == 32) && dv % g_force_slab == 0) forced = g_force_slab;
#endif
  if (impl != 0 && !forced && kda::prefill_pipe_supported(io, dk, dv, chunk, H))
    return {impl == 1 ? IMPL_PIPE : IMPL_CHAIN, 32};
  if (forced) return {IMPL_GENERIC, forced};
  if (io == 1 && dv % 32 == 0 && (long long)B * H * (dv / 32) >= 256) return {IMPL_GENERIC, 32};
  return {IMPL_GENERIC, 16};
}

// ---- sequence split ----------------------------------------------------------------
// The pipelined kernel serves one (b, h, 32-column slab) chain per workgroup and
// keeps one workgroup per compute unit, so with few chains most of the GPU
// idles.  A split prefill cuts every sequence into parts of whole 32-token
// chunks: pass 1 runs parts 0..P-2 from a zero state over d_v + d_k columns
// (their contributions and transitions), a combine kernel chains them into each
// part's incoming state, and pass 2 reruns all P parts from those states.
constexpr int kMaxParts = 1024;
struct SplitShape {
  int parts, part_len;  // part_len: tokens per part, a multiple of 32
};

SplitShape split_shape_for(int T, int P) {
  const int nch = (T + 31) / 32;
  if (nch <= 1 || P <= 1) return {1, T};
  const int pc = (nch + P - 1) / P;  // chunks per part
  return {(nch + pc - 1) / pc, 32 * pc};
}

// Combine cost in pipeline steps (about 2 us each): the chain costs about two
// per part (about 4 us each); the tree about three per level plus the apply.
double combine_steps(int P) {
  if (P < kda::kTreeParts) return 2.0 * (P - 1);
  int levels = 0;
  for (int d = 1; d < P - 1; d *= 2) ++levels;
  return 3.0 * (levels + 1);
}

// The part count with the smallest modelled time.  The model counts pipeline
// steps: a launch of G workgroups on `cus` compute units runs ceil(G / cus)
// rounds of (chunks per part + 3) steps; the combine as above, and the two
// extra launches about two steps.  The single pass it is weighed against is
// the two-stage prefill where that is what one part runs (its chain steps
// about 0.42 pipeline steps, after stage 1 at about 160 records per pipeline
// step on 256 compute units), else the pipeline.  A split is taken only when
// it models at least 25% (two-stage) or 10% (pipeline) faster.
size_t split_ws_bytes(int B, int H, int dk, int dv, int P);

SplitShape split_shape_auto(int B, int T, int H, int dk, int dv, int cus, bool two_stage, size_t max_ws = SIZE_MAX) {
  const int nch = (T + 31) / 32;
  const long long bh = (long long)B * H, ns = dv / 32, nsa = (dv + dk) / 32;
  auto rounds = [&](long long g) { return (double)((g + cus - 1) / cus); };
  const double single = two_stage ? rounds(bh * ns) * (nch + 3) * 0.42 + (double)bh * nch / (160.0 * cus / 256) + 2.0
                                  : rounds(bh * ns) * (nch + 3);
  SplitShape best{1, T};
  double best_cost = (two_stage ? 0.75 : 0.9) * single;
  for (int P = 2; P <= nch && P <= kMaxParts; ++P) {
    const SplitShape sh = split_shape_for(T, P);
    if (sh.parts != P || split_ws_bytes(B, H, dk, dv, P) > max_ws) continue;
    const double cost = (rounds(bh * (P - 1) * nsa) + rounds(bh * P * ns)) * (sh.part_len / 32 + 3) +
                        combine_steps(P) + 2.0;
    if (cost < best_cost) {
      best_cost = cost;
      best = sh;
    }
  }
  return best;
}

// (N | M) of parts 0..P-2 (twice when the combine is a tree) and S_in of every part
size_t split_ws_bytes(int B, int H, int dk, int dv, int P) {
  if (P <= 1) return 0;
  const size_t trans = (size_t)(P - 1) * (dv + dk) * (P >= kda::kTreeParts ? 2 : 1);
  return (size_t)4 * B * H * dk * (trans + (size_t)P * dv);
}

// Compute units of the current device (0 on failure).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// ---- two-stage prefill: the chunk records' workspace ----------------------------------
// The records (one per sequence, head and 32-token chunk) live in a memory pool
// the library owns on each device, allocated and freed in stream order on the
// caller's stream around the two stages; the pool keeps its memory, so later
// calls reuse it without synchronising.  At most kRecCapBytes at a time: a longer
// batch of equal-length sequences runs in blocks of chunks (stage 1 then stage 2
// per block, the state carried through S_T or a pool buffer); a packed batch
// whose records exceed the cap runs on the single-kernel pipeline instead.
constexpr size_t kRecCapBytes = (size_t)1 << 30;

size_t rec_cap() {
#ifdef KDA_TEST_HOOKS
  if (g_rec_cap) return g_rec_cap;
#endif
  return kRecCapBytes;
}

constexpr int kMaxPoolDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxPoolDevices];

hipError_t pool_of_current_device(hipMemPool_t* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxPoolDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof props);
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;  // never hand memory back at synchronisation
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

int overlap_mode() {
#ifdef KDA_TEST_HOOKS
  return g_force_overlap;
#else
  return -1;
#endif
}

// Compute units of the current device (queried once per device).
std::mutex g_cus_mu;
int g_cus[kMaxPoolDevices];
hipError_t cus_of_current_device(int* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxPoolDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_cus_mu);
  if (!g_cus[dev]) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus[dev] = n > 0 ? n : 1;
  }
  *out = g_cus[dev];
  return hipSuccess;
}

// Runs the two-stage prefill.  *ran = false (nothing enqueued, hipSuccess) when
// the workspace is over the cap or cannot be allocated: the caller then runs
// the single-kernel pipeline.
//
// A batch of equal-length sequences whose records exceed the cap runs in
// blocks of chunks.  When its chain leaves at least half of the compute units
// free (few heads: one workgroup per 32-column slab, one per compute unit), the
// blocks alternate between two record buffers and each launch runs the chain
// over block k beside stage 1 of block k + 1; otherwise stage 1 and the chain
// of each block run one after the other in one buffer.
hipError_t run_two_stage(kda::PrefillParams p, const kda::SnapList& snap, hipStream_t hs, bool* ran) {
  *ran = false;
  const size_t rb = (size_t)kda::chunk_rec_bytes(p.dk);
  const size_t cap = rec_cap();
  const long long nch = ((long long)p.T + kda::kPipeChunk - 1) / kda::kPipeChunk;
  long long nslots, nc = 0, nblk = 1;
  bool overlap = false;
  if (p.cu) {
    nslots = (long long)p.T / kda::kPipeChunk + p.B + 1;  // slots cu[b] / 32 + b + c
    if ((size_t)nslots * p.H * rb > cap) return hipSuccess;
  } else {
    const size_t per_chunk = (size_t)p.B * p.H * rb;  // one chunk of every sequence
    if (per_chunk > cap) return hipSuccess;
    nc = std::max(1LL, std::min(nch, (long long)(cap / per_chunk)));
    nblk = std::max(1LL, (nch + nc - 1) / nc);
    nslots = (long long)p.B * nc;
    const int mode = overlap_mode();
    if (nblk > 1 && mode != 0) {
      int cus = 0;
      hipError_t ce = cus_of_current_device(&cus);
      if (ce != hipSuccess) return ce;
      const long long chain_grid = (long long)p.B * p.H * (p.dv / 32);
      overlap = mode == 1 || 2 * chain_grid <= cus;
    }
  }
  const int nbuf = overlap ? 2 : 1;
  const size_t rec_bytes = (size_t)nslots * p.H * rb;  // one buffer
  const size_t carry_bytes = (nblk > 1 && !p.S_T) ? (size_t)4 * p.B * p.H * p.dk * p.dv : 0;
  hipMemPool_t pool = nullptr;
  hipError_t e = pool_of_current_device(&pool);
  if (e != hipSuccess) return e;
  void* ws = nullptr;
  if (hipMallocFromPoolAsync(&ws, nbuf * rec_bytes + carry_bytes, pool, hs) != hipSuccess || !ws) {
    (void)hipGetLastError();  // out of memory here is not an error of the call
    return hipSuccess;
  }
  *ran = true;
  const float* S0 = p.S0;
  float* S_T = p.S_T;
  float* carry = S_T ? S_T : reinterpret_cast<float*>(static_cast<char*>(ws) + nbuf * rec_bytes);
  auto block = [&](long long blk) {
    kda::PrefillParams q = p;
    q.rec = static_cast<char*>(ws) + (blk % nbuf) * rec_bytes;
    q.rec_c0 = (int)(blk * nc);
    q.rec_nc = (int)nc;
    q.S0 = blk == 0 ? S0 : carry;         // each workgroup reads its slab of S0 before
    q.S_T = blk == nblk - 1 ? S_T : carry;  // it writes the same slab of S_T
    return q;
  };
  if (!overlap) {
    for (long long blk = 0; blk < nblk && e == hipSuccess; ++blk) {
      const kda::PrefillParams q = block(blk);
      e = kda::launch_prefill_prep(q, nslots, hs);
      if (e == hipSuccess) e = kda::launch_prefill_chain(q, snap, hs);
    }
  } else {
    e = kda::launch_prefill_prep(block(0), nslots, hs);
    for (long long blk = 0; blk < nblk && e == hipSuccess; ++blk) {
      if (blk + 1 < nblk) e = kda::launch_prefill_chain_prep(block(blk), block(blk + 1), nslots, snap, hs);
      else e = kda::launch_prefill_chain(block(blk), snap, hs);
    }
  }
  const hipError_t fe = hipFreeAsync(ws, hs);
  return e != hipSuccess ? e : fe;
}

// A split request: parts == 0 lets the library choose (num_cus == 0: the current
// device's compute units).
struct SplitReq {
  int parts;
  int num_cus;
  void* ws;
  size_t ws_bytes;
  bool scratch;  // the workspace is this GPU's scratch array (ws unused)
};

// ---- allocation-free split: a fixed scratch array per GPU --------------------------
// kda_chunk_fwd_split_noalloc keeps its workspace in this array.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per GPU (with that GPU current) and only that address is
// passed to kernels.  Every call on one GPU shares the array.
__device__ __align__(256) unsigned char scratch[KDA_SPLIT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current GPU's scratch array.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (raw_enum(s)) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: invalid B/T/H or sizes too large";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown q/k/v or o dtype";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size, chunk size or dtype combination not built";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a pointer is not 16-byte aligned";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed (see kda_last_hip_error)";
  }
  return "KDA: unknown status";
}

int kda_last_hip_error(void) { return g_last_hip_error; }

int kda_version(void) { return kVersion; }

#ifdef KDA_TEST_HOOKS
// Test builds only: force the prefill kernel (impl -1: the library's choice, 0:
// the generic kernel, 1: the single-kernel pipeline where it applies, 2: the
// two-stage prefill where it applies) and the generic
// kernel's slab width (0: the library's choice, 16 or 32).  Not thread-safe.
void kda_test_force_prefill(int impl, int slab) {
  g_force_impl = impl;
  g_force_slab = slab;
}
// Test builds only: the two-stage prefill's workspace cap in bytes (0: the
// library's), so small calls exercise the blocked path.  Not thread-safe.
void kda_test_set_rec_cap(unsigned long long bytes) { g_rec_cap = (size_t)bytes; }
// Test builds only: whether blocked two-stage batches run each block's chain
// beside stage 1 of the next (-1: the library's choice, 0: never, 1: always).
// Not thread-safe.
void kda_test_set_overlap(int mode) { g_force_overlap = mode; }

// Test builds only: the two stages of the two-stage prefill run alone, on B
// sequences of T tokens (bf16 q/k/v, d_k in {64, 128}, no checks beyond the
// shape): stage 1 writes the records of every chunk to rec (ceil(T/32) * B * H
// records, slot b * ceil(T/32) + c); stage 2 runs the chain from records in rec.
int kda_test_prep(const void* q, const void* k, const float* alpha, const float* beta, int B, int T, int H,
                  int d_k, void* rec, hipStream_t stream) {
  if (kda::chunk_rec_bytes(d_k) == 0 || B < 1 || H < 1 || T < 1) return KDA_ERR_UNSUPPORTED;
  kda::PrefillParams p{};
  p.q = q;
  p.k = k;
  p.alpha = alpha;
  p.beta = beta;
  p.B = B;
  p.T = T;
  p.H = H;
  p.dk = d_k;
  p.rec = static_cast<char*>(rec);
  p.rec_c0 = 0;
  p.rec_nc = (T + kda::kPipeChunk - 1) / kda::kPipeChunk;
  const hipError_t e = kda::launch_prefill_prep(p, (long long)B * p.rec_nc, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
int kda_test_chain(const void* v, const void* rec, const float* S0, float* o, float* S_T, int B, int T, int H,
                   int d_k, int d_v, hipStream_t stream) {
  if (kda::chunk_rec_bytes(d_k) == 0 || B < 1 || H < 1 || T < 1 || d_v % 32) return KDA_ERR_UNSUPPORTED;
  kda::PrefillParams p{};
  p.v = v;
  p.S0 = S0;
  p.o = o;
  p.S_T = S_T;
  p.B = B;
  p.T = T;
  p.H = H;
  p.dk = d_k;
  p.dv = d_v;
  p.o_f32 = 1;
  p.rec = static_cast<char*>(const_cast<void*>(rec));
  p.rec_c0 = 0;
  p.rec_nc = (T + kda::kPipeChunk - 1) / kda::kPipeChunk;
  kda::SnapList snap{};
  const hipError_t e = kda::launch_prefill_chain(p, snap, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
#endif

}  // extern "C"

namespace {

// Shared body of kda_chunk_fwd and kda_chunk_fwd_snapshots (n_snap == 0: none).
// cu != NULL: a packed batch of B sequences over T token rows (T = the packed
// length); otherwise B sequences of T tokens each.
// z != NULL: fused gate (alpha formed from z and A in the kernels; alpha unused).
kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, int qkv_dtype, const float* alpha,
                          const float* beta, const float* S0, void* o, int o_dtype, float* S_T,
                          const int* snap_tokens, int n_snap, float* snaps, const int* cu, const void* z,
                          const float* A, int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream,
                          const SplitReq* split = nullptr) {
  if (!dtype_ok(qkv_dtype)) return KDA_ERR_DTYPE;
  if (!dtype_ok(o_dtype)) return KDA_ERR_DTYPE;
  if (B < 1 || H < 1 || T < 0) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(cu ? 1 : B, T, H, d_k, d_v) || (long long)B * H > (1LL << 26)) return KDA_ERR_SHAPE;
  if (n_snap < 0 || n_snap > KDA_MAX_SNAPSHOTS) return KDA_ERR_SHAPE;
  if (T > 0 && (!q || !k || !v || !(z ? (const void*)A : (const void*)alpha) || !beta || !o)) return KDA_ERR_NULL;
  if (n_snap > 0 && (!snap_tokens || !snaps)) return KDA_ERR_NULL;
  kda::SnapList snap{};
  for (int j = 0; j < n_snap; ++j) {
    const int t = snap_tokens[j];
    if (t < 1 || t > T || (t % chunk != 0 && t != T)) return KDA_ERR_SHAPE;
    if (j > 0 && t <= snap_tokens[j - 1]) return KDA_ERR_SHAPE;
    snap.pos[j] = t;
  }
  if (cu && n_snap > 0) return KDA_ERR_UNSUPPORTED;
  if (z) alpha = nullptr;
  const void* ptrs[] = {q, k, v, alpha, beta, S0, o, S_T, n_snap > 0 ? snaps : nullptr, cu, z, A};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const int io = io_of(qkv_dtype);
  const PrefillPlan plan = plan_prefill(B, H, d_k, d_v, chunk, io);
  if (plan.impl == IMPL_GENERIC && !kda::prefill_supported(io, d_k, chunk, plan.slab)) return KDA_ERR_UNSUPPORTED;

  const size_t esz = io_of(qkv_dtype) ? 2 : 4;
  const size_t osz = io_of(o_dtype) ? 2 : 4;
  const size_t ntok = (size_t)(cu ? 1 : B) * T * H;
  const size_t sbytes = (size_t)B * H * d_k * d_v * 4;
  const Span none{0, 0};
  const Span in_spans[] = {T > 0 ? span(q, ntok * d_k * esz) : none, T > 0 ? span(k, ntok * d_k * esz) : none,
                           T > 0 ? span(v, ntok * d_v * esz) : none,
                           T > 0 ? (z ? span(z, ntok * d_k * esz) : span(alpha, ntok * d_k * 4)) : none,
                           T > 0 ? span(beta, ntok * 4) : none, S0 ? span(S0, sbytes) : none,
                           cu ? span(cu, (size_t)(B + 1) * 4) : none, z && T > 0 ? span(A, (size_t)H * 4) : none};
  const Span so = T > 0 ? span(o, ntok * d_v * osz) : none;
  const Span st = S_T ? span(S_T, sbytes) : none;
  const Span sn = n_snap > 0 ? span(snaps, sbytes * n_snap) : none;
  // o and the snapshots may overlap nothing; S_T may be S0 itself but overlap
  // no other input
  for (const Span& s : in_spans) {
    if (overlap(so, s) || overlap(sn, s)) return KDA_ERR_ALIAS;
    if (&s != &in_spans[5] && overlap(st, s)) return KDA_ERR_ALIAS;  // S_T may be S0 itself
  }
  if (S0 && S_T && S0 != S_T && overlap(st, in_spans[5])) return KDA_ERR_ALIAS;
  if (overlap(so, st) || overlap(so, sn) || overlap(st, sn)) return KDA_ERR_ALIAS;

  SplitShape sh{1, T};
  if (split) {
    if (split->parts < 0 || split->num_cus < 0) return KDA_ERR_SHAPE;
    if (split->parts != 1 && (cu || n_snap > 0)) return KDA_ERR_UNSUPPORTED;
    if (plan.impl == IMPL_GENERIC) {
      if (split->parts > 1) return KDA_ERR_UNSUPPORTED;
    } else if (split->parts > 1) {
      sh = split_shape_for(T, split->parts);
    } else if (split->parts == 0) {
      const int cus = split->num_cus ? split->num_cus : device_cus();
      if (cus <= 0) {
        g_last_hip_error = (int)hipErrorNoDevice;
        return KDA_ERR_HIP;
      }
      // one part of the allocation-free call runs the pipeline (no workspace)
      sh = split_shape_auto(B, T, H, d_k, d_v, cus, plan.impl == IMPL_CHAIN && !split->scratch,
                            split->scratch ? KDA_SPLIT_SCRATCH_BYTES : SIZE_MAX);
    }
  }
  char* ws = nullptr;
  if (sh.parts > 1 && split->scratch) {
    if (split_ws_bytes(B, H, d_k, d_v, sh.parts) > KDA_SPLIT_SCRATCH_BYTES) return KDA_ERR_SHAPE;
    void* sp = nullptr;
    const hipError_t se = scratch_of_current_device(&sp);
    if (se != hipSuccess) {
      g_last_hip_error = (int)se;
      return KDA_ERR_HIP;
    }
    ws = static_cast<char*>(sp);
  } else if (sh.parts > 1) {
    const size_t need = split_ws_bytes(B, H, d_k, d_v, sh.parts);
    if (!split->ws) return KDA_ERR_NULL;
    if (!aligned16(split->ws)) return KDA_ERR_MISALIGNED;
    if (split->ws_bytes < need) return KDA_ERR_SHAPE;
    const Span sw = span(split->ws, need);
    for (const Span& s : in_spans)
      if (overlap(sw, s)) return KDA_ERR_ALIAS;
    if (overlap(sw, so) || overlap(sw, st)) return KDA_ERR_ALIAS;
    ws = static_cast<char*>(split->ws);
  }

  kda::PrefillParams p{q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, io_of(o_dtype) ? 0 : 1,
                       n_snap > 0 ? snaps : nullptr, n_snap, cu, T > 0 ? z : nullptr, A,
                       /*split*/ 0, /*nparts*/ 0, /*part_len*/ 0, nullptr, nullptr, nullptr};
  const hipStream_t hs = stream;
  hipError_t e;
  if (sh.parts > 1) {
    // pass 1: (N | M) of parts 0..P-2; combine: the state entering each part;
    // pass 2: every part from its state (S0 is read only by the combine, so
    // S_T may alias it)
    p.nparts = sh.parts;
    p.part_len = sh.part_len;
    const size_t trans_bytes = (size_t)4 * B * H * d_k * (size_t)(sh.parts - 1) * (d_v + d_k);
    p.ws_trans = reinterpret_cast<float*>(ws);
    p.ws_tree = sh.parts >= kda::kTreeParts ? reinterpret_cast<float*>(ws + trans_bytes) : nullptr;
    p.ws_in = reinterpret_cast<float*>(ws + trans_bytes * (p.ws_tree ? 2 : 1));
    p.split = 1;
    e = kda::launch_prefill_pipe(p, snap, hs);
    if (e == hipSuccess) e = kda::launch_split_combine(p, hs);
    p.split = 2;
    if (e == hipSuccess) e = kda::launch_prefill_pipe(p, snap, hs);
  } else if (plan.impl == IMPL_CHAIN && !(split && split->scratch)) {
    // (a one-part split is this same single pass; the allocation-free call
    // takes the pipeline, which needs no workspace)
    bool ran = false;
    e = run_two_stage(p, snap, hs, &ran);
    if (e == hipSuccess && !ran) e = kda::launch_prefill_pipe(p, snap, hs);
  } else {
    e = plan.impl == IMPL_GENERIC ? kda::launch_prefill(p, snap, io, chunk, plan.slab, hs)
                                  : kda::launch_prefill_pipe(p, snap, hs);
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KDA_ERR_HIP;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                         const float* alpha, const float* beta, const float* S0,
                         void* o, kda_dtype o_dtype, float* S_T,
                         int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), alpha, beta, S0, o, raw_enum(o_dtype), S_T, nullptr, 0, nullptr, nullptr, nullptr,
                        nullptr, B, T, H, d_k, d_v, chunk, stream);
}

kda_status kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                   const float* alpha, const float* beta, const float* S0,
                                   void* o, kda_dtype o_dtype, float* S_T,
                                   const int* snap_tokens, int n_snap, float* snaps,
                                   int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), alpha, beta, S0, o, raw_enum(o_dtype), S_T, snap_tokens, n_snap, snaps, nullptr,
                        nullptr, nullptr, B, T, H, d_k, d_v, chunk, stream);
}

kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                const float* alpha, const float* beta, const float* S0,
                                void* o, kda_dtype o_dtype, float* S_T,
                                const int* cu_seqlens, int N, int total_T,
                                int H, int d_k, int d_v, int chunk, hipStream_t stream) {
  if (!cu_seqlens) return KDA_ERR_NULL;
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), alpha, beta, S0, o, raw_enum(o_dtype), S_T, nullptr, 0, nullptr, cu_seqlens,
                        nullptr, nullptr, N, total_T, H, d_k, d_v, chunk, stream);
}

kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const void* z, const float* A, const float* beta, const float* S0,
                               void* o, kda_dtype o_dtype, float* S_T,
                               int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream) {
  if (T > 0 && !z) return KDA_ERR_NULL;
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), nullptr, beta, S0, o, raw_enum(o_dtype), S_T, nullptr, 0, nullptr, nullptr, z, A,
                        B, T, H, d_k, d_v, chunk, stream);
}

kda_status kda_chunk_fwd_run_chunk(kda_dtype qkv_dtype, int H, int d_k, int d_v, int chunk, int* run_chunk) {
  if (!dtype_ok(raw_enum(qkv_dtype))) return KDA_ERR_DTYPE;
  if (H < 1) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (!run_chunk) return KDA_ERR_NULL;
  const int io = io_of(raw_enum(qkv_dtype));
  const PrefillPlan plan = plan_prefill(1, H, d_k, d_v, chunk, io);
  if (plan.impl == IMPL_PIPE || plan.impl == IMPL_CHAIN) {
    *run_chunk = kda::kPipeChunk;
    return KDA_OK;
  }
  const int run = kda::prefill_run_chunk(io, d_k, chunk, plan.slab);
  if (run <= 0) return KDA_ERR_UNSUPPORTED;
  *run_chunk = run;
  return KDA_OK;
}

kda_status kda_chunk_fwd_split_plan(kda_dtype qkv_dtype, int B, int T, int H, int d_k, int d_v, int chunk,
                                    int parts, int num_cus, int* parts_out, size_t* workspace_bytes) {
  if (!dtype_ok(raw_enum(qkv_dtype))) return KDA_ERR_DTYPE;
  if (B < 1 || H < 1 || T < 0 || parts < 0 || num_cus < 0) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, T, H, d_k, d_v)) return KDA_ERR_SHAPE;
  if (!parts_out || !workspace_bytes) return KDA_ERR_NULL;
  const int io = io_of(raw_enum(qkv_dtype));
  SplitShape sh{1, T};
  const PrefillImpl impl = plan_prefill(B, H, d_k, d_v, chunk, io).impl;
  if (impl == IMPL_GENERIC) {  // splits run the pipeline kernel
    if (parts > 1) return KDA_ERR_UNSUPPORTED;
  } else if (parts > 1) {
    sh = split_shape_for(T, parts);
  } else if (parts == 0) {
    const int cus = num_cus ? num_cus : device_cus();
    if (cus <= 0) {
      g_last_hip_error = (int)hipErrorNoDevice;
      return KDA_ERR_HIP;
    }
    sh = split_shape_auto(B, T, H, d_k, d_v, cus, impl == IMPL_CHAIN);
  }
  *parts_out = sh.parts;
  *workspace_bytes = split_ws_bytes(B, H, d_k, d_v, sh.parts);
  return KDA_OK;
}

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* alpha, const float* beta, const float* S0,
                               void* o, kda_dtype o_dtype, float* S_T,
                               int B, int T, int H, int d_k, int d_v, int chunk,
                               int parts, int num_cus, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const SplitReq req{parts, num_cus, workspace, workspace_bytes, false};
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), alpha, beta, S0, o, raw_enum(o_dtype), S_T, nullptr, 0, nullptr, nullptr,
                        nullptr, nullptr, B, T, H, d_k, d_v, chunk, stream, &req);
}

kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                       const float* alpha, const float* beta, const float* S0,
                                       void* o, kda_dtype o_dtype, float* S_T,
                                       int B, int T, int H, int d_k, int d_v, int chunk,
                                       int parts, int num_cus, hipStream_t stream) {
  const SplitReq req{parts, num_cus, nullptr, 0, true};
  return chunk_fwd_impl(q, k, v, raw_enum(qkv_dtype), alpha, beta, S0, o, raw_enum(o_dtype), S_T, nullptr, 0,
                        nullptr, nullptr, nullptr, nullptr, B, T, H, d_k, d_v, chunk, stream, &req);
}

}  // extern "C"

namespace {

// z != NULL: fused gate, as chunk_fwd_impl.
kda_status decode_impl(const void* q, const void* k, const void* v, int qkv_dtype, const float* alpha,
                       const void* z, const float* A, const float* beta, float* S, void* o, int o_dtype,
                       int B, int H, int d_k, int d_v, hipStream_t stream) {
  if (!dtype_ok(qkv_dtype)) return KDA_ERR_DTYPE;
  if (!dtype_ok(o_dtype)) return KDA_ERR_DTYPE;
  if (B < 1 || H < 1) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, 1, H, d_k, d_v)) return KDA_ERR_SHAPE;
  if (!q || !k || !v || !(z ? (const void*)A : (const void*)alpha) || !beta || !S || !o) return KDA_ERR_NULL;
  if (z) alpha = nullptr;
  const void* ptrs[] = {q, k, v, alpha, beta, S, o, z, A};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const int io = io_of(qkv_dtype);
  if (!kda::decode_supported(io, d_k, d_v)) return KDA_ERR_UNSUPPORTED;

  const size_t esz = io_of(qkv_dtype) ? 2 : 4;
  const size_t osz = io_of(o_dtype) ? 2 : 4;
  const size_t nbh = (size_t)B * H;
  const Span so = span(o, nbh * d_v * osz);
  const Span ss = span(S, nbh * d_k * d_v * 4);
  const Span ins[] = {span(q, nbh * d_k * esz), span(k, nbh * d_k * esz), span(v, nbh * d_v * esz),
                      z ? span(z, nbh * d_k * esz) : span(alpha, nbh * d_k * 4), span(beta, nbh * 4),
                      z ? span(A, (size_t)H * 4) : Span{0, 0}};
  if (overlap(so, ss)) return KDA_ERR_ALIAS;
  for (const Span& s : ins)
    if (overlap(so, s) || overlap(ss, s)) return KDA_ERR_ALIAS;

  kda::DecodeParams p{q, k, v, alpha, beta, S, o, B, H, d_k, d_v, io_of(o_dtype) ? 0 : 1, z, A};
  const hipError_t e = kda::launch_decode(p, io, stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KDA_ERR_HIP;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                           const float* alpha, const float* beta, float* S, void* o, kda_dtype o_dtype,
                           int B, int H, int d_k, int d_v, hipStream_t stream) {
  return decode_impl(q, k, v, raw_enum(qkv_dtype), alpha, nullptr, nullptr, beta, S, o, raw_enum(o_dtype), B, H, d_k, d_v, stream);
}

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const void* z, const float* A, const float* beta, float* S, void* o,
                                 kda_dtype o_dtype, int B, int H, int d_k, int d_v, hipStream_t stream) {
  if (!z) return KDA_ERR_NULL;
  return decode_impl(q, k, v, raw_enum(qkv_dtype), nullptr, z, A, beta, S, o, raw_enum(o_dtype), B, H, d_k, d_v, stream);
}

kda_status kda_decode_verify(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const float* alpha, const float* beta, const float* S,
                             void* o, kda_dtype o_dtype, float* u,
                             int B, int K, int H, int d_k, int d_v, hipStream_t stream) {
  if (!dtype_ok(raw_enum(qkv_dtype))) return KDA_ERR_DTYPE;
  if (!dtype_ok(raw_enum(o_dtype))) return KDA_ERR_DTYPE;
  if (B < 1 || H < 1 || K < 1 || K > KDA_MAX_DRAFT) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, K, H, d_k, d_v)) return KDA_ERR_SHAPE;
  if (!q || !k || !v || !alpha || !beta || !S || !o || !u) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S, o, u};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const int io = io_of(raw_enum(qkv_dtype));
  if (!kda::spec_supported(io, d_k, d_v)) return KDA_ERR_UNSUPPORTED;

  const size_t esz = io_of(raw_enum(qkv_dtype)) ? 2 : 4;
  const size_t osz = io_of(raw_enum(o_dtype)) ? 2 : 4;
  const size_t ntok = (size_t)B * K * H;
  const Span ins[] = {span(q, ntok * d_k * esz), span(k, ntok * d_k * esz), span(v, ntok * d_v * esz),
                      span(alpha, ntok * d_k * 4), span(beta, ntok * 4), span(S, (size_t)B * H * d_k * d_v * 4)};
  const Span so = span(o, ntok * d_v * osz), su = span(u, ntok * d_v * 4);
  if (overlap(so, su)) return KDA_ERR_ALIAS;
  for (const Span& s : ins)
    if (overlap(so, s) || overlap(su, s)) return KDA_ERR_ALIAS;

  kda::VerifyParams p{q, k, v, alpha, beta, S, o, u, B, K, H, d_k, d_v, io_of(raw_enum(o_dtype)) ? 0 : 1};
  const hipError_t e = kda::launch_verify(p, io, stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KDA_ERR_HIP;
  }
  return KDA_OK;
}

kda_status kda_decode_commit(const void* k, kda_dtype qkv_dtype, const float* alpha, const float* u,
                             const int* n_accept, float* S,
                             int B, int K, int H, int d_k, int d_v, hipStream_t stream) {
  if (!dtype_ok(raw_enum(qkv_dtype))) return KDA_ERR_DTYPE;
  if (B < 1 || H < 1 || K < 1 || K > KDA_MAX_DRAFT) return KDA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, K, H, d_k, d_v)) return KDA_ERR_SHAPE;
  if (!k || !alpha || !u || !n_accept || !S) return KDA_ERR_NULL;
  const void* ptrs[] = {k, alpha, u, n_accept, S};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const int io = io_of(raw_enum(qkv_dtype));
  if (!kda::spec_supported(io, d_k, d_v)) return KDA_ERR_UNSUPPORTED;

  const size_t esz = io_of(raw_enum(qkv_dtype)) ? 2 : 4;
  const size_t ntok = (size_t)B * K * H;
  const Span ss = span(S, (size_t)B * H * d_k * d_v * 4);
  const Span ins[] = {span(k, ntok * d_k * esz), span(alpha, ntok * d_k * 4), span(u, ntok * d_v * 4),
                      span(n_accept, (size_t)B * 4)};
  for (const Span& s : ins)
    if (overlap(ss, s)) return KDA_ERR_ALIAS;

  kda::CommitParams p{k, alpha, u, n_accept, S, B, K, H, d_k, d_v};
  const hipError_t e = kda::launch_commit(p, io, stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KDA_ERR_HIP;
  }
  return KDA_OK;
}

}  // extern "C"
