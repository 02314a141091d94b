// Internal host-side interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;  // may be null (zeros)
  void* o;
  float* S_T;       // may be null (not written)
  int B, T, H, dk, dv;
  int o_f32;        // 1: o is fp32, 0: o is bf16
  float* snaps;     // [B][H][nsnap][dk][dv], written when nsnap > 0
  int nsnap;
  // Packed variable-length batch: sequence b covers tokens [cu[b], cu[b+1]) of
  // a [T][H][d] tensor (T = the packed length; values clamped to [0, T]).
  // Null: B sequences of T tokens each.
  const int* cu;
  // Fused gate: when z is set, alpha = exp(-5 sigmoid(e^{A_h} z)) is formed in
  // the kernel from z ([.][H][dk], q/k/v dtype) and A ([H] fp32); alpha is unused.
  const void* z;
  const float* A;
  // Sequence split (a two-level scan over parts of each sequence).  split = 0:
  // off.  Otherwise every sequence is cut into nparts parts of part_len tokens
  // (a multiple of 32; the last part may be shorter).
  //   split = 1: parts 0 .. nparts-2, each from a zero state over d_v + d_k
  //     state columns: the d_v value columns give the part's own contribution N,
  //     the d_k extra columns start as the identity with V = 0 and give the
  //     part's transition M (state after the part = M S_in + N).  Both go to
  //     ws_trans [B][nparts-1][H][dk][dv+dk]; o is not written.
  //   split = 2: parts 0 .. nparts-1, each from the state entering it, ws_in
  //     [B][nparts][H][dk][dv]; o is written, and S_T by the last part.
  int split, nparts, part_len;
  float* ws_trans;
  float* ws_in;
  float* ws_tree;  // nparts >= kTreeParts: a second [B][nparts-1][H][dk][dv+dk] buffer
  // Two-stage prefill: the chunk records of stage 1 (ChunkRec layout), indexed
  // by slot * H + h.  Without cu, slot = b * rec_nc + (c - rec_c0) for the chunks
  // c in [rec_c0, rec_c0 + rec_nc) of every sequence (one block of a sequence
  // processed in several blocks); with cu, slot = cu[b] / 32 + b + c (rec_c0 = 0).
  char* rec;
  int rec_c0, rec_nc;
};

// Part counts from which the combine runs as a tree over the parts (log2 levels)
// instead of a sequential chain.
constexpr int kTreeParts = 9;

// The lower-bounded retention exp(-5 sigmoid(e^A z)) for x = e^A z.
__device__ __forceinline__ float gate_retention(float x) {
  const float log2e = 1.4426950408889634f;
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * log2e));
  return __builtin_amdgcn_exp2f(-5.0f * log2e * s);
}

// Packed batches of at most this many sequences are scheduled longest first.
constexpr int kMaxRankedSeqs = 256;

// The sequence a workgroup serves in rank slot r: for a packed batch of at most
// kMaxRankedSeqs sequences, the one of r-th largest length (ties by index), so
// the first workgroups to start take the longest sequences and the short ones
// fill in behind them; otherwise r itself.  Every thread of the workgroup
// calls it; `lens` is LDS for kMaxRankedSeqs ints.
__device__ __forceinline__ int seq_by_length_rank(const int* cu, int n, int T, int r, int* lens, int* pick) {
  if (!cu || n > kMaxRankedSeqs) return r;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int s = min(max(cu[j], 0), T);
    lens[j] = min(max(cu[j + 1], s), T) - s;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int lj = lens[j];
    int rank = 0;
    for (int i = 0; i < n; ++i) rank += (lens[i] > lj) || (lens[i] == lj && i < j);
    if (rank == r) *pick = j;  // ranks are a permutation: exactly one writer
  }
  __syncthreads();
  return *pick;
}

// Workgroup bi of G -> (task, slab), a task being one (sequence rank, head) pair served
// by nslab workgroups.  Workgroups are dispatched in index order, round-robin
// over the 8 XCDs (each with its own L2): a task's slabs go to one XCD, so they
// share its L2 for the task's keys, queries and decays, and consecutive tasks
// go to consecutive XCDs, so the tasks dispatched first -- the longest
// sequences of a packed batch -- are spread over all of them.
__device__ __forceinline__ void task_of_index(int nslab, int G, int bi, int& task, int& slab) {
  if ((G / nslab) % 8 == 0) {
    const int x = bi % 8, q = bi / 8;
    slab = q % nslab;
    task = (q / nslab) * 8 + x;
  } else {
    task = bi / nslab;
    slab = bi % nslab;
  }
}
// The same for this workgroup of a launch of its tasks alone.
__device__ __forceinline__ void task_of_block(int nslab, int& task, int& slab) {
  task_of_index(nslab, gridDim.x, blockIdx.x, task, slab);
}

// Token range of sequence b: first packed token and length.
__device__ __forceinline__ void seq_range(const PrefillParams& p, int b, long long& tok0, int& len) {
  if (p.cu) {
    const int s = min(max(p.cu[b], 0), p.T);
    const int e = min(max(p.cu[b + 1], s), p.T);
    tok0 = s;
    len = e - s;
  } else {
    tok0 = (long long)b * p.T;
    len = p.T;
  }
}

// Token counts after which the state is recorded (ascending; a separate kernel
// argument, read in place by the state waves).
constexpr int kMaxSnapshots = 128;
struct SnapList {
  int pos[kMaxSnapshots];
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* S;
  void* o;
  int B, H, dk, dv;
  int o_f32;
  const void* z;  // fused gate (see PrefillParams); null: alpha is given
  const float* A;
};

// io_dtype: 0 = fp32, 1 = bf16.  `slab` is the number of state columns one
// workgroup owns (16, 32 or 64).  Returns hipErrorInvalidValue when no kernel is
// built for the combination.
bool prefill_supported(int io_dtype, int dk, int chunk, int slab);
// Tokens per chunk the generic kernel runs for a requested chunk size (0: not built).
int prefill_run_chunk(int io_dtype, int dk, int chunk, int slab);
hipError_t launch_prefill(const PrefillParams& p, const SnapList& snap, int io_dtype, int chunk, int slab,
                          hipStream_t s);

// Warp-specialised pipeline prefill (bf16 q/k/v, d_k in {64,128}, d_v % 32 == 0,
// requested chunk 32 or 64; runs kPipeChunk-token chunks).
constexpr int kPipeChunk = 32;
bool prefill_pipe_supported(int io_dtype, int dk, int dv, int chunk, int H);
hipError_t launch_prefill_pipe(const PrefillParams& p, const SnapList& snap, hipStream_t s);

// ---- two-stage prefill -------------------------------------------------------------
// Stage 1 (prep) computes, for every (sequence, head, 32-token chunk) at once,
// the chunk-local operands of the chunkwise form; stage 2 (chain) streams them
// through the sequential state update.  The record of one chunk: KG, T, -KH^T
// and gamma (the chain's state part), then QG, -P T and its remainder (the
// output part); every matrix as fp16 matrix-core fragments of 64 lanes x 16
// bytes.  Lane l = 16 g + n of a fragment holds 8 values (columns listed in slot
// order):
//   KG, QG [rt][kb] : token 16 rt + n, channels 32 kb + {4g..4g+3, 16+4g..16+4g+3}
//   T, -P T [rt]    : row 16 rt + n, columns {4g..4g+3, 16+4g..16+4g+3}
//   (-P T)_lo [rt]  : the fp16 rounding remainder of -P T, same layout
//   -KH^T  [i]      : channel 16 i + n, tokens {4g..4g+3, 16+4g..16+4g+3}
//   gamma           : d_k fp32
template <int DK>
struct ChunkRec {
  static constexpr int NKB = DK / 32, NKT = DK / 16;
  // what the chain's state waves read, then what its output waves read
  static constexpr int KG = 0;
  static constexpr int TT = KG + 2 * NKB * 1024;
  static constexpr int KH = TT + 2 * 1024;
  static constexpr int GAM = KH + NKT * 1024;
  static constexpr int OUT = GAM + DK * 4;
  static constexpr int QG = OUT;
  static constexpr int PP = QG + 2 * NKB * 1024;
  static constexpr int PL = PP + 2 * 1024;
  static constexpr int BYTES = PL + 2 * 1024;
};
// Bytes of one chunk record (0: no two-stage kernels for d_k).
inline int chunk_rec_bytes(int dk) {
  return dk == 128 ? ChunkRec<128>::BYTES : dk == 64 ? ChunkRec<64>::BYTES : 0;
}
// bf16 q/k/v, d_k in {64, 128}, d_v % 32 == 0.
bool prefill_chain_supported(int io_dtype, int dk, int dv, int chunk, int H);
// Stage 1 over the records that p.rec, p.rec_c0 and p.rec_nc describe (nslots
// slots of H records each).
hipError_t launch_prefill_prep(const PrefillParams& p, long long nslots, hipStream_t s);
// Stage 2: without cu, the chunks [rec_c0, rec_c0 + rec_nc) of every sequence,
// from S0 to S_T (either may be null: zeros / not written).
hipError_t launch_prefill_chain(const PrefillParams& p, const SnapList& snap, hipStream_t s);
// The chain over the block of chunks pc describes and, beside it in the same
// launch, stage 1 of the block pp describes (nslots record slots).
hipError_t launch_prefill_chain_prep(const PrefillParams& pc, const PrefillParams& pp, long long nslots,
                                     const SnapList& snap, hipStream_t s);

// Between the two split passes: ws_in[b][0] = S0 (zeros when null) and
// ws_in[b][j+1] = M_j ws_in[b][j] + N_j from ws_trans, for every (b, h): a
// sequential chain below kTreeParts parts, else a tree (ws_trans and ws_tree
// are both overwritten).
hipError_t launch_split_combine(const PrefillParams& p, hipStream_t s);

// Speculative decoding: K draft tokens per (sequence, head).
constexpr int kMaxDraft = 16;
struct VerifyParams {
  const void* q;  // [B][K][H][dk]
  const void* k;
  const void* v;  // [B][K][H][dv]
  const float* alpha;
  const float* beta;  // [B][K][H]
  const float* S;     // [B][H][dk][dv], read only
  void* o;            // [B][K][H][dv]
  float* u;           // [B][H][K][dv]
  int B, K, H, dk, dv;
  int o_f32;
};
struct CommitParams {
  const void* k;  // [B][K][H][dk]
  const float* alpha;
  const float* u;         // [B][H][K][dv]
  const int* n_accept;    // [B], clamped to [0, K]
  float* S;               // [B][H][dk][dv], updated in place
  int B, K, H, dk, dv;
};
bool spec_supported(int io_dtype, int dk, int dv);
hipError_t launch_verify(const VerifyParams& p, int io_dtype, hipStream_t s);
hipError_t launch_commit(const CommitParams& p, int io_dtype, hipStream_t s);

bool decode_supported(int io_dtype, int dk, int dv);
hipError_t launch_decode(const DecodeParams& p, int io_dtype, hipStream_t s);

}  // namespace kda
