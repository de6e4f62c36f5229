// Internal interface between the C-ABI host code and the kernel translation
// units: argument blocks and launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

struct RopeArgs {
  const void* in;
  void* out;
  int64_t is_b, is_s, is_h;   // input strides (elements)
  int64_t os_b, os_s, os_h;   // output strides
  int H;                      // heads of this tensor
  const int32_t* positions;   // [B, S] or null
  int B, S;
};

// theta_k / (2 pi) = base^(-2k/D) / (2 pi) for k < D/2, formed on the host in
// fp64: RoPE angles in revolutions
struct RopeAngles {
  double theta_rev[64];
  int half;   // pair k is channels (k, k + D/2) instead of (2k, 2k+1)
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // [B, Hq, S] or null
  int64_t qs_b, qs_s, qs_h;
  int64_t ks_b, ks_s, ks_h;
  int64_t vs_b, vs_s, vs_h;
  int64_t os_b, os_s, os_h;
  const int32_t* cu_docs;     // [B, n_docs + 1] or null
  int n_docs;
  int B, S, Hq, Hkv;           // S: keys (and key positions) per sequence
  int Sq, q_off;              // query rows per sequence, at positions q_off .. q_off + Sq - 1
  int n_qtiles;               // ceil(Sq / tokens per workgroup)
  float scale_log2;           // softmax scale * log2(e)
  float scale;                // softmax scale
  // RoPE of the queries inside the kernel (gqa_prefill_rope); rope_q = 0: the
  // queries arrive rotated
  int rope_q;
  int rope_half;              // pair k is channels (k, k + D/2) instead of (2k, 2k+1)
  const int32_t* positions;   // [B, Sq] or null (position = q_off + row)
  double theta_rev[64];       // theta_k / (2 pi), k < D/2: angles in revolutions
  // split key ranges (split_tiles > 0): partials in o_part fp32
  // [max_splits, B, Sq, Hq, D] and lse_part fp32 [max_splits, B, Hq, Sq]
  int split_tiles, max_splits;
  float* o_part;
  float* lse_part;
  // context-parallel ring step: keys at positions k_off .. k_off + S - 1;
  // acc_mode 1 writes, 2 merges this shard's (o, lse) into the fp32
  // accumulators o_acc [B, Sq, Hq, D] and lse_acc [B, Hq, Sq]; 3 merges
  // them and writes the final o and lse instead (the ring's last step).
  // ring_out: the step writes the final o and lse (acc_mode 0: a first and
  // last step, the plain prefill of the shard; acc_mode 3)
  int k_off, acc_mode, ring_out;
  float* o_acc;
  float* lse_acc;
  // persistent grid (bf16, no split, no ring step): nine work-queue counters
  // (zero between launches; the kernel leaves them zero) and the grid size;
  // sched = null: one workgroup per work item
  unsigned* sched;
  int pgrid;
};

struct DecodeArgs {
  const void* q;
  int64_t qs_b, qs_h;
  const void* k;
  const void* v;
  int64_t cs_b, cs_h, cs_l;
  const int32_t* seq_lens;
  int B, Hq, Hkv, Lmax, kv_chunk, max_splits;
  float scale_log2;
  float scale;
  float* o_part;              // [B, Hq, max_splits, D]
  float* lse_part;            // [B, Hq, max_splits]
  // paged cache (block_table non-null): key j of sequence b sits in page
  // block_table[b * bt_stride + (j >> page_shift)], slot j & (2^page_shift - 1);
  // cs_b is then the page stride
  const int32_t* block_table;
  int bt_stride, page_shift;
  int grid;                   // workgroups of the persistent grid (compute units)
  // compact partials (hdr non-null): wave w writes hdr[2w], hdr[2w+1] = the
  // first and last (sequence, KV head) index b * Hkv + kvh it holds a run of
  // (INT_MAX, -1 when it holds none), and the run of pair bh goes to slot
  // w + bh: o_part [slot][G][D], lse_part [slot][G]
  int* hdr;
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* seq_lens;
  int B, Hq, kv_chunk, max_splits;
  void* o;
  int64_t os_b, os_h;
  float* lse;                 // [B, Hq] or null
  // compact partials (hdr non-null): see DecodeArgs; W waves wrote headers
  const int* hdr;
  int Hkv, W;
};

// Gradient pass (bf16 tensors): q, k rotated; o, lse from the forward; dout
// the output gradient; delta fp32 [B, Hq, S] a workspace (-rowsum(dout o)).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;           // [B, Hq, S], natural log
  float* delta;               // [B, Hq, S]
  void* dq;
  void* dk;
  void* dv;
  int64_t qs_b, qs_s, qs_h;
  int64_t ks_b, ks_s, ks_h;
  int64_t vs_b, vs_s, vs_h;
  int64_t os_b, os_s, os_h;
  int64_t gs_b, gs_s, gs_h;   // dout
  int64_t dqs_b, dqs_s, dqs_h;
  int64_t dks_b, dks_s, dks_h;
  int64_t dvs_b, dvs_s, dvs_h;
  const int32_t* cu_docs;     // [B, n_docs + 1] or null
  int n_docs;
  int B, S, Hq, Hkv;
  float scale, scale_log2;
  // key blocks with long query ranges split into kBwdPieces pieces, each
  // writing fp32 partial dk, dv to its slot of dkv_part
  // [kBwdPieces, B, S, Hkv, 2, D] (null: no split)
  float* dkv_part;
};

// Launchers: return hipSuccess or the launch error. dt: 0 = bf16, 1 = fp32.
hipError_t launch_rope_pair(const RopeArgs& q, const RopeArgs& k, const RopeAngles& ang, int D, int dt,
                            hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int D, int G, int dt, hipStream_t st);
hipError_t launch_prefill_merge(const PrefillArgs& a, int D, int dt, hipStream_t st);
// The ring's finalize: the fp32 accumulators (o_part, lse_part, one slot) to o and lse.
hipError_t launch_ring_finalize(const PrefillArgs& a, int D, int dt, hipStream_t st);
// The work-queue counters of the persistent prefill grid for launches on
// stream st (null: launch one workgroup per item instead).
hipError_t prefill_sched(hipStream_t st, unsigned** sched);
// Sequences per gqa_decode call (the kernel keeps per-sequence tables in LDS).
constexpr int kDecodeMaxBatch = 1024;
// Waves per workgroup of the persistent decode grid (one workgroup per CU).
constexpr int kDecodeWaves = 4;
// The allocation-free decode's scratch: its device address on the current
// device (looked up once per device) and its size in bytes.
hipError_t decode_scratch(void** ptr, size_t* bytes);

hipError_t launch_decode(const DecodeArgs& a, int D, int G, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, int D, int dt, hipStream_t st);

hipError_t launch_backward(const BwdArgs& a, int D, int G, hipStream_t st);
// Keys per workgroup of the key-stationary gradient kernel (dk, dv) and
// tokens per workgroup of the query-stationary one (dq).
constexpr int kBwdKeysPerBlock = 128;
constexpr int kBwdPieces = 4;
constexpr int bwd_dq_tokens_per_block(int G) { return 256 / G; }

// Tokens of one sequence handled by one prefill workgroup for group size G.
constexpr int prefill_tokens_per_block(int G) { return 256 / G; }

}  // namespace la
