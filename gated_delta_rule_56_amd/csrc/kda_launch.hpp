// Internal launcher interface between the C-ABI layer (kda_api.cpp) and the
// kernel translation units.  Arguments arrive validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// The layer's own elementwise work around the recurrence.  prologue: q and k
// pass through Swish then L2 normalisation per (token, head), v through
// Swish, beta through the sigmoid.  gate != nullptr: the output becomes the
// head-wise RMSNorm of o times norm_weight (per value channel) times
// sigmoid(gate); gate has the element type and layout of v.
struct Layer {
  bool prologue = false;
  const void* gate = nullptr;
  const float* norm_weight = nullptr;
  float norm_eps = 0.f;
  // Short causal convolution of q, k, v before Swish (prologue only):
  // conv_w = 0 for none, else the width (1..4); weights [H][D][conv_w]
  // float32; carried inputs [num_seqs][H][conv_w - 1][D] in the input dtype
  // (state_in nullptr: zeros; state_out nullptr: not written).
  int conv_w = 0;
  const float* conv_weight[3] = {nullptr, nullptr, nullptr};
  const void* conv_state_in[3] = {nullptr, nullptr, nullptr};
  void* conv_state_out[3] = {nullptr, nullptr, nullptr};
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* state;
  void* o;
  int N, H, D;
  bool in_bf16, out_bf16;
  bool scalar_g;  // g holds one log-decay per (sequence, head)
  Layer layer;
  hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);

// Choices the prefill normally makes itself; zero fields mean automatic.
struct PrefillTuning {
  int segment_chunks = 0;    // local chunks per segment (>= 1), or 0
  size_t segment_bytes = 0;  // operand budget of one segment, or 0
  int value_block = 0;       // value columns per carry-pass workgroup (16 or 32), or 0
  size_t workspace_cap = 0;  // the whole workspace must fit this many bytes, or 0 (no cap)
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* o;
  const float* initial_state;
  float* final_state;
  const int32_t* cu_seqlens;  // device, or NULL => num_seqs sequences of seq_len
  const int32_t* cu_seqlens_host;  // host copy of cu_seqlens (or NULL with it)
  int num_seqs;
  int seq_len;                // tokens per sequence when cu_seqlens == NULL
  int total_tokens;
  int H, D, chunk;
  bool in_bf16, out_bf16;
  bool scalar_g;              // g holds one log-decay per (token, head)
  Layer layer;
  PrefillTuning tuning;
  void* workspace;
  hipStream_t stream;
};

// Bytes of intra-chunk operands stored per (chunk, head).
size_t prefill_chunk_bytes(int D, int chunk, bool in_bf16);
// Prefill segments: segment s covers local chunks [s L, (s + 1) L) of every
// sequence; the workspace holds the largest segment's operands.
struct SegmentPlan {
  int L = 0;          // local chunks per segment (0: no sequence has tokens)
  int nseg = 1;       // segments (at least one inter-chunk pass runs)
  int max_slots = 0;  // (sequence, chunk) slots of the largest segment, the first
};
// With tuning.workspace_cap set, a plan whose workspace exceeds the cap has
// L = 0 and nseg = 0 (the call cannot run within it).
SegmentPlan plan_segments(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D,
                          int chunk, bool in_bf16, bool epilogue, const PrefillTuning& tuning);
// Total workspace bytes (segment slot table, state carry between segments,
// one segment's operands, and with the layer epilogue one segment's raw
// fp32 output), 256-byte aligned pieces; SIZE_MAX when no plan fits the cap.
size_t prefill_workspace_bytes(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D,
                               int chunk, bool in_bf16, bool epilogue,
                               const PrefillTuning& tuning);
hipError_t launch_prefill(const PrefillArgs& a);

struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* initial_state;  // or nullptr (zeros)
  const float* d_o;            // [tokens, H, D] gradient of o
  const float* d_final_state;  // or nullptr (zeros)
  float *dq, *dk, *dv, *dg, *dbeta;
  float* d_initial_state;      // or nullptr (not written)
  const int32_t* cu_seqlens;   // device, or nullptr => num_seqs sequences of seq_len
  const int32_t* cu_seqlens_host;  // host copy (varlen), for the segment plan
  int num_seqs, seq_len, total_tokens, total_chunks;
  int H, D, chunk;
  bool in_bf16;
  PrefillTuning tuning;  // segment_chunks / segment_bytes (value_block unused)
  void* workspace;
  hipStream_t stream;
};

// Workspace of the backward pass, which runs in segments of local chunks:
// the segment's slot table (varlen), the states entering segments 1.. and
// the carried dS (more than one segment), and one segment's fp32
// per-(chunk, head) planes.  SIZE_MAX if no plan fits.
size_t backward_workspace_bytes(int num_seqs, const int32_t* cu_host, int seq_len, int H, int D, int chunk,
                                const PrefillTuning& tuning);
hipError_t launch_backward(const BackwardArgs& a);

// General DPLR forward (fp32 chunk pipeline); tied = KDA through the same
// pipeline (a = k_write = beta k, b = exp(g) k).
struct DplrArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* a;       // general form only
  const void* b;       // general form only
  const float* g;
  const float* beta;   // tied form only
  float* o;
  const float* initial_state;
  float* final_state;
  const int32_t* cu_seqlens;
  int num_seqs, seq_len, total_tokens, total_chunks;
  int H, D, chunk;
  bool in_bf16, tied;
  void* workspace;
  hipStream_t stream;
};

size_t dplr_workspace_bytes(long long total_chunks, int num_seqs, int H, int D, int chunk);
hipError_t launch_dplr(const DplrArgs& a);

struct DplrDecodeArgs {
  const void *q, *k, *v, *a, *b;
  const float* g;
  float* state;
  void* o;
  int N, H, D;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};

hipError_t launch_dplr_decode(const DplrDecodeArgs& a);

}  // namespace kda
