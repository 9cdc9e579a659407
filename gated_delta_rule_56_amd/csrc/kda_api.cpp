// C-ABI layer: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kda_launch.hpp"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head(int Dk, int Dv) { return Dk == Dv && (Dk == 64 || Dk == 128); }

bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

bool valid_dtype(kda_dtype d) { return d == KDA_BF16 || d == KDA_F32; }

// Validates the sequence description and returns the chunk count.
kda_status seq_layout(int B, int T, int num_seqs, const int32_t* cu_dev, const int32_t* cu_host,
                      int chunk, int64_t* total_chunks) {
  if (B < 1 || T < 0 || num_seqs < 1) return KDA_ERR_INVALID_ARG;
  int64_t chunks = 0;
  if (cu_dev == nullptr) {
    if (cu_host != nullptr || num_seqs != B) return KDA_ERR_INVALID_ARG;
    chunks = (int64_t)B * ((T + chunk - 1) / chunk);
  } else {
    if (cu_host == nullptr || B != 1) return KDA_ERR_INVALID_ARG;
    if (cu_host[0] != 0 || cu_host[num_seqs] != T) return KDA_ERR_INVALID_ARG;
    for (int n = 0; n < num_seqs; ++n) {
      const int64_t len = (int64_t)cu_host[n + 1] - cu_host[n];
      if (len < 0) return KDA_ERR_INVALID_ARG;
      chunks += (len + chunk - 1) / chunk;
    }
  }
  if ((int64_t)B * T > INT32_MAX || chunks > INT32_MAX) return KDA_ERR_INVALID_ARG;
  *total_chunks = chunks;
  return KDA_OK;
}

// The layer epilogue needs a weight with the gate and a finite eps >= 0; the
// convolution a width of 1..4 and its three weights.
kda_status check_layer(const kda::Layer& L) {
  if (L.conv_w < 0 || L.conv_w > 4) return KDA_ERR_INVALID_ARG;
  for (int x = 0; x < 3; ++x) {
    if (L.conv_w > 0 && !L.conv_weight[x]) return KDA_ERR_INVALID_ARG;
    if (!aligned(L.conv_weight[x], 4) || !aligned(L.conv_state_in[x], 16) ||
        !aligned(L.conv_state_out[x], 16))
      return KDA_ERR_INVALID_ARG;
  }
  if (!L.gate) return KDA_OK;
  if (!L.norm_weight || !aligned(L.gate, 16) || !aligned(L.norm_weight, 16))
    return KDA_ERR_INVALID_ARG;
  if (!(L.norm_eps >= 0.f) || !isfinite(L.norm_eps)) return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

// The prologue always runs; epilogue and convolution as the caller asks.
kda::Layer make_layer(const kda_layer_params* p) {
  kda::Layer L;
  L.prologue = true;
  if (!p) return L;
  L.gate = p->gate;
  L.norm_weight = p->gate ? p->norm_weight : nullptr;
  L.norm_eps = p->norm_eps;
  L.conv_w = p->conv_width;
  if (p->conv_width > 0) {
    for (int x = 0; x < 3; ++x) {
      L.conv_weight[x] = p->conv_weight[x];
      L.conv_state_in[x] = p->conv_state_in[x];
      L.conv_state_out[x] = p->conv_state_out[x];
    }
  }
  return L;
}

// Options of kda_prefill_ex as the launcher's tuning (NULL: automatic).
kda_status make_tuning(const kda_prefill_options* o, kda::PrefillTuning* t) {
  *t = kda::PrefillTuning();
  if (!o) return KDA_OK;
  if (o->segment_chunks < 0) return KDA_ERR_INVALID_ARG;
  if (o->value_block != 0 && o->value_block != 16 && o->value_block != 32)
    return KDA_ERR_INVALID_ARG;
  t->segment_chunks = o->segment_chunks;
  t->segment_bytes = o->segment_bytes;
  t->value_block = o->value_block;
  return KDA_OK;
}

kda_status workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                          const int32_t* cu_seqlens_host, int chunk_size, kda_dtype in_dtype,
                          bool epilogue, const kda::PrefillTuning& tuning, size_t* bytes) {
  if (bytes == nullptr || H < 1 || !valid_dtype(in_dtype)) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  int64_t chunks = 0;
  // Any non-NULL host table stands for a device copy when sizing.
  const int32_t* cu_dev = cu_seqlens_host;
  kda_status st = seq_layout(B, T, num_seqs, cu_dev, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  *bytes = kda::prefill_workspace_bytes(num_seqs, cu_seqlens_host, cu_seqlens_host ? 0 : T, H, Dk,
                                        chunk_size, in_dtype == KDA_BF16, epilogue, tuning);
  return KDA_OK;
}

// Static scratch of kda_prefill_noalloc: the prefill's workspace for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy of
// this array until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in); it uses the device
// address that hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = KDA_PREFILL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size or chunk size not supported";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
  }
  return "KDA_ERR_UNKNOWN";
}

int kda_version(void) { return 100; }

kda_status kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                      const int32_t* cu_seqlens_host, int chunk_size,
                                      kda_dtype in_dtype, size_t* bytes) {
  return workspace_size(B, T, H, Dk, Dv, num_seqs, cu_seqlens_host, chunk_size, in_dtype, false,
                        kda::PrefillTuning(), bytes);
}

kda_status kda_prefill_layer_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                            const int32_t* cu_seqlens_host, int chunk_size,
                                            kda_dtype in_dtype, const kda_layer_params* layer,
                                            size_t* bytes) {
  return workspace_size(B, T, H, Dk, Dv, num_seqs, cu_seqlens_host, chunk_size, in_dtype,
                        layer != nullptr && layer->gate != nullptr, kda::PrefillTuning(), bytes);
}

static kda_status prefill_impl(bool scalar_g, const kda::Layer& layer, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, void* o,
                               const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                               int B, int T, int H, int Dk, int Dv, int num_seqs,
                               int chunk_size, kda_dtype in_dtype, kda_dtype out_dtype,
                               const kda::PrefillTuning& tuning, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (H < 1 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  if (check_layer(layer) != KDA_OK) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, o, initial_state, final_state, cu_seqlens};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  int64_t chunks = 0;
  kda_status st = seq_layout(B, T, num_seqs, cu_seqlens, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  // Token tensors may be empty (and then NULL) only when there are no tokens.
  if ((int64_t)B * T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_INVALID_ARG;
  const size_t need = kda::prefill_workspace_bytes(num_seqs, cu_seqlens_host, cu_seqlens ? 0 : T,
                                                   H, Dk, chunk_size, in_dtype == KDA_BF16,
                                                   layer.gate != nullptr, tuning);
  if (need == SIZE_MAX) return KDA_ERR_WORKSPACE;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;

  kda::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.cu_seqlens = cu_seqlens;
  a.cu_seqlens_host = cu_seqlens ? cu_seqlens_host : nullptr;
  a.num_seqs = num_seqs;
  a.seq_len = cu_seqlens ? 0 : T;
  a.total_tokens = B * T;
  a.H = H;
  a.D = Dk;
  a.chunk = chunk_size;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.out_bf16 = out_dtype == KDA_BF16;
  a.scalar_g = scalar_g;
  a.layer = layer;
  a.tuning = tuning;
  a.workspace = workspace;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static kda_status decode_impl(bool scalar_g, const kda::Layer& layer, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, float* state, void* o, int N,
                              int H, int Dk, int Dv, kda_dtype in_dtype, kda_dtype out_dtype,
                              void* stream) {
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
  if (N < 0 || H < 1 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  if (check_layer(layer) != KDA_OK) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, state, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)N * H > INT32_MAX) return KDA_ERR_INVALID_ARG;
  kda::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.N = N;
  a.H = H;
  a.D = Dk;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.out_bf16 = out_dtype == KDA_BF16;
  a.scalar_g = scalar_g;
  a.layer = layer;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_prefill(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, void* o, const float* initial_state,
                       float* final_state, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                       int num_seqs, int chunk_size, kda_dtype in_dtype, kda_dtype out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(false, kda::Layer(), q, k, v, g, beta, o, initial_state, final_state,
                      cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size,
                      in_dtype, out_dtype, kda::PrefillTuning(), workspace, workspace_bytes, stream);
}

kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, void* o, const float* initial_state,
                               float* final_state, const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int B, int T, int H, int Dk,
                               int Dv, int num_seqs, int chunk_size, kda_dtype in_dtype,
                               kda_dtype out_dtype, void* stream) {
  // The segment plan is the longest whose whole workspace fits the scratch
  // array; prefill_impl returns KDA_ERR_WORKSPACE when even one-chunk
  // segments do not fit.  Every argument is checked before the scratch
  // address is looked up.
  kda::PrefillTuning t;
  t.workspace_cap = kScratchBytes;
  if (H < 1 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  int64_t chunks = 0;
  const kda_status st = seq_layout(B, T, num_seqs, cu_seqlens, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  const size_t need = kda::prefill_workspace_bytes(num_seqs, cu_seqlens_host, cu_seqlens ? 0 : T,
                                                   H, Dk, chunk_size, in_dtype == KDA_BF16, false,
                                                   t);
  if (need == SIZE_MAX) return KDA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, g, beta, o, initial_state, final_state, cu_seqlens};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (!ws) return KDA_ERR_HIP;
  }
  return prefill_impl(false, kda::Layer(), q, k, v, g, beta, o, initial_state, final_state,
                      cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size,
                      in_dtype, out_dtype, t, ws, kScratchBytes, stream);
}

kda_status gdn_prefill(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, void* o, const float* initial_state,
                       float* final_state, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                       int num_seqs, int chunk_size, kda_dtype in_dtype, kda_dtype out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(true, kda::Layer(), q, k, v, g, beta, o, initial_state, final_state,
                      cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size,
                      in_dtype, out_dtype, kda::PrefillTuning(), workspace, workspace_bytes, stream);
}

kda_status kda_prefill_workspace_size_ex(int form, int B, int T, int H, int Dk, int Dv,
                                         int num_seqs, const int32_t* cu_seqlens_host,
                                         int chunk_size, kda_dtype in_dtype, const void* layer,
                                         const kda_prefill_options* options, size_t* bytes) {
  if (form != KDA_FORM_KDA && form != KDA_FORM_GDN && form != KDA_FORM_LAYER)
    return KDA_ERR_INVALID_ARG;
  kda::PrefillTuning t;
  const kda_status st = make_tuning(options, &t);
  if (st != KDA_OK) return st;
  const kda_layer_params* lp = static_cast<const kda_layer_params*>(layer);
  const bool epi = form == KDA_FORM_LAYER && lp != nullptr && lp->gate != nullptr;
  return workspace_size(B, T, H, Dk, Dv, num_seqs, cu_seqlens_host, chunk_size, in_dtype, epi, t,
                        bytes);
}

kda_status kda_prefill_ex(int form, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const void* layer, void* o,
                          const float* initial_state, float* final_state,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int B, int T,
                          int H, int Dk, int Dv, int num_seqs, int chunk_size,
                          kda_dtype in_dtype, kda_dtype out_dtype,
                          const kda_prefill_options* options, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (form != KDA_FORM_KDA && form != KDA_FORM_GDN && form != KDA_FORM_LAYER)
    return KDA_ERR_INVALID_ARG;
  kda::PrefillTuning t;
  const kda_status st = make_tuning(options, &t);
  if (st != KDA_OK) return st;
  const kda::Layer L = form == KDA_FORM_LAYER
                           ? make_layer(static_cast<const kda_layer_params*>(layer))
                           : kda::Layer();
  return prefill_impl(form == KDA_FORM_GDN, L, q, k, v, g, beta, o, initial_state, final_state,
                      cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size,
                      in_dtype, out_dtype, t, workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int N, int H, int Dk,
                           int Dv, kda_dtype in_dtype, kda_dtype out_dtype, void* stream) {
  return decode_impl(false, kda::Layer(), q, k, v, g, beta, state, o, N, H, Dk, Dv, in_dtype,
                     out_dtype, stream);
}

kda_status gdn_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int N, int H, int Dk,
                           int Dv, kda_dtype in_dtype, kda_dtype out_dtype, void* stream) {
  return decode_impl(true, kda::Layer(), q, k, v, g, beta, state, o, N, H, Dk, Dv, in_dtype,
                     out_dtype, stream);
}

kda_status kda_prefill_layer(const void* q_pre, const void* k_pre, const void* v_pre,
                             const float* g, const float* beta_logit,
                             const kda_layer_params* layer, void* o, const float* initial_state,
                             float* final_state, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                             int num_seqs, int chunk_size, kda_dtype in_dtype,
                             kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return prefill_impl(false, make_layer(layer), q_pre, k_pre, v_pre, g, beta_logit, o,
                      initial_state, final_state, cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv,
                      num_seqs, chunk_size, in_dtype, out_dtype, kda::PrefillTuning(), workspace,
                      workspace_bytes, stream);
}

kda_status kda_decode_step_layer(const void* q_pre, const void* k_pre, const void* v_pre,
                                 const float* g, const float* beta_logit,
                                 const kda_layer_params* layer, float* state, void* o, int N,
                                 int H, int Dk, int Dv, kda_dtype in_dtype, kda_dtype out_dtype,
                                 void* stream) {
  return decode_impl(false, make_layer(layer), q_pre, k_pre, v_pre, g, beta_logit, state, o, N,
                     H, Dk, Dv, in_dtype, out_dtype, stream);
}

static kda_status backward_size_impl(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                     const int32_t* cu_seqlens_host, int chunk_size,
                                     const kda_prefill_options* options, size_t* bytes) {
  if (bytes == nullptr || H < 1) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  kda::PrefillTuning t;
  if (make_tuning(options, &t) != KDA_OK || t.value_block != 0) return KDA_ERR_INVALID_ARG;
  int64_t chunks = 0;
  kda_status st = seq_layout(B, T, num_seqs, cu_seqlens_host, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  const size_t n = kda::backward_workspace_bytes(num_seqs, cu_seqlens_host, cu_seqlens_host ? 0 : T, H, Dk,
                                                 chunk_size, t);
  if (n == SIZE_MAX) return KDA_ERR_INVALID_ARG;
  *bytes = n;
  return KDA_OK;
}

kda_status kda_backward_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                       const int32_t* cu_seqlens_host, int chunk_size,
                                       size_t* bytes) {
  return backward_size_impl(B, T, H, Dk, Dv, num_seqs, cu_seqlens_host, chunk_size, nullptr, bytes);
}

kda_status kda_backward_workspace_size_ex(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                          const int32_t* cu_seqlens_host, int chunk_size,
                                          const kda_prefill_options* options, size_t* bytes) {
  return backward_size_impl(B, T, H, Dk, Dv, num_seqs, cu_seqlens_host, chunk_size, options, bytes);
}

static kda_status backward_impl(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* initial_state, const float* d_o,
                                const float* d_final_state, float* dq, float* dk, float* dv,
                                float* dg, float* dbeta, float* d_initial_state,
                                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int B,
                                int T, int H, int Dk, int Dv, int num_seqs, int chunk_size,
                                kda_dtype in_dtype, const kda_prefill_options* options,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (H < 1 || !valid_dtype(in_dtype)) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  kda::PrefillTuning t;
  if (make_tuning(options, &t) != KDA_OK || t.value_block != 0) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg,
                        dbeta, d_initial_state, cu_seqlens};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  int64_t chunks = 0;
  kda_status st = seq_layout(B, T, num_seqs, cu_seqlens, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  if ((int64_t)B * T > 0 &&
      (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
    return KDA_ERR_INVALID_ARG;
  if (chunks * (int64_t)H > INT32_MAX) return KDA_ERR_INVALID_ARG;
  const size_t need = kda::backward_workspace_bytes(num_seqs, cu_seqlens_host, cu_seqlens ? 0 : T, H, Dk,
                                                    chunk_size, t);
  if (need == SIZE_MAX) return KDA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;
  kda::BackwardArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.initial_state = initial_state;
  a.d_o = d_o;
  a.d_final_state = d_final_state;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.d_initial_state = d_initial_state;
  a.cu_seqlens = cu_seqlens;
  a.cu_seqlens_host = cu_seqlens ? cu_seqlens_host : nullptr;
  a.num_seqs = num_seqs;
  a.seq_len = cu_seqlens ? 0 : T;
  a.total_tokens = B * T;
  a.total_chunks = (int)chunks;
  a.H = H;
  a.D = Dk;
  a.chunk = chunk_size;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.tuning = t;
  a.workspace = workspace;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return kda::launch_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_backward(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* initial_state, const float* d_o,
                        const float* d_final_state, float* dq, float* dk, float* dv, float* dg,
                        float* dbeta, float* d_initial_state, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                        int num_seqs, int chunk_size, kda_dtype in_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                       d_initial_state, cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs,
                       chunk_size, in_dtype, nullptr, workspace, workspace_bytes, stream);
}

kda_status kda_backward_ex(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* initial_state, const float* d_o,
                           const float* d_final_state, float* dq, float* dk, float* dv, float* dg,
                           float* dbeta, float* d_initial_state, const int32_t* cu_seqlens,
                           const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                           int num_seqs, int chunk_size, kda_dtype in_dtype,
                           const kda_prefill_options* options, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                       d_initial_state, cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs,
                       chunk_size, in_dtype, options, workspace, workspace_bytes, stream);
}

kda_status dplr_prefill_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                       const int32_t* cu_seqlens_host, int chunk_size,
                                       size_t* bytes) {
  if (bytes == nullptr || H < 1) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  int64_t chunks = 0;
  kda_status st = seq_layout(B, T, num_seqs, cu_seqlens_host, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  *bytes = kda::dplr_workspace_bytes(chunks, num_seqs, H, Dk, chunk_size);
  return KDA_OK;
}

static kda_status dplr_impl(bool tied, const void* q, const void* k, const void* v,
                            const void* a_, const void* b_, const float* g, const float* beta,
                            float* o, const float* initial_state, float* final_state,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int B,
                            int T, int H, int Dk, int Dv, int num_seqs, int chunk_size,
                            kda_dtype in_dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (H < 1 || !valid_dtype(in_dtype)) return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv) || !supported_chunk(chunk_size)) return KDA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, a_, b_, g, beta, o, initial_state, final_state, cu_seqlens};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  int64_t chunks = 0;
  kda_status st = seq_layout(B, T, num_seqs, cu_seqlens, cu_seqlens_host, chunk_size, &chunks);
  if (st != KDA_OK) return st;
  if ((int64_t)B * T > 0 && (!q || !k || !v || !g || !o || (tied ? !beta : (!a_ || !b_))))
    return KDA_ERR_INVALID_ARG;
  if (chunks * (int64_t)H > INT32_MAX) return KDA_ERR_INVALID_ARG;
  const size_t need = kda::dplr_workspace_bytes(chunks, num_seqs, H, Dk, chunk_size);
  if (workspace == nullptr || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;
  kda::DplrArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.a = a_;
  a.b = b_;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.seq_len = cu_seqlens ? 0 : T;
  a.total_tokens = B * T;
  a.total_chunks = (int)chunks;
  a.H = H;
  a.D = Dk;
  a.chunk = chunk_size;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.tied = tied;
  a.workspace = workspace;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return kda::launch_dplr(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status dplr_prefill(const void* q, const void* k, const void* v, const void* a,
                        const void* b, const float* g, float* o, const float* initial_state,
                        float* final_state, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, int B, int T, int H, int Dk, int Dv,
                        int num_seqs, int chunk_size, kda_dtype in_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return dplr_impl(false, q, k, v, a, b, g, nullptr, o, initial_state, final_state, cu_seqlens,
                   cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size, in_dtype, workspace,
                   workspace_bytes, stream);
}

kda_status kda_prefill_chunk_fp32(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* o, const float* initial_state,
                                  float* final_state, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int B, int T, int H, int Dk,
                                  int Dv, int num_seqs, int chunk_size, kda_dtype in_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return dplr_impl(true, q, k, v, nullptr, nullptr, g, beta, o, initial_state, final_state,
                   cu_seqlens, cu_seqlens_host, B, T, H, Dk, Dv, num_seqs, chunk_size, in_dtype,
                   workspace, workspace_bytes, stream);
}

kda_status dplr_decode_step(const void* q, const void* k, const void* v, const void* a_,
                            const void* b_, const float* g, float* state, void* o, int N, int H,
                            int Dk, int Dv, kda_dtype in_dtype, kda_dtype out_dtype,
                            void* stream) {
  if (!q || !k || !v || !a_ || !b_ || !g || !state || !o) return KDA_ERR_INVALID_ARG;
  if (N < 0 || H < 1 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return KDA_ERR_INVALID_ARG;
  if (!supported_head(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, a_, b_, g, state, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)N * H > INT32_MAX) return KDA_ERR_INVALID_ARG;
  kda::DplrDecodeArgs a{q, k, v, a_, b_, g, state, o, N, H, Dk, in_dtype == KDA_BF16,
                        out_dtype == KDA_BF16, reinterpret_cast<hipStream_t>(stream)};
  return kda::launch_dplr_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
