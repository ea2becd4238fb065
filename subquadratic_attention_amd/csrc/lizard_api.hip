// C ABI of the Lizard hybrid attention library: argument checks, sizing and
// dispatch.  Every check runs before the first HIP call, so invalid calls
// return their status without touching the device.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "lizard_attn.h"
#include "lizard_kernels.hpp"

#define LIZARD_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxBH = 1 << 24;
constexpr int64_t kMaxL = 1 << 26;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Sizes common to every call.  need_seq: the call walks a sequence of L tokens.
lizard_status_t check_params(const lizard_params_t* p, bool need_seq) {
  if (p == nullptr) return LIZARD_E_NULL;
  if (p->dtype != LIZARD_F32 && p->dtype != LIZARD_BF16) return LIZARD_E_DTYPE;
  if (p->B < 0 || p->H < 0 || p->dk <= 0 || p->dv <= 0 || p->window < 1 || p->n_meta < 0 || p->chunk < 1)
    return LIZARD_E_SHAPE;
  if (need_seq && (p->L < 0 || p->L > kMaxL)) return LIZARD_E_SHAPE;
  if ((int64_t)p->B * p->H > kMaxBH) return LIZARD_E_SHAPE;
  if (!isfinite(p->alpha) || !isfinite(p->softmax_scale) || p->softmax_scale < 0.f) return LIZARD_E_SHAPE;
  if (p->dk != p->dv) return LIZARD_E_UNSUPPORTED;
  if (p->dtype == LIZARD_BF16 && p->dk != 64 && p->dk != 128) return LIZARD_E_UNSUPPORTED;
  if (p->dtype == LIZARD_F32 && p->dk != 64) return LIZARD_E_UNSUPPORTED;
  if (p->chunk != 64 || p->window > 64 || p->n_meta > 16) return LIZARD_E_UNSUPPORTED;
  return LIZARD_OK;
}

float scale_of(const lizard_params_t* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)p->dk);
}

lizard_status_t launched(hipError_t e) { return e == hipSuccess ? LIZARD_OK : LIZARD_E_LAUNCH; }

// The fixed scratch of lizard_attn_fwd_split_noalloc: one copy per GPU, held
// until the process ends.  Host code never uses this name as an address (on
// the host it is only a handle); the device address of each GPU's copy comes
// from hipGetSymbolAddress with that GPU current, once, and is kept here.
static __device__ __align__(256) unsigned char scratch[LIZARD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch (nullptr on a HIP error).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Segments per head of a split forward pass (1: one pass) and its workspace.
int split_segments(const lizard_params_t* p) {
  const int DV = lizard::fwd_value_slice(p->dtype == LIZARD_BF16, p->dk);
  if (DV <= 0) return 1;
  return lizard::fwd_segments(p->B * p->H, p->dv / DV, p->L);
}
size_t split_workspace(const lizard_params_t* p, int nseg, size_t* offsets = nullptr) {
  return lizard::fwd_split_workspace_bytes(p->B * p->H, p->L, p->dk, p->dtype == LIZARD_BF16 ? 2 : 4, nseg, offsets);
}

// The forward pass with the gates given as log-gates (log_g) or as logits
// (gate_logit); exactly one of the two is used.  state_in / halo: a
// continued sequence (NULL / 0 for a sequence that starts at position 0).
lizard_status_t attn_fwd(const lizard_params_t* p, const void* q, const void* k, const void* v, const float* log_g,
                         const void* gate_logit, bool logit, const void* meta_k, const float* state_in,
                         const void* k_halo, const void* v_halo, int32_t halo_len, void* y, float* lse,
                         void* y_anchor, float* state_out, void* stream, bool split = false,
                         void* workspace = nullptr, size_t workspace_bytes = 0, void* chunk_states = nullptr,
                         bool fixed_scratch = false, bool auto_split = false) {
  lizard_status_t s = check_params(p, true);
  if (s != LIZARD_OK) return s;
  if (halo_len < 0 || halo_len > p->window - 1) return LIZARD_E_SHAPE;
  int nseg = split || auto_split ? split_segments(p) : 1;
  if (auto_split) {
    // the workspace is taken from the stream-ordered allocator below
  } else if (fixed_scratch) {
    // the workspace comes from the library's fixed scratch (checked here,
    // taken after every other check)
    if (split_workspace(p, nseg) > (size_t)LIZARD_NOALLOC_SCRATCH_BYTES) return LIZARD_E_WORKSPACE;
  } else if (nseg > 1 && (workspace == nullptr || workspace_bytes < split_workspace(p, nseg))) {
    return LIZARD_E_WORKSPACE;
  }
  const int BH = p->B * p->H;
  if (BH == 0) return LIZARD_OK;  // nothing to read or write; empty tensors may have NULL data
  const bool seq = p->L > 0;
  const void* gate = logit ? gate_logit : static_cast<const void*>(log_g);
  if ((seq && (!q || !k || !v || !gate || !y)) || (p->n_meta > 0 && !meta_k) ||
      (seq && halo_len > 0 && (!k_halo || !v_halo)))
    return LIZARD_E_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(gate) || misaligned(y) ||
      misaligned(meta_k) || misaligned(lse) || misaligned(y_anchor) || misaligned(state_out) ||
      misaligned(state_in) || misaligned(k_halo) || misaligned(v_halo) || misaligned(workspace) ||
      misaligned(chunk_states))
    return LIZARD_E_ALIGN;
  if (!seq && state_out == nullptr) return LIZARD_OK;
  if (fixed_scratch && nseg > 1) {
    workspace = scratch_ptr();
    if (workspace == nullptr) return LIZARD_E_LAUNCH;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  bool owned = false;   // a workspace of this call, freed after its kernels (stream order)
  if (auto_split && nseg > 1) {
    if (hipMallocAsync(&workspace, split_workspace(p, nseg), hs) == hipSuccess && workspace != nullptr) {
      owned = true;
    } else {
      (void)hipGetLastError();   // clear the failed allocation; the one-pass schedule needs no workspace
      workspace = nullptr;
      nseg = 1;
    }
  }
  const int bf = p->dtype == LIZARD_BF16;
  const int DV = lizard::fwd_value_slice(bf, p->dk);
  lizard::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_g = logit ? nullptr : log_g;
  a.gate_logit = logit ? gate_logit : nullptr;
  a.meta = meta_k;
  a.y = y;
  a.lse = lse;
  a.y_anchor = y_anchor;
  a.state_out = state_out;
  a.states = chunk_states;
  a.state_in = state_in;
  a.k_halo = halo_len > 0 ? k_halo : nullptr;
  a.v_halo = halo_len > 0 ? v_halo : nullptr;
  a.halo = halo_len;
  a.BH = BH;
  a.H = p->H;
  a.L = p->L;
  a.n_meta = p->n_meta;
  a.window = p->window;
  a.nsplit = p->dv / DV;
  a.alpha = p->alpha;
  a.scale_log2 = scale_of(p) * 1.4426950408889634f;
  a.nseg = nseg;
  if (nseg > 1) {
    size_t off[4];
    split_workspace(p, nseg, off);
    char* w = static_cast<char*>(workspace);
    a.seg_state = reinterpret_cast<float*>(w);
    a.seg_total = reinterpret_cast<float*>(w + off[0]);
    a.chunk_cum = reinterpret_cast<float*>(w + off[1]);
    a.seg_in_t = w + off[2];
    a.seg_live = reinterpret_cast<int*>(w + off[3]);
  }
  const hipError_t e = lizard::launch_fwd(a, bf, p->dk, hs);
  if (owned) (void)hipFreeAsync(workspace, hs);
  return launched(e);
}

// The backward pass; with logits, dgate (element type) replaces dlog_g.
// saved_states: the chunk-start states a training forward kept (NULL: the
// pass recomputes them).
lizard_status_t attn_bwd(const lizard_params_t* p, const void* q, const void* k, const void* v, const float* log_g,
                         const void* gate_logit, bool logit, const void* meta_k, const float* lse, const void* dy,
                         void* dq, void* dk, void* dv, float* dlog_g, void* dgate, float* dmeta_k, void* workspace,
                         size_t workspace_bytes, void* stream, const void* saved_states = nullptr) {
  lizard_status_t s = check_params(p, true);
  if (s != LIZARD_OK) return s;
  const int BH = p->B * p->H;
  const bool seq = BH > 0 && p->L > 0;   // otherwise only dmeta_k (zero) is written
  const void* gate = logit ? gate_logit : static_cast<const void*>(log_g);
  const void* dgo = logit ? dgate : static_cast<void*>(dlog_g);
  if ((seq && (!q || !k || !v || !gate || !lse || !dy || !dq || !dk || !dv || !dgo)) ||
      (p->n_meta > 0 && p->H > 0 && !dmeta_k) || (seq && p->n_meta > 0 && !meta_k))
    return LIZARD_E_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(gate) || misaligned(meta_k) ||
      misaligned(lse) || misaligned(dy) || misaligned(dq) || misaligned(dk) || misaligned(dv) ||
      misaligned(dgo) || misaligned(dmeta_k) || misaligned(workspace) || misaligned(saved_states))
    return LIZARD_E_ALIGN;
  const size_t need = lizard::bwd_workspace_bytes(p->dtype == LIZARD_BF16, BH, p->L, p->dk, p->n_meta);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LIZARD_E_WORKSPACE;
  if (!seq && (p->n_meta == 0 || p->H == 0)) return LIZARD_OK;
  lizard::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_g = logit ? nullptr : log_g;
  a.gate_logit = logit ? gate_logit : nullptr;
  a.meta = meta_k;
  a.lse = lse;
  a.dy = dy;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = logit ? nullptr : dlog_g;
  a.dgate = logit ? dgate : nullptr;
  a.dmeta = dmeta_k;
  a.workspace = workspace;
  a.saved_states = saved_states;
  a.B = p->B;
  a.BH = BH;
  a.H = p->H;
  a.L = p->L;
  a.n_meta = p->n_meta;
  a.window = p->window;
  a.alpha = p->alpha;
  a.scale = scale_of(p);
  return launched(lizard::launch_bwd(a, p->dtype == LIZARD_BF16, p->dk, static_cast<hipStream_t>(stream)));
}

constexpr int32_t kMaxTokens = 1 << 16;

// T decode tokens per row (T = 1: one step); the gates as log-gates or as
// logits; one position for every row (pos_rows NULL) or one per batch row.
lizard_status_t decode_step(const lizard_params_t* p, int64_t pos, const int64_t* pos_rows, int32_t T,
                            const void* q_t, const void* k_t, const void* v_t, const float* log_g_t,
                            const void* gate_logit_t, bool logit, const void* meta_k, float* state, void* k_ring,
                            void* v_ring, void* y_t, void* stream) {
  lizard_status_t s = check_params(p, false);
  if (s != LIZARD_OK) return s;
  if (pos < 0 || T < 1 || T > kMaxTokens) return LIZARD_E_SHAPE;
  const int BH = p->B * p->H;
  if (BH == 0) return LIZARD_OK;
  const void* gate = logit ? gate_logit_t : static_cast<const void*>(log_g_t);
  if (!q_t || !k_t || !v_t || !gate || !state || !k_ring || !v_ring || !y_t || (p->n_meta > 0 && !meta_k))
    return LIZARD_E_NULL;
  if (misaligned(q_t) || misaligned(k_t) || misaligned(v_t) || misaligned(gate) || misaligned(meta_k) ||
      misaligned(state) || misaligned(k_ring) || misaligned(v_ring) || misaligned(y_t) ||
      (reinterpret_cast<uintptr_t>(pos_rows) & 7u) != 0)
    return LIZARD_E_ALIGN;
  lizard::DecodeArgs a{};
  a.q = q_t;
  a.k = k_t;
  a.v = v_t;
  a.log_g = logit ? nullptr : log_g_t;
  a.gate_logit = logit ? gate_logit_t : nullptr;
  a.meta = meta_k;
  a.state = state;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.y = y_t;
  a.pos = pos;
  a.pos_rows = reinterpret_cast<const long long*>(pos_rows);
  a.T = T;
  a.BH = BH;
  a.H = p->H;
  a.n_meta = p->n_meta;
  a.window = p->window;
  a.alpha = p->alpha;
  a.scale_log2 = scale_of(p) * 1.4426950408889634f;
  return launched(lizard::launch_decode(a, p->dtype == LIZARD_BF16, p->dk, static_cast<hipStream_t>(stream)));
}

}  // namespace

LIZARD_API lizard_status_t lizard_attn_fwd(const lizard_params_t* p, const void* q, const void* k, const void* v,
                                           const float* log_g, const void* meta_k, void* y, float* lse,
                                           void* y_anchor, float* state_out, void* stream) {
  return attn_fwd(p, q, k, v, log_g, nullptr, false, meta_k, nullptr, nullptr, nullptr, 0, y, lse, y_anchor, state_out,
                  stream, false, nullptr, 0, nullptr, false, true);
}

LIZARD_API lizard_status_t lizard_attn_fwd_logit(const lizard_params_t* p, const void* q, const void* k,
                                                 const void* v, const void* gate_logit, const void* meta_k, void* y,
                                                 float* lse, void* y_anchor, float* state_out, void* stream) {
  return attn_fwd(p, q, k, v, nullptr, gate_logit, true, meta_k, nullptr, nullptr, nullptr, 0, y, lse, y_anchor,
                  state_out, stream, false, nullptr, 0, nullptr, false, true);
}

LIZARD_API lizard_status_t lizard_attn_fwd_continue(const lizard_params_t* p, const void* q, const void* k,
                                                    const void* v, const float* log_g, const void* gate_logit,
                                                    const void* meta_k, const float* state_in, const void* k_halo,
                                                    const void* v_halo, int32_t halo_len, void* y, float* lse,
                                                    void* y_anchor, float* state_out, void* stream) {
  if (log_g != nullptr && gate_logit != nullptr) return LIZARD_E_SHAPE;
  return attn_fwd(p, q, k, v, log_g, gate_logit, gate_logit != nullptr, meta_k, state_in, k_halo, v_halo, halo_len, y,
                  lse, y_anchor, state_out, stream, false, nullptr, 0, nullptr, false, true);
}

LIZARD_API size_t lizard_attn_fwd_split_workspace_size(const lizard_params_t* p) {
  if (check_params(p, true) != LIZARD_OK) return 0;
  return split_workspace(p, split_segments(p));
}

LIZARD_API lizard_status_t lizard_attn_fwd_split(const lizard_params_t* p, const void* q, const void* k,
                                                 const void* v, const float* log_g, const void* gate_logit,
                                                 const void* meta_k, const float* state_in, const void* k_halo,
                                                 const void* v_halo, int32_t halo_len, void* y, float* lse,
                                                 void* y_anchor, float* state_out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  if (log_g != nullptr && gate_logit != nullptr) return LIZARD_E_SHAPE;
  return attn_fwd(p, q, k, v, log_g, gate_logit, gate_logit != nullptr, meta_k, state_in, k_halo, v_halo, halo_len, y,
                  lse, y_anchor, state_out, stream, true, workspace, workspace_bytes);
}

LIZARD_API lizard_status_t lizard_attn_fwd_split_noalloc(const lizard_params_t* p, const void* q, const void* k,
                                                         const void* v, const float* log_g, const void* gate_logit,
                                                         const void* meta_k, const float* state_in,
                                                         const void* k_halo, const void* v_halo, int32_t halo_len,
                                                         void* y, float* lse, void* y_anchor, float* state_out,
                                                         void* stream) {
  if (log_g != nullptr && gate_logit != nullptr) return LIZARD_E_SHAPE;
  return attn_fwd(p, q, k, v, log_g, gate_logit, gate_logit != nullptr, meta_k, state_in, k_halo, v_halo, halo_len, y,
                  lse, y_anchor, state_out, stream, true, nullptr, 0, nullptr, true);
}

LIZARD_API size_t lizard_attn_chunk_states_size(const lizard_params_t* p) {
  if (check_params(p, true) != LIZARD_OK) return 0;
  const size_t nc = (size_t)(p->L + 63) / 64;
  return (size_t)p->B * p->H * nc * p->dk * p->dv * (p->dtype == LIZARD_BF16 ? 2 : 4);
}

LIZARD_API lizard_status_t lizard_attn_fwd_train(const lizard_params_t* p, const void* q, const void* k,
                                                 const void* v, const float* log_g, const void* gate_logit,
                                                 const void* meta_k, void* y, float* lse, void* y_anchor,
                                                 float* state_out, void* chunk_states, void* stream) {
  if (log_g != nullptr && gate_logit != nullptr) return LIZARD_E_SHAPE;
  if (p != nullptr && (int64_t)p->B * p->H > 0 && p->L > 0 && chunk_states == nullptr) return LIZARD_E_NULL;
  return attn_fwd(p, q, k, v, log_g, gate_logit, gate_logit != nullptr, meta_k, nullptr, nullptr, nullptr, 0, y, lse,
                  y_anchor, state_out, stream, false, nullptr, 0, chunk_states);
}

LIZARD_API lizard_status_t lizard_attn_bwd_train(const lizard_params_t* p, const void* q, const void* k,
                                                 const void* v, const float* log_g, const void* gate_logit,
                                                 const void* meta_k, const float* lse, const void* chunk_states,
                                                 const void* dy, void* dq, void* dk, void* dv, void* dgate,
                                                 float* dmeta_k, void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  if (log_g != nullptr && gate_logit != nullptr) return LIZARD_E_SHAPE;
  if (p != nullptr && (int64_t)p->B * p->H > 0 && p->L > 0 && chunk_states == nullptr) return LIZARD_E_NULL;
  const bool logit = gate_logit != nullptr;
  return attn_bwd(p, q, k, v, log_g, gate_logit, logit, meta_k, lse, dy, dq, dk, dv,
                  logit ? nullptr : static_cast<float*>(dgate), logit ? dgate : nullptr, dmeta_k, workspace,
                  workspace_bytes, stream, chunk_states);
}

LIZARD_API size_t lizard_attn_bwd_workspace_size(const lizard_params_t* p) {
  if (check_params(p, true) != LIZARD_OK) return 0;
  return lizard::bwd_workspace_bytes(p->dtype == LIZARD_BF16, p->B * p->H, p->L, p->dk, p->n_meta);
}

LIZARD_API lizard_status_t lizard_attn_bwd(const lizard_params_t* p, const void* q, const void* k, const void* v,
                                           const float* log_g, const void* meta_k, const float* lse,
                                           const void* dy, void* dq, void* dk, void* dv, float* dlog_g,
                                           float* dmeta_k, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return attn_bwd(p, q, k, v, log_g, nullptr, false, meta_k, lse, dy, dq, dk, dv, dlog_g, nullptr, dmeta_k,
                  workspace, workspace_bytes, stream);
}

LIZARD_API lizard_status_t lizard_attn_bwd_logit(const lizard_params_t* p, const void* q, const void* k,
                                                 const void* v, const void* gate_logit, const void* meta_k,
                                                 const float* lse, const void* dy, void* dq, void* dk, void* dv,
                                                 void* dgate_logit, float* dmeta_k, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  return attn_bwd(p, q, k, v, nullptr, gate_logit, true, meta_k, lse, dy, dq, dk, dv, nullptr, dgate_logit, dmeta_k,
                  workspace, workspace_bytes, stream);
}

LIZARD_API lizard_status_t lizard_decode_step(const lizard_params_t* p, int64_t pos, const void* q_t,
                                              const void* k_t, const void* v_t, const float* log_g_t,
                                              const void* meta_k, float* state, void* k_ring, void* v_ring,
                                              void* y_t, void* stream) {
  return decode_step(p, pos, nullptr, 1, q_t, k_t, v_t, log_g_t, nullptr, false, meta_k, state, k_ring, v_ring, y_t,
                     stream);
}

LIZARD_API lizard_status_t lizard_decode_step_logit(const lizard_params_t* p, int64_t pos, const void* q_t,
                                                    const void* k_t, const void* v_t, const void* gate_logit_t,
                                                    const void* meta_k, float* state, void* k_ring, void* v_ring,
                                                    void* y_t, void* stream) {
  return decode_step(p, pos, nullptr, 1, q_t, k_t, v_t, nullptr, gate_logit_t, true, meta_k, state, k_ring, v_ring,
                     y_t, stream);
}

LIZARD_API lizard_status_t lizard_decode_tokens(const lizard_params_t* p, const int64_t* pos, int32_t T,
                                                const void* q, const void* k, const void* v, const float* log_g,
                                                const void* meta_k, float* state, void* k_ring, void* v_ring,
                                                void* y, void* stream) {
  if (pos == nullptr && p != nullptr && p->B * (int64_t)p->H > 0) return LIZARD_E_NULL;
  return decode_step(p, 0, pos, T, q, k, v, log_g, nullptr, false, meta_k, state, k_ring, v_ring, y, stream);
}

LIZARD_API lizard_status_t lizard_decode_tokens_logit(const lizard_params_t* p, const int64_t* pos, int32_t T,
                                                      const void* q, const void* k, const void* v,
                                                      const void* gate_logit, const void* meta_k, float* state,
                                                      void* k_ring, void* v_ring, void* y, void* stream) {
  if (pos == nullptr && p != nullptr && p->B * (int64_t)p->H > 0) return LIZARD_E_NULL;
  return decode_step(p, 0, pos, T, q, k, v, nullptr, gate_logit, true, meta_k, state, k_ring, v_ring, y, stream);
}

LIZARD_API lizard_status_t lizard_softmax_attn_fwd(const lizard_params_t* p, const void* q, const void* k,
                                                   const void* v, void* y, float* lse, void* stream) {
  lizard_status_t s = check_params(p, true);
  if (s != LIZARD_OK) return s;
  const int BH = p->B * p->H;
  if (BH == 0 || p->L == 0) return LIZARD_OK;
  if (!q || !k || !v || !y) return LIZARD_E_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(y) || misaligned(lse)) return LIZARD_E_ALIGN;
  lizard::TeacherArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.y = y;
  a.lse = lse;
  a.BH = BH;
  a.L = p->L;
  a.scale_log2 = scale_of(p) * 1.4426950408889634f;
  return launched(lizard::launch_teacher(a, p->dtype == LIZARD_BF16, p->dk, static_cast<hipStream_t>(stream)));
}

LIZARD_API lizard_status_t lizard_transfer_loss(const lizard_params_t* p, const void* y, const void* y_teacher,
                                                void* dy, float* loss_bh, void* stream) {
  lizard_status_t s = check_params(p, true);
  if (s != LIZARD_OK) return s;
  const int BH = p->B * p->H;
  if (BH == 0) return LIZARD_OK;
  if (!loss_bh || (p->L > 0 && (!y || !y_teacher || !dy))) return LIZARD_E_NULL;
  if (misaligned(y) || misaligned(y_teacher) || misaligned(dy) || misaligned(loss_bh)) return LIZARD_E_ALIGN;
  const long long per_head = (long long)p->L * p->dv;
  const double n = (double)BH * (double)per_head;
  const float inv_n = n > 0 ? (float)(1.0 / n) : 0.f;
  return launched(lizard::launch_transfer_loss(y, y_teacher, dy, loss_bh, BH, per_head, inv_n,
                                               p->dtype == LIZARD_BF16, static_cast<hipStream_t>(stream)));
}

LIZARD_API const char* lizard_status_string(lizard_status_t s) {
  switch (s) {
    case LIZARD_OK: return "ok";
    case LIZARD_E_NULL: return "a required pointer is NULL";
    case LIZARD_E_SHAPE: return "a size or constant is out of range";
    case LIZARD_E_DTYPE: return "unknown dtype";
    case LIZARD_E_ALIGN: return "a pointer is not 16-byte aligned";
    case LIZARD_E_WORKSPACE: return "backward workspace too small";
    case LIZARD_E_UNSUPPORTED: return "no kernel for these sizes in this library";
    case LIZARD_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

LIZARD_API int lizard_abi_version(void) { return 4; }
