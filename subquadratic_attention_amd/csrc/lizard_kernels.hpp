// Internal interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lizard {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const void* gate_logit;   // non-null: the gates come as logits (element type), log_g unused
  const void* meta;     // [H, n_meta, D]
  void* y;
  float* lse;           // nullable
  void* y_anchor;       // nullable
  float* state_out;     // nullable
  void* states;         // nullable: chunk-start states S_c, [BH, nc, D, D] element type, row-major
  // continuation of a longer sequence (all nullable / 0): the state before
  // the first token, and the keys / values of the halo tokens just before it
  const float* state_in;   // [BH, D, D] float32
  const void* k_halo;      // [BH, halo, D] element type
  const void* v_halo;      // [BH, halo, D] element type
  int halo;                // 0 .. window - 1
  int BH, H, L, n_meta, window, nsplit;
  float alpha;
  float scale_log2;     // softmax scale * log2(e)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const void* gate_logit;   // non-null: the gates come as logits (element type), log_g unused
  const void* meta;
  float* state;
  void* k_ring;
  void* v_ring;
  void* y;
  long long pos;              // absolute position of each row's first new token ...
  const long long* pos_rows;  // ... or, when non-null, per batch row [B] (negative: row inactive)
  int T;                      // new tokens per row, appended in order (q, k, v, gates, y: [BH, T, D])
  int BH, H, n_meta, window;
  float alpha;
  float scale_log2;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const void* gate_logit;   // non-null: the gates come as logits; dgate (element type) replaces dlog_g
  const void* meta;
  const float* lse;
  const void* dy;
  void* dq;
  void* dk;
  void* dv;
  float* dlog_g;
  void* dgate;           // gradient w.r.t. the gate logits (when gate_logit is set)
  float* dmeta;          // [H, n_meta, D]
  void* workspace;
  // carved from the workspace by launch_bwd
  void* ws_states;       // S_c          [BH, nc, D, D] element type
  void* ws_dS;           // G_{c+1}      [BH, nc, D, D] element type
  void* ws_dST;          // G_{c+1}^T    [BH, nc, D, D] element type
  float* ws_D;           // D_t          [BH, L]
  float* ws_dmu;         // sink-key partials [BH, nc, n_meta, D]
  int B, BH, H, L, n_meta, window;
  float alpha;
  float scale;           // softmax scale (natural units)
};

// Causal softmax attention over all earlier tokens (the stage-1 teacher).
struct TeacherArgs {
  const void* q;
  const void* k;
  const void* v;
  void* y;
  float* lse;            // nullable [BH, L]
  int BH, L;
  float scale_log2;      // softmax scale * log2(e)
};

// Value-column slice width the forward kernel uses (0 = unsupported).
int fwd_value_slice(int dtype_bf16, int D);
hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int D, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int D, hipStream_t st);
size_t bwd_workspace_bytes(int dtype_bf16, int BH, int L, int D, int n_meta);
hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int D, hipStream_t st);
hipError_t launch_teacher(const TeacherArgs& a, int dtype_bf16, int D, hipStream_t st);
hipError_t launch_transfer_loss(const void* y, const void* yt, void* dy, float* loss_bh, int BH, long long per_head,
                                float inv_n, int dtype_bf16, hipStream_t st);

}  // namespace lizard
