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
  // sequence split (nseg > 1): every head's chunks are cut into nseg
  // segments run in parallel, each from a zero state (segment 0 from
  // state_in); each writes its final state and gate sums, which a scan and
  // an output correction turn into the one-pass result
  int nseg = 1;            // 1: one pass
  float* seg_state;        // [BH, nseg, D, D] float32: each segment's final state
  float* seg_total;        // [BH, nseg, D] float32: each segment's log2-gate total
  float* chunk_cum;        // [BH, nc, D] float32: log2-gate sum from the segment start to each chunk start
  void* seg_in_t;          // [BH, nseg, D, D] element type: S_in(s) transposed (s >= 1)
  int* seg_live;           // [BH, nseg]: first chunk of each segment whose decay from its start is below the cut
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
  const void* saved_states;   // nullable: chunk-start states kept by the forward pass (no states pass)
  // carved from the workspace by launch_bwd
  void* ws_states;       // S_c          [BH, nc, D, D] element type
  void* ws_dS;           // G_{c+1}      [BH, nc, D, D] element type
  void* ws_dST;          // G_{c+1}^T    [BH, nc, D, D] element type
  float* ws_D;           // D_t          [BH, L]
  float* ws_dmu;         // sink-key partials [BH, nc, n_meta, D]
  unsigned char* ws_flag;   // [BH, nc]: the reverse walk left chunk c to the per-chunk gate kernel
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

// Chunks [lo, hi) of segment seg when nc chunks are cut into nseg segments
// (sizes differ by at most one; none is empty while nseg <= nc).
__host__ __device__ inline void segment_chunks(int seg, int nseg, int nc, int& lo, int& hi) {
  lo = (int)((long long)seg * nc / nseg);
  hi = (int)((long long)(seg + 1) * nc / nseg);
}

// Segments per head for a split forward pass: enough workgroups for the
// 256 compute units, at least 8 chunks per segment; 1 = one pass.
inline int fwd_segments(int BH, int nsplit, int L) {
  const long long blocks = (long long)BH * nsplit;
  const int nc = (L + 63) / 64;
  if (blocks <= 0 || blocks >= 256 || nc < 16) return 1;
  long long n = 256 / blocks;
  if (n > nc / 8) n = nc / 8;
  if (n > 32) n = 32;
  return n >= 2 ? (int)n : 1;
}

// Workspace of a split forward pass, in this order (each part 256-byte
// aligned): segment states, segment gate totals, per-chunk gate sums, the
// incoming states transposed in the element type of esize bytes, each
// segment's live chunk end.
inline size_t fwd_split_workspace_bytes(int BH, int L, int D, int esize, int nseg, size_t* offsets = nullptr) {
  if (nseg <= 1) return 0;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t nc = (size_t)(L + 63) / 64;
  const size_t o1 = al((size_t)BH * nseg * D * D * 4);
  const size_t o2 = o1 + al((size_t)BH * nseg * D * 4);
  const size_t o3 = o2 + al((size_t)BH * nc * D * 4);
  const size_t o4 = o3 + al((size_t)BH * nseg * D * D * esize);
  if (offsets) {
    offsets[0] = o1;
    offsets[1] = o2;
    offsets[2] = o3;
    offsets[3] = o4;
  }
  return o4 + al((size_t)BH * nseg * 4);
}
hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int D, hipStream_t st);
size_t bwd_workspace_bytes(int dtype_bf16, int BH, int L, int D, int n_meta);
hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int D, hipStream_t st);
hipError_t launch_teacher(const TeacherArgs& a, int dtype_bf16, int D, hipStream_t st);
hipError_t launch_transfer_loss(const void* y, const void* yt, void* dy, float* loss_bh, int BH, long long per_head,
                                float inv_n, int dtype_bf16, hipStream_t st);

}  // namespace lizard
