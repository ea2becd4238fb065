// Recurrent decode step of the Lizard hybrid attention layer on gfx950.
//
// Constant-memory inference by incremental state updates ("Lizard"
// explainer, gist.science (de), section 2 "Kernkomponenten" item 1, and
// section 4 "Effizienz": memory stays constant with context length).  One
// token per (batch, head) at absolute position pos:
//
//   S <- diag(g) S + k v^T              (float32, in place; g = e^{log_g},
//                                        or sigmoid(x) from the gate logit x)
//   o  = S^T q
//   ring slot pos mod w <- (k, v)
//   y_anchor = softmax over the window max(0, pos-w+1)..pos and the m sink
//              keys (zero values), applied to the window values
//   y  = o + alpha * y_anchor
//
// The step is bound by HBM bandwidth: the 64 KiB float32 state of a d=128
// head is read and written once, the window's keys and values are read
// once.  One workgroup of 256 threads per (b, h); each thread streams whole
// 16-byte runs of state rows so every wavefront touches contiguous 1 KiB.
//
// Serving forms of the same kernel: each batch row may sit at its own
// position (continuous batching; a negative position leaves the row
// untouched), and a call may append T > 1 tokens per row in order (a
// speculative draft, a short continuation): the state stays in registers
// across the T tokens and is read and written once per call.
#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

// MULTI = false: one token per row (the loop below runs once and the state
// registers die after the update, which keeps the kernel at ~90 VGPRs and
// five workgroups per CU); MULTI = true: a.T tokens with the state held in
// registers across them.  In bf16 the multi-token form is held to three
// wavefronts per SIMD (168 VGPRs, a 20-byte spill): at d = 128 it would
// otherwise take 203 VGPRs and two, and the third workgroup per CU hides
// more of the state and window reads (4 tokens per call: 29.1 -> 27.6 us
// per token at batch 64).
template <typename T, int D, bool LOGIT, bool MULTI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MULTI && sizeof(T) == 2 ? 3 : 1)))
void lizard_decode_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;            // float4 column groups per row
  constexpr int RG = 256 / CG;         // row groups
  constexpr int RPT = D / RG;          // rows per thread
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int QVD = D / 4 / EPV;     // 16-byte vectors in a quarter row
  constexpr int NCG = D / EPV;         // window product: column groups of EPV columns
  constexpr int NSG = 256 / NCG;       // ... and slot groups
  constexpr int SPG = 64 / NSG;        // slots per slot group
  static_assert(NCG * NSG == 256 && SPG * NSG == 64, "decode shape");
  __shared__ float sq[D], sk[D], sv[D], sg[D];
  __shared__ float sO[RG][D];
  __shared__ float sZ[80];
  __shared__ float sYa[NSG][D];
  __shared__ float sDen;

  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int tid = threadIdx.x;
  const int w = a.window;
  const long long pos0 = a.pos_rows ? a.pos_rows[bh / a.H] : a.pos;
  if (pos0 < 0) return;                // inactive row: nothing read or written

  T* kr = reinterpret_cast<T*>(a.k_ring) + (size_t)bh * w * D;
  T* vr = reinterpret_cast<T*>(a.v_ring) + (size_t)bh * w * D;
  float* S = a.state + (size_t)bh * D * D;

  // the state rows first: they do not depend on the tokens, and their loads
  // then overlap the first token's loads and the barrier below; they stay in
  // registers for all T tokens and are written back once
  const int cg = tid % CG;
  const int rg = tid / CG;
  float4 s[RPT];
#pragma unroll
  for (int ii = 0; ii < RPT; ++ii) s[ii] = *reinterpret_cast<const float4*>(S + (size_t)(ii * RG + rg) * D + 4 * cg);

  const int ntok = MULTI ? a.T : 1;
  for (int j = 0; j < ntok; ++j) {
    const long long pos = pos0 + j;
    const int cur = (int)(pos % w);
    const size_t tok = ((size_t)bh * ntok + j) * D;
    const T* qg = reinterpret_cast<const T*>(a.q) + tok;
    const T* kg = reinterpret_cast<const T*>(a.k) + tok;
    const T* vg = reinterpret_cast<const T*>(a.v) + tok;

    if (j > 0) __syncthreads();        // the previous token's readers of sq .. sYa are done
    if (tid < D) {
      sq[tid] = to_f32(qg[tid]);
      sk[tid] = to_f32(kg[tid]);
      sv[tid] = to_f32(vg[tid]);
      if constexpr (LOGIT) {
        // the gate from its logit: sigmoid(x) = 1 / (1 + e^{-x})
        sg[tid] = sigmoid_neg(-to_f32(reinterpret_cast<const T*>(a.gate_logit)[tok + tid]));
      } else {
        sg[tid] = exp_e(a.log_g[tok + tid]);
      }
    }
    __syncthreads();

    // ---- state update and readout partials ----
    {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 vv = make_float4(sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]);
      const bool last = j + 1 == ntok;
#pragma unroll
      for (int ii = 0; ii < RPT; ++ii) {
        const int i = ii * RG + rg;
        const float gi = sg[i], ki = sk[i], qi = sq[i];
        float4 n;
        n.x = gi * s[ii].x + ki * vv.x;
        n.y = gi * s[ii].y + ki * vv.y;
        n.z = gi * s[ii].z + ki * vv.z;
        n.w = gi * s[ii].w + ki * vv.w;
        s[ii] = n;
        if (last) *reinterpret_cast<float4*>(S + (size_t)i * D + 4 * cg) = n;
        o.x += qi * n.x;
        o.y += qi * n.y;
        o.z += qi * n.z;
        o.w += qi * n.w;
      }
      *reinterpret_cast<float4*>(&sO[rg][4 * cg]) = o;
    }

    // ---- window and sink logits: entry e < 64 is ring slot e, 64 + i is sink i ----
    {
      const int part = tid & 3;         // quarter of the dims
      for (int e = tid >> 2; e < 80; e += 64) {
        float zv = -INFINITY;
        bool live;
        const T* kp;
        if (e < 64) {
          const int slot = e;
          const long long p = pos - (long long)(((pos - slot) % w + w) % w);
          live = slot < w && p >= 0;
          kp = kr + (size_t)slot * D;
        } else {
          live = (e - 64) < a.n_meta;
          kp = reinterpret_cast<const T*>(a.meta) + ((size_t)h * a.n_meta + (e - 64)) * D;
        }
        if (live) {
          float dot = 0.f;
          const int i0 = part * (D / 4);
          if (e == cur) {
#pragma unroll 8
            for (int i = i0; i < i0 + D / 4; ++i) dot += sq[i] * sk[i];
          } else {
            // the key's quarter row as 16-byte loads
            uint4 raw[QVD];
#pragma unroll
            for (int v = 0; v < QVD; ++v) raw[v] = ld16(kp + i0 + v * EPV);
#pragma unroll
            for (int v = 0; v < QVD; ++v) {
              float kv[EPV];
              unpack16<T>(raw[v], kv);
#pragma unroll
              for (int u = 0; u < EPV; ++u) dot += sq[i0 + v * EPV + u] * kv[u];
            }
          }
          zv = dot;
        }
        zv += __shfl_xor(zv, 1, 64);
        zv += __shfl_xor(zv, 2, 64);
        if (part == 0) sZ[e] = live ? zv * a.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();

    // the incoming token goes to its ring slot (that slot is never read from
    // the ring above; the next token reads it after the barriers below)
    if (tid < D) {
      kr[(size_t)cur * D + tid] = kg[tid];
      vr[(size_t)cur * D + tid] = vg[tid];
    }

    // ---- softmax over window + sinks (wavefront 0) ----
    if (tid < 64) {
      const float z0 = sZ[tid];
      const float z1 = tid < 16 ? sZ[64 + tid] : -INFINITY;
      const float mx = wave_max(fmaxf(z0, z1));
      const float p0 = exp_2(z0 - mx);
      const float p1 = exp_2(z1 - mx);
      const float den = wave_sum(p0 + p1);
      sZ[tid] = p0;
      if (tid == 0) sDen = den;
    }
    __syncthreads();

    // ---- window values: thread (column group of EPV columns, slot group),
    // 16-byte loads; partial sums per slot group, reduced below ----
    {
      const int cgi = tid % NCG;
      const int sgi = tid / NCG;
      float ya[EPV];
#pragma unroll
      for (int u = 0; u < EPV; ++u) ya[u] = 0.f;
#pragma unroll
      for (int ss = 0; ss < SPG; ++ss) {
        const int slot = sgi * SPG + ss;
        const float p = slot < w ? sZ[slot] : 0.f;
        if (p != 0.f) {            // dead slots (p = 0) are not read: they may hold anything
          float vv[EPV];
          if (slot == cur) {
#pragma unroll
            for (int u = 0; u < EPV; ++u) vv[u] = sv[cgi * EPV + u];
          } else {
            unpack16<T>(ld16(vr + (size_t)slot * D + cgi * EPV), vv);
          }
#pragma unroll
          for (int u = 0; u < EPV; ++u) ya[u] += p * vv[u];
        }
      }
#pragma unroll
      for (int u = 0; u < EPV; ++u) sYa[sgi][cgi * EPV + u] = ya[u];
    }
    __syncthreads();

    if (tid < D) {
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) o += sO[r][tid];
      float ya = 0.f;
#pragma unroll
      for (int r = 0; r < NSG; ++r) ya += sYa[r][tid];
      ya /= sDen;
      reinterpret_cast<T*>(a.y)[tok + tid] = from_f32<T>(o + a.alpha * ya);
    }
  }
}

template <typename T, int D, bool LOGIT>
static void launch_decode_g(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.BH);
  if (a.T > 1) hipLaunchKernelGGL((lizard_decode_kernel<T, D, LOGIT, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((lizard_decode_kernel<T, D, LOGIT, false>), grid, dim3(256), 0, st, a);
}

template <typename T, int D>
static void launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  if (a.gate_logit) launch_decode_g<T, D, true>(a, st);
  else launch_decode_g<T, D, false>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int D, hipStream_t st) {
  if (dtype_bf16 && D == 128) launch_decode_t<bf16, 128>(a, st);
  else if (dtype_bf16 && D == 64) launch_decode_t<bf16, 64>(a, st);
  else if (!dtype_bf16 && D == 64) launch_decode_t<float, 64>(a, st);
  else if (!dtype_bf16 && D == 128) launch_decode_t<float, 128>(a, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lizard
