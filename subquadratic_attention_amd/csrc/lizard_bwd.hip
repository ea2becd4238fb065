// Backward pass of the Lizard hybrid attention layer on gfx950.
//
// The layer is trained end to end ("Lizard" explainer, gist.science (de),
// section 2 "Trainingsprozess"); this file computes the gradients of
// loss = sum(dY * Y) for Y = Y_gate + alpha * Y_anchor.  Notation as in the
// forward kernel: per chunk of 64 tokens, beta_t is the log2-gate prefix
// from the chunk start, B the chunk total, Qe = q*2^beta, Kp = k*2^-beta,
// Kh = k*2^{B-beta}, A[t][s] = Qe_t . Kp_s (s <= t), S_c the state entering
// chunk c and G_c = dL/dS_c.
//
//   gated branch, chunk c, dO = dY:
//     G_c    = diag(2^B) G_{c+1} + Qe^T dO
//     dA     = dO V^T (s <= t)
//     dq_t   = 2^{beta_t} * (S_c dO_t + sum_s dA_ts Kp_s)
//     dk_s   = 2^{-beta_s} * sum_t dA_ts Qe_t + 2^{B-beta_s} * (G_{c+1} v_s)
//     dv_s   = sum_t A_ts dO_t + G_{c+1}^T Kh_s
//     dlog_g_t = sum_{u >= t} (q_u * dq_u - k_u * dk_u)      (natural log)
//              = sum_{u >= t, u in c} (...) + rowsum(S_{c+1} * G_{c+1}),
//       the last term formed from S_c and the inter-chunk part of dk
//   anchor branch (softmax over the window and sinks, P = exp(z - lse)):
//     dP = alpha dY V^T (window; zero for sinks), D_t = sum P dP,
//     dZ = P (dP - D_t); dq += scale (dZ K + dZs mu); dk += scale dZ^T Q;
//     dv += alpha P^T dY; dmu += scale dZs^T Q (summed over batch and time)
//
// Kernels, in launch order (all on the caller's stream):
//   1. the forward kernel in its states-only mode writes S_c for every chunk;
//   2. bwd_dstate walks the chunks in reverse and writes G_{c+1} (and its
//      transpose) for every chunk;
//   3. bwd_anchor_q (per chunk of queries): D_t, the anchor part of dq
//      (written into dq), and per-chunk sink-key gradients;
//   4. bwd_anchor_k (per chunk of keys, queries of this and the next chunk):
//      the anchor parts of dk and dv (written into dk, dv);
//   5. bwd_gate (per chunk): the gated dq, dk, dv, added to the anchor parts
//      in the outputs, and dlog_g: the suffix sums of q*dq - k*dk inside the
//      chunk plus, for everything after it, rowsum(S_{c+1} * G_{c+1});
//   6. bwd_dmeta_reduce: sums the sink-key partials over batch and chunks in
//      a fixed order (deterministic, no float atomics); after the two walks
//      below, the launch that takes the flagged chunks also does this sum.
// Kernels 3-5 run the full chunks in one launch and a ragged last chunk in a
// range-checked launch of its own.  For bf16 at d = 128, two walks over each
// head's chunks replace kernels 2-5: the reverse walk (5, bf16) writes the
// gated dq, dk, dv and dlog_g, carrying G in registers, and the anchor walk
// (5b) adds the anchor parts to them.  Chunks whose decay span exceeds 2^184
// form the gated intra terms pairwise in fp32; spans between 2^92 and 2^184
// move each dimension's reference point to half its chunk total (as the
// forward pass does).
#include <type_traits>

#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

namespace {

constexpr int C = 64;
constexpr float kMaxSpan = 92.0f;   // log2 units, as in the forward kernel

template <typename T> __device__ __forceinline__ float elem_of(const uint4* raw, int i) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, raw[i >> 3]);
    return static_cast<float>(v[i & 7]);
  } else {
    const uint4 r = raw[i >> 2];
    const uint32_t u = (i & 3) == 0 ? r.x : (i & 3) == 1 ? r.y : (i & 3) == 2 ? r.z : r.w;
    return __builtin_bit_cast(float, u);
  }
}
template <typename T> __device__ __forceinline__ typename Mfma<T>::frag frag_of(const uint4* raw, int e) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, raw[e]);
  } else {
    return elem_of<float>(raw, e);
  }
}
// The lane's k-quarter [g*D/4, (g+1)*D/4) of global row `row` (zeros if the
// row is outside [0, L)).  GUARD = false: the caller guarantees the row is
// inside (no selects on the loaded data, which the compiler would otherwise
// place right after the loads and so wait for them early).
template <typename T, int D, bool GUARD = true>
__device__ __forceinline__ void load_quarter(uint4* raw, const T* base, int row, int L, int g) {
  constexpr int QV = D / 4 / (16 / sizeof(T));
  const bool ok = !GUARD || (row >= 0 && row < L);
  const T* p = base + (size_t)(ok ? row : 0) * D + g * (D / 4);
#pragma unroll
  for (int e = 0; e < QV; ++e) {
    const uint4 r = ld16(p + e * (16 / sizeof(T)));
    raw[e] = ok ? r : make_uint4(0, 0, 0, 0);
  }
}
// Lane group g's interleaved share of row `row` (zeros if the row is outside
// [0, L)): raw[e] holds the 16 bytes at values (4e + g) * V .. + V - 1, V =
// 16 / sizeof(T) (bf16 d = 128: values 8g + 32e .. + 7).  The transposing
// reads that pair with it then take LDS rows 8 apart across the lane groups
// (a quarter's rows would be 32 apart, which puts the groups on one bank set).
template <typename T, int D, bool GUARD = true>
__device__ __forceinline__ void load_interleaved(uint4* raw, const T* base, int row, int L, int g) {
  constexpr int V = 16 / sizeof(T);
  constexpr int QV = D / 4 / V;
  const bool ok = !GUARD || (row >= 0 && row < L);
  const T* p = base + (size_t)(ok ? row : 0) * D + g * V;
#pragma unroll
  for (int e = 0; e < QV; ++e) {
    const uint4 r = ld16(p + 4 * e * V);
    raw[e] = ok ? r : make_uint4(0, 0, 0, 0);
  }
}
// The same quarter of row `row` clamped into [0, L): for rows that the
// caller masks out after the product (their values never reach a result),
// without the data selects of the guarded form.
template <typename T, int D>
__device__ __forceinline__ void load_quarter_clamped(uint4* raw, const T* base, int row, int L, int g) {
  load_quarter<T, D, false>(raw, base, min(max(row, 0), L - 1), L, g);
}
// element i of a packed 32-bit word of T values
template <typename T> __device__ __forceinline__ float elem32(uint32_t u, int i) {
  if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, u);
  else return __builtin_bit_cast(float, i == 0 ? (u << 16) : (u & 0xffff0000u));
}

// Stage rows [r0, r0 + NR) x columns [c0, c0 + COLS) of a [L, D] tensor into
// LDS transposed: dst[col * ld + row] (rows outside [0, L) are zero).  Each
// thread loads 32-bit words (VC columns) of RPT consecutive rows and writes
// 8-row runs with 16-byte stores.  scale multiplies every value.
template <typename T, int COLS, int NR, int NTH = 256>
struct StageT {
  static constexpr int VC = 4 / sizeof(T);
  static constexpr int VRW = COLS / VC;
  static constexpr int RPT = NR * VRW / NTH;   // 32-bit words per thread
  static_assert(RPT % 8 == 0 && RPT * NTH == NR * VRW, "stage_T shape");
};
template <typename T, int D, int COLS, int NR, int NTH = 256, bool GUARD = true>
__device__ __forceinline__ void stage_T_load(uint32_t* w, const T* src, int r0, int c0,
                                             int L) {
  typedef StageT<T, COLS, NR, NTH> S;
  const int tid = threadIdx.x;
  const int vj = tid % S::VRW;
  const int vs = tid / S::VRW;
#pragma unroll
  for (int rr = 0; rr < S::RPT; ++rr) {
    const int row = r0 + vs * S::RPT + rr;
    const bool ok = !GUARD || (row >= 0 && row < L);
    const uint32_t u = *reinterpret_cast<const uint32_t*>(src + (size_t)(ok ? row : 0) * D + c0 + S::VC * vj);
    w[rr] = ok ? u : 0u;
  }
}
template <typename T, int COLS, int NR, int NTH = 256, bool A8 = false>
__device__ __forceinline__ void stage_T_store(T* dst, int ld, const uint32_t* w,
                                              float scale) {
  typedef StageT<T, COLS, NR, NTH> S;
  constexpr int VC = S::VC, RPT = S::RPT;
  const int tid = threadIdx.x;
  const int vj = tid % S::VRW;
  const int vs = tid / S::VRW;
#pragma unroll
  for (int cc = 0; cc < VC; ++cc)
#pragma unroll
    for (int b = 0; b < RPT / 8; ++b) {
      float v8[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) v8[rr] = elem32<T>(w[8 * b + rr], cc) * scale;
      T* d = dst + (VC * vj + cc) * ld + vs * RPT + 8 * b;
      if constexpr (A8) {   // rows only 8-byte aligned: two 8-byte stores
        store_pack<T, 4>(d, v8);
        store_pack<T, 4>(d + 4, v8 + 4);
      } else {
        store_pack<T, 8>(d, v8);
      }
    }
}
template <typename T, int D, int COLS, int NR, int NTH = 256>
__device__ __forceinline__ void stage_T(T* dst, int ld, const T* src, int r0, int c0, int L, float scale) {
  uint32_t w[StageT<T, COLS, NR, NTH>::RPT];
  stage_T_load<T, D, COLS, NR, NTH>(w, src, r0, c0, L);
  stage_T_store<T, COLS, NR, NTH>(dst, ld, w, scale);
}

// Block -> (bh, chunk) with every chunk of one head on the same XCD.
__device__ __forceinline__ bool chunk_block(int BH, int nc, int& bh, int& c) {
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int idx = x >> 3;
  c = idx % nc;
  bh = (idx / nc) * 8 + xcd;
  return bh < BH;
}

// Chunk-local log2-gate prefix for 256 threads: thread (w, l) owns rows
// 16w..16w+15 and dims DPL*l..; returns beta (chunk-inclusive prefix) and B
// (chunk total) for those; sTot is [4][D] scratch.  Contains one barrier.
// The log-gates of those rows and dims (zero past L).
template <int D>
__device__ __forceinline__ void chunk_gates(const float* lg, int t0, int L, float (&lv)[16][D / 64]) {
  constexpr int DPL = D / 64;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int t = t0 + 16 * w + rr;
    const bool ok = t < L;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const float v = lg[(size_t)(ok ? t : 0) * D + DPL * l + dd];
      lv[rr][dd] = ok ? v : 0.f;
    }
  }
}
// The prefix from gates loaded by chunk_gates.
template <int D>
__device__ __forceinline__ void chunk_prefix_of(const float (&lv)[16][D / 64], float* sTot,
                                                float (&beta)[16][D / 64], float (&Bt)[D / 64]) {
  constexpr int DPL = D / 64;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  float tot[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) tot[dd] = 0.f;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      tot[dd] += log2_gate(lv[rr][dd]);
      beta[rr][dd] = tot[dd];
    }
  }
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) sTot[w * D + DPL * l + dd] = tot[dd];
  __syncthreads();
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    const int i = DPL * l + dd;
    const float a0 = sTot[i], a1 = sTot[D + i], a2 = sTot[2 * D + i], a3 = sTot[3 * D + i];
    const float off = w == 0 ? 0.f : w == 1 ? a0 : w == 2 ? a0 + a1 : a0 + a1 + a2;
    Bt[dd] = a0 + a1 + a2 + a3;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) beta[rr][dd] += off;
  }
}

template <int D>
__device__ __forceinline__ void chunk_prefix(const float* lg, int t0, int L, float* sTot,
                                             float (&beta)[16][D / 64], float (&Bt)[D / 64]) {
  float lv[16][D / 64];
  chunk_gates<D>(lg, t0, L, lv);
  chunk_prefix_of<D>(lv, sTot, beta, Bt);
}

}  // namespace

// ---------------------------------------------------------------------------
// 2. reverse state-gradient pass: G_c = diag(2^B) G_{c+1} + Qe^T dO
// ---------------------------------------------------------------------------
template <typename T, int D, int DV, bool LOGIT>
__global__ __launch_bounds__(256, 1) void bwd_dstate_kernel(BwdArgs a) {
  typedef Mfma<T> M;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LDQ = 64 + PAD;
  constexpr int NCT = DV / 16;
  constexpr int NRT = D / 64;
  constexpr int DPL = D / 64;
  __shared__ __align__(16) T sQeT[D * LDQ];
  __shared__ __align__(16) T sdOT[DV * LDQ];
  __shared__ float sTot[4 * D];
  __shared__ float sBexp[D];
  // G_{c+1}'s block (rows 0..D, columns j0..j0+DV) and its transpose, staged
  // so that both leave in whole 16-byte rows
  constexpr int LDG = DV + PAD, LDT = D + PAD;
  __shared__ __align__(16) T sG[D * LDG];
  __shared__ __align__(16) T sGT[DV * LDT];

  const int nsplit = D / DV;
  const int x = blockIdx.x, xcd = x & 7, idx = x >> 3;
  const int split = idx % nsplit;
  const int bh = (idx / nsplit) * 8 + xcd;
  if (bh >= a.BH) return;
  const int j0 = split * DV;
  const int L = a.L, nc = (L + C - 1) / C;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* dyg = reinterpret_cast<const T*>(a.dy) + (size_t)bh * L * D;
  const float* lgg = LOGIT ? nullptr : a.log_g + (size_t)bh * L * D;
  const T* xg = LOGIT ? reinterpret_cast<const T*>(a.gate_logit) + (size_t)bh * L * D : nullptr;
  T* Gg = reinterpret_cast<T*>(a.ws_dS) + (size_t)bh * nc * D * D;
  T* GTg = reinterpret_cast<T*>(a.ws_dST) + (size_t)bh * nc * D * D;

  f32x4 acc[NRT][NCT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = zero4();

  // one chunk's inputs, loaded a chunk ahead: log-gates and queries of rows
  // 16w + rr, dims DPL*l..; dO words for the transposed staging
  typedef StageT<T, DV, 64> ST;
  float lv[16][DPL];
  uint32_t xv[16];      // gate logits (DPL elements packed), when the gates come as logits
  uint32_t qv[16];
  uint32_t dyw[ST::RPT];
  auto load = [&](int c) __attribute__((always_inline)) {
    const int t0 = c * C;
    if constexpr (LOGIT) {
      // raw bits; past L a logit of +inf (a gate of one, log gate 0)
      constexpr uint32_t kInf = sizeof(T) == 4 ? 0x7f800000u : 0x7f807f80u;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int t = t0 + 16 * w + rr;
        const bool ok = t < L;
        const T* xp = xg + (size_t)(ok ? t : 0) * D + DPL * l;
        uint32_t u;
        if constexpr (DPL * sizeof(T) == 4) u = *reinterpret_cast<const uint32_t*>(xp);
        else u = *reinterpret_cast<const uint16_t*>(xp);
        xv[rr] = ok ? u : kInf;
      }
    } else {
      chunk_gates<D>(lgg, t0, L, lv);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = t0 + 16 * w + rr;
      const bool ok = t < L;
      const T* qp = qg + (size_t)(ok ? t : 0) * D + DPL * l;
      uint32_t u;
      if constexpr (DPL * sizeof(T) == 4) u = *reinterpret_cast<const uint32_t*>(qp);
      else u = *reinterpret_cast<const uint16_t*>(qp);
      qv[rr] = ok ? u : 0u;
    }
    stage_T_load<T, D, DV, 64>(dyw, dyg, t0, j0, L);
  };
  if (nc > 0) load(nc - 1);

  for (int c = nc - 1; c >= 0; --c) {
    // chunk c's operands from the registers: Qe^T and dO^T into LDS
    if constexpr (LOGIT) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) lv[rr][dd] = log_sigmoid(elem32<T>(xv[rr], dd));
    }
    float beta[16][DPL], Bt[DPL];
    chunk_prefix_of<D>(lv, sTot, beta, Bt);
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      float qe[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float qf = elem32<T>(qv[rr], dd);
        qe[rr] = qf * exp_2(beta[rr][dd]);
      }
      store_pack<T, 16>(sQeT + i * LDQ + 16 * w, qe);
      if (w == 0) sBexp[i] = exp_2(Bt[dd]);
    }
    stage_T_store<T, DV, 64>(sdOT, LDQ, dyw, 1.0f);
    // G_{c+1} from the accumulators: rows i, columns j (row-major) and its transpose
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int i = w * (D / 4) + 16 * rt + 4 * g;
        const int jl = 16 * ct + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) sG[(i + r) * LDG + jl] = from_f32<T>(acc[rt][ct][r]);
        const float v4[4] = {acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]};
        store_pack<T, 4>(sGT + jl * LDT + i, v4);
      }
    // the next chunk's loads fly while this one is stored and multiplied
    if (c > 0) load(c - 1);
    __syncthreads();
    {
      typedef uint4 V;
      constexpr int E = 16 / sizeof(T);            // elements per 16-byte vector
      constexpr int GR = DV / E, TR = D / E;       // vectors per row of G's block and of G^T's
      static_assert((D * GR) % 256 == 0 && (DV * TR) % 256 == 0, "whole passes");
      T* G = Gg + (size_t)c * D * D;
      T* GT = GTg + (size_t)c * D * D;
#pragma unroll
      for (int p = 0; p < D * GR / 256; ++p) {
        const int u = 256 * p + tid, row = u / GR, col = (u % GR) * E;
        *reinterpret_cast<V*>(G + (size_t)row * D + j0 + col) = *reinterpret_cast<const V*>(sG + row * LDG + col);
      }
#pragma unroll
      for (int p = 0; p < DV * TR / 256; ++p) {
        const int u = 256 * p + tid, row = u / TR, col = (u % TR) * E;
        *reinterpret_cast<V*>(GT + (size_t)(j0 + row) * D + col) = *reinterpret_cast<const V*>(sGT + row * LDT + col);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int ib = w * (D / 4) + 16 * rt;
      float dec[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) dec[r] = sBexp[ib + 4 * g + r];
      const T* ap = sQeT + (ib + m) * LDQ + g * 16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 s = acc[rt][ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] *= dec[r];
        const T* bp = sdOT + (16 * ct + m) * LDQ + g * 16;
#pragma unroll
        for (int e = 0; e < 16 / M::KPL; ++e) s = M::mma(M::load(ap + e * M::KPL), M::load(bp + e * M::KPL), s);
        acc[rt][ct] = s;
      }
    }
    __syncthreads();
  }
}

// The window's key (or query) tiles of 16 around a block of 16 queries (or
// keys): a query reaches back at most 63 keys, so 80 positions cover a block.
constexpr int kWinTiles = 5;

// Fragment e of a window-ordered operand row: the MFMA contraction runs over
// the 80 window positions (keys for the query side, queries for the key
// side) in the order the score tiles leave them in a lane's registers (value
// v = 4 kt + r of lane group g is position 16 kt + 4 g + r), so the scores
// feed the next product from registers; the other operand (row p of a
// transposed tile, positions from q0) is gathered in that order.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag window_frag(const T* p, int q0, int g, int e) {
  typedef Mfma<T> M;
  if constexpr (sizeof(T) == 2) {
    // values 8e .. 8e+7: tiles 2e and 2e+1, four consecutive positions each;
    // the window has five tiles, so the last step's second half is zero
    const uint2 a = *reinterpret_cast<const uint2*>(p + q0 + 32 * e + 4 * g);
    const uint2 b = 2 * e + 1 < kWinTiles ? *reinterpret_cast<const uint2*>(p + q0 + 32 * e + 16 + 4 * g)
                                          : make_uint2(0u, 0u);
    return __builtin_bit_cast(typename M::frag, make_uint4(a.x, a.y, b.x, b.y));
  } else {
    return p[q0 + 16 * (e >> 2) + 4 * g + (e & 3)];
  }
}
// MFMA steps over the window values (bf16: 8 per step, the last one half
// used; fp32: one per step)
template <typename T> constexpr int window_steps() { return sizeof(T) == 2 ? 3 : 4 * kWinTiles; }

// Fragment of the sink operand row p (16 sinks) in the same register order:
// lane group g holds sinks 4g .. 4g + 3 (bf16: one step, the other four
// slots zero; fp32: step e is sink 4g + e).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag sink_frag(const T* p, int g, int e) {
  typedef Mfma<T> M;
  if constexpr (sizeof(T) == 2) {
    const uint2 a = *reinterpret_cast<const uint2*>(p + 4 * g);
    return __builtin_bit_cast(typename M::frag, make_uint4(a.x, a.y, 0u, 0u));
  } else {
    return p[4 * g + e];
  }
}

// Transposing LDS read (bf16): within each 16-lane group, lane j reads the
// 8 bytes at its address and receives, in slot k, value j % 4 of the 8 bytes
// lane 4k + j / 4 of its group read.  So if lane j reads row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3 of a row-major tile X, lane j receives
// X[r0 .. r0 + 3][c0 + j]: four consecutive k of column j, as an MFMA
// operand wants them from a tile stored [k][n].
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_tr(const bf16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(uint2, r);
}
// The operand fragment of rows k0 .. k0 + 7 of column c0 + (lane % 16) of a
// row-major bf16 tile with ld values per row; p = tile + c0.
__device__ __forceinline__ bf16x8 frag_tr(const bf16* p, int ld, int k0, int j) {
  const bf16* a = p + (k0 + (j >> 2)) * ld + 4 * (j & 3);
  const uint2 lo = ld_tr(a), hi = ld_tr(a + 4 * ld);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// ---------------------------------------------------------------------------
// 3. anchor branch, query side (per chunk of queries)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct AqLayout {
  static constexpr int PAD = 16 / sizeof(T);
  // bf16: the logit tiles' key and value operands come from the transposed
  // window tiles by transposing LDS reads (fp32: from memory, per wavefront)
  static constexpr bool TR = sizeof(T) == 2;
  static constexpr int LDKT = 128 + PAD;   // sKT, sVT [D][LDKT]: window keys / values transposed
  static constexpr int LDMT = 16 + PAD;    // sMuT [D][LDMT]: sink keys transposed (zero padded)
  static constexpr int LDQ = D + PAD;      // sQ [64][LDQ]
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_Q = 0;          // after the dq products, the chunk's queries replace the keys
  static_assert(64 * LDQ <= D * LDKT, "query rows fit in the key tile");
  static constexpr int OFF_VT = OFF_KT + a16(D * LDKT * (int)sizeof(T));
  static constexpr int OFF_MT = OFF_VT + (TR ? a16(D * LDKT * (int)sizeof(T)) : 0);
  static constexpr int OFF_DZS = OFF_MT + a16(D * LDMT * (int)sizeof(T));   // sink dZ, fp32 [64][16]
  static constexpr int TOTAL = OFF_DZS + a16(64 * 16 * 4);
};

// The grid covers chunks cb .. cb + ncl - 1; GUARD = false: they are full
// (every query inside [0, L)); window keys before position 0 (chunk 0) are
// read from row 0 and masked out with the rest of the window.
template <typename T, int D, bool GUARD>
__global__ __launch_bounds__(256, 2) void bwd_anchor_q_kernel(BwdArgs a, int cb, int ncl) {
  typedef AqLayout<T, D> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int QV = D / 4 / EPV;
  constexpr int NF = D / 4 / M::KPL;
  constexpr int NDT = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  T* sKT = reinterpret_cast<T*>(smem + Lay::OFF_KT);
  T* sVT = reinterpret_cast<T*>(smem + Lay::OFF_VT);
  T* sMuT = reinterpret_cast<T*>(smem + Lay::OFF_MT);
  T* sQ = reinterpret_cast<T*>(smem + Lay::OFF_Q);
  float* sdZs = reinterpret_cast<float*>(smem + Lay::OFF_DZS);

  const int L = a.L, nc = (L + C - 1) / C;
  int bh, c;
  if (!chunk_block(a.BH, ncl, bh, c)) return;
  c += cb;
  const int h = bh % a.H;
  const int t0 = c * C;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  const T* dyg = reinterpret_cast<const T*>(a.dy) + (size_t)bh * L * D;
  const T* mug = reinterpret_cast<const T*>(a.meta) + (size_t)h * a.n_meta * D;
  const float sl2 = a.scale * kLog2e;

  const int I = w;
  const int tme = t0 + 16 * I + m;
  const int U0 = 16 * I;                  // first window key of the tiles (of [t0 - 64, t0 + 64))
  // this lane's query and dY row; fp32: the window keys / values of its
  // first three tiles, issued before the staging (their loads then overlap
  // it), the other tiles reuse the registers
  constexpr bool TR = Lay::TR;
  // (bf16: the interleaved share; its step e covers values 8g + 32e .. + 7)
  uint4 qraw[QV], dyraw[QV];
  if constexpr (TR) {
    load_interleaved<T, D, GUARD>(qraw, qg, tme, L, g);
    load_interleaved<T, D, GUARD>(dyraw, dyg, tme, L, g);
  } else {
    load_quarter<T, D, GUARD>(qraw, qg, tme, L, g);
    load_quarter<T, D, GUARD>(dyraw, dyg, tme, L, g);
  }
  uint4 kraw[TR ? 1 : 3][QV], vraw[TR ? 1 : 3][QV];
  auto load_tiles = [&](int k0, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < n; ++kk) {
      const int s = t0 - 64 + U0 + 16 * (k0 + kk) + m;   // key row of this lane (MFMA row)
      if constexpr (GUARD) {
        load_quarter<T, D>(kraw[kk], kg, s, L, g);
        load_quarter<T, D>(vraw[kk], vg, s, L, g);
      } else {
        load_quarter_clamped<T, D>(kraw[kk], kg, s, L, g);
        load_quarter_clamped<T, D>(vraw[kk], vg, s, L, g);
      }
    }
  };
  if constexpr (!TR) load_tiles(0, 3);
  const float lse2 = !GUARD || tme < L ? a.lse[(size_t)bh * L + (tme < L ? tme : 0)] * kLog2e : 0.f;

  // window keys [t0 - 64, t0 + 64) transposed; sink keys transposed
  // (the sink rows, slots 0 .. 15 of the tile, the ones the products read:
  // one 16-byte run of one sink per item, every load issued before the
  // first store, so the whole tile waits for one round trip)
  constexpr int MPI = 16 / sizeof(T);             // values per item
  constexpr int MIT = 16 * D / MPI;               // items: 16 sink slots x D / MPI runs
  constexpr int MPT = (MIT + 255) / 256;          // items per thread
  uint4 mv[MPT];
#pragma unroll
  for (int p = 0; p < MPT; ++p) {
    const int it = tid + 256 * p, s = it / (D / MPI), j = it % (D / MPI);
    mv[p] = it < MIT && s < a.n_meta ? ld16(mug + (size_t)s * D + MPI * j) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int p = 0; p < MPT; ++p) {
    const int it = tid + 256 * p, s = it / (D / MPI), j = it % (D / MPI);
    const T* pv = reinterpret_cast<const T*>(&mv[p]);
    if (it < MIT) {
#pragma unroll
      for (int e = 0; e < MPI; ++e) sMuT[(MPI * j + e) * Lay::LDMT + s] = pv[e];
    }
  }
  if constexpr (TR) {
    // keys and values of the window, every load issued before the first store
    uint32_t wk[StageT<T, D, 128>::RPT], wv[StageT<T, D, 128>::RPT];
    stage_T_load<T, D, D, 128>(wk, kg, t0 - 64, 0, L);
    stage_T_load<T, D, D, 128>(wv, vg, t0 - 64, 0, L);
    stage_T_store<T, D, 128>(sKT, Lay::LDKT, wk, 1.0f);
    stage_T_store<T, D, 128>(sVT, Lay::LDKT, wv, 1.0f);
  } else {
    stage_T<T, D, D, 128>(sKT, Lay::LDKT, kg, t0 - 64, 0, L, 1.0f);
  }
  __syncthreads();

  // logits Z^T[u][t] and value products dP^T[u][t] for window keys u
  f32x4 z[kWinTiles], dp[kWinTiles];
  if constexpr (TR) {
    // key / value rows u = U0 + 16 kk + m of the window over the lane group's
    // dims 8g + 32e .. + 7, those of its share of the query row
#pragma unroll
    for (int kk = 0; kk < kWinTiles; ++kk) {
      f32x4 zc = zero4(), pc = zero4();
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        zc = M::mma(frag_tr(sKT + U0 + 16 * kk, Lay::LDKT, 8 * g + 32 * e, m), frag_of<T>(qraw, e), zc);
        pc = M::mma(frag_tr(sVT + U0 + 16 * kk, Lay::LDKT, 8 * g + 32 * e, m), frag_of<T>(dyraw, e), pc);
      }
      z[kk] = zc;
      dp[kk] = pc;
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1) load_tiles(3, kWinTiles - 3);
#pragma unroll
      for (int kk = 0; kk < (half == 0 ? 3 : kWinTiles - 3); ++kk) {
        f32x4 zc = zero4(), pc = zero4();
#pragma unroll
        for (int e = 0; e < NF; ++e) {
          zc = M::mma(frag_of<T>(kraw[kk], e), frag_of<T>(qraw, e), zc);
          pc = M::mma(frag_of<T>(vraw[kk], e), frag_of<T>(dyraw, e), pc);
        }
        z[3 * half + kk] = zc;
        dp[3 * half + kk] = pc;
      }
    }
  }
  f32x4 zs = zero4();
  if (a.n_meta > 0) {
    if constexpr (TR) {
#pragma unroll
      for (int e = 0; e < NF; ++e)
        zs = M::mma(frag_tr(sMuT, Lay::LDMT, 8 * g + 32 * e, m), frag_of<T>(qraw, e), zs);
    } else {
      uint4 mraw[QV];
      load_quarter<T, D>(mraw, mug, m < a.n_meta ? m : -1, a.n_meta, g);
#pragma unroll
      for (int e = 0; e < NF; ++e) zs = M::mma(frag_of<T>(mraw, e), frag_of<T>(qraw, e), zs);
    }
  }
  // probabilities from the forward normaliser, D_t, dZ
  float dsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < kWinTiles; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = t0 - 64 + U0 + 16 * kt + 4 * g + r;
      const bool ok = s >= 0 && s <= tme && s > tme - a.window && tme < L;
      const float p = ok ? exp_2(z[kt][r] * sl2 - lse2) : 0.f;
      z[kt][r] = p;
      dp[kt][r] *= a.alpha;
      dsum += p * dp[kt][r];
    }
  const float Dt = xgroup_sum(dsum);
  if (g == 0 && tme < L) a.ws_D[(size_t)bh * L + tme] = Dt;
  float ps[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    ps[r] = (4 * g + r < a.n_meta && tme < L) ? exp_2(zs[r] * sl2 - lse2) : 0.f;
  // dZ[t][u] of the lane's query over its 24 window keys, as operand
  // fragments in the window order, and the sink part dZs[t][i] = -P D_t
  constexpr int NWS = window_steps<T>();
  float dz[NWS * M::KPL];
#pragma unroll
  for (int kt = 0; kt < kWinTiles; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dz[4 * kt + r] = z[kt][r] * (dp[kt][r] - Dt);
#pragma unroll
  for (int v = 4 * kWinTiles; v < NWS * M::KPL; ++v) dz[v] = 0.f;
  typename M::frag zf[NWS];
#pragma unroll
  for (int e = 0; e < NWS; ++e) zf[e] = M::pack(dz + e * M::KPL);
  float zsv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    zsv[r] = -ps[r] * Dt;
    sdZs[(16 * I + m) * 16 + 4 * g + r] = zsv[r];
  }
  constexpr int NS = sizeof(T) == 2 ? 1 : 4;      // sink steps
  typename M::frag sf[NS];
#pragma unroll
  for (int e = 0; e < NS; ++e) sf[e] = M::pack(zsv + e * M::KPL);
  // dq^T[d][t] = scale (K^T dZ^T + mu^T dZs^T)
  T* dqa = reinterpret_cast<T*>(a.dq) + (size_t)bh * L * D;   // the anchor part
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    f32x4 o = zero4();
    const T* ap = sKT + (16 * dt + m) * Lay::LDKT;
#pragma unroll
    for (int e = 0; e < NWS; ++e) o = M::mma(window_frag<T>(ap, U0, g, e), zf[e], o);
    const T* az = sMuT + (16 * dt + m) * Lay::LDMT;
#pragma unroll
    for (int e = 0; e < NS; ++e) o = M::mma(sink_frag<T>(az, g, e), sf[e], o);
    if (tme < L) {
      float v4[4] = {o[0] * a.scale, o[1] * a.scale, o[2] * a.scale, o[3] * a.scale};
      store_pack<T, 4>(dqa + (size_t)tme * D + 16 * dt + 4 * g, v4);
    }
  }
  // per-chunk sink-key gradient dmu^T[d][i] = scale sum_t q[t][d] dZs[t][i],
  // on the matrix cores: the chunk's query rows (from the registers) replace
  // the key tile; wavefront w takes dim tiles w, w + 4, ...
  if (a.n_meta > 0) {
    __syncthreads();                      // the key tile is free
#pragma unroll
    for (int e = 0; e < QV; ++e)
      st16(sQ + (16 * I + m) * Lay::LDQ + (TR ? (g + 4 * e) * EPV : g * (D / 4) + e * EPV), qraw[e]);
    __syncthreads();
    float* part = a.ws_dmu + ((size_t)bh * nc + c) * a.n_meta * D;
#pragma unroll
    for (int dt = w; dt < NDT; dt += 4) {
      f32x4 o = zero4();
#pragma unroll
      for (int e = 0; e < 64 / M::KSTEP; ++e) {
        float qa[M::KPL], za[M::KPL];
#pragma unroll
        for (int u = 0; u < M::KPL; ++u) {
          const int t = e * M::KSTEP + g * M::KPL + u;
          qa[u] = to_f32(sQ[t * Lay::LDQ + 16 * dt + m]);
          za[u] = sdZs[t * 16 + m];
        }
        o = M::mma(M::pack(qa), M::pack(za), o);
      }
      // lane: dims 16 dt + 4 g + r of sink m
      if (m < a.n_meta) {
        const float v4[4] = {o[0] * a.scale, o[1] * a.scale, o[2] * a.scale, o[3] * a.scale};
        *reinterpret_cast<float4*>(part + (size_t)m * D + 16 * dt + 4 * g) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4. anchor branch, key side (per chunk of keys; queries of this and the next chunk)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct AkLayout {
  static constexpr int PAD = 16 / sizeof(T);
  // sQT, sdYT [D][LDT].  bf16: rows of 296 bytes, so that both ways they are
  // read, transposing reads (four rows per 16-lane group, the groups 32 rows
  // apart) and pairs of 8-byte runs 32 bytes apart on 16 consecutive rows,
  // spread over the LDS banks (272-byte rows conflict on both); the rows are
  // then only 8-byte aligned and are staged with 8-byte stores
  static constexpr bool A8 = sizeof(T) == 2;
  static constexpr int LDT = 128 + (A8 ? 20 : PAD);
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_QT = 0;
  static constexpr int OFF_DYT = OFF_QT + a16(D * LDT * (int)sizeof(T));
  static constexpr int OFF_RW = OFF_DYT + a16(D * LDT * (int)sizeof(T));   // lse*log2e, D_t: [2][128] fp32
  static constexpr int TOTAL = OFF_RW + a16(2 * 128 * 4);
};

// The grid covers chunks cb .. cb + ncl - 1; GUARD = false: they are full
// (every key inside [0, L)); window queries past L (the last full chunk's
// next chunk) are read from row L - 1 and masked out.  Two workgroups per CU.
template <typename T, int D, bool GUARD>
__global__ __launch_bounds__(256, 2) void bwd_anchor_k_kernel(BwdArgs a, int cb, int ncl) {
  typedef AkLayout<T, D> Lay;
  typedef Mfma<T> M;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int QV = D / 4 / EPV;
  constexpr int NF = D / 4 / M::KPL;
  constexpr int NDT = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  T* sQT = reinterpret_cast<T*>(smem + Lay::OFF_QT);
  T* sdYT = reinterpret_cast<T*>(smem + Lay::OFF_DYT);
  float* sLse = reinterpret_cast<float*>(smem + Lay::OFF_RW);
  float* sD = sLse + 128;

  const int L = a.L;
  int bh, c;
  if (!chunk_block(a.BH, ncl, bh, c)) return;
  c += cb;
  const int t0 = c * C;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  const T* dyg = reinterpret_cast<const T*>(a.dy) + (size_t)bh * L * D;
  const float sl2 = a.scale * kLog2e;

  const int J = w;                        // key block
  const int sme = t0 + 16 * J + m;        // this lane's key
  const int Q0 = 16 * J;                  // first window query of the tiles (relative to t0)
  // this lane's key and value rows, issued before the staging
  uint4 kraw[QV], vraw[QV];
  load_quarter<T, D, GUARD>(kraw, kg, sme, L, g);
  load_quarter<T, D, GUARD>(vraw, vg, sme, L, g);

  // the query operands of the logit tiles (queries on the MFMA rows): bf16,
  // from the staged transposed tiles by transposing LDS reads; fp32, rows
  // loaded from memory one tile ahead
  constexpr bool TR = sizeof(T) == 2;
  constexpr int NB = TR ? 1 : 2;
  uint4 qraw[NB][QV], dyraw[NB][QV];
  auto load_query = [&](uint4* qr, uint4* dr, int t) __attribute__((always_inline)) {
    if constexpr (GUARD) {
      load_quarter<T, D>(qr, qg, t, L, g);
      load_quarter<T, D>(dr, dyg, t, L, g);
    } else {
      load_quarter_clamped<T, D>(qr, qg, t, L, g);
      load_quarter_clamped<T, D>(dr, dyg, t, L, g);
    }
  };
  if constexpr (!TR) {
#pragma unroll
    for (int kt = 0; kt < NB - 1; ++kt) load_query(qraw[kt], dyraw[kt], t0 + Q0 + 16 * kt + m);
  }
  // queries [t0, t0 + 128): transposed q and dY, lse (log2 units) and D_t;
  // every load issued before the first store
  {
    uint32_t wq[StageT<T, D, 128>::RPT], wy[StageT<T, D, 128>::RPT];
    stage_T_load<T, D, D, 128>(wq, qg, t0, 0, L);
    stage_T_load<T, D, D, 128>(wy, dyg, t0, 0, L);
    float lse_t = 0.f, d_t = 0.f;
    if (tid < 128) {
      const int t = t0 + tid;
      if (t < L) {
        lse_t = a.lse[(size_t)bh * L + t] * kLog2e;
        d_t = a.ws_D[(size_t)bh * L + t];
      }
    }
    stage_T_store<T, D, 128, 256, Lay::A8>(sQT, Lay::LDT, wq, 1.0f);
    stage_T_store<T, D, 128, 256, Lay::A8>(sdYT, Lay::LDT, wy, 1.0f);
    if (tid < 128) {
      sLse[tid] = lse_t;
      sD[tid] = d_t;
    }
  }
  __syncthreads();

  // Z[t][s] and dP[t][s] tiles
  f32x4 z[kWinTiles], dp[kWinTiles];
#pragma unroll
  for (int kt = 0; kt < kWinTiles; ++kt) {
    f32x4 zc = zero4(), pc = zero4();
    if constexpr (TR) {
      // rows t = Q0 + 16 kt + m of q and dY over the lane group's dims
      // (D / 4) g + 8 e .. + 7, the dims of its quarter of the key row
      const T* qp = sQT + Q0 + 16 * kt;
      const T* yp = sdYT + Q0 + 16 * kt;
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        zc = M::mma(frag_tr(qp, Lay::LDT, (D / 4) * g + 8 * e, m), frag_of<T>(kraw, e), zc);
        pc = M::mma(frag_tr(yp, Lay::LDT, (D / 4) * g + 8 * e, m), frag_of<T>(vraw, e), pc);
      }
    } else {
      if (kt + NB - 1 < kWinTiles)
        load_query(qraw[(kt + NB - 1) % NB], dyraw[(kt + NB - 1) % NB], t0 + Q0 + 16 * (kt + NB - 1) + m);
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        zc = M::mma(frag_of<T>(qraw[kt % NB], e), frag_of<T>(kraw, e), zc);
        pc = M::mma(frag_of<T>(dyraw[kt % NB], e), frag_of<T>(vraw, e), pc);
      }
    }
    z[kt] = zc;
    dp[kt] = pc;
  }
  // dZ and P of key sme for the lane's 20 window queries, kept as operand
  // fragments in the window order (value 4 kt + r; zero past the window)
  constexpr int NWS = window_steps<T>();
  float pz[NWS * M::KPL], pp[NWS * M::KPL];
#pragma unroll
  for (int v = 4 * kWinTiles; v < NWS * M::KPL; ++v) pz[v] = pp[v] = 0.f;
#pragma unroll
  for (int kt = 0; kt < kWinTiles; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = Q0 + 16 * kt + 4 * g + r;   // query relative to t0
      const int t = t0 + tr;
      const bool ok = t < L && sme < L && t >= sme && t < sme + a.window;
      const float p = ok ? exp_2(z[kt][r] * sl2 - sLse[tr]) : 0.f;
      pz[4 * kt + r] = p * (dp[kt][r] * a.alpha - sD[tr]);
      pp[4 * kt + r] = p * a.alpha;
    }
  }
  typename M::frag zf[NWS], pf[NWS];
#pragma unroll
  for (int e = 0; e < NWS; ++e) {
    zf[e] = M::pack(pz + e * M::KPL);
    pf[e] = M::pack(pp + e * M::KPL);
  }
  // the anchor parts of dk and dv
  T* dka = reinterpret_cast<T*>(a.dk) + (size_t)bh * L * D;
  T* dva = reinterpret_cast<T*>(a.dv) + (size_t)bh * L * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    f32x4 ok_ = zero4(), ov = zero4();
    const T* aq = sQT + (16 * dt + m) * Lay::LDT;
    const T* ay = sdYT + (16 * dt + m) * Lay::LDT;
#pragma unroll
    for (int e = 0; e < NWS; ++e) {
      ok_ = M::mma(window_frag<T>(aq, Q0, g, e), zf[e], ok_);
      ov = M::mma(window_frag<T>(ay, Q0, g, e), pf[e], ov);
    }
    if (sme < L) {
      float k4[4] = {ok_[0] * a.scale, ok_[1] * a.scale, ok_[2] * a.scale, ok_[3] * a.scale};
      float v4[4] = {ov[0], ov[1], ov[2], ov[3]};
      store_pack<T, 4>(dka + (size_t)sme * D + 16 * dt + 4 * g, k4);
      store_pack<T, 4>(dva + (size_t)sme * D + 16 * dt + 4 * g, v4);
    }
  }
}

// ---------------------------------------------------------------------------
// 5. gated branch (per chunk), combined with the anchor parts
// ---------------------------------------------------------------------------
template <typename T, int D>
struct GateLayout {
  static constexpr int NW = D / 16;        // wavefronts: one 16-dim tile each in the output phase
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDT = 64 + PAD;     // [D][LDT] transposed tiles; [64][LDT] staged scores
  static constexpr int LDB = D + 4;        // sBeta [64][LDB] fp32
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_B = 0;
  static constexpr int OFF_QT = OFF_B + a16(64 * LDB * 4);
  static constexpr int OFF_KT = OFF_QT + a16(D * LDT * (int)sizeof(T));
  static constexpr int OFF_OT = OFF_KT + a16(D * LDT * (int)sizeof(T));
  static constexpr int OFF_DA = OFF_OT + a16(D * LDT * (int)sizeof(T));
  static constexpr int OFF_DAT = OFF_DA + a16(64 * LDT * (int)sizeof(T));
  static constexpr int OFF_AT = OFF_DAT + a16(64 * LDT * (int)sizeof(T));
  static constexpr int LDR = D + PAD;      // [64][LDR] row-major token tiles
  static constexpr int OFF_KH = OFF_AT + a16(64 * LDT * (int)sizeof(T));
  static constexpr int OFF_QE = OFF_KH + a16(64 * LDR * (int)sizeof(T));
  static constexpr int OFF_TOT = OFF_QE + a16(64 * LDR * (int)sizeof(T));
  static constexpr int OFF_BX = OFF_TOT + a16(NW * D * 4);
  static constexpr int OFF_EB = OFF_BX + a16(D * 4);       // 2^B and 2^-B per dim
  static constexpr int TOTAL = OFF_EB + a16(2 * D * 4);
};

// One workgroup of D/16 wavefronts per (b*h, chunk).  Phase A: log-gate
// prefix and the chunk's operands in LDS; phase B: the intra-chunk score
// tiles dA, dA^T, A^T; phase C: wavefront w owns dims / value columns
// [16w, 16w + 16) of every token and writes dq, dk, dv, dlog_g.  The global
// loads of each phase are issued before the barrier that precedes it.  The
// grid covers chunks cb .. cb + ncl - 1; RAGGED: they may end past L (only
// the last chunk of a sequence does), so token rows are range-checked.
template <typename T, int D, bool RAGGED, bool LOGIT>
__device__ __forceinline__ void gate_chunk(const BwdArgs& a, const int bh, const int c) {
  typedef GateLayout<T, D> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int NW = Lay::NW;
  constexpr int NT = 64 * NW;
  constexpr int RPW = 64 / NW;            // prefix rows per wavefront
  constexpr int JPW = 16 / NW;            // phase B: blocks J per wavefront
  constexpr int EPV = 16 / sizeof(T);
  constexpr int QV = D / 4 / EPV;
  constexpr int NF = D / 4 / M::KPL;
  constexpr int DPL = D / 64;
  static_assert(NW == 4 || NW == 8, "gate kernel shape");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sBeta = reinterpret_cast<float*>(smem + Lay::OFF_B);
  T* sQT = reinterpret_cast<T*>(smem + Lay::OFF_QT);    // Qe^T (or q^T on the pairwise path)
  T* sKT = reinterpret_cast<T*>(smem + Lay::OFF_KT);    // Kp^T (or k^T on the pairwise path)
  T* sOT = reinterpret_cast<T*>(smem + Lay::OFF_OT);    // dO^T
  T* sDA = reinterpret_cast<T*>(smem + Lay::OFF_DA);    // dA[t][s]
  T* sDAT = reinterpret_cast<T*>(smem + Lay::OFF_DAT);  // dA^T[s][t]
  T* sAT = reinterpret_cast<T*>(smem + Lay::OFF_AT);    // A^T[s][t]
  T* sKh = reinterpret_cast<T*>(smem + Lay::OFF_KH);    // Kh[s][i] = k 2^{B - beta}, row-major
  T* sQe = reinterpret_cast<T*>(smem + Lay::OFF_QE);    // Qe[t][i] = q 2^{beta}, row-major
  float* sTot = reinterpret_cast<float*>(smem + Lay::OFF_TOT);
  float* sBx = reinterpret_cast<float*>(smem + Lay::OFF_BX);   // pairwise: chunk total B (log2); else 2^r per dim
  float* sEB = reinterpret_cast<float*>(smem + Lay::OFF_EB);   // fast path: [0][i] = 2^{B_i - r_i}, [1][i] = 2^{r_i - B_i}

  const int L = a.L, nc = (L + C - 1) / C;
  const int t0 = c * C;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, m = l & 15, g = l >> 4;
  constexpr bool RG = RAGGED;
  const T* __restrict__ qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  const T* __restrict__ dyg = reinterpret_cast<const T*>(a.dy) + (size_t)bh * L * D;
  const float* __restrict__ lgg = LOGIT ? nullptr : a.log_g + (size_t)bh * L * D;
  const T* __restrict__ xg = LOGIT ? reinterpret_cast<const T*>(a.gate_logit) + (size_t)bh * L * D : nullptr;
  const T* __restrict__ Sg = reinterpret_cast<const T*>(a.ws_states) + ((size_t)bh * nc + c) * D * D;
  const T* __restrict__ Gg = reinterpret_cast<const T*>(a.ws_dS) + ((size_t)bh * nc + c) * D * D;
  const T* __restrict__ GTg = reinterpret_cast<const T*>(a.ws_dST) + ((size_t)bh * nc + c) * D * D;
  T* __restrict__ dqo = reinterpret_cast<T*>(a.dq) + (size_t)bh * L * D;
  T* __restrict__ dko = reinterpret_cast<T*>(a.dk) + (size_t)bh * L * D;
  T* __restrict__ dvo = reinterpret_cast<T*>(a.dv) + (size_t)bh * L * D;
  float* __restrict__ dbo = LOGIT ? nullptr : a.dlog_g + (size_t)bh * L * D;
  T* __restrict__ dxo = LOGIT ? reinterpret_cast<T*>(a.dgate) + (size_t)bh * L * D : nullptr;
  const int ib = 16 * w;                  // phase C: first dim of this wavefront's tile


  // ---- phase A: log-gates, q and k of rows RPW*w + rr, dims DPL*l + dd ----
  float lv[RPW][DPL];
  uint32_t qw[RPW], kw[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int t = t0 + RPW * w + rr;
    const bool ok = !RG || t < L;
    const size_t ro = (size_t)(ok ? t : 0) * D + DPL * l;
    if constexpr (LOGIT) {
      uint32_t u;
      if constexpr (DPL * sizeof(T) == 4) u = *reinterpret_cast<const uint32_t*>(xg + ro);
      else u = *reinterpret_cast<const uint16_t*>(xg + ro);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) lv[rr][dd] = ok ? log_sigmoid(elem32<T>(u, dd)) : 0.f;
    } else if constexpr (DPL == 2) {
      const float2 f = *reinterpret_cast<const float2*>(lgg + ro);
      lv[rr][0] = ok ? f.x : 0.f;
      lv[rr][1] = ok ? f.y : 0.f;
    } else {
      const float f = lgg[ro];
      lv[rr][0] = ok ? f : 0.f;
    }
    uint32_t qu, ku;
    if constexpr (DPL * sizeof(T) == 4) {
      qu = *reinterpret_cast<const uint32_t*>(qg + ro);
      ku = *reinterpret_cast<const uint32_t*>(kg + ro);
    } else {
      qu = *reinterpret_cast<const uint16_t*>(qg + ro);
      ku = *reinterpret_cast<const uint16_t*>(kg + ro);
    }
    qw[rr] = ok ? qu : 0u;
    kw[rr] = ok ? ku : 0u;
  }
  uint32_t dyw[StageT<T, D, 64, NT>::RPT];
  stage_T_load<T, D, D, 64, NT, RG>(dyw, dyg, t0, 0, L);
  // phase B's rows: block I of this wavefront (see phase B)
  int I;
  if constexpr (NW == 8) {
    // (I, J) tiles cost about 1 (J < I), 2.5 (J > I) or 3.5 (J = I) units;
    // wavefronts w and w + 4 share a SIMD, so each SIMD gets two blocks I of
    // complementary cost: SIMD loads 8, 9.5, 9, 8.5 units
    I = w < 4 ? w >> 1 : (w < 6 ? 3 : 2);
  } else {
    I = w;
  }
  uint4 dyI[QV], vI[QV];
  load_quarter<T, D, RG>(dyI, dyg, t0 + 16 * I + m, L, g);
  load_quarter<T, D, RG>(vI, vg, t0 + 16 * I + m, L, g);
  uint4 Sr[QV], Gr[QV], GTr[QV];

  // prefix: inside the wavefront's rows, then across wavefronts
  float beta[RPW][DPL], off[DPL], Bt[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    float run = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      run += log2_gate(lv[rr][dd]);
      beta[rr][dd] = run;
    }
    sTot[w * D + DPL * l + dd] = run;
  }
  __syncthreads();
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    const int i = DPL * l + dd;
    off[dd] = 0.f;
    Bt[dd] = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float v = sTot[w2 * D + i];
      off[dd] += w2 < w ? v : 0.f;
      Bt[dd] += v;
    }
  }
  bool wide = false, wider = false;
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    wide |= -Bt[dd] > kMaxSpan;
    wider |= -Bt[dd] > 2.f * kMaxSpan;
  }
  // spans up to twice the limit stay factorised with each dimension's
  // reference point at half its chunk total r = B/2 (as in the forward
  // pass): the stored prefixes are b - r, Qe = q 2^{b-r}, Kp = k 2^{r-b},
  // and the epilogue restores 2^r on the inter-chunk dq term.  The key tile
  // then holds Kp, from which Kh = Kp 2^{B-r} is derived: Kp stays within
  // 2^{+-92}, while Kh may underflow where its true value is that small
  // (Kp derived from an underflowed Kh would be lost)
  const bool pairwise = __any(wider);
  const bool midref = !pairwise && __any(wide);
  float kh[RPW][DPL], qer[RPW][DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    const int i = DPL * l + dd;
    float qe[RPW], kp[RPW];
    if (!pairwise) {
      // every factor from one exponential per element and operand (Kh = Kp 2^{B-r})
      const float r = midref ? 0.5f * Bt[dd] : 0.f;
      const float eB = exp_2(Bt[dd] - r);
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const float b = beta[rr][dd] + off[dd] - r;
        qe[rr] = elem32<T>(qw[rr], dd) * exp_2(b);
        kp[rr] = elem32<T>(kw[rr], dd) * exp_2(-b);
        kh[rr][dd] = midref ? kp[rr] : kp[rr] * eB;
        qer[rr][dd] = qe[rr];
        sBeta[(RPW * w + rr) * Lay::LDB + i] = b;
      }
      if (w == 0) {
        sEB[i] = eB;
        sEB[D + i] = exp_2(r - Bt[dd]);
      }
    } else {
      // wide span: raw q, k for the pairwise terms (2^-beta may overflow)
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const float b = beta[rr][dd] + off[dd];
        const float kv = elem32<T>(kw[rr], dd);
        qe[rr] = elem32<T>(qw[rr], dd);
        kp[rr] = kv;
        kh[rr][dd] = kv * exp_2(Bt[dd] - b);
        qer[rr][dd] = qe[rr];
        sBeta[(RPW * w + rr) * Lay::LDB + i] = b;
      }
    }
    store_pack<T, RPW>(sQT + i * Lay::LDT + RPW * w, qe);
    store_pack<T, RPW>(sKT + i * Lay::LDT + RPW * w, kp);
    // the pairwise epilogue's chunk total, or the fast path's 2^r
    if (w == 0) sBx[i] = pairwise ? Bt[dd] : (midref ? exp_2(0.5f * Bt[dd]) : 1.f);
  }
  // Kh rows (Kp rows with the shifted reference; phase C) and Qe rows (phase
  // B), once for all wavefronts
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    T* kr = sKh + (RPW * w + rr) * Lay::LDR + DPL * l;
    T* qr = sQe + (RPW * w + rr) * Lay::LDR + DPL * l;
    if constexpr (DPL == 2 && sizeof(T) == 2) {
      *reinterpret_cast<bf16x2*>(kr) = bf16x2{static_cast<bf16>(kh[rr][0]), static_cast<bf16>(kh[rr][1])};
      *reinterpret_cast<bf16x2*>(qr) = bf16x2{static_cast<bf16>(qer[rr][0]), static_cast<bf16>(qer[rr][1])};
    } else {
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        kr[dd] = from_f32<T>(kh[rr][dd]);
        qr[dd] = from_f32<T>(qer[rr][dd]);
      }
    }
  }
  stage_T_store<T, D, 64, NT>(sOT, Lay::LDT, dyw, 1.0f);
  __syncthreads();

  // phase C's first token tile (the last one: the dlog_g suffix sums run
  // backwards): its rows and, for the epilogue, the anchor parts already in
  // dq, dk, dv and q, k of the lane's 4 dims; issued during phase B
  constexpr int NEP = LOGIT ? 6 : 5;
  uint4 rows[2][2][QV];   // [buffer][dO, v][k-quarter]
  float ep[2][NEP][4];    // [buffer][dq, dk, dv, q, k (, gate logit)][dim]
  auto load_ep = [&](int tt, float (&dst)[NEP][4]) __attribute__((always_inline)) {
    const int trow = t0 + 16 * tt + m;
    const size_t o4 = (size_t)(!RG || trow < L ? trow : 0) * D + ib + 4 * g;
    load_pack<T, 4>(dqo + o4, dst[0]);
    load_pack<T, 4>(dko + o4, dst[1]);
    load_pack<T, 4>(dvo + o4, dst[2]);
    load_pack<T, 4>(qg + o4, dst[3]);
    load_pack<T, 4>(kg + o4, dst[4]);
    if constexpr (LOGIT) load_pack<T, 4>(xg + o4, dst[NEP - 1]);
  };

  // ---- phase B: wavefront w stages the score tiles of token block I
  // against JPW blocks J ----
  {
    // rows of the blocks J (two at a time)
    uint4 rowsJ[2][2][QV];
    auto load_J = [&](int J, uint4 (&dst)[2][QV]) __attribute__((always_inline)) {
      const int rJ = t0 + 16 * J + m;
      load_quarter<T, D, RG>(dst[0], vg, rJ, L, g);
      load_quarter<T, D, RG>(dst[1], dyg, rJ, L, g);
    };
    // the blocks J of this wavefront: all four (four wavefronts), or two
    auto J_of = [&](int jj) __attribute__((always_inline)) -> int {
      if constexpr (NW == 8) {
        const int ja[8] = {0, 2, 0, 2, 1, 0, 1, 0};
        const int jb[8] = {1, 3, 1, 3, 2, 3, 2, 3};
        return jj == 0 ? ja[w] : jb[w];
      } else {
        return jj;
      }
    };
    load_J(J_of(0), rowsJ[0]);
    load_J(J_of(1), rowsJ[1]);
    // phase C's state rows, after phase B's rows (the load counter is waited
    // on in issue order); they arrive while phase B computes
    load_quarter<T, D, false>(Sr, Sg, ib + m, D, g);      // S_c rows i (k = j)
    load_quarter<T, D, false>(Gr, Gg, ib + m, D, g);      // G_{c+1} rows i (k = j)
    load_quarter<T, D, false>(GTr, GTg, ib + m, D, g);    // G_{c+1}^T rows j (k = i)
    // Kp of this lane's key row as fragments: Kh 2^-B, or the stored Kp with the shifted
    // reference (unused on the pairwise path)
    frag kpf[NF];
    if (midref) {
      const T* hp = sKh + (16 * I + m) * Lay::LDR + g * (D / 4);    // Kp rows
#pragma unroll
      for (int e = 0; e < NF; ++e) kpf[e] = M::load(hp + e * M::KPL);
    } else if (!pairwise) {
      const T* hp = sKh + (16 * I + m) * Lay::LDR + g * (D / 4);
      const float* enb = sEB + D + g * (D / 4);
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        float hv[M::KPL], tk[M::KPL];
        if constexpr (sizeof(T) == 2) unpack16<T>(*reinterpret_cast<const uint4*>(hp + e * M::KPL), hv);
        else hv[0] = hp[e];
#pragma unroll
        for (int u = 0; u < M::KPL; ++u) tk[u] = hv[u] * enb[e * M::KPL + u];
        kpf[e] = M::pack(tk);
      }
    } else {
#pragma unroll
      for (int e = 0; e < NF; ++e) kpf[e] = M::zero();
    }
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int J = J_of(jj);
      // (a) dA^T tile: keys s in block J (rows), queries t in block I (cols) -> sDA[t][s]
      // (b) dA tile: queries t in block J (rows), keys s in block I (cols) -> sDAT[s][t]
      // (c) A tile: queries t in block J (rows), keys s in block I (cols) -> sAT[s][t]
      const uint4* vJ = rowsJ[jj & 1][0];
      const uint4* dyJ = rowsJ[jj & 1][1];
      f32x4 ta = zero4(), tb = zero4(), tc = zero4();
      if (J <= I) {
#pragma unroll
        for (int e = 0; e < NF; ++e) ta = M::mma(frag_of<T>(vJ, e), frag_of<T>(dyI, e), ta);
      }
      if (J >= I) {
#pragma unroll
        for (int e = 0; e < NF; ++e) tb = M::mma(frag_of<T>(dyJ, e), frag_of<T>(vI, e), tb);
        if (!pairwise) {
          const T* qp = sQe + (16 * J + m) * Lay::LDR + g * (D / 4);    // Qe rows t (k = i)
#pragma unroll
          for (int e = 0; e < NF; ++e) tc = M::mma(M::load(qp + e * M::KPL), kpf[e], tc);
        } else {
          // A[t][s] = sum_i q_ti k_si 2^{beta_ti - beta_si} pairwise
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tr = 16 * J + 4 * g + r, sr = 16 * I + m;
            float sum = 0.f;
            if (sr <= tr && t0 + tr < L) {
              const float* bt = sBeta + tr * Lay::LDB;
              const float* bs = sBeta + sr * Lay::LDB;
              for (int i = 0; i < D; ++i)
                sum += to_f32(sQT[i * Lay::LDT + tr]) * to_f32(sKT[i * Lay::LDT + sr]) * exp_2(bt[i] - bs[i]);
            }
            tc[r] = sum;
          }
        }
      }
      // masks: s <= t
      float va[4], vb[4], vc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rowk = 16 * J + 4 * g + r, colt = 16 * I + m;   // (a): key row, query col
        va[r] = rowk <= colt ? ta[r] : 0.f;
        const int rowt = 16 * J + 4 * g + r, cols = 16 * I + m;   // (b), (c): query row, key col
        vb[r] = cols <= rowt ? tb[r] : 0.f;
        vc[r] = cols <= rowt ? tc[r] : 0.f;
      }
      store_pack<T, 4>(sDA + (16 * I + m) * Lay::LDT + 16 * J + 4 * g, va);
      store_pack<T, 4>(sDAT + (16 * I + m) * Lay::LDT + 16 * J + 4 * g, vb);
      store_pack<T, 4>(sAT + (16 * I + m) * Lay::LDT + 16 * J + 4 * g, vc);
      if (jj + 2 < JPW) load_J(J_of(jj + 2), rowsJ[jj & 1]);
      if (jj == JPW - 2) {
        // rowsJ[jj & 1] is free from here on
        load_quarter<T, D, RG>(rows[1][0], dyg, t0 + 48 + m, L, g);
        load_quarter<T, D, RG>(rows[1][1], vg, t0 + 48 + m, L, g);
        load_ep(3, ep[1]);
      }
    }
  }
  __syncthreads();

  // ---- phase C: dims / value columns [ib, ib + 16) of every token ----
  // dlog_g of every token of the chunk gets, from all later tokens, the
  // boundary term x_i = sum_j S_{c+1}[i][j] G_{c+1}[i][j]: the terms of
  // q_u.dq_u - k_u.dk_u over u past the chunk cancel in pairs except those
  // of a query after the boundary and a key before it, which sum to this
  // product (zero after the last chunk, where G_{c+1} = 0).  With
  // S_{c+1} = diag(2^B) S_c + sum_s Kh_s v_s^T it is
  //   x_i = 2^{B_i} (S_c G_{c+1}^T)_ii + sum_s k_si (2^{B_i - beta_si} (G_{c+1} v_s)_i),
  // the second factor of the sum being the inter-chunk part of dk_si: the
  // first term from the state rows in registers, the second summed over the
  // tiles below.  xin[r] / xk[r] are the two terms of dim ib + 4g + r (xk
  // per lane, over its tokens), so the dlog_g values wait for the last tile.
  float xin[4], xk[4] = {0.f, 0.f, 0.f, 0.f};
  {
    float x = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) x += elem_of<T>(Sr, kk) * elem_of<T>(Gr, kk);
    x = xgroup_sum(x);
    const int i = ib + m;
    // 2^{B_i}: from the chunk total (pairwise) or from 2^{B-r} and 2^r
    x *= pairwise ? exp_2(sBx[i]) : sEB[i] * (midref ? sBx[i] : 1.f);
#pragma unroll
    for (int r = 0; r < 4; ++r) xin[r] = __shfl(x, 4 * g + r, 64);
  }
  float carry[4] = {0.f, 0.f, 0.f, 0.f};   // sums of q.dq - k.dk over the later tiles
  float dls[4][4];                         // [tile][dim]: dlog_g without the boundary term
  float sgn[LOGIT ? 4 : 1][4];             // [tile][dim]: sigmoid(-x) of the gate logits
#pragma unroll
  for (int tt = 3; tt >= 0; --tt) {
    const int cur = tt & 1;
    const int trow = t0 + 16 * tt + m;        // token of this lane's output column
    const bool live = !RG || trow < L;
    const size_t o4 = (size_t)(live ? trow : 0) * D + ib + 4 * g;
    const float* aq = ep[cur][0];
    const float* ak = ep[cur][1];
    const float* av = ep[cur][2];
    const float* q4 = ep[cur][3];
    const float* k4 = ep[cur][4];
    // the next tile's rows and epilogue inputs
    if (tt > 0) {
      load_quarter<T, D, RG>(rows[cur ^ 1][0], dyg, trow - 16, L, g);
      load_quarter<T, D, RG>(rows[cur ^ 1][1], vg, trow - 16, L, g);
      load_ep(tt - 1, ep[cur ^ 1]);
    }
    const uint4* dyr = rows[cur][0];
    const uint4* vr = rows[cur][1];
    // Kh_s = k_s * 2^{B - beta_s} as fragments (rows s, k = i)
    frag khf[NF];
    {
      const T* kp = sKh + (16 * tt + m) * Lay::LDR + g * (D / 4);
      if (!midref) {
#pragma unroll
        for (int e = 0; e < NF; ++e) khf[e] = M::load(kp + e * M::KPL);
      } else {
        const float* ehb = sEB + g * (D / 4);    // 2^{B-r}
#pragma unroll
        for (int e = 0; e < NF; ++e) {
          float hv[M::KPL], tk[M::KPL];
          if constexpr (sizeof(T) == 2) unpack16<T>(*reinterpret_cast<const uint4*>(kp + e * M::KPL), hv);
          else hv[0] = kp[e];
#pragma unroll
          for (int u = 0; u < M::KPL; ++u) tk[u] = hv[u] * ehb[e * M::KPL + u];
          khf[e] = M::pack(tk);
        }
      }
    }
    // inter-chunk parts
    f32x4 qi = zero4(), ki = zero4(), vi = zero4();
#pragma unroll
    for (int e = 0; e < NF; ++e) {
      qi = M::mma(frag_of<T>(Sr, e), frag_of<T>(dyr, e), qi);     // (S dO_t)_i
      ki = M::mma(frag_of<T>(Gr, e), frag_of<T>(vr, e), ki);      // (G v_s)_i
      vi = M::mma(frag_of<T>(GTr, e), khf[e], vi);                // (G^T Kh_s)_j
    }
    // intra-chunk parts
    f32x4 qa = zero4(), ka = zero4(), va = zero4();
    {
      const T* bO = sOT + (ib + m) * Lay::LDT + g * 16;            // dO^T rows j (k = t)
      const T* bAT = sAT + (16 * tt + m) * Lay::LDT + g * 16;      // A^T rows s (k = t)
#pragma unroll
      for (int e = 0; e < 16 / M::KPL; ++e) va = M::mma(M::load(bO + e * M::KPL), M::load(bAT + e * M::KPL), va);
    }
    if (!pairwise) {
      const T* aK = sKT + (ib + m) * Lay::LDT + g * 16;            // Kp^T rows i (k = s)
      const T* bDA = sDA + (16 * tt + m) * Lay::LDT + g * 16;      // dA rows t (k = s)
      const T* aQ = sQT + (ib + m) * Lay::LDT + g * 16;            // Qe^T rows i (k = t)
      const T* bDAT = sDAT + (16 * tt + m) * Lay::LDT + g * 16;    // dA^T rows s (k = t)
#pragma unroll
      for (int e = 0; e < 16 / M::KPL; ++e) {
        qa = M::mma(M::load(aK + e * M::KPL), M::load(bDA + e * M::KPL), qa);
        ka = M::mma(M::load(aQ + e * M::KPL), M::load(bDAT + e * M::KPL), ka);
      }
    }
    // epilogue for the 4 dims i = ib + 4g + r of token trow
    const int tl = 16 * tt + m;
    const float* bt = sBeta + tl * Lay::LDB + ib + 4 * g;
    float dqv[4], dkv[4], dvv[4], dbv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ib + 4 * g + r;
      const float b = bt[r];
      float qin = qa[r], kin = ka[r];
      float kint;   // the inter-chunk part of dk
      if (pairwise) {
        // dq_ti += sum_s dA_ts k_si 2^{b_ti - b_si};  dk_ti += sum_u dA_ut q_ui 2^{b_ui - b_ti}
        qin = 0.f;
        kin = 0.f;
        for (int s = 0; s <= tl; ++s)
          qin += to_f32(sDA[tl * Lay::LDT + s]) * to_f32(sKT[i * Lay::LDT + s]) * exp_2(b - sBeta[s * Lay::LDB + i]);
        for (int u = tl; u < 64; ++u)
          kin += to_f32(sDAT[tl * Lay::LDT + u]) * to_f32(sQT[i * Lay::LDT + u]) * exp_2(sBeta[u * Lay::LDB + i] - b);
        qin = exp_2(b) * qi[r] + qin;
        kint = exp_2(sBx[i] - b) * ki[r];
        kin = kint + kin;
      } else {
        const float ep = exp_2(b), en = exp_2(-b);
        const float rx = midref ? sBx[i] : 1.f;
        qin = ep * (rx * qi[r] + qin);
        kint = en * (sEB[i] * ki[r]);
        kin = kint + en * kin;
      }
      xk[r] += live ? k4[r] * kint : 0.f;
      const float dqg = qin;
      const float dkg = kin;
      dbv[r] = live ? q4[r] * dqg - k4[r] * dkg : 0.f;
      dqv[r] = dqg + aq[r];
      dkv[r] = dkg + ak[r];
      dvv[r] = vi[r] + va[r] + av[r];
    }
    if (live) {
      store_pack<T, 4>(dqo + o4, dqv);
      store_pack<T, 4>(dko + o4, dkv);
      store_pack<T, 4>(dvo + o4, dvv);
    }
    // dlog_g_t = sum over the tile's tokens u >= t (lanes of this lane
    // group with m' >= m) + the later tiles (+ the boundary term, below)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sfx = dbv[r];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float y = __shfl_down(sfx, o, 16);
        sfx += m + o < 16 ? y : 0.f;
      }
      const float tile = __shfl(sfx, l & 48, 64);   // m = 0: the whole tile
      dls[tt][r] = sfx + carry[r];
      carry[r] += tile;
      // gradient w.r.t. the logits: d log sigmoid(x) / dx = sigmoid(-x)
      if constexpr (LOGIT) sgn[tt][r] = sigmoid_neg(ep[cur][NEP - 1][r]);
    }
  }
  // the boundary term: xk summed over the 16 tokens of each tile (lanes m)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = xk[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
    xin[r] += x;
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int trow = t0 + 16 * tt + m;
    if (RG && trow >= L) continue;
    const size_t o4 = (size_t)trow * D + ib + 4 * g;
    float dl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[r] = dls[tt][r] + xin[r];
    if constexpr (LOGIT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dl[r] *= sgn[tt][r];
      store_pack<T, 4>(dxo + o4, dl);
    } else {
      *reinterpret_cast<f32x4*>(dbo + o4) = f32x4{dl[0], dl[1], dl[2], dl[3]};
    }
  }
}

template <typename T, int D, bool RAGGED, bool LOGIT>
__global__ __launch_bounds__(D / 16 * 64, 1) void bwd_gate_kernel(BwdArgs a, int cb, int ncl) {
  int bh, c;
  if (!chunk_block(a.BH, ncl, bh, c)) return;
  gate_chunk<T, D, RAGGED, LOGIT>(a, bh, c + cb);
}

// The last launch of the two walks, in two roles by block index.
// Blocks [0, nflag): the chunks the reverse walk flagged (decay span beyond
// twice the factorisable limit in some dimension), from G_{c+1} and its
// transpose the walk wrote for them, added to the anchor parts already in
// dq, dk, dv (the walk left zeros there): a persistent grid, each
// workgroup scanning every nflag-th flag (uniform per workgroup),
// range-checked rows.  Blocks nflag + h: the sink-key gradient of head h,
// the anchor walk's B partials of the head summed in batch order (a fixed
// order: deterministic).  One launch instead of two.
template <typename T, int D, bool LOGIT>
__global__ __launch_bounds__(D / 16 * 64, 1) void bwd_tail_kernel(BwdArgs a, int nflag) {
  constexpr int NT = D / 16 * 64;
  if ((int)blockIdx.x >= nflag) {
    const int h = blockIdx.x - nflag;
    const int nmD = a.n_meta * D;
    for (int o = threadIdx.x; o < nmD; o += NT) {
      float sum = 0.f;
      for (int b = 0; b < a.B; ++b) sum += a.ws_dmu[(size_t)(b * a.H + h) * nmD + o];
      a.dmeta[(size_t)h * nmD + o] = sum;
    }
    return;
  }
  const int nc = (a.L + C - 1) / C;
  const long long n = (long long)a.BH * nc;
  // the workgroup's flags idx = base + t nflag, one per thread, read
  // together: the common case (none set) costs one load per thread
  for (long long base = blockIdx.x; base < n; base += (long long)nflag * NT) {
    const long long mine = base + (long long)threadIdx.x * nflag;
    const int f = mine < n ? a.ws_flag[mine] : 0;
    if (!__syncthreads_or(f)) continue;
    for (int t = 0; t < NT; ++t) {
      const long long idx = base + (long long)t * nflag;
      if (idx < n && a.ws_flag[idx]) {
        gate_chunk<T, D, true, LOGIT>(a, (int)(idx / nc), (int)(idx % nc));
        __syncthreads();   // the next chunk's operands overwrite this one's in LDS
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 5 (bf16, d = 128). Reverse walk: the gated branch of every chunk of one
// head, last chunk first, with the state gradient held in MFMA accumulators
// ---------------------------------------------------------------------------
//
// G_c = diag(2^B) G_{c+1} + Qe^T dO is carried from chunk to chunk in
// registers instead of a pass that writes every G_{c+1} (and its transpose)
// to memory for a per-chunk kernel to read back.  One workgroup of 8
// wavefronts per (b, h).  Wavefront w owns the 16-dim group dg = w of the
// key dims / value columns: lane (m, g) holds token 16tt + m and dims
// 16dg + 4g + r (r = 0..3) of every 16-token tile tt of the chunk, for the log-gate prefix
// (a scan over the 16 lanes of a row), the decay factors and the outputs
// alike, so every global load and store of token data is a whole 8- or
// 16-byte piece and no value changes lanes between the prefix and the
// epilogue.  Per group the wavefront also holds two copies of G in fp32
// accumulators: X[it] = G[16it .. +16][16dg .. +16] and
// Y[jt] = G[16dg .. +16][16jt .. +16]^T.
// Rounded to bf16, the registers of X are directly the rows of G^T (for
// dv = G^T Kh, contraction over i) and those of Y the rows of G (for
// dk = G V, contraction over j) in the lane order the accumulators leave
// them: the contraction runs over {32e + 4g + r, 32e + 16 + 4g + r}, and the
// other operand is gathered in that order (two 8-byte LDS reads).
//
// Per chunk, three barriers: (1) prefix, factors, operands into LDS, the
// state rows and the next chunk's rows issued; (2) the causal score tiles
// A = Qe Kp^T and dA = dO V^T; (3) per token tile, last to first: the
// inter-chunk terms (S dO, G V, G^T Kh), the intra-chunk terms (Kp^T dA,
// Qe^T dA^T, dO^T A^T), the outputs (dq, dk, dv: the gated parts, which the
// anchor walk adds to) and dlog_g; then the update of G.
//
// dlog_g of a token t of chunk c is the suffix sum of q.dq - k.dk over the
// chunk's tokens u >= t plus, for everything after the chunk, the boundary
// term rowsum(S_{c+1} * G_{c+1}) (the identity the per-chunk kernel uses),
// formed at the end of the previous step from the state rows this lane
// loaded for S dO, gathered in Y's column order, and from Y.
//
// Chunks whose decay span exceeds twice the factorisable limit in some
// dimension are not computed here: the walk writes G_{c+1} and its transpose
// for them and flags them, and the per-chunk kernel (pairwise fp32 terms)
// completes them afterwards.  Spans between the limit and twice it move
// that dimension's reference point to half its chunk total (per dimension:
// Qe = q 2^{beta - r}, Kp = k 2^{r - beta}, G updated as
// 2^r (2^{B - r} G + Qe^T dO)).
struct WalkLayout {
  static constexpr int D = 128;
  // row-major token tiles [64][LDR]: rows of 264 bytes, whose 8-byte reads
  // (16 rows at a time, two runs 32 bytes apart) spread over the banks
  // (272-byte rows would not); they are then 8-byte aligned only
  static constexpr int LDR = D + 4;
  // transposed tiles [D][64] and score tiles [64][64], fragment-major (fm)
  static constexpr int ROWS = 64 * LDR * 2, TRANS = D * 64 * 2, SCORE = 64 * 64 * 2;
  static constexpr int OFF_QE = 0;                   // Qe[t][i]
  static constexpr int OFF_KP = OFF_QE + ROWS;       // Kp[s][i]
  static constexpr int OFF_O = OFF_KP + ROWS;        // dO[t][j]
  static constexpr int OFF_V = OFF_O + ROWS;         // V[s][j]
  static constexpr int OFF_QET = OFF_V + ROWS;       // Qe^T[i][t]
  static constexpr int OFF_KPT = OFF_QET + TRANS;    // Kp^T[i][s]
  static constexpr int OFF_OT = OFF_KPT + TRANS;     // dO^T[j][t]
  static constexpr int OFF_AT = OFF_OT + TRANS;      // A^T[s][t]
  static constexpr int OFF_DA = OFF_AT + SCORE;      // dA[t][s]
  static constexpr int OFF_DAT = OFF_DA + SCORE;     // dA^T[s][t]
  static constexpr int OFF_EBR = OFF_DAT + SCORE;    // 2^{B_i - r_i}
  static constexpr int OFF_RX = OFF_EBR + D * 4;     // 2^{r_i}
  static constexpr int OFF_FLAG = OFF_RX + D * 4;    // per wavefront: 1 = a dim beyond twice the limit, 2 = a shifted reference
  static constexpr int TOTAL = OFF_FLAG + 64;
};

__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
// An int passed through an empty asm (values derived from it are not hoisted
// out of the loop they are used in).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ __forceinline__ uint2 pack4(const float* v) {
  bf16x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = static_cast<bf16>(v[i]);
  return __builtin_bit_cast(uint2, p);
}
__device__ __forceinline__ uint2 pack4(f32x4 v) {
  const float f[4] = {v[0], v[1], v[2], v[3]};
  return pack4(f);
}
__device__ __forceinline__ void unpack4(uint2 u, float* v) {
  const bf16x4 p = __builtin_bit_cast(bf16x4, u);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = static_cast<float>(p[i]);
}
__device__ __forceinline__ bf16 half_of(uint2 u, int r) {
  const uint32_t w = r < 2 ? u.x : u.y;
  return __builtin_bit_cast(bf16, (unsigned short)((r & 1) ? (w >> 16) : (w & 0xffffu)));
}
// Inclusive prefix (sum over lanes m' <= m) and suffix (m' >= m) scans over
// the 16 lanes of a row, on the VALU: DPP row shifts with zero fill.
template <int N> __device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true));
}
template <int N> __device__ __forceinline__ float row_shl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_prefix(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  return x + row_shr<8>(x);
}
__device__ __forceinline__ float row_suffix(float x) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  return x + row_shl<8>(x);
}

__device__ __forceinline__ bf16x8 frag2(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ bf16x8 frag2(f32x4 a, f32x4 b) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = static_cast<bf16>(a[i]);
    f[4 + i] = static_cast<bf16>(b[i]);
  }
  return f;
}
// Element offset of (row, col) in a fragment-major [rows][64] tile: the run
// of eight values (row, 8c .. 8c + 7) sits at ((row / 16) * 8 + c) * 128 +
// (row % 16) * 8, so the 16 rows of a row tile read their runs of one column
// block from 256 contiguous bytes (no two lanes of a 16-lane group on one
// bank, where a padded row-major tile would put two).
__device__ __forceinline__ int fm(int row, int col) {
  return (((row >> 4) << 3) + (col >> 3)) * 128 + (row & 15) * 8 + (col & 7);
}
// A K = 64 product of row ra of fragment-major tile A and row rb of B (the
// lane's rows): lane group g takes values 16g .. 16g + 15 of both.
__device__ __forceinline__ f32x4 mma_fm(f32x4 c, const bf16* A, int ra, const bf16* B, int rb, int g) {
  typedef Mfma<bf16> M;
#pragma unroll
  for (int e = 0; e < 2; ++e) c = M::mma(M::load(A + fm(ra, 16 * g + 8 * e)), M::load(B + fm(rb, 16 * g + 8 * e)), c);
  return c;
}
// A K = 128 product over two row-major tiles whose rows are 8-byte aligned
// (not 16): each step's eight values of the lane's quarter come as two 8-byte
// reads.
__device__ __forceinline__ f32x4 mma_rows8(f32x4 c, const bf16* a, const bf16* b) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = Mfma<bf16>::mma(frag2(ld8(a + 8 * e), ld8(a + 8 * e + 4)), frag2(ld8(b + 8 * e), ld8(b + 8 * e + 4)), c);
  return c;
}

template <bool LOGIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_walk_kernel(BwdArgs a) {
  typedef WalkLayout Lay;
  typedef bf16 T;
  typedef Mfma<T> M;
  constexpr int D = Lay::D, LDR = Lay::LDR;
  constexpr int NW = 8;       // wavefronts
  constexpr int GPW = 1;      // 16-dim groups per wavefront
  extern __shared__ __align__(16) unsigned char smem[];
  T* sQe = reinterpret_cast<T*>(smem + Lay::OFF_QE);
  T* sKp = reinterpret_cast<T*>(smem + Lay::OFF_KP);
  T* sO = reinterpret_cast<T*>(smem + Lay::OFF_O);
  T* sV = reinterpret_cast<T*>(smem + Lay::OFF_V);
  T* sQeT = reinterpret_cast<T*>(smem + Lay::OFF_QET);
  T* sKpT = reinterpret_cast<T*>(smem + Lay::OFF_KPT);
  T* sOT = reinterpret_cast<T*>(smem + Lay::OFF_OT);
  T* sAT = reinterpret_cast<T*>(smem + Lay::OFF_AT);
  T* sDA = reinterpret_cast<T*>(smem + Lay::OFF_DA);
  T* sDAT = reinterpret_cast<T*>(smem + Lay::OFF_DAT);
  float* sEBr = reinterpret_cast<float*>(smem + Lay::OFF_EBR);
  float* sRx = reinterpret_cast<float*>(smem + Lay::OFF_RX);
  int* sFlag = reinterpret_cast<int*>(smem + Lay::OFF_FLAG);

  const int bh = blockIdx.x;
  if (bh >= a.BH) return;
  const int L = a.L, nc = (L + C - 1) / C;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // lane indices, passed through an empty asm at the top of every chunk so
  // that the many addresses derived from them are formed where they are used
  // instead of being hoisted out of the chunk loop (which would hold them in
  // registers for the whole walk)
  int l = tid & 63, m = l & 15, g = l >> 4;
  // dim group dg = GPW w + h (dims / value columns [16 dg, 16 dg + 16)); this
  // lane's first dim in it is 16 dg + 4g
  auto i0_of = [&](int h) __attribute__((always_inline)) { return 16 * (GPW * w + h) + 4 * g; };
  const size_t hb = (size_t)bh * L * D;
  const T* __restrict__ qg = reinterpret_cast<const T*>(a.q) + hb;
  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + hb;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + hb;
  const T* __restrict__ dyg = reinterpret_cast<const T*>(a.dy) + hb;
  const float* __restrict__ lgg = LOGIT ? nullptr : a.log_g + hb;
  const T* __restrict__ xg = LOGIT ? reinterpret_cast<const T*>(a.gate_logit) + hb : nullptr;
  const T* __restrict__ Sg = reinterpret_cast<const T*>(a.ws_states) + (size_t)bh * nc * D * D;
  T* __restrict__ dqo = reinterpret_cast<T*>(a.dq) + hb;
  T* __restrict__ dko = reinterpret_cast<T*>(a.dk) + hb;
  T* __restrict__ dvo = reinterpret_cast<T*>(a.dv) + hb;
  float* __restrict__ dbo = LOGIT ? nullptr : a.dlog_g + hb;
  T* __restrict__ dxo = LOGIT ? reinterpret_cast<T*>(a.dgate) + hb : nullptr;

  // the score tiles above the diagonal are never written: zero once
  for (int x = tid; x < 3 * Lay::SCORE / 16; x += 64 * NW)
    reinterpret_cast<uint4*>(smem + Lay::OFF_AT)[x] = make_uint4(0u, 0u, 0u, 0u);

  f32x4 X[GPW][8], Y[GPW][8];
#pragma unroll
  for (int h = 0; h < GPW; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      X[h][x] = zero4();
      Y[h][x] = zero4();
    }
  // rowsum(S_{c+1} * G_{c+1}) of dims i0 + r (zero after the last chunk)
  float bnd[GPW][4];
#pragma unroll
  for (int h = 0; h < GPW; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) bnd[h][r] = 0.f;

  // one chunk's rows of this lane: the queries, keys and gates loaded a
  // chunk ahead (at the start of the previous chunk), the values and dO at
  // the end of the previous chunk (they go to LDS last in step 1)
  uint2 pq[GPW][4], pk[GPW][4], pv[GPW][4], po[GPW][4], px[GPW][4];
  float4 plg[GPW][4];
  auto load_qkg = [&](int c, bool full) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < GPW; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = c * C + 16 * tt + m;
        const bool ok = full || t < L;
        const size_t off = (size_t)(ok ? t : 0) * D + i0_of(h);
        const uint2 z = make_uint2(0u, 0u);
        const uint2 q_ = ld8(qg + off), k_ = ld8(kg + off);
        pq[h][tt] = ok ? q_ : z;
        pk[h][tt] = ok ? k_ : z;
        if constexpr (LOGIT) {
          const uint2 x_ = ld8(xg + off);
          px[h][tt] = ok ? x_ : make_uint2(0x7f807f80u, 0x7f807f80u);   // past L: a logit of +inf, a gate of one
        } else {
          const float4 f = *reinterpret_cast<const float4*>(lgg + off);
          plg[h][tt] = ok ? f : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
  };
  auto load_vo = [&](int c, bool full) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < GPW; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = c * C + 16 * tt + m;
        const bool ok = full || t < L;
        const size_t off = (size_t)(ok ? t : 0) * D + i0_of(h);
        const uint2 z = make_uint2(0u, 0u);
        const uint2 v_ = ld8(vg + off), o_ = ld8(dyg + off);
        pv[h][tt] = ok ? v_ : z;
        po[h][tt] = ok ? o_ : z;
      }
  };
  if (nc > 0) {
    if (nc * C <= L) {
      load_qkg(nc - 1, true);
      load_vo(nc - 1, true);
    } else {
      load_qkg(nc - 1, false);
      load_vo(nc - 1, false);
    }
  }

  for (int c = nc - 1; c >= 0; --c) {
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
    const int t0 = c * C;
    const bool full = t0 + C <= L;
    // ================= step 1: prefix, factors, operands ==================
    uint2 cq[GPW][4], ck[GPW][4], cx[GPW][4];
    float lgv[GPW][4][4];
#pragma unroll
    for (int h = 0; h < GPW; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        cq[h][tt] = pq[h][tt];
        ck[h][tt] = pk[h][tt];
        if constexpr (LOGIT) {
          cx[h][tt] = px[h][tt];
#pragma unroll
          for (int r = 0; r < 4; ++r) lgv[h][tt][r] = log_sigmoid(static_cast<float>(half_of(cx[h][tt], r)));
        } else {
          lgv[h][tt][0] = plg[h][tt].x;
          lgv[h][tt][1] = plg[h][tt].y;
          lgv[h][tt][2] = plg[h][tt].z;
          lgv[h][tt][3] = plg[h][tt].w;
        }
      }
    // the state rows for S dO (row 16 dg + m, columns 16x + 4g .. +3), then
    // the next chunk's rows
    uint2 Sr[GPW][8];
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
      const T* sp = Sg + (size_t)c * D * D + (size_t)(16 * (GPW * w + h) + m) * D + 4 * g;
#pragma unroll
      for (int x = 0; x < 8; ++x) Sr[h][x] = ld8(sp + 16 * x);
    }
    // log2-gate prefix: a scan over the 16 lanes of each row (the tile's
    // tokens), then the earlier tiles' totals
    float beta[GPW][4][4], Bt[GPW][4], rr[GPW][4];
    bool wide = false, mid = false;
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
      float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = row_prefix(log2_gate(lgv[h][tt][r]));
          beta[h][tt][r] = x + run[r];
          run[r] += __shfl(x, (l & 48) | 15, 64);
        }
      // reference points: the chunk start, or half the chunk total for spans
      // between the factorisable limit and twice it (beyond that the chunk
      // is left to the per-chunk kernel; its dims keep the chunk start, so
      // that Qe = q 2^beta stays bounded for the update of G)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Bt[h][r] = run[r];
        const float span = -run[r];
        const bool wd = span > 2.f * kMaxSpan;
        const bool md = !wd && span > kMaxSpan;
        wide |= wd;
        mid |= md;
        rr[h][r] = md ? 0.5f * run[r] : 0.f;
      }
      // from here on beta holds b = beta - r
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) beta[h][tt][r] -= rr[h][r];
    }
    // Qe = q 2^{beta - r}, Kp = k 2^{r - beta}: row-major and transposed
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
      const int i0 = i0_of(h);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int row = 16 * tt + m;
        float qf[4], kf[4], qe[4], kp[4];
        unpack4(cq[h][tt], qf);
        unpack4(ck[h][tt], kf);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float b = beta[h][tt][r];
          qe[r] = qf[r] * exp_2(b);
          kp[r] = kf[r] * exp_2(fminf(-b, 126.f));   // (finite where the chunk is left to the per-chunk kernel)
        }
        const uint2 qe4 = pack4(qe), kp4 = pack4(kp);
        st8(sQe + row * LDR + i0, qe4);
        st8(sKp + row * LDR + i0, kp4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sQeT[fm(i0 + r, row)] = half_of(qe4, r);
          sKpT[fm(i0 + r, row)] = half_of(kp4, r);
        }
      }
      if (m == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sEBr[i0 + r] = exp_2(Bt[h][r] - rr[h][r]);
          sRx[i0 + r] = exp_2(rr[h][r]);
        }
      }
      // dO and V rows (loaded at the end of the previous chunk) into LDS:
      // row-major, and dO transposed
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int row = 16 * tt + m;
        st8(sO + row * LDR + i0, po[h][tt]);
        st8(sV + row * LDR + i0, pv[h][tt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sOT[fm(i0 + r, row)] = half_of(po[h][tt], r);
      }
    }
    {
      const bool ww = __any(wide), wm = __any(mid);
      if (l == 0) sFlag[w] = (ww ? 1 : 0) | (wm ? 2 : 0);
    }
    __syncthreads();

    // ================= step 2: score tiles ==================================
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
    int fl = 0;
#pragma unroll
    for (int x = 0; x < NW; ++x) fl |= sFlag[x];
    const bool cwide = (fl & 1) != 0, cmid = (fl & 2) != 0;
    if (!cwide) {
      // 10 causal (I, J <= I) tiles of A and of dA: jobs w, w + NW, ...
#pragma unroll
      for (int jb = 0; jb < (20 + NW - 1) / NW; ++jb) {
        const int j = w + NW * jb;
        if (j >= 20) break;
        const int tl = j % 10;
        const int I = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
        const int J = tl - I * (I + 1) / 2;
        if (j < 10) {
          // A[t][s] = Qe_t . Kp_s: rows t = 16I + 4g + r, column s = 16J + m -> A^T[s][t..t+3]
          const f32x4 v = mma_rows8(zero4(), sQe + (16 * I + m) * LDR + 32 * g, sKp + (16 * J + m) * LDR + 32 * g);
          float a4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) a4[r] = (16 * J + m <= 16 * I + 4 * g + r) ? v[r] : 0.f;
          st8(sAT + fm(16 * J + m, 16 * I + 4 * g), pack4(a4));
        } else {
          // dA[t][s] = dO_t . v_s: rows s = 16J + 4g + r, column t = 16I + m -> dA[t][s..s+3] and dA^T
          const f32x4 v = mma_rows8(zero4(), sV + (16 * J + m) * LDR + 32 * g, sO + (16 * I + m) * LDR + 32 * g);
          float a4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) a4[r] = (16 * J + 4 * g + r <= 16 * I + m) ? v[r] : 0.f;
          const uint2 p4 = pack4(a4);
          st8(sDA + fm(16 * I + m, 16 * J + 4 * g), p4);
#pragma unroll
          for (int r = 0; r < 4; ++r) sDAT[fm(16 * J + 4 * g + r, 16 * I + m)] = half_of(p4, r);
        }
      }
    } else {
      // left to the per-chunk kernel: G_{c+1} (rows of Y) and its transpose
      // (rows of X), in the element type; the chunk's dq, dk, dv rows zero
      // (that kernel adds its gated parts to them, the anchor walk its own)
#pragma unroll
      for (int h = 0; h < GPW; ++h) {
        const size_t ro = ((size_t)bh * nc + c) * D * D + (size_t)(16 * (GPW * w + h) + m) * D + 4 * g;
        T* Gd = reinterpret_cast<T*>(a.ws_dS) + ro;
        T* GTd = reinterpret_cast<T*>(a.ws_dST) + ro;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          st8(GTd + 16 * x, pack4(X[h][x]));
          st8(Gd + 16 * x, pack4(Y[h][x]));
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = t0 + 16 * tt + m;
          if (full || t < L) {
            const size_t off = (size_t)t * D + i0_of(h);
            st8(dqo + off, make_uint2(0u, 0u));
            st8(dko + off, make_uint2(0u, 0u));
            st8(dvo + off, make_uint2(0u, 0u));
          }
        }
      }
    }
    if (tid == 0) a.ws_flag[(size_t)bh * nc + c] = cwide ? 1 : 0;
    __syncthreads();

    // ================= step 3: outputs of the chunk, then G ================
    // G_{c+1} with each row i scaled by 2^{B_i - r_i}: the first half of
    // the update of G, and the factor the inter-chunk terms need
    // (2^{B - beta} G v = 2^{-b} (2^{B - r} G) v; G^T Kh = (2^{B - r} G)^T Kp)
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const float4 f = *reinterpret_cast<const float4*>(sEBr + 16 * it + 4 * g);
        X[h][it][0] *= f.x;
        X[h][it][1] *= f.y;
        X[h][it][2] *= f.z;
        X[h][it][3] *= f.w;
      }
      const float f = sEBr[16 * (GPW * w + h) + m];
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[h][jt][r] *= f;
    }
    if (!cwide) {
#pragma unroll
      for (int h = 0; h < GPW; ++h) {
        const int dg = GPW * w + h;
        float tcarry[4] = {0.f, 0.f, 0.f, 0.f};   // q.dq - k.dk over the chunk's later tiles
#pragma unroll
        for (int tt = 3; tt >= 0; --tt) {
          asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
          const int row = 16 * tt + m;
          const int i0 = i0_of(h);
          const int t = t0 + row;
          const bool live = full || t < L;
          const size_t off = (size_t)(live ? t : 0) * D + i0;

          const T* orow = sO + row * LDR + 4 * g;
          const T* vrow = sV + row * LDR + 4 * g;
          const T* krow = sKp + row * LDR + 4 * g;
          float iq[4], ik[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            iq[r] = exp_2(beta[h][tt][r]);    // 2^{beta - r}
            ik[r] = exp_2(-beta[h][tt][r]);   // 2^{r - beta}
          }
          // (the three outputs one after another: fewer operands and
          // accumulators live at a time)
          // dq = 2^{beta} S dO + 2^{beta - r} Kp^T dA
          float dqg[4];
          {
            f32x4 qi = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e)
              qi = M::mma(frag2(Sr[h][2 * e], Sr[h][2 * e + 1]),
                          frag2(ld8(orow + 32 * e), ld8(orow + 32 * e + 16)), qi);   // (S dO_t)_i
            const f32x4 qa = mma_fm(zero4(), sKpT, 16 * dg + m, sDA, row, g);
            const float4 rx = *reinterpret_cast<const float4*>(sRx + i0);     // 2^r
            const float rxv[4] = {rx.x, rx.y, rx.z, rx.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) dqg[r] = iq[r] * fmaf(rxv[r], qi[r], qa[r]);
            if (live) st8(dqo + off, pack4(dqg));
          }
          __builtin_amdgcn_sched_barrier(0);
          // dk = 2^{B - beta} G v + 2^{r - beta} Qe^T dA^T
          float dkg[4];
          {
            f32x4 ki = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e)
              ki = M::mma(frag2(Y[h][2 * e], Y[h][2 * e + 1]),
                          frag2(ld8(vrow + 32 * e), ld8(vrow + 32 * e + 16)), ki);   // (2^{B - r} G v_s)_i
            const f32x4 ka = mma_fm(zero4(), sQeT, 16 * dg + m, sDAT, row, g);
#pragma unroll
            for (int r = 0; r < 4; ++r) dkg[r] = ik[r] * (ki[r] + ka[r]);
            if (live) st8(dko + off, pack4(dkg));
          }
          __builtin_amdgcn_sched_barrier(0);
          // dv = G^T Kh + A^T dO
          {
            f32x4 vi = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e)
              vi = M::mma(frag2(X[h][2 * e], X[h][2 * e + 1]),
                          frag2(ld8(krow + 32 * e), ld8(krow + 32 * e + 16)), vi);   // ((2^{B - r} G)^T Kp_s)_j
            const f32x4 va = mma_fm(zero4(), sOT, 16 * dg + m, sAT, row, g);
            float dv4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) dv4[r] = vi[r] + va[r];
            if (live) st8(dvo + off, pack4(dv4));
          }
          __builtin_amdgcn_sched_barrier(0);
          // dlog_g: the tile's tokens u >= t (lanes m' >= m of the row), the
          // later tiles, and everything after the chunk
          {
            float qf[4], kf[4], dl[4];
            unpack4(cq[h][tt], qf);
            unpack4(ck[h][tt], kf);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sfx = row_suffix(qf[r] * dqg[r] - kf[r] * dkg[r]);
              dl[r] = sfx + tcarry[r] + bnd[h][r];
              tcarry[r] += __shfl(sfx, l & 48, 64);
              if constexpr (LOGIT) dl[r] *= sigmoid_neg(static_cast<float>(half_of(cx[h][tt], r)));
            }
            if (live) {
              if constexpr (LOGIT) st8(dxo + off, pack4(dl));
              else *reinterpret_cast<float4*>(dbo + off) = make_float4(dl[0], dl[1], dl[2], dl[3]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);   // one tile at a time
        }
      }
    }
    // the next chunk's rows (they fly during the update of G and the next
    // chunk's prefix; issued after every load of this chunk, whose waits
    // would otherwise include them)
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
    if (c > 0) {
      load_qkg(c - 1, true);
      load_vo(c - 1, true);
    }
    // G_c = 2^r (2^{B - r} G_{c+1} + Qe^T dO) (the rows already scaled above):
    // X rows i = 16it + 4g + r, Y columns i = 16 dg + m
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
      const int dg = GPW * w + h;
      // (scheduled two products at a time: their operand reads overlap the
      // previous pair's matrix work without holding more registers)
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        X[h][it] = mma_fm(X[h][it], sQeT, 16 * it + m, sOT, 16 * dg + m, g);
        if (it & 1) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        Y[h][jt] = mma_fm(Y[h][jt], sOT, 16 * jt + m, sQeT, 16 * dg + m, g);
        if (jt & 1) __builtin_amdgcn_sched_barrier(0);
      }
      if (cmid) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const float4 fr = *reinterpret_cast<const float4*>(sRx + 16 * it + 4 * g);
          X[h][it][0] *= fr.x;
          X[h][it][1] *= fr.y;
          X[h][it][2] *= fr.z;
          X[h][it][3] *= fr.w;
        }
        const float fr = sRx[16 * dg + m];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Y[h][jt][r] *= fr;
      }
      // the boundary term of the previous chunk: rowsum(S_c * G_c), row
      // 16 dg + m over this lane's columns (Y's), summed over the row's lanes
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sv[4];
        unpack4(Sr[h][e], sv);
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaf(sv[r], Y[h][e][r], x);
      }
      x = xgroup_sum(x);
#pragma unroll
      for (int r = 0; r < 4; ++r) bnd[h][r] = __shfl(x, 4 * g + r, 64);
    }
    __syncthreads();
  }
}

// 4 x 4 transpose of 4-register blocks over the four 16-lane groups of a
// wavefront: on return, block j of lane group g holds what block g of lane
// group j held.  (gfx950 lane swaps: permlane32 exchanges the upper 32 lanes
// of its first operand with the lower 32 of its second, permlane16 the odd
// 16-lane rows of the first with the even rows of the second.)
__device__ __forceinline__ void xgroup_transpose(f32x4 (&x)[4]) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[b][r]), __float_as_uint(x[b + 2][r]), false, false);
      x[b][r] = __uint_as_float(p[0]);
      x[b + 2][r] = __uint_as_float(p[1]);
    }
#pragma unroll
  for (int b = 0; b < 4; b += 2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[b][r]), __float_as_uint(x[b + 1][r]), false, false);
      x[b][r] = __uint_as_float(p[0]);
      x[b + 1][r] = __uint_as_float(p[1]);
    }
}

// A row's 16 consecutive values 16g .. 16g + 15 of a 64-value half: what
// the transposed output blocks hold (block j, value r: 16g + 4j + r), plus
// the 16 values `in` as bf16, scaled by `sc`, rounded and stored.
__device__ __forceinline__ void add_store16(bf16* dst, const f32x4 (&x)[4], float sc, const uint4 (&in)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float lo[4], hi[4], a4[4], b4[4];
    unpack4(make_uint2(in[h].x, in[h].y), lo);
    unpack4(make_uint2(in[h].z, in[h].w), hi);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a4[r] = fmaf(x[2 * h][r], sc, lo[r]);
      b4[r] = fmaf(x[2 * h + 1][r], sc, hi[r]);
    }
    const uint2 pa = pack4(a4), pb = pack4(b4);
    *reinterpret_cast<uint4*>(dst + 8 * h) = make_uint4(pa.x, pa.y, pb.x, pb.y);
  }
}

// ---------------------------------------------------------------------------
// 5b. anchor branch, both sides in one forward walk over each head's chunks
// (bf16, d = 128)
// ---------------------------------------------------------------------------
// At chunk c the window block row of the chunk's queries (keys of chunks c-1
// and c) gives P, dP, D_t and dS once; from it come dq of chunk c
// (complete), the second and last part of dk, dv of chunk c-1 (the first came
// from its own queries one chunk earlier and waited in registers) and the
// first part of dk, dv of chunk c.  Each chunk's q, k, v, dY are read once
// and each gradient row is read and written once (added to the gated part
// the reverse walk wrote).
//
// Lane orders: the contraction runs over values 8g + 32e .. + 7 of lane group
// g in step e (both operands alike), so that fragment reads of the 288-byte
// token rows take lane groups 16 bytes apart and transposing reads take rows
// 8 apart, both free of LDS bank conflicts at that row stride.
struct AwLayout {
  static constexpr int D = 128;
  static constexpr int LD = D + 16;                   // [64][LD] bf16 token tiles
  static constexpr int LDZ = 16 + 8;                  // sink dZ [64][LDZ] bf16
  static constexpr int TILE = 64 * LD * 2;
  static constexpr int OFF_K = 0;                     // keys, a slot per chunk parity
  static constexpr int OFF_V = OFF_K + 2 * TILE;      // values, likewise
  static constexpr int OFF_Q = OFF_V + 2 * TILE;      // queries of chunk c
  static constexpr int OFF_Y = OFF_Q + TILE;          // dY of chunk c
  static constexpr int OFF_P = OFF_Y + TILE;          // alpha P[t][s]: s = keys of c-1 (0..63), of c (64..127)
  static constexpr int OFF_DS = OFF_P + TILE;         // dS[t][s], the same
  static constexpr int OFF_MU = OFF_DS + TILE;        // sink keys [16][LD]
  static constexpr int OFF_ZS = OFF_MU + 16 * LD * 2; // sink dZ[t][i]
  static constexpr int OFF_DH = OFF_ZS + 64 * LDZ * 2;   // D_t over each half of the keys [2][64] fp32
  static constexpr int OFF_LSE = OFF_DH + 2 * 64 * 4;    // lse (log2 units) of chunk c [64] fp32
  static constexpr int TOTAL = OFF_LSE + 64 * 4;
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_anchor_walk_kernel(BwdArgs a) {
  typedef AwLayout Lay;
  typedef Mfma<bf16> M;
  typedef bf16 T;
  constexpr int D = Lay::D, LD = Lay::LD;
  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + Lay::OFF_K);
  T* sV = reinterpret_cast<T*>(smem + Lay::OFF_V);
  T* sQ = reinterpret_cast<T*>(smem + Lay::OFF_Q);
  T* sY = reinterpret_cast<T*>(smem + Lay::OFF_Y);
  T* sP = reinterpret_cast<T*>(smem + Lay::OFF_P);
  T* sDS = reinterpret_cast<T*>(smem + Lay::OFF_DS);
  T* sMu = reinterpret_cast<T*>(smem + Lay::OFF_MU);
  T* sZs = reinterpret_cast<T*>(smem + Lay::OFF_ZS);
  float* sDh = reinterpret_cast<float*>(smem + Lay::OFF_DH);
  float* sLse = reinterpret_cast<float*>(smem + Lay::OFF_LSE);

  const int bh = blockIdx.x;
  if (bh >= a.BH) return;
  const int h = bh % a.H, L = a.L, nc = (L + C - 1) / C;
  const int tid = threadIdx.x, w = tid >> 6;
  int l = tid & 63, m = l & 15, g = l >> 4;
  const int qt = w & 3;   // query tile of the scores and of dq; key tile of dk, dv
  const int hf = w >> 2;  // half: keys of chunk c-1 / c in the scores; dims 0..63 / 64..127 in the outputs
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  const T* yg = reinterpret_cast<const T*>(a.dy) + (size_t)bh * L * D;
  T* dqg = reinterpret_cast<T*>(a.dq) + (size_t)bh * L * D;
  T* dkg = reinterpret_cast<T*>(a.dk) + (size_t)bh * L * D;
  T* dvg = reinterpret_cast<T*>(a.dv) + (size_t)bh * L * D;
  const float* lseg = a.lse + (size_t)bh * L;
  const float sl2 = a.scale * kLog2e;

  // rows of chunk c of a [L, D] tensor: thread -> 16-byte runs of rows
  // tid / 16 and tid / 16 + 32 (zeros outside [0, L))
  auto load_rows = [&](uint4* buf, const T* base, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int t = c * C + 32 * p + (tid >> 4);
      const bool ok = c >= 0 && t < L;
      const uint4 u = ld16(base + (size_t)(ok ? t : 0) * D + 8 * (tid & 15));
      buf[p] = ok ? u : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_rows = [&](T* tile, const uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<uint4*>(tile + (32 * p + (tid >> 4)) * LD + 8 * (tid & 15)) = buf[p];
  };
  auto load_lse = [&](int c) __attribute__((always_inline)) -> float {
    const int t = c * C + (tid & 63);
    return t < L ? lseg[t] * kLog2e : 0.f;
  };

  // chunk 0 (and an empty chunk -1), the sink keys
  {
    uint4 bq[2], bk[2], bv[2], by[2], bz[2];
    load_rows(bq, qg, 0);
    load_rows(bk, kg, 0);
    load_rows(bv, vg, 0);
    load_rows(by, yg, 0);
    load_rows(bz, kg, -1);   // zeros
    const float ls = load_lse(0);
    uint4 mu = make_uint4(0u, 0u, 0u, 0u);
    const int mrow = tid >> 4;   // threads 0..255: sink rows 0..15
    if (tid < 256 && mrow < a.n_meta)
      mu = ld16(reinterpret_cast<const T*>(a.meta) + ((size_t)h * a.n_meta + mrow) * D + 8 * (tid & 15));
    store_rows(sQ, bq);
    store_rows(sK, bk);
    store_rows(sV, bv);
    store_rows(sY, by);
    store_rows(sK + 64 * LD, bz);
    store_rows(sV + 64 * LD, bz);
    if (tid < 64) sLse[tid] = ls;
    if (tid < 256) *reinterpret_cast<uint4*>(sMu + mrow * LD + 8 * (tid & 15)) = mu;
  }
  __syncthreads();

  // this wavefront's part of dk, dv of the current chunk from its own
  // queries (key tile qt, dims 64 hf + 16 dt + 4 g + r), unscaled
  f32x4 ck[4], cv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ck[dt] = cv[dt] = zero4();
  // the head's sink-key gradient over all its chunks (sink m, dims 16 w + 4 g + r)
  f32x4 dmu = zero4();

  for (int c = 0; c < nc; ++c) {
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
    const int t0 = c * C;
    const int cs = c & 1, ps = cs ^ 1;
    T* sKc = sK + cs * 64 * LD;
    T* sKp = sK + ps * 64 * LD;
    T* sVc = sV + cs * 64 * LD;
    T* sVp = sV + ps * 64 * LD;
    // the next chunk's rows (written after this chunk's last reads) and the
    // rows of dq (chunk c) and dk, dv (chunk c - 1) this wavefront adds to
    uint4 nq[2], nk[2], nv[2], ny[2];
    const bool more = c + 1 < nc;
    if (more) {
      load_rows(nq, qg, c + 1);
      load_rows(nk, kg, c + 1);
      load_rows(nv, vg, c + 1);
      load_rows(ny, yg, c + 1);
    }
    const float nls = more ? load_lse(c + 1) : 0.f;
    const int tq = t0 + 16 * qt + m;               // dq row of this lane
    const int sk = t0 - C + 16 * qt + m;           // dk, dv row (chunk c - 1) of this lane
    // (the lane's row, values 64 hf + 16 g .. + 15: the gradient blocks
    // are transposed over the lane groups before they are added and stored)
    const int gcol = 64 * hf + 16 * g;
    uint4 pq[2], pk[2], pv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pq[h] = tq < L ? ld16(dqg + (size_t)tq * D + gcol + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
      pk[h] = c > 0 ? ld16(dkg + (size_t)(c > 0 ? sk : 0) * D + gcol + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
      pv[h] = c > 0 ? ld16(dvg + (size_t)(c > 0 ? sk : 0) * D + gcol + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- scores: keys of chunk c - 1 (hf = 0) or c (hf = 1) against the
    // queries of tile qt: Z^T[s][t], dP^T[s][t] (key s = 16 kt + 4g + r of
    // the half, query t = 16 qt + m) ----
    const T* sKh = hf ? sKc : sKp;
    const T* sVh = hf ? sVc : sVp;
    f32x4 z[4], dp[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 zc = zero4(), pc = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 8 * g + 32 * e;
        zc = M::mma(M::load(sKh + (16 * kt + m) * LD + col), M::load(sQ + (16 * qt + m) * LD + col), zc);
        pc = M::mma(M::load(sVh + (16 * kt + m) * LD + col), M::load(sY + (16 * qt + m) * LD + col), pc);
      }
      z[kt] = zc;
      dp[kt] = pc;
    }
    const float lse2 = sLse[16 * qt + m];
    float dsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sgl = t0 - C + 64 * hf + 16 * kt + 4 * g + r;   // key position
        const bool ok = tq < L && sgl >= 0 && sgl <= tq && sgl > tq - a.window;
        const float p = ok ? exp_2(z[kt][r] * sl2 - lse2) : 0.f;
        z[kt][r] = p;
        dp[kt][r] *= a.alpha;
        dsum += p * dp[kt][r];
      }
    dsum = xgroup_sum(dsum);
    if (g == 0) sDh[hf * 64 + 16 * qt + m] = dsum;
    f32x4 zs = zero4();
    if (hf == 0 && a.n_meta > 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 8 * g + 32 * e;
        zs = M::mma(M::load(sMu + m * LD + col), M::load(sQ + (16 * qt + m) * LD + col), zs);
      }
    }
    __syncthreads();

    // ---- dS = P (alpha dP - D), alpha P, sink dZ = -P D into LDS ----
    {
      const float Dt = sDh[16 * qt + m] + sDh[64 + 16 * qt + m];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float ds4[4], pa4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ds4[r] = z[kt][r] * (dp[kt][r] - Dt);
          pa4[r] = z[kt][r] * a.alpha;
        }
        const int off = (16 * qt + m) * LD + 64 * hf + 16 * kt + 4 * g;
        st8(sDS + off, pack4(ds4));
        st8(sP + off, pack4(pa4));
      }
      if (hf == 0) {
        float zv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          zv[r] = (4 * g + r < a.n_meta && tq < L) ? -exp_2(zs[r] * sl2 - lse2) * Dt : 0.f;
        st8(sZs + (16 * qt + m) * Lay::LDZ + 4 * g, pack4(zv));
      }
    }
    __syncthreads();

    // ---- dq of chunk c: dq^T[d][t] = scale (K^T dS^T + mu^T dZs^T), the
    // wavefront's query tile qt and dims 64 hf .. + 63 ----
    {
      f32x4 o[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const M::frag b = M::load(sDS + (16 * qt + m) * LD + 8 * g + 32 * e);   // dS[t][s], s = 8g + 32e ..
        const T* kb = e < 2 ? sKp : sKc;                                        // keys c - 1, then c
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = M::mma(frag_tr(kb + 64 * hf + 16 * dt, LD, 8 * g + 32 * (e & 1), m), b, o[dt]);
      }
      if (a.n_meta > 0) {
        // sinks 8g .. 8g + 7 for g < 2; the other lane groups add zeros
        M::frag b = M::load(sZs + (16 * qt + m) * Lay::LDZ + 8 * (g & 1));
        if (g >= 2) b = M::zero();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = M::mma(frag_tr(sMu + 64 * hf + 16 * dt, LD, 8 * (g & 1), m), b, o[dt]);
      }
      xgroup_transpose(o);
      if (tq < L) add_store16(dqg + (size_t)tq * D + gcol, o, a.scale, pq);
    }

    // ---- dk, dv: keys of chunk c - 1 (second part, then complete) and of
    // chunk c (first part): dk^T[d][s] = Q^T dS, dv^T[d][s] = dY^T (alpha P),
    // over the chunk's queries (key tile qt, dims 64 hf .. + 63) ----
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 ok4[4], ov4[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ok4[dt] = ov4[dt] = zero4();
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k0 = 8 * g + 32 * e;   // queries
        const M::frag bs = frag_tr(sDS + 64 * half + 16 * qt, LD, k0, m);
        const M::frag bp = frag_tr(sP + 64 * half + 16 * qt, LD, k0, m);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          ok4[dt] = M::mma(frag_tr(sQ + 64 * hf + 16 * dt, LD, k0, m), bs, ok4[dt]);
          ov4[dt] = M::mma(frag_tr(sY + 64 * hf + 16 * dt, LD, k0, m), bp, ov4[dt]);
        }
      }
      if (half == 0) {
        // chunk c - 1 complete: its first part (ck, cv) plus this one
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ok4[dt][r] += ck[dt][r];
            ov4[dt][r] += cv[dt][r];
          }
        xgroup_transpose(ok4);
        xgroup_transpose(ov4);
        if (c > 0 && sk < L) {
          add_store16(dkg + (size_t)sk * D + gcol, ok4, a.scale, pk);
          add_store16(dvg + (size_t)sk * D + gcol, ov4, 1.f, pv);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          ck[dt] = ok4[dt];
          cv[dt] = ov4[dt];
        }
      }
    }

    // ---- sink keys: dmu^T[d][i] += Q^T dZs over the chunk, dims 16 w .. + 15 ----
    if (a.n_meta > 0) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k0 = 8 * g + 32 * e;
        dmu = M::mma(frag_tr(sQ + 16 * w, LD, k0, m), frag_tr(sZs, Lay::LDZ, k0, m), dmu);
      }
    }
    __syncthreads();

    // ---- the next chunk's rows into the freed tiles ----
    if (more) {
      store_rows(sQ, nq);
      store_rows(sY, ny);
      store_rows(sKp, nk);
      store_rows(sVp, nv);
      if (tid < 64) sLse[tid] = nls;
    }
    __syncthreads();
  }
  // the head's sink-key partial (one per head: the reduction over the batch
  // takes one chunk per head)
  if (a.n_meta > 0 && m < a.n_meta) {
    float* part = a.ws_dmu + (size_t)bh * a.n_meta * D;
    *reinterpret_cast<float4*>(part + (size_t)m * D + 16 * w + 4 * g) =
        make_float4(dmu[0] * a.scale, dmu[1] * a.scale, dmu[2] * a.scale, dmu[3] * a.scale);
  }
  // the last chunk's dk, dv: its own queries' part is all there is
  {
    asm volatile("" : "+v"(l), "+v"(m), "+v"(g));
    const int sk = (nc - 1) * C + 16 * qt + m;
    const size_t off = (size_t)(sk < L ? sk : 0) * D + 64 * hf + 16 * g;
    xgroup_transpose(ck);
    xgroup_transpose(cv);
    if (sk < L) {
      const uint4 pk[2] = {ld16(dkg + off), ld16(dkg + off + 8)};
      const uint4 pv[2] = {ld16(dvg + off), ld16(dvg + off + 8)};
      add_store16(dkg + off, ck, a.scale, pk);
      add_store16(dvg + off, cv, 1.f, pv);
    }
  }
}

// ---------------------------------------------------------------------------
// 6. dmeta[h][i][d] = sum over batch rows and chunks of the partials (fixed order)
// ---------------------------------------------------------------------------
// Block (x, h) sums outputs o = 64x .. 64x + 63: thread (o, part) adds the
// terms k = part, part + 4, ... of the B*nc partials (k = b*nc + c) in order,
// then the 4 part sums are added in order.
__global__ __launch_bounds__(256) void bwd_dmeta_reduce_kernel(const float* part, float* out, int B, int H, int nc,
                                                               int nmD) {
  __shared__ float sPart[4][64];
  const int h = blockIdx.y;
  const int ol = threadIdx.x & 63, pi = threadIdx.x >> 6;
  const int o = blockIdx.x * 64 + ol;
  const bool live = o < nmD;
  const int nk = B * nc;
  float s = 0.f;
  if (live) {
    int k = pi;
    for (; k + 28 < nk; k += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = k + 4 * u, b = kk / nc, c = kk % nc;
        v[u] = part[((size_t)(b * H + h) * nc + c) * nmD + o];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < nk; k += 4) {
      const int b = k / nc, c = k % nc;
      s += part[((size_t)(b * H + h) * nc + c) * nmD + o];
    }
  }
  sPart[pi][ol] = s;
  __syncthreads();
  if (pi == 0 && live) out[(size_t)h * nmD + o] = ((sPart[0][ol] + sPart[1][ol]) + sPart[2][ol]) + sPart[3][ol];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct WsPlan {
  size_t states, dS, dST, Dt, dmu, flag, total;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

WsPlan plan_ws(int elem, int BH, int L, int D, int n_meta) {
  const size_t nc = (size_t)(L + C - 1) / C;
  const size_t st = al256((size_t)BH * nc * D * D * elem);
  WsPlan p;
  p.states = 0;
  p.dS = p.states + st;
  p.dST = p.dS + st;
  p.Dt = p.dST + st;
  p.dmu = p.Dt + al256((size_t)BH * L * 4);
  p.flag = p.dmu + al256((size_t)BH * nc * n_meta * D * 4);
  p.total = p.flag + al256((size_t)BH * nc);
  return p;
}

template <typename K>
hipError_t set_lds(K kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// the gate kernel over the full chunks, then over the last chunk if it ends past L
template <typename T, int D, bool LOGIT>
hipError_t launch_gate(const BwdArgs& a, int nfull, int nc, int groups, hipStream_t st) {
  typedef GateLayout<T, D> GL;
  static_assert(GL::TOTAL <= 160 * 1024, "LDS");
  hipError_t e;
  if (nfull > 0) {
    if ((e = set_lds(&bwd_gate_kernel<T, D, false, LOGIT>, GL::TOTAL)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gate_kernel<T, D, false, LOGIT>), dim3(8 * groups * nfull), dim3(GL::NW * 64), GL::TOTAL,
                       st, a, 0, nfull);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (nfull < nc) {
    if ((e = set_lds(&bwd_gate_kernel<T, D, true, LOGIT>, GL::TOTAL)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gate_kernel<T, D, true, LOGIT>), dim3(8 * groups), dim3(GL::NW * 64), GL::TOTAL, st, a,
                       nfull, 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D, int DV>
hipError_t launch_bwd_t(BwdArgs a, hipStream_t st) {
  // bf16 at d = 128: two walks over each head's chunks
  constexpr bool WALK = sizeof(T) == 2 && D == 128;
  const int L = a.L, nc = (L + C - 1) / C;
  const int groups = (a.BH + 7) / 8;
  hipError_t e;
  if (a.BH > 0 && L > 0) {
    if (a.saved_states) {
      // 1. the chunk-start states the forward pass kept (read only)
      a.ws_states = const_cast<void*>(a.saved_states);
    } else {
      // 1. chunk-start states (forward kernel, states only)
      FwdArgs f{};
      f.q = a.q;
      f.k = a.k;
      f.v = a.v;
      f.log_g = a.log_g;
      f.gate_logit = a.gate_logit;
      f.meta = a.meta;
      f.y = nullptr;
      f.lse = nullptr;
      f.y_anchor = nullptr;
      f.state_out = nullptr;
      f.states = a.ws_states;
      f.BH = a.BH;
      f.H = a.H;
      f.L = L;
      f.n_meta = a.n_meta;
      f.window = a.window;
      f.nsplit = D / fwd_value_slice(sizeof(T) == 2, D);
      f.alpha = a.alpha;
      f.scale_log2 = a.scale * kLog2e;
      e = launch_fwd(f, sizeof(T) == 2, D, st);
      if (e != hipSuccess) return e;
    }
    // the reverse walk carries the state gradients itself (bf16, d = 128)
    if constexpr (!WALK) {
      // 2. state gradients
      if (a.gate_logit)
        hipLaunchKernelGGL((bwd_dstate_kernel<T, D, DV, true>), dim3(8 * groups * (D / DV)), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((bwd_dstate_kernel<T, D, DV, false>), dim3(8 * groups * (D / DV)), dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int nfull = L / C;
    if constexpr (WALK) {
      // 3. the reverse walk (gated parts of dq, dk, dv; dlog_g; zeros in
      // dq, dk, dv for the chunks it leaves to the last launch)
      const bool logit = a.gate_logit != nullptr;
      static_assert(WalkLayout::TOTAL <= 160 * 1024, "LDS");
      const void* wk = logit ? reinterpret_cast<const void*>(&bwd_walk_kernel<true>)
                             : reinterpret_cast<const void*>(&bwd_walk_kernel<false>);
      if ((e = hipFuncSetAttribute(wk, hipFuncAttributeMaxDynamicSharedMemorySize, WalkLayout::TOTAL)) != hipSuccess)
        return e;
      if (logit)
        hipLaunchKernelGGL((bwd_walk_kernel<true>), dim3(a.BH), dim3(512), WalkLayout::TOTAL, st, a);
      else
        hipLaunchKernelGGL((bwd_walk_kernel<false>), dim3(a.BH), dim3(512), WalkLayout::TOTAL, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (WALK) {
      // 4. the anchor branch, a forward walk per head (added to the gated parts)
      static_assert(AwLayout::TOTAL <= 160 * 1024, "LDS");
      if ((e = set_lds(&bwd_anchor_walk_kernel, AwLayout::TOTAL)) != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_anchor_walk_kernel, dim3(a.BH), dim3(512), AwLayout::TOTAL, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      // 5. the chunks the reverse walk flagged (none for ordinary gates) and
      // the sink-key gradient, in one launch: one flag per thread, enough
      // workgroups to read every flag at once (the common case, no chunk
      // flagged, then ends after one load), and one workgroup per head
      typedef GateLayout<T, D> GL;
      const long long n = (long long)a.BH * nc;
      const long long need = (n + GL::NW * 64 - 1) / (GL::NW * 64);
      const int nflag = (int)(need < 256 ? need : 256);
      const int grid = nflag + (a.n_meta > 0 ? a.H : 0);
      if (a.gate_logit) {
        if ((e = set_lds(&bwd_tail_kernel<T, D, true>, GL::TOTAL)) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_tail_kernel<T, D, true>), dim3(grid), dim3(GL::NW * 64), GL::TOTAL, st, a, nflag);
      } else {
        if ((e = set_lds(&bwd_tail_kernel<T, D, false>, GL::TOTAL)) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_tail_kernel<T, D, false>), dim3(grid), dim3(GL::NW * 64), GL::TOTAL, st, a, nflag);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      // 3, 4. anchor, query and key side: the full chunks in one launch each,
      // a ragged last chunk range-checked in its own (written alone, the gate
      // kernel adds its own)
      typedef AqLayout<T, D> AQ;
      static_assert(AQ::TOTAL <= 80 * 1024, "LDS: two workgroups per CU");
      typedef AkLayout<T, D> AK;
      static_assert(AK::TOTAL <= 80 * 1024, "LDS: two workgroups per CU");
      if ((e = set_lds(&bwd_anchor_q_kernel<T, D, true>, AQ::TOTAL)) != hipSuccess) return e;
      if ((e = set_lds(&bwd_anchor_q_kernel<T, D, false>, AQ::TOTAL)) != hipSuccess) return e;
      if ((e = set_lds(&bwd_anchor_k_kernel<T, D, true>, AK::TOTAL)) != hipSuccess) return e;
      if ((e = set_lds(&bwd_anchor_k_kernel<T, D, false>, AK::TOTAL)) != hipSuccess) return e;
      if (nfull > 0)
        hipLaunchKernelGGL((bwd_anchor_q_kernel<T, D, false>), dim3(8 * groups * nfull), dim3(256), AQ::TOTAL, st, a,
                           0, nfull);
      if (nfull < nc)
        hipLaunchKernelGGL((bwd_anchor_q_kernel<T, D, true>), dim3(8 * groups), dim3(256), AQ::TOTAL, st, a, nfull, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (nfull > 0)
        hipLaunchKernelGGL((bwd_anchor_k_kernel<T, D, false>), dim3(8 * groups * nfull), dim3(256), AK::TOTAL, st, a,
                           0, nfull);
      if (nfull < nc)
        hipLaunchKernelGGL((bwd_anchor_k_kernel<T, D, true>), dim3(8 * groups), dim3(256), AK::TOTAL, st, a, nfull, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 5. gated branch and outputs (the per-chunk kernel)
    if constexpr (!WALK) {
      if (a.gate_logit) {
        if ((e = launch_gate<T, D, true>(a, nfull, nc, groups, st)) != hipSuccess) return e;
      } else {
        if ((e = launch_gate<T, D, false>(a, nfull, nc, groups, st)) != hipSuccess) return e;
      }
    }
  }
  // 6. sink keys (written even when B*L == 0: then zero)
  if (a.n_meta > 0 && a.H > 0) {
    const int nmD = a.n_meta * D;
    if (a.BH > 0 && L > 0) {
      // (bf16 at d = 128: the last launch of the walks has summed them)
      if constexpr (!WALK)
        hipLaunchKernelGGL(bwd_dmeta_reduce_kernel, dim3((nmD + 63) / 64, a.H), dim3(256), 0, st, a.ws_dmu, a.dmeta,
                           a.B, a.H, nc, nmD);
    } else {
      hipLaunchKernelGGL(bwd_dmeta_reduce_kernel, dim3((nmD + 63) / 64, a.H), dim3(256), 0, st, a.ws_dmu, a.dmeta,
                         0, a.H, 0, nmD);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(int dtype_bf16, int BH, int L, int D, int n_meta) {
  if (BH == 0 || L == 0) return 0;
  return plan_ws(dtype_bf16 ? 2 : 4, BH, L, D, n_meta).total;
}

hipError_t launch_bwd(const BwdArgs& in, int dtype_bf16, int D, hipStream_t st) {
  BwdArgs a = in;
  if (a.BH > 0 && a.L > 0) {
    const WsPlan p = plan_ws(dtype_bf16 ? 2 : 4, a.BH, a.L, D, a.n_meta);
    char* base = static_cast<char*>(a.workspace);
    a.ws_states = base + p.states;
    a.ws_dS = base + p.dS;
    a.ws_dST = base + p.dST;
    a.ws_D = reinterpret_cast<float*>(base + p.Dt);
    a.ws_dmu = reinterpret_cast<float*>(base + p.dmu);
    a.ws_flag = reinterpret_cast<unsigned char*>(base + p.flag);
  }
  if (dtype_bf16 && D == 128) return launch_bwd_t<bf16, 128, 64>(a, st);
  if (dtype_bf16 && D == 64) return launch_bwd_t<bf16, 64, 64>(a, st);
  if (!dtype_bf16 && D == 64) return launch_bwd_t<float, 64, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lizard
