// Chunked forward pass of the Lizard hybrid attention layer on gfx950.
//
// What it computes ("Lizard" explainer, gist.science (de), section 2
// "Methodik", "Kernkomponenten" items 1-3): Y = Y_gate + alpha * Y_anchor,
// with the gated branch S_t = diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t,
// and the anchor branch a softmax over the keys [t-w+1, t] plus m
// meta-memory sink keys whose values are zero.
//
// How (section 2 "Hardware-bewusster Algorithmus" on the same page: the
// cumulative gate products are moved into log space and folded into the
// query and key operands so the chunk work is plain matrix products on the
// matrix cores).  The sequence is cut into chunks of 64 tokens.  Inside a
// chunk, with beta_t the inclusive log2-gate prefix from the chunk start and
// B the chunk total (all <= 0):
//
//   Qe_t = q_t * 2^{beta_t}            (<= |q|)      readout and intra queries
//   Kp_s = k_s * 2^{-beta_s}                          intra keys
//   Kh_s = k_s * 2^{B - beta_s}        (<= |k|)      state-carry keys
//   o_t  = Qe_t^T S_c + sum_{s<=t} (Qe_t . Kp_s) v_s
//   S_{c+1} = diag(2^B) S_c + Kh^T V
//
// Kp grows like 2^{-beta}; a chunk is taken this way only while its decay
// span max_i(-B_i) stays within 2^{92} (far inside the float/bfloat16 range,
// and every product Qe_t . Kp_s with s <= t is a gate product <= 1).  Chunks
// with a larger span (gates near zero) compute the intra scores pairwise in
// fp32 from 2^{beta_t - beta_s}.  Nothing ever divides by a gate product.
//
// Work decomposition: one workgroup of 8 wavefronts (2 per SIMD) per
// (batch, head, slice of DV value columns).  The workgroup walks the chunks
// in order and keeps its slice of the float32 state in MFMA accumulators,
// 16 state rows per wavefront.  Query block I (16 rows) of a chunk belongs
// to the wavefront pair (I, I+4): each computes half of the 96 window-key
// logits (and the intra scores among them), the pair exchanges softmax
// maxima and sums through LDS, then each produces half of the value
// columns.  Keys and values of the previous chunk stay in an LDS ring for
// the window.  All products are computed transposed (keys or value columns
// on the MFMA rows, the block's 16 queries on its columns), so each lane
// ends with 4 consecutive keys / columns of one query: packed LDS and global
// writes, and softmax reductions across 4 lane groups only.
#include <type_traits>

#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

template <typename T, int D, int DV>
struct FwdLayout {
  static constexpr int C = 64;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDK = D + PAD;       // sK ring [128][LDK], sKp [64][LDK]
  static constexpr int LDVT = 128 + PAD;    // sVt ring [DV][LDVT]
  static constexpr int LDKH = 64 + PAD;     // sKhT [D][LDKH]
  static constexpr int LDST = D + PAD;      // sSt [DV][LDST]
  static constexpr int LDE = D + 4;         // pairwise path: beta [64][LDE] float in the sQ/sQe region
  static constexpr int LDSTG = 96 + PAD;    // staging per query block [16][LDSTG]
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_K = 0;
  static constexpr int OFF_VT = OFF_K + a16(128 * LDK * (int)sizeof(T));
  static constexpr int OFF_KP = OFF_VT + a16(DV * LDVT * (int)sizeof(T));
  static constexpr int OFF_KHT = OFF_KP + a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_ST = OFF_KHT + a16(D * LDKH * (int)sizeof(T));
  static constexpr int OFF_Q = OFF_ST + a16(DV * LDST * (int)sizeof(T));      // raw q [64][LDK]
  static constexpr int OFF_QE = OFF_Q + a16(64 * LDK * (int)sizeof(T));       // q * 2^beta [64][LDK]
  static constexpr int QQ_END = OFF_QE + a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_TOT = (QQ_END > OFF_Q + a16(64 * LDE * 4) ? QQ_END : OFF_Q + a16(64 * LDE * 4));
  static constexpr int OFF_BEXP = OFF_TOT + a16(8 * D * 4);
  static constexpr int OFF_STAT = OFF_BEXP + a16(D * 4);
  static constexpr int OFF_STG = OFF_STAT + a16(8 * 16 * 2 * 4);
  static constexpr int TOTAL = OFF_STG + a16(4 * 16 * LDSTG * (int)sizeof(T));
};

// Raw 16-byte vectors -> MFMA fragment e of a lane's contiguous k-quarter.
template <typename T> __device__ __forceinline__ typename Mfma<T>::frag frag_at(const uint4* raw, int e);
template <> __device__ __forceinline__ bf16x8 frag_at<bf16>(const uint4* raw, int e) {
  return __builtin_bit_cast(bf16x8, raw[e]);
}
template <> __device__ __forceinline__ float frag_at<float>(const uint4* raw, int e) {
  const uint4 r = raw[e >> 2];
  const uint32_t u = (e & 3) == 0 ? r.x : (e & 3) == 1 ? r.y : (e & 3) == 2 ? r.z : r.w;
  return __builtin_bit_cast(float, u);
}
// Element i of a run of raw vectors, as float.
template <typename T> __device__ __forceinline__ float elem_f32(const uint4* raw, int i);
template <> __device__ __forceinline__ float elem_f32<bf16>(const uint4* raw, int i) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, raw[i >> 3]);
  return static_cast<float>(v[i & 7]);
}
template <> __device__ __forceinline__ float elem_f32<float>(const uint4* raw, int i) {
  return frag_at<float>(raw, i);
}

// Largest chunk decay span (log2 units) taken by the factorised path: 2^92
// leaves a factor 2^36 of headroom below the float / bfloat16 maximum.
constexpr float kMaxSpanLog2 = 92.0f;

template <typename T, int D, int DV, bool STATES>
__global__ __launch_bounds__(512, 1) void lizard_fwd_kernel(FwdArgs a) {
  typedef FwdLayout<T, D, DV> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int C = 64;
  constexpr int DPL = D / 64;                 // phase-A dims per lane
  constexpr int EPV = 16 / sizeof(T);         // elements per 16-byte vector
  constexpr int QV = D / 4 / EPV;             // 16-byte vectors in a lane's k-quarter of a row
  constexpr int NF = D / 4 / M::KPL;          // MFMA steps over a D contraction
  constexpr int NCT = DV / 16;                // value column tiles
  constexpr int NCH = NCT / 2;                // value column tiles per wavefront of a pair
  constexpr int VC = 4 / sizeof(T);           // value columns per thread in the value load
  constexpr int VRW = DV / VC;                // threads across a value row
  constexpr int VR = 64 * VRW / 512;          // value rows per thread
  static_assert(VR == 4 && NCH >= 1, "shape");

  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + Lay::OFF_K);
  T* sVt = reinterpret_cast<T*>(smem + Lay::OFF_VT);
  T* sKp = reinterpret_cast<T*>(smem + Lay::OFF_KP);
  T* sKhT = reinterpret_cast<T*>(smem + Lay::OFF_KHT);
  T* sSt = reinterpret_cast<T*>(smem + Lay::OFF_ST);
  T* sQ = reinterpret_cast<T*>(smem + Lay::OFF_Q);
  T* sQe = reinterpret_cast<T*>(smem + Lay::OFF_QE);
  float* sBeta = reinterpret_cast<float*>(smem + Lay::OFF_Q);   // pairwise path only (aliases sQ, sQe)
  float* sTot = reinterpret_cast<float*>(smem + Lay::OFF_TOT);
  float* sBexp = reinterpret_cast<float*>(smem + Lay::OFF_BEXP);
  float* sStat = reinterpret_cast<float*>(smem + Lay::OFF_STAT);
  T* sStgAll = reinterpret_cast<T*>(smem + Lay::OFF_STG);

  // ---- block -> (b*h, value slice); siblings of one head share an XCD ----
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int idx = x >> 3;
  const int split = idx % a.nsplit;
  const int bh = (idx / a.nsplit) * 8 + xcd;
  if (bh >= a.BH) return;
  const int h = bh % a.H;
  const int j0 = split * DV;
  const int L = a.L;

  const int tid = threadIdx.x;
  const int w = tid >> 6;      // wavefront 0..7: phase-A rows 8w.., state rows 16w..
  const int l = tid & 63;
  const int m = l & 15;        // MFMA row / column within a tile
  const int g = l >> 4;        // MFMA lane group
  const int I = w & 3;         // query block of this wavefront
  const bool srow = w < D / 16;   // owns state rows 16w..16w+15
  const int vj = tid % VRW;    // value-load role: columns VC*vj.., rows VR*vs..
  const int vs = tid / VRW;

  const T* __restrict__ qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D + j0;
  const float* __restrict__ lgg = a.log_g + (size_t)bh * L * D;
  T* __restrict__ yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D + j0;
  T* __restrict__ yag = a.y_anchor ? reinterpret_cast<T*>(a.y_anchor) + (size_t)bh * L * D + j0 : nullptr;
  float* __restrict__ lseg = (a.lse && split == 0) ? a.lse + (size_t)bh * L : nullptr;
  T* sStg = sStgAll + I * 16 * Lay::LDSTG;

  // ---- zero the key/value rings (the window of chunk 0 reads "chunk -1") ----
  for (int i = tid; i < 128 * Lay::LDK; i += 512) sK[i] = from_f32<T>(0.f);
  for (int i = tid; i < DV * Lay::LDVT; i += 512) sVt[i] = from_f32<T>(0.f);

  // ---- sink keys as A-operand fragments (rows = sinks), resident throughout ----
  frag muf[NF];
  {
    const bool live = m < a.n_meta;
    const T* mp = reinterpret_cast<const T*>(a.meta) + ((size_t)h * a.n_meta + (live ? m : 0)) * D + g * (D / 4);
    uint4 raw[QV];
#pragma unroll
    for (int e = 0; e < QV; ++e) raw[e] = live ? ld16(mp + e * EPV) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < NF; ++e) muf[e] = frag_at<T>(raw, e);
  }

  // ---- state slice in accumulators: rows 16w + 4g + r, cols 16ct + m (w < D/16) ----
  f32x4 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = zero4();

  // ---- per-chunk global data (prefetched one chunk ahead, kept as raw bits) ----
  float lgA[8][DPL];    // phase A: rows 8w+rr, dims DPL*l + dd
  uint32_t kA[8];       // the same rows' keys: DPL elements packed in 32 bits
  uint32_t qA[8];       // ... and queries
  uint32_t vA[VR];      // values: rows VR*vs + rr, columns VC*vj.. packed in 32 bits

  auto load_rows = [&](int c, bool full) __attribute__((always_inline)) {
    const int t0 = c * C;
    {
      const int tb = t0 + 8 * w;
      const float* lp = lgg + (size_t)tb * D + DPL * l;
      const T* kp = kg + (size_t)tb * D + DPL * l;
      const T* qp = qg + (size_t)tb * D + DPL * l;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const bool ok = full || tb + rr < L;
        const int ro = ok ? rr * D : -tb * D;       // row 0 of the slice when out of range
        float lv[DPL];
        if constexpr (DPL == 2) {
          const float2 f = *reinterpret_cast<const float2*>(lp + ro);
          lv[0] = f.x;
          lv[1] = f.y;
        } else {
          lv[0] = lp[ro];
        }
        uint32_t kv, qv;
        if constexpr (DPL * sizeof(T) == 4) {
          kv = *reinterpret_cast<const uint32_t*>(kp + ro);
          qv = *reinterpret_cast<const uint32_t*>(qp + ro);
        } else {
          kv = *reinterpret_cast<const uint16_t*>(kp + ro);
          qv = *reinterpret_cast<const uint16_t*>(qp + ro);
        }
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) lgA[rr][dd] = ok ? lv[dd] : 0.f;
        kA[rr] = ok ? kv : 0u;
        qA[rr] = ok ? qv : 0u;
      }
    }
    {
      const int tb = t0 + VR * vs;
      const T* vp = vg + (size_t)tb * D + VC * vj;
#pragma unroll
      for (int rr = 0; rr < VR; ++rr) {
        const bool ok = full || tb + rr < L;
        const uint32_t u = *reinterpret_cast<const uint32_t*>(vp + (ok ? rr * D : -tb * D));
        vA[rr] = ok ? u : 0u;
      }
    }
  };
  // a uniform branch: full chunks load without per-row guards
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    if ((c + 1) * C <= L) load_rows(c, true);
    else load_rows(c, false);
  };
  // element dd of a packed 32-bit word, as float
  auto elem32 = [&](uint32_t u, int dd) __attribute__((always_inline)) -> float {
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, u);
    else return __builtin_bit_cast(float, dd == 0 ? (u << 16) : (u & 0xffff0000u));
  };

  const int nc = (L + C - 1) / C;
  if (nc > 0) load_chunk(0);
  __syncthreads();

  for (int c = 0; c < nc; ++c) {
    const int t0 = c * C;
    const int cur = (c & 1) * 64;       // ring half of this chunk
    const int prv = 64 - cur;           // ring half of the previous chunk

    // ================= phase A: log2-gate prefix and operand staging ========
    float loc[8][DPL];                  // prefix inside this wavefront's 8 rows
    float tot[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        run += log2_gate(lgA[rr][dd]);
        loc[rr][dd] = run;
      }
      tot[dd] = run;
    }
    if constexpr (DPL == 2) *reinterpret_cast<float2*>(sTot + w * D + 2 * l) = make_float2(tot[0], tot[1]);
    else sTot[w * D + l] = tot[0];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      T* krp = sK + (cur + 8 * w + rr) * Lay::LDK + DPL * l;
      T* qrp = sQ + (8 * w + rr) * Lay::LDK + DPL * l;
      if constexpr (DPL * sizeof(T) == 4) {
        *reinterpret_cast<uint32_t*>(krp) = kA[rr];
        *reinterpret_cast<uint32_t*>(qrp) = qA[rr];
      } else {
        krp[0] = from_f32<T>(elem32(kA[rr], 0));
        qrp[0] = from_f32<T>(elem32(qA[rr], 0));
      }
    }
    // values, transposed into the ring: sVt[j][cur + s], 4 tokens per write
#pragma unroll
    for (int cc = 0; cc < VC; ++cc) {
      float vv[VR];
#pragma unroll
      for (int rr = 0; rr < VR; ++rr) vv[rr] = elem32(vA[rr], cc);
      store_pack<T, 4>(sVt + (VC * vj + cc) * Lay::LDVT + cur + VR * vs, vv);
    }
    // S_c (rounded to the element type) for the readout: sSt[j][i], 4 rows i per write
    if (srow) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float sv[4] = {acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]};
        store_pack<T, 4>(sSt + (16 * ct + m) * Lay::LDST + 16 * w + 4 * g, sv);
      }
    }
    if (STATES && srow) {
      // chunk-start state for the backward pass: S_c[i][j], row-major
      T* sg = reinterpret_cast<T*>(a.states) + ((size_t)bh * nc + c) * D * D + j0;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) sg[(size_t)(16 * w + 4 * g + r) * D + 16 * ct + m] = from_f32<T>(acc[ct][r]);
    }
    __syncthreads();

    // chunk prefix beta = offset of this wavefront's rows + loc; B = chunk total
    float Bt[DPL], off[DPL];
    bool wide = false;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      float o = 0.f, b = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        const float tv = sTot[ww * D + i];
        o += ww < w ? tv : 0.f;
        b += tv;
      }
      off[dd] = o;
      Bt[dd] = b;
      wide |= -b > kMaxSpanLog2;
    }
    // every wavefront covers all D dims, so this ballot is the chunk's decision
    const bool pairwise = __any(wide);
    float kh[DPL][8];
    if (!pairwise) {
      float eB[DPL];
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) eB[dd] = exp_2(Bt[dd]);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int s = 8 * w + rr;
        float qe[DPL], kp[DPL];
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          const float beta = off[dd] + loc[rr][dd];
          kp[dd] = elem32(kA[rr], dd) * exp_2(-beta);
          kh[dd][rr] = kp[dd] * eB[dd];
          qe[dd] = elem32(qA[rr], dd) * exp_2(beta);
        }
        if constexpr (DPL == 2) {
          *reinterpret_cast<bf16x2*>(sQe + s * Lay::LDK + 2 * l) = bf16x2{static_cast<bf16>(qe[0]), static_cast<bf16>(qe[1])};
          *reinterpret_cast<bf16x2*>(sKp + s * Lay::LDK + 2 * l) = bf16x2{static_cast<bf16>(kp[0]), static_cast<bf16>(kp[1])};
        } else {
          sQe[s * Lay::LDK + l] = from_f32<T>(qe[0]);
          sKp[s * Lay::LDK + l] = from_f32<T>(kp[0]);
        }
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int s = 8 * w + rr;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          const float beta = off[dd] + loc[rr][dd];
          kh[dd][rr] = elem32(kA[rr], dd) * exp_2(Bt[dd] - beta);
          sBeta[s * Lay::LDE + DPL * l + dd] = beta;
        }
      }
    }
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      store_pack<T, 8>(sKhT + (DPL * l + dd) * Lay::LDKH + 8 * w, kh[dd]);
      if (w == 0) sBexp[DPL * l + dd] = exp_2(Bt[dd]);
    }
    if (c + 1 < nc) load_chunk(c + 1);
    __syncthreads();

    // ================= phase B: the pair (I, I+4) works on query block I =====
    auto phase_b = [&](auto Ic, auto Hc) __attribute__((always_inline)) {
      constexpr int QB = decltype(Ic)::value;         // query block
      constexpr int HF = decltype(Hc)::value;         // half
      constexpr int U0 = 16 * QB < 32 ? 16 * QB : 32; // first window key (of [prev; cur]) staged
      constexpr int JB = QB < 2 ? QB : 2;             // window tile kt holds intra key block kt - 4 + JB
      constexpr int K0 = 3 * HF;                      // this wavefront's window tiles K0..K0+2
      const int tme = t0 + 16 * QB + m;               // this lane's query

      // raw q (anchor logits) and Qe = q * 2^beta (readout, intra scores): B operands
      frag qf[NF], qe[NF];
      if (!pairwise) {
        const T* qp = sQ + (16 * QB + m) * Lay::LDK + g * (D / 4);
        const T* ep = sQe + (16 * QB + m) * Lay::LDK + g * (D / 4);
#pragma unroll
        for (int e = 0; e < NF; ++e) {
          qf[e] = M::load(qp + e * M::KPL);
          qe[e] = M::load(ep + e * M::KPL);
        }
      } else {
        uint4 raw[QV];
        const T* qp = qg + (size_t)(tme < L ? tme : 0) * D + g * (D / 4);
#pragma unroll
        for (int e = 0; e < QV; ++e) raw[e] = tme < L ? ld16(qp + e * EPV) : make_uint4(0, 0, 0, 0);
        const float* bp = sBeta + (16 * QB + m) * Lay::LDE + g * (D / 4);
#pragma unroll
        for (int e = 0; e < NF; ++e) {
          float tmp[M::KPL];
#pragma unroll
          for (int u = 0; u < M::KPL; ++u) tmp[u] = elem_f32<T>(raw, e * M::KPL + u) * exp_2(bp[e * M::KPL + u]);
          qf[e] = frag_at<T>(raw, e);
          qe[e] = M::pack(tmp);
        }
      }

      // ---- anchor logits Z^T[u][t] for this half's keys, plus sinks (first half) ----
      // Window tile kt (keys u in [U0+16kt, U0+16kt+16) of [prev; cur]) is
      // needed if any query of the block has a key of it inside its window:
      // valid u lie in [16QB+65-w, 16QB+79], and u >= 64 in the first chunk.
      bool need[3];
      {
        const int vlo = 16 * QB + 65 - a.window;
        const int vlo0 = (c == 0 && vlo < 64) ? 64 : vlo;
#pragma unroll
        for (int k3 = 0; k3 < 3; ++k3) {
          const int ulo = U0 + 16 * (K0 + k3);
          need[k3] = ulo + 15 >= vlo0 && ulo <= 16 * QB + 79;
        }
      }
      f32x4 z[3];
#pragma unroll
      for (int k3 = 0; k3 < 3; ++k3) {
        z[k3] = zero4();
        if (!need[k3]) continue;
        const int u = U0 + 16 * (K0 + k3) + m;
        const T* kp = sK + ((u + prv) & 127) * Lay::LDK + g * (D / 4);
        f32x4 cacc = zero4();
#pragma unroll
        for (int e = 0; e < NF; ++e) cacc = M::mma(M::load(kp + e * M::KPL), qf[e], cacc);
        z[k3] = cacc;
      }
      f32x4 zs = zero4();
      if constexpr (HF == 0) {
#pragma unroll
        for (int e = 0; e < NF; ++e) zs = M::mma(muf[e], qf[e], zs);
      }

      // ---- intra-chunk gated scores A^T[s][t] among this half's tiles ----
      f32x4 ai[3];
#pragma unroll
      for (int k3 = 0; k3 < 3; ++k3) {
        ai[k3] = zero4();
        const int J = K0 + k3 - 4 + JB;
        if (J < 0 || J > QB) continue;
        if (!pairwise) {
          const T* kp = sKp + (16 * J + m) * Lay::LDK + g * (D / 4);
          f32x4 sc = zero4();
#pragma unroll
          for (int e = 0; e < NF; ++e) sc = M::mma(M::load(kp + e * M::KPL), qe[e], sc);
          ai[k3] = sc;
        } else {
          // pairwise gate products in fp32 (a decay span too wide to factorise)
          const T* qrow = qg + (size_t)(tme < L ? tme : 0) * D;
          const float* bt = sBeta + (16 * QB + m) * Lay::LDE;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ks = 16 * J + 4 * g + r;
            float sum = 0.f;
            if (ks <= 16 * QB + m && tme < L) {
              const T* krow = sK + (cur + ks) * Lay::LDK;
              const float* bs = sBeta + ks * Lay::LDE;
              for (int i = 0; i < D; ++i) sum += to_f32(qrow[i]) * to_f32(krow[i]) * exp_2(bt[i] - bs[i]);
            }
            ai[k3][r] = sum;
          }
        }
        if (J == QB) {
#pragma unroll
          for (int r = 0; r < 4; ++r) ai[k3][r] = 4 * g + r <= m ? ai[k3][r] : 0.f;
        }
      }

      // ---- softmax over this half's keys (+ sinks); the pair combines (max, sum) ----
      // Maxima are taken on raw logits (the scale is positive) and the scale
      // is folded into the exponent: P = 2^{z * scale*log2e - max}.
      float mxo, smo;
      {
        float mr = -INFINITY;
        if constexpr (HF == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            zs[r] = 4 * g + r < a.n_meta ? zs[r] : -INFINITY;
            mr = fmaxf(mr, zs[r]);
          }
        }
        // key valid iff 0 <= t - s < lim; in the first chunk also s >= 0 (t - s <= t)
        const int lim = (c == 0 && 16 * QB + m + 1 < a.window) ? 16 * QB + m + 1 : a.window;
        const int dbase = 16 * QB + 64 - U0 + m - 4 * g;   // t - s for window tile 0, r = 0
#pragma unroll
        for (int k3 = 0; k3 < 3; ++k3)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int dts = dbase - 16 * (K0 + k3) - r;
            const bool ok = need[k3] && (unsigned)dts < (unsigned)lim;
            z[k3][r] = ok ? z[k3][r] : -INFINITY;
            mr = fmaxf(mr, z[k3][r]);
          }
        mr = xgroup_max(mr);
        mxo = mr * a.scale_log2;                            // -inf for a half without a valid key
        const float mref = mr == -INFINITY ? 0.f : mxo;
        float sr = 0.f;
        if constexpr (HF == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sr += exp_2(fmaf(zs[r], a.scale_log2, -mref));
        }
#pragma unroll
        for (int k3 = 0; k3 < 3; ++k3)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            z[k3][r] = exp_2(fmaf(z[k3][r], a.scale_log2, -mref));   // 2^-inf = 0 for masked keys
            sr += z[k3][r];
          }
        smo = xgroup_sum(sr);
        // (the query's own key is always valid, so the pair's combined maximum is finite)
        if (g == 0) *reinterpret_cast<float2*>(sStat + (w * 16 + m) * 2) = make_float2(mxo, smo);
      }
      __syncthreads();
      const float2 pst = *reinterpret_cast<const float2*>(sStat + ((w ^ 4) * 16 + m) * 2);
      const float mx = fmaxf(mxo, pst.x);
      const float den = smo * exp_2(mxo - mx) + pst.y * exp_2(pst.x - mx);
      const float inv = 1.0f / den;
      const float fo = exp_2(mxo - mx) * inv;         // this half's P -> softmax weight
      // ---- staged matrix M[t][u] = alpha * P/den (+ A on this chunk's keys) ----
#pragma unroll
      for (int k3 = 0; k3 < 3; ++k3) {
        float v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = fmaf(z[k3][r], a.alpha * fo, ai[k3][r]);
        store_pack<T, 4>(sStg + m * Lay::LDSTG + 16 * (K0 + k3) + 4 * g, v4);
      }
      if (HF == 0 && lseg && g == 0 && tme < L) lseg[tme] = (mx + __log2f(den)) * kLn2;
      __syncthreads();

      // ---- output O^T[j][t] = V^T M^T over the 96 staged keys + S_c^T Qe^T ----
      const T* bp = sStg + m * Lay::LDSTG + g * 24;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int ct = HF * NCH + ch;
        f32x4 o = zero4();
#pragma unroll
        for (int e = 0; e < 24 / M::KPL; ++e) {
          const int u = U0 + g * 24 + e * M::KPL;
          const T* ap = sVt + (16 * ct + m) * Lay::LDVT + ((u + prv) & 127);
          o = M::mma(M::load(ap), M::load(bp + e * M::KPL), o);
        }
        const T* sp = sSt + (16 * ct + m) * Lay::LDST + g * (D / 4);
#pragma unroll
        for (int e = 0; e < NF; ++e) o = M::mma(M::load(sp + e * M::KPL), qe[e], o);
        if (tme < L) {
          const float v4[4] = {o[0], o[1], o[2], o[3]};
          store_pack<T, 4>(yg + (size_t)tme * D + 16 * ct + 4 * g, v4);
        }
      }
      if (yag) {
        // the anchor branch alone (optional output): stage P/den and repeat V^T P^T
        __syncthreads();
#pragma unroll
        for (int k3 = 0; k3 < 3; ++k3) {
          float v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = z[k3][r] * fo;
          store_pack<T, 4>(sStg + m * Lay::LDSTG + 16 * (K0 + k3) + 4 * g, v4);
        }
        __syncthreads();
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          const int ct = HF * NCH + ch;
          f32x4 o = zero4();
#pragma unroll
          for (int e = 0; e < 24 / M::KPL; ++e) {
            const int u = U0 + g * 24 + e * M::KPL;
            const T* ap = sVt + (16 * ct + m) * Lay::LDVT + ((u + prv) & 127);
            o = M::mma(M::load(ap), M::load(bp + e * M::KPL), o);
          }
          if (tme < L) {
            const float v4[4] = {o[0], o[1], o[2], o[3]};
            store_pack<T, 4>(yag + (size_t)tme * D + 16 * ct + 4 * g, v4);
          }
        }
      }
    };
    if (!STATES) {
      switch (w) {
        case 0: phase_b(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}); break;
        case 1: phase_b(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}); break;
        case 2: phase_b(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{}); break;
        case 3: phase_b(std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{}); break;
        case 4: phase_b(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}); break;
        case 5: phase_b(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); break;
        case 6: phase_b(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}); break;
        default: phase_b(std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}); break;
      }
    }

    // ---- state carry: S = 2^B * S + Kh^T V over this chunk's keys ----
    if (srow) {
      const int ib = 16 * w;
      float dec[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) dec[r] = sBexp[ib + 4 * g + r];
      const T* ap = sKhT + (ib + m) * Lay::LDKH + g * 16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 s = acc[ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] *= dec[r];
        const T* bv = sVt + (16 * ct + m) * Lay::LDVT + cur + g * 16;
#pragma unroll
        for (int e = 0; e < 16 / M::KPL; ++e) s = M::mma(M::load(ap + e * M::KPL), M::load(bv + e * M::KPL), s);
        acc[ct] = s;
      }
    }
    __syncthreads();
  }

  if (a.state_out && srow) {
    float* so = a.state_out + (size_t)bh * D * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) so[(size_t)(16 * w + 4 * g + r) * D + j0 + 16 * ct + m] = acc[ct][r];
  }
}

template <typename T, int D, int DV, bool STATES>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  typedef FwdLayout<T, D, DV> Lay;
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS budget");
  static_assert(D == 128 || (D == 64 && sizeof(T) == 2) || (D == 64 && DV == 32), "shapes");
  const int smem = Lay::TOTAL;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lizard_fwd_kernel<T, D, DV, STATES>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  const int groups = (a.BH + 7) / 8;
  dim3 grid(8 * groups * a.nsplit);
  hipLaunchKernelGGL((lizard_fwd_kernel<T, D, DV, STATES>), grid, dim3(512), smem, st, a);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_fwd_s(const FwdArgs& a, hipStream_t st) {
  return a.states ? launch_fwd_t<T, D, DV, true>(a, st) : launch_fwd_t<T, D, DV, false>(a, st);
}

int fwd_value_slice(int dtype_bf16, int D) {
  if (dtype_bf16) return 64;       // D = 64: one slice; D = 128: two
  return D == 64 ? 32 : 0;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int D, hipStream_t st) {
  if (dtype_bf16 && D == 128) return launch_fwd_s<bf16, 128, 64>(a, st);
  if (dtype_bf16 && D == 64) return launch_fwd_s<bf16, 64, 64>(a, st);
  if (!dtype_bf16 && D == 64) return launch_fwd_s<float, 64, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lizard
