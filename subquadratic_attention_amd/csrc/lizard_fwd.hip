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
// Work decomposition: one workgroup of 4 wavefronts per (batch, head, slice
// of DV value columns).  The workgroup walks the chunks in order and keeps
// its slice of the float32 state in MFMA accumulators; wavefront I owns
// query block I (16 rows) of every chunk and rows [I*D/4, (I+1)*D/4) of the
// state.  Keys and values of the previous chunk stay in an LDS ring for the
// window.  All products are computed transposed (keys or value columns on
// the MFMA rows, the block's 16 queries on its columns), so each lane ends
// with 4 consecutive keys / columns of one query: packed LDS and global
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
  static constexpr int LDE = D + 4;         // sE [64][LDE] float: 2^beta (or beta on the pairwise path)
  static constexpr int LDSTG = 96 + PAD;    // per-wave staging [16][LDSTG]
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_K = 0;
  static constexpr int OFF_VT = OFF_K + a16(128 * LDK * (int)sizeof(T));
  static constexpr int OFF_KP = OFF_VT + a16(DV * LDVT * (int)sizeof(T));
  static constexpr int OFF_KHT = OFF_KP + a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_ST = OFF_KHT + a16(D * LDKH * (int)sizeof(T));
  static constexpr int OFF_E = OFF_ST + a16(DV * LDST * (int)sizeof(T));
  static constexpr int OFF_TOT = OFF_E + a16(64 * LDE * 4);
  static constexpr int OFF_BEXP = OFF_TOT + a16(4 * D * 4);
  static constexpr int OFF_STG = OFF_BEXP + a16(D * 4);
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

template <typename T, int D, int DV>
__global__ __launch_bounds__(256, 1) void lizard_fwd_kernel(FwdArgs a) {
  typedef FwdLayout<T, D, DV> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int C = 64;
  constexpr int DPL = D / 64;                 // phase-A dims per lane
  constexpr int EPV = 16 / sizeof(T);         // elements per 16-byte vector
  constexpr int QV = D / 4 / EPV;             // 16-byte vectors in a lane's k-quarter of a row
  constexpr int NF = D / 4 / M::KPL;          // MFMA steps over a D contraction
  constexpr int NCT = DV / 16;                // value column tiles
  constexpr int NRT = D / 64;                 // state row tiles per wavefront
  constexpr int VC = 4 / sizeof(T);           // value columns per thread in the value load
  constexpr int VRW = DV / VC;                // threads across a value row
  static_assert(VRW * 8 == 256, "value load: 8 rows per thread");

  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + Lay::OFF_K);
  T* sVt = reinterpret_cast<T*>(smem + Lay::OFF_VT);
  T* sKp = reinterpret_cast<T*>(smem + Lay::OFF_KP);
  T* sKhT = reinterpret_cast<T*>(smem + Lay::OFF_KHT);
  T* sSt = reinterpret_cast<T*>(smem + Lay::OFF_ST);
  float* sE = reinterpret_cast<float*>(smem + Lay::OFF_E);
  float* sTot = reinterpret_cast<float*>(smem + Lay::OFF_TOT);
  float* sBexp = reinterpret_cast<float*>(smem + Lay::OFF_BEXP);
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
  const int w = tid >> 6;      // wavefront = query block I = state row group
  const int l = tid & 63;
  const int m = l & 15;        // MFMA row / column within a tile
  const int g = l >> 4;        // MFMA lane group
  const int vj = tid % VRW;    // value-load role: columns VC*vj.., rows 8*vs..
  const int vs = tid / VRW;

  const T* __restrict__ qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D + j0;
  const float* __restrict__ lgg = a.log_g + (size_t)bh * L * D;
  T* __restrict__ yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D + j0;
  T* __restrict__ yag = a.y_anchor ? reinterpret_cast<T*>(a.y_anchor) + (size_t)bh * L * D + j0 : nullptr;
  float* __restrict__ lseg = (a.lse && split == 0) ? a.lse + (size_t)bh * L : nullptr;
  T* sStg = sStgAll + w * 16 * Lay::LDSTG;

  // ---- zero the key/value rings (the window of chunk 0 reads "chunk -1") ----
  for (int i = tid; i < 128 * Lay::LDK; i += 256) sK[i] = from_f32<T>(0.f);
  for (int i = tid; i < DV * Lay::LDVT; i += 256) sVt[i] = from_f32<T>(0.f);

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

  // ---- state slice in accumulators: rows w*D/4 + 16*rt + 4*g + r, cols 16*ct + m ----
  f32x4 acc[NRT][NCT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = zero4();

  // ---- per-chunk global data (prefetched one chunk ahead, kept as raw bits) ----
  float lgA[16][DPL];   // phase A: rows 16w+rr, dims DPL*l + dd
  uint32_t kA[16];      // the same rows' keys: DPL elements packed in 32 bits
  uint32_t vA[8];       // values: rows 8*vs + rr, columns VC*vj.. packed in 32 bits
  uint4 qraw[QV];       // query row 16w+m, k-quarter g

  auto load_rows = [&](int c, bool full) __attribute__((always_inline)) {
    const int t0 = c * C;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = t0 + 16 * w + rr;
      const bool ok = full || t < L;
      const size_t off = (size_t)(ok ? t : 0) * D + DPL * l;
      float lv[DPL];
      if constexpr (DPL == 2) {
        const float2 f = *reinterpret_cast<const float2*>(lgg + off);
        lv[0] = f.x;
        lv[1] = f.y;
      } else {
        lv[0] = lgg[off];
      }
      uint32_t kv;
      if constexpr (DPL * sizeof(T) == 4) kv = *reinterpret_cast<const uint32_t*>(kg + off);
      else kv = *reinterpret_cast<const uint16_t*>(kg + off);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) lgA[rr][dd] = ok ? lv[dd] : 0.f;
      kA[rr] = ok ? kv : 0u;
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int t = t0 + 8 * vs + rr;
      const bool ok = full || t < L;
      const uint32_t u = *reinterpret_cast<const uint32_t*>(vg + (size_t)(ok ? t : 0) * D + VC * vj);
      vA[rr] = ok ? u : 0u;
    }
    {
      const int t = t0 + 16 * w + m;
      const bool ok = full || t < L;
#pragma unroll
      for (int e = 0; e < QV; ++e) {
        const uint4 r = ld16(qg + (size_t)(ok ? t : 0) * D + g * (D / 4) + e * EPV);
        qraw[e] = ok ? r : make_uint4(0, 0, 0, 0);
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
    float loc[16][DPL];                 // prefix inside this wavefront's 16 rows
    float tot[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        run += log2_gate(lgA[rr][dd]);
        loc[rr][dd] = run;
      }
      tot[dd] = run;
    }
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) sTot[w * D + DPL * l + dd] = tot[dd];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      T* krp = sK + (cur + 16 * w + rr) * Lay::LDK + DPL * l;
      if constexpr (DPL * sizeof(T) == 4) *reinterpret_cast<uint32_t*>(krp) = kA[rr];
      else krp[0] = from_f32<T>(elem32(kA[rr], 0));
    }
    // values, transposed into the ring: sVt[j][cur + s], 8 tokens per 16-byte run
#pragma unroll
    for (int cc = 0; cc < VC; ++cc) {
      float vv[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) vv[rr] = elem32(vA[rr], cc);
      store_pack<T, 8>(sVt + (VC * vj + cc) * Lay::LDVT + cur + 8 * vs, vv);
    }
    // S_c (rounded to the element type) for the readout: sSt[j][i], 4 rows i per write
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float sv[4] = {acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]};
        store_pack<T, 4>(sSt + (16 * ct + m) * Lay::LDST + w * (D / 4) + 16 * rt + 4 * g, sv);
      }
    if (a.states) {
      // chunk-start state for the backward pass: S_c[i][j], row-major
      T* sg = reinterpret_cast<T*>(a.states) + ((size_t)bh * nc + c) * D * D + j0;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sg[(size_t)(w * (D / 4) + 16 * rt + 4 * g + r) * D + 16 * ct + m] = from_f32<T>(acc[rt][ct][r]);
    }
    __syncthreads();

    // chunk prefix beta = offset of this wavefront's rows + loc; B = chunk total
    float Bt[DPL], off[DPL];
    bool wide = false;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      const float t0v = sTot[0 * D + i], t1v = sTot[1 * D + i], t2v = sTot[2 * D + i], t3v = sTot[3 * D + i];
      off[dd] = w == 0 ? 0.f : w == 1 ? t0v : w == 2 ? t0v + t1v : t0v + t1v + t2v;
      Bt[dd] = t0v + t1v + t2v + t3v;
      wide |= -Bt[dd] > kMaxSpanLog2;
    }
    // every wavefront covers all D dims, so this ballot is the chunk's decision
    const bool pairwise = __any(wide);
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      float kh[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int s = 16 * w + rr;
        const float beta = off[dd] + loc[rr][dd];
        const float kf = elem32(kA[rr], dd);
        if (!pairwise) {
          const float kp = kf * exp_2(-beta);
          kh[rr] = kp * exp_2(Bt[dd]);
          sE[s * Lay::LDE + i] = exp_2(beta);
          sKp[s * Lay::LDK + i] = from_f32<T>(kp);
        } else {
          kh[rr] = kf * exp_2(Bt[dd] - beta);
          sE[s * Lay::LDE + i] = beta;
        }
      }
      store_pack<T, 16>(sKhT + i * Lay::LDKH + 16 * w, kh);
      if (w == 0) sBexp[i] = exp_2(Bt[dd]);
    }
    uint4 qcur[QV];
#pragma unroll
    for (int e = 0; e < QV; ++e) qcur[e] = qraw[e];
    if (c + 1 < nc) load_chunk(c + 1);
    __syncthreads();

    // ================= phase B: wavefront I = w works on query block I ======
    auto phase_b = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int I = decltype(Ic)::value;
      constexpr int U0 = 16 * I < 32 ? 16 * I : 32;  // first window key (of [prev; cur]) staged
      constexpr int JB = I < 2 ? I : 2;               // window tile kt holds intra key block kt - 4 + JB
      const int tme = t0 + 16 * I + m;                // this lane's query

      // Qe = q * 2^beta for the readout and the intra scores (B operand: queries)
      frag qe[NF];
      {
        const float* ep = sE + (16 * I + m) * Lay::LDE + g * (D / 4);
#pragma unroll
        for (int e = 0; e < NF; ++e) {
          float tmp[M::KPL];
#pragma unroll
          for (int u = 0; u < M::KPL; ++u) {
            const int kk = e * M::KPL + u;
            const float ev = pairwise ? exp_2(ep[kk]) : ep[kk];
            tmp[u] = elem_f32<T>(qcur, kk) * ev;
          }
          qe[e] = M::pack(tmp);
        }
      }

      // ---- anchor logits Z^T[u][t]: keys u in [U0, U0 + 96) of [prev; cur], sinks ----
      f32x4 z[6];
#pragma unroll
      for (int kt = 0; kt < 6; ++kt) {
        const int u = U0 + 16 * kt + m;
        const T* kp = sK + ((u + prv) & 127) * Lay::LDK + g * (D / 4);
        f32x4 cacc = zero4();
#pragma unroll
        for (int e = 0; e < NF; ++e) cacc = M::mma(M::load(kp + e * M::KPL), frag_at<T>(qcur, e), cacc);
        z[kt] = cacc;
      }
      f32x4 zs = zero4();
#pragma unroll
      for (int e = 0; e < NF; ++e) zs = M::mma(muf[e], frag_at<T>(qcur, e), zs);

      // ---- intra-chunk gated scores A^T[s][t], key blocks J <= I, s <= t ----
      f32x4 ai[6];
#pragma unroll
      for (int kt = 0; kt < 6; ++kt) {
        ai[kt] = zero4();
        const int J = kt - 4 + JB;
        if (J < 0 || J > I) continue;
        if (!pairwise) {
          const T* kp = sKp + (16 * J + m) * Lay::LDK + g * (D / 4);
          f32x4 sc = zero4();
#pragma unroll
          for (int e = 0; e < NF; ++e) sc = M::mma(M::load(kp + e * M::KPL), qe[e], sc);
          ai[kt] = sc;
        } else {
          // pairwise gate products in fp32 (a decay span too wide to factorise)
          const T* qrow = qg + (size_t)(tme < L ? tme : 0) * D;
          const float* bt = sE + (16 * I + m) * Lay::LDE;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ks = 16 * J + 4 * g + r;
            float sum = 0.f;
            if (ks <= 16 * I + m && tme < L) {
              const T* krow = sK + (cur + ks) * Lay::LDK;
              const float* bs = sE + ks * Lay::LDE;
              for (int i = 0; i < D; ++i) sum += to_f32(qrow[i]) * to_f32(krow[i]) * exp_2(bt[i] - bs[i]);
            }
            ai[kt][r] = sum;
          }
        }
        if (J == I) {
#pragma unroll
          for (int r = 0; r < 4; ++r) ai[kt][r] = 4 * g + r <= m ? ai[kt][r] : 0.f;
        }
      }

      // ---- softmax over window + sinks for this lane's query (keys across lanes) ----
      float mx, den;
      {
        float mr = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          zs[r] = 4 * g + r < a.n_meta ? zs[r] * a.scale_log2 : -INFINITY;
          mr = fmaxf(mr, zs[r]);
        }
#pragma unroll
        for (int kt = 0; kt < 6; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // key s = t0 - 64 + U0 + 16 kt + 4 g + r; query t = t0 + 16 I + m
            const int dts = (16 * I + 64 - U0 - 16 * kt) + m - 4 * g - r;   // t - s
            const bool ok = dts >= 0 && dts < a.window && (c > 0 || U0 + 16 * kt + 4 * g + r >= 64);
            z[kt][r] = ok ? z[kt][r] * a.scale_log2 : -INFINITY;
            mr = fmaxf(mr, z[kt][r]);
          }
        mx = xgroup_max(mr);
        float sr = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) sr += exp_2(zs[r] - mx);
#pragma unroll
        for (int kt = 0; kt < 6; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            z[kt][r] = exp_2(z[kt][r] - mx);   // exp2(-inf) = 0 for masked keys
            sr += z[kt][r];
          }
        den = xgroup_sum(sr);
      }
      const float inv = 1.0f / den;

      // ---- one staged matrix M[t][u] = alpha * P/den (+ A on this chunk's keys) ----
      {
        const float pa = a.alpha * inv;
#pragma unroll
        for (int kt = 0; kt < 6; ++kt) {
          float v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = fmaf(z[kt][r], pa, ai[kt][r]);
          store_pack<T, 4>(sStg + m * Lay::LDSTG + 16 * kt + 4 * g, v4);
        }
      }
      wave_lds_sync();

      // ---- output O^T[j][t] = V^T M^T over the 96 staged keys + S_c^T Qe^T ----
      const T* bp = sStg + m * Lay::LDSTG + g * 24;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
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
      if (lseg && g == 0 && tme < L) lseg[tme] = (mx + __log2f(den)) * kLn2;
      if (yag) {
        // the anchor branch alone (optional output): stage P/den and repeat V^T P^T
        wave_lds_sync();
#pragma unroll
        for (int kt = 0; kt < 6; ++kt) {
          float v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = z[kt][r] * inv;
          store_pack<T, 4>(sStg + m * Lay::LDSTG + 16 * kt + 4 * g, v4);
        }
        wave_lds_sync();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
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
    if (a.y) {  // (no outputs: the states-only pass of the backward)
      switch (w) {
        case 0: phase_b(std::integral_constant<int, 0>{}); break;
        case 1: phase_b(std::integral_constant<int, 1>{}); break;
        case 2: phase_b(std::integral_constant<int, 2>{}); break;
        default: phase_b(std::integral_constant<int, 3>{}); break;
      }
    }

    // ---- state carry: S = 2^B * S + Kh^T V over this chunk's keys ----
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int ib = w * (D / 4) + 16 * rt;
      float dec[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) dec[r] = sBexp[ib + 4 * g + r];
      const T* ap = sKhT + (ib + m) * Lay::LDKH + g * 16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 s = acc[rt][ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] *= dec[r];
        const T* bv = sVt + (16 * ct + m) * Lay::LDVT + cur + g * 16;
#pragma unroll
        for (int e = 0; e < 16 / M::KPL; ++e) s = M::mma(M::load(ap + e * M::KPL), M::load(bv + e * M::KPL), s);
        acc[rt][ct] = s;
      }
    }
    __syncthreads();
  }

  if (a.state_out) {
    float* so = a.state_out + (size_t)bh * D * D;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          so[(size_t)(w * (D / 4) + 16 * rt + 4 * g + r) * D + j0 + 16 * ct + m] = acc[rt][ct][r];
  }
}

template <typename T, int D, int DV>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  typedef FwdLayout<T, D, DV> Lay;
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS budget");
  const int smem = Lay::TOTAL;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lizard_fwd_kernel<T, D, DV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  const int groups = (a.BH + 7) / 8;
  dim3 grid(8 * groups * a.nsplit);
  hipLaunchKernelGGL((lizard_fwd_kernel<T, D, DV>), grid, dim3(256), smem, st, a);
  return hipGetLastError();
}

int fwd_value_slice(int dtype_bf16, int D) {
  if (dtype_bf16) return 64;       // D = 64: one slice; D = 128: two
  return D == 64 ? 32 : 0;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int D, hipStream_t st) {
  if (dtype_bf16 && D == 128) return launch_fwd_t<bf16, 128, 64>(a, st);
  if (dtype_bf16 && D == 64) return launch_fwd_t<bf16, 64, 64>(a, st);
  if (!dtype_bf16 && D == 64) return launch_fwd_t<float, 64, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lizard
