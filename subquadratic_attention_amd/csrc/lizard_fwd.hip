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
// matrix cores).  The sequence is cut into chunks of 64 tokens and each
// chunk into four 16-row blocks.  With loc_t the log-gate prefix of token t
// inside its block, tot_J the block total and R_J the chunk prefix at the
// end of block J-1 (R_0 = 0, R_4 = chunk total):
//
//   Qt   = q_t * e^{loc_t}                       (<= |q|)
//   Kown = k_s * e^{tot_J - loc_s}               (<= |k|)
//   intra block (I, J<I):  (Qt * e^{R_I - R_{J+1}}) . Kown_s      exps <= 0
//   intra block (I, I):    (Qt * e^{-tot_I}) . Kown_s, masked s <= t
//   inter readout:         (Qt * e^{R_I}) . S_c
//   carry:  S_{c+1} = e^{R_4} * S_c + (Kown * e^{R_4 - R_{J+1}})^T V
//
// Every factor except the diagonal block's e^{-tot_I} is <= 1, so nothing
// divides by a gate product and nothing overflows.  The diagonal factor is
// bounded by the block's own decay span; a block whose span exceeds 64
// (gates near zero) is computed pairwise in fp32 instead.
//
// Work decomposition: one workgroup of 4 wavefronts per (batch, head, slice
// of DV value columns).  The workgroup walks the chunks in order and keeps
// its slice of the float32 state in MFMA accumulators; wavefront I owns
// query block I of every chunk and rows [I*D/4, (I+1)*D/4) of the state.
// Keys and values of the previous chunk stay in an LDS ring for the window.
#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

template <typename T, int D, int DV>
struct FwdLayout {
  static constexpr int C = 64;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDK = D + PAD;       // sK ring [128][LDK], sKown [64][LDK]
  static constexpr int LDVT = 128 + PAD;    // sVt ring [DV][LDVT]
  static constexpr int LDKH = 64 + PAD;     // sKhT [D][LDKH]
  static constexpr int LDST = D + PAD;      // sSt [DV][LDST]
  static constexpr int LDLOC = D + 4;       // sLoc [64][LDLOC] float
  static constexpr int LDSTG = 96 + PAD;    // per-wave staging [16][LDSTG]
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int OFF_K = 0;
  static constexpr int OFF_VT = OFF_K + a16(128 * LDK * (int)sizeof(T));
  static constexpr int OFF_KOWN = OFF_VT + a16(DV * LDVT * (int)sizeof(T));
  static constexpr int OFF_KHT = OFF_KOWN + a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_ST = OFF_KHT + a16(D * LDKH * (int)sizeof(T));
  static constexpr int OFF_LOC = OFF_ST + a16(DV * LDST * (int)sizeof(T));
  static constexpr int OFF_TOT = OFF_LOC + a16(64 * LDLOC * 4);
  static constexpr int OFF_F = OFF_TOT + a16(4 * D * 4);
  static constexpr int OFF_BEXP = OFF_F + a16(16 * D * 4);
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
  constexpr int VV = DV / (4 * EPV);          // value vectors per thread per chunk
  constexpr int NCT = DV / 16;                // output column tiles
  constexpr int NRT = D / 64;                 // state row tiles per wavefront

  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + Lay::OFF_K);
  T* sVt = reinterpret_cast<T*>(smem + Lay::OFF_VT);
  T* sKown = reinterpret_cast<T*>(smem + Lay::OFF_KOWN);
  T* sKhT = reinterpret_cast<T*>(smem + Lay::OFF_KHT);
  T* sSt = reinterpret_cast<T*>(smem + Lay::OFF_ST);
  float* sLoc = reinterpret_cast<float*>(smem + Lay::OFF_LOC);
  float* sTot = reinterpret_cast<float*>(smem + Lay::OFF_TOT);
  float* sF = reinterpret_cast<float*>(smem + Lay::OFF_F);
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

  // ---- sink keys as B-operand fragments, resident for the whole sequence ----
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

  // ---- per-chunk global data (prefetched one chunk ahead) ----
  float lgA[16][DPL];   // phase A: rows 16w+rr, dims DPL*l + dd
  float kA[16][DPL];
  uint4 vraw[VV];       // value vectors
  uint4 qraw[QV];       // query row 16w+m, k-quarter g

  auto load_chunk = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = t0 + 16 * w + rr;
      const bool ok = t < L;
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        lgA[rr][dd] = ok ? lgg[(size_t)t * D + DPL * l + dd] : 0.f;
        kA[rr][dd] = ok ? to_f32(kg[(size_t)t * D + DPL * l + dd]) : 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < VV; ++p) {
      const int vi = tid + 256 * p;
      const int row = vi / (DV / EPV);
      const int cv = vi % (DV / EPV);
      const int t = t0 + row;
      vraw[p] = t < L ? ld16(vg + (size_t)t * D + cv * EPV) : make_uint4(0, 0, 0, 0);
    }
    {
      const int t = t0 + 16 * w + m;
#pragma unroll
      for (int e = 0; e < QV; ++e)
        qraw[e] = t < L ? ld16(qg + (size_t)t * D + g * (D / 4) + e * EPV) : make_uint4(0, 0, 0, 0);
    }
  };

  const int nc = (L + C - 1) / C;
  if (nc > 0) load_chunk(0);
  __syncthreads();

  for (int c = 0; c < nc; ++c) {
    const int t0 = c * C;
    const int cur = (c & 1) * 64;       // ring half of this chunk
    const int prv = 64 - cur;           // ring half of the previous chunk

    // ================= phase A: log-gate prefix and operand staging =========
    float loc[16][DPL];
    float tot[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        run += lgA[rr][dd];
        loc[rr][dd] = run;
      }
      tot[dd] = run;
    }
    float kown[16][DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      sTot[w * D + i] = tot[dd];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int s = 16 * w + rr;
        sLoc[s * Lay::LDLOC + i] = loc[rr][dd];
        kown[rr][dd] = kA[rr][dd] * exp_e(tot[dd] - loc[rr][dd]);
        sKown[s * Lay::LDK + i] = from_f32<T>(kown[rr][dd]);
        sK[(cur + s) * Lay::LDK + i] = from_f32<T>(kA[rr][dd]);
      }
    }
    // values, transposed into the ring: sVt[j][cur + s]
#pragma unroll
    for (int p = 0; p < VV; ++p) {
      const int vi = tid + 256 * p;
      const int row = vi / (DV / EPV);
      const int cv = vi % (DV / EPV);
#pragma unroll
      for (int e = 0; e < EPV; ++e) sVt[(cv * EPV + e) * Lay::LDVT + cur + row] = from_f32<T>(elem_f32<T>(vraw + p, e));
    }
    // S_c (rounded to the element type) for the readout: sSt[j][i]
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sSt[(16 * ct + m) * Lay::LDST + w * (D / 4) + 16 * rt + 4 * g + r] = from_f32<T>(acc[rt][ct][r]);
    __syncthreads();

#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const int i = DPL * l + dd;
      const float t0v = sTot[0 * D + i], t1v = sTot[1 * D + i], t2v = sTot[2 * D + i], t3v = sTot[3 * D + i];
      const float R1 = t0v, R2 = t0v + t1v, R3 = R2 + t2v, R4 = R3 + t3v;
      const float Rw = w == 0 ? 0.f : w == 1 ? R1 : w == 2 ? R2 : R3;
      const float Rw1 = Rw + tot[dd];
      const float fK = exp_e(R4 - Rw1);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sKhT[i * Lay::LDKH + 16 * w + rr] = from_f32<T>(kown[rr][dd] * fK);
      float* F = sF + (w * 4) * D + i;
      F[0 * D] = exp_e(Rw);
      F[1 * D] = exp_e(fminf(-tot[dd], 80.f));
      F[2 * D] = exp_e(Rw - R1);
      F[3 * D] = exp_e(Rw - R2);
      if (w == 0) sBexp[i] = exp_e(R4);
    }
    uint4 qcur[QV];
#pragma unroll
    for (int e = 0; e < QV; ++e) qcur[e] = qraw[e];
    if (c + 1 < nc) load_chunk(c + 1);
    __syncthreads();

    // ================= phase B: wavefront I = w works on query block I ======
    const int I = w;
    const int tq = t0 + 16 * I;               // first query row of this block
    float qt[D / 4];                          // Qt = q * e^{loc}, lane's k-quarter
    {
      const float* lp = sLoc + (16 * I + m) * Lay::LDLOC + g * (D / 4);
#pragma unroll
      for (int e = 0; e < D / 4; ++e) qt[e] = elem_f32<T>(qcur, e) * exp_e(lp[e]);
    }
    const float* FI = sF + (I * 4) * D + g * (D / 4);

    // ---- anchor logits: window keys u in [u0, u0 + 96) of [prev; cur], sinks ----
    const int u0 = 16 * I < 32 ? 16 * I : 32;
    f32x4 z[6];
#pragma unroll
    for (int kt = 0; kt < 6; ++kt) {
      const int u = u0 + 16 * kt + m;
      const T* kp = sK + ((u + prv) & 127) * Lay::LDK + g * (D / 4);
      f32x4 cacc = zero4();
#pragma unroll
      for (int e = 0; e < NF; ++e) cacc = M::mma(frag_at<T>(qcur, e), M::load(kp + e * M::KPL), cacc);
      z[kt] = cacc;
    }
    f32x4 zs = zero4();
#pragma unroll
    for (int e = 0; e < NF; ++e) zs = M::mma(frag_at<T>(qcur, e), muf[e], zs);

    float mx[4], den[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tq + 4 * g + r;
      float mr = m < a.n_meta ? zs[r] * a.scale_log2 : -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 6; ++kt) {
        const int s = t0 - 64 + u0 + 16 * kt + m;
        const bool ok = s >= 0 && s <= t && s > t - a.window;
        z[kt][r] = ok ? z[kt][r] * a.scale_log2 : -INFINITY;
        mr = fmaxf(mr, z[kt][r]);
      }
      mx[r] = group16_max(mr);
      float sr = m < a.n_meta ? exp_2(zs[r] * a.scale_log2 - mx[r]) : 0.f;
#pragma unroll
      for (int kt = 0; kt < 6; ++kt) {
        z[kt][r] = exp_2(z[kt][r] - mx[r]);   // exp2(-inf) = 0 for masked keys
        sr += z[kt][r];
      }
      den[r] = group16_sum(sr);
    }

    // ---- intra-chunk gated scores A[t][s], s <= t, staged for A * V ----
    {
      const int KI = I < 2 ? 32 : 64;
      float ub = 0.f;                       // largest diagonal decay span seen by this lane
#pragma unroll
      for (int e = 0; e < D / 4; ++e) ub = fmaxf(ub, -sTot[I * D + g * (D / 4) + e]);
      const bool fallback = __any(ub > 64.f);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= I) {
          f32x4 sc = zero4();
          if (J == I && fallback) {
            // pairwise exponents in fp32 (gates near zero inside this block)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int mt = 4 * g + r;
              float sum = 0.f;
              if (m <= mt && tq + mt < L) {
                const T* qrow = qg + (size_t)(tq + mt) * D;
                const T* krow = sK + (cur + 16 * I + m) * Lay::LDK;
                const float* lt = sLoc + (16 * I + mt) * Lay::LDLOC;
                const float* ls = sLoc + (16 * I + m) * Lay::LDLOC;
                for (int i = 0; i < D; ++i) sum += to_f32(qrow[i]) * to_f32(krow[i]) * exp_e(lt[i] - ls[i]);
              }
              sc[r] = sum;
            }
          } else {
            // query factor for key block J: 1 (J = I-1), e^{-tot_I} (J = I),
            // e^{R_I - R_1} (J = 0 < I-1), e^{R_I - R_2} (J = 1 < I-1)
            const int slot = J == I ? 1 : J == I - 1 ? -1 : J == 0 ? 2 : 3;
            const T* kp = sKown + (16 * J + m) * Lay::LDK + g * (D / 4);
#pragma unroll
            for (int e = 0; e < NF; ++e) {
              float tmp[M::KPL];
#pragma unroll
              for (int u = 0; u < M::KPL; ++u) {
                const int kk = e * M::KPL + u;
                tmp[u] = slot < 0 ? qt[kk] : qt[kk] * FI[slot * D + kk];
              }
              sc = M::mma(M::pack(tmp), M::load(kp + e * M::KPL), sc);
            }
            if (J == I) {
#pragma unroll
              for (int r = 0; r < 4; ++r) sc[r] = m <= 4 * g + r ? sc[r] : 0.f;
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sStg[(4 * g + r) * Lay::LDSTG + 16 * J + m] = from_f32<T>(sc[r]);
        } else if (J * 16 < KI) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sStg[(4 * g + r) * Lay::LDSTG + 16 * J + m] = from_f32<T>(0.f);
        }
      }
    }
    wave_lds_sync();

    // ---- gated output: intra A * V (keys of this chunk) + readout Qe * S_c ----
    f32x4 og[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) og[ct] = zero4();
    {
      const int KI = I < 2 ? 32 : 64;
      const int kq = KI / 4;                  // keys per lane group
      const T* ap = sStg + m * Lay::LDSTG + g * kq;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const T* bp = sVt + (16 * ct + m) * Lay::LDVT + cur + g * kq;
        f32x4 o = og[ct];
        for (int e = 0; e < kq / M::KPL; ++e) o = M::mma(M::load(ap + e * M::KPL), M::load(bp + e * M::KPL), o);
        og[ct] = o;
      }
      frag qe[NF];
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        float tmp[M::KPL];
#pragma unroll
        for (int u = 0; u < M::KPL; ++u) tmp[u] = qt[e * M::KPL + u] * FI[0 * D + e * M::KPL + u];
        qe[e] = M::pack(tmp);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const T* bp = sSt + (16 * ct + m) * Lay::LDST + g * (D / 4);
        f32x4 o = og[ct];
#pragma unroll
        for (int e = 0; e < NF; ++e) o = M::mma(qe[e], M::load(bp + e * M::KPL), o);
        og[ct] = o;
      }
    }
    wave_lds_sync();

    // ---- anchor output: P * V over the 96 staged window keys ----
#pragma unroll
    for (int kt = 0; kt < 6; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sStg[(4 * g + r) * Lay::LDSTG + 16 * kt + m] = from_f32<T>(z[kt][r]);
    wave_lds_sync();
    f32x4 oa[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 o = zero4();
      const T* ap = sStg + m * Lay::LDSTG + g * 24;
#pragma unroll
      for (int e = 0; e < 24 / M::KPL; ++e) {
        const int u = u0 + g * 24 + e * M::KPL;
        const T* bp = sVt + (16 * ct + m) * Lay::LDVT + ((u + prv) & 127);
        o = M::mma(M::load(ap + e * M::KPL), M::load(bp), o);
      }
      oa[ct] = o;
    }

    // ---- combine and store ----
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tq + 4 * g + r;
      if (t < L) {
        const float inv = 1.0f / den[r];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float ya = oa[ct][r] * inv;
          yg[(size_t)t * D + 16 * ct + m] = from_f32<T>(og[ct][r] + a.alpha * ya);
          if (yag) yag[(size_t)t * D + 16 * ct + m] = from_f32<T>(ya);
        }
        if (lseg && m == 0) lseg[t] = (mx[r] + __log2f(den[r])) * kLn2;
      }
    }

    // ---- state carry: S = e^{R_4} * S + Khat^T V over this chunk's keys ----
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
        const T* bp = sVt + (16 * ct + m) * Lay::LDVT + cur + g * 16;
#pragma unroll
        for (int e = 0; e < 16 / M::KPL; ++e) s = M::mma(M::load(ap + e * M::KPL), M::load(bp + e * M::KPL), s);
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
