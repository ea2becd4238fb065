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
// Work decomposition: one workgroup of 8 wavefronts per (batch, head, slice
// of DV value columns), walking the chunks in order.  Wavefronts I and I+4
// share a SIMD and split query block I (16 rows) of every chunk by kind of
// work: wavefront I ("softmax") computes the window logits, the softmax and
// the unnormalised weights P; wavefront I+4 ("gate") computes the gated
// intra-chunk scores, the readout of the state, the anchor product V^T P^T
// and the output, and owns D/4 rows of the float32 state in MFMA
// accumulators.  So the VALU-heavy and the MFMA-heavy half of each block run
// side by side on one SIMD.  Two workgroup barriers per chunk c:
//
//   interval 1: softmax(c) | gated scores, readout, state carry (c);
//               then every wavefront: prefix partial sums of chunk c+1
//   interval 2: gate wavefronts: V^T P^T and the output of chunk c;
//               every wavefront: decay factors and operands of chunk c+1
//               into LDS, global loads of chunk c+2
//
// Keys of the last two chunks stay in an LDS ring for the window, values of
// the last three (the output of chunk c reads two while chunk c+1's are
// written).  All products are computed transposed (keys or value columns on
// the MFMA rows, the block's 16 queries on its columns), so each lane ends
// with 4 consecutive keys / columns of one query: packed LDS and global
// writes and softmax reductions across 4 lane groups only.
#include <type_traits>

#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

// STATES: the states-only pass, which needs only the value ring, the Kh tile
// and the prefix totals (two workgroups per CU).
template <typename T, int D, int DV, bool STATES = false>
struct FwdLayout {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDK = D + PAD;       // sK ring [128][LDK]; sKp, sQe [64][LDK]; sMeta [16][LDK]
  static constexpr int LDVT = 192 + PAD;    // sVt ring of 3 chunk slots [DV][LDVT]
  static constexpr int LDKH = 64 + PAD;     // sKhT [D][LDKH]
  static constexpr int LDST = D + PAD;      // sSt [DV][LDST]
  static constexpr int LDP = 96 + PAD;      // window weights P, per query block [16][LDP]
  static constexpr int LDA = 64 + PAD;      // bf16: intra scores A, per query block [16][LDA]
  static constexpr int LDE = D + 4;         // wide-span chunks: beta [64][LDE] float over sKp, sQe
  static constexpr bool STAGE_A = sizeof(T) == 2 && !STATES;
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int N = STATES ? 0 : 1;  // buffers the states-only pass leaves out
  static constexpr int OFF_K = 0;
  static constexpr int OFF_VT = OFF_K + N * a16(128 * LDK * (int)sizeof(T));
  static constexpr int OFF_KP = OFF_VT + a16(DV * LDVT * (int)sizeof(T));
  static constexpr int OFF_QE = OFF_KP + N * a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_KHT = OFF_QE + N * a16(64 * LDK * (int)sizeof(T));
  static constexpr int OFF_ST = OFF_KHT + a16(D * LDKH * (int)sizeof(T));
  static constexpr int OFF_P = OFF_ST + N * a16(DV * LDST * (int)sizeof(T));
  static constexpr int OFF_A = OFF_P + N * a16(4 * 16 * LDP * (int)sizeof(T));
  static constexpr int A_BYTES = STAGE_A ? a16(4 * 16 * LDA * (int)sizeof(T)) : 0;
  static constexpr int OFF_TOT = OFF_A + A_BYTES;
  // wide-span totals: over the A staging when there is one (both are free in
  // the operand step), else a region of their own
  static constexpr int OFF_TOTC = STAGE_A ? OFF_A : OFF_TOT + a16(8 * D * 4);
  static constexpr int OFF_BEXP = OFF_TOT + a16(8 * D * 4) + (STAGE_A ? 0 : a16(8 * D * 4));
  static constexpr int OFF_SC = OFF_BEXP + a16(D * 4);          // [2][64]: alpha/den, 1/den
  static constexpr int OFF_META = OFF_SC + N * a16(2 * 64 * 4);
  // wide-span chunks: per query block, whether its own span needs the pairwise
  // diagonal (set in the operand step, read in the next score step; not in
  // the A staging the totals share, which the score step writes)
  static constexpr int OFF_WIDE = OFF_META + N * a16(16 * LDK * (int)sizeof(T));
  // the states-only pass: the chunk-start state in row-major order [D][LDSS],
  // staged for whole-row global stores
  static constexpr int LDSS = DV + PAD;
  static constexpr int OFF_SS = a16(OFF_WIDE + N * 16);
  static constexpr int TOTAL = OFF_SS + (STATES ? a16(D * LDSS * (int)sizeof(T)) : 0);
  static_assert(STATES || 64 * LDE * 4 <= OFF_KHT - OFF_KP, "beta fits over sKp and sQe");
  static_assert(!STAGE_A || 8 * D * 4 <= A_BYTES, "wide-span totals fit over the A staging");
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

// float: o += V^T A^T over one 16-key tile, with the B operand (A^T[s][t]
// for keys 4g..4g+3 of the tile, query m) straight from the registers of the
// MFMA that produced it: in step r, lane group g supplies key 4g + r, so the
// contraction pairs the same key on both operands.  vt points at
// V^T[j = 16ct + m][first key of the tile + 4g].  (bfloat16 scores are
// staged through LDS instead and use the 16x16x32 product.)
__device__ __forceinline__ f32x4 mma_tile_regs_f32(const float* vt, f32x4 ai, f32x4 o) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(vt);
#pragma unroll
  for (int r = 0; r < 4; ++r) o = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], ai[r], o, 0, 0, 0);
  return o;
}

// An int passed through an empty asm: values derived from it are computed
// where they are used instead of being hoisted out of the chunk loop (which
// would hold them in registers across the whole loop).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Largest chunk decay span (log2 units) taken by the factorised path: 2^92
// leaves a factor 2^36 of headroom below the float / bfloat16 maximum.
constexpr float kMaxSpanLog2 = 92.0f;

// Split sequences: below this log2 decay from a segment's start the state
// carried into the segment adds under 2^-128 of its size to an output (gates
// are at most one, so every later chunk decays further); the output
// correction stops at the first such chunk.
constexpr float kSegSkipLog2 = -128.0f;

// MODE: kPlain, kSeg (a segment of a split sequence) or kTrain (the full
// forward that also keeps the chunk-start states); STATES: the states-only pass.
enum { kPlain = 0, kSeg = 1, kTrain = 2 };
template <typename T, int D, int DV, bool STATES, bool LOGIT, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(STATES ? 4 : 2))) void lizard_fwd_kernel(FwdArgs a) {
  typedef FwdLayout<T, D, DV, STATES> Lay;
  constexpr bool SEG = MODE == kSeg;
  constexpr bool KEEP_STATES = STATES || MODE == kTrain;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int C = 64;
  constexpr int DPL = D / 64;                 // prep dims per lane; state row tiles per gate wavefront
  constexpr int EPV = 16 / sizeof(T);         // elements per 16-byte vector
  constexpr int QV = D / 4 / EPV;             // 16-byte vectors in a lane's k-quarter of a row
  constexpr int NF = D / 4 / M::KPL;          // MFMA steps over a D contraction
  constexpr int NCT = DV / 16;                // value column tiles
  constexpr int VC = 4 / sizeof(T);           // value columns per thread in the value load
  constexpr int VRW = DV / VC;                // threads across a value row
  constexpr int VR = 64 * VRW / 512;          // value rows per thread
  static_assert(VR == 4, "shape");

  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + Lay::OFF_K);
  T* sVt = reinterpret_cast<T*>(smem + Lay::OFF_VT);
  T* sKp = reinterpret_cast<T*>(smem + Lay::OFF_KP);
  T* sQe = reinterpret_cast<T*>(smem + Lay::OFF_QE);
  float* sBeta = reinterpret_cast<float*>(smem + Lay::OFF_KP);   // wide-span chunks only
  T* sKhT = reinterpret_cast<T*>(smem + Lay::OFF_KHT);
  T* sSt = reinterpret_cast<T*>(smem + Lay::OFF_ST);
  T* sP = reinterpret_cast<T*>(smem + Lay::OFF_P);
  float* sTot = reinterpret_cast<float*>(smem + Lay::OFF_TOT);
  T* sA = reinterpret_cast<T*>(smem + Lay::OFF_A);                // bfloat16 only
  float* sTotC = reinterpret_cast<float*>(smem + Lay::OFF_TOTC);  // wide-span chunks only
  int* sWide = reinterpret_cast<int*>(smem + Lay::OFF_WIDE);       // wide-span chunks only
  float* sBexp = reinterpret_cast<float*>(smem + Lay::OFF_BEXP);
  float* sSc = reinterpret_cast<float*>(smem + Lay::OFF_SC);
  T* sMeta = reinterpret_cast<T*>(smem + Lay::OFF_META);
  T* sSS = reinterpret_cast<T*>(smem + Lay::OFF_SS);               // states-only pass

  // ---- block -> (b*h, value slice, segment); the blocks of one head share an XCD ----
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int idx = x >> 3;
  const int split = idx % a.nsplit;
  const int seg = SEG ? (idx / a.nsplit) % a.nseg : 0;
  const int bh = (idx / (SEG ? a.nsplit * a.nseg : a.nsplit)) * 8 + xcd;
  if (bh >= a.BH) return;
  const int h = bh % a.H;
  const int j0 = split * DV;
  const int L = a.L;
  const int nc = (L + C - 1) / C;
  int c_lo = 0, c_hi = nc;
  if constexpr (SEG) {
    segment_chunks(seg, a.nseg, nc, c_lo, c_hi);
    if (c_lo >= c_hi) return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront 0..7: prep rows 8w..8w+7
  const int l = tid & 63;
  const int m_lane = l & 15;   // MFMA row / column within a tile
  const int g_lane = l >> 4;   // MFMA lane group
  const int vj = tid % VRW;    // value-load role: columns VC*vj.., rows VR*vs..
  const int vs = tid / VRW;

  const T* __restrict__ qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D + j0;
  const float* __restrict__ lgg = LOGIT ? nullptr : a.log_g + (size_t)bh * L * D;
  const T* __restrict__ xg = LOGIT ? reinterpret_cast<const T*>(a.gate_logit) + (size_t)bh * L * D : nullptr;
  T* __restrict__ yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D + j0;
  T* __restrict__ yag = a.y_anchor ? reinterpret_cast<T*>(a.y_anchor) + (size_t)bh * L * D + j0 : nullptr;
  float* __restrict__ lseg = (a.lse && split == 0) ? a.lse + (size_t)bh * L : nullptr;

  // ---- the key/value rings: the window of the first chunk c_lo reads the
  // ring positions of chunk c_lo - 1 (key ring half (c_lo - 1) & 1, value
  // ring slot (c_lo - 1) mod 3), which hold, in their last nh entries, the
  // previous chunk of a split sequence or the halo tokens of a continued
  // sequence; everything else is zero ----
  {
    const int cp = c_lo - 1;                       // -1 for the first segment
    const int ph = (cp & 1) * 64, ps = ((cp % 3 + 3) % 3) * 64;
    const int nh = c_lo > 0 ? 64 : a.halo;
    const T* khp = nullptr;
    const T* vhp = nullptr;
    if (c_lo > 0) {
      khp = kg + (size_t)(c_lo * C - 64) * D;
      vhp = vg + (size_t)(c_lo * C - 64) * D;
    } else if (a.halo > 0) {
      khp = reinterpret_cast<const T*>(a.k_halo) + (size_t)bh * a.halo * D;
      vhp = reinterpret_cast<const T*>(a.v_halo) + (size_t)bh * a.halo * D + j0;
    }
    const int hb = ph + 64 - nh;                   // first filled key ring row
    const int vb = ps + 64 - nh;                   // first filled value ring column
    if constexpr (!STATES) {                       // (the states-only pass reads neither ring across chunks)
      for (int i = tid; i < 128 * Lay::LDK; i += 512) {
        const int row = i / Lay::LDK, col = i % Lay::LDK;
        sK[i] = row >= hb && row < ph + 64 && col < D ? khp[(size_t)(row - hb) * D + col] : from_f32<T>(0.f);
      }
      for (int i = tid; i < DV * Lay::LDVT; i += 512) {
        const int j = i / Lay::LDVT, col = i % Lay::LDVT;
        sVt[i] = col >= vb && col < ps + 64 ? vhp[(size_t)(col - vb) * D + j] : from_f32<T>(0.f);
      }
    }
  }
  // ---- sink keys (rows >= n_meta zero), resident in LDS throughout; the
  // window weights' last 16 slots (the sixth key tile of the V^T P^T
  // product, which the five logit tiles never reach) stay zero ----
  if constexpr (!STATES) {
    for (int i = tid; i < 16 * D; i += 512) {
      const int r = i / D, cidx = i % D;
      sMeta[r * Lay::LDK + cidx] =
          r < a.n_meta ? reinterpret_cast<const T*>(a.meta)[((size_t)h * a.n_meta + r) * D + cidx] : from_f32<T>(0.f);
    }
    for (int i = tid; i < 64 * 16; i += 512) sP[(i / 16) * Lay::LDP + 80 + i % 16] = from_f32<T>(0.f);
  }

  // Each (role, query block) runs its own copy of the chunk loop: role 0 the
  // softmax wavefronts, role 1 the gate wavefronts (in the states-only mode
  // role 0 only prepares operands and role 1 carries the state).  Separate
  // loops keep one role's registers and outstanding loads out of the other's
  // (a shared loop would make the compiler hold both roles' registers and
  // wait for every load in flight); the barrier sequence is the same in all.
  auto run = [&](auto Rc, auto Ic) __attribute__((always_inline)) {
    constexpr bool GATE = decltype(Rc)::value == 1;
    constexpr int QB = decltype(Ic)::value;
    // ---- gate wavefronts: state rows 16*(DPL*I + rt) + 4g + r, cols 16ct + m ----
    const int I = QB;
    f32x4 acc[DPL][NCT];
  #pragma unroll
    for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = zero4();
    if constexpr (GATE && !STATES) {
      if (a.state_in && seg == 0) {
        // a continued sequence: the state before its first token
        const float* si = a.state_in + (size_t)bh * D * D + j0;
  #pragma unroll
        for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[rt][ct][r] = si[(size_t)(16 * (DPL * I + rt) + 4 * g_lane + r) * D + 16 * ct + m_lane];
        // consume the loads here: otherwise the accumulators enter the chunk
        // loop with loads in flight on one path only, and their first use in
        // every chunk would wait for all loads in flight
  #pragma unroll
        for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
          for (int ct = 0; ct < NCT; ++ct) asm volatile("" : "+v"(acc[rt][ct]));
      }
    }

    // ---- per-chunk global data (prefetched ahead, kept as raw bits) ----
    float lgA[8][DPL];    // prep rows 8w+rr, dims DPL*l + dd (from xA when the gates come as logits)
    uint32_t xA[8];       // gate logits of those rows: DPL elements packed in 32 bits
    float loc[8][DPL];    // their prefix inside the wavefront's 8 rows
    // the states-only pass with log-gates keeps the gates instead and forms
    // the prefix again where the operands use it (the same sums in the same
    // order): holding both had spilled registers at four wavefronts per SIMD
    constexpr bool REPREFIX = STATES && !LOGIT;
    uint32_t kA[8];       // the same rows' keys: DPL elements packed in 32 bits
    uint32_t qA[8];       // ... and queries
    uint32_t vA[VR];      // values: rows VR*vs + rr, columns VC*vj.. packed in 32 bits
    uint4 qraw[QV];       // softmax wavefronts: raw q of row 16I + m, the lane's k-quarter
    f32x4 og[NCT];        // gate wavefronts: gated output of the block, carried over a barrier
    float rcum[DPL] = {};  // split sequences: log2-gate sum from the segment start (one gate wavefront)
    int live_end = c_hi;   // ... and the first chunk whose decay from the segment start is below the cut

    auto load_rows = [&](int c, bool full) __attribute__((always_inline)) {
      const int t0 = c * C;
      const int tid = opaque(threadIdx.x);
      const int l = tid & 63;
      const int vj = tid % VRW, vs = tid / VRW;
      {
        const int tb = t0 + 8 * w;
        const float* lp = lgg + (size_t)tb * D + DPL * l;
        const T* xp = xg + (size_t)tb * D + DPL * l;
        const T* kp = kg + (size_t)tb * D + DPL * l;
        const T* qp = qg + (size_t)tb * D + DPL * l;
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const bool ok = full || tb + rr < L;
          const ptrdiff_t ro = (ptrdiff_t)(ok ? rr : -tb) * D;   // row 0 of the slice when out of range
          float lv[DPL];
          uint32_t xv = 0;
          if constexpr (LOGIT) {
            if constexpr (DPL * sizeof(T) == 4) xv = *reinterpret_cast<const uint32_t*>(xp + ro);
            else xv = *reinterpret_cast<const uint16_t*>(xp + ro);
          } else if constexpr (DPL == 2) {
            const float2 f = *reinterpret_cast<const float2*>(lp + ro);
            lv[0] = f.x;
            lv[1] = f.y;
          } else {
            lv[0] = lp[ro];
          }
          uint32_t kv, qv = 0u;   // the states-only pass needs no queries
          if constexpr (DPL * sizeof(T) == 4) {
            kv = *reinterpret_cast<const uint32_t*>(kp + ro);
            if constexpr (!STATES) qv = *reinterpret_cast<const uint32_t*>(qp + ro);
          } else {
            kv = *reinterpret_cast<const uint16_t*>(kp + ro);
            if constexpr (!STATES) qv = *reinterpret_cast<const uint16_t*>(qp + ro);
          }
          if constexpr (LOGIT) {
            // past L: a logit of +inf, a gate of one (as log_g = 0 below)
            constexpr uint32_t kInf = sizeof(T) == 4 ? 0x7f800000u : 0x7f807f80u;
            xA[rr] = ok ? xv : kInf;
          } else {
  #pragma unroll
            for (int dd = 0; dd < DPL; ++dd) lgA[rr][dd] = ok ? lv[dd] : 0.f;
          }
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
          const uint32_t u = *reinterpret_cast<const uint32_t*>(vp + (ptrdiff_t)(ok ? rr : -tb) * D);
          vA[rr] = ok ? u : 0u;
        }
      }
    };
    // a uniform branch: full chunks load without per-row guards
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
      if ((c + 1) * C <= L) load_rows(c, true);
      else load_rows(c, false);
    };
    auto load_q = [&](int c) __attribute__((always_inline)) {
      const int l = opaque(threadIdx.x) & 63;
      const int tq = c * C + 16 * I + (l & 15);
      const bool ok = tq < L;
      const T* qp = qg + (size_t)(ok ? tq : 0) * D + (l >> 4) * (D / 4);
  #pragma unroll
      for (int e = 0; e < QV; ++e) qraw[e] = ok ? ld16(qp + e * EPV) : make_uint4(0, 0, 0, 0);
    };
    // element dd of a packed 32-bit word, as float
    auto elem32 = [&](uint32_t u, int dd) __attribute__((always_inline)) -> float {
      if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, u);
      else return __builtin_bit_cast(float, dd == 0 ? (u << 16) : (u & 0xffff0000u));
    };
    // the natural-log gate of prep row rr, dim dd: loaded, or formed from
    // the logit by the prefix step; the states-only pass forms it where it is
    // used instead (the logits take half the registers of the gates, which
    // that pass, at four wavefronts per SIMD, is short of)
    auto lg_of = [&](int rr, int dd) __attribute__((always_inline)) -> float {
      if constexpr (LOGIT && STATES) return log_sigmoid(elem32(xA[rr], dd));
      else return lgA[rr][dd];
    };

    // ---- prefix sums inside this wavefront's 8 rows (natural-log units; exact
    // for the factorised path, where no single gate is small enough for the
    // 2^-100 floor of the wide-span path) ----
    auto prefix_part = [&]() __attribute__((always_inline)) {
      const int l = opaque(threadIdx.x) & 63;
      if constexpr (LOGIT && !STATES) {
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr)
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd) lgA[rr][dd] = log_sigmoid(elem32(xA[rr], dd));
      }
      float tot[DPL];
  #pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        float run = 0.f;
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          run += lg_of(rr, dd);
          if constexpr (!REPREFIX) loc[rr][dd] = run;
        }
        tot[dd] = run;
      }
      if constexpr (DPL == 2) *reinterpret_cast<float2*>(sTot + w * D + 2 * l) = make_float2(tot[0], tot[1]);
      else sTot[w * D + l] = tot[0];
    };

    // offset of this wavefront's rows (sum of the earlier wavefronts' totals)
    // and the chunk total, from the 8 partial totals in tp
    auto offsets = [&](const float* tp, float* off, float* Bt) __attribute__((always_inline)) {
      const int l = opaque(threadIdx.x) & 63;
      float tv[8][DPL];
  #pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        if constexpr (DPL == 2) {
          const float2 f = *reinterpret_cast<const float2*>(tp + ww * D + 2 * l);
          tv[ww][0] = f.x;
          tv[ww][1] = f.y;
        } else {
          tv[ww][0] = tp[ww * D + l];
        }
      }
  #pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        float run = 0.f, o = 0.f;
  #pragma unroll
        for (int ww = 0; ww < 8; ++ww) {
          o = ww == w ? run : o;
          run += tv[ww][dd];
        }
        off[dd] = o;
        Bt[dd] = run;
      }
    };

    // ---- chunk cc's operands into LDS (decay factors, Qe, Kp, Kh, keys,
    // values, the chunk-start state); returns whether it takes the pairwise path
    auto operand_part = [&](int cc) __attribute__((always_inline)) -> bool {
      const int kc = (cc & 1) * 64;       // key ring half
      const int vc = (cc % 3) * 64;       // value ring slot
      const int tid = opaque(threadIdx.x);
      const int l = tid & 63, m_lane = l & 15, g_lane = l >> 4;
      const int vj = tid % VRW, vs = tid / VRW;
      float Bt[DPL], off[DPL];
      offsets(sTot, off, Bt);
      bool wide = false, wider = false;
  #pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        wide |= -Bt[dd] * kLog2e > kMaxSpanLog2;
        wider |= -Bt[dd] * kLog2e > 2.f * kMaxSpanLog2;
      }
      // every wavefront covers all D dims, so these ballots are the chunk's
      // decision.  Spans up to twice the limit take the factorised path with
      // each dimension's reference point moved from the chunk start to half
      // its total r = B/2: then Qe = q 2^{beta - r} and Kp = k 2^{r - beta}
      // are both within 2^{span/2}, and the readout takes 2^r into the state
      // copy.
      const bool pairwise = __any(wider);
      const bool midref = !pairwise && __any(wide);
      float kh[DPL][8];
      float eB[DPL];
      float rexp[DPL];    // 2^r (one unless midref)
      if (!pairwise) {
        float ehr[DPL];   // 2^{B - r}: Kh = Kp 2^{B - r}
        if (!midref) {
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            eB[dd] = exp_2(Bt[dd] * kLog2e);
            ehr[dd] = eB[dd];
            off[dd] *= kLog2e;
          }
        } else {
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            const float B2 = Bt[dd] * kLog2e;
            const float r = 0.5f * B2;
            eB[dd] = exp_2(B2);
            ehr[dd] = exp_2(B2 - r);
            rexp[dd] = exp_2(r);
            off[dd] = fmaf(off[dd], kLog2e, -r);
          }
        }
        float lrun[DPL] = {};   // the prefix formed again (REPREFIX)
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int s = 8 * w + rr;
          float qe[DPL], kp[DPL];
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            if constexpr (REPREFIX) lrun[dd] += lgA[rr][dd];
            const float beta = fmaf(REPREFIX ? lrun[dd] : loc[rr][dd], kLog2e, off[dd]);
            kp[dd] = elem32(kA[rr], dd) * exp_2(-beta);
            kh[dd][rr] = kp[dd] * ehr[dd];
            qe[dd] = STATES ? 0.f : elem32(qA[rr], dd) * exp_2(beta);
          }
          // (the states-only pass needs only Kh)
          if constexpr (STATES) {
          } else if constexpr (DPL == 2) {
            *reinterpret_cast<bf16x2*>(sQe + s * Lay::LDK + 2 * l) = bf16x2{static_cast<bf16>(qe[0]), static_cast<bf16>(qe[1])};
            *reinterpret_cast<bf16x2*>(sKp + s * Lay::LDK + 2 * l) = bf16x2{static_cast<bf16>(kp[0]), static_cast<bf16>(kp[1])};
          } else {
            sQe[s * Lay::LDK + l] = from_f32<T>(qe[0]);
            sKp[s * Lay::LDK + l] = from_f32<T>(kp[0]);
          }
        }
      } else {
        // wide span: log2 prefixes with every gate floored at 2^-100, so that
        // differences of prefixes keep float precision (a uniform branch)
        float locc[8][DPL], totc[DPL];
  #pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          float run = 0.f;
  #pragma unroll
          for (int rr = 0; rr < 8; ++rr) {
            run += log2_gate(lg_of(rr, dd));
            locc[rr][dd] = run;
          }
          totc[dd] = run;
        }
  #pragma unroll
        for (int dd = 0; dd < DPL; ++dd) sTotC[w * D + DPL * l + dd] = totc[dd];
        __syncthreads();
        offsets(sTotC, off, Bt);
        if (!STATES && w < 4) {
          // query block w's own span per dim: minus its two 8-row partial totals
          bool wb = false;
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd)
            wb |= -(sTotC[2 * w * D + DPL * l + dd] + sTotC[(2 * w + 1) * D + DPL * l + dd]) > kMaxSpanLog2;
          const bool any = __any(wb);
          if (l == 0) sWide[w] = any ? 1 : 0;
        }
  #pragma unroll
        for (int dd = 0; dd < DPL; ++dd) eB[dd] = exp_2(Bt[dd]);
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int s = 8 * w + rr;
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            const float beta = off[dd] + locc[rr][dd];
            kh[dd][rr] = elem32(kA[rr], dd) * exp_2(Bt[dd] - beta);
            if constexpr (!STATES) sBeta[s * Lay::LDE + DPL * l + dd] = beta;
          }
        }
      }
  #pragma unroll
      for (int dd = 0; dd < DPL; ++dd) {
        store_pack<T, 8>(sKhT + (DPL * l + dd) * Lay::LDKH + 8 * w, kh[dd]);
        if (w == 0) sBexp[DPL * l + dd] = eB[dd];
      }
      if constexpr (SEG && GATE && QB == 0) {
        // a split sequence: the decay from the segment start to this chunk's
        // start, and its running sum (the exponents of eB)
        float mx = rcum[0];
  #pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          if (split == 0) a.chunk_cum[((size_t)bh * nc + cc) * D + DPL * l + dd] = rcum[dd];
          mx = fmaxf(mx, rcum[dd]);
          rcum[dd] += pairwise ? Bt[dd] : Bt[dd] * kLog2e;
        }
        // this wavefront's lanes cover all D dimensions: a uniform value
        if (live_end == c_hi && wave_max(mx) < kSegSkipLog2) live_end = cc;
      }
      // raw keys into the ring (for the window; not in the states-only pass)
      if constexpr (!STATES) {
  #pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          T* krp = sK + (kc + 8 * w + rr) * Lay::LDK + DPL * l;
          if constexpr (DPL * sizeof(T) == 4) *reinterpret_cast<uint32_t*>(krp) = kA[rr];
          else krp[0] = from_f32<T>(elem32(kA[rr], 0));
        }
      }
      // values, transposed into their ring slot: sVt[j][vc + s], 4 tokens per write
      if constexpr (sizeof(T) == 2) {
        // columns 2vj and 2vj+1 of 4 consecutive rows: regroup the 16-bit halves
        const uint2 lo = make_uint2(__builtin_amdgcn_perm(vA[1], vA[0], 0x05040100u),
                                    __builtin_amdgcn_perm(vA[3], vA[2], 0x05040100u));
        const uint2 hi = make_uint2(__builtin_amdgcn_perm(vA[1], vA[0], 0x07060302u),
                                    __builtin_amdgcn_perm(vA[3], vA[2], 0x07060302u));
        *reinterpret_cast<uint2*>(sVt + (2 * vj) * Lay::LDVT + vc + VR * vs) = lo;
        *reinterpret_cast<uint2*>(sVt + (2 * vj + 1) * Lay::LDVT + vc + VR * vs) = hi;
      } else {
        *reinterpret_cast<uint4*>(sVt + vj * Lay::LDVT + vc + VR * vs) = make_uint4(vA[0], vA[1], vA[2], vA[3]);
      }
      if constexpr (GATE) {
        if constexpr (!STATES) {
          // S_cc (rounded to the element type) for the readout: sSt[j][i], 4 rows i per write;
          // row i scaled by 2^{r_i} when the reference point moved (2^r of
          // dimension i sits in lane i / DPL)
          if (!midref) {
  #pragma unroll
            for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
              for (int ct = 0; ct < NCT; ++ct) {
                const float sv[4] = {acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]};
                store_pack<T, 4>(sSt + (16 * ct + m_lane) * Lay::LDST + 16 * (DPL * I + rt) + 4 * g_lane, sv);
              }
          } else {
            float rs[DPL][4];
  #pragma unroll
            for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int i = 16 * (DPL * I + rt) + 4 * g_lane + r;
                rs[rt][r] = __shfl(rexp[r % DPL], i / DPL, 64);
              }
  #pragma unroll
            for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
              for (int ct = 0; ct < NCT; ++ct) {
                const float sv[4] = {acc[rt][ct][0] * rs[rt][0], acc[rt][ct][1] * rs[rt][1],
                                     acc[rt][ct][2] * rs[rt][2], acc[rt][ct][3] * rs[rt][3]};
                store_pack<T, 4>(sSt + (16 * ct + m_lane) * Lay::LDST + 16 * (DPL * I + rt) + 4 * g_lane, sv);
              }
          }
        }
        if constexpr (STATES) {
          // chunk-start state for the backward pass: S_cc[i][j] into LDS,
          // row-major; the other wavefronts store whole rows of it during
          // the next interval
  #pragma unroll
          for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
  #pragma unroll
              for (int r = 0; r < 4; ++r)
                sSS[(16 * (DPL * I + rt) + 4 * g_lane + r) * Lay::LDSS + 16 * ct + m_lane] = from_f32<T>(acc[rt][ct][r]);
        } else if constexpr (KEEP_STATES) {
          // chunk-start state S_cc[i][j], row-major (a training forward that
          // keeps them for the backward pass)
          const int ncs = (L + C - 1) / C;
          T* sg = reinterpret_cast<T*>(a.states) + ((size_t)bh * ncs + cc) * D * D + j0;
  #pragma unroll
          for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
  #pragma unroll
              for (int r = 0; r < 4; ++r)
                sg[(size_t)(16 * (DPL * I + rt) + 4 * g_lane + r) * D + 16 * ct + m_lane] = from_f32<T>(acc[rt][ct][r]);
        }
      }
      return pairwise;
    };

    // ---- state carry over chunk c: S = 2^B * S + Kh^T V (gate wavefronts) ----
    auto carry = [&](int vc, int m, int g) __attribute__((always_inline)) {
  #pragma unroll
      for (int rt = 0; rt < DPL; ++rt) {
        const int ib = 16 * (DPL * I + rt);
        float dec[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) dec[r] = sBexp[ib + 4 * g + r];
        const T* kp = sKhT + (ib + m) * Lay::LDKH + g * 16;
  #pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 s = acc[rt][ct];
  #pragma unroll
          for (int r = 0; r < 4; ++r) s[r] *= dec[r];
          const T* vp = sVt + (16 * ct + m) * Lay::LDVT + vc + g * 16;
  #pragma unroll
          for (int e = 0; e < 16 / M::KPL; ++e) s = M::mma(M::load(kp + e * M::KPL), M::load(vp + e * M::KPL), s);
          acc[rt][ct] = s;
        }
      }
    };

    bool pw = false;                      // pairwise path for the chunk about to be processed
    if (c_hi > c_lo) {
      load_chunk(c_lo);
      if constexpr (!GATE && !STATES) load_q(c_lo);
      prefix_part();
    }
    __syncthreads();
    if (c_hi > c_lo) {
      pw = operand_part(c_lo);
      if (c_hi > c_lo + 1) load_chunk(c_lo + 1);
    }
    __syncthreads();

    for (int c = c_lo; c < c_hi; ++c) {
      const int t0 = c * C;
      const int kcur = (c & 1) * 64;      // key ring half of this chunk
      const int kprv = 64 - kcur;         // ... and of the previous chunk
      const int vcur = (c % 3) * 64;      // value ring slot of this chunk
      const int vprv = ((c + 2) % 3) * 64;   // ... and of the previous chunk
      const bool pairwise = pw;

      // ================= interval 1, softmax wavefront: weights of block QB ====
      auto softmax_part = [&](auto Ic) __attribute__((always_inline)) {
        constexpr int QB = decltype(Ic)::value;
        constexpr int U0 = 16 * QB;          // first window key (of [prev; cur]) staged
        // Lane indices laundered through an empty asm: addresses derived from
        // them are recomputed per chunk instead of being hoisted out of the
        // chunk loop by every instance (which would exhaust registers).
        int m = m_lane, g = g_lane;
        asm volatile("" : "+v"(m), "+v"(g));
        const int tme = t0 + 16 * QB + m;
        frag qf[NF];
  #pragma unroll
        for (int e = 0; e < NF; ++e) qf[e] = frag_at<T>(qraw, e);
        // the next chunk's queries (qf holds this chunk's).  Issued on every
        // chunk (the last one reloads itself) so that the number of memory
        // operations between a load and its use is the same on every path:
        // the wait for it then counts, instead of draining all loads in flight.
        load_q(c + 1 < c_hi ? c + 1 : c);

        // anchor logits Z^T[u][t] over the 5 window tiles kt (keys u in
        // [U0+16kt, U0+16kt+16) of [prev; cur]: the block's queries reach
        // back at most 63 keys from [U0+64, U0+80)); every tile is computed,
        // keys outside the window are masked below (branch-free: a skipped
        // tile would make the compiler copy the logit arrays between paths)
        f32x4 z[5];
  #pragma unroll
        for (int kt = 0; kt < 5; ++kt) {
          const T* kp = sK + ((U0 + 16 * kt + kprv + m) & 127) * Lay::LDK + g * (D / 4);
          z[kt] = zero4();
  #pragma unroll
          for (int e = 0; e < NF; ++e) z[kt] = M::mma(M::load(kp + e * M::KPL), qf[e], z[kt]);
        }
        f32x4 zs = zero4();
  #pragma unroll
        for (int e = 0; e < NF; ++e) zs = M::mma(M::load(sMeta + m * Lay::LDK + g * (D / 4) + e * M::KPL), qf[e], zs);

        // Softmax: maxima on raw logits (the scale is positive), scale folded
        // into the exponent: P = 2^{z * scale*log2e - max}.
        float mr = -__builtin_huge_valf();
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          zs[r] = 4 * g + r < a.n_meta ? zs[r] : -INFINITY;
          mr = fmaxf(mr, zs[r]);
        }
        // key valid iff 0 <= t - s < lim; in the first chunk also s >= -halo
        // (t - s <= t + halo: no keys before the sequence or its halo)
        const int hl1 = a.halo + 1;
        const int lim = (c == 0 && 16 * QB + m + hl1 < a.window) ? 16 * QB + m + hl1 : a.window;
        const int lim_lo = (c == 0 && 16 * QB + hl1 < a.window) ? 16 * QB + hl1 : a.window;   // over the block
        const int dl = m - 4 * g;            // t - s = K_kt + dl - r
  #pragma unroll
        for (int kt = 0; kt < 5; ++kt) {
          // t - s over the tile spans [K_kt - 15, K_kt + 15]: tiles inside the band skip the mask
          constexpr int K0 = 16 * QB + 64 - U0;
          const int Kt = K0 - 16 * kt;
          if (!(Kt - 15 >= 0 && Kt + 15 < lim_lo)) {
  #pragma unroll
            for (int r = 0; r < 4; ++r) z[kt][r] = (unsigned)(Kt + dl - r) < (unsigned)lim ? z[kt][r] : -INFINITY;
          }
  #pragma unroll
          for (int r = 0; r < 4; ++r) mr = fmaxf(mr, z[kt][r]);
        }
        mr = xgroup_max(mr);                 // finite: the query's own key is always valid
        const float mref = mr * a.scale_log2;
        float sr = 0.f;
  #pragma unroll
        for (int r = 0; r < 4; ++r) sr += exp_2(fmaf(zs[r], a.scale_log2, -mref));
  #pragma unroll
        for (int kt = 0; kt < 5; ++kt) {
          float p[4];
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = exp_2(fmaf(z[kt][r], a.scale_log2, -mref));   // 2^-inf = 0 for masked keys
            sr += p[r];
          }
          store_pack<T, 4>(sP + (16 * QB + m) * Lay::LDP + 16 * kt + 4 * g, p);
        }
        const float den = xgroup_sum(sr);
        if (g == 0) {
          const float inv = 1.0f / den;
          sSc[16 * QB + m] = a.alpha * inv;
          sSc[64 + 16 * QB + m] = inv;
          if (lseg && tme < L) lseg[tme] = (mref + __log2f(den)) * kLn2;
        }
      };

      // ========== interval 1, gate wavefront: gated output, state carry ========
      auto gate_part = [&](auto Ic) __attribute__((always_inline)) {
        constexpr int QB = decltype(Ic)::value;
        int m = m_lane, g = g_lane;
        asm volatile("" : "+v"(m), "+v"(g));
        const int tme = t0 + 16 * QB + m;

        // Qe = q * 2^beta of this lane's query (B operand)
        frag qe[NF];
        uint4 raw[QV];        // wide span: the raw query, this lane's k-quarter
        if (!pairwise) {
          const T* ep = sQe + (16 * QB + m) * Lay::LDK + g * (D / 4);
  #pragma unroll
          for (int e = 0; e < NF; ++e) qe[e] = M::load(ep + e * M::KPL);
        } else {
          const T* qp = qg + (size_t)(tme < L ? tme : 0) * D + g * (D / 4);
  #pragma unroll
          for (int e = 0; e < QV; ++e) raw[e] = tme < L ? ld16(qp + e * EPV) : make_uint4(0, 0, 0, 0);
          const float* bp = sBeta + (16 * QB + m) * Lay::LDE + g * (D / 4);
  #pragma unroll
          for (int e = 0; e < NF; ++e) {
            float tmp[M::KPL];
  #pragma unroll
            for (int u = 0; u < M::KPL; ++u) tmp[u] = elem_f32<T>(raw, e * M::KPL + u) * exp_2(bp[e * M::KPL + u]);
            qe[e] = M::pack(tmp);
          }
        }

        // ---- intra-chunk gated scores A^T[s][t], key blocks J <= QB ----
        f32x4 ai[QB + 1];
        if (!pairwise) {
  #pragma unroll
          for (int J = 0; J <= QB; ++J) {
            ai[J] = zero4();
            const T* kp = sKp + (16 * J + m) * Lay::LDK + g * (D / 4);
  #pragma unroll
            for (int e = 0; e < NF; ++e) ai[J] = M::mma(M::load(kp + e * M::KPL), qe[e], ai[J]);
          }
        } else {
          // a decay span too wide to factorise over the chunk: factorised
          // per 16-key block J at a reference point b instead, A^T[s][t] =
          // (k_s 2^{beta_b - beta_s}) . (q_t 2^{beta_t - beta_b}).  For J < QB,
          // b = the last key of J, which lies between every key of J and every
          // query of QB, so both factors are <= 1.
          const float* bt = sBeta + (16 * QB + m) * Lay::LDE + g * (D / 4);
          auto factored = [&](int J, const float* bb) __attribute__((always_inline)) -> f32x4 {
            f32x4 acc_j = zero4();
            const float* bs = sBeta + (16 * J + m) * Lay::LDE + g * (D / 4);
            const T* kr = sK + (kcur + 16 * J + m) * Lay::LDK + g * (D / 4);
  #pragma unroll
            for (int e = 0; e < NF; ++e) {
              float tq[M::KPL], tk[M::KPL];
  #pragma unroll
              for (int u = 0; u < M::KPL; ++u) {
                const int x = e * M::KPL + u;
                const float rb = bb ? bb[x] : 0.f;
                tq[u] = elem_f32<T>(raw, x) * exp_2(bt[x] - rb);
                tk[u] = to_f32(kr[x]) * exp_2(rb - bs[x]);
              }
              acc_j = M::mma(M::pack(tk), M::pack(tq), acc_j);
              __builtin_amdgcn_sched_barrier(0);   // one k-step's operands live at a time
            }
            return acc_j;
          };
  #pragma unroll
          for (int J = 0; J < QB; ++J) ai[J] = factored(J, sBeta + (16 * J + 15) * Lay::LDE + g * (D / 4));
          // the diagonal block: factorised at the block start a while the
          // block's own span stays within the factorisable range (then
          // 2^{beta_a - beta_s} <= 2^span), else every pair (t, s) in fp32,
          // each lane over its k-quarter, summed across the quarters
          // (the block's span, as the operand step found it)
          if (sWide[QB] == 0) {
            ai[QB] = factored(QB, QB > 0 ? sBeta + (16 * QB - 1) * Lay::LDE + g * (D / 4) : nullptr);
          } else {
            ai[QB] = zero4();
  #pragma unroll 1
            for (int s4 = 0; s4 < 4; ++s4) {
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int s16 = 4 * s4 + r;
                const T* kr = sK + (kcur + 16 * QB + s16) * Lay::LDK + g * (D / 4);
                const float* bs = sBeta + (16 * QB + s16) * Lay::LDE + g * (D / 4);
                float sum = 0.f;
  #pragma unroll
                for (int x = 0; x < D / 4; ++x)
                  sum = fmaf(elem_f32<T>(raw, x) * to_f32(kr[x]), exp_2(fminf(bt[x] - bs[x], 0.f)), sum);
                sum = xgroup_sum(sum);
                ai[QB][r] = s4 == g ? sum : ai[QB][r];     // lane group g keeps keys 4g .. 4g + 3
              }
            }
          }
        }
  #pragma unroll
        for (int r = 0; r < 4; ++r) ai[QB][r] = 4 * g + r <= m ? ai[QB][r] : 0.f;

        if constexpr (Lay::STAGE_A) {
          // A[t][s] of this block into its own staging rows (keys of blocks
          // J > QB are zero), read back by this wavefront only
  #pragma unroll
          for (int J = 0; J < 4; ++J) {
            float v4[4] = {0.f, 0.f, 0.f, 0.f};
            if (J <= QB) {
  #pragma unroll
              for (int r = 0; r < 4; ++r) v4[r] = ai[J < QB + 1 ? J : 0][r];
            }
            store_pack<T, 4>(sA + (16 * QB + m) * Lay::LDA + 16 * J + 4 * g, v4);
          }
          wave_lds_sync();
        }

        // ---- gated output O^T[j][t] = S_c^T Qe^T + V^T A^T ----
  #pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 o = zero4();
          const T* sp = sSt + (16 * ct + m) * Lay::LDST + g * (D / 4);
  #pragma unroll
          for (int e = 0; e < NF; ++e) o = M::mma(M::load(sp + e * M::KPL), qe[e], o);
          if constexpr (Lay::STAGE_A) {
            const T* vp = sVt + (16 * ct + m) * Lay::LDVT + vcur + g * 16;
            const T* ap = sA + (16 * QB + m) * Lay::LDA + g * 16;
  #pragma unroll
            for (int e = 0; e < 16 / M::KPL; ++e) o = M::mma(M::load(vp + e * M::KPL), M::load(ap + e * M::KPL), o);
          } else {
            const float* vp = reinterpret_cast<const float*>(sVt) + (16 * ct + m) * Lay::LDVT + vcur + 4 * g;
  #pragma unroll
            for (int J = 0; J <= QB; ++J) o = mma_tile_regs_f32(vp + 16 * J, ai[J], o);
          }
          og[ct] = o;
        }
        carry(vcur, m, g);
      };

      // ========== interval 2, gate wavefront: anchor product and output =======
      auto output_part = [&](auto Ic) __attribute__((always_inline)) {
        constexpr int QB = decltype(Ic)::value;
        constexpr int U0 = 16 * QB;
        int m = m_lane, g = g_lane;
        asm volatile("" : "+v"(m), "+v"(g));
        const int tme = t0 + 16 * QB + m;
        const float sc = sSc[16 * QB + m];
        const float inv = sSc[64 + 16 * QB + m];
        const T* pp = sP + (16 * QB + m) * Lay::LDP + g * 24;
        // V^T column of window key u of [prev; cur]: the previous slot is
        // followed by the current one in the 3-slot ring
        int col[24 / M::KPL];
  #pragma unroll
        for (int e = 0; e < 24 / M::KPL; ++e) {
          const unsigned v = vprv + U0 + g * 24 + e * M::KPL;
          col[e] = (int)min(v, v - 192u);
        }
        // all column tiles first (independent MFMA chains in one block), then
        // the stores under one condition
        f32x4 oa[NCT];
  #pragma unroll
        for (int ct = 0; ct < NCT; ++ct) oa[ct] = zero4();
  #pragma unroll
        for (int e = 0; e < 24 / M::KPL; ++e) {
          const typename M::frag pf = M::load(pp + e * M::KPL);
  #pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            oa[ct] = M::mma(M::load(sVt + (16 * ct + m) * Lay::LDVT + col[e]), pf, oa[ct]);
        }
        if (tme < L) {
  #pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 o = oa[ct];
            const float v4[4] = {fmaf(sc, o[0], og[ct][0]), fmaf(sc, o[1], og[ct][1]),
                                 fmaf(sc, o[2], og[ct][2]), fmaf(sc, o[3], og[ct][3])};
            store_pack<T, 4>(yg + (size_t)tme * D + 16 * ct + 4 * g, v4);
          }
          if (yag) {
  #pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              const f32x4 o = oa[ct];
              const float a4[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
              store_pack<T, 4>(yag + (size_t)tme * D + 16 * ct + 4 * g, a4);
            }
          }
        }
      };

      // ---- interval 1 ----
      if constexpr (STATES) {
        if constexpr (GATE) {
          carry(vcur, m_lane, g_lane);
        } else {
          // S_c (staged by the gate wavefronts) to memory: 16-byte pieces of
          // whole rows, threads 0..255
          constexpr int VPR = DV / EPV;
          const int tq = opaque(threadIdx.x);
          T* sg = reinterpret_cast<T*>(a.states) + ((size_t)bh * nc + c) * D * D + j0;
          static_assert(D * VPR % 256 == 0, "whole passes of threads 0..255");
  #pragma unroll
          for (int it = 0; it < D * VPR / 256; ++it) {
            const int v = tq + 256 * it;
            const int i = v / VPR, col = (v % VPR) * EPV;
            *reinterpret_cast<uint4*>(sg + (size_t)i * D + col) = *reinterpret_cast<const uint4*>(sSS + i * Lay::LDSS + col);
          }
        }
      } else if constexpr (GATE) {
        gate_part(Ic);
      } else {
        softmax_part(Ic);
      }
      if (c + 1 < c_hi) prefix_part();
      __syncthreads();

      // ---- interval 2 ----
      if constexpr (GATE && !STATES) output_part(Ic);
      if (c + 1 < c_hi) pw = operand_part(c + 1);
      // chunk c+2 (clamped: issued on every chunk for the same reason as load_q)
      load_chunk(c + 2 < c_hi ? c + 2 : c_hi - 1);
      __syncthreads();
    }

    if constexpr (SEG) {
      if constexpr (GATE) {
        // a split sequence: this segment's final state (from a zero state,
        // except the first segment) and its log2-gate total, for the scan
        float* so = a.seg_state + ((size_t)bh * a.nseg + seg) * D * D;
  #pragma unroll
        for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              so[(size_t)(16 * (DPL * I + rt) + 4 * g_lane + r) * D + j0 + 16 * ct + m_lane] = acc[rt][ct][r];
        if constexpr (QB == 0) {
          const int l = threadIdx.x & 63;
  #pragma unroll
          for (int dd = 0; dd < DPL; ++dd)
            if (split == 0) a.seg_total[((size_t)bh * a.nseg + seg) * D + DPL * l + dd] = rcum[dd];
          if (split == 0 && l == 0) a.seg_live[(size_t)bh * a.nseg + seg] = live_end;
        }
      }
    } else if (GATE && a.state_out) {
      float* so = a.state_out + (size_t)bh * D * D;
  #pragma unroll
      for (int rt = 0; rt < DPL; ++rt)
  #pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
  #pragma unroll
          for (int r = 0; r < 4; ++r)
            so[(size_t)(16 * (DPL * I + rt) + 4 * g_lane + r) * D + j0 + 16 * ct + m_lane] = acc[rt][ct][r];
    }
  };
  switch (w) {
    case 0: run(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{}); break;
    case 4: run(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}); break;
    case 5: run(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); break;
    case 6: run(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{}); break;
  }
}

// ---- split sequences (few heads, long sequences) ----
//
// With S_in(s) the state entering segment s, DS_s segment s's final state
// from a zero state and A_s its log2-gate total, the recurrence is linear:
//   S_in(s+1) = diag(2^{A_s}) S_in(s) + DS_s
// and a token t of chunk c in segment s misses from its output the term
//   (q_t * 2^{R_c + beta_t})^T S_in(s),
// R_c being the log2-gate sum from the segment start to chunk c's start.

// The chain over segments: S_in(s) for s >= 1, transposed and in the element
// type (the operand layout of the output correction), and the final state
// into state_out.  A workgroup owns RPB rows i of one head's state, a thread
// 4 consecutive columns of one row; grid (D / RPB, BH).
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_seg_scan_kernel(FwdArgs a) {
  constexpr int RPB = 1024 / D;                    // state rows per workgroup
  constexpr int NV = RPB * (int)sizeof(T) / 16;    // 16-byte vectors per transposed row piece
  __shared__ float tile[RPB][D + 4];
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * RPB;
  const int tid = threadIdx.x;
  const int ri = tid / (D / 4), j = 4 * (tid % (D / 4));
  const int i = i0 + ri;
  const float* base = a.seg_state + (size_t)bh * a.nseg * D * D + (size_t)i * D + j;
  float4 S = *reinterpret_cast<const float4*>(base);      // segment 0 ends with its complete state
  for (int sg = 1; sg < a.nseg; ++sg) {
    const float4 ds = *reinterpret_cast<const float4*>(base + (size_t)sg * D * D);
    const float dec = exp_2(a.seg_total[((size_t)bh * a.nseg + sg) * D + i]);
    // S_in(sg)^T rows j .. j + 3, columns i0 .. i0 + RPB
    *reinterpret_cast<float4*>(&tile[ri][j]) = S;
    __syncthreads();
    if (tid < D * NV) {
      const int jj = tid / NV, part = tid % NV;
      constexpr int EV = 16 / sizeof(T);
      float x[EV];
  #pragma unroll
      for (int e = 0; e < EV; ++e) x[e] = tile[part * EV + e][jj];
      uint4 o;
      store_pack<T, EV>(reinterpret_cast<T*>(&o), x);
      T* dst = reinterpret_cast<T*>(a.seg_in_t) + (((size_t)bh * a.nseg + sg) * D + jj) * D + i0 + part * EV;
      *reinterpret_cast<uint4*>(dst) = o;
    }
    __syncthreads();
    S.x = fmaf(dec, S.x, ds.x);
    S.y = fmaf(dec, S.y, ds.y);
    S.z = fmaf(dec, S.z, ds.z);
    S.w = fmaf(dec, S.w, ds.w);
  }
  if (a.state_out) *reinterpret_cast<float4*>(a.state_out + (size_t)bh * D * D + (size_t)i * D + j) = S;
}

constexpr int kFixChunks = 2;           // chunks per workgroup of the output correction

template <typename T, int D>
struct FixLayout {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDS = D + PAD;        // sSt [D][LDS]: S_in transposed, element type
  static constexpr int LDQ = D + PAD;        // sQs [64][LDQ]: scaled queries
  static constexpr int LDC = D + 4;          // sC [64][LDC] float, over sQs: the correction
  static constexpr int DG = D / 8;           // threads per token row (8 dimensions each)
  static constexpr int TG = 256 / DG;        // token groups
  static constexpr int NTT = 64 / TG;        // consecutive tokens per thread
  static constexpr int QC = 64 * LDQ * (int)sizeof(T) > 64 * LDC * 4 ? 64 * LDQ * (int)sizeof(T) : 64 * LDC * 4;
  static constexpr int OFF_S = 0;
  static constexpr int OFF_Q = OFF_S + D * LDS * (int)sizeof(T);
  static constexpr int OFF_P = OFF_Q + QC;                // token groups' gate totals [TG][D] float
  static constexpr int TOTAL = OFF_P + TG * D * 4;
};

// y_t += (q_t * 2^{R_c + beta_t})^T S_in(s) for the chunks of segments
// s >= 1.  Grid (nseg - 1, BH, chunk groups of FG): the groups at the start
// of every segment, where the carried state matters most, are dispatched
// first.  4 wavefronts.  Thread
// (tg, dg) loads tokens NTT*tg .. of the chunk in dimensions 8dg .. 8dg+7
// (16-byte vectors, all issued at the chunk start); wavefront w computes the
// chunk's rows 16w .. 16w+15 on the matrix cores.
template <typename T, int D, bool LOGIT>
__global__ __launch_bounds__(256, 2) void fwd_seg_fix_kernel(FwdArgs a) {
  typedef FixLayout<T, D> Lay;
  constexpr int FG = kFixChunks;         // chunks per workgroup
  constexpr int DG = Lay::DG, NTT = Lay::NTT;
  constexpr int VT = 8 * (int)sizeof(T) / 16;    // 16-byte vectors per 8 elements of T
  extern __shared__ __align__(16) unsigned char smem[];
  T* sSt = reinterpret_cast<T*>(smem + Lay::OFF_S);
  T* sQs = reinterpret_cast<T*>(smem + Lay::OFF_Q);
  float* sC = reinterpret_cast<float*>(smem + Lay::OFF_Q);
  float* sP = reinterpret_cast<float*>(smem + Lay::OFF_P);

  const int sg = blockIdx.x + 1;
  const int bh = blockIdx.y;
  const int L = a.L;
  const int nc = (L + 63) / 64;
  int c_lo, c_hi;
  segment_chunks(sg, a.nseg, nc, c_lo, c_hi);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int dg = tid % DG, tg = tid / DG;
  const int d0 = 8 * dg;


  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D + d0;
  T* yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D + d0;
  const float* lgg = a.log_g ? a.log_g + (size_t)bh * L * D + d0 : nullptr;
  const T* xg = LOGIT ? reinterpret_cast<const T*>(a.gate_logit) + (size_t)bh * L * D + d0 : nullptr;
  // chunk groups blockIdx.z, blockIdx.z + gridDim.z, ... up to the first
  // chunk below the cut (found by the forward pass)
  const int c_end = a.seg_live[(size_t)bh * a.nseg + sg];
  if (c_lo + (int)blockIdx.z * FG >= c_end) return;
  // the incoming state, S_in^T rows, 16-byte vectors (read after the first
  // chunk's barriers)
  {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.seg_in_t) +
                                                      ((size_t)bh * a.nseg + sg) * D * D);
    constexpr int VPR = D * (int)sizeof(T) / 16;     // vectors per row
    constexpr int N = D * VPR / 256;
    uint4 buf[N];
  #pragma unroll
    for (int e = 0; e < N; ++e) buf[e] = src[tid + 256 * e];
  #pragma unroll
    for (int e = 0; e < N; ++e) {
      const int v = tid + 256 * e;
      *reinterpret_cast<uint4*>(sSt + (v / VPR) * Lay::LDS + (v % VPR) * (16 / sizeof(T))) = buf[e];
    }
  }
  for (int cb = c_lo + blockIdx.z * FG; cb < c_end; cb += gridDim.z * FG) {
    const int ce = cb + FG < c_end ? cb + FG : c_end;
    for (int c = cb; c < ce; ++c) {
      const int t0 = c * 64 + NTT * tg;             // this thread's first token
      // ---- every global load of the chunk first (rows past L: row L - 1, masked below) ----
      uint4 qv[NTT][VT], yv[NTT][VT], gv[NTT][LOGIT ? VT : 2];
  #pragma unroll
      for (int r = 0; r < NTT; ++r) {
        const size_t row = (size_t)(t0 + r < L ? t0 + r : L - 1) * D;
  #pragma unroll
        for (int e = 0; e < VT; ++e) {
          qv[r][e] = ld16(qg + row + e * (16 / sizeof(T)));
          yv[r][e] = ld16(yg + row + e * (16 / sizeof(T)));
        }
        if constexpr (LOGIT) {
  #pragma unroll
          for (int e = 0; e < VT; ++e) gv[r][e] = ld16(xg + row + e * (16 / sizeof(T)));
        } else {
          gv[r][0] = ld16(lgg + row);
          gv[r][1] = ld16(lgg + row + 4);
        }
      }
      float Rv[8];
      {
        const float* rp = a.chunk_cum + ((size_t)bh * nc + c) * D + d0;
        const float4 r0 = *reinterpret_cast<const float4*>(rp), r1 = *reinterpret_cast<const float4*>(rp + 4);
        Rv[0] = r0.x; Rv[1] = r0.y; Rv[2] = r0.z; Rv[3] = r0.w;
        Rv[4] = r1.x; Rv[5] = r1.y; Rv[6] = r1.z; Rv[7] = r1.w;
      }
      // ---- log2-gate prefix over the thread's tokens, totals per token group ----
      float lb[NTT][8];
  #pragma unroll
      for (int r = 0; r < NTT; ++r) {
        if constexpr (LOGIT) {
  #pragma unroll
          for (int e = 0; e < VT; ++e) unpack16<T>(gv[r][e], lb[r] + e * (16 / sizeof(T)));
  #pragma unroll
          for (int x = 0; x < 8; ++x) lb[r][x] = log_sigmoid(lb[r][x]);
        } else {
          unpack16<float>(gv[r][0], lb[r]);
          unpack16<float>(gv[r][1], lb[r] + 4);
        }
      }
  #pragma unroll
      for (int x = 0; x < 8; ++x) {
        float run = 0.f;
  #pragma unroll
        for (int r = 0; r < NTT; ++r) {
          run += t0 + r < L ? log2_gate(lb[r][x]) : 0.f;
          lb[r][x] = run;
        }
        sP[tg * D + d0 + x] = run;
      }
      __syncthreads();
      // ---- scaled queries into sQs ----
      {
        float off[8];
  #pragma unroll
        for (int x = 0; x < 8; ++x) off[x] = Rv[x];
        for (int gg = 0; gg < tg; ++gg) {
          const float4 p0 = *reinterpret_cast<const float4*>(sP + gg * D + d0);
          const float4 p1 = *reinterpret_cast<const float4*>(sP + gg * D + d0 + 4);
          off[0] += p0.x; off[1] += p0.y; off[2] += p0.z; off[3] += p0.w;
          off[4] += p1.x; off[5] += p1.y; off[6] += p1.z; off[7] += p1.w;
        }
  #pragma unroll
        for (int r = 0; r < NTT; ++r) {
          float qf[8];
  #pragma unroll
          for (int e = 0; e < VT; ++e) unpack16<T>(qv[r][e], qf + e * (16 / sizeof(T)));
          const bool ok = t0 + r < L;
  #pragma unroll
          for (int x = 0; x < 8; ++x) qf[x] = ok ? qf[x] * exp_2(off[x] + lb[r][x]) : 0.f;
          store_pack<T, 8>(sQs + (NTT * tg + r) * Lay::LDQ + d0, qf);
        }
      }
      __syncthreads();
      // ---- the correction: rows 16w + 4g + r, columns 16ct + m ----
      f32x4 cv[D / 16];
  #pragma unroll
      for (int ct = 0; ct < D / 16; ++ct)
        cv[ct] = mma_rows<T, D>(zero4(), sQs + (16 * w + m) * Lay::LDQ + g * (D / 4),
                                sSt + (16 * ct + m) * Lay::LDS + g * (D / 4));
      __syncthreads();                              // sC overlays sQs
  #pragma unroll
      for (int ct = 0; ct < D / 16; ++ct)
  #pragma unroll
        for (int r = 0; r < 4; ++r) sC[(16 * w + 4 * g + r) * Lay::LDC + 16 * ct + m] = cv[ct][r];
      __syncthreads();
      // ---- y += correction ----
  #pragma unroll
      for (int r = 0; r < NTT; ++r) {
        if (t0 + r >= L) continue;
        float yf[8];
  #pragma unroll
        for (int e = 0; e < VT; ++e) unpack16<T>(yv[r][e], yf + e * (16 / sizeof(T)));
        const float* cp = sC + (NTT * tg + r) * Lay::LDC + d0;
        const float4 c0 = *reinterpret_cast<const float4*>(cp), c1 = *reinterpret_cast<const float4*>(cp + 4);
        yf[0] += c0.x; yf[1] += c0.y; yf[2] += c0.z; yf[3] += c0.w;
        yf[4] += c1.x; yf[5] += c1.y; yf[6] += c1.z; yf[7] += c1.w;
        uint4 o[VT];
        store_pack<T, 8>(reinterpret_cast<T*>(o), yf);
  #pragma unroll
        for (int e = 0; e < VT; ++e) st16(yg + (size_t)(t0 + r) * D + e * (16 / sizeof(T)), o[e]);
      }
      __syncthreads();                              // sC / sP reused by the next chunk
    }
  }
}

template <typename T, int D, int DV, bool STATES, bool LOGIT, int MODE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  constexpr bool SEG = MODE == kSeg;
  typedef FwdLayout<T, D, DV, STATES> Lay;
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS budget");
  static_assert(!STATES || Lay::TOTAL <= 80 * 1024, "LDS: the states-only pass runs two workgroups per CU");
  static_assert(D == 128 || (D == 64 && sizeof(T) == 2) || (D == 64 && DV == 32), "shapes");
  const int smem = Lay::TOTAL;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lizard_fwd_kernel<T, D, DV, STATES, LOGIT, MODE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  const int groups = (a.BH + 7) / 8;
  dim3 grid(8 * groups * a.nsplit * (SEG ? a.nseg : 1));
  hipLaunchKernelGGL((lizard_fwd_kernel<T, D, DV, STATES, LOGIT, MODE>), grid, dim3(512), smem, st, a);
  return hipGetLastError();
}

template <typename T, int D, bool LOGIT>
static hipError_t launch_seg_finish(const FwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((fwd_seg_scan_kernel<T, D>), dim3(D / (1024 / D), a.BH), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  typedef FixLayout<T, D> Lay;
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS budget");
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_seg_fix_kernel<T, D, LOGIT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, Lay::TOTAL);
  if (e != hipSuccess) return e;
  const int nc = (a.L + 63) / 64;
  const int longest = (nc + a.nseg - 1) / a.nseg;
  const int groups = (longest + kFixChunks - 1) / kFixChunks;
  hipLaunchKernelGGL((fwd_seg_fix_kernel<T, D, LOGIT>), dim3(a.nseg - 1, a.BH, groups < 2048 ? groups : 2048),
                     dim3(256), Lay::TOTAL, st, a);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_fwd_s(const FwdArgs& a, hipStream_t st) {
  // states and no outputs: the states-only pass of the backward; states and
  // outputs: the full forward, keeping the states as well
  if (a.states && !a.y) {
    if (a.nseg != 1) return hipErrorInvalidValue;
    return a.gate_logit ? launch_fwd_t<T, D, DV, true, true, kPlain>(a, st)
                        : launch_fwd_t<T, D, DV, true, false, kPlain>(a, st);
  }
  if (a.states) {
    if (a.nseg != 1) return hipErrorInvalidValue;
    return a.gate_logit ? launch_fwd_t<T, D, DV, false, true, kTrain>(a, st)
                        : launch_fwd_t<T, D, DV, false, false, kTrain>(a, st);
  }
  if (a.nseg <= 1)
    return a.gate_logit ? launch_fwd_t<T, D, DV, false, true, kPlain>(a, st)
                        : launch_fwd_t<T, D, DV, false, false, kPlain>(a, st);
  hipError_t e = a.gate_logit ? launch_fwd_t<T, D, DV, false, true, kSeg>(a, st)
                              : launch_fwd_t<T, D, DV, false, false, kSeg>(a, st);
  if (e != hipSuccess) return e;
  return a.gate_logit ? launch_seg_finish<T, D, true>(a, st) : launch_seg_finish<T, D, false>(a, st);
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
