// Stage-1 attention transfer on gfx950: the causal softmax teacher and the
// output-matching loss.
//
// The layer is trained in two stages; in the first, the linearised attention
// is fitted to reproduce the outputs of the softmax attention it replaces
// ("Lizard" explainer, gist.science (de), section 2 "Trainingsprozess": stage
// 1 matches the teacher's attention outputs; it section 2 "Fase di
// Addestramento").  With the same q, k, v feeding both, one synthetic step is
//
//   Y_T  = softmax(scale * q k^T, causal) v        (this file, teacher kernel)
//   Y    = the Lizard layer's forward               (lizard_fwd.hip)
//   loss = mean((Y - Y_T)^2),  dY = 2 (Y - Y_T) / N (this file, loss kernel)
//   the Lizard backward of dY                       (lizard_bwd.hip)
//
// Teacher kernel: one workgroup of 4 wavefronts per (b*h, block of 64 QT
// queries); wavefront w owns query tiles of 16 (MFMA column m): queries
// 64qt + 16w .. + 15 of the block for qt < QT (QT = 2 in bf16, 1 in fp32),
// and walks the key blocks up to the diagonal.  Per key block the keys and
// the transposed values are staged in LDS, and each key or value fragment a
// wavefront reads feeds the products of all its query tiles.  S^T tiles
// (keys x queries) come from MFMA with the queries as the B operand, the
// online softmax keeps one reference point and sum per query in every lane
// of its column, and P goes into the O^T = V^T P^T product, whose
// accumulators hold O[query m][j = 16jt + 4g + r].  In bf16, P stays in
// registers: the S^T tiles take their key rows in an order under which the
// scores a lane holds are exactly the keys its lane group contracts over in
// the product (see key_of below); in fp32 it goes through LDS (per
// wavefront).
#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

namespace {

// Query tiles of 16 per wavefront: bf16 takes two, so each key and value
// fragment read from LDS feeds two products; float32 passes P through an LDS
// tile per wavefront and takes one.
template <typename T>
constexpr int teacher_query_tiles() { return sizeof(T) == 2 ? 2 : 1; }

template <typename T, int D>
struct TeacherLayout {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDK = D + PAD;      // sK [64][LDK]: keys of the block
  static constexpr int LDV = 64 + PAD;     // sVt [D][LDV]: values transposed
  static constexpr int LDP = 64 + PAD;     // sP [4][16][LDP]: P of each wavefront
  static constexpr int BUF = 64 * LDK * (int)sizeof(T) + D * LDV * (int)sizeof(T);   // one key block
  static constexpr int OFF_K = 0;                       // + b * BUF for buffer b
  static constexpr int OFF_V = 64 * LDK * (int)sizeof(T);
  static constexpr int OFF_P = 2 * BUF;
  static constexpr int TOTAL = OFF_P + (sizeof(T) == 2 ? 0 : 4 * 16 * LDP * (int)sizeof(T));
};

}  // namespace

template <typename T, int D>
// Two wavefronts per SIMD (the registers a wavefront needs allow no more):
// with that budget the compiler keeps the output accumulators in VGPRs, so
// the per-block softmax work on them needs no moves to and from AGPRs.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void teacher_attn_kernel(TeacherArgs a) {
  typedef TeacherLayout<T, D> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int QV = D / 4 / EPV;          // 16-byte vectors in a lane's k-quarter of a row
  constexpr int NF = D / 4 / M::KPL;       // MFMA steps over a D contraction
  constexpr int NJT = D / 16;              // output column tiles
  constexpr int QT = teacher_query_tiles<T>();  // query tiles of 16 per wavefront
  constexpr int QB = 64 * QT;              // queries per workgroup
  __shared__ __align__(16) unsigned char smem[Lay::TOTAL];
  T* sP = reinterpret_cast<T*>(smem + Lay::OFF_P);

  const int L = a.L, nqb = (L + QB - 1) / QB;
  // block -> (b*h, query block), the longest rows (last query blocks) first
  const int x = blockIdx.x;
  const int bh = x % a.BH;
  const int qb = nqb - 1 - x / a.BH;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  // the key (within the block) of row rho of S^T tile kt.  bf16: tile kt =
  // 2e + h takes keys 32e + 8(rho / 4) + 4h + rho % 4, so lane group g's
  // output rows 4g .. 4g + 3 of tiles 2e and 2e + 1 are keys 32e + 8g .. + 7,
  // its operand run in the product's contraction step e; fp32: row order
  auto key_of = [](int kt, int rho) __attribute__((always_inline)) -> int {
    if constexpr (sizeof(T) == 2) return 32 * (kt >> 1) + 8 * (rho >> 2) + 4 * (kt & 1) + (rho & 3);
    else return 16 * kt + rho;
  };
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  T* yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D;
  T* sPw = sP + w * 16 * Lay::LDP;

  // this lane's query in tile qt (column m of the wavefront's tiles): row
  // 16w + m of the workgroup's 64-query half qt, so every wavefront has one
  // tile in each half; its k-quarter g
  int tq[QT];
  frag qf[QT][NF];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    tq[qt] = qb * QB + 64 * qt + 16 * w + m;
    uint4 raw[QV];
    const bool ok = tq[qt] < L;
    const T* p = qg + (size_t)(ok ? tq[qt] : 0) * D + g * (D / 4);
#pragma unroll
    for (int e = 0; e < QV; ++e) raw[e] = ok ? ld16(p + e * EPV) : make_uint4(0, 0, 0, 0);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < NF; ++e) qf[qt][e] = __builtin_bit_cast(bf16x8, raw[e]);
    } else {
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        const uint4 r = raw[e >> 2];
        const uint32_t u = (e & 3) == 0 ? r.x : (e & 3) == 1 ? r.y : (e & 3) == 2 ? r.z : r.w;
        qf[qt][e] = __builtin_bit_cast(float, u);
      }
    }
  }

  f32x4 oacc[QT][NJT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) oacc[qt][jt] = zero4();
  // per query tq[qt]: reference point (log2 units, scaled) and sum
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
  }
  constexpr float kLazyLog2 = 8.f;        // largest log2 of a weight before the reference moves

  // one key block's keys (16-byte vectors, row-major) and values (32-bit
  // words of VC columns, RPT consecutive keys per thread), loaded a block ahead
  constexpr int KVEC = 64 * (D / EPV) / 256;  // key vectors per thread
  constexpr int VC = 4 / sizeof(T);
  constexpr int VRW = D / VC;                 // threads across a value row
  constexpr int RPT = 64 * VRW / 256;         // keys per thread in the value load
  static_assert(KVEC * 256 == 64 * (D / EPV) && RPT % 8 == 0, "teacher staging shape");
  uint4 kreg[KVEC];
  uint32_t vreg[RPT];
  auto load_rows = [&](int kb, bool full) __attribute__((always_inline)) {
    const int k0 = kb * 64;
    if (full) {
      // one address per thread and array, the other rows at fixed offsets
      // from it (no per-row 64-bit address arithmetic): key vector tid % KRV
      // of rows tid / KRV + KRS u, value words of rows RPT (tid / VRW) + rr
      constexpr int KRV = D / EPV, KRS = 256 / KRV;
      const unsigned ut = static_cast<unsigned>(tid);
      const T* kb0 = kg + ((size_t)k0 + ut / KRV) * D + (ut % KRV) * EPV;
#pragma unroll
      for (int u = 0; u < KVEC; ++u) kreg[u] = ld16(kb0 + (size_t)(KRS * u) * D);
      const uint32_t* vb0 =
          reinterpret_cast<const uint32_t*>(vg + ((size_t)k0 + (size_t)RPT * (ut / VRW)) * D + VC * (ut % VRW));
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) vreg[rr] = vb0[rr * (D / VC)];
      return;
    }
#pragma unroll
    for (int u = 0; u < KVEC; ++u) {
      const int i = tid + 256 * u;
      const int row = i / (D / EPV), cv = i % (D / EPV);
      const bool ok = full || k0 + row < L;
      const uint4 r = ld16(kg + (size_t)(ok ? k0 + row : 0) * D + cv * EPV);
      kreg[u] = ok ? r : make_uint4(0, 0, 0, 0);
    }
    const int vj = tid % VRW, vs = tid / VRW;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int row = k0 + RPT * vs + rr;
      const bool ok = full || row < L;
      const uint32_t r = *reinterpret_cast<const uint32_t*>(vg + (size_t)(ok ? row : 0) * D + VC * vj);
      vreg[rr] = ok ? r : 0u;
    }
  };
  // a uniform branch: full blocks load without row guards (selects on the
  // loaded data would make the compiler wait for the loads right away)
  auto load_block = [&](int kb) __attribute__((always_inline)) {
    if ((kb + 1) * 64 <= L) load_rows(kb, true);
    else load_rows(kb, false);
  };
  // the registers into LDS buffer b: keys row-major, values transposed (8-key runs)
  auto store_block = [&](int b) __attribute__((always_inline)) {
    T* sK = reinterpret_cast<T*>(smem + b * Lay::BUF + Lay::OFF_K);
    T* sVt = reinterpret_cast<T*>(smem + b * Lay::BUF + Lay::OFF_V);
#pragma unroll
    for (int u = 0; u < KVEC; ++u) {
      const int i = tid + 256 * u;
      const int row = i / (D / EPV), cv = i % (D / EPV);
      *reinterpret_cast<uint4*>(sK + row * Lay::LDK + cv * EPV) = kreg[u];
    }
    const int vj = tid % VRW, vs = tid / VRW;
#pragma unroll
    for (int cc = 0; cc < VC; ++cc)
#pragma unroll
      for (int b8 = 0; b8 < RPT / 8; ++b8) {
        float v8[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const uint32_t wv = vreg[8 * b8 + rr];
          if constexpr (sizeof(T) == 2) v8[rr] = __builtin_bit_cast(float, cc == 0 ? (wv << 16) : (wv & 0xffff0000u));
          else v8[rr] = __builtin_bit_cast(float, wv);
        }
        store_pack<T, 8>(sVt + (VC * vj + cc) * Lay::LDV + RPT * vs + 8 * b8, v8);
      }
  };
  load_block(0);
  store_block(0);
  __syncthreads();

  // Key block kb is in buffer kb & 1.  Block kb + 1's loads fly while kb is
  // multiplied, then go to the other buffer, whose last readers (block kb - 1)
  // finished before the previous barrier: one barrier per block.  The last
  // key block is the one holding the workgroup's last query (or key L - 1).
  const int kb_end = (min(qb * QB + QB, L) - 1) / 64;
  for (int kb = 0; kb <= kb_end; ++kb) {
    const int k0 = kb * 64;
    const T* sK = reinterpret_cast<const T*>(smem + (kb & 1) * Lay::BUF + Lay::OFF_K);
    const T* sVt = reinterpret_cast<const T*>(smem + (kb & 1) * Lay::BUF + Lay::OFF_V);
    if (kb < kb_end) load_block(kb + 1);

    // ---- S^T tiles: keys key_of(kt, 4g + r) (rows) x query tq[qt] (column m);
    // each key fragment read once for all QT query tiles ----
    f32x4 z[QT][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const T* kp = sK + key_of(kt, m) * Lay::LDK + g * (D / 4);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) z[qt][kt] = zero4();
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        const frag kf = M::load(kp + e * M::KPL);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) z[qt][kt] = M::mma(kf, qf[qt][e], z[qt][kt]);
      }
    }
    // causal mask, only on the key blocks from the workgroup's first query on
    // (keys past L lie only there: every earlier block is full); a tile whose
    // queries all precede the block gets -inf everywhere, weights 0.  Maxima
    // on raw logits (the scale is positive), the scale folded into the exponent
    if (kb >= qb * QT) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = k0 + key_of(kt, 4 * g + r);
            z[qt][kt][r] = s <= tq[qt] && s < L ? z[qt][kt][r] : -INFINITY;
          }
    }
    float p[QT][4][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, z[qt][kt][r]);
      // finite on the first block (key 0 is valid for every query); -inf for a
      // tile the block lies wholly after, which then leaves its state alone
      const float mblk = xgroup_max(mx) * a.scale_log2;
      // The reference point of the exponentials moves only when some query's
      // block maximum exceeds it by more than 2^kLazyLog2 (so every weight
      // stays at most 2^kLazyLog2, and most blocks skip rescaling the
      // accumulators); O / l and the lse are the same up to rounding.  Always
      // taken on the first block (mrun = -inf), where corr = 0.
      if (__any(mblk > mrun[qt] + kLazyLog2)) {
        const float mnew = fmaxf(mrun[qt], mblk);
        const float corr = exp_2(mrun[qt] - mnew);
        mrun[qt] = mnew;
        lrun[qt] *= corr;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[qt][jt][r] *= corr;
      }
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[qt][kt][r] = exp_2(fmaf(z[qt][kt][r], a.scale_log2, -mrun[qt]));
          ls += p[qt][kt][r];
        }
      lrun[qt] += xgroup_sum(ls);
    }
    if constexpr (sizeof(T) != 2) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) store_pack<T, 4>(sPw + m * Lay::LDP + 16 * kt + 4 * g, p[0][kt]);
    }

    // ---- O^T[j][tq] += sum over the block's keys of V^T[j][s] P[tq][s] ----
    if constexpr (sizeof(T) == 2) {
      // contraction step e over keys 32e .. 32e + 31: lane group g takes
      // keys 32e + 8g .. + 7, which are the scores of tiles 2e and 2e + 1
      // this lane holds
      frag pf[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          bf16x8 f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f[r] = static_cast<bf16>(p[qt][2 * e][r]);
            f[4 + r] = static_cast<bf16>(p[qt][2 * e + 1][r]);
          }
          pf[qt][e] = f;
        }
      // each value fragment read once for all QT query tiles
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const frag vf = M::load(sVt + (16 * jt + m) * Lay::LDV + 32 * e + 8 * g);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) oacc[qt][jt] = M::mma(vf, pf[qt][e], oacc[qt][jt]);
        }
    } else {
      static_assert(QT == 1, "the float32 teacher passes P through one LDS tile per wavefront");
      wave_lds_sync();
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
        oacc[0][jt] = mma_rows<T, 64>(oacc[0][jt], sVt + (16 * jt + m) * Lay::LDV + g * 16, sPw + m * Lay::LDP + g * 16);
    }
    if (kb < kb_end) store_block((kb + 1) & 1);
    // the next block is in place; this wavefront's P tile is free again
    __syncthreads();
  }

  // ---- epilogue: O[tq][16jt + 4g + r] = O^T / l ----
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (tq[qt] < L) {
      const float inv = 1.0f / lrun[qt];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const float o4[4] = {oacc[qt][jt][0] * inv, oacc[qt][jt][1] * inv, oacc[qt][jt][2] * inv,
                             oacc[qt][jt][3] * inv};
        store_pack<T, 4>(yg + (size_t)tq[qt] * D + 16 * jt + 4 * g, o4);
      }
      if (a.lse && g == 0) a.lse[(size_t)bh * L + tq[qt]] = (mrun[qt] + __log2f(lrun[qt])) * kLn2;
    }
  }
}

// dY = 2 (Y - Y_T) / N and, per (b, h), sum((Y - Y_T)^2) / N in a fixed order.
// One workgroup of kLossThreads threads per (b, h) (16 wavefronts, so a
// head's stream has four per SIMD in flight); thread t sums elements t,
// t + kLossThreads, ... of the head, then the partial sums are added by a
// fixed tree.
constexpr int kLossThreads = 1024;
template <typename T>
__global__ __launch_bounds__(kLossThreads) void transfer_loss_kernel(const T* y, const T* yt, T* dy, float* loss_bh,
                                                                     long long per_head, float inv_n) {
  __shared__ float sRed[kLossThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const T* yp = y + (size_t)bh * per_head;
  const T* tp = yt + (size_t)bh * per_head;
  T* dp = dy + (size_t)bh * per_head;
  float acc = 0.f;
  constexpr int V = 16 / sizeof(T);
  const long long nvec = per_head / V;
  for (long long i = tid; i < nvec; i += kLossThreads) {
    float a8[V], b8[V], d8[V];
    unpack16<T>(ld16(yp + i * V), a8);
    unpack16<T>(ld16(tp + i * V), b8);
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const float e = a8[u] - b8[u];
      acc += e * e;
      d8[u] = 2.f * inv_n * e;
    }
    if constexpr (V == 8) store_pack<T, 8>(dp + i * V, d8);
    else store_pack<T, 4>(dp + i * V, d8);
  }
  for (long long i = nvec * V + tid; i < per_head; i += kLossThreads) {   // tail (per_head not a multiple of V)
    const float e = to_f32(yp[i]) - to_f32(tp[i]);
    acc += e * e;
    dp[i] = from_f32<T>(2.f * inv_n * e);
  }
  sRed[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int s = kLossThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) sRed[tid] += sRed[tid + s];
    __syncthreads();
  }
  if (tid == 0) loss_bh[bh] = sRed[0] * inv_n;
}

hipError_t launch_teacher(const TeacherArgs& a, int dtype_bf16, int D, hipStream_t st) {
  const int qb_rows = 64 * (dtype_bf16 ? teacher_query_tiles<bf16>() : teacher_query_tiles<float>());
  const int nqb = (a.L + qb_rows - 1) / qb_rows;
  dim3 grid(a.BH * nqb);
  if (dtype_bf16 && D == 128) hipLaunchKernelGGL((teacher_attn_kernel<bf16, 128>), grid, dim3(256), 0, st, a);
  else if (dtype_bf16 && D == 64) hipLaunchKernelGGL((teacher_attn_kernel<bf16, 64>), grid, dim3(256), 0, st, a);
  else if (!dtype_bf16 && D == 64) hipLaunchKernelGGL((teacher_attn_kernel<float, 64>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_transfer_loss(const void* y, const void* yt, void* dy, float* loss_bh, int BH, long long per_head,
                                float inv_n, int dtype_bf16, hipStream_t st) {
  if (dtype_bf16)
    hipLaunchKernelGGL(transfer_loss_kernel<bf16>, dim3(BH), dim3(kLossThreads), 0, st, static_cast<const bf16*>(y),
                       static_cast<const bf16*>(yt), static_cast<bf16*>(dy), loss_bh, per_head, inv_n);
  else
    hipLaunchKernelGGL(transfer_loss_kernel<float>, dim3(BH), dim3(kLossThreads), 0, st, static_cast<const float*>(y),
                       static_cast<const float*>(yt), static_cast<float*>(dy), loss_bh, per_head, inv_n);
  return hipGetLastError();
}

}  // namespace lizard
