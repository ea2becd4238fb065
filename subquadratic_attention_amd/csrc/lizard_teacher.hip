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
// Teacher kernel: one workgroup of 4 wavefronts per (b*h, block of 64
// queries); wavefront w owns queries 16w..16w+15 of the block (MFMA column m)
// and walks the key blocks up to the diagonal.  Per key block the keys and
// the transposed values are staged in LDS; S^T tiles (keys x queries) come
// from MFMA with the queries as the B operand, the online softmax keeps one
// running maximum and sum per query in every lane of its column, P goes
// through LDS (per wavefront) into the O^T = V^T P^T product, whose
// accumulators hold O[query m][j = 16jt + 4g + r].
#include "lizard_common.hpp"
#include "lizard_kernels.hpp"

namespace lizard {

namespace {

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
  static constexpr int TOTAL = OFF_P + 4 * 16 * LDP * (int)sizeof(T);
};

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(256) void teacher_attn_kernel(TeacherArgs a) {
  typedef TeacherLayout<T, D> Lay;
  typedef Mfma<T> M;
  typedef typename M::frag frag;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int QV = D / 4 / EPV;          // 16-byte vectors in a lane's k-quarter of a row
  constexpr int NF = D / 4 / M::KPL;       // MFMA steps over a D contraction
  constexpr int NJT = D / 16;              // output column tiles
  __shared__ __align__(16) unsigned char smem[Lay::TOTAL];
  T* sP = reinterpret_cast<T*>(smem + Lay::OFF_P);

  const int L = a.L, nqb = (L + 63) / 64;
  // block -> (b*h, query block), the longest rows (last query blocks) first
  const int x = blockIdx.x;
  const int bh = x % a.BH;
  const int qb = nqb - 1 - x / a.BH;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * L * D;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * L * D;
  T* yg = reinterpret_cast<T*>(a.y) + (size_t)bh * L * D;
  T* sPw = sP + w * 16 * Lay::LDP;

  // this lane's query (column m of the wavefront's tiles), its k-quarter g
  const int tq = qb * 64 + 16 * w + m;
  frag qf[NF];
  {
    uint4 raw[QV];
    const bool ok = tq < L;
    const T* p = qg + (size_t)(ok ? tq : 0) * D + g * (D / 4);
#pragma unroll
    for (int e = 0; e < QV; ++e) raw[e] = ok ? ld16(p + e * EPV) : make_uint4(0, 0, 0, 0);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < NF; ++e) qf[e] = __builtin_bit_cast(bf16x8, raw[e]);
    } else {
#pragma unroll
      for (int e = 0; e < NF; ++e) {
        const uint4 r = raw[e >> 2];
        const uint32_t u = (e & 3) == 0 ? r.x : (e & 3) == 1 ? r.y : (e & 3) == 2 ? r.z : r.w;
        qf[e] = __builtin_bit_cast(float, u);
      }
    }
  }

  f32x4 oacc[NJT];
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) oacc[jt] = zero4();
  float mrun = -INFINITY, lrun = 0.f;     // running max (log2 units, scaled) and sum for query tq

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
  // finished before the previous barrier: one barrier per block.
  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * 64;
    const T* sK = reinterpret_cast<const T*>(smem + (kb & 1) * Lay::BUF + Lay::OFF_K);
    const T* sVt = reinterpret_cast<const T*>(smem + (kb & 1) * Lay::BUF + Lay::OFF_V);
    if (kb < qb) load_block(kb + 1);

    // ---- S^T tiles: keys 16kt + 4g + r (rows) x query tq (column m) ----
    f32x4 z[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const T* kp = sK + (16 * kt + m) * Lay::LDK + g * (D / 4);
      z[kt] = zero4();
#pragma unroll
      for (int e = 0; e < NF; ++e) z[kt] = M::mma(M::load(kp + e * M::KPL), qf[e], z[kt]);
    }
    // causal mask, only on the diagonal block (keys past L lie only there:
    // every earlier block is full); maxima on raw logits (the scale is
    // positive), the scale folded into the exponent
    if (kb == qb) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = k0 + 16 * kt + 4 * g + r;
          z[kt][r] = s <= tq && s < L ? z[kt][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, z[kt][r]);
    // finite: key tq (or key 0) is always valid in the first block
    const float mnew = fmaxf(mrun, xgroup_max(mx) * a.scale_log2);
    const float corr = exp_2(mrun - mnew);  // 0 on the first block (mrun = -inf)
    mrun = mnew;
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = exp_2(fmaf(z[kt][r], a.scale_log2, -mnew));
        ls += p[r];
      }
      store_pack<T, 4>(sPw + m * Lay::LDP + 16 * kt + 4 * g, p);
    }
    lrun = lrun * corr + xgroup_sum(ls);
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[jt][r] *= corr;
    wave_lds_sync();

    // ---- O^T[j][tq] += sum over the block's keys of V^T[j][s] P[tq][s] ----
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
      oacc[jt] = mma_rows<T, 64>(oacc[jt], sVt + (16 * jt + m) * Lay::LDV + g * 16, sPw + m * Lay::LDP + g * 16);
    if (kb < qb) store_block((kb + 1) & 1);
    // the next block is in place; this wavefront's P tile is free again
    __syncthreads();
  }

  // ---- epilogue: O[tq][16jt + 4g + r] = O^T / l ----
  if (tq < L) {
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      const float o4[4] = {oacc[jt][0] * inv, oacc[jt][1] * inv, oacc[jt][2] * inv, oacc[jt][3] * inv};
      store_pack<T, 4>(yg + (size_t)tq * D + 16 * jt + 4 * g, o4);
    }
    if (a.lse && g == 0) a.lse[(size_t)bh * L + tq] = (mrun + __log2f(lrun)) * kLn2;
  }
}

// dY = 2 (Y - Y_T) / N and, per (b, h), sum((Y - Y_T)^2) / N in a fixed order.
// One workgroup of 256 threads per (b, h); thread t sums elements t, t + 256,
// ... of the head, then the 256 partial sums are added by a fixed tree.
template <typename T>
__global__ __launch_bounds__(256) void transfer_loss_kernel(const T* y, const T* yt, T* dy, float* loss_bh,
                                                            long long per_head, float inv_n) {
  __shared__ float sRed[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const T* yp = y + (size_t)bh * per_head;
  const T* tp = yt + (size_t)bh * per_head;
  T* dp = dy + (size_t)bh * per_head;
  float acc = 0.f;
  constexpr int V = 16 / sizeof(T);
  const long long nvec = per_head / V;
  for (long long i = tid; i < nvec; i += 256) {
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
  for (long long i = nvec * V + tid; i < per_head; i += 256) {   // tail (per_head not a multiple of V)
    const float e = to_f32(yp[i]) - to_f32(tp[i]);
    acc += e * e;
    dp[i] = from_f32<T>(2.f * inv_n * e);
  }
  sRed[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int s = 128; s >= 1; s >>= 1) {
    if (tid < s) sRed[tid] += sRed[tid + s];
    __syncthreads();
  }
  if (tid == 0) loss_bh[bh] = sRed[0] * inv_n;
}

hipError_t launch_teacher(const TeacherArgs& a, int dtype_bf16, int D, hipStream_t st) {
  const int nqb = (a.L + 63) / 64;
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
    hipLaunchKernelGGL(transfer_loss_kernel<bf16>, dim3(BH), dim3(256), 0, st, static_cast<const bf16*>(y),
                       static_cast<const bf16*>(yt), static_cast<bf16*>(dy), loss_bh, per_head, inv_n);
  else
    hipLaunchKernelGGL(transfer_loss_kernel<float>, dim3(BH), dim3(256), 0, st, static_cast<const float*>(y),
                       static_cast<const float*>(yt), static_cast<float*>(dy), loss_bh, per_head, inv_n);
  return hipGetLastError();
}

}  // namespace lizard
