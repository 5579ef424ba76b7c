// S2-Attn backward kernels for gfx950.
//
// The pages only say gradients flow through the attention while fine-tuning
// (page "LongLoRA: Efficient Fine-tuning of Long-Context Large Language
// Models", section 3.2, Phase 1 item 5); the gradients are those of causal
// softmax attention inside every (batch, head, group) of the rolled frame
// described in section 3.4 ("The shifting mechanism", Algorithm 1):
//     P  = exp(scale * Q K^T - lse)            (causal within the group)
//     dV = P^T dO,   dP = dO V^T,   Dvec = rowsum(dO * O)
//     dS = P * (dP - Dvec)
//     dQ = scale * dS K,   dK = scale * dS^T Q
// with dK, dV summed over the query heads that share a key/value head.
//
// Three kernels on one stream:
//   1. s2attn_bwd_pre   : Dvec[b,h,t] = sum_d dO*O (fp32), and zeroes the fp32
//                         dQ accumulator rows.
//   2. s2attn_bwd_main  : one workgroup per 128 key rows of one (batch, KV
//                         head).  Its K and V stay in registers (each wave owns
//                         32 keys).  It walks every query head sharing the KV
//                         head and, in that head's rolled frame, every 64-row
//                         query tile of the group from the diagonal to the
//                         group end.  Per tile: S and dP (keys on lanes), P and
//                         dS, dV^T += dO^T P and dK^T += Q^T dS in registers,
//                         dS through LDS, then dQ = dS K added atomically into
//                         the fp32 accumulator at the original rows.
//   3. s2attn_bwd_cvt   : dq = accumulator, rounded to the output type.
#include "s2attn_common.h"

namespace s2a {

// ---------------------------------------------------------------------------
// 1. Dvec and accumulator clear
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_pre(
    const T* __restrict__ o, const T* __restrict__ dO, float* __restrict__ dvec,
    float* __restrict__ dq_acc, int N, int H, long long rows) {
  constexpr int TPR = D / 8;                    // threads per (b, t, h) row
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;                      // rows is a multiple of 256 / TPR: whole groups exit
  const v8<T> a = *reinterpret_cast<const v8<T>*>(o + row * D + part * 8);
  const v8<T> g = *reinterpret_cast<const v8<T>*>(dO + row * D + part * 8);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf((float)a[i], (float)g[i], s);
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  *reinterpret_cast<f32x4*>(dq_acc + row * D + part * 8) = z;
  *reinterpret_cast<f32x4*>(dq_acc + row * D + part * 8 + 4) = z;
  if (part == 0) {
    const long long h = row % H;
    const long long bt = row / H;
    const long long t = bt % N, b = bt / N;
    dvec[(b * H + h) * N + t] = s;
  }
}

// ---------------------------------------------------------------------------
// 3. accumulator -> dq
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void s2attn_bwd_cvt(const float* __restrict__ acc, T* __restrict__ dq,
                                                      long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + i * 8);
  const f32x4 b2 = *reinterpret_cast<const f32x4*>(acc + i * 8 + 4);
  f32x16 x;
#pragma unroll
  for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b2[j]; }
  *reinterpret_cast<v8<T>*>(dq + i * 8) = pack8<T>(x, 0);
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
struct BwdShape {
  static constexpr int kThreads = 256;
  static constexpr int kBKV = 128;                          // key rows per workgroup (32 per wave)
  static constexpr int kBQ = sizeof(T) == 2 ? 64 : 32;      // query rows per step
  static constexpr int kNQS = kBQ / 32;
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kQCPR = D / 8;                       // chunks per row of Qs / dOs
  static constexpr int kTCPR = kBQ / 8;                     // chunks per row of Qt / dOt
  static constexpr int kKCPR = kBKV / 8;                    // chunks per row of Kt / dSs
  static constexpr int kQRowsPerThread = kBQ * D / 8 / kThreads;   // transposed staging
  static constexpr int kKRowsPerThread = kBKV * D / 8 / kThreads;
  // LDS layout (in 8-element chunks)
  static constexpr int kQs = 0;
  static constexpr int kdOs = kQs + kBQ * kQCPR;
  static constexpr int kQt = kdOs + kBQ * kQCPR;
  static constexpr int kdOt = kQt + D * kTCPR;
  static constexpr int kKt = kdOt + D * kTCPR;
  static constexpr int kdSs = kKt + D * kKCPR;
  static constexpr int kChunks = kdSs + kBQ * kKCPR;
  static constexpr size_t kLdsBytes = kChunks * 8 * sizeof(T) + 2 * kBQ * sizeof(float);
};

template <typename T, int N_>
struct alignas(sizeof(T) * N_) PackB { T x[N_]; };

// Write RPT rows x 8 columns held in registers as RPT consecutive columns of
// 8 rows of a transposed LDS tile with CPR chunks per row.
template <typename T, int RPT, int CPR>
__device__ __forceinline__ void store_transposed(v8<T>* tile, const v8<T>* regs, int dchunk, int col0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = dchunk * 8 + e;
    PackB<T, RPT> pk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) pk.x[i] = regs[i][e];
    T* rowp = reinterpret_cast<T*>(&tile[chunk_at<CPR>(d, col0 / 8)]);
    *reinterpret_cast<PackB<T, RPT>*>(rowp + (col0 % 8)) = pk;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_main(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dvec,
    float* __restrict__ dq_acc, T* __restrict__ dk, T* __restrict__ dv,
    int N, int H, int Hkv, int G, int shift_heads, float scale) {
  using S = BwdShape<T, D>;
  constexpr int BKV = S::kBKV, BQ = S::kBQ, NQS = S::kNQS;
  constexpr int QCPR = S::kQCPR, TCPR = S::kTCPR, KCPR = S::kKCPR;
  constexpr int QRPT = S::kQRowsPerThread, KRPT = S::kKRowsPerThread;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  v8<T>* smem = reinterpret_cast<v8<T>*>(smem_raw);
  v8<T>* Qs = smem + S::kQs;
  v8<T>* dOs = smem + S::kdOs;
  v8<T>* Qt = smem + S::kQt;
  v8<T>* dOt = smem + S::kdOt;
  v8<T>* Kt = smem + S::kKt;
  v8<T>* dSs = smem + S::kdSs;
  float* lse_s = reinterpret_cast<float*>(smem + S::kChunks);   // lse * log2(e)
  float* dvec_s = lse_s + BQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // Key tiles at the start of a group meet the most queries: dispatched first.
  const int groups = N / G;
  const int x = blockIdx.x;
  const int pos = x / groups, grp = x % groups;
  const int c = blockIdx.y, b = blockIdx.z;
  const int r = H / Hkv;
  const int h0 = c * r;
  const int sig0 = (h0 >= H - shift_heads) ? G / 2 : 0;
  const int j0 = grp * G + pos * BKV;           // first key row, rolled frame of head h0

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const T* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const T* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // ---- this wave's 32 keys as B operands (key on lanes, head dim in k-slots)
  const int key_local = wave * 32 + l32;
  const int tk = orig_row(j0 + key_local, sig0, N);
  v8<T> kf[S::kDC], vf[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc) {
    kf[cc] = *reinterpret_cast<const v8<T>*>(kb + (size_t)tk * kvstride + cc * 16 + hf * 8);
    vf[cc] = *reinterpret_cast<const v8<T>*>(vb + (size_t)tk * kvstride + cc * 16 + hf * 8);
  }
  // ---- K transposed into LDS (B operand of dQ = dS K)
  {
    const int dc = tid % (D / 8), kg = tid / (D / 8);
    v8<T> kr[KRPT];
#pragma unroll
    for (int i = 0; i < KRPT; ++i) {
      const int t = orig_row(j0 + kg * KRPT + i, sig0, N);
      kr[i] = *reinterpret_cast<const v8<T>*>(kb + (size_t)t * kvstride + dc * 8);
    }
    store_transposed<T, KRPT, KCPR>(Kt, kr, dc, kg * KRPT);
  }

  f32x16 dkacc[S::kDT], dvacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dkacc[dt][i] = 0.f; dvacc[dt][i] = 0.f; }

  const float c2 = scale * kLog2e;
  const int q_dc = tid % (D / 8), q_qg = tid / (D / 8);

  for (int hh = 0; hh < r; ++hh) {
    const int h = h0 + hh;
    const int sig = (h >= H - shift_heads) ? G / 2 : 0;
    int jk0 = j0 + sig0 - sig;                  // same key rows in head h's rolled frame
    if (jk0 < 0) jk0 += N;
    if (jk0 >= N) jk0 -= N;
    const int gstart = (jk0 / G) * G;
    const int qt_begin = jk0 / BQ, qt_end = (gstart + G) / BQ;
    const T* qb = q + (size_t)b * N * qstride + (size_t)h * D;
    const T* dob = dO + (size_t)b * N * qstride + (size_t)h * D;
    const float* lse_h = lse + ((size_t)b * H + h) * N;
    const float* dvec_h = dvec + ((size_t)b * H + h) * N;
    float* dqacc_h = dq_acc + (size_t)b * N * qstride + (size_t)h * D;
    const int jkey = jk0 + key_local;           // this lane's key, rolled frame of h

    v8<T> qr[QRPT], dr[QRPT];
    float lse_r = 0.f, dvec_r = 0.f;
    auto load_q = [&](int jq0) {
#pragma unroll
      for (int i = 0; i < QRPT; ++i) {
        const int t = orig_row(jq0 + q_qg * QRPT + i, sig, N);
        qr[i] = *reinterpret_cast<const v8<T>*>(qb + (size_t)t * qstride + q_dc * 8);
        dr[i] = *reinterpret_cast<const v8<T>*>(dob + (size_t)t * qstride + q_dc * 8);
      }
      if (tid < BQ) {
        const int t = orig_row(jq0 + tid, sig, N);
        lse_r = lse_h[t] * kLog2e;
        dvec_r = dvec_h[t];
      }
    };

    load_q(qt_begin * BQ);
    for (int qt = qt_begin; qt < qt_end; ++qt) {
      const int jq0 = qt * BQ;
      // stage Q, dO (row-major and transposed), lse, Dvec
#pragma unroll
      for (int i = 0; i < QRPT; ++i) {
        const int row = q_qg * QRPT + i;
        Qs[chunk_at<QCPR>(row, q_dc)] = qr[i];
        dOs[chunk_at<QCPR>(row, q_dc)] = dr[i];
      }
      store_transposed<T, QRPT, TCPR>(Qt, qr, q_dc, q_qg * QRPT);
      store_transposed<T, QRPT, TCPR>(dOt, dr, q_dc, q_qg * QRPT);
      if (tid < BQ) { lse_s[tid] = lse_r; dvec_s[tid] = dvec_r; }
      __syncthreads();
      if (qt + 1 < qt_end) load_q(jq0 + BQ);

      // S = Q K^T and dP = dO V^T, keys on lanes, queries in registers
      f32x16 sacc[NQS], pacc[NQS];
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[qs][i] = 0.f; pacc[qs][i] = 0.f; }
        const int row = qs * 32 + perm32(l32);
#pragma unroll
        for (int cc = 0; cc < S::kDC; ++cc) {
          mma32(sacc[qs], Qs[chunk_at<QCPR>(row, cc * 2 + hf)], kf[cc]);
          mma32(pacc[qs], dOs[chunk_at<QCPR>(row, cc * 2 + hf)], vf[cc]);
        }
      }
      // P and dS (dS carries the softmax scale)
      const bool need_mask = jk0 + wave * 32 + 31 > jq0;
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qs * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          float p = fast_exp2(fmaf(sacc[qs][i], c2, -lse_s[qi]));
          if (need_mask && jkey > jq0 + qi) p = 0.f;
          sacc[qs][i] = p;
          pacc[qs][i] = p * (pacc[qs][i] - dvec_s[qi]) * scale;
        }
      // dV^T += dO^T P,  dK^T += Q^T dS  (16 queries per k-step)
#pragma unroll
      for (int kc = 0; kc < BQ / 16; ++kc) {
        const v8<T> pf = pack8<T>(sacc[kc >> 1], (kc & 1) * 8);
        const v8<T> sf = pack8<T>(pacc[kc >> 1], (kc & 1) * 8);
#pragma unroll
        for (int dt = 0; dt < S::kDT; ++dt) {
          const int row = dt * 32 + perm32(l32);
          mma32(dvacc[dt], dOt[chunk_at<TCPR>(row, kc * 2 + hf)], pf);
          mma32(dkacc[dt], Qt[chunk_at<TCPR>(row, kc * 2 + hf)], sf);
        }
      }
      // dS -> LDS as [query][key]
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qs * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          T* rowp = reinterpret_cast<T*>(&dSs[chunk_at<KCPR>(qi, key_local >> 3)]);
          rowp[key_local & 7] = (T)pacc[qs][i];
        }
      __syncthreads();

      // dQ = dS K for this query tile, added into the fp32 accumulator
      constexpr int n_out = NQS * S::kDT;
      for (int ot = wave; ot < n_out; ot += 4) {
        const int qs = ot / S::kDT, dt = ot % S::kDT;
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const int rowq = qs * 32 + perm32(l32);
        const int rowd = dt * 32 + l32;
#pragma unroll
        for (int kc = 0; kc < BKV / 16; ++kc)
          mma32(acc, dSs[chunk_at<KCPR>(rowq, kc * 2 + hf)], Kt[chunk_at<KCPR>(rowd, kc * 2 + hf)]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qs * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          const int t = orig_row(jq0 + qi, sig, N);
          atomicAdd(dqacc_h + (size_t)t * qstride + rowd, acc[i]);
        }
      }
    }
  }

  // ---- dK, dV at the original key rows
  T* dkrow = dk + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
  T* dvrow = dv + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<v8<T>*>(dkrow + dt * 32 + u * 16 + hf * 8) = pack8<T>(dkacc[dt], u * 8);
      *reinterpret_cast<v8<T>*>(dvrow + dt * 32 + u * 16 + hf * 8) = pack8<T>(dvacc[dt], u * 8);
    }
}

template <typename T, int D>
hipError_t launch_bwd_prep(const void* o, const void* dO, float* dvec, float* dq_acc,
                           int B, int H, int N, hipStream_t stream) {
  const long long rows = (long long)B * N * H;
  constexpr int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((s2attn_bwd_pre<T, D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                     (const T*)o, (const T*)dO, dvec, dq_acc, N, H, rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                           void* dk, void* dv, const float* dvec, float* dq_acc,
                           int B, int H, int Hkv, int N, int G, int shift_heads, hipStream_t stream) {
  using S = BwdShape<T, D>;
  const float scale = 1.0f / sqrtf((float)D);
  static bool attr_set = false;   // raising the LDS limit is idempotent; a race only repeats it
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&s2attn_bwd_main<T, D>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((s2attn_bwd_main<T, D>), dim3(N / S::kBKV, Hkv, B), dim3(256), S::kLdsBytes, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dO, lse, dvec,
                     dq_acc, (T*)dk, (T*)dv, N, H, Hkv, G, shift_heads, scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_finish(void* dq, const float* dq_acc, int B, int H, int N, hipStream_t stream) {
  const long long n8 = (long long)B * N * H * D / 8;
  hipLaunchKernelGGL((s2attn_bwd_cvt<T>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     dq_acc, (T*)dq, n8);
  return hipGetLastError();
}

#define S2A_INST_BWD(T, D)                                                                               \
  template hipError_t launch_bwd_prep<T, D>(const void*, const void*, float*, float*, int, int, int,    \
                                            hipStream_t);                                              \
  template hipError_t launch_bwd_main<T, D>(const void*, const void*, const void*, const float*,        \
                                            const void*, void*, void*, const float*, float*, int, int,  \
                                            int, int, int, int, hipStream_t);                           \
  template hipError_t launch_bwd_finish<T, D>(void*, const float*, int, int, int, hipStream_t);
S2A_INST_BWD(bf16, 64)
S2A_INST_BWD(bf16, 128)
S2A_INST_BWD(float, 64)
S2A_INST_BWD(float, 128)

}  // namespace s2a
