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
//   1. s2attn_bwd_pre   : Dvec[b,h,t] = sum_d dO*O (fp32) and lse*log2(e), and
//                         zeroes the fp32 dQ accumulator rows.
//   2. s2attn_bwd_main  : one workgroup per 128 key rows of one (batch, KV
//                         head).  Its K and V stay in registers (each wave owns
//                         32 keys).  It walks every query head sharing the KV
//                         head and, in that head's rolled frame, every 64-row
//                         query tile of the group from the diagonal to the
//                         group end.  Per tile: S and dP (keys on lanes), P and
//                         dS, dV^T += dO^T P and dK^T += Q^T dS in registers,
//                         dS through LDS, then dS K added atomically into
//                         the fp32 accumulator at the original rows.
//                         (fp32 tensors; the bf16 kernel below is the same
//                         algorithm laid out for the bf16 matrix cores.)
//   3. s2attn_bwd_cvt   : dq = scale * accumulator, rounded to the output type.
// dS is kept without the softmax scale; dK and dQ take it at their stores.
#include "s2attn_common.h"

namespace s2a {

// ---------------------------------------------------------------------------
// 1. Dvec and accumulator clear
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_pre(
    const T* __restrict__ o, const T* __restrict__ dO, const float* __restrict__ lse, float* __restrict__ dvec,
    float* __restrict__ lse2, float* __restrict__ dq_acc, int N, int H, long long rows) {
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
    lse2[(b * H + h) * N + t] = lse[(b * H + h) * N + t] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 3. accumulator -> dq
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void s2attn_bwd_cvt(const float* __restrict__ acc, T* __restrict__ dq,
                                                      long long n8, float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + i * 8);
  const f32x4 b2 = *reinterpret_cast<const f32x4*>(acc + i * 8 + 4);
  f32x16 x;
#pragma unroll
  for (int j = 0; j < 4; ++j) { x[j] = a[j] * scale; x[4 + j] = b2[j] * scale; }
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
      // P and dS
      const bool need_mask = jk0 + wave * 32 + 31 > jq0;
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qs * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          float p = fast_exp2(fmaf(sacc[qs][i], c2, -lse_s[qi]));
          if (need_mask && jkey > jq0 + qi) p = 0.f;
          sacc[qs][i] = p;
          pacc[qs][i] = p * (pacc[qs][i] - dvec_s[qi]);
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
      *reinterpret_cast<v8<T>*>(dkrow + dt * 32 + u * 16 + hf * 8) = scale8<T>(dkacc[dt], u * 8, scale);
      *reinterpret_cast<v8<T>*>(dvrow + dt * 32 + u * 16 + hf * 8) = pack8<T>(dvacc[dt], u * 8);
    }
}


// ---------------------------------------------------------------------------
// 2'. bf16 main kernel.
//
// Same work split as above (one workgroup per 128 key rows of one (batch, KV
// head), 4 waves x 32 keys, K and V of the wave's keys in registers, 64-row
// query steps over every query head sharing the KV head), laid out for bf16:
//   * Q, dO, lse*log2(e) and Dvec tiles go from HBM straight into LDS
//     (global_load_lds), double-buffered, row-major; a 64-row query tile never
//     straddles the roll's wrap point, so each tile is one scalar base row.
//   * Transposed operands (dO^T, Q^T for dV, dK; dS and K for dQ) are read with
//     ds_read_b64_tr_b16 from the row-major tiles: nothing is transposed on
//     store.  dS is written as [key][query] with 16-byte stores.
//   * dS is double-buffered so the dQ product of step j-1 runs inside step j:
//     one barrier per step.
// LDS swizzle: 16-byte chunk column c of row r is stored at c ^ swz(r), which
// keeps both the row-major A-operand reads (16 rows perm32(0..15), one column)
// and the transposing reads (4 consecutive rows, 4 consecutive columns) free of
// bank conflicts.
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swz2(int row) {
  if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
struct BwdB16Shape {
  static constexpr int kThreads = 256;
  static constexpr int kBKV = 128;
  static constexpr int kBQ = 64;
  static constexpr int kCPR = D / 8;                    // chunks per Q / dO / K row
  static constexpr int kSCPR = kBQ / 8;                 // chunks per dS row
  static constexpr int kQTile = kBQ * kCPR;             // chunks
  static constexpr int kKTile = kBKV * kCPR;
  static constexpr int kSTile = kBKV * kSCPR;
  static constexpr int kK = 0;
  static constexpr int kQ = kK + kKTile;                // [2 stages]
  static constexpr int kdO = kQ + 2 * kQTile;           // [2 stages]
  static constexpr int kdS = kdO + 2 * kQTile;          // [2 buffers]
  static constexpr int kChunks = kdS + 2 * kSTile;
  static constexpr size_t kLdsBytes = (size_t)kChunks * 16 + 2 * 2 * kBQ * sizeof(float);
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kQLoads = kQTile / kThreads;     // chunks per thread per Q (or dO) tile
  static constexpr int kKLoads = kKTile / kThreads;
};

template <int D>
__global__ __launch_bounds__(256) void s2attn_bwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ dvec,
    float* __restrict__ dq_acc, bf16* __restrict__ dk, bf16* __restrict__ dv,
    int N, int H, int Hkv, int G, int shift_heads, float scale) {
  using S = BwdB16Shape<D>;
  constexpr int BKV = S::kBKV, BQ = S::kBQ, CPR = S::kCPR, SCPR = S::kSCPR;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16x8* smem = reinterpret_cast<bf16x8*>(smem_raw);
  float* fsm = reinterpret_cast<float*>(smem + S::kChunks);   // [stage][lse2 | dvec][BQ]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int g16 = lane >> 4, li = lane & 15, ts = li >> 2, tm = li & 3;

  const int groups = N / G;
  const int x = blockIdx.x;
  const int pos = x / groups, grp = x % groups;       // key tiles early in a group first
  const int c = blockIdx.y, b = blockIdx.z;
  const int r = H / Hkv;
  const int h0 = c * r;
  const int sig0 = (h0 >= H - shift_heads) ? G / 2 : 0;
  const int j0 = grp * G + pos * BKV;                 // key rows, rolled frame of head h0

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const bf16* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const bf16* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // ---- K tile into LDS (row-major, rows may cross the wrap point: per-row addresses)
  {
    bf16x8* Ks = smem + S::kK;
#pragma unroll
    for (int i = 0; i < S::kKLoads; ++i) {
      const int cb = (wave + 4 * i) * 64;
      const int p = cb + lane;
      const int row = p / CPR, pc = p % CPR;
      const int t = orig_row(j0 + row, sig0, N);
      load_lds16(kb + (size_t)t * kvstride + (pc ^ swz2<CPR>(row)) * 8, Ks + cb);
    }
  }
  // ---- this wave's 32 keys: V as B operands in registers (K is read from the LDS tile)
  const int key_local = wave * 32 + l32;
  const int tk = orig_row(j0 + key_local, sig0, N);
  bf16x8 vf[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc)
    vf[cc] = *reinterpret_cast<const bf16x8*>(vb + (size_t)tk * kvstride + cc * 16 + hf * 8);

  // per-lane element offsets of the Q / dO tile chunks this lane moves
  int qoff[S::kQLoads];
#pragma unroll
  for (int i = 0; i < S::kQLoads; ++i) {
    const int p = (wave + 4 * i) * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    qoff[i] = row * (int)qstride + (pc ^ swz2<CPR>(row)) * 8;
  }

  // ---- step cursor over (query head, query tile)
  auto head_frame = [&](int hh, int& sig, int& jk0, int& qt_b, int& qt_e) {
    const int h = h0 + hh;
    sig = (h >= H - shift_heads) ? G / 2 : 0;
    jk0 = j0 + sig0 - sig;
    if (jk0 < 0) jk0 += N;
    if (jk0 >= N) jk0 -= N;
    qt_b = jk0 / BQ;
    qt_e = (jk0 / G) * G / BQ + G / BQ;
  };
  auto issue_step = [&](int hh, int qt, int sig, int stage) {
    const int h = h0 + hh;
    const int t0 = orig_row(qt * BQ, sig, N);         // whole tile contiguous
    const bf16* qg = q + ((size_t)b * N + t0) * qstride + (size_t)h * D;
    const bf16* dog = dO + ((size_t)b * N + t0) * qstride + (size_t)h * D;
    bf16x8* Qs = smem + S::kQ + stage * S::kQTile;
    bf16x8* dOs = smem + S::kdO + stage * S::kQTile;
#pragma unroll
    for (int i = 0; i < S::kQLoads; ++i) {
      const int cb = (wave + 4 * i) * 64;
      load_lds16(qg + qoff[i], Qs + cb);
      load_lds16(dog + qoff[i], dOs + cb);
    }
    const size_t rowbase = ((size_t)b * H + h) * N + t0;
    if (wave == 0) load_lds4(lse2 + rowbase + lane, fsm + stage * 2 * BQ);
    if (wave == 1) load_lds4(dvec + rowbase + lane, fsm + stage * 2 * BQ + BQ);
  };

  f32x16 dkacc[S::kDT], dvacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dkacc[dt][i] = 0.f; dvacc[dt][i] = 0.f; }
  const float c2 = scale * kLog2e;

  // dQ of one finished step: 32x32 (query, head-dim) tiles; with d = 128 a wave
  // owns head-dim block dt = wave for both 32-query halves (sharing its K reads),
  // with d = 64 one tile (qs, dt) per wave.
  constexpr int NT = S::kDT / 2;
  const int dq_dt = S::kDT == 4 ? wave : (wave & 1);
  const int dq_qs0 = S::kDT == 4 ? 0 : (wave >> 1);
  const int rowbytes = (int)(qstride * sizeof(float));
  auto dq_step = [&](int buf, int h, int t0) {
    const bf16* dSs = reinterpret_cast<const bf16*>(smem + S::kdS + buf * S::kSTile);
    const bf16* Ks = reinterpret_cast<const bf16*>(smem + S::kK);
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    const int dcol = dq_dt * 32 + ((g16 & 1) << 4) + 4 * tm;     // B: K columns = head dim
#pragma unroll
    for (int kc = 0; kc < BKV / 16; ++kc) {
      const int r0 = kc * 16 + hf * 8 + ts, r1 = r0 + 4;
      const bf16x8 bk = tr_read8(Ks + (r0 * CPR + ((dcol >> 3) ^ swz2<CPR>(r0))) * 8 + (dcol & 7),
                                 Ks + (r1 * CPR + ((dcol >> 3) ^ swz2<CPR>(r1))) * 8 + (dcol & 7));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int qcol = (dq_qs0 + t) * 32 + ((g16 & 1) << 4) + 4 * tm;   // A: dS rows = queries
        const bf16x8 a = tr_read8(dSs + (r0 * SCPR + ((qcol >> 3) ^ swz2<SCPR>(r0))) * 8 + (qcol & 7),
                                  dSs + (r1 * SCPR + ((qcol >> 3) ^ swz2<SCPR>(r1))) * 8 + (qcol & 7));
        mma32(acc[t], a, bk);
      }
    }
    // lane holds head-dim column dt*32 + l32 of query rows qs*32 + 8*(i>>2) + 4*hf + (i&3)
    float* tile = dq_acc + ((size_t)b * N + t0) * qstride + (size_t)h * D;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile, BQ * rowbytes);
    const int voff = (hf * 4 * (int)qstride + dq_dt * 32 + l32) * (int)sizeof(float);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        buffer_atomic_add(acc[t][i], rs, voff, ((dq_qs0 + t) * 32 + (i >> 2) * 8 + (i & 3)) * rowbytes);
  };

  int hh = 0, sig, jk0, qt_b, qt_e;
  head_frame(0, sig, jk0, qt_b, qt_e);
  int qt = qt_b;
  issue_step(hh, qt, sig, 0);
  int prev_h = -1, prev_t0 = 0, last_stage = 0;
  for (int step = 0;; ++step) {
    const int stage = step & 1;
    // next step's cursor
    int nhh = hh, nqt = qt + 1, nsig = sig, njk0 = jk0, nqt_b = qt_b, nqt_e = qt_e;
    if (nqt == qt_e) {
      ++nhh;
      if (nhh < r) {
        head_frame(nhh, nsig, njk0, nqt_b, nqt_e);
        nqt = nqt_b;
      }
    }
    const bool has_next = nhh < r;

    wait_vmem_all();
    __syncthreads();
    if (has_next) issue_step(nhh, nqt, nsig, stage ^ 1);

    const int h = h0 + hh;
    const int jq0 = qt * BQ;
    const bf16* Qs = reinterpret_cast<const bf16*>(smem + S::kQ + stage * S::kQTile);
    const bf16* dOs = reinterpret_cast<const bf16*>(smem + S::kdO + stage * S::kQTile);
    const float* lse_s = fsm + stage * 2 * BQ;
    const float* dvec_s = lse_s + BQ;

    // S = Q K^T, dP = dO V^T : keys on lanes, queries in registers
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int i = 0; i < 16; ++i) { sacc[qs][i] = 0.f; pacc[qs][i] = 0.f; }
    {
      const bf16* Ks = reinterpret_cast<const bf16*>(smem + S::kK);
      const int ksw = swz2<CPR>(key_local);
      const int row = perm32(l32);                 // qs * 32 + row keeps the same swizzle
      const int sw = swz2<CPR>(row);
#pragma unroll
      for (int cc = 0; cc < S::kDC; ++cc) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (key_local * CPR + ((2 * cc + hf) ^ ksw)) * 8);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          const int off = ((qs * 32 + row) * CPR + ((2 * cc + hf) ^ sw)) * 8;
          mma32(sacc[qs], *reinterpret_cast<const bf16x8*>(Qs + off), kf);
          mma32(pacc[qs], *reinterpret_cast<const bf16x8*>(dOs + off), vf[cc]);
        }
      }
    }

    // dQ of the previous step (its dS is complete in LDS after the barrier)
    if (prev_h >= 0) dq_step(stage ^ 1, prev_h, prev_t0);

    // P = exp2(S c - lse log2 e), dS = P (dP - Dvec)
    const int jkey = jk0 + key_local;
    const bool need_mask = jk0 + wave * 32 + 31 > jq0;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q8 = qs * 32 + u * 16 + hf * 8;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_s + q8);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_s + q8 + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dvec_s + q8);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dvec_s + q8 + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float lq = i < 4 ? l0[i] : l1[i - 4];
          const float dq = i < 4 ? d0[i] : d1[i - 4];
          float p = fast_exp2(fmaf(sacc[qs][u * 8 + i], c2, -lq));
          if (need_mask && jkey > jq0 + q8 + i) p = 0.f;
          sacc[qs][u * 8 + i] = p;
          pacc[qs][u * 8 + i] = p * (pacc[qs][u * 8 + i] - dq);
        }
      }

    // dV^T += dO^T P, dK^T += Q^T dS (A operands through transposing reads)
    bf16x8 pf[4], sf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      pf[kc] = pack8<bf16>(sacc[kc >> 1], (kc & 1) * 8);
      sf[kc] = pack8<bf16>(pacc[kc >> 1], (kc & 1) * 8);
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int r0 = kc * 16 + hf * 8 + ts, r1 = r0 + 4;
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const int dbase = dt * 32 + perm32(((g16 & 1) << 4) + 4 * tm);
        const int o0 = (r0 * CPR + ((dbase >> 3) ^ swz2<CPR>(r0))) * 8 + (dbase & 7);
        const int o1 = (r1 * CPR + ((dbase >> 3) ^ swz2<CPR>(r1))) * 8 + (dbase & 7);
        mma32(dvacc[dt], tr_read8(dOs + o0, dOs + o1), pf[kc]);
        mma32(dkacc[dt], tr_read8(Qs + o0, Qs + o1), sf[kc]);
      }
    }

    // dS -> LDS as [key][query]: 8 consecutive queries per 16-byte store
    {
      bf16x8* dSs = smem + S::kdS + stage * S::kSTile;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int chunk = kc * 2 + hf;       // queries kc*16 + hf*8 .. +7
        dSs[key_local * SCPR + (chunk ^ swz2<SCPR>(key_local))] = sf[kc];
      }
    }

    prev_h = h;
    prev_t0 = orig_row(jq0, sig, N);
    last_stage = stage;
    if (!has_next) break;
    hh = nhh; qt = nqt; sig = nsig; jk0 = njk0; qt_b = nqt_b; qt_e = nqt_e;
  }
  __syncthreads();                               // the last step's dS is complete
  dq_step(last_stage, prev_h, prev_t0);

  // ---- dK (scaled), dV at the original key rows
  bf16* dkrow = dk + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
  bf16* dvrow = dv + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<bf16x8*>(dkrow + dt * 32 + u * 16 + hf * 8) = scale8<bf16>(dkacc[dt], u * 8, scale);
      *reinterpret_cast<bf16x8*>(dvrow + dt * 32 + u * 16 + hf * 8) = pack8<bf16>(dvacc[dt], u * 8);
    }
}

template <typename T, int D>
hipError_t launch_bwd_prep(const void* o, const void* dO, const float* lse, float* dvec, float* lse2,
                           float* dq_acc, int B, int H, int N, hipStream_t stream) {
  const long long rows = (long long)B * N * H;
  constexpr int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((s2attn_bwd_pre<T, D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                     (const T*)o, (const T*)dO, lse, dvec, lse2, dq_acc, N, H, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_main_bf16(const void* q, const void* k, const void* v, const float* lse2, const void* dO,
                                void* dk, void* dv, const float* dvec, float* dq_acc,
                                int B, int H, int Hkv, int N, int G, int shift_heads, float scale,
                                hipStream_t stream) {
  using S = BwdB16Shape<D>;
  static bool attr_set = false;   // raising the LDS limit is idempotent; a race only repeats it
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&s2attn_bwd_bf16_kernel<D>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((s2attn_bwd_bf16_kernel<D>), dim3(N / S::kBKV, Hkv, B), dim3(S::kThreads), S::kLdsBytes,
                     stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, lse2, dvec, dq_acc,
                     (bf16*)dk, (bf16*)dv, N, H, Hkv, G, shift_heads, scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const float* lse, const float* lse2,
                           const void* dO, void* dk, void* dv, const float* dvec, float* dq_acc,
                           int B, int H, int Hkv, int N, int G, int shift_heads, hipStream_t stream) {
  using S = BwdShape<T, D>;
  const float scale = 1.0f / sqrtf((float)D);
  if constexpr (sizeof(T) == 2)
    return launch_bwd_main_bf16<D>(q, k, v, lse2, dO, dk, dv, dvec, dq_acc, B, H, Hkv, N, G, shift_heads, scale,
                                   stream);
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
                     dq_acc, (T*)dq, n8, 1.0f / sqrtf((float)D));
  return hipGetLastError();
}

#define S2A_INST_BWD(T, D)                                                                               \
  template hipError_t launch_bwd_prep<T, D>(const void*, const void*, const float*, float*, float*,     \
                                            float*, int, int, int, hipStream_t);                       \
  template hipError_t launch_bwd_main<T, D>(const void*, const void*, const void*, const float*,        \
                                            const float*, const void*, void*, void*, const float*,     \
                                            float*, int, int, int, int, int, int, hipStream_t);         \
  template hipError_t launch_bwd_finish<T, D>(void*, const float*, int, int, int, hipStream_t);
S2A_INST_BWD(bf16, 64)
S2A_INST_BWD(bf16, 128)
S2A_INST_BWD(float, 64)
S2A_INST_BWD(float, 128)

}  // namespace s2a
