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
// Three stages on one stream, no atomics:
//   prep : -Dvec[b,h,t] = -sum_d dO*O and lse*log2(e), fp32, into the workspace
//          (Dvec negated, so that the bf16 dK/dV kernel starts its dP sums there).
//   dkdv : one workgroup per 128 key rows of one (batch, KV head); it walks
//          every query head sharing the KV head and, in that head's rolled
//          frame, every query tile of the group from the diagonal to the group
//          end, accumulating dK and dV in registers (keys on lanes).
//   dq   : one workgroup per query tile of one (batch, head); it walks the key
//          tiles of the group up to the diagonal, recomputing S and dP (queries
//          on lanes), so dS feeds dQ^T = K^T dS^T straight from registers.
// dS is kept without the softmax scale; dK and dQ take it at their stores.
// Each stage has an fp32 kernel (register-staged LDS tiles, fp32 matrix cores)
// and a bf16 kernel laid out for the bf16 matrix cores (direct-to-LDS tile
// loads, transposing LDS reads), which serves bf16 inputs of every size, with
// a separate instantiation for groups that are not whole tiles.
#include "s2attn_common.h"

#include <type_traits>

namespace s2a {

// ===========================================================================
// prep
// ===========================================================================
template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_pre(
    const T* __restrict__ o, const T* __restrict__ dO, const float* __restrict__ lse, float* __restrict__ dvec,
    float* __restrict__ lse2, int N, int H, long long rows) {
  constexpr int TPR = D / 8;                    // threads per (b, t, h) row
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;                      // whole TPR-lane groups exit together
  const v8<T> a = *reinterpret_cast<const v8<T>*>(o + row * D + part * 8);
  const v8<T> g = *reinterpret_cast<const v8<T>*>(dO + row * D + part * 8);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf((float)a[i], (float)g[i], s);
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (part == 0) {
    const long long h = row % H;
    const long long bt = row / H;
    const long long t = bt % N, b = bt / N;
    dvec[(b * H + h) * N + t] = -s;               // stored negated (see the dK/dV kernel)
    lse2[(b * H + h) * N + t] = lse[(b * H + h) * N + t] * kLog2e;
  }
}

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

// Query heads [hb, he) of the KV head whose first query head is h0 that a dK/dV
// launch takes, and its epilogue mode (0: store dK, dV; 1: store fp32 sums to the
// partial buffer; 2: add the partial buffer's sums, then store).  pass 0 takes
// every head.  A KV head shared by unshifted and shifted query heads (whose two
// frames do not cut its keys into the same tiles) runs in two launches: pass 1
// takes its unshifted heads, pass 2 its shifted ones; a KV head with one kind
// only is finished by the one pass that has heads for it.  Returns false if this
// launch has nothing to do for the KV head.
__device__ __forceinline__ bool dkdv_head_range(int pass, int H, int shift_heads, int h0, int r, int& hb, int& he,
                                                int& mode) {
  const int nu = min(max(H - shift_heads - h0, 0), r);   // its unshifted query heads (they come first)
  hb = 0;
  he = r;
  mode = 0;
  if (pass == 1) {
    he = nu;
    mode = nu == r ? 0 : 1;
    return nu > 0;
  }
  if (pass == 2) {
    hb = nu;
    mode = nu == 0 ? 0 : 2;
    return nu < r;
  }
  return true;
}
// fp32 partial sums of one key row (the layout of a dK / dV row): the lane's
// elements dt * 32 + u * 16 + 8 hf + e, from register 8 u + e of tile dt, times s.
template <int D>
__device__ __forceinline__ void store_part(float* row, const f32x16* acc, float s, int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = acc[dt][u * 8 + e] * s;
        b[e] = acc[dt][u * 8 + 4 + e] * s;
      }
      *reinterpret_cast<f32x4*>(row + dt * 32 + u * 16 + hf * 8) = a;
      *reinterpret_cast<f32x4*>(row + dt * 32 + u * 16 + hf * 8 + 4) = b;
    }
}
// acc = acc * s + the partial sums of the row (same layout)
template <int D>
__device__ __forceinline__ void add_part(const float* row, f32x16* acc, float s, int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + dt * 32 + u * 16 + hf * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(row + dt * 32 + u * 16 + hf * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[dt][u * 8 + e] = fmaf(acc[dt][u * 8 + e], s, a[e]);
        acc[dt][u * 8 + 4 + e] = fmaf(acc[dt][u * 8 + 4 + e], s, b[e]);
      }
    }
}

// ===========================================================================
// dkdv, fp32 ("generic": written for any element type, instantiated for
// fp32 only).  Also takes groups that are not whole tiles: key rows past
// the group compute on a copy of its last row and are not stored; query rows of
// the next group in the last query tile are masked; rows past N are clamped.
// ===========================================================================
template <typename T, int D>
struct DkdvShape {
  static constexpr int kThreads = 256;
  static constexpr int kBKV = 128;                          // key rows per workgroup (32 per wave)
  static constexpr int kBQ = sizeof(T) == 2 ? 64 : 32;      // query rows per step
  static constexpr int kNQS = kBQ / 32;
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kQCPR = D / 8;                       // chunks per row of Qs / dOs
  static constexpr int kTCPR = kBQ / 8;                     // chunks per row of Qt / dOt
  static constexpr int kQRowsPerThread = kBQ * D / 8 / kThreads;
  static constexpr int kQs = 0;
  static constexpr int kdOs = kQs + kBQ * kQCPR;
  static constexpr int kQt = kdOs + kBQ * kQCPR;
  static constexpr int kdOt = kQt + D * kTCPR;
  static constexpr int kChunks = kdOt + D * kTCPR;
  static constexpr size_t kLdsBytes = kChunks * 8 * sizeof(T) + 2 * kBQ * sizeof(float);
};

template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ dvec,
    T* __restrict__ dk, T* __restrict__ dv, int N, int H, int Hkv, int G, int shift_heads, int wrap,
    float scale, int pass, float* __restrict__ part) {
  using S = DkdvShape<T, D>;
  constexpr int BKV = S::kBKV, BQ = S::kBQ, NQS = S::kNQS;
  constexpr int QCPR = S::kQCPR, TCPR = S::kTCPR, QRPT = S::kQRowsPerThread;
  __shared__ __align__(16) unsigned char smem_raw[S::kLdsBytes];
  v8<T>* smem = reinterpret_cast<v8<T>*>(smem_raw);
  v8<T>* Qs = smem + S::kQs;
  v8<T>* dOs = smem + S::kdOs;
  v8<T>* Qt = smem + S::kQt;
  v8<T>* dOt = smem + S::kdOt;
  float* lse_s = reinterpret_cast<float*>(smem + S::kChunks);   // lse * log2(e)
  float* dvec_s = lse_s + BQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // Key tiles at the start of a group meet the most queries: dispatched first.
  const int groups = num_groups(N, G), tiles_per_group = (G + BKV - 1) / BKV;
  const TileOrder to = tile_order(blockIdx.x, gridDim.x / tiles_per_group, tiles_per_group);
  const int pos = to.rank, grp = to.pair % groups;
  const int c = (to.pair / groups) % Hkv, b = to.pair / (groups * Hkv);
  const int r = H / Hkv;
  const int h0 = c * r;
  int hb, he, mode;                             // the query heads this launch takes (dkdv_head_range)
  if (!dkdv_head_range(pass, H, shift_heads, h0, r, hb, he, mode)) return;
  const int sig0 = (h0 + hb >= H - shift_heads) ? G / 2 : 0;
  const bool swap = wrap == kWrapSwap;
  const WrapGroup wg = wrap_group(N, G);
  auto tok = [&](int j, int sig) { return swap ? token_of_row<true>(j, sig, N, wg) : orig_row(j, sig, N); };
  const int ge0 = min(grp * G + G, N);          // end of the group (a last group may be short)
  const int j0 = grp * G + pos * BKV;           // first key row, rolled frame of head h0 + hb
  if (j0 >= ge0) return;                        // a tile past the end of a short group

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const T* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const T* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // this wave's 32 keys as B operands (key on lanes, head dim in k-slots);
  // keys past the group compute on a copy of its last row and are not stored
  const int key_local = wave * 32 + l32;
  const bool k_ok = j0 + key_local < ge0;
  const int tk = tok(k_ok ? j0 + key_local : ge0 - 1, sig0);
  v8<T> kf[S::kDC], vf[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc) {
    kf[cc] = *reinterpret_cast<const v8<T>*>(kb + (size_t)tk * kvstride + cc * 16 + hf * 8);
    vf[cc] = *reinterpret_cast<const v8<T>*>(vb + (size_t)tk * kvstride + cc * 16 + hf * 8);
  }

  f32x16 dkacc[S::kDT], dvacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dkacc[dt][i] = 0.f; dvacc[dt][i] = 0.f; }

  const float c2 = scale * kLog2e;
  const int q_dc = tid % (D / 8), q_qg = tid / (D / 8);

  for (int hh = hb; hh < he; ++hh) {
    const int h = h0 + hh;
    const int sig = (h >= H - shift_heads) ? G / 2 : 0;
    // same key rows in head h's rolled frame
    const int jk0 = swap ? frame_row<true>(j0, sig0, sig, N, wg) : frame_row<false>(j0, sig0, sig, N, wg);
    const bool split_head = wrap == kWrapSplit && sig != 0;
    // query tiles meeting the workgroup's keys, and the end of this wave's queries
    // (queries from the next group in the last tile are masked); with the split
    // option the later of two keys sees queries at least as far
    const int q_end_g = query_end_row(jk0, G, N, false, wg);
    const int qt_begin = jk0 / BQ;
    const int qt_end = (min(query_end_row(min(jk0 + BKV - 1, q_end_g - 1), G, N, split_head, wg), q_end_g) + BQ - 1) / BQ;
    const int q_end_w = min(query_end_row(min(jk0 + wave * 32 + 31, q_end_g - 1), G, N, split_head, wg), q_end_g);
    const int cut = split_cut(jk0 - jk0 % G, split_head, wg);   // queries from here see no key before it
    const T* qb = q + (size_t)b * N * qstride + (size_t)h * D;
    const T* dob = dO + (size_t)b * N * qstride + (size_t)h * D;
    const float* lse_h = lse2 + ((size_t)b * H + h) * N;
    const float* dvec_h = dvec + ((size_t)b * H + h) * N;
    const int jkey = jk0 + key_local;

    v8<T> qr[QRPT], dr[QRPT];
    float lse_r = 0.f, dvec_r = 0.f;
    auto load_q = [&](int jq0) {
#pragma unroll
      for (int i = 0; i < QRPT; ++i) {
        const int t = tok(min(jq0 + q_qg * QRPT + i, N - 1), sig);   // rows past N are masked
        qr[i] = *reinterpret_cast<const v8<T>*>(qb + (size_t)t * qstride + q_dc * 8);
        dr[i] = *reinterpret_cast<const v8<T>*>(dob + (size_t)t * qstride + q_dc * 8);
      }
      if (tid < BQ) {
        const int t = tok(min(jq0 + tid, N - 1), sig);
        lse_r = lse_h[t];
        dvec_r = -dvec_h[t];
      }
    };

    load_q(qt_begin * BQ);
    for (int qt = qt_begin; qt < qt_end; ++qt) {
      const int jq0 = qt * BQ;
      __syncthreads();                          // previous tile's LDS reads are done
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
      if (jq0 >= q_end_w) continue;             // these queries are in another group than the wave's keys

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
      const bool need_mask = jk0 + wave * 32 + 31 > jq0 || jq0 + BQ > q_end_g ||
                             (jk0 + wave * 32 < cut && jq0 + BQ - 1 >= cut);
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qs * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
          float p = fast_exp2(fmaf(sacc[qs][i], c2, -lse_s[qi]));
          if (need_mask && (jkey > jq0 + qi || jq0 + qi >= q_end_g || (jkey < cut && jq0 + qi >= cut))) p = 0.f;
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
    }
    __syncthreads();                            // next head restages the tiles
  }

  if (!k_ok) return;
  float dk_scale = scale;
  if (mode != 0) {
    // two passes (dkdv_head_range): the first stores fp32 sums, the second adds them
    const size_t dv_part = (size_t)(gridDim.x / tiles_per_group / groups) * N * D;   // B * Hkv * N * D
    float* pk = part + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
    if (mode == 1) {
      store_part<D>(pk, dkacc, scale, hf);
      store_part<D>(pk + dv_part, dvacc, 1.f, hf);
      return;
    }
    add_part<D>(pk, dkacc, scale, hf);
    add_part<D>(pk + dv_part, dvacc, 1.f, hf);
    dk_scale = 1.f;
  }
  T* dkrow = dk + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
  T* dvrow = dv + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<v8<T>*>(dkrow + dt * 32 + u * 16 + hf * 8) = scale8<T>(dkacc[dt], u * 8, dk_scale);
      *reinterpret_cast<v8<T>*>(dvrow + dt * 32 + u * 16 + hf * 8) = pack8<T>(dvacc[dt], u * 8);
    }
}

// ===========================================================================
// dq, fp32 ("generic", as above).  Groups that are not whole tiles as in the
// fp32 forward.
// ===========================================================================
template <typename T, int D>
struct DqShape {
  static constexpr int kThreads = 256;
  static constexpr int kBR = 128;               // query rows per workgroup (32 per wave)
  static constexpr int kBC = 64;                // key rows per tile
  static constexpr int kKCPR = D / 8;
  static constexpr int kTCPR = kBC / 8;
  static constexpr int kKRowsPerThread = kBC * D / 8 / kThreads;
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kKs = 0;
  static constexpr int kVs = kKs + kBC * kKCPR;
  static constexpr int kKt = kVs + kBC * kKCPR;
  static constexpr int kChunks = kKt + D * kTCPR;
  static constexpr size_t kLdsBytes = kChunks * 8 * sizeof(T);
};

template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ dvec, T* __restrict__ dq,
    int N, int H, int Hkv, int G, int shift_heads, int wrap, float scale) {
  using S = DqShape<T, D>;
  constexpr int BR = S::kBR, BC = S::kBC, KCPR = S::kKCPR, TCPR = S::kTCPR, KRPT = S::kKRowsPerThread;
  __shared__ __align__(16) unsigned char smem_raw[S::kLdsBytes];
  v8<T>* smem = reinterpret_cast<v8<T>*>(smem_raw);
  v8<T>* Ks = smem + S::kKs;
  v8<T>* Vs = smem + S::kVs;
  v8<T>* Kt = smem + S::kKt;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int groups = num_groups(N, G), tiles_per_group = (G + BR - 1) / BR;
  const TileOrder to = tile_order(blockIdx.x, gridDim.x / tiles_per_group, tiles_per_group);
  const int pos = tiles_per_group - 1 - to.rank;   // heaviest query tiles first
  const int grp = to.pair % groups;
  const int h = (to.pair / groups) % H, b = to.pair / (groups * H);
  const int c = h / (H / Hkv);
  const int sigma = (h >= H - shift_heads) ? G / 2 : 0;
  const bool split_head = wrap == kWrapSplit && sigma != 0;
  const bool swap_head = wrap == kWrapSwap && sigma != 0;
  const WrapGroup wg = wrap_group(N, G);
  auto tok = [&](int j) { return swap_head ? token_of_row<true>(j, sigma, N, wg) : orig_row(j, sigma, N); };
  const int ge = min(grp * G + G, N);           // end of the group (a last group may be short)
  const int j0 = grp * G + pos * BR;
  if (j0 >= ge) return;                         // a tile past the end of a short group
  const int kv_begin = first_key_row(j0, G, split_head, wg);  // first key row any wave sees
  const int cut = split_cut(grp * G, split_head, wg);         // split option: rows from here see no key before
  const int ntiles = (min(j0 + BR, ge) - kv_begin + BC - 1) / BC;

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const T* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const T* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T): query on lanes;
  // rows past the group compute on a copy of its last row and are not stored
  const int jw = j0 + wave * 32;
  const int jq = jw + l32;
  const bool q_ok = jq < ge;
  const int tq = tok(q_ok ? jq : ge - 1);
  const int kw0 = first_key_row(jw, G, split_head, wg);       // this wave's first key
  v8<T> qf[S::kDC], dof[S::kDC];
  {
    const T* qrow = q + ((size_t)b * N + tq) * qstride + (size_t)h * D;
    const T* dorow = dO + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) {
      qf[cc] = *reinterpret_cast<const v8<T>*>(qrow + cc * 16 + hf * 8);
      dof[cc] = *reinterpret_cast<const v8<T>*>(dorow + cc * 16 + hf * 8);
    }
  }
  const float lse_q = lse2[((size_t)b * H + h) * N + tq];
  const float dvec_q = -dvec[((size_t)b * H + h) * N + tq];

  const int k_dc = tid % (D / 8), k_kg = tid / (D / 8);
  v8<T> kr[KRPT], vr[KRPT];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < KRPT; ++i) {
      const int t = tok(min(kt0 + k_kg * KRPT + i, N - 1));   // rows past N are masked keys
      kr[i] = *reinterpret_cast<const v8<T>*>(kb + (size_t)t * kvstride + k_dc * 8);
      vr[i] = *reinterpret_cast<const v8<T>*>(vb + (size_t)t * kvstride + k_dc * 8);
    }
  };

  f32x16 dqacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[dt][i] = 0.f;
  const float c2 = scale * kLog2e;

  load_tile(kv_begin);
  for (int it = 0; it < ntiles; ++it) {
    const int kt0 = kv_begin + it * BC;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KRPT; ++i) {
      const int row = k_kg * KRPT + i;
      Ks[chunk_at<KCPR>(row, k_dc)] = kr[i];
      Vs[chunk_at<KCPR>(row, k_dc)] = vr[i];
    }
    store_transposed<T, KRPT, TCPR>(Kt, kr, k_dc, k_kg * KRPT);
    __syncthreads();
    if (it + 1 < ntiles) load_tile(kt0 + BC);
    if (kt0 > jw + 31 || kt0 + BC <= kw0 || jw >= ge) continue;   // nothing of this tile for this wave

    // S^T = K Q^T, dP^T = V dO^T : keys on tile rows, queries on lanes
    f32x16 s[2], dp[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[ks][i] = 0.f; dp[ks][i] = 0.f; }
      const int row = ks * 32 + perm32(l32);
#pragma unroll
      for (int cc = 0; cc < S::kDC; ++cc) {
        mma32(s[ks], Ks[chunk_at<KCPR>(row, cc * 2 + hf)], qf[cc]);
        mma32(dp[ks], Vs[chunk_at<KCPR>(row, cc * 2 + hf)], dof[cc]);
      }
    }
    const bool need_mask = kt0 + BC - 1 > jw || (kt0 < cut && jw + 31 >= cut);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s[ks][i], c2, -lse_q));
        const int key = kt0 + ks * 32 + (i >> 3) * 16 + hf * 8 + (i & 7);
        if (need_mask && (key > jq || (key < cut && jq >= cut))) p = 0.f;
        dp[ks][i] = p * (dp[ks][i] - dvec_q);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      const v8<T> sf = pack8<T>(dp[kc >> 1], (kc & 1) * 8);
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const int row = dt * 32 + perm32(l32);
        mma32(dqacc[dt], Kt[chunk_at<TCPR>(row, kc * 2 + hf)], sf);
      }
    }
  }

  if (!q_ok) return;
  T* dqrow = dq + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<v8<T>*>(dqrow + dt * 32 + u * 16 + hf * 8) = scale8<T>(dqacc[dt], u * 8, scale);
}

// ===========================================================================
// bf16 kernels
//
// LDS tiles are row-major and filled straight from HBM (global_load_lds);
// a 64-row query or key tile never straddles the roll's wrap point (G/2 is a
// multiple of 64), so each tile is one scalar base row.  Transposed operands
// come from ds_read_b64_tr_b16.  16-byte chunk column c of row r is stored at
// c ^ swz2(r), which keeps both the row-major operand reads (16 rows
// perm32(0..15), one column) and the transposing reads (4 consecutive rows,
// 4 consecutive columns) free of bank conflicts.
// ===========================================================================
template <int CPR>
__device__ __forceinline__ int swz2(int row) {
  if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// ---------------------------------------------------------------------------
// dkdv, bf16: 8 waves (two per SIMD, so one wave's matrix-core work overlaps
// its partner's softmax).  Wave w owns keys 32*(w & 3) .. +31 of the 128-key
// tile and query half w >> 2 of every 64-row query step; the two halves' dK,
// dV partial sums meet in LDS at the end.  K and V tiles stay in LDS for the
// whole workgroup; Q, dO, lse*log2(e) and Dvec tiles are double-buffered with
// one barrier per step.  Every LDS read is a per-lane offset fixed before the
// loop plus a compile-time immediate (the step loop is unrolled over the two
// buffer stages); diagonal steps run a masked instantiation and steps whose
// keys all follow the wave's queries are skipped.
// ---------------------------------------------------------------------------
template <int D>
struct DkdvB16Shape {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 512;
  static constexpr int kBKV = 128;
  static constexpr int kBQ = 64;
  static constexpr int kCPR = D / 8;
  static constexpr int kRowB = D * 2;                     // bytes per tile row
  static constexpr int kQTileB = kBQ * kRowB;
  static constexpr int kKTileB = kBKV * kRowB;
  // byte offsets: the per-step stages (lse*log2(e) and Dvec, Q, dO) first, so
  // that every read of them is a per-lane offset plus a 16-bit immediate; the
  // resident K and V tiles above them share one set of per-lane addresses
  // (V = K + immediate)
  static constexpr int kF = 0;                            // floats [stage][lse2 | dvec][kBQ]
  static constexpr int kQ = kF + 2 * 2 * kBQ * (int)sizeof(float);   // [2 stages]
  static constexpr int kdO = kQ + 2 * kQTileB;            // [2 stages]
  static constexpr int kK = kdO + 2 * kQTileB;
  static constexpr int kV = kK + kKTileB;
  static constexpr size_t kLdsBytes = (size_t)kV + kKTileB;
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kQLoads = kBQ * kCPR / kThreads;   // 16-byte chunks per thread per Q (or dO) tile
  static constexpr int kKLoads = kBKV * kCPR / kThreads;
  // end-of-kernel exchange of the dK, dV partial sums: [key group][dK|dV][dt][reg][lane] floats
  static constexpr size_t kXchgBytes = (size_t)4 * 2 * kDT * 16 * 64 * sizeof(float);
  static_assert(kXchgBytes <= kLdsBytes, "partial sums must fit in the LDS tiles");
};

__device__ __forceinline__ bf16x8 lds_b128(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}
__device__ __forceinline__ f32x4 lds_f32x4(const char* base, int off) {
  return *reinterpret_cast<const f32x4*>(base + off);
}

// Store a gradient row held as D/32 accumulator tiles (element
// dt * 32 + u * 16 + 8 hf + e in register 8 u + e of tile dt), times `scale`,
// turned back by the rotary embedding at position pos (the transpose of the
// forward rotation): the gradient with respect to the unrotated input.
// Element i < D/2 and its partner i + D/2 sit in tiles dt and dt + D/64 of the
// same lane.
template <int D>
__device__ __forceinline__ void store_turned_back(bf16* row, const f32x16* acc, float scale, double pos,
                                                  double log2_base, int hf) {
  constexpr int HT = D / 64;
#pragma unroll
  for (int dt = 0; dt < HT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 ya, yb;
      double g[8];
      rope_revs8<D>(dt * 32 + u * 16 + hf * 8, log2_base, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn, y0, y1;
        rope_cs(pos, g[e], cs, sn);
        rope_turn(acc[dt][u * 8 + e] * scale, acc[dt + HT][u * 8 + e] * scale, cs, -sn, y0, y1);
        ya[e] = (bf16)y0;
        yb[e] = (bf16)y1;
      }
      *reinterpret_cast<bf16x8*>(row + dt * 32 + u * 16 + hf * 8) = ya;
      *reinterpret_cast<bf16x8*>(row + (dt + HT) * 32 + u * 16 + hf * 8) = yb;
    }
}

// SPLIT: the split wrap option; EDGE: groups that are not whole tiles (query
// rows of the next group are masked, tiles that cross the wrap point or the
// end of the sequence take per-row addresses, keys past the group are not
// stored); SWAP: the swap wrap option's row map (token_of_row).  Each is
// compiled separately, so that the main method's step loop carries no trace
// of any of them.
// ROPE (launched for rope.on): q and k arrive rotated by the rotary embedding; dk is turned back
// (the transpose of the rotation) before it is stored, so it is the gradient
// with respect to the unrotated k.
template <int D, bool SPLIT, bool EDGE, bool SWAP, bool ROPE, bool PART>
__global__ __launch_bounds__(512) void s2attn_bwd_dkdv_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ dvec,
    bf16* __restrict__ dk, bf16* __restrict__ dv, int N, int H, int Hkv, int G, int shift_heads, float scale,
    RopeArgs rope, int pass, float* __restrict__ part) {
  using S = DkdvB16Shape<D>;
  constexpr int BKV = S::kBKV, BQ = S::kBQ, CPR = S::kCPR, RB = S::kRowB;
  // static, so that tile addresses are compile-time constants and every LDS
  // read is a per-lane offset plus an immediate
  __shared__ __align__(16) unsigned char smem_raw[S::kLdsBytes];
  char* lds = reinterpret_cast<char*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int g16 = lane >> 4, li = lane & 15, ts = li >> 2, tm = li & 3;
  const int kg = wave & 3, qh = wave >> 2;

  const int groups = EDGE ? num_groups(N, G) : N / G;
  const int tiles_per_group = EDGE ? (G + BKV - 1) / BKV : G / BKV;
  const TileOrder to = tile_order(blockIdx.x, gridDim.x / tiles_per_group, tiles_per_group);
  const int grp = to.pair % groups;
  const int c = (to.pair / groups) % Hkv, b = to.pair / (groups * Hkv);
  const int r = H / Hkv;
  const int h0 = c * r;
  // Key tiles early in a group first (they meet the most queries).  A key/value
  // head read by unshifted and shifted query heads in one pass (whole tiles, G/2
  // a whole number of them): its tile at position p in the first frame sits at
  // p + T/2 (mod T) in the other, so the work of p and of p + T/2 is alike and
  // falls with p within each half: the two halves go interleaved.
  const int n_unsh = min(max(H - shift_heads - h0, 0), r);
  const bool mixed = !EDGE && !PART && n_unsh != 0 && n_unsh != r && (tiles_per_group & 1) == 0;
  const int pos = mixed ? (to.rank >> 1) + (to.rank & 1) * (tiles_per_group >> 1) : to.rank;
  // the query heads [hb, he) of this KV head that this launch takes, and what
  // the epilogue does (pass 0: all heads; passes 1, 2: unshifted, then shifted)
  int hb, he, mode;
  if (!dkdv_head_range(PART ? pass : 0, H, shift_heads, h0, r, hb, he, mode)) return;
  const int sig0 = (h0 + hb >= H - shift_heads) ? G / 2 : 0;
  const WrapGroup wg = wrap_group(N, G);
  const int j0 = grp * G + pos * BKV;                 // key rows, rolled frame of head h0 + hb
  const int ge0 = EDGE ? min(grp * G + G, N) : grp * G + G;   // end of their group
  if (EDGE && j0 >= ge0) return;                      // a tile past the end of a short group

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const bf16* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const bf16* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // K and V tiles into LDS once (their 128 rows may cross the wrap point)
#pragma unroll
  for (int i = 0; i < S::kKLoads; ++i) {
    const int cb = (wave + S::kWaves * i) * 64;
    const int p = cb + lane;
    const int row = p / CPR, pc = p % CPR;
    const size_t g = (size_t)token_of_row<SWAP>(EDGE ? min(j0 + row, N - 1) : j0 + row, sig0, N, wg) * kvstride +
                     (pc ^ swz2<CPR>(row)) * 8;
    load_lds16(kb + g, lds + S::kK + cb * 16);
    load_lds16(vb + g, lds + S::kV + cb * 16);
  }
  // Q, dO of this batch and lse*log2(e), Dvec of its heads; a query tile is
  // loaded through buffers based at its first row, with the per-lane byte
  // offsets inside the tile fixed here (the host bounds 64 rows of Q below
  // 2^31 bytes)
  const bf16* qbb = q + (size_t)b * N * qstride;
  const bf16* dobb = dO + (size_t)b * N * qstride;
  const float* lbb = lse2 + (size_t)b * H * N;
  const float* dbb = dvec + (size_t)b * H * N;
  int qoff[S::kQLoads];
#pragma unroll
  for (int i = 0; i < S::kQLoads; ++i) {
    const int p = (wave + S::kWaves * i) * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    qoff[i] = (row * (int)qstride + (pc ^ swz2<CPR>(row)) * 8) * 2;
  }

  // ---- per-lane LDS byte offsets
  const int key_row = kg * 32 + l32;                  // B operand of S and dP: this lane's key
  int offB[S::kDC];                                   // LDS addresses of the K operand; V = K + kKTileB
  const int arow = qh * 32 + perm32(l32);             // A operand of S and dP: query rows
  int offA[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc) {
    offB[cc] = S::kK + key_row * RB + (((2 * cc + hf) ^ swz2<CPR>(key_row)) << 4);
    offA[cc] = arow * RB + (((2 * cc + hf) ^ swz2<CPR>(arow)) << 4);
    // hide the value from the optimiser, so that the V reads address it plus an
    // immediate instead of taking registers of their own (K and V lie beyond
    // the 16-bit immediate range)
    asm volatile("" : "+v"(offB[cc]));
  }
  // transposing reads of dO^T / Q^T: rows (queries) qh*32 + 16u + 8hf + 4t + ts, head-dim columns of block dt
  int offT[S::kDT][2];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = qh * 32 + hf * 8 + 4 * t + ts;
      const int dbase = dt * 32 + perm32(((g16 & 1) << 4) + 4 * tm);
      offT[dt][t] = row * RB + (((dbase >> 3) ^ swz2<CPR>(row)) << 4) + (dbase & 7) * 2;
    }
  const int offL = (qh * 32 + hf * 8) * 4;            // lse / Dvec floats of this lane's queries

  // The key tile seen from a query head: only two frames exist (unshifted,
  // shifted), so they are fixed here: first key row in the head's rolled frame,
  // the head's query tiles [qt_b, qt_e) meeting the tile's keys, and the end
  // row of the queries meeting this wave's keys.
  // EDGE: the group end qge bounds every query (the last query tile may run
  // into the next group), and keys past it belong to the next group.
  int fr_jk0[2], fr_qb[2], fr_qe[2], fr_wqe[2], fr_qge[2];
#pragma unroll
  for (int sh = 0; sh < 2; ++sh) {
    const int jk = frame_row<SWAP>(j0, sig0, sh * (G / 2), N, wg);
    const bool split_head = SPLIT && sh;
    const int qge = query_end_row(jk, G, N, false, wg);
    fr_jk0[sh] = jk;
    fr_qb[sh] = jk / BQ;
    // EDGE: the split option's cut may fall inside a 32-key run, whose later
    // keys see queries at least as far: take the run's last key in the group
    fr_qe[sh] = EDGE ? (min(query_end_row(min(jk + BKV - 1, qge - 1), G, N, split_head, wg), qge) + BQ - 1) / BQ
                     : query_end_row(jk + BKV - 32, G, N, split_head, wg) / BQ;
    fr_wqe[sh] = EDGE ? min(query_end_row(min(jk + kg * 32 + 31, qge - 1), G, N, split_head, wg), qge)
                      : query_end_row(jk + kg * 32, G, N, split_head, wg);
    fr_qge[sh] = qge;
  }
  auto head_frame = [&](int hh, int& sig, int& jk0, int& qt_b, int& qt_e, int& wqe) {
    const int sh = h0 + hh >= H - shift_heads;
    sig = sh ? G / 2 : 0;
    jk0 = fr_jk0[sh];
    qt_b = fr_qb[sh];
    qt_e = fr_qe[sh];
    wqe = fr_wqe[sh];
  };
  // EDGE: the group end; one frame only (a KV head shared by shifted and
  // unshifted query heads either has whole tiles in both frames or runs its
  // two kinds of heads in two passes)
  const int qge = fr_qge[sig0 != 0];
  // EDGE with the split option: query rows from the cut on see no key row before it
  const int cut = (EDGE && SPLIT) ? split_cut(fr_jk0[sig0 != 0] - fr_jk0[sig0 != 0] % G, sig0 != 0, wg) : -1;
  auto issue_step = [&](int hh, int qt, int sig, int stage) {
    const int h = h0 + hh;
    // EDGE: a query tile whose rows are not consecutive tokens (it crosses the
    // wrap from token N-1 to token 0, a break of the swap option's map, or row
    // N) takes each row's own address (rows past N read row N-1: masked)
    if (EDGE && !rows_contiguous<SWAP>(qt * BQ, BQ, sig, N, wg)) {
#pragma unroll
      for (int i = 0; i < S::kQLoads; ++i) {
        const int p = (wave + S::kWaves * i) * 64 + lane;
        const int row = p / CPR, pc = p % CPR;
        const size_t tok = token_of_row<SWAP>(min(qt * BQ + row, N - 1), sig, N, wg);
        const size_t off = tok * qstride + (size_t)h * D + (pc ^ swz2<CPR>(row)) * 8;
        const int cb = (wave + S::kWaves * i) * 64 * 16;
        load_lds16(qbb + off, lds + S::kQ + stage * S::kQTileB + cb);
        load_lds16(dobb + off, lds + S::kdO + stage * S::kQTileB + cb);
      }
      const size_t loff = (size_t)h * N + token_of_row<SWAP>(min(qt * BQ + lane, N - 1), sig, N, wg);
      if (wave == 0) load_lds4(lbb + loff, lds + S::kF + stage * 2 * BQ * 4);
      if (wave == 1) load_lds4(dbb + loff, lds + S::kF + stage * 2 * BQ * 4 + BQ * 4);
      return;
    }
    const size_t t0 = token_of_row<SWAP>(qt * BQ, sig, N, wg);   // a 64-row tile is contiguous
    const size_t qo = t0 * qstride + (size_t)h * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(const_cast<bf16*>(qbb + qo), BQ * (int)qstride * 2);
    const __amdgpu_buffer_rsrc_t dors = make_rsrc(const_cast<bf16*>(dobb + qo), BQ * (int)qstride * 2);
#pragma unroll
    for (int i = 0; i < S::kQLoads; ++i) {
      const int cb = (wave + S::kWaves * i) * 64 * 16;
      buffer_load_lds16(qrs, qoff[i], 0, lds + S::kQ + stage * S::kQTileB + cb);
      buffer_load_lds16(dors, qoff[i], 0, lds + S::kdO + stage * S::kQTileB + cb);
    }
    const size_t lo = (size_t)h * N + t0;
    if (wave == 0) buffer_load_lds4(make_rsrc(const_cast<float*>(lbb + lo), BQ * 4), lane * 4, 0, lds + S::kF + stage * 2 * BQ * 4);
    if (wave == 1) buffer_load_lds4(make_rsrc(const_cast<float*>(dbb + lo), BQ * 4), lane * 4, 0, lds + S::kF + stage * 2 * BQ * 4 + BQ * 4);
  };

  f32x16 dkacc[S::kDT], dvacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dkacc[dt][i] = 0.f; dvacc[dt][i] = 0.f; }
  const float c2 = scale * kLog2e;

  // one query step for this wave: STG = LDS stage, MASK = causal mask needed
  // qend (EDGE): the end of the queries this lane's key meets: the group end,
  // or, with the split option, the cut for a key before it
  auto compute = [&](auto stg_c, auto mask_c, int jkey, int jq_first, int qend) __attribute__((always_inline)) {
    constexpr int STG = decltype(stg_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const char* Qs = lds + S::kQ + STG * S::kQTileB;
    const char* dOs = lds + S::kdO + STG * S::kQTileB;
    const char* Fs = lds + S::kF + STG * 2 * BQ * 4;
    // dP accumulates onto -Dvec (stored negated), so it ends as dP - Dvec
    f32x16 sacc, pacc;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x4 n0 = lds_f32x4(Fs, BQ * 4 + offL + u * 64), n1 = lds_f32x4(Fs, BQ * 4 + offL + u * 64 + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) { pacc[u * 8 + i] = n0[i]; pacc[u * 8 + 4 + i] = n1[i]; }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) {
      mma32(sacc, lds_b128(Qs, offA[cc]), lds_b128(lds, offB[cc]));
      mma32(pacc, lds_b128(dOs, offA[cc]), lds_b128(lds, offB[cc] + S::kKTileB));
    }
    // P and dS of each 16-query half, then that half's dV / dK products, so the
    // second half's vector work can overlap the first half's matrix work
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x4 l0 = lds_f32x4(Fs, offL + u * 64), l1 = lds_f32x4(Fs, offL + u * 64 + 16);
      f32x8 pv, sv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lq = i < 4 ? l0[i] : l1[i - 4];
        float p = fast_exp2(fmaf(sacc[u * 8 + i], c2, -lq));
        if (MASK) {
          // bitwise, not short-circuit: one select, no branch per element
          const int qi = jq_first + u * 16 + i;
          bool mk = jkey > qi;
          if (EDGE) mk = mk | (qi >= qend);
          p = mk ? 0.f : p;
        }
        pv[i] = p;
        sv[i] = p * pacc[u * 8 + i];
      }
      const bf16x8 pf = __builtin_convertvector(pv, bf16x8);
      const bf16x8 sf = __builtin_convertvector(sv, bf16x8);
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const int o0 = offT[dt][0] + u * 16 * RB, o1 = offT[dt][1] + u * 16 * RB;
        mma32(dvacc[dt], tr_read8(reinterpret_cast<const bf16*>(dOs + o0), reinterpret_cast<const bf16*>(dOs + o1)),
              pf);
        mma32(dkacc[dt], tr_read8(reinterpret_cast<const bf16*>(Qs + o0), reinterpret_cast<const bf16*>(Qs + o1)),
              sf);
      }
    }
  };
  auto step = [&](auto stg_c, int jk0, int wqe, int qt) {
    const int jq0 = qt * BQ;
    const int key_lo = jk0 + kg * 32, q_lo = jq0 + qh * 32;
    if (key_lo > q_lo + 31) return;                   // every key follows every query: P = 0
    if ((SPLIT || EDGE) && q_lo >= wqe) return;       // queries of another group than the wave's keys
    const int jkey = key_lo + l32, jq_first = q_lo + hf * 8;
    const int qend = (EDGE && SPLIT && jkey < cut) ? min(cut, qge) : qge;
    if constexpr (EDGE && SPLIT) {
      // every step masked: one copy of the step body, which keeps this
      // instantiation within the register file
      compute(stg_c, std::integral_constant<bool, true>(), jkey, jq_first, qend);
    } else {
      if (key_lo + 31 > q_lo || (EDGE && q_lo + 31 >= qge))
        compute(stg_c, std::integral_constant<bool, true>(), jkey, jq_first, qend);
      else
        compute(stg_c, std::integral_constant<bool, false>(), jkey, jq_first, qend);
    }
  };

  int hh = hb, sig, jk0, qt_b, qt_e, wqe;
  head_frame(hb, sig, jk0, qt_b, qt_e, wqe);
  int qt = qt_b;
  issue_step(hh, qt, sig, 0);
  // advance the cursor to the next (head, query tile); returns false past the end
  auto advance = [&](int& nhh, int& nqt, int& nsig, int& njk0, int& nqb, int& nqe, int& nwqe) {
    nhh = hh; nqt = qt + 1; nsig = sig; njk0 = jk0; nqb = qt_b; nqe = qt_e; nwqe = wqe;
    if (nqt == qt_e) {
      ++nhh;
      if (nhh < he) {
        head_frame(nhh, nsig, njk0, nqb, nqe, nwqe);
        nqt = nqb;
      }
    }
    return nhh < he;
  };
  auto one = [&](auto stg_c) {
    constexpr int STG = decltype(stg_c)::value;
    int nhh, nqt, nsig, njk0, nqb, nqe, nwqe;
    const bool more = advance(nhh, nqt, nsig, njk0, nqb, nqe, nwqe);
    wait_vmem_all();
    __syncthreads();                                  // this stage landed for all; the other is free
    if (more) issue_step(nhh, nqt, nsig, STG ^ 1);
    step(stg_c, jk0, wqe, qt);
    hh = nhh; qt = nqt; sig = nsig; jk0 = njk0; qt_b = nqb; qt_e = nqe; wqe = nwqe;
    return more;
  };
  while (one(std::integral_constant<int, 0>()) && one(std::integral_constant<int, 1>())) {
  }

  // ---- sum the two query halves' partials, store dK (scaled) and dV at the original key rows
  __syncthreads();                                    // all tiles are dead: reuse LDS
  float* xs = reinterpret_cast<float*>(lds) + (size_t)kg * 2 * S::kDT * 16 * 64;
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xs[((0 * S::kDT + dt) * 16 + i) * 64 + lane] = dkacc[dt][i];
        xs[((1 * S::kDT + dt) * 16 + i) * 64 + lane] = dvacc[dt][i];
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dkacc[dt][i] += xs[((0 * S::kDT + dt) * 16 + i) * 64 + lane];
        dvacc[dt][i] += xs[((1 * S::kDT + dt) * 16 + i) * 64 + lane];
      }
    if (EDGE && j0 + key_row >= ge0) return;          // a key of the next group
    const int tk = token_of_row<SWAP>(j0 + key_row, sig0, N, wg);
    if (mode != 0) {
      // two passes: the first stores its fp32 sums (dK scaled), the second adds them
      const size_t dv_part = (size_t)(gridDim.x / tiles_per_group / groups) * N * D;   // B * Hkv * N * D
      float* pk = part + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
      if (mode == 1) {
        store_part<D>(pk, dkacc, scale, hf);
        store_part<D>(pk + dv_part, dvacc, 1.f, hf);
        return;
      }
      add_part<D>(pk, dkacc, scale, hf);
      add_part<D>(pk + dv_part, dvacc, 1.f, hf);
    }
    const float dk_scale = mode == 2 ? 1.f : scale;   // pass 2's dK sums are scaled already
    bf16* dkrow = dk + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
    bf16* dvrow = dv + ((size_t)b * N + tk) * kvstride + (size_t)c * D;
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<bf16x8*>(dvrow + dt * 32 + u * 16 + hf * 8) = pack8<bf16>(dvacc[dt], u * 8);
    if (ROPE) {
      store_turned_back<D>(dkrow, dkacc, dk_scale, (double)tk * rope.pos_scale, rope.log2_base, hf);
      return;
    }
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<bf16x8*>(dkrow + dt * 32 + u * 16 + hf * 8) = scale8<bf16>(dkacc[dt], u * 8, dk_scale);
  }
}
// ---------------------------------------------------------------------------
// dq, bf16: W waves x 32 queries (W = 8: two waves per SIMD; W = 4 for short
// groups that are not whole tiles, as in the forward), 64-row key / value tiles
// double-buffered in LDS.  Per tile: S^T = K Q^T and dP^T = V dO^T (queries
// on lanes, so lse and Dvec are one value per lane), dS^T in registers, and
// dQ^T += K^T dS^T with K^T read through transposing reads.
// PREP: the prep stage fused in.  Every query row belongs to exactly one
// workgroup, which already holds its dO row, so it computes Dvec = dO . O and
// lse * log2(e) itself and writes both to the workspace for the dK/dV stage.
// EDGE: groups that are not whole tiles, as in the forward kernel.
// ---------------------------------------------------------------------------
template <int D, int W = 8>
struct DqB16Shape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kBR = 32 * W;
  static constexpr int kBC = 64;
  static constexpr int kCPR = D / 8;
  static constexpr int kTile = kBC * kCPR;               // chunks per K (or V) tile
  static constexpr int kLoads = kTile / kThreads;
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
};

// ROPE (launched for rope.on): q and k arrive rotated; dq is turned back before it is stored (the
// gradient with respect to the unrotated q).
// CUT (with EDGE, the split option): the cut may fall inside a tile, masked
// per element.
template <int D, int W, bool PREP, bool EDGE, bool SWAP, bool CUT, bool ROPE>
__global__ __launch_bounds__(64 * W, 8 / W) void s2attn_bwd_dq_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const bf16* __restrict__ o, const float* __restrict__ lse,
    float* __restrict__ lse2, float* __restrict__ dvec,
    bf16* __restrict__ dq, int N, int H, int Hkv, int G, int shift_heads, int split, float scale, RopeArgs rope) {
  using S = DqB16Shape<D, W>;
  constexpr int BR = S::kBR, BC = S::kBC, CPR = S::kCPR, TC = S::kTile;
  constexpr int RB = D * 2;
  // one LDS object per (stage, tensor), so reads of one stage are not made to
  // wait for the direct-to-LDS loads in flight into the other
  __shared__ bf16x8 k_st0[TC], v_st0[TC], k_st1[TC], v_st1[TC];
  auto kbuf = [&](int st) { return reinterpret_cast<char*>(st ? k_st1 : k_st0); };
  auto vbuf = [&](int st) { return reinterpret_cast<char*>(st ? v_st1 : v_st0); };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int g16 = lane >> 4, li = lane & 15, ts = li >> 2, tm = li & 3;

  const int groups = EDGE ? num_groups(N, G) : N / G;
  const int tiles_per_group = EDGE ? (G + BR - 1) / BR : G / BR;
  const TileOrder to = tile_order(blockIdx.x, gridDim.x / tiles_per_group, tiles_per_group);
  const int pos = tiles_per_group - 1 - to.rank;
  const int grp = to.pair % groups;
  const int h = (to.pair / groups) % H, b = to.pair / (groups * H);
  const int c = h / (H / Hkv);
  const int sigma = (h >= H - shift_heads) ? G / 2 : 0;
  const bool split_head = split && sigma != 0;
  const WrapGroup wg = wrap_group(N, G);
  const int ge = EDGE ? min(grp * G + G, N) : grp * G + G;   // end of the group
  const int j0 = grp * G + pos * BR;
  if (EDGE && j0 >= ge) return;                      // a tile past the end of a short group
  const int kv_begin = first_key_row(j0, G, split_head, wg);  // first key row any wave sees
  // CUT: the split option's cut may fall inside a tile (per-element mask)
  const int cut = CUT ? split_cut(grp * G, split_head, wg) : -1;
  const int ntiles = EDGE ? (min(j0 + BR, ge) - kv_begin + BC - 1) / BC : (j0 + BR - kv_begin) / BC;

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const bf16* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const bf16* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  const int jw = j0 + wave * 32;
  const int jq = jw + l32;
  const bool q_ok = !EDGE || jq < ge;                // EDGE: rows past the group read its last row
  const int tq = token_of_row<SWAP>(q_ok ? jq : ge - 1, sigma, N, wg);
  const int kw0 = first_key_row(jw, G, split_head, wg);       // this wave's first key
  bf16x8 qf[S::kDC], dof[S::kDC];
  {
    const bf16* qrow = q + ((size_t)b * N + tq) * qstride + (size_t)h * D;
    const bf16* dorow = dO + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) {
      qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + cc * 16 + hf * 8);
      dof[cc] = *reinterpret_cast<const bf16x8*>(dorow + cc * 16 + hf * 8);
    }
  }
  const size_t rix = ((size_t)b * H + h) * N + tq;
  float lse_q, dvec_q;
  bf16x8 oc[PREP ? S::kDC : 1];
  float lse_raw = 0.f;
  if constexpr (PREP) {
    const bf16* orow = o + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) oc[cc] = *reinterpret_cast<const bf16x8*>(orow + cc * 16 + hf * 8);
    lse_raw = lse[rix];
  }

  // Per-lane byte offsets, inside a 64-row tile, of the chunks this lane moves
  // (the host bounds 64 rows of K / V below 2^31 bytes)
  int toff[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int p = (wave + S::kWaves * i) * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    toff[i] = (row * (int)kvstride + (pc ^ swz2<CPR>(row)) * 8) * 2;
  }
  auto issue_tile = [&](int kt0, int stage) {
    char* kd = kbuf(stage);
    char* vd = vbuf(stage);
    // EDGE: a tile whose rows are not consecutive tokens (the wrap from token
    // N-1 to token 0, a break of the swap option's map, or row N inside it)
    // takes each row's own 64-bit address (rows past N read row N-1: masked keys)
    if (EDGE && !rows_contiguous<SWAP>(kt0, BC, sigma, N, wg)) {
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i) {
        const int p = (wave + S::kWaves * i) * 64 + lane;
        const int row = p / CPR, pc = p % CPR;
        const size_t tok = token_of_row<SWAP>(min(kt0 + row, N - 1), sigma, N, wg);
        const int cb = (wave + S::kWaves * i) * 64 * 16;
        const size_t off = tok * kvstride + (pc ^ swz2<CPR>(row)) * 8;
        load_lds16(kb + off, kd + cb);
        load_lds16(vb + off, vd + cb);
      }
      return;
    }
    // a whole tile is contiguous: buffers based at its first row
    const size_t t0 = token_of_row<SWAP>(kt0, sigma, N, wg);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(const_cast<bf16*>(kb + t0 * kvstride), BC * (int)kvstride * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(const_cast<bf16*>(vb + t0 * kvstride), BC * (int)kvstride * 2);
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int cb = (wave + S::kWaves * i) * 64 * 16;
      buffer_load_lds16(krs, toff[i], 0, kd + cb);
      buffer_load_lds16(vrs, toff[i], 0, vd + cb);
    }
  };


  // the first key / value tile is in flight while the prep arithmetic runs
  issue_tile(kv_begin, 0);
  if constexpr (PREP) {
    // Dvec = dO . O over this lane's half of the row, then the two halves
    float part = 0.f;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc)
#pragma unroll
      for (int i = 0; i < 8; ++i) part = fmaf((float)oc[cc][i], (float)dof[cc][i], part);
    dvec_q = sum_halves(part);
    lse_q = lse_raw * kLog2e;
    if (hf == 0 && q_ok) {
      dvec[rix] = -dvec_q;
      lse2[rix] = lse_q;
    }
  } else {
    lse_q = lse2[rix];
    dvec_q = -dvec[rix];
  }

  // per-lane LDS byte offsets: K / V A-operand rows perm32(l32) (+32 for the
  // second half of the tile); K^T transposing reads, rows 8hf + 4t + ts (+16 kc)
  const int krow = perm32(l32);
  int offA[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc) offA[cc] = krow * RB + (((2 * cc + hf) ^ swz2<CPR>(krow)) << 4);
  int offT[S::kDT][2];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = hf * 8 + 4 * t + ts;        // + 16 kc: swz2 only sees row bits 0..3
      const int dbase = dt * 32 + perm32(((g16 & 1) << 4) + 4 * tm);
      offT[dt][t] = row * RB + (((dbase >> 3) ^ swz2<CPR>(row)) << 4) + (dbase & 7) * 2;
    }

  f32x16 dqacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.f;
  const float c2 = scale * kLog2e;

  auto compute = [&](auto stg_c, auto mask_c, int kt0) {
    constexpr int STG = decltype(stg_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const char* Ks = kbuf(STG);
    const char* Vs = vbuf(STG);
    bf16x8 sf[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {             // one 32-key half at a time keeps S, dP small
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int cc = 0; cc < S::kDC; ++cc) {
        mma32(s, *reinterpret_cast<const bf16x8*>(Ks + offA[cc] + ks * 32 * RB), qf[cc]);
        mma32(dp, *reinterpret_cast<const bf16x8*>(Vs + offA[cc] + ks * 32 * RB), dof[cc]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x8 dsv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float p = fast_exp2(fmaf(s[u * 8 + i], c2, -lse_q));
          const int key = kt0 + ks * 32 + u * 16 + hf * 8 + i;
          if (MASK) {
            bool mk = key > jq;
            if (CUT) mk = mk | ((key < cut) & (jq >= cut));   // bitwise: no branch per element
            p = mk ? 0.f : p;
          }
          dsv[i] = p * (dp[u * 8 + i] - dvec_q);
        }
        sf[2 * ks + u] = __builtin_convertvector(dsv, bf16x8);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const char* p0 = Ks + offT[dt][0] + kc * 16 * RB;
        const char* p1 = Ks + offT[dt][1] + kc * 16 * RB;
        mma32(dqacc[dt], tr_read8(reinterpret_cast<const bf16*>(p0), reinterpret_cast<const bf16*>(p1)), sf[kc]);
      }
  };
  auto tile = [&](auto stg_c, int it) {
    constexpr int STG = decltype(stg_c)::value;
    const int kt0 = kv_begin + it * BC;
    wait_vmem_all();
    __syncthreads();
    if (it + 1 < ntiles) issue_tile(kt0 + BC, STG ^ 1);
    if (kt0 > jw + 31 || kt0 + BC <= kw0) return;   // tile after this wave's queries, or before its first key
    if (EDGE && jw >= ge) return;                // every query of this wave is past the group
    if (kt0 + BC - 1 > jw || (CUT && kt0 < cut && jw + 31 >= cut))
      compute(stg_c, std::integral_constant<bool, true>(), kt0);
    else
      compute(stg_c, std::integral_constant<bool, false>(), kt0);
  };

  for (int it = 0;;) {
    tile(std::integral_constant<int, 0>(), it);
    if (++it == ntiles) break;
    tile(std::integral_constant<int, 1>(), it);
    if (++it == ntiles) break;
  }

  if (!q_ok) return;
  bf16* dqrow = dq + ((size_t)b * N + tq) * qstride + (size_t)h * D;
  if (ROPE) {
    store_turned_back<D>(dqrow, dqacc, scale, (double)tq * rope.pos_scale, rope.log2_base, hf);
    return;
  }
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<bf16x8*>(dqrow + dt * 32 + u * 16 + hf * 8) = scale8<bf16>(dqacc[dt], u * 8, scale);
}

// ===========================================================================
// launchers
// ===========================================================================
template <typename T, int D>
hipError_t launch_bwd_prep(const void* o, const void* dO, const float* lse, float* dvec, float* lse2,
                           int B, int H, int N, hipStream_t stream) {
  const long long rows = (long long)B * N * H;
  constexpr int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((s2attn_bwd_pre<T, D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                     (const T*)o, (const T*)dO, lse, dvec, lse2, N, H, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_bf16_pass(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                                 const float* dvec, void* dk, void* dv, int B, int H, int Hkv, int N, int G,
                                 int shift_heads, int wrap, float scale, RopeArgs rope, hipStream_t stream, int pass,
                                 float* part) {
  using S = DkdvB16Shape<D>;
  constexpr int BKV = S::kBKV;
  const bool whole = N % G == 0 && G % BKV == 0;
  const dim3 grid(whole ? B * Hkv * (N / BKV) : B * Hkv * ((N + G - 1) / G) * ((G + BKV - 1) / BKV));
  const dim3 block(S::kThreads);
#define S2A_DKDV_LAUNCH_R(SPLIT, EDGE, SWAP, ROPE, PART)                                                       \
  hipLaunchKernelGGL((s2attn_bwd_dkdv_bf16<D, SPLIT, EDGE, SWAP, ROPE, PART>), grid, block, 0, stream,        \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, lse2, dvec, (bf16*)dk,   \
                     (bf16*)dv, N, H, Hkv, G, shift_heads, scale, rope, pass, part)
  // PART (the two-pass epilogue) is its own instantiation, so that the one-pass
  // kernels keep their register allocation
#define S2A_DKDV_LAUNCH(SPLIT, EDGE, SWAP)                                       \
  do {                                                                           \
    if (pass != 0 && rope.on) S2A_DKDV_LAUNCH_R(SPLIT, EDGE, SWAP, true, true);  \
    else if (pass != 0) S2A_DKDV_LAUNCH_R(SPLIT, EDGE, SWAP, false, true);       \
    else if (rope.on) S2A_DKDV_LAUNCH_R(SPLIT, EDGE, SWAP, true, false);         \
    else S2A_DKDV_LAUNCH_R(SPLIT, EDGE, SWAP, false, false);                     \
  } while (0)
  if (wrap == kWrapSplit) {
    if (whole) S2A_DKDV_LAUNCH(true, false, false); else S2A_DKDV_LAUNCH(true, true, false);
  } else if (wrap == kWrapSwap) {
    if (whole) S2A_DKDV_LAUNCH(false, false, true); else S2A_DKDV_LAUNCH(false, true, true);
  } else if (whole)
    S2A_DKDV_LAUNCH(false, false, false);
  else
    S2A_DKDV_LAUNCH(false, true, false);
#undef S2A_DKDV_LAUNCH
#undef S2A_DKDV_LAUNCH_R
  return hipGetLastError();
}

// part == NULL: one launch over every query head; else the two passes of
// dkdv_head_range, part holding the first pass's fp32 sums (2 B N Hkv D floats).
template <int D>
hipError_t launch_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                            const float* dvec, void* dk, void* dv, int B, int H, int Hkv, int N, int G,
                            int shift_heads, int wrap, float scale, RopeArgs rope, hipStream_t stream,
                            float* part = nullptr) {
  if (part) {
    const hipError_t e = launch_dkdv_bf16_pass<D>(q, k, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads,
                                                  wrap, scale, rope, stream, 1, part);
    if (e != hipSuccess) return e;
    return launch_dkdv_bf16_pass<D>(q, k, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads, wrap, scale,
                                    rope, stream, 2, part);
  }
  return launch_dkdv_bf16_pass<D>(q, k, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads, wrap, scale, rope,
                                  stream, 0, nullptr);
}

template <typename T, int D>
hipError_t launch_dkdv_generic(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                               const float* dvec, void* dk, void* dv, int B, int H, int Hkv, int N, int G,
                               int shift_heads, int wrap, float scale, hipStream_t stream, float* part) {
  using S = DkdvShape<T, D>;
  const dim3 grid(B * Hkv * ((N + G - 1) / G) * ((G + S::kBKV - 1) / S::kBKV));
  for (int pass = part ? 1 : 0; pass <= (part ? 2 : 0); ++pass) {
    hipLaunchKernelGGL((s2attn_bwd_dkdv<T, D>), grid, dim3(S::kThreads), 0,
                       stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, lse2, dvec, (T*)dk, (T*)dv, N,
                       H, Hkv, G, shift_heads, wrap, scale, pass, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                           const float* dvec, void* dk, void* dv, int B, int H, int Hkv, int N, int G,
                           int shift_heads, int wrap, hipStream_t stream, float* part) {
  const float scale = 1.0f / sqrtf((float)D);
  if constexpr (std::is_same_v<T, bf16>)
    return launch_dkdv_bf16<D>(q, k, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads, wrap, scale,
                               RopeArgs{nullptr, 0, 0, 0}, stream, part);
  else
    return launch_dkdv_generic<T, D>(q, k, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads, wrap, scale,
                                     stream, part);
}

// Wave count of a dq launch: as the forward's (8 waves for whole 256-row
// tiles and long groups, 4 for short groups that are not whole tiles).
inline int dq_waves(int N, int G) {
  const bool whole = N % G == 0 && G % 256 == 0;
  return (!whole && G % 256 != 0 && G < 4096) ? 4 : 8;
}

template <int D, int W>
hipError_t launch_dq_bf16_w(const void* q, const void* k, const void* v, const void* dO, const void* o,
                            const float* lse, float* lse2, float* dvec, void* dq, int B, int H, int Hkv, int N,
                            int G, int shift_heads, int wrap, float scale, hipStream_t stream, RopeArgs rope) {
  using S = DqB16Shape<D, W>;
  constexpr int BR = S::kBR;
  const bool whole = N % G == 0 && G % BR == 0;
  const dim3 grid(whole ? B * H * (N / BR) : B * H * ((N + G - 1) / G) * ((G + BR - 1) / BR)), block(S::kThreads);
  const bf16* ob = (const bf16*)o;
#define S2A_DQ_LAUNCH(PREP, EDGE, SWAP, CUT, ROPE)                                                            \
  hipLaunchKernelGGL((s2attn_bwd_dq_bf16<D, W, PREP, EDGE, SWAP, CUT, ROPE>), grid, block, 0, stream,       \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, ob, lse, lse2, dvec,    \
                     (bf16*)dq, N, H, Hkv, G, shift_heads, (int)(wrap == kWrapSplit), scale, rope)
  // the rotary route runs with the prep fused in (s2attn_bwd_rope)
#define S2A_DQ_LAUNCH_P(EDGE, SWAP, CUT)                       \
  do {                                                         \
    if (o && rope.on) S2A_DQ_LAUNCH(true, EDGE, SWAP, CUT, true); \
    else if (o) S2A_DQ_LAUNCH(true, EDGE, SWAP, CUT, false);   \
    else S2A_DQ_LAUNCH(false, EDGE, SWAP, CUT, false);         \
  } while (0)
  if constexpr (W == 8) {
    if (whole) {
      if (wrap == kWrapSwap) S2A_DQ_LAUNCH_P(false, true, false);
      else S2A_DQ_LAUNCH_P(false, false, false);
      return hipGetLastError();
    }
  }
  if (wrap == kWrapSwap) S2A_DQ_LAUNCH_P(true, true, false);
  else if (wrap == kWrapSplit) S2A_DQ_LAUNCH_P(true, false, true);
  else S2A_DQ_LAUNCH_P(true, false, false);
#undef S2A_DQ_LAUNCH_P
#undef S2A_DQ_LAUNCH
  return hipGetLastError();
}

// o and lse non-NULL: prep fused in (writes lse2 and dvec); else reads them.
template <int D>
hipError_t launch_dq_bf16(const void* q, const void* k, const void* v, const void* dO, const void* o,
                          const float* lse, float* lse2, float* dvec, void* dq, int B, int H, int Hkv, int N, int G,
                          int shift_heads, int wrap, float scale, hipStream_t stream,
                          RopeArgs rope = RopeArgs{nullptr, 0, 0, 0}) {
  return dq_waves(N, G) == 4 ? launch_dq_bf16_w<D, 4>(q, k, v, dO, o, lse, lse2, dvec, dq, B, H, Hkv, N, G,
                                                      shift_heads, wrap, scale, stream, rope)
                             : launch_dq_bf16_w<D, 8>(q, k, v, dO, o, lse, lse2, dvec, dq, B, H, Hkv, N, G,
                                                      shift_heads, wrap, scale, stream, rope);
}

template <typename T, int D>
hipError_t launch_dq_generic(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                             const float* dvec, void* dq, int B, int H, int Hkv, int N, int G, int shift_heads,
                             int wrap, float scale, hipStream_t stream) {
  using S = DqShape<T, D>;
  const dim3 grid(B * H * ((N + G - 1) / G) * ((G + S::kBR - 1) / S::kBR));
  hipLaunchKernelGGL((s2attn_bwd_dq<T, D>), grid, dim3(S::kThreads), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dO, lse2, dvec, (T*)dq, N, H, Hkv, G,
                     shift_heads, wrap, scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                         const float* dvec, void* dq, int B, int H, int Hkv, int N, int G, int shift_heads,
                         int wrap, hipStream_t stream) {
  const float scale = 1.0f / sqrtf((float)D);
  if constexpr (std::is_same_v<T, bf16>)
    return launch_dq_bf16<D>(q, k, v, dO, nullptr, nullptr, const_cast<float*>(lse2), const_cast<float*>(dvec),
                             dq, B, H, Hkv, N, G, shift_heads, wrap, scale, stream);
  else
    return launch_dq_generic<T, D>(q, k, v, dO, lse2, dvec, dq, B, H, Hkv, N, G, shift_heads, wrap, scale, stream);
}

// prep and dq: one launch for bf16 (prep fused into the dq kernel), prep then
// dq for fp32
template <typename T, int D>
hipError_t launch_bwd_prep_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, float* lse2, float* dvec, void* dq, int B, int H, int Hkv, int N,
                              int G, int shift_heads, int wrap, hipStream_t stream) {
  if constexpr (std::is_same_v<T, bf16>) {
    return launch_dq_bf16<D>(q, k, v, dO, o, lse, lse2, dvec, dq, B, H, Hkv, N, G, shift_heads, wrap,
                             1.0f / sqrtf((float)D), stream);
  } else {
    const hipError_t e = launch_bwd_prep<T, D>(o, dO, lse, dvec, lse2, B, H, N, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq<T, D>(q, k, v, dO, lse2, dvec, dq, B, H, Hkv, N, G, shift_heads, wrap, stream);
  }
}

// The backward with the rotary embedding fused (bf16): q_rot and k_rot are the
// rotated inputs the forward used; dq and dk come out turned back, i.e. with
// respect to the unrotated q and k.  Prep + dq in one launch, then dK/dV.
template <int D>
hipError_t launch_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o, const float* lse,
                           const void* dO, float* lse2, float* dvec, void* dq, void* dk, void* dv, int B, int H,
                           int Hkv, int N, int G, int shift_heads, int wrap, double pos_scale, double log2_base,
                           hipStream_t stream, float* part) {
  const float scale = 1.0f / sqrtf((float)D);
  const RopeArgs rope{nullptr, pos_scale, log2_base, 1};
  const hipError_t e = launch_dq_bf16<D>(q_rot, k_rot, v, dO, o, lse, lse2, dvec, dq, B, H, Hkv, N, G, shift_heads,
                                         wrap, scale, stream, rope);
  if (e != hipSuccess) return e;
  return launch_dkdv_bf16<D>(q_rot, k_rot, v, dO, lse2, dvec, dk, dv, B, H, Hkv, N, G, shift_heads, wrap, scale,
                             rope, stream, part);
}
template hipError_t launch_bwd_rope<64>(const void*, const void*, const void*, const void*, const float*, const void*,
                                        float*, float*, void*, void*, void*, int, int, int, int, int, int, int, double,
                                        double, hipStream_t, float*);
template hipError_t launch_bwd_rope<128>(const void*, const void*, const void*, const void*, const float*,
                                         const void*, float*, float*, void*, void*, void*, int, int, int, int, int, int,
                                         int, double, double, hipStream_t, float*);

#define S2A_INST_BWD(T, D)                                                                                 \
  template hipError_t launch_bwd_prep<T, D>(const void*, const void*, const float*, float*, float*, int,  \
                                            int, int, hipStream_t);                                        \
  template hipError_t launch_bwd_dkdv<T, D>(const void*, const void*, const void*, const void*,           \
                                            const float*, const float*, void*, void*, int, int, int, int,  \
                                            int, int, int, hipStream_t, float*);                           \
  template hipError_t launch_bwd_dq<T, D>(const void*, const void*, const void*, const void*, const float*, \
                                          const float*, void*, int, int, int, int, int, int, int, hipStream_t); \
  template hipError_t launch_bwd_prep_dq<T, D>(const void*, const void*, const void*, const void*,           \
                                               const float*, const void*, float*, float*, void*, int, int, int, \
                                               int, int, int, int, hipStream_t);
S2A_INST_BWD(bf16, 64)
S2A_INST_BWD(bf16, 128)
S2A_INST_BWD(float, 64)
S2A_INST_BWD(float, 128)

}  // namespace s2a
