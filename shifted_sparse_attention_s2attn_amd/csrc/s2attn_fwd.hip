// S2-Attn forward kernel for gfx950.
//
// Method: page "LongLoRA: Efficient Fine-tuning of Long-Context Large Language
// Models", section 3.4 ("The core computational problem", "The solution: group
// tokens and compute attention locally", "The shifting mechanism" Steps 1-3,
// "Algorithmic implementation" / Algorithm 1).  Each (batch, head, group) is an
// independent causal attention over G tokens; heads h >= H - shift_heads read
// their tokens rolled by G/2, so rolled row j is original token (j + G/2) mod N,
// and write their outputs back at the original rows (the roll-back).
// Wrap options of the shifted heads' last rolled group (Table 8 / Figure 6):
// split (Variant 2) cuts it at G/2, so its second-half queries start at key G/2
// of the group; swap (Variant 3) puts the tokens carried from the front first
// (a different row -> token map for that group, token_of_row).
//
// One workgroup = 4 waves = 128 consecutive query rows (rolled frame) of one
// (batch, head).  Each wave owns 32 query rows; its Q operand stays in
// registers.  Key/value tiles of 64 rows stream through LDS (K row-major,
// V transposed), with the next tile's global loads issued before the current
// tile is computed.  Per tile and wave:
//     S^T = K Q^T        (keys on the tile rows, the wave's 32 queries on lanes)
//     causal mask on the diagonal tiles, online softmax (one query per lane,
//     its 32 keys split across lanes l and l ^ 32)
//     O^T += V^T P^T     (P^T comes straight from the S^T registers)
// Finally O = O^T / l is stored at the original rows with lse = m + ln l.
// This kernel (fp32 inputs: fp32 matrix cores) also takes groups that are not
// whole tiles (a short last group when G does not divide N, or any G): query
// rows past the group compute on a copy of its last row and are not stored, key
// rows past it (the next group, or past N, clamped to a real row) follow every
// query of the group and are masked.
#include "s2attn_common.h"

#include <type_traits>

namespace s2a {

template <typename T, int D>
struct FwdShape {
  static constexpr int kThreads = 256;
  static constexpr int kBR = 128;               // query rows per workgroup
  static constexpr int kBC = 64;                // key rows per tile
  static constexpr int kKCPR = D / 8;           // chunks per K row
  static constexpr int kVCPR = kBC / 8;         // chunks per transposed V row
  static constexpr int kKChunksPerThread = kBC * kKCPR / kThreads;
  static constexpr int kVKeysPerThread = kBC * D / 8 / kThreads;
  static constexpr int kDC = D / 16;            // k-steps over the head dim
  static constexpr int kDT = D / 32;            // 32-wide output tiles over the head dim
  static constexpr int kKS = kBC / 32;          // 32-key score tiles per key tile
};

template <typename T, int N_>
struct alignas(sizeof(T) * N_) PackN { T x[N_]; };

template <typename T, int D>
__global__ __launch_bounds__(256) void s2attn_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ o, float* __restrict__ lse,
    int N, int H, int Hkv, int G, int shift_heads, int wrap, float scale) {
  using S = FwdShape<T, D>;
  constexpr int BR = S::kBR, BC = S::kBC, KCPR = S::kKCPR, VCPR = S::kVCPR;
  constexpr int KPT = S::kKChunksPerThread, VKPT = S::kVKeysPerThread;
  __shared__ v8<T> Ks[BC * KCPR];
  __shared__ v8<T> Vt[D * VCPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // Heaviest query tiles (last in their group) are dispatched first.
  const int groups = num_groups(N, G), tiles_per_group = (G + BR - 1) / BR;
  const TileOrder to = tile_order(blockIdx.x, gridDim.x / tiles_per_group, tiles_per_group);
  const int pos = tiles_per_group - 1 - to.rank;
  const int grp = to.pair % groups;
  const int h = (to.pair / groups) % H, b = to.pair / (groups * H);
  const int c = h / (H / Hkv);
  const int sigma = (h >= H - shift_heads) ? G / 2 : 0;

  const bool split_head = wrap == kWrapSplit && sigma != 0;
  const bool swap_head = wrap == kWrapSwap && sigma != 0;
  const WrapGroup wg = wrap_group(N, G);
  auto tok = [&](int j) { return swap_head ? token_of_row<true>(j, sigma, N, wg) : orig_row(j, sigma, N); };
  const int ge = min(grp * G + G, N);           // end of the group (a last group may be short)
  const int j0 = grp * G + pos * BR;            // first query row (rolled)
  if (j0 >= ge) return;                         // a tile past the end of a short group
  const int kv_begin = first_key_row(j0, G, split_head, wg);  // first key row any wave sees
  const int cut = split_cut(grp * G, split_head, wg);         // split option: rows from here see no key before
  const int ntiles = (min(j0 + BR, ge) - kv_begin + BC - 1) / BC;

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const T* qb = q + (size_t)b * N * qstride + (size_t)h * D;
  const T* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const T* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // ---- Q operand (B of S^T = K Q^T): query (l32), 8 head-dim values per k-step
  const int jw = j0 + wave * 32;                // wave's first query (rolled)
  const int jq = jw + l32;                      // this lane's query (rolled)
  const bool q_ok = jq < ge;                    // rows past the group compute on a copy, are not stored
  const int tq = tok(q_ok ? jq : ge - 1);
  const int kw0 = first_key_row(jw, G, split_head, wg);       // ... and this wave's first key
  v8<T> qf[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc)
    qf[cc] = *reinterpret_cast<const v8<T>*>(qb + (size_t)tq * qstride + cc * 16 + hf * 8);

  // ---- key / value tile staging: global -> registers -> LDS
  v8<T> kreg[KPT];
  v8<T> vreg[VKPT];
  const int v_dc = tid % (D / 8);               // head-dim chunk this thread transposes
  const int v_kg = tid / (D / 8);               // key group (VKPT keys)

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ci = tid + i * 256;
      const int row = ci / KCPR, cc = ci % KCPR;
      const int t = tok(min(kt0 + row, N - 1));   // rows past N are masked keys
      kreg[i] = *reinterpret_cast<const v8<T>*>(kb + (size_t)t * kvstride + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < VKPT; ++i) {
      const int t = tok(min(kt0 + v_kg * VKPT + i, N - 1));
      vreg[i] = *reinterpret_cast<const v8<T>*>(vb + (size_t)t * kvstride + v_dc * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ci = tid + i * 256;
      const int row = ci / KCPR, cc = ci % KCPR;
      Ks[chunk_at<KCPR>(row, cc)] = kreg[i];
    }
    // V transposed: row = head-dim index, VKPT consecutive keys per write
    const int kcol = v_kg * VKPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = v_dc * 8 + e;
      PackN<T, VKPT> pk;
#pragma unroll
      for (int i = 0; i < VKPT; ++i) pk.x[i] = vreg[i][e];
      T* rowp = reinterpret_cast<T*>(&Vt[chunk_at<VCPR>(d, kcol / 8)]);
      *reinterpret_cast<PackN<T, VKPT>*>(rowp + (kcol % 8)) = pk;
    }
  };

  f32x16 oacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = scale * kLog2e;

  load_tile(kv_begin);
  for (int it = 0; it < ntiles; ++it) {
    const int kt0 = kv_begin + it * BC;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(kt0 + BC);

    if (kt0 > jw + 31 || kt0 + BC <= kw0 || jw >= ge) continue;   // nothing of this tile for this wave
    const bool need_mask = kt0 + BC - 1 > jw || (kt0 < cut && jw + 31 >= cut);

    // S^T = K Q^T
    f32x16 s[S::kKS];
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ks][r] = 0.f;
      const int row = ks * 32 + perm32(l32);
#pragma unroll
      for (int cc = 0; cc < S::kDC; ++cc) mma32(s[ks], Ks[chunk_at<KCPR>(row, cc * 2 + hf)], qf[cc]);
    }

    // causal mask + online softmax (raw scores; the scale is folded into exp2)
    float mloc = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (need_mask) {
          const int key = kt0 + ks * 32 + (r >> 3) * 16 + hf * 8 + (r & 7);
          if (key > jq || (key < cut && jq >= cut)) s[ks][r] = -INFINITY;
        }
        mloc = fmaxf(mloc, s[ks][r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // m_new stays -inf for a row behind the split cut whose keys so far are all
    // masked: then nothing is accumulated (alpha 0) and its p are 0
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * c2);
    const float nm = m_new == -INFINITY ? 0.f : -m_new * c2;
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[ks][r], c2, nm));
        s[ks][r] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

    // O^T += V^T P^T : 16 keys per k-step, P^T from the S^T registers
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      const v8<T> pf = pack8<T>(s[kc >> 1], (kc & 1) * 8);
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const int row = dt * 32 + perm32(l32);
        mma32(oacc[dt], Vt[chunk_at<VCPR>(row, kc * 2 + hf)], pf);
      }
    }
  }

  // ---- epilogue: normalise, store O and lse at the original row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) return;
  const float inv = 1.f / l_tot;
  T* orow = o + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<v8<T>*>(orow + dt * 32 + u * 16 + hf * 8) = scale8<T>(oacc[dt], u * 8, inv);
  if (hf == 0) lse[((size_t)b * H + h) * N + tq] = m_run * scale + logf(l_tot);
}

// ---------------------------------------------------------------------------
// bf16 forward (any G: whole 256-row query tiles of whole groups, or the EDGE
// instantiation below).
//
// W waves share each 64-row key/value tile; each wave owns 32 query rows, so a
// workgroup covers 32 W query rows.  W = 8 (256 rows, one workgroup and two
// waves per SIMD, so one wave's matrix-core work overlaps another's softmax)
// except for short groups that are not whole tiles, which take W = 4 (128
// rows, two workgroups per CU).  Key and value tiles go from HBM straight into
// LDS (buffer loads to LDS, no register staging), double-buffered with one
// barrier per tile, each through a buffer descriptor based at its first row;
// a tile whose rows are not consecutive tokens (EDGE) is loaded row by row.
// V stays row-major in LDS: the V^T operand is read with ds_read_b64_tr_b16,
// whose 16-lane groups return 4 consecutive keys of one head-dim column.
// The running max is only raised when a tile exceeds it by more than 2^8 (in
// exp2 units), so the accumulator is rarely rescaled; P stays <= 256.
// Row sums are taken on the bf16 P actually fed to the matrix cores.
// ---------------------------------------------------------------------------
template <int D, int W = 8>
struct FwdB16Shape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kBR = 32 * W;
  static constexpr int kBC = 64;
  static constexpr int kCPR = D / 8;                      // 16-byte chunks per tile row
  static constexpr int kTileChunks = kBC * kCPR;
  static constexpr int kLoads = kTileChunks / kThreads;   // chunks per thread per tensor
  static constexpr int kDC = D / 16;
  static constexpr int kDT = D / 32;
};

// XOR swizzles of the 16-byte chunk column.  K: the 16 rows perm32(0..15) read
// together by an A-operand load get distinct columns.  V: the 4 rows read by
// one 16-lane transpose read (4 consecutive keys) get disjoint column pairs.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  return CPR == 16 ? ((row & 3) | ((row >> 1) & 4) | ((row << 1) & 8)) : ((row & 3) | ((row >> 1) & 4));
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row) {
  return CPR == 16 ? ((4 * (row & 3)) ^ (2 * ((row >> 1) & 1))) : (2 * (row & 3));
}

// EDGE: groups that are not whole tiles (a short last group, any G): query
// rows past the group compute on a copy of its last row and are not stored,
// key rows past it follow every query of the group and are masked, and a key
// tile that crosses the roll's wrap point (or the end of the sequence) is
// loaded with per-row addresses.  Compiled separately from the whole-tile case.
// SWAP: the swap wrap option's row map (token_of_row); `split` is 1 for the
// split option.
// ROPE (launched for rope.on): q arrives unrotated; the kernel turns its Q rows by the rotary
// embedding with Position Interpolation (k arrives rotated) and, after its
// key loop, writes the rotated rows to rope.q_rot for the backward.
// CUT (with EDGE, the split option): the cut may fall inside a tile, masked
// per element.
template <int D, int W, bool EDGE, bool SWAP, bool CUT, bool ROPE>
__global__ __launch_bounds__(64 * W, 8 / W) void s2attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse,
    int N, int H, int Hkv, int G, int shift_heads, int split, float scale, RopeArgs rope) {
  using S = FwdB16Shape<D, W>;
  constexpr int BR = S::kBR, BC = S::kBC, CPR = S::kCPR, TC = S::kTileChunks;
  constexpr int RB = D * 2;                       // bytes per tile row
  // one LDS object per (stage, tensor): the compiler then sees that reads of one
  // stage do not alias the direct-to-LDS loads in flight into the other, and
  // does not wait for those loads before reading
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
  const int pos = tiles_per_group - 1 - to.rank;     // heaviest query tiles first
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
  // CUT: the split option's cut may fall inside a tile; query rows at or
  // after it see no key row before it (per element)
  const int cut = CUT ? split_cut(grp * G, split_head, wg) : -1;
  const int ntiles = EDGE ? (min(j0 + BR, ge) - kv_begin + BC - 1) / BC : (j0 + BR - kv_begin) / BC;

  const size_t qstride = (size_t)H * D, kvstride = (size_t)Hkv * D;
  const bf16* kb = k + (size_t)b * N * kvstride + (size_t)c * D;
  const bf16* vb = v + (size_t)b * N * kvstride + (size_t)c * D;

  // Q operand in registers (EDGE: rows past the group read its last row)
  const int jw = j0 + wave * 32;
  const int jq = jw + l32;
  const bool q_ok = !EDGE || jq < ge;
  const int tq = token_of_row<SWAP>(q_ok ? jq : ge - 1, sigma, N, wg);
  const int kw0 = first_key_row(jw, G, split_head, wg);       // this wave's first key
  bf16x8 qf[S::kDC];
  {
    const bf16* qrow = q + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + cc * 16 + hf * 8);
  }
  // Per-lane byte offsets, inside a 64-row tile, of the chunks this lane moves
  // (the host bounds 64 rows of K / V below 2^31 bytes)
  int koff[S::kLoads], voff[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int p = (wave + S::kWaves * i) * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    koff[i] = (row * (int)kvstride + (pc ^ swz_k<CPR>(row)) * 8) * 2;
    voff[i] = (row * (int)kvstride + (pc ^ swz_v<CPR>(row)) * 8) * 2;
  }
  auto issue_tile = [&](int kt0, int stage) {
    char* kd = kbuf(stage);
    char* vd = vbuf(stage);
    // EDGE: a tile whose rows are not consecutive tokens (it crosses the wrap
    // from token N-1 to token 0, a break of the swap option's map, or row N)
    // takes each row's own 64-bit address (rows past N read row N-1: masked keys)
    if (EDGE && !rows_contiguous<SWAP>(kt0, BC, sigma, N, wg)) {
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i) {
        const int p = (wave + S::kWaves * i) * 64 + lane;
        const int row = p / CPR, pc = p % CPR;
        const size_t tok = token_of_row<SWAP>(min(kt0 + row, N - 1), sigma, N, wg);
        const int cb = (wave + S::kWaves * i) * 64 * 16;
        load_lds16(kb + tok * kvstride + (pc ^ swz_k<CPR>(row)) * 8, kd + cb);
        load_lds16(vb + tok * kvstride + (pc ^ swz_v<CPR>(row)) * 8, vd + cb);
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
      buffer_load_lds16(krs, koff[i], 0, kd + cb);
      buffer_load_lds16(vrs, voff[i], 0, vd + cb);
    }
  };

  // per-lane LDS byte offsets: K A-operand rows perm32(l32) (+32 rows for the
  // second 32-key half), V^T transposing reads (rows 8hf + 4t + ts (+16 kc))
  const int krow = perm32(l32);
  int offK[S::kDC];
#pragma unroll
  for (int cc = 0; cc < S::kDC; ++cc) offK[cc] = krow * RB + (((2 * cc + hf) ^ swz_k<CPR>(krow)) << 4);
  int offV[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt) {
    const int row = hf * 8 + ts;                  // + 4t + 16kc: swz_v only sees row & 3 and bit 1
    const int dbase = dt * 32 + perm32(((g16 & 1) << 4) + 4 * tm);
    offV[dt] = row * RB + (((dbase >> 3) ^ swz_v<CPR>(row)) << 4) + (dbase & 7) * 2;
  }

  f32x16 oacc[S::kDT];
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = scale * kLog2e;

  auto compute = [&](auto stg_c, auto mask_c, int kt0) {
    constexpr int STG = decltype(stg_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const char* st = kbuf(STG);
    const char* vst = vbuf(STG);

    // S^T = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ks][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < S::kDC; ++cc)
        mma32(s[ks], *reinterpret_cast<const bf16x8*>(st + offK[cc] + ks * 32 * RB), qf[cc]);
    }
    if (MASK) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + ks * 32 + (r >> 3) * 16 + hf * 8 + (r & 7);
          bool mk = key > jq;
          if (CUT) mk = mk | ((key < cut) & (jq >= cut));   // bitwise: no branch per element
          s[ks][r] = mk ? -INFINITY : s[ks][r];
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[ks][r]);
    mloc = max_halves(mloc);
    if (wave_any((mloc - m_run) * c2 > 8.f)) {
      const float m_new = fmaxf(m_run, mloc);
      // (CUT: m_run = -inf means nothing accumulated yet; scaling by 0 avoids -inf - -inf)
      const float alpha = (CUT && m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = m_new;
    }
    // CUT: a row behind the split cut may meet only masked keys in its first
    // tiles (m_run still -inf): its p are 0 until its first key
    const float nm = (CUT && m_run == -INFINITY) ? 0.f : -m_run * c2;
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      f32x8 pv;
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(fmaf(s[kc >> 1][(kc & 1) * 8 + i], c2, nm));
      pf[kc] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run = dot2_bf16_acc(pf[kc][2 * i], pf[kc][2 * i + 1], l_run);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int dt = 0; dt < S::kDT; ++dt) {
        const char* p0 = vst + offV[dt] + kc * 16 * RB;
        mma32(oacc[dt], tr_read8(reinterpret_cast<const bf16*>(p0), reinterpret_cast<const bf16*>(p0 + 4 * RB)),
              pf[kc]);
      }
  };
  auto tile = [&](auto stg_c, int it) {
    constexpr int STG = decltype(stg_c)::value;
    const int kt0 = kv_begin + it * BC;
    wait_vmem_all();                             // this lane's tile loads have landed
    __syncthreads();                             // ... and everyone's; the other stage is free
    if (it + 1 < ntiles) issue_tile(kt0 + BC, STG ^ 1);
    if (kt0 > jw + 31 || kt0 + BC <= kw0) return;   // tile after this wave's queries, or before its first key
    if (EDGE && jw >= ge) return;                // every query of this wave is past the group
    if (kt0 + BC - 1 > jw || (CUT && kt0 < cut && jw + 31 >= cut))
      compute(stg_c, std::integral_constant<bool, true>(), kt0);
    else
      compute(stg_c, std::integral_constant<bool, false>(), kt0);
  };

  issue_tile(kv_begin, 0);
  if (ROPE) {
    // (after the first tile is issued, so its loads fly while the rows turn)
    // element i < D/2 of the row sits in chunk i / 16 and its partner i + D/2 in
    // chunk i / 16 + D/32 of the same lane: the rotation is lane-local
    const double pos = (double)tq * rope.pos_scale;
#pragma unroll
    for (int cc = 0; cc < S::kDC / 2; ++cc) {
      bf16x8 ya, yb;
      double g[8];
      rope_revs8<D>(cc * 16 + hf * 8, rope.log2_base, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn, y0, y1;
        rope_cs(pos, g[e], cs, sn);
        rope_turn((float)qf[cc][e], (float)qf[cc + S::kDC / 2][e], cs, sn, y0, y1);
        ya[e] = (bf16)y0;
        yb[e] = (bf16)y1;
      }
      qf[cc] = ya;
      qf[cc + S::kDC / 2] = yb;
    }
  }

  for (int it = 0;;) {
    tile(std::integral_constant<int, 0>(), it);
    if (++it == ntiles) break;
    tile(std::integral_constant<int, 1>(), it);
    if (++it == ntiles) break;
  }

  const float l_tot = sum_halves(l_run);
  if (!q_ok) return;
  if (ROPE) {
    // the rotated rows for the backward, written here rather than before the
    // loop, where the stores would compete with the first tiles' loads
    bf16* qr = rope.q_rot + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
    for (int cc = 0; cc < S::kDC; ++cc) *reinterpret_cast<bf16x8*>(qr + cc * 16 + hf * 8) = qf[cc];
  }
  const float inv = 1.f / l_tot;
  bf16* orow = o + ((size_t)b * N + tq) * qstride + (size_t)h * D;
#pragma unroll
  for (int dt = 0; dt < S::kDT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<bf16x8*>(orow + dt * 32 + u * 16 + hf * 8) = scale8<bf16>(oacc[dt], u * 8, inv);
  if (hf == 0) lse[((size_t)b * H + h) * N + tq] = m_run * scale + logf(l_tot);
}

// Wave count of a launch.  Whole tiles of whole groups: 8 waves (256 query
// rows: each K/V tile serves twice as many queries as with 4).  Groups that
// are not whole 256-row tiles and shorter than 4096 rows: 4 waves (128 rows,
// two workgroups per CU), so less of each group's partial tile and diagonal
// block sits idle.
inline int fwd_waves(int N, int G) {
  const bool whole = N % G == 0 && G % 256 == 0;
  return (!whole && G % 256 != 0 && G < 4096) ? 4 : 8;
}

template <int D, int W>
hipError_t launch_fwd_bf16_w(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Hkv, int N, int G, int shift_heads, int wrap, float scale,
                             RopeArgs rope, hipStream_t stream) {
  constexpr int BR = FwdB16Shape<D, W>::kBR;
  const dim3 block(FwdB16Shape<D, W>::kThreads);
  const bool whole = N % G == 0 && G % BR == 0;
  const dim3 grid(whole ? B * H * (N / BR) : B * H * ((N + G - 1) / G) * ((G + BR - 1) / BR));
#define S2A_FWD_LAUNCH_R(EDGE, SWAP, CUT, ROPE)                                                                \
  hipLaunchKernelGGL((s2attn_fwd_bf16_kernel<D, W, EDGE, SWAP, CUT, ROPE>), grid, block, 0, stream,           \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, H, Hkv, G, shift_heads, \
                     (int)(wrap == kWrapSplit), scale, rope)
#define S2A_FWD_LAUNCH(EDGE, SWAP, CUT)        \
  do {                                         \
    if (rope.on) S2A_FWD_LAUNCH_R(EDGE, SWAP, CUT, true); \
    else S2A_FWD_LAUNCH_R(EDGE, SWAP, CUT, false);        \
  } while (0)
  if constexpr (W == 8) {
    if (whole) {
      if (wrap == kWrapSwap) S2A_FWD_LAUNCH(false, true, false);
      else S2A_FWD_LAUNCH(false, false, false);
      return hipGetLastError();
    }
  }
  if (wrap == kWrapSwap) S2A_FWD_LAUNCH(true, true, false);
  else if (wrap == kWrapSplit) S2A_FWD_LAUNCH(true, false, true);
  else S2A_FWD_LAUNCH(true, false, false);
#undef S2A_FWD_LAUNCH
#undef S2A_FWD_LAUNCH_R
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int N, int G, int shift_heads, int wrap, float scale,
                           RopeArgs rope, hipStream_t stream) {
  return fwd_waves(N, G) == 4
             ? launch_fwd_bf16_w<D, 4>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, scale, rope, stream)
             : launch_fwd_bf16_w<D, 8>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, scale, rope, stream);
}

// bf16: the kernel above at every size; fp32: the fp32 kernel.
template <typename T, int D>
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int N, int G, int shift_heads, int wrap, hipStream_t stream) {
  const float scale = 1.0f / sqrtf((float)D);
  if constexpr (std::is_same_v<T, bf16>) {
    return launch_fwd_bf16<D>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, scale, RopeArgs{nullptr, 0, 0, 0},
                              stream);
  } else {
    constexpr int BR = FwdShape<T, D>::kBR;
    dim3 grid(B * H * ((N + G - 1) / G) * ((G + BR - 1) / BR));
    hipLaunchKernelGGL((s2attn_fwd_kernel<T, D>), grid, dim3(256), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, N, H, Hkv, G, shift_heads, wrap, scale);
    return hipGetLastError();
  }
}

// bf16 with the rotary embedding fused: q unrotated, k rotated; writes q_rot.
template <int D>
hipError_t launch_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* q_rot,
                           int B, int H, int Hkv, int N, int G, int shift_heads, int wrap, double pos_scale,
                           double log2_base, hipStream_t stream) {
  return launch_fwd_bf16<D>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, 1.0f / sqrtf((float)D),
                            RopeArgs{(bf16*)q_rot, pos_scale, log2_base, 1}, stream);
}
template hipError_t launch_fwd_rope<64>(const void*, const void*, const void*, void*, float*, void*, int, int, int,
                                        int, int, int, int, double, double, hipStream_t);
template hipError_t launch_fwd_rope<128>(const void*, const void*, const void*, void*, float*, void*, int, int, int,
                                         int, int, int, int, double, double, hipStream_t);

template hipError_t launch_fwd<bf16, 64>(const void*, const void*, const void*, void*, float*, int, int, int, int, int, int, int, hipStream_t);
template hipError_t launch_fwd<bf16, 128>(const void*, const void*, const void*, void*, float*, int, int, int, int, int, int, int, hipStream_t);
template hipError_t launch_fwd<float, 64>(const void*, const void*, const void*, void*, float*, int, int, int, int, int, int, int, hipStream_t);
template hipError_t launch_fwd<float, 128>(const void*, const void*, const void*, void*, float*, int, int, int, int, int, int, int, hipStream_t);

}  // namespace s2a
