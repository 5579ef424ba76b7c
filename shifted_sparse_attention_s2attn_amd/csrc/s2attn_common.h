// Device helpers shared by the S2-Attn kernels (gfx950 / CDNA4).
//
// Matrix-core convention used everywhere: one wave (64 lanes) computes a 32x32
// fp32 tile C += A (32 x 16) * B (16 x 32) per step.
//   A operand: lane l holds row (l & 31), k-slots 8*(l >> 5) .. +7
//   B operand: lane l holds col (l & 31), k-slots 8*(l >> 5) .. +7
//   C tile   : lane l holds col (l & 31); register r holds
//              row 8*(r >> 2) + 4*(l >> 5) + (r & 3)
// bf16 issues one v_mfma_f32_32x32x16_bf16; fp32 issues eight
// v_mfma_f32_32x32x2_f32, the i-th one consuming k-slot 8*(l >> 5) + i.
//
// When the rows of A are loaded in the order perm32(row) (bits 2 and 3 of the
// row index swapped), register r of C holds row
//     16*(r >> 3) + 8*(l >> 5) + (r & 7),
// so registers 0..7 and 8..15 of a lane are two runs of 8 consecutive rows.
// That run is exactly the k-slot layout of the next product's B operand, which
// lets a softmax tile feed the following matrix product straight from
// registers, and lets epilogues store 8 consecutive elements at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2a {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { using type = bf16x8; };
template <> struct Vec8<float> { using type = f32x8; };
// Eight consecutive elements: the per-lane share of one A or B operand.
template <typename T> using v8 = typename Vec8<T>::type;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}

// Eight fp32 accumulator values (registers base..base+7) as an operand of type T.
template <typename T>
__device__ __forceinline__ v8<T> pack8(const f32x16& x, int base);

template <>
__device__ __forceinline__ bf16x8 pack8<bf16>(const f32x16& x, int base) {
  f32x8 f = {x[base + 0], x[base + 1], x[base + 2], x[base + 3],
             x[base + 4], x[base + 5], x[base + 6], x[base + 7]};
  return __builtin_convertvector(f, bf16x8);   // round to nearest even
}

template <>
__device__ __forceinline__ f32x8 pack8<float>(const f32x16& x, int base) {
  f32x8 f = {x[base + 0], x[base + 1], x[base + 2], x[base + 3],
             x[base + 4], x[base + 5], x[base + 6], x[base + 7]};
  return f;
}

template <typename T>
__device__ __forceinline__ v8<T> scale8(const f32x16& x, int base, float s) {
  f32x16 y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[base + i] = x[base + i] * s;
  return pack8<T>(y, base);
}

// Swap bits 2 and 3 of a row index inside a 32-row tile.
__device__ __forceinline__ int perm32(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// LDS tiles are arrays of 8-element chunks.  The chunk column of a row is
// XOR-ed with swz(row) so that the eight rows perm32(0..7) read by one
// quarter-wave land on eight different chunk columns.
template <int CPR>  // chunks per row (power of two)
__device__ __forceinline__ int swz(int row) {
  return ((row & 3) | ((row >> 1) & 4)) & (CPR - 1);
}

template <int CPR>
__device__ __forceinline__ int chunk_at(int row, int chunk) {
  return row * CPR + (chunk ^ swz<CPR>(row));
}

// Original token index of rolled position j for a head rolled by sigma
// (0 <= j < N, 0 <= sigma < N): the roll of the method folded into addresses.
__device__ __forceinline__ int orig_row(int j, int sigma, int N) {
  int t = j + sigma;
  return t >= N ? t - N : t;
}

// Groups of one head: N / G rounded up.  When G does not divide N the last
// group holds the N mod G rows that remain (the reading taken for group sizes
// like Table 7's 1/6 of the context).
__device__ __forceinline__ int num_groups(int N, int G) { return (N + G - 1) / G; }

// The wrap group of a shifted head (rolled by sigma = floor(G/2)): the rolled
// group in which the rolled order wraps from token N-1 to token 0.  It spans
// rows [gw0, ge); rows [gw0, c) hold tokens gw0 + sigma .. N-1 and rows
// [c, ge) the L = ge - c tokens 0 .. L-1 that the roll carried from the front,
// with c = N - sigma.  When G divides N it is the last group (gw0 = N - G,
// c = N - G/2, ge = N, L = G/2).  L = 0 when the wrap falls on a group
// boundary: no group wraps.
struct WrapGroup { int gw0, c, ge, L; };
__device__ __forceinline__ WrapGroup wrap_group(int N, int G) {
  const int c = N - G / 2;
  const int gw0 = c - c % G;
  const int ge = min(gw0 + G, N);
  return {gw0, c, ge, c > gw0 ? ge - c : 0};
}

// Wrap options as the kernels take them (the values of s2attn_wrap).
constexpr int kWrapRoll = 0, kWrapSplit = 1, kWrapSwap = 2;

// Split wrap option (page section 5, "Ablation Studies and Robustness Checks",
// Table 8 / Figure 6, Variant 2).  With `split_head` (the option is on and the
// head is shifted) the wrap group is cut at row c into two causal groups: the
// end tokens [gw0, c) and the front tokens [c, ge); every other group is
// unchanged.  Rows are in the head's rolled frame.
// First key row visible to query row j:
__device__ __forceinline__ int first_key_row(int j, int G, bool split_head, const WrapGroup& wg) {
  const int gs = j - j % G;
  return (split_head && wg.L > 0 && gs == wg.gw0 && j >= wg.c) ? wg.c : gs;
}
// One past the last query row that sees key row j (a group that G does not
// fill ends at N):
__device__ __forceinline__ int query_end_row(int j, int G, int N, bool split_head, const WrapGroup& wg) {
  const int gs = j - j % G;
  return (split_head && wg.L > 0 && gs == wg.gw0 && j < wg.c) ? wg.c : min(gs + G, N);
}
// The split option's cut inside the group starting at row gs: query rows at or
// after it see no key row before it.  -1 (no cut) for every other group.
__device__ __forceinline__ int split_cut(int gs, bool split_head, const WrapGroup& wg) {
  return (split_head && wg.L > 0 && gs == wg.gw0) ? wg.c : -1;
}

// Swap wrap option (Table 8 / Figure 6, Variant 3): in a shifted head the wrap
// group keeps its tokens, but the L tokens the roll carried from the front of
// the sequence come first, so that causal order in that group is token order:
// rows gw0 .. gw0+L-1 hold tokens 0 .. L-1 and rows gw0+L .. ge-1 hold tokens
// gw0 + sigma .. N-1.
// Token held at rolled row j of a head rolled by sigma:
template <bool SWAP>
__device__ __forceinline__ int token_of_row(int j, int sigma, int N, const WrapGroup& wg) {
  if (SWAP && sigma != 0 && j >= wg.gw0 && j < wg.ge && wg.L > 0)
    return j < wg.gw0 + wg.L ? j - wg.gw0 : j - wg.L + sigma;
  return orig_row(j, sigma, N);
}
// ... and its inverse, the row of token t:
template <bool SWAP>
__device__ __forceinline__ int row_of_token(int t, int sigma, int N, const WrapGroup& wg) {
  if (SWAP && sigma != 0 && wg.L > 0) {
    if (t < wg.L) return wg.gw0 + t;
    if (t >= wg.gw0 + sigma) return t - sigma + wg.L;
  }
  const int j = t - sigma;
  return j < 0 ? j + N : j;
}

// The row that rolled row j of a head rolled by sig_from has in the frame of a
// head rolled by sig_to (the same token).
template <bool SWAP>
__device__ __forceinline__ int frame_row(int j, int sig_from, int sig_to, int N, const WrapGroup& wg) {
  if (SWAP) return row_of_token<true>(token_of_row<true>(j, sig_from, N, wg), sig_to, N, wg);
  int r = j + sig_from - sig_to;
  if (r < 0) r += N;
  if (r >= N) r -= N;
  return r;
}

// Whether rows [j, j + n) of a head rolled by sigma hold n consecutive tokens
// (one buffer based at the first row's token then serves the whole tile): all
// rows below N and no break of the row -> token map strictly inside.  Breaks:
// row c (token N-1 -> 0) of the roll; under the swap option rows gw0, gw0 + L
// and ge instead; and row N.
template <bool SWAP>
__device__ __forceinline__ bool rows_contiguous(int j, int n, int sigma, int N, const WrapGroup& wg) {
  if (j + n > N) return false;
  auto inside = [&](int r) { return j < r && r < j + n; };
  if (sigma == 0) return true;
  if (SWAP && wg.L > 0) return !inside(wg.gw0) && !inside(wg.gw0 + wg.L) && !inside(wg.ge);
  return !inside(N - sigma);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotary embedding with Position Interpolation (page "LongLoRA: Efficient
// Fine-tuning of Long-Context Large Language Models", section 3.2 Phase 1
// item 2, and "Model setup": the pre-trained rotary embeddings rescaled by
// Position Interpolation; the pages give no formula, the rotate-half pairing is
// the published rotary embedding).  Pair (i, i + D/2), i < D/2, of token n turns
// by n * pos_scale * base^(-2i/D) radians.  One set of helpers serves the
// stand-alone pass and the attention kernels that fuse the rotation, so the two
// produce the same bits.
// Revolutions per position of the 8 pairs i0 .. i0+7 (i0 a multiple of 8),
// float64: base^(-2 i0 / D) / (2 pi) from one exp2, then successive products
// with base^(-2/D) (7 roundings: a relative error below 1e-15, ~1e-11
// revolutions at positions near 1e5), so each run of 8 costs two exp2 instead
// of eight.  Every kernel takes its frequencies from here.
template <int D>
__device__ __forceinline__ void rope_revs8(int i0, double log2_base, double g[8]) {
  const double r = exp2(-(2.0 / D) * log2_base);
  g[0] = exp2(-(2.0 * i0 / D) * log2_base) * 0.15915494309189533577;
#pragma unroll
  for (int e = 1; e < 8; ++e) g[e] = g[e - 1] * r;
}
// Cosine and sine of pos * g revolutions, pos = n * pos_scale: the angle is
// formed in float64 and reduced to [-1/2, 1/2] revolutions (a float32 angle
// would be off by ~1e-2 rad at positions near 1e5) before the hardware sine
// and cosine of revolutions.
__device__ __forceinline__ void rope_cs(double pos, double g, float& cs, float& sn) {
  const double u = pos * g;
  const float fr = (float)(u - rint(u));
  sn = __builtin_amdgcn_sinf(fr);
  cs = __builtin_amdgcn_cosf(fr);
}
// The pair (a, b) = (x_i, x_{i + D/2}) turned by the angle (sn < 0: backwards).
// Explicit fused multiply-adds, so every kernel rounds the same way.
__device__ __forceinline__ void rope_turn(float a, float b, float cs, float sn, float& ya, float& yb) {
  ya = fmaf(a, cs, -(b * sn));
  yb = fmaf(b, cs, a * sn);
}
// Fused rotation of the attention kernels: `on` = rotate; pos_scale and
// log2(base) as above; q_rot receives the rotated q written by the forward.
struct RopeArgs {
  bf16* q_rot;
  double pos_scale;
  double log2_base;
  int on;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Global memory straight into LDS (no registers): lane i of the wave fills
// bytes [16 i, 16 i + 16) after the wave-uniform LDS base.
// (amdgcn builtins sit in helpers like these, not in kernel bodies, so that
// the host pass still emits every kernel's launch stub.)
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// The same with 4 bytes per lane.
__device__ __forceinline__ void load_lds4(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Raw buffer resource over [base, base + nbytes): loads through it take a
// 32-bit byte offset, per lane (voff) plus wave-uniform (soff, a scalar
// register); offsets past nbytes read zeros.  The kernels base one at the
// first row of each tile they load (a 64-bit scalar address), so that no
// offset grows with the sequence length or the batch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, 0x00020000);
}
// n bytes per lane (16 or 4) from a buffer straight into LDS: lane i fills
// bytes [n i, n i + n) after the wave-uniform LDS base, reading resource base
// + voff (per lane) + soff (wave-uniform) bytes.  The 32-bit offsets keep the
// address arithmetic in scalar registers.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, voff, soff, 0, 0);
}

// max of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the two
// 32-lane halves without a trip through LDS)
__device__ __forceinline__ float max_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                   __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                   __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
}

// Block numbering shared by the attention kernels.  A launch covers `pairs`
// (batch, head, group) pairs times `ranks` tiles per pair, rank 0 being the
// tile with the most work.  Blocks are numbered chunk by chunk, kPairChunk
// pairs per chunk, rank-major inside a chunk: a chunk's heavy tiles start
// first and its light ones fill the tail of the launch.  Round-robin dispatch
// over the 8 XCDs then places every block of one pair of a full chunk on the
// same XCD (kPairChunk is a multiple of 8), close together in time, so the
// pair's K/V tiles are reused from that XCD's L2.
constexpr int kPairChunk = 32;
struct TileOrder { int pair, rank; };
__device__ __forceinline__ TileOrder tile_order(int idx, int pairs, int ranks) {
  const int per_chunk = kPairChunk * ranks;
  const int chunk = idx / per_chunk;
  const int first = chunk * kPairChunk;
  const int n = min(kPairChunk, pairs - first);
  const int rem = idx - chunk * per_chunk;
  return {first + rem % n, rem / n};
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float dot2_bf16_acc(bf16 a, bf16 b, float acc) {
  const bf16x2_t pr = {a, b};
  const bf16x2_t ones = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane i receives element (i & 3) of the 8-byte pieces addressed by lanes
// 4s + (i >> 2), s = 0..3, in that order.  If lane 4s + m addresses row r0 + s
// at column c(m), lane i therefore gets rows r0..r0+3 of column c(i >> 2) + (i & 3):
// four consecutive k-values of one operand row, from a tile stored k-major.
// tr_read8 joins two such reads (rows r0..r0+3 and r0+4..r0+7).
__device__ __forceinline__ bf16x8 tr_read8(const bf16* p0, const bf16* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}


}  // namespace s2a
