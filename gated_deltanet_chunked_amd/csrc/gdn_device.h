// gdn_device.h -- device-side helpers shared by the libgdn HIP kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions (v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 x 32):  lane l holds row (l % 16), 8 consecutive k values of k-group (l / 16)
//   B operand (32 x 16):  lane l holds column (l % 16), the 8 k values of k-group (l / 16)
//   C/D (16 x 16, fp32):  lane l holds column (l % 16), rows 4*(l / 16) + r, r = 0..3
// Element e of lane group g in A multiplies element e of lane group g in B, so any consistent
// assignment of contraction indices to (g, e) slots gives the same product; the kernels use that
// freedom to feed accumulators back as operands without moving data between lanes.
// v_mfma_f32_16x16x4_f32 has the same C/D layout; A lane l holds A[l % 16][k = l / 16] and B lane l
// holds B[k = l / 16][l % 16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kDim = 128;    // dk = dv
constexpr int kDvTile = 16;  // value columns per state-pass workgroup
constexpr int kDvTiles = kDim / kDvTile;

// ---- per-(chunk slot, v-head) record written by the prep kernel, read by the state pass ----
// Six 16x32 A-operand fragments cover the lower block triangle of a 64x64 chunk matrix:
//   fragment f -> (row block, k step): 0:(0,0) 1:(1,0) 2:(2,0) 3:(2,1) 4:(3,0) 5:(3,1)
// Row block w therefore owns fragments kFragBase[w] .. kFragBase[w] + kFragCount[w] - 1.
constexpr int kFrags = 6;
constexpr int kFragBytes = 64 * 16;                       // 64 lanes x 8 bf16
constexpr int kRecTpHi = 0;                               // T' = (I+A)^-1 diag(beta), bf16 high part
constexpr int kRecTpLo = kRecTpHi + kFrags * kFragBytes;  // T' low part (T' - hi rounded to bf16)
// P = tril(Q K^T o e^{G_i - G_j}), bf16; its k-slots are permuted: fragment (row block, k step
// ks), lane (row i, group g), slot e holds column 32 ks + 16 (e / 4) + 4 g + e % 4.  (T' uses the
// plain order: slot e holds column 32 ks + 8 g + e.)
constexpr int kRecP = kRecTpLo + kFrags * kFragBytes;
constexpr int kRecEG = kRecP + kFrags * kFragBytes;       // e^{G_i}           fp32[64]
constexpr int kRecED = kRecEG + kChunk * 4;               // e^{G_last - G_i}  fp32[64]
constexpr int kRecBytes = kRecED + kChunk * 4;            // 18944

__host__ __device__ constexpr int frag_row_block(int f) { return f < 2 ? f : (f < 4 ? 2 : 3); }
__host__ __device__ constexpr int frag_k_step(int f) { return (f == 3 || f == 5) ? 1 : 0; }

// One pass of the time split of a single long sequence (segs > 0): the sequence's chunks are cut
// into segments of m chunks, and grid "sequence" n is segment n.  mode 0: each segment from a
// zero state, end states to h_out, o not written; mode 1: v taken as zero and the identity as
// initial state, so the end state is the segment's transition matrix, to h_out, o not written;
// mode 2: each segment from h_in[n], o written, the last segment's end state to hT.  h_in and h_out
// are [segs, Hv, 128, 128] fp32, key-major.
struct SplitPass {
  int segs, m, mode;
  const float *h_in;
  float *h_out;
};
// With a split, the state buffers hold at most kSplitStates (segment, v-head) states each.
constexpr int kSplitStates = 32;

// The mixer's gated RMSNorm fused into the state pass's output path: the pass writes
// y = o / sqrt(mean_dv(o^2) + eps) * w * silu(z) per (token, v-head) instead of o.  A row's 128
// columns are spread over the kDvTiles column workgroups of its head; each publishes its tile's
// sum of squares of the bf16 row as one device-scope atomic word of part ([T, Hv, kDvTiles]),
// which the chunk prep fills with kPartEmpty first, so every word is its own "written" flag.
struct NormOut {
  const unsigned short *z, *w;  // bf16 [T, Hv, 128], bf16 [128]
  unsigned short *y;            // bf16 [T, Hv, 128]
  uint32_t *part;
  float eps;
};
constexpr uint32_t kPartEmpty = 0xffffffffu;

// Chunk-slot numbering: chunk c of sequence n lives in slot cu[n] / 64 + n + c.  The map is
// injective and monotone, and every slot index is below T / 64 + N.
__host__ __device__ inline int64_t num_slots(int64_t T, int32_t N) { return T / kChunk + N; }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }
__device__ __forceinline__ float bits_to_float(unsigned short b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ unsigned short bf16_bits(__bf16 x) {
  return __builtin_bit_cast(unsigned short, x);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 significant bits in total.
__device__ __forceinline__ void split_hilo(float x, __bf16 &hi, __bf16 &lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - from_bf16(hi));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// 16-byte global load of 8 bf16 (caller guarantees 16-byte alignment).
__device__ __forceinline__ bf16x8 load_bf16x8(const void *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void store_bf16x8(void *p, bf16x8 x) {
  *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, x);
}

// x of another lane through a DPP lane pattern (a vector ALU operand modifier, no LDS round trip);
// lanes that the pattern gives no source, or that RowMask leaves out, read 0.
template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, RowMask, 0xf, true));
}
// Inclusive prefix sum across the 64 lanes of a wave, on DPP: a Hillis-Steele scan inside each
// 16-lane row (row_shr 1, 2, 4, 8), then each row's total carried into the rows after it
// (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3; gfx9 DPP).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_or_zero<0x111>(x);
  x += dpp_or_zero<0x112>(x);
  x += dpp_or_zero<0x114>(x);
  x += dpp_or_zero<0x118>(x);
  x += dpp_or_zero<0x142, 0xa>(x);
  x += dpp_or_zero<0x143, 0xc>(x);
  return x;
}
// x of lane `lane` (wave-uniform) in every lane.
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---- GDN mixer input prep (conv + SiLU + L2 norm): shared by mixer_prep_kernel and the prep
// kernel that makes q, k, v from the packed input itself ----
// x sigmoid(x) with the hardware exp2 and reciprocal (each about 1 ulp): the result is rounded
// to bf16 (8 bits) right after, far above their error.  Saturates correctly: exp2 overflows to
// inf for x << 0 (result -0), underflows to 0 for x >> 0 (result x).
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// 1 / sqrt(x) for x > 0 with the hardware reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ float sum16(float x) {
  // sum over the 16 lanes that share l / 16, on DPP: rotations by 8 and 4 inside the row, then
  // the quad permutations [1,0,3,2] and [2,3,0,1]; every lane ends with the row's sum
  x += dpp_or_zero<0x128>(x);
  x += dpp_or_zero<0x124>(x);
  x += dpp_or_zero<0xB1>(x);
  x += dpp_or_zero<0x4E>(x);
  return x;
}

// Gate parameters made from the layer's projections (gdn_mixer_fwd_gates): for token t and v-head
// h, g = -exp(A_log[h]) softplus(a[t,h] + dt_bias[h]) and beta = sigmoid(b[t,h]), with a, b bf16
// [T, Hv] and A_log, dt_bias fp32 [Hv].  With a null the kernels read g and beta as given.
struct GateArgs {
  const unsigned short *a, *b;
  const float *A_log, *dt_bias;
};
// The inputs of one (token i, v-head h), loaded apart from the arithmetic so that the loads can be
// issued with the kernel's other loads.
struct GateIn {
  unsigned short a, b;
  float A_log, dt_bias;
};
__device__ __forceinline__ GateIn gate_load(const GateArgs &ga, size_t i, int h) {
  return GateIn{ga.a[i], ga.b[i], ga.A_log[h], ga.dt_bias[h]};
}
// On the hardware exp2, log2 and reciprocal (about 1 ulp each): softplus(x) = max(x, 0) +
// ln 2 log2(1 + 2^(-|x| log2 e)) never overflows, and its absolute error stays near 1e-7 where the
// log2 argument rounds to 1 (|x| > 17, softplus below 4e-8), far inside what the decay needs.
__device__ __forceinline__ void gate_values(const GateIn &in, float &g, float &beta) {
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float x = bits_to_float(in.a) + in.dt_bias;
  const float sp = fmaxf(x, 0.f) + kLn2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e));
  g = -__builtin_amdgcn_exp2f(in.A_log * kLog2e) * sp;
  beta = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-bits_to_float(in.b) * kLog2e));
}

// Carried conv window of sequence n ([W, C] bf16, oldest row first), or null for zeros.
__device__ __forceinline__ const unsigned short *window_of(const unsigned short *conv_in,
                                                           const int32_t *state_index,
                                                           int num_states, int n, size_t rows) {
  if (!conv_in) return nullptr;
  const int r = state_index ? state_index[n] : n;
  return (r >= 0 && r < num_states) ? conv_in + (size_t)r * rows : nullptr;
}

// Workgroups are dealt to the 8 XCDs round-robin (hardware id b runs on XCD b % 8).  Renumber
// so that consecutive logical ids share an XCD and therefore its L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace gdn
